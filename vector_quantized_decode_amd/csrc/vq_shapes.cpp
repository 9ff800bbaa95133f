// Host-side shape rules of libvqd: how each call's rows and subvectors are
// split over waves and workgroups, and which shapes each kernel's 32-bit
// buffer offsets allow.  Plain C++ with no HIP call, shared by the kernel
// launchers (vq_kernels*.hip) and the host API (vq_api.cpp).
#include "vq_internal.h"

namespace vqd {

int wc12_rows_per_wg(int jsplit) { return WC12_W / jsplit * 16; }
// Waves per row group along J for the 12-bit kernel.  Two chunks in flight
// per wave and short segments measured fastest: with fewer loads queued the
// codebook and each wave's first chunks come back sooner.
int wc12_jsplit(int J) {
  const int JT = J / 64;
  return JT <= 12 ? 1 : (JT <= 24 ? 2 : 4);
}
// Waves per row group along J for the 8-bit kernels: the smallest power of
// two (at most 8) that leaves each wave at most four 64-subvector chunks,
// doubled while the matrix has fewer than 64 workgroups of 8 waves and the
// row has chunks to spare.  It depends on the matrix alone, so a matrix sums
// in the same order alone or in a group, whichever kernel serves the group.
int wc8_jsplit(int N, int J) {
  const int64_t ng = (N + 15) / 16;
  const int jt = J / 64;
  int s = 1;
  while (s < WC8_W && (jt + s - 1) / s > WC8_NCH) s *= 2;
  while (2 * s <= WC8_W && 2 * s <= jt && (ng * s + WC8_W - 1) / WC8_W < 64 &&
         (jt <= 2 || (jt + 2 * s - 1) / (2 * s) >= 2))
    s *= 2;
  return s;
}
// Waves per workgroup: 8, or 4 for one-token calls of at most 2^20 indices
// whose splits allow it (there more, smaller workgroups start sooner; measured 2.7 against
// 3.1 us for one 512 x 512 matrix).  Only the number of row groups per
// workgroup changes, not the order of any sum.
int wc8_waves(int64_t indices, int max_split, int B) {
  return (B == 1 && indices <= ((int64_t)1 << 20) && max_split <= 4) ? 4 : WC8_W;
}
int wc8_rows_per_wg(int jsplit, int waves) { return waves / jsplit * 16; }
// Waves per workgroup of the burst kernel (the waves for which it is built).
int wc8_burst_waves() { return WC8_W; }
// The burst kernel serves a call when every row fits in its waves' chunks
// and the matrix's indices lie within one 32-bit buffer offset.
bool wc8_burst_fits(int N, int J, int jsplit) {
  const int64_t bytes = (int64_t)((N + 15) / 16) * 1024 * (J / 64);
  return (J / 64 + jsplit - 1) / jsplit <= WC8_NCH && bytes < ((int64_t)1 << 31);
}

// Waves of the fused gate/up kernel: two row-group slots per output row
// group, so 8 waves for a split of up to 4 and 16 for a split of 8.
int wc8_swiglu_waves(int max_split) { return max_split <= 4 ? WC8_W : 2 * WC8_W; }
// Waves per row group along J for the 16-bit kernel: the smallest count (at
// most 16) that leaves each wave at most 12 blocks of 32 subvectors, else 16
// (a wave's indices stay in registers for the eight passes, up to 16
// blocks).  A workgroup of 16 waves holds 16 / S row groups and leaves
// 16 mod S waves without rows: S need not divide 16, so that matrices of
// different row lengths in one call get about the same blocks per wave
// (LLaMA-13B shapes: 10 blocks per wave at K = 5120, 11 at K = 13824, where
// a power-of-two split gave 14).
int wc16t_jsplit(int J) {
  const int JB = J / 32;
  int s = 1;
  while (s < 16 && (JB + s - 1) / s > 12) ++s;
  return s;
}
int wc16t_rows_per_wg(int jsplit) { return 16 / jsplit * 16; }
// Rows of at most 256 blocks (K <= 65536), indices within 32-bit offsets.
bool wc16t_fits(int N, int J, int jsplit) {
  return (J / 32 + jsplit - 1) / jsplit <= 16 && (int64_t)((N + 15) / 16) * (J / 32) * 1024 < ((int64_t)1 << 31);
}
// Columns of 64 subvectors per wave and the most row groups per wave: more
// tokens mean more x per column, which more row groups per wave share, and
// shorter segments keep more waves on the rows (measured on 4 x 4096 x 4096:
// up to 12 tokens four columns and two row groups, above that two columns
// and four row groups).
int wc8t_max_cols(int B) { return B > 12 ? 2 : 4; }
int wc8t_max_rw(int B) { return B > 12 ? 4 : 2; }
// Waves per row group along J for the token kernel: the smallest power of
// two (at most 8) that leaves each wave at most wc8t_max_cols(B) columns.  It
// depends on the row length and the token count alone, so a matrix sums in
// the same order alone or in a group.
int wc8t_jsplit(int J, int B) {
  const int jt = J / 64, cols = wc8t_max_cols(B);
  int s = 1;
  while (s < TK_W && (jt + s - 1) / s > cols) s *= 2;
  return s;
}
int wc8t_rows_per_wg(int jsplit, int rw) { return TK_W / jsplit * rw * 16; }
int64_t stream_read_workgroups(uint32_t max_bytes) {
  const int64_t per_wg = (int64_t)RD_W * RD_NCH * 1024;
  return ((int64_t)max_bytes + per_wg - 1) / per_wg;
}

int stream_read_sink_words_per_wg() { return RD_W; }

}  // namespace vqd
