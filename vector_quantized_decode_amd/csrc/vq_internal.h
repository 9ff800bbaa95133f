// Internal declarations shared by the host API (vq_api.cpp) and the HIP
// kernels (vq_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/vqd.h"

namespace vqd {

// Launch shapes shared by the kernels' launchers and the host shape rules.
constexpr int WC12_W = 4;      // waves per workgroup, 12-bit kernel
constexpr int WC12_PF = 2;     // chunks in flight per wave, 12-bit kernel
constexpr int WC8_W = 8;       // waves per workgroup, 8-bit kernels
constexpr int WC8_NCH = 4;     // chunks per wave of the burst kernel
constexpr int TK_W = 8;        // waves per workgroup, token kernel
constexpr int RD_W = 8;        // waves per workgroup, streaming read (as the 8-bit lookup kernels)
constexpr int RD_NCH = 4;      // 1 KiB chunks per wave, streaming read (as the burst kernel)

// Per-matrix descriptor of the 8-bit lookup GEMV kernels.  Lives in the
// kernel-argument segment; all pointers are device pointers.
struct Lut8Mat {
  const uint8_t *wi;      // WI, device layout tile-16x64
  const uint16_t *wc;     // fp16 codebook [256][4]
  const uint16_t *x;      // fp16 input [K] (plain kernel)
  const float *xr;        // fp32 rotated input [K] (residual kernel)
  const uint8_t *signs;   // sign bits, device layout tile-32x32 (residual)
  const uint16_t *alpha;  // fp16 scales, device layout (residual)
  float *y;               // fp32 output [N]
  float *partial;         // fp32 split partial sums [nsplit][rows_pad]
  uint32_t *counter;      // completion counters [nrb]
  uint64_t *acc;          // packed fixed-point row accumulators [rows_pad]
  const int8_t *rs;       // residual: rotation signs [K] (+-1), or null
  const uint32_t *alpha_hdr;  // residual: largest |alpha| (fp16 magnitude bits)
  float had_scale;        // residual: 1/sqrt(had)
  int32_t had;            // residual: Hadamard block (1: no rotation)
  int32_t fused;          // residual: rotate x inside the lookup kernel (else xr holds it)
  int32_t rpw;            // residual: 32-row pairs per workgroup
  int32_t J;              // subvectors per row, K/4
  int32_t N;              // output rows
  int32_t rows_pad;       // rows of the padded layout (multiple of 32)
  int32_t nsplit;         // workgroups sharing a row block (split along J)
  int32_t nrb;            // row blocks
  int32_t nwg;            // workgroups of this matrix (nsplit * nrb)
};

// Matrix m of a grouped call is served by workgroups (x, m) of a 2-D grid
// with x < mat[m].nwg; the grid is as wide as the largest matrix needs.
struct Lut8Args {
  Lut8Mat mat[VQ_MAX_GROUP];
  int32_t count;
};

// Per-matrix descriptor of the per-index kernels (n = 8, 12 and 16, and the
// token kernel).  Matrix m is served by workgroups (x, m) of a 2-D grid as
// wide as the largest matrix needs, except for the 16-bit lookup kernel,
// which takes a flat grid of every matrix's workgroups in turn.
struct WcMat {
  const uint8_t *wi;      // WI: device layout tile-16x64(-12), tile-16x32-16 or row tiles
  const uint16_t *wc;     // fp16 codebook [2^n][d]
  const uint16_t *x;      // fp16 input [B][K]
  float *y;               // output [B][N], row stride ldy: fp32, or fp16 when yf16
  int32_t J;              // subvectors per row, K/d
  int32_t N;              // output rows
  int32_t B;              // tokens
  int32_t ldy;            // y row stride (N)
  int32_t nwg;            // workgroups of this matrix
  int32_t jsplit;         // waves sharing a row group along J
  int32_t yf16;           // 1: y holds fp16 (the fp32 sum rounded to nearest even)
  int32_t nmem;           // 8-bit burst kernel: matrices sharing wc, x and shape laid
                          // end to end by row group (1: this matrix alone)
  int32_t mem0;           // nmem > 1: the first member's slot in WcUnitArgs::mwi / my
};

struct WcArgs {
  WcMat mat[VQ_MAX_GROUP];
  int32_t count;
};

// A grouped 8-bit call whose matrices sharing the codebook, x and shape are
// merged into units (WcMat::nmem > 1): the members' indices and outputs.
// Kept out of WcArgs so that calls without shared matrices pass the smaller
// argument block (measured 0.15 us per LLaMA-7B q/k/v/o call).
struct WcUnitArgs {
  WcArgs a;
  const uint8_t *mwi[VQ_MAX_GROUP];
  float *my[VQ_MAX_GROUP];
};

// Gate/up pairs of the fused SiLU-gated call: a.mat[i] is the gate matrix
// (with x and y), wi2 / wc2 the up matrix of the same shape.
struct WcPairArgs {
  WcArgs a;
  const uint8_t *wi2[VQ_MAX_GROUP];
  const uint16_t *wc2[VQ_MAX_GROUP];
};

// The 16-bit kernel's per-matrix scratch (in the caller's workspace): x's
// values by dimension in the order the kernel reads them.  The codebook
// (WcMat::wc) is in the dimension-major layout of vq_repack_wc.
struct Wc16tArgs {
  WcArgs a;
  uint16_t *xt[VQ_MAX_GROUP];    // [8][B][K/8] fp16
};

int wc12_rows_per_wg(int jsplit);
int wc12_jsplit(int J);
int wc8_waves(int64_t indices, int max_split, int B);
int wc8_rows_per_wg(int jsplit, int waves);
int wc8_burst_waves();
int wc8_jsplit(int N, int J);
bool wc8_burst_fits(int N, int J, int jsplit);
int launch_wc8(const WcArgs &a, int grid_x, int waves, bool burst, int B, void *stream);
int launch_wc8_units(const WcUnitArgs &a, int grid_x, int B, void *stream);
int launch_wc12(const WcArgs &a, int grid_x, int max_j, void *stream);
int wc8_swiglu_waves(int max_split);
int launch_wc8_swiglu(const WcPairArgs &a, int grid_x, int waves, int B, void *stream);
int wc8t_jsplit(int J, int B);
int wc8t_max_rw(int B);
int wc8t_max_cols(int B);
int wc8t_rows_per_wg(int jsplit, int rw);
int launch_wc8t(const WcArgs &a, int grid_x, int rw, void *stream);
int launch_repack_wi8_rows(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream);
int wc16t_jsplit(int J);
int wc16t_rows_per_wg(int jsplit);
bool wc16t_fits(int N, int J, int jsplit);
// The 16-bit lookup kernel takes a flat grid of grid_x = the call's total
// workgroups (the pre-pass keeps its (prep_blocks, count) grid).
int launch_wc16t(const Wc16tArgs &a, int grid_x, int prep_blocks, void *stream);
int launch_repack_wc16(const uint16_t *wc, uint16_t *wct, void *stream);
int launch_repack_wi12(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream);
int launch_repack_wi16(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream);

// Launch shape of one lookup-kernel variant.
struct Lut8Shape {
  int waves;    // wavefronts per workgroup
  int steps;    // 32-row steps per wave (at least the run / waves)
  int nbx;      // 16-byte chunks of x per thread for the hand-off bound (2 or 4)
  int pairs;    // target 32-row pairs per workgroup
};

// Variant selection (shared by workspace sizing and launch).
Lut8Shape lut8_shape_residual(const vq_matrix *m, int32_t count);

// Kernel launchers: return a hipError_t value (0 = success).
// Lookup kernels: grid (grid_x, a.count), grid_x = the most workgroups any
// matrix of the call needs.
int launch_lut8_residual(const Lut8Args &a, const Lut8Shape &s, int grid_x, void *stream,
                         bool residual);
int launch_pack(const uint32_t *idx, int64_t count, int nbits, uint8_t *out, void *stream);
int launch_unpack(const uint8_t *packed, int64_t count, int nbits, uint32_t *out, void *stream);
int launch_repack_wi8(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream);
int launch_repack_signs(const uint8_t *canon, int N, int P, uint8_t *dev, void *stream);
int launch_repack_alpha(const uint16_t *canon, int N, int G, uint16_t *dev, uint32_t *hdr,
                        void *stream);
int launch_build_oc(const uint16_t *x, int B, int K, int d, int nbits, const uint16_t *wc,
                    void *oc, int f16_out, void *stream);
int launch_rht(const uint16_t *x, const int8_t *sign, int B, int K, int h, float scale,
               float *x_rot, void *stream);
int launch_fill_u32(uint32_t *p, size_t n, uint32_t v, void *stream);
// Device address of the calling thread's current GPU's no-allocation scratch
// (VQ_NOALLOC_SCRATCH_BYTES); returns a hipError_t value.
int noalloc_scratch(void **out);

// Plain streaming read of up to VQ_MAX_READ device buffers in one launch
// (measurement only): sink[(m * grid_x + x) * words_per_wg + w] receives the
// XOR of what wave w of workgroup (x, m) read.
constexpr int VQ_MAX_READ = 64;
struct ReadArgs {
  const uint8_t *buf[VQ_MAX_READ];
  uint32_t bytes[VQ_MAX_READ];
  uint32_t *sink;
  int32_t count;
};
int64_t stream_read_workgroups(uint32_t max_bytes);
int stream_read_sink_words_per_wg();
int launch_stream_read(const ReadArgs &a, int grid_x, void *stream);

}  // namespace vqd
