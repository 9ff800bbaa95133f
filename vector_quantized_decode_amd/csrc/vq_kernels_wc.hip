// HIP kernels of libvqd in the per-index form (gfx950): each output-codebook
// entry OC[j][c] = x_j . WC[c] is formed when an index asks for it, from a
// codebook held in LDS, and a workgroup covers whole rows.
//
// Sources, cited by page title and section:
//   [EVA]  "EVA: Accelerating LLM Decoding via an Efficient Vector
//          Quantization Architecture" -- explainer page, technical summary,
//          section 2.A (input-codebook products form the output codebook;
//          lookups into it by the weight indices) and section 2.B (the
//          codebooks stay on chip while indices stream in tiles).
//
// Why per index.  An OC tile in LDS (vq_kernels.hip) covers 256 inputs of
// every centroid, so a row spans K / 256 workgroups that must meet again; on
// MI355X that join cost more than forming entries per index at n = 8 (LLaMA-7B
// q/k/v/o: 7.4 against 5.8 us), and at n = 12 or 16 any tile costs at least
// one LDS store per lookup.  Forming the entry at lookup time costs the same
// d-term dot product and needs only the codebook on chip:
//   * wc8_burst_kernel / wc8_kernel (d = 4, n = 8, 1-4 tokens): the 2 KiB
//     codebook in 16 LDS copies; a lane owns one subvector of a 16-row chunk
//     and forms x_j . WC[c] for its 16 indices with two fp16 dot products
//     each.  wc8_swiglu_kernel and wc8_burst_units_kernel are its gate/up and
//     shared-codebook forms.
//   * wc12_kernel (d = 4, n = 12, one token): WC (4096 x 4 fp16, 32 KiB) sits
//     in LDS; a lane owns one subvector j, reads WC[c] (8 bytes) for each
//     index and adds x_j . WC[c] with two packed fp16 dot products into fp32.
//   * wc16t_kernel (d = 8, n = 16, up to 16 tokens): the codebook (65536 x 8
//     fp16, 1 MiB) does not fit in LDS, but one of its dimensions does
//     (65536 fp16, 128 KiB).  The kernel makes eight passes, one per
//     dimension t, with that dimension's table in LDS; the 16-token
//     contraction sum_j x_b,8j+t WC[c_rj][t] runs on the matrix cores (one
//     v_mfma_f32_16x16x32_f16 per 16 rows x 32 subvectors) with x's
//     dimension-t values as A and the looked-up table values as B.  The
//     wave's indices stay in registers across the passes.
#include <hip/hip_runtime.h>

#include "vq_internal.h"

namespace vqd {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ half2_t h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ float f_of(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t u_of(float f) { return __builtin_bit_cast(uint32_t, f); }

constexpr int WDPP_QUAD_XOR1 = 0xB1;
constexpr int WDPP_QUAD_XOR2 = 0x4E;
constexpr int WDPP_ROW_ROR8 = 0x128;
constexpr int WDPP_ROW_HALF_MIRROR = 0x141;

template <int CTRL>
__device__ __forceinline__ float wdpp(float v) {
  return f_of((uint32_t)__builtin_amdgcn_update_dpp(0, (int)u_of(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ void wswap32(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane32_swap(u_of(a), u_of(b), false, false);
  a = f_of(r[0]);
  b = f_of(r[1]);
}
__device__ __forceinline__ void wswap16(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane16_swap(u_of(a), u_of(b), false, false);
  a = f_of(r[0]);
  b = f_of(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float wtstage(float lo, float hi, bool bit) {
  const float send = bit ? lo : hi;
  const float keep = bit ? hi : lo;
  return keep + wdpp<CTRL>(send);
}
// a[0..15]: per-lane partial sums of rows 0..15 -> full 64-lane sum of row
// (lane >> 2) & 15 in every lane (transposing butterfly, [EVA] 2.B adder tree)
__device__ __forceinline__ float wreduce_rows16(float (&a)[16], int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) { wswap32(a[i], a[i + 8]); a[i] += a[i + 8]; }
#pragma unroll
  for (int i = 0; i < 4; ++i) { wswap16(a[i], a[i + 4]); a[i] += a[i + 4]; }
  const bool b3 = lane & 8, b2 = lane & 4;
  a[0] = wtstage<WDPP_ROW_ROR8>(a[0], a[2], b3);
  a[1] = wtstage<WDPP_ROW_ROR8>(a[1], a[3], b3);
  float v = wtstage<WDPP_ROW_HALF_MIRROR>(a[0], a[1], b2);
  v += wdpp<WDPP_QUAD_XOR1>(v);
  v += wdpp<WDPP_QUAD_XOR2>(v);
  return v;
}

// The descriptor of this workgroup's matrix.  Every field is read from the
// kernel arguments before the first one is used, so the scalar loads share
// one round trip instead of one per dependent use (the early exit, then the
// split, then the pointers), which the first vector loads would wait for.
__device__ __forceinline__ WcMat load_wcmat(const WcArgs &args, int m) {
  const WcMat &R = args.mat[m];
  WcMat M;
  M.wi = R.wi;
  M.wc = R.wc;
  M.x = R.x;
  M.y = R.y;
  M.J = R.J;
  M.N = R.N;
  M.B = R.B;
  M.ldy = R.ldy;
  M.nwg = R.nwg;
  M.jsplit = R.jsplit;
  M.yf16 = R.yf16;
  M.nmem = 1;                                 // units read their member fields themselves
  M.mem0 = 0;
  __asm__ volatile("" ::"s"(M.wi), "s"(M.wc), "s"(M.x), "s"(M.y), "s"(M.J), "s"(M.N), "s"(M.B),
                   "s"(M.ldy), "s"(M.nwg), "s"(M.jsplit), "s"(M.yf16));
  return M;
}
__device__ __forceinline__ WcMat load_wcmat(const WcArgs &args) { return load_wcmat(args, blockIdx.y); }

// Output element i of y: the fp32 sum, or (fp16 epilogue) that sum rounded
// to the nearest fp16, ties to even, for a consumer that reads fp16.
__device__ __forceinline__ void store_y(float *y, int yf16, size_t i, float v) {
  if (yf16)
    reinterpret_cast<_Float16 *>(y)[i] = (_Float16)v;
  else
    y[i] = v;
}
__device__ __forceinline__ void store_y(const WcMat &M, size_t i, float v) { store_y(M.y, M.yf16, i, v); }

// --------------------------------------------------------------------------
// d = 4, n = 12, one token
// --------------------------------------------------------------------------
// Byte address in LDS of WC[c] for index i (0..7) of a 96-bit group of eight
// 12-bit indices (index i in bits [12 i, 12 i + 12)), times 8 bytes per entry.
template <int I>
__device__ __forceinline__ uint32_t wc12_addr(uint32_t w0, uint32_t w1, uint32_t w2) {
  uint32_t c;
  if (I == 0) c = w0 & 0xfffu;
  else if (I == 1) c = (w0 >> 12) & 0xfffu;
  else if (I == 2) c = __builtin_amdgcn_alignbit(w1, w0, 24) & 0xfffu;
  else if (I == 3) c = (w1 >> 4) & 0xfffu;
  else if (I == 4) c = (w1 >> 16) & 0xfffu;
  else if (I == 5) c = __builtin_amdgcn_alignbit(w2, w1, 28) & 0xfffu;
  else if (I == 6) c = (w2 >> 8) & 0xfffu;
  else c = w2 >> 20;
  return c << 3;
}

__device__ __forceinline__ uint2 lds_u2(const char *base, uint32_t byte_addr) {
  return *reinterpret_cast<const uint2 *>(base + byte_addr);
}

// One 64-subvector chunk of 16 rows: w[0..2] rows 0-7, w[3..5] rows 8-15.
// All 16 reads are issued before the first product (16 LDS requests in
// flight); row r adds its two products in dimension order.
__device__ __forceinline__ void wc12_chunk(float (&acc)[16], const uint32_t (&w)[6], uint2 xj,
                                           const char *wc) {
  uint2 e[16];
#define WC12_RD(R, I, A, B, C) e[R] = lds_u2(wc, wc12_addr<I>(A, B, C));
  WC12_RD(0, 0, w[0], w[1], w[2]) WC12_RD(1, 1, w[0], w[1], w[2])
  WC12_RD(2, 2, w[0], w[1], w[2]) WC12_RD(3, 3, w[0], w[1], w[2])
  WC12_RD(4, 4, w[0], w[1], w[2]) WC12_RD(5, 5, w[0], w[1], w[2])
  WC12_RD(6, 6, w[0], w[1], w[2]) WC12_RD(7, 7, w[0], w[1], w[2])
  WC12_RD(8, 0, w[3], w[4], w[5]) WC12_RD(9, 1, w[3], w[4], w[5])
  WC12_RD(10, 2, w[3], w[4], w[5]) WC12_RD(11, 3, w[3], w[4], w[5])
  WC12_RD(12, 4, w[3], w[4], w[5]) WC12_RD(13, 5, w[3], w[4], w[5])
  WC12_RD(14, 6, w[3], w[4], w[5]) WC12_RD(15, 7, w[3], w[4], w[5])
#undef WC12_RD
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[r] = __builtin_amdgcn_fdot2(h2(xj.x), h2(e[r].x), acc[r], false);
    acc[r] = __builtin_amdgcn_fdot2(h2(xj.y), h2(e[r].y), acc[r], false);
  }
}

__device__ __forceinline__ void load_chunk12(uint32_t (&w)[6], const uint8_t *p) {
  const u32x3 a = *reinterpret_cast<const u32x3 *>(p);
  const u32x3 b = *reinterpret_cast<const u32x3 *>(p + 12);
  w[0] = a[0]; w[1] = a[1]; w[2] = a[2];
  w[3] = b[0]; w[4] = b[1]; w[5] = b[2];
}

// Workgroup: W waves over W/S row groups of 16 rows; the S waves of a row
// group split its J/64 subvector chunks into S contiguous segments (S = 1, 2
// or 4, chosen by the host so no wave walks much more than the others), each
// with PF chunks of indices (and the matching x slices) in flight.  The S
// partial row sums meet in LDS and are added in segment order.  LDS holds the
// codebook (32 KiB), so several workgroups share a compute unit.
template <int W, int PF>
__global__ void __launch_bounds__(W * 64) wc12_kernel(const WcArgs args) {
  constexpr int NT = W * 64;
  constexpr int WCP = 2048 / NT;              // 16-byte codebook pieces per thread
  __shared__ __align__(16) char wc[4096 * 8];
  __shared__ float part[W * 64];
  const WcMat M = load_wcmat(args);
  if ((int)blockIdx.x >= M.nwg) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = M.jsplit;
  const int rgl = wave / S, sg = wave % S;
  const int JT = M.J >> 6;
  const int NG = (M.N + 15) >> 4;
  const int rgw = (int)blockIdx.x * (W / S) + rgl;
  const int rg = min(rgw, NG - 1);
  const int seg = (JT + S - 1) / S;
  const int kbeg = min(sg * seg, JT), kend = min(kbeg + seg, JT);

  // 1. codebook pieces for LDS, then the first PF index chunks and x slices:
  //    every load is issued before the first wait
  u32x4 wcp[WCP];
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(M.wc);
#pragma unroll
    for (int u = 0; u < WCP; ++u) wcp[u] = src[threadIdx.x + u * NT];
  }
  const uint8_t *wi = M.wi + ((size_t)rg * JT * 64 + lane) * 24;
  const uint2 *xg = reinterpret_cast<const uint2 *>(M.x) + lane;   // x_j, j = 64 k + lane
  uint32_t buf[PF][6];
  uint2 xbuf[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int k = min(kbeg + p, JT - 1);
    load_chunk12(buf[p], wi + (size_t)k * 64 * 24);
    xbuf[p] = xg[k * 64];
  }
  {
    u32x4 *dst = reinterpret_cast<u32x4 *>(wc);
#pragma unroll
    for (int u = 0; u < WCP; ++u) dst[threadIdx.x + u * NT] = wcp[u];
  }
  __syncthreads();

  // 2. lookups: OC[j][c] = x_j . WC[c] formed per index, summed per row
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int k0 = kbeg; k0 < kend; k0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int k = k0 + p;
      uint32_t cur[6];
#pragma unroll
      for (int q = 0; q < 6; ++q) cur[q] = buf[p][q];
      const uint2 xj = xbuf[p];
      // refill this slot with chunk k + PF (clamped: in bounds, unused)
      const int kn = min(k + PF, JT - 1);
      load_chunk12(buf[p], wi + (size_t)kn * 64 * 24);
      xbuf[p] = xg[kn * 64];
      if (k < kend) wc12_chunk(acc, cur, xj, wc);
    }
  }

  // 3. rows out: lane 4r holds row r of the 16 (segments added in order)
  float v = wreduce_rows16(acc, lane);
  if (S > 1) {
    part[wave * 64 + lane] = v;
    __syncthreads();
    if (sg != 0) return;
    v = part[wave * 64 + lane];
    for (int t = 1; t < S; ++t) v += part[(wave + t) * 64 + lane];
  }
  const int row = rgw * 16 + ((lane >> 2) & 15);
  if ((lane & 3) == 0 && rgw < NG && row < M.N) store_y(M, row, v);
}

// --------------------------------------------------------------------------
// d = 4, n = 8, one token
// --------------------------------------------------------------------------
// Same walk as wc12_kernel over the 8-bit tile layout of vq_kernels.hip
// (chunk (jt, rg): lane l = subvector 64 jt + l, byte i = row 16 rg + i).
// The output codebook is formed per index, OC[j][c] = x_j . WC[c], from a
// codebook (256 x 4 fp16, 2 KiB) kept in LDS as 16 copies: entry c of copy
// k at byte 256 c + 8 k, so copy k sits in banks 2k and 2k + 1 whatever c
// is.  Lane l reads copy l % 16; the address is one byte permute (byte 1 =
// the index, byte 0 = 8 (l % 16)).  Lanes l and l + 16 share a bank pair,
// so each 64-lane 8-byte read takes two bank-conflict cycles whatever the
// indices are (rocprofv3: 44% of the LDS-active cycles of the LLaMA-7B
// q/k/v/o call).  32 copies, one bank pair per lane of a 32-lane half, are
// conflict-free but measured no faster: staging twice the copies before the
// first lookup costs what the conflicts save.  No partial sums leave the
// workgroup: there is no hand-off, no workspace and no bound.
template <int K>
__device__ __forceinline__ uint32_t wc8_addr(uint32_t w, uint32_t base) {
  return __builtin_amdgcn_perm(w, base, 0x0C0C0000u | ((4u + K) << 8));
}

// One chunk for TB tokens: each codebook entry read from LDS serves every
// token (two dot2 per token); row r of token b adds its two products in
// dimension order.  Up to two tokens, all 16 reads are issued before the
// first product, so the wave has 16 LDS requests in flight instead of the
// few the compiler's own schedule keeps (measured 0.1 us faster per
// LLaMA-7B q/k/v/o call).  For four tokens the read results would push the
// kernels past the register budget of two workgroups per CU, so each read
// meets its products at once.
template <int TB>
__device__ __forceinline__ void wc8_chunk_tb(float (&acc)[TB][16], const u32x4 &w,
                                             const uint2 (&xj)[TB], const char *wcr, uint32_t base) {
  if constexpr (TB <= 2) {
    uint2 e[16];
#define WC8TB_RD(R, Q, K) e[R] = lds_u2(wcr, wc8_addr<K>(w[Q], base));
    WC8TB_RD(0, 0, 0) WC8TB_RD(1, 0, 1) WC8TB_RD(2, 0, 2) WC8TB_RD(3, 0, 3)
    WC8TB_RD(4, 1, 0) WC8TB_RD(5, 1, 1) WC8TB_RD(6, 1, 2) WC8TB_RD(7, 1, 3)
    WC8TB_RD(8, 2, 0) WC8TB_RD(9, 2, 1) WC8TB_RD(10, 2, 2) WC8TB_RD(11, 2, 3)
    WC8TB_RD(12, 3, 0) WC8TB_RD(13, 3, 1) WC8TB_RD(14, 3, 2) WC8TB_RD(15, 3, 3)
#undef WC8TB_RD
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        acc[b][r] = __builtin_amdgcn_fdot2(h2(xj[b].x), h2(e[r].x), acc[b][r], false);
        acc[b][r] = __builtin_amdgcn_fdot2(h2(xj[b].y), h2(e[r].y), acc[b][r], false);
      }
  } else {
#define WC8TB_ONE(R, Q, K)                                                           \
  {                                                                                  \
    const uint2 e = lds_u2(wcr, wc8_addr<K>(w[Q], base));                            \
    _Pragma("unroll") for (int b = 0; b < TB; ++b) {                                 \
      acc[b][R] = __builtin_amdgcn_fdot2(h2(xj[b].x), h2(e.x), acc[b][R], false);    \
      acc[b][R] = __builtin_amdgcn_fdot2(h2(xj[b].y), h2(e.y), acc[b][R], false);    \
    }                                                                                \
  }
    WC8TB_ONE(0, 0, 0) WC8TB_ONE(1, 0, 1) WC8TB_ONE(2, 0, 2) WC8TB_ONE(3, 0, 3)
    WC8TB_ONE(4, 1, 0) WC8TB_ONE(5, 1, 1) WC8TB_ONE(6, 1, 2) WC8TB_ONE(7, 1, 3)
    WC8TB_ONE(8, 2, 0) WC8TB_ONE(9, 2, 1) WC8TB_ONE(10, 2, 2) WC8TB_ONE(11, 2, 3)
    WC8TB_ONE(12, 3, 0) WC8TB_ONE(13, 3, 1) WC8TB_ONE(14, 3, 2) WC8TB_ONE(15, 3, 3)
#undef WC8TB_ONE
  }
}

// The 2 KiB codebook of the 8-bit kernels, for workgroups of 8 waves,
// fetched through the scalar data cache.  Thread t = 64 w + l of such a
// workgroup writes entry 8 w + l/8 + 64 u (u < 4) into the replicas, so wave
// w reads four 64-byte blocks with scalar loads (the codebook is not written
// during the kernel).  Scalar loads do not queue behind the wave's vector
// index loads: issued before them, and selected into lanes after them, the
// codebook reaches LDS sooner than through vector loads (measured 0.25 us
// per LLaMA-7B q/k/v/o call).
struct Cb8Scalar {
  uint32_t s[4][16];
};
__device__ __forceinline__ void cb8_scalar_issue(Cb8Scalar &c, const uint16_t *wc, int wave) {
  typedef const __attribute__((address_space(4))) uint32_t cu32;
  cu32 *cb = (cu32 *)wc;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) c.s[u][i] = cb[16 * wave + 128 * u + i];
}
// Lane l's entries 8 w + l/8 + 64 u, as the vector path would have loaded them.
__device__ __forceinline__ void cb8_scalar_select(const Cb8Scalar &c, int lane, uint2 (&ent)[4]) {
  const int q = lane >> 3;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t a = c.s[u][0], b = c.s[u][1];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      a = (q == k) ? c.s[u][2 * k] : a;
      b = (q == k) ? c.s[u][2 * k + 1] : b;
    }
    ent[u] = uint2{a, b};
  }
}

// TB: tokens per call the kernel is built for (1, 2 or 4; B <= TB).  A token
// past B loads the last token's x (in bounds) and is not stored.
template <int W, int PF, int TB>
__global__ void __launch_bounds__(W * 64) wc8_kernel(const WcArgs args) {
  constexpr int NT = W * 64;
  constexpr int RP = 2048 / NT;               // 16-byte replica stores per thread
  __shared__ __align__(16) char wcr[256 * 256];
  __shared__ float part[TB][W * 64];
  const WcMat M = load_wcmat(args);
  if ((int)blockIdx.x >= M.nwg) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = M.jsplit;
  const int rgl = wave / S, sg = wave % S;
  const int JT = M.J >> 6;
  const int NG = (M.N + 15) >> 4;
  const int rgw = (int)blockIdx.x * (W / S) + rgl;
  const int rg = min(rgw, NG - 1);
  const int seg = (JT + S - 1) / S;
  const int kbeg = min(sg * seg, JT), kend = min(kbeg + seg, JT);

  // 1. codebook entries for the replicas (8 waves and up to two tokens:
  //    scalar loads; four tokens keep the register budget of vector loads),
  //    then the first PF index chunks and x slices: every load is issued
  //    before the first wait
  constexpr bool kScalarCb = W == 8 && TB <= 2;
  uint2 ent[RP];
  Cb8Scalar cbs;
  if constexpr (kScalarCb) {
    cb8_scalar_issue(cbs, M.wc, wave);
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int u = 0; u < RP; ++u) ent[u] = reinterpret_cast<const uint2 *>(M.wc)[(threadIdx.x + u * NT) >> 3];
  }
  const uint8_t *wi = M.wi + (size_t)lane * 16;
  const size_t kstride = (size_t)NG * 1024;   // one 64-subvector tile of all row groups
  const uint8_t *wrg = wi + (size_t)rg * 1024;
  const uint2 *xg = reinterpret_cast<const uint2 *>(M.x) + lane;   // x_j, j = 64 k + lane
  size_t xt[TB];                              // token rows of x, in uint2 units
#pragma unroll
  for (int b = 0; b < TB; ++b) xt[b] = (size_t)min(b, M.B - 1) * M.J;
  u32x4 buf[PF];
  uint2 xbuf[PF][TB];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int k = min(kbeg + p, JT - 1);
    buf[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrg + (size_t)k * kstride));
#pragma unroll
    for (int b = 0; b < TB; ++b) xbuf[p][b] = xg[xt[b] + k * 64];
  }
  if constexpr (kScalarCb) {
    __builtin_amdgcn_sched_barrier(0);
    cb8_scalar_select(cbs, lane, ent);
  }
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int s = threadIdx.x + u * NT;       // entry s >> 3, copies 2 (s & 7) and + 1
    *reinterpret_cast<u32x4 *>(wcr + (s >> 3) * 256 + (s & 7) * 16) =
        u32x4{ent[u].x, ent[u].y, ent[u].x, ent[u].y};
  }
  __syncthreads();

  // 2. lookups: OC[j][c] = x_j . WC[c] formed per index, summed per row
  const uint32_t base = (uint32_t)(lane & 15) << 3;
  float acc[TB][16];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
  for (int k0 = kbeg; k0 < kend; k0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int k = k0 + p;
      const u32x4 cur = buf[p];
      uint2 xj[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) xj[b] = xbuf[p][b];
      // refill this slot with chunk k + PF (clamped: in bounds, unused)
      const int kn = min(k + PF, JT - 1);
      buf[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrg + (size_t)kn * kstride));
#pragma unroll
      for (int b = 0; b < TB; ++b) xbuf[p][b] = xg[xt[b] + kn * 64];
      if (k < kend) wc8_chunk_tb<TB>(acc, cur, xj, wcr, base);
    }
  }

  // 3. rows out: lane 4r holds row r of the 16 (segments added in order)
  float v[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) v[b] = wreduce_rows16(acc[b], lane);
  if (S > 1) {
#pragma unroll
    for (int b = 0; b < TB; ++b) part[b][wave * 64 + lane] = v[b];
    __syncthreads();
    if (sg != 0) return;
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      v[b] = part[b][wave * 64 + lane];
      for (int t = 1; t < S; ++t) v[b] += part[b][(wave + t) * 64 + lane];
    }
  }
  const int row = rgw * 16 + ((lane >> 2) & 15);
  if ((lane & 3) == 0 && rgw < NG && row < M.N) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
      if (b < M.B) store_y(M, (size_t)b * M.ldy + row, v[b]);
  }
}

// Raw buffer descriptors (gfx9 word 3), an offset past any buffer the
// kernels address, and the nontemporal cache-policy bit.
constexpr uint32_t kWcOutOfRange = 0x80000000u;
constexpr int kWcBufferWord3 = 0x00020000;
constexpr int kWcNontemporal = 2;

// The same walk for rows of at most 4 S chunks (K <= 8192 at S = 8): a wave's
// whole segment is requested at once, in two parts.  The codebook, the x
// slices and the first two chunks go out first; the other chunks only once
// the codebook has arrived and been written to LDS.  Issued together with
// the codebook, the whole layer's index stream held the codebook back
// behind it; issued one chunk per lookup pass, too little was in flight
// while the codebook was on its way.  Chunks past the segment load through
// a buffer descriptor with an out-of-range offset (zeros, no memory access)
// and are not looked up.  Sums are formed in the same order as wc8_kernel,
// so the two kernels give bitwise the same y for the same split.
// TB: tokens per call the kernel is built for (1, 2 or 4; the call's B <= TB,
// tokens past B read zeros and are not stored).  Every token's sums are
// formed in the same order as for one token.
// UNITS: the call merged matrices that share the codebook, x and shape into
// units (WcUnitArgs); mwi / my list the members' indices and outputs.
template <int W, int NCH, int PF0, int TB, bool UNITS>
__device__ __forceinline__ void wc8_burst_body(const WcArgs &args, const WcUnitArgs *ua) {
  constexpr int NT = W * 64;
  constexpr int RP = 2048 / NT;               // 16-byte replica stores per thread
  __shared__ __align__(16) char wcr[256 * 256];
  __shared__ float part[TB][W * 64];
  const int unit = blockIdx.y, bx = blockIdx.x;   // workgroup x of matrix (or unit) y
  const WcMat M = load_wcmat(args, unit);
  if (bx >= M.nwg) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lS = 31 - __builtin_clz((unsigned)M.jsplit);   // the split is a power of two
  const int S = 1 << lS;
  const int rgl = wave >> lS, sg = wave & (S - 1);
  const int JT = M.J >> 6;
  const int NG = (M.N + 15) >> 4;
  // Row group of the wave.  Matrices that share the codebook, x and their
  // shape are laid end to end (nmem > 1): row group rgall of the unit is
  // row group rgall mod NG of member rgall / NG, so one workgroup's staged
  // codebook and x serve rows of several of them.  Each row's sums keep the
  // order they have when its matrix is called alone.
  const int rgall = bx * (W >> lS) + rgl;
  int rgw = rgall;
  const uint8_t *wib = M.wi;
  float *yb = M.y;
  if constexpr (UNITS) {
    const int nmem = args.mat[unit].nmem, mem0 = args.mat[unit].mem0;
    if (nmem > 1) {
      const int mem = min(rgall / NG, nmem - 1);
      rgw = rgall - mem * NG;
      wib = ua->mwi[mem0 + mem];
      yb = ua->my[mem0 + mem];
    }
  }
  const int rg = min(rgw, NG - 1);
  const int seg = (JT + S - 1) >> lS;
  const int kbeg = min(sg * seg, JT), kend = min(kbeg + seg, JT);
  const uint32_t kstride = (uint32_t)NG * 1024u;   // one 64-subvector tile of all row groups
  const __amdgpu_buffer_rsrc_t rwi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(wib + (size_t)rg * 1024), (short)0, (int)(kstride * (uint32_t)JT),
      kWcBufferWord3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(M.x), (short)0, M.B * M.J * 8, kWcBufferWord3);
  auto wi_off = [&](int k) -> uint32_t {
    return k < kend ? (uint32_t)k * kstride + (uint32_t)lane * 16u : kWcOutOfRange;
  };
  auto x_off = [&](int k, int b) -> uint32_t {
    return (k < kend && b < M.B) ? (uint32_t)(b * M.J + k * 64 + lane) * 8u : kWcOutOfRange;
  };

  // 1. the codebook (up to two tokens: scalar loads; four tokens keep the
  //    register budget of vector loads), the x slices, the first PF0 chunks
  static_assert(W == 8, "the scalar codebook fetch serves workgroups of 8 waves");
  constexpr bool kScalarCb = TB <= 2;
  uint2 ent[RP];
  Cb8Scalar cbs;
  if constexpr (kScalarCb) {
    cb8_scalar_issue(cbs, M.wc, wave);
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int u = 0; u < RP; ++u) ent[u] = reinterpret_cast<const uint2 *>(M.wc)[(threadIdx.x + u * NT) >> 3];
  }
  u32x4 buf[NCH];
  uint2 xbuf[NCH][TB];
#pragma unroll
  for (int p = 0; p < NCH; ++p)
#pragma unroll
    for (int b = 0; b < TB; ++b)
      xbuf[p][b] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, x_off(kbeg + p, b), 0, 0));
#pragma unroll
  for (int p = 0; p < PF0; ++p)
    buf[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, wi_off(kbeg + p), 0, kWcNontemporal));
  // 2. replicas into LDS (waits for the codebook), then the rest of the segment
  if constexpr (kScalarCb) {
    __builtin_amdgcn_sched_barrier(0);
    cb8_scalar_select(cbs, lane, ent);
  }
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int s = threadIdx.x + u * NT;       // entry s >> 3, copies 2 (s & 7) and + 1
    *reinterpret_cast<u32x4 *>(wcr + (s >> 3) * 256 + (s & 7) * 16) =
        u32x4{ent[u].x, ent[u].y, ent[u].x, ent[u].y};
  }
  __builtin_amdgcn_sched_barrier(0);          // keep the remaining loads after the codebook wait
#pragma unroll
  for (int p = PF0; p < NCH; ++p)
    buf[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, wi_off(kbeg + p), 0, kWcNontemporal));
  __syncthreads();

  // 3. lookups in chunk order, each as soon as its indices arrive
  const uint32_t base = (uint32_t)(lane & 15) << 3;
  float acc[TB][16];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
#pragma unroll
  for (int p = 0; p < NCH; ++p)
    if (kbeg + p < kend) wc8_chunk_tb<TB>(acc, buf[p], xbuf[p], wcr, base);

  // 4. rows out: lane 4r holds row r of the 16 (segments added in order)
  float v[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) v[b] = wreduce_rows16(acc[b], lane);
  if (S > 1) {
#pragma unroll
    for (int b = 0; b < TB; ++b) part[b][wave * 64 + lane] = v[b];
    __syncthreads();
    if (sg != 0) return;
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      v[b] = part[b][wave * 64 + lane];
      for (int t = 1; t < S; ++t) v[b] += part[b][(wave + t) * 64 + lane];
    }
  }
  const int row = rgw * 16 + ((lane >> 2) & 15);
  if ((lane & 3) == 0 && rgw < NG && row < M.N) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
      if (b < M.B) store_y(yb, M.yf16, (size_t)b * M.ldy + row, v[b]);
  }
}

template <int W, int NCH, int PF0, int TB>
__global__ void __launch_bounds__(W * 64) wc8_burst_kernel(const WcArgs args) {
  wc8_burst_body<W, NCH, PF0, TB, false>(args, nullptr);
}

template <int W, int NCH, int PF0, int TB>
__global__ void __launch_bounds__(W * 64) wc8_burst_units_kernel(const WcUnitArgs args) {
  wc8_burst_body<W, NCH, PF0, TB, true>(args.a, &args);
}

// --------------------------------------------------------------------------
// d = 4, n = 8: gate and up projections with the SiLU-gated product fused
// --------------------------------------------------------------------------
// y[b][r] = silu(gate x_b)[r] * (up x_b)[r], silu(z) = z / (1 + e^-z), for
// the gate/up pairs of a SiLU-gated MLP that share x.  The burst kernel's
// walk, with the workgroup's row-group slots taken in pairs: slot 2q looks up
// gate rows, slot 2q + 1 the same rows of up, so every wave does the work of
// a plain call.  The up codebook's 16 copies sit in the half of each
// 256-byte LDS row the gate copies leave free (bytes 128-255, banks 32-63),
// so an up lookup's address is a gate lookup's with bit 7 set.  Both sums
// are formed in the one-matrix order; the two meet in LDS and only their
// gated product is stored.
template <int W, int NCH, int PF0, int TB>
__global__ void __launch_bounds__(W * 64) wc8_swiglu_kernel(const WcPairArgs args) {
  constexpr int NT = W * 64;
  constexpr int RP = 2048 / NT;               // 16-byte replica stores per thread and codebook
  __shared__ __align__(16) char wcr[256 * 256];
  __shared__ float part[TB][W * 64];
  __shared__ float upv[TB][W / 2][64];        // up row sums of each slot pair
  const WcMat M = load_wcmat(args.a);
  if ((int)blockIdx.x >= M.nwg) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lS = 31 - __builtin_clz((unsigned)M.jsplit);
  const int S = 1 << lS;
  const int slot = wave >> lS, sg = wave & (S - 1);
  const int pr = slot >> 1, up = slot & 1;    // output row group of the workgroup, matrix
  const int JT = M.J >> 6;
  const int NG = (M.N + 15) >> 4;
  const int rgw = (int)blockIdx.x * (W >> (lS + 1)) + pr;
  const int rg = min(rgw, NG - 1);
  const int seg = (JT + S - 1) >> lS;
  const int kbeg = min(sg * seg, JT), kend = min(kbeg + seg, JT);
  const uint32_t kstride = (uint32_t)NG * 1024u;
  const uint8_t *wsel = up ? args.wi2[blockIdx.y] : M.wi;
  const __amdgpu_buffer_rsrc_t rwi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(wsel + (size_t)rg * 1024), (short)0, (int)(kstride * (uint32_t)JT),
      kWcBufferWord3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(M.x), (short)0, M.B * M.J * 8, kWcBufferWord3);
  auto wi_off = [&](int k) -> uint32_t {
    return k < kend ? (uint32_t)k * kstride + (uint32_t)lane * 16u : kWcOutOfRange;
  };
  auto x_off = [&](int k, int b) -> uint32_t {
    return (k < kend && b < M.B) ? (uint32_t)(b * M.J + k * 64 + lane) * 8u : kWcOutOfRange;
  };

  uint2 eg[RP], eu[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    eg[u] = reinterpret_cast<const uint2 *>(M.wc)[(threadIdx.x + u * NT) >> 3];
    eu[u] = reinterpret_cast<const uint2 *>(args.wc2[blockIdx.y])[(threadIdx.x + u * NT) >> 3];
  }
  u32x4 buf[NCH];
  uint2 xbuf[NCH][TB];
#pragma unroll
  for (int p = 0; p < NCH; ++p)
#pragma unroll
    for (int b = 0; b < TB; ++b)
      xbuf[p][b] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, x_off(kbeg + p, b), 0, 0));
#pragma unroll
  for (int p = 0; p < PF0; ++p)
    buf[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, wi_off(kbeg + p), 0, kWcNontemporal));
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int s = threadIdx.x + u * NT;       // entry s >> 3, copies 2 (s & 7) and + 1
    char *row = wcr + (s >> 3) * 256 + (s & 7) * 16;
    *reinterpret_cast<u32x4 *>(row) = u32x4{eg[u].x, eg[u].y, eg[u].x, eg[u].y};
    *reinterpret_cast<u32x4 *>(row + 128) = u32x4{eu[u].x, eu[u].y, eu[u].x, eu[u].y};
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = PF0; p < NCH; ++p)
    buf[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, wi_off(kbeg + p), 0, kWcNontemporal));
  __syncthreads();

  const uint32_t base = ((uint32_t)(lane & 15) << 3) | ((uint32_t)up << 7);
  float acc[TB][16];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
#pragma unroll
  for (int p = 0; p < NCH; ++p)
    if (kbeg + p < kend) wc8_chunk_tb<TB>(acc, buf[p], xbuf[p], wcr, base);

  float v[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) v[b] = wreduce_rows16(acc[b], lane);
  if (S > 1) {
#pragma unroll
    for (int b = 0; b < TB; ++b) part[b][wave * 64 + lane] = v[b];
    __syncthreads();
    if (sg == 0) {
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        v[b] = part[b][wave * 64 + lane];
        for (int t = 1; t < S; ++t) v[b] += part[b][(wave + t) * 64 + lane];
      }
    }
  }
  // the up sums meet the gate sums of the same rows
  if (sg == 0 && up) {
#pragma unroll
    for (int b = 0; b < TB; ++b) upv[b][pr][lane] = v[b];
  }
  __syncthreads();
  if (sg != 0 || up) return;
  const int row = rgw * 16 + ((lane >> 2) & 15);
  if ((lane & 3) == 0 && rgw < NG && row < M.N) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
      if (b < M.B) store_y(M, (size_t)b * M.ldy + row, v[b] / (1.f + expf(-v[b])) * upv[b][pr][lane]);
  }
}

// --------------------------------------------------------------------------
// d = 8, n = 16, up to 16 tokens: the codebook split by dimension
// --------------------------------------------------------------------------
// y[b][r] = sum_t sum_j x[b][8 j + t] WC[c_rj][t]: for each dimension t the
// table WC[.][t] (65536 fp16, 128 KiB) fits in LDS, and the contraction over
// j runs on the matrix cores with x's dimension-t values as A and the looked-
// up table values as B.  The codebook comes in its load-time dimension-major
// layout (vq_repack_wc: wct[t][c] = WC[c][t]); a pre-pass writes x's
// dimension-t values in the order the A operand reads them:
//   xt[t][b][jb][s][i] (16 B runs) = x[b][8 (32 jb + s + 4 i) + t]
__global__ void wc16_prep_kernel(const Wc16tArgs args) {
  const WcMat &M = args.a.mat[blockIdx.y];
  uint16_t *xt = args.xt[blockIdx.y];
  const int J = M.J, JB = J >> 5;
  const int64_t nx = (int64_t)M.B * J;
  for (int64_t f = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; f < nx;
       f += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(f / J), j = (int)(f % J);
    const u32x4 v = reinterpret_cast<const u32x4 *>(M.x + (size_t)b * J * 8)[j];
    const int jb = j >> 5, r = j & 31, sub = r & 3, i = r >> 2;
    const size_t pos = ((size_t)b * JB + jb) * 32 + sub * 8 + i;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      xt[(size_t)t * M.B * J + pos] = (uint16_t)(v[t >> 1] >> (16 * (t & 1)));
  }
}

// Load-time layout of a (d = 8, n = 16) codebook: wct[t][c] = WC[c][t].
__global__ void repack_wc16_kernel(const uint16_t *wc, uint16_t *wct) {
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < 65536; c += gridDim.x * blockDim.x) {
    const u32x4 v = reinterpret_cast<const u32x4 *>(wc)[c];
#pragma unroll
    for (int t = 0; t < 8; ++t) wct[(size_t)t * 65536 + c] = (uint16_t)(v[t >> 1] >> (16 * (t & 1)));
  }
}

template <int W, int NBLK>
__global__ void __launch_bounds__(W * 64) wc16t_kernel(const Wc16tArgs args) {
  constexpr int NT = W * 64;
  __shared__ __align__(16) _Float16 tbl[65536];
  // A flat grid of the call's workgroups, matrix after matrix: workgroup
  // blockIdx.x is workgroup b of matrix m.  One workgroup fills a CU, and
  // workgroups go to the XCDs in turn, so a grid without empty workgroups
  // gives every XCD the same count (a 2-D grid padded to the largest matrix
  // put 33 on some XCDs of 32 CUs and ran them in two rounds).
  int m = 0, b = (int)blockIdx.x;
  while (m + 1 < args.a.count && b >= args.a.mat[m].nwg) {
    b -= args.a.mat[m].nwg;
    ++m;
  }
  const WcMat M = load_wcmat(args.a, m);
  if (b >= M.nwg) return;
  const uint16_t *wct = M.wc;                         // dimension-major (vq_repack_wc)
  const uint16_t *xt = args.xt[m];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // S waves per row group, W / S row groups per workgroup; the W mod S
  // waves past them fill tables and wait at the barriers but own no rows
  // (the divisions by the run-time S are made wave-uniform again, so that
  // the segment bounds stay scalar and the block loop branches on them)
  const int S = M.jsplit;
  const int rpg = __builtin_amdgcn_readfirstlane(W / S);
  const int rgl = __builtin_amdgcn_readfirstlane(wave / S);
  const int sg = wave - rgl * S;
  const bool active = rgl < rpg;
  const int JB = M.J >> 5;
  const int NG = (M.N + 15) >> 4;
  const int rgw = b * rpg + rgl;
  const int rg = min(rgw, NG - 1);
  const int seg = __builtin_amdgcn_readfirstlane((JB + S - 1) / S);
  const int kbeg = active ? min(sg * seg, JB) : JB, kend = min(kbeg + seg, JB);
  const int tok = lane & 15, sub = lane >> 4;
  const bool has_tok = tok < M.B;

  // the wave's index blocks, all in registers for the eight passes
  const __amdgpu_buffer_rsrc_t rwi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(M.wi + (size_t)rg * JB * 1024), (short)0, JB * 1024, kWcBufferWord3);
  u32x4 ib[NBLK];
#pragma unroll
  for (int p = 0; p < NBLK; ++p) {
    const uint32_t off = kbeg + p < kend ? (uint32_t)(kbeg + p) * 1024u + (uint32_t)lane * 16u : kWcOutOfRange;
    ib[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, off, 0, kWcNontemporal));
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const size_t xplane = (size_t)M.B * M.J;          // fp16 values per dimension plane of xt
  const uint16_t *xrow = xt + ((size_t)(has_tok ? tok : 0) * JB) * 32 + sub * 8;
  for (int t = 0; t < 8; ++t) {
    __syncthreads();                                 // the previous table is no longer read
    {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(wct + (size_t)t * 65536);
      u32x4 *dst = reinterpret_cast<u32x4 *>(tbl);
#pragma unroll
      for (int u = 0; u < 8192 / NT; ++u) dst[threadIdx.x + u * NT] = src[threadIdx.x + u * NT];
    }
    __syncthreads();
    const uint16_t *xp = xrow + (size_t)t * xplane;
    // an opaque zero per pass keeps the 8 NBLK table addresses from being
    // computed once before the passes and held in registers
    uint32_t z;
    __asm__ volatile("s_mov_b32 %0, 0" : "=s"(z));
    const char *tb = reinterpret_cast<const char *>(tbl);
#pragma unroll
    for (int p = 0; p < NBLK; ++p) {
      if (kbeg + p < kend) {
        const u32x4 xv = has_tok ? *reinterpret_cast<const u32x4 *>(xp + (size_t)(kbeg + p) * 32)
                                 : u32x4{0u, 0u, 0u, 0u};
        half8_t b;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          b[i] = *reinterpret_cast<const _Float16 *>(tb + 2 * (((ib[p][i >> 1] | z) >> (16 * (i & 1))) & 0xffffu));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, xv), b, acc, 0, 0, 0);
      }
    }
  }
  if (S > 1) {                                       // segments added in order through LDS
    __syncthreads();
    f32x4_t *part = reinterpret_cast<f32x4_t *>(tbl);
    part[wave * 64 + lane] = acc;
    __syncthreads();
    if (!active || sg != 0) return;
    for (int q = 1; q < S; ++q) {
      const f32x4_t o = part[(wave + q) * 64 + lane];
      acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
    }
  }
  if (active && rgw < NG) {
    const int row = rgw * 16 + tok;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = sub * 4 + i;
      if (tt < M.B && row < M.N) store_y(M, (size_t)tt * M.ldy + row, acc[i]);
    }
  }
}

// --------------------------------------------------------------------------
// device layouts
// --------------------------------------------------------------------------
// canonical 12-bit rows ([N] rows of J indices, LSB-first bit stream, each row
// 1.5 J bytes) -> tile-16x64-12: chunk (rg, jt), lane l = subvector 64 jt + l,
// 24 bytes = indices of rows 16 rg + i (i < 16) at bits [12 i, 12 i + 12)
__global__ void repack_wi12_kernel(const uint8_t *canon, int N, int J, uint8_t *dev) {
  const int NG = (N + 15) >> 4, JT = J >> 6;
  const int64_t total = (int64_t)NG * JT * 64;
  const int64_t rb = (int64_t)J * 3 / 2;   // bytes per canonical row
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(e & 63);
    const int64_t chunk = e >> 6;
    const int jt = (int)(chunk % JT);
    const int rg = (int)(chunk / JT);
    const int j = jt * 64 + l;
    uint32_t out[6] = {0u, 0u, 0u, 0u, 0u, 0u};
    for (int i = 0; i < 16; ++i) {
      const int r = rg * 16 + i;
      uint32_t c = 0u;
      if (r < N) {
        const int64_t bit = (int64_t)j * 12;
        const uint8_t *p = canon + (int64_t)r * rb + (bit >> 3);
        const uint32_t two = (uint32_t)p[0] | ((uint32_t)p[1] << 8);
        c = (two >> (bit & 7)) & 0xfffu;
      }
      const int q = i >> 3, ib = (i & 7) * 12;     // 96-bit half q, bit offset ib
      const int w = ib >> 5, s = ib & 31;
      out[q * 3 + w] |= c << s;
      if (s > 20) out[q * 3 + w + 1] |= c >> (32 - s);
    }
    uint8_t *d = dev + e * 24;
    for (int q = 0; q < 6; ++q) *reinterpret_cast<uint32_t *>(d + 4 * q) = out[q];
  }
}

// canonical 16-bit rows (little-endian uint16, [N][J]) -> tile-16x32-16:
// chunk (rg, jb), lane l holds the indices of row 16 rg + l%16 at subvectors
// 32 jb + l/16 + 4 q, q < 8 (the q-th is the lane's B-operand value at
// k = 8 (l/16) + q of the block's MFMA)
__global__ void repack_wi16_kernel(const uint8_t *canon, int N, int J, uint8_t *dev) {
  const int NG = (N + 15) >> 4, JB = J >> 5;
  const int64_t total = (int64_t)NG * JB * 64;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(e & 63);
    const int64_t chunk = e >> 6;
    const int jb = (int)(chunk % JB);
    const int rg = (int)(chunk / JB);
    const int r = rg * 16 + (l & 15);
    uint16_t v[8];
    for (int q = 0; q < 8; ++q) {
      const int j = jb * 32 + (l >> 4) + 4 * q;
      v[q] = (r < N) ? reinterpret_cast<const uint16_t *>(canon)[(int64_t)r * J + j] : (uint16_t)0;
    }
    uint16_t *d = reinterpret_cast<uint16_t *>(dev + e * 16);
    for (int q = 0; q < 8; ++q) d[q] = v[q];
  }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
static int wgrid(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

int launch_wc12(const WcArgs &a, int grid_x, int max_j, void *stream) {
  (void)max_j;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL((wc12_kernel<WC12_W, WC12_PF>), dim3(grid_x, a.count), dim3(WC12_W * 64), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_wc8_swiglu(const WcPairArgs &a, int grid_x, int waves, int B, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // report only this launch's error
  const dim3 grid(grid_x, a.a.count);
  if (waves == WC8_W && B == 1)
    hipLaunchKernelGGL((wc8_swiglu_kernel<WC8_W, WC8_NCH, 2, 1>), grid, dim3(WC8_W * 64), 0, st, a);
  else if (waves == WC8_W && B == 2)
    hipLaunchKernelGGL((wc8_swiglu_kernel<WC8_W, WC8_NCH, 2, 2>), grid, dim3(WC8_W * 64), 0, st, a);
  else if (waves == 2 * WC8_W && B == 1)
    hipLaunchKernelGGL((wc8_swiglu_kernel<2 * WC8_W, WC8_NCH, 2, 1>), grid, dim3(2 * WC8_W * 64), 0, st, a);
  else if (waves == 2 * WC8_W && B == 2)
    hipLaunchKernelGGL((wc8_swiglu_kernel<2 * WC8_W, WC8_NCH, 2, 2>), grid, dim3(2 * WC8_W * 64), 0, st, a);
  else
    return (int)hipErrorInvalidConfiguration;
  return (int)hipGetLastError();
}

int launch_wc8_units(const WcUnitArgs &a, int grid_x, int B, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // report only this launch's error
  const dim3 grid(grid_x, a.a.count), block(WC8_W * 64);
  if (B == 1)
    hipLaunchKernelGGL((wc8_burst_units_kernel<WC8_W, WC8_NCH, 2, 1>), grid, block, 0, st, a);
  else if (B == 2)
    hipLaunchKernelGGL((wc8_burst_units_kernel<WC8_W, WC8_NCH, 2, 2>), grid, block, 0, st, a);
  else if (B <= 4)
    hipLaunchKernelGGL((wc8_burst_units_kernel<WC8_W, WC8_NCH, 2, 4>), grid, block, 0, st, a);
  else
    return (int)hipErrorInvalidConfiguration;
  return (int)hipGetLastError();
}

int launch_wc8(const WcArgs &a, int grid_x, int waves, bool burst, int B, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // report only this launch's error
  if (B < 1 || B > 4) return (int)hipErrorInvalidConfiguration;
  const dim3 grid(grid_x, a.count), block(WC8_W * 64);
  if (waves == 4 && B == 1)
    hipLaunchKernelGGL((wc8_kernel<4, 1, 1>), grid, dim3(4 * 64), 0, st, a);
  else if (burst && B == 1)
    hipLaunchKernelGGL((wc8_burst_kernel<WC8_W, WC8_NCH, 2, 1>), grid, block, 0, st, a);
  else if (burst && B == 2)
    hipLaunchKernelGGL((wc8_burst_kernel<WC8_W, WC8_NCH, 2, 2>), grid, block, 0, st, a);
  else if (burst)
    hipLaunchKernelGGL((wc8_burst_kernel<WC8_W, WC8_NCH, 2, 4>), grid, block, 0, st, a);
  else if (B == 1)
    hipLaunchKernelGGL((wc8_kernel<WC8_W, 2, 1>), grid, block, 0, st, a);
  else if (B == 2)
    hipLaunchKernelGGL((wc8_kernel<WC8_W, 2, 2>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((wc8_kernel<WC8_W, 2, 4>), grid, block, 0, st, a);
  return (int)hipGetLastError();
}

int launch_repack_wc16(const uint16_t *wc, uint16_t *wct, void *stream) {
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(repack_wc16_kernel, dim3(256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     wc, wct);
  return (int)hipGetLastError();
}

int launch_wc16t(const Wc16tArgs &a, int grid_x, int prep_blocks, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(wc16_prep_kernel, dim3(prep_blocks, a.a.count), dim3(256), 0, st, a);
  hipLaunchKernelGGL((wc16t_kernel<16, 16>), dim3(grid_x), dim3(16 * 64), 0, st, a);
  return (int)hipGetLastError();
}


int launch_repack_wi12(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream) {
  const int64_t total = (int64_t)((N + 15) >> 4) * (J >> 6) * 64;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(repack_wi12_kernel, dim3(wgrid(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), canon, N, J, dev);
  return (int)hipGetLastError();
}

int launch_repack_wi16(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream) {
  const int64_t total = (int64_t)((N + 15) >> 4) * (J >> 5) * 64;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(repack_wi16_kernel, dim3(wgrid(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), canon, N, J, dev);
  return (int)hipGetLastError();
}

}  // namespace vqd
