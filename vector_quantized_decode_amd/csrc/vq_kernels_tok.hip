// HIP kernel of libvqd for several tokens per call at d = 4, n = 8 (gfx950):
// the output codebook is kept virtual -- each looked-up entry WC[c] meets
// every token's subvector x_b,j -- and the token contraction runs on the
// matrix cores.
//
// Source, cited by page title and section:
//   [EVA]  "EVA: Accelerating LLM Decoding via an Efficient Vector
//          Quantization Architecture" -- explainer page, technical summary,
//          section 2.A (input-codebook products form the output codebook;
//          lookups into it by the weight indices) and section 2.B (the
//          codebooks stay on chip while indices stream in tiles).
#include <hip/hip_runtime.h>

#include "vq_internal.h"

namespace vqd {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every record: loads zeros
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNontemporal = 2;

__device__ __forceinline__ uint2 lds_u2(const char *base, uint32_t byte_addr) {
  return *reinterpret_cast<const uint2 *>(base + byte_addr);
}

// The descriptor of this workgroup's matrix, every field read before the
// first use so the scalar loads share one round trip.
__device__ __forceinline__ WcMat load_mat(const WcArgs &args) {
  const WcMat &R = args.mat[blockIdx.y];
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
  __asm__ volatile("" ::"s"(M.wi), "s"(M.wc), "s"(M.x), "s"(M.y), "s"(M.J), "s"(M.N), "s"(M.B),
                   "s"(M.ldy), "s"(M.nwg), "s"(M.jsplit));
  return M;
}

// --------------------------------------------------------------------------
// d = 4, n = 8, up to 16 tokens, on the matrix cores
// --------------------------------------------------------------------------
// With several tokens each looked-up entry WC[c_rj] meets every token's x_j,
// so 16 rows x 16 tokens x 8 subvectors (32 weights) form one
// v_mfma_f32_16x16x32_f16: x's tokens as A, the rows' looked-up entries as
// B.  B wants a lane per row -- lane l serves row l % 16 and subvectors
// 16 (l / 16) + q, q < 16, of a 64-subvector column -- so WI is laid out
// in row tiles: chunk (column k, row group rg) is 1 KiB, and its 16 bytes at
// 16 l are those 16 indices of lane l (consecutive bytes of the canonical
// row), so a wave's chunk is one contiguous 1 KiB read.  The codebook sits
// in LDS in 32 copies (entry c, copy k at byte 256 c + 8 k) and lane l reads
// copy l % 32: the 32 lanes of one LDS read pass reach 32 different bank
// pairs whatever the indices are ([EVA] 2.A).  A wave owns RW row groups and
// one segment of the columns (S waves per row group, added in order through
// LDS); a column's x operands (8 KiB for the wave at 16 tokens) are loaded
// once for its RW row groups, and the next column's indices and x are
// requested before the current column's lookups.
//
// x's operands.  Lane (m, g) (token m = l % 16, k-group g = l / 16) needs
// block g of token m's column slice -- 128 bytes, eight 16-byte pieces, piece
// q the A operand of the q-th product.  Loaded that way, each load would
// touch 64 different lines; instead load i gives lane (m, g) piece
// g + 4 (i & 1) of block i >> 1, so the four lanes of a token read 64
// contiguous bytes, and a 4 x 4 exchange among those lanes (two stages of
// lane swaps, 32 and 16 lanes apart) hands every lane its own block.
__device__ __forceinline__ uint32_t wc8t_addr(uint32_t w, uint32_t base, uint32_t k) {
  return __builtin_amdgcn_perm(w, base, 0x0C0C0000u | ((4u + k) << 8));
}
// X[b] = (v[2b], v[2b+1]).  Lanes 32-63 of X[a] take lanes 0-31 of X[b] and
// lanes 0-31 of X[b] take lanes 32-63 of X[a] (STAGE 32), or the same between
// the odd and even 16-lane rows (STAGE 16).
template <int STAGE>
__device__ __forceinline__ void wc8t_swap(u32x4 (&v)[8], int a, int b) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if constexpr (STAGE == 32) {
        auto r = __builtin_amdgcn_permlane32_swap(v[2 * a + h][d], v[2 * b + h][d], false, false);
        v[2 * a + h][d] = r[0];
        v[2 * b + h][d] = r[1];
      } else {
        auto r = __builtin_amdgcn_permlane16_swap(v[2 * a + h][d], v[2 * b + h][d], false, false);
        v[2 * a + h][d] = r[0];
        v[2 * b + h][d] = r[1];
      }
    }
}
// After the loads: lane (m, g) holds, as X[b], pieces g and g + 4 of block b.
// After the exchange: X[g'] holds pieces g' and g' + 4 of block g, so piece q
// is v[2 q] for q < 4 and v[2 (q - 4) + 1] for q >= 4.
__device__ __forceinline__ void wc8t_exchange(u32x4 (&v)[8]) {
  wc8t_swap<32>(v, 0, 2);
  wc8t_swap<32>(v, 1, 3);
  wc8t_swap<16>(v, 0, 1);
  wc8t_swap<16>(v, 2, 3);
}

template <int W, int RW>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4))) wc8t_kernel(const WcArgs args) {
  constexpr int NT = W * 64;
  constexpr int RP = 4096 / NT;               // 16-byte replica stores per thread
  __shared__ __align__(16) char wcr[256 * 256];
  const WcMat M = load_mat(args);
  if ((int)blockIdx.x >= M.nwg) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lS = 31 - __builtin_clz((unsigned)M.jsplit);   // the split is a power of two
  const int S = 1 << lS;
  const int slot = wave >> lS, sg = wave & (S - 1);
  const int JT = M.J >> 6;
  const int rg0 = ((int)blockIdx.x * (W >> lS) + slot) * RW;
  const int seg = (JT + S - 1) >> lS;
  const int kbeg = min(sg * seg, JT), kend = min(kbeg + seg, JT);
  const int m16 = lane & 15, g = lane >> 4;
  const int NG = (M.N + 15) >> 4;
  const __amdgpu_buffer_rsrc_t rwi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(M.wi), (short)0, NG * 16 * M.J, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(M.x), (short)0, M.B * M.J * 8, kBufferWord3);
  // row groups past the matrix, columns past the segment and tokens past B
  // read zeros (rows past N within the last group are zero in the layout)
  // (a wave-uniform select of the base, then the lane's offset: no branch,
  // so the scalar codebook loads stay ahead of these loads)
  auto wi_off = [&](int r, int k) -> uint32_t {
    const int rg = rg0 + r;
    const bool in = (k < kend) & (rg < NG);
    const uint32_t b = in ? ((uint32_t)k * (uint32_t)NG + (uint32_t)rg) * 1024u : kOutOfRange;
    return b + (uint32_t)lane * 16u;
  };
  auto x_off = [&](int k, int i) -> uint32_t {
    return (k < kend && m16 < M.B)
               ? (uint32_t)(m16 * M.J + k * 64) * 8u + (uint32_t)(128 * (i >> 1) + 16 * (g + 4 * (i & 1)))
               : kOutOfRange;
  };

  // 1. codebook entries for the replicas, through the scalar data cache:
  //    thread 64 w + l replicates entries 4 w + l / 16 + 32 u (u < 8), so
  //    wave w reads the eight 32-byte runs at entry 4 w + 32 u with scalar
  //    loads, issued before the vector loads of the first column (they do
  //    not queue behind those), and each lane picks its entry of each run
  //    after them.  Then the first column's indices and x.
  static_assert(W == 8 && RP == 8, "the scalar codebook fetch serves workgroups of 8 waves");
  typedef const __attribute__((address_space(4))) uint32_t cu32;
  cu32 *cbs = (cu32 *)M.wc;
  uint32_t sc[RP][8];
#pragma unroll
  for (int u = 0; u < RP; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[u][i] = cbs[8 * wave + 64 * u + i];
  __builtin_amdgcn_sched_barrier(0);
  u32x4 ib[RW], xa[8];
#pragma unroll
  for (int r = 0; r < RW; ++r)
    ib[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, wi_off(r, kbeg), 0, kNontemporal));
#pragma unroll
  for (int q = 0; q < 8; ++q)
    xa[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off(kbeg, q), 0, 0));
  __builtin_amdgcn_sched_barrier(0);
  uint2 ent[RP];
  {
    const int q = lane >> 4;
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      uint32_t a = sc[u][0], b = sc[u][1];
#pragma unroll
      for (int k = 1; k < 4; ++k) {
        a = (q == k) ? sc[u][2 * k] : a;
        b = (q == k) ? sc[u][2 * k + 1] : b;
      }
      ent[u] = uint2{a, b};
    }
  }
  // 2. replicas into LDS: entry s >> 4, copies 2 (s & 15) and + 1
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int s = threadIdx.x + u * NT;
    *reinterpret_cast<u32x4 *>(wcr + (s >> 4) * 256 + (s & 15) * 16) = u32x4{ent[u].x, ent[u].y, ent[u].x, ent[u].y};
  }
  __syncthreads();

  // 3. columns in order: request the next, then look up and multiply this one
  const uint32_t base = (uint32_t)(lane & 31) << 3;
  f32x4_t acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = kbeg; k < kend; ++k) {
    // this column's x (requested one column earlier) to the product order,
    // then the next column's requests, kept ahead of the lookups
    wc8t_exchange(xa);
    u32x4 ibn[RW], xn[8];
#pragma unroll
    for (int r = 0; r < RW; ++r)
      ibn[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, wi_off(r, k + 1), 0, kNontemporal));
#pragma unroll
    for (int q = 0; q < 8; ++q)
      xn[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off(k + 1, q), 0, 0));
    __builtin_amdgcn_sched_barrier(0);
    // product (q, r) in order q-major; its two entries (subvectors 16 g + 2 q
    // and + 1: bytes 2 (q & 1) and + 1 of word q >> 1) are read one product
    // ahead, so each LDS read overlaps the previous product
    auto entries = [&](int q, int r) -> u32x4 {
      const uint32_t w = ib[r][q >> 1];
      const uint2 e0 = lds_u2(wcr, wc8t_addr(w, base, 2u * (q & 1)));
      const uint2 e1 = lds_u2(wcr, wc8t_addr(w, base, 2u * (q & 1) + 1u));
      return u32x4{e0.x, e0.y, e1.x, e1.y};
    };
    u32x4 bnext = entries(0, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const u32x4 bw = bnext;
        if (q * RW + r + 1 < 8 * RW) bnext = entries((q * RW + r + 1) / RW, (q * RW + r + 1) % RW);
        __builtin_amdgcn_sched_barrier(0);     // the next reads stay ahead of this product
        const u32x4 xq = xa[q < 4 ? 2 * q : 2 * (q - 4) + 1];
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, xq),
                                                        __builtin_bit_cast(half8_t, bw), acc[r], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) ib[r] = ibn[r];
#pragma unroll
    for (int q = 0; q < 8; ++q) xa[q] = xn[q];
  }

  // 4. segments added in order; lane l holds tokens 4 (l / 16) + i of row l % 16
  if (S > 1) {
    __syncthreads();                                 // the codebook is no longer read
    f32x4_t *part = reinterpret_cast<f32x4_t *>(wcr);
#pragma unroll
    for (int r = 0; r < RW; ++r) part[(r * W + wave) * 64 + lane] = acc[r];
    __syncthreads();
    if (sg != 0) return;
#pragma unroll
    for (int r = 0; r < RW; ++r)
      for (int t = 1; t < S; ++t) {
        const f32x4_t o = part[(r * W + wave + t) * 64 + lane];
        acc[r][0] += o[0]; acc[r][1] += o[1]; acc[r][2] += o[2]; acc[r][3] += o[3];
      }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = (rg0 + r) * 16 + m16;
    if (row < M.N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = g * 4 + i;
        if (tt < M.B) M.y[(size_t)tt * M.ldy + row] = acc[r][i];
      }
    }
  }
}

// canonical 8-bit rows ([N][J] bytes) -> row tiles: chunk (column k, row
// group rg) at (k NG + rg) KiB, its 16 bytes at 16 l = row 16 rg + l % 16,
// subvectors 64 k + 16 (l / 16) .. + 15 (zeros for rows past N)
__global__ void repack_wi8_rows_kernel(const uint8_t *canon, int N, int J, uint8_t *dev) {
  const int NG = (N + 15) >> 4;
  const int64_t total = (int64_t)(J >> 6) * NG * 64;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(e & 63);
    const int64_t chunk = e >> 6;
    const int rg = (int)(chunk % NG);
    const int k = (int)(chunk / NG);
    const int row = rg * 16 + (l & 15);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < N) v = *reinterpret_cast<const u32x4 *>(canon + (size_t)row * J + k * 64 + (l >> 4) * 16);
    *reinterpret_cast<u32x4 *>(dev + e * 16) = v;
  }
}

}  // namespace

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
int launch_repack_wi8_rows(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream) {
  const int64_t total = (int64_t)(J >> 6) * ((N + 15) >> 4) * 64;
  int64_t blocks = (total + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(repack_wi8_rows_kernel, dim3((int)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), canon, N, J, dev);
  return (int)hipGetLastError();
}

int launch_wc8t(const WcArgs &a, int grid_x, int rw, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // report only this launch's error
  const dim3 grid(grid_x, a.count), block(TK_W * 64);
  if (rw == 4)
    hipLaunchKernelGGL((wc8t_kernel<TK_W, 4>), grid, block, 0, st, a);
  else if (rw == 2)
    hipLaunchKernelGGL((wc8t_kernel<TK_W, 2>), grid, block, 0, st, a);
  else if (rw == 1)
    hipLaunchKernelGGL((wc8t_kernel<TK_W, 1>), grid, block, 0, st, a);
  else
    return (int)hipErrorInvalidConfiguration;
  return (int)hipGetLastError();
}

}  // namespace vqd
