// HIP kernels of libvqd for gfx950 (CDNA4, wave64).
//
// Sources, cited by page title and section:
//   [EVA]  "EVA: Accelerating LLM Decoding via an Efficient Vector
//          Quantization Architecture" -- explainer page, technical summary,
//          sections 2.A (input-codebook products form the output codebook OC;
//          lookups into OC are arranged so that simultaneous accesses fall in
//          different memory banks) and 2.B (an epilogue unit performs the
//          lookups and sums them with adder trees; the codebooks stay on chip
//          while indices stream in tiles).
//   [EDGE] "Replacing MatMul with SRAM lookup: a 3-bit edge inference
//          architecture" -- article page, section details (randomized
//          Hadamard rotation, 1-bit sign residual with one fp16 scale per
//          group of 128 weights, LUT inference with bit operations).
//
// This file holds the lookup GEMV with a materialized output-codebook tile
// (used for the rotated 8-bit matrices with a 1-bit sign residual), the
// rotation kernel for large Hadamard blocks, the explicit OC build, and the
// packing / layout helpers.  The plain GEMVs (no residual) keep the output
// codebook virtual: vq_kernels_wc.hip.
//
// How the residual lookup GEMV maps onto a CDNA4 compute unit (d = 4, n = 8,
// B = 1):
//   * A workgroup owns one tile of 64 subvectors (256 inputs) and a run of
//     32-row pairs.  It builds the OC tile for its subvectors in LDS, fp32,
//     laid out as word(c*64 + l) for subvector l of the tile and centroid c,
//     so the LDS bank of an entry depends only on l.  Lane l of every
//     wavefront always works on subvector l: the 64 lanes of one LDS read hit
//     64 different banks whatever the indices are -- the conflict-free lookup
//     of [EVA 2.A] expressed as a bank layout.  The OC entries come from the
//     matrix cores: OC = x_rot . WC^T is a (64 x 4) x (4 x 256) product.
//   * Indices stream from HBM in 1 KiB chunks (16 rows x 64 subvectors, one
//     16-byte load per lane, fully coalesced), read once, one row step in
//     flight per wave.
//   * One v_perm_b32 turns an index byte into the LDS byte address
//     (lane*4 | c<<8 | region<<16): one VALU op, one LDS read and one add per
//     lookup.
//   * Each lane accumulates 32 rows; the cross-lane "adder tree" of
//     [EVA 2.B] is a transposing butterfly built from gfx950 permlane swaps
//     and DPP moves.
//   * Workgroups that share rows (a split along K) hand their partial sums
//     over with one 64-bit fixed-point atomic per row, so y does not depend
//     on the order in which they arrive (bitwise reproducible).
#include <hip/hip_runtime.h>

#include <mutex>

#include "vq_internal.h"

namespace vqd {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float f32x32_t __attribute__((ext_vector_type(32)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float lds_at(const float *base, uint32_t byte_addr) {
  return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + byte_addr);
}

// DPP controls (GCN/CDNA encoding)
constexpr int DPP_QUAD_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR8 = 0x128;        // rotate a 16-lane row by 8 == lane ^ 8
constexpr int DPP_ROW_HALF_MIRROR = 0x141; // lane i <-> 7 - i within 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), CTRL, 0xF, 0xF, false));
}

// Swap the upper 32 lanes of a with the lower 32 lanes of b.
__device__ __forceinline__ void swap32(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
  a = as_f(r[0]);
  b = as_f(r[1]);
}
// Swap the odd 16-lane rows of a with the even 16-lane rows of b.
__device__ __forceinline__ void swap16(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane16_swap(as_u(a), as_u(b), false, false);
  a = as_f(r[0]);
  b = as_f(r[1]);
}

// Transposing stage over a lane bit handled by a DPP move: lanes with the bit
// clear keep `lo` and receive the partner's `lo`; lanes with it set keep `hi`.
template <int CTRL>
__device__ __forceinline__ float tstage(float lo, float hi, bool bit) {
  float send = bit ? lo : hi;
  float keep = bit ? hi : lo;
  return keep + dpp<CTRL>(send);
}

// Rows 0..15 in A, rows 16..31 in Bv.  Returns the full sum of row
// (lane >> 1) & 31 in every lane.
__device__ __forceinline__ float reduce_rows32(float (&A)[16], float (&Bv)[16], int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) { swap32(A[i], Bv[i]); A[i] = A[i] + Bv[i]; }
  // A[i]: row i + 16*bit5
#pragma unroll
  for (int i = 0; i < 8; ++i) { swap16(A[i], A[i + 8]); A[i] += A[i + 8]; }
  // A[i], i < 8: row i + 8*bit4 + 16*bit5
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) A[i] = tstage<DPP_ROW_ROR8>(A[i], A[i + 4], b3);
  // A[i], i < 4: row i + 4*bit3 + ...
#pragma unroll
  for (int i = 0; i < 2; ++i) A[i] = tstage<DPP_ROW_HALF_MIRROR>(A[i], A[i + 2], b2);
  // A[i], i < 2: row i + 2*bit2 + ...; partial over {i, 7-i}
  float v = tstage<DPP_QUAD_XOR2>(A[0], A[1], b1);
  // v: row bit1 + 2*bit2 + ...; partial over {i, 7-i, i^2, 7-(i^2)}
  v += dpp<DPP_QUAD_XOR1>(v);
  return v;
}

// byte k of w -> LDS byte address: byte0 from base (lane*4), byte1 = index,
// byte2 from base (64 KiB region), byte3 = 0.
template <int K>
__device__ __forceinline__ uint32_t lut_addr(uint32_t w, uint32_t base) {
  return __builtin_amdgcn_perm(w, base, 0x0C020000u | ((4u + K) << 8));
}

// Raw buffer descriptors (gfx9 word 3), an offset past any buffer the kernels
// address (they stay below 2 GiB), and the nontemporal cache-policy bit.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kNontemporal = 2;

__device__ __forceinline__ u32x4 load16(const uint8_t *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// Cross-workgroup hand-off of split partial sums without cache maintenance.
// Each XCD has its own L2, so a device-scope fence would write back and
// invalidate the whole L2 once per wave.  Instead the partials travel with
// device-scope (sc1) stores and loads, which are coherent across XCDs by
// themselves; the only ordering needed is that a workgroup's partial stores
// are acknowledged before it bumps the row block's counter.
__device__ __forceinline__ void store_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Last workgroup of a row block adds the split partials in fixed order.
__device__ __forceinline__ void split_finish(const Lut8Mat &M, int rb, int R, uint32_t *flag) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&M.counter[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (prev == (uint32_t)(M.nsplit - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (*flag == 0u) return;
  for (int t = threadIdx.x; t < R; t += blockDim.x) {
    const int row = rb * R + t;
    if (row < M.N) {
      // loads go out eight at a time; the sum order (split 0, 1, ...) is fixed
      const float *p = M.partial + row;
      float s = 0.f;
      int q = 0;
      for (; q + 8 <= M.nsplit; q += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = load_dev(p + (size_t)(q + u) * M.rows_pad);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      for (; q < M.nsplit; ++q) s += load_dev(p + (size_t)q * M.rows_pad);
      M.y[row] = s;
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(&M.counter[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One-round-trip hand-off of split partials.  Every workgroup converts its
// partial of a row to fixed point with a power-of-two step q shared by the
// whole matrix, and adds it together with a split count into the row's 64-bit
// accumulator with one device-scope atomic:
//   word += 2^57 + (round(p / q) + 2^49)
// The workgroup whose add completes the count (old count == nsplit - 1) has
// the full sum in old + own term, writes y and clears the word.  q comes from
// a bound B >= |p| that every workgroup of the matrix computes identically,
// with |p|/q < 2^48, so each biased term lies in (0, 2^50) and up to 127
// splits fit below the count field.  Integer adds are exact and associative:
// y does not depend on the order in which workgroups arrive.
struct FixedScale {
  double inv_q;   // 1 / q
  double q;       // step, a power of two
};

__device__ __forceinline__ FixedScale fixed_scale(float bound) {
  FixedScale f;
  if (bound > 0.f) {
    const int e = ilogbf(bound) + 1 - 48;   // bound < 2^(e + 48)
    f.q = ldexp(1.0, e);
    f.inv_q = ldexp(1.0, -e);
  } else {
    f.q = 1.0;
    f.inv_q = 1.0;
  }
  return f;
}

__device__ __forceinline__ uint64_t packed_term(float p, const FixedScale &f) {
  const int64_t v = llrint((double)p * f.inv_q);
  return (1ull << 57) + (uint64_t)(v + (1ll << 49));
}
__device__ __forceinline__ uint64_t packed_add(uint64_t *acc, uint64_t term) {
  return __hip_atomic_fetch_add(acc, term, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// After the add: the workgroup whose add completed the count writes y and
// clears the word.  The clear is a plain store: no other workgroup touches
// the word again in this launch, and the kernel's end writes it back (L2
// write-back is byte-masked) before the next launch's atomics reach it.
__device__ __forceinline__ void packed_finish(uint64_t *acc, float *y, uint64_t old, uint64_t term,
                                              const FixedScale &f, int nsplit) {
  if ((int)(old >> 57) == nsplit - 1) {
    const uint64_t tot = old + term;
    const int64_t sv = (int64_t)(tot & ((1ull << 57) - 1)) - (int64_t)nsplit * (1ll << 49);
    *y = (float)((double)sv * f.q);
    *acc = 0ull;
  }
}

// Sum of squares of 8 fp16 values (fp32).
__device__ __forceinline__ float sq_sum8(u32x4 c) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t h = as_h2(c[i]);
    s = __builtin_fmaf((float)h.x, (float)h.x, s);
    s = __builtin_fmaf((float)h.y, (float)h.y, s);
  }
  return s;
}

// Wave-wide sum and max: quad and row butterflies with DPP, then 16- and
// 32-lane swaps.  Every lane ends with the same value (IEEE add and max are
// commutative), identical in every workgroup that holds the same data in the
// same lanes.
constexpr int DPP_ROW_MIRROR = 0x140;      // lane i <-> 15 - i within 16 lanes
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<DPP_QUAD_XOR1>(v);
  v += dpp<DPP_QUAD_XOR2>(v);
  v += dpp<DPP_ROW_MIRROR>(v);             // quad q + quad 3-q
  v += dpp<DPP_ROW_ROR8>(v);               // + the other pair: whole row
  float a = v, b = v;
  swap16(a, b);
  v = a + b;                               // rows 2k + rows 2k+1
  a = v; b = v;
  swap32(a, b);
  return a + b;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
  float a = v, b = v;
  swap16(a, b);
  v = fmaxf(a, b);
  a = v; b = v;
  swap32(a, b);
  return fmaxf(a, b);
}

// --------------------------------------------------------------------------
// Rotated lookup GEMV + 1-bit sign residual   [EDGE section details]
// LDS: the sign table at 0 and the OC tile of the workgroup's 64 subvectors
// (from x_rot) at 64 KiB.  For the 32 sign bytes of the same 256 weights the
// table holds T[v][p] = sum_i (bit_i(v) ? +1 : -1) * x_rot[8p + i] in columns
// p and p + 32, so that a lane can always find its position in a column no
// other lane of its half-wave reads.
//
// The rotation is fused for Hadamard blocks h <= 2048.  In Sylvester (natural)
// order H_h = H_{h/256} (x) H_256 for h >= 256, so the 256 rotated inputs of a
// tile, which sit in sub-block q of their block, are the 256-point transform
// of sum_{q'} (-1)^popcount(q & q') (s (.) x)[sub-block q'].  Wave 0 forms
// that combination and the 256-point butterfly in registers (lane l holds
// elements 4l .. 4l+3, partners across lanes by xor shuffles) and leaves
// x_rot of the tile in LDS for the other waves.  For h < 256 the tile holds
// whole blocks and only the butterfly stages below h run.  Larger blocks are
// rotated by rht_kernel into the workspace first (M.xr).
// --------------------------------------------------------------------------
__device__ __forceinline__ float sign_of_byte(uint32_t s4, int t) {
  return (float)(int8_t)((s4 >> (8 * t)) & 0xffu);
}

// RES = false is the plain lookup GEMV in the output-codebook form [EVA
// section 2.A]: the same OC tile, gather and hand-off with no rotation, no
// sign table and no residual term (x itself is the tile's input).
template <int W, int STEPS, int NBX, bool RES>
__global__ void __launch_bounds__(W * 64) lut8_residual_kernel(const Lut8Args args) {
  static_assert(W == 16, "the OC tile takes waves 0-7, the sign table waves 8-15");
  constexpr int NT = W * 64;
  // LDS: sign table [256 byte values][64 columns] at 0, OC tile [256
  // centroids][64 subvectors] at 64 KiB (so the sign lookups' addresses have
  // a zero third byte), x_rot, bound parts, hand-off flag
  __shared__ __align__(16) float lds[2 * 16384 + 256 + 2 * W + 16];
  float *xrs = lds + 2 * 16384;              // x_rot of the tile, 4 per subvector
  float *bnd = xrs + 256;
  uint32_t *flag = reinterpret_cast<uint32_t *>(bnd + 2 * W);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Lut8Mat &M = args.mat[blockIdx.y];
  if ((int)blockIdx.x >= M.nwg) return;
  const int local = blockIdx.x;
  const int sp = local % M.nsplit, rb = local / M.nsplit;
  const int NG = (M.N + 15) >> 4;
  const int NP = (M.N + 31) >> 5;
  const int pl = lane & 31;
  const uint8_t *xb = reinterpret_cast<const uint8_t *>(M.x);
  const bool oc_wave = wave < 8;

  // 1. small loads first; every load here is unconditional within its wave
  //    (a branch around a load makes the compiler wait for the whole index
  //    stream at the join).  The vector memory pipe of a CU is shared by its
  //    16 waves, so work that every wave would repeat is done once: wave 0
  //    alone loads the rotation inputs, sub-block u of the tile's Hadamard
  //    block at elements 4 lane .. 4 lane + 3 (clamped, in bounds) with their
  //    signs (x itself stands in when there are none), or the rotated tile
  //    the rotation kernel left in the workspace.
  const int h = M.had;                       // 1: no rotation
  const int k0 = sp * 256;
  const int QS = h > 256 ? (h >> 8) : 1;
  const int kb = h > 256 ? (k0 / h) * h : k0;
  const int qt = h > 256 ? ((k0 - kb) >> 8) : 0;
  const bool fused = M.fused != 0;
  uint2 xq[8];
  uint32_t sq[8];
  float4 xrw;
  if (wave == 0) {
    if constexpr (RES) {
      const uint8_t *rsb = M.rs ? reinterpret_cast<const uint8_t *>(M.rs) : xb;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = kb + 256 * min(u, QS - 1) + 4 * lane;
        xq[u] = *reinterpret_cast<const uint2 *>(xb + 2 * (size_t)e);
        sq[u] = *reinterpret_cast<const uint32_t *>(rsb + e);
      }
      xrw = *reinterpret_cast<const float4 *>(M.xr + k0 + 4 * lane);
    } else {
      xq[0] = *reinterpret_cast<const uint2 *>(xb + 2 * (size_t)(k0 + 4 * lane));
    }
  }
  //    OC waves: centroids 32 wave + (lane % 32) as the MFMA A operand.  The
  //    eight OC waves hold the whole codebook, so max |WC| is taken from them.
  const uint2 wraw = reinterpret_cast<const uint2 *>(M.wc)[(oc_wave ? wave : 0) * 32 + (lane & 31)];
  const half4_t wa = __builtin_bit_cast(half4_t, wraw);
  //    bound inputs: x in 16-byte chunks t0 + u NT, max |alpha|
  const int nxc = M.J >> 1;
  const int t0 = threadIdx.x;
  u32x4 xbw[NBX];
#pragma unroll
  for (int u = 0; u < NBX; ++u) xbw[u] = load16(xb + 16 * (size_t)min(t0 + u * NT, nxc - 1));
  const uint32_t amax_bits = RES ? *M.alpha_hdr : 0u;
  __builtin_amdgcn_s_barrier();

  // 2. index, sign and alpha loads: per 32-row step, two index chunks, one
  //    sign chunk and the scale of the lane's (row, group).  Only the first
  //    step is loaded here, the second after the OC tile is built, and step
  //    g + 2 when step g's lookups start.  With few steps in flight per wave
  //    the memory queues stay short, so the rotation inputs and each step's
  //    data come back in issue order instead of behind every workgroup's
  //    whole stream.
  u32x4 va[STEPS], vb[STEPS], vs[STEPS];
  uint16_t al[STEPS];
  //    Loads go through buffer descriptors: a step past the workgroup's run
  //    gets an out-of-range offset, which returns zeros without touching
  //    memory.  The load is still issued (a branch around it would make the
  //    compiler wait for every load in flight) but is not looked up.
  const __amdgpu_buffer_rsrc_t rwi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(M.wi), (short)0, M.nsplit * NG * 1024, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsg = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(M.signs), (short)0, M.nsplit * NP * 1024, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ral = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(M.alpha), (short)0, M.nsplit * NP * 128, kBufferWord3);
  auto load_step = [&](int g) {
    const bool mine = g * W + wave < M.rpw;
    const int rp = min(rb * M.rpw + g * W + wave, NP - 1);
    const int rga = min(2 * rp, NG - 1), rgb = min(2 * rp + 1, NG - 1);
    const uint32_t oa = mine ? (uint32_t)(((sp * NG + rga) * 64 + lane) * 16) : kOutOfRange;
    const uint32_t ob = mine ? (uint32_t)(((sp * NG + rgb) * 64 + lane) * 16) : kOutOfRange;
    const uint32_t os = mine ? (uint32_t)(((sp * NP + rp) * 64 + lane) * 16) : kOutOfRange;
    const uint32_t oal = mine ? (uint32_t)(((sp * NP + rp) * 64 + lane) * 2) : kOutOfRange;
    va[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, oa, 0, kNontemporal));
    vb[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rwi, ob, 0, kNontemporal));
    if constexpr (RES) {
      vs[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsg, os, 0, kNontemporal));
      al[g] = __builtin_amdgcn_raw_buffer_load_b16(ral, oal, 0, 0);
    } else {
      (void)os; (void)oal;
    }
  };
  load_step(0);

  // 3. x_rot of subvector `lane` of this tile, formed by wave 0 into LDS
  if (wave == 0 && !RES) {
    const half2_t a = as_h2(xq[0].x), b = as_h2(xq[0].y);
    *reinterpret_cast<float4 *>(xrs + 4 * lane) = make_float4((float)a.x, (float)a.y, (float)b.x, (float)b.y);
  } else if (wave == 0) {
    float c[4] = {xrw.x, xrw.y, xrw.z, xrw.w};
    if (fused) {
      c[0] = c[1] = c[2] = c[3] = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < QS) {
          if (!M.rs) sq[u] = 0x01010101u;
          const float sg = (__builtin_popcount(qt & u) & 1) ? -1.f : 1.f;
          const half2_t a = as_h2(xq[u].x), b = as_h2(xq[u].y);
          c[0] += sg * sign_of_byte(sq[u], 0) * (float)a.x;
          c[1] += sg * sign_of_byte(sq[u], 1) * (float)a.y;
          c[2] += sg * sign_of_byte(sq[u], 2) * (float)b.x;
          c[3] += sg * sign_of_byte(sq[u], 3) * (float)b.y;
        }
      }
      const int hl = h < 256 ? h : 256;
      if (hl >= 2) {
        const float a0 = c[0] + c[1], a1 = c[0] - c[1], a2 = c[2] + c[3], a3 = c[2] - c[3];
        c[0] = a0; c[1] = a1; c[2] = a2; c[3] = a3;
      }
      if (hl >= 4) {
        const float a0 = c[0] + c[2], a2 = c[0] - c[2], a1 = c[1] + c[3], a3 = c[1] - c[3];
        c[0] = a0; c[1] = a1; c[2] = a2; c[3] = a3;
      }
      for (int m = 1; 4 * m < hl; m <<= 1) {
        const bool upper = lane & m;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float p = __shfl_xor(c[t], m, 64);
          c[t] = upper ? (p - c[t]) : (c[t] + p);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) c[t] *= M.had_scale;
    }
    *reinterpret_cast<float4 *>(xrs + 4 * lane) = make_float4(c[0], c[1], c[2], c[3]);
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  if (oc_wave) {
    // 4. OC tile, centroids 32 wave .. +31, on the matrix cores.  x_rot is
    //    split into fp16 high and low parts (x = hi + lo to ~2^-22), so two
    //    fp16 MFMAs give the fp32 product; the output registers are placed as
    //    in the plain kernel (one centroid per register after the swap).
    const float4 xv = *reinterpret_cast<const float4 *>(xrs + 4 * lane);
    const float xr[4] = {xv.x, xv.y, xv.z, xv.w};
    half4_t xh, xl;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const _Float16 hi = (_Float16)xr[t];
      xh[t] = hi;
      // the low part of an infinite input is zero, not inf - inf
      xl[t] = __builtin_isfinite(xr[t]) ? (_Float16)(xr[t] - (float)hi) : (_Float16)0.f;
    }
    f32x32_t o = {};
    o = __builtin_amdgcn_mfma_f32_32x32x4f16(wa, xh, o, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_32x32x4f16(wa, xl, o, 0, 0, 0);
    float *dst = lds + 16384 + (wave * 32) * 64 + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = o[i], b = o[i + 16];
      swap32(a, b);
      const int m = (i >> 2) * 8 + (i & 3);
      dst[m * 64] = a;
      dst[(m + 4) * 64] = b;
    }
  } else if (RES) {
    // 5. sign table for sign byte p = 32*sp + (lane & 31): its 8 rotated
    //    inputs are x_rot 8p' .. 8p'+7 of the tile (p' = lane & 31); this
    //    wave writes high nibbles 2 (wave - 8) and 2 (wave - 8) + 1
    const float4 l4 = *reinterpret_cast<const float4 *>(xrs + 8 * pl);
    const float4 h4 = *reinterpret_cast<const float4 *>(xrs + 8 * pl + 4);
    const float lo4[4] = {l4.x, l4.y, l4.z, l4.w};
    const float hi4[4] = {h4.x, h4.y, h4.z, h4.w};
    // T = sum_i (+-1) x_i formed from signed pairs, never as 2 (sum of the
    // set inputs) - (sum of all): no cancellation, so an infinite input
    // gives an infinite entry as the sum itself does
    const float pa[4] = {-(lo4[0] + lo4[1]), lo4[0] - lo4[1], lo4[1] - lo4[0], lo4[0] + lo4[1]};
    const float pb[4] = {-(lo4[2] + lo4[3]), lo4[2] - lo4[3], lo4[3] - lo4[2], lo4[2] + lo4[3]};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int hi = 2 * (wave - 8) + e;
      const float H = (((hi & 1) ? hi4[0] : -hi4[0]) + ((hi & 2) ? hi4[1] : -hi4[1])) +
                      (((hi & 4) ? hi4[2] : -hi4[2]) + ((hi & 8) ? hi4[3] : -hi4[3]));
      float *dst = lds + (hi * 16) * 64 + lane;
#pragma unroll
      for (int lo = 0; lo < 16; ++lo) dst[lo * 64] = (pa[lo & 3] + pb[lo >> 2]) + H;
    }
  }
  // the second row step goes out once the tables are written (the OC inputs
  // are in by then); from here on two steps are in flight per wave
  if (STEPS > 1) load_step(1);
  // 6. per-wave parts of the bound sum_k |x_rot_k| <= sqrt(K) ||x||_2
  {
    float s2 = 0.f;
#pragma unroll
    for (int u = 0; u < NBX; ++u)
      if (t0 + u * NT < nxc) s2 += sq_sum8(xbw[u]);
    if (nxc > NBX * NT) s2 = __builtin_inff();   // longer inputs take the float hand-off
    uint32_t m = max(max(wraw.x & 0x7fffu, (wraw.x >> 16) & 0x7fffu),
                     max(wraw.y & 0x7fffu, (wraw.y >> 16) & 0x7fffu));
    const float mw = !oc_wave ? 0.f
                     : m >= 0x7c00u ? __builtin_inff()
                                    : (float)__builtin_bit_cast(_Float16, (uint16_t)m);
    const float ws = wave_sum(s2), wm = wave_max(mw);
    if (lane == 0) { bnd[wave] = ws; bnd[W + wave] = wm; }
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // 7. lookups.  Index chunks: lane = subvector, bytes = 16 rows.  Sign
  //    chunk: lane L = 2r + g holds the 16 sign bytes of row r and group g of
  //    the tile, byte j at position 16 g + (j ^ (r & 15)); its column in the
  //    table, 32 (r >> 4) + 16 g + (j ^ (r & 15)), differs across the 64
  //    lanes for every j.  byte0 of the address comes from bsel[j >> 2] byte
  //    (j & 3), byte1 is the sign byte.
  const uint32_t baseoc = ((uint32_t)lane << 2) | 0x10000u;
  const int rr = lane >> 1, gg = lane & 1;
  const uint32_t c0 = (uint32_t)(32 * (rr >> 4) + 16 * gg + (rr & 15));
  uint32_t bsel[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t v = 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t) v |= (((c0 ^ (uint32_t)(4 * q + t)) << 2) & 0xffu) << (8 * t);
    bsel[q] = v;
  }
  // the hand-off's scale (uniform): fixed point unless an input is not
  // finite; each step's atomics are issued before the next step's lookups so
  // their round trips overlap
  float X2 = 0.f, Mw = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) { X2 += bnd[w]; Mw = fmaxf(Mw, bnd[W + w]); }
  const float amax = (amax_bits & 0x7fffu) >= 0x7c00u
                         ? __builtin_inff()
                         : (float)__builtin_bit_cast(_Float16, (uint16_t)(amax_bits & 0x7fffu));
  const float bound = __builtin_sqrtf((float)(M.J * 4) * X2) * (Mw + amax) * 1.0009765625f;
  const bool packed = M.nsplit > 1 && bound <= 3.0e38f && M.nsplit <= 127;
  const FixedScale fs = fixed_scale(bound);
  const int rsel = (lane >> 1) & 31;
  float rowval[STEPS];
  uint64_t term[STEPS], old[STEPS];
#pragma unroll
  for (int g = 0; g < STEPS; ++g) {
    if (g + 2 < STEPS) load_step(g + 2);
    rowval[g] = 0.f;
    old[g] = 0ull;
    term[g] = 0ull;
    if (g * W + wave >= M.rpw) continue;      // past the run: nothing to look up
    float A[16], Bv[16], S[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wq = va[g][q], wbq = vb[g][q];
      A[4 * q + 0] = lds_at(lds, lut_addr<0>(wq, baseoc));
      A[4 * q + 1] = lds_at(lds, lut_addr<1>(wq, baseoc));
      A[4 * q + 2] = lds_at(lds, lut_addr<2>(wq, baseoc));
      A[4 * q + 3] = lds_at(lds, lut_addr<3>(wq, baseoc));
      Bv[4 * q + 0] = lds_at(lds, lut_addr<0>(wbq, baseoc));
      Bv[4 * q + 1] = lds_at(lds, lut_addr<1>(wbq, baseoc));
      Bv[4 * q + 2] = lds_at(lds, lut_addr<2>(wbq, baseoc));
      Bv[4 * q + 3] = lds_at(lds, lut_addr<3>(wbq, baseoc));
      if constexpr (RES) {
        const uint32_t ws4 = vs[g][q];
        S[4 * q + 0] = lds_at(lds, __builtin_amdgcn_perm(ws4, bsel[q], 0x0C0C0400u));
        S[4 * q + 1] = lds_at(lds, __builtin_amdgcn_perm(ws4, bsel[q], 0x0C0C0501u));
        S[4 * q + 2] = lds_at(lds, __builtin_amdgcn_perm(ws4, bsel[q], 0x0C0C0602u));
        S[4 * q + 3] = lds_at(lds, __builtin_amdgcn_perm(ws4, bsel[q], 0x0C0C0703u));
      }
    }
    rowval[g] = reduce_rows32(A, Bv, lane);
    if constexpr (RES) {
      // residual of (row r, group g): alpha times the sum over its 16 sign
      // bytes; the two groups of a row sit in lanes 2r and 2r + 1
#pragma unroll
      for (int i = 0; i < 8; ++i) S[i] += S[i + 8];
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] += S[i + 4];
      const float sres = ((S[0] + S[2]) + (S[1] + S[3])) * (float)__builtin_bit_cast(_Float16, al[g]);
      rowval[g] += sres + dpp<DPP_QUAD_XOR1>(sres);
    }
    const int row = (rb * M.rpw + g * W + wave) * 32 + rsel;
    if (packed && (lane & 1) == 0 && row < M.N) {
      term[g] = packed_term(rowval[g], fs);
      old[g] = packed_add(M.acc + row, term[g]);
    }
  }

  // 8. rows out: lane 2r holds row r of each 32-row group
  if (M.nsplit == 1) {
#pragma unroll
    for (int g = 0; g < STEPS; ++g) {
      const int rp = rb * M.rpw + g * W + wave;
      const int row = rp * 32 + rsel;
      if ((lane & 1) == 0 && g * W + wave < M.rpw && row < M.N) M.y[row] = rowval[g];
    }
    return;
  }
  if (packed) {
#pragma unroll
    for (int g = 0; g < STEPS; ++g) {
      const int row = (rb * M.rpw + g * W + wave) * 32 + rsel;
      if ((lane & 1) == 0 && g * W + wave < M.rpw && row < M.N)
        packed_finish(M.acc + row, M.y + row, old[g], term[g], fs, M.nsplit);
    }
    return;
  }
  // non-finite inputs or more than 127 splits: float partials and a
  // last-workgroup sum
#pragma unroll
  for (int g = 0; g < STEPS; ++g) {
    const int rp = rb * M.rpw + g * W + wave;
    const int row = rp * 32 + rsel;
    if ((lane & 1) == 0 && g * W + wave < M.rpw && rp < NP) store_dev(M.partial + (size_t)sp * M.rows_pad + row, rowval[g]);
  }
  split_finish(M, rb, 32 * M.rpw, flag);
}

// --------------------------------------------------------------------------
// device scratch of vq_gemv_residual_noalloc
// --------------------------------------------------------------------------
// One array per GPU the library runs on, held until the process ends.  Bytes
// [0, VQ_NOALLOC_COUNTER_BYTES) hold completion counters and fixed-point
// accumulators: zero when the code object is loaded, and returned to zero by
// every call that completes (the last workgroup of a row block clears what
// it used), so no call has to clear them first.  The bytes above hold float
// partials and rotated inputs, written before they are read in each call.
static __device__ __align__(256) uint8_t scratch[VQ_NOALLOC_SCRATCH_BYTES];

// Device address of this GPU's scratch (the array's name in host code is a
// host-side stand-in, not a device address).  Looked up once per device,
// with that device current, and kept.
int noalloc_scratch(void **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return 0;
}

// --------------------------------------------------------------------------
// launchers of the lookup kernels
// --------------------------------------------------------------------------
template <int STEPS, int NBX, bool RES>
static int launch_residual_t(const Lut8Args &a, int grid_x, hipStream_t st) {
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL((lut8_residual_kernel<16, STEPS, NBX, RES>), dim3(grid_x, a.count), dim3(16 * 64), 0, st, a);
  return (int)hipGetLastError();
}

template <bool RES>
static int launch_lut8_t(const Lut8Args &a, const Lut8Shape &s, int grid_x, hipStream_t st) {
  if (s.steps == 1 && s.nbx == 2) return launch_residual_t<1, 2, RES>(a, grid_x, st);
  if (s.steps == 1 && s.nbx == 4) return launch_residual_t<1, 4, RES>(a, grid_x, st);
  if (s.steps == 2 && s.nbx == 2) return launch_residual_t<2, 2, RES>(a, grid_x, st);
  if (s.steps == 2 && s.nbx == 4) return launch_residual_t<2, 4, RES>(a, grid_x, st);
  if (s.steps == 4 && s.nbx == 2) return launch_residual_t<4, 2, RES>(a, grid_x, st);
  if (s.steps == 4 && s.nbx == 4) return launch_residual_t<4, 4, RES>(a, grid_x, st);
  if (s.steps == 8 && s.nbx == 2) return launch_residual_t<8, 2, RES>(a, grid_x, st);
  if (s.steps == 8 && s.nbx == 4) return launch_residual_t<8, 4, RES>(a, grid_x, st);
  return (int)hipErrorInvalidConfiguration;
}

int launch_lut8_residual(const Lut8Args &a, const Lut8Shape &s, int grid_x, void *stream,
                         bool residual) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (s.waves != 16) return (int)hipErrorInvalidConfiguration;
  return residual ? launch_lut8_t<true>(a, s, grid_x, st) : launch_lut8_t<false>(a, s, grid_x, st);
}

// --------------------------------------------------------------------------
// packing helpers (load time; bit layout of vqd.h)
// --------------------------------------------------------------------------
__global__ void pack_kernel(const uint32_t *idx, int64_t count, int nbits, uint8_t *out, int64_t nbytes) {
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < nbytes;
       o += (int64_t)gridDim.x * blockDim.x) {
    uint32_t byte = 0u;
    for (int b = 0; b < 8; ++b) {
      const int64_t q = o * 8 + b;
      const int64_t t = q / nbits;
      const int i = (int)(q - t * nbits);
      if (t < count) byte |= ((idx[t] >> i) & 1u) << b;
    }
    out[o] = (uint8_t)byte;
  }
}

__global__ void unpack_kernel(const uint8_t *packed, int64_t count, int nbits, uint32_t *out) {
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < count;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q0 = t * nbits;
    uint32_t v = 0u;
    for (int i = 0; i < nbits; ++i) {
      const int64_t q = q0 + i;
      v |= ((uint32_t)(packed[q >> 3] >> (q & 7)) & 1u) << i;
    }
    out[t] = v;
  }
}

// canonical [N][J] bytes -> tile-16x64
__global__ void repack_wi8_kernel(const uint8_t *canon, int N, int J, uint8_t *dev) {
  const int NG = (N + 15) >> 4;
  const int64_t total = (int64_t)(J >> 6) * NG * 64;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(e & 63);
    const int64_t chunk = e >> 6;
    const int rg = (int)(chunk % NG);
    const int jt = (int)(chunk / NG);
    const int j = jt * 64 + l;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 16; ++i) {
      const int r = rg * 16 + i;
      const uint32_t b = (r < N) ? canon[(size_t)r * J + j] : 0u;
      w[i >> 2] |= b << (8 * (i & 3));
    }
    *reinterpret_cast<u32x4 *>(dev + e * 16) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// canonical signs [N][P] bytes -> tile-32x32
__global__ void repack_signs_kernel(const uint8_t *canon, int N, int P, uint8_t *dev) {
  const int NP = (N + 31) >> 5;
  const int64_t total = (int64_t)(P >> 5) * NP * 64;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(e & 63);
    const int64_t chunk = e >> 6;
    const int rp = (int)(chunk % NP);
    const int pt = (int)(chunk / NP);
    const int rr = l >> 1, gg = l & 1;
    const int r = rp * 32 + rr;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 16; ++j) {
      const int p = pt * 32 + 16 * gg + (j ^ (rr & 15));
      const uint32_t b = (r < N) ? canon[(size_t)r * P + p] : 0u;
      w[j >> 2] |= b << (8 * (j & 3));
    }
    *reinterpret_cast<u32x4 *>(dev + e * 16) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// canonical alpha [N][G] fp16 -> ((g/2*NP + r/32)*64 + 2*(r%32) + g%2)
__global__ void repack_alpha_kernel(const uint16_t *canon, int N, int G, uint16_t *dev, uint32_t *hdr) {
  const int NP = (N + 31) >> 5;
  const int64_t total = (int64_t)((G + 1) >> 1) * NP * 64;
  uint32_t mx = 0u;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(e & 63);
    const int64_t chunk = e >> 6;
    const int rp = (int)(chunk % NP);
    const int g2 = (int)(chunk / NP);
    const int g = g2 * 2 + (l & 1), r = rp * 32 + (l >> 1);
    const uint16_t v = (r < N && g < G) ? canon[(size_t)r * G + g] : (uint16_t)0;
    dev[e] = v;
    mx = max(mx, (uint32_t)(v & 0x7fffu));
  }
  atomicMax(hdr, mx);    // largest fp16 magnitude, compared as bits
}

// --------------------------------------------------------------------------
// output codebook materialized in memory   [EVA 2.A]
// --------------------------------------------------------------------------
template <int D>
__global__ void build_oc_kernel(const _Float16 *x, int B, int K, int nbits, const _Float16 *wc,
                                void *oc, int f16_out) {
  const int J = K / D;
  const int64_t ncent = (int64_t)1 << nbits;
  const int64_t total = (int64_t)B * J * ncent;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = e & (ncent - 1);
    const int64_t row = e >> nbits;          // b*J + j
    const int64_t b = row / J, j = row - b * J;
    const _Float16 *xp = x + b * K + j * D;
    const _Float16 *wp = wc + c * D;
    float o = 0.f;
#pragma unroll
    for (int t = 0; t < D; ++t) o = __builtin_fmaf((float)xp[t], (float)wp[t], o);
    if (f16_out)
      reinterpret_cast<_Float16 *>(oc)[e] = (_Float16)o;
    else
      reinterpret_cast<float *>(oc)[e] = o;
  }
}

// --------------------------------------------------------------------------
// randomized Hadamard rotation   [EDGE section details]
// One workgroup per (token, block of h): signed input in LDS, in-place
// radix-2 butterflies in natural (Sylvester) order, scaled by 1/sqrt(h).
// --------------------------------------------------------------------------
__global__ void rht_kernel(const _Float16 *x, const int8_t *sign, int K, int h, float scale, float *x_rot) {
  extern __shared__ float buf[];
  const int blocks = K / h;
  const int b = blockIdx.x / blocks, blk = blockIdx.x % blocks;
  const size_t off = (size_t)b * K + (size_t)blk * h;
  for (int i = threadIdx.x; i < h; i += blockDim.x) {
    float v = (float)x[off + i];
    if (sign) v *= (float)sign[blk * h + i];
    buf[i] = v;
  }
  for (int len = 1; len < h; len <<= 1) {
    __syncthreads();
    for (int t = threadIdx.x; t < (h >> 1); t += blockDim.x) {
      const int i = (t / len) * 2 * len + (t % len);
      const float a = buf[i], c = buf[i + len];
      buf[i] = a + c;
      buf[i + len] = a - c;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < h; i += blockDim.x) x_rot[off + i] = buf[i] * scale;
}

__global__ void fill_u32_kernel(uint32_t *p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

static int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

int launch_pack(const uint32_t *idx, int64_t count, int nbits, uint8_t *out, void *stream) {
  const int64_t nbytes = (count * nbits + 7) / 8;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(nbytes, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), idx, count, nbits, out, nbytes);
  return (int)hipGetLastError();
}

int launch_unpack(const uint8_t *packed, int64_t count, int nbits, uint32_t *out, void *stream) {
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(count, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), packed, count, nbits, out);
  return (int)hipGetLastError();
}

int launch_repack_wi8(const uint8_t *canon, int N, int J, uint8_t *dev, void *stream) {
  const int64_t total = (int64_t)(J >> 6) * ((N + 15) >> 4) * 64;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(repack_wi8_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), canon, N, J, dev);
  return (int)hipGetLastError();
}

int launch_repack_signs(const uint8_t *canon, int N, int P, uint8_t *dev, void *stream) {
  const int64_t total = (int64_t)(P >> 5) * ((N + 31) >> 5) * 64;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(repack_signs_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), canon, N, P, dev);
  return (int)hipGetLastError();
}

int launch_repack_alpha(const uint16_t *canon, int N, int G, uint16_t *dev, uint32_t *hdr, void *stream) {
  const int64_t total = (int64_t)((G + 1) >> 1) * ((N + 31) >> 5) * 64;
  const int err = launch_fill_u32(hdr, 64, 0u, stream);
  if (err) return err;
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(repack_alpha_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), canon, N, G, dev, hdr);
  return (int)hipGetLastError();
}

int launch_build_oc(const uint16_t *x, int B, int K, int d, int nbits, const uint16_t *wc, void *oc,
                    int f16_out, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t total = (int64_t)B * (K / d) << nbits;
  const dim3 grid(grid_for(total, 256)), block(256);
  const _Float16 *xh = reinterpret_cast<const _Float16 *>(x);
  const _Float16 *wh = reinterpret_cast<const _Float16 *>(wc);
  switch (d) {
    case 1: hipLaunchKernelGGL(build_oc_kernel<1>, grid, block, 0, st, xh, B, K, nbits, wh, oc, f16_out); break;
    case 2: hipLaunchKernelGGL(build_oc_kernel<2>, grid, block, 0, st, xh, B, K, nbits, wh, oc, f16_out); break;
    case 4: hipLaunchKernelGGL(build_oc_kernel<4>, grid, block, 0, st, xh, B, K, nbits, wh, oc, f16_out); break;
    case 8: hipLaunchKernelGGL(build_oc_kernel<8>, grid, block, 0, st, xh, B, K, nbits, wh, oc, f16_out); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_rht(const uint16_t *x, const int8_t *sign, int B, int K, int h, float scale, float *x_rot,
               void *stream) {
  const int threads = h >= 256 ? 256 : (h >= 64 ? h : 64);
  const int grid = B * (K / h);
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(rht_kernel, dim3(grid), dim3(threads), (size_t)h * sizeof(float),
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const _Float16 *>(x), sign, K, h,
                     scale, x_rot);
  return (int)hipGetLastError();
}

int launch_fill_u32(uint32_t *p, size_t n, uint32_t v, void *stream) {
  (void)hipGetLastError();  // report only this launch's error
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for((int64_t)n, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), p, n, v);
  return (int)hipGetLastError();
}

}  // namespace vqd
