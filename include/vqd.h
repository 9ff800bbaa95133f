/*
 * vqd.h -- C ABI of libvqd, vector-quantized (VQ) decode GEMV for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [EVA]  "EVA: Accelerating LLM Decoding via an Efficient Vector
 *          Quantization Architecture" -- explainer page, technical summary,
 *          sections 1, 2.A and 2.B.
 *   [EDGE] "Replacing MatMul with SRAM lookup: a 3-bit edge inference
 *          architecture" -- article page, section details (the 3.125-bit
 *          quantization pipeline sketch and the LUT-inference paragraph).
 *
 * The operation.  A weight matrix W (N outputs x K inputs) is stored as a
 * codebook WC of 2^n centroids of dimension d (fp16, [2^n][d]) and an index
 * matrix WI ([N][K/d] n-bit indices) [EVA 2.A].  For each token b the layer
 * returns y[b][r] = sum_j OC[b*K/d + j][WI[r][j]] where the output codebook
 * OC[b*K/d + j][c] = sum_t x[b][j*d + t] * WC[c][t] is the product of the
 * input cut into K/d contiguous length-d subvectors with the codebook
 * [EVA 2.A].  This equals the dense product of the dequantized W with x.
 * [EDGE] adds an optional randomized Hadamard rotation of x and a 1-bit
 * residual: y[r] += sum_g alpha[r][g] * sum_{k in g} s[r][k] * x_rot[k] with
 * s = +1 for a set sign bit and -1 for a clear one, group g = weights
 * [128 g, 128 g + 128) of the row.
 *
 * Conventions for every call below.
 *   - Tensor pointers are DEVICE pointers owned by the caller unless a
 *     parameter says "host".  The library never allocates, frees, copies
 *     between host and device or synchronizes inside these calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; on return the results are not yet ready.
 *   - Every argument is validated on the host first.  On any error the call
 *     returns a negative vq_status and enqueues nothing.  A launch failure
 *     reported by the HIP runtime returns VQ_EHIP.
 *   - fp16 values are IEEE binary16 bit patterns in uint16_t.
 *   - Outputs y are fp32 and overwritten (never accumulated into).
 *   - Results are bitwise reproducible run to run: every cross-workgroup
 *     reduction sums in a fixed order.
 *   - Calls are thread-safe; the library holds no mutable global state.
 */
#ifndef VQD_H
#define VQD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VQ_OK = 0,
  VQ_EINVAL = -1,        /* null pointer, bad size or shape */
  VQ_EUNSUPPORTED = -2,  /* valid but not implemented (d, nbits, B, K) */
  VQ_EALIGN = -3,        /* a pointer misses its required alignment */
  VQ_EWORKSPACE = -4,    /* workspace missing or smaller than required */
  VQ_EHIP = -5           /* the HIP runtime reported an error */
} vq_status;

typedef enum { VQ_F16 = 0, VQ_F32 = 1 } vq_dtype;

/* Largest `count` accepted by one vq_gemv / vq_gemv_residual call. */
#define VQ_MAX_GROUP 16

/*
 * One quantized matrix.  A host struct, read only during the call.
 *   K, N      input and output features.
 *   d, nbits  supported pairs: (4, 8).  K must be a multiple of 64*d.
 *   wi        packed indices in the DEVICE layout made by vq_repack_wi
 *             (16-byte aligned).
 *   wc        fp16 codebook [2^nbits][d] (16-byte aligned).
 *   Residual fields (vq_gemv_residual only; ignored by vq_gemv):
 *   signs     sign bits in the DEVICE layout made by vq_repack_signs.
 *   alpha     fp16 scales in the DEVICE layout made by vq_repack_alpha.
 *   group     residual group size along K; must be 128.
 *   rht_sign  int8 [K] of +1/-1 for the randomized Hadamard rotation of x,
 *             or NULL when x is already rotated.
 *   had_block Hadamard block size h: a power of two dividing K, <= 16384.
 */
typedef struct {
  int32_t K, N, d, nbits;
  const void *wi;
  const uint16_t *wc;
  const void *signs;
  const void *alpha;
  int32_t group;
  const int8_t *rht_sign;
  int32_t had_block;
} vq_matrix;

/* Name of a vq_status value (static string; unknown codes give "unknown"). */
const char *vq_status_str(int status);

/*
 * Description of the HIP runtime error behind the most recent VQ_EHIP
 * returned to the calling thread ("no HIP error" if there was none).  The
 * string is static and owned by the HIP runtime.
 */
const char *vq_last_error(void);

/*
 * Bytes of the device layouts.  Zero means the shape is unsupported.
 *
 * WI device layout for nbits = 8 ("tile-16x64"): rows are padded with zero
 * indices to NG = ceil(N/16) groups of 16; index (r, j) of the canonical
 * matrix sits at byte ((j/64 * NG + r/16) * 64 + j%64) * 16 + r%16.  One
 * 1 KiB chunk holds 16 rows x 64 subvectors; lane l of a wavefront reads the
 * 16 bytes of subvector l, so a lane always works on one subvector and one
 * output-codebook column [EVA 2.A conflict-free lookup].
 */
size_t vq_wi_device_bytes(int32_t N, int32_t K, int32_t d, int32_t nbits);

/*
 * Sign-bit device layout ("tile-32x32"): P = K/8 sign bytes per row,
 * NP = ceil(N/32) groups of 32 rows.  Sign byte p of row r (bits of weights
 * 8p .. 8p+7, canonical [N][K/8], bit k%8 = weight k, 1 means +1) sits at
 * byte ((p/32 * NP + r/32) * 64 + ((r%32)/16) * 32 + p%32) * 16 + r%16.
 */
size_t vq_signs_device_bytes(int32_t N, int32_t K);

/*
 * Alpha device layout: fp16 scale (r, g) of the canonical [N][K/128] sits at
 * element ((g/2 * NP + r/32) * 4 + ((r%32)/16) * 2 + g%2) * 16 + r%16,
 * NP = ceil(N/32); padding is zero.
 */
size_t vq_alpha_device_bytes(int32_t N, int32_t K, int32_t group);

/*
 * Workspace bytes needed by vq_gemv (residual = 0) or vq_gemv_residual
 * (residual = 1) for these matrices and B tokens: split-K partial sums,
 * completion counters and, for the residual call, the rotated inputs.
 * Returns 0 on invalid arguments.  The workspace must be set up once with
 * vq_workspace_init before its first use; every call that completes leaves
 * it ready for the next one.  Calls sharing one workspace must be ordered
 * (same stream or explicit dependencies).
 */
size_t vq_workspace_bytes(const vq_matrix *m, int32_t count, int32_t B,
                          int32_t residual);

/* Zero the completion counters of a workspace (a fill kernel, no memset). */
int vq_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/*
 * Pack `count` indices (uint32, only the low `nbits` bits are used) into a
 * little-endian bit stream: index t occupies stream bits
 * [nbits*t, nbits*t + nbits), stream bit q is bit q%8 of byte q/8; the
 * output has ceil(count*nbits/8) bytes, unused high bits of the last byte
 * are zero.  1 <= nbits <= 16.  With nbits = 1 this packs residual sign
 * bits densely into bytes [EDGE section details].  [EVA 2.A] for WI.
 */
int vq_pack_indices(const uint32_t *idx, int64_t count, int32_t nbits,
                    uint8_t *out, void *stream);

/* Inverse of vq_pack_indices: `count` uint32 indices. 1 <= nbits <= 16. */
int vq_unpack_indices(const uint8_t *packed, int64_t count, int32_t nbits,
                      uint32_t *out, void *stream);

/*
 * Rearrange a canonical packed WI ([N] rows of K/d n-bit indices, each row
 * starting on a byte) into the device layout above.  `device_layout` must
 * hold vq_wi_device_bytes(N, K, d, nbits) bytes and must not overlap the
 * input.  A load-time step, not part of the timed decode.
 */
int vq_repack_wi(const uint8_t *canonical, int32_t N, int32_t K, int32_t d,
                 int32_t nbits, void *device_layout, void *stream);

/* Canonical sign bytes [N][K/8] -> sign device layout (K % 256 == 0). */
int vq_repack_signs(const uint8_t *canonical, int32_t N, int32_t K,
                    void *device_layout, void *stream);

/* Canonical fp16 alpha [N][K/group] -> alpha device layout (group == 128,
 * K % 256 == 0). */
int vq_repack_alpha(const uint16_t *canonical, int32_t N, int32_t K,
                    int32_t group, void *device_layout, void *stream);

/*
 * Output codebook [EVA 2.A]: OC[b*K/d + j][c] = sum_t x[b][j*d+t] * WC[c][t]
 * for b < B, j < K/d, c < 2^nbits, written row-major to `oc` as fp32
 * (VQ_F32) or fp16 round-to-nearest-even (VQ_F16).  Products of fp16 values
 * are exact in fp32 and summed in fp32.  d in {1, 2, 4, 8}, 1 <= nbits <= 16,
 * x fp16 [B][K].  `oc` must not overlap the inputs.
 */
int vq_build_oc(const uint16_t *x, int32_t B, int32_t K, int32_t d,
                int32_t nbits, const uint16_t *wc, void *oc,
                vq_dtype oc_dtype, void *stream);

/*
 * Randomized Hadamard rotation [EDGE section details]:
 * x_rot[b] = blockdiag(H_h, ..., H_h) (sign * x[b]) / sqrt(h), H_h the
 * Sylvester (natural-order) Hadamard matrix of order h = had_block, a power
 * of two dividing K, 1 <= h <= 16384.  x fp16 [B][K], sign int8 [K] of +-1,
 * x_rot fp32 [B][K].
 */
int vq_rht(const uint16_t *x, const int8_t *sign, int32_t B, int32_t K,
           int32_t had_block, float *x_rot, void *stream);

/*
 * VQ GEMV [EVA 2.A, 2.B]: for each of `count` matrices m,
 * y[m][b][r] = sum_j OC_m[b*K/d + j][WI_m[r][j]], OC built from x[m].
 *   m        host array of `count` matrix descriptors.
 *   x        host array of `count` device pointers, fp16 [B][K_m] each
 *            (16-byte aligned).
 *   y        host array of `count` device pointers, fp32 [B][N_m] each
 *            (4-byte aligned), overwritten.
 *   workspace / ws_bytes  at least vq_workspace_bytes(m, count, B, 0)
 *            bytes, 256-byte aligned, set up by vq_workspace_init.
 * All matrices are served by one kernel launch.  Supported: B == 1,
 * (d, nbits) == (4, 8), 1 <= count <= VQ_MAX_GROUP.
 */
int vq_gemv(const vq_matrix *m, int32_t count, const uint16_t *const *x,
            int32_t B, float *const *y, void *workspace, size_t ws_bytes,
            void *stream);

/*
 * Rotated VQ GEMV plus 1-bit residual [EDGE section details]: with
 * x_rot = rotation of x[m] (or x[m] itself when rht_sign is NULL),
 * y[m][b][r] = sum_j OC(x_rot)[b*K/d + j][WI[r][j]]
 *            + sum_g alpha[r][g] * sum_{k in g} s[r][k] * x_rot[b][k].
 * Same arguments and support as vq_gemv plus the residual fields of each
 * vq_matrix; workspace from vq_workspace_bytes(m, count, B, 1).
 */
int vq_gemv_residual(const vq_matrix *m, int32_t count,
                     const uint16_t *const *x, int32_t B, float *const *y,
                     void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VQD_H */
