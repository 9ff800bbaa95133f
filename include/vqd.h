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
 * Two forms compute it.  The output-codebook tile (vq_gemv_oc and
 * vq_gemv_residual) holds an OC tile in LDS with one bank per lane, so its
 * lookups never collide [EVA 2.A], and joins the K-slices of a row with one
 * fixed-point atomic per row.  The per-index form (vq_gemv and the other
 * calls) forms each OC entry when an index asks for it, from codebook copies
 * in LDS, with whole rows per workgroup and no join; at d = 4, n = 8 its 16
 * copies put two lanes on each bank pair, so about 44% of its LDS-active
 * cycles are bank conflicts (the token call's 32 copies have none).  The
 * per-index form measured faster on MI355X and is the default.
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
 *   - Calls are thread-safe; the library holds no mutable global state,
 *     except the per-GPU device scratch of vq_gemv_residual_noalloc (and its
 *     address, looked up once per GPU under a lock).
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
 *   d, nbits  supported pairs: (4, 8), (4, 12) and (8, 16); K must be a
 *             multiple of 256.  All matrices of one call share (d, nbits).
 *   wi        packed indices in the DEVICE layout made by vq_repack_wi
 *             (16-byte aligned).
 *   wc        fp16 codebook in the DEVICE layout made by vq_repack_wc
 *             (16-byte aligned): for (4, 8) and (4, 12) that is the
 *             canonical [2^nbits][d]; for (8, 16) it is dimension-major,
 *             [8][65536] (element (t, c) = WC[c][t]).
 *   Residual fields (vq_gemv_residual only, (d, nbits) = (4, 8); ignored
 *   by vq_gemv):
 *   signs     sign bits in the DEVICE layout made by vq_repack_signs
 *             (16-byte aligned).
 *   alpha     fp16 scales in the DEVICE layout made by vq_repack_alpha,
 *             header included (32-byte aligned).
 *   group     residual group size along K; must be 128.
 *   rht_sign  int8 [K] of +1/-1 for the randomized Hadamard rotation of x
 *             (4-byte aligned), or NULL when x is already rotated.
 *   had_block Hadamard block size h: a power of two dividing K, <= 16384.
 *   A residual matrix must stay below 2^31 bytes of device indices
 *   ((N rounded up to 32) * K/4 < 2^31): its kernel addresses them with
 *   32-bit buffer offsets.
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
 * Rows are padded with zero indices to NG = ceil(N/16) groups of 16.
 *
 * WI device layout for (4, 8) ("tile-16x64", K/4 % 64 == 0): index (r, j)
 * of the canonical matrix sits at byte
 * ((j/64 * NG + r/16) * 64 + j%64) * 16 + r%16.  One 1 KiB chunk holds 16
 * rows x 64 subvectors; lane l of a wavefront reads the 16 bytes of
 * subvector l, so a lane always works on one subvector: one x slice and,
 * with an output-codebook tile, one OC column [EVA 2.A conflict-free
 * lookup].
 *
 * (4, 12) ("tile-16x64-12", K/4 % 64 == 0): chunk (row group rg, subvector
 * tile jt), ordered row group first, is 1536 bytes; lane l's 24 bytes hold
 * the indices of rows 16 rg + i at subvector 64 jt + l, index i in bits
 * [12 i, 12 i + 12) of a little-endian 192-bit word.
 *
 * (8, 16) ("tile-16x32-16", K/8 % 32 == 0): chunk (rg, subvector block jb
 * of 32), ordered row group first, is 1 KiB; lane l holds 8 little-endian
 * uint16, the q-th the index of row 16 rg + l%16 at subvector
 * 32 jb + l/16 + 4 q.
 */
size_t vq_wi_device_bytes(int32_t N, int32_t K, int32_t d, int32_t nbits);

/*
 * Codebook device layout [EVA 2.B: the codebook stays on chip while indices
 * stream; with 65536 centroids one dimension of it fits in LDS at a time].
 * vq_wc_device_bytes gives its size (2^nbits * d * 2 bytes, zero for a
 * format without a kernel).  vq_repack_wc writes it from the canonical fp16
 * codebook wc [2^nbits][d]: for (8, 16) dimension-major, element t * 65536 + c
 * = WC[c][t]; for (4, 8) and (4, 12) an unchanged copy.  Both pointers
 * 16-byte aligned (VQ_EALIGN), not overlapping.  A load-time step,
 * asynchronous on `stream`, not part of the timed decode.
 */
size_t vq_wc_device_bytes(int32_t d, int32_t nbits);
int vq_repack_wc(const uint16_t *wc, int32_t d, int32_t nbits, void *device_layout,
                 void *stream);

/*
 * Sign-bit device layout ("tile-32x32-skew"): NP = ceil(N/32) pairs of 16
 * row groups.  Canonical sign byte p of row r holds the bits of weights
 * 8p .. 8p+7 (canonical [N][K/8], bit k%8 = weight k, 1 means +1).  Chunk
 * (tile pt = p/32, pair rp = r/32) is 1 KiB, ordered tile first; within it
 * lane L = 2 (r%32) + g (g = (p%32)/16, the 128-weight group of the tile)
 * holds 16 bytes, byte j being sign byte 32 pt + 16 g + (j ^ (r%16)) of row
 * r.  Padding rows are zero.
 */
size_t vq_signs_device_bytes(int32_t N, int32_t K);

/*
 * Alpha device layout: fp16 scale (r, g) of the canonical [N][K/128] sits at
 * element ((g/2 * NP + r/32) * 64 + 2 * (r%32) + g%2), NP = ceil(N/32),
 * padding zero -- one scale per lane of the matching sign chunk.  After the
 * scales a 256-byte header follows; its first 32-bit word is the largest
 * |alpha| as fp16 magnitude bits (written by vq_repack_alpha).  The returned
 * size includes the header.
 */
size_t vq_alpha_device_bytes(int32_t N, int32_t K, int32_t group);

/*
 * Workspace bytes needed by vq_gemv (residual = 0) or by vq_gemv_residual
 * and vq_gemv_oc (residual = 1) for these matrices and B tokens.  vq_gemv takes none (0)
 * except for (d, nbits) = (8, 16): B*K*2 bytes (rounded up to 256) per
 * matrix; the residual call needs its split-K accumulators, completion
 * counters, float partials for non-finite inputs and the rotated inputs of
 * Hadamard blocks above 2048.  Returns 0 on invalid arguments too.
 *
 * A workspace serves one call kind on one group of matrices: the (m, count,
 * B, residual) it was sized for.  Set it up with vq_workspace_init before
 * the first call of that kind and group; every vq_gemv_residual or
 * vq_gemv_oc call on that group that completes leaves its counters and accumulators at
 * zero again, so further calls on the same group need no set-up.  Before
 * the same buffer serves another group or another call kind, call
 * vq_workspace_init again: the residual call places its counters at offsets
 * that depend on the group, and the (8, 16) vq_gemv call rewrites its
 * buffer from offset 0, so either can leave non-zero bytes where the next
 * group's counters sit, and a residual call started on such bytes returns
 * wrong rows without an error.  Calls sharing one workspace must be ordered
 * (same stream or explicit dependencies).
 */
size_t vq_workspace_bytes(const vq_matrix *m, int32_t count, int32_t B,
                          int32_t residual);

/* Zero all ws_bytes of a workspace (a fill kernel, no memset). */
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

/* Canonical fp16 alpha [N][K/group] -> alpha device layout and header
 * (group == 128, K % 256 == 0). */
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
 * y[m][b][r] = sum_j OC_m[b*K/d + j][WI_m[r][j]], OC of x[m].  Each OC
 * entry x_j . WC[c] is formed when an index asks for it, from a codebook
 * held on chip (for (8, 16), one dimension of it at a time); a workgroup
 * covers whole rows.
 *   m        host array of `count` matrix descriptors.
 *   x        host array of `count` device pointers, fp16 [B][K_m] each
 *            (16-byte aligned).
 *   y        host array of `count` device pointers, fp32 [B][N_m] each
 *            (4-byte aligned), overwritten.
 *   workspace / ws_bytes  (d, nbits) = (8, 16): at least
 *            vq_workspace_bytes(m, count, B, 0) bytes, 256-byte aligned
 *            (VQ_EWORKSPACE / VQ_EALIGN otherwise): per matrix x by
 *            dimension, rewritten by every call.
 *            Other formats: unused (vq_workspace_bytes gives 0); any value.
 * All matrices are served by one kernel launch ((8, 16): a pre-pass that
 * writes x by dimension into the workspace, then the lookup kernel).  Supported:
 * (d, nbits) = (4, 8) with 1 <= B <= 4, (4, 12) with B == 1, (8, 16) with
 * 1 <= B <= 16 and K <= 65536; 1 <= count <= VQ_MAX_GROUP.  A matrix sums in
 * the same order alone or in a group.
 */
int vq_gemv(const vq_matrix *m, int32_t count, const uint16_t *const *x,
            int32_t B, float *const *y, void *workspace, size_t ws_bytes,
            void *stream);

/*
 * vq_gemv for groups whose matrices share their codebook and input [EVA 2.A:
 * one output codebook, the product of x with WC, serves the lookups of
 * every row that uses that x and WC; EVA 2.B: the codebook stays on chip
 * while indices stream].  Matrices of the group that pass the same wc and x
 * pointers and have the same K and N are merged into one unit: their row
 * groups are laid end to end and a workgroup's staged codebook and x serve
 * rows of several of them.  Results are bitwise those of vq_gemv (every
 * row's sums keep their order).  Arguments, formats, limits and errors as
 * vq_gemv; the merge applies to (d, nbits) = (4, 8) calls that take the
 * 8-wave burst kernel and is skipped otherwise.  On MI355X it measured no
 * faster than vq_gemv (LLaMA-7B q/k/v sharing one codebook and x: 5.78
 * against 5.63 us): each workgroup stages its own codebook copy either way,
 * and the member lookup adds a dependent argument load to every wave's
 * start.  vq_gemv therefore never merges.
 */
int vq_gemv_shared(const vq_matrix *m, int32_t count, const uint16_t *const *x,
                   int32_t B, float *const *y, void *workspace, size_t ws_bytes,
                   void *stream);

/*
 * vq_gemv with an fp16 epilogue: the same sums, stored as fp16 for a
 * consumer that reads fp16 (the next layer's input), so no separate
 * conversion launch follows [EVA 2.B: the epilogue unit finishes the
 * reduced outputs on chip].  y[m][b][r] is the fp32 sum vq_gemv would store,
 * rounded to the nearest fp16 value, ties to even (values beyond the fp16
 * range become infinities).  y: host array of `count` device pointers, fp16
 * [B][N_m] each (2-byte aligned), overwritten.  Formats, limits, workspace,
 * errors and ordering as vq_gemv.
 */
int vq_gemv_f16(const vq_matrix *m, int32_t count, const uint16_t *const *x,
                int32_t B, uint16_t *const *y, void *workspace, size_t ws_bytes,
                void *stream);

/*
 * VQ GEMV in the output-codebook form [EVA 2.A, 2.B]: the y of vq_gemv,
 * computed as the pages lay it out.  Each workgroup forms the output
 * codebook tile OC[j][c] = x_j . WC[c] of 64 subvectors and all 256
 * centroids in LDS (fp32, on the matrix cores), stored so that subvector
 * j's entries sit in LDS bank j mod 64 and lane j always reads them: the 64
 * lookups of a wave hit 64 different banks whatever the indices.  Rows are
 * split along K into tiles of 256 inputs; the workgroups sharing a row add
 * their partial sums with one fixed-point atomic per row (integer adds, so
 * the result does not depend on arrival order and is bitwise reproducible)
 * and the last one stores the row.  The sums run in another order than
 * vq_gemv's, so the two agree within rounding, not bitwise.
 *   Arguments as vq_gemv.  workspace / ws_bytes: at least
 *   vq_workspace_bytes(m, count, B, 1) bytes, 256-byte aligned, set up by
 *   vq_workspace_init, under the residual call's rules (a completed call
 *   leaves the counters and accumulators at zero again).  Supported: (d,
 *   nbits) = (4, 8), B == 1, K a multiple of 256, the vq_repack_wi index
 *   layout that vq_gemv reads, and below 2^31 bytes of device indices per
 *   matrix.  On MI355X vq_gemv, which forms each entry when an index asks
 *   for it and needs no cross-workgroup hand-off, measured faster; this
 *   call keeps the pages' formulation available and measurable.
 */
int vq_gemv_oc(const vq_matrix *m, int32_t count, const uint16_t *const *x,
               int32_t B, float *const *y, void *workspace, size_t ws_bytes,
               void *stream);

/*
 * Rotated VQ GEMV plus 1-bit residual [EDGE section details]: with
 * x_rot = rotation of x[m] (or x[m] itself when rht_sign is NULL),
 * y[m][b][r] = sum_j OC(x_rot)[b*K/d + j][WI[r][j]]
 *            + sum_g alpha[r][g] * sum_{k in g} s[r][k] * x_rot[b][k].
 * Each workgroup builds an output-codebook tile of 64 subvectors in LDS
 * [EVA 2.A] and workgroups sharing rows meet in one fixed-point atomic per
 * row.  Arguments as vq_gemv plus the residual fields of each vq_matrix;
 * workspace / ws_bytes at least vq_workspace_bytes(m, count, B, 1) bytes,
 * 256-byte aligned, set up by vq_workspace_init (VQ_EWORKSPACE or
 * VQ_EALIGN otherwise).  Supported: (d, nbits) = (4, 8), B == 1.
 */
int vq_gemv_residual(const vq_matrix *m, int32_t count,
                     const uint16_t *const *x, int32_t B, float *const *y,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * vq_gemv_residual for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results (bitwise) as vq_gemv_residual,
 * with the workspace replaced by a fixed scratch array in the library's
 * device code, one per GPU, kept until the process ends.  Its first
 * VQ_NOALLOC_COUNTER_BYTES hold the completion counters and fixed-point
 * accumulators, which every completed call leaves at zero; the rest of the
 * VQ_NOALLOC_SCRATCH_BYTES hold float partials and rotated inputs.  No
 * allocation, free or memset is made: the first call on a GPU looks up the
 * array's device address once (hipGetSymbolAddress).  A call whose
 * counters and accumulators need more than VQ_NOALLOC_COUNTER_BYTES, or
 * whose partials and rotated inputs need more than VQ_NOALLOC_SCRATCH_BYTES
 * - VQ_NOALLOC_COUNTER_BYTES, returns VQ_EWORKSPACE and enqueues nothing
 * (the Gemma-2-9B MLP pair 3584 -> 14336 and 14336 -> 3584 needs 0.14 MB
 * and 1.7 MB of them).  Every call on one GPU
 * shares that GPU's array: calls that may overlap (different streams
 * without ordering, or several host threads) race and give wrong results;
 * order them.  A call that does not complete (a fault) can leave counters
 * set for every later call in the process.  Other arguments, formats,
 * limits and errors as vq_gemv_residual.
 */
#define VQ_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
#define VQ_NOALLOC_COUNTER_BYTES ((size_t)1 << 20)
int vq_gemv_residual_noalloc(const vq_matrix *m, int32_t count, const uint16_t *const *x,
                             int32_t B, float *const *y, void *stream);

/*
 * Gate and up projections of a SiLU-gated MLP with the gating fused (the
 * LLaMA, Mixtral and Qwen3 models the EVA page evaluates use it): for each of
 * `count` pairs i, y[i][b][r] = silu(g)[r] * u[r], silu(z) = z / (1 + e^-z),
 * where g and u are vq_gemv of gate[i] and up[i] on the shared x[i]
 * [EVA 2.A, 2.B].  gate[i] and up[i] must have the same K, N and format;
 * one workgroup looks up both for the same rows, so the two products never
 * leave it.  Supported: (d, nbits) = (4, 8), 1 <= B <= 2, rows of at most
 * 4 * S chunks of 64 subvectors (S the split of the row, at most 8, i.e.
 * K <= 8192), VQ_EUNSUPPORTED otherwise.  workspace / ws_bytes unused.
 * Arguments otherwise as vq_gemv.
 */
int vq_gemv_swiglu(const vq_matrix *gate, const vq_matrix *up, int32_t count,
                   const uint16_t *const *x, int32_t B, float *const *y,
                   void *workspace, size_t ws_bytes, void *stream);

/*
 * vq_gemv_swiglu with an fp16 epilogue: y[i][b][r] is the fp32 gated
 * product vq_gemv_swiglu would store, rounded to the nearest fp16 value
 * (ties to even), the form the down projection's fp16 input takes, so no
 * conversion launch follows [EVA 2.B: the epilogue unit].  y: host array of
 * `count` device pointers, fp16 [B][N] each (2-byte aligned), overwritten.
 * Everything else as vq_gemv_swiglu.
 */
int vq_gemv_swiglu_f16(const vq_matrix *gate, const vq_matrix *up, int32_t count,
                       const uint16_t *const *x, int32_t B, uint16_t *const *y,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * Several tokens per call at (d, nbits) = (4, 8) on the matrix cores:
 * y[m][b][r] = sum_j x[m][b][4j..4j+3] . WC[WI[r][j]] for 1 <= B <= 16, the
 * same product as vq_gemv [EVA 2.A: the output codebook OC = X WC^T and the
 * sum of OC entries picked by the weight indices, here formed entry by entry
 * from the codebook in LDS].  Each looked-up entry serves all B tokens, so a
 * call of B tokens streams the indices once.  Unlike vq_gemv, m[i].wi is in
 * the ROW-TILE layout written by vq_repack_wi_rows, not the vq_repack_wi
 * layout: the matrix-core operand wants a lane per row.  x[m] is fp16
 * [B][K] (16-byte aligned), y[m] fp32 [B][N] (overwritten).  No workspace.
 * Requires K % 256 == 0, ceil(N/16) * 16 * K/4 < 2^31 and B * K * 2 < 2^31
 * (VQ_EUNSUPPORTED otherwise, also for other formats or B > 16; B < 1 is
 * VQ_EINVAL).  The sums of a matrix are formed in the same order alone or in
 * a group, and run to run.
 */
int vq_gemv_tokens(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                   float *const *y, void *stream);

/*
 * Row-tile layout of 8-bit indices for vq_gemv_tokens [EVA 2.B: indices
 * stream in tiles], from the canonical form (one byte per index, row r's K/4
 * indices at canonical + r * K/4, as vq_pack_indices writes it with
 * nbits = 8).  Chunk (column t of 64 subvectors, row group g of 16 rows) is
 * 1 KiB at byte (t * ceil(N/16) + g) * 1024; its 16 bytes at 16 l hold the
 * indices of row 16 g + l % 16 at subvectors 64 t + 16 (l / 16) + i, i < 16;
 * rows past N are zero.  The layout is vq_wi_device_bytes(N, K, 4, 8) bytes.
 * Load-time, asynchronous on `stream`.  Requires K % 256 == 0 and
 * ceil(N/16) * 16 * K/4 < 2^31 (VQ_EUNSUPPORTED); both pointers 16-byte
 * aligned (VQ_EALIGN).
 */
int vq_repack_wi_rows(const uint8_t *canonical, int32_t N, int32_t K, void *device_layout,
                      void *stream);

/*
 * Measurement helper, not part of the method: a plain streaming read of
 * `count` device buffers (1 <= count <= 64, each 16-byte aligned, 1 <= size
 * < 2^31 bytes) in one kernel launch.  Each workgroup of 8 wavefronts reads
 * 32 KiB; each wavefront requests four 1 KiB chunks with 16-byte
 * non-temporal loads (the index loads of the 8-bit lookup kernels) before
 * it uses the first.  Each wavefront stores the XOR of the words it read to
 * sink (uint32, sink_words >= vq_stream_read_sink_words(bytes, count),
 * 4-byte aligned; VQ_EWORKSPACE if smaller), so none of the reads can be
 * dropped.  Timed over a layer's device index layouts, its launch period
 * is the read floor of a lookup call of the same bytes.
 *   buffers  host array of `count` device pointers.
 *   bytes    host array of `count` byte counts.
 */
size_t vq_stream_read_sink_words(const size_t *bytes, int32_t count);
int vq_stream_read(const void *const *buffers, const size_t *bytes, int32_t count, uint32_t *sink,
                   size_t sink_words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VQD_H */
