// Host side of libvqd: argument validation, variant selection, workspace
// layout and kernel launches behind the C ABI of include/vqd.h.
//
// Every entry point validates all of its arguments before it enqueues
// anything; validation touches no HIP API, so an invalid call returns its
// status even on a machine without a GPU.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <string.h>

#include <algorithm>

#include "vq_internal.h"

namespace vqd {

// HIP error behind the most recent VQ_EHIP of the calling thread.
static thread_local int t_last_hip = 0;

static int hip_status(int err) {
  if (err == 0) return VQ_OK;
  t_last_hip = err;
  return VQ_EHIP;
}

static bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
static bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- shapes
// One workgroup per CU (256 CUs): the residual kernel's resident round, and
// the workgroup count the token call's row-groups-per-wave rule aims for.
static constexpr int64_t kResidentWorkgroups = 256;

// Row pairs per workgroup of a matrix with np pairs for a target run of T:
// the runs of its ceil(np / T) row blocks made as even as possible.
static int residual_pairs_per_wg(int64_t np, int T) {
  const int64_t nrb = (np + T - 1) / T;
  return (int)((np + nrb - 1) / nrb);
}

Lut8Shape lut8_shape_residual(const vq_matrix *m, int32_t count) {
  // A workgroup takes a run of 32-row pairs of one 256-input tile; wave w
  // takes pairs w, w + 16, ... of the run.  One workgroup fills a CU (its LDS
  // tables take 128 KiB) and the waves keep their loads in flight while they
  // work, so the layer is best spread over one round of workgroups with equal
  // runs: the run length T is the smallest (at least one pair per wave) for
  // which every workgroup is resident at once, up to 8 pairs per wave.
  int64_t max_k = 0;
  for (int i = 0; i < count; ++i)
    if (m[i].K > max_k) max_k = m[i].K;
  Lut8Shape s{};
  s.waves = 16;
  int T = 16;
  for (; T < 16 * 8; ++T) {
    int64_t wgs = 0;
    for (int i = 0; i < count; ++i) {
      const int64_t np = (m[i].N + 31) / 32;
      wgs += (int64_t)(m[i].K / 256) * ((np + T - 1) / T);
    }
    if (wgs <= kResidentWorkgroups) break;
  }
  s.pairs = T;
  int max_rpw = 1;
  for (int i = 0; i < count; ++i) {
    const int rpw = residual_pairs_per_wg((m[i].N + 31) / 32, T);
    if (rpw > max_rpw) max_rpw = rpw;
  }
  s.steps = 1;
  while (16 * s.steps < max_rpw) s.steps *= 2;
  // x chunks per thread for the hand-off bound: 2 cover K <= 16384, 4 cover
  // every K that the fixed-point hand-off takes (at most 127 splits)
  s.nbx = max_k > 16384 ? 4 : 2;
  return s;
}

// ---------------------------------------------------------------- workspace
struct MatPlan {
  int J, nsplit, nrb, rows_pad, rpw;
  size_t partial_off, counter_off, acc_off, xrot_off;
};

struct Plan {
  Lut8Shape shape;
  MatPlan mp[VQ_MAX_GROUP];
  size_t zero_bytes;   // counters and accumulators: [0, zero_bytes)
  size_t bytes;
  int64_t grid;
};

// Workspace plan of the residual kernel (the other kernels take none).
// Counters and accumulators come first; partials and rotated inputs start at
// scratch_base, or right after the counters when scratch_base is 0.
static void make_plan(const vq_matrix *m, int32_t count, int32_t B, Plan &p,
                      size_t scratch_base = 0) {
  p.shape = lut8_shape_residual(m, count);
  const int JT = 64;
  size_t off = 0;
  // counters and packed accumulators first (both must start at zero and are
  // left at zero by every call), then partials, then x_rot
  for (int i = 0; i < count; ++i) {
    MatPlan &q = p.mp[i];
    q.J = m[i].K / m[i].d;
    q.nsplit = (q.J + JT - 1) / JT;
    const int64_t np = (m[i].N + 31) / 32;
    q.rpw = residual_pairs_per_wg(np, p.shape.pairs);
    q.nrb = (int)((np + q.rpw - 1) / q.rpw);
    q.rows_pad = (m[i].N + 31) / 32 * 32;
    q.counter_off = off;
    off += round_up((size_t)q.nrb * sizeof(uint32_t), 256);
    q.acc_off = off;
    if (q.nsplit > 1) off += round_up((size_t)q.rows_pad * sizeof(uint64_t), 256);
  }
  p.zero_bytes = off;
  if (scratch_base > off) off = scratch_base;
  p.grid = 0;
  for (int i = 0; i < count; ++i) {
    MatPlan &q = p.mp[i];
    q.partial_off = off;
    if (q.nsplit > 1) off += round_up((size_t)q.nsplit * q.rows_pad * sizeof(float), 256);
    p.grid += (int64_t)q.nsplit * q.nrb;
  }
  for (int i = 0; i < count; ++i) {
    MatPlan &q = p.mp[i];
    q.xrot_off = off;
    off += round_up((size_t)B * m[i].K * sizeof(float), 256);
  }
  p.bytes = off;
}

// Alpha device layout: the tiled scales, then a 256-byte header whose first
// word holds the largest |alpha| as fp16 magnitude bits (written by
// vq_repack_alpha, read by the residual kernel to scale its hand-off).
static size_t alpha_body_bytes(int32_t N, int32_t K) {
  const size_t G = (size_t)(K / 128);
  return (size_t)((N + 31) / 32) * 32 * ((G + 1) / 2 * 2) * sizeof(uint16_t);
}

// ---------------------------------------------------------------- formats
// (d, nbits) pairs with a kernel: the 8-bit output-codebook tile kernels, and
// the virtual-OC kernels for 4096 and 65536 centroids.
enum Format { FMT_NONE = 0, FMT_LUT8, FMT_WC12, FMT_WC16 };

static Format format_of(int32_t d, int32_t nbits) {
  if (d == 4 && nbits == 8) return FMT_LUT8;
  if (d == 4 && nbits == 12) return FMT_WC12;
  if (d == 8 && nbits == 16) return FMT_WC16;
  return FMT_NONE;
}
static Format format_of(const vq_matrix &a) { return format_of(a.d, a.nbits); }

// ---------------------------------------------------------------- validation
static int check_matrix(const vq_matrix &a, int32_t B, bool residual) {
  if (a.K <= 0 || a.N <= 0) return VQ_EINVAL;
  if (!(a.d == 1 || a.d == 2 || a.d == 4 || a.d == 8)) return VQ_EINVAL;
  if (a.nbits < 1 || a.nbits > 16) return VQ_EINVAL;
  if (a.K % a.d) return VQ_EINVAL;
  if (!a.wi || !a.wc) return VQ_EINVAL;
  if ((int64_t)a.N * (a.K / a.d) > ((int64_t)1 << 40)) return VQ_EINVAL;
  if (residual) {
    if (!a.signs || !a.alpha) return VQ_EINVAL;
    if (a.group != 128) return VQ_EUNSUPPORTED;
    // the residual kernel addresses indices, signs and scales with 32-bit
    // buffer offsets below 2^31
    if ((int64_t)(a.N + 31) / 32 * 32 * (a.K / 4) >= ((int64_t)1 << 31)) return VQ_EUNSUPPORTED;
    if (a.rht_sign) {
      if (!is_pow2(a.had_block) || a.had_block > 16384 || a.K % a.had_block) return VQ_EINVAL;
    }
  }
  switch (format_of(a)) {
    case FMT_LUT8:
      if (B > 1 && (residual || B > 4)) return VQ_EUNSUPPORTED;   // several tokens: plain only
      break;
    case FMT_WC12: if (residual || B != 1) return VQ_EUNSUPPORTED; break;
    case FMT_WC16:
      if (residual || B > 16) return VQ_EUNSUPPORTED;
      if (!wc16t_fits(a.N, a.K / a.d, wc16t_jsplit(a.K / a.d))) return VQ_EUNSUPPORTED;
      break;
    default: return VQ_EUNSUPPORTED;
  }
  if (a.K % 256) return VQ_EUNSUPPORTED;
  if (!aligned(a.wi, 16) || !aligned(a.wc, 16)) return VQ_EALIGN;
  if (residual && (!aligned(a.signs, 16) || !aligned(a.alpha, 32))) return VQ_EALIGN;
  if (residual && a.rht_sign && !aligned(a.rht_sign, 4)) return VQ_EALIGN;
  return VQ_OK;
}

static int check_group(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                       float *const *y, bool residual, uintptr_t y_align = 4) {
  if (!m || !x || !y) return VQ_EINVAL;
  if (count < 1 || count > VQ_MAX_GROUP) return VQ_EINVAL;
  if (B < 1) return VQ_EINVAL;
  for (int i = 0; i < count; ++i) {
    const int st = check_matrix(m[i], B, residual);
    if (st != VQ_OK) return st;
    if (format_of(m[i]) != format_of(m[0])) return VQ_EUNSUPPORTED;   // one kernel per call
    if (!x[i] || !y[i]) return VQ_EINVAL;
    if (!aligned(x[i], 16)) return VQ_EALIGN;
    if (!aligned(y[i], y_align)) return VQ_EALIGN;
  }
  return VQ_OK;
}

// Workspace of the 16-bit kernel: per matrix x's values by dimension
// (B K fp16), 256-byte aligned.
static size_t wc16_ws_bytes(const vq_matrix &a, int32_t B) {
  return ((size_t)B * a.K * 2 + 255) / 256 * 256;
}

// Units of the 8-bit burst kernel: descriptors a.mat[0..count) (one matrix
// each) merged where matrices share the codebook and x pointers and have
// the same K and N (so the same split along J).  A unit of several members
// lists their indices and outputs in u.mwi / u.my from u.a.mat[k].mem0 on
// and covers nmem * ceil(N/16) row groups.  Returns false when no two
// matrices share, so the call keeps one descriptor per matrix.
static bool share_units(const WcArgs &a, WcUnitArgs &u) {
  int unit_of[VQ_MAX_GROUP];
  int nu = 0;
  int lead[VQ_MAX_GROUP];
  bool any = false;
  for (int s = 0; s < a.count; ++s) {
    const WcMat &d = a.mat[s];
    unit_of[s] = -1;
    for (int k = 0; k < nu; ++k) {
      const WcMat &l = a.mat[lead[k]];
      if (l.wc == d.wc && l.x == d.x && l.J == d.J && l.N == d.N && l.jsplit == d.jsplit) {
        unit_of[s] = k;
        any = true;
        break;
      }
    }
    if (unit_of[s] < 0) {
      lead[nu] = s;
      unit_of[s] = nu++;
    }
  }
  if (!any) return false;
  memset(&u, 0, sizeof(u));
  u.a.count = nu;
  int slot = 0;
  for (int k = 0; k < nu; ++k) {
    WcMat m = a.mat[lead[k]];
    int n = 0;
    for (int s = 0; s < a.count; ++s)
      if (unit_of[s] == k) {
        u.mwi[slot + n] = a.mat[s].wi;
        u.my[slot + n] = a.mat[s].y;
        ++n;
      }
    m.nmem = n;
    m.mem0 = slot;
    slot += n;
    const int64_t ng = (m.N + 15) / 16;
    const int per_wg = wc8_rows_per_wg(m.jsplit, wc8_burst_waves()) / 16;
    m.nwg = (int32_t)((n * ng + per_wg - 1) / per_wg);
    u.a.mat[k] = m;
  }
  return true;
}

// Virtual-OC kernels: whole rows per workgroup; only the 16-bit kernel takes
// a workspace.
static int gemv_wc(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                   void *const *y, bool yf16, void *workspace, size_t ws_bytes, void *stream,
                   bool merge = false) {
  const Format f = format_of(m[0]);
  WcArgs args;
  memset(&args, 0, sizeof(args));
  args.count = count;
  int64_t max_wg = 0;
  int max_j = 0;
  bool burst = true;   // 8-bit: every row short enough for the burst kernel
  int64_t indices = 0;
  int max_split = 1;
  // Workgroups are dispatched in grid order, matrix by matrix; the matrices
  // with the longest rows (most work per wave) go first so they do not start
  // last and set the tail.  Results do not depend on the order.
  int order[VQ_MAX_GROUP];
  for (int i = 0; i < count; ++i) order[i] = i;
  for (int a = 1; a < count; ++a)
    for (int b = a; b > 0 && m[order[b]].K / m[order[b]].d > m[order[b - 1]].K / m[order[b - 1]].d; --b) {
      const int t = order[b];
      order[b] = order[b - 1];
      order[b - 1] = t;
    }
  for (int s = 0; s < count; ++s) {
    const int i = order[s];
    WcMat &d = args.mat[s];
    d.wi = static_cast<const uint8_t *>(m[i].wi);
    d.wc = m[i].wc;
    d.x = x[i];
    d.y = static_cast<float *>(y[i]);
    d.yf16 = yf16 ? 1 : 0;
    d.J = m[i].K / m[i].d;
    d.N = m[i].N;
    d.B = B;
    d.ldy = m[i].N;
    d.jsplit = (f == FMT_LUT8)   ? wc8_jsplit(m[i].N, d.J)
               : (f == FMT_WC12) ? wc12_jsplit(d.J)
                                 : wc16t_jsplit(d.J);
    if (f == FMT_LUT8) {
      if (!wc8_burst_fits(d.N, d.J, d.jsplit)) burst = false;
      indices += (int64_t)d.N * d.J;
      if (d.jsplit > max_split) max_split = d.jsplit;
    }
    if (d.J > max_j) max_j = d.J;
  }
  const int w8 = (f == FMT_LUT8) ? wc8_waves(indices, max_split, B) : 0;
  for (int s = 0; s < count; ++s) {
    WcMat &d = args.mat[s];
    const int R = (f == FMT_LUT8)   ? wc8_rows_per_wg(d.jsplit, w8)
                  : (f == FMT_WC12) ? wc12_rows_per_wg(d.jsplit)
                                    : wc16t_rows_per_wg(d.jsplit);
    d.nwg = (d.N + R - 1) / R;
    if (d.nwg > max_wg) max_wg = d.nwg;
  }
  if (max_wg > 0x7fffffff) return VQ_EUNSUPPORTED;
  if (f == FMT_WC16) {
    Wc16tArgs t;
    memset(&t, 0, sizeof(t));
    t.a = args;
    size_t need = 0;
    int64_t maxbj = 0;
    for (int s = 0; s < count; ++s) need += wc16_ws_bytes(m[order[s]], B);
    if (!workspace || ws_bytes < need) return VQ_EWORKSPACE;
    if (!aligned(workspace, 256)) return VQ_EALIGN;
    char *w = static_cast<char *>(workspace);
    for (int s = 0; s < count; ++s) {
      const vq_matrix &a = m[order[s]];
      t.xt[s] = reinterpret_cast<uint16_t *>(w);
      w += wc16_ws_bytes(a, B);
      maxbj = std::max<int64_t>(maxbj, (int64_t)B * (a.K / a.d));
    }
    const int prep_blocks = (int)std::min<int64_t>((maxbj + 255) / 256, 4096);
    int64_t total_wg = 0;                            // the lookup kernel's flat grid
    for (int s = 0; s < count; ++s) total_wg += args.mat[s].nwg;
    if (total_wg > 0x7fffffff) return VQ_EUNSUPPORTED;
    return hip_status(launch_wc16t(t, (int)total_wg, prep_blocks, stream));
  }
  if (merge && f == FMT_LUT8 && burst && w8 == wc8_burst_waves()) {
    // vq_gemv_shared: matrices that pass the same codebook and x and have
    // the same shape become one unit; their row groups are laid end to end,
    // so a workgroup's staged codebook and x serve rows of several of them.
    WcUnitArgs u;
    if (share_units(args, u)) {
      int64_t uwg = 0;
      for (int k = 0; k < u.a.count; ++k) uwg = std::max<int64_t>(uwg, u.a.mat[k].nwg);
      if (uwg > 0x7fffffff) return VQ_EUNSUPPORTED;
      return hip_status(launch_wc8_units(u, (int)uwg, B, stream));
    }
  }
  const int err = (f == FMT_LUT8)   ? launch_wc8(args, (int)max_wg, w8, burst, B, stream)
                                    : launch_wc12(args, (int)max_wg, max_j, stream);
  return hip_status(err);
}

static int gemv_plain(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                      float *const *y, void *workspace, size_t ws_bytes, void *stream) {
  const int st = check_group(m, count, x, B, y, false);
  if (st != VQ_OK) return st;
  return gemv_wc(m, count, x, B, reinterpret_cast<void *const *>(y), false, workspace, ws_bytes, stream);
}

static int residual_launch(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                           float *const *y, const Plan &p, char *ws, void *stream,
                           bool residual = true);

static int gemv_residual(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                         float *const *y, void *workspace, size_t ws_bytes, void *stream) {
  int st = check_group(m, count, x, B, y, true);
  if (st != VQ_OK) return st;
  Plan p;
  make_plan(m, count, B, p);
  if (p.grid > 0x7fffffff) return VQ_EUNSUPPORTED;
  if (!workspace || ws_bytes < p.bytes) return VQ_EWORKSPACE;
  if (!aligned(workspace, 256)) return VQ_EALIGN;
  return residual_launch(m, count, x, B, y, p, static_cast<char *>(workspace), stream);
}

// The residual call on this GPU's fixed device scratch: counters and
// accumulators within its zero region, partials and rotated inputs above it.
static int gemv_residual_noalloc(const vq_matrix *m, int32_t count, const uint16_t *const *x,
                                 int32_t B, float *const *y, void *stream) {
  int st = check_group(m, count, x, B, y, true);
  if (st != VQ_OK) return st;
  Plan p;
  make_plan(m, count, B, p, VQ_NOALLOC_COUNTER_BYTES);
  if (p.grid > 0x7fffffff) return VQ_EUNSUPPORTED;
  if (p.zero_bytes > VQ_NOALLOC_COUNTER_BYTES || p.bytes > VQ_NOALLOC_SCRATCH_BYTES)
    return VQ_EWORKSPACE;
  void *ws = nullptr;
  const int err = noalloc_scratch(&ws);
  if (err) return hip_status(err);
  return residual_launch(m, count, x, B, y, p, static_cast<char *>(ws), stream);
}

// The output-codebook form of the plain call: the residual call's kernel,
// plan and workspace with no rotation and no residual term.
static int gemv_oc(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                   float *const *y, void *workspace, size_t ws_bytes, void *stream) {
  int st = check_group(m, count, x, B, y, false);
  if (st != VQ_OK) return st;
  if (format_of(m[0]) != FMT_LUT8 || B != 1) return VQ_EUNSUPPORTED;
  for (int i = 0; i < count; ++i)
    if ((int64_t)(m[i].N + 31) / 32 * 32 * (m[i].K / 4) >= ((int64_t)1 << 31)) return VQ_EUNSUPPORTED;
  Plan p;
  make_plan(m, count, B, p);
  if (p.grid > 0x7fffffff) return VQ_EUNSUPPORTED;
  if (!workspace || ws_bytes < p.bytes) return VQ_EWORKSPACE;
  if (!aligned(workspace, 256)) return VQ_EALIGN;
  return residual_launch(m, count, x, B, y, p, static_cast<char *>(workspace), stream, false);
}

static int residual_launch(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                           float *const *y, const Plan &p, char *ws, void *stream, bool residual) {
  Lut8Args args;
  memset(&args, 0, sizeof(args));
  args.count = count;
  int max_wg = 0;
  for (int i = 0; i < count; ++i) {
    const MatPlan &q = p.mp[i];
    Lut8Mat &d = args.mat[i];
    d.wi = static_cast<const uint8_t *>(m[i].wi);
    d.wc = m[i].wc;
    d.x = x[i];
    d.xr = reinterpret_cast<const float *>(ws + q.xrot_off);
    d.signs = residual ? static_cast<const uint8_t *>(m[i].signs) : nullptr;
    d.alpha = residual ? static_cast<const uint16_t *>(m[i].alpha) : nullptr;
    d.y = y[i];
    d.partial = q.nsplit > 1 ? reinterpret_cast<float *>(ws + q.partial_off) : nullptr;
    d.counter = reinterpret_cast<uint32_t *>(ws + q.counter_off);
    d.J = q.J;
    d.N = m[i].N;
    d.rows_pad = q.rows_pad;
    d.nsplit = q.nsplit;
    d.nrb = q.nrb;
    d.rpw = q.rpw;
    d.acc = reinterpret_cast<uint64_t *>(ws + q.acc_off);
    const int h = residual && m[i].rht_sign ? m[i].had_block : 1;
    d.rs = residual ? m[i].rht_sign : nullptr;
    d.had = h;
    d.had_scale = (float)(1.0 / sqrt((double)h));
    d.alpha_hdr = residual ? reinterpret_cast<const uint32_t *>(static_cast<const char *>(m[i].alpha) +
                                                                alpha_body_bytes(m[i].N, m[i].K))
                           : nullptr;
    // blocks up to 2048 are rotated inside the lookup kernel; larger ones first
    // by the rotation kernel, into the workspace
    d.fused = h <= 2048 ? 1 : 0;
    d.nwg = q.nsplit * q.nrb;
    if (d.nwg > max_wg) max_wg = d.nwg;
  }
  int err;
  for (int i = 0; i < count; ++i) {
    if (args.mat[i].fused) continue;          // rotated inside the lookup kernel
    const int h = args.mat[i].had;
    err = launch_rht(x[i], m[i].rht_sign, B, m[i].K, h, args.mat[i].had_scale,
                     reinterpret_cast<float *>(ws + p.mp[i].xrot_off), stream);
    if (err) return hip_status(err);
  }
  err = launch_lut8_residual(args, p.shape, max_wg, stream, residual);
  return hip_status(err);
}

}  // namespace vqd

using namespace vqd;

extern "C" {

const char *vq_status_str(int status) {
  switch (status) {
    case VQ_OK: return "VQ_OK";
    case VQ_EINVAL: return "VQ_EINVAL: invalid argument";
    case VQ_EUNSUPPORTED: return "VQ_EUNSUPPORTED: shape or format not supported";
    case VQ_EALIGN: return "VQ_EALIGN: pointer misaligned";
    case VQ_EWORKSPACE: return "VQ_EWORKSPACE: workspace missing or too small";
    case VQ_EHIP: return "VQ_EHIP: HIP runtime error";
    default: return "unknown";
  }
}

const char *vq_last_error(void) {
  if (t_last_hip == 0) return "no HIP error";
  return hipGetErrorString(static_cast<hipError_t>(t_last_hip));
}

size_t vq_wi_device_bytes(int32_t N, int32_t K, int32_t d, int32_t nbits) {
  if (N <= 0 || K <= 0 || d <= 0 || K % d) return 0;
  const int64_t J = K / d;
  const size_t rows = (size_t)((N + 15) / 16) * 16;
  switch (format_of(d, nbits)) {
    case FMT_LUT8: return (J % 64) ? 0 : rows * (size_t)J;
    case FMT_WC12: return (J % 64) ? 0 : rows * (size_t)J * 3 / 2;
    case FMT_WC16: return (J % 32) ? 0 : rows * (size_t)J * 2;
    default: return 0;
  }
}

size_t vq_wc_device_bytes(int32_t d, int32_t nbits) {
  if (format_of(d, nbits) == FMT_NONE) return 0;
  return ((size_t)1 << nbits) * (size_t)d * 2;
}

int vq_repack_wc(const uint16_t *wc, int32_t d, int32_t nbits, void *device_layout, void *stream) {
  if (!wc || !device_layout) return VQ_EINVAL;
  const Format f = format_of(d, nbits);
  if (f == FMT_NONE) return VQ_EUNSUPPORTED;
  if (!aligned(wc, 16) || !aligned(device_layout, 16)) return VQ_EALIGN;
  if (f != FMT_WC16) {                 // the canonical layout is the device layout
    const size_t n = vq_wc_device_bytes(d, nbits);
    return hip_status((int)hipMemcpyAsync(device_layout, wc, n, hipMemcpyDeviceToDevice,
                                          reinterpret_cast<hipStream_t>(stream)));
  }
  return hip_status(launch_repack_wc16(wc, static_cast<uint16_t *>(device_layout), stream));
}

size_t vq_signs_device_bytes(int32_t N, int32_t K) {
  if (N <= 0 || K <= 0 || K % 256) return 0;
  return (size_t)((N + 31) / 32) * 32 * (size_t)(K / 8);
}

size_t vq_alpha_device_bytes(int32_t N, int32_t K, int32_t group) {
  if (N <= 0 || K <= 0 || group != 128 || K % 256) return 0;
  return alpha_body_bytes(N, K) + 256;
}

size_t vq_workspace_bytes(const vq_matrix *m, int32_t count, int32_t B, int32_t residual) {
  if (!m || count < 1 || count > VQ_MAX_GROUP || B < 1) return 0;
  for (int i = 0; i < count; ++i) {
    const vq_matrix &a = m[i];
    if (a.K <= 0 || a.N <= 0 || a.d <= 0 || a.K % a.d) return 0;
  }
  if (!residual && format_of(m[0]) == FMT_WC16) {
    size_t n = 0;
    for (int i = 0; i < count; ++i) n += wc16_ws_bytes(m[i], B);
    return n;
  }
  if (!residual || format_of(m[0]) != FMT_LUT8) return 0;   // only the residual kernel takes one
  Plan p;
  make_plan(m, count, B, p);
  return p.bytes;
}

int vq_workspace_init(void *workspace, size_t ws_bytes, void *stream) {
  if (ws_bytes == 0) return VQ_OK;
  if (!workspace) return VQ_EINVAL;
  if (!aligned(workspace, 256)) return VQ_EALIGN;
  return hip_status(launch_fill_u32(static_cast<uint32_t *>(workspace), ws_bytes / 4, 0u, stream));
}

int vq_pack_indices(const uint32_t *idx, int64_t count, int32_t nbits, uint8_t *out, void *stream) {
  if (nbits < 1 || nbits > 16 || count < 0) return VQ_EINVAL;
  if (count == 0) return VQ_OK;
  if (!idx || !out) return VQ_EINVAL;
  if (!aligned(idx, 4)) return VQ_EALIGN;
  return hip_status(launch_pack(idx, count, nbits, out, stream));
}

int vq_unpack_indices(const uint8_t *packed, int64_t count, int32_t nbits, uint32_t *out, void *stream) {
  if (nbits < 1 || nbits > 16 || count < 0) return VQ_EINVAL;
  if (count == 0) return VQ_OK;
  if (!packed || !out) return VQ_EINVAL;
  if (!aligned(out, 4)) return VQ_EALIGN;
  return hip_status(launch_unpack(packed, count, nbits, out, stream));
}

int vq_repack_wi(const uint8_t *canonical, int32_t N, int32_t K, int32_t d, int32_t nbits,
                 void *device_layout, void *stream) {
  if (!canonical || !device_layout) return VQ_EINVAL;
  if (N <= 0 || K <= 0 || d <= 0 || K % d || nbits < 1 || nbits > 16) return VQ_EINVAL;
  if (vq_wi_device_bytes(N, K, d, nbits) == 0) return VQ_EUNSUPPORTED;
  if (!aligned(device_layout, 16)) return VQ_EALIGN;
  uint8_t *dev = static_cast<uint8_t *>(device_layout);
  switch (format_of(d, nbits)) {
    case FMT_LUT8: return hip_status(launch_repack_wi8(canonical, N, K / d, dev, stream));
    case FMT_WC12: return hip_status(launch_repack_wi12(canonical, N, K / d, dev, stream));
    case FMT_WC16:
      if (!aligned(canonical, 2)) return VQ_EALIGN;
      return hip_status(launch_repack_wi16(canonical, N, K / d, dev, stream));
    default: return VQ_EUNSUPPORTED;
  }
}

int vq_repack_wi_rows(const uint8_t *canonical, int32_t N, int32_t K, void *device_layout, void *stream) {
  if (!canonical || !device_layout || N <= 0 || K <= 0) return VQ_EINVAL;
  if (K % 256) return VQ_EUNSUPPORTED;
  if ((int64_t)(N + 15) / 16 * 16 * (K / 4) >= ((int64_t)1 << 31)) return VQ_EUNSUPPORTED;
  if (!aligned(canonical, 16) || !aligned(device_layout, 16)) return VQ_EALIGN;
  return hip_status(launch_repack_wi8_rows(canonical, N, K / 4, static_cast<uint8_t *>(device_layout), stream));
}

int vq_repack_signs(const uint8_t *canonical, int32_t N, int32_t K, void *device_layout, void *stream) {
  if (!canonical || !device_layout || N <= 0 || K <= 0 || K % 8) return VQ_EINVAL;
  if (vq_signs_device_bytes(N, K) == 0) return VQ_EUNSUPPORTED;
  if (!aligned(device_layout, 16)) return VQ_EALIGN;
  return hip_status(launch_repack_signs(canonical, N, K / 8, static_cast<uint8_t *>(device_layout), stream));
}

int vq_repack_alpha(const uint16_t *canonical, int32_t N, int32_t K, int32_t group, void *device_layout,
                    void *stream) {
  if (!canonical || !device_layout || N <= 0 || K <= 0 || group <= 0 || K % group) return VQ_EINVAL;
  if (vq_alpha_device_bytes(N, K, group) == 0) return VQ_EUNSUPPORTED;
  if (!aligned(canonical, 2) || !aligned(device_layout, 32)) return VQ_EALIGN;
  uint32_t *hdr = reinterpret_cast<uint32_t *>(static_cast<char *>(device_layout) + alpha_body_bytes(N, K));
  return hip_status(launch_repack_alpha(canonical, N, K / group, static_cast<uint16_t *>(device_layout), hdr,
                                        stream));
}

int vq_build_oc(const uint16_t *x, int32_t B, int32_t K, int32_t d, int32_t nbits, const uint16_t *wc,
                void *oc, vq_dtype oc_dtype, void *stream) {
  if (!x || !wc || !oc) return VQ_EINVAL;
  if (B < 1 || K <= 0 || !(d == 1 || d == 2 || d == 4 || d == 8) || K % d) return VQ_EINVAL;
  if (nbits < 1 || nbits > 16) return VQ_EINVAL;
  if (oc_dtype != VQ_F16 && oc_dtype != VQ_F32) return VQ_EINVAL;
  if ((int64_t)B * (K / d) > ((int64_t)1 << 40) >> nbits) return VQ_EINVAL;
  if (!aligned(x, 2) || !aligned(wc, 2) || !aligned(oc, oc_dtype == VQ_F32 ? 4 : 2)) return VQ_EALIGN;
  return hip_status(launch_build_oc(x, B, K, d, nbits, wc, oc, oc_dtype == VQ_F16, stream));
}

int vq_rht(const uint16_t *x, const int8_t *sign, int32_t B, int32_t K, int32_t had_block, float *x_rot,
           void *stream) {
  if (!x || !sign || !x_rot) return VQ_EINVAL;
  if (B < 1 || K <= 0 || !is_pow2(had_block) || had_block > 16384 || K % had_block) return VQ_EINVAL;
  if ((int64_t)B * (K / had_block) > 0x7fffffff) return VQ_EINVAL;
  if (!aligned(x, 2) || !aligned(x_rot, 4)) return VQ_EALIGN;
  const float scale = (float)(1.0 / sqrt((double)had_block));
  return hip_status(launch_rht(x, sign, B, K, had_block, scale, x_rot, stream));
}

int vq_gemv(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B, float *const *y,
            void *workspace, size_t ws_bytes, void *stream) {
  return gemv_plain(m, count, x, B, y, workspace, ws_bytes, stream);
}

int vq_gemv_shared(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                   float *const *y, void *workspace, size_t ws_bytes, void *stream) {
  const int st = check_group(m, count, x, B, y, false);
  if (st != VQ_OK) return st;
  return gemv_wc(m, count, x, B, reinterpret_cast<void *const *>(y), false, workspace, ws_bytes,
                 stream, true);
}

int vq_gemv_residual(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                     float *const *y, void *workspace, size_t ws_bytes, void *stream) {
  return gemv_residual(m, count, x, B, y, workspace, ws_bytes, stream);
}

int vq_gemv_oc(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
               float *const *y, void *workspace, size_t ws_bytes, void *stream) {
  return gemv_oc(m, count, x, B, y, workspace, ws_bytes, stream);
}

int vq_gemv_residual_noalloc(const vq_matrix *m, int32_t count, const uint16_t *const *x,
                             int32_t B, float *const *y, void *stream) {
  return gemv_residual_noalloc(m, count, x, B, y, stream);
}

int vq_gemv_f16(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                uint16_t *const *y, void *workspace, size_t ws_bytes, void *stream) {
  const int st = check_group(m, count, x, B, reinterpret_cast<float *const *>(y), false, 2);
  if (st != VQ_OK) return st;
  return gemv_wc(m, count, x, B, reinterpret_cast<void *const *>(y), true, workspace, ws_bytes, stream);
}

static int gemv_swiglu(const vq_matrix *gate, const vq_matrix *up, int32_t count,
                       const uint16_t *const *x, int32_t B, void *const *y, bool yf16,
                       void *stream) {
  if (!up) return VQ_EINVAL;
  int st = check_group(gate, count, x, B, reinterpret_cast<float *const *>(y), false, yf16 ? 2 : 4);
  if (st != VQ_OK) return st;
  for (int i = 0; i < count; ++i) {
    st = check_matrix(up[i], B, false);
    if (st != VQ_OK) return st;
    if (up[i].K != gate[i].K || up[i].N != gate[i].N || up[i].d != gate[i].d ||
        up[i].nbits != gate[i].nbits)
      return VQ_EINVAL;
  }
  if (format_of(gate[0]) != FMT_LUT8 || B > 2) return VQ_EUNSUPPORTED;
  WcPairArgs args;
  memset(&args, 0, sizeof(args));
  args.a.count = count;
  // longest rows first, as in the plain call; the split is the plain one
  int order[VQ_MAX_GROUP];
  for (int i = 0; i < count; ++i) order[i] = i;
  for (int a = 1; a < count; ++a)
    for (int b = a; b > 0 && gate[order[b]].K > gate[order[b - 1]].K; --b) {
      const int t = order[b];
      order[b] = order[b - 1];
      order[b - 1] = t;
    }
  int max_split = 1;
  for (int s = 0; s < count; ++s) {
    const int i = order[s];
    WcMat &d = args.a.mat[s];
    d.wi = static_cast<const uint8_t *>(gate[i].wi);
    d.wc = gate[i].wc;
    d.x = x[i];
    d.y = static_cast<float *>(y[i]);
    d.yf16 = yf16 ? 1 : 0;
    d.J = gate[i].K / gate[i].d;
    d.N = gate[i].N;
    d.B = B;
    d.ldy = gate[i].N;
    d.jsplit = wc8_jsplit(d.N, d.J);
    if (!wc8_burst_fits(d.N, d.J, d.jsplit)) return VQ_EUNSUPPORTED;
    if (d.jsplit > max_split) max_split = d.jsplit;
    args.wi2[s] = static_cast<const uint8_t *>(up[i].wi);
    args.wc2[s] = up[i].wc;
  }
  // two row-group slots (gate, up) per output row group
  const int waves = wc8_swiglu_waves(max_split);
  int64_t max_wg = 0;
  for (int s = 0; s < count; ++s) {
    WcMat &d = args.a.mat[s];
    const int R = waves / d.jsplit / 2 * 16;
    d.nwg = (d.N + R - 1) / R;
    if (d.nwg > max_wg) max_wg = d.nwg;
  }
  if (max_wg > 0x7fffffff) return VQ_EUNSUPPORTED;
  return hip_status(launch_wc8_swiglu(args, (int)max_wg, waves, B, stream));
}

int vq_gemv_swiglu(const vq_matrix *gate, const vq_matrix *up, int32_t count,
                   const uint16_t *const *x, int32_t B, float *const *y, void *workspace,
                   size_t ws_bytes, void *stream) {
  (void)workspace;
  (void)ws_bytes;
  return gemv_swiglu(gate, up, count, x, B, reinterpret_cast<void *const *>(y), false, stream);
}

int vq_gemv_swiglu_f16(const vq_matrix *gate, const vq_matrix *up, int32_t count,
                       const uint16_t *const *x, int32_t B, uint16_t *const *y, void *workspace,
                       size_t ws_bytes, void *stream) {
  (void)workspace;
  (void)ws_bytes;
  return gemv_swiglu(gate, up, count, x, B, reinterpret_cast<void *const *>(y), true, stream);
}

int vq_gemv_tokens(const vq_matrix *m, int32_t count, const uint16_t *const *x, int32_t B,
                   float *const *y, void *stream) {
  if (B < 1) return VQ_EINVAL;
  int st = check_group(m, count, x, 1, y, false);
  if (st != VQ_OK) return st;
  if (format_of(m[0]) != FMT_LUT8 || B > 16) return VQ_EUNSUPPORTED;
  for (int i = 0; i < count; ++i) {
    // 32-bit buffer offsets: the row tiles and x below 2^31 bytes
    if ((int64_t)(m[i].N + 15) / 16 * 16 * (m[i].K / 4) >= ((int64_t)1 << 31)) return VQ_EUNSUPPORTED;
    if ((int64_t)B * m[i].K * 2 >= ((int64_t)1 << 31)) return VQ_EUNSUPPORTED;
  }
  WcArgs args;
  memset(&args, 0, sizeof(args));
  args.count = count;
  for (int i = 0; i < count; ++i) {
    WcMat &d = args.mat[i];
    d.wi = static_cast<const uint8_t *>(m[i].wi);
    d.wc = m[i].wc;
    d.x = x[i];
    d.y = y[i];
    d.J = m[i].K / 4;
    d.N = m[i].N;
    d.B = B;
    d.ldy = m[i].N;
    d.jsplit = wc8t_jsplit(d.J, B);
  }
  // row groups per wave: the most (up to wc8t_max_rw(B)) that still gives
  // the call 256 workgroups; it changes which wave adds a row, not the order
  // of its sums
  int rw = wc8t_max_rw(B);
  for (; rw > 1; rw /= 2) {
    int64_t wgs = 0;
    for (int i = 0; i < count; ++i) {
      const int R = wc8t_rows_per_wg(args.mat[i].jsplit, rw);
      wgs += (args.mat[i].N + R - 1) / R;
    }
    if (wgs >= kResidentWorkgroups) break;
  }
  int64_t max_wg = 0;
  for (int i = 0; i < count; ++i) {
    WcMat &d = args.mat[i];
    const int R = wc8t_rows_per_wg(d.jsplit, rw);
    d.nwg = (d.N + R - 1) / R;
    if (d.nwg > max_wg) max_wg = d.nwg;
  }
  if (max_wg > 0x7fffffff) return VQ_EUNSUPPORTED;
  return hip_status(launch_wc8t(args, (int)max_wg, rw, stream));
}

size_t vq_stream_read_sink_words(const size_t *bytes, int32_t count) {
  if (!bytes || count < 1 || count > VQ_MAX_READ) return 0;
  size_t mx = 0;
  for (int i = 0; i < count; ++i) {
    if (bytes[i] == 0 || bytes[i] >= ((size_t)1 << 31)) return 0;
    mx = std::max(mx, bytes[i]);
  }
  return (size_t)count * (size_t)stream_read_workgroups((uint32_t)mx) *
         (size_t)stream_read_sink_words_per_wg();
}

int vq_stream_read(const void *const *buffers, const size_t *bytes, int32_t count, uint32_t *sink,
                   size_t sink_words, void *stream) {
  if (!buffers || !bytes || !sink || count < 1) return VQ_EINVAL;
  if (count > VQ_MAX_READ) return VQ_EUNSUPPORTED;
  const size_t need = vq_stream_read_sink_words(bytes, count);
  if (need == 0) return VQ_EINVAL;
  if (sink_words < need) return VQ_EWORKSPACE;
  if (!aligned(sink, 4)) return VQ_EALIGN;
  ReadArgs a;
  memset(&a, 0, sizeof(a));
  a.count = count;
  a.sink = sink;
  size_t mx = 0;
  for (int i = 0; i < count; ++i) {
    if (!buffers[i]) return VQ_EINVAL;
    if (!aligned(buffers[i], 16)) return VQ_EALIGN;
    a.buf[i] = static_cast<const uint8_t *>(buffers[i]);
    a.bytes[i] = (uint32_t)bytes[i];
    mx = std::max(mx, bytes[i]);
  }
  return hip_status(launch_stream_read(a, (int)stream_read_workgroups((uint32_t)mx), stream));
}

}  // extern "C"
