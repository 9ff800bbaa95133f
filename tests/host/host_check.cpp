// Host checks of libvqd's C ABI without a GPU: the library's host code
// (vq_api.cpp, vq_shapes.cpp) is built with g++ and the address and
// undefined-behaviour sanitizers against this file, which stands in for the
// kernel launchers and the two HIP runtime calls the host code makes.  Each
// launcher records its arguments instead of launching, so the checks below
// can verify what every call would hand to its kernel: grids that cover
// every row, splits and chunk counts the kernels are built for, 32-bit
// buffer offsets below 2^31, and workspace regions inside the caller's
// buffer (or the no-allocation scratch) without overlaps.  No pointer passed
// here is ever dereferenced.
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../vector_quantized_decode_amd/csrc/vq_internal.h"

// ------------------------------------------------------------------ stand-ins
namespace {
enum Kind { NONE, WC8, WC8_UNITS, WC12, WC16T, SWIGLU, WC8T, RESIDUAL, OCTILE, READ, OTHER };
struct Last {
  Kind kind = NONE;
  int grid_x = 0, waves = 0, B = 0, rw = 0, prep_blocks = 0;
  bool burst = false;
  vqd::WcArgs wc;
  vqd::WcUnitArgs units;
  vqd::Wc16tArgs w16;
  vqd::WcPairArgs pair;
  vqd::Lut8Args res;
  vqd::Lut8Shape shape;
  vqd::ReadArgs rd;
  std::vector<vqd::ReadArgs> rhts;
} last;
uintptr_t g_scratch = 0x7e0000000000ull;   // stand-in device address of the scratch
int failures = 0;
}  // namespace

#define CHECK(cond, ...)                                                     \
  do {                                                                       \
    if (!(cond)) {                                                           \
      ++failures;                                                            \
      fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond);        \
      fprintf(stderr, __VA_ARGS__);                                          \
      fprintf(stderr, "\n");                                                 \
    }                                                                        \
  } while (0)

extern "C" {
const char *hipGetErrorString(hipError_t) { return "stand-in"; }
hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) {
  last.kind = OTHER;
  return hipSuccess;
}
}

namespace vqd {
int launch_wc8(const WcArgs &a, int grid_x, int waves, bool burst, int B, void *) {
  last = Last();
  last.kind = WC8; last.wc = a; last.grid_x = grid_x; last.waves = waves; last.burst = burst; last.B = B;
  return 0;
}
int launch_wc8_units(const WcUnitArgs &a, int grid_x, int B, void *) {
  last = Last();
  last.kind = WC8_UNITS; last.units = a; last.grid_x = grid_x; last.B = B;
  return 0;
}
int launch_wc12(const WcArgs &a, int grid_x, int, void *) {
  last = Last();
  last.kind = WC12; last.wc = a; last.grid_x = grid_x;
  return 0;
}
int launch_wc8_swiglu(const WcPairArgs &a, int grid_x, int waves, int B, void *) {
  last = Last();
  last.kind = SWIGLU; last.pair = a; last.grid_x = grid_x; last.waves = waves; last.B = B;
  return 0;
}
int launch_wc8t(const WcArgs &a, int grid_x, int rw, void *) {
  last = Last();
  last.kind = WC8T; last.wc = a; last.grid_x = grid_x; last.rw = rw;
  return 0;
}
int launch_wc16t(const Wc16tArgs &a, int grid_x, int prep_blocks, void *) {
  last = Last();
  last.kind = WC16T; last.w16 = a; last.grid_x = grid_x; last.prep_blocks = prep_blocks;
  return 0;
}
int launch_lut8_residual(const Lut8Args &a, const Lut8Shape &s, int grid_x, void *, bool residual) {
  last.kind = residual ? RESIDUAL : OCTILE; last.res = a; last.shape = s; last.grid_x = grid_x;
  return 0;
}
int launch_rht(const uint16_t *, const int8_t *, int, int, int, float, float *, void *) {
  last = Last();                           // the rotation launch precedes the lookup launch
  return 0;
}
int launch_stream_read(const ReadArgs &a, int grid_x, void *) {
  last = Last();
  last.kind = READ; last.rd = a; last.grid_x = grid_x;
  return 0;
}
int launch_repack_wi8_rows(const uint8_t *, int, int, uint8_t *, void *) { last.kind = OTHER; return 0; }
int launch_repack_wc16(const uint16_t *, uint16_t *, void *) { last.kind = OTHER; return 0; }
int launch_repack_wi12(const uint8_t *, int, int, uint8_t *, void *) { last.kind = OTHER; return 0; }
int launch_repack_wi16(const uint8_t *, int, int, uint8_t *, void *) { last.kind = OTHER; return 0; }
int launch_pack(const uint32_t *, int64_t, int, uint8_t *, void *) { last.kind = OTHER; return 0; }
int launch_unpack(const uint8_t *, int64_t, int, uint32_t *, void *) { last.kind = OTHER; return 0; }
int launch_repack_wi8(const uint8_t *, int, int, uint8_t *, void *) { last.kind = OTHER; return 0; }
int launch_repack_signs(const uint8_t *, int, int, uint8_t *, void *) { last.kind = OTHER; return 0; }
int launch_repack_alpha(const uint16_t *, int, int, uint16_t *, uint32_t *, void *) { last.kind = OTHER; return 0; }
int launch_build_oc(const uint16_t *, int, int, int, int, const uint16_t *, void *, int, void *) {
  last.kind = OTHER;
  return 0;
}
int launch_fill_u32(uint32_t *, size_t, uint32_t, void *) { last.kind = OTHER; return 0; }
int noalloc_scratch(void **out) {
  *out = reinterpret_cast<void *>(g_scratch);
  return 0;
}
}  // namespace vqd

// ------------------------------------------------------------------ helpers
namespace {
const uintptr_t FAKE = 0x7f0000000000ull;   // 256-byte aligned, never dereferenced
void *P(uintptr_t off = 0) { return reinterpret_cast<void *>(FAKE + off); }

vq_matrix mat(int K, int N, int d = 4, int nbits = 8) {
  vq_matrix m;
  memset(&m, 0, sizeof(m));
  m.K = K; m.N = N; m.d = d; m.nbits = nbits;
  m.wi = P(); m.wc = static_cast<const uint16_t *>(P(0x100000));
  m.signs = P(0x200000); m.alpha = P(0x300000); m.group = 128;
  return m;
}

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Every WcMat of a plain 8/12/16-bit launch: the rows its workgroups cover,
// its split, and the offsets its kernel forms.
void check_wcmats(const vqd::WcArgs &a, int grid_x, Kind kind, int waves, bool burst, const vq_matrix *m,
                  int count, int B) {
  CHECK(a.count == count, "count %d vs %d", a.count, count);
  int64_t maxwg = 0;
  for (int s = 0; s < a.count; ++s) {
    const vqd::WcMat &d = a.mat[s];
    CHECK(d.B == B, "B");
    if (kind != WC16T) CHECK(pow2(d.jsplit), "split %d not a power of two", d.jsplit);
    const int64_t NG = (d.N + 15) / 16;
    int rows_per_wg = 0;
    if (kind == WC8) {
      CHECK(d.jsplit <= waves, "split %d > waves %d", d.jsplit, waves);
      rows_per_wg = vqd::wc8_rows_per_wg(d.jsplit, waves);
      const int JT = d.J / 64;
      CHECK(d.J % 64 == 0, "J %d", d.J);
      if (burst) {
        CHECK((JT + d.jsplit - 1) / d.jsplit <= vqd::WC8_NCH, "burst segment of %d chunks",
              (JT + d.jsplit - 1) / d.jsplit);
        CHECK(NG * 1024 * JT < ((int64_t)1 << 31), "burst buffer of %lld bytes", (long long)(NG * 1024 * JT));
        CHECK((int64_t)d.B * d.J * 8 < ((int64_t)1 << 31), "x buffer");
      }
    } else if (kind == WC12) {
      rows_per_wg = vqd::wc12_rows_per_wg(d.jsplit);
      CHECK(d.jsplit <= vqd::WC12_W, "split");
    } else if (kind == WC16T) {
      rows_per_wg = vqd::wc16t_rows_per_wg(d.jsplit);
      const int JB = d.J / 32;
      CHECK(d.jsplit >= 1 && d.jsplit <= 16 && rows_per_wg >= 16, "16-bit split %d", d.jsplit);
      CHECK((JB + d.jsplit - 1) / d.jsplit <= 16, "16-bit segment of %d blocks", (JB + d.jsplit - 1) / d.jsplit);
      // the S segments of ceil(JB / S) blocks cover the row
      const int seg = (JB + d.jsplit - 1) / d.jsplit;
      CHECK((int64_t)seg * d.jsplit >= JB, "16-bit segments miss blocks: JB=%d S=%d", JB, d.jsplit);
      CHECK(NG * JB * 1024 < ((int64_t)1 << 31), "16-bit buffer");
    }
    CHECK((int64_t)d.nwg * rows_per_wg >= d.N, "rows %d not covered: %d x %d", d.N, d.nwg, rows_per_wg);
    CHECK((int64_t)(d.nwg - 1) * rows_per_wg < d.N, "an idle workgroup");
    maxwg = std::max<int64_t>(maxwg, d.nwg);
    bool found = false;
    for (int i = 0; i < count; ++i)
      if (d.wi == static_cast<const uint8_t *>(m[i].wi) && d.N == m[i].N && d.J == m[i].K / m[i].d) found = true;
    CHECK(found, "descriptor %d matches no matrix", s);
  }
  if (kind == WC16T) {                              // a flat grid of every workgroup
    int64_t total = 0;
    for (int s = 0; s < a.count; ++s) total += a.mat[s].nwg;
    CHECK(grid_x == total, "16-bit grid %d vs %lld", grid_x, (long long)total);
  } else {
    CHECK(grid_x == maxwg, "grid %d vs %lld", grid_x, (long long)maxwg);
  }
}

int gemv(vq_matrix *m, int count, int B, void *ws = nullptr, size_t wsb = 0) {
  std::vector<const uint16_t *> x(count);
  std::vector<float *> y(count);
  for (int i = 0; i < count; ++i) {
    x[i] = static_cast<const uint16_t *>(P(0x400000 + 0x10000 * i));
    y[i] = static_cast<float *>(P(0x800000 + 0x10000 * i));
  }
  return vq_gemv(m, count, x.data(), B, y.data(), ws, wsb, nullptr);
}

// ------------------------------------------------------------------ checks
void check_validation() {
  vq_matrix m = mat(1024, 64);
  const uint16_t *x[2] = {static_cast<const uint16_t *>(P()), static_cast<const uint16_t *>(P())};
  float *y[2] = {static_cast<float *>(P()), static_cast<float *>(P())};
  CHECK(vq_gemv(&m, 0, x, 1, y, nullptr, 0, nullptr) == VQ_EINVAL, "count 0");
  CHECK(vq_gemv(&m, 1, nullptr, 1, y, nullptr, 0, nullptr) == VQ_EINVAL, "x null");
  CHECK(vq_gemv(&m, 1, x, 0, y, nullptr, 0, nullptr) == VQ_EINVAL, "B 0");
  CHECK(vq_gemv(&m, 1, x, 5, y, nullptr, 0, nullptr) == VQ_EUNSUPPORTED, "B 5");
  vq_matrix bad = mat(1088, 64);
  CHECK(vq_gemv(&bad, 1, x, 1, y, nullptr, 0, nullptr) == VQ_EUNSUPPORTED, "K %% 256");
  bad = mat(1024, 64, 3, 8);
  CHECK(vq_gemv(&bad, 1, x, 1, y, nullptr, 0, nullptr) == VQ_EINVAL, "d 3");
  bad = mat(1024, 64);
  bad.wi = P(8);
  CHECK(vq_gemv(&bad, 1, x, 1, y, nullptr, 0, nullptr) == VQ_EALIGN, "wi alignment");
  vq_matrix many[17];
  for (auto &q : many) q = mat(1024, 64);
  std::vector<const uint16_t *> xs(17, static_cast<const uint16_t *>(P()));
  std::vector<float *> ys(17, static_cast<float *>(P()));
  CHECK(vq_gemv(many, 17, xs.data(), 1, ys.data(), nullptr, 0, nullptr) == VQ_EINVAL, "17 matrices");
  CHECK(vq_gemv_tokens(&m, 1, x, 17, y, nullptr) == VQ_EUNSUPPORTED, "17 tokens");
  CHECK(vq_gemv_residual(&m, 1, x, 1, y, nullptr, 0, nullptr) == VQ_EWORKSPACE, "no workspace");
  CHECK(vq_gemv_residual_noalloc(&m, 1, x, 2, y, nullptr) == VQ_EUNSUPPORTED, "noalloc B 2");
  CHECK(vq_stream_read(nullptr, nullptr, 1, nullptr, 0, nullptr) == VQ_EINVAL, "read nulls");
  CHECK(strcmp(vq_status_str(VQ_EALIGN), "VQ_EALIGN: pointer misaligned") == 0, "status string");
  CHECK(strcmp(vq_status_str(12345), "unknown") == 0, "unknown status");
  CHECK(vq_wc_device_bytes(8, 16) == ((size_t)1 << 20) && vq_wc_device_bytes(4, 9) == 0, "wc bytes");
}

void check_plain_shapes() {
  const int Ns[] = {1, 15, 16, 17, 333, 768, 4096, 4103, 11008, 131071};
  const int Ks[] = {256, 512, 768, 2048, 4096, 8192, 8448, 11008, 12288, 65536};
  for (int B : {1, 2, 4})
    for (int K : Ks)
      for (int N : Ns) {
        vq_matrix m[2] = {mat(K, N), mat(4096, 700)};
        m[1].wi = P(0x1000000);
        CHECK(gemv(m, 2, B) == VQ_OK, "8-bit K=%d N=%d B=%d", K, N, B);
        CHECK(last.kind == WC8 || last.kind == WC8_UNITS, "kind");
        if (last.kind == WC8) check_wcmats(last.wc, last.grid_x, WC8, last.waves, last.burst, m, 2, B);
      }
  // the 2^31-byte edge of the burst kernel's index buffer: rows of K = 8192
  // (32 chunks of 1 KiB per row group) reach 2^31 bytes at 65536 row groups
  for (int N : {1048560, 1048576, 1048592}) {
    vq_matrix m = mat(8192, N);
    CHECK(gemv(&m, 1, 1) == VQ_OK, "8-bit edge N=%d", N);
    check_wcmats(last.wc, last.grid_x, WC8, last.waves, last.burst, &m, 1, 1);
    const int64_t bytes = (int64_t)((N + 15) / 16) * 1024 * 32;
    if (bytes >= ((int64_t)1 << 31)) CHECK(!last.burst, "burst kernel past 2^31 bytes (N=%d)", N);
    else CHECK(last.burst, "streaming kernel below 2^31 bytes (N=%d)", N);
  }
  CHECK(vqd::wc8_burst_fits(1048560, 2048, 8) && !vqd::wc8_burst_fits(1048576, 2048, 8), "burst edge");
  for (int K : {256, 4096, 11008, 16384, 65536})
    for (int N : {1, 40, 4096, 11008}) {
      if ((K / 4) % 64) continue;
      vq_matrix m = mat(K, N, 4, 12);
      CHECK(gemv(&m, 1, 1) == VQ_OK, "12-bit K=%d N=%d", K, N);
      check_wcmats(last.wc, last.grid_x, WC12, 0, false, &m, 1, 1);
    }
  for (int B : {1, 5, 16})
    for (int K : {256, 5120, 13824, 65536})
      for (int N : {1, 20, 5120, 13824}) {
        vq_matrix m[2] = {mat(K, N, 8, 16), mat(5120, 100, 8, 16)};
        m[1].wi = P(0x1000000);
        const size_t need = vq_workspace_bytes(m, 2, B, 0);
        CHECK(gemv(m, 2, B, P(0x4000000), need) == VQ_OK, "16-bit K=%d N=%d B=%d", K, N, B);
        check_wcmats(last.w16.a, last.grid_x, WC16T, 0, false, m, 2, B);
        // x by dimension in the workspace, one region per matrix, in bounds
        for (int s = 0; s < 2; ++s) {
          const uintptr_t lo = reinterpret_cast<uintptr_t>(last.w16.xt[s]);
          const vqd::WcMat &d = last.w16.a.mat[s];
          const uintptr_t hi = lo + (size_t)d.B * d.J * 8 * 2;
          CHECK(lo >= FAKE + 0x4000000 && hi <= FAKE + 0x4000000 + need, "x planes outside the workspace");
          for (int t = 0; t < s; ++t) {
            const uintptr_t lo2 = reinterpret_cast<uintptr_t>(last.w16.xt[t]);
            const vqd::WcMat &e = last.w16.a.mat[t];
            CHECK(hi <= lo2 || lo2 + (size_t)e.B * e.J * 16 <= lo, "x planes overlap");
          }
        }
      }
  // rows past 16 blocks per wave, or past 2^31 bytes of indices, are refused
  vq_matrix big = mat(65792, 16, 8, 16);
  CHECK(gemv(&big, 1, 1, P(0x4000000), 1 << 30) == VQ_EUNSUPPORTED, "16-bit K=65792");
  // 32 blocks of 1 KiB per row group of K = 8192: 2^31 bytes at 65536 row groups
  CHECK(!vqd::wc16t_fits(1048576, 1024, vqd::wc16t_jsplit(1024)), "16-bit 2^31 edge");
  CHECK(vqd::wc16t_fits(1048560, 1024, vqd::wc16t_jsplit(1024)), "16-bit below the edge");
}

void check_tokens() {
  for (int B : {1, 3, 8, 13, 16})
    for (int K : {256, 4096, 11008, 65536})
      for (int N : {1, 17, 4096, 4103}) {
        if ((K / 4) % 64) continue;
        vq_matrix m = mat(K, N);
        const uint16_t *x[1] = {static_cast<const uint16_t *>(P(0x400000))};
        float *y[1] = {static_cast<float *>(P(0x800000))};
        CHECK(vq_gemv_tokens(&m, 1, x, B, y, nullptr) == VQ_OK, "tokens K=%d N=%d B=%d", K, N, B);
        CHECK(last.kind == WC8T, "kind");
        const vqd::WcMat &d = last.wc.mat[0];
        const int R = vqd::wc8t_rows_per_wg(d.jsplit, last.rw);
        CHECK((int64_t)d.nwg * R >= N && (int64_t)(d.nwg - 1) * R < N, "token rows %d: %d x %d", N, d.nwg, R);
        CHECK(pow2(d.jsplit) && d.jsplit <= vqd::TK_W, "token split");
        CHECK(last.rw >= 1 && last.rw <= vqd::wc8t_max_rw(B), "rows per wave");
        CHECK((int64_t)(N + 15) / 16 * 16 * (K / 4) < ((int64_t)1 << 31), "token buffer");
      }
  vq_matrix edge = mat(65536, 131072);
  const uint16_t *x[1] = {static_cast<const uint16_t *>(P())};
  float *y[1] = {static_cast<float *>(P())};
  CHECK(vq_gemv_tokens(&edge, 1, x, 4, y, nullptr) == VQ_EUNSUPPORTED, "token 2^31 edge");
}

// The residual plan's regions, in the caller's workspace or the scratch.
void check_residual_regions(uintptr_t ws, size_t bytes, size_t zero_limit, const vq_matrix *m, int count) {
  struct R { uintptr_t lo, hi; bool zero; };
  std::vector<R> rs;
  const vqd::Lut8Args &a = last.res;
  CHECK(a.count == count, "residual count");
  int64_t maxwg = 0;
  for (int i = 0; i < a.count; ++i) {
    const vqd::Lut8Mat &d = a.mat[i];
    CHECK(d.rows_pad >= d.N && d.rows_pad % 32 == 0, "rows_pad");
    CHECK((int64_t)d.nrb * d.rpw * 32 >= d.N, "row blocks cover the rows");
    CHECK(d.nwg == d.nsplit * d.nrb, "workgroups");
    CHECK((int64_t)d.nsplit * 64 >= d.J, "splits cover the subvectors");
    maxwg = std::max<int64_t>(maxwg, d.nwg);
    rs.push_back({reinterpret_cast<uintptr_t>(d.counter), reinterpret_cast<uintptr_t>(d.counter) + (size_t)d.nrb * 4, true});
    if (d.nsplit > 1) {
      rs.push_back({reinterpret_cast<uintptr_t>(d.acc), reinterpret_cast<uintptr_t>(d.acc) + (size_t)d.rows_pad * 8, true});
      rs.push_back({reinterpret_cast<uintptr_t>(d.partial),
                    reinterpret_cast<uintptr_t>(d.partial) + (size_t)d.nsplit * d.rows_pad * 4, false});
    }
    if (!d.fused)
      rs.push_back({reinterpret_cast<uintptr_t>(d.xr), reinterpret_cast<uintptr_t>(d.xr) + (size_t)m[i].K * 4, false});
  }
  CHECK(last.grid_x == maxwg, "residual grid");
  for (size_t i = 0; i < rs.size(); ++i) {
    CHECK(rs[i].lo >= ws && rs[i].hi <= ws + bytes, "region %zu outside [%#lx, +%zu)", i, (unsigned long)ws, bytes);
    if (rs[i].zero) CHECK(rs[i].hi <= ws + zero_limit, "counter region %zu past the zero region", i);
    else CHECK(rs[i].lo >= ws + (zero_limit == bytes ? 0 : zero_limit), "scratch region %zu in the zero region", i);
    for (size_t j = 0; j < i; ++j) CHECK(rs[i].hi <= rs[j].lo || rs[j].hi <= rs[i].lo, "regions %zu and %zu overlap", i, j);
  }
}

void check_residual() {
  struct G { std::vector<int> K, N, h; };
  const G groups[] = {{{3584, 14336}, {14336, 3584}, {512, 2048}},
                      {{1024}, {300}, {1024}},
                      {{256, 8192, 33024}, {40, 100, 64}, {256, 8192, 256}},
                      {{4096}, {9000}, {4096}},
                      {{20480}, {6144}, {4096}}};
  for (const G &g : groups) {
    const int n = (int)g.K.size();
    std::vector<vq_matrix> m;
    for (int i = 0; i < n; ++i) {
      vq_matrix q = mat(g.K[i], g.N[i]);
      q.rht_sign = static_cast<const int8_t *>(P(0x500000));
      q.had_block = g.h[i];
      q.wi = P(0x1000000 * (i + 1));
      m.push_back(q);
    }
    std::vector<const uint16_t *> x(n, static_cast<const uint16_t *>(P(0x400000)));
    std::vector<float *> y(n, static_cast<float *>(P(0x800000)));
    const size_t need = vq_workspace_bytes(m.data(), n, 1, 1);
    const uintptr_t ws = FAKE + 0x40000000;
    CHECK(vq_gemv_residual(m.data(), n, x.data(), 1, y.data(), reinterpret_cast<void *>(ws), need, nullptr) == VQ_OK,
          "residual group K0=%d", g.K[0]);
    CHECK(last.kind == RESIDUAL, "residual kind");
    check_residual_regions(ws, need, need, m.data(), n);
    CHECK(vq_gemv_residual(m.data(), n, x.data(), 1, y.data(), reinterpret_cast<void *>(ws), need - 1, nullptr) ==
              VQ_EWORKSPACE, "short workspace");
    const int st = vq_gemv_residual_noalloc(m.data(), n, x.data(), 1, y.data(), nullptr);
    if (st == VQ_OK) {
      CHECK(last.kind == RESIDUAL, "noalloc kind");
      check_residual_regions(g_scratch, VQ_NOALLOC_SCRATCH_BYTES, VQ_NOALLOC_COUNTER_BYTES, m.data(), n);
    } else {
      CHECK(st == VQ_EWORKSPACE, "noalloc status %d", st);
    }
  }
}

// The output-codebook form of the plain call: the residual kernel with no
// rotation, signs or scales, on the residual call's workspace plan.
void check_oc() {
  const std::vector<std::vector<int>> groups[] = {{{4096, 4096, 4096, 4096}, {4096, 4096, 4096, 4096}},
                                                  {{256, 11008, 33024}, {17, 4096, 40}},
                                                  {{512}, {512}}};
  for (const auto &g : groups) {
    const int n = (int)g[0].size();
    std::vector<vq_matrix> m;
    for (int i = 0; i < n; ++i) {
      vq_matrix q = mat(g[0][i], g[1][i]);
      q.signs = nullptr; q.alpha = nullptr;         // not read by this call
      q.wi = P(0x1000000 * (i + 1));
      m.push_back(q);
    }
    std::vector<const uint16_t *> x(n, static_cast<const uint16_t *>(P(0x400000)));
    std::vector<float *> y(n, static_cast<float *>(P(0x800000)));
    const size_t need = vq_workspace_bytes(m.data(), n, 1, 1);
    CHECK(need > 0, "oc workspace");
    const uintptr_t ws = FAKE + 0x40000000;
    CHECK(vq_gemv_oc(m.data(), n, x.data(), 1, y.data(), reinterpret_cast<void *>(ws), need, nullptr) == VQ_OK,
          "oc group K0=%d", g[0][0]);
    CHECK(last.kind == OCTILE, "oc kind");
    for (int i = 0; i < n; ++i) {
      const vqd::Lut8Mat &d = last.res.mat[i];
      CHECK(!d.signs && !d.alpha && !d.alpha_hdr && !d.rs, "oc matrix %d reads residual inputs", i);
      CHECK(d.had == 1 && d.fused == 1, "oc matrix %d rotates", i);
    }
    check_residual_regions(ws, need, need, m.data(), n);
    CHECK(vq_gemv_oc(m.data(), n, x.data(), 1, y.data(), reinterpret_cast<void *>(ws), need - 1, nullptr) ==
              VQ_EWORKSPACE, "short oc workspace");
    CHECK(vq_gemv_oc(m.data(), n, x.data(), 2, y.data(), reinterpret_cast<void *>(ws), need, nullptr) ==
              VQ_EUNSUPPORTED, "oc with two tokens");
  }
  vq_matrix q = mat(4096, 4096, 4, 12);
  const uint16_t *x1[] = {static_cast<const uint16_t *>(P(0x400000))};
  float *y1[] = {static_cast<float *>(P(0x800000))};
  CHECK(vq_gemv_oc(&q, 1, x1, 1, y1, reinterpret_cast<void *>(FAKE + 0x40000000), (size_t)1 << 30, nullptr) ==
            VQ_EUNSUPPORTED, "oc with 12-bit indices");
  q = mat(4096, 2097152);                         // 2^31 bytes of device indices
  CHECK(vq_gemv_oc(&q, 1, x1, 1, y1, reinterpret_cast<void *>(FAKE + 0x40000000), (size_t)1 << 30, nullptr) ==
            VQ_EUNSUPPORTED, "oc past 2^31 index bytes");
  q = mat(4096, 2097120);                         // the largest row count below it
  CHECK(vq_gemv_oc(&q, 1, x1, 1, y1, reinterpret_cast<void *>(FAKE + 0x40000000), (size_t)1 << 30, nullptr) ==
            VQ_OK, "oc just below 2^31 index bytes");
}

// The fused gate/up call: every output row covered by a workgroup's slot
// pairs, and the split and wave count its kernel is built for (16 waves for
// a split of 8, else 8).
void check_swiglu() {
  for (int B : {1, 2})
    for (int K : {256, 2048, 4096, 8192, 14336, 32768})
      for (int N : {1, 17, 700, 11008, 14336}) {
        vq_matrix g[2] = {mat(K, N), mat(K, N)};
        vq_matrix u[2] = {mat(K, N), mat(K, N)};
        g[1].wi = P(0x1000000); u[0].wi = P(0x2000000); u[1].wi = P(0x3000000);
        const uint16_t *x[2] = {static_cast<const uint16_t *>(P(0x400000)), static_cast<const uint16_t *>(P(0x410000))};
        float *y[2] = {static_cast<float *>(P(0x800000)), static_cast<float *>(P(0x810000))};
        for (int cnt : {1, 2}) {
          const int st = vq_gemv_swiglu(g, u, cnt, x, B, y, nullptr, 0, nullptr);
          if (st == VQ_EUNSUPPORTED) continue;                 // rows past the burst kernel
          CHECK(st == VQ_OK, "swiglu K=%d N=%d B=%d: %d", K, N, B, st);
          CHECK(last.kind == SWIGLU, "swiglu kind");
          CHECK(last.waves == 8 || last.waves == 16, "swiglu waves %d", last.waves);
          int64_t maxwg = 0;
          for (int s = 0; s < cnt; ++s) {
            const vqd::WcMat &d = last.pair.a.mat[s];
            CHECK(pow2(d.jsplit) && 2 * d.jsplit <= last.waves, "swiglu split %d waves %d", d.jsplit, last.waves);
            const int R = last.waves / d.jsplit / 2 * 16;
            CHECK((int64_t)d.nwg * R >= d.N && (int64_t)(d.nwg - 1) * R < d.N, "swiglu rows N=%d", d.N);
            maxwg = std::max<int64_t>(maxwg, d.nwg);
          }
          CHECK(last.grid_x == maxwg, "swiglu grid");
          int maxs = 1;
          for (int s = 0; s < cnt; ++s) maxs = std::max(maxs, last.pair.a.mat[s].jsplit);
          CHECK(last.waves == (maxs > 4 ? 16 : 8), "swiglu waves %d for split %d", last.waves, maxs);
        }
      }
}

void check_stream_read() {
  const size_t sizes[] = {16, 1 << 20, 4194304, 12845056, ((size_t)1 << 31) - 16};
  std::vector<const void *> b(5, P());
  const size_t words = vq_stream_read_sink_words(sizes, 5);
  CHECK(words > 0, "sink words");
  CHECK(vq_stream_read(b.data(), sizes, 5, static_cast<uint32_t *>(P()), words, nullptr) == VQ_OK, "read");
  CHECK((size_t)last.grid_x * 5 * vqd::RD_W <= words, "sink too small for the grid");
  CHECK((int64_t)last.grid_x * vqd::RD_W * vqd::RD_NCH * 1024 >= (int64_t)sizes[4], "grid covers the bytes");
  CHECK(vq_stream_read(b.data(), sizes, 5, static_cast<uint32_t *>(P()), words - 1, nullptr) == VQ_EWORKSPACE,
        "short sink");
  const size_t huge[] = {(size_t)1 << 31};
  CHECK(vq_stream_read_sink_words(huge, 1) == 0, "2^31-byte buffer");
}
}  // namespace

int main() {
  check_validation();
  check_plain_shapes();
  check_tokens();
  check_residual();
  check_oc();
  check_swiglu();
  check_stream_read();
  if (failures) {
    fprintf(stderr, "%d host check(s) failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
