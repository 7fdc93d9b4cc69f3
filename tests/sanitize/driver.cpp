// Test infrastructure: drives every host-side call of the C ABI over a sweep
// of shapes, flags and mask variants, with every caller buffer allocated at
// exactly the size the header documents, inside an AddressSanitizer /
// UndefinedBehaviorSanitizer build (see fake_device.cpp).  Exit status 0
// means every call returned what the header promises and no sanitizer fired.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "radial.h"

extern "C" int fake_device_failures();

namespace {

int g_bad = 0;

#define EXPECT(cond)                                                         \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "driver: %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      g_bad = 1;                                                             \
    }                                                                        \
  } while (0)

// a 16-byte aligned heap block of exactly `bytes` bytes
void *block(size_t bytes) {
  void *p = nullptr;
  if (posix_memalign(&p, 16, bytes ? bytes : 1) != 0) std::abort();
  std::memset(p, 0, bytes);
  return p;
}

struct Shape {
  int64_t f, s;
  int32_t T;
  uint32_t flags;
  radial_mask_params prm;
};

void exercise(const Shape &sh) {
  radial_layout *L = nullptr;
  EXPECT(radial_mask_build_ex(sh.f, sh.s, sh.T, sh.flags, &sh.prm, &L) == RADIAL_OK);
  if (!L) return;
  int64_t n = 0, nz = 0, pairs = 0;
  int32_t nb = 0;
  EXPECT(radial_layout_info(L, &n, &nb, &nz, &pairs) == RADIAL_OK);
  EXPECT(n == sh.f * sh.s && nb == (n + sh.T - 1) / sh.T && nz >= 1 && pairs >= 1);
  EXPECT(radial_layout_info(L, nullptr, nullptr, nullptr, nullptr) == RADIAL_OK);

  std::vector<int32_t> rp(nb + 1), ci(nz), cp(nb + 1), ri(nz);
  EXPECT(radial_layout_export(L, rp.data(), ci.data(), cp.data(), ri.data()) == RADIAL_OK);
  EXPECT(rp[nb] == nz && cp[nb] == nz);
  std::vector<uint8_t> fa(nz), fb(nz);
  EXPECT(radial_layout_tile_flags(L, fa.data(), fb.data()) == RADIAL_OK);
  std::vector<int32_t> band(sh.f);
  std::vector<int64_t> width(sh.f), period(sh.f);
  EXPECT(radial_layout_band_table(L, band.data(), width.data(), period.data()) == RADIAL_OK);
  if (n <= 700) {
    std::vector<uint8_t> m(n * n);
    EXPECT(radial_layout_token_mask(L, m.data(), n * n) == RADIAL_OK);
    EXPECT(radial_layout_token_mask(L, m.data(), n * n - 1) == RADIAL_E_INVALID);
  }

  // compute calls before the upload: state error, nothing touched
  const int32_t D = sh.T, B = 1, H = 2;
  const bool supported = (D == 64 || D == 128);
  const size_t x = size_t(B) * H * n * D * 2, r = size_t(B) * H * n * 4;
  void *q = block(x), *k = block(x), *v = block(x), *o = block(x), *dout = block(x);
  void *dq = block(x), *dk = block(x), *dv = block(x);
  float *lse = static_cast<float *>(block(r));
  const float sc = 0.125f;
  EXPECT(radial_attn_fwd(L, B, H, n, D, sc, q, k, v, o, lse, nullptr) ==
         (supported ? RADIAL_E_STATE : RADIAL_E_UNSUPPORTED));
  EXPECT(radial_attn_bwd_noalloc(L, B, H, n, D, sc, q, k, v, o, lse, dout, dq, dk, dv, nullptr) ==
         (supported ? RADIAL_E_STATE : RADIAL_E_UNSUPPORTED));

  EXPECT(radial_layout_upload(L) == RADIAL_OK);
  EXPECT(radial_layout_upload(L) == RADIAL_OK);  // second upload: no-op
  if (supported) {
    EXPECT(radial_attn_fwd(L, B, H, n, D, sc, q, k, v, o, lse, nullptr) == RADIAL_OK);
    const size_t ws_bytes = radial_attn_bwd_workspace_bytes(L, B, H, n, D);
    EXPECT(ws_bytes >= 2 * r);
    void *ws = block(ws_bytes);
    EXPECT(radial_attn_bwd(L, B, H, n, D, sc, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes,
                           nullptr) == RADIAL_OK);
    EXPECT(radial_attn_bwd(L, B, H, n, D, sc, q, k, v, o, lse, dout, dq, dk, dv, ws,
                           ws_bytes - 1, nullptr) == RADIAL_E_INVALID);
    // the allocation-free variant: the same launches on the static scratch
    EXPECT(radial_attn_bwd_noalloc(L, B, H, n, D, sc, q, k, v, o, lse, dout, dq, dk, dv,
                                   nullptr) == RADIAL_OK);
    EXPECT(radial_attn_bwd_noalloc(L, B, H, n, D, sc, q, k, v, o, lse, dout, dq, dk, nullptr,
                                   nullptr) == RADIAL_E_INVALID);
    // misaligned and missing pointers, wrong sizes
    EXPECT(radial_attn_fwd(L, B, H, n, D, sc, static_cast<char *>(q) + 2, k, v, o, lse,
                           nullptr) == RADIAL_E_INVALID);
    EXPECT(radial_attn_fwd(L, B, H, n, D, sc, q, k, v, nullptr, lse, nullptr) ==
           RADIAL_E_INVALID);
    EXPECT(radial_attn_fwd(L, B, H, n + 1, D, sc, q, k, v, o, lse, nullptr) == RADIAL_E_SHAPE);
    EXPECT(radial_attn_fwd(L, 0, H, n, D, sc, q, k, v, o, lse, nullptr) == RADIAL_E_INVALID);
    std::free(ws);
  }
  for (void *p : {q, k, v, o, dout, dq, dk, dv, static_cast<void *>(lse)}) std::free(p);
  if (sh.T == 128) {  // head dim 64 on 128-wide tiles
    const size_t x64 = size_t(B) * H * n * 64 * 2;
    void *a = block(x64), *b = block(x64), *c = block(x64), *d = block(x64), *e = block(x64);
    void *f = block(x64), *g2 = block(x64), *h = block(x64);
    float *l64 = static_cast<float *>(block(r));
    EXPECT(radial_attn_fwd(L, B, H, n, 64, sc, a, b, c, d, l64, nullptr) == RADIAL_OK);
    const size_t ws_bytes = radial_attn_bwd_workspace_bytes(L, B, H, n, 64);
    void *ws = block(ws_bytes);
    EXPECT(radial_attn_bwd(L, B, H, n, 64, sc, a, b, c, d, l64, e, f, g2, h, ws, ws_bytes,
                           nullptr) == RADIAL_OK);
    for (void *p : {a, b, c, d, e, f, g2, h, ws, static_cast<void *>(l64)}) std::free(p);
  }
  radial_layout_destroy(L);
}

}  // namespace

int main() {
  const radial_mask_params def = {RADIAL_DECAY_RADIAL, 1, 2, 1};
  std::vector<radial_mask_params> variants = {
      def,
      {RADIAL_DECAY_RADIAL, 0, 2, 1},
      {RADIAL_DECAY_RADIAL, 2, 2, 1},
      {RADIAL_DECAY_RADIAL, 1, 3, 2},
      {RADIAL_DECAY_RADIAL, 1, 4, 1},
      {RADIAL_DECAY_RADIAL, 3, 16, 4},
      {RADIAL_DECAY_HARMONIC, 1, 0, 0},
      {RADIAL_DECAY_HARMONIC, 5, 2, 1},
  };
  const int64_t shapes[][3] = {{1, 1, 64},   {1, 5, 2},   {4, 9, 4},    {8, 256, 64},
                               {5, 300, 128}, {7, 100, 64}, {3, 40, 128}, {40, 20, 64},
                               {300, 2, 64},  {600, 3, 16}, {33, 36, 128}, {129, 20, 128},
                               {33, 3600, 128}};
  const uint32_t flag_sets[] = {RADIAL_SINK, 0, RADIAL_SINK | RADIAL_TOKEN_EXACT,
                                RADIAL_TOKEN_EXACT, RADIAL_SINK | RADIAL_DENSE,
                                RADIAL_DENSE | RADIAL_TOKEN_EXACT};
  for (const auto &s : shapes)
    for (uint32_t fl : flag_sets)
      for (const auto &p : variants) {
        // the largest shape with the default mask and two flag sets only
        if (s[0] * s[1] > 100000 && (p.decay != def.decay || p.central_band != def.central_band ||
                                     p.scale_num != def.scale_num || fl > RADIAL_SINK))
          continue;
        exercise({s[0], s[1], static_cast<int32_t>(s[2]), fl, p});
      }

  // argument validation of the builders
  radial_layout *L = reinterpret_cast<radial_layout *>(0x1);
  EXPECT(radial_mask_build(0, 10, 8, RADIAL_SINK, &L) == RADIAL_E_INVALID && L == nullptr);
  EXPECT(radial_mask_build(4, 10, 8, 8u, &L) == RADIAL_E_INVALID);
  EXPECT(radial_mask_build(int64_t(1) << 20, int64_t(1) << 12, 128, 1, &L) == RADIAL_E_INVALID);
  EXPECT(radial_mask_build(4, 10, 8, RADIAL_SINK, nullptr) == RADIAL_E_INVALID);
  const radial_mask_params bad[] = {{2, 1, 2, 1}, {0, -1, 2, 1}, {0, 1, 2, 2}, {0, 1, 17, 1},
                                    {0, 1, 9, 5}};
  for (const auto &p : bad) EXPECT(radial_mask_build_ex(8, 64, 16, 1, &p, &L) == RADIAL_E_INVALID);
  radial_mask_params d = {9, 9, 9, 9};
  radial_mask_params_default(&d);
  EXPECT(d.decay == 0 && d.central_band == 1 && d.scale_num == 2 && d.scale_den == 1);
  radial_mask_params_default(nullptr);

  // null layouts, failing device, failing allocation
  EXPECT(radial_layout_info(nullptr, nullptr, nullptr, nullptr, nullptr) == RADIAL_E_INVALID);
  EXPECT(radial_layout_upload(nullptr) == RADIAL_E_INVALID);
  radial_layout_destroy(nullptr);
  EXPECT(radial_mask_build(8, 256, 64, RADIAL_SINK, &L) == RADIAL_OK);
  setenv("FAKE_DEVICE_NONE", "1", 1);
  EXPECT(radial_layout_upload(L) == RADIAL_E_HIP);
  unsetenv("FAKE_DEVICE_NONE");
  EXPECT(radial_test_set_fail_alloc(1) == 0);
  EXPECT(radial_layout_upload(L) == RADIAL_E_NOMEM);
  radial_layout *L2 = nullptr;
  EXPECT(radial_mask_build(8, 256, 64, RADIAL_SINK, &L2) == RADIAL_E_NOMEM && L2 == nullptr);
  EXPECT(radial_test_set_fail_alloc(0) == 1);
  EXPECT(radial_test_set_fail_alloc(5) == RADIAL_E_INVALID);
  EXPECT(radial_layout_upload(L) == RADIAL_OK);
  // slices of 2^31 bytes or more are refused before any launch (no buffer
  // of that size exists here: a launch would touch the small blocks below
  // far out of range)
  {
    const size_t x = 2048 * 128 * 2;
    void *q = block(x), *k = block(x), *v = block(x), *o = block(x), *dout = block(x);
    void *dq = block(x), *dk = block(x), *dv = block(x), *ws = block(1 << 16);
    float *lse = static_cast<float *>(block(2048 * 4));
    for (int64_t N : {int64_t(1) << 23, int64_t(1) << 30, int64_t(1) << 40}) {
      EXPECT(radial_attn_fwd(L, 1, 1, N, 128, 0.1f, q, k, v, o, lse, nullptr) ==
             RADIAL_E_UNSUPPORTED);
      EXPECT(radial_attn_bwd(L, 1, 1, N, 128, 0.1f, q, k, v, o, lse, dout, dq, dk, dv, ws,
                             1 << 16, nullptr) == RADIAL_E_UNSUPPORTED);
    }
    for (void *p : {q, k, v, o, dout, dq, dk, dv, ws, static_cast<void *>(lse)}) std::free(p);
  }
  {
    // the allocation-free backward refuses row arrays beyond its scratch
    // (B * H * n = 4100 * 2048 rows: 67.2 MB) before touching any pointer
    const size_t x = 64;
    void *p = block(x);
    const float *lp = static_cast<const float *>(p);
    EXPECT(radial_attn_bwd_workspace_bytes(L, 1, 4100, 2048, 64) > RADIAL_BWD_SCRATCH_BYTES);
    EXPECT(radial_attn_bwd_noalloc(L, 1, 4100, 2048, 64, 0.1f, p, p, p, p, lp, p, p, p, p,
                                   nullptr) == RADIAL_E_UNSUPPORTED);
    std::free(p);
  }
  radial_layout_destroy(L);
  // the forward's group cap
  EXPECT(radial_test_set_fwd_group(0) == RADIAL_E_INVALID);
  EXPECT(radial_test_set_fwd_group(2) == 3);
  EXPECT(radial_test_set_fwd_group(3) == 2);

  // schedule decisions, status strings
  for (int l = 0; l < 4; ++l)
    for (int t = 0; t < 14; ++t)
      EXPECT(radial_schedule_dense(l, t, 2, 12) == ((l < 2 || t < 12) ? 1 : 0));
  EXPECT(radial_schedule_dense(-1, 0, 2, 12) == RADIAL_E_INVALID);
  for (int st = 1; st >= -7; --st) EXPECT(radial_status_string(st) != nullptr);
  EXPECT(radial_last_error() != nullptr);

  if (fake_device_failures()) g_bad = 1;
  std::printf("%s\n", g_bad ? "FAILED" : "ok");
  return g_bad;
}
