// C ABI of libradial.so: argument validation, layout lifetime and upload,
// kernel dispatch.  Never throws or aborts across the boundary.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "kernels.h"
#include "layout.h"
#include "radial.h"

static_assert(radial::kBwdScratchBytes == RADIAL_BWD_SCRATCH_BYTES, "scratch size");

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string &msg) {
  g_last_error = msg;
  return status;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Allocation-failure flag for tests (radial_test_set_fail_alloc): while set,
// the layout build and upload report RADIAL_E_NOMEM instead of allocating.
std::atomic<int32_t> g_fail_alloc{0};
bool forced_alloc_failure() { return g_fail_alloc.load(std::memory_order_relaxed) != 0; }

// Largest query-tile group the forward uses (3: triples); lowered only by
// radial_test_set_fwd_group, so tests can compare the three forms.
std::atomic<int32_t> g_fwd_max_group{3};

void free_device(radial_layout *L) {
  if (L->d_base) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != L->device) (void)hipSetDevice(L->device);
    (void)hipFree(L->d_base);
    if (cur != L->device && cur >= 0) (void)hipSetDevice(cur);
  }
  L->d_base = nullptr;
  L->d_row_ptr = L->d_col_idx = L->d_col_ptr = L->d_row_idx = L->d_col_order = nullptr;
  L->d_band_rtab = L->d_pair_ptr = L->d_pair_idx = L->d_tri_ptr = L->d_tri_idx = nullptr;
  L->d_tri_tiles = nullptr;
  L->device = -1;
}

// Common checks of the compute calls; fills `stream`.
int check_common(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D,
                 float scale) {
  if (!L) return fail(RADIAL_E_INVALID, "layout is NULL");
  if (B < 1 || H < 1) return fail(RADIAL_E_INVALID, "B and H must be >= 1");
  // one (batch, head) slice must stay below 2^31 bytes: the kernels address
  // rows within a slice with 32-bit offsets
  if (N < 1) return fail(RADIAL_E_INVALID, "N must be >= 1");
  if (D > 0 && N > ((int64_t(1) << 31) - 1) / (2 * (int64_t)D))
    return fail(RADIAL_E_UNSUPPORTED, "N = " + std::to_string(N) + " at D = " + std::to_string(D) +
                                          ": one (batch, head) slice of N * D bf16 values must "
                                          "hold fewer than 2^31 bytes");
  if (N != L->n)
    return fail(RADIAL_E_SHAPE, "N = " + std::to_string(N) + " but the layout has n = " +
                                    std::to_string(L->n) + " (frames * tokens_per_frame)");
  if (!((D == 64 && L->block == 64) || (D == 64 && L->block == 128) ||
        (D == 128 && L->block == 128)))
    return fail(RADIAL_E_UNSUPPORTED, "(D, block_size) = (" + std::to_string(D) + ", " +
                                          std::to_string(L->block) +
                                          ") not supported; use (64, 64), (64, 128) or (128, 128)");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(RADIAL_E_INVALID, "scale must be finite and > 0");
  if ((int64_t)B * H > (int64_t(1) << 31) / (L->nb > 0 ? L->nb : 1))
    return fail(RADIAL_E_INVALID, "B * H * n_blocks must be < 2^31");
  if (!L->d_base) return fail(RADIAL_E_STATE, "layout not uploaded: call radial_layout_upload");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RADIAL_E_HIP, "hipGetDevice failed");
  if (dev != L->device)
    return fail(RADIAL_E_STATE, "layout uploaded to device " + std::to_string(L->device) +
                                    " but the current device is " + std::to_string(dev));
  return RADIAL_OK;
}

int check_ptrs(std::initializer_list<std::pair<const void *, const char *>> ptrs) {
  for (const auto &p : ptrs) {
    if (!p.first) return fail(RADIAL_E_INVALID, std::string(p.second) + " is NULL");
    if (!aligned16(p.first))
      return fail(RADIAL_E_INVALID, std::string(p.second) + " is not 16-byte aligned");
  }
  return RADIAL_OK;
}

}  // namespace

extern "C" {

void radial_mask_params_default(radial_mask_params *p) {
  if (p) *p = radial_mask_params{RADIAL_DECAY_RADIAL, 1, 2, 1};
}

int radial_mask_build(int64_t frames, int64_t tokens_per_frame, int32_t block_size,
                      uint32_t flags, radial_layout **out) {
  return radial_mask_build_ex(frames, tokens_per_frame, block_size, flags, nullptr, out);
}

int radial_mask_build_ex(int64_t frames, int64_t tokens_per_frame, int32_t block_size,
                         uint32_t flags, const radial_mask_params *params,
                         radial_layout **out) {
  if (!out) return fail(RADIAL_E_INVALID, "out is NULL");
  radial_mask_params prm;
  radial_mask_params_default(&prm);
  if (params) prm = *params;
  *out = nullptr;
  if (forced_alloc_failure()) return fail(RADIAL_E_NOMEM, "allocation failure (forced by test hook)");
  radial_layout *L = new (std::nothrow) radial_layout();
  if (!L) return fail(RADIAL_E_NOMEM, "out of host memory");
  try {
    const std::string err =
        radial::build_layout(frames, tokens_per_frame, block_size, flags, prm, *L);
    if (!err.empty()) {
      delete L;
      return fail(RADIAL_E_INVALID, err);
    }
  } catch (const std::bad_alloc &) {
    delete L;
    return fail(RADIAL_E_NOMEM, "out of host memory while building the layout");
  } catch (...) {
    delete L;
    return fail(RADIAL_E_INVALID, "unexpected error while building the layout");
  }
  *out = L;
  return RADIAL_OK;
}

int radial_layout_info(const radial_layout *L, int64_t *n_tokens, int32_t *n_blocks,
                       int64_t *nnz_tiles, int64_t *nnz_pairs) {
  if (!L) return fail(RADIAL_E_INVALID, "layout is NULL");
  if (n_tokens) *n_tokens = L->n;
  if (n_blocks) *n_blocks = L->nb;
  if (nnz_tiles) *nnz_tiles = L->nnz_tiles;
  if (nnz_pairs) *nnz_pairs = L->nnz_pairs;
  return RADIAL_OK;
}

int radial_layout_export(const radial_layout *L, int32_t *row_ptr, int32_t *col_idx,
                         int32_t *col_ptr, int32_t *row_idx) {
  if (!L) return fail(RADIAL_E_INVALID, "layout is NULL");
  const size_t nb1 = (size_t)L->nb + 1, nz = (size_t)L->nnz_tiles;
  if (row_ptr) std::memcpy(row_ptr, L->row_ptr.data(), nb1 * sizeof(int32_t));
  if (col_idx) std::memcpy(col_idx, L->col_idx.data(), nz * sizeof(int32_t));
  if (col_ptr) std::memcpy(col_ptr, L->col_ptr.data(), nb1 * sizeof(int32_t));
  if (row_idx) std::memcpy(row_idx, L->row_idx.data(), nz * sizeof(int32_t));
  return RADIAL_OK;
}

int radial_layout_tile_flags(const radial_layout *L, uint8_t *csr_full, uint8_t *csc_full) {
  if (!L) return fail(RADIAL_E_INVALID, "layout is NULL");
  if (csr_full && L->nnz_tiles) std::copy(L->full.begin(), L->full.end(), csr_full);
  if (csc_full && L->nnz_tiles) std::copy(L->full_csc.begin(), L->full_csc.end(), csc_full);
  return RADIAL_OK;
}

int radial_schedule_dense(int32_t layer, int32_t step, int32_t dense_layers,
                          int32_t warmup_steps) {
  if (layer < 0 || step < 0 || dense_layers < 0 || warmup_steps < 0)
    return fail(RADIAL_E_INVALID, "schedule arguments must be >= 0");
  return (layer < dense_layers || step < warmup_steps) ? 1 : 0;
}

int radial_layout_band_table(const radial_layout *L, int32_t *band, int64_t *width,
                             int64_t *period) {
  if (!L) return fail(RADIAL_E_INVALID, "layout is NULL");
  const size_t f = (size_t)L->frames;
  if (band) std::memcpy(band, L->band_r.data(), f * sizeof(int32_t));
  if (width) std::memcpy(width, L->band_w.data(), f * sizeof(int64_t));
  if (period) std::memcpy(period, L->band_period.data(), f * sizeof(int64_t));
  return RADIAL_OK;
}

int radial_layout_token_mask(const radial_layout *L, uint8_t *out, int64_t cap) {
  if (!L) return fail(RADIAL_E_INVALID, "layout is NULL");
  if (!out) return fail(RADIAL_E_INVALID, "out is NULL");
  const int64_t n = L->n;
  if (n > 3037000499LL || n * n > cap)
    return fail(RADIAL_E_INVALID, "token mask needs n * n bytes");
  for (int64_t q = 0; q < n; ++q)
    for (int64_t k = 0; k < n; ++k) out[q * n + k] = radial::token_allowed(*L, q, k) ? 1 : 0;
  return RADIAL_OK;
}

int radial_layout_upload(radial_layout *L) {
  if (!L) return fail(RADIAL_E_INVALID, "layout is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RADIAL_E_HIP, "no HIP device available");
  if (L->d_base && L->device == dev) return RADIAL_OK;
  if (L->d_base) free_device(L);
  if (forced_alloc_failure()) return fail(RADIAL_E_NOMEM, "allocation failure (forced by test hook)");
  const size_t nb1 = (size_t)L->nb + 1, nz = (size_t)L->nnz_tiles, nb = (size_t)L->nb;
  const size_t words =
      2 * nb1 + 2 * nz + nb + L->band_rtab.size() + L->pair_ptr.size() + L->pair_idx.size() +
      L->tri_ptr.size() + L->tri_idx.size() + L->tri_tiles.size();
  void *p = nullptr;
  if (hipMalloc(&p, words * sizeof(int32_t)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return fail(RADIAL_E_NOMEM, "hipMalloc of the layout failed");
  }
  int32_t *b = static_cast<int32_t *>(p);
  size_t off = 0;
  // Token-exact layouts mark partial tiles in bit 31 of the device tile
  // indices (the kernels mask the token predicate inside those tiles only).
  std::vector<int32_t> col_dev, row_dev;
  const std::vector<int32_t> *col_src = &L->col_idx, *row_src = &L->row_idx;
  if ((L->flags & RADIAL_TOKEN_EXACT) && !(L->flags & RADIAL_DENSE)) {
    col_dev = L->col_idx;
    row_dev = L->row_idx;
    for (size_t t = 0; t < nz; ++t) {
      if (!L->full[t]) col_dev[t] = int32_t(uint32_t(col_dev[t]) | 0x80000000u);
      if (!L->full_csc[t]) row_dev[t] = int32_t(uint32_t(row_dev[t]) | 0x80000000u);
    }
    col_src = &col_dev;
    row_src = &row_dev;
  }
  struct Part {
    const std::vector<int32_t> *src;
    const int32_t **dst;
  } parts[] = {{&L->row_ptr, &L->d_row_ptr},
               {col_src, &L->d_col_idx},
               {&L->col_ptr, &L->d_col_ptr},
               {row_src, &L->d_row_idx},
               {&L->col_order, &L->d_col_order},
               {&L->band_rtab, &L->d_band_rtab},
               {&L->pair_ptr, &L->d_pair_ptr},
               {&L->pair_idx, &L->d_pair_idx},
               {&L->tri_ptr, &L->d_tri_ptr},
               {&L->tri_idx, &L->d_tri_idx},
               {&L->tri_tiles, &L->d_tri_tiles}};
  for (auto &pt : parts) {
    const size_t cnt = pt.src->size();
    if (cnt && hipMemcpy(b + off, pt.src->data(), cnt * sizeof(int32_t),
                         hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(p);
      (void)hipGetLastError();
      return fail(RADIAL_E_HIP, "hipMemcpy of the layout failed");
    }
    *pt.dst = cnt ? b + off : nullptr;  // empty arrays (group lists not built) stay null
    off += cnt;
  }
  L->d_base = p;
  L->device = dev;
  return RADIAL_OK;
}

void radial_layout_destroy(radial_layout *L) {
  if (!L) return;
  free_device(L);
  delete L;
}

static radial::MaskGeom mask_geom(const radial_layout *L) {
  radial::MaskGeom m;
  m.s = static_cast<int32_t>(L->tokens_per_frame);
  m.frames = static_cast<int32_t>(L->frames);
  m.sink = (L->flags & RADIAL_SINK) ? 1 : 0;
  m.exact = ((L->flags & RADIAL_TOKEN_EXACT) && !(L->flags & RADIAL_DENSE)) ? 1 : 0;
  m.decay = L->params.decay;
  m.central = L->params.central_band;
  m.band_rtab = L->d_band_rtab;
  const radial_mask_params &p = L->params;
  m.pow2_shift = -1;
  if (p.decay == RADIAL_DECAY_RADIAL && p.scale_den > 0 && p.scale_num % p.scale_den == 0) {
    const int32_t c = p.scale_num / p.scale_den;
    if ((c & (c - 1)) == 0) m.pow2_shift = 31 - __builtin_clz(uint32_t(c));
  }
  // division by s for dividends below 2^31: p = 31 + ceil(log2 s) and
  // m = ceil(2^p / s) (< 2^33) give floor(x / s) = (x m) >> p exactly,
  // since x (m s - 2^p) < 2^31 s <= 2^p
  const uint64_t sv = uint64_t(L->tokens_per_frame);
  int lg = 0;
  while ((uint64_t(1) << lg) < sv) ++lg;
  m.s_shift = 31 + lg;
  m.s_magic = ((uint64_t(1) << m.s_shift) + sv - 1) / sv;
  return m;
}

int radial_attn_fwd(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D,
                    float scale, const void *q, const void *k, const void *v, void *o,
                    float *lse, void *hip_stream) {
  int st = check_common(L, B, H, N, D, scale);
  if (st) return st;
  st = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {lse, "lse"}});
  if (st) return st;
  radial::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.row_ptr = L->d_row_ptr;
  a.col_idx = L->d_col_idx;
  a.pair_ptr = L->d_pair_ptr;
  a.pair_idx = L->d_pair_idx;
  a.tri_ptr = L->d_tri_ptr;
  a.tri_idx = L->d_tri_idx;
  a.tri_tiles = L->d_tri_tiles;
  a.n_tri = static_cast<int32_t>(L->tri_tiles.size() / 3);
  a.max_group = g_fwd_max_group.load(std::memory_order_relaxed);
  a.BH = B * H;
  a.N = static_cast<int32_t>(N);
  a.D = D;
  a.T = L->block;
  a.nb = L->nb;
  a.scale = scale;
  a.mask = mask_geom(L);
  const hipError_t e = radial::launch_fwd(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess)
    return fail(RADIAL_E_HIP, std::string("forward launch failed: ") + hipGetErrorString(e));
  return RADIAL_OK;
}

size_t radial_attn_bwd_workspace_bytes(const radial_layout *L, int32_t B, int32_t H, int64_t N,
                                       int32_t D) {
  (void)L;
  (void)D;
  if (B < 1 || H < 1 || N < 1) return 0;
  // two fp32 row arrays: -Delta and -LSE * log2(e), each 256-byte aligned
  const size_t bytes = (size_t)B * (size_t)H * (size_t)N * sizeof(float);
  return 2 * ((bytes + 255) & ~size_t(255));
}

}  // extern "C"

namespace {

// The backward's launches once every argument has been checked; `workspace`
// holds `need` bytes (the two row arrays, need / 2 bytes each).
int run_bwd(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D, float scale,
            const void *q, const void *k, const void *v, const void *o, const float *lse,
            const void *dout, void *dq, void *dk, void *dv, void *workspace, size_t need,
            void *hip_stream) {
  radial::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ndelta = static_cast<float *>(workspace);
  a.nlse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + need / 2);
  a.row_ptr = L->d_row_ptr;
  a.col_idx = L->d_col_idx;
  a.pair_ptr = L->d_pair_ptr;
  a.pair_idx = L->d_pair_idx;
  a.col_ptr = L->d_col_ptr;
  a.row_idx = L->d_row_idx;
  a.col_order = L->d_col_order;
  a.BH = B * H;
  a.N = static_cast<int32_t>(N);
  a.D = D;
  a.T = L->block;
  a.nb = L->nb;
  a.scale = scale;
  a.mask = mask_geom(L);
  const hipError_t e = radial::launch_bwd(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess)
    return fail(RADIAL_E_HIP, std::string("backward launch failed: ") + hipGetErrorString(e));
  return RADIAL_OK;
}

}  // namespace

extern "C" {

int radial_attn_bwd(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D,
                    float scale, const void *q, const void *k, const void *v, const void *o,
                    const float *lse, const void *dout, void *dq, void *dk, void *dv,
                    void *workspace, size_t workspace_bytes, void *hip_stream) {
  int st = check_common(L, B, H, N, D, scale);
  if (st) return st;
  st = check_ptrs({{q, "q"},
                   {k, "k"},
                   {v, "v"},
                   {o, "o"},
                   {lse, "lse"},
                   {dout, "dout"},
                   {dq, "dq"},
                   {dk, "dk"},
                   {dv, "dv"},
                   {workspace, "workspace"}});
  if (st) return st;
  const size_t need = radial_attn_bwd_workspace_bytes(L, B, H, N, D);
  if (workspace_bytes < need)
    return fail(RADIAL_E_INVALID, "workspace too small: need " + std::to_string(need) +
                                      " bytes, got " + std::to_string(workspace_bytes));
  return run_bwd(L, B, H, N, D, scale, q, k, v, o, lse, dout, dq, dk, dv, workspace, need,
                 hip_stream);
}

int radial_attn_bwd_noalloc(const radial_layout *L, int32_t B, int32_t H, int64_t N, int32_t D,
                            float scale, const void *q, const void *k, const void *v,
                            const void *o, const float *lse, const void *dout, void *dq,
                            void *dk, void *dv, void *hip_stream) {
  int st = check_common(L, B, H, N, D, scale);
  if (st) return st;
  st = check_ptrs({{q, "q"},
                   {k, "k"},
                   {v, "v"},
                   {o, "o"},
                   {lse, "lse"},
                   {dout, "dout"},
                   {dq, "dq"},
                   {dk, "dk"},
                   {dv, "dv"}});
  if (st) return st;
  const size_t need = radial_attn_bwd_workspace_bytes(L, B, H, N, D);
  if (need > radial::kBwdScratchBytes)
    return fail(RADIAL_E_UNSUPPORTED,
                "B * H * N too large for the static scratch: the row arrays need " +
                    std::to_string(need) + " bytes, the scratch holds " +
                    std::to_string(radial::kBwdScratchBytes) + " (RADIAL_BWD_SCRATCH_BYTES)");
  // check_common made sure the layout's device is the current one
  void *scratch = nullptr;
  const hipError_t e = radial::bwd_scratch(L->device, &scratch);
  if (e != hipSuccess)
    return fail(RADIAL_E_HIP, std::string("static scratch lookup failed: ") +
                                  hipGetErrorString(e));
  return run_bwd(L, B, H, N, D, scale, q, k, v, o, lse, dout, dq, dk, dv, scratch, need,
                 hip_stream);
}

int radial_test_set_fail_alloc(int32_t on) {
  if (on != 0 && on != 1) return fail(RADIAL_E_INVALID, "on must be 0 or 1");
  return g_fail_alloc.exchange(on);
}

int radial_test_set_fwd_group(int32_t max_group) {
  if (max_group < 1 || max_group > 3)
    return fail(RADIAL_E_INVALID, "max_group must be 1, 2 or 3");
  return g_fwd_max_group.exchange(max_group);
}

const char *radial_status_string(int status) {
  switch (status) {
    case RADIAL_OK: return "ok";
    case RADIAL_E_INVALID: return "invalid argument";
    case RADIAL_E_UNSUPPORTED: return "unsupported shape or size";
    case RADIAL_E_SHAPE: return "shape mismatch";
    case RADIAL_E_NOMEM: return "out of memory";
    case RADIAL_E_HIP: return "HIP error";
    case RADIAL_E_STATE: return "layout not on the current device";
    default: return "unknown status";
  }
}

const char *radial_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
