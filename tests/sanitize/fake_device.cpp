// Test infrastructure: a host-memory stand-in for the HIP runtime and the
// kernel launchers, linked with the library's host sources (mask compiler and
// C ABI) into an AddressSanitizer / UndefinedBehaviorSanitizer build.
//
// Device allocations are plain heap blocks, so the sanitizers see every
// layout copy the C ABI makes.  The launchers run no kernel: they check the
// arguments the C ABI assembled and read or write the first and last element
// of every range a kernel would touch (inputs read, outputs and workspace
// written), so a wrong size or offset shows up as a heap overflow.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kernels.h"

namespace {

int g_fail = 0;

void check(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "fake device: check failed: %s\n", what);
    g_fail = 1;
  }
}

// volatile accesses so the compiler keeps them
void read_range(const void *p, size_t bytes) {
  if (!bytes) return;
  const volatile unsigned char *c = static_cast<const volatile unsigned char *>(p);
  (void)c[0];
  (void)c[bytes - 1];
}
void write_range(void *p, size_t bytes) {
  if (!bytes) return;
  volatile unsigned char *c = static_cast<volatile unsigned char *>(p);
  c[0] = 0;
  c[bytes - 1] = 0;
}

// tile lists: row_ptr (nb + 1) and its index list, indices below nb once bit
// 31 (the partial-tile mark) is cleared
void check_lists(const int32_t *ptr, const int32_t *idx, int32_t nb, const char *what) {
  check(ptr[0] == 0, what);
  for (int32_t u = 0; u < nb; ++u) check(ptr[u + 1] >= ptr[u], what);
  for (int32_t t = 0; t < ptr[nb]; ++t) {
    const int32_t v = idx[t] & 0x7fffffff;
    check(v >= 0 && v < nb, what);
  }
}

void check_mask(const radial::MaskGeom &m) {
  check(m.s >= 1 && m.frames >= 1, "mask geometry");
  check(m.band_rtab != nullptr, "band table uploaded");
  read_range(m.band_rtab, 64 * sizeof(int32_t));
  check(m.s_shift >= 31 && m.s_shift <= 62, "division shift");
}

// group lists: for query tiles G g .. G g + G - 1, the sorted union of their
// CSR rows, each entry marked with a membership bit per row (in << k) and, in
// token-exact uploads, a partial bit per member row (part << k) equal to the
// partial mark (bit 31) of that row's CSR entry
// tiles: the query tiles of each group (G per group, -1 for none; every
// tile exactly once), or null for groups of consecutive tiles
void check_groups(int G, const int32_t *row_ptr, const int32_t *col_idx, const int32_t *gptr,
                  const int32_t *gidx, const int32_t *tiles, int32_t ng, int32_t nb,
                  int32_t tile_mask, int32_t in, int32_t part, bool exact) {
  check(gptr != nullptr && gidx != nullptr, "group lists uploaded");
  if (!gptr || !gidx) return;
  if (!tiles) check(ng == (nb + G - 1) / G, "group count");
  if (tiles) {
    read_range(tiles, size_t(ng) * G * 4);
    std::vector<int> seen(nb, 0);
    for (int32_t i = 0; i < ng * G; ++i) {
      check(tiles[i] >= -1 && tiles[i] < nb, "group tile in range");
      if (tiles[i] >= 0) ++seen[tiles[i]];
    }
    for (int32_t u = 0; u < nb; ++u) check(seen[u] == 1, "every query tile in one group");
  }
  check(gptr[0] == 0, "group lists start");
  for (int32_t g = 0; g < ng; ++g) {
    int32_t pos[3] = {0, 0, 0}, end[3] = {0, 0, 0};
    for (int k = 0; k < G; ++k) {
      const int32_t u = tiles ? tiles[G * g + k] : G * g + k;
      if (u >= 0 && u < nb) {
        pos[k] = row_ptr[u];
        end[k] = row_ptr[u + 1];
      }
    }
    int32_t prev = -1;
    for (int32_t t = gptr[g]; t < gptr[g + 1]; ++t) {
      const int32_t e = gidx[t], v = e & tile_mask;
      check(v > prev && v < nb, "group list sorted, in range");
      prev = v;
      bool any = false;
      for (int k = 0; k < G; ++k) {
        const bool mem = pos[k] < end[k] && (col_idx[pos[k]] & 0x7fffffff) == v;
        check(((e & (in << k)) != 0) == mem, "membership bits");
        if (mem && exact) check(((e & (part << k)) != 0) == (col_idx[pos[k]] < 0), "partial bits");
        if (mem) ++pos[k];
        any = any || mem;
      }
      check(any, "group entry comes from a row");
    }
    for (int k = 0; k < G; ++k) check(pos[k] == end[k], "group list covers every row");
  }
}
void check_pairs(const int32_t *row_ptr, const int32_t *col_idx, const int32_t *pair_ptr,
                 const int32_t *pair_idx, int32_t nb, bool exact) {
  check_groups(2, row_ptr, col_idx, pair_ptr, pair_idx, nullptr, (nb + 1) / 2, nb,
               radial::kPairTile, radial::kPairInA, radial::kPairPartA, exact);
}

}  // namespace

extern "C" int fake_device_failures() { return g_fail; }

// ---- HIP runtime entry points the C ABI uses --------------------------------
hipError_t hipGetDevice(int *device) {
  if (std::getenv("FAKE_DEVICE_NONE")) return hipErrorNoDevice;
  *device = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipMalloc(void **ptr, size_t size) {
  *ptr = std::malloc(size ? size : 1);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *ptr) {
  std::free(ptr);
  return hipSuccess;
}
hipError_t hipMemcpy(void *dst, const void *src, size_t bytes, hipMemcpyKind) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char *hipGetErrorString(hipError_t) { return "fake device error"; }

// ---- kernel launchers ---------------------------------------------------------
namespace radial {

hipError_t launch_fwd(const FwdArgs &a, hipStream_t) {
  const size_t x = size_t(a.BH) * a.N * a.D * 2, r = size_t(a.BH) * a.N * 4;
  check(a.BH >= 1 && a.N >= 1 && a.nb == (a.N + a.T - 1) / a.T, "forward sizes");
  check(int64_t(a.N) * a.D * 2 < (int64_t(1) << 31), "forward slice below 2^31 bytes");
  read_range(a.q, x);
  read_range(a.k, x);
  read_range(a.v, x);
  write_range(a.o, x);
  write_range(a.lse, r);
  check_lists(a.row_ptr, a.col_idx, a.nb, "forward CSR");
  check_pairs(a.row_ptr, a.col_idx, a.pair_ptr, a.pair_idx, a.nb, a.mask.exact);
  check(a.tri_tiles != nullptr && a.n_tri >= (a.nb + 2) / 3 && a.n_tri <= a.nb, "triples");
  if (a.tri_tiles)
    check_groups(3, a.row_ptr, a.col_idx, a.tri_ptr, a.tri_idx, a.tri_tiles, a.n_tri, a.nb,
                 radial::kTriTile, radial::kTriIn, radial::kTriPart, a.mask.exact);
  check(a.max_group >= 1 && a.max_group <= 3, "forward group cap");
  check_mask(a.mask);
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t) {
  const size_t x = size_t(a.BH) * a.N * a.D * 2, r = size_t(a.BH) * a.N * 4;
  check(a.BH >= 1 && a.N >= 1 && a.nb == (a.N + a.T - 1) / a.T, "backward sizes");
  check(int64_t(a.N) * a.D * 2 < (int64_t(1) << 31), "backward slice below 2^31 bytes");
  for (const void *p : {a.q, a.k, a.v, a.o, a.dout}) read_range(p, x);
  read_range(a.lse, r);
  for (void *p : {a.dq, a.dk, a.dv}) write_range(p, x);
  write_range(a.ndelta, r);
  write_range(a.nlse2, r);
  check(a.nlse2 >= a.ndelta + size_t(a.BH) * a.N, "workspace arrays overlap");
  check_lists(a.row_ptr, a.col_idx, a.nb, "backward CSR");
  check_lists(a.col_ptr, a.row_idx, a.nb, "backward CSC");
  check_pairs(a.row_ptr, a.col_idx, a.pair_ptr, a.pair_idx, a.nb, a.mask.exact);
  // col_order: a permutation of the key tiles
  unsigned char *seen = static_cast<unsigned char *>(std::calloc(a.nb, 1));
  for (int32_t i = 0; i < a.nb; ++i) {
    const int32_t v = a.col_order[i];
    check(v >= 0 && v < a.nb && !seen[v], "column order is a permutation");
    if (v >= 0 && v < a.nb) seen[v] = 1;
  }
  std::free(seen);
  check_mask(a.mask);
  return hipSuccess;
}

// the static scratch: a heap block of the stated size, looked up per device
hipError_t bwd_scratch(int device, void **ptr) {
  static void *block = nullptr;
  check(device == 0, "scratch looked up on the current device");
  if (!block) block = std::malloc(kBwdScratchBytes);
  *ptr = block;
  return block ? hipSuccess : hipErrorOutOfMemory;
}

}  // namespace radial
