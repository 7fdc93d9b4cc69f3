// Host-side launchers of the radial attention kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace radial {

// Fields of an entry of the forward pass's pair lists (per pair of query
// tiles 2p, 2p + 1, the sorted union of their key tiles): the key tile, a
// membership bit per row (A = 2p, B = 2p + 1) and a partial-tile bit per row.
constexpr int32_t kPairTile = (1 << 27) - 1;
constexpr int32_t kPairInA = 1 << 27, kPairInB = 1 << 28;
constexpr int32_t kPairPartA = 1 << 29, kPairPartB = 1 << 30;

// Fields of an entry of the forward pass's triple lists (per triple of query
// tiles 3t, 3t + 1, 3t + 2, the sorted union of their key tiles): the key
// tile, membership bit kTriIn << k and partial-tile bit kTriPart << k for
// row 3t + k of the triple.
constexpr int32_t kTriTile = (1 << 25) - 1;
constexpr int32_t kTriIn = 1 << 25, kTriPart = 1 << 28;

// What the kernels need of the mask to apply it token by token inside the
// tiles a token-exact layout marks partial (bit 31 of the tile indices).
struct MaskGeom {
  int32_t s = 1;        // tokens per frame
  int32_t frames = 1;
  int32_t sink = 0;     // frame 0 keys always allowed
  int32_t exact = 0;    // token-exact layout
  int32_t decay = 0;    // RADIAL_DECAY_RADIAL (0) or RADIAL_DECAY_HARMONIC (1)
  int32_t central = 1;  // central band d
  // device: per band index r < 32, width at [r] and period at [32 + r]
  // (radial decay)
  const int32_t *band_rtab = nullptr;
  // radial decay with a width scale 2^pow2_shift: the width is s >> (k r)
  // without the table; -1 for other scales
  int32_t pow2_shift = 1;
  // x / s == (x * s_magic) >> s_shift for 0 <= x < 2^31
  uint64_t s_magic = uint64_t(1) << 31;
  int32_t s_shift = 31;
};

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *row_ptr, *col_idx;  // device CSR of the layout
  // per pair / triple of query tiles: the union of their key tiles (see
  // layout.h); null when not built
  const int32_t *pair_ptr, *pair_idx;
  const int32_t *tri_ptr, *tri_idx;
  const int32_t *tri_tiles;  // the query tiles of each triple (3 each, -1: none)
  int32_t n_tri;             // triples per (batch, head)
  // largest query-tile group the forward may use (3; lower only in tests)
  int32_t max_group;
  int32_t BH, N, D, T, nb;
  float scale;
  MaskGeom mask;
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *ndelta;                     // workspace: -rowsum(dO * O), fp32 [BH, N]
  float *nlse2;                      // workspace: -LSE * log2(e), fp32 [BH, N]
  const int32_t *row_ptr, *col_idx;  // CSR (dQ pass)
  const int32_t *pair_ptr, *pair_idx;  // pair lists (dQ pass, see above)
  const int32_t *col_ptr, *row_idx;  // CSC (dK/dV pass)
  const int32_t *col_order;          // key tiles, longest column first
  int32_t BH, N, D, T, nb;
  float scale;
  MaskGeom mask;
};

// Both return hipErrorInvalidValue for an unsupported (D, T) pair.
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);

// Size of the backward's static device scratch (attn_bwd.hip): room for the
// two fp32 row arrays of radial_attn_bwd's workspace at B * H * N rows up to
// about 8.4 million.  Held by every device the library runs on until the
// process ends.
constexpr size_t kBwdScratchBytes = size_t(64) << 20;

// Device address of the backward's static scratch array on `device`, which
// must be the current device: looked up once per device, then cached.
hipError_t bwd_scratch(int device, void **ptr);

}  // namespace radial
