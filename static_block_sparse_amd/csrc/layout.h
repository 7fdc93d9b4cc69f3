// Internal definition of the radial layout (host arrays + device copy).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "radial.h"

struct radial_layout {
  int64_t frames = 0;
  int64_t tokens_per_frame = 0;
  int64_t n = 0;           // frames * tokens_per_frame
  int32_t block = 0;       // tile edge T
  uint32_t flags = 0;
  radial_mask_params params{RADIAL_DECAY_RADIAL, 1, 2, 1};
  int32_t nb = 0;          // ceil(n / T)
  int64_t nnz_tiles = 0;
  int64_t nnz_pairs = 0;

  std::vector<int32_t> band_r;      // per frame distance
  std::vector<int64_t> band_w;
  std::vector<int64_t> band_period;
  // per band index r in [0, 32): w at [r], period at [32 + r] (radial decay;
  // what the device predicate looks up)
  std::vector<int32_t> band_rtab;

  std::vector<int32_t> row_ptr, col_idx;  // CSR: key tiles per query tile
  std::vector<int32_t> col_ptr, row_idx;  // CSC: query tiles per key tile
  std::vector<int32_t> col_order;         // key tiles, longest column first
  // forward pass, per pair of query tiles (2p, 2p + 1): the sorted union of
  // their key tiles; entry = key tile | kPairInA | kPairInB (member of row
  // 2p / 2p + 1) | kPairPartA | kPairPartB (partial in that row).  Built when
  // the tile index fits below 2^27 (every supported tile size).
  std::vector<int32_t> pair_ptr, pair_idx;
  // the same per triple of query tiles tri_tiles[3t + k], k < 3 (-1: no
  // tile), chosen to share key tiles (see group_triples): entry = key tile
  // | kTriIn << k (member of row tri_tiles[3t + k]) | kTriPart << k (partial
  // in that row).  Built when the tile index fits below 2^25.
  std::vector<int32_t> tri_tiles, tri_ptr, tri_idx;
  // full[t] = 1 when every valid token pair of CSR tile t is allowed (no
  // masking needed under token-exact semantics), else 0; full_csc in CSC order
  std::vector<uint8_t> full, full_csc;

  // device copy (one allocation): row_ptr | col_idx | col_ptr | row_idx |
  // col_order | band_rtab | pair_ptr | pair_idx | tri_ptr | tri_idx |
  // tri_tiles
  int device = -1;
  void *d_base = nullptr;
  const int32_t *d_row_ptr = nullptr;
  const int32_t *d_col_idx = nullptr;
  const int32_t *d_col_ptr = nullptr;
  const int32_t *d_row_idx = nullptr;
  const int32_t *d_col_order = nullptr;
  const int32_t *d_band_rtab = nullptr;
  const int32_t *d_pair_ptr = nullptr;
  const int32_t *d_pair_idx = nullptr;
  const int32_t *d_tri_ptr = nullptr;
  const int32_t *d_tri_idx = nullptr;
  const int32_t *d_tri_tiles = nullptr;
};

namespace radial {

// Fills everything above except the device copy.  Returns an empty string
// on success, else a description of what was invalid.
std::string build_layout(int64_t frames, int64_t tokens_per_frame, int32_t block,
                         uint32_t flags, const radial_mask_params &params, radial_layout &L);

// Token predicate of the layout's mask (tests only).
bool token_allowed(const radial_layout &L, int64_t q, int64_t k);

}  // namespace radial
