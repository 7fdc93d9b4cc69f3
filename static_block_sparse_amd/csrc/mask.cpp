// Radial mask compiler: (frames, tokens per frame, tile edge, flags) ->
// block-sparse tile lists (CSR for the forward and dQ passes, CSC for the
// dK/dV pass).
//
// Mask definition (jaehun.me review "Radial Attention: O(n log n) Sparse
// Attention with Energy Decay for Long Video Generation", Prompt 1.3.1):
//   * temporal band of a frame pair at distance delta:
//       r = floor(log2(max(delta, 1)))           (Step 2-A; paper §4.2 Fig.5a)
//   * spatial half width kept inside that frame pair:
//       w = floor(s / 2^r)                        (Step 2-B; paper Fig.5b)
//     and a key at in-frame position b is reachable from position a iff
//     |a - b| < w (strict edge, as the toy example with s = 9, w = 4 admits
//     positions 1..7 around the centre 4);
//   * below unit width (w == 0) only the diagonal b == a is kept, and only
//     for frame pairs whose distance is a multiple of ceil(2^r / s), which
//     keeps the band's amortised density near 2^-r (Step 2-C; paper Fig.5
//     caption);
//   * mask variants (rebuttal ablations; review 1.3.2 / Appx C.3): the
//     distance is shifted by the central band d, e = max(delta - d + 1, 1),
//     r = floor(log2 e), and the width divisor 2^r becomes c^r for a width
//     scale c, or e for the harmonic-series decay (the period likewise);
//   * attention sink: all of frame 0 is reachable (Step 4; paper Eq.8);
//   * tiles: a T x T tile is kept iff it holds at least one allowed pair,
//     and kept tiles are computed in full (Step 5; paper §4.2).  For
//     token-exact semantics (paper Eq.4 at token granularity) each kept tile
//     is also marked full (every valid pair allowed) or partial.
//
// Construction: for one query tile, its rows fall into one or more frame
// segments (frame i, positions a0..a1).  Against key frame j the keys
// reachable from a whole segment form a single position run
// [a0 - w + 1, a1 + w - 1] clipped to the frame (runs of consecutive query
// positions overlap because every run is at least one key wide), or
// [a0, a1] on the sampled diagonal, or the whole frame for the sink.  Each
// run maps to a run of key tiles; the union of the runs of a query tile,
// sorted and merged, is its CSR row.  The keys of frame j reachable from
// *every* position of a segment are [a1 - w + 1, a0 + w - 1] (clipped), the
// single position a0 on the sampled diagonal when a0 == a1, or the whole
// frame for the sink; intersected over the tile's segments this gives, per
// key frame, the keys every query of the tile may attend, and a kept tile
// whose keys lie inside that set in each of its frames is full.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "kernels.h"
#include "layout.h"
#include "radial.h"

namespace radial {

// Triples of query tiles for the forward, three tiles per triple (-1: none).
// A greedy pass in tile order puts each tile not yet grouped with the two
// ungrouped tiles among the next W that leave its group the fewest key tiles
// outside their own rows (ties: the nearest).  W spans two frames of tiles:
// tiles at the same place in neighbouring frames select nearly the same key
// tiles in the narrow far bands, where adjacent tiles of one frame do not.
// Consecutive triples when the layout is too large for the search.
static std::vector<int32_t> group_triples(const radial_layout &L) {
  const int64_t nb = L.nb, T = L.block, s = L.tokens_per_frame;
  const int64_t W = std::min<int64_t>(256, 2 * ((s + T - 1) / T) + 2);
  const int64_t words = (nb + 63) / 64;
  std::vector<int32_t> out;
  if (nb * words > (int64_t(1) << 23) || nb * W * words > (int64_t(1) << 30)) {
    for (int64_t u = 0; u < nb; u += 3)
      for (int64_t k = 0; k < 3; ++k) out.push_back(u + k < nb ? int32_t(u + k) : -1);
    return out;
  }
  std::vector<uint64_t> rows(nb * words, 0), un(words);
  for (int64_t u = 0; u < nb; ++u)
    for (int32_t t = L.row_ptr[u]; t < L.row_ptr[u + 1]; ++t)
      rows[u * words + L.col_idx[t] / 64] |= uint64_t(1) << (L.col_idx[t] % 64);
  std::vector<uint8_t> used(nb, 0);
  for (int64_t u = 0; u < nb; ++u) {
    if (used[u]) continue;
    used[u] = 1;
    std::copy(rows.begin() + u * words, rows.begin() + (u + 1) * words, un.begin());
    int32_t g[3] = {int32_t(u), -1, -1};
    for (int k = 1; k < 3; ++k) {
      int64_t best = -1, best_cost = INT64_MAX;
      for (int64_t v = u + 1; v < nb && v <= u + W; ++v) {
        if (used[v]) continue;
        const uint64_t *rv = &rows[v * words];
        int64_t cost = 0;  // key tiles of the group outside row v
        for (int64_t w = 0; w < words; ++w) cost += __builtin_popcountll(un[w] & ~rv[w]);
        if (cost < best_cost) {
          best_cost = cost;
          best = v;
        }
      }
      if (best < 0) break;
      used[best] = 1;
      g[k] = int32_t(best);
      for (int64_t w = 0; w < words; ++w) un[w] |= rows[best * words + w];
    }
    out.insert(out.end(), g, g + 3);
  }
  return out;
}
namespace {

inline int bit_length(uint64_t x) { return x == 0 ? 0 : 64 - __builtin_clzll(x); }

struct Band {
  int32_t r;
  int64_t w;
  int64_t period;
};

// sampling periods beyond every frame distance are stored as this
constexpr int64_t kPeriodCap = (int64_t(1) << 31) - 1;

using u128 = unsigned __int128;

inline u128 pow_u128(u128 b, int e) {
  u128 x = 1;
  while (e-- > 0) x *= b;
  return x;
}

// Width and period of a band whose width divisor is num / den (exact
// rational arithmetic: num <= 16^31 < 2^128, s * den <= 2^31 * 4^31 < 2^128).
inline void width_of(u128 num, u128 den, int64_t s, Band &b) {
  const u128 sd = u128(s) * den;
  b.w = static_cast<int64_t>(sd / num);
  if (b.w >= 1) {
    b.period = 1;
  } else {
    const u128 q = (num + sd - 1) / sd;
    b.period = q > u128(kPeriodCap) ? kPeriodCap : static_cast<int64_t>(q);
  }
}

inline Band band_of(int64_t delta, int64_t s, const radial_mask_params &p) {
  const int64_t e = std::max<int64_t>(delta - p.central_band + 1, 1);
  Band b;
  b.r = bit_length(static_cast<uint64_t>(e)) - 1;
  if (p.decay == RADIAL_DECAY_HARMONIC)
    width_of(u128(e), 1, s, b);
  else
    width_of(pow_u128(u128(p.scale_num), b.r), pow_u128(u128(p.scale_den), b.r), s, b);
  return b;
}

}  // namespace

std::string build_layout(int64_t frames, int64_t s, int32_t T, uint32_t flags,
                         const radial_mask_params &params, radial_layout &L) {
  if (frames < 1) return "frames must be >= 1";
  if (params.decay != RADIAL_DECAY_RADIAL && params.decay != RADIAL_DECAY_HARMONIC)
    return "unknown decay";
  if (params.central_band < 0) return "central_band must be >= 0";
  if (params.decay == RADIAL_DECAY_RADIAL &&
      (params.scale_den < 1 || params.scale_den > 4 || params.scale_num <= params.scale_den ||
       params.scale_num > 16))
    return "width scale must be num/den with 1 <= den <= 4 and den < num <= 16";
  if (s < 1) return "tokens_per_frame must be >= 1";
  if (T < 1 || T > 4096) return "block_size must be in [1, 4096]";
  if (flags & ~uint32_t(RADIAL_SINK | RADIAL_DENSE | RADIAL_TOKEN_EXACT))
    return "unknown flag bits";
  if (frames > (int64_t(1) << 31) / s) return "frames * tokens_per_frame must be < 2^31";
  const int64_t n = frames * s;
  if (n >= (int64_t(1) << 31)) return "frames * tokens_per_frame must be < 2^31";
  const bool sink = flags & RADIAL_SINK;
  const bool dense = flags & RADIAL_DENSE;

  L.frames = frames;
  L.tokens_per_frame = s;
  L.n = n;
  L.block = T;
  L.flags = flags;
  L.params = params;
  const int64_t nb = (n + T - 1) / T;
  L.nb = static_cast<int32_t>(nb);

  L.band_r.resize(frames);
  L.band_w.resize(frames);
  L.band_period.resize(frames);
  for (int64_t d = 0; d < frames; ++d) {
    const Band b = band_of(d, s, params);
    L.band_r[d] = b.r;
    L.band_w[d] = b.w;
    L.band_period[d] = b.period;
  }
  // per band index: the radial decay's width depends on r alone
  L.band_rtab.assign(64, 0);
  for (int r = 0; r < 32; ++r) {
    Band b;
    width_of(pow_u128(u128(params.scale_num > 0 ? params.scale_num : 2), r),
             pow_u128(u128(params.scale_den > 0 ? params.scale_den : 1), r), s, b);
    L.band_rtab[r] = static_cast<int32_t>(b.w);
    L.band_rtab[32 + r] = static_cast<int32_t>(b.period);
  }

  L.row_ptr.assign(nb + 1, 0);
  L.col_idx.clear();
  std::vector<std::pair<int64_t, int64_t>> runs;
  for (int64_t u = 0; u < nb; ++u) {
    const int64_t q0 = u * T;
    const int64_t q1 = std::min(n, q0 + T) - 1;
    if (dense) {
      for (int64_t v = 0; v < nb; ++v) L.col_idx.push_back(static_cast<int32_t>(v));
      L.row_ptr[u + 1] = static_cast<int32_t>(L.col_idx.size());
      continue;
    }
    runs.clear();
    for (int64_t i = q0 / s; i <= q1 / s; ++i) {
      const int64_t a0 = (i == q0 / s) ? q0 % s : 0;
      const int64_t a1 = (i == q1 / s) ? q1 % s : s - 1;
      for (int64_t j = 0; j < frames; ++j) {
        int64_t lo, hi;
        if (sink && j == 0) {
          lo = 0;
          hi = s - 1;
        } else {
          const int64_t delta = i > j ? i - j : j - i;
          const int64_t w = L.band_w[delta];
          if (w >= 1) {
            lo = std::max<int64_t>(0, a0 - w + 1);
            hi = std::min<int64_t>(s - 1, a1 + w - 1);
          } else if (delta % L.band_period[delta] == 0) {
            lo = a0;
            hi = a1;
          } else {
            continue;
          }
        }
        runs.emplace_back((j * s + lo) / T, (j * s + hi) / T);
      }
    }
    std::sort(runs.begin(), runs.end());
    int64_t next = -1;  // first key tile not yet emitted
    for (const auto &rv : runs) {
      for (int64_t v = std::max(rv.first, next); v <= rv.second; ++v)
        L.col_idx.push_back(static_cast<int32_t>(v));
      next = std::max(next, rv.second + 1);
    }
    L.row_ptr[u + 1] = static_cast<int32_t>(L.col_idx.size());
  }
  L.nnz_tiles = static_cast<int64_t>(L.col_idx.size());
  if (L.nnz_tiles >= (int64_t(1) << 31)) return "too many tiles for 32-bit indices";

  // full / partial kept tiles
  L.full.assign(L.nnz_tiles, 1);
  if (!dense) {
    std::vector<int64_t> clo(frames), chi(frames);  // common keys per key frame, [clo, chi]
    for (int64_t u = 0; u < nb; ++u) {
      const int64_t q0 = u * T;
      const int64_t q1 = std::min(n, q0 + T) - 1;
      std::fill(clo.begin(), clo.end(), int64_t(0));
      std::fill(chi.begin(), chi.end(), s - 1);
      for (int64_t i = q0 / s; i <= q1 / s; ++i) {
        const int64_t a0 = (i == q0 / s) ? q0 % s : 0;
        const int64_t a1 = (i == q1 / s) ? q1 % s : s - 1;
        for (int64_t j = 0; j < frames; ++j) {
          int64_t lo, hi;
          if (sink && j == 0) {
            lo = 0;
            hi = s - 1;
          } else {
            const int64_t delta = i > j ? i - j : j - i;
            const int64_t w = L.band_w[delta];
            if (w >= 1) {
              lo = std::max<int64_t>(0, a1 - w + 1);
              hi = std::min<int64_t>(s - 1, a0 + w - 1);
            } else if (a0 == a1 && delta % L.band_period[delta] == 0) {
              lo = hi = a0;
            } else {
              lo = 1;
              hi = 0;  // empty
            }
          }
          clo[j] = std::max(clo[j], lo);
          chi[j] = std::min(chi[j], hi);
        }
      }
      for (int32_t t = L.row_ptr[u]; t < L.row_ptr[u + 1]; ++t) {
        const int64_t k0 = int64_t(L.col_idx[t]) * T;
        const int64_t k1 = std::min(n, k0 + T) - 1;
        bool full = true;
        for (int64_t j = k0 / s; j <= k1 / s && full; ++j) {
          const int64_t b0 = std::max(k0, j * s) - j * s;
          const int64_t b1 = std::min(k1, j * s + s - 1) - j * s;
          full = clo[j] <= b0 && b1 <= chi[j];
        }
        L.full[t] = full ? 1 : 0;
      }
    }
  }

  // forward groups: per G query tiles (G consecutive ones, or those that
  // `members` lists, G per group, -1 for none), the sorted union of their
  // key tiles, each entry tagged with a membership bit and a partial bit per
  // tile of the group (pairs: the kPair fields; triples: the kTri fields)
  auto build_groups = [&](int G, int32_t tile_mask, const int32_t *in_bit,
                          const int32_t *part_bit, const std::vector<int32_t> *members,
                          std::vector<int32_t> &ptr, std::vector<int32_t> &idx) {
    ptr.clear();
    idx.clear();
    if (nb > tile_mask) return;
    const int64_t ng = members ? int64_t(members->size()) / G : (nb + G - 1) / G;
    ptr.assign(ng + 1, 0);
    idx.reserve(L.nnz_tiles);
    for (int64_t gi = 0; gi < ng; ++gi) {
      int32_t pos[3] = {0, 0, 0}, end[3] = {0, 0, 0};
      for (int k = 0; k < G; ++k) {
        const int64_t u = members ? (*members)[G * gi + k] : G * gi + k;
        if (u >= 0 && u < nb) {
          pos[k] = L.row_ptr[u];
          end[k] = L.row_ptr[u + 1];
        }
      }
      for (;;) {
        int32_t v = INT32_MAX;
        for (int k = 0; k < G; ++k)
          if (pos[k] < end[k] && L.col_idx[pos[k]] < v) v = L.col_idx[pos[k]];
        if (v == INT32_MAX) break;
        int32_t e = v;
        for (int k = 0; k < G; ++k)
          if (pos[k] < end[k] && L.col_idx[pos[k]] == v) {
            e |= in_bit[k] | (L.full[pos[k]] ? 0 : part_bit[k]);
            ++pos[k];
          }
        idx.push_back(e);
      }
      ptr[gi + 1] = static_cast<int32_t>(idx.size());
    }
  };
  const int32_t pair_in[3] = {kPairInA, kPairInB, 0}, pair_part[3] = {kPairPartA, kPairPartB, 0};
  build_groups(2, kPairTile, pair_in, pair_part, nullptr, L.pair_ptr, L.pair_idx);
  const int32_t tri_in[3] = {kTriIn, kTriIn << 1, kTriIn << 2};
  const int32_t tri_part[3] = {kTriPart, kTriPart << 1, kTriPart << 2};
  L.tri_tiles = group_triples(L);
  build_groups(3, kTriTile, tri_in, tri_part, &L.tri_tiles, L.tri_ptr, L.tri_idx);
  if (L.tri_ptr.empty()) L.tri_tiles.clear();

  // transpose to CSC (query tiles ascending within each key tile)
  L.col_ptr.assign(nb + 1, 0);
  for (int32_t v : L.col_idx) L.col_ptr[v + 1]++;
  for (int64_t v = 0; v < nb; ++v) L.col_ptr[v + 1] += L.col_ptr[v];
  L.row_idx.assign(L.nnz_tiles, 0);
  L.full_csc.assign(L.nnz_tiles, 1);
  {
    std::vector<int32_t> fill(L.col_ptr.begin(), L.col_ptr.end() - 1);
    for (int64_t u = 0; u < nb; ++u)
      for (int32_t t = L.row_ptr[u]; t < L.row_ptr[u + 1]; ++t) {
        const int32_t at = fill[L.col_idx[t]]++;
        L.row_idx[at] = static_cast<int32_t>(u);
        L.full_csc[at] = L.full[t];
      }
  }

  // longest columns first for the dK/dV pass (the sink columns of frame 0
  // hold every query tile); ties keep ascending tile order
  L.col_order.resize(nb);
  for (int64_t v = 0; v < nb; ++v) L.col_order[v] = static_cast<int32_t>(v);
  std::stable_sort(L.col_order.begin(), L.col_order.end(), [&](int32_t a, int32_t b) {
    return (L.col_ptr[a + 1] - L.col_ptr[a]) > (L.col_ptr[b + 1] - L.col_ptr[b]);
  });

  // valid token pairs inside kept tiles
  int64_t pairs = 0;
  for (int64_t u = 0; u < nb; ++u) {
    const int64_t rows = std::min<int64_t>(T, n - u * T);
    int64_t cols = 0;
    for (int32_t t = L.row_ptr[u]; t < L.row_ptr[u + 1]; ++t)
      cols += std::min<int64_t>(T, n - int64_t(L.col_idx[t]) * T);
    pairs += rows * cols;
  }
  L.nnz_pairs = pairs;
  return std::string();
}

bool token_allowed(const radial_layout &L, int64_t q, int64_t k) {
  const int64_t s = L.tokens_per_frame;
  if (L.flags & RADIAL_DENSE) return true;
  const int64_t i = q / s, a = q % s, j = k / s, b = k % s;
  if ((L.flags & RADIAL_SINK) && j == 0) return true;
  const int64_t delta = i > j ? i - j : j - i;
  const int64_t w = L.band_w[delta];
  if (w >= 1) return (a > b ? a - b : b - a) < w;
  return a == b && delta % L.band_period[delta] == 0;
}

}  // namespace radial
