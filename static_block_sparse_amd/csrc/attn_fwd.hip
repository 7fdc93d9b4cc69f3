// Radial block-sparse attention forward on gfx950.
//
// A workgroup computes G query tiles u (T rows each) of one (batch, head);
// for every u (with its own waves):
//   for each kept key tile v of row u (CSR, ascending), in chunks of KC keys:
//     S^T = K_c Q_u^T                (bf16 MFMA, fp32 accumulate)
//     online softmax over keys       (running max and sum per query, fp32)
//     O^T += V_c^T P^T               (P rounded to bf16)
//   O = O / l,  LSE = m + ln l.
// This is masked softmax attention (jaehun.me review "Radial Attention:
// O(n log n) Sparse Attention with Energy Decay for Long Video Generation",
// Prompt 1.3.1 Step 0; paper §3 Eq.1-2) evaluated tile by tile over the
// kept tiles of the radial mask (Step 5; paper §4.2), with keys >= N masked.
//
// Layout of the work:
//  * wave w owns queries [32w, 32w + 32) of its tile; its Q rows stay in
//    registers as the B operand of S^T = K Q^T.  Computing S transposed puts
//    one query per lane column: a row's max and sum need one exchange
//    between lanes l and l ^ 32 (v_permlane32_swap), and P feeds P V as the
//    B operand with no lane movement (see device_common.h).
//  * K and V chunks sit row-major in LDS with an XOR swizzle of the 16-byte
//    column blocks; the V^T operand is read with the gfx950 transposing LDS
//    load (ds_read_b64_tr_b16).
//  * K and V chunks are copied global -> LDS by the buffer unit directly (no
//    staging registers); the swizzle is chosen through each lane's source
//    offset and keys past N read as zeros.  Chunks are double buffered: the
//    copy of chunk c + 1 is issued before the products of chunk c, with one
//    barrier per chunk.
//  * the running max is a reference value that moves lazily: a chunk's
//    probabilities are formed against it directly, and only when one of a
//    lane's exceeds 2^16 (seen from the lane's chunk sum, which bounds them
//    all) is the chunk redone with its true row max, moving the reference
//    when that exceeds it by more than 8 (log2 units).  The ratios O / l
//    and the LSE are exact whatever the reference; the max reduction and
//    the O rescale are skipped on almost every chunk.
//  * query-tile groups: a workgroup of G T / 32 waves takes G query tiles
//    (G = 3, three waves per SIMD; pairs or single tiles only when the mask
//    compiler built no triple lists) and walks the sorted union of their key
//    tiles.  Every staged chunk then serves G tiles' waves, which divides
//    the global -> LDS copies per product by about G; at the power cap the
//    copies' energy is a large share of the budget.  A wave skips the chunks
//    of key tiles its own tile does not keep.  Pairs are adjacent tiles
//    (6% of a pair's walk skipped at 720p); the mask compiler picks triples
//    that share key tiles, often the tiles at one place in neighbouring
//    frames (10% of a triple's walk skipped at 720p, 10% at 129 frames,
//    against 12% and 23% for adjacent tiles).
//  * token-exact layouts (EXACT): in the chunks of tiles marked partial,
//    each lane masks the keys outside its query's allowed runs (one per key
//    frame the chunk touches, however many) before the max.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

#ifndef RADIAL_FWD_XCD_BLOCK
#define RADIAL_FWD_XCD_BLOCK 16  // work items per XCD block (see xcd_remap)
#endif

namespace radial {

template <int D, int T, int G>
struct FwdCfg {
  static constexpr int NWR = T / 32;    // waves per query tile
  static constexpr int NW = NWR * G;    // waves per workgroup
  static constexpr int NT = NW * 64;    // threads per workgroup
  static constexpr int KC = 64;         // keys per pipeline chunk
  static constexpr int CPT = T / KC;    // chunks per tile
  static constexpr int NKB = KC / 32;   // 32-key blocks per chunk
  static constexpr int NDB = D / 32;    // 32-wide blocks of the head dim
  static constexpr int NKK = D / 16;    // K steps of the Q K^T product
  static constexpr int CHUNK = KC * D;  // elements of one staged operand
  static constexpr int BUF = 2 * CHUNK; // elements per buffer (K then V)
  static constexpr int NKB1 = CHUNK * 2 / 1024;       // 1 KB copies per operand
  // copying waves: the largest power of two up to NW (all waves for single
  // tiles and pairs; 8 of the 12 for triples of 128-row tiles)
  static constexpr int NCW = NW >= 16 ? 16 : NW >= 8 ? 8 : NW >= 4 ? 4 : NW >= 2 ? 2 : 1;
  static constexpr int NDMA = NKB1 / NCW;             // 1 KB copies per copying wave
  static_assert(NDMA >= 1 && NKB1 % NCW == 0, "chunk must split evenly");
};

template <int V>
struct FwdBuf {
  static constexpr int value = V;
};

// Query-tile group lists: tile-index mask and the shifts of a row's
// membership and partial bits (G = 1 reads the CSR rows, partial = bit 31).
template <int G>
struct GroupBits {
  static constexpr int32_t kTile = G == 3 ? kTriTile : G == 2 ? kPairTile : 0x7fffffff;
  static constexpr int kIn = G == 3 ? 25 : 27, kPart = G == 3 ? 28 : 29;
};

template <int D, int T, bool EXACT, int G>
__global__ __launch_bounds__(T / 32 * 64 * G, G > 1 ? 256 / (T / 32 * 64) : 2) void
radial_fwd_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                  const bf16 *__restrict__ V, bf16 *__restrict__ O, float *__restrict__ LSE,
                  const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
                  const int32_t *__restrict__ grp_ptr, const int32_t *__restrict__ grp_idx,
                  const int32_t *__restrict__ grp_tiles, int32_t n_grp, int32_t N, int32_t nb,
                  int32_t n_work, float scale_log2, MaskGeom mg) {
  using C = FwdCfg<D, T, G>;
  using GB = GroupBits<G>;
  constexpr float kSlack = 8.f;  // lazy-rescale threshold (log2 units)
  constexpr float kBound = 65536.f;  // probabilities accepted without a new max
  __shared__ __attribute__((aligned(1024))) bf16 lds[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g = lane >> 5;
  // work item: G query tiles (waves [k NWR, (k + 1) NWR) take tile k) over
  // the union of their key tiles, so every staged K/V chunk serves G times
  // the queries; pairs are tiles 2 p + k, triples the listed ones
  const int work = xcd_remap(blockIdx.x, n_work, RADIAL_FWD_XCD_BLOCK);
  const int bh = work / n_grp;
  const int wi = work - bh * n_grp;
  const int sub = G > 1 ? wave / C::NWR : 0;  // which tile of the group
  int u = G * wi + sub;
  if constexpr (G == 3) {
    u = grp_tiles[3 * wi + sub];
    if (u < 0) u = nb;  // no tile: the waves only help with the copies
  }
  const int64_t base = (int64_t)bh * N * D;
  const bf16 *Kb = K + base;
  const bf16 *Vb = V + base;

  const int qrow = u * T + (wave % C::NWR) * 32 + c32;
  const bool q_ok = u < nb && qrow < N;
  // token-exact: the mask's per-band table, read by the predicate from LDS
  __shared__ int lds_rtab[64];
  int rtab_v = 0;
  if constexpr (EXACT) rtab_v = tid < 64 ? mg.band_rtab[tid] : 0;
  bf16x8 qf[C::NKK];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk)
    qf[kk] = q_ok ? ld8(Q + base + (int64_t)qrow * D + kk * 16 + g * 8) : zero_bf16x8();

  // chunk list: every KC-key chunk of every listed key tile, minus the
  // chunks of the last key tile that lie entirely at or beyond N.  A list
  // entry is a key tile (CSR: bit 31 marks a partial tile; pair and triple
  // lists: membership and partial bits per tile of the group, see kernels.h).
  const int32_t *lptr = G > 1 ? grp_ptr : row_ptr;
  const int32_t *lidx = G > 1 ? grp_idx : col_idx;
  constexpr int32_t TMASK = GB::kTile;
  const int t_begin = lptr[wi], t_end = lptr[wi + 1];
  int nchunks = (t_end - t_begin) * C::CPT;
  if (t_end > t_begin && (lidx[t_end - 1] & TMASK) == nb - 1)
    nchunks -= C::CPT - (N - (nb - 1) * T + C::KC - 1) / C::KC;
  // list entry of chunk c: scalar loads, fetched one chunk ahead so their
  // wait lands where no LDS or vector-memory work is outstanding
  auto chunk_raw = [&](int c) { return lidx[t_begin + c / C::CPT]; };
  auto key_of = [&](int raw, int c) { return (raw & TMASK) * T + (c % C::CPT) * C::KC; };
  // this lane's query as (frame, position), for the token predicate
  // (computed where a partial chunk needs it, from the wave's scalar tile
  // and row offsets and the lane index, so nothing stays live across the
  // chunk loop: with triples every register is taken, and values kept live
  // there were spilled and reloaded inside the loop)
  const int qrow0 = u * T + (wave % C::NWR) * 32;  // wave-uniform

  // Chunk staging by direct global -> LDS copies (no staging registers):
  // copy jj of copying wave w (w < NCW) fills LDS bytes
  // [(w*NDMA + jj) * 1024, +1024) of an operand; lane l writes element
  // e = blk*512 + 8l, i.e. row e / D and physical 16-byte block (e % D) / 8,
  // which holds logical block physical ^ swz_f(row) of that row.  Lanes past
  // N write zeros.
  const bool copier = wave < C::NCW;
  int dma_off[C::NDMA];
#pragma unroll
  for (int jj = 0; jj < C::NDMA; ++jj) {
    const int e = ((wave % C::NCW) * C::NDMA + jj) * 512 + 8 * lane;
    const int row = e / D, pblk = (e % D) / 8;
    dma_off[jj] = row * D * 2 + 16 * (pblk ^ swz_f<D>(row));
  }
  auto issue_copy = [&](int buf, int k0) {
    if (!copier) return;
    // the resource covers this chunk's keys only (at most KC rows, so the
    // byte count stays small whatever N); keys at or past N read as zeros
    const int rows = N - k0 < C::KC ? N - k0 : C::KC;
    const int bytes = rows * D * 2;
    const auto rk = make_rsrc(Kb + (int64_t)k0 * D, bytes);
    const auto rv = make_rsrc(Vb + (int64_t)k0 * D, bytes);
    bf16 *kd = lds + buf * C::BUF;
#pragma unroll
    for (int jj = 0; jj < C::NDMA; ++jj) {
      const int blk = (wave * C::NDMA + jj) * 512;
      dma16(rk, kd + blk, dma_off[jj]);
      dma16(rv, kd + C::CHUNK + blk, dma_off[jj]);
    }
  };

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = zero16();
  float m_run = kNoMax;     // reference max of the log2-scaled logits
  float l_run = 0.f;        // this lane's share of the running sum

  int raw_next = nchunks > 0 ? chunk_raw(0) : 0;             // chunk c + 1
  int raw_after = nchunks > 1 ? chunk_raw(1) : 0;            // chunk c + 2
  if (nchunks > 0) issue_copy(0, key_of(raw_next, 0));
  wait_vmem();  // Q fragments and the first chunk
  if constexpr (EXACT) {
    if (tid < 64) lds_rtab[tid] = rtab_v;
  }
  __syncthreads();
  const BandCtx bctx = make_band_ctx(mg, lds_rtab);

  // Per-lane LDS offsets of the operand reads, the same for both buffers and
  // every 16-row step (the swizzle depends on the row modulo 16 only):
  //   kof[kk]: S product, key row c32, 16-byte column block 2 kk + g (ld8)
  //   vof[db][h]: the transposing V reads of column block db, rows r0 and
  //   r0 + 8 of a 16-row step; lane (g, c32) in lane group lg = lane / 16
  //   addresses row r0 = 4 (lg / 2) + j / 4 and columns 32 db + 16 (lg % 2) + 4 (j % 4),
  //   j = lane % 16
  // With the chunk loop unrolled over the two buffers, every read is one of
  // these registers plus an immediate offset.
  int kof[C::NKK], vof[C::NDB][2];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) kof[kk] = swz<D>(c32, 2 * kk + g);
  {
    const int j = lane & 15, lg = lane >> 4;
    const int r0 = 4 * (lg >> 1) + (j >> 2);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int col = db * 32 + 16 * (lg & 1) + 4 * (j & 3);
      vof[db][0] = swz<D>(r0, col >> 3) + (col & 7);
      vof[db][1] = swz<D>(r0 + 8, col >> 3) + (col & 7);
    }
  }

  // The tail chunk (keys key0 .. key0 + KC - 1 with key0 + KC > N, the
  // last chunk when KC does not divide N): its keys at or past N sit at
  // offsets N - key0 - 4 g and beyond from the lane's base key0 + 4 g, so
  // the mask words of the two lane halves are constants of the launch.
  const int tail_y = N - (N - 1) / C::KC * C::KC;
  const unsigned tail_ok0 = rank_mask<C::NKB>(tail_y), tail_ok1 = rank_mask<C::NKB>(tail_y - 4);

  // chunk c from buffer BS (0 or 1, = c % 2)
  auto chunk = [&](int c, auto BS) __attribute__((always_inline)) {
    constexpr int bsel = decltype(BS)::value;
    const bf16 *Ks = lds + bsel * C::BUF;
    const bf16 *Vs = Ks + C::KC * D;
    const int raw = raw_next;
    const int key0 = key_of(raw, c);
    // this wave's tile takes part in the chunk (always for single tiles)
    const bool member = G > 1 ? ((raw >> (GB::kIn + sub)) & 1) != 0 : true;
    const bool partial = EXACT && (G > 1 ? ((raw >> (GB::kPart + sub)) & 1) != 0 : raw < 0);
    raw_next = raw_after;
    // the next chunk's copy lands in the other buffer during these products
    if (c + 1 < nchunks) issue_copy(1 - bsel, key_of(raw_next, c + 1));
    if (c + 2 < nchunks) raw_after = chunk_raw(c + 2);

    if (member) {
      // S^T for the wave's 32 queries against the chunk's KC keys, the K
      // fragments read four products ahead (products in the order kk, kb);
      // two in token-exact mode, whose predicate needs registers of its own
      // (with four, triples spill inside the chunk loop there).  Keys outside
      // the query's runs get -inf in token-exact mode, and with MT keys at or
      // past N too (the tail chunk, see below).
      f32x16 s[C::NKB];
      const bool tail = key0 + C::KC > N;
      auto scores = [&](auto MT) __attribute__((always_inline)) {
        constexpr bool mask_tail = decltype(MT)::value;
        bf16x8 kf[C::NKB][C::NKK];
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
            kf[kb][kk] = ld8(Ks + kb * 32 * D + kof[kk]);
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) s[kb] = zero16();
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) s[kb] = mfma32(kf[kb][kk], qf[kk], s[kb]);
        read_ahead_order<1, EXACT ? 2 : 4, C::NKK * C::NKB, 1>();
        if constexpr (mask_tail) {
          if (tail) mask_elems(s, g ? tail_ok1 : tail_ok0);  // the tail chunk
        }
        if (partial) {
          const unsigned lid =
              __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
          const int qr = qrow0 + (int)(lid & 31u);  // this lane's query row
          const int qi = bctx.div_s(qr), qa = qr - qi * bctx.s;
          const unsigned ok = lane_key_bits<C::NKB>(bctx, qi, qa, key0, g);
          if (__ballot(ok != ~0u)) mask_elems(s, ok);  // some key of the wave's block is masked
        }
      };
      // P = 2^(scale_log2 S - m_run) rounded to bf16, and this lane's sum
      bf16x8 pf[C::NKB][2];
      float lc;
      auto probs = [&]() __attribute__((always_inline)) {
        float psum[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short add chains
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -m_run));
            psum[r & 3] += p;
            pf[kb][r >> 3][r & 7] = bf16(p);
          }
        }
        lc = (psum[0] + psum[1]) + (psum[2] + psum[3]);
        // the bf16 P is formed here, not after the branch below: sunk past
        // it, the fp32 probabilities stay live and the loop spills
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(pf[kb][h]));
      };
      // The reference max is checked through the sum, not a max over the
      // chunk: lc >= every probability of the lane, so lc <= kBound bounds
      // them all (and fails on inf or NaN).  Only when that fails, which is
      // every wave's first chunk (m_run starts at kNoMax) and rarely after
      // it, or in the tail chunk, the chunk is redone: S again (the
      // exponentials overwrote it), its row max, the lazy move of m_run and
      // the rescale of O and l, after which every probability is at most
      // 2^kSlack.  The first pass leaves the tail chunk's keys past N
      // unmasked (the redo discards its probabilities), so the common pass
      // has no branch between the products and the exponentials, and the
      // compiler schedules the two together.
      scores(FwdBuf<0>{});
      probs();
      if (__ballot(tail || !(lc <= kBound))) {
        scores(FwdBuf<1>{});
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const float m_new = pair_max(mx) * scale_log2;
        const bool mv = m_new > m_run + kSlack;
        const float alpha = mv ? fast_exp2(m_run - m_new) : 1.f;
        m_run = mv ? m_new : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        probs();
      }
      l_run += lc;

      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const bf16 *vs = Vs + (kb * 32 + ks * 16) * D;
            const bf16x4 lo = ld_tr(vs + vof[db][0]);
            const bf16x4 hi = ld_tr(vs + vof[db][1]);
            oacc[db] = mfma32(cat(lo, hi), pf[kb][ks], oacc[db]);
          }
        }
      }
      // transposing reads run four ahead of the products that consume them
      constexpr int NPV = C::NDB * C::NKB * 2;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
#pragma unroll
      for (int i = 0; i < NPV - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
    }  // member

    wait_vmem();      // this wave's copies of chunk c + 1 have landed
    __syncthreads();  // ... everyone's, and chunk c is no longer read
  };
  for (int c = 0; c < nchunks; c += 2) {
    chunk(c, FwdBuf<0>{});
    if (c + 1 < nchunks) chunk(c + 1, FwdBuf<1>{});
  }

  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  if (q_ok) {
    bf16 *orow = O + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 out;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) out[jj] = bf16(oacc[db][4 * i + jj] * inv);
        st4(orow + db * 32 + 8 * i + 4 * g, out);
      }
    }
    if (g == 0) LSE[(int64_t)bh * N + qrow] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, int T, bool EXACT, int G>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t stream) {
  const int32_t n_grp = G == 3 ? a.n_tri : (a.nb + G - 1) / G;
  const int64_t works = (int64_t)a.BH * n_grp;
  hipLaunchKernelGGL((radial_fwd_kernel<D, T, EXACT, G>), dim3((unsigned)works),
                     dim3(FwdCfg<D, T, G>::NT), 0, stream, (const bf16 *)a.q,
                     (const bf16 *)a.k, (const bf16 *)a.v, (bf16 *)a.o, a.lse, a.row_ptr,
                     a.col_idx, G == 3 ? a.tri_ptr : a.pair_ptr,
                     G == 3 ? a.tri_idx : a.pair_idx, a.tri_tiles, n_grp, a.N, a.nb,
                     (int32_t)works,
                     a.scale * kLog2e, a.mask);
  return hipGetLastError();
}

// Query tiles in triples, else in pairs, else single, as far as the layout
// has the group lists and max_group allows.
template <int D, int T, bool EXACT>
hipError_t launch_fwd_g(const FwdArgs &a, hipStream_t stream) {
  if (a.max_group >= 3 && a.tri_ptr && a.tri_tiles) return launch_fwd_t<D, T, EXACT, 3>(a, stream);
  if (a.max_group >= 2 && a.pair_ptr) return launch_fwd_t<D, T, EXACT, 2>(a, stream);
  return launch_fwd_t<D, T, EXACT, 1>(a, stream);
}

template <int D, int T>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t stream) {
  return a.mask.exact ? launch_fwd_g<D, T, true>(a, stream) : launch_fwd_g<D, T, false>(a, stream);
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
  if (a.D == 64 && a.T == 64) return launch_fwd_t<64, 64>(a, stream);
  if (a.D == 64 && a.T == 128) return launch_fwd_t<64, 128>(a, stream);
  if (a.D == 128 && a.T == 128) return launch_fwd_t<128, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace radial
