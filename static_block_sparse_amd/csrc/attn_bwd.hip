// Radial block-sparse attention backward on gfx950.
//
// Gradients of O = softmax(scale * Q K^T + M) V (jaehun.me review "Radial
// Attention: O(n log n) Sparse Attention with Energy Decay for Long Video
// Generation", Prompt 1.3.1 Step 0; paper §3 Eq.1-2) for the radial mask's
// kept tiles (Step 5; paper §4.2).  With P recomputed from the forward's
// LSE, P = exp(scale * S - LSE):
//   Delta = rowsum(dO * O)
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta)
//   dK = scale * dS^T Q,  dQ = scale * dS K
// Three launches on one stream, no atomics (deterministic):
//   1. pre:  -Delta and -LSE log2(e) for every row       (memory bound)
//   2. dkdv: one workgroup per key tile, walking its CSC column of query
//            tiles; dK and dV stay in registers for the whole walk
//   3. dq:   one workgroup per query tile, walking its CSR row of key tiles
// The product kernels start each dP accumulation from -Delta, so the
// products give dP - Delta, and take the exponent's row term ready-made.
// Both product kernels stage 64-row chunks with direct global -> LDS copies
// (row-major, XOR-swizzled; rows past N read as zeros, which contribute
// exactly zero to every product here) and read transposed operands with the
// gfx950 transposing LDS load, so each operand is staged once.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "kernels.h"

#ifndef RADIAL_DQ_PAIR
#define RADIAL_DQ_PAIR 1  // dQ over pairs of query tiles sharing K/V chunks
#endif
#ifndef RADIAL_BWD_XCD_BLOCK
#define RADIAL_BWD_XCD_BLOCK 16  // tiles per XCD block (see xcd_remap)
#endif

namespace radial {

// ---------------------------------------------------------------------------
// 1. -Delta = -rowsum(dO * O) in fp32, and the exponent's row term
//    -LSE log2(e) (P = exp2(scale log2(e) S - LSE log2(e)))
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void radial_bwd_pre_kernel(const bf16 *__restrict__ O,
                                                             const bf16 *__restrict__ dO,
                                                             const float *__restrict__ lse,
                                                             float *__restrict__ ndelta,
                                                             float *__restrict__ nlse2,
                                                             int64_t rows) {
  constexpr int CH = D / 8;       // threads per row, 8 elements each
  constexpr int RPB = 256 / CH;   // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / CH;
  const int ch = tid % CH;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = ld8(O + row * D + ch * 8);
    const bf16x8 b = ld8(dO + row * D + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += float(a[e]) * float(b[e]);
  }
#pragma unroll
  for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && ch == 0) {
    ndelta[row] = -acc;
    nlse2[row] = -lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: workgroup per (batch*head, key tile).  Wave w owns keys
//    [32w, 32w + 32) of the tile, with K and V rows held as B operands.
//    Query rows arrive in chunks of MC = 64 (Q, dO, LSE, Delta) in four LDS
//    buffers.  Each 32-query block j goes through three stages:
//      1. S = Q K^T and dP = dO V^T        (matrix cores; Q, dO row-major)
//      2. P = exp(scale S - LSE), dS = P (dP - Delta)   (vector ALU)
//      3. dV^T += dO^T P, dK^T += Q^T dS   (matrix cores; dO^T, Q^T read
//                                           with transposing loads)
//    S and dP come out with one key per lane column, so P and dS feed stage 3
//    as B operands without lane exchange.  The stages are software pipelined:
//    step j runs stage 3 of block j - 2, stage 2 of block j - 1 and stage 1
//    of block j in one basic block, so the vector work of one block overlaps
//    the products of two others within the wave (one wave per SIMD here).
//    Step pairs form a chunk iteration c, which reads chunks c and c - 1 while
//    the copies of chunk c + 2 are in flight.
// ---------------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16 with its result and accumulator in vector
// registers and B in accumulation registers, written out so that one kernel
// can mix this form with the compiler's accumulation-register form (the
// compiler picks one form per function).  Callers keep its hazards: the
// result is read by vector instructions only several products later, and a
// chain of these on one accumulator alternates with another chain.
__device__ __forceinline__ f32x16 mfma_v(bf16x8 a, bf16x8 b, f32x16 c) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
  return c;
}
__device__ __forceinline__ f32x16 mfma_v0(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  return d;
}

template <int D, int T>
struct DkdvCfg {
  static constexpr int NW = T / 32;
  static constexpr int NT = NW * 64;
  static constexpr int MC = 64;          // query rows per chunk
  static constexpr int CPT = T / MC;     // chunks per query tile
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NBUF = 4;         // chunk buffers
  static constexpr int CHUNK = MC * D;   // elements of one staged operand
  using Copier = TileCopier<D, MC, NW>;
  static constexpr int NCOPY = 2 * Copier::NDMA + 2;  // copies per wave per chunk
  static_assert(NCOPY < 16, "copy counts");
};

template <int V>
struct BwdFlag {
  static constexpr int value = V;
};

// v = -inf unless bit `bit` (a constant after unrolling) of ok is set: the
// bit sign-extended is a bit-select mask, two vector instructions and no
// compare (a compare and select per element cost three, in every chunk of a
// token-exact dK/dV walk, full tiles included)
__device__ __forceinline__ float mask_bit(float v, unsigned ok, int bit) {
  int m;
  asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(ok), "i"(bit));
  asm("v_bfi_b32 %0, %1, %0, %2" : "+v"(v) : "v"(m), "v"(-INFINITY));
  return v;
}

template <int D, int T, bool EXACT>
__global__ __launch_bounds__(T / 32 * 64, 1) void radial_bwd_dkdv_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const float *__restrict__ NLse2,
    const float *__restrict__ NDelta, bf16 *__restrict__ dK, bf16 *__restrict__ dV,
    const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ row_idx,
    const int32_t *__restrict__ col_order, int32_t N, int32_t nb, int32_t n_work,
    float scale_log2, float scale, MaskGeom mg) {
  using C = DkdvCfg<D, T>;
  constexpr int NB = C::NBUF;
  // Q and dO chunk buffers in two arrays of NB * CHUNK elements (64 KB each
  // at D = 128), so every LDS read is a per-lane register plus an immediate
  // offset (below 64 KB) whatever the buffer
  __shared__ __attribute__((aligned(1024))) bf16 lds_q[NB * C::CHUNK];
  __shared__ __attribute__((aligned(1024))) bf16 lds_do[NB * C::CHUNK];
  __shared__ __attribute__((aligned(16))) float lds_r[NB * 2 * C::MC];
  // per buffer: first query row of its chunk, bit 31 set when the chunk's
  // tile is marked partial (token-exact layouts)
  __shared__ int lds_meta[NB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g = lane >> 5;
  const int work = xcd_remap(blockIdx.x, n_work, RADIAL_BWD_XCD_BLOCK);
  const int bh = work / nb;
  const int v = col_order[work - bh * nb];
  const int64_t base = (int64_t)bh * N * D;
  const int64_t rbase = (int64_t)bh * N;
  const bf16 *Qb = Q + base;
  const bf16 *dOb = dO + base;

  const int key = v * T + wave * 32 + c32;
  const bool k_ok = key < N;
  // this lane's key as (frame, position), for the token predicate
  const int kj = key / mg.s, kpos = key - (key / mg.s) * mg.s;
  // token-exact: the mask's per-band table, read by the predicate from LDS
  __shared__ int lds_rtab[64];
  int rtab_v = 0;
  if constexpr (EXACT) rtab_v = tid < 64 ? mg.band_rtab[tid] : 0;
  const BandCtx bctx = make_band_ctx(mg, lds_rtab);
  bf16x8 kf[C::NKK], vf[C::NKK];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
    kf[kk] = k_ok ? ld8(K + base + (int64_t)key * D + kk * 16 + g * 8) : zero_bf16x8();
    vf[kk] = k_ok ? ld8(V + base + (int64_t)key * D + kk * 16 + g * 8) : zero_bf16x8();
    // K and V are only ever MFMA operands: keep them in accumulation
    // registers, leaving the vector registers to the pipeline stages
    asm volatile("" : "+a"(kf[kk]), "+a"(vf[kk]));
  }
  f32x16 adk[C::NDB], adv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    adk[db] = zero16();
    adv[db] = zero16();
  }

  // chunk list: every MC-row chunk of every query tile of the column, minus
  // the chunks of the last query tile at or past N
  const int t_begin = col_ptr[v], t_end = col_ptr[v + 1];
  int nch = (t_end - t_begin) * C::CPT;
  if (t_end > t_begin && (row_idx[t_end - 1] & 0x7fffffff) == nb - 1)
    nch -= C::CPT - (N - (nb - 1) * T + C::MC - 1) / C::MC;
  // first query row of chunk c with bit 31 set when its tile is partial
  auto code_of = [&](int raw, int c) __attribute__((always_inline)) {
    return ((raw & 0x7fffffff) * T + (c % C::CPT) * C::MC) | (raw & int(0x80000000));
  };
  auto row0_of = [&](int c) __attribute__((always_inline)) {
    return code_of(row_idx[t_begin + c / C::CPT], c);
  };
  // the query tile of chunk c (clamped to the column), a raw scalar load
  auto tile_of = [&](int c) __attribute__((always_inline)) {
    return row_idx[t_begin + (c < nch ? c : nch - 1) / C::CPT];
  };

  typename C::Copier cp;
  cp.init(wave, lane);
  // Copies of chunk c (first row m0) into buffer c % NB, issued from inline
  // assembly (see dma16_async), so every wait below is explicit.  Half 0 is
  // Q and the LSE terms, half 1 dO and the Delta terms; each half is
  // NDMA + 1 pieces per wave: piece 0 the MC row terms (every wave copies
  // all of them, 4 bytes a lane, the same values to the same LDS words, so
  // no lane mask is needed), pieces 1 .. NDMA the wave's share of the rows.
  // The pieces are spread over a pipeline step's product slots.
  static_assert(C::MC == 64, "row terms: one 4-byte copy per lane");
  constexpr int NPIECE = C::Copier::NDMA + 1;
  auto copy_piece = [&](int buf, int code, int half, int k) __attribute__((always_inline)) {
    const int m0 = code & 0x7fffffff;
    // the resources cover this chunk's rows only (at most MC, so the byte
    // counts stay small whatever N); rows at or past N read as zeros
    const int rows = N - m0 < C::MC ? N - m0 : C::MC;
    if (k == 0) {
      const u32x4 rl = rsrc_words((half ? NDelta : NLse2) + rbase + m0, rows * 4);
      dma4_async(rl, lds_r + buf * 2 * C::MC + half * C::MC, 4 * lane);
    } else {
      const u32x4 rq = rsrc_words((half ? dOb : Qb) + (int64_t)m0 * D, rows * D * 2);
      const int jj = k - 1;
      dma16_async(rq, (half ? lds_do : lds_q) + buf * C::CHUNK + (wave * C::Copier::NDMA + jj) * 512,
                  cp.off[jj]);
    }
  };
  auto meta = [&](int buf, int code) __attribute__((always_inline)) {
    if (EXACT && tid == 0) lds_meta[buf] = code;
  };
  auto issue = [&](int c, int code) __attribute__((always_inline)) {
    meta(c % NB, code);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int k = 0; k < NPIECE; ++k) copy_piece(c % NB, code, half, k);
  };

  // Per-lane LDS offsets of the operand reads, the same for every chunk
  // buffer, block half and k step: the swizzle term of a row depends on the
  // row modulo 16 only, and blocks start at multiples of 16 rows.
  //   soff[kk]: stage 1, row c32, 16-byte column block 2 kk + g (ld8)
  //   toff[db][h]: stage 3, the transposing reads for column block db
  //                (lane (g, c32) in group G = lane / 16 addresses row
  //                r0 + 8 h, r0 = 4 (G / 2) + j / 4, and columns
  //                32 db + 16 (G % 2) + 4 (j % 4), j = lane % 16)
  int soff[C::NKK], toff[C::NDB][2];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) soff[kk] = swz<D>(c32, 2 * kk + g);
  {
    const int j = lane & 15, G = lane >> 4;
    const int r0 = 4 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int col = db * 32 + 16 * (G & 1) + 4 * (j & 3);
      toff[db][0] = swz<D>(r0, col >> 3) + (col & 7);
      toff[db][1] = swz<D>(r0 + 8, col >> 3) + (col & 7);
    }
  }

  // stage-1 results of a block: sd[0] = S, sd[1] = dP (register r holds
  // query row 32 mb + 8 (r / 4) + 4 g + r % 4 of the chunk, for key column
  // c32)
  struct Blk {
    f32x16 sd[2];
  };

  // Step j: stage 3 of block j - 2 (chunk buffer b3, half m3), stage 2 of
  // block j - 1 (b2, m2), stage 1 of block j (b1, m1), as flagged.  The step
  // is written as an explicit schedule of product slots (stage 3's and stage
  // 1's products, see pid): slot i issues the LDS reads of slot i + RA, its own
  // product and, from slot 4 on, a share of stage 2's elements (whose LSE
  // terms are read in slot 0; the -Delta terms that start stage 1's dP are
  // read in slot 1, or 0 without stage 3); a scheduling barrier after each slot
  // keeps that order.  With one wave per SIMD, LDS latency is hidden only by
  // this read-ahead and the vector work only by this interleaving.
  // The first RA operands of a step with stage 3 are carried in `pre`: the
  // step before reads them in its last slots (flag FN, with the next step's
  // stage-3 buffer b3n and half m3n), and the step takes them from there
  // (flag FP), so no step starts by waiting for LDS.  Those operands belong
  // to a chunk that landed at least one barrier earlier and whose buffer is
  // refilled two barriers later.
  constexpr int RA = 8;                                 // read-ahead (slots)
  auto step = [&](auto F1, auto F2, auto F3, auto FP, auto FN, int b1, int m1, int b2, int m2,
                  int b3, int m3, int b3n, int m3n, bf16x8 (&pre)[RA], Blk &sd_new,
                  const Blk &sd_old, bf16x8 (&pd_new)[2][2], const bf16x8 (&pd_old)[2][2],
                  unsigned okm, auto NCPc, auto &&cpy) __attribute__((always_inline)) {
    constexpr bool s1 = decltype(F1)::value, s2 = decltype(F2)::value,
                   s3 = decltype(F3)::value;
    constexpr bool from_pre = decltype(FP)::value, to_pre = decltype(FN)::value;
    constexpr int NM = 4 * C::NDB;                      // products per stage
    constexpr int N3 = s3 ? NM : 0, NSL = N3 + (s1 ? NM : 0);
    static_assert(!from_pre || N3 >= RA, "carried operands are stage-3 operands");
    const bf16 *Qs3 = lds_q + b3 * C::CHUNK, *dOs3 = lds_do + b3 * C::CHUNK;
    const bf16 *Qs1 = lds_q + b1 * C::CHUNK, *dOs1 = lds_do + b1 * C::CHUNK;
    const float *rt2 = lds_r + b2 * 2 * C::MC + 32 * m2;           // -LSE log2(e), stage 2
    const float *rt1 = lds_r + b1 * 2 * C::MC + C::MC + 32 * m1;   // -Delta, stage 1
    // operand of slot i (lane offsets precomputed; the block's row offset is
    // a constant).  Stage 3 slot i: k step ks = i / (2 NDB), dV (w = 0) or
    // dK (w = 1) by (i / NDB) % 2, column block db = i % NDB, so runs of NDB
    // consecutive products share their P or dS operand (less switching).
    // Stage 1 slot: (kk, S or dP).
    auto frag = [&](int i) __attribute__((always_inline)) {
      if (i < N3) {
        const int db = i % C::NDB, ks = i / (2 * C::NDB), w = (i / C::NDB) % 2;
        const bf16 *t = (w ? Qs3 : dOs3) + (m3 * 32 + ks * 16) * D;
        return cat(ld_tr(t + toff[db][0]), ld_tr(t + toff[db][1]));
      }
      const int kk = (i - N3) / 2;
      return ld8((((i - N3) % 2) ? dOs1 : Qs1) + m1 * 32 * D + soff[kk]);
    };
    // stage-3 operand i < RA of the next step
    auto frag_next = [&](int i) __attribute__((always_inline)) {
      const int db = i % C::NDB, ks = i / (2 * C::NDB), w = (i / C::NDB) % 2;
      const bf16 *t = (w ? lds_q : lds_do) + b3n * C::CHUNK + (m3n * 32 + ks * 16) * D;
      return cat(ld_tr(t + toff[db][0]), ld_tr(t + toff[db][1]));
    };
    auto product = [&](int i, bf16x8 a) __attribute__((always_inline)) {
      if (i < N3) {
        const int db = i % C::NDB, ks = i / (2 * C::NDB), w = (i / C::NDB) % 2;
        if (w == 0)
          adv[db] = mfma32(a, pd_old[0][ks], adv[db]);
        else
          adk[db] = mfma32(a, pd_old[1][ks], adk[db]);
      } else {
        // S starts from zero, dP from -Delta (read into it earlier), so
        // stage 2 gets dP - Delta without a subtraction
        const int kk = (i - N3) / 2, w = (i - N3) % 2;
        sd_new.sd[w] = (kk == 0 && w == 0) ? mfma_v0(a, kf[kk])
                                           : mfma_v(a, w ? vf[kk] : kf[kk], sd_new.sd[w]);
      }
    };
    f32x4 rt[4];  // stage 2's -LSE log2(e) terms
    auto rt_read = [&](int q) __attribute__((always_inline)) {
      rt[q] = *reinterpret_cast<const f32x4 *>(&rt2[8 * q + 4 * g]);
    };
    // stage 1's -Delta terms, straight into the dP accumulator (register r
    // holds row 8 (r / 4) + 4 g + r % 4, as the terms' layout)
    auto nd_read = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 t = *reinterpret_cast<const f32x4 *>(&rt1[8 * q + 4 * g]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sd_new.sd[1][4 * q + jj] = t[jj];
      }
    };
    // stage 2, element pair e (rows r = 2e, 2e + 1 of the block)
    auto stage2_pair = [&](int e) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = 2 * e + t, i = r / 4, jj = r % 4;
        float sv = sd_old.sd[0][r];
        // token-exact: okm holds the stage-2 block's allowed rows (bit r)
        if constexpr (EXACT) sv = mask_bit(sv, okm, r);
        const float p = fast_exp2(fmaf(sv, scale_log2, rt[i][jj]));
        pd_new[0][r >> 3][r & 7] = bf16(p);
        pd_new[1][r >> 3][r & 7] = bf16(p * sd_old.sd[1][r]);
      }
    };
    // stage 2 runs alongside stage 3's products when there are any (so the
    // old S, dP die before stage 1 produces the new ones), else stage 1's
    constexpr int S0 = 4;                                  // first stage-2 slot
    constexpr int SEND = N3 > 0 ? N3 : NSL;                // slots [S0, SEND) carry it
    constexpr int SPAN = SEND > S0 ? SEND - S0 : 1;
    // product of slot i: with both stages, the first RA slots take stage
    // 3's first products (their operands may come from the step before),
    // then each of stage 3's remaining NR products follows K1 of stage 1's,
    // so consecutive products of stage 1's two accumulation chains (S and
    // dP) sit K1 + 1 slots apart instead of two (D = 128: K1 = 2, 1% faster;
    // D = 64 has no stage-3 product past the first RA and keeps the order)
    constexpr int NR = N3 - RA;
    constexpr bool ILV = s1 && s3 && NR > 0;
    constexpr int K1 = ILV ? (NSL - N3) / NR : 1;
    static_assert(!ILV || (NSL - N3) % NR == 0, "slot interleave");
    auto pid = [&](int i) __attribute__((always_inline)) {
      if (!ILV || i < RA) return i;
      const int j = i - RA, grp = j / (K1 + 1), r = j % (K1 + 1);
      return r < K1 ? N3 + K1 * grp + r : RA + grp;
    };
    bf16x8 fr[NSL > 0 ? NSL : 1];
#pragma unroll
    for (int i = 0; i < RA && i < NSL; ++i) fr[i] = from_pre ? pre[i] : frag(pid(i));
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      if constexpr (s2) {
        if (i == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) rt_read(q);
        }
      }
      // the -Delta terms land before the first dP product (slot N3 + 1)
      if constexpr (s1) {
        if (i == (N3 > 0 ? 1 : 0)) nd_read();
      }
      if (i + RA < NSL)
        fr[i + RA] = frag(pid(i + RA));
      else if constexpr (to_pre)
        pre[i + RA - NSL] = frag_next(i + RA - NSL);
      product(pid(i), fr[i]);
      // copy pieces cpy(0 .. NCP - 1), evenly spread over the slots
      if constexpr (decltype(NCPc)::value > 0) {
        constexpr int NCP = decltype(NCPc)::value, ST = NSL / (NCP + 1);
        if (i % ST == ST - 1 && i / ST < NCP) cpy(i / ST);
      }
      if constexpr (s2) {
        // pairs [e0, e1) go with slot i
        if (i >= S0 && i < SEND) {
          const int e0 = (i - S0) * 8 / SPAN, e1 = (i - S0 + 1) * 8 / SPAN;
#pragma unroll
          for (int e = e0; e < e1; ++e) stage2_pair(e);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (s2 && SEND <= S0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) rt_read(q);
#pragma unroll
      for (int e = 0; e < 8; ++e) stage2_pair(e);
    }
    // keeps stage 2 in this block (otherwise it may be sunk past the chunk
    // end's branches, away from the products it overlaps with)
    if constexpr (s2)
      asm volatile("" ::"v"(pd_new[0][0]), "v"(pd_new[0][1]), "v"(pd_new[1][0]),
                   "v"(pd_new[1][1]));
  };

  Blk sdA, sdB;                     // stage-1 results of even / odd blocks
  bf16x8 pdA[2][2], pdB[2][2];      // stage-2 results of even / odd blocks
  const BwdFlag<0> NO;
  const BwdFlag<1> YES;
  // token-exact: this lane's allowed rows of block (buffer b, half m), read
  // between steps (outside their fixed schedule); all rows when the block's
  // tile is full
  auto s2_bits = [&](int b, int m) __attribute__((always_inline)) {
    if constexpr (!EXACT) {
      return ~0u;
    } else {
      const int meta = lds_meta[b];
      if (meta >= 0) return ~0u;
      return lane_query_bits(bctx, kj, kpos, (meta & 0x7fffffff) + 32 * m, g);
    }
  };

  int row_a = nch > 0 ? row0_of(0) : 0;  // first rows of chunks c + 1, c + 2
  int row_b = nch > 1 ? row0_of(1) : 0;
  if (nch > 0) issue(0, row_a);
  if (nch > 1) {
    issue(1, row_b);
    wait_vmem_n<C::NCOPY>();
  } else {
    wait_vmem();
  }
  if constexpr (EXACT) {
    if (tid < 64) lds_rtab[tid] = rtab_v;
  }
  __syncthreads();
  int row_c = nch > 2 ? row0_of(2) : 0;

  // end of chunk iteration c: chunk c + 1 landed and visible (c + 2 may be
  // in flight); the buffer of chunk c - 1 is free afterwards
  auto chunk_end = [&](int c) __attribute__((always_inline)) {
    if (c + 2 < nch)
      wait_vmem_n<C::NCOPY>();
    else
      wait_vmem();
    __syncthreads();
  };

  bf16x8 pre[RA];  // first operands of the next step
  const BwdFlag<0> NOCOPY;
  const BwdFlag<NPIECE> PIECES;
  auto no_copy = [](int) {};
  if (nch > 0) {
    // chunk iteration 0: steps 0 and 1
    if (nch > 2) issue(2, row_c);
    // (every later step has stage 3; the next one's reads buffer 0, half 0)
    step(YES, NO, NO, NO, NO, 0, 0, 0, 0, 0, 0, 0, 0, pre, sdA, sdB, pdB, pdA, ~0u, NOCOPY,
         no_copy);
    step(YES, YES, NO, NO, YES, 0, 1, 0, 0, 0, 0, 0, 0, pre, sdB, sdA, pdA, pdB, s2_bits(0, 0),
         NOCOPY, no_copy);
    // The query tile of the chunk after next is loaded here, after the
    // step's last LDS read and unused until the next iteration: scalar loads
    // return out of order with LDS reads, so while one is in flight every
    // LDS wait would have to drain everything.
    int tile_d = tile_of(3);
    chunk_end(0);
    // chunk iterations 1 .. nch - 1: steps 2c and 2c + 1; the copies of
    // chunk c + 2 go out one half per step, their pieces spread over the
    // step's product slots (a burst queues at the CU's address unit and
    // stalls instruction issue)
    // In the last two iterations (no chunk c + 2) the copies still go out,
    // unconditionally so that no branch splits a step: they copy the last
    // chunk again into buffer (c + 2) % NB, whose chunk c - 2 is done and
    // which nothing reads afterwards.
    // The loop is unrolled over the NB buffers, so every buffer index is a
    // constant and every LDS access a per-lane register plus an immediate.
    static_assert(NB == 4, "unrolled over four buffers");
    auto iteration = [&](int c, auto BC) __attribute__((always_inline)) {
      constexpr int bc = decltype(BC)::value, bp = (bc + NB - 1) % NB, bn = (bc + 2) % NB;
      const bool more = c + 2 < nch;
      const int row_e = code_of(tile_d, more ? c + 2 : nch - 1);
      if (more) meta(bn, row_e);
      auto copy_q = [&](int k) __attribute__((always_inline)) { copy_piece(bn, row_e, 0, k); };
      auto copy_do = [&](int k) __attribute__((always_inline)) { copy_piece(bn, row_e, 1, k); };
      step(YES, YES, YES, YES, YES, bc, 0, bp, 1, bp, 0, bp, 1, pre, sdA, sdB, pdB, pdA,
           s2_bits(bp, 1), PIECES, copy_q);
      step(YES, YES, YES, YES, YES, bc, 1, bc, 0, bp, 1, bc, 0, pre, sdB, sdA, pdA, pdB,
           s2_bits(bc, 0), PIECES, copy_do);
      tile_d = tile_of(c + 3);
      chunk_end(c);
    };
    for (int c = 1; c < nch; c += NB) {
      iteration(c, BwdFlag<1>{});
      if (c + 1 < nch) iteration(c + 1, BwdFlag<2>{});
      if (c + 2 < nch) iteration(c + 2, BwdFlag<3>{});
      if (c + 3 < nch) iteration(c + 3, BwdFlag<0>{});
    }
    // drain: steps 2 nch, 2 nch + 1 (chunk nch - 1)
    const int bl = (nch - 1) % NB;
    step(NO, YES, YES, YES, YES, 0, 0, bl, 1, bl, 0, bl, 1, pre, sdA, sdB, pdB, pdA,
         s2_bits(bl, 1), NOCOPY, no_copy);
    step(NO, NO, YES, YES, NO, 0, 0, 0, 0, bl, 1, 0, 0, pre, sdB, sdA, pdA, pdB, ~0u, NOCOPY,
         no_copy);
  }

  if (k_ok) {
    bf16 *dkrow = dK + base + (int64_t)key * D;
    bf16 *dvrow = dV + base + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 ok4, ov4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          ok4[jj] = bf16(adk[db][4 * i + jj] * scale);
          ov4[jj] = bf16(adv[db][4 * i + jj]);
        }
        st4(dkrow + db * 32 + 8 * i + 4 * g, ok4);
        st4(dvrow + db * 32 + 8 * i + 4 * g, ov4);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: workgroup per (batch*head, query tile).  Wave w owns queries
//    [32w, 32w + 32), with Q and dO rows held as B operands and the lane's
//    LSE and Delta in registers.  Key chunks of KC rows (K, V) are double
//    buffered: S^T = K Q^T and dP^T = V dO^T read K and V row-major, and
//    dQ^T += K^T dS^T reads K^T with transposing loads.
// ---------------------------------------------------------------------------
template <int D, int T, bool PAIR>
struct DqCfg {
  static constexpr int NWR = T / 32;                // waves per query tile
  static constexpr int NW = NWR * (PAIR ? 2 : 1);   // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int KC = 64;
  static constexpr int CPT = T / KC;
  static constexpr int NKB = KC / 32;
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int CHUNK = KC * D;
  using Copier = TileCopier<D, KC, NW>;
};

template <int D, int T, bool EXACT, bool PAIR>
__global__ __launch_bounds__(T / 32 * 64 * (PAIR ? 2 : 1),
                             PAIR ? 256 / (T / 32 * 64) : 2) void radial_bwd_dq_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const float *__restrict__ NLse2,
    const float *__restrict__ NDelta, bf16 *__restrict__ dQ,
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const int32_t *__restrict__ pair_ptr, const int32_t *__restrict__ pair_idx, int32_t N,
    int32_t nb, int32_t n_work, float scale_log2, float scale, MaskGeom mg) {
  using C = DqCfg<D, T, PAIR>;
  __shared__ __attribute__((aligned(1024))) bf16 lds[4 * C::CHUNK];  // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g = lane >> 5;
  // work item: one query tile, or with PAIR the query tiles 2p (waves
  // [0, NWR)) and 2p + 1 over the union of their key tiles, so every staged
  // K/V chunk serves twice the queries (as in the forward pass)
  const int nwork_head = PAIR ? (nb + 1) / 2 : nb;
  const int work = xcd_remap(blockIdx.x, n_work, RADIAL_BWD_XCD_BLOCK);
  const int bh = work / nwork_head;
  const int wi = work - bh * nwork_head;
  const int sub = PAIR ? wave / C::NWR : 0;
  const int u = PAIR ? 2 * wi + sub : wi;
  const int64_t base = (int64_t)bh * N * D;
  const bf16 *Kb = K + base;
  const bf16 *Vb = V + base;

  const int qrow = u * T + (wave % C::NWR) * 32 + c32;
  const bool q_ok = u < nb && qrow < N;
  bf16x8 qf[C::NKK], dof[C::NKK];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
    qf[kk] = q_ok ? ld8(Q + base + (int64_t)qrow * D + kk * 16 + g * 8) : zero_bf16x8();
    dof[kk] = q_ok ? ld8(dO + base + (int64_t)qrow * D + kk * 16 + g * 8) : zero_bf16x8();
  }
  // rows past N: Q, dO are zero and the row terms are taken as 0, so dS = 0
  const float nl2 = q_ok ? NLse2[(int64_t)bh * N + qrow] : 0.f;   // -LSE log2(e)
  const float ndl = q_ok ? NDelta[(int64_t)bh * N + qrow] : 0.f;  // -Delta

  f32x16 adq[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) adq[db] = zero16();

  // chunk list over the CSR row or the pair list (entries as in the forward)
  const int32_t *lptr = PAIR ? pair_ptr : row_ptr;
  const int32_t *lidx = PAIR ? pair_idx : col_idx;
  constexpr int32_t TMASK = PAIR ? kPairTile : 0x7fffffff;
  const int t_begin = lptr[wi], t_end = lptr[wi + 1];
  int nch = (t_end - t_begin) * C::CPT;
  if (t_end > t_begin && (lidx[t_end - 1] & TMASK) == nb - 1)
    nch -= C::CPT - (N - (nb - 1) * T + C::KC - 1) / C::KC;
  auto chunk_raw = [&](int c) { return lidx[t_begin + c / C::CPT]; };
  auto key_of = [&](int raw, int c) { return (raw & TMASK) * T + (c % C::CPT) * C::KC; };
  // this lane's query as (frame, position), for the token predicate
  const int qi = qrow / mg.s, qa = qrow - (qrow / mg.s) * mg.s;
  // token-exact: the mask's per-band table, read by the predicate from LDS
  __shared__ int lds_rtab[64];
  int rtab_v = 0;
  if constexpr (EXACT) rtab_v = threadIdx.x < 64 ? mg.band_rtab[threadIdx.x] : 0;

  // Copies issued from inline assembly (copy_async): the compiler adds no
  // wait of its own before the transposing K reads, which it cannot prove
  // disjoint from the other buffer; the waits are the explicit ones below.
  typename C::Copier cp;
  cp.init(wave, lane);
  auto issue = [&](int buf, int k0) {
    bf16 *kd = lds + buf * 2 * C::CHUNK;
    cp.copy_async(kd, Kb + (int64_t)k0 * D, N - k0, wave);
    cp.copy_async(kd + C::CHUNK, Vb + (int64_t)k0 * D, N - k0, wave);
  };

  // Per-lane LDS offsets, the same for both buffers and every 16-row step
  // (the swizzle depends on the row modulo 16 only):
  //   kof[kk]: S and dP products, key row c32, 16-byte block 2 kk + g
  //   tof[db][h]: transposing K reads of column block db, rows r0 + 8 h
  // With the chunk loop unrolled over the two buffers, every LDS read is one
  // of these registers plus an immediate offset.
  int kof[C::NKK], tof[C::NDB][2];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) kof[kk] = swz<D>(c32, 2 * kk + g);
  {
    const int j = lane & 15, G = lane >> 4;
    const int r0 = 4 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int col = db * 32 + 16 * (G & 1) + 4 * (j & 3);
      tof[db][0] = swz<D>(r0, col >> 3) + (col & 7);
      tof[db][1] = swz<D>(r0 + 8, col >> 3) + (col & 7);
    }
  }

  int raw_n = nch > 0 ? chunk_raw(0) : 0;   // list entries of chunks c and c + 1
  int raw_nn = nch > 1 ? chunk_raw(1) : 0;
  if (nch > 0) issue(0, key_of(raw_n, 0));
  wait_vmem();  // Q, dO fragments, LSE, Delta and the first chunk
  if constexpr (EXACT) {
    if (threadIdx.x < 64) lds_rtab[threadIdx.x] = rtab_v;
  }
  __syncthreads();
  const BandCtx bctx = make_band_ctx(mg, lds_rtab);

  // chunk c from buffer BS (= c % 2)
  auto chunk = [&](int c, auto BS) __attribute__((always_inline)) {
    constexpr int bsel = decltype(BS)::value;
    const int key0 = key_of(raw_n, c);
    // this wave's tile takes part in the chunk (always without PAIR)
    const bool member = PAIR ? ((raw_n >> (27 + sub)) & 1) != 0 : true;
    const bool partial = EXACT && (PAIR ? ((raw_n >> (29 + sub)) & 1) != 0 : raw_n < 0);
    if (c + 1 < nch) issue(1 - bsel, key_of(raw_nn, c + 1));  // lands during this chunk
    const int raw_3 = c + 2 < nch ? chunk_raw(c + 2) : 0;
    const bf16 *Ks = lds + bsel * 2 * C::CHUNK;
    const bf16 *Vs = Ks + C::CHUNK;

    if (member) {
      // token-exact: this lane's allowed keys of the chunk
      const unsigned ok =
          partial ? lane_key_bits<C::NKB>(bctx, qi, qa, key0, g) : ~0u;
      const bool masked = partial && __ballot(ok != ~0u);  // some key of the block is masked

#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        bf16x8 ka[C::NKK], va[C::NKK];
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
          ka[kk] = ld8(Ks + kb * 32 * D + kof[kk]);
          va[kk] = ld8(Vs + kb * 32 * D + kof[kk]);
        }
        // dP starts from -Delta, so the products give dP - Delta directly
        f32x16 s = zero16(), dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = ndl;
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
          s = mfma32(ka[kk], qf[kk], s);
          dp = mfma32(va[kk], dof[kk], dp);
        }
        // reads run four operands ahead of the products (left to itself the
        // compiler issues each read right before its product and waits)
        if (kb == 0)
          read_ahead_order<1, 4, 2 * C::NKK, 1>();
        else
          read_ahead_order<3, 4, 2 * C::NKK, 1>();
        // register r holds key kb*32 + 8*(r/4) + 4g + r%4 of the chunk
        if (masked) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = mask_bit(s[r], ok, 16 * kb + r);
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[r], scale_log2, nl2));
          dsb[r >> 3][r & 7] = bf16(p * dp[r]);
        }
        // consecutive products share their dS operand (less switching); two
        // operands (four transposing reads) ahead
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            adq[db] = mfma32(cat(ld_tr(Ks + (kb * 32 + ks * 16) * D + tof[db][0]),
                                 ld_tr(Ks + (kb * 32 + ks * 16) * D + tof[db][1])),
                             dsb[ks], adq[db]);
        if (kb == 0)
          read_ahead_order<2, 4, 2 * C::NDB, 2>();
        else
          read_ahead_order<4, 4, 2 * C::NDB, 2>();
      }
    }  // member

    wait_vmem();      // chunk c + 1 has landed here ...
    __syncthreads();  // ... and everywhere; chunk c is no longer read
    raw_n = raw_nn;
    raw_nn = raw_3;
  };
  for (int c = 0; c < nch; c += 2) {
    chunk(c, BwdFlag<0>{});
    if (c + 1 < nch) chunk(c + 1, BwdFlag<1>{});
  }

  if (q_ok) {
    bf16 *row = dQ + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 o4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o4[jj] = bf16(adq[db][4 * i + jj] * scale);
        st4(row + db * 32 + 8 * i + 4 * g, o4);
      }
    }
  }
}

template <int D, int T, bool EXACT, bool PAIR>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((radial_bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                     dim3(256), 0, stream, (const bf16 *)a.o, (const bf16 *)a.dout, a.lse,
                     a.ndelta, a.nlse2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t works = (int64_t)a.BH * a.nb;
  const float sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((radial_bwd_dkdv_kernel<D, T, EXACT>), dim3((unsigned)works),
                     dim3(DkdvCfg<D, T>::NT), 0, stream, (const bf16 *)a.q, (const bf16 *)a.k,
                     (const bf16 *)a.v, (const bf16 *)a.dout, a.nlse2, a.ndelta, (bf16 *)a.dk,
                     (bf16 *)a.dv, a.col_ptr, a.row_idx, a.col_order, a.N, a.nb, (int32_t)works,
                     sl2, a.scale, a.mask);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t dq_works = (int64_t)a.BH * (PAIR ? (a.nb + 1) / 2 : a.nb);
  hipLaunchKernelGGL((radial_bwd_dq_kernel<D, T, EXACT, PAIR>), dim3((unsigned)dq_works),
                     dim3(DqCfg<D, T, PAIR>::NT), 0, stream, (const bf16 *)a.q,
                     (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.nlse2,
                     a.ndelta, (bf16 *)a.dq, a.row_ptr, a.col_idx, a.pair_ptr, a.pair_idx, a.N,
                     a.nb, (int32_t)dq_works, sl2, a.scale, a.mask);
  return hipGetLastError();
}

template <int D, int T>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
  if (RADIAL_DQ_PAIR && a.pair_ptr)
    return a.mask.exact ? launch_bwd_t<D, T, true, true>(a, stream)
                        : launch_bwd_t<D, T, false, true>(a, stream);
  return a.mask.exact ? launch_bwd_t<D, T, true, false>(a, stream)
                      : launch_bwd_t<D, T, false, false>(a, stream);
}

// Static scratch for the allocation-free backward entry point: the two
// fp32 row arrays (-Delta, -LSE log2(e)) that radial_attn_bwd keeps in its
// caller's workspace.  Each device holds its own copy at its own address;
// host code uses only the addresses bwd_scratch looks up (the array's name
// is a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

hipError_t bwd_scratch(int device, void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  if (!ptr || device < 0 || device >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
  if (a.D == 64 && a.T == 64) return launch_bwd_t<64, 64>(a, stream);
  if (a.D == 64 && a.T == 128) return launch_bwd_t<64, 128>(a, stream);
  if (a.D == 128 && a.T == 128) return launch_bwd_t<128, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace radial
