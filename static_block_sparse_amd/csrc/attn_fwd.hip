// Radial block-sparse attention forward on gfx950.
//
// One workgroup computes one query tile u (T rows) of one (batch, head):
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
//  * wave w owns queries [32w, 32w + 32) of the tile; its Q rows stay in
//    registers as the B operand of S^T = K Q^T.  Computing S transposed puts
//    one query per lane column: a row's max and sum need one exchange
//    between lanes l and l ^ 32 (v_permlane32_swap), and P feeds P V as the
//    B operand with no lane movement (see device_common.h).
//  * K and V chunks are staged row-major in LDS with an XOR swizzle of the
//    16-byte column blocks; the V^T operand is read with the gfx950
//    transposing LDS load (ds_read_b64_tr_b16).
//  * chunks are double buffered: the next chunk's global loads are issued
//    into registers at the start of a chunk and written to the other LDS
//    buffer after its products, so there is one barrier per chunk.
//  * the running max is only moved when a chunk's max exceeds it by more
//    than 8 (log2 units); probabilities then stay below 2^8, exact in the
//    final O / l and LSE, and the O rescale is skipped on most chunks.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace radial {

template <int D, int T>
struct FwdCfg {
  static constexpr int NW = T / 32;     // waves per workgroup
  static constexpr int NT = NW * 64;    // threads per workgroup
  static constexpr int KC = 64;         // keys per pipeline chunk
  static constexpr int CPT = T / KC;    // chunks per tile
  static constexpr int NKB = KC / 32;   // 32-key blocks per chunk
  static constexpr int NDB = D / 32;    // 32-wide blocks of the head dim
  static constexpr int NKK = D / 16;    // K steps of the Q K^T product
  static constexpr int NCH = D / 8;     // 16-byte blocks per row
  static constexpr int LPT = KC * NCH / NT;  // 16-byte loads per thread per operand
  static constexpr int BUF = 2 * KC * D;     // elements per buffer (K then V)
  static_assert(LPT >= 1 && KC * NCH % NT == 0, "chunk must split evenly");
};

template <int D, int T>
__global__ __launch_bounds__(T / 32 * 64, 2) void radial_fwd_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    bf16 *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, int32_t N, int32_t nb, int32_t n_work,
    float scale_log2) {
  using C = FwdCfg<D, T>;
  constexpr float kSlack = 8.f;  // lazy-rescale threshold (log2 units)
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  const int work = xcd_remap(blockIdx.x, n_work);
  const int bh = work / nb;
  const int u = work - bh * nb;
  const int64_t base = (int64_t)bh * N * D;
  const bf16 *Kb = K + base;
  const bf16 *Vb = V + base;

  const int qrow = u * T + wave * 32 + c32;
  const bool q_ok = qrow < N;
  bf16x8 qf[C::NKK];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk)
    qf[kk] = q_ok ? ld8(Q + base + (int64_t)qrow * D + kk * 16 + g * 8) : zero_bf16x8();

  // chunk list: every KC-key chunk of every kept tile, minus the chunks of
  // the last key tile that lie entirely at or beyond N
  const int t_begin = row_ptr[u], t_end = row_ptr[u + 1];
  int nchunks = (t_end - t_begin) * C::CPT;
  if (t_end > t_begin && col_idx[t_end - 1] == nb - 1)
    nchunks -= C::CPT - (N - (nb - 1) * T + C::KC - 1) / C::KC;
  // key tile of chunk c: scalar loads, fetched one chunk ahead so their
  // wait lands where no LDS or vector-memory work is outstanding
  auto chunk_key0 = [&](int c) {
    return col_idx[t_begin + c / C::CPT] * T + (c % C::CPT) * C::KC;
  };

  // chunk staging: thread `tid` moves the 16-byte blocks idx = tid + it * NT
  // (row idx / NCH, block idx % NCH); buffer loads past N read zeros
  bf16x8 pk[C::LPT], pv[C::LPT];
  auto load_chunk = [&](int k0) {
    const int bytes = (N - k0) * D * 2;
    const auto rk = make_rsrc(Kb + (int64_t)k0 * D, bytes);
    const auto rv = make_rsrc(Vb + (int64_t)k0 * D, bytes);
#pragma unroll
    for (int it = 0; it < C::LPT; ++it) {
      pk[it] = buf_ld8(rk, (tid + it * C::NT) * 16);
      pv[it] = buf_ld8(rv, (tid + it * C::NT) * 16);
    }
  };
  auto store_chunk = [&](int buf) {
    bf16 *kd = lds + buf * C::BUF;
    bf16 *vd = kd + C::KC * D;
#pragma unroll
    for (int it = 0; it < C::LPT; ++it) {
      const int idx = tid + it * C::NT;
      const int row = idx / C::NCH, ch = idx % C::NCH;
      st8(kd + swz<D>(row, ch), pk[it]);
      st8(vd + swz<D>(row, ch), pv[it]);
    }
  };

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = zero16();
  float m_run = -INFINITY;  // reference max of the log2-scaled logits
  float l_run = 0.f;        // this lane's share of the running sum

  int key_next = nchunks > 0 ? chunk_key0(0) : 0;            // chunk c + 1
  int key_after = nchunks > 1 ? chunk_key0(1) : 0;           // chunk c + 2
  if (nchunks > 0) {
    load_chunk(key_next);
    store_chunk(0);
  }
  // Q fragments have landed on every path into the loop, so no wait for
  // them is left inside it (vmcnt(0); expcnt and lgkmcnt at their maximum)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // lane (g, c32) in transposing-read group G = lane / 16 addresses row
  // n0 + j / 4 and columns d0 + 4 (j % 4), j = lane % 16
  const int j = lane & 15, G = lane >> 4;

  for (int c = 0; c < nchunks; ++c) {
    const bf16 *Ks = lds + (c & 1) * C::BUF;
    const bf16 *Vs = Ks + C::KC * D;
    const int key0 = key_next;
    key_next = key_after;
    // next chunk's global loads fly during this chunk's products
    if (c + 1 < nchunks) load_chunk(key_next);
    if (c + 2 < nchunks) key_after = chunk_key0(c + 2);

    // S^T for the wave's 32 queries against the chunk's KC keys
    f32x16 s[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      const int row = kb * 32 + c32;
      bf16x8 kf[C::NKK];
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) kf[kk] = ld8(Ks + swz<D>(row, 2 * kk + g));
      s[kb] = zero16();
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) s[kb] = mfma32(kf[kk], qf[kk], s[kb]);
    }
    if (key0 + C::KC > N) {  // the tail chunk: keys at or past N get -inf
      // register r of block kb holds key key0 + kb*32 + 8*(r/4) + 4g + r%4
      const int lim = N - key0 - 4 * g;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    const float m_new = pair_max(mx) * scale_log2;
    if (__ballot(m_new > m_run + kSlack)) {
      const bool mv = m_new > m_run + kSlack;
      const float alpha = mv ? fast_exp2(m_run - m_new) : 1.f;
      m_run = mv ? m_new : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }

    bf16x8 pf[C::NKB][2];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -m_run));
        l_run += p;
        pf[kb][r >> 3][r & 7] = bf16(p);
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int col = db * 32 + 16 * (G & 1) + 4 * (j & 3);
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int n0 = kb * 32 + ks * 16 + 4 * (G >> 1) + (j >> 2);
          const bf16x4 lo = ld_tr(Vs + swz<D>(n0, col >> 3) + (col & 7));
          const bf16x4 hi = ld_tr(Vs + swz<D>(n0 + 8, col >> 3) + (col & 7));
          oacc[db] = mfma32(cat(lo, hi), pf[kb][ks], oacc[db]);
        }
      }
    }

    if (c + 1 < nchunks) store_chunk((c + 1) & 1);
    __syncthreads();
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

template <int D, int T>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t stream) {
  const int64_t works = (int64_t)a.BH * a.nb;
  hipLaunchKernelGGL((radial_fwd_kernel<D, T>), dim3((unsigned)works), dim3(FwdCfg<D, T>::NT),
                     0, stream, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     (bf16 *)a.o, a.lse, a.row_ptr, a.col_idx, a.N, a.nb, (int32_t)works,
                     a.scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
  if (a.D == 64 && a.T == 64) return launch_fwd_t<64, 64>(a, stream);
  if (a.D == 128 && a.T == 128) return launch_fwd_t<128, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace radial
