// Radial block-sparse attention forward on gfx950.
//
// One workgroup computes one query tile u (T rows) of one (batch, head):
//   for each kept key tile v of row u (CSR, ascending):
//     S^T = K_v Q_u^T                (bf16 MFMA, fp32 accumulate)
//     online softmax over keys       (running max and sum per query, fp32)
//     O^T += V_v^T P^T               (P rounded to bf16)
//   O = O / l,  LSE = m + ln l.
// This is masked softmax attention (jaehun.me review "Radial Attention:
// O(n log n) Sparse Attention with Energy Decay for Long Video Generation",
// Prompt 1.3.1 Step 0; paper §3 Eq.1-2) evaluated tile by tile over the
// kept tiles of the radial mask (Step 5; paper §4.2), with keys >= N masked.
//
// Wave w owns queries [32w, 32w + 32) of the tile.  Computing S transposed
// puts one query per lane column, so each lane's registers hold 16 keys of
// its query per 32-key block: the row max and row sum need only one
// exchange between lanes l and l ^ 32, and the probabilities feed the P V
// product as the B operand directly (see device_common.h).  K is staged in
// LDS row-major (A operand, contiguous along D); V is staged transposed
// (A operand of V^T, contiguous along keys).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace radial {

template <int D, int T>
struct FwdCfg {
  static constexpr int NW = T / 32;   // waves per workgroup
  static constexpr int NT = NW * 64;  // threads per workgroup
  static constexpr int NKB = T / 32;  // 32-key blocks per tile
  static constexpr int NDB = D / 32;  // 32-wide blocks of the head dim
  static constexpr int NKK = D / 16;  // K steps of the Q K^T product
  static constexpr int KS = D + 8;    // LDS row stride of K (elements)
  static constexpr int VS = T + 4;    // LDS row stride of V^T (elements)
};

template <int D, int T>
__global__ __launch_bounds__(T / 32 * 64, 2) void radial_fwd_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    bf16 *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, int32_t N, int32_t nb, int32_t n_work,
    float scale_log2) {
  using C = FwdCfg<D, T>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[T * C::KS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * C::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  const int work = xcd_remap(blockIdx.x, n_work);
  const int bh = work / nb;
  const int u = work - bh * nb;
  const int64_t base = (int64_t)bh * N * D;
  const bf16 *Qb = Q + base;
  const bf16 *Kb = K + base;
  const bf16 *Vb = V + base;

  const int qrow = u * T + wave * 32 + c32;
  const bool q_ok = qrow < N;

  bf16x8 qf[C::NKK];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk)
    qf[kk] = q_ok ? ld8(Qb + (int64_t)qrow * D + kk * 16 + g * 8) : zero_bf16x8();

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = zero16();
  float m_run = -INFINITY;  // running max of the log2-scaled logits
  float l_run = 0.f;        // this lane's share of the running sum

  const int t_begin = row_ptr[u], t_end = row_ptr[u + 1];
  for (int t = t_begin; t < t_end; ++t) {
    const int k0 = col_idx[t] * T;
    const int valid = N - k0;  // keys of this tile below N (>= 1)
    // every wave has finished the previous tile's reads of Ks and Vt
    __syncthreads();
    load_rows<T, D, C::KS, C::NT>(Ks, Kb + (int64_t)k0 * D, valid, tid);
    __syncthreads();

    // S^T for the wave's 32 queries against all T keys
    f32x16 s[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk)
        s[kb] = mfma32(ld8(&Ks[(kb * 32 + c32) * C::KS + kk * 16 + g * 8]), qf[kk], s[kb]);
    }

    // V^T is staged after the S product so that its staging registers do
    // not overlap the K staging ones
    load_rows_t<T, D, C::VS, C::NT>(Vt, Vb + (int64_t)k0 * D, valid, tid);

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const float x = key < valid ? s[kb][r] * scale_log2 : -INFINITY;
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    bf16x8 pf[C::NKB][2];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[kb][r] - m_new);
        psum += p;
        pf[kb][r >> 3][r & 7] = bf16(p);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    __syncthreads();  // Vt complete
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = ld_perm(&Vt[(db * 32 + c32) * C::VS + kb * 32 + ks * 16 + 4 * g]);
          oacc[db] = mfma32(a, pf[kb][ks], oacc[db]);
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (q_ok) {
    bf16 *orow = O + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 out;
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = bf16(oacc[db][4 * i + j] * inv);
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
