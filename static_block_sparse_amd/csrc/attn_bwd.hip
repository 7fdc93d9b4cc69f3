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
//   1. pre:  Delta for every row                         (memory bound)
//   2. dkdv: one workgroup per key tile, walking its CSC column of query
//            tiles; dK and dV stay in registers for the whole walk
//   3. dq:   one workgroup per query tile, walking its CSR row of key tiles
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace radial {

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO * O) in fp32
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void radial_bwd_pre_kernel(const bf16 *__restrict__ O,
                                                             const bf16 *__restrict__ dO,
                                                             float *__restrict__ delta,
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
  if (row < rows && ch == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV: workgroup per (batch*head, key tile).  Wave w owns keys
//    [32w, 32w + 32) of the tile, with K and V rows held as B operands.
//    Query rows are staged MC at a time, row-major (A operand of S = Q K^T
//    and dP = dO V^T) and transposed (A operand of dK^T = Q^T dS and
//    dV^T = dO^T P).  S and dP come out with one key per lane column, so P
//    and dS feed the next products as B operands without lane exchange.
// ---------------------------------------------------------------------------
template <int D, int T, int MC>
struct DkdvCfg {
  static constexpr int NW = T / 32;
  static constexpr int NT = NW * 64;
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NMB = MC / 32;
  static constexpr int RS = D + 8;   // row-major stride (elements)
  static constexpr int TS = MC + 4;  // transposed stride (elements)
};

template <int D, int T, int MC>
__global__ __launch_bounds__(T / 32 * 64, 1) void radial_bwd_dkdv_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const float *__restrict__ LSE,
    const float *__restrict__ Delta, bf16 *__restrict__ dK, bf16 *__restrict__ dV,
    const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ row_idx,
    const int32_t *__restrict__ col_order, int32_t N, int32_t nb, int32_t n_work,
    float scale_log2, float scale) {
  using C = DkdvCfg<D, T, MC>;
  __shared__ __attribute__((aligned(16))) bf16 Qs[MC * C::RS];
  __shared__ __attribute__((aligned(16))) bf16 dOs[MC * C::RS];
  __shared__ __attribute__((aligned(16))) bf16 Qt[D * C::TS];
  __shared__ __attribute__((aligned(16))) bf16 dOt[D * C::TS];
  __shared__ __attribute__((aligned(16))) float lse_s[MC];
  __shared__ __attribute__((aligned(16))) float dl_s[MC];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  const int work = xcd_remap(blockIdx.x, n_work, 0);
  const int bh = work / nb;
  const int v = col_order[work - bh * nb];
  const int64_t base = (int64_t)bh * N * D;
  const int64_t rbase = (int64_t)bh * N;
  const bf16 *Qb = Q + base;
  const bf16 *dOb = dO + base;

  const int key = v * T + wave * 32 + c32;
  const bool k_ok = key < N;
  bf16x8 kf[C::NKK], vf[C::NKK];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
    kf[kk] = k_ok ? ld8(K + base + (int64_t)key * D + kk * 16 + g * 8) : zero_bf16x8();
    vf[kk] = k_ok ? ld8(V + base + (int64_t)key * D + kk * 16 + g * 8) : zero_bf16x8();
  }
  f32x16 adk[C::NDB], adv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    adk[db] = zero16();
    adv[db] = zero16();
  }

  const int t_begin = col_ptr[v], t_end = col_ptr[v + 1];
  for (int t = t_begin; t < t_end; ++t) {
    const int u = row_idx[t];
#pragma unroll 1
    for (int c = 0; c < T / MC; ++c) {
      const int m0 = u * T + c * MC;
      const int valid = N - m0;
      if (valid <= 0) break;
      __syncthreads();
      load_rows<MC, D, C::RS, C::NT>(Qs, Qb + (int64_t)m0 * D, valid, tid);
      load_rows<MC, D, C::RS, C::NT>(dOs, dOb + (int64_t)m0 * D, valid, tid);
      load_rows_t<MC, D, C::TS, C::NT>(Qt, Qb + (int64_t)m0 * D, valid, tid);
      load_rows_t<MC, D, C::TS, C::NT>(dOt, dOb + (int64_t)m0 * D, valid, tid);
      if (tid < MC) {
        lse_s[tid] = tid < valid ? LSE[rbase + m0 + tid] * kLog2e : INFINITY;
        dl_s[tid] = tid < valid ? Delta[rbase + m0 + tid] : 0.f;
      }
      __syncthreads();

#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
          s = mfma32(ld8(&Qs[(mb * 32 + c32) * C::RS + kk * 16 + g * 8]), kf[kk], s);
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
          dp = mfma32(ld8(&dOs[(mb * 32 + c32) * C::RS + kk * 16 + g * 8]), vf[kk], dp);

        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lse_s[mb * 32 + 8 * i + 4 * g]);
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&dl_s[mb * 32 + 8 * i + 4 * g]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * i + j;
            const float p = fast_exp2(s[r] * scale_log2 - l4[j]);
            const float ds = p * (dp[r] - d4[j]);
            pb[r >> 3][r & 7] = bf16(p);
            dsb[r >> 3][r & 7] = bf16(ds);
          }
        }
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int off = (db * 32 + c32) * C::TS + mb * 32 + ks * 16 + 4 * g;
            adv[db] = mfma32(ld_perm(&dOt[off]), pb[ks], adv[db]);
            adk[db] = mfma32(ld_perm(&Qt[off]), dsb[ks], adk[db]);
          }
        }
      }
    }
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
        for (int j = 0; j < 4; ++j) {
          ok4[j] = bf16(adk[db][4 * i + j] * scale);
          ov4[j] = bf16(adv[db][4 * i + j]);
        }
        st4(dkrow + db * 32 + 8 * i + 4 * g, ok4);
        st4(dvrow + db * 32 + 8 * i + 4 * g, ov4);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: workgroup per (batch*head, query tile).  Wave w owns queries
//    [32w, 32w + 32), with Q and dO rows held as B operands.  Key tiles are
//    staged KC keys at a time: K and V row-major (A operands of S^T = K Q^T
//    and dP^T = V dO^T) and K transposed (A operand of dQ^T = K^T dS^T).
// ---------------------------------------------------------------------------
template <int D, int T, int KC>
struct DqCfg {
  static constexpr int NW = T / 32;
  static constexpr int NT = NW * 64;
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NKB = KC / 32;
  static constexpr int RS = D + 8;
  static constexpr int TS = KC + 4;
};

template <int D, int T, int KC>
__global__ __launch_bounds__(T / 32 * 64, 2) void radial_bwd_dq_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const float *__restrict__ LSE,
    const float *__restrict__ Delta, bf16 *__restrict__ dQ,
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx, int32_t N,
    int32_t nb, int32_t n_work, float scale_log2, float scale) {
  using C = DqCfg<D, T, KC>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[KC * C::RS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[KC * C::RS];
  __shared__ __attribute__((aligned(16))) bf16 Kt[D * C::TS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  const int work = xcd_remap(blockIdx.x, n_work, 0);
  const int bh = work / nb;
  const int u = work - bh * nb;
  const int64_t base = (int64_t)bh * N * D;
  const bf16 *Kb = K + base;
  const bf16 *Vb = V + base;

  const int qrow = u * T + wave * 32 + c32;
  const bool q_ok = qrow < N;
  bf16x8 qf[C::NKK], dof[C::NKK];
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
    qf[kk] = q_ok ? ld8(Q + base + (int64_t)qrow * D + kk * 16 + g * 8) : zero_bf16x8();
    dof[kk] = q_ok ? ld8(dO + base + (int64_t)qrow * D + kk * 16 + g * 8) : zero_bf16x8();
  }
  const float lse2 = q_ok ? LSE[(int64_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dl = q_ok ? Delta[(int64_t)bh * N + qrow] : 0.f;

  f32x16 adq[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) adq[db] = zero16();

  const int t_begin = row_ptr[u], t_end = row_ptr[u + 1];
  for (int t = t_begin; t < t_end; ++t) {
    const int k0 = col_idx[t] * T;
#pragma unroll 1
    for (int c = 0; c < T / KC; ++c) {
      const int kc0 = k0 + c * KC;
      const int valid = N - kc0;
      if (valid <= 0) break;
      __syncthreads();
      load_rows<KC, D, C::RS, C::NT>(Ks, Kb + (int64_t)kc0 * D, valid, tid);
      load_rows<KC, D, C::RS, C::NT>(Vs, Vb + (int64_t)kc0 * D, valid, tid);
      load_rows_t<KC, D, C::TS, C::NT>(Kt, Kb + (int64_t)kc0 * D, valid, tid);
      __syncthreads();

#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
          s = mfma32(ld8(&Ks[(kb * 32 + c32) * C::RS + kk * 16 + g * 8]), qf[kk], s);
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
          dp = mfma32(ld8(&Vs[(kb * 32 + c32) * C::RS + kk * 16 + g * 8]), dof[kk], dp);
        bf16x8 dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          const float p = kr < valid ? fast_exp2(s[r] * scale_log2 - lse2) : 0.f;
          dsb[r >> 3][r & 7] = bf16(p * (dp[r] - dl));
        }
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            adq[db] = mfma32(ld_perm(&Kt[(db * 32 + c32) * C::TS + kb * 32 + ks * 16 + 4 * g]),
                             dsb[ks], adq[db]);
        }
      }
    }
  }

  if (q_ok) {
    bf16 *row = dQ + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 o4;
#pragma unroll
        for (int j = 0; j < 4; ++j) o4[j] = bf16(adq[db][4 * i + j] * scale);
        st4(row + db * 32 + 8 * i + 4 * g, o4);
      }
    }
  }
}

template <int D, int T>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
  constexpr int MC = 64, KC = 64;
  const int64_t rows = (int64_t)a.BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((radial_bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                     dim3(256), 0, stream, (const bf16 *)a.o, (const bf16 *)a.dout, a.delta,
                     rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t works = (int64_t)a.BH * a.nb;
  const float sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((radial_bwd_dkdv_kernel<D, T, MC>), dim3((unsigned)works),
                     dim3(DkdvCfg<D, T, MC>::NT), 0, stream, (const bf16 *)a.q,
                     (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.lse, a.delta,
                     (bf16 *)a.dk, (bf16 *)a.dv, a.col_ptr, a.row_idx, a.col_order, a.N, a.nb,
                     (int32_t)works, sl2, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((radial_bwd_dq_kernel<D, T, KC>), dim3((unsigned)works),
                     dim3(DqCfg<D, T, KC>::NT), 0, stream, (const bf16 *)a.q, (const bf16 *)a.k,
                     (const bf16 *)a.v, (const bf16 *)a.dout, a.lse, a.delta, (bf16 *)a.dq,
                     a.row_ptr, a.col_idx, a.N, a.nb, (int32_t)works, sl2, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
  if (a.D == 64 && a.T == 64) return launch_bwd_t<64, 64>(a, stream);
  if (a.D == 128 && a.T == 128) return launch_bwd_t<128, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace radial
