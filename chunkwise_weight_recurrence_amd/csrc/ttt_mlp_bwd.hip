// Outer backward of the two-layer fast net (TTT-MLP) forward in ttt_mlp.hip, on
// the tile GEMM of tile_gemm.h.  The Modular TTT summary page ("Method step
// details", Algorithm 1) fixes the forward it differentiates; "Technical
// novelty" credits hand-written backward operators over autograd.

#include <type_traits>

#include "tile_gemm.h"
#include "ttt_device.h"
#include "ttt_internal.h"
#include "ttt_mlp_common.h"

namespace ttt {
namespace {

// ---------------------------------------------------------------------------
// Outer backward: the reverse chunk sweep.  For the outer loss
// <dO, O> + <dW1_T, W1_T> + <dW2_T, W2_T>, chunk i (from the last to the first)
// recomputes its forward from the checkpoints W1_i, W2_i and differentiates its
// steps in reverse order, carrying dW1_{i+1}, dW2_{i+1} (written D1, D2 below):
//   dS2 = -Tril(dO (eta G2)^T);  d(eta G2) = -S2^T dO - A D2
//   dX1 = (dO W2^T + dS2 A) (.) f'(X1);  dA = dS2^T A_q - (eta G2) D2^T
//   dS1 = -Tril(dX1 (eta G1)^T);  dQ = dX1 W1^T + dS1 K
//   d(eta G1) = -S1^T dX1 - K D1;  dG1 = eta d(eta G1);  dP = dG1 (.) f'(Z1)
//   dZ1 = dG1 (.) P (.) f''(Z1) + (dA + dV_hat W2^T) (.) f'(Z1)
//   dG2 = eta d(eta G2) + dP W2;  dV_hat = dG2 (MSE, else 0);  dV = -dG2 (MSE, IP) or 0 (L1)
//   dK = dS1^T Q - (eta G1) D1^T + dZ1 W1^T
//   dW1_i = g D1 + Q^T dX1 + K^T dZ1;  dW2_i = g D2 + A_q^T dO + dP^T G2 + A^T dV_hat
//   d eta_t = <d(eta G1)_t, G1_t> + <d(eta G2)_t, G2_t>;  d beta = d eta eta (1 - eta / 2)
//   d gamma += <D1, W1_i> + <D2, W2_i>
// with P = G2 W2^T and G1 = P (.) f'(Z1) as in the forward.  Every product is a
// GEMM of the same tile machinery; the chunk's intermediates live in the
// workspace.
// ---------------------------------------------------------------------------

struct MlpBwdScratch {
  int64_t dw1[2], dw2[2], q, k, v, dout, z1, a, x1, aq, p, gh1, dx1, dgh1, da, dp, dz1, g2, gh2, dgh2, dg2, dkp,
      s1, s2, ds, total;
  __host__ __device__ MlpBwdScratch(int C, int dk, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t ch = static_cast<int64_t>(C) * dh, cv = static_cast<int64_t>(C) * dv,
                  ckk = static_cast<int64_t>(C) * dk, cc = static_cast<int64_t>(C) * C;
    dw1[0] = take(static_cast<int64_t>(dk) * dh);
    dw1[1] = take(static_cast<int64_t>(dk) * dh);
    dw2[0] = take(static_cast<int64_t>(dh) * dv);
    dw2[1] = take(static_cast<int64_t>(dh) * dv);
    q = take(ckk);
    k = take(ckk);
    v = take(cv);
    dout = take(cv);
    z1 = take(ch);
    a = take(ch);
    x1 = take(ch);
    aq = take(ch);
    p = take(ch);
    gh1 = take(ch);
    dx1 = take(ch);
    dgh1 = take(ch);
    da = take(ch);
    dp = take(ch);
    dz1 = take(ch);
    g2 = take(cv);
    gh2 = take(cv);
    dgh2 = take(cv);
    dg2 = take(cv);
    dkp = take(ckk);
    s1 = take(cc);
    s2 = take(cc);
    ds = take(cc);
    total = o;
  }
};

struct MlpBwdArgs {
  int B, H, T, dk, dh, dv, C, NC, decay;
  float b;
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* gamma;
  const float* w1_ckpt;
  const float* w2_ckpt;
  const float* saved;  // the forward's MlpSaved per (chain, chunk), or null: recompute
  const void* d_o;
  const float* d_w1final;
  const float* d_w2final;
  void* dq;
  void* dk_out;
  void* dv_out;
  float* dbeta;
  float* dgamma;
  float* dw1_0;
  float* dw2_0;
  float* scratch;
};

template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void mlp_bwd_kernel(MlpBwdArgs a) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  __shared__ float eta[256];
  __shared__ float rinv[256];  // RMSE: 1 / (sqrt(d_v) ||V_hat - V||) per token of the chunk
  __shared__ float wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x;
  const int dk = a.dk, dh = a.dh, dv = a.dv, C = a.C;
  const MlpBwdScratch L(C, dk, dh, dv);
  float* sc = a.scratch + static_cast<int64_t>(bh) * L.total;
  float* Qc = sc + L.q;
  float* Kc = sc + L.k;
  float* Vc = sc + L.v;
  float* dOc = sc + L.dout;
  float* const Z1_ws = sc + L.z1;
  float* const Ac_ws = sc + L.a;
  float* const X1_ws = sc + L.x1;
  float* const Aq_ws = sc + L.aq;
  float* const P_ws = sc + L.p;
  float* const Gh1_ws = sc + L.gh1;
  float* dX1 = sc + L.dx1;
  float* dGh1 = sc + L.dgh1;
  float* dA = sc + L.da;
  float* dP = sc + L.dp;
  float* dZ1 = sc + L.dz1;
  float* const G2_ws = sc + L.g2;
  float* const Gh2_ws = sc + L.gh2;
  float* dGh2 = sc + L.dgh2;
  float* dG2 = sc + L.dg2;
  float* dKp = sc + L.dkp;
  float* const S1_ws = sc + L.s1;
  float* const S2_ws = sc + L.s2;
  float* dS = sc + L.ds;
  const bool scalar_decay = a.decay == TTT_DECAY_SCALAR;
  const float g = scalar_decay ? a.gamma[bh % a.H] : 1.0f;

  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk;
  const int64_t off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  const T* dO = static_cast<const T*>(a.d_o) + off_v;
  T* dq = static_cast<T*>(a.dq) + off_k;
  T* dkk = static_cast<T*>(a.dk_out) + off_k;
  T* dvv = static_cast<T*>(a.dv_out) + off_v;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  float* dbeta = a.dbeta + static_cast<int64_t>(bh) * a.T;
  const int64_t n1 = static_cast<int64_t>(dk) * dh, n2 = static_cast<int64_t>(dh) * dv;

  {  // dW_T: the final states' gradients (zero when not given)
    float* D1 = sc + L.dw1[0];
    float* D2 = sc + L.dw2[0];
    const float* s1 = a.d_w1final ? a.d_w1final + bh * n1 : nullptr;
    const float* s2 = a.d_w2final ? a.d_w2final + bh * n2 : nullptr;
    for (int64_t i = tid; i < n1; i += kThreads) D1[i] = s1 ? s1[i] : 0.0f;
    for (int64_t i = tid; i < n2; i += kThreads) D2[i] = s2 ? s2[i] : 0.0f;
  }
  int cur = 0;
  float dgam = 0.0f;  // this thread's share of d gamma, summed in a fixed order
  __syncthreads();

  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int t0 = ci * C;
    const int c = min(C, a.T - t0);
    const int64_t ck = static_cast<int64_t>(bh) * a.NC + ci;
    const float* W1 = a.w1_ckpt + ck * n1;
    const float* W2 = a.w2_ckpt + ck * n2;
    const float* D1 = sc + (cur ? L.dw1[1] : L.dw1[0]);  // dW1_{i+1}
    const float* D2 = sc + (cur ? L.dw2[1] : L.dw2[0]);
    float* D1o = sc + (cur ? L.dw1[0] : L.dw1[1]);  // dW1_i (written)
    float* D2o = sc + (cur ? L.dw2[0] : L.dw2[1]);

    // The chunk's forward intermediates: recomputed into the workspace, or read from the
    // forward's saved context.
    float *Z1 = Z1_ws, *Ac = Ac_ws, *X1 = X1_ws, *Aq = Aq_ws, *P = P_ws, *Gh1 = Gh1_ws, *G2 = G2_ws, *Gh2 = Gh2_ws,
          *S1 = S1_ws, *S2 = S2_ws;
    const bool have = a.saved != nullptr;
    if (have) {
      const MlpSaved SV(C, dh, dv);
      float* sb = const_cast<float*>(a.saved) + ck * SV.per_chunk;
      Z1 = sb + SV.z1; Ac = sb + SV.a; X1 = sb + SV.x1; Aq = sb + SV.aq; P = sb + SV.p; Gh1 = sb + SV.gh1;
      G2 = sb + SV.g2; Gh2 = sb + SV.gh2; S1 = sb + SV.s1; S2 = sb + SV.s2;
      if (LOSS == 3)
        for (int t = tid; t < c; t += kThreads) rinv[t] = sb[SV.ri + t];
    }
    stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
    if (!have) stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
    stage_rows<E>(dOc, dO + static_cast<int64_t>(t0) * dv, c * dv);
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    if (scalar_decay) {
      for (int64_t i = tid; i < n1; i += kThreads) dgam = fmaf(D1[i], W1[i], dgam);
      for (int64_t i = tid; i < n2; i += kThreads) dgam = fmaf(D2[i], W2[i], dgam);
    }
    __syncthreads();

    if (!have) {  // ---- the chunk's forward again ----
      gemm1<0, 0>(c, dh, Term{Kc, dk, W1, dh, dk, 1.0f}, kNoAux, lds, [&](int m, int n, float x, float, float, float) {
        Z1[m * dh + n] = x;
        Ac[m * dh + n] = act_f<ACT>(x);
      });
      if constexpr (LOSS == 1) {
        for (int i = tid; i < c * dv; i += kThreads) {
          G2[i] = -Vc[i];
          Gh2[i] = -eta[i / dv] * Vc[i];
        }
      }
      __syncthreads();
      if constexpr (LOSS != 1) {
        gemm1<0, 0>(c, dv, Term{Ac, dh, W2, dv, dh, 1.0f}, Aux{{Vc, nullptr, nullptr}, dv}, lds,
                    [&](int m, int n, float x, float vv, float, float) {
                      const float e = loss_signal<(LOSS == 3 ? 0 : LOSS), 0>(x, vv);
                      G2[m * dv + n] = e;
                      Gh2[m * dv + n] = eta[m] * e;
                    });
        __syncthreads();
      }
      if constexpr (LOSS == 3) {  // RMSE: scale e to the signal, keep 1 / (sqrt(d_v) ||e||)
        for (int t = wv; t < c; t += kThreads / 64) {
          float ss = 0.0f;
          for (int j = lane; j < dv; j += 64) ss = fmaf(G2[t * dv + j], G2[t * dv + j], ss);
          ss = wave_sum(ss);
          const float ri = ss > 0.0f ? rsqrtf(ss * dv) : 0.0f;
          for (int j = lane; j < dv; j += 64) {
            const float e = G2[t * dv + j] * ri;
            G2[t * dv + j] = e;
            Gh2[t * dv + j] = eta[t] * e;
          }
          if (lane == 0) rinv[t] = ri;
        }
        __syncthreads();
      }
      gemm1<0, 1>(c, dh, Term{G2, dv, W2, dv, dv, 1.0f}, Aux{{Z1, nullptr, nullptr}, dh}, lds,
                  [&](int m, int n, float x, float z, float, float) {
                    P[m * dh + n] = x;
                    Gh1[m * dh + n] = eta[m] * x * act_df<ACT>(z);
                  });
      gemm1<0, 1, true>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                        [&](int m, int n, float x, float, float, float) { S1[m * C + n] = (n <= m) ? x : 0.0f; });
      zero_upper_tiles(S1, c, C);
      __syncthreads();
      gemm<0, 0, 0, 0, false, true>(c, dh, Term{Qc, dk, W1, dh, dk, 1.0f}, Term{S1, C, Gh1, dh, c, -1.0f}, kNoAux,
                                    lds, [&](int m, int n, float x, float, float, float) {
                                      X1[m * dh + n] = x;
                                      Aq[m * dh + n] = act_f<ACT>(x);
                                    });
      __syncthreads();
      gemm1<0, 1, true>(c, c, Term{Aq, dh, Ac, dh, dh, 1.0f}, kNoAux, lds,
                        [&](int m, int n, float x, float, float, float) { S2[m * C + n] = (n <= m) ? x : 0.0f; });
      zero_upper_tiles(S2, c, C);
      __syncthreads();
    }

    // ---- its backward ----
    gemm1<0, 1, true>(c, c, Term{dOc, dv, Gh2, dv, dv, -1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(dS, c, C);
    gemm<1, 0, 0, 0>(c, dv, Term{S2, C, dOc, dv, c, -1.0f}, Term{Ac, dh, D2, dv, dh, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dGh2[m * dv + n] = x; });
    __syncthreads();
    gemm<0, 1, 0, 0, false, true>(c, dh, Term{dOc, dv, W2, dv, dv, 1.0f}, Term{dS, C, Ac, dh, c, 1.0f},
                                  Aux{{X1, nullptr, nullptr}, dh}, lds,
                                  [&](int m, int n, float x, float x1, float, float) {
                                    dX1[m * dh + n] = x * act_df<ACT>(x1);
                                  });
    gemm<1, 0, 0, 1>(c, dh, Term{dS, C, Aq, dh, c, 1.0f}, Term{Gh2, dv, D2, dv, dv, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dA[m * dh + n] = x; });
    __syncthreads();
    gemm1<0, 1, true>(c, c, Term{dX1, dh, Gh1, dh, dh, -1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(dS, c, C);
    __syncthreads();
    gemm<0, 1, 0, 0, false, true>(c, dk, Term{dX1, dh, W1, dh, dh, 1.0f}, Term{dS, C, Kc, dk, c, 1.0f}, kNoAux, lds,
                                  [&](int m, int n, float x, float, float, float) {
                                    E::st(dq, static_cast<int64_t>(t0 + m) * dk + n, x);
                                  });
    gemm<1, 0, 0, 0>(c, dh, Term{S1, C, dX1, dh, c, -1.0f}, Term{Kc, dk, D1, dh, dk, -1.0f},
                     Aux{{P, Z1, nullptr}, dh}, lds, [&](int m, int n, float x, float pp, float z, float) {
                       dGh1[m * dh + n] = x;
                       const float dg1 = eta[m] * x;
                       dP[m * dh + n] = dg1 * act_df<ACT>(z);
                       dZ1[m * dh + n] = dg1 * pp * act_d2f<ACT>(z);
                     });
    gemm<1, 0, 0, 1>(c, dk, Term{dS, C, Qc, dk, c, 1.0f}, Term{Gh1, dh, D1, dh, dh, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dKp[m * dk + n] = x; });
    __syncthreads();
    gemm1<0, 0>(c, dv, Term{dP, dh, W2, dv, dh, 1.0f}, Aux{{dGh2, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float dgh, float, float) {
                  const float d = fmaf(eta[m], dgh, x);
                  dG2[m * dv + n] = d;
                  if constexpr (LOSS != 3) E::st(dvv, static_cast<int64_t>(t0 + m) * dv + n, loss_dsignal_dv<LOSS>() * d);
                });
    // d eta per token, one wave per row
    for (int t = wv; t < c; t += kThreads / 64) {
      float sum = 0.0f;
      for (int j = lane; j < dh; j += 64) sum += dGh1[t * dh + j] * P[t * dh + j] * act_df<ACT>(Z1[t * dh + j]);
      for (int j = lane; j < dv; j += 64) sum += dGh2[t * dv + j] * G2[t * dv + j];
      sum = wave_sum(sum);
      if (lane == 0) {
        const float et = eta[t];
        dbeta[t0 + t] = sum * et * (1.0f - 0.5f * et);
      }
    }
    __syncthreads();
    if constexpr (LOSS == 3) {  // dV_hat = J^T dG2 = ri (dG2 - d_v G2 <G2, dG2>) in place of dG2;  dV = -dV_hat
      for (int t = wv; t < c; t += kThreads / 64) {
        float dot = 0.0f;
        for (int j = lane; j < dv; j += 64) dot = fmaf(G2[t * dv + j], dG2[t * dv + j], dot);
        dot = wave_sum(dot) * dv;
        const float ri = rinv[t];
        for (int j = lane; j < dv; j += 64) {
          const float dvh = ri * fmaf(-dot, G2[t * dv + j], dG2[t * dv + j]);
          dG2[t * dv + j] = dvh;
          E::st(dvv, static_cast<int64_t>(t0 + t) * dv + j, -dvh);
        }
      }
      __syncthreads();
    }
    if constexpr (LOSS == 0 || LOSS == 3) {  // dZ1 += (dA + dV_hat W2^T) (.) f'(Z1), dV_hat = dG2 (MSE)
      gemm1<0, 1>(c, dh, Term{dG2, dv, W2, dv, dv, 1.0f}, Aux{{dA, dZ1, Z1}, dh}, lds,
                  [&](int m, int n, float x, float da, float dz, float z) {
                    dZ1[m * dh + n] = fmaf(da + x, act_df<ACT>(z), dz);
                  });
    } else {  // dZ1 += dA (.) f'(Z1)
      constexpr int kU = 4;
      const int nz = c * dh;
      for (int i0 = tid; i0 < nz; i0 += kThreads * kU) {
        float da[kU], dz[kU], z[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = min(i0 + u * kThreads, nz - 1);
          da[u] = dA[i];
          dz[u] = dZ1[i];
          z[u] = Z1[i];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (i0 + u * kThreads < nz) dZ1[i0 + u * kThreads] = fmaf(da[u], act_df<ACT>(z[u]), dz[u]);
      }
    }
    __syncthreads();
    gemm1<0, 1>(c, dk, Term{dZ1, dh, W1, dh, dh, 1.0f}, Aux{{dKp, nullptr, nullptr}, dk}, lds,
                [&](int m, int n, float x, float dkp, float, float) {
                  E::st(dkk, static_cast<int64_t>(t0 + m) * dk + n, dkp + x);
                });
    gemm<1, 0, 1, 0>(dk, dh, Term{Qc, dk, dX1, dh, c, 1.0f}, Term{Kc, dk, dZ1, dh, c, 1.0f},
                     Aux{{D1, nullptr, nullptr}, dh}, lds,
                     [&](int m, int n, float x, float d1, float, float) { D1o[m * dh + n] = fmaf(g, d1, x); });
    gemm<1, 0, 1, 0>(dh, dv, Term{Aq, dh, dOc, dv, c, 1.0f}, Term{dP, dh, G2, dv, c, 1.0f},
                     Aux{{D2, nullptr, nullptr}, dv}, lds,
                     [&](int m, int n, float x, float d2, float, float) { D2o[m * dv + n] = fmaf(g, d2, x); });
    if constexpr (LOSS == 0 || LOSS == 3) {  // + A^T dV_hat
      __syncthreads();
      gemm1<1, 0>(dh, dv, Term{Ac, dh, dG2, dv, c, 1.0f}, Aux{{D2o, nullptr, nullptr}, dv}, lds,
                  [&](int m, int n, float x, float d2, float, float) { D2o[m * dv + n] = d2 + x; });
    }
    __syncthreads();
    cur ^= 1;
  }

  const float* D1 = sc + (cur ? L.dw1[1] : L.dw1[0]);
  const float* D2 = sc + (cur ? L.dw2[1] : L.dw2[0]);
  if (a.dw1_0)
    for (int64_t i = tid; i < n1; i += kThreads) a.dw1_0[bh * n1 + i] = D1[i];
  if (a.dw2_0)
    for (int64_t i = tid; i < n2; i += kThreads) a.dw2_0[bh * n2 + i] = D2[i];
  if (scalar_decay) {
    dgam = wave_sum(dgam);
    if (lane == 0) wsum[wv] = dgam;
    __syncthreads();
    if (tid == 0) {
      float t = 0.0f;
      for (int w = 0; w < kThreads / 64; ++w) t += wsum[w];
      a.dgamma[bh] = t;
    }
  }
}

template <typename T, int LOSS, int ACT>
hipError_t launch_bwd_t(const MlpBwdArgs& a, hipStream_t s) {
  auto kern = mlp_bwd_kernel<T, LOSS, ACT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (e != hipSuccess) return e;
  KernelScope timing(TTT_KERNEL_MLP_BWD, s);
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

struct BwdL {
  template <typename T, int LOSS, int ACT>
  static hipError_t run(const MlpBwdArgs& a, hipStream_t s) { return launch_bwd_t<T, LOSS, ACT>(a, s); }
};

}  // namespace

size_t mlp_saved_bytes(const ttt_mlp_desc& d) {
  const MlpSaved SV(d.C, d.dh, d.dv);
  const int64_t nc = (static_cast<int64_t>(d.T) + d.C - 1) / d.C;
  return align256(sizeof(float) * static_cast<size_t>(d.B) * d.H * nc * SV.per_chunk);
}

size_t mlp_bwd_workspace(const ttt_mlp_desc& d) {
  const MlpBwdScratch L(d.C, d.dk, d.dh, d.dv);
  return align256(sizeof(float) * static_cast<size_t>(d.B) * d.H * L.total);
}

hipError_t mlp_bwd_launch(const ttt_mlp_desc& d, const void* q, const void* k, const void* v, const float* beta,
                          const float* gamma, const float* w1_ckpt, const float* w2_ckpt, const void* saved,
                          const void* d_o, const float* d_w1final, const float* d_w2final, void* dq, void* dk,
                          void* dv, float* dbeta, float* dgamma, float* dw1_0, float* dw2_0, void* ws,
                          hipStream_t s) {
  MlpBwdArgs a{};
  a.B = d.B; a.H = d.H; a.T = d.T; a.dk = d.dk; a.dh = d.dh; a.dv = d.dv; a.C = d.C;
  a.NC = (d.T + d.C - 1) / d.C;
  a.decay = d.decay;
  a.b = d.lr_bias;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gamma = gamma; a.w1_ckpt = w1_ckpt; a.w2_ckpt = w2_ckpt;
  a.saved = static_cast<const float*>(saved);
  a.d_o = d_o; a.d_w1final = d_w1final; a.d_w2final = d_w2final;
  a.dq = dq; a.dk_out = dk; a.dv_out = dv; a.dbeta = dbeta; a.dgamma = dgamma; a.dw1_0 = dw1_0; a.dw2_0 = dw2_0;
  a.scratch = static_cast<float*>(ws);
  return by_enums<BwdL>(a, d, s);
}

}  // namespace ttt
