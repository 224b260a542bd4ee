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
// Outer backward.  For the outer loss <dO, O> + <dW1_T, W1_T> + <dW2_T, W2_T>,
// chunk i (from the last to the first) takes its forward from the checkpoints
// W1_i, W2_i (or the forward's saved context) and differentiates its steps in
// reverse order, carrying dW1_{i+1}, dW2_{i+1} (written D1, D2 below):
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
// workspace (or the saved context).
// ---------------------------------------------------------------------------

// Two kernels.  Only the adjoints of the states, D1 = dW1_{i+1} and D2 =
// dW2_{i+1}, are carried from chunk to chunk; every other term either does not
// involve them or enters linearly beside them.  mlp_bwd_pre_kernel (one
// workgroup per (chain, chunk), all at once) takes the chunk's forward (saved,
// or recomputed from the checkpoints) and forms everything free of D1, D2:
//   dS2, dX1, dS1, the final dQ, and the partial terms
//   Pg2 = -S2^T dO,  dA_p = dS2^T A_q,  Pg1 = -S1^T dX1,  dK_p = dS1^T Q,
//   A1 = Q^T dX1,  A2 = A_q^T dO.
// mlp_bwd_kernel (one workgroup per chain, chunks in reverse) then does only the
// products with D1, D2 and what follows from them:
//   d(eta G2) = Pg2 - A D2;  dA = dA_p - (eta G2) D2^T;  d(eta G1) = Pg1 - K D1
//   (with dP, the f'' part of dZ1);  dK_p -= (eta G1) D1^T;  dG2, dV, d eta;
//   dZ1 += (dA + dV_hat W2^T) (.) f'(Z1);  dK = dZ1 W1^T + dK_p;
//   dW1_i = g D1 + A1 + K^T dZ1;  dW2_i = g D2 + A2 + dP^T G2 + A^T dV_hat.

// Per (chain, chunk): what the sweep reads back (the forward's intermediates when
// there is no saved context, the staged K, the pre-pass's terms), then the
// pre-pass's own operands and scratch.
struct MlpBwdChunk {
  int64_t k, z1, a, aq, p, gh1, g2, gh2, pg2, dap, pg1, dkp, a1, a2, ri, eta, total;
  __host__ __device__ MlpBwdChunk(int C, int dk, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t ch = static_cast<int64_t>(C) * dh, cv = static_cast<int64_t>(C) * dv,
                  ckk = static_cast<int64_t>(C) * dk;
    k = take(ckk); z1 = take(ch); a = take(ch); aq = take(ch); p = take(ch); gh1 = take(ch); g2 = take(cv);
    gh2 = take(cv); pg2 = take(cv); dap = take(ch); pg1 = take(ch); dkp = take(ckk);
    a1 = take(static_cast<int64_t>(dk) * dh); a2 = take(static_cast<int64_t>(dh) * dv);
    ri = take(C); eta = take(C);
    total = o;
  }
};
struct MlpBwdPre {
  int64_t q, v, dout, x1, dx1, s1, s2, ds, total;
  __host__ __device__ MlpBwdPre(int C, int dk, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t ch = static_cast<int64_t>(C) * dh, cv = static_cast<int64_t>(C) * dv,
                  ckk = static_cast<int64_t>(C) * dk, cc = static_cast<int64_t>(C) * C;
    q = take(ckk); v = take(cv); dout = take(cv); x1 = take(ch); dx1 = take(ch);
    s1 = take(cc); s2 = take(cc); ds = take(cc);
    total = o;
  }
};
// Per chain: the sweep's carried adjoints (two buffers each) and its per-chunk terms.
struct MlpBwdSeq {
  int64_t dw1[2], dw2[2], dgh1, da, dp, dz1, dgh2, dg2, dkp, total;
  __host__ __device__ MlpBwdSeq(int C, int dk, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t ch = static_cast<int64_t>(C) * dh, cv = static_cast<int64_t>(C) * dv,
                  ckk = static_cast<int64_t>(C) * dk;
    dw1[0] = take(static_cast<int64_t>(dk) * dh);
    dw1[1] = take(static_cast<int64_t>(dk) * dh);
    dw2[0] = take(static_cast<int64_t>(dh) * dv);
    dw2[1] = take(static_cast<int64_t>(dh) * dv);
    dgh1 = take(ch); da = take(ch); dp = take(ch); dz1 = take(ch); dgh2 = take(cv); dg2 = take(cv); dkp = take(ckk);
    total = o;
  }
};
struct MlpBwdWs {
  int64_t chunk, pre, seq, total;
  __host__ __device__ MlpBwdWs(int B, int H, int T, int C, int dk, int dh, int dv) {
    const int64_t BH = static_cast<int64_t>(B) * H, items = BH * ((T + C - 1) / C);
    chunk = 0;
    pre = items * MlpBwdChunk(C, dk, dh, dv).total;
    seq = pre + items * MlpBwdPre(C, dk, dh, dv).total;
    total = seq + BH * MlpBwdSeq(C, dk, dh, dv).total;
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

// The forward intermediates of chunk item = (chain, chunk) that the sweep reads:
// the forward's saved context, or the pre-pass's recomputation.
struct MlpFwdViews {
  const float *z1, *a, *aq, *p, *gh1, *g2, *gh2, *ri;
};
__device__ __forceinline__ MlpFwdViews mlp_fwd_views(const MlpBwdArgs& a, int64_t item, float* ch,
                                                     const MlpBwdChunk& L) {
  MlpFwdViews f;
  if (a.saved) {
    const MlpSaved SV(a.C, a.dh, a.dv);
    const float* sb = a.saved + item * SV.per_chunk;
    f.z1 = sb + SV.z1; f.a = sb + SV.a; f.aq = sb + SV.aq; f.p = sb + SV.p; f.gh1 = sb + SV.gh1;
    f.g2 = sb + SV.g2; f.gh2 = sb + SV.gh2; f.ri = sb + SV.ri;
  } else {
    f.z1 = ch + L.z1; f.a = ch + L.a; f.aq = ch + L.aq; f.p = ch + L.p; f.gh1 = ch + L.gh1;
    f.g2 = ch + L.g2; f.gh2 = ch + L.gh2; f.ri = ch + L.ri;
  }
  return f;
}

template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads, 2) void mlp_bwd_pre_kernel(MlpBwdArgs a) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x / a.NC, ci = blockIdx.x % a.NC;
  const int dk = a.dk, dh = a.dh, dv = a.dv, C = a.C;
  const int t0 = ci * C;
  const int c = min(C, a.T - t0);
  const int64_t item = blockIdx.x;
  const MlpBwdWs WS(a.B, a.H, a.T, C, dk, dh, dv);
  const MlpBwdChunk L(C, dk, dh, dv);
  const MlpBwdPre P(C, dk, dh, dv);
  float* ch = a.scratch + WS.chunk + item * L.total;
  float* pr = a.scratch + WS.pre + item * P.total;
  float *Kc = ch + L.k, *Pg2 = ch + L.pg2, *dAp = ch + L.dap, *Pg1 = ch + L.pg1, *dKp = ch + L.dkp, *A1 = ch + L.a1,
        *A2 = ch + L.a2, *eta = ch + L.eta;
  float *Qc = pr + P.q, *Vc = pr + P.v, *dOc = pr + P.dout, *dX1 = pr + P.dx1, *dS = pr + P.ds;
  // the forward's intermediates: recomputed here into the chunk's area, or the saved context
  float *Z1 = ch + L.z1, *Ac = ch + L.a, *Aq = ch + L.aq, *Pp = ch + L.p, *Gh1 = ch + L.gh1, *G2 = ch + L.g2,
        *Gh2 = ch + L.gh2, *RI = ch + L.ri, *X1 = pr + P.x1, *S1 = pr + P.s1, *S2 = pr + P.s2;
  const bool have = a.saved != nullptr;
  if (have) {
    const MlpSaved SV(C, dh, dv);
    float* sb = const_cast<float*>(a.saved) + item * SV.per_chunk;
    Z1 = sb + SV.z1; Ac = sb + SV.a; X1 = sb + SV.x1; Aq = sb + SV.aq; Pp = sb + SV.p; Gh1 = sb + SV.gh1;
    G2 = sb + SV.g2; Gh2 = sb + SV.gh2; S1 = sb + SV.s1; S2 = sb + SV.s2; RI = sb + SV.ri;
  }
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk;
  const int64_t off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  const T* dO = static_cast<const T*>(a.d_o) + off_v;
  T* dq = static_cast<T*>(a.dq) + off_k;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  const float* W1 = a.w1_ckpt + item * dk * dh;
  const float* W2 = a.w2_ckpt + item * dh * dv;

  stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
  stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
  if (!have) stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
  stage_rows<E>(dOc, dO + static_cast<int64_t>(t0) * dv, c * dv);
  for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
  __syncthreads();

  if (!have) {  // ---- the chunk's forward again ----
    gemm1<0, 0, false, 1>(c, dh, Term{Kc, dk, W1, dh, dk, 1.0f}, kNoAux, lds, [&](int m, int n, float x, float, float, float) {
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
      gemm1<0, 0, false, 1>(c, dv, Term{Ac, dh, W2, dv, dh, 1.0f}, Aux{{Vc, nullptr, nullptr}, dv}, lds,
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
        if (lane == 0) RI[t] = ri;
      }
      __syncthreads();
    }
    gemm1<0, 1, false, 1>(c, dh, Term{G2, dv, W2, dv, dv, 1.0f}, Aux{{Z1, nullptr, nullptr}, dh}, lds,
                [&](int m, int n, float x, float z, float, float) {
                  Pp[m * dh + n] = x;
                  Gh1[m * dh + n] = eta[m] * x * act_df<ACT>(z);
                });
    gemm1<0, 1, true, 1>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { S1[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(S1, c, C);
    __syncthreads();
    gemm<0, 0, 0, 0, false, true, 1>(c, dh, Term{Qc, dk, W1, dh, dk, 1.0f}, Term{S1, C, Gh1, dh, c, -1.0f}, kNoAux,
                                  lds, [&](int m, int n, float x, float, float, float) {
                                    X1[m * dh + n] = x;
                                    Aq[m * dh + n] = act_f<ACT>(x);
                                  });
    __syncthreads();
    gemm1<0, 1, true, 1>(c, c, Term{Aq, dh, Ac, dh, dh, 1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { S2[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(S2, c, C);
    __syncthreads();
  }

  // ---- the backward's terms free of D1, D2 ----
  gemm1<0, 1, true, 1>(c, c, Term{dOc, dv, Gh2, dv, dv, -1.0f}, kNoAux, lds,
                    [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
  zero_upper_tiles(dS, c, C);
  gemm1<1, 0, false, 1>(c, dv, Term{S2, C, dOc, dv, c, -1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { Pg2[m * dv + n] = x; });
  __syncthreads();
  gemm<0, 1, 0, 0, false, true, 1>(c, dh, Term{dOc, dv, W2, dv, dv, 1.0f}, Term{dS, C, Ac, dh, c, 1.0f},
                                Aux{{X1, nullptr, nullptr}, dh}, lds,
                                [&](int m, int n, float x, float x1, float, float) {
                                  dX1[m * dh + n] = x * act_df<ACT>(x1);
                                });
  gemm1<1, 0, false, 1>(c, dh, Term{dS, C, Aq, dh, c, 1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { dAp[m * dh + n] = x; });
  gemm1<1, 0, false, 1>(dh, dv, Term{Aq, dh, dOc, dv, c, 1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { A2[m * dv + n] = x; });
  __syncthreads();
  gemm1<0, 1, true, 1>(c, c, Term{dX1, dh, Gh1, dh, dh, -1.0f}, kNoAux, lds,
                    [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
  zero_upper_tiles(dS, c, C);
  __syncthreads();
  gemm<0, 1, 0, 0, false, true, 1>(c, dk, Term{dX1, dh, W1, dh, dh, 1.0f}, Term{dS, C, Kc, dk, c, 1.0f}, kNoAux, lds,
                                [&](int m, int n, float x, float, float, float) {
                                  E::st(dq, static_cast<int64_t>(t0 + m) * dk + n, x);
                                });
  gemm1<1, 0, false, 1>(c, dh, Term{S1, C, dX1, dh, c, -1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { Pg1[m * dh + n] = x; });
  gemm1<1, 0, false, 1>(c, dk, Term{dS, C, Qc, dk, c, 1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { dKp[m * dk + n] = x; });
  gemm1<1, 0, false, 1>(dk, dh, Term{Qc, dk, dX1, dh, c, 1.0f}, kNoAux, lds,
              [&](int m, int n, float x, float, float, float) { A1[m * dh + n] = x; });
}

template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void mlp_bwd_kernel(MlpBwdArgs a) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  __shared__ float wsum[kThreads / 64];
  __shared__ float eta[256];  // the chunk's eta, read by the epilogues and the row pass
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x;
  const int dk = a.dk, dh = a.dh, dv = a.dv, C = a.C;
  const MlpBwdWs WS(a.B, a.H, a.T, C, dk, dh, dv);
  const MlpBwdChunk L(C, dk, dh, dv);
  const MlpBwdSeq Q(C, dk, dh, dv);
  float* sq = a.scratch + WS.seq + static_cast<int64_t>(bh) * Q.total;
  float *dGh1 = sq + Q.dgh1, *dA = sq + Q.da, *dP = sq + Q.dp, *dZ1 = sq + Q.dz1, *dGh2 = sq + Q.dgh2,
        *dG2 = sq + Q.dg2, *dKp = sq + Q.dkp;
  const bool scalar_decay = a.decay == TTT_DECAY_SCALAR;
  const float g = scalar_decay ? a.gamma[bh % a.H] : 1.0f;

  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk;
  const int64_t off_v = static_cast<int64_t>(bh) * a.T * dv;
  T* dkk = static_cast<T*>(a.dk_out) + off_k;
  T* dvv = static_cast<T*>(a.dv_out) + off_v;
  float* dbeta = a.dbeta + static_cast<int64_t>(bh) * a.T;
  const int64_t n1 = static_cast<int64_t>(dk) * dh, n2 = static_cast<int64_t>(dh) * dv;

  {  // dW_T: the final states' gradients (zero when not given)
    float* D1 = sq + Q.dw1[0];
    float* D2 = sq + Q.dw2[0];
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
    const int64_t item = static_cast<int64_t>(bh) * a.NC + ci;
    const float* W1 = a.w1_ckpt + item * n1;
    const float* W2 = a.w2_ckpt + item * n2;
    const float* D1 = sq + (cur ? Q.dw1[1] : Q.dw1[0]);  // dW1_{i+1}
    const float* D2 = sq + (cur ? Q.dw2[1] : Q.dw2[0]);
    float* D1o = sq + (cur ? Q.dw1[0] : Q.dw1[1]);  // dW1_i (written)
    float* D2o = sq + (cur ? Q.dw2[0] : Q.dw2[1]);
    float* ch = a.scratch + WS.chunk + item * L.total;
    const MlpFwdViews F = mlp_fwd_views(a, item, ch, L);
    const float *Kc = ch + L.k, *Pg2 = ch + L.pg2, *dAp = ch + L.dap, *Pg1 = ch + L.pg1, *dKpp = ch + L.dkp,
                *A1 = ch + L.a1, *A2 = ch + L.a2;
    // to LDS: the first product's barriers order these writes before any read, and
    // the previous chunk's last reads end at its closing barrier
    for (int t = tid; t < c; t += kThreads) eta[t] = ch[L.eta + t];
    if (scalar_decay) {
      dgam = strided_dot(D1, W1, n1, dgam);
      dgam = strided_dot(D2, W2, n2, dgam);
    }

    gemm1<0, 0>(c, dv, Term{F.a, dh, D2, dv, dh, -1.0f}, Aux{{Pg2, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float pg, float, float) { dGh2[m * dv + n] = pg + x; });
    gemm1<0, 1>(c, dh, Term{F.gh2, dv, D2, dv, dv, -1.0f}, Aux{{dAp, nullptr, nullptr}, dh}, lds,
                [&](int m, int n, float x, float dap, float, float) { dA[m * dh + n] = dap + x; });
    gemm1<0, 0>(c, dh, Term{Kc, dk, D1, dh, dk, -1.0f}, Aux{{Pg1, F.p, F.z1}, dh}, lds,
                [&](int m, int n, float x, float pg, float pp, float z) {
                  const float v1 = pg + x;
                  dGh1[m * dh + n] = v1;
                  const float dg1 = eta[m] * v1;
                  dP[m * dh + n] = dg1 * act_df<ACT>(z);
                  dZ1[m * dh + n] = dg1 * pp * act_d2f<ACT>(z);
                });
    gemm1<0, 1>(c, dk, Term{F.gh1, dh, D1, dh, dh, -1.0f}, Aux{{dKpp, nullptr, nullptr}, dk}, lds,
                [&](int m, int n, float x, float dkp, float, float) { dKp[m * dk + n] = dkp + x; });
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
      for (int j = lane; j < dh; j += 64) sum += dGh1[t * dh + j] * F.p[t * dh + j] * act_df<ACT>(F.z1[t * dh + j]);
      for (int j = lane; j < dv; j += 64) sum += dGh2[t * dv + j] * F.g2[t * dv + j];
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
        for (int j = lane; j < dv; j += 64) dot = fmaf(F.g2[t * dv + j], dG2[t * dv + j], dot);
        dot = wave_sum(dot) * dv;
        const float ri = F.ri[t];
        for (int j = lane; j < dv; j += 64) {
          const float dvh = ri * fmaf(-dot, F.g2[t * dv + j], dG2[t * dv + j]);
          dG2[t * dv + j] = dvh;
          E::st(dvv, static_cast<int64_t>(t0 + t) * dv + j, -dvh);
        }
      }
      __syncthreads();
    }
    if constexpr (LOSS == 0 || LOSS == 3) {  // dZ1 += (dA + dV_hat W2^T) (.) f'(Z1), dV_hat = dG2 (MSE)
      gemm1<0, 1>(c, dh, Term{dG2, dv, W2, dv, dv, 1.0f}, Aux{{dA, dZ1, F.z1}, dh}, lds,
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
          z[u] = F.z1[i];
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
    gemm1<1, 0>(dk, dh, Term{Kc, dk, dZ1, dh, c, 1.0f}, Aux{{D1, A1, nullptr}, dh}, lds,
                [&](int m, int n, float x, float d1, float a1, float) { D1o[m * dh + n] = fmaf(g, d1, a1 + x); });
    gemm1<1, 0>(dh, dv, Term{dP, dh, F.g2, dv, c, 1.0f}, Aux{{D2, A2, nullptr}, dv}, lds,
                [&](int m, int n, float x, float d2, float a2, float) { D2o[m * dv + n] = fmaf(g, d2, a2 + x); });
    if constexpr (LOSS == 0 || LOSS == 3) {  // + A^T dV_hat
      __syncthreads();
      gemm1<1, 0>(dh, dv, Term{F.a, dh, dG2, dv, c, 1.0f}, Aux{{D2o, nullptr, nullptr}, dv}, lds,
                  [&](int m, int n, float x, float d2, float, float) { D2o[m * dv + n] = d2 + x; });
    }
    __syncthreads();
    cur ^= 1;
  }

  const float* D1 = sq + (cur ? Q.dw1[1] : Q.dw1[0]);
  const float* D2 = sq + (cur ? Q.dw2[1] : Q.dw2[0]);
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

template <class K>
hipError_t launch_bwd_k(K kern, const MlpBwdArgs& a, ttt_kernel id, int nblk, hipStream_t s,
                        size_t lds = kLdsBytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  KernelScope timing(id, s);
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename T, int LOSS, int ACT>
hipError_t launch_bwd_t(const MlpBwdArgs& a, hipStream_t s) {
  hipError_t e =
      launch_bwd_k(mlp_bwd_pre_kernel<T, LOSS, ACT>, a, TTT_KERNEL_MLP_BWD_PRE, a.B * a.H * a.NC, s, kLdsBytes1);
  if (e != hipSuccess) return e;
  return launch_bwd_k(mlp_bwd_kernel<T, LOSS, ACT>, a, TTT_KERNEL_MLP_BWD, a.B * a.H, s);
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
  return align256(sizeof(float) * static_cast<size_t>(MlpBwdWs(d.B, d.H, d.T, d.C, d.dk, d.dh, d.dv).total));
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
