// The fast net Linear -> Norm (the Norm primitive) as the act of the chunkwise
// layer (TTT_ACT_NORM): forward and analytic outer backward, one workgroup per
// chain on the tile GEMM of tile_gemm.h.
//
// The Modular TTT summary page composes a fast net's chunk computation from its
// primitives' rules (section "Method step details", Algorithm 1) and names Norm
// among them, with a hand-written backward (sections "Experimental results" and
// "Technical novelty").  Here V_hat = N(K W), N the per-token normalisation over
// the d_v features, and the query view reads O = N(Y).

#include <type_traits>

#include "tile_gemm.h"
#include "ttt_device.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

// ---------------------------------------------------------------------------
// The fast net Linear -> Norm (the Norm primitive): V_hat = N(K W) with the
// per-token normalisation N(z) = (z - mean(z)) / s(z), s(z) = sqrt(var(z) + eps)
// over the d_v features; the query view O = N(Y) with the Linear's dual form Y.
// The normalisation couples a token's features, so one workgroup carries one
// chain (no column split); the products use the tile GEMM and the
// per-token steps are one wave per row.
// ---------------------------------------------------------------------------

constexpr float kNormEps = 1e-5f;

struct NormScratch {
  int64_t w[2], dw[2], q, k, v, dout, z, gh, g, e, n, rs, y, dy, dgh, dz, dkp, s, ds, total;
  __host__ __device__ NormScratch(int C, int dk, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t kv = static_cast<int64_t>(dk) * dv, cv = static_cast<int64_t>(C) * dv,
                  ck = static_cast<int64_t>(C) * dk, cc = static_cast<int64_t>(C) * C;
    w[0] = take(kv); w[1] = take(kv); dw[0] = take(kv); dw[1] = take(kv);
    q = take(ck); k = take(ck); v = take(cv); dout = take(cv);
    z = take(cv); gh = take(cv); g = take(cv); e = take(cv); n = take(cv); rs = take(C);
    y = take(cv); dy = take(cv); dgh = take(cv); dz = take(cv); dkp = take(ck);
    s = take(cc); ds = take(cc);
    total = o;
  }
};

// Row t of the train view.  V_hat = N(z) (ACT 3) or f(z) (ACT 0..2); the loss
// signal E (LOSS 3 = RMSE: e / (sqrt(d) ||e||), e = V_hat - v, 0 where e = 0);
// G = J_N^T E = (E - mean E - n <E, n> / d) / s (Norm) or E (.) f'(z).  Returns
// 1/s (Norm) in rs_out and 1 / (sqrt(d) ||e||) (RMSE) in ri_out.
template <int LOSS, int ACT>
__device__ __forceinline__ void train_row(const float* z, const float* vv, float* vh, float* e, float* G, float* Gh,
                                          float& rs_out, float& ri_out, float et, int dv, int lane) {
  float mu = 0.0f, rs = 1.0f;
  if constexpr (ACT == 3) {
    mu = row_sum(dv, lane, [&](int j) { return z[j]; }) / dv;
    const float var = row_sum(dv, lane, [&](int j) { return (z[j] - mu) * (z[j] - mu); });
    rs = rsqrtf(var / dv + kNormEps);
  }
  auto vhat = [&](int j) { return ACT == 3 ? (z[j] - mu) * rs : act_f<ACT>(z[j]); };
  float ri = 0.0f;
  if constexpr (LOSS == 3) {
    const float ne2 = row_sum(dv, lane, [&](int j) { const float d = vhat(j) - vv[j]; return d * d; });
    ri = ne2 > 0.0f ? rsqrtf(ne2 * dv) : 0.0f;
  }
  auto sig = [&](int j) { return LOSS == 3 ? (vhat(j) - vv[j]) * ri : loss_signal<LOSS, 0>(vhat(j), vv[j]); };
  float me = 0.0f, en = 0.0f;
  if constexpr (ACT == 3) {
    me = row_sum(dv, lane, [&](int j) { return sig(j); }) / dv;
    en = row_sum(dv, lane, [&](int j) { return sig(j) * vhat(j); }) / dv;
  }
  for (int j = lane; j < dv; j += 64) {
    const float nj = vhat(j), ej = sig(j);
    const float gj = (ACT == 3) ? (ej - me - nj * en) * rs : ej * act_df<ACT>(z[j]);
    if (vh) vh[j] = nj;
    if (e) e[j] = ej;
    if (G) G[j] = gj;
    Gh[j] = et * gj;
  }
  rs_out = rs;
  ri_out = ri;
}

template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void norm_fwd_kernel(FwdArgs a, float* scratch) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  __shared__ float eta[256];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x;
  const int dk = a.dk, dv = a.dv, C = a.C;
  const NormScratch L(C, dk, dv);
  float* sc = scratch + static_cast<int64_t>(bh) * L.total;
  float *Qc = sc + L.q, *Kc = sc + L.k, *Vc = sc + L.v, *Z = sc + L.z, *Gh = sc + L.gh, *Y = sc + L.y, *S = sc + L.s;
  const bool scalar_decay = a.decay == TTT_DECAY_SCALAR;
  const float g = scalar_decay ? a.gamma[bh % a.H] : 1.0f;
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk, off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  T* o = static_cast<T*>(a.o) + off_v;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  const int64_t nw = static_cast<int64_t>(dk) * dv;
  {
    float* W = sc + L.w[0];
    const float* src = a.w0 ? a.w0 + bh * nw : nullptr;
    for (int64_t i = tid; i < nw; i += kThreads) W[i] = src ? src[i] : 0.0f;
  }
  int cur = 0;
  for (int ci = 0; ci < a.NC; ++ci) {
    const int t0 = ci * C, c = min(C, a.T - t0);
    float* W = sc + (cur ? L.w[1] : L.w[0]);
    float* Wn = sc + (cur ? L.w[0] : L.w[1]);
    stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    if (a.w_ckpt) stage_rows<Elem<float>>(a.w_ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * nw, W,
                                          static_cast<int>(nw));
    __syncthreads();
    gemm1<0, 0>(c, dv, Term{Kc, dk, W, dv, dk, 1.0f}, kNoAux, lds,
                [&](int m, int n, float x, float, float, float) { Z[m * dv + n] = x; });
    __syncthreads();
    for (int t = wv; t < c; t += kThreads / 64) {
      float rs, ri;
      train_row<LOSS, ACT>(Z + t * dv, Vc + t * dv, nullptr, nullptr, nullptr, Gh + t * dv, rs, ri, eta[t], dv, lane);
    }
    gemm1<0, 1, true>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { S[m * C + n] = (n <= m) ? x : 0.0f; });
    __syncthreads();
    gemm<0, 0, 0, 0, false, true>(c, dv, Term{Qc, dk, W, dv, dk, 1.0f}, Term{S, C, Gh, dv, c, -1.0f}, kNoAux, lds,
                                  [&](int m, int n, float x, float, float, float) { Y[m * dv + n] = x; });
    __syncthreads();
    for (int t = wv; t < c; t += kThreads / 64) {  // O = N(Y) or f(Y)
      const float* y = Y + t * dv;
      float mu = 0.0f, rs = 1.0f;
      if constexpr (ACT == 3) {
        mu = row_sum(dv, lane, [&](int j) { return y[j]; }) / dv;
        const float var = row_sum(dv, lane, [&](int j) { return (y[j] - mu) * (y[j] - mu); });
        rs = rsqrtf(var / dv + kNormEps);
      }
      for (int j = lane; j < dv; j += 64)
        E::st(o, static_cast<int64_t>(t0 + t) * dv + j, ACT == 3 ? (y[j] - mu) * rs : act_f<ACT>(y[j]));
    }
    gemm1<1, 0>(dk, dv, Term{Kc, dk, Gh, dv, c, -1.0f}, Aux{{W, nullptr, nullptr}, dv}, lds,
                [&](int m, int n, float x, float w, float, float) { Wn[m * dv + n] = fmaf(g, w, x); });
    __syncthreads();
    cur ^= 1;
  }
  const float* W = sc + (cur ? L.w[1] : L.w[0]);
  if (a.w_final)
    for (int64_t i = tid; i < nw; i += kThreads) a.w_final[bh * nw + i] = W[i];
}

template <typename T, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void norm_bwd_kernel(BwdArgs a, float* scratch) {
  using E = Elem<T>;
  extern __shared__ __align__(16) float lds[];
  __shared__ float eta[256];
  __shared__ float rsv[256];
  __shared__ float riv[256];
  __shared__ float wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
  const int bh = blockIdx.x;
  const int dk = a.dk, dv = a.dv, C = a.C;
  const NormScratch L(C, dk, dv);
  float* sc = scratch + static_cast<int64_t>(bh) * L.total;
  float *Qc = sc + L.q, *Kc = sc + L.k, *Vc = sc + L.v, *dOc = sc + L.dout, *Z = sc + L.z, *Gh = sc + L.gh,
        *G = sc + L.g, *Ec = sc + L.e, *Nc = sc + L.n, *Y = sc + L.y, *dY = sc + L.dy, *dGh = sc + L.dgh,
        *dZ = sc + L.dz, *dKp = sc + L.dkp, *S = sc + L.s, *dS = sc + L.ds;
  const bool scalar_decay = a.decay == TTT_DECAY_SCALAR;
  const float g = scalar_decay ? a.gamma[bh % a.H] : 1.0f;
  const int64_t off_k = static_cast<int64_t>(bh) * a.T * dk, off_v = static_cast<int64_t>(bh) * a.T * dv;
  const T* q = static_cast<const T*>(a.q) + off_k;
  const T* k = static_cast<const T*>(a.k) + off_k;
  const T* v = static_cast<const T*>(a.v) + off_v;
  const T* dO = static_cast<const T*>(a.d_o) + off_v;
  T* dq = static_cast<T*>(a.dq) + off_k;
  T* dkk = static_cast<T*>(a.dk_out) + off_k;
  T* dvv = static_cast<T*>(a.dv_out) + off_v;
  const float* beta = a.beta + static_cast<int64_t>(bh) * a.T;
  float* dbeta = a.dbeta + static_cast<int64_t>(bh) * a.T;
  const int64_t nw = static_cast<int64_t>(dk) * dv;
  {
    float* D = sc + L.dw[0];
    const float* src = a.d_wfinal ? a.d_wfinal + bh * nw : nullptr;
    for (int64_t i = tid; i < nw; i += kThreads) D[i] = src ? src[i] : 0.0f;
  }
  int cur = 0;
  float dgam = 0.0f;
  __syncthreads();
  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int t0 = ci * C, c = min(C, a.T - t0);
    const float* W = a.w_ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * nw;
    const float* D = sc + (cur ? L.dw[1] : L.dw[0]);  // dW_{i+1}
    float* Do = sc + (cur ? L.dw[0] : L.dw[1]);       // dW_i
    stage_rows<E>(Qc, q + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Kc, k + static_cast<int64_t>(t0) * dk, c * dk);
    stage_rows<E>(Vc, v + static_cast<int64_t>(t0) * dv, c * dv);
    stage_rows<E>(dOc, dO + static_cast<int64_t>(t0) * dv, c * dv);
    for (int t = tid; t < c; t += kThreads) eta[t] = lr_gate(beta[t0 + t], a.b);
    if (scalar_decay)
      for (int64_t i = tid; i < nw; i += kThreads) dgam = fmaf(D[i], W[i], dgam);
    __syncthreads();
    // the chunk's forward again
    gemm1<0, 0>(c, dv, Term{Kc, dk, W, dv, dk, 1.0f}, kNoAux, lds,
                [&](int m, int n, float x, float, float, float) { Z[m * dv + n] = x; });
    __syncthreads();
    for (int t = wv; t < c; t += kThreads / 64) {
      float rs, ri;
      train_row<LOSS, ACT>(Z + t * dv, Vc + t * dv, Nc + t * dv, Ec + t * dv, G + t * dv, Gh + t * dv, rs, ri,
                           eta[t], dv, lane);
      if (lane == 0) {
        rsv[t] = rs;
        riv[t] = ri;
      }
    }
    gemm1<0, 1, true>(c, c, Term{Qc, dk, Kc, dk, dk, 1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { S[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(S, c, C);
    __syncthreads();
    gemm<0, 0, 0, 0, false, true>(c, dv, Term{Qc, dk, W, dv, dk, 1.0f}, Term{S, C, Gh, dv, c, -1.0f}, kNoAux, lds,
                                  [&](int m, int n, float x, float, float, float) { Y[m * dv + n] = x; });
    __syncthreads();
    for (int t = wv; t < c; t += kThreads / 64) {  // dY = J_N(Y)^T dO, or dO (.) f'(Y)
      const float* y = Y + t * dv;
      const float* d = dOc + t * dv;
      if constexpr (ACT == 3) {
        const float mu = row_sum(dv, lane, [&](int j) { return y[j]; }) / dv;
        const float var = row_sum(dv, lane, [&](int j) { return (y[j] - mu) * (y[j] - mu); });
        const float rs = rsqrtf(var / dv + kNormEps);
        const float md = row_sum(dv, lane, [&](int j) { return d[j]; }) / dv;
        const float dn = row_sum(dv, lane, [&](int j) { return d[j] * ((y[j] - mu) * rs); }) / dv;
        for (int j = lane; j < dv; j += 64) dY[t * dv + j] = (d[j] - md - (y[j] - mu) * rs * dn) * rs;
      } else {
        for (int j = lane; j < dv; j += 64) dY[t * dv + j] = d[j] * act_df<ACT>(y[j]);
      }
    }
    __syncthreads();
    // its backward
    gemm1<0, 1, true>(c, c, Term{dY, dv, Gh, dv, dv, -1.0f}, kNoAux, lds,
                      [&](int m, int n, float x, float, float, float) { dS[m * C + n] = (n <= m) ? x : 0.0f; });
    zero_upper_tiles(dS, c, C);
    gemm<1, 0, 0, 0>(c, dv, Term{S, C, dY, dv, c, -1.0f}, Term{Kc, dk, D, dv, dk, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dGh[m * dv + n] = x; });
    __syncthreads();
    gemm<0, 1, 0, 0, false, true>(c, dk, Term{dY, dv, W, dv, dv, 1.0f}, Term{dS, C, Kc, dk, c, 1.0f}, kNoAux, lds,
                                  [&](int m, int n, float x, float, float, float) {
                                    E::st(dq, static_cast<int64_t>(t0 + m) * dk + n, x);
                                  });
    gemm<1, 0, 0, 1>(c, dk, Term{dS, C, Qc, dk, c, 1.0f}, Term{Gh, dv, D, dv, dv, -1.0f}, kNoAux, lds,
                     [&](int m, int n, float x, float, float, float) { dKp[m * dk + n] = x; });
    for (int t = wv; t < c; t += kThreads / 64) {  // dZ, dV, d eta of row t
      const float et = eta[t], rs = rsv[t], ri = riv[t];
      const float *dgh = dGh + t * dv, *gg = G + t * dv, *ee = Ec + t * dv, *nn = Nc + t * dv, *zz = Z + t * dv;
      const float dgg = row_sum(dv, lane, [&](int j) { return dgh[j] * gg[j]; });  // <d(eta G), G>: d eta
      if (lane == 0) dbeta[t0 + t] = dgg * et * (1.0f - 0.5f * et);
      // (dE / dV_hat)^T x of the loss: x (MSE), (x - e_hat <e_hat, x>) / (sqrt(d) ||e||) (RMSE,
      // e_hat = sqrt(d) E), 0 (IP, L1); its derivative in V is the negative (IP: -I)
      auto rt = [&](auto x, float ehx, int j) {
        if constexpr (LOSS == 0) return x(j);
        else if constexpr (LOSS == 3) return (x(j) - sqrtf(static_cast<float>(dv)) * ee[j] * ehx) * ri;
        else return 0.0f;
      };
      if constexpr (ACT == 3) {
        // dG = eta d(eta G);  M x = x - mean x - n <x, n> / d
        const float mdg = row_sum(dv, lane, [&](int j) { return dgh[j]; }) * et / dv;
        const float dgn = row_sum(dv, lane, [&](int j) { return dgh[j] * nn[j]; }) * et / dv;
        const float en = row_sum(dv, lane, [&](int j) { return ee[j] * nn[j]; }) / dv;
        const float dggd = dgg * et / dv;
        auto mdgf = [&](int j) { return et * dgh[j] - mdg - nn[j] * dgn; };
        float ehm = 0.0f;
        if constexpr (LOSS == 3)
          ehm = row_sum(dv, lane, [&](int j) { return sqrtf(static_cast<float>(dv)) * ee[j] * mdgf(j); });
        auto uf = [&](int j) { return rt(mdgf, ehm, j) - en * et * dgh[j] - dgn * ee[j]; };
        const float mu_u = row_sum(dv, lane, [&](int j) { return uf(j); }) / dv;
        const float un = row_sum(dv, lane, [&](int j) { return uf(j) * nn[j]; }) / dv;
        for (int j = lane; j < dv; j += 64) {
          dZ[t * dv + j] = ((uf(j) - mu_u - nn[j] * un) * rs - nn[j] * dggd) * rs;
          const float dvj = (LOSS == 1) ? -mdgf(j) * rs : -rt(mdgf, ehm, j) * rs;
          E::st(dvv, static_cast<int64_t>(t0 + t) * dv + j, dvj);
        }
      } else {
        // dE = dG (.) f'(z);  dZ = dG (.) E (.) f''(z) + f'(z) (.) (dE/dV_hat)^T dE
        auto def = [&](int j) { return et * dgh[j] * act_df<ACT>(zz[j]); };
        float ehd = 0.0f;
        if constexpr (LOSS == 3)
          ehd = row_sum(dv, lane, [&](int j) { return sqrtf(static_cast<float>(dv)) * ee[j] * def(j); });
        for (int j = lane; j < dv; j += 64) {
          const float r = rt(def, ehd, j);
          dZ[t * dv + j] = et * dgh[j] * ee[j] * act_d2f<ACT>(zz[j]) + act_df<ACT>(zz[j]) * r;
          E::st(dvv, static_cast<int64_t>(t0 + t) * dv + j, (LOSS == 1) ? -def(j) : -r);
        }
      }
    }
    __syncthreads();
    gemm1<0, 1>(c, dk, Term{dZ, dv, W, dv, dv, 1.0f}, Aux{{dKp, nullptr, nullptr}, dk}, lds,
                [&](int m, int n, float x, float dkp, float, float) {
                  E::st(dkk, static_cast<int64_t>(t0 + m) * dk + n, dkp + x);
                });
    gemm<1, 0, 1, 0>(dk, dv, Term{Qc, dk, dY, dv, c, 1.0f}, Term{Kc, dk, dZ, dv, c, 1.0f},
                     Aux{{D, nullptr, nullptr}, dv}, lds,
                     [&](int m, int n, float x, float d, float, float) { Do[m * dv + n] = fmaf(g, d, x); });
    __syncthreads();
    cur ^= 1;
  }
  const float* D = sc + (cur ? L.dw[1] : L.dw[0]);
  if (a.dw0)
    for (int64_t i = tid; i < nw; i += kThreads) a.dw0[bh * nw + i] = D[i];
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

template <class Args, class K>
hipError_t launch_norm(K kern, const Args& a, float* scratch, ttt_kernel id, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (e != hipSuccess) return e;
  KernelScope timing(id, s);
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(kThreads), kLdsBytes, s, a, scratch);
  return hipGetLastError();
}

// The row path runs the Norm act with every loss, and the RMSE loss with every
// elementwise act; the decay is a runtime flag.
template <bool BWD, class Args>
hipError_t norm_dispatch(const Args& a, hipStream_t s) {
  float* sc = reinterpret_cast<float*>(a.ws);
  auto go = [&](auto tt, auto ll, auto aa) -> hipError_t {
    using T = typename decltype(tt)::type;
    constexpr int LS = decltype(ll)::value, AC = decltype(aa)::value;
    if constexpr (BWD) return launch_norm(norm_bwd_kernel<T, LS, AC>, a, sc, TTT_KERNEL_NORM_BWD, s);
    else return launch_norm(norm_fwd_kernel<T, LS, AC>, a, sc, TTT_KERNEL_NORM_FWD, s);
  };
  auto per_type = [&](auto tt) -> hipError_t {
    using I = std::integral_constant<int, 0>;
    if (a.act == TTT_ACT_NORM) {
      if (a.loss == TTT_LOSS_IP) return go(tt, std::integral_constant<int, 1>{}, std::integral_constant<int, 3>{});
      if (a.loss == TTT_LOSS_L1) return go(tt, std::integral_constant<int, 2>{}, std::integral_constant<int, 3>{});
      if (a.loss == TTT_LOSS_RMSE) return go(tt, std::integral_constant<int, 3>{}, std::integral_constant<int, 3>{});
      return go(tt, I{}, std::integral_constant<int, 3>{});
    }
    if (a.act == TTT_ACT_SILU) return go(tt, std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{});
    if (a.act == TTT_ACT_GELU) return go(tt, std::integral_constant<int, 3>{}, std::integral_constant<int, 2>{});
    return go(tt, std::integral_constant<int, 3>{}, I{});
  };
  if (a.dtype == TTT_BF16) return per_type(std::type_identity<bf16_t>{});
  return per_type(std::type_identity<float>{});
}

}  // namespace

size_t norm_fwd_workspace(const FwdArgs& a) {
  const NormScratch L(a.C, a.dk, a.dv);
  return align256(sizeof(float) * static_cast<size_t>(a.B) * a.H * L.total);
}
size_t norm_bwd_workspace(const BwdArgs& a) {
  const NormScratch L(a.C, a.dk, a.dv);
  return align256(sizeof(float) * static_cast<size_t>(a.B) * a.H * L.total);
}
hipError_t norm_fwd_launch(const FwdArgs& a, hipStream_t s) { return norm_dispatch<false>(a, s); }
hipError_t norm_bwd_launch(const BwdArgs& a, hipStream_t s) { return norm_dispatch<true>(a, s); }

}  // namespace ttt
