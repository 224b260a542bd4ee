// Pieces shared by the two-layer fast net's forward (ttt_mlp.hip) and backward
// (ttt_mlp_bwd.hip): the saved-context layout and the enum dispatch.
#pragma once

#include <type_traits>

#include "tile_gemm.h"
#include "ttt_internal.h"

namespace ttt {
namespace {

// Saved context of the forward for its backward, per (chain, chunk), in floats:
// the train view's Z1, A, G2, eta G2, P = G2 W2^T and eta G1, the query view's X1
// and A_q, and both causal score matrices (strictly upper tiles zeroed).
struct MlpSaved {
  int64_t z1, a, x1, aq, p, gh1, g2, gh2, s1, s2, ri, per_chunk;
  __host__ __device__ MlpSaved(int C, int dh, int dv) {
    int64_t o = 0;
    auto take = [&](int64_t n) {
      int64_t r = o;
      o += (n + 63) & ~static_cast<int64_t>(63);
      return r;
    };
    const int64_t ch = static_cast<int64_t>(C) * dh, cv = static_cast<int64_t>(C) * dv,
                  cc = static_cast<int64_t>(C) * C;
    z1 = take(ch);
    a = take(ch);
    x1 = take(ch);
    aq = take(ch);
    p = take(ch);
    gh1 = take(ch);
    g2 = take(cv);
    gh2 = take(cv);
    s1 = take(cc);
    s2 = take(cc);
    ri = take(C);  // RMSE: 1 / (sqrt(d_v) ||V_hat - V||) per token
    per_chunk = o;
  }
};

// Runtime enums to template instantiations; F is the forward or the backward launcher.
// The decay is a runtime flag of the kernels (it scales the state once per chunk).
template <class F, typename T, int LOSS, class A>
hipError_t by_act(const A& a, int act, int, hipStream_t s) {
  if (act == TTT_ACT_SILU) return F::template run<T, LOSS, 1>(a, s);
  if (act == TTT_ACT_GELU) return F::template run<T, LOSS, 2>(a, s);
  return F::template run<T, LOSS, 0>(a, s);
}

template <class F, class A>
hipError_t by_enums(const A& a, const ttt_mlp_desc& d, hipStream_t s) {
  auto per_loss = [&](auto tt) -> hipError_t {
    using T = typename decltype(tt)::type;
    if (d.loss == TTT_LOSS_IP) return by_act<F, T, 1>(a, d.act, d.decay, s);
    if (d.loss == TTT_LOSS_L1) return by_act<F, T, 2>(a, d.act, d.decay, s);
    if (d.loss == TTT_LOSS_RMSE) return by_act<F, T, 3>(a, d.act, d.decay, s);
    return by_act<F, T, 0>(a, d.act, d.decay, s);
  };
  if (d.dtype == TTT_BF16) return per_loss(std::type_identity<bf16_t>{});
  return per_loss(std::type_identity<float>{});
}

}  // namespace
}  // namespace ttt
