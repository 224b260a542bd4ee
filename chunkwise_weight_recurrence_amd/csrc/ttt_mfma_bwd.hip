// Matrix-core outer backward of the chunkwise TTT layer (bf16 I/O), gfx950.
//
// The reverse-mode derivative of each forward step (Modular TTT summary page,
// "Method step details": Algorithm 1's train view, query view and the state
// transition; the hand-written Linear backward the page credits in "Technical
// novelty").  Per chunk i, with dW' = dW_{i+1}:
//   dY = dO (.) f'(Y);  dG~ = -Tril(S)^T dY - K_bar dW';  dG = eta (.) dG~
//   dZ = dG (.) E (.) f''(Z) [+ dG (.) f'(Z)^2 for MSE];  dV = -dG (.) f'(Z)
//   dW_i = diag(lambda) dW' + Q~^T dY + K^T dZ
//   dQ~ = dY W_i^T + dS K~,  dK~ = dS^T Q~,  dS = -Tril(dY G~^T)
//   dK = dZ W_i^T + dK_bar (.) (decay) + dK~ (.) (decay),  dK_bar = -G~ dW'^T
//   deta_s = <dG~_s, G_s>,  dbeta = deta eta (1 - eta/2),  decay chain for lambda, L.
//
// Two kernels, because only the d_v columns of W separate the sequential work:
// * bwd_seq: one workgroup per (chain, 32-column block of d_v), sweeping the
//   chunks in reverse and carrying its dk x 32 slice of dW' in fp32 registers.
//   It recomputes the chunk's forward (Z, G~, S, Y) and produces every
//   column-local term: dV, the dW chain, and per-column-block partial sums of
//   deta.  dY, G~ and dZ (bf16) and the dW_{i+1} checkpoints go to
//   the workspace for the second kernel.
// * bwd_cross: one workgroup per (chain, chunk, 64-row block of d_k), fully
//   parallel.  It forms the terms that sum over all d_v columns (dQ, dK, the
//   decay chain d log a with dlambda = <dW_{i+1}, W_i> per row, dbeta) from dY,
//   G~, dZ, W_i and dW_{i+1}; the score
//   gradient dS is rebuilt tile by tile in registers and never stored.

#include "mfma_util.h"
#include "ttt_device.h"
#include "ttt_internal.h"
#include "ttt_mfma_common.h"

namespace ttt {
namespace {

constexpr int kNB = 32;
constexpr int kSeqThreads = 512;    // bwd_seq: 8 waves, two per SIMD
constexpr int kCrossThreads = 512;  // bwd_cross: 8 waves (the prologue maps 2 x 32 x 8 threads)
constexpr int kDB = 64;  // d_k rows per bwd_cross workgroup

// Token tile of wave w (bwd_seq and bwd_cross).  Waves are dealt to the four SIMDs
// round-robin, so waves s and s + 4 share SIMD s; they get tiles s and 7 - s,
// which balances the causal work per SIMD.
__device__ __forceinline__ int tile_of_wave(int w) { return w < 4 ? w : 11 - w; }

// Workspace carve-up of the matrix-core backward.
struct BwdWs {
  uint16_t* dY;      // [B,H,T,dv] bf16
  uint16_t* Gh;      // [B,H,T,dv] bf16  eta (.) G
  uint16_t* dZ;      // [B,H,T,dv] bf16
  float* dWn;        // [B,H,NC,dk,dv]   dW_{i+1} seen by chunk i
  float* deta_part;  // [NCB][B*H*T]
  float* dlam_part;  // [B*H*NC][dk]  <dW_{i+1}, W_i> per row (scalar decay)
};

size_t ws_layout(const BwdArgs& a, BwdWs* w, char* base) {
  const size_t BH = static_cast<size_t>(a.B) * a.H;
  const size_t tv = BH * a.T * a.dv;
  const int ncb = a.dv / kNB;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  char* p0 = take(tv * 2);
  char* p1 = take(tv * 2);
  char* p2 = take(tv * 2);
  char* p3 = take(BH * a.NC * a.dk * a.dv * 4);
  char* p4 = take(static_cast<size_t>(ncb) * BH * a.T * 4);
  char* p5 = take(BH * a.NC * a.dk * 4);
  if (w) {
    w->dY = reinterpret_cast<uint16_t*>(p0);
    w->Gh = reinterpret_cast<uint16_t*>(p1);
    w->dZ = reinterpret_cast<uint16_t*>(p2);
    w->dWn = reinterpret_cast<float*>(p3);
    w->deta_part = reinterpret_cast<float*>(p4);
    w->dlam_part = reinterpret_cast<float*>(p5);
  }
  return off;
}


// ============================================================================
// bwd_seq
// ============================================================================
// SAVED: the forward's saved context provides G~, f'(Y) and Z (with an act), so the
// chunk's train and query views are not recomputed (no W_i, no Y, no S for Y).
// PAR (inner-product loss without an act only): dW' of every chunk was formed
// beforehand by the reverse scan of ttt_linear.hip (dZ = 0, so the increments
// Q~^T dO of the dW chain do not depend on it); each workgroup then takes one
// (chain, column block, chunk), reads dW' from the workspace and forms the
// chunk's column-local terms only.
template <int DK, int LOSS, int ACT, int DECAY, bool SAVED, bool PAR = false>
__global__ __launch_bounds__(kSeqThreads) void ttt_bwd_seq_kernel(BwdArgs a, BwdWs ws, DecayPrep dp, SavedCtx sv) {
  static_assert(!PAR || (LOSS == 1 && ACT == 0), "chunk-parallel only without a state-dependent G");
  __shared__ __attribute__((aligned(16))) uint16_t KS[kCMax * DK];  // K~ [t][d]
  __shared__ __attribute__((aligned(16))) uint16_t QS[kCMax * DK];  // Q~ [t][d]; raw K late in the chunk (vector)
  __shared__ __attribute__((aligned(16))) uint16_t B1[kNB * kCMax];  // G~^T, then dY^T, then dZ^T  [n][t]
  __shared__ __attribute__((aligned(16))) uint16_t B3[kNB * DK];     // W_i^T, then (lambda dW')^T  [n][d]
  __shared__ float ETA[kCMax];
  __shared__ float LAM[DK];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int C = a.C, dv = a.dv, T = a.T;
  const int ncb = dv / kNB;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = PAR ? L / (ncb * a.NC) : L / ncb, cb = L % ncb;
  const int ci_par = PAR ? (L / ncb) % a.NC : 0;
  const int h = bh % a.H;
  const int col0 = cb * kNB;

  const int64_t offk = static_cast<int64_t>(bh) * T * DK;
  const int64_t offv = static_cast<int64_t>(bh) * T * dv;
  const bf16_t* q = static_cast<const bf16_t*>(a.q) + offk;
  const bf16_t* k = static_cast<const bf16_t*>(a.k) + offk;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + offv;
  const bf16_t* dO = static_cast<const bf16_t*>(a.d_o) + offv;
  bf16_t* dvo = static_cast<bf16_t*>(a.dv_out) + offv;
  bf16_t* wdY = ws.dY + offv;
  bf16_t* wGh = ws.Gh + offv;
  bf16_t* wdZ = ws.dZ + offv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * T;
  // staging sources: K~ = K, Q~ = Q unless vector decay prepared them
  const bf16_t* ksrc = (DECAY == 2) ? dp.kt + offk : k;
  const bf16_t* qsrc = (DECAY == 2) ? dp.qt + offk : q;
  float* deta_p = ws.deta_part + (static_cast<int64_t>(cb) * a.B * a.H + bh) * T;

  const bool has_w = w < DK / 32;
  float dW[16];  // dW' = dW_{i+1}: lane holds dW'[32 w + l32][col0 + row_of(r, hi)]
#pragma unroll
  for (int r = 0; r < 16; ++r) dW[r] = 0.0f;
  if (has_w && (PAR || a.d_wfinal)) {
    const int l32 = tid & 31, hi = (tid >> 5) & 1;
    const float* p = PAR ? ws.dWn + ((static_cast<int64_t>(bh) * a.NC + ci_par) * DK + 32 * w + l32) * dv + col0
                         : a.d_wfinal + (static_cast<int64_t>(bh) * DK + 32 * w + l32) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 x = *reinterpret_cast<const float4*>(p + 8 * r4 + 4 * hi);
      dW[4 * r4] = x.x; dW[4 * r4 + 1] = x.y; dW[4 * r4 + 2] = x.z; dW[4 * r4 + 3] = x.w;
    }
  }

  const int ntile = C / 32;
  const int X = tile_of_wave(w);  // this wave's token tile
  const bool own = X < ntile;

  uint32_t sink = 0;
  for (int ci = PAR ? ci_par : a.NC - 1; ci >= (PAR ? ci_par : 0); --ci) {
    const int t0 = ci * C;
    const int c = min(C, T - t0);
    const int lane = opaque(threadIdx.x & 63), l32 = lane & 31, hi = lane >> 5;
    const int dw = 32 * w + l32;
    const int t = 32 * X + l32;  // this lane's token in the own tile

    // (0) W_i from the checkpoint -> bf16 W^T in B3 (recompute path)
    if (!SAVED && has_w) {
      const float* p = a.w_ckpt + ((static_cast<int64_t>(bh) * a.NC + ci) * DK + dw) * dv + col0;
      float Wr[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 x = *reinterpret_cast<const float4*>(p + 8 * r4 + 4 * hi);
        Wr[4 * r4] = x.x; Wr[4 * r4 + 1] = x.y; Wr[4 * r4 + 2] = x.z; Wr[4 * r4 + 3] = x.w;
      }
      store_tile_t<DK>(B3, dw, hi, Wr);
    }
    // the saved own-tile rows (SAVED): issued before the staging so their latency
    // hides behind it -- dO and f'(Y) for dY; Z and V (with an act) or G~ for the epilogue
    uint4 sv_do[2], sv_fy[2], sv_gh[2], sv_z[2], sv_v[2];
    if constexpr (SAVED) {
      load_row32(sv_do, dO, dv, t0, t, c, col0, hi);
      if constexpr (ACT != 0) {
        load_row32(sv_fy, sv.dfy + offv, dv, t0, t, c, col0, hi);
        load_row32(sv_z, sv.z + offv, dv, t0, t, c, col0, hi);
        load_row32(sv_v, v, dv, t0, t, c, col0, hi);
      } else {
        load_row32(sv_gh, sv.gh + offv, dv, t0, t, c, col0, hi);
      }
    }
    // (1) stage eta, lambda, K~, Q~ (ends with a barrier)
    stage_chunk<DK, DECAY, kSeqThreads>(KS, QS, ETA, LAM, ksrc, qsrc,
                                        (DECAY == 2) ? dp.lam + (static_cast<int64_t>(bh) * a.NC + ci) * DK : nullptr,
                                        beta, a.b, DECAY == 1 ? a.gamma[h] : 1.0f, t0, c, C);

    float Zr[16];  // Z of the own tile (recomputed, or saved with an act)
    float dYr[16];
    uint2 doraw[4];
    if constexpr (!SAVED) {
    // own-tile operands from HBM: V and the raw keys of the train view (vector decay)
    uint2 vraw[4];
    bf16x8_t kraw[DK / 16];
    load_row16(vraw, v, dv, t0, t, c, col0, hi);
    if constexpr (DECAY == 2) load_row_frags<DK / 16>(kraw, k, DK, t0, t, c, 0, hi);

    // (2) train view: Z^T = W^T K^T, G~ -> B1 (G~^T) and the workspace
    if (own) {
      f32x16_t z = zero16();
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb) {
        const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(&B3[swz<DK>(l32, 16 * kb + 8 * hi)]);
        const bf16x8_t Bk = (DECAY == 2) ? kraw[kb]
                                         : *reinterpret_cast<const bf16x8_t*>(&KS[swz<DK>(t, 16 * kb + 8 * hi)]);
        z = mfma32(A, Bk, z);
      }
      const float et = ETA[t];
      float vv[16];
      unpack16(vraw, vv);
      float gh[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float zz = z[r];
        const float e = loss_signal<LOSS, ACT>(zz, vv[r]);
        Zr[r] = zz;
        gh[r] = et * e * act_df<ACT>(zz);
      }
      store_tile_t<kCMax>(B1, t, hi, gh);
      store_row16_x2(wGh, dv, t0, t, c, col0, hi, gh);
    }
    // dO of the own tile, needed after the query view is recomputed
    load_row16(doraw, dO, dv, t0, t, c, col0, hi);
    __syncthreads();

    }
    // L2 prefetch of the previous chunk (the next one of this reverse sweep)
    uint32_t pk[1] = {0}, pq[1] = {0}, pv[1] = {0}, pd[1] = {0}, pr[1] = {0}, pf[1] = {0}, pz[1] = {0};
    if (!PAR && ci > 0) {
      const int tp = t0 - C;
      l2_touch<1, kSeqThreads>(pk, ksrc + static_cast<int64_t>(tp) * DK, C * DK * 2, cb, ncb);
      l2_touch<1, kSeqThreads>(pq, qsrc + static_cast<int64_t>(tp) * DK, C * DK * 2, cb, ncb);
      l2_touch<1, kSeqThreads>(pv, v + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
      l2_touch<1, kSeqThreads>(pd, dO + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
      if constexpr (DECAY == 2)
        l2_touch<1, kSeqThreads>(pr, k + static_cast<int64_t>(tp) * DK, C * DK * 2, cb, ncb);
      if constexpr (SAVED && ACT != 0) {
        l2_touch<1, kSeqThreads>(pf, sv.dfy + offv + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
        l2_touch<1, kSeqThreads>(pz, sv.z + offv + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
      }
    }

    if constexpr (SAVED) {
      // dY = dO (.) f'(Y) from the saved f'(Y); no LDS is read, so no barrier before (4)
      float dd[16];
      {
        uint2 x[4];
        row32_frags(sv_do, x, t < c);
        unpack16(x, dd);
      }
      if constexpr (ACT != 0) {
        float ff[16];
        uint2 x[4];
        row32_frags(sv_fy, x, t < c);
        unpack16(x, ff);
#pragma unroll
        for (int r = 0; r < 16; ++r) dYr[r] = dd[r] * ff[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) dYr[r] = dd[r];
      }
      if (own) store_row16_x2(wdY, dv, t0, t, c, col0, hi, dYr);
    } else {
    // (3) query view again: Y^T = W^T Q~^T - G~^T Tril(S)^T; dY = dO (.) f'(Y)
    if (own) {
      bf16x8_t qf[DK / 16];
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb) qf[kb] = *reinterpret_cast<const bf16x8_t*>(&QS[swz<DK>(t, 16 * kb + 8 * hi)]);
      f32x16_t y = zero16();
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb)
        y = mfma32(*reinterpret_cast<const bf16x8_t*>(&B3[swz<DK>(l32, 16 * kb + 8 * hi)]), qf[kb], y);
      for (int J = 0; J <= X; ++J) {
        f32x16_t s = zero16();
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
          s = mfma32(*reinterpret_cast<const bf16x8_t*>(&KS[swz<DK>(32 * J + l32, 16 * kb + 8 * hi)]), qf[kb], s);
        if (J == X) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (row_of(r, hi) > l32) s[r] = 0.0f;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float nb[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) nb[jj] = -s[8 * m + jj];
          const int s0 = 32 * J + 16 * m + 4 * hi;
          const bf16x4_t g0 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, s0)]);
          const bf16x4_t g1 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, s0 + 8)]);
          y = mfma32(cat44(g0, g1), pack8(nb), y);
        }
      }
      float dd[16];
      unpack16(doraw, dd);
#pragma unroll
      for (int r = 0; r < 16; ++r) dYr[r] = dd[r] * act_df<ACT>(y[r]);
      store_row16_x2(wdY, dv, t0, t, c, col0, hi, dYr);
    }
    __syncthreads();

    }
    // (4) dY^T -> B1; (lambda dW')^T -> B3
    if (own) {
      store_tile_t<kCMax>(B1, t, hi, dYr);
    }
    if (has_w) {
      const float lam = (DECAY == 2) ? LAM[dw] : 1.0f;  // K_bar = K~ e^{L_last} (vector); K (otherwise)
      float ld[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ld[r] = lam * dW[r];
      store_tile_t<DK>(B3, dw, hi, ld);
    }
    __syncthreads();

    // (5) R = Q~^T dY  (lane holds R[dw][row_of(r, hi)])
    f32x16_t R = zero16();
    if (!PAR && has_w) {
      ColumnReaderTR<DK> qcol(QS, 32 * w, l32, hi);
      RowReader<kCMax> arow(B1, l32, hi);
      int kb0 = 0;
      for (; kb0 + 4 <= C / 16; kb0 += 4) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) R = mfma32(arow(kk), qcol(kk), R);
        qcol.advance();
        arow.advance();
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)  // the last, partial group (C = 32)
        if (kb0 + kk < C / 16) R = mfma32(arow(kk), qcol(kk), R);
    }

    // (6)-(7) dG~ for the own tile, then dG, dZ, dV and the deta partial
    float dZr[16];
    if (own) {
      const int J = X;
      const int s = t;
      f32x16_t acc = zero16();  // (dG~)^T tile: lane holds -dG~[s][row_of(r, hi)]
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb)
        acc = mfma32(*reinterpret_cast<const bf16x8_t*>(&B3[swz<DK>(l32, 16 * kb + 8 * hi)]),
                     *reinterpret_cast<const bf16x8_t*>(&KS[swz<DK>(s, 16 * kb + 8 * hi)]), acc);
      for (int I = J; I < ntile; ++I) {
        f32x16_t st = zero16();  // S_IJ: lane holds S[32I + row_of(r, hi)][s]
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
          st = mfma32(*reinterpret_cast<const bf16x8_t*>(&QS[swz<DK>(32 * I + l32, 16 * kb + 8 * hi)]),
                      *reinterpret_cast<const bf16x8_t*>(&KS[swz<DK>(s, 16 * kb + 8 * hi)]), st);
        if (I == J) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (row_of(r, hi) < l32) st[r] = 0.0f;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float sb[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) sb[jj] = st[8 * m + jj];
          const int u0 = 32 * I + 16 * m + 4 * hi;
          const bf16x4_t d0 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, u0)]);
          const bf16x4_t d1 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, u0 + 8)]);
          acc = mfma32(cat44(d0, d1), pack8(sb), acc);
        }
      }
      const float es = ETA[s];
      float part = 0.0f, dvv[16];
      if constexpr (SAVED && ACT == 0) {
        // G = G~ / eta; f' = 1 and dZ/dG = 1 (MSE) or 0 (IP) without an activation
        float gg[16];
        uint2 x[4];
        row32_frags(sv_gh, x, s < c);
        unpack16(x, gg);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dgh = -acc[r];
          part += dgh * gg[r];  // <dG~, G~>, divided by eta below
          const float dg = es * dgh;
          dZr[r] = (LOSS == 0) ? dg : 0.0f;
          dvv[r] = loss_dsignal_dv<LOSS>() * dg;
        }
        part *= (s < c) ? 1.0f / es : 0.0f;
      } else {
        // Z recomputed or saved; V again (L2-resident on the recompute path:
        // cheaper than keeping it in registers across the chunk)
        float vv[16];
        if constexpr (SAVED) {
          uint2 x[4];
          row32_frags(sv_z, x, s < c);
          unpack16(x, Zr);
          row32_frags(sv_v, x, s < c);
          unpack16(x, vv);
        } else {
          uint2 vre[4];
          load_row16(vre, v, dv, t0, s, c, col0, hi);
          unpack16(vre, vv);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dgh = -acc[r];
          const float zz = Zr[r];
          const float e = loss_signal<LOSS, ACT>(zz, vv[r]);
          const float f1 = act_df<ACT>(zz);
          part += dgh * e * f1;  // <dG~, G>
          const float dg = es * dgh;
          const float de = dg * f1;
          float dz = dg * e * act_d2f<ACT>(zz);
          if (LOSS == 0) dz += de * f1;
          dZr[r] = dz;
          dvv[r] = loss_dsignal_dv<LOSS>() * de;
        }
      }
      part += __shfl_xor(part, 32);
      if (s < c && hi == 0) deta_p[t0 + s] = part;
      store_row16_x2(dvo, dv, t0, s, c, col0, hi, dvv);
      store_row16_x2(wdZ, dv, t0, s, c, col0, hi, dZr);
    }
    __syncthreads();

    if constexpr (PAR) continue;  // the dW chain was formed by the reverse scan

    // (8) dZ^T -> B1; raw keys -> QS (vector decay: the train view used K, not K~)
    if (own) {
      store_tile_t<kCMax>(B1, t, hi, dZr);
    }
    if constexpr (DECAY == 2) stage_raw_k<DK, kSeqThreads>(QS, k, t0, c, C);
    __syncthreads();

    // (9)-(10) K^T dZ, the dW_{i+1} checkpoint, dW_i
    if (has_w) {
      const uint16_t* KR = (DECAY == 2) ? QS : KS;
      f32x16_t kz = zero16();
      ColumnReaderTR<DK> kcol(KR, 32 * w, l32, hi);
      RowReader<kCMax> arow(B1, l32, hi);
      int kb0 = 0;
      for (; kb0 + 4 <= C / 16; kb0 += 4) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kz = mfma32(arow(kk), kcol(kk), kz);
        kcol.advance();
        arow.advance();
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)  // the last, partial group (C = 32)
        if (kb0 + kk < C / 16) kz = mfma32(arow(kk), kcol(kk), kz);
      float* ck = ws.dWn + ((static_cast<int64_t>(bh) * a.NC + ci) * DK + dw) * dv + col0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<float4*>(ck + 8 * r4 + 4 * hi) =
            make_float4(dW[4 * r4], dW[4 * r4 + 1], dW[4 * r4 + 2], dW[4 * r4 + 3]);
      }
      const float lam = LAM[dw];
#pragma unroll
      for (int r = 0; r < 16; ++r) dW[r] = lam * dW[r] + R[r] + kz[r];
    }
    sink ^= pk[0] ^ pq[0] ^ pv[0] ^ pd[0] ^ pr[0] ^ pf[0] ^ pz[0];
    __syncthreads();
  }
  if (T < 0) ws.deta_part[0] = __uint_as_float(sink);  // never taken: keeps the prefetch loads alive
  if (!PAR && a.dw0 && has_w) {
    const int l32 = tid & 31, hi = (tid >> 5) & 1;
    float* p = a.dw0 + (static_cast<int64_t>(bh) * DK + 32 * w + l32) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(p + 8 * r4 + 4 * hi) = make_float4(dW[4 * r4], dW[4 * r4 + 1], dW[4 * r4 + 2], dW[4 * r4 + 3]);
  }
}

// ============================================================================
// bwd_seq, vector decay (tile-relative)
// ============================================================================
// The reverse sweep of ttt_fwd_vec_kernel: with the tile-relative Q^m, K^m and
// the tile-boundary prefixes P_I of the preparation kernel, the terms of dG~
// that reach key tile J from later query tiles and from the transition regroup
// into one d_k x 32 state per tile,
//   Xi_last = mu dW',   Xi_{J-1} = rho_J (Xi_J + R_J),   R_J = Q^m_J^T dY_J,
//   dG~_J = -K^m_J Xi_J - Tril(Q^m_J K^m_J^T)^T dY_J,
//   dW_i = rho_0 (Xi_0 + R_0) + K^T dZ    (= lambda dW' + Q~^T dY + K^T dZ),
// with rho_J = e^{M_J - M_{J-1}}, rho_0 = e^{M_0}, mu = e^{L_last - M_last}, all
// <= 1.  The waves that carry dW' run the reverse recurrence (two MFMAs per
// tile; the bf16 states Xi_J^T go to LDS) while every wave forms its diagonal
// tile; then each wave reads its state Xi_J.
// SAVED: G~, f'(Y) and Z come from the forward's saved context; otherwise the
// chunk's forward (train view, tile recurrence of the states X_I, Y) is
// recomputed from the checkpoint W_i first.
template <int DK, int LOSS, int ACT, bool SAVED, bool PAR = false>
__global__ __launch_bounds__(kSeqThreads) void ttt_bwd_seq_vec_kernel(BwdArgs a, BwdWs ws, DecayPrep dp, SavedCtx sv) {
  static_assert(!PAR || (LOSS == 1 && ACT == 0), "chunk-parallel only without a state-dependent G");
  constexpr int kNT = kCMax / 32;
  __shared__ __attribute__((aligned(16))) uint16_t QS[kCMax * DK];        // K^m, then Q^m, then raw K [t][d]
  __shared__ __attribute__((aligned(16))) uint16_t XI[kNT * DK * kNB];    // X_I / Xi_J [tile][d][n]
  __shared__ __attribute__((aligned(16))) uint16_t B1[kNB * kCMax];       // G~^T, then dY^T, then dZ^T [n][t]
  __shared__ __attribute__((aligned(16))) uint16_t B3[SAVED ? 8 : DK * kNB];  // W_i [d][n] (recompute)
  __shared__ float ETA[kCMax];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int C = a.C, dv = a.dv, T = a.T;
  const int ncb = dv / kNB;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = PAR ? L / (ncb * a.NC) : L / ncb, cb = L % ncb;
  const int ci_par = PAR ? (L / ncb) % a.NC : 0;
  const int col0 = cb * kNB;
  const int ntile = C / 32;

  const int64_t offk = static_cast<int64_t>(bh) * T * DK;
  const int64_t offv = static_cast<int64_t>(bh) * T * dv;
  const bf16_t* k = static_cast<const bf16_t*>(a.k) + offk;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + offv;
  const bf16_t* dO = static_cast<const bf16_t*>(a.d_o) + offv;
  bf16_t* dvo = static_cast<bf16_t*>(a.dv_out) + offv;
  bf16_t* wdY = ws.dY + offv;
  bf16_t* wGh = ws.Gh + offv;
  bf16_t* wdZ = ws.dZ + offv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * T;
  const bf16_t* ksrc = dp.kt + offk;  // K^m
  const bf16_t* qsrc = dp.qt + offk;  // Q^m
  const float* lpsrc = dp.lpre + static_cast<int64_t>(bh) * a.NC * (ntile + 1) * DK;
  float* deta_p = ws.deta_part + (static_cast<int64_t>(cb) * a.B * a.H + bh) * T;

  const bool has_w = w < DK / 32;
  float dW[16];  // dW' = dW_{i+1}: lane holds dW'[32 w + l32][col0 + row_of(r, hi)]
#pragma unroll
  for (int r = 0; r < 16; ++r) dW[r] = 0.0f;
  if (has_w && (PAR || a.d_wfinal)) {
    const int l32 = tid & 31, hi = (tid >> 5) & 1;
    const float* p = PAR ? ws.dWn + ((static_cast<int64_t>(bh) * a.NC + ci_par) * DK + 32 * w + l32) * dv + col0
                         : a.d_wfinal + (static_cast<int64_t>(bh) * DK + 32 * w + l32) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 x = *reinterpret_cast<const float4*>(p + 8 * r4 + 4 * hi);
      dW[4 * r4] = x.x; dW[4 * r4 + 1] = x.y; dW[4 * r4 + 2] = x.z; dW[4 * r4 + 3] = x.w;
    }
  }

  const int X = tile_of_wave(w);  // this wave's token tile
  const bool own = X < ntile;

  uint32_t sink = 0;
  for (int ci = PAR ? ci_par : a.NC - 1; ci >= (PAR ? ci_par : 0); --ci) {
    const int t0 = ci * C;
    const int c = min(C, T - t0);
    const int lane = opaque(threadIdx.x & 63), l32 = lane & 31, hi = lane >> 5;
    const int dw = 32 * w + l32;
    const int t = 32 * X + l32;  // this lane's token in the own tile

    // tile prefixes P_0 .. P_ntile of the state rows
    float pl[kNT + 1];
    {
      const float* lp = lpsrc + static_cast<int64_t>(ci) * (ntile + 1) * DK + (has_w ? dw : 0);
#pragma unroll
      for (int j = 0; j <= kNT; ++j) pl[j] = lp[min(j, ntile) * DK];
    }
    // the own tile's K^m rows (B operand of the diagonal scores and of K^m Xi);
    // on the recompute path they are loaded after the forward's recompute
    bf16x8_t kmf[DK / 16];
    if constexpr (SAVED) load_row_frags<DK / 16>(kmf, ksrc, DK, t0, t, c, 0, hi);

    // saved own-tile rows, issued before the staging so their latency hides behind it
    uint4 sv_do[2], sv_fy[2], sv_gh[2], sv_z[2], sv_v[2];
    if constexpr (SAVED) {
      load_row32(sv_do, dO, dv, t0, t, c, col0, hi);
      if constexpr (ACT != 0) {
        load_row32(sv_fy, sv.dfy + offv, dv, t0, t, c, col0, hi);
        load_row32(sv_z, sv.z + offv, dv, t0, t, c, col0, hi);
        load_row32(sv_v, v, dv, t0, t, c, col0, hi);
      } else {
        load_row32(sv_gh, sv.gh + offv, dv, t0, t, c, col0, hi);
      }
    }

    float Zr[16];
    float dYr[16];
    if constexpr (!SAVED) {
      // ---- recompute the chunk's forward: train view, tile states, Y ----
      float Xs[16];  // X_0 = rho_0 W_i, then the later tile states
      if (has_w) {
        const float* p = a.w_ckpt + ((static_cast<int64_t>(bh) * a.NC + ci) * DK + dw) * dv + col0;
        float Wr[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float4 x = *reinterpret_cast<const float4*>(p + 8 * r4 + 4 * hi);
          Wr[4 * r4] = x.x; Wr[4 * r4 + 1] = x.y; Wr[4 * r4 + 2] = x.z; Wr[4 * r4 + 3] = x.w;
        }
        store_tile_rows<kNB>(B3, dw, hi, Wr);
        const float rho0 = __expf(0.5f * pl[1]);  // e^{M_0}, P_0 = 0
#pragma unroll
        for (int r = 0; r < 16; ++r) Xs[r] = rho0 * Wr[r];
        store_tile_rows<kNB>(XI, dw, hi, Xs);
      }
      uint4 vraw[2];
      bf16x8_t kraw[DK / 16], qf[DK / 16];
      load_row32(vraw, v, dv, t0, t, c, col0, hi);
      load_row_frags<DK / 16>(kraw, k, DK, t0, t, c, 0, hi);
      load_row_frags<DK / 16>(qf, qsrc, DK, t0, t, c, 0, hi);
      uint2 doraw[4];
      load_row16(doraw, dO, dv, t0, t, c, col0, hi);
      // K^m -> QS (the states' recurrence and the diagonal scores read it), eta
      stage_raw_k<DK, kSeqThreads>(QS, ksrc, t0, c, C);
      if (tid < C) ETA[tid] = (tid < c) ? lr_gate(beta[t0 + min(tid, c - 1)], a.b) : 0.0f;
      __syncthreads();

      // train view: Z^T = W^T K^T, G~ -> B1 (G~^T) and the workspace
      if (own) {
        f32x16_t z = zero16();
        ColumnReaderTR<kNB> wcol(B3, 0, l32, hi);  // A = W^T
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb) z = mfma32(wcol(kb), kraw[kb], z);
        const float et = ETA[t];
        float vv[16];
        {
          uint2 vx[4];
          row32_frags(vraw, vx, t < c);
          unpack16(vx, vv);
        }
        float gh[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float zz = z[r];
          Zr[r] = zz;
          gh[r] = et * loss_signal<LOSS, ACT>(zz, vv[r]) * act_df<ACT>(zz);
        }
        store_tile_t<kCMax>(B1, t, hi, gh);
        store_row16_x2(wGh, dv, t0, t, c, col0, hi, gh);
      }
      __syncthreads();

      // diagonal tile of the query view, and the states X_1 .. X_{ntile-1}
      f32x16_t y = zero16();
      if (own) {
        f32x16_t sc = zero16();
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
          sc = mfma32(*reinterpret_cast<const bf16x8_t*>(&QS[swz<DK>(32 * X + l32, 16 * kb + 8 * hi)]), qf[kb], sc);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (row_of(r, hi) > l32) sc[r] = 0.0f;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float nb[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) nb[jj] = -sc[8 * m + jj];
          const int s0 = 32 * X + 16 * m + 4 * hi;
          const bf16x4_t g0 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, s0)]);
          const bf16x4_t g1 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, s0 + 8)]);
          y = mfma32(cat44(g0, g1), pack8(nb), y);
        }
      }
      if (has_w) {
        ColumnReaderTR<DK> kcol(QS, 32 * w, l32, hi);
        RowReader<kCMax> arow(B1, l32, hi);
        static_for<kNT - 1>([&](auto Ic) {
          constexpr int Ti = Ic;
          if (Ti + 1 < ntile) {
            f32x16_t u = zero16();
            constexpr int k0 = 2 * (Ti & 1);
            u = mfma32(arow(k0), kcol(k0), u);
            u = mfma32(arow(k0 + 1), kcol(k0 + 1), u);
            if constexpr ((Ti & 1) == 1) {
              kcol.advance();
              arow.advance();
            }
            // rho_{I+1} = e^{-h_I} e^{-h_{I+1}}, one factor at a time (ttt_fwd_vec_kernel)
            const float f1 = __expf(0.5f * (pl[Ti + 1] - pl[Ti]));
            const float f2 = __expf(0.5f * (pl[Ti + 2] - pl[Ti + 1]));
#pragma unroll
            for (int r = 0; r < 16; ++r) Xs[r] = f2 * (f1 * (Xs[r] - u[r]));
            store_tile_rows<kNB>(XI + (Ti + 1) * DK * kNB, dw, hi, Xs);
          }
        });
      }
      __syncthreads();
      if (own) {
        ColumnReaderTR<kNB> xcol(XI + X * DK * kNB, 0, l32, hi);  // A = X_X^T
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb) y = mfma32(xcol(kb), qf[kb], y);
        float dd[16];
        unpack16(doraw, dd);
#pragma unroll
        for (int r = 0; r < 16; ++r) dYr[r] = dd[r] * act_df<ACT>(y[r]);
        store_row16_x2(wdY, dv, t0, t, c, col0, hi, dYr);
      }
      __syncthreads();  // every read of QS (K^m), B1 (G~^T) and XI (X_I) is done
      load_row_frags<DK / 16>(kmf, ksrc, DK, t0, t, c, 0, hi);
      stage_raw_k<DK, kSeqThreads>(QS, qsrc, t0, c, C);  // Q^m -> QS
    } else {
      stage_raw_k<DK, kSeqThreads>(QS, qsrc, t0, c, C);  // Q^m -> QS
      if (tid < C) ETA[tid] = (tid < c) ? lr_gate(beta[t0 + min(tid, c - 1)], a.b) : 0.0f;
      // dY = dO (.) f'(Y) from the saved f'(Y)
      float dd[16];
      {
        uint2 x[4];
        row32_frags(sv_do, x, t < c);
        unpack16(x, dd);
      }
      if constexpr (ACT != 0) {
        float ff[16];
        uint2 x[4];
        row32_frags(sv_fy, x, t < c);
        unpack16(x, ff);
#pragma unroll
        for (int r = 0; r < 16; ++r) dYr[r] = dd[r] * ff[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) dYr[r] = dd[r];
      }
      if (own) store_row16_x2(wdY, dv, t0, t, c, col0, hi, dYr);
    }
    // dY^T -> B1
    if (own) store_tile_t<kCMax>(B1, t, hi, dYr);
    __syncthreads();

    // L2 prefetch of the previous chunk (the next one of this reverse sweep)
    uint32_t pk[1] = {0}, pq[1] = {0}, pv[1] = {0}, pd[1] = {0}, pr[1] = {0}, pf[1] = {0}, pz[1] = {0};
    if (!PAR && ci > 0) {
      const int tp = t0 - C;
      l2_touch<1, kSeqThreads>(pk, ksrc + static_cast<int64_t>(tp) * DK, C * DK * 2, cb, ncb);
      l2_touch<1, kSeqThreads>(pq, qsrc + static_cast<int64_t>(tp) * DK, C * DK * 2, cb, ncb);
      l2_touch<1, kSeqThreads>(pv, v + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
      l2_touch<1, kSeqThreads>(pd, dO + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
      l2_touch<1, kSeqThreads>(pr, k + static_cast<int64_t>(tp) * DK, C * DK * 2, cb, ncb);
      if constexpr (SAVED && ACT != 0) {
        l2_touch<1, kSeqThreads>(pf, sv.dfy + offv + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
        l2_touch<1, kSeqThreads>(pz, sv.z + offv + static_cast<int64_t>(tp) * dv, C * dv * 2, cb, ncb);
      }
    }

    f32x16_t acc = zero16();  // (dG~)^T tile: lane holds -dG~[s][row_of(r, hi)]
    // the reverse recurrence of the states Xi_J (dW' rows): Xi_J^T -> XI[J]
    float Xi[16];
    if (has_w) {
      ColumnReaderTR<DK> qcol(QS, 32 * w, l32, hi);
      RowReader<kCMax> arow(B1, l32, hi);
      // mu = e^{L_last - M_{ntile-1}} = e^{(P_nt - P_{nt-1}) / 2}
      float mu = 1.0f;
      static_for<kNT>([&](auto Ic) {
        constexpr int Ti = Ic;
        if (Ti + 1 == ntile) mu = __expf(0.5f * (pl[Ti + 1] - pl[Ti]));
      });
#pragma unroll
      for (int r = 0; r < 16; ++r) Xi[r] = mu * dW[r];
      static_for<kNT>([&](auto jc) {
        constexpr int J = kNT - 1 - jc;
        if (J < ntile) {
          store_tile_rows<kNB>(XI + J * DK * kNB, dw, hi, Xi);
          f32x16_t rr = zero16();  // R_J = Q^m_J^T dY_J: lane holds R[dw][row_of(r, hi)]
          constexpr int ks = 2 * J;
          rr = mfma32(arow.at(ks), qcol(ks), rr);
          rr = mfma32(arow.at(ks + 1), qcol(ks + 1), rr);
          // rho_J = e^{-h_J} e^{-h_{J-1}} (rho_0 = e^{-h_0}), h_J = (P_J - P_{J+1}) / 2,
          // applied one factor at a time: R_J carries up to e^{h_J} (Q^m), and rho
          // itself can leave the fp32 range where neither factor does
          const float f1 = __expf(0.5f * (pl[J + 1] - pl[J]));
#pragma unroll
          for (int r = 0; r < 16; ++r) Xi[r] = f1 * (Xi[r] + rr[r]);
          if constexpr (J > 0) {
            const float f2 = __expf(0.5f * (pl[J] - pl[J > 0 ? J - 1 : 0]));
#pragma unroll
            for (int r = 0; r < 16; ++r) Xi[r] *= f2;
          }
        }
      });
      // Xi = rho_0 (Xi_0 + R_0) = lambda dW' + Q~^T dY
    }
    // diagonal part of dG~ for the own key tile: Tril(S_XX)^T dY_X  (lane (s, hi)); after
    // the recurrence on the waves that run it (the longer chain), at once on the others
    if (own) {
      f32x16_t st = zero16();  // S: lane holds S[32 X + row_of(r, hi)][s]
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb)
        st = mfma32(*reinterpret_cast<const bf16x8_t*>(&QS[swz<DK>(32 * X + l32, 16 * kb + 8 * hi)]), kmf[kb], st);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (row_of(r, hi) < l32) st[r] = 0.0f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float sb[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sb[jj] = st[8 * m + jj];
        const int u0 = 32 * X + 16 * m + 4 * hi;
        const bf16x4_t d0 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, u0)]);
        const bf16x4_t d1 = *reinterpret_cast<const bf16x4_t*>(&B1[swz<kCMax>(l32, u0 + 8)]);
        acc = mfma32(cat44(d0, d1), pack8(sb), acc);
      }
    }
    __syncthreads();  // every Xi_J is in XI; every read of B1 (dY^T) and QS (Q^m) is done

    // dG~ of the own key tile: += K^m_X Xi_X, then dG, dZ, dV and the deta partial
    float dZr[16];
    if (own) {
      const int s = t;
      ColumnReaderTR<kNB> xcol(XI + X * DK * kNB, 0, l32, hi);  // A = Xi_X^T
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb) acc = mfma32(xcol(kb), kmf[kb], acc);
      const float es = ETA[s];
      float part = 0.0f, dvv[16];
      if constexpr (SAVED && ACT == 0) {
        float gg[16];
        uint2 x[4];
        row32_frags(sv_gh, x, s < c);
        unpack16(x, gg);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dgh = -acc[r];
          part += dgh * gg[r];
          const float dg = es * dgh;
          dZr[r] = (LOSS == 0) ? dg : 0.0f;
          dvv[r] = loss_dsignal_dv<LOSS>() * dg;
        }
        part *= (s < c) ? 1.0f / es : 0.0f;
      } else {
        float vv[16];
        if constexpr (SAVED) {
          uint2 x[4];
          row32_frags(sv_z, x, s < c);
          unpack16(x, Zr);
          row32_frags(sv_v, x, s < c);
          unpack16(x, vv);
        } else {
          uint2 vre[4];
          load_row16(vre, v, dv, t0, s, c, col0, hi);
          unpack16(vre, vv);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dgh = -acc[r];
          const float zz = Zr[r];
          const float e = loss_signal<LOSS, ACT>(zz, vv[r]);
          const float f1 = act_df<ACT>(zz);
          part += dgh * e * f1;
          const float dg = es * dgh;
          const float de = dg * f1;
          float dz = dg * e * act_d2f<ACT>(zz);
          if (LOSS == 0) dz += de * f1;
          dZr[r] = dz;
          dvv[r] = loss_dsignal_dv<LOSS>() * de;
        }
      }
      part += __shfl_xor(part, 32);
      if (s < c && hi == 0) deta_p[t0 + s] = part;
      store_row16_x2(dvo, dv, t0, s, c, col0, hi, dvv);
      store_row16_x2(wdZ, dv, t0, s, c, col0, hi, dZr);
      store_tile_t<kCMax>(B1, t, hi, dZr);  // dZ^T (every read of dY^T is behind the barrier)
    }
    if constexpr (PAR) continue;  // dZ = 0, and the dW chain was formed by the reverse scan
    stage_raw_k<DK, kSeqThreads>(QS, k, t0, c, C);  // raw K -> QS
    __syncthreads();

    // K^T dZ, the dW_{i+1} checkpoint, dW_i
    if (has_w) {
      f32x16_t kz = zero16();
      ColumnReaderTR<DK> kcol(QS, 32 * w, l32, hi);
      RowReader<kCMax> arow(B1, l32, hi);
      int kb0 = 0;
      for (; kb0 + 4 <= C / 16; kb0 += 4) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kz = mfma32(arow(kk), kcol(kk), kz);
        kcol.advance();
        arow.advance();
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (kb0 + kk < C / 16) kz = mfma32(arow(kk), kcol(kk), kz);
      float* ck = ws.dWn + ((static_cast<int64_t>(bh) * a.NC + ci) * DK + dw) * dv + col0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(ck + 8 * r4 + 4 * hi) =
            make_float4(dW[4 * r4], dW[4 * r4 + 1], dW[4 * r4 + 2], dW[4 * r4 + 3]);
#pragma unroll
      for (int r = 0; r < 16; ++r) dW[r] = Xi[r] + kz[r];
    }
    sink ^= pk[0] ^ pq[0] ^ pv[0] ^ pd[0] ^ pr[0] ^ pf[0] ^ pz[0];
    __syncthreads();
  }
  if (T < 0) ws.deta_part[0] = __uint_as_float(sink);
  if (!PAR && a.dw0 && has_w) {
    const int l32 = tid & 31, hi = (tid >> 5) & 1;
    float* p = a.dw0 + (static_cast<int64_t>(bh) * DK + 32 * w + l32) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(p + 8 * r4 + 4 * hi) = make_float4(dW[4 * r4], dW[4 * r4 + 1], dW[4 * r4 + 2], dW[4 * r4 + 3]);
  }
}

// ============================================================================
// bwd_cross
// ============================================================================
// In-tile scans along the tokens of a 32 x 32 MFMA output held as
// lane (col = l32, hi): rows row_of(r, hi) = 8*(r/4) + 4*hi + r%4.
// The partner lane (l ^ 32) holds the other four rows of every group of eight.
__device__ __forceinline__ void tile_inclusive_prefix(float (&x)[16], int hi) {
  float gs[4], og[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    gs[q] = x[4 * q] + x[4 * q + 1] + x[4 * q + 2] + x[4 * q + 3];
    og[q] = __shfl_xor(gs[q], 32);
  }
  float base = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float b = base + (hi ? og[q] : 0.0f);
    float run = b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      run += x[4 * q + e];
      x[4 * q + e] = run;
    }
    base += gs[q] + og[q];
  }
}
__device__ __forceinline__ void tile_inclusive_suffix(float (&x)[16], int hi) {
  float gs[4], og[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    gs[q] = x[4 * q] + x[4 * q + 1] + x[4 * q + 2] + x[4 * q + 3];
    og[q] = __shfl_xor(gs[q], 32);
  }
  float base = 0.0f;
#pragma unroll
  for (int q = 3; q >= 0; --q) {
    float b = base + (hi ? 0.0f : og[q]);
    float run = b;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      run += x[4 * q + e];
      x[4 * q + e] = run;
    }
    base += gs[q] + og[q];
  }
}

template <int DK, int DV, int DECAY>
__global__ __launch_bounds__(kCrossThreads) void ttt_bwd_cross_kernel(BwdArgs a, BwdWs ws, DecayPrep dp) {
  __shared__ __attribute__((aligned(16))) uint16_t GH[kCMax * DV];   // G~ [s][n]
  __shared__ __attribute__((aligned(16))) uint16_t KT[kDB * kCMax];  // K~^T [d][t] (this d-block)
  __shared__ __attribute__((aligned(16))) uint16_t QT[kDB * kCMax];  // Q~^T [d][t]
  __shared__ float ETA[kCMax];
  __shared__ float LP[9 * kDB];    // vector: P_0 .. P_{C/32}, L at the 32-token tile boundaries
  __shared__ float HF[8 * kDB];    // vector: e^{-h_I} = e^{(P_{I+1} - P_I) / 2}, half of tile I's decay
  __shared__ float TOT[8 * kDB];   // per tile: dL tile totals
  __shared__ float KKB[8 * kDB];   // per wave: sum_s dK_bar (.) K_bar over its tile
  __shared__ float DLAM[kDB];      // <dW', W_i> of each row (vector decay)
  __shared__ __attribute__((aligned(16))) uint16_t WB[kDB * DV];     // bf16 W_i rows of the d-block [d][n]

  constexpr int NDB = DK / kDB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int C = a.C, T = a.T;
  const int Lb = xcd_remap(blockIdx.x, gridDim.x);
  const int db = Lb % NDB;
  const int ci = (Lb / NDB) % a.NC;
  const int bh = Lb / (NDB * a.NC);
  const int d0 = db * kDB;
  const int t0 = ci * C;
  const int c = min(C, T - t0);
  const int ntile = C / 32;
  const int ncb = DV / kNB;

  const int64_t offk = static_cast<int64_t>(bh) * T * DK;
  const int64_t offv = static_cast<int64_t>(bh) * T * DV;
  const bf16_t* q = static_cast<const bf16_t*>(a.q) + offk;
  const bf16_t* k = static_cast<const bf16_t*>(a.k) + offk;
  const float* la = (DECAY == 2) ? a.log_decay + offk : nullptr;
  const bf16_t* gdY = ws.dY + offv;
  const bf16_t* gGh = ws.Gh + offv;
  const bf16_t* gdZ = ws.dZ + offv;
  const float* Wc = a.w_ckpt + (static_cast<int64_t>(bh) * a.NC + ci) * DK * DV;
  const float* dWc = ws.dWn + (static_cast<int64_t>(bh) * a.NC + ci) * DK * DV;
  bf16_t* dqo = static_cast<bf16_t*>(a.dq) + offk;
  bf16_t* dko = static_cast<bf16_t*>(a.dk_out) + offk;

  // ---------------- staging ----------------
  // Every global load of the prologue is issued first (one round trip), then
  // the LDS writes: with one workgroup per CU this latency is not hidden.
  //  * WB: the d-block's rows of dW' and then of W_i pass through WB as bf16,
  //    read once per workgroup instead of by every wave: dW' first (for dK_bar),
  //    then W_i (for dY W^T and dZ W^T), held in registers until then.
  //  * GH: G~ rows; KT, QT: K~^T, Q~^T of the d-block (thread = (matrix, 8-token
  //    slice, 8-feature group); the transposition happens in registers).
  constexpr int kWG = DV / 8;                                   // 16-byte pieces per row
  constexpr int kWU = (kDB * kWG + kCrossThreads - 1) / kCrossThreads;
  constexpr int kGG = DV / 8;
  constexpr int kGU = (kCMax * kGG + kCrossThreads - 1) / kCrossThreads;
  float4 wreg[kWU][2], dwreg[kWU][2];
  uint4 gg[kGU], kq[8];
  float beta_t = 0.0f, lp_v = 0.0f, lp_n = 0.0f, lc_v = 0.0f;
  const int kq_m = tid >> 8, kq_sl = (tid >> 3) & 31, kq_g = tid & 7;  // matrix, slice, group
  {
#pragma unroll
    for (int u = 0; u < kWU; ++u) {
      const int idx = u * kCrossThreads + tid;
      const bool ok = idx < kDB * kWG;
      const int64_t off = static_cast<int64_t>(d0 + (ok ? idx / kWG : 0)) * DV + 8 * (ok ? idx % kWG : 0);
      dwreg[u][0] = *reinterpret_cast<const float4*>(dWc + off);
      dwreg[u][1] = *reinterpret_cast<const float4*>(dWc + off + 4);
      wreg[u][0] = *reinterpret_cast<const float4*>(Wc + off);
      wreg[u][1] = *reinterpret_cast<const float4*>(Wc + off + 4);
    }
#pragma unroll
    for (int u = 0; u < kGU; ++u) {
      const int idx = u * kCrossThreads + tid;
      const int t = idx / kGG;
      const bool ok = t < c;
      gg[u] = *reinterpret_cast<const uint4*>(gGh + static_cast<int64_t>(t0 + (ok ? t : 0)) * DV + 8 * (ok ? idx % kGG : 0));
    }
    const bf16_t* src = (kq_m == 0) ? ((DECAY == 2) ? dp.kt + offk : k) : ((DECAY == 2) ? dp.qt + offk : q);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = 8 * kq_sl + u;
      const bool ok = t < c;
      kq[u] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(t0 + (ok ? t : 0)) * DK + d0 + 8 * kq_g);
    }
    if (tid < C) beta_t = a.beta[static_cast<int64_t>(bh) * T + t0 + min(tid, c - 1)];
    if constexpr (DECAY == 2) {
      const int64_t pc = static_cast<int64_t>(bh) * a.NC + ci;
      const float* lp = dp.lpre + pc * (ntile + 1) * DK + d0;
      if (tid < ntile * kDB) {
        lp_v = lp[(tid / kDB) * DK + tid % kDB];
        lp_n = lp[(tid / kDB + 1) * DK + tid % kDB];
      }
      if (tid < kDB) lc_v = lp[ntile * DK + tid];  // P_ntile = L_last
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    // dlambda = <dW', W_i> per row (scalar and vector decay): the kWG consecutive
    // lanes that hold a row's 16-byte pieces reduce it by shuffles
    if constexpr (DECAY != 0) {
#pragma unroll
      for (int u = 0; u < kWU; ++u) {
        const int idx = u * kCrossThreads + tid;
        float dot = dwreg[u][0].x * wreg[u][0].x + dwreg[u][0].y * wreg[u][0].y + dwreg[u][0].z * wreg[u][0].z +
                    dwreg[u][0].w * wreg[u][0].w + dwreg[u][1].x * wreg[u][1].x + dwreg[u][1].y * wreg[u][1].y +
                    dwreg[u][1].z * wreg[u][1].z + dwreg[u][1].w * wreg[u][1].w;
#pragma unroll
        for (int m = 1; m < kWG; m <<= 1) dot += __shfl_xor(dot, m);
        if (idx < kDB * kWG && idx % kWG == 0) {
          if constexpr (DECAY == 2)
            DLAM[idx / kWG] = dot;
          else
            ws.dlam_part[(static_cast<int64_t>(bh) * a.NC + ci) * DK + d0 + idx / kWG] = dot;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kWU; ++u) {
      const int idx = u * kCrossThreads + tid;
      if (idx < kDB * kWG) {
        const float f[8] = {dwreg[u][0].x, dwreg[u][0].y, dwreg[u][0].z, dwreg[u][0].w,
                            dwreg[u][1].x, dwreg[u][1].y, dwreg[u][1].z, dwreg[u][1].w};
        *reinterpret_cast<bf16x8_t*>(&WB[swz<DV>(idx / kWG, 8 * (idx % kWG))]) = pack8(f);
      }
    }
#pragma unroll
    for (int u = 0; u < kGU; ++u) {
      const int idx = u * kCrossThreads + tid;
      const int t = idx / kGG;
      if (t < C) *reinterpret_cast<uint4*>(&GH[swz<DV>(t, 8 * (idx % kGG))]) = mask4(gg[u], okmask(t < c));
    }
    if (8 * kq_sl < C) {
      // transposed writes: feature d = 8 g + j, tokens 8 sl .. 8 sl + 7 (16 bytes)
      uint16_t* dst = (kq_m == 0) ? KT : QT;
      uint16_t hb[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint4 km = mask4(kq[u], okmask(8 * kq_sl + u < c));
        const uint32_t kw[4] = {km.x, km.y, km.z, km.w};
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          hb[2 * j2][u] = static_cast<uint16_t>(kw[j2] & 0xffffu);
          hb[2 * j2 + 1][u] = static_cast<uint16_t>(kw[j2] >> 16);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint4 r;
        r.x = hb[j][0] | (static_cast<uint32_t>(hb[j][1]) << 16);
        r.y = hb[j][2] | (static_cast<uint32_t>(hb[j][3]) << 16);
        r.z = hb[j][4] | (static_cast<uint32_t>(hb[j][5]) << 16);
        r.w = hb[j][6] | (static_cast<uint32_t>(hb[j][7]) << 16);
        *reinterpret_cast<uint4*>(&dst[swz<kCMax>(8 * kq_g + j, 8 * kq_sl)]) = r;
      }
    }
    if (tid < C) ETA[tid] = (tid < c) ? lr_gate(beta_t, a.b) : 0.0f;
    if constexpr (DECAY == 2) {
      if (tid < ntile * kDB) {
        LP[tid] = lp_v;
        HF[tid] = __expf(0.5f * (lp_n - lp_v));
      }
      if (tid < kDB) LP[ntile * kDB + tid] = lc_v;
    }
  }
  __syncthreads();

  // ---------------- per own tile: dQ~ and the three parts of dK ----------------
  const int X = tile_of_wave(w);  // this wave's token tile
  const bool own = X < ntile;
  constexpr int NK = DV / 16;

  float dL[2][16];  // [d-tile][r]  (vector decay)
  const int tx = 32 * X + l32;
  bf16x8_t dyf[NK];
  f32x16_t E[2];
  if (own) {
    load_row_frags<NK>(dyf, gdY, DV, t0, tx, c, 0, hi);

    // (a) E = dK~ + lambda (.) dK_bar (only that sum reaches dk and dL), started from
    //     lambda (.) dK_bar = -lambda (.) G~ dW'^T, then += dS^T Q~ over query tiles
    //     I >= X (dS = -Tril(dY G~^T)); the dY rows of the next tile are fetched
    //     while the current one is multiplied.
    //     Vector decay, tile-relative (K^m, Q^m of ttt_decay_prep.hip): the keys of
    //     tile X see query tile I >= X through e^{M_I - M_X} <= 1 per feature, and
    //     the transition through c_X = e^{L_last - M_X}; with the query tiles taken
    //     in descending order and the running sum scaled by rho_{I+1} =
    //     e^{M_{I+1} - M_I} before tile I is added (a Horner scheme over tiles),
    //     E = sum_I e^{M_I - M_X} dS_IX^T Q^m_I + c_X dK_bar starts from
    //     mu dK_bar, mu = e^{L_last - M_{last tile}}, and every factor stays <= 1;
    //     dk = dK_z + e^{M_X - L} (.) E.
    {
      f32x16_t dkb[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) dkb[dt] = zero16();
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        const bf16x8_t gf = *reinterpret_cast<const bf16x8_t*>(&GH[swz<DV>(tx, 16 * kb + 8 * hi)]);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
          dkb[dt] = mfma32(gf, *reinterpret_cast<const bf16x8_t*>(&WB[swz<DV>(32 * dt + l32, 16 * kb + 8 * hi)]),
                           dkb[dt]);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int dl = 32 * dt + l32;
        // vector: c_X = e^{L_last - M_X} (K_bar = K^m c_X on tile X) and the start
        // value mu = e^{L_last - M_{ntile-1}}; otherwise lambda = 1 or gamma
        // enters through dlambda only
        // (c_X = e^{-h_X} e^{P_nt - P_{X+1}} as two factors, h_X = (P_X - P_{X+1}) / 2:
        // K^m carries up to e^{h_X}, and c_X alone can leave the fp32 range)
        float lc1 = 1.0f, lc2 = 1.0f, mu = 1.0f;
        if constexpr (DECAY == 2) {
          const float pl = LP[ntile * kDB + dl];
          lc1 = HF[X * kDB + dl];
          lc2 = __expf(pl - LP[(X + 1) * kDB + dl]);
          mu = HF[(ntile - 1) * kDB + dl];
        }
        float kkb = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float dKb = -dkb[dt][r];
          if constexpr (DECAY == 2) {  // sum_s dK_bar (.) K_bar, K_bar = K^m c_X
            const int t = 32 * X + row_of(r, hi);
            const float ktl = from_bf(bits_to_bf(KT[swz<kCMax>(dl, t)]));
            kkb += (t < c) ? lc2 * (lc1 * (dKb * ktl)) : 0.0f;
          }
          E[dt][r] = mu * dKb;
        }
        if constexpr (DECAY == 2) {  // to LDS now: carrying it to its use would keep dK_bar alive
          kkb += __shfl_xor(kkb, 32);
          if (hi == 0) KKB[w * kDB + dl] = kkb;
        }
      }
    }
  }
  __syncthreads();  // every wave is done with dW' in WB: W_i takes its place
#pragma unroll
  for (int u = 0; u < kWU; ++u) {
    const int idx = u * kCrossThreads + tid;
    if (idx < kDB * kWG) {
      const float f[8] = {wreg[u][0].x, wreg[u][0].y, wreg[u][0].z, wreg[u][0].w,
                          wreg[u][1].x, wreg[u][1].y, wreg[u][1].z, wreg[u][1].w};
      *reinterpret_cast<bf16x8_t*>(&WB[swz<DV>(idx / kWG, 8 * (idx % kWG))]) = pack8(f);
    }
  }
  __syncthreads();
  // dk and dq of the own tile, bf16 pairs of consecutive rows (r, r + 1), stored
  // through LDS at the end (see there)
  uint32_t dkp[2][8], dqp[2][8];
  if (own) {
    {
      // vector decay: query tiles in descending order (Horner over tiles, above);
      // otherwise ascending.  The dY rows of the next tile in that order are
      // fetched while the current one is multiplied.
      constexpr bool DESC = DECAY == 2;
      bf16x8_t cur[NK], nxt[NK];
      if constexpr (DESC) load_row_frags<NK>(cur, gdY, DV, t0, 32 * (ntile - 1) + l32, c, 0, hi);
      else {
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) cur[kb] = dyf[kb];
      }
      for (int step = 0; step < ntile - X; ++step) {
        const int I = DESC ? ntile - 1 - step : X + step;
        if (step + 1 < ntile - X) load_row_frags<NK>(nxt, gdY, DV, t0, 32 * (DESC ? I - 1 : I + 1) + l32, c, 0, hi);
        if constexpr (DESC) {
          if (step > 0) {  // E *= rho_{I+1} = e^{-h_{I+1}} e^{-h_I}, one factor at a time
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
              const int dl = 32 * dt + l32;
              const float f1 = HF[(I + 1) * kDB + dl];
              const float f2 = HF[I * kDB + dl];
#pragma unroll
              for (int r = 0; r < 16; ++r) E[dt][r] = f2 * (f1 * E[dt][r]);
            }
          }
        }
        f32x16_t st = zero16();  // rows t (tile I), cols s: lane (s, hi) holds dY_t . G~_s
#pragma unroll
        for (int kb = 0; kb < NK; ++kb)
          st = mfma32(cur[kb], *reinterpret_cast<const bf16x8_t*>(&GH[swz<DV>(tx, 16 * kb + 8 * hi)]), st);
        if (I == X) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (row_of(r, hi) < l32) st[r] = 0.0f;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float sa[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) sa[jj] = -st[8 * m + jj];
          const bf16x8_t A = pack8(sa);
          const int u0 = 32 * I + 16 * m + 4 * hi;
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            const int dl = 32 * dt + l32;
            const bf16x4_t q0 = *reinterpret_cast<const bf16x4_t*>(&QT[swz<kCMax>(dl, u0)]);
            const bf16x4_t q1 = *reinterpret_cast<const bf16x4_t*>(&QT[swz<kCMax>(dl, u0 + 8)]);
            E[dt] = mfma32(A, cat44(q0, q1), E[dt]);
          }
        }
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) cur[kb] = nxt[kb];
      }
    }

    // (b) e = L_t - M_X of the own rows (vector decay): the in-tile inclusive
    //     prefix of log a minus half the tile's decay; lane (d = d0 + 32 dt + l32,
    //     hi) holds rows t = 32 X + row_of(r, hi)
    float Lt[2][16];
    if constexpr (DECAY == 2) {
      const int l32b = opaque(l32);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int dl = 32 * dt + l32b;
        float lraw[16];
        const float* la_row = la + static_cast<int64_t>(t0 + 32 * X + 4 * hi) * DK + d0 + dl;
        const bool full_tile = 32 * X + 32 <= c;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * X + row_of(r, hi);
          const int off = full_tile || t < c ? (t - 32 * X - 4 * hi) * DK : -(32 * X + 4 * hi) * DK;
          lraw[r] = la_row[off];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Lt[dt][r] = (32 * X + row_of(r, hi) < c) ? lraw[r] : 0.0f;
        tile_inclusive_prefix(Lt[dt], hi);
        const float half = 0.5f * (LP[(X + 1) * kDB + dl] - LP[X * kDB + dl]);
#pragma unroll
        for (int r = 0; r < 16; ++r) Lt[dt][r] -= half;
      }
    }

    // (c) dK_z = dZ W^T; dk = dK_z + E (.) e^{M_X - L} (vector decay), and E's part
    //     of dL: -E (.) K^m
    {
      f32x16_t dkz[2];
      bf16x8_t dzf[NK];
      load_row_frags<NK>(dzf, gdZ, DV, t0, tx, c, 0, hi);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) dkz[dt] = zero16();
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
          dkz[dt] = mfma32(dzf[kb], *reinterpret_cast<const bf16x8_t*>(&WB[swz<DV>(32 * dt + l32, 16 * kb + 8 * hi)]),
                           dkz[dt]);
      }
      const int l32c = opaque(l32);  // addresses formed here, not hoisted to the kernel start
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int dl = 32 * dt + l32c;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * X + row_of(r, hi);
          const float Et = E[dt][r];
          float dkv = dkz[dt][r] + Et;
          if constexpr (DECAY == 2) {
            dkv = dkz[dt][r] + Et * __expf(-Lt[dt][r]);
            dL[dt][r] = -Et * from_bf(bits_to_bf(KT[swz<kCMax>(dl, t)]));
          }
          const uint32_t hv = bf_bits(to_bf(dkv));
          dkp[dt][r >> 1] = (r & 1) ? (dkp[dt][r >> 1] | (hv << 16)) : hv;
        }
      }
    }

    // (d) dQ~ = dY W^T + dS K~ over key tiles J <= X; dq = dQ~ (.) e^{L} and its part of dL.
    //     Vector decay, tile-relative: dq = e^{L - M_X} (.) A with
    //     A = e^{M_X} dY W^T + sum_{J <= X} e^{M_X - M_J} dS_XJ K^m_J, formed as a
    //     Horner scheme over ascending J: A = rho_0 dY W^T, then before each J > 0
    //     A *= rho_J = e^{M_J - M_{J-1}} (rho_0 = e^{M_0}); every factor <= 1.
    //     Its part of dL is A (.) Q^m.
    f32x16_t dq[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) dq[dt] = zero16();
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        dq[dt] = mfma32(dyf[kb], *reinterpret_cast<const bf16x8_t*>(&WB[swz<DV>(32 * dt + l32, 16 * kb + 8 * hi)]),
                        dq[dt]);
    }
    for (int J = 0; J <= X; ++J) {
      if constexpr (DECAY == 2) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int dl = 32 * dt + l32;
          // rho_J = e^{-h_{J-1}} e^{-h_J} for J > 0 (one factor at a time: dS K^m_{J-1}
          // carries up to e^{h_{J-1}}), rho_0 = e^{-h_0} (P_0 = 0)
          const float f1 = HF[J * kDB + dl];
          const float f0 = J > 0 ? HF[(J - 1) * kDB + dl] : 1.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) dq[dt][r] = f1 * (f0 * dq[dt][r]);
        }
      }
      f32x16_t st = zero16();  // rows s (tile J), cols t: lane (t, hi) holds dY_t . G~_s
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
        st = mfma32(*reinterpret_cast<const bf16x8_t*>(&GH[swz<DV>(32 * J + l32, 16 * kb + 8 * hi)]), dyf[kb], st);
      if (J == X) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (row_of(r, hi) > l32) st[r] = 0.0f;
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float sa[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sa[jj] = -st[8 * m + jj];
        const bf16x8_t A = pack8(sa);
        const int s0 = 32 * J + 16 * m + 4 * hi;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int dl = 32 * dt + l32;
          const bf16x4_t k0 = *reinterpret_cast<const bf16x4_t*>(&KT[swz<kCMax>(dl, s0)]);
          const bf16x4_t k1 = *reinterpret_cast<const bf16x4_t*>(&KT[swz<kCMax>(dl, s0 + 8)]);
          dq[dt] = mfma32(A, cat44(k0, k1), dq[dt]);
        }
      }
    }
    const int l32d = opaque(l32);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const int dl = 32 * dt + l32d;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * X + row_of(r, hi);
        const float dQt = dq[dt][r];
        float dqv = dQt;
        if constexpr (DECAY == 2) {
          dqv = dQt * __expf(Lt[dt][r]);
          dL[dt][r] += dQt * from_bf(bits_to_bf(QT[swz<kCMax>(dl, t)]));
        }
        const uint32_t hv = bf_bits(to_bf(dqv));
        dqp[dt][r >> 1] = (r & 1) ? (dqp[dt][r >> 1] | (hv << 16)) : hv;
      }
    }
  }

  // ---------------- decay chain: d log a = reverse cumsum of dL (vector) ----------------
  if constexpr (DECAY == 2) {
    // tile totals of dL and the sum of dK_bar (.) K_bar over the chunk
    if (own) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        float s = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += dL[dt][r];
        s += __shfl_xor(s, 32);
        if (hi == 0) TOT[X * kDB + 32 * dt + l32] = s;
      }
    }
    if (!own) {
      for (int i = lane; i < kDB; i += 64) KKB[w * kDB + i] = 0.0f;
    }
    __syncthreads();
    if (own) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int dl = 32 * dt + l32;
        // dL_last = sum_s dK_bar K_bar + dlambda lambda  (lambda = e^{L_last})
        float dlc = DLAM[dl] * __expf(LP[ntile * kDB + dl]);
        for (int w2 = 0; w2 < kCrossThreads / 64; ++w2) dlc += KKB[w2 * kDB + dl];
        float later = 0.0f;
        for (int X2 = X + 1; X2 < ntile; ++X2) later += TOT[X2 * kDB + dl];
        tile_inclusive_suffix(dL[dt], hi);
#pragma unroll
        for (int r = 0; r < 16; ++r) dL[dt][r] += later + dlc;
      }
    }
  } else {
    __syncthreads();  // every wave is past its reads of KT and QT
  }

  // ---------------- the own tile's dk, dq and d log a, stored by rows ----------------
  // A lane holds 16 rows of one feature; each wave turns its tiles into rows
  // through its own 4 KiB slices of KT and QT (free now: the barrier above
  // follows every read of them) and stores whole 16-byte pieces of rows.
  if (own) {
    uint16_t* rk = KT + w * (kCMax * kDB / 8);
    uint16_t* rq = QT + w * (kCMax * kDB / 8);
    const int prow = lane >> 3, piece = lane & 7;  // read-back: 8 rows x 8 pieces per step
    const int l32e = opaque(l32);
    // bf16 tile [32 t][64 d] -> rows of dst (d-block columns d0 .. d0 + 63)
    auto tile_out = [&](uint16_t* reg, const uint32_t (&pk)[2][8], bf16_t* dst) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          reg[row_of(r, hi) * kDB + 32 * dt + l32e] =
              static_cast<uint16_t>((r & 1) ? (pk[dt][r >> 1] >> 16) : (pk[dt][r >> 1] & 0xffffu));
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int row = 8 * k4 + prow;
        const uint4 x = *reinterpret_cast<const uint4*>(&reg[row * kDB + 8 * piece]);
        if (32 * X + row < c) *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(t0 + 32 * X + row) * DK + d0 + 8 * piece) = x;
      }
    };
    tile_out(rk, dkp, dko);
    tile_out(rq, dqp, dqo);
    if constexpr (DECAY == 2) {
      // fp32 [32 t][32 d] per feature tile dt, in rk (dt = 0) and rq (dt = 1)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        float* reg = reinterpret_cast<float*>(dt == 0 ? rk : rq);
#pragma unroll
        for (int r = 0; r < 16; ++r) reg[row_of(r, hi) * 32 + l32e] = dL[dt][r];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int row = 8 * k4 + prow;
          const float4 x = *reinterpret_cast<const float4*>(&reg[row * 32 + 4 * piece]);
          if (32 * X + row < c)
            *reinterpret_cast<float4*>(a.dlog_decay + offk + static_cast<int64_t>(t0 + 32 * X + row) * DK + d0 + 32 * dt +
                                       4 * piece) = x;
        }
      }
    }
  }

  // ---------------- dbeta (one d-block does it) ----------------
  if (db == 0) {
    for (int t = tid; t < c; t += kCrossThreads) {
      float de = 0.0f;
      for (int cc = 0; cc < ncb; ++cc)
        de += ws.deta_part[(static_cast<int64_t>(cc) * a.B * a.H + bh) * T + t0 + t];
      const float e = ETA[t];
      a.dbeta[static_cast<int64_t>(bh) * T + t0 + t] = de * e * (1.0f - 0.5f * e);
    }
  }
}

// dgamma[b,h] = sum over chunks and rows of <dW_{i+1}, W_i>.
__global__ void dgamma_reduce_kernel(const float* __restrict__ dlam_part, float* __restrict__ dgamma, int NC,
                                     int DK) {
  __shared__ float red[256];
  const int bh = blockIdx.x;
  float s = 0.0f;
  for (int i = threadIdx.x; i < NC * DK; i += blockDim.x) s += dlam_part[static_cast<int64_t>(bh) * NC * DK + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) dgamma[bh] = red[0];
}

template <int DK, int LOSS, int ACT, int DECAY>
hipError_t launch_seq(const BwdArgs& a, const BwdWs& w, const DecayPrep& dp, const SavedCtx& sv, bool par,
                      hipStream_t s) {
  const int nblk = a.B * a.H * (a.dv / kNB);
  KernelScope timing(TTT_KERNEL_BWD_SEQ, s);
  if constexpr (LOSS == 1 && ACT == 0) {
    if (par) {  // one workgroup per (chain, column block, chunk); dW' from the reverse scan
      const dim3 grid(static_cast<unsigned>(nblk * a.NC));
      if constexpr (DECAY == 2) {
        if (sv.gh)
          hipLaunchKernelGGL((ttt_bwd_seq_vec_kernel<DK, LOSS, ACT, true, true>), grid, dim3(kSeqThreads), 0, s, a, w,
                             dp, sv);
        else
          hipLaunchKernelGGL((ttt_bwd_seq_vec_kernel<DK, LOSS, ACT, false, true>), grid, dim3(kSeqThreads), 0, s, a,
                             w, dp, sv);
        return hipGetLastError();
      }
      if (sv.gh)
        hipLaunchKernelGGL((ttt_bwd_seq_kernel<DK, LOSS, ACT, DECAY, true, true>), grid, dim3(kSeqThreads), 0, s, a,
                           w, dp, sv);
      else
        hipLaunchKernelGGL((ttt_bwd_seq_kernel<DK, LOSS, ACT, DECAY, false, true>), grid, dim3(kSeqThreads), 0, s, a,
                           w, dp, sv);
      return hipGetLastError();
    }
  }
  if constexpr (DECAY == 2) {
    if (sv.gh)
      hipLaunchKernelGGL((ttt_bwd_seq_vec_kernel<DK, LOSS, ACT, true>), dim3(nblk), dim3(kSeqThreads), 0, s, a, w, dp,
                         sv);
    else
      hipLaunchKernelGGL((ttt_bwd_seq_vec_kernel<DK, LOSS, ACT, false>), dim3(nblk), dim3(kSeqThreads), 0, s, a, w,
                         dp, sv);
    return hipGetLastError();
  }
  if (sv.gh)
    hipLaunchKernelGGL((ttt_bwd_seq_kernel<DK, LOSS, ACT, DECAY, true>), dim3(nblk), dim3(kSeqThreads), 0, s, a, w,
                       dp, sv);
  else
    hipLaunchKernelGGL((ttt_bwd_seq_kernel<DK, LOSS, ACT, DECAY, false>), dim3(nblk), dim3(kSeqThreads), 0, s, a, w,
                       dp, sv);
  return hipGetLastError();
}

template <int DK, int DECAY>
hipError_t launch_cross(const BwdArgs& a, const BwdWs& w, const DecayPrep& dp, hipStream_t s) {
  const int nblk = a.B * a.H * a.NC * (DK / kDB);
  KernelScope timing(TTT_KERNEL_BWD_CROSS, s);
  switch (a.dv) {
    case 32: hipLaunchKernelGGL((ttt_bwd_cross_kernel<DK, 32, DECAY>), dim3(nblk), dim3(kCrossThreads), 0, s, a, w, dp); break;
    case 64: hipLaunchKernelGGL((ttt_bwd_cross_kernel<DK, 64, DECAY>), dim3(nblk), dim3(kCrossThreads), 0, s, a, w, dp); break;
    default: hipLaunchKernelGGL((ttt_bwd_cross_kernel<DK, 128, DECAY>), dim3(nblk), dim3(kCrossThreads), 0, s, a, w, dp); break;
  }
  return hipGetLastError();
}

template <int DK>
hipError_t bwd_by_enums(const BwdArgs& a, const BwdWs& w, const DecayPrep& dp, const SavedCtx& sv, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  // inner-product loss without an act on few chains: the dW chain by a reverse
  // scan of per-chunk increments, then the reverse sweep's terms chunk by chunk
  const bool par = linear_bwd_applies(a);
  if (par) {
    e = linear_bwd_chain(a, dp, w.dWn, s);
    if (e != hipSuccess) return e;
  }
#define TTT_BWD_CASE(LS, AC, DC) \
  if (a.loss == LS && a.act == AC && a.decay == DC) e = launch_seq<DK, LS, AC, DC>(a, w, dp, sv, par, s);
  TTT_BWD_CASE(0, 0, 0) TTT_BWD_CASE(0, 0, 1) TTT_BWD_CASE(0, 0, 2)
  TTT_BWD_CASE(0, 1, 0) TTT_BWD_CASE(0, 1, 1) TTT_BWD_CASE(0, 1, 2)
  TTT_BWD_CASE(1, 0, 0) TTT_BWD_CASE(1, 0, 1) TTT_BWD_CASE(1, 0, 2)
  TTT_BWD_CASE(1, 1, 0) TTT_BWD_CASE(1, 1, 1) TTT_BWD_CASE(1, 1, 2)
  TTT_BWD_CASE(0, 2, 0) TTT_BWD_CASE(0, 2, 1) TTT_BWD_CASE(0, 2, 2)
  TTT_BWD_CASE(1, 2, 0) TTT_BWD_CASE(1, 2, 1) TTT_BWD_CASE(1, 2, 2)
  TTT_BWD_CASE(2, 0, 0) TTT_BWD_CASE(2, 0, 1) TTT_BWD_CASE(2, 0, 2)
  TTT_BWD_CASE(2, 1, 0) TTT_BWD_CASE(2, 1, 1) TTT_BWD_CASE(2, 1, 2)
  TTT_BWD_CASE(2, 2, 0) TTT_BWD_CASE(2, 2, 1) TTT_BWD_CASE(2, 2, 2)
#undef TTT_BWD_CASE
  if (e != hipSuccess) return e;
  if (a.decay == 0) e = launch_cross<DK, 0>(a, w, dp, s);
  else if (a.decay == 1) e = launch_cross<DK, 1>(a, w, dp, s);
  else e = launch_cross<DK, 2>(a, w, dp, s);
  if (e != hipSuccess) return e;
  if (a.decay == 1) {
    KernelScope timing(TTT_KERNEL_DGAMMA, s);
    hipLaunchKernelGGL(dgamma_reduce_kernel, dim3(a.B * a.H), dim3(256), 0, s, w.dlam_part, a.dgamma, a.NC, DK);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

bool mfma_bwd_supported(const BwdArgs& a) {
  const bool c_ok = a.C == 32 || a.C == 64 || a.C == 128 || a.C == 256;
  const bool dv_ok = a.dv == 32 || a.dv == 64 || a.dv == 128;
  return a.dtype == TTT_BF16 && (a.dk == 64 || a.dk == 128) && dv_ok && c_ok;
}

// Workspace: the BwdWs regions, then (vector decay) the decay preparation.
size_t mfma_bwd_workspace(const BwdArgs& a) {
  size_t n = ws_layout(a, nullptr, nullptr);
  if (a.decay == TTT_DECAY_VECTOR) n += decay_prep_layout(a.B, a.H, a.T, a.dk, a.C, a.NC, nullptr, nullptr);
  return n;
}

hipError_t mfma_bwd_launch(const BwdArgs& a, hipStream_t s) {
  BwdWs w{};
  const size_t n = ws_layout(a, &w, a.ws);
  SavedCtx sv{};
  DecayPrep dp{};
  if (a.saved) {  // the forward's saved context: its decay preparation and G~
    mfma_saved_layout(a.B, a.H, a.T, a.dk, a.dv, a.C, a.NC, a.act, a.decay, &sv, const_cast<char*>(a.saved));
    dp = sv.prep;
    w.Gh = sv.gh;
  } else if (a.decay == TTT_DECAY_VECTOR) {
    decay_prep_layout(a.B, a.H, a.T, a.dk, a.C, a.NC, &dp, a.ws + n);
    hipError_t e = decay_prep_launch(a.log_decay, a.q, a.k, a.B, a.H, a.T, a.dk, a.C, a.NC, dp, s);
    if (e != hipSuccess) return e;
  }
  return a.dk == 128 ? bwd_by_enums<128>(a, w, dp, sv, s) : bwd_by_enums<64>(a, w, dp, sv, s);
}

}  // namespace ttt
