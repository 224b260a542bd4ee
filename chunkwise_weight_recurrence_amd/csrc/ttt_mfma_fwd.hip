// Matrix-core forward of the chunkwise TTT layer (bf16 I/O, fp32 state), gfx950.
//
// Modular TTT summary page, "Method step details": per chunk, Pass 1 (train-view
// forward Z = K W_i), Pass 2 (G = dL/dZ through the act), Pass 3 (query view,
// the chunked dual form O = f(Q W_i - Tril(Q K^T) diag(eta) G)), then the state
// transition W_{i+1} = diag(lambda) W_i - K_bar^T diag(eta) G ("Core method":
// W = W - dW); "Prerequisites": eta = 2 Sigmoid(beta + b), scalar / vector decay.
//
// Layout of the work on MI355X:
// * One workgroup (8 waves, two per SIMD) per (chain, 32-column block of d_v).  Everything but
//   the C x C scores acts column by column on W, so the column blocks of a chain
//   never communicate; B*H*d_v/32 workgroups fill the 256 CUs (64 chains x 4).
//   Workgroup ids are remapped so the column blocks of a chain land on the same
//   XCD and share its L2 for the K / Q / log-decay tiles they all read.
// * The dk x 32 fp32 state slice lives in registers (wave w < dk/32 holds d
//   rows [32w, 32w+32)) for the whole chunk loop; a bf16 copy W^T sits in LDS as
//   the MFMA operand.
// * Each wave owns one 32-token tile of the chunk for the train and query views.
//   The two waves of a SIMD get tiles s and 7 - s, so the causal work of the
//   query view is the same on every SIMD, and each SIMD has a second wave to
//   issue from while the other waits on memory or a dependent product.
// * Per chunk, K~ and Q~ (decay-scaled, bf16) are staged once in LDS with an XOR
//   swizzle of 16-byte granules; G~ = eta (.) G is written to LDS transposed.
// * All products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//     Z^T = W^T K^T,  Y^T = W^T Q~^T - G~^T Tril(S)^T,  S^T = K~ Q~^T,  U^T = G~^T K~.
//   The score tile S^T comes out of the MFMA in exactly the register layout the
//   next MFMA takes as its B operand, so the causal mask is applied in registers
//   and S never touches LDS or HBM.
// * Vector decay: L = in-chunk inclusive cumsum of log a, Q~ = Q e^L,
//   K~ = K e^-L and lambda = e^{L_last} come from the preparation kernel
//   (ttt_decay_prep.hip, once per chunk); the transition uses K_bar = K~ lambda,
//   so W_{i+1} = lambda (.) (W_i - K~^T G~).

#include "mfma_util.h"
#include "ttt_device.h"
#include "ttt_internal.h"
#include "ttt_mfma_common.h"

namespace ttt {
namespace {

constexpr int kNB = 32;        // d_v columns per workgroup
constexpr int kThreads = 512;  // 8 waves

// Token tile of wave w.  Waves are dealt to the four SIMDs round-robin, so waves
// s and s + 4 share SIMD s; they get tiles s and 7 - s.
__device__ __forceinline__ int tile_of_wave(int w) { return w < 4 ? w : 11 - w; }

template <int DK, int LOSS, int ACT, int DECAY>
__global__ __launch_bounds__(kThreads) void ttt_fwd_mfma_kernel(FwdArgs a, DecayPrep dp, SavedCtx sv) {
  __shared__ __attribute__((aligned(16))) uint16_t KS[2][kCMax * DK];  // K~ [t][d] of this / the next chunk
  __shared__ __attribute__((aligned(16))) uint16_t GT[kNB * kCMax];     // G~^T [n][t], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t WT[kNB * DK];        // bf16(W)^T [n][d], swizzled
  __shared__ float ETA[2][kCMax];
  __shared__ float LAM[2][DK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int C = a.C, dv = a.dv, T = a.T;
  const int ncb = dv / kNB;

  // XCD-aware block mapping: hardware hands block L to XCD L % 8.
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / ncb, cb = L % ncb;
  const int h = bh % a.H;
  const int col0 = cb * kNB;

  const bf16_t* k = static_cast<const bf16_t*>(a.k) + static_cast<int64_t>(bh) * T * DK;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + static_cast<int64_t>(bh) * T * dv;
  bf16_t* o = static_cast<bf16_t*>(a.o) + static_cast<int64_t>(bh) * T * dv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * T;
  // K~ = K, Q~ = Q unless vector decay prepared them
  const bf16_t* ksrc = (DECAY == 2) ? dp.kt + static_cast<int64_t>(bh) * T * DK : k;
  const bf16_t* qsrc = (DECAY == 2) ? dp.qt + static_cast<int64_t>(bh) * T * DK
                                    : static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(bh) * T * DK;
  const float* lamsrc = (DECAY == 2) ? dp.lam + static_cast<int64_t>(bh) * a.NC * DK : nullptr;
  const float gam = (DECAY == 1) ? a.gamma[h] : 1.0f;

  // ---- state: wave w < DK/32 owns W[32w + l32][col0 + row_of(r, hi)] ----
  const bool has_w = w < DK / 32;
  const int dw = 32 * w + l32;
  float W[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) W[r] = 0.0f;
  if (has_w && a.w0) {
    const float* w0 = a.w0 + (static_cast<int64_t>(bh) * DK + dw) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 x = *reinterpret_cast<const float4*>(w0 + 8 * r4 + 4 * hi);
      W[4 * r4] = x.x; W[4 * r4 + 1] = x.y; W[4 * r4 + 2] = x.z; W[4 * r4 + 3] = x.w;
    }
  }
  if (has_w) {
    store_tile_t<DK>(WT, dw, hi, W);
  }

  uint32_t sink = 0;
  const int ntile = C / 32;
  const int I = tile_of_wave(w);  // this wave's token tile
  const bool own = I < ntile;
  const int t = 32 * I + l32;     // this lane's token in the own tile

  // Software pipeline over chunks: while chunk i is computed, K~ of chunk i + 1
  // and each lane's own rows of chunk i + 1 (Q~, V, raw K) are in flight to
  // registers; K~ goes to the other LDS buffer at the end of chunk i.  Every
  // prefetch is issued unconditionally (the last chunk fetches its own rows
  // again) so the compiler's memory-counter waits stay exact.  Chunk 0's
  // operands are fetched here.
  bf16x8_t kst[RowStageSize<DK, kThreads>::U];
  uint4 vraw[2];
  bf16x8_t kraw[DK / 16], qf[DK / 16];
  {
    const int c0 = min(C, T);
    rows_load<DK, kThreads>(kst, ksrc, 0, c0);
    const float bt = beta[min(tid, c0 - 1)];
    const float lm = (DECAY == 2) ? lamsrc[min(tid, DK - 1)] : gam;
    load_row32(vraw, v, dv, 0, t, c0, col0, hi);
    load_row_frags_nomask<DK / 16>(qf, qsrc, DK, 0, t, c0, 0, hi);
    if constexpr (DECAY == 2) load_row_frags_nomask<DK / 16>(kraw, k, DK, 0, t, c0, 0, hi);
    rows_store<DK, kThreads>(KS[0], kst);
    if (tid < C) ETA[0][tid] = (tid < c0) ? lr_gate(bt, a.b) : 0.0f;
    if (tid < DK) LAM[0][tid] = (DECAY == 0) ? 1.0f : lm;
    lds_barrier();
  }

  for (int ci = 0; ci < a.NC; ++ci) {
    const int t0 = ci * C;
    const int c = min(C, T - t0);
    const int b = ci & 1;
    const bool more = ci + 1 < a.NC;
    const int t1 = more ? t0 + C : t0;  // the chunk to prefetch (the last one refetches itself)
    const int c1 = more ? min(C, T - t1) : c;
    uint16_t* KSb = KS[b];
    const int lane = opaque(threadIdx.x & 63), l32 = lane & 31, hi = lane >> 5;
    const int dw = 32 * w + l32;
    const int t = 32 * I + l32;

    // (1) K~ of the next chunk and its eta / lambda inputs, to registers
    rows_load<DK, kThreads>(kst, ksrc, t1, c1);
    const float bt = beta[t1 + min(tid, c1 - 1)];
    const float lm = (DECAY == 2) ? lamsrc[(t1 / C) * DK + min(tid, DK - 1)] : gam;

    // (2) checkpoint W_i (the state this chunk starts from)
    if (a.w_ckpt && has_w) {
      float* ck = a.w_ckpt + ((static_cast<int64_t>(bh) * a.NC + ci) * DK + dw) * dv + col0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(ck + 8 * r4 + 4 * hi) =
            make_float4(W[4 * r4], W[4 * r4 + 1], W[4 * r4 + 2], W[4 * r4 + 3]);
    }

    // (3) Pass 1 + 2: Z^T = W^T K^T, G~ = eta (.) dL/dZ; and the state part of the
    //     query view, Y^T = W^T Q~^T (every read of W^T happens before the barrier)
    f32x16_t y = zero16();
    if (own) {
      f32x16_t z = zero16();
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb) {
        const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(&WT[swz<DK>(l32, 16 * kb + 8 * hi)]);
        // the train view uses the raw keys (vector decay: prefetched rows; otherwise K~ = K in LDS)
        const bf16x8_t Bk = (DECAY == 2) ? kraw[kb]
                                         : *reinterpret_cast<const bf16x8_t*>(&KSb[swz<DK>(t, 16 * kb + 8 * hi)]);
        z = mfma32(A, Bk, z);
        y = mfma32(A, qf[kb], y);
      }
      // lane holds Z[t][n = row_of(r, hi)]
      const float et = ETA[b][t];  // 0 for tokens past the end: G~ = 0 there
      float vv[16];
      {
        uint2 vx[4];
        row32_frags(vraw, vx, true);  // rows past the end: finite values whose G~ is zeroed by eta
        unpack16(vx, vv);
      }
      float gt[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float zz = z[r];
        const float e = loss_signal<LOSS, ACT>(zz, vv[r]);
        gt[r] = et * e * act_df<ACT>(zz);
      }
      store_tile_t<kCMax>(GT, t, hi, gt);
      if (sv.gh) {  // saved for the backward: G~, and with an act Z itself
        const int64_t offv = static_cast<int64_t>(bh) * T * dv;
        store_row16_x2(sv.gh + offv, dv, t0, t, c, col0, hi, gt);
        if constexpr (ACT != 0) {
          float zs[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) zs[r] = z[r];
          store_row16_x2(sv.z + offv, dv, t0, t, c, col0, hi, zs);
        }
      }
    }
    lds_barrier();

    // L2 prefetch of the chunk after the next one (this workgroup's quarter of its
    // K~, Q~, raw-K and V lines): the register prefetch of the next chunk then
    // finds its lines in L2, and a shorter latency is more bytes per outstanding
    // request of the CU.  The dwords only feed a never-taken store.
    uint32_t pf2[4] = {0, 0, 0, 0};
    if (ci + 2 < a.NC) {
      const int t2 = t0 + 2 * C;
      const int c2 = min(C, T - t2);
      uint32_t w1[1];
      l2_touch<1, kThreads>(w1, ksrc + static_cast<int64_t>(t2) * DK, c2 * DK * 2, cb, ncb); pf2[0] = w1[0];
      l2_touch<1, kThreads>(w1, qsrc + static_cast<int64_t>(t2) * DK, c2 * DK * 2, cb, ncb); pf2[1] = w1[0];
      l2_touch<1, kThreads>(w1, v + static_cast<int64_t>(t2) * dv, c2 * dv * 2, cb, ncb); pf2[2] = w1[0];
      if constexpr (DECAY == 2) {
        l2_touch<1, kThreads>(w1, k + static_cast<int64_t>(t2) * DK, c2 * DK * 2, cb, ncb);
        pf2[3] = w1[0];
      }
    }

    // (4) Pass 3: Y^T -= G~^T Tril(S)^T, O = f(Y)
    if (own) {
      // The A fragments of key tile J + 1 are read from LDS while tile J is
      // multiplied (one LDS round trip per tile instead of one per product); the
      // empty asm makes the loop-carried fragments non-loads, so the optimiser
      // does not fold the two reads back into one at the top of the loop.
      bf16x8_t ka[DK / 16];
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb)
        ka[kb] = *reinterpret_cast<const bf16x8_t*>(&KSb[swz<DK>(l32, 16 * kb + 8 * hi)]);
      for (int J = 0; J <= I; ++J) {
        bf16x8_t kc[DK / 16];
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb) {
          kc[kb] = ka[kb];
          asm volatile("" : "+v"(kc[kb]));
        }
        const int Jn = min(J + 1, I);  // the last tile reads itself again
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
          ka[kb] = *reinterpret_cast<const bf16x8_t*>(&KSb[swz<DK>(32 * Jn + l32, 16 * kb + 8 * hi)]);
        f32x16_t s = zero16();
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb) s = mfma32(kc[kb], qf[kb], s);
        // lane holds S[t][32J + row_of(r, hi)]; keep s <= t only
        if (J == I) {
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
          const bf16x4_t g0 = *reinterpret_cast<const bf16x4_t*>(&GT[swz<kCMax>(l32, s0)]);
          const bf16x4_t g1 = *reinterpret_cast<const bf16x4_t*>(&GT[swz<kCMax>(l32, s0 + 8)]);
          y = mfma32(cat44(g0, g1), pack8(nb), y);
        }
      }
      // lane holds Y[t][n = row_of(r, hi)] -> O = f(Y)
      if constexpr (ACT != 0) {
        if (sv.dfy) {  // saved for the backward: f'(Y)
          float dfy[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) dfy[r] = act_df<ACT>(y[r]);
          store_row16_x2(sv.dfy + static_cast<int64_t>(bh) * T * dv, dv, t0, t, c, col0, hi, dfy);
        }
      }
      float of[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) of[r] = act_f<ACT>(y[r]);
      store_row16_x2(o, dv, t0, t, c, col0, hi, of);
    }

    // (5) this lane's rows of the next chunk (the current ones are consumed)
    load_row32(vraw, v, dv, t1, t, c1, col0, hi);
    load_row_frags_nomask<DK / 16>(qf, qsrc, DK, t1, t, c1, 0, hi);
    if constexpr (DECAY == 2) load_row_frags_nomask<DK / 16>(kraw, k, DK, t1, t, c1, 0, hi);

    // (6) transition: W <- diag(lam) W - K_bar^T G~, and its bf16 copy for the next chunk
    if (has_w) {
      f32x16_t u = zero16();
      ColumnReaderTR<DK> kcol(KSb, 32 * w, l32, hi);
      RowReader<kCMax> arow(GT, l32, hi);
      int kb0 = 0;
      for (; kb0 + 4 <= C / 16; kb0 += 4) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) u = mfma32(arow(kk), kcol(kk), u);
        kcol.advance();
        arow.advance();
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)  // the last, partial group (C = 32)
        if (kb0 + kk < C / 16) u = mfma32(arow(kk), kcol(kk), u);
      // lane holds U[d = dw][n = row_of(r, hi)] = (K~^T G~)[d][n]
      const float lam = LAM[b][dw];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (DECAY == 2) W[r] = lam * (W[r] - u[r]);
        else if constexpr (DECAY == 1) W[r] = lam * W[r] - u[r];
        else W[r] = W[r] - u[r];
      }
      store_tile_t<DK>(WT, dw, hi, W);
    }

    // (7) the next chunk's K~, eta and lambda into the other buffers
    if (more) {
      rows_store<DK, kThreads>(KS[b ^ 1], kst);
      if (tid < C) ETA[b ^ 1][tid] = (tid < c1) ? lr_gate(bt, a.b) : 0.0f;
      if (tid < DK) LAM[b ^ 1][tid] = (DECAY == 0) ? 1.0f : lm;
    }
    sink ^= pf2[0] ^ pf2[1] ^ pf2[2] ^ pf2[3];
    lds_barrier();
  }
  if (T < 0) static_cast<uint32_t*>(a.o)[0] = sink;  // never taken: keeps the prefetch loads alive

  if (a.w_final && has_w) {
    float* wf = a.w_final + (static_cast<int64_t>(bh) * DK + dw) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(wf + 8 * r4 + 4 * hi) =
          make_float4(W[4 * r4], W[4 * r4 + 1], W[4 * r4 + 2], W[4 * r4 + 3]);
  }
}

// ----------------------------------------------------------------------------
// Vector decay: the same chunk steps, with the decay split at 32-token tiles.
// ----------------------------------------------------------------------------
// With L the in-chunk cumsum of log a, query t sees key s <= t through
// e^{L_t - L_s} per feature and the chunk-start state through e^{L_t}.  The
// preparation kernel gives tile-relative Q^m = Q e^{L - M_I}, K^m = K e^{M_I - L}
// (M_I the midpoint of tile I's range of L) and the tile-boundary prefixes P_I.
// Per column block the chunk then runs as a recurrence over its eight tiles on
// the token-level state at each tile start, kept scaled by e^{M_I}:
//   X_0 = e^{M_0} W_i,   X_{I+1} = rho_{I+1} (X_I - K^m_I^T G~_I),
//   W_{i+1} = mu (X_{last} - K^m_last^T G~_last),
//   Y_I = Q^m_I X_I - Tril(Q^m_I K^m_I^T) G~_I,
// rho_{I+1} = e^{M_{I+1} - M_I}, rho_0 = e^{M_0}, mu = e^{L_last - M_last}: every
// factor is <= 1, so nothing grows with the decay between tiles; inside a tile
// Q^m and K^m grow by at most half the tile's own decay.  This is the chunk's
// dual form (Modular TTT summary page, "Method step details") with the
// cross-tile part of Tril(S) G~ regrouped through the tile states; it also
// needs one d_k-deep product per query tile instead of one score tile per
// earlier key tile.
//
// Per chunk: Pass 1+2 as above (raw K for the train view); then the waves that
// hold W run the tile recurrence (two MFMAs per tile; the bf16 states X_I^T go
// to LDS) while every wave forms its diagonal tile; then each wave reads its
// state X_I and writes O.  K^m of the next chunk waits in registers until the
// recurrence has finished with the single K^m buffer.
template <int DK, int LOSS, int ACT>
__global__ __launch_bounds__(kThreads) void ttt_fwd_vec_kernel(FwdArgs a, DecayPrep dp, SavedCtx sv) {
  constexpr int kNT = kCMax / 32;                                        // tiles per chunk at C = 256
  __shared__ __attribute__((aligned(16))) uint16_t KS[kCMax * DK];        // K^m [t][d] of this chunk
  __shared__ __attribute__((aligned(16))) uint16_t XT[kNT * DK * kNB];    // X_I [I][d][n], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t GT[kNB * kCMax];       // G~^T [n][t], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t WT[kNB * DK];          // bf16(W_i)^T [n][d], swizzled
  __shared__ float ETA[2][kCMax];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int C = a.C, dv = a.dv, T = a.T;
  const int ncb = dv / kNB;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / ncb, cb = L % ncb;
  const int col0 = cb * kNB;
  const int ntile = C / 32;

  const bf16_t* k = static_cast<const bf16_t*>(a.k) + static_cast<int64_t>(bh) * T * DK;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + static_cast<int64_t>(bh) * T * dv;
  bf16_t* o = static_cast<bf16_t*>(a.o) + static_cast<int64_t>(bh) * T * dv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * T;
  const bf16_t* ksrc = dp.kt + static_cast<int64_t>(bh) * T * DK;  // K^m
  const bf16_t* qsrc = dp.qt + static_cast<int64_t>(bh) * T * DK;  // Q^m
  const float* lpsrc = dp.lpre + static_cast<int64_t>(bh) * a.NC * (ntile + 1) * DK;

  const bool has_w = w < DK / 32;
  const int dw = 32 * w + l32;
  float W[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) W[r] = 0.0f;
  if (has_w && a.w0) {
    const float* w0 = a.w0 + (static_cast<int64_t>(bh) * DK + dw) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 x = *reinterpret_cast<const float4*>(w0 + 8 * r4 + 4 * hi);
      W[4 * r4] = x.x; W[4 * r4 + 1] = x.y; W[4 * r4 + 2] = x.z; W[4 * r4 + 3] = x.w;
    }
  }
  if (has_w) store_tile_t<DK>(WT, dw, hi, W);

  uint32_t sink = 0;
  const int I = tile_of_wave(w);  // this wave's token tile
  const bool own = I < ntile;

  bf16x8_t kst[RowStageSize<DK, kThreads>::U];
  uint4 vraw[2];
  bf16x8_t kraw[DK / 16], qf[DK / 16];
  {
    const int c0 = min(C, T);
    const int t = 32 * I + l32;
    rows_load<DK, kThreads>(kst, ksrc, 0, c0);
    const float bt = beta[min(tid, c0 - 1)];
    load_row32(vraw, v, dv, 0, t, c0, col0, hi);
    load_row_frags_nomask<DK / 16>(qf, qsrc, DK, 0, t, c0, 0, hi);
    load_row_frags_nomask<DK / 16>(kraw, k, DK, 0, t, c0, 0, hi);
    rows_store<DK, kThreads>(KS, kst);
    if (tid < C) ETA[0][tid] = (tid < c0) ? lr_gate(bt, a.b) : 0.0f;
    lds_barrier();
  }

  for (int ci = 0; ci < a.NC; ++ci) {
    const int t0 = ci * C;
    const int c = min(C, T - t0);
    const int b = ci & 1;
    const bool more = ci + 1 < a.NC;
    const int t1 = more ? t0 + C : t0;
    const int c1 = more ? min(C, T - t1) : c;
    const int lane = opaque(threadIdx.x & 63), l32 = lane & 31, hi = lane >> 5;
    const int dw = 32 * w + l32;
    const int t = 32 * I + l32;

    // (1) K^m of the next chunk and its eta input, to registers; this chunk's
    //     tile prefixes P_0 .. P_ntile of the state rows (used after Pass 1+2)
    rows_load<DK, kThreads>(kst, ksrc, t1, c1);
    const float bt = beta[t1 + min(tid, c1 - 1)];
    float pl[kNT + 1];
    if (has_w) {  // only the waves that run the recurrence
      const float* lp = lpsrc + static_cast<int64_t>(ci) * (ntile + 1) * DK + dw;
#pragma unroll
      for (int j = 0; j <= kNT; ++j) pl[j] = lp[min(j, ntile) * DK];
    }

    // (2) checkpoint W_i
    if (a.w_ckpt && has_w) {
      float* ck = a.w_ckpt + ((static_cast<int64_t>(bh) * a.NC + ci) * DK + dw) * dv + col0;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(ck + 8 * r4 + 4 * hi) =
            make_float4(W[4 * r4], W[4 * r4 + 1], W[4 * r4 + 2], W[4 * r4 + 3]);
    }

    // (3) Pass 1 + 2: Z^T = W^T K^T (raw keys), G~ = eta (.) dL/dZ -> GT
    if (own) {
      f32x16_t z = zero16();
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb)
        z = mfma32(*reinterpret_cast<const bf16x8_t*>(&WT[swz<DK>(l32, 16 * kb + 8 * hi)]), kraw[kb], z);
      const float et = ETA[b][t];
      float vv[16];
      {
        uint2 vx[4];
        row32_frags(vraw, vx, true);
        unpack16(vx, vv);
      }
      // the next chunk's raw keys and values (their last use here is above): a
      // whole chunk of latency to hide behind
      load_row_frags_nomask<DK / 16>(kraw, k, DK, t1, t, c1, 0, hi);
      load_row32(vraw, v, dv, t1, t, c1, col0, hi);
      float gt[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float zz = z[r];
        const float e = loss_signal<LOSS, ACT>(zz, vv[r]);
        gt[r] = et * e * act_df<ACT>(zz);
      }
      store_tile_t<kCMax>(GT, t, hi, gt);
      if (sv.gh) {
        const int64_t offv = static_cast<int64_t>(bh) * T * dv;
        store_row16_x2(sv.gh + offv, dv, t0, t, c, col0, hi, gt);
        if constexpr (ACT != 0) {
          float zs[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) zs[r] = z[r];
          store_row16_x2(sv.z + offv, dv, t0, t, c, col0, hi, zs);
        }
      }
    }
    lds_barrier();

    uint32_t pf2[4] = {0, 0, 0, 0};
    if (ci + 2 < a.NC) {
      const int t2 = t0 + 2 * C;
      const int c2 = min(C, T - t2);
      uint32_t w1[1];
      l2_touch<1, kThreads>(w1, ksrc + static_cast<int64_t>(t2) * DK, c2 * DK * 2, cb, ncb); pf2[0] = w1[0];
      l2_touch<1, kThreads>(w1, qsrc + static_cast<int64_t>(t2) * DK, c2 * DK * 2, cb, ncb); pf2[1] = w1[0];
      l2_touch<1, kThreads>(w1, v + static_cast<int64_t>(t2) * dv, c2 * dv * 2, cb, ncb); pf2[2] = w1[0];
      l2_touch<1, kThreads>(w1, k + static_cast<int64_t>(t2) * DK, c2 * DK * 2, cb, ncb); pf2[3] = w1[0];
    }

    // (4a) the tile recurrence of the state rows: X_I^T -> XT[I]; W <- W_{i+1}
    f32x16_t y = zero16();
    if (has_w) {
      ColumnReaderTR<DK> kcol(KS, 32 * w, l32, hi);
      RowReader<kCMax> arow(GT, l32, hi);
      float X[16];
      {
        const float rho0 = __expf(0.5f * pl[1]);  // e^{M_0}, P_0 = 0
#pragma unroll
        for (int r = 0; r < 16; ++r) X[r] = rho0 * W[r];
      }
      static_for<kNT>([&](auto Ic) {
        constexpr int Ti = Ic;
        if (Ti < ntile) {
          store_tile_rows<kNB>(XT + Ti * DK * kNB, dw, hi, X);
          f32x16_t u = zero16();
          constexpr int k0 = 2 * (Ti & 1);
          u = mfma32(arow(k0), kcol(k0), u);
          u = mfma32(arow(k0 + 1), kcol(k0 + 1), u);
          if constexpr ((Ti & 1) == 1) {
            kcol.advance();
            arow.advance();
          }
          // X_{I+1} = rho_{I+1} (X_I - U_I), rho_{I+1} = e^{-h_I} e^{-h_{I+1}} with
          // h_I = (P_I - P_{I+1}) / 2 half of tile I's decay, applied one factor at a
          // time: U_I carries up to e^{h_I} (K^m), and rho itself can leave the fp32
          // range where neither factor does.  After the last tile W_{i+1} = mu (X - U),
          // mu = e^{-h_last}.
          if (Ti + 1 < ntile) {
            const float f1 = __expf(0.5f * (pl[Ti + 1] - pl[Ti]));
            const float f2 = __expf(0.5f * (pl[Ti + 2 <= kNT ? Ti + 2 : kNT] - pl[Ti + 1]));
#pragma unroll
            for (int r = 0; r < 16; ++r) X[r] = f2 * (f1 * (X[r] - u[r]));
          } else {
            const float mu = __expf(0.5f * (pl[Ti + 1 <= kNT ? Ti + 1 : kNT] - pl[Ti]));
#pragma unroll
            for (int r = 0; r < 16; ++r) W[r] = mu * (X[r] - u[r]);
          }
        }
      });
      store_tile_t<DK>(WT, dw, hi, W);  // once per chunk, after the recurrence
    }
    // (4b) the diagonal tile: S^T = K^m_I Q^m_I^T (s <= t kept), Y^T = -G~_I^T Tril(S)^T;
    //      after the recurrence on the waves that run it (its chain of dependent steps
    //      is the longer path), at once on the others
    if (own) {
      f32x16_t sc = zero16();
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb)
        sc = mfma32(*reinterpret_cast<const bf16x8_t*>(&KS[swz<DK>(32 * I + l32, 16 * kb + 8 * hi)]), qf[kb], sc);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (row_of(r, hi) > l32) sc[r] = 0.0f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float nb[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) nb[jj] = -sc[8 * m + jj];
        const int s0 = 32 * I + 16 * m + 4 * hi;
        const bf16x4_t g0 = *reinterpret_cast<const bf16x4_t*>(&GT[swz<kCMax>(l32, s0)]);
        const bf16x4_t g1 = *reinterpret_cast<const bf16x4_t*>(&GT[swz<kCMax>(l32, s0 + 8)]);
        y = mfma32(cat44(g0, g1), pack8(nb), y);
      }
    }

    // the next chunk's eta (ETA[b ^ 1] is not read in this chunk)
    if (more && tid < C) ETA[b ^ 1][tid] = (tid < c1) ? lr_gate(bt, a.b) : 0.0f;
    lds_barrier();

    // the next chunk's K^m: every read of KS in this chunk is behind the barrier, and
    // the next chunk reads it only after its own first barrier
    if (more) rows_store<DK, kThreads>(KS, kst);

    // (5) Y^T += X_I^T Q^m_I^T; O = f(Y)
    if (own) {
      ColumnReaderTR<kNB> xcol(XT + I * DK * kNB, 0, l32, hi);  // A = X_I^T
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb) y = mfma32(xcol(kb), qf[kb], y);
      if constexpr (ACT != 0) {
        if (sv.dfy) {
          float dfy[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) dfy[r] = act_df<ACT>(y[r]);
          store_row16_x2(sv.dfy + static_cast<int64_t>(bh) * T * dv, dv, t0, t, c, col0, hi, dfy);
        }
      }
      float of[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) of[r] = act_f<ACT>(y[r]);
      store_row16_x2(o, dv, t0, t, c, col0, hi, of);
    }

    // (6) this lane's Q^m rows of the next chunk (raw K and V were issued after Pass 2;
    //     a wave without a tile issues all three here)
    load_row_frags_nomask<DK / 16>(qf, qsrc, DK, t1, t, c1, 0, hi);
    if (!own) {
      load_row_frags_nomask<DK / 16>(kraw, k, DK, t1, t, c1, 0, hi);
      load_row32(vraw, v, dv, t1, t, c1, col0, hi);
    }

    sink ^= pf2[0] ^ pf2[1] ^ pf2[2] ^ pf2[3];
  }
  if (T < 0) static_cast<uint32_t*>(a.o)[0] = sink;

  if (a.w_final && has_w) {
    float* wf = a.w_final + (static_cast<int64_t>(bh) * DK + dw) * dv + col0;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(wf + 8 * r4 + 4 * hi) =
          make_float4(W[4 * r4], W[4 * r4 + 1], W[4 * r4 + 2], W[4 * r4 + 3]);
  }
}

template <int DK, int LOSS, int ACT, int DECAY>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  const int nblk = a.B * a.H * (a.dv / kNB);
  // With a saved context the decay preparation goes there (the backward reads it);
  // otherwise into the workspace.
  SavedCtx sv{};
  if (a.saved) mfma_saved_layout(a.B, a.H, a.T, a.dk, a.dv, a.C, a.NC, a.act, a.decay, &sv, a.saved);
  DecayPrep dp{};
  if (DECAY == 2) {
    if (a.saved) dp = sv.prep;
    else decay_prep_layout(a.B, a.H, a.T, a.dk, a.C, a.NC, &dp, a.ws);
    hipError_t e = decay_prep_launch(a.log_decay, a.q, a.k, a.B, a.H, a.T, a.dk, a.C, a.NC, dp, s);
    if (e != hipSuccess) return e;
  }
  KernelScope timing(TTT_KERNEL_FWD, s);
  if constexpr (DECAY == 2)
    hipLaunchKernelGGL((ttt_fwd_vec_kernel<DK, LOSS, ACT>), dim3(nblk), dim3(kThreads), 0, s, a, dp, sv);
  else
    hipLaunchKernelGGL((ttt_fwd_mfma_kernel<DK, LOSS, ACT, DECAY>), dim3(nblk), dim3(kThreads), 0, s, a, dp, sv);
  return hipGetLastError();
}

template <int DK>
hipError_t fwd_by_enums(const FwdArgs& a, hipStream_t s) {
#define TTT_FWD_CASE(LS, AC, DC) \
  if (a.loss == LS && a.act == AC && a.decay == DC) return launch_fwd<DK, LS, AC, DC>(a, s);
  TTT_FWD_CASE(0, 0, 0) TTT_FWD_CASE(0, 0, 1) TTT_FWD_CASE(0, 0, 2)
  TTT_FWD_CASE(0, 1, 0) TTT_FWD_CASE(0, 1, 1) TTT_FWD_CASE(0, 1, 2)
  TTT_FWD_CASE(1, 0, 0) TTT_FWD_CASE(1, 0, 1) TTT_FWD_CASE(1, 0, 2)
  TTT_FWD_CASE(1, 1, 0) TTT_FWD_CASE(1, 1, 1) TTT_FWD_CASE(1, 1, 2)
  TTT_FWD_CASE(0, 2, 0) TTT_FWD_CASE(0, 2, 1) TTT_FWD_CASE(0, 2, 2)
  TTT_FWD_CASE(1, 2, 0) TTT_FWD_CASE(1, 2, 1) TTT_FWD_CASE(1, 2, 2)
  TTT_FWD_CASE(2, 0, 0) TTT_FWD_CASE(2, 0, 1) TTT_FWD_CASE(2, 0, 2)
  TTT_FWD_CASE(2, 1, 0) TTT_FWD_CASE(2, 1, 1) TTT_FWD_CASE(2, 1, 2)
  TTT_FWD_CASE(2, 2, 0) TTT_FWD_CASE(2, 2, 1) TTT_FWD_CASE(2, 2, 2)
#undef TTT_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

size_t mfma_saved_layout(int B, int H, int T, int dk, int dv, int C, int NC, int act, int decay, SavedCtx* sv,
                         char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return base ? base + o : nullptr;
  };
  SavedCtx v{};
  if (decay == TTT_DECAY_VECTOR) {
    char* p = take(decay_prep_layout(B, H, T, dk, C, NC, nullptr, nullptr));
    if (base) decay_prep_layout(B, H, T, dk, C, NC, &v.prep, p);
  }
  const size_t tv = static_cast<size_t>(B) * H * T * dv * 2;
  v.gh = reinterpret_cast<uint16_t*>(take(tv));
  if (act != TTT_ACT_NONE) {
    v.dfy = reinterpret_cast<uint16_t*>(take(tv));
    v.z = reinterpret_cast<uint16_t*>(take(tv));
  }
  if (sv) *sv = v;
  return off;
}

bool mfma_fwd_supported(const FwdArgs& a) {
  const bool c_ok = a.C == 32 || a.C == 64 || a.C == 128 || a.C == 256;
  return a.dtype == TTT_BF16 && (a.dk == 64 || a.dk == 128) && a.dv % kNB == 0 && a.dv <= 256 && c_ok;
}

bool mfma_saved_supported(const FwdArgs& a) {
  return mfma_fwd_supported(a) && (a.dv == 32 || a.dv == 64 || a.dv == 128);  // the backward's d_v set
}

size_t mfma_fwd_workspace(const FwdArgs& a) {
  if (linear_fwd_applies(a)) return linear_fwd_workspace(a);
  return a.decay == TTT_DECAY_VECTOR ? decay_prep_layout(a.B, a.H, a.T, a.dk, a.C, a.NC, nullptr, nullptr) : 0;
}

hipError_t mfma_fwd_launch(const FwdArgs& a, hipStream_t s) {
  if (linear_fwd_applies(a)) return linear_fwd_launch(a, s);
  return a.dk == 128 ? fwd_by_enums<128>(a, s) : fwd_by_enums<64>(a, s);
}


}  // namespace ttt
