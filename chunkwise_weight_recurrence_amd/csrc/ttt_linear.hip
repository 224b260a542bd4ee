// Chunk-parallel forward of the inner-product / linear TTT layer (bf16 I/O,
// fp32 state), gfx950.
//
// With the inner-product loss and no activation the train-view gradient does
// not depend on the state: G = dL/dV_hat = -V (Modular TTT summary page,
// "Method step details": Pass 2 of Algorithm 1 for the inner-product loss), so
// G~ = eta (.) G = -eta (.) V is known for every chunk up front.  The state
// transition ("Core method", W = W - dW, with the decay of "Prerequisites")
//   none:   W_{i+1} = W_i - K^T G~
//   scalar: W_{i+1} = gamma_h W_i - K^T G~
//   vector: W_{i+1} = lambda_i (.) W_i - K_bar_i^T G~_i      (row scale lambda = e^{L_last},
//           K_bar = K e^{L_last - L})
// is then an affine recurrence whose increments U_i = K_bar_i^T G~_i (K^T G~
// without decay) are independent of each other, and the query view of a chunk
//   O_i = Q~_i W_i - Tril(Q~_i K~_i^T) G~_i      (vector decay: Q~ = Q e^{L}, and the
//           score of query t and key s carries e^{L_t - L_s} per feature)
// needs only its own chunk and W_i.  Vector decay is formed from the tile-relative
// Q^m, K^m and tile prefixes P_I of ttt_decay_prep.hip so that nothing leaves the
// fp32 range: K_bar = K^m e^{-h_I} e^{P_last - P_{I+1}} and Q~ = Q^m e^{-h_I} e^{P_I}
// on the rows of tile I (h_I half the tile's decay, every factor <= 1), and a
// score across tiles J < I is Q^m_t e^{M_I - M_J} K^m_s (M the tile midpoints),
// the factor applied to Q^m in two steps, e^{-h_I} and e^{P_I - M_J}.  So the forward runs as three launches:
//   1. lin_state_kernel: U_i for every (chain, chunk) at once (and G~ into the
//      saved context for the backward);
//   2. lin_scan_kernel: W_i for every chunk by the recurrence above, elementwise
//      (fp32), into the checkpoints (or over U_i in place) and w_final;
//   3. lin_out_kernel: O_i for every (chain, chunk) at once.
// This fills the GPU whatever B * H is: the sequential kernel has B * H * d_v / 32
// workgroups in all, this one that many per chunk.  The results equal the
// sequential kernel's up to fp32 summation order.

#include "mfma_util.h"
#include "ttt_device.h"
#include "ttt_internal.h"
#include "ttt_mfma_common.h"

namespace ttt {
namespace {

constexpr int kLinThreads = 512;  // 8 waves
constexpr int kLinNB = 32;        // d_v columns of the sequential kernel's workgroups

__device__ __forceinline__ int lin_tile_of_wave(int w) { return w < 4 ? w : 11 - w; }

// ---------------------------------------------------------------------------
// 1. U_i = K~_i^T G~_i, one workgroup per (chain, chunk).
// ---------------------------------------------------------------------------
// The contraction over the chunk's tokens runs in pieces of kLinPiece tokens:
// K~ [piece][DK] and G~ [piece][DV] are staged as they lie (rows = tokens,
// swizzled) and both operands are column reads (ColumnReaderTR).  The staging
// buffers (64 KB at DK = DV = 128) let two workgroups share a CU, so one
// stages while the other multiplies.  The DK x DV output has (DK / 32) x
// (DV / 32) tiles of 32 x 32; wave w takes tiles w, w + 8, ...
constexpr int kLinPiece = 128;

// The same kernel forms the backward's increments R_i = Q~_i^T dO_i of the dW
// chain (A = Q~, B = dO as it is): the operands are passed as plain sources.
struct LinStateArgs {
  int B, H, T, C, NC;
  float b;
  const bf16_t* A;     // [B,H,T,DK]: K~ (forward) or Q~ (backward)
  const bf16_t* Bsrc;  // [B,H,T,DV]: V (forward, scaled to G~ = -eta V) or dO (backward)
  const float* beta;   // [B,H,T]: the forward's scale; NULL: B is used as it is
  float* U;            // [B,H,NC,DK,DV] fp32 out
  uint16_t* gh;        // optional [B,H,T,DV] bf16 copy of the scaled B (the forward's G~)
  // vector decay: A is K^m or Q^m (tile-relative) and its rows of tile I are scaled
  // per feature by e^{-h_I} and then e^{P_last - P_{I+1}} (mode 1: K_bar, the
  // forward's increments) or e^{P_I} (mode 2: Q~, the backward's); 0: no scaling
  const float* lpre;   // [B,H,NC,C/32+1,DK] tile prefixes P_0 .. P_{C/32}
  int scale_mode;
};

template <int DK, int DV>
__global__ __launch_bounds__(kLinThreads, 4) void lin_state_kernel(LinStateArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t KS[kLinPiece * DK];  // K~ [t][d]
  __shared__ __attribute__((aligned(16))) uint16_t GS[kLinPiece * DV];  // G~ [t][n]
  __shared__ float F1[kCMax / 32][DK], F2[kCMax / 32][DK];             // the row factors of each tile
  constexpr int TD = DK / 32, TN = DV / 32, NTILE = TD * TN;
  constexpr int PER_WAVE = (NTILE + 7) / 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int C = a.C, T = a.T;
  const int ci = blockIdx.x % a.NC;
  const int bh = blockIdx.x / a.NC;
  const int t0 = ci * C;
  const int c = min(C, T - t0);
  const int64_t offk = static_cast<int64_t>(bh) * T * DK;
  const int64_t offv = static_cast<int64_t>(bh) * T * DV;
  const bf16_t* ks = a.A + offk;
  const bf16_t* v = a.Bsrc + offv;
  const bool scaled = a.beta != nullptr;
  const float* beta = scaled ? a.beta + static_cast<int64_t>(bh) * T : nullptr;
  uint16_t* gh = a.gh;
  float* U = a.U;
  constexpr int GK = DK / 8, GV = DV / 8;
  constexpr int UK = (kLinPiece * GK + kLinThreads - 1) / kLinThreads;
  constexpr int UV = (kLinPiece * GV + kLinThreads - 1) / kLinThreads;

  f32x16_t acc[PER_WAVE];
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p) acc[p] = zero16();

  const int mode = a.scale_mode;
  if (mode) {  // the tile factors of this chunk, written before the first piece's barrier
    const int ntile = C / 32;
    const float* lp = a.lpre + (static_cast<int64_t>(bh) * a.NC + ci) * (ntile + 1) * DK;
    for (int i = tid; i < ntile * DK; i += kLinThreads) {
      const int I = i / DK, d = i % DK;
      const float pI = lp[I * DK + d], pN = lp[(I + 1) * DK + d];
      F1[I][d] = __expf(0.5f * (pN - pI));
      F2[I][d] = __expf(mode == 1 ? lp[ntile * DK + d] - pN : pI);
    }
    __syncthreads();
  }

  for (int p0 = 0; p0 < C; p0 += kLinPiece) {
    const int np = min(kLinPiece, C - p0);  // rows of this piece (C = 32 or 64: all of it)
    // staging: every load first (rows >= c read row 0, zeroed when written)
    uint4 kk[UK], vv[UV];
    float et[UV];
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int idx = min(u * kLinThreads + tid, kLinPiece * GK - 1), t = p0 + idx / GK, g = idx % GK;
      kk[u] = *reinterpret_cast<const uint4*>(ks + static_cast<int64_t>(t0 + (t < c ? t : 0)) * DK + 8 * g);
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int idx = min(u * kLinThreads + tid, kLinPiece * GV - 1), t = p0 + idx / GV, g = idx % GV;
      vv[u] = *reinterpret_cast<const uint4*>(v + static_cast<int64_t>(t0 + (t < c ? t : 0)) * DV + 8 * g);
      et[u] = scaled ? beta[t0 + (t < c ? t : 0)] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int idx = u * kLinThreads + tid, r = idx / GK, g = idx % GK;
      if (idx < kLinPiece * GK && r < np) {
        uint4 x = mask4(kk[u], okmask(p0 + r < c));
        if (mode) {  // K_bar or Q~ from the tile-relative rows, one factor at a time
          const int I = (p0 + r) / 32;
          float f[8];
          unpack8(x, f);
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = F2[I][8 * g + j] * (F1[I][8 * g + j] * f[j]);
          const bf16x8_t y = pack8(f);
          x = *reinterpret_cast<const uint4*>(&y);
        }
        *reinterpret_cast<uint4*>(&KS[swz<DK>(r, 8 * g)]) = x;
      }
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int idx = u * kLinThreads + tid, r = idx / GV, g = idx % GV;
      const int t = p0 + r;
      if (idx < kLinPiece * GV && r < np) {
        if (scaled) {
          // G~ = eta (.) G = -eta v (inner-product loss, no activation); 0 past the chunk
          const float e = (t < c) ? -lr_gate(et[u], a.b) : 0.0f;
          float f[8];
          unpack8(vv[u], f);
          float gf[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) gf[j] = e * f[j];
          const bf16x8_t x = pack8(gf);
          *reinterpret_cast<bf16x8_t*>(&GS[swz<DV>(r, 8 * g)]) = x;
          if (gh && t < c) *reinterpret_cast<bf16x8_t*>(gh + offv + static_cast<int64_t>(t0 + t) * DV + 8 * g) = x;
        } else {
          *reinterpret_cast<uint4*>(&GS[swz<DV>(r, 8 * g)]) = mask4(vv[u], okmask(t < c));
        }
      }
    }
    __syncthreads();

    // U[d][n] += sum_t K~[t][d] G~[t][n]: A = K~^T (rows d), B = G~ (columns n)
#pragma unroll
    for (int p = 0; p < PER_WAVE; ++p) {
      const int tile = w + 8 * p;
      if (tile < NTILE) {
        const int td = tile / TN, tn = tile % TN;
        ColumnReaderTR<DK> acol(KS, 32 * td, l32, hi);
        ColumnReaderTR<DV> bcol(GS, 32 * tn, l32, hi);
        int kb0 = 0;
        for (; kb0 + 4 <= np / 16; kb0 += 4) {
#pragma unroll
          for (int kq = 0; kq < 4; ++kq) acc[p] = mfma32(acol(kq), bcol(kq), acc[p]);
          acol.advance();
          bcol.advance();
        }
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)  // the last, partial group (a piece of 32 tokens)
          if (kb0 + kq < np / 16) acc[p] = mfma32(acol(kq), bcol(kq), acc[p]);
      }
    }
    __syncthreads();  // before the next piece overwrites the buffers
  }

  // lane (n = l32, hi) of tile (td, tn) holds U[32 td + row_of(r, hi)][32 tn + l32]
  float* Ub = U + (static_cast<int64_t>(bh) * a.NC + ci) * DK * DV;
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p) {
    const int tile = w + 8 * p;
    if (tile < NTILE) {
      const int td = tile / TN, tn = tile % TN;
#pragma unroll
      for (int r = 0; r < 16; ++r) Ub[(32 * td + row_of(r, hi)) * DV + 32 * tn + l32] = acc[p][r];
    }
  }
}

// ---------------------------------------------------------------------------
// 2. The state recurrence over chunks, elementwise: thread = 4 consecutive
//    elements of one chain's W; U_i is replaced by W_i in place.
// ---------------------------------------------------------------------------
template <int DECAY>
__global__ __launch_bounds__(256) void lin_scan_kernel(FwdArgs a, const float* __restrict__ lam, float* U) {
  const int per_chain = a.dk * a.dv / 4;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(a.B) * a.H * per_chain) return;
  const int bh = static_cast<int>(gid / per_chain);
  const int e = 4 * static_cast<int>(gid % per_chain);
  const int d = e / a.dv;
  const int64_t wo = static_cast<int64_t>(bh) * a.dk * a.dv + e;
  float4 W = a.w0 ? *reinterpret_cast<const float4*>(a.w0 + wo) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float gam = (DECAY == 1) ? a.gamma[bh % a.H] : 1.0f;
  const int64_t stride = static_cast<int64_t>(a.dk) * a.dv;  // one chunk's state
  float* Up = U + static_cast<int64_t>(bh) * a.NC * stride + e;
  float* ck = a.w_ckpt ? a.w_ckpt + static_cast<int64_t>(bh) * a.NC * stride + e : nullptr;
  const float* lm = (DECAY == 2) ? lam + static_cast<int64_t>(bh) * a.NC * a.dk + d : nullptr;
  constexpr int kAhead = 4;  // chunks whose increments are loaded together
  for (int i0 = 0; i0 < a.NC; i0 += kAhead) {
    float4 u[kAhead];
    float l[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int i = min(i0 + j, a.NC - 1);
      u[j] = *reinterpret_cast<const float4*>(Up + i * stride);
      l[j] = (DECAY == 2) ? lm[static_cast<int64_t>(i) * a.dk] : gam;
    }
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int i = i0 + j;
      if (i < a.NC) {
        // W_i, read by the output kernel: from the checkpoints when they are kept
        if (ck) *reinterpret_cast<float4*>(ck + i * stride) = W;
        else *reinterpret_cast<float4*>(Up + i * stride) = W;
        W.x = l[j] * W.x - u[j].x; W.y = l[j] * W.y - u[j].y;
        W.z = l[j] * W.z - u[j].z; W.w = l[j] * W.w - u[j].w;
      }
    }
  }
  if (a.w_final) *reinterpret_cast<float4*>(a.w_final + wo) = W;
}

// The backward's dW chain in reverse, elementwise: dW_i = Lambda_i dW_{i+1} + R_i
// (Lambda: lambda_i row scale, gamma_h or 1), started from dW_T (or 0); the
// slot of R_i receives dW_{i+1}, the dW' that chunk i's backward reads, and
// dW_0 goes to dw0.
template <int DECAY>
__global__ __launch_bounds__(256) void lin_bscan_kernel(int BH, int H, int NC, int dk, int dv,
                                                        const float* __restrict__ gamma, const float* __restrict__ lam,
                                                        const float* __restrict__ d_wfinal, float* dWn,
                                                        float* __restrict__ dw0) {
  const int per_chain = dk * dv / 4;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(BH) * per_chain) return;
  const int bh = static_cast<int>(gid / per_chain);
  const int e = 4 * static_cast<int>(gid % per_chain);
  const int d = e / dv;
  const int64_t wo = static_cast<int64_t>(bh) * dk * dv + e;
  float4 dW = d_wfinal ? *reinterpret_cast<const float4*>(d_wfinal + wo) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float gam = (DECAY == 1) ? gamma[bh % H] : 1.0f;
  const int64_t stride = static_cast<int64_t>(dk) * dv;
  float* P = dWn + static_cast<int64_t>(bh) * NC * stride + e;
  const float* lm = (DECAY == 2) ? lam + static_cast<int64_t>(bh) * NC * dk + d : nullptr;
  constexpr int kAhead = 4;
  for (int i0 = NC - 1; i0 >= 0; i0 -= kAhead) {
    float4 r[kAhead];
    float l[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int i = max(i0 - j, 0);
      r[j] = *reinterpret_cast<const float4*>(P + i * stride);
      l[j] = (DECAY == 2) ? lm[static_cast<int64_t>(i) * dk] : gam;
    }
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int i = i0 - j;
      if (i >= 0) {
        *reinterpret_cast<float4*>(P + i * stride) = dW;  // dW_{i+1}
        dW.x = l[j] * dW.x + r[j].x; dW.y = l[j] * dW.y + r[j].y;
        dW.z = l[j] * dW.z + r[j].z; dW.w = l[j] * dW.w + r[j].w;
      }
    }
  }
  if (dw0) *reinterpret_cast<float4*>(dw0 + wo) = dW;
}

// ---------------------------------------------------------------------------
// 3. O_i = Q~_i W_i - Tril(Q~_i K~_i^T) G~_i, one workgroup per (chain, chunk)
//    covering every d_v column: the query view of the sequential kernel, with
//    W_i read from the scan's output.  Each score tile S is formed once and
//    multiplies all DV / 32 column blocks of G~.
// ---------------------------------------------------------------------------
// Eight rows of eight 16-bit values, transposed in registers: out[j] holds
// element j of every input row (row u in its 16-bit lane u).
__device__ __forceinline__ void transpose8x8(const uint32_t (&in)[8][4], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint16_t h[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      h[u] = static_cast<uint16_t>((j & 1) ? (in[u][j >> 1] >> 16) : (in[u][j >> 1] & 0xffffu));
    out[j] = make_uint4(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16),
                        h[4] | (static_cast<uint32_t>(h[5]) << 16), h[6] | (static_cast<uint32_t>(h[7]) << 16));
  }
}

// x (.) e^{m[j] - p[j]} (.) e^{p[j] - r[j]} for the 8 features of a fragment (vector
// decay), one factor at a time: for a query row of tile I (x = Q^m, m = M_I, p = P_I)
// the first brings Q^m down to Q e^{L - P_I} <= Q, so the second (e^{P_I - M_J},
// e^{-h_J} for the adjacent tile) cannot flush a product that is in range to zero,
// as e^{M_I - M_J} alone does once two tiles decay by e^{-88}.
__device__ __forceinline__ bf16x8_t scale_frag(bf16x8_t x, const float* m, const float* p, const float* r) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (from_bf(x[j]) * __expf(m[j] - p[j])) * __expf(p[j] - r[j]);
  return pack8(f);
}

template <int DK, int DV, int DECAY>
__global__ __launch_bounds__(kLinThreads) void lin_out_kernel(FwdArgs a, DecayPrep dp, const float* __restrict__ Wi) {
  constexpr bool VEC = DECAY == 2;
  __shared__ __attribute__((aligned(16))) uint16_t KS[kCMax * DK];  // K~ [t][d]; vector decay: then bf16(W_i)^T
  __shared__ __attribute__((aligned(16))) uint16_t GT[DV * kCMax];  // G~^T [n][t]
  __shared__ __attribute__((aligned(16))) uint16_t WTs[VEC ? 8 : DV * DK];  // bf16(W_i)^T [n][d]
  __shared__ float MT[VEC ? kCMax / 32 + 1 : 1][DK];  // vector decay: the tile midpoints M_I, and 0
  __shared__ float PT[VEC ? kCMax / 32 : 1][DK];      // vector decay: the prefixes P_I
  static_assert(!VEC || kCMax * DK >= DV * DK, "W_i^T fits where K^m was");
  uint16_t* WT = VEC ? KS : WTs;
  constexpr int NCB = DV / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int C = a.C, T = a.T;
  const int ci = blockIdx.x % a.NC;
  const int bh = blockIdx.x / a.NC;
  const int t0 = ci * C;
  const int c = min(C, T - t0);
  const int64_t offk = static_cast<int64_t>(bh) * T * DK;
  const int64_t offv = static_cast<int64_t>(bh) * T * DV;
  const bf16_t* ks = (DECAY == 2) ? dp.kt + offk : static_cast<const bf16_t*>(a.k) + offk;
  const bf16_t* qs = (DECAY == 2) ? dp.qt + offk : static_cast<const bf16_t*>(a.q) + offk;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + offv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * T;
  const float* W = Wi + (static_cast<int64_t>(bh) * a.NC + ci) * DK * DV;

  const int I = lin_tile_of_wave(w);
  const bool own = I * 32 < C;
  const int t = 32 * I + l32;

  // ---- loads, all issued before the first LDS write ----
  // K~ rows: 16-byte pieces
  constexpr int GK = DK / 8;
  constexpr int UK = kCMax * GK / kLinThreads;
  uint4 kk[UK];
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int idx = u * kLinThreads + tid, tr = idx / GK, g = idx % GK;
    kk[u] = *reinterpret_cast<const uint4*>(ks + static_cast<int64_t>(t0 + (tr < c ? tr : 0)) * DK + 8 * g);
  }
  // V: blocks of 8 tokens x 8 columns (G~^T is written transposed); one or two per thread
  constexpr int VB = (kCMax / 8) * (DV / 8);
  constexpr int UVB = (VB + kLinThreads - 1) / kLinThreads;
  uint32_t vb[UVB][8][4];
  float bt[UVB][8];
#pragma unroll
  for (int u = 0; u < UVB; ++u) {
    const int blk = min(u * kLinThreads + tid, VB - 1), ts = blk / (DV / 8), g = blk % (DV / 8);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tr = 8 * ts + r;
      const uint4 x = *reinterpret_cast<const uint4*>(v + static_cast<int64_t>(t0 + (tr < c ? tr : 0)) * DV + 8 * g);
      vb[u][r][0] = x.x; vb[u][r][1] = x.y; vb[u][r][2] = x.z; vb[u][r][3] = x.w;
      bt[u][r] = beta[t0 + (tr < c ? tr : 0)];
    }
  }
  // W_i: blocks of 8 rows d x 8 columns n, fp32 (vector decay: after the scores)
  constexpr int WB = (DK / 8) * (DV / 8);
  const int wblk = min(tid, WB - 1), wds = wblk / (DV / 8), wg = wblk % (DV / 8);
  float4 wr[8][2];
  auto load_w = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float* p = W + static_cast<int64_t>(8 * wds + r) * DV + 8 * wg;
      wr[r][0] = *reinterpret_cast<const float4*>(p);
      wr[r][1] = *reinterpret_cast<const float4*>(p + 4);
    }
  };
  auto store_w = [&]() {
    if (tid < WB) {
      uint32_t wb[8][4];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float f[8] = {wr[r][0].x, wr[r][0].y, wr[r][0].z, wr[r][0].w, wr[r][1].x, wr[r][1].y, wr[r][1].z, wr[r][1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wb[r][j] = static_cast<uint32_t>(bf_bits(to_bf(f[2 * j]))) | (static_cast<uint32_t>(bf_bits(to_bf(f[2 * j + 1]))) << 16);
      }
      uint4 tb[8];
      transpose8x8(wb, tb);
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(&WT[swz<DK>(8 * wg + j, 8 * wds)]) = tb[j];
    }
  };
  if constexpr (!VEC) load_w();
  float mlp[2] = {0.0f, 0.0f}, plp[2] = {0.0f, 0.0f};  // vector decay: this thread's M_I and P_I
  if constexpr (VEC) {
    const int ntile = C / 32;
    const float* lp = dp.lpre + (static_cast<int64_t>(bh) * a.NC + ci) * (ntile + 1) * DK;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = u * kLinThreads + tid, I = i / DK, d = i % DK;
      if (I < ntile) {
        plp[u] = lp[I * DK + d];
        mlp[u] = 0.5f * (plp[u] + lp[(I + 1) * DK + d]);
      }
    }
  }
  bf16x8_t qf[DK / 16];
  load_row_frags<DK / 16>(qf, qs, DK, t0, t, c, 0, hi);

  // ---- LDS writes ----
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int idx = u * kLinThreads + tid, tr = idx / GK, g = idx % GK;
    if (tr < C) *reinterpret_cast<uint4*>(&KS[swz<DK>(tr, 8 * g)]) = mask4(kk[u], okmask(tr < c));
  }
#pragma unroll
  for (int u = 0; u < UVB; ++u) {
    const int blk = u * kLinThreads + tid, ts = blk / (DV / 8), g = blk % (DV / 8);
    if (blk < VB && 8 * ts < C) {
      // G~ = -eta v for the block's 8 tokens (0 past the chunk), then transposed
      uint32_t gb[8][4];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float e = (8 * ts + r < c) ? -lr_gate(bt[u][r], a.b) : 0.0f;
        float f[8];
        unpack8(make_uint4(vb[u][r][0], vb[u][r][1], vb[u][r][2], vb[u][r][3]), f);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          gb[r][j] = static_cast<uint32_t>(bf_bits(to_bf(e * f[2 * j]))) |
                     (static_cast<uint32_t>(bf_bits(to_bf(e * f[2 * j + 1]))) << 16);
      }
      uint4 tb[8];
      transpose8x8(gb, tb);
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(&GT[swz<kCMax>(8 * g + j, 8 * ts)]) = tb[j];
    }
  }
  if constexpr (!VEC) store_w();
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = u * kLinThreads + tid, I = i / DK, d = i % DK;
      if (I < C / 32) {
        MT[I][d] = mlp[u];
        PT[I][d] = plp[u];
      }
    }
    if (tid < DK) MT[VEC ? kCMax / 32 : 0][tid] = 0.0f;
  }
  __syncthreads();

  // Y^T = W^T Q~^T - G~^T Tril(S)^T per column block; lane (t, hi) holds
  // Y[t][32 cb + row_of(r, hi)].  Vector decay: the scores first (K^m leaves KS
  // for W_i afterwards), then W^T Q~^T with Q~ = Q^m e^{M_I}.
  f32x16_t y[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) y[cb] = zero16();
  auto w_term = [&]() {
#pragma unroll
    for (int kb = 0; kb < DK / 16; ++kb) {
      bf16x8_t qq = qf[kb];
      if constexpr (VEC)  // Q~ = Q^m e^{M_I} = (Q^m e^{M_I - P_I}) e^{P_I}
        qq = scale_frag(qq, &MT[I][16 * kb + 8 * hi], &PT[I][16 * kb + 8 * hi], &MT[kCMax / 32][16 * kb + 8 * hi]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        y[cb] = mfma32(*reinterpret_cast<const bf16x8_t*>(&WT[swz<DK>(32 * cb + l32, 16 * kb + 8 * hi)]), qq, y[cb]);
    }
  };
  if (own) {
    if constexpr (!VEC) w_term();
    for (int J = 0; J <= I; ++J) {
      f32x16_t s = zero16();  // lane (t, hi) holds S[t][32 J + row_of(r, hi)]
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb) {
        bf16x8_t qq = qf[kb];
        // across tiles: e^{M_I - M_J} per feature (<= 1); inside the tile Q^m K^m as they are
        if constexpr (VEC) {
          if (J < I)
            qq = scale_frag(qq, &MT[I][16 * kb + 8 * hi], &PT[I][16 * kb + 8 * hi], &MT[J][16 * kb + 8 * hi]);
        }
        s = mfma32(*reinterpret_cast<const bf16x8_t*>(&KS[swz<DK>(32 * J + l32, 16 * kb + 8 * hi)]), qq, s);
      }
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
        const bf16x8_t B = pack8(nb);
        const int s0 = 32 * J + 16 * m + 4 * hi;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x4_t g0 = *reinterpret_cast<const bf16x4_t*>(&GT[swz<kCMax>(32 * cb + l32, s0)]);
          const bf16x4_t g1 = *reinterpret_cast<const bf16x4_t*>(&GT[swz<kCMax>(32 * cb + l32, s0 + 8)]);
          y[cb] = mfma32(cat44(g0, g1), B, y[cb]);
        }
      }
    }
  }
  if constexpr (VEC) {
    load_w();
    __syncthreads();  // every wave is done with K^m
    store_w();
    __syncthreads();
    if (own) w_term();
  }
  if (own) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float of[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) of[r] = y[cb][r];
      store_row16_x2(static_cast<bf16_t*>(a.o) + offv, DV, t0, t, c, 32 * cb, hi, of);
    }
  }
}

template <int DK>
hipError_t launch_state(const LinStateArgs& la, int dv, hipStream_t s) {
  const unsigned nchunk = static_cast<unsigned>(la.B * la.H * la.NC);
  KernelScope timing(TTT_KERNEL_LIN_STATE, s);
  switch (dv) {
    case 32: hipLaunchKernelGGL((lin_state_kernel<DK, 32>), dim3(nchunk), dim3(kLinThreads), 0, s, la); break;
    case 64: hipLaunchKernelGGL((lin_state_kernel<DK, 64>), dim3(nchunk), dim3(kLinThreads), 0, s, la); break;
    default: hipLaunchKernelGGL((lin_state_kernel<DK, 128>), dim3(nchunk), dim3(kLinThreads), 0, s, la); break;
  }
  return hipGetLastError();
}

template <int DK, int DECAY>
hipError_t launch_linear(const FwdArgs& a, const DecayPrep& dp, uint16_t* gh, float* U, hipStream_t s) {
  const unsigned nchunk = static_cast<unsigned>(a.B * a.H * a.NC);
  {
    const LinStateArgs la{a.B, a.H, a.T, a.C, a.NC, a.b,
                          (DECAY == 2) ? dp.kt : static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.v),
                          a.beta, U, gh, dp.lpre, DECAY == 2 ? 1 : 0};
    hipError_t e = launch_state<DK>(la, a.dv, s);
    if (e != hipSuccess) return e;
  }
  {
    KernelScope timing(TTT_KERNEL_LIN_SCAN, s);
    const int64_t threads = static_cast<int64_t>(a.B) * a.H * a.dk * a.dv / 4;
    hipLaunchKernelGGL((lin_scan_kernel<DECAY>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, a,
                       dp.lam, U);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // W_i: the checkpoints when the caller keeps them, else the scan's copy in U
  const float* Wi = a.w_ckpt ? a.w_ckpt : U;
  KernelScope timing(TTT_KERNEL_LIN_OUT, s);
  switch (a.dv) {
    case 32: hipLaunchKernelGGL((lin_out_kernel<DK, 32, DECAY>), dim3(nchunk), dim3(kLinThreads), 0, s, a, dp, Wi); break;
    case 64: hipLaunchKernelGGL((lin_out_kernel<DK, 64, DECAY>), dim3(nchunk), dim3(kLinThreads), 0, s, a, dp, Wi); break;
    default: hipLaunchKernelGGL((lin_out_kernel<DK, 128, DECAY>), dim3(nchunk), dim3(kLinThreads), 0, s, a, dp, Wi); break;
  }
  return hipGetLastError();
}

template <int DK>
hipError_t linear_by_decay(const FwdArgs& a, const DecayPrep& dp, uint16_t* gh, float* U, hipStream_t s) {
  if (a.decay == TTT_DECAY_VECTOR) return launch_linear<DK, 2>(a, dp, gh, U, s);
  if (a.decay == TTT_DECAY_SCALAR) return launch_linear<DK, 1>(a, dp, gh, U, s);
  return launch_linear<DK, 0>(a, dp, gh, U, s);
}

template <int DK>
hipError_t linear_bwd_by_dk(const BwdArgs& a, const DecayPrep& dp, float* dWn, hipStream_t s) {
  // R_i = Q~_i^T dO_i (dY = dO without an act) into the dW' slots
  const LinStateArgs la{a.B, a.H, a.T, a.C, a.NC, a.b,
                        (a.decay == TTT_DECAY_VECTOR) ? dp.qt : static_cast<const bf16_t*>(a.q),
                        static_cast<const bf16_t*>(a.d_o), nullptr, dWn, nullptr, dp.lpre,
                        a.decay == TTT_DECAY_VECTOR ? 2 : 0};
  hipError_t e = launch_state<DK>(la, a.dv, s);
  if (e != hipSuccess) return e;
  KernelScope timing(TTT_KERNEL_LIN_SCAN, s);
  const int64_t threads = static_cast<int64_t>(a.B) * a.H * a.dk * a.dv / 4;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  const int BH = a.B * a.H;
  if (a.decay == TTT_DECAY_VECTOR)
    hipLaunchKernelGGL(lin_bscan_kernel<2>, grid, dim3(256), 0, s, BH, a.H, a.NC, a.dk, a.dv, a.gamma, dp.lam,
                       a.d_wfinal, dWn, a.dw0);
  else if (a.decay == TTT_DECAY_SCALAR)
    hipLaunchKernelGGL(lin_bscan_kernel<1>, grid, dim3(256), 0, s, BH, a.H, a.NC, a.dk, a.dv, a.gamma, dp.lam,
                       a.d_wfinal, dWn, a.dw0);
  else
    hipLaunchKernelGGL(lin_bscan_kernel<0>, grid, dim3(256), 0, s, BH, a.H, a.NC, a.dk, a.dv, a.gamma, dp.lam,
                       a.d_wfinal, dWn, a.dw0);
  return hipGetLastError();
}

}  // namespace

// The backward's dW chain on the same condition (the rest of the backward is
// the two-kernel backward, with the reverse sweep taken chunk by chunk).
bool linear_bwd_applies(const BwdArgs& a) {
  const bool shape_ok = a.loss == TTT_LOSS_IP && a.act == TTT_ACT_NONE && a.dtype == TTT_BF16 &&
                        (a.dk == 64 || a.dk == 128) && (a.dv == 32 || a.dv == 64 || a.dv == 128) &&
                        (a.C == 32 || a.C == 64 || a.C == 128 || a.C == 256);
  return shape_ok && static_cast<int64_t>(a.B) * a.H * (a.dv / kLinNB) * 2 <= device_cu_count();
}

hipError_t linear_bwd_chain(const BwdArgs& a, const DecayPrep& dp, float* dWn, hipStream_t s) {
  return a.dk == 128 ? linear_bwd_by_dk<128>(a, dp, dWn, s) : linear_bwd_by_dk<64>(a, dp, dWn, s);
}

// Taken when the sequential kernel would leave half of the GPU or more idle:
// its B * H * d_v / 32 workgroups, one per CU, at most half of the CUs.  With
// more chains the sequential kernel is faster (it pipelines chunk after chunk
// and moves no per-chunk state through HBM).
bool linear_fwd_applies(const FwdArgs& a) {
  const bool shape_ok = a.loss == TTT_LOSS_IP && a.act == TTT_ACT_NONE && mfma_fwd_supported(a) &&
                        (a.dv == 32 || a.dv == 64 || a.dv == 128);
  return shape_ok && static_cast<int64_t>(a.B) * a.H * (a.dv / kLinNB) * 2 <= device_cu_count();
}

// Workspace: [decay preparation (vector decay without a saved context)] [U / W_i].
size_t linear_fwd_workspace(const FwdArgs& a) {
  size_t n = 0;
  if (a.decay == TTT_DECAY_VECTOR) n += decay_prep_layout(a.B, a.H, a.T, a.dk, a.C, a.NC, nullptr, nullptr);
  return n + align256(static_cast<size_t>(a.B) * a.H * a.NC * a.dk * a.dv * sizeof(float));
}

hipError_t linear_fwd_launch(const FwdArgs& a, hipStream_t s) {
  SavedCtx sv{};
  if (a.saved) mfma_saved_layout(a.B, a.H, a.T, a.dk, a.dv, a.C, a.NC, a.act, a.decay, &sv, a.saved);
  DecayPrep dp{};
  size_t off = 0;
  if (a.decay == TTT_DECAY_VECTOR) {
    const size_t n = decay_prep_layout(a.B, a.H, a.T, a.dk, a.C, a.NC, nullptr, nullptr);
    if (a.saved) dp = sv.prep;
    else decay_prep_layout(a.B, a.H, a.T, a.dk, a.C, a.NC, &dp, a.ws);
    off = n;
    hipError_t e = decay_prep_launch(a.log_decay, a.q, a.k, a.B, a.H, a.T, a.dk, a.C, a.NC, dp, s);
    if (e != hipSuccess) return e;
  }
  float* U = reinterpret_cast<float*>(a.ws + off);
  return a.dk == 128 ? linear_by_decay<128>(a, dp, sv.gh, U, s) : linear_by_decay<64>(a, dp, sv.gh, U, s);
}

}  // namespace ttt
