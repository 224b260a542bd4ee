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
//   vector: W_{i+1} = lambda_i (.) (W_i - K~_i^T G~_i)      (row scale, K_bar = K~ lambda)
// is then an affine recurrence whose increments U_i = K~_i^T G~_i are
// independent of each other, and the query view of a chunk
//   O_i = Q~_i W_i - Tril(Q~_i K~_i^T) G~_i
// needs only its own chunk and W_i.  So the forward runs as three launches:
//   1. lin_state_kernel: U_i for every (chain, chunk) at once (and G~ into the
//      saved context for the backward);
//   2. lin_scan_kernel: W_i for every chunk by the recurrence above, elementwise
//      (fp32), written over U_i in place, to the checkpoints and to w_final;
//   3. lin_out_kernel: O_i for every (chain, chunk, 32-column block) at once.
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
constexpr int kLinNB = 32;        // d_v columns per lin_out workgroup

__device__ __forceinline__ int lin_tile_of_wave(int w) { return w < 4 ? w : 11 - w; }

// ---------------------------------------------------------------------------
// 1. U_i = K~_i^T G~_i, one workgroup per (chain, chunk).
// ---------------------------------------------------------------------------
// K~ [C][DK] and G~ [C][DV] are staged as they lie (rows = tokens, swizzled);
// both operands of the contraction over tokens are column reads
// (ColumnReaderTR).  The DK x DV output has (DK / 32) x (DV / 32) tiles of
// 32 x 32; wave w takes tiles w, w + 8, ...
template <int DK, int DV, int DECAY>
__global__ __launch_bounds__(kLinThreads) void lin_state_kernel(FwdArgs a, DecayPrep dp, float* __restrict__ U,
                                                                uint16_t* __restrict__ gh) {
  __shared__ __attribute__((aligned(16))) uint16_t KS[kCMax * DK];  // K~ [t][d]
  __shared__ __attribute__((aligned(16))) uint16_t GS[kCMax * DV];  // G~ [t][n]
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
  const bf16_t* ks = (DECAY == 2) ? dp.kt + offk : static_cast<const bf16_t*>(a.k) + offk;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + offv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * T;

  // staging: every load first (rows >= c read row 0, zeroed when written)
  constexpr int GK = DK / 8, GV = DV / 8;
  constexpr int UK = kCMax * GK / kLinThreads, UV = kCMax * GV / kLinThreads;
  uint4 kk[UK], vv[UV];
  float et[UV];
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int idx = u * kLinThreads + tid, t = idx / GK, g = idx % GK;
    kk[u] = *reinterpret_cast<const uint4*>(ks + static_cast<int64_t>(t0 + (t < c ? t : 0)) * DK + 8 * g);
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int idx = u * kLinThreads + tid, t = idx / GV, g = idx % GV;
    vv[u] = *reinterpret_cast<const uint4*>(v + static_cast<int64_t>(t0 + (t < c ? t : 0)) * DV + 8 * g);
    et[u] = beta[t0 + (t < c ? t : 0)];
  }
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int idx = u * kLinThreads + tid, t = idx / GK, g = idx % GK;
    if (t < C) *reinterpret_cast<uint4*>(&KS[swz<DK>(t, 8 * g)]) = mask4(kk[u], okmask(t < c));
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int idx = u * kLinThreads + tid, t = idx / GV, g = idx % GV;
    if (t < C) {
      // G~ = eta (.) G = -eta v (inner-product loss, no activation); 0 past the chunk
      const float e = (t < c) ? -lr_gate(et[u], a.b) : 0.0f;
      float f[8];
      unpack8(vv[u], f);
      float gf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) gf[j] = e * f[j];
      const bf16x8_t x = pack8(gf);
      *reinterpret_cast<bf16x8_t*>(&GS[swz<DV>(t, 8 * g)]) = x;
      if (gh && t < c) *reinterpret_cast<bf16x8_t*>(gh + offv + static_cast<int64_t>(t0 + t) * DV + 8 * g) = x;
    }
  }
  __syncthreads();

  // U[d][n] = sum_t K~[t][d] G~[t][n]: A = K~^T (rows d), B = G~ (columns n);
  // lane (n = l32, hi) of tile (td, tn) holds U[32 td + row_of(r, hi)][32 tn + l32]
  float* Ub = U + (static_cast<int64_t>(bh) * a.NC + ci) * DK * DV;
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p) {
    const int tile = w + 8 * p;
    if (tile < NTILE) {
      const int td = tile / TN, tn = tile % TN;
      ColumnReaderTR<DK> acol(KS, 32 * td, l32, hi);
      ColumnReaderTR<DV> bcol(GS, 32 * tn, l32, hi);
      f32x16_t acc = zero16();
      int kb0 = 0;
      for (; kb0 + 4 <= C / 16; kb0 += 4) {
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) acc = mfma32(acol(kq), bcol(kq), acc);
        acol.advance();
        bcol.advance();
      }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)  // the last, partial group (C = 32)
        if (kb0 + kq < C / 16) acc = mfma32(acol(kq), bcol(kq), acc);
#pragma unroll
      for (int r = 0; r < 16; ++r) Ub[(32 * td + row_of(r, hi)) * DV + 32 * tn + l32] = acc[r];
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
        *reinterpret_cast<float4*>(Up + i * stride) = W;  // W_i, read by the output kernel
        if (ck) *reinterpret_cast<float4*>(ck + i * stride) = W;
        if constexpr (DECAY == 2) {
          W.x = l[j] * (W.x - u[j].x); W.y = l[j] * (W.y - u[j].y);
          W.z = l[j] * (W.z - u[j].z); W.w = l[j] * (W.w - u[j].w);
        } else {
          W.x = l[j] * W.x - u[j].x; W.y = l[j] * W.y - u[j].y;
          W.z = l[j] * W.z - u[j].z; W.w = l[j] * W.w - u[j].w;
        }
      }
    }
  }
  if (a.w_final) *reinterpret_cast<float4*>(a.w_final + wo) = W;
}

// ---------------------------------------------------------------------------
// 3. O_i = Q~_i W_i - Tril(Q~_i K~_i^T) G~_i, one workgroup per (chain, chunk,
//    32-column block); the query view of the sequential kernel, with W_i read
//    from the scan's output.
// ---------------------------------------------------------------------------
template <int DK, int DECAY>
__global__ __launch_bounds__(kLinThreads) void lin_out_kernel(FwdArgs a, DecayPrep dp, const float* __restrict__ Wi) {
  __shared__ __attribute__((aligned(16))) uint16_t KS[kCMax * DK];    // K~ [t][d]
  __shared__ __attribute__((aligned(16))) uint16_t GT[kLinNB * kCMax];  // G~^T [n][t]
  __shared__ __attribute__((aligned(16))) uint16_t WT[kLinNB * DK];     // bf16(W_i)^T [n][d]
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int C = a.C, T = a.T, dv = a.dv;
  const int ncb = dv / kLinNB;
  const int L = xcd_remap(blockIdx.x, gridDim.x);  // the column blocks of a chunk on one XCD
  const int cb = L % ncb;
  const int ci = (L / ncb) % a.NC;
  const int bh = L / (ncb * a.NC);
  const int col0 = cb * kLinNB;
  const int t0 = ci * C;
  const int c = min(C, T - t0);
  const int64_t offk = static_cast<int64_t>(bh) * T * DK;
  const int64_t offv = static_cast<int64_t>(bh) * T * dv;
  const bf16_t* ks = (DECAY == 2) ? dp.kt + offk : static_cast<const bf16_t*>(a.k) + offk;
  const bf16_t* qs = (DECAY == 2) ? dp.qt + offk : static_cast<const bf16_t*>(a.q) + offk;
  const bf16_t* v = static_cast<const bf16_t*>(a.v) + offv;
  const float* beta = a.beta + static_cast<int64_t>(bh) * T;
  const float* W = Wi + (static_cast<int64_t>(bh) * a.NC + ci) * DK * dv;

  const int I = lin_tile_of_wave(w);
  const bool own = I * 32 < C;
  const int t = 32 * I + l32;

  // loads: K~ rows, this block's V columns with eta, W_i columns, own Q~ rows
  constexpr int GK = DK / 8;
  constexpr int UK = kCMax * GK / kLinThreads;
  constexpr int UV = kCMax * (kLinNB / 8) / kLinThreads;  // 2
  uint4 kk[UK], vv[UV];
  float et[UV];
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int idx = u * kLinThreads + tid, tr = idx / GK, g = idx % GK;
    kk[u] = *reinterpret_cast<const uint4*>(ks + static_cast<int64_t>(t0 + (tr < c ? tr : 0)) * DK + 8 * g);
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int idx = u * kLinThreads + tid, tr = idx / (kLinNB / 8), g = idx % (kLinNB / 8);
    vv[u] = *reinterpret_cast<const uint4*>(v + static_cast<int64_t>(t0 + (tr < c ? tr : 0)) * dv + col0 + 8 * g);
    et[u] = beta[t0 + (tr < c ? tr : 0)];
  }
  // W_i rows d, columns col0 + 8 g .. +7 (DK * 4 pieces <= 512 threads)
  const int wd = tid / (kLinNB / 8), wg = tid % (kLinNB / 8);
  float4 w0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), w1 = w0;
  if (wd < DK) {
    w0 = *reinterpret_cast<const float4*>(W + static_cast<int64_t>(wd) * dv + col0 + 8 * wg);
    w1 = *reinterpret_cast<const float4*>(W + static_cast<int64_t>(wd) * dv + col0 + 8 * wg + 4);
  }
  bf16x8_t qf[DK / 16];
  load_row_frags<DK / 16>(qf, qs, DK, t0, t, c, 0, hi);

#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int idx = u * kLinThreads + tid, tr = idx / GK, g = idx % GK;
    if (tr < C) *reinterpret_cast<uint4*>(&KS[swz<DK>(tr, 8 * g)]) = mask4(kk[u], okmask(tr < c));
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int idx = u * kLinThreads + tid, tr = idx / (kLinNB / 8), g = idx % (kLinNB / 8);
    if (tr < C) {
      const float e = (tr < c) ? -lr_gate(et[u], a.b) : 0.0f;  // G~ = -eta v
      float f[8];
      unpack8(vv[u], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) GT[swz<kCMax>(8 * g + j, tr)] = bf_bits(to_bf(e * f[j]));
    }
  }
  if (wd < DK) {
    const float f[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) WT[swz<DK>(8 * wg + j, wd)] = bf_bits(to_bf(f[j]));
  }
  __syncthreads();

  if (own) {
    // Y^T = W^T Q~^T - G~^T Tril(S)^T; lane (t, hi) holds Y[t][n = row_of(r, hi)]
    f32x16_t y = zero16();
#pragma unroll
    for (int kb = 0; kb < DK / 16; ++kb)
      y = mfma32(*reinterpret_cast<const bf16x8_t*>(&WT[swz<DK>(l32, 16 * kb + 8 * hi)]), qf[kb], y);
    for (int J = 0; J <= I; ++J) {
      f32x16_t s = zero16();  // lane (t, hi) holds S[t][32 J + row_of(r, hi)]
#pragma unroll
      for (int kb = 0; kb < DK / 16; ++kb)
        s = mfma32(*reinterpret_cast<const bf16x8_t*>(&KS[swz<DK>(32 * J + l32, 16 * kb + 8 * hi)]), qf[kb], s);
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
    float of[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) of[r] = y[r];
    store_row16_x2(static_cast<bf16_t*>(a.o) + offv, dv, t0, t, c, col0, hi, of);
  }
}

template <int DK, int DECAY>
hipError_t launch_linear(const FwdArgs& a, const DecayPrep& dp, uint16_t* gh, float* U, hipStream_t s) {
  const unsigned nchunk = static_cast<unsigned>(a.B * a.H * a.NC);
  {
    KernelScope timing(TTT_KERNEL_LIN_STATE, s);
    switch (a.dv) {
      case 32: hipLaunchKernelGGL((lin_state_kernel<DK, 32, DECAY>), dim3(nchunk), dim3(kLinThreads), 0, s, a, dp, U, gh); break;
      case 64: hipLaunchKernelGGL((lin_state_kernel<DK, 64, DECAY>), dim3(nchunk), dim3(kLinThreads), 0, s, a, dp, U, gh); break;
      default: hipLaunchKernelGGL((lin_state_kernel<DK, 128, DECAY>), dim3(nchunk), dim3(kLinThreads), 0, s, a, dp, U, gh); break;
    }
    hipError_t e = hipGetLastError();
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
  KernelScope timing(TTT_KERNEL_LIN_OUT, s);
  hipLaunchKernelGGL((lin_out_kernel<DK, DECAY>), dim3(nchunk * (a.dv / kLinNB)), dim3(kLinThreads), 0, s, a, dp,
                     static_cast<const float*>(U));
  return hipGetLastError();
}

template <int DK>
hipError_t linear_by_decay(const FwdArgs& a, const DecayPrep& dp, uint16_t* gh, float* U, hipStream_t s) {
  if (a.decay == TTT_DECAY_VECTOR) return launch_linear<DK, 2>(a, dp, gh, U, s);
  if (a.decay == TTT_DECAY_SCALAR) return launch_linear<DK, 1>(a, dp, gh, U, s);
  return launch_linear<DK, 0>(a, dp, gh, U, s);
}

}  // namespace

// Taken when the sequential kernel would leave most of the GPU idle: its
// B * H * d_v / 32 workgroups, one per CU, at most a quarter of the CUs.  With
// more chains the sequential kernel is faster (it pipelines chunk after chunk
// and moves no per-chunk state through HBM): measured at B * H = 16, T = 32768
// the chunk-parallel forward takes 0.48 ms against 0.70 ms, at B * H = 64,
// T = 4096 0.24 ms against 0.14 ms.
bool linear_fwd_applies(const FwdArgs& a) {
  const bool shape_ok = a.loss == TTT_LOSS_IP && a.act == TTT_ACT_NONE && mfma_fwd_supported(a) &&
                        (a.dv == 32 || a.dv == 64 || a.dv == 128);
  return shape_ok && static_cast<int64_t>(a.B) * a.H * (a.dv / kLinNB) * 4 <= device_cu_count();
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
