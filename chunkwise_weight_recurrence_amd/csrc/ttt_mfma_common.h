// Device pieces shared by the matrix-core forward and backward kernels.
//
// Chunk staging: eta, the transition's row scale lambda, and the decay-scaled
// keys and queries of one chunk, written to LDS as bf16 with the 16-byte
// granule XOR swizzle of mfma_util.h.
//   none / scalar decay: K~ = K, Q~ = Q, lambda = 1 / gamma_h;
//   vector decay: L = inclusive cumsum of log a over the chunk's tokens,
//     K~ = K e^-L, Q~ = Q e^L, lambda = e^{L_last}  (Modular TTT summary page,
//     "Prerequisites", weight decay: per-feature decay as in linear attention).
// Global loads are issued in unrolled batches so that many are in flight.
#pragma once

#include "mfma_util.h"
#include "ttt_device.h"

namespace ttt {

constexpr int kMfmaThreads = 256;  // 4 waves per workgroup
constexpr int kCMax = 256;         // largest chunk on the matrix-core path

__device__ __forceinline__ void unpack8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

// Fill ETA[0..C), LAM[0..DK), KS = K~ [C][DK], QS = Q~ [C][DK] for the chunk
// starting at token t0 with c valid tokens (rows >= c are zero).  `scratch`
// needs (256 / (DK/8)) * DK floats for the vector-decay slice totals.  Ends
// with a workgroup barrier.
template <int DK, int DECAY>
__device__ __forceinline__ void stage_chunk(uint16_t* KS, uint16_t* QS, float* ETA, float* LAM, float* scratch,
                                            const bf16_t* k, const bf16_t* q, const float* la,
                                            const float* beta, float b, float gamma_h, int t0, int c, int C) {
  const int tid = threadIdx.x;
  for (int t = tid; t < C; t += kMfmaThreads) ETA[t] = (t < c) ? lr_gate(beta[t0 + t], b) : 0.0f;
  constexpr int G = DK / 8;
  if constexpr (DECAY != 2) {
    for (int d = tid; d < DK; d += kMfmaThreads) LAM[d] = (DECAY == 1) ? gamma_h : 1.0f;
    const int total = C * G;
    constexpr int U = 8;
    for (int base = 0; base < total; base += kMfmaThreads * U) {
      uint4 kk[U], qq[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = base + u * kMfmaThreads + tid;
        const int t = idx / G, g = idx % G;
        kk[u] = make_uint4(0, 0, 0, 0);
        qq[u] = make_uint4(0, 0, 0, 0);
        if (idx < total && t < c) {
          kk[u] = *reinterpret_cast<const uint4*>(k + static_cast<int64_t>(t0 + t) * DK + 8 * g);
          qq[u] = *reinterpret_cast<const uint4*>(q + static_cast<int64_t>(t0 + t) * DK + 8 * g);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = base + u * kMfmaThreads + tid;
        if (idx < total) {
          const int t = idx / G, g = idx % G;
          *reinterpret_cast<uint4*>(&KS[swz<DK>(t, 8 * g)]) = kk[u];
          *reinterpret_cast<uint4*>(&QS[swz<DK>(t, 8 * g)]) = qq[u];
        }
      }
    }
  } else {
    // thread = (token slice sl, feature group g of 8 features)
    constexpr int NSL = kMfmaThreads / G;
    const int g = tid % G, sl = tid / G;
    const int tps = C / NSL;
    float tot[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tot[j] = 0.0f;
    constexpr int U1 = 8;
    for (int i0 = 0; i0 < tps; i0 += U1) {
      float4 x0[U1], x1[U1];
#pragma unroll
      for (int u = 0; u < U1; ++u) {
        const int t = sl * tps + i0 + u;
        x0[u] = x1[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i0 + u < tps && t < c) {
          const float* p = la + static_cast<int64_t>(t0 + t) * DK + 8 * g;
          x0[u] = *reinterpret_cast<const float4*>(p);
          x1[u] = *reinterpret_cast<const float4*>(p + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < U1; ++u) {
        tot[0] += x0[u].x; tot[1] += x0[u].y; tot[2] += x0[u].z; tot[3] += x0[u].w;
        tot[4] += x1[u].x; tot[5] += x1[u].y; tot[6] += x1[u].z; tot[7] += x1[u].w;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) scratch[sl * DK + 8 * g + j] = tot[j];
    __syncthreads();
    float run[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) run[j] = 0.0f;
    for (int s = 0; s < sl; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) run[j] += scratch[s * DK + 8 * g + j];
    constexpr int U2 = 4;
    for (int i0 = 0; i0 < tps; i0 += U2) {
      float4 x0[U2], x1[U2];
      uint4 kk[U2], qq[U2];
#pragma unroll
      for (int u = 0; u < U2; ++u) {
        const int t = sl * tps + i0 + u;
        x0[u] = x1[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        kk[u] = qq[u] = make_uint4(0, 0, 0, 0);
        if (i0 + u < tps && t < c) {
          const float* p = la + static_cast<int64_t>(t0 + t) * DK + 8 * g;
          x0[u] = *reinterpret_cast<const float4*>(p);
          x1[u] = *reinterpret_cast<const float4*>(p + 4);
          kk[u] = *reinterpret_cast<const uint4*>(k + static_cast<int64_t>(t0 + t) * DK + 8 * g);
          qq[u] = *reinterpret_cast<const uint4*>(q + static_cast<int64_t>(t0 + t) * DK + 8 * g);
        }
      }
#pragma unroll
      for (int u = 0; u < U2; ++u) {
        if (i0 + u >= tps) break;
        const int t = sl * tps + i0 + u;
        run[0] += x0[u].x; run[1] += x0[u].y; run[2] += x0[u].z; run[3] += x0[u].w;
        run[4] += x1[u].x; run[5] += x1[u].y; run[6] += x1[u].z; run[7] += x1[u].w;
        float kf[8], qf[8], kt[8], qt[8];
        unpack8(kk[u], kf);
        unpack8(qq[u], qf);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kt[j] = kf[j] * __expf(-run[j]);
          qt[j] = qf[j] * __expf(run[j]);
        }
        *reinterpret_cast<bf16x8_t*>(&KS[swz<DK>(t, 8 * g)]) = pack8(kt);
        *reinterpret_cast<bf16x8_t*>(&QS[swz<DK>(t, 8 * g)]) = pack8(qt);
      }
    }
    if (sl == NSL - 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) LAM[8 * g + j] = __expf(run[j]);
    }
  }
  __syncthreads();
}

// Stage the raw keys K [C][DK] of a chunk (rows >= c zero) into LDS; no barrier.
template <int DK>
__device__ __forceinline__ void stage_raw_k(uint16_t* KR, const bf16_t* k, int t0, int c, int C) {
  const int tid = threadIdx.x;
  constexpr int G = DK / 8;
  const int total = C * G;
  constexpr int U = 8;
  for (int base = 0; base < total; base += kMfmaThreads * U) {
    uint4 kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * kMfmaThreads + tid;
      const int t = idx / G, g = idx % G;
      kk[u] = make_uint4(0, 0, 0, 0);
      if (idx < total && t < c) kk[u] = *reinterpret_cast<const uint4*>(k + static_cast<int64_t>(t0 + t) * DK + 8 * g);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * kMfmaThreads + tid;
      if (idx < total) *reinterpret_cast<uint4*>(&KR[swz<DK>(idx / G, 8 * (idx % G))]) = kk[u];
    }
  }
}

// Workgroup id remap: hardware hands block L to XCD L % 8; this places the
// d_v column blocks of one chain (consecutive after the remap) on one XCD.
__device__ __forceinline__ int xcd_remap(int L, int nblk) {
  if ((nblk & 7) == 0) return (L & 7) * (nblk >> 3) + (L >> 3);
  return L;
}

}  // namespace ttt
