// Device pieces shared by the matrix-core forward and backward kernels.
//
// Chunk staging: eta, the transition's row scale lambda, and the decay-scaled
// keys and queries of one chunk, written to LDS as bf16 with the 16-byte
// granule XOR swizzle of mfma_util.h.
//   none / scalar decay: K~ = K, Q~ = Q, lambda = 1 (none) or gamma_h (scalar);
//   vector decay: K~ = K e^-L, Q~ = Q e^L, lambda = e^{L_last} with L the
//     in-chunk cumsum of log a (Modular TTT summary page, "Prerequisites",
//     weight decay), prepared once per chunk by ttt_decay_prep.hip.
// Global loads are issued in unrolled batches so that many are in flight.
#pragma once

#include "mfma_util.h"
#include "ttt_device.h"

namespace ttt {

constexpr int kMfmaThreads = 256;  // 4 waves per workgroup
constexpr int kCMax = 256;         // largest chunk on the matrix-core path

// Bitwise zeroing of a loaded value without a branch (a branch that overwrote a
// load's destination would have to wait for the load first).
__device__ __forceinline__ uint4 mask4(uint4 x, uint32_t m) { return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m); }
__device__ __forceinline__ float4 mask4f(float4 x, uint32_t m) {
  return make_float4(__uint_as_float(__float_as_uint(x.x) & m), __uint_as_float(__float_as_uint(x.y) & m),
                     __uint_as_float(__float_as_uint(x.z) & m), __uint_as_float(__float_as_uint(x.w) & m));
}
__device__ __forceinline__ uint2 mask2(uint2 x, uint32_t m) { return make_uint2(x.x & m, x.y & m); }
__device__ __forceinline__ uint32_t okmask(bool ok) { return ok ? 0xffffffffu : 0u; }

__device__ __forceinline__ void unpack8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

// Fill ETA[0..C), LAM[0..DK), KS = K~ [C][DK], QS = Q~ [C][DK] for the chunk
// starting at token t0 with c >= 1 valid tokens (rows >= c are zero).
//   none / scalar decay: ks, qs are K and Q; lambda = 1 or gamma_h;
//   vector decay: ks, qs are the prepared K~ = K e^-L and Q~ = Q e^L and lam
//   holds the chunk's e^{L_last} (see ttt_decay_prep.hip).
// Loads are branch-free (addresses clamped to a valid token, values selected
// to zero) so that each batch is issued back to back.  Ends with a barrier.
template <int DK, int DECAY, bool FULL, int NT>
__device__ __forceinline__ void stage_chunk_impl(uint16_t* KS, uint16_t* QS, float* ETA, float* LAM,
                                                 const bf16_t* ks, const bf16_t* qs, const float* lam,
                                                 const float* beta, float b, float gamma_h, int t0, int c, int C) {
  const int tid = threadIdx.x;
  for (int t = tid; t < C; t += NT) ETA[t] = (t < c) ? lr_gate(beta[t0 + min(t, c - 1)], b) : 0.0f;
  for (int d = tid; d < DK; d += NT) LAM[d] = (DECAY == 2) ? lam[d] : (DECAY == 1) ? gamma_h : 1.0f;
  constexpr int G = DK / 8;
  const int total = C * G;
  constexpr int U = 2048 / NT;  // 8 rows-groups per thread at 256 threads
  for (int base = 0; base < total; base += NT * U) {
    uint4 kk[U], qq[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * NT + tid;
      const int t = idx / G, g = idx % G;
      const bool ok = idx < total && (FULL || t < c);
      const int64_t off = static_cast<int64_t>(t0 + (ok ? t : 0)) * DK + 8 * (ok ? g : 0);
      kk[u] = *reinterpret_cast<const uint4*>(ks + off);
      qq[u] = *reinterpret_cast<const uint4*>(qs + off);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * NT + tid;
      const int t = idx / G, g = idx % G;
      const uint32_t m = okmask(idx < total && (FULL || t < c));
      if (idx < total) {
        *reinterpret_cast<uint4*>(&KS[swz<DK>(t, 8 * g)]) = mask4(kk[u], m);
        *reinterpret_cast<uint4*>(&QS[swz<DK>(t, 8 * g)]) = mask4(qq[u], m);
      }
    }
  }
  __syncthreads();
}

template <int DK, int DECAY, int NT = kMfmaThreads>
__device__ __forceinline__ void stage_chunk(uint16_t* KS, uint16_t* QS, float* ETA, float* LAM, const bf16_t* ks,
                                            const bf16_t* qs, const float* lam, const float* beta, float b,
                                            float gamma_h, int t0, int c, int C) {
  if (c == C)  // every chunk but a short last one: no per-token validity test
    stage_chunk_impl<DK, DECAY, true, NT>(KS, QS, ETA, LAM, ks, qs, lam, beta, b, gamma_h, t0, c, C);
  else
    stage_chunk_impl<DK, DECAY, false, NT>(KS, QS, ETA, LAM, ks, qs, lam, beta, b, gamma_h, t0, c, C);
}

// B operand for a contraction over tokens: lane (col, hi) takes src[16 kb + 8 hi + jj][col]
// (jj < 8) from a [rows][NCOL] swizzled bf16 LDS matrix.  The eight row offsets
// within a k-step do not depend on kb (16 kb + 8 hi is a multiple of 8, so the
// swizzle key of row 16 kb + 8 hi + jj is that of row jj): the reader keeps one
// LDS pointer per jj, reads k-steps kb0 + kk (kk < 4) at constant offsets and
// then advances all eight by four k-steps.
template <int NCOL>
struct ColumnReader {
  const lds_t<const uint16_t>* p[8];
  __device__ __forceinline__ ColumnReader(const uint16_t* lds, int col, int hi) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) p[jj] = lds_base(lds + 8 * hi * NCOL + swz<NCOL>(jj, col));
  }
  __device__ __forceinline__ bf16x8_t operator()(int kk) const {
    bf16x8_t r;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) r[jj] = bits_to_bf(p[jj][kk * 16 * NCOL]);
    return r;
  }
  __device__ __forceinline__ void advance() {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) p[jj] += 4 * 16 * NCOL;
  }
};

// A operand along a row: lane (row, hi) takes src[row][16 kb + 8 hi .. +7] from a
// [rows][NCOL] swizzled bf16 LDS matrix (NCOL >= 64).  For kb = kb0 + kk with kb0
// a multiple of 4 the swizzled granule is 2 kb0 + ((2 kk + hi) ^ (row & 7)), so
// four per-lane pointers (one per kk) advanced by 64 elements per four k-steps
// cover every kb.
template <int NCOL>
struct RowReader {
  static_assert(NCOL >= 64, "the swizzle key must span 8 granules");
  const lds_t<const bf16x8_t>* p[4];
  __device__ __forceinline__ RowReader(const uint16_t* lds, int row, int hi) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      p[kk] = lds_base(reinterpret_cast<const bf16x8_t*>(lds + swz<NCOL>(row, 16 * kk + 8 * hi)));
  }
  __device__ __forceinline__ bf16x8_t operator()(int kk) const { return *p[kk]; }
  __device__ __forceinline__ void advance() {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) p[kk] += 8;  // 64 bf16 = 8 vectors of 8
  }
};

__device__ __forceinline__ void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
  const uint32_t lo = static_cast<uint32_t>(bf_bits(to_bf(a))) | (static_cast<uint32_t>(bf_bits(to_bf(b))) << 16);
  const uint32_t hi = static_cast<uint32_t>(bf_bits(to_bf(c))) | (static_cast<uint32_t>(bf_bits(to_bf(d))) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

// The 16 values of a 32x32 MFMA output lane -- row `t` of a token-major
// [*, ld] bf16 matrix, columns col0 + row_of(r, hi) -- stored as four 8-byte
// pieces (rows t >= c are skipped).
__device__ __forceinline__ void store_row16(bf16_t* dst, int64_t ld, int t0, int t, int c, int col0, int hi,
                                            const float (&v)[16]) {
  if (t >= c) return;
  bf16_t* p = dst + static_cast<int64_t>(t0 + t) * ld + col0 + 4 * hi;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) store_bf16x4(p + 8 * r4, v[4 * r4], v[4 * r4 + 1], v[4 * r4 + 2], v[4 * r4 + 3]);
}

// Store the 16 values a 32x32 MFMA output lane holds -- rows n = row_of(r, hi) of
// column `col` -- transposed into a [rows][NCOL] swizzled bf16 LDS matrix, i.e. to
// element (n, col).  The swizzle key n & 7 = 4 hi + r % 4 takes four values, so
// four per-lane base pointers and constant offsets (8 rows per r / 4) cover all 16.
template <int NCOL>
__device__ __forceinline__ void store_tile_t(uint16_t* lds, int col, int hi, const float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lds_t<uint16_t>* b = lds_base(lds + swz<NCOL>(4 * hi + q, col));
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) b[r4 * 8 * NCOL] = bf_bits(to_bf(v[4 * r4 + q]));
  }
}

// Stage the raw keys K [C][DK] of a chunk (rows >= c zero) into LDS; no barrier.
template <int DK, int NT = kMfmaThreads>
__device__ __forceinline__ void stage_raw_k(uint16_t* KR, const bf16_t* k, int t0, int c, int C) {
  const int tid = threadIdx.x;
  constexpr int G = DK / 8;
  const int total = C * G;
  constexpr int U = 2048 / NT;
  for (int base = 0; base < total; base += NT * U) {
    uint4 kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * NT + tid;
      const int t = idx / G, g = idx % G;
      const bool ok = idx < total && t < c;
      kk[u] = *reinterpret_cast<const uint4*>(k + static_cast<int64_t>(t0 + (ok ? t : 0)) * DK + 8 * (ok ? g : 0));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * NT + tid;
      const uint32_t m = okmask(idx < total && idx / G < c);
      if (idx < total) *reinterpret_cast<uint4*>(&KR[swz<DK>(idx / G, 8 * (idx % G))]) = mask4(kk[u], m);
    }
  }
}

// Own-tile row fragments of a token-major bf16 matrix (row stride `ld`): the
// 16-byte B/A-operand pieces src[t0 + t][16 kb + 8 hi ..] for kb < NK, zero for
// rows t >= c (address clamped so every load is issued unconditionally).
template <int NK>
__device__ __forceinline__ void load_row_frags(bf16x8_t (&f)[NK], const bf16_t* src, int64_t ld, int t0, int t, int c,
                                               int col0, int hi) {
  const bool ok = t < c;
  const bf16_t* p = src + static_cast<int64_t>(t0 + (ok ? t : 0)) * ld + col0 + 8 * hi;
  const uint32_t m = okmask(ok);
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) f[kb] = __builtin_bit_cast(bf16x8_t, mask4(*reinterpret_cast<const uint4*>(p + 16 * kb), m));
}

// Four 8-byte pieces src[t0 + t][col0 + 8 r4 + 4 hi .. +3] (the 16 values a
// 32x32 MFMA output lane holds for one row), zero for t >= c.
__device__ __forceinline__ void load_row16(uint2 (&x)[4], const bf16_t* src, int64_t ld, int t0, int t, int c,
                                           int col0, int hi) {
  const bool ok = t < c;
  const bf16_t* p = src + static_cast<int64_t>(t0 + (ok ? t : 0)) * ld + col0 + 4 * hi;
  const uint32_t m = okmask(ok);
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) x[r4] = mask2(*reinterpret_cast<const uint2*>(p + 8 * r4), m);
}
__device__ __forceinline__ void unpack16(const uint2 (&x)[4], float (&f)[16]) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    f[4 * r4] = __uint_as_float(x[r4].x << 16);
    f[4 * r4 + 1] = __uint_as_float(x[r4].x & 0xffff0000u);
    f[4 * r4 + 2] = __uint_as_float(x[r4].y << 16);
    f[4 * r4 + 3] = __uint_as_float(x[r4].y & 0xffff0000u);
  }
}

// L2 prefetch: load one dword from the 128-byte line number `threadIdx.x + i * NT`
// (i < NL) of part `part` (of `nparts`) of [p, p + bytes) into w[i].  Out-of-range
// lines reload line 0; the values only feed a never-taken store, so the loads stay
// in flight until the caller consumes w late.  bytes < 2^31.
template <int NL, int NT = kMfmaThreads>
__device__ __forceinline__ void l2_touch(uint32_t (&w)[NL], const void* p, int bytes, int part, int nparts) {
  const char* base = static_cast<const char*>(p);
  const int lines = (bytes + 127) >> 7;
  const int per = (lines + nparts - 1) / nparts;
  const int l0 = per * part;
  const int l1 = min(lines, l0 + per);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int l = l0 + static_cast<int>(threadIdx.x) + i * NT;
    w[i] = *reinterpret_cast<const uint32_t*>(base + (static_cast<int64_t>(l < l1 ? l : 0) << 7));
  }
}

// Workgroup id remap: hardware hands block L to XCD L % 8; this places the
// d_v column blocks of one chain (consecutive after the remap) on one XCD.
__device__ __forceinline__ int xcd_remap(int L, int nblk) {
  if ((nblk & 7) == 0) return (L & 7) * (nblk >> 3) + (L >> 3);
  return L;
}

}  // namespace ttt
