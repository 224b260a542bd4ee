// Tile GEMM machinery of the one-workgroup-per-chain kernels (the two-layer fast
// net and the Linear -> Norm fast net): a workgroup of 8 waves computes
// out = epi(op(A1) op(B1) [+ op(A2) op(B2)]) in 64 x 64 output tiles on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32), operands staged through double-buffered
// LDS in 64-deep k-slices, plus the per-row and staging helpers those kernels
// share.  Everything here has internal linkage: each kernel file has its copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_device.h"

namespace ttt {
namespace {

constexpr int kThreads = 512;     // 8 waves: two per output quadrant, one per half of each k-slice
constexpr int kTile = 64;          // output tile (rows and columns)
constexpr int kKS = 64;            // k-slice staged per LDS round
constexpr int kPitch = kTile + 4;  // LDS row pitch (floats): 16-byte aligned rows
constexpr int kPerThr = kTile * kKS / kThreads;  // staged elements per operand and thread
constexpr int kBuf = 2 * kKS * kPitch;           // floats of one staged slice: A, then B
constexpr size_t kLdsBytes = sizeof(float) * (2 * kBuf + 4 * 16 * 64);
// LDS of a kernel whose GEMMs stage one slice at a time (NBUF = 1): 51 KB, so
// two or three such workgroups share a CU.
constexpr size_t kLdsBytes1 = sizeof(float) * (kBuf + 4 * 16 * 64);

// One product term alpha * op(A) op(B) of a GEMM over fp32 memory, op(A)
// [M x K], op(B) [K x N].  Element (m, k) of op(A) is a[m * lda + k], or
// a[k * lda + m] when A is taken transposed (AT); likewise (k, n) of op(B) is
// b[k * ldb + n], or b[n * ldb + k] (BT).
struct Term {
  const float* a;
  int lda;
  const float* b;
  int ldb;
  int K;
  float alpha;
};

// The thread index as a value the compiler cannot see through.  The staging
// offsets derive from it; taking it anew at every slice keeps them from being
// hoisted out of the chunk loop for each of the chunk's GEMMs at once (which
// would hold hundreds of registers for the whole kernel).
__device__ __forceinline__ int opaque_tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

template <int TR> struct SliceMap;
template <> struct SliceMap<0> {  // contiguous along k: (row, k) = (tid / 64 + 8 i, tid % 64)
  static __device__ __forceinline__ int row(int tid, int i) { return tid / kKS + (kThreads / kKS) * i; }
  static __device__ __forceinline__ int kk(int tid, int) { return tid % kKS; }
};
template <> struct SliceMap<1> {  // contiguous along the row index: (row, k) = (tid % 64, tid / 64 + 8 i)
  static __device__ __forceinline__ int row(int tid, int) { return tid % kTile; }
  static __device__ __forceinline__ int kk(int tid, int i) { return tid / kTile + (kThreads / kTile) * i; }
};

// The registers of one staged k-slice.  A row-major A and a transposed B are
// contiguous along k (map 0); a transposed A and a row-major B along the row
// or column index (map 1).
struct Slice {
  float a[kPerThr], b[kPerThr];
};

// Buffer resource of an operand: its base, a 2 GiB range and the gfx9
// default format word.  A raw buffer load whose byte offset lies at or past
// the range returns 0 without touching memory, which is how elements outside
// the operand stage as zero.
// The whole workgroup stages one operand together, so its base is the same in
// every lane; reading it from the first lane keeps the resource in scalar
// registers where the compiler cannot prove that by itself (it would otherwise
// loop over the distinct values around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const float* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  float* base = reinterpret_cast<float*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
}
constexpr unsigned kOutside = 0x80000000u;  // a byte offset past every operand's range

__device__ __forceinline__ float buffer_ld(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(byte_off), 0, 0));
}

// The loads are unconditional (an element outside the operand takes an offset
// past the buffer range and reads as 0): a load under a branch makes the
// compiler wait for it on the spot, which would serialise the prefetch.  The
// offsets are 32-bit byte offsets from the operand's base: an operand spans at
// most max(M, K) rows of a leading dimension of at most 1024 floats.
template <int AT, int BT>
__device__ __forceinline__ void load_slice(Slice& r, const Term& t, int M, int N, int m0, int n0, int k0) {
  using MA = SliceMap<AT>;
  using MB = SliceMap<BT ? 0 : 1>;
  const int tid = opaque_tid();
  const __amdgpu_buffer_rsrc_t ra = operand_rsrc(t.a), rb = operand_rsrc(t.b);
#pragma unroll
  for (int i = 0; i < kPerThr; ++i) {
    const int gm = m0 + MA::row(tid, i), gk = k0 + MA::kk(tid, i);
    const bool in = gm < M && gk < t.K;
    const unsigned off = AT ? gk * t.lda + gm : gm * t.lda + gk;
    r.a[i] = buffer_ld(ra, in ? 4u * off : kOutside);
  }
#pragma unroll
  for (int i = 0; i < kPerThr; ++i) {
    const int gn = n0 + MB::row(tid, i), gk = k0 + MB::kk(tid, i);
    const bool in = gk < t.K && gn < N;
    const unsigned off = BT ? gn * t.ldb + gk : gk * t.ldb + gn;
    r.b[i] = buffer_ld(rb, in ? 4u * off : kOutside);
  }
}

template <int AT, int BT>
__device__ __forceinline__ void store_slice(const Slice& r, float alpha, float* buf) {
  using MA = SliceMap<AT>;
  using MB = SliceMap<BT ? 0 : 1>;
  const int tid = opaque_tid();
  float* As = buf;
  float* Bs = buf + kKS * kPitch;
#pragma unroll
  for (int i = 0; i < kPerThr; ++i) As[MA::kk(tid, i) * kPitch + MA::row(tid, i)] = alpha * r.a[i];
#pragma unroll
  for (int i = 0; i < kPerThr; ++i) Bs[MB::kk(tid, i) * kPitch + MB::row(tid, i)] = r.b[i];
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Wave w of the workgroup owns the 32 x 32 quadrant q = w % 4, at (32 (q % 2),
// 32 (q / 2)), of a 64 x 64 output tile, for the half g = w / 4 of every
// k-slice (k = 32 g ... 32 g + 31), and accumulates it with
// v_mfma_f32_32x32x2_f32 (fp32 operands, fp32 accumulation): per step lane l
// feeds op(A)[l % 32][k + l / 32] and op(B)[k + l / 32][l % 32], and after it
// holds element r of the quadrant at row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.  The two halves are added at the end of the tile.
__device__ __forceinline__ int quad_row(int r) { return 8 * (r / 4) + 4 * (static_cast<int>(threadIdx.x) % 64 / 32) + r % 4; }

// This wave's products of one staged slice: acc += its k-half of A_s B_s.
__device__ __forceinline__ void slice_products(floatx16& acc, const float* buf) {
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64, q = w % 4, g = w / 4;
  const int a_off = (kKS / 2 * g + lane / 32) * kPitch + 32 * (q % 2) + lane % 32;
  const int b_off = kKS * kPitch + (kKS / 2 * g + lane / 32) * kPitch + 32 * (q / 2) + lane % 32;
  float av[kKS / 4], bv[kKS / 4];  // all LDS reads of the half-slice first, then the products
#pragma unroll
  for (int j = 0; j < kKS / 4; ++j) {
    av[j] = buf[2 * j * kPitch + a_off];
    bv[j] = buf[2 * j * kPitch + b_off];
  }
#pragma unroll
  for (int j = 0; j < kKS / 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j], acc, 0, 0, 0);
}

// out(m, n) = epi(m, n, op(A1) op(B1) [+ op(A2) op(B2)]) for m < M, n < N, in
// 64 x 64 tiles.  The second term is used when K2 = t2.K > 0.
// Causal shortcuts: LOWER computes only the tiles that reach the diagonal or
// below (n0 < m0 + 64; a causal score matrix, whose strictly upper tiles are
// never read), and TRI2 ends the second term's k range at the row tile's last
// row (its A is such a score matrix, zero right of the diagonal).
//
// The GEMM is one flat sequence of steps (tile, term, k-slice).  Slices are
// double-buffered in LDS: the next step's slice -- in the same tile or the
// next -- is fetched into registers before this step's products and written to
// the other buffer after them, so one barrier per step suffices and a tile's
// first slice is not waited for.  At a tile's end the two k-halves are added
// through a separate LDS area: group 0 finishes elements 0..7 of its quadrant,
// group 1 elements 8..15.
// Up to three operands of the epilogue, each read at the output position (m, n)
// as p[j][m * ld + n]; a null p[j] reads as 0.
struct Aux {
  const float* p[3];
  int ld;
};

//
// NBUF = 1 stages one slice at a time: the next slice is written after every
// wave is past the current one's products (a second barrier per step), in half
// the LDS, for kernels that run several workgroups per CU to cover the waits.
template <int AT1, int BT1, int AT2, int BT2, bool LOWER = false, bool TRI2 = false, int NBUF = 2, class Epi>
__device__ __forceinline__ void gemm(int M, int N, const Term& t1, const Term& t2, const Aux& aux, float* lds,
                                     Epi epi) {
  static_assert(NBUF == 1 || NBUF == 2, "one or two slice buffers");
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64, q = w % 4, g = w / 4;
  float* red = lds + NBUF * kBuf + q * 16 * 64;  // [quadrant][element][lane]
  const int ntm = (M + kTile - 1) / kTile, ntn = (N + kTile - 1) / kTile;
  auto k2_of = [&](int mt) { return TRI2 ? min(t2.K, (mt + 1) * kTile) : t2.K; };
  auto ntn_of = [&](int mt) { return LOWER ? min(ntn, mt + 1) : ntn; };
  // step state: row tile, column tile, term (0 / 1), slice
  int mt = 0, nt = 0, tm = 0, sl = 0;
  auto fetch = [&](Slice& r, int mt_, int nt_, int tm_, int sl_) {
    if (tm_ == 0) {
      load_slice<AT1, BT1>(r, t1, M, N, mt_ * kTile, nt_ * kTile, sl_ * kKS);
    } else {
      Term u = t2;
      u.K = k2_of(mt_);
      load_slice<AT2, BT2>(r, u, M, N, mt_ * kTile, nt_ * kTile, sl_ * kKS);
    }
  };
  auto put = [&](const Slice& r, int tm_, float* buf) {
    if (tm_ == 0) store_slice<AT1, BT1>(r, t1.alpha, buf);
    else store_slice<AT2, BT2>(r, t2.alpha, buf);
  };
  Slice r;
  fetch(r, 0, 0, 0, 0);
  put(r, 0, lds);
  __syncthreads();
  floatx16 acc = {};
  int b = 0;
  for (;;) {
    // the step after (mt, nt, tm, sl)
    int mt2 = mt, nt2 = nt, tm2 = tm, sl2 = sl + 1;
    const int nsl = ((tm == 0 ? t1.K : k2_of(mt)) + kKS - 1) / kKS;
    if (sl2 >= nsl) {
      sl2 = 0;
      if (tm == 0 && k2_of(mt) > 0) {
        tm2 = 1;
      } else {
        tm2 = 0;
        if (++nt2 >= ntn_of(mt)) {
          nt2 = 0;
          ++mt2;
        }
      }
    }
    const bool more = mt2 < ntm;
    const bool tile_end = !more || mt2 != mt || nt2 != nt;
    if (more) fetch(r, mt2, nt2, tm2, sl2);
    // The epilogue's own operands (aux at the output position) of a tile that
    // this step completes are loaded for all eight elements now, so their
    // latency overlaps the step's products and the k-half exchange.
    const int n = nt * kTile + 32 * (q / 2) + lane % 32;
    const int mq = mt * kTile + 32 * (q % 2);
    const int eb = 8 * g;  // this group finishes elements eb .. eb + 7
    float ax[3][8];
    if (tile_end) {
      const int nc = min(n, N - 1);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (aux.p[j]) {
          const __amdgpu_buffer_rsrc_t rx = operand_rsrc(aux.p[j]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            ax[j][e] = buffer_ld(rx, 4u * static_cast<unsigned>(min(mq + quad_row(e + eb), M - 1) * aux.ld + nc));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) ax[j][e] = 0.0f;
        }
      }
    }
    slice_products(acc, lds + b * kBuf);
    if constexpr (NBUF == 1) {
      __syncthreads();  // every wave is past this slice's products
      if (more) put(r, tm2, lds);
    } else {
      if (more) put(r, tm2, lds + (b ^ 1) * kBuf);
    }
    __syncthreads();
    if (tile_end) {  // the tile (mt, nt) is complete
      if (g == 0) {
#pragma unroll
        for (int e = 8; e < 16; ++e) red[e * 64 + lane] = acc[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[e * 64 + lane] = acc[e];
      }
      __syncthreads();
      if (g == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = mq + quad_row(e);
          if (m < M && n < N) epi(m, n, acc[e] + red[e * 64 + lane], ax[0][e], ax[1][e], ax[2][e]);
        }
      } else {
#pragma unroll
        for (int e = 8; e < 16; ++e) {
          const int m = mq + quad_row(e);
          if (m < M && n < N) epi(m, n, acc[e] + red[e * 64 + lane], ax[0][e - 8], ax[1][e - 8], ax[2][e - 8]);
        }
      }
      acc = floatx16{};
      // red is next written at the following tile's end, after at least one more step barrier
    }
    if (!more) break;
    mt = mt2; nt = nt2; tm = tm2; sl = sl2;
    if constexpr (NBUF == 2) b ^= 1;
  }
  __syncthreads();  // the caller's next GEMM restages slice buffer 0 and red
}

constexpr Aux kNoAux{{nullptr, nullptr, nullptr}, 0};

template <int AT, int BT, bool LOWER = false, int NBUF = 2, class Epi>
__device__ __forceinline__ void gemm1(int M, int N, const Term& t, const Aux& aux, float* lds, Epi epi) {
  gemm<AT, BT, 0, 0, LOWER, false, NBUF>(M, N, t, Term{nullptr, 0, nullptr, 0, 0, 0.0f}, aux, lds, epi);
}

// Zero the strictly upper 64 x 64 tiles of a c x c causal score matrix (row
// pitch ld), which a LOWER GEMM leaves unwritten: the backward also reads these
// matrices transposed over their full width.
__device__ __forceinline__ void zero_upper_tiles(float* S, int c, int ld) {
  for (int i = threadIdx.x; i < c * c; i += kThreads) {
    const int m = i / c, n = i % c;
    if (n >= (m / kTile + 1) * kTile) S[m * ld + n] = 0.0f;
  }
}

// dst[i] = src[i] as fp32 for i < n: each thread issues U loads (clamped to the
// last element) before it stores, so their latencies overlap.  The per-chain
// kernels, whose chunk staging nothing else hides, take U = 32: a 256 x 64
// chunk in one round trip.
template <class E, int U = 8, typename T>
__device__ __forceinline__ void stage_rows(float* __restrict__ dst, const T* __restrict__ src, int n) {
  constexpr int kU = U;
  for (int i0 = threadIdx.x; i0 < n; i0 += kThreads * kU) {
    float x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) x[u] = E::ld(src, min(i0 + u * kThreads, n - 1));
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i0 + u * kThreads < n) dst[i0 + u * kThreads] = x[u];
  }
}

// acc + sum of a[i] b[i] over this thread's i = tid, tid + kThreads, ... < n,
// added in that order, with 16 pairs of loads in flight (a plain loop waits out
// a full memory latency for every pair).
__device__ __forceinline__ float strided_dot(const float* __restrict__ a, const float* __restrict__ b, int64_t n,
                                             float acc) {
  constexpr int kU = 16;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += static_cast<int64_t>(kThreads) * kU) {
    float x[kU], y[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t iu = i0 + static_cast<int64_t>(u) * kThreads;
      const int64_t i = iu < n ? iu : n - 1;
      x[u] = a[i];
      y[u] = b[i];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i0 + static_cast<int64_t>(u) * kThreads < n) acc = fmaf(x[u], y[u], acc);
  }
  return acc;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Per-row sum of f(j) over the d_v features by one wave: lane l takes features
// l, l + 64, ...
template <class F>
__device__ __forceinline__ float row_sum(int dv, int lane, F f) {
  float acc = 0.0f;
  for (int j = lane; j < dv; j += 64) acc += f(j);
  return wave_sum(acc);
}

}  // namespace
}  // namespace ttt
