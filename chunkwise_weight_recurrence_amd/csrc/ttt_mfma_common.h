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

#include <utility>

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
// Every global load (beta, lambda and all of K~, Q~) is issued before the first
// LDS write, so the staging costs one memory round trip; loads are branch-free
// (addresses clamped to a valid token, values selected to zero).  Ends with a
// barrier.
template <int DK, int DECAY, bool FULL, int NT>
__device__ __forceinline__ void stage_chunk_impl(uint16_t* KS, uint16_t* QS, float* ETA, float* LAM,
                                                 const bf16_t* ks, const bf16_t* qs, const float* lam,
                                                 const float* beta, float b, float gamma_h, int t0, int c, int C) {
  static_assert(NT >= kCMax && NT >= DK, "one eta and one lambda per thread");
  constexpr int G = DK / 8;
  constexpr int U = kCMax * G / NT;  // 16-byte pieces per thread and matrix at C = kCMax
  const int tid = threadIdx.x;
  const int total = C * G;
  const float bt = (tid < C) ? beta[t0 + min(tid, c - 1)] : 0.0f;
  const float lm = (DECAY == 2 && tid < DK) ? lam[tid] : 1.0f;
  uint4 kk[U], qq[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u * NT < total) {  // uniform: total is a multiple of NT or below it
      const int idx = u * NT + tid;
      const int t = idx / G, g = idx % G;
      const bool ok = idx < total && (FULL || t < c);
      const int64_t off = static_cast<int64_t>(t0 + (ok ? t : 0)) * DK + 8 * (ok ? g : 0);
      kk[u] = *reinterpret_cast<const uint4*>(ks + off);
      qq[u] = *reinterpret_cast<const uint4*>(qs + off);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (tid < C) ETA[tid] = (tid < c) ? lr_gate(bt, b) : 0.0f;
  if (tid < DK) LAM[tid] = (DECAY == 2) ? lm : (DECAY == 1) ? gamma_h : 1.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u * NT < total) {
      const int idx = u * NT + tid;
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

// B operand for a contraction over tokens: lane (col, hi) takes
// src[16 kb + 8 hi + jj][col] (jj < 8) from a [rows][NCOL] swizzled bf16 LDS
// matrix, with two transpose reads per k-step.  ds_read_b64_tr_b16 (gfx950)
// works on groups of 16 lanes: each
// lane names an 8-byte piece (4 consecutive bf16), and lane 4a + b of the group
// receives element b of the pieces named by lanes a, a + 4, a + 8, a + 12.  So
// lane L = (l32, hi) names row 8 hi + 4 h + (l32 % 16) / 4 (h = 0, 1: rows 0..3
// and 4..7 of its eight) and columns 16 (l32 / 16) + 4 (l32 % 4) .. +3 of the
// 32-column block, and gets back column l32 at four consecutive rows.  A piece
// of four columns starting at a multiple of 4 stays inside one swizzle granule;
// the swizzle key of row 16 kb + r does not depend on kb (it depends on the
// row modulo 16), so the two row pointers advance by whole k-steps.
template <int NCOL>
struct ColumnReaderTR {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const lds_t<const uint16_t>* p[2];
  __device__ __forceinline__ ColumnReaderTR(const uint16_t* lds, int col_block, int l32, int hi) {
    const int col = col_block + 16 * (l32 >> 4) + 4 * (l32 & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) p[h] = lds_base(lds + swz<NCOL>(8 * hi + 4 * h + ((l32 & 15) >> 2), col));
  }
  __device__ __forceinline__ bf16x8_t operator()(int kk) const {
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p[0] + kk * 16 * NCOL));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p[1] + kk * 16 * NCOL));
    bf16x8_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = bits_to_bf(static_cast<uint16_t>(a[j]));
      r[4 + j] = bits_to_bf(static_cast<uint16_t>(b[j]));
    }
    return r;
  }
  __device__ __forceinline__ void advance() {
#pragma unroll
    for (int h = 0; h < 2; ++h) p[h] += 4 * 16 * NCOL;
  }
};

// A operand along a row: lane (row, hi) takes src[row][16 kb + 8 hi .. +7] from a
// [rows][NCOL] swizzled bf16 LDS matrix (NCOL >= 64).  For kb = 4 m + kk the
// logical granule is 8 m + (2 kk + hi), stored at slot
// 8 (m ^ (key / 8)) + ((2 kk + hi) ^ (key % 8)): four per-lane pointers (one per
// kk) for m = 0, moved to the slot of block m ^ (key / 8) as m advances.
template <int NCOL>
struct RowReader {
  static_assert(NCOL >= 64, "the swizzle key must span 8 granules");
  const lds_t<const bf16x8_t>* p[4];
  const lds_t<const bf16x8_t>* b[4];  // the pointers of block 0
  int k3, m = 0;                      // key / 8 (0 or 1) and the block of four k-steps
  __device__ __forceinline__ RowReader(const uint16_t* lds, int row, int hi) {
    const int key = swz_key<NCOL>(row);
    k3 = key >> 3;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      b[kk] = lds_base(reinterpret_cast<const bf16x8_t*>(lds + row * NCOL + (((2 * kk + hi) ^ (key & 7)) << 3)));
      p[kk] = b[kk] + 8 * k3;
    }
  }
  __device__ __forceinline__ bf16x8_t operator()(int kk) const { return *p[kk]; }
  // k-step kb of the row, independent of advance()
  __device__ __forceinline__ bf16x8_t at(int kb) const { return *(b[kb & 3] + 8 * ((kb >> 2) ^ k3)); }
  __device__ __forceinline__ void advance() {
    ++m;
    const int off = 8 * (m ^ k3);  // 64 bf16 = 8 vectors per block
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) p[kk] = b[kk] + off;
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

// Same row store with half the memory instructions: the two lanes of a row
// (hi = 0, 1) trade their column groups with v_permlane32_swap so that lane hi
// holds the 16 consecutive columns 16 hi .. 16 hi + 15, then store 32 bytes each
// as two 16-byte pieces.  Before the swap lane (t, hi) holds columns
// 8 g + 4 hi .. +3 in group g = 0..3 (two bf16 pairs per group); swapping group g
// with group g + 2 across the halves leaves lane 0 with groups (0,0),(1,0),(0,1),
// (1,1) = columns 0..15 and lane 1 with columns 16..31.  Must be reached by all
// 64 lanes (the swap reads the other half); rows t >= c are not written.
__device__ __forceinline__ void store_row16_x2(bf16_t* dst, int64_t ld, int t0, int t, int c, int col0, int hi,
                                               const float (&v)[16]) {
  uint32_t d[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    d[j] = static_cast<uint32_t>(bf_bits(to_bf(v[2 * j]))) | (static_cast<uint32_t>(bf_bits(to_bf(v[2 * j + 1]))) << 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(d[j], d[j + 4], false, false);
    d[j] = r[0];
    d[j + 4] = r[1];
  }
  if (t < c) {
    bf16_t* p = dst + static_cast<int64_t>(t0 + t) * ld + col0 + 16 * hi;
    *reinterpret_cast<uint4*>(p) = make_uint4(d[0], d[1], d[4], d[5]);
    *reinterpret_cast<uint4*>(p + 8) = make_uint4(d[2], d[3], d[6], d[7]);
  }
}

// The inverse for loads, also with half the memory instructions: lane (t, hi)
// loads the 32 contiguous bytes of columns 16 hi .. 16 hi + 15 of row t (rows
// t >= c read row 0 of the chunk instead); row32_frags then trades column groups
// with the partner lane into the layout load_row16 gives (group g = columns
// 8 g + 4 hi .. +3), zeroing rows t >= c.  The two steps are separate so that the
// exchange, which needs the data, sits where the values are used and not where
// the loads are issued.  row32_frags must be reached by all 64 lanes.
__device__ __forceinline__ void load_row32(uint4 (&raw)[2], const bf16_t* src, int64_t ld, int t0, int t, int c,
                                           int col0, int hi) {
  const bf16_t* p = src + static_cast<int64_t>(t0 + (t < c ? t : 0)) * ld + col0 + 16 * hi;
  raw[0] = *reinterpret_cast<const uint4*>(p);
  raw[1] = *reinterpret_cast<const uint4*>(p + 8);
}
__device__ __forceinline__ void row32_frags(const uint4 (&raw)[2], uint2 (&x)[4], bool ok) {
  uint32_t d[8] = {raw[0].x, raw[0].y, raw[1].x, raw[1].y, raw[0].z, raw[0].w, raw[1].z, raw[1].w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(d[j], d[j + 4], false, false);
    d[j] = r[0];
    d[j + 4] = r[1];
  }
  const uint32_t m = okmask(ok);
#pragma unroll
  for (int g = 0; g < 4; ++g) x[g] = make_uint2(d[2 * g] & m, d[2 * g + 1] & m);
}

// Store the 16 values a 32x32 MFMA output lane holds -- rows n = row_of(r, hi) of
// column `col` -- transposed into a [rows][NCOL] swizzled bf16 LDS matrix, i.e. to
// element (n, col).  The swizzle key depends on n % 16 = 8 ((r / 4) % 2) + 4 hi +
// r % 4 only, so eight per-lane base pointers and constant offsets (16 rows per
// two r / 4) cover all 16.
template <int NCOL>
__device__ __forceinline__ void store_tile_t(uint16_t* lds, int col, int hi, const float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      lds_t<uint16_t>* b = lds_base(lds + swz<NCOL>(8 * par + 4 * hi + q, col));
#pragma unroll
      for (int r4 = par; r4 < 4; r4 += 2) b[(r4 >> 1) * 16 * NCOL] = bf_bits(to_bf(v[4 * r4 + q]));
    }
}

// Store the 16 values a 32x32 MFMA output lane holds -- columns n = row_of(r, hi)
// of row `row` -- into row `row` of a [rows][NCOL] swizzled bf16 LDS matrix, as
// four 8-byte pieces (columns 8 q + 4 hi .. +3).  Read back as an MFMA operand
// along the rows (k = row) with ColumnReaderTR.
template <int NCOL>
__device__ __forceinline__ void store_tile_rows(uint16_t* lds, int row, int hi, const float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = static_cast<uint32_t>(bf_bits(to_bf(v[4 * q]))) |
                        (static_cast<uint32_t>(bf_bits(to_bf(v[4 * q + 1]))) << 16);
    const uint32_t up = static_cast<uint32_t>(bf_bits(to_bf(v[4 * q + 2]))) |
                        (static_cast<uint32_t>(bf_bits(to_bf(v[4 * q + 3]))) << 16);
    *reinterpret_cast<uint2*>(&lds[swz<NCOL>(row, 8 * q + 4 * hi)]) = make_uint2(lo, up);
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

// Barrier that orders LDS traffic only: it waits for this wave's LDS reads and
// writes but leaves its global loads and stores in flight (__syncthreads would
// drain those too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// f(0), ..., f(N - 1) with compile-time indices, expanded without a loop (a
// register array indexed this way stays in registers even where an unrolled
// loop over it would not).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
      std::make_integer_sequence<int, N>{});
}

// K~ rows of a chunk staged through registers, a chunk ahead: rows [t0, t0 + C)
// of a token-major bf16 [*, DK] matrix, 16 bytes per thread and step (thread =
// (row, 16-byte granule), coalesced; a native vector type, so the copies are
// plain loads and stores).  Every step loads, also past the chunk's
// C rows, so the count of loads is fixed; rows at or past c repeat row c - 1:
// finite values, and every consumer zeroes or masks those tokens (their eta
// is 0).
template <int DK, int NT>
struct RowStageSize {
  static constexpr int U = kCMax * (DK / 8) / NT;  // 16-byte pieces per thread
};
template <int DK, int NT, int U>
__device__ __forceinline__ void rows_load(bf16x8_t (&x)[U], const bf16_t* src, int t0, int c) {
  static_assert(U == RowStageSize<DK, NT>::U, "one piece per thread and step");
  constexpr int G = DK / 8;
  static_for<U>([&](auto u) {
    const int idx = u * NT + static_cast<int>(threadIdx.x);
    const int row = idx / G, g = idx % G;
    x[u] = *reinterpret_cast<const bf16x8_t*>(src + static_cast<int64_t>(t0 + min(row, c - 1)) * DK + 8 * g);
  });
}
// ... into a [kCMax][DK] buffer with the 16-byte granule XOR swizzle (all kCMax
// rows; those past the chunk's C are never read)
template <int DK, int NT, int U>
__device__ __forceinline__ void rows_store(uint16_t* dst, const bf16x8_t (&x)[U]) {
  static_assert(U == RowStageSize<DK, NT>::U, "one piece per thread and step");
  constexpr int G = DK / 8;
  static_for<U>([&](auto u) {
    const int idx = u * NT + static_cast<int>(threadIdx.x);
    *reinterpret_cast<bf16x8_t*>(&dst[swz<DK>(idx / G, 8 * (idx % G))]) = x[u];
  });
}

// Unmasked own-row loads for prefetching a chunk ahead: rows at or past c read
// row 0 of the chunk instead (no select on the loaded value, which would make
// the load complete where it is issued).
template <int NK>
__device__ __forceinline__ void load_row_frags_nomask(bf16x8_t (&f)[NK], const bf16_t* src, int64_t ld, int t0, int t,
                                                      int c, int col0, int hi) {
  const bf16_t* p = src + static_cast<int64_t>(t0 + (t < c ? t : 0)) * ld + col0 + 8 * hi;
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) f[kb] = *reinterpret_cast<const bf16x8_t*>(p + 16 * kb);
}
__device__ __forceinline__ void load_row16_nomask(uint2 (&x)[4], const bf16_t* src, int64_t ld, int t0, int t, int c,
                                                  int col0, int hi) {
  const bf16_t* p = src + static_cast<int64_t>(t0 + (t < c ? t : 0)) * ld + col0 + 4 * hi;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) x[r4] = *reinterpret_cast<const uint2*>(p + 8 * r4);
}

// Workgroup id remap: hardware hands block L to XCD L % 8; this places the
// d_v column blocks of one chain (consecutive after the remap) on one XCD.
__device__ __forceinline__ int xcd_remap(int L, int nblk) {
  if ((nblk & 7) == 0) return (L & 7) * (nblk >> 3) + (L >> 3);
  return L;
}

}  // namespace ttt
