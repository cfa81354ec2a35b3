// kda_prefill.hip -- chunked KDA prefill for gfx950.
//
// The method is the chunkwise form sketched in the "Kimi Linear" deep-read
// report (zako-mio knowledge base), section 3.1: inside a chunk, two gated
// secondary-chunk matrices (k k^T and q k^T, because the DPLR low-rank factors
// are both tied to k), a UT transform whose triangular inverse is obtained by
// forward substitution, and WY-form factors, so that the bulk of the work is
// half-precision matrix multiplication; across chunks a sequential state pass.
// The pages give no chunk equations; the ones below are derived from the
// recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T.
//
// Per (sequence, head), chunk of n <= C rows, S the state at chunk start,
// g_r = sum_{u<=r} log_alpha_u (chunk-local, per key channel):
//   A_rs = b_r sum_c k_r[c] k_s[c] e^{g_r[c]-g_s[c]}   (s < r)
//   P_rs =     sum_c q_r[c] k_s[c] e^{g_r[c]-g_s[c]}   (s <= r)
//   T    = (I + A)^{-1}                                 (unit lower triangular)
//   R_r  = b_r e^{g_r} * k_r,  Qh_r = e^{g_r} * q_r,  Kb_r = e^{g_last-g_r} * k_r
//   D    = T (b*V - R S)            the per-token delta-rule corrections
//   O    = Qh S + P D
//   S   <- Diag(e^{g_last}) S + Kb^T D
// Every equation of the state pass acts column by column on the value axis.
//
// Kernels:
//   chunk_offsets_kernel  chunk offsets per sequence + longest-first order
//   prep_kernel           persistent, (chunk, head) items: everything that
//                         does not depend on S (gate cumsum, A and P via MFMA,
//                         T by blocked forward substitution with the diagonal
//                         blocks from a nilpotent product, R, Qh, Kb^T,
//                         e^{g_last}), written to one workspace block per
//                         (chunk, head)
//   scan_kernel           grid (sequence, head, value tile): the serial chunk
//                         loop with S held in MFMA accumulators, chunk blocks
//                         streamed into LDS ahead of use (their first
//                         products' operands two chunks ahead, the rest one)
//   ready_kernel          segment counter of the overlapped schedule
// With few (sequence, head) pairs the scan runs on half of the CUs beside
// the prep of later chunks on the other half (launch_prefill below).
//
// Exponent safety.  Every gate factor is e^x of a sum x of log_alpha over a
// contiguous token range, formed directly as such a sum (never as the
// difference of two sums), so its rounding is relative to itself.  Inside a
// chunk, per key channel and 16-row block I: d_r sums the block's rows up to
// and including r, s_r the block's rows after r, D_I the whole block.  For
// s <= r (r in block I, s in block J <= I)
//   e^{g_r - g_s} = e^{d_r} e^{s_s} e^{D_{J+1} + ... + D_{I-1}}   (J < I)
//                 = e^{d_r} e^{s_s} e^{-D_I}                      (J = I)
// The row operands carry e^{d_r} <= 1 and the column operand e^{s_s} <= 1;
// an off-diagonal pair scales the column operand by a factor <= 1, so every
// factor is at most 1 and an underflow only stands for a negligible ratio.
// A diagonal pair scales it by e^{-D_I} >= 1, which fp32 holds while the
// block decays by at most 2^86 (about e^{59.6}); for channels that decay
// faster the diagonal block's products are formed pair by pair from the
// per-token gates (e^{g_r - g_s} as a product of alphas) instead.  The result
// is exact up to rounding for every finite log_alpha <= 0.

#include <hip/hip_ext.h>

#include <cstdlib>
#include <atomic>
#include <mutex>
#include <vector>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------------------
// MFMA 16x16 output tile for the two element types.
//   A fragment: lane l holds row (l % 16), B fragment: column (l % 16); the
//   lane group g = l / 16 and the slot j inside the lane select the k index.
//   Output (f32x4): lane l holds column (l % 16), rows 4 g + i, i = 0..3.
// Any k assignment works as long as A and B use the same (g, j) -> k map.
// ---------------------------------------------------------------------------
template <typename T>
struct mma16;

template <>
struct mma16<bf16_t> {
  static constexpr int KS = 32;  // k per instruction: slots j = 0..7 per lane
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct mma16<float> {
  static constexpr int KS = 4;  // one slot per lane
  typedef float frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ __bf16 to_bf(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float from_bf(__bf16 x) { return static_cast<float>(x); }

// Scalar element access in LDS arrays of the io type.
template <typename T>
__device__ __forceinline__ float lds_get(const T* p);
template <>
__device__ __forceinline__ float lds_get<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float lds_get<bf16_t>(const bf16_t* p) { return bf16_to_f32(p->bits); }

template <typename T>
__device__ __forceinline__ void lds_put(T* p, float x);
template <>
__device__ __forceinline__ void lds_put<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void lds_put<bf16_t>(bf16_t* p, float x) { p->bits = f32_to_bf16(x); }

// ---------------------------------------------------------------------------
// Fragments in the "natural" k map (prep kernel): slot (g, j) <-> k = k0 + 8 g + j
// for bf16, k = k0 + g for fp32.  The value is X[row][k] * scale[k].
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 frag_nat(const bf16_t* row, const float* scale, int k0, int g) {
  const int kb = k0 + 8 * g;
  const uint4 u = *reinterpret_cast<const uint4*>(row + kb);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(scale + kb);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(scale + kb + 4);
  bf16x8 r;
  r[0] = to_bf(__uint_as_float(u.x << 16) * s0[0]);
  r[1] = to_bf(__uint_as_float(u.x & 0xFFFF0000u) * s0[1]);
  r[2] = to_bf(__uint_as_float(u.y << 16) * s0[2]);
  r[3] = to_bf(__uint_as_float(u.y & 0xFFFF0000u) * s0[3]);
  r[4] = to_bf(__uint_as_float(u.z << 16) * s1[0]);
  r[5] = to_bf(__uint_as_float(u.z & 0xFFFF0000u) * s1[1]);
  r[6] = to_bf(__uint_as_float(u.w << 16) * s1[2]);
  r[7] = to_bf(__uint_as_float(u.w & 0xFFFF0000u) * s1[3]);
  return r;
}
__device__ __forceinline__ bf16x8 frag_nat(const bf16_t* row, int k0, int g) {
  const uint4 u = *reinterpret_cast<const uint4*>(row + k0 + 8 * g);
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ float frag_nat(const float* row, const float* scale, int k0, int g) {
  return row[k0 + g] * scale[k0 + g];
}
__device__ __forceinline__ float frag_nat(const float* row, int k0, int g) { return row[k0 + g]; }

// ---------------------------------------------------------------------------
// Fragments for contractions whose B operand is a set of accumulator tiles
// (scan kernel).  For bf16, k-step s covers accumulator tiles 2s and 2s+1 and
// slot j of lane group g is row 4g+j of tile 2s (j < 4) or row 4g+j-4 of tile
// 2s+1; for fp32, k-step s is row 4g + (s % 4) of tile s / 4.  The A operand
// X[row][k] must be read with the same map (afrag below).
// ---------------------------------------------------------------------------
template <typename T>
struct accb;

template <>
struct accb<bf16_t> {
  static constexpr int KS = 32;
  __device__ __forceinline__ static bf16x8 b(const f32x4* tiles, int s) {
    const f32x4 x = tiles[2 * s], y = tiles[2 * s + 1];
    bf16x8 r;
    r[0] = to_bf(x[0]); r[1] = to_bf(x[1]); r[2] = to_bf(x[2]); r[3] = to_bf(x[3]);
    r[4] = to_bf(y[0]); r[5] = to_bf(y[1]); r[6] = to_bf(y[2]); r[7] = to_bf(y[3]);
    return r;
  }
};

template <>
struct accb<float> {
  static constexpr int KS = 4;
  __device__ __forceinline__ static float b(const f32x4* tiles, int s) { return tiles[s >> 2][s & 3]; }
};

// ---------------------------------------------------------------------------
// a1: chunk offsets per sequence and the longest-first processing order.
// One workgroup of 1024 threads.  chunk_off[n] = sum_{i<n} ceil(L_i / C).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int32_t* __restrict__ cu, int N, int C,
                                                             int32_t* __restrict__ chunk_off,
                                                             int32_t* __restrict__ order, int sort,
                                                             int32_t* __restrict__ ready) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  // overlapped schedule: [0] last segment written, [1] set when a scan
  // loader wave stopped waiting for a segment (its results are then wrong)
  if (tid < 2 && ready) ready[tid] = 0;
  const int per = (N + 1023) / 1024;
  const int b = min(N, tid * per), e = min(N, b + per);
  int s = 0;
  for (int i = b; i < e; ++i) s += (cu[i + 1] - cu[i] + C - 1) / C;
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int i = b; i < e; ++i) {
    chunk_off[i] = run;
    run += (cu[i + 1] - cu[i] + C - 1) / C;
  }
  if (tid == 1023) chunk_off[N] = part[1023];
  for (int i = tid; i < N; i += 1024) {
    if (sort) {
      const int Li = cu[i + 1] - cu[i];
      int r = 0;
      for (int j = 0; j < N; ++j) {
        const int Lj = cu[j + 1] - cu[j];
        r += (Lj > Li) || (Lj == Li && j < i);
      }
      order[r] = i;
    } else {
      order[i] = i;
    }
  }
}

hipError_t launch_chunk_offsets(const int32_t* cu, int N, int C, int32_t* chunk_off, int32_t* order, int sort,
                                hipStream_t st) {
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, st, cu, N, C, chunk_off, order, sort, nullptr);
  return hipGetLastError();
}

// Overlapped schedule: segments 0 .. j of the workspace blocks are written.
// Launched on the prep stream after the last segment's prep, so the prep's
// writes are complete and visible before the counter moves (the prep
// launches of segments 2, 3, ... publish their predecessor the same way, from
// their first thread).
__global__ void ready_kernel(int32_t* ready, int j) {
  if (threadIdx.x == 0) __hip_atomic_store(ready, j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Output stage over o in place: head-wise RMSNorm over the value channels
// (when a weight is given), then the sigmoid output gate (when its
// pre-activation is given).  A row of DV values is LPR lanes, each holding
// 16 bytes (8 bf16 or 4 fp32); a wave covers 64 / LPR rows per step.  The
// state pass's value tiles split dv, so the norm, which spans a whole row,
// runs as this pass.
template <typename T, int DV>
__global__ __launch_bounds__(256) void out_stage_kernel(T* __restrict__ o, const T* __restrict__ zo,
                                                        const float* __restrict__ w, float eps, int64_t rows) {
  constexpr int EPL = 16 / static_cast<int>(sizeof(T));  // elements per lane
  constexpr int LPR = DV / EPL;                           // lanes per row
  constexpr int RPW = 64 / LPR;                           // rows per wave step
  static_assert(LPR >= 4 && LPR <= 32 && 64 % LPR == 0, "row geometry");
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, c0 = (lane % LPR) * EPL;
  const int64_t step = static_cast<int64_t>(gridDim.x) * 4 * RPW;
  for (int64_t base = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RPW; base < rows; base += step) {
    const int64_t row = base + sub;
    const bool live = row < rows;
    const int64_t off = (live ? row : 0) * DV + c0;
    float x[EPL];
    if constexpr (sizeof(T) == 2) {
      const uint4 u = *reinterpret_cast<const uint4*>(o + off);
      const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(wds[j] << 16);
        x[2 * j + 1] = __uint_as_float(wds[j] & 0xFFFF0000u);
      }
    } else {
      const f32x4 u = *reinterpret_cast<const f32x4*>(o + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = u[j];
    }
    if (w) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) ss += x[j] * x[j];
      ss = group_sum<LPR>(ss);
      const float r = 1.f / __builtin_sqrtf(ss * (1.f / DV) + eps);
#pragma unroll
      for (int j = 0; j < EPL; ++j) x[j] *= r * w[c0 + j];
    }
    if (zo) {
      float z[EPL];
      if constexpr (sizeof(T) == 2) {
        const uint4 u = *reinterpret_cast<const uint4*>(zo + off);
        const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[2 * j] = __uint_as_float(wds[j] << 16);
          z[2 * j + 1] = __uint_as_float(wds[j] & 0xFFFF0000u);
        }
      } else {
        const f32x4 u = *reinterpret_cast<const f32x4*>(zo + off);
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] = u[j];
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j) x[j] *= 1.f / (1.f + __expf(-z[j]));
    }
    if (live) {
      if constexpr (sizeof(T) == 2) {
        uint4 u;
        u.x = f32x2_to_bf16x2(x[0], x[1]);
        u.y = f32x2_to_bf16x2(x[2], x[3]);
        u.z = f32x2_to_bf16x2(x[4], x[5]);
        u.w = f32x2_to_bf16x2(x[6], x[7]);
        *reinterpret_cast<uint4*>(o + off) = u;
      } else {
        *reinterpret_cast<f32x4*>(o + off) = f32x4{x[0], x[1], x[2], x[3]};
      }
    }
  }
}

// Overlapped schedule with S_T == S0: the state pass leaves the final states
// in a workspace carry (S0 must survive until the call knows it needs no
// recovery); this copies them to S_T unless the flag word is set, in which
// case the recovery launches rewrite S_T from S0.  n4 float4 elements.
__global__ __launch_bounds__(256) void carry_out_kernel(const f32x4* __restrict__ carry, f32x4* __restrict__ S_T,
                                                        size_t n4, const int* flag) {
  if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n4; i += static_cast<size_t>(gridDim.x) * 256)
    S_T[i] = carry[i];
}

// ---------------------------------------------------------------------------
// Per-(chunk, head) workspace block.  Everything the serial pass needs for one
// chunk is one contiguous block, so the scan streams it into LDS with plain
// linear 16-byte direct-to-LDS loads; the LDS image equals this layout.
//   R   [C][DK]  io   b_r e^{g_r} k_r
//   Qh  [C][DK]  io   e^{g_r} q_r
//   KbT [DK][C]  io   (e^{g_last - g_r} k_r)^T
//   P   [C][C]   io   gated q k^T, lower triangle incl. diagonal
//   T   [C][C]   io   (I + A)^{-1}
//   Gam [DK]     f32  e^{g_last}
//   Bet [C]      f32  beta
// Tiles are stored with two index transforms that the scan's reads undo:
//   * for bf16, each 32-column group is permuted so that the eight k values
//     an MFMA A-fragment needs (4g..4g+3 and 16+4g..16+4g+3, matching the
//     accumulator rows a lane holds) are one contiguous 16-byte granule;
//   * the 16-byte granules of a row are XOR-swizzled by a function of the
//     row so that 16 lanes reading the same logical granule of 16 rows hit
//     16 different LDS bank groups (no padding needed).
// ---------------------------------------------------------------------------
template <typename T, int C, int DK>
struct Blk {
  static constexpr int ES = sizeof(T);
  static constexpr int RB_R = DK * ES;  // row bytes of R, Qh
  static constexpr int RB_K = C * ES;   // row bytes of KbT, P, T
  // P and T are lower triangular; with C = 64 the scan reads rows 0..31
  // only in their first 32 columns (one k-step), so those rows are stored
  // at half width
  static constexpr bool TRI = C == 64;
  static constexpr size_t tri_bytes = TRI ? static_cast<size_t>(32) * (RB_K / 2) + static_cast<size_t>(C - 32) * RB_K
                                          : static_cast<size_t>(C) * RB_K;
  static constexpr size_t oR = 0;
  static constexpr size_t oQ = oR + static_cast<size_t>(C) * DK * ES;
  static constexpr size_t oK = oQ + static_cast<size_t>(C) * DK * ES;
  static constexpr size_t oP = oK + static_cast<size_t>(DK) * C * ES;
  static constexpr size_t oT = oP + tri_bytes;
  static constexpr size_t oG = oT + tri_bytes;
  static constexpr size_t oB = oG + static_cast<size_t>(DK) * 4;
  static constexpr size_t bytes = (oB + static_cast<size_t>(C) * 4 + 1023) / 1024 * 1024;
};

// Index helpers work in unsigned arithmetic (every index is non-negative), so
// divisions and remainders by powers of two stay shifts and masks.
template <int RB>
__device__ __forceinline__ unsigned swz(unsigned row) {
  if constexpr (RB >= 256) return row & 15u;
  else if constexpr (RB == 128) return (row >> 1) & 7u;
  else return (row >> 2) & 3u;
}

template <typename T>
__device__ __forceinline__ unsigned pcol(unsigned c);
template <>
__device__ __forceinline__ unsigned pcol<float>(unsigned c) { return c; }
template <>
__device__ __forceinline__ unsigned pcol<bf16_t>(unsigned c) {
  const unsigned k = c & 31u;
  return (c & ~31u) | (8u * ((k & 15u) >> 2) + 4u * (k >> 4) + (k & 3u));
}

// byte offset of element (row, c) in a stored tile with RB-byte rows
template <typename T, int RB>
__device__ __forceinline__ unsigned toff(unsigned row, unsigned c) {
  constexpr unsigned EPG = 16 / sizeof(T);
  const unsigned p = pcol<T>(c);
  return row * RB + 16u * ((p / EPG) ^ swz<RB>(row)) + (p % EPG) * static_cast<unsigned>(sizeof(T));
}

// byte offset of logical 16-byte granule gi of `row`
template <int RB>
__device__ __forceinline__ unsigned goff(unsigned row, unsigned gi) { return row * RB + 16u * (gi ^ swz<RB>(row)); }

// Triangular tiles (P, T) with C = 64: rows 0..31 are half width (their
// own swizzle), rows 32..63 follow at full width.
template <typename T, int C>
__device__ __forceinline__ unsigned tri_off(unsigned row, unsigned c) {
  constexpr int RB = C * static_cast<int>(sizeof(T));
  if constexpr (C == 64) {
    if (row < 32) return toff<T, RB / 2>(row, c);
    return 32 * (RB / 2) + toff<T, RB>(row - 32, c);
  } else {
    return toff<T, RB>(row, c);
  }
}
template <typename T, int C>
__device__ __forceinline__ unsigned tri_goff(unsigned row, unsigned gi) {
  constexpr int RB = C * static_cast<int>(sizeof(T));
  if constexpr (C == 64) {
    if (row < 32) return goff<RB / 2>(row, gi);
    return 32 * (RB / 2) + goff<RB>(row - 32, gi);
  } else {
    return goff<RB>(row, gi);
  }
}

// A fragment of a stored tile for the accumulator k map (see accb).
template <typename T, int RB>
struct afrag;
template <int RB>
struct afrag<bf16_t, RB> {
  __device__ __forceinline__ static bf16x8 get(const unsigned char* tile, int row, int s, int g) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tile + goff<RB>(row, 4 * s + g)));
  }
};
template <int RB>
struct afrag<float, RB> {
  __device__ __forceinline__ static float get(const unsigned char* tile, int row, int s, int g) {
    return reinterpret_cast<const float*>(tile + goff<RB>(row, 4 * (s >> 2) + g))[s & 3];
  }
};

// hi / lo parts of accumulator tiles used as a B operand (bf16 only; the
// fp32 path has no lo part)
template <typename T>
struct split;
template <>
struct split<bf16_t> {
  static constexpr bool has_lo = true;
  // hi = x rounded to bf16 (nearest even, so the hi part alone -- as used in
  // the state update -- carries no bias), lo = x - hi (exact in fp32)
  // rounded to bf16: hi + lo = x to ~2^-17 relative.  Six VALU per pair.
  __device__ __forceinline__ static void hilo(const f32x4* tiles, int s, bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float x0 = tiles[2 * s + (j >> 2)][j & 3], x1 = tiles[2 * s + (j >> 2)][(j & 3) + 1];
      const uint32_t hp = f32x2_to_bf16x2(x0, x1);
      h[j >> 1] = hp;
      l[j >> 1] = f32x2_to_bf16x2(x0 - __uint_as_float(hp << 16), x1 - __uint_as_float(hp & 0xFFFF0000u));
    }
    hi = __builtin_bit_cast(bf16x8, uint4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, uint4{l[0], l[1], l[2], l[3]});
  }
};
template <>
struct split<float> {
  static constexpr bool has_lo = false;
  __device__ __forceinline__ static void hilo(const f32x4* tiles, int s, float& hi, float& lo) {
    hi = tiles[s >> 2][s & 3];
    lo = 0.f;
  }
};

// Four consecutive io elements through a buffer resource (out-of-range
// offsets are dropped).
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 x, const bf16_t*) {
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  const u32x2 u = {f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3])};
  __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 x, const float*) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

// Four consecutive io elements already in io format (bf16 bits or fp32).
__device__ __forceinline__ void buffer_store_raw4(__amdgpu_buffer_rsrc_t r, int off, uint2 x) {
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{x.x, x.y}, r, off, 0, 0);
}
__device__ __forceinline__ void buffer_store_raw4(__amdgpu_buffer_rsrc_t r, int off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Prep kernel: one workgroup (kPrepThreads threads) per (chunk, head).  The grid's x
// index is the head, so the workgroups that run together cover whole token
// rows of q, k and log_alpha.
//
// Gated products.  For rows r of 16-row block I and columns s of block J <= I
// the row operands (Krd, Qrd) hold k_r e^{d_r}, q_r e^{d_r} and the column
// operand (Kc) k_s e^{s_s}; the pair (I, J) scales the column fragment by one
// per-channel vector: e^{D_{J+1} + ... + D_{I-1}} (<= 1) for J < I, e^{-D_I}
// for J = I, or 0 for a channel whose block decay is out of range, whose
// diagonal products are then added pair by pair (see the note at the top).
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 512;
// Largest block decay (base 2) a diagonal pair's column scale e^{-D_I} may
// carry: past it the channel's diagonal products are formed pair by pair.
constexpr float kDiagRange = 86.f;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int C, int DK>
struct PrepLds {
  static constexpr int NB = C / 16;
  static constexpr int NLB = NB * (NB + 1) / 2;  // lower blocks incl. the diagonal
  static constexpr int NRB = 4 * kPrepThreads / DK;  // row blocks (threads per channel group)
  static constexpr int RBK = DK * static_cast<int>(sizeof(T));  // row bytes of Krd / Qrd / Kc
  static constexpr int AP = C + 1;               // pitch (floats) of A / Ti
  static constexpr int CP = C + 8;               // pitch (elements) of the P staging tile
  static constexpr size_t a16(size_t x) { return (x + 15) / 16 * 16; }
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t szTi = static_cast<size_t>(C) * AP * 4;
  // region 0: Krd, Qrd, Kc (io, swizzled rows) -> later Ti (f32)
  static constexpr size_t r0 = a16(mx(static_cast<size_t>(3) * C * RBK, szTi));
  // region 1: cumsum partials [NRB][DK] (f32) -> later A (f32)
  static constexpr size_t r1 = a16(mx(static_cast<size_t>(C) * AP * 4, static_cast<size_t>(NRB) * DK * 4));
  // region 2: block gate sums D [NB][DK] (f32) -> later P staging (io)
  static constexpr size_t r2 = a16(mx(static_cast<size_t>(NB) * DK * 4, static_cast<size_t>(C) * CP * sizeof(T)));
  // region 3: block-pair vectors f[NLB][DK] (f32)
  static constexpr size_t r3 = a16(static_cast<size_t>(NLB) * DK * 4);
  static constexpr size_t o0 = 0, o1 = r0, o2 = o1 + r1, o3 = o2 + r2, o4 = o3 + r3;
  // after beta: per-row and per-block gate sums of the scalar gate (not
  // reused by later phases: the pair products read them while region 2
  // already stages P)
  static constexpr size_t o5 = o4 + static_cast<size_t>(C) * 4;
  // then per-row inverse norms of k and q (input stage), read by the exact
  // diagonal path
  static constexpr size_t o6 = o5 + static_cast<size_t>(3 * C + NB) * 4;
  static constexpr size_t total = o6 + static_cast<size_t>(2 * C) * 4;
};

// byte offset of element (row, c) in an unpadded LDS tile with RB-byte rows,
// 16-byte granules XOR-swizzled by row (conflict-free 16-row fragment reads)
template <typename T, int RB>
__device__ __forceinline__ unsigned loff(unsigned row, unsigned c) {
  constexpr unsigned EPG = 16 / sizeof(T);
  return row * RB + 16u * ((c / EPG) ^ swz<RB>(row)) + (c % EPG) * static_cast<unsigned>(sizeof(T));
}

// natural-map fragments (slot (g, j) <-> k = k0 + 8 g + j for bf16, k0 + g for fp32)
template <typename T, int RB>
struct natf;
template <int RB>
struct natf<bf16_t, RB> {
  __device__ __forceinline__ static bf16x8 raw(const unsigned char* t, int row, int k0, int g) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(t + loff<bf16_t, RB>(row, k0 + 8 * g)));
  }
  // x * a per channel
  __device__ __forceinline__ static bf16x8 scaled(const unsigned char* t, int row, const float* a, int k0, int g) {
    const uint4 u = *reinterpret_cast<const uint4*>(t + loff<bf16_t, RB>(row, k0 + 8 * g));
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(a + k0 + 8 * g);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(a + k0 + 8 * g + 4);
    bf16x8 r;
    r[0] = to_bf(__uint_as_float(u.x << 16) * a0[0]);
    r[1] = to_bf(__uint_as_float(u.x & 0xFFFF0000u) * a0[1]);
    r[2] = to_bf(__uint_as_float(u.y << 16) * a0[2]);
    r[3] = to_bf(__uint_as_float(u.y & 0xFFFF0000u) * a0[3]);
    r[4] = to_bf(__uint_as_float(u.z << 16) * a1[0]);
    r[5] = to_bf(__uint_as_float(u.z & 0xFFFF0000u) * a1[1]);
    r[6] = to_bf(__uint_as_float(u.w << 16) * a1[2]);
    r[7] = to_bf(__uint_as_float(u.w & 0xFFFF0000u) * a1[3]);
    return r;
  }
};
template <int RB>
struct natf<float, RB> {
  __device__ __forceinline__ static float raw(const unsigned char* t, int row, int k0, int g) {
    return *reinterpret_cast<const float*>(t + loff<float, RB>(row, k0 + g));
  }
  __device__ __forceinline__ static float scaled(const unsigned char* t, int row, const float* a, int k0, int g) {
    return raw(t, row, k0, g) * a[k0 + g];
  }
};

// (I + A_II)^{-1} of one 16x16 diagonal block on fp32 MFMA, in registers.
// With M = -A_II (strictly lower, so M^16 = 0) the inverse is
// (I + M)(I + M^2)(I + M^4)(I + M^8).  m and mt hold M and M^T in accumulator
// layout (lane (n, g) holds X[4g + i][n] in slot i).  A product X Y takes its
// left factor as X^T in accumulator layout, so the powers of M are formed in
// both layouts (M^8 only transposed), and since powers of M commute with each
// other and with the partial products, every product puts a power on the left.
__device__ __forceinline__ f32x4 unit_lower_inverse16(f32x4 m, f32x4 mt, int n, int g) {
  auto mul = [](f32x4 xt, f32x4 y) {  // X Y
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mma16<float>::mma(xt[s], y[s], acc);
    return acc;
  };
  const f32x4 m2 = mul(mt, m), m2t = mul(m, mt);
  const f32x4 m4t = mul(m2, m2t);
  const f32x4 m8t = mul(mul(m2t, m2), m4t);  // (M^4 M^4)^T from M^4 and (M^4)^T
  const f32x4 m3 = mul(mt, m2);
  f32x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = ((4 * g + i) == n ? 1.f : 0.f) + m[i] + m2[i] + m3[i];  // (I + M)(I + M^2)
  p += mul(m4t, p);  // ... (I + M^4)
  p += mul(m8t, p);  // ... (I + M^8)
  return p;
}

// Waves per SIMD the prep kernel is built for: as many workgroups as LDS
// allows per CU, each of kPrepThreads / 64 waves over 4 SIMDs, at most 4
// (128 registers per lane).
template <typename T, int C, int DK>
constexpr int prep_waves_per_eu() {
  constexpr int wgs = (160 * 1024) / PrepLds<T, C, DK>::total > 0 ? (160 * 1024) / PrepLds<T, C, DK>::total : 1;
  return wgs * kPrepThreads / 256 < 4 ? wgs * kPrepThreads / 256 : 4;
}

// G is the gate form (kda_gate): per key channel, one per head, or none.
// With one rate per head every gate factor is a per-row scalar, the gated
// products are the plain k k^T and q k^T products scaled element by element
// by e^{g_r - g_s} (formed from sums over the rows in between), and without
// a gate all factors are 1.
// IN selects the input stage (L2-normalised q and k, gate activation).
template <typename T, int C, int DK, int G, bool IN>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(prep_waves_per_eu<T, C, DK>())))
void prep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const float* __restrict__ la, const float* __restrict__ beta,
                                                   const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ chunk_off, int N, int H,
                                                   unsigned char* __restrict__ ws, int cbase, int count,
                                                   int32_t* publish, int published, const int* guard, int cl,
                                                   int l2n, float l2eps, int softplus_gate) {
  typedef PrepLds<T, C, DK> L;
  typedef Blk<T, C, DK> B;
  typedef mma16<T> M;
  typedef mma16<float> MF;
  // Recovery launch: runs only if the flag word is nonzero (see scan_kernel).
  if (guard && __hip_atomic_load(guard, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;
  // Stream order started this launch after the previous one on its stream
  // had ended (and released its writes): tell the scan those blocks exist.
  if (publish && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(publish, published, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr int NB = L::NB;
  constexpr int RPT = C / L::NRB;  // rows per thread
  static_assert(RPT >= 1 && 16 % RPT == 0, "row blocks must tile 16-row sub-blocks");
  static_assert(NB < kPrepThreads / 64, "diagonal pairs take one wave each, and at least one wave is left");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* Krd = smem + L::o0;
  unsigned char* Qrd = Krd + C * L::RBK;
  unsigned char* Kc = Qrd + C * L::RBK;
  float* Ti = reinterpret_cast<float*>(smem + L::o0);
  float* A = reinterpret_cast<float*>(smem + L::o1);
  float* Dblk = reinterpret_cast<float*>(smem + L::o2);  // block gate sums [NB][DK]
  T* Ps = reinterpret_cast<T*>(smem + L::o2);
  float* fv = reinterpret_cast<float*>(smem + L::o3);
  float* bet = reinterpret_cast<float*>(smem + L::o4);
  // scalar gate: per row, its log_alpha (base 2), d and s (see a2); per block D
  float* lrow = reinterpret_cast<float*>(smem + L::o5);
  float* drow = lrow + C;
  float* srow = drow + C;
  float* dsum = srow + C;
  float* rinv = reinterpret_cast<float*>(smem + L::o6);  // [2][C]: 1/||k_r||, 1/||q_r|| (input stage)
  constexpr bool kChannel = G == KDA_GATE_CHANNEL, kScalar = G == KDA_GATE_SCALAR;

  // thread owns channels c4..c4+3 of rows r0..r0+RPT-1 in the elementwise steps
  constexpr int NCG = DK / 4;  // channel groups of 4

  // Persistent: the workgroup walks items (chunk c = cbase + i / H, head
  // h = i % H) with stride gridDim.x, loading the next item's inputs into
  // registers while it works on the current one.
  const int total = chunk_off[N];
  const int nitems = count * H;
  struct Item {
    int c, h, t0, len;
  };
  auto locate = [&](int item) {
    Item it{total, 0, 0, 0};  // c >= total: nothing to do
    if (item >= nitems) return it;
    it.c = cbase + item / H;
    it.h = item % H;
    if (it.c >= total) return it;
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_off[mid] <= it.c) lo = mid; else hi = mid - 1;
    }
    it.t0 = cu[lo] + (it.c - chunk_off[lo]) * cl;
    it.len = min(cl, cu[lo + 1] - it.t0);
    return it;
  };
  struct Raw {
    f32x4 lg[RPT];
    typename raw4<T>::type kr[RPT], qr[RPT];
    float bt;
  };
  // Rows past the end re-read the last row (all loads issue back to back);
  // their log_alpha is zeroed and beta = 0 masks them everywhere else.  The
  // gates (log_alpha, beta) and q, k can be fetched separately.
  auto fetch = [&](const Item& it, Raw& r, bool gates, bool qk) {
    if (it.c >= total) return;
    // thread indices from a zero the compiler cannot see (len <= C): they
    // are recomputed here rather than held in registers across the item loop
    const int t = static_cast<int>(threadIdx.x) + (it.len >> 30);
    const int fr0 = (t / NCG) * RPT, fc4 = 4 * (t % NCG);
    const size_t tbase = (static_cast<size_t>(it.t0) * H + it.h) * DK;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int e = min(fr0 + i, it.len - 1) * H * DK + fc4;  // < C H DK: 32-bit
      if constexpr (kChannel) {
        if (gates) r.lg[i] = *reinterpret_cast<const f32x4*>(la + tbase + e);
      } else if constexpr (kScalar) {
        if (gates) {
          const float x = la[(static_cast<size_t>(it.t0) + min(fr0 + i, it.len - 1)) * H + it.h];
          r.lg[i] = f32x4{x, x, x, x};
        }
      }
      if (qk) {
        r.kr[i] = load4raw(k + tbase + e);
        r.qr[i] = load4raw(q + tbase + e);
      }
    }
    if (gates) r.bt = (t < C && t < it.len) ? beta[static_cast<size_t>(it.t0 + t) * H + it.h] : 0.f;
  };
  int item = blockIdx.x;
  Item it = locate(item);
  Raw cur;
  fetch(it, cur, true, true);
  for (; item < nitems; item += gridDim.x) {
    const Item nit = locate(item + gridDim.x);
    Raw nxt;
    const int c = it.c, h = it.h, t0 = it.t0, len = it.len;
    // Per-thread index math is redone per item (a zero the compiler cannot
    // see, len <= C, keeps it from hoisting the math out of the loop, where
    // it would hold registers across every item).
    const int tid = static_cast<int>(threadIdx.x) + (len >> 30);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int cg = tid % NCG, rbk = tid / NCG;
    const int c4 = 4 * cg, r0 = rbk * RPT;
    if (it.c < total) {
  unsigned char* blk = ws + (static_cast<size_t>(c) * H + h) * B::bytes;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(blk, 0, static_cast<int>(B::bytes), 0x00020000);
  // Gates in base 2 (log2(e) * log_alpha), so every factor is one v_exp_f32.
  f32x4 lg[RPT], kv[RPT], qv[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    if constexpr (G == KDA_GATE_NONE) {
      lg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      f32x4 la4 = cur.lg[i];
      if (IN && softplus_gate) {
#pragma unroll
        for (int j = 0; j < 4; ++j) la4[j] = neg_softplus(la4[j]);
      }
      lg[i] = r0 + i < len ? la4 * kLog2e : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    kv[i] = cvt4(cur.kr[i]);
    qv[i] = cvt4(cur.qr[i]);
  }
  // input stage: each row of k and q divided by max(its norm, eps); the
  // NCG threads of a row are consecutive lanes of one wave
  if (IN && l2n) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float sk = kv[i][0] * kv[i][0] + kv[i][1] * kv[i][1] + kv[i][2] * kv[i][2] + kv[i][3] * kv[i][3];
      float sq = qv[i][0] * qv[i][0] + qv[i][1] * qv[i][1] + qv[i][2] * qv[i][2] + qv[i][3] * qv[i][3];
      sk = group_sum<NCG>(sk);
      sq = group_sum<NCG>(sq);
      const float ik = 1.f / fmaxf(__builtin_sqrtf(sk), l2eps), iq = 1.f / fmaxf(__builtin_sqrtf(sq), l2eps);
      kv[i] *= ik;
      qv[i] *= iq;
      if (cg == 0) {
        rinv[r0 + i] = ik;
        rinv[C + r0 + i] = iq;
      }
    }
  }
  if (tid < C) bet[tid] = cur.bt;

  // ---- a2: gate sums inside each 16-row block (base 2) ---------------------
  // The thread's rows r0 .. r0 + RPT - 1 lie in block I; TPB threads of its
  // channel group share the block.  dl[i] = d (rows of the block up to and
  // including the row), sl[i] = s (rows after it), both summed directly.
  constexpr int TPB = 16 / RPT;
  const int I = r0 >> 4, pos = rbk % TPB, rb0 = rbk - pos;
  f32x4 dl[RPT], sl[RPT];
  {
    float* part = reinterpret_cast<float*>(smem + L::o1);
    f32x4 tot = lg[0];
#pragma unroll
    for (int i = 1; i < RPT; ++i) tot += lg[i];
    *reinterpret_cast<f32x4*>(part + rbk * DK + c4) = tot;
    __syncthreads();
    f32x4 before = {0.f, 0.f, 0.f, 0.f}, after = {0.f, 0.f, 0.f, 0.f}, whole = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pp = 0; pp < TPB; ++pp) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(part + (rb0 + pp) * DK + c4);
      if (pp < pos) before += x;
      if (pp > pos) after += x;
      whole += x;
    }
    f32x4 run = before;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      run += lg[i];
      dl[i] = run;
    }
    run = after;
#pragma unroll
    for (int i = RPT - 1; i >= 0; --i) {
      sl[i] = run;
      run += lg[i];
    }
    if (pos == 0) *reinterpret_cast<f32x4*>(Dblk + I * DK + c4) = whole;
    if constexpr (kScalar) {
      if (cg == 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          lrow[r0 + i] = lg[i][0];
          drow[r0 + i] = dl[i][0];
          srow[r0 + i] = sl[i][0];
        }
        if (pos == 0) dsum[I] = whole[0];
      }
    }
  }
  __syncthreads();

  // ---- block-pair vectors: for J < I, e^{D_{J+1} + ... + D_{I-1}} (<= 1);
  // for the diagonal pair (J, J), e^{-D_J} (>= 1), or 0 where it would
  // exceed 2^86 (that channel's diagonal products are formed pair by pair)
  for (int idx = tid; kChannel && idx < L::NLB * DK; idx += kPrepThreads) {
    const unsigned pp = static_cast<unsigned>(idx) / DK, ch = static_cast<unsigned>(idx) % DK;
    unsigned bI = 0;
#pragma unroll
    for (unsigned t = 1; t < static_cast<unsigned>(NB); ++t) bI += pp >= t * (t + 1) / 2 ? 1u : 0u;
    const unsigned bJ = pp - bI * (bI + 1) / 2;
    float x;
    if (bI == bJ) {
      x = -Dblk[bJ * DK + ch];
      fv[idx] = x <= kDiagRange ? __builtin_amdgcn_exp2f(x) : 0.f;
    } else {
      x = 0.f;
      for (unsigned kk = bJ + 1; kk < bI; ++kk) x += Dblk[kk * DK + ch];
      fv[idx] = __builtin_amdgcn_exp2f(x);
    }
  }
  if (tid < DK) {
    float x = 0.f;
#pragma unroll
    for (int kk = 0; kk < NB; ++kk) x += Dblk[kk * DK + tid];
    reinterpret_cast<float*>(blk + B::oG)[tid] = G == KDA_GATE_NONE ? 1.f : __builtin_amdgcn_exp2f(x);  // e^{g_last}
  }
  if (tid < C) reinterpret_cast<float*>(blk + B::oB)[tid] = bet[tid];

  // The next item's gates (half of its input bytes) load from here on: this
  // item's copies are dead and the registers stay free through the factor
  // pass.  Issued one phase later, behind this item's block stores, the
  // prep ran 4-6% slower.
  fetch(nit, nxt, true, false);

  // ---- element factors, S-independent outputs ---------------------------
  {
    // e^{sum of D over the blocks before I} and after I, per channel
    f32x4 sb = {0.f, 0.f, 0.f, 0.f}, sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NB; ++kk) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(Dblk + kk * DK + c4);
      if (kk < I) sb += x;
      if (kk > I) sa += x;
    }
    f32x4 ebv, eav, kb[RPT];
    float bt[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) bt[i] = bet[r0 + i];
    if constexpr (kChannel) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ebv[j] = __builtin_amdgcn_exp2f(sb[j]);  // <= 1
        eav[j] = __builtin_amdgcn_exp2f(sa[j]);  // <= 1
      }
    } else if constexpr (kScalar) {
      const float eb = __builtin_amdgcn_exp2f(sb[0]), ea = __builtin_amdgcn_exp2f(sa[0]);
      ebv = f32x4{eb, eb, eb, eb};
      eav = f32x4{ea, ea, ea, ea};
    } else {
      ebv = f32x4{1.f, 1.f, 1.f, 1.f};
      eav = ebv;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const unsigned r = static_cast<unsigned>(r0 + i);
      f32x4 ed, es;
      if constexpr (kChannel) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ed[j] = __builtin_amdgcn_exp2f(dl[i][j]);  // e^{d_r} <= 1
          es[j] = __builtin_amdgcn_exp2f(sl[i][j]);  // e^{s_r} <= 1
        }
      } else if constexpr (kScalar) {
        const float a = __builtin_amdgcn_exp2f(dl[i][0]), b = __builtin_amdgcn_exp2f(sl[i][0]);
        ed = f32x4{a, a, a, a};
        es = f32x4{b, b, b, b};
      } else {
        ed = f32x4{1.f, 1.f, 1.f, 1.f};
        es = ed;
      }
      const f32x4 fre = ed * ebv;  // e^{g_r}
      const unsigned lo = loff<T, L::RBK>(r, static_cast<unsigned>(c4));
      if constexpr (kChannel) {
        store4(reinterpret_cast<T*>(Krd + lo), kv[i] * ed);
        store4(reinterpret_cast<T*>(Qrd + lo), qv[i] * ed);
        store4(reinterpret_cast<T*>(Kc + lo), kv[i] * es);
      } else {
        // plain operands (the column operand is Krd itself); the gate is
        // applied to the products element by element
        store4(reinterpret_cast<T*>(Krd + lo), kv[i]);
        store4(reinterpret_cast<T*>(Qrd + lo), qv[i]);
      }
      const f32x4 kc = kv[i] * es;
      const int to = static_cast<int>(toff<T, B::RB_R>(r, static_cast<unsigned>(c4)));
      buffer_store4(wr, static_cast<int>(B::oQ) + to, qv[i] * fre, static_cast<T*>(nullptr));
      buffer_store4(wr, static_cast<int>(B::oR) + to, bt[i] * (kv[i] * fre), static_cast<T*>(nullptr));
      kb[i] = kc * eav;  // e^{g_last - g_r} k_r
    }
  // Kb^T tile (rows = key channel): this thread's rows are consecutive, so
    // groups of 4 stay contiguous under the column permutation.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (RPT % 4 == 0) {
#pragma unroll
        for (int i4 = 0; i4 < RPT; i4 += 4) {
          const f32x4 x4 = {kb[i4][j], kb[i4 + 1][j], kb[i4 + 2][j], kb[i4 + 3][j]};
          buffer_store4(wr, static_cast<int>(B::oK + toff<T, B::RB_K>(c4 + j, r0 + i4)), x4, static_cast<T*>(nullptr));
        }
      } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
          io<T>::store(reinterpret_cast<T*>(blk + B::oK + toff<T, B::RB_K>(c4 + j, r0 + i)), kb[i][j]);
      }
    }
  }
  __syncthreads();
    }  // item, first half
    // The next item's q and k, whose registers are free from here on.  Issued
    // before this barrier (among or right after the block stores), or row by
    // row inside the factor pass, the prep ran 11-16% slower.
    fetch(nit, nxt, false, true);
    if (it.c < total) {
  unsigned char* blk = ws + (static_cast<size_t>(c) * H + h) * B::bytes;

  // ---- a3: gated k k^T (A, fp32 in LDS) and q k^T (P) via MFMA, and the
  // diagonal blocks of the UT inverse T = (I + A)^{-1} ----------------------
  // Channels of diagonal block I whose scale is 0 (decay beyond 2^86 across
  // the block): their contributions to this lane's A and P values, from the
  // per-token gates, e^{g_r - g_s} = prod_{s < u <= r} alpha_u.  Rows past
  // the end take alpha = 1 (and are masked by beta = 0, or unused).
  auto diag_exact = [&](int I, f32x4& aA, f32x4& aP) {
    const float* sd = fv + (I * (I + 1) / 2 + I) * DK;
#pragma unroll
    for (int j = 0; j < (DK + 63) / 64; ++j) {
      unsigned long long m = __ballot(lane < DK - 64 * j && sd[64 * j + lane] == 0.f);
      while (m) {
        const int ch = 64 * j + static_cast<int>(__builtin_ctzll(m));
        m &= m - 1;
        const int row = 16 * I + n;
        const size_t e = (static_cast<size_t>(t0 + min(row, len - 1)) * H + h) * DK + ch;
        const float lz = (IN && softplus_gate) ? neg_softplus(la[e]) : la[e];
        const float an = row < len ? __builtin_amdgcn_exp2f(lz * kLog2e) : 1.f;
        float kn = io<T>::load(k + e), qn = io<T>::load(q + e);
        if (IN && l2n) {
          kn *= rinv[row];
          qn *= rinv[C + row];
        }
        float prod = 1.f, ef[4] = {1.f, 1.f, 1.f, 1.f}, kr[4] = {0.f, 0.f, 0.f, 0.f}, qr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float au = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(an), u));
          const float ku = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kn), u));
          const float qu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qn), u));
          if (u > n) prod *= au;
          if (g == (u >> 2)) {
            ef[u & 3] = prod;
            kr[u & 3] = ku;
            qr[u & 3] = qu;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          aA[i] += kr[i] * kn * ef[i];
          aP[i] += qr[i] * kn * ef[i];
        }
      }
    }
  };
  // Block pair (I, J <= I); returns this lane's A values (beta-scaled, masked).
  auto pair = [&](int I, int J) {
    f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kChannel) {
      const float* f = fv + (I * (I + 1) / 2 + J) * DK;  // column scale of the pair
#pragma unroll 8
      for (int k0 = 0; k0 < DK; k0 += M::KS) {
        const typename M::frag bf = natf<T, L::RBK>::scaled(Kc, 16 * J + n, f, k0, g);
        aA = M::mma(natf<T, L::RBK>::raw(Krd, 16 * I + n, k0, g), bf, aA);
        aP = M::mma(natf<T, L::RBK>::raw(Qrd, 16 * I + n, k0, g), bf, aP);
      }
      if (I == J) diag_exact(I, aA, aP);
    } else {
#pragma unroll 8
      for (int k0 = 0; k0 < DK; k0 += M::KS) {
        const typename M::frag bf = natf<T, L::RBK>::raw(Krd, 16 * J + n, k0, g);
        aA = M::mma(natf<T, L::RBK>::raw(Krd, 16 * I + n, k0, g), bf, aA);
        aP = M::mma(natf<T, L::RBK>::raw(Qrd, 16 * I + n, k0, g), bf, aP);
      }
      if constexpr (kScalar) {
        // e^{g_r - g_s} for this lane's (row, column): the rows s+1 .. r of
        // a diagonal block summed one by one, else d_r + s_s + the blocks
        // strictly between -- every term <= 0
        f32x4 x;
        if (I == J) {
          x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 1; u < 16; ++u) {
            const float lu = lrow[16 * I + u];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (u > n && u <= 4 * g + i) x[i] += lu;
          }
        } else {
          float mid = srow[16 * J + n];
          for (int kk = J + 1; kk < I; ++kk) mid += dsum[kk];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = drow[16 * I + 4 * g + i] + mid;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w = __builtin_amdgcn_exp2f(x[i]);
          aA[i] *= w;
          aP[i] *= w;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * g + i;
      const int row = 16 * I + rr, col = 16 * J + n;
      float a = aA[i] * bet[row];
      float pv = aP[i];
      if (I == J && rr <= n) a = 0.f;
      if (I == J && rr < n) pv = 0.f;
      A[row * L::AP + col] = a;
      lds_put<T>(Ps + row * L::CP + col, pv);
      aA[i] = a;
    }
    return aA;
  };
  // Waves 0..NB-1 take one diagonal pair each and invert I + A_II right away
  // from registers; the other waves take the off-diagonal pairs.  Until the
  // barrier the T tile's LDS still holds Krd/Qrd/Kc, so the inverse stays in
  // registers and a transposed copy goes to the upper triangle of A's block
  // (I, I), which A (strictly lower) leaves unused: T_II[r][c], r >= c, at
  // A_II's position (c, r).
  f32x4 tii = {0.f, 0.f, 0.f, 0.f};
  if (wave < NB) {
    const f32x4 a = pair(wave, wave);
    float* Ab = A + (16 * wave) * L::AP + 16 * wave;
    __builtin_amdgcn_wave_barrier();  // other lanes' A_II stores before the reads below
    f32x4 m, mt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = -a[i];
      mt[i] = -Ab[n * L::AP + 4 * g + i];  // written by other lanes of this wave
    }
    tii = unit_lower_inverse16(m, mt, n, g);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i >= n) Ab[n * L::AP + 4 * g + i] = tii[i];
  } else {
    // the o-th off-diagonal pair, row by row: (1,0), (2,0), (2,1), (3,0), ...
    for (int o = wave - NB; o < NB * (NB - 1) / 2; o += kPrepThreads / 64 - NB) {
      int I = 1;
      while ((I + 1) * I / 2 <= o) ++I;
      pair(I, o - I * (I - 1) / 2);
    }
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(blk, 0, static_cast<int>(B::bytes), 0x00020000);
  if (wave < NB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Ti[(16 * wave + 4 * g + i) * L::AP + 16 * wave + n] = tii[i];
  }
  if (wave < NB - 1) {
    // ---- a4: column J of T below the diagonal, top to bottom, one wave:
    //   T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
    // every T_KJ is this wave's own earlier result; T_II is read from its
    // transposed copy in A.
    const int J = wave;
    for (int I = J + 1; I < NB; ++I) {
      __builtin_amdgcn_wave_barrier();  // T_KJ stored by other lanes of this wave
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          x = MF::mma(A[(16 * I + n) * L::AP + 16 * K + 4 * s + g], Ti[(16 * K + 4 * s + g) * L::AP + 16 * J + n], x);
      }
      const float* Ab = A + (16 * I) * L::AP + 16 * I;
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int cc = 4 * g + s;  // T_II[n][cc]
        t = MF::mma(cc <= n ? Ab[cc * L::AP + n] : 0.f, x[s], t);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Ti[(16 * I + 4 * g + i) * L::AP + 16 * J + n] = -t[i];
    }
  } else {
    // the remaining waves store P meanwhile
    for (int idx = tid - 64 * (NB - 1); idx < C * C / 4; idx += kPrepThreads - 64 * (NB - 1)) {
      const unsigned r = static_cast<unsigned>(idx) / (C / 4), c4b = (static_cast<unsigned>(idx) % (C / 4)) * 4;
      typename raw4<T>::type x = {};
      if ((c4b >> 4) <= (r >> 4)) x = *reinterpret_cast<const typename raw4<T>::type*>(Ps + r * L::CP + c4b);
      if (!B::TRI || r >= 32 || c4b < 32) buffer_store_raw4(wr, static_cast<int>(B::oP + tri_off<T, C>(r, c4b)), x);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < C * C / 4; idx += kPrepThreads) {
    const unsigned r = static_cast<unsigned>(idx) / (C / 4), c4b = (static_cast<unsigned>(idx) % (C / 4)) * 4;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if ((c4b >> 4) <= (r >> 4)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = Ti[r * L::AP + c4b + j];
    }
    if (!B::TRI || r >= 32 || c4b < 32)
      buffer_store4(wr, static_cast<int>(B::oT + tri_off<T, C>(r, c4b)), x, static_cast<T*>(nullptr));
  }
    }  // item
    __syncthreads();  // LDS is reused by the next item
    it = nit;
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// Scan kernel: one workgroup per (sequence, head, value tile of 16*WAVES
// columns); wave w owns 16 columns and keeps its dk x 16 slice of the state
// in MFMA accumulators for the whole sequence.  Chunk blocks stream into LDS
// (double-buffered when two fit) with direct 16-byte loads issued one chunk
// ahead; the bf16 path splits Y and D into hi + lo bf16 parts where they feed
// the output (T Y and P D), keeping those contractions at ~fp32 accuracy.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void lds_load16(const unsigned char* src, unsigned char* dst_wave_base) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                   (__attribute__((address_space(3))) void*)(dst_wave_base), 16, 0, 0);
}

// s_waitcnt for at most N outstanding vector-memory loads (lgkmcnt, expcnt
// left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The first NS k-step A fragments of one stored-tile row (accumulator k map).
template <typename T, int RB, int NS>
struct RowFrags;
template <int RB, int NS>
struct RowFrags<bf16_t, RB, NS> {
  bf16x8 f[NS];
  __device__ __forceinline__ void load(const unsigned char* tile, int row, int g) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      f[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tile + goff<RB>(row, 4 * s + g)));
  }
};
template <int RB, int NS>
struct RowFrags<float, RB, NS> {
  float f[NS];
  __device__ __forceinline__ void load(const unsigned char* tile, int row, int g) {
#pragma unroll
    for (int t = 0; t < (NS + 3) / 4; ++t) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(tile + goff<RB>(row, 4 * t + g));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * t + j < NS) f[4 * t + j] = x[j];
    }
  }
};

// The k-steps a 16-row block mt of a triangular tile (P, T) needs: those
// covering columns 0 .. 16 mt + 15.
template <typename T, int C, int NS>
struct TriFrags;
template <int C, int NS>
struct TriFrags<bf16_t, C, NS> {
  bf16x8 f[NS];
  __device__ __forceinline__ void load(const unsigned char* tile, int mt, int n, int g) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s <= (16 * mt + 15) / 32)
        f[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tile + tri_goff<bf16_t, C>(16 * mt + n, 4 * s + g)));
  }
};
template <int C, int NS>
struct TriFrags<float, C, NS> {
  float f[NS];
  __device__ __forceinline__ void load(const unsigned char* tile, int mt, int n, int g) {
#pragma unroll
    for (int t = 0; t < (NS + 3) / 4; ++t) {
      if (4 * t <= (16 * mt + 15) / 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(tile + tri_goff<float, C>(16 * mt + n, 4 * t + g));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * t + j < NS) f[4 * t + j] = x[j];
      }
    }
  }
};

// Loader waves per scan workgroup: they only stream chunk blocks into LDS.
constexpr int kLoaderWaves = 4;

// 4x4 transpose inside each quad of lanes: lane j of the quad holds x[i] =
// element (row i, column j) on entry and (row j, column i) on exit.  Two
// rounds of quad_perm swaps (partner lane j ^ 1, then j ^ 2).
template <int D>
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), D == 1 ? 0xB1 : 0x4E, 0xF, 0xF, true));
}
template <int D>
__device__ __forceinline__ void quad_round(f32x4& x, bool up, int a, int b) {
  const float r = quad_swap<D>(up ? x[a] : x[b]);
  const float xa = up ? r : x[a], xb = up ? x[b] : r;
  x[a] = xa;
  x[b] = xb;
}
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int j) {
  quad_round<1>(x, (j & 1) != 0, 0, 1);
  quad_round<1>(x, (j & 1) != 0, 2, 3);
  quad_round<2>(x, (j & 2) != 0, 0, 2);
  quad_round<2>(x, (j & 2) != 0, 1, 3);
  return x;
}

// One io element into LDS.
__device__ __forceinline__ void lds_put1(unsigned char* p, float x, const bf16_t*) {
  *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(x);
}
__device__ __forceinline__ void lds_put1(unsigned char* p, float x, const float*) {
  *reinterpret_cast<float*>(p) = x;
}

// Workgroup barrier that waits only for this wave's LDS traffic (lgkmcnt 0),
// not for its global loads and stores, which may stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scan LDS.  Double-buffered (NBUF = 2) when two chunks fit: the block is
// split into an early part (R, Qh: read by the first products only) and a
// late part (Kb^T, P, T, Gamma, beta, then the v tile), each with two slots,
// so the early part of chunk cc + 2 can stream in from the middle of chunk cc.
// Otherwise one slot holds the whole block and v tile.
template <typename T, int C, int DK, int TILE>
struct ScanLds {
  typedef Blk<T, C, DK> B;
  static constexpr size_t vtile = static_cast<size_t>(C) * TILE * sizeof(T);  // v rows of this tile
  static constexpr size_t vbytes = (vtile + 1023) / 1024 * 1024;
  static constexpr size_t stage = B::bytes + vbytes;
  static constexpr int NBUF = (2 * stage <= 160 * 1024) ? 2 : 1;
  static constexpr size_t early = B::oK;                          // R, Qh
  static constexpr size_t late = B::bytes - B::oK + vbytes;       // Kb^T, P, T, Gamma, beta, v
  static constexpr size_t late0 = NBUF == 2 ? 2 * early : early;  // first late slot
  // Output staging (double-buffered scheme only): the compute waves leave a
  // chunk's output tile here; the loader waves store it to HBM.
  static constexpr size_t orow = static_cast<size_t>(TILE) * sizeof(T);  // bytes per output row
  static constexpr size_t ostage = NBUF * stage;
  static constexpr bool stage_o = NBUF == 2 && ostage + C * orow <= 160 * 1024;
  static constexpr size_t dx = ostage + (stage_o ? C * orow : 0);
  // Split roles (with the staged output): per 16-column group a state wave
  // (R S, T Y, Kb^T D) and an output wave (Qh S, P D) that takes the
  // state's B fragments and D (hi and lo bf16 parts, or fp32) from LDS.
  // Per lane: D takes C bytes, the state fragments DK / 2 (bf16) or DK (fp32).
  static constexpr size_t sx_group = 64 * static_cast<size_t>(DK) * (sizeof(T) == 2 ? 1 : 2) / 2;
  static constexpr size_t dx_group = 64 * static_cast<size_t>(C) + sx_group;
  static constexpr bool split = stage_o && dx + (TILE / 16) * dx_group <= 160 * 1024;
  static constexpr int roles = split ? 2 : 1;
  // per column group: a 4-byte counter of D hand-overs (state -> output wave)
  static constexpr size_t xflag = dx + (split ? (TILE / 16) * dx_group : 0);
  // 256 bytes that the loader waves' L2 prefetches land in (never read)
  static constexpr size_t pfsink = xflag + (split ? (TILE / 16) * 4 : 0);
  static constexpr size_t total = pfsink + (NBUF == 2 ? 256 : 0);
};

template <typename T, int C, int DK, int WAVES>
constexpr int scan_threads() {
  return 64 * (WAVES * ScanLds<T, C, DK, 16 * WAVES>::roles + kLoaderWaves);
}

template <typename T, int C, int DK, int DV, int WAVES, bool SEG>
__global__ __launch_bounds__((scan_threads<T, C, DK, WAVES>())) void scan_kernel(
    const T* __restrict__ v, const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ order, int N, int H, const unsigned char* __restrict__ ws, const float* S0,
    T* __restrict__ o, float* S_T, int* ready, int seg, int wait_polls, const int* guard, int cl, float* carry,
    int gb, int ge) {
  typedef Blk<T, C, DK> B;
  typedef mma16<T> M;
  typedef accb<T> AB;
  typedef split<T> SP;
  typedef typename M::frag F;
  constexpr int TILE = 16 * WAVES;
  typedef ScanLds<T, C, DK, TILE> SL;
  constexpr int NSPLIT = DV / TILE;
  constexpr int MT = C / 16;
  constexpr int ST = DK / 16;
  constexpr int NSK = DK / AB::KS;  // k-steps over key channels
  constexpr int NSC = C / AB::KS;   // k-steps over chunk rows
  constexpr int NG = static_cast<int>(B::bytes / 1024);  // 1 KB wave-loads per block
  constexpr int VROWB = TILE * static_cast<int>(sizeof(T));  // bytes of one v row of the tile
  constexpr int VLPR = VROWB / 16;                            // lanes per v row
  constexpr int VRPL = 64 / VLPR;                             // v rows per wave-load
  constexpr int NVG = C / VRPL;                               // wave-loads per v tile
  static_assert(VROWB % 16 == 0 && 64 % VLPR == 0 && C % VRPL == 0, "v tile geometry");
  extern __shared__ __align__(1024) unsigned char smem[];
  // Recovery launch of the overlapped schedule: runs only if the state pass
  // of the call stopped waiting for prepared chunks (flag word nonzero).
  if (guard && __hip_atomic_load(guard, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;

  const int x = blockIdx.x;
  const int xcd = x & 7, slot8 = x >> 3;
  const int tile = slot8 % NSPLIT, grp = slot8 / NSPLIT;
  const int p = grp * 8 + xcd;
  if (p >= N * H) return;
  const int seq = order[p / H];
  const int h = p % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loops scalar
  constexpr int CW = WAVES * SL::roles;  // compute waves
  const bool loader = wave >= CW;
  const int tbeg = cu[seq], L_seq = cu[seq + 1] - tbeg;
  const int c0 = chunk_off[seq];
  const int nch = (L_seq + cl - 1) / cl;
  // The sequence's chunks [cb, ce): all of them, or with SEG (bounded
  // schedule) those among global chunks [gb, ge), starting from the state
  // the previous segment left in `carry` unless the sequence starts here and
  // leaving it there unless the sequence ends here.  When `ready` is given,
  // the blocks of global chunks [j seg, (j + 1) seg) exist once *ready >= j
  // (segment 0 from the start): the loader waves wait for that before they
  // touch them.
  int cb = 0, ce = nch;
  const float* s_in = S0;
  float* s_out = S_T;
  if constexpr (SEG) {
    cb = min(max(gb - c0, 0), nch);
    ce = min(max(ge - c0, 0), nch);
    if (cb == ce && !(nch == 0 && gb == 0)) return;  // nothing of this sequence in the segment
    if (cb > 0) s_in = carry;
    if (ce < nch) s_out = carry;
  }

  // Loader waves: `upto` is the last chunk of this sequence (index relative
  // to it) whose segment the counter showed as written when last read
  // (wave-uniform), so the common case is one compare, not a division per
  // chunk on the scalar unit the CU's waves share.  The counter is polled
  // with device-scope loads before a block is touched.  The wait is bounded
  // (wait_polls polls of ~1 us); a wave that runs out sets the flag word
  // beside the counter and stops waiting for the rest of the launch, so a
  // stalled producer cannot hold the GPU, and the call's recovery launches
  // (guarded by that flag) recompute every result on the caller's stream.
  auto upto_of = [&](int seen) { return (seen + 1) * seg - 1 - c0; };
  int upto = ready ? upto_of(0) : 0x7fffffff;
  bool patient = true;
  auto ensure = [&](int cc) {
    const int need = min(cc, ce - 1);
    if (need <= upto || !patient) return;
    int spin = 0;
    for (; need > upto && spin < wait_polls; ++spin) {
      upto = upto_of(
          __builtin_amdgcn_readfirstlane(__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
      if (need > upto) __builtin_amdgcn_s_sleep(8);
    }
    if (need > upto) {
      patient = false;
      if (lane == 0) __hip_atomic_store(ready + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // Single-slot scheme (NBUF = 1): the whole block of chunk cc and its v
  // tile, one chunk ahead.
  auto issue = [&](int cc) {
    ensure(cc);
    const int lw = wave - CW;
    const unsigned char* src = ws + (static_cast<size_t>(c0 + cc) * H + h) * B::bytes;
    for (int j = lw; j < NG; j += kLoaderWaves) lds_load16(src + j * 1024 + lane * 16, smem + j * 1024);
    const int t0 = tbeg + cc * cl, len = min(cl, L_seq - cc * cl);
    for (int j = lw; j < NVG; j += kLoaderWaves) {
      const int r = j * VRPL + lane / VLPR;
      const int rr = r < len ? r : len - 1;  // rows past the end are masked by beta = 0
      const unsigned char* vsrc = reinterpret_cast<const unsigned char*>(
                                      v + (static_cast<size_t>(t0 + rr) * H + h) * DV + tile * TILE) +
                                  (lane % VLPR) * 16;
      lds_load16(vsrc, smem + B::bytes + j * 1024);
    }
  };

  if (loader) {
    if constexpr (SL::NBUF == 2) {
      // Early part of chunk x: issued once chunk x - 2 has passed its first
      // products (barrier M(x - 2)); late part of chunk x: issued at the end
      // of chunk x - 2.  Both are resident by the end of chunk x - 1.
      // Every loader wave moves the same number of granules (the tail
      // granule with Gamma, beta and v granules may be moved twice, with
      // identical bytes), so one vmcnt bound serves every wait; chunks past
      // the end re-load the last chunk into an idle slot.
      constexpr int EG = static_cast<int>(B::oK / 1024);          // early granules
      constexpr int LG = static_cast<int>((B::oG - B::oK) / 1024);  // late granules before the tail
      static_assert(B::oK % 1024 == 0 && B::oG % 1024 == 0 && EG % kLoaderWaves == 0 && LG % kLoaderWaves == 0 &&
                        B::bytes - B::oG == 1024,
                    "block granules");
      constexpr int NVW = (NVG + kLoaderWaves - 1) / kLoaderWaves;
      constexpr int NE = EG / kLoaderWaves, NLT = LG / kLoaderWaves + 1 + NVW;
      const int lw = wave - CW;
      if (cb >= ce) {  // empty sequence: the compute waves only pass the first barrier
        lds_barrier();
        return;
      }
      auto blk_base = [&](int cc) { return ws + (static_cast<size_t>(c0 + min(cc, ce - 1)) * H + h) * B::bytes; };
      auto blk_src = [&](int cc) { return blk_base(cc) + lane * 16; };
      // L2 prefetch of a chunk's block two chunks before its first loads: the
      // value tiles of a (sequence, head) share their XCD's L2, so tile t
      // touches a quarter of the block's 128-byte lines, one 4-byte
      // direct-to-LDS load per lane into a sink nobody reads.
      constexpr int LINES = static_cast<int>(B::bytes / 128);
      constexpr int LPT = (LINES + NSPLIT - 1) / NSPLIT;                       // lines per tile
      constexpr int NPF = (LPT + 64 * kLoaderWaves - 1) / (64 * kLoaderWaves);  // loads per loader wave
      // lanes of a loader wave's first prefetch that touch block lines; when
      // there is room, the lanes after them touch C / kLoaderWaves rows of
      // the chunk's v tile (read from the input, so not in L2 otherwise)
      constexpr int LPW = (LPT + kLoaderWaves - 1) / kLoaderWaves;
      constexpr bool PFV = NPF == 1 && LPW + C / kLoaderWaves <= 64;
      auto prefetch = [&](int cc) {
        // A block not written yet must not be touched (its lines would be
        // cached stale): then the last chunk of the newest written segment
        // is touched instead, so every call issues exactly NPF loads and the
        // loader's vmcnt bounds hold.
        if (cc > upto) cc = upto;
        const unsigned char* base = blk_base(cc);
        if constexpr (PFV) {
          const unsigned char* src;
          if (lane < LPW) {
            src = base + min(tile * LPT + min(lw + kLoaderWaves * lane, LPT - 1), LINES - 1) * 128;
          } else {
            const int cx = min(cc, ce - 1);
            const int len = min(cl, L_seq - cx * cl);
            const int r = min(lw * (C / kLoaderWaves) + min(lane - LPW, C / kLoaderWaves - 1), len - 1);
            src = reinterpret_cast<const unsigned char*>(v + (static_cast<size_t>(tbeg + cx * cl + r) * H + h) * DV +
                                                         tile * TILE);
          }
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                           (__attribute__((address_space(3))) void*)(smem + SL::pfsink), 4, 0, 0);
        } else {
#pragma unroll
          for (int m = 0; m < NPF; ++m) {
            const int line = min(tile * LPT + min((lw + kLoaderWaves * m) * 64 + lane, LPT - 1), LINES - 1);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + line * 128),
                                             (__attribute__((address_space(3))) void*)(smem + SL::pfsink), 4, 0, 0);
          }
        }
      };
      auto early = [&](int cc, int slot) {
        const unsigned char* src = blk_src(cc);
        unsigned char* dst = smem + slot * SL::early;
#pragma unroll
        for (int m = 0; m < NE; ++m) lds_load16(src + (lw + kLoaderWaves * m) * 1024, dst + (lw + kLoaderWaves * m) * 1024);
      };
      auto late = [&](int cc, int slot) {
        const unsigned char* src = blk_src(cc) + B::oK;
        unsigned char* dst = smem + SL::late0 + slot * SL::late;
#pragma unroll
        for (int m = 0; m < LG / kLoaderWaves; ++m)
          lds_load16(src + (lw + kLoaderWaves * m) * 1024, dst + (lw + kLoaderWaves * m) * 1024);
        lds_load16(src + (B::oG - B::oK), dst + (B::oG - B::oK));
        cc = min(cc, ce - 1);
        const int t0 = tbeg + cc * cl, len = min(cl, L_seq - cc * cl);
#pragma unroll
        for (int m = 0; m < NVW; ++m) {
          const int j = (lw + kLoaderWaves * m) % NVG;
          const int rr = min(j * VRPL + lane / VLPR, len - 1);  // rows past the end are masked by beta = 0
          lds_load16(reinterpret_cast<const unsigned char*>(
                         v + (static_cast<size_t>(t0 + rr) * H + h) * DV + tile * TILE) +
                         (lane % VLPR) * 16,
                     dst + (B::bytes - B::oK) + j * 1024);
        }
      };
      // Output rows of chunk cc (staged in LDS by the compute waves before
      // the end-of-chunk barrier): each wave stores NSW 16-byte row pieces
      // per lane, through a buffer resource spanning the chunk's valid rows.
      constexpr int LPR = static_cast<int>(SL::orow / 16), RPI = 64 / LPR, NSI = C / RPI;
      constexpr int NSW = SL::stage_o ? (NSI + kLoaderWaves - 1) / kLoaderWaves : 0;
      static_assert(!SL::stage_o || (SL::orow % 16 == 0 && 64 % LPR == 0 && C % RPI == 0), "output tile geometry");
      auto ostore = [&](int cc) {
        if constexpr (SL::stage_o) {
          const int len = cc < cb ? 0 : min(cl, L_seq - cc * cl);  // nothing before the first chunk
          const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
              o + (static_cast<size_t>(tbeg + max(cc, 0) * cl) * H + h) * DV + tile * TILE, 0,
              len * H * DV * static_cast<int>(sizeof(T)), 0x00020000);
#pragma unroll
          for (int m = 0; m < NSW; ++m) {
            const int row = ((lw + kLoaderWaves * m) % NSI) * RPI + lane / LPR, cb16 = (lane % LPR) * 16;
            const u32x4 x = *reinterpret_cast<const u32x4*>(smem + SL::ostage + row * SL::orow + cb16);
            __builtin_amdgcn_raw_buffer_store_b128(x, ro, row * H * DV * static_cast<int>(sizeof(T)) + cb16, 0, 0);
          }
        }
      };
      ensure(cb + 1);
      early(cb, 0);
      late(cb, 0);
      early(cb + 1, 1);
      prefetch(cb + 2);
      wait_vm<NE + NPF>();  // chunk cb resident (early and late parts)
      lds_barrier();
      for (int cc = cb; cc < ce; ++cc) {
        const int b = (cc - cb) & 1;
        ensure(cc + 1);
        late(cc + 1, b ^ 1);
        if constexpr (SL::split) {
          // With split roles the output wave stages chunk cc - 1's tile
          // between the end of that chunk and M(cc), so it is stored after M.
          // In flight, oldest first: early part of chunk cc + 1, the
          // previous prefetch, late part of cc + 1.
          wait_vm<NPF + NLT>();  // early part of chunk cc + 1 resident
          lds_barrier();  // M(cc): early slot b free; the state waves read chunk cc + 1's R rows from here on
          ostore(cc - 1);
          ensure(cc + 2);
          early(cc + 2, b);
          prefetch(cc + 4);
          wait_vm<NSW + NE + NPF>();  // all but the stores, chunk cc + 2's early part and the prefetch
        } else {
          ostore(cc - 1);
          // in flight, oldest first: early part of chunk cc + 1, the previous
          // prefetch, late part of cc + 1, output stores of cc - 1
          wait_vm<NPF + NLT + NSW>();  // early part of chunk cc + 1 resident
          lds_barrier();  // M(cc): early slot b free; the state waves read chunk cc + 1's R rows from here on
          ensure(cc + 2);
          early(cc + 2, b);
          prefetch(cc + 4);
          wait_vm<NE + NPF>();  // all but the early part of chunk cc + 2 and the prefetch: chunk cc + 1 resident
        }
        lds_barrier();  // end of chunk cc
      }
      if constexpr (SL::split) lds_barrier();  // F: the last chunk's output tile staged
      ostore(ce - 1);
      return;
    }
    if (cb < ce) issue(cb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int cc = cb; cc < ce; ++cc) {
      __syncthreads();  // chunk cc consumed
      if (cc + 1 < ce) {
        issue(cc + 1);
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();  // chunk cc + 1 resident
    }
    return;
  }

  // Compute waves: 16 value columns per column group; every compute wave
  // keeps the group's dk x 16 state slice in MFMA accumulators.  With split
  // roles, wave cg (< WAVES) is the group's state wave and wave WAVES + cg
  // its output wave; otherwise one wave does both.
  const int n = lane & 15, g = lane >> 4;
  const int role = SL::split ? wave / WAVES : 0;
  const int cg = SL::split ? wave % WAVES : wave;
  const bool do_state = role == 0;
  const int col = tile * TILE + cg * 16 + n;
  f32x4 S[ST];
  const size_t sbase = (static_cast<size_t>(seq) * H + h) * DK * DV;
  if (s_in && do_state) {
#pragma unroll
    for (int st = 0; st < ST; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[st][i] = s_in[sbase + static_cast<size_t>(16 * st + 4 * g + i) * DV + col];
  } else {
#pragma unroll
    for (int st = 0; st < ST; ++st) S[st] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Output tiles are stored after a quad transpose: lane (n, g) writes row
  // 16 mt + 4 g + (n & 3), columns (n & ~3) .. (n & ~3) + 3 of its 16.  Byte
  // offsets from the chunk's first row; the host keeps C H DV sizeof(T) < 2^31.
  int ooff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    ooff[mt] = ((16 * mt + 4 * g + (n & 3)) * H * DV + col - (n & 3)) * static_cast<int>(sizeof(T));
  if constexpr (SL::split) {
    if (role == 0 && lane == 0) reinterpret_cast<int*>(smem + SL::xflag)[cg] = 0;  // D hand-over counter
  }
  if constexpr (SL::NBUF == 2) lds_barrier(); else __syncthreads();  // first chunk resident

  // Output tile of a chunk: staged row-major in LDS for the loader waves, or
  // transposed within lane quads (four consecutive columns of one row per
  // lane) and stored directly through a buffer resource spanning the chunk's
  // valid rows (rows past the end are dropped by the hardware range check).
  auto put_o = [&](const f32x4 (&O)[MT], int t0, int len) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (SL::stage_o) {
        unsigned char* dst = smem + SL::ostage + (16 * mt + 4 * g) * SL::orow + (cg * 16 + n) * sizeof(T);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_put1(dst + i * SL::orow, O[mt][i], static_cast<T*>(nullptr));
      } else {
        const f32x4 x = quad_transpose(O[mt], n & 3);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            o + (static_cast<size_t>(t0) * H + h) * DV, 0, len * H * DV * static_cast<int>(sizeof(T)), 0x00020000);
        buffer_store4(ro, ooff[mt], x, static_cast<T*>(nullptr));
      }
    }
  };
  // Per-chunk pieces.  View of chunk cc: early part (R, Qh) and late part
  // (from Kb^T on, then the v tile); lat(off) addresses block offset
  // off >= oK in the late slot.
  auto eblk_of = [&](int cc) { return smem + ((SL::NBUF == 2) ? ((cc - cb) & 1) : 0) * SL::early; };
  auto lblk_of = [&](int cc) { return smem + SL::late0 + ((SL::NBUF == 2) ? ((cc - cb) & 1) : 0) * SL::late; };
  // rows of a stored tile times the state fragments: A[mt] = X[rows of mt] sb
  auto rows_x_state = [&](const RowFrags<T, B::RB_R, NSK> (&fr)[MT], const F (&sb)[NSK], f32x4 (&A)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NSK; ++s) a = M::mma(fr[mt].f[s], sb[s], a);
      A[mt] = a;
    }
  };
  // Late-part inputs of D: beta v (this lane's accumulator positions) and
  // the row fragments of T.
  struct DIn {
    f32x4 bv[MT];
    TriFrags<T, C, NSC> tf[MT];
  };
  auto load_din = [&](const unsigned char* lblk, DIn& in) {
    const T* vt = reinterpret_cast<const T*>(lblk + (B::bytes - B::oK));
    const float* Bet = reinterpret_cast<const float*>(lblk + (B::oB - B::oK));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 bt = *reinterpret_cast<const f32x4*>(Bet + 16 * mt + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) in.bv[mt][i] = bt[i] * io<T>::load(vt + (16 * mt + 4 * g + i) * TILE + cg * 16 + n);
      in.tf[mt].load(lblk + (B::oT - B::oK), mt, n, g);
    }
  };
  // Y = b V - R S; D = T Y with Y split into hi + lo (T unit lower
  // triangular); D split into hi + lo
  auto make_d = [&](const DIn& in, f32x4 (&Y)[MT], F (&dh)[NSC], F (&dl)[NSC]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) Y[mt] = in.bv[mt] - Y[mt];
    F yh[NSC], yl[NSC];
#pragma unroll
    for (int s = 0; s < NSC; ++s) SP::hilo(Y, s, yh[s], yl[s]);
    const TriFrags<T, C, NSC>(&tf)[MT] = in.tf;
    f32x4 D[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= (16 * mt + 15) / AB::KS; ++s) {
        acc = M::mma(tf[mt].f[s], yh[s], acc);
        if (SP::has_lo) acc = M::mma(tf[mt].f[s], yl[s], acc);
      }
      D[mt] = acc;
    }
#pragma unroll
    for (int s = 0; s < NSC; ++s) SP::hilo(D, s, dh[s], dl[s]);
  };
  // O += P D (D as hi + lo)
  auto add_pd = [&](const TriFrags<T, C, NSC> (&pf)[MT], const F (&dh)[NSC], const F (&dl)[NSC],
                    f32x4 (&O)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s <= (16 * mt + 15) / AB::KS; ++s) {
        O[mt] = M::mma(pf[mt].f[s], dh[s], O[mt]);
        if (SP::has_lo) O[mt] = M::mma(pf[mt].f[s], dl[s], O[mt]);
      }
  };
  // S = Diag(e^{g_last}) S + Kb^T D (D's hi part)
  auto update_s = [&](const unsigned char* lblk, const RowFrags<T, B::RB_K, NSC> (&kf)[ST], const F (&dh)[NSC]) {
    const float* Gam = reinterpret_cast<const float*>(lblk + (B::oG - B::oK));
#pragma unroll
    for (int st = 0; st < ST; ++st) S[st] *= *reinterpret_cast<const f32x4*>(Gam + 16 * st + 4 * g);
#pragma unroll
    for (int st = 0; st < ST; ++st)
#pragma unroll
      for (int s = 0; s < NSC; ++s) S[st] = M::mma(kf[st].f[s], dh[s], S[st]);
  };
  auto chunk_end = [&]() {
    if constexpr (SL::NBUF == 2) {
      lds_barrier();  // end of chunk: late slot free; early part of the next chunk resident
    } else {
      __syncthreads();  // chunk consumed
      __syncthreads();  // next chunk resident
    }
  };

  if constexpr (SL::split) {
    static_assert(SL::NBUF == 2, "split roles come with the staged output, which needs two slots");
    // D (hi, lo) and the state fragments pass from state to output wave here
    F* const dxp = reinterpret_cast<F*>(smem + SL::dx + cg * SL::dx_group) + lane;
    F* const sxp = dxp + 64 * C / static_cast<int>(sizeof(F));
    int* const xfl = reinterpret_cast<int*>(smem + SL::xflag) + cg;
    if (do_state) {
      // R rows of the first chunk; the rows of chunk cc + 1 are read during
      // chunk cc, after M (the loaders have its early part resident by
      // then), so the next chunk's products start at once
      RowFrags<T, B::RB_R, NSK> fr[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) fr[mt].load(eblk_of(cb) + B::oR, 16 * mt + n, g);
      for (int cc = cb; cc < ce; ++cc) {
        const unsigned char* lblk = lblk_of(cc);
        DIn din;
        load_din(lblk, din);
        // Kb^T rows for the state update, read now so their latency hides
        // under R S and D
        RowFrags<T, B::RB_K, NSC> kf[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st) kf[st].load(lblk, 16 * st + n, g);
        F sb[NSK];
#pragma unroll
        for (int s = 0; s < NSK; ++s) {
          sb[s] = AB::b(S, s);
          sxp[64 * s] = sb[s];
        }
        f32x4 Y[MT];
        rows_x_state(fr, sb, Y);
        lds_barrier();  // M: early slot consumed; state fragments in LDS
        // next chunk's R rows (resident from M on; past the last chunk: a
        // slot no load is filling, values unused), read before D is formed
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) fr[mt].load(eblk_of(cc + 1) + B::oR, 16 * mt + n, g);
        F dh[NSC], dl[NSC];
        make_d(din, Y, dh, dl);
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
          dxp[64 * s] = dh[s];
          if (SP::has_lo) dxp[64 * (NSC + s)] = dl[s];
        }
        // hand D over: the counter is raised once this wave's D writes are done
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0
        if (lane == 0) __hip_atomic_store(xfl, cc - cb + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        update_s(lblk, kf, dh);
        chunk_end();
      }
      if (s_out) {
#pragma unroll
        for (int st = 0; st < ST; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) s_out[sbase + static_cast<size_t>(16 * st + 4 * g + i) * DV + col] = S[st][i];
      }
      if (ce > cb) lds_barrier();  // F (see the output wave)
    } else {
      // Chunk cc's P D and its output tile are finished at the start of
      // chunk cc + 1 (before M), off the path from the state wave's D to the
      // end-of-chunk barrier: O, the P fragments and D are carried across
      // the barrier in registers (the late slot holding P is refilled after
      // it), and the loader waves store the staged tile after M.
      f32x4 O[MT];
      TriFrags<T, C, NSC> pf[MT];
      F dh[NSC], dl[NSC];
      for (int cc = cb; cc < ce; ++cc) {
        const unsigned char* eblk = eblk_of(cc);
        const unsigned char* lblk = lblk_of(cc);
        if (cc > cb) {
          add_pd(pf, dh, dl, O);
          put_o(O, 0, 0);  // staged in LDS (split roles come with the staged output)
        }
        RowFrags<T, B::RB_R, NSK> fr[MT];  // Qh rows: the early slot is refilled after M
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) fr[mt].load(eblk + B::oQ, 16 * mt + n, g);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) pf[mt].load(lblk + (B::oP - B::oK), mt, n, g);
        lds_barrier();  // M
        F sb[NSK];
#pragma unroll
        for (int s = 0; s < NSK; ++s) sb[s] = sxp[64 * s];
        rows_x_state(fr, sb, O);
        // wait for the state wave's D of this chunk (bounded: the state wave
        // raises the counter without waiting on this wave)
        for (int spin = 0; spin < (1 << 26); ++spin) {
          if (__hip_atomic_load(xfl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) > cc - cb) break;
          __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
          dh[s] = dxp[64 * s];
          if (SP::has_lo) dl[s] = dxp[64 * (NSC + s)];
        }
        chunk_end();
      }
      if (ce > cb) {
        add_pd(pf, dh, dl, O);
        put_o(O, 0, 0);
        lds_barrier();  // F: the last output tile staged for the loader waves
      }
    }
  } else {
    for (int cc = cb; cc < ce; ++cc) {
      const unsigned char* eblk = eblk_of(cc);
      const unsigned char* lblk = lblk_of(cc);
      const int t0 = tbeg + cc * cl, len = min(cl, L_seq - cc * cl);
      // B fragments of the state (shared by R S and Qh S)
      F sb[NSK];
#pragma unroll
      for (int s = 0; s < NSK; ++s) sb[s] = AB::b(S, s);
      // Y = R S and O = Qh S together: 2 MT independent accumulator chains
      f32x4 Y[MT], O[MT];
      {
        RowFrags<T, B::RB_R, NSK> rc, qc, rn, qn;
        rc.load(eblk + B::oR, n, g);
        qc.load(eblk + B::oQ, n, g);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt + 1 < MT) {
            rn.load(eblk + B::oR, 16 * (mt + 1) + n, g);
            qn.load(eblk + B::oQ, 16 * (mt + 1) + n, g);
          }
          f32x4 ay = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NSK; ++s) {
            ay = M::mma(rc.f[s], sb[s], ay);
            ao = M::mma(qc.f[s], sb[s], ao);
          }
          Y[mt] = ay;
          O[mt] = ao;
          if (mt + 1 < MT) {
            rc = rn;
            qc = qn;
          }
        }
      }
      if constexpr (SL::NBUF == 2) lds_barrier();  // M: early slot consumed
      DIn din;
      load_din(lblk, din);
      F dh[NSC], dl[NSC];
      make_d(din, Y, dh, dl);
      TriFrags<T, C, NSC> pf[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) pf[mt].load(lblk + (B::oP - B::oK), mt, n, g);
      RowFrags<T, B::RB_K, NSC> kf[ST];
#pragma unroll
      for (int st = 0; st < ST; ++st) kf[st].load(lblk, 16 * st + n, g);
      add_pd(pf, dh, dl, O);
      update_s(lblk, kf, dh);
      put_o(O, t0, len);
      chunk_end();
    }
    if (s_out) {
#pragma unroll
      for (int st = 0; st < ST; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_out[sbase + static_cast<size_t>(16 * st + 4 * g + i) * DV + col] = S[st][i];
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: plan and launch.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Raise a kernel's dynamic LDS limit once per (kernel, device): the call is
// slow enough on the host to open gaps between the launches of one call.
static hipError_t set_lds_limit(const void* fn, size_t bytes) {
  constexpr int kMaxDev = 64, kMaxFn = 64;
  static std::mutex mu;
  static const void* done[kMaxDev][kMaxFn] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const bool cached = dev >= 0 && dev < kMaxDev;
  if (cached) {
    for (int i = 0; i < kMaxFn && done[dev][i]; ++i)
      if (done[dev][i] == fn) return hipSuccess;
  }
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e == hipSuccess && cached) {
    for (int i = 0; i < kMaxFn; ++i)
      if (!done[dev][i]) {
        done[dev][i] = fn;
        break;
      }
  }
  return e;
}


// Scan workgroups of the narrow (32-column) configuration.
static int64_t narrow_scan_wgs(int64_t N, int64_t H, int dv) { return (N * H + 7) / 8 * 8 * (dv / 32); }

// Overlapped schedule: when the scan has at most this many workgroups (one per
// CU) it runs on half of the CUs while the prep of the next segment runs on
// the other half.
constexpr int64_t kPipeMaxScanWgs = 128;
constexpr int64_t kPipeMinSeg = 64;    // chunks per segment, at least
constexpr int64_t kPipeMaxSegs = 16;   // segments, at most (each adds a prep launch beside the scan)

static size_t block_bytes(kda_dtype dt, int C, int dk) {
  const size_t es = dt == KDA_BF16 ? 2 : 4;
  // P and T: rows 0..31 at half width when C = 64 (see Blk)
  const size_t tri = (C == 64 ? static_cast<size_t>(32) * (C / 2) + static_cast<size_t>(C - 32) * C
                              : static_cast<size_t>(C) * C) * es;
  const size_t b = static_cast<size_t>(C) * dk * es * 3 + tri * 2 + dk * 4 + C * 4;
  return (b + 1023) / 1024 * 1024;
}

bool make_prefill_plan(const kda_prefill_desc* d, int64_t max_chunks, PrefillPlan* p) {
  p->N = d->num_seqs;
  p->T = d->total_tokens;
  p->H = d->num_heads;
  p->dk = d->dk;
  p->dv = d->dv;
  // chunks of 16 tokens run through the 32-row kernels (rows 16..31 stay
  // empty, as in a partial last chunk)
  p->C = d->chunk < 32 ? 32 : d->chunk;
  p->CL = d->chunk;
  p->dt = d->io_dtype;
  p->gate = d->gate;
  const kda_stages* sg = d->stages;
  p->l2norm_qk = sg && sg->l2norm_qk ? 1 : 0;
  p->l2norm_eps = sg ? sg->l2norm_eps : 0.f;
  p->gate_softplus = sg && sg->gate_softplus && d->gate != KDA_GATE_NONE ? 1 : 0;
  p->norm_weight = sg ? sg->norm_weight : nullptr;
  p->norm_eps = sg ? sg->norm_eps : 0.f;
  p->out_gate = sg ? sg->out_gate : nullptr;
  p->max_chunks = max_chunks;
  p->sort = d->num_seqs <= 8192;
  const size_t slots = static_cast<size_t>(max_chunks) * d->num_heads;
  size_t off = 0;
  p->off_chunk_off = off; off = align256(off + 4 * (static_cast<size_t>(d->num_seqs) + 1));
  p->off_order = off;     off = align256(off + 4 * (static_cast<size_t>(d->num_seqs) + 1));
  off = (off + 1023) / 1024 * 1024;
  p->off_blocks = off;    off += slots * block_bytes(d->io_dtype, p->C, d->dk);
  off = align256(off);
  p->seg = 0;
  p->off_ready = 0;
  p->off_carry = 0;
  if (!(d->flags & (KDA_PREFILL_ONE_STREAM | KDA_PREFILL_BOUNDED)) && narrow_scan_wgs(d->num_seqs, d->num_heads, d->dv) <= kPipeMaxScanWgs &&
      max_chunks >= 2 * kPipeMinSeg) {
    const int64_t seg = (max_chunks + kPipeMaxSegs - 1) / kPipeMaxSegs;
    p->seg = seg > kPipeMinSeg ? seg : kPipeMinSeg;
    p->off_ready = off;
    off += 256;
    // final states of an in-place call, held until the call knows it needs
    // no recovery
    p->off_carry = off;
    off = align256(off + static_cast<size_t>(d->num_seqs) * d->num_heads * d->dk * d->dv * 4);
  }
  p->total_bytes = align256(off);
  p->bseg = 0;
  p->off_bcarry = 0;
  p->rseg = 0;
  p->rslots = 0;
  return true;
}

bool make_bounded_plan(const kda_prefill_desc* d, int64_t max_chunks, size_t workspace_bytes, bool carry_in_ws,
                       PrefillPlan* p) {
  kda_prefill_desc one = *d;
  one.flags |= KDA_PREFILL_ONE_STREAM;
  if (!make_prefill_plan(&one, max_chunks, p)) return false;
  const size_t chunk_bytes = static_cast<size_t>(d->num_heads) * block_bytes(d->io_dtype, p->C, d->dk);
  const size_t carry =
      carry_in_ws ? align256(static_cast<size_t>(d->num_seqs) * d->num_heads * d->dk * d->dv * 4) : 0;
  if (max_chunks < 1) return true;  // nothing to segment: the one-stream plan
  if (workspace_bytes < p->off_blocks + carry + chunk_bytes) return false;
  int64_t seg = static_cast<int64_t>((workspace_bytes - p->off_blocks - carry) / chunk_bytes);
  if (seg > max_chunks) seg = max_chunks;
  p->bseg = seg;
  // Few (sequence, head) pairs: a ring of segments of the overlapped
  // schedule's length, when at least two fit (see launch_prefill_t)
  if (!(d->flags & KDA_PREFILL_ONE_STREAM) && narrow_scan_wgs(d->num_seqs, d->num_heads, d->dv) <= kPipeMaxScanWgs &&
      max_chunks >= 2 * kPipeMinSeg) {
    int64_t rseg = (max_chunks + kPipeMaxSegs - 1) / kPipeMaxSegs;
    if (rseg < kPipeMinSeg) rseg = kPipeMinSeg;
    const int64_t nseg = (max_chunks + rseg - 1) / rseg;
    const int64_t slots = seg / rseg < nseg ? seg / rseg : nseg;
    if (slots >= 2) {
      p->rseg = rseg;
      p->rslots = slots;
    }
  }
  // the block area ends on a 1024-byte boundary (off_blocks and chunk_bytes are multiples)
  const size_t end = p->off_blocks + static_cast<size_t>(seg) * chunk_bytes;
  p->off_bcarry = carry ? end : 0;
  p->total_bytes = end + carry;
  return true;
}

size_t bounded_min_bytes(const kda_prefill_desc* d, int64_t max_chunks) {
  PrefillPlan p;
  kda_prefill_desc one = *d;
  one.flags |= KDA_PREFILL_ONE_STREAM;
  if (!make_prefill_plan(&one, max_chunks, &p)) return 0;
  if (max_chunks < 1) return p.total_bytes;
  return p.off_blocks + static_cast<size_t>(d->num_heads) * block_bytes(d->io_dtype, p.C, d->dk) +
         align256(static_cast<size_t>(d->num_seqs) * d->num_heads * d->dk * d->dv * 4);
}

// Polls (each about a microsecond) a scan loader wave of the overlapped
// schedule waits for a prepared segment before it gives up; a test hook
// can lower it.
constexpr int kDefaultWaitPolls = 1 << 17;
static std::atomic<int> g_wait_polls{kDefaultWaitPolls};
static int prefill_wait_polls() { return g_wait_polls.load(std::memory_order_relaxed); }

int set_prefill_wait_polls(int polls) {
  return g_wait_polls.exchange(polls > 0 ? polls : (polls == 0 ? 0 : kDefaultWaitPolls));
}

template <typename T, int C, int DK, int DV, int WAVES, bool SEG = false>
static hipError_t launch_scan(const PrefillPlan& p, const void* v, const int32_t* cu, const int32_t* chunk_off,
                              const int32_t* order, const unsigned char* blocks, const float* S0, void* o,
                              float* S_T, hipStream_t st, int* ready = nullptr, int seg = 1,
                              const int* guard = nullptr, float* carry = nullptr, int64_t gb = 0,
                              int64_t ge = 0) {
  typedef ScanLds<T, C, DK, 16 * WAVES> SL;
  static_assert(SL::total <= 160 * 1024, "scan LDS");
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&scan_kernel<T, C, DK, DV, WAVES, SEG>), SL::total);
  if (e != hipSuccess) return e;
  const int pairs = p.N * p.H;
  const int nsplit = DV / (16 * WAVES);
  const unsigned grid = static_cast<unsigned>((pairs + 7) / 8 * 8 * nsplit);
  hipLaunchKernelGGL((scan_kernel<T, C, DK, DV, WAVES, SEG>), dim3(grid), dim3(scan_threads<T, C, DK, WAVES>()), SL::total, st,
                     static_cast<const T*>(v), cu, chunk_off, order, p.N, p.H, blocks, S0, static_cast<T*>(o), S_T,
                     ready, seg, prefill_wait_polls(), guard, p.CL, carry, static_cast<int>(gb),
                     static_cast<int>(ge));
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus) {
  static int cache[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *cus = cache[dev];
    return hipSuccess;
  }
  int n = 0;
  if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *cus = n;
  return hipSuccess;
}

// Per-device pair of CU-masked streams (default priority) and the events of
// the overlapped schedule; created on first use and destroyed at process
// exit (from an atexit handler, registered after the HIP runtime has
// started, so it runs while the runtime and any tool attached to it are
// still alive).
struct PipeStreams {
  hipStream_t prep = nullptr, scan = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, join_prep = nullptr;
  // ring schedule: segment j prepared / passed over by the state pass
  hipEvent_t prepped[kPipeMaxSegs] = {}, scanned[kPipeMaxSegs] = {};
  int scan_cus = 0;
  std::mutex mu;  // one schedule at a time may use the shared streams/events
};

constexpr int kMaxDev = 64;
static std::mutex g_pipe_mu;
static PipeStreams* g_pipe[kMaxDev] = {};
static bool g_pipe_unavailable[kMaxDev] = {};

static void destroy_pipe(PipeStreams* ps) {
  if (ps->scan) (void)hipStreamDestroy(ps->scan);
  if (ps->prep) (void)hipStreamDestroy(ps->prep);
  if (ps->fork) (void)hipEventDestroy(ps->fork);
  if (ps->join) (void)hipEventDestroy(ps->join);
  if (ps->join_prep) (void)hipEventDestroy(ps->join_prep);
  for (int i = 0; i < kPipeMaxSegs; ++i) {
    if (ps->prepped[i]) (void)hipEventDestroy(ps->prepped[i]);
    if (ps->scanned[i]) (void)hipEventDestroy(ps->scanned[i]);
  }
  delete ps;
}

static void release_pipe_streams() {
  std::lock_guard<std::mutex> lock(g_pipe_mu);
  for (int dev = 0; dev < kMaxDev; ++dev) {
    if (!g_pipe[dev]) continue;
    if (hipSetDevice(dev) == hipSuccess) {
      (void)hipStreamSynchronize(g_pipe[dev]->scan);
      (void)hipStreamSynchronize(g_pipe[dev]->prep);
      destroy_pipe(g_pipe[dev]);
    }
    g_pipe[dev] = nullptr;
  }
  (void)hipGetLastError();
}

// Returns in *out the current device's streams when the scan (scan_wgs
// workgroups) fits on its half of the CUs, else nullptr.
static hipError_t pipe_streams(int64_t scan_wgs, PipeStreams** out) {
  static bool registered = false;
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_pipe_mu);
  if (!g_pipe[dev] && !g_pipe_unavailable[dev]) {
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess) return e;
    const int cus = prop.multiProcessorCount, words = (cus + 31) / 32;
    // Runs of 8 consecutive mask bits alternate between the two streams.  The
    // runtime deals mask bit i to XCD i mod 8, so each stream gets half of the
    // CUs of every XCD and the scan keeps its XCD-aware placement.
    std::vector<uint32_t> ms(words, 0u), mp(words, 0u);
    int ns = 0, np = 0;
    for (int i = 0; i < cus; ++i) {
      std::vector<uint32_t>& m = ((i >> 3) & 1) ? mp : ms;
      m[i >> 5] |= 1u << (i & 31);
      ++(((i >> 3) & 1) ? np : ns);
    }
    PipeStreams* ps = new PipeStreams;
    bool ok = ns >= 8 && np >= 8 &&
              hipExtStreamCreateWithCUMask(&ps->scan, words, ms.data()) == hipSuccess &&
              hipExtStreamCreateWithCUMask(&ps->prep, words, mp.data()) == hipSuccess &&
              hipEventCreateWithFlags(&ps->fork, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&ps->join, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&ps->join_prep, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; ok && i < kPipeMaxSegs; ++i)
      ok = hipEventCreateWithFlags(&ps->prepped[i], hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&ps->scanned[i], hipEventDisableTiming) == hipSuccess;
    if (ok) {
      ps->scan_cus = ns;
      g_pipe[dev] = ps;
      if (!registered) registered = std::atexit(release_pipe_streams) == 0;
    } else {  // no CU masks here: fall back to the single-stream schedule
      destroy_pipe(ps);
      (void)hipGetLastError();
      g_pipe_unavailable[dev] = true;
    }
  }
  if (g_pipe[dev] && scan_wgs <= g_pipe[dev]->scan_cus) *out = g_pipe[dev];
  return hipSuccess;
}

template <typename T, int C, int DK, int DV, int G, bool IN>
static hipError_t launch_prefill_t(const PrefillPlan& p, const void* q, const void* k, const void* v,
                                   const float* la, const float* beta, const int32_t* cu, const float* S0,
                                   void* o, float* S_T, void* ws, hipStream_t st) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(w + p.off_chunk_off);
  int32_t* order = reinterpret_cast<int32_t*>(w + p.off_order);
  unsigned char* blocks = w + p.off_blocks;
  if (p.N == 0) return hipSuccess;
  int32_t* ready = p.seg > 0 ? reinterpret_cast<int32_t*>(w + p.off_ready) : nullptr;
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, st, cu, p.N, p.CL, chunk_off, order, p.sort, ready);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lp = PrepLds<T, C, DK>::total;
  static_assert(PrepLds<T, C, DK>::total <= 160 * 1024, "prep LDS");
  // Persistent prep: as many workgroups as fit on the CUs the stream may
  // use (LDS-limited), each walking (chunk, head) items.
  auto prep = [&](int64_t cbase, int64_t count, hipStream_t s, int cus, int32_t* publish, int published,
                  const int* guard, unsigned char* blks) -> hipError_t {
    hipError_t r = set_lds_limit(reinterpret_cast<const void*>(&prep_kernel<T, C, DK, G, IN>), lp);
    if (r != hipSuccess) return r;
    const int64_t per_cu = (160 * 1024) / static_cast<int64_t>(lp) > 0 ? (160 * 1024) / static_cast<int64_t>(lp) : 1;
    const int64_t items = count * p.H;
    const int64_t grid = items < per_cu * cus ? items : per_cu * cus;
    hipLaunchKernelGGL((prep_kernel<T, C, DK, G, IN>), dim3(static_cast<unsigned>(grid)), dim3(kPrepThreads), lp, s,
                       static_cast<const T*>(q), static_cast<const T*>(k), la, beta, cu, chunk_off, p.N, p.H,
                       blks, static_cast<int>(cbase), static_cast<int>(count), publish, published, guard, p.CL,
                       p.l2norm_qk, p.l2norm_eps, p.gate_softplus);
    return hipGetLastError();
  };
  int cus = 0;
  if ((e = device_cus(&cus)) != hipSuccess) return e;
  // Overlapped schedule: one scan launch (half of the CUs) walks every
  // chunk while the prep of segments 1, 2, ... runs beside it (the other
  // half); the ready counter that the scan's loader waves wait on is
  // raised to j - 1 by the first thread of segment j's prep launch and to
  // the last segment by a ready_kernel; both streams fork from and join
  // back into the caller's stream.  Segment 0's prep has the whole device.
  // If a loader wave stops waiting (the device did not run the two streams
  // side by side), the flag word ready[1] is set and the two guarded
  // recovery launches at the end recompute every result on the caller's
  // stream; otherwise they return at once.
  PipeStreams* ps = nullptr;
  if (p.seg > 0) {
    e = pipe_streams(narrow_scan_wgs(p.N, p.H, DV), &ps);
    if (e != hipSuccess) return e;
  }
  if (ps) {
    const int64_t nseg = (p.max_chunks + p.seg - 1) / p.seg;
    const bool in_place = S_T != nullptr && S_T == S0;
    float* carry = reinterpret_cast<float*>(w + p.off_carry);
    const int* flag = ready + 1;
    {
      std::lock_guard<std::mutex> lock(ps->mu);
      e = prep(0, p.seg < p.max_chunks ? p.seg : p.max_chunks, st, cus, nullptr, 0, nullptr, blocks);
      if (e != hipSuccess) return e;
      if ((e = hipEventRecord(ps->fork, st)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(ps->prep, ps->fork, 0)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(ps->scan, ps->fork, 0)) != hipSuccess) return e;
      e = launch_scan<T, C, DK, DV, 2>(p, v, cu, chunk_off, order, blocks, S0, o, in_place ? carry : S_T, ps->scan,
                                       ready, static_cast<int>(p.seg));
      if (e != hipSuccess) return e;
      for (int64_t j = 1; j < nseg; ++j) {
        const int64_t c0 = j * p.seg, c1 = c0 + p.seg < p.max_chunks ? c0 + p.seg : p.max_chunks;
        if ((e = prep(c0, c1 - c0, ps->prep, cus - ps->scan_cus, j > 1 ? ready : nullptr, static_cast<int>(j - 1),
                      nullptr, blocks)) != hipSuccess)
          return e;
      }
      hipLaunchKernelGGL(ready_kernel, dim3(1), dim3(64), 0, ps->prep, ready, static_cast<int>(nseg - 1));
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = hipEventRecord(ps->join, ps->scan)) != hipSuccess) return e;
      if ((e = hipEventRecord(ps->join_prep, ps->prep)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(st, ps->join, 0)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(st, ps->join_prep, 0)) != hipSuccess) return e;
    }
    if (in_place) {
      const size_t n4 = static_cast<size_t>(p.N) * p.H * DK * DV / 4;
      const unsigned grid = static_cast<unsigned>(n4 / 256 < 1024 ? (n4 + 255) / 256 : 1024);
      hipLaunchKernelGGL(carry_out_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<const f32x4*>(carry),
                         reinterpret_cast<f32x4*>(S_T), n4, flag);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // recovery (runs only if the flag word is set)
    if ((e = prep(0, p.max_chunks, st, cus, nullptr, 0, flag, blocks)) != hipSuccess) return e;
    return launch_scan<T, C, DK, DV, 2>(p, v, cu, chunk_off, order, blocks, S0, o, S_T, st, nullptr, 1, flag);
  }
  // Few (sequence, head) pairs: narrower value tiles to put more CUs on the
  // serial pass; many pairs: wider tiles to load each chunk block fewer times.
  const long wide_wgs = static_cast<long>(p.N) * p.H * (DV / 64);
  if (p.bseg > 0) {
    // Bounded schedule: segment by segment of global chunk indices, the
    // prep fills the one block area (addressed as if it started at the
    // segment's first chunk) and the state pass resumes every (sequence,
    // head) from the state in `carry`; stream order separates the launches.
    float* carry = p.off_bcarry ? reinterpret_cast<float*>(w + p.off_bcarry) : S_T;
    const size_t chunk_bytes = static_cast<size_t>(p.H) * Blk<T, C, DK>::bytes;
    PipeStreams* ps = nullptr;
    if (p.rslots >= 2) {
      e = pipe_streams(narrow_scan_wgs(p.N, p.H, DV), &ps);
      if (e != hipSuccess) return e;
    }
    if (ps) {
      // Ring: segment j (rseg global chunk indices) is prepared into slot
      // j mod rslots on the prep stream (half of the CUs) once the state
      // pass of segment j - rslots, the slot's previous reader, has ended,
      // and passed over by a state-pass launch of its own on the scan
      // stream (the other half) once its prep has ended.  Every dependency
      // is a stream event: no kernel waits on another.  Segment 0 is
      // prepared on the caller's stream over the whole device first.
      const int64_t nseg = (p.max_chunks + p.rseg - 1) / p.rseg;
      auto ring_blocks = [&](int64_t j) {
        const uintptr_t slot = reinterpret_cast<uintptr_t>(blocks) +
                               static_cast<uintptr_t>(j % p.rslots) * static_cast<uintptr_t>(p.rseg) * chunk_bytes;
        return reinterpret_cast<unsigned char*>(slot - static_cast<uintptr_t>(j * p.rseg) * chunk_bytes);
      };
      std::lock_guard<std::mutex> lock(ps->mu);
      if ((e = prep(0, p.rseg < p.max_chunks ? p.rseg : p.max_chunks, st, cus, nullptr, 0, nullptr,
                    ring_blocks(0))) != hipSuccess)
        return e;
      if ((e = hipEventRecord(ps->fork, st)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(ps->prep, ps->fork, 0)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(ps->scan, ps->fork, 0)) != hipSuccess) return e;
      for (int64_t j = 0; j < nseg; ++j) {
        const int64_t gb = j * p.rseg, ge = gb + p.rseg < p.max_chunks ? gb + p.rseg : p.max_chunks;
        if (j > 0) {
          if (j >= p.rslots && (e = hipStreamWaitEvent(ps->prep, ps->scanned[j - p.rslots], 0)) != hipSuccess)
            return e;
          if ((e = prep(gb, ge - gb, ps->prep, cus - ps->scan_cus, nullptr, 0, nullptr, ring_blocks(j))) !=
              hipSuccess)
            return e;
          if ((e = hipEventRecord(ps->prepped[j], ps->prep)) != hipSuccess) return e;
          if ((e = hipStreamWaitEvent(ps->scan, ps->prepped[j], 0)) != hipSuccess) return e;
        }
        if ((e = launch_scan<T, C, DK, DV, 2, true>(p, v, cu, chunk_off, order, ring_blocks(j), S0, o, S_T, ps->scan,
                                              nullptr, 1, nullptr, carry, gb, ge)) != hipSuccess)
          return e;
        if ((e = hipEventRecord(ps->scanned[j], ps->scan)) != hipSuccess) return e;
      }
      if ((e = hipEventRecord(ps->join, ps->scan)) != hipSuccess) return e;
      if ((e = hipEventRecord(ps->join_prep, ps->prep)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(st, ps->join, 0)) != hipSuccess) return e;
      return hipStreamWaitEvent(st, ps->join_prep, 0);
    }
    for (int64_t gb = 0; gb < p.max_chunks; gb += p.bseg) {
      const int64_t ge = gb + p.bseg < p.max_chunks ? gb + p.bseg : p.max_chunks;
      unsigned char* seg_blocks =
          reinterpret_cast<unsigned char*>(reinterpret_cast<uintptr_t>(blocks) - static_cast<uintptr_t>(gb) * chunk_bytes);
      if ((e = prep(gb, ge - gb, st, cus, nullptr, 0, nullptr, seg_blocks)) != hipSuccess) return e;
      e = wide_wgs < 512 ? launch_scan<T, C, DK, DV, 2, true>(p, v, cu, chunk_off, order, seg_blocks, S0, o, S_T, st,
                                                               nullptr, 1, nullptr, carry, gb, ge)
                         : launch_scan<T, C, DK, DV, 4, true>(p, v, cu, chunk_off, order, seg_blocks, S0, o, S_T, st,
                                                               nullptr, 1, nullptr, carry, gb, ge);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (p.max_chunks > 0) {
    e = prep(0, p.max_chunks, st, cus, nullptr, 0, nullptr, blocks);
    if (e != hipSuccess) return e;
  }
  if (wide_wgs < 512) return launch_scan<T, C, DK, DV, 2>(p, v, cu, chunk_off, order, blocks, S0, o, S_T, st);
  return launch_scan<T, C, DK, DV, 4>(p, v, cu, chunk_off, order, blocks, S0, o, S_T, st);
}

template <typename T, int C, int DK, int DV>
static hipError_t dispatch_gate(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                                void* ws, hipStream_t st) {
  const bool in = p.l2norm_qk || p.gate_softplus;
  if (p.gate == KDA_GATE_CHANNEL)
    return in ? launch_prefill_t<T, C, DK, DV, KDA_GATE_CHANNEL, true>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st)
              : launch_prefill_t<T, C, DK, DV, KDA_GATE_CHANNEL, false>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.gate == KDA_GATE_SCALAR)
    return in ? launch_prefill_t<T, C, DK, DV, KDA_GATE_SCALAR, true>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st)
              : launch_prefill_t<T, C, DK, DV, KDA_GATE_SCALAR, false>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  return in ? launch_prefill_t<T, C, DK, DV, KDA_GATE_NONE, true>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st)
            : launch_prefill_t<T, C, DK, DV, KDA_GATE_NONE, false>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
}

template <typename T, int C>
static hipError_t dispatch_dims(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                                void* ws, hipStream_t st) {
  if (p.dk == 128 && p.dv == 128) return dispatch_gate<T, C, 128, 128>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.dk == 128 && p.dv == 64) return dispatch_gate<T, C, 128, 64>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.dk == 64 && p.dv == 128) return dispatch_gate<T, C, 64, 128>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.dk == 64 && p.dv == 64) return dispatch_gate<T, C, 64, 64>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dispatch_chunk(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                                 const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                                 void* ws, hipStream_t st) {
  if (p.C == 64) return dispatch_dims<T, 64>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.C == 32) return dispatch_dims<T, 32>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_out_stage(const PrefillPlan& p, void* o, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.T) * p.H;
  if (rows == 0) return hipSuccess;
  const int64_t want = (rows + 15) / 16;  // 4 waves of at least 4 rows per workgroup step
  const unsigned grid = static_cast<unsigned>(want < 8192 ? want : 8192);
  if (p.dv == 128)
    hipLaunchKernelGGL((out_stage_kernel<T, 128>), dim3(grid), dim3(256), 0, st, static_cast<T*>(o),
                       static_cast<const T*>(p.out_gate), p.norm_weight, p.norm_eps, rows);
  else
    hipLaunchKernelGGL((out_stage_kernel<T, 64>), dim3(grid), dim3(256), 0, st, static_cast<T*>(o),
                       static_cast<const T*>(p.out_gate), p.norm_weight, p.norm_eps, rows);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                          const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                          void* workspace, hipStream_t stream) {
  const bool bf = p.dt == KDA_BF16;
  hipError_t e = bf ? dispatch_chunk<bf16_t>(p, q, k, v, la, beta, cu, S0, o, S_T, workspace, stream)
                    : dispatch_chunk<float>(p, q, k, v, la, beta, cu, S0, o, S_T, workspace, stream);
  if (e != hipSuccess || (!p.norm_weight && !p.out_gate)) return e;
  return bf ? launch_out_stage<bf16_t>(p, o, stream) : launch_out_stage<float>(p, o, stream);
}

}  // namespace kda
