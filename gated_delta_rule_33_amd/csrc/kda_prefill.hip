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
// Kernels (all on the caller's stream):
//   chunk_offsets_kernel  chunk offsets per sequence + longest-first order
//   prep_kernel           grid (chunk, head): everything that does not depend
//                         on S (gate cumsum, A and P via MFMA, T by blocked
//                         forward substitution, R, Qh, Kb^T, e^{g_last}),
//                         written to the workspace
//   scan_kernel           grid (sequence, head, 64-column value tile): the
//                         serial chunk loop with S held in MFMA accumulators
//
// Exponent safety.  e^{g_r-g_s} is factorised around references inside the
// chunk so that no factor exceeds the fp32 range: for a 16-row block I below
// the diagonal (rows r in I, columns s in J < I) the row side uses
// e^{g_r - g_{b_I}} e^{g_{b_I} - g_{e_J}} and the column side e^{g_{e_J} - g_s}
// (b_I first row of I, e_J last row of J; every factor <= 1).  Diagonal
// blocks use the block's 9th row as reference, so a factor can reach
// e^{8 * max|log_alpha|}; the library requires log_alpha >= -10.

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
// X[row][k] must be read with the same map.
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
  // X row pointer (LDS), k-step s, lane group g
  __device__ __forceinline__ static bf16x8 a(const bf16_t* row, int s, int g) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + 32 * s + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + 32 * s + 16 + 4 * g);
    const uint4 u = {lo.x, lo.y, hi.x, hi.y};
    return __builtin_bit_cast(bf16x8, u);
  }
};

template <>
struct accb<float> {
  static constexpr int KS = 4;
  __device__ __forceinline__ static float b(const f32x4* tiles, int s) { return tiles[s >> 2][s & 3]; }
  __device__ __forceinline__ static float a(const float* row, int s, int g) {
    return row[16 * (s >> 2) + 4 * g + (s & 3)];
  }
};

// ---------------------------------------------------------------------------
// a1: chunk offsets per sequence and the longest-first processing order.
// One workgroup of 1024 threads.  chunk_off[n] = sum_{i<n} ceil(L_i / C).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int32_t* __restrict__ cu, int N, int C,
                                                             int32_t* __restrict__ chunk_off,
                                                             int32_t* __restrict__ order, int sort) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
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

// ---------------------------------------------------------------------------
// Workspace geometry per (chunk, head) slot.
// ---------------------------------------------------------------------------
template <typename T, int C, int DK>
struct WsGeom {
  static constexpr size_t R = static_cast<size_t>(C) * DK;   // elements of R (and Qh, Kb^T)
  static constexpr size_t P = static_cast<size_t>(C) * C;    // elements of P (and T)
};

// ---------------------------------------------------------------------------
// Prep kernel LDS layout.
// ---------------------------------------------------------------------------
template <typename T, int C, int DK>
struct PrepLds {
  static constexpr int NB = C / 16;
  static constexpr int NPAIR = NB * (NB - 1) / 2;
  static constexpr int PADG = 4;                          // fp32 G pitch pad
  static constexpr int PADK = 8;                          // element pad for [C][DK] io arrays (16 B rows for bf16)
  static constexpr int GP = DK + PADG;                    // G pitch (floats)
  static constexpr int KP = DK + PADK;                    // Kr/Qr/Kc pitch (elements)
  static constexpr int AP = C + 1;                        // A / Tinv pitch (floats)
  static constexpr size_t szG = static_cast<size_t>(C) * GP * 4;
  static constexpr size_t szKQ = static_cast<size_t>(2) * C * KP * sizeof(T);
  static constexpr size_t szTi = static_cast<size_t>(C) * AP * 4;
  static constexpr size_t reg0 = (((szG > szKQ ? szG : szKQ) > szTi ? (szG > szKQ ? szG : szKQ) : szTi) + 15) / 16 * 16;
  static constexpr size_t reg1 = (static_cast<size_t>(C) * KP * sizeof(T) + 15) / 16 * 16;  // Kr
  static constexpr size_t szVec = static_cast<size_t>(4 * NB + NPAIR) * DK * 4;   // eb ee dr dc pair
  static constexpr size_t szX = static_cast<size_t>(NB > 1 ? NB - 1 : 1) * 256 * 4;
  static constexpr size_t reg2 = ((szVec > szX ? szVec : szX) + 15) / 16 * 16;
  static constexpr size_t szA = static_cast<size_t>(C) * AP * 4;
  static constexpr size_t szKt = static_cast<size_t>(DK) * (C + PADK) * sizeof(T);
  static constexpr size_t reg3 = ((szA > szKt ? szA : szKt) + 15) / 16 * 16;      // A, earlier Kb^T staging
  static constexpr size_t szBeta = static_cast<size_t>(C) * 4;
  static constexpr size_t szPart = static_cast<size_t>(256 / DK) * DK * 4;
  static constexpr size_t o0 = 0, o1 = reg0, o2 = o1 + reg1, o3 = o2 + reg2, o4 = o3 + reg3,
                          o5 = o4 + szBeta;
  static constexpr size_t total = o5 + szPart;
};

template <typename T, int C, int DK>
__global__ __launch_bounds__(256) void prep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const float* __restrict__ la, const float* __restrict__ beta,
                                                   const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ chunk_off, int N, int H,
                                                   T* __restrict__ wsR, T* __restrict__ wsQ,
                                                   T* __restrict__ wsKt, T* __restrict__ wsP,
                                                   T* __restrict__ wsT, float* __restrict__ wsG) {
  typedef PrepLds<T, C, DK> L;
  typedef mma16<T> M;
  constexpr int NB = L::NB;
  extern __shared__ __align__(16) unsigned char smem[];
  float* G = reinterpret_cast<float*>(smem + L::o0);             // [C][GP]
  T* Kc = reinterpret_cast<T*>(smem + L::o0);                    // [C][KP]  (after G is consumed)
  T* Qr = Kc + C * L::KP;                                        // [C][KP]
  float* Ti = reinterpret_cast<float*>(smem + L::o0);            // [C][AP]  (after Kc/Qr are consumed)
  T* Kr = reinterpret_cast<T*>(smem + L::o1);                    // [C][KP]
  float* vec = reinterpret_cast<float*>(smem + L::o2);           // eb ee dr dc pair, [.][DK]
  float* eb = vec;
  float* ee = vec + NB * DK;
  float* dr = vec + 2 * NB * DK;
  float* dc = vec + 3 * NB * DK;
  float* pr = vec + 4 * NB * DK;
  float* X = vec;                                                // inverse scratch (after vectors)
  float* A = reinterpret_cast<float*>(smem + L::o3);             // [C][AP]
  T* Kts = reinterpret_cast<T*>(smem + L::o3);                   // [DK][C + PADK] staging
  float* bet = reinterpret_cast<float*>(smem + L::o4);           // [C]
  float* part = reinterpret_cast<float*>(smem + L::o5);          // [256/DK][DK]

  const int c = blockIdx.x, h = blockIdx.y;
  const int total = chunk_off[N];
  if (c >= total) return;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
  }
  const int t0 = cu[lo] + (c - chunk_off[lo]) * C;
  const int len = min(C, cu[lo + 1] - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t slot = static_cast<size_t>(c) * H + h;
  const size_t rowstride = static_cast<size_t>(H) * DK;  // elements between tokens in q/k/la

  // ---- a2: chunk-local inclusive cumsum of log_alpha per key channel ------
  {
    constexpr int PARTS = 256 / DK;
    constexpr int RPT = C / PARTS;
    const int ch = tid % DK, pt = tid / DK;
    float gl[RPT];
    float run = 0.f;
    const float* lap = la + (static_cast<size_t>(t0) * H + h) * DK + ch;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = pt * RPT + i;
      run += r < len ? lap[static_cast<size_t>(r) * rowstride] : 0.f;
      gl[i] = run;
    }
    part[pt * DK + ch] = run;
    if (tid < C) bet[tid] = tid < len ? beta[static_cast<size_t>(t0 + tid) * H + h] : 0.f;
    __syncthreads();
    float off = 0.f;
    for (int p = 0; p < pt; ++p) off += part[p * DK + ch];
#pragma unroll
    for (int i = 0; i < RPT; ++i) G[(pt * RPT + i) * L::GP + ch] = gl[i] + off;
    __syncthreads();
  }

  // ---- per-block reference vectors --------------------------------------
  for (int idx = tid; idx < NB * DK; idx += 256) {
    const int I = idx / DK, ch = idx % DK;
    const float gb = G[(16 * I) * L::GP + ch];
    const float gm = G[(16 * I + 8) * L::GP + ch];
    const float ge = G[(16 * I + 15) * L::GP + ch];
    const float gz = G[(C - 1) * L::GP + ch];
    eb[idx] = __expf(gb);         // e^{g_b}:          row-side ref -> chunk start
    ee[idx] = __expf(gz - ge);    // e^{g_last - g_e}: column-side ref -> chunk end
    dr[idx] = __expf(gb - gm);    // diagonal block row-side correction
    dc[idx] = __expf(gm - ge);    // diagonal block column-side correction
  }
  for (int idx = tid; idx < L::NPAIR * DK; idx += 256) {
    const int p = idx / DK, ch = idx % DK;
    int I = 1;
    while ((I + 1) * I / 2 <= p) ++I;
    const int J = p - I * (I - 1) / 2;
    pr[idx] = __expf(G[(16 * I) * L::GP + ch] - G[(16 * J + 15) * L::GP + ch]);
  }
  for (int ch = tid; ch < DK; ch += 256) wsG[slot * DK + ch] = __expf(G[(C - 1) * L::GP + ch]);
  __syncthreads();  // reference vectors visible to every thread

  // ---- element factors and the S-independent outputs ---------------------
  // Each thread owns groups of 4 channels of one row.
  constexpr int NG = C * DK / 4 / 256;  // groups per thread
  f32x4 keepQ[NG], keepK[NG];
  {
    typedef WsGeom<T, C, DK> W;
    T* oR = wsR + slot * W::R;
    T* oQ = wsQ + slot * W::R;
#pragma unroll
    for (int it = 0; it < NG; ++it) {
      const int idx = tid + 256 * it;
      const int r = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
      const int I = r >> 4;
      const f32x4 g = *reinterpret_cast<const f32x4*>(G + r * L::GP + c4);
      const f32x4 gb = *reinterpret_cast<const f32x4*>(G + (16 * I) * L::GP + c4);
      const f32x4 ge = *reinterpret_cast<const f32x4*>(G + (16 * I + 15) * L::GP + c4);
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qq = {0.f, 0.f, 0.f, 0.f};
      if (r < len) {
        kk = load4(k + (static_cast<size_t>(t0 + r) * H + h) * DK + c4);
        qq = load4(q + (static_cast<size_t>(t0 + r) * H + h) * DK + c4);
      }
      f32x4 fr, fc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        fr[j] = __expf(g[j] - gb[j]);
        fc[j] = __expf(ge[j] - g[j]);
      }
      const f32x4 kr = kk * fr;
      const f32x4 qr = qq * fr;
      const f32x4 kc = kk * fc;
      const f32x4 ebv = *reinterpret_cast<const f32x4*>(eb + I * DK + c4);
      const f32x4 eev = *reinterpret_cast<const f32x4*>(ee + I * DK + c4);
      store4(oQ + r * DK + c4, qr * ebv);              // Qh = e^{g_r} q_r
      store4(oR + r * DK + c4, bet[r] * (kr * ebv));   // R  = b_r e^{g_r} k_r
      const f32x4 kb = kc * eev;                       // Kb = e^{g_last - g_r} k_r
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_put<T>(Kts + (c4 + j) * (C + L::PADK) + r, kb[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_put<T>(Kr + r * L::KP + c4 + j, kr[j]);
      keepQ[it] = qr;
      keepK[it] = kc;
    }
  }
  __syncthreads();  // G no longer read; Kb^T staged
  {
    typedef WsGeom<T, C, DK> W;
    T* oK = wsKt + slot * W::R;
#pragma unroll
    for (int it = 0; it < NG; ++it) {
      const int idx = tid + 256 * it;
      const int r = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lds_put<T>(Qr + r * L::KP + c4 + j, keepQ[it][j]);
        lds_put<T>(Kc + r * L::KP + c4 + j, keepK[it][j]);
      }
      // Kb^T rows are [DK][C]: element (row ch, col rr)
      const int ch = idx / (C / 4), r4 = (idx % (C / 4)) * 4;
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = lds_get<T>(Kts + ch * (C + L::PADK) + r4 + j);
      store4(oK + ch * C + r4, x);
    }
  }
  __syncthreads();  // Kr, Qr, Kc ready; Kb^T staging free for A

  // ---- a3: gated k k^T (A) and q k^T (P), 16x16 blocks via MFMA ----------
  {
    typedef WsGeom<T, C, DK> W;
    T* oP = wsP + slot * W::P;
    const int n = lane & 15, g = lane >> 4;
    for (int blk = wave; blk < NB * NB; blk += 4) {
      const int I = blk / NB, J = blk % NB;
      f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
      if (J <= I) {
        const float* rs = (I == J) ? dr + I * DK : pr + (I * (I - 1) / 2 + J) * DK;
        const T* krow = Kr + (16 * I + n) * L::KP;
        const T* qrow = Qr + (16 * I + n) * L::KP;
        const T* crow = Kc + (16 * J + n) * L::KP;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += M::KS) {
          typename M::frag bf;
          if (I == J) bf = frag_nat(crow, dc + I * DK, k0, g);
          else bf = frag_nat(crow, k0, g);
          const typename M::frag ak = frag_nat(krow, rs, k0, g);
          const typename M::frag aq = frag_nat(qrow, rs, k0, g);
          aA = M::mma(ak, bf, aA);
          aP = M::mma(aq, bf, aP);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * g + i;
        const int row = 16 * I + rr, col = 16 * J + n;
        float a = aA[i] * bet[row];
        float p = aP[i];
        if (J > I || (I == J && rr <= n)) a = 0.f;
        if (J > I || (I == J && rr < n)) p = 0.f;
        A[row * L::AP + col] = a;
        io<T>::store(oP + row * C + col, p);
      }
    }
  }
  __syncthreads();

  // ---- a4: T = (I + A)^{-1} by blocked forward substitution --------------
  // Diagonal 16x16 blocks: lane j of wave I solves column j.
  for (int I = wave; I < NB; I += 4) {
    if (lane < 16) {
      const int j = lane;
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == j) ? 1.f : 0.f;
        const float* arow = A + (16 * I + r) * L::AP + 16 * I;
#pragma unroll
        for (int s = 0; s < r; ++s) acc -= arow[s] * t[s];
        t[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Ti[(16 * I + r) * L::AP + 16 * I + j] = t[r];
    }
  }
  // zero the strictly upper blocks
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, cc = idx % C;
    if ((cc >> 4) > (r >> 4)) Ti[r * L::AP + cc] = 0.f;
  }
  __syncthreads();
  // Off-diagonal blocks by distance d: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ.
  for (int d = 1; d < NB; ++d) {
    const int nblk = NB - d;
    const int i = tid >> 4, jj = tid & 15;
    for (int b = 0; b < nblk; ++b) {
      const int J = b, I = b + d;
      float x = 0.f;
      for (int K = J; K < I; ++K) {
        const float* arow = A + (16 * I + i) * L::AP + 16 * K;
        const float* tcol = Ti + (16 * K) * L::AP + 16 * J + jj;
#pragma unroll
        for (int s = 0; s < 16; ++s) x += arow[s] * tcol[s * L::AP];
      }
      X[b * 256 + i * 16 + jj] = x;
    }
    __syncthreads();
    for (int b = 0; b < nblk; ++b) {
      const int J = b, I = b + d;
      const float* trow = Ti + (16 * I + i) * L::AP + 16 * I;
      float y = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) y += trow[m] * X[b * 256 + m * 16 + jj];
      Ti[(16 * I + i) * L::AP + 16 * J + jj] = -y;
    }
    __syncthreads();
  }

  // ---- write T -----------------------------------------------------------
  {
    typedef WsGeom<T, C, DK> W;
    T* oT = wsT + slot * W::P;
    for (int idx = tid; idx < C * C / 4; idx += 256) {
      const int r = idx / (C / 4), c4 = (idx % (C / 4)) * 4;
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = Ti[r * L::AP + c4 + j];
      store4(oT + r * C + c4, x);
    }
  }
}

// ---------------------------------------------------------------------------
// Scan kernel: one workgroup per (sequence, head, 64-column value tile); four
// waves, each owning 16 value columns.  The state tile lives in MFMA
// accumulators (DK/16 tiles of 16x16 fp32 per wave) for the whole sequence.
// ---------------------------------------------------------------------------
template <typename T, int C, int DK>
struct ScanLds {
  static constexpr int PAD = 8;
  static constexpr int RP = DK + PAD;  // pitch of R and Qh rows
  static constexpr int CP = C + PAD;   // pitch of Kb^T, P and T rows
  static constexpr size_t oR = 0;
  static constexpr size_t oQ = oR + static_cast<size_t>(C) * RP * sizeof(T);
  static constexpr size_t oK = oQ + static_cast<size_t>(C) * RP * sizeof(T);
  static constexpr size_t oP = oK + static_cast<size_t>(DK) * CP * sizeof(T);
  static constexpr size_t oT = oP + static_cast<size_t>(C) * CP * sizeof(T);
  static constexpr size_t oG = oT + static_cast<size_t>(C) * CP * sizeof(T);
  static constexpr size_t oB = oG + static_cast<size_t>(DK) * 4;
  static constexpr size_t total = oB + static_cast<size_t>(C) * 4;
};

// Copy `rows` rows of `cols` io elements (contiguous in global) into LDS with
// pitch `pitch`, 16 bytes per lane.
template <typename T>
__device__ __forceinline__ void copy_rows(T* dst, int pitch, const T* src, int rows, int cols, int tid) {
  constexpr int E = 16 / sizeof(T);
  const int per_row = cols / E;
  for (int idx = tid; idx < rows * per_row; idx += 256) {
    const int r = idx / per_row, c = (idx % per_row) * E;
    *reinterpret_cast<uint4*>(dst + r * pitch + c) = *reinterpret_cast<const uint4*>(src + r * cols + c);
  }
}

template <typename T, int C, int DK, int DV>
__global__ __launch_bounds__(256) void scan_kernel(const T* __restrict__ v, const float* __restrict__ beta,
                                                   const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ chunk_off,
                                                   const int32_t* __restrict__ order, int N, int H,
                                                   const T* __restrict__ wsR, const T* __restrict__ wsQ,
                                                   const T* __restrict__ wsKt, const T* __restrict__ wsP,
                                                   const T* __restrict__ wsT, const float* __restrict__ wsG,
                                                   const float* S0, T* __restrict__ o, float* S_T) {
  typedef ScanLds<T, C, DK> L;
  typedef mma16<T> M;
  typedef accb<T> AB;
  typedef WsGeom<T, C, DK> W;
  constexpr int NSPLIT = DV / 64;
  constexpr int MT = C / 16;   // chunk-row tiles
  constexpr int ST = DK / 16;  // state row tiles
  extern __shared__ __align__(16) unsigned char smem[];
  T* Rs = reinterpret_cast<T*>(smem + L::oR);
  T* Qs = reinterpret_cast<T*>(smem + L::oQ);
  T* Ks = reinterpret_cast<T*>(smem + L::oK);
  T* Ps = reinterpret_cast<T*>(smem + L::oP);
  T* Ts = reinterpret_cast<T*>(smem + L::oT);
  float* Gs = reinterpret_cast<float*>(smem + L::oG);
  float* Bs = reinterpret_cast<float*>(smem + L::oB);

  // blockIdx -> (pair, tile) with all tiles of a pair on one XCD (x % 8).
  const int x = blockIdx.x;
  const int xcd = x & 7, slot8 = x >> 3;
  const int tile = slot8 % NSPLIT, grp = slot8 / NSPLIT;
  const int p = grp * 8 + xcd;
  if (p >= N * H) return;
  const int seq = order[p / H];
  const int h = p % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int col = tile * 64 + wave * 16 + n;  // this lane's value column
  const int tbeg = cu[seq], L_seq = cu[seq + 1] - tbeg;
  const int c0 = chunk_off[seq];
  const int nch = (L_seq + C - 1) / C;

  f32x4 S[ST];
  const size_t sbase = (static_cast<size_t>(seq) * H + h) * DK * DV;
#pragma unroll
  for (int st = 0; st < ST; ++st)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[st][i] = S0 ? S0[sbase + static_cast<size_t>(16 * st + 4 * g + i) * DV + col] : 0.f;

  for (int cc = 0; cc < nch; ++cc) {
    const size_t wslot = static_cast<size_t>(c0 + cc) * H + h;
    const int t0 = tbeg + cc * C;
    const int len = min(C, L_seq - cc * C);
    __syncthreads();
    copy_rows<T>(Rs, L::RP, wsR + wslot * W::R, C, DK, tid);
    copy_rows<T>(Qs, L::RP, wsQ + wslot * W::R, C, DK, tid);
    copy_rows<T>(Ks, L::CP, wsKt + wslot * W::R, DK, C, tid);
    copy_rows<T>(Ps, L::CP, wsP + wslot * W::P, C, C, tid);
    copy_rows<T>(Ts, L::CP, wsT + wslot * W::P, C, C, tid);
    for (int i = tid; i < DK; i += 256) Gs[i] = wsG[wslot * DK + i];
    if (tid < C) Bs[tid] = tid < len ? beta[static_cast<size_t>(t0 + tid) * H + h] : 0.f;
    __syncthreads();

    // Y = b*V - R S
    f32x4 Y[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const T* arow = Rs + (16 * mt + n) * L::RP;
#pragma unroll
      for (int s = 0; s < DK / AB::KS; ++s) acc = M::mma(AB::a(arow, s, g), AB::b(S, s), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * g + i;
        const float vv = row < len ? io<T>::load(v + (static_cast<size_t>(t0 + row) * H + h) * DV + col) : 0.f;
        Y[mt][i] = Bs[row] * vv - acc[i];
      }
    }
    // D = T Y   (T unit lower triangular: k-steps past the diagonal are zero)
    f32x4 D[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const T* arow = Ts + (16 * mt + n) * L::CP;
#pragma unroll
      for (int s = 0; s <= (16 * mt + 15) / AB::KS; ++s) acc = M::mma(AB::a(arow, s, g), AB::b(Y, s), acc);
      D[mt] = acc;
    }
    // O = Qh S + P D
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const T* qrow = Qs + (16 * mt + n) * L::RP;
#pragma unroll
      for (int s = 0; s < DK / AB::KS; ++s) acc = M::mma(AB::a(qrow, s, g), AB::b(S, s), acc);
      const T* prow = Ps + (16 * mt + n) * L::CP;
#pragma unroll
      for (int s = 0; s <= (16 * mt + 15) / AB::KS; ++s) acc = M::mma(AB::a(prow, s, g), AB::b(D, s), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * g + i;
        if (row < len) io<T>::store(o + (static_cast<size_t>(t0 + row) * H + h) * DV + col, acc[i]);
      }
    }
    // S = Diag(e^{g_last}) S + Kb^T D
#pragma unroll
    for (int st = 0; st < ST; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[st][i] *= Gs[16 * st + 4 * g + i];
      const T* krow = Ks + (16 * st + n) * L::CP;
#pragma unroll
      for (int s = 0; s < C / AB::KS; ++s) S[st] = M::mma(AB::a(krow, s, g), AB::b(D, s), S[st]);
    }
  }
  if (S_T) {
#pragma unroll
    for (int st = 0; st < ST; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) S_T[sbase + static_cast<size_t>(16 * st + 4 * g + i) * DV + col] = S[st][i];
  }
}

// ---------------------------------------------------------------------------
// Host side: plan and launch.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool make_prefill_plan(const kda_prefill_desc* d, int64_t max_chunks, PrefillPlan* p) {
  p->N = d->num_seqs;
  p->T = d->total_tokens;
  p->H = d->num_heads;
  p->dk = d->dk;
  p->dv = d->dv;
  p->C = d->chunk;
  p->dt = d->io_dtype;
  p->max_chunks = max_chunks;
  p->sort = d->num_seqs <= 8192;
  const size_t es = d->io_dtype == KDA_BF16 ? 2 : 4;
  const size_t slots = static_cast<size_t>(max_chunks) * d->num_heads;
  size_t off = 0;
  p->off_chunk_off = off; off = align256(off + 4 * (static_cast<size_t>(d->num_seqs) + 1));
  p->off_order = off;     off = align256(off + 4 * (static_cast<size_t>(d->num_seqs) + 1));
  p->off_R = off;  off = align256(off + slots * d->chunk * d->dk * es);
  p->off_Q = off;  off = align256(off + slots * d->chunk * d->dk * es);
  p->off_Kt = off; off = align256(off + slots * d->chunk * d->dk * es);
  p->off_P = off;  off = align256(off + slots * d->chunk * d->chunk * es);
  p->off_T = off;  off = align256(off + slots * d->chunk * d->chunk * es);
  p->off_G = off;  off = align256(off + slots * d->dk * 4);
  p->total_bytes = off;
  return true;
}

template <typename T, int C, int DK, int DV>
static hipError_t launch_prefill_t(const PrefillPlan& p, const void* q, const void* k, const void* v,
                                   const float* la, const float* beta, const int32_t* cu, const float* S0,
                                   void* o, float* S_T, void* ws, hipStream_t st) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(w + p.off_chunk_off);
  int32_t* order = reinterpret_cast<int32_t*>(w + p.off_order);
  T* R = reinterpret_cast<T*>(w + p.off_R);
  T* Q = reinterpret_cast<T*>(w + p.off_Q);
  T* Kt = reinterpret_cast<T*>(w + p.off_Kt);
  T* P = reinterpret_cast<T*>(w + p.off_P);
  T* Tm = reinterpret_cast<T*>(w + p.off_T);
  float* Gm = reinterpret_cast<float*>(w + p.off_G);
  if (p.N == 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, st, cu, p.N, C, chunk_off, order, p.sort);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.max_chunks > 0) {
    const size_t lp = PrepLds<T, C, DK>::total;
    static_assert(PrepLds<T, C, DK>::total <= 160 * 1024, "prep LDS");
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<T, C, DK>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lp));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prep_kernel<T, C, DK>), dim3(static_cast<unsigned>(p.max_chunks), p.H), dim3(256), lp, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), la, beta, cu, chunk_off, p.N, p.H, R, Q,
                       Kt, P, Tm, Gm);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t ls = ScanLds<T, C, DK>::total;
  static_assert(ScanLds<T, C, DK>::total <= 160 * 1024, "scan LDS");
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_kernel<T, C, DK, DV>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(ls));
  if (e != hipSuccess) return e;
  const int pairs = p.N * p.H;
  const int nsplit = DV / 64;
  const unsigned grid = static_cast<unsigned>((pairs + 7) / 8 * 8 * nsplit);
  hipLaunchKernelGGL((scan_kernel<T, C, DK, DV>), dim3(grid), dim3(256), ls, st, static_cast<const T*>(v), beta, cu,
                     chunk_off, order, p.N, p.H, R, Q, Kt, P, Tm, Gm, S0, static_cast<T*>(o), S_T);
  return hipGetLastError();
}

template <typename T, int C>
static hipError_t dispatch_dims(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                                void* ws, hipStream_t st) {
  if (p.dk == 128 && p.dv == 128) return launch_prefill_t<T, C, 128, 128>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.dk == 128 && p.dv == 64) return launch_prefill_t<T, C, 128, 64>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.dk == 64 && p.dv == 128) return launch_prefill_t<T, C, 64, 128>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
  if (p.dk == 64 && p.dv == 64) return launch_prefill_t<T, C, 64, 64>(p, q, k, v, la, beta, cu, S0, o, S_T, ws, st);
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

hipError_t launch_prefill(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                          const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                          void* workspace, hipStream_t stream) {
  if (p.dt == KDA_BF16)
    return dispatch_chunk<bf16_t>(p, q, k, v, la, beta, cu, S0, o, S_T, workspace, stream);
  return dispatch_chunk<float>(p, q, k, v, la, beta, cu, S0, o, S_T, workspace, stream);
}

}  // namespace kda
