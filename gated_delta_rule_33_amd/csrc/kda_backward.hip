// kda_backward.hip -- chunkwise backward pass of the KDA prefill (gfx950).
//
// The model of the "Kimi Linear" deep-read report (zako-mio knowledge base)
// is trained (section 3.4, training recipe); the pages give the forward
// recurrence (section 2.3: S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
// + beta_t k_t v_t^T, o_t = S_t^T q_t) and its chunked form (section 3.1:
// WY / UT representation, sequential state passing between chunks) but no
// gradient.  This file computes the gradient of
//   L = sum_t <dO_t, o_t> + <dS_T, S_T>
// with respect to q, k, v, log alpha, beta and S0 through the same chunked
// form.  Per chunk of C = 64 tokens (chunk-local cumulative gate G_r =
// sum_{u <= r} log alpha_u, per key channel; gamma = e^{G_C}):
//
//   forward   Kg = k e^{G}, Qg = q e^{G}, Kb = k e^{G_C - G}
//             A[r][s] = sum_i k_ri k_si e^{G_ri - G_si}  (s < r)
//             P[r][s] = sum_i q_ri k_si e^{G_ri - G_si}  (s <= r)
//             T = (I + Diag(beta) A)^{-1}
//             W = Diag(beta)(V - Kg S0), U = T W
//             O = Qg S0 + P U,  S_C = Diag(gamma) S0 + Kb^T U
//   backward  dU = P^T dO + Kb dS_C,  dW = T^T dU,  dV = Diag(beta) dW
//             dS0 = Diag(gamma) dS_C + Qg^T dO - Kg^T dV
//             dbeta_r = <dW_r, (V - Kg S0)_r> + sum_s dM[r][s] A[r][s],
//             dM = -dW U^T (s < r),  dA = Diag(beta) dM,  dP = dO U^T (s <= r)
//             dQg = dO S0^T, dKg = -dV S0^T, dKb = U dS_C^T,
//             dgamma_i = sum_j S0[i][j] dS_C[i][j]
//   and the gated pair sums give dq, dk and dG (hence dlog alpha, a
//   reverse running sum of dG inside the chunk).
//
// Kernels, in stream order:
//   prep      (chunk, head) parallel: G, Kg, Kb, Qg, A, P, T, gamma -> block
//   state     sequential over chunks per (sequence, head, 16 value columns):
//             the chunk-entry states S_c
//   dstate    sequential in reverse: the cotangents dS of every chunk's
//             final state, and dS0
//   grad_v    (chunk, head) parallel over value columns: dv, dbeta and the
//             value-side cotangents dQg, dKg, dKb, dP, dA, dgamma (written
//             over the chunk's block)
//   grad_k    (chunk, head, 16 key channels) parallel: the gated pair sums,
//             dq, dk and dlog alpha
//
// Exactness of the gates.  Every factor e^{G_r - G_s} (s <= r) is at most 1.
// For a pair of 16-row blocks I > J the factor is split at a reference row
// between them (e^{G_r - G_ref} e^{G_ref - G_s}, both <= 1), so an underflow
// only ever stands for a negligible product; inside a diagonal 16 x 16 block
// each pair's factor is formed directly.  No range condition on log alpha.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "kda_device.h"
#include <algorithm>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int BC = 64;   // tokens per chunk
constexpr int P20 = 20;  // LDS pitch (floats) of 16-column tiles
constexpr int LPC = BC + 4;  // LDS pitch of chunk x chunk matrices
// Largest decay (natural log) across a 16-row block for which the prep forms
// the block's own gated products from operands scaled at the row before it:
// the column factor e^{G_ref - G_s} then stays below e^{59.6} < 2^86.
constexpr float kBwdDiagRange = 59.6f;

__device__ __forceinline__ f32x4 mf(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier for LDS hand-overs: waits for this wave's LDS traffic
// only (lgkmcnt 0), not for its global loads and stores, so loads issued
// ahead (the next chunk's operands) stay in flight across it.  Every
// exchange between waves in this file goes through LDS; global results are
// only read by later kernels.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-(chunk, head) block (offsets in floats).  The factors the products
// read are split-bf16 planes (below): an R x K plane takes R K floats'
// bytes, in 16 x 32 fragment tiles, so a wave reads an MFMA fragment as two
// contiguous kilobytes with no conversion.  Each factor is stored in the orientation its consumers
// read it in ("T" planes are transposed: KbT[i][r] = Kb[r][i], PT[s][r] =
// P[r][s]).  A, gamma and beta are fp32.
template <int DK>
struct BwdBlk {
  static constexpr size_t CD = static_cast<size_t>(BC) * DK;
  static constexpr size_t oKg = 0;              // [BC][DK]  k e^{G}
  static constexpr size_t oKb = oKg + CD;       // [BC][DK]  k e^{G_C - G}
  static constexpr size_t oKbT = oKb + CD;      // [DK][BC]
  static constexpr size_t oKgT = oKbT + CD;     // [DK][BC]
  static constexpr size_t oQgT = oKgT + CD;     // [DK][BC]  (q e^{G})^T
  static constexpr size_t oT = oQgT + CD;       // [BC][BC]  lower, unit diagonal
  static constexpr size_t oTT = oT + BC * BC;   // [BC][BC]  T^T
  static constexpr size_t oPT = oTT + BC * BC;  // [BC][BC]  P^T (P lower incl. diagonal)
  static constexpr size_t oA = oPT + BC * BC;   // [BC][BC]  strictly lower
  static constexpr size_t oGam = oA + BC * BC;  // [DK]
  static constexpr size_t oBeta = oGam + DK;    // [BC] (0 past the sequence)
  static constexpr size_t floats = (oBeta + BC + 63) / 64 * 64;
  // the value-side cotangents grad_v writes over the block it has read
  static constexpr size_t odQg = oKg, odKg = oKb, odKb = oKbT, odP = oT, odA = oA, odGam = oGam;
};

size_t blk_floats(int dk) { return dk == 128 ? BwdBlk<128>::floats : BwdBlk<64>::floats; }

// ---------------------------------------------------------------------------
// Split-bf16 products.  An fp32 operand x is carried as hi = bf16(x) and
// lo = bf16(x - hi) (hi + lo = x to ~2^-17 relative); a product of two such
// operands is formed by three bf16 MFMAs (lo*hi + hi*lo + hi*hi, the small
// terms first), dropping lo*lo: ~2^-16 relative per product, at 16,384 flops
// per 16x16x32 instruction against 2,048 for the fp32 16x16x4 MFMA.
// Fragments use the natural k map: lane (row or column l % 16, group
// g = l / 16) holds k = 8 g .. 8 g + 7 of the 32-wide k step.
// ---------------------------------------------------------------------------
struct F3 {
  bf16x8 h, l;
};
__device__ __forceinline__ F3 split8(f32x4 a, f32x4 b, float scale = 1.f) {
  F3 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = a[i] * scale, y = b[i] * scale;
    f.h[i] = static_cast<__bf16>(x);
    f.h[4 + i] = static_cast<__bf16>(y);
    f.l[i] = static_cast<__bf16>(x - static_cast<float>(f.h[i]));
    f.l[4 + i] = static_cast<__bf16>(y - static_cast<float>(f.h[4 + i]));
  }
  return f;
}
// eight consecutive floats (16-byte aligned) from LDS or global memory
__device__ __forceinline__ F3 split8(const float* p, float scale = 1.f) {
  return split8(*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4), scale);
}
__device__ __forceinline__ f32x4 mm3(const F3& a, const F3& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.l, b.h, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.l, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.h, c, 0, 0, 0);
}

// Split-bf16 plane of R x K (R a multiple of 16, K of 32), stored as
// fragment tiles: tile (row / 16, k / 32) is 1,024 bf16, the 16 x 32 hi
// values then the lo values, each in fragment order (eight consecutive k of
// one row at (((k / 8) % 4) * 16 + row % 16) * 8).  A wave's fragment read
// (lane = row % 16 + 16 ((k / 8) % 4)) is then one contiguous kilobyte per
// half.  k0 below is a multiple of 8.
__device__ __forceinline__ size_t ptile(int K, int row, int k0) {
  return static_cast<size_t>((row >> 4) * (K >> 5) + (k0 >> 5)) * 1024 + (((k0 >> 3) & 3) * 16 + (row & 15)) * 8;
}
__device__ __forceinline__ F3 pfrag(const float* plane, int K, int row, int k0) {
  const __bf16* p = reinterpret_cast<const __bf16*>(plane) + ptile(K, row, k0);
  return F3{*reinterpret_cast<const bf16x8*>(p), *reinterpret_cast<const bf16x8*>(p + 512)};
}
// hi part only (planes read only as single bf16)
__device__ __forceinline__ void pstore8_hi(float* plane, int K, int row, int k0, const float* x) {
  bf16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = static_cast<__bf16>(x[i]);
  *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(plane) + ptile(K, row, k0)) = h;
}

// The two chain passes with bf16 io read the block factors as single bf16
// (their hi planes) and form each product from the hi part of the factor
// and both parts of the value handed along the chain: two MFMAs instead of
// three and half the bytes per chunk, which is what bounds these passes;
// fp32 io keeps both parts of both.
template <bool HI>
__device__ __forceinline__ F3 pfragx(const float* plane, int K, int row, int k0) {
  const __bf16* p = reinterpret_cast<const __bf16*>(plane) + ptile(K, row, k0);
  if constexpr (HI) return F3{*reinterpret_cast<const bf16x8*>(p), bf16x8{}};
  else return F3{*reinterpret_cast<const bf16x8*>(p), *reinterpret_cast<const bf16x8*>(p + 512)};
}
template <bool HI>
__device__ __forceinline__ f32x4 mmx(const F3& a, const F3& b, f32x4 c) {
  if constexpr (HI) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.l, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.h, c, 0, 0, 0);
  } else {
    return mm3(a, b, c);
  }
}
__device__ __forceinline__ void pstore8(float* plane, int K, int row, int k0, const float* x) {
  F3 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f.h[i] = static_cast<__bf16>(x[i]);
    f.l[i] = static_cast<__bf16>(x[i] - static_cast<float>(f.h[i]));
  }
  __bf16* p = reinterpret_cast<__bf16*>(plane) + ptile(K, row, k0);
  *reinterpret_cast<bf16x8*>(p) = f.h;
  *reinterpret_cast<bf16x8*>(p + 512) = f.l;
}

// One io element kept as loaded (bf16 bits or fp32) until it is used, so a
// load issued ahead is not waited for at the load.
template <typename T>
struct raw1;
template <>
struct raw1<float> {
  typedef float type;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float cvt(float x) { return x; }
};
template <>
struct raw1<bf16_t> {
  typedef uint32_t type;
  __device__ __forceinline__ static uint32_t load(const bf16_t* p) { return p->bits; }
  __device__ __forceinline__ static float cvt(uint32_t b) { return __uint_as_float(b << 16); }
};

// (sequence, chunk, token range) of global chunk j (chunk_off non-decreasing,
// chunk_off[N] > j).
struct ChunkLoc {
  int n, t0, len;
};
__device__ __forceinline__ ChunkLoc locate(const int32_t* cu, const int32_t* chunk_off, int N, int j) {
  int lo = 0, hi = N;  // chunk_off[lo] <= j < chunk_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_off[mid] <= j) lo = mid;
    else hi = mid;
  }
  const int t0 = cu[lo] + (j - chunk_off[lo]) * BC;
  return ChunkLoc{lo, t0, min(BC, cu[lo + 1] - t0)};
}

// Eight consecutive io elements as floats, and back.
__device__ __forceinline__ void load8(const float* p, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = a[i], x[4 + i] = b[i];
}
__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) x[2 * i] = __uint_as_float(w[i] << 16), x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
}
__device__ __forceinline__ void store8(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void store8(bf16_t* p, const float* x) {
  *reinterpret_cast<uint4*>(p) = uint4{f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3]),
                                       f32x2_to_bf16x2(x[4], x[5]), f32x2_to_bf16x2(x[6], x[7])};
}

// N (4 or 8) consecutive elements as floats, and back.
template <int N, typename E>
__device__ __forceinline__ void loadn(const E* p, float* x) {
  if constexpr (N == 8) {
    load8(p, x);
  } else {
    const f32x4 a = load4(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = a[i];
  }
}
template <int N, typename E>
__device__ __forceinline__ void storen(E* p, const float* x) {
  if constexpr (N == 8) store8(p, x);
  else store4(p, f32x4{x[0], x[1], x[2], x[3]});
}

// log alpha of token t, head h, channel ch for the three gate forms.
template <int G, int DK>
__device__ __forceinline__ float gate_at(const float* la, size_t t, int H, int h, int ch) {
  if constexpr (G == KDA_GATE_CHANNEL) return la[(t * H + h) * DK + ch];
  else if constexpr (G == KDA_GATE_SCALAR) return la[t * H + h];
  else return 0.f;
}

// Inclusive running sum over the 64 rows of an NCH-channel slice in LDS
// (pitch PS), forward (REV = false) or from the last row back (REV = true).
// 256 threads: thread (channel t % NCH, segment t / NCH) owns 64 NCH / 256
// consecutive rows.
template <bool REV, int PS, int NCH = 32>
__device__ __forceinline__ void row_scan(float* x, float* tot /* [256 / NCH][NCH] */) {
  constexpr int SEG = 256 / NCH, RPS = BC / SEG;
  const int ch = threadIdx.x % NCH, seg = threadIdx.x / NCH;
  float v[RPS];
#pragma unroll
  for (int i = 0; i < RPS; ++i) v[i] = x[(seg * RPS + i) * PS + ch];
  if constexpr (!REV) {
#pragma unroll
    for (int i = 1; i < RPS; ++i) v[i] += v[i - 1];
    tot[seg * NCH + ch] = v[RPS - 1];
  } else {
#pragma unroll
    for (int i = RPS - 2; i >= 0; --i) v[i] += v[i + 1];
    tot[seg * NCH + ch] = v[0];
  }
  lds_sync();
  float off = 0.f;
  if constexpr (!REV) {
    for (int s = 0; s < seg; ++s) off += tot[s * NCH + ch];
  } else {
    for (int s = seg + 1; s < SEG; ++s) off += tot[s * NCH + ch];
  }
#pragma unroll
  for (int i = 0; i < RPS; ++i) x[(seg * RPS + i) * PS + ch] = v[i] + off;
  lds_sync();
}


// ---------------------------------------------------------------------------
// prep: one workgroup (4 waves) per (chunk, head); grid (chunks, H).  The key
// channels are taken 32 at a time; A and P accumulate over the slices in
// MFMA tiles: wave w holds the diagonal block pair (w, w) and up to two
// off-diagonal pairs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int off_pair_i(int w, int u) {
  return u == 0 ? (w == 0 ? 1 : (w == 3 ? 3 : 2)) : (w == 0 ? 3 : (w == 1 ? 3 : -1));
}
__device__ __forceinline__ int off_pair_j(int w, int u) {
  return u == 0 ? (w == 2 ? 1 : (w == 3 ? 2 : 0)) : (w == 0 ? 0 : 1);
}

template <typename T, int DK, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_prep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const float* __restrict__ la, const float* __restrict__ beta,
                                                       const int32_t* __restrict__ cu,
                                                       const int32_t* __restrict__ chunk_off, int N, int H,
                                                       float* __restrict__ blk) {
  typedef BwdBlk<DK> B;
  constexpr int PS = 33;  // pitch of the 32-channel slices
  __shared__ float qs[BC * PS], ks[BC * PS], gs[BC * PS];
  __shared__ float Lm[BC * LPC], Tm[BC * LPC];
  __shared__ float Xs[4][16 * 17];
  __shared__ float tot[8 * 32];
  __shared__ float bet[BC];
  const int j = blockIdx.x, h = blockIdx.y;
  if (j >= chunk_off[N]) return;
  const ChunkLoc cl = locate(cu, chunk_off, N, j);
  float* bk = blk + (static_cast<size_t>(j) * H + h) * B::floats;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  if (tid < BC) {
    const float b = tid < cl.len ? beta[static_cast<size_t>(cl.t0 + tid) * H + h] : 0.f;
    bet[tid] = b;
    bk[B::oBeta + tid] = b;
  }
  f32x4 aD = zero4(), pD = zero4(), aO[2] = {zero4(), zero4()}, pO[2] = {zero4(), zero4()};
  // A slice's q, k (raw, thread (row, 4 channels), two rows each) and gates
  // (thread (channel, 8 rows)), read one slice ahead so the loads of slice
  // sl + 1 are in flight while slice sl computes; rows past the sequence
  // read its last row and are zeroed when written to LDS.
  typedef typename raw4<T>::type R4;
  struct SliceIn {
    R4 q[2], k[2];
    float gt[8];
  };
  const int gch = tid & 31, gseg = tid >> 5;
  auto issue = [&](int sl, SliceIn& in) {
    const int c0 = sl * 32;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u, row = min(e >> 3, cl.len - 1), c4 = (e & 7) * 4;
      const size_t o = (static_cast<size_t>(cl.t0 + row) * H + h) * DK + c0 + c4;
      in.q[u] = load4raw(q + o);
      in.k[u] = load4raw(k + o);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      in.gt[i] = gate_at<G, DK>(la, static_cast<size_t>(cl.t0 + min(gseg * 8 + i, cl.len - 1)), H, h, c0 + gch);
  };
  SliceIn cur, nxt;
  issue(0, cur);
  for (int sl = 0; sl < DK / 32; ++sl) {
    const int c0 = sl * 32;
    if (sl + 1 < DK / 32) issue(sl + 1, nxt);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u, row = e >> 3, c4 = (e & 7) * 4;
      const bool live = row < cl.len;
      const f32x4 xq = cvt4(cur.q[u]), xk = cvt4(cur.k[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i) qs[row * PS + c4 + i] = live ? xq[i] : 0.f, ks[row * PS + c4 + i] = live ? xk[i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = gseg * 8 + i;
      gs[row * PS + gch] = row < cl.len ? cur.gt[i] : 0.f;
    }
    lds_sync();
    row_scan<false, PS>(gs, tot);
    {  // Kg, Kb: thread (row, 8-channel group) writes one fragment group of each
      const int row = tid >> 2, c8 = (tid & 3) * 8;
      float xg[8], xb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = c8 + i;
        const float Gr = gs[row * PS + ch], GC = gs[(BC - 1) * PS + ch];
        const float kv = ks[row * PS + ch];
        xg[i] = kv * __expf(Gr);
        xb[i] = kv * __expf(GC - Gr);
      }
      pstore8(bk + B::oKg, DK, row, c0 + c8, xg);
      pstore8(bk + B::oKb, DK, row, c0 + c8, xb);
    }
    {  // transposed planes: thread (channel, 8-row group)
      const int ch = tid >> 3, r8 = (tid & 7) * 8;
      float xb[8], xg[8], xq[8];
      const float GC = gs[(BC - 1) * PS + ch];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = r8 + i;
        const float Gr = gs[row * PS + ch];
        const float eg = __expf(Gr);
        xb[i] = ks[row * PS + ch] * __expf(GC - Gr);
        xg[i] = ks[row * PS + ch] * eg;
        xq[i] = qs[row * PS + ch] * eg;
      }
      // read only by the chain passes: with bf16 io only as single bf16
      if constexpr (sizeof(T) == 2) {
        pstore8_hi(bk + B::oKbT, BC, c0 + ch, r8, xb);
        pstore8_hi(bk + B::oKgT, BC, c0 + ch, r8, xg);
        pstore8_hi(bk + B::oQgT, BC, c0 + ch, r8, xq);
      } else {
        pstore8(bk + B::oKbT, BC, c0 + ch, r8, xb);
        pstore8(bk + B::oKgT, BC, c0 + ch, r8, xg);
        pstore8(bk + B::oQgT, BC, c0 + ch, r8, xq);
      }
    }
    if (tid < 32) bk[B::oGam + c0 + tid] = __expf(gs[(BC - 1) * PS + tid]);
    // off-diagonal block pairs (I, J < I), split at row 16 I - 1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int I = off_pair_i(w, u), J = off_pair_j(w, u);
      if (I < 0) continue;
      const int ref = 16 * I - 1, ri = 16 * I + r, sj = 16 * J + r;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int ch = 4 * kk + g;
        const float gr = gs[ref * PS + ch];
        const float er = __expf(gs[ri * PS + ch] - gr);
        const float b = ks[sj * PS + ch] * __expf(gr - gs[sj * PS + ch]);
        aO[u] = mf(ks[ri * PS + ch] * er, b, aO[u]);
        pO[u] = mf(qs[ri * PS + ch] * er, b, pO[u]);
      }
    }
    // diagonal block pair (w, w) on fp32 MFMA, its operands scaled at the
    // row before the block: k_r e^{G_r - G_ref} (<= 1) against
    // k_s e^{G_ref - G_s} (>= 1, at most e^{kBwdDiagRange} for a channel
    // whose decay across the block is within range; the entries on and
    // above the diagonal are dropped after the last slice).  A channel that
    // decays faster takes the pair-by-pair path below instead.
    unsigned bad = 0;  // the slice's out-of-range channels (wave-uniform)
    {
      const int rr = 16 * w + r;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int ch = 4 * kk + g;
        const float gref = w > 0 ? gs[(16 * w - 1) * PS + ch] : 0.f;
        const bool inr = gref - gs[(16 * w + 15) * PS + ch] <= kBwdDiagRange;
        const float gr = gs[rr * PS + ch], kv = ks[rr * PS + ch];
        const float er = __expf(gr - gref);
        const float b = inr ? kv * __expf(gref - gr) : 0.f;
        aD = mf(kv * er, b, aD);
        pD = mf(qs[rr * PS + ch] * er, b, pD);
        const unsigned long long bl = __ballot(!inr);  // lane (r, g) holds channel 4 kk + g
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) bad |= ((bl >> (16 * gg)) & 1ull) ? (1u << (4 * kk + gg)) : 0u;
      }
    }
    {
      const int s = 16 * w + r;
      while (bad) {
        const int ch = __builtin_ctz(bad);
        bad &= bad - 1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int ri = 16 * w + 4 * g + m;
          if (s <= ri) {
            const float kE = ks[s * PS + ch] * __expf(gs[ri * PS + ch] - gs[s * PS + ch]);
            if (s < ri) aD[m] += ks[ri * PS + ch] * kE;
            pD[m] += qs[ri * PS + ch] * kE;
          }
        }
      }
    }
    lds_sync();
    cur = nxt;
  }
  // the diagonal block's products hold every pair: keep s < r for A, s <= r for P
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (r >= 4 * g + m) aD[m] = 0.f;
    if (r > 4 * g + m) pD[m] = 0.f;
  }
  // A to the block (upper blocks zero), L = Diag(beta) A and T = 0 in LDS
  // (P stays in its accumulators until T is done; it then goes through Lm)
  auto putA = [&](int I, int J, f32x4 a) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 16 * I + 4 * g + m, col = 16 * J + r;
      bk[B::oA + row * BC + col] = a[m];
      Lm[row * LPC + col] = bet[row] * a[m];
    }
  };
  putA(w, w, aD);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (off_pair_i(w, u) >= 0) putA(off_pair_i(w, u), off_pair_j(w, u), aO[u]);
  for (int e = tid; e < BC * BC; e += 256) {
    const int row = e >> 6, col = e & 63;
    if ((col >> 4) > (row >> 4)) {
      bk[B::oA + e] = 0.f;
      Lm[row * LPC + col] = 0.f;
    }
    Tm[row * LPC + col] = 0.f;
  }
  lds_sync();
  // T = (I + L)^{-1}, unit lower triangular.  Diagonal 16-blocks: one
  // thread per column, forward substitution.
  if (tid < BC) {
    const int base = tid & ~15, c = tid & 15;
    float x[16];
#pragma unroll
    for (int a = 0; a < 16; ++a) x[a] = a == c ? 1.f : 0.f;
#pragma unroll
    for (int a = 1; a < 16; ++a) {
      float s = 0.f;
#pragma unroll
      for (int b = 0; b < a; ++b) s += Lm[(base + a) * LPC + base + b] * x[b];
      if (a > c) x[a] = -s;
    }
#pragma unroll
    for (int a = 0; a < 16; ++a) Tm[(base + a) * LPC + base + c] = x[a];
  }
  lds_sync();
  // Off-diagonal blocks, one block row at a time:
  // T_IJ = -T_II sum_{K=J}^{I-1} L_IK T_KJ (wave J of block row I).
  for (int I = 1; I < 4; ++I) {
    const bool act = w < I;
    if (act) {
      f32x4 acc = zero4();
      for (int K = w; K < I; ++K)
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4)
          acc = mf(Lm[(16 * I + r) * LPC + 16 * K + kk + g], Tm[(16 * K + kk + g) * LPC + 16 * w + r], acc);
#pragma unroll
      for (int m = 0; m < 4; ++m) Xs[w][(4 * g + m) * 17 + r] = acc[m];
    }
    lds_sync();
    if (act) {
      f32x4 t = zero4();
#pragma unroll
      for (int kk = 0; kk < 16; kk += 4) t = mf(Tm[(16 * I + r) * LPC + 16 * I + kk + g], Xs[w][(kk + g) * 17 + r], t);
#pragma unroll
      for (int m = 0; m < 4; ++m) Tm[(16 * I + 4 * g + m) * LPC + 16 * w + r] = -t[m];
    }
    lds_sync();
  }
  // P into Lm (L is no longer needed), zero above the diagonal blocks
  auto putP = [&](int I, int J, f32x4 pv) {
#pragma unroll
    for (int m = 0; m < 4; ++m) Lm[(16 * I + 4 * g + m) * LPC + 16 * J + r] = pv[m];
  };
  putP(w, w, pD);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (off_pair_i(w, u) >= 0) putP(off_pair_i(w, u), off_pair_j(w, u), pO[u]);
  for (int e = tid; e < BC * BC; e += 256) {
    const int row = e >> 6, col = e & 63;
    if ((col >> 4) > (row >> 4)) Lm[row * LPC + col] = 0.f;
  }
  lds_sync();
  // T, T^T and P^T planes: thread (row, 8-column group), two groups each
  for (int e = tid; e < BC * 8; e += 256) {
    const int row = e >> 3, c8 = (e & 7) * 8;
    float xt[8], xtt[8], xpt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xt[i] = Tm[row * LPC + c8 + i];
      xtt[i] = Tm[(c8 + i) * LPC + row];
      xpt[i] = Lm[(c8 + i) * LPC + row];
    }
    pstore8(bk + B::oT, BC, row, c8, xt);
    pstore8(bk + B::oTT, BC, row, c8, xtt);
    pstore8(bk + B::oPT, BC, row, c8, xpt);
  }
}

// ---------------------------------------------------------------------------
// state: the chunk-entry states.  One workgroup (4 waves) per (sequence,
// head, 32 value columns), walking the sequence's chunks in order; the
// state (DK x 32) is held in MFMA accumulators, wave w owning key-channel
// rows [16 TPW w, 16 TPW (w + 1)) of both 16-column halves.  Per chunk:
//   W = Diag(beta)(V - Kg S)   (wave w: rows 16 w .. 16 w + 15)
//   U = T W
//   S = Diag(gamma) S + Kb^T U
// as split-bf16 products: the block factors are read as ready-split
// fragments, shared by the two halves; S, W and U are split once, when they
// are handed over through LDS (transposed, so that a B fragment is eight
// consecutive k of one column).  Every operand of chunk c + 1 is read into
// registers during chunk c, a third in each phase (one workgroup per CU,
// one wave per SIMD, so each wave has the whole register file for it).  Workgroup x: the value
// slices of a (sequence, head) share an XCD (x % 8), so they read each
// block through one L2.
// ---------------------------------------------------------------------------
constexpr int SCOLS = 32;  // value columns per state-pass workgroup

// A split-bf16 [NC][K] hand-over tile in LDS (NC columns, k contiguous): hi
// plane then lo plane, pitch K + 8 elements.
template <int K, int NC = SCOLS>
struct HTile {
  static constexpr int P = K + 8;
  static constexpr int elems = 2 * NC * P;
  __bf16* b;
  __device__ __forceinline__ F3 frag(int n, int k0) const {
    return F3{*reinterpret_cast<const bf16x8*>(b + n * P + k0), *reinterpret_cast<const bf16x8*>(b + NC * P + n * P + k0)};
  }
  // four consecutive k of column n (8-byte aligned)
  __device__ __forceinline__ void put4(int n, int k, f32x4 x) const {
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = static_cast<__bf16>(x[i]);
      lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(hi[i]));
    }
    *reinterpret_cast<bf16x4*>(b + n * P + k) = hi;
    *reinterpret_cast<bf16x4*>(b + NC * P + n * P + k) = lo;
  }
  __device__ __forceinline__ void put(int n, int k, float x) const {
    const __bf16 hi = static_cast<__bf16>(x);
    b[n * P + k] = hi;
    b[NC * P + n * P + k] = static_cast<__bf16>(x - static_cast<float>(hi));
  }
};

// Loop-carried accumulators that start from a global load: the compiler's
// memory-counter bookkeeping cannot tell the first iteration from the
// others, so inside the loop it would wait at every step for loads issued
// after these (the next chunk's operands).  Redefining the registers once,
// before the loop, ends that: the wait happens here, once.
template <int N>
__device__ __forceinline__ void settle(f32x4 (&x)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) asm volatile("" : "+v"(x[t]));
}

// A per-lane index the compiler cannot see through: addresses derived from it
// inside a loop are formed where they are used instead of being hoisted out
// of the loop and held (or spilled) across it.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Eight consecutive io elements kept as loaded until they are used.
template <typename T>
struct raw8;
template <>
struct raw8<float> {
  struct type {
    f32x4 a, b;
  };
  __device__ __forceinline__ static type load(const float* p) {
    return type{*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4)};
  }
  __device__ __forceinline__ static float get(const type& x, int i) { return i < 4 ? x.a[i] : x.b[i - 4]; }
};
template <>
struct raw8<bf16_t> {
  typedef uint4 type;
  __device__ __forceinline__ static type load(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static float get(const type& x, int i) {
    const uint32_t w = i < 2 ? x.x : (i < 4 ? x.y : (i < 6 ? x.z : x.w));
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};

template <typename T, int DK, int DV>
__device__ __forceinline__ void bwd_state_body(int x, const T* __restrict__ v, const int32_t* __restrict__ cu,
                                               const int32_t* __restrict__ chunk_off,
                                               const int32_t* __restrict__ order, int N, int H,
                                               const float* __restrict__ blk, const float* __restrict__ S0,
                                               float* __restrict__ sc) {
  typedef BwdBlk<DK> B;
  constexpr bool kHi = sizeof(T) == 2;  // bf16 io: single-bf16 block factors
  constexpr int NSP = DV / SCOLS, NKB = DK / 16, TPW = NKB / 4, NKS = DK / 32;
  __shared__ __align__(16) __bf16 lds_s[HTile<DK>::elems + 2 * HTile<BC>::elems];
  const HTile<DK> XT{lds_s};
  const HTile<BC> WT{lds_s + HTile<DK>::elems}, UT{lds_s + HTile<DK>::elems + HTile<BC>::elems};
  const int xcd = x & 7, s8 = x >> 3, sp = s8 % NSP, p = (s8 / NSP) * 8 + xcd;
  if (p >= N * H) return;
  const int n = order[p / H], h = p % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int tb = cu[n], L = cu[n + 1] - tb, nch = (L + BC - 1) / BC, j0 = chunk_off[n];
  const int col0 = sp * SCOLS + r;  // column of half hf: col0 + 16 hf
  const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * DV;
  const int kT1 = w >= 2 ? 1 : 0;  // k steps of T's row tile w: rows <= 16 w + 15
  f32x4 X[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 16 * (w * TPW + t) + 4 * g + m;
        X[t][hf][m] = S0 ? S0[sbase + static_cast<size_t>(row) * DV + col0 + 16 * hf] : 0.f;
      }
#pragma unroll
  for (int t = 0; t < TPW; ++t) settle(X[t]);
  struct Ops {
    F3 kg[NKS], tt[2], kbt[TPW][2];
    typename raw1<T>::type vv[2][4];
    float bet[4], gam[TPW][4];
  };
  // A chunk's operands in three parts (the parts of chunk c + 1 are issued
  // in the three phases of chunk c, so the memory pipe drains while the
  // wave computes instead of holding it at the chunk's start)
  auto load_a = [&](int c, Ops& o) {
    const float* bk = blk + (static_cast<size_t>(j0 + c) * H + h) * B::floats;
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) o.kg[kk] = pfragx<kHi>(bk + B::oKg, DK, 16 * w + r, 32 * kk + 8 * g);
  };
  auto load_c = [&](int c, Ops& o) {
    const float* bk = blk + (static_cast<size_t>(j0 + c) * H + h) * B::floats;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) o.kbt[t][kk] = pfragx<kHi>(bk + B::oKbT, BC, 16 * (w * TPW + t) + r, 32 * kk + 8 * g);
  };
  auto load_b = [&](int c, Ops& o) {
    const float* bk = blk + (static_cast<size_t>(j0 + c) * H + h) * B::floats;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) o.tt[kk] = pfragx<kHi>(bk + B::oT, BC, 16 * w + r, 32 * kk + 8 * g);
    const int t0 = tb + c * BC, len = min(BC, L - c * BC);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // rows past the sequence read its last row: their beta is 0, so W is 0
      // there whatever v holds (no branch, no wait on the load here)
      const int rr = 16 * w + 4 * g + m, rc = min(rr, len - 1);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        o.vv[hf][m] = raw1<T>::load(v + (static_cast<size_t>(t0 + rc) * H + h) * DV + col0 + 16 * hf);
      o.bet[m] = bk[B::oBeta + rr];
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) o.gam[t][m] = bk[B::oGam + 16 * (w * TPW + t) + 4 * g + m];
  };
  // Two operand sets used in turn (the loop is unrolled by two), so chunk
  // c + 1's operands stay in the registers they were loaded into: with one
  // set copied into the other at the end of every chunk, the copy would wait
  // there for the loads issued in the chunk's last phase.
  Ops opa, opb;
  if (nch > 0) {
    load_a(0, opa);
    load_b(0, opa);
    load_c(0, opa);
  }
  auto step = [&](int c, const Ops& cur, Ops& nxt) {
    const bool more = c + 1 < nch;
    float* so = sc + (static_cast<size_t>(j0 + c) * H + h) * DK * DV;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        XT.put4(16 * hf + r, 16 * (w * TPW + t) + 4 * g, X[t][hf]);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          so[static_cast<size_t>(16 * (w * TPW + t) + 4 * g + m) * DV + col0 + 16 * hf] = X[t][hf][m];
      }
    lds_sync();
    if (more) load_a(c + 1, nxt);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) acc = mmx<kHi>(cur.kg[kk], XT.frag(16 * hf + r, 32 * kk + 8 * g), acc);
      f32x4 wv;
#pragma unroll
      for (int m = 0; m < 4; ++m) wv[m] = cur.bet[m] * (raw1<T>::cvt(cur.vv[hf][m]) - acc[m]);
      WT.put4(16 * hf + r, 16 * w + 4 * g, wv);
    }
    lds_sync();
    if (more) load_b(c + 1, nxt);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (kk <= kT1) acc = mmx<kHi>(cur.tt[kk], WT.frag(16 * hf + r, 32 * kk + 8 * g), acc);
      UT.put4(16 * hf + r, 16 * w + 4 * g, acc);
    }
    lds_sync();
    if (more) load_c(c + 1, nxt);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int m = 0; m < 4; ++m) X[t][hf][m] *= cur.gam[t][m];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) X[t][hf] = mmx<kHi>(cur.kbt[t][kk], UT.frag(16 * hf + r, 32 * kk + 8 * g), X[t][hf]);
      }
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, opa, opb);
    if (c + 1 < nch) step(c + 1, opb, opa);
  }
}

// ---------------------------------------------------------------------------
// dstate: the cotangents of the chunk-final states, in reverse chunk order,
// with the same workgroup layout as the state pass.  Per chunk (X = dS of
// the chunk's final state on entry, of its entry state on exit):
//   Z = P^T dO + Kb X,  Y = T^T Z,  X = Diag(gamma) X + Qg^T dO - Kg^T Diag(beta) Y
// as split-bf16 products (dO, Z and -beta Y handed over through LDS,
// transposed); every operand of chunk c - 1 is read during chunk c, a third
// in each phase.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
__device__ __forceinline__ void bwd_dstate_body(int x, const T* __restrict__ dO, const int32_t* __restrict__ cu,
                                                const int32_t* __restrict__ chunk_off,
                                                const int32_t* __restrict__ order, int N, int H,
                                                const float* __restrict__ blk, const float* __restrict__ dST,
                                                float* __restrict__ dsc, float* __restrict__ dS0) {
  typedef BwdBlk<DK> B;
  constexpr bool kHi = sizeof(T) == 2;  // bf16 io: single-bf16 block factors
  constexpr int NSP = DV / SCOLS, NKB = DK / 16, TPW = NKB / 4, NKS = DK / 32;
  __shared__ __align__(16) __bf16 lds_d[HTile<DK>::elems + 3 * HTile<BC>::elems];
  const HTile<DK> XT{lds_d};
  const HTile<BC> DT{lds_d + HTile<DK>::elems}, ZT{lds_d + HTile<DK>::elems + HTile<BC>::elems},
      YT{lds_d + HTile<DK>::elems + 2 * HTile<BC>::elems};
  const int xcd = x & 7, s8 = x >> 3, sp = s8 % NSP, p = (s8 / NSP) * 8 + xcd;
  if (p >= N * H) return;
  const int n = order[p / H], h = p % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int tb = cu[n], L = cu[n + 1] - tb, nch = (L + BC - 1) / BC, j0 = chunk_off[n];
  const int col0 = sp * SCOLS + r;
  const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * DV;
  const int kU0 = w >= 2 ? 1 : 0;  // k steps of P^T, T^T row tile w: rows >= 16 w
  f32x4 X[TPW][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 16 * (w * TPW + t) + 4 * g + m;
        X[t][hf][m] = dST ? dST[sbase + static_cast<size_t>(row) * DV + col0 + 16 * hf] : 0.f;
      }
#pragma unroll
  for (int t = 0; t < TPW; ++t) settle(X[t]);
  struct Ops {
    F3 pt[2], tt[2], kb[NKS], qgt[TPW][2], kgt[TPW][2];
    typename raw8<T>::type dov;
    float bet[4], gam[TPW][4];
  };
  const int drow = tid >> 2, dc8 = (tid & 3) * 8;  // this thread's 8 dO values for the hand-over tile
  // a chunk's operands in three parts, issued in the three phases of the
  // chunk before (see bwd_state_body)
  auto load_a = [&](int c, Ops& o) {
    const float* bk = blk + (static_cast<size_t>(j0 + c) * H + h) * B::floats;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) o.pt[kk] = pfragx<kHi>(bk + B::oPT, BC, 16 * w + r, 32 * kk + 8 * g);
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) o.kb[kk] = pfragx<kHi>(bk + B::oKb, DK, 16 * w + r, 32 * kk + 8 * g);
  };
  auto load_c = [&](int c, Ops& o) {
    const float* bk = blk + (static_cast<size_t>(j0 + c) * H + h) * B::floats;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        o.qgt[t][kk] = pfragx<kHi>(bk + B::oQgT, BC, 16 * (w * TPW + t) + r, 32 * kk + 8 * g);
        o.kgt[t][kk] = pfragx<kHi>(bk + B::oKgT, BC, 16 * (w * TPW + t) + r, 32 * kk + 8 * g);
      }
  };
  auto load_b = [&](int c, Ops& o) {
    const float* bk = blk + (static_cast<size_t>(j0 + c) * H + h) * B::floats;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) o.tt[kk] = pfragx<kHi>(bk + B::oTT, BC, 16 * w + r, 32 * kk + 8 * g);
    const int t0 = tb + c * BC, len = min(BC, L - c * BC);
    // rows past the sequence read the last row: P and Qg are zero in those
    // rows, so their dO never contributes (no branch, no wait on the load here)
    o.dov = raw8<T>::load(dO + (static_cast<size_t>(t0 + min(drow, len - 1)) * H + h) * DV + sp * SCOLS + dc8);
#pragma unroll
    for (int m = 0; m < 4; ++m) o.bet[m] = bk[B::oBeta + 16 * w + 4 * g + m];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) o.gam[t][m] = bk[B::oGam + 16 * (w * TPW + t) + 4 * g + m];
  };
  // two operand sets used in turn, as in the state pass
  Ops opa, opb;
  if (nch > 0) {
    load_a(nch - 1, opa);
    load_b(nch - 1, opa);
    load_c(nch - 1, opa);
  }
  auto step = [&](int c, const Ops& cur, Ops& nxt) {
    const bool more = c > 0;
    float* so = dsc + (static_cast<size_t>(j0 + c) * H + h) * DK * DV;
    lds_sync();  // the previous chunk's readers of DT and YT are done
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        XT.put4(16 * hf + r, 16 * (w * TPW + t) + 4 * g, X[t][hf]);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          so[static_cast<size_t>(16 * (w * TPW + t) + 4 * g + m) * DV + col0 + 16 * hf] = X[t][hf][m];
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) DT.put(dc8 + i, drow, raw8<T>::get(cur.dov, i));
    lds_sync();
    if (more) load_a(c - 1, nxt);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (kk >= kU0) acc = mmx<kHi>(cur.pt[kk], DT.frag(16 * hf + r, 32 * kk + 8 * g), acc);
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) acc = mmx<kHi>(cur.kb[kk], XT.frag(16 * hf + r, 32 * kk + 8 * g), acc);
      ZT.put4(16 * hf + r, 16 * w + 4 * g, acc);
    }
    lds_sync();
    if (more) load_b(c - 1, nxt);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (kk >= kU0) acc = mmx<kHi>(cur.tt[kk], ZT.frag(16 * hf + r, 32 * kk + 8 * g), acc);
      f32x4 yb;
#pragma unroll
      for (int m = 0; m < 4; ++m) yb[m] = -cur.bet[m] * acc[m];
      YT.put4(16 * hf + r, 16 * w + 4 * g, yb);
    }
    lds_sync();
    if (more) load_c(c - 1, nxt);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int m = 0; m < 4; ++m) X[t][hf][m] *= cur.gam[t][m];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          X[t][hf] = mmx<kHi>(cur.qgt[t][kk], DT.frag(16 * hf + r, 32 * kk + 8 * g), X[t][hf]);
          X[t][hf] = mmx<kHi>(cur.kgt[t][kk], YT.frag(16 * hf + r, 32 * kk + 8 * g), X[t][hf]);
        }
      }
  };
  for (int c = nch - 1; c >= 0; c -= 2) {
    step(c, opa, opb);
    if (c > 0) step(c - 1, opb, opa);
  }
  if (dS0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int row = 16 * (w * TPW + t) + 4 * g + m;
          dS0[sbase + static_cast<size_t>(row) * DV + col0 + 16 * hf] = X[t][hf][m];
        }
  }
}


// The two state passes in one launch: workgroups [0, half) run the forward
// state pass, [half, 2 half) the reverse cotangent pass.  They share no data,
// and two of these workgroups fit on a CU (LDS and registers), so the two
// latency-bound chains interleave on every CU instead of running one after
// the other.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_states_kernel(const T* __restrict__ v, const T* __restrict__ dO,
                                                         const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ chunk_off,
                                                         const int32_t* __restrict__ order, int N, int H,
                                                         const float* __restrict__ blk, const float* __restrict__ S0,
                                                         const float* __restrict__ dST, float* __restrict__ sc,
                                                         float* __restrict__ dsc, float* __restrict__ dS0, int half) {
  const int x = blockIdx.x;
  if (x < half) bwd_state_body<T, DK, DV>(x, v, cu, chunk_off, order, N, H, blk, S0, sc);
  else bwd_dstate_body<T, DK, DV>(x - half, dO, cu, chunk_off, order, N, H, blk, dST, dsc, dS0);
}



// ---------------------------------------------------------------------------
// grad_v: persistent workgroups (4 waves, one per CU), each taking (chunk,
// head) items in turn; per item it walks the value columns 32 at a time (one 32-wide k step of the products over
// value columns).  Per slice, wave w on rows 16 w .. 16 w + 15:
//   Vt = V - Kg S0, W = Diag(beta) Vt, U = T W
//   dU = P^T dO + Kb dS_C, dW = T^T dU, dv = Diag(beta) dW
// then every wave adds the slice's share of the contractions over value
// columns into its MFMA tiles: dP, dM = -dW U^T, dQg, dKg = -dv S0^T, dKb.
// Each operand sits in LDS in the orientation whose fragments are eight
// consecutive floats (the S0, dS_C and dO slices both ways, W, dU transposed,
// U and dW by rows); a slice's inputs are loaded while the previous slice
// runs, and the next item's first slice and block operands while the
// current item's last slice runs.  At the end dbeta and dv are written out, and dQg, dKg,
// dKb, dP, dA = Diag(beta) dM, dgamma over the chunk's block (everything it
// read from the block has been consumed by then).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tri_ij(int e, int& I, int& J) {
  I = e >= 6 ? 3 : (e >= 3 ? 2 : (e >= 1 ? 1 : 0));
  J = e - I * (I + 1) / 2;
}

// A split-bf16 matrix in LDS: hi and lo planes with a row pitch of P
// elements (P * 2 bytes a multiple of 16, so a fragment is one 16-byte read).
struct Plane {
  __bf16* h;
  __bf16* l;
  int P;
  __device__ __forceinline__ F3 frag(int row, int k0) const {
    return F3{*reinterpret_cast<const bf16x8*>(h + row * P + k0), *reinterpret_cast<const bf16x8*>(l + row * P + k0)};
  }
  __device__ __forceinline__ void put(int row, int col, float x) const {
    const __bf16 hi = static_cast<__bf16>(x);
    h[row * P + col] = hi;
    l[row * P + col] = static_cast<__bf16>(x - static_cast<float>(hi));
  }
  // four consecutive elements of one row (8-byte aligned)
  __device__ __forceinline__ void put4(int row, int col, f32x4 x) const {
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = static_cast<__bf16>(x[i]);
      lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(hi[i]));
    }
    *reinterpret_cast<bf16x4*>(h + row * P + col) = hi;
    *reinterpret_cast<bf16x4*>(l + row * P + col) = lo;
  }
};

template <int DK>
struct GradVLds {
  static constexpr int PW = 40;       // pitch of [*][32] planes (k = value column)
  static constexpr int PC = BC + 8;   // pitch of [32][BC] planes (k = chunk row)
  static constexpr int PK = DK + 8;   // pitch of [32][DK] planes (k = key channel)
  // element offsets of each plane's hi part; its lo part follows at + rows * pitch
  static constexpr int oS0 = 0;                          // [DK][PW]  S0 columns of the slice
  static constexpr int odS = oS0 + 2 * DK * PW;          // [DK][PW]
  static constexpr int odO = odS + 2 * DK * PW;          // [BC][PW]
  static constexpr int oWT = odO + 2 * BC * PW;          // [32][PC]
  static constexpr int odUT = oWT + 2 * 32 * PC;         // [32][PC]
  static constexpr int oU = odUT + 2 * 32 * PC;          // [BC][PW]
  static constexpr int odW = oU + 2 * BC * PW;           // [BC][PW]
  static constexpr int odV = odW + 2 * BC * PW;          // [BC][PW]  dv = beta dW
  static constexpr int elems = odV + 2 * BC * PW;        // bf16 elements
  // the transposed slice inputs, an array of their own (it takes the next
  // slice's raw inputs while the rest of the slice runs)
  static constexpr int tS0 = 0;                          // [32][PK]
  static constexpr int tdS = tS0 + 2 * 32 * PK;          // [32][PK]
  static constexpr int tdO = tdS + 2 * 32 * PK;          // [32][PC]
  static constexpr int telems = tdO + 2 * 32 * PC;
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_grad_v_kernel(
    const T* __restrict__ v, const T* __restrict__ dO, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_off, int N, int H, float* __restrict__ blk, const float* __restrict__ sc,
    const float* __restrict__ dsc, T* __restrict__ dv, float* __restrict__ dbeta) {
  typedef BwdBlk<DK> B;
  typedef GradVLds<DK> LL;
  constexpr int NSP = DV / 32, NKB = DK / 16, NKS = DK / 32;
  constexpr int NTILE = 20 + 3 * 4 * NKB;  // dP (10), dM (10), dQg, dKg, dKb (4 NKB each)
  constexpr int NT = (NTILE + 3) / 4;
  constexpr int PW = LL::PW, PC = LL::PC, PK = LL::PK;
  __shared__ __align__(16) __bf16 lds[LL::elems];
  __shared__ __align__(16) __bf16 ldsT[LL::telems];
  __shared__ float betl[BC], dbp[BC * 5];
  __shared__ __align__(16) float Al[10 * 256];
  auto plane = [&](int off, int rows, int pitch) { return Plane{lds + off, lds + off + rows * pitch, pitch}; };
  auto tplane = [&](int off, int pitch) { return Plane{ldsT + off, ldsT + off + 32 * pitch, pitch}; };
  const Plane S0p = plane(LL::oS0, DK, PW), S0T = tplane(LL::tS0, PK);
  const Plane dSp = plane(LL::odS, DK, PW), dST = tplane(LL::tdS, PK);
  const Plane Dp = plane(LL::odO, BC, PW), DT = tplane(LL::tdO, PC);
  const Plane WT = plane(LL::oWT, 32, PC), dUT = plane(LL::odUT, 32, PC);
  const Plane Up = plane(LL::oU, BC, PW), dWp = plane(LL::odW, BC, PW), dVp = plane(LL::odV, BC, PW);
  const int nch = chunk_off[N], items = nch * H;
  int it = blockIdx.x;
  if (it >= items) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // dbeta's partial sums (five per row); the slots of blocks above the
  // diagonal are never written and stay 0 for every item
  for (int e = tid; e < BC * 5; e += 256) dbp[e] = 0.f;
  // Work item i: chunk i % nch of head i / nch (chunks of a head adjacent)
  struct Item {
    int h;
    ChunkLoc cl;
    float* bk;
    const float* s0;
    const float* dsC;
  };
  auto item_at = [&](int i) {
    Item x;
    const int j = i % nch;
    x.h = i / nch;
    x.cl = locate(cu, chunk_off, N, j);
    const size_t slot = static_cast<size_t>(j) * H + x.h;
    x.bk = blk + slot * B::floats;
    x.s0 = sc + slot * DK * DV;
    x.dsC = dsc + slot * DK * DV;
    return x;
  };
  // block operands of the wave's row tile (rows 16 w + r), ready split:
  // Kg, Kb, P^T (first phase), T, T^T and beta (second phase)
  F3 kgf[NKS], kbf[NKS], tf[2], ptf[2], ttf[2];
  float bet[4];
  // (the addresses below, and in the other per-item steps, are formed from
  // an opaque lane index so that they are not held across the item loop)
  auto load_first = [&](const Item& x) {
    const int ln = opaque(lane), row = 16 * w + (ln & 15), k8 = 8 * (ln >> 4);
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      kgf[kk] = pfrag(x.bk + B::oKg, DK, row, 32 * kk + k8);
      kbf[kk] = pfrag(x.bk + B::oKb, DK, row, 32 * kk + k8);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ptf[kk] = pfrag(x.bk + B::oPT, BC, row, 32 * kk + k8);
  };
  auto load_second = [&](const Item& x) {
    const int ln = opaque(lane), row = 16 * w + (ln & 15), k8 = 8 * (ln >> 4);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      tf[kk] = pfrag(x.bk + B::oT, BC, row, 32 * kk + k8);
      ttf[kk] = pfrag(x.bk + B::oTT, BC, row, 32 * kk + k8);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) bet[m] = x.bk[B::oBeta + 16 * w + 4 * (ln >> 4) + m];
  };
  // k steps (32 chunk rows each) a triangular factor of row tile w needs:
  // T (lower): rows <= 16 w + 15;  T^T, P^T: rows >= 16 w
  const int kT1 = w >= 2 ? 1 : 0, kU0 = w >= 2 ? 1 : 0;
  // The slice inputs (S0 and dS_C [DK][32] fp32, dO [BC][32] io) land raw in
  // LDS by direct global-to-LDS loads, in the area of the transposed S0, dS_C
  // and dO planes.  Those planes are read only in the first phase, so the
  // loads of the next slice (the next item's first slice, after an item's
  // last) are issued right after it and arrive while the current slice
  // finishes; the split of a slice writes the row planes from the raw inputs
  // and then copies them into the transposed planes, over the raw inputs.
  // The area is an LDS array of its own: the compiler then knows that the
  // reads of the other planes do not wait for those loads.
  unsigned char* const rawS0 = reinterpret_cast<unsigned char*>(ldsT + LL::tS0);
  unsigned char* const rawdS = reinterpret_cast<unsigned char*>(ldsT + LL::tdS);
  unsigned char* const rawdO = reinterpret_cast<unsigned char*>(ldsT + LL::tdO);
  static_assert(DK * 128 <= 2 * 32 * PK * 2 && BC * 32 * static_cast<int>(sizeof(T)) <= 2 * 32 * PC * 2,
                "raw slice inputs fit the transposed planes");
  static_assert((LL::tdS * 2) % 16 == 0 && (LL::tdO * 2) % 16 == 0, "raw areas are 16-byte aligned");
  auto dma = [&](const void* src, void* dst) {  // one wave: 64 lanes x 16 bytes to dst (wave-uniform)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  auto issue = [&](const Item& x, int sp) {
    const int ln = opaque(lane);
    // S0, dS_C: a wave load is 8 rows x 128 bytes
#pragma unroll
    for (int i = 0; i < DK / 32; ++i) {
      const int r0 = 8 * (wu + 4 * i), row = r0 + (ln >> 3);
      const size_t o = static_cast<size_t>(row) * DV + sp * 32 + (ln & 7) * 4;
      dma(x.s0 + o, rawS0 + r0 * 128);
      dma(x.dsC + o, rawdS + r0 * 128);
    }
    // dO: a wave load is 1024 / VROW rows; rows past the sequence read its
    // last row (zeroed at the split)
    constexpr int VROW = 32 * static_cast<int>(sizeof(T)), RPL = 1024 / VROW, LPR = VROW / 16, NL = BC / RPL;
#pragma unroll
    for (int i = 0; i < (NL + 3) / 4; ++i) {
      const int li = min(wu + 4 * i, NL - 1);  // a wave past the last load repeats it (same bytes)
      const int row = li * RPL + ln / LPR;
      const size_t o = (static_cast<size_t>(x.cl.t0 + min(row, x.cl.len - 1)) * H + x.h) * DV + sp * 32 +
                       (ln % LPR) * (16 / static_cast<int>(sizeof(T)));
      dma(dO + o, rawdO + li * 1024);
    }
  };
  // v where the first phase uses it (rows 16 w + 4 g + m, columns 16 nt + r
  // of the slice), read one slice ahead; rows past the sequence read its
  // last row (beta, dU and dW are 0 there)
  typename raw1<T>::type vr[2][4];
  auto issue_v = [&](const Item& x, int sp) {
    const int ln = opaque(lane), rb = 16 * w + 4 * (ln >> 4);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = min(rb + m, x.cl.len - 1);
        vr[nt][m] = raw1<T>::load(v + (static_cast<size_t>(x.cl.t0 + row) * H + x.h) * DV + sp * 32 + 16 * nt +
                                  (ln & 15));
      }
  };
  // A's ten lower 16 x 16 blocks, for dbeta's inverse share at the end
  auto issue_A = [&](const Item& x) {
    const int ln = opaque(lane);
    for (int t = wu; t < 10; t += 4) {
      int I, J;
      tri_ij(t, I, J);
      dma(x.bk + B::oA + (16 * I + (ln >> 2)) * BC + 16 * J + (ln & 3) * 4, Al + t * 256);
    }
  };
  Item cur = item_at(it);
  load_first(cur);
  load_second(cur);
  issue_A(cur);
  issue(cur, 0);
  issue_v(cur, 0);
  const T* const rdO = reinterpret_cast<const T*>(rawdO);
  for (;;) {
    const int nx = it + static_cast<int>(gridDim.x);
    const bool more = nx < items;
    const Item nxt = item_at(more ? nx : it);
    f32x4 acc[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[u] = zero4();
    float db1[4] = {0.f, 0.f, 0.f, 0.f};
    float dg[DK / 32];  // dgamma of rows (tid >> 3) + 32 i (every lane of a row's eight holds it)
#pragma unroll
    for (int i = 0; i < DK / 32; ++i) dg[i] = 0.f;
    for (int sp = 0; sp < NSP; ++sp) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's loads of the slice are in LDS
      lds_sync();
      if (sp == 0 && r == 0) {  // beta of the item's rows, for the end (read after several barriers)
#pragma unroll
        for (int m = 0; m < 4; ++m) betl[16 * w + 4 * g + m] = bet[m];
      }
      // slice inputs, split once, by rows; dgamma's share of the slice (a
      // row's 32 columns, fixed order)
      const int c4 = (tid & 7) * 4;
#pragma unroll
      for (int i = 0; i < DK / 32; ++i) {
        const int row = (tid >> 3) + 32 * i;
        const f32x4 a = *reinterpret_cast<const f32x4*>(rawS0 + (row * 32 + c4) * 4);
        const f32x4 b = *reinterpret_cast<const f32x4*>(rawdS + (row * 32 + c4) * 4);
        S0p.put4(row, c4, a);
        dSp.put4(row, c4, b);
        float pr = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
        pr += __shfl_xor(pr, 1);
        pr += __shfl_xor(pr, 2);
        pr += __shfl_xor(pr, 4);
        dg[i] += pr;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = (tid >> 3) + 32 * i;
        Dp.put4(row, c4, row < cur.cl.len ? load4(rdO + row * 32 + c4) : zero4());
      }
      lds_sync();
      // the raw inputs are read: the transposed planes, copied from the split
      // rows, go over them.  A lane takes two consecutive rows (2 p, 2 p + 1)
      // of four columns (4 q ..) and writes each column's pair as one dword;
      // a wave covers 16 row pairs x 4 column quads, so its writes fall in
      // distinct banks.
      auto tput = [&](const Plane& src, const Plane& dst, int p, int q) {
        const int r0 = 2 * p, c0 = 4 * q;
        const bf16x4 h0 = *reinterpret_cast<const bf16x4*>(src.h + r0 * src.P + c0);
        const bf16x4 h1 = *reinterpret_cast<const bf16x4*>(src.h + (r0 + 1) * src.P + c0);
        const bf16x4 l0 = *reinterpret_cast<const bf16x4*>(src.l + r0 * src.P + c0);
        const bf16x4 l1 = *reinterpret_cast<const bf16x4*>(src.l + (r0 + 1) * src.P + c0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x2 hp, lp;
          hp[0] = h0[c], hp[1] = h1[c];
          lp[0] = l0[c], lp[1] = l1[c];
          *reinterpret_cast<bf16x2*>(dst.h + (c0 + c) * dst.P + r0) = hp;
          *reinterpret_cast<bf16x2*>(dst.l + (c0 + c) * dst.P + r0) = lp;
        }
      };
      // task t of a plane with R rows: row pair 16 (t / 2) + lane % 16,
      // column quad 4 (t % 2) + lane / 16; R / 32 * 2 tasks, wave w takes w, w + 4, ..
      const int tl = opaque(lane);
#pragma unroll
      for (int t = w; t < DK / 16; t += 4) {
        tput(S0p, S0T, 16 * (t >> 1) + (tl & 15), 4 * (t & 1) + (tl >> 4));
        tput(dSp, dST, 16 * (t >> 1) + (tl & 15), 4 * (t & 1) + (tl >> 4));
      }
#pragma unroll
      for (int t = w; t < BC / 16; t += 4) tput(Dp, DT, 16 * (t >> 1) + (tl & 15), 4 * (t & 1) + (tl >> 4));
      lds_sync();
      // Vt, W = beta Vt (transposed) and dU (transposed) for the two 16-column tiles
      f32x4 vt[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int n = 16 * nt + r;
        f32x4 a = zero4(), d = zero4();
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          a = mm3(kgf[kk], S0T.frag(n, 32 * kk + 8 * g), a);
          d = mm3(kbf[kk], dST.frag(n, 32 * kk + 8 * g), d);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          if (kk >= kU0) d = mm3(ptf[kk], DT.frag(n, 32 * kk + 8 * g), d);
        f32x4 wv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          vt[nt][m] = raw1<T>::cvt(vr[nt][m]) - a[m];
          wv[m] = bet[m] * vt[nt][m];
        }
        WT.put4(n, 16 * w + 4 * g, wv);
        dUT.put4(n, 16 * w + 4 * g, d);
      }
      lds_sync();
      // the transposed planes are free: the next slice's inputs go there
      // (after the item's last slice, the next item's first, with its
      // first-phase block operands)
      // (one call site each: the loads then go straight into the registers
      // that carry them, with no copy that would wait for them)
      const bool same = sp + 1 < NSP;
      if (same || more) {
        const Item& x = same ? cur : nxt;
        issue(x, same ? sp + 1 : 0);
        issue_v(x, same ? sp + 1 : 0);
      }
      if (!same && more) load_first(nxt);
      // U = T W (rows) and dW = T^T dU (rows), dv, dbeta's write share
      const int ln2 = opaque(lane);
      T* const dvrow =
          dv + (static_cast<size_t>(cur.cl.t0 + 16 * w + 4 * (ln2 >> 4)) * H + cur.h) * DV + sp * 32 + (ln2 & 15);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int n = 16 * nt + r;
        f32x4 a = zero4(), d = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk <= kT1) a = mm3(tf[kk], WT.frag(n, 32 * kk + 8 * g), a);
          if (kk >= kU0) d = mm3(ttf[kk], dUT.frag(n, 32 * kk + 8 * g), d);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int row = 16 * w + 4 * g + m;
          Up.put(row, n, a[m]);
          dWp.put(row, n, d[m]);
          dVp.put(row, n, bet[m] * d[m]);
          db1[m] += d[m] * vt[nt][m];
          if (row < cur.cl.len) io<T>::store(dvrow + static_cast<size_t>(m) * H * DV + 16 * nt, bet[m] * d[m]);
        }
      }
      if (sp + 1 == NSP && more) load_second(nxt);  // the second-phase operands are used
      lds_sync();
      // the slice's share of the contractions over value columns.  Every
      // operand is a [rows][PW] plane, so a fragment is the lane's base
      // (r PW + 8 g) plus a wave-uniform offset: no per-wave code paths.
      {
        const __bf16* const lb = lds + opaque(r * PW + 8 * g);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const int tau = w + 4 * u;
          if (tau >= NTILE) break;
          int oa, ob, la, lo;  // hi-plane offsets of the A and B rows, lo-plane displacements
          if (u < 5) {         // dP (tau < 10) and dM tiles: rows of dO or dW against rows of U
            int I, J;
            tri_ij(tau % 10, I, J);
            oa = (tau < 10 ? LL::odO : LL::odW) + 16 * I * PW;
            ob = LL::oU + 16 * J * PW;
            la = BC * PW;
            lo = BC * PW;
          } else {  // dQg (dO S0^T), dKg (dv S0^T), dKb (U dS^T): kind and row tile fixed by u
            const int e = tau - 20, kind = e / (4 * NKB), rem = e % (4 * NKB), I = rem / NKB, Jc = rem % NKB;
            oa = (kind == 0 ? LL::odO : (kind == 1 ? LL::odV : LL::oU)) + 16 * I * PW;
            ob = (kind == 2 ? LL::odS : LL::oS0) + 16 * Jc * PW;
            la = BC * PW;
            lo = DK * PW;
          }
          oa = __builtin_amdgcn_readfirstlane(oa);
          ob = __builtin_amdgcn_readfirstlane(ob);
          const F3 fa{*reinterpret_cast<const bf16x8*>(lb + oa), *reinterpret_cast<const bf16x8*>(lb + oa + la)};
          const F3 fb{*reinterpret_cast<const bf16x8*>(lb + ob), *reinterpret_cast<const bf16x8*>(lb + ob + lo)};
          acc[u] = mm3(fa, fb, acc[u]);
        }
      }
    }
    // dbeta: the write's share (dW . Vt, summed over value columns) and the
    // inverse's share (sum_s dM[r][s] A[r][s]), each part in its own slot and
    // summed in a fixed order
    const int ln3 = opaque(lane), r3 = ln3 & 15, g3 = ln3 >> 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float x = group_sum<16>(db1[m]);
      if (r == 0) dbp[(16 * w + 4 * g + m) * 5 + 4] = x;
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int tau = w + 4 * u;
      if (tau >= 10 && tau < 20) {
        int I, J;
        tri_ij(tau - 10, I, J);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int row = 16 * I + 4 * g3 + m;
          const float x = group_sum<16>(-acc[u][m] * Al[(tau - 10) * 256 + (4 * g3 + m) * 16 + r3]);
          if (r3 == 0) dbp[row * 5 + J] = x;
        }
      }
    }
    lds_sync();
    if (more) issue_A(nxt);  // A is read: the next item's goes there
    float* const bk = cur.bk;
    if (tid < cur.cl.len) {
      const float* x = dbp + tid * 5;
      dbeta[static_cast<size_t>(cur.cl.t0 + tid) * H + cur.h] = x[4] + x[0] + x[1] + x[2] + x[3];
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int tau = w + 4 * u;
      if (tau >= NTILE) break;
      if (tau < 20) {
        int I, J;
        tri_ij(tau % 10, I, J);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int row = 16 * I + 4 * g3 + m, col = 16 * J + r3;
          if (tau < 10) bk[B::odP + row * BC + col] = (I == J && col > row) ? 0.f : acc[u][m];
          else bk[B::odA + row * BC + col] = (I == J && col >= row) ? 0.f : -betl[row] * acc[u][m];
        }
      } else {
        const int e = tau - 20, kind = e / (4 * NKB), rem = e % (4 * NKB), I = rem / NKB, Jc = rem % NKB;
        const size_t o = kind == 0 ? B::odQg : (kind == 1 ? B::odKg : B::odKb);
        const float sgn = kind == 1 ? -1.f : 1.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) bk[o + (16 * I + 4 * g3 + m) * DK + 16 * Jc + r3] = sgn * acc[u][m];
      }
    }
    if ((tid & 7) == 0) {
#pragma unroll
      for (int i = 0; i < DK / 32; ++i) bk[B::odGam + (tid >> 3) + 32 * i] = dg[i];
    }
    if (!more) break;
    it = nx;
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// grad_k: one workgroup (4 waves) per (chunk, head), walking the key
// channels SW at a time (for the one-rate-per-head gate the per-head gate
// cotangent is then summed inside the workgroup).  Thread t works on row
// t / 4 and SW / 4 consecutive channels of the slice; SW = 16 keeps the LDS
// of two workgroups on a CU.
//   GQ[r]  = sum_{s <= r} dP[r][s] k_s e^{G_r - G_s}
//   GA[r]  = sum_{s <  r} dA[r][s] k_s e^{G_r - G_s}
//   G2[s]  = sum_{r >= s} (dP[r][s] q_r + dA[r][s] k_r) e^{G_r - G_s}
//   dq = dQg e^{G} + GQ,   dk = dKg e^{G} + dKb e^{G_C - G} + GA + G2
//   dG = dQg Qg + dKg Kg - dKb Kb + q GQ + k (GA - G2)
//        (+ sum_s dKb_s Kb_s + dgamma gamma on the last row, for G_C)
//   dlog alpha_u = sum_{r >= u} dG_r
// Block pairs use operands scaled at a reference row (row side: rows s of
// the earlier blocks and of the block itself scaled by e^{G_{16I-1} - G_s};
// column side: rows r of the block and the later ones by e^{G_r - G_{16I+15}});
// the block's own pairs of a channel that decays by more than e^{59.6}
// across it are taken pair by pair instead.
// ---------------------------------------------------------------------------
template <typename T, int DK, int G, int SW>
__global__ __launch_bounds__(256) void bwd_grad_k_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const float* __restrict__ la, const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ chunk_off, int N, int H,
                                                         const float* __restrict__ blk, T* __restrict__ dq,
                                                         T* __restrict__ dk, float* __restrict__ dla) {
  typedef BwdBlk<DK> B;
  constexpr int PS = SW + 4;  // pitch of the SW-channel slices (16-byte rows)
  constexpr int CPT = SW / 4;  // channels per thread (a row's four threads cover the slice)
  // every slice of the (chunk, head) in one workgroup: dP and dA are staged
  // in LDS once for all of them (with one workgroup per slice they were
  // loaded DK / SW times: 3.5% of the backward call at 131k)
  constexpr int NSW = DK / SW;
  __shared__ float qs[BC * PS], ks[BC * PS], gs[BC * PS];
  __shared__ float dPl[BC * LPC], dAl[BC * LPC];
  __shared__ float Ksc[96 * PS], Xq[96 * PS], Xk[96 * PS];
  __shared__ float tot[256], rsum[BC];
  // 1-D grid, XCD-aware: the NZ channel slices of one (chunk, head) get
  // workgroup ids that differ by multiples of 8, i.e. one XCD and adjacent
  // dispatch, so the dP and dA they all read come through one L2
  constexpr int NZ = DK / SW / NSW;
  const int x = blockIdx.x, xcd = x & 7, rest = x >> 3, zs = rest % NZ, item = (rest / NZ) * 8 + xcd;
  const int j = item / H, h = item % H;
  if (j >= chunk_off[N]) return;
  const ChunkLoc cl = locate(cu, chunk_off, N, j);
  const float* bk = blk + (static_cast<size_t>(j) * H + h) * B::floats;
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
  // thread: row 16 w + l % 16 of 16-row block I = w, channels CPT (l / 16) .. + CPT - 1,
  // the output layout of the transposed MFMA tiles below
  static_assert(CPT == 4, "four channels per thread (the MFMA output rows)");
  const int row = 16 * (tid >> 6) + ln, c8 = lg * CPT;
  const int I = __builtin_amdgcn_readfirstlane(tid >> 6);  // = row / 16, the wave's block (uniform)
  // Every global input of a slice is issued before the first is used, so
  // their latencies overlap: the slice's q, k, gates and the dQg, dKg, dKb
  // cotangents (read at the end), then (first slice) dP and dA into LDS.
  // Rows past the sequence read its last row and are zeroed at the use.
  constexpr int RPS = BC * SW / 256;  // rows per thread of the gate load
  const int gch = tid % SW, gseg = tid / SW;
  const int rowc = min(row, cl.len - 1);
  // two sets used in turn: a slice's inputs are issued into the other set
  // while the slice before it computes
  struct KIn {
    float xq[CPT], xk[CPT], xg[RPS], dQg[CPT], dKg[CPT], dKb[CPT];
  };
  auto issue = [&](int c0, KIn& in) {
    const size_t o = (static_cast<size_t>(cl.t0 + rowc) * H + h) * DK + c0 + c8;
    loadn<CPT>(q + o, in.xq);
    loadn<CPT>(k + o, in.xk);
#pragma unroll
    for (int i = 0; i < RPS; ++i)
      in.xg[i] = gate_at<G, DK>(la, static_cast<size_t>(cl.t0 + min(gseg * RPS + i, cl.len - 1)), H, h, c0 + gch);
    const size_t ob = static_cast<size_t>(row) * DK + c0 + c8;
    loadn<CPT>(bk + B::odQg + ob, in.dQg);
    loadn<CPT>(bk + B::odKg + ob, in.dKg);
    loadn<CPT>(bk + B::odKb + ob, in.dKb);
  };
  KIn ina, inb;
  issue(zs * NSW * SW, ina);
  {
    f32x4 a[BC * BC / 4 / 256], b[BC * BC / 4 / 256];
#pragma unroll
    for (int u = 0; u < BC * BC / 4 / 256; ++u) {
      const int e = tid + 256 * u, rr = e >> 4, c4 = (e & 15) * 4;
      a[u] = *reinterpret_cast<const f32x4*>(bk + B::odP + rr * BC + c4);
      b[u] = *reinterpret_cast<const f32x4*>(bk + B::odA + rr * BC + c4);
    }
#pragma unroll
    for (int u = 0; u < BC * BC / 4 / 256; ++u) {
      const int e = tid + 256 * u, rr = e >> 4, c4 = (e & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) dPl[rr * LPC + c4 + i] = a[u][i], dAl[rr * LPC + c4 + i] = b[u][i];
    }
  }
  if (tid < BC) rsum[tid] = 0.f;
  auto slice = [&](int si, const KIn& cur, KIn& nxt) {
    const int c0 = (zs * NSW + si) * SW;
    {
      const bool live = row < cl.len;
#pragma unroll
      for (int i = 0; i < CPT; ++i) qs[row * PS + c8 + i] = live ? cur.xq[i] : 0.f, ks[row * PS + c8 + i] = live ? cur.xk[i] : 0.f;
#pragma unroll
      for (int i = 0; i < RPS; ++i) {
        const int rr = gseg * RPS + i;
        gs[rr * PS + gch] = rr < cl.len ? cur.xg[i] : 0.f;
      }
    }
    lds_sync();
    if (si + 1 < NSW) issue(c0 + SW, nxt);  // this slice's inputs are in LDS or kept in cur
    row_scan<false, PS, SW>(gs, tot);
    // scaled operands of the off-diagonal block pairs
    for (int e = tid; e < 96 * SW; e += 256) {
      const int r96 = e / SW, ch = e % SW;
      {
        const int Ib = r96 < 16 ? 1 : (r96 < 48 ? 2 : 3);
        const int s = r96 - (Ib == 1 ? 0 : (Ib == 2 ? 16 : 48));
        Ksc[r96 * PS + ch] = ks[s * PS + ch] * __expf(gs[(16 * Ib - 1) * PS + ch] - gs[s * PS + ch]);
      }
      {
        const int Jb = r96 < 48 ? 0 : (r96 < 80 ? 1 : 2);
        const int rr = 16 * Jb + 16 + r96 - (Jb == 0 ? 0 : (Jb == 1 ? 48 : 80));
        const float E = __expf(gs[rr * PS + ch] - gs[(16 * Jb + 15) * PS + ch]);
        Xq[r96 * PS + ch] = qs[rr * PS + ch] * E;
        Xk[r96 * PS + ch] = ks[rr * PS + ch] * E;
      }
    }
    lds_sync();
    float GQ[CPT], GA[CPT], G2[CPT], Gr[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) Gr[i] = gs[row * PS + c8 + i];
    // A channel whose decay across the wave's block is within range has the
    // block's own pairs on the MFMA path too; one that decays faster takes
    // them pair by pair (below).
    const float gpre = I > 0 ? gs[(16 * I - 1) * PS + ln] : 0.f, gend = gs[(16 * I + 15) * PS + ln];
    const bool inr = gpre - gend <= kBwdDiagRange;  // channel ln (the MFMA row operand's)
    bool bad[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      bad[i] = (I > 0 ? gs[(16 * I - 1) * PS + c8 + i] : 0.f) - gs[(16 * I + 15) * PS + c8 + i] > kBwdDiagRange;
    // Block pairs on fp32 MFMA (exact fp32 products), each computed
    // transposed, C^T = X^T D^T, so that output lane l holds row l % 16 and
    // channels 4 (l / 16) .. + 3: this thread's.  Row side over the rows
    // s < r up to the wave's block (operands scaled at row 16 I - 1: the
    // earlier blocks' from LDS, the block's own formed here, masked to s < r),
    // column side over the rows r > s from the wave's block on (scaled at
    // row 16 I + 15; the block's own masked to r > s); the block index is
    // the wave's, so the k loops are uniform.
    {
      const int off = I == 1 ? 0 : (I == 2 ? 16 : 48);
      f32x4 aq = zero4(), aa = zero4();
      for (int kq = 0; kq < 4 * I; ++kq) {
        const int s = 4 * kq + lg;
        const float a = Ksc[(off + s) * PS + ln];
        aq = mf(a, dPl[(16 * I + ln) * LPC + s], aq);
        aa = mf(a, dAl[(16 * I + ln) * LPC + s], aa);
      }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int sl = 4 * kq + lg, s = 16 * I + sl;
        const float a = inr ? ks[s * PS + ln] * __expf(gpre - gs[s * PS + ln]) : 0.f;
        const bool lower = sl < ln;
        aq = mf(a, lower ? dPl[(16 * I + ln) * LPC + s] : 0.f, aq);
        aa = mf(a, lower ? dAl[(16 * I + ln) * LPC + s] : 0.f, aa);
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const float sc_ = __expf(Gr[i] - (I > 0 ? gs[(16 * I - 1) * PS + c8 + i] : 0.f));
        GQ[i] = aq[i] * sc_;
        GA[i] = aa[i] * sc_;
      }
    }
    // column side (this thread's row is the column index s)
    {
      const int off = I == 0 ? 0 : (I == 1 ? 48 : 80);
      f32x4 a2 = zero4();
      for (int kq = 0; kq < 12 - 4 * I; ++kq) {
        const int rp = 4 * kq + lg, rr = 16 * I + 16 + rp;
        a2 = mf(Xq[(off + rp) * PS + ln], dPl[rr * LPC + 16 * I + ln], a2);
        a2 = mf(Xk[(off + rp) * PS + ln], dAl[rr * LPC + 16 * I + ln], a2);
      }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int rl = 4 * kq + lg, rr = 16 * I + rl;
        const float E = inr ? __expf(gs[rr * PS + ln] - gend) : 0.f;
        const bool upper = rl > ln;
        a2 = mf(qs[rr * PS + ln] * E, upper ? dPl[rr * LPC + 16 * I + ln] : 0.f, a2);
        a2 = mf(ks[rr * PS + ln] * E, upper ? dAl[rr * LPC + 16 * I + ln] : 0.f, a2);
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) G2[i] = a2[i] * __expf(gs[(16 * I + 15) * PS + c8 + i] - Gr[i]);
    }
    // the block's own pairs, one by one, for the channels out of range
    if (__ballot(bad[0] || bad[1] || bad[2] || bad[3])) {
      for (int s = 16 * I; s < row; ++s) {
        const float dp = dPl[row * LPC + s], da = dAl[row * LPC + s];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          if (bad[i]) {
            const float kE = ks[s * PS + c8 + i] * __expf(Gr[i] - gs[s * PS + c8 + i]);
            GQ[i] += dp * kE;
            GA[i] += da * kE;
          }
        }
      }
      for (int rr = row + 1; rr < 16 * I + 16; ++rr) {
        const float dp = dPl[rr * LPC + row], da = dAl[rr * LPC + row];
#pragma unroll
        for (int i = 0; i < CPT; ++i)
          if (bad[i])
            G2[i] += (dp * qs[rr * PS + c8 + i] + da * ks[rr * PS + c8 + i]) * __expf(gs[rr * PS + c8 + i] - Gr[i]);
      }
    }
    // elementwise
    float dqv[CPT], dkv[CPT], dG[CPT], cs[CPT];
    // The pair s = r enters P with factor 1 and its contributions to dG
    // (q_r dP_rr k_r - k_r dP_rr q_r) cancel exactly, as do the last token's
    // own dKb Kb terms (its factor e^{G_C - G_r} is 1; in a partial chunk the
    // last token is row len - 1, the rows after it have no decay): both are
    // left out of dG rather than added and subtracted, which would leave
    // rounding error of the size of the terms where the true dG is tiny
    // (strong decay).
    const float dpd = dPl[row * LPC + row];
    const bool last = row == BC - 1 || row == cl.len - 1;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const float qv = qs[row * PS + c8 + i], kv = ks[row * PS + c8 + i];
      const float eg = __expf(Gr[i]), eb = __expf(gs[(BC - 1) * PS + c8 + i] - Gr[i]);
      dqv[i] = cur.dQg[i] * eg + GQ[i] + dpd * kv;
      dkv[i] = cur.dKg[i] * eg + cur.dKb[i] * eb + GA[i] + G2[i] + dpd * qv;
      cs[i] = last ? 0.f : cur.dKb[i] * kv * eb;
      dG[i] = (cur.dQg[i] * qv + cur.dKg[i] * kv) * eg - cs[i] + qv * GQ[i] + kv * (GA[i] - G2[i]);
    }
    if (row < cl.len) {
      const size_t o = (static_cast<size_t>(cl.t0 + row) * H + h) * DK + c0 + c8;
      storen<CPT>(dq + o, dqv);
      storen<CPT>(dk + o, dkv);
    }
    if constexpr (G != KDA_GATE_NONE) {
      lds_sync();  // every reader of qs and Xk is done
#pragma unroll
      for (int i = 0; i < CPT; ++i) qs[row * PS + c8 + i] = dG[i], Xk[row * PS + c8 + i] = cs[i];
      lds_sync();
      if (tid < SW) {  // G_C: the column sum of dKb Kb over the other rows (fixed order), dgamma gamma
        float x = 0.f;
        for (int rr = 0; rr < BC; ++rr) x += Xk[rr * PS + tid];
        qs[(BC - 1) * PS + tid] += x + bk[B::odGam + c0 + tid] * __expf(gs[(BC - 1) * PS + tid]);
      }
      lds_sync();
      row_scan<true, PS, SW>(qs, tot);
      if constexpr (G == KDA_GATE_CHANNEL) {
        if (row < cl.len) {
          float x[CPT];
#pragma unroll
          for (int i = 0; i < CPT; ++i) x[i] = qs[row * PS + c8 + i];
          storen<CPT>(dla + (static_cast<size_t>(cl.t0 + row) * H + h) * DK + c0 + c8, x);
        }
      } else {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) x += qs[row * PS + c8 + i];
        x += shfl_xor(x, 16);  // the row's four threads are lanes l % 16 + 16 j
        x += shfl_xor(x, 32);
        if (lg == 0) rsum[row] += x;
      }
    }
    lds_sync();
    };
  static_assert(NSW % 2 == 0, "slices taken two at a time");
  for (int si = 0; si < NSW; si += 2) {
    slice(si, ina, inb);
    slice(si + 1, inb, ina);
  }
  if constexpr (G == KDA_GATE_SCALAR) {
    if (tid < cl.len) dla[static_cast<size_t>(cl.t0 + tid) * H + h] = rsum[tid];
  }
}

}  // namespace
}  // namespace kda

namespace kda {

static size_t align256b(size_t x) { return (x + 255) / 256 * 256; }

bool make_backward_plan(const kda_prefill_desc* d, int64_t max_chunks, BackwardPlan* p) {
  p->N = d->num_seqs;
  p->T = d->total_tokens;
  p->H = d->num_heads;
  p->dk = d->dk;
  p->dv = d->dv;
  p->dt = d->io_dtype;
  p->gate = d->gate;
  p->max_chunks = max_chunks;
  p->sort = d->num_seqs <= 8192;
  const size_t slots = static_cast<size_t>(max_chunks) * d->num_heads;
  size_t off = 0;
  p->off_chunk_off = off; off = align256b(off + 4 * (static_cast<size_t>(d->num_seqs) + 1));
  p->off_order = off;     off = align256b(off + 4 * (static_cast<size_t>(d->num_seqs) + 1));
  p->off_blocks = off;    off = align256b(off + slots * blk_floats(d->dk) * 4);
  p->off_states = off;    off = align256b(off + slots * d->dk * d->dv * 4);
  p->off_dstates = off;   off = align256b(off + slots * d->dk * d->dv * 4);
  p->total_bytes = off;
  return true;
}

template <typename T, int DK, int DV, int G>
static hipError_t launch_backward_t(const BackwardPlan& p, const void* q, const void* k, const void* v,
                                    const float* la, const float* beta, const int32_t* cu, const float* S0,
                                    const void* dO, const float* dS_T, void* dq, void* dk, void* dv, float* dla,
                                    float* dbeta, float* dS0, void* ws, hipStream_t st) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(w + p.off_chunk_off);
  int32_t* order = reinterpret_cast<int32_t*>(w + p.off_order);
  float* blk = reinterpret_cast<float*>(w + p.off_blocks);
  float* sc = reinterpret_cast<float*>(w + p.off_states);
  float* dsc = reinterpret_cast<float*>(w + p.off_dstates);
  hipError_t e = launch_chunk_offsets(cu, p.N, BC, chunk_off, order, p.sort, st);
  if (e != hipSuccess) return e;
  const unsigned mc = static_cast<unsigned>(p.max_chunks);
  const T* tq = static_cast<const T*>(q);
  const T* tk = static_cast<const T*>(k);
  const T* tv = static_cast<const T*>(v);
  const T* tdo = static_cast<const T*>(dO);
  if (mc > 0) {
    hipLaunchKernelGGL((bwd_prep_kernel<T, DK, G>), dim3(mc, p.H), dim3(256), 0, st, tq, tk, la, beta, cu, chunk_off,
                       p.N, p.H, blk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t NH = static_cast<int64_t>(p.N) * p.H;
  const unsigned seq_wgs = static_cast<unsigned>((NH + 7) / 8 * 8 * (DV / SCOLS));
  hipLaunchKernelGGL((bwd_states_kernel<T, DK, DV>), dim3(2 * seq_wgs), dim3(256), 0, st, tv, tdo, cu, chunk_off,
                     order, p.N, p.H, blk, S0, dS_T, sc, dsc, dS0, static_cast<int>(seq_wgs));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (mc > 0) {
    // persistent: one workgroup per CU (its LDS allows no more), each walking
    // the (chunk, head) items gridDim apart
    int cus = 0;
    if ((e = device_cus(&cus)) != hipSuccess) return e;
    const unsigned gv = static_cast<unsigned>(std::min<int64_t>(static_cast<int64_t>(mc) * p.H, cus));
    hipLaunchKernelGGL((bwd_grad_v_kernel<T, DK, DV>), dim3(gv), dim3(256), 0, st, tv, tdo, cu, chunk_off, p.N, p.H,
                       blk, sc, dsc, static_cast<T*>(dv), dbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    constexpr int SW = 16;  // key channels per grad_k slice (LDS for two workgroups per CU)
    const unsigned nz = 1u;  // one workgroup per (chunk, head): every channel slice inside it
    const unsigned items = (mc * static_cast<unsigned>(p.H) + 7u) / 8u * 8u;
    hipLaunchKernelGGL((bwd_grad_k_kernel<T, DK, G, SW>), dim3(items * nz), dim3(256), 0, st, tq, tk, la, cu,
                       chunk_off, p.N, p.H, blk, static_cast<T*>(dq), static_cast<T*>(dk), dla);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int DK, int DV>
static hipError_t backward_gate(const BackwardPlan& p, const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const int32_t* cu, const float* S0, const void* dO,
                                const float* dS_T, void* dq, void* dk, void* dv, float* dla, float* dbeta,
                                float* dS0, void* ws, hipStream_t st) {
  if (p.gate == KDA_GATE_CHANNEL)
    return launch_backward_t<T, DK, DV, KDA_GATE_CHANNEL>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla,
                                                          dbeta, dS0, ws, st);
  if (p.gate == KDA_GATE_SCALAR)
    return launch_backward_t<T, DK, DV, KDA_GATE_SCALAR>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla,
                                                         dbeta, dS0, ws, st);
  return launch_backward_t<T, DK, DV, KDA_GATE_NONE>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla, dbeta,
                                                     dS0, ws, st);
}

template <typename T>
static hipError_t backward_dims(const BackwardPlan& p, const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const int32_t* cu, const float* S0, const void* dO,
                                const float* dS_T, void* dq, void* dk, void* dv, float* dla, float* dbeta,
                                float* dS0, void* ws, hipStream_t st) {
  if (p.dk == 128 && p.dv == 128)
    return backward_gate<T, 128, 128>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla, dbeta, dS0, ws, st);
  if (p.dk == 128 && p.dv == 64)
    return backward_gate<T, 128, 64>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla, dbeta, dS0, ws, st);
  if (p.dk == 64 && p.dv == 128)
    return backward_gate<T, 64, 128>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla, dbeta, dS0, ws, st);
  return backward_gate<T, 64, 64>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla, dbeta, dS0, ws, st);
}

hipError_t launch_backward(const BackwardPlan& p, const void* q, const void* k, const void* v, const float* la,
                           const float* beta, const int32_t* cu, const float* S0, const void* dO, const float* dS_T,
                           void* dq, void* dk, void* dv, float* dla, float* dbeta, float* dS0, void* workspace,
                           hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  if (p.dt == KDA_BF16)
    return backward_dims<bf16_t>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla, dbeta, dS0, workspace,
                                 stream);
  return backward_dims<float>(p, q, k, v, la, beta, cu, S0, dO, dS_T, dq, dk, dv, dla, dbeta, dS0, workspace,
                              stream);
}

}  // namespace kda
