// kda_decode.hip -- batched single-token KDA state update (decode), gfx950.
//
// For each (request b, head h) with fp32 state S (dk x dv, row = key channel):
//   S~ = Diag(exp(log_alpha)) S                 per-key-channel forget
//   r  = S~^T k                                 read-back along the key
//   d  = beta (v - r)                           delta-rule correction
//   S' = S~ + k d^T                             erase-and-write in one rank-1 update
//   o  = S'^T q = S~^T q + d (k^T q)
// which is S' = (I - beta k k^T) Diag(alpha) S + beta k v^T, the KDA update of
// the "Kimi Linear" deep-read report (zako-mio knowledge base), section 2.3.
// Every value column j of S evolves independently (r_j, d_j, o_j use only
// column j), so the state can be split by columns without communication.
//
// Mapping.  One workgroup per (b, h, slice of CW = min(64, dv) value
// columns); its waves split the key rows, kNR = 2 consecutive rows per lane.
// Lane l of a wave owns 4 adjacent columns (l mod CW/4) and its rows' state
// values stay in VGPRs for the whole step; one float4 load instruction of a
// wave covers 256 / CW rows x 4 CW contiguous bytes (whole 128-byte lines),
// the lane's gates, k and q come in one load each, and the state is read
// once and written once.  The column sums (S~^T k, S~^T q) and k^T q are
// reduced over the row phases of a wave with xor shuffles, then over the
// waves through LDS (one barrier).  Shape choice (in-place 512 MiB stream,
// measured): few loads per lane and row pieces of at least 256 bytes per
// instruction matter most — 16 float4 loads per lane in one 64 KiB
// workgroup per state ran 13% slower, 32-column slices (128-byte pieces)
// 7% slower, 16-column slices twice as slow.  The kernel is HBM-bound:
// 2 * 4 * dk * dv bytes of state per update against ~4 * dk * dv flops.
//
// Gate forms (template G): one rate per key row (KDA), one rate for the
// whole state (Gated DeltaNet: one 4-byte load and one exponential), or none
// (DeltaNet: the decay is skipped).

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kNR = 2;   // key rows per lane
constexpr int kCW = 64;  // value columns per workgroup (at most dv)

template <int DV>
struct DecodeShape {
  static constexpr int CW = kCW < DV ? kCW : DV;
  static constexpr int LPR = CW / 4;   // lanes per key row (4 columns each)
  static constexpr int RPI = 64 / LPR;  // key rows per wave load instruction
};

// kNR consecutive elements, loaded with one instruction
template <typename T>
struct alignas(sizeof(T) * kNR) RowPack {
  T x[kNR];
};

template <typename T, int DK, int DV, int G>
__global__ __launch_bounds__(DK / kNR * DecodeShape<DV>::LPR) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                              const T* __restrict__ v, const float* __restrict__ la,
                                                              const float* __restrict__ beta, float* __restrict__ S,
                                                              T* __restrict__ o) {
  typedef DecodeShape<DV> DS;
  constexpr int RW = DK / (DS::RPI * kNR);  // row waves per workgroup
  constexpr int NS = DV / DS::CW;           // column slices per state
  __shared__ f32x4 red[RW][2][DS::LPR];     // per wave: S~^T k and S~^T q of its rows
  __shared__ float redkq[RW];            // per wave: k^T q of its rows
  const int bh = blockIdx.x / NS;
  const int slice = blockIdx.x % NS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c4 = lane % DS::LPR;
  const int row0 = (wave * DS::RPI + lane / DS::LPR) * kNR;
  const int col = slice * DS::CW + c4 * 4;

  float* Sb = S + static_cast<size_t>(bh) * DK * DV;
  const T* qb = q + static_cast<size_t>(bh) * DK;
  const T* kb = k + static_cast<size_t>(bh) * DK;

  f32x4 s[kNR];
#pragma unroll
  for (int i = 0; i < kNR; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (row0 + i) * DV + col));

  float alpha[kNR];
  if constexpr (G == KDA_GATE_CHANNEL) {
    const RowPack<float> lr = *reinterpret_cast<const RowPack<float>*>(la + static_cast<size_t>(bh) * DK + row0);
#pragma unroll
    for (int i = 0; i < kNR; ++i) alpha[i] = __expf(lr.x[i]);
  } else if constexpr (G == KDA_GATE_SCALAR) {
    const float a = __expf(la[bh]);
#pragma unroll
    for (int i = 0; i < kNR; ++i) alpha[i] = a;
  }
  const RowPack<T> kp = *reinterpret_cast<const RowPack<T>*>(kb + row0);
  const RowPack<T> qp = *reinterpret_cast<const RowPack<T>*>(qb + row0);
  float kr[kNR];
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  f32x4 sq = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < kNR; ++i) {
    const float kk = io<T>::load(&kp.x[i]);
    const float qq = io<T>::load(&qp.x[i]);
    if constexpr (G != KDA_GATE_NONE) s[i] *= alpha[i];
    r += kk * s[i];
    sq += qq * s[i];
    kq += kk * qq;
    kr[i] = kk;
  }
#pragma unroll
  for (int m = DS::LPR; m < 64; m <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] += shfl_xor(r[c], m);
      sq[c] += shfl_xor(sq[c], m);
    }
    kq += shfl_xor(kq, m);
  }
  if (lane < DS::LPR) {
    red[wave][0][c4] = r;
    red[wave][1][c4] = sq;
    if (lane == 0) redkq[wave] = kq;
  }
  const f32x4 vv = load4(v + static_cast<size_t>(bh) * DV + col);
  const float b = beta[bh];
  __syncthreads();
  r = red[0][0][c4];
  sq = red[0][1][c4];
  kq = redkq[0];
#pragma unroll
  for (int w = 1; w < RW; ++w) {
    r += red[w][0][c4];
    sq += red[w][1][c4];
    kq += redkq[w];
  }
  const f32x4 d = b * (vv - r);
#pragma unroll
  for (int i = 0; i < kNR; ++i) {
    s[i] += kr[i] * d;
    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Sb + (row0 + i) * DV + col));
  }
  if (threadIdx.x < DS::LPR) store4(o + static_cast<size_t>(bh) * DV + col, sq + d * kq);
}

template <typename T, int DK, int DV, int G>
static hipError_t launch_decode_t(int BH, const void* q, const void* k, const void* v, const float* la,
                                  const float* beta, float* S, void* o, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<T, DK, DV, G>), dim3(BH * (DV / DecodeShape<DV>::CW)),
                     dim3(DK / kNR * DecodeShape<DV>::LPR), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), la, beta, S,
                     static_cast<T*>(o));
  return hipGetLastError();
}

template <typename T, int G>
static hipError_t launch_decode_dt(int dk, int dv, int BH, const void* q, const void* k, const void* v,
                                   const float* la, const float* beta, float* S, void* o, hipStream_t st) {
  if (dk == 128 && dv == 128) return launch_decode_t<T, 128, 128, G>(BH, q, k, v, la, beta, S, o, st);
  if (dk == 128 && dv == 64) return launch_decode_t<T, 128, 64, G>(BH, q, k, v, la, beta, S, o, st);
  if (dk == 64 && dv == 128) return launch_decode_t<T, 64, 128, G>(BH, q, k, v, la, beta, S, o, st);
  if (dk == 64 && dv == 64) return launch_decode_t<T, 64, 64, G>(BH, q, k, v, la, beta, S, o, st);
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_gate(kda_gate g, int dk, int dv, int BH, const void* q, const void* k, const void* v,
                                     const float* la, const float* beta, float* S, void* o, hipStream_t st) {
  if (g == KDA_GATE_CHANNEL) return launch_decode_dt<T, KDA_GATE_CHANNEL>(dk, dv, BH, q, k, v, la, beta, S, o, st);
  if (g == KDA_GATE_SCALAR) return launch_decode_dt<T, KDA_GATE_SCALAR>(dk, dv, BH, q, k, v, la, beta, S, o, st);
  return launch_decode_dt<T, KDA_GATE_NONE>(dk, dv, BH, q, k, v, la, beta, S, o, st);
}

hipError_t launch_decode(kda_dtype dt, kda_gate gate, int dk, int dv, int BH, const void* q, const void* k,
                         const void* v, const float* la, const float* beta, float* S, void* o, hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (dt == KDA_BF16) return launch_decode_gate<bf16_t>(gate, dk, dv, BH, q, k, v, la, beta, S, o, stream);
  return launch_decode_gate<float>(gate, dk, dv, BH, q, k, v, la, beta, S, o, stream);
}

}  // namespace kda
