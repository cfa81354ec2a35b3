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

// Shape of the decode mapping.  The plain form covers CW = min(64, dv)
// value columns per workgroup with NR = 2 key rows per lane; the staged form
// (input/output stages) takes a whole state per workgroup (CW = dv, NR rows
// per lane so that it stays within 1024 threads), because its head-wise norm
// spans every value column.
template <int DK, int DV, bool STG>
struct DecodeShape {
  static constexpr int CW = STG ? DV : (64 < DV ? 64 : DV);
  static constexpr int LPR = CW / 4;    // lanes per key row (4 columns each)
  static constexpr int RPI = 64 / LPR;  // key rows per wave load instruction
  static constexpr int NR = (STG && DK * LPR / 1024 > 2) ? DK * LPR / 1024 : 2;  // key rows per lane
  static constexpr int THREADS = DK / NR * LPR;
};

// NR consecutive elements, loaded with one instruction
template <typename T, int NR>
struct alignas(sizeof(T) * NR) RowPack {
  T x[NR];
};

// Stage arguments of the staged form (see kda_stages).
template <typename T>
struct DecodeStages {
  int l2norm, softplus_gate;
  float l2eps, norm_eps;
  const float* norm_weight;
  const T* out_gate;
};

template <typename T, int DK, int DV, int G, bool STG>
__global__ __launch_bounds__((DecodeShape<DK, DV, STG>::THREADS)) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ la,
    const float* __restrict__ beta, float* __restrict__ S, T* __restrict__ o, DecodeStages<T> stg) {
  typedef DecodeShape<DK, DV, STG> DS;
  constexpr int NR = DS::NR;
  constexpr int RW = DK / (DS::RPI * NR);  // row waves per workgroup
  constexpr int NS = DV / DS::CW;          // column slices per state
  __shared__ f32x4 red[RW][2][DS::LPR];    // per wave: S~^T k and S~^T q of its rows
  __shared__ float redkq[RW][3];           // per wave: k^T q, |k|^2, |q|^2 of its rows
  const int bh = blockIdx.x / NS;
  const int slice = blockIdx.x % NS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c4 = lane % DS::LPR;
  const int row0 = (wave * DS::RPI + lane / DS::LPR) * NR;
  const int col = slice * DS::CW + c4 * 4;

  float* Sb = S + static_cast<size_t>(bh) * DK * DV;
  const T* qb = q + static_cast<size_t>(bh) * DK;
  const T* kb = k + static_cast<size_t>(bh) * DK;

  f32x4 s[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (row0 + i) * DV + col));

  // gate: log alpha, or -softplus of the gate projection's output (staged)
  auto log_alpha = [&](float x) { return (STG && stg.softplus_gate) ? neg_softplus(x) : x; };
  float alpha[NR];
  if constexpr (G == KDA_GATE_CHANNEL) {
    const RowPack<float, NR> lr = *reinterpret_cast<const RowPack<float, NR>*>(la + static_cast<size_t>(bh) * DK + row0);
#pragma unroll
    for (int i = 0; i < NR; ++i) alpha[i] = __expf(log_alpha(lr.x[i]));
  } else if constexpr (G == KDA_GATE_SCALAR) {
    const float a = __expf(log_alpha(la[bh]));
#pragma unroll
    for (int i = 0; i < NR; ++i) alpha[i] = a;
  }
  const RowPack<T, NR> kp = *reinterpret_cast<const RowPack<T, NR>*>(kb + row0);
  const RowPack<T, NR> qp = *reinterpret_cast<const RowPack<T, NR>*>(qb + row0);
  float kr[NR];
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  f32x4 sq = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f, kk2 = 0.f, qq2 = 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const float kk = io<T>::load(&kp.x[i]);
    const float qq = io<T>::load(&qp.x[i]);
    if constexpr (G != KDA_GATE_NONE) s[i] *= alpha[i];
    r += kk * s[i];
    sq += qq * s[i];
    kq += kk * qq;
    if constexpr (STG) {
      kk2 += kk * kk;
      qq2 += qq * qq;
    }
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
    if constexpr (STG) {
      kk2 += shfl_xor(kk2, m);
      qq2 += shfl_xor(qq2, m);
    }
  }
  if (lane < DS::LPR) {
    red[wave][0][c4] = r;
    red[wave][1][c4] = sq;
    if (lane == 0) {
      redkq[wave][0] = kq;
      redkq[wave][1] = kk2;
      redkq[wave][2] = qq2;
    }
  }
  const f32x4 vv = load4(v + static_cast<size_t>(bh) * DV + col);
  const float b = beta[bh];
  __syncthreads();
  r = red[0][0][c4];
  sq = red[0][1][c4];
  kq = redkq[0][0];
  if constexpr (STG) {
    kk2 = redkq[0][1];
    qq2 = redkq[0][2];
  }
#pragma unroll
  for (int w = 1; w < RW; ++w) {
    r += red[w][0][c4];
    sq += red[w][1][c4];
    kq += redkq[w][0];
    if constexpr (STG) {
      kk2 += redkq[w][1];
      qq2 += redkq[w][2];
    }
  }
  if constexpr (STG) {
    // input stage: every product with k or q was formed with the raw vectors
    // and is linear in them, so the norms are applied now
    if (stg.l2norm) {
      const float ik = 1.f / fmaxf(__builtin_sqrtf(kk2), stg.l2eps), iq = 1.f / fmaxf(__builtin_sqrtf(qq2), stg.l2eps);
      r *= ik;
      sq *= iq;
      kq *= ik * iq;
#pragma unroll
      for (int i = 0; i < NR; ++i) kr[i] *= ik;
    }
  }
  const f32x4 d = b * (vv - r);
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    s[i] += kr[i] * d;
    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Sb + (row0 + i) * DV + col));
  }
  if (wave == 0) {
    f32x4 y = sq + d * kq;
    if constexpr (STG) {
      // output stage: each group of LPR lanes of wave 0 holds the whole
      // output row (the groups hold copies); the reductions stay in a group
      if (stg.norm_weight) {
        float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
#pragma unroll
        for (int m = 1; m < DS::LPR; m <<= 1) ss += shfl_xor(ss, m);
        const float rs = 1.f / __builtin_sqrtf(ss * (1.f / DV) + stg.norm_eps);
        y *= rs * *reinterpret_cast<const f32x4*>(stg.norm_weight + col);
      }
      if (stg.out_gate) {
        const f32x4 z = load4(stg.out_gate + static_cast<size_t>(bh) * DV + col);
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] *= 1.f / (1.f + __expf(-z[j]));
      }
    }
    if (lane < DS::LPR) store4(o + static_cast<size_t>(bh) * DV + col, y);
  }
}

template <typename T, int DK, int DV, int G, bool STG>
static hipError_t launch_decode_t(int BH, const void* q, const void* k, const void* v, const float* la,
                                  const float* beta, float* S, void* o, const DecodeStages<T>& stg, hipStream_t st) {
  typedef DecodeShape<DK, DV, STG> DS;
  hipLaunchKernelGGL((decode_kernel<T, DK, DV, G, STG>), dim3(BH * (DV / DS::CW)), dim3(DS::THREADS), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), la, beta, S,
                     static_cast<T*>(o), stg);
  return hipGetLastError();
}

template <typename T, int G, bool STG>
static hipError_t launch_decode_dt(int dk, int dv, int BH, const void* q, const void* k, const void* v,
                                   const float* la, const float* beta, float* S, void* o, const DecodeStages<T>& stg,
                                   hipStream_t st) {
  if (dk == 128 && dv == 128) return launch_decode_t<T, 128, 128, G, STG>(BH, q, k, v, la, beta, S, o, stg, st);
  if (dk == 128 && dv == 64) return launch_decode_t<T, 128, 64, G, STG>(BH, q, k, v, la, beta, S, o, stg, st);
  if (dk == 64 && dv == 128) return launch_decode_t<T, 64, 128, G, STG>(BH, q, k, v, la, beta, S, o, stg, st);
  if (dk == 64 && dv == 64) return launch_decode_t<T, 64, 64, G, STG>(BH, q, k, v, la, beta, S, o, stg, st);
  return hipErrorInvalidValue;
}

template <typename T, bool STG>
static hipError_t launch_decode_gate(kda_gate g, int dk, int dv, int BH, const void* q, const void* k, const void* v,
                                     const float* la, const float* beta, float* S, void* o,
                                     const DecodeStages<T>& stg, hipStream_t st) {
  if (g == KDA_GATE_CHANNEL)
    return launch_decode_dt<T, KDA_GATE_CHANNEL, STG>(dk, dv, BH, q, k, v, la, beta, S, o, stg, st);
  if (g == KDA_GATE_SCALAR)
    return launch_decode_dt<T, KDA_GATE_SCALAR, STG>(dk, dv, BH, q, k, v, la, beta, S, o, stg, st);
  return launch_decode_dt<T, KDA_GATE_NONE, STG>(dk, dv, BH, q, k, v, la, beta, S, o, stg, st);
}

template <typename T>
static hipError_t launch_decode_io(kda_gate g, const kda_stages* sg, int dk, int dv, int BH, const void* q,
                                   const void* k, const void* v, const float* la, const float* beta, float* S,
                                   void* o, hipStream_t st) {
  DecodeStages<T> stg{};
  const bool staged = sg && (sg->l2norm_qk || (sg->gate_softplus && g != KDA_GATE_NONE) || sg->norm_weight ||
                             sg->out_gate);
  if (!staged) return launch_decode_gate<T, false>(g, dk, dv, BH, q, k, v, la, beta, S, o, stg, st);
  stg.l2norm = sg->l2norm_qk ? 1 : 0;
  stg.softplus_gate = sg->gate_softplus ? 1 : 0;
  stg.l2eps = sg->l2norm_eps;
  stg.norm_eps = sg->norm_eps;
  stg.norm_weight = sg->norm_weight;
  stg.out_gate = static_cast<const T*>(sg->out_gate);
  return launch_decode_gate<T, true>(g, dk, dv, BH, q, k, v, la, beta, S, o, stg, st);
}

hipError_t launch_decode(kda_dtype dt, kda_gate gate, const kda_stages* stages, int dk, int dv, int BH,
                         const void* q, const void* k, const void* v, const float* la, const float* beta, float* S,
                         void* o, hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (dt == KDA_BF16) return launch_decode_io<bf16_t>(gate, stages, dk, dv, BH, q, k, v, la, beta, S, o, stream);
  return launch_decode_io<float>(gate, stages, dk, dv, BH, q, k, v, la, beta, S, o, stream);
}

}  // namespace kda
