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
// Mapping.  One workgroup per (b, h); one wavefront per 32 value columns.
// Lane l of a wave owns 4 adjacent columns (l % 8) and the key rows
// (l / 8) + 8 i, i = 0 .. dk/8 - 1, held in VGPRs for the whole step: each
// float4 load instruction of the wave covers 8 rows x 128 contiguous bytes,
// i.e. whole 128-byte lines, and the state is read once and written once.
// The two column reductions (S~^T k and S~^T q) and k^T q run over the 8 row
// phases with cross-lane xor shuffles; there is no LDS and no barrier.
// The kernel is HBM-bound: 2 * 4 * dk * dv bytes of state per update against
// ~4 * dk * dv flops.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename T, int DK, int DV>
__global__ __launch_bounds__(DV * 2) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v, const float* __restrict__ la,
                                                        const float* __restrict__ beta, float* __restrict__ S,
                                                        T* __restrict__ o) {
  constexpr int NR = DK / 8;  // key rows per lane
  const int bh = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c4 = lane & 7;
  const int rph = lane >> 3;
  const int col = wave * 32 + c4 * 4;

  float* Sb = S + static_cast<size_t>(bh) * DK * DV;
  const T* qb = q + static_cast<size_t>(bh) * DK;
  const T* kb = k + static_cast<size_t>(bh) * DK;
  const float* lab = la + static_cast<size_t>(bh) * DK;

  f32x4 s[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (rph + 8 * i) * DV + col));

  float kr[NR];
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  f32x4 sq = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = rph + 8 * i;
    const float a = __expf(lab[row]);
    const float kk = io<T>::load(kb + row);
    const float qq = io<T>::load(qb + row);
    s[i] *= a;
    r += kk * s[i];
    sq += qq * s[i];
    kq += kk * qq;
    kr[i] = kk;
  }
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] += shfl_xor(r[c], m);
      sq[c] += shfl_xor(sq[c], m);
    }
    kq += shfl_xor(kq, m);
  }
  const f32x4 vv = load4(v + static_cast<size_t>(bh) * DV + col);
  const float b = beta[bh];
  const f32x4 d = b * (vv - r);
  const f32x4 out = sq + d * kq;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    s[i] += kr[i] * d;
    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Sb + (rph + 8 * i) * DV + col));
  }
  if (rph == 0) store4(o + static_cast<size_t>(bh) * DV + col, out);
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(int BH, const void* q, const void* k, const void* v, const float* la,
                                  const float* beta, float* S, void* o, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<T, DK, DV>), dim3(BH), dim3(DV * 2), 0, st, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v), la, beta, S, static_cast<T*>(o));
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dt(int dk, int dv, int BH, const void* q, const void* k, const void* v,
                                   const float* la, const float* beta, float* S, void* o, hipStream_t st) {
  if (dk == 128 && dv == 128) return launch_decode_t<T, 128, 128>(BH, q, k, v, la, beta, S, o, st);
  if (dk == 128 && dv == 64) return launch_decode_t<T, 128, 64>(BH, q, k, v, la, beta, S, o, st);
  if (dk == 64 && dv == 128) return launch_decode_t<T, 64, 128>(BH, q, k, v, la, beta, S, o, st);
  if (dk == 64 && dv == 64) return launch_decode_t<T, 64, 64>(BH, q, k, v, la, beta, S, o, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(kda_dtype dt, int dk, int dv, int BH, const void* q, const void* k, const void* v,
                         const float* la, const float* beta, float* S, void* o, hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (dt == KDA_BF16) return launch_decode_dt<bf16_t>(dk, dv, BH, q, k, v, la, beta, S, o, stream);
  return launch_decode_dt<float>(dk, dv, BH, q, k, v, la, beta, S, o, stream);
}

}  // namespace kda
