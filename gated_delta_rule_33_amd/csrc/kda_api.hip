// kda_api.hip -- the extern "C" boundary of libkda: host-side validation,
// workspace sizing and launch orchestration.  Kernels live in kda_decode.hip
// and kda_prefill.hip.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "kda.h"
#include "kda_internal.h"

namespace {

bool dims_supported(int32_t dk, int32_t dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128); }
bool dtype_valid(kda_dtype dt) { return dt == KDA_F32 || dt == KDA_BF16; }
size_t io_size(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

struct Range {
  uintptr_t b, e;
};
Range range(const void* p, size_t bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return Range{b, b + bytes};
}
bool overlap(Range x, Range y) { return x.b != x.e && y.b != y.e && x.b < y.e && y.b < x.e; }

// Checks the shape fields; fills the exact chunk count when host offsets exist.
kda_status check_desc(const kda_prefill_desc* d, int64_t* max_chunks) {
  if (!d) return KDA_ERR_INVALID_ARGUMENT;
  if (d->num_seqs < 0 || d->total_tokens < 0 || d->num_heads < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (!dtype_valid(d->io_dtype)) return KDA_ERR_INVALID_ARGUMENT;
  if (!dims_supported(d->dk, d->dv)) return KDA_ERR_UNSUPPORTED;
  if (d->chunk != 32 && d->chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0 && d->total_tokens != 0) return KDA_ERR_INVALID_ARGUMENT;
  const int64_t C = d->chunk;
  // one chunk of rows of any per-token tensor must span fewer than 2^31
  // bytes (the kernels use 32-bit offsets within a chunk)
  if (C * d->num_heads * (d->dk > d->dv ? d->dk : d->dv) * 4 >= (int64_t(1) << 31)) return KDA_ERR_UNSUPPORTED;
  if (d->cu_seqlens_host) {
    const int32_t* cu = d->cu_seqlens_host;
    if (cu[0] != 0) return KDA_ERR_INVALID_ARGUMENT;
    int64_t n = 0;
    for (int32_t i = 0; i < d->num_seqs; ++i) {
      if (cu[i + 1] < cu[i]) return KDA_ERR_INVALID_ARGUMENT;
      n += (static_cast<int64_t>(cu[i + 1]) - cu[i] + C - 1) / C;
    }
    if (cu[d->num_seqs] != d->total_tokens) return KDA_ERR_INVALID_ARGUMENT;
    *max_chunks = n;
  } else {
    // sum_i ceil(L_i / C) <= (T + N (C - 1)) / C
    *max_chunks = (static_cast<int64_t>(d->total_tokens) + static_cast<int64_t>(d->num_seqs) * (C - 1)) / C;
  }
  if (*max_chunks > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE";
  }
  return "KDA_ERR_UNKNOWN";
}

int32_t kda_version(void) { return 100; }

size_t kda_prefill_workspace_size(const kda_prefill_desc* d) {
  int64_t mc = 0;
  if (check_desc(d, &mc) != KDA_OK) return 0;
  kda::PrefillPlan p;
  if (!kda::make_prefill_plan(d, mc, &p)) return 0;
  return p.total_bytes;
}

kda_status kda_prefill(const kda_prefill_desc* d, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const int32_t* cu_seqlens, const float* S0,
                       void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
  int64_t mc = 0;
  const kda_status s = check_desc(d, &mc);
  if (s != KDA_OK) return s;
  if (d->num_seqs == 0) return KDA_OK;
  kda::PrefillPlan p;
  if (!kda::make_prefill_plan(d, mc, &p)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARGUMENT;
  const size_t T = static_cast<size_t>(d->total_tokens), H = static_cast<size_t>(d->num_heads);
  const size_t es = io_size(d->io_dtype);
  if (T > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_INVALID_ARGUMENT;
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < p.total_bytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
  const size_t state_bytes = static_cast<size_t>(d->num_seqs) * H * d->dk * d->dv * 4;
  const Range rq = range(q, T * H * d->dk * es), rk = range(k, T * H * d->dk * es),
              rv = range(v, T * H * d->dv * es), rla = range(log_alpha, T * H * d->dk * 4),
              rb = range(beta, T * H * 4), rcu = range(cu_seqlens, (static_cast<size_t>(d->num_seqs) + 1) * 4),
              rs0 = range(S0, S0 ? state_bytes : 0), ro = range(o, T * H * d->dv * es),
              rst = range(S_T, S_T ? state_bytes : 0), rws = range(workspace, p.total_bytes);
  // outputs must not overlap anything else (S_T may equal S0 exactly)
  const Range ins[] = {rq, rk, rv, rla, rb, rcu, rs0, rws};
  for (const Range& x : ins)
    if (overlap(ro, x)) return KDA_ERR_INVALID_ARGUMENT;
  const Range ins2[] = {rq, rk, rv, rla, rb, rcu, ro, rws};
  for (const Range& x : ins2)
    if (overlap(rst, x)) return KDA_ERR_INVALID_ARGUMENT;
  if (S_T && S0 && overlap(rst, rs0) && S_T != S0) return KDA_ERR_INVALID_ARGUMENT;
  const Range ins3[] = {rq, rk, rv, rla, rb, rcu, rs0};
  for (const Range& x : ins3)
    if (overlap(rws, x)) return KDA_ERR_INVALID_ARGUMENT;
  const hipError_t e = kda::launch_prefill(p, q, k, v, log_alpha, beta, cu_seqlens, S0, o, S_T, workspace,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

kda_status kda_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv, kda_dtype io_dtype, const void* q,
                           const void* k, const void* v, const float* log_alpha, const float* beta, float* S,
                           void* o, void* stream) {
  if (B < 0 || H < 1 || !dtype_valid(io_dtype)) return KDA_ERR_INVALID_ARGUMENT;
  if (!dims_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (!q || !k || !v || !log_alpha || !beta || !S || !o) return KDA_ERR_INVALID_ARGUMENT;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  const size_t es = io_size(io_dtype), n = static_cast<size_t>(BH);
  const Range rs = range(S, n * dk * dv * 4), ro = range(o, n * dv * es);
  const Range others[] = {range(q, n * dk * es), range(k, n * dk * es), range(v, n * dv * es),
                          range(log_alpha, n * dk * 4), range(beta, n * 4)};
  for (const Range& x : others)
    if (overlap(rs, x) || overlap(ro, x)) return KDA_ERR_INVALID_ARGUMENT;
  if (overlap(rs, ro)) return KDA_ERR_INVALID_ARGUMENT;
  const hipError_t e = kda::launch_decode(io_dtype, dk, dv, static_cast<int>(BH), q, k, v, log_alpha, beta, S, o,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

}  // extern "C"
