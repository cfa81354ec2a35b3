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
bool gate_valid(kda_gate g) { return g == KDA_GATE_CHANNEL || g == KDA_GATE_SCALAR || g == KDA_GATE_NONE; }
// log_alpha elements per (token, head)
size_t gate_width(kda_gate g, int32_t dk) { return g == KDA_GATE_CHANNEL ? dk : (g == KDA_GATE_SCALAR ? 1 : 0); }
size_t io_size(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

struct Range {
  uintptr_t b, e;
};
Range range(const void* p, size_t bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return Range{b, b + bytes};
}
bool overlap(Range x, Range y) { return x.b != x.e && y.b != y.e && x.b < y.e && y.b < x.e; }

// Stage arguments: epsilons must be positive where a stage uses them.
bool stages_valid(const kda_stages* s) {
  if (!s) return true;
  if (s->l2norm_qk && !(s->l2norm_eps > 0.f)) return false;
  if (s->norm_weight && !(s->norm_eps > 0.f)) return false;
  return true;
}

// Checks the shape fields; fills the exact chunk count when host offsets exist.
kda_status check_desc(const kda_prefill_desc* d, int64_t* max_chunks) {
  if (!d) return KDA_ERR_INVALID_ARGUMENT;
  if (d->num_seqs < 0 || d->total_tokens < 0 || d->num_heads < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (!dtype_valid(d->io_dtype) || !gate_valid(d->gate) || !stages_valid(d->stages)) return KDA_ERR_INVALID_ARGUMENT;
  if (!dims_supported(d->dk, d->dv)) return KDA_ERR_UNSUPPORTED;
  if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return KDA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0 && d->total_tokens != 0) return KDA_ERR_INVALID_ARGUMENT;
  if (d->flags & ~static_cast<uint32_t>(KDA_PREFILL_ONE_STREAM | KDA_PREFILL_BOUNDED)) return KDA_ERR_INVALID_ARGUMENT;
  const int64_t CL = d->chunk;                 // tokens per chunk
  const int64_t C = d->chunk < 32 ? 32 : d->chunk;  // rows of the kernels' chunk tiles
  // one chunk of rows of any per-token tensor must span fewer than 2^31
  // bytes (the kernels use 32-bit offsets within a chunk)
  if (C * d->num_heads * (d->dk > d->dv ? d->dk : d->dv) * 4 >= (int64_t(1) << 31)) return KDA_ERR_UNSUPPORTED;
  if (d->cu_seqlens_host) {
    const int32_t* cu = d->cu_seqlens_host;
    if (cu[0] != 0) return KDA_ERR_INVALID_ARGUMENT;
    int64_t n = 0;
    for (int32_t i = 0; i < d->num_seqs; ++i) {
      if (cu[i + 1] < cu[i]) return KDA_ERR_INVALID_ARGUMENT;
      n += (static_cast<int64_t>(cu[i + 1]) - cu[i] + CL - 1) / CL;
    }
    if (cu[d->num_seqs] != d->total_tokens) return KDA_ERR_INVALID_ARGUMENT;
    *max_chunks = n;
  } else {
    // sum_i ceil(L_i / CL) <= (T + N (CL - 1)) / CL
    *max_chunks = (static_cast<int64_t>(d->total_tokens) + static_cast<int64_t>(d->num_seqs) * (CL - 1)) / CL;
  }
  if (*max_chunks > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

}  // namespace

namespace kda {

kda_status prefill_checked(const kda_prefill_desc* d, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const int32_t* cu_seqlens, const float* S0,
                           void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
  int64_t mc = 0;
  const kda_status s = check_desc(d, &mc);
  if (s != KDA_OK) return s;
  if (d->num_seqs == 0) return KDA_OK;
  PrefillPlan p;
  if (!make_prefill_plan(d, mc, &p)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARGUMENT;
  const size_t T = static_cast<size_t>(d->total_tokens), H = static_cast<size_t>(d->num_heads);
  const size_t es = io_size(d->io_dtype);
  const size_t gw = gate_width(d->gate, d->dk);
  if (gw == 0) log_alpha = nullptr;
  if (T > 0 && (!q || !k || !v || (gw && !log_alpha) || !beta || !o)) return KDA_ERR_INVALID_ARGUMENT;
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_INVALID_ARGUMENT;
  if (d->flags & KDA_PREFILL_BOUNDED) {
    // segments as long as the given workspace allows (the carried states in
    // S_T when the caller wants it, else in the workspace)
    if (!make_bounded_plan(d, mc, workspace_bytes, S_T == nullptr, &p)) return KDA_ERR_WORKSPACE_TOO_SMALL;
  } else if (workspace_bytes < p.total_bytes) {
    return KDA_ERR_WORKSPACE_TOO_SMALL;
  }
  const size_t state_bytes = static_cast<size_t>(d->num_seqs) * H * d->dk * d->dv * 4;
  const Range rq = range(q, T * H * d->dk * es), rk = range(k, T * H * d->dk * es),
              rv = range(v, T * H * d->dv * es), rla = range(log_alpha, log_alpha ? T * H * gw * 4 : 0),
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
  if (d->stages) {
    // the output stage rewrites o in place from o and the output gate
    const Range rg = range(d->stages->out_gate, d->stages->out_gate ? T * H * d->dv * es : 0),
                rw = range(d->stages->norm_weight, d->stages->norm_weight ? d->dv * 4 : 0);
    const Range outs[] = {ro, rst, rws};
    for (const Range& x : outs)
      if (overlap(rg, x) || overlap(rw, x)) return KDA_ERR_INVALID_ARGUMENT;
  }
  const hipError_t e = launch_prefill(p, q, k, v, log_alpha, beta, cu_seqlens, S0, o, S_T, workspace,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

}  // namespace kda

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

int32_t kda_version(void) { return 20100; }

size_t kda_prefill_workspace_size(const kda_prefill_desc* d) {
  int64_t mc = 0;
  if (check_desc(d, &mc) != KDA_OK) return 0;
  if (d->flags & KDA_PREFILL_BOUNDED) return kda::bounded_min_bytes(d, mc);
  kda::PrefillPlan p;
  if (!kda::make_prefill_plan(d, mc, &p)) return 0;
  return p.total_bytes;
}

kda_status kda_prefill(const kda_prefill_desc* d, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const int32_t* cu_seqlens, const float* S0,
                       void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
  return kda::prefill_checked(d, q, k, v, log_alpha, beta, cu_seqlens, S0, o, S_T, workspace, workspace_bytes, stream);
}

size_t kda_prefill_backward_workspace_size(const kda_prefill_desc* d) {
  int64_t mc = 0;
  if (check_desc(d, &mc) != KDA_OK || d->chunk != 64 || d->stages) return 0;
  kda::BackwardPlan p;
  if (!kda::make_backward_plan(d, mc, &p)) return 0;
  return p.total_bytes;
}

kda_status kda_prefill_backward(const kda_prefill_desc* d, const void* q, const void* k, const void* v,
                                const float* log_alpha, const float* beta, const int32_t* cu_seqlens,
                                const float* S0, const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                                float* dlog_alpha, float* dbeta, float* dS0, void* workspace,
                                size_t workspace_bytes, void* stream) {
  int64_t mc = 0;
  const kda_status s = check_desc(d, &mc);
  if (s != KDA_OK) return s;
  if (d->chunk != 64 || d->stages) return KDA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0) return KDA_OK;
  kda::BackwardPlan p;
  if (!kda::make_backward_plan(d, mc, &p)) return KDA_ERR_UNSUPPORTED;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARGUMENT;
  const size_t T = static_cast<size_t>(d->total_tokens), H = static_cast<size_t>(d->num_heads);
  const size_t es = io_size(d->io_dtype);
  const size_t gw = gate_width(d->gate, d->dk);
  if (gw == 0) log_alpha = nullptr, dlog_alpha = nullptr;
  if (T > 0 && (!q || !k || !v || (gw && (!log_alpha || !dlog_alpha)) || !beta || !dO || !dq || !dk || !dv ||
                !dbeta))
    return KDA_ERR_INVALID_ARGUMENT;
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < p.total_bytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
  const size_t state_bytes = static_cast<size_t>(d->num_seqs) * H * d->dk * d->dv * 4;
  const Range ins[] = {range(q, T * H * d->dk * es), range(k, T * H * d->dk * es), range(v, T * H * d->dv * es),
                       range(log_alpha, log_alpha ? T * H * gw * 4 : 0), range(beta, T * H * 4),
                       range(cu_seqlens, (static_cast<size_t>(d->num_seqs) + 1) * 4),
                       range(S0, S0 ? state_bytes : 0), range(dO, T * H * d->dv * es),
                       range(dS_T, dS_T ? state_bytes : 0)};
  const Range outs[] = {range(dq, T * H * d->dk * es), range(dk, T * H * d->dk * es), range(dv, T * H * d->dv * es),
                        range(dlog_alpha, dlog_alpha ? T * H * gw * 4 : 0), range(dbeta, T * H * 4),
                        range(dS0, dS0 ? state_bytes : 0), range(workspace, p.total_bytes)};
  constexpr int NO = sizeof(outs) / sizeof(outs[0]);
  for (int a = 0; a < NO; ++a) {
    for (const Range& x : ins)
      if (overlap(outs[a], x)) return KDA_ERR_INVALID_ARGUMENT;
    for (int b = a + 1; b < NO; ++b)
      if (overlap(outs[a], outs[b])) return KDA_ERR_INVALID_ARGUMENT;
  }
  const hipError_t e = kda::launch_backward(p, q, k, v, log_alpha, beta, cu_seqlens, S0, dO, dS_T, dq, dk, dv,
                                            dlog_alpha, dbeta, dS0, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

kda_status kda_prefill_recovered(const kda_prefill_desc* d, const void* workspace, int32_t* recovered,
                                 void* stream) {
  int64_t mc = 0;
  if (!recovered) return KDA_ERR_INVALID_ARGUMENT;
  *recovered = 0;
  const kda_status s = check_desc(d, &mc);
  if (s != KDA_OK) return s;
  kda::PrefillPlan p;
  if (!kda::make_prefill_plan(d, mc, &p)) return KDA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0 || p.off_ready == 0) return KDA_OK;
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  int32_t flag = 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&flag, static_cast<const unsigned char*>(workspace) + p.off_ready + 4, 4, hipMemcpyDeviceToHost,
                     st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return KDA_ERR_DEVICE;
  *recovered = flag != 0;
  return KDA_OK;
}

int32_t kda_prefill_set_wait_limit(int32_t polls) { return kda::set_prefill_wait_polls(polls); }

kda_status kda_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv, kda_dtype io_dtype, kda_gate gate,
                           const kda_stages* stages, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, float* S, void* o, void* stream) {
  if (B < 0 || H < 1 || !dtype_valid(io_dtype) || !gate_valid(gate) || !stages_valid(stages))
    return KDA_ERR_INVALID_ARGUMENT;
  if (!dims_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  const size_t gw = gate_width(gate, dk);
  if (gw == 0) log_alpha = nullptr;
  if (!q || !k || !v || (gw && !log_alpha) || !beta || !S || !o) return KDA_ERR_INVALID_ARGUMENT;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > 0x7fffffff) return KDA_ERR_UNSUPPORTED;
  const size_t es = io_size(io_dtype), n = static_cast<size_t>(BH);
  const Range rs = range(S, n * dk * dv * 4), ro = range(o, n * dv * es);
  const Range others[] = {range(q, n * dk * es), range(k, n * dk * es), range(v, n * dv * es),
                          range(log_alpha, log_alpha ? n * gw * 4 : 0), range(beta, n * 4)};
  for (const Range& x : others)
    if (overlap(rs, x) || overlap(ro, x)) return KDA_ERR_INVALID_ARGUMENT;
  if (overlap(rs, ro)) return KDA_ERR_INVALID_ARGUMENT;
  if (stages) {
    const Range rg = range(stages->out_gate, stages->out_gate ? n * dv * es : 0),
                rw = range(stages->norm_weight, stages->norm_weight ? static_cast<size_t>(dv) * 4 : 0);
    if (overlap(rg, rs) || overlap(rg, ro) || overlap(rw, rs) || overlap(rw, ro)) return KDA_ERR_INVALID_ARGUMENT;
  }
  const hipError_t e = kda::launch_decode(io_dtype, gate, stages, dk, dv, static_cast<int>(BH), q, k, v, log_alpha,
                                          beta, S, o, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_DEVICE;
}

}  // extern "C"
