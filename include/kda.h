/*
 * kda.h -- C ABI of libkda, a gfx950 (MI355X) implementation of Kimi Delta
 * Attention (KDA).
 *
 * The operator.  For every sequence and head, with a dk x dv fp32 state S:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * alpha_t = exp(log_alpha_t) is a per-key-channel forget gate (one rate per
 * row of S), beta_t a scalar write strength.  Source: the "Kimi Linear: An
 * Expressive, Efficient Attention Architecture" deep-read report (zako-mio
 * knowledge base), section 2.3 (diagonal per-channel gate inside the gated
 * delta rule; forget, erase along k, write), and the zhaixingw.cn explainer's
 * KDA section (alpha is a dk-vector, the state is dk x dv).  The output has no
 * extra scale: fold any 1/sqrt(d) into q.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says host.
 *   - Tensors are dense, row-major, contiguous, in the shapes given.
 *   - The caller owns every buffer; the library never allocates or frees
 *     device memory.  Scratch for prefill comes from a caller workspace.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  Results are defined once
 *     the stream reaches that point.  Faults inside kernels surface at the
 *     caller's next synchronisation, not as a return code.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed validation returns an error and launches nothing.  No C++
 *     exception crosses this boundary.
 *   - Calls are thread-safe.  The library's only process state is created
 *     once under a lock: per-device kernel attributes and, for the
 *     overlapped prefill schedule, two CU-masked streams with their events
 *     per device, on which concurrent overlapped calls for one device take
 *     turns to enqueue their work.
 *   - Device-side preconditions that are documented but not checked:
 *     finite inputs; log_alpha <= 0; for the chunked prefill additionally,
 *     per channel, the log_alpha of any 9 consecutive tokens of a sequence
 *     sum to at least -80 (log_alpha >= -8 per element suffices): the
 *     intra-chunk gate ratios are factorised around references inside each
 *     16-token block, and every factor must stay inside the fp32 range
 *     (beyond it a scale factor of an off-diagonal block underflows while the
 *     ratio it stands for need not be small, so results are wrong); when no host mirror of
 *     cu_seqlens is given, cu_seqlens[0] = 0, non-decreasing and
 *     cu_seqlens[N] = total_tokens.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, bad offsets, aliasing */
  KDA_ERR_UNSUPPORTED = 2,       /* valid but not implemented: head dim, chunk, dtype */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_DEVICE = 4             /* a HIP runtime call or kernel launch failed */
} kda_status;

typedef enum {
  KDA_F32 = 0,   /* q, k, v and o in float32 */
  KDA_BF16 = 1   /* q, k, v and o in bfloat16 */
} kda_dtype;

/* Problem description for the packed variable-length prefill. */
typedef struct {
  int32_t num_seqs;      /* N >= 0 sequences packed back to back */
  int32_t total_tokens;  /* T_tot = cu_seqlens[N] >= 0 */
  int32_t num_heads;     /* H >= 1 */
  int32_t dk, dv;        /* key / value head dims, each 64 or 128 */
  int32_t chunk;         /* tokens per chunk: 64 (32 also accepted) */
  kda_dtype io_dtype;    /* dtype of q, k, v and o */
  const int32_t* cu_seqlens_host; /* optional HOST copy of cu_seqlens [N+1]; when
                                     given it is validated and used to size the
                                     launch exactly; may be NULL */
} kda_prefill_desc;

/*
 * Bytes of device workspace kda_prefill needs for `desc` (256-byte aligned
 * pointer expected).  Returns 0 for an invalid or unsupported desc.
 * Host-only; launches nothing.
 */
size_t kda_prefill_workspace_size(const kda_prefill_desc* desc);

/*
 * Chunked prefill over a packed batch of sequences.
 *
 * Computes o_t for every token and the final state of every (sequence, head)
 * with the recurrence above; sequence n owns tokens cu_seqlens[n] ..
 * cu_seqlens[n+1]-1 and starts from S0[n] (zero when S0 is NULL).  The method
 * is the chunkwise form the deep-read report describes in section 3.1: within
 * a chunk the two gated secondary-chunk matrices (k k^T and q k^T, tied by the
 * a = b = k binding), a UT-transform triangular inverse by forward
 * substitution and WY-form factors; across chunks a sequential state pass.
 *
 *   q, k       [T_tot, H, dk]  io_dtype
 *   v          [T_tot, H, dv]  io_dtype
 *   log_alpha  [T_tot, H, dk]  float32, log of the forget gate (<= 0)
 *   beta       [T_tot, H]      float32
 *   cu_seqlens [N + 1]         int32 offsets (device)
 *   S0         [N, H, dk, dv]  float32, or NULL for a zero initial state
 *   o          [T_tot, H, dv]  io_dtype, written
 *   S_T        [N, H, dk, dv]  float32, written; NULL to skip.  S_T may be the
 *                              same pointer as S0 (updated in place); any
 *                              other overlap between buffers is invalid.
 *   workspace  >= kda_prefill_workspace_size(desc) bytes, 256-byte aligned;
 *              its contents on entry are ignored and on return undefined.
 *   stream     hipStream_t or NULL.
 *
 * Streams: the work is ordered on `stream`.  For few (sequence, head) pairs
 * (N * H * dv / 32 <= 128) the call forks onto two library-owned streams that
 * split the CUs (one runs the serial state pass, the other prepares later
 * chunks and advances a counter in the workspace that the first waits on) and
 * joins back into `stream` with events.  That schedule needs the device to
 * run the two library streams at the same time (each has its own CU-masked
 * hardware queue): the state pass waits, for a bounded time, for the other
 * stream's prepared chunks, and if they never come (a tool that serialises
 * kernel dispatches, such as hardware-counter collection, or an
 * oversubscribed device) it stops waiting and its results are wrong; it then
 * sets the second 4-byte word of the workspace's last 256 bytes.  The
 * environment variable KDA_PREFILL_OVERLAP=0, read once per process, selects
 * the one-stream schedule (same kernels and results) for such settings.
 *
 * Errors: KDA_ERR_INVALID_ARGUMENT (null pointer where data is required,
 * negative sizes, bad host offsets, misaligned workspace, overlapping buffers),
 * KDA_ERR_UNSUPPORTED (dk/dv not in {64,128}, chunk not in {32,64}),
 * KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_DEVICE (launch failure).  With
 * total_tokens == 0 only S_T = S0 (or zero) is written.
 */
kda_status kda_prefill(const kda_prefill_desc* desc,
                       const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta,
                       const int32_t* cu_seqlens, const float* S0,
                       void* o, float* S_T,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step for B independent requests: the recurrence applied once
 * per (b, h), updating the fixed-size state in place.  Each request keeps one
 * dk x dv state per head whatever its context length (the zhaixingw.cn
 * explainer's serving section: per-request fixed-size state instead of a KV
 * cache).
 *
 *   q, k       [B, H, dk]      io_dtype
 *   v          [B, H, dv]      io_dtype
 *   log_alpha  [B, H, dk]      float32
 *   beta       [B, H]          float32
 *   S          [B, H, dk, dv]  float32, read as S_{t-1} and overwritten with S_t
 *   o          [B, H, dv]      io_dtype, written
 *
 * Errors: KDA_ERR_INVALID_ARGUMENT (null pointer with B > 0, B < 0, H < 1),
 * KDA_ERR_UNSUPPORTED (dk/dv not in {64,128}), KDA_ERR_DEVICE.  B == 0 is a
 * no-op.  S must not overlap any other argument.
 */
kda_status kda_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv, kda_dtype io_dtype,
                           const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           float* S, void* o, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
