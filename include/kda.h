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
 *     overlapped prefill schedule (and the ring form of KDA_PREFILL_BOUNDED),
 *     two CU-masked streams with their events per device, on which
 *     concurrent calls for one device take turns to enqueue their work; the
 *     streams are destroyed at process exit.
 *   - Device-side preconditions that are documented but not checked: finite
 *     inputs; log_alpha <= 0; when no host mirror of cu_seqlens is given,
 *     cu_seqlens[0] = 0, non-decreasing and cu_seqlens[N] = total_tokens.
 *     Any finite log_alpha <= 0 is supported (no range limit): the chunked
 *     prefill forms every intra-chunk gate ratio from sums of log_alpha over
 *     contiguous token ranges with factors at most 1, and forms a diagonal
 *     16-token block's ratios token by token for channels whose decay across
 *     the block leaves the fp32 range.
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

/* Forget-gate form.  KDA's gate is one rate per key channel; the scalar
   form (one rate per head and token) is Gated DeltaNet and no gate at all
   (alpha = 1) is DeltaNet -- the two special cases the deep-read report
   (sections 2.2 and 2.3) and the zhaixingw.cn explainer's KDA section (the
   GDN update with a scalar gate) place KDA against.  They run as
   specialisations of the same kernels with cheaper gate handling. */
typedef enum {
  KDA_GATE_CHANNEL = 0,  /* log_alpha [.., dk]: one rate per key channel (KDA) */
  KDA_GATE_SCALAR = 1,   /* log_alpha [..]: one rate per head (Gated DeltaNet) */
  KDA_GATE_NONE = 2      /* no forget gate, alpha = 1 (DeltaNet); log_alpha unused, may be NULL */
} kda_gate;

/* Input and output stages fused around the recurrence.  The deep-read
   report, section 3.2, places KDA between an input side (q and k
   L2-normalised per head; the forget gate out of a low-rank projection) and
   an output side (a head-wise RMSNorm and a low-rank, data-dependent sigmoid
   output gate).  The projections themselves (and the short convolutions with
   Swish) produce these stages' inputs and are outside the library.  Every
   field at zero/NULL leaves the stage out; a NULL kda_stages pointer leaves
   all out. */
typedef struct {
  int32_t l2norm_qk;        /* nonzero: q and k are raw; each (token, head) vector is
                               divided by max(||x||_2, l2norm_eps) before use */
  float l2norm_eps;         /* > 0 when l2norm_qk */
  int32_t gate_softplus;    /* nonzero: log_alpha holds the gate projection's output z;
                               the kernels use log alpha = -softplus(z) (any finite z) */
  const float* norm_weight; /* [dv] fp32 DEVICE: o <- o / sqrt(mean_j o_j^2 + norm_eps) *
                               norm_weight per (token, head); NULL: no norm */
  float norm_eps;           /* > 0 when norm_weight is given */
  const void* out_gate;     /* DEVICE, io dtype, shaped like o: z_o; o <- o * sigmoid(z_o)
                               after the norm; NULL: no output gate */
} kda_stages;

/* kda_prefill_desc.flags */
enum {
  /* Run the chunk preparation and the state pass one after the other on the
     caller's stream, never on the library's two CU-masked streams (for tools
     that serialise kernel dispatches, such as hardware-counter collection;
     results are identical, and the workspace is smaller). */
  KDA_PREFILL_ONE_STREAM = 1,
  /* Bounded workspace: kda_prefill_workspace_size returns the smallest
     workspace kda_prefill then accepts (the chunk table, the blocks of one
     chunk index for every head, and room for N*H*dk*dv fp32 carried states),
     and kda_prefill takes the chunks in segments of global chunk indices as
     long as the workspace it is given allows: each segment is prepared into
     the one block area, then the state pass resumes every (sequence, head)
     from the state the previous segment left (kept in S_T, or in the
     workspace when S_T is NULL), all on `stream`.  The workspace need not
     grow with the number of tokens; results are bit-identical to
     KDA_PREFILL_ONE_STREAM, which is what a workspace of at least that
     flag's size amounts to (one segment).  Shorter segments cost time: each
     segment's state pass waits for the longest chain in it. */
  KDA_PREFILL_BOUNDED = 2
};

/* Problem description for the packed variable-length prefill. */
typedef struct {
  int32_t num_seqs;      /* N >= 0 sequences packed back to back */
  int32_t total_tokens;  /* T_tot = cu_seqlens[N] >= 0 */
  int32_t num_heads;     /* H >= 1 */
  int32_t dk, dv;        /* key / value head dims, each 64 or 128 */
  int32_t chunk;         /* tokens per chunk: 64 (32 and 16 also accepted; 16-token
                            chunks run through the 32-row kernels) */
  kda_dtype io_dtype;    /* dtype of q, k, v and o */
  const int32_t* cu_seqlens_host; /* optional HOST copy of cu_seqlens [N+1]; when
                                     given it is validated and used to size the
                                     launch exactly; may be NULL */
  uint32_t flags;        /* KDA_PREFILL_* bits; 0 for the default schedule */
  kda_gate gate;         /* form of log_alpha; KDA_GATE_CHANNEL for KDA */
  const kda_stages* stages; /* optional HOST struct: input/output stages; may be NULL */
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
 *   log_alpha  [T_tot, H, dk]  float32, log of the forget gate (<= 0); [T_tot, H]
 *                              for KDA_GATE_SCALAR; unused for KDA_GATE_NONE
 *   beta       [T_tot, H]      float32
 *   cu_seqlens [N + 1]         int32 offsets (device)
 *   S0         [N, H, dk, dv]  float32, or NULL for a zero initial state
 *   o          [T_tot, H, dv]  io_dtype, written
 *   S_T        [N, H, dk, dv]  float32, written; NULL to skip.  S_T may be the
 *                              same pointer as S0 (updated in place); any
 *                              other overlap between buffers is invalid.
 *   workspace  >= kda_prefill_workspace_size(desc) bytes, 256-byte aligned;
 *              its contents on entry are ignored and on return undefined.
 *              With KDA_PREFILL_BOUNDED, workspace_bytes sets the segment
 *              length (see the flag).
 *   stream     hipStream_t or NULL.
 *   desc->stages  optional input/output stages (kda_stages): with an output
 *              stage, o holds its result (the stage runs as one more pass over
 *              o on `stream`: the state pass's value tiles split dv, which
 *              the head-wise norm spans); the output gate is [T_tot, H, dv].
 *
 * Streams: the work is ordered on `stream`.  For few (sequence, head) pairs
 * (N * H * dv / 32 <= 128), unless flags has KDA_PREFILL_ONE_STREAM, the call
 * forks onto two library-owned streams that split the CUs (one runs the
 * serial state pass, the other prepares later chunks and advances a counter
 * in the workspace that the first waits on) and joins back into `stream`
 * with events.  The wait is bounded: if the device does not run the two
 * streams side by side (a tool that serialises dispatches, an oversubscribed
 * device), the state pass stops waiting, and two recovery launches on
 * `stream`, which otherwise return at once, recompute every output there.
 * Results are correct either way; kda_prefill_recovered reports which.
 * With KDA_PREFILL_BOUNDED and such few pairs, when two or more segments
 * fit the workspace, the segments rotate through slots of it on the same
 * two streams, every dependency a stream event (nothing waits inside a
 * kernel, nothing to recover); otherwise that flag runs every launch on
 * `stream`.
 *
 * Errors: KDA_ERR_INVALID_ARGUMENT (null pointer where data is required,
 * negative sizes, bad host offsets, misaligned workspace, overlapping buffers),
 * KDA_ERR_UNSUPPORTED (dk/dv not in {64,128}, chunk not in {16,32,64}),
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
 * kda_prefill for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid allocation).
 * The workspace is a static device array of KDA_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the call
 * allocates nothing.  It always runs the one-stream schedule (only kernel
 * launches on `stream`); a problem whose one-stream workspace
 * (kda_prefill_workspace_size with KDA_PREFILL_ONE_STREAM: about 976 bytes
 * per token and head for bf16, dk = 128, chunk 64, so about 8,000 tokens x
 * 32 heads) exceeds the array runs the bounded schedule of
 * KDA_PREFILL_BOUNDED inside it, with identical results.  Arguments and
 * results as for kda_prefill.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * on it and must not be issued.  Errors: as kda_prefill, and
 * KDA_ERR_WORKSPACE_TOO_SMALL (nothing launched) when not even the bounded
 * schedule fits: the blocks of one chunk index for every head (about 61 KB
 * per head) plus, when S_T is NULL, the N*H*dk*dv fp32 carried states, more
 * than the array holds.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (256u << 20)
kda_status kda_prefill_noalloc(const kda_prefill_desc* desc,
                               const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta,
                               const int32_t* cu_seqlens, const float* S0,
                               void* o, float* S_T, void* stream);

/*
 * After a kda_prefill call that used `workspace` for `desc` on `stream`:
 * waits for `stream` (host synchronisation) and sets *recovered to 1 if
 * that call's overlapped schedule stopped waiting for its prepared chunks
 * and recomputed its outputs on the caller's stream, else 0.  Calls that
 * ran the one-stream schedule report 0 without synchronising.  Errors:
 * KDA_ERR_INVALID_ARGUMENT (bad desc, null pointer), KDA_ERR_DEVICE.
 */
kda_status kda_prefill_recovered(const kda_prefill_desc* desc, const void* workspace, int32_t* recovered,
                                 void* stream);

/*
 * Test hook (process-wide): the number of polls, each about a microsecond,
 * for which the overlapped schedule's state pass waits for a prepared
 * segment before it gives up and the call recovers.  polls > 0 sets it,
 * 0 makes the state pass never wait (every overlapped call then recovers),
 * polls < 0 restores the default.  Returns the previous value.  For tests
 * of the recovery path; calls in flight on other threads see either value.
 */
int32_t kda_prefill_set_wait_limit(int32_t polls);

/*
 * One decode step for B independent requests: the recurrence applied once
 * per (b, h), updating the fixed-size state in place.  Each request keeps one
 * dk x dv state per head whatever its context length (the zhaixingw.cn
 * explainer's serving section: per-request fixed-size state instead of a KV
 * cache).
 *
 *   q, k       [B, H, dk]      io_dtype
 *   v          [B, H, dv]      io_dtype
 *   log_alpha  [B, H, dk]      float32 ([B, H] for KDA_GATE_SCALAR; unused, may be
 *                              NULL, for KDA_GATE_NONE)
 *   beta       [B, H]          float32
 *   S          [B, H, dk, dv]  float32, read as S_{t-1} and overwritten with S_t
 *   o          [B, H, dv]      io_dtype, written
 *   stages     optional HOST struct (see kda_stages); the output gate is [B, H, dv]
 *
 * Errors: KDA_ERR_INVALID_ARGUMENT (null pointer with B > 0, B < 0, H < 1,
 * unknown gate, a stage with a non-positive epsilon or an output gate that
 * overlaps S or o), KDA_ERR_UNSUPPORTED (dk/dv not in {64,128}), KDA_ERR_DEVICE.  B == 0 is a
 * no-op.  S must not overlap any other argument.
 */
kda_status kda_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv, kda_dtype io_dtype, kda_gate gate,
                           const kda_stages* stages,
                           const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           float* S, void* o, void* stream);

/*
 * Bytes of device workspace kda_prefill_backward needs for `desc` (256-byte
 * aligned pointer expected): per (64-token chunk, head) a block of chunk
 * factors and two dk x dv states, fp32 (353 KiB for dk = dv = 128; the
 * 131,072-token, 32-head case takes 23.7 GB).  Returns 0 for an invalid or
 * unsupported desc.  Host-only; launches nothing.
 */
size_t kda_prefill_backward_workspace_size(const kda_prefill_desc* desc);

/*
 * Backward pass of kda_prefill (training).  The deep-read report trains the
 * model (section 3.4) and gives the chunked forward (section 3.1) but no
 * gradient; this is the exact derivative of the recurrence above, computed
 * through the same chunked form (64-token chunks): for the scalar
 *
 *     L = sum_t <dO_t, o_t> + sum_{n,h} <dS_T[n,h], S_T[n,h]>
 *
 * it writes dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/dbeta and dL/dS0.
 *
 *   q, k, v, log_alpha, beta, cu_seqlens, S0   as passed to kda_prefill
 *   dO         [T_tot, H, dv]  io_dtype, cotangent of o
 *   dS_T       [N, H, dk, dv]  float32 cotangent of S_T, or NULL (zero)
 *   dq, dk     [T_tot, H, dk]  io_dtype, written
 *   dv         [T_tot, H, dv]  io_dtype, written
 *   dlog_alpha float32, written, shaped like log_alpha ([T_tot, H, dk]; [T_tot, H]
 *              for KDA_GATE_SCALAR, where it is the sum over key channels);
 *              unused (may be NULL) for KDA_GATE_NONE
 *   dbeta      [T_tot, H]      float32, written
 *   dS0        [N, H, dk, dv]  float32, written; NULL to skip
 *   workspace  >= kda_prefill_backward_workspace_size(desc) bytes, 256-byte
 *              aligned; contents on entry ignored, on return undefined.
 *
 * desc: as for kda_prefill, with chunk = 64 and no stages (the stages'
 * derivatives are left to the caller's framework).  flags are ignored: the
 * backward runs on `stream` only.  Outputs must not overlap any input, the
 * workspace or each other.  Same device-side preconditions as kda_prefill
 * (any finite log_alpha <= 0).  Results are deterministic: the same inputs
 * give the same bits.
 *
 * Errors: KDA_ERR_INVALID_ARGUMENT (null pointer where data is required,
 * overlapping buffers, misaligned workspace, bad host offsets),
 * KDA_ERR_UNSUPPORTED (dk/dv not in {64,128}, chunk != 64, stages given),
 * KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_DEVICE.  With total_tokens == 0 only
 * dS0 = dS_T (or zero) is written.
 */
kda_status kda_prefill_backward(const kda_prefill_desc* desc,
                                const void* q, const void* k, const void* v,
                                const float* log_alpha, const float* beta,
                                const int32_t* cu_seqlens, const float* S0,
                                const void* dO, const float* dS_T,
                                void* dq, void* dk, void* dv, float* dlog_alpha,
                                float* dbeta, float* dS0,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH (2.0.0: desc.flags,
   desc.gate and the gate argument of kda_decode_step; 2.1.0: the prefill
   backward). */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
