// kda_internal.h -- launchers shared between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Decode: one recurrence step for B*H states (all pointers device).
hipError_t launch_decode(kda_dtype dt, kda_gate gate, const kda_stages* stages, int dk, int dv, int BH, const void* q, const void* k, const void* v,
                         const float* la, const float* beta, float* S, void* o, hipStream_t stream);

// Prefill workspace carve-up, computed on the host.
struct PrefillPlan {
  int N, T, H, dk, dv;
  int C;   // rows of the kernels' chunk tiles (32 or 64)
  int CL;  // tokens per chunk (16, 32 or 64; at most C)
  kda_dtype dt;
  kda_gate gate;
  // input and output stages (kda_stages)
  int l2norm_qk, gate_softplus;
  float l2norm_eps, norm_eps;
  const float* norm_weight;
  const void* out_gate;
  int64_t max_chunks;  // upper bound (exact when the host offsets are known)
  int sort;            // 1: longest-first order is computed on the device
  // byte offsets inside the workspace
  size_t off_chunk_off, off_order, off_blocks;
  size_t off_ready;  // segment counter and recovery flag of the overlapped schedule (0: none)
  size_t off_carry;  // final states of an in-place overlapped call (0: none)
  size_t total_bytes;
  // Segment length in global chunk indices for the overlapped two-stream
  // schedule (0: one prep launch, then one scan launch).
  int64_t seg;
  // Bounded schedule (bseg > 0): segments of bseg global chunk indices, each
  // prepared into the one block area and then passed over by the state
  // pass, which resumes every (sequence, head) from the state the previous
  // segment left; that state is kept at off_bcarry (0: in S_T).
  int64_t bseg;
  size_t off_bcarry;
  // Its ring form for few (sequence, head) pairs (rslots >= 2): segments of
  // rseg chunk indices in rslots slots of the block area, prepared on one
  // half of the CUs while the state pass runs on the other (0: none).
  int64_t rseg, rslots;
};

// Returns false when the shape is unsupported.
bool make_prefill_plan(const kda_prefill_desc* d, int64_t max_chunks, PrefillPlan* p);
// Plan of the bounded schedule inside workspace_bytes (the carried states in
// the workspace when carry_in_ws, else in S_T); false if not even one chunk
// index per segment fits.
bool make_bounded_plan(const kda_prefill_desc* d, int64_t max_chunks, size_t workspace_bytes, bool carry_in_ws,
                       PrefillPlan* p);
// Smallest workspace of the bounded schedule (room for the carried states
// included).
size_t bounded_min_bytes(const kda_prefill_desc* d, int64_t max_chunks);

// Test hook behind kda_prefill_set_wait_limit: polls > 0 sets the bound of
// the overlapped schedule's wait, 0 makes it never wait, < 0 restores the
// default.  Returns the previous bound.
int set_prefill_wait_polls(int polls);

// kda_prefill after host validation (shared by the entry points that take
// or provide a workspace).
kda_status prefill_checked(const kda_prefill_desc* d, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const int32_t* cu_seqlens, const float* S0,
                           void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream);

hipError_t launch_prefill(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                          const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                          void* workspace, hipStream_t stream);

// Chunk offsets per sequence (chunk_off[n] = sum_{i<n} ceil(L_i / C), [N + 1])
// and the longest-first sequence order (identity when sort is 0).
hipError_t launch_chunk_offsets(const int32_t* cu, int N, int C, int32_t* chunk_off, int32_t* order, int sort,
                                hipStream_t st);

// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus);

// Backward workspace carve-up, computed on the host.
struct BackwardPlan {
  int N, T, H, dk, dv;
  kda_dtype dt;
  kda_gate gate;
  int64_t max_chunks;
  int sort;
  size_t off_chunk_off, off_order, off_blocks, off_states, off_dstates, total_bytes;
};

bool make_backward_plan(const kda_prefill_desc* d, int64_t max_chunks, BackwardPlan* p);

hipError_t launch_backward(const BackwardPlan& p, const void* q, const void* k, const void* v, const float* la,
                           const float* beta, const int32_t* cu, const float* S0, const void* dO, const float* dS_T,
                           void* dq, void* dk, void* dv, float* dla, float* dbeta, float* dS0, void* workspace,
                           hipStream_t stream);

}  // namespace kda
