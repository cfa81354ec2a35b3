// kda_internal.h -- launchers shared between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Decode: one recurrence step for B*H states (all pointers device).
hipError_t launch_decode(kda_dtype dt, int dk, int dv, int BH, const void* q, const void* k, const void* v,
                         const float* la, const float* beta, float* S, void* o, hipStream_t stream);

// Prefill workspace carve-up, computed on the host.
struct PrefillPlan {
  int N, T, H, dk, dv, C;
  kda_dtype dt;
  int64_t max_chunks;  // upper bound (exact when the host offsets are known)
  int sort;            // 1: longest-first order is computed on the device
  // byte offsets inside the workspace
  size_t off_chunk_off, off_order, off_blocks;
  size_t off_ready;  // segment counter of the overlapped schedule (0: none)
  size_t total_bytes;
  // Segment length in global chunk indices for the overlapped two-stream
  // schedule (0: one prep launch, then one scan launch).
  int64_t seg;
};

// Returns false when the shape is unsupported.
bool make_prefill_plan(const kda_prefill_desc* d, int64_t max_chunks, PrefillPlan* p);

hipError_t launch_prefill(const PrefillPlan& p, const void* q, const void* k, const void* v, const float* la,
                          const float* beta, const int32_t* cu, const float* S0, void* o, float* S_T,
                          void* workspace, hipStream_t stream);

}  // namespace kda
