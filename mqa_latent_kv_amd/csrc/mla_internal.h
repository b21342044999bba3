// Internal host-side interface between the C ABI layer (api.cpp) and the
// kernel launchers (decode.hip, query.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Everything a decode launch needs, after host validation.
struct DecodeLaunch {
  const void* q;
  const void* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* topk_idx;  // nullptr: dense
  const float* kv_scales;   // nullptr: bf16 cache
  void* out;
  float* lse;
  void* workspace;
  int32_t batch, heads, num_pages, max_pages, topk;
  bool q_fp8, kv_fp8;
  float softmax_scale, q_descale;
  int32_t ranges;  // KV ranges of the split-KV decode (workgroups per head slab)
};

// KV ranges for a device with `cus` compute units.
int32_t decode_ranges(int32_t cus, int32_t batch, int32_t max_pages, int32_t topk, int32_t heads);
// Workspace bytes for a decode launch with `ranges` KV ranges.
size_t decode_workspace_bytes(int32_t ranges, int32_t batch, int32_t heads, int32_t topk);
// Clear the per-sequence piece records of a decode workspace (optional: every call rewrites them).
hipError_t init_decode_workspace(void* workspace, int32_t batch, int32_t heads, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream);

struct QueryLaunch {
  const void* qkv;
  const void* w_qa;
  const void* w_qb;
  const void* w_uk;
  const float* q_scale_inv;
  void* out;
  void* workspace;
  int32_t batch, heads, qkv_stride;
  float eps;
};

size_t query_workspace_bytes(int32_t batch, int32_t heads);
hipError_t launch_query(const QueryLaunch& q, hipStream_t stream);

}  // namespace mla
