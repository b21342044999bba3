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
  const float* kv_scales;   // nullptr: bf16 cache; per-tensor FP8: the one k_scale_inv
  void* out;
  float* lse;
  void* workspace;
  int32_t batch, heads, num_pages, max_pages, topk;
  int32_t tq;  // query tokens per sequence (T >= 1); batch and heads are per the C ABI (B, H)
  bool q_fp8;
  int32_t kv_format;  // kKvFormat*
  float softmax_scale, q_descale;
  int32_t ranges;  // KV ranges of the split-KV decode (workgroups per head slab)
};

// The decode kernels' argument block (device pointers and sizes, set up by
// launch_decode).
struct DecodeArgs {
  const void* q;
  const char* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* topk_idx;
  const float* kv_scales;
  void* out;
  float* lse;
  float* ws_o;    // [(ranges + B) slots][H][512] normalised partial O, fp32 (split-reduction kernel)
  _Float16* ws_o16;  // the same region as [(ranges + B)][H][512] fp16 of O / 2^e (wave-specialised kernel)
  float* ws_sc;      // then [(ranges + B)][H][4] the factors 2^e, one per row and 128 columns
  float* ws_lse;  // [(ranges + B)][H] base-2 LSE of partials
  int2* ws_seq;   // [B] {range of piece 0, pieces}; pieces 0: nothing to attend
  int32_t compact;   // partial slots: 2 per range (slot 2r + (r == first range)) instead of one per (b + r)
  int32_t topk_tq;           // top-k: lists per sequence (T); list b belongs to sequence b / T
  int32_t batch, heads, num_pages, max_pages, topk;
  int32_t tq;         // dense, several query tokens: T (rows of a sequence = T x heads_tok), else 1
  int32_t heads_tok;  // query heads per token
  int32_t ranges;    // KV ranges (workgroups per head slab)
  int32_t seg_pad;   // virtual units at each end of a sequence on the split line (segment overhead)
  int32_t slabs;     // head slabs per range
  int32_t per_xcd;   // ranges per XCD in the block -> (range, slab) mapping
  float scale_log2;  // softmax_scale * log2(e)
  float q_descale;
};

// Cache layouts of a decode launch.
constexpr int32_t kKvFormatBf16 = 0;       // bf16 rows of 576
constexpr int32_t kKvFormatFp8Tile = 1;    // 512 e4m3 codes + 64 bf16 rope, fp32 scale per 128 columns
constexpr int32_t kKvFormatFp8Tensor = 2;  // 576 e4m3 codes, one per-tensor k_scale_inv

// Sequences and rows per sequence the kernels see for B sequences of T query
// tokens of H heads (the ranges and the workspace are sized on these).
void effective_dims(int32_t batch, int32_t heads, int32_t topk, int32_t tq, int32_t* eb, int32_t* eh);
// KV ranges for a device with `cus` compute units.
int32_t decode_ranges(int32_t cus, int32_t batch, int32_t max_pages, int32_t topk, int32_t heads);
// Workspace bytes for a decode launch with `ranges` KV ranges.
size_t decode_workspace_bytes(int32_t ranges, int32_t batch, int32_t heads, int32_t topk);
// Partial slots of a decode workspace: one per (sequence + range) index, or,
// when that is more, two per range (each range holds at most two pieces of
// split sequences: one continuing from before its start, one running past
// its end).
inline int64_t decode_partial_slots(int32_t ranges, int32_t batch) {
  return (int64_t)ranges + batch <= 2 * (int64_t)ranges ? (int64_t)ranges + batch : 2 * (int64_t)ranges;
}
// Clear the per-sequence piece records of a decode workspace (optional: every call rewrites them).
hipError_t init_decode_workspace(void* workspace, int32_t batch, int32_t heads, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream);
// The library-owned decode scratch of the current device (scratch.hip): its
// device address and size.  Looks the address up on a device's first call.
hipError_t decode_scratch(void** ptr, size_t* bytes);
// The wave-specialised decode (decode_ws.hip): bf16 paged caches, dense,
// at least 64 query rows per sequence.
bool decode_ws_supported(int32_t kv_format, int32_t topk, int32_t eff_heads, int32_t num_pages);
hipError_t launch_decode_ws(const DecodeArgs& a, int32_t kv_format, bool q_fp8, bool causal, hipStream_t stream);
// Split-line padding of the wave-specialised decode: a segment costs about
// as much as this many pages at each of its two ends (query load, pipeline
// fill, epilogue), so each sequence's pages sit between that many virtual
// units on each side and the equal cut balances pages plus segment ends.
constexpr int32_t kWsSegPad = 4;

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

struct InsertLaunch {
  const void* qkv;
  const void* w_kva;
  const int64_t* slots;
  const float* k_scale_inv;
  void* cache;
  int32_t tokens, num_pages, qkv_stride;
  float eps;
};

hipError_t launch_kv_insert(const InsertLaunch& k, hipStream_t stream);

size_t query_workspace_bytes(int32_t batch, int32_t heads);
hipError_t launch_query(const QueryLaunch& q, hipStream_t stream);

}  // namespace mla
