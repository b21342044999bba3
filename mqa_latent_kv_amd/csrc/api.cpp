// api.cpp - the C ABI of libmla: argument validation, workspace sizing and
// dispatch to the gfx950 kernels.  Validation runs on the host before any HIP
// call, so every rejected argument is testable without a GPU.
#include "../../include/mla.h"
#include "mla_internal.h"

#include <mutex>

namespace {

bool valid_dtype(int32_t d) { return d == MLA_DTYPE_BF16 || d == MLA_DTYPE_FP8_E4M3; }
bool valid_kv_dtype(int32_t d) { return valid_dtype(d) || d == MLA_DTYPE_FP8_E4M3_TENSOR; }

bool supported_heads(int32_t h) { return h == 8 || h == 16 || h == 32 || h == 64 || h == 128; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int32_t check_decode_params(const mla_decode_params* p) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads < 1 || p->num_pages < 1 || p->max_pages_per_seq < 1 || p->topk < 0)
    return MLA_ERR_INVALID_ARG;
  if (!valid_dtype(p->q_dtype) || !valid_kv_dtype(p->kv_dtype)) return MLA_ERR_INVALID_ARG;
  if (!(p->softmax_scale > 0.0f) || !(p->q_descale > 0.0f)) return MLA_ERR_INVALID_ARG;
  if (p->tokens_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (p->batch > MLA_MAX_BATCH || !supported_heads(p->heads) || p->tokens_per_seq > MLA_MAX_TOKENS_PER_SEQ)
    return MLA_ERR_UNSUPPORTED;
  // 32-bit offsets inside the kernels: logical positions and pool rows
  if ((int64_t)p->max_pages_per_seq * MLA_PAGE_SIZE > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_pages * MLA_PAGE_SIZE > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  // top-k entries index a [B*T, topk] int32 array; keep B*T*topk in 32 bits
  if ((int64_t)p->batch * p->tokens_per_seq * p->topk > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// Compute units of the current device, cached per device id.
int32_t device_cus(int32_t* cus) {
  static std::mutex mu;
  static int32_t cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_DEVICE;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] > 0) {
      *cus = cache[dev];
      return MLA_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return MLA_ERR_DEVICE;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    cache[dev] = n;
  }
  *cus = n;
  return MLA_OK;
}

// Host validation shared by mla_decode and mla_decode_noalloc (a NULL
// workspace passes here; mla_decode rejects it afterwards).
int32_t decode_checked(const mla_decode_params* p, const void* q, const void* kv_cache,
                       const int32_t* block_table, const int32_t* seqlens, const int32_t* topk_idx,
                       const float* kv_scales, void* out, float* lse, const void* workspace) {
  int32_t st = check_decode_params(p);
  if (st != MLA_OK) return st;
  if (!q || !kv_cache || !block_table || !seqlens || !out || !lse) return MLA_ERR_INVALID_ARG;
  // q rows, cache rows, scales and outputs are accessed as 8/16-byte vectors
  // (a per-tensor scale is one float)
  const bool tile_scales = p->kv_dtype == MLA_DTYPE_FP8_E4M3;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) || (kv_scales && tile_scales && !aligned16(kv_scales)) ||
      (kv_scales && ((uintptr_t)kv_scales & 3)) || !aligned16(workspace))
    return MLA_ERR_INVALID_ARG;
  if ((p->topk > 0) != (topk_idx != nullptr)) return MLA_ERR_INVALID_ARG;
  if ((p->kv_dtype != MLA_DTYPE_BF16) != (kv_scales != nullptr)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// KV ranges and workspace bytes of a validated decode on the current device.
int32_t decode_plan(const mla_decode_params* p, int32_t* ranges, size_t* bytes) {
  int32_t cus = 0;
  const int32_t st = device_cus(&cus);
  if (st != MLA_OK) return st;
  int32_t eb = 0, eh = 0;
  mla::effective_dims(p->batch, p->heads, p->topk, p->tokens_per_seq, &eb, &eh);
  *ranges = mla::decode_ranges(cus, eb, p->max_pages_per_seq, p->topk, eh);
  *bytes = mla::decode_workspace_bytes(*ranges, eb, eh, p->topk);
  return MLA_OK;
}

int32_t decode_launch(const mla_decode_params* p, const void* q, const void* kv_cache,
                      const int32_t* block_table, const int32_t* seqlens, const int32_t* topk_idx,
                      const float* kv_scales, void* out, float* lse, void* workspace, int32_t ranges,
                      void* stream) {
  mla::DecodeLaunch d;
  d.q = q;
  d.kv = kv_cache;
  d.block_table = block_table;
  d.seqlens = seqlens;
  d.topk_idx = topk_idx;
  d.kv_scales = kv_scales;
  d.out = out;
  d.lse = lse;
  d.workspace = workspace;
  d.batch = p->batch;
  d.heads = p->heads;
  d.num_pages = p->num_pages;
  d.max_pages = p->max_pages_per_seq;
  d.topk = p->topk;
  d.tq = p->tokens_per_seq;
  d.q_fp8 = p->q_dtype == MLA_DTYPE_FP8_E4M3;
  d.kv_format = p->kv_dtype == MLA_DTYPE_BF16       ? mla::kKvFormatBf16
                : p->kv_dtype == MLA_DTYPE_FP8_E4M3 ? mla::kKvFormatFp8Tile
                                                    : mla::kKvFormatFp8Tensor;
  d.softmax_scale = p->softmax_scale;
  d.q_descale = p->q_descale;
  d.ranges = ranges;
  if (mla::launch_decode(d, (hipStream_t)stream) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_version(void) { return 300; }

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_DEVICE: return "no usable HIP device";
    case MLA_ERR_SCRATCH_LIMIT: return "problem needs more scratch than the library's static decode scratch holds";
    default: return "unknown status";
  }
}

int32_t mla_decode_workspace_size(const mla_decode_params* p, size_t* bytes) {
  if (!bytes) return MLA_ERR_INVALID_ARG;
  int32_t st = check_decode_params(p);
  if (st != MLA_OK) return st;
  int32_t ranges = 0;
  return decode_plan(p, &ranges, bytes);
}

int32_t mla_decode_workspace_init(const mla_decode_params* p, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  size_t need = 0;
  int32_t st = mla_decode_workspace_size(p, &need);
  if (st != MLA_OK) return st;
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  int32_t eb = 0, eh = 0;
  mla::effective_dims(p->batch, p->heads, p->topk, p->tokens_per_seq, &eb, &eh);
  if (mla::init_decode_workspace(workspace, eb, eh, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

int32_t mla_decode(const mla_decode_params* p, const void* q, const void* kv_cache,
                   const int32_t* block_table, const int32_t* seqlens, const int32_t* topk_idx,
                   const float* kv_scales, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int32_t st = decode_checked(p, q, kv_cache, block_table, seqlens, topk_idx, kv_scales, out, lse, workspace);
  if (st != MLA_OK) return st;
  if (!workspace) return MLA_ERR_WORKSPACE;
  int32_t ranges = 0;
  size_t need = 0;
  st = decode_plan(p, &ranges, &need);
  if (st != MLA_OK) return st;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  return decode_launch(p, q, kv_cache, block_table, seqlens, topk_idx, kv_scales, out, lse, workspace, ranges,
                       stream);
}

int32_t mla_decode_noalloc(const mla_decode_params* p, const void* q, const void* kv_cache,
                           const int32_t* block_table, const int32_t* seqlens, const int32_t* topk_idx,
                           const float* kv_scales, void* out, float* lse, void* stream) {
  int32_t st = decode_checked(p, q, kv_cache, block_table, seqlens, topk_idx, kv_scales, out, lse, nullptr);
  if (st != MLA_OK) return st;
  int32_t ranges = 0;
  size_t need = 0;
  st = decode_plan(p, &ranges, &need);
  if (st != MLA_OK) return st;
  if (need > MLA_DECODE_SCRATCH_BYTES) return MLA_ERR_SCRATCH_LIMIT;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (mla::decode_scratch(&scratch, &scratch_bytes) != hipSuccess || !scratch || !aligned16(scratch) ||
      scratch_bytes < need)
    return MLA_ERR_DEVICE;
  return decode_launch(p, q, kv_cache, block_table, seqlens, topk_idx, kv_scales, out, lse, scratch, ranges,
                       stream);
}

int32_t mla_query_workspace_size(const mla_query_params* p, size_t* bytes) {
  if (!p || !bytes) return MLA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads < 1 || p->qkv_stride < 1536 || !(p->eps >= 0.0f)) return MLA_ERR_INVALID_ARG;
  // rows are read as 16-byte vectors
  if (p->qkv_stride % 8 != 0) return MLA_ERR_UNSUPPORTED;
  if (p->batch > MLA_MAX_BATCH || p->heads > MLA_MAX_HEADS) return MLA_ERR_UNSUPPORTED;
  *bytes = mla::query_workspace_bytes(p->batch, p->heads);
  return MLA_OK;
}

int32_t mla_query(const mla_query_params* p, const void* qkv, const void* w_qa, const void* w_qb,
                  const void* w_uk, const float* q_scale_inv, void* out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  size_t need = 0;
  int32_t st = mla_query_workspace_size(p, &need);
  if (st != MLA_OK) return st;
  if (!qkv || !w_qa || !w_qb || !w_uk || !q_scale_inv || !out) return MLA_ERR_INVALID_ARG;
  // q_scale_inv is read as a uniform scalar load, which ignores the low address bits
  if (!aligned16(qkv) || !aligned16(w_qa) || !aligned16(w_qb) || !aligned16(w_uk) || !aligned16(workspace) ||
      ((uintptr_t)q_scale_inv & 3))
    return MLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  mla::QueryLaunch ql;
  ql.qkv = qkv;
  ql.w_qa = w_qa;
  ql.w_qb = w_qb;
  ql.w_uk = w_uk;
  ql.q_scale_inv = q_scale_inv;
  ql.out = out;
  ql.workspace = workspace;
  ql.batch = p->batch;
  ql.heads = p->heads;
  ql.qkv_stride = p->qkv_stride;
  ql.eps = p->eps;
  if (mla::launch_query(ql, (hipStream_t)stream) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

int32_t mla_kv_insert(const mla_kv_insert_params* p, const void* qkv, const void* w_kva,
                      const int64_t* slots, const float* k_scale_inv, void* kv_cache, void* stream) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->tokens < 0 || p->num_pages < 1 || p->qkv_stride < MLA_QKV_WIDTH || !(p->eps >= 0.0f))
    return MLA_ERR_INVALID_ARG;
  // rows are read as 16-byte vectors; slots and cache rows use 32-bit row numbers
  if (p->qkv_stride % 8 != 0) return MLA_ERR_UNSUPPORTED;
  if (p->tokens > MLA_MAX_INSERT_TOKENS || (int64_t)p->num_pages * MLA_PAGE_SIZE > INT32_MAX)
    return MLA_ERR_UNSUPPORTED;
  if (!qkv || !w_kva || !slots || !k_scale_inv || !kv_cache) return MLA_ERR_INVALID_ARG;
  if (!aligned16(qkv) || !aligned16(w_kva) || ((uintptr_t)slots & 7) || ((uintptr_t)k_scale_inv & 3) ||
      !aligned16(kv_cache))
    return MLA_ERR_INVALID_ARG;
  if (p->tokens == 0) return MLA_OK;
  mla::InsertLaunch k;
  k.qkv = qkv;
  k.w_kva = w_kva;
  k.slots = slots;
  k.k_scale_inv = k_scale_inv;
  k.cache = kv_cache;
  k.tokens = p->tokens;
  k.num_pages = p->num_pages;
  k.qkv_stride = p->qkv_stride;
  k.eps = p->eps;
  if (mla::launch_kv_insert(k, (hipStream_t)stream) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

}  // extern "C"
