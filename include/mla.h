/*
 * mla.h - C ABI of the MI355X (gfx950) absorbed multi-head latent attention
 * (MLA) decode library.
 *
 * Three operations:
 *
 *  mla_decode  Absorbed MLA decode for one query token per sequence.  All H
 *              query heads of a sequence attend to the same latent KV rows of
 *              576 values (512 latent "nope" columns, then 64 rope columns):
 *                  S[h,t] = scale * (q[h,0:512].k[t,0:512] + q[h,512:576].k[t,512:576])
 *                  LSE[h] = ln sum_t exp(S[h,t]),  O[h,:] = sum_t exp(S[h,t]-LSE[h]) k[t,0:512]
 *              Sources: the "STAGE_D2" MQA decode design note (section "DSV4 is
 *              MQA": one shared K/V for all query heads; "Strategy A: Head-Packed
 *              M Dimension": all heads of a token share one K/V read, softmax per
 *              head row), and FlashMLA issue "dual gemm" (the 64 rope columns
 *              are an extra block of the same QK^T product; invalid KV slots are
 *              masked when P is formed).  V is the 512 latent columns of the same
 *              row.  Variants: dense paged bf16 cache, FP8 e4m3 cache with one
 *              fp32 scale per 128 latent columns (rope kept in bf16), the
 *              all-FP8 cache with one per-tensor scale that mla_kv_insert
 *              writes, and top-k sparse index lists.
 *
 *  mla_query   The query front end of the vLLM MlaQuery kernel (API page of
 *              vllm.models.kimi_k3...mla.query, class MlaQuery, method
 *              `kernel`): RMSNorm of the 1536-wide q_a part of qkv with w_qa,
 *              Q_B projection to 192 rows per head (128 nope + 64 rope), W_UK
 *              absorption of the nope rows into 512 latent columns, and e4m3
 *              encoding of [absorbed 512 | rope 64] after multiplying by
 *              q_scale_inv.  Intermediates are rounded to bf16 after RMSNorm,
 *              after Q_B and after W_UK, as on that page.
 *
 *  mla_kv_insert  The KV-cache insert of the same vLLM MlaQuery page (method
 *              `insert`): RMSNorm of each new token's 512-wide latent KV row
 *              (qkv columns 1536..2047) with w_kva, rounded to bf16, then the
 *              e4m3 codes of (normed * k_scale_inv) and of the 64 rope values
 *              (qkv columns 2048..2111) * k_scale_inv written to the token's
 *              cache slot: page slot / 64, row slot % 64.  A slot < 0 writes
 *              nothing.
 *
 * Conventions (all entry points):
 *  - Every data pointer is device memory owned by the caller.  The library
 *    keeps no per-call state and allocates no device memory in these calls;
 *    scratch space is the caller's `workspace`, sized by the *_workspace_size
 *    call, except in mla_decode_noalloc, which uses a library-owned static
 *    device array instead.  Host structs are read during the call only.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the legacy
 *    default stream) and may be issued from several host threads on different
 *    streams.  Two calls that share a workspace must be ordered on one stream.
 *  - Arguments are validated on the host before any HIP call; on a validation
 *    error nothing is launched and outputs are untouched.  Return value 0 on
 *    success, a negative MLA_ERR_* code otherwise; mla_status_string() names it.
 *  - Device-side preconditions that cannot be checked without reading device
 *    memory are stated per argument; the kernels clamp every table-derived
 *    index into its documented range so that a violated precondition yields
 *    wrong values, never an out-of-bounds access.
 *  - Layouts are row-major and contiguous unless a stride is given.
 *  - bf16 = IEEE binary32 upper half; FP8 = OCP e4m3fn (max 448, 0x7F/0xFF NaN).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1)  /* null pointer, non-positive size, bad enum */
#define MLA_ERR_UNSUPPORTED (-2)  /* shape/dtype combination not implemented */
#define MLA_ERR_WORKSPACE (-3)    /* workspace NULL or smaller than required */
#define MLA_ERR_LAUNCH (-4)       /* a kernel launch failed (hipGetLastError) */
#define MLA_ERR_DEVICE (-5)       /* no usable HIP device / device query failed */
#define MLA_ERR_SCRATCH_LIMIT (-6) /* mla_decode_noalloc: the problem needs more than MLA_DECODE_SCRATCH_BYTES */

/* ---- element types ---- */
#define MLA_DTYPE_BF16 1
#define MLA_DTYPE_FP8_E4M3 2
/* KV cache only: every one of the 576 columns (rope too) is an e4m3 code of
   value * k_scale_inv, one fp32 k_scale_inv for the whole cache (the layout
   mla_kv_insert writes). */
#define MLA_DTYPE_FP8_E4M3_TENSOR 3

/* ---- fixed geometry ---- */
#define MLA_D_QK 576        /* latent row width: 512 nope + 64 rope */
#define MLA_D_V 512         /* value width: the 512 nope columns */
#define MLA_PAGE_SIZE 64    /* tokens per KV page */
#define MLA_FP8_ROW_BYTES 640 /* FP8 cache row: 512 e4m3 codes + 64 bf16 rope */
#define MLA_FP8T_ROW_BYTES 576 /* per-tensor FP8 cache row: 576 e4m3 codes */
#define MLA_QKV_WIDTH 2112  /* qkv row read by mla_kv_insert: q_a 1536 | latent 512 | rope 64 */
#define MLA_MAX_INSERT_TOKENS (1 << 24)
#define MLA_MAX_TOKENS_PER_SEQ 16
#define MLA_MAX_HEADS 128
#define MLA_MAX_BATCH 8192
/* Size of the library-owned decode scratch of mla_decode_noalloc (64 MiB per GPU). */
#define MLA_DECODE_SCRATCH_BYTES ((size_t)64 << 20)

typedef struct mla_decode_params {
  int32_t batch;             /* B >= 1, <= MLA_MAX_BATCH */
  int32_t heads;             /* H: 8, 16, 32, 64 or 128 query heads (one token each) */
  int32_t num_pages;         /* pages in the KV pool, >= 1 */
  int32_t max_pages_per_seq; /* columns of block_table, >= 1 */
  int32_t topk;              /* 0: dense over [0, seqlen); > 0: entries per row of topk_idx */
  int32_t q_dtype;           /* MLA_DTYPE_BF16 or MLA_DTYPE_FP8_E4M3 */
  int32_t kv_dtype;          /* MLA_DTYPE_BF16, MLA_DTYPE_FP8_E4M3 or MLA_DTYPE_FP8_E4M3_TENSOR */
  float softmax_scale;       /* multiplies the full 576-wide dot, e.g. 192^-0.5 */
  float q_descale;           /* FP8 queries: value = code * q_descale (= 1/q_scale_inv); ignored for bf16 */
  int32_t tokens_per_seq;    /* T new query tokens per sequence, 1 <= T <= MLA_MAX_TOKENS_PER_SEQ */
} mla_decode_params;

/*
 * Bytes of scratch that mla_decode needs for `p` on the current HIP device
 * (split-KV partial results and a record per sequence of where its pieces
 * are).  Writes *bytes; queries the device's compute unit count, so it
 * returns MLA_ERR_DEVICE without a GPU.
 */
int32_t mla_decode_workspace_size(const mla_decode_params* p, size_t* bytes);

/*
 * Clear the per-sequence records of a decode workspace for `p`
 * (asynchronously on `stream`, with a kernel, no memset node).  mla_decode
 * rewrites every record it reads back in the same call, so this is optional;
 * it keeps a freshly allocated workspace free of stale bytes.
 */
int32_t mla_decode_workspace_init(const mla_decode_params* p, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Absorbed MLA decode of T = tokens_per_seq new query tokens per sequence.
 * With T > 1 (multi-token prediction, speculative decode) the mask is causal:
 * the cache already holds the T new tokens, and query token t (0-based) sees
 * positions [0, seqlens[b] - T + 1 + t).  The STAGE_D2 note packs the T*H
 * query rows of a sequence into one tile; here a dense decode reads each KV
 * row once for all T*H rows.
 *
 *  q           [B, T, H, 576] bf16, or e4m3 codes when q_dtype is FP8 (the
 *              MlaQuery output layout: cols 0..511 absorbed latent q, 512..575
 *              rope q).  Row stride 576 elements.
 *  kv_cache    bf16 cache: [num_pages, 64, 576] bf16.
 *              FP8 cache:  [num_pages, 64, 640] bytes per row = 512 e4m3 codes
 *              of the latent columns, then the 64 rope values as bf16.
 *              Per-tensor FP8 cache: [num_pages, 64, 576] e4m3 codes.
 *  block_table [B, max_pages_per_seq] int32: physical page of logical page j of
 *              sequence b; logical position t lives in row
 *              block_table[b, t/64]*64 + t%64 (the page/offset split of a slot
 *              in MlaQuery.insert).  Precondition: entries in [0, num_pages).
 *  seqlens     [B] int32: tokens of each sequence (the T new ones included).
 *              Precondition: 0 <= seqlens[b] <= 64*max_pages_per_seq.  A query
 *              token with nothing to attend gets O = 0 and LSE = -inf.
 *  topk_idx    NULL when topk == 0; else [B, T, topk] int32 logical positions
 *              (sparse decode), one list per query token.  Entries that are -1
 *              or outside [0, seqlens[b] - T + 1 + t) are masked (contribute
 *              nothing); duplicates count once per entry.
 *  kv_scales   NULL for a bf16 cache; for an FP8 cache [num_pages, 64, 4] fp32,
 *              one scale per row and 128-column tile: k[d] = code[d]*scale[d/128]
 *              for d < 512.  Per-tensor FP8 cache: one fp32, the k_scale_inv
 *              the cache was written with; k[d] = code[d] / k_scale_inv for all
 *              576 columns.  Precondition: k_scale_inv finite and > 0.
 *  out         [B, T, H, 512] bf16 (round to nearest even).
 *  lse         [B, T, H] fp32, natural-log log-sum-exp of the scaled scores.
 *  workspace   device scratch of at least mla_decode_workspace_size bytes;
 *              its contents are clobbered.  Calls that share a workspace must
 *              be ordered (one stream).
 *
 * Runs two kernels on `stream`: the split-KV decode and, for sequences it
 * split over several KV ranges, the merge of their pieces.
 */
int32_t mla_decode(const mla_decode_params* p, const void* q, const void* kv_cache,
                   const int32_t* block_table, const int32_t* seqlens,
                   const int32_t* topk_idx, const float* kv_scales, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, arguments and kernels, with the scratch taken from a
 * library-owned static device array of MLA_DECODE_SCRATCH_BYTES instead of a
 * workspace argument.  Each GPU the library runs on holds its own copy of
 * that array from the library's first use there until the process ends; its
 * address is looked up on this entry point's first call on a device.
 *
 * Returns MLA_ERR_SCRATCH_LIMIT, launching nothing, when
 * mla_decode_workspace_size(p) exceeds MLA_DECODE_SCRATCH_BYTES (the dense
 * 64 x 128-head, 4096-token decode needs about 50 MB).  Calls no hipMalloc,
 * hipFree or allocating library routine.
 *
 * Every call on a GPU shares that GPU's array, which keeps what the last call
 * left (no call relies on its contents at entry: the decode rewrites every
 * record it reads back).  Calls that overlap on one GPU (on different
 * streams, or from host threads without ordering) race on it and give wrong
 * results: order them on one stream.
 */
int32_t mla_decode_noalloc(const mla_decode_params* p, const void* q, const void* kv_cache,
                           const int32_t* block_table, const int32_t* seqlens,
                           const int32_t* topk_idx, const float* kv_scales, void* out,
                           float* lse, void* stream);

typedef struct mla_query_params {
  int32_t batch;       /* tokens B >= 1, <= MLA_MAX_BATCH */
  int32_t heads;       /* H >= 1, <= MLA_MAX_HEADS */
  int32_t qkv_stride;  /* elements between rows of qkv, >= 1536 */
  float eps;           /* RMSNorm epsilon, >= 0 */
} mla_query_params;

/* Bytes of scratch that mla_query needs for `p` (the bf16 nope rows of Q_B). */
int32_t mla_query_workspace_size(const mla_query_params* p, size_t* bytes);

/*
 * MLA query front end.
 *
 *  qkv         [B, qkv_stride] bf16; columns 0..1535 (q_a) are read.
 *  w_qa        [1536] bf16 RMSNorm weight.
 *  w_qb        [H*192, 1536] bf16; row h*192 + r is head h's Q_B row r
 *              (r < 128 nope, 128 <= r < 192 rope).
 *  w_uk        [H, 128, 512] bf16; absorbed q[h, c] = sum_p qb_nope[h, p] * w_uk[h, p, c].
 *  q_scale_inv device fp32 scalar; FP8 output = e4m3(value * q_scale_inv[0]),
 *              rounded to nearest even and saturated to +-448 (never 0xFF).
 *  out         [B, H, 576] e4m3 codes: cols 0..511 the absorbed latent query,
 *              512..575 the rope query.
 *  workspace   at least mla_query_workspace_size bytes.
 *
 *  RMSNorm: rr = 1/sqrt(sum(x^2)/1536 + eps), xn = bf16((x*rr)*w_qa).
 */
int32_t mla_query(const mla_query_params* p, const void* qkv, const void* w_qa,
                  const void* w_qb, const void* w_uk, const float* q_scale_inv,
                  void* out, void* workspace, size_t workspace_bytes, void* stream);

typedef struct mla_kv_insert_params {
  int32_t tokens;      /* T new tokens, 0 <= T <= MLA_MAX_INSERT_TOKENS (0: nothing is launched) */
  int32_t num_pages;   /* pages in the cache, >= 1, num_pages*64 <= INT32_MAX */
  int32_t qkv_stride;  /* elements between rows of qkv, >= 2112, a multiple of 8 */
  float eps;           /* RMSNorm epsilon, >= 0 */
} mla_kv_insert_params;

/*
 * KV-cache insert into the per-tensor FP8 cache (vLLM MlaQuery page, method
 * `insert`; it runs there beside the query front end).
 *
 *  qkv         [T, qkv_stride] bf16; columns 1536..2047 are the latent KV row,
 *              2048..2111 the rope key.
 *  w_kva       [512] bf16 RMSNorm weight.
 *  slots       [T] int64: the cache slot of each token, page slot / 64 and row
 *              slot % 64.  Negative slots are skipped.  Precondition: the
 *              non-negative slots are distinct and < num_pages*64 (a slot past
 *              the end is skipped, never written out of bounds; which of two
 *              equal slots lands is unspecified).
 *  k_scale_inv device fp32 scalar; codes are e4m3(value * k_scale_inv[0]),
 *              rounded to nearest even from the exact product and saturated
 *              to +-448 (never 0xFF).
 *  kv_cache    [num_pages, 64, 576] e4m3 codes (MLA_DTYPE_FP8_E4M3_TENSOR
 *              layout); only the rows of the given slots are written.
 *
 *  RMSNorm: rr = 1/sqrt(sum(x^2)/512 + eps) over the 512 latent values,
 *  normed = bf16((x*rr)*w_kva); the rope values are encoded as they are.
 *  No workspace.  One kernel on `stream`.
 */
int32_t mla_kv_insert(const mla_kv_insert_params* p, const void* qkv, const void* w_kva,
                      const int64_t* slots, const float* k_scale_inv, void* kv_cache, void* stream);

/* Static text for a status code. */
const char* mla_status_string(int32_t status);

/* Library ABI version (major*10000 + minor*100 + patch). */
int32_t mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
