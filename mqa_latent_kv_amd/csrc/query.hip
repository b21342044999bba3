// query.hip - MLA query front end for gfx950 (MI355X).
//
// What is computed, per token b (the query front end of the vLLM MlaQuery
// page, its narrow-batch `kernel` and wide-batch `tiled` forms):
//   rr  = 1 / sqrt(sum_k x[k]^2 / 1536 + eps)      x = qkv[b, 0:1536] (q_a)
//   xn  = bf16((x * rr) * w_qa)                    RMSNorm
//   qb  = bf16(xn . W_qb^T)                        [H, 192]: 128 nope + 64 rope
//   ql  = bf16(qb[:, :128] . W_uk[h])              [H, 512]: absorbed latent q
//   out = e4m3(ql * qsi) | e4m3(qb[:, 128:] * qsi)  qsi = q_scale_inv[0]
// with e4m3 rounded to nearest even and saturated to +-448.
//
// Above 128 tokens, three kernels, the products on v_mfma_f32_32x32x16_bf16
// with 32 tokens as M (from 9 to 128 tokens, the two kernels of the medium
// form further below):
//  * mla_norm_kernel: the RMSNorm of every token, once, into the workspace.
//  * mla_qb_kernel: a workgroup owns 32 tokens, 32 rows of W_qb and (when
//    the tiles alone would not fill the chip, e.g. 64 tokens x 8 heads) a
//    quarter of the 1536-long reduction; its four waves each take a quarter
//    of its columns with both operands loaded straight from memory, the four
//    partial tiles are summed in LDS in a fixed order and stored as fp32.
//  * mla_ql_kernel: a workgroup owns 32 tokens, one head and 128 output
//    columns; the W_uk tile [128 p][128 c] is staged in LDS and read as the B
//    operand with ds_read_b64_tr_b16 (W_uk is stored c-contiguous, the
//    reduction runs over p).  The A operand is the nope q: the Q_B partials
//    added in split order and rounded to bf16.  The workgroups of column
//    block 0 also encode the rope rows of Q_B to FP8.
//
// Up to eight tokens take the page's narrow-batch form instead: the two
// products are GEMVs bound by reading the weights, computed with wave FMAs
// in many small workgroups (mla_qb_gemv_kernel, mla_ql_gemv_kernel).
//
// And the KV-cache insert of the same page (method `insert`), per new token t
// with slot >= 0:
//   rr   = 1 / sqrt(sum_k x[k]^2 / 512 + eps)      x = qkv[t, 1536:2048]
//   row  = e4m3(bf16((x * rr) * w_kva) * ksi) | e4m3(qkv[t, 2048:2112] * ksi)
//   cache[slot / 64][slot % 64][0:576] = row        ksi = k_scale_inv[0]
//  * mla_kv_insert_kernel: one wave per token, all in registers (lane l holds
//    latent values 8l..8l+7 and rope value l); the sum of squares is a DPP
//    wave reduction, so the kernel has no LDS and no barrier.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS char lds_char;

constexpr int kQA = 1536;       // q_a width (RMSNorm length, Q_B reduction)
constexpr int kQB = 192;        // Q_B rows per head
constexpr int kNope = 128;      // nope rows of Q_B (W_UK reduction)
constexpr int kDV = 512;        // absorbed latent width
constexpr int kOut = 576;       // output row: 512 latent + 64 rope
constexpr int kThreads = 256;
constexpr int kTok = 32;        // tokens per workgroup (MFMA M)

struct QueryArgs {
  const __bf16* qkv;
  const __bf16* w_qa;
  const __bf16* w_qb;
  const __bf16* w_uk;
  const float* q_scale_inv;
  uint8_t* out;
  __bf16* qn;   // workspace, narrow batch: [B][H][128] bf16 nope rows of Q_B
  __bf16* xn;   // workspace, tiled: [B][1536] normalised q_a rows
  float* qbp;   // workspace, tiled: [ksplit][B][H*192] fp32 partial Q_B products
  __bf16* qbm;  // workspace, medium batch: [B][H*192] bf16 Q_B
  int32_t batch, heads, qkv_stride;
  float eps;
};

// e4m3fn code of the exact product v * q (v at most 24 significant bits, q
// fp32): round to nearest even, saturate to +-448, NaN -> 0x7F.  The
// product is rounded once, from its exact value: an fp32 product can land
// exactly on an e4m3 midpoint (v * 0.3f does whenever v * 3/10 is one) and
// would then break the tie by its own rounding error.  hi = fl(v * q) and
// lo = fma(v, q, -hi) = v * q - hi exactly; every e4m3 midpoint is an fp32
// number, so the exact value lies on the same side of each midpoint as hi,
// except when hi is the midpoint itself, where the sign of lo (in magnitude)
// decides and lo = 0 is a true tie.  Normal range (|hi| >= 2^-6): the three
// leading mantissa bits of hi are the e4m3 mantissa and the twenty below are
// the discarded part (half = 0x80000); below 2^-6 the step is the subnormal
// 2^-9 and |hi| * 512 (exact) is rounded to an integer 0..8.
__host__ __device__ __forceinline__ uint8_t e4m3_of_product(float v, float q) {
  const float hi = v * q;
  if (hi != hi) return 0x7F;
  const float lo = __builtin_fmaf(v, q, -hi);
  const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
  const uint32_t sign = (hb >> 24) & 0x80u;
  const float a = __builtin_fabsf(hi);
  // where the exact magnitude lies relative to |hi|: above (+1), below (-1)
  const int dir = lo == 0.0f ? 0 : ((lo > 0.0f) == (hi > 0.0f) ? 1 : -1);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7E;
  } else if (a < 0.015625f) {  // 2^-6: subnormal codes 0..7 (8 is the smallest normal)
    const float t = a * 512.0f;
    const float n = __builtin_floorf(t);
    const float f = t - n;
    const uint32_t ni = (uint32_t)n;
    const bool up = f > 0.5f || (f == 0.5f && (dir > 0 || (dir == 0 && (ni & 1u))));
    code = ni + (up ? 1u : 0u);
  } else {
    const uint32_t ab = __builtin_bit_cast(uint32_t, a);
    const uint32_t e = (ab >> 23) - 120u;  // e4m3 exponent field 1..15
    const uint32_t m3 = (ab >> 20) & 7u, rest = ab & 0xFFFFFu;
    const bool up = rest > 0x80000u || (rest == 0x80000u && (dir > 0 || (dir == 0 && (m3 & 1u))));
    code = ((e << 3) | m3) + (up ? 1u : 0u);  // a mantissa carry moves into the exponent field
    code = code > 0x7Eu ? 0x7Eu : code;       // rounding up past 448 saturates
  }
  return (uint8_t)(sign | code);
}

// The same codes for two products v0 * q and v1 * q (bits 0..7 and 8..15),
// mostly by the hardware conversion: it rounds its fp32 input to nearest
// even, so fed the fp32 product hi clamped to +-448 (which it encodes as
// 0x7E / 0xFE, the saturation above) it returns the exact product's code
// unless hi is an e4m3 midpoint with lo != 0, the one case where the exact
// value and hi round apart.  Those products, and NaN, take the encoder above
// (rare: the branch is almost never taken by any lane).  Midpoints: in the
// normal range the fp32 bits below the three kept mantissa bits are exactly
// half (0x80000); below 2^-6, adding 2^-6 moves the subnormal step 2^-9 onto
// that same mantissa bit, and a midpoint (k + 1/2) 2^-9 stays exact (an
// inexact sum can only add a false alarm, which the exact encoder absorbs).
// Computed without branches.
__device__ __forceinline__ uint32_t e4m3_needs_exact(float v, float q, float hi) {
  const float lo = __builtin_fmaf(v, q, -hi);
  const float a = __builtin_fabsf(hi);
  const float s = a < 0.015625f ? a + 0.015625f : a;
  const uint32_t mid = (__builtin_bit_cast(uint32_t, s) & 0xFFFFFu) == 0x80000u;
  return (uint32_t)(hi != hi) | ((uint32_t)(lo != 0.0f) & mid);
}
__device__ __forceinline__ uint32_t e4m3x2_of_products(float v0, float v1, float q) {
  const float h0 = v0 * q, h1 = v1 * q;
  const float c0 = __builtin_fminf(__builtin_fmaxf(h0, -448.0f), 448.0f);
  const float c1 = __builtin_fminf(__builtin_fmaxf(h1, -448.0f), 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false) & 0xFFFFu;
  if (__builtin_expect(e4m3_needs_exact(v0, q, h0) | e4m3_needs_exact(v1, q, h1), 0))
    r = (uint32_t)e4m3_of_product(v0, q) | ((uint32_t)e4m3_of_product(v1, q) << 8);
  return r;
}

// Sum over the 64 lanes, every lane receiving it, in registers only: two
// quad permutations, the half-row and row mirrors (16 lanes summed), then
// the 16- and 32-lane swaps.  (A shuffle loop would go through ds_bpermute,
// six dependent round trips through the LDS crossbar.)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror: the other quad of the 8-lane half
  v += dpp_f<0x140>(v);  // row_mirror: the other half of the 16-lane row
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// ---------------------------------------------------------------- KV-cache insert

constexpr int kQkvLatent = 1536;  // first qkv column of the latent KV row
constexpr int kQkvRope = 2048;    // first qkv column of the rope key
constexpr int kLatent = 512;
constexpr int kCacheRow = 576;    // per-tensor FP8 cache row: 576 e4m3 codes
constexpr int kCachePage = 64;

struct InsertArgs {
  const __bf16* qkv;
  const __bf16* w_kva;
  const int64_t* slots;
  const float* k_scale_inv;
  uint8_t* cache;
  int64_t cache_rows;  // num_pages * 64
  int32_t tokens, qkv_stride;
  float eps;
};

__global__ void __launch_bounds__(kThreads) mla_kv_insert_kernel(InsertArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= a.tokens) return;  // whole waves
  // every load is issued before the slot decides anything (one memory latency)
  const int64_t slot = a.slots[t];
  const __bf16* row = a.qkv + (size_t)t * a.qkv_stride;
  const bf16x8 x = *(const bf16x8*)(row + kQkvLatent + 8 * lane);
  const bf16x8 wv = *(const bf16x8*)(a.w_kva + 8 * lane);
  const float rope = (float)row[kQkvRope + lane];
  const float ksi = *a.k_scale_inv;
  // (the empty asm takes the loaded values, so the compiler cannot sink the
  // loads below the branch)
  asm volatile("" ::"v"(x), "v"(wv), "v"(rope), "s"(ksi));
  if (slot < 0 || slot >= a.cache_rows) return;  // skipped token (uniform per wave)
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = __builtin_fmaf((float)x[i], (float)x[i], ss);
  ss = wave_sum(ss);
  // 1/512 is a power of two: the mean is the exact quotient
  const float rr = 1.0f / __builtin_sqrtf(ss * (1.0f / kLatent) + a.eps);
  float n[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) n[i] = (float)(__bf16)(((float)x[i] * rr) * (float)wv[i]);  // round to nearest even
  const uint32_t lo = e4m3x2_of_products(n[0], n[1], ksi) | (e4m3x2_of_products(n[2], n[3], ksi) << 16);
  const uint32_t hi = e4m3x2_of_products(n[4], n[5], ksi) | (e4m3x2_of_products(n[6], n[7], ksi) << 16);
  uint8_t* dst = a.cache + (size_t)slot * kCacheRow;
  *(uint2*)(dst + 8 * lane) = uint2{lo, hi};
  dst[kLatent + lane] = e4m3_of_product(rope, ksi);
}

// ---------------------------------------------------------------- RMSNorm + Q_B

// RMSNorm of the q_a rows into the workspace (bf16): one wave per token,
// lane l holding columns 512k + 8l .. +7 (k = 0..2).
__global__ void __launch_bounds__(kThreads) mla_norm_kernel(QueryArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= a.batch) return;  // wave-uniform
  bf16x8 xr[3], wq[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    xr[k] = *(const bf16x8*)(a.qkv + (size_t)t * a.qkv_stride + 512 * k + 8 * lane);
    wq[k] = *(const bf16x8*)(a.w_qa + 512 * k + 8 * lane);
  }
  float x[24];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[8 * k + e] = (float)xr[k][e];
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 24; ++e) ss += x[e] * x[e];
  ss = wave_sum(ss);
  const float rr = 1.0f / __builtin_sqrtf(ss / (float)kQA + a.eps);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)((x[8 * k + e] * rr) * (float)wq[k][e]);
    *(bf16x8*)(a.xn + (size_t)t * kQA + 512 * k + 8 * lane) = o;
  }
}

// Q_B: a workgroup owns 32 tokens, 32 rows of W_qb and 1/KSPLIT of the
// 1536-long reduction (KSPLIT = 4 when the tiles alone would leave most
// compute units idle, e.g. 64 tokens x 8 heads); its four waves take a
// quarter of its columns each, with both operands loaded straight from
// memory (all of a wave's fragments in flight at once).  The four partial
// tiles are summed in LDS in a fixed order and stored as an fp32 partial.
template <int KSPLIT>
__global__ void __launch_bounds__(kThreads) mla_qb_kernel(QueryArgs a) {
  __shared__ __attribute__((aligned(16))) f32x4 red[4 * 4 * 64];  // partial tiles of waves 1..3
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n0 = blockIdx.x * 32;    // first W_qb row (output column) of this workgroup
  const int m0 = blockIdx.y * kTok;  // first token
  constexpr int KW = kQA / KSPLIT / 4;  // reduction columns per wave
  constexpr int KSW = KW / 16;          // k-steps per wave
  const int k0 = blockIdx.z * (kQA / KSPLIT) + KW * w;
  const int nrows = a.heads * kQB;
  // lane l: B = W_qb row n0 + l%32, A = token m0 + l%32, columns 16i + 8*(l/32)
  // .. +7 of this wave's range (clamped rows, unconditional loads; values of
  // rows past the end are zeroed)
  const int nrow = n0 + (lane & 31), h8 = 8 * (lane >> 5);
  const bool row_ok = nrow < nrows;
  const int nrow_c = row_ok ? nrow : nrows - 1;
  const int b = m0 + (lane & 31);
  const bool b_ok = b < a.batch;
  const int b_c = b_ok ? b : a.batch - 1;
  bf16x8 bf[KSW], af[KSW];
#pragma unroll
  for (int i = 0; i < KSW; ++i) {
    bf[i] = *(const bf16x8*)(a.w_qb + (size_t)nrow_c * kQA + k0 + 16 * i + h8);
    af[i] = *(const bf16x8*)(a.xn + (size_t)b_c * kQA + k0 + 16 * i + h8);
  }
  f32x16 acc = {};
#pragma unroll
  for (int i = 0; i < KSW; ++i) {
    const bf16x8 x = b_ok ? af[i] : bf16x8{};
    const bf16x8 y = row_ok ? bf[i] : bf16x8{};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc, 0, 0, 0);
  }
  // fixed-order sum of the four partial tiles
  if (w > 0) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      red[((w - 1) * 4 + r4) * 64 + lane] = f32x4{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    f32x4 s = {acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
#pragma unroll
    for (int j = 0; j < 3; ++j) s += red[(j * 4 + r4) * 64 + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[4 * r4 + e] = s[e];
  }
  if (!row_ok) return;
  // lane l, register r: token m0 + 8*(r/4) + 4*(l/32) + r%4, W_qb row nrow
  float* const dst = a.qbp + (size_t)blockIdx.z * a.batch * nrows;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int bb = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (bb >= a.batch) continue;
    dst[(size_t)bb * nrows + nrow] = acc[i];
  }
}

// ---------------------------------------------------------------- W_UK absorption + FP8

// LDS tile of W_uk[h][p][c0 .. c0+127]: 128-byte rows (64 columns) in two
// column groups of 128 rows, 16-byte chunks XOR-swizzled by bits 1..3 of the
// row (the layout the decode kernel uses for its V^T reads).
constexpr int kUkGroup = 128 * 128;  // bytes per column group
__device__ __forceinline__ int uk_swz(int m) { return (((m >> 1) & 1) << 2) | (((m >> 3) & 1) << 1) | ((m >> 2) & 1); }

constexpr int kQsPitch = kNope + 8;  // LDS row pitch (bf16 elements) of the nope q tile
template <int KSPLIT>
__global__ void __launch_bounds__(kThreads) mla_ql_kernel(QueryArgs a) {
  __shared__ __attribute__((aligned(16))) char uk_mem[2 * kUkGroup];
  __shared__ __attribute__((aligned(16))) __bf16 qs_mem[kTok * kQsPitch];  // nope q tile, bf16
  LDS_AS __bf16* const qs = (LDS_AS __bf16*)qs_mem;
  lds_char* const uk = (lds_char*)uk_mem;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int head = blockIdx.x, c0 = blockIdx.y * 128, m0 = blockIdx.z * kTok;

  // this lane's token in the A operand (rows past the batch are zeroed)
  const int b = m0 + (lane & 31);
  const bool b_ok = b < a.batch;
  // The nope q tile [32 tokens][128] in LDS as bf16: the KSPLIT fp32 partials
  // of Q_B added in split order and rounded once.  Thread i reads four
  // consecutive values of token i/32 from each partial (a token's 512 bytes
  // come from 32 neighbouring threads).
  const size_t nrows = (size_t)a.heads * kQB;
  f32x4 qp[4][KSPLIT];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + j * kThreads, t = i >> 5, c4 = 4 * (i & 31);
    const int bt = min(m0 + t, a.batch - 1);
#pragma unroll
    for (int k = 0; k < KSPLIT; ++k)
      qp[j][k] = *(const f32x4*)(a.qbp + ((size_t)k * a.batch + bt) * nrows + (size_t)head * kQB + c4);
  }
  // W_uk[head][0..127][c0..c0+127]: 2048 chunks of 16 bytes, all eight of a
  // thread requested (with the partials above) before anything is stored
  constexpr int kStage = 128 * 16 / kThreads;
  u32x4 wv[kStage];
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int i = tid + j * kThreads, p = i >> 4, ch = i & 15;  // row p, chunk ch (8 columns)
    wv[j] = *(const u32x4*)(a.w_uk + ((size_t)head * kNope + p) * kDV + c0 + 8 * ch);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + j * kThreads, t = i >> 5, c4 = 4 * (i & 31);
    f32x4 sum = qp[j][0];
#pragma unroll
    for (int k = 1; k < KSPLIT; ++k) sum += qp[j][k];
    *(LDS_AS bf16x4*)(qs + t * kQsPitch + c4) = __builtin_convertvector(sum, bf16x4);
  }
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int i = tid + j * kThreads, p = i >> 4, ch = i & 15;
    const int g = ch >> 3, x = ch & 7;
    *(LDS_AS u32x4*)(uk + g * kUkGroup + p * 128 + 16 * (x ^ uk_swz(p))) = wv[j];
  }
  __syncthreads();
  // A fragments: token m0 + l%32 (rows past the batch zeroed), nope columns
  // 16ks + 8*(l/32) .. +7
  bf16x8 af[kNope / 16];
#pragma unroll
  for (int ks = 0; ks < kNope / 16; ++ks) {
    af[ks] = *(const LDS_AS bf16x8*)(qs + (lane & 31) * kQsPitch + 16 * ks + 8 * (lane >> 5));
    af[ks] = b_ok ? af[ks] : bf16x8{};
  }
  // B operand B[k][n] = W_uk[head][16ks + k][c] by transposed reads: lane l
  // needs column n = l%32 of rows k = 8*(l/32) + i, i = 0..7, the order the A
  // operand uses.  Wave w owns columns c0 + 32w .. +31; within 16-lane group
  // G, lane 4j + q supplies columns 16*(G&1) + 4q .. +3 of row 8*(G>>1) +
  // 4tt + j for element group tt (elements 4tt .. 4tt+3 of every lane).
  const int G = lane >> 4, i16 = lane & 15, j = i16 >> 2, q = i16 & 3, hh = G >> 1, cpart = G & 1;
  uint32_t va[2];
  for (int tt = 0; tt < 2; ++tt) {
    const int m = 8 * hh + 4 * tt + j;
    va[tt] = (w >> 1) * kUkGroup + m * 128 + 16 * (((2 * cpart + (q >> 1)) ^ uk_swz(m))) + 8 * (q & 1);
    if (w & 1) va[tt] ^= 64u;
  }
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < kNope / 16; ++ks) {
    // rows 16ks .. 16ks+15: the swizzle only sees bits 1..3, so 16ks moves the
    // address by whole rows
    const bf16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(uk + va[0] + ks * 16 * 128));
    const bf16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(uk + va[1] + ks * 16 * 128));
    const bf16x8 bfr = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], bfr, acc, 0, 0, 0);
  }
  // lane l, register r: token m0 + 8*(r/4) + 4*(l/32) + r%4, column c0 + 32w + l%32
  const float qsi = a.q_scale_inv[0];
  const int c = c0 + 32 * w + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t cc = e4m3x2_of_products((float)(__bf16)acc[i], (float)(__bf16)acc[i + 1], qsi);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int bb = m0 + 8 * ((i + k) >> 2) + 4 * (lane >> 5) + ((i + k) & 3);
      if (bb < a.batch) a.out[((size_t)bb * a.heads + head) * kOut + c] = (uint8_t)(cc >> (8 * k));
    }
  }
  // the rope rows of Q_B go to the output as they are (bf16 of the summed
  // partials, then FP8): the workgroups of column block 0, eight values per
  // thread
  if (blockIdx.y == 0) {
    const int t = m0 + (tid >> 3), r0 = kNope + 8 * (tid & 7);
    if (t < a.batch) {
      f32x4 s0 = {}, s1 = {};
#pragma unroll
      for (int k = 0; k < KSPLIT; ++k) {
        const float* src = a.qbp + ((size_t)k * a.batch + t) * nrows + (size_t)head * kQB + r0;
        s0 += *(const f32x4*)src;
        s1 += *(const f32x4*)(src + 4);
      }
      uint8_t* dst = a.out + ((size_t)t * a.heads + head) * kOut + kDV + (r0 - kNope);
      uint32_t w4[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 sv = h ? s1 : s0;
        w4[h] = e4m3x2_of_products((float)(__bf16)sv[0], (float)(__bf16)sv[1], qsi) |
                (e4m3x2_of_products((float)(__bf16)sv[2], (float)(__bf16)sv[3], qsi) << 16);
      }
      *(uint2*)dst = uint2{w4[0], w4[1]};
    }
  }
}


// ---------------------------------------------------------------- narrow batch: wave FMAs

// Up to kNarrow tokens, the MlaQuery page's narrow-batch form: the products
// are GEMVs whose cost is reading the weights once, so the weights are
// spread over many workgroups and reduced with wave FMAs; no MFMA tile would
// be more than a quarter full.
constexpr int kNarrow = 8;                                  // batches up to this size take this path
constexpr int kQbLanes = 8;                                 // lanes per W_qb row
constexpr int kQbRowsPerWave = 64 / kQbLanes;               // 8
constexpr int kQbRowsPerWg = kQbRowsPerWave * (kThreads / 64);  // 32 W_qb rows per workgroup
constexpr int kQbLoads = kQA / (kQbLanes * 8);              // 24 loads of 8 weights per lane

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// RMSNorm + Q_B: a workgroup owns 32 rows of W_qb (8 per wave) for every
// token; eight lanes share a row, lane s of a row holding columns 64k + 8s
// .. +7 (k = 0..23), so that each load instruction reads 128 contiguous
// bytes of each of the wave's eight rows, and all 24 loads are issued before
// anything else.  Each wave normalises tokens w, w + 4 into LDS (the
// workgroup's every token), then every lane forms the dot products of its
// 192 weights with every token (bf16 pairs multiplied and added in fp32 by
// v_dot2c_f32_bf16, reading the token's matching 8 columns from LDS, the
// same 128 bytes for all eight rows), and the eight lanes of a row add their
// sums (three lane swaps).
__global__ void __launch_bounds__(kThreads) mla_qb_gemv_kernel(QueryArgs a) {
  __shared__ __attribute__((aligned(16))) bf16x8 xn[kNarrow][kQA / 8];  // normalised tokens, 24 KB
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nrows = a.heads * kQB;
  const int sub = lane & (kQbLanes - 1);
  const int row = blockIdx.x * kQbRowsPerWg + kQbRowsPerWave * w + lane / kQbLanes;
  // every load first: w_qa and the q_a rows of the tokens this wave
  // normalises, then this lane's W_qb weights (row clamped, unconditional);
  // loads complete in order, so the normalisation runs while the weights
  // are still arriving, and the products follow them in
  bf16x8 wq[3], xr[2][3];
#pragma unroll
  for (int k = 0; k < 3; ++k) wq[k] = *(const bf16x8*)(a.w_qa + 512 * k + 8 * lane);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = min(w + 4 * i, a.batch - 1);
#pragma unroll
    for (int k = 0; k < 3; ++k) xr[i][k] = *(const bf16x8*)(a.qkv + (size_t)t * a.qkv_stride + 512 * k + 8 * lane);
  }
  asm volatile("" ::: "memory");  // (keeps the weight loads behind these)
  bf16x8 wr[kQbLoads];
  {
    const bf16x8* wrow = (const bf16x8*)(a.w_qb + (size_t)min(row, nrows - 1) * kQA) + sub;
#pragma unroll
    for (int k = 0; k < kQbLoads; ++k) wr[k] = wrow[8 * k];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = w + 4 * i;
    if (t >= a.batch) break;  // wave-uniform
    float x[24];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * k + e] = (float)xr[i][k][e];
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 24; ++e) ss += x[e] * x[e];
    ss = wave_sum(ss);
    const float rr = 1.0f / __builtin_sqrtf(ss / (float)kQA + a.eps);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)((x[8 * k + e] * rr) * (float)wq[k][e]);
      xn[t][64 * k + lane] = o;
    }
  }
  __syncthreads();
  float acc[kNarrow];
#pragma unroll
  for (int t = 0; t < kNarrow; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int k = 0; k < kQbLoads; ++k) {
#pragma unroll
    for (int t = 0; t < kNarrow; ++t) {
      if (t >= a.batch) break;  // uniform
      const bf16x8 xv = xn[t][8 * k + sub];
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        acc[t] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{xv[e], xv[e + 1]}, bf16x2{wr[k][e], wr[k][e + 1]}, acc[t],
                                                  false);
    }
  }
#pragma unroll
  for (int t = 0; t < kNarrow; ++t) {
    acc[t] += __shfl_xor(acc[t], 1);
    acc[t] += __shfl_xor(acc[t], 2);
    acc[t] += __shfl_xor(acc[t], 4);
  }
  if (sub != 0 || row >= nrows) return;
  const float qsi = a.q_scale_inv[0];
  const int head = row / kQB, r = row % kQB;
#pragma unroll
  for (int t = 0; t < kNarrow; ++t) {
    if (t >= a.batch) break;
    const __bf16 v = (__bf16)acc[t];
    if (r < kNope) a.qn[((size_t)t * a.heads + head) * kNope + r] = v;
    else a.out[((size_t)t * a.heads + head) * kOut + kDV + (r - kNope)] = e4m3_of_product((float)v, qsi);
  }
}

// W_UK absorption + FP8: a workgroup owns one head and 64 output columns for
// every token.  Thread t takes columns c0 + 8(t%8) .. +7 of the W_uk rows p =
// t/8 + 32j (j = 0..3): each row's 128 bytes come from eight neighbouring
// threads.  The 32 partial sums of a column are added in LDS in a fixed
// order, then rounded to bf16 and encoded.
constexpr int kQlCols = 64;
__global__ void __launch_bounds__(kThreads) mla_ql_gemv_kernel(QueryArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 qs[kNarrow][kNope];                 // the tokens' nope q, 2 KB
  __shared__ __attribute__((aligned(16))) f32x4 red[32][kNarrow][kQlCols / 4];       // partial sums, 64 KB
  const int tid = threadIdx.x;
  const int head = blockIdx.x, c0 = blockIdx.y * kQlCols;
  const int cg = tid & 7, g = tid >> 3;
  u32x4 wv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wv[j] = *(const u32x4*)(a.w_uk + ((size_t)head * kNope + g + 32 * j) * kDV + c0 + 8 * cg);
  {
    // nope q of every token: thread t loads 4 values of token t/32
    const int t = tid >> 5, p4 = 4 * (tid & 31);
    if (t < a.batch) *(LDS_AS bf16x4*)&qs[t][p4] = *(const bf16x4*)(a.qn + ((size_t)t * a.heads + head) * kNope + p4);
  }
  __syncthreads();
  for (int t = 0; t < a.batch; ++t) {
    float acc[8] = {};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float qv = (float)qs[t][g + 32 * j];
      const bf16x8 wb = __builtin_bit_cast(bf16x8, wv[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(qv, (float)wb[e], acc[e]);
    }
    red[g][t][2 * cg] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    red[g][t][2 * cg + 1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  __syncthreads();
  const float qsi = a.q_scale_inv[0];
  for (int o = tid; o < a.batch * kQlCols; o += kThreads) {
    const int t = o / kQlCols, c = o % kQlCols;
    float s = 0.0f;
    for (int gg = 0; gg < 32; ++gg) s += red[gg][t][c >> 2][c & 3];
    const float v = (float)(__bf16)s;
    a.out[((size_t)t * a.heads + head) * kOut + c0 + c] = e4m3_of_product(v, qsi);
  }
}

// ---------------------------------------------------------------- medium batch: fused RMSNorm + Q_B, then W_UK

// From kNarrow + 1 to kMedium tokens the 32 x 32 tiles are too few to spread
// the weights over the chip, and the three-kernel form pays a launch and a
// dependent load chain per step.  Two kernels instead, with small tiles:
//  * mla_qbn_kernel: a workgroup owns 16 tokens and 32 W_qb rows over the
//    whole 1536-long reduction, an eighth per wave.  It loads its tokens'
//    q_a rows in full anyway (they are the A operand), so it forms their
//    RMSNorm itself: per-wave sums of squares, added in wave order in LDS.
//    v_mfma_f32_16x16x32_bf16 with tokens on M; the four partial tiles are
//    added in wave order and Q_B is stored once, rounded to bf16.
//  * mla_qlm_kernel: a one-wave workgroup owns 32 tokens, one head and 32
//    output columns: W_uk[h][0..127][32 columns] staged in LDS and read with
//    ds_read_b64_tr_b16, the nope rows of Q_B as the A operand, then FP8.
constexpr int kMedium = 128;
constexpr int kMTok = 16;                 // tokens per Q_B workgroup (MFMA M)
constexpr int kMRows = 32;                // W_qb rows per Q_B workgroup (two MFMA N blocks)
constexpr int kQbnThreads = 512;          // eight waves, an eighth of the reduction each
constexpr int kMKs = kQA / 8 / 32;        // k-steps of 32 per wave
constexpr int kUkCols = 32;               // W_UK output columns per workgroup

// One direct global->LDS copy of 16 bytes per lane (lane i's bytes land at
// lds + 16i): base and lds wave-uniform, voff the lane's byte offset.
// (one wait state between the write of m0 and the copy that reads it)
// (m0 is named in the clobber list on purpose: clang warns that it is reserved)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void qdma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ const void* qd_uniform(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Staging of one wave's slice (192 columns = 384 bytes = three 128-byte lines
// per row) of 8-row groups: copy j holds line j / G of rows 8(j % G) .. +7,
// lane i of it row 8(j % G) + i/8 and, at position i % 8, source chunk
// (i % 8) ^ qb_swz(row) of that line.  The XOR spreads the 16 rows that one
// fragment read touches over all 64 banks.
__device__ __forceinline__ int qb_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// LDS byte offset of chunk c (0..23) of row r in a staging of G row groups
template <int G>
__device__ __forceinline__ uint32_t qb_stage_off(int r, int c) {
  const int j = G * (c >> 3) + (r >> 3);
  return 1024u * j + 16u * (8 * (r & 7) + ((c & 7) ^ qb_swz(r)));
}

__global__ void __launch_bounds__(kQbnThreads) mla_qbn_kernel(QueryArgs a) {
  constexpr int W = kQbnThreads / 64;
  constexpr int kXBytes = kMTok * 384, kWBytes = kMRows * 384;  // per wave: 6 + 12 KB, and 1 KB for w_qa
  __shared__ __attribute__((aligned(1024))) char stage[W][kXBytes + kWBytes + 1024];
  __shared__ float ssp[W][kMTok];  // per-wave sums of squares
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const int nrows = a.heads * kQB;
  const int n0 = blockIdx.x * kMRows, m0 = blockIdx.y * kMTok;
  LDS_AS char* const xs = (LDS_AS char*)stage[w];
  LDS_AS char* const wsg = xs + kXBytes;
  const uint32_t xs_a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)xs);
  // copies of this wave's slice, columns 192w .. +191: the tokens' q_a rows
  // (two row groups), then the w_qa slice (lanes 0..23; the others repeat
  // it) and the 32 W_qb rows (four), whole 128-byte lines per eight lanes.
  // Tokens past the batch and rows past the heads read the last valid one
  // (zeroed below).  The RMSNorm only needs the first two, so the W_qb rows
  // keep landing while it runs.
  LDS_AS char* const wqs = xs + kXBytes + kWBytes;
  {
    const int rr = lane >> 3, ch = lane & 7;
    const void* xb = qd_uniform(a.qkv);
    const void* wb = qd_uniform(a.w_qb);
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int r = 8 * (j & 1) + rr, line = j >> 1;
      const int t = min(m0 + r, a.batch - 1);
      const uint32_t off = (uint32_t)t * (uint32_t)a.qkv_stride * 2u + 384u * w + 128u * line + 16u * (ch ^ qb_swz(r));
      qdma16(xb, off, xs_a + 1024u * j);
    }
    qdma16(qd_uniform(a.w_qa), 384u * w + 16u * (lane % 24), xs_a + kXBytes + kWBytes);
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int r = 8 * (j & 3) + rr, line = j >> 2;
      const int n = min(n0 + r, nrows - 1);
      const uint32_t off = (uint32_t)n * (uint32_t)(kQA * 2) + 384u * w + 128u * line + 16u * (ch ^ qb_swz(r));
      qdma16(wb, off, xs_a + kXBytes + 1024u * j);
    }
  }
  // lane l: A = token m0 + l%16, B = W_qb rows n0 + 16nb + l%16 (nb = 0, 1),
  // k-step i: columns 192w + 32i + 8(l/16) .. +7, i.e. chunk 4i + l/16 of the
  // slice
  const int t = m0 + i16;
  const bool t_ok = t < a.batch;
  bool row_ok[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) row_ok[nb] = n0 + 16 * nb + i16 < nrows;
  // vm operations complete in order: all but the twelve W_qb copies done
  // means the q_a rows and the w_qa slice are in
  __builtin_amdgcn_s_waitcnt((12 & 15) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
  bf16x8 xr[kMKs], wq[kMKs];
#pragma unroll
  for (int i = 0; i < kMKs; ++i) {
    xr[i] = *(const LDS_AS bf16x8*)(xs + qb_stage_off<2>(i16, 4 * i + g));
    wq[i] = *(const LDS_AS bf16x8*)(wqs + 16 * (4 * i + g));  // columns 192w + 32i + 8g .. +7
  }
  // sum of squares of token t over this wave's eighth: the lane's 48 values,
  // then the four lanes l, l^16, l^32, l^48 that share the token
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kMKs; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (float)xr[i][e];
      ss = __builtin_fmaf(x, x, ss);
    }
  {
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
    ss = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
    ss = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  }
  if (g == 0) ssp[w][i16] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int v = 0; v < W; ++v) tot += ssp[v][i16];
  const float rr = 1.0f / __builtin_sqrtf(tot / (float)kQA + a.eps);
  bf16x8 xq[kMKs];
#pragma unroll
  for (int i = 0; i < kMKs; ++i) {
    bf16x8 xn;
#pragma unroll
    for (int e = 0; e < 8; ++e) xn[e] = (__bf16)(((float)xr[i][e] * rr) * (float)wq[i][e]);
    xq[i] = t_ok ? xn : bf16x8{};
  }
  // (the empty asm takes the normalised rows, so that the compiler cannot
  // sink their computation below the wait for the W_qb rows)
  asm volatile("" ::"v"(xq[0]), "v"(xq[1]), "v"(xq[2]), "v"(xq[3]), "v"(xq[4]), "v"(xq[5]));
  __builtin_amdgcn_s_waitcnt(0);  // the W_qb rows landed
  asm volatile("" ::: "memory");
  f32x4 acc[2] = {};
#pragma unroll
  for (int i = 0; i < kMKs; ++i) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bf16x8 wv = *(const LDS_AS bf16x8*)(wsg + qb_stage_off<4>(16 * nb + i16, 4 * i + g));
      const bf16x8 y = row_ok[nb] ? wv : bf16x8{};
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xq[i], y, acc[nb], 0, 0, 0);
    }
  }
  // this wave's partial tiles into its own staging (read into registers
  // above; nothing else reads it)
  LDS_AS f32x4* const red = (LDS_AS f32x4*)xs;
  red[lane] = acc[0];
  red[64 + lane] = acc[1];
  __syncthreads();
  // thread (nb, r, l): register r of lane l in block nb, i.e. token
  // m0 + 4(l/16) + r and W_qb row n0 + 16nb + l%16; the waves' tiles added
  // in wave order, rounded to bf16 once
  const int l = tid & 63, r = (tid >> 6) & 3, nb = tid >> 8;
  float v = 0.0f;
#pragma unroll
  for (int u = 0; u < W; ++u) v += ((const LDS_AS f32x4*)stage[u])[64 * nb + l][r];
  const int tt = m0 + 4 * (l >> 4) + r, nn = n0 + 16 * nb + (l & 15);
  if (tt < a.batch && nn < nrows) a.qbm[(size_t)tt * nrows + nn] = (__bf16)v;
}

__global__ void __launch_bounds__(64) mla_qlm_kernel(QueryArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 uk[kNope][kUkCols];  // W_uk[h][p][c0 .. c0+31], 8 KB
  const int lane = threadIdx.x;
  const int head = blockIdx.x, c0 = blockIdx.y * kUkCols, m0 = blockIdx.z * kTok;
  const int nrows = a.heads * kQB;
  // the scale and this lane's two rope values (below) load with everything else
  const float qsi = a.q_scale_inv[0];
  const int rt = m0 + (lane >> 1), rr = 4 * blockIdx.y + 2 * (lane & 1);
  const bool rt_ok = rt < a.batch;
  const __bf16* rsrc = a.qbm + (size_t)min(rt, a.batch - 1) * nrows + (size_t)head * kQB + kNope + rr;
  const __bf16 rv[2] = {rsrc[0], rsrc[1]};
  // W_uk rows: 128 rows of 64 bytes, four 16-byte chunks each; lane l takes
  // chunk l%4 of rows l/4 + 16j
  u32x4 wv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = (lane >> 2) + 16 * j;
    wv[j] = *(const u32x4*)(a.w_uk + ((size_t)head * kNope + p) * kDV + c0 + 8 * (lane & 3));
  }
  // A fragments: token m0 + l%32 (tokens past the batch zeroed), nope rows
  // 16ks + 8(l/32) .. +7 of its Q_B
  const int b = m0 + (lane & 31);
  const bool b_ok = b < a.batch;
  const int b_c = b_ok ? b : a.batch - 1;
  bf16x8 af[kNope / 16];
#pragma unroll
  for (int ks = 0; ks < kNope / 16; ++ks) {
    const bf16x8 x = *(const bf16x8*)(a.qbm + (size_t)b_c * nrows + (size_t)head * kQB + 16 * ks + 8 * (lane >> 5));
    af[ks] = b_ok ? x : bf16x8{};
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = (lane >> 2) + 16 * j;
    *(LDS_AS u32x4*)((LDS_AS char*)&uk[p][0] + 16 * (lane & 3)) = wv[j];
  }
  __syncthreads();
  // B[k][n] = W_uk[head][16ks + k][c0 + n] by transposing reads: lane l gets
  // column l%32 of rows 8(l/32) + i; within 16-lane group G lane 4j + q reads
  // columns 16(G&1) + 4q .. +3 of row 8(G>>1) + 4tt + j for elements 4tt ..
  const int G = lane >> 4, i16 = lane & 15, jj = i16 >> 2, q = i16 & 3;
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < kNope / 16; ++ks) {
    const int m = 16 * ks + 8 * (G >> 1) + jj;
    const bf16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)&uk[m][16 * (G & 1) + 4 * q]);
    const bf16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)&uk[m + 4][16 * (G & 1) + 4 * q]);
    const bf16x8 bfr = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], bfr, acc, 0, 0, 0);
  }
  // lane l, register r: token tb + 8(r/4) + r%4 with tb = m0 + 4(l/32),
  // column c0 + l%32; byte offsets fit 32 bits (at most 128 tokens here)
  const int tb = m0 + 4 * (lane >> 5);
  const uint32_t tstride = (uint32_t)a.heads * kOut;
  const uint32_t o0 = ((uint32_t)tb * a.heads + head) * kOut + c0 + (lane & 31);
  uint32_t cc[8];
#pragma unroll
  for (int i = 0; i < 16; i += 2) cc[i / 2] = e4m3x2_of_products((float)(__bf16)acc[i], (float)(__bf16)acc[i + 1], qsi);
  if (m0 + kTok <= a.batch) {  // (uniform) every token of the tile exists
#pragma unroll
    for (int i = 0; i < 16; ++i)
      a.out[o0 + (uint32_t)(8 * (i >> 2) + (i & 3)) * tstride] = (uint8_t)(cc[i / 2] >> (8 * (i & 1)));
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ti = 8 * (i >> 2) + (i & 3);
      if (tb + ti < a.batch) a.out[o0 + (uint32_t)ti * tstride] = (uint8_t)(cc[i / 2] >> (8 * (i & 1)));
    }
  }
  // the rope rows of Q_B, encoded as they are: column block y takes rope
  // values 4y .. 4y+3 of the 32 tokens, lane l two of them for token m0 + l/2
  {
    const uint32_t cc = e4m3x2_of_products((float)rv[0], (float)rv[1], qsi);
    if (rt_ok) *(uint16_t*)(a.out + ((size_t)rt * a.heads + head) * kOut + kDV + rr) = (uint16_t)cc;
  }
}
}  // namespace

hipError_t launch_kv_insert(const InsertLaunch& k, hipStream_t stream) {
  InsertArgs a;
  a.qkv = (const __bf16*)k.qkv;
  a.w_kva = (const __bf16*)k.w_kva;
  a.slots = k.slots;
  a.k_scale_inv = k.k_scale_inv;
  a.cache = (uint8_t*)k.cache;
  a.cache_rows = (int64_t)k.num_pages * kCachePage;
  a.tokens = k.tokens;
  a.qkv_stride = k.qkv_stride;
  a.eps = k.eps;
  constexpr int per_wg = kThreads / 64;
  hipLaunchKernelGGL(mla_kv_insert_kernel, dim3((k.tokens + per_wg - 1) / per_wg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Q_B reduction split over workgroups when the 32-token x 32-row tiles
// alone would leave most compute units idle
int query_ksplit(int32_t batch, int32_t heads) {
  const int tiles = ((heads * kQB + 31) / 32) * ((batch + kTok - 1) / kTok);
  return tiles < 256 ? 4 : 1;
}

// Narrow batch: [B][H][128] bf16.  Tiled: [B][1536] bf16 normalised rows,
// then [ksplit][B][H*192] fp32 Q_B partials.
size_t query_workspace_bytes(int32_t batch, int32_t heads) {
  if (batch <= kNarrow) return (size_t)batch * heads * kNope * 2 + 256;
  if (batch <= kMedium) return (size_t)batch * heads * kQB * 2 + 256;
  return (((size_t)batch * kQA * 2 + 255) & ~(size_t)255) +
         (size_t)query_ksplit(batch, heads) * batch * heads * kQB * 4 + 256;
}

hipError_t launch_query(const QueryLaunch& q, hipStream_t stream) {
  QueryArgs a;
  a.qkv = (const __bf16*)q.qkv;
  a.w_qa = (const __bf16*)q.w_qa;
  a.w_qb = (const __bf16*)q.w_qb;
  a.w_uk = (const __bf16*)q.w_uk;
  a.q_scale_inv = q.q_scale_inv;
  a.out = (uint8_t*)q.out;
  a.qn = (__bf16*)q.workspace;
  a.xn = (__bf16*)q.workspace;
  a.qbp = (float*)((char*)q.workspace + (((size_t)q.batch * kQA * 2 + 255) & ~(size_t)255));
  a.qbm = (__bf16*)q.workspace;
  a.batch = q.batch;
  a.heads = q.heads;
  a.qkv_stride = q.qkv_stride;
  a.eps = q.eps;
  if (q.batch <= kNarrow) {
    hipLaunchKernelGGL(mla_qb_gemv_kernel, dim3((q.heads * kQB + kQbRowsPerWg - 1) / kQbRowsPerWg), dim3(kThreads), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_ql_gemv_kernel, dim3(q.heads, kDV / kQlCols), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int mt = (q.batch + kTok - 1) / kTok;
  if (q.batch <= kMedium) {
    hipLaunchKernelGGL(mla_qbn_kernel, dim3((q.heads * kQB + kMRows - 1) / kMRows, (q.batch + kMTok - 1) / kMTok),
                       dim3(kQbnThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_qlm_kernel, dim3(q.heads, kDV / kUkCols, mt), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  const int ksplit = query_ksplit(q.batch, q.heads);
  hipLaunchKernelGGL(mla_norm_kernel, dim3((q.batch + 3) / 4), dim3(kThreads), 0, stream, a);
  const dim3 qb_grid((q.heads * kQB + 31) / 32, mt, ksplit), ql_grid(q.heads, kDV / 128, mt);
  if (ksplit == 4) {
    hipLaunchKernelGGL(mla_qb_kernel<4>, qb_grid, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(mla_ql_kernel<4>, ql_grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(mla_qb_kernel<1>, qb_grid, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(mla_ql_kernel<1>, ql_grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
