// query.hip - MLA query front end for gfx950 (MI355X).
//
// What is computed, per token b (FlashMLA query path, "MlaQuery" forward):
//   rr  = 1 / sqrt(sum_k x[k]^2 / 1536 + eps)      x = qkv[b, 0:1536] (q_a)
//   xn  = bf16((x * rr) * w_qa)                    RMSNorm
//   qb  = bf16(xn . W_qb^T)                        [H, 192]: 128 nope + 64 rope
//   ql  = bf16(qb[:, :128] . W_uk[h])              [H, 512]: absorbed latent q
//   out = e4m3(ql * qsi) | e4m3(qb[:, 128:] * qsi)  qsi = q_scale_inv[0]
// with e4m3 rounded to nearest even and saturated to +-448.
//
// Two kernels, both on v_mfma_f32_32x32x16_bf16 with 32 tokens as M:
//  * mla_qb_kernel: a workgroup owns 32 tokens and 32 rows of W_qb.  It
//    normalises its tokens into LDS (bf16, the A operand), then its four
//    waves each take a quarter of the 1536-long reduction with the W_qb
//    fragments loaded straight from HBM (all 24 of a wave in flight at
//    once); the four partial tiles are summed in LDS in a fixed order.  Nope
//    rows go to the workspace as bf16, rope rows straight to FP8.
//  * mla_ql_kernel: a workgroup owns 32 tokens, one head and 128 output
//    columns; the W_uk tile [128 p][128 c] is staged in LDS and read as the B
//    operand with ds_read_b64_tr_b16 (W_uk is stored c-contiguous, the
//    reduction runs over p), the A operand is the bf16 nope q from the
//    workspace.
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
constexpr int kXnPitch = kQA * 2 + 16;  // LDS row pitch of the normalised tile (bank spread)

struct QueryArgs {
  const __bf16* qkv;
  const __bf16* w_qa;
  const __bf16* w_qb;
  const __bf16* w_uk;
  const float* q_scale_inv;
  uint8_t* out;
  __bf16* qn;  // workspace: [B][H][128] bf16 nope rows of Q_B
  int32_t batch, heads, qkv_stride;
  float eps;
};

// e4m3fn code of x: round to nearest even, saturate to +-448, NaN -> 0x7F.
// Callers pass the exact product of a bf16 value and the fp32 q_scale_inv
// (at most 8 + 24 significant bits, exact in f64), so this is the single
// rounding of the exact value; an fp32 product would first round onto e4m3
// midpoints (v * 0.3f lands next to one whenever v * 3/10 is one) and then
// break the tie the wrong way.  With the exponent e of |x| (normal range e >=
// -6) the mantissa step is 2^(e-3), so rint(|x| * 2^(3-e)) is the rounded
// significand in units of that step (8..16, 16 carrying into the next
// exponent); below 2^-6 the step is the subnormal 2^-9.  Scaling by powers of
// two is exact and rint rounds to nearest even.
__device__ __forceinline__ uint8_t e4m3_code(double x) {
  if (x != x) return 0x7F;
  const uint32_t sign = x < 0.0 || (x == 0.0 && __builtin_signbit(x)) ? 0x80u : 0u;
  const double a = __builtin_fabs(x);
  uint32_t code;
  if (a >= 448.0) {
    code = 0x7E;
  } else if (a < 0.015625) {  // 2^-6: subnormal codes 0..7 (8 is the smallest normal)
    code = (uint32_t)__builtin_rint(a * 512.0);
  } else {
    const int e = (int)((__double_as_longlong(a) >> 52) & 0x7FF) - 1023;  // -6 .. 8
    const uint32_t m = (uint32_t)__builtin_rint(__builtin_ldexp(a, 3 - e));  // 8 .. 16
    code = (uint32_t)(e + 7) * 8 + (m - 8);  // m == 16 carries into the exponent field
    code = code > 0x7E ? 0x7E : code;         // rounding up past 448 saturates
  }
  return (uint8_t)(sign | code);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------- RMSNorm + Q_B

__global__ void __launch_bounds__(kThreads) mla_qb_kernel(QueryArgs a) {
  __shared__ __attribute__((aligned(16))) char xn_mem[kTok * kXnPitch];  // normalised tokens, bf16
  __shared__ __attribute__((aligned(16))) f32x4 red[4 * 4 * 64];          // partial tiles of waves 1..3
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n0 = blockIdx.x * 32;     // first W_qb row (output column) of this workgroup
  const int m0 = blockIdx.y * kTok;   // first token

  // RMSNorm: wave w normalises tokens m0 + 8w .. +7; lane i holds columns
  // 8i + 512k .. +7 (k = 0..2)
  for (int t = 0; t < 8; ++t) {
    const int m = 8 * w + t, b = m0 + m;
    float x[24];
    if (b < a.batch) {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const bf16x8 v = *(const bf16x8*)(a.qkv + (size_t)b * a.qkv_stride + 512 * k + 8 * lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * k + e] = (float)v[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 24; ++e) x[e] = 0.0f;
    }
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 24; ++e) ss += x[e] * x[e];
    ss = wave_sum(ss);
    const float rr = 1.0f / __builtin_sqrtf(ss / (float)kQA + a.eps);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const bf16x8 wv = *(const bf16x8*)(a.w_qa + 512 * k + 8 * lane);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)((x[8 * k + e] * rr) * (float)wv[e]);
      *(LDS_AS bf16x8*)((lds_char*)xn_mem + m * kXnPitch + 2 * (512 * k + 8 * lane)) = o;
    }
  }

  // B fragments of this wave's 24 k-steps (reduction columns 384w ..): lane
  // l holds W_qb row n0 + l%32, columns 16ks + 8*(l/32) .. +7
  constexpr int KSW = kQA / 16 / 4;
  const int nrow = n0 + (lane & 31), h8 = 8 * (lane >> 5);
  const bool row_ok = nrow < a.heads * kQB;
  bf16x8 bf[KSW];
#pragma unroll
  for (int i = 0; i < KSW; ++i) {
    const int k = 16 * (KSW * w + i) + h8;
    bf[i] = row_ok ? *(const bf16x8*)(a.w_qb + (size_t)nrow * kQA + k) : bf16x8{};
  }
  __syncthreads();
  f32x16 acc = {};
#pragma unroll
  for (int i = 0; i < KSW; ++i) {
    const int k = 16 * (KSW * w + i) + h8;
    const bf16x8 af = *(const LDS_AS bf16x8*)((const lds_char*)xn_mem + (lane & 31) * kXnPitch + 2 * k);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[i], acc, 0, 0, 0);
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
  // lane l, register r: token 8*(r/4) + 4*(l/32) + r%4, W_qb row nrow
  const int head = nrow / kQB, r = nrow % kQB;
  const float qsi = a.q_scale_inv[0];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (b >= a.batch) continue;
    const __bf16 v = (__bf16)acc[i];
    if (r < kNope) a.qn[((size_t)b * a.heads + head) * kNope + r] = v;
    else a.out[((size_t)b * a.heads + head) * kOut + kDV + (r - kNope)] = e4m3_code((double)(float)v * (double)qsi);
  }
}

// ---------------------------------------------------------------- W_UK absorption + FP8

// LDS tile of W_uk[h][p][c0 .. c0+127]: 128-byte rows (64 columns) in two
// column groups of 128 rows, 16-byte chunks XOR-swizzled by bits 1..3 of the
// row (the layout the decode kernel uses for its V^T reads).
constexpr int kUkGroup = 128 * 128;  // bytes per column group
__device__ __forceinline__ int uk_swz(int m) { return (((m >> 1) & 1) << 2) | (((m >> 3) & 1) << 1) | ((m >> 2) & 1); }

__global__ void __launch_bounds__(kThreads) mla_ql_kernel(QueryArgs a) {
  __shared__ __attribute__((aligned(16))) char uk_mem[2 * kUkGroup];
  lds_char* const uk = (lds_char*)uk_mem;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int head = blockIdx.x, c0 = blockIdx.y * 128, m0 = blockIdx.z * kTok;

  // stage W_uk[head][0..127][c0..c0+127]: 2048 chunks of 16 bytes
  for (int i = tid; i < 128 * 16; i += kThreads) {
    const int p = i >> 4, ch = i & 15;  // row p, chunk ch (8 columns)
    const u32x4 v = *(const u32x4*)(a.w_uk + ((size_t)head * kNope + p) * kDV + c0 + 8 * ch);
    const int g = ch >> 3, x = ch & 7;
    *(LDS_AS u32x4*)(uk + g * kUkGroup + p * 128 + 16 * (x ^ uk_swz(p))) = v;
  }
  // A fragments: token m0 + l%32, nope columns 16ks + 8*(l/32) .. +7
  const int b = m0 + (lane & 31);
  const bool b_ok = b < a.batch;
  bf16x8 af[kNope / 16];
#pragma unroll
  for (int ks = 0; ks < kNope / 16; ++ks)
    af[ks] = b_ok ? *(const bf16x8*)(a.qn + ((size_t)b * a.heads + head) * kNope + 16 * ks + 8 * (lane >> 5))
                  : bf16x8{};
  __syncthreads();
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
  for (int i = 0; i < 16; ++i) {
    const int bb = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (bb >= a.batch) continue;
    const float v = (float)(__bf16)acc[i];
    a.out[((size_t)bb * a.heads + head) * kOut + c] = e4m3_code((double)v * (double)qsi);
  }
}

}  // namespace

size_t query_workspace_bytes(int32_t batch, int32_t heads) { return (size_t)batch * heads * kNope * 2 + 256; }

hipError_t launch_query(const QueryLaunch& q, hipStream_t stream) {
  QueryArgs a;
  a.qkv = (const __bf16*)q.qkv;
  a.w_qa = (const __bf16*)q.w_qa;
  a.w_qb = (const __bf16*)q.w_qb;
  a.w_uk = (const __bf16*)q.w_uk;
  a.q_scale_inv = q.q_scale_inv;
  a.out = (uint8_t*)q.out;
  a.qn = (__bf16*)q.workspace;
  a.batch = q.batch;
  a.heads = q.heads;
  a.qkv_stride = q.qkv_stride;
  a.eps = q.eps;
  const int mt = (q.batch + kTok - 1) / kTok;
  hipLaunchKernelGGL(mla_qb_kernel, dim3((q.heads * kQB + 31) / 32, mt), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_ql_kernel, dim3(q.heads, kDV / 128, mt), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
