// decode.hip - split-KV absorbed MLA decode for gfx950 (MI355X).
//
// What is computed (one query token per sequence): for every head h of
// sequence b, scores against the shared 576-wide latent rows (512 nope + 64
// rope; the rope block is one more slice of the same QK^T), a scaled softmax
// per head row, and O = P.V with V the 512 nope columns.  Output O in bf16 and
// the natural-log LSE per head.
//
// Design (MI355X-first; the pages' Hopper/Blackwell kernels are prior art):
//  * Head-packed tile (the STAGE_D2 note, "Strategy A: Head-Packed M
//    Dimension"): a workgroup reads each KV row once for a slab of up to 64
//    heads of its sequence.  The MFMA is v_mfma_f32_32x32x16_bf16 with the 32
//    KV tokens of an LDS slot as M and 32 heads as N:
//        S^T[t][h] = sum_d K[t][d] Q[h][d]          (36 steps of 16)
//        O^T[c][h] += sum_t V^T[c][t] P^T[t][h]     (2 steps per 32 columns)
//    With tokens on M the S^T accumulator is the P^T operand of the PV
//    product as it stands (the k <-> token permutation is absorbed by the V^T
//    read), and every O^T register of a lane belongs to one head.
//  * Split reduction (the CDNA counterpart of the FlashMLA "dual gemm" idea of
//    halving the QK^T reduction across warpgroups): the NSPLIT waves of a
//    32-head group each own 576/NSPLIT of the QK^T reduction and 512/NSPLIT
//    output columns.  Partial S^T go through LDS; every wave of the group
//    adds them in one fixed order (for two parts, own + partner, which is the
//    same sum in either wave), so all of them hold bit-identical scores and
//    softmax state.  A wave keeps 144/NSPLIT query VGPRs and 256/NSPLIT
//    accumulator AGPRs.
//  * Token-split softmax (bf16 rows copied by the DMA, or per-tensor FP8
//    rows through the register fill; two parts): after a
//    segment's first slot, each wave of a pair forms the scores and the
//    softmax of its own 16 tokens only (half of the partner's partial read,
//    8 exponentials per lane instead of 16), and the pair swaps bf16 P^T
//    halves through LDS for the PV.  Both keep the reference the first slot
//    fixed; each sums p over its own tokens, and the two sums are added
//    once at the end.
//  * Slabs: H = 128 runs as two 64-head workgroups per KV range, on one XCD,
//    so the second reader of every KV line finds it in that XCD's L2.
//  * KV streaming: 32-token slots of 36 KB in a 4-deep LDS ring filled by
//    direct global->LDS DMA (global_load_lds_dwordx4), laid out in 128-byte
//    column groups and XOR-swizzled so that the ds_read_b128 K reads and the
//    ds_read_b64_tr_b16 V^T reads are free of bank conflicts.  The DMA is
//    issued from inline assembly and accounted for by explicit vmcnt waits,
//    so the compiler never serialises LDS reads behind copies in flight.
//  * Software pipeline: while slot s is exchanged, softmaxed and multiplied
//    into O, the partial QK^T of slot s+1 runs on the matrix core; two more
//    slots are in flight from HBM.  Two workgroup barriers per slot: one
//    publishes the partial scores (and the landed slot), one frees the ring
//    slot and the exchange buffer (token-split: one publishes the P^T
//    halves, and the next slot's first barrier frees the ring slot).
//  * Split-KV: pages of all sequences are laid end to end and cut into equal
//    ranges, one per workgroup and slab (a static form of the persistent
//    scheduler the STAGE_D2 note describes under "Grid vs. Persistent Tile
//    Scheduler").  A sequence inside one range is finished in place;
//    otherwise each piece writes its normalised partial O and its base-2
//    LSE (both fp32), and a second kernel (mla_merge_kernel, or
//    mla_merge_wide_kernel where sequences have many pieces) combines the
//    pieces.  The merge is not done by the last piece to arrive: that
//    would need a device-scope release fence per piece, which on gfx950
//    writes back the whole XCD L2.
//  * Cache formats: bf16 rows are copied by the DMA; FP8 rows (512 codes
//    with per-128-column scales and bf16 rope, or 576 codes with one
//    per-tensor scale) and gathered top-k rows pass through registers, where
//    the e4m3 codes become bf16 exactly.  Tile scales multiply the partial
//    scores in fp32; the per-tensor 1/k_scale_inv folds into the score scale
//    and the output normalisation.
//  * Several query tokens per sequence (CAUSAL): the T*H query rows of a
//    sequence are packed like heads (row t*H + h), so one read of each KV row
//    serves all of them; row t sees positions below seqlen - T + 1 + t.  The
//    rows' limits differ only in the last T - 1 positions, so the masked
//    softmax runs only from the first slot that hides a position from some
//    row.  Top-k lists are per query token: each token is its own sequence
//    of H rows, and the fill pipeline cuts its list at the token's limit.
//  * Softmax in base 2 against a fixed reference per head: the first slot's
//    max.  Later slots may exceed it by up to 16 (P <= 2^16, exact in fp32 and
//    as relative bf16); if any head's scores rise further, the workgroup
//    redoes the segment once with the true maxima (then P <= 1).  Realistic
//    score distributions never trigger the redo.  With no rescale inside the
//    KV loop the fp32 accumulators are only written by MFMAs and stay in
//    fixed AGPRs.
#include "decode_common.h"

namespace mla {
namespace {

constexpr int kFillRing = 3;                 // positions of the register-fill ring
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKSteps = kD / 16;                         // 36 MFMA k-steps for QK^T
constexpr int kCB = kDV / 32;                            // 16 O^T column blocks



struct LaneTables {
  uint32_t dma;       // source byte offset of this lane's chunk in a full slot (rows 8w + lane/8)
  uint32_t kaddr[4];  // QK^T A operand of this wave's k-step i: kaddr[i & 3] + 4096 * (i >> 2)
  uint32_t kaddr_r[2];  // tiled split: the rope k-steps
  uint32_t vaddr[2];  // PV A operand (tr reads) of this wave's first column block, rows 8tt + 4h + j: [tt]
  uint32_t vswap;     // token-split softmax, part 1: 2048 (its PV k-step 0 is the slot's rows 16..31), else 0
};

// How the QK^T reduction is cut between the NSPLIT waves of a head group.
// Contiguous (bf16 cache): wave part p takes global k-steps p*KS .. +KS-1.
// Tiled (FP8 cache): part p takes whole 128-column code tiles, TPP of them
// (k-steps CS*p .. +CS-1), then RS rope k-steps 32 + RS*p ..; every code tile
// sums into an fp32 accumulator of its own, so that the per-token tile scale
// can be applied exactly.  Either way part p owns output columns 512p/NSPLIT
// .. +512/NSPLIT-1, which in the tiled case are the same tiles.
template <int NSPLIT>
struct Tiling {
  static constexpr int KS = kKSteps / NSPLIT;
  static constexpr int TPP = 4 / NSPLIT;  // code tiles per part
  static constexpr int CS = 8 * TPP;      // code k-steps per part
  static constexpr int RS = 4 / NSPLIT;   // rope k-steps per part
  static_assert(CS + RS == KS, "tiled split covers the 36 k-steps");
};

// global k-step of this part's local step i
template <int NSPLIT, bool TILED>
__device__ __forceinline__ int global_step(int part, int i) {
  using T = Tiling<NSPLIT>;
  if constexpr (TILED) return i < T::CS ? T::CS * part + i : 32 + T::RS * part + (i - T::CS);
  else return T::KS * part + i;
}

// LDS address of the K fragment of global k-step g for this lane: logical
// chunk 2g + h of row m (dims 16g + 8h .. +7), column group g / 4
__device__ __forceinline__ uint32_t k_frag_addr(int g, int lane, int perm = 0) {
  const int m = (lane & 31) ^ perm, h = lane >> 5;
  return kGroupBytes * (g >> 2) + m * 128 + 16 * ((2 * (g & 3) + h) ^ row_swz(m));
}

// Wave part `part` of a head group covers the k-steps above and column
// blocks part*NCB .. +NCB-1.
// perm = 16 (token-split softmax, part 1): the QK^T A operand takes the
// slot's rows in the order 16..31, 0..15, so that this wave's own token half
// lands in S^T registers 0..7 as it does for part 0.
template <int NSPLIT, bool TILED>
__device__ __forceinline__ void make_tables(LaneTables& t, int lane, int w, int part, int perm = 0) {
  using T = Tiling<NSPLIT>;
  constexpr int NCB = kCB / NSPLIT;
  t.dma = dma_lane_off(lane, w, kTS);
  t.vswap = perm ? 2048u : 0u;
  // steps g0 + 4q + j (code steps, contiguous) differ from step g0 + j by q
  // column groups
  for (int j = 0; j < 4; ++j) t.kaddr[j] = k_frag_addr(global_step<NSPLIT, TILED>(part, j), lane, perm);
  for (int k = 0; k < 2; ++k) t.kaddr_r[k] = TILED && k < T::RS ? k_frag_addr(global_step<NSPLIT, TILED>(part, T::CS + k), lane) : 0;
  {
    // ds_read_b64_tr_b16 for column block cb, k-step 0: within 16-lane group
    // G lane 4j + q supplies columns 32cb + 16*(G&1) + 4q .. +3 of token row
    // 8tt + 4*(G>>1) + j.  Odd column blocks flip chunk bit 2 (address ^ 64),
    // k-step 1 adds 16 rows (2048 bytes), block pair cb/2 is column group
    // cb/2.  part * NCB is even, so local and global block parity agree.
    const int G = lane >> 4, i = lane & 15, j = i >> 2, q = i & 3, h = G >> 1, cpart = G & 1;
    for (int tt = 0; tt < 2; ++tt) {
      const int m = 8 * tt + 4 * h + j;
      t.vaddr[tt] = kGroupBytes * (part * NCB / 2) + m * 128 + 16 * ((2 * cpart + (q >> 1)) ^ row_swz(m)) +
                    8 * (q & 1);
    }
  }
}


// ---------------------------------------------------------------- register fill (FP8 cache, top-k)


// The register fill: every slot row is loaded by the eight lanes of one
// wave that share lane % 8 (wave w: rows 8w .. 8w+7), lane / 8 = q picking
// 128-byte pieces, so each load instruction reads 128 contiguous bytes per
// row.  The lanes then write the row as bf16 into the same swizzled ring
// layout the DMA produces, dequantising FP8 codes on the way as
// bf16_rne(e4m3(code) * scale) with an exact fp32 product.
template <int KVM>
struct RawRow;

template <>
struct RawRow<kKvFp8> {
  u32x4 code[4];  // codes 128k + 16q .. +15 of the row, k = 0..3 (column tile k)
  u32x4 rope;     // rope bytes 16q .. +15
  f32x4 scale;    // the row's four tile scales
};
template <>
struct RawRow<kKvFp8TopK> : RawRow<kKvFp8> {};
template <>
struct RawRow<kKvFp8T> {
  u32x4 code[4];  // codes 128k + 16q .. +15 of the row, k = 0..3
  uint2 rope;     // rope codes 8q .. +7
};
template <>
struct RawRow<kKvFp8TTopK> : RawRow<kKvFp8T> {};
template <>
struct RawRow<kKvBf16TopK> {
  u32x4 v[9];  // bytes 128k + 16q .. +15 of the row, k = 0..8 (column group k)
};

template <int KVM>
__device__ __forceinline__ void load_row(RawRow<KVM>& rr, const DecodeArgs& a, int row, int q) {
  if constexpr (kv_fp8(KVM)) {
    const char* base = a.kv + (size_t)row * kFp8RowBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k) rr.code[k] = *(const u32x4*)(base + 128 * k + 16 * q);
    rr.rope = *(const u32x4*)(base + 512 + 16 * q);
    rr.scale = *(const f32x4*)(a.kv_scales + (size_t)row * 4);
  } else if constexpr (kv_tensor(KVM)) {
    const char* base = a.kv + (size_t)row * kFp8TRowBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k) rr.code[k] = *(const u32x4*)(base + 128 * k + 16 * q);
    rr.rope = *(const uint2*)(base + 512 + 8 * q);
  } else {
#pragma unroll
    for (int k = 0; k < 9; ++k) rr.v[k] = *(const u32x4*)(a.kv + (size_t)row * kRowBytes + 128 * k + 16 * q);
  }
}

// 8 e4m3 codes (two words) as 8 bf16: every e4m3 value is exact in bf16
// (the scaled conversion with scale 1 changes nothing)
__device__ __forceinline__ u32x4 codes8(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// Write row r (this lane's q share) into the slot at `buf`; an FP8 row puts
// its codes (unscaled) in columns 0..511 and its four tile scales into the
// slot's scale table `stab` [tile][token].
template <int KVM>
__device__ __forceinline__ void fill_row(lds_char* buf, LDS_AS float* stab, const RawRow<KVM>& rr, int r, int q) {
  const int sw = row_swz(r);
  lds_char* rowp = buf + r * 128;
  if constexpr (kv_fp8(KVM)) {
    // codes 128k + 16q .. +15: column group 2k + q/4, chunks 2(q%4), 2(q%4)+1
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c0 = 2 * (q & 3);
      lds_char* gp = rowp + kGroupBytes * (2 * k + (q >> 2));
      *(LDS_AS u32x4*)(gp + 16 * (c0 ^ sw)) = codes8(rr.code[k][0], rr.code[k][1]);
      *(LDS_AS u32x4*)(gp + 16 * ((c0 + 1) ^ sw)) = codes8(rr.code[k][2], rr.code[k][3]);
    }
    // rope (bf16 as stored): column group 8, chunk q
    *(LDS_AS u32x4*)(rowp + kGroupBytes * 8 + 16 * (q ^ sw)) = rr.rope;
    if (q < 4) stab[q * kTS + r] = rr.scale[q];
  } else if constexpr (kv_tensor(KVM)) {
    // codes as above; the rope codes 8q .. +7 go to chunk q of column group 8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c0 = 2 * (q & 3);
      lds_char* gp = rowp + kGroupBytes * (2 * k + (q >> 2));
      *(LDS_AS u32x4*)(gp + 16 * (c0 ^ sw)) = codes8(rr.code[k][0], rr.code[k][1]);
      *(LDS_AS u32x4*)(gp + 16 * ((c0 + 1) ^ sw)) = codes8(rr.code[k][2], rr.code[k][3]);
    }
    *(LDS_AS u32x4*)(rowp + kGroupBytes * 8 + 16 * (q ^ sw)) = codes8(rr.rope.x, rr.rope.y);
  } else {
#pragma unroll
    for (int k = 0; k < 9; ++k) *(LDS_AS u32x4*)(rowp + kGroupBytes * k + 16 * (q ^ sw)) = rr.v[k];
  }
}

// ---------------------------------------------------------------- compute on one slot

template <int NSPLIT>
struct Acc {
  f32x16 o[kCB / NSPLIT];  // O^T accumulators (AGPRs), relative to the reference max
};

// Softmax state of one lane's head.  The reference max is fixed after the
// segment's first slot (or, in a redo, to the true max); the accumulators
// are only ever zeroed or fed by MFMAs inside the KV loop, which keeps them
// in fixed AGPRs.
struct SoftmaxState {
  float m_ref;   // base-2 reference: p = 2^(x - m_ref)
  float m_seen;  // largest score seen (base 2)
  float l_sum;   // this lane's share of sum p
};

// This wave's partial S^T of one slot: 32 tokens x 32 heads over its KS
// k-steps, fp32.
// K fragments are read kRA - 1 steps ahead of the MFMA that consumes them.
// A read must not land in the registers of an operand that an issued MFMA
// is still reading: the wave would then wait for that MFMA to finish, and
// everything it issues between MFMAs would serialise with the matrix core.
// The register allocator does not know this, so every operand is kept
// visibly alive (keep_alive) until the reads that follow its MFMA have been
// issued; MFMA I - 1 has completed once MFMA I (which accumulates onto its
// result) issues, so the reads may reuse its registers.  The scheduling
// fences keep LDS reads and MFMAs in this order and let only VALU work move
// between them.
constexpr int kRA = 5;

// An empty use that keeps a register operand live to this point; the memory
// clobber keeps LDS reads from moving across it.
template <typename T>
__device__ __forceinline__ void keep_alive(const T& v) {
  asm volatile("" ::"v"(v) : "memory");
}
// What rides between the QK^T MFMAs of a step: the next slot's copies, the
// previous slot's softmax, and (top-k) that softmax's validity mask.
constexpr int kPipeDma = 1, kPipeSoft = 2, kPipeMask = 4;
constexpr int kPipeHalf = 8;   // token-split softmax: this wave's 16 tokens (S^T registers 0..7) only
constexpr int kPipeOwnL = 16;  // full softmax, but only registers 0..7 (this wave's tokens) enter l_sum
constexpr int kPipePv2 = 32;   // the PV that follows reads two V^T blocks ahead (pv_slot2)

// Publish this wave's partial: [wave][r4][lane] 16-byte rows, lane-contiguous.
__device__ __forceinline__ void put_partial(LDS_AS f32x4* xch, const f32x16& s, int w, int lane) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 v = {s[4 * r4], s[4 * r4 + 1], s[4 * r4 + 2], s[4 * r4 + 3]};
    xch[(w * 4 + r4) * 64 + lane] = v;
  }
}

// Token-split softmax (two parts): the partner needs only S^T registers
// 8..15 of this wave's partial (its own token half); r4 slot 0 of this
// wave's region then carries this wave's bf16 P^T half.
__device__ __forceinline__ void put_partial_half(LDS_AS f32x4* xch, const f32x16& s, int w, int lane) {
#pragma unroll
  for (int r4 = 2; r4 < 4; ++r4) xch[(w * 4 + r4) * 64 + lane] = f32x4{s[4 * r4], s[4 * r4 + 1], s[4 * r4 + 2], s[4 * r4 + 3]};
}

// Full S^T of the head group.  Two parts: own + partner (fp32 addition is
// commutative, so both waves get the same bits).  Four parts: (p0 + p1) +
// (p2 + p3), every term read back from LDS.
template <int NSPLIT>
__device__ __forceinline__ f32x16 total_scores(const LDS_AS f32x4* xch, const f32x16& own, int w, int lane,
                                               int cross = 0) {
  f32x16 tot;
  if constexpr (NSPLIT == 2) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      // (cross = 2, token-split softmax: the partner holds this wave's
      // registers 0..7 in its 8..15 and the reverse)
      const f32x4 v = xch[((w ^ 1) * 4 + (r4 ^ cross)) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[4 * r4 + e] = own[4 * r4 + e] + v[e];
    }
  } else {
    const int g0 = w & ~3;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 p0 = xch[((g0 + 0) * 4 + r4) * 64 + lane];
      const f32x4 p1 = xch[((g0 + 1) * 4 + r4) * 64 + lane];
      const f32x4 p2 = xch[((g0 + 2) * 4 + r4) * 64 + lane];
      const f32x4 p3 = xch[((g0 + 3) * 4 + r4) * 64 + lane];
      const f32x4 v = (p0 + p1) + (p2 + p3);
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[4 * r4 + e] = v[e];
    }
  }
  return tot;
}


// Softmax of a full slot, cut into micro-stages that ride between the QK^T
// MFMAs of the next slot: the score sums, a tree max, the max across the two
// token halves, the reference, eight pairs of exponentials (each also adding
// the previous pair into two running sums) and the row sums.  The partners'
// partial scores are read from LDS right after the barrier that publishes
// them, together with the first K fragments, and are first used three
// k-steps later, so the read latency hides behind MFMAs.  No stage holds a
// dependency chain longer than one MFMA.
struct SoftPipe {
  uint32_t mask;    // valid tokens of the slot (top-k), bit t = token t
  f32x16 own;       // this wave's partial S^T of the slot
  f32x4 xr[16];     // the partners' partials: [part * 4 + r4] (two parts: the partner's, [r4])
  f32x16 x;         // full S^T
  float t[5];       // partial maxima
  float mx, nref;
  f32x8 p0, p1;
  float la, lb;     // running sums of p0, p1
};

struct SoftCtx {
  const LDS_AS f32x4* xch;
  int w, lane;
  float scale_log2;
  int cross = 0;  // token-split softmax: partner register group of r4 is r4 ^ 2
};

// Scores of tokens whose bit in `mask` is clear become -inf.  Lane l,
// register r holds token 8*(r/4) + 4*(l/32) + r%4.
template <int R0 = 0, int R1 = 16>
__device__ __forceinline__ void apply_mask(f32x16& x, uint32_t mask, int lane) {
  const uint32_t mh = mask >> (4 * (lane >> 5));
#pragma unroll
  for (int r = R0; r < R1; ++r)
    x[r] = (mh >> (8 * (r >> 2) + (r & 3))) & 1u ? x[r] : -INFINITY;
}


// The partials this wave adds: two parts, the partner's; four parts, all
// four (the own one too, so that every wave forms the same sum).
template <int NSPLIT>
__device__ __forceinline__ void soft_read(SoftPipe& sp, const SoftCtx& c) {
  if constexpr (NSPLIT == 2) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) sp.xr[r4] = c.xch[((c.w ^ 1) * 4 + (r4 ^ c.cross)) * 64 + c.lane];
  } else {
    const int g0 = c.w & ~3;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) sp.xr[4 * q + r4] = c.xch[((g0 + q) * 4 + r4) * 64 + c.lane];
  }
}

// Token-split softmax, steady state: only the partner's registers 8..15
// (this wave's token half)
__device__ __forceinline__ void soft_read_half(SoftPipe& sp, const SoftCtx& c) {
  sp.xr[0] = c.xch[((c.w ^ 1) * 4 + 2) * 64 + c.lane];
  sp.xr[1] = c.xch[((c.w ^ 1) * 4 + 3) * 64 + c.lane];
}

enum : int {
  kStSum0,  // x[0..7]
  kStSum1,  // x[8..15]
  kStMaxA,
  kStMaxB,
  kStHalves,
  kStRef,
  kStExp0,  // .. kStExp0 + 7
  kStLsum = kStExp0 + 8,
  kSoftStages
};
// The token-split softmax stages: 8 scores per lane (x[0..7] = own
// registers 0..7 + the partner's 8..15), 8 exponentials into p0.
template <int ST, bool MASKED>
__device__ __forceinline__ void soft_stage_half(SoftPipe& sp, SoftmaxState& st, const SoftCtx& c) {
  if constexpr (ST == kStSum0) {
#pragma unroll
    for (int r4 = 0; r4 < 2; ++r4) {
      const f32x4 v = f32x4{sp.own[4 * r4], sp.own[4 * r4 + 1], sp.own[4 * r4 + 2], sp.own[4 * r4 + 3]} + sp.xr[r4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sp.x[4 * r4 + e] = v[e];
    }
    // (the mask as this wave's registers see the tokens)
    if constexpr (MASKED) apply_mask<0, 8>(sp.x, sp.mask, c.lane);
  } else if constexpr (ST == kStMaxA) {
    sp.t[0] = fmaxf(fmaxf(sp.x[0], sp.x[1]), sp.x[2]);
    sp.t[1] = fmaxf(fmaxf(sp.x[3], sp.x[4]), sp.x[5]);
    sp.t[2] = fmaxf(sp.x[6], sp.x[7]);
  } else if constexpr (ST == kStMaxB) {
    sp.mx = fmaxf(fmaxf(sp.t[0], sp.t[1]), sp.t[2]);
  } else if constexpr (ST == kStHalves) {
    sp.mx = max_halves(sp.mx) * c.scale_log2;
  } else if constexpr (ST == kStRef) {
    st.m_ref = st.m_ref == -INFINITY ? sp.mx : st.m_ref;
    st.m_seen = fmaxf(st.m_seen, sp.mx);
    sp.nref = neg_ref(st.m_ref);
  } else if constexpr (ST >= kStExp0 && ST < kStExp0 + 8) {
    constexpr int k = ST - kStExp0;
    sp.p0[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sp.x[k], c.scale_log2, sp.nref));
    if constexpr (k == 1) sp.la = sp.p0[0];
    else if constexpr (k > 1) sp.la += sp.p0[k - 1];
  } else if constexpr (ST == kStLsum) {
    st.l_sum += sp.la + sp.p0[7];
  }
}

template <int NSPLIT, int ST, bool MASKED, bool OWNL = false>
__device__ __forceinline__ void soft_stage(SoftPipe& sp, SoftmaxState& st, const SoftCtx& c) {
  if constexpr (ST == kStSum0 || ST == kStSum1) {
    constexpr int r0 = ST == kStSum0 ? 0 : 2;  // first row group of four
#pragma unroll
    for (int r4 = r0; r4 < r0 + 2; ++r4) {
      f32x4 v;
      if constexpr (NSPLIT == 2) {
        v = f32x4{sp.own[4 * r4], sp.own[4 * r4 + 1], sp.own[4 * r4 + 2], sp.own[4 * r4 + 3]} + sp.xr[r4];
      } else {
        v = (sp.xr[r4] + sp.xr[4 + r4]) + (sp.xr[8 + r4] + sp.xr[12 + r4]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sp.x[4 * r4 + e] = v[e];
    }
    if constexpr (MASKED) apply_mask<4 * r0, 4 * r0 + 8>(sp.x, sp.mask, c.lane);
  } else if constexpr (ST == kStMaxA) {
#pragma unroll
    for (int k = 0; k < 5; ++k) sp.t[k] = fmaxf(fmaxf(sp.x[3 * k], sp.x[3 * k + 1]), sp.x[3 * k + 2]);
  } else if constexpr (ST == kStMaxB) {
    sp.mx = fmaxf(fmaxf(fmaxf(sp.t[0], sp.t[1]), sp.t[2]), fmaxf(fmaxf(sp.t[3], sp.t[4]), sp.x[15]));
  } else if constexpr (ST == kStHalves) {
    sp.mx = max_halves(sp.mx) * c.scale_log2;  // scale_log2 > 0: the max commutes with the scaling
  } else if constexpr (ST == kStRef) {
    st.m_ref = st.m_ref == -INFINITY ? sp.mx : st.m_ref;
    st.m_seen = fmaxf(st.m_seen, sp.mx);
    sp.nref = neg_ref(st.m_ref);
  } else if constexpr (ST >= kStExp0 && ST < kStExp0 + 8) {
    constexpr int k = ST - kStExp0;
    sp.p0[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sp.x[k], c.scale_log2, sp.nref));
    sp.p1[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sp.x[k + 8], c.scale_log2, sp.nref));
    if constexpr (k == 1) {
      sp.la = sp.p0[0];
      sp.lb = sp.p1[0];
    } else if constexpr (k > 1) {
      sp.la += sp.p0[k - 1];
      sp.lb += sp.p1[k - 1];
    }
  } else if constexpr (ST == kStLsum) {
    if constexpr (OWNL) st.l_sum += sp.la + sp.p0[7];
    else st.l_sum += (sp.la + sp.p0[7]) + (sp.lb + sp.p1[7]);
  }
}

// Micro-stages [stage_lo, stage_hi) run at k-step I of KS: with 18 steps one
// per step from step 3 on (the partners' partials, read right after the
// barrier, are first used three MFMAs later); with 9 steps, two per step from
// step 1 on (the sums of four parts one per step).
constexpr int stage_lo(int KS, int I) {
  if (KS >= 18) return I < 3 ? 0 : (I - 3 < kSoftStages ? I - 3 : kSoftStages);
  constexpr int lo9[9] = {0, 0, 1, 2, 4, 6, 8, 10, 12};
  return lo9[I];
}
constexpr int stage_hi(int KS, int I) {
  if (KS >= 18) return I < 3 ? 0 : (I - 2 < kSoftStages ? I - 2 : kSoftStages);
  constexpr int hi9[9] = {0, 1, 2, 4, 6, 8, 10, 12, kSoftStages};
  return hi9[I];
}
static_assert(stage_hi(18, 17) == kSoftStages && stage_hi(9, 8) == kSoftStages, "every stage is scheduled");

template <int NSPLIT, int ST0, int ST1, bool MASKED, int PIPE = 0>
__device__ __forceinline__ void soft_stages(SoftPipe& sp, SoftmaxState& st, const SoftCtx& c) {
  if constexpr (ST0 < ST1 && ST0 < kSoftStages) {
    if constexpr ((PIPE & kPipeHalf) != 0) soft_stage_half<ST0, MASKED>(sp, st, c);
    else soft_stage<NSPLIT, ST0, MASKED, (PIPE & kPipeOwnL) != 0>(sp, st, c);
    soft_stages<NSPLIT, ST0 + 1, ST1, MASKED, PIPE>(sp, st, c);
  }
}

template <int NSPLIT, bool TILED, int I>
__device__ __forceinline__ uint32_t k_addr(const LaneTables& t) {
  if constexpr (TILED && I >= Tiling<NSPLIT>::CS) return t.kaddr_r[I - Tiling<NSPLIT>::CS];
  else return t.kaddr[I & 3] + kGroupBytes * (I >> 2);
}

// accumulators of the partial QK^T: one, or (tiled) one per code tile + rope;
// arrays are sized for the largest case, unused entries cost nothing
constexpr int kMaxAcc = 3;

// V^T operands of one PV column block: two k-steps, each two tr reads
typedef bf16x4 VBlock[4];

// ds_read_b64_tr_b16 of column block cb of this wave's PV
__device__ __forceinline__ void pv_load(const lds_char* buf, const LaneTables& t, int cb, VBlock& v) {
  const uint32_t x = (cb & 1) ? 64u : 0u;
  const lds_char* p0 = buf + (t.vaddr[0] ^ x) + kGroupBytes * (cb >> 1);
  const lds_char* p1 = buf + (t.vaddr[1] ^ x) + kGroupBytes * (cb >> 1);
  // (k-step 0 reads rows 0..15 of the slot, or 16..31 when vswap = 2048)
  v[0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p0 + t.vswap));
  v[1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p1 + t.vswap));
  v[2] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p0 + (16 * 128 - t.vswap)));
  v[3] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p1 + (16 * 128 - t.vswap)));
}

// The first kRA - 1 K fragments of a slot, issued before the rest of the
// step's work so that their latency overlaps it.
template <int NSPLIT, bool TILED>
__device__ __forceinline__ void qk_preload(bf16x8 (&kb)[kRA], const lds_char* buf, const LaneTables& t) {
  static_assert(kRA == 5, "preload covers kRA - 1 fragments");
  kb[0] = *(const LDS_AS bf16x8*)(buf + k_addr<NSPLIT, TILED, 0>(t));
  kb[1] = *(const LDS_AS bf16x8*)(buf + k_addr<NSPLIT, TILED, 1>(t));
  kb[2] = *(const LDS_AS bf16x8*)(buf + k_addr<NSPLIT, TILED, 2>(t));
  kb[3] = *(const LDS_AS bf16x8*)(buf + k_addr<NSPLIT, TILED, 3>(t));
}

// What else runs during a partial QK^T: the previous slot's softmax, the
// first V^T block of its PV, and (copy ring) the copies of a later slot.
struct QkSide {
  DmaJob job;
  const lds_char* pvbuf;  // slot whose PV follows
  VBlock* va0;            // where its first V^T block goes
  VBlock* va1;            // (kPipePv2) where its second V^T block goes
};

template <int NSPLIT, int I, int PIPE, bool TILED>
__device__ __forceinline__ void qk_steps(f32x16 (&acc)[kMaxAcc], bf16x8 (&kb)[kRA], const lds_char* buf,
                                         const bf16x8 (&qf)[kKSteps / NSPLIT], const LaneTables& t,
                                         const QkSide& side, SoftPipe& sp, SoftmaxState& st, const SoftCtx& c) {
  using T = Tiling<NSPLIT>;
  constexpr int KS = T::KS;
  if constexpr (I < KS) {
    constexpr int ai = TILED ? (I < T::CS ? I / 8 : T::TPP) : 0;
    constexpr bool first = TILED ? (I < T::CS ? I % 8 == 0 : I == T::CS) : I == 0;
    __builtin_amdgcn_sched_barrier(0);
    acc[ai] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[I % kRA], qf[I], first ? f32x16{} : acc[ai], 0, 0, 0);
    if constexpr (I + kRA - 1 < KS)
      kb[(I + kRA - 1) % kRA] = *(const LDS_AS bf16x8*)(buf + k_addr<NSPLIT, TILED, I + kRA - 1>(t));
    keep_alive(kb[I % kRA]);
    if constexpr ((PIPE & kPipeDma) != 0) {
      // the next slot's copies ride between the MFMAs, so that the wave
      // never stalls on a full memory queue with nothing else to issue
      constexpr int R = KS / kDmaPerWave;
      if constexpr (I % R == R - 1) dma_issue<I / R>(side.job);
    }
    if constexpr ((PIPE & kPipeSoft) != 0) {
      soft_stages<NSPLIT, stage_lo(KS, I), stage_hi(KS, I), (PIPE & kPipeMask) != 0, PIPE>(sp, st, c);
      // the PV that follows starts on data already in registers
      if constexpr (I == KS - 3) pv_load(side.pvbuf, t, 0, *side.va0);
      if constexpr ((PIPE & kPipePv2) != 0 && I == KS - 2) pv_load(side.pvbuf, t, 1, *side.va1);
    }
    qk_steps<NSPLIT, I + 1, PIPE, TILED>(acc, kb, buf, qf, t, side, sp, st, c);
  }
}

// Per-token scales of code tile `tile` for the 16 tokens this lane holds in
// an S^T or P^T fragment (register r: token 8*(r/4) + 4*(l/32) + r%4), from a
// slot's scale table [tile][token] in LDS.
__device__ __forceinline__ f32x16 tile_scales(const LDS_AS float* tab, int tile, int lane) {
  const LDS_AS f32x4* p = (const LDS_AS f32x4*)(tab + tile * kTS + 4 * (lane >> 5));
  f32x16 s;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4 v = p[2 * k];  // tokens 8k + 4*(l/32) .. +3
#pragma unroll
    for (int e = 0; e < 4; ++e) s[4 * k + e] = v[e];
  }
  return s;
}

// Tiled (FP8 cache) partial S^T: the code-tile accumulators scaled per
// token (scale table `stab` of the slot) and added to the rope accumulator,
// in fp32.
template <int NSPLIT, bool TILED>
__device__ __forceinline__ f32x16 qk_combine(const f32x16 (&acc)[kMaxAcc], const LDS_AS float* stab, int part,
                                             int lane) {
  if constexpr (TILED) {
    constexpr int TPP = Tiling<NSPLIT>::TPP;
    f32x16 s = acc[TPP];
#pragma unroll
    for (int j = 0; j < TPP; ++j) {
      const f32x16 sc = tile_scales(stab, TPP * part + j, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(sc[r], acc[j][r], s[r]);
    }
    return s;
  } else {
    return acc[0];
  }
}

// Partial QK^T of one slot, its first kRA - 1 fragments already loaded
// (kb); with PIPE the previous slot's softmax, the first V^T block of its PV
// and the copies of a later slot are interleaved with it.
template <int NSPLIT, int PIPE, bool TILED = false>
__device__ __forceinline__ f32x16 qk_partial(bf16x8 (&kb)[kRA], const lds_char* buf,
                                             const bf16x8 (&qf)[kKSteps / NSPLIT], const LaneTables& t,
                                             const QkSide& side, SoftPipe& sp, SoftmaxState& st, const SoftCtx& c,
                                             const LDS_AS float* stab = nullptr, int part = 0) {
  static_assert((kKSteps / NSPLIT) % kDmaPerWave == 0, "copies spread evenly over the k-steps");
  f32x16 acc[kMaxAcc];
  qk_steps<NSPLIT, 0, PIPE, TILED>(acc, kb, buf, qf, t, side, sp, st, c);
  __builtin_amdgcn_sched_barrier(0);
  return qk_combine<NSPLIT, TILED>(acc, stab, part, c.lane);
}

// Softmax numerators of one slot as bf16 P^T operands.  Lane l, register r
// holds token 8*(r/4) + 4*(l/32) + r%4 of head l%32; tokens at and beyond
// nvalid (only the last slot of a segment has any) get p = 0.
__device__ __forceinline__ void softmax_slot(const f32x16& s, uint32_t mask, SoftmaxState& st, float scale_log2,
                                             f32x8& p0, f32x8& p1, int lane, bool own_l = false) {
  f32x16 x = s;
  apply_mask(x, mask, lane);
  float mx = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
  mx = max_halves(mx) * scale_log2;  // scale_log2 > 0: the max commutes with the scaling
  // the first slot fixes the reference; later slots may exceed it by up to
  // kTau without loss (p <= 2^kTau), beyond that the segment is redone
  st.m_ref = st.m_ref == -INFINITY ? mx : st.m_ref;
  st.m_seen = fmaxf(st.m_seen, mx);
  const float nref = neg_ref(st.m_ref);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    p0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], scale_log2, nref));
    p1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r + 8], scale_log2, nref));
  }
  float lsum = 0.0f;
  // (own_l: token-split softmax, only this wave's tokens, registers 0..7)
#pragma unroll
  for (int r = 0; r < 8; ++r) lsum += own_l ? p0[r] : p0[r] + p1[r];
  st.l_sum += lsum;
}

// P^T operands of the PV product: the numerators as bf16; tiled (FP8 cache),
// once per code tile of this part with each token's tile scale folded in, so
// that the codes themselves serve as V: sum_t p_t (code_t,c * s_t,tile(c)).
template <int NSPLIT, bool TILED>
struct POps {
  static constexpr int N = TILED ? Tiling<NSPLIT>::TPP : 1;
  bf16x8 b0[N], b1[N];
};

template <int NSPLIT, bool TILED>
__device__ __forceinline__ void make_pops(POps<NSPLIT, TILED>& po, const f32x8& p0, const f32x8& p1,
                                          const LDS_AS float* stab, int part, int lane) {
  if constexpr (TILED) {
#pragma unroll
    for (int j = 0; j < POps<NSPLIT, TILED>::N; ++j) {
      const f32x16 sc = tile_scales(stab, POps<NSPLIT, TILED>::N * part + j, lane);
      f32x8 a, b;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        a[r] = p0[r] * sc[r];
        b[r] = p1[r] * sc[r + 8];
      }
      po.b0[j] = __builtin_convertvector(a, bf16x8);
      po.b1[j] = __builtin_convertvector(b, bf16x8);
    }
  } else {
    po.b0[0] = __builtin_convertvector(p0, bf16x8);
    po.b1[0] = __builtin_convertvector(p1, bf16x8);
  }
}


// O^T[c][head] += V^T . P^T over this wave's column blocks.  k-step 0 of a
// block covers tokens 0..15 in the order the S^T layout hands them to this
// lane (rows 4h+j and 8+4h+j), k-step 1 tokens 16..31.  The first block's
// V^T operands arrive loaded (va0).  Three operand buffers: the reads for
// block cb + 1 go to the buffer of block cb - 2, whose MFMAs have left the
// matrix core (block cb - 1's may not have).
template <int NSPLIT, bool TILED>
__device__ __forceinline__ void pv_slot(const lds_char* buf, const VBlock& va0, const POps<NSPLIT, TILED>& po,
                                        const LaneTables& t, Acc<NSPLIT>& acc) {
  constexpr int NCB = kCB / NSPLIT;
  constexpr int BPS = NCB / POps<NSPLIT, TILED>::N;  // column blocks per operand set
  VBlock va[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) va[0][i] = va0[i];
  bf16x8 prev0 = {}, prev1 = {};  // operands of the previous block's MFMAs
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    __builtin_amdgcn_sched_barrier(0);
    const VBlock& v = va[cb % 3];
    const bf16x8 v0 = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 v1 = __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3, 4, 5, 6, 7);
    acc.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, po.b0[cb / BPS], acc.o[cb], 0, 0, 0);
    acc.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, po.b1[cb / BPS], acc.o[cb], 0, 0, 0);
    if (cb + 1 < NCB) pv_load(buf, t, cb + 1, va[(cb + 1) % 3]);
    // this block's operands, and the previous block's (its MFMAs are
    // independent of these and may still be in the matrix core), stay
    // out of the reads' way
    keep_alive(v0);
    keep_alive(v1);
    if (cb > 0) {
      keep_alive(prev0);
      keep_alive(prev1);
    }
    prev0 = v0;
    prev1 = v1;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// pv_slot with the reads two column blocks ahead: blocks 0 and 1 arrive
// loaded, and the reads for block cb + 2 go to the buffer of block cb - 2
// (four buffers), whose MFMAs have left the matrix core.  Token-split
// softmax: the PV starts right after the barrier that publishes the
// partner's P^T half, and its read is then the only one in flight.
template <int NSPLIT>
__device__ __forceinline__ void pv_slot2(const lds_char* buf, const VBlock& va0, const VBlock& va1,
                                         const POps<NSPLIT, false>& po, const LaneTables& t, Acc<NSPLIT>& acc) {
  constexpr int NCB = kCB / NSPLIT;
  VBlock va[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    va[0][i] = va0[i];
    va[1][i] = va1[i];
  }
  bf16x8 prev0 = {}, prev1 = {};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    __builtin_amdgcn_sched_barrier(0);
    const VBlock& v = va[cb % 4];
    const bf16x8 v0 = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 v1 = __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3, 4, 5, 6, 7);
    acc.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, po.b0[0], acc.o[cb], 0, 0, 0);
    acc.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, po.b1[0], acc.o[cb], 0, 0, 0);
    if (cb + 2 < NCB) pv_load(buf, t, cb + 2, va[(cb + 2) % 4]);
    keep_alive(v0);
    keep_alive(v1);
    if (cb > 0) {
      keep_alive(prev0);
      keep_alive(prev1);
    }
    prev0 = v0;
    prev1 = v1;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------- the kernel

template <int NSPLIT, bool Q_FP8, int KVM, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char ring_mem[kRing * kSlotBytes];  // KV ring, 4 x 36 KB
  __shared__ __attribute__((aligned(16))) f32x4 xbuf[kWaves * 4 * 64];         // partial S^T, 16 KB
  lds_char* const ring = (lds_char*)ring_mem;
  LDS_AS f32x4* const xch = (LDS_AS f32x4*)xbuf;
  // redo votes reuse the exchange buffer between segments, after barriers
  // that every wave reaches past its last exchange read
  volatile int* const votes = (volatile int*)xbuf;

  constexpr int KS = kKSteps / NSPLIT;
  constexpr int NCB = kCB / NSPLIT;
  constexpr int HG = kWaves / NSPLIT;  // 32-head groups per workgroup
  constexpr bool TILED = kv_fp8(KVM);  // FP8 cache: tiled QK^T split, scales applied in fp32
  // Token-split softmax (bf16 copy ring or per-tensor FP8 fill, two parts): after a
  // segment's first slot, each wave of a pair takes the softmax of its own 16
  // tokens only and the pair swaps bf16 P^T halves before PV.  Part 1 reads
  // its K rows as 16..31, 0..15, so its own tokens sit in S^T registers 0..7
  // as part 0's do.  The first slot runs the full exchange, so the two waves
  // fix the same reference; l_sum holds own tokens only and the pair adds its
  // two sums at the end.  Part 1 applies token masks rotated by 16
  // (own_mask).  A row whose tokens in the first slot are all
  // masked sees none later in the segment either (the limit only falls
  // behind), so its reference stays -inf in both waves.
  // (dense caches without tile scales: a top-k slot 0 may be all padding
  // while later slots are not, which would leave the two references apart)
  constexpr bool TSOFT = NSPLIT == 2 && (KVM == kKvBf16 || KVM == kKvFp8T);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = w / NSPLIT, part = w % NSPLIT;

  const int g = blockIdx.x;
  // workgroups are dealt round-robin to the 8 XCDs: each XCD gets a run of
  // consecutive ranges with all their slabs, so the slabs share KV lines in
  // one L2 and the pieces of a sequence mostly merge from it
  const int idx = g / 8;
  const int r = (g % 8) * a.per_xcd + idx / a.slabs;
  const int slab = idx % a.slabs;
  Plan pl;
  // (the plan also loads the length of sequence g, checked for emptiness below)
  int units_g = 1;
  const bool has_work = make_plan<kThreads>(a, r, (int*)ring_mem, pl, units_g) && r < a.ranges;
  // sequences with nothing to attend: O = 0, LSE = -inf (spread over the
  // grid; the lengths were just read by the plan)
  for (int b = g; b < a.batch; b += gridDim.x) {
    if ((b == g ? units_g : units_of(a, b)) == 0) {
      for (int i = tid; i < a.heads * (kDV / 4); i += kThreads)
        *(bf16x4*)((__bf16*)a.out + ((size_t)b * a.heads) * kDV + 4 * i) = bf16x4{};
      for (int i = tid; i < a.heads; i += kThreads) a.lse[(size_t)b * a.heads + i] = -INFINITY;
      if (tid == 0) a.ws_seq[b] = int2{0, 0};
    }
  }
  if (!has_work) return;

  const int head = slab * (HG * 32) + hg * 32 + (lane & 31);
  const bool head_ok = head < a.heads;
  // per-tensor FP8 cache: every value is code / k_scale_inv; the factor goes
  // into the score scale and the output normalisation, the ring holds codes
  float kdesc = 1.0f;
  if constexpr (kv_tensor(KVM)) kdesc = 1.0f / a.kv_scales[0];
  const float scale_log2 = a.scale_log2 * kdesc;
  // T query tokens per sequence (causal): row `head` is head head % heads_tok
  // of query token t = head / heads_tok, which sees the positions below
  // seqlen - lag with lag = T - 1 - t
  int lag = 0;
  if constexpr (CAUSAL) lag = a.tq - 1 - min(head, a.heads - 1) / a.heads_tok;

  LaneTables tab;
  make_tables<NSPLIT, TILED>(tab, lane, w, part, TSOFT && part == 1 ? 16 : 0);

  int b = pl.b0, p = pl.p0;
  bool first_seg = true;
  while (true) {
    const int n = units_of(a, b);
    const int gs = max(pl.start, p), ge = min(pl.end, p + n);
    if (gs < ge) {
      // ---- one segment: sequence b, units [gs - p, ge - p)
      if (!first_seg) {
        // every wave is done with the ring before it is refilled
        wait_vm_lgkm0<0>();
        barrier();
      }
      first_seg = false;
      // tokens of the sequence: positions [0, seqlen), or top-k entries [0, topk)
      const int seglen = kv_topk(KVM) ? a.topk : min(max(a.seqlens[b], 0), a.max_pages * kPage);
      SegCtx sg;
      sg.tok0 = (gs - p) * kPage;
      sg.tok1 = min((ge - p) * kPage, seglen);
      sg.nslots = (sg.tok1 - sg.tok0 + kTS - 1) / kTS;
      sg.npages = (sg.nslots + 1) / 2;
      sg.bt_seg = a.block_table + (size_t)b * a.max_pages + (gs - p);
      sg.idx_seg = a.topk_idx + (size_t)b * a.topk + sg.tok0;
      const int first_r = p / pl.C, last_r = (p + n - 1) / pl.C;
      const int nsplit = last_r - first_r + 1;
      const int nslots = sg.nslots;
      // causal: this lane's row sees the segment's tokens below lim; slots
      // from causal_from on hide a token from some row (at most the last two)
      int lim = sg.tok1, causal_from = nslots;
      if constexpr (CAUSAL) {
        lim = min(sg.tok1, seglen - lag);
        const int lim0 = seglen - (a.tq - 1);
        causal_from = lim0 >= sg.tok1 ? nslots : max(0, (lim0 - sg.tok0) / kTS);
      }
      auto causal_mask = [&](int s) -> uint32_t {
        const int nv = lim - (sg.tok0 + s * kTS);
        return nv <= 0 ? 0u : low_mask(nv);
      };
      // a token mask as this wave's S^T registers hold the tokens
      auto own_mask = [&](uint32_t m) -> uint32_t { return TSOFT && part == 1 ? (m >> 16) | (m << 16) : m; };

      // query fragments (B operand of S^T = K.Q^T): head `head`, columns
      // 16g + 8*(lane/32) .. +7 for global k-step g of this wave's local step i
      bf16x8 qf[KS];
      if constexpr (!Q_FP8) {
        const bf16x8* qrow = (const bf16x8*)((const __bf16*)a.q + ((size_t)b * a.heads + (head_ok ? head : 0)) * kD);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const bf16x8 v = qrow[2 * global_step<NSPLIT, TILED>(part, i) + (lane >> 5)];
          qf[i] = head_ok ? v : bf16x8{};
        }
      } else {
        const uint2* qrow = (const uint2*)((const uint8_t*)a.q + ((size_t)b * a.heads + (head_ok ? head : 0)) * kD);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const uint2 v = qrow[2 * global_step<NSPLIT, TILED>(part, i) + (lane >> 5)];
          qf[i] = head_ok ? fp8x8_to_bf16(v, a.q_descale) : bf16x8{};
        }
      }

      PageCache pc;
      // (also completes the query loads, so the ring's vmcnt accounting
      // counts DMA only)
      if constexpr (!kv_topk(KVM)) page_cache_load(pc, sg.bt_seg, 0, sg.npages, lane);
      // register fill: this lane's row of a slot and its 128-byte piece
      const int frow = 8 * w + (lane & 7), fq = lane >> 3;
      // physical row that this lane fills for slot t of the segment (slots
      // past the end repeat the last one; rows past the valid count repeat
      // the last valid row)
      auto fill_src = [&](int t) -> int {
        t = min(t, nslots - 1);
        const int page = page_of(pc, sg.bt_seg, t >> 1, sg.npages, lane, a.num_pages);
        const int nv = min(kTS, sg.tok1 - (sg.tok0 + t * kTS));
        return page * kPage + (t & 1) * kTS + min(frow, nv - 1);
      };
      // top-k, in two stages one pipeline step apart: the listed position of
      // this lane's row of slot t (-1 past the segment's end), then its pool
      // row block_table[b / T][j / 64]*64 + j % 64.  A position is valid iff
      // 0 <= j < the list's causal limit (seqlen when T = 1); a masked entry
      // reads row 0, and its p is 0.  Both loads are unconditional, from
      // clamped addresses.
      int tk_limit = 0;
      const int32_t* tk_bt = a.block_table;
      if constexpr (kv_topk(KVM)) {
        const int bs = b / a.topk_tq;
        tk_limit = min(max(a.seqlens[bs], 0), a.max_pages * kPage) - (a.topk_tq - 1 - b % a.topk_tq);
        tk_bt = a.block_table + (size_t)bs * a.max_pages;
      }
      auto topk_pos = [&](int t) -> int {
        const int e = min(t, nslots - 1) * kTS + frow;
        const int ne = sg.tok1 - sg.tok0;
        const int j = sg.idx_seg[min(e, ne - 1)];
        return e < ne ? j : -1;
      };
      auto topk_ok = [&](int j) -> bool { return j >= 0 && j < tk_limit; };
      auto topk_row = [&](int j) -> int {
        const int jc = topk_ok(j) ? j : 0;
        const int row = clamp_page(tk_bt[jc >> 6], a.num_pages) * kPage + (jc & (kPage - 1));
        return topk_ok(j) ? row : 0;
      };
      // top-k validity words, one per ring position (the fill of a slot sets
      // byte w from wave w's eight rows), after the scale tables
      LDS_AS uint32_t* const tk_masks = (LDS_AS uint32_t*)(ring + kFillRing * kSlotBytes + 2048);
      auto put_mask = [&](int pos, bool ok) {
        const uint32_t bits = (uint32_t)__ballot(ok) & 0xFFu;  // lanes 0..7: rows 8w .. 8w+7
        if (lane == 0) ((LDS_AS uint8_t*)(tk_masks + pos))[w] = (uint8_t)bits;
      };
      // validity of the tokens of slot s (dense: only the last slot is
      // short; top-k: the word its fill wrote, at position s % 3)
      auto slot_mask = [&](int s) -> uint32_t {
        if constexpr (kv_topk(KVM)) {
          return tk_masks[s % kFillRing];
        } else {
          return low_mask(sg.tok1 - (sg.tok0 + s * kTS));
        }
      };

      SoftmaxState st;
      st.m_ref = -INFINITY;
      Acc<NSPLIT> acc;
      // At most two passes: the second only if some head's scores rose more
      // than kTau above the reference its first slot set (p would exceed
      // 2^kTau); it then runs with the true maxima, so all p <= 1.
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int c = 0; c < NCB; ++c) acc.o[c] = f32x16{};
        st.l_sum = 0.0f;
        st.m_seen = -INFINITY;
        const SoftCtx sctx{xch, w, lane, scale_log2, TSOFT ? 2 : 0};
        SoftPipe sp;
        POps<NSPLIT, TILED> po;
        bf16x8 kb[kRA];
        VBlock va0, va1;
        f32x16 sc;
        int last_pos;  // ring position of the last slot
        if constexpr (KVM == kKvBf16) {
          // prologue: slots 0..2 in flight (slots past the end re-copy the
          // last one), partial QK^T of slot 0
#pragma unroll
          for (int s = 0; s < 3; ++s) dma_issue_all(prep_slot(s, s, ring, a, sg, pc, tab.dma, w, lane));
          wait_vm_lgkm0<2 * kDmaPerWave>();
          barrier();
          qk_preload<NSPLIT, false>(kb, ring, tab);
          sc = qk_partial<NSPLIT, 0>(kb, ring, qf, tab, QkSide{}, sp, st, sctx);
          // steady state, slot s: publish its partial (computed one step
          // earlier) and wait for slot s+1 (slot s+2 stays in flight);
          // barrier; then the partial QK^T of slot s+1 runs beside the
          // softmax of slot s with the copies of slot s+3 (into the ring
          // position that slot s-1 left) between its MFMAs, then PV of slot
          // s; a second barrier frees ring position s and the exchange buffer
          int s_first = 0;
          if constexpr (TSOFT) {
            if (nslots > 1) {
              // slot 0 as below, full exchange (own tokens into l_sum)
              put_partial(xch, sc, w, lane);
              wait_vm_lgkm0<kDmaPerWave>();
              barrier();
              const lds_char* const kbuf = ring + kSlotBytes;
              qk_preload<NSPLIT, false>(kb, kbuf, tab);
              soft_read<NSPLIT>(sp, sctx);
              __builtin_amdgcn_sched_barrier(0);
              QkSide side;
              side.job = prep_slot(3, 3, ring, a, sg, pc, tab.dma, w, lane);
              side.pvbuf = ring;
              side.va0 = &va0;
              sp.own = sc;
              if (CAUSAL && causal_from == 0) {
                sp.mask = own_mask(causal_mask(0));
                sc = qk_partial<NSPLIT, kPipeDma | kPipeSoft | kPipeOwnL | kPipeMask>(kb, kbuf, qf, tab, side, sp, st,
                                                                                    sctx);
              } else {
                sc = qk_partial<NSPLIT, kPipeDma | kPipeSoft | kPipeOwnL>(kb, kbuf, qf, tab, side, sp, st, sctx);
              }
              make_pops<NSPLIT, TILED>(po, sp.p0, sp.p1, nullptr, part, lane);
              pv_slot<NSPLIT, TILED>(side.pvbuf, va0, po, tab, acc);
              wait_vm_lgkm0<63>();
              barrier();
              s_first = 1;
            }
            // slots 1 ..: the partner needs only this wave's registers
            // 8..15; after the QK^T of slot s+1 (with the own-half softmax of
            // slot s) the pair swaps P^T halves through r4 slot 0 of each
            // wave's exchange region; a barrier orders the swap, and the
            // next slot's first barrier (after lgkmcnt(0)) frees the ring
            // position and the exchange buffer
            for (int s = s_first; s + 1 < nslots; ++s) {
              put_partial_half(xch, sc, w, lane);
              wait_vm_lgkm0<kDmaPerWave>();
              barrier();
              const lds_char* const kbuf = ring + ((s + 1) & (kRing - 1)) * kSlotBytes;
              qk_preload<NSPLIT, false>(kb, kbuf, tab);
              soft_read_half(sp, sctx);
              __builtin_amdgcn_sched_barrier(0);
              QkSide side;
              side.job = prep_slot(s + 3, s + 3, ring, a, sg, pc, tab.dma, w, lane);
              side.pvbuf = ring + (s & (kRing - 1)) * kSlotBytes;
              side.va0 = &va0;
              side.va1 = &va1;
              sp.own = sc;
              if (CAUSAL && s >= causal_from) {
                sp.mask = own_mask(causal_mask(s));
                sc = qk_partial<NSPLIT, kPipeDma | kPipeSoft | kPipeHalf | kPipePv2 | kPipeMask>(kb, kbuf, qf, tab, side,
                                                                                               sp, st, sctx);
              } else {
                sc = qk_partial<NSPLIT, kPipeDma | kPipeSoft | kPipeHalf | kPipePv2>(kb, kbuf, qf, tab, side, sp, st,
                                                                                     sctx);
              }
              const bf16x8 mine = __builtin_convertvector(sp.p0, bf16x8);
              *(LDS_AS bf16x8*)(xch + (w * 4) * 64 + lane) = mine;
              wait_vm_lgkm0<63>();
              barrier();
              po.b0[0] = mine;
              po.b1[0] = *(const LDS_AS bf16x8*)(xch + ((w ^ 1) * 4) * 64 + lane);
              pv_slot2<NSPLIT>(side.pvbuf, va0, va1, po, tab, acc);
            }
            // the partner may still be reading this wave's P^T half
            wait_vm_lgkm0<63>();
            barrier();
          }
          for (int s = 0; !TSOFT && s + 1 < nslots; ++s) {
            put_partial(xch, sc, w, lane);
            wait_vm_lgkm0<kDmaPerWave>();
            barrier();
            // LDS reads first: the next slot's first K fragments and the
            // partners' partials of this one
            const lds_char* const kbuf = ring + ((s + 1) & (kRing - 1)) * kSlotBytes;
            qk_preload<NSPLIT, false>(kb, kbuf, tab);
            soft_read<NSPLIT>(sp, sctx);
            __builtin_amdgcn_sched_barrier(0);
            QkSide side;
            side.job = prep_slot(s + 3, s + 3, ring, a, sg, pc, tab.dma, w, lane);
            side.pvbuf = ring + (s & (kRing - 1)) * kSlotBytes;
            side.va0 = &va0;
            sp.own = sc;
            if constexpr (CAUSAL) {
              if (s >= causal_from) {
                sp.mask = causal_mask(s);
                sc = qk_partial<NSPLIT, kPipeDma | kPipeSoft | kPipeMask>(kb, kbuf, qf, tab, side, sp, st, sctx);
              } else {
                sc = qk_partial<NSPLIT, kPipeDma | kPipeSoft>(kb, kbuf, qf, tab, side, sp, st, sctx);
              }
            } else {
              sc = qk_partial<NSPLIT, kPipeDma | kPipeSoft>(kb, kbuf, qf, tab, side, sp, st, sctx);
            }
            make_pops<NSPLIT, TILED>(po, sp.p0, sp.p1, nullptr, part, lane);
            pv_slot<NSPLIT, TILED>(side.pvbuf, va0, po, tab, acc);
            wait_vm_lgkm0<63>();  // lgkmcnt(0): this wave's LDS reads are done
            barrier();
          }
          put_partial(xch, sc, w, lane);
          wait_vm_lgkm0<0>();
          last_pos = (nslots - 1) & (kRing - 1);
        } else {
          // register fill through a ring of three positions (slot s at
          // position s % 3); the fourth slot region holds the FP8 scale
          // tables, one per position.  A slot's rows are loaded one step
          // before the lanes write them into the ring, and (top-k) each
          // row's index one step before that.  Prologue: slots 0 and 1
          // written, slot 2 loaded, partial QK^T of slot 0.
          LDS_AS float* const stabs = (LDS_AS float*)(ring + kFillRing * kSlotBytes);
          auto pos_buf = [&](int pos) { return ring + pos * kSlotBytes; };
          auto pos_tab = [&](int pos) { return stabs + pos * (4 * kTS); };
          // (the rows of slots 0..2, and their indices, are all requested
          // before the first is needed: one memory latency, not three)
          RawRow<KVM> rr;
          int next_row;
          bool rr_ok = true, next_ok = true;  // top-k: validity of the rows of rr / next_row
          int next_j = 0;                     // top-k: listed position of slot s+5
          if constexpr (kv_topk(KVM)) {
            const int j0 = topk_pos(0), j1 = topk_pos(1), j2 = topk_pos(2), j3 = topk_pos(3);
            next_j = topk_pos(4);
            const int i0 = topk_row(j0), i1 = topk_row(j1), i2 = topk_row(j2);
            next_row = topk_row(j3);
            next_ok = topk_ok(j3);
            RawRow<KVM> r0, r1;
            load_row<KVM>(r0, a, i0, fq);
            load_row<KVM>(r1, a, i1, fq);
            load_row<KVM>(rr, a, i2, fq);
            rr_ok = topk_ok(j2);
            fill_row<KVM>(pos_buf(0), pos_tab(0), r0, frow, fq);
            put_mask(0, topk_ok(j0));
            fill_row<KVM>(pos_buf(1), pos_tab(1), r1, frow, fq);
            put_mask(1, topk_ok(j1));
          } else {
            const int i0 = fill_src(0), i1 = fill_src(1), i2 = fill_src(2);
            next_row = fill_src(3);
            RawRow<KVM> r0, r1;
            load_row<KVM>(r0, a, i0, fq);
            load_row<KVM>(r1, a, i1, fq);
            load_row<KVM>(rr, a, i2, fq);
            fill_row<KVM>(pos_buf(0), pos_tab(0), r0, frow, fq);
            fill_row<KVM>(pos_buf(1), pos_tab(1), r1, frow, fq);
          }
          wait_vm_lgkm0<63>();
          barrier();
          qk_preload<NSPLIT, TILED>(kb, pos_buf(0), tab);
          sc = qk_partial<NSPLIT, 0, TILED>(kb, pos_buf(0), qf, tab, QkSide{}, sp, st, sctx, pos_tab(0), part);
          // steady state, slot s: as in the copy ring, with no copies in the
          // QK^T; after PV of slot s the lanes write slot s+2 (loaded one
          // step earlier) into the position that slot s-1 left, and load
          // slot s+3
          int p0 = 0, p1 = 1, p2 = 2;  // positions of slots s, s+1, s+2
          for (int s = 0; s + 1 < nslots; ++s) {
            // token-split: slot 0 as the copy ring's first slot, later
            // slots with the half exchange and the P^T swap, whose barrier
            // takes the place of the end-of-slot one
            const bool half = TSOFT && s > 0;
            if (half) put_partial_half(xch, sc, w, lane);
            else put_partial(xch, sc, w, lane);
            wait_vm_lgkm0<63>();
            barrier();
            qk_preload<NSPLIT, TILED>(kb, pos_buf(p1), tab);
            if (half) soft_read_half(sp, sctx);
            else soft_read<NSPLIT>(sp, sctx);
            __builtin_amdgcn_sched_barrier(0);
            QkSide side;
            side.pvbuf = pos_buf(p0);
            side.va0 = &va0;
            sp.own = sc;
            if constexpr (TSOFT) {
              const bool masked = CAUSAL && s >= causal_from;
              if (masked) sp.mask = own_mask(causal_mask(s));
              if (half) {
                if (masked)
                  sc = qk_partial<NSPLIT, kPipeSoft | kPipeHalf | kPipeMask>(kb, pos_buf(p1), qf, tab, side, sp, st,
                                                                            sctx);
                else
                  sc = qk_partial<NSPLIT, kPipeSoft | kPipeHalf>(kb, pos_buf(p1), qf, tab, side, sp, st, sctx);
                const bf16x8 mine = __builtin_convertvector(sp.p0, bf16x8);
                *(LDS_AS bf16x8*)(xch + (w * 4) * 64 + lane) = mine;
                wait_vm_lgkm0<63>();
                barrier();
                po.b0[0] = mine;
                po.b1[0] = *(const LDS_AS bf16x8*)(xch + ((w ^ 1) * 4) * 64 + lane);
              } else {
                if (masked)
                  sc = qk_partial<NSPLIT, kPipeSoft | kPipeOwnL | kPipeMask>(kb, pos_buf(p1), qf, tab, side, sp, st,
                                                                            sctx);
                else
                  sc = qk_partial<NSPLIT, kPipeSoft | kPipeOwnL>(kb, pos_buf(p1), qf, tab, side, sp, st, sctx);
                make_pops<NSPLIT, TILED>(po, sp.p0, sp.p1, nullptr, part, lane);
              }
            } else if constexpr (kv_topk(KVM)) {
              sp.mask = slot_mask(s);
              sc = qk_partial<NSPLIT, kPipeSoft | kPipeMask, TILED>(kb, pos_buf(p1), qf, tab, side, sp, st, sctx,
                                                                   pos_tab(p1), part);
            } else if (CAUSAL && s >= causal_from) {
              sp.mask = causal_mask(s);
              sc = qk_partial<NSPLIT, kPipeSoft | kPipeMask, TILED>(kb, pos_buf(p1), qf, tab, side, sp, st, sctx,
                                                                   pos_tab(p1), part);
            } else {
              sc = qk_partial<NSPLIT, kPipeSoft, TILED>(kb, pos_buf(p1), qf, tab, side, sp, st, sctx, pos_tab(p1),
                                                        part);
            }
            if constexpr (!TSOFT) make_pops<NSPLIT, TILED>(po, sp.p0, sp.p1, pos_tab(p0), part, lane);
            pv_slot<NSPLIT, TILED>(side.pvbuf, va0, po, tab, acc);
            fill_row<KVM>(pos_buf(p2), pos_tab(p2), rr, frow, fq);
            const int row = next_row;
            if constexpr (kv_topk(KVM)) {
              put_mask(p2, rr_ok);
              rr_ok = next_ok;
              next_ok = topk_ok(next_j);
              next_row = topk_row(next_j);  // slot s+4
              next_j = topk_pos(s + 5);
            } else {
              next_row = fill_src(s + 4);
            }
            load_row<KVM>(rr, a, row, fq);
            if (!half) {
              wait_vm_lgkm0<63>();  // this wave's LDS reads and writes are done
              barrier();
            }
            const int pn = p0;
            p0 = p1;
            p1 = p2;
            p2 = pn;
          }
          if constexpr (TSOFT) {
            // the partner may still be reading this wave's P^T half
            wait_vm_lgkm0<63>();
            barrier();
          }
          put_partial(xch, sc, w, lane);
          wait_vm_lgkm0<63>();
          last_pos = p0;
        }
        {
          // last slot (the only dense one that can be short)
          barrier();
          const f32x16 tot = total_scores<NSPLIT>(xch, sc, w, lane, TSOFT ? 2 : 0);
          f32x8 q0, q1;
          const uint32_t lmask = own_mask(CAUSAL ? causal_mask(nslots - 1) : slot_mask(nslots - 1));
          softmax_slot(tot, lmask, st, scale_log2, q0, q1, lane, TSOFT);
          const LDS_AS float* ltab = (const LDS_AS float*)(ring + kFillRing * kSlotBytes) + last_pos * (4 * kTS);
          pv_load(ring + last_pos * kSlotBytes, tab, 0, va0);
          make_pops<NSPLIT, TILED>(po, q0, q1, ltab, part, lane);
          pv_slot<NSPLIT, TILED>(ring + last_pos * kSlotBytes, va0, po, tab, acc);
        }
        // workgroup vote on a redo (every wave is past its last exchange read)
        wait_vm_lgkm0<0>();
        barrier();
        const int my_vote = __any(st.m_seen > st.m_ref + kTau) ? 1 : 0;  // all lanes vote
        if (lane == 0) votes[w] = my_vote;
        // token-split: m_seen covers this wave's tokens; a redo takes the
        // pair's max (exchanged beside the votes)
        LDS_AS float* const mx_x = (LDS_AS float*)xbuf + 1024;
        if constexpr (TSOFT) mx_x[w * 64 + lane] = st.m_seen;
        wait_vm_lgkm0<0>();
        barrier();
        int vote = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) vote |= votes[i];
        float m_pair = st.m_seen;
        if constexpr (TSOFT) m_pair = fmaxf(m_pair, mx_x[(w ^ 1) * 64 + lane]);
        wait_vm_lgkm0<0>();
        barrier();  // votes read before the buffer is reused
        if (!__builtin_amdgcn_readfirstlane(vote)) break;
        st.m_ref = m_pair;
        if (!kv_topk(KVM) && sg.npages > 64) page_cache_load(pc, sg.bt_seg, 0, sg.npages, lane);
      }

      // ---- epilogue: normalise and store this wave's columns (final output,
      // or this piece's partial in its workspace slot)
      float l_tot = sum_halves(st.l_sum);
      if constexpr (TSOFT) {
        // the pair's two token halves (the buffer is free after the vote)
        LDS_AS float* const l_x = (LDS_AS float*)xbuf + 2048;
        l_x[w * 64 + lane] = l_tot;
        wait_vm_lgkm0<0>();
        barrier();
        l_tot += l_x[(w ^ 1) * 64 + lane];
      }
      const float inv = l_tot > 0.0f ? kdesc / l_tot : 0.0f;
      const float lse2 = l_tot > 0.0f ? st.m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
      if (head_ok) {
        const size_t pslot = piece_slot(a, b, r, first_r);
        __bf16* orow = (__bf16*)a.out + ((size_t)b * a.heads + head) * kDV;
        float* prow = a.ws_o + (pslot * a.heads + head) * kDV;
#pragma unroll
        for (int cbi = 0; cbi < NCB; ++cbi) {
          const int cb = part * NCB + cbi;
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int col = 32 * cb + 8 * rg + 4 * (lane >> 5);
            f32x4 v = {acc.o[cbi][4 * rg], acc.o[cbi][4 * rg + 1], acc.o[cbi][4 * rg + 2], acc.o[cbi][4 * rg + 3]};
            v *= inv;
            // partials stay fp32: a second bf16 rounding would double the
            // output's rounding error where |O| is large
            if (nsplit == 1) *(bf16x4*)(orow + col) = __builtin_convertvector(v, bf16x4);
            else *(f32x4*)(prow + col) = v;
          }
        }
        if (part == 0 && lane < 32) {
          if (nsplit == 1) a.lse[(size_t)b * a.heads + head] = lse2 * kLn2;
          else a.ws_lse[pslot * a.heads + head] = lse2;
        }
      }
      // where the pieces of b sit (every piece writes the same record); the
      // merge kernel that follows on the stream combines split sequences
      if (tid == 0) a.ws_seq[b] = int2{first_r, nsplit};
    }
    p += n;
    ++b;
    if (p >= pl.end || b >= a.batch) break;
  }
}

// ---------------------------------------------------------------- split-KV merge

struct MergeArgs {
  const int2* seq;   // [B] {workspace slot of piece 0, pieces}
  const float* ws_o;
  const _Float16* ws_o16;  // scaled fp16 partials and their factors (wave-specialised kernel)
  const float* ws_sc;
  const float* ws_lse;
  void* out;
  float* lse;
  int32_t heads;
  int32_t compact;  // the slot layout of DecodeArgs::compact
  // top-k lists (topk_units = ceil(topk / 64) > 0): the decode's cut of the
  // line has a closed form (even_cut), so the pieces of a list are known
  // without reading its record; 0 for pages
  int32_t topk_units;
  int32_t batch;
  int32_t ranges;
  int32_t seg_pad;
};

// workspace slot of piece s of sequence b whose first range is first_r
__device__ __forceinline__ size_t merge_slot(const MergeArgs& m, int b, int first_r, int s) {
  const int r = first_r + s;
  return m.compact ? (size_t)(2 * r + (s == 0 ? 1 : 0)) : (size_t)(b + r);
}

constexpr int kMergeHeads = 4;  // heads per merge workgroup, 64 threads each

// O = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M) with M = max_s lse_s, and
// LSE = M + log2 sum_s 2^(lse_s - M) (back to natural log), for sequences the
// decode kernel split over several ranges; piece s sits in workspace slot
// first + s.  A thread owns two float4 column groups of one head, and the
// grid has B * H / 4 workgroups.  Pieces go in chunks of up to eight whose LSEs
// and O columns are all requested together (one memory latency per chunk);
// a later chunk with a larger max rescales the sums so far (up to eight
// pieces, M is the max of all of them, as written above).
// Partials come as fp32 (F16 false) or, from the wave-specialised kernel, as
// fp16 values v with a power-of-two factor f per row and 128 columns, O_s =
// v * f exactly as the piece rounded it.
constexpr int kMergeChunk = 8;
constexpr int kMergeU = kDV / 4 / (kThreads / kMergeHeads);  // float4 columns per thread

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Pieces s0 .. s0+N-1 of one column group: every load issued before any is
// used (a fixed count, so no branch separates them).  `col` is the first
// column of the thread's group u = 0 (group u starts 4 * TPH * u later).
template <int N, bool F16>
__device__ __forceinline__ void merge_chunk(const MergeArgs& m, int b, int first_r, int head, int col,
                                            int s0, f32x4 (&acc)[kMergeU], float& mx, float& wsum) {
  constexpr int TPH = kThreads / kMergeHeads;
  const int heads = m.heads;
  float l[N];
  f32x4 v[N][kMergeU];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const size_t row = merge_slot(m, b, first_r, s0 + i) * heads + head;  // (slot, head) row of piece s0 + i
    l[i] = m.ws_lse[row];
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
      const int c = col + 4 * TPH * u;
      if constexpr (F16) {
        const f16x4 h = *(const f16x4*)(m.ws_o16 + row * kDV + c);
        const float f = m.ws_sc[row * 4 + c / 128];
        v[i][u] = __builtin_convertvector(h, f32x4) * f;
      } else {
        v[i][u] = *(const f32x4*)(m.ws_o + row * kDV + c);
      }
    }
  }
  float cm = mx;
#pragma unroll
  for (int i = 0; i < N; ++i) cm = fmaxf(cm, l[i]);
  // rescale what the earlier chunks summed (nothing before the first)
  const float r = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mx - cm);
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) acc[u] *= r;
  wsum *= r;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float wgt = l[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(l[i] - cm);
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) acc[u] += wgt * v[i][u];
    wsum += wgt;
  }
  mx = cm;
}

// The pieces of sequence b: its first range and their count.
__device__ __forceinline__ void merge_pieces(const MergeArgs& m, int b, int& first, int& nsplit) {
  if (m.topk_units > 0) {
    // list b's units [q, q + u) on the padded line, q = b (u + 2 pad) + pad
    int pad, C, total;
    even_cut(m.batch, m.topk_units, m.ranges, m.seg_pad, pad, C, total);
    const int q = b * (m.topk_units + 2 * pad) + pad;
    first = q / C;
    nsplit = (q + m.topk_units - 1) / C - first + 1;
  } else {
    const int2 info = m.seq[b];
    first = info.x;
    nsplit = info.y;
  }
}

// Pieces s_begin .. s_end-1 of one column group into a running state.
template <bool F16>
__device__ __forceinline__ void merge_run(const MergeArgs& m, int b, int first, int head, int col, int s_begin,
                                          int s_end, f32x4 (&acc)[kMergeU], float& mx, float& wsum) {
  for (int s0 = s_begin; s0 < s_end; s0 += kMergeChunk) {
    switch (min(kMergeChunk, s_end - s0)) {  // uniform over the wave
      case 1: merge_chunk<1, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
      case 2: merge_chunk<2, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
      case 3: merge_chunk<3, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
      case 4: merge_chunk<4, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
      case 5: merge_chunk<5, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
      case 6: merge_chunk<6, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
      case 7: merge_chunk<7, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
      default: merge_chunk<8, F16>(m, b, first, head, col, s0, acc, mx, wsum); break;
    }
  }
}

template <bool F16>
__global__ void __launch_bounds__(kThreads) mla_merge_kernel(MergeArgs m) {
  const int b = blockIdx.x;
  int first, nsplit;
  merge_pieces(m, b, first, nsplit);
  if (nsplit <= 1) return;
  constexpr int TPH = kThreads / kMergeHeads;
  const int head = blockIdx.y * kMergeHeads + threadIdx.x / TPH, sub = threadIdx.x % TPH;
  if (head >= m.heads) return;
  const int col = 4 * sub;
  constexpr int U = kMergeU;
  f32x4 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = f32x4{};
  float mx = -INFINITY, wsum = 0.0f;
  merge_run<F16>(m, b, first, head, col, 0, nsplit, acc, mx, wsum);
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  bf16x4* dst = (bf16x4*)((__bf16*)m.out + ((size_t)b * m.heads + head) * kDV) + sub;
#pragma unroll
  for (int u = 0; u < U; ++u) dst[u * TPH] = __builtin_convertvector(acc[u] * inv, bf16x4);
  if (sub == 0) m.lse[(size_t)b * m.heads + head] = wsum > 0.0f ? (mx + __builtin_amdgcn_logf(wsum)) * kLn2 : -INFINITY;
}

// The same combine for sequences split into many pieces, or grids too small
// to fill the chip: one workgroup per (sequence, head), its four waves taking
// consecutive quarters of the pieces (each in chunks, as above), then their
// running states (max, sum, O columns) combined through LDS in wave order.
// A lane owns the same two float4 column groups as in mla_merge_kernel.
template <bool F16>
__global__ void __launch_bounds__(kThreads) mla_merge_wide_kernel(MergeArgs m) {
  static_assert(kThreads / kMergeHeads == 64, "one wave per column set");
  constexpr int W = kThreads / 64;
  __shared__ f32x4 sacc[W][kMergeU][64];
  __shared__ float smx[W], ssum[W];
  const int b = blockIdx.x, head = blockIdx.y;
  int first, nsplit;
  merge_pieces(m, b, first, nsplit);
  if (nsplit <= 1) return;  // (uniform over the workgroup, before its barrier)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = (nsplit + W - 1) / W;
  const int s_begin = min(nsplit, w * per), s_end = min(nsplit, s_begin + per);
  f32x4 acc[kMergeU];
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) acc[u] = f32x4{};
  float mx = -INFINITY, wsum = 0.0f;
  merge_run<F16>(m, b, first, head, 4 * lane, s_begin, s_end, acc, mx, wsum);
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) sacc[w][u][lane] = acc[u];
  if (lane == 0) {
    smx[w] = mx;
    ssum[w] = wsum;
  }
  __syncthreads();
  if (w != 0) return;
  float cm = -INFINITY;
#pragma unroll
  for (int v = 0; v < W; ++v) cm = fmaxf(cm, smx[v]);
  f32x4 o[kMergeU];
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) o[u] = f32x4{};
  float tot = 0.0f;
#pragma unroll
  for (int v = 0; v < W; ++v) {
    // a wave without pieces (or with only empty ones) has max -inf, sum 0
    const float r = smx[v] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(smx[v] - cm);
    tot += r * ssum[v];
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) o[u] += r * sacc[v][u][lane];
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  bf16x4* dst = (bf16x4*)((__bf16*)m.out + ((size_t)b * m.heads + head) * kDV) + lane;
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) dst[u * 64] = __builtin_convertvector(o[u] * inv, bf16x4);
  if (lane == 0) m.lse[(size_t)b * m.heads + head] = tot > 0.0f ? (cm + __builtin_amdgcn_logf(tot)) * kLn2 : -INFINITY;
}

int nsplit_for_heads(int heads) { return heads > 32 ? 2 : 4; }
int heads_per_slab(int heads) { return 32 * (kWaves / nsplit_for_heads(heads)); }
int slabs_for_heads(int heads) { return (heads + heads_per_slab(heads) - 1) / heads_per_slab(heads); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__global__ void mla_zero_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

// Sequences and query rows per sequence that the kernels see: T query tokens
// of a dense decode are T*H rows over one sequence's KV (the KV is read once
// for all of them); top-k lists are per query token, so each token is its own
// sequence of H rows.
void effective_dims(int32_t batch, int32_t heads, int32_t topk, int32_t tq, int32_t* eb, int32_t* eh) {
  *eb = topk > 0 ? batch * tq : batch;
  *eh = topk > 0 ? heads : heads * tq;
}

int32_t decode_ranges(int32_t cus, int32_t batch, int32_t max_pages, int32_t topk, int32_t heads) {
  const int64_t units = (int64_t)batch * (topk > 0 ? (topk + kPage - 1) / kPage : max_pages);
  int64_t r = cus / slabs_for_heads(heads);
  if (r > units) r = units;
  if (r < 1) r = 1;
  return (int32_t)r;
}


// Workspace: [B] int2 piece records | [slots][H] fp32 LSE | [slots][H][512] fp32 O, with
// slots = decode_partial_slots(ranges, B) (piece_slot gives a piece's slot).
size_t decode_workspace_bytes(int32_t ranges, int32_t batch, int32_t heads, int32_t topk) {
  const size_t slots = (size_t)decode_partial_slots(ranges, batch);
  size_t n = align256(sizeof(int2) * (size_t)batch) + align256(sizeof(float) * slots * heads) +
             align256(sizeof(float) * slots * heads * kDV);
  (void)topk;
  return n;
}

// Every decode call rewrites all the state it reads back, so a workspace
// needs no preparation; this clears the piece records so that a workspace
// never holds stale ones.
hipError_t init_decode_workspace(void* workspace, int32_t batch, int32_t heads, hipStream_t stream) {
  (void)heads;
  const int n = 2 * batch;
  hipLaunchKernelGGL(mla_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, (int*)workspace, n);
  return hipGetLastError();
}

// The split-reduction kernel of this file, for every layout the
// wave-specialised kernel does not take.
static hipError_t launch_decode_tiled(const DecodeArgs& a, const DecodeLaunch& d, int kvm, bool causal, hipStream_t stream) {
  const dim3 grid(a.per_xcd * 8 * a.slabs), block(kThreads);
  const int ns = nsplit_for_heads(d.heads);
  // one instantiation per (split, query format, cache layout)
#define MLA_LAUNCH(NS, QF, KVM, C)                                                           \
  if (ns == NS && d.q_fp8 == QF && kvm == KVM && causal == C)                               \
    hipLaunchKernelGGL((mla_decode_kernel<NS, QF, KVM, C>), grid, block, 0, stream, a);
#define MLA_LAUNCH_KV(NS, QF)            \
  MLA_LAUNCH(NS, QF, kKvBf16, false)     \
  MLA_LAUNCH(NS, QF, kKvFp8, false)      \
  MLA_LAUNCH(NS, QF, kKvFp8TopK, false)  \
  MLA_LAUNCH(NS, QF, kKvBf16TopK, false) \
  MLA_LAUNCH(NS, QF, kKvFp8T, false)     \
  MLA_LAUNCH(NS, QF, kKvFp8TTopK, false) \
  MLA_LAUNCH(NS, QF, kKvBf16, true)      \
  MLA_LAUNCH(NS, QF, kKvFp8, true)       \
  MLA_LAUNCH(NS, QF, kKvFp8T, true)
  MLA_LAUNCH_KV(2, false)
  MLA_LAUNCH_KV(2, true)
  MLA_LAUNCH_KV(4, false)
  MLA_LAUNCH_KV(4, true)
#undef MLA_LAUNCH_KV
#undef MLA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch& din, hipStream_t stream) {
  // the kernels see the effective batch and rows (d.heads: rows per sequence)
  DecodeLaunch d = din;
  effective_dims(din.batch, din.heads, din.topk, din.tq, &d.batch, &d.heads);
  const bool causal = din.tq > 1 && din.topk == 0;
  DecodeArgs a;
  a.q = d.q;
  a.kv = (const char*)d.kv;
  a.block_table = d.block_table;
  a.seqlens = d.seqlens;
  a.topk_idx = d.topk_idx;
  a.kv_scales = d.kv_scales;
  a.out = d.out;
  a.lse = d.lse;
  a.slabs = slabs_for_heads(d.heads);
  char* ws = (char*)d.workspace;
  const size_t slots = (size_t)decode_partial_slots(d.ranges, d.batch);
  a.compact = (int64_t)d.ranges + d.batch > 2 * (int64_t)d.ranges ? 1 : 0;
  a.ws_seq = (int2*)ws;
  ws += align256(sizeof(int2) * (size_t)d.batch);
  a.ws_lse = (float*)ws;
  ws += align256(sizeof(float) * slots * d.heads);
  a.ws_o = (float*)ws;
  // the fp16 partials and their factors share the fp32 partials' region:
  // 2 + 16/512 of its 4 bytes per value
  a.ws_o16 = (_Float16*)ws;
  a.ws_sc = (float*)(ws + align256(sizeof(_Float16) * slots * d.heads * kDV));
  ws += align256(sizeof(float) * slots * d.heads * kDV);
  a.topk_tq = din.topk > 0 ? din.tq : 1;
  a.batch = d.batch;
  a.heads = d.heads;
  a.num_pages = d.num_pages;
  a.max_pages = d.max_pages;
  a.topk = d.topk;
  a.tq = causal ? din.tq : 1;
  a.heads_tok = din.heads;
  a.ranges = d.ranges;
  a.seg_pad = 0;
  a.per_xcd = (d.ranges + 7) / 8;
  a.scale_log2 = d.softmax_scale * kLog2e;
  a.q_descale = d.q_descale;

  const int kvm = d.kv_format == kKvFormatFp8Tile     ? (d.topk > 0 ? kKvFp8TopK : kKvFp8)
                  : d.kv_format == kKvFormatFp8Tensor ? (d.topk > 0 ? kKvFp8TTopK : kKvFp8T)
                                                      : (d.topk > 0 ? kKvBf16TopK : kKvBf16);
  hipError_t e;
  const bool ws_kernel = decode_ws_supported(d.kv_format, d.topk, d.heads, d.num_pages);
  if (ws_kernel) {
    // dense bf16 pages with at least 64 rows per sequence: the wave-specialised
    // kernel (decode_ws.hip), the same plan, slabs of 64 rows and workspace
    a.seg_pad = kWsSegPad;
    e = launch_decode_ws(a, d.kv_format, d.q_fp8, causal, stream);
  } else {
    e = launch_decode_tiled(a, d, kvm, causal, stream);
  }
  if (e != hipSuccess) return e;
  MergeArgs m;
  m.seq = a.ws_seq;
  m.ws_o = a.ws_o;
  m.ws_o16 = a.ws_o16;
  m.ws_sc = a.ws_sc;
  m.ws_lse = a.ws_lse;
  m.out = d.out;
  m.lse = d.lse;
  m.heads = d.heads;
  m.compact = a.compact;
  m.topk_units = d.topk > 0 ? (d.topk + kPage - 1) / kPage : 0;
  m.batch = d.batch;
  m.ranges = d.ranges;
  m.seg_pad = a.seg_pad;
  // many pieces per sequence (eight or more ranges per sequence on average)
  // or a grid of under 256 workgroups: a workgroup per (sequence, head),
  // the pieces split over its waves
  const int64_t narrow_wgs = (int64_t)d.batch * ((d.heads + kMergeHeads - 1) / kMergeHeads);
  const bool wide = d.ranges >= 8 * (int64_t)d.batch || narrow_wgs < 256;
  const dim3 mgrid(d.batch, wide ? d.heads : (d.heads + kMergeHeads - 1) / kMergeHeads);
  if (wide) {
    if (ws_kernel) hipLaunchKernelGGL(mla_merge_wide_kernel<true>, mgrid, dim3(kThreads), 0, stream, m);
    else hipLaunchKernelGGL(mla_merge_wide_kernel<false>, mgrid, dim3(kThreads), 0, stream, m);
  } else {
    if (ws_kernel) hipLaunchKernelGGL(mla_merge_kernel<true>, mgrid, dim3(kThreads), 0, stream, m);
    else hipLaunchKernelGGL(mla_merge_kernel<false>, mgrid, dim3(kThreads), 0, stream, m);
  }
  return hipGetLastError();
}

}  // namespace mla
