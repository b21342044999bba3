// decode_ws.hip - the wave-specialised absorbed MLA decode for gfx950
// (MI355X): paged bf16 caches, 64 query rows per workgroup.
//
// What is computed is the same as in decode.hip: for every query row (head)
// of a sequence, scores against the shared 576-wide latent rows, a scaled
// softmax per row, O = P.V with V the 512 latent columns, and the
// natural-log LSE.
//
// Design.  A workgroup of eight waves, two per SIMD, holds one slab of 64
// query rows of one sequence (the STAGE_D2 note's head-packed tile, "Strategy
// A: Head-Packed M Dimension": every KV row is read once for all 64).  Waves
// w and w+4 share a SIMD and have different jobs, so that one issues matrix
// instructions while the other waits for LDS or runs its softmax:
//  * score waves (0..3): wave q takes rows 32*(q&1) .. +31 and the token half
//    (q>>1) of every 32-token slot, over the whole 576-wide reduction
//    (v_mfma_f32_16x16x32_bf16: tokens on M, rows on N, the queries of its 32
//    rows in 144 VGPRs).  With the full reduction in one wave no partial
//    scores cross LDS; the wave forms its own exponentials and writes them as
//    bf16 into a P tile in LDS.
//  * value waves (4..7): wave 4+v owns output columns 128v .. +127 of all 64
//    rows and forms O^T = V^T P^T (v_mfma_f32_32x32x16_bf16: columns on M,
//    rows on N, 128 fp32 accumulators, so that a lane ends up holding runs of
//    four consecutive columns of one row, stored 16 bytes at a time), reading
//    P from the tile and V through transposing LDS reads; each V fragment
//    serves both 32-row blocks.  They also issue the direct global->LDS
//    copies of the KV slots.
// One workgroup barrier per slot.  Between barriers B_i and B_i+1 the score
// waves work on slot i, while the value waves multiply slot i-1 (its P was
// written before B_i, its V fragments read into registers during i-1) and
// copy slot i+3 into the ring position of slot i-1, which nobody reads after
// B_i.  The ring holds four
// 36 KB slots (three in flight); the P tile is double-buffered.
// The two roles run their own copies of the segment and slot loops with the
// same barrier sequence: the score waves' queries and the value waves'
// accumulators are then never live in the same code, and each role fits the
// 256 registers of a wave at two waves per SIMD.
//
// Softmax: base 2 against a fixed reference per row, the maximum of the
// segment's first slot (the two token halves exchange their maxima once, in
// LDS).  Later slots may rise above it by up to 16 (p <= 2^16, exact in fp32,
// a relative rounding in bf16); if a row rises further the workgroup redoes
// the segment with the true maxima.  O is never rescaled.
//
// Split-KV: the same plan as decode.hip (units of all sequences laid end to
// end, cut into equal ranges); a piece of a split sequence writes its
// normalised partial and base-2 LSE to the workspace for mla_merge_kernel.
#include "decode_common.h"

#include <type_traits>

namespace mla {
namespace {

constexpr int kWsWaves = 8;
constexpr int kWsThreads = 64 * kWsWaves;
constexpr int kWsRows = 64;       // query rows per workgroup
constexpr int kQk = kD / 32;      // 18 k-steps of 32 in the 576-wide reduction
constexpr int kPRowBytes = 80;    // a row of the P tile: 32 bf16 + 16 bytes of pad
constexpr int kPTile = kWsRows * kPRowBytes;
constexpr int kKRead = 4;         // K fragments in flight ahead of their MFMA

// Cache layouts of this kernel.  The e4m3 rows stay codes in the ring (the
// same direct copies, 128-byte column groups of 32 rows, the same swizzle)
// and become bf16 as the MFMA fragments are read: K rows with plain 8-byte
// reads, V^T with the 8-bit transposing read.
constexpr int kFmtBf16 = 0;  // [P,64,576] bf16
constexpr int kFmtFp8 = 1;   // [P,64,640]: 512 codes + 64 bf16 rope; fp32 scales [P,64,4], one per 128 columns
constexpr int kFmtFp8T = 2;  // [P,64,576] codes; one per-tensor k_scale_inv
template <int F>
struct WsFmt;
template <>
struct WsFmt<kFmtBf16> {
  static constexpr int kRow = kRowBytes;    // bytes per cache row
  static constexpr int kSlot = kSlotBytes;  // ring slot: nine column groups
  static constexpr int kOps = kDmaPerWave;  // copies per value wave and slot
  static constexpr int kPTiles = 1;         // P tiles per slot
};
template <>
struct WsFmt<kFmtFp8> {
  static constexpr int kRow = kFp8RowBytes;
  static constexpr int kScaleOff = 5 * kGroupBytes;     // four codes groups, the rope group, then scales
  static constexpr int kSlot = kScaleOff + 4 * 1024;    // each value wave copies the 32 rows' scales
  static constexpr int kOps = 6;
  static constexpr int kPTiles = 4;                     // P scaled by each column tile's scale
};
template <>
struct WsFmt<kFmtFp8T> {
  static constexpr int kRow = kFp8TRowBytes;
  static constexpr int kSlot = 5 * kGroupBytes;  // four codes groups, half a group of rope codes
  static constexpr int kOps = 5;
  static constexpr int kPTiles = 1;
};

// s_waitcnt vmcnt(N) alone (LDS reads stay in flight), GFX9 encoding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// vm operations of copy epoch e of an n-slot segment, per value wave: the
// N copies of slot e+3
template <int N>
__device__ __forceinline__ int epoch_ops(int e, int n) { return e + 3 < n ? N : 0; }

// s_waitcnt vmcnt(k) lgkmcnt(0) for the counts epoch_ops can add up to
// (anything else waits for everything, which is always safe)
template <int N>
__device__ __forceinline__ void wait_ops_lgkm0(int k) {
  if (k == 2 * N) wait_vm_lgkm0<2 * N>();
  else if (k == N) wait_vm_lgkm0<N>();
  else wait_vm_lgkm0<0>();
}
// the same with x (2 or 4) more operations allowed in flight: the top-k
// staging loads of one or two epochs
template <int N>
__device__ __forceinline__ void wait_ops_lgkm0(int k, int x) {
  if (x == 4) {
    if (k == 2 * N) wait_vm_lgkm0<2 * N + 4>();
    else if (k == N) wait_vm_lgkm0<N + 4>();
    else wait_vm_lgkm0<4>();
  } else {
    if (k == 2 * N) wait_vm_lgkm0<2 * N + 2>();
    else if (k == N) wait_vm_lgkm0<N + 2>();
    else wait_vm_lgkm0<2>();
  }
}

// One direct global->LDS copy of 4 bytes per lane (lane i's word lands at
// lds_base + 4i), issued and accounted like the 16-byte copies.
// (m0 is named in the clobber list on purpose: clang warns that it is reserved)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const char* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// 8 e4m3 codes as bf16 (exact: every e4m3 value is a bf16 value)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 codes_bf16(u32x2 c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false);
  const bf16x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true);
  const bf16x2 x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false);
  const bf16x2 x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true);
  return bf16x8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

// The copy offsets of a cache with rows of ROW bytes: lane i of copy rb
// writes row 8rb + i/8, position i%8 of a column group and so fetches
// source chunk (i%8) ^ row_swz(row) (of at most CHUNKS chunks: beyond, the
// last one again; rows at and beyond row_cap read row row_cap).
template <int ROW, int CHUNKS>
__device__ __forceinline__ uint32_t dma_lane_off_fmt(int lane, int rb, int row_cap) {
  int row = 8 * rb + (lane >> 3);
  int src_chunk = (lane & 7) ^ row_swz(row);
  if constexpr (CHUNKS < 8) src_chunk = min(src_chunk, CHUNKS - 1);
  row = row < row_cap ? row : row_cap;
  return (uint32_t)(row * ROW + 16 * src_chunk);
}

// The P tile: [row][position] bf16, 80-byte rows (the 16-byte reads of 16
// consecutive rows then hit 16 distinct bank groups).  Position p of a
// 16-token k-step holds token pi(p), pi swapping bits 2 and 3: the order in
// which the transposing V reads hand a lane its eight tokens (lane half h:
// tokens 4h .. 4h+3, then 8+4h .. 8+4h+3).  pi is its own inverse.

// LDS address (slot-relative) of the K fragment of token half th for an
// even (odd = 0) or odd k-step: row m = 16th + (lane & 15), 16-byte chunk
// 4*odd + lane/16 of the k-step pair's column group, in the swizzled layout;
// k-step g adds g/2 column groups.
__device__ __forceinline__ uint32_t ws_kaddr(int th, int lane, int odd) {
  const int m = 16 * th + (lane & 15);
  const int c = 4 * odd + (lane >> 4);
  return m * 128 + 16 * (c ^ row_swz(m));
}

// LDS address (slot-relative) of the 8 codes a lane reads for k-step i
// (0..3) of a 128-column group: row m = 16th + (lane & 15), columns 32i +
// 8(lane/16) .. +7, i.e. chunk 2i + lane/32 of the group, half lane/16 % 2.
__device__ __forceinline__ uint32_t ws_kaddr8(int th, int lane, int i) {
  const int m = 16 * th + (lane & 15), g4 = lane >> 4;
  return m * 128 + 16 * ((2 * i + (g4 >> 1)) ^ row_swz(m)) + 8 * (g4 & 1);
}

// 8-bit transposing V^T reads of value wave v (column group v): for k-step
// ks the eight lane pairs of each 16-lane group G supply rows 16ks + 8(G>>1)
// .. +7 (pair 2k, 2k+1: row k, bytes 16(G&1) + 8(lane&1) of the 32-column
// block), and lane l receives column l%32 of those eight tokens in natural
// order.  Column block cb only flips address bits 5 and 6 (the chunk bits
// above the half-block bit): address = vaddr8 ^ 32cb.
__device__ __forceinline__ uint32_t ws_vaddr8(int v, int lane, int ks) {
  const int m = 16 * ks + 8 * (lane >> 5) + ((lane & 15) >> 1);
  const int swz = row_swz(m), g1 = (lane >> 4) & 1;
  return kGroupBytes * v + m * 128 + 32 * ((swz >> 1) & 3) + 16 * (g1 ^ (swz & 1)) + 8 * (lane & 1);
}

// Transposing V reads of value wave v: for column block cb (columns
// 128v + 32cb .. +31) and k-step ks (slot tokens 16ks .. +15) the two reads
// give lane l column 128v + 32cb + l%32 of tokens pi(8h + e), h = l/32.
// Within 16-lane group G lane 4j + q reads columns 16(G&1) + 4q .. +3 of row
// 4(G>>1) + j (tt = 0) and of row 8 + 4(G>>1) + j (tt = 1).
__device__ __forceinline__ uint32_t ws_vaddr(int v, int lane, int tt) {
  const int G = lane >> 4, i = lane & 15, j = i >> 2, q = i & 3;
  const int m = 8 * tt + 4 * (G >> 1) + j;
  return kGroupBytes * (2 * v) + m * 128 + 16 * ((2 * (G & 1) + (q >> 1)) ^ row_swz(m)) + 8 * (q & 1);
}

typedef bf16x4 VFrag[4];  // [2 * ks + tt]

__device__ __forceinline__ void ws_vload(const lds_char* buf, const uint32_t (&va)[2], int cb, VFrag& f) {
  const uint32_t x = (cb & 1) ? 64u : 0u;  // odd 32-column block: chunk bit 2
  const lds_char* p0 = buf + (va[0] ^ x) + kGroupBytes * (cb >> 1);
  const lds_char* p1 = buf + (va[1] ^ x) + kGroupBytes * (cb >> 1);
  f[0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p0);
  f[1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p1);
  f[2] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p0 + 16 * 128));
  f[3] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p1 + 16 * 128));
}

// max / sum over lanes l, l^16, l^32, l^48: the four token groups of one row
// in a 16x16 score fragment
__device__ __forceinline__ float max_rows4(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_rows4(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Score wave, QK^T of one slot: S^T[16 tokens][32 rows] as two 16x16
// fragments; lane l, register e: token 4(l/16) + e of the wave's half, row
// 16j + l%16 of its block.
__device__ __forceinline__ void ws_scores(const lds_char* buf, const uint32_t (&ka)[2], const bf16x8 (&qf)[kQk][2],
                                          f32x4 (&s)[2]) {
  bf16x8 kb[kKRead];
#pragma unroll
  for (int g = 0; g < kKRead - 1; ++g) kb[g] = *(const LDS_AS bf16x8*)(buf + ka[g & 1] + kGroupBytes * (g >> 1));
#pragma unroll
  for (int g = 0; g < kQk; ++g) {
    constexpr int A = kKRead - 1;
    // (a scheduling fence per k-step keeps each read kKRead - 1 steps ahead
    // of its MFMAs instead of letting the scheduler sink it next to them)
    __builtin_amdgcn_sched_barrier(0);
    if (g + A < kQk) kb[(g + A) % kKRead] = *(const LDS_AS bf16x8*)(buf + ka[(g + A) & 1] + kGroupBytes * ((g + A) >> 1));
    s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[g % kKRead], qf[g][0], g == 0 ? f32x4{} : s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[g % kKRead], qf[g][1], g == 0 ? f32x4{} : s[1], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Score wave, QK^T of one slot of e4m3 codes: S^T[16 tokens][32 rows], each
// code fragment converted to bf16 as it is read.  Per-tile scales (F =
// kFmtFp8): each 128-column tile sums into an accumulator of its own and is
// added with the token's tile scale (sc[e][t]: token e of the lane, tile t);
// the bf16 rope adds unscaled.  Per-tensor codes: one accumulation, the
// scale applies outside.
template <int F>
__device__ __forceinline__ void ws_scores8(const lds_char* buf, const uint32_t (&ka)[4], const uint32_t (&kr)[2],
                                           const bf16x8 (&qf)[kQk][2], const f32x4 (&sc)[4], f32x4 (&s)[2]) {
  if constexpr (F == kFmtFp8) {
    // rope first (bf16 as stored, group 4)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const bf16x8 kb = *(const LDS_AS bf16x8*)(buf + kr[g]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qf[16 + g][j], g == 0 ? f32x4{} : s[j], 0, 0, 0);
    }
    u32x2 raw[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[0][i] = *(const LDS_AS u32x2*)(buf + ka[i]);
    // tile t's dot products go to tt[t & 1]; their scaled sum into s waits
    // until tile t+1's MFMAs are issued, so the matrix core does not drain
    // between tiles
    f32x4 tt[2][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t + 1 < 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[(t + 1) & 1][i] = *(const LDS_AS u32x2*)(buf + ka[i] + kGroupBytes * (t + 1));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 kb = codes_bf16(raw[t & 1][i]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          tt[t & 1][j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qf[4 * t + i][j], i == 0 ? f32x4{} : tt[t & 1][j], 0, 0, 0);
      }
      if (t > 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[j][e] = __builtin_fmaf(sc[e][t - 1], tt[(t - 1) & 1][j][e], s[j][e]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[j][e] = __builtin_fmaf(sc[e][3], tt[1][j][e], s[j][e]);
  } else {
    u32x2 raw[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[0][i] = *(const LDS_AS u32x2*)(buf + ka[i]);
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      // groups 0..3: codes of the 512 latent columns; group 4: the 64 rope codes
      const int nk = t < 4 ? 4 : 2;
      if (t + 1 < 5) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t + 1 < 4 || i < 2) raw[(t + 1) & 1][i] = *(const LDS_AS u32x2*)(buf + ka[i] + kGroupBytes * (t + 1));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nk) break;
        const bf16x8 kb = codes_bf16(raw[t & 1][i]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qf[4 * t + i][j], t == 0 && i == 0 ? f32x4{} : s[j], 0, 0,
                                                         0);
      }
    }
  }
}

// LDS shared by the two roles.
struct WsLds {
  lds_char* ring;    // KV ring, kRing slots
  lds_char* ptile;   // two P tiles
  LDS_AS float* xref;  // [half][row]: first-slot maxima
  LDS_AS float* xl;    // [half][row]: sums of p
  LDS_AS float* xm;    // [half][row]: largest scores seen (base 2)
  LDS_AS int* votes;   // [score wave]: redo votes
  LDS_AS uint32_t* tkmask;  // top-k: [ring position] validity of the slot's 32 entries
  LDS_AS int32_t* tk;       // top-k: per value wave, entries [8][64] then their pages [8][64]
};

constexpr int kTkWords = 8 * 64 + 8 * 64;  // top-k staging words per value wave

// A wave-uniform load of table data that no kernel writes (sequence
// lengths): through the scalar cache rather than the vector memory pipeline,
// where it would queue behind the workgroup's copies and query loads.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// One segment of the range: sequence b, tokens [tok0, tok1).
struct WsSeg {
  int b;
  SegCtx sg;
  int seglen;
  int first_r, nsplit;
};

// Calls body(seg) for every segment of the range, in order, with a barrier
// between segments (every wave is done with the ring and the exchanges).
template <bool TOPK, class F>
__device__ __forceinline__ void for_segments(const DecodeArgs& a, const Plan& pl, F&& body) {
  // p: line position of sequence b; its pages are units [p + pad, p + pad + n)
  const int pad = pl.pad;
  int b = pl.b0, p = pl.p0;
  bool first = true;
  while (true) {
    // dense: a sequence's units are its pages; top-k: a list's 64-entry chunks
    const int seglen = TOPK ? a.topk : min(max(ld_uniform(a.seqlens + b), 0), a.max_pages * kPage);
    const int n = (seglen + kPage - 1) / kPage;
    const int q = p + pad;
    const int gs = max(pl.start, q), ge = min(pl.end, q + n);
    if (gs < ge) {
      if (!first) {
        wait_vm_lgkm0<0>();
        barrier();
      }
      first = false;
      WsSeg s;
      s.b = b;
      s.seglen = seglen;
      s.sg.tok0 = (gs - q) * kPage;
      s.sg.tok1 = min((ge - q) * kPage, s.seglen);
      s.sg.nslots = (s.sg.tok1 - s.sg.tok0 + kTS - 1) / kTS;
      s.sg.npages = (s.sg.nslots + 1) / 2;
      s.sg.bt_seg = a.block_table + (size_t)b * a.max_pages + (gs - q);
      s.sg.idx_seg = TOPK ? a.topk_idx + (size_t)b * a.topk + s.sg.tok0 : nullptr;
      s.first_r = q / pl.C;
      s.nsplit = (q + n - 1) / pl.C - s.first_r + 1;
      body(s);
    }
    p += n > 0 ? n + 2 * pad : 0;
    ++b;
    if (p >= pl.end || b >= a.batch) break;
  }
}

// ---------------------------------------------------------------- score waves

template <int F, bool Q_FP8, bool CAUSAL, bool TOPK>
__device__ __forceinline__ void score_role(const DecodeArgs& a, const Plan& pl, const WsLds& L, int w, int lane,
                                           int row0, int r) {
  // (lane and wave pass through empty asm statements: nothing computed from
  // them can be hoisted above the role split, where it would stay live in the
  // other role's code too)
  asm volatile("" : "+v"(lane), "+s"(w));
  const int hb = w & 1, th = w >> 1;
  const int i16 = lane & 15, g4 = lane >> 4;
  // per-tensor codes: value = code / k_scale_inv, folded into the score scale
  const float scale_log2 = F == kFmtFp8T ? a.scale_log2 * (1.0f / a.kv_scales[0]) : a.scale_log2;
  int qrow[2], lag[2] = {0, 0};
  bool qok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    qrow[j] = row0 + 32 * hb + 16 * j + i16;
    qok[j] = qrow[j] < a.heads;
    if constexpr (CAUSAL) lag[j] = a.tq - 1 - min(qrow[j], a.heads - 1) / a.heads_tok;
  }
  const uint32_t ka[2] = {ws_kaddr(th, lane, 0), ws_kaddr(th, lane, 1)};
  uint32_t ka8[4], kr8[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) ka8[i] = ws_kaddr8(th, lane, i);
  // rope of the tile format: bf16 in group 4, read as the bf16 cache's
  // column groups are
#pragma unroll
  for (int i = 0; i < 2; ++i) kr8[i] = 4 * kGroupBytes + ws_kaddr(th, lane, i);
  // this lane's four p of block j: row 32hb + 16j + i16 of the P tile,
  // positions 16th + 4*pi-group(lane / 16) .. +3 (bf16 cache: the order of
  // the 16-bit transposing V reads) or 16th + 4(lane/16) .. +3 (codes: the
  // 8-bit transposing reads keep the natural order)
  const int g4p = F == kFmtBf16 ? ((g4 & 1) << 1) | (g4 >> 1) : g4;
  uint32_t pw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) pw[j] = (32 * hb + 16 * j + i16) * kPRowBytes + (16 * th + 4 * g4p) * 2;
  const int xrow = 32 * hb + i16;  // + 16j: this lane's rows in the exchange arrays

  for_segments<TOPK>(a, pl, [&](const WsSeg& sgm) {
    const int b = sgm.b;
    const int nslots = sgm.sg.nslots;
    int lim[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) lim[j] = CAUSAL ? min(sgm.sg.tok1, sgm.seglen - lag[j]) : sgm.sg.tok1;
    const int lim_lo = min(lim[0], lim[1]);

    // queries (B operand): row qrow[j], columns 32k + 8(lane/16) .. +7.
    // Dense pages: after barrier X, so that they queue behind the value
    // waves' copies of slot 0.  Top-k lists (bf16 queries): before it, where
    // they load while the value waves wait for the list entries and their
    // pages, two round trips before any copy can be issued.
    bf16x8 qf[kQk][2];
    constexpr bool kEarlyQ = TOPK && !Q_FP8;
    if constexpr (!kEarlyQ) barrier();  // X
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rr = qok[j] ? qrow[j] : 0;
      if constexpr (!Q_FP8) {
        const bf16x8* qp = (const bf16x8*)((const __bf16*)a.q + ((size_t)b * a.heads + rr) * kD);
        // (rows past the heads read row 0: finite scores for rows that are
        // never stored, and no use of the loaded data before barrier Y)
#pragma unroll
        for (int k = 0; k < kQk; ++k) qf[k][j] = qp[4 * k + g4];
      } else {
        const uint2* qp = (const uint2*)((const uint8_t*)a.q + ((size_t)b * a.heads + rr) * kD);
#pragma unroll
        for (int k = 0; k < kQk; ++k) {
          const uint2 x = qp[4 * k + g4];
          qf[k][j] = qok[j] ? fp8x8_to_bf16(x, a.q_descale) : bf16x8{};
        }
      }
    }
    if constexpr (kEarlyQ) barrier();  // X
    barrier();  // Y: the query loads are issued; the value waves copy slots 1 and 2 behind them
    wait_vm_lgkm0<0>();

    float ref[2] = {-INFINITY, -INFINITY};  // base-2 reference per row
    for (int pass = 0; pass < 2; ++pass) {
      float lsum[2] = {0.0f, 0.0f};
      float mraw[2] = {-INFINITY, -INFINITY};  // largest raw score seen
      barrier();  // B_0: slot 0 landed
      for (int it = 0; it <= nslots; ++it) {
        if (it < nslots) {
          const lds_char* buf = L.ring + (it & (kRing - 1)) * WsFmt<F>::kSlot;
          f32x4 s[2];
          f32x4 sc[4];  // tile format: tile scales of this lane's tokens 16th + 4(lane/16) + e
          if constexpr (F == kFmtFp8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[e] = *(const LDS_AS f32x4*)(buf + WsFmt<F>::kScaleOff + 16 * (16 * th + 4 * g4 + e));
          }
          // the score MFMAs go first on the SIMD's matrix core; the value
          // wave's MFMAs then fill the time of this wave's softmax
          __builtin_amdgcn_s_setprio(1);
          if constexpr (F == kFmtBf16) ws_scores(buf, ka, qf, s);
          else ws_scores8<F>(buf, ka8, kr8, qf, sc, s);
          __builtin_amdgcn_s_setprio(0);
          if constexpr (TOPK) {
            // list entries that are padding, negative or past the token's
            // limit: the validity word the value waves wrote with the copies
            const uint32_t vm = L.tkmask[it & (kRing - 1)] >> (16 * th + 4 * g4);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) s[j][e] = (vm >> e) & 1u ? s[j][e] : -INFINITY;
          }
          const int tk = sgm.sg.tok0 + it * kTS + 16 * th + 4 * g4;  // this lane's first token
          if (sgm.sg.tok0 + it * kTS + kTS > lim_lo) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) s[j][e] = tk + e < lim[j] ? s[j][e] : -INFINITY;
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) mraw[j] = fmaxf(mraw[j], fmaxf(fmaxf(s[j][0], s[j][1]), fmaxf(s[j][2], s[j][3])));
          if (pass == 0 && it == 0) {
            // the first slot fixes the reference: the max over both token halves
            float mx[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) mx[j] = max_rows4(mraw[j]);
            if (g4 == 0) {
#pragma unroll
              for (int j = 0; j < 2; ++j) L.xref[th * 64 + xrow + 16 * j] = mx[j];
            }
            wait_vm_lgkm0<0>();
            barrier();
#pragma unroll
            for (int j = 0; j < 2; ++j) ref[j] = fmaxf(mx[j], L.xref[(th ^ 1) * 64 + xrow + 16 * j]) * scale_log2;
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float nref = neg_ref(ref[j]);
            f32x4 pj;
#pragma unroll
            for (int e = 0; e < 4; ++e) pj[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][e], scale_log2, nref));
            lsum[j] += (pj[0] + pj[1]) + (pj[2] + pj[3]);
            lds_char* pt = L.ptile + (it & 1) * WsFmt<F>::kPTiles * kPTile + pw[j];
            if constexpr (F == kFmtFp8) {
              // one P tile per column tile, p times the token's tile scale
              // rounded once to bf16: the codes then serve as that tile's V
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                f32x4 pt4;
#pragma unroll
                for (int e = 0; e < 4; ++e) pt4[e] = pj[e] * sc[e][t];
                *(LDS_AS bf16x4*)(pt + t * kPTile) = __builtin_convertvector(pt4, bf16x4);
              }
            } else {
              *(LDS_AS bf16x4*)pt = __builtin_convertvector(pj, bf16x4);
            }
          }
          wait_vm_lgkm0<0>();
        }
        barrier();  // B_it+1
      }
      // end of the pass: row sums, largest scores, redo vote
      bool up = false;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float l = sum_rows4(lsum[j]);
        const float m = max_rows4(mraw[j]);
        const float ms = m == -INFINITY ? -INFINITY : m * scale_log2;
        up |= ms > ref[j] + kTau;
        if (g4 == 0) {
          L.xl[th * 64 + xrow + 16 * j] = l;
          L.xm[th * 64 + xrow + 16 * j] = ms;
        }
      }
      const bool vote = __any(up);
      if (lane == 0) L.votes[w] = vote ? 1 : 0;
      wait_vm_lgkm0<0>();
      barrier();
      const int votes = L.votes[0] | L.votes[1] | L.votes[2] | L.votes[3];
      if (__builtin_amdgcn_readfirstlane(votes) == 0) {
        // LSE of rows 32hb + 16j + i16 (token half 0 writes it)
        if (th == 0 && g4 == 0) {
          const size_t pslot = piece_slot(a, b, r, sgm.first_r);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int lr = xrow + 16 * j;
            const float lt = L.xl[lr] + L.xl[64 + lr];
            const float lse2 = lt > 0.0f ? ref[j] + __builtin_amdgcn_logf(lt) : -INFINITY;
            if (qok[j]) {
              if (sgm.nsplit == 1) a.lse[(size_t)b * a.heads + qrow[j]] = lse2 * kLn2;
              else a.ws_lse[pslot * a.heads + qrow[j]] = lse2;
            }
          }
        }
        if (w == 0 && lane == 0) a.ws_seq[b] = int2{sgm.first_r, sgm.nsplit};
        break;
      }
      // redo with the true maxima (then p <= 1)
#pragma unroll
      for (int j = 0; j < 2; ++j) ref[j] = fmaxf(L.xm[xrow + 16 * j], L.xm[64 + xrow + 16 * j]);
      wait_vm_lgkm0<0>();
      barrier();  // every wave has read the votes
    }
  });
}

// ---------------------------------------------------------------- value waves

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef u32x2 VFrag8[2];  // [ks]: 8 codes of column lane%32, tokens 16ks + 8(lane/32) .. +7

template <int F, bool TOPK>
__device__ __forceinline__ void value_role(const DecodeArgs& a, const Plan& pl, const WsLds& L, int v, int lane,
                                           int row0, int r) {
  typedef WsFmt<F> Fm;
  constexpr int N = Fm::kOps;
  typedef typename std::conditional<F == kFmtBf16, VFrag, VFrag8>::type VF;
  asm volatile("" : "+v"(lane), "+s"(v));  // (as in score_role)
  const int i32 = lane & 31, h2 = lane >> 5;
  // P fragment (A operand) of row block rb, k-step ks: row 32rb + i32 of the
  // tile, positions 16ks + 8h2 .. +7
  const uint32_t prd = i32 * kPRowBytes + 16 * h2;
  const uint32_t va[2] = {F == kFmtBf16 ? ws_vaddr(v, lane, 0) : ws_vaddr8(v, lane, 0),
                          F == kFmtBf16 ? ws_vaddr(v, lane, 1) : ws_vaddr8(v, lane, 1)};
  // P tile of this wave (tile format: the one scaled for its column tile v)
  const uint32_t ptv = F == kFmtFp8 ? v * kPTile : 0;
  // copies: this wave takes the column groups it multiplies (bf16: 2v and
  // 2v+1; codes: v) of all 32 rows and rows 8v .. 8v+7 of the rope group
  // (bf16: group 8; codes: group 4; the per-tensor rope codes fill half of
  // it), plus, for the tile format, a copy of the 32 rows' scales
  constexpr int kChunks = F == kFmtFp8T ? 4 : 8;  // source chunks of a row in the rope group
  uint32_t dfull[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) dfull[rb] = dma_lane_off_fmt<Fm::kRow, 8>(lane, rb, kTS);
  const uint32_t dfull_r = dma_lane_off_fmt<Fm::kRow, kChunks>(lane, v, kTS);
  // per-tensor codes: value = code / k_scale_inv, applied at the output
  const float kdesc = F == kFmtFp8T ? 1.0f / a.kv_scales[0] : 1.0f;


  // top-k staging of this wave: entries of slot s at [s % 8][64], their
  // block-table entries at [s % 8][64] (lane l: entry 32s + l % 32)
  LDS_AS int32_t* const tk_idx = L.tk + v * kTkWords;
  LDS_AS int32_t* const tk_pg = tk_idx + 8 * 64;

  for_segments<TOPK>(a, pl, [&](const WsSeg& sgm) {
    const int b = sgm.b;
    const SegCtx& sg = sgm.sg;
    const int nslots = sg.nslots;
    PageCache pc;
    if constexpr (!TOPK) page_cache_load(pc, sg.bt_seg, 0, sg.npages, lane);
    // top-k: list b belongs to query token b % T of sequence b / T, which
    // sees positions [0, seqlen - T + 1 + t); entries outside, and padding,
    // are masked and copy a fallback row of the sequence (page 0, row 0)
    int tk_nent = 0, tk_limit = 0, tk_fallback = 0;
    const char* tk_lst = nullptr;
    const char* tk_bt = nullptr;
    if constexpr (TOPK) {
      const int bq = b / a.topk_tq, tq = b - bq * a.topk_tq;
      const int32_t* bt = a.block_table + (size_t)bq * a.max_pages;
      const int seqlen = min(max(ld_uniform(a.seqlens + bq), 0), a.max_pages * kPage);
      tk_limit = seqlen - a.topk_tq + 1 + tq;
      tk_nent = sg.tok1 - sg.tok0;
      tk_fallback = clamp_page(ld_uniform(bt), a.num_pages) * kPage;
      tk_lst = uniform_ptr((const char*)sg.idx_seg);
      tk_bt = uniform_ptr((const char*)bt);
    }
    // entries of slot s (clamped to the segment) into the staging
    auto tk_idx_dma = [&](int s) {
      const uint32_t off = 4u * (uint32_t)min(32 * s + (lane & 31), tk_nent - 1);
      dma4(tk_lst, off, __builtin_amdgcn_readfirstlane(lds_addr((lds_char*)(tk_idx + (s & 7) * 64))));
    };
    // block-table entries of slot s's entries (landed) into the staging
    auto tk_pg_dma = [&](int s) {
      const int idx = tk_idx[(s & 7) * 64 + lane];
      const int p = min(max(idx >> 6, 0), a.max_pages - 1);
      dma4(tk_bt, 4u * (uint32_t)p, __builtin_amdgcn_readfirstlane(lds_addr((lds_char*)(tk_pg + (s & 7) * 64))));
    };
    // cache rows of entries js[0..5] of slot s (their entries and pages
    // landed).  The twelve LDS reads are all issued before any is used: the
    // empty asm takes every loaded value at once, so the compiler neither
    // waits after each read nor sinks the page read into the validity test
    // (a lookup each, one LDS round trip after another).
    auto tk_rows = [&](int s, const int (&js)[6], int (&row)[6], bool (&ok)[6]) {
      int idx[6], pg[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        idx[i] = tk_idx[(s & 7) * 64 + js[i]];
        pg[i] = tk_pg[(s & 7) * 64 + js[i]];
      }
      asm volatile("" : "+v"(idx[0]), "+v"(idx[1]), "+v"(idx[2]), "+v"(idx[3]), "+v"(idx[4]), "+v"(idx[5]),
                        "+v"(pg[0]), "+v"(pg[1]), "+v"(pg[2]), "+v"(pg[3]), "+v"(pg[4]), "+v"(pg[5]));
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        ok[i] = 32 * s + js[i] < tk_nent && idx[i] >= 0 && idx[i] < tk_limit;
        row[i] = ok[i] ? clamp_page(pg[i], a.num_pages) * kPage + (idx[i] & 63) : tk_fallback;
      }
    };
    // this wave's copies of slot s into ring position pos (s < nslots)
    auto dma_cols = [&](int s, int pos) {
      if constexpr (TOPK) {
        // gathered rows: lane i of copy rb fetches row 8rb + i/8 of the slot,
        // position i%8 of the column group, from that entry's cache row.
        // The six lookups go out together before the first copy (the copies
        // are asm statements that no load moves across).
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(L.ring + (pos & (kRing - 1)) * Fm::kSlot));
        const char* kvu = uniform_ptr(a.kv);
        int js[6], row[6];
        bool ok[6];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) js[rb] = 8 * rb + (lane >> 3);
        js[4] = 8 * v + (lane >> 3);  // the rope group: rows 8v .. 8v+7
        js[5] = lane & 31;            // the scales and the validity word: every row
        tk_rows(s, js, row, ok);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const uint32_t off = (uint32_t)row[rb] * Fm::kRow + 128u * v + 16u * ((lane & 7) ^ row_swz(js[rb]));
          dma16<0>(kvu, off, base + v * kGroupBytes + rb * 1024);
        }
        {
          const int c = min((lane & 7) ^ row_swz(js[4]), kChunks - 1);
          dma16<0>(kvu, (uint32_t)row[4] * Fm::kRow + 512u + 16u * c, base + 4 * kGroupBytes + v * 1024);
        }
        {
          if constexpr (F == kFmtFp8)
            dma16<0>(uniform_ptr((const char*)a.kv_scales), 16u * (uint32_t)row[5], base + Fm::kScaleOff + v * 1024);
          const uint64_t vm = __ballot(ok[5]);
          if (v == 0 && lane == 0) L.tkmask[pos & (kRing - 1)] = (uint32_t)vm;
        }
        return;
      }
      const int page = page_of(pc, sg.bt_seg, s >> 1, sg.npages, lane, a.num_pages);
      const size_t row0s = (size_t)page * kPage + (s & 1) * kTS;  // cache row of the slot's token 0
      const char* src = a.kv + row0s * Fm::kRow;
      const int nvalid = min(kTS, sg.tok1 - (sg.tok0 + s * kTS));
      uint32_t off[4], offr;
      if (nvalid >= kTS) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) off[rb] = dfull[rb];
        offr = dfull_r;
      } else {
        // rows at and beyond the valid count re-read the last valid row
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) off[rb] = dma_lane_off_fmt<Fm::kRow, 8>(lane, rb, nvalid - 1);
        offr = dma_lane_off_fmt<Fm::kRow, kChunks>(lane, v, nvalid - 1);
      }
      const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(L.ring + (pos & (kRing - 1)) * Fm::kSlot));
      if constexpr (F == kFmtBf16) {
        const char* s0 = uniform_ptr(src + 256 * v);  // column group 2v
        const char* s8 = uniform_ptr(src + 8 * 128);  // the rope group
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          // (the immediate offset moves the source and the destination alike)
          dma16<0>(s0, off[rb], base + (2 * v) * kGroupBytes + rb * 1024);
          dma16<128>(s0, off[rb], base + (2 * v + 1) * kGroupBytes + rb * 1024 - 128);
        }
        dma16<0>(s8, offr, base + 8 * kGroupBytes + v * 1024);
      } else {
        const char* s0 = uniform_ptr(src + 128 * v);  // codes group v
        const char* s4 = uniform_ptr(src + 512);      // rope group
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) dma16<0>(s0, off[rb], base + v * kGroupBytes + rb * 1024);
        dma16<0>(s4, offr, base + 4 * kGroupBytes + v * 1024);
        if constexpr (F == kFmtFp8) {
          // the slot's 32 rows of tile scales (16 bytes each): lanes 0..31
          // rows 0..31, lanes 32..63 again (into the second half of this
          // wave's 1 KB, never read); past the valid rows the last valid one
          const char* ssrc = uniform_ptr((const char*)(a.kv_scales + row0s * 4));
          const uint32_t soff = (uint32_t)(16 * min(lane & 31, nvalid - 1));
          dma16<0>(ssrc, soff, base + Fm::kScaleOff + v * 1024);
        }
      }
    };
    for (int pass = 0; pass < 2; ++pass) {
      f32x16 o[2][4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) o[rb][cb] = f32x16{};
      // copy epochs -3 .. -1 (the prologue): slots 0 .. 2; slot 0 landed
      const int pre = min(nslots, 3);
      if constexpr (TOPK) {
        // translate slots 0..4 (entries, then their pages) and stage the
        // entries of slots 5 and 6; the slot loop keeps the pages five and
        // the entries seven slots ahead
        // (each wait is followed by a compiler barrier: the copies write LDS
        // behind the compiler's back, and the waits alone do not keep the
        // LDS reads of the staged words below them)
        for (int s = 0; s < 7; ++s) tk_idx_dma(s);
        wait_vm_lgkm0<0>();
        asm volatile("" ::: "memory");
        for (int s = 0; s < 5; ++s) tk_pg_dma(s);
        wait_vm_lgkm0<0>();
        asm volatile("" ::: "memory");
      }
      // slot 0 first, then X: the score waves load their queries only after
      // these copies are issued, so that slot 0 is not queued behind them;
      // slots 1 and 2 follow after Y, behind the query loads, which the first
      // slot needs sooner
      if (pre > 0) dma_cols(0, 0);
      if (pass == 0) {
        barrier();  // X
        barrier();  // Y
      }
      for (int s = 1; s < pre; ++s) dma_cols(s, s);
      wait_ops_lgkm0<N>(epoch_ops<N>(-2, nslots) + epoch_ops<N>(-1, nslots));
      barrier();  // B_0
      VF vx[4], vy[4];
      // iteration it (between B_it and B_it+1): epoch it issues the copies of
      // slot it+3 (into the ring position of slot it-1, whose last reads were
      // in iteration it-1); PV of slot it-1 from vc, while the V fragments of
      // slot it (landed before B_it) are read into vn for the next iteration
      auto iteration = [&](int it, VF (&vc)[4], VF (&vn)[4]) {
        if constexpr (TOPK) {
          // the entries of slot it+5 and the pages of slot it+3, both staged
          // two iterations ago, landed: everything of this wave's but the
          // copies of slots it+1 and it+2 and the two staging loads between
          // them (completion is in order); then stage the pages of slot it+5
          // and the entries of slot it+7
          const int k = (it >= 2 ? epoch_ops<N>(it - 2, nslots) : 0) + epoch_ops<N>(it - 1, nslots);
          if (k == 2 * N) wait_vm_lgkm0<2 * N + 2>();
          else if (k == N) wait_vm_lgkm0<N + 2>();
          else wait_vm_lgkm0<2>();
          asm volatile("" ::: "memory");
          tk_pg_dma(it + 5);
          tk_idx_dma(it + 7);
        }
        if (it + 3 < nslots) dma_cols(it + 3, it + 3);
        const lds_char* nbuf = L.ring + (it & (kRing - 1)) * Fm::kSlot;
        // this wave's V^T fragments of slot it, column block cb
        auto vload = [&](int cb, VF& f) {
          if constexpr (F == kFmtBf16) {
            ws_vload(nbuf, va, cb, f);
          } else {
            typedef int v2i __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(nbuf + (va[ks] ^ (32u * cb))));
              f[ks] = u32x2{(uint32_t)x[0], (uint32_t)x[1]};
            }
          }
        };
        if (it >= 1) {
          const lds_char* pt = L.ptile + ((it - 1) & 1) * Fm::kPTiles * kPTile + ptv;
          bf16x8 pf[2][2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) pf[rb][ks] = *(const LDS_AS bf16x8*)(pt + prd + rb * 32 * kPRowBytes + 32 * ks);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            bf16x8 v0, v1;
            if constexpr (F == kFmtBf16) {
              v0 = __builtin_shufflevector(vc[cb][0], vc[cb][1], 0, 1, 2, 3, 4, 5, 6, 7);
              v1 = __builtin_shufflevector(vc[cb][2], vc[cb][3], 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
              v0 = codes_bf16(vc[cb][0]);
              v1 = codes_bf16(vc[cb][1]);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              o[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pf[rb][0], o[rb][cb], 0, 0, 0);
              o[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pf[rb][1], o[rb][cb], 0, 0, 0);
            }
            if (it < nslots) vload(cb, vn[cb]);
          }
        } else if (it < nslots) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) vload(cb, vn[cb]);
        }
        if (pass == 0 && it == 0) barrier();  // the score waves' reference exchange
        // slot it+1 landed (the operations of epochs it-1 and it may stay in
        // flight), and this wave's LDS reads of slot it are done before the
        // next iteration's copies refill the ring position of slot it-1
        if constexpr (TOPK) {
          // slot it+1 landed; the copies of the two later epochs and their
          // staging loads (two per iteration; the prologue issues none after
          // its copies) may stay in flight
          wait_ops_lgkm0<N>(epoch_ops<N>(it - 1, nslots) + epoch_ops<N>(it, nslots), it >= 1 ? 4 : 2);
        } else {
          wait_ops_lgkm0<N>(epoch_ops<N>(it - 1, nslots) + epoch_ops<N>(it, nslots));
        }
        barrier();  // B_it+1
      };
      for (int it = 0; it <= nslots; it += 2) {
        iteration(it, vy, vx);
        if (it + 1 <= nslots) iteration(it + 1, vx, vy);
      }
      barrier();  // the score waves' sums and votes
      const int votes = L.votes[0] | L.votes[1] | L.votes[2] | L.votes[3];
      if (__builtin_amdgcn_readfirstlane(votes) == 0) {
        // normalise this wave's 128 columns of the 64 rows, round them (bf16
        // output, or the fp16 partial below), and store them through LDS: the
        // lane holds row 32rb + lane%32 and, per column block and register
        // quad, four consecutive columns, so direct stores would scatter each
        // instruction over 32 rows; the wave writes its 64 x 128 block into
        // the ring (idle after the last slot; the next segment's copies start
        // after a workgroup barrier), then stores two whole 256-byte rows per
        // instruction.  The lane index is passed through an empty asm so
        // that the compiler cannot hoist these per-lane addresses out of the
        // slot loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int i32 = ln & 31, h2 = ln >> 5;
        const size_t pslot = piece_slot(a, b, r, sgm.first_r);
        constexpr int kPitch = 264;  // bytes per staged row: 256 + 8, so that 32 rows spread over the banks
        static_assert(4 * 64 * kPitch <= kRing * Fm::kSlot, "the four waves' staging fits in the ring");
        LDS_AS char* const stg = (LDS_AS char*)L.ring + v * (64 * kPitch);
        const bool split = sgm.nsplit > 1;
        char* const gbase = split ? (char*)(a.ws_o16 + pslot * a.heads * kDV)
                                  : (char*)((__bf16*)a.out + (size_t)b * a.heads * kDV);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int lr = 32 * rb + i32;
          const float lt = L.xl[lr] + L.xl[64 + lr];
          const float inv = lt > 0.0f ? kdesc / lt : 0.0f;
          // a piece of a split sequence stores the normalised values v of
          // this row's 128 columns as fp16 of v / 2^e, with e chosen from
          // their largest magnitude m (= f 2^x, f in [0.5, 1)) as x - 15,
          // which puts m / 2^e in [2^14, 2^15) below the fp16 maximum; the
          // scaling is exact, so each value carries one fp16 rounding, at
          // most 2^-11 m.  (Zero, inf and NaN maxima give x = 0: the values
          // pass unchanged in range or as inf and NaN.)  The clamp keeps
          // 2^-e and 2^e normal fp32 numbers.  (The largest |o| times inv is
          // the largest |o inv|: inv > 0 and rounding is monotonic.)  The
          // scaling folds into inv: o (inv 2^-e) = (o inv) 2^-e exactly
          // while inv 2^-e stays a normal number, that is unless the values
          // reach 2^100.
          float sinv = inv;
          int ex = 0;
          if (split) {
            float mx = 0.0f;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
              for (int k = 0; k < 16; ++k) mx = fmaxf(mx, fabsf(o[rb][cb][k]));
            mx = max_halves(mx) * inv;  // lanes l and l^32 hold the same row
            ex = min(max(__builtin_amdgcn_frexp_expf(mx) - 15, -110), 113);
            sinv = __builtin_amdgcn_ldexpf(inv, -ex);
          }
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              // accumulator registers 4q .. 4q+3: columns 32cb + 8q + 4h2 .. +3
              f32x4 val;
#pragma unroll
              for (int e = 0; e < 4; ++e) val[e] = o[rb][cb][4 * q + e] * sinv;
              LDS_AS char* const dst = stg + lr * kPitch + 2 * (32 * cb + 8 * q + 4 * h2);
              if (split) *(LDS_AS f16x4*)dst = __builtin_convertvector(val, f16x4);
              else *(LDS_AS bf16x4*)dst = __builtin_convertvector(val, bf16x4);
            }
          // this block's 32 rows: rows 32rb + 2k and +1 from lanes 0..31 and
          // 32..63, four columns each (the stores drain while the next
          // block is formed)
#pragma unroll
          for (int k0 = 0; k0 < 16; k0 += 8) {
            u32x2 x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = *(const LDS_AS u32x2*)(stg + (32 * rb + 2 * (k0 + k) + h2) * kPitch + 8 * i32);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int row = row0 + 32 * rb + 2 * (k0 + k) + h2;
              if (row < a.heads) *(u32x2*)(gbase + ((size_t)row * kDV + 128 * v + 4 * i32) * 2) = x[k];
            }
          }
          if (split && h2 == 0 && row0 + lr < a.heads)
            a.ws_sc[(pslot * a.heads + row0 + lr) * 4 + v] = __builtin_amdgcn_ldexpf(1.0f, ex);
        }
        break;
      }
      if constexpr (!TOPK) {
        if (sg.npages > 64) page_cache_load(pc, sg.bt_seg, 0, sg.npages, lane);
      }
      wait_vm_lgkm0<0>();
      barrier();  // every wave has read the votes
    }
  });
}

template <int F, bool Q_FP8, bool CAUSAL, bool TOPK>
__global__ void __attribute__((amdgpu_flat_work_group_size(kWsThreads, kWsThreads), amdgpu_waves_per_eu(2, 2)))
mla_decode_ws_kernel(DecodeArgs a) {
  // KV ring (4 slots) and P tiles (two slots' worth)
  __shared__ __attribute__((aligned(1024))) char ring_mem[kRing * WsFmt<F>::kSlot];
  __shared__ __attribute__((aligned(16))) char ptile_mem[2 * WsFmt<F>::kPTiles * kPTile];
  __shared__ __attribute__((aligned(16))) float xs[512];                        // row exchanges, votes
  __shared__ __attribute__((aligned(16))) int32_t tk_mem[TOPK ? 4 * kTkWords : 4];  // top-k staging
  WsLds L;
  L.tkmask = (LDS_AS uint32_t*)xs + 448;
  L.tk = (LDS_AS int32_t*)tk_mem;
  L.ring = (lds_char*)ring_mem;
  L.ptile = (lds_char*)ptile_mem;
  L.xref = (LDS_AS float*)xs;
  L.xl = (LDS_AS float*)xs + 128;
  L.xm = (LDS_AS float*)xs + 256;
  L.votes = (LDS_AS int*)xs + 384;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x;
  // XCD-aware mapping, as in decode.hip: workgroup g runs on XCD g % 8, which
  // gets a run of consecutive ranges with all their slabs
  const int idx = g / 8;
  const int r = (g % 8) * a.per_xcd + idx / a.slabs;
  const int slab = idx % a.slabs;
  Plan pl;
  // (the plan also loads the length of sequence g, checked for emptiness below)
  int units_g = 1;
  const bool has_work = make_plan<kWsThreads>(a, r, (int*)ring_mem, pl, units_g) && r < a.ranges;
  // sequences with nothing to attend: O = 0, LSE = -inf
  for (int b = g; b < a.batch; b += gridDim.x) {
    if ((b == g ? units_g : units_of(a, b)) == 0) {
      for (int i = tid; i < a.heads * (kDV / 4); i += kWsThreads)
        *(bf16x4*)((__bf16*)a.out + ((size_t)b * a.heads) * kDV + 4 * i) = bf16x4{};
      for (int i = tid; i < a.heads; i += kWsThreads) a.lse[(size_t)b * a.heads + i] = -INFINITY;
      if (tid == 0) a.ws_seq[b] = int2{0, 0};
    }
  }
  if (!has_work) return;
  const int row0 = slab * kWsRows;
  if (w < 4) score_role<F, Q_FP8, CAUSAL, TOPK>(a, pl, L, w, lane, row0, r);
  else value_role<F, TOPK>(a, pl, L, w - 4, lane, row0, r);
}

}  // namespace

bool decode_ws_supported(int32_t kv_format, int32_t topk, int32_t eff_heads, int32_t num_pages) {
  if (eff_heads < kWsRows) return false;
  if (topk == 0) return true;
  // top-k lists: the FP8 caches (the bf16 ring leaves no room for the
  // staging), with every cache row reachable by a 32-bit byte offset
  const int64_t row_bytes = kv_format == kKvFormatFp8Tile ? kFp8RowBytes : kFp8TRowBytes;
  return kv_format != kKvFormatBf16 && (int64_t)num_pages * kPage * row_bytes < ((int64_t)1 << 32);
}

hipError_t launch_decode_ws(const DecodeArgs& a, int32_t kv_format, bool q_fp8, bool causal, hipStream_t stream) {
  const dim3 grid(a.per_xcd * 8 * a.slabs), block(kWsThreads);
#define MLA_WS_LAUNCH(F, QF, C)                                                                          \
  if (fmt == F && q_fp8 == QF && causal == C && !topk)                                                   \
    hipLaunchKernelGGL((mla_decode_ws_kernel<F, QF, C, false>), grid, block, 0, stream, a);
#define MLA_WS_LAUNCH_TOPK(F, QF)                                                                        \
  if (fmt == F && q_fp8 == QF && topk) hipLaunchKernelGGL((mla_decode_ws_kernel<F, QF, false, true>), grid, block, 0, stream, a);
  const bool topk = a.topk > 0;
  const int fmt = kv_format == kKvFormatFp8Tile ? kFmtFp8 : kv_format == kKvFormatFp8Tensor ? kFmtFp8T : kFmtBf16;
  MLA_WS_LAUNCH(kFmtBf16, false, false)
  MLA_WS_LAUNCH(kFmtBf16, false, true)
  MLA_WS_LAUNCH(kFmtBf16, true, false)
  MLA_WS_LAUNCH(kFmtBf16, true, true)
  MLA_WS_LAUNCH(kFmtFp8, false, false)
  MLA_WS_LAUNCH(kFmtFp8, false, true)
  MLA_WS_LAUNCH(kFmtFp8, true, false)
  MLA_WS_LAUNCH(kFmtFp8, true, true)
  MLA_WS_LAUNCH(kFmtFp8T, false, false)
  MLA_WS_LAUNCH(kFmtFp8T, false, true)
  MLA_WS_LAUNCH(kFmtFp8T, true, false)
  MLA_WS_LAUNCH(kFmtFp8T, true, true)
  MLA_WS_LAUNCH_TOPK(kFmtFp8, false)
  MLA_WS_LAUNCH_TOPK(kFmtFp8, true)
  MLA_WS_LAUNCH_TOPK(kFmtFp8T, false)
  MLA_WS_LAUNCH_TOPK(kFmtFp8T, true)
#undef MLA_WS_LAUNCH
#undef MLA_WS_LAUNCH_TOPK
  return hipGetLastError();
}

}  // namespace mla
