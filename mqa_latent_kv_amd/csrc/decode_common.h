// decode_common.h - device-side pieces shared by the decode kernels:
// element types, the KV row geometry, the kernel arguments, the in-kernel
// work split over KV ranges, the swizzled LDS slot layout and its direct
// global->LDS copies, and the per-segment block-table cache.
#pragma once

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS char lds_char;

constexpr int kD = 576;
constexpr int kDV = 512;
constexpr int kPage = 64;
constexpr int kRowBytes = kD * 2;            // bf16 latent row
constexpr int kTS = 32;                      // tokens per LDS slot
constexpr int kSlotBytes = kTS * kRowBytes;  // 36864
constexpr int kRing = 4;                     // LDS slots (DMA ring)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 16.0f;  // largest rise of a head's max over its first-slot reference (base 2)
// a slot's 36 copies of 1 KB are shared by four waves: nine each
constexpr int kDmaWaves = 4;
constexpr int kDmaPerWave = kSlotBytes / 1024 / kDmaWaves;

// (DecodeArgs, the kernel argument block, is declared in mla_internal.h)

// ---------------------------------------------------------------- helpers

// Slot layout in LDS: the 1152-byte rows are cut into 9 column groups of 128
// bytes (64 latent columns); group c of all 32 rows is stored contiguously,
// row m at c*4096 + m*128.  Inside a row's 128 bytes the 16-byte chunk x sits
// at position x ^ row_swz(m).  The 64 banks of 4 bytes see a 256-byte period,
// so a 16-byte chunk's bank group is 8*(m&1) + position; row_swz makes
//  * the b128 K reads (16 lanes = 16 consecutive rows, one chunk) hit 16
//    distinct bank groups: for even rows, and for odd rows, bits 1..3 of m
//    map one-to-one onto the three bits of the swizzle;
//  * the tr_b16 V^T reads (32 lanes = rows r, r+1, r+2, r+3 with r % 4 == 0,
//    chunks 0..3 of a half group) conflict-free: rows r and r+2 share a
//    parity and differ in swizzle bit 2, so their four chunks fall in
//    opposite halves of the eight positions.
__device__ __forceinline__ int row_swz(int m) { return (((m >> 1) & 1) << 2) | (((m >> 3) & 1) << 1) | ((m >> 2) & 1); }

constexpr int kGroupBytes = kTS * 128;  // one 128-byte column group of all 32 rows

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  // s_waitcnt vmcnt(N) expcnt(7) lgkmcnt(0), GFX9 encoding.
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Workspace slot of the piece of sequence b in range r (its first range
// first_r): b + r, or in the compact layout 2r for a piece that continues a
// sequence from an earlier range and 2r + 1 for one that starts in r.
__device__ __forceinline__ size_t piece_slot(const DecodeArgs& a, int b, int r, int first_r) {
  return a.compact ? (size_t)(2 * r + (r == first_r ? 1 : 0)) : (size_t)(b + r);
}

__device__ __forceinline__ int units_of_len(const DecodeArgs& a, int s) {
  s = s < 0 ? 0 : (s > a.max_pages * kPage ? a.max_pages * kPage : s);
  return (s + kPage - 1) / kPage;
}
__device__ __forceinline__ int units_of(const DecodeArgs& a, int b) {
  if (a.topk > 0) return (a.topk + kPage - 1) / kPage;
  return units_of_len(a, a.seqlens[b]);
}

__device__ __forceinline__ int clamp_page(int p, int num_pages) {
  return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 codes, float scale) {
  f32x8 f;
  f32x2 t;
  t = __builtin_amdgcn_cvt_pk_f32_fp8(codes.x, false); f[0] = t[0]; f[1] = t[1];
  t = __builtin_amdgcn_cvt_pk_f32_fp8(codes.x, true);  f[2] = t[0]; f[3] = t[1];
  t = __builtin_amdgcn_cvt_pk_f32_fp8(codes.y, false); f[4] = t[0]; f[5] = t[1];
  t = __builtin_amdgcn_cvt_pk_f32_fp8(codes.y, true);  f[6] = t[0]; f[7] = t[1];
  f = f * scale;
  return __builtin_convertvector(f, bf16x8);
}

// ---------------------------------------------------------------- plan

// Every workgroup derives the same partition from seqlens: units (64-token
// pages, or 64-entry top-k chunks) of all sequences end to end, cut into
// `ranges` ranges of C units.  Returns false if range r has no work.
struct Plan {
  int C;      // units per range
  int start;  // first global unit of the range
  int end;    // one past the last
  int b0;     // first sequence overlapping [start, end)
  int p0;     // global index of b0's first unit
  int pad;    // virtual units at each end of every non-empty sequence on the line
};

// inclusive scan over the lanes of a wave (ds_bpermute moves data between
// lanes; it touches no LDS memory)
// (in registers: shifts by 1, 2, 4 and 8 lanes inside each 16-lane row by
// DPP row_shr, lanes shifted in from outside the row adding 0, then the
// three row totals taken by readlane and added to the rows after them)
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// The cut of the line when every sequence has the same number u of units
// (top-k lists: u = ceil(topk / 64) for every list, whatever its length):
// the plan below in closed form.  The unpadded line puts sequence b at b u,
// so some sequence starts strictly inside a range of the unpadded cut
// exactly when there are two or more and u is not a multiple of the cut
// C0 = ceil(B u / ranges) (b = 1 is then such a start; otherwise every
// start b u is a multiple of C0).
__host__ __device__ __forceinline__ void even_cut(int batch, int u, int ranges, int seg_pad, int& pad, int& C,
                                                  int& total) {
  const int c0 = (batch * u + ranges - 1) / ranges;
  pad = (seg_pad > 0 && batch >= 2 && u % c0 != 0) ? seg_pad : 0;
  total = batch * (u + 2 * pad);
  C = (total + ranges - 1) / ranges;
}

// The range of workgroup r.  The units of all sequences (pages, or top-k
// chunks of 64 entries) are laid end to end and cut into a.ranges equal
// ranges.  With a.seg_pad > 0 each non-empty sequence also gets that many
// virtual units at each end (the cost of a segment's start and end), but
// only when some sequence starts strictly inside a range of the unpadded
// cut: when every boundary falls on a cut (sequences of equal length, a
// whole number of ranges each), every range runs one segment and the pads
// would only unbalance them.
// Top-k lists all have the same length, so their cut (even_cut) needs no
// loads and no barriers.  Pages: the two block-wide scans (units and
// non-empty sequences) share one pass and one barrier, the padding vote a
// second, and the range's first sequence a third and fourth; every
// exchange has its own scratch words, so no barrier guards a reuse.
// (NT threads per workgroup; scratch holds 3 NT / 64 + 2 ints)
template <int NT>
__device__ bool make_plan(const DecodeArgs& a, int r, int* scratch, Plan& pl, int& units_g) {
  const int tid = threadIdx.x;
  const int B = a.batch;
  if (a.topk > 0) {
    const int u = (a.topk + kPage - 1) / kPage;
    units_g = u;
    int pad, C, total;
    even_cut(B, u, a.ranges, a.seg_pad, pad, C, total);
    const int start = r * C;
    if (start >= total) return false;
    const int line = u + 2 * pad;
    pl.C = C;
    pl.start = start;
    pl.end = min(start + C, total);
    pl.b0 = start / line;
    pl.p0 = pl.b0 * line;
    pl.pad = pad;
    return true;
  }
  const int per = (B + NT - 1) / NT;
  const int lo = tid * per, hi = min(B, lo + per);
  // a thread's first kCache sequences' units stay in registers for the two
  // later passes (one sequence per thread up to NT sequences)
  // (the loads go out together, from clamped indices, and are selected
  // afterwards; the same pass loads the length of sequence blockIdx.x, which
  // the kernel checks for emptiness: units_g, 1 past the batch)
  constexpr int kCache = 2;
  int uc[kCache];
  const int bg = blockIdx.x;
  {
    int sl[kCache + 1];
#pragma unroll
    for (int i = 0; i < kCache; ++i) sl[i] = a.seqlens[min(lo + i, B - 1)];
    sl[kCache] = a.seqlens[min(bg, B - 1)];
#pragma unroll
    for (int i = 0; i < kCache; ++i) uc[i] = units_of_len(a, sl[i]);
    units_g = units_of_len(a, sl[kCache]);
  }
  units_g = bg < B ? units_g : 1;
#pragma unroll
  for (int i = 0; i < kCache; ++i) uc[i] = lo + i < hi ? uc[i] : 0;
  auto units_at = [&](int b) {
    const int i = b - lo;
    return i == 0 ? uc[0] : i == 1 ? uc[1] : units_of(a, b);
  };
  int units = 0, seqs = 0;
  for (int b = lo; b < hi; ++b) {
    const int n = units_at(b);
    units += n;
    seqs += n > 0 ? 1 : 0;
  }
  // exclusive scans of units and of non-empty sequences, with their totals
  constexpr int W = NT / 64;
  const int lane = tid & 63, wv = tid >> 6;
  const int iu = wave_incl_scan(units, lane), iq = wave_incl_scan(seqs, lane);
  if (lane == 63) {
    scratch[wv] = iu;
    scratch[W + wv] = iq;
  }
  __syncthreads();
  int bu = 0, bq = 0, total0 = 0, nseq = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const int tu = scratch[i], tq = scratch[W + i];
    bu += i < wv ? tu : 0;
    bq += i < wv ? tq : 0;
    total0 += tu;
    nseq += tq;
  }
  total0 = __builtin_amdgcn_readfirstlane(total0);
  nseq = __builtin_amdgcn_readfirstlane(nseq);
  const int excl0 = bu + iu - units, exclq = bq + iq - seqs;
  if (total0 == 0) return false;
  int pad = 0;
  if (a.seg_pad > 0) {
    const int C0 = (total0 + a.ranges - 1) / a.ranges;
    int inside = 0, p = excl0;
    for (int b = lo; b < hi; ++b) {
      const int n = units_at(b);
      inside += (n > 0 && p % C0 != 0) ? 1 : 0;
      p += n;
    }
    const bool w_any = __builtin_amdgcn_ballot_w64(inside != 0) != 0;
    if (lane == 0) scratch[2 * W + wv] = w_any ? 1 : 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) any |= scratch[2 * W + i];
    pad = __builtin_amdgcn_readfirstlane(any) != 0 ? a.seg_pad : 0;
  }
  // padded line: sequence b starts at (its unpadded start) + 2 pad (non-empty sequences before it)
  const int total = total0 + 2 * pad * nseq;
  const int excl = excl0 + 2 * pad * exclq;
  const int incl = excl + units + 2 * pad * seqs;
  const int C = (total + a.ranges - 1) / a.ranges;
  const int start = r * C;
  if (start >= total) return false;
  if (start >= excl && start < incl) {
    int p = excl;
    for (int b = lo; b < hi; ++b) {
      const int u = units_at(b);
      const int n = u > 0 ? u + 2 * pad : 0;
      if (start < p + n) {
        scratch[3 * W] = b;
        scratch[3 * W + 1] = p;
        break;
      }
      p += n;
    }
  }
  __syncthreads();
  // values read back from LDS are wave-uniform: keep them in SGPRs
  pl.C = __builtin_amdgcn_readfirstlane(C);
  pl.start = __builtin_amdgcn_readfirstlane(start);
  pl.end = __builtin_amdgcn_readfirstlane(min(start + C, total));
  pl.b0 = __builtin_amdgcn_readfirstlane(scratch[3 * W]);
  pl.p0 = __builtin_amdgcn_readfirstlane(scratch[3 * W + 1]);
  pl.pad = __builtin_amdgcn_readfirstlane(pad);
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------- per-lane address tables

// DMA kk (0..8) of wave w fills rows 8w .. 8w+7 of column group kk: lane i
// writes LDS bytes 16i.. of that 1 KB block, which is row 8w + i/8, position
// i%8, and so fetches source chunk (i%8) ^ row_swz(row) of column group kk.
// The per-lane source offset is the same for all nine copies of a wave;
// the column group is the instruction's immediate offset.  Rows at and
// beyond row_cap read row row_cap.
__device__ __forceinline__ uint32_t dma_lane_off(int lane, int w, int row_cap) {
  int row = 8 * w + (lane >> 3);
  const int src_chunk = (lane & 7) ^ row_swz(row);
  row = row < row_cap ? row : row_cap;
  return (uint32_t)(row * kRowBytes + 16 * src_chunk);
}

// One direct global->LDS copy of 16 bytes per lane: lane i's bytes land at
// LDS address lds_base + 16*i.  Written as inline assembly so that the
// compiler's wait-count insertion does not see it: it cannot tell which ring
// slot a DMA targets and would otherwise wait for every copy in flight before
// each LDS read.  The ring accounts for these copies itself (explicit vmcnt
// before each barrier).  m0 is declared clobbered, and one wait state (s_nop 0)
// separates the scalar write of m0 from the copy that reads it, as the
// hardware requires between an SALU write of m0 and a VMEM load to LDS.
// (m0 is named in the clobber list on purpose: clang warns that it is reserved)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int OFF>
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff), "s"(sbase),
               "s"(lds_base), "n"(OFF)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// This wave's share of one slot's DMA, prepared in scalar registers: nine
// copies of 1 KB (rows 8w .. 8w+7 of each column group).  Rows at and beyond
// the slot's valid count re-read its last valid row, so a slot never holds
// foreign or unwritten data.
struct DmaJob {
  const char* base;  // source row 0 of the slot
  uint32_t off;      // per-lane source offset
  uint32_t lds0;     // LDS address of rows 8w.. of column group 0
};

// The instruction's immediate offset moves both the global source and the
// LDS destination; the M0 base takes it back out of the latter.
template <int KK>
__device__ __forceinline__ void dma_issue(const DmaJob& j) {
  dma16<128 * KK>(j.base, j.off, j.lds0 + KK * (kGroupBytes - 128));
}

template <int KK = 0>
__device__ __forceinline__ void dma_issue_all(const DmaJob& j) {
  if constexpr (KK < kDmaPerWave) {
    dma_issue<KK>(j);
    dma_issue_all<KK + 1>(j);
  }
}

// Block-table entries of the current segment, 64 at a time, one per lane:
// a page lookup is a readlane, not a memory access inside the ring.
struct PageCache {
  int v;     // lane i: block_table[row][base + i]
  int base;  // first segment page held
};

__device__ __forceinline__ void page_cache_load(PageCache& pc, const int32_t* bt_seg, int base, int npages, int lane) {
  pc.base = base;
  pc.v = (base + lane < npages) ? bt_seg[base + lane] : 0;
  // complete the load here, on this (rare) path, so that no wait for it is
  // left pending where the paths merge in the ring
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ int page_of(PageCache& pc, const int32_t* bt_seg, int k, int npages, int lane,
                                       int num_pages) {
  if (k >= pc.base + 64) page_cache_load(pc, bt_seg, k, npages, lane);  // segments longer than 64 pages
  return clamp_page(__builtin_amdgcn_readlane(pc.v, k - pc.base), num_pages);
}

// KV layouts the kernels read.
constexpr int kKvBf16 = 0;        // bf16 rows [P,64,576], whole pages (LDS DMA)
constexpr int kKvFp8 = 1;         // e4m3 rows [P,64,640] + fp32 scales [P,64,4], whole pages
constexpr int kKvFp8TopK = 2;     // e4m3 rows, gathered top-k entries
constexpr int kKvBf16TopK = 3;    // bf16 rows, gathered top-k entries
constexpr int kKvFp8T = 4;        // e4m3 rows [P,64,576], one per-tensor k_scale_inv, whole pages
constexpr int kKvFp8TTopK = 5;    // the same rows, gathered top-k entries
constexpr bool kv_fp8(int m) { return m == kKvFp8 || m == kKvFp8TopK; }  // per-tile scales (tiled QK^T)
constexpr bool kv_tensor(int m) { return m == kKvFp8T || m == kKvFp8TTopK; }
constexpr bool kv_topk(int m) { return m == kKvFp8TopK || m == kKvBf16TopK || m == kKvFp8TTopK; }
constexpr int kFp8RowBytes = 640;   // 512 e4m3 codes, 64 bf16 rope values
constexpr int kFp8TRowBytes = 576;  // 576 e4m3 codes

// max over lanes l and l^32 (the two token halves of one head's S^T column)
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// p = 2^(x*scale - m_ref) with the reference's negation; while no valid token
// has been seen (top-k slots of padding only) the reference is -inf and every
// score is -inf too, which must give p = 0, not NaN.
__device__ __forceinline__ float neg_ref(float m_ref) { return m_ref == -INFINITY ? 0.0f : -m_ref; }

struct SegCtx {
  const int32_t* bt_seg;     // block-table entries of the segment's pages
  const int32_t* idx_seg;    // top-k: the list's entries from tok0 on
  int tok0, tok1, nslots, npages;
};

// mask of the tokens [0, n) of a slot
__device__ __forceinline__ uint32_t low_mask(int n) { return n >= 32 ? 0xffffffffu : (1u << n) - 1u; }

// DMA job that fills ring position pos with slot s of the segment.  Slots at
// or beyond the end are replaced by the last slot: the copy then lands in a
// free ring position that is never read, which keeps the number of copies
// per step, and with it every vmcnt wait, the same on every step.
__device__ __forceinline__ DmaJob prep_slot(int s, int pos, lds_char* ring, const DecodeArgs& a, const SegCtx& sg,
                                            PageCache& pc, uint32_t dma_off, int w, int lane) {
  s = min(s, sg.nslots - 1);
  const int tk = sg.tok0 + s * kTS;
  const int page = page_of(pc, sg.bt_seg, s >> 1, sg.npages, lane, a.num_pages);
  const char* src = a.kv + ((size_t)page * kPage + (s & 1) * kTS) * kRowBytes;
  const int nvalid = min(kTS, sg.tok1 - tk);
  DmaJob j;
  j.base = uniform_ptr(src);
  j.lds0 = __builtin_amdgcn_readfirstlane(lds_addr(ring + (pos & (kRing - 1)) * kSlotBytes) + w * 1024);
  j.off = nvalid >= kTS ? dma_off : dma_lane_off(lane, w, nvalid - 1);
  return j;
}

}  // namespace
}  // namespace mla
