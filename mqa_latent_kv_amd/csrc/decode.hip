// decode.hip - split-KV absorbed MLA decode for gfx950 (MI355X).
//
// What is computed (one query token per sequence): for every head h of
// sequence b, scores against the shared 576-wide latent rows (512 nope + 64
// rope; the rope block is one more slice of the same QK^T, as in FlashMLA
// issue "dual gemm"), a scaled softmax per head row, and O = P.V with V the
// 512 nope columns.  Output O in bf16 and the natural-log LSE per head.
//
// Design (MI355X-first; the pages' Blackwell designs are prior art only):
//  * Head-packed tile ("STAGE_D2" note, "Strategy A: Head-Packed M
//    Dimension"): a workgroup reads each KV row once for a slab of up to 64
//    heads of its sequence.  The MFMA is v_mfma_f32_32x32x16_bf16 with the 32
//    KV tokens of an LDS slot as M and 32 heads as N:
//        S^T[t][h] = sum_d K[t][d] Q[h][d]          (K = 576 = 36 steps)
//        O^T[c][h] += sum_t V^T[c][t] P^T[t][h]     (2 steps per 32 columns)
//    With tokens on M the S^T accumulator is already the P^T operand of the
//    PV product (the k <-> token permutation is absorbed in the V^T read), and
//    all O^T registers of a lane belong to one head, so the online-softmax
//    rescale is a per-lane scalar multiply.
//  * Split reduction (the CDNA counterpart of the issue's "dual gemm", which
//    halves the QK^T K dimension across warpgroups and sums the halves): the
//    NSPLIT waves of a 32-head group each own 576/NSPLIT of the QK^T
//    reduction and 512/NSPLIT output columns.  Partial S^T go through LDS and
//    every wave of the group adds them in the same order, so all of them hold
//    bit-identical scores and softmax state.  A wave keeps 144/NSPLIT query
//    VGPRs and 256/NSPLIT accumulator AGPRs, which leaves the compiler room.
//  * Slabs: H = 128 runs as two 64-head workgroups per KV range; the pair is
//    placed on one XCD (workgroups are dealt round-robin to the 8 XCDs) so the
//    second reader of every KV line finds it in that XCD's L2.
//  * KV streaming: 32-token slots of 36 KB in a 4-deep LDS ring filled by
//    direct global->LDS DMA (global_load_lds_dwordx4), three slots in flight
//    while one is consumed.  Rows are XOR-swizzled in 16-byte chunks so the
//    ds_read_b128 K reads and the ds_read_b64_tr_b16 V^T reads are free of
//    bank conflicts.  The DMA is issued from inline assembly and accounted
//    for by explicit vmcnt waits, so the compiler never serialises LDS reads
//    behind copies still in flight.
//  * Split-KV: pages of all sequences are laid end to end and cut into equal
//    ranges, one per workgroup (a static form of the persistent scheduler the
//    STAGE_D2 note mentions under "Grid vs. Persistent Tile Scheduler").  A
//    sequence covered by one range is finished in place; otherwise each piece
//    writes a normalised fp32 partial and its base-2 LSE and bumps a counter,
//    and the last piece to arrive merges them (one launch, no waiting on other
//    workgroups) and resets the counter for the next call.
//  * Softmax in base 2 against a fixed reference per head: the first slot's
//    max.  Later slots may exceed it by up to 16 (P <= 2^16, exact in fp32 and
//    as relative bf16); if any head's scores rise further, the workgroup
//    redoes the segment once with the true maxima (then P <= 1).  Realistic
//    score distributions never trigger the redo.  With no rescale inside the
//    KV loop the fp32 accumulators are only ever written by MFMAs and stay in
//    fixed AGPRs.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS char lds_char;

constexpr int kD = 576;
constexpr int kDV = 512;
constexpr int kPage = 64;
constexpr int kRowBytes = kD * 2;            // bf16 latent row
constexpr int kTS = 32;                      // tokens per LDS slot
constexpr int kSlotBytes = kTS * kRowBytes;  // 36864
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kDmaPerWave = kSlotBytes / 1024 / kWaves;  // 9 x 1 KB per wave per slot
constexpr int kKSteps = kD / 16;                         // 36 MFMA k-steps for QK^T
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 16.0f;  // largest rise of a head's max over its first-slot reference (base 2)

struct DecodeArgs {
  const void* q;
  const char* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* topk_idx;
  const float* kv_scales;
  void* out;
  float* lse;
  float* ws_o;    // [(ranges + B) slots][H][512] fp32 partials
  float* ws_lse;  // [(ranges + B)][H] base-2 LSE of partials
  int* ws_count;  // [B][slabs] arrival counters of split sequences; zero between calls
  int32_t batch, heads, num_pages, max_pages, topk;
  int32_t ranges;  // KV ranges (workgroups per head slab)
  int32_t slabs;   // head slabs per range
  float scale_log2;  // softmax_scale * log2(e)
  float q_descale;
};

// ---------------------------------------------------------------- helpers

// Chunk swizzle inside each 128-byte group of a 1152-byte row: the low three
// bits of the 16-byte chunk index are XORed with f(row).  f maps 8 consecutive
// rows to 8 distinct values (b128 reads of 8 rows) and 4 consecutive rows
// starting at a multiple of 4 to 4 values whose XOR with an even chunk pair
// covers all 8 positions (tr_b16 reads of 4 rows x 32 bytes).
__device__ __forceinline__ int row_swz(int m) { return ((m & 3) << 1) | ((m >> 2) & 1); }

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  // s_waitcnt vmcnt(N) expcnt(7) lgkmcnt(0), GFX9 encoding.
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ int units_of(const DecodeArgs& a, int b) {
  if (a.topk > 0) return (a.topk + kPage - 1) / kPage;
  int s = a.seqlens[b];
  s = s < 0 ? 0 : (s > a.max_pages * kPage ? a.max_pages * kPage : s);
  return (s + kPage - 1) / kPage;
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
};

__device__ bool make_plan(const DecodeArgs& a, int r, int* scratch, Plan& pl) {
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int per = (B + kThreads - 1) / kThreads;
  const int lo = tid * per, hi = min(B, lo + per);
  int local = 0;
  for (int b = lo; b < hi; ++b) local += units_of(a, b);
  // inclusive scan of the per-thread sums (Hillis-Steele in LDS)
  scratch[tid] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int v = tid >= off ? scratch[tid - off] : 0;
    __syncthreads();
    scratch[tid] += v;
    __syncthreads();
  }
  const int incl = scratch[tid];
  const int total = scratch[kThreads - 1];
  const int excl = incl - local;
  __syncthreads();
  if (total == 0) return false;
  const int C = (total + a.ranges - 1) / a.ranges;
  const int start = r * C;
  if (start >= total) return false;
  if (start >= excl && start < incl) {
    int p = excl;
    for (int b = lo; b < hi; ++b) {
      int n = units_of(a, b);
      if (start < p + n) {
        scratch[kThreads] = b;
        scratch[kThreads + 1] = p;
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
  pl.b0 = __builtin_amdgcn_readfirstlane(scratch[kThreads]);
  pl.p0 = __builtin_amdgcn_readfirstlane(scratch[kThreads + 1]);
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------- per-lane address tables

template <int NSPLIT>
struct LaneTables {
  uint32_t dma[kDmaPerWave];  // (row << 16) | (source byte offset of the chunk within its row)
  uint32_t kaddr[4];          // QK A operand for this wave's k-step i: kaddr[i & 3] + 128*(i >> 2)
  uint32_t vaddr;             // PV A operand (tr reads) for ks = tt = 0 and an even column block
};

template <int NSPLIT>
__device__ __forceinline__ void make_tables(LaneTables<NSPLIT>& t, int lane, int w, int part) {
  constexpr int KS = kKSteps / NSPLIT;
  constexpr int NCB = 16 / NSPLIT;
  for (int k = 0; k < kDmaPerWave; ++k) {
    int cl = (w * kDmaPerWave + k) * 64 + lane;  // LDS chunk written by this lane
    int m = cl / 72, pos = cl % 72;
    int col = (pos & ~7) | ((pos ^ row_swz(m)) & 7);  // source chunk (the swizzle is an involution)
    t.dma[k] = ((uint32_t)m << 16) | (uint32_t)(col * 16);
  }
  {
    // k-step ks = part*KS + i reads chunk 2*ks + h of row m
    const int m = lane & 31, h = lane >> 5;
    for (int i = 0; i < 4; ++i) {
      const int chunk = 2 * (part * KS + i) + h;
      t.kaddr[i] = m * kRowBytes + 16 * ((chunk & ~7) | ((chunk ^ row_swz(m)) & 7));
    }
  }
  {
    // tr read of rows m = 16ks + 8tt + 4h + j (j = row in the 4-row block),
    // columns 32cb + 16cpart + 4q .. +3 with cb = part*NCB + cbi.
    const int G = lane >> 4, i = lane & 15, j = i >> 2, q = i & 3, h = G >> 1, cpart = G & 1;
    const int m = 4 * h + j;  // ks = tt = 0; row_swz(m) is the same for all (ks, tt)
    const int low = (2 * cpart + (q >> 1)) ^ row_swz(m);
    t.vaddr = m * kRowBytes + 128 * (part * NCB / 2) + 16 * (low & 7) + 8 * (q & 1);
  }
}

// One direct global->LDS copy of 16 bytes per lane: lane i's bytes land at
// LDS address lds_base + 16*i.  Written as inline assembly so that the
// compiler's wait-count insertion does not see it: it cannot tell which ring
// slot a DMA targets and would otherwise wait for every copy in flight before
// each LDS read.  The ring accounts for these copies itself (explicit vmcnt
// before each barrier).  The kernel keeps no other value in m0.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory");
}

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// Issue this wave's share of one slot's DMA: 32 rows starting at `src`; rows
// at and beyond `nvalid` re-read row nvalid-1 (a valid row), so the slot never
// holds foreign or unwritten data.
template <int NSPLIT>
__device__ __forceinline__ void dma_slot(lds_char* dst, const char* src, int nvalid, const LaneTables<NSPLIT>& t,
                                         int w) {
  const char* base = uniform_ptr(src);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(dst) + w * kDmaPerWave * 1024);
#pragma unroll
  for (int k = 0; k < kDmaPerWave; ++k) {
    const uint32_t m = t.dma[k] >> 16, off = t.dma[k] & 0xffff;
    const uint32_t mm = m < (uint32_t)nvalid ? m : (uint32_t)(nvalid - 1);
    dma16(base, mm * kRowBytes + off, lds0 + k * 1024);
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

// ---------------------------------------------------------------- compute on one slot

template <int NSPLIT>
struct Acc {
  f32x16 o[16 / NSPLIT];  // O^T accumulators (AGPRs), relative to the reference max
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

template <int NSPLIT>
__device__ __forceinline__ void compute_slot(const lds_char* buf, LDS_AS f32x4* xch, int nvalid,
                                             const bf16x8 (&qf)[kKSteps / NSPLIT], const LaneTables<NSPLIT>& t,
                                             SoftmaxState& st, Acc<NSPLIT>& acc, float scale_log2, int lane, int w) {
  constexpr int KS = kKSteps / NSPLIT;
  constexpr int NCB = 16 / NSPLIT;
  // partial S^T[token][head] over this wave's share of the 576 columns
  f32x16 s = {};
#pragma unroll
  for (int i = 0; i < KS; ++i) {
    bf16x8 kf = *(const LDS_AS bf16x8*)(buf + t.kaddr[i & 3] + 128 * (i >> 2));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i], s, 0, 0, 0);
  }
  // keep three K fragments in flight ahead of the MFMA that consumes them
  __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
  for (int i = 0; i < KS - 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  // exchange partials inside the head group; every wave sums them in the
  // same order so the group holds bit-identical scores
  const int grp = (w / NSPLIT) * NSPLIT;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    f32x4 v = {s[4 * r4], s[4 * r4 + 1], s[4 * r4 + 2], s[4 * r4 + 3]};
    xch[(w * 4 + r4) * 64 + lane] = v;
  }
  wait_vm_lgkm0<63>();  // lgkmcnt(0): this wave's LDS writes are done
  barrier();
  f32x16 tot;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    f32x4 acc = xch[(grp * 4 + r4) * 64 + lane];
#pragma unroll
    for (int p = 1; p < NSPLIT; ++p) acc += xch[((grp + p) * 4 + r4) * 64 + lane];
    tot[4 * r4] = acc[0];
    tot[4 * r4 + 1] = acc[1];
    tot[4 * r4 + 2] = acc[2];
    tot[4 * r4 + 3] = acc[3];
  }
  // online softmax (base 2) over the slot's tokens for this lane's head
  float x[16];
  float mx = -INFINITY;
  const int hi = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * hi + (r & 3);
    x[r] = m < nvalid ? tot[r] * scale_log2 : -INFINITY;
    mx = fmaxf(mx, x[r]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));  // lanes l and l^32 hold the two token halves of a head
  // the first slot fixes the reference; later slots may exceed it by up to
  // kTau without loss (p <= 2^kTau), beyond that the segment is redone
  if (st.m_ref == -INFINITY) st.m_ref = mx;
  st.m_seen = fmaxf(st.m_seen, mx);
  const float mref = st.m_ref;
  f32x8 p0, p1;
  float lsum = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    p0[r] = __builtin_amdgcn_exp2f(x[r] - mref);
    p1[r] = __builtin_amdgcn_exp2f(x[r + 8] - mref);
    lsum += p0[r] + p1[r];
  }
  st.l_sum += lsum;
  const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
  const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
  // O^T[c][head] += V^T . P^T over this wave's column blocks.  k-step 0 of a
  // block covers tokens 0..15 in the order the S^T layout hands them to this
  // lane (rows 4h+j and 8+4h+j), k-step 1 tokens 16..31.
  const uint32_t va0 = t.vaddr, va1 = t.vaddr ^ 64u;
#pragma unroll
  for (int cbi = 0; cbi < NCB; ++cbi) {
    const uint32_t va = (cbi & 1) ? va1 : va0;
    const int step = 128 * (cbi >> 1);
    bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(buf + va + step));
    bf16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(buf + va + step + 8 * kRowBytes));
    bf16x4 c0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(buf + va + step + 16 * kRowBytes));
    bf16x4 c1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(buf + va + step + 24 * kRowBytes));
    const bf16x8 v0 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 v1 = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc.o[cbi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pb0, acc.o[cbi], 0, 0, 0);
    acc.o[cbi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pb1, acc.o[cbi], 0, 0, 0);
  }
  // the four V^T reads of block cbi+1 are in flight while block cbi's two
  // MFMAs run
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
  for (int cbi = 0; cbi < NCB - 1; ++cbi) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
}

struct SegCtx {
  const int32_t* bt_seg;  // block-table entries of the segment's pages
  int tok0, tok1, nslots, npages;
};

// One step of the ring: wait for slot s, free the ring slot consumed in the
// previous step and refill it with slot s+3, compute slot s.  A plain loop
// with a run-time slot offset: the DMA is invisible to the compiler, so the
// slots need no compile-time identity, and a loop body without early exits
// lets the accumulators stay in fixed AGPRs.
template <int NSPLIT>
__device__ __forceinline__ void ring_step(int s, lds_char* ring, LDS_AS f32x4* xch, const DecodeArgs& a,
                                          const SegCtx& sg, PageCache& pc, const bf16x8 (&qf)[kKSteps / NSPLIT],
                                          const LaneTables<NSPLIT>& t, SoftmaxState& st, Acc<NSPLIT>& acc,
                                          int lane, int w) {
  const int later = min(sg.nslots - 1 - s, 2);
  if (later == 2) wait_vm_lgkm0<2 * kDmaPerWave>();
  else if (later == 1) wait_vm_lgkm0<kDmaPerWave>();
  else wait_vm_lgkm0<0>();
  barrier();
  if (s + 3 < sg.nslots) {
    const int ns = s + 3;
    const int tk = sg.tok0 + ns * kTS;
    const int page = page_of(pc, sg.bt_seg, ns >> 1, sg.npages, lane, a.num_pages);
    const char* src = a.kv + ((size_t)page * kPage + (ns & 1) * kTS) * kRowBytes;
    dma_slot<NSPLIT>(ring + (ns & 3) * kSlotBytes, src, min(kTS, sg.tok1 - tk), t, w);
  }
  compute_slot<NSPLIT>(ring + (s & 3) * kSlotBytes, xch, min(kTS, sg.tok1 - (sg.tok0 + s * kTS)), qf, t, st, acc,
                       a.scale_log2, lane, w);
}

// Merge the nsplit pieces of sequence b for the heads of one slab:
// LSE = log2 sum_s 2^lse_s, O = sum_s 2^(lse_s - LSE) O_s.  Piece s of the
// sequence sits in workspace slot first + s.
template <int HPS>
__device__ void merge_pieces(const DecodeArgs& a, int b, int slab, int first, int nsplit) {
  for (int idx = threadIdx.x; idx < HPS * (kDV / 4); idx += kThreads) {
    const int head = slab * HPS + idx / (kDV / 4), c4 = idx % (kDV / 4);
    if (head >= a.heads) break;
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, a.ws_lse[((size_t)first + s) * a.heads + head]);
    f32x4 acc = {};
    float wsum = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float l = a.ws_lse[((size_t)first + s) * a.heads + head];
      const float wgt = (l == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(l - mx);
      const f32x4 v = *(const f32x4*)(a.ws_o + (((size_t)first + s) * a.heads + head) * kDV + 4 * c4);
      acc += wgt * v;
      wsum += wgt;
    }
    acc *= wsum > 0.0f ? 1.0f / wsum : 0.0f;
    *(bf16x4*)((__bf16*)a.out + ((size_t)b * a.heads + head) * kDV + 4 * c4) = __builtin_convertvector(acc, bf16x4);
    if (c4 == 0) a.lse[(size_t)b * a.heads + head] = wsum > 0.0f ? (mx + __builtin_amdgcn_logf(wsum)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- the kernel

template <int NSPLIT, bool Q_FP8>
__global__ void __launch_bounds__(kThreads, 1) mla_decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char ring_mem[4 * kSlotBytes];  // KV ring, 4 x 36 KB
  __shared__ __attribute__((aligned(16))) f32x4 xbuf[kWaves * 4 * 64];  // partial S^T exchange, 16 KB
  // the epilogue's "last piece" flag reuses the exchange buffer: it is written
  // after a barrier that all waves reach only once their last slot is done
  volatile int& xlast = *(int*)xbuf;
  lds_char* const ring = (lds_char*)ring_mem;
  LDS_AS f32x4* const xch = (LDS_AS f32x4*)xbuf;

  constexpr int KS = kKSteps / NSPLIT;
  constexpr int NCB = 16 / NSPLIT;
  constexpr int HG = kWaves / NSPLIT;  // 32-head groups per workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = w / NSPLIT, part = w % NSPLIT;

  // workgroup -> (range, head slab); the slabs of a range sit 8 ids apart so
  // they land on the same XCD.
  const int g = blockIdx.x;
  // sequences with nothing to attend: O = 0, LSE = -inf (spread over the grid)
  for (int b = g; b < a.batch; b += gridDim.x) {
    if (units_of(a, b) == 0) {
      for (int i = tid; i < a.heads * (kDV / 4); i += kThreads)
        *(bf16x4*)((__bf16*)a.out + ((size_t)b * a.heads) * kDV + 4 * i) = bf16x4{};
      for (int i = tid; i < a.heads; i += kThreads) a.lse[(size_t)b * a.heads + i] = -INFINITY;
    }
  }
  const int r = (g / (8 * a.slabs)) * 8 + (g % 8);
  const int slab = (g / 8) % a.slabs;
  if (r >= a.ranges) return;

  Plan pl;
  if (!make_plan(a, r, (int*)ring_mem, pl)) return;

  const int head = slab * (HG * 32) + hg * 32 + (lane & 31);
  const bool head_ok = head < a.heads;

  LaneTables<NSPLIT> tab;
  make_tables<NSPLIT>(tab, lane, w, part);

  int b = pl.b0, p = pl.p0;
  bool first_seg = true;
  while (true) {
    const int n = units_of(a, b);
    const int gs = max(pl.start, p), ge = min(pl.end, p + n);
    if (gs < ge) {
      // ---- one segment: sequence b, units [gs - p, ge - p)
      if (!first_seg) {
        // every wave is done with the ring and its stores before it is refilled
        wait_vm_lgkm0<0>();
        barrier();
      }
      first_seg = false;
      const int seqlen = min(max(a.seqlens[b], 0), a.max_pages * kPage);
      SegCtx sg;
      sg.tok0 = (gs - p) * kPage;
      sg.tok1 = min((ge - p) * kPage, seqlen);
      sg.nslots = (sg.tok1 - sg.tok0 + kTS - 1) / kTS;
      sg.npages = (sg.nslots + 1) / 2;
      sg.bt_seg = a.block_table + (size_t)b * a.max_pages + (gs - p);
      const int first_r = p / pl.C, last_r = (p + n - 1) / pl.C;
      const int nsplit = last_r - first_r + 1;

      // query fragments (B operand of S^T = K.Q^T): head `head`, columns
      // 16*ks + 8*(lane/32) .. +7 for this wave's k-steps
      bf16x8 qf[KS];
      if constexpr (!Q_FP8) {
        const bf16x8* qrow = (const bf16x8*)((const __bf16*)a.q + ((size_t)b * a.heads + (head_ok ? head : 0)) * kD);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const bf16x8 v = qrow[2 * (part * KS + i) + (lane >> 5)];
          qf[i] = head_ok ? v : bf16x8{};
        }
      } else {
        const uint2* qrow = (const uint2*)((const uint8_t*)a.q + ((size_t)b * a.heads + (head_ok ? head : 0)) * kD);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const uint2 v = qrow[2 * (part * KS + i) + (lane >> 5)];
          qf[i] = head_ok ? fp8x8_to_bf16(v, a.q_descale) : bf16x8{};
        }
      }

      PageCache pc;
      page_cache_load(pc, sg.bt_seg, 0, sg.npages, lane);
      // query and block-table loads complete before any DMA is issued, so the
      // ring's vmcnt accounting counts DMA only
      wait_vm_lgkm0<0>();

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
        // prologue DMA: slots 0..2
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          if (s < sg.nslots) {
            const int tk = sg.tok0 + s * kTS;
            const int page = page_of(pc, sg.bt_seg, s >> 1, sg.npages, lane, a.num_pages);
            const char* src = a.kv + ((size_t)page * kPage + (s & 1) * kTS) * kRowBytes;
            dma_slot<NSPLIT>(ring + s * kSlotBytes, src, min(kTS, sg.tok1 - tk), tab, w);
          }
        }
        for (int s = 0; s < sg.nslots; ++s) ring_step<NSPLIT>(s, ring, xch, a, sg, pc, qf, tab, st, acc, lane, w);
        // workgroup vote on a redo (every wave is past its last exchange read)
        wait_vm_lgkm0<0>();
        barrier();
        const int my_vote = __any(st.m_seen > st.m_ref + kTau) ? 1 : 0;  // all lanes vote
        if (lane == 0) ((volatile int*)xbuf)[w] = my_vote;
        wait_vm_lgkm0<0>();
        barrier();
        const int vote = ((volatile int*)xbuf)[0] | ((volatile int*)xbuf)[1] | ((volatile int*)xbuf)[2] |
                         ((volatile int*)xbuf)[3];
        wait_vm_lgkm0<0>();
        barrier();  // votes read before the buffer is reused
        if (!__builtin_amdgcn_readfirstlane(vote)) break;
        st.m_ref = st.m_seen;
        if (sg.npages > 64) page_cache_load(pc, sg.bt_seg, 0, sg.npages, lane);
      }

      // ---- epilogue: normalise and store this wave's columns (final output,
      // or this piece's partial in its workspace slot)
      const float l_tot = st.l_sum + __shfl_xor(st.l_sum, 32);
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const float lse2 = l_tot > 0.0f ? st.m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
      if (head_ok) {
        const size_t pslot = (size_t)(b + r);
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
            if (nsplit == 1) *(bf16x4*)(orow + col) = __builtin_convertvector(v, bf16x4);
            else *(f32x4*)(prow + col) = v;
          }
        }
        if (part == 0 && lane < 32) {
          if (nsplit == 1) a.lse[(size_t)b * a.heads + head] = lse2 * kLn2;
          else a.ws_lse[pslot * a.heads + head] = lse2;
        }
      }
      if (nsplit > 1) {
        // publish this piece; the last of the nsplit pieces merges them
        __threadfence();
        __syncthreads();
        int* cnt = a.ws_count + (size_t)b * a.slabs + slab;
        if (tid == 0) xlast = atomicAdd(cnt, 1) == nsplit - 1;
        __syncthreads();
        if (xlast) {
          __threadfence();
          merge_pieces<HG * 32>(a, b, slab, b + first_r, nsplit);
          if (tid == 0) *cnt = 0;
        }
      }
    }
    p += n;
    ++b;
    if (p >= pl.end || b >= a.batch) break;
  }
}

int nsplit_for_heads(int heads) { return heads > 32 ? 2 : 4; }
int slabs_for_heads(int heads) { return heads > 64 ? 2 : 1; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__global__ void mla_zero_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

int32_t decode_ranges(int32_t cus, int32_t batch, int32_t max_pages, int32_t topk, int32_t heads) {
  const int64_t units = (int64_t)batch * (topk > 0 ? (topk + kPage - 1) / kPage : max_pages);
  int64_t r = cus / slabs_for_heads(heads);
  if (r > units) r = units;
  if (r < 1) r = 1;
  return (int32_t)r;
}

// Workspace: [B][slabs] int counters | [(ranges + B)][H] fp32 LSE | [(ranges + B)][H][512] fp32 O.
size_t decode_workspace_bytes(int32_t ranges, int32_t batch, int32_t heads) {
  const size_t slots = (size_t)ranges + (size_t)batch;
  return align256(sizeof(int) * (size_t)batch * slabs_for_heads(heads)) + align256(sizeof(float) * slots * heads) +
         align256(sizeof(float) * slots * heads * kDV);
}

hipError_t init_decode_workspace(void* workspace, int32_t batch, int32_t heads, hipStream_t stream) {
  const int n = batch * slabs_for_heads(heads);
  hipLaunchKernelGGL(mla_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, (int*)workspace, n);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream) {
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
  const size_t slots = (size_t)d.ranges + (size_t)d.batch;
  a.ws_count = (int*)ws;
  ws += align256(sizeof(int) * (size_t)d.batch * a.slabs);
  a.ws_lse = (float*)ws;
  ws += align256(sizeof(float) * slots * d.heads);
  a.ws_o = (float*)ws;
  a.batch = d.batch;
  a.heads = d.heads;
  a.num_pages = d.num_pages;
  a.max_pages = d.max_pages;
  a.topk = d.topk;
  a.ranges = d.ranges;
  a.scale_log2 = d.softmax_scale * kLog2e;
  a.q_descale = d.q_descale;

  if (d.kv_fp8 || d.topk > 0) return hipErrorNotSupported;
  // the slabs of a range are 8 workgroup ids apart: round the grid up to that
  const int groups = (d.ranges + 7) / 8;
  const dim3 grid(groups * 8 * a.slabs), block(kThreads);
  if (nsplit_for_heads(d.heads) == 2) {
    if (d.q_fp8) hipLaunchKernelGGL((mla_decode_bf16_kernel<2, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((mla_decode_bf16_kernel<2, false>), grid, block, 0, stream, a);
  } else {
    if (d.q_fp8) hipLaunchKernelGGL((mla_decode_bf16_kernel<4, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((mla_decode_bf16_kernel<4, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
