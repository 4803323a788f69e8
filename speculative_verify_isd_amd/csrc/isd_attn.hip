// isd_paged_attn: strictly causal GQA attention of the 2N-1 ISD step rows
// over a paged KV cache, for gfx950 (CDNA4).
//
// What the step computes (per sequence b, KV head h, step row r and query
// head g of the group): o = sum_{t <= pos_r} softmax_t(q.k_t / sqrt(D)) v_t
// with pos_r = ctx_b - R + r.  Strict causality over every position and the
// 2N-1 queries per forward are from "Introspective Diffusion Language
// Models" (sections "Training", "Serving (SGLang)" and "How do DLMs perform
// as they approach compute-bound?"); the paged cache is from "Serving
// (SGLang)".
//
// Work decomposition (bf16 path)
//   The batch's KV is a list of units, one per (sequence b, KV head h, page),
//   in (b, h, page) order.  A persistent grid of wave-lanes splits that list
//   into equal contiguous runs, so every lane streams the same number of
//   pages whatever the context mix.  A run crosses (b, h) pairs: each piece
//   of a pair is a segment.  A segment that covers its whole pair writes the
//   final output; a partial one writes its softmax state (m, l, O) to one of
//   the lane's two slots (a partial segment can only be a lane's first or
//   last), and attn_merge_kernel combines the pieces in unit order.  Run
//   boundaries depend only on the sizes, so results do not depend on timing.
//
//   All R*G query rows of a pair share every K/V page, so each page is read
//   once and reused across the query tile: a wave carries RB 16-row MFMA
//   blocks (rows r*G + g on the MFMA N side): 32 rows for R*G <= 32, else
//   64.  For R*G > 64, WR = 2 waves of a work-group walk the same run, one
//   64-row group each; otherwise the 4 waves are 4 independent lanes.  The
//   HBM rate follows the number of independent runs, so rows go to as few
//   waves per run as the registers allow.
//
//   Per page (16 tokens) and 16-row block a wave runs
//     S^T[tok][row] = K[tok][:] . Q[row][:]   (D/32 x mfma_f32_16x16x32_bf16)
//     weights 2^(S c - m) against the segment's reference max m
//     O^T[d][row]  += V^T[d][tok] . P^T[tok][row]  (D/16 x mfma_f32_16x16x16_bf16)
//   The S^T accumulator layout is exactly the B-operand layout P^T needs,
//   and O^T keeps rows in lanes, so the softmax moves no data except two
//   row-swap permutes for the first page's max.
//
//   The page layout is chosen for these operands: each K fragment load is a
//   contiguous 1 KiB per wave (16 B per lane) and each V^T fragment load a
//   contiguous 512 B, so pages stream straight into VGPRs.  A ring of page
//   buffers keeps several pages' loads in flight while one page computes
//   (the query fragments live in LDS to leave registers to the ring); page
//   ids are wave-uniform loads.
#include <hip/hip_runtime.h>

#include <atomic>
#include <math.h>

#include "isd_internal.hpp"

namespace idlm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

struct AttnArgs {
  const void* q;
  const void* kv;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  void* out;
  float* part_o;    // [2 * max_lanes][ROWS][D]: two slots per wave-lane
  float2* part_ml;  // [2 * max_lanes][ROWS]
  int32_t* status;
  int B, R, Hq, Hkv, G, RG, D, max_pages, num_pages;
  int nlanes;       // wave-lanes of the streaming grid
  int mslices;      // merge work-groups per pair: 1, or one per kMergeRows query rows
  float scale_log2;  // log2(e) / sqrt(D)
};

__device__ inline u16 f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  // NaN stays NaN (quiet, sign kept); the bias below would carry a NaN
  // whose payload sits in the low half into infinity or zero.
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u16)(((u >> 16) & 0x8000u) | 0x7FC0u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

// Status bits may be set from any XCD; the XCDs' L2 caches are not coherent
// with each other, so the OR is done at system scope (at memory).
__device__ inline void flag(int32_t* status, int32_t bit) {
  __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Context length clamped to [R, 16*max_pages]; `report` sets the status bit
// when it had to clamp.
__device__ inline int clamp_ctx(const AttnArgs& a, int ctx, bool report) {
  const int hi = kPage * a.max_pages;
  if (ctx < a.R || ctx > hi) {
    if (report) flag(a.status, kBadCtx);
    ctx = ctx < a.R ? a.R : hi;
  }
  return ctx;
}

__device__ inline int pages_of(int ctx) { return (ctx + kPage - 1) / kPage; }

// Read-only loads of wave-uniform addresses through the constant address
// space, so they are scalar-cache loads (counted apart from the vector
// loads the K/V pipeline waits on).
typedef const int32_t __attribute__((address_space(4)))* cint_ptr;
__device__ inline int sload(const int32_t* p, size_t i) { return ((cint_ptr)p)[i]; }

// Marks a wave-uniform value as such, so address arithmetic built from it
// stays scalar and its loads go through the scalar cache.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uni64(int64_t x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(uint64_t)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// bf16 MFMA building blocks
// ---------------------------------------------------------------------------

// K and V^T fragments of one page for one wave (32 registers).
template <int D>
struct PageFrag {
  bf16x8 k[D / 32];  // A operand of S^T = K Q^T: token lane%16, d chunk 4c + lane/16
  s16x4 v[D / 16];   // A operand of O^T += V^T P^T: d = 16j + lane%16, tokens 4(lane/16)+0..3
};

// Issue one page's loads.  K: one contiguous 1 KiB per 32-wide d step (16 B
// per lane); V^T: one contiguous 512 B per 16-wide d block (8 B per lane).
// A page read by one wave only is read once per step, so those loads are
// non-temporal (NT): on gfx950 that streams them past the caches and
// sustains ~13% more HBM bandwidth than ordinary loads.  When two waves
// share a run each page is read twice, close together; ordinary loads let
// the second read hit in L2 (non-temporal ones fetched ~9% more from HBM).
template <int D, bool NT>
__device__ inline void load_page(PageFrag<D>& f, const u16* kv, size_t v_off, int lane) {
  constexpr int NC = D / 32, ND = D / 16;
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const u32x4* pk = (const u32x4*)(kv + 512 * c + 8 * lane);
    f.k[c] = __builtin_bit_cast(bf16x8, NT ? __builtin_nontemporal_load(pk) : *pk);
  }
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const u32x2* pv = (const u32x2*)(kv + v_off + (size_t)(16 * j + col) * kPage + 4 * grp);
    f.v[j] = __builtin_bit_cast(s16x4, NT ? __builtin_nontemporal_load(pv) : *pv);
  }
}

// Max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap permutes (no LDS round trip).
__device__ inline float max_over_rows(float v) {
  const unsigned b = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const unsigned c = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// The softmax of a segment is taken against a fixed reference max per row
// (log2 units): the row max of the segment's first page.  Later pages never
// rescale the accumulators (a rescale branch in the page loop costs register
// copies on every page), so a weight 2^(s - m) exceeds 1 when a later score
// beats the first page.  A lane whose partial row sum passes kRefBound = 2^24
// (which every weight that large forces) sends the segment to a slow path: a
// sweep for the true row max, then the segment again with that max as the
// reference, where no weight exceeds 1.  Below that bound no weight, sum or
// accumulator can overflow, and the final normalisation and the merge use
// the same reference, so the result does not depend on which one was taken.
constexpr float kRefBound = (float)(1 << 24);

__device__ inline float max4(const f32x4& v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }

// S^T = K Q^T of one page for the 16-row blocks h0, h0 + 1 (mfma
// 16x16x32).  MASKED sets the scores of tokens past a row's position (all
// of them when !has, a padding step) to -inf.
template <int D, int RB, bool MASKED>
__device__ inline void scores_pair(const PageFrag<D>& f, const bf16x8* qs, int lane, int h0,
                                   const int (&pos)[RB], int t, bool has, f32x4 (&sc)[2]) {
  constexpr int NC = D / 32;
  // Query fragments come from this wave's LDS copy (registers are kept for
  // the K/V pipeline).
  bf16x8 qf[2][NC];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[i][c] = qs[((h0 + i) * NC + c) * 64 + lane];
#pragma unroll
  for (int i = 0; i < 2; ++i) sc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      sc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[c], qf[i][c], sc[i], 0, 0, 0);
  if (MASKED) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[i][e] = (has && t + e <= pos[h0 + i]) ? sc[i][e] : -INFINITY;
  }
}

// Weights p = 2^(s c2 - m) of the blocks h0, h0 + 1, their row sums, and
// O^T += V^T P^T (mfma 16x16x16: the S^T accumulator is already P^T's
// B-operand layout).
template <int D, int RB>
__device__ inline void accumulate_pair(const PageFrag<D>& f, int h0, const f32x4 (&sc)[2],
                                       float c2, const float (&mneg)[RB], float (&l)[RB],
                                       f32x4 (&acc)[RB][D / 16]) {
  constexpr int ND = D / 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rb = h0 + i;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[i][e], c2, mneg[rb]));
    l[rb] += (p[0] + p[1]) + (p[2] + p[3]);
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 lo = __builtin_convertvector((f32x2){p[0], p[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2){p[2], p[3]}, bf16x2);
    const s16x4 pf = __builtin_bit_cast(s16x4, (u32x2){__builtin_bit_cast(unsigned, lo),
                                                        __builtin_bit_cast(unsigned, hi)});
#pragma unroll
    for (int j = 0; j < ND; ++j)
      acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(f.v[j], pf, acc[rb][j], 0, 0, 0);
  }
}

// One page (16 tokens) for all RB row blocks of this wave, two blocks at a
// time (a scheduling barrier between the pairs keeps their temporaries from
// being live together, so 64-row waves fit in registers at D = 128).  FIRST
// marks a segment's first page: with set_ref it takes the rows' max over
// this page as the reference m (mneg = -m, or 0 for a row with nothing
// visible).
template <int D, int RB, bool MASKED, bool FIRST>
__device__ inline void compute_page(const PageFrag<D>& f, const bf16x8* qs, int lane,
                                    const int (&pos)[RB], int t, bool has, float c2, bool set_ref,
                                    float (&m)[RB], float (&mneg)[RB], float (&l)[RB],
                                    f32x4 (&acc)[RB][D / 16]) {
  static_assert(RB % 2 == 0, "row blocks go in pairs");
#pragma unroll
  for (int h0 = 0; h0 < RB; h0 += 2) {
    if (h0 > 0) __builtin_amdgcn_sched_barrier(0);
    f32x4 sc[2];
    scores_pair<D, RB, MASKED>(f, qs, lane, h0, pos, t, has, sc);
    if (FIRST && set_ref) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rb = h0 + i;
        m[rb] = max_over_rows(max4(sc[i])) * c2;
        mneg[rb] = m[rb] == -INFINITY ? 0.f : -m[rb];
      }
    }
    accumulate_pair<D, RB>(f, h0, sc, c2, mneg, l, acc);
  }
}

// Slow path: the lane-local max of one page's raw scores, folded into mloc.
template <int D, int RB, bool MASKED>
__device__ inline void max_page(const PageFrag<D>& f, const bf16x8* qs, int lane,
                                const int (&pos)[RB], int t, bool has, float (&mloc)[RB]) {
#pragma unroll
  for (int h0 = 0; h0 < RB; h0 += 2) {
    f32x4 sc[2];
    scores_pair<D, RB, MASKED>(f, qs, lane, h0, pos, t, has, sc);
#pragma unroll
    for (int i = 0; i < 2; ++i) mloc[h0 + i] = fmaxf(mloc[h0 + i], max4(sc[i]));
  }
}

// Finds the sequence holding unit u with a wave-wide scan over ctx_lens;
// returns it with its first unit in *ub and its clamped context in *ctx_out.
// Every lane returns the same values.
__device__ inline int locate_seq(const AttnArgs& a, int64_t u, int64_t* ub, int* ctx_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int blk = 0; blk * 64 < a.B; ++blk) {
    const int b = blk * 64 + lane;
    const int ctx = b < a.B ? clamp_ctx(a, a.ctx_lens[b], false) : a.R;
    const int64_t units = b < a.B ? (int64_t)pages_of(ctx) * a.Hkv : 0;
    int64_t incl = units;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int64_t total = __shfl(incl, 63);
    if (u < base + total) {
      const int64_t excl = incl - units;
      const unsigned long long hit = __ballot(base + excl <= u && u < base + incl);
      const int src = __ffsll((long long)hit) - 1;
      *ub = base + __shfl(excl, src);
      *ctx_out = __shfl(ctx, src);
      return blk * 64 + src;
    }
    base += total;
  }
  *ub = base;
  *ctx_out = a.R;
  return a.B;
}

// Total units of the batch (same clamping as the kernels), on every lane.
__device__ inline int64_t total_units_wave(const AttnArgs& a) {
  const int lane = threadIdx.x & 63;
  int64_t s = 0;
  for (int b = lane; b < a.B; b += 64)
    s += (int64_t)pages_of(clamp_ctx(a, a.ctx_lens[b], false)) * a.Hkv;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  return s;
}

// Units per lane: equal contiguous runs of at least kMinRunPages.
__device__ inline int64_t run_length(int64_t total, int nlanes) {
  const int64_t r = (total + nlanes - 1) / nlanes;
  return r < kMinRunPages ? kMinRunPages : r;
}

// ---------------------------------------------------------------------------
// bf16 streaming kernel
// ---------------------------------------------------------------------------
template <int D, int WR, int RB>
__global__ __launch_bounds__(256) void attn_stream_kernel(AttnArgs a) {
  constexpr int kRing = D == 128 ? kRingPages : kRingPages + 2;  // page buffers per wave
  constexpr int NC = D / 32;  // K-dim steps of the QK product
  constexpr int ND = D / 16;  // 16-wide d blocks of the PV product
  constexpr int WROWS = 16 * RB;  // query rows of one wave
  constexpr int ROWS = WROWS * WR;  // query rows of a run

  __shared__ bf16x8 lds_q[4][RB * NC * 64];  // each wave's query fragments

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rgrp = wave % WR;  // row group of this wave within its run
  // Wave-lanes are numbered across work-groups first (lane = slot in the
  // work-group * grid + work-group), so a batch with few busy lanes spreads
  // them over every CU (B = 1: 256 busy lanes on 256 CUs instead of 64;
  // 23.4 -> 21.6 us).
  const int wl = (wave / WR) * gridDim.x + blockIdx.x;  // this wave-lane
  bf16x8* qs = lds_q[wave];
  const int col = lane & 15, grp = lane >> 4;

  // Bad contexts are flagged once, by the first wave of the grid.
  if (blockIdx.x == 0 && wave == 0)
    for (int b = lane; b < a.B; b += 64) clamp_ctx(a, a.ctx_lens[b], true);

  const int64_t total = uni64(total_units_wave(a));
  const int64_t span = run_length(total, a.nlanes);

  const u16* qb = (const u16*)a.q;
  const u16* kvb = (const u16*)a.kv;
  const size_t page_elems = (size_t)2 * a.Hkv * kPage * D;
  const size_t v_off = (size_t)a.Hkv * kPage * D;
  u16* outp = (u16*)a.out;

  float m[RB], l[RB];
  f32x4 acc[RB][ND];

  // Streams pages [p0, p1) of pair (b, h) into (m, l, acc), starting from an
  // empty state: m is the softmax reference (log2 units), l and acc are
  // relative to it.
  auto stream = [&](int b, int h, int ctx, int p0, int p1) __attribute__((always_inline)) {
    const size_t head_off = (size_t)h * kPage * D;
    const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
    // Query fragments (B operand of S^T = K Q^T): row = lane's column, eight
    // consecutive d per lane; k-step c covers d chunk 4c + grp.  Staged in
    // this wave's LDS slot; a wave's own LDS accesses stay in order.
    int pos[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = rgrp * WROWS + rb * 16 + col;
      const bool valid = i < a.RG;
      const int r = valid ? i / a.G : a.R - 1;
      const int g = valid ? i % a.G : 0;
      pos[rb] = ctx - a.R + r;
      const u16* qp = qb + (((size_t)b * a.R + r) * a.Hq + (size_t)h * a.G + g) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {  // padding rows load a real row, then zero it
        uint4 v = *(const uint4*)(qp + 8 * (4 * c + grp));
        if (!valid) v = make_uint4(0, 0, 0, 0);
        qs[(rb * NC + c) * 64 + lane] = __builtin_bit_cast(bf16x8, v);
      }
    }
    const float c2 = a.scale_log2;
    float mneg[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m[rb] = -INFINITY;
      mneg[rb] = 0.f;
      l[rb] = 0.f;
#pragma unroll
      for (int j = 0; j < ND; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int cnt = p1 - p0;
    // One page per step through a ring of kRing register buffers: kRing-1
    // pages are in flight while one computes.  Every prefetch is issued
    // unconditionally (so the compiler waits for exactly one buffer at a
    // time); prefetches past the end re-read the last page (a cache hit) and
    // their compute is fully masked.  The scheduling barriers keep each
    // prefetch ahead of the compute it must overlap.  Page q sits in buffer
    // q % kRing.
    const int last = cnt - 1;
    const int nrun = 1 + ((cnt - 1 + kRing - 1) / kRing) * kRing;  // steps, first page included
    const int minpos = ctx - a.R;  // every row sees tokens up to here
    auto issue = [&](PageFrag<D>& f, int st) __attribute__((always_inline)) {
      const int pg = p0 + min(st, last);
      int id = sload(pt, pg);
      if ((unsigned)id >= (unsigned)a.num_pages) {
        flag(a.status, kBadPage);
        id = 0;
      }
      load_page<D, (WR == 1)>(f, kvb + (size_t)id * page_elems + head_off, v_off, lane);
    };
    // Pass 0 takes its reference from the first page; pass 1 (the slow path)
    // runs only after a max sweep has set the reference to the true row max.
    for (int pass = 0; pass < 2 && cnt > 0; ++pass) {
      const bool set_ref = pass == 0;
      if (pass == 1) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          l[rb] = 0.f;
#pragma unroll
          for (int j = 0; j < ND; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      auto run = [&](const PageFrag<D>& f, int st) __attribute__((always_inline)) {
        const int t0 = (p0 + st) * kPage;
        const bool has = st < cnt;
        if (has && t0 + kPage - 1 <= minpos)
          compute_page<D, RB, false, false>(f, qs, lane, pos, t0 + 4 * grp, true, c2, false, m,
                                            mneg, l, acc);
        else
          compute_page<D, RB, true, false>(f, qs, lane, pos, t0 + 4 * grp, has, c2, false, m,
                                           mneg, l, acc);
      };
      PageFrag<D> ring[kRing];
#pragma unroll
      for (int i = 0; i < kRing; ++i) issue(ring[i], i);
      __builtin_amdgcn_sched_barrier(0);
      {  // the first page sets the reference
        const int t0 = p0 * kPage;
        if (t0 + kPage - 1 <= minpos)
          compute_page<D, RB, false, true>(ring[0], qs, lane, pos, t0 + 4 * grp, true, c2, set_ref,
                                           m, mneg, l, acc);
        else
          compute_page<D, RB, true, true>(ring[0], qs, lane, pos, t0 + 4 * grp, true, c2, set_ref,
                                          m, mneg, l, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
      for (int st = 1; st < nrun; st += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) {
          issue(ring[i], st + i + kRing - 1);
          __builtin_amdgcn_sched_barrier(0);
          run(ring[(i + 1) % kRing], st + i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      bool over = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) over = over || !(l[rb] <= kRefBound);
      if (pass == 1 || !__any(over)) break;
      // Slow path: the true row max of the segment, then the segment again.
      float mloc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) mloc[rb] = -INFINITY;
      for (int st = 0; st < cnt; ++st) {
        PageFrag<D> f;
        issue(f, st);
        const int t0 = (p0 + st) * kPage;
        max_page<D, RB, true>(f, qs, lane, pos, t0 + 4 * grp, true, mloc);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        m[rb] = max_over_rows(mloc[rb]) * c2;
        mneg[rb] = m[rb] == -INFINITY ? 0.f : -m[rb];
      }
    }
    // Row sums: every lane holds a partial over its tokens.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l[rb] += __shfl_xor(l[rb], 16);
      l[rb] += __shfl_xor(l[rb], 32);
    }
  };

  // Final rows of pair (b, h): lane holds O^T[16j + 4grp + e][row col].
  auto write_out = [&](int b, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = rgrp * WROWS + rb * 16 + col;
      if (i < a.RG) {
        const int r = i / a.G, g = i % a.G;
        const float il = 1.f / l[rb];
        u16* op = outp + (((size_t)b * a.R + r) * a.Hq + (size_t)h * a.G + g) * D + 4 * grp;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
          const unsigned lo = f32_to_bf16_rne(acc[rb][j][0] * il) |
                              ((unsigned)f32_to_bf16_rne(acc[rb][j][1] * il) << 16);
          const unsigned hi = f32_to_bf16_rne(acc[rb][j][2] * il) |
                              ((unsigned)f32_to_bf16_rne(acc[rb][j][3] * il) << 16);
          *(uint2*)(op + 16 * j) = make_uint2(lo, hi);
        }
      }
    }
  };
  // Softmax state of a piece of a pair, for attn_merge_kernel.
  auto write_part = [&](size_t slot) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = rgrp * WROWS + rb * 16 + col;
      float* po = a.part_o + (slot * ROWS + row) * D + 4 * grp;
#pragma unroll
      for (int j = 0; j < ND; ++j)
        *(float4*)(po + 16 * j) =
            make_float4(acc[rb][j][0], acc[rb][j][1], acc[rb][j][2], acc[rb][j][3]);
      if (grp == 0) a.part_ml[slot * ROWS + row] = make_float2(m[rb], l[rb]);
    }
  };
  // This lane's run, pair by pair; slots slot0 + 0 / + 1 hold its first /
  // last piece when those are partial.
  auto walk = [&](int64_t u, int64_t uend, size_t slot0) __attribute__((always_inline)) {
    int64_t ub;
    int ctx;
    int b = locate_seq(a, u, &ub, &ctx);
    b = uni(b);
    ub = uni64(ub);
    ctx = uni(ctx);
    int np = pages_of(ctx);
    int h = (int)((u - ub) / np);
    bool first = true;
    while (u < uend) {
      const int64_t pair_start = ub + (int64_t)h * np;
      const int p0 = (int)(u - pair_start);
      const int p1 = (int)min<int64_t>(np, p0 + (uend - u));
      const bool whole = (p0 == 0 && p1 == np);
      stream(b, h, ctx, p0, p1);
      if (whole)
        write_out(b, h);
      else
        write_part(slot0 + (first ? 0 : 1));
      u += p1 - p0;
      first = false;
      if (u < uend) {
        if (++h == a.Hkv) {
          h = 0;
          ub += (int64_t)np * a.Hkv;
          ++b;
          ctx = uni(clamp_ctx(a, sload(a.ctx_lens, b), false));
          np = pages_of(ctx);
        }
      }
    }
  };

  const int64_t u = (int64_t)wl * span;
  const int64_t uend = min(u + span, total);
  if (u < uend) walk(u, uend, (size_t)wl * 2);
}

constexpr int kMergeRows = 8;  // query rows of a merge slice

// Folds rows [r0, r0 + kMergeRows) of a split pair's pieces (collective over
// the work-group): every piece's (max, sum) for those rows, then the partial
// outputs in unit order, kSBatch pieces' loads at a time.
template <int D, int ROWS>
__device__ void merge_slice(const AttnArgs& a, int b, int h, int r0, int npieces, int wa,
                            int64_t start, int64_t span) {
  constexpr int D4 = D / 4;
  constexpr int kSVec = (kMergeRows * D4 + 255) / 256;  // float4 outputs per thread
  constexpr int kSBatch = 16 / kSVec;
  __shared__ float sm_M[kMergeRows], sm_iL[kMergeRows];
  __shared__ float sm_f[kSBatch][kMergeRows];
  const int tid = threadIdx.x;
  const int nrows = min(kMergeRows, a.RG - r0);
  const int nvec = nrows * D4;
  auto slot_of = [&](int k) -> size_t {
    return (size_t)(wa + k) * 2 + ((k == 0 && start != (int64_t)wa * span) ? 1 : 0);
  };
  auto load_batch = [&](int k0, float4 (&v)[kSBatch][kSVec]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kSBatch; ++t) {
      const int k = min(k0 + t, npieces - 1);  // clamped, unconditional
      const float4* po = (const float4*)(a.part_o + (slot_of(k) * ROWS + r0) * D);
#pragma unroll
      for (int e = 0; e < kSVec; ++e) v[t][e] = po[min(tid + 256 * e, nvec - 1)];
    }
  };
  float4 v[kSBatch][kSVec];
  load_batch(0, v);
  if (tid < nrows) {
    // Row maxima and normalisers, 16 pieces' loads in flight at a time
    // (clamped, unconditional), summed in unit order.
    const int row = r0 + tid;
    float M = -INFINITY;
    for (int k0 = 0; k0 < npieces; k0 += 16) {
      float mx[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) mx[j] = a.part_ml[slot_of(min(k0 + j, npieces - 1)) * ROWS + row].x;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (k0 + j < npieces) M = fmaxf(M, mx[j]);
    }
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
    for (int k0 = 0; k0 < npieces; k0 += 16) {
      float2 ml[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) ml[j] = a.part_ml[slot_of(min(k0 + j, npieces - 1)) * ROWS + row];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (k0 + j < npieces) L += ml[j].y * exp2f(ml[j].x - Mu);
    }
    sm_M[tid] = Mu;
    sm_iL[tid] = 1.f / L;
  }
  float4 O[kSVec];
#pragma unroll
  for (int e = 0; e < kSVec; ++e) O[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < npieces; k0 += kSBatch) {
    __syncthreads();  // (M, 1/L) written; the previous batch's factors consumed
    if (k0 > 0) load_batch(k0, v);
    if (tid < nrows) {
      const float Mu = sm_M[tid], iL = sm_iL[tid];
#pragma unroll
      for (int t = 0; t < kSBatch; ++t)
        sm_f[t][tid] = k0 + t < npieces
                           ? exp2f(a.part_ml[slot_of(k0 + t) * ROWS + r0 + tid].x - Mu) * iL
                           : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kSBatch; ++t)
#pragma unroll
      for (int e = 0; e < kSVec; ++e) {
        const int i = min(tid + 256 * e, nvec - 1);
        const float f = sm_f[t][i / D4];
        O[e].x += v[t][e].x * f;
        O[e].y += v[t][e].y * f;
        O[e].z += v[t][e].z * f;
        O[e].w += v[t][e].w * f;
      }
  }
  u16* outp = (u16*)a.out;
#pragma unroll
  for (int e = 0; e < kSVec; ++e) {
    const int i = tid + 256 * e;
    if (i < nvec) {
      const int row = r0 + i / D4, d = 4 * (i % D4);
      const int r = row / a.G, g = row % a.G;
      const unsigned lo = f32_to_bf16_rne(O[e].x) | ((unsigned)f32_to_bf16_rne(O[e].y) << 16);
      const unsigned hi = f32_to_bf16_rne(O[e].z) | ((unsigned)f32_to_bf16_rne(O[e].w) << 16);
      *(uint2*)(outp + (((size_t)b * a.R + r) * a.Hq + (size_t)h * a.G + g) * D + d) =
          make_uint2(lo, hi);
    }
  }
}

// merge_slice for a pair of at most kSlicePieces pieces: every piece's partial
// outputs for the slice and its (max, sum) rows are loaded in one round (one
// (max, sum) per thread), the row maxima, normalisers and scale factors go
// through LDS, and the pieces are folded in unit order with the same
// arithmetic as merge_slice.
constexpr int kSlicePieces = 256 / kMergeRows;

template <int D, int ROWS>
__device__ void merge_slice_one_round(const AttnArgs& a, int b, int h, int r0, int npieces, int wa,
                                      int64_t start, int64_t span) {
  constexpr int D4 = D / 4;
  constexpr int kSVec = (kMergeRows * D4 + 255) / 256;  // float4 outputs per thread
  __shared__ float sf_m[kSlicePieces][kMergeRows], sf_l[kSlicePieces][kMergeRows];
  __shared__ float sf_M[kMergeRows], sf_iL[kMergeRows];
  const int tid = threadIdx.x;
  const int nrows = min(kMergeRows, a.RG - r0);
  const int nvec = nrows * D4;
  auto slot_of = [&](int k) -> size_t {
    return (size_t)(wa + k) * 2 + ((k == 0 && start != (int64_t)wa * span) ? 1 : 0);
  };
  float4 v[kSlicePieces][kSVec];
#pragma unroll
  for (int t = 0; t < kSlicePieces; ++t) {
    const int k = min(t, npieces - 1);  // clamped, unconditional
    const float4* po = (const float4*)(a.part_o + (slot_of(k) * ROWS + r0) * D);
#pragma unroll
    for (int e = 0; e < kSVec; ++e) v[t][e] = po[min(tid + 256 * e, nvec - 1)];
  }
  {
    const int k = tid / kMergeRows, row = tid % kMergeRows;
    const float2 ml = a.part_ml[slot_of(min(k, npieces - 1)) * ROWS + r0 + min(row, nrows - 1)];
    sf_m[k][row] = ml.x;
    sf_l[k][row] = ml.y;
  }
  __syncthreads();
  if (tid < nrows) {
    float M = -INFINITY;
    for (int k = 0; k < npieces; ++k) M = fmaxf(M, sf_m[k][tid]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
    for (int k = 0; k < npieces; ++k) L += sf_l[k][tid] * exp2f(sf_m[k][tid] - Mu);
    sf_M[tid] = Mu;
    sf_iL[tid] = 1.f / L;
  }
  __syncthreads();
  {
    const int k = tid / kMergeRows, row = tid % kMergeRows;
    sf_l[k][row] = exp2f(sf_m[k][row] - sf_M[row]) * sf_iL[row];  // piece k's scale factor
  }
  __syncthreads();
  float4 O[kSVec];
#pragma unroll
  for (int e = 0; e < kSVec; ++e) O[e] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int t = 0; t < kSlicePieces; ++t)
    if (t < npieces) {
#pragma unroll
      for (int e = 0; e < kSVec; ++e) {
        const int i = min(tid + 256 * e, nvec - 1);
        const float f = sf_l[t][i / D4];
        O[e].x += v[t][e].x * f;
        O[e].y += v[t][e].y * f;
        O[e].z += v[t][e].z * f;
        O[e].w += v[t][e].w * f;
      }
    }
  u16* outp = (u16*)a.out;
#pragma unroll
  for (int e = 0; e < kSVec; ++e) {
    const int i = tid + 256 * e;
    if (i < nvec) {
      const int row = r0 + i / D4, d = 4 * (i % D4);
      const int r = row / a.G, g = row % a.G;
      const unsigned lo = f32_to_bf16_rne(O[e].x) | ((unsigned)f32_to_bf16_rne(O[e].y) << 16);
      const unsigned hi = f32_to_bf16_rne(O[e].z) | ((unsigned)f32_to_bf16_rne(O[e].w) << 16);
      *(uint2*)(outp + (((size_t)b * a.R + r) * a.Hq + (size_t)h * a.G + g) * D + d) =
          make_uint2(lo, hi);
    }
  }
}

// Combines the pieces of (b, h) pairs that were split across wave-lane runs,
// in unit order.  a.mslices work-groups per pair: with one, the pair is
// folded whole, kBatch pieces' loads at a time; with one per slice of
// kMergeRows query rows (chosen when few pairs are spread over many runs), a
// pair of more than kBatch pieces is folded slice by slice, so several
// compute units share its pieces, and a pair of at most kBatch pieces is
// still folded whole by its first work-group.  Pairs written whole by one run
// exit at once.
template <int D, int ROWS>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int kMergeVec = (ROWS * D / 4 + 255) / 256;  // float4 outputs per thread
  constexpr int kBatch = kMergeVec < 32 ? 32 / kMergeVec : 1;  // pieces loaded together
  constexpr int kMlHeld = kBatch < 8 ? 8 : kBatch;  // pieces' (max, sum) a row thread holds
  __shared__ int64_t sh_sum[4][2];
  __shared__ float sh_M[ROWS], sh_iL[ROWS];
  __shared__ float sh_f[kBatch][ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.x / a.mslices, slice = blockIdx.x % a.mslices;
  const int b = pair / a.Hkv, h = pair % a.Hkv;

  // Units before sequence b and in the whole batch.
  int64_t before = 0, total = 0;
  for (int s = tid; s < a.B; s += 256) {
    const int64_t units = (int64_t)pages_of(clamp_ctx(a, a.ctx_lens[s], false)) * a.Hkv;
    total += units;
    if (s < b) before += units;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off);
    total += __shfl_xor(total, off);
  }
  if (lane == 0) {
    sh_sum[wave][0] = before;
    sh_sum[wave][1] = total;
  }
  __syncthreads();
  before = sh_sum[0][0] + sh_sum[1][0] + sh_sum[2][0] + sh_sum[3][0];
  total = sh_sum[0][1] + sh_sum[1][1] + sh_sum[2][1] + sh_sum[3][1];
  const int np = pages_of(clamp_ctx(a, a.ctx_lens[b], false));
  const int64_t start = before + (int64_t)h * np;
  const int64_t span = run_length(total, a.nlanes);
  const int wa = (int)(start / span), wb = (int)((start + np - 1) / span);
  if (wa == wb) return;  // one lane held the whole pair and wrote the output

  // Piece k comes from lane wa + k: its run's first segment (slot + 0),
  // except that the pair's first piece is lane wa's last segment (slot + 1)
  // when the pair starts inside that lane's run.
  const int npieces = wb - wa + 1;
  auto slot_of = [&](int k) -> size_t {
    return (size_t)(wa + k) * 2 + ((k == 0 && start != (int64_t)wa * span) ? 1 : 0);
  };
  if (npieces > kBatch && a.mslices > 1) {
    if (kMergeRows * slice < a.RG) {
      if (npieces <= kSlicePieces)
        merge_slice_one_round<D, ROWS>(a, b, h, kMergeRows * slice, npieces, wa, start, span);
      else
        merge_slice<D, ROWS>(a, b, h, kMergeRows * slice, npieces, wa, start, span);
    }
    return;
  }
  if (slice != 0) return;
  // Each thread owns up to kMergeVec 4-wide d groups of the R*G x D output.
  // The first kBatch pieces' partial outputs are loaded before anything
  // waits, together with the pieces' (max, sum) rows, so a pair of up to
  // kBatch pieces costs one round of loads after the lane range.
  constexpr int D4 = D / 4;
  const int nvec = a.RG * D4;
  auto load_batch = [&](int k0, float4 (&v)[kBatch][kMergeVec]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int k = min(k0 + t, npieces - 1);  // clamped, unconditional
      const float4* po = (const float4*)(a.part_o + slot_of(k) * ROWS * D);
#pragma unroll
      for (int e = 0; e < kMergeVec; ++e) v[t][e] = po[min(tid + 256 * e, nvec - 1)];
    }
  };
  float4 v[kBatch][kMergeVec];
  load_batch(0, v);
  // Row maxima and normalisers over all pieces (row threads), the first
  // kMlHeld pieces' (max, sum) kept in registers.
  float2 mlr[kMlHeld];
  if (tid < a.RG) {
#pragma unroll
    for (int j = 0; j < kMlHeld; ++j) mlr[j] = a.part_ml[slot_of(min(j, npieces - 1)) * ROWS + tid];
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMlHeld; ++j)
      if (j < npieces) M = fmaxf(M, mlr[j].x);
    for (int k = kMlHeld; k < npieces; ++k) M = fmaxf(M, a.part_ml[slot_of(k) * ROWS + tid].x);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int j = 0; j < kMlHeld; ++j)
      if (j < npieces) L += mlr[j].y * exp2f(mlr[j].x - Mu);
    for (int k = kMlHeld; k < npieces; ++k) {
      const float2 ml = a.part_ml[slot_of(k) * ROWS + tid];
      L += ml.y * exp2f(ml.x - Mu);
    }
    sh_M[tid] = Mu;
    sh_iL[tid] = 1.f / L;
    // Scale factors of the first batch.
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
      sh_f[t][tid] = t < npieces ? exp2f(mlr[t].x - Mu) * (1.f / L) : 0.f;
  }
  __syncthreads();
  float4 O[kMergeVec];
#pragma unroll
  for (int e = 0; e < kMergeVec; ++e) O[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  // Fold the pieces in unit order, kBatch at a time.
  for (int k0 = 0; k0 < npieces; k0 += kBatch) {
    if (k0 > 0) {
      __syncthreads();  // the previous batch's factors are consumed
      load_batch(k0, v);
      if (tid < a.RG) {
        const float Mu = sh_M[tid], iL = sh_iL[tid];
#pragma unroll
        for (int t = 0; t < kBatch; ++t)
          sh_f[t][tid] = k0 + t < npieces
                             ? exp2f(a.part_ml[slot_of(k0 + t) * ROWS + tid].x - Mu) * iL
                             : 0.f;
      }
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
#pragma unroll
      for (int e = 0; e < kMergeVec; ++e) {
        const int i = min(tid + 256 * e, nvec - 1);
        const float f = sh_f[t][i / D4];
        O[e].x += v[t][e].x * f;
        O[e].y += v[t][e].y * f;
        O[e].z += v[t][e].z * f;
        O[e].w += v[t][e].w * f;
      }
  }
  u16* outp = (u16*)a.out;
#pragma unroll
  for (int e = 0; e < kMergeVec; ++e) {
    const int i = tid + 256 * e;
    if (i < nvec) {
      const int row = i / D4, d = 4 * (i % D4);
      const int r = row / a.G, g = row % a.G;
      const unsigned lo = f32_to_bf16_rne(O[e].x) | ((unsigned)f32_to_bf16_rne(O[e].y) << 16);
      const unsigned hi = f32_to_bf16_rne(O[e].z) | ((unsigned)f32_to_bf16_rne(O[e].w) << 16);
      *(uint2*)(outp + (((size_t)b * a.R + r) * a.Hq + (size_t)h * a.G + g) * D + d) =
          make_uint2(lo, hi);
    }
  }
}

// ---------------------------------------------------------------------------
// float32 FMA path: one work-group per (b, kv head); each wave takes query
// rows in turn and walks the context with lanes over d.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int E = D / 64;  // d values per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.x;
  const int b = pair / a.Hkv, kvh = pair % a.Hkv;
  const int ctx = clamp_ctx(a, a.ctx_lens[b], tid == 0 && kvh == 0);
  const float* qf = (const float*)a.q;
  const float* kv = (const float*)a.kv;
  float* outp = (float*)a.out;
  const size_t page_elems = (size_t)2 * a.Hkv * kPage * D;
  const size_t head_off = (size_t)kvh * kPage * D;
  const size_t v_off = (size_t)a.Hkv * kPage * D;
  const float scale = a.scale_log2;
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;

  for (int i = wave; i < a.RG; i += 4) {
    const int r = i / a.G, g = i % a.G;
    const int pos = ctx - a.R + r;
    const size_t qo = (((size_t)b * a.R + r) * a.Hq + (size_t)kvh * a.G + g) * D;
    float qv[E], o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      qv[e] = qf[qo + lane + 64 * e];
      o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int t = 0; t <= pos; ++t) {
      int phys = pt[t / kPage];
      if ((unsigned)phys >= (unsigned)a.num_pages) {
        flag(a.status, kBadPage);
        phys = 0;
      }
      const int s = t % kPage;
      const float* blk = kv + (size_t)phys * page_elems + head_off;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = lane + 64 * e;
        dot += qv[e] * blk[((d >> 2) * kPage + s) * 4 + (d & 3)];
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
      const float x = dot * scale;
      const float mn = fmaxf(m, x);
      const float alpha = exp2f(m - mn);
      const float p = exp2f(x - mn);
      l = l * alpha + p;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = lane + 64 * e;
        o[e] = o[e] * alpha + p * blk[v_off + (size_t)d * kPage + s];
      }
      m = mn;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) outp[qo + lane + 64 * e] = o[e] / l;
  }
}

// Work-groups the streaming kernel keeps resident on this device (queried
// once per device, cached in an atomic so concurrent first calls from
// several host threads are well defined; devices past the cache are queried
// every time): every CU times the kernel's occupancy.
template <int D, int WR, int RB>
int stream_grid(int device) {
  static std::atomic<int> cached[64];
  const bool cache = device >= 0 && device < 64;
  if (cache) {
    const int g = cached[device].load(std::memory_order_relaxed);
    if (g) return g;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_stream_kernel<D, WR, RB>, 256, 0) !=
          hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  int g = cus * per_cu;
  const int cap = kMaxWaves / 4;
  if (g > cap) g = cap;
  if (cache) cached[device].store(g, std::memory_order_relaxed);
  return g;
}

template <int D, int WR, int RB>
int32_t launch_stream(AttnArgs a, hipStream_t s) {
  constexpr int ROWS = 16 * RB * WR;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return IDLM_ERR_HIP;
  const int grid = stream_grid<D, WR, RB>(dev);
  a.nlanes = grid * (4 / WR);
  hipLaunchKernelGGL((attn_stream_kernel<D, WR, RB>), dim3(grid), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  // Slices only while they fit in one round of resident work-groups (two per
  // CU): otherwise every early-exiting slice costs a round of its own.
  const int slices = ROWS / kMergeRows;
  a.mslices = (int64_t)a.B * a.Hkv * slices <= 2 * 256 ? slices : 1;
  hipLaunchKernelGGL((attn_merge_kernel<D, ROWS>), dim3(a.B * a.Hkv * a.mslices), dim3(256), 0, s,
                     a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

}  // namespace

int32_t launch_paged_attn(const idlm_isd_dims& d, const Plan& p, const void* q, const void* kv,
                          const int32_t* page_table, const int32_t* ctx_lens, void* out,
                          char* ws, hipStream_t s) {
  const AttnPlan& ap = p.attn;
  if (d.B == 0) return IDLM_OK;
  AttnArgs a;
  a.q = q;
  a.kv = kv;
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.out = out;
  a.part_o = (float*)(ws + p.off_attn_o);
  a.part_ml = (float2*)(ws + p.off_attn_ml);
  a.status = (int32_t*)(ws + p.off_status);
  a.B = d.B;
  a.R = ap.R;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = ap.G;
  a.RG = ap.RG;
  a.D = d.D;
  a.max_pages = d.max_pages;
  a.num_pages = d.num_pages;
  a.nlanes = 0;
  a.mslices = 1;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d.D));
  if (d.qkv_dtype == IDLM_F32) {
    if (d.D == 64)
      hipLaunchKernelGGL((attn_f32_kernel<64>), dim3(ap.npairs), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attn_f32_kernel<128>), dim3(ap.npairs), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
  }
  if (d.D == 64) {
    if (ap.RB == 2) return launch_stream<64, 1, 2>(a, s);
    if (ap.WR == 1) return launch_stream<64, 1, 4>(a, s);
    return launch_stream<64, 2, 4>(a, s);
  }
  if (ap.RB == 2) return launch_stream<128, 1, 2>(a, s);
  if (ap.WR == 1) return launch_stream<128, 1, 4>(a, s);
  return launch_stream<128, 2, 4>(a, s);
}

}  // namespace idlm
