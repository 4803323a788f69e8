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
// Work decomposition
//   One work-group (4 waves of 64) owns one context chunk of CP pages of one
//   (b, kv head) pair.  All R*G query rows of the pair share every K/V page,
//   so the page is read once and reused across the whole query tile: the
//   tile rows are the MFMA "N" side, 16 per block.  Each wave carries 32
//   query rows (two 16-row blocks); WR = ceil(R*G/32) waves split the rows
//   and the other 4/WR wave lanes split the chunk's pages two at a time.
//
//   Per two pages (32 tokens) and 16-row block a wave runs
//     S^T[tok][row] = K[tok][:] . Q[row][:]   (D/32 x mfma_f32_16x16x32_bf16)
//     online softmax on S^T (rows live in lanes, tokens in registers)
//     O^T[d][row]  += V^T[d][tok] . P^T[tok][row]  (D/16 x 16x16x32)
//   The S^T accumulator layout is exactly the B-operand layout P^T needs,
//   and O^T keeps rows in lanes, so the softmax rescale needs no shuffles.
//
//   The page layout is chosen for these operands: every K fragment load is
//   one contiguous 1 KiB per wave (16 B per lane) and every V^T fragment load
//   one contiguous 512 B, so the stream is fully coalesced straight into
//   VGPRs with no LDS round trip.  LDS is used only to merge the waves'
//   partial softmax states at the end of the chunk.
//
//   Split-K across work-groups: a chunk writes (m, l, O) partials; the last
//   work-group of a pair to finish (atomic counter) merges them in fixed
//   chunk order, so results do not depend on scheduling.  Work-groups are
//   laid out so that all chunks of a pair land on the same XCD (dispatch is
//   round-robin over the 8 XCDs), which keeps the merge reads in that XCD's
//   L2.
#include <hip/hip_runtime.h>
#include <math.h>

#include "isd_internal.hpp"

namespace idlm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

struct AttnArgs {
  const void* q;
  const void* kv;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  void* out;
  float* part_o;
  float2* part_ml;
  unsigned* counters;
  int32_t* status;
  int B, R, Hq, Hkv, G, RG, max_pages, num_pages, CP, maxc, npairs, ppx;
  float scale_log2;  // log2(e) / sqrt(D)
};

__device__ inline float bf16_to_f32(u16 v) { return __uint_as_float(((unsigned)v) << 16); }

__device__ inline u16 f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

__device__ inline void flag(int32_t* status, int32_t bit) { atomicOr(status, bit); }

// Map a work-group index to (pair, chunk) so every chunk of a pair shares an
// XCD: dispatch sends work-group i to XCD i % 8.
__device__ inline void decode_wg(int64_t wg, int ppx, int* pair, int* chunk) {
  const int x = (int)(wg & 7);
  const int64_t k = wg >> 3;
  *pair = x + 8 * (int)(k % ppx);
  *chunk = (int)(k / ppx);
}

// Validated context length of sequence b (clamped, flagged).
__device__ inline int load_ctx(const AttnArgs& a, int b) {
  int ctx = a.ctx_lens[b];
  const int hi = kPage * a.max_pages;
  if (ctx < a.R || ctx > hi) {
    if (threadIdx.x == 0) flag(a.status, kBadCtx);
    ctx = ctx < a.R ? a.R : hi;
  }
  return ctx;
}

__device__ inline int load_page(const AttnArgs& a, int b, int p) {
  int phys = a.page_table[(size_t)b * a.max_pages + p];
  if ((unsigned)phys >= (unsigned)a.num_pages) {
    flag(a.status, kBadPage);
    phys = 0;
  }
  return phys;
}

// ---------------------------------------------------------------------------
// bf16 MFMA path
// ---------------------------------------------------------------------------
template <int D, int WR>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NC = D / 32;  // K-dim steps of the QK product
  constexpr int ND = D / 16;  // 16-wide d blocks of the PV product
  constexpr int WK = 4 / WR;  // waves walking the pages
  constexpr int ROWS = 32 * WR;

  __shared__ float lds_o[4][32][D];
  __shared__ float lds_ml[4][32][2];
  __shared__ int lds_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int rgrp = wave % WR, pw = wave / WR;
  const int col = lane & 15, grp = lane >> 4;

  int pair, chunk;
  decode_wg(blockIdx.x, a.ppx, &pair, &chunk);
  if (pair >= a.npairs) return;
  const int b = pair / a.Hkv, kvh = pair % a.Hkv;
  const int ctx = load_ctx(a, b);
  const int npages = (ctx + kPage - 1) / kPage;
  const int nch = (npages + a.CP - 1) / a.CP;
  if (chunk >= nch) return;
  const int pbeg = chunk * a.CP;
  const int pend = min(npages, pbeg + a.CP);

  const u16* qb = (const u16*)a.q;
  const u16* kvb = (const u16*)a.kv;

  // Query fragments (B operand of S^T = K Q^T): row = lane's column, eight
  // consecutive d per lane; k-step c covers d chunk 4c + grp.
  bf16x8 qf[2][NC];
  int pos[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int i = rgrp * 32 + rb * 16 + col;
    const bool valid = i < a.RG;
    const int r = valid ? i / a.G : a.R - 1;
    const int g = valid ? i % a.G : 0;
    pos[rb] = ctx - a.R + r;
    const u16* qp = qb + (((size_t)b * a.R + r) * a.Hq + (size_t)kvh * a.G + g) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 v = valid ? *(const uint4*)(qp + 8 * (4 * c + grp)) : make_uint4(0, 0, 0, 0);
      qf[rb][c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};
  f32x4 acc[2][ND];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < ND; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t page_elems = (size_t)2 * a.Hkv * kPage * D;
  const size_t head_off = (size_t)kvh * kPage * D;
  const size_t v_off = (size_t)a.Hkv * kPage * D;

  for (int p0 = pbeg + 2 * pw; p0 < pend; p0 += 2 * WK) {
    const bool hasb = p0 + 1 < pend;
    const int phys_a = load_page(a, b, p0);
    const int phys_b = hasb ? load_page(a, b, p0 + 1) : phys_a;
    const u16* Ka = kvb + (size_t)phys_a * page_elems + head_off;
    const u16* Kb = kvb + (size_t)phys_b * page_elems + head_off;

    bf16x8 ka[NC], kb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ka[c] = __builtin_bit_cast(bf16x8, *(const uint4*)(Ka + 512 * c + 8 * lane));
      kb[c] = __builtin_bit_cast(bf16x8, *(const uint4*)(Kb + 512 * c + 8 * lane));
    }
    bf16x4 va[ND], vb[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const size_t o = v_off + (size_t)(16 * j + col) * kPage + 4 * grp;
      va[j] = __builtin_bit_cast(bf16x4, *(const uint2*)(Ka + o));
      vb[j] = __builtin_bit_cast(bf16x4, *(const uint2*)(Kb + o));
    }

    const int ta = p0 * kPage + 4 * grp;  // first token of this lane in page a
    const int tb = ta + kPage;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qf[rb][c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[c], qf[rb][c], sb, 0, 0, 0);
      }
      float xa[4], xb[4];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = (ta + e <= pos[rb]) ? sa[e] * a.scale_log2 : -INFINITY;
        xb[e] = (hasb && tb + e <= pos[rb]) ? sb[e] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, fmaxf(xa[e], xb[e]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[rb], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(m[rb] - muse);
      m[rb] = mnew;
      float ps = 0.f;
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pa = exp2f(xa[e] - muse);
        const float pb = exp2f(xb[e] - muse);
        ps += pa + pb;
        pf[e] = (__bf16)pa;
        pf[4 + e] = (__bf16)pb;
      }
      l[rb] = l[rb] * alpha + ps;
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        acc[rb][j] *= alpha;
        bf16x8 vf = {va[j][0], va[j][1], va[j][2], va[j][3], vb[j][0], vb[j][1], vb[j][2], vb[j][3]};
        acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[rb][j], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    l[rb] += __shfl_xor(l[rb], 16);
    l[rb] += __shfl_xor(l[rb], 32);
  }

  // Stage every wave's (m, l, O) in LDS: lane holds O^T[16j + 4grp + e][row col].
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) lds_o[wave][rb * 16 + col][16 * j + 4 * grp + e] = acc[rb][j][e];
    if (grp == 0) {
      lds_ml[wave][rb * 16 + col][0] = m[rb];
      lds_ml[wave][rb * 16 + col][1] = l[rb];
    }
  }
  __syncthreads();

  const int G = a.G;
  u16* outp = (u16*)a.out;
  const size_t slot = (size_t)pair * a.maxc + chunk;
  // Merge the page-walking waves of each row group.
  for (int idx = tid; idx < ROWS * D; idx += 256) {
    const int row = idx / D, d = idx % D;
    const int rg = row / 32, rr = row % 32;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WK; ++w) M = fmaxf(M, lds_ml[w * WR + rg][rr][0]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < WK; ++w) {
      const float f = exp2f(lds_ml[w * WR + rg][rr][0] - Mu);
      L += lds_ml[w * WR + rg][rr][1] * f;
      O += lds_o[w * WR + rg][rr][d] * f;
    }
    if (nch == 1) {
      if (row < a.RG) {
        const int r = row / G, g = row % G;
        outp[(((size_t)b * a.R + r) * a.Hq + (size_t)kvh * G + g) * D + d] = f32_to_bf16_rne(O / L);
      }
    } else {
      a.part_o[slot * (size_t)ROWS * D + idx] = O;
      if (d == 0) a.part_ml[slot * ROWS + row] = make_float2(M, L);
    }
  }
  if (nch == 1) return;

  // Last work-group of this pair merges the chunk partials in chunk order.
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(&a.counters[pair], 1u);
    lds_last = (prev == (unsigned)(nch - 1));
  }
  __syncthreads();
  if (!lds_last) return;
  __threadfence();
  const size_t base = (size_t)pair * a.maxc;
  for (int idx = tid; idx < ROWS * D; idx += 256) {
    const int row = idx / D, d = idx % D;
    if (row >= a.RG) continue;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, a.part_ml[(base + c) * ROWS + row].x);
    float L = 0.f, O = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float2 ml = a.part_ml[(base + c) * ROWS + row];
      const float f = exp2f(ml.x - M);
      L += ml.y * f;
      O += a.part_o[(base + c) * (size_t)ROWS * D + idx] * f;
    }
    const int r = row / G, g = row % G;
    outp[(((size_t)b * a.R + r) * a.Hq + (size_t)kvh * G + g) * D + d] = f32_to_bf16_rne(O / L);
  }
  if (tid == 0) a.counters[pair] = 0u;
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
  if (pair >= a.npairs) return;
  const int b = pair / a.Hkv, kvh = pair % a.Hkv;
  const int ctx = load_ctx(a, b);
  const float* qf = (const float*)a.q;
  const float* kv = (const float*)a.kv;
  float* outp = (float*)a.out;
  const size_t page_elems = (size_t)2 * a.Hkv * kPage * D;
  const size_t head_off = (size_t)kvh * kPage * D;
  const size_t v_off = (size_t)a.Hkv * kPage * D;
  const float scale = a.scale_log2;

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
      const int phys = load_page(a, b, t / kPage);
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

template <int D, int WR>
int32_t launch_bf16(const AttnArgs& args, const AttnPlan& ap, hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, WR>), dim3((unsigned)ap.grid), dim3(256), 0, s, args);
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
  a.counters = (unsigned*)(ws + p.off_attn_cnt);
  a.status = (int32_t*)(ws + p.off_status);
  a.B = d.B;
  a.R = ap.R;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = ap.G;
  a.RG = ap.RG;
  a.max_pages = d.max_pages;
  a.num_pages = d.num_pages;
  a.CP = ap.CP;
  a.maxc = ap.maxc;
  a.npairs = ap.npairs;
  a.ppx = ap.ppx;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d.D));
  if (d.qkv_dtype == IDLM_F32) {
    if (d.D == 64)
      hipLaunchKernelGGL((attn_f32_kernel<64>), dim3(ap.npairs), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attn_f32_kernel<128>), dim3(ap.npairs), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
  }
  if (d.D == 64) {
    if (ap.WR == 1) return launch_bf16<64, 1>(a, ap, s);
    if (ap.WR == 2) return launch_bf16<64, 2>(a, ap, s);
    return launch_bf16<64, 4>(a, ap, s);
  }
  if (ap.WR == 1) return launch_bf16<128, 1>(a, ap, s);
  if (ap.WR == 2) return launch_bf16<128, 2>(a, ap, s);
  return launch_bf16<128, 4>(a, ap, s);
}

}  // namespace idlm
