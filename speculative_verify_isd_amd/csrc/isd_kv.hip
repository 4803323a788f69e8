// KV-cache append (before attention) and rollback to the accepted prefix
// (after acceptance), for gfx950.
//
// The cache is paged and serves continuous batching ("Introspective
// Diffusion Language Models" and its GeekNews summary, section "Serving
// (SGLang)").  A step's R = 2N-1 rows get positions ctx_before ..
// ctx_before + R - 1 before attention; after acceptance only the anchor and
// the accepted drafts stay context ("Inference & ISD": the first rejection
// ends the kept prefix), so the context becomes ctx_lens - R + accept_len and
// pages no longer needed go back to the free list.
//
// The free list is a stack of page ids.  A call takes (or returns) its pages
// as one block at the top, sequence by sequence in batch order, each
// sequence's pages in page order: one work-group computes the per-sequence
// counts, their exclusive prefix and the page-table updates in batch order,
// so page assignment is the same on every run (no atomics).  A second launch
// scatters the new rows' K and V into the paged layout.
#include <hip/hip_runtime.h>

#include "isd_internal.hpp"

namespace idlm {
namespace {

struct KvArgs {
  const void* k_new;   // [B][R][Hkv][D]
  const void* v_new;
  const int32_t* ctx_in;
  int32_t* ctx_out;
  const int32_t* accept_len;
  void* kv;            // [P][2][Hkv][16*D]
  int32_t* page_table; // [B][max_pages]
  int32_t* free_pages; // [num_pages] stack
  int32_t* free_count; // stack height
  uint8_t* valid;      // [B] scatter flags (workspace)
  int32_t* status;
  int B, R, Hkv, D, max_pages, num_pages, f32;
};

__device__ inline int64_t pages_of(int64_t n) { return (n + kPage - 1) / kPage; }

__device__ inline void flag(int32_t* status, int32_t bit) {
  __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

constexpr int kPlanThreads = 1024;

// Exclusive prefix of v over the work-group (thread order) and the total.
__device__ inline int64_t block_excl(int64_t v, int64_t* sh_w, int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh_w[wave] = x;
  __syncthreads();
  int64_t base = 0, tot = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    if (w < wave) base += sh_w[w];
    tot += sh_w[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Pages sequence b needs for the append (0 for a context out of range).
__device__ inline int64_t append_need(const KvArgs& a, int b, bool* valid, bool report) {
  const int64_t c = a.ctx_in[b];
  *valid = c >= 0 && c + a.R <= (int64_t)kPage * a.max_pages;
  if (!*valid && report) flag(a.status, kBadCtx);
  return *valid ? pages_of(c + a.R) - pages_of(c) : 0;
}

__global__ __launch_bounds__(kPlanThreads) void kv_append_plan_kernel(KvArgs a) {
  __shared__ int64_t sh_w[kPlanThreads / 64];
  __shared__ int sh_bad;
  const int tid = threadIdx.x;
  if (tid == 0) sh_bad = 0;
  if (a.B <= kPlanThreads) {
    // One pass: every sequence's values stay in its thread's registers.
    const int64_t fc = *a.free_count;
    bool v = false;
    int64_t c = 0, need = 0;
    if (tid < a.B) {
      c = a.ctx_in[tid];
      need = append_need(a, tid, &v, true);
    }
    int64_t total;
    const int64_t ex = block_excl(need, sh_w, &total);
    const int64_t base = fc - total;
    const bool enough = total <= fc;
    int32_t ids[4];  // at most ceil(R / 16) + 1 <= 3 new pages per sequence
    const int nn = (int)(need < 4 ? need : 4);
    if (enough)
      for (int i = 0; i < nn; ++i) {
        ids[i] = a.free_pages[base + ex + i];
        if (ids[i] < 0 || ids[i] >= a.num_pages) sh_bad = 1;
      }
    __syncthreads();
    const bool ok = enough && !sh_bad;
    if (tid == 0 && !enough) flag(a.status, kFreeList);
    if (tid == 0 && enough && sh_bad) flag(a.status, kBadPage);
    if (tid < a.B) {
      const bool w = ok && v;
      if (w) {
        int32_t* row = a.page_table + (size_t)tid * a.max_pages;
        for (int i = 0; i < nn; ++i) row[pages_of(c) + i] = ids[i];
      }
      a.ctx_out[tid] = w ? (int32_t)(c + a.R) : (int32_t)c;
      a.valid[tid] = w ? 1 : 0;
    }
    if (tid == 0 && ok) *a.free_count = (int32_t)base;
    return;
  }
  // Pass 1: pages needed by the whole batch.
  int64_t mine = 0;
  for (int b = tid; b < a.B; b += kPlanThreads) {
    bool v;
    mine += append_need(a, b, &v, true);
  }
  int64_t total;
  block_excl(mine, sh_w, &total);
  const int64_t fc = *a.free_count;
  const int64_t base = fc - total;
  bool ok = total <= fc;
  if (ok)
    for (int64_t i = tid; i < total; i += kPlanThreads) {
      const int32_t id = a.free_pages[base + i];
      if (id < 0 || id >= a.num_pages) sh_bad = 1;
    }
  __syncthreads();
  if (!ok) {
    if (tid == 0) flag(a.status, kFreeList);
  } else if (sh_bad) {
    ok = false;
    if (tid == 0) flag(a.status, kBadPage);
  }
  // Pass 2: batch-order prefix of the needs; each sequence takes its block.
  int64_t run = 0;
  for (int c0 = 0; c0 < a.B; c0 += kPlanThreads) {
    const int b = c0 + tid;
    bool v = false;
    const int64_t need = b < a.B ? append_need(a, b, &v, false) : 0;
    int64_t chunk;
    const int64_t ex = block_excl(need, sh_w, &chunk);
    if (b < a.B) {
      const int64_t c = a.ctx_in[b];
      const bool w = ok && v;
      if (w) {
        int32_t* row = a.page_table + (size_t)b * a.max_pages;
        for (int64_t i = 0; i < need; ++i) row[pages_of(c) + i] = a.free_pages[base + run + ex + i];
      }
      a.ctx_out[b] = w ? (int32_t)(c + a.R) : (int32_t)c;
      a.valid[b] = w ? 1 : 0;
    }
    run += chunk;
  }
  if (tid == 0 && ok) *a.free_count = (int32_t)base;
}

// One thread per (b, r, h, 8 consecutive d): K goes to its 16-byte column
// chunk(s), V to the transposed block.
template <bool F32>
__global__ __launch_bounds__(256) void kv_scatter_kernel(KvArgs a) {
  // Thread order (b, h, g, r), r fastest: a step's rows sit in consecutive
  // slots of a page, so neighbouring threads write neighbouring K chunks
  // (16 bytes apart) and neighbouring V elements of each transposed d row.
  const int G8 = a.D / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)a.B * a.R * a.Hkv * G8;
  if (i >= n) return;
  const int r = (int)(i % a.R);
  int64_t t = i / a.R;
  const int g = (int)(t % G8);
  t /= G8;
  const int h = (int)(t % a.Hkv);
  const int b = (int)(t / a.Hkv);
  if (!a.valid[b]) return;
  const int64_t pos = (int64_t)a.ctx_out[b] - a.R + r;
  const int page = a.page_table[(size_t)b * a.max_pages + pos / kPage];
  const int s = (int)(pos % kPage);
  const size_t src = (((size_t)b * a.R + r) * a.Hkv + h) * a.D + 8 * g;
  const size_t blk = (size_t)kPage * a.D;
  const size_t kbase = ((size_t)page * 2 * a.Hkv + h) * blk;
  const size_t vbase = ((size_t)page * 2 * a.Hkv + a.Hkv + h) * blk;
  if (F32) {
    const float* kn = (const float*)a.k_new + src;
    const float* vn = (const float*)a.v_new + src;
    float* kv = (float*)a.kv;
    // x = 4: d 8g..8g+3 is chunk 2g, d 8g+4..8g+7 chunk 2g+1.
    *(float4*)(kv + kbase + ((size_t)(2 * g) * kPage + s) * 4) = *(const float4*)kn;
    *(float4*)(kv + kbase + ((size_t)(2 * g + 1) * kPage + s) * 4) = *(const float4*)(kn + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) kv[vbase + (size_t)(8 * g + e) * kPage + s] = vn[e];
  } else {
    const uint16_t* kn = (const uint16_t*)a.k_new + src;
    const uint16_t* vn = (const uint16_t*)a.v_new + src;
    uint16_t* kv = (uint16_t*)a.kv;
    // x = 8: d 8g..8g+7 is chunk g.
    *(uint4*)(kv + kbase + ((size_t)g * kPage + s) * 8) = *(const uint4*)kn;
    const uint4 vv = *(const uint4*)vn;
    const unsigned w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      kv[vbase + (size_t)(8 * g + e) * kPage + s] = (uint16_t)(w[e / 2] >> (16 * (e & 1)));
  }
}

// Rollback of sequence b: kept context and pages to free.
__device__ inline int64_t rollback_freed(const KvArgs& a, int b, int64_t* keep, bool* valid,
                                         bool report) {
  const int64_t c = a.ctx_in[b];
  *valid = c >= a.R && c <= (int64_t)kPage * a.max_pages;
  int64_t acc = a.accept_len[b];
  if (acc < 1 || acc > a.R) {
    if (report) flag(a.status, kBadLen);
    acc = acc < 1 ? 1 : a.R;
  }
  if (!*valid && report) flag(a.status, kBadCtx);
  *keep = *valid ? c - a.R + acc : c;
  return *valid ? pages_of(c) - pages_of(*keep) : 0;
}

__global__ __launch_bounds__(kPlanThreads) void kv_rollback_kernel(KvArgs a) {
  __shared__ int64_t sh_w[kPlanThreads / 64];
  const int tid = threadIdx.x;
  if (a.B <= kPlanThreads) {
    // One pass; the entries to free are read before the prefix is known.
    const int64_t fc = *a.free_count;
    int64_t keep = 0, freed = 0;
    bool v = false;
    int32_t ids[4];
    int nn = 0;
    if (tid < a.B) {
      freed = rollback_freed(a, tid, &keep, &v, true);
      nn = (int)(freed < 4 ? freed : 4);
      const int32_t* row = a.page_table + (size_t)tid * a.max_pages;
      for (int i = 0; i < nn; ++i) ids[i] = row[pages_of(keep) + i];
    }
    int64_t total;
    const int64_t ex = block_excl(freed, sh_w, &total);
    const bool ok = fc + total <= a.num_pages;
    if (!ok && tid == 0) flag(a.status, kFreeList);
    if (tid < a.B) {
      if (ok && v) {
        int32_t* row = a.page_table + (size_t)tid * a.max_pages;
        for (int i = 0; i < nn; ++i) {
          a.free_pages[fc + ex + i] = ids[i];
          row[pages_of(keep) + i] = -1;
        }
      }
      a.ctx_out[tid] = (ok && v) ? (int32_t)keep : a.ctx_in[tid];
    }
    if (tid == 0 && ok) *a.free_count = (int32_t)(fc + total);
    return;
  }
  int64_t mine = 0;
  for (int b = tid; b < a.B; b += kPlanThreads) {
    int64_t keep;
    bool v;
    mine += rollback_freed(a, b, &keep, &v, true);
  }
  int64_t total;
  block_excl(mine, sh_w, &total);
  const int64_t fc = *a.free_count;
  const bool ok = fc + total <= a.num_pages;
  if (!ok && tid == 0) flag(a.status, kFreeList);
  int64_t run = 0;
  for (int c0 = 0; c0 < a.B; c0 += kPlanThreads) {
    const int b = c0 + tid;
    int64_t keep = 0;
    bool v = false;
    const int64_t freed = b < a.B ? rollback_freed(a, b, &keep, &v, false) : 0;
    int64_t chunk;
    const int64_t ex = block_excl(freed, sh_w, &chunk);
    if (b < a.B) {
      if (ok && v) {
        int32_t* row = a.page_table + (size_t)b * a.max_pages;
        for (int64_t i = 0; i < freed; ++i) {
          const int64_t p = pages_of(keep) + i;
          a.free_pages[fc + run + ex + i] = row[p];
          row[p] = -1;
        }
      }
      a.ctx_out[b] = (ok && v) ? (int32_t)keep : a.ctx_in[b];
    }
    run += chunk;
  }
  if (tid == 0 && ok) *a.free_count = (int32_t)(fc + total);
}

KvArgs make_args(const idlm_isd_dims& d, char* ws, const Plan& p) {
  KvArgs a = {};
  a.valid = (uint8_t*)(ws + p.off_kv_valid);
  a.status = (int32_t*)(ws + p.off_status);
  a.B = d.B;
  a.R = 2 * d.N - 1;
  a.Hkv = d.Hkv;
  a.D = d.D;
  a.max_pages = d.max_pages;
  a.num_pages = d.num_pages;
  a.f32 = d.qkv_dtype == IDLM_F32;
  return a;
}

}  // namespace

int32_t launch_kv_append(const idlm_isd_dims& d, const Plan& p, const void* k_new,
                         const void* v_new, const int32_t* ctx_before, int32_t* ctx_after,
                         void* kv_pages, int32_t* page_table, int32_t* free_pages,
                         int32_t* free_count, char* ws, hipStream_t s) {
  if (d.B == 0) return IDLM_OK;
  KvArgs a = make_args(d, ws, p);
  a.k_new = k_new;
  a.v_new = v_new;
  a.ctx_in = ctx_before;
  a.ctx_out = ctx_after;
  a.kv = kv_pages;
  a.page_table = page_table;
  a.free_pages = free_pages;
  a.free_count = free_count;
  hipLaunchKernelGGL(kv_append_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  const int64_t n = (int64_t)a.B * a.R * a.Hkv * (a.D / 8);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (a.f32)
    hipLaunchKernelGGL(kv_scatter_kernel<true>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_scatter_kernel<false>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

int32_t launch_kv_rollback(const idlm_isd_dims& d, const Plan& p, const int32_t* ctx_lens,
                           const int32_t* accept_len, int32_t* ctx_after, int32_t* page_table,
                           int32_t* free_pages, int32_t* free_count, char* ws, hipStream_t s) {
  if (d.B == 0) return IDLM_OK;
  KvArgs a = make_args(d, ws, p);
  a.ctx_in = ctx_lens;
  a.ctx_out = ctx_after;
  a.accept_len = accept_len;
  a.page_table = page_table;
  a.free_pages = free_pages;
  a.free_count = free_count;
  hipLaunchKernelGGL(kv_rollback_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

}  // namespace idlm
