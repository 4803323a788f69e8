// isd_accept: the ISD acceptance stage for gfx950.
//
// Clean rows give the anchor distribution p, MASK rows the proposal
// distribution q; draft x is kept with probability min(1, p(x)/q(x)), which
// is what makes the committed tokens follow the autoregressive distribution
// ("Introspective Diffusion Language Models", section "Inference & ISD";
// GeekNews summary, section "Inference & ISD").  The first rejection is
// resampled from normalize(max(0, p - q)) (the rule under which that
// guarantee holds) and the committed prefix ends there; with every draft
// kept, the last clean row supplies a bonus token.
//
// Three launches; kernel boundaries are the only synchronisation (no
// atomics, no fences), and every reduction runs in a fixed order, so results
// do not depend on scheduling:
//
//   accept_stats       grid B*R*S1.  Each work-group reduces one slice of one
//                      logit row to (max m, sum of exp2((l - m) c)) with
//                      c = log2(e)/T: every load of the slice is issued before
//                      any arithmetic, the slice max is reduced first so each
//                      element costs one float32 exponential, sums are
//                      float64.  The slice holding the row's draft also
//                      records the draft's logit.  Greedy (T = 0): (max,
//                      lowest argmax).
//   accept_decide_sum  grid B*S2.  Every work-group of a sequence merges the
//                      slices of each row in order, evaluates p_i(x_i) and
//                      q_i(x_i) in float64, draws the Philox uniforms and runs
//                      the sequential ratio test (one round of loads), then
//                      sums the sampling weights (residual max(0, p_j - q_j)
//                      or bonus p) of its 2048-element sub-chunks.  The first
//                      work-group writes the kept prefix, the accept length
//                      and the sampling plan (the whole answer when T = 0).
//   accept_select      grid B.  Prefixes the sub-chunk sums in order, finds
//                      the sub-chunk holding t = u' * sum(w), recomputes it
//                      bit for bit and scans it to the smallest v whose
//                      running sum exceeds t.
#include <hip/hip_runtime.h>
#include <math.h>

#include "isd_internal.hpp"

namespace idlm {
namespace {

typedef unsigned short u16;

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of two
// 64x64->128 multiplies on counter words 0 and 2, key bumped by two Weyl
// constants between rounds.
// ---------------------------------------------------------------------------
struct U64x4 {
  uint64_t w[4];
};

__device__ inline U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                      uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
    const uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return U64x4{{c0, c1, c2, c3}};
}

__device__ inline double top24(uint64_t w) { return (double)(w >> 40) * 0x1.0p-24; }

struct AccArgs {
  const void* lc;
  const void* lm;
  const int32_t* drafts;
  uint64_t seed;
  float c2;      // log2(e) / T  (T > 0)
  double invT;   // 1 / T        (T > 0)
  int greedy;    // T == 0
  int32_t* out_tokens;
  int32_t* out_len;
  double* debug;
  int32_t* status;
  double2* stats;   // [B][R][S1]: (m, s) or, greedy, (best value, best index)
  SamplePlan* plan; // [B]
  double* subsum;   // [B][nsub]
  float* dlog;      // [B][R]: raw logit of the row's draft (rows that verify or proposed one)
  int B, N, K, R, V, S1, nsub, spw, S2, f32;
};

// Row rho of sequence b: rho < N is clean row rho, otherwise MASK row rho - N.
__device__ inline const void* row_ptr(const AccArgs& a, int b, int rho) {
  const size_t es = a.f32 ? 4 : 2;
  if (rho < a.N) return (const char*)a.lc + ((size_t)b * a.N + rho) * a.V * es;
  return (const char*)a.lm + ((size_t)b * a.K + (rho - a.N)) * a.V * es;
}

__device__ inline float load1(const void* row, int v, int f32) {
  return f32 ? ((const float*)row)[v] : __uint_as_float(((unsigned)((const u16*)row)[v]) << 16);
}

// Eight consecutive logits starting at v; elements at or past hi read as
// -inf.  VEC (rows 16-byte aligned, V a multiple of 8, so v and hi are
// multiples of 8): one vector load, from a clamped in-row address when the
// group lies past hi, with no branch, so a thread's loads can all be in
// flight together.  Otherwise element by element.
template <bool VEC, bool F32>
__device__ inline void load8(const void* row, int v, int hi, float x[8]) {
  if (VEC) {
    const bool in = v < hi;
    const int vi = in ? v : hi - 8;
    if (F32) {
      const float4 p0 = *(const float4*)((const float*)row + vi);
      const float4 p1 = *(const float4*)((const float*)row + vi + 4);
      x[0] = p0.x; x[1] = p0.y; x[2] = p0.z; x[3] = p0.w;
      x[4] = p1.x; x[5] = p1.y; x[6] = p1.z; x[7] = p1.w;
    } else {
      const uint4 p = *(const uint4*)((const u16*)row + vi);
      const unsigned w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = in ? x[e] : -INFINITY;
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (v + e < hi) ? load1(row, v + e, F32) : -INFINITY;
}

// Greedy order: larger value wins, lower index on ties.
__device__ inline void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// Inclusive scans of NS doubles per thread over the work-group, run side by
// side (one scan per index k, each in the same fixed order whatever NS is):
// thread t's inclusive value for scan k lands in sh_incl[k][t].
template <int NS>
__device__ inline void wg_scan_incl(const double (&x0)[NS], double (*sh_wave)[4],
                                    double (*sh_incl)[256]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double x[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) x[k] = x0[k];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const double y = __shfl_up(x[k], off);
      if (lane >= off) x[k] += y;
    }
  }
  if (lane == 63)
#pragma unroll
    for (int k = 0; k < NS; ++k) sh_wave[k][wave] = x[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    double base = 0.0;
    for (int w = 0; w < wave; ++w) base += sh_wave[k][w];
    sh_incl[k][threadIdx.x] = base + x[k];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Kernel 1: row-slice statistics.
// ---------------------------------------------------------------------------
template <int U, bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_stats_kernel(AccArgs a) {
  __shared__ double sh_s[4];
  __shared__ float sh_m[4];
  __shared__ int sh_i[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t wg = blockIdx.x;
  const int c = (int)(wg % a.S1);
  const int64_t tmp = wg / a.S1;
  const int rho = (int)(tmp % a.R);
  const int b = (int)(tmp / a.R);
  const void* row = row_ptr(a, b, rho);
  const int lo = c * kSub * U;
  const int hi = min(a.V, lo + kSub * U);

  // The row's draft (clean row i < K verifies draft i; MASK row i proposed
  // it; clean row K has none): the thread whose registers hold its logit
  // records it, so the decision needs no second round of loads.
  const int di = rho < a.N ? rho : rho - a.N;
  const int xd = (!a.greedy && di < a.K) ? min(a.drafts[(size_t)b * a.K + di], a.V - 1) : -1;

  // All of this thread's loads first, then the arithmetic.
  float x[U][8];
#pragma unroll
  for (int k = 0; k < U; ++k) load8<VEC, F32>(row, lo + k * kSub + 8 * tid, hi, x[k]);
  if (xd >= lo && xd < hi && ((xd - lo) % kSub) / 8 == tid) {
    const int kd = (xd - lo) / kSub, ed = xd % 8;
    float val = 0.f;
#pragma unroll
    for (int k = 0; k < U; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) val = (k == kd && e == ed) ? x[k][e] : val;
    a.dlog[(size_t)b * a.R + rho] = val;
  }

  double2 res;
  if (a.greedy) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int k = 0; k < U; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = lo + k * kSub + 8 * tid + e;
        if (v < hi) better(bv, bi, x[k][e], v);
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float vo = __shfl_xor(bv, off);
      const int io = __shfl_xor(bi, off);
      better(bv, bi, vo, io);
    }
    if (lane == 0) {
      sh_m[wave] = bv;
      sh_i[wave] = bi;
    }
    __syncthreads();
    if (tid != 0) return;
    bv = sh_m[0];
    bi = sh_i[0];
    for (int w = 1; w < 4; ++w) better(bv, bi, sh_m[w], sh_i[w]);
    res = make_double2((double)bv, (double)bi);
  } else {
    // Slice max first (float32), then one exponential per element relative
    // to it, so the sums need no rescaling.
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < U; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, x[k][e]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) sh_m[wave] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));
    double s = 0.0;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part += __builtin_amdgcn_exp2f((x[k][e] - M) * a.c2);
        s += (double)part;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sh_s[wave] = s;
    __syncthreads();
    if (tid != 0) return;
    res = make_double2((double)M, ((sh_s[0] + sh_s[1]) + sh_s[2]) + sh_s[3]);
  }
  a.stats[((size_t)b * a.R + rho) * a.S1 + c] = res;
}

// ---------------------------------------------------------------------------
// The sequence's decision, recomputed by every work-group that needs it.
// Collective: all 256 threads call it.  Leaves the plan in *out_plan, the
// draft count in *out_kp, the per-draft (p, q, u, u') in sh_draft and the
// raw draft ids in sh_ids.
// ---------------------------------------------------------------------------
__device__ void decide(const AccArgs& a, int b, SamplePlan* out_plan, int* out_kp,
                       double (*sh_draft)[4], double* sh_m, double* sh_s, int* sh_ids,
                       double2* sh_st) {
  const int tid = threadIdx.x;
  const int R = a.R, N = a.N, K = a.K;
  const int nst = R * a.S1;
  const bool st_in_lds = nst <= kDecideStats;
  const double2* st_g = a.stats + (size_t)b * nst;
  // One round of independent loads: the slice statistics and the drafts.
  if (st_in_lds)
    for (int i = tid; i < nst; i += 256) sh_st[i] = st_g[i];
  double lp = 0.0, lq = 0.0;  // the draft's raw logits, recorded by accept_stats
  if (tid < K) {
    sh_ids[tid] = a.drafts[(size_t)b * K + tid];
    if (!a.greedy) {
      lp = (double)a.dlog[(size_t)b * R + tid];
      lq = (double)a.dlog[(size_t)b * R + N + tid];
    }
  }
  __syncthreads();
  bool listed = false;
  if (tid < K) {
    listed = true;  // no -1 terminator up to this draft
    for (int i = 0; i <= tid; ++i) listed = listed && (sh_ids[i] >= 0);
  }
  // Row merge.  Row maxima first (thread rho, slices in order); then, when
  // the statistics sit in LDS, every (row, slice) weight exp2((m_k - M) c)
  // is formed by its own thread, and thread rho sums them in slice order.
  if (tid < R) {
    const double2* st = st_in_lds ? sh_st + tid * a.S1 : st_g + tid * a.S1;
    if (a.greedy) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int k = 0; k < a.S1; ++k) {
        const double2 v = st[k];
        better(bv, bi, (float)v.x, (int)v.y);
      }
      sh_m[tid] = bv;
      sh_s[tid] = (double)bi;
    } else {
      double M = -INFINITY;
      for (int k = 0; k < a.S1; ++k) M = fmax(M, st[k].x);
      sh_m[tid] = M;
      if (!st_in_lds) {
        double S = 0.0;
        for (int k = 0; k < a.S1; ++k) {
          const double2 v = st[k];
          if (v.x != -INFINITY) S += v.y * exp2((v.x - M) * (double)a.c2);
        }
        sh_s[tid] = S;
      }
    }
  }
  if (st_in_lds && !a.greedy) {
    __syncthreads();
    for (int i = tid; i < nst; i += 256) {
      const double2 v = sh_st[i];
      const double M = sh_m[i / a.S1];
      sh_st[i].y = (v.x != -INFINITY) ? v.y * exp2((v.x - M) * (double)a.c2) : 0.0;
    }
    __syncthreads();
    if (tid < R) {
      double S = 0.0;
      for (int k = 0; k < a.S1; ++k) S += sh_st[tid * a.S1 + k].y;
      sh_s[tid] = S;
    }
  }
  __syncthreads();
  // Per-draft inputs of the ratio test, one thread per draft.
  if (tid < K && listed) {
    const int x = min(sh_ids[tid], a.V - 1);
    const U64x4 w = philox4x64_10((uint64_t)tid, 0, 0, 0, a.seed, (uint64_t)b);
    double p, q;
    if (a.greedy) {
      p = (x == (int)sh_s[tid]) ? 1.0 : 0.0;
      q = (x == (int)sh_s[N + tid]) ? 1.0 : 0.0;
    } else {
      p = exp((lp - sh_m[tid]) * a.invT) / sh_s[tid];
      q = exp((lq - sh_m[N + tid]) * a.invT) / sh_s[N + tid];
    }
    sh_draft[tid][0] = p;
    sh_draft[tid][1] = q;
    sh_draft[tid][2] = top24(w.w[0]);
    sh_draft[tid][3] = top24(w.w[1]);
  }
  __syncthreads();
  if (tid == 0) {
    int kp = K;
    for (int i = 0; i < K; ++i)
      if (sh_ids[i] < 0) {
        kp = i;
        break;
      }
    int j = kp;
    for (int i = 0; i < kp; ++i) {
      const double p = sh_draft[i][0], q = sh_draft[i][1], u = sh_draft[i][2];
      if (!(p >= q || u * q < p)) {
        j = i;
        break;
      }
    }
    SamplePlan sp;
    sp.j = j;
    sp.u2 = j < kp ? sh_draft[j][3]
                   : top24(philox4x64_10((uint64_t)j, 0, 0, 0, a.seed, (uint64_t)b).w[1]);
    sp.row_p = j;
    sp.row_q = (j < kp) ? j : 0;
    sp.mode = a.greedy ? 2 : ((j < kp) ? 0 : 1);
    sp.mp = sh_m[j];
    sp.sp = sh_s[j];
    sp.mq = (j < kp) ? sh_m[N + j] : 0.0;
    sp.sq = (j < kp) ? sh_s[N + j] : 1.0;
    sp.pad = a.greedy ? sh_s[j] : 0.0;  // greedy: the clean argmax of row j
    *out_plan = sp;
    *out_kp = kp;
  }
  __syncthreads();
}

// Writes the kept prefix, accept length, debug rows and (greedy) the token.
__device__ void write_prefix(const AccArgs& a, int b, const SamplePlan& sp, int kp,
                             double (*sh_draft)[4], const int* sh_ids) {
  const int tid = threadIdx.x, N = a.N, j = sp.j;
  if (tid < N) {
    int tok = -1;
    if (tid < j) tok = sh_ids[tid];
    if (tid == j && sp.mode == 2) tok = (int)sp.pad;
    a.out_tokens[(size_t)b * N + tid] = tok;
  }
  if (tid == 0) {
    a.out_len[b] = j + 1;
    for (int i = 0; i < a.K; ++i) {
      const int x = sh_ids[i];
      if (x < -1 || x >= a.V) atomicOr(a.status, kBadDraft);
      if (x < 0) break;
    }
  }
  if (a.debug) {
    double* dbg = a.debug + (size_t)b * (N + 1) * 4;
    for (int i = tid; i < 4 * (N + 1); i += 256) {
      const int r = i / 4, k = i % 4;
      double v = NAN;
      if (r < N - 1 && r <= j && r < kp) v = sh_draft[r][k];
      if (r == N && sp.mode == 2) v = (k == 0) ? 1.0 : (k == 3 ? sp.pad : sp.u2);
      dbg[i] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: decision + sub-chunk sums of the sampling weights.
// ---------------------------------------------------------------------------

// Sampling weights of 8 elements, scaled by the p row's sum S_p (sampling is
// scale-free: t and the running sums scale together).  Mode 1 (p only):
// w = exp2((l_p - m_p) c).  Mode 0 (residual): w = max(0, e_p - e_q * S_p/S_q)
// with the ratio applied as a two-float product (hi + lo), so p and q keep
// the exact relative scale their float64 row sums gave them and the
// residual carries no systematic float32 scale error; what remains is the
// per-element rounding of the float32 exponentials.
__device__ inline void weights8(const AccArgs& a, const SamplePlan& sp, int mode,
                                const float xp[8], const float xq[8], double w[8]) {
  const float c2 = a.c2;
  const float mp = (float)sp.mp;
  if (mode == 0) {
    const float mq = (float)sp.mq;
    const double r = sp.sp / sp.sq;
    const float r_hi = (float)r;
    const float r_lo = (float)(r - (double)r_hi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ep = __builtin_amdgcn_exp2f((xp[e] - mp) * c2);
      const float eq = __builtin_amdgcn_exp2f((xq[e] - mq) * c2);
      w[e] = (double)fmaxf(0.f, ep - fmaf(eq, r_hi, eq * r_lo));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (double)__builtin_amdgcn_exp2f((xp[e] - mp) * c2);
  }
}

// This thread's sum of its 8 weights, accumulated in a fixed order.
__device__ inline double thread_sum(const double w[8]) {
  double ts = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ts += w[e];
  return ts;
}

// This thread's 8 logits of sub-chunk sc in the p row (and q row, mode 0).
template <bool VEC, bool F32>
__device__ inline void load_sub(const AccArgs& a, int b, const SamplePlan& sp, int mode, int sc,
                                float xp[8], float xq[8]) {
  const int v = sc * kSub + 8 * threadIdx.x;
  load8<VEC, F32>(row_ptr(a, b, sp.row_p), v, a.V, xp);
  if (mode == 0) {
    load8<VEC, F32>(row_ptr(a, b, a.N + sp.row_q), v, a.V, xq);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) xq[e] = -INFINITY;
  }
}

constexpr int kMaxSpw = 4;  // upper bound of AcceptPlan::spw

// The decision (recomputed by every work-group of the sequence from the
// slice statistics and recorded draft logits: one round of loads), then the
// sub-chunk sums of the sampling weights.  The sequence's first work-group
// also writes the kept prefix, the accept length and the plan.
template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_decide_sum_kernel(AccArgs a) {
  __shared__ double2 sh_st[kDecideStats];
  __shared__ double sh_draft[16][4];
  __shared__ double sh_m[32], sh_s[32];
  __shared__ int sh_ids[16];
  __shared__ SamplePlan sh_plan;
  __shared__ int sh_kp;
  __shared__ double sh_wave[kMaxSpw][4], sh_incl[kMaxSpw][256];
  const int tid = threadIdx.x;
  const int b = (int)(blockIdx.x / a.S2);
  const int w0 = (int)(blockIdx.x % a.S2);
  decide(a, b, &sh_plan, &sh_kp, sh_draft, sh_m, sh_s, sh_ids, sh_st);
  const SamplePlan sp = sh_plan;
  if (w0 == 0) {
    write_prefix(a, b, sp, sh_kp, sh_draft, sh_ids);
    if (tid == 0) a.plan[b] = sp;
  }
  if (sp.mode == 2) return;  // greedy: the decision already wrote the token

  const int sc_lo = w0 * a.spw, n = min(a.nsub - sc_lo, a.spw);
  float xp[kMaxSpw][8], xq[kMaxSpw][8];
#pragma unroll
  for (int k = 0; k < kMaxSpw; ++k)  // clamped, unconditional: all loads in flight together
    load_sub<VEC, F32>(a, b, sp, sp.mode, sc_lo + min(k, n - 1), xp[k], xq[k]);
  double ts[kMaxSpw];
#pragma unroll
  for (int k = 0; k < kMaxSpw; ++k) {
    double w[8];
    weights8(a, sp, sp.mode, xp[k], xq[k], w);
    ts[k] = thread_sum(w);
  }
  wg_scan_incl<kMaxSpw>(ts, sh_wave, sh_incl);
  if (tid < n) a.subsum[(size_t)b * a.nsub + sc_lo + tid] = sh_incl[tid][255];
}

// ---------------------------------------------------------------------------
// Kernel 3: locate t and scan one sub-chunk.
// ---------------------------------------------------------------------------
template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_select_kernel(AccArgs a) {
  __shared__ double sh_wave[1][4], sh_incl[1][256];
  __shared__ double sh_sub[kMaxSubChunks];
  __shared__ double sh_t, sh_base, sh_W;
  __shared__ int sh_sc, sh_past, sh_mode;
  __shared__ int found_tok, found_last;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const double* subs = a.subsum + (size_t)b * a.nsub;
  for (int i = tid; i < a.nsub; i += 256) sh_sub[i] = subs[i];
  const SamplePlan sp = a.plan[b];
  if (sp.mode == 2) return;
  float xp[8], xq[8];
  double w[8];
  __syncthreads();
  if (tid == 0) {
    double W = 0.0;
    for (int sc = 0; sc < a.nsub; ++sc) W += sh_sub[sc];
    sh_W = W;
    sh_mode = sp.mode;
  }
  __syncthreads();
  if (!(sh_W > 0.0)) {
    // The residual vanished to rounding: fall back to p_j over the whole row.
    for (int sc = 0; sc < a.nsub; ++sc) {
      load_sub<VEC, F32>(a, b, sp, 1, sc, xp, xq);
      weights8(a, sp, 1, xp, xq, w);
      const double ts[1] = {thread_sum(w)};
      wg_scan_incl<1>(ts, sh_wave, sh_incl);
      if (tid == 0) sh_sub[sc] = sh_incl[0][255];
    }
    __syncthreads();
    if (tid == 0) {
      double W = 0.0;
      for (int sc = 0; sc < a.nsub; ++sc) W += sh_sub[sc];
      sh_W = W;
      sh_mode = 1;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double t = sp.u2 * sh_W;
    double cum = 0.0, base = 0.0;
    int sel = -1, lastpos = 0;
    for (int sc = 0; sc < a.nsub; ++sc) {
      const double nx = cum + sh_sub[sc];
      if (sh_sub[sc] > 0.0) lastpos = sc;
      if (sel < 0 && nx > t) {
        sel = sc;
        base = cum;
      }
      cum = nx;
    }
    sh_past = sel < 0;  // rounding put t at or past the total
    if (sel < 0) sel = lastpos;
    sh_t = t;
    sh_base = base;
    sh_sc = sel;
    found_tok = 0x7FFFFFFF;
    found_last = -1;
  }
  __syncthreads();
  const double t = sh_t, base = sh_base;
  const int sc = sh_sc, mode = sh_mode;
  load_sub<VEC, F32>(a, b, sp, mode, sc, xp, xq);
  weights8(a, sp, mode, xp, xq, w);
  {
    const double ts[1] = {thread_sum(w)};
    wg_scan_incl<1>(ts, sh_wave, sh_incl);  // the same per-sub-chunk scan as accept_decide_sum
  }
  const int v0 = sc * kSub + 8 * tid;
  int lastp = -1;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (w[e] > 0.0) lastp = v0 + e;
  if (!sh_past) {
    // Thread k owns [base + incl[k-1], base + incl[k]): the intervals tile
    // [base, base + total) exactly, so exactly one thread holds t.
    const double lo = base + (tid ? sh_incl[0][tid - 1] : 0.0);
    const double hi = base + sh_incl[0][tid];
    if (lo <= t && t < hi) {
      double run = lo;
      int tok = lastp;
      for (int e = 0; e < 8; ++e) {
        run += w[e];
        if (run > t) {
          tok = v0 + e;
          break;
        }
      }
      found_tok = tok;
    }
  } else if (lastp >= 0) {
    atomicMax(&found_last, lastp);
  }
  __syncthreads();
  if (tid == 0) {
    int tok = sh_past ? found_last : found_tok;
    if (tok < 0 || tok == 0x7FFFFFFF) tok = min(a.V - 1, sc * kSub);
    a.out_tokens[(size_t)b * a.N + sp.j] = tok;
    if (a.debug) {
      double* dbg = a.debug + ((size_t)b * (a.N + 1) + a.N) * 4;
      dbg[0] = sh_W;
      dbg[1] = t;
      dbg[2] = sp.u2;
      dbg[3] = (double)tok;
    }
  }
}

template <int U, bool VEC, bool F32>
int32_t launch_stats(const AccArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)a.B * a.R * a.S1;
  hipLaunchKernelGGL((accept_stats_kernel<U, VEC, F32>), dim3((unsigned)g), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

template <bool VEC, bool F32>
int32_t launch_all(AccArgs a, int U1, hipStream_t s) {
  int32_t r;
  switch (U1) {
    case 8: r = launch_stats<8, VEC, F32>(a, s); break;
    case 4: r = launch_stats<4, VEC, F32>(a, s); break;
    case 2: r = launch_stats<2, VEC, F32>(a, s); break;
    default: r = launch_stats<1, VEC, F32>(a, s); break;
  }
  if (r != IDLM_OK) return r;
  // Greedy needs one decision work-group per sequence and no sampling.
  if (a.greedy) a.S2 = 1;
  const int64_t g2 = (int64_t)a.B * a.S2;
  hipLaunchKernelGGL((accept_decide_sum_kernel<VEC, F32>), dim3((unsigned)g2), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  if (a.greedy) return IDLM_OK;
  hipLaunchKernelGGL((accept_select_kernel<VEC, F32>), dim3((unsigned)a.B), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

}  // namespace

int32_t launch_accept(const idlm_isd_dims& d, const Plan& p, const void* lc, const void* lm,
                      const int32_t* drafts, uint64_t seed, float T, int32_t* out_tokens,
                      int32_t* out_len, double* out_debug, char* ws, hipStream_t s) {
  if (d.B == 0) return IDLM_OK;
  const AcceptPlan& ap = p.acc;
  AccArgs a;
  a.lc = lc;
  a.lm = lm;
  a.drafts = drafts;
  a.seed = seed;
  a.greedy = (T == 0.0f);
  a.c2 = a.greedy ? 0.f : (float)(1.4426950408889634 / (double)T);
  a.invT = a.greedy ? 0.0 : 1.0 / (double)T;
  a.out_tokens = out_tokens;
  a.out_len = out_len;
  a.debug = out_debug;
  a.status = (int32_t*)(ws + p.off_status);
  a.stats = (double2*)(ws + p.off_stats);
  a.plan = (SamplePlan*)(ws + p.off_splan);
  a.subsum = (double*)(ws + p.off_subsum);
  a.dlog = (float*)(ws + p.off_dlog);
  a.B = d.B;
  a.N = d.N;
  a.K = d.N - 1;
  a.R = ap.R;
  a.V = d.V;
  a.S1 = ap.S1;
  a.nsub = ap.nsub;
  a.spw = ap.spw;
  a.S2 = ap.S2;
  a.f32 = d.logits_dtype == IDLM_F32;
  const bool vec = d.V % 8 == 0 && ((uintptr_t)lc % 16) == 0 &&
                   (lm == nullptr || ((uintptr_t)lm % 16) == 0);
  if (a.f32) return vec ? launch_all<true, true>(a, ap.U1, s) : launch_all<false, true>(a, ap.U1, s);
  return vec ? launch_all<true, false>(a, ap.U1, s) : launch_all<false, false>(a, ap.U1, s);
}

}  // namespace idlm
