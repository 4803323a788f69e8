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
// Three launches; kernel boundaries are the only synchronisation between
// work-groups (no atomic counters, no fences), and every reduction runs in a
// fixed order, so results do not depend on scheduling:
//
//   accept_stats       grid B*R*S1.  Each work-group reduces one slice of one
//                      logit row to (max m, sum of exp2((l - m) c)) with
//                      c = log2(e)/T: every load of the slice is issued before
//                      any arithmetic and the logits stay packed in registers,
//                      the slice max is reduced first so each element costs
//                      one float32 exponential, sums are float64.  The slice
//                      holding the row's draft also records the draft's
//                      logit.  The sequence's bonus row (clean row k, k the
//                      listed drafts) also records each 2048-element
//                      sub-chunk's sum, relative to the slice max.  Greedy
//                      (T = 0): (max, lowest argmax).
//   accept_decide_sum  grid B*S2, S2 sized so the grid fits on the chip at
//                      once.  In every work-group of a sequence, wave 0 alone
//                      merges the slices of each row (a lane group per row,
//                      butterfly reductions), evaluates p_i(x_i) and q_i(x_i)
//                      in float64 and finds the first rejection with two
//                      ballots; one barrier hands the plan to the other
//                      waves.  The first work-group writes the kept prefix,
//                      the accept length and the plan (the whole answer when
//                      T = 0).  After a rejection, each work-group sums the
//                      residual weights max(0, p_j - q_j) of its sub-chunks;
//                      with every draft kept nothing more is read (the bonus
//                      row's sub-chunk sums came from accept_stats).
//   accept_select      grid B, four waves each.  Wave 0 prefixes the
//                      sub-chunk weights and finds the sub-chunk holding
//                      t = u' * sum(w); all threads recompute that
//                      sub-chunk's weights (8 consecutive elements each) and
//                      a block prefix finds the smallest v whose running sum
//                      exceeds t.  Where the sub-chunk's own sum and its
//                      entry in the prefix differ in the last bits, t is
//                      clamped into the sub-chunk, so the pick is always an
//                      element with positive weight.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

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
  double2* bstats;  // [B][nsub]: (max, sum of exp2((l - max) c)) per sub-chunk of the bonus row
  double2* unif;    // [B][16]: (u_i, u'_i) for i = 0..K
  int B, N, K, R, V, S1, nsub, spw, S2, f32;  // spw, S2: chosen at launch
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

// Eight consecutive logits as loaded.  bf16 rows on the vector path stay
// packed two to a register until used, which halves the registers a batch of
// loads occupies; float32 rows and the element-wise path hold float bits.
template <bool VEC, bool F32>
struct Logits8 {
  static constexpr bool kPacked = VEC && !F32;
  static constexpr int NW = kPacked ? 4 : 8;
  unsigned w[NW];
  __device__ float operator[](int e) const {
    if constexpr (kPacked)
      return __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
    else
      return __uint_as_float(w[e]);
  }
};

// Logits v .. v+7 of a row; elements at or past hi read as -inf.  VEC (rows
// 16-byte aligned, V a multiple of 8, so v and hi are multiples of 8): one
// vector load, from a clamped in-row address when the group lies past hi,
// with no branch, so a thread's loads can all be in flight together.
// Otherwise element by element.
template <bool VEC, bool F32>
__device__ inline Logits8<VEC, F32> load8(const void* row, int v, int hi) {
  Logits8<VEC, F32> r;
  if constexpr (VEC) {
    const bool in = v < hi;
    const int vi = in ? v : hi - 8;
    if constexpr (F32) {
      const uint4 p0 = *(const uint4*)((const float*)row + vi);
      const uint4 p1 = *(const uint4*)((const float*)row + vi + 4);
      const unsigned w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) r.w[e] = in ? w[e] : 0xFF800000u;
    } else {
      const uint4 p = *(const uint4*)((const u16*)row + vi);
      const unsigned w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) r.w[e] = in ? w[e] : 0xFF80FF80u;  // two bf16 -inf
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r.w[e] = (v + e < hi) ? __float_as_uint(load1(row, v + e, F32)) : 0xFF800000u;
  }
  return r;
}

// Greedy order: larger value wins, lower index on ties.
__device__ inline void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// The wave's total of x in a fixed order (an xor butterfly); every call
// with the same inputs gives the same bits, read at any one lane.
__device__ inline double wave_total(double x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// ---------------------------------------------------------------------------
// Kernel 1: row-slice statistics.
// ---------------------------------------------------------------------------
template <int U, bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_stats_kernel(AccArgs a) {
  __shared__ double sh_s[4];
  __shared__ double sh_sk[8][4];
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
  // Clean row kp (kp = the listed drafts, up to the first negative id) is the
  // row the bonus token comes from when every draft is kept: it also records
  // each sub-chunk's sum (relative to the slice max), so sampling from it
  // rescans one sub-chunk instead of re-reading the row.
  bool bonus = false;
  if (!a.greedy && rho < a.N) {
    int kp = a.K;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = i < a.K ? a.drafts[(size_t)b * a.K + i] : 0;
      if (id < 0 && kp == a.K) kp = i;
    }
    bonus = rho == kp;
  }

  // All of this thread's loads first, then the arithmetic.
  Logits8<VEC, F32> x[U];
#pragma unroll
  for (int k = 0; k < U; ++k) x[k] = load8<VEC, F32>(row, lo + k * kSub + 8 * tid, hi);
  // The sequence's uniforms, drawn while the loads are in flight by the
  // first slice of its first row: thread i <= K draws (u_i, u'_i).
  if (rho == 0 && c == 0 && tid <= a.K) {
    const U64x4 ph = philox4x64_10((uint64_t)tid, 0, 0, 0, a.seed, (uint64_t)b);
    a.unif[(size_t)b * 16 + tid] = make_double2(top24(ph.w[0]), top24(ph.w[1]));
  }
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
        if (bonus) {  // work-group uniform: sub-chunk k's own sum, same exponentials
          double sk = (double)part;
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) sk += __shfl_xor(sk, off);
          if (lane == 0) sh_sk[k][wave] = sk;
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sh_s[wave] = s;
    __syncthreads();
    if (bonus && tid < U && c * U + tid < a.nsub) {
      // (slice max, sub-chunk sum relative to it); empty slice: sum 0.
      const double sk = M == -INFINITY ? 0.0
                                       : ((sh_sk[tid][0] + sh_sk[tid][1]) + sh_sk[tid][2]) +
                                             sh_sk[tid][3];
      a.bstats[(size_t)b * a.nsub + c * U + tid] = make_double2((double)M, sk);
    }
    if (tid != 0) return;
    res = make_double2((double)M, ((sh_s[0] + sh_s[1]) + sh_s[2]) + sh_s[3]);
  }
  a.stats[((size_t)b * a.R + rho) * a.S1 + c] = res;
}

// ---------------------------------------------------------------------------
// The sequence's decision, recomputed by every work-group that needs it.
// Collective: all threads call it; wave 0 does the work.  Leaves the plan in
// *sh_plan, the draft count in *sh_kp, the per-draft (p, q, u, u') in
// sh_draft and the raw draft ids in sh_ids.
// ---------------------------------------------------------------------------
constexpr int kStatCache = 4;  // slice statistics a lane keeps in registers

__device__ void decide(const AccArgs& a, int b, SamplePlan* sh_plan, int* sh_kp,
                       double (*sh_draft)[4], int* sh_ids) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int R = a.R, N = a.N, K = a.K, S1 = a.S1;
    // L lanes per row (R rounded up to a power of two rows in one wave).
    int rp = 1;
    while (rp < R) rp <<= 1;
    const int L = 64 / rp;
    const int rho = lane / L, q = lane % L;
    const bool row_ok = rho < R;
    const double2* st = a.stats + ((size_t)b * R + (row_ok ? rho : 0)) * S1;

    // One round of independent loads: this lane's slice statistics, and for
    // lane i < K draft i and the logits recorded for it.
    double2 cs[kStatCache];
#pragma unroll
    for (int j = 0; j < kStatCache; ++j) cs[j] = st[min(q + j * L, S1 - 1)];
    int id = -1;
    float lpf = 0.f, lqf = 0.f;
    if (K > 0) {
      const int ic = min(lane, K - 1);
      id = a.drafts[(size_t)b * K + ic];
      lpf = a.dlog[(size_t)b * R + ic];
      lqf = a.dlog[(size_t)b * R + N + ic];
    }
    // Lane i <= K: (u_i, u'_i), drawn by accept_stats.
    const double2 uu = a.unif[(size_t)b * 16 + min(lane, K)];
    const double u = uu.x, u2 = uu.y;

    // Row merge inside each L-lane group.  M (max) is exact in any order; S
    // is summed by a fixed butterfly and read from the group's lane 0.
    double M, S;
    if (a.greedy) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < kStatCache; ++j)
        if (row_ok && q + j * L < S1) better(bv, bi, (float)cs[j].x, (int)cs[j].y);
      for (int k = q + kStatCache * L; row_ok && k < S1; k += L) {
        const double2 v = st[k];
        better(bv, bi, (float)v.x, (int)v.y);
      }
      for (int off = 1; off < L; off <<= 1) {
        const float vo = __shfl_xor(bv, off);
        const int io = __shfl_xor(bi, off);
        better(bv, bi, vo, io);
      }
      M = bv;
      S = (double)bi;
    } else {
      M = -INFINITY;
#pragma unroll
      for (int j = 0; j < kStatCache; ++j)
        if (row_ok && q + j * L < S1) M = fmax(M, cs[j].x);
      for (int k = q + kStatCache * L; row_ok && k < S1; k += L) M = fmax(M, st[k].x);
      for (int off = 1; off < L; off <<= 1) M = fmax(M, __shfl_xor(M, off));
      const double c2 = (double)a.c2;
      S = 0.0;
#pragma unroll
      for (int j = 0; j < kStatCache; ++j)
        if (row_ok && q + j * L < S1 && cs[j].x != -INFINITY)
          S += cs[j].y * exp2((cs[j].x - M) * c2);
      for (int k = q + kStatCache * L; row_ok && k < S1; k += L) {
        const double2 v = st[k];
        if (v.x != -INFINITY) S += v.y * exp2((v.x - M) * c2);
      }
      for (int off = 1; off < L; off <<= 1) S += __shfl_xor(S, off);
    }

    // Lane i < K: p_i(x_i) from clean row i, q_i(x_i) from MASK row i.
    const int ia = min(lane, R - 1), ib = min(N + lane, R - 1);
    const double Mp = __shfl(M, ia * L), Sp = __shfl(S, ia * L);
    const double Mq = __shfl(M, ib * L), Sq = __shfl(S, ib * L);
    const int x = min(id, a.V - 1);
    double p, qq;
    if (a.greedy) {
      p = (x == (int)Sp) ? 1.0 : 0.0;
      qq = (x == (int)Sq) ? 1.0 : 0.0;
    } else {
      p = exp(((double)lpf - Mp) * a.invT) / Sp;
      qq = exp(((double)lqf - Mq) * a.invT) / Sq;
    }
    // A negative id ends the list; the first rejection among the listed
    // drafts ends the kept prefix.
    const bool is_draft = lane < K;
    const unsigned long long term = __ballot(is_draft && id < 0);
    const int kp = term ? (int)__builtin_ctzll(term) : K;
    const bool rej = is_draft && lane < kp && !(p >= qq || u * qq < p);
    const unsigned long long rm = __ballot(rej);
    const int j = rm ? (int)__builtin_ctzll(rm) : kp;

    const bool resid = j < kp;
    const double mp = __shfl(M, j * L), sp_ = __shfl(S, j * L);
    const int jq = resid ? N + j : 0;
    const double mq = __shfl(M, jq * L), sq = __shfl(S, jq * L);
    const double u2j = __shfl(u2, j);
    if (lane < K) {
      sh_ids[lane] = id;
      sh_draft[lane][0] = p;
      sh_draft[lane][1] = qq;
      sh_draft[lane][2] = u;
      sh_draft[lane][3] = u2;
    }
    if (lane == 0) {
      SamplePlan pl;
      pl.mode = a.greedy ? 2 : (resid ? 0 : 1);
      pl.row_p = j;
      pl.row_q = resid ? j : 0;
      pl.j = j;
      pl.mp = mp;
      pl.sp = sp_;
      pl.mq = resid ? mq : 0.0;
      pl.sq = resid ? sq : 1.0;
      pl.u2 = u2j;
      pl.pad = a.greedy ? sp_ : 0.0;  // greedy: the clean argmax of row j
      *sh_plan = pl;
      *sh_kp = kp;
    }
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
      if (x < -1 || x >= a.V)  // system scope: XCD L2 caches are not coherent
        __hip_atomic_fetch_or(a.status, kBadDraft, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
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
template <bool VEC, bool F32>
__device__ inline void weights8(const AccArgs& a, const SamplePlan& sp, int mode,
                                const Logits8<VEC, F32>& xp, const Logits8<VEC, F32>& xq,
                                double w[8]) {
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

// Logits v .. v+7 of the p row (and q row, mode 0).
template <bool VEC, bool F32>
__device__ inline void load_sub_at(const AccArgs& a, int b, const SamplePlan& sp, int mode, int v,
                                   Logits8<VEC, F32>& xp, Logits8<VEC, F32>& xq) {
  xp = load8<VEC, F32>(row_ptr(a, b, sp.row_p), v, a.V);
  if (mode == 0) {
    xq = load8<VEC, F32>(row_ptr(a, b, a.N + sp.row_q), v, a.V);
  } else {
#pragma unroll
    for (int e = 0; e < Logits8<VEC, F32>::NW; ++e)
      xq.w[e] = Logits8<VEC, F32>::kPacked ? 0xFF80FF80u : 0xFF800000u;
  }
}

// This thread's 8 logits of sub-chunk sc (thread t: elements 8t .. 8t+7).
template <bool VEC, bool F32>
__device__ inline void load_sub(const AccArgs& a, int b, const SamplePlan& sp, int mode, int sc,
                                Logits8<VEC, F32>& xp, Logits8<VEC, F32>& xq) {
  load_sub_at<VEC, F32>(a, b, sp, mode, sc * kSub + 8 * (int)threadIdx.x, xp, xq);
}

constexpr int kMaxSpw = 4;  // most sub-chunks one summing work-group takes

// The decision (recomputed by every work-group of the sequence from the
// slice statistics and recorded draft logits: one round of loads), then the
// sub-chunk sums of the sampling weights.  The sequence's first work-group
// also writes the kept prefix, the accept length and the plan.
template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_decide_sum_kernel(AccArgs a) {
  __shared__ double sh_draft[16][4];
  __shared__ int sh_ids[16];
  __shared__ SamplePlan sh_plan;
  __shared__ int sh_kp;
  __shared__ double sh_wave[kMaxSpw][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = (int)(blockIdx.x / a.S2);
  const int w0 = (int)(blockIdx.x % a.S2);
  decide(a, b, &sh_plan, &sh_kp, sh_draft, sh_ids);
  const SamplePlan sp = sh_plan;
  if (w0 == 0) {
    write_prefix(a, b, sp, sh_kp, sh_draft, sh_ids);
    if (tid == 0) a.plan[b] = sp;
  }
  // Greedy: the decision already wrote the token.  Bonus row: its sub-chunk
  // statistics came from the stats pass.
  if (sp.mode != 0) return;

  const int sc_lo = w0 * a.spw, n = min(a.nsub - sc_lo, a.spw);
  Logits8<VEC, F32> xp[kMaxSpw], xq[kMaxSpw];
#pragma unroll
  for (int k = 0; k < kMaxSpw; ++k)  // clamped, unconditional: all loads in flight together
    load_sub<VEC, F32>(a, b, sp, sp.mode, sc_lo + min(k, n - 1), xp[k], xq[k]);
#pragma unroll
  for (int k = 0; k < kMaxSpw; ++k) {
    double w[8];
    weights8<VEC, F32>(a, sp, sp.mode, xp[k], xq[k], w);
    const double tot = wave_total(thread_sum(w));
    if (lane == 63) sh_wave[k][wave] = tot;
  }
  __syncthreads();
  if (tid < n)
    a.subsum[(size_t)b * a.nsub + sc_lo + tid] =
        ((sh_wave[tid][0] + sh_wave[tid][1]) + sh_wave[tid][2]) + sh_wave[tid][3];
}

// ---------------------------------------------------------------------------
// Kernel 3: locate t and scan one sub-chunk.
// ---------------------------------------------------------------------------

// Wave 0 locates the sub-chunk holding t = u' * W, W = the sum of sh_sub.
// Lane l takes a contiguous run of sub-chunks; the runs' sums are prefixed by
// an inclusive wave scan; each lane then walks its run from its exclusive
// prefix.  The chosen sub-chunk is the first with a positive sum whose end
// exceeds t (base = its start); with no such sub-chunk (t at or past the
// total by rounding) it is the last sub-chunk with a positive sum and *past
// is set.  Results go to the shared variables; the caller synchronises.
__device__ void locate(const double* sh_sub, int nsub, double u2, double* sh_W, double* sh_t,
                       double* sh_base, int* sh_sc, int* sh_past) {
  const int lane = threadIdx.x;
  const int per = (nsub + 63) / 64;
  const int k0 = min(nsub, lane * per), k1 = min(nsub, k0 + per);
  double ls = 0.0;
  int lastpos = -1;
  for (int k = k0; k < k1; ++k) {
    const double v = sh_sub[k];
    ls += v;
    if (v > 0.0) lastpos = k;
  }
  double inc = ls;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  const double W = __shfl(inc, 63);
  double ex = __shfl_up(inc, 1);
  if (lane == 0) ex = 0.0;
  const double t = u2 * W;
  double run = ex, hbase = 0.0;
  int hit = -1;
  for (int k = k0; k < k1; ++k) {
    const double v = sh_sub[k];
    const double nx = run + v;
    if (hit < 0 && v > 0.0 && nx > t) {
      hit = k;
      hbase = run;
    }
    run = nx;
  }
  const unsigned long long hm = __ballot(hit >= 0);
  int sel = 0, past = 0;
  double base = 0.0;
  if (hm) {
    const int src = (int)__builtin_ctzll(hm);
    sel = __shfl(hit, src);
    base = __shfl(hbase, src);
  } else {
    past = 1;
    const unsigned long long pm = __ballot(lastpos >= 0);
    if (pm) sel = __shfl(lastpos, 63 - (int)__builtin_clzll(pm));
  }
  if (lane == 0) {
    *sh_W = W;
    *sh_t = t;
    *sh_base = base;
    *sh_sc = sel;
    *sh_past = past;
  }
}

// One work-group (four waves) per sequence.  The sub-chunk weights are staged
// in LDS and located by wave 0 (locate()); the chosen sub-chunk is then
// scanned by all 256 threads, thread t owning its elements 8t .. 8t + 7
// (vocabulary order), under a block prefix of the thread sums.
template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_select_kernel(AccArgs a) {
  __shared__ double sh_sub[kMaxSubChunks];
  __shared__ float sh_mc[kMaxSubChunks];
  __shared__ double sh_t, sh_base, sh_W;
  __shared__ int sh_sc, sh_past;
  __shared__ double sh_wsum[4];
  __shared__ int sh_last[4];
  __shared__ int sh_tok;
  __shared__ float sh_mref;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const SamplePlan sp = a.plan[b];
  // Residual mode samples from the sub-chunk sums of the previous launch,
  // bonus mode from the bonus row's sub-chunk (max, sum) of the stats pass;
  // both are loaded with the plan, in one round.
  const bool from_stats = sp.mode == 1;
  {
    const double* subs = a.subsum + (size_t)b * a.nsub;
    const double2* bs = a.bstats + (size_t)b * a.nsub;
    for (int i0 = 0; i0 < a.nsub; i0 += 256) {
      const int i = i0 + tid, ic = min(i, a.nsub - 1);
      const double sv = subs[ic];
      const double2 bv = bs[ic];
      if (i < a.nsub) {
        sh_sub[i] = from_stats ? bv.y : sv;
        sh_mc[i] = (float)bv.x;
      }
    }
  }
  if (sp.mode == 2) return;
  int mode = sp.mode;
  if (tid == 0) sh_tok = -1;
  __syncthreads();
  if (from_stats) {
    // Bonus mode: sub-chunk weights s_c * 2^((m_c - M) c), M the row max.
    if (wave == 0) {
      float m = -INFINITY;
      for (int i = lane; i < a.nsub; i += 64) m = fmaxf(m, sh_mc[i]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      if (lane == 0) sh_mref = m;
    }
    __syncthreads();
    const double mref = sh_mref;
    for (int i = tid; i < a.nsub; i += 256) {
      const float m = sh_mc[i];
      sh_sub[i] = m == -INFINITY ? 0.0 : sh_sub[i] * exp2(((double)m - mref) * (double)a.c2);
    }
    __syncthreads();
  }
  if (wave == 0) locate(sh_sub, a.nsub, sp.u2, &sh_W, &sh_t, &sh_base, &sh_sc, &sh_past);
  __syncthreads();
  bool rescale = from_stats;
  if (!(sh_W > 0.0)) {
    // The residual vanished to rounding: fall back to p_j over the whole row,
    // summed per sub-chunk as the summing launch does.
    mode = 1;
    rescale = false;
    for (int sc = 0; sc < a.nsub; ++sc) {
      Logits8<VEC, F32> xp, xq;
      load_sub<VEC, F32>(a, b, sp, 1, sc, xp, xq);
      double w[8];
      weights8<VEC, F32>(a, sp, 1, xp, xq, w);
      const double tot = wave_total(thread_sum(w));
      if (lane == 0) sh_wsum[wave] = tot;
      __syncthreads();
      if (tid == 0) sh_sub[sc] = ((sh_wsum[0] + sh_wsum[1]) + sh_wsum[2]) + sh_wsum[3];
      __syncthreads();
    }
    if (wave == 0) locate(sh_sub, a.nsub, sp.u2, &sh_W, &sh_t, &sh_base, &sh_sc, &sh_past);
    __syncthreads();
  }
  double base = sh_base;
  const int sc = sh_sc, past = sh_past;
  // t sits in [base, base + sum of the sub-chunk) up to rounding at a
  // sub-chunk boundary; clamping it to base keeps it inside.
  double t = fmax(sh_t, base);
  SamplePlan ps = sp;
  if (rescale) {
    // Scan the bonus sub-chunk with exponentials relative to its own
    // reference max, as its sum was formed: t moves to that scale, measured
    // from base.
    const double f = exp2(((double)sh_mc[sc] - (double)sh_mref) * (double)a.c2);
    t = (t - base) / f;
    base = 0.0;
    ps.mp = sh_mc[sc];
  }
  Logits8<VEC, F32> xp, xq;
  load_sub<VEC, F32>(a, b, ps, mode, sc, xp, xq);
  double w[8];
  weights8<VEC, F32>(a, ps, mode, xp, xq, w);
  const int v0 = sc * kSub + 8 * tid;
  const double ls = thread_sum(w);
  int lastp = -1;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (w[e] > 0.0) lastp = v0 + e;
  // Block prefix: inclusive scan in each wave, then the waves' totals in
  // order.  Thread t owns [base + ex_t, base + inc_t); consecutive threads
  // share their end points exactly (across a wave boundary too: the next
  // wave's offset is this wave's offset plus the same total), so at most one
  // thread holds t.
  double inc = ls;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) sh_wsum[wave] = inc;
  const unsigned long long pm = __ballot(lastp >= 0);
  const int lastw = __shfl(lastp, pm ? 63 - (int)__builtin_clzll(pm) : 0);  // all lanes
  if (lane == 0) sh_last[wave] = pm ? lastw : -1;
  __syncthreads();
  double woff = 0.0;
  for (int q = 0; q < wave; ++q) woff += sh_wsum[q];
  inc += woff;
  double ex = __shfl_up(inc, 1);
  if (lane == 0) ex = woff;
  const double lo = base + ex, hi = base + inc;
  if (!past && lo <= t && t < hi) {
    double run = lo;
    int tok = lastp;
    bool done = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      run += w[e];
      if (!done && run > t) {
        tok = v0 + e;
        done = true;
      }
    }
    sh_tok = tok;
  }
  __syncthreads();
  if (tid == 0) {
    int tok = sh_tok;
    if (tok < 0) {
      // No holder (t past the total, or a sub-chunk too small to move base):
      // the last element with positive weight.
      for (int q = 3; q >= 0 && tok < 0; --q) tok = sh_last[q];
      if (tok < 0) tok = min(a.V - 1, sc * kSub);
    }
    a.out_tokens[(size_t)b * a.N + sp.j] = tok;
    if (a.debug) {
      double* dbg = a.debug + ((size_t)b * (a.N + 1) + a.N) * 4;
      dbg[0] = sh_W;
      dbg[1] = sh_t;
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
int32_t launch_all(AccArgs a, hipStream_t s) {
  const int32_t r = launch_stats<kStatsU, VEC, F32>(a, s);
  if (r != IDLM_OK) return r;
  if (a.greedy) {
    // One decision work-group per sequence and no sampling.
    a.spw = a.nsub;
    a.S2 = 1;
  } else {
    // kMaxSpw sub-chunks per work-group: every work-group repeats the
    // decision, and fewer, larger work-groups measured faster at C = 64
    // (spw 4: 11.0 us, 3: 12.0 us, 2: 14.4 us) while the grid still fits on
    // the chip at once up to about a hundred sequences.
    a.spw = std::min(kMaxSpw, a.nsub);
    a.S2 = (a.nsub + a.spw - 1) / a.spw;
  }
  const int64_t g2 = (int64_t)a.B * a.S2;
  hipLaunchKernelGGL((accept_decide_sum_kernel<VEC, F32>), dim3((unsigned)g2), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  if (a.greedy) return IDLM_OK;
  hipLaunchKernelGGL((accept_select_kernel<VEC, F32>), dim3((unsigned)a.B), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Proposals for the next step.
//
// MASK rows propose the next tokens from q ("Introspective Diffusion
// Language Models", section "Inference & ISD").  A sequence whose listed
// drafts were all kept (accept_len == k + 1) continues verifying: draft i of
// its next step is drawn from softmax(next_i / T) by inverse CDF with the
// uniform of Philox counter (i, 1, 0, 0); T = 0 takes the argmax.  Otherwise
// the next step is fresh and its drafts are all -1.
//
//   propose_stats   grid B*K*ceil(nsub/8): each wave reduces whole 2048-element
//                   sub-chunks to (max m_c, sum of exp2((l - m_c) c)) (greedy:
//                   max, lowest argmax).  Rows of sequences that will not
//                   continue are skipped, so their logits are never read.
//   propose_select  grid B*K, four waves per row: wave 0 takes the weights
//                   s_c * 2^((m_c - M) c) in sub-chunk order and a wave scan
//                   locates the sub-chunk holding t = u * total; all 256
//                   threads rescan it (8 elements each, a block prefix) with
//                   the same exponentials (relative to m_c) as the stats pass.
// ---------------------------------------------------------------------------
struct PropArgs {
  const void* ln;           // [B][K][V]
  const int32_t* drafts;    // [B][K] this step's list
  const int32_t* accept_len;
  int32_t* next;            // [B][K]
  double2* st;              // [B][K][nsub]
  uint64_t seed;
  float c2;                 // log2(e) / T
  int greedy, B, K, V, nsub, f32;
};

constexpr int kPropSubPerWave = 2;

// Whether sequence b's next step verifies (all listed drafts kept).
__device__ inline bool continues(const PropArgs& a, int b) {
  int k = a.K;
  for (int i = 0; i < a.K; ++i)
    if (a.drafts[(size_t)b * a.K + i] < 0) {
      k = i;
      break;
    }
  return a.accept_len[b] == k + 1;
}

__device__ inline const void* prop_row(const PropArgs& a, int b, int i) {
  const size_t es = a.f32 ? 4 : 2;
  return (const char*)a.ln + ((size_t)b * a.K + i) * a.V * es;
}

template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void propose_stats_kernel(PropArgs a) {
  constexpr int kSubPerWg = 4 * kPropSubPerWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int S = (a.nsub + kSubPerWg - 1) / kSubPerWg;
  const int64_t wg = blockIdx.x;
  const int slice = (int)(wg % S);
  const int i = (int)((wg / S) % a.K);
  const int b = (int)(wg / ((int64_t)S * a.K));
  if (!continues(a, b)) return;
  const void* row = prop_row(a, b, i);
  double2* out = a.st + ((size_t)b * a.K + i) * a.nsub;
  const int sc0 = slice * kSubPerWg + wave * kPropSubPerWave;
  // Both sub-chunks' loads first (clamped to a real sub-chunk), then math.
  Logits8<VEC, F32> x[kPropSubPerWave][4];
#pragma unroll
  for (int k = 0; k < kPropSubPerWave; ++k) {
    const int sc = min(sc0 + k, a.nsub - 1);
#pragma unroll
    for (int g = 0; g < 4; ++g) x[k][g] = load8<VEC, F32>(row, sc * kSub + 512 * g + 8 * lane, a.V);
  }
#pragma unroll
  for (int k = 0; k < kPropSubPerWave; ++k) {
    const int sc = sc0 + k;
    if (sc >= a.nsub) break;  // wave-uniform
    if (a.greedy) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = sc * kSub + 512 * g + 8 * lane + e;
          if (v < a.V) better(bv, bi, x[k][g][e], v);
        }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float vo = __shfl_xor(bv, off);
        const int io = __shfl_xor(bi, off);
        better(bv, bi, vo, io);
      }
      if (lane == 0) out[sc] = make_double2((double)bv, (double)bi);
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, x[k][g][e]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      double s = 0.0;
      if (m != -INFINITY) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) part += __builtin_amdgcn_exp2f((x[k][g][e] - m) * a.c2);
          s += (double)part;
        }
      }
      s = wave_total(s);
      if (lane == 0) out[sc] = make_double2((double)m, s);
    }
  }
}

template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void propose_select_kernel(PropArgs a) {
  __shared__ int sh_sc, sh_past, sh_tok;
  __shared__ double sh_tl;
  __shared__ float sh_mc;
  __shared__ double sh_wsum[4];
  __shared__ int sh_last[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / a.K, i = blockIdx.x % a.K;
  int32_t* dst = a.next + (size_t)b * a.K + i;
  if (!continues(a, b)) {
    if (tid == 0) *dst = -1;
    return;
  }
  const double2* st = a.st + ((size_t)b * a.K + i) * a.nsub;
  const int per = (a.nsub + 63) / 64;
  const int k0 = min(a.nsub, lane * per), k1 = min(a.nsub, k0 + per);
  if (a.greedy) {
    if (wave != 0) return;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int k = k0; k < k1; ++k) better(bv, bi, (float)st[k].x, (int)st[k].y);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float vo = __shfl_xor(bv, off);
      const int io = __shfl_xor(bi, off);
      better(bv, bi, vo, io);
    }
    if (lane == 0) *dst = bi == 0x7FFFFFFF ? 0 : bi;
    return;
  }
  if (wave == 0) {
    // Wave 0 locates the sub-chunk: weights s_c 2^((m_c - M) c) in order,
    // each lane a contiguous run, a wave scan, the first sub-chunk with
    // positive weight whose end exceeds t = u * W.
    const double c2 = (double)a.c2;
    double M = -INFINITY;
    for (int k = k0; k < k1; ++k) M = fmax(M, st[k].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmax(M, __shfl_xor(M, off));
    double ls = 0.0;
    for (int k = k0; k < k1; ++k) {
      const double2 v = st[k];
      ls += v.x == -INFINITY ? 0.0 : v.y * exp2((v.x - M) * c2);
    }
    double inc = ls;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    const double W = __shfl(inc, 63);
    double ex = __shfl_up(inc, 1);
    if (lane == 0) ex = 0.0;
    const double u = top24(philox4x64_10((uint64_t)i, 1, 0, 0, a.seed, (uint64_t)b).w[0]);
    const double t = u * W;
    double run = ex, hbase = 0.0, hscale = 0.0;
    int hit = -1, lastpos = -1;
    for (int k = k0; k < k1; ++k) {
      const double2 v = st[k];
      const double f = v.x == -INFINITY ? 0.0 : exp2((v.x - M) * c2);
      const double w = v.y * f;
      if (w > 0.0) lastpos = k;
      if (hit < 0 && w > 0.0 && run + w > t) {
        hit = k;
        hbase = run;
        hscale = f;
      }
      run += w;
    }
    const unsigned long long hm = __ballot(hit >= 0);
    int sc;
    double tl;  // t relative to the sub-chunk, in its own units (weights relative to m_c)
    int past = 0;
    if (hm) {
      const int src = (int)__builtin_ctzll(hm);
      sc = __shfl(hit, src);
      const double base = __shfl(hbase, src), scale = __shfl(hscale, src);
      tl = fmax(0.0, (t - base) / scale);
    } else {
      const unsigned long long pm = __ballot(lastpos >= 0);
      sc = pm ? __shfl(lastpos, 63 - (int)__builtin_clzll(pm)) : 0;
      tl = 0.0;
      past = 1;
    }
    if (lane == 0) {
      sh_sc = sc;
      sh_tl = tl;
      sh_past = past;
      sh_mc = (float)st[sc].x;
      sh_tok = -1;
    }
  }
  __syncthreads();
  const int sc = sh_sc, past = sh_past;
  const double tl = sh_tl;
  const float mc = sh_mc;
  // Rescan with all 256 threads: thread t owns elements sc*kSub + 8t .. 8t + 7
  // (vocabulary order), under a block prefix of the thread sums.
  const void* row = prop_row(a, b, i);
  const int v0 = sc * kSub + 8 * tid;
  const Logits8<VEC, F32> xs = load8<VEC, F32>(row, v0, a.V);
  float w[8];
  float part = 0.f;
  int lastp = -1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = xs[e];
    w[e] = x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((x - mc) * a.c2);
    part += w[e];
    if (w[e] > 0.f) lastp = v0 + e;
  }
  double inc = (double)part;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) sh_wsum[wave] = inc;
  const unsigned long long pm = __ballot(lastp >= 0);
  const int lastw = __shfl(lastp, pm ? 63 - (int)__builtin_clzll(pm) : 0);  // all lanes
  if (lane == 0) sh_last[wave] = pm ? lastw : -1;
  __syncthreads();
  double woff = 0.0;
  for (int q = 0; q < wave; ++q) woff += sh_wsum[q];
  inc += woff;
  double ex = __shfl_up(inc, 1);
  if (lane == 0) ex = woff;
  // [ex, inc): consecutive threads share end points exactly, so at most one
  // thread holds tl.
  if (!past && ex <= tl && tl < inc) {
    double r = ex;
    int tok = lastp;
    bool done = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      r += (double)w[e];
      if (!done && r > tl) {
        tok = v0 + e;
        done = true;
      }
    }
    sh_tok = tok;
  }
  __syncthreads();
  if (tid == 0) {
    int tok = sh_tok;
    for (int q = 3; q >= 0 && tok < 0; --q) tok = sh_last[q];
    *dst = tok < 0 ? min(a.V - 1, sc * kSub) : tok;
  }
}

template <bool VEC, bool F32>
int32_t launch_propose_t(PropArgs a, hipStream_t s) {
  constexpr int kSubPerWg = 4 * kPropSubPerWave;
  const int S = (a.nsub + kSubPerWg - 1) / kSubPerWg;
  const int64_t g1 = (int64_t)a.B * a.K * S;
  hipLaunchKernelGGL((propose_stats_kernel<VEC, F32>), dim3((unsigned)g1), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  hipLaunchKernelGGL((propose_select_kernel<VEC, F32>), dim3((unsigned)(a.B * a.K)), dim3(256), 0,
                     s, a);
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
  a.unif = (double2*)(ws + p.off_unif);
  a.bstats = (double2*)(ws + p.off_bstats);
  a.B = d.B;
  a.N = d.N;
  a.K = d.N - 1;
  a.R = ap.R;
  a.V = d.V;
  a.S1 = ap.S1;
  a.nsub = ap.nsub;
  a.spw = 1;  // set per launch
  a.S2 = 1;
  a.f32 = d.logits_dtype == IDLM_F32;
  const bool vec = d.V % 8 == 0 && ((uintptr_t)lc % 16) == 0 &&
                   (lm == nullptr || ((uintptr_t)lm % 16) == 0);
  if (a.f32) return vec ? launch_all<true, true>(a, s) : launch_all<false, true>(a, s);
  return vec ? launch_all<true, false>(a, s) : launch_all<false, false>(a, s);
}

}  // namespace idlm

namespace idlm {

int32_t launch_propose(const idlm_isd_dims& d, const Plan& p, const void* logits_next,
                       const int32_t* drafts, const int32_t* accept_len, uint64_t seed, float T,
                       int32_t* next_drafts, char* ws, hipStream_t s) {
  if (d.B == 0 || d.N == 1) return IDLM_OK;
  PropArgs a = {};
  a.ln = logits_next;
  a.drafts = drafts;
  a.accept_len = accept_len;
  a.next = next_drafts;
  a.st = (double2*)(ws + p.off_pstats);
  a.seed = seed;
  a.greedy = (T == 0.0f);
  a.c2 = a.greedy ? 0.f : (float)(1.4426950408889634 / (double)T);
  a.B = d.B;
  a.K = d.N - 1;
  a.V = d.V;
  a.nsub = p.acc.nsub;
  a.f32 = d.logits_dtype == IDLM_F32;
  const bool vec = d.V % 8 == 0 && ((uintptr_t)logits_next % 16) == 0;
  if (a.f32) return vec ? launch_propose_t<true, true>(a, s) : launch_propose_t<false, true>(a, s);
  return vec ? launch_propose_t<true, false>(a, s) : launch_propose_t<false, false>(a, s);
}

}  // namespace idlm
