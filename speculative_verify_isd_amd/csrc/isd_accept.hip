// isd_accept: the ISD acceptance stage for gfx950, and the next step's
// proposals.
//
// Clean rows give the anchor distribution p, MASK rows the proposal
// distribution q; draft x is kept with probability min(1, p(x)/q(x)), which
// is what makes the committed tokens follow the autoregressive distribution
// ("Introspective Diffusion Language Models", section "Inference & ISD";
// GeekNews summary, section "Inference & ISD").  The first rejection is
// resampled from normalize(max(0, p - q)) (the rule under which that
// guarantee holds) and the committed prefix ends there; with every draft
// kept, clean row k (k = the listed drafts) supplies a bonus token.
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
//                      holding the row's draft records the draft's logit.
//                      Greedy (T = 0): (max, lowest argmax).
//   accept_decide_sum  grid B*S2.  In every work-group of a sequence, wave 0
//                      merges the slices of each row, evaluates p_i(x_i) and
//                      q_i(x_i) in float64 and finds the first rejection with
//                      two ballots; one barrier hands the plan to the other
//                      waves.  The first work-group writes the kept prefix,
//                      the accept length and the plan (the whole answer when
//                      T = 0).  After a rejection, each work-group sums its
//                      sub-chunks of the residual pair in float64: all of
//                      e_p = 2^((l_p - m_p) c) and of e_q (the exact row sums),
//                      and both over the elements where p > q by the row
//                      statistics.  With every draft kept it sums the bonus
//                      row's 2^((l - m) c) per sub-chunk instead.  These
//                      exponentials are float64 (exp2t, from a table of
//                      2^(j/64) in LDS).
//   accept_select      grid B.  The exact ratio S_p/S_q turns the residual
//                      sums into sub-chunk weights (bonus: the bonus row's
//                      sub-chunk sums); wave 0 prefixes them and finds the
//                      sub-chunk holding t = u' * sum(w); all threads rescan
//                      it in float64 (8 consecutive elements each) and a block
//                      prefix finds the smallest v whose running sum exceeds
//                      t.
//
// With the MASK-row statistics the proposals recorded for these drafts
// (the decode loop: MASK rows propose with q, and the same q tests the
// drafts one step later), accept_stats reduces only the N clean rows and the
// decision reads each MASK row's (max, sum) and the drafts' logits from the
// record, after checking it was made for these drafts, this T and these
// sizes.
//
// Float64 sampling weights: the token is the smallest v whose running sum of
// w passes t.  Float32 exponentials move those running sums by ~1e-7 of the
// total, enough to change the pick in about one draw in a thousand; with
// float64 exponentials and row sums the pick agrees with an exact evaluation
// unless t lies within ~1e-14 of a running sum.  The row statistics that
// decide acceptance stay float32 exponentials summed in float64 (the ratio
// test needs p(x) and q(x) to ~1e-7, not the running sums of a whole row).
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "isd_exp2d.hpp"
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

struct D4 {
  double x, y, z, w;
};

struct AccArgs {
  const void* lc;
  const void* lm;
  const int32_t* drafts;
  uint64_t seed;
  float c2;      // log2(e) / T as float32 (row statistics)
  double c2d;    // log2(e) / T as float64 (sampling weights)
  double c64;    // 64 c2d (exact): exp2t64's argument scale
  Exp2Coef cf;   // exp2d's coefficients (kept in scalar registers)
  Exp2Coef64 cf64;
  int greedy;    // T == 0
  int32_t* out_tokens;
  int32_t* out_len;
  double* debug;
  int32_t* status;
  double2* stats;   // [B][R][S1]: (m, s) or, greedy, (best value, best index)
  SamplePlan* plan; // [B]
  D4* subsum;       // [B][nsub]: residual pair (S_p, S_q, A, B) or bonus row (E, 0, 0, 0)
  float* dlog;      // [B][R]: raw logit of the row's draft
  double2* unif;    // [B][16]: (u_i, u'_i) for i = 0..K
  D4* rowstat;      // [B][R]: (max, sum, kind, scale) for the probability dump
  double* subw;     // [B][nsub]: normalised sub-chunk sampling weights
  // MASK-row statistics recorded by the proposals that made these drafts
  // (null: the statistics launch reduces the MASK rows itself).
  const MaskStatsHeader* mhdr;
  const double2* mst;     // [B][K]: each MASK row's (max, sum), or greedy (max, argmax)
  const float* mdlog;     // [B][K]: logit of each proposed draft
  const int32_t* mtok;    // [B][K]: the proposed drafts
  int nrows;        // rows the statistics launch reduces per sequence: R, or N with mst
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

// 2^((l - m) c) in float64, c = log2(e) / T, with the work-group's table of
// 2^(j/64) in LDS: exp2t64 of 64 (l - m) c, bit-identical to exp2t of
// (l - m) c.  m is the row's maximum (from the statistics or the proposals'
// record), so the argument is never positive, as exp2t64 requires.
__device__ inline double wexp(const AccArgs& a, const double* tab, float l, double m) {
  return exp2t64(((double)l - m) * a.c64, tab, a.cf64);
}

// v[i] for a run-time i in [0, 4), by selects (no indexed register array).
template <typename T>
__device__ inline T pick4(const T v[4], int i) {
  return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
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
  const int rho = (int)(tmp % a.nrows);
  const int b = (int)(tmp / a.nrows);
  const void* row = row_ptr(a, b, rho);
  const int lo = c * kSub * U;
  const int hi = min(a.V, lo + kSub * U);

  // All of this thread's loads first (they depend on nothing loaded), then
  // the arithmetic.
  Logits8<VEC, F32> x[U];
#pragma unroll
  for (int k = 0; k < U; ++k) x[k] = load8<VEC, F32>(row, lo + k * kSub + 8 * tid, hi);

  // The row's draft (clean row i < K verifies draft i; MASK row i proposed
  // it): the thread whose registers hold its logit records it, so the
  // decision needs no second round of loads.
  const int di = rho < a.N ? rho : rho - a.N;
  const int xd = (!a.greedy && di < a.K) ? min(a.drafts[(size_t)b * a.K + di], a.V - 1) : -1;
  // The sequence's uniforms, drawn by the first slice of its first row:
  // thread i <= K draws (u_i, u'_i).
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
      // (l - M) is exact (two bf16 values); scaling it by c rounds once.
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
// Collective: all threads call it; wave 0 does the work.  Leaves the plan in
// *sh_plan, the draft count in *sh_kp, the per-draft (p, q, u, u') in
// sh_draft, the raw draft ids in sh_ids and each row's (max, sum) in sh_rowM,
// sh_rowS.
// ---------------------------------------------------------------------------
constexpr int kStatCache = 4;  // slice statistics a lane keeps in registers

__device__ void decide(const AccArgs& a, int b, SamplePlan* sh_plan, int* sh_kp,
                       double (*sh_draft)[4], int* sh_ids, double* sh_rowM, double* sh_rowS) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int R = a.R, N = a.N, K = a.K, S1 = a.S1;
    // L lanes per row (R rounded up to a power of two rows in one wave).
    int rp = 1;
    while (rp < R) rp <<= 1;
    const int L = 64 / rp;
    const int rho = lane / L, q = lane % L;
    const bool row_ok = rho < R;
    // A row's entries: the statistics launch's slices, or (MASK rows, when
    // the proposals recorded them) the one (max, sum) the proposals merged.
    const bool carried = a.mst && row_ok && rho >= N;
    const double2* st = carried ? a.mst + ((size_t)b * K + (rho - N))
                                : a.stats + ((size_t)b * R + (row_ok ? rho : 0)) * S1;
    const int ns = carried ? 1 : S1;

    // One round of independent loads: this lane's slice statistics, and for
    // lane i < K draft i and the logits recorded for it.
    double2 cs[kStatCache];
#pragma unroll
    for (int j = 0; j < kStatCache; ++j) cs[j] = st[min(q + j * L, ns - 1)];
    int id = -1;
    float lpf = 0.f, lqf = 0.f;
    if (K > 0) {
      const int ic = min(lane, K - 1);
      id = a.drafts[(size_t)b * K + ic];
      lpf = a.dlog[(size_t)b * R + ic];
      lqf = a.mst ? a.mdlog[(size_t)b * K + ic] : a.dlog[(size_t)b * R + N + ic];
      // The recorded statistics must be the proposals' of these very drafts,
      // at this temperature and these sizes.
      if (a.mst && lane < K && id >= 0 &&
          (a.mtok[(size_t)b * K + ic] != id || a.mhdr->magic != kMaskStatsMagic ||
           a.mhdr->c2_bits != __float_as_uint(a.c2) || a.mhdr->B != a.B || a.mhdr->K != K ||
           a.mhdr->V != a.V))
        __hip_atomic_fetch_or(a.status, kBadMaskStats, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_SYSTEM);
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
        if (row_ok && q + j * L < ns) better(bv, bi, (float)cs[j].x, (int)cs[j].y);
      for (int k = q + kStatCache * L; row_ok && k < ns; k += L) {
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
        if (row_ok && q + j * L < ns) M = fmax(M, cs[j].x);
      for (int k = q + kStatCache * L; row_ok && k < ns; k += L) M = fmax(M, st[k].x);
      for (int off = 1; off < L; off <<= 1) M = fmax(M, __shfl_xor(M, off));
      const double c2 = (double)a.c2;  // the scale the slice sums were formed with
      S = 0.0;
#pragma unroll
      for (int j = 0; j < kStatCache; ++j)
        if (row_ok && q + j * L < ns && cs[j].x != -INFINITY)
          S += cs[j].y * exp2d((cs[j].x - M) * c2, a.cf);
      for (int k = q + kStatCache * L; row_ok && k < ns; k += L) {
        const double2 v = st[k];
        if (v.x != -INFINITY) S += v.y * exp2d((v.x - M) * c2, a.cf);
      }
      for (int off = 1; off < L; off <<= 1) S += __shfl_xor(S, off);
    }
    if (q == 0 && row_ok) {
      sh_rowM[rho] = M;
      sh_rowS[rho] = S;
    }

    // Lane i < K: p_i(x_i) from clean row i, q_i(x_i) from MASK row i, with
    // the scale of the row sums: 2^((l - M) c) / S.
    const int ia = min(lane, R - 1), ib = min(N + lane, R - 1);
    const double Mp = __shfl(M, ia * L), Sp = __shfl(S, ia * L);
    const double Mq = __shfl(M, ib * L), Sq = __shfl(S, ib * L);
    const int x = min(id, a.V - 1);
    double p, qq;
    if (a.greedy) {
      p = (x == (int)Sp) ? 1.0 : 0.0;
      qq = (x == (int)Sq) ? 1.0 : 0.0;
    } else {
      p = exp2d(((double)lpf - Mp) * (double)a.c2, a.cf) / Sp;
      qq = exp2d(((double)lqf - Mq) * (double)a.c2, a.cf) / Sq;
    }
    // A negative id ends the list.  Draft i is kept iff p > 0 and (p >= q
    // or u q < p): probability min(1, p/q), and never a token p gives no
    // mass.  The first rejection among the listed drafts ends the kept
    // prefix.
    const bool is_draft = lane < K;
    const unsigned long long term = __ballot(is_draft && id < 0);
    const int kp = term ? (int)__builtin_ctzll(term) : K;
    const bool keep = p > 0.0 && (p >= qq || u * qq < p);
    const unsigned long long rm = __ballot(is_draft && lane < kp && !keep);
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
      pl.j = j;
      pl.kp = kp;
      pl.mp = mp;
      pl.mq = resid ? mq : 0.0;
      pl.rho = resid ? sp_ / sq : 0.0;
      pl.sp = sp_;
      pl.u2 = u2j;
      pl.pad = a.greedy ? sp_ : 0.0;  // greedy: the clean argmax of row j
      *sh_plan = pl;
      *sh_kp = kp;
    }
  }
  __syncthreads();
}

// Writes the kept prefix, accept length, debug rows, row statistics for the
// probability dump and (greedy) the token.
__device__ void write_prefix(const AccArgs& a, int b, const SamplePlan& sp, int kp,
                             double (*sh_draft)[4], const int* sh_ids, const double* sh_rowM,
                             const double* sh_rowS) {
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
      if (r == N && sp.mode == 2) v = (k == 0) ? 1.0 : (k == 3 ? sp.pad : (k == 2 ? sp.u2 : NAN));
      dbg[i] = v;
    }
  }
  // Row statistics for the probability dump: the rows of the decision
  // (clean rows i < k and MASK rows i < k; greedy also clean row k); the
  // bonus row's statistics come from the sampler.
  for (int r = tid; r < a.R; r += 256) {
    const bool used = r < N ? (sp.mode == 2 ? r <= kp : r < kp) : r - N < kp;
    D4 st;
    st.x = used ? sh_rowM[r] : NAN;
    st.y = used ? sh_rowS[r] : NAN;
    st.z = used ? (sp.mode == 2 ? 2.0 : 1.0) : 0.0;
    st.w = (double)a.c2;  // the scale of the row sums
    a.rowstat[(size_t)b * a.R + r] = st;
  }
  if (sp.mode == 2)  // greedy: nothing is sampled
    for (int c = tid; c < a.nsub; c += 256) a.subw[(size_t)b * a.nsub + c] = NAN;
}

// Block-wide totals of four values per thread, in a fixed order (butterfly
// in each wave, then the waves in order); valid in every thread after the
// call.
__device__ inline void block_total4(double v[4], double (*red)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = wave_total(v[i]);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][i] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
}

// ---------------------------------------------------------------------------
// Kernel 2: decision + the residual pair's float64 sums per sub-chunk.
// ---------------------------------------------------------------------------
constexpr int kMaxSpw = 2;  // most sub-chunks one summing work-group takes
// Batches of at most this many sub-chunks (about eight work-groups per CU)
// take one sub-chunk per summing work-group.
constexpr int64_t kOneSubMax = 2048;

template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_decide_sum_kernel(AccArgs a) {
  __shared__ double sh_draft[16][4];
  __shared__ int sh_ids[16];
  __shared__ SamplePlan sh_plan;
  __shared__ int sh_kp;
  __shared__ double sh_rowM[32], sh_rowS[32];
  __shared__ double sh_red[4][4];
  __shared__ double sh_tab[64];
  const int tid = threadIdx.x;
  const int b = (int)(blockIdx.x / a.S2);
  const int w0 = (int)(blockIdx.x % a.S2);
  if (tid < 64) sh_tab[tid] = exp2t_entry(tid, a.cf);  // ordered by decide's barrier
  decide(a, b, &sh_plan, &sh_kp, sh_draft, sh_ids, sh_rowM, sh_rowS);
  const SamplePlan sp = sh_plan;
  if (w0 == 0) {
    write_prefix(a, b, sp, sh_kp, sh_draft, sh_ids, sh_rowM, sh_rowS);
    if (tid == 0) a.plan[b] = sp;
  }
  // Greedy: the decision already wrote the token.
  if (sp.mode == 2) return;
  const bool resid = sp.mode == 0;
  const int sc_lo = w0 * a.spw, n = min(a.nsub - sc_lo, a.spw);
  const void* rp = row_ptr(a, b, sp.row_p);
  const void* rq = row_ptr(a, b, a.N + (resid ? sp.row_p : 0));
  Logits8<VEC, F32> xp[kMaxSpw], xq[kMaxSpw];
#pragma unroll
  for (int k = 0; k < kMaxSpw; ++k) {  // clamped, unconditional: all loads in flight together
    if (k >= a.spw) break;               // work-group uniform
    const int v = (sc_lo + min(k, n - 1)) * kSub + 8 * tid;
    xp[k] = load8<VEC, F32>(rp, v, a.V);
    if (resid) xq[k] = load8<VEC, F32>(rq, v, a.V);
  }
#pragma unroll
  for (int k = 0; k < kMaxSpw; ++k) {
    if (k >= n) break;  // work-group uniform
    double v[4] = {0.0, 0.0, 0.0, 0.0};
    if (resid) {
      // e_p = 2^((l_p - m_p) c), e_q likewise, relative to the row maxima:
      // all-element sums (the float64 row sums) and the sums over the
      // elements where p > q by the row statistics' ratio (A, B; the
      // sampler forms A - (S_p/S_q) B).
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double ep = wexp(a, sh_tab, xp[k][e], sp.mp);
        const double eq = wexp(a, sh_tab, xq[k][e], sp.mq);
        // 1 or 0: e times it added by an fma is e added or nothing, in one
        // instruction per sum instead of a 64-bit select and an add
        const double in = ep > sp.rho * eq ? 1.0 : 0.0;
        v[0] += ep;
        v[1] += eq;
        v[2] = fma(ep, in, v[2]);
        v[3] = fma(eq, in, v[3]);
      }
    } else {
      // Bonus row (clean row k): e = 2^((l - m) c) relative to the row max.
#pragma unroll
      for (int e = 0; e < 8; ++e) v[0] += wexp(a, sh_tab, xp[k][e], sp.mp);
    }
    block_total4(v, sh_red);
    if (tid == 0) {
      D4 r;
      r.x = v[0];
      r.y = v[1];
      r.z = v[2];
      r.w = v[3];
      a.subsum[(size_t)b * a.nsub + sc_lo + k] = r;
    }
  }
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

// The weight of one rescanned element: residual max(0, e_p - rho e_q),
// bonus / p-only e_p (relative to the given reference max).
template <bool VEC, bool F32>
__device__ inline double elem_w(const AccArgs& a, const double* tab, int mode,
                                const Logits8<VEC, F32>& xp, const Logits8<VEC, F32>& xq, int e,
                                double mref, double mq, double rho) {
  if (mode == 0) return fmax(0.0, wexp(a, tab, xp[e], mref) - rho * wexp(a, tab, xq[e], mq));
  return wexp(a, tab, xp[e], mref);
}

// One work-group (four waves) per sequence.  Residual: each thread sums its
// sub-chunks' (S_p, S_q), the block forms S_p / S_q exactly, and the
// sub-chunk weights A - (S_p/S_q) B go to LDS; bonus: the bonus row's
// sub-chunk sums rescaled to its max.  Wave 0 locates t; the chosen
// sub-chunk is then rescanned in float64 by all 256 threads, thread t owning
// its elements 8t .. 8t + 7 (vocabulary order), under a block prefix; the
// thread holding t walks its 8 weights again.
template <bool VEC, bool F32>
__global__ __launch_bounds__(256) void accept_select_kernel(AccArgs a) {
  __shared__ double sh_w[kMaxSubChunks];
  __shared__ double sh_aux[kMaxSubChunks];
  __shared__ double sh_t, sh_base, sh_W;
  __shared__ int sh_sc, sh_past;
  __shared__ double sh_wsum[4];
  __shared__ int sh_last[4];
  __shared__ int sh_tok;
  __shared__ double sh_red[4][4];
  __shared__ double sh_tab[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const SamplePlan sp = a.plan[b];
  if (sp.mode == 2) return;
  if (tid < 64) sh_tab[tid] = exp2t_entry(tid, a.cf);  // ordered by the barriers below
  const int nsub = a.nsub;
  const bool resid = sp.mode == 0;
  double rho = 0.0, Sp = 0.0, M = 0.0;
  if (resid) {
    // S_p, S_q: float64 sums over every element of the two rows (sub-chunk
    // order within a thread, then the fixed block order); the sub-chunk
    // weights A - (S_p/S_q) B.
    const D4* ss = a.subsum + (size_t)b * nsub;
    double v[4] = {0.0, 0.0, 0.0, 0.0};
    for (int c = tid; c < nsub; c += 256) {
      const D4 r = ss[c];
      v[0] += r.x;
      v[1] += r.y;
      sh_w[c] = r.z;
      sh_aux[c] = r.w;
    }
    block_total4(v, sh_red);
    Sp = v[0];
    rho = v[0] / v[1];
    for (int c = tid; c < nsub; c += 256) sh_w[c] = fmax(0.0, sh_w[c] - rho * sh_aux[c]);
  } else {
    // Bonus row: its sub-chunk sums of 2^((l - M) c), M the row max.
    M = sp.mp;
    for (int c = tid; c < nsub; c += 256) sh_w[c] = a.subsum[(size_t)b * nsub + c].x;
  }
  if (tid == 0) sh_tok = -1;
  __syncthreads();
  if (wave == 0) locate(sh_w, nsub, sp.u2, &sh_W, &sh_t, &sh_base, &sh_sc, &sh_past);
  __syncthreads();
  int mode = resid ? 0 : 1;  // 0 residual, 1 bonus, 2 p_j alone (the residual vanished)
  if (resid && !(sh_W > 0.0)) {
    // max(0, p_j - q_j) summed to nothing: sample p_j itself, from the
    // sub-chunk sums of e_p.
    mode = 2;
    for (int c = tid; c < nsub; c += 256) sh_w[c] = a.subsum[(size_t)b * nsub + c].x;
    __syncthreads();
    if (wave == 0) locate(sh_w, nsub, sp.u2, &sh_W, &sh_t, &sh_base, &sh_sc, &sh_past);
    __syncthreads();
  }
  const double W = sh_W, tW = sh_t;
  double base = sh_base;
  const int sc = sh_sc, past = sh_past;
  // t sits in [base, base + sum of the sub-chunk) up to rounding at a
  // sub-chunk boundary; clamping it to base keeps it inside.
  double t = fmax(tW, base);
  const double mref = sp.mp;
  const int v0 = sc * kSub + 8 * tid;
  const Logits8<VEC, F32> xp = load8<VEC, F32>(row_ptr(a, b, sp.row_p), v0, a.V);
  Logits8<VEC, F32> xq;
  if (mode == 0) xq = load8<VEC, F32>(row_ptr(a, b, a.N + sp.row_p), v0, a.V);
  double ls = 0.0;
  int lastp = -1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double we = elem_w<VEC, F32>(a, sh_tab, mode, xp, xq, e, mref, sp.mq, rho);
    ls += we;
    if (we > 0.0) lastp = v0 + e;
  }
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
    // The same weights, in the same order, as the thread sum above.
    double run = lo;
    int tok = lastp;
    bool done = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      run += elem_w<VEC, F32>(a, sh_tab, mode, xp, xq, e, mref, sp.mq, rho);
      if (!done && run > t) {
        tok = v0 + e;
        done = true;
      }
    }
    sh_tok = tok;
  }
  __syncthreads();
  for (int i = tid; i < nsub; i += 256)  // normalised sub-chunk weights, for the dump
    a.subw[(size_t)b * nsub + i] = W > 0.0 ? sh_w[i] / W : NAN;
  if (tid == 0) {
    int tok = sh_tok;
    if (tok < 0) {
      // No holder (t past the total, or a sub-chunk too small to move base):
      // the last element with positive weight.
      for (int q = 3; q >= 0 && tok < 0; --q) tok = sh_last[q];
      if (tok < 0) tok = min(a.V - 1, sc * kSub);
    }
    a.out_tokens[(size_t)b * a.N + sp.j] = tok;
    // The bonus row's statistics, for the probability dump: (M, W) with W in
    // units of 2^((l - M) c).
    if (mode == 1) {
      D4 st;
      st.x = M;
      st.y = W;
      st.z = 1.0;
      st.w = a.c2d;
      a.rowstat[(size_t)b * a.R + sp.kp] = st;
    }
    if (a.debug) {
      // (sum of w, t) in probability units, the uniform, the token.
      double* dbg = a.debug + ((size_t)b * (a.N + 1) + a.N) * 4;
      const double unit = mode == 1 ? W : Sp;
      dbg[0] = W / unit;
      dbg[1] = tW / unit;
      dbg[2] = sp.u2;
      dbg[3] = (double)tok;
    }
  }
}

template <int U, bool VEC, bool F32>
int32_t launch_stats(const AccArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)a.B * a.nrows * a.S1;
  hipLaunchKernelGGL((accept_stats_kernel<U, VEC, F32>), dim3((unsigned)g), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

// Sub-chunks per summing work-group.  The float64 sums are bound by the
// vector ALUs, so small batches spread them over as many work-groups as
// there are sub-chunks (b1 25.5 -> 19.2 us per acceptance against four per
// work-group, b16 38.6 -> 35.1, B = 8 of C = 64 32.4 -> 28.3); C = 64 is
// fastest at two (56.5 us, against 57.8 at one or four), where every
// work-group repeating the decision starts to weigh.  Greedy: the decision
// alone, one work-group per sequence.
inline int sums_per_wg(int64_t B, int nsub, bool greedy) {
  if (greedy) return nsub;
  return std::min(B * nsub <= kOneSubMax ? 1 : kMaxSpw, nsub);
}

template <bool VEC, bool F32>
int32_t launch_all(AccArgs a, hipStream_t s) {
  const int32_t r = launch_stats<kStatsU, VEC, F32>(a, s);
  if (r != IDLM_OK) return r;
  a.spw = sums_per_wg(a.B, a.nsub, a.greedy);
  a.S2 = (a.nsub + a.spw - 1) / a.spw;
  const int64_t g2 = (int64_t)a.B * a.S2;
  hipLaunchKernelGGL((accept_decide_sum_kernel<VEC, F32>), dim3((unsigned)g2), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  if (a.greedy) return IDLM_OK;
  hipLaunchKernelGGL((accept_select_kernel<VEC, F32>), dim3((unsigned)a.B), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Probability dump: p and q over the whole vocabulary from the row
// statistics the last acceptance left in the workspace, with the expression
// the decision evaluates at the drafts, 2^((l - M) c) / S.
// ---------------------------------------------------------------------------
struct DumpArgs {
  const void* lc;
  const void* lm;
  const D4* rowstat;
  const double* subw;
  double* out_p;
  double* out_q;
  double* out_subw;
  Exp2Coef cf;
  int B, N, K, R, V, nsub, f32, chunks;
};

__global__ __launch_bounds__(256) void accept_dump_kernel(DumpArgs a) {
  const int64_t wg = blockIdx.x;
  const int chunk = (int)(wg % a.chunks);
  const int64_t br = wg / a.chunks;
  const int ridx = (int)(br % a.R), b = (int)(br / a.R);
  double* out = ridx < a.N ? (a.out_p ? a.out_p + ((size_t)b * a.N + ridx) * a.V : nullptr)
                           : (a.out_q ? a.out_q + ((size_t)b * a.K + (ridx - a.N)) * a.V : nullptr);
  if (ridx == 0 && chunk == 0 && a.out_subw)
    for (int i = threadIdx.x; i < a.nsub; i += 256)
      a.out_subw[(size_t)b * a.nsub + i] = a.subw[(size_t)b * a.nsub + i];
  if (!out) return;
  const D4 st = a.rowstat[(size_t)b * a.R + ridx];
  const size_t es = a.f32 ? 4 : 2;
  const void* row = ridx < a.N ? (const char*)a.lc + ((size_t)b * a.N + ridx) * a.V * es
                               : (const char*)a.lm + ((size_t)b * a.K + (ridx - a.N)) * a.V * es;
  const int kind = (int)st.z;
  for (int v = chunk * 4096 + threadIdx.x; v < min(a.V, (chunk + 1) * 4096); v += 256) {
    double pv = NAN;
    if (kind == 1) pv = exp2d(((double)load1(row, v, a.f32) - st.x) * st.w, a.cf) / st.y;
    if (kind == 2) pv = v == (int)st.y ? 1.0 : 0.0;
    out[v] = pv;
  }
}

}  // namespace

int64_t accept_max_grid(const idlm_isd_dims& d) {
  const int R = 2 * d.N - 1;
  const int64_t S1 = (d.V + (int64_t)kSub * kStatsU - 1) / ((int64_t)kSub * kStatsU);
  const int nsub = (int)((d.V + kSub - 1) / kSub);
  const int64_t stats = (int64_t)d.B * R * S1;
  const int spw = sums_per_wg(d.B, nsub, false);
  const int64_t sums = (int64_t)d.B * ((nsub + spw - 1) / spw);
  return std::max(stats, sums);
}

int32_t launch_accept(const idlm_isd_dims& d, const Plan& p, const void* lc, const void* lm,
                      const int32_t* drafts, uint64_t seed, float T, int32_t* out_tokens,
                      int32_t* out_len, double* out_debug, char* ws, hipStream_t s,
                      int32_t* status, const void* mstats) {
  if (d.B == 0) return IDLM_OK;
  const AcceptPlan& ap = p.acc;
  AccArgs a;
  a.lc = lc;
  a.lm = lm;
  a.drafts = drafts;
  a.seed = seed;
  a.greedy = (T == 0.0f);
  a.c2 = a.greedy ? 0.f : (float)(1.4426950408889634 / (double)T);
  a.c2d = a.greedy ? 0.0 : 1.4426950408889634 / (double)T;
  a.c64 = 64.0 * a.c2d;
  a.cf = kExp2Coef;
  a.cf64 = kExp2Coef64;
  a.out_tokens = out_tokens;
  a.out_len = out_len;
  a.debug = out_debug;
  a.status = status ? status : (int32_t*)(ws + p.off_status);
  a.stats = (double2*)(ws + p.off_stats);
  a.plan = (SamplePlan*)(ws + p.off_splan);
  a.subsum = (D4*)(ws + p.off_subsum);
  a.dlog = (float*)(ws + p.off_dlog);
  a.unif = (double2*)(ws + p.off_unif);
  a.rowstat = (D4*)(ws + p.off_rowstat);
  a.subw = (double*)(ws + p.off_subw);
  a.mhdr = nullptr;
  a.mst = nullptr;
  a.mdlog = nullptr;
  a.mtok = nullptr;
  a.nrows = ap.R;
  if (mstats && d.N > 1) {
    const MaskStatsLayout ml = mask_stats_layout(d);
    const char* m = (const char*)mstats;
    a.mhdr = (const MaskStatsHeader*)m;
    a.mst = (const double2*)(m + ml.off_st);
    a.mdlog = (const float*)(m + ml.off_dlog);
    a.mtok = (const int32_t*)(m + ml.off_tok);
    a.nrows = d.N;  // the clean rows only
  }
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

int32_t launch_accept_dump(const idlm_isd_dims& d, const Plan& p, const void* lc, const void* lm,
                           float T, const char* ws, double* out_p, double* out_q,
                           double* out_subw, hipStream_t s) {
  (void)T;
  if (d.B == 0) return IDLM_OK;
  DumpArgs a;
  a.lc = lc;
  a.lm = lm;
  a.rowstat = (const D4*)(ws + p.off_rowstat);
  a.subw = (const double*)(ws + p.off_subw);
  a.out_p = out_p;
  a.out_q = d.N > 1 ? out_q : nullptr;
  a.out_subw = out_subw;
  a.cf = kExp2Coef;
  a.B = d.B;
  a.N = d.N;
  a.K = d.N - 1;
  a.R = p.acc.R;
  a.V = d.V;
  a.nsub = p.acc.nsub;
  a.f32 = d.logits_dtype == IDLM_F32;
  a.chunks = (d.V + 4095) / 4096;
  const int64_t grid = (int64_t)d.B * a.R * a.chunks;
  hipLaunchKernelGGL(accept_dump_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

namespace {
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
//   propose_stats   grid B*K*ceil(nsub/4): each wave reduces one 2048-element
//                   sub-chunk to (max m_c, float64 sum of 2^((l - m_c) c),
//                   each weight a table exponential exp2t64) (greedy: max,
//                   lowest argmax).  Rows of sequences that will not continue
//                   are skipped, so their logits are never read.
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
  MaskStatsHeader* mhdr;    // with the next three: the MASK-row statistics record, or null
  double2* mrow;            // [B][K]: each row's (max, sum) or greedy (max, argmax)
  float* mdlog;             // [B][K]
  int32_t* mtok;            // [B][K]
  uint64_t seed;
  float c2;                 // log2(e) / T as float32 (identifies T in the record)
  double c2d;               // log2(e) / T as float64 (sampling weights)
  double c64;               // 64 c2d (exact): exp2t64's argument scale
  Exp2Coef cf;              // for the table of 2^(j/64)
  Exp2Coef64 cf64;
  int greedy, B, K, V, nsub, f32;
};

// Thread 0 of each (b, i) work-group: the draft, and in the MASK-row
// statistics record its logit and the record's header.
__device__ inline void put_draft(const PropArgs& a, int b, int i, int tok) {
  a.next[(size_t)b * a.K + i] = tok;
  if (!a.mtok) return;
  a.mtok[(size_t)b * a.K + i] = tok;
  const size_t es = a.f32 ? 4 : 2;
  const void* row = (const char*)a.ln + ((size_t)b * a.K + i) * a.V * es;
  a.mdlog[(size_t)b * a.K + i] = tok >= 0 ? load1(row, tok, a.f32) : 0.f;
  if (b == 0 && i == 0) {
    MaskStatsHeader h;
    h.magic = kMaskStatsMagic;
    h.c2_bits = __float_as_uint(a.c2);
    h.B = a.B;
    h.K = a.K;
    h.V = a.V;
    h.nsub = a.nsub;
    *a.mhdr = h;
  }
}

// Sub-chunks per wave of propose_stats.  Its float64 weights are bound by
// the vector ALUs and only continuing sequences' rows have work, so one
// sub-chunk per wave spreads them best (c64: 25.8 us per call against 32.6
// with two; float32 weights took 19.9).
constexpr int kPropSubPerWave = 1;

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
  __shared__ double sh_tab[64];  // 2^(j/64), built while the loads are in flight
  if (!a.greedy) {
    if (threadIdx.x < 64) sh_tab[threadIdx.x] = exp2t_entry((int)threadIdx.x, a.cf);
    __syncthreads();
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
      // float64 weights 2^((l - m_c) c) relative to the sub-chunk max (the
      // rescan in propose_select evaluates the same expression).
      double s = 0.0;
      if (m != -INFINITY) {
        const double md = (double)m;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) s += exp2t64(((double)x[k][g][e] - md) * a.c64, sh_tab, a.cf64);
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
  __shared__ double sh_tab[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / a.K, i = blockIdx.x % a.K;
  if (!continues(a, b)) {
    if (tid == 0) {
      put_draft(a, b, i, -1);
      if (a.mrow) a.mrow[(size_t)b * a.K + i] = make_double2(0.0, 0.0);  // no draft: unused
    }
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
    if (lane == 0) {
      put_draft(a, b, i, bi == 0x7FFFFFFF ? 0 : bi);
      if (a.mrow) a.mrow[(size_t)b * a.K + i] = make_double2((double)bv, (double)bi);
    }
    return;
  }
  if (wave == 0) {
    // Wave 0 locates the sub-chunk: weights s_c 2^((m_c - M) c) in order,
    // each lane a contiguous run, a wave scan, the first sub-chunk with
    // positive weight whose end exceeds t = u * W.
    const double c2 = a.c2d;
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
      if (a.mrow) a.mrow[(size_t)b * a.K + i] = make_double2(M, W);  // the row's (max, sum)
    }
  }
  if (tid < 64) sh_tab[tid] = exp2t_entry(tid, a.cf);
  __syncthreads();
  const int sc = sh_sc, past = sh_past;
  const double tl = sh_tl;
  const float mc = sh_mc;
  // Rescan with all 256 threads: thread t owns elements sc*kSub + 8t .. 8t + 7
  // (vocabulary order), under a block prefix of the thread sums.
  const void* row = prop_row(a, b, i);
  const int v0 = sc * kSub + 8 * tid;
  const Logits8<VEC, F32> xs = load8<VEC, F32>(row, v0, a.V);
  double w[8];
  double part = 0.0;
  int lastp = -1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    w[e] = exp2t64(((double)xs[e] - (double)mc) * a.c64, sh_tab, a.cf64);
    part += w[e];
    if (w[e] > 0.0) lastp = v0 + e;
  }
  double inc = part;
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
      r += w[e];
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
    put_draft(a, b, i, tok < 0 ? min(a.V - 1, sc * kSub) : tok);
  }
}

constexpr int kPropSubPerWg = 4 * kPropSubPerWave;

template <bool VEC, bool F32>
int32_t launch_propose_t(PropArgs a, hipStream_t s) {
  const int S = (a.nsub + kPropSubPerWg - 1) / kPropSubPerWg;
  const int64_t g1 = (int64_t)a.B * a.K * S;
  hipLaunchKernelGGL((propose_stats_kernel<VEC, F32>), dim3((unsigned)g1), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  hipLaunchKernelGGL((propose_select_kernel<VEC, F32>), dim3((unsigned)(a.B * a.K)), dim3(256), 0,
                     s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

}  // namespace

}  // namespace idlm

namespace idlm {

int64_t propose_max_grid(const idlm_isd_dims& d) {
  const int64_t nsub = (d.V + kSub - 1) / kSub;
  const int64_t stats = (int64_t)d.B * (d.N - 1) * ((nsub + kPropSubPerWg - 1) / kPropSubPerWg);
  return std::max(stats, (int64_t)d.B * (d.N - 1));
}

int32_t launch_propose(const idlm_isd_dims& d, const Plan& p, const void* logits_next,
                       const int32_t* drafts, const int32_t* accept_len, uint64_t seed, float T,
                       int32_t* next_drafts, char* ws, hipStream_t s, void* mstats) {
  if (d.B == 0 || d.N == 1) return IDLM_OK;
  PropArgs a = {};
  a.ln = logits_next;
  a.drafts = drafts;
  a.accept_len = accept_len;
  a.next = next_drafts;
  a.st = (double2*)(ws + p.off_pstats);
  if (mstats) {
    const MaskStatsLayout ml = mask_stats_layout(d);
    char* m = (char*)mstats;
    a.mhdr = (MaskStatsHeader*)m;
    a.mrow = (double2*)(m + ml.off_st);
    a.mdlog = (float*)(m + ml.off_dlog);
    a.mtok = (int32_t*)(m + ml.off_tok);
  }
  a.seed = seed;
  a.greedy = (T == 0.0f);
  a.c2 = a.greedy ? 0.f : (float)(1.4426950408889634 / (double)T);
  a.c2d = a.greedy ? 0.0 : 1.4426950408889634 / (double)T;
  a.c64 = 64.0 * a.c2d;
  a.cf = kExp2Coef;
  a.cf64 = kExp2Coef64;
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
