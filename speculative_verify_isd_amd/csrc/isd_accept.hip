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
// Two launches, both HBM streams over bfloat16/float32 logits:
//
//   accept_stats  grid = B * R * S1.  Each work-group reduces one slice of
//                 one logit row to (raw max m, sum of exp2((l - m) c)) with
//                 c = log2(e)/T; exponentials in float32, sums in float64.
//                 The last work-group of a sequence (atomic counter) merges
//                 the slices in fixed order, evaluates p_i(x_i) and q_i(x_i)
//                 in float64, draws the Philox uniforms, runs the sequential
//                 ratio test and writes the kept prefix plus a sampling plan.
//   accept_sample grid = B * S2.  Each work-group forms the sampling weights
//                 w (residual or bonus row) over its 2048-element
//                 sub-chunks and stores each sub-chunk's float64 sum.  The
//                 last work-group of a sequence prefixes those sums in order,
//                 finds the sub-chunk holding t = u' * sum(w), recomputes it
//                 and scans it to the token: the smallest v whose running sum
//                 exceeds t.
//
// Every merge runs in a fixed order, so results do not depend on scheduling.
// Counters return to zero after use.
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
  unsigned* cnt1;   // [B]
  unsigned* cnt2;   // [B]
  SamplePlan* plan; // [B]
  double* subsum;   // [B][nsub]
  int B, N, K, R, V, S1, chunk1, nsub, spw, S2, f32, vec_ok;
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

// Eight consecutive logits starting at v (< hi); elements at or past hi read
// as -inf.
__device__ inline void load8(const void* row, int v, int hi, int f32, int vec_ok, float x[8]) {
  if (vec_ok && v + 8 <= hi) {
    if (f32) {
      const float4 p0 = *(const float4*)((const float*)row + v);
      const float4 p1 = *(const float4*)((const float*)row + v + 4);
      x[0] = p0.x; x[1] = p0.y; x[2] = p0.z; x[3] = p0.w;
      x[4] = p1.x; x[5] = p1.y; x[6] = p1.z; x[7] = p1.w;
    } else {
      const uint4 p = *(const uint4*)((const u16*)row + v);
      const unsigned w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (v + e < hi) ? load1(row, v + e, f32) : -INFINITY;
}

// Greedy reduction: larger value wins, lower index on ties.
__device__ inline void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

__device__ inline void wg_argmax(float& bv, int& bi, float* sh_v, int* sh_i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float vo = __shfl_xor(bv, off);
    const int io = __shfl_xor(bi, off);
    better(bv, bi, vo, io);
  }
  if (lane == 0) {
    sh_v[wave] = bv;
    sh_i[wave] = bi;
  }
  __syncthreads();
  bv = sh_v[0];
  bi = sh_i[0];
  for (int w = 1; w < 4; ++w) better(bv, bi, sh_v[w], sh_i[w]);
  __syncthreads();
}

// Inclusive scan of one double per thread over the work-group; every
// thread's inclusive value lands in sh_incl[256].
__device__ inline void wg_scan_incl(double x, double* sh_wave, double* sh_incl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh_wave[wave] = x;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += sh_wave[w];
  sh_incl[threadIdx.x] = base + x;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Kernel 1: row statistics, then the ratio test in the sequence's last WG.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void accept_stats_kernel(AccArgs a) {
  __shared__ double sh_s[4];
  __shared__ float sh_m[4];
  __shared__ int sh_i[4];
  __shared__ double row_m[32], row_s[32];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int64_t wg = blockIdx.x;
  const int c = (int)(wg % a.S1);
  const int64_t tmp = wg / a.S1;
  const int rho = (int)(tmp % a.R);
  const int b = (int)(tmp / a.R);
  const void* row = row_ptr(a, b, rho);
  const int lo = c * a.chunk1;
  const int hi = min(a.V, lo + a.chunk1);

  if (a.greedy) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int v = lo + 8 * tid; v < hi; v += 8 * 256) {
      float x[8];
      load8(row, v, hi, a.f32, a.vec_ok, x);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (v + e < hi) better(bv, bi, x[e], v + e);
    }
    wg_argmax(bv, bi, sh_m, sh_i);
    if (tid == 0) a.stats[((size_t)b * a.R + rho) * a.S1 + c] = make_double2(bv, (double)bi);
  } else {
    float m = -INFINITY;
    double s = 0.0;
    for (int v = lo + 8 * tid; v < hi; v += 8 * 256) {
      float x[8];
      load8(row, v, hi, a.f32, a.vec_ok, x);
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      if (mx > m) {
        if (m != -INFINITY) s *= exp2((double)(m - mx) * (double)a.c2);
        m = mx;
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part += exp2f((x[e] - m) * a.c2);
      s += (double)part;
    }
    // Work-group merge; m is a raw logit, so rescale with the same c2.
    {
      const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float mo = __shfl_xor(m, off);
        const double so = __shfl_xor(s, off);
        const float M = fmaxf(m, mo);
        if (M != -INFINITY)
          s = s * exp2((double)(m - M) * a.c2) + so * exp2((double)(mo - M) * a.c2);
        m = M;
      }
      if (lane == 0) {
        sh_m[wave] = m;
        sh_s[wave] = s;
      }
      __syncthreads();
      if (tid == 0) {
        float M = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));
        double S = 0.0;
        for (int w = 0; w < 4; ++w)
          if (sh_m[w] != -INFINITY) S += sh_s[w] * exp2((double)(sh_m[w] - M) * a.c2);
        a.stats[((size_t)b * a.R + rho) * a.S1 + c] = make_double2((double)M, S);
      }
    }
  }

  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(&a.cnt1[b], 1u);
    is_last = (prev == (unsigned)(a.R * a.S1 - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // ---- finalisation for sequence b (one work-group) ----
  if (tid < a.R) {
    const double2* st = a.stats + ((size_t)b * a.R + tid) * a.S1;
    if (a.greedy) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int k = 0; k < a.S1; ++k) better(bv, bi, (float)st[k].x, (int)st[k].y);
      row_m[tid] = bv;
      row_s[tid] = (double)bi;
    } else {
      double M = -INFINITY;
      for (int k = 0; k < a.S1; ++k) M = fmax(M, st[k].x);
      double S = 0.0;
      for (int k = 0; k < a.S1; ++k)
        if (st[k].x != -INFINITY) S += st[k].y * exp2((st[k].x - M) * (double)a.c2);
      row_m[tid] = M;
      row_s[tid] = S;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int K = a.K, N = a.N;
    const int32_t* dr = a.drafts + (size_t)b * K;
    int kp = K;
    for (int i = 0; i < K; ++i) {
      const int x = dr[i];
      if (x < 0) {
        if (x != -1) atomicOr(a.status, kBadDraft);
        kp = i;
        break;
      }
    }
    double* dbg = a.debug ? a.debug + (size_t)b * (N + 1) * 4 : nullptr;
    if (dbg)
      for (int i = 0; i < 4 * (N + 1); ++i) dbg[i] = NAN;
    int j = kp;
    for (int i = 0; i < kp; ++i) {
      int x = dr[i];
      if (x >= a.V) {
        atomicOr(a.status, kBadDraft);
        x = a.V - 1;
      }
      const U64x4 w = philox4x64_10((uint64_t)i, 0, 0, 0, a.seed, (uint64_t)b);
      const double u = top24(w.w[0]), u2 = top24(w.w[1]);
      double p, q;
      if (a.greedy) {
        p = (x == (int)row_s[i]) ? 1.0 : 0.0;
        q = (x == (int)row_s[N + i]) ? 1.0 : 0.0;
      } else {
        const double lp = (double)load1(row_ptr(a, b, i), x, a.f32);
        const double lq = (double)load1(row_ptr(a, b, N + i), x, a.f32);
        p = exp((lp - row_m[i]) * a.invT) / row_s[i];
        q = exp((lq - row_m[N + i]) * a.invT) / row_s[N + i];
      }
      if (dbg) {
        dbg[4 * i + 0] = p;
        dbg[4 * i + 1] = q;
        dbg[4 * i + 2] = u;
        dbg[4 * i + 3] = u2;
      }
      if (!(p >= q || u * q < p)) {
        j = i;
        break;
      }
    }
    int32_t* ot = a.out_tokens + (size_t)b * N;
    for (int i = 0; i < N; ++i) ot[i] = (i < j) ? dr[i] : -1;
    a.out_len[b] = j + 1;
    const U64x4 wj = philox4x64_10((uint64_t)j, 0, 0, 0, a.seed, (uint64_t)b);
    SamplePlan sp;
    sp.j = j;
    sp.u2 = top24(wj.w[1]);
    sp.row_p = j;
    sp.row_q = (j < kp) ? j : 0;
    sp.mode = (j < kp) ? 0 : 1;
    sp.mp = row_m[j];
    sp.sp = row_s[j];
    sp.mq = (j < kp) ? row_m[N + j] : 0.0;
    sp.sq = (j < kp) ? row_s[N + j] : 1.0;
    sp.pad = 0.0;
    if (a.greedy) {
      // p and q are one-hot: the residual (or its fallback) is the clean argmax.
      const int tok = (int)row_s[j];
      ot[j] = tok;
      sp.mode = 2;
      if (dbg) {
        dbg[4 * N + 0] = 1.0;
        dbg[4 * N + 1] = sp.u2;
        dbg[4 * N + 2] = sp.u2;
        dbg[4 * N + 3] = (double)tok;
      }
    }
    a.plan[b] = sp;
    a.cnt1[b] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: residual / bonus sampling by chunked inverse CDF.
// ---------------------------------------------------------------------------

// Sampling weights of the 8 elements at v (mode 0 residual, 1 p only).
// Exponentials are float32; the normalisation and the difference p - q are
// float64, so p and q keep exactly the scales their row sums gave them and
// the residual carries no systematic float32 scale error.
__device__ inline void weights8(const AccArgs& a, const SamplePlan& sp, int b, int v, double w[8]) {
  const float c2 = a.c2;
  const float mp = (float)sp.mp;
  const double ip = 1.0 / sp.sp;
  float xp[8];
  load8(row_ptr(a, b, sp.row_p), v, a.V, a.f32, a.vec_ok, xp);
  if (sp.mode == 0) {
    const float mq = (float)sp.mq;
    const double iq = 1.0 / sp.sq;
    float xq[8];
    load8(row_ptr(a, b, a.N + sp.row_q), v, a.V, a.f32, a.vec_ok, xq);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      w[e] = fmax(0.0, (double)exp2f((xp[e] - mp) * c2) * ip - (double)exp2f((xq[e] - mq) * c2) * iq);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (double)exp2f((xp[e] - mp) * c2) * ip;
  }
}

// Weights of one sub-chunk (this thread's 8 in w) and the inclusive scan of
// the per-thread sums in sh_incl.  Recomputing a sub-chunk reproduces every
// value bit for bit, so the total stored in the first pass and the scan used
// to locate t agree exactly.
__device__ inline void subchunk_scan(const AccArgs& a, const SamplePlan& sp, int b, int sc,
                                     double w[8], double* sh_wave, double* sh_incl) {
  const int v = sc * kSub + 8 * threadIdx.x;
  weights8(a, sp, b, v, w);
  double ts = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ts += w[e];
  wg_scan_incl(ts, sh_wave, sh_incl);
}

__global__ __launch_bounds__(256) void accept_sample_kernel(AccArgs a) {
  __shared__ double sh_wave[4];
  __shared__ double sh_incl[256];
  __shared__ int is_last;
  __shared__ int found_tok, found_last;
  __shared__ double sh_t, sh_base, sh_W;
  __shared__ int sh_sc, sh_past;

  const int tid = threadIdx.x;
  const int b = (int)(blockIdx.x / a.S2);
  const int w0 = (int)(blockIdx.x % a.S2);
  SamplePlan sp = a.plan[b];
  double* subs = a.subsum + (size_t)b * a.nsub;
  double w[8];

  const int sc_lo = w0 * a.spw, sc_hi = min(a.nsub, sc_lo + a.spw);
  for (int sc = sc_lo; sc < sc_hi; ++sc) {
    subchunk_scan(a, sp, b, sc, w, sh_wave, sh_incl);
    if (tid == 0) subs[sc] = sh_incl[255];
    __syncthreads();
  }

  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(&a.cnt2[b], 1u);
    is_last = (prev == (unsigned)(a.S2 - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // ---- last work-group of sequence b: total, locate, scan ----
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (tid == 0) {
      double W = 0.0;
      for (int sc = 0; sc < a.nsub; ++sc) W += subs[sc];
      sh_W = W;
    }
    __syncthreads();
    if (sh_W > 0.0 || attempt == 1) break;
    // The residual vanished to rounding: fall back to p_j over the whole row.
    sp.mode = 1;
    for (int sc = 0; sc < a.nsub; ++sc) {
      subchunk_scan(a, sp, b, sc, w, sh_wave, sh_incl);
      if (tid == 0) subs[sc] = sh_incl[255];
      __syncthreads();
    }
  }
  if (tid == 0) {
    const double t = sp.u2 * sh_W;
    double cum = 0.0, base = 0.0;
    int sel = -1, lastpos = 0;
    for (int sc = 0; sc < a.nsub; ++sc) {
      const double nx = cum + subs[sc];
      if (subs[sc] > 0.0) lastpos = sc;
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
  const int sc = sh_sc;
  subchunk_scan(a, sp, b, sc, w, sh_wave, sh_incl);
  const int v0 = sc * kSub + 8 * tid;
  int lastp = -1;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (w[e] > 0.0) lastp = v0 + e;
  if (!sh_past) {
    // Thread k owns [base + incl[k-1], base + incl[k]): the intervals tile
    // [base, base + total) exactly, so exactly one thread holds t.
    const double lo = base + (tid ? sh_incl[tid - 1] : 0.0);
    const double hi = base + sh_incl[tid];
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
    a.cnt2[b] = 0u;
  }
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
  a.cnt1 = (unsigned*)(ws + p.off_cnt1);
  a.cnt2 = (unsigned*)(ws + p.off_cnt2);
  a.plan = (SamplePlan*)(ws + p.off_splan);
  a.subsum = (double*)(ws + p.off_subsum);
  a.B = d.B;
  a.N = d.N;
  a.K = d.N - 1;
  a.R = ap.R;
  a.V = d.V;
  a.S1 = ap.S1;
  a.chunk1 = ap.chunk1;
  a.nsub = ap.nsub;
  a.spw = ap.spw;
  a.S2 = ap.S2;
  a.f32 = d.logits_dtype == IDLM_F32;
  const size_t es = a.f32 ? 4 : 2;
  a.vec_ok = ((size_t)d.V * es) % 16 == 0 && ((uintptr_t)lc % 16) == 0 &&
             (lm == nullptr || ((uintptr_t)lm % 16) == 0);
  const int64_t g1 = (int64_t)d.B * ap.R * ap.S1;
  hipLaunchKernelGGL(accept_stats_kernel, dim3((unsigned)g1), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  if (a.greedy) return IDLM_OK;
  const int64_t g2 = (int64_t)d.B * ap.S2;
  hipLaunchKernelGGL(accept_sample_kernel, dim3((unsigned)g2), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

}  // namespace idlm
