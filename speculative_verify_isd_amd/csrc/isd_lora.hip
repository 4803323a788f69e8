// R-ISD's gated LoRA at MASK rows, applied after the base projection, for
// gfx950.
//
// Residual ISD adds a gated LoRA adapter (rank 128) that is active only at
// MASK positions; verify positions use the base weights alone, so their
// outputs are bit-for-bit the base model's ("Introspective Diffusion
// Language Models", section "Lossless R-ISD").  The library takes the base
// projection's float32 accumulator y_base [M][O] and writes the bfloat16
// output: verify rows are y_base rounded (the base-only output exactly; no
// operation of the adapter touches them), MASK rows are
// y_base + scale * (x A^T) B^T rounded once, with the adapter products
// accumulated in float32.  Rows are sequences' blocks of R = 2N-1; row r of
// a block is a MASK row iff r >= N.
//
//   lora_down  partial T = x_mask A^T over one share of H: [Mq][H] x [H][rank],
//              Mq = B*(N-1).  bf16 MFMA (v_mfma_f32_16x16x32_bf16); a
//              work-group is 16 MASK rows x all ranks (one 16-rank block per
//              wave, the x tile shared through L1) x one of KS shares of H,
//              so the loads spread over many compute units.  Further
//              work-groups of the same launch round the verify rows:
//              bf16(y_base), nothing else.
//   lora_sum   T = the KS partials summed in share order (float32).
//   lora_up    MASK rows: T times B^T, scale * that added to y_base and
//              rounded once.  Each float32 T value is split exactly into
//              three bf16 parts, T = hi + mid + lo (8 + 8 + 8 significant
//              bits); every part times a bf16 weight is exact in float32, so
//              three v_mfma_f32_16x16x32_bf16 per 32 ranks accumulate the same
//              float32 products as float32 MFMA would, at the bf16 rate.
//
// Every work-group issues its global loads before it stores anything (stores
// to y_out could alias y_base as far as the compiler knows), so each launch
// costs about one memory round trip per work-group.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "isd_internal.hpp"

namespace idlm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct LoraArgs {
  const float* y_base;    // [M][O]
  const uint16_t* x;      // [M][H] bf16
  const uint16_t* a;      // [rank][H] bf16
  const uint16_t* bw;     // [O][rank] bf16
  uint16_t* y_out;        // [M][O] bf16
  float* tpart;           // [KS][Mq][rank] float32
  float* t;               // [Mq][rank] float32
  float scale;
  int B, N, R, K, M, Mq, H, O, rank;
  int KS, sps;            // shares of H and MFMA steps (32 h) per share
  int vec;                // verify rounding with 16-byte vectors (O % 8 == 0, aligned)
};

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  // NaN stays NaN (quiet, sign kept); the bias below would carry a NaN
  // whose payload sits in the low half into infinity or zero.
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Full-M row of MASK row q (q = b * K + i) and of verify row v (v = b * N + r).
__device__ inline int mask_row(const LoraArgs& a, int q) { return (q / a.K) * a.R + a.N + q % a.K; }
__device__ inline int verify_row(const LoraArgs& a, int v) { return (v / a.N) * a.R + v % a.N; }

constexpr int kDownThreads = 512;    // lora_down: 8 waves, one 16-rank block each
constexpr int kDownBlocks = kDownThreads / 64;
constexpr int kStepsPerShare = 8;   // target MFMA steps per share of H
constexpr int kMaxShares = 64;
constexpr int kRoundPerThread = 8;  // verify elements per rounding thread
constexpr int kRoundPerGroup = kDownThreads * kRoundPerThread;

// Shares of H for the down projection: about kStepsPerShare steps each.
inline int lora_shares(int H) {
  const int steps = H / 32;
  return std::min(kMaxShares, std::max(1, (steps + kStepsPerShare - 1) / kStepsPerShare));
}

// Down-launch work-groups that round verify rows (after the T work-groups).
inline int64_t round_groups(const LoraArgs& a) {
  return ((int64_t)a.B * a.N * a.O + kRoundPerGroup - 1) / kRoundPerGroup;
}

__device__ void round_verify(const LoraArgs& a, int64_t wg) {
  const int tid = threadIdx.x;
  const int64_t nv = (int64_t)a.B * a.N * a.O;
  if (a.vec) {
    // 8 columns of one row per element group; kRoundPerThread / 8 groups per thread.
    const int o8n = a.O / 8;
    const int64_t g = wg * kDownThreads + tid;
    if (g * 8 >= nv) return;
    const int v = (int)(g / o8n), o = 8 * (int)(g % o8n);
    const size_t base = (size_t)verify_row(a, v) * a.O + o;
    const float4 lo = *(const float4*)(a.y_base + base);
    const float4 hi = *(const float4*)(a.y_base + base + 4);
    uint4 w;
    w.x = f32_to_bf16_rne(lo.x) | ((unsigned)f32_to_bf16_rne(lo.y) << 16);
    w.y = f32_to_bf16_rne(lo.z) | ((unsigned)f32_to_bf16_rne(lo.w) << 16);
    w.z = f32_to_bf16_rne(hi.x) | ((unsigned)f32_to_bf16_rne(hi.y) << 16);
    w.w = f32_to_bf16_rne(hi.z) | ((unsigned)f32_to_bf16_rne(hi.w) << 16);
    *(uint4*)(a.y_out + base) = w;
    return;
  }
  // Any O: element idx = wg * kRoundPerGroup + e * kDownThreads + tid.
  float val[kRoundPerThread];
  size_t off[kRoundPerThread];
#pragma unroll
  for (int e = 0; e < kRoundPerThread; ++e) {
    const int64_t idx = wg * kRoundPerGroup + (int64_t)e * kDownThreads + tid;
    const int64_t ic = idx < nv ? idx : nv - 1;  // clamped, unconditional load
    off[e] = (size_t)verify_row(a, (int)(ic / a.O)) * a.O + ic % a.O;
    val[e] = a.y_base[off[e]];
  }
#pragma unroll
  for (int e = 0; e < kRoundPerThread; ++e) {
    const int64_t idx = wg * kRoundPerGroup + (int64_t)e * kDownThreads + tid;
    if (idx < nv) a.y_out[off[e]] = f32_to_bf16_rne(val[e]);
  }
}

// Grid: ceil(Mq/16) row tiles x ceil(rank/128) rank groups x KS shares, then
// round_groups.  Wave w of a T work-group computes rank block 16 w of its
// group over its share's steps.
__global__ __launch_bounds__(kDownThreads) void lora_down_kernel(LoraArgs a) {
  const int nrg = (a.rank + 16 * kDownBlocks - 1) / (16 * kDownBlocks);
  const int ntile = (a.Mq + 15) / 16 * nrg * a.KS;
  if ((int)blockIdx.x >= ntile) {
    round_verify(a, (int64_t)blockIdx.x - ntile);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = blockIdx.x % a.KS;
  const int rg = (blockIdx.x / a.KS) % nrg;
  const int mt = blockIdx.x / (a.KS * nrg);
  const int j0 = (rg * kDownBlocks + wave) * 16;
  if (j0 >= a.rank) return;  // wave-uniform
  // A operand: x row (lane % 16), 8 consecutive h at 8 * (lane / 16);
  // B operand: A row j0 + lane % 16, the same h.
  const int qa = min(mt * 16 + (lane & 15), a.Mq - 1);
  const uint16_t* xr = a.x + (size_t)mask_row(a, qa) * a.H + 8 * (lane >> 4);
  const uint16_t* ar = a.a + (size_t)(j0 + (lane & 15)) * a.H + 8 * (lane >> 4);
  const int steps = a.H / 32;
  const int s_lo = min(ks * a.sps, steps), s_hi = min(s_lo + a.sps, steps);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kBatch = 8;  // steps whose loads are in flight together
  for (int s0 = s_lo; s0 < s_hi; s0 += kBatch) {
    bf16x8 xa[kBatch], wa[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // clamped, unconditional
      const int h = 32 * min(s0 + u, s_hi - 1);
      xa[u] = __builtin_bit_cast(bf16x8, *(const uint4*)(xr + h));
      wa[u] = __builtin_bit_cast(bf16x8, *(const uint4*)(ar + h));
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (s0 + u < s_hi) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u], wa[u], acc, 0, 0, 0);
  }
  // acc[e]: MASK row 16 mt + 4 (lane / 16) + e, rank j0 + lane % 16.
  float* tp = a.tpart + (size_t)ks * a.Mq * a.rank;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int q = mt * 16 + 4 * (lane >> 4) + e;
    if (q < a.Mq) tp[(size_t)q * a.rank + j0 + (lane & 15)] = acc[e];
  }
}

// T = sum over shares ks = 0, 1, ... of the partials, one float4 per thread;
// the loads of up to 16 shares are in flight together.
constexpr int kSumThreads = 64;  // small work-groups: the partials spread over many CUs

__global__ __launch_bounds__(kSumThreads) void lora_sum_kernel(LoraArgs a) {
  const int64_t n4 = (int64_t)a.Mq * a.rank / 4;
  const int64_t i = (int64_t)blockIdx.x * kSumThreads + threadIdx.x;
  if (i >= n4) return;
  const float4* p = (const float4*)a.tpart + i;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < a.KS; k0 += 16) {
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = p[(size_t)min(k0 + u, a.KS - 1) * n4];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (k0 + u < a.KS) {
        sum.x += v[u].x;
        sum.y += v[u].y;
        sum.z += v[u].z;
        sum.w += v[u].w;
      }
  }
  ((float4*)a.t)[i] = sum;
}

// LDS of a lora_up work-group with NB 16-column blocks per wave: the three
// bf16 parts of T [3][16][rank] and B [64 NB][rank] bf16, rows padded by 8
// elements (16-byte aligned for vector reads, on different banks).
// Rows hold the ranks rounded up to 32 (the MFMA's k, zero beyond the rank)
// plus 8 elements of padding.
inline int up_stride(int rank) { return (rank + 31) / 32 * 32 + 8; }
inline size_t up_lds(int rank, int NB) { return (size_t)(3 * 16 + 64 * NB) * up_stride(rank) * 2; }
// One 16-column block per wave (64 columns per work-group): more, smaller
// work-groups measured faster than 128-column tiles (7.4 vs 8.2 us at
// M = 448, H = O = 4096, rank 128); LDS stays under 50 KiB up to rank 256.
constexpr int kUpBlocks = 1;

// Grid: ceil(Mq/16) row tiles x ceil(O / (64 NB)) column tiles.  T rows and
// weight rows are staged in LDS, then each wave runs NB 16x16 float32 MFMA
// blocks over the rank and writes bf16(y_base + scale * delta).
template <int NB>
__global__ __launch_bounds__(256) void lora_up_kernel(LoraArgs a) {
  extern __shared__ float sh[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int cols = 64 * NB;
  const int nct = (a.O + cols - 1) / cols;
  const int mt = blockIdx.x / nct, ct = blockIdx.x % nct;
  const int row = lane & 15, kq = lane >> 4;
  // This lane's outputs: MASK row 16 mt + 4 kq + e, column of block c.
  // Their y_base values are loaded first, with the staging loads.
  float yb[NB][4];
  size_t yo[NB][4];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int o = min(ct * cols + wave * 16 * NB + c * 16 + row, a.O - 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = min(mt * 16 + 4 * kq + e, a.Mq - 1);
      yo[c][e] = (size_t)mask_row(a, q) * a.O + o;
      yb[c][e] = a.y_base[yo[c][e]];
    }
  }
  const int rk = (a.rank + 31) / 32 * 32;   // ranks rounded up to the MFMA's k
  const int str = rk + 8;                     // padded row stride (elements)
  uint16_t* sh_t = (uint16_t*)sh;            // [3][16][str]: hi, mid, lo parts of T
  uint16_t* sh_b = sh_t + 3 * 16 * str;      // [cols][str]
  if (rk != a.rank) {  // ranks [rank, rk) of every row are zero (16 elements)
    for (int i = tid; i < (3 * 16 + cols) * 2; i += 256)
      *(uint4*)(sh_t + (i >> 1) * str + a.rank + 8 * (i & 1)) = make_uint4(0, 0, 0, 0);
  }
  // T rows (16 x rank float32: at most 4 float4 per thread) and the first
  // 2048 16-byte pieces of the weight rows are loaded together.
  const int r4 = a.rank / 4, rc8 = a.rank / 8;
  float4 tv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = u * 256 + tid;
    const int q = min(mt * 16 + i / r4, a.Mq - 1);
    tv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < 16 * r4) tv[u] = *(const float4*)(a.t + (size_t)q * a.rank + 4 * (i % r4));
  }
  for (int i0 = 0; i0 < cols * rc8; i0 += 8 * 256) {
    uint4 bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      const int o = min(ct * cols + i / rc8, a.O - 1);  // clamped rows are never used
      bv[u] = make_uint4(0, 0, 0, 0);
      if (i < cols * rc8) bv[u] = *(const uint4*)(a.bw + (size_t)o * a.rank + 8 * (i % rc8));
    }
    if (i0 == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = u * 256 + tid;
        if (i < 16 * r4) {
          const float x[4] = {tv[u].x, tv[u].y, tv[u].z, tv[u].w};
          unsigned part[3][2];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // Exact split: each residual is representable, the last part exactly.
            const uint16_t h = f32_to_bf16_rne(x[e]);
            const float r1 = x[e] - __uint_as_float((unsigned)h << 16);
            const uint16_t m = f32_to_bf16_rne(r1);
            const float r2 = r1 - __uint_as_float((unsigned)m << 16);
            const uint16_t l = f32_to_bf16_rne(r2);
            const int sh16 = 16 * (e & 1);
            if ((e & 1) == 0) part[0][e >> 1] = part[1][e >> 1] = part[2][e >> 1] = 0u;
            part[0][e >> 1] |= (unsigned)h << sh16;
            part[1][e >> 1] |= (unsigned)m << sh16;
            part[2][e >> 1] |= (unsigned)l << sh16;
          }
#pragma unroll
          for (int pp = 0; pp < 3; ++pp)
            *(uint2*)(sh_t + (pp * 16 + i / r4) * str + 4 * (i % r4)) =
                make_uint2(part[pp][0], part[pp][1]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < cols * rc8) *(uint4*)(sh_b + (i / rc8) * str + 8 * (i % rc8)) = bv[u];
    }
  }
  __syncthreads();
  // A operand: part of T[row][kk + 8 kq .. + 7]; B operand: B[col][same k].
  f32x4 acc[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < rk; kk += 32) {
    const int k = kk + 8 * kq;
    const bf16x8 th = __builtin_bit_cast(bf16x8, *(const uint4*)(sh_t + (0 * 16 + row) * str + k));
    const bf16x8 tm = __builtin_bit_cast(bf16x8, *(const uint4*)(sh_t + (1 * 16 + row) * str + k));
    const bf16x8 tl = __builtin_bit_cast(bf16x8, *(const uint4*)(sh_t + (2 * 16 + row) * str + k));
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const bf16x8 bq = __builtin_bit_cast(
          bf16x8, *(const uint4*)(sh_b + (wave * 16 * NB + c * 16 + row) * str + k));
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl, bq, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tm, bq, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th, bq, acc[c], 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int o = ct * cols + wave * 16 * NB + c * 16 + row;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = mt * 16 + 4 * kq + e;
      if (o < a.O && q < a.Mq) a.y_out[yo[c][e]] = f32_to_bf16_rne(yb[c][e] + a.scale * acc[c][e]);
    }
  }
}

}  // namespace

// Work-items of the three launches for these sizes: down (with the verify
// rounding groups), partial sum, up.  Host only.
void gated_lora_work_items(const idlm_isd_lora_dims& L, int64_t items[3]) {
  const int64_t Mq = (int64_t)L.B * (L.N - 1);
  const int64_t nrg = (L.rank + 16 * kDownBlocks - 1) / (16 * kDownBlocks);
  const int64_t rounds = ((int64_t)L.B * L.N * L.O + kRoundPerGroup - 1) / kRoundPerGroup;
  const int64_t g1 = (Mq + 15) / 16 * nrg * lora_shares(L.H) + rounds;
  const int64_t gs = (Mq * L.rank / 4 + kSumThreads - 1) / kSumThreads;
  const int64_t g2 = (Mq + 15) / 16 * ((L.O + 64 * kUpBlocks - 1) / (64 * kUpBlocks));
  items[0] = g1 * kDownThreads;
  items[1] = gs * kSumThreads;
  items[2] = g2 * 256;
}

size_t gated_lora_workspace(const idlm_isd_lora_dims& L) {
  return (size_t)(lora_shares(L.H) + 1) * L.B * (L.N - 1) * L.rank * sizeof(float);
}

int32_t launch_gated_lora(const idlm_isd_lora_dims& L, const float* y_base, const void* x,
                          const void* lora_a, const void* lora_b, float scale, void* y_out,
                          char* ws, hipStream_t s) {
  LoraArgs a;
  a.y_base = y_base;
  a.x = (const uint16_t*)x;
  a.a = (const uint16_t*)lora_a;
  a.bw = (const uint16_t*)lora_b;
  a.y_out = (uint16_t*)y_out;
  a.scale = scale;
  a.B = L.B;
  a.N = L.N;
  a.R = 2 * L.N - 1;
  a.K = L.N - 1;
  a.M = L.B * a.R;
  a.Mq = L.B * a.K;
  a.H = L.H;
  a.O = L.O;
  a.rank = L.rank;
  a.KS = lora_shares(a.H);
  a.sps = (a.H / 32 + a.KS - 1) / a.KS;
  a.tpart = (float*)ws;
  a.t = a.tpart + (size_t)a.KS * a.Mq * a.rank;
  a.vec = (a.O % 8 == 0) && ((((uintptr_t)y_base) | (uintptr_t)y_out) & 15) == 0;
  if (a.M == 0) return IDLM_OK;
  const int nrg = (a.rank + 16 * kDownBlocks - 1) / (16 * kDownBlocks);
  const int64_t g1 = (int64_t)(a.Mq + 15) / 16 * nrg * a.KS + round_groups(a);
  hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)g1), dim3(kDownThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  if (a.Mq == 0) return IDLM_OK;
  const unsigned gs = (unsigned)(((int64_t)a.Mq * a.rank / 4 + kSumThreads - 1) / kSumThreads);
  hipLaunchKernelGGL(lora_sum_kernel, dim3(gs), dim3(kSumThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return IDLM_ERR_HIP;
  constexpr int NB = kUpBlocks;
  const unsigned g2 = (unsigned)((a.Mq + 15) / 16 * ((a.O + 64 * NB - 1) / (64 * NB)));
  hipLaunchKernelGGL((lora_up_kernel<NB>), dim3(g2), dim3(256), up_lds(a.rank, NB), s, a);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

}  // namespace idlm
