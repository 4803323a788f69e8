// C ABI of libidlm_isd.so: host validation, workspace planning and dispatch.
// Validation and planning are plain host code and never touch the GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "isd_internal.hpp"

namespace idlm {
namespace {

// idlm_isd_step runs the acceptance on a second stream of its own, forked
// from the caller's stream and joined back to it with events: the two stages
// read different inputs and write disjoint workspace regions (the sticky
// status word is set with atomic ORs), and run side by side on the chip.
// One set per device, created once; enqueueing a fork holds that device's
// mutex so the event record / wait pairs of concurrent host threads on one
// device do not interleave (steps on different devices do not wait for each
// other).  The events release at device scope: both streams run on the one
// device, where that orders every earlier write of either stream for the
// other (the system-scope default also serves the host, which synchronises
// for itself); per step at C = 64 this saved 1.2 us, at N = 8 9 us.
struct ForkSet {
  hipStream_t aux = nullptr;
  hipEvent_t start = nullptr, done = nullptr;
  bool ok = false;
};
constexpr int kMaxDevices = 64;
ForkSet g_fork[kMaxDevices];
// The event hand-over between the streams adds ~30 us of latency on this
// runtime, so a step forks only when its acceptance reads at least this many
// logits (B * R * V).  Measured per step: B = 16, V = 151936 (17M logits)
// 87.9 -> 81.2 us; C = 64 (68M) 414 -> 394 us; B = 1 (1M) 38.7 -> 66.8 us.
constexpr int64_t kForkMinLogits = (int64_t)1 << 23;
std::mutex g_fork_mu[kMaxDevices];

// The current device, or -1 when it cannot be had or lies past the sets.
int fork_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

// Device dev's set (created on first use), or nullptr when it cannot be had;
// the caller holds g_fork_mu[dev].
ForkSet* fork_set(int dev) {
  ForkSet& f = g_fork[dev];
  if (f.ok) return &f;
  if (!f.aux && hipStreamCreateWithFlags(&f.aux, hipStreamNonBlocking) != hipSuccess) {
    f.aux = nullptr;
    return nullptr;
  }
  if (!f.start && hipEventCreateWithFlags(&f.start, hipEventDisableTiming | hipEventReleaseToDevice) != hipSuccess) {
    f.start = nullptr;
    return nullptr;
  }
  if (!f.done && hipEventCreateWithFlags(&f.done, hipEventDisableTiming | hipEventReleaseToDevice) != hipSuccess) {
    f.done = nullptr;
    return nullptr;
  }
  f.ok = true;
  return &f;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A launch's work-items (work-groups x threads) must fit the 32-bit grid
// size of a dispatch.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;
bool grid_fits(int64_t groups, int64_t threads) {
  return groups >= 0 && groups <= kMaxWorkItems / threads;
}

int32_t check_dims(const idlm_isd_dims* d) {
  if (!d) return IDLM_ERR_NULL;
  if (d->B < 0 || d->B > (1 << 24)) return IDLM_ERR_DIMS;
  if (d->N < 1 || d->N > 16) return IDLM_ERR_DIMS;
  if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return IDLM_ERR_DIMS;
  if (d->V < 1 || d->page_size < 1 || d->max_pages < 1 || d->num_pages < 1) return IDLM_ERR_DIMS;
  if ((int64_t)d->max_pages * 16 > (1ll << 30)) return IDLM_ERR_DIMS;
  if (d->qkv_dtype != IDLM_BF16 && d->qkv_dtype != IDLM_F32) return IDLM_ERR_DIMS;
  if (d->logits_dtype != IDLM_BF16 && d->logits_dtype != IDLM_F32) return IDLM_ERR_DIMS;
  if (d->page_size != kPage) return IDLM_ERR_UNSUPPORTED;
  if (d->D != 64 && d->D != 128) return IDLM_ERR_UNSUPPORTED;
  if ((int64_t)d->V > (int64_t)kSub * kMaxSubChunks) return IDLM_ERR_UNSUPPORTED;
  const int64_t R = 2 * (int64_t)d->N - 1;
  if (R * (d->Hq / d->Hkv) > 128) return IDLM_ERR_UNSUPPORTED;
  if ((int64_t)d->B * d->Hkv > (1 << 24)) return IDLM_ERR_DIMS;
  // Every grid the sizes imply must fit one dispatch: the attention's merge
  // and float32 kernels (one work-group per (b, KV head)), the acceptance
  // (greedy and sampled), its probability dump, the proposals and the KV
  // scatter (one work-item per 8 dims of a row's head).
  const int64_t B = d->B;
  bool ok = grid_fits(B * d->Hkv, 256);
  ok = ok && grid_fits(accept_max_grid(*d), 256);
  ok = ok && grid_fits(B * R * ceil_div(d->V, 4096), 256);
  ok = ok && grid_fits(propose_max_grid(*d), 256);
  ok = ok && grid_fits(B * R * d->Hkv * (d->D / 8), 1);
  if (!ok) return IDLM_ERR_UNSUPPORTED;
  return IDLM_OK;
}

// T >= 0 and finite; a positive T below the smallest normal float (2^-126)
// is refused: log2(e)/T, the scale of every exponent, would overflow float32.
int32_t check_T(float T) {
  if (!(T >= 0.0f) || !isfinite(T)) return IDLM_ERR_TEMPERATURE;
  if (T > 0.0f && T < 0x1.0p-126f) return IDLM_ERR_TEMPERATURE;
  return IDLM_OK;
}

// The acceptance's scratch from offset o on: sampling plans, slice
// statistics, four sums per sub-chunk (residual pair, or the bonus row's in
// .x), draft logits, uniforms; what the probability dump reads (row
// statistics, sub-chunk weights).  Returns the end offset.
size_t layout_accept(const idlm_isd_dims& d, const AcceptPlan& c, size_t o, Plan* p) {
  p->off_splan = o;
  o = align256(o + (size_t)d.B * sizeof(SamplePlan));
  p->off_stats = o;
  o = align256(o + (size_t)d.B * c.R * c.S1 * 16);
  p->off_subsum = o;
  o = align256(o + (size_t)d.B * c.nsub * 32);
  p->off_dlog = o;
  o = align256(o + (size_t)d.B * c.R * 4);
  p->off_unif = o;
  o = align256(o + (size_t)d.B * 16 * 16);
  p->off_rowstat = o;
  o = align256(o + (size_t)d.B * c.R * 32);
  p->off_subw = o;
  o = align256(o + (size_t)d.B * c.nsub * 8);
  return o;
}

}  // namespace

MaskStatsLayout mask_stats_layout(const idlm_isd_dims& d) {
  MaskStatsLayout m;
  const size_t BK = (size_t)d.B * (d.N - 1);
  m.off_st = 256;
  m.off_dlog = align256(m.off_st + BK * 16);
  m.off_tok = align256(m.off_dlog + BK * 4);
  m.total = align256(m.off_tok + BK * 4);
  return m;
}

bool make_plan(const idlm_isd_dims& d, Plan* p) {
  if (check_dims(&d) != IDLM_OK) return false;
  memset(p, 0, sizeof(*p));
  // ---- attention ----
  AttnPlan& a = p->attn;
  a.R = 2 * d.N - 1;
  a.G = d.Hq / d.Hkv;
  a.RG = a.R * a.G;
  // 16-row MFMA blocks per wave and waves per run: one wave of 32 or 64
  // rows, else two waves of 64 rows walking the same run.
  a.RB = a.RG <= 32 ? 2 : 4;
  a.WR = a.RG <= 64 ? 1 : 2;
  a.RGp = 16 * a.RB * a.WR;
  a.npairs = d.B * d.Hkv;
  a.max_lanes = kMaxWaves / a.WR;
  // ---- acceptance ----
  AcceptPlan& c = p->acc;
  c.R = 2 * d.N - 1;
  c.nsub = (int)ceil_div(d.V, kSub);
  c.S1 = (int)ceil_div(d.V, (int64_t)kSub * kStatsU);
  // ---- workspace layout ----
  // [0, state_end): the sticky status word, the only state kept between
  // calls (zeroed by workspace_init).  Everything after it is scratch that
  // every call writes before it reads (launch boundaries order each
  // hand-over).
  size_t o = 0;
  p->off_status = o;
  o = align256(o + 4);
  p->state_end = o;
  // Streaming attention: two partial-state slots per wave-lane (bf16 path).
  const size_t nslots = d.qkv_dtype == IDLM_BF16 ? (size_t)a.max_lanes * 2 : 0;
  p->off_attn_ml = o;
  o = align256(o + nslots * a.RGp * 8);
  p->off_attn_o = o;
  o = align256(o + nslots * a.RGp * d.D * 4);
  o = layout_accept(d, c, o, p);
  p->off_kv_valid = o;
  o = align256(o + (size_t)d.B);
  // Proposal statistics: (max, sum) per sub-chunk of every next-step MASK row.
  p->off_pstats = o;
  o = align256(o + (size_t)d.B * (d.N - 1) * c.nsub * 16);
  p->total = o;
  return true;
}

__global__ void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// ---- the allocation-free acceptance's scratch ----
// One static array per GPU: each device that loads the library's code object
// holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, looked up once per device
// (with that device current) and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = IDLM_ISD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`.
int32_t scratch_ptr(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return IDLM_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return IDLM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return IDLM_OK;
}

int32_t launch_fill_zero(void* ws, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes % 16;
  const unsigned blocks = (unsigned)std::min<size_t>(4096, std::max<size_t>(1, (n16 + 255) / 256));
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, (uint4*)ws, n16,
                     (unsigned char*)ws + n16 * 16, ntail);
  return hipGetLastError() == hipSuccess ? IDLM_OK : IDLM_ERR_HIP;
}

}  // namespace idlm

using namespace idlm;

extern "C" {

size_t idlm_isd_workspace_bytes(const idlm_isd_dims* d) {
  Plan p;
  if (!d || !make_plan(*d, &p)) return 0;
  return p.total;
}

size_t idlm_isd_workspace_state_bytes(const idlm_isd_dims* d) {
  Plan p;
  if (!d || !make_plan(*d, &p)) return 0;
  return p.state_end;
}

size_t idlm_isd_mask_stats_bytes(const idlm_isd_dims* d) {
  if (!d || check_dims(d) != IDLM_OK) return 0;
  return mask_stats_layout(*d).total;
}

int32_t idlm_isd_validate(const idlm_isd_dims* d, float T) {
  const int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  return check_T(T);
}

int32_t idlm_isd_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace) return IDLM_ERR_NULL;
  if (((uintptr_t)workspace & 255) != 0) return IDLM_ERR_WORKSPACE;
  const int dev = fork_device();
  if (dev >= 0) {  // the step's second stream and events, made here outside any capture
    std::lock_guard<std::mutex> g(g_fork_mu[dev]);
    fork_set(dev);
  }
  if (ws_bytes == 0) return IDLM_OK;
  return launch_fill_zero(workspace, ws_bytes, (hipStream_t)stream);
}

static int32_t check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (!ws) return IDLM_ERR_NULL;
  if (((uintptr_t)ws & 255) != 0 || ws_bytes < p.total) return IDLM_ERR_WORKSPACE;
  return IDLM_OK;
}

int32_t idlm_isd_paged_attn(const idlm_isd_dims* d, const void* q, const void* kv_pages,
                            const int32_t* page_table, const int32_t* ctx_lens, void* attn_out,
                            void* workspace, size_t ws_bytes, void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  if ((r = check_ws(p, workspace, ws_bytes)) != IDLM_OK) return r;
  if (d->B == 0) return IDLM_OK;
  if (!q || !kv_pages || !page_table || !ctx_lens || !attn_out) return IDLM_ERR_NULL;
  return launch_paged_attn(*d, p, q, kv_pages, page_table, ctx_lens, attn_out, (char*)workspace,
                           (hipStream_t)stream);
}

int32_t idlm_isd_accept(const idlm_isd_dims* d, const void* logits_clean, const void* logits_mask,
                        const int32_t* draft_tokens, uint64_t seed, float T, int32_t* out_tokens,
                        int32_t* out_accept_len, double* out_debug, const void* mask_stats,
                        void* workspace, size_t ws_bytes, void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  if ((r = check_T(T)) != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  if ((r = check_ws(p, workspace, ws_bytes)) != IDLM_OK) return r;
  if (((uintptr_t)mask_stats & 255) != 0) return IDLM_ERR_WORKSPACE;
  if (d->B == 0) return IDLM_OK;
  if (!logits_clean || !out_tokens || !out_accept_len) return IDLM_ERR_NULL;
  if (d->N > 1 && (!logits_mask || !draft_tokens)) return IDLM_ERR_NULL;
  return launch_accept(*d, p, logits_clean, logits_mask, draft_tokens, seed, T, out_tokens,
                       out_accept_len, out_debug, (char*)workspace, (hipStream_t)stream,
                       nullptr, mask_stats);
}

int32_t idlm_isd_accept_noalloc(const idlm_isd_dims* d, const void* logits_clean,
                                const void* logits_mask, const int32_t* draft_tokens,
                                uint64_t seed, float T, int32_t* out_tokens,
                                int32_t* out_accept_len, double* out_debug,
                                const void* mask_stats, int32_t* out_status, void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  if ((r = check_T(T)) != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  // The acceptance's buffers alone, packed after the status word.
  p.off_status = 0;
  if (layout_accept(*d, p.acc, 256, &p) > kNoAllocScratchBytes) return IDLM_ERR_SCRATCH;
  if (((uintptr_t)mask_stats & 255) != 0) return IDLM_ERR_WORKSPACE;
  if (d->B == 0) return IDLM_OK;
  if (!logits_clean || !out_tokens || !out_accept_len) return IDLM_ERR_NULL;
  if (d->N > 1 && (!logits_mask || !draft_tokens)) return IDLM_ERR_NULL;
  char* base = nullptr;
  if ((r = scratch_ptr(&base)) != IDLM_OK) return r;
  hipStream_t s = (hipStream_t)stream;
  // The status word is the only scratch read before this call writes it:
  // cleared by a fill kernel (no memset node under graph capture).
  int32_t* status = out_status ? out_status : (int32_t*)(base + p.off_status);
  if ((r = launch_fill_zero(status, sizeof(int32_t), s)) != IDLM_OK) return r;
  return launch_accept(*d, p, logits_clean, logits_mask, draft_tokens, seed, T, out_tokens,
                       out_accept_len, out_debug, base, s, status, mask_stats);
}

int32_t idlm_isd_accept_probs(const idlm_isd_dims* d, const void* logits_clean,
                              const void* logits_mask, float T, const void* workspace,
                              size_t ws_bytes, double* out_p, double* out_q, double* out_subw,
                              void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  if ((r = check_T(T)) != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  if ((r = check_ws(p, (void*)workspace, ws_bytes)) != IDLM_OK) return r;
  if (d->B == 0) return IDLM_OK;
  if (!logits_clean || (d->N > 1 && !logits_mask)) return IDLM_ERR_NULL;
  return launch_accept_dump(*d, p, logits_clean, logits_mask, T, (const char*)workspace, out_p,
                            out_q, out_subw, (hipStream_t)stream);
}

// The next step's proposals of a loop step (absent for idlm_isd_step).
struct NextProposals {
  const void* logits_next;
  int32_t* next_drafts;
  void* mask_stats_next;
};

static int32_t step_impl(const idlm_isd_dims* d, const void* q, const void* kv_pages,
                         const int32_t* page_table, const int32_t* ctx_lens,
                         const void* logits_clean, const void* logits_mask,
                         const int32_t* draft_tokens, uint64_t seed, int32_t N, float T,
                         int32_t* out_tokens, int32_t* out_accept_len, void* attn_out,
                         const void* mask_stats, const NextProposals* np, void* workspace,
                         size_t ws_bytes, void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  if (N != d->N) return IDLM_ERR_DIMS;
  if ((r = check_T(T)) != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  if ((r = check_ws(p, workspace, ws_bytes)) != IDLM_OK) return r;
  if (((uintptr_t)mask_stats & 255) != 0) return IDLM_ERR_WORKSPACE;
  if (d->B == 0) return IDLM_OK;
  if (!q || !kv_pages || !page_table || !ctx_lens || !attn_out) return IDLM_ERR_NULL;
  if (!logits_clean || !out_tokens || !out_accept_len) return IDLM_ERR_NULL;
  if (d->N > 1 && (!logits_mask || !draft_tokens)) return IDLM_ERR_NULL;
  if (np) {
    if (((uintptr_t)np->mask_stats_next & 255) != 0) return IDLM_ERR_WORKSPACE;
    if (d->N > 1 && (!np->logits_next || !np->next_drafts)) return IDLM_ERR_NULL;
  }
  hipStream_t s = (hipStream_t)stream;
  const int64_t logits = (int64_t)d->B * (2 * d->N - 1) * d->V;
  const int dev = logits >= kForkMinLogits ? fork_device() : -1;
  // Held for the whole enqueue: the fork's events are shared by the
  // device's steps.
  std::unique_lock<std::mutex> g;
  if (dev >= 0) g = std::unique_lock<std::mutex>(g_fork_mu[dev]);
  ForkSet* f = dev >= 0 ? fork_set(dev) : nullptr;
  hipStream_t sa = s;  // the acceptance's stream: the fork, or `stream` itself without one
  if (f) {
    if (hipEventRecord(f->start, s) != hipSuccess) return IDLM_ERR_HIP;
    if (hipStreamWaitEvent(f->aux, f->start, 0) != hipSuccess) return IDLM_ERR_HIP;
    sa = f->aux;
  }
  r = launch_paged_attn(*d, p, q, kv_pages, page_table, ctx_lens, attn_out, (char*)workspace, s);
  if (r == IDLM_OK)
    r = launch_accept(*d, p, logits_clean, logits_mask, draft_tokens, seed, T, out_tokens,
                      out_accept_len, nullptr, (char*)workspace, sa, nullptr, mask_stats);
  // The proposals follow the acceptance on its stream: they need its accept
  // lengths, and a record they write may be the one it read.
  if (r == IDLM_OK && np)
    r = launch_propose(*d, p, np->logits_next, draft_tokens, out_accept_len, seed, T,
                       np->next_drafts, (char*)workspace, sa, np->mask_stats_next);
  // Join the second stream back whatever happened above, so a failed call
  // never leaves it forked (a capture in progress stays joined).
  if (f && (hipEventRecord(f->done, f->aux) != hipSuccess ||
            hipStreamWaitEvent(s, f->done, 0) != hipSuccess) && r == IDLM_OK)
    r = IDLM_ERR_HIP;
  return r;
}

int32_t idlm_isd_step(const idlm_isd_dims* d, const void* q, const void* kv_pages,
                      const int32_t* page_table, const int32_t* ctx_lens,
                      const void* logits_clean, const void* logits_mask,
                      const int32_t* draft_tokens, uint64_t seed, int32_t N, float T,
                      int32_t* out_tokens, int32_t* out_accept_len, void* attn_out,
                      const void* mask_stats, void* workspace, size_t ws_bytes, void* stream) {
  return step_impl(d, q, kv_pages, page_table, ctx_lens, logits_clean, logits_mask, draft_tokens,
                   seed, N, T, out_tokens, out_accept_len, attn_out, mask_stats, nullptr,
                   workspace, ws_bytes, stream);
}

int32_t idlm_isd_loop_step(const idlm_isd_dims* d, const void* q, const void* kv_pages,
                           const int32_t* page_table, const int32_t* ctx_lens,
                           const void* logits_clean, const void* logits_mask,
                           const int32_t* draft_tokens, const void* mask_stats,
                           const void* logits_next, uint64_t seed, int32_t N, float T,
                           int32_t* out_tokens, int32_t* out_accept_len, void* attn_out,
                           int32_t* next_drafts, void* mask_stats_next, void* workspace,
                           size_t ws_bytes, void* stream) {
  const NextProposals np{logits_next, next_drafts, mask_stats_next};
  return step_impl(d, q, kv_pages, page_table, ctx_lens, logits_clean, logits_mask, draft_tokens,
                   seed, N, T, out_tokens, out_accept_len, attn_out, mask_stats, &np,
                   workspace, ws_bytes, stream);
}

int32_t idlm_isd_propose(const idlm_isd_dims* d, const void* logits_next,
                         const int32_t* draft_tokens, const int32_t* accept_len, uint64_t seed,
                         float T, int32_t* next_drafts, void* mask_stats, void* workspace,
                         size_t ws_bytes, void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  if ((r = check_T(T)) != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  if ((r = check_ws(p, workspace, ws_bytes)) != IDLM_OK) return r;
  if (((uintptr_t)mask_stats & 255) != 0) return IDLM_ERR_WORKSPACE;
  if (d->B == 0 || d->N == 1) return IDLM_OK;
  if (!logits_next || !draft_tokens || !accept_len || !next_drafts) return IDLM_ERR_NULL;
  return launch_propose(*d, p, logits_next, draft_tokens, accept_len, seed, T, next_drafts,
                        (char*)workspace, (hipStream_t)stream, mask_stats);
}

static int32_t check_lora(const idlm_isd_lora_dims* L) {
  if (!L) return IDLM_ERR_NULL;
  if (L->B < 0 || L->B > (1 << 20) || L->N < 1 || L->N > 16) return IDLM_ERR_DIMS;
  if (L->H < 1 || L->O < 1 || L->rank < 1) return IDLM_ERR_DIMS;
  if ((int64_t)L->B * (2 * L->N - 1) * L->O > (1ll << 31)) return IDLM_ERR_DIMS;
  if (L->H % 32 != 0 || L->H > (1 << 20) || L->rank % 16 != 0 || L->rank > 256)
    return IDLM_ERR_UNSUPPORTED;
  int64_t items[3];
  gated_lora_work_items(*L, items);
  for (int i = 0; i < 3; ++i)
    if (items[i] > kMaxWorkItems) return IDLM_ERR_UNSUPPORTED;
  return IDLM_OK;
}

size_t idlm_isd_lora_workspace_bytes(const idlm_isd_lora_dims* L) {
  if (check_lora(L) != IDLM_OK) return 0;
  const size_t n = gated_lora_workspace(*L);
  return align256(n > 0 ? n : 256);
}

int32_t idlm_isd_gated_lora(const idlm_isd_lora_dims* L, const float* y_base, const void* x,
                            const void* lora_a, const void* lora_b, float scale, void* y_out,
                            void* workspace, size_t ws_bytes, void* stream) {
  int32_t r = check_lora(L);
  if (r != IDLM_OK) return r;
  if (!isfinite(scale)) return IDLM_ERR_DIMS;
  const size_t need = idlm_isd_lora_workspace_bytes(L);
  if (!workspace) return IDLM_ERR_NULL;
  if (((uintptr_t)workspace & 255) != 0 || ws_bytes < need) return IDLM_ERR_WORKSPACE;
  if (L->B == 0) return IDLM_OK;
  if (!y_base || !x || !lora_a || !lora_b || !y_out) return IDLM_ERR_NULL;
  if (((uintptr_t)x | (uintptr_t)lora_a | (uintptr_t)lora_b) & 15) return IDLM_ERR_UNSUPPORTED;
  return launch_gated_lora(*L, y_base, x, lora_a, lora_b, scale, y_out, (char*)workspace,
                           (hipStream_t)stream);
}

int32_t idlm_isd_kv_append(const idlm_isd_dims* d, const void* k_new, const void* v_new,
                           const int32_t* ctx_before, int32_t* ctx_after, void* kv_pages,
                           int32_t* page_table, int32_t* free_pages, int32_t* free_count,
                           void* workspace, size_t ws_bytes, void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  if ((r = check_ws(p, workspace, ws_bytes)) != IDLM_OK) return r;
  if (d->B == 0) return IDLM_OK;
  if (!k_new || !v_new || !ctx_before || !ctx_after || !kv_pages || !page_table || !free_pages ||
      !free_count)
    return IDLM_ERR_NULL;
  return launch_kv_append(*d, p, k_new, v_new, ctx_before, ctx_after, kv_pages, page_table,
                          free_pages, free_count, (char*)workspace, (hipStream_t)stream);
}

int32_t idlm_isd_kv_rollback(const idlm_isd_dims* d, const int32_t* ctx_lens,
                             const int32_t* accept_len, int32_t* ctx_after, int32_t* page_table,
                             int32_t* free_pages, int32_t* free_count, void* workspace,
                             size_t ws_bytes, void* stream) {
  int32_t r = check_dims(d);
  if (r != IDLM_OK) return r;
  Plan p;
  make_plan(*d, &p);
  if ((r = check_ws(p, workspace, ws_bytes)) != IDLM_OK) return r;
  if (d->B == 0) return IDLM_OK;
  if (!ctx_lens || !accept_len || !ctx_after || !page_table || !free_pages || !free_count)
    return IDLM_ERR_NULL;
  return launch_kv_rollback(*d, p, ctx_lens, accept_len, ctx_after, page_table, free_pages,
                            free_count, (char*)workspace, (hipStream_t)stream);
}

int32_t idlm_isd_read_status(const void* workspace, void* stream, int32_t* host_code) {
  if (!workspace || !host_code) return IDLM_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return IDLM_ERR_HIP;
  int32_t word = 0;
  if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return IDLM_ERR_HIP;
  *host_code = word ? IDLM_ERR_DEVICE_DATA : IDLM_OK;
  return IDLM_OK;
}

const char* idlm_isd_strerror(int32_t status) {
  switch (status) {
    case IDLM_OK: return "ok";
    case IDLM_ERR_NULL: return "a required pointer is NULL";
    case IDLM_ERR_DIMS: return "sizes out of range or inconsistent";
    case IDLM_ERR_UNSUPPORTED: return "sizes valid but not supported (D, page size or tile rows)";
    case IDLM_ERR_TEMPERATURE: return "temperature must be 0 or finite and >= 2^-126";
    case IDLM_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case IDLM_ERR_HIP: return "HIP runtime error";
    case IDLM_ERR_DEVICE_DATA:
      return "kernels saw invalid device data (page id, context, draft or free list)";
    case IDLM_ERR_SCRATCH:
      return "sizes need more than the allocation-free acceptance's static scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
