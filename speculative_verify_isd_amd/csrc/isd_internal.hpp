// Internal declarations shared by the library's translation units: the
// workspace plan and the kernel launchers.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/idlm_isd.h"

#ifndef RING_PAGES_DEFAULT
#define RING_PAGES_DEFAULT 2
#endif
#ifndef MIN_RUN_PAGES_DEFAULT
#define MIN_RUN_PAGES_DEFAULT 8
#endif

namespace idlm {

constexpr int kPage = 16;
constexpr int kSub = 2048;  // acceptance sub-chunk: 256 threads x 8 elements
// 16-byte vectors per thread in an acceptance stats work-group (a slice of
// kSub * kStatsU logits).  Measured per acceptance call: C = 64: 4 vectors
// 26.4 us, 8 vectors 27.7, 2 vectors 34; B = 1: 4 vectors 15.4 us, 2
// vectors 15.3, 1 vector 17.4 (the decision then merges 75 slices per row
// instead of 19); B = 16: 23.9 / 25.8 / 32.0 us for 4 / 2 / 1.
constexpr int kStatsU = 4;
constexpr int kMaxSubChunks = 1024;  // V <= kSub * kMaxSubChunks
constexpr int kMaxWaves = 2048;   // streaming-attention waves resident at once (upper bound)
constexpr int kMinRunPages = MIN_RUN_PAGES_DEFAULT;  // shortest run of pages given to one wave-lane
constexpr int kRingPages = RING_PAGES_DEFAULT;  // page buffers per attention wave (D = 128)

// Sticky device status bits (workspace word 0).
enum : int32_t {
  kBadPage = 1,
  kBadCtx = 2,
  kBadDraft = 4,
  kFreeList = 8,
  kBadLen = 16,
  kBadMaskStats = 32
};

// MASK-row statistics that idlm_isd_propose records for the acceptance of
// the drafts it makes (layout: this header in the first 256 bytes, then
// each MASK row's (max, sum) [B][K] double2 (greedy: max and argmax), the
// drafts' logits [B][K] float, the drafts [B][K] int32, each region
// 256-byte aligned).
struct MaskStatsHeader {
  uint32_t magic;
  uint32_t c2_bits;  // log2(e)/T as float32 bits (0 when greedy)
  int32_t B, K, V, nsub;
};
constexpr uint32_t kMaskStatsMagic = 0x1D15A75Bu;
struct MaskStatsLayout {
  size_t off_st, off_dlog, off_tok, total;
};
MaskStatsLayout mask_stats_layout(const idlm_isd_dims& d);

// Attention sizes derived from the dims.
struct AttnPlan {
  int R, G, RG;   // step rows, heads per KV head, query rows per (b, kv head)
  int RB;         // 16-row MFMA blocks per wave (2 or 4)
  int WR;         // waves sharing a run (1 or 2)
  int RGp;        // RG padded to 16 * RB * WR
  int npairs;     // B * Hkv
  int max_lanes;  // wave-lanes the partial-state slots are sized for
};

// How one acceptance call is cut.
struct AcceptPlan {
  int R;          // rows per sequence: N clean + K mask
  int nsub;       // kSub-element sub-chunks per row
  int S1;         // stats work-groups per row: ceil(V / (kSub * kStatsU))
};

// Per-sequence hand-over from the decision to the sampler.
struct SamplePlan {
  int32_t mode;    // 0 residual max(0, p_j - q_j), 1 bonus row (p only), 2 done (greedy)
  int32_t row_p;   // clean row holding p (residual: j; bonus: k, the listed drafts)
  int32_t j;       // output index of the sampled token
  int32_t kp;      // listed drafts
  double mp, mq;   // row maxima of clean row j and MASK row j (raw logits)
  double rho;      // S_p / S_q from the row statistics (splits p > q from p <= q)
  double sp;       // row sum of clean row j from the row statistics
  double u2;       // sampling uniform
  double pad;
};

struct Plan {
  AttnPlan attn;
  AcceptPlan acc;
  size_t off_status, state_end;  // state kept between calls: [0, state_end)
  size_t off_attn_ml, off_attn_o;
  size_t off_splan, off_stats, off_subsum, off_dlog, off_unif;
  size_t off_rowstat, off_subw;
  size_t off_kv_valid, off_pstats;
  size_t total;
};

bool make_plan(const idlm_isd_dims& d, Plan* p);

int32_t launch_paged_attn(const idlm_isd_dims& d, const Plan& p, const void* q, const void* kv,
                          const int32_t* page_table, const int32_t* ctx_lens, void* out,
                          char* ws, hipStream_t s);

// The acceptance's buffers are ws + p.off_*; `status` (when not null)
// replaces the status word at ws + p.off_status.
int32_t launch_accept(const idlm_isd_dims& d, const Plan& p, const void* lc, const void* lm,
                      const int32_t* drafts, uint64_t seed, float T, int32_t* out_tokens,
                      int32_t* out_len, double* out_debug, char* ws, hipStream_t s,
                      int32_t* status = nullptr, const void* mstats = nullptr);

// Work-groups of the acceptance's launches (stats, decide + sums, select),
// the largest of the three.  Host only; shared by validation and launch.
int64_t accept_max_grid(const idlm_isd_dims& d);
int64_t propose_max_grid(const idlm_isd_dims& d);  // work-groups of the largest proposal launch

int32_t launch_accept_dump(const idlm_isd_dims& d, const Plan& p, const void* lc, const void* lm,
                           float T, const char* ws, double* out_p, double* out_q,
                           double* out_subw, hipStream_t s);

int32_t launch_fill_zero(void* ws, size_t bytes, hipStream_t s);

// Gated LoRA: workspace bytes (split partials and T) and the launcher.
size_t gated_lora_workspace(const idlm_isd_lora_dims& L);
void gated_lora_work_items(const idlm_isd_lora_dims& L, int64_t items[3]);
int32_t launch_gated_lora(const idlm_isd_lora_dims& L, const float* y_base, const void* x,
                          const void* lora_a, const void* lora_b, float scale, void* y_out,
                          char* ws, hipStream_t s);

// mstats (may be null): where to record the MASK-row statistics for the
// next acceptance (else the workspace holds them).
int32_t launch_propose(const idlm_isd_dims& d, const Plan& p, const void* logits_next,
                       const int32_t* drafts, const int32_t* accept_len, uint64_t seed, float T,
                       int32_t* next_drafts, char* ws, hipStream_t s, void* mstats = nullptr);

int32_t launch_kv_append(const idlm_isd_dims& d, const Plan& p, const void* k_new,
                         const void* v_new, const int32_t* ctx_before, int32_t* ctx_after,
                         void* kv_pages, int32_t* page_table, int32_t* free_pages,
                         int32_t* free_count, char* ws, hipStream_t s);

int32_t launch_kv_rollback(const idlm_isd_dims& d, const Plan& p, const int32_t* ctx_lens,
                           const int32_t* accept_len, int32_t* ctx_after, int32_t* page_table,
                           int32_t* free_pages, int32_t* free_count, char* ws, hipStream_t s);

}  // namespace idlm
