/* Host-side driver for the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against a host-only build of the library (no
 * device code): every entry point's validation paths, which return before
 * anything is enqueued, and a seeded sweep of extreme sizes through the size
 * and workspace arithmetic.  Prints "checks <n> failures <m>"; a sanitizer
 * report aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "idlm_isd.h"

static int checks = 0, failures = 0;

#define EXPECT(expr, want)                                                     \
  do {                                                                         \
    long long got_ = (long long)(expr);                                        \
    ++checks;                                                                  \
    if (got_ != (long long)(want)) {                                           \
      ++failures;                                                              \
      fprintf(stderr, "line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_, \
              (long long)(want));                                              \
    }                                                                          \
  } while (0)

static idlm_isd_dims good(void) {
  idlm_isd_dims d = {64, 4, 32, 8, 128, 151936, 16, 1024, 40000, IDLM_BF16, IDLM_BF16};
  return d;
}

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void) {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(rng_state >> 32);
}
/* Mostly small values, sometimes the int32 extremes. */
static int32_t pick(int32_t small_max) {
  const uint32_t r = next_u32();
  switch (r & 7) {
    case 0: return INT32_MIN;
    case 1: return INT32_MAX;
    case 2: return -(int32_t)(next_u32() & 0xFFFF);
    case 3: return (int32_t)(next_u32() & 0x7FFFFFFF);
    default: return (int32_t)(next_u32() % (uint32_t)(small_max + 1));
  }
}

int main(void) {
  void* fake = (void*)(uintptr_t)(1u << 20); /* never dereferenced */
  void* misaligned = (void*)(uintptr_t)((1u << 20) + 8);
  idlm_isd_dims d = good();
  const size_t n = idlm_isd_workspace_bytes(&d);
  EXPECT(n > 0 && n % 256 == 0, 1);
  EXPECT(idlm_isd_workspace_state_bytes(&d), 256);
  EXPECT(idlm_isd_validate(&d, 1.0f), IDLM_OK);
  EXPECT(idlm_isd_validate(&d, 0.0f), IDLM_OK);
  EXPECT(idlm_isd_validate(&d, -1.0f), IDLM_ERR_TEMPERATURE);
  EXPECT(idlm_isd_validate(&d, NAN), IDLM_ERR_TEMPERATURE);
  EXPECT(idlm_isd_validate(&d, INFINITY), IDLM_ERR_TEMPERATURE);
  EXPECT(idlm_isd_validate(&d, 1e-39f), IDLM_ERR_TEMPERATURE);
  EXPECT(idlm_isd_validate(NULL, 1.0f), IDLM_ERR_NULL);
  EXPECT(idlm_isd_workspace_bytes(NULL), 0);
  EXPECT(idlm_isd_workspace_state_bytes(NULL), 0);
  EXPECT(idlm_isd_mask_stats_bytes(NULL), 0);
  EXPECT(idlm_isd_mask_stats_bytes(&d) > 256, 1);

  /* NULL dims everywhere */
  EXPECT(idlm_isd_paged_attn(NULL, fake, fake, fake, fake, fake, fake, n, NULL), IDLM_ERR_NULL);
  EXPECT(idlm_isd_accept(NULL, fake, fake, fake, 1, 1.0f, fake, fake, NULL, NULL, fake, n, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_accept_probs(NULL, fake, fake, 1.0f, fake, n, fake, fake, fake, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_step(NULL, fake, fake, fake, fake, fake, fake, fake, 1, 4, 1.0f, fake, fake,
                       fake, NULL, fake, n, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_propose(NULL, fake, fake, fake, 1, 1.0f, fake, NULL, fake, n, NULL), IDLM_ERR_NULL);
  EXPECT(idlm_isd_loop_step(NULL, fake, fake, fake, fake, fake, fake, fake, NULL, fake, 1, 4, 1.0f,
                            fake, fake, fake, fake, NULL, fake, n, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_loop_step(&d, fake, fake, fake, fake, fake, fake, fake, NULL, fake, 1, 4, 1.0f,
                            fake, fake, fake, fake, misaligned, fake, n, NULL),
         IDLM_ERR_WORKSPACE);
  EXPECT(idlm_isd_kv_append(NULL, fake, fake, fake, fake, fake, fake, fake, fake, fake, n, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_kv_rollback(NULL, fake, fake, fake, fake, fake, fake, fake, n, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_gated_lora(NULL, fake, fake, fake, fake, 1.0f, fake, fake, 1024, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_read_status(NULL, NULL, NULL), IDLM_ERR_NULL);

  /* workspace: NULL, short, misaligned */
  EXPECT(idlm_isd_paged_attn(&d, fake, fake, fake, fake, fake, NULL, n, NULL), IDLM_ERR_NULL);
  EXPECT(idlm_isd_paged_attn(&d, fake, fake, fake, fake, fake, fake, n - 256, NULL),
         IDLM_ERR_WORKSPACE);
  EXPECT(idlm_isd_accept(&d, fake, fake, fake, 1, 1.0f, fake, fake, NULL, NULL, misaligned, n, NULL),
         IDLM_ERR_WORKSPACE);
  EXPECT(idlm_isd_accept_probs(&d, fake, fake, 1.0f, fake, n - 256, fake, fake, fake, NULL),
         IDLM_ERR_WORKSPACE);
  EXPECT(idlm_isd_propose(&d, fake, fake, fake, 1, 1.0f, fake, NULL, misaligned, n, NULL),
         IDLM_ERR_WORKSPACE);
  EXPECT(idlm_isd_workspace_init(misaligned, 1024, NULL), IDLM_ERR_WORKSPACE);

  /* temperature and required pointers */
  EXPECT(idlm_isd_accept(&d, fake, fake, fake, 1, -1.0f, fake, fake, NULL, NULL, fake, n, NULL),
         IDLM_ERR_TEMPERATURE);
  EXPECT(idlm_isd_accept(&d, NULL, fake, fake, 1, 1.0f, fake, fake, NULL, NULL, fake, n, NULL),
         IDLM_ERR_NULL);
  EXPECT(idlm_isd_accept_probs(&d, fake, fake, NAN, fake, n, fake, fake, fake, NULL),
         IDLM_ERR_TEMPERATURE);
  EXPECT(idlm_isd_propose(&d, fake, fake, fake, 1, INFINITY, fake, NULL, fake, n, NULL),
         IDLM_ERR_TEMPERATURE);
  EXPECT(idlm_isd_step(&d, fake, fake, fake, fake, fake, fake, fake, 1, 3, 1.0f, fake, fake,
                       fake, NULL, fake, n, NULL),
         IDLM_ERR_DIMS); /* N repeated must match */

  /* B = 0 is a no-op that touches nothing */
  idlm_isd_dims z = good();
  z.B = 0;
  const size_t nz = idlm_isd_workspace_bytes(&z);
  EXPECT(idlm_isd_step(&z, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 4, 1.0f, NULL, NULL, NULL,
                       NULL, fake, nz, NULL),
         IDLM_OK);
  EXPECT(idlm_isd_accept(&z, NULL, NULL, NULL, 1, 1.0f, NULL, NULL, NULL, NULL, fake, nz, NULL),
         IDLM_OK);

  /* gated LoRA */
  idlm_isd_lora_dims L = {64, 4, 4096, 4096, 128};
  const size_t nl = idlm_isd_lora_workspace_bytes(&L);
  EXPECT(nl > 0 && nl % 256 == 0, 1);
  EXPECT(idlm_isd_gated_lora(&L, fake, fake, fake, fake, 1.0f, fake, fake, nl - 256, NULL),
         IDLM_ERR_WORKSPACE);
  EXPECT(idlm_isd_gated_lora(&L, fake, fake, fake, fake, NAN, fake, fake, nl, NULL), IDLM_ERR_DIMS);
  idlm_isd_lora_dims Lh = {1 << 20, 2, 65536, 1, 256};
  EXPECT(idlm_isd_lora_workspace_bytes(&Lh), 0);

  /* strerror over every code and beyond */
  for (int32_t c = -3; c < 12; ++c) {
    const char* s = idlm_isd_strerror(c);
    EXPECT(s != NULL && strlen(s) > 0, 1);
  }

  /* seeded sweep of extreme sizes: no sanitizer report, consistent answers */
  for (int it = 0; it < 200000; ++it) {
    idlm_isd_dims r;
    r.B = pick(1 << 12);
    r.N = pick(17);
    r.Hq = pick(130);
    r.Hkv = pick(17);
    r.D = (next_u32() & 1) ? 128 : pick(130);
    r.V = pick(1 << 18);
    r.page_size = (next_u32() & 3) ? 16 : pick(32);
    r.max_pages = pick(1 << 16);
    r.num_pages = pick(1 << 20);
    r.qkv_dtype = (int32_t)(next_u32() % 3);
    r.logits_dtype = (int32_t)(next_u32() % 3);
    const float T = (next_u32() & 1) ? 1.0f : (float)(int32_t)next_u32() * 1e-30f;
    const int32_t v = idlm_isd_validate(&r, T);
    const size_t w = idlm_isd_workspace_bytes(&r);
    const size_t s = idlm_isd_workspace_state_bytes(&r);
    const int32_t vd = idlm_isd_validate(&r, 1.0f);
    EXPECT(v == IDLM_OK || v == IDLM_ERR_DIMS || v == IDLM_ERR_UNSUPPORTED ||
               v == IDLM_ERR_TEMPERATURE,
           1);
    EXPECT((vd == IDLM_OK) == (w > 0), 1);
    EXPECT((vd == IDLM_OK) == (s > 0 && s < w), 1);
    EXPECT((vd == IDLM_OK) == (idlm_isd_mask_stats_bytes(&r) >= 256), 1);
    idlm_isd_lora_dims l = {pick(1 << 12), pick(17), pick(1 << 16), pick(1 << 16), pick(300)};
    (void)idlm_isd_lora_workspace_bytes(&l);
  }
  printf("checks %d failures %d\n", checks, failures);
  return failures != 0;
}
