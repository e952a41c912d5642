// Host-side check of the C ABI's validation layer, built with AddressSanitizer
// on the host code (libxattn's api.hip and this file; device code unchanged).
// Every call here must be refused on the host before anything is enqueued, so
// no GPU is needed; ASan reports any out-of-bounds or use-after-free access in
// the validation, the workspace arithmetic or the error strings. Exit code 0
// when every status is the expected one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/xattn.h"

static int g_fail = 0;
#define EXPECT(cond, ...)                         \
  do {                                            \
    if (!(cond)) {                                \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);          \
      std::fprintf(stderr, "\n");                 \
      ++g_fail;                                   \
    }                                             \
  } while (0)

static xattn_problem base() {
  xattn_problem p;
  std::memset(&p, 0, sizeof(p));
  p.B = 1; p.Hq = 4; p.Hkv = 2; p.M = 1024; p.C = 128; p.block = 128; p.stride = 8;
  p.causal = 1; p.dtype = XATTN_BF16; p.pattern = XATTN_ANTIDIAGONAL; p.selection = XATTN_SELECT_ROW; p.Mk = 0;
  p.flags = 0;
  return p;
}

// a non-NULL address that is never dereferenced (validation fails first)
static void* const FAKE = reinterpret_cast<void*>(0x1000);

static size_t strlen_checked(const char* s) { return s ? std::strlen(s) : 0; }

int main() {
  const float tau4[4] = {0.9f, 0.9f, 0.9f, 0.9f};
  // status strings and the last-error message are valid C strings
  for (int s = -2; s < 10; ++s) EXPECT(strlen_checked(xattn_status_string((xattn_status)s)) > 0, "status %d", s);
  EXPECT(xattn_abi_version() == XATTN_ABI_VERSION, "abi version");

  // problems that must be refused, with their status
  struct Case { const char* what; void (*edit)(xattn_problem&); xattn_status want; };
  const Case cases[] = {
      {"Hkv not dividing Hq", [](xattn_problem& p) { p.Hkv = 3; }, XATTN_ERR_SHAPE},
      {"negative M", [](xattn_problem& p) { p.M = -5; }, XATTN_ERR_SHAPE},
      {"zero B", [](xattn_problem& p) { p.B = 0; }, XATTN_ERR_SHAPE},
      {"Mk < M", [](xattn_problem& p) { p.Mk = 1000; }, XATTN_ERR_SHAPE},
      {"chunk offset off the block grid", [](xattn_problem& p) { p.Mk = 1100; }, XATTN_ERR_SHAPE},
      {"stride not dividing block", [](xattn_problem& p) { p.stride = 3; }, XATTN_ERR_SHAPE},
      {"head dim", [](xattn_problem& p) { p.C = 96; }, XATTN_ERR_UNSUPPORTED},
      {"block", [](xattn_problem& p) { p.block = 32; p.stride = 4; }, XATTN_ERR_UNSUPPORTED},
      {"r = 1", [](xattn_problem& p) { p.stride = 128; }, XATTN_ERR_UNSUPPORTED},
      {"dtype", [](xattn_problem& p) { p.dtype = 7; }, XATTN_ERR_DTYPE},
      {"causal flag", [](xattn_problem& p) { p.causal = 2; }, XATTN_ERR_ARG},
      {"pattern", [](xattn_problem& p) { p.pattern = 3; }, XATTN_ERR_ARG},
      {"selection", [](xattn_problem& p) { p.selection = -1; }, XATTN_ERR_ARG},
      {"unknown flag bit", [](xattn_problem& p) { p.flags = 2; }, XATTN_ERR_ARG},
      {"negative flags", [](xattn_problem& p) { p.flags = -1; }, XATTN_ERR_ARG},
      {"too many heads", [](xattn_problem& p) { p.Hq = 512; p.Hkv = 1; }, XATTN_ERR_UNSUPPORTED},
      {"too many key blocks", [](xattn_problem& p) { p.M = 4096 * 128 + 128; }, XATTN_ERR_UNSUPPORTED},
      {"int32 extremes", [](xattn_problem& p) { p.B = 2147483647; p.Hq = 256; p.Hkv = 1; p.M = 2147483647 / 2048 * 128; }, XATTN_ERR_UNSUPPORTED},
      {"fp32 envelope", [](xattn_problem& p) { p.dtype = XATTN_F32; p.M = 16384 + 128; }, XATTN_ERR_UNSUPPORTED},
      {"DuSA1 in fp32", [](xattn_problem& p) { p.pattern = XATTN_DUSA1; p.dtype = XATTN_F32; }, XATTN_ERR_UNSUPPORTED},
      {"DuSA1 ragged", [](xattn_problem& p) { p.pattern = XATTN_DUSA1; p.M = 1004; }, XATTN_ERR_SHAPE},
  };
  for (const Case& c : cases) {
    xattn_problem p = base();
    c.edit(p);
    const xattn_status s = xattn_score(&p, FAKE, FAKE, 0.01f, (float*)FAKE, FAKE, (size_t)1 << 40, nullptr);
    EXPECT(s == c.want, "%s: status %d, want %d (%s)", c.what, (int)s, (int)c.want, xattn_last_error());
    EXPECT(strlen_checked(xattn_last_error()) > 0, "%s: empty message", c.what);
    EXPECT(xattn_workspace_bytes(&p) == 0, "%s: workspace of an invalid problem", c.what);
    EXPECT(xattn_score_workspace_bytes(&p) == 0, "%s", c.what);
    EXPECT(xattn_prefill_workspace_bytes(&p) == 0, "%s", c.what);
  }
  EXPECT(xattn_score(nullptr, FAKE, FAKE, 0.01f, (float*)FAKE, FAKE, 1 << 20, nullptr) == XATTN_ERR_NULL, "NULL problem");
  EXPECT(xattn_workspace_bytes(nullptr) == 0, "NULL problem workspace");

  xattn_problem p = base();
  // scales, pointers, workspaces
  EXPECT(xattn_score(&p, FAKE, FAKE, -1.f, (float*)FAKE, FAKE, (size_t)1 << 40, nullptr) == XATTN_ERR_ARG, "scale");
  EXPECT(xattn_score(&p, FAKE, FAKE, std::numeric_limits<float>::quiet_NaN(), (float*)FAKE, FAKE, (size_t)1 << 40,
                     nullptr) == XATTN_ERR_ARG, "NaN scale");
  EXPECT(xattn_score(&p, nullptr, FAKE, 0.01f, (float*)FAKE, FAKE, (size_t)1 << 40, nullptr) == XATTN_ERR_NULL, "q");
  EXPECT(xattn_score(&p, FAKE, FAKE, 0.01f, (float*)FAKE, FAKE, 16, nullptr) == XATTN_ERR_WORKSPACE, "small ws");
  const float bad_tau[3][4] = {{0.9f, 0.9f, 1.5f, 0.9f}, {0.9f, -0.1f, 0.9f, 0.9f},
                               {0.9f, 0.9f, 0.9f, std::numeric_limits<float>::quiet_NaN()}};
  for (const auto& t : bad_tau)
    EXPECT(xattn_select(&p, (const float*)FAKE, t, nullptr, (int32_t*)FAKE, (int32_t*)FAKE, nullptr, 0, nullptr) ==
               XATTN_ERR_ARG, "tau");
  EXPECT(xattn_select(&p, (const float*)FAKE, nullptr, nullptr, (int32_t*)FAKE, (int32_t*)FAKE, nullptr, 0, nullptr) ==
             XATTN_ERR_NULL, "NULL tau");
  EXPECT(bsa_fwd(&p, FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 0.1f, FAKE, nullptr, FAKE, 1023,
                 nullptr) == XATTN_ERR_WORKSPACE, "attention queues");
  EXPECT(dense_fwd(&p, FAKE, FAKE, nullptr, 0.1f, FAKE, nullptr, nullptr) == XATTN_ERR_NULL, "dense v");
  EXPECT(xattn_prefill(&p, FAKE, FAKE, FAKE, tau4, 0.01f, 0.1f, nullptr, nullptr, (int32_t*)FAKE, (int32_t*)FAKE,
                       FAKE, xattn_score_workspace_bytes(&p), FAKE, nullptr, nullptr) == XATTN_ERR_WORKSPACE,
         "prefill workspace");
  xattn_problem g = base();
  g.selection = XATTN_SELECT_GLOBAL;
  EXPECT(xattn_prefill(&g, FAKE, FAKE, FAKE, tau4, 0.01f, 0.1f, nullptr, nullptr, (int32_t*)FAKE, (int32_t*)FAKE,
                       FAKE, xattn_workspace_bytes(&g), FAKE, nullptr, nullptr) == XATTN_ERR_NULL,
         "global selection needs block scores");
  // the no-allocation entry point refuses problems past its scratch before touching the device
  xattn_problem big = base();
  big.Hq = 32; big.Hkv = 8; big.M = 32768;
  float tau32[32];
  for (float& t : tau32) t = 0.9f;
  EXPECT(xattn_workspace_bytes(&big) > XATTN_NOALLOC_SCRATCH_BYTES, "big problem");
  EXPECT(xattn_prefill_noalloc(&big, FAKE, FAKE, FAKE, tau32, 0.01f, 0.1f, nullptr, nullptr, (int32_t*)FAKE,
                               (int32_t*)FAKE, FAKE, nullptr, nullptr) == XATTN_ERR_WORKSPACE, "noalloc limit");

  // workspace sizes over a grid of valid problems: one size serves every call
  const int Ms[] = {1, 127, 128, 1000, 4096, 262144};
  const int strides[] = {2, 4, 8, 16, 32};
  for (int M : Ms)
    for (int S : strides)
      for (int sel = 0; sel < 3; ++sel)
        for (int pat = 0; pat < 3; ++pat) {
          xattn_problem q = base();
          q.M = M; q.stride = S; q.selection = sel; q.pattern = pat;
          q.block = S == 2 ? 64 : 128;  // r = block / S at most 32
          if (pat == XATTN_DUSA1 && M % S) continue;
          const size_t all = xattn_workspace_bytes(&q);
          EXPECT(all > 0, "M=%d S=%d sel=%d pat=%d", M, S, sel, pat);
          EXPECT(all >= xattn_score_workspace_bytes(&q) && all >= xattn_select_workspace_bytes(&q) &&
                     all >= xattn_attn_workspace_bytes(&q),
                 "M=%d S=%d", M, S);
        }
  if (g_fail) std::fprintf(stderr, "%d check(s) failed\n", g_fail);
  else std::printf("abi_check: all validation paths refused as expected\n");
  return g_fail ? 1 : 0;
}
