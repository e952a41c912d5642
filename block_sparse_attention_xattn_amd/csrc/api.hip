// C ABI of libxattn.so: argument validation on the host, then kernel launches
// on the caller's stream. Nothing is allocated and no state is kept, apart
// from a per-thread message for the last failure.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/xattn.h"
#include "kernels.h"

namespace {

thread_local char g_err[256] = "";

xattn_status fail(xattn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
xattn_status fail(xattn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// need_stride: the scoring stages use the stride; attention ignores it.
xattn_status check_problem(const xattn_problem* p, bool need_stride = true) {
  if (!p) return fail(XATTN_ERR_NULL, "problem pointer is NULL");
  if (p->dtype != XATTN_BF16 && p->dtype != XATTN_F32)
    return fail(XATTN_ERR_DTYPE, "dtype %d is neither XATTN_BF16 nor XATTN_F32", p->dtype);
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->M < 1 || p->C < 1 || p->block < 1 ||
      (need_stride && p->stride < 1))
    return fail(XATTN_ERR_SHAPE, "B, Hq, Hkv, M, C, block and stride must be positive");
  if (p->causal != 0 && p->causal != 1) return fail(XATTN_ERR_ARG, "causal must be 0 or 1");
  if (p->pattern != XATTN_ANTIDIAGONAL && p->pattern != XATTN_DIAGONAL && p->pattern != XATTN_DUSA1)
    return fail(XATTN_ERR_ARG, "pattern %d is not an xattn_pattern", p->pattern);
  if (p->selection != XATTN_SELECT_ROW && p->selection != XATTN_SELECT_GLOBAL &&
      p->selection != XATTN_SELECT_GQA_UNION)
    return fail(XATTN_ERR_ARG, "selection %d is not an xattn_selection", p->selection);
  if (p->flags & ~(int32_t)XATTN_SELECT_IN_SCORE)
    return fail(XATTN_ERR_ARG, "flags 0x%x hold bits that are not xattn_flags", (unsigned)p->flags);
  const int mk = p->Mk ? p->Mk : p->M;
  if (mk < p->M) return fail(XATTN_ERR_SHAPE, "Mk=%d is shorter than M=%d", p->Mk, p->M);
  if (p->Hq % p->Hkv) return fail(XATTN_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->Hq > XATTN_MAX_HEADS) return fail(XATTN_ERR_UNSUPPORTED, "Hq=%d exceeds %d", p->Hq, XATTN_MAX_HEADS);
  if ((mk - p->M) % p->block)
    return fail(XATTN_ERR_SHAPE, "Mk - M = %d is not a multiple of block=%d", mk - p->M, p->block);
  if (need_stride && p->block % p->stride)
    return fail(XATTN_ERR_SHAPE, "block=%d is not a multiple of stride=%d", p->block, p->stride);
  if (p->C != 64 && p->C != 128) return fail(XATTN_ERR_UNSUPPORTED, "head dim C=%d (supported: 64, 128)", p->C);
  if (p->block != 64 && p->block != 128) return fail(XATTN_ERR_UNSUPPORTED, "block=%d (supported: 64, 128)", p->block);
  const int r = need_stride ? p->block / p->stride : 2;
  if (!pow2(r) || r < 2 || r > 32)
    return fail(XATTN_ERR_UNSUPPORTED, "block/stride=%d (supported: 2, 4, 8, 16, 32)", r);
  const int nbk = (mk + p->block - 1) / p->block;
  if (nbk > XATTN_MAX_BLOCKS)
    return fail(XATTN_ERR_UNSUPPORTED, "%d key blocks exceed %d", nbk, XATTN_MAX_BLOCKS);
  if (need_stride && p->pattern == XATTN_DUSA1) {
    if (p->dtype != XATTN_BF16) return fail(XATTN_ERR_UNSUPPORTED, "DuSA1 scoring runs on bf16 inputs only");
    if (p->M % p->stride || mk % p->stride)
      return fail(XATTN_ERR_SHAPE, "DuSA1 scoring needs M=%d and Mk=%d to be multiples of the stride %d", p->M, mk,
                  p->stride);
  }
  if (p->dtype == XATTN_F32 && mk > XATTN_F32_MAX_TOKENS)
    return fail(XATTN_ERR_UNSUPPORTED, "float32 problems take at most %d key tokens (Mk=%d); use bf16",
                XATTN_F32_MAX_TOKENS, mk);
  const size_t per_head = (size_t)mk * p->C;
  if ((size_t)p->B * p->Hq * per_head > ((size_t)1 << 40))
    return fail(XATTN_ERR_UNSUPPORTED, "problem too large");
  return XATTN_OK;
}

xattn::Shape shape_of(const xattn_problem* p) {
  return xattn::Shape{p->B,      p->Hq,     p->Hkv,    p->M,       p->C,
                      p->block,  p->stride, p->causal, p->pattern, p->selection,
                      p->Mk ? p->Mk : p->M};
}

xattn_status check_scale(float x, const char* name) {
  if (!(x > 0.f) || !std::isfinite(x)) return fail(XATTN_ERR_ARG, "%s=%g must be positive and finite", name, (double)x);
  return XATTN_OK;
}

xattn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return XATTN_OK;
  return fail(XATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

xattn_status check_tau(const xattn_problem* p, const float* tau, xattn::TauArray* out) {
  if (!tau) return fail(XATTN_ERR_NULL, "tau is NULL");
  std::memset(out, 0, sizeof(*out));
  for (int h = 0; h < p->Hq; ++h) {
    const float t = tau[h];
    if (!(t >= 0.f && t <= 1.f)) return fail(XATTN_ERR_ARG, "tau[%d]=%g is outside [0, 1]", h, (double)t);
    out->v[h] = t;
  }
  return XATTN_OK;
}

xattn_status do_partials(const xattn_problem* p, const void* q, const void* k, float score_scale,
                         void* ws, hipStream_t st) {
  const xattn::Shape s = shape_of(p);
  hipError_t e;
  if (p->dtype == XATTN_BF16)
    e = xattn::launch_score_partials_bf16(s, static_cast<const uint16_t*>(q),
                                          static_cast<const uint16_t*>(k), score_scale,
                                          static_cast<float*>(ws), st);
  else
    e = xattn::launch_score_partials_f32(s, static_cast<const float*>(q), static_cast<const float*>(k),
                                         score_scale, static_cast<float*>(ws), st);
  return hip_status(e, "score partials launch");
}

// DuSA1: log-sum-exps into the workspace, block scores written directly
xattn_status do_score_dusa1(const xattn_problem* p, const void* q, const void* k, float score_scale,
                            float* block_scores, void* ws, hipStream_t st) {
  return hip_status(xattn::launch_score_dusa1(shape_of(p), static_cast<const uint16_t*>(q),
                                              static_cast<const uint16_t*>(k), score_scale, static_cast<float*>(ws),
                                              block_scores, st),
                    "DuSA1 score launch");
}

// Partials, then the normalised block scores (the separate scoring stage).
xattn_status do_score(const xattn_problem* p, const void* q, const void* k, float score_scale,
                      float* block_scores, void* ws, hipStream_t st) {
  if (p->pattern == XATTN_DUSA1) return do_score_dusa1(p, q, k, score_scale, block_scores, ws, st);
  const xattn_status r = do_partials(p, q, k, score_scale, ws, st);
  if (r != XATTN_OK) return r;
  return hip_status(xattn::launch_score_finalize(shape_of(p), static_cast<const float*>(ws), block_scores, st),
                    "score finalize launch");
}

xattn_status do_attn(const xattn_problem* p, const void* q, const void* k, const void* v,
                     const int32_t* kv_idx, const int32_t* kv_cnt, float sm_scale, void* out,
                     float* lse, void* queue, hipStream_t st, bool queue_zeroed = false) {
  const xattn::Shape s = shape_of(p);
  hipError_t e;
  if (p->dtype == XATTN_BF16)
    e = xattn::launch_attn_bf16(s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                static_cast<const uint16_t*>(v), kv_idx, kv_cnt, sm_scale,
                                static_cast<uint16_t*>(out), lse, static_cast<uint32_t*>(queue), st,
                                queue_zeroed);
  else
    e = xattn::launch_attn_f32(s, static_cast<const float*>(q), static_cast<const float*>(k),
                               static_cast<const float*>(v), kv_idx, kv_cnt, sm_scale,
                               static_cast<float*>(out), lse, st);
  return hip_status(e, "attention launch");
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

xattn_status check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need)
    return fail(XATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  return XATTN_OK;
}

xattn_status do_select(const xattn_problem* p, const float* block_scores, const xattn::TauArray& t,
                       uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, void* ws, hipStream_t st) {
  const xattn::Shape s = shape_of(p);
  if (p->selection == XATTN_SELECT_GLOBAL)
    return hip_status(xattn::launch_select_global(s, block_scores, t, mask, kv_idx, kv_cnt, ws, st),
                      "global select launch");
  xattn_status r = hip_status(xattn::launch_select(s, block_scores, t, mask, kv_idx, kv_cnt, st), "select launch");
  if (r == XATTN_OK && p->selection == XATTN_SELECT_GQA_UNION)
    r = hip_status(xattn::launch_gqa_union(s, mask, kv_idx, kv_cnt, st), "GQA union launch");
  return r;
}

// xattn_prefill normalises and selects inside the scoring launch when asked
// to and the scoring runs on the DMA kernel
bool select_in_score(const xattn_problem* p) {
  return (p->flags & XATTN_SELECT_IN_SCORE) && p->dtype == XATTN_BF16 && xattn::tile_select_ok(shape_of(p));
}

// xattn_prefill's workspace: score partials | select scratch | arrival
// counters (when selection runs in the scoring launch) | attention queues,
// each part starting on a 256-byte boundary; the last two are zeroed by one
// launch.
struct PrefillLayout {
  size_t select_off, arrive_off, queue_off, total;
};
PrefillLayout prefill_layout(const xattn_problem* p) {
  const xattn::Shape s = shape_of(p);
  const size_t score = xattn_score_workspace_bytes(p);
  const size_t sel = xattn::select_workspace_bytes(s, p->selection);
  PrefillLayout l;
  l.select_off = align256(score);
  l.arrive_off = align256(l.select_off + sel);
  const bool one_launch = select_in_score(p);
  l.queue_off = align256(l.arrive_off + (one_launch ? xattn::arrive_words(s) * sizeof(uint32_t) : 0));
  l.total = l.queue_off + xattn_attn_workspace_bytes(p);
  return l;
}

// Scratch of xattn_prefill_noalloc: one file-scope device array (each GPU the
// library runs on holds its own copy until the process ends). Host code never
// uses the array's name as an address: it is a host-side stand-in. The device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
static __device__ __align__(256) unsigned char scratch[XATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

xattn_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(XATTN_ERR_UNSUPPORTED, "device %d is beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(XATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return XATTN_OK;
}

}  // namespace

extern "C" {

int32_t xattn_abi_version(void) { return XATTN_ABI_VERSION; }

const char* xattn_status_string(xattn_status s) {
  switch (s) {
    case XATTN_OK: return "ok";
    case XATTN_ERR_NULL: return "null pointer";
    case XATTN_ERR_SHAPE: return "inconsistent shape";
    case XATTN_ERR_DTYPE: return "unknown dtype";
    case XATTN_ERR_ARG: return "argument out of range";
    case XATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case XATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case XATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* xattn_last_error(void) { return g_err; }

size_t xattn_score_workspace_bytes(const xattn_problem* p) {
  if (check_problem(p) != XATTN_OK) return 0;
  const xattn::Shape s = shape_of(p);
  if (p->pattern == XATTN_DUSA1)  // per (phase, strided row) log-sum-exps, then room for block scores
    return align256(xattn::dusa1_lse_bytes(s)) + (size_t)p->B * p->Hq * (size_t)s.NBq() * s.NBk() * sizeof(float);
  return (size_t)p->B * p->Hq * (size_t)s.NBq() * s.NBk() * s.r() * sizeof(float);
}

size_t xattn_attn_workspace_bytes(const xattn_problem* p) {
  if (check_problem(p, false) != XATTN_OK) return 0;
  return xattn::kQueueWords * sizeof(uint32_t);
}

size_t xattn_prefill_workspace_bytes(const xattn_problem* p) {
  if (check_problem(p) != XATTN_OK) return 0;
  return prefill_layout(p).total;
}

size_t xattn_workspace_bytes(const xattn_problem* p) {
  // xattn_prefill's layout holds every other entry point's scratch
  return xattn_prefill_workspace_bytes(p);
}

xattn_status xattn_score(const xattn_problem* p, const void* q, const void* k, float score_scale,
                         float* block_scores, void* ws, size_t ws_bytes, void* stream) {
  xattn_status s = check_problem(p);
  if (s != XATTN_OK) return s;
  if (!q || !k || !block_scores) return fail(XATTN_ERR_NULL, "q, k and block_scores must be non-NULL");
  if ((s = check_scale(score_scale, "score_scale")) != XATTN_OK) return s;
  if ((s = check_workspace(ws, ws_bytes, xattn_score_workspace_bytes(p))) != XATTN_OK) return s;
  return do_score(p, q, k, score_scale, block_scores, ws, static_cast<hipStream_t>(stream));
}

size_t xattn_select_workspace_bytes(const xattn_problem* p) {
  if (check_problem(p) != XATTN_OK) return 0;
  return xattn::select_workspace_bytes(shape_of(p), p->selection);
}

xattn_status xattn_select(const xattn_problem* p, const float* block_scores, const float* tau,
                          uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, void* ws, size_t ws_bytes,
                          void* stream) {
  xattn_status s = check_problem(p);
  if (s != XATTN_OK) return s;
  if (!block_scores || !kv_idx || !kv_cnt)
    return fail(XATTN_ERR_NULL, "block_scores, kv_idx and kv_cnt must be non-NULL");
  xattn::TauArray t;
  if ((s = check_tau(p, tau, &t)) != XATTN_OK) return s;
  const size_t need = xattn_select_workspace_bytes(p);
  if (need && (s = check_workspace(ws, ws_bytes, need)) != XATTN_OK) return s;
  return do_select(p, block_scores, t, mask, kv_idx, kv_cnt, ws, static_cast<hipStream_t>(stream));
}

xattn_status bsa_fwd(const xattn_problem* p, const void* q, const void* k, const void* v,
                     const int32_t* kv_idx, const int32_t* kv_cnt, float sm_scale, void* out,
                     float* lse, void* ws, size_t ws_bytes, void* stream) {
  xattn_status s = check_problem(p, false);
  if (s != XATTN_OK) return s;
  if (!q || !k || !v || !kv_idx || !kv_cnt || !out)
    return fail(XATTN_ERR_NULL, "q, k, v, kv_idx, kv_cnt and out must be non-NULL");
  if ((s = check_scale(sm_scale, "sm_scale")) != XATTN_OK) return s;
  if ((s = check_workspace(ws, ws_bytes, xattn_attn_workspace_bytes(p))) != XATTN_OK) return s;
  return do_attn(p, q, k, v, kv_idx, kv_cnt, sm_scale, out, lse, ws, static_cast<hipStream_t>(stream));
}

xattn_status dense_fwd(const xattn_problem* p, const void* q, const void* k, const void* v,
                       float sm_scale, void* out, float* lse, void* stream) {
  xattn_status s = check_problem(p, false);
  if (s != XATTN_OK) return s;
  if (!q || !k || !v || !out) return fail(XATTN_ERR_NULL, "q, k, v and out must be non-NULL");
  if ((s = check_scale(sm_scale, "sm_scale")) != XATTN_OK) return s;
  return do_attn(p, q, k, v, nullptr, nullptr, sm_scale, out, lse, nullptr,
                 static_cast<hipStream_t>(stream));
}

xattn_status xattn_prefill(const xattn_problem* p, const void* q, const void* k, const void* v,
                           const float* tau, float score_scale, float sm_scale, float* block_scores,
                           uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, void* ws,
                           size_t ws_bytes, void* out, float* lse, void* stream) {
  xattn_status s = check_problem(p);
  if (s != XATTN_OK) return s;
  if (!q || !k || !v || !kv_idx || !kv_cnt || !out)
    return fail(XATTN_ERR_NULL, "q, k, v, kv_idx, kv_cnt and out must be non-NULL");
  if (!block_scores && p->selection == XATTN_SELECT_GLOBAL)
    return fail(XATTN_ERR_NULL, "global selection ranks the whole block-score matrix: block_scores must be non-NULL");
  if ((s = check_scale(score_scale, "score_scale")) != XATTN_OK) return s;
  if ((s = check_scale(sm_scale, "sm_scale")) != XATTN_OK) return s;
  xattn::TauArray t;
  if ((s = check_tau(p, tau, &t)) != XATTN_OK) return s;
  if ((s = check_workspace(ws, ws_bytes, xattn_prefill_workspace_bytes(p))) != XATTN_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const PrefillLayout lay = prefill_layout(p);
  char* wsb = static_cast<char*>(ws);
  const xattn::Shape sh = shape_of(p);
  if (p->pattern == XATTN_DUSA1) {
    // block scores first (into the workspace when the caller does not want them),
    // then the selection on them
    float* sc = block_scores ? block_scores
                             : reinterpret_cast<float*>(wsb + align256(xattn::dusa1_lse_bytes(sh)));
    if ((s = do_score_dusa1(p, q, k, score_scale, sc, ws, st)) != XATTN_OK) return s;
    if ((s = do_select(p, sc, t, mask, kv_idx, kv_cnt, wsb + lay.select_off, st)) != XATTN_OK) return s;
    return do_attn(p, q, k, v, kv_idx, kv_cnt, sm_scale, out, lse, wsb + lay.queue_off, st);
  }
  if (select_in_score(p)) {
    // one launch zeroes the arrival counters and the attention queues; the
    // scoring launch then normalises and selects each query tile's rows as
    // soon as the tile's last partials are stored
    uint32_t* arrive = reinterpret_cast<uint32_t*>(wsb + lay.arrive_off);
    const size_t words = (lay.queue_off - lay.arrive_off) / sizeof(uint32_t) + xattn::kQueueWords;
    if ((s = hip_status(xattn::launch_clear_words(arrive, words, st), "workspace clear launch")) != XATTN_OK)
      return s;
    xattn::TileSelect ts{arrive, block_scores, mask, kv_idx, kv_cnt, sh.qoff(), t};
    if ((s = hip_status(xattn::launch_score_tile_select(sh, static_cast<const uint16_t*>(q),
                                                        static_cast<const uint16_t*>(k), score_scale,
                                                        static_cast<float*>(ws), ts, st),
                        "score+select launch")) != XATTN_OK)
      return s;
    if (p->selection == XATTN_SELECT_GQA_UNION &&
        (s = hip_status(xattn::launch_gqa_union(sh, mask, kv_idx, kv_cnt, st), "GQA union launch")) != XATTN_OK)
      return s;
    return do_attn(p, q, k, v, kv_idx, kv_cnt, sm_scale, out, lse, wsb + lay.queue_off, st, true);
  }
  if ((s = do_partials(p, q, k, score_scale, ws, st)) != XATTN_OK) return s;
  if (p->selection == XATTN_SELECT_GLOBAL) {
    // the head's whole block matrix is needed first
    if ((s = hip_status(xattn::launch_score_finalize(sh, static_cast<const float*>(ws), block_scores, st),
                        "score finalize launch")) != XATTN_OK)
      return s;
    if ((s = hip_status(xattn::launch_select_global(sh, block_scores, t, mask, kv_idx, kv_cnt,
                                                    wsb + lay.select_off, st),
                        "global select launch")) != XATTN_OK)
      return s;
  } else {
    // normalisation and per-row selection fused in one launch
    if ((s = hip_status(xattn::launch_score_select(sh, static_cast<const float*>(ws), block_scores, t, mask,
                                                   kv_idx, kv_cnt, st),
                        "score+select launch")) != XATTN_OK)
      return s;
    if (p->selection == XATTN_SELECT_GQA_UNION &&
        (s = hip_status(xattn::launch_gqa_union(sh, mask, kv_idx, kv_cnt, st), "GQA union launch")) != XATTN_OK)
      return s;
  }
  return do_attn(p, q, k, v, kv_idx, kv_cnt, sm_scale, out, lse, wsb + lay.queue_off, st);
}

#if XATTN_DEBUG
// Debug builds only: the kernels' failed bounds checks per category (see
// include/xattn_debug.h), summed over the sources; reset clears them.
xattn_status xattn_debug_violations(uint32_t* out, int32_t n, int32_t reset) {
  if (!out || n < (int32_t)xattn::DBG_CATEGORIES) return fail(XATTN_ERR_ARG, "need %d counters", (int)xattn::DBG_CATEGORIES);
  unsigned int c[xattn::DBG_CATEGORIES] = {};
  hipError_t e;
  if ((e = xattn::debug_counts_score(c, reset)) != hipSuccess || (e = xattn::debug_counts_select(c, reset)) != hipSuccess ||
      (e = xattn::debug_counts_attn(c, reset)) != hipSuccess || (e = xattn::debug_counts_dusa1(c, reset)) != hipSuccess)
    return hip_status(e, "reading the debug counters");
  for (int i = 0; i < (int)xattn::DBG_CATEGORIES; ++i) out[i] = c[i];
  return XATTN_OK;
}
#endif

xattn_status xattn_prefill_noalloc(const xattn_problem* p, const void* q, const void* k, const void* v,
                                   const float* tau, float score_scale, float sm_scale, float* block_scores,
                                   uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, void* out, float* lse,
                                   void* stream) {
  xattn_status s = check_problem(p);
  if (s != XATTN_OK) return s;
  const size_t need = xattn_prefill_workspace_bytes(p);
  if (need > (size_t)XATTN_NOALLOC_SCRATCH_BYTES)
    return fail(XATTN_ERR_WORKSPACE,
                "problem needs %zu bytes of scratch; xattn_prefill_noalloc holds %zu (use xattn_prefill with a "
                "caller workspace)",
                need, (size_t)XATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != XATTN_OK) return s;
  return xattn_prefill(p, q, k, v, tau, score_scale, sm_scale, block_scores, mask, kv_idx, kv_cnt, ws,
                       (size_t)XATTN_NOALLOC_SCRATCH_BYTES, out, lse, stream);
}

}  // extern "C"
