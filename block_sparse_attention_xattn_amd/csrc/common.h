// Shared device helpers for the gfx950 kernels: bf16 <-> f32, MFMA fragment
// types, wave-level exchanges, and the launch plans the host layer hands over.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

// Debug builds (-DXATTN_DEBUG=1, libxattn_debug.so): bounds checks at the
// kernels' indexing sites. A failed check adds one to a per-source device
// counter of its category (no trap: the access that follows is the release
// code's, already bounded); the host reads the counters through
// xattn_debug_violations(). Release builds compile the checks away.
#ifndef XATTN_DEBUG
#define XATTN_DEBUG 0
#endif
// (the categories are xattn::DebugCheck, in kernels.h)
#if XATTN_DEBUG
#define XATTN_DEBUG_COUNTERS static __device__ unsigned int debug_counts[DBG_CATEGORIES];
#define XATTN_DCHECK(cond, cat)                                      \
  do {                                                               \
    if (!(cond)) atomicAdd(&debug_counts[(cat)], 1u);                \
  } while (0)
#else
#define XATTN_DEBUG_COUNTERS
#define XATTN_DCHECK(cond, cat) \
  do {                          \
  } while (0)
#endif

namespace xattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the hardware exp unit (v_exp_f32, about 1 ulp). Results below 2^-126
// flush towards zero, which is harmless for softmax weights; the library's exp2f
// would add a 5-instruction denormal-range fix-up around each call.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2 on the hardware unit (v_log_f32) for normal positive inputs.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even float -> bf16 (gfx950 has a native conversion; the
// compiler selects it for this cast).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float v) {
  return __shfl_xor(v, 32, 64);
}

// Reductions across the two wave halves without an LDS round trip: the gfx950
// v_permlane32_swap(a, a) returns r0 = (lo, lo) and r1 = (hi, hi), so
// op(r0, r1) is op(v[l], v[l ^ 32]) in every lane, with identical operand order
// in both halves.
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Read 4 bf16 from LDS with the gfx950 transposing read: within each group of
// 16 lanes, lane t receives element (t % 4) of the 8-byte chunks addressed by
// lanes 4c + t/4, for c = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* lds_ptr) {
  typedef i16x4 __attribute__((address_space(3))) * lp;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(lds_ptr));
}

// Work-item order for XCD locality and balance. Workgroups are dispatched
// round-robin over the 8 XCDs (workgroup w runs on XCD w % 8), each XCD with its
// own L2. With K items per group (e.g. the workgroups that share one KV head),
// every window of 8K consecutive dispatches hands XCD x the K consecutive
// logical items 8Ka + K((x + (a >> rot_shift)) % 8) .. +K-1. A group stays on
// one XCD (one L2) for 2^rot_shift consecutive windows (e.g. neighbouring query
// rows, which select overlapping key blocks), and the rotation then spreads the
// groups over all XCDs, so uneven per-group work does not pile up on one XCD.
// The tail beyond the last full window keeps its own order.
__device__ __forceinline__ uint32_t xcd_map(uint32_t w, uint32_t n, uint32_t K,
                                            uint32_t rot_shift = 0) {
  const uint32_t win = 8u * K;
  const uint32_t full = n - n % win;
  if (w >= full) return w;
  const uint32_t j = w >> 3, x = w & 7u;
  const uint32_t a = j / K;
  return a * win + ((x + (a >> rot_shift)) & 7u) * K + j % K;
}

// Index of the XCD (accelerator complex die) the calling wave runs on: the
// XCC_ID hardware register, bits [3:0].
__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 7u;
}

// LDS byte address of a pointer into a __shared__ array, made wave-uniform.
__device__ __forceinline__ uint32_t lds_addr_u(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// A 64-bit pointer that is the same in every lane, in scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// DMA of 16 bytes per lane from global memory (wave-uniform base plus a
// per-lane byte offset) straight into LDS: the 64 lanes fill the 1 KiB at
// lds_base in lane order. Written as asm so the compiler, which would treat
// every LDS read after such a load as dependent on it, adds no waits of its
// own: the loop that issues these waits for them explicitly (vm_wait) before
// the barrier that publishes the data. It has no register results.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds_base) : "memory", "m0");
}

// Waits until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// s_waitcnt immediate that waits on the vector-memory counter only: at most n
// loads (including LDS DMA) of this wave outstanding.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroups of one kernel instance that fit on the current device at once
// (0 if the runtime cannot tell). The answer is kept per (kernel, block size,
// device) after the first call, so launches do not ask the runtime again.
template <class Kern>
static int resident_workgroups(Kern kern, int threads) {
  struct Entry {
    const void* kern;
    int threads, dev, n;
  };
  static std::mutex mu;
  static Entry known[64];  // a fixed table: no allocation; when full, nothing more is kept
  static int used = 0;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const void* k = reinterpret_cast<const void*>(kern);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (known[i].kern == k && known[i].threads == threads && known[i].dev == dev) return known[i].n;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess) return 0;
  const int n = cus * per_cu;
  if (n > 0) {
    std::lock_guard<std::mutex> lock(mu);
    if (used < 64) known[used++] = Entry{k, threads, dev, n};
  }
  return n;
}

}  // namespace xattn
