// Stage 3: minimal-set threshold selection, one workgroup per query-block row
// (the row procedure, its definition and the radix select of the cut are in
// select_row.h), the fused normalise+select pass, the global (per-head) and
// GQA-union variants.
#include "common.h"
#include "kernels.h"
#include "score_row.h"
#include "select_row.h"

namespace xattn {

XATTN_DEBUG_COUNTERS

// Rows are (b, h, I) with I < NBq; row I's candidates are key blocks
// J <= I + qoff (causal) or all J < NBk, and its diagonal block is I + qoff.
struct SelectArgs {
  const float* scores;
  uint8_t* mask;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int Hq, NBq, NBk, qoff, causal;
  TauArray tau;
};

// Candidate p (score bits, index) as a descending-sortable key. Block scores
// are non-negative, so their IEEE bits order like the values.
__device__ __forceinline__ uint64_t sel_key(float score, int p) {
  return ((uint64_t)__float_as_uint(score) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)p);
}

#if XATTN_SELECT_SORT
// With keys[0, npad) filled (keys[p] = 0 for p >= n), flags[0, NB) zeroed and
// a barrier passed: sort, cut at tau, add the diagonal, write the row.
__device__ void select_from_keys(SelectLds& sh, int n, int npad, int NB, int I, float tau, size_t row,
                                 uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t* keys = sh.keys;
  uint8_t* flags = sh.flags;
  // bitonic sort, descending
  for (int k = 2; k <= npad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int x = tid; x < (npad >> 1); x += 256) {
        const int i = (x / j) * 2 * j + (x % j);
        const int ixj = i + j;
        const uint64_t u = keys[i], w = keys[ixj];
        const bool big_first = (i & k) == 0;
        if (big_first ? (u < w) : (u > w)) {
          keys[i] = w;
          keys[ixj] = u;
        }
      }
      __syncthreads();
    }
  }

  int kstar;
  if (tau >= 1.f) {
    kstar = n;
  } else {
    // per-thread contiguous runs of the sorted order
    const int per = (npad + 255) / 256;
    const int p0 = tid * per;
    const int p1 = min(p0 + per, n);
    double run = 0.0;
    for (int p = p0; p < p1; ++p) run += (double)__uint_as_float((uint32_t)(keys[p] >> 32));
    const double incl = wave_incl_scan(run, lane);
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    double before = incl - run;
    for (int w = 0; w < wave; ++w) before += sh.wsum[w];
    const double total = sh.wsum[0] + sh.wsum[1] + sh.wsum[2] + sh.wsum[3];
    const double thresh = (double)tau * total;
    int below = 0;
    double c = before;
    for (int p = p0; p < p1; ++p) {
      c += (double)__uint_as_float((uint32_t)(keys[p] >> 32));
      if (c < thresh) ++below;
    }
    const int wb = wave_incl_scan_i(below, lane);
    if (lane == 63) sh.wcnt[wave] = wb;
    __syncthreads();
    const int nbelow = sh.wcnt[0] + sh.wcnt[1] + sh.wcnt[2] + sh.wcnt[3];
    kstar = (thresh <= 0.0) ? 0 : min(nbelow + 1, n);
  }
  for (int p = tid; p < kstar; p += 256) flags[0xFFFFFFFFu - (uint32_t)(keys[p] & 0xFFFFFFFFu)] = 1;
  if (tid == 0) flags[I] = 1;  // diagonal block
  __syncthreads();
  compact_row(threadIdx.x, flags, NB, row, mask, kv_idx, kv_cnt, sh.wcnt);
}

#endif

template <int CAP>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  __shared__ SelectLdsT<CAP> sh;
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;  // (b*Hq + h)*NBq + I
  const int I = (int)(row % a.NBq);
  const int h = (int)((row / a.NBq) % a.Hq);
  const int NB = a.NBk;
  const int Ia = I + a.qoff;
  const int n = a.causal ? Ia + 1 : NB;
  int npad = 1;
  while (npad < n) npad <<= 1;
  const float* srow = a.scores + row * NB;
  XATTN_DCHECK(n <= CAP && NB <= CAP, DBG_SELECT_ROW);
#if XATTN_SELECT_SORT
  for (int p = tid; p < npad; p += 256) sh.keys[p] = p < n ? sel_key(srow[p], p) : 0;
  for (int p = tid; p < NB; p += 256) sh.flags[p] = 0;
  __syncthreads();
  select_from_keys(sh, n, npad, NB, Ia, a.tau.v[h], row, a.mask, a.kv_idx, a.kv_cnt);
#else
  (void)npad;
  for (int p = tid; p < n; p += 256) sh.sc[p] = srow[p];
  for (int p = tid; p < NB; p += 256) sh.flags[p] = 0;
  __syncthreads();
  select_radix(sh, tid, n, NB, Ia, a.tau.v[h], row, a.mask, a.kv_idx, a.kv_cnt);
#endif
}

// Fused stage 2 + 3: the row's block scores are computed from the partials
// (written out as xattn_score would, unless the output pointer is null), kept
// in LDS, and selected without a round trip through HBM.
struct FusedArgs {
  const float* ws;
  float* scores;
  uint8_t* mask;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int Hq, NBq, NBk, qoff, Rq, causal;
  TauArray tau;
};

template <int RB, int CAP>
__global__ __launch_bounds__(256) void score_select_kernel(FusedArgs a) {
  __shared__ SelectLdsT<CAP> sh;
  __shared__ ScoreRowLds shs;
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;  // (b*Hq + h)*NBq + I
  const int I = (int)(row % a.NBq);
  const size_t bh = row / a.NBq;
  const int h = (int)(bh % a.Hq);
  const int NB = a.NBk;
  const int Ia = I + a.qoff;
  const int n = a.causal ? Ia + 1 : NB;
  const int rows = min(RB, a.Rq - I * RB);
  int npad = 1;
  while (npad < n) npad <<= 1;
  const float* L = a.ws + (bh * (size_t)a.NBq + I) * (size_t)NB * RB;
  float* orow = a.scores ? a.scores + row * NB : nullptr;  // block scores are an optional output
  XATTN_DCHECK(n <= CAP && NB <= CAP && rows >= 1 && rows <= RB, DBG_SELECT_ROW);
  for (int p = tid; p < NB; p += 256) sh.flags[p] = 0;
#if XATTN_SELECT_SORT
  for (int p = n + tid; p < npad; p += 256) sh.keys[p] = 0;
  block_score_row<RB>(L, n, NB, rows, shs, tid, [&](int J, float sc) {
    if (orow) orow[J] = sc;
    if (J < n) sh.keys[J] = sel_key(sc, J);
  });
  __syncthreads();
  select_from_keys(sh, n, npad, NB, Ia, a.tau.v[h], row, a.mask, a.kv_idx, a.kv_cnt);
#else
  (void)npad;
  block_score_row<RB>(L, n, NB, rows, shs, tid, [&](int J, float sc) {
    if (orow) orow[J] = sc;
    if (J < n) sh.sc[J] = sc;
  });
  __syncthreads();
  select_radix(sh, tid, n, NB, Ia, a.tau.v[h], row, a.mask, a.kv_idx, a.kv_cnt);
#endif
}

hipError_t launch_score_select(const Shape& s, const float* ws, float* block_scores, const TauArray& tau,
                               uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st) {
  FusedArgs a{ws, block_scores, mask, kv_idx, kv_cnt, s.Hq, s.NBq(), s.NBk(), s.qoff(), s.Rq(), s.causal, tau};
  const dim3 grid((unsigned)((size_t)s.B * s.Hq * s.NBq()));
  const bool small = s.NBk() <= SEL_SMALL;
  switch (s.r()) {
#define XATTN_FUSED_CASE(R)                                                                   \
  case R:                                                                                     \
    if (small)                                                                                \
      hipLaunchKernelGGL((score_select_kernel<R, SEL_SMALL>), grid, dim3(256), 0, st, a);     \
    else                                                                                      \
      hipLaunchKernelGGL((score_select_kernel<R, SEL_MAX>), grid, dim3(256), 0, st, a);       \
    break;
    XATTN_FUSED_CASE(2)
    XATTN_FUSED_CASE(4)
    XATTN_FUSED_CASE(8)
    XATTN_FUSED_CASE(16)
    XATTN_FUSED_CASE(32)
#undef XATTN_FUSED_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const float* block_scores, const TauArray& tau,
                         uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st) {
  SelectArgs a{block_scores, mask, kv_idx, kv_cnt, s.Hq, s.NBq(), s.NBk(), s.qoff(), s.causal, tau};
  const dim3 grid((unsigned)((size_t)s.B * s.Hq * s.NBq()));
  if (s.NBk() <= SEL_SMALL)
    hipLaunchKernelGGL(select_kernel<SEL_SMALL>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(select_kernel<SEL_MAX>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ GQA union
//
// The sibling heads that read one KV head keep one shared list per query-block
// row: the union of their per-row selections (a reuse variant, not from the
// pages: one K/V tile then serves every sibling). One workgroup per (b, g, I)
// reads the siblings' lists, then writes the union back to each of them.

struct UnionArgs {
  uint8_t* mask;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int Hq, Hkv, NBq, NBk;
};

__global__ __launch_bounds__(256) void gqa_union_kernel(UnionArgs a) {
  __shared__ uint8_t flags[SEL_MAX];
  __shared__ int wcnt[4];
  const int tid = threadIdx.x;
  const int NB = a.NBk;
  const size_t gi = blockIdx.x;  // (b*Hkv + g)*NBq + I
  const int I = (int)(gi % a.NBq);
  const size_t bg = gi / a.NBq;
  const int g = (int)(bg % a.Hkv);
  const size_t b = bg / a.Hkv;
  const int G = a.Hq / a.Hkv;
  for (int p = tid; p < NB; p += 256) flags[p] = 0;
  __syncthreads();
  for (int s2 = 0; s2 < G; ++s2) {
    const size_t row = (b * a.Hq + (size_t)(g * G + s2)) * a.NBq + I;
    int c = a.kv_cnt[row];
    c = c < 0 ? 0 : (c > NB ? NB : c);
    const int32_t* idx = a.kv_idx + row * NB;
    for (int t = tid; t < c; t += 256) {
      const int j = idx[t];
      if (j >= 0 && j < NB) flags[j] = 1;
    }
  }
  __syncthreads();  // every sibling list is read before any is rewritten
  for (int s2 = 0; s2 < G; ++s2) {
    const size_t row = (b * a.Hq + (size_t)(g * G + s2)) * a.NBq + I;
    compact_row(threadIdx.x, flags, NB, row, a.mask, a.kv_idx, a.kv_cnt, wcnt);
  }
}

hipError_t launch_gqa_union(const Shape& s, uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt,
                            hipStream_t st) {
  UnionArgs a{mask, kv_idx, kv_cnt, s.Hq, s.Hkv, s.NBq(), s.NBk()};
  hipLaunchKernelGGL(gqa_union_kernel, dim3((unsigned)((size_t)s.B * s.Hkv * s.NBq())), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ global selection
//
// FlexPrefill rebuttal, "R Q3": the blocks of a head may be chosen globally,
// over the flattened block-score matrix, rather than row by row. Per head, the
// candidates (I, J) (J <= I + qoff when causal) are ordered by score
// descending, ties by (I, J) row-major; the kept set is the shortest prefix
// whose mass reaches tau * T (T = the head's candidate mass; tau >= 1 keeps
// all), plus the diagonal blocks (I, I + qoff).
//
// Implementation: a radix select on the score bits (non-negative floats order
// like their bit patterns). Three histogram passes over bits [31:20], [19:8]
// and [7:0] accumulate candidate mass per bucket, each restricted to the
// bucket chosen so far; a per-head step finds the bucket where the mass
// counted from the top first reaches tau * T. Masses are 64-bit fixed-point
// integers (score * 2^50), so the sums are exact and independent of the order
// the atomics land in. The last step yields the threshold score v* and how many
// of the candidates equal to v* to keep (the first ones in (I, J) order). A
// final pass writes every row.

namespace {
constexpr int GSEL_BUCKETS = 4096;
constexpr int GSEL_ROWS_PER_WG = 32;
constexpr double GSEL_FX = 1125899906842624.0;  // 2^50

struct GselHead {
  unsigned long long target;  // ceil(tau * T) in fixed point
  unsigned long long above;   // mass of the candidates above the current bucket
  uint32_t prefix;            // score bits fixed so far
  uint32_t vstar;             // threshold score bits (after the last level)
  uint32_t need_ties;         // candidates equal to v* that are kept
  uint32_t count_v;           // candidates equal to v*
  int32_t mode;               // 0: threshold, 1: keep every candidate, 2: keep none
  int32_t pad[7];
};
static_assert(sizeof(GselHead) == 64, "head state is one 64-byte record");

struct GselHist {
  unsigned long long mass[GSEL_BUCKETS];
  uint32_t cnt[GSEL_BUCKETS];
};

struct GselArgs {
  const float* scores;
  uint8_t* mask;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  GselHead* head;   // [B*Hq]
  GselHist* hist;   // [B*Hq]
  uint32_t* tieoff; // [B*Hq][NBq]: ties at v* in the rows before I
  int Hq, NBq, NBk, qoff, causal;
  TauArray tau;
};

__device__ __forceinline__ unsigned long long gsel_fx(float score) {
  return (unsigned long long)((double)score * GSEL_FX);
}

template <int LEVEL>
struct GselLevel {
  static constexpr int SHIFT = LEVEL == 0 ? 20 : (LEVEL == 1 ? 8 : 0);
  static constexpr int BITS = LEVEL == 2 ? 8 : 12;
  static constexpr int NBK = 1 << BITS;
};
}  // namespace

size_t select_workspace_bytes(const Shape& s, int mode) {
  if (mode != SEL_GLOBAL) return 0;
  const size_t heads = (size_t)s.B * s.Hq;
  return heads * (sizeof(GselHead) + sizeof(GselHist) + sizeof(uint32_t) * (size_t)s.NBq());
}

// Zeroes words[0, n): the head records and histograms of a global selection,
// the arrival counters of selection in the scoring launch.
__global__ __launch_bounds__(256) void gsel_clear_kernel(uint32_t* words, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) words[i] = 0u;
}

hipError_t launch_clear_words(uint32_t* words, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(gsel_clear_kernel, dim3((unsigned)(blocks < 256 ? blocks : 256)), dim3(256), 0, st, words, n);
  return hipGetLastError();
}

template <int LEVEL>
__global__ __launch_bounds__(256) void gsel_hist_kernel(GselArgs a) {
  using Lv = GselLevel<LEVEL>;
  __shared__ unsigned long long mass[Lv::NBK];
  __shared__ uint32_t cnt[Lv::NBK];
  const int tid = threadIdx.x;
  const size_t bh = blockIdx.y;
  const GselHead* st = a.head + bh;
  if (LEVEL > 0 && st->mode != 0) return;  // uniform
  const uint32_t prefix = LEVEL > 0 ? st->prefix : 0u;
  for (int b = tid; b < Lv::NBK; b += 256) {
    mass[b] = 0ull;
    cnt[b] = 0u;
  }
  __syncthreads();
  const int NB = a.NBk;
  const int I0 = blockIdx.x * GSEL_ROWS_PER_WG;
  const int I1 = min(I0 + GSEL_ROWS_PER_WG, a.NBq);
  for (int I = I0; I < I1; ++I) {
    const int n = a.causal ? I + a.qoff + 1 : NB;
    const float* srow = a.scores + (bh * a.NBq + I) * (size_t)NB;
    for (int J = tid; J < n; J += 256) {
      const float sc = srow[J];
      const uint32_t key = __float_as_uint(sc);
      if (LEVEL == 0 || (key >> (Lv::SHIFT + Lv::BITS)) == prefix) {
        const int b = (key >> Lv::SHIFT) & (Lv::NBK - 1);
        atomicAdd(&mass[b], gsel_fx(sc));
        atomicAdd(&cnt[b], 1u);
      }
    }
  }
  __syncthreads();
  GselHist* gh = a.hist + bh;
  for (int b = tid; b < Lv::NBK; b += 256)
    if (cnt[b]) {
      atomicAdd(&gh->mass[b], mass[b]);
      atomicAdd(&gh->cnt[b], cnt[b]);
    }
}

template <int LEVEL>
__global__ __launch_bounds__(256) void gsel_find_kernel(GselArgs a) {
  using Lv = GselLevel<LEVEL>;
  constexpr int PER = Lv::NBK / 256;
  __shared__ unsigned long long tsum[256];
  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x;
  const int h = (int)(bh % a.Hq);
  GselHead* st = a.head + bh;
  GselHist* gh = a.hist + bh;
  // this thread's buckets, highest first: [NBK - PER (tid + 1), NBK - PER tid)
  const int top = Lv::NBK - PER * tid - 1;
  unsigned long long my = 0ull;
  for (int u = 0; u < PER; ++u) my += gh->mass[top - u];
  tsum[tid] = my;
  __syncthreads();
  if (tid == 0) {
    unsigned long long run = 0ull;
    for (int t = 0; t < 256; ++t) {
      const unsigned long long x = tsum[t];
      tsum[t] = run;  // exclusive: mass of the buckets above thread t's
      run += x;
    }
    if (LEVEL == 0) {
      const float tau = a.tau.v[h];
      st->prefix = 0u;
      st->above = 0ull;
      st->vstar = 0u;
      st->need_ties = 0u;
      st->count_v = 0u;
      if (tau >= 1.f) {
        st->mode = 1;
      } else {
        const double t = ceil((double)tau * (double)run);
        const unsigned long long target = (unsigned long long)t;
        st->target = target;
        st->mode = target == 0ull ? 2 : 0;
      }
    }
  }
  __syncthreads();
  const int mode = st->mode;
  const unsigned long long target = st->target, above = st->above;
  const uint32_t prefix0 = st->prefix;
  __syncthreads();  // every thread holds the state before one of them rewrites it
  if (mode == 0) {
    unsigned long long c = above + tsum[tid];
    for (int u = 0; u < PER; ++u) {
      const int b = top - u;
      const unsigned long long m = gh->mass[b];
      if (c < target && c + m >= target) {  // exactly one bucket of the head
        const uint32_t prefix = (prefix0 << Lv::BITS) | (uint32_t)b;
        if (LEVEL == 2) {
          const unsigned long long need = target - c;
          const unsigned long long vfx = gsel_fx(__uint_as_float(prefix));
          st->vstar = prefix;
          st->need_ties = (uint32_t)((need + vfx - 1) / vfx);
          st->count_v = gh->cnt[b];
        }
        st->prefix = prefix;
        st->above = c;
      }
      c += m;
    }
  }
  __syncthreads();
  // leave the histogram cleared for the next level
  for (int u = 0; u < PER; ++u) {
    gh->mass[top - u] = 0ull;
    gh->cnt[top - u] = 0u;
  }
}

// Candidates equal to v* in the rows before each row, when only some of them
// are kept (rare: equal scores straddling the cut).
__global__ __launch_bounds__(256) void gsel_ties_kernel(GselArgs a) {
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t bh = blockIdx.x;
  const GselHead* st = a.head + bh;
  if (st->mode != 0 || st->count_v <= st->need_ties) return;  // uniform
  const uint32_t vstar = st->vstar;
  const int NB = a.NBk;
  uint32_t run = 0u;
  for (int I = 0; I < a.NBq; ++I) {
    const int n = a.causal ? I + a.qoff + 1 : NB;
    const float* srow = a.scores + (bh * a.NBq + I) * (size_t)NB;
    int c = 0;
    for (int J = tid; J < n; J += 256) c += __float_as_uint(srow[J]) == vstar;
    c = wave_incl_scan_i(c, lane);
    if (lane == 63) wsum[wave] = (uint32_t)c;
    __syncthreads();
    if (tid == 0) a.tieoff[bh * a.NBq + I] = run;
    run += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void gsel_compact_kernel(GselArgs a) {
  __shared__ uint8_t flags[SEL_MAX];
  __shared__ int wcnt[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = a.NBk;
  const size_t row = blockIdx.x;  // (b*Hq + h)*NBq + I
  const int I = (int)(row % a.NBq);
  const size_t bh = row / a.NBq;
  const GselHead* st = a.head + bh;
  const int mode = st->mode;
  const uint32_t vstar = st->vstar, need = st->need_ties;
  const bool all_ties = st->count_v <= need;
  const int Ia = I + a.qoff;
  const int n = a.causal ? Ia + 1 : NB;
  const float* srow = a.scores + row * NB;
  // per-thread contiguous runs of J, so tie ranks follow ascending J
  const int per = (NB + 255) / 256;
  const int p0 = tid * per, p1 = min(p0 + per, NB);
  int ties = 0;
  for (int p = p0; p < p1; ++p) {
    uint8_t f = 0;
    if (p < n) {
      if (mode == 1) {
        f = 1;
      } else if (mode == 0) {
        const uint32_t key = __float_as_uint(srow[p]);
        if (key > vstar) f = 1;
        else if (key == vstar) { f = all_ties ? 1 : 2; ties += !all_ties; }
      }
    }
    flags[p] = f;
  }
  if (!all_ties && mode == 0) {
    const int incl = wave_incl_scan_i(ties, lane);
    if (lane == 63) wcnt[wave] = incl;
    __syncthreads();
    uint32_t rank = a.tieoff[row] + (uint32_t)(incl - ties);
    for (int w = 0; w < wave; ++w) rank += (uint32_t)wcnt[w];
    for (int p = p0; p < p1; ++p)
      if (flags[p] == 2) flags[p] = rank++ < need ? 1 : 0;
  }
  __syncthreads();
  if (tid == 0) flags[Ia] = 1;  // diagonal block
  __syncthreads();
  compact_row(threadIdx.x, flags, NB, row, a.mask, a.kv_idx, a.kv_cnt, wcnt);
}

hipError_t launch_select_global(const Shape& s, const float* block_scores, const TauArray& tau,
                                uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, void* ws,
                                hipStream_t st) {
  const size_t heads = (size_t)s.B * s.Hq;
  const int NBq = s.NBq();
  char* base = static_cast<char*>(ws);
  GselArgs a{block_scores, mask, kv_idx, kv_cnt,
             reinterpret_cast<GselHead*>(base),
             reinterpret_cast<GselHist*>(base + heads * sizeof(GselHead)),
             reinterpret_cast<uint32_t*>(base + heads * (sizeof(GselHead) + sizeof(GselHist))),
             s.Hq, NBq, s.NBk(), s.qoff(), s.causal, tau};
  const size_t clear_words = heads * (sizeof(GselHead) + sizeof(GselHist)) / 4;
  hipLaunchKernelGGL(gsel_clear_kernel, dim3(256), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(base), clear_words);
  const dim3 hgrid((unsigned)((NBq + GSEL_ROWS_PER_WG - 1) / GSEL_ROWS_PER_WG), (unsigned)heads);
  hipLaunchKernelGGL(gsel_hist_kernel<0>, hgrid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(gsel_find_kernel<0>, dim3((unsigned)heads), dim3(256), 0, st, a);
  hipLaunchKernelGGL(gsel_hist_kernel<1>, hgrid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(gsel_find_kernel<1>, dim3((unsigned)heads), dim3(256), 0, st, a);
  hipLaunchKernelGGL(gsel_hist_kernel<2>, hgrid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(gsel_find_kernel<2>, dim3((unsigned)heads), dim3(256), 0, st, a);
  hipLaunchKernelGGL(gsel_ties_kernel, dim3((unsigned)heads), dim3(256), 0, st, a);
  hipLaunchKernelGGL(gsel_compact_kernel, dim3((unsigned)(heads * NBq)), dim3(256), 0, st, a);
  return hipGetLastError();
}


hipError_t debug_counts_select(unsigned int* out, bool reset) {
#if XATTN_DEBUG
  unsigned int h[DBG_CATEGORIES];
  hipError_t e = hipMemcpyFromSymbol(h, HIP_SYMBOL(debug_counts), sizeof(h));
  if (e != hipSuccess) return e;
  for (int c = 0; c < DBG_CATEGORIES; ++c) out[c] += h[c];
  if (reset) {
    const unsigned int z[DBG_CATEGORIES] = {};
    e = hipMemcpyToSymbol(HIP_SYMBOL(debug_counts), z, sizeof(z));
  }
  return e;
#else
  (void)out;
  (void)reset;
  return hipSuccess;
#endif
}

}  // namespace xattn
