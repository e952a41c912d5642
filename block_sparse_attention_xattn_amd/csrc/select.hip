// Stage 3: minimal-set threshold selection, one workgroup per query-block row.
//
// Definition (XAttention AI summary, "Approach": keep the minimal set of
// blocks whose softmax-normalised mass exceeds the per-head threshold;
// FlexPrefill rebuttal, "R Q3": the minimal |S| under a cumulative-mass
// constraint is the descending-order prefix that first meets it):
//   candidates J <= I (causal) or all J; order by score descending, ties by J
//   ascending; prefix masses c_k in float64, T = c_n; keep the first
//   k* = min{k >= 0 : c_k >= tau * T} (tau >= 1 keeps all); then add J = I.
//
// Implementation: each candidate becomes a 64-bit key (score bits << 32 |
// ~J); block scores are non-negative, so their IEEE bits order like the
// values and one descending integer sort yields (score desc, J asc). Bitonic
// sort in LDS, float64 prefix sums (per-thread runs + wave shuffles + a
// 4-wave combine), a count of prefixes below tau*T, then flags and an
// ascending compaction to kv_idx.
#include "common.h"
#include "kernels.h"
#include "score_row.h"

namespace xattn {

struct SelectArgs {
  const float* scores;
  uint8_t* mask;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int Hq, NB, causal;
  TauArray tau;
};

constexpr int SEL_MAX = 4096;

__device__ __forceinline__ double wave_incl_scan(double x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

struct SelectLds {
  uint64_t keys[SEL_MAX];
  uint8_t flags[SEL_MAX];
  double wsum[4];
  int wcnt[4];
};

// Candidate p (score bits, index) as a descending-sortable key. Block scores
// are non-negative, so their IEEE bits order like the values.
__device__ __forceinline__ uint64_t sel_key(float score, int p) {
  return ((uint64_t)__float_as_uint(score) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)p);
}

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

  if (mask) {
    uint8_t* mrow = mask + row * NB;
    for (int p = tid; p < NB; p += 256) mrow[p] = flags[p];
  }
  // ascending compaction: per-thread contiguous runs of J
  const int per = (NB + 255) / 256;
  const int p0 = tid * per, p1 = min(p0 + per, NB);
  int mine = 0;
  for (int p = p0; p < p1; ++p) mine += flags[p];
  const int incl = wave_incl_scan_i(mine, lane);
  __syncthreads();  // wcnt reuse
  if (lane == 63) sh.wcnt[wave] = incl;
  __syncthreads();
  int pos = incl - mine;
  for (int w = 0; w < wave; ++w) pos += sh.wcnt[w];
  int32_t* irow = kv_idx + row * NB;
  for (int p = p0; p < p1; ++p)
    if (flags[p]) irow[pos++] = p;
  if (tid == 0) kv_cnt[row] = sh.wcnt[0] + sh.wcnt[1] + sh.wcnt[2] + sh.wcnt[3];
}

__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  __shared__ SelectLds sh;
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;  // (b*Hq + h)*NB + I
  const int I = (int)(row % a.NB);
  const int h = (int)((row / a.NB) % a.Hq);
  const int NB = a.NB;
  const int n = a.causal ? I + 1 : NB;
  int npad = 1;
  while (npad < n) npad <<= 1;
  const float* srow = a.scores + row * NB;
  for (int p = tid; p < npad; p += 256) sh.keys[p] = p < n ? sel_key(srow[p], p) : 0;
  for (int p = tid; p < NB; p += 256) sh.flags[p] = 0;
  __syncthreads();
  select_from_keys(sh, n, npad, NB, I, a.tau.v[h], row, a.mask, a.kv_idx, a.kv_cnt);
}

// Fused stage 2 + 3: the row's block scores are computed from the partials
// (written out as xattn_score would), kept in LDS as sort keys, and selected
// without a round trip through HBM.
struct FusedArgs {
  const float* ws;
  float* scores;
  uint8_t* mask;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int Hq, NB, causal;
  TauArray tau;
};

template <int RB>
__global__ __launch_bounds__(256) void score_select_kernel(FusedArgs a) {
  __shared__ SelectLds sh;
  __shared__ ScoreRowLds shs;
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;  // (b*Hq + h)*NB + I
  const int I = (int)(row % a.NB);
  const size_t bh = row / a.NB;
  const int h = (int)(bh % a.Hq);
  const int NB = a.NB;
  const int n = a.causal ? I + 1 : NB;
  int npad = 1;
  while (npad < n) npad <<= 1;
  const float* L = a.ws + (bh * (size_t)NB + I) * (size_t)NB * RB;
  float* orow = a.scores + row * NB;
  for (int p = tid; p < NB; p += 256) sh.flags[p] = 0;
  for (int p = n + tid; p < npad; p += 256) sh.keys[p] = 0;
  block_score_row<RB>(L, n, NB, shs, [&](int J, float sc) {
    orow[J] = sc;
    if (J < n) sh.keys[J] = sel_key(sc, J);
  });
  __syncthreads();
  select_from_keys(sh, n, npad, NB, I, a.tau.v[h], row, a.mask, a.kv_idx, a.kv_cnt);
}

hipError_t launch_score_select(const Shape& s, const float* ws, float* block_scores, const TauArray& tau,
                               uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st) {
  FusedArgs a{ws, block_scores, mask, kv_idx, kv_cnt, s.Hq, s.NB(), s.causal, tau};
  const dim3 grid((unsigned)((size_t)s.B * s.Hq * s.NB()));
  switch (s.r()) {
    case 2: hipLaunchKernelGGL(score_select_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(score_select_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(score_select_kernel<8>, grid, dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL(score_select_kernel<16>, grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(score_select_kernel<32>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const float* block_scores, const TauArray& tau,
                         uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st) {
  SelectArgs a{block_scores, mask, kv_idx, kv_cnt, s.Hq, s.NB(), s.causal, tau};
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)((size_t)s.B * s.Hq * s.NB())), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace xattn
