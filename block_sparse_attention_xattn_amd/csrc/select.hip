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

__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  __shared__ uint64_t keys[SEL_MAX];
  __shared__ uint8_t flags[SEL_MAX];
  __shared__ double wsum[4];
  __shared__ int wcnt[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = blockIdx.x;  // (b*Hq + h)*NB + I
  const int I = (int)(row % a.NB);
  const int h = (int)((row / a.NB) % a.Hq);
  const int NB = a.NB;
  const int n = a.causal ? I + 1 : NB;
  int npad = 1;
  while (npad < n) npad <<= 1;
  const float* srow = a.scores + row * NB;

  for (int p = tid; p < npad; p += 256) {
    uint64_t key = 0;
    if (p < n) {
      const uint32_t bits = __float_as_uint(srow[p]);
      key = ((uint64_t)bits << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)p);
    }
    keys[p] = key;
  }
  for (int p = tid; p < NB; p += 256) flags[p] = 0;
  __syncthreads();

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

  const float tau = a.tau.v[h];
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
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    double before = incl - run;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const double total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    const double thresh = (double)tau * total;
    int below = 0;
    double c = before;
    for (int p = p0; p < p1; ++p) {
      c += (double)__uint_as_float((uint32_t)(keys[p] >> 32));
      if (c < thresh) ++below;
    }
    const int wb = wave_incl_scan_i(below, lane);
    if (lane == 63) wcnt[wave] = wb;
    __syncthreads();
    const int nbelow = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    kstar = (thresh <= 0.0) ? 0 : min(nbelow + 1, n);
  }
  for (int p = tid; p < kstar; p += 256) flags[0xFFFFFFFFu - (uint32_t)(keys[p] & 0xFFFFFFFFu)] = 1;
  if (tid == 0) flags[I] = 1;  // diagonal block
  __syncthreads();

  if (a.mask) {
    uint8_t* mrow = a.mask + row * NB;
    for (int p = tid; p < NB; p += 256) mrow[p] = flags[p];
  }
  // ascending compaction: per-thread contiguous runs of J
  const int per = (NB + 255) / 256;
  const int p0 = tid * per, p1 = min(p0 + per, NB);
  int mine = 0;
  for (int p = p0; p < p1; ++p) mine += flags[p];
  const int incl = wave_incl_scan_i(mine, lane);
  __syncthreads();  // wcnt reuse
  if (lane == 63) wcnt[wave] = incl;
  __syncthreads();
  int pos = incl - mine;
  for (int w = 0; w < wave; ++w) pos += wcnt[w];
  int32_t* irow = a.kv_idx + row * NB;
  for (int p = p0; p < p1; ++p)
    if (flags[p]) irow[pos++] = p;
  if (tid == 0) a.kv_cnt[row] = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
}

hipError_t launch_select(const Shape& s, const float* block_scores, const TauArray& tau,
                         uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st) {
  SelectArgs a{block_scores, mask, kv_idx, kv_cnt, s.Hq, s.NB(), s.causal, tau};
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)((size_t)s.B * s.Hq * s.NB())), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace xattn
