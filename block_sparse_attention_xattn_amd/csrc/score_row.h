// One query-block row of normalised block scores from the per-(strided row,
// key block) partial log2-sum-exps, shared by the score finalize pass and the
// fused score+select kernel so both produce bit-identical scores.
//
// Row I's partials are L[J][t] (J < NB key blocks, t < RB); the first `rows`
// strided rows are real (fewer than RB only in a partial last query block) and
// candidates are J < n_cand.
// lse_t = log2 sum_J 2^L[J][t]; score[J] = (1/rows) sum_{t<rows} 2^(L[J][t] - lse_t).
// emit(J, score) is called once for every J in [0, NB) (0 for non-candidates).
// Needs 256 threads and the given LDS scratch.
#pragma once

#include "common.h"

namespace xattn {

struct ScoreRowLds {
  float red_m[4][32];
  float red_s[4][32];
  float lse[32];
};

template <int RB, class Emit>
__device__ __forceinline__ void block_score_row(const float* L, int n_cand, int NB, int rows,
                                                ScoreRowLds& sh, Emit&& emit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // pass 1: per strided row t, log2-sum-exp over candidate blocks
  float m[RB], s[RB];
#pragma unroll
  for (int t = 0; t < RB; ++t) { m[t] = -INFINITY; s[t] = 0.f; }
  for (int J = tid; J < n_cand; J += 256) {
    const float* p = L + (size_t)J * RB;
    float xs[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) xs[t] = p[t];  // unconditional, so the loads stay vectorised
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      const float x = t < rows ? xs[t] : -INFINITY;  // rows past the end were never written
      const float mn = fmaxf(m[t], x);
      if (mn != -INFINITY) {
        s[t] = s[t] * fast_exp2(m[t] - mn) + fast_exp2(x - mn);
        m[t] = mn;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < RB; ++t) {
    float mt = m[t], stv = s[t];
    for (int off = 32; off > 0; off >>= 1) {
      const float mo = __shfl_xor(mt, off, 64), so = __shfl_xor(stv, off, 64);
      const float mn = fmaxf(mt, mo);
      if (mn != -INFINITY) {
        stv = stv * fast_exp2(mt - mn) + so * fast_exp2(mo - mn);
        mt = mn;
      }
    }
    if (lane == 0) { sh.red_m[wave][t] = mt; sh.red_s[wave][t] = stv; }
  }
  __syncthreads();
  if (tid < RB) {
    float mt = -INFINITY, stv = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float mo = sh.red_m[w][tid], so = sh.red_s[w][tid];
      const float mn = fmaxf(mt, mo);
      if (mn != -INFINITY) {
        stv = stv * fast_exp2(mt - mn) + so * fast_exp2(mo - mn);
        mt = mn;
      }
    }
    sh.lse[tid] = mt + log2f(stv);
  }
  __syncthreads();
  // pass 2: block score = (1/rows) sum_t 2^(L[J][t] - lse_t)
  const float inv_r = 1.f / (float)rows;
  for (int J = tid; J < NB; J += 256) {
    float sc = 0.f;
    if (J < n_cand) {
      const float* p = L + (size_t)J * RB;
      float xs[RB];
#pragma unroll
      for (int t = 0; t < RB; ++t) xs[t] = p[t];
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        const float e = fast_exp2(xs[t] - sh.lse[t]);
        sc += t < rows ? e : 0.f;
      }
      sc *= inv_r;
    }
    emit(J, sc);
  }
}

}  // namespace xattn
