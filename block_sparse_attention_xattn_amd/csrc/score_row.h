// One query-block row of normalised block scores from the per-(strided row,
// key block) partial log2-sum-exps, shared by the score finalize pass and the
// fused score+select kernel so both produce bit-identical scores.
//
// Row I's partials are L[J][t] (J < NB key blocks, t < RB); the first `rows`
// strided rows are real (fewer than RB only in a partial last query block) and
// candidates are J < n_cand.
// lse_t = log2 sum_J 2^L[J][t]; score[J] = (1/rows) sum_{t<rows} 2^(L[J][t] - lse_t).
// emit(J, score) is called once for every J in [0, NB) (0 for non-candidates),
// from some thread of the group. Runs on a group of 256 threads, `tid` being
// the thread's index in it (a 512-thread workgroup may run two rows at once);
// needs the given LDS scratch and passes two workgroup barriers in either
// form; callers synchronise before reading what emit wrote.
#pragma once

#include "common.h"

namespace xattn {

struct ScoreRowLds {
  float red_m[4][32];
  float red_s[4][32];
  float lse[32];
};

// Long rows: thread = key block J (strided by 256), the RB partials of J read
// as one vector; per t an online log2-sum-exp over the thread's blocks, then
// across the wave and the four waves.
template <int RB, class Emit>
__device__ __forceinline__ void block_score_row_long(const float* L, int n_cand, int NB, int rows,
                                                ScoreRowLds& sh, int tid, Emit&& emit) {
  const int lane = tid & 63, wave = tid >> 6;
  // pass 1: per strided row t, log2-sum-exp over candidate blocks
  // U key blocks per thread are loaded together before any is used, so their
  // latencies overlap; they are then taken in the order of J
  constexpr int U = RB >= 32 ? 1 : 32 / RB;
  float m[RB], s[RB];
#pragma unroll
  for (int t = 0; t < RB; ++t) { m[t] = -INFINITY; s[t] = 0.f; }
  for (int J0 = tid; J0 < n_cand; J0 += 256 * U) {
    float xs[U][RB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int J = min(J0 + 256 * u, n_cand - 1);  // in bounds; blocks past n_cand are skipped below
      const float* p = L + (size_t)J * RB;
#pragma unroll
      for (int t = 0; t < RB; ++t) xs[u][t] = p[t];  // unconditional, so the loads stay vectorised
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (J0 + 256 * u >= n_cand) break;
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        const float x = t < rows ? xs[u][t] : -INFINITY;  // rows past the end were never written
        const float mn = fmaxf(m[t], x);
        if (mn != -INFINITY) {
          s[t] = s[t] * fast_exp2(m[t] - mn) + fast_exp2(x - mn);
          m[t] = mn;
        }
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
  for (int J0 = tid; J0 < NB; J0 += 256 * U) {
    float xs[U][RB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int J = min(J0 + 256 * u, n_cand - 1);
      const float* p = L + (size_t)J * RB;
#pragma unroll
      for (int t = 0; t < RB; ++t) xs[u][t] = p[t];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int J = J0 + 256 * u;
      if (J >= NB) break;
      float sc = 0.f;
      if (J < n_cand) {
#pragma unroll
        for (int t = 0; t < RB; ++t) {
          const float e = fast_exp2(xs[u][t] - sh.lse[t]);
          sc += t < rows ? e : 0.f;
        }
        sc *= inv_r;
      }
      emit(J, sc);
    }
  }
}

// Short rows (the many early rows of a causal layer), where the fixed cost of
// the long form's RB wave-wide reductions dominates. Thread layout: t = tid %
// RB (strided row), jl = tid / RB (one of 256/RB key-block lanes); a wave reads
// 64/RB consecutive key-block rows of RB floats, i.e. 256 contiguous bytes. The
// per-t reductions over key blocks run over the lanes sharing t (shuffles at
// offsets RB .. 32, then four waves through LDS) as a max and then a sum of
// 2^(x - max), and the block sums over t run over RB adjacent lanes.
template <int RB, class Emit>
__device__ __forceinline__ void block_score_row_short(const float* L, int n_cand, int NB, int rows,
                                                      ScoreRowLds& sh, int tid, Emit&& emit) {
  static_assert(RB >= 2 && RB <= 32 && (RB & (RB - 1)) == 0, "RB");
  constexpr int JL = 256 / RB;  // key-block lanes
  const int lane = tid & 63, wave = tid >> 6;
  const int t = tid % RB, jl = tid / RB;
  const bool live = t < rows;  // rows past the end were never written
  // A lane's partials (at most RB of them: n_cand <= 256 = JL * RB) are all
  // loaded up front, so their latencies overlap instead of adding up over
  // three dependent passes; the arithmetic below keeps the order of J.
  float xv[RB];
#pragma unroll
  for (int it = 0; it < RB; ++it) {
    const int J = jl + it * JL;
    xv[it] = (live && J < n_cand) ? L[(size_t)J * RB + t] : -INFINITY;
  }
  // pass 1: lse_t = log2 sum_J 2^L[J][t], as a max then a sum of 2^(x - max)
  float m = -INFINITY;
#pragma unroll
  for (int it = 0; it < RB; ++it) m = fmaxf(m, xv[it]);
#pragma unroll
  for (int off = RB; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane < RB) sh.red_m[wave][lane] = m;
  __syncthreads();
  const float mt = fmaxf(fmaxf(sh.red_m[0][t], sh.red_m[1][t]), fmaxf(sh.red_m[2][t], sh.red_m[3][t]));
  float s = 0.f;
  if (live && mt != -INFINITY) {
#pragma unroll
    for (int it = 0; it < RB; ++it)
      if (jl + it * JL < n_cand) s += fast_exp2(xv[it] - mt);
  }
#pragma unroll
  for (int off = RB; off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
  if (lane < RB) sh.red_s[wave][lane] = s;
  __syncthreads();
  const float st = (sh.red_s[0][t] + sh.red_s[1][t]) + (sh.red_s[2][t] + sh.red_s[3][t]);
  const float lse = (mt == -INFINITY) ? -INFINITY : mt + log2f(st);
  // pass 2: score[J] = (1/rows) sum_t 2^(L[J][t] - lse_t), summed over the RB
  // adjacent lanes of key block J (a uniform trip count keeps the shuffles
  // converged)
  const float inv_r = 1.f / (float)rows;
  const int iters = (NB + JL - 1) / JL;  // uniform, so the shuffles stay converged
#pragma unroll
  for (int it = 0; it < RB; ++it) {
    if (it >= iters) break;
    const int J = jl + it * JL;
    float e = 0.f;
    if (J < n_cand && live && lse != -INFINITY) e = fast_exp2(xv[it] - lse);
#pragma unroll
    for (int off = 1; off < RB; off <<= 1) e += __shfl_xor(e, off, 64);
    if (t == 0 && J < NB) emit(J, J < n_cand ? e * inv_r : 0.f);
  }
  // key blocks past the candidates (J >= JL * RB > n_cand) score 0
  for (int it = RB; it < iters; ++it) {
    const int J = jl + it * JL;
    if (t == 0 && J < NB) emit(J, 0.f);
  }
}

// Both forms compute the same sums in a different order; the choice depends
// only on the row, so every caller gets the same bits for a given row.
constexpr int kScoreRowShortMax = 256;

template <int RB, class Emit>
__device__ __forceinline__ void block_score_row(const float* L, int n_cand, int NB, int rows,
                                                ScoreRowLds& sh, int tid, Emit&& emit) {
  if (n_cand <= kScoreRowShortMax)
    block_score_row_short<RB>(L, n_cand, NB, rows, sh, tid, emit);
  else
    block_score_row_long<RB>(L, n_cand, NB, rows, sh, tid, emit);
}

}  // namespace xattn
