// DuSA1 multi-stride block scores (a scoring variant next to the
// antidiagonal and diagonal patterns).
//
// "DuSA: Fast and Accurate Dual-Stage Sparse Attention Mechanism ...",
// rebuttal, "Response to Q2": Q and K of shape (B, H, M, C) are reshaped to
// (B, H, M/S, S, C) and transposed to (B, H, S, M/S, C), and an attention with
// its softmax on the final two dimensions is computed for each of the S
// phases. Phase s holds tokens s, s + S, s + 2S, ...; with strided row i of
// phase s = token i*S + s,
//   p_s[i][j] = softmax_j(score_scale * q[i*S+s] . k[j*S+s])   (j <= i + off/S when causal)
//   block_scores[I][J] = (1 / (S * r_I)) * sum_s sum_{i in I, j in J} p_s[i][j],
// so each row of block scores sums to 1 (r_I = the strided rows of block I).
// Lengths must be multiples of S.
//
// Two passes over the same MFMA work, so no (strided row, key block) partials
// are stored (S times the antidiagonal pattern's would not fit):
//  1. dusa1_lse_kernel: per (phase, strided row), the log2-sum-exp of the scaled
//     logits over all its keys (online over 64-key tiles) -> ws, M floats per head;
//  2. dusa1_block_kernel: per (128 strided query rows, 64 strided keys) tile and
//     every phase, 2^(logit - lse) summed into the tile's blocks in registers,
//     the two halves of each wave added in LDS, and every block score written
//     once (zeros above the causal diagonal).
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (one query row per lane, as in the
// attention kernel); operands are read straight from global memory (the four
// waves of a workgroup share them through the caches).
#include "common.h"
#include "kernels.h"

namespace xattn {

XATTN_DEBUG_COUNTERS

struct Dusa1Args {
  const uint16_t* q;
  const uint16_t* k;
  float* lse;           // [b][h][s][i], log2 units
  float* scores;        // [b][h][I][J]
  int B, Hq, Hkv, S, Rq, Rk, NBq, NBk, offs;  // offs = (Mk - Mq) / S, strided position of query row 0
  float sl2;            // score_scale * log2(e)
};

constexpr int D1_QT = 128;  // strided query rows per workgroup (4 waves x 32)
constexpr int D1_KT = 64;   // strided keys per tile

// Q fragments (B operand) of this wave's 32 strided rows of phase s:
// row i0 + l32 -> token (i0 + l32) * S + s; rows past Rq read row Rq - 1.
template <int C>
__device__ __forceinline__ void d1_load_q(const Dusa1Args& a, const uint16_t* qh, int i0, int s, int l32, int hh,
                                          bf16x8 (&qf)[C / 16]) {
  const int i = min(i0 + l32, a.Rq - 1);
  const uint16_t* row = qh + ((size_t)i * a.S + s) * C + 8 * hh;
#pragma unroll
  for (int kk = 0; kk < C / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * kk));
}

// S^T for keys j0 .. j0+63 of phase s against the wave's queries:
// acc[n][r] = logit(key j0 + 32n + 8(r/4) + 4hh + r%4, query l32); keys past
// Rk read key Rk - 1 (masked by the caller).
template <int C>
__device__ __forceinline__ void d1_tile(const Dusa1Args& a, const uint16_t* kh, int j0, int s, int l32, int hh,
                                        const bf16x8 (&qf)[C / 16], f32x16 (&acc)[2]) {
  acc[0] = acc[1] = f32x16{};
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int j = min(j0 + 32 * n + l32, a.Rk - 1);
    const uint16_t* row = kh + ((size_t)j * a.S + s) * C + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < C / 16; ++kk) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * kk));
      acc[n] = mfma32x32x16(kf, qf[kk], acc[n]);
    }
  }
}

// the strided key of accumulator element (n, r) in this lane, relative to j0
__device__ __forceinline__ int d1_key(int n, int r, int hh) { return 32 * n + 8 * (r >> 2) + 4 * hh + (r & 3); }

template <int C, bool CAUSAL>
__global__ __launch_bounds__(256) void dusa1_lse_kernel(Dusa1Args a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int n_qt = (a.Rq + D1_QT - 1) / D1_QT;
  const int qt = blockIdx.x % n_qt;
  const int s = (blockIdx.x / n_qt) % a.S;
  const size_t bh = blockIdx.x / n_qt / a.S;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = h / (a.Hq / a.Hkv);
  const uint16_t* qh = a.q + bh * (size_t)a.Rq * a.S * C;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.Rk * a.S * C;
  const int i0 = qt * D1_QT + 32 * wave;
  if (i0 >= a.Rq) return;  // no barriers in this kernel
  bf16x8 qf[C / 16];
  d1_load_q<C>(a, qh, i0, s, l32, hh, qf);
  const int qi = i0 + l32 + a.offs;  // this lane's query, strided position among the keys
  const int jmax = CAUSAL ? min(a.Rk - 1, i0 + 31 + a.offs) : a.Rk - 1;  // last key of any of the wave's rows
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 <= jmax; j0 += D1_KT) {
    f32x16 acc[2];
    d1_tile<C>(a, kh, j0, s, l32, hh, qf, acc);
    float x[2][16];
    float mt = -INFINITY;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + d1_key(n, r, hh);
        const bool keep = j < a.Rk && (!CAUSAL || j <= qi);
        x[n][r] = keep ? acc[n][r] * a.sl2 : -INFINITY;
        mt = fmaxf(mt, x[n][r]);
      }
    mt = halves_max(mt);
    const float mn = fmaxf(m, mt);
    if (mn == -INFINITY) continue;  // nothing visible yet for this row
    float sum = 0.f;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += fast_exp2(x[n][r] - mn);
    l = l * fast_exp2(m - mn) + sum;  // m = -inf on the first visible tile: 2^-inf = 0
    m = mn;
  }
  const float lt = halves_sum(l);
  const int i = i0 + l32;
  XATTN_DCHECK(bh < (size_t)a.B * a.Hq && s < a.S, DBG_DUSA1_INDEX);
  if (hh == 0 && i < a.Rq) a.lse[(bh * a.S + s) * (size_t)a.Rq + i] = m + log2f(lt);
}

template <int C, int RB, bool CAUSAL>
__global__ __launch_bounds__(256) void dusa1_block_kernel(Dusa1Args a) {
  constexpr int QB = D1_QT / RB;   // query blocks per tile
  constexpr int KB = D1_KT / RB;   // key blocks per tile
  __shared__ float red[D1_QT][KB + 1];  // per query row, per key block of the tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int n_kt = (a.Rk + D1_KT - 1) / D1_KT;
  const int n_qt = (a.Rq + D1_QT - 1) / D1_QT;
  const int kt = blockIdx.x % n_kt;
  const int qt = (blockIdx.x / n_kt) % n_qt;
  const size_t bh = blockIdx.x / n_kt / n_qt;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = h / (a.Hq / a.Hkv);
  const uint16_t* qh = a.q + bh * (size_t)a.Rq * a.S * C;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.Rk * a.S * C;
  const int q0 = qt * D1_QT, j0 = kt * D1_KT;
  for (int x = tid; x < D1_QT * (KB + 1); x += 256) (&red[0][0])[x] = 0.f;
  __syncthreads();
  const int i0 = q0 + 32 * wave;
  // the tile holds a visible pair for this wave's rows
  const bool work = i0 < a.Rq && (!CAUSAL || j0 <= i0 + 31 + a.offs);
  if (work) {
    const int i = min(i0 + l32, a.Rq - 1);
    const int qi = i + a.offs;
    // per lane: the mass of each key block of the tile for this lane's row,
    // summed over the phases. Element (n, r) holds key A + 4 hh with
    // A = 32n + 8(r/4) + r%4, which falls in key block A / RB + 4 hh / RB of the
    // tile (exact: 4 hh is a multiple of RB when RB <= 4, and A % 8 + 4 hh < 8
    // when RB >= 8), so the register index A / RB is compile-time and the lane's
    // shift 4 hh / RB is applied once at the end
    float acc_kb[KB];
#pragma unroll
    for (int x = 0; x < KB; ++x) acc_kb[x] = 0.f;
    for (int s = 0; s < a.S; ++s) {
      bf16x8 qf[C / 16];
      d1_load_q<C>(a, qh, i0, s, l32, hh, qf);
      const float lse = a.lse[(bh * a.S + s) * (size_t)a.Rq + i];
      f32x16 acc[2];
      d1_tile<C>(a, kh, j0, s, l32, hh, qf, acc);
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = d1_key(n, r, hh);
          const int j = j0 + kl;
          const bool keep = j < a.Rk && (!CAUSAL || j <= qi);
          const float p = keep ? fast_exp2(fmaf(acc[n][r], a.sl2, -lse)) : 0.f;
          acc_kb[(32 * n + 8 * (r >> 2) + (r & 3)) / RB] += p;
        }
    }
    if (i0 + l32 < a.Rq) {
      const int shift = (4 * hh) / RB;
#pragma unroll
      for (int x = 0; x < KB; ++x)
        if (x + shift < KB) atomicAdd(&red[32 * wave + l32][x + shift], acc_kb[x]);
    }
  }
  __syncthreads();
  // block sums over RB strided rows, divided by S * (rows of the block)
  for (int x = tid; x < QB * KB; x += 256) {
    const int ib = x / KB, jb = x % KB;
    const int I = qt * QB + ib, J = kt * KB + jb;
    if (I >= a.NBq || J >= a.NBk) continue;
    const int rows = min(RB, a.Rq - I * RB);
    XATTN_DCHECK(rows >= 1 && bh < (size_t)a.B * a.Hq, DBG_DUSA1_INDEX);
    float sum = 0.f;
    for (int t = 0; t < rows; ++t) sum += red[ib * RB + t][jb];
    a.scores[(bh * a.NBq + I) * (size_t)a.NBk + J] = sum / (float)(a.S * rows);
  }
}

template <int C, int RB>
static hipError_t launch_dusa1_cr(const Shape& s, const Dusa1Args& a, hipStream_t st) {
  const int n_qt = (a.Rq + D1_QT - 1) / D1_QT, n_kt = (a.Rk + D1_KT - 1) / D1_KT;
  const dim3 g1((unsigned)((size_t)s.B * s.Hq * s.stride * n_qt));
  const dim3 g2((unsigned)((size_t)s.B * s.Hq * n_qt * n_kt));
  if (s.causal) {
    hipLaunchKernelGGL((dusa1_lse_kernel<C, true>), g1, dim3(256), 0, st, a);
    hipLaunchKernelGGL((dusa1_block_kernel<C, RB, true>), g2, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((dusa1_lse_kernel<C, false>), g1, dim3(256), 0, st, a);
    hipLaunchKernelGGL((dusa1_block_kernel<C, RB, false>), g2, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int C>
static hipError_t launch_dusa1_c(const Shape& s, const Dusa1Args& a, hipStream_t st) {
  switch (s.r()) {
    case 2: return launch_dusa1_cr<C, 2>(s, a, st);
    case 4: return launch_dusa1_cr<C, 4>(s, a, st);
    case 8: return launch_dusa1_cr<C, 8>(s, a, st);
    case 16: return launch_dusa1_cr<C, 16>(s, a, st);
    case 32: return launch_dusa1_cr<C, 32>(s, a, st);
  }
  return hipErrorInvalidValue;
}

size_t dusa1_lse_bytes(const Shape& s) { return (size_t)s.B * s.Hq * s.M * sizeof(float); }

hipError_t launch_score_dusa1(const Shape& s, const uint16_t* q, const uint16_t* k, float score_scale,
                              float* lse_ws, float* block_scores, hipStream_t st) {
  if (s.M % s.stride || s.Mk % s.stride) return hipErrorInvalidValue;
  Dusa1Args a{q, k, lse_ws, block_scores, s.B, s.Hq, s.Hkv, s.stride, s.M / s.stride, s.Mk / s.stride,
              s.NBq(), s.NBk(), (s.Mk - s.M) / s.stride, score_scale * kLog2e};
  if (s.C == 128) return launch_dusa1_c<128>(s, a, st);
  if (s.C == 64) return launch_dusa1_c<64>(s, a, st);
  return hipErrorInvalidValue;
}


hipError_t debug_counts_dusa1(unsigned int* out, bool reset) {
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
