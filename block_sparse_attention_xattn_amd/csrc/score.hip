// Stages 1-2: strided antidiagonal scoring and softmax-normalised block scores.
//
// Definition ("XAttention: Block Sparse Attention with Antidiagonal Scoring":
// arXiv abstract — antidiagonal sums, lower-left to upper-right, rank block
// importance; AI summary, "Approach" — strided sums within each block,
// softmax-normalised; "DuSA ..." rebuttal, "Response to Q2" — Q and K are
// reshaped to (M/stride, stride*C) and a softmax attention runs on them):
//   A'[i][j] = sum_{s<S} q[i*S+s] . k[j*S+S-1-s],  logit = score_scale * A',
//   causal: j <= i at the strided level; softmax over j per strided row i;
//   block score [I][J] = (1/r) sum_{i in I, j in J} p[i][j].
// Ragged and chunked lengths: tokens past the end of a partial stride group are
// zero vectors; strided keys past the last one are masked; a partial last
// query block divides by its count of real strided rows; with the queries the
// last M of Mk tokens, strided query row i is absolute row i + (Mk - M) / S.
//
// Design: the strided logits are an R x R x (S*C) GEMM per head. The
// (M/S)^2 logit matrix never reaches HBM. Each 256 x 256 output tile
// reduces, in registers, every (strided row i, key block J) cell to a partial
// log2-sum-exp L[J][i]; a second kernel turns each query-block row of partials
// into normalised block scores. Partials are stored [I][J][t] (query block,
// key block, strided row within the block), so one query-block row of partials
// is contiguous and the second pass reads it with unit stride.
//
// GEMM (bf16, gfx950 MFMA 32x32x16): S^T = K~' Q'^T on 256 x 256 output tiles,
// 8 waves in a 2 x 4 grid of 128 x 64 sub-tiles. The tile size is set by L2
// bandwidth: a 256 x 256 tile moves half the L2 bytes per FLOP of a 128 x 128
// one (128 vs 64 FLOP per byte), and its fp32 accumulators already take half the
// register file. The S*C contraction is streamed in chunks: with complete
// stride groups straight from global memory into a four-stage LDS ring (see
// score_partials_dma_kernel); with a partial last stride group through
// registers (zero fill) into a double-buffered LDS tile of 64-element chunks.
// K~' row j, element e is k[j*S + S-1 - e/C][e%C] — the stride group read in
// reverse, so the reversal costs only address arithmetic.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "score_row.h"
#include "select_row.h"

namespace xattn {

XATTN_DEBUG_COUNTERS

struct ScoreArgs {
  const uint16_t* q;
  const uint16_t* k;
  float* ws;
  int B, Hq, Hkv, Mq, Mk, S, Rq, Rk, NBq, NBk;
  int qoff_s;     // absolute strided row of strided query row 0: (Mk - Mq) / S
  int diagonal;   // 1: key row j*S + s instead of j*S + S-1-s
  int Tq, Tk;     // strided tiles per head: ceil(Rq / SC_TILE), ceil(Rk / SC_TILE)
  int c0;         // causal: key tiles of query tile tq are tk <= tq + c0
  int pairs;      // tile pairs per head
  int tail;       // 1: Mq or Mk is not a multiple of S (partial stride groups)
  float scale2;   // score_scale * log2(e)
};

#ifndef XATTN_SCORE_TILE
#define XATTN_SCORE_TILE 256
#endif
constexpr int SC_TILE = XATTN_SCORE_TILE;   // strided keys x strided queries per tile
// Output sub-tile of one wave, strided keys x strided queries (WK x WQ): 128 x 64
// or 64 x 128 (4 x 2 or 2 x 4 MFMA tiles, two waves per SIMD), 64 x 64 (2 x 2,
// four waves per SIMD; 4/3 of the LDS fragment reads per MFMA) or 128 x 128
// (4 x 4, one wave per SIMD with its accumulators in AGPRs). Measured: the DMA
// kernel is fastest with 128 x 64, 1.2% ahead of 64 x 128 at 32K, 128K and 256K
// (64 x 64 about 2% and 128 x 128 about 6% behind 64 x 128 at 256K); the
// register-staged kernel with 64 x 64 (64 x 128 about 3% slower: its staging
// registers leave two waves per SIMD too little room).
// 1: the two-waves-per-SIMD DMA kernel (one workgroup per tile) also runs the
// hand-pipelined chunk loop (fragment reads of the next k-step ahead of the
// MFMAs, across the barrier); 0: the plain loop. Measured with one workgroup
// per tile: 2.4% faster at 256K, 1.2% at 128K, neutral at 32K; the same loop
// in the persistent kernel was 3-8% slower than its plain loop (registers
// spilled around the chunk loop, reloaded every tile), and the persistent
// plain loop is the faster of all, so this stays off.
#ifndef XATTN_SCORE_KPIPE
#define XATTN_SCORE_KPIPE 0
#endif
#ifndef XATTN_SCORE_DMA_WK
#define XATTN_SCORE_DMA_WK 128
#endif
#ifndef XATTN_SCORE_DMA_WQ
#define XATTN_SCORE_DMA_WQ 64
#endif
#ifndef XATTN_SCORE_REG_WK
#define XATTN_SCORE_REG_WK 64
#endif
#ifndef XATTN_SCORE_REG_WQ
#define XATTN_SCORE_REG_WQ 64
#endif
template <int WK_, int WQ_>
struct ScWave {
  static constexpr int WK = WK_, WQ = WQ_;
  static constexpr int MTK = WK / 32, MTQ = WQ / 32;            // MFMA tiles per wave, each side
  static constexpr int WNK = SC_TILE / WK, WNQ = SC_TILE / WQ;  // waves per tile side
  static constexpr int NT = 64 * WNK * WNQ;                     // threads per workgroup
  static constexpr int MINW = NT / 256;                         // waves per SIMD the kernel is built for
};
using ScDma = ScWave<XATTN_SCORE_DMA_WK, XATTN_SCORE_DMA_WQ>;
using ScReg = ScWave<XATTN_SCORE_REG_WK, XATTN_SCORE_REG_WQ>;
#ifndef XATTN_SCORE_KC
#define XATTN_SCORE_KC 64
#endif
constexpr int SC_KC = XATTN_SCORE_KC;  // contraction chunk (elements): 32 or 64
constexpr int SC_CPR = SC_KC / 8;      // 16-byte chunks per operand row
// LDS layout of one operand buffer (128 rows x SC_KC bf16), in elements.
//  KC = 64: rows padded to 144 B (16 B mod 128 B).
//  KC = 32: unpadded 64 B rows, the 4 chunks of a row XOR-permuted by
//           (row / 4) % 4, so 16 lanes reading one chunk of 16 consecutive rows,
//           and 16 lanes writing 4 whole rows, each touch 256 distinct bytes.
constexpr int SC_OP = SC_KC == 64 ? SC_TILE * (SC_KC + 8) : SC_TILE * SC_KC;
__device__ __forceinline__ int sc_off(int row, int chunk) {
  if constexpr (SC_KC == 64) return row * (SC_KC + 8) + chunk * 8;
  return row * SC_KC + 8 * (chunk ^ ((row >> 2) & 3));
}

// Tile pair p of a head -> (query tile, key tile). Causal: query tile tq meets
// key tiles 0 .. min(Tk - 1, tq + c0), a trapezoid (a triangle when the
// queries start at the first token): rows tq < cap hold tq + c0 + 1 pairs
// (cap = Tk - c0 - 1, the first row that reaches Tk), the rest Tk each.
__device__ __forceinline__ void tile_pair(int p, bool causal, int Tq, int Tk, int c0, int& tq, int& tk) {
  if (!causal) {
    tq = p / Tk;
    tk = p % Tk;
    return;
  }
  const int cap = max(0, min(Tq, Tk - c0 - 1));
  const int p1 = cap * (cap + 1) / 2 + c0 * cap;  // pairs in the rows below cap
  if (p >= p1) {
    tq = cap + (p - p1) / Tk;
    tk = (p - p1) % Tk;
    return;
  }
  // largest x with x (x + 1) / 2 + c0 x <= p
  const float b = 2.f * (float)c0 + 1.f;
  int x = (int)((sqrtf(b * b + 8.f * (float)p) - b) * 0.5f);
  while ((x + 1) * (x + 2) / 2 + c0 * (x + 1) <= p) ++x;
  while (x * (x + 1) / 2 + c0 * x > p) --x;
  tq = x;
  tk = p - (x * (x + 1) / 2 + c0 * x);
}

// The (b, h, query tile, key tile) of this workgroup. Consecutive items are the
// query heads of one KV group on one tile pair, tile pairs in row order (key
// tiles of one query tile), and XATTN_SCORE_XCD_GROUP consecutive items share
// an XCD: with 32 (eight tile pairs of four heads), the strided-query tile is
// read by eight workgroups and each strided-key tile by four through one L2.
// Measured on the 256K layer: groups of 32 score about 6% faster than groups of
// 4 (one tile pair), 64 about the same, 128 and 256 1% slower.
#ifndef XATTN_SCORE_XCD_GROUP
#define XATTN_SCORE_XCD_GROUP 32
#endif
struct ScoreTile {
  size_t bh, bg;
  int i0, j0;  // first strided query row / strided key of the tile
  // w: the workgroup's index in launch order (blockIdx.x, or the k-th tile of a
  // persistent workgroup: blockIdx.x + k gridDim.x)
  __device__ ScoreTile(const ScoreArgs& a, bool causal, uint32_t w) {
    const uint32_t n_items = (uint32_t)a.B * a.Hq * a.pairs;
    const uint32_t item = xcd_map(w, n_items, XATTN_SCORE_XCD_GROUP);
    const int G = a.Hq / a.Hkv;
    const int hq_in = item % G;
    uint32_t rest = item / G;
    const int pair = rest % a.pairs;
    rest /= a.pairs;
    const int g = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int h = g * G + hq_in;
    int tq, tk;
    tile_pair(pair, causal, a.Tq, a.Tk, a.c0, tq, tk);
    bh = (size_t)b * a.Hq + h;
    bg = (size_t)b * a.Hkv + g;
    i0 = tq * SC_TILE;
    j0 = tk * SC_TILE;
  }
};

// Tile epilogue: per (strided row i, run of RB strided keys) the partial
// log2-sum-exp of the scaled logits, masked causally and past the last key.
template <int RB, bool CAUSAL, class W>
__device__ __forceinline__ void score_epilogue(const ScoreArgs& a, const f32x16 (&acc)[W::MTK][W::MTQ],
                                               size_t bh, int i0, int j0, int wk, int wq, int l32, int hh) {
  // acc[x][y][r] is strided key j = j0 + WK wk + 32x + 8(r/4) + 4hh + r%4 and
  // strided query i = i0 + WQ wq + 32y + l32; each run of RB keys is reduced.
  float* wsh = a.ws + bh * (size_t)a.NBq * a.NBk * RB;
  if constexpr (RB <= 4) {
    // each run of RB keys lies inside one lane's group of 4 registers
#pragma unroll
    for (int y = 0; y < W::MTQ; ++y) {
      const int i = i0 + W::WQ * wq + 32 * y + l32;
      const int ia = i + a.qoff_s;  // absolute strided row
#pragma unroll
      for (int x = 0; x < W::MTK; ++x) {
        const int jb = j0 + W::WK * wk + 32 * x;  // first strided key of this 32-key sub-tile
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jb + 8 * (r >> 2) + 4 * hh + (r & 3);
          float xv = acc[x][y][r] * a.scale2;
          if ((CAUSAL && j > ia) || j >= a.Rk) xv = -INFINITY;
          v[r] = xv;
        }
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += RB) {
          float m = v[r0];
#pragma unroll
          for (int u = 1; u < RB; ++u) m = fmaxf(m, v[r0 + u]);
          float s = 0.f;
          if (m != -INFINITY) {
#pragma unroll
            for (int u = 0; u < RB; ++u) s += fast_exp2(v[r0 + u] - m);
          }
          const float Lv = (m == -INFINITY) ? -INFINITY : m + log2f(s);
          const int j = jb + 8 * (r0 >> 2) + 4 * hh + (r0 & 3);
          const int J = j / RB;
          if (i < a.Rq && j < a.Rk) {
            XATTN_DCHECK(i / RB < a.NBq && J < a.NBk, DBG_SCORE_STORE);
            wsh[((size_t)(i / RB) * a.NBk + J) * RB + i % RB] = Lv;
          }
        }
      }
    }
  } else {
    // A run of RB >= 8 keys occupies registers [r0, r0 + RB/2) in both wave
    // halves. Neighbouring runs A and B are exchanged between the halves with
    // one v_permlane32_swap per register pair, after which each lane holds all
    // RB logits of one run (the lower half run A, the upper half run B): max
    // and sum need no cross-lane step, and every lane stores a result.
    constexpr int NR = RB / 2;              // registers per half per run
    constexpr int RUNS = 32 * W::MTK / RB;  // runs along this wave's keys (even)
    // wave-uniform: only waves holding keys past a query's causal limit or past
    // the last strided key mask anything
    const int jw = j0 + W::WK * wk;         // first strided key of the wave
    const bool need_mask = (CAUSAL && jw + W::WK - 1 > i0 + W::WQ * wq + a.qoff_s) || jw + W::WK > a.Rk;
#pragma unroll
    for (int y = 0; y < W::MTQ; ++y) {
      const int i = i0 + W::WQ * wq + 32 * y + l32;
      const int ia = i + a.qoff_s;  // absolute strided row
#pragma unroll
      for (int q = 0; q < RUNS; q += 2) {
        const int xa = (q * RB) / 32, ra = ((q * RB) % 32) / 2;
        const int xb = ((q + 1) * RB) / 32, rb = (((q + 1) * RB) % 32) / 2;
        // lo[k], hi[k]: keys jr + 8(k/4) + k%4 and that + 4 of this lane's run
        float lo[NR], hi[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[xa][y][ra + k]),
                                                          __float_as_uint(acc[xb][y][rb + k]), false, false);
          lo[k] = __uint_as_float(r[0]);
          hi[k] = __uint_as_float(r[1]);
        }
        const int jr = jw + (q + hh) * RB;  // first key of this lane's run
        if (need_mask) {
#pragma unroll
          for (int k = 0; k < NR; ++k) {
            const int jl = jr + 8 * (k >> 2) + (k & 3), jh = jl + 4;
            if ((CAUSAL && jl > ia) || jl >= a.Rk) lo[k] = -INFINITY;
            if ((CAUSAL && jh > ia) || jh >= a.Rk) hi[k] = -INFINITY;
          }
        }
        float m = lo[0];
#pragma unroll
        for (int k = 0; k < NR; ++k) m = fmaxf(fmaxf(m, lo[k]), hi[k]);
        // scale2 > 0, so the max of the scaled logits is the scaled max; the
        // scale is folded into one FMA per logit
        const float ms = m * a.scale2;
        const float mu = (ms == -INFINITY) ? 0.f : ms;
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < NR; ++k)
          sum += fast_exp2(fmaf(lo[k], a.scale2, -mu)) + fast_exp2(fmaf(hi[k], a.scale2, -mu));
        // sum >= 1 (the max term), so the hardware log2 needs no denormal care
        const float Lv = (ms == -INFINITY) ? -INFINITY : ms + __builtin_amdgcn_logf(sum);
        if (i < a.Rq && jr < a.Rk) {
          XATTN_DCHECK(i / RB < a.NBq && jr / RB < a.NBk, DBG_SCORE_STORE);
          wsh[((size_t)(i / RB) * a.NBk + jr / RB) * RB + i % RB] = Lv;
        }
      }
    }
  }
}

// Register-staged pipeline, used when Mq or Mk is not a multiple of S (TAIL:
// the last stride group of Q or K is partial and reads as zeros; a separate
// instantiation keeps the common loop branch-free) or when the DMA kernel is
// switched off.
template <int C, int RB, bool CAUSAL, bool TAIL>
__global__ __launch_bounds__(ScReg::NT, ScReg::MINW) void score_partials_bf16_kernel(ScoreArgs a) {
  using W = ScReg;
  static_assert(RB == 2 || RB == 4 || RB == 8 || RB == 16 || RB == 32, "r");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * SC_OP];
  uint16_t* Ks = smem;               // [2][SC_TILE rows] strided keys (A operand)
  uint16_t* Qs = smem + 2 * SC_OP;   // [2][SC_TILE rows] strided queries (B operand)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wk = wave / W::WNQ, wq = wave % W::WNQ;

  const ScoreTile tl(a, CAUSAL, blockIdx.x);
  const size_t bh = tl.bh;
  const uint16_t* qh = a.q + tl.bh * a.Mq * C;
  const uint16_t* kh = a.k + tl.bg * a.Mk * C;
  const int i0 = tl.i0, j0 = tl.j0;  // strided row / key origin
  const int S = a.S;
  const int n_chunks = S * C / SC_KC;

  // global -> register staging: SC_TILE rows x SC_KC elements per operand.
  // Row pointers are formed once; per chunk only a uniform offset changes.
  // Rows past the last strided row (a ragged last tile) are clamped to it: they
  // load valid memory and their outputs are never stored.
  constexpr int LPT = SC_TILE * SC_CPR / W::NT;  // 16-byte loads per thread per operand
  static_assert(LPT * W::NT == SC_TILE * SC_CPR, "tile load must divide evenly");
  const uint16_t* kp[LPT];
  const uint16_t* qp[LPT];
  int ktok[LPT], qtok[LPT];  // token of the row's first (Q) / base (K) element
#pragma unroll
  for (int p = 0; p < LPT; ++p) {
    const int id = tid + W::NT * p;
    const int row = id / SC_CPR, col = (id % SC_CPR) * 8;
    const int j = min(j0 + row, a.Rk - 1), i = min(i0 + row, a.Rq - 1);
    // antidiagonal: the stride group is read in reverse (row j*S + S-1-s)
    ktok[p] = j * S + (a.diagonal ? 0 : S - 1);
    qtok[p] = i * S;
    kp[p] = kh + (size_t)ktok[p] * C + col;
    qp[p] = qh + (size_t)qtok[p] * C + col;
  }
  const int kdir = a.diagonal ? 1 : -1;
  typedef u32x4 Stage[2 * LPT];  // K chunks then Q chunks
  auto load_chunk = [&](int c, Stage& r) {
    const int srow = (SC_KC * c) / C, col0 = (SC_KC * c) % C;
    const int koff = kdir * srow * C + col0, qoff = srow * C + col0;
    if constexpr (!TAIL) {
#pragma unroll
      for (int p = 0; p < LPT; ++p) {
        r[p] = *reinterpret_cast<const u32x4*>(kp[p] + koff);
        r[LPT + p] = *reinterpret_cast<const u32x4*>(qp[p] + qoff);
      }
    } else {
      // tokens past the end of a partial stride group read as zeros; the load
      // address is pulled back to the last token, so it stays in bounds
#pragma unroll
      for (int p = 0; p < LPT; ++p) {
        const int kover = max(0, ktok[p] + kdir * srow - (a.Mk - 1));
        const int qover = max(0, qtok[p] + srow - (a.Mq - 1));
        const u32x4 kv = *reinterpret_cast<const u32x4*>(kp[p] + koff - (ptrdiff_t)kover * C);
        const u32x4 qv = *reinterpret_cast<const u32x4*>(qp[p] + qoff - (ptrdiff_t)qover * C);
        r[p] = kover ? u32x4{0u, 0u, 0u, 0u} : kv;
        r[LPT + p] = qover ? u32x4{0u, 0u, 0u, 0u} : qv;
      }
    }
  };
  auto store_chunk = [&](int buf, const Stage& r) {
#pragma unroll
    for (int p = 0; p < LPT; ++p) {
      const int id = tid + W::NT * p;
      const int row = id / SC_CPR, chunk = id % SC_CPR;
      *reinterpret_cast<u32x4*>(Ks + buf * SC_OP + sc_off(row, chunk)) = r[p];
      *reinterpret_cast<u32x4*>(Qs + buf * SC_OP + sc_off(row, chunk)) = r[LPT + p];
    }
  };

  f32x16 acc[W::MTK][W::MTQ];
#pragma unroll
  for (int x = 0; x < W::MTK; ++x)
#pragma unroll
    for (int y = 0; y < W::MTQ; ++y) acc[x][y] = f32x16{};

  auto mma_chunk = [&](int buf) {
    const uint16_t* Kb = Ks + buf * SC_OP;
    const uint16_t* Qb = Qs + buf * SC_OP;
#pragma unroll
    for (int ks = 0; ks < SC_KC / 16; ++ks) {
      bf16x8 af[W::MTK], bfr[W::MTQ];
#pragma unroll
      for (int x = 0; x < W::MTK; ++x)
        af[x] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Kb + sc_off(W::WK * wk + 32 * x + l32, 2 * ks + hh)));
#pragma unroll
      for (int y = 0; y < W::MTQ; ++y)
        bfr[y] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Qb + sc_off(W::WQ * wq + 32 * y + l32, 2 * ks + hh)));
#pragma unroll
      for (int x = 0; x < W::MTK; ++x)
#pragma unroll
        for (int y = 0; y < W::MTQ; ++y) acc[x][y] = mfma32x32x16(af[x], bfr[y], acc[x][y]);
    }
  };

  // one chunk in flight: chunk c+1 is fetched while chunk c is multiplied
  Stage rs;
  load_chunk(0, rs);
  store_chunk(0, rs);
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    const bool more = c + 1 < n_chunks;
    if (more) load_chunk(c + 1, rs);
    mma_chunk(c & 1);
    if (more) store_chunk((c + 1) & 1, rs);
    __syncthreads();
  }

  score_epilogue<RB, CAUSAL, W>(a, acc, bh, i0, j0, wk, wq, l32, hh);
}

// Complete stride groups (Mq and Mk multiples of S): the operand tiles go from
// global memory straight into LDS (global_load_lds_dwordx4, no register
// staging), three contraction chunks ahead of the MFMAs through a ring of four
// LDS stages. Register staging could keep only one chunk in flight (the
// accumulators fill the register budget of four waves per SIMD), which left the
// waves waiting on L2 misses about a quarter of the time.
//   * chunk: 32 contraction elements; a stage holds SC_TILE strided-key rows
//     then SC_TILE strided-query rows of 64 bytes, the four 16-byte pieces of a
//     row XOR-permuted by (row / 4) % 4 (conflict-free fragment reads);
//   * a DMA instruction fills 1 KiB of LDS, 16 lanes' bytes per row in lane
//     order, so each lane fetches the global piece that belongs at its slot;
//   * per chunk: wait for this wave's DMA of the chunk, barrier (every wave's
//     DMA has landed, and every wave is done with the stage to be refilled),
//     issue the DMA three chunks ahead, multiply. The stages are distinct LDS
//     objects and the loop is unrolled over them, so the compiler tracks which
//     DMA each fragment read depends on and adds no waits of its own.
constexpr int SD_KC = 32;                     // contraction elements per chunk
constexpr int SD_ROW = SD_KC;                 // elements per LDS row
constexpr int SD_STAGE = 2 * SC_TILE * SD_ROW;  // elements per stage (keys, then queries)
constexpr int SD_BLK = 1024 / (2 * SD_ROW);   // rows per 1 KiB DMA block (16)
constexpr int SD_BPW = (SC_TILE / SD_BLK) / (ScDma::NT / 64);  // DMA blocks per operand per wave
static_assert(SD_BPW >= 1 && SD_BPW * (ScDma::NT / 64) * SD_BLK == SC_TILE, "DMA blocks must cover the tile");

__device__ __forceinline__ int sd_off(int row, int chunk) { return row * SD_ROW + 8 * (chunk ^ ((row >> 2) & 3)); }

// Waits until at most N of this wave's loads (DMA included) are outstanding,
// then the workgroup barrier; the empty asm statements keep LDS accesses from
// being moved across it.
// ------------------------------------------------------------------ selection in the scoring launch
//
// xattn_prefill with per-row or GQA-union selection runs normalisation and
// selection inside the scoring launch. Each (b, h, query tile) has an arrival
// counter, zero before the launch. A workgroup that has stored its tile's
// partials adds one to the counter with an agent-scope acquire-release atomic
// (its barrier first orders every wave's stores before that release); the
// workgroup that brings the counter to the query tile's number of key tiles
// then sees every partial of the tile's query-block rows and normalises and
// selects those rows at once, two at a time, one per 256-thread half, with the
// row code of the fused normalise+select kernel, so block scores, masks and
// lists are bit-identical to the staged path's. The halves pass the same
// number of barriers per row (the row code's count depends only on the head's
// tau), and with an odd number of rows the second half repeats the last row,
// writing the same values. The row state of each half lives in one stage of
// the now idle operand ring.
#if !XATTN_SELECT_SORT
template <int RB, bool CAUSAL>
__device__ __forceinline__ void tile_select(const ScoreArgs& a, const TileSelect& sel, size_t bh, int i0,
                                            uint16_t* ring0, uint16_t* ring1, int ring_bytes) {
  using SL = SelectLdsT<SEL_MAX>;
  __shared__ uint32_t last;
  const int tid = threadIdx.x;
  const int tq = i0 / SC_TILE;
  __syncthreads();  // every wave's partials are stored; the ring is no longer read
  if (tid == 0) {
    const uint32_t need = CAUSAL ? (uint32_t)min(a.Tk, tq + a.c0 + 1) : (uint32_t)a.Tk;
    const uint32_t old = __hip_atomic_fetch_add(sel.arrive + bh * a.Tq + tq, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    XATTN_DCHECK(old < need, DBG_SCORE_STORE);
    last = old + 1 == need;
  }
  __syncthreads();
  if (!last) return;
  const int half = tid >> 8, t = tid & 255;
  char* base = reinterpret_cast<char*>(half ? ring1 : ring0);
  SL& sh = *reinterpret_cast<SL*>(base);
  ScoreRowLds& shs = *reinterpret_cast<ScoreRowLds*>(base + sizeof(SL));
  XATTN_DCHECK(sizeof(SL) + sizeof(ScoreRowLds) <= (size_t)ring_bytes, DBG_SELECT_ROW);
  (void)ring_bytes;
  const int NB = a.NBk;
  const int I0 = i0 / RB, I1 = min(a.NBq, I0 + SC_TILE / RB);
  const float tau = sel.tau.v[bh % a.Hq];
  for (int I = I0 + half; I - half < I1; I += 2) {
    const int Ir = min(I, I1 - 1);
    const int Ia = Ir + sel.qoff;
    const int n = CAUSAL ? Ia + 1 : NB;
    const int rows = min(RB, a.Rq - Ir * RB);
    const size_t row = bh * a.NBq + Ir;
    const float* L = a.ws + row * (size_t)NB * RB;
    float* orow = sel.scores ? sel.scores + row * NB : nullptr;
    XATTN_DCHECK(n <= SEL_MAX && NB <= SEL_MAX && rows >= 1 && rows <= RB, DBG_SELECT_ROW);
    __syncthreads();  // the previous row's state is no longer read
    for (int p = t; p < NB; p += 256) sh.flags[p] = 0;
    block_score_row<RB>(L, n, NB, rows, shs, t, [&](int J, float sc) {
      if (orow) orow[J] = sc;
      if (J < n) sh.sc[J] = sc;
    });
    __syncthreads();
    select_radix(sh, t, n, NB, Ia, tau, row, sel.mask, sel.kv_idx, sel.kv_cnt);
  }
}
#endif

template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int C, int RB, bool CAUSAL, bool SELECT>
__global__ __launch_bounds__(ScDma::NT, ScDma::MINW) void score_partials_dma_kernel(ScoreArgs a, TileSelect sel) {
  using W = ScDma;
  static_assert(RB == 2 || RB == 4 || RB == 8 || RB == 16 || RB == 32, "r");
  __shared__ __attribute__((aligned(1024))) uint16_t st0[SD_STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[SD_STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[SD_STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[SD_STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wk = wave / W::WNQ, wq = wave % W::WNQ;
  const ScoreTile tl(a, CAUSAL, blockIdx.x);
  const uint16_t* qh = a.q + tl.bh * a.Mq * C;
  const uint16_t* kh = a.k + tl.bg * a.Mk * C;
  const int S = a.S;
  const int n_chunks = S * C / SD_KC;

  // this lane's piece of DMA block (wave + (NT/64) u): row 16 blk + lane/4,
  // LDS slot lane % 4, holding the row's piece (lane % 4) ^ ((row / 4) % 4);
  // rows past the last strided row are clamped (never stored)
  const int piece = (lane & 3) ^ ((lane >> 4) & 3);
  const uint16_t* kp[SD_BPW];
  const uint16_t* qp[SD_BPW];
#pragma unroll
  for (int u = 0; u < SD_BPW; ++u) {
    const int row = SD_BLK * (wave + (W::NT / 64) * u) + (lane >> 2);
    const int j = min(tl.j0 + row, a.Rk - 1), i = min(tl.i0 + row, a.Rq - 1);
    // antidiagonal: the stride group is read in reverse (row j*S + S-1-s)
    kp[u] = kh + ((size_t)j * S + (a.diagonal ? 0 : S - 1)) * C + 8 * piece;
    qp[u] = qh + (size_t)i * S * C + 8 * piece;
  }
  const int kdir = a.diagonal ? 1 : -1;
  auto issue = [&](int c, uint16_t* stg) {
    const int srow = (SD_KC * c) / C, col0 = (SD_KC * c) % C;
    const ptrdiff_t koff = (ptrdiff_t)kdir * srow * C + col0, qoff = (ptrdiff_t)srow * C + col0;
#pragma unroll
    for (int u = 0; u < SD_BPW; ++u) {
      const int blk = wave + (W::NT / 64) * u;
      __builtin_amdgcn_global_load_lds(kp[u] + koff, (__attribute__((address_space(3))) void*)(stg + blk * 1024 / 2),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(qp[u] + qoff,
                                       (__attribute__((address_space(3))) void*)(stg + SC_TILE * SD_ROW + blk * 1024 / 2),
                                       16, 0, 0);
    }
  };

  f32x16 acc[W::MTK][W::MTQ];
#pragma unroll
  for (int x = 0; x < W::MTK; ++x)
#pragma unroll
    for (int y = 0; y < W::MTQ; ++y) acc[x][y] = f32x16{};

  // chunk c sits in stage cur; the stage nxt (chunk c - 1, done) is refilled
  // with chunk c + 3
  auto mma = [&](const uint16_t* cur) {
#pragma unroll
    for (int ks = 0; ks < SD_KC / 16; ++ks) {
      bf16x8 af[W::MTK], bfr[W::MTQ];
#pragma unroll
      for (int x = 0; x < W::MTK; ++x)
        af[x] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(cur + sd_off(W::WK * wk + 32 * x + l32, 2 * ks + hh)));
#pragma unroll
      for (int y = 0; y < W::MTQ; ++y)
        bfr[y] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(cur + SC_TILE * SD_ROW +
                                                                           sd_off(W::WQ * wq + 32 * y + l32, 2 * ks + hh)));
#pragma unroll
      for (int x = 0; x < W::MTK; ++x)
#pragma unroll
        for (int y = 0; y < W::MTQ; ++y) acc[x][y] = mfma32x32x16(af[x], bfr[y], acc[x][y]);
    }
  };
  // one chunk per barrier; chunk c+3 refills the stage of chunk c-1 (two chunks
  // per barrier, with c+2 and c+3 refilled a step ahead, measured 9% slower:
  // the shorter lookahead costs more than the barriers saved)
  auto step = [&](int c, const uint16_t* cur, uint16_t* nxt) {
    vm_wait_barrier<2 * 2 * SD_BPW>();  // chunks c+1, c+2 may be in flight
    issue(c + 3, nxt);
    __builtin_amdgcn_sched_barrier(0);  // keep the refill ahead of this chunk's work
    mma(cur);
  };
  if constexpr (W::MINW == 1 || XATTN_SCORE_KPIPE) {
    // One wave per SIMD (128 x 128 wave tiles): no second wave hides the
    // fragment reads, so the loop is software-pipelined by hand. The fragments
    // of k-step 1 of chunk c are read while the MFMAs of its k-step 0 run;
    // then the barrier (chunk c+1 landed, every wave done with chunk c's
    // stage), the reads of chunk c+1's k-step 0, and the MFMAs of k-step 1
    // with the refill of chunk c's stage (chunk c+4) issued between them. The
    // ring holds chunk c and three ahead.
    bf16x8 fa0[W::MTK], fb0[W::MTQ], fa1[W::MTK], fb1[W::MTQ];
    auto frags = [&](const uint16_t* stg, int ks, bf16x8 (&af)[W::MTK], bf16x8 (&bq)[W::MTQ]) {
#pragma unroll
      for (int x = 0; x < W::MTK; ++x)
        af[x] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stg + sd_off(W::WK * wk + 32 * x + l32, 2 * ks + hh)));
#pragma unroll
      for (int y = 0; y < W::MTQ; ++y)
        bq[y] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stg + SC_TILE * SD_ROW +
                                                                          sd_off(W::WQ * wq + 32 * y + l32, 2 * ks + hh)));
    };
    // DMA piece p of chunk c: p < SD_BPW a key block, else a query block
    auto piece = [&](int c, uint16_t* stg, int p) {
      const int srow = (SD_KC * c) / C, col0 = (SD_KC * c) % C;
      const int u = p % SD_BPW, blk = wave + (W::NT / 64) * u;
      if (p < SD_BPW)
        __builtin_amdgcn_global_load_lds(kp[u] + ((ptrdiff_t)kdir * srow * C + col0),
                                         (__attribute__((address_space(3))) void*)(stg + blk * 1024 / 2), 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(qp[u] + ((ptrdiff_t)srow * C + col0),
                                         (__attribute__((address_space(3))) void*)(stg + SC_TILE * SD_ROW + blk * 1024 / 2),
                                         16, 0, 0);
    };
    constexpr int NM = W::MTK * W::MTQ;            // MFMAs per k-step
    constexpr int PER = NM / (2 * SD_BPW);         // MFMAs per DMA piece
    static_assert(PER >= 1 && PER * 2 * SD_BPW == NM, "DMA pieces must spread over the k-step's MFMAs");
    // WAITN: chunks that may still be in flight once chunk c+1 has landed;
    // REFILL: chunk c+4 exists; NEXT: chunk c+1 exists
    auto iter = [&](auto waitn, auto refill, auto next, int c, const uint16_t* cur, const uint16_t* nxt,
                    uint16_t* cur_w) {
      // the reads of k-step 1 go out after the first MFMAs of k-step 0: issued
      // first, they would be waited for with k-step 0's (the LDS counter is
      // waited to zero before the first use)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        acc[m / W::MTQ][m % W::MTQ] = mfma32x32x16(fa0[m / W::MTQ], fb0[m % W::MTQ], acc[m / W::MTQ][m % W::MTQ]);
        if (m == W::MTQ - 1) {
          __builtin_amdgcn_sched_barrier(0);
          frags(cur, 1, fa1, fb1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(next)::value) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of chunk c are done
        vm_wait_barrier<decltype(waitn)::value * 2 * SD_BPW>();
        frags(nxt, 0, fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        acc[m / W::MTQ][m % W::MTQ] = mfma32x32x16(fa1[m / W::MTQ], fb1[m % W::MTQ], acc[m / W::MTQ][m % W::MTQ]);
        if constexpr (decltype(refill)::value) {
          if (m % PER == PER - 1) piece(c + 4, cur_w, m / PER);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using T = std::true_type;
    using F = std::false_type;
    issue(0, st0);
    issue(1, st1);
    issue(2, st2);
    issue(3, st3);
    vm_wait_barrier<3 * 2 * SD_BPW>();  // chunk 0 landed; 1, 2, 3 may be in flight
    frags(st0, 0, fa0, fb0);
    for (int c = 0; c < n_chunks - 4; c += 4) {
      iter(I2{}, T{}, T{}, c, st0, st1, st0);
      iter(I2{}, T{}, T{}, c + 1, st1, st2, st1);
      iter(I2{}, T{}, T{}, c + 2, st2, st3, st2);
      iter(I2{}, T{}, T{}, c + 3, st3, st0, st3);
    }
    iter(I2{}, F{}, T{}, n_chunks - 4, st0, st1, st0);
    iter(I1{}, F{}, T{}, n_chunks - 3, st1, st2, st1);
    iter(I0{}, F{}, T{}, n_chunks - 2, st2, st3, st2);
    iter(I0{}, F{}, F{}, n_chunks - 1, st3, st3, st3);
  } else {
    issue(0, st0);
    issue(1, st1);
    issue(2, st2);
    // n_chunks is a multiple of 4, at least 4 (checked by the launcher); the
    // last group refills only its first step's stage, and its waits count down
    // as fewer chunks remain in flight
    for (int c = 0; c < n_chunks - 4; c += 4) {
      step(c, st0, st3);
      step(c + 1, st1, st0);
      step(c + 2, st2, st1);
      step(c + 3, st3, st2);
    }
    step(n_chunks - 4, st0, st3);
    vm_wait_barrier<2 * 2 * SD_BPW>();  // chunks n-2, n-1 may be in flight
    mma(st1);
    vm_wait_barrier<1 * 2 * SD_BPW>();  // chunk n-1 may be in flight
    mma(st2);
    vm_wait_barrier<0>();
    mma(st3);
  }
  score_epilogue<RB, CAUSAL, W>(a, acc, tl.bh, tl.i0, tl.j0, wk, wq, l32, hh);
#if !XATTN_SELECT_SORT
  if constexpr (SELECT) {
    static_assert(sizeof(SelectLdsT<SEL_MAX>) + sizeof(ScoreRowLds) <= sizeof(st0), "row state must fit a stage");
    tile_select<RB, CAUSAL>(a, sel, tl.bh, tl.i0, st0, st1, (int)sizeof(st0));
  }
#else
  (void)sel;
#endif
}

// Persistent form of the DMA kernel (two waves per SIMD, no selection in the
// launch): one workgroup per CU takes the tiles w, w + grid, w + 2 grid, ...
// of the launch order, the grid a multiple of 8, so every tile still runs on
// the XCD that xcd_map gives it and the tiles in flight at any time are the
// same window as with one workgroup per tile. Once every wave is past chunk
// n-2 of a tile, the first three chunks of the next tile go into the three
// free stages; the last chunk's MFMAs and the epilogue then cover their
// latency, so neither a workgroup launch nor the first chunk's memory latency
// sits between two tiles. The first wait of a tile is a full one: the
// previous tile's partial stores are then in flight too, and loads and stores
// need not complete in issue order, so a partial count would not prove that
// chunk 0 has landed. Needs at least eight chunks (the launcher checks).
template <int C, int RB, bool CAUSAL>
__global__ __launch_bounds__(ScDma::NT, ScDma::MINW) void score_partials_dma_persist_kernel(ScoreArgs a) {
  using W = ScDma;
  static_assert(W::MINW == 2, "persistent form of the two-waves-per-SIMD kernel");
  static_assert(RB == 2 || RB == 4 || RB == 8 || RB == 16 || RB == 32, "r");
  __shared__ __attribute__((aligned(1024))) uint16_t st0[SD_STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[SD_STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[SD_STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[SD_STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wk = wave / W::WNQ, wq = wave % W::WNQ;
  const uint32_t n_items = (uint32_t)a.B * a.Hq * a.pairs;
  const int S = a.S;
  const int n_chunks = S * C / SD_KC;
  const int kdir = a.diagonal ? 1 : -1;
  const int piece = (lane & 3) ^ ((lane >> 4) & 3);

  // this lane's DMA sources for a tile (as in score_partials_dma_kernel)
  const uint16_t* kp[SD_BPW];
  const uint16_t* qp[SD_BPW];
  auto sources = [&](const ScoreTile& t) {
    const uint16_t* qh = a.q + t.bh * a.Mq * C;
    const uint16_t* kh = a.k + t.bg * a.Mk * C;
#pragma unroll
    for (int u = 0; u < SD_BPW; ++u) {
      const int row = SD_BLK * (wave + (W::NT / 64) * u) + (lane >> 2);
      const int j = min(t.j0 + row, a.Rk - 1), i = min(t.i0 + row, a.Rq - 1);
      kp[u] = kh + ((size_t)j * S + (a.diagonal ? 0 : S - 1)) * C + 8 * piece;
      qp[u] = qh + (size_t)i * S * C + 8 * piece;
    }
  };
  auto issue = [&](int c, uint16_t* stg) {
    const int srow = (SD_KC * c) / C, col0 = (SD_KC * c) % C;
    const ptrdiff_t koff = (ptrdiff_t)kdir * srow * C + col0, qoff = (ptrdiff_t)srow * C + col0;
#pragma unroll
    for (int u = 0; u < SD_BPW; ++u) {
      const int blk = wave + (W::NT / 64) * u;
      __builtin_amdgcn_global_load_lds(kp[u] + koff, (__attribute__((address_space(3))) void*)(stg + blk * 1024 / 2),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(qp[u] + qoff,
                                       (__attribute__((address_space(3))) void*)(stg + SC_TILE * SD_ROW + blk * 1024 / 2),
                                       16, 0, 0);
    }
  };
  f32x16 acc[W::MTK][W::MTQ];
  auto mma = [&](const uint16_t* cur) {
#pragma unroll
    for (int ks = 0; ks < SD_KC / 16; ++ks) {
      bf16x8 af[W::MTK], bfr[W::MTQ];
#pragma unroll
      for (int x = 0; x < W::MTK; ++x)
        af[x] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(cur + sd_off(W::WK * wk + 32 * x + l32, 2 * ks + hh)));
#pragma unroll
      for (int y = 0; y < W::MTQ; ++y)
        bfr[y] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(cur + SC_TILE * SD_ROW +
                                                                           sd_off(W::WQ * wq + 32 * y + l32, 2 * ks + hh)));
#pragma unroll
      for (int x = 0; x < W::MTK; ++x)
#pragma unroll
        for (int y = 0; y < W::MTQ; ++y) acc[x][y] = mfma32x32x16(af[x], bfr[y], acc[x][y]);
    }
  };
  auto step = [&](int c, const uint16_t* cur, uint16_t* nxt) {
    vm_wait_barrier<2 * 2 * SD_BPW>();  // chunks c+1, c+2 may be in flight
    issue(c + 3, nxt);
    __builtin_amdgcn_sched_barrier(0);
    mma(cur);
  };

  uint32_t w = blockIdx.x;
  ScoreTile tl(a, CAUSAL, w);
  sources(tl);
  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
  for (;;) {
    // The next tile (after the last one, this tile again: its chunks are
    // fetched once more and never read, an unconditional issue keeps the
    // compiler's own waits out of the loop). Decoded here, while chunk 0 is in
    // flight; the empty asm keeps the decode from sinking to the tail, where
    // it would delay the next tile's first fetches and the last MFMAs.
    const uint32_t wn = w + gridDim.x;
    const bool more = wn < n_items;
    ScoreTile tn(a, CAUSAL, more ? wn : w);
    asm volatile("" : "+s"(tn.bh), "+s"(tn.bg), "+s"(tn.i0), "+s"(tn.j0));
#pragma unroll
    for (int x = 0; x < W::MTK; ++x)
#pragma unroll
      for (int y = 0; y < W::MTQ; ++y) acc[x][y] = f32x16{};
    vm_wait_barrier<0>();  // chunks 0-2 and the previous tile's stores
    issue(3, st3);
    __builtin_amdgcn_sched_barrier(0);
    mma(st0);
    step(1, st1, st0);
    step(2, st2, st1);
    step(3, st3, st2);
    for (int c = 4; c < n_chunks - 4; c += 4) {
      step(c, st0, st3);
      step(c + 1, st1, st0);
      step(c + 2, st2, st1);
      step(c + 3, st3, st2);
    }
    step(n_chunks - 4, st0, st3);
    vm_wait_barrier<2 * 2 * SD_BPW>();  // chunks n-2, n-1 may be in flight
    mma(st1);
    vm_wait_barrier<1 * 2 * SD_BPW>();  // chunk n-1 may be in flight
    mma(st2);
    // every wave is past chunks n-4 .. n-2, its own LDS reads of them included
    // (lgkmcnt too: the scheduler may leave the fragment reads of chunk n-2 in
    // flight across the barrier): stages 0-2 are free for the next tile
    __builtin_amdgcn_s_waitcnt(0);
    vm_wait_barrier<0>();
    sources(tn);
    issue(0, st0);
    issue(1, st1);
    issue(2, st2);
    __builtin_amdgcn_sched_barrier(0);
    mma(st3);
    score_epilogue<RB, CAUSAL, W>(a, acc, tl.bh, tl.i0, tl.j0, wk, wq, l32, hh);
    if (!more) break;
    w = wn;
    tl = tn;
  }
  // the spare fetch lands before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// fp32 inputs: one thread per (strided row i, key block J), plain FMA.
struct ScoreArgsF32 {
  const float* q;
  const float* k;
  float* ws;
  int B, Hq, Hkv, Mq, Mk, C, S, Rq, Rk, NBq, NBk, r, qoff_s, causal, diagonal;
  float scale2;
};

__global__ __launch_bounds__(256) void score_partials_f32_kernel(ScoreArgsF32 a) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t per_head = (size_t)a.Rq * a.NBk;
  const size_t total = per_head * a.B * a.Hq;
  if (gid >= total) return;
  const size_t bh = gid / per_head;
  const int rem = (int)(gid % per_head);
  const int J = rem / a.Rq, i = rem % a.Rq;
  const int ia = i + a.qoff_s;  // absolute strided row
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = h / (a.Hq / a.Hkv);
  if (a.causal && J > ia / a.r) return;   // never read by the finalize pass
  const float* qh = a.q + bh * (size_t)a.Mq * a.C;
  const float* kh = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.Mk * a.C;
  float m = -INFINITY, s = 0.f;
  for (int u = 0; u < a.r; ++u) {
    const int j = J * a.r + u;
    if ((a.causal && j > ia) || j >= a.Rk) break;
    float dot = 0.f;
    for (int st = 0; st < a.S; ++st) {
      const int qt = i * a.S + st, kt = j * a.S + (a.diagonal ? st : a.S - 1 - st);
      if (qt >= a.Mq || kt >= a.Mk) continue;  // zero past the end of a stride group
      const float* qr = qh + (size_t)qt * a.C;
      const float* kr = kh + (size_t)kt * a.C;
      for (int c = 0; c < a.C; ++c) dot = fmaf(qr[c], kr[c], dot);
    }
    const float x = dot * a.scale2;
    const float mn = fmaxf(m, x);
    s = s * fast_exp2(m - mn) + fast_exp2(x - mn);
    m = mn;
  }
  a.ws[bh * (size_t)a.NBq * a.NBk * a.r + ((size_t)(i / a.r) * a.NBk + J) * a.r + i % a.r] =
      (m == -INFINITY) ? -INFINITY : m + log2f(s);
}

// Block scores from partials: one workgroup per (b, h, I).
struct FinalizeArgs {
  const float* ws;
  float* out;
  int B, Hq, Rq, NBq, NBk, qoff, r, causal;
};

template <int RB>
__global__ __launch_bounds__(256) void score_finalize_kernel(FinalizeArgs a) {
  __shared__ ScoreRowLds sh;
  const size_t row = blockIdx.x;  // bh * NBq + I
  const int I = (int)(row % a.NBq);
  const size_t bh = row / a.NBq;
  const int n_cand = a.causal ? I + a.qoff + 1 : a.NBk;
  const int rows = min(RB, a.Rq - I * RB);
  const float* L = a.ws + (bh * (size_t)a.NBq + I) * (size_t)a.NBk * RB;  // [J][t] of row I
  float* orow = a.out + row * a.NBk;
  block_score_row<RB>(L, n_cand, a.NBk, rows, sh, threadIdx.x, [&](int J, float sc) { orow[J] = sc; });
}

// ------------------------------------------------------------------ launchers

#ifndef XATTN_SCORE_DMA
#define XATTN_SCORE_DMA 1
#endif
// 1: the DMA kernel without selection runs persistent workgroups that fetch
// the next tile's first chunks during a tile's last MFMAs and epilogue
// (score_partials_dma_persist_kernel); 0: one workgroup per tile
#ifndef XATTN_SCORE_PERSIST
#define XATTN_SCORE_PERSIST 1
#endif

// The DMA kernel needs complete stride groups and a chunk count that is a
// multiple of the ring's four stages.
static bool dma_ok(const Shape& s) {
  return XATTN_SCORE_DMA && s.M % s.stride == 0 && s.Mk % s.stride == 0 && (s.stride * s.C / SD_KC) % 4 == 0;
}

template <int C, int RB, bool TAIL>
static hipError_t launch_partials_crt(const Shape& s, const ScoreArgs& a, const TileSelect* sel, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)s.B * s.Hq * a.pairs);
  if (!TAIL && dma_ok(s)) {
    static const TileSelect none{};
    if (sel) {
#if XATTN_SELECT_SORT
      return hipErrorInvalidValue;
#else
      if (s.causal)
        hipLaunchKernelGGL((score_partials_dma_kernel<C, RB, true, true>), dim3(grid), dim3(ScDma::NT), 0, st, a, *sel);
      else
        hipLaunchKernelGGL((score_partials_dma_kernel<C, RB, false, true>), dim3(grid), dim3(ScDma::NT), 0, st, a, *sel);
      return hipGetLastError();
#endif
    }
#if XATTN_SCORE_PERSIST
    if (ScDma::MINW == 2 && s.stride * s.C / SD_KC >= 8) {
      auto kern = s.causal ? score_partials_dma_persist_kernel<C, RB, true>
                           : score_partials_dma_persist_kernel<C, RB, false>;
      // whole XCD rounds of resident workgroups (the tile order relies on
      // workgroup w running on XCD w % 8)
      // (below two tiles per workgroup nothing is gained: 2% slower on the
      // 8K layer's 320 tiles, 3-4% faster at 32K, 2% at 128K and 256K)
      const unsigned slots = (unsigned)(resident_workgroups(kern, ScDma::NT) & ~7);
      if (slots > 0 && grid >= 2 * slots) {
        hipLaunchKernelGGL(kern, dim3(std::min(grid, slots)), dim3(ScDma::NT), 0, st, a);
        return hipGetLastError();
      }
    }
#endif
    if (s.causal)
      hipLaunchKernelGGL((score_partials_dma_kernel<C, RB, true, false>), dim3(grid), dim3(ScDma::NT), 0, st, a, none);
    else
      hipLaunchKernelGGL((score_partials_dma_kernel<C, RB, false, false>), dim3(grid), dim3(ScDma::NT), 0, st, a, none);
    return hipGetLastError();
  }
  if (sel) return hipErrorInvalidValue;
  if (s.causal)
    hipLaunchKernelGGL((score_partials_bf16_kernel<C, RB, true, TAIL>), dim3(grid), dim3(ScReg::NT), 0, st, a);
  else
    hipLaunchKernelGGL((score_partials_bf16_kernel<C, RB, false, TAIL>), dim3(grid), dim3(ScReg::NT), 0, st, a);
  return hipGetLastError();
}

template <int C, int RB>
static hipError_t launch_partials_cr(const Shape& s, const ScoreArgs& a, const TileSelect* sel, hipStream_t st) {
  return a.tail ? launch_partials_crt<C, RB, true>(s, a, sel, st) : launch_partials_crt<C, RB, false>(s, a, sel, st);
}

template <int C>
static hipError_t launch_partials_c(const Shape& s, const ScoreArgs& a, const TileSelect* sel, hipStream_t st) {
  switch (s.r()) {
    case 2: return launch_partials_cr<C, 2>(s, a, sel, st);
    case 4: return launch_partials_cr<C, 4>(s, a, sel, st);
    case 8: return launch_partials_cr<C, 8>(s, a, sel, st);
    case 16: return launch_partials_cr<C, 16>(s, a, sel, st);
    case 32: return launch_partials_cr<C, 32>(s, a, sel, st);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_partials(const Shape& s, const uint16_t* q, const uint16_t* k, float score_scale,
                                  float* ws, const TileSelect* sel, hipStream_t st) {
  const int Rq = s.Rq(), Rk = s.Rk();
  const int Tq = (Rq + SC_TILE - 1) / SC_TILE, Tk = (Rk + SC_TILE - 1) / SC_TILE;
  const int qoff_s = (s.Mk - s.M) / s.stride;
  const int c0 = (qoff_s + SC_TILE - 1) / SC_TILE;
  int pairs = 0;
  if (s.causal)
    for (int tq = 0; tq < Tq; ++tq) pairs += std::min(Tk, tq + c0 + 1);
  else
    pairs = Tq * Tk;
  const int tail = (s.M % s.stride) != 0 || (s.Mk % s.stride) != 0;
  ScoreArgs a{q, k, ws, s.B, s.Hq, s.Hkv, s.M, s.Mk, s.stride, Rq, Rk, s.NBq(), s.NBk(), qoff_s,
              s.diagonal, Tq, Tk, c0, pairs, tail, score_scale * kLog2e};
  if (s.C == 128) return launch_partials_c<128>(s, a, sel, st);
  if (s.C == 64) return launch_partials_c<64>(s, a, sel, st);
  return hipErrorInvalidValue;
}

hipError_t launch_score_partials_bf16(const Shape& s, const uint16_t* q, const uint16_t* k,
                                      float score_scale, float* ws, hipStream_t st) {
  return launch_partials(s, q, k, score_scale, ws, nullptr, st);
}

bool tile_select_ok(const Shape& s) {
  const int r = s.r();
  return !XATTN_SELECT_SORT && dma_ok(s) && (s.C == 64 || s.C == 128) && s.diagonal != 2 &&
         s.selection != SEL_GLOBAL && (r == 2 || r == 4 || r == 8 || r == 16 || r == 32) && s.NBk() <= SEL_MAX;
}

size_t arrive_words(const Shape& s) {
  return (size_t)s.B * s.Hq * (size_t)((s.Rq() + SC_TILE - 1) / SC_TILE);
}

hipError_t launch_score_tile_select(const Shape& s, const uint16_t* q, const uint16_t* k, float score_scale,
                                    float* ws, const TileSelect& sel, hipStream_t st) {
  if (!tile_select_ok(s) || !sel.arrive || !sel.kv_idx || !sel.kv_cnt) return hipErrorInvalidValue;
  return launch_partials(s, q, k, score_scale, ws, &sel, st);
}

hipError_t launch_score_partials_f32(const Shape& s, const float* q, const float* k,
                                     float score_scale, float* ws, hipStream_t st) {
  ScoreArgsF32 a{q, k, ws, s.B, s.Hq, s.Hkv, s.M, s.Mk, s.C, s.stride, s.Rq(), s.Rk(), s.NBq(), s.NBk(),
                 s.r(), (s.Mk - s.M) / s.stride, s.causal, s.diagonal, score_scale * kLog2e};
  const size_t total = (size_t)s.Rq() * s.NBk() * s.B * s.Hq;
  hipLaunchKernelGGL(score_partials_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_finalize(const Shape& s, const float* ws, float* block_scores,
                                 hipStream_t st) {
  FinalizeArgs a{ws, block_scores, s.B, s.Hq, s.Rq(), s.NBq(), s.NBk(), s.qoff(), s.r(), s.causal};
  const dim3 grid((unsigned)((size_t)s.B * s.Hq * s.NBq()));
  switch (s.r()) {
    case 2: hipLaunchKernelGGL(score_finalize_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(score_finalize_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(score_finalize_kernel<8>, grid, dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL(score_finalize_kernel<16>, grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(score_finalize_kernel<32>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


hipError_t debug_counts_score(unsigned int* out, bool reset) {
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
