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
//  1. dusa1_lse_kernel: per (phase, 512 strided query rows), the log2-sum-exp of
//     each row's scaled logits over all its keys, online over 64-key tiles
//     (each lane keeps its own running maximum and sum over its keys; the two
//     halves of the wave, which hold the same rows, are merged at the end)
//     -> ws, M floats per head;
//  2. dusa1_block_kernel: per (512 strided query rows, a range of strided
//     keys), for every phase and key tile of the range, 2^(logit - lse)
//     summed per (row, key block) in registers, over the block's rows by lane
//     shuffles, and into a per-workgroup LDS table of block sums by the one
//     lane that owns each entry (so the order of the additions is fixed); every
//     block score of the range is written once (zeros above the causal
//     diagonal).
// Both: 8 waves of 64 query rows (two 32-row MFMA tiles, so every K fragment
// read feeds two v_mfma_f32_32x32x16_bf16); the phase's K tiles (strided rows
// j*S + s, 64 at a time) go by DMA into a four-tile LDS ring (rows stored with
// their 16-byte chunks XOR-permuted by the row, so fragment reads are
// conflict-free), three tiles in flight; Q fragments stay in registers.
#include <type_traits>

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
  int n_qt, n_kr;       // query tiles of D1_QR rows; key ranges of the block pass
  float sl2;            // score_scale * log2(e)
};

#ifndef XATTN_D1_RPW
#define XATTN_D1_RPW 32
#endif
constexpr int D1_QR = 512;             // strided query rows per workgroup
constexpr int D1_RPW = XATTN_D1_RPW;   // ... per wave: 64 (two 32-row MFMA tiles) or 32
constexpr int D1_QTW = D1_RPW / 32;    // 32-row MFMA tiles per wave
constexpr int D1_NW = D1_QR / D1_RPW;  // waves per workgroup
constexpr int D1_NT = 64 * D1_NW;      // threads per workgroup
static_assert(D1_RPW == 32 || D1_RPW == 64, "rows per wave");
constexpr int D1_KT = 64;              // strided keys per K tile
constexpr int D1_RING = 4;             // K tiles in the LDS ring

// Keys per workgroup of the block pass: its table of block sums,
// (D1_QR / RB) x (keys / RB) floats, stays within 32 KiB.
constexpr int d1_range_keys(int rb) { return 16 * rb * rb < 1024 ? 16 * rb * rb : 1024; }

template <int C>
struct D1Lds {
  static constexpr int ROW_B = 2 * C;                  // bytes per key row
  static constexpr int TILE_B = D1_KT * ROW_B;         // bytes per K tile
  static constexpr int ROWS_PER_256 = 256 / ROW_B;
  static constexpr int BLKS = TILE_B / 1024;           // 1 KiB DMA blocks per tile
  static constexpr int BPW = BLKS >= D1_NW ? BLKS / D1_NW : 1;  // ... per wave (waves past BLKS issue none)
  static constexpr int RPB = 1024 / ROW_B;             // key rows per DMA block
  static constexpr int LPR = ROW_B / 16;               // lanes per key row in a DMA block
  // byte offset of 16-byte chunk `chunk` of key row `row`
  __device__ static int off(int row, int chunk) {
    return row * ROW_B + 16 * (chunk ^ ((row / ROWS_PER_256) % (C / 8)));
  }
};
static_assert(D1Lds<128>::BPW * D1_NW >= D1Lds<128>::BLKS && D1Lds<64>::BPW * D1_NW >= D1Lds<64>::BLKS,
              "DMA blocks per wave");

// DMA of K tile (phase s, strided keys j0 .. j0+63) into ring slot `slot`:
// this wave's BPW blocks; lane L of block b fills key row b*RPB + L/LPR at slot
// L%LPR, i.e. the row's chunk (L%LPR) ^ swizzle. The per-lane byte offsets
// within a tile are fixed, so a whole tile costs a scalar base; only a tile
// that runs past Rk clamps its keys (to key Rk - 1, masked by the caller).
template <int C>
struct D1Dma {
  using L = D1Lds<C>;
  uint32_t voff[L::BPW];  // key row * S * 2C + 16 * chunk
  int row[L::BPW], chunk[L::BPW];
  int wave, S;
  __device__ D1Dma(int wave_, int lane, int S_) : wave(wave_), S(S_) {
#pragma unroll
    for (int u = 0; u < L::BPW; ++u) {
      const int b = wave * L::BPW + u;
      row[u] = b * L::RPB + lane / L::LPR;
      chunk[u] = (lane % L::LPR) ^ ((row[u] / L::ROWS_PER_256) % (C / 8));
      voff[u] = (uint32_t)((row[u] * S * C + 8 * chunk[u]) * 2);
    }
  }
  __device__ void issue(const Dusa1Args& a, const uint16_t* kh, unsigned char* ring, int slot, int s, int j0) const {
    unsigned char* tile = ring + slot * L::TILE_B;
    XATTN_DCHECK(slot >= 0 && slot < D1_RING, DBG_DUSA1_INDEX);
    if (j0 + D1_KT <= a.Rk) {
      const void* base = uniform_ptr(kh + ((size_t)j0 * S + s) * C);
#pragma unroll
      for (int u = 0; u < L::BPW; ++u) {
        const int b = wave * L::BPW + u;
        if (b < L::BLKS) dma16(base, voff[u], lds_addr_u(tile + b * 1024));  // wave-uniform
      }
    } else {
      const void* base = uniform_ptr(kh);
#pragma unroll
      for (int u = 0; u < L::BPW; ++u) {
        const int b = wave * L::BPW + u;
        const int j = min(j0 + row[u], a.Rk - 1);
        const size_t byte = (((size_t)j * S + s) * C + 8 * chunk[u]) * 2;
        XATTN_DCHECK(byte < ((size_t)1 << 32), DBG_DUSA1_INDEX);
        if (b < L::BLKS) dma16(base, (uint32_t)byte, lds_addr_u(tile + b * 1024));
      }
    }
  }
};

// Q fragments (B operand) of this wave's strided rows of phase s:
// row i0 + 32y + l32 -> token (i0 + 32y + l32) * S + s; rows past Rq read row Rq - 1.
template <int C>
__device__ __forceinline__ void d1_load_q(const Dusa1Args& a, const uint16_t* qh, int i0, int s, int l32, int hh,
                                          bf16x8 (&qf)[D1_QTW][C / 16]) {
#pragma unroll
  for (int y = 0; y < D1_QTW; ++y) {
    const int i = min(i0 + 32 * y + l32, a.Rq - 1);
    const uint16_t* row = qh + ((size_t)i * a.S + s) * C + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < C / 16; ++kk)
      qf[y][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * kk));
  }
}

// S^T of a K tile (in LDS) against the wave's rows: acc[n][y][r] = logit of
// key 32n + 8(r/4) + 4hh + r%4 of the tile and query row i0 + 32y + l32.
template <int C>
__device__ __forceinline__ void d1_mma(const unsigned char* kt, const bf16x8 (&qf)[D1_QTW][C / 16], f32x16 (&acc)[2][D1_QTW],
                                       int l32, int hh) {
  using L = D1Lds<C>;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int y = 0; y < D1_QTW; ++y) acc[n][y] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < C / 16; ++kk)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kt + L::off(32 * n + l32, 2 * kk + hh)));
#pragma unroll
      for (int y = 0; y < D1_QTW; ++y) acc[n][y] = mfma32x32x16(kf, qf[y][kk], acc[n][y]);
    }
}

// the strided key of accumulator element (n, r) in this lane, relative to the tile
__device__ __forceinline__ int d1_key(int n, int r, int hh) { return 32 * n + 8 * (r >> 2) + 4 * hh + (r & 3); }

template <int C, bool CAUSAL>
__global__ __launch_bounds__(D1_NT, 1) void dusa1_lse_kernel(Dusa1Args a) {
  using L = D1Lds<C>;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[D1_RING * L::TILE_B];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  // (b, h, s, query tile); causal: the query tiles that see the most keys first
  const int qr = blockIdx.x % a.n_qt;
  const int qt = CAUSAL ? a.n_qt - 1 - qr : qr;
  const int s = (blockIdx.x / a.n_qt) % a.S;
  const size_t bh = blockIdx.x / a.n_qt / a.S;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = h / (a.Hq / a.Hkv);
  const uint16_t* qh = a.q + bh * (size_t)a.Rq * a.S * C;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.Rk * a.S * C;
  const D1Dma<C> dma(wave, lane, a.S);
  const int q0 = qt * D1_QR, i0 = q0 + D1_RPW * wave;
  const int last_row = min(q0 + D1_QR, a.Rq) - 1;
  const int jend = CAUSAL ? min(a.Rk, last_row + a.offs + 1) : a.Rk;  // keys seen by some row of the tile
  const int n_t = (jend + D1_KT - 1) / D1_KT;                          // >= 1
  bf16x8 qf[D1_QTW][C / 16];
  d1_load_q<C>(a, qh, i0, s, l32, hh, qf);
  // the Q loads complete before any DMA is issued: a wait the compiler sees,
  // so it places none of its own in the loop (its count ignores the DMA,
  // and such a wait would drain the ring's lookahead every step)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  float m[D1_QTW], l[D1_QTW];
#pragma unroll
  for (int y = 0; y < D1_QTW; ++y) {
    m[y] = -INFINITY;
    l[y] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < D1_RING - 1; ++u) dma.issue(a, kh, ring, u, s, min(u, n_t - 1) * D1_KT);
  for (int t = 0; t < n_t; ++t) {
    vm_wait<2 * L::BPW>();  // tile t landed (t+1, t+2 may be in flight)
    __syncthreads();        // ... for every wave; all are done with tile t-1's slot
    // past the end: the last tile again, into a slot that is never read
    dma.issue(a, kh, ring, (t + 3) % D1_RING, s, min(t + 3, n_t - 1) * D1_KT);
    const int j0 = t * D1_KT;
    if (i0 < a.Rq && (!CAUSAL || j0 <= i0 + D1_RPW - 1 + a.offs)) {
      f32x16 acc[2][D1_QTW];
      d1_mma<C>(ring + (t % D1_RING) * L::TILE_B, qf, acc, l32, hh);
      // the masked form only on tiles that cross the diagonal or the last key
      // (one branch per tile, not per element)
      auto update = [&](auto masked) {
#pragma unroll
        for (int y = 0; y < D1_QTW; ++y) {
          const int qi = i0 + 32 * y + l32 + a.offs;  // this lane's row among the keys
          float mt = -INFINITY;  // raw maximum: sl2 > 0, so the scaled maximum is mt * sl2
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if constexpr (decltype(masked)::value) {
                const int j = j0 + d1_key(n, r, hh);
                acc[n][y][r] = (j >= a.Rk || (CAUSAL && j > qi)) ? -INFINITY : acc[n][y][r];
              }
              mt = fmaxf(mt, acc[n][y][r]);
            }
          const float mn = fmaxf(m[y], mt * a.sl2);
          const float mu = mn == -INFINITY ? 0.f : mn;  // no visible key yet: every term is 0
          float sum = 0.f;
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += fast_exp2(fmaf(acc[n][y][r], a.sl2, -mu));
          l[y] = l[y] * fast_exp2(m[y] - mu) + sum;  // m = -inf before the first visible key: 2^-inf = 0
          m[y] = mn;
        }
      };
      if ((CAUSAL && j0 + D1_KT - 1 > i0 + a.offs) || j0 + D1_KT > a.Rk)
        update(std::true_type{});
      else
        update(std::false_type{});
    }
  }
  vm_wait<0>();  // the trailing loads, so no DMA reaches the ring after the workgroup
#pragma unroll
  for (int y = 0; y < D1_QTW; ++y) {
    // the two halves of the wave hold the same row over different keys
    const float mt = halves_max(m[y]);
    const float lt = halves_sum(m[y] == -INFINITY ? 0.f : l[y] * fast_exp2(m[y] - mt));
    const int i = i0 + 32 * y + l32;
    XATTN_DCHECK(bh < (size_t)a.B * a.Hq && s < a.S, DBG_DUSA1_INDEX);
    if (hh == 0 && i < a.Rq) a.lse[(bh * a.S + s) * (size_t)a.Rq + i] = mt + log2f(lt);
  }
}

template <int C, int RB, bool CAUSAL>
__global__ __launch_bounds__(D1_NT, 1) void dusa1_block_kernel(Dusa1Args a) {
  using L = D1Lds<C>;
  constexpr int KR = d1_range_keys(RB);  // strided keys per workgroup
  constexpr int QB = D1_QR / RB;         // query blocks per workgroup
  constexpr int KBR = KR / RB;           // key blocks per workgroup
  constexpr int KBT = D1_KT / RB;        // key blocks per K tile
  static_assert(KR % D1_KT == 0 && QB * KBR * 4 <= 32768, "block-sum table");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[D1_RING * L::TILE_B];
  __shared__ float red[QB][KBR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int kr = blockIdx.x % a.n_kr;
  const int qt = (blockIdx.x / a.n_kr) % a.n_qt;
  const size_t bh = blockIdx.x / a.n_kr / a.n_qt;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = h / (a.Hq / a.Hkv);
  const uint16_t* qh = a.q + bh * (size_t)a.Rq * a.S * C;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.Rk * a.S * C;
  const D1Dma<C> dmap(wave, lane, a.S);
  const int q0 = qt * D1_QR, k0 = kr * KR, i0 = q0 + D1_RPW * wave;
  for (int x = tid; x < QB * KBR; x += D1_NT) (&red[0][0])[x] = 0.f;
  const int last_row = min(q0 + D1_QR, a.Rq) - 1;
  int kend = min(k0 + KR, a.Rk);
  if (CAUSAL) kend = min(kend, last_row + a.offs + 1);
  const int n_t = kend > k0 ? (kend - k0 + D1_KT - 1) / D1_KT : 0;  // visible tiles of the range
  const int n_u = n_t * a.S;                                        // (phase, tile) steps, phase-major
  __syncthreads();
  if (n_u > 0) {
    auto dma = [&](int u) {  // step u (clamped to the last)
      const int uu = min(u, n_u - 1), su = uu / n_t;
      dmap.issue(a, kh, ring, u % D1_RING, su, k0 + (uu - su * n_t) * D1_KT);
    };
#pragma unroll
    for (int u = 0; u < D1_RING - 1; ++u) dma(u);
    bf16x8 qf[D1_QTW][C / 16];
    float lse_r[D1_QTW] = {};
    for (int u = 0; u < n_u; ++u) {
      const int s = u / n_t, t = u - s * n_t;
      vm_wait<2 * L::BPW>();  // step u landed (u+1, u+2 may be in flight)
      __syncthreads();        // ... for every wave; all are done with step u-1's slot
      if (t == 0) {
        // a new phase: its Q rows and log-sum-exps, waited for (with a wait
        // the compiler sees) before this step's DMA, so no wait of the
        // compiler's lands behind a DMA in flight
        d1_load_q<C>(a, qh, i0, s, l32, hh, qf);
#pragma unroll
        for (int y = 0; y < D1_QTW; ++y)
          lse_r[y] = a.lse[(bh * a.S + s) * (size_t)a.Rq + min(i0 + 32 * y + l32, a.Rq - 1)];
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      dma(u + 3);  // past the end: the last step again, into a slot that is never read
      const int j0 = k0 + t * D1_KT;
      if (i0 < a.Rq && (!CAUSAL || j0 <= i0 + D1_RPW - 1 + a.offs)) {
        f32x16 acc[2][D1_QTW];
        d1_mma<C>(ring + (u % D1_RING) * L::TILE_B, qf, acc, l32, hh);
        // rows past Rq (a partial last query block) read row Rq - 1 and must add
        // nothing to their block's sum; the masked form only where a mask
        // applies (one branch per tile, not per element)
        auto sums = [&](auto masked) {
#pragma unroll
        for (int y = 0; y < D1_QTW; ++y) {
          const int qi = i0 + 32 * y + l32 + a.offs;
          const bool row_ok = i0 + 32 * y + l32 < a.Rq;
          // per key block of the tile: this lane's mass. Element (n, r) holds key
          // A + 4hh with A = 32n + 8(r/4) + r%4, in block A / RB + 4hh / RB (exact:
          // 4hh is a multiple of RB when RB <= 4, and A % 8 + 4hh < 8 when RB >= 8)
          float kb[KBT];
#pragma unroll
          for (int x = 0; x < KBT; ++x) kb[x] = 0.f;
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float p = fast_exp2(fmaf(acc[n][y][r], a.sl2, -lse_r[y]));
              if constexpr (decltype(masked)::value) {
                const int j = j0 + d1_key(n, r, hh);
                p = (j >= a.Rk || (CAUSAL && j > qi) || !row_ok) ? 0.f : p;
              }
              kb[(32 * n + 8 * (r >> 2) + (r & 3)) / RB] += p;
            }
          // RB >= 8: both halves hold the same blocks; then the block's RB rows,
          // RB consecutive lanes of a half
#pragma unroll
          for (int x = 0; x < KBT; ++x) {
            if constexpr (RB >= 8) kb[x] = halves_sum(kb[x]);
#pragma unroll
            for (int off = 1; off < RB; off <<= 1) kb[x] += __shfl_xor(kb[x], off, 64);
          }
          const int rl = D1_RPW * wave + 32 * y + l32;  // row within the workgroup
          // the owner of each entry: the block's first row, in the half that
          // holds its keys; with RB <= 4 a lane holds only the blocks whose keys
          // start in the first half of an 8-key group (the other half's lanes
          // hold the rest), and writes no other entry of the shared row
          if (rl % RB == 0 && (RB <= 4 || hh == 0) && i0 + 32 * y + l32 < a.Rq) {
            const int shift = (4 * hh) / RB;
#pragma unroll
            for (int x = 0; x < KBT; ++x)
              if ((RB >= 8 || (x * RB) % 8 < 4) && x + shift < KBT) {
                XATTN_DCHECK(rl / RB < QB && t * KBT + x + shift < KBR, DBG_DUSA1_INDEX);
                red[rl / RB][t * KBT + x + shift] += kb[x];
              }
          }
        }
        };
        if ((CAUSAL && j0 + D1_KT - 1 > i0 + a.offs) || j0 + D1_KT > a.Rk || i0 + D1_RPW > a.Rq)
          sums(std::true_type{});
        else
          sums(std::false_type{});
      }
    }
    vm_wait<0>();  // the trailing loads, so no DMA reaches the ring after the workgroup
  }
  __syncthreads();
  // block sums over the phases and the block's strided rows, divided by S * rows
  for (int x = tid; x < QB * KBR; x += D1_NT) {
    const int il = x / KBR, jl = x % KBR;
    const int I = q0 / RB + il, J = k0 / RB + jl;
    if (I >= a.NBq || J >= a.NBk) continue;
    const int rows = min(RB, a.Rq - I * RB);
    XATTN_DCHECK(rows >= 1 && bh < (size_t)a.B * a.Hq, DBG_DUSA1_INDEX);
    a.scores[(bh * a.NBq + I) * (size_t)a.NBk + J] = red[il][jl] / (float)(a.S * rows);
  }
}

template <int C, int RB>
static hipError_t launch_dusa1_cr(const Shape& s, Dusa1Args a, hipStream_t st) {
  a.n_kr = (a.Rk + d1_range_keys(RB) - 1) / d1_range_keys(RB);
  const dim3 g1((unsigned)((size_t)s.B * s.Hq * s.stride * a.n_qt));
  const dim3 g2((unsigned)((size_t)s.B * s.Hq * a.n_qt * a.n_kr));
  if (s.causal) {
    hipLaunchKernelGGL((dusa1_lse_kernel<C, true>), g1, dim3(D1_NT), 0, st, a);
    hipLaunchKernelGGL((dusa1_block_kernel<C, RB, true>), g2, dim3(D1_NT), 0, st, a);
  } else {
    hipLaunchKernelGGL((dusa1_lse_kernel<C, false>), g1, dim3(D1_NT), 0, st, a);
    hipLaunchKernelGGL((dusa1_block_kernel<C, RB, false>), g2, dim3(D1_NT), 0, st, a);
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
  const int Rq = s.M / s.stride;
  Dusa1Args a{q, k, lse_ws, block_scores, s.B, s.Hq, s.Hkv, s.stride, Rq, s.Mk / s.stride,
              s.NBq(), s.NBk(), (s.Mk - s.M) / s.stride, (Rq + D1_QR - 1) / D1_QR, 0, score_scale * kLog2e};
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
