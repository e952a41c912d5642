// Stage 4: block-sparse (and dense) attention forward.
//
// Semantics ("XAttention: Block Sparse Attention with Antidiagonal Scoring",
// arXiv abstract: block-sparse attention computes only on the important
// blocks): for query i of block I, exact softmax attention over the keys of
// the listed key blocks, restricted to keys <= i when causal.
//
// bf16 path (gfx950 MFMA):
//  * one workgroup per (b, h, I) query block; BLK/32 waves, each wave owns 32
//    query rows whose Q fragments stay in VGPRs for the whole row;
//  * key blocks are consumed in 64-key sub-tiles: K and V rows are fetched from
//    HBM into registers one sub-tile ahead and written to a double-buffered LDS
//    tile, so one barrier per sub-tile orders reuse;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 puts one query per lane, so the
//    row max/sum is an in-lane reduction plus one exchange between the wave
//    halves; P^T stays in registers and feeds O^T += V^T P^T directly, with V^T
//    fragments taken from row-major LDS by the transposing LDS read;
//  * online softmax in the log2 domain in fp32; P rounded to bf16 for the PV
//    product; O normalised once at the end and rounded to bf16 (RNE).
// f32 path: one thread per query row with fp32 FMA (small problems only).
#include "common.h"
#include "kernels.h"

namespace xattn {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_idx;  // nullptr: dense
  const int32_t* kv_cnt;
  uint16_t* out;
  float* lse;
  int B, Hq, Hkv, M, NB;
  float scale_log2;  // sm_scale * log2(e)
};

template <int C>
struct AttnLds {
  static constexpr int KT = 64;               // keys per sub-tile
  static constexpr int ROW_B = 2 * C;         // bytes per K or V row (no padding)
  static constexpr int TILE_B = KT * ROW_B;   // bytes per K (or V) sub-tile
  static constexpr int ROWS_PER_256 = 256 / ROW_B;
  static constexpr int IDX_MAX = 4096;        // block-index row cached as uint16
  static constexpr int BYTES = 2 * 2 * TILE_B + 2 * IDX_MAX;
  // LDS serves 256 B per clock in 64 banks of 4 B. Rows are stored unpadded and
  // the 16-byte chunks (K) or 64-byte segments (V) of each row are XOR-permuted
  // by the row index so that
  //  * K fragment reads (16 lanes x 16 B, 16 consecutive rows, same column) and
  //  * V transposing reads (32 lanes x 8 B over 4 consecutive rows x 64 B)
  // each cover 256 distinct bytes of the bank window, while row-major 16-byte
  // tile writes stay conflict-free.
  __device__ static int k_off(int row, int chunk16) {
    return row * ROW_B + 16 * (chunk16 ^ ((row / ROWS_PER_256) % (C / 8)));
  }
  __device__ static int v_off(int row, int byte_in_row) {
    return row * ROW_B + (byte_in_row ^ (64 * ((row / ROWS_PER_256) % (C / 32))));
  }
};

template <int C, int BLK, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(BLK * 2, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  using L = AttnLds<C>;
  constexpr int NT = BLK * 2;                 // threads: BLK/32 waves of 64
  constexpr int SUB = BLK / L::KT;            // sub-tiles per key block
  constexpr int CHUNKS = L::KT * C / 8;       // 16-byte chunks per K (or V) sub-tile
  constexpr int PER_T = CHUNKS / NT;
  constexpr int KK = C / 16;                  // MFMA k-steps over the head dim
  constexpr int DN = C / 32;                  // 32-wide d tiles of O^T
  static_assert(CHUNKS % NT == 0, "tile load must divide evenly");

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
  unsigned char* Ks = smem;                      // [2][KT rows][2C bytes], swizzled
  unsigned char* Vs = smem + 2 * L::TILE_B;      // [2][KT rows][2C bytes], swizzled
  uint16_t* idx_s = reinterpret_cast<uint16_t*>(smem + 4 * L::TILE_B);  // kept key blocks

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work item: heavy query blocks first, GQA siblings on one XCD
  const uint32_t n_items = (uint32_t)a.B * a.Hq * a.NB;
  const uint32_t item = xcd_group4(blockIdx.x, n_items);
  const int G = a.Hq / a.Hkv;
  const int hq_in = item % G;
  uint32_t rest = item / G;
  const int g = rest % a.Hkv;
  rest /= a.Hkv;
  const int b = rest % a.B;
  const int I = a.NB - 1 - (int)(rest / a.B);
  const int h = g * G + hq_in;

  const size_t bh = (size_t)b * a.Hq + h;
  const size_t bg = (size_t)b * a.Hkv + g;
  const uint16_t* qh = a.q + bh * a.M * C;
  const uint16_t* kh = a.k + bg * a.M * C;
  const uint16_t* vh = a.v + bg * a.M * C;

  int cnt;
  constexpr bool sparse = SPARSE;
  if constexpr (SPARSE) {
    cnt = a.kv_cnt[bh * a.NB + I];
    cnt = cnt < 0 ? 0 : (cnt > a.NB ? a.NB : cnt);
    // cache the row's block list in LDS once, so no dependent global load sits
    // in front of each tile fetch; out-of-range entries are clamped
    const int32_t* idx = a.kv_idx + (bh * a.NB + I) * a.NB;
    for (int t = tid; t < cnt; t += NT) {
      int jb = idx[t];
      jb = jb < 0 ? 0 : (jb >= a.NB ? a.NB - 1 : jb);
      idx_s[t] = (uint16_t)jb;
    }
  } else {
    cnt = CAUSAL ? I + 1 : a.NB;
  }
  const int n_sub = cnt * SUB;

  // ---- Q fragments (B operand of S^T = K Q^T): Q[q0 + l32][16kk + 8hh .. +7]
  const int q0 = I * BLK + wave * 32;
  bf16x8 qf[KK];
  {
    const uint16_t* qrow = qh + (size_t)(q0 + l32) * C + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * kk));
  }

  f32x16 o[DN];
#pragma unroll
  for (int d = 0; d < DN; ++d) o[d] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  auto key_start = [&](int t) -> int {
    const int jb = sparse ? (int)idx_s[t / SUB] : t / SUB;
    return jb * BLK + (t % SUB) * L::KT;
  };

  u32x4 kreg[PER_T], vreg[PER_T];
  auto load_tile = [&](int t) {
    const int k0 = key_start(t);
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const int c = tid + p * NT;
      const int row = c / (C / 8), col = (c % (C / 8)) * 8;
      kreg[p] = *reinterpret_cast<const u32x4*>(kh + (size_t)(k0 + row) * C + col);
      vreg[p] = *reinterpret_cast<const u32x4*>(vh + (size_t)(k0 + row) * C + col);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const int c = tid + p * NT;
      const int row = c / (C / 8), chunk = c % (C / 8);
      *reinterpret_cast<u32x4*>(Ks + buf * L::TILE_B + L::k_off(row, chunk)) = kreg[p];
      *reinterpret_cast<u32x4*>(Vs + buf * L::TILE_B + L::v_off(row, 16 * chunk)) = vreg[p];
    }
  };

  __syncthreads();  // block list visible
  if (n_sub > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < n_sub; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < n_sub;
    const int k0 = key_start(t);
    if (more) load_tile(t + 1);

    const bool skip = CAUSAL && (k0 > q0 + 31);  // whole sub-tile above this wave's rows
    if (!skip) {
      const unsigned char* Kb = Ks + buf * L::TILE_B;
      const unsigned char* Vb = Vs + buf * L::TILE_B;
      // S^T tiles n = 0, 1: keys k0 + 32n + [8(r/4) + 4hh + r%4], query q0 + l32
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const bf16x8 ka = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(Kb + L::k_off(32 * n + l32, 2 * kk + hh)));
          s[n] = mfma32x32x16(ka, qf[kk], s[n]);
        }
      }
      if (CAUSAL && (k0 + L::KT - 1 > q0)) {
        const int qi = q0 + l32;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * n + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key > qi) s[n][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[n][r]);
      mx = fmaxf(mx, xor32(mx));
      // Lazy rescaling (exact): O and l share the reference m_run, so the
      // reference may lag the true running max as long as 2^(s*c - m_run) stays
      // small. It is raised only when the tile max exceeds it by more than
      // 2^8, which bounds P by 256 (fine for bf16 and fp32); the final O / l
      // is unchanged. The branch is uniform per wave.
      const float m_tile = mx * a.scale_log2;
      const bool raise = m_tile > m_run + 8.f;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = fmaxf(m_run, m_tile);
        // 0 on a lane's first visible tile; 1 while a lane has seen no key
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DN; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

      bf16x8 pb[4];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(fmaf(s[n][r], a.scale_log2, -m_use));
          l_run += p;
          pb[2 * n + (r >> 3)][r & 7] = static_cast<__bf16>(p);
        }

      // O^T[d][q] += V^T[d][key] P^T[key][q] over 16-key chunks tc
      const int G16 = lane >> 4, s16 = lane & 15;
#pragma unroll
      for (int tc = 0; tc < 4; ++tc) {
        const int vrow = 16 * tc + 4 * (G16 >> 1) + (s16 >> 2);
#pragma unroll
        for (int d = 0; d < DN; ++d) {
          const int vbyte = 2 * (32 * d + 16 * (G16 & 1) + 4 * (s16 & 3));
          const i16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow, vbyte)));
          const i16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow + 8, vbyte)));
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[d] = mfma32x32x16(__builtin_bit_cast(bf16x8, both), pb[tc], o[d]);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = (m + log2 l) * ln 2
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
  const int qi = q0 + l32;
  uint16_t* orow = a.out + (bh * a.M + qi) * C;
#pragma unroll
  for (int d = 0; d < DN; ++d)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int dc = 32 * d + 8 * g4 + 4 * hh;
      u32x2 w;
      w[0] = (uint32_t)f32_to_bf16(o[d][4 * g4 + 0] * inv) |
             ((uint32_t)f32_to_bf16(o[d][4 * g4 + 1] * inv) << 16);
      w[1] = (uint32_t)f32_to_bf16(o[d][4 * g4 + 2] * inv) |
             ((uint32_t)f32_to_bf16(o[d][4 * g4 + 3] * inv) << 16);
      *reinterpret_cast<u32x2*>(orow + dc) = w;
    }
  if (a.lse && hh == 0) a.lse[bh * a.M + qi] = (m_run + log2f(l_tot)) * kLn2;
}

// ------------------------------------------------------------------ fp32 path

struct AttnArgsF32 {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  float* out;
  float* lse;
  int B, Hq, Hkv, M, NB, block, causal;
  float scale_log2;
};

template <int C>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnArgsF32 a) {
  const int qi = blockIdx.x * 64 + threadIdx.x;   // M is a multiple of 64
  const int h = blockIdx.y % a.Hq;
  const int b = blockIdx.y / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const size_t bh = (size_t)b * a.Hq + h, bg = (size_t)b * a.Hkv + g;
  const float* qrow = a.q + (bh * a.M + qi) * C;
  const float* kh = a.k + bg * a.M * C;
  const float* vh = a.v + bg * a.M * C;
  const int I = qi / a.block;
  float qv[C], acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) { qv[c] = qrow[c]; acc[c] = 0.f; }
  float m = -INFINITY, l = 0.f;
  int cnt;
  const int32_t* idx = nullptr;
  if (a.kv_idx) {
    cnt = a.kv_cnt[bh * a.NB + I];
    cnt = cnt < 0 ? 0 : (cnt > a.NB ? a.NB : cnt);
    idx = a.kv_idx + (bh * a.NB + I) * a.NB;
  } else {
    cnt = a.causal ? I + 1 : a.NB;
  }
  for (int t = 0; t < cnt; ++t) {
    int jb = idx ? idx[t] : t;
    jb = jb < 0 ? 0 : (jb >= a.NB ? a.NB - 1 : jb);
    for (int kj = jb * a.block; kj < (jb + 1) * a.block; ++kj) {
      if (a.causal && kj > qi) break;
      const float* kr = kh + (size_t)kj * C;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) s = fmaf(qv[c], kr[c], s);
      s *= a.scale_log2;
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float p = exp2f(s - mn);
      l = l * alpha + p;
      const float* vr = vh + (size_t)kj * C;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = fmaf(p, vr[c], acc[c] * alpha);
      m = mn;
    }
  }
  const float inv = 1.f / l;
  float* orow = a.out + (bh * a.M + qi) * C;
#pragma unroll
  for (int c = 0; c < C; ++c) orow[c] = acc[c] * inv;
  if (a.lse) a.lse[bh * a.M + qi] = (m + log2f(l)) * kLn2;
}

// ------------------------------------------------------------------ launchers

template <int C, int BLK>
static hipError_t launch_bf16_cb(const Shape& s, const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)s.B * s.Hq * s.NB())), block(BLK * 2);
  const bool sp = a.kv_idx != nullptr;
  if (s.causal && sp)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<C, BLK, true, true>), grid, block, 0, st, a);
  else if (s.causal)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<C, BLK, true, false>), grid, block, 0, st, a);
  else if (sp)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<C, BLK, false, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<C, BLK, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const Shape& s, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                            float sm_scale, uint16_t* out, float* lse, hipStream_t st) {
  AttnArgs a{q, k, v, kv_idx, kv_cnt, out, lse, s.B, s.Hq, s.Hkv, s.M, s.NB(), sm_scale * kLog2e};
  if (s.C == 128 && s.block == 128) return launch_bf16_cb<128, 128>(s, a, st);
  if (s.C == 128 && s.block == 64) return launch_bf16_cb<128, 64>(s, a, st);
  if (s.C == 64 && s.block == 128) return launch_bf16_cb<64, 128>(s, a, st);
  if (s.C == 64 && s.block == 64) return launch_bf16_cb<64, 64>(s, a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_f32(const Shape& s, const float* q, const float* k, const float* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, float sm_scale,
                           float* out, float* lse, hipStream_t st) {
  AttnArgsF32 a{q, k, v, kv_idx, kv_cnt, out, lse, s.B, s.Hq, s.Hkv, s.M, s.NB(), s.block,
                s.causal, sm_scale * kLog2e};
  dim3 grid(s.M / 64, s.B * s.Hq);
  if (s.C == 64)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<64>), grid, dim3(64), 0, st, a);
  else if (s.C == 128)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<128>), grid, dim3(64), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace xattn
