// Stage 4: block-sparse (and dense) attention forward.
//
// Semantics ("XAttention: Block Sparse Attention with Antidiagonal Scoring",
// arXiv abstract: block-sparse attention computes only on the important
// blocks): for query i of block I, exact softmax attention over the keys of
// the listed key blocks, restricted to keys <= i when causal. The queries may
// be the last Mq of Mk tokens (query i is then at position Mk - Mq + i), and
// either length may end in a partial block: keys past the end are masked,
// query rows past the end are not written.
//
// bf16 path (gfx950 MFMA):
//  * a work item is one (b, h, I) query block (or a pair, see the modes);
//    BLK/32 waves, each wave owns 32 query rows whose Q fragments stay in VGPRs
//    for the whole row. Dense launches one workgroup per item; sparse runs
//    persistent workgroups that pull items from per-XCD queues;
//  * key blocks are consumed in 64-key sub-tiles: K and V rows are fetched from
//    HBM into registers one sub-tile ahead (two in the 8-wave modes) and
//    written to a double-buffered LDS tile, so one barrier per sub-tile orders
//    reuse;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 puts one query per lane, so the
//    row max/sum is an in-lane reduction plus one exchange between the wave
//    halves; P^T stays in registers and feeds O^T += V^T P^T directly, with V^T
//    fragments taken from row-major LDS by the transposing LDS read;
//  * online softmax in the log2 domain in fp32; P rounded to bf16 for the PV
//    product; O normalised once at the end and rounded to bf16 (RNE).
// f32 path: one thread per query row with fp32 FMA (small problems only).
#include "common.h"
#include "kernels.h"

// Sparse workgroups pair neighbouring rows of a head (one K/V tile load serves
// both rows of the union list) once a head has at least this many query blocks;
// shorter rows keep one row per workgroup.
#ifndef XATTN_SPARSE_PAIR_ROWS_MIN_NB
#define XATTN_SPARSE_PAIR_ROWS_MIN_NB 1024
#endif
// The same threshold for non-causal heads: every row draws on the whole key
// range, so neighbouring rows' lists overlap more (7% off bsa_fwd on a
// non-causal layer of 600 query blocks at 48% density; pairing the 256 rows of
// a causal layer at 1.6% density was 20% slower).
#ifndef XATTN_SPARSE_PAIR_ROWS_MIN_NB_NC
#define XATTN_SPARSE_PAIR_ROWS_MIN_NB_NC 512
#endif
// 1: dense workgroups of an odd GQA group (no sibling pair) take two
// neighbouring rows of one head, which read the same key blocks (all of them,
// or all but the later row's diagonal); 0: one row per workgroup
#ifndef XATTN_DENSE_PAIR_ROWS
#define XATTN_DENSE_PAIR_ROWS 1
#endif
// 1: the sparse workgroups of one KV group share an XCD; 0: spread them
#ifndef XATTN_SPARSE_GROUP_ON_XCD
#define XATTN_SPARSE_GROUP_ON_XCD 1
#endif
// 1: sparse items are ordered KV group by KV group (all rows of one group
// before the next), so the device works on one KV head's K/V at a time and the
// infinity cache keeps it; 0: row by row across all heads
#ifndef XATTN_SPARSE_GROUP_MAJOR
#define XATTN_SPARSE_GROUP_MAJOR 1
#endif
// the same order for dense launches (1), or row by row across all heads (0)
#ifndef XATTN_DENSE_GROUP_MAJOR
#define XATTN_DENSE_GROUP_MAJOR 1
#endif
// consecutive items (rows, with GROUP_MAJOR) handed to one XCD together
#ifndef XATTN_SPARSE_ROWS_PER_CHUNK
#define XATTN_SPARSE_ROWS_PER_CHUNK 1
#endif
// log2 of the neighbouring query-block rows a KV group keeps on one XCD in the
// sparse kernel (see xcd_map)
#ifndef XATTN_SPARSE_ROWS_PER_XCD_LOG2
#define XATTN_SPARSE_ROWS_PER_XCD_LOG2 0
#endif

// k-steps of K fragments read from LDS ahead of their MFMAs
#ifndef XATTN_KBATCH
#define XATTN_KBATCH 2
#endif
// 1: the 8-wave modes run the software-pipelined loop (K/V sub-tiles DMA'd
// into a four-slot LDS ring; the S MFMAs of sub-tile t+1 interleaved with the
// exponentials of sub-tile t, and the row maximum of t+1 with the PV MFMAs of
// t); 0: the register-staged loop with one barrier per sub-tile
#ifndef XATTN_ATTN_PIPE
#define XATTN_ATTN_PIPE 1
#endif
// 1: the pipelined loop issues each sub-tile's DMA pieces spread over the S
// MFMAs of the common path (one piece every four MFMAs) instead of all at once
// after the barrier; 0: all at once
#ifndef XATTN_DMA_SPREAD
#define XATTN_DMA_SPREAD 1
#endif
// 1: in the pipelined step a wave raises its priority (s_setprio) over the
// S(t+1) MFMAs with tile t's exponentials, so the arbiter favours the phase
// that feeds both the matrix unit and the exponentials over the other wave's
// PV phase. Measured 1.5% off the 128K and 256K steps (A/B on one box);
// raising it over the PV phase instead was 0.5% slower, and two levels (S
// phase above PV phase) the same as one.
#ifndef XATTN_ATTN_PRIO
#define XATTN_ATTN_PRIO 1
#endif
// 1: the epilogue stages each wave's output rows in LDS and stores whole rows;
// 0: each lane stores its pieces of 32 rows straight from the accumulators
#ifndef XATTN_O_STAGE
#define XATTN_O_STAGE 1
#endif
// 1: Q is loaded and O stored with the non-temporal hint (read once and
// written once, so they need not displace K/V from the caches)
#ifndef XATTN_NT_QO
#define XATTN_NT_QO 0
#endif

namespace xattn {

XATTN_DEBUG_COUNTERS

// Queries are the last Mq of Mk tokens: query block I is key block I + qoff.
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_idx;  // nullptr: dense
  const int32_t* kv_cnt;
  uint16_t* out;
  float* lse;
  uint32_t* queue;   // sparse: kQueueWords zeroed words (per-XCD item counters)
  int B, Hq, Hkv, Mq, Mk, NBq, NBk, qoff;
  float scale_log2;  // sm_scale * log2(e)
};

constexpr uint32_t kNoItem = 0xffffffffu;

template <int C>
struct AttnLds {
  static constexpr int KT = 64;               // keys per sub-tile
  static constexpr int ROW_B = 2 * C;         // bytes per K or V row (no padding)
  static constexpr int TILE_B = KT * ROW_B;   // bytes per K (or V) sub-tile
  static constexpr int ROWS_PER_256 = 256 / ROW_B;
  static constexpr int IDX_MAX = 4096;        // block-index row cached as uint16
  // K and V double buffers and the block list (u16); with several heads per
  // workgroup also per-entry head bits and a per-block flag scratch (u8 each)
  static constexpr int bytes(int hpw) { return 2 * 2 * TILE_B + 2 * IDX_MAX + (hpw > 1 ? 2 * IDX_MAX : 0); }
  // the pipelined loop: a ring of RING sub-tile slots (K then V), then the lists
  static constexpr int RING = 4;
  static constexpr int bytes_pipe(int hpw) { return RING * 2 * TILE_B + 2 * IDX_MAX + (hpw > 1 ? 2 * IDX_MAX : 0); }
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

// Workgroup modes: what the 4 or 8 waves of one workgroup cover.
//   SINGLE    one (head, query block); 4 waves.
//   SIBLINGS  two GQA sibling heads, same query block; 8 waves. Every K/V tile
//             load serves both heads (dense attention, identical block lists).
//   ROWS      one head, two neighbouring query blocks 2p and 2p+1; 8 waves over
//             the union of the two block lists. Neighbouring rows of a head keep
//             similar numbers of largely the same blocks, so the shared loads
//             are rarely wasted and neither half idles for long (sparse; and
//             dense when the GQA group is odd, where both rows read the same
//             blocks, the earlier row skipping the later one's diagonal).
// The 8-wave modes hold two sub-tiles in flight (registers), SINGLE one.
enum { MODE_SINGLE = 0, MODE_SIBLINGS = 1, MODE_ROWS = 2 };

// Per-mode constants: SLOTS (head, row) pairs per workgroup of NT threads.
template <int MODE>
struct AttnMode {
  static constexpr int SLOTS = MODE == MODE_SINGLE ? 1 : 2;
};

// Work items of a launch: one per workgroup-sized unit of (b, g, pw, P), where
// pw numbers the workgroups of one KV group and P the query rows (row pairs).
struct AttnItems {
  uint32_t GW, NP, n;
  __device__ AttnItems(const AttnArgs& a, int MODE) {
    const uint32_t G = a.Hq / a.Hkv;
    NP = MODE == MODE_ROWS ? (a.NBq + 1) / 2 : a.NBq;
    GW = MODE == MODE_SIBLINGS ? G / 2 : G;
    n = (uint32_t)a.B * a.Hkv * GW * NP;
  }
};

// One work item: all rows of the slots it covers, from the block list to the
// normalised output. Starts and ends with every wave of the workgroup past a
// barrier after its last LDS read, so consecutive items may reuse the LDS.
// KTAIL: the last key block is partial (Mk % BLK != 0): key rows past the end
// are clamped on load and masked out of the softmax.
// RPW: query rows per wave, 32 or 64. With 64 a wave holds two 32-row q-tiles,
// and every K and V^T fragment read from LDS feeds two MFMAs (half the LDS
// traffic per FLOP); the wave then needs more than 256 registers, so it runs
// alone on its SIMD.
template <int C, int BLK, bool CAUSAL, bool SPARSE, int MODE, bool KTAIL, int RPW>
__device__ __forceinline__ void attn_item(const AttnArgs& a, const uint32_t item,
                                          unsigned char* smem, int* scan_s) {
  using L = AttnLds<C>;
  constexpr int SLOTS = AttnMode<MODE>::SLOTS;
  constexpr int WPH = BLK / RPW;              // waves per slot
  constexpr int QT = RPW / 32;                // 32-row q-tiles per wave
  constexpr int NT = 64 * WPH * SLOTS;        // threads
  constexpr int SUB = BLK / L::KT;            // sub-tiles per key block
  constexpr int CHUNKS = L::KT * C / 8;       // 16-byte chunks per K (or V) sub-tile
  constexpr int PER_T = CHUNKS / NT;
  constexpr int KK = C / 16;                  // MFMA k-steps over the head dim
  constexpr int DN = C / 32;                  // 32-wide d tiles of O^T
  constexpr int DEPTH = SLOTS == 2 && RPW == 32 ? 2 : 1;  // sub-tiles in flight in registers
  static_assert(CHUNKS % NT == 0, "tile load must divide evenly");

  // the pipelined loop serves the 8-wave modes
  constexpr bool PIPE = XATTN_ATTN_PIPE != 0 && SLOTS == 2 && RPW == 32;
  constexpr int TILES_B = (PIPE ? L::RING : 2) * 2 * L::TILE_B;  // bytes of K/V tiles
  unsigned char* Ks = smem;                      // [2][KT rows][2C bytes], swizzled
  unsigned char* Vs = smem + 2 * L::TILE_B;      // [2][KT rows][2C bytes], swizzled
  // block list (union over the workgroup's slots) and, per entry, a bit per
  // slot that selected it
  uint16_t* idx_s = reinterpret_cast<uint16_t*>(smem + TILES_B);
  uint8_t* memb_s = smem + TILES_B + 2 * L::IDX_MAX;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int hs = wave / WPH;                   // slot of this wave
  const int slice = wave % WPH;                // RPW-row slice of the query block

  // ---- decode the item: heavy query rows (large P) come first in item order
  // (within each KV group when the order is KV-group-major)
  const int G = a.Hq / a.Hkv;
  const AttnItems its(a, MODE);
  const int NP = (int)its.NP;
  const int GW = (int)its.GW;
  const int pw = item % GW;
  uint32_t rest = item / GW;
  int g, b, P;
  constexpr bool group_major = SPARSE ? XATTN_SPARSE_GROUP_MAJOR != 0 : XATTN_DENSE_GROUP_MAJOR != 0;
  if (group_major) {
    // KV-group-major: every row of one KV group before the next group
    P = NP - 1 - (int)(rest % NP);
    rest /= NP;
    b = rest % a.B;
    g = rest / a.B;
  } else {
    g = rest % a.Hkv;
    rest /= a.Hkv;
    b = rest % a.B;
    P = NP - 1 - (int)(rest / a.B);
  }
  // slot s covers head slot_h(s) and query block slot_I(s)
  auto slot_h = [&](int s2) { return g * G + (MODE == MODE_SIBLINGS ? 2 * pw + s2 : pw); };
  auto slot_I = [&](int s2) { return MODE == MODE_ROWS ? 2 * P + s2 : P; };
  const int h = slot_h(hs);                    // this wave's head
  const int I = slot_I(hs);                    // this wave's query block
  XATTN_DCHECK(b < a.B && g < a.Hkv && h < a.Hq && P < NP && I <= a.NBq, DBG_ATTN_ITEM);
  const bool live = I < a.NBq;                 // the odd row count leaves a half-empty pair

  const size_t bh = (size_t)b * a.Hq + h;
  const size_t bg = (size_t)b * a.Hkv + g;
  const uint16_t* qh = a.q + bh * a.Mq * C;
  const uint16_t* kh = a.k + bg * a.Mk * C;
  const uint16_t* vh = a.v + bg * a.Mk * C;
  const int NBk = a.NBk;

  int cnt;  // entries in the (union) block list
  if constexpr (SPARSE) {
    // cache the row's block list in LDS once, so no dependent global load sits
    // in front of each tile fetch; out-of-range entries are clamped
    if constexpr (SLOTS == 1) {
      cnt = a.kv_cnt[bh * a.NBq + I];
      cnt = cnt < 0 ? 0 : (cnt > NBk ? NBk : cnt);
      const int32_t* idx = a.kv_idx + (bh * a.NBq + I) * NBk;
      for (int t = tid; t < cnt; t += NT) {
        int jb = idx[t];
        jb = jb < 0 ? 0 : (jb >= NBk ? NBk - 1 : jb);
        idx_s[t] = (uint16_t)jb;
      }
    } else {
      // union of the slots' ascending lists: per-block slot bits, then an
      // ascending compaction
      uint8_t* flag = memb_s + L::IDX_MAX;     // [NB] scratch bits
      for (int j = tid; j < NBk; j += NT) flag[j] = 0;
      __syncthreads();
      for (int s2 = 0; s2 < SLOTS; ++s2) {
        if (slot_I(s2) >= a.NBq) continue;
        const size_t row = ((size_t)b * a.Hq + slot_h(s2)) * a.NBq + slot_I(s2);
        int c2 = a.kv_cnt[row];
        c2 = c2 < 0 ? 0 : (c2 > NBk ? NBk : c2);
        const int32_t* idx = a.kv_idx + row * NBk;
        for (int t = tid; t < c2; t += NT) {
          int jb = idx[t];
          jb = jb < 0 ? 0 : (jb >= NBk ? NBk - 1 : jb);
          // slots write distinct bits; byte-wide OR through a word atomic
          __hip_atomic_fetch_or(reinterpret_cast<unsigned*>(flag + (jb & ~3)),
                                (unsigned)(1u << s2) << (8 * (jb & 3)), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      __syncthreads();
      const int per = (NBk + NT - 1) / NT;
      // redefined here (empty asm) so that values derived from the thread
      // index alone are not hoisted out of the item loop and kept live
      // across the key loop
      int tidu = tid;
      asm volatile("" : "+v"(tidu));
      const int j0 = tidu * per, j1 = min(j0 + per, NBk);
      int mine = 0;
      for (int j = j0; j < j1; ++j) mine += flag[j] != 0;
      int incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (lane == 63) scan_s[wave] = incl;
      __syncthreads();
      int pos = incl - mine;
      int total = 0;
      for (int w2 = 0; w2 < NT / 64; ++w2) {
        if (w2 < wave) pos += scan_s[w2];
        total += scan_s[w2];
      }
      for (int j = j0; j < j1; ++j) {
        const uint8_t f = flag[j];
        if (f) {
          idx_s[pos] = (uint16_t)j;
          memb_s[pos] = f;
          ++pos;
        }
      }
      cnt = total;
    }
  } else {
    // dense: every candidate of the workgroup's (latest) row
    const int Imax = slot_I(SLOTS - 1) < a.NBq ? slot_I(SLOTS - 1) : slot_I(0);
    cnt = CAUSAL ? Imax + a.qoff + 1 : NBk;
  }
  const int n_sub = cnt * SUB;

  // ---- Q fragments (B operand of S^T = K Q^T): Q[q0 + 32y + l32][16kk + 8hh .. +7]
  const int q0 = I * BLK + slice * RPW;          // first query row of this wave
  const int qa0 = q0 + a.qoff * BLK;             // its position in the key sequence
  bf16x8 qf[QT][KK];
#pragma unroll
  for (int y = 0; y < QT; ++y) {
    // rows past the end (a partial last block, or a dead slot) read the last
    // query row instead; their outputs are never stored
    const uint16_t* qrow = qh + (size_t)min(live ? q0 + 32 * y + l32 : l32, a.Mq - 1) * C + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4* src = reinterpret_cast<const u32x4*>(qrow + 16 * kk);
      qf[y][kk] = __builtin_bit_cast(bf16x8, XATTN_NT_QO ? __builtin_nontemporal_load(src) : *src);
    }
  }
  // Complete the Q loads here. Otherwise the compiler may leave them in flight
  // into the key loop, and since the load counter is in-order, every first use
  // of qf per sub-tile would also wait for the next tile's prefetch issued just
  // before it, serialising the prefetch with the compute.
#pragma unroll
  for (int y = 0; y < QT; ++y)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qf[y][kk]));

  f32x16 o[QT][DN];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int y = 0; y < QT; ++y) {
#pragma unroll
    for (int d = 0; d < DN; ++d) o[y][d] = f32x16{};
    m_run[y] = -INFINITY;
    l_run[y] = 0.f;
  }

  // List entry of sub-tile t, packed as (key block | slot bits << 16). Entries
  // are held 64 at a time, one per lane of a VGPR window, and picked out with
  // v_readlane: no LDS round trip sits in front of a tile fetch or its MFMAs.
  // The loops ask for entries in increasing order, t + 2 or t + 3 ahead.
  uint32_t ewin = 0;
  int ebase = -64;
  auto entry = [&](int t) -> uint32_t {
    const int e = min(t / SUB, cnt > 0 ? cnt - 1 : 0);
    if constexpr (!SPARSE) {
      return (uint32_t)e;
    } else {
      if (e >= ebase + 64) {  // uniform: refresh the window
        ebase = e & ~63;
        const int el = min(ebase + lane, cnt > 0 ? cnt - 1 : 0);
        XATTN_DCHECK(el < L::IDX_MAX, DBG_ATTN_LDS);
        ewin = SLOTS > 1 ? (uint32_t)idx_s[el] | ((uint32_t)memb_s[el] << 16) : (uint32_t)idx_s[el];
      }
      return (uint32_t)__builtin_amdgcn_readlane((int)ewin, e - ebase);
    }
  };
  auto key_start = [&](uint32_t en, int t) -> int {
    return (int)(en & 0xFFFFu) * BLK + (t % SUB) * L::KT;
  };
  auto mine_tile = [&](uint32_t en) -> bool {
    if constexpr (SPARSE && SLOTS > 1) return (en >> (16 + hs)) & 1u;
    return live;
  };

  // this thread's 16-byte K and V chunks of a sub-tile
  struct Stage {
    u32x4 k[PER_T];
    u32x4 v[PER_T];
  };
  auto load_tile = [&](int k0, Stage& r) {
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const int c = tid + p * NT;
      const int row = c / (C / 8), col = (c % (C / 8)) * 8;
      // keys past the end (a partial last block) load the last key; they are
      // masked out of the softmax
      const size_t kr = KTAIL ? (size_t)min(k0 + row, a.Mk - 1) : (size_t)(k0 + row);
      XATTN_DCHECK(k0 >= 0 && kr < (size_t)a.Mk, DBG_ATTN_KV_ROW);
      r.k[p] = *reinterpret_cast<const u32x4*>(kh + kr * C + col);
      r.v[p] = *reinterpret_cast<const u32x4*>(vh + kr * C + col);
    }
  };
  auto store_tile = [&](int buf, const Stage& r) {
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const int c = tid + p * NT;
      const int row = c / (C / 8), chunk = c % (C / 8);
      *reinterpret_cast<u32x4*>(Ks + buf * L::TILE_B + L::k_off(row, chunk)) = r.k[p];
      *reinterpret_cast<u32x4*>(Vs + buf * L::TILE_B + L::v_off(row, 16 * chunk)) = r.v[p];
    }
  };

  // one sub-tile of online-softmax attention for this wave
  auto compute = [&](int k0, bool mine, int buf) {
    if (CAUSAL && (k0 > qa0 + RPW - 1)) return; // whole sub-tile above this wave's rows
    if (KTAIL && k0 >= a.Mk) return;            // whole sub-tile past the last key
    if (!mine) return;                          // selected only by the other head
    const unsigned char* Kb = Ks + buf * L::TILE_B;
    const unsigned char* Vb = Vs + buf * L::TILE_B;
    // S^T tiles (y, n): keys k0 + 32n + [8(r/4) + 4hh + r%4], query q0 + 32y + l32
    f32x16 sacc[QT][2];
#pragma unroll
    for (int y = 0; y < QT; ++y) sacc[y][0] = sacc[y][1] = f32x16{};
    // K fragments are read XATTN_KBATCH k-steps at a time ahead of their MFMAs
    constexpr int KB = XATTN_KBATCH < KK ? XATTN_KBATCH : KK;
#pragma unroll
    for (int k0b = 0; k0b < KK; k0b += KB) {
      bf16x8 ka[KB][2];
#pragma unroll
      for (int u = 0; u < KB; ++u)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          ka[u][n] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(Kb + L::k_off(32 * n + l32, 2 * (k0b + u) + hh)));
      // keep the batch's reads ahead of its MFMAs (the scheduler would sink
      // each read next to its use and expose the LDS latency per pair)
      if (KB > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < KB; ++u)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int y = 0; y < QT; ++y) sacc[y][n] = mfma32x32x16(ka[u][n], qf[y][k0b + u], sacc[y][n]);
    }
    bf16x8 pb[QT][4];
#pragma unroll
    for (int y = 0; y < QT; ++y) {
      const int qay = qa0 + 32 * y;  // first query of q-tile y (key-sequence position)
      if ((CAUSAL && (k0 + L::KT - 1 > qay)) || (KTAIL && k0 + L::KT > a.Mk)) {
        const int qi = qay + l32;
        const int kmax = !KTAIL ? qi : (CAUSAL ? min(qi, a.Mk - 1) : a.Mk - 1);  // last visible key
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * n + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key > kmax) sacc[y][n][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[y][n][r]);
      mx = halves_max(mx);
      // Lazy rescaling (exact): O and l share the reference m_run, so the
      // reference may lag the true running max as long as 2^(s*c - m_run) stays
      // small. It is raised only when the tile max exceeds it by more than 8
      // (in log2 units), which bounds P by 256 (fine for bf16 and fp32); the
      // final O / l is unchanged. The branch is uniform per wave.
      const float m_tile = mx * a.scale_log2;
      const bool raise = m_tile > m_run[y] + 8.f;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = fmaxf(m_run[y], m_tile);
        // 0 on a lane's first visible tile; 1 while a lane has seen no key
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[y] - m_new);
        m_run[y] = m_new;
        l_run[y] *= alpha;
#pragma unroll
        for (int d = 0; d < DN; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[y][d][r] *= alpha;
      }
      const float m_use = (m_run[y] == -INFINITY) ? 0.f : m_run[y];
      // row sums in four partial sums, in the pipelined loop's order (the two
      // loops then give bitwise the same output)
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(sacc[y][n][r], a.scale_log2, -m_use));
          ls[r & 3] += pr;
          pb[y][2 * n + (r >> 3)][r & 7] = static_cast<__bf16>(pr);
        }
      l_run[y] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }

    // O^T[d][q] += V^T[d][key] P^T[key][q] over 16-key chunks tc
    const int G16 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int tc = 0; tc < 4; ++tc) {
#pragma unroll
      for (int d = 0; d < DN; ++d) {
        const int vrow = 16 * tc + 4 * (G16 >> 1) + (s16 >> 2);
        const int vbyte = 2 * (32 * d + 16 * (G16 & 1) + 4 * (s16 & 3));
        const i16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow, vbyte)));
        const i16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow + 8, vbyte)));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int y = 0; y < QT; ++y) o[y][d] = mfma32x32x16(vf, pb[y][tc], o[y][d]);
      }
    }
  };

  if constexpr (PIPE) {
    // ---- software-pipelined loop over the sub-tiles of the block list.
    // K/V sub-tiles reach LDS by DMA (no staging registers) into a ring of
    // four slots: tile t sits in slot t % 4. Iteration t, after one barrier:
    //   * DMA of tile t+3 into the slot of tile t-1 (every wave is past it);
    //   * lazy rescale for tile t (rare);
    //   * S(t+1) = K(t+1) Q^T on the matrix cores, interleaved with the
    //     exponentials of tile t (P(t), the row sums);
    //   * O += V(t)^T P(t) on the matrix cores, interleaved with the masks and
    //     the row maximum of tile t+1.
    // So the softmax VALU work of a wave overlaps its own MFMAs, and the
    // loads of tile t+3 have two iterations to land.
    constexpr int BLKS = L::TILE_B / 1024;           // 1 KiB DMA blocks per K (or V) sub-tile
    constexpr int BPW = BLKS / (NT / 64);            // ... per wave
    static_assert(BPW >= 1 && BPW * (NT / 64) == BLKS, "DMA blocks must cover the sub-tile");
    constexpr int DPT = 2 * BPW;                     // DMA loads per wave per sub-tile
    constexpr int RPB = 1024 / L::ROW_B;             // key rows per DMA block
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // lane's 16 bytes of each of its DMA blocks: the tile row, and the byte
    // offset in that row of the global piece that belongs at its LDS position
    // under the K and V swizzles of AttnLds
    // (without a key tail: byte offsets from the sub-tile's first row; with
    // one: the row and the in-row offsets, clamped per sub-tile)
    uint32_t kcb[BPW], vcb[BPW];
    int lrow[KTAIL ? BPW : 1];
#pragma unroll
    for (int b2 = 0; b2 < BPW; ++b2) {
      const int row = (wv * BPW + b2) * RPB + (16 * lane) / L::ROW_B;
      const int pos = (16 * lane) % L::ROW_B;
      const int sw = row / L::ROWS_PER_256;
      const uint32_t kc = 16 * ((pos / 16) ^ (sw % (C / 8)));
      const uint32_t vc = pos ^ (64 * (sw % (C / 32)));
      if constexpr (KTAIL) {
        lrow[b2] = row;
        kcb[b2] = kc;
        vcb[b2] = vc;
      } else {
        kcb[b2] = (uint32_t)row * (2 * C) + kc;
        vcb[b2] = (uint32_t)row * (2 * C) + vc;
      }
    }
    auto slot_k = [&](int slot) { return smem + slot * 2 * L::TILE_B; };
    auto slot_v = [&](int slot) { return smem + slot * 2 * L::TILE_B + L::TILE_B; };
    // piece p of a sub-tile's DMA: block p / 2 of this wave, K (p even) or V
    constexpr int NPIECE = 2 * BPW;
    auto dma_piece = [&](int k0, int slot, int p) {
      XATTN_DCHECK(KTAIL || (k0 >= 0 && k0 + L::KT <= a.Mk), DBG_ATTN_KV_ROW);
      XATTN_DCHECK(slot >= 0 && slot < L::RING, DBG_ATTN_LDS);
      const int b2 = p >> 1;
      const bool isv = p & 1;
      const uint32_t lds = lds_addr_u((isv ? slot_v(slot) : slot_k(slot)) + (wv * BPW + b2) * 1024);
      const uint16_t* base = isv ? vh : kh;
      const uint32_t cb = isv ? vcb[b2] : kcb[b2];
      if constexpr (KTAIL) {
        // keys past the end load the last key; they are masked out of the softmax
        const uint32_t r = (uint32_t)min(k0 + lrow[b2], a.Mk - 1) * (2 * C);
        dma16(uniform_ptr(base), r + cb, lds);
      } else {
        dma16(uniform_ptr(base + (size_t)k0 * C), cb, lds);
      }
    };
    auto dma_tile = [&](int k0, int slot) {
#pragma unroll
      for (int p2 = 0; p2 < NPIECE; ++p2) dma_piece(k0, slot, p2);
    };
    // is sub-tile t (entry en) computed by this wave: selected by its slot,
    // not wholly above its rows (causal), not wholly past the last key
    auto active = [&](uint32_t en, int t) -> bool {
      const int k0 = key_start(en, t);
      if (CAUSAL && k0 > qa0 + RPW - 1) return false;
      if (KTAIL && k0 >= a.Mk) return false;
      return mine_tile(en);
    };
    // S^T tiles (n): keys k0 + 32n + [8(r/4) + 4hh + r%4], query q0 + l32
    auto s_mma = [&](int slot, f32x16 (&acc)[2]) {
      const unsigned char* Kb = slot_k(slot);
      acc[0] = acc[1] = f32x16{};
      constexpr int KB = XATTN_KBATCH < KK ? XATTN_KBATCH : KK;
#pragma unroll
      for (int k0b = 0; k0b < KK; k0b += KB) {
        bf16x8 ka[KB][2];
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
          for (int n = 0; n < 2; ++n)
            ka[u][n] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(Kb + L::k_off(32 * n + l32, 2 * (k0b + u) + hh)));
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
          for (int n = 0; n < 2; ++n) acc[n] = mfma32x32x16(ka[u][n], qf[0][k0b + u], acc[n]);
      }
    };
    // masks (causal diagonal, key tail) and the row maximum, log2 units
    auto mask_max = [&](int k0, f32x16 (&acc)[2]) -> float {
      if ((CAUSAL && (k0 + L::KT - 1 > qa0)) || (KTAIL && k0 + L::KT > a.Mk)) {
        const int qi = qa0 + l32;
        const int kmax = !KTAIL ? qi : (CAUSAL ? min(qi, a.Mk - 1) : a.Mk - 1);  // last visible key
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * n + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key > kmax) acc[n][r] = -INFINITY;
          }
      }
      float m0 = fmaxf(acc[0][0], acc[1][0]), m1 = fmaxf(acc[0][1], acc[1][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        m0 = fmaxf(m0, fmaxf(acc[0][r], acc[1][r]));
        m1 = fmaxf(m1, fmaxf(acc[0][r + 1], acc[1][r + 1]));
      }
      return halves_max(fmaxf(m0, m1)) * a.scale_log2;
    };
    bf16x8 pb[4];
    // P = 2^(s*c - m) rounded to bf16, row sums in fp32
    auto exp_tile = [&](f32x16 (&acc)[2], float m_use) {
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(acc[n][r], a.scale_log2, -m_use));
          ls[r & 3] += pr;
          pb[2 * n + (r >> 3)][r & 7] = static_cast<__bf16>(pr);
        }
      l_run[0] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    // O^T[d][q] += V^T[d][key] P^T[key][q] over 16-key chunks tc
    auto pv = [&](int slot) {
      const unsigned char* Vb = slot_v(slot);
      const int G16 = lane >> 4, s16 = lane & 15;
#pragma unroll
      for (int tc = 0; tc < 4; ++tc) {
#pragma unroll
        for (int d = 0; d < DN; ++d) {
          const int vrow = 16 * tc + 4 * (G16 >> 1) + (s16 >> 2);
          const int vbyte = 2 * (32 * d + 16 * (G16 & 1) + 4 * (s16 & 3));
          const i16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow, vbyte)));
          const i16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow + 8, vbyte)));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[0][d] = mfma32x32x16(vf, pb[tc], o[0][d]);
        }
      }
    };
    // lazy exact rescaling (as in the register-staged loop): the reference
    // m_run is raised only when a tile's maximum exceeds it by more than 8
    auto rescale_if_needed = [&](float m_tile) {
      if (__builtin_amdgcn_ballot_w64(m_tile > m_run[0] + 8.f) != 0) {
        const float m_new = fmaxf(m_run[0], m_tile);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[0] - m_new);
        m_run[0] = m_new;
        l_run[0] *= alpha;
#pragma unroll
        for (int d = 0; d < DN; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[0][d][r] *= alpha;
      }
    };

    // masks (causal diagonal, key tail) needed on sub-tile t with first key k0
    auto needs_mask = [&](int k0) -> bool {
      return (CAUSAL && (k0 + L::KT - 1 > qa0)) || (KTAIL && k0 + L::KT > a.Mk);
    };
    // the row maximum of an unmasked sub-tile (log2 units)
    auto row_max = [&](f32x16 (&acc)[2]) -> float {
      float m0 = fmaxf(acc[0][0], acc[1][0]), m1 = fmaxf(acc[0][1], acc[1][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        m0 = fmaxf(m0, fmaxf(acc[0][r], acc[1][r]));
        m1 = fmaxf(m1, fmaxf(acc[0][r + 1], acc[1][r + 1]));
      }
      return halves_max(fmaxf(m0, m1)) * a.scale_log2;
    };

    // One pipelined sub-tile step for a wave that computes both tiles:
    //  phase A, NSA = 2 KK groups: a K fragment read (4 ahead), one S(t+1)
    //    MFMA, 32 / NSA exponentials of tile t (scaled logit, 2^x, row sum,
    //    bf16 pairs);
    //  phase B, NPV = 4 DN groups: two V^T fragment reads (4 MFMAs ahead), one
    //    PV(t) MFMA, and (from the second quarter on) a share of the running
    //    maximum of tile t+1.
    // Fences keep the groups in this order; within a group the compiler
    // schedules freely.
    constexpr int NSA = 2 * KK;
    constexpr int VPG = 32 / NSA;
    constexpr int NPV = 4 * DN;
    constexpr int MX0 = NPV / 4;  // first group that takes part of the maximum
    static_assert(NSA >= 4 && NPV >= 4 && 32 % NSA == 0, "pipeline shape");
    constexpr int DSTEP = NSA / NPIECE;  // S MFMAs per DMA piece
    static_assert(DSTEP >= 1 && DSTEP * NPIECE == NSA, "the DMA pieces are issued within the S MFMAs");
    float mx_run[2];
    auto full_step = [&](int kslot, int vslot, f32x16 (&cur)[2], f32x16 (&acc)[2], float m_use, int dk0,
                         int dslot) {
      const unsigned char* Kb = slot_k(kslot);
      const unsigned char* Vb = slot_v(vslot);
      auto read_k = [&](int g) {  // S MFMA g = 2 kk + n
        return __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Kb + L::k_off(32 * (g & 1) + l32, 2 * (g >> 1) + hh)));
      };
      const int G16 = lane >> 4, s16 = lane & 15;
      auto read_v = [&](int g) {  // PV MFMA g = DN tc + d
        const int tc = g / DN, d = g % DN;
        const int vrow = 16 * tc + 4 * (G16 >> 1) + (s16 >> 2);
        const int vbyte = 2 * (32 * d + 16 * (G16 & 1) + 4 * (s16 & 3));
        const i16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow, vbyte)));
        const i16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(Vb + L::v_off(vrow + 8, vbyte)));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      acc[0] = acc[1] = f32x16{};
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
      bf16x8 kf[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) kf[g] = read_k(g);
      __builtin_amdgcn_sched_barrier(0);
      if (XATTN_ATTN_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int g = 0; g < NSA; ++g) {
        const bf16x8 f = kf[g & 3];
        if (g + 4 < NSA) kf[g & 3] = read_k(g + 4);
        acc[g & 1] = mfma32x32x16(f, qf[0][g >> 1], acc[g & 1]);
        if (XATTN_DMA_SPREAD && g % DSTEP == (DSTEP > 1 ? 1 : 0)) dma_piece(dk0, dslot, g / DSTEP);
#pragma unroll
        for (int u = 0; u < VPG; ++u) {
          const int v = VPG * g + u, n = v >> 4, r = v & 15;
          const float pr = fast_exp2(fmaf(cur[n][r], a.scale_log2, -m_use));
          ls[r & 3] += pr;
          pb[2 * n + (r >> 3)][r & 7] = static_cast<__bf16>(pr);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (XATTN_ATTN_PRIO) __builtin_amdgcn_s_setprio(0);
      l_run[0] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
      bf16x8 vf[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) vf[g] = read_v(g);
      mx_run[0] = mx_run[1] = -INFINITY;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < NPV; ++g) {
        const bf16x8 f = vf[g & 3];
        if (g + 4 < NPV) vf[g & 3] = read_v(g + 4);
        o[0][g % DN] = mfma32x32x16(f, pb[g / DN], o[0][g % DN]);
        if (g >= MX0) {
          // values [32 (g - MX0), 32 (g + 1 - MX0)) / (NPV - MX0) of tile t+1's S^T
          const int v0 = (32 * (g - MX0)) / (NPV - MX0), v1 = (32 * (g + 1 - MX0)) / (NPV - MX0);
#pragma unroll
          for (int v = v0; v < v1; ++v) mx_run[v & 1] = fmaxf(mx_run[v & 1], acc[v >> 4][v & 15]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Prologue: tiles 0 and 1 in flight. Iteration t = -1 then computes only
    // S(0) (and refills with tile 2), so every iteration has one shape.
    // Every iteration issues one sub-tile's DMA (past the end: the last
    // sub-tile again, never read), so the count of loads in flight is the same
    // at every wait; the loop drains them before the item ends.
    __syncthreads();  // block list visible
    const int t_last = n_sub - 1;
    uint32_t e1 = entry(0), e2 = entry(1);  // entries of tiles t+1, t+2 (clamped to the last)
    if (n_sub > 0) {
      dma_tile(key_start(e1, 0), 0);
      dma_tile(key_start(e2, min(1, t_last)), 1);
    }
    f32x16 sa[2], sb[2];
    bool act = false;        // tile t computed by this wave
    float mt = -INFINITY;    // its maximum
    // iteration t: tile t's S^T in cur, tile t+1's into nxt
    auto iter = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
      vm_wait<DPT>();                       // tile t+1 landed (t+2 may be in flight)
      __syncthreads();                      // ... for every wave; all are past iteration t-1
      const uint32_t e3 = entry(t + 3);
      const int k3 = key_start(e3, min(t + 3, t_last));
      const int slot3 = (t + 3) & 3;
      const int k1 = key_start(e1, t + 1);
      const bool act1 = t + 1 < n_sub && active(e1, t + 1);
      float mt1 = -INFINITY;
      if (act) rescale_if_needed(mt);
      const float m_use = (m_run[0] == -INFINITY) ? 0.f : m_run[0];
      if (act && act1 && !needs_mask(k1)) {
        // the common case, written in issue order with scheduling fences:
        // S(t+1) with the exponentials of t, then PV(t) with the maximum of
        // t+1; K/V fragments are read four MFMAs ahead
        if (!XATTN_DMA_SPREAD) dma_tile(k3, slot3);
        full_step((t + 1) & 3, t & 3, cur, nxt, m_use, k3, slot3);
        mt1 = halves_max(fmaxf(mx_run[0], mx_run[1])) * a.scale_log2;
      } else {
        dma_tile(k3, slot3);
        if (act1) s_mma((t + 1) & 3, nxt);
        if (act) {
          exp_tile(cur, m_use);
          pv(t & 3);
        }
        if (act1) mt1 = mask_max(k1, nxt);
      }
      act = act1;
      mt = mt1;
      e1 = e2;
      e2 = e3;
    };
    if (n_sub > 0) {
      for (int t = -1; t < n_sub; t += 2) {
        iter(t, sb, sa);
        if (t + 1 < n_sub) iter(t + 1, sa, sb);
      }
      vm_wait<0>();  // the trailing loads, so no DMA reaches the ring after the item
    }
  } else {
    __syncthreads();  // block list visible
    if constexpr (DEPTH == 1) {
      Stage r0;
      uint32_t e0 = entry(0), e1 = entry(1);  // entries of tiles t, t+1
      if (n_sub > 0) {
        load_tile(key_start(e0, 0), r0);
        store_tile(0, r0);
      }
      __syncthreads();
      for (int t = 0; t < n_sub; ++t) {
        const bool more = t + 1 < n_sub;
        const uint32_t e2 = entry(t + 2);
        if (more) load_tile(key_start(e1, t + 1), r0);
        compute(key_start(e0, t), mine_tile(e0), t & 1);
        if (more) store_tile((t + 1) & 1, r0);
        __syncthreads();
        e0 = e1;
        e1 = e2;
      }
    } else {
      // two sub-tiles in flight: tile t+2 is fetched while tile t is computed and
      // tile t+1 (fetched one iteration earlier) waits in registers
      Stage ra, rb;
      uint32_t e0 = entry(0), e1 = entry(1), e2 = entry(2);  // entries of tiles t .. t+2
      if (n_sub > 0) load_tile(key_start(e0, 0), ra);
      if (n_sub > 1) load_tile(key_start(e1, 1), rb);
      if (n_sub > 0) store_tile(0, ra);
      __syncthreads();
      auto iter = [&](int t, Stage& ld, const Stage& st) {
        const uint32_t e3 = entry(t + 3);
        if (t + 2 < n_sub) load_tile(key_start(e2, t + 2), ld);
        compute(key_start(e0, t), mine_tile(e0), t & 1);
        if (t + 1 < n_sub) store_tile((t + 1) & 1, st);
        __syncthreads();
        e0 = e1;
        e1 = e2;
        e2 = e3;
      };
      for (int t = 0; t < n_sub; t += 2) {
        iter(t, ra, rb);
        if (t + 1 < n_sub) iter(t + 1, rb, ra);
      }
    }
  }

  // ---- epilogue: O = O^T / l, lse = (m + log2 l) * ln 2
#if XATTN_O_STAGE
  // Each wave stages its rows of O (bf16) in LDS over the K/V tiles and then
  // stores whole rows, 1 KiB of consecutive bytes per store instruction,
  // instead of 16 bytes in each of 32 rows straight from the accumulators.
  // On the short layers, where every row keeps two blocks and the kernel is
  // bound by memory traffic, that took about a tenth off bsa_fwd (the store
  // had been about a quarter of its time); on the long ones about 1%.
  if constexpr (PIPE) __syncthreads();  // every wave past its last read of the ring
  if (!live) return;
  constexpr int ROWB = 2 * C;           // bytes per output row
  constexpr int CH = ROWB / 16;         // 16-byte chunks per row
  constexpr int PIECES = RPW * CH;      // 16-byte pieces of a wave's rows
  static_assert((NT / 64) * RPW * ROWB <= TILES_B, "O staging fits over the K/V tiles");
  static_assert(PIECES % 64 == 0, "whole store instructions");
  unsigned char* stage = smem + wave * (RPW * ROWB);
  // The staging addresses depend on the lane only. Redefined here (empty
  // asm), they cannot be hoisted out of the item loop, where they would stay
  // live across the key loop and push it into spills.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int l32s = ln & 31, hhs = ln >> 5;
  // chunk c of staged row r sits at chunk c ^ (r % CH), so the 32 rows of one
  // write instruction (256 bytes apart) spread over every bank
#pragma unroll
  for (int y = 0; y < QT; ++y) {
    const float l_tot = halves_sum(l_run[y]);
    const float inv = 1.f / l_tot;
    const int r = 32 * y + l32s;
#pragma unroll
    for (int d = 0; d < DN; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 w;
        w[0] = (uint32_t)f32_to_bf16(o[y][d][4 * g4 + 0] * inv) |
               ((uint32_t)f32_to_bf16(o[y][d][4 * g4 + 1] * inv) << 16);
        w[1] = (uint32_t)f32_to_bf16(o[y][d][4 * g4 + 2] * inv) |
               ((uint32_t)f32_to_bf16(o[y][d][4 * g4 + 3] * inv) << 16);
        // dims 32 d + 8 g4 + 4 hh .. + 3: chunk 4 d + g4, its half hh
        *reinterpret_cast<u32x2*>(stage + r * ROWB + 16 * ((4 * d + g4) ^ (r % CH)) + 8 * hhs) = w;
      }
    const int qi = q0 + r;
    if (qi < a.Mq && a.lse && hhs == 0) a.lse[bh * a.Mq + qi] = (m_run[y] + log2f(l_tot)) * kLn2;
  }
  // the stage is private to the wave: its LDS operations complete in order
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int it = 0; it < PIECES / 64; ++it) {
    const int pc = it * 64 + ln;
    const int r = pc / CH, c = pc % CH;
    const int qi = q0 + r;
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * ROWB + 16 * (c ^ (r % CH)));
    if (qi < a.Mq) {  // rows past the end of a partial last block are not written
      u32x4* dst = reinterpret_cast<u32x4*>(a.out + (bh * a.Mq + qi) * C + 8 * c);
      if (XATTN_NT_QO)
        __builtin_nontemporal_store(val, dst);
      else
        *dst = val;
    }
  }
#else
  if (!live) return;
#pragma unroll
  for (int y = 0; y < QT; ++y) {
    const float l_tot = halves_sum(l_run[y]);
    const float inv = 1.f / l_tot;
    const int qi = q0 + 32 * y + l32;
    if (qi < a.Mq) {  // rows past the end of a partial last block are not written
      uint16_t* orow = a.out + (bh * a.Mq + qi) * C;
#pragma unroll
      for (int d = 0; d < DN; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dc = 32 * d + 8 * g4 + 4 * hh;
          u32x2 w;
          w[0] = (uint32_t)f32_to_bf16(o[y][d][4 * g4 + 0] * inv) |
                 ((uint32_t)f32_to_bf16(o[y][d][4 * g4 + 1] * inv) << 16);
          w[1] = (uint32_t)f32_to_bf16(o[y][d][4 * g4 + 2] * inv) |
                 ((uint32_t)f32_to_bf16(o[y][d][4 * g4 + 3] * inv) << 16);
          if (XATTN_NT_QO)
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(orow + dc));
          else
            *reinterpret_cast<u32x2*>(orow + dc) = w;
        }
      if (a.lse && hh == 0) a.lse[bh * a.Mq + qi] = (m_run[y] + log2f(l_tot)) * kLn2;
    }
  }
#endif
}

// Claims the next item for a persistent workgroup. queue[32 x] counts the
// items handed out from XCD x's share: the positions w = 8 j + x of xcd_map's
// order, which the hardware would have dispatched to XCD x. A workgroup serves
// the share of the XCD it runs on first, then the other shares in turn
// (stealing once its own runs dry); q, the offset of the share being served,
// only grows, so a workgroup makes at most (items it runs) + 8 claims. Each
// position is handed out once; items never wait on one another.
__device__ __forceinline__ uint32_t claim_item(uint32_t* queue, const uint32_t n,
                                               const uint32_t K, const uint32_t x0, uint32_t& q) {
  for (; q < 8; ++q) {
    const uint32_t x = (x0 + q) & 7u;
    const uint32_t j = __hip_atomic_fetch_add(queue + 32 * x, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t w = 8ull * j + x;
    if (w < n) return xcd_map((uint32_t)w, n, K, XATTN_SPARSE_ROWS_PER_XCD_LOG2);
  }
  return kNoItem;
}

// Dense: one workgroup per item, in xcd_map order (rows of equal length
// within a window, so the hardware's in-order dispatch keeps every engine busy).
// Sparse: persistent workgroups (as many as fit on the device at once) pull
// items from per-XCD queues in the same order. Rows of one query block differ
// by orders of magnitude in length between heads; the hardware dispatches the
// workgroups of an XCD in order and round-robin over its shader engines, so a
// one-workgroup-per-item launch parks the long rows of a dense head on one
// engine and stalls the others behind it. Pulling from a queue keeps every
// workgroup slot busy until the queues run dry.
template <int C, int BLK, bool CAUSAL, bool SPARSE, int MODE, bool KTAIL, int RPW>
__global__ __launch_bounds__(64 * (BLK / RPW) * AttnMode<MODE>::SLOTS, MODE == MODE_SINGLE ? 2 : 1)
void attn_fwd_bf16_kernel(AttnArgs a) {
  using L = AttnLds<C>;
  constexpr int SLOTS = AttnMode<MODE>::SLOTS;
  constexpr int NT = 64 * (BLK / RPW) * SLOTS;
  constexpr bool PIPE = XATTN_ATTN_PIPE != 0 && SLOTS == 2 && RPW == 32;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[PIPE ? L::bytes_pipe(SLOTS) : L::bytes(SLOTS)];
  __shared__ int scan_s[SLOTS > 1 ? NT / 64 : 1];
  const AttnItems its(a, MODE);
  if constexpr (!SPARSE) {
    attn_item<C, BLK, CAUSAL, SPARSE, MODE, KTAIL, RPW>(a, xcd_map(blockIdx.x, its.n, its.GW, 0), smem, scan_s);
  } else {
    __shared__ uint32_t item_s;
    const uint32_t K = (XATTN_SPARSE_GROUP_ON_XCD ? its.GW : 1) * XATTN_SPARSE_ROWS_PER_CHUNK;
    const uint32_t x0 = xcc_id();
    uint32_t q = 0;
    for (;;) {
      if (threadIdx.x == 0) item_s = claim_item(a.queue, its.n, K, x0, q);
      __syncthreads();
      const uint32_t item = item_s;
      if (item == kNoItem) break;  // uniform over the workgroup
      // every thread reads item_s before the barriers inside attn_item, and
      // thread 0 rewrites it only after them
      attn_item<C, BLK, CAUSAL, SPARSE, MODE, KTAIL, RPW>(a, item, smem, scan_s);
    }
  }
}

// Clears the item queues of a sparse launch (graph-safe: a kernel, not a memset).
__global__ void clear_queue_kernel(uint32_t* queue) { queue[threadIdx.x] = 0u; }

// ------------------------------------------------------------------ fp32 path

struct AttnArgsF32 {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  float* out;
  float* lse;
  int B, Hq, Hkv, Mq, Mk, NBq, NBk, qoff, block, causal;
  float scale_log2;
};

template <int C>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnArgsF32 a) {
  const int qi = blockIdx.x * 64 + threadIdx.x;
  if (qi >= a.Mq) return;  // no barriers below
  const int h = blockIdx.y % a.Hq;
  const int b = blockIdx.y / a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const size_t bh = (size_t)b * a.Hq + h, bg = (size_t)b * a.Hkv + g;
  const float* qrow = a.q + (bh * a.Mq + qi) * C;
  const float* kh = a.k + bg * a.Mk * C;
  const float* vh = a.v + bg * a.Mk * C;
  const int I = qi / a.block;
  const int qa = qi + a.qoff * a.block;           // position in the key sequence
  const int kmax = a.causal ? min(qa, a.Mk - 1) : a.Mk - 1;
  float qv[C], acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) { qv[c] = qrow[c]; acc[c] = 0.f; }
  float m = -INFINITY, l = 0.f;
  int cnt;
  const int32_t* idx = nullptr;
  if (a.kv_idx) {
    cnt = a.kv_cnt[bh * a.NBq + I];
    cnt = cnt < 0 ? 0 : (cnt > a.NBk ? a.NBk : cnt);
    idx = a.kv_idx + (bh * a.NBq + I) * a.NBk;
  } else {
    cnt = a.causal ? I + a.qoff + 1 : a.NBk;
  }
  for (int t = 0; t < cnt; ++t) {
    int jb = idx ? idx[t] : t;
    jb = jb < 0 ? 0 : (jb >= a.NBk ? a.NBk - 1 : jb);
    for (int kj = jb * a.block; kj < (jb + 1) * a.block; ++kj) {
      if (kj > kmax) break;
      const float* kr = kh + (size_t)kj * C;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) s = fmaf(qv[c], kr[c], s);
      s *= a.scale_log2;
      const float mn = fmaxf(m, s);
      const float alpha = fast_exp2(m - mn);
      const float p = fast_exp2(s - mn);
      l = l * alpha + p;
      const float* vr = vh + (size_t)kj * C;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = fmaf(p, vr[c], acc[c] * alpha);
      m = mn;
    }
  }
  const float inv = 1.f / l;
  float* orow = a.out + (bh * a.Mq + qi) * C;
#pragma unroll
  for (int c = 0; c < C; ++c) orow[c] = acc[c] * inv;
  if (a.lse) a.lse[bh * a.Mq + qi] = (m + log2f(l)) * kLn2;
}

// ------------------------------------------------------------------ launchers

template <int C, int BLK, int MODE, bool KTAIL, int RPW>
static hipError_t launch_bf16_cbmt(const Shape& s, const AttnArgs& a, hipStream_t st, bool queue_zeroed) {
  const int G = s.Hq / s.Hkv;
  const int NP = MODE == MODE_ROWS ? (s.NBq() + 1) / 2 : s.NBq();
  const int GW = MODE == MODE_SIBLINGS ? G / 2 : G;
  const size_t n_items = (size_t)s.B * s.Hkv * GW * NP;
  const int threads = 64 * (BLK / RPW) * AttnMode<MODE>::SLOTS;
  if (a.kv_idx == nullptr) {
    const dim3 grid((unsigned)n_items);
    if (s.causal)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<C, BLK, true, false, MODE, KTAIL, RPW>), grid, dim3(threads), 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<C, BLK, false, false, MODE, KTAIL, RPW>), grid, dim3(threads), 0, st, a);
    return hipGetLastError();
  }
  if (a.queue == nullptr) return hipErrorInvalidValue;
  auto kern = s.causal ? attn_fwd_bf16_kernel<C, BLK, true, true, MODE, KTAIL, RPW>
                       : attn_fwd_bf16_kernel<C, BLK, false, true, MODE, KTAIL, RPW>;
  const int slots = resident_workgroups(kern, threads);
  if (slots <= 0) return hipErrorInvalidDeviceFunction;
  if (!queue_zeroed) {
    hipLaunchKernelGGL(clear_queue_kernel, dim3(1), dim3(kQueueWords), 0, st, a.queue);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(n_items < (size_t)slots ? n_items : (size_t)slots));
  hipLaunchKernelGGL(kern, grid, dim3(threads), 0, st, a);
  return hipGetLastError();
}

// Sparse launches use XATTN_SPARSE_RPW query rows per wave, dense ones
// XATTN_DENSE_RPW.
#ifndef XATTN_SPARSE_RPW
#define XATTN_SPARSE_RPW 32
#endif
#ifndef XATTN_DENSE_RPW
#define XATTN_DENSE_RPW 32
#endif

template <int C, int BLK, int MODE, int RPW>
static hipError_t launch_bf16_cbmr(const Shape& s, const AttnArgs& a, hipStream_t st, bool qz) {
  return s.Mk % BLK ? launch_bf16_cbmt<C, BLK, MODE, true, RPW>(s, a, st, qz)
                    : launch_bf16_cbmt<C, BLK, MODE, false, RPW>(s, a, st, qz);
}

template <int C, int BLK, int MODE>
static hipError_t launch_bf16_cbm(const Shape& s, const AttnArgs& a, hipStream_t st, bool qz) {
  constexpr int SR = BLK >= XATTN_SPARSE_RPW ? XATTN_SPARSE_RPW : 32;
  constexpr int DR = BLK >= XATTN_DENSE_RPW ? XATTN_DENSE_RPW : 32;
  return a.kv_idx != nullptr ? launch_bf16_cbmr<C, BLK, MODE, SR>(s, a, st, qz)
                             : launch_bf16_cbmr<C, BLK, MODE, DR>(s, a, st, qz);
}

// 128-row blocks: dense attention pairs GQA siblings (identical block lists)
// when the group size is even and neighbouring rows of a head when it is odd;
// sparse attention over GQA-union lists pairs siblings too. Other sparse lists
// pair neighbouring rows of one head on long sequences (their lists share most
// blocks, so the union costs little and each K/V tile is fetched once for both
// rows) and run one (head, row) per workgroup otherwise; sibling heads keep
// very different numbers of blocks, so a sibling pair would leave one half
// idle. 64-row blocks use one (head, row) per workgroup.
template <int C, int BLK>
static hipError_t launch_bf16_cb(const Shape& s, const AttnArgs& a, hipStream_t st, bool qz) {
  if (BLK == 128) {
    const bool pairs = (s.Hq / s.Hkv) % 2 == 0;
    if (a.kv_idx == nullptr && pairs) return launch_bf16_cbm<C, BLK, MODE_SIBLINGS>(s, a, st, qz);
    // GQA-union lists are shared by the siblings: one tile load serves both
    if (a.kv_idx != nullptr && pairs && s.selection == SEL_GQA_UNION)
      return launch_bf16_cbm<C, BLK, MODE_SIBLINGS>(s, a, st, qz);
    if (a.kv_idx != nullptr &&
        s.NBq() >= (s.causal ? XATTN_SPARSE_PAIR_ROWS_MIN_NB : XATTN_SPARSE_PAIR_ROWS_MIN_NB_NC))
      return launch_bf16_cbm<C, BLK, MODE_ROWS>(s, a, st, qz);
    if (a.kv_idx == nullptr && XATTN_DENSE_PAIR_ROWS) return launch_bf16_cbm<C, BLK, MODE_ROWS>(s, a, st, qz);
  }
  return launch_bf16_cbm<C, BLK, MODE_SINGLE>(s, a, st, qz);
}

hipError_t launch_attn_bf16(const Shape& s, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                            float sm_scale, uint16_t* out, float* lse, uint32_t* queue,
                            hipStream_t st, bool queue_zeroed) {
  AttnArgs a{q,   k,    v,        kv_idx,  kv_cnt,  out,    lse,    queue,
             s.B, s.Hq, s.Hkv,    s.M,     s.Mk,    s.NBq(), s.NBk(), s.qoff(),
             sm_scale * kLog2e};
  if (s.C == 128 && s.block == 128) return launch_bf16_cb<128, 128>(s, a, st, queue_zeroed);
  if (s.C == 128 && s.block == 64) return launch_bf16_cb<128, 64>(s, a, st, queue_zeroed);
  if (s.C == 64 && s.block == 128) return launch_bf16_cb<64, 128>(s, a, st, queue_zeroed);
  if (s.C == 64 && s.block == 64) return launch_bf16_cb<64, 64>(s, a, st, queue_zeroed);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_f32(const Shape& s, const float* q, const float* k, const float* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, float sm_scale,
                           float* out, float* lse, hipStream_t st) {
  AttnArgsF32 a{q,    k,       v,       kv_idx,   kv_cnt,  out,      lse,
                s.B,  s.Hq,    s.Hkv,   s.M,      s.Mk,    s.NBq(),  s.NBk(),
                s.qoff(), s.block, s.causal, sm_scale * kLog2e};
  dim3 grid((s.M + 63) / 64, s.B * s.Hq);
  if (s.C == 64)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<64>), grid, dim3(64), 0, st, a);
  else if (s.C == 128)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<128>), grid, dim3(64), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}


hipError_t debug_counts_attn(unsigned int* out, bool reset) {
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
