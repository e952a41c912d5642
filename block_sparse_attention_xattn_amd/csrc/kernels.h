// Host-side launch declarations shared by the kernel sources and the C ABI
// layer. Every launcher only enqueues on `stream` and returns the HIP status of
// the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xattn {

// Queries are the last M of Mk tokens (Mk = M: plain prefill); Mk - M is a
// multiple of the block. Lengths need not be multiples of the stride or block:
// the last stride group and the last block may be partial.
struct Shape {
  int B, Hq, Hkv, M, C, block, stride, causal;
  int diagonal;  // scoring pattern: 0 antidiagonal, 1 diagonal (q[iS+s] with k[jS+s]), 2 DuSA1
  int selection; // SEL_ROW, SEL_GLOBAL or SEL_GQA_UNION
  int Mk;        // key length
  int NBq() const { return (M + block - 1) / block; }
  int NBk() const { return (Mk + block - 1) / block; }
  int qoff() const { return (Mk - M) / block; }  // key block of query block 0
  int Rq() const { return (M + stride - 1) / stride; }
  int Rk() const { return (Mk + stride - 1) / stride; }
  int r() const { return block / stride; }
};

// Stage 1: per (strided row i, key block J) partial log2-sum-exp of the scaled
// strided antidiagonal logits, written to ws as [b][h][I][J][t] float32 with
// I = i / r < NBq, J < NBk, t = i % r (rows past the last strided query row of
// a partial block are not written).
hipError_t launch_score_partials_bf16(const Shape& s, const uint16_t* q, const uint16_t* k,
                                      float score_scale, float* ws, hipStream_t st);
hipError_t launch_score_partials_f32(const Shape& s, const float* q, const float* k,
                                     float score_scale, float* ws, hipStream_t st);
// DuSA1 multi-stride scoring (pattern 2, bf16, lengths multiples of the
// stride): per (phase, strided row) log2-sum-exps into lse_ws (B*Hq*M floats,
// dusa1_lse_bytes), then the block scores written directly.
size_t dusa1_lse_bytes(const Shape& s);
hipError_t launch_score_dusa1(const Shape& s, const uint16_t* q, const uint16_t* k, float score_scale,
                              float* lse_ws, float* block_scores, hipStream_t st);

// Stage 2: block scores from the partials (row-normalised, divided by r).
hipError_t launch_score_finalize(const Shape& s, const float* ws, float* block_scores,
                                 hipStream_t st);

// Stage 3: per-row minimal-set selection.
struct TauArray {
  float v[256];
};
hipError_t launch_select(const Shape& s, const float* block_scores, const TauArray& tau,
                         uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st);

// Selection variants (xattn_selection): per-row minimal sets, one minimal set
// per head over the flattened block matrix, or per-row sets united over each
// KV group.
enum { SEL_ROW = 0, SEL_GLOBAL = 1, SEL_GQA_UNION = 2 };
// Device scratch of a selection in `mode` (0 unless global).
size_t select_workspace_bytes(const Shape& s, int mode);
hipError_t launch_select_global(const Shape& s, const float* block_scores, const TauArray& tau,
                                uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, void* ws,
                                hipStream_t st);
// Rewrites the per-row lists of every KV group's heads with their union.
hipError_t launch_gqa_union(const Shape& s, uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt,
                            hipStream_t st);

// Stages 2+3 fused (one launch per layer in xattn_prefill): block scores from
// the partials, written out, then selected without re-reading them.
hipError_t launch_score_select(const Shape& s, const float* ws, float* block_scores, const TauArray& tau,
                               uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st);

// Stages 1-3 in the scoring launch (xattn_prefill, per-row or GQA-union
// selection, bf16 with complete stride groups): the workgroup that stores the
// last partials of a (b, h, query tile) normalises and selects that tile's
// query-block rows. `arrive` holds arrive_words(s) counters that must be zero
// when the launch starts; block scores and the mask are optional outputs. The
// results equal launch_score_partials_bf16 followed by launch_score_select.
struct TileSelect {
  uint32_t* arrive;
  float* scores;
  uint8_t* mask;
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int qoff;  // key block of query block 0
  TauArray tau;
};
bool tile_select_ok(const Shape& s);
size_t arrive_words(const Shape& s);
hipError_t launch_score_tile_select(const Shape& s, const uint16_t* q, const uint16_t* k, float score_scale,
                                    float* ws, const TileSelect& sel, hipStream_t st);
// Zeroes n words of device memory (a kernel, so the call can be captured).
hipError_t launch_clear_words(uint32_t* words, size_t n, hipStream_t st);

// Stage 4: attention over listed key blocks (kv_idx == nullptr: every candidate).
// The sparse bf16 kernel schedules its rows through per-XCD item queues held
// in `queue` (kQueueWords words of device memory, cleared by the launcher on
// the stream first unless queue_zeroed says an earlier launch on the stream
// already did); dense launches ignore it.
constexpr int kQueueWords = 256;
hipError_t launch_attn_bf16(const Shape& s, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                            float sm_scale, uint16_t* out, float* lse, uint32_t* queue,
                            hipStream_t st, bool queue_zeroed = false);
hipError_t launch_attn_f32(const Shape& s, const float* q, const float* k, const float* v,
                           const int32_t* kv_idx, const int32_t* kv_cnt, float sm_scale,
                           float* out, float* lse, hipStream_t st);

// Categories of the debug build's bounds checks (XATTN_DCHECK in common.h).
enum DebugCheck {
  DBG_SCORE_STORE = 0,   // score partial written outside its head's [NBq][NBk][r] slab
  DBG_SELECT_ROW = 1,    // selection row or candidate count outside its state
  DBG_ATTN_KV_ROW = 2,   // K/V sub-tile rows outside [0, Mk)
  DBG_ATTN_LDS = 3,      // LDS ring slot or list entry outside its region
  DBG_ATTN_ITEM = 4,     // work item decoded outside (B, Hq, NBq)
  DBG_DUSA1_INDEX = 5,   // DuSA1 log-sum-exp or block-score index out of range
  DBG_CATEGORIES = 8
};

// Debug builds: adds each source's check counters into out[8] (and clears
// them when reset); release builds leave out untouched.
hipError_t debug_counts_score(unsigned int* out, bool reset);
hipError_t debug_counts_select(unsigned int* out, bool reset);
hipError_t debug_counts_attn(unsigned int* out, bool reset);
hipError_t debug_counts_dusa1(unsigned int* out, bool reset);

}  // namespace xattn
