/*
 * xattn.h — C ABI of the MI355X (gfx950) XAttention-style block-sparse
 * prefill attention library (libxattn.so).
 *
 * The method (sources are web pages; cited by page title and section):
 *   [XA-abs] "XAttention: Block Sparse Attention with Antidiagonal Scoring",
 *            arXiv abstract: the sum of antidiagonal values (lower-left to
 *            upper-right) of the attention matrix ranks block importance;
 *            block-sparse attention then runs on the important blocks.
 *   [XA-sum] same title, AI summary page, "Approach": strided antidiagonal sums
 *            inside each block, softmax-normalised, then the minimal set of
 *            blocks whose mass reaches a per-head threshold.
 *   [DuSA]   "DuSA: Fast and Accurate Dual-Stage Sparse Attention Mechanism
 *            Accelerating Both Training and Inference", rebuttal, "Response to
 *            Q2": Q and K of shape (B, H, M, C) are reshaped to
 *            (B, H, M/stride, stride*C) and a softmax attention is computed on
 *            the reshaped tensors.
 *   [Flex]   "FlexPrefill: ...", rebuttal, "R Q2: Integration Feasibility":
 *            a single function call replacing standard attention.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Q is (B, Hq, M, C); K and V are (B, Hkv, Mk, C) with Mk = p->Mk (0 means
 *    M); O has Q's shape. All are contiguous row-major DEVICE buffers of the
 *    problem dtype. Query head h reads KV head h / (Hq / Hkv) (grouped-query
 *    attention).
 *  - Chunked prefill: the queries are the last M of the Mk tokens, so query i
 *    sits at position off + i, off = Mk - M (0 for a plain prefill); off must
 *    be a multiple of the block size.
 *  - Block size Bk = p->block, stride S = p->stride, r = Bk / S strided rows
 *    per block; NBq = ceil(M / Bk) query blocks and NBk = ceil(Mk / Bk) key
 *    blocks; query block I is key block I + off / Bk ("its diagonal").
 *  - Lengths need not be multiples of S or Bk ([DuSA] rebuttal, Response to
 *    Q1: padding makes the length divisible by the block size): the missing
 *    tokens of a partial stride group count as zero vectors in the scoring,
 *    keys past the end take no part in any softmax, and query rows past the end
 *    of a partial last block are not written.
 *  - Block tensors are (B, Hq, NBq, NBk) row-major, indexed [b][h][I][J]
 *    (query block I, key block J).
 *  - The caller owns and allocates every buffer. The library keeps no state,
 *    never allocates, and is re-entrant; scratch memory comes only through
 *    the workspace arguments. A workspace's contents on entry are ignored
 *    (each call clears what it needs on its stream); calls that may overlap
 *    in time (other streams) need distinct workspaces.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *    call only enqueues work on it and returns without synchronising. The work
 *    is kernels only (no memsets, copies or host waits), so a call can be
 *    captured in a HIP graph and replayed; host arrays such as tau are read at
 *    the call (at capture, for a graph).
 *  - Arguments are validated on the host before anything is enqueued. On any
 *    error the call returns a non-zero status and enqueues nothing; a failed
 *    kernel launch returns XATTN_ERR_HIP. xattn_last_error() gives a message
 *    for the calling thread's last failure. No C++ exception crosses the ABI.
 *  - NaN or Inf inside Q/K/V gives unspecified values in the outputs; the
 *    kernels still terminate and stay within the buffers.
 *
 * Supported shapes: dtype XATTN_BF16 or XATTN_F32; C in {64, 128};
 * block in {64, 128}; r = block/stride in {2, 4, 8, 16, 32};
 * 1 <= M <= Mk with Mk - M a multiple of block and NBk <= 4096;
 * 1 <= Hq <= 256; Hq a multiple of Hkv; causal in {0, 1}. XATTN_F32 runs
 * scalar fp32 kernels meant for small layers at reference precision and
 * accepts Mk <= XATTN_F32_MAX_TOKENS (otherwise XATTN_ERR_UNSUPPORTED); the
 * bf16 path runs the MFMA kernels at every supported size.
 *
 * Workspaces: one size fits every call. xattn_workspace_bytes(p) is the
 * scratch that xattn_prefill needs, and it is enough for each stage entry
 * point on the same problem; the per-stage queries below return the smaller
 * amounts each stage alone needs.
 */
#ifndef XATTN_H
#define XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define XATTN_ABI_VERSION 5
#define XATTN_MAX_HEADS 256
#define XATTN_MAX_BLOCKS 4096
/* XATTN_F32 problems run scalar fp32 kernels (reference precision for small
 * layers) and take key lengths of at most this many tokens. */
#define XATTN_F32_MAX_TOKENS 16384

typedef enum {
  XATTN_OK = 0,
  XATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  XATTN_ERR_SHAPE = 2,       /* sizes inconsistent (divisibility, ranges) */
  XATTN_ERR_DTYPE = 3,       /* unknown dtype */
  XATTN_ERR_ARG = 4,         /* a scalar argument is out of range (tau, scales) */
  XATTN_ERR_UNSUPPORTED = 5, /* valid but not implemented (C, block, r) */
  XATTN_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  XATTN_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} xattn_status;

typedef enum { XATTN_BF16 = 0, XATTN_F32 = 1 } xattn_dtype;

/* Problem description. All fields are plain int32. */
typedef struct {
  int32_t B;      /* batch */
  int32_t Hq;     /* query heads */
  int32_t Hkv;    /* key/value heads, divides Hq */
  int32_t M;      /* query length (= key length unless Mk says otherwise) */
  int32_t C;      /* head dimension */
  int32_t block;  /* block size Bk (queries and keys) */
  int32_t stride; /* antidiagonal stride S, divides block */
  int32_t causal; /* 1: key j visible to query i iff j <= i; 0: all keys */
  int32_t dtype;  /* xattn_dtype of Q, K, V and O */
  int32_t pattern; /* xattn_pattern of the strided scoring (0 = antidiagonal) */
  int32_t selection; /* xattn_selection of the block selection (0 = per row) */
  int32_t Mk;     /* key length; 0 means M. Mk - M is a multiple of block */
  int32_t flags;  /* xattn_flags, OR-ed; 0 = the defaults */
} xattn_problem;

/* Options of xattn_problem.flags (unknown bits return XATTN_ERR_ARG):
 *  SELECT_IN_SCORE: xattn_prefill normalises and selects inside the scoring
 *  launch ([XA-sum] Approach runs the three steps back to back; here the
 *  workgroup that stores a query tile's last partials selects that tile's
 *  rows at once), one launch fewer per call, with block scores, masks, lists
 *  and output bit-identical to the default. It applies where the scoring
 *  streams whole stride groups (bf16, M and Mk multiples of S, S*C a multiple
 *  of 128, antidiagonal or diagonal pattern, per-row or GQA-union selection)
 *  and is ignored elsewhere. On MI355X it is slower than the default separate
 *  selection launch: the scoring kernel holds a whole compute unit, which then
 *  idles its matrix cores through the latency-bound selection, while the
 *  separate launch overlaps seven selections per compute unit. */
typedef enum { XATTN_SELECT_IN_SCORE = 1 } xattn_flags;

/* How the strided scoring forms its logits:
 *  ANTIDIAGONAL (the method, [XA-abs]): query row i*S+s with key row j*S+S-1-s,
 *  summed over s, one softmax per strided row;
 *  DIAGONAL (the older variant compared in [DuSA] Response to Q2 and in the
 *  [XA-sum] ablation table): query row i*S+s with key row j*S+s, summed over s;
 *  DUSA1 ([DuSA] Response to Q2, DuSA1: Q and K reshaped to (S, M/S, C)
 *  phases, a softmax per phase): each phase row q[i*S+s] is softmaxed over its
 *  phase's keys k[j*S+s] on its own (logit score_scale * q.k, j <= i + off/S
 *  when causal), and block (I, J) scores the phases' summed mass over its
 *  S * r_I rows divided by S * r_I. DUSA1 takes bf16 inputs whose lengths M and
 *  Mk are multiples of S (else XATTN_ERR_UNSUPPORTED / XATTN_ERR_SHAPE); its
 *  natural score_scale is the attention scale 1/sqrt(C). */
typedef enum { XATTN_ANTIDIAGONAL = 0, XATTN_DIAGONAL = 1, XATTN_DUSA1 = 2 } xattn_pattern;

/* How xattn_select (and xattn_prefill) choose blocks:
 *  ROW (the method, [XA-sum] Approach): a minimal set per query-block row;
 *  GLOBAL ([Flex] R Q3, global index selection over the flattened block
 *  matrix): one minimal set per head over every candidate (I, J) at once,
 *  ordered by score descending, ties by (I, J) row-major, against tau_h times
 *  the head's candidate mass; then every diagonal block is added;
 *  GQA_UNION (a reuse variant, not from the pages): ROW, then every head of a
 *  KV group keeps the union of the group's rows. bsa_fwd then serves two
 *  sibling heads per workgroup from one K/V tile. */
typedef enum {
  XATTN_SELECT_ROW = 0,
  XATTN_SELECT_GLOBAL = 1,
  XATTN_SELECT_GQA_UNION = 2
} xattn_selection;

/* ABI version of the loaded library (XATTN_ABI_VERSION). */
int32_t xattn_abi_version(void);

/* Static description of a status code. */
const char* xattn_status_string(xattn_status s);

/* Message describing the calling thread's most recent failed call. */
const char* xattn_last_error(void);

/* Device workspace bytes that serve every entry point for problem p (equal
 * to xattn_prefill_workspace_bytes(p)); 0 if p is invalid. */
size_t xattn_workspace_bytes(const xattn_problem* p);

/* Device workspace bytes xattn_score needs for problem p;
 * 0 if p is invalid. The workspace holds per-(strided row, key block) partial
 * log-sum-exp values: B*Hq*NBq*NBk*r float32 (DUSA1: per (phase, strided row)
 * log-sum-exps, B*Hq*M float32 rounded up to 256 bytes, then room for
 * B*Hq*NBq*NBk float32 block scores). */
size_t xattn_score_workspace_bytes(const xattn_problem* p);

/*
 * Stage 1+2 — strided antidiagonal block scores ([XA-abs]; [XA-sum] Approach;
 * [DuSA] Response to Q2).
 *
 * For strided query row i < ceil(M/S) and strided key row j < ceil(Mk/S):
 *   A'[i][j] = sum_{s<S} dot(q[i*S+s], k[j*S+S-1-s]),  logit = score_scale*A'
 * (k[j*S+s] instead for p->pattern = XATTN_DIAGONAL; tokens past the end are
 * zero). Causal problems keep j <= i + off/S. Each strided row is
 * softmax-normalised over its keys, and the probabilities are summed over each
 * r x r tile:
 *   block_scores[b][h][I][J] = (1/r_I) * sum_{i in I, j in J} softmax_j(logit[i][j]),
 * r_I = the strided rows of query block I (r unless I is a partial last block).
 * Every row of block_scores sums to 1; causal entries with J > I + off/Bk are 0.
 *
 *  q, k          device, problem dtype, layouts above.
 *  score_scale   > 0 and finite (e.g. 1/(S*sqrt(C)): the mean antidiagonal logit).
 *  block_scores  device float32 (B, Hq, NBq, NBk), fully written.
 *  ws, ws_bytes  device scratch of at least xattn_score_workspace_bytes(p).
 */
xattn_status xattn_score(const xattn_problem* p, const void* q, const void* k,
                         float score_scale, float* block_scores, void* ws,
                         size_t ws_bytes, void* stream);

/* Device workspace bytes xattn_select needs: 0 for ROW and GQA_UNION; for
 * GLOBAL, per head a 64-byte state, a 48 KiB mass histogram and NBq words. */
size_t xattn_select_workspace_bytes(const xattn_problem* p);

/*
 * Stage 3 — minimal-set threshold selection ([XA-sum] Approach: the minimal
 * set of blocks whose normalised mass exceeds the per-head threshold;
 * [Flex] R Q3: minimal |S| under the cumulative-mass constraint).
 *
 * Per row (b, h, I): candidates are J <= I + off/Bk (causal) or all J < NBk.
 * They are ordered by score descending, ties by J ascending; with prefix
 * masses c_k (float64) and total T = c_n, the kept set is the first
 * k* = min{k >= 0 : c_k >= tau_h*T} candidates (tau_h >= 1 keeps all). The
 * diagonal block J = I + off/Bk is then added.
 * p->selection picks the GLOBAL or GQA_UNION variant instead (see
 * xattn_selection); GLOBAL sums fixed-point masses (score * 2^50, exact and
 * order-independent) instead of float64 prefixes.
 *
 *  block_scores  device float32 (B, Hq, NBq, NBk), as written by xattn_score.
 *  tau           HOST array of Hq floats, each in [0, 1] (copied at the call).
 *  mask          device uint8 (B, Hq, NBq, NBk) or NULL; 1 = kept.
 *  kv_idx        device int32 (B, Hq, NBq, NBk): per row the kept J in
 *                ascending order; only the first kv_cnt entries are written.
 *  kv_cnt        device int32 (B, Hq, NBq): kept blocks per row (>= 1).
 *  ws, ws_bytes  device scratch of xattn_select_workspace_bytes(p) (may be
 *                NULL when that is 0).
 */
xattn_status xattn_select(const xattn_problem* p, const float* block_scores,
                          const float* tau, uint8_t* mask, int32_t* kv_idx,
                          int32_t* kv_cnt, void* ws, size_t ws_bytes, void* stream);

/* Device workspace bytes bsa_fwd needs (a fixed 1 KiB of per-XCD work-queue
 * counters); 0 if p is invalid. */
size_t xattn_attn_workspace_bytes(const xattn_problem* p);

/*
 * Stage 4 — block-sparse attention forward ([XA-abs]: block-sparse attention
 * computes only on the important blocks).
 *
 * For query i in block I of head h:
 *   O[i] = sum_{j in A(i)} softmax_j(sm_scale * q_i . k_j) v_j,
 *   A(i) = union of key blocks kv_idx[b][h][I][0 .. kv_cnt-1], restricted to
 *          keys j < Mk, and to j <= off + i when causal.
 *
 *  kv_idx, kv_cnt  device int32 as produced by xattn_select; each listed J
 *                  must be in [0, NBk) (and <= I + off/Bk when causal), kv_cnt
 *                  in [1, NBk], and for causal problems the list must hold the
 *                  diagonal J = I + off/Bk.
 *  sm_scale        > 0 and finite (usually 1/sqrt(C)).
 *  out             device, problem dtype, (B, Hq, M, C).
 *  lse             device float32 (B, Hq, M), natural-log log-sum-exp of the
 *                  scaled logits over A(i); may be NULL.
 *  ws, ws_bytes    device scratch of at least xattn_attn_workspace_bytes(p):
 *                  the queues from which the workgroups pull query rows.
 */
xattn_status bsa_fwd(const xattn_problem* p, const void* q, const void* k,
                     const void* v, const int32_t* kv_idx, const int32_t* kv_cnt,
                     float sm_scale, void* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Dense attention forward: bsa_fwd with every candidate block kept (all
 * J <= I + off/Bk when causal, all J otherwise). The reference point for
 * speedups: the pages measure the method's prefill speedup against dense
 * FlashAttention ([XA-sum] "Key results": speedup relative to FlashInfer's
 * FlashAttention at 256K tokens). Arguments as in bsa_fwd; no block lists and
 * no workspace (one workgroup per query-block row or row pair, no queues).
 */
xattn_status dense_fwd(const xattn_problem* p, const void* q, const void* k,
                       const void* v, float sm_scale, void* out, float* lse,
                       void* stream);

/* Device workspace bytes xattn_prefill needs: the score partials, the
 * selection scratch, the per-(b, h, query tile) arrival counters when
 * XATTN_SELECT_IN_SCORE applies, and the attention queues, each part starting
 * on a 256-byte boundary; 0 if p is invalid. */
size_t xattn_prefill_workspace_bytes(const xattn_problem* p);

/*
 * The three stages in one call ([Flex] R Q2: one call in place of standard
 * attention): xattn_score, then xattn_select, then bsa_fwd, all enqueued on
 * `stream`. Arguments as in those calls; mask and lse may be NULL, and so may
 * block_scores unless p->selection is XATTN_SELECT_GLOBAL (which ranks the
 * head's whole block matrix): with per-row selection the scores of each row
 * are normalised and selected in one pass and need not be written. ws holds
 * at least xattn_prefill_workspace_bytes(p) (= xattn_workspace_bytes(p)).
 */
xattn_status xattn_prefill(const xattn_problem* p, const void* q, const void* k,
                           const void* v, const float* tau, float score_scale,
                           float sm_scale, float* block_scores, uint8_t* mask,
                           int32_t* kv_idx, int32_t* kv_cnt, void* ws,
                           size_t ws_bytes, void* out, float* lse, void* stream);

/* Scratch held by xattn_prefill_noalloc on each GPU it runs on. */
#define XATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * xattn_prefill without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Its scratch is a library-owned array of
 * XATTN_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held until the process ends;
 * the call itself allocates nothing (no hipMalloc or allocating library
 * routine). The caller still passes every input and output, with the
 * meanings, layouts and NULL rules of xattn_prefill, and the results are
 * those of xattn_prefill.
 *
 * Limits: problems whose xattn_workspace_bytes(p) exceeds
 * XATTN_NOALLOC_SCRATCH_BYTES return XATTN_ERR_WORKSPACE before anything is
 * enqueued (e.g. 32 query heads, r = 16: up to about 22K tokens). Every call on
 * one GPU shares that GPU's array, and each call clears what must start at
 * zero on its stream: calls that may overlap in time on one GPU (several
 * streams or threads) race and give undefined results; serialise them.
 */
xattn_status xattn_prefill_noalloc(const xattn_problem* p, const void* q, const void* k,
                                   const void* v, const float* tau, float score_scale,
                                   float sm_scale, float* block_scores, uint8_t* mask,
                                   int32_t* kv_idx, int32_t* kv_cnt, void* out, float* lse,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */
