/*
 * libtttattn: multi-pass EAGLE-3 test-time-training (TTT) draft attention for
 * AMD Instinct MI355X (gfx950).  C ABI; plain pointers and sizes only.
 *
 * What one call computes (one TTT pass p, 1-based).  Sources: NeMo-RL issue
 * "DFlash/DSpark and EAGLE-3 TTT draft co-training for speculative decoding
 * (Megatron backend)", section "What I'm working on", item 1 (sequential draft
 * passes, two-part trunk+branch flash attention, exact joint-LSE merge,
 * inference-aligned per-pass RoPE offsets) and item 4 (THD varlen layout);
 * NeMo-RL PR #3725 (bounded multi-pass EAGLE-3 TTT provider), Summary (no dense
 * pass logits or sequence-square masks; rotary support validated up front)
 * and the self-review comment (staircase visibility, rotate-half RoPE, the
 * attention core owns no parameters).
 *
 *   Query row i of pass p (position i+p-1) attends to
 *     trunk : pass-1 keys/values at rows j <= i of its own sequence (position j)
 *     branch: the keys/values that passes q = 2..p produced at row i
 *             (position i+q-1)
 *   Keys and queries get rotate-half RoPE (pair k with k+D/2,
 *   theta_k = base^(-2k/D)); values are not rotated.  The trunk and branch
 *   partial softmaxes are joined by an exact log-sum-exp merge, so
 *     O_i   = sum over visible keys a of softmax(scale * <R q_i, R k_a>) v_a
 *     LSE_i = ln sum over visible keys a of exp(scale * <R q_i, R k_a>)
 *   GQA: query head h reads key/value head h / (Hq / Hkv).
 *
 * Tensors (element strides; the head_dim axis must be contiguous):
 *   q, o, dout, dq : BSHD [B, S, Hq, D] or THD [T, Hq, D]
 *   k[q], v[q], dk[q], dv[q] (q = 0..p-1, index 0 = pass 1 = trunk):
 *                    BSHD [B, S, Hkv, D] or THD [T, Hkv, D]
 *   lse (fp32, contiguous): BSHD [B, Hq, S], THD [Hq, T]
 * q/dq use q_stride, o/dout use o_stride, every k/v/dk/dv uses kv_stride.
 * A zero stride triple selects the contiguous default.  Token strides above
 * 2^25 elements are rejected (TTT_ERR_BAD_SHAPE): tile loads address up to 32
 * rows past a base with 32-bit byte offsets.
 *
 * Ownership and state: the caller owns every buffer, including the
 * workspace, and the optional second stream of the backward (aux_stream).
 * The library allocates no device memory and keeps no state between calls
 * (ttt_attn_fwd_noalloc's static scratch array aside).  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL is the default stream) and
 * re-entrant.  Outputs are overwritten, never accumulated: gradients of a
 * key/value tensor used by several passes are summed by the caller.  Two
 * calls that share a workspace must be ordered on one stream.
 *
 * Empty problems (zero tokens) return TTT_OK at once, after the descriptor is
 * checked; their tensor pointers are not examined.
 *
 * Errors: every argument is checked on the host before anything is launched;
 * a non-zero status means nothing was enqueued.  ttt_attn_last_error() gives
 * the detail (thread-local).  Faults inside kernels surface at the caller's
 * next synchronisation.  No C++ exception crosses this interface.
 */
#ifndef TTTATTN_H
#define TTTATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: ttt_attn_chunk, ttt_attn_block and ttt_soft_ce_desc gained the packed
 * (THD) and per-row / per-group fields; each struct's struct_size check
 * refuses a caller built against an older layout.  4: ttt_attn_desc gained
 * aux_stream (the library keeps no stream of its own). */
#define TTT_ATTN_ABI_VERSION 4

enum ttt_attn_layout { TTT_LAYOUT_BSHD = 0, TTT_LAYOUT_THD = 1 };
/* BF16: the score products run on fp16 operands.  q and k are rotated in fp32
 * and rounded once to fp16, which keeps more of the rotated values' mantissa
 * than bf16 does (an LSE error of ~4e-4 at worst instead of ~2e-3), so the
 * rotated values must stay inside fp16's range: |R q|, |R k| < 65504 per
 * element (|q|, |k| < 46000 suffices), else scores become inf or NaN.  The
 * forward's P V product runs on fp16 too (P <= 256, 11-bit rounding), so
 * |v| < 65504 as well.  The backward's fp16 dS operands are scaled by powers
 * of two set from a bound on |dS|, so dO has no such limit.  FP32 runs in
 * fp32 throughout. */
enum ttt_attn_dtype { TTT_DTYPE_BF16 = 0, TTT_DTYPE_FP32 = 1 };

enum ttt_attn_status {
  TTT_OK = 0,
  TTT_ERR_NULL_ARG = 1,       /* a required pointer is NULL                         */
  TTT_ERR_BAD_SHAPE = 2,      /* sizes or strides inconsistent or out of range (also
                                 problems past the kernels' 32-bit workspace offsets:
                                 2 (D-1) slots < 2^31 and 4 B Hq slots < 2^31, slots
                                 ~ tokens per batch rounded up to 64)               */
  TTT_ERR_UNSUPPORTED = 3,    /* head_dim / dtype combination not built             */
  TTT_ERR_MISALIGNED = 4,     /* base pointer or stride not 16-byte aligned         */
  TTT_ERR_WORKSPACE = 5,      /* workspace NULL, too small or not 256-byte aligned  */
  TTT_ERR_HIP = 6,            /* a HIP runtime call failed                          */
  TTT_ERR_ABI = 7             /* descriptor struct_size does not match this library */
};

#define TTT_MAX_PASSES 16

typedef struct ttt_attn_desc {
  uint32_t struct_size;       /* = sizeof(ttt_attn_desc)                                   */
  int32_t layout;             /* ttt_attn_layout                                           */
  int32_t dtype;              /* dtype of q, k, v, dout, dq, dk, dv                        */
  int32_t o_dtype;            /* dtype of o: = dtype, or FP32 with bf16 inputs             */
  int32_t batch;              /* B (BSHD); ignored for THD                                 */
  int32_t seqlen;             /* S (BSHD) or total tokens T (THD)                          */
  int32_t num_seqs;           /* THD: number of packed sequences                           */
  int32_t check_cu_seqlens;   /* THD: non-zero = copy cu_seqlens to the host and validate
                                 (synchronises the stream); zero = trust them, the kernels
                                 then clamp every sequence to [0, T)                       */
  const int32_t* cu_seqlens;  /* THD: device int32 [num_seqs + 1], cu[0] = 0, cu[n] = T,
                                 non-decreasing                                            */
  int32_t num_q_heads;        /* Hq                                                        */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0                                        */
  int32_t head_dim;           /* D: 32, 64 or 128.  bf16 32 / 64 (ttt_attn_fwd / _bwd /
                                 _workspace_bytes only): the D = 128 kernels on zero-
                                 padded copies of the heads in the workspace (entry k <
                                 D/2 at (128/D) k, D/2 + k at 64 + (128/D) k: the same
                                 rotate-half pairs and angles), softmax_scale <= 0 meaning
                                 1/sqrt(D); 2x / 4x the D = 128 MFMA work                  */
  int32_t pass_index;         /* p, 1 .. TTT_MAX_PASSES                                    */
  float softmax_scale;        /* <= 0 selects 1/sqrt(D)                                    */
  float rope_base;            /* RoPE base; 0 disables the rotation                        */
  int64_t q_stride[3];        /* batch, token, head strides of q / dq (elements)           */
  int64_t kv_stride[3];       /* ... of every k, v, dk, dv                                 */
  int64_t o_stride[3];        /* ... of o / dout                                           */
  int32_t window;             /* sliding-window trunk: > 0 limits row i to the pass-1 keys
                                 j with i - window < j <= i (positions, so ring steps too);
                                 0 = full causal trunk; the branch is unchanged.  Same
                                 issue, item 4 (sliding-window layers).  bf16 only      */
  int32_t bwd_mode;           /* ttt_attn_bwd only (0 elsewhere):
                                 TTT_BWD_RECOMPUTE (0): dQ recomputes S and dP (the
                                   smallest workspace; the default).
                                 TTT_BWD_STORED_DS (1): for bf16 BSHD passes without a
                                   window, the dK/dV kernel also stores the trunk dS
                                   (fp16, one power-of-two scale per KV group) in the
                                   workspace and dQ is formed from it, when those blocks
                                   take at most TTT_ATTN_STORED_DS_MAX_BYTES (B * Hq *
                                   n (n + 1) / 2 * 2048 bytes, n = ceil(S / 32));
                                   otherwise as RECOMPUTE.  Fewer matrix products, more
                                   HBM traffic: see the measurements in the docs.
                                 Both are deterministic.                                  */
  void* aux_stream;           /* ttt_attn_bwd / ttt_attn_bwd_chunk, bf16 (ignored elsewhere):
                                 an optional second stream of the caller's (a
                                 hipStream_t, NULL = none, different from `stream`).
                                 When given, the HBM-bound Delta and branch-gradient
                                 kernels run on it beside the staging and dK/dV kernels,
                                 ordered against `stream` with events and joined back
                                 into `stream` before the call returns; results are the
                                 same either way.  Two calls in flight at once must not
                                 share an aux stream.                                     */
} ttt_attn_desc;

enum ttt_attn_bwd_mode { TTT_BWD_RECOMPUTE = 0, TTT_BWD_STORED_DS = 1 };
#define TTT_ATTN_STORED_DS_MAX_BYTES ((size_t)40 << 30)

/* Bytes of caller-provided device workspace a forward (for_bwd = 0) or
 * backward (for_bwd = 1) call with this descriptor needs.  Returns 0 and sets
 * the last error if the descriptor is invalid (a valid call may also need 0). */
size_t ttt_attn_workspace_bytes(const ttt_attn_desc* d, int for_bwd);

/* Forward of pass p.
 *   q            : device, pass-p queries (pre-RoPE)
 *   k, v         : HOST arrays of p device pointers, pass 1 .. p keys/values (pre-RoPE)
 *   o            : device output, o_dtype
 *   lse          : device output, fp32 natural-log LSE of the merged softmax
 *   ws, ws_bytes : device workspace of at least ttt_attn_workspace_bytes(d, 0)
 * Returns a ttt_attn_status. */
int ttt_attn_fwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v,
                 void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Forward of pass p without a workspace argument and without allocating: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments and
 * results as ttt_attn_fwd.  The workspace is a static device array of
 * TTT_ATTN_NOALLOC_SCRATCH_BYTES per GPU, held from this entry point's first
 * call on that GPU until the process ends; a call whose workspace need
 * (ttt_attn_workspace_bytes(d, 0)) exceeds it returns TTT_ERR_WORKSPACE before
 * any launch.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and give undefined
 * results; calls in order on one stream are fine.  The array keeps the last
 * call's contents, and the forward writes every byte of it that it reads, so
 * nothing is cleared between calls.  THD's check_cu_seqlens (a host copy and
 * a synchronisation) is rejected with TTT_ERR_UNSUPPORTED. */
#define TTT_ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int ttt_attn_fwd_noalloc(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v,
                         void* o, float* lse, void* stream);

/* Backward of pass p, recomputing probabilities from the forward's LSE.
 *   o, lse       : the forward's outputs for the same inputs
 *   dout         : gradient of o (dtype, o_stride)
 *   dq           : device output, gradient of q
 *   dk, dv       : HOST arrays of p device pointers, gradients of k[0..p-1], v[0..p-1]
 *   ws, ws_bytes : device workspace of at least ttt_attn_workspace_bytes(d, 1)
 * LSE is an auxiliary output: no gradient flows into it.  Returns a ttt_attn_status. */
int ttt_attn_bwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v,
                 const void* o, const float* lse, const void* dout, void* dq, void* const* dk,
                 void* const* dv, void* ws, size_t ws_bytes, void* stream);

/* ---- Ring steps: the pass-1 trunk in chunks ---------------------------------
 * NeMo-RL issue "DFlash/DSpark and EAGLE-3 TTT draft co-training for
 * speculative decoding (Megatron backend)", "What I'm working on", item 4:
 * under context parallelism the pass-1 trunk K/V of a sequence travels on a
 * (zig-zag) ring and the partial results are joined by the exact joint-LSE
 * merge.  One ring step is the attention of a chunk of query rows against a
 * chunk of pass-1 keys, at their positions in the sequence:
 *   query row i of q (i < d->seqlen) sits at position q_offset + i (RoPE
 *   position q_offset + i + p - 1); pass-1 key j of k[0]/v[0] (j < kv_len) at
 *   position kv_offset + j; key j is visible to row i iff
 *   kv_offset + j <= q_offset + i.
 *   with_branch != 0 also folds in the branch keys of passes 2..p, which k[q],
 *   v[q] (q >= 1) hold for the query rows (d->seqlen rows, positions
 *   q_offset + i + q); a sequence's ring folds them in exactly once.
 * Output: O normalised over the keys this step sees and its LSE; a row that
 * sees no key gets O = 0 and LSE = -inf.  dtype bf16 only.
 * BSHD: every batch row uses the same offsets (q_offset, kv_offset); the
 * THD fields below are NULL / 0.
 * THD (packed sequences, d->cu_seqlens): every sequence s takes its own ring
 * step.  Its query rows cu_seqlens[s] .. cu_seqlens[s+1] of q sit at
 * positions q_offsets[s] + i, its pass-1 key rows kv_cu_seqlens[s] ..
 * kv_cu_seqlens[s+1] of k[0] / v[0] at kv_offsets[s] + j (same visibility
 * rule); sequences never see each other.  q_offset = kv_offset = 0, kv_len =
 * kv_cu_seqlens[num_seqs] (the packed key rows), and every position the call
 * touches (q_offsets[s] + rows + p - 1, kv_offsets[s] + keys) must be below
 * max_position, which sizes the RoPE table (positions past it get the angles
 * of max_position - 1: wrong values, never an access outside the table).
 * The three arrays are device int32 arrays the kernels read; the host reads
 * kv_cu_seqlens only with d->check_cu_seqlens (then it must start at 0, not
 * decrease and end at kv_len). */
typedef struct ttt_attn_chunk {
  uint32_t struct_size;       /* = sizeof(ttt_attn_chunk)                                  */
  int32_t with_branch;        /* non-zero: fold in the branch keys of passes 2..p         */
  int64_t q_offset;           /* BSHD: position of query row 0 in the sequence            */
  int64_t kv_offset;          /* BSHD: position of pass-1 key 0 in the sequence           */
  int64_t kv_len;             /* rows of k[0] / v[0] (THD: packed rows of every sequence) */
  int64_t kv0_stride[3];      /* batch, token, head strides of k[0] / v[0] (elements); a
                                 zero triple selects the contiguous default [B, kv_len,
                                 Hkv, D] ([kv_len, Hkv, D] in THD); kv_stride applies to
                                 k[q], v[q], q >= 1                                        */
  const int32_t* q_offsets;     /* THD: device [num_seqs], query row 0's position per sequence */
  const int32_t* kv_offsets;    /* THD: device [num_seqs], pass-1 key 0's position           */
  const int32_t* kv_cu_seqlens; /* THD: device [num_seqs + 1], packed pass-1 key rows        */
  int64_t max_position;         /* THD: bound on every position of the call (>= 1)          */
} ttt_attn_chunk;

/* Bytes of workspace ttt_attn_fwd_chunk needs (0 and the last error if invalid). */
size_t ttt_attn_chunk_workspace_bytes(const ttt_attn_desc* d, const ttt_attn_chunk* c);

/* Forward of one ring step; arguments as ttt_attn_fwd, plus the chunk. */
int ttt_attn_fwd_chunk(const ttt_attn_desc* d, const ttt_attn_chunk* c, const void* q, const void* const* k,
                       const void* const* v, void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward of one ring step (the backward ring also carries dK/dV): the
 * chain-rule terms of this step's keys, given the rows' FINAL outputs.
 *   o, lse, dout : the query rows' merged O (o_dtype, o_stride), merged LSE
 *                  (dense fp32 [B][Hq][seqlen] for these rows) and dO (o_stride)
 *                  over the whole sequence (the ring's forward result)
 *   dq           : fp32, q's element strides: this step's terms of dQ
 *   dk, dv       : HOST arrays of fp32 device pointers: dk[0] / dv[0] the terms
 *                  of the step's pass-1 keys (kv0 strides); with with_branch,
 *                  dk[q] / dv[q] (q >= 1) the branch keys' gradients of the rows
 *                  (kv_stride)
 * Outputs are overwritten (not accumulated); summing every step's terms gives
 * the whole-sequence gradients.  BSHD or THD (as for the forward), bf16
 * inputs; in THD, pass-1 keys of a sequence without query rows get zero
 * terms, and the LSE is [Hq][total query rows].  Workspace:
 * ttt_attn_chunk_bwd_workspace_bytes. */
size_t ttt_attn_chunk_bwd_workspace_bytes(const ttt_attn_desc* d, const ttt_attn_chunk* c);
int ttt_attn_bwd_chunk(const ttt_attn_desc* d, const ttt_attn_chunk* c, const void* q, const void* const* k,
                       const void* const* v, const void* o, const float* lse, const void* dout, float* dq,
                       float* const* dk, float* const* dv, void* ws, size_t ws_bytes, void* stream);

/* Joint-LSE merge of two partial results over disjoint key sets of the same
 * rows (same issue and item as above; the operator that also joins trunk and
 * branch):  LSE = ln(e^LSE_a + e^LSE_b),  O = e^(LSE_a-LSE) O_a + e^(LSE_b-LSE) O_b;
 * a row with LSE_a = LSE_b = -inf gets O = 0, LSE = -inf.  Shapes, strides and
 * o_dtype from d (BSHD or THD; o_stride for every O, lse layout as in
 * ttt_attn_fwd).  o/lse may alias o_a/lse_a or o_b/lse_b (in-place
 * accumulation).  An fp32 o_dtype keeps a long ring exact to fp32 rounding. */
int ttt_attn_merge(const ttt_attn_desc* d, const void* o_a, const float* lse_a, const void* o_b,
                   const float* lse_b, void* o, float* lse, void* stream);

/* ---- Block drafting: anchor + mask-token blocks ----------------------------
 * Same issue, "What I'm working on", item 2: block drafters predict a block of
 * tokens at once from an anchor followed by mask tokens; attention is
 * bidirectional inside the block and the trunk (context) is cut at the
 * anchor.  Reading taken here (the pages leave the exact mask open): block n
 * of batch row b has bs slots and anchor a = anchors[b * nblk + n] (clamped
 * to [0, ctx_len]); slot t is the token at position a + t (slot 0 is the
 * anchor, 1.. the mask tokens); every slot of the block sees the context keys
 * at positions j < a and all bs keys of its own block.  RoPE (rotate-half)
 * at those positions, as in ttt_attn_fwd.
 * The descriptor gives the block rows: dtype BF16, pass_index 1, q_stride
 * for q, kv_stride for k_blk / v_blk, o_stride, softmax_scale, rope_base.
 * BSHD: seqlen = nblk * bs rows per batch row (row i = slot i % bs of block
 * i / bs), k_blk / v_blk [B, seqlen, Hkv, D], output O [B, seqlen, Hq, D]
 * and LSE [B, Hq, seqlen] as in ttt_attn_fwd; ctx_cu_seqlens is NULL.
 * THD (same issue, item 4: the block-draft attention on the packed layout):
 * sequence s holds block rows cu_seqlens[s] .. cu_seqlens[s+1] of q / k_blk
 * / v_blk [T, H, D] (whole blocks: every cu_seqlens entry is a multiple of
 * bs) and context rows ctx_cu_seqlens[s] .. ctx_cu_seqlens[s+1] of k_ctx /
 * v_ctx [ctx_len, Hkv, D] (ctx_len = all sequences' context rows); anchors
 * has one entry per block in packed order (T / bs) and clamps to the
 * sequence's own context length; O [T, Hq, D], LSE [Hq, T].  Sequences
 * never see each other.  With d->check_cu_seqlens the host checks both
 * arrays (start 0, non-decreasing, totals T and ctx_len, whole blocks). */
typedef struct ttt_attn_block {
  uint32_t struct_size;       /* = sizeof(ttt_attn_block)                                 */
  int32_t block_size;         /* bs: 1, 2, 4, 8, 16 or 32                                 */
  int64_t ctx_len;            /* context rows of k_ctx / v_ctx (THD: of every sequence)   */
  const int32_t* anchors;     /* device int32 [B][seqlen / bs] (THD: [T / bs]), read-only;
                                 values outside [0, the context length] are clamped       */
  int64_t ctx_stride[3];      /* batch, token, head strides of k_ctx / v_ctx (elements); a
                                 zero triple selects the contiguous [B, ctx_len, Hkv, D]
                                 ([ctx_len, Hkv, D] in THD)                                */
  const int32_t* ctx_cu_seqlens; /* THD: device int32 [num_seqs + 1], the contexts' rows;
                                 BSHD: NULL                                                */
} ttt_attn_block;

/* Bytes of workspace ttt_attn_block_fwd (for_bwd = 0) or ttt_attn_block_bwd
 * (for_bwd != 0) needs (0 and the last error if invalid). */
size_t ttt_attn_block_workspace_bytes(const ttt_attn_desc* d, const ttt_attn_block* blk, int for_bwd);

/* Forward of block-draft attention.  q [B, seqlen, Hq, D]; k_ctx, v_ctx the
 * context keys/values (may be NULL when ctx_len = 0); k_blk, v_blk the block
 * keys/values; o, lse outputs; ws, ws_bytes workspace as for ttt_attn_fwd.
 * Checked on the host before any launch (same status codes); the anchors are
 * not read on the host.  Returns a ttt_attn_status. */
int ttt_attn_block_fwd(const ttt_attn_desc* d, const ttt_attn_block* blk, const void* q, const void* k_ctx,
                       const void* v_ctx, const void* k_blk, const void* v_blk, void* o, float* lse, void* ws,
                       size_t ws_bytes, void* stream);

/* Backward of block-draft attention, recomputing probabilities from the
 * forward's LSE (no gradient flows into LSE).  o, lse: the forward's outputs;
 * dout: gradient of o (o's dtype and strides).  Outputs (overwritten): dq
 * (q's strides), dk_ctx / dv_ctx (ctx_stride; GQA: summed over the heads of
 * a group; may be NULL when ctx_len = 0), dk_blk / dv_blk (kv_stride).
 * Any anchor order; the workspace is ttt_attn_block_workspace_bytes(d, blk, 1). */
int ttt_attn_block_bwd(const ttt_attn_desc* d, const ttt_attn_block* blk, const void* q, const void* k_ctx,
                       const void* v_ctx, const void* k_blk, const void* v_blk, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk_ctx, void* dv_ctx, void* dk_blk, void* dv_blk, void* ws,
                       size_t ws_bytes, void* stream);

/* ---- Distillation loss after the attention ---------------------------------
 * Same issue, "What I'm working on", item 3 (chunked soft cross-entropy,
 * normalised per pass over the whole batch) and NeMo-RL PR #3725, self-review
 * comment (teacher_offset = pass_index + 1).  Reading: pass p's student logits
 * at row i are scored against softmax(teacher logits at row i + teacher_offset)
 * of the same batch row, teacher_offset = p for 1-based p; a row is counted iff
 * that teacher row exists (i + teacher_offset < seqlen) and mask[b][i] != 0;
 * loss = sum over counted rows of -sum_v softmax(teacher)_v log softmax(student)_v
 * divided by the number of counted rows (0 if none).  bf16 logits [B][S][V],
 * vocab contiguous; V a multiple of 8; row strides multiples of 8 elements. */
typedef struct ttt_soft_ce_desc {
  uint32_t struct_size;       /* = sizeof(ttt_soft_ce_desc)                               */
  int32_t batch, seqlen, vocab;
  int32_t teacher_offset;     /* >= 0; row i is scored against teacher row i + offset
                                 unless teacher_rows is given                             */
  int32_t teacher_seqlen;     /* teacher rows per batch; 0 = seqlen                       */
  int64_t student_stride[2];  /* batch, row strides of the student logits (elements); a
                                 zero pair selects the contiguous [B, S, V]; the gradient
                                 uses the same strides                                    */
  int64_t teacher_stride[2];  /* the same for the teacher logits ([B, teacher_seqlen, V]) */
  const uint8_t* mask;        /* device [B][S] (row counted iff != 0) or NULL             */
  const int32_t* teacher_rows;/* device [B][S] or NULL: the teacher row of each student
                                 row; outside [0, teacher_seqlen) = row not counted.  A
                                 block-draft slot at position a + t takes row a + t + 1
                                 (same issue, item 3: per-slot normalisation)             */
  const int32_t* groups;      /* device [B][S] or NULL: normalisation group of each row
                                 (e.g. the block slot index); outside [0, num_groups) =
                                 not counted; NULL = every row in group 0                 */
  int32_t num_groups;         /* 1 .. 64 (0 = 1)                                          */
  int32_t reserved;           /* 0                                                        */
} ttt_soft_ce_desc;

/* Bytes of workspace ttt_soft_ce_fwd needs when its row_ce argument is NULL (it then
 * keeps the rows' cross-entropies there): B * S floats, rounded up to 256.  0 and the
 * last error if the descriptor is invalid. */
size_t ttt_soft_ce_workspace_bytes(const ttt_soft_ce_desc* d);

/* Forward: stats (device float[2 + 2 G], G = num_groups): stats[0] = loss = the sum
 * over groups of each group's mean cross-entropy over its counted rows (one group:
 * the mean over counted rows), stats[1] = counted rows, stats[2 + 2g] and
 * stats[3 + 2g] = group g's mean and count; row_lse [B][S][2] (device fp32):
 * natural-log LSE of the student and teacher rows, needed by the backward; row_ce
 * [B][S] (device fp32, optional): each counted row's cross-entropy, 0 elsewhere (when
 * NULL the workspace holds it).  Deterministic (fixed-order sums). */
int ttt_soft_ce_fwd(const ttt_soft_ce_desc* d, const void* student, const void* teacher, float* stats,
                    float* row_lse, float* row_ce, void* ws, size_t ws_bytes, void* stream);

/* Backward: dstudent = dloss[g] / count_g * (softmax(student) - softmax(the row's
 * teacher row)) on counted rows of group g, 0 on the others (bf16, student strides).
 * row_lse and stats come from ttt_soft_ce_fwd; dloss is device float[G], the upstream
 * gradient of each group's mean (all equal for the gradient of stats[0]; a weighted
 * sum of the group losses passes its weights).  No gradient for the teacher. */
int ttt_soft_ce_bwd(const ttt_soft_ce_desc* d, const void* student, const void* teacher, const float* row_lse,
                    const float* stats, const float* dloss, void* dstudent, void* stream);

/* Static text of a status code. */
const char* ttt_attn_status_string(int status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* ttt_attn_last_error(void);

/* TTT_ATTN_ABI_VERSION of the loaded library. */
int ttt_attn_abi_version(void);

/* Launch trace hook, a profiling aid outside the method.  When set (per host
 * thread), every kernel that a later ttt_attn_fwd / ttt_attn_bwd call on this
 * thread enqueues is bracketed by fn(user, name, 0, stream) just before and
 * fn(user, name, 1, stream) just after its launch, on the calling thread, so a
 * caller can record HIP events around single kernels.  `name` is a static
 * string.  fn = NULL removes the hook.  Never fails. */
typedef void (*ttt_attn_trace_fn)(void* user, const char* kernel, int phase, void* stream);
void ttt_attn_set_trace_hook(ttt_attn_trace_fn fn, void* user);

#ifdef __cplusplus
}
#endif

#endif /* TTTATTN_H */
