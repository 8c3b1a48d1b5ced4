// Launcher declarations of libtttattn's kernels (host side).
#pragma once

#include "common.hpp"

namespace ttt {

void launch_rope_table(const Prob& P, float* cosT, float* sinT, double base, hipStream_t st);
void launch_prep_rot_f32(const Prob& P, const float* x, int64_t sb, int64_t st_, int64_t sh, int H, int pos_off,
                         const float* cosT, const float* sinT, float* out_row, hipStream_t st);
// One staging job of the bf16 prologue (D = 128): the tensor x (element
// strides sb, st, sh; H heads) into fp16 rows, rotated at row + pos_off when
// rot, and/or a transposed copy (bf16 when col_bf16, else fp16).
// pos_anchor: rotate at the block-slot position of the row (block_anchor of
// the Prob plus the slot index) instead of row + pos_off.
struct PrepJob {
  const uint16_t* x;
  int64_t sb, st, sh;
  int H, pos_off, rot, col_bf16;
  _Float16* out_row;
  uint16_t* out_col;
  int pos_anchor;
  int* out_lim;  // pos_anchor jobs: per slot [(b)][spad] the clamped anchor of the row's block (0 past the end)
  int rows;      // BSHD: rows of this tensor when they differ from the Prob's (0: P.stok, < 0: none)
  const int* cu; // THD: this tensor's own cu_seqlens (ntok rows) on the Prob's slots, or null (the Prob's)
  int ntok;
  const int* seg_pos;  // THD: per-sequence position offset added to every row's, or null
};
struct PrepJobs {
  PrepJob j[2];
  int n;
  int heads_fast;  // grid order: heads of one 64-slot tile side by side (row-major outputs) instead of tiles of one head
};
void launch_prep_bf16(const Prob& P, const PrepJobs& J, const float* cosT, const float* sinT, hipStream_t st);
// Delta (and, with lse, the LSE in log2 units right after it, +inf past the
// rows' ends) in the workspace slot layout.  v: the trunk V (bf16, P.cs_*
// strides), read only when P.vpart is set.
void launch_delta(const Prob& P, const void* o, bool o_f32, const void* dout, bool g_f32, const float* lse,
                  float* delta, const void* v, hipStream_t st);
// bf16 backward: P.dmax[B*Hkv][2] from the Delta kernel's P.dpart entries (and
// P.vgmax from P.vpart when set)
void launch_dmax(const Prob& P, hipStream_t st);
// bf16 head_dim 32 / 64 on the D = 128 kernels: zero-padded heads (see prep.hip)
void launch_pad_heads(const void* src, bool f32, int64_t sb, int64_t st, int64_t sh, int64_t rows, int S, int H,
                      int D, void* dst, hipStream_t stream);
void launch_unpad_heads(const void* src, bool f32, int64_t rows, int S, int H, int D, void* dst, int64_t sb,
                        int64_t st, int64_t sh, hipStream_t stream);
// THD: workspace slots (when slot_base is given) and the sequence-major tile
// list (when out is given); desc: tiles descending within a sequence.
void launch_tile_sched(const Prob& P, int tile, int desc, int4* out, int max_entries, int* slot_base,
                       hipStream_t st);

// fp32 path (VALU)
void launch_fwd_f32(const Prob& P, const float* q, const PassPtrs& kv, const float* kt, const float* cosT,
                    const float* sinT, float* o, float* lse, hipStream_t st);
void launch_bwd_f32(const Prob& P, const PassPtrs& kv, const float* lse, const float* dout, const float* kt,
                    const float* qt, const float* delta, const float* cosT, const float* sinT, float* dq,
                    const PassGradPtrs& g, hipStream_t st);

// bf16 path (MFMA trunk + shuffle-reduction branch)
int fwd_tile_rows(int r);        // rows per forward work item (TTT passes; THD tile lists)
int block_fwd_tile_rows(int r);  // the same for block drafting
// Block-draft forward (BSHD, D = 128): context K~ / V^T in kt / vt (P.spad
// slots), block K~ / V^T in kbt / vbt (P.spad_b slots); P.anchors, P.bs_log2,
// P.nblk, P.kv_len (context rows) describe the blocks.
// Block-draft backward (BSHD, D = 128; P as for the forward, P.ks_* the
// block K/V strides, P.cs_* the context ones).  dK/dV of the context keys
// (ctx_keys, kt = context K~ slab, v = context V) or of the block keys (kt =
// block K~ slab, v = block V); P.ks_* must then be the strides of v/dk/dv.
void launch_block_dkdv_bf16(const Prob& P, bool ctx_keys, const uint16_t* v, const float* lse, const uint16_t* dout,
                            const _Float16* kt, const _Float16* qt, const float* delta, const int4* tiles,
                            const float* cosT, const float* sinT, void* dk, void* dv, hipStream_t st);
// dQ: context keys (ckt, cktt, v_ctx) up to each row's anchor, then its block's keys (bkt, bktt, v_blk).
void launch_block_dq_bf16(const Prob& P, const uint16_t* v_ctx, const uint16_t* v_blk, const float* lse,
                          const uint16_t* dout, const _Float16* ckt, const _Float16* cktt, const _Float16* bkt,
                          const _Float16* bktt, const _Float16* qt, const float* delta, const int4* tiles,
                          const float* cosT, const float* sinT, uint16_t* dq, hipStream_t st);
// Per-pass soft cross-entropy (bf16 logits [B][S][V], vocab contiguous, V % 8 == 0).
struct CeProb {
  int B, S, V, offset;
  int T;                 // teacher rows per batch
  const uint8_t* mask;   // [B][S] or null
  const int* trows;      // [B][S] teacher row of each student row, or null (row + offset)
  const int* groups;     // [B][S] normalisation group, or null (group 0)
  int G;                 // groups, 1..64
  int64_t ss_b, ss_t, ts_b, ts_t;
};
// row_lse [B*S][2] (student, teacher), row_ce [B*S], stats [2 + 2G] = (loss, counted rows,
// then each group's (mean, count)); dloss [G]
void launch_soft_ce_fwd(const CeProb& C, const uint16_t* s, const uint16_t* t, float* row_lse, float* row_ce,
                        float* stats, hipStream_t st);
void launch_soft_ce_bwd(const CeProb& C, const uint16_t* s, const uint16_t* t, const float* row_lse,
                        const float* stats, const float* dloss, uint16_t* g, hipStream_t st);
void launch_block_fwd_bf16(const Prob& P, const uint16_t* q, const _Float16* kt, const _Float16* vt,
                           const _Float16* kbt, const _Float16* vbt, const int4* tiles, const float* cosT,
                           const float* sinT, void* o, bool o_f32, float* lse, hipStream_t st);     // query rows per forward work item for GQA ratio r (32, 64 or 128)
constexpr int kFwdMinRows = 32;
int dq_tile_rows(int r);
// whether the dQ kernel's work item holds every query head of a KV group, so
// that it can also produce the branch dK/dV (Prob::dq_branch)
bool dq_fuses_branch(int r);      // query rows per dQ work item for GQA ratio r (32, 64 or 128)
constexpr int kBwdBKV = 128;  // key rows per dK/dV workgroup
void launch_fwd_bf16(const Prob& P, const uint16_t* q, const PassPtrs& kv, const _Float16* kt, const _Float16* vt,
                     const int4* tiles, const float* cosT, const float* sinT, void* o, bool o_f32, float* lse,
                     hipStream_t st);
void launch_dkdv_bf16(const Prob& P, const PassPtrs& kv, const float* lse, const uint16_t* dout, const _Float16* kt,
                      const _Float16* qt, const float* delta, const int4* tiles_kv, const float* cosT,
                      const float* sinT, const PassGradPtrs& g, hipStream_t st);
void launch_dq_bf16(const Prob& P, const uint16_t* q, const PassPtrs& kv, const float* lse, const uint16_t* dout,
                    const _Float16* kt, const _Float16* ktt, const _Float16* qt, const float* delta,
                    const int4* tiles_q, const float* cosT, const float* sinT, uint16_t* dq, const PassGradPtrs& g,
                    hipStream_t st);
void launch_branch_bwd_bf16(const Prob& P, const uint16_t* q, const PassPtrs& kv, const float* lse,
                            const uint16_t* dout, const float* delta, const float* cosT, const float* sinT,
                            const PassGradPtrs& g, hipStream_t st);

// joint-LSE merge of two partial (O, LSE) over disjoint key sets (prep.hip)
void launch_merge(const Prob& P, bool o_f32, const void* o_a, const float* lse_a, const void* o_b,
                  const float* lse_b, void* o, float* lse, hipStream_t st);

// launch trace hook (host.hip)
void trace(const char* name, int phase, hipStream_t st);

}  // namespace ttt
