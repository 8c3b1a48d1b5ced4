// bf16 forward: trunk flash attention on MFMA, continued over the branch keys,
// so the joint log-sum-exp merge of the two partial softmaxes is exact.
//
// Method (NeMo-RL issue "DFlash/DSpark and EAGLE-3 TTT draft co-training for
// speculative decoding (Megatron backend)", "What I'm working on", item 1;
// NeMo-RL PR #3725, Summary and self-review comment): at pass p, query row i
// (position i+p-1) attends causally to the pass-1 keys j <= i (trunk) and to
// the keys passes 2..p produced at row i (branch, position i+q-1).  No score
// matrix or mask is ever stored.  The online softmax state (running max m,
// sum l, unnormalised O) after the trunk is the trunk partial; folding the
// branch keys into the same state is the joint-LSE merge
// LSE = logaddexp(LSE_trunk, LSE_branch), O = sum_x e^(LSE_x - LSE) O_x.
//
// gfx950 design
// * A workgroup is NW wave64s: the R' query heads of one KV head that it
//   covers (R' = 4 for GQA 4:1) times 32*NW/R' rows.  With R' = 4 the TTT
//   passes run NW = 8 (4 heads x 64 rows, one workgroup of two waves per SIMD
//   per CU: every K~/V^T tile staged in LDS serves twice the rows of the
//   4-wave shape, which the other modes and head ratios keep).
// * Scores are computed transposed, S^T = K~ Q~^T, with
//   v_mfma_f32_32x32x16_f16: each lane then holds 16 keys of ONE query, so the
//   running max/sum are per-lane scalars (one cross-half exchange per tile)
//   and the O rescale needs no broadcast.  K~ rows for the A operand are read
//   in a permuted order (bits 2 and 3 of the row index swapped) so that the
//   score accumulator is already the B operand of O^T = V^T P^T
//   (v_mfma_f32_32x32x16_f16: P <= 2^8 and V in fp16, so the row sum of the
//   rounded P that normalises O is 8x finer than with bf16 P).
// * Q~ = R(i+p-1) q is rotated in fp32 once and kept in VGPRs as fp16 (bf16
//   inputs are exact in fp16 up to 65504; the rotated values round 8x finer
//   than in bf16).  K~ = R(j) k^(1) (fp16) and V^(1)^T (fp16) come from the
//   prologue, so the hot loop is copies and MFMAs.
// * K~ and V^T tiles of 64 keys move HBM -> LDS with buffer_load_dwordx4 ... lds
//   (no VGPR staging), double-buffered, XOR-swizzled 16-byte chunks so that
//   the MFMA operand reads are bank-conflict free; one barrier per tile; the
//   operand reads run three ahead of their MFMAs.
// * Softmax in the log2 domain with one FMA per score; the running max only
//   moves when a score exceeds it by 2^8 (P <= 256), and the 64-register O
//   rescale is skipped wave-wide otherwise.  Only diagonal tiles are masked.
// * Branch: for q = 2..p the workgroup stages R(i+q-1) k^(q) (fp16) and
//   v^(q) (bf16) of its rows in LDS once for all its heads; each lane dots
//   its fp16 Q~ fragment with packed v_dot2_f32_f16, exchanges halves once,
//   and updates (m, l, O) in the MFMA accumulator layout.
// * Epilogue: O / l through LDS to 16-byte row-major stores; LSE = (m + log2 l) ln 2.
#include <type_traits>

#include "kernels.hpp"

namespace ttt {

namespace fwd {

constexpr int D = 128;
constexpr int BN = 64;  // keys per tile
constexpr int OPAD = D + 4;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

constexpr int NBUF = 2;          // tiles in the LDS ring (loads run NBUF-1 tiles ahead)
constexpr int CH = BN / 8;         // 16-byte chunks per V^T d-row
struct Tile {
  _Float16 k[BN * D];  // K~ tile: row r at r*D, 16-byte chunk c at slot c ^ (r & 15)
  _Float16 v[D * BN];  // V^T tile (fp16): d-row at d*BN, chunk c at slot c ^ ((d >> 1) & (CH - 1))
};
constexpr int QST_ROWS = 64, QST_PITCH = 1024 + 16;
template <int NW>
struct Smem {
  union {
    Tile ring[NBUF];
    struct {
      _Float16 k[128][D + 8];  // branch keys R(i+q-1) k^(q), fp16, per row of the tile
      uint16_t v[128][D + 8];  // branch values, bf16
    } br;
    float o[32 * NW][OPAD];    // normalised O rows for the stores (32 per wave)
    struct {  // 8-wave work items: Q rows and angles staged beside the first tile (4 waves: unused)
      unsigned char first_tile[NW == 8 ? sizeof(Tile) : 16];
      unsigned char q[NW == 8 ? QST_ROWS * QST_PITCH : 16];      // token rows: 4 heads' 1 KB, 16-byte pad
      unsigned char c[NW == 8 ? QST_ROWS / 4 * QST_PITCH : 16];  // cos rows, 4 positions per padded 1 KB
      unsigned char s[NW == 8 ? QST_ROWS / 4 * QST_PITCH : 16];  // sin rows
    } qst;
  };
};
constexpr int kFwdWaves = 8;  // TTT passes at GQA 4:1: waves per work item (4 or 8)

__device__ __forceinline__ int perm_row(int a) { return (a & ~0xC) | ((a & 4) << 1) | ((a & 8) >> 1); }

// Rows of one work item, per R' (heads per workgroup).
__host__ __device__ constexpr int tile_rows(int heads_per_wg, int nw = 4) { return 32 * nw / heads_per_wg; }

// MODE 0: TTT pass (trunk + branch); MODE 4: the same with a sliding-window
// trunk (a separate instantiation, so the windowless loop carries no window
// test).  MODE 1: block drafting -- the trunk is
// the context prefix j < anchor of each row's block (kt/vt), then the keys of
// the work item's own blocks (kbt/vbt) in one more masked tile pass.
template <int RH, bool O_F32, int MODE, int NW = 4>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
    fwd_bf16_kernel(Prob P, const uint16_t* __restrict__ q, PassPtrs kv, const _Float16* __restrict__ kt,
                    const _Float16* __restrict__ vt, const int4* __restrict__ tiles, const float* __restrict__ cosT,
                    const float* __restrict__ sinT, void* __restrict__ o, float* __restrict__ lse,
                    const _Float16* __restrict__ kbt, const _Float16* __restrict__ vbt) {
  constexpr int RT = tile_rows(RH, NW);  // rows per work item
  __shared__ __attribute__((aligned(16))) Smem<NW> sm;
  constexpr bool TTT_ = MODE == 0 || MODE == 4;  // TTT pass (4: with a sliding window)
  const int win = MODE == 4 ? P.win : 0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- work item: heavy-first over (row tile), then (batch, KV head, head sub-group)
  const int nsub = P.r / RH;
  const int sub = blockIdx.x % nsub, rest = blockIdx.x / nsub;
  const int g = rest % P.Hkv, tix = rest / P.Hkv;
  int b, t, start, L, slot0;
  if (P.layout == 0) {
    const int nqt = (P.stok + RT - 1) / RT;
    if (tix >= P.B * nqt) return;
    t = nqt - 1 - tix / P.B;
    b = tix % P.B;
    start = 0;
    L = P.stok;
    slot0 = 0;
  } else {
    if (tix >= tiles[0].x) return;
    const int4 e = tiles[1 + tix];
    t = e.x, start = e.y, L = e.z, slot0 = e.w, b = 0;
  }
  // Ring geometry: row i sits at position qoff + i and sees pass-1 key j
  // (j < kv_len, staged at the work item's slots) iff j <= i + dq_; for
  // whole-sequence calls qoff = dq_ = 0 and kv_len = L.
  int qoff = 0, dq_ = 0, kvs_ = 0, kv_len = 0;
  if constexpr (TTT_)
    seq_ring(P, (P.layout == 1 && P.kv_cu) ? seq_at(P.cu, P.nseq, start) : b, start, L, qoff, dq_, kvs_, kv_len);
  (void)kvs_;
  BlkSeq bq{};  // block drafting: the sequence's anchors and context
  if constexpr (MODE == 1) bq = blk_seq(P, b, start);
  const int hw = wv % RH, rbk = wv / RH;
  const int h = g * P.r + sub * RH + hw;
  const int row0 = t * RT;
  const int wave_row0 = row0 + rbk * 32;
  const int my_row = wave_row0 + l32;  // this lane's query row (B/C column)

  // ---- trunk main loop
  const int qend = min(row0 + RT, L);
  // Block drafting: row i sees context keys j < lim (its block's anchor); the
  // work item's extent is the largest lim of its blocks, a wave's unmasked
  // prefix the smallest lim of the wave's blocks (loops are uniform).
  int lim = 0, lim_hi = 0, lim_lo = 0;
  if constexpr (MODE == 1) {
    lim = my_row < L ? blk_anchor(P, bq, my_row) : 0;
    const int wend = min(wave_row0 + 32, L);
    lim_lo = wend > wave_row0 ? bq.cn : 0;
    for (int blk = row0 >> P.bs_log2; (blk << P.bs_log2) < qend; ++blk) {
      const int a = blk_anchor(P, bq, blk << P.bs_log2);
      lim_hi = max(lim_hi, a);
      if ((blk << P.bs_log2) < wend && ((blk + 1) << P.bs_log2) > wave_row0) lim_lo = min(lim_lo, a);
    }
  }
  const int kmax = TTT_ ? min(qend - 1 + dq_, kv_len - 1) : lim_hi - 1;  // last key any row sees
  const int nkt = kmax < 0 ? 0 : kmax / BN + 1;
  // sliding window: the first tile any row of the work item sees
  const int kt_lo = (TTT_ && win > 0) ? max(0, row0 + dq_ - win + 1) / BN : 0;
  const _Float16* kbase = kt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0) * D;
  // V^T slabs come in 32-key tiles of D x 32 (a 64-key tile: two adjacent ones, 16 KB)
  const _Float16* vbase = vt + (int64_t)(b * P.Hkv + g) * D * P.spad + (int64_t)(slot0 >> 5) * D * 32;
  // DMA lane roles, loads n = w*KL + i.  K~: 1 KB = rows 4n + lane/16, slot
  // lane%16.  V^T: 1 KB = d-rows RPL*n + lane/CH, slot lane%CH.  Per-lane 32-bit
  // offsets, tile bases are wave-uniform.
  constexpr int KL = BN / 4 / NW;    // K~ loads per wave per tile
  constexpr int RPL = 64 / CH;       // V^T d-rows per load
  constexpr int VL = D / RPL / NW;   // V^T loads per wave per tile
  constexpr int TL = KL + VL;        // loads per wave per tile
  uint32_t koff[KL], voff[VL];
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    const int r = 4 * (wv * KL + i) + (lane >> 4);
    koff[i] = (uint32_t)(r * D + ((lane & 15) ^ (r & 15)) * 8);
  }
#pragma unroll
  for (int i = 0; i < VL; ++i) {
    const int d = RPL * (wv * VL + i) + lane / CH;
    const int c = (lane % CH) ^ ((d >> 1) & (CH - 1));  // the 8-key chunk landing in this lane's LDS slot
    voff[i] = (uint32_t)((((c >> 2) * D) + d) * 32 + (c & 3) * 8);
  }
  // a tile's K~ rows are BN*D contiguous halves, and so is its V^T (two 32-key pieces)
  const uint32_t vt_bytes = (uint32_t)(BN * D * 2);
  auto dma_from = [&](Tile* __restrict__ dst, const _Float16* kb_t, const _Float16* vb_t)
                      __attribute__((always_inline)) {
    const buf_rsrc kr = make_rsrc(kb_t, BN * D * 2), vr = make_rsrc(vb_t, vt_bytes);
    const int wu = __builtin_amdgcn_readfirstlane(wv);  // the LDS bases stay scalar
#pragma unroll
    for (int i = 0; i < KL; ++i) lds_dma16(kr, koff[i] * 2, &dst->k[4 * (wu * KL + i) * D]);
#pragma unroll
    for (int i = 0; i < VL; ++i) lds_dma16(vr, voff[i] * 2, &dst->v[RPL * (wu * VL + i) * BN]);
  };
  auto dma = [&](Tile* __restrict__ dst, int kt_) __attribute__((always_inline)) {
    dma_from(dst, kbase + (int64_t)kt_ * BN * D, vbase + (int64_t)kt_ * BN * D);
  };
  // wait_tiles(n): all but this wave's last n tiles of loads have landed
  static_assert((NBUF - 2) * TL < 64, "vmcnt threshold");
  auto wait_tiles = [&](int n) __attribute__((always_inline)) {
    if (n <= 0) TTT_WAIT_VMCNT(0);
    else if (NBUF <= 2 || n == 1) TTT_WAIT_VMCNT(TL);
    else if (NBUF <= 3 || n == 2) TTT_WAIT_VMCNT(2 * TL);
    else TTT_WAIT_VMCNT(3 * TL);
  };
  static_assert(NBUF <= 4, "wait_tiles covers at most 3 tiles in flight");

  if (kt_lo < nkt) dma(&sm.ring[0], kt_lo);
#pragma unroll
  for (int tt = 1; tt < NBUF - 1; ++tt)
    if (kt_lo + tt < nkt) dma(&sm.ring[tt], kt_lo + tt);
  // ---- Q~ = R(i+p-1) q in fp16 (while the first tiles load), B operand chunks c = 0..7 (d = 16c + 8hf + e)
  f16x8 qf[8];
  // 64-row work items over the 4 heads of a group (contiguous in a token
  // row): the rows and their angles come in through LDS as whole 1 KB token
  // rows and table rows (each lane reading 32-byte pieces of 32 rows from
  // memory would move several times the bytes through the load path), then
  // each lane reads its own pieces back.
  constexpr bool QSTAGE = TTT_ && NW == 8 && RH == 4 && RT == QST_ROWS;
  if (QSTAGE && P.qs_h == D) {
    static_assert(!QSTAGE || NBUF == 2, "the staging shares the LDS of ring slot 1");
    const int wu = __builtin_amdgcn_readfirstlane(wv);
    const int nrows = min(RT, L - row0);  // >= 1
    const uint16_t* qb = q + b * P.qs_b + (int64_t)(start + row0) * P.qs_t + (int64_t)(g * P.r + sub * RH) * P.qs_h;
    const buf_rsrc qr = make_rsrc(qb, (uint32_t)((nrows - 1) * P.qs_t * 2 + RH * D * 2));
#pragma unroll
    for (int j = 0; j < RT / NW; ++j) {
      const int r = wu * (RT / NW) + j;
      lds_dma16(qr, (uint32_t)(r * P.qs_t * 2) + lane * 16, &sm.qst.q[r * QST_PITCH]);
    }
    const int pos0 = min(max(qoff + row0 + P.p - 1, 0), P.npos - 1);
    const uint32_t tab_bytes = (uint32_t)(P.npos - pos0) * 64 * 4;  // rows past the table read zeros
    const buf_rsrc cr = make_rsrc(cosT + (int64_t)pos0 * 64, tab_bytes), sr = make_rsrc(sinT + (int64_t)pos0 * 64, tab_bytes);
#pragma unroll
    for (int j = 0; j < RT / 4 / NW; ++j) {
      const int k4 = wu * (RT / 4 / NW) + j;
      lds_dma16(cr, (uint32_t)(k4 * 1024) + lane * 16, &sm.qst.c[k4 * QST_PITCH]);
      lds_dma16(sr, (uint32_t)(k4 * 1024) + lane * 16, &sm.qst.s[k4 * QST_PITCH]);
    }
    TTT_WAIT_VMCNT(0);
    __syncthreads();
    const bool valid = my_row < L;
    const int rr = rbk * 32 + l32;
    const unsigned char* ql = &sm.qst.q[rr * QST_PITCH + hw * D * 2];
    const unsigned char* cl = &sm.qst.c[(rr >> 2) * QST_PITCH + (rr & 3) * 256];
    const unsigned char* sl = &sm.qst.s[(rr >> 2) * QST_PITCH + (rr & 3) * 256];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = c * 16 + hf * 8;
      float x1[8], x2[8];
      unpack_bf8(*(const u32x4*)(ql + d0 * 2), x1);
      unpack_bf8(*(const u32x4*)(ql + (d0 + 64) * 2), x2);
      const f32x4 c0 = *(const f32x4*)(cl + d0 * 4), c1 = *(const f32x4*)(cl + d0 * 4 + 16);
      const f32x4 s0 = *(const f32x4*)(sl + d0 * 4), s1 = *(const f32x4*)(sl + d0 * 4 + 16);
      const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y1 = x1[e] * cs[e] - x2[e] * sn[e];
        const float y2 = x2[e] * cs[e] + x1[e] * sn[e];
        qf[c][e] = (_Float16)(valid ? y1 : 0.f);
        qf[c + 4][e] = (_Float16)(valid ? y2 : 0.f);
      }
    }
    lds_ring_barrier();  // every wave has its rows before ring slot 1 is refilled
  } else {
    const bool valid = my_row < L;
    const uint16_t* qrow = q + b * P.qs_b + (int64_t)(start + my_row) * P.qs_t + h * P.qs_h;
    const int pos = TTT_ ? qoff + my_row + P.p - 1
                              : (valid ? blk_anchor(P, bq, my_row) + (my_row & ((1 << P.bs_log2) - 1)) : 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = c * 16 + hf * 8;
      float x1[8], x2[8];
      if (valid) {
        unpack_bf8(*(const u32x4*)(qrow + d0), x1);
        unpack_bf8(*(const u32x4*)(qrow + d0 + 64), x2);
        const f32x4* cp = (const f32x4*)(cosT + rope_off(P, pos) + d0);
        const f32x4* sp = (const f32x4*)(sinT + rope_off(P, pos) + d0);
        const f32x4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
        const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y1 = x1[e] * cs[e] - x2[e] * sn[e];
          const float y2 = x2[e] * cs[e] + x1[e] * sn[e];
          x1[e] = y1;
          x2[e] = y2;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x1[e] = x2[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf[c][e] = (_Float16)x1[e];
        qf[c + 4][e] = (_Float16)x2[e];
      }
    }
  }

  wait_tiles(min(nkt - kt_lo, NBUF - 1) - 1);
  __syncthreads();

  f32x16 oacc[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d4][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f, scale_o = 1.f;
  const int prow = perm_row(l32);
  const float sl2 = P.scale_log2;
  // Tiles whose every key precedes every row of this wave need no mask.
  const int n_free = TTT_ ? max(0, min(wave_row0 + 1 + dq_, kv_len)) / BN : lim_lo / BN;
  // and, with a window, tiles from f_lo on: every key is inside every row's window
  const int f_lo = (TTT_ && win > 0) ? max(0, wave_row0 + 31 + dq_ - win + 1 + BN - 1) / BN : 0;

  // Moves the running max to mx when mx exceeds it by more than 8 (log2 units).
  auto raise_max = [&](float mx) {
    if (mx > m_run + 8.f) {
      const float alpha = fast_exp2(m_run - mx);
      l_run *= alpha;
      m_run = mx;
      scale_o *= alpha;
    }
  };
  auto apply_scale = [&]() {
    if (__builtin_amdgcn_ballot_w64(scale_o != 1.f)) {
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[d4][v] *= scale_o;
      scale_o = 1.f;
    }
  };

  // One key tile: S^T = K~ Q~^T, online softmax, O^T += V^T P^T.
  auto tile = [&](const Tile* __restrict__ cur, const int key0, auto masked) __attribute__((always_inline)) {
    constexpr int KB = BN / 32;
    const _Float16* kl = cur->k;
    const _Float16* vl = cur->v;
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int r = kb * 32 + prow;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
      f16x8 a[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) a[c] = *(const f16x8*)&kl[r * D + (((2 * c + hf) ^ (r & 15)) * 8)];
#pragma unroll
      for (int c = 0; c < 8; ++c) sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c], qf[c], sacc[kb], 0, 0, 0);
      // three operand reads ahead of the MFMAs, then one read per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
    // masks: 1 causal trunk, 2 context prefix j < lim, 3 the row's own block
    constexpr int M = decltype(masked)::value;
    if constexpr (M != 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + kb * 32 + (v >> 3) * 16 + hf * 8 + (v & 7);
          bool off;
          if constexpr (M == 1)
            off = key > my_row + dq_ || key >= kv_len || (MODE == 4 && key <= my_row + dq_ - win);
          else if constexpr (M == 2) off = key >= lim;
          else off = (key >> P.bs_log2) != (my_row >> P.bs_log2) || key >= L;
          if (off) sacc[kb][v] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = xhalf_max(mx) * sl2;
    raise_max(mx);
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;  // no key seen yet: every P is 0
    // P in fp16 (<= 2^8 with the lazy max; 11 significant bits, so one
    // dominant key's rounding moves the LSE by < 5e-4) for the PV product
    f16x8 pb[2 * KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) pb[kb * 2 + (v >> 3)][v & 7] = (_Float16)fast_exp2(__builtin_fmaf(sacc[kb][v], sl2, neg_m));
    // row sum of the fp16 probabilities the PV product uses, two per v_dot2:
    // O's weights then sum to 1 exactly
    const h2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int c2 = 0; c2 < 2 * KB; ++c2)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const h2 pr = {pb[c2][e], pb[c2][e + 1]};
        l_run = __builtin_amdgcn_fdot2(pr, one, l_run, false);
      }
    apply_scale();
    {
      f16x8 a[2 * KB][4];
#pragma unroll
      for (int c2 = 0; c2 < 2 * KB; ++c2)
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
          const int d = d4 * 32 + l32;
          a[c2][d4] = *(const f16x8*)&vl[d * BN + (((2 * c2 + hf) ^ ((d >> 1) & (CH - 1))) * 8)];
        }
#pragma unroll
      for (int c2 = 0; c2 < 2 * KB; ++c2)
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) oacc[d4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c2][d4], pb[c2], oacc[d4], 0, 0, 0);
      // three operand reads ahead of the MFMAs, then one read per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int c = 0; c < 8 * KB - 3; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
  };

  // Iteration j loads tile j+NBUF-1 into the buffer tile j-1 used and runs
  // tile j.  The two buffers go through distinct restrict pointers, so the
  // compiler knows the loads cannot alias this tile's LDS reads.
  for (int kt_ = kt_lo; kt_ < nkt; ++kt_) {
    auto step = [&](const Tile* __restrict__ cur, Tile* __restrict__ dst) __attribute__((always_inline)) {
      if (kt_ + NBUF - 1 < nkt) dma(dst, kt_ + NBUF - 1);
      if (kt_ < n_free && kt_ >= f_lo) tile(cur, kt_ * BN, std::integral_constant<int, 0>{});
      else tile(cur, kt_ * BN, std::integral_constant<int, TTT_ ? 1 : 2>{});
    };
    const int rb = kt_ - kt_lo;
    step(&sm.ring[rb % NBUF], &sm.ring[(rb + NBUF - 1) % NBUF]);
    if (kt_ + 1 < nkt) wait_tiles(min(nkt, kt_ + NBUF) - (kt_ + 2));  // tile kt_+1 has landed
    lds_ring_barrier();                                                 // every wave is done with tile kt_
  }

  // ---- block drafting: the keys of the work item's own blocks (rows row0 ..
  // row0+RT-1; bs divides 32, so no block straddles the work item), one
  // 64-key tile at a time, masked to the row's block
  if constexpr (MODE == 1) {
    const _Float16* kbb = kbt + ((int64_t)(b * P.Hkv + g) * P.spad_b + slot0) * D;
    const _Float16* vbb = vbt + (int64_t)(b * P.Hkv + g) * D * P.spad_b + (int64_t)(slot0 >> 5) * D * 32;
    for (int k0 = row0; k0 < qend; k0 += BN) {  // k0: a multiple of 32
      dma_from(&sm.ring[0], kbb + (int64_t)k0 * D, vbb + (int64_t)(k0 >> 5) * D * 32);
      TTT_WAIT_VMCNT(0);
      __syncthreads();
      tile(&sm.ring[0], k0, std::integral_constant<int, 3>{});
      __syncthreads();
    }
  }

  // ---- branch: keys/values of passes 2..p at the same row, folded into (m, l, O)
  const int lr = rbk * 32 + l32;  // this lane's row within the tile
  // Staging roles: 8 threads per row, rows RPS*j + tid/8.  With one row set
  // per work item the raw k^(q+1), v^(q+1) rows are loaded while pass q is
  // computed, so a pass waits for no global load of its own (larger work
  // items load each row set just before staging it: registers).
  constexpr int RPS = 8 * NW;  // rows per staged set
  constexpr int NR = RT / RPS;
  const int bc8 = tid & 7, bdlo = bc8 * 8, bdhi = 64 + bc8 * 8;
  auto load_rows = [&](int j, int qq, u32x4 (&kr)[2], u32x4 (&vr)[2]) __attribute__((always_inline)) {
    const int i = row0 + j * RPS + (tid >> 3);
    kr[0] = kr[1] = vr[0] = vr[1] = u32x4{0, 0, 0, 0};
    if (i < L) {
      const int64_t koff = b * P.ks_b + (int64_t)(start + i) * P.ks_t + g * P.ks_h;
      const uint16_t* krow = (const uint16_t*)kv.k[qq - 1] + koff;
      const uint16_t* vrow = (const uint16_t*)kv.v[qq - 1] + koff;
      kr[0] = *(const u32x4*)(krow + bdlo);
      kr[1] = *(const u32x4*)(krow + bdhi);
      vr[0] = *(const u32x4*)(vrow + bdlo);
      vr[1] = *(const u32x4*)(vrow + bdhi);
    }
  };
  // R(i+q-1) k^(q) (fp16) and v^(q) (bf16) of row set j into LDS
  auto stage_rows = [&](int j, int qq, const u32x4 (&kr)[2], const u32x4 (&vr)[2]) __attribute__((always_inline)) {
    const int rr = j * RPS + (tid >> 3);
    const int i = row0 + rr;
    u32x4 klo = {0, 0, 0, 0}, khi = {0, 0, 0, 0};
    if (i < L) {
      float x1[8], x2[8], y1[8], y2[8];
      unpack_bf8(kr[0], x1);
      unpack_bf8(kr[1], x2);
      const int pk = qoff + i + qq - 1;
      const float* cp = cosT + rope_off(P, pk) + bdlo;
      const float* sp = sinT + rope_off(P, pk) + bdlo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y1[e] = x1[e] * cp[e] - x2[e] * sp[e];
        y2[e] = x2[e] * cp[e] + x1[e] * sp[e];
      }
      klo = pack_h8(y1);
      khi = pack_h8(y2);
    }
    *(u32x4*)&sm.br.k[rr][bdlo] = klo;
    *(u32x4*)&sm.br.k[rr][bdhi] = khi;
    *(u32x4*)&sm.br.v[rr][bdlo] = vr[0];
    *(u32x4*)&sm.br.v[rr][bdhi] = vr[1];
  };
  const int pmax = TTT_ && P.branch ? P.p : 1;
  u32x4 kpre[2], vpre[2];  // one row set: the next pass's raw rows
  if (NR == 1 && pmax >= 2) load_rows(0, 2, kpre, vpre);
  for (int qq = 2; qq <= pmax; ++qq) {
    if constexpr (NR == 1) {
      stage_rows(0, qq, kpre, vpre);
    } else {
#pragma unroll 1
      for (int j = 0; j < NR; ++j) {
        u32x4 kr[2], vr[2];
        load_rows(j, qq, kr, vr);
        stage_rows(j, qq, kr, vr);
      }
    }
    __syncthreads();
    if (NR == 1 && qq < pmax) load_rows(0, qq + 1, kpre, vpre);
    // score: lane's Q~ fragment (d = 16c + 8hf + e) against the staged key row
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f16x8 kk = *(const f16x8*)&sm.br.k[lr][c * 16 + hf * 8];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const h2 a = {qf[c][e], qf[c][e + 1]}, bq = {kk[e], kk[e + 1]};
        part = __builtin_amdgcn_fdot2(a, bq, part, false);
      }
    }
    const float s2 = xhalf_sum(part) * sl2;
    raise_max(s2);
    apply_scale();
    const float pe = fast_exp2(s2 - m_run);
    if (hf == 0) l_run += pe;
    // O^T[d][row] += pe * v^(q)[row][d], d = 32*d4 + 8*v4 + 4*hf + e
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const u32x2 w = *(const u32x2*)&sm.br.v[lr][d4 * 32 + v4 * 8 + hf * 4];
        oacc[d4][v4 * 4 + 0] += pe * __uint_as_float(w[0] << 16);
        oacc[d4][v4 * 4 + 1] += pe * __uint_as_float(w[0] & 0xffff0000u);
        oacc[d4][v4 * 4 + 2] += pe * __uint_as_float(w[1] << 16);
        oacc[d4][v4 * 4 + 3] += pe * __uint_as_float(w[1] & 0xffff0000u);
      }
    __syncthreads();
  }

  // ---- epilogue: O / l, LSE
  const float l_tot = xhalf_sum(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;  // a row that sees no key: O = 0, LSE = -inf
  const int orow = wv * 32 + l32;  // LDS row: (wave, lane row)
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = oacc[d4][v4 * 4 + e] * inv_l;
      *(f32x4*)&sm.o[orow][d4 * 32 + v4 * 8 + hf * 4] = w;
    }
  if (hf == 0 && my_row < L) lse[b * P.lse_b + h * P.lse_h + start + my_row] = (l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY);
  __syncthreads();
  // each wave stores its own 32 rows: 8 lanes per row, 16 elements per lane
  const int c8 = lane & 7;
  const int dlo = c8 * 8, dhi = 64 + c8 * 8;
#pragma unroll
  for (int rp = 0; rp < 32; rp += 8) {
    const int rr = rp + (lane >> 3);
    const int i = wave_row0 + rr;
    if (i >= L) continue;
    const float* src = sm.o[wv * 32 + rr];
    float res[16];
    const f32x4 a0 = *(const f32x4*)&src[dlo], a1 = *(const f32x4*)&src[dlo + 4];
    const f32x4 b0 = *(const f32x4*)&src[dhi], b1 = *(const f32x4*)&src[dhi + 4];
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = a0[e], res[4 + e] = a1[e], res[8 + e] = b0[e], res[12 + e] = b1[e];
    const int64_t oo = b * P.os_b + (int64_t)(start + i) * P.os_t + h * P.os_h;
    if (O_F32) {
      float* op = (float*)o + oo;
      *(f32x4*)(op + dlo) = a0;
      *(f32x4*)(op + dlo + 4) = a1;
      *(f32x4*)(op + dhi) = b0;
      *(f32x4*)(op + dhi + 4) = b1;
    } else {
      uint16_t* op = (uint16_t*)o + oo;
      *(u32x4*)(op + dlo) = pack_bf8(res);
      *(u32x4*)(op + dhi) = pack_bf8(res + 8);
    }
  }
}

int heads_per_wg(int r) { return r % 4 == 0 ? 4 : (r % 2 == 0 ? 2 : 1); }

template <int RH, int MODE>
static void launch_rh(const Prob& P, const uint16_t* q, const PassPtrs& kv, const _Float16* kt, const _Float16* vt,
                      const int4* tiles, const float* cosT, const float* sinT, void* o, bool o_f32, float* lse,
                      const _Float16* kbt, const _Float16* vbt, hipStream_t st) {
  if constexpr (RH == 4 && MODE != 1 && kFwdWaves == 8) {  // TTT passes: 4 heads x 64 rows per work item
    constexpr int RT8 = tile_rows(4, 8);
    const int ntiles8 = P.layout == 0 ? P.B * ((P.stok + RT8 - 1) / RT8) : (P.stok + RT8 - 1) / RT8 + P.nseq;
    const int64_t grid8 = (int64_t)ntiles8 * P.Hkv * (P.r / 4);
    if (o_f32)
      fwd_bf16_kernel<4, true, MODE, 8>
          <<<(unsigned)grid8, 512, 0, st>>>(P, q, kv, kt, vt, tiles, cosT, sinT, o, lse, kbt, vbt);
    else
      fwd_bf16_kernel<4, false, MODE, 8>
          <<<(unsigned)grid8, 512, 0, st>>>(P, q, kv, kt, vt, tiles, cosT, sinT, o, lse, kbt, vbt);
    return;
  }
  constexpr int RT = tile_rows(RH);
  int ntiles;
  if (P.layout == 0) ntiles = P.B * ((P.stok + RT - 1) / RT);
  else ntiles = (P.stok + RT - 1) / RT + P.nseq;
  const int64_t grid = (int64_t)ntiles * P.Hkv * (P.r / RH);
  if (o_f32)
    fwd_bf16_kernel<RH, true, MODE>
        <<<(unsigned)grid, 256, 0, st>>>(P, q, kv, kt, vt, tiles, cosT, sinT, o, lse, kbt, vbt);
  else
    fwd_bf16_kernel<RH, false, MODE>
        <<<(unsigned)grid, 256, 0, st>>>(P, q, kv, kt, vt, tiles, cosT, sinT, o, lse, kbt, vbt);
}

template <int MODE>
static void launch_mode(const Prob& P, const uint16_t* q, const PassPtrs& kv, const _Float16* kt,
                        const _Float16* vt, const int4* tiles, const float* cosT, const float* sinT, void* o,
                        bool o_f32, float* lse, const _Float16* kbt, const _Float16* vbt, hipStream_t st) {
  switch (heads_per_wg(P.r)) {
    case 4: launch_rh<4, MODE>(P, q, kv, kt, vt, tiles, cosT, sinT, o, o_f32, lse, kbt, vbt, st); break;
    case 2: launch_rh<2, MODE>(P, q, kv, kt, vt, tiles, cosT, sinT, o, o_f32, lse, kbt, vbt, st); break;
    default: launch_rh<1, MODE>(P, q, kv, kt, vt, tiles, cosT, sinT, o, o_f32, lse, kbt, vbt, st); break;
  }
}

}  // namespace fwd

int fwd_tile_rows(int r) {
  const int rh = fwd::heads_per_wg(r);
  return fwd::tile_rows(rh, rh == 4 ? fwd::kFwdWaves : 4);
}
int block_fwd_tile_rows(int r) { return fwd::tile_rows(fwd::heads_per_wg(r)); }

void launch_fwd_bf16(const Prob& P, const uint16_t* q, const PassPtrs& kv, const _Float16* kt, const _Float16* vt,
                     const int4* tiles, const float* cosT, const float* sinT, void* o, bool o_f32, float* lse,
                     hipStream_t st) {
  if (P.win > 0)
    fwd::launch_mode<4>(P, q, kv, kt, vt, tiles, cosT, sinT, o, o_f32, lse, nullptr, nullptr, st);
  else
    fwd::launch_mode<0>(P, q, kv, kt, vt, tiles, cosT, sinT, o, o_f32, lse, nullptr, nullptr, st);
}

void launch_block_fwd_bf16(const Prob& P, const uint16_t* q, const _Float16* kt, const _Float16* vt,
                           const _Float16* kbt, const _Float16* vbt, const int4* tiles, const float* cosT,
                           const float* sinT, void* o, bool o_f32, float* lse, hipStream_t st) {
  const PassPtrs none = {};
  fwd::launch_mode<1>(P, q, none, kt, vt, tiles, cosT, sinT, o, o_f32, lse, kbt, vbt, st);
}

}  // namespace ttt
