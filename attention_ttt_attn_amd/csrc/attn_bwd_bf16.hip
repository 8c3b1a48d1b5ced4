// bf16 backward of the multi-pass TTT attention: probabilities are recomputed
// from the forward's merged LSE (NeMo-RL issue "DFlash/DSpark and EAGLE-3 TTT
// draft co-training ...", "What I'm working on", item 1: exact joint-LSE merge
// -- the merged LSE normalises trunk and branch probabilities alike).
//
//   Delta_i = <dO_i, O_i>,  P_a = exp(s_a - LSE_i),  dS_a = P_a (<dO_i, v_a> - Delta_i)
//   dq~_i  = sigma sum_a dS_a k~_a            (trunk keys and branch keys)
//   dk~_a  = sigma sum_{i,h} dS_a q~_i,  dv_a = sum_{i,h} P_a dO_i
//   dq = R(i+p-1)^T dq~,  dk^(1)_j = R(j)^T dk~,  dk^(q)_i = R(i+q-1)^T dk~
//
// Three kernels:
// * dq_bf16_kernel (query-outer, MFMA): per 32 query rows of the heads of one
//   KV group, loops over the causal key tiles and accumulates
//   dQ~^T = K~^T dS^T; the epilogue adds the branch terms of passes 2..p
//   (row-local, xor-shuffle reductions), un-rotates and writes dQ.  When the
//   work item holds every query head of the group it also sums the branch
//   dK/dV of passes 2..p over those heads and writes them.  No atomics:
//   deterministic.
// * dkdv_bf16_kernel (key-outer, MFMA): per 128 trunk keys of one KV head,
//   loops over the r query heads of the group and the query rows i >= j;
//   dK~^T and dV^T stay in VGPRs; un-rotated in the epilogue.
// * branch_bwd_bf16_kernel (HBM-bound, no MFMA): dK^(q), dV^(q) for q = 2..p at
//   every row, summed over the group's heads with xor-shuffle dot products,
//   for groups wider than a dQ work item.
// MFMA operand layouts follow the forward: transposed products so that one
// product's accumulator is the next one's B operand (A rows read permuted).
#include <type_traits>

#include "kernels.hpp"

namespace ttt {

namespace bwd {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));
constexpr int D = 128;
constexpr int BKV = kBwdBKV;  // dK/dV kernel: keys per workgroup
constexpr int BQ = 32;        // dK/dV kernel: query rows per step
constexpr int OPAD = D + 4;

__device__ __forceinline__ int perm_row(int a) { return (a & ~0xC) | ((a & 4) << 1) | ((a & 8) >> 1); }

// Largest of p[lo..hi) over the wave (0 for an empty range), eight loads in
// flight per lane.
__device__ __forceinline__ float range_max(const float* __restrict__ p, int lo, int hi, int lane) {
  float m = 0.f;
  for (int i = lo + lane; i < hi; i += 512) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = i + 64 * k < hi ? p[i + 64 * k] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, x[k]);
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  return m;
}

// ============================================================================= dQ
// A workgroup is 4 wave64s: the R' query heads of one KV group that it covers
// (R' = 4 for GQA 4:1) times 32*4/R' rows; each wave owns 32 query rows of one
// head, so with R' = 4 all four waves share one causal extent.  Key tiles of
// 32 keys -- K~ rows (A of S^T), V rows (A of dP^T) and K~^T (A of dQ^T) --
// move HBM -> LDS with direct loads (buffer_load ... lds), XOR-swizzled, double
// buffered: the next tile's loads run under this tile's products; one barrier
// per tile.  Two workgroups per CU keep the matrix pipe busy while the other
// one's vector ALUs form dS.
constexpr int QBN = 32;  // keys per dQ tile
struct DqBuf {
  _Float16 k[QBN * D];   // K~ rows: row r at r*D, 16-byte chunk c at slot c ^ (r & 15)
  uint16_t v[QBN * D];   // V rows, same layout
  _Float16 kt[D * QBN];  // K~^T: d-row at d*QBN, chunk c at slot c ^ ((d >> 2) & 3)
};
// Stored dS (MODE 5): two rings -- K~^T tiles (as in DqBuf), loaded DS_NK - 1
// tiles ahead, and every wave's 32x32 dS block of a tile, loaded DS_NS - 1
// tiles ahead (the dS stream comes from HBM, K~^T mostly from the caches).  A
// dS block lies at [key][quarter u*2 + w][8 rows 16 u + 8 w + 0..7] (64
// bytes per key): a transposing read then meets each bank twice per
// instruction, the least its 512 bytes allow.
constexpr int DS_NK = 3, DS_NS = 6;
struct DsRing {
  _Float16 kt[DS_NK][D * QBN];
  _Float16 ds[DS_NS][4][32 * 32];
};
constexpr int GST_PITCH = 1024 + 16;  // one token row of 4 heads' dO, padded
struct DqSmem {
  union {
    DqBuf buf[2];
    DsRing dr;
    float acc[128][OPAD];  // dQ~ rows (wave, row) for the row-major epilogue
    struct {               // 4-head work items: dO rows staged beside the first key tile
      unsigned char first_tile[sizeof(DqBuf)];
      unsigned char g[32 * GST_PITCH];
    } gst;
  };
};

__host__ __device__ constexpr int dq_rows(int heads_per_wg) { return 32 * 4 / heads_per_wg; }
static int dq_heads_per_wg(int r) { return r % 4 == 0 ? 4 : (r % 2 == 0 ? 2 : 1); }

// MODE 0: TTT pass; MODE 4: the same with a sliding-window trunk (its own
// instantiation); MODE 5: a whole-sequence BSHD TTT pass whose trunk dS the
// dK/dV kernel stored (P.ds): dQ~^T = K~^T dS^T from those blocks, no S or dP
// products.  MODE 1: block drafting -- key tiles of the context (kt/ktt, V =
// kv.v[0] with the P.cs strides) up to each row's block anchor, then the keys
// of the work item's own blocks (kbt/kbtt, V = kv.v[1]).
template <int RH, int MODE>
__global__ void __launch_bounds__(256, 2)
    dq_bf16_kernel(Prob P, const uint16_t* __restrict__ q, PassPtrs kv, const float* __restrict__ lse,
                   const uint16_t* __restrict__ dout, const _Float16* __restrict__ kt,
                   const _Float16* __restrict__ ktt, const _Float16* __restrict__ qt, const float* __restrict__ delta,
                   const int4* __restrict__ tiles, const float* __restrict__ cosT, const float* __restrict__ sinT,
                   uint16_t* __restrict__ dq, const _Float16* __restrict__ kbt, const _Float16* __restrict__ kbtt,
                   PassGradPtrs gr) {
  constexpr int RT = dq_rows(RH);  // rows per work item
  __shared__ __attribute__((aligned(16))) DqSmem sm;
  constexpr bool DSM = MODE == 5;  // trunk dS stored by the dK/dV kernel
  constexpr bool TTT_ = MODE == 0 || MODE == 4 || DSM;  // TTT pass (4: with a sliding window)
  const int win = MODE == 4 ? P.win : 0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- work item.  BSHD: row tiles heavy-first, every (batch, KV head, head
  // sub-group) unit pinned to one XCD (blockIdx % 8) so that the row tiles
  // running together there share its L2 for the keys they stream.  THD: the
  // scheduler's list (heavy-first), KV head = blockIdx % Hkv.
  const int nsub = P.r / RH;
  int b, t, start, L, slot0, g, sub;
  if (P.layout == 0) {
    const int units = P.B * P.Hkv * nsub;
    const int ntl = (P.stok + RT - 1) / RT;
    const int upx = (units + 7) / 8;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tix = slot / upx, unit = (slot % upx) * 8 + xcd;
    if (tix >= ntl || unit >= units) return;
    t = ntl - 1 - tix;
    sub = unit % nsub;
    const int pair = unit / nsub;
    g = pair % P.Hkv;
    b = pair / P.Hkv;
    start = 0;
    L = P.stok;
    slot0 = 0;
  } else {
    const int per = P.Hkv * nsub;
    const int unit = blockIdx.x % per, tix = blockIdx.x / per;
    if (tix >= tiles[0].x) return;
    const int4 e = tiles[1 + tix];
    t = e.x, start = e.y, L = e.z, slot0 = e.w, b = 0;
    g = unit / nsub;
    sub = unit % nsub;
  }
  const int hw = wv % RH, rbk = wv / RH;
  const int h = g * P.r + sub * RH + hw;
  const int row0 = t * RT;
  const int wave_row0 = row0 + rbk * 32;
  const int my_row = wave_row0 + l32;
  const bool row_ok = my_row < L;
  const int qend = min(row0 + RT, L);
  // Block drafting: row i sees context keys j < lim (its block's anchor); the
  // work item spans the largest lim of its blocks, a wave's unmasked prefix
  // is the smallest lim of the wave's blocks.
  int lim = 0, lim_hi = 0, lim_lo = 0;
  BlkSeq bq{};  // block drafting: the sequence's anchors and context
  if constexpr (MODE == 1) {
    bq = blk_seq(P, b, start);
    lim = row_ok ? blk_anchor(P, bq, my_row) : 0;
    const int wend = min(wave_row0 + 32, L);
    lim_lo = wend > wave_row0 ? bq.cn : 0;
    for (int blk = row0 >> P.bs_log2; (blk << P.bs_log2) < qend; ++blk) {
      const int a = blk_anchor(P, bq, blk << P.bs_log2);
      lim_hi = max(lim_hi, a);
      if ((blk << P.bs_log2) < wend && ((blk + 1) << P.bs_log2) > wave_row0) lim_lo = min(lim_lo, a);
    }
  }
  // TTT ring steps (BSHD): row i sits at position q_off + i, trunk key j at
  // kv_off + j (j < kv_len); whole-sequence calls have dq_ = 0, kvn = L.
  // (THD ring steps: the segment's own offsets and key rows kvs .. kvs + kvn.)
  // (Block drafting: the sequence's context rows.)
  int qoff = 0, dq_ = 0, kvs = start, kvn = P.kv_len;
  if constexpr (TTT_)
    seq_ring(P, (P.layout == 1 && P.kv_cu) ? seq_at(P.cu, P.nseq, start) : b, start, L, qoff, dq_, kvs, kvn);
  if constexpr (MODE == 1) kvs = bq.cs, kvn = bq.cn;
  const int kmax = TTT_ ? min(qend - 1 + dq_, kvn - 1) : lim_hi - 1;  // last key any row sees
  const int nkt = kmax < 0 ? 0 : kmax / QBN + 1;
  // sliding window: the first key tile any row of the work item sees
  const int kt_lo = (TTT_ && win > 0) ? max(0, row0 + dq_ - win + 1) / QBN : 0;

  // DMA lane roles, 6 loads per wave per tile (load n = 2w + i):
  // K~ and V rows 4n + lane/16, slot lane%16; K~^T d-rows 16n + lane/4, slot lane%4.
  const _Float16* kbase = kt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0) * D;
  // K~^T slabs come in 32-key tiles of D x 32 (one contiguous 8 KB piece each)
  const _Float16* ktbase = ktt + (int64_t)(b * P.Hkv + g) * D * P.spad + (int64_t)(slot0 >> 5) * D * QBN;
  // trunk V: P.cs_* strides (the pass-1 / context V; P.ks_* stay with the branch)
  const int64_t vs_t = P.cs_t;
  const uint16_t* vbase = (const uint16_t*)kv.v[0] + b * P.cs_b + (int64_t)kvs * vs_t + g * P.cs_h;
  const int vlast = kvn - 1;  // last key row of the trunk
  uint32_t roff[2], toff[2];
  int rrow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = 2 * wv + i;
    const int r = 4 * n + (lane >> 4);
    rrow[i] = r;
    roff[i] = (uint32_t)(((lane & 15) ^ (r & 15)) * 8);
    const int d = 16 * n + (lane >> 2);
    toff[i] = (uint32_t)(d * QBN + ((lane & 3) ^ ((d >> 2) & 3)) * 8);
  }
  // buffer descriptors at the tile's bases; the lanes add byte offsets
  const uint32_t kt_bytes = (uint32_t)(D * QBN * 2);  // one K~^T tile
  auto dma_from = [&](DqBuf* __restrict__ dst, const _Float16* kb, const _Float16* ktb, const uint16_t* vb,
                      int64_t vst, int key0, int last) __attribute__((always_inline)) {
    DqBuf& B_ = *dst;
    const buf_rsrc kr = make_rsrc(kb + (int64_t)key0 * D, QBN * D * 2);
    const buf_rsrc vr = make_rsrc(vb + (int64_t)key0 * vst, 0xFFFFFFFFu);
    const buf_rsrc tr = make_rsrc(ktb + (int64_t)(key0 / QBN) * D * QBN, kt_bytes);  // key0: a multiple of 32
    const int wu = __builtin_amdgcn_readfirstlane(wv);  // the LDS bases stay scalar
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = 2 * wu + i;
      const int rg = min(rrow[i], last - key0);  // V rows past the end repeat the last row (masked)
      lds_dma16(kr, (uint32_t)((rrow[i] * D + (int)roff[i]) * 2), &B_.k[4 * n * D]);
      lds_dma16(vr, (uint32_t)((rg * vst + roff[i]) * 2), &B_.v[4 * n * D]);
      lds_dma16(tr, toff[i] * 2, &B_.kt[16 * n * QBN]);
    }
  };
  auto dma = [&](DqBuf* __restrict__ dst, int j) __attribute__((always_inline)) {
    dma_from(dst, kbase, ktbase, vbase, vs_t, j * QBN, vlast);
  };
  if (!DSM && kt_lo < nkt) dma(&sm.buf[0], kt_lo);

  // B operands of this lane's query: Q~ (fp16, pre-rotated) and dO (bf16).
  // With the 4 heads of a group in one work item (adjacent in a token row),
  // the dO rows come in through LDS as whole 1 KB token rows (per-lane
  // 32-byte pieces of 32 rows would move several times the bytes through the
  // load path); the pre-rotated Q~ rows are contiguous per head already.
  f16x8 qf[8];
  bf16x8 dof[8];
  const bool gstage = !DSM && RH == 4 && P.os_h == D;
  if constexpr (!DSM) {
    const _Float16* qrow = qt + ((int64_t)(b * P.Hq + h) * P.spad + slot0 + my_row) * D;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = *(const f16x8*)(qrow + c * 16 + hf * 8);
    if (gstage) {
      const int wu = __builtin_amdgcn_readfirstlane(wv);
      const int nrows = min(32, L - row0);  // >= 1
      const uint16_t* gb = dout + b * P.os_b + (int64_t)(start + row0) * P.os_t + (int64_t)(g * P.r + sub * RH) * P.os_h;
      const buf_rsrc gr_ = make_rsrc(gb, (uint32_t)((nrows - 1) * P.os_t * 2 + RH * D * 2));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = wu * 8 + j;
        lds_dma16(gr_, (uint32_t)(r * P.os_t * 2) + lane * 16, &sm.gst.g[r * GST_PITCH]);
      }
    } else {
      const uint16_t* grow = dout + b * P.os_b + (int64_t)(start + my_row) * P.os_t + h * P.os_h;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4 gv = row_ok ? *(const u32x4*)(grow + c * 16 + hf * 8) : u32x4{0, 0, 0, 0};
        dof[c] = __builtin_bit_cast(bf16x8, gv);
      }
    }
  }
  // rows past the sequence end get LSE = +inf: every probability is then 0
  const float lse2 = DSM ? 0.f : (row_ok ? lse[b * P.lse_b + h * P.lse_h + start + my_row] * kLog2e : INFINITY);
  float dl = DSM ? 0.f : delta[(int64_t)(b * P.Hq + h) * P.spad + slot0 + my_row];
  // fp16 dS operands of this row carry the factor 2^e: |dS_ij| <= ||dO_i||_1
  // max_j |v_jd| + |Delta_i| over the keys this work item visits (their
  // per-32-key maxima come from the dK/dV kernel, which runs first).  The
  // factor scales the row's dO operand (which feeds dP only) and Delta, so
  // P (dP - Delta) 2^e is formed exactly; the epilogue takes it out again.
  int eq;
  if constexpr (DSM) {  // the stored blocks' exponent: the dK/dV kernel's, for the whole group
    const float2 nd = *(const float2*)&P.dmax[(int64_t)(b * P.Hkv + g) * 2];
    eq = ds_exp(__builtin_fmaf(nd.x, P.vgmax[b * P.Hkv + g], nd.y));
  } else {
    const int64_t vb = (int64_t)(b * P.Hkv + g) * (P.spad / 32) + slot0 / 32;
    float vm = TTT_ ? range_max(P.vmax + vb, kt_lo, nkt, lane) : range_max(P.vmax + vb, 0, nkt, lane);
    if constexpr (MODE == 1) vm = fmaxf(vm, range_max(P.vmax_b + vb, row0 / 32, (qend + 31) / 32, lane));
    const float dn = P.dnorm[(int64_t)(b * P.Hq + h) * P.spad + slot0 + my_row];
    eq = ds_exp(__builtin_fmaf(dn, vm, fabsf(dl)));
    const float cq = __builtin_amdgcn_ldexpf(1.0f, eq);
    dl *= cq;
    if (gstage) {  // the staged dO rows (rows past the end: zero)
      TTT_WAIT_VMCNT(0);
      __syncthreads();
      const unsigned char* gl = &sm.gst.g[(rbk * 32 + l32) * GST_PITCH + hw * D * 2];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4 gv = *(const u32x4*)(gl + (c * 16 + hf * 8) * 2);
        if (!row_ok) gv = u32x4{0, 0, 0, 0};
        dof[c] = __builtin_bit_cast(bf16x8, gv);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 x = __builtin_bit_cast(u32x4, dof[c]);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        x[w] = pack_bf2(__uint_as_float(x[w] << 16) * cq, __uint_as_float(x[w] & 0xffff0000u) * cq);
      dof[c] = __builtin_bit_cast(bf16x8, x);
    }
  }
  const float sl2 = P.scale_log2;
  TTT_WAIT_VMCNT(0);
  asm volatile("" ::"v"(lse2), "v"(dl));  // their loads complete here, not inside the loop
  __syncthreads();

  f32x16 acc[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[d4][v] = 0.f;
  const int prow = perm_row(l32);
  // Tiles whose every key precedes every row of this wave need no mask.
  const int n_free = TTT_ ? max(0, min(wave_row0 + 1 + dq_, kvn)) / QBN : lim_lo / QBN;
  // with a window, tiles from f_lo on lie inside every row's window
  const int f_lo = (TTT_ && win > 0) ? max(0, wave_row0 + 31 + dq_ - win + 1 + QBN - 1) / QBN : 0;

  // S^T = K~ Q~^T, dP^T = V dO^T, dS = P (dP - Delta), dQ~^T += K~^T dS^T.
  // Masks: 1 causal, 2 context prefix key < lim, 3 the row's own block.
  auto tile = [&](const DqBuf* __restrict__ src, const int key0, auto masked) __attribute__((always_inline)) {
    const DqBuf& B_ = *src;
    f32x16 s, dp;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = dp[v] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < 8; c0 += 4) {
      f16x8 a[4];
      bf16x8 a2[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int off = prow * D + (((2 * (c0 + c) + hf) ^ (prow & 15)) * 8);
        a[c] = *(const f16x8*)&B_.k[off];
        a2[c] = *(const bf16x8*)&B_.v[off];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c], qf[c0 + c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[c], dof[c0 + c], dp, 0, 0, 0);
      }
    }
    // key of (v, hf) = key0 + 16*(v/8) + 8*hf + v%8
    f16x8 dsb[2];
    constexpr int M = decltype(masked)::value;
    const int thr = my_row + dq_ - (key0 + 8 * hf);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float pr = fast_exp2(__builtin_fmaf(s[v], sl2, -lse2));
      const int key = key0 + (v >> 3) * 16 + 8 * hf + (v & 7);
      if constexpr (M == 1)
        pr = ((v >> 3) * 16 + (v & 7) > thr || key >= kvn || (MODE == 4 && key <= my_row + dq_ - win)) ? 0.f : pr;
      else if constexpr (M == 2) pr = key >= lim ? 0.f : pr;
      else if constexpr (M == 3) pr = ((key >> P.bs_log2) != (my_row >> P.bs_log2) || key >= L) ? 0.f : pr;
      dsb[v >> 3][v & 7] = (_Float16)(pr * (dp[v] - dl));
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      f16x8 a[4];
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        const int d = d4 * 32 + l32;
        a[d4] = *(const f16x8*)&B_.kt[d * QBN + (((2 * c2 + hf) ^ ((d >> 2) & 3)) * 8)];
      }
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) acc[d4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[d4], dsb[c2], acc[d4], 0, 0, 0);
    }
  };
  if constexpr (!DSM) {
    for (int j = kt_lo; j < nkt; ++j) {
      // distinct restrict pointers: the loads into the other buffer cannot alias
      // this tile's LDS reads, so the compiler puts no wait on them
      auto step = [&](const DqBuf* __restrict__ cur, DqBuf* __restrict__ nxt) __attribute__((always_inline)) {
        if (j + 1 < nkt) dma(nxt, j + 1);
        if (j < n_free && j >= f_lo) tile(cur, j * QBN, std::integral_constant<int, 0>{});
        else tile(cur, j * QBN, std::integral_constant<int, TTT_ ? 1 : 2>{});
      };
      step(&sm.buf[(j - kt_lo) & 1], &sm.buf[(j - kt_lo + 1) & 1]);
      TTT_WAIT_VMCNT(0);  // tile j+1 has landed
      __syncthreads();    // and every wave is done with tile j
    }
  } else {
    // dQ~^T += K~^T dS^T over key groups j = 0 .. rb of this wave's row block
    // rb.  Each wave loads the K~^T quarter of its lanes' roles and its own dS
    // block (2 + 2 loads per tile); the dS loads run DS_NS - 1 tiles ahead, the
    // K~^T loads DS_NK - 1.
    // wave-uniform in scalar registers: the dS loads' buffer descriptors and
    // the compute branch stay scalar
    const int rbw = __builtin_amdgcn_readfirstlane(wave_row0 >> 5);
    const int hu = __builtin_amdgcn_readfirstlane(h);
    const int wu = __builtin_amdgcn_readfirstlane(wv);  // the LDS bases stay scalar
    const bool wave_on = (rbw << 5) < L;
    const int rbl = min(rbw, ((L + 31) >> 5) - 1);  // loads stay inside this head's blocks
    const _Float16* dsh = P.ds + ((int64_t)(b * P.Hq + hu) * P.ds_tri + (int64_t)rbl * (rbl + 1) / 2) * 1024;
    uint32_t dso[2];  // piece c = 64 i + lane -> LDS slot c: key c/4, quarter c%4
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = 64 * i + lane, key = c >> 2, qu = c & 3;
      dso[i] = (uint32_t)((qu >> 1) * 1024 + ((qu & 1) * 32 + key) * 16);
    }
    // transposing reads of the dS^T operand (lane: row n = lane % 32, keys
    // 8 (lane / 32) + 4 ri + 0..3 of chunk c2): 16-lane group G serves rows
    // 16 (G % 2) + 0..15; its lane s points at key 4 ri + s/4 + (chunk base),
    // rows 4 (s % 4) + 0..3 of that half
    uint32_t tro[2][2];
    {
      const int G = lane >> 4, s16 = lane & 15;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int ri = 0; ri < 2; ++ri) {
          const int key = 16 * c2 + 8 * (G >> 1) + 4 * ri + (s16 >> 2);
          const int qu = (G & 1) * 2 + ((s16 & 3) >> 1);
          tro[c2][ri] = (uint32_t)((key * 4 + qu) * 16 + (s16 & 1) * 8);
        }
    }
    auto kdma = [&](_Float16* __restrict__ dst, int j) __attribute__((always_inline)) {
      const buf_rsrc tr = make_rsrc(ktbase + (int64_t)j * D * QBN, kt_bytes);
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16(tr, toff[i] * 2, dst + 16 * (2 * wu + i) * QBN);
    };
    auto sdma = [&](_Float16* __restrict__ dst, int j) __attribute__((always_inline)) {
      const buf_rsrc dr = make_rsrc(dsh + (int64_t)min(j, rbl) * 1024, 2048);
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16_nt(dr, dso[i], dst + 512 * i);
    };
    // Issue order: the prologue's dS tiles, then its K~^T tiles; then per tile
    // j the dS of j + DS_NS - 1 and the K~^T of j + DS_NK - 1.  Loads retire in
    // issue order, so after tile j's loads the ones for tile j + 1 are done
    // once at most the count issued during tile j is still in flight.
#pragma unroll
    for (int t = 0; t < DS_NS - 1; ++t)
      if (t < nkt) sdma(&sm.dr.ds[t][wu][0], t);
#pragma unroll
    for (int t = 0; t < DS_NK - 1; ++t)
      if (t < nkt) kdma(&sm.dr.kt[t][0], t);
    if (nkt > 1) TTT_WAIT_VMCNT(2);  // tile 0 (K~^T of tile 1 may fly)
    else TTT_WAIT_VMCNT(0);
    lds_ring_barrier();
    for (int j = 0; j < nkt; ++j) {
      auto step = [&](const _Float16* __restrict__ ck, const _Float16* __restrict__ cs, _Float16* __restrict__ nk,
                      _Float16* __restrict__ ns) __attribute__((always_inline)) {
        const bool ls = j + DS_NS - 1 < nkt, lk = j + DS_NK - 1 < nkt;
        if (ls) sdma(ns, j + DS_NS - 1);
        if (lk) kdma(nk, j + DS_NK - 1);
        if (wave_on && j <= rbw) {
          const char* dsw = (const char*)cs;
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const s16x4 x0 = lds_read_tr16(dsw + tro[c2][0]), x1 = lds_read_tr16(dsw + tro[c2][1]);
            const f16x8 bop = __builtin_bit_cast(f16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
            f16x8 a[4];
#pragma unroll
            for (int d4 = 0; d4 < 4; ++d4) {
              const int d = d4 * 32 + l32;
              a[d4] = *(const f16x8*)&ck[d * QBN + (((2 * c2 + hf) ^ ((d >> 2) & 3)) * 8)];
            }
#pragma unroll
            for (int d4 = 0; d4 < 4; ++d4) acc[d4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[d4], bop, acc[d4], 0, 0, 0);
          }
        }
        // tile j+1 has landed when only this tile's issues may still fly
        const int fly = (ls ? 2 : 0) + (lk ? 2 : 0);
        if (fly == 4) TTT_WAIT_VMCNT(4);
        else if (fly == 2) TTT_WAIT_VMCNT(2);
        else TTT_WAIT_VMCNT(0);
      };
      step(&sm.dr.kt[j % DS_NK][0], &sm.dr.ds[j % DS_NS][wu][0], &sm.dr.kt[(j + DS_NK - 1) % DS_NK][0],
           &sm.dr.ds[(j + DS_NS - 1) % DS_NS][wu][0]);
      lds_ring_barrier();  // and every wave is done with tile j
    }
  }
  // block drafting: the keys of the work item's own blocks (bs divides 32, so
  // the blocks of rows row0 .. qend-1 are exactly key rows row0 .. qend-1)
  if constexpr (MODE == 1) {
    const _Float16* kbb = kbt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0) * D;
    const _Float16* ktbb = kbtt + (int64_t)(b * P.Hkv + g) * D * P.spad + (int64_t)(slot0 >> 5) * D * QBN;
    const uint16_t* vbb = (const uint16_t*)kv.v[1] + b * P.ks_b + (int64_t)start * P.ks_t + g * P.ks_h;
    for (int k0 = row0; k0 < qend; k0 += QBN) {
      dma_from(&sm.buf[0], kbb, ktbb, vbb, P.ks_t, k0, L - 1);
      TTT_WAIT_VMCNT(0);
      __syncthreads();
      tile(&sm.buf[0], k0, std::integral_constant<int, 3>{});
      __syncthreads();
    }
  }
  {
    const int lr = wv * 32 + l32;
    const float qsc = P.scale * __builtin_amdgcn_ldexpf(1.0f, -eq);  // sigma, and the dS factor undone
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[d4][v4 * 4 + e] * qsc;
        *(f32x4*)&sm.acc[lr][d4 * 32 + v4 * 8 + hf * 4] = w;
      }
  }
  __syncthreads();

  // Fused branch gradients (every query head of the KV group in this work
  // item, P.dq_branch): per 16 rows, passes outer and heads inner, 16 threads
  // per row, 8 elements (4 rotate-half pairs d, d + 64) per thread.  For
  // branch key q of row i and head h: P = exp(s - LSE), dS = P (<dO, v> -
  // Delta); dQ~ += sigma dS k~ (into the LDS rows), dk~^(q) += sigma dS q~ and
  // dv^(q) += P dO summed over the heads in registers, then un-rotated and
  // stored once: no atomics, no second pass over Q and dO.
  if constexpr (TTT_) {
    if (P.dq_branch && P.branch && P.p > 1) {
      const int c16 = tid & 15;
      const int flo = c16 * 4, fhi = 64 + c16 * 4;
#pragma unroll 1
      for (int r16 = 0; r16 < RT; r16 += 16) {
        const int rr = r16 + (tid >> 4);  // row within the work item
        const int i = row0 + rr;
        if (i >= L) continue;
        const int pos = qoff + i + P.p - 1;
        // per head: q~ as fp16 pairs and dO as its bf16 pairs (8 values each)
        u32x2 qh[RH][2], gh[RH][2];
        float lse_[RH], dl_[RH];
        {
          const f32x4 cq = *(const f32x4*)(cosT + rope_off(P, pos) + flo);
          const f32x4 sq = *(const f32x4*)(sinT + rope_off(P, pos) + flo);
#pragma unroll
          for (int hw_ = 0; hw_ < RH; ++hw_) {
            const int hh = g * P.r + hw_;
            const uint16_t* qrow = q + b * P.qs_b + (int64_t)(start + i) * P.qs_t + hh * P.qs_h;
            const uint16_t* grow = dout + b * P.os_b + (int64_t)(start + i) * P.os_t + hh * P.os_h;
            const u32x2 qa = *(const u32x2*)(qrow + flo), qb = *(const u32x2*)(qrow + fhi);
            float y1[4], y2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t wa = qa[e >> 1], wb = qb[e >> 1];
              const float x1 = __uint_as_float((e & 1) ? (wa & 0xffff0000u) : (wa << 16));
              const float x2 = __uint_as_float((e & 1) ? (wb & 0xffff0000u) : (wb << 16));
              y1[e] = x1 * cq[e] - x2 * sq[e];
              y2[e] = x2 * cq[e] + x1 * sq[e];
            }
            qh[hw_][0] = u32x2{pack_h2(y1[0], y1[1]), pack_h2(y1[2], y1[3])};
            qh[hw_][1] = u32x2{pack_h2(y2[0], y2[1]), pack_h2(y2[2], y2[3])};
            gh[hw_][0] = *(const u32x2*)(grow + flo);
            gh[hw_][1] = *(const u32x2*)(grow + fhi);
            lse_[hw_] = lse[b * P.lse_b + hh * P.lse_h + start + i];
            dl_[hw_] = delta[(int64_t)(b * P.Hq + hh) * P.spad + slot0 + i];
          }
        }
        const int64_t koff = b * P.ks_b + (int64_t)(start + i) * P.ks_t + g * P.ks_h;
        // pass q's key/value pieces and cos/sin, loaded one pass ahead
        u32x2 nka, nkb, nva, nvb;
        f32x4 nck, nsk;
        auto load_pass = [&](int qq) __attribute__((always_inline)) {
          const uint16_t* krow_ = (const uint16_t*)kv.k[qq - 1] + koff;
          const uint16_t* vrow_ = (const uint16_t*)kv.v[qq - 1] + koff;
          nka = *(const u32x2*)(krow_ + flo);
          nkb = *(const u32x2*)(krow_ + fhi);
          nva = *(const u32x2*)(vrow_ + flo);
          nvb = *(const u32x2*)(vrow_ + fhi);
          const int pk = qoff + i + qq - 1;
          nck = *(const f32x4*)(cosT + rope_off(P, pk) + flo);
          nsk = *(const f32x4*)(sinT + rope_off(P, pk) + flo);
        };
        load_pass(2);
        for (int qq = 2; qq <= P.p; ++qq) {
          const u32x2 ka = nka, kb = nkb;
          const u32x2 vv[2] = {nva, nvb};
          const f32x4 ck = nck, sk = nsk;
          if (qq < P.p) load_pass(qq + 1);
          float kr[8], dk_[8], dv_[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wa = ka[e >> 1], wb = kb[e >> 1];
            const float x1 = __uint_as_float((e & 1) ? (wa & 0xffff0000u) : (wa << 16));
            const float x2 = __uint_as_float((e & 1) ? (wb & 0xffff0000u) : (wb << 16));
            kr[e] = x1 * ck[e] - x2 * sk[e];
            kr[4 + e] = x2 * ck[e] + x1 * sk[e];
          }
          const uint32_t krh[4] = {pack_h2(kr[0], kr[1]), pack_h2(kr[2], kr[3]), pack_h2(kr[4], kr[5]),
                                   pack_h2(kr[6], kr[7])};
#pragma unroll
          for (int e = 0; e < 8; ++e) dk_[e] = dv_[e] = 0.f;
#pragma unroll
          for (int hw_ = 0; hw_ < RH; ++hw_) {
            float ps = 0.f, pd = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                // vector elements go through scalars: a bit cast of an element
                // subscript itself reads element 0
                const uint32_t qw = qh[hw_][c][w], gw = gh[hw_][c][w], vw = vv[c][w], kw = krh[2 * c + w];
                ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qw), __builtin_bit_cast(h2v, kw), ps, false);
                pd = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2v, gw), __builtin_bit_cast(b2v, vw), pd, false);
              }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
              ps += __shfl_xor(ps, m, 64);
              pd += __shfl_xor(pd, m, 64);
            }
            const float pr = __expf(ps * P.scale - lse_[hw_]);
            const float dsv = pr * (pd - dl_[hw_]) * P.scale;
            // the LDS row of (head, row): wave (rr/32)*RH + head, lane row rr%32
            float* arow = sm.acc[((rr >> 5) * RH + hw_) * 32 + (rr & 31)];
            f32x4 xl = *(const f32x4*)&arow[flo], xh = *(const f32x4*)&arow[fhi];
#pragma unroll
            for (int e = 0; e < 4; ++e) xl[e] += dsv * kr[e], xh[e] += dsv * kr[4 + e];
            *(f32x4*)&arow[flo] = xl;
            *(f32x4*)&arow[fhi] = xh;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                const uint32_t qw = qh[hw_][c][w], gw = gh[hw_][c][w];
                const h2v qv = __builtin_bit_cast(h2v, qw);
                dk_[c * 4 + 2 * w] += dsv * (float)qv[0];
                dk_[c * 4 + 2 * w + 1] += dsv * (float)qv[1];
                dv_[c * 4 + 2 * w] += pr * __uint_as_float(gw << 16);
                dv_[c * 4 + 2 * w + 1] += pr * __uint_as_float(gw & 0xffff0000u);
              }
          }
          float lo[4], hi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = dk_[e] * ck[e] + dk_[4 + e] * sk[e];
            hi[e] = dk_[4 + e] * ck[e] - dk_[e] * sk[e];
          }
          if (P.out_f32) {  // ring-step terms: fp32
            float* fk = (float*)gr.dk[qq - 1] + koff;
            float* fv = (float*)gr.dv[qq - 1] + koff;
            *(f32x4*)(fk + flo) = f32x4{lo[0], lo[1], lo[2], lo[3]};
            *(f32x4*)(fk + fhi) = f32x4{hi[0], hi[1], hi[2], hi[3]};
            *(f32x4*)(fv + flo) = f32x4{dv_[0], dv_[1], dv_[2], dv_[3]};
            *(f32x4*)(fv + fhi) = f32x4{dv_[4], dv_[5], dv_[6], dv_[7]};
          } else {
            uint16_t* dkrow = (uint16_t*)gr.dk[qq - 1] + koff;
            uint16_t* dvrow = (uint16_t*)gr.dv[qq - 1] + koff;
            *(u32x2*)(dkrow + flo) = u32x2{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3])};
            *(u32x2*)(dkrow + fhi) = u32x2{pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])};
            *(u32x2*)(dvrow + flo) = u32x2{pack_bf2(dv_[0], dv_[1]), pack_bf2(dv_[2], dv_[3])};
            *(u32x2*)(dvrow + fhi) = u32x2{pack_bf2(dv_[4], dv_[5]), pack_bf2(dv_[6], dv_[7])};
          }
        }
      }
      __syncthreads();  // the dQ~ rows are updated across threads
    }
  }

  const int c8 = tid & 7;
  const int dlo = c8 * 8, dhi = 64 + c8 * 8;
  // row-major epilogue: branch terms (unless fused above), un-rotation, store.
  // LDS row lr holds wave lr/32's row lr%32.
  for (int rp = 0; rp < 128; rp += 32) {
    const int lr = rp + (tid >> 3);
    const int w_ = lr >> 5;
    const int hh = g * P.r + sub * RH + w_ % RH;
    const int i = row0 + (w_ / RH) * 32 + (lr & 31);
    if (i >= L) continue;
    float a[16];
    {
      const f32x4* x = (const f32x4*)&sm.acc[lr][dlo];
      const f32x4* y = (const f32x4*)&sm.acc[lr][dhi];
      f32x4 x0 = x[0], x1 = x[1], y0 = y[0], y1 = y[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = x0[e], a[4 + e] = x1[e], a[8 + e] = y0[e], a[12 + e] = y1[e];
    }
    const int pos = TTT_ ? qoff + i + P.p - 1 : blk_anchor(P, bq, i) + (i & ((1 << P.bs_log2) - 1));
    const float* cq = cosT + rope_off(P, pos) + dlo;
    const float* sq = sinT + rope_off(P, pos) + dlo;
    if (TTT_ && P.p > 1 && P.branch && !P.dq_branch) {
      float qr[16], go[16];
      {
        const uint16_t* qrow = q + b * P.qs_b + (int64_t)(start + i) * P.qs_t + hh * P.qs_h;
        const uint16_t* grow = dout + b * P.os_b + (int64_t)(start + i) * P.os_t + hh * P.os_h;
        float x1[8], x2[8];
        unpack_bf8(*(const u32x4*)(qrow + dlo), x1);
        unpack_bf8(*(const u32x4*)(qrow + dhi), x2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qr[e] = x1[e] * cq[e] - x2[e] * sq[e];
          qr[8 + e] = x2[e] * cq[e] + x1[e] * sq[e];
        }
        unpack_bf8(*(const u32x4*)(grow + dlo), go);
        unpack_bf8(*(const u32x4*)(grow + dhi), go + 8);
      }
      const float lse_i = lse[b * P.lse_b + hh * P.lse_h + start + i];
      const float dl_i = delta[(int64_t)(b * P.Hq + hh) * P.spad + slot0 + i];
      const int64_t koff = b * P.ks_b + (int64_t)(start + i) * P.ks_t + g * P.ks_h;
      for (int qq = 2; qq <= P.p; ++qq) {
        const uint16_t* krow_ = (const uint16_t*)kv.k[qq - 1] + koff;
        const uint16_t* vrow_ = (const uint16_t*)kv.v[qq - 1] + koff;
        float x1[8], x2[8], v1[8], v2[8];
        unpack_bf8(*(const u32x4*)(krow_ + dlo), x1);
        unpack_bf8(*(const u32x4*)(krow_ + dhi), x2);
        unpack_bf8(*(const u32x4*)(vrow_ + dlo), v1);
        unpack_bf8(*(const u32x4*)(vrow_ + dhi), v2);
        const int pk = qoff + i + qq - 1;
        const float* ck = cosT + rope_off(P, pk) + dlo;
        const float* sk = sinT + rope_off(P, pk) + dlo;
        float kr[16];
        float ps = 0.f, pd = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kr[e] = x1[e] * ck[e] - x2[e] * sk[e];
          kr[8 + e] = x2[e] * ck[e] + x1[e] * sk[e];
          ps += qr[e] * kr[e] + qr[8 + e] * kr[8 + e];
          pd += go[e] * v1[e] + go[8 + e] * v2[e];
        }
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) {
          ps += __shfl_xor(ps, m, 64);
          pd += __shfl_xor(pd, m, 64);
        }
        const float pr = __expf(ps * P.scale - lse_i);
        const float dsv = pr * (pd - dl_i) * P.scale;
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] += dsv * kr[e];
      }
    }
    float res[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      res[e] = a[e] * cq[e] + a[8 + e] * sq[e];
      res[8 + e] = a[8 + e] * cq[e] - a[e] * sq[e];
    }
    const int64_t oi = b * P.qs_b + (int64_t)(start + i) * P.qs_t + hh * P.qs_h;
    if (P.out_f32) {  // ring-step terms: fp32, q's element strides
      float* orow = (float*)dq + oi;
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        *(f32x4*)(orow + dlo + e) = f32x4{res[e], res[e + 1], res[e + 2], res[e + 3]};
        *(f32x4*)(orow + dhi + e) = f32x4{res[8 + e], res[9 + e], res[10 + e], res[11 + e]};
      }
    } else {
      uint16_t* orow = dq + oi;
      *(u32x4*)(orow + dlo) = pack_bf8(res);
      *(u32x4*)(orow + dhi) = pack_bf8(res + 8);
    }
  }
}

// ============================================================================= dK/dV (trunk)
// Per 32-query step the workgroup stages Q~ rows and dO rows (8 KB each) plus
// the rows' LSE and Delta HBM -> LDS with direct loads (buffer_load ... lds),
// XOR-swizzled (16-byte chunk c of row r at slot c ^ swz(r), swz swapping the
// two 2-bit halves of r & 15) so that the MFMA operand reads are conflict-free:
// a row read covers 16 distinct rows, and a transposed read's 4 consecutive
// rows land on 4 distinct 64-byte bank groups.  The transposed operands of
// dV^T += dO^T P and dK~^T += Q~^T dS are column reads of the same tiles
// (ds_read_b64_tr_b16), so no transposed copy is streamed.
// Software pipeline (one wave per SIMD): iteration i issues the loads of step
// i+3 into a 4-deep ring of LDS buffers, runs the S/dP products of step i+1,
// the softmax of step i (whose S/dP came from iteration i-1) and step i's
// dV/dK products, so the matrix pipe has independent work while the vector
// ALUs run the softmax.  Each wave issues 4 loads per step (wave 0 a fifth:
// the LSE and Delta; block drafting, context keys: wave 1 a fifth, the
// anchors), so one vmcnt threshold per wave releases exactly the step two
// ahead.
constexpr int NBUF = 4;
constexpr int KST_PITCH = 1024 + 16;  // dK/dV key staging: 4 rows of 256 bytes, padded
constexpr int kDsStoreAux = 2;  // cache policy of the stored-dS writes: non-temporal
__device__ __forceinline__ int kv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
struct KvBuf {
  _Float16 q[BQ * D];   // Q~ rows   (A of S; columns: A of dK^T)
  uint16_t g[BQ * D];   // dO rows   (A of dP; columns: A of dV^T)
  float lse[BQ];        // LSE of the rows, log2 units
  float dl[BQ];         // Delta of the rows
  int anc[2 * BQ];      // block drafting, context keys: the rows' clamped block anchors (twice)
};


// MODE 0: TTT pass (trunk keys, rows i >= j); MODE 4: the same with a
// sliding window (rows j <= i < j + win).  Block drafting: MODE 2 the
// context keys (P.kv_len of them; row i sees key j < its block's anchor),
// MODE 3 the block keys (seen by the rows of their own block only).  kt, kv.v[0]
// and gr.dk[0] / gr.dv[0] are those keys' K~ slab, V and gradients (P.ks_*
// strides).
template <int MODE>
__global__ void __launch_bounds__(256, 1)
    dkdv_bf16_kernel(Prob P, PassPtrs kv, const float* __restrict__ lse, const uint16_t* __restrict__ dout,
                     const _Float16* __restrict__ kt, const _Float16* __restrict__ qt,
                     const float* __restrict__ delta, const int4* __restrict__ tiles, const float* __restrict__ cosT,
                     const float* __restrict__ sinT, PassGradPtrs gr) {
  __shared__ __attribute__((aligned(16))) KvBuf sm[NBUF];
  // the work item's K~ and V rows, staged once (4 rows per padded 1 KB) in
  // the step ring before its first loads: no LDS beyond the ring
  static_assert(2 * BKV / 4 * KST_PITCH <= NBUF * sizeof(KvBuf), "key staging fits the ring");
  typedef unsigned char KvStage[BKV / 4 * KST_PITCH];
  KvStage* kvst = reinterpret_cast<KvStage*>(&sm[0]);
  // TTT pass (4: with a sliding window; 5: also storing dS for the dQ kernel)
  constexpr bool TTT_ = MODE == 0 || MODE == 4 || MODE == 5;
  const int win = MODE == 4 ? P.win : 0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  // Order: key tiles heavy-first (ascending tile index), and every (batch, KV
  // group) pair pinned to one XCD (blockIdx % 8), so the tiles of a pair that
  // run together share that XCD's L2 for the query rows they all stream.
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  int b, t, start, L, slot0, g;
  int kst = 0, kln;  // this work item's keys: token rows kst .. kst + kln of the key tensors
  int kvoff = 0, dq_ = 0;  // TTT: key j sits at kvoff + j; row i sees it iff i >= j - dq_
  const int nkeys = MODE == 3 ? P.stok : P.kv_len;  // TTT: kv_len = stok for whole-sequence calls
  if (P.layout == 0) {
    const int nkt = (nkeys + BKV - 1) / BKV;
    const int ppx = (P.B * P.Hkv + 7) / 8;  // pairs per XCD
    t = slot / ppx;
    const int pair = (slot % ppx) * 8 + xcd;
    if (t >= nkt || pair >= P.B * P.Hkv) return;
    b = pair / P.Hkv;
    g = pair % P.Hkv;
    start = 0;
    L = P.stok;
    slot0 = 0;
  } else {
    g = blockIdx.x % P.Hkv;
    const int tix = blockIdx.x / P.Hkv;
    if (tix >= tiles[0].x) return;
    const int4 e = tiles[1 + tix];
    t = e.x, start = e.y, L = e.z, slot0 = e.w, b = 0;
  }
  kln = (MODE == 2 || (TTT_ && P.layout == 0)) ? nkeys : L;
  BlkSeq bq{};  // block drafting: the sequence's anchors and context
  if constexpr (MODE == 2 || MODE == 3) {
    if (P.layout == 1) {
      // THD lists key tiles: context keys (MODE 2) per context segment, block
      // keys (MODE 3) per sequence; the rows are the sequence's block rows
      kst = start;
      kln = L;
      if constexpr (MODE == 2) {
        const int s = seq_at(P.kv_cu, P.nseq, start);
        int b_;
        seq_info(P, s, b_, start, L);
        bq = blk_seq_of(P, s);
      } else {
        bq = blk_seq(P, 0, start);
      }
    } else {
      bq = blk_seq(P, b, 0);
    }
  }
  if constexpr (TTT_) {
    // THD ring steps list key segments: the rows are the same segment's query rows
    if (P.layout == 1 && P.kv_cu) {
      const int s = seq_at(P.kv_cu, P.nseq, start);
      int b_;
      kst = start;
      seq_info(P, s, b_, start, L);
    } else {
      kst = P.layout == 1 ? start : 0;
    }
    int qoff, kvs_, kvn_;
    seq_ring(P, P.layout == 1 && P.kv_cu ? seq_at(P.kv_cu, P.nseq, kst) : b, start, L, qoff, dq_, kvs_, kvn_);
    kvoff = qoff - dq_;
  }
  const int kv0 = t * BKV;
  const int my_key = kv0 + wv * 32 + l32;
  const int key_end = kln;  // keys of this slab
  const bool key_ok = my_key < key_end;
  // query rows [row_lo, row_hi) that can see this key tile
  int row_lo = TTT_ ? max(0, kv0 - dq_) & ~(BQ - 1) : kv0, row_hi = L;
  if constexpr (MODE == 3) row_hi = min(kv0 + BKV, L);
  if constexpr (TTT_)
    if (win > 0) row_hi = min(L, max(0, kv0 + BKV - 1 - dq_ + win));  // sliding window: rows i < j - dq_ + win
  if constexpr (MODE == 2) {
    // the first block whose anchor passes kv0 (any anchor order): rows before
    // it see no key here.  Every wave scans all anchors itself: no shared
    // memory or barrier before the staging ring.
    const int nb = L >> P.bs_log2;  // the sequence's blocks
    int first = nb;
    for (int n = lane; n < nb; n += 64)
      if (blk_anchor(P, bq, n << P.bs_log2) > kv0) first = min(first, n);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) first = min(first, __shfl_xor(first, m, 64));
    row_lo = min(__builtin_amdgcn_readfirstlane(first) << P.bs_log2, L) & ~(BQ - 1);
  }
  // position of this lane's key (block keys: the slot position in its block)
  int kpos = TTT_ ? kvoff + my_key : my_key;
  if constexpr (MODE == 3) kpos = key_ok ? blk_anchor(P, bq, my_key) + (my_key & ((1 << P.bs_log2) - 1)) : 0;
  if constexpr (!TTT_) {
    // every global load above has landed before the first staging load: the
    // compiler's load counter is then exact and no full wait lands in the loop
    TTT_WAIT_VMCNT(0);
    asm volatile("" ::"v"(kpos), "s"(row_lo));
  }

  // This lane's key fragments: the work item's K~ rows (contiguous) and V rows
  // come in through LDS as whole 256-byte rows, 16 lanes per row (per-lane
  // 32-byte pieces of 32 rows would move several times the bytes through the
  // load path), and each lane reads its pieces back.
  f16x8 kf[8];
  bf16x8 vf[8];
  {
    const int wu = __builtin_amdgcn_readfirstlane(wv);
    const int nk = min(BKV, kln - kv0);  // keys of the slab in this work item (may be <= 0)
    const buf_rsrc kr = make_rsrc(kt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0 + kv0) * D, BKV * D * 2);
    const buf_rsrc vr = make_rsrc((const uint16_t*)kv.v[0] + b * P.ks_b + (int64_t)(kst + kv0) * P.ks_t + g * P.ks_h,
                                  nk > 0 ? (uint32_t)((nk - 1) * P.ks_t * 2 + D * 2) : 0u);
#pragma unroll
    for (int j = 0; j < BKV / 4 / 4; ++j) {  // each wave stages 32 rows, 4 per instruction
      const int n = wu * (BKV / 4) + 4 * j;   // first row of this instruction's four
      const int r = n + (lane >> 4);
      lds_dma16(kr, (uint32_t)((r * D + (lane & 15) * 8) * 2), &kvst[0][(n >> 2) * KST_PITCH]);
      lds_dma16(vr, (uint32_t)(r * P.ks_t * 2 + (lane & 15) * 16), &kvst[1][(n >> 2) * KST_PITCH]);
    }
    TTT_WAIT_VMCNT(0);
    __syncthreads();
    const int rr = wv * 32 + l32;
    const int lo = (rr >> 2) * KST_PITCH + (rr & 3) * D * 2;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d0 = c * 16 + hf * 8;
      kf[c] = *(const f16x8*)&kvst[0][lo + d0 * 2];
      u32x4 x = *(const u32x4*)&kvst[1][lo + d0 * 2];
      if (!key_ok) x = u32x4{0, 0, 0, 0};
      vf[c] = __builtin_bit_cast(bf16x8, x);
    }
    lds_ring_barrier();  // every wave has its fragments before the ring is refilled
  }
  // fp16 dS operands carry a per-key factor 2^e: |dS_ij| <= P_ij (|<dO_i, v_j>|
  // + |Delta_i|) <= N ||v_j||_inf + Dm, with N = max ||dO_i||_1 and Dm = max
  // |Delta_i| over the rows of the group's heads (reduced after the Delta
  // kernel).  Folded in exactly: V is scaled by 2^e (so dP is), Delta is
  // scaled inside the fma that forms dP - Delta, and dK~ is unscaled in the
  // epilogue; dV (from P) is untouched.
  float vinf = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4 x = __builtin_bit_cast(u32x4, vf[c]);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      vinf = fmaxf(vinf, fmaxf(fabsf(__uint_as_float(x[w] << 16)), fabsf(__uint_as_float(x[w] & 0xffff0000u))));
  }
  vinf = xhalf_max(vinf);  // the key's whole row
  if constexpr (MODE != 5) {
    float wmax = vinf;  // the wave's 32 keys, for the dQ kernel's bound
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, m, 64));
    // only waves whose keys start inside the slab: in THD the slots past a
    // short sequence's end belong to the next sequence
    float* vm = MODE == 3 ? P.vmax_b : P.vmax;
    if (lane == 0 && kv0 + wv * 32 < key_end)
      vm[(int64_t)(b * P.Hkv + g) * (P.spad / 32) + (slot0 + kv0) / 32 + wv] = wmax;
  }
  const float2 nd = *(const float2*)&P.dmax[(int64_t)(b * P.Hkv + g) * 2];
  // stored dS: one exponent for the whole KV group (the dQ kernel forms the
  // same one), from the group's largest |v_jd|
  const int ek = ds_exp(__builtin_fmaf(nd.x, MODE == 5 ? P.vgmax[b * P.Hkv + g] : vinf, nd.y));
  const float cj = __builtin_amdgcn_ldexpf(1.0f, ek);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    u32x4 x = __builtin_bit_cast(u32x4, vf[c]);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      x[w] = pack_bf2(__uint_as_float(x[w] << 16) * cj, __uint_as_float(x[w] & 0xffff0000u) * cj);
    vf[c] = __builtin_bit_cast(bf16x8, x);
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[d4][v] = dv[d4][v] = 0.f;
  const int prow = perm_row(l32);
  const float sl2 = P.scale_log2;

  // Steps st = 0..nsteps-1: head st % r of row block nq-1-st/r (from the
  // sequence end downwards).  The loads run three steps ahead of the compute;
  // both sides advance (head, row block) counters instead of dividing.
  const int nq = max(0, (row_hi - row_lo + BQ - 1) / BQ);
  const int nsteps = P.r * nq;
  // DMA lane roles (wave w issues instructions j = 2w, 2w+1 of each 8 KB tile):
  // rows r = 4j + lane/16, slot lane%16.  Every step builds buffer descriptors
  // at its (head, first row) bases; the lanes add fixed byte offsets.
  int rrow[2];
  uint32_t q_lane[2], c_lane[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = 2 * wv + i;
    const int r = 4 * j + (lane >> 4);
    const int roff = ((lane & 15) ^ kv_swz(r)) * 8;
    rrow[i] = r;
    q_lane[i] = (uint32_t)((r * D + roff) * 2);
    c_lane[i] = (uint32_t)(roff * 2);
  }
  const _Float16* q_base = qt + ((int64_t)(b * P.Hq + g * P.r) * P.spad + slot0) * D;
  const uint16_t* g_base = dout + b * P.os_b + (int64_t)start * P.os_t + (int64_t)(g * P.r) * P.os_h;
  // LSE (log2 units, +inf past the rows' end) and Delta of a step's 32 rows:
  // one dword load by wave 0 from the workspace, lanes 0..31 the LSE, lanes
  // 32..63 Delta (they land in lse[] and the dl[] that follows it).
  const float* m_base = delta + (int64_t)(b * P.Hq + g * P.r) * P.spad + slot0;
  const uint32_t m_lane = (uint32_t)(((lane < 32 ? (int64_t)P.B * P.Hq * P.spad : 0) + (lane & 31)) * 4);
  int is_h = 0, is_q0 = row_lo + (nq - 1) * BQ;  // the next step to load
  // block drafting, context keys: wave 1 loads the step's rows' visible context
  // lengths (clamped anchors, staged per slot in the workspace after the LSE)
  const bool w1a = MODE == 2 && wv == 1;
  const int* a_base =
      MODE == 2 ? (const int*)(delta + (int64_t)2 * P.B * P.Hq * P.spad) + (int64_t)b * P.spad + slot0 : nullptr;
  auto issue = [&](KvBuf* __restrict__ Bd) __attribute__((always_inline)) {
    KvBuf& B = *Bd;
    const buf_rsrc qr = make_rsrc(q_base + ((int64_t)is_h * P.spad + is_q0) * D, BQ * D * 2);
    const buf_rsrc gr_ = make_rsrc(g_base + (int64_t)is_h * P.os_h + (int64_t)is_q0 * P.os_t, 0xFFFFFFFFu);
    // dO rows past the sequence end repeat the last row: their probabilities
    // are 0 (LSE +inf), so they add nothing
    const int rmax = L - 1 - is_q0;
    const int wu = __builtin_amdgcn_readfirstlane(wv);  // the LDS bases stay scalar
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = 2 * wu + i;
      lds_dma16(qr, q_lane[i], &B.q[4 * j * D]);
      lds_dma16(gr_, (uint32_t)(min(rrow[i], rmax) * P.os_t * 2) + c_lane[i], &B.g[4 * j * D]);
    }
    if (wv == 0) lds_dma4(make_rsrc(m_base + (int64_t)is_h * P.spad + is_q0, 0xFFFFFFFFu), m_lane, &B.lse[0]);
    if (w1a) lds_dma4(make_rsrc(a_base + is_q0, BQ * 4), (uint32_t)(lane & 31) * 4, &B.anc[0]);
    if (++is_h == P.r) {
      is_h = 0;
      is_q0 -= BQ;
    }
  };
  // loads each wave has in flight per step (wave 0 also loads LSE/Delta, and
  // wave 1 the anchors for the context keys of block drafting)
  const bool w0 = wv == 0 || w1a;

  // S = Q~ K~^T and dP = dO V^T for step st (this wave's 32 keys x 32 rows).
  auto products = [&](const KvBuf* __restrict__ Bp, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    const KvBuf& B = *Bp;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = dp[v] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < 8; c0 += 4) {
      f16x8 a[4];
      bf16x8 a2[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int off = prow * D + (((2 * (c0 + c) + hf) ^ kv_swz(prow)) * 8);
        a[c] = *(const f16x8*)&B.q[off];
        a2[c] = *(const bf16x8*)&B.g[off];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c], kf[c0 + c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[c], vf[c0 + c], dp, 0, 0, 0);
      }
    }
  };
  // prologue: steps 0..2 in flight, steps 0 and 1 landed
#pragma unroll
  for (int st = 0; st < 3; ++st)
    if (st < nsteps) issue(&sm[st]);
  if (nsteps >= 3) {  // leaves only step 2's loads outstanding
    if (w0) TTT_WAIT_VMCNT(5);
    else TTT_WAIT_VMCNT(4);
  } else {
    TTT_WAIT_VMCNT(0);
  }
  __syncthreads();
  f32x16 s_c, dp_c;
  products(&sm[0], s_c, dp_c);

  // Rows past the sequence end need no mask: their staged LSE is +inf, so
  // their probabilities are 0 and they add nothing to dK or dV.
  // The causal mask (rows before this lane's key) is one compare per score.
  // The three ring buffers an iteration touches go through distinct restrict
  // pointers: the compiler then knows the loads into the step-(st+3) buffer
  // cannot alias this iteration's LDS reads and puts no wait on them.
  int cs_h = 0, cs_q0 = row_lo + (nq - 1) * BQ;  // the step being computed
  // Stored dS (MODE 5): step st's block is written in step st+1, right after
  // that step's loads are issued.  Vector memory operations retire in issue
  // order, so a step's closing wait -- for the loads issued one step earlier --
  // can leave every younger operation in flight: the newest loads and the
  // stores of this and the previous step.  Each store thus has two steps to
  // drain.  Blocks above the diagonal (row block < key group) are not part of
  // the layout.
  f16x8 dsp[2];
  int sp_h = 0, sp_q0 = 0;
  int stored_prev = 0, stored_now = 0;  // stores issued in the previous / this step (0 or 2)
  const int kgrp = (kv0 >> 5) + wv;  // this wave's key group of 32
  auto store_ds = [&]() __attribute__((always_inline)) {
    const int rb = sp_q0 >> 5;
    if (rb < kgrp) return 0;
    const _Float16* blk =
        P.ds + ((int64_t)(b * P.Hq + g * P.r + sp_h) * P.ds_tri + (int64_t)rb * (rb + 1) / 2 + kgrp) * 1024;
    // read once, by the dQ kernel: non-temporal, so the Q~ / dO rows this
    // kernel re-reads keep their cache lines
    const buf_rsrc r = make_rsrc(blk, 2048);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dsp[0]), r, lane * 16, 0, kDsStoreAux);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dsp[1]), r, 1024 + lane * 16, 0, kDsStoreAux);
    return 2;
  };
  auto wait_vm = [&](int n) __attribute__((always_inline)) {
    switch (n) {
      case 2: TTT_WAIT_VMCNT(2); break;
      case 4: TTT_WAIT_VMCNT(4); break;
      case 5: TTT_WAIT_VMCNT(5); break;
      case 6: TTT_WAIT_VMCNT(6); break;
      case 7: TTT_WAIT_VMCNT(7); break;
      case 8: TTT_WAIT_VMCNT(8); break;
      case 9: TTT_WAIT_VMCNT(9); break;
      default: TTT_WAIT_VMCNT(0); break;
    }
  };
  for (int st = 0; st < nsteps; ++st) {
   auto step = [&](const KvBuf* __restrict__ Bcp, const KvBuf* __restrict__ Bnp, KvBuf* __restrict__ Bdp)
                   __attribute__((always_inline)) {
    if (st + 3 < nsteps) issue(Bdp);
    if constexpr (MODE == 5) {
      stored_prev = stored_now;
      stored_now = st > 0 ? store_ds() : 0;
    }
    const KvBuf& Bc = *Bcp;
    const int q0 = cs_q0;
    // S/dP products of step st+1 (stale data past the last step is computed and
    // ignored) interleaved with the softmax of step st (S, dP from the previous
    // iteration): the matrix pipe runs while the vector ALUs do the softmax.
    f32x16 s_n, dp_n;
    products(Bnp, s_n, dp_n);
    bf16x8 pb[2];
    f16x8 dsb[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int m0 = half * 16 + hf * 8;  // this lane's rows m = 16*(v/8) + 8*hf + v%8
      const int thr = my_key - dq_ - (q0 + m0);
      const f32x4 l0 = *(const f32x4*)&Bc.lse[m0], l1 = *(const f32x4*)&Bc.lse[m0 + 4];
      const f32x4 d0 = *(const f32x4*)&Bc.dl[m0], d1 = *(const f32x4*)&Bc.dl[m0 + 4];
      int4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
      if constexpr (MODE == 2) a0 = *(const int4*)&Bc.anc[m0], a1 = *(const int4*)&Bc.anc[m0 + 4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = half * 8 + e;
        const float lv = e < 4 ? l0[e] : l1[e - 4];  // log2 units
        const float dv_ = e < 4 ? d0[e] : d1[e - 4];
        float pr = fast_exp2(__builtin_fmaf(s_c[v], sl2, -lv));
        if constexpr (TTT_) {  // row - key = e - thr: visible iff 0 <= e - thr (< win)
          if constexpr (MODE == 4) pr = (unsigned)(e - thr) < (unsigned)win ? pr : 0.f;  // win > 0 here
          else pr = e >= thr ? pr : 0.f;
        } else if constexpr (MODE == 2) {  // key j visible iff j < the row's (clamped) anchor
          const int an = e == 0 ? a0.x : e == 1 ? a0.y : e == 2 ? a0.z : e == 3 ? a0.w
                       : e == 4 ? a1.x : e == 5 ? a1.y : e == 6 ? a1.z : a1.w;
          pr = my_key < an ? pr : 0.f;
        } else {  // the row's own block
          pr = ((q0 + m0 + e) >> P.bs_log2) == (my_key >> P.bs_log2) ? pr : 0.f;
        }
        pb[half][e] = (__bf16)pr;
        dsb[half][e] = (_Float16)(pr * __builtin_fmaf(dv_, -cj, dp_c[v]));  // 2^e dS
      }
    }
    if constexpr (MODE == 5) {
      dsp[0] = dsb[0];
      dsp[1] = dsb[1];
      sp_h = cs_h;
      sp_q0 = q0;
    }
    s_c = s_n;
    dp_c = dp_n;
    // dV += dO^T P, dK~ += Q~^T dS for step st: A operands are columns of the
    // dO and Q~ tiles (lane d = 32*d4 + l32, rows 16*c2 + 8*hf + 0..7).
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      bf16x8 a[4];
      f16x8 a2[4];
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        s16x4 x[2], y[2];
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const int r = c2 * 16 + hf * 8 + part * 4 + ((lane & 15) >> 2);
          const int col = d4 * 32 + (lane & 16) + 4 * (lane & 3);
          const int off = r * D + (((col >> 3) ^ kv_swz(r)) << 3) + (col & 7);
          x[part] = lds_read_tr16(&Bc.g[off]);
          y[part] = lds_read_tr16(&Bc.q[off]);
        }
        a[d4] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7));
        a2[d4] = __builtin_bit_cast(f16x8, __builtin_shufflevector(y[0], y[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        dv[d4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[d4], pb[c2], dv[d4], 0, 0, 0);
        dk[d4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a2[d4], dsb[c2], dk[d4], 0, 0, 0);
      }
    }
   };
    step(&sm[st % NBUF], &sm[(st + 1) % NBUF], &sm[(st + 3) % NBUF]);
    if (++cs_h == P.r) {
      cs_h = 0;
      cs_q0 -= BQ;
    }
    // step st+2 must have landed before the next iteration reads it
    if constexpr (MODE == 5) {
      wait_vm((st + 3 < nsteps ? (w0 ? 5 : 4) : 0) + stored_prev + stored_now);
    } else if (st + 3 < nsteps) {
      if (w0) TTT_WAIT_VMCNT(5);
      else TTT_WAIT_VMCNT(4);
    } else {
      TTT_WAIT_VMCNT(0);
    }
    lds_ring_barrier();
  }
  if constexpr (MODE == 5)
    if (nsteps > 0) store_ds();
  if (!key_ok) return;
  // epilogue: dK = sigma R(j)^T dK~, dV; lane owns key my_key, d = 32*d4 + 8*v4 + 4*hf + e
  const int64_t off = b * P.ks_b + (int64_t)(kst + my_key) * P.ks_t + g * P.ks_h;
  uint16_t* dkrow = (uint16_t*)gr.dk[0] + off;
  uint16_t* dvrow = (uint16_t*)gr.dv[0] + off;
  const float* cp = cosT + rope_off(P, kpos);
  const float* sp = sinT + rope_off(P, kpos);
  const float ksc = P.scale * __builtin_amdgcn_ldexpf(1.0f, -ek);  // sigma, and the dS factor undone
#pragma unroll
  for (int d4 = 0; d4 < 2; ++d4)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int d = d4 * 32 + v4 * 8 + hf * 4;
      float lo[4], hi[4], vlo[4], vhi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = dk[d4][v4 * 4 + e] * ksc, y = dk[d4 + 2][v4 * 4 + e] * ksc;
        const float c = cp[d + e], s_ = sp[d + e];
        lo[e] = x * c + y * s_;
        hi[e] = y * c - x * s_;
        vlo[e] = dv[d4][v4 * 4 + e];
        vhi[e] = dv[d4 + 2][v4 * 4 + e];
      }
      if (P.out_f32) {  // ring-step terms: fp32, the keys' element strides
        float* fk = (float*)gr.dk[0] + off;
        float* fv = (float*)gr.dv[0] + off;
        *(f32x4*)(fk + d) = f32x4{lo[0], lo[1], lo[2], lo[3]};
        *(f32x4*)(fk + d + 64) = f32x4{hi[0], hi[1], hi[2], hi[3]};
        *(f32x4*)(fv + d) = f32x4{vlo[0], vlo[1], vlo[2], vlo[3]};
        *(f32x4*)(fv + d + 64) = f32x4{vhi[0], vhi[1], vhi[2], vhi[3]};
      } else {
        *(u32x2*)(dkrow + d) = u32x2{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3])};
        *(u32x2*)(dkrow + d + 64) = u32x2{pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])};
        *(u32x2*)(dvrow + d) = u32x2{pack_bf2(vlo[0], vlo[1]), pack_bf2(vlo[2], vlo[3])};
        *(u32x2*)(dvrow + d + 64) = u32x2{pack_bf2(vhi[0], vhi[1]), pack_bf2(vhi[2], vhi[3])};
      }
    }
}

// ============================================================================= branch dK/dV
// Grid (ceil(stok/16), Hkv, B), 256 threads: 16 rows per block, 16 lanes per
// row, each lane 4 rotate-half pairs (d and d + 64).
__global__ void __launch_bounds__(256)
    branch_bwd_bf16_kernel(Prob P, const uint16_t* __restrict__ q, PassPtrs kv, const float* __restrict__ lse,
                           const uint16_t* __restrict__ dout, const float* __restrict__ delta,
                           const float* __restrict__ cosT, const float* __restrict__ sinT, PassGradPtrs gr) {
  const int tid = threadIdx.x, c16 = tid & 15;
  const int tok = blockIdx.x * 16 + (tid >> 4);
  const int g = blockIdx.y, b = blockIdx.z;
  int s, start, L;
  if (tok >= P.stok || !token_seq(P, tok, s, start, L)) return;
  const int i = tok - start, slot = seq_slot0(P, s) + i;
  const int dlo = c16 * 4, dhi = 64 + c16 * 4;
  const int qo = (P.layout == 1 && P.kv_cu) ? P.seg_qoff[s] : P.q_off;  // the row's position offset
  const int pq = qo + i + P.p - 1;
  const f32x4 cqa = *(const f32x4*)(cosT + rope_off(P, pq) + dlo);
  const f32x4 sqa = *(const f32x4*)(sinT + rope_off(P, pq) + dlo);
  const int64_t koff = b * P.ks_b + (int64_t)tok * P.ks_t + g * P.ks_h;
  for (int qq = 2; qq <= P.p; ++qq) {
    const uint16_t* krow = (const uint16_t*)kv.k[qq - 1] + koff;
    const uint16_t* vrow = (const uint16_t*)kv.v[qq - 1] + koff;
    const u32x2 ka = *(const u32x2*)(krow + dlo), kb2 = *(const u32x2*)(krow + dhi);
    const u32x2 va = *(const u32x2*)(vrow + dlo), vb2 = *(const u32x2*)(vrow + dhi);
    const int pk = qo + i + qq - 1;
    const f32x4 ck = *(const f32x4*)(cosT + rope_off(P, pk) + dlo);
    const f32x4 sk = *(const f32x4*)(sinT + rope_off(P, pk) + dlo);
    float kr[8], vv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t wa = ka[e >> 1], wb = kb2[e >> 1];
      const float x1 = __uint_as_float((e & 1) ? (wa & 0xffff0000u) : (wa << 16));
      const float x2 = __uint_as_float((e & 1) ? (wb & 0xffff0000u) : (wb << 16));
      kr[e] = x1 * ck[e] - x2 * sk[e];
      kr[4 + e] = x2 * ck[e] + x1 * sk[e];
      const uint32_t ua = va[e >> 1], ub = vb2[e >> 1];
      vv[e] = __uint_as_float((e & 1) ? (ua & 0xffff0000u) : (ua << 16));
      vv[4 + e] = __uint_as_float((e & 1) ? (ub & 0xffff0000u) : (ub << 16));
    }
    float dk[8] = {}, dv[8] = {};
    for (int hh = 0; hh < P.r; ++hh) {
      const int h = g * P.r + hh;
      const uint16_t* qrow = q + b * P.qs_b + (int64_t)tok * P.qs_t + h * P.qs_h;
      const uint16_t* grow = dout + b * P.os_b + (int64_t)tok * P.os_t + h * P.os_h;
      const u32x2 qa = *(const u32x2*)(qrow + dlo), qb2 = *(const u32x2*)(qrow + dhi);
      const u32x2 ga = *(const u32x2*)(grow + dlo), gb2 = *(const u32x2*)(grow + dhi);
      float qr[8], go[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wa = qa[e >> 1], wb = qb2[e >> 1];
        const float x1 = __uint_as_float((e & 1) ? (wa & 0xffff0000u) : (wa << 16));
        const float x2 = __uint_as_float((e & 1) ? (wb & 0xffff0000u) : (wb << 16));
        qr[e] = x1 * cqa[e] - x2 * sqa[e];
        qr[4 + e] = x2 * cqa[e] + x1 * sqa[e];
        const uint32_t ua = ga[e >> 1], ub = gb2[e >> 1];
        go[e] = __uint_as_float((e & 1) ? (ua & 0xffff0000u) : (ua << 16));
        go[4 + e] = __uint_as_float((e & 1) ? (ub & 0xffff0000u) : (ub << 16));
      }
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ps += qr[e] * kr[e], pd += go[e] * vv[e];
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        ps += __shfl_xor(ps, m, 64);
        pd += __shfl_xor(pd, m, 64);
      }
      const float pr = __expf(ps * P.scale - lse[b * P.lse_b + h * P.lse_h + tok]);
      const float dsv = pr * (pd - delta[(int64_t)(b * P.Hq + h) * P.spad + slot]) * P.scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) dk[e] += dsv * qr[e], dv[e] += pr * go[e];
    }
    float lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = dk[e] * ck[e] + dk[4 + e] * sk[e];
      hi[e] = dk[4 + e] * ck[e] - dk[e] * sk[e];
    }
    if (P.out_f32) {  // ring-step terms: fp32
      float* fk = (float*)gr.dk[qq - 1] + koff;
      float* fv = (float*)gr.dv[qq - 1] + koff;
      *(f32x4*)(fk + dlo) = f32x4{lo[0], lo[1], lo[2], lo[3]};
      *(f32x4*)(fk + dhi) = f32x4{hi[0], hi[1], hi[2], hi[3]};
      *(f32x4*)(fv + dlo) = f32x4{dv[0], dv[1], dv[2], dv[3]};
      *(f32x4*)(fv + dhi) = f32x4{dv[4], dv[5], dv[6], dv[7]};
    } else {
      uint16_t* dkrow = (uint16_t*)gr.dk[qq - 1] + koff;
      uint16_t* dvrow = (uint16_t*)gr.dv[qq - 1] + koff;
      *(u32x2*)(dkrow + dlo) = u32x2{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3])};
      *(u32x2*)(dkrow + dhi) = u32x2{pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])};
      *(u32x2*)(dvrow + dlo) = u32x2{pack_bf2(dv[0], dv[1]), pack_bf2(dv[2], dv[3])};
      *(u32x2*)(dvrow + dhi) = u32x2{pack_bf2(dv[4], dv[5]), pack_bf2(dv[6], dv[7])};
    }
  }
}

}  // namespace bwd

void launch_dkdv_bf16(const Prob& P, const PassPtrs& kv, const float* lse, const uint16_t* dout, const _Float16* kt,
                      const _Float16* qt, const float* delta, const int4* tiles_kv, const float* cosT,
                      const float* sinT, const PassGradPtrs& g, hipStream_t st) {
  const int64_t grid = P.layout == 0
                           ? (int64_t)8 * ((P.B * P.Hkv + 7) / 8) * ((P.kv_len + bwd::BKV - 1) / bwd::BKV)
                           : (int64_t)P.Hkv * (((P.kv_cu ? P.kv_tok : P.stok) + bwd::BKV - 1) / bwd::BKV + P.nseq);
  if (grid == 0) return;
  if (P.win > 0)  // sliding window: its own instantiation (MODE 4)
    bwd::dkdv_bf16_kernel<4><<<(unsigned)grid, 256, 0, st>>>(P, kv, lse, dout, kt, qt, delta, tiles_kv, cosT, sinT, g);
  else if (P.ds)  // also storing dS for the dQ kernel (MODE 5)
    bwd::dkdv_bf16_kernel<5><<<(unsigned)grid, 256, 0, st>>>(P, kv, lse, dout, kt, qt, delta, tiles_kv, cosT, sinT, g);
  else
    bwd::dkdv_bf16_kernel<0><<<(unsigned)grid, 256, 0, st>>>(P, kv, lse, dout, kt, qt, delta, tiles_kv, cosT, sinT, g);
}

void launch_block_dkdv_bf16(const Prob& P, bool ctx_keys, const uint16_t* v, const float* lse, const uint16_t* dout,
                            const _Float16* kt, const _Float16* qt, const float* delta, const int4* tiles,
                            const float* cosT, const float* sinT, void* dk, void* dv, hipStream_t st) {
  PassPtrs kv = {};
  kv.v[0] = v;
  PassGradPtrs g = {};
  g.dk[0] = dk;
  g.dv[0] = dv;
  const int nkeys = ctx_keys ? P.kv_len : P.stok;
  const int64_t grid = P.layout == 0 ? (int64_t)8 * ((P.B * P.Hkv + 7) / 8) * ((nkeys + bwd::BKV - 1) / bwd::BKV)
                                     : (int64_t)P.Hkv * ((nkeys + bwd::BKV - 1) / bwd::BKV + P.nseq);
  if (grid == 0) return;
  if (ctx_keys)
    bwd::dkdv_bf16_kernel<2><<<(unsigned)grid, 256, 0, st>>>(P, kv, lse, dout, kt, qt, delta, tiles, cosT, sinT, g);
  else
    bwd::dkdv_bf16_kernel<3><<<(unsigned)grid, 256, 0, st>>>(P, kv, lse, dout, kt, qt, delta, tiles, cosT, sinT, g);
}

template <int RH, int MODE>
static void launch_dq_rh(const Prob& P, const uint16_t* q, const PassPtrs& kv, const float* lse, const uint16_t* dout,
                         const _Float16* kt, const _Float16* ktt, const _Float16* qt, const float* delta,
                         const int4* tiles_q, const float* cosT, const float* sinT, uint16_t* dq,
                         const _Float16* kbt, const _Float16* kbtt, const PassGradPtrs& g, hipStream_t st) {
  constexpr int RT = bwd::dq_rows(RH);
  const int nsub = P.r / RH;
  int64_t grid;
  if (P.layout == 0) {
    const int64_t units = (int64_t)P.B * P.Hkv * nsub;
    grid = 8 * ((units + 7) / 8) * ((P.stok + RT - 1) / RT);
  } else {
    grid = (int64_t)((P.stok + RT - 1) / RT + P.nseq) * P.Hkv * nsub;
  }
  bwd::dq_bf16_kernel<RH, MODE><<<(unsigned)grid, 256, 0, st>>>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q,
                                                                cosT, sinT, dq, kbt, kbtt, g);
}

int dq_tile_rows(int r) { return bwd::dq_rows(bwd::dq_heads_per_wg(r)); }

bool dq_fuses_branch(int r) { return bwd::dq_heads_per_wg(r) == r; }

void launch_dq_bf16(const Prob& P, const uint16_t* q, const PassPtrs& kv, const float* lse, const uint16_t* dout,
                    const _Float16* kt, const _Float16* ktt, const _Float16* qt, const float* delta,
                    const int4* tiles_q, const float* cosT, const float* sinT, uint16_t* dq, const PassGradPtrs& g,
                    hipStream_t st) {
  const bool w = P.win > 0;  // sliding window: its own instantiation (MODE 4)
  if (P.ds) {  // from the dK/dV kernel's stored dS (MODE 5)
    switch (bwd::dq_heads_per_wg(P.r)) {
      case 4: launch_dq_rh<4, 5>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st); break;
      case 2: launch_dq_rh<2, 5>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st); break;
      default: launch_dq_rh<1, 5>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st); break;
    }
    return;
  }
  switch (bwd::dq_heads_per_wg(P.r)) {
    case 4:
      if (w) launch_dq_rh<4, 4>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st);
      else launch_dq_rh<4, 0>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st);
      break;
    case 2:
      if (w) launch_dq_rh<2, 4>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st);
      else launch_dq_rh<2, 0>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st);
      break;
    default:
      if (w) launch_dq_rh<1, 4>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st);
      else launch_dq_rh<1, 0>(P, q, kv, lse, dout, kt, ktt, qt, delta, tiles_q, cosT, sinT, dq, nullptr, nullptr, g, st);
      break;
  }
}

void launch_block_dq_bf16(const Prob& P, const uint16_t* v_ctx, const uint16_t* v_blk, const float* lse,
                          const uint16_t* dout, const _Float16* ckt, const _Float16* cktt, const _Float16* bkt,
                          const _Float16* bktt, const _Float16* qt, const float* delta, const int4* tiles,
                          const float* cosT, const float* sinT, uint16_t* dq, hipStream_t st) {
  PassPtrs kv = {};
  kv.v[0] = v_ctx;
  kv.v[1] = v_blk;
  const PassGradPtrs none = {};
  switch (bwd::dq_heads_per_wg(P.r)) {
    case 4: launch_dq_rh<4, 1>(P, nullptr, kv, lse, dout, ckt, cktt, qt, delta, tiles, cosT, sinT, dq, bkt, bktt, none, st); break;
    case 2: launch_dq_rh<2, 1>(P, nullptr, kv, lse, dout, ckt, cktt, qt, delta, tiles, cosT, sinT, dq, bkt, bktt, none, st); break;
    default: launch_dq_rh<1, 1>(P, nullptr, kv, lse, dout, ckt, cktt, qt, delta, tiles, cosT, sinT, dq, bkt, bktt, none, st); break;
  }
}

void launch_branch_bwd_bf16(const Prob& P, const uint16_t* q, const PassPtrs& kv, const float* lse,
                            const uint16_t* dout, const float* delta, const float* cosT, const float* sinT,
                            const PassGradPtrs& g, hipStream_t st) {
  dim3 gb((P.stok + 15) / 16, P.Hkv, P.B);
  bwd::branch_bwd_bf16_kernel<<<gb, 256, 0, st>>>(P, q, kv, lse, dout, delta, cosT, sinT, g);
}

}  // namespace ttt
