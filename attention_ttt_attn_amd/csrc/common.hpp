// Shared device/host definitions of libtttattn (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Kernel-side view of one call.  Every "sequence" s is a batch row (BSHD) or a
// packed sequence (THD); its tokens are tok = start + i, i = 0..L-1, inside
// batch b.  Workspace tensors hold one row per "slot": BSHD slot = token;
// THD sequence s owns slots [slot_base[s], slot_base[s+1]), a multiple of 64
// long, so every 64-row workspace tile lies inside one sequence, starts
// 16-byte aligned and is zero past the sequence end.
struct Prob {
  int layout;          // 0 BSHD, 1 THD
  int B;               // batches (1 for THD)
  int stok;            // tokens per batch: S (BSHD) or T (THD)
  int spad;            // workspace slots per (batch, head): multiple of 64, >= 64 past the last used slot
  int nseq;            // sequences: B (BSHD) or num_seqs (THD)
  const int* cu;       // THD cu_seqlens (device)
  const int* slot_base;  // THD: [nseq + 1] first slot of every sequence (device workspace)
  int Hq, Hkv, D, p, r;
  int npos;            // rows of the RoPE table: positions 0 .. npos-1
  float scale;         // softmax scale sigma
  float scale_log2;    // sigma * log2(e)
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t os_b, os_t, os_h;
  int64_t lse_b, lse_h;  // LSE element (b, h, tok) = b*lse_b + h*lse_h + tok
  // Ring steps (BSHD forward): query row i sits at position q_off + i, pass-1
  // key j at kv_off + j for j < kv_len; branch = 0 leaves passes 2..p out.
  // Whole-sequence calls: q_off = kv_off = 0, kv_len = stok, branch = 1.
  int q_off, kv_off, kv_len, branch;
  // Block drafting (BSHD forward): row i is slot i % bs of block i / bs, whose
  // anchor a = anchors[b * nblk + i / bs] (clamped to [0, kv_len]) puts the
  // slot at position a + i % bs; it sees context keys j < a (kv_len context
  // rows) and the bs keys of its block (staged with spad_b slots per head;
  // the forward kernel requires spad_b == spad).
  const int* anchors;
  int bs_log2, nblk, spad_b;
  int64_t cs_b, cs_t, cs_h;  // block-draft backward: context K/V strides (P.ks_*: the block K/V)
  // Sliding-window trunk (TTT passes): win > 0 limits row i's trunk to the
  // pass-1 keys at positions (pos_i - win, pos_i]; 0 = the full causal trunk.
  int win;
  // backward outputs in fp32 (ring-step terms the caller sums) instead of the inputs' bf16
  int out_f32;
  // the dQ kernel also produces the branch dK/dV of passes 2..p (its work
  // item holds every query head of a KV group); no separate branch kernel
  int dq_branch;
  // bf16 backward: bounds that set the power-of-two scale of the fp16 dS
  // operands (see ds_exp).  All in the workspace, slot-indexed.
  float* dnorm;  // [B*Hq][spad]: ||dO_i||_1 of the row in that slot (0 past a sequence's end)
  float* dpart;  // [B*Hq][spad/64][2]: per 64-slot block, max ||dO_i||_1 and max |Delta_i|
  float* dmax;   // [B*Hkv][2]: the same over every row of the KV group's heads
  float* vmax;   // [B*Hkv][spad/32]: per 32 trunk (block drafting: context) keys, max |v_jd|
  float* vmax_b; // block drafting: the same for the block keys
  // THD ring steps (kv_cu set): query segment s (rows cu[s] .. cu[s+1]) sits at
  // positions seg_qoff[s] + i and attends to pass-1 key segment s (packed rows
  // kv_cu[s] .. kv_cu[s+1] of k[0] / v[0], kv_tok of them) at positions
  // seg_kvoff[s] + j.  Both segments of s share the workspace slots
  // slot_base[s] .. slot_base[s+1] (the longer of the two, rounded up to 64).
  const int* seg_qoff;
  const int* seg_kvoff;
  const int* kv_cu;
  int kv_tok;
  // Stored dS (asked for; bf16 whole-sequence BSHD passes without a window): the dK/dV
  // kernel writes every causal 32x32 block of 2^e dS in fp16 -- one exponent
  // e per KV group, from dmax and vgmax -- and the dQ kernel forms dQ~ = dS K~
  // from them instead of recomputing S and dP.  Block (rb, kg) of query head
  // (b, h) holds rows 32 rb .. +31 and keys 32 kg .. +31 (kg <= rb) at
  // ds + ((b Hq + h) ds_tri + rb (rb + 1) / 2 + kg) * 1024; inside it, dS of
  // row 16 u + 8 w + e and key k sits at element 512 u + 8 (32 w + k) + e
  // (the dK/dV kernel's register layout: one 16-byte piece per lane).
  _Float16* ds;
  int64_t ds_tri;  // blocks per (batch, head): n (n + 1) / 2, n = ceil(S / 32)
  float* vpart;    // [B*Hkv][spad/64]: per 64-slot block, max |v_jd| of the trunk keys
  float* vgmax;    // [B*Hkv]: the same over the whole group
};

// Ring geometry of one sequence (or THD segment): its query rows' position
// offset qoff, the query-minus-key position offset dq (query row i sees key
// j iff j <= i + dq), and its pass-1 key rows kvs .. kvs + kvn (token indices
// of k[0] / v[0]).  start / L: the query rows.
__device__ __forceinline__ void seq_ring(const Prob& P, int s, int start, int L, int& qoff, int& dq, int& kvs,
                                         int& kvn) {
  if (P.layout == 0) {
    qoff = P.q_off, dq = P.q_off - P.kv_off, kvs = 0, kvn = P.kv_len;
  } else if (!P.kv_cu) {
    qoff = 0, dq = 0, kvs = start, kvn = L;
  } else {
    qoff = P.seg_qoff[s];
    dq = qoff - P.seg_kvoff[s];
    int a = P.kv_cu[s], e = P.kv_cu[s + 1];
    a = a < 0 ? 0 : (a > P.kv_tok ? P.kv_tok : a);
    e = e < a ? a : (e > P.kv_tok ? P.kv_tok : e);
    kvs = a;
    kvn = e - a;
    const int room = P.slot_base[s + 1] - P.slot_base[s];
    if (kvn > room) kvn = room;
  }
}

// Element offset of position pos's row in the D = 128 RoPE table (64 angles
// per row), clamped into the table's npos rows: THD ring steps take their
// position offsets from device arrays the host does not read, so an offset
// past the declared maximum gives wrong angles, never a read outside the table.
__device__ __forceinline__ int64_t rope_off(const Prob& P, int pos) {
  return (int64_t)(pos < 0 ? 0 : (pos >= P.npos ? P.npos - 1 : pos)) * 64;
}

// Last s with cu[s] <= tok: the sequence whose (non-empty) rows start at tok.
__device__ __forceinline__ int seq_at(const int* cu, int nseq, int tok) {
  int lo = 0, hi = nseq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= tok) lo = mid; else hi = mid;
  }
  return lo;
}

// Exponent e of the power-of-two factor 2^e applied to fp16 dS operands whose
// magnitude is bounded by x: |dS 2^e| <= x 2^e < 2^15 < 65504 (fp16 max), and
// >= 2^14 at the bound, so neither small nor large dO leaves fp16's range.
// Clamped to [-64, 64] (operands stay finite in fp32 and bf16).  Pure
// exponent arithmetic: scaling dO by 2^k shifts e by exactly -k.
__device__ __forceinline__ int ds_exp(float x) {
  const int e = 15 - __builtin_amdgcn_frexp_expf(x);
  return e < -64 ? -64 : (e > 64 ? 64 : e);
}


// Passes' key/value pointers (up to 16), passed by value to kernels.
struct PassPtrs {
  const void* k[16];
  const void* v[16];
};
struct PassGradPtrs {
  void* dk[16];
  void* dv[16];
};

// Sequence s of the call: batch, first token and length.  THD bounds are
// clamped into [0, stok) and to the sequence's slot range.
__device__ __forceinline__ void seq_info(const Prob& P, int s, int& b, int& start, int& L) {
  if (P.layout == 0) {
    b = s;
    start = 0;
    L = P.stok;
  } else {
    b = 0;
    int a = P.cu[s], e = P.cu[s + 1];
    a = a < 0 ? 0 : (a > P.stok ? P.stok : a);
    e = e < a ? a : (e > P.stok ? P.stok : e);
    start = a;
    L = e - a;
    int room = P.slot_base[s + 1] - P.slot_base[s];
    if (L > room) L = room;
  }
}

// THD: whether the 64 slots from slot0 (64-aligned) lie past every read of
// the rows cu[s] .. cu[s+1] (ntok rows in all) of the sequence s owning them.
// A sequence's readers touch at most 127 slots past its last row (128-key
// dK/dV tiles, 128-row dQ work items; those lanes are masked), so staging
// may skip such a tile: with block rows and a longer context sharing one
// sequence's slots (or the other way round), most of the range is never read.
__device__ __forceinline__ bool thd_tile_unread(const Prob& P, const int* cu, int ntok, int slot0) {
  int lo = 0, hi = P.nseq;  // last s with slot_base[s] <= slot0 (the last sequence for the tail)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P.slot_base[mid] <= slot0) lo = mid; else hi = mid;
  }
  int a = cu[lo], e = cu[lo + 1];
  a = a < 0 ? 0 : (a > ntok ? ntok : a);
  e = e < a ? a : (e > ntok ? ntok : e);
  return slot0 - P.slot_base[lo] >= e - a + 128;
}

// Block drafting, the geometry of one sequence: its blocks' anchors start at
// anchors[ab], and its context is rows cs .. cs + cn of k_ctx / v_ctx
// (staged at the sequence's own slots in THD).  BSHD: batch row b, the whole
// context.  THD (kv_cu = the contexts' cu_seqlens): sequence s, whose rows
// are whole blocks, so its first block is its first row / bs.
struct BlkSeq {
  int64_t ab;
  int cs, cn;
};
__device__ __forceinline__ BlkSeq blk_seq_of(const Prob& P, int s) {  // THD
  int b_, start, L;
  seq_info(P, s, b_, start, L);
  int a = P.kv_cu[s], e = P.kv_cu[s + 1];
  a = a < 0 ? 0 : (a > P.kv_tok ? P.kv_tok : a);
  e = e < a ? a : (e > P.kv_tok ? P.kv_tok : e);
  const int room = P.slot_base[s + 1] - P.slot_base[s];
  return BlkSeq{(int64_t)(start >> P.bs_log2), a, e - a < room ? e - a : room};
}
// b: the batch row (BSHD); start: the first row of a THD work item.
__device__ __forceinline__ BlkSeq blk_seq(const Prob& P, int b, int start) {
  if (P.layout == 0) return BlkSeq{(int64_t)b * P.nblk, 0, P.kv_len};
  return blk_seq_of(P, seq_at(P.cu, P.nseq, start));
}
// Anchor of the block holding row `row` (sequence-relative), clamped to [0, cn].
__device__ __forceinline__ int blk_anchor(const Prob& P, const BlkSeq& q, int row) {
  const int a = P.anchors[q.ab + (row >> P.bs_log2)];
  return a < 0 ? 0 : (a > q.cn ? q.cn : a);
}

__device__ __forceinline__ int seq_slot0(const Prob& P, int s) { return P.layout == 0 ? 0 : P.slot_base[s]; }

// Sequence holding token `tok` (THD: binary search over cu_seqlens).
__device__ __forceinline__ bool token_seq(const Prob& P, int tok, int& s, int& start, int& L) {
  if (P.layout == 0) {
    s = 0;
    start = 0;
    L = P.stok;
    return tok < P.stok;
  }
  int lo = 0, hi = P.nseq;  // last s with cu[s] <= tok
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (P.cu[mid] <= tok) lo = mid; else hi = mid;
  }
  s = lo;
  int b_;
  seq_info(P, s, b_, start, L);
  return tok >= start && tok < start + L;
}

// Sequence owning workspace slot `slot`; tok is its token when the slot holds
// one, seq the sequence (THD).
__device__ __forceinline__ bool slot_token(const Prob& P, int slot, int& tok, int& row, int* seq = nullptr) {
  if (P.layout == 0) {
    tok = row = slot;
    if (seq) *seq = 0;
    return slot < P.stok;
  }
  int lo = 0, hi = P.nseq;  // last s with slot_base[s] <= slot
  if (slot >= P.slot_base[P.nseq]) return false;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (P.slot_base[mid] <= slot) lo = mid; else hi = mid;
  }
  int b_, start, L;
  seq_info(P, lo, b_, start, L);
  row = slot - P.slot_base[lo];
  tok = start + row;
  if (seq) *seq = lo;
  return row < L;
}

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ void unpack_bf8(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack_bf8(const float* f) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf2(f[2 * i], f[2 * i + 1]);
  return w;
}

__device__ __forceinline__ u32x4 pack_h8(const float* f) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_h2(f[2 * i], f[2 * i + 1]);
  return w;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// HBM -> LDS without VGPR staging, through a buffer descriptor
// (buffer_load_dword* ... lds): base and byte range in SGPRs, a 32-bit byte
// offset per lane; lane l's 16 (or 4) bytes land at l * 16 (or l * 4) bytes
// past the wave-uniform LDS address, and a lane whose bytes reach past the
// range reads zeros.  The flat form (global_load_lds) is not used: the
// compiler's wait insertion treats it as an access that may count on the LDS
// counter and then forces lgkmcnt(0) at every later LDS-read dependency while
// one is in flight; these count on vmcnt alone, so LDS operand reads keep
// graded waits and stay pipelined under the prefetches.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(buf_rsrc r, uint32_t off, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)l, 16, off, 0, 0, 0);
}
// The same for data read once (streamed): the non-temporal hint keeps it from
// displacing reused lines in the caches.
__device__ __forceinline__ void lds_dma16_nt(buf_rsrc r, uint32_t off, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)l, 16, off, 0, 0, 2);
}
__device__ __forceinline__ void lds_dma4(buf_rsrc r, uint32_t off, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)l, 4, off, 0, 0, 0);
}
// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left open (gfx9 encoding).
#define TTT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// Workgroup barrier for LDS rings filled by direct-to-LDS loads.  The release
// fence of __syncthreads() waits for every outstanding load of the wave (a
// direct-to-LDS load counts as an LDS write), which would also drain the
// prefetches issued for later steps; here the caller waits (TTT_WAIT_VMCNT) for
// exactly the buffers the next step reads.  The wave's LDS reads complete
// before it, and the memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void lds_ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within every 16-lane group,
// lane 4e + a supplies the address of 4 consecutive 16-bit elements; lane
// 4a + b receives element b of the chunks of lanes a, a+4, a+8, a+12.  So if
// lane s points at row r0 + s/4, column c0 + 4*(s%4) of a row-major tile,
// lane s receives column c0 + s, rows r0..r0+3: a column read.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// Max and sum over the two 32-lane halves of a wave (v_permlane32_swap: the
// two results hold the low and the high half's value in every lane).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workspace layout shared by host launchers.
struct WsPlan {
  size_t table, slots, tiles_q, tiles_kv, kt, vt, ktt, qt, delta, bnd, ds, total;
};

}  // namespace ttt
