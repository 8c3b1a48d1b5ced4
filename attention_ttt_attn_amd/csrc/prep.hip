// Prologue kernels: RoPE table, rotate/transposed staging copies, Delta, and
// the varlen tile scheduler.  All are HBM-bound single passes.
#include "kernels.hpp"

namespace ttt {

// cos/sin of pos * theta_k, theta_k = base^(-2k/D), evaluated in fp64 and stored
// as fp32 [npos][D/2].  base == 0 fills the identity rotation (cos 1, sin 0).
// Rotate-half RoPE: NeoX pairing of k and k + D/2 (NeMo-RL PR #3725,
// self-review comment: rotate-half oracle).
// theta_k is evaluated once per workgroup (half <= 64: D <= 128, checked by
// the caller), then one fp64 sincos per entry.
__global__ void __launch_bounds__(256) rope_table_kernel(float* __restrict__ cosT, float* __restrict__ sinT,
                                                         int npos, int half, double base) {
  __shared__ double th[64];
  if ((int)threadIdx.x < half) th[threadIdx.x] = pow(base, -2.0 * (double)threadIdx.x / (double)(2 * half));
  __syncthreads();
  int64_t n = (int64_t)npos * half;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    int pos = (int)(e / half), k = (int)(e % half);
    if (base == 0.0) {
      cosT[e] = 1.f;
      sinT[e] = 0.f;
    } else {
      double sn, cs;
      sincos((double)pos * th[k], &sn, &cs);
      cosT[e] = (float)cs;
      sinT[e] = (float)sn;
    }
  }
}

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ void st(T* p, float x);
template <> __device__ __forceinline__ void st<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void st<_Float16>(_Float16* p, float x) { *p = (_Float16)x; }
template <> __device__ __forceinline__ void st<uint16_t>(uint16_t* p, float x) { *p = f2bf(x); }

// Staging copy of one tensor X [b][tok][h][D] (element strides sb, st_, sh):
//   out_row [(b*H + h)][spad][D]  rotated at position (row + pos_off) when ROT
//   out_col [(b*H + h)][D][spad]  the same values transposed
// indexed by workspace slot; slots that hold no token are written as 0.
// Grid (spad/64, H, B), 256 threads; tile = 64 slots of one (b, h).
template <int D, typename InT, bool ROT, typename RowT, typename ColT>
__global__ void __launch_bounds__(256) prep_rows_kernel(Prob P, const InT* __restrict__ x, int64_t sb, int64_t st_,
                                                        int64_t sh, int H, int pos_off,
                                                        const float* __restrict__ cosT,
                                                        const float* __restrict__ sinT, RowT* __restrict__ out_row,
                                                        ColT* __restrict__ out_col) {
  constexpr int HALF = D / 2;
  constexpr int TPR = HALF / 4;              // threads per token row, each 4 pairs (k, k + D/2)
  constexpr int ROWS = 256 / TPR;            // token rows per pass
  __shared__ float tile[64][D + 1];
  const int h = blockIdx.y, b = blockIdx.z;
  const int tok0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const int c = tid % TPR, rr = tid / TPR;
  const int64_t slab = (int64_t)(b * H + h) * P.spad;
  for (int r0 = 0; r0 < 64; r0 += ROWS) {
    int lr = r0 + rr, slot = tok0 + lr;
    float a[4], bb[4];
    int tok, row;
    bool valid = slot_token(P, slot, tok, row);
    if (valid) {
      const InT* src = x + (int64_t)b * sb + (int64_t)tok * st_ + (int64_t)h * sh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = ld<InT>(src + 4 * c + e);
        bb[e] = ld<InT>(src + HALF + 4 * c + e);
      }
      if (ROT) {
        int pos = row + pos_off;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float cs = cosT[(int64_t)pos * HALF + 4 * c + e], sn = sinT[(int64_t)pos * HALF + 4 * c + e];
          float y1 = a[e] * cs - bb[e] * sn, y2 = bb[e] * cs + a[e] * sn;
          a[e] = y1;
          bb[e] = y2;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = bb[e] = 0.f;
    }
    if (out_row) {
      RowT* dst = out_row + (slab + slot) * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st<RowT>(dst + 4 * c + e, a[e]);
        st<RowT>(dst + HALF + 4 * c + e, bb[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[lr][4 * c + e] = a[e];
      tile[lr][HALF + 4 * c + e] = bb[e];
    }
  }
  if (!out_col) return;
  __syncthreads();
  // transposed write: each thread owns (d, 8 consecutive tokens)
  for (int w = tid; w < D * 8; w += 256) {
    int d = w / 8, t8 = (w % 8) * 8;
    ColT* dst = out_col + ((int64_t)(b * H + h) * D + d) * P.spad + tok0 + t8;
#pragma unroll
    for (int e = 0; e < 8; ++e) st<ColT>(dst + e, tile[t8 + e][d]);
  }
}

// bf16 staging of up to two tensors in one launch (D = 128), 16-byte accesses:
// job j stages X_j [b][tok][h][128] (bf16) into
//   out_row [(b*H + h)][spad][128]  fp16, rotated at position (row + pos_off) when rot
//   out_col [(b*H + h)][128][spad]  the same values transposed, fp16 or bf16
// by workspace slot (slots without a token are written as 0).  Grid
// ((spad/64) * (H_0 + H_1), 1, B): head index hy = H_0 + H_1 entries, hy < H_0
// selects job 0.  J.heads_fast puts the heads of one 64-slot tile in
// consecutive workgroups, so that workgroups running together read whole token
// rows (better for row-major outputs); otherwise the tiles of one head are
// consecutive, which keeps neighbouring transposed writes adjacent.  Each
// thread owns 8 rotation pairs (k, k + 64) of a row; 32 rows per pass, two passes.
__global__ void __launch_bounds__(256) prep_bf16_kernel(Prob P, PrepJobs J, const float* __restrict__ cosT,
                                                        const float* __restrict__ sinT) {
  constexpr int D = 128, HALF = 64;
  __shared__ uint32_t tile[64][D / 2 + 1];  // 16-bit pairs; 65-dword rows: conflict-free column reads
  const unsigned Ht = (unsigned)(J.j[0].H + (J.n > 1 ? J.j[1].H : 0)), ntile = (unsigned)P.spad / 64;
  const int hy = (int)(J.heads_fast ? blockIdx.x % Ht : blockIdx.x / ntile);
  const int tix = (int)(J.heads_fast ? blockIdx.x / Ht : blockIdx.x % ntile);
  const bool second = hy >= J.j[0].H;
  const PrepJob jb = second ? J.j[1] : J.j[0];
  const int h = second ? hy - J.j[0].H : hy;
  const int b = blockIdx.z, tok0 = tix * 64, tid = threadIdx.x;
  const int c8 = tid & 7, rr = tid >> 3;
  const int64_t slab = (int64_t)(b * jb.H + h) * P.spad;
  if (P.layout == 1 && thd_tile_unread(P, jb.cu ? jb.cu : P.cu, jb.cu ? jb.ntok : P.stok, tok0)) return;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int lr = pass * 32 + rr, slot = tok0 + lr;
    float a[8], c[8];
    int tok, row, sq = 0;
    bool valid;
    if (jb.rows != 0 && P.layout == 0) {  // jb.rows < 0: an empty tensor
      tok = row = slot;
      valid = slot < jb.rows;
    } else if (jb.cu) {  // a THD tensor with its own sequence lengths on the shared slots
      Prob Pj = P;
      Pj.cu = jb.cu;
      Pj.stok = jb.ntok;
      valid = slot_token(Pj, slot, tok, row, &sq);
    } else {
      valid = slot_token(P, slot, tok, row, &sq);
    }
    BlkSeq bq{};  // block drafting: the row's sequence (anchors, context)
    if ((jb.out_lim || jb.pos_anchor) && valid) bq = P.layout == 0 ? blk_seq(P, b, 0) : blk_seq_of(P, sq);
    if (jb.out_lim && h == 0 && c8 == 0) jb.out_lim[(int64_t)b * P.spad + slot] = valid ? blk_anchor(P, bq, row) : 0;
    if (valid) {
      const uint16_t* src = jb.x + (int64_t)b * jb.sb + (int64_t)tok * jb.st + (int64_t)h * jb.sh + 8 * c8;
      unpack_bf8(*(const u32x4*)src, a);
      unpack_bf8(*(const u32x4*)(src + HALF), c);
      if (jb.rot) {
        const int pos = jb.pos_anchor ? blk_anchor(P, bq, row) + (row & ((1 << P.bs_log2) - 1))
                                      : row + jb.pos_off + (jb.seg_pos ? jb.seg_pos[sq] : 0);
        const int64_t t = rope_off(P, pos) + 8 * c8;
        const f32x4 c0 = *(const f32x4*)(cosT + t), c1 = *(const f32x4*)(cosT + t + 4);
        const f32x4 s0 = *(const f32x4*)(sinT + t), s1 = *(const f32x4*)(sinT + t + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cs = e < 4 ? c0[e] : c1[e - 4], sn = e < 4 ? s0[e] : s1[e - 4];
          const float y1 = a[e] * cs - c[e] * sn, y2 = c[e] * cs + a[e] * sn;
          a[e] = y1;
          c[e] = y2;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = c[e] = 0.f;
    }
    if (jb.out_row) {
      _Float16* dst = jb.out_row + (slab + slot) * D + 8 * c8;
      *(u32x4*)dst = pack_h8(a);
      *(u32x4*)(dst + HALF) = pack_h8(c);
    }
    if (jb.out_col) {
      const u32x4 wa = jb.col_bf16 ? pack_bf8(a) : pack_h8(a);
      const u32x4 wc = jb.col_bf16 ? pack_bf8(c) : pack_h8(c);
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[lr][4 * c8 + i] = wa[i], tile[lr][HALF / 2 + 4 * c8 + i] = wc[i];
    }
  }
  if (!jb.out_col) return;
  __syncthreads();
  // transposed write: work item (d, 8 consecutive slots) -> one 16-byte store
#pragma unroll
  for (int w = tid; w < D * 8; w += 256) {
    const int d = w >> 3, t8 = (w & 7) * 8, sh = 16 * (d & 1);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = ((tile[t8 + 2 * i][d >> 1] >> sh) & 0xffffu) | (((tile[t8 + 2 * i + 1][d >> 1] >> sh) & 0xffffu) << 16);
    const int sl = tok0 + t8;
    *(u32x4*)(jb.out_col + (int64_t)(b * jb.H + h) * D * P.spad + ((int64_t)(sl >> 5) * D + d) * 32 + (sl & 31)) = o;
  }
}

// 8 consecutive elements (16-byte aligned) as fp32, in 16-byte loads.
__device__ __forceinline__ void load8(const uint16_t* p, float* x) { unpack_bf8(*(const u32x4*)p, x); }
__device__ __forceinline__ void load8(const float* p, float* x) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = a[e], x[4 + e] = b[e];
}

// Delta[(b*Hq + h)][slot] = <dO row, O row> in fp32 (0 in slots without a
// token).  With lse given, also the rows' LSE in log2 units in the same slot
// layout right after Delta (+inf in slots without a token, so every
// probability recomputed for them is exactly 0).  With P.dnorm / P.dpart set
// (bf16 backward), also every row's ||dO||_1 and, per 64-slot block, the
// largest ||dO||_1 and |Delta| (the bounds of the dS scale).  With P.vpart
// set (stored dS), the first head of every KV group also writes the block's
// largest |v_jd| of the trunk V (key rows = the block's tokens).  Grid
// (spad/64, Hq, B), 256 threads, D/8 threads per row; each thread issues all
// its rows' loads first.
template <int D, typename OT, typename GT>
__global__ void __launch_bounds__(256) delta_kernel(Prob P, const OT* __restrict__ o, const GT* __restrict__ dout,
                                                    const float* __restrict__ lse, float* __restrict__ delta,
                                                    const uint16_t* __restrict__ vtr) {
  constexpr int TPR = D / 8;
  constexpr int ROWS = 256 / TPR;
  constexpr int NR = 64 / ROWS;  // rows per thread
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, c = tid % TPR;
  const bool vblk = P.vpart && h % P.r == 0;  // this block also bounds its keys' |v|
  const int64_t vo = ((int64_t)b * P.Hkv + h / P.r) * (P.spad / 64) + blockIdx.x;
  if (P.layout == 1 && thd_tile_unread(P, P.cu, P.stok, blockIdx.x * 64)) {
    if (P.dpart && tid == 0) {  // the group maxima still read this block's entry
      const int64_t bo = ((int64_t)(b * P.Hq + h) * (P.spad / 64) + blockIdx.x) * 2;
      P.dpart[bo] = P.dpart[bo + 1] = 0.f;
    }
    if (vblk && tid == 0) P.vpart[vo] = 0.f;
    return;
  }
  int slot[NR], tok[NR];
  bool valid[NR];
  float x[NR][8], y[NR][8];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    int row;
    slot[i] = blockIdx.x * 64 + i * ROWS + tid / TPR;
    valid[i] = slot_token(P, slot[i], tok[i], row);
    const int64_t off = (int64_t)b * P.os_b + (int64_t)(valid[i] ? tok[i] : 0) * P.os_t + (int64_t)h * P.os_h + 8 * c;
    load8(o + off, x[i]);
    load8(dout + off, y[i]);
  }
  float* lse2 = delta + (int64_t)P.B * P.Hq * P.spad;
  float nmax = 0.f, dmax = 0.f;  // this thread's rows: max ||dO||_1, max |Delta|
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float acc = 0.f, n1 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += x[i][e] * y[i][e], n1 += fabsf(y[i][e]);
    if (!valid[i]) acc = n1 = 0.f;
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, 64), n1 += __shfl_xor(n1, m, 64);
    const int64_t so = (int64_t)(b * P.Hq + h) * P.spad + slot[i];
    if (c == 0) delta[so] = acc;
    if (lse && c == 1)
      lse2[so] = valid[i] ? lse[(int64_t)b * P.lse_b + (int64_t)h * P.lse_h + tok[i]] * kLog2e : INFINITY;
    if (P.dnorm && c == 2) P.dnorm[so] = n1;
    nmax = fmaxf(nmax, n1);
    dmax = fmaxf(dmax, fabsf(acc));
  }
  float vmax = 0.f;
  if (vblk) {  // the same slots' rows of the group's trunk V (bf16)
    const int g = h / P.r;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (!valid[i]) continue;
      float v[8];
      load8(vtr + (int64_t)b * P.cs_b + (int64_t)tok[i] * P.cs_t + (int64_t)g * P.cs_h + 8 * c, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) vmax = fmaxf(vmax, fabsf(v[e]));
    }
  }
  if (P.dpart) {  // the block's 64 slots: one (max ||dO||_1, max |Delta|) entry
    __shared__ float red[3][4];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      nmax = fmaxf(nmax, __shfl_xor(nmax, m, 64));
      dmax = fmaxf(dmax, __shfl_xor(dmax, m, 64));
      vmax = fmaxf(vmax, __shfl_xor(vmax, m, 64));
    }
    if ((tid & 63) == 0) red[0][tid >> 6] = nmax, red[1][tid >> 6] = dmax, red[2][tid >> 6] = vmax;
    __syncthreads();
    if (tid == 0) {
      const int64_t bo = ((int64_t)(b * P.Hq + h) * (P.spad / 64) + blockIdx.x) * 2;
      P.dpart[bo] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
      P.dpart[bo + 1] = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
      if (vblk) P.vpart[vo] = fmaxf(fmaxf(red[2][0], red[2][1]), fmaxf(red[2][2], red[2][3]));
    }
  }
}

// Per KV group: the largest ||dO_i||_1 and |Delta_i| over every slot of the
// group's r query heads (the Delta kernel's 64-slot block entries), the bound
// from which the dK/dV kernel sets its fp16 dS scale.  Grid B*Hkv, 256
// threads.
__global__ void __launch_bounds__(256) dmax_kernel(Prob P) {
  __shared__ float red[2][4];
  const int bg = blockIdx.x, tid = threadIdx.x;
  const int nb = P.spad / 64;
  const float2* src = (const float2*)P.dpart + (int64_t)bg * P.r * nb;  // heads g*r .. g*r+r-1 are contiguous
  float n = 0.f, d = 0.f;
  for (int i = tid; i < P.r * nb; i += 256) {
    const float2 x = src[i];
    n = fmaxf(n, x.x);
    d = fmaxf(d, x.y);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) n = fmaxf(n, __shfl_xor(n, m, 64)), d = fmaxf(d, __shfl_xor(d, m, 64));
  if ((tid & 63) == 0) red[0][tid >> 6] = n, red[1][tid >> 6] = d;
  __syncthreads();
  if (tid == 0) {
    P.dmax[2 * bg] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    P.dmax[2 * bg + 1] = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  }
  if (P.vgmax) {  // stored dS: the group's largest |v_jd| (its trunk keys' 64-slot blocks)
    float v = 0.f;
    for (int i = tid; i < nb; i += 256) v = fmaxf(v, P.vpart[(int64_t)bg * nb + i]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    __syncthreads();
    if ((tid & 63) == 0) red[0][tid >> 6] = v;
    __syncthreads();
    if (tid == 0) P.vgmax[bg] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  }
}

// Varlen tile scheduler (THD).  First lays out the workspace slots: sequence
// s gets slot_base[s] .. slot_base[s+1], its length rounded up to 64 (clamped
// so the total stays inside the workspace).  Then, when `out` is given, splits
// every sequence into tiles of `tile` rows and lists them sequence-major:
// longest sequence first (ties: lower index first), and within a sequence the
// heavy tiles first -- descending tile index for the query-outer kernels
// (`desc`: a query tile's causal work grows with its index), ascending for
// the key-outer kernel (a key tile's work shrinks with its index).  The
// kernels map consecutive entries of one KV head to one XCD, so tiles of one
// sequence run side by side there and share the rows they stream through its
// L2; ranking by length keeps the heaviest tiles early.  Past 1024 sequences
// the sequences stay in index order.  Entry = {tile index, first token,
// length, first slot}; out[0].x = count.  One workgroup; deterministic order.
__global__ void __launch_bounds__(1024) tile_sched_kernel(Prob P, int tile, int desc, int4* __restrict__ out,
                                                          int max_entries, int* __restrict__ slot_base) {
  __shared__ int s_total;
  __shared__ int s_base;
  __shared__ int s_scan[1024];
  __shared__ int4 s_seq[1024];  // {first token, length, first slot, tiles} of each sequence
  const int tid = threadIdx.x;
  const int slot_cap = P.spad - 64;
  auto raw_len = [&](int s, int& a) {
    a = P.cu[s];
    int e = P.cu[s + 1];
    a = a < 0 ? 0 : (a > P.stok ? P.stok : a);
    e = e < a ? a : (e > P.stok ? P.stok : e);
    return e - a;
  };
  auto block_scan = [&](int v) {  // inclusive scan of v over the block
    s_scan[tid] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      int x = tid >= o ? s_scan[tid - o] : 0;
      __syncthreads();
      s_scan[tid] += x;
      __syncthreads();
    }
    return s_scan[tid];
  };
  if (tid == 0) s_base = 0, s_total = 0;
  __syncthreads();
  if (slot_base) {
    for (int s0 = 0; s0 < P.nseq; s0 += 1024) {
      int s = s0 + tid, a, w = 0;
      if (s < P.nseq) {
        int len = raw_len(s, a);
        if (P.kv_cu) {  // THD ring step: the segment's keys share its slots
          int ka = P.kv_cu[s], ke = P.kv_cu[s + 1];
          ka = ka < 0 ? 0 : (ka > P.kv_tok ? P.kv_tok : ka);
          ke = ke < ka ? ka : (ke > P.kv_tok ? P.kv_tok : ke);
          len = max(len, ke - ka);
        }
        w = (len + 63) & ~63;
      }
      int inc = block_scan(w);
      if (s < P.nseq) {
        int lo = s_base + inc - w;
        slot_base[s] = lo < slot_cap ? lo : slot_cap;
      }
      __syncthreads();
      if (tid == 1023) s_base += s_scan[1023];
      __syncthreads();
    }
    if (tid == 0) slot_base[P.nseq] = s_base < slot_cap ? s_base : slot_cap;
    __threadfence_block();
    __syncthreads();
    if (tid == 0) s_base = 0;
    __syncthreads();
  }
  if (!out) return;
  Prob Q = P;
  Q.slot_base = slot_base ? slot_base : P.slot_base;
  if (P.nseq <= 1024) {
    // a sequence's entries start after the tiles of every sequence ranked before it
    int st0 = 0, L = 0, nt = 0;
    if (tid < P.nseq) {
      int b;
      seq_info(Q, tid, b, st0, L);
      nt = (L + tile - 1) / tile;
      s_seq[tid] = make_int4(st0, L, Q.slot_base[tid], nt);
      atomicAdd(&s_total, nt);
    }
    __syncthreads();
    if (tid < P.nseq) {
      int base = 0;
      for (int s2 = 0; s2 < P.nseq; ++s2) {
        const int4 o = s_seq[s2];
        if (o.y > L || (o.y == L && s2 < tid)) base += o.w;
      }
      const int slot = s_seq[tid].z;
      for (int t = 0; t < nt; ++t)
        if (base + t < max_entries) out[1 + base + t] = make_int4(desc ? nt - 1 - t : t, st0, L, slot);
    }
    if (tid == 0) out[0] = make_int4(s_total < max_entries ? s_total : max_entries, 0, 0, 0);
    return;
  }
  for (int s0 = 0; s0 < P.nseq; s0 += 1024) {  // more sequences: index order
    const int s = s0 + tid;
    int b, st0 = 0, L = 0, nt = 0;
    if (s < P.nseq) {
      seq_info(Q, s, b, st0, L);
      nt = (L + tile - 1) / tile;
    }
    const int inc = block_scan(nt);
    const int base = s_base + inc - nt;
    for (int t = 0; t < nt; ++t)
      if (base + t < max_entries) out[1 + base + t] = make_int4(desc ? nt - 1 - t : t, st0, L, Q.slot_base[s]);
    __syncthreads();
    if (tid == 1023) s_base += s_scan[1023];
    __syncthreads();
  }
  if (tid == 0) out[0] = make_int4(s_base < max_entries ? s_base : max_entries, 0, 0, 0);
}

// bf16 head_dim 32 / 64 run on the D = 128 kernels with each head zero-padded:
// element k < D/2 of a head goes to entry (128/D) k, element D/2 + k to
// 64 + (128/D) k, and every other entry is 0.  The D = 128 rotate-half pair
// (j, j + 64) at angle pos * base^(-2j/128) is then exactly the D-dim pair
// (k, k + D/2) at pos * base^(-2k/D), zero entries stay zero under rotation,
// and every dot product and weighted sum over the padded head equals the one
// over the D real entries.  rows: tokens (B*S or T); the caller's tensor has
// element strides (sb, st, sh) with S tokens per batch row.
template <typename T>
__global__ void __launch_bounds__(256) pad_heads_kernel(const T* __restrict__ src, int64_t sb, int64_t st,
                                                        int64_t sh, int S, int H, int D, int64_t n,
                                                        T* __restrict__ dst) {
  // one thread per 16 bytes of a padded head (V entries)
  constexpr int V = 16 / sizeof(T), CH = 128 / V;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int c = (int)(idx % CH);
  const int64_t rh = idx / CH;
  const int h = (int)(rh % H);
  const int64_t r = rh / H;
  const T* row = src + (r / S) * sb + (r % S) * st + h * sh;
  const int sp = 128 / D, half = D / 2;
  T v[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const int j = c * V + e, jj = j & 63;
    v[e] = (jj % sp == 0) ? row[jj / sp + (j >= 64 ? half : 0)] : T(0);
  }
  *(u32x4*)(dst + idx * V) = *(const u32x4*)v;
}

// The inverse: the D real entries of each padded head back to the caller's strides.
// VEC: one thread per 16 bytes of a head (the caller's pointer and strides allow
// it), else one thread per entry.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256) unpad_heads_kernel(const T* __restrict__ src, int S, int H, int D, int64_t n,
                                                          T* __restrict__ dst, int64_t sb, int64_t st, int64_t sh) {
  constexpr int V = VEC ? 16 / sizeof(T) : 1;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int per = D / V;
  const int c = (int)(idx % per);
  const int64_t rh = idx / per;
  const int h = (int)(rh % H);
  const int64_t r = rh / H;
  const T* in = src + rh * 128;
  T* out = dst + (r / S) * sb + (r % S) * st + h * sh + c * V;
  const int sp = 128 / D, half = D / 2;
  T v[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const int k = c * V + e;
    v[e] = in[k < half ? sp * k : 64 + sp * (k - half)];
  }
  if constexpr (VEC)
    *(u32x4*)out = *(const u32x4*)v;
  else
    out[0] = v[0];
}

// ----------------------------------------------------------------------------- launchers
void launch_rope_table(const Prob& P, float* cosT, float* sinT, double base, hipStream_t st) {
  int64_t n = (int64_t)P.npos * (P.D / 2);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 65535) blocks = 65535;
  rope_table_kernel<<<blocks, 256, 0, st>>>(cosT, sinT, P.npos, P.D / 2, base);
}

template <int D, typename InT, bool ROT, typename RowT, typename ColT>
static void prep_rows_d(const Prob& P, const void* x, int64_t sb, int64_t st_, int64_t sh, int H, int pos_off,
                        const float* cosT, const float* sinT, void* out_row, void* out_col, hipStream_t st) {
  dim3 grid(P.spad / 64, H, P.B);
  prep_rows_kernel<D, InT, ROT, RowT, ColT><<<grid, 256, 0, st>>>(P, (const InT*)x, sb, st_, sh, H, pos_off, cosT,
                                                                  sinT, (RowT*)out_row, (ColT*)out_col);
}

template <typename InT, bool ROT, typename RowT, typename ColT>
static void prep_rows_any(const Prob& P, const void* x, int64_t sb, int64_t st_, int64_t sh, int H, int pos_off,
                          const float* cosT, const float* sinT, void* out_row, void* out_col, hipStream_t st) {
  if (P.D == 32)
    prep_rows_d<32, InT, ROT, RowT, ColT>(P, x, sb, st_, sh, H, pos_off, cosT, sinT, out_row, out_col, st);
  else if (P.D == 64)
    prep_rows_d<64, InT, ROT, RowT, ColT>(P, x, sb, st_, sh, H, pos_off, cosT, sinT, out_row, out_col, st);
  else
    prep_rows_d<128, InT, ROT, RowT, ColT>(P, x, sb, st_, sh, H, pos_off, cosT, sinT, out_row, out_col, st);
}

void launch_prep_rot_f32(const Prob& P, const float* x, int64_t sb, int64_t st_, int64_t sh, int H, int pos_off,
                         const float* cosT, const float* sinT, float* out_row, hipStream_t st) {
  prep_rows_any<float, true, float, float>(P, x, sb, st_, sh, H, pos_off, cosT, sinT, out_row, nullptr, st);
}

void launch_prep_bf16(const Prob& P, const PrepJobs& J, const float* cosT, const float* sinT, hipStream_t st) {
  dim3 grid((P.spad / 64) * (J.j[0].H + (J.n > 1 ? J.j[1].H : 0)), 1, P.B);
  prep_bf16_kernel<<<grid, 256, 0, st>>>(P, J, cosT, sinT);
}

void launch_dmax(const Prob& P, hipStream_t st) { dmax_kernel<<<P.B * P.Hkv, 256, 0, st>>>(P); }

void launch_delta(const Prob& P, const void* o, bool o_f32, const void* dout, bool g_f32, const float* lse,
                  float* delta, const void* v, hipStream_t st) {
  dim3 grid(P.spad / 64, P.Hq, P.B);
  const uint16_t* vt = (const uint16_t*)v;
#define TTT_DELTA(DD)                                                                              \
  if (P.D == DD) {                                                                                 \
    if (o_f32 && g_f32)                                                                            \
      delta_kernel<DD, float, float><<<grid, 256, 0, st>>>(P, (const float*)o, (const float*)dout, lse, delta, vt); \
    else if (o_f32)                                                                                \
      delta_kernel<DD, float, uint16_t><<<grid, 256, 0, st>>>(P, (const float*)o, (const uint16_t*)dout, lse, delta, vt); \
    else                                                                                           \
      delta_kernel<DD, uint16_t, uint16_t><<<grid, 256, 0, st>>>(P, (const uint16_t*)o, (const uint16_t*)dout, lse, delta, vt); \
    return;                                                                                        \
  }
  TTT_DELTA(32)
  TTT_DELTA(64)
  TTT_DELTA(128)
#undef TTT_DELTA
}

// Joint-LSE merge of two partial results over disjoint key sets of the same
// rows: LSE = ln(e^LSE_a + e^LSE_b), O = e^(LSE_a-LSE) O_a + e^(LSE_b-LSE) O_b
// (NeMo-RL issue on EAGLE-3 TTT draft co-training, "What I'm working on",
// items 1 and 4).  One thread per 8 elements of a row (a row's threads are in
// one wave, so in-place merges read every input before any output is written).
template <typename OT>
__global__ void __launch_bounds__(256) merge_kernel(Prob P, const OT* oa, const float* la,
                                                    const OT* ob, const float* lb, OT* o, float* l) {
  const int cpr = P.D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / cpr;
  const int c = (int)(gid % cpr);
  if (row >= (int64_t)P.B * P.stok * P.Hq) return;
  const int h = (int)(row % P.Hq);
  const int64_t bt = row / P.Hq;
  const int t = (int)(bt % P.stok), b = (int)(bt / P.stok);
  const int64_t li = b * P.lse_b + h * P.lse_h + t;
  const int64_t oi = b * P.os_b + (int64_t)t * P.os_t + h * P.os_h + c * 8;
  const float A = la[li], Bv = lb[li];
  const float m = fmaxf(A, Bv);
  float wa = 0.f, wb = 0.f, L = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(A - m), eb = expf(Bv - m), sum = ea + eb;
    wa = ea / sum;
    wb = eb / sum;
    L = m + logf(sum);
  }
  float x[8], y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = ld<OT>(oa + oi + e), y[e] = ld<OT>(ob + oi + e);
#pragma unroll
  for (int e = 0; e < 8; ++e) st<OT>(o + oi + e, wa * x[e] + wb * y[e]);
  if (c == 0) l[li] = L;
}

void launch_merge(const Prob& P, bool o_f32, const void* o_a, const float* lse_a, const void* o_b,
                  const float* lse_b, void* o, float* lse, hipStream_t st) {
  const int64_t threads = (int64_t)P.B * P.stok * P.Hq * (P.D / 8);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (o_f32)
    merge_kernel<float><<<grid, 256, 0, st>>>(P, (const float*)o_a, lse_a, (const float*)o_b, lse_b, (float*)o, lse);
  else
    merge_kernel<uint16_t><<<grid, 256, 0, st>>>(P, (const uint16_t*)o_a, lse_a, (const uint16_t*)o_b, lse_b,
                                                 (uint16_t*)o, lse);
}

void launch_tile_sched(const Prob& P, int tile, int desc, int4* out, int max_entries, int* slot_base,
                       hipStream_t st) {
  tile_sched_kernel<<<1, 1024, 0, st>>>(P, tile, desc, out, max_entries, slot_base);
}

void launch_pad_heads(const void* src, bool f32, int64_t sb, int64_t st, int64_t sh, int64_t rows, int S, int H,
                      int D, void* dst, hipStream_t st_) {
  const int64_t n = rows * H * (f32 ? 32 : 16);  // 16-byte pieces of the padded heads
  if (n == 0) return;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (f32)
    pad_heads_kernel<float><<<blocks, 256, 0, st_>>>((const float*)src, sb, st, sh, S, H, D, n, (float*)dst);
  else
    pad_heads_kernel<uint16_t><<<blocks, 256, 0, st_>>>((const uint16_t*)src, sb, st, sh, S, H, D, n, (uint16_t*)dst);
}

template <typename T>
static void unpad_as(const void* src, int64_t rows, int S, int H, int D, void* dst, int64_t sb, int64_t st,
                     int64_t sh, hipStream_t st_) {
  constexpr int V = 16 / sizeof(T);
  const bool vec = ((uintptr_t)dst % 16) == 0 && sb % V == 0 && st % V == 0 && sh % V == 0;
  const int64_t n = rows * H * (vec ? D / V : D);
  if (n == 0) return;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (vec)
    unpad_heads_kernel<T, true><<<blocks, 256, 0, st_>>>((const T*)src, S, H, D, n, (T*)dst, sb, st, sh);
  else
    unpad_heads_kernel<T, false><<<blocks, 256, 0, st_>>>((const T*)src, S, H, D, n, (T*)dst, sb, st, sh);
}

void launch_unpad_heads(const void* src, bool f32, int64_t rows, int S, int H, int D, void* dst, int64_t sb,
                        int64_t st, int64_t sh, hipStream_t st_) {
  if (f32)
    unpad_as<float>(src, rows, S, H, D, dst, sb, st, sh, st_);
  else
    unpad_as<uint16_t>(src, rows, S, H, D, dst, sb, st, sh, st_);
}

}  // namespace ttt
