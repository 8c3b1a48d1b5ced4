// Per-pass soft cross-entropy distillation loss (the step after the attention).
//
// Method (NeMo-RL issue "DFlash/DSpark and EAGLE-3 TTT draft co-training for
// speculative decoding (Megatron backend)", "What I'm working on", item 3:
// chunked soft cross-entropy normalised per pass over the whole batch; NeMo-RL
// PR #3725, self-review comment: teacher_offset = pass_index + 1): pass p's
// student logits at row i are scored against softmax(teacher logits at row
// i + offset) of the same sequence; rows without such a teacher row, or with
// mask 0, are not counted; loss = sum of the counted rows' cross-entropies /
// number of counted rows.  Block-draft slots (same item: per-slot
// normalisation) pass a teacher row per student row (slot at position a + t:
// row a + t + 1) and a group per row (the slot index); each group is then
// normalised by its own count and the loss is the sum of the group means.
// Chunking over tokens only bounds memory in a
// framework implementation; these kernels stream every row once, so no [T, V]
// intermediate exists at all.
//
// gfx950 design: HBM-bound.  One 256-thread workgroup per row; each thread
// streams 16-byte chunks of the student and teacher rows, U of each in flight,
// with an online (max, sum) in the log2 domain for both, plus the
// teacher-weighted student sum, so the forward reads each logit once.  States merge across lanes with
// shuffles and across the 4 waves through LDS.  The mean over rows is a
// fixed-order reduction (deterministic).  The backward reads both rows once
// more and writes (softmax(student) - teacher distribution) * dloss / count.
#include "kernels.hpp"

namespace ttt {

namespace ce {

constexpr int NT = 256;
constexpr int U = 4;  // 16-byte chunks of each row a thread has in flight

// merges (m2, l2, w2) into (m, l, w); w is scaled like l
__device__ __forceinline__ void merge(float& m, float& l, float& w, float m2, float l2, float w2) {
  const float mx = fmaxf(m, m2);
  if (mx == -INFINITY) return;
  const float a = fast_exp2(m - mx), b = fast_exp2(m2 - mx);
  l = l * a + l2 * b;
  w = w * a + w2 * b;
  m = mx;
}

// Row (b, i): whether it is counted, its teacher row and its group.
__device__ __forceinline__ bool counted(const CeProb& C, int b, int i, int& trow, int& grp) {
  const int64_t r = (int64_t)b * C.S + i;
  trow = C.trows ? C.trows[r] : i + C.offset;
  grp = C.groups ? C.groups[r] : 0;
  return trow >= 0 && trow < C.T && grp >= 0 && grp < C.G && (!C.mask || C.mask[r] != 0);
}

__global__ void __launch_bounds__(NT) soft_ce_fwd_kernel(CeProb C, const uint16_t* __restrict__ s,
                                                         const uint16_t* __restrict__ t,
                                                         float* __restrict__ row_lse, float* __restrict__ row_ce) {
  const int row = blockIdx.x;
  const int b = row / C.S, i = row % C.S;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int trow, grp;
  if (!counted(C, b, i, trow, grp)) {
    if (tid == 0) {
      row_lse[2 * (int64_t)row] = 0.f;
      row_lse[2 * (int64_t)row + 1] = 0.f;
      if (row_ce) row_ce[row] = 0.f;
    }
    return;
  }
  const uint16_t* sr = s + (int64_t)b * C.ss_b + (int64_t)i * C.ss_t;
  const uint16_t* tr = t + (int64_t)b * C.ts_b + (int64_t)trow * C.ts_t;
  // student: (ms, ls); teacher: (mt, lt) and wt = sum 2^(t2 - mt) * s.  All
  // U chunks' loads are issued before any of them is used.
  float ms = -INFINITY, ls = 0.f, mt = -INFINITY, lt = 0.f, wt = 0.f;
  for (int v0 = tid * 8; v0 < C.V; v0 += NT * 8 * U) {
    u32x4 xs[U], ys[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * NT * 8 < C.V) {
        xs[u] = *(const u32x4*)(sr + v0 + u * NT * 8);
        ys[u] = *(const u32x4*)(tr + v0 + u * NT * 8);
      }
    float cx = -INFINITY, cy = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * NT * 8 < C.V) {
        float x[8], y[8];
        unpack_bf8(xs[u], x);
        unpack_bf8(ys[u], y);
#pragma unroll
        for (int e = 0; e < 8; ++e) cx = fmaxf(cx, x[e]), cy = fmaxf(cy, y[e]);
      }
    cx *= kLog2e;
    cy *= kLog2e;
    if (cx > ms) {
      ls *= fast_exp2(ms - cx);
      ms = cx;
    }
    if (cy > mt) {
      const float a = fast_exp2(mt - cy);
      lt *= a;
      wt *= a;
      mt = cy;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * NT * 8 < C.V) {
        float x[8], y[8];
        unpack_bf8(xs[u], x);
        unpack_bf8(ys[u], y);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ls += fast_exp2(__builtin_fmaf(x[e], kLog2e, -ms));
          const float pe = fast_exp2(__builtin_fmaf(y[e], kLog2e, -mt));
          lt += pe;
          wt = __builtin_fmaf(pe, x[e], wt);
        }
      }
  }
  // lanes, then waves
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    float dummy = 0.f;
    merge(ms, ls, dummy, __shfl_xor(ms, m, 64), __shfl_xor(ls, m, 64), 0.f);
    merge(mt, lt, wt, __shfl_xor(mt, m, 64), __shfl_xor(lt, m, 64), __shfl_xor(wt, m, 64));
  }
  __shared__ float red[4][5];
  if (lane == 0) red[wv][0] = ms, red[wv][1] = ls, red[wv][2] = mt, red[wv][3] = lt, red[wv][4] = wt;
  __syncthreads();
  if (tid == 0) {
    float dummy = 0.f;
    for (int w = 1; w < 4; ++w) {
      merge(ms, ls, dummy, red[w][0], red[w][1], 0.f);
      merge(mt, lt, wt, red[w][2], red[w][3], red[w][4]);
    }
    const float lse_s = (ms + fast_log2(ls)) * kLn2;
    const float lse_t = (mt + fast_log2(lt)) * kLn2;
    row_lse[2 * (int64_t)row] = lse_s;
    row_lse[2 * (int64_t)row + 1] = lse_t;
    // cross-entropy = lse(s) - E_teacher[s]
    if (row_ce) row_ce[row] = lse_s - wt / lt;
  }
}

// Fixed-order means per group: for each group, thread k sums its rows k,
// k + 1024, ...; then a fixed tree.  out = (sum of the group means, counted
// rows, then each group's (mean, count)).
__global__ void __launch_bounds__(1024) soft_ce_mean_kernel(CeProb C, const float* __restrict__ row_ce,
                                                            float* __restrict__ out) {
  __shared__ double sum[1024];
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  const int rows = C.B * C.S;
  double loss = 0.0;
  int total = 0;
  for (int g = 0; g < C.G; ++g) {
    double a = 0.0;
    int n = 0;
    for (int r = tid; r < rows; r += 1024) {
      int trow, grp;
      if (counted(C, r / C.S, r % C.S, trow, grp) && grp == g) {
        a += (double)row_ce[r];
        ++n;
      }
    }
    sum[tid] = a;
    cnt[tid] = n;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
      if (tid < w) {
        sum[tid] += sum[tid + w];
        cnt[tid] += cnt[tid + w];
      }
      __syncthreads();
    }
    const double mean = cnt[0] ? sum[0] / cnt[0] : 0.0;
    loss += mean;
    total += cnt[0];
    if (tid == 0) {
      out[2 + 2 * g] = (float)mean;
      out[3 + 2 * g] = (float)cnt[0];
    }
    __syncthreads();  // sum/cnt are reused by the next group
  }
  if (tid == 0) {
    out[0] = (float)loss;
    out[1] = (float)total;
  }
}

// dstudent = dloss[g] / count_g * (softmax(student) - teacher distribution) on
// counted rows of group g, 0 elsewhere.
__global__ void __launch_bounds__(NT) soft_ce_bwd_kernel(CeProb C, const uint16_t* __restrict__ s,
                                                         const uint16_t* __restrict__ t,
                                                         const float* __restrict__ row_lse,
                                                         const float* __restrict__ stats,
                                                         const float* __restrict__ dloss, uint16_t* __restrict__ g) {
  const int row = blockIdx.x;
  const int b = row / C.S, i = row % C.S;
  const int tid = threadIdx.x;
  uint16_t* gr = g + (int64_t)b * C.ss_b + (int64_t)i * C.ss_t;
  int trow, grp;
  if (!counted(C, b, i, trow, grp)) {
    for (int v0 = tid * 8; v0 < C.V; v0 += NT * 8) *(u32x4*)(gr + v0) = u32x4{0, 0, 0, 0};
    return;
  }
  const uint16_t* sr = s + (int64_t)b * C.ss_b + (int64_t)i * C.ss_t;
  const uint16_t* tr = t + (int64_t)b * C.ts_b + (int64_t)trow * C.ts_t;
  const float n = stats[3 + 2 * grp];
  const float scale = n > 0.f ? dloss[grp] / n : 0.f;
  const float ls2 = row_lse[2 * (int64_t)row] * kLog2e, lt2 = row_lse[2 * (int64_t)row + 1] * kLog2e;
  for (int v0 = tid * 8; v0 < C.V; v0 += NT * 8 * U) {
    u32x4 xs[U], ys[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * NT * 8 < C.V) {
        xs[u] = *(const u32x4*)(sr + v0 + u * NT * 8);
        ys[u] = *(const u32x4*)(tr + v0 + u * NT * 8);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v0 + u * NT * 8 < C.V) {
        float x[8], y[8], o[8];
        unpack_bf8(xs[u], x);
        unpack_bf8(ys[u], y);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] = scale * (fast_exp2(__builtin_fmaf(x[e], kLog2e, -ls2)) - fast_exp2(__builtin_fmaf(y[e], kLog2e, -lt2)));
        *(u32x4*)(gr + v0 + u * NT * 8) = pack_bf8(o);
      }
  }
}

}  // namespace ce

void launch_soft_ce_fwd(const CeProb& C, const uint16_t* s, const uint16_t* t, float* row_lse, float* row_ce,
                        float* stats, hipStream_t st) {
  const unsigned rows = (unsigned)(C.B * C.S);
  if (rows) ce::soft_ce_fwd_kernel<<<rows, ce::NT, 0, st>>>(C, s, t, row_lse, row_ce);
  ce::soft_ce_mean_kernel<<<1, 1024, 0, st>>>(C, row_ce, stats);
}

void launch_soft_ce_bwd(const CeProb& C, const uint16_t* s, const uint16_t* t, const float* row_lse,
                        const float* stats, const float* dloss, uint16_t* g, hipStream_t st) {
  ce::soft_ce_bwd_kernel<<<(unsigned)(C.B * C.S), ce::NT, 0, st>>>(C, s, t, row_lse, stats, dloss, g);
}

}  // namespace ttt
