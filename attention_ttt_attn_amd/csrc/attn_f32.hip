// fp32 path: plain VALU kernels, one wavefront per output row.
//
// On MI355X the fp32 matrix-core rate equals the fp32 vector rate, so this
// precision runs on the vector ALUs with fp32 accumulation throughout.  It
// computes the same two-part attention as the bf16 path: a causal trunk over
// the pass-1 keys, the branch over the passes 2..p keys of the same row, and
// the exact log-sum-exp merge of the two partial softmaxes (NeMo-RL issue
// "DFlash/DSpark and EAGLE-3 TTT draft co-training ...", "What I'm working
// on", item 1).
#include "kernels.hpp"

namespace ttt {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// R(pos) applied to row x into LDS dst (lanes < D/2 each own one pair).
template <int D>
__device__ __forceinline__ void rotate_into(float* dst, const float* x, int pos, const float* cosT,
                                            const float* sinT, int lane) {
  constexpr int HALF = D / 2;
  if (lane < HALF) {
    float a = x[lane], b = x[lane + HALF];
    float c = cosT[(int64_t)pos * HALF + lane], s = sinT[(int64_t)pos * HALF + lane];
    dst[lane] = a * c - b * s;
    dst[lane + HALF] = b * c + a * s;
  }
}

// R(pos)^T applied to LDS row src, written to global dst.
template <int D>
__device__ __forceinline__ void unrotate_store(float* dst, const float* src, int pos, const float* cosT,
                                               const float* sinT, int lane) {
  constexpr int HALF = D / 2;
  if (lane < HALF) {
    float a = src[lane], b = src[lane + HALF];
    float c = cosT[(int64_t)pos * HALF + lane], s = sinT[(int64_t)pos * HALF + lane];
    dst[lane] = a * c + b * s;
    dst[lane + HALF] = b * c - a * s;
  }
}

// Forward: grid (stok, Hq, B), one wave per (token, head).
template <int D>
__global__ void __launch_bounds__(64) fwd_f32_kernel(Prob P, const float* __restrict__ q, PassPtrs kv,
                                                     const float* __restrict__ kt, const float* __restrict__ cosT,
                                                     const float* __restrict__ sinT, float* __restrict__ o,
                                                     float* __restrict__ lse) {
  constexpr int NPL = (D + 63) / 64;
  const int tok = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int s, start, L;
  if (!token_seq(P, tok, s, start, L)) return;
  const int i = tok - start, g = h / P.r, slot0 = seq_slot0(P, s);
  __shared__ float qs[D], kq[D], ps[64];
  rotate_into<D>(qs, q + b * P.qs_b + tok * P.qs_t + h * P.qs_h, i + P.p - 1, cosT, sinT, lane);
  __syncthreads();

  // trunk: keys j = 0..i of pass 1 (rotated copy in kt), online softmax
  float m = -INFINITY, l = 0.f, acc[NPL] = {};
  const float* kb = kt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0) * D;
  const float* v1 = (const float*)kv.v[0] + b * P.ks_b + (int64_t)start * P.ks_t + g * P.ks_h;
  for (int j0 = 0; j0 <= i; j0 += 64) {
    int j = j0 + lane;
    float sc = -INFINITY;
    if (j <= i) {
      float d0 = 0.f;
      for (int d = 0; d < D; ++d) d0 += qs[d] * kb[(int64_t)j * D + d];
      sc = d0 * P.scale;
    }
    float mn = fmaxf(m, wave_max(sc));
    float alpha = expf(m - mn);
    float pj = j <= i ? expf(sc - mn) : 0.f;
    l = l * alpha + wave_sum(pj);
    ps[lane] = pj;
    __syncthreads();
    int cnt = min(64, i + 1 - j0);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      if (d < D) {
        float a = acc[e] * alpha;
        for (int jj = 0; jj < cnt; ++jj) a += ps[jj] * v1[(int64_t)(j0 + jj) * P.ks_t + d];
        acc[e] = a;
      }
    }
    __syncthreads();
    m = mn;
  }

  // branch: the key/value of passes 2..p at this row
  float mb = -INFINITY, lb = 0.f, accb[NPL] = {};
  for (int qq = 2; qq <= P.p; ++qq) {
    const int64_t off = b * P.ks_b + (int64_t)tok * P.ks_t + g * P.ks_h;
    rotate_into<D>(kq, (const float*)kv.k[qq - 1] + off, i + qq - 1, cosT, sinT, lane);
    __syncthreads();
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      if (d < D) part += qs[d] * kq[d];
    }
    float sc = wave_sum(part) * P.scale;
    float mn = fmaxf(mb, sc);
    float alpha = expf(mb - mn), pe = expf(sc - mn);
    lb = lb * alpha + pe;
    const float* vr = (const float*)kv.v[qq - 1] + off;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      if (d < D) accb[e] = accb[e] * alpha + pe * vr[d];
    }
    mb = mn;
    __syncthreads();
  }

  // exact joint log-sum-exp merge of the two partials
  float lse_t = m + logf(l);
  float lse_b = P.p > 1 ? mb + logf(lb) : -INFINITY;
  float M = fmaxf(lse_t, lse_b);
  float LSE = M + logf(expf(lse_t - M) + expf(lse_b - M));
  float wt = expf(lse_t - LSE) / l;
  float wb = P.p > 1 ? expf(lse_b - LSE) / lb : 0.f;
  float* orow = o + b * P.os_b + (int64_t)tok * P.os_t + h * P.os_h;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < D) orow[d] = wt * acc[e] + wb * accb[e];
  }
  if (lane == 0) lse[b * P.lse_b + h * P.lse_h + tok] = LSE;
}

// dQ: grid (stok, Hq, B), one wave per (token, head).
template <int D>
__global__ void __launch_bounds__(64) dq_f32_kernel(Prob P, PassPtrs kv, const float* __restrict__ lse,
                                                    const float* __restrict__ dout, const float* __restrict__ kt,
                                                    const float* __restrict__ qt, const float* __restrict__ delta,
                                                    const float* __restrict__ cosT, const float* __restrict__ sinT,
                                                    float* __restrict__ dq) {
  constexpr int NPL = (D + 63) / 64;
  const int tok = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int s, start, L;
  if (!token_seq(P, tok, s, start, L)) return;
  const int i = tok - start, g = h / P.r, slot0 = seq_slot0(P, s);
  __shared__ float qs[D], gs[D], kq[D], ds[64];
  const float* qrow = qt + ((int64_t)(b * P.Hq + h) * P.spad + slot0 + i) * D;
  const float* grow = dout + b * P.os_b + (int64_t)tok * P.os_t + h * P.os_h;
  for (int d = lane; d < D; d += 64) qs[d] = qrow[d], gs[d] = grow[d];
  const float LSE = lse[b * P.lse_b + h * P.lse_h + tok];
  const float dl = delta[(int64_t)(b * P.Hq + h) * P.spad + slot0 + i];
  __syncthreads();
  float acc[NPL] = {};
  const float* kb = kt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0) * D;
  const float* v1 = (const float*)kv.v[0] + b * P.ks_b + (int64_t)start * P.ks_t + g * P.ks_h;
  for (int j0 = 0; j0 <= i; j0 += 64) {
    int j = j0 + lane;
    float dsj = 0.f;
    if (j <= i) {
      float sc = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        sc += qs[d] * kb[(int64_t)j * D + d];
        dp += gs[d] * v1[(int64_t)j * P.ks_t + d];
      }
      float pr = expf(sc * P.scale - LSE);
      dsj = pr * (dp - dl);
    }
    ds[lane] = dsj;
    __syncthreads();
    int cnt = min(64, i + 1 - j0);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      if (d < D)
        for (int jj = 0; jj < cnt; ++jj) acc[e] += ds[jj] * kb[(int64_t)(j0 + jj) * D + d];
    }
    __syncthreads();
  }
  for (int qq = 2; qq <= P.p; ++qq) {
    const int64_t off = b * P.ks_b + (int64_t)tok * P.ks_t + g * P.ks_h;
    rotate_into<D>(kq, (const float*)kv.k[qq - 1] + off, i + qq - 1, cosT, sinT, lane);
    __syncthreads();
    const float* vr = (const float*)kv.v[qq - 1] + off;
    float ps = 0.f, pd = 0.f;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      if (d < D) ps += qs[d] * kq[d], pd += gs[d] * vr[d];
    }
    float sc = wave_sum(ps), dp = wave_sum(pd);
    float pr = expf(sc * P.scale - LSE);
    float dsb = pr * (dp - dl);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      if (d < D) acc[e] += dsb * kq[d];
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < D) kq[d] = acc[e] * P.scale;
  }
  __syncthreads();
  unrotate_store<D>(dq + b * P.qs_b + (int64_t)tok * P.qs_t + h * P.qs_h, kq, i + P.p - 1, cosT, sinT, lane);
}

// Trunk dK/dV: grid (stok, Hkv, B), one wave per (key token j, KV head);
// sums over the r query heads of the group and every row i >= j.
template <int D>
__global__ void __launch_bounds__(64) dkdv_f32_kernel(Prob P, PassPtrs kv, const float* __restrict__ lse,
                                                      const float* __restrict__ dout, const float* __restrict__ kt,
                                                      const float* __restrict__ qt, const float* __restrict__ delta,
                                                      const float* __restrict__ cosT, const float* __restrict__ sinT,
                                                      PassGradPtrs gr) {
  constexpr int NPL = (D + 63) / 64;
  const int tok = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int s, start, L;
  if (!token_seq(P, tok, s, start, L)) return;
  const int j = tok - start, slot0 = seq_slot0(P, s);
  __shared__ float ks_[D], vs_[D], pp[64], dd[64];
  const float* krow = kt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0 + j) * D;
  const float* vrow = (const float*)kv.v[0] + b * P.ks_b + (int64_t)tok * P.ks_t + g * P.ks_h;
  for (int d = lane; d < D; d += 64) ks_[d] = krow[d], vs_[d] = vrow[d];
  __syncthreads();
  float dk[NPL] = {}, dv[NPL] = {};
  for (int hh = 0; hh < P.r; ++hh) {
    const int h = g * P.r + hh;
    const float* qb = qt + ((int64_t)(b * P.Hq + h) * P.spad + slot0) * D;
    const float* gb = dout + b * P.os_b + (int64_t)start * P.os_t + h * P.os_h;
    for (int i0 = j; i0 < L; i0 += 64) {
      int i = i0 + lane;
      float pv = 0.f, dsv = 0.f;
      if (i < L) {
        float sc = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          sc += qb[(int64_t)i * D + d] * ks_[d];
          dp += gb[(int64_t)i * P.os_t + d] * vs_[d];
        }
        float LSE = lse[b * P.lse_b + h * P.lse_h + start + i];
        float dl = delta[(int64_t)(b * P.Hq + h) * P.spad + slot0 + i];
        pv = expf(sc * P.scale - LSE);
        dsv = pv * (dp - dl);
      }
      pp[lane] = pv;
      dd[lane] = dsv;
      __syncthreads();
      int cnt = min(64, L - i0);
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        int d = lane + 64 * e;
        if (d < D)
          for (int ii = 0; ii < cnt; ++ii) {
            dv[e] += pp[ii] * gb[(int64_t)(i0 + ii) * P.os_t + d];
            dk[e] += dd[ii] * qb[(int64_t)(i0 + ii) * D + d];
          }
      }
      __syncthreads();
    }
  }
  const int64_t off = b * P.ks_b + (int64_t)tok * P.ks_t + g * P.ks_h;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    int d = lane + 64 * e;
    if (d < D) {
      ((float*)gr.dv[0])[off + d] = dv[e];
      ks_[d] = dk[e] * P.scale;
    }
  }
  __syncthreads();
  unrotate_store<D>((float*)gr.dk[0] + off, ks_, j, cosT, sinT, lane);
}

// Branch dK/dV for passes 2..p: grid (stok, Hkv, B), one wave per (row, KV head).
template <int D>
__global__ void __launch_bounds__(64) branch_bwd_f32_kernel(Prob P, PassPtrs kv, const float* __restrict__ lse,
                                                            const float* __restrict__ dout,
                                                            const float* __restrict__ qt,
                                                            const float* __restrict__ delta,
                                                            const float* __restrict__ cosT,
                                                            const float* __restrict__ sinT, PassGradPtrs gr) {
  constexpr int NPL = (D + 63) / 64;
  const int tok = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int s, start, L;
  if (!token_seq(P, tok, s, start, L)) return;
  const int i = tok - start, slot0 = seq_slot0(P, s);
  __shared__ float kq[D];
  const int64_t off = b * P.ks_b + (int64_t)tok * P.ks_t + g * P.ks_h;
  for (int qq = 2; qq <= P.p; ++qq) {
    rotate_into<D>(kq, (const float*)kv.k[qq - 1] + off, i + qq - 1, cosT, sinT, lane);
    __syncthreads();
    const float* vr = (const float*)kv.v[qq - 1] + off;
    float dk[NPL] = {}, dv[NPL] = {};
    for (int hh = 0; hh < P.r; ++hh) {
      const int h = g * P.r + hh;
      const float* qrow = qt + ((int64_t)(b * P.Hq + h) * P.spad + slot0 + i) * D;
      const float* grow = dout + b * P.os_b + (int64_t)tok * P.os_t + h * P.os_h;
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        int d = lane + 64 * e;
        if (d < D) ps += qrow[d] * kq[d], pd += grow[d] * vr[d];
      }
      float sc = wave_sum(ps), dp = wave_sum(pd);
      float pr = expf(sc * P.scale - lse[b * P.lse_b + h * P.lse_h + tok]);
      float dsb = pr * (dp - delta[(int64_t)(b * P.Hq + h) * P.spad + slot0 + i]);
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        int d = lane + 64 * e;
        if (d < D) dk[e] += dsb * qrow[d], dv[e] += pr * grow[d];
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      int d = lane + 64 * e;
      if (d < D) {
        ((float*)gr.dv[qq - 1])[off + d] = dv[e];
        kq[d] = dk[e] * P.scale;
      }
    }
    __syncthreads();
    unrotate_store<D>((float*)gr.dk[qq - 1] + off, kq, i + qq - 1, cosT, sinT, lane);
    __syncthreads();
  }
}

void launch_fwd_f32(const Prob& P, const float* q, const PassPtrs& kv, const float* kt, const float* cosT,
                    const float* sinT, float* o, float* lse, hipStream_t st) {
  dim3 grid(P.stok, P.Hq, P.B);
  if (P.D == 32) fwd_f32_kernel<32><<<grid, 64, 0, st>>>(P, q, kv, kt, cosT, sinT, o, lse);
  else if (P.D == 64) fwd_f32_kernel<64><<<grid, 64, 0, st>>>(P, q, kv, kt, cosT, sinT, o, lse);
  else fwd_f32_kernel<128><<<grid, 64, 0, st>>>(P, q, kv, kt, cosT, sinT, o, lse);
}

template <int D>
static void bwd_f32_d(const Prob& P, const PassPtrs& kv, const float* lse, const float* dout, const float* kt,
                      const float* qt, const float* delta, const float* cosT, const float* sinT, float* dq,
                      const PassGradPtrs& g, hipStream_t st) {
  trace("dq_f32", 0, st);
  dq_f32_kernel<D><<<dim3(P.stok, P.Hq, P.B), 64, 0, st>>>(P, kv, lse, dout, kt, qt, delta, cosT, sinT, dq);
  trace("dq_f32", 1, st);
  trace("dkdv_f32", 0, st);
  dkdv_f32_kernel<D><<<dim3(P.stok, P.Hkv, P.B), 64, 0, st>>>(P, kv, lse, dout, kt, qt, delta, cosT, sinT, g);
  trace("dkdv_f32", 1, st);
  if (P.p > 1) {
    trace("branch_bwd_f32", 0, st);
    branch_bwd_f32_kernel<D><<<dim3(P.stok, P.Hkv, P.B), 64, 0, st>>>(P, kv, lse, dout, qt, delta, cosT, sinT, g);
    trace("branch_bwd_f32", 1, st);
  }
}

void launch_bwd_f32(const Prob& P, const PassPtrs& kv, const float* lse, const float* dout, const float* kt,
                    const float* qt, const float* delta, const float* cosT, const float* sinT, float* dq,
                    const PassGradPtrs& g, hipStream_t st) {
  if (P.D == 32) bwd_f32_d<32>(P, kv, lse, dout, kt, qt, delta, cosT, sinT, dq, g, st);
  else if (P.D == 64) bwd_f32_d<64>(P, kv, lse, dout, kt, qt, delta, cosT, sinT, dq, g, st);
  else bwd_f32_d<128>(P, kv, lse, dout, kt, qt, delta, cosT, sinT, dq, g, st);
}

}  // namespace ttt
