// bf16 forward: trunk flash attention on MFMA with the branch reduction and
// the joint log-sum-exp merge fused into its epilogue.
//
// Method (NeMo-RL issue "DFlash/DSpark and EAGLE-3 TTT draft co-training for
// speculative decoding (Megatron backend)", "What I'm working on", item 1;
// NeMo-RL PR #3725, Summary and self-review comment): at pass p, query row i
// (position i+p-1) attends causally to the pass-1 keys j <= i (trunk) and to
// the keys passes 2..p produced at row i (branch, position i+q-1); the two
// partial softmaxes are joined exactly through their log-sum-exps.  No score
// matrix or mask is ever stored.
//
// gfx950 design
// * One workgroup = 4 wave64s = 128 query rows of one head; each wave owns 32
//   rows.  Scores are computed transposed, S^T = K~ Q~^T, with
//   v_mfma_f32_32x32x16_f16: in the accumulator each lane then holds 16 keys
//   of ONE query, so the running max/sum are per-lane scalars (one
//   cross-half exchange per tile) and the O rescale needs no broadcast.
// * K~ rows for the A operand are read in a permuted order (bits 2 and 3 of the
//   row swapped) so that the score accumulator is already laid out as the B
//   operand of O^T = V^T P^T (v_mfma_f32_32x32x16_bf16): no shuffle between
//   the two matrix products.
// * Q~ = R(i+p-1) q is rotated in fp32 once per workgroup and kept in VGPRs as
//   fp16 (exact for the bf16 inputs' range, 8x finer rounding than bf16 after
//   the rotation); K~ = R(j) k^(1) arrives pre-rotated in fp16 and V^(1)
//   pre-transposed in bf16 from the prologue, so the hot loop is copies and
//   MFMAs.  K~ and V^T tiles of 64 keys are double-buffered in padded LDS rows
//   (conflict-free 16-byte reads); one barrier per tile.
// * Softmax runs in the log2 domain (scale*log2e folded into one FMA,
//   v_exp_f32).  Only tiles that reach past a wave's first row are masked;
//   tiles above the diagonal are never visited.
// * Epilogue: O_t and (m, l) go through LDS to a row-major layout (8 lanes per
//   row, each lane a rotate-half pair of 8-element chunks).  The branch keys of
//   passes 2..p are read, rotated in fp32 and reduced with 3 xor-shuffles per
//   key; the joint-LSE merge then writes O (bf16 or fp32, 16-byte stores) and
//   the natural-log LSE.
// * Grid: heavy-first (descending query tile), and the r = Hq/Hkv heads that
//   share a KV head are placed on the same XCD back to back so that their
//   K/V tiles are served from that XCD's L2.
#include <type_traits>

#include "kernels.hpp"

namespace ttt {

namespace fwd {

constexpr int D = 128;
constexpr int BM = kFwdBM;  // 128 query rows per workgroup
constexpr int BN = 64;      // keys per tile
constexpr int KPAD = D + 8;
constexpr int VPAD = BN + 8;
constexpr int OPAD = D + 4;

struct Smem {
  union {
    struct {
      _Float16 k[2][BN][KPAD];
      uint16_t v[2][D][VPAD];
    } loop;
    struct {
      float o[BM][OPAD];
      float m[BM];
      float l[BM];
    } epi;
  };
};

__device__ __forceinline__ int perm_row(int a) { return (a & ~0xC) | ((a & 4) << 1) | ((a & 8) >> 1); }

template <bool O_F32>
__global__ void __launch_bounds__(256, 2)
    fwd_bf16_kernel(Prob P, const uint16_t* __restrict__ q, PassPtrs kv, const _Float16* __restrict__ kt,
                    const uint16_t* __restrict__ vt, const int4* __restrict__ tiles, const float* __restrict__ cosT,
                    const float* __restrict__ sinT, void* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- work item: XCD-aware, heavy-first
  const int r = P.r;
  const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int logical = ((kk / r) * 8 + xcd) * r + (kk % r);
  const int hr = logical % r, rest = logical / r;
  const int g = rest % P.Hkv, tix = rest / P.Hkv;
  int b, t, start, L, slot0;
  if (P.layout == 0) {
    const int nqt = (P.stok + BM - 1) / BM;
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
  const int h = g * r + hr;
  const int row0 = t * BM;
  const int my_row = row0 + wv * 32 + l32;  // this lane's query row (B/C column)

  // ---- Q~ = R(i+p-1) q in fp16, B operand chunks c = 0..7 (d = 16c + 8hf + e)
  f16x8 qf[8];
  {
    const bool valid = my_row < L;
    const uint16_t* qrow = q + b * P.qs_b + (int64_t)(start + my_row) * P.qs_t + h * P.qs_h;
    const int pos = my_row + P.p - 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = c * 16 + hf * 8;
      float x1[8], x2[8];
      if (valid) {
        unpack_bf8(*(const u32x4*)(qrow + d0), x1);
        unpack_bf8(*(const u32x4*)(qrow + d0 + 64), x2);
        const f32x4* cp = (const f32x4*)(cosT + (int64_t)pos * 64 + d0);
        const f32x4* sp = (const f32x4*)(sinT + (int64_t)pos * 64 + d0);
        f32x4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
        float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float y1 = x1[e] * cs[e] - x2[e] * sn[e];
          float y2 = x2[e] * cs[e] + x1[e] * sn[e];
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

  // ---- trunk main loop
  const int qend = min(row0 + BM, L);
  const int nkt = (qend + BN - 1) / BN;
  const _Float16* kbase = kt + ((int64_t)(b * P.Hkv + g) * P.spad + slot0) * D;
  const uint16_t* vbase = vt + (int64_t)(b * P.Hkv + g) * D * P.spad + slot0;
  const int krow = tid >> 4, kch = tid & 15;  // K tile: rows krow + 16*it, 16-byte chunk kch
  const int vrow = tid >> 3, vch = tid & 7;   // V^T tile: d rows vrow + 32*it, 8-key chunk vch
  u32x4 kreg[4], vreg[4];
  auto gload = [&](int kt_) {
    const _Float16* ks = kbase + (int64_t)kt_ * BN * D;
#pragma unroll
    for (int it = 0; it < 4; ++it) kreg[it] = *(const u32x4*)(ks + (krow + 16 * it) * D + kch * 8);
    const uint16_t* vs = vbase + kt_ * BN;
#pragma unroll
    for (int it = 0; it < 4; ++it) vreg[it] = *(const u32x4*)(vs + (int64_t)(vrow + 32 * it) * P.spad + vch * 8);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) *(u32x4*)&sm.loop.k[buf][krow + 16 * it][kch * 8] = kreg[it];
#pragma unroll
    for (int it = 0; it < 4; ++it) *(u32x4*)&sm.loop.v[buf][vrow + 32 * it][vch * 8] = vreg[it];
  };

  gload(0);
  sstore(0);
  __syncthreads();

  f32x16 oacc[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d4][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f, scale_o = 1.f;
  const int prow = perm_row(l32);
  const float sl2 = P.scale_log2;
  const int wave_row0 = row0 + wv * 32;

  // Tiles whose every key precedes every row of this wave need no mask.
  const int n_free = wave_row0 + 1 >= BN ? (wave_row0 + 1) / BN : 0;

  // One key tile: S^T = K~ Q~^T, online softmax (log2 domain), O^T += V^T P^T.
  // The running max is lazy: it only moves when a score exceeds it by more than
  // 2^8, so P <= 256 and the O rescale is skipped wave-wide otherwise (exact:
  // O and l always share the max they were accumulated with).
  auto tile = [&](const int buf, const int key0, auto masked) {
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f16x8 a = *(const f16x8*)&sm.loop.k[buf][kb * 32 + prow][c * 16 + hf * 8];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[c], sacc[kb], 0, 0, 0);
      }
    }
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + kb * 32 + (v >> 3) * 16 + hf * 8 + (v & 7);
          if (key > my_row) sacc[kb][v] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
    if (mx > m_run + 8.f) {  // only then move the running max
      const float alpha = fast_exp2(m_run - mx);
      l_run *= alpha;
      m_run = mx;
      scale_o = scale_o * alpha;
    }
    const float neg_m = -m_run;
    float lsum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = fast_exp2(__builtin_fmaf(sacc[kb][v], sl2, neg_m));
        lsum += pv;
        pb[kb * 2 + (v >> 3)][v & 7] = (__bf16)pv;
      }
    l_run += lsum;
    if (__builtin_amdgcn_ballot_w64(scale_o != 1.f)) {
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[d4][v] *= scale_o;
      scale_o = 1.f;
    }
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        const bf16x8 a = *(const bf16x8*)&sm.loop.v[buf][d4 * 32 + l32][c2 * 16 + hf * 8];
        oacc[d4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c2], oacc[d4], 0, 0, 0);
      }
  };

  for (int kt_ = 0; kt_ < nkt; ++kt_) {
    const int buf = kt_ & 1;
    if (kt_ + 1 < nkt) gload(kt_ + 1);
    if (kt_ < n_free) tile(buf, kt_ * BN, std::false_type{});
    else tile(buf, kt_ * BN, std::true_type{});
    if (kt_ + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue 1: normalised trunk partial to LDS, row-major
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv_l = 1.f / l_tot;
  {
    const int lr = wv * 32 + l32;
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = oacc[d4][v4 * 4 + e] * inv_l;
        *(f32x4*)&sm.epi.o[lr][d4 * 32 + v4 * 8 + hf * 4] = w;
      }
    if (hf == 0) {
      sm.epi.m[lr] = m_run;
      sm.epi.l[lr] = l_tot;
    }
  }
  __syncthreads();

  // ---- epilogue 2: branch partial (passes 2..p, same row) + joint-LSE merge
  const int c8 = tid & 7;
  const int dlo = c8 * 8, dhi = 64 + c8 * 8;
  for (int rp = 0; rp < BM; rp += 32) {
    const int lr = rp + (tid >> 3);
    const int i = row0 + lr;
    if (i >= L) continue;  // uniform across the row's 8 lanes
    float ot[16];
    {
      const f32x4* a = (const f32x4*)&sm.epi.o[lr][dlo];
      const f32x4* bq = (const f32x4*)&sm.epi.o[lr][dhi];
      f32x4 a0 = a[0], a1 = a[1], b0 = bq[0], b1 = bq[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) ot[e] = a0[e], ot[4 + e] = a1[e], ot[8 + e] = b0[e], ot[12 + e] = b1[e];
    }
    const float lse_t = sm.epi.m[lr] + fast_log2(sm.epi.l[lr]);  // log2 units
    float ob[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) ob[e] = 0.f;
    float mb = -INFINITY, lb = 0.f;
    if (P.p > 1) {
      float qr[16];
      {
        const uint16_t* qrow = q + b * P.qs_b + (int64_t)(start + i) * P.qs_t + h * P.qs_h;
        float x1[8], x2[8];
        unpack_bf8(*(const u32x4*)(qrow + dlo), x1);
        unpack_bf8(*(const u32x4*)(qrow + dhi), x2);
        const int pos = i + P.p - 1;
        const float* cp = cosT + (int64_t)pos * 64 + dlo;
        const float* sp = sinT + (int64_t)pos * 64 + dlo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qr[e] = x1[e] * cp[e] - x2[e] * sp[e];
          qr[8 + e] = x2[e] * cp[e] + x1[e] * sp[e];
        }
      }
      const int64_t koff = b * P.ks_b + (int64_t)(start + i) * P.ks_t + g * P.ks_h;
      for (int qq = 2; qq <= P.p; ++qq) {
        const uint16_t* krow_ = (const uint16_t*)kv.k[qq - 1] + koff;
        const uint16_t* vrow_ = (const uint16_t*)kv.v[qq - 1] + koff;
        float x1[8], x2[8], v1[8], v2[8];
        unpack_bf8(*(const u32x4*)(krow_ + dlo), x1);
        unpack_bf8(*(const u32x4*)(krow_ + dhi), x2);
        unpack_bf8(*(const u32x4*)(vrow_ + dlo), v1);
        unpack_bf8(*(const u32x4*)(vrow_ + dhi), v2);
        const int pos = i + qq - 1;
        const float* cp = cosT + (int64_t)pos * 64 + dlo;
        const float* sp = sinT + (int64_t)pos * 64 + dlo;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float k1 = x1[e] * cp[e] - x2[e] * sp[e];
          const float k2 = x2[e] * cp[e] + x1[e] * sp[e];
          part += qr[e] * k1 + qr[8 + e] * k2;
        }
        part += __shfl_xor(part, 1, 64);
        part += __shfl_xor(part, 2, 64);
        part += __shfl_xor(part, 4, 64);
        const float s2 = part * sl2;
        const float mn = fmaxf(mb, s2);
        const float al = fast_exp2(mb - mn), pe = fast_exp2(s2 - mn);
        lb = lb * al + pe;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ob[e] = ob[e] * al + pe * v1[e];
          ob[8 + e] = ob[8 + e] * al + pe * v2[e];
        }
        mb = mn;
      }
    }
    const float lse_b = P.p > 1 ? mb + fast_log2(lb) : -INFINITY;
    const float M = fmaxf(lse_t, lse_b);
    const float LSE2 = M + fast_log2(fast_exp2(lse_t - M) + fast_exp2(lse_b - M));
    const float wt = fast_exp2(lse_t - LSE2);
    const float wb = P.p > 1 ? fast_exp2(lse_b - LSE2) / lb : 0.f;
    float res[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) res[e] = wt * ot[e] + wb * ob[e];
    const int64_t oo = b * P.os_b + (int64_t)(start + i) * P.os_t + h * P.os_h;
    if (O_F32) {
      float* orow = (float*)o + oo;
      *(f32x4*)(orow + dlo) = f32x4{res[0], res[1], res[2], res[3]};
      *(f32x4*)(orow + dlo + 4) = f32x4{res[4], res[5], res[6], res[7]};
      *(f32x4*)(orow + dhi) = f32x4{res[8], res[9], res[10], res[11]};
      *(f32x4*)(orow + dhi + 4) = f32x4{res[12], res[13], res[14], res[15]};
    } else {
      uint16_t* orow = (uint16_t*)o + oo;
      *(u32x4*)(orow + dlo) = pack_bf8(res);
      *(u32x4*)(orow + dhi) = pack_bf8(res + 8);
    }
    if (c8 == 0) lse[b * P.lse_b + h * P.lse_h + start + i] = LSE2 * kLn2;
  }
}

}  // namespace fwd

void launch_fwd_bf16(const Prob& P, const uint16_t* q, const PassPtrs& kv, const _Float16* kt, const uint16_t* vt,
                     const int4* tiles, const float* cosT, const float* sinT, void* o, bool o_f32, float* lse,
                     hipStream_t st) {
  int ntiles;
  if (P.layout == 0) ntiles = P.B * ((P.stok + fwd::BM - 1) / fwd::BM);
  else ntiles = (P.stok + fwd::BM - 1) / fwd::BM + P.nseq;
  const int64_t items = (int64_t)ntiles * P.Hq;
  const int64_t unit = 8 * (int64_t)P.r;
  const int64_t grid = (items + unit - 1) / unit * unit;
  if (o_f32)
    fwd::fwd_bf16_kernel<true><<<(unsigned)grid, 256, 0, st>>>(P, q, kv, kt, vt, tiles, cosT, sinT, o, lse);
  else
    fwd::fwd_bf16_kernel<false><<<(unsigned)grid, 256, 0, st>>>(P, q, kv, kt, vt, tiles, cosT, sinT, o, lse);
}

}  // namespace ttt
