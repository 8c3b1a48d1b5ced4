// C-ABI entry points of libtttattn: argument validation, workspace plan and
// launch order.  Nothing is launched unless every check passes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/tttattn.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;
thread_local ttt_attn_trace_fn g_trace_fn = nullptr;
thread_local void* g_trace_user = nullptr;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bf16 backward: the bounds behind the fp16 dS scale (Prob::dnorm .. vmax_b,
// and with stored dS vpart / vgmax), one workspace region; key_sets = 2 for
// block drafting (context and block keys).
size_t bound_bytes(const ttt::Prob& P, int key_sets, bool ds = false) {
  return align256((size_t)P.B * P.Hq * P.spad * 4) + align256((size_t)P.B * P.Hq * (P.spad / 64) * 8) +
         align256((size_t)P.B * P.Hkv * 8) + key_sets * align256((size_t)P.B * P.Hkv * (P.spad / 32) * 4) +
         (ds ? align256((size_t)P.B * P.Hkv * (P.spad / 64) * 4) + align256((size_t)P.B * P.Hkv * 4) : 0);
}
void set_bounds(ttt::Prob& P, void* region, int key_sets, bool ds = false) {
  char* c = (char*)region;
  P.dnorm = (float*)c;
  c += align256((size_t)P.B * P.Hq * P.spad * 4);
  P.dpart = (float*)c;
  c += align256((size_t)P.B * P.Hq * (P.spad / 64) * 8);
  P.dmax = (float*)c;
  c += align256((size_t)P.B * P.Hkv * 8);
  P.vmax = (float*)c;
  c += align256((size_t)P.B * P.Hkv * (P.spad / 32) * 4);
  P.vmax_b = key_sets > 1 ? (float*)c : nullptr;
  c += (key_sets - 1) * align256((size_t)P.B * P.Hkv * (P.spad / 32) * 4);
  P.vpart = ds ? (float*)c : nullptr;
  c += align256((size_t)P.B * P.Hkv * (P.spad / 64) * 4);
  P.vgmax = ds ? (float*)c : nullptr;
}

// Largest token stride (elements) of a caller tensor: the kernels' tile loads
// reach 32 rows past a base with 32-bit byte offsets.
constexpr int64_t kMaxTokenStride = (int64_t)1 << 25;

struct Plan {
  ttt::Prob P;
  ttt::WsPlan ws;
  bool bf16;
  bool o_f32;
  bool ds;  // backward with stored dS (TTT_BWD_STORED_DS on a BSHD pass whose blocks fit the cap)
  int max_tiles_q, max_tiles_kv;
  int64_t k0s_b, k0s_t, k0s_h;  // strides of k[0] / v[0] (ring steps; = kv strides otherwise)
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The kernels address workspace slabs through buffer descriptors with 32-bit
// byte offsets: a transposed slab spans (D-1) * spad + one tile of 2-byte
// elements, and the log2 LSE staged after Delta starts B * Hq * spad floats
// past it.  Larger problems would wrap (and read zeros past the range).
int check_slab_offsets(const ttt::Prob& P) {
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)(P.D - 1) * P.spad * 2 + 1024 >= lim || (int64_t)P.B * P.Hq * P.spad * 4 >= lim)
    return fail(TTT_ERR_BAD_SHAPE,
                "%d workspace slots per head with %d batches x %d query heads: past the kernels' 32-bit workspace "
                "offsets (2 (D-1) slots and 4 B Hq slots must stay below 2^31)",
                P.spad, P.B, P.Hq);
  return 0;
}

// bf16 head_dim 32 / 64: the whole-sequence calls run the D = 128 kernels on
// zero-padded copies of the heads (defined after the D = 128 entry points).
bool padded_head(const ttt_attn_desc* d) {
  return d && d->struct_size == sizeof(ttt_attn_desc) && d->dtype == TTT_DTYPE_BF16 &&
         (d->head_dim == 32 || d->head_dim == 64);
}
size_t padded_ws_bytes(const ttt_attn_desc* d, int for_bwd);
int padded_fwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v, void* o,
               float* lse, void* ws, size_t ws_bytes, void* stream);
int padded_bwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v, const void* o,
               const float* lse, const void* dout, void* dq, void* const* dk, void* const* dv, void* ws,
               size_t ws_bytes, void* stream);

// Validates the descriptor (and the ring-step chunk, if any) and fills the
// kernel view and workspace plan.
int make_plan(const ttt_attn_desc* d, int for_bwd, Plan& pl, const ttt_attn_chunk* c = nullptr) {
  if (!d) return fail(TTT_ERR_NULL_ARG, "descriptor is NULL");
  if (d->struct_size != sizeof(ttt_attn_desc))
    return fail(TTT_ERR_ABI, "struct_size %u != %zu (ABI version %d)", d->struct_size, sizeof(ttt_attn_desc),
                TTT_ATTN_ABI_VERSION);
  if (d->layout != TTT_LAYOUT_BSHD && d->layout != TTT_LAYOUT_THD)
    return fail(TTT_ERR_BAD_SHAPE, "layout %d is neither BSHD (0) nor THD (1)", d->layout);
  if (d->dtype != TTT_DTYPE_BF16 && d->dtype != TTT_DTYPE_FP32)
    return fail(TTT_ERR_UNSUPPORTED, "dtype %d is neither BF16 (0) nor FP32 (1)", d->dtype);
  if (d->o_dtype != d->dtype && !(d->dtype == TTT_DTYPE_BF16 && d->o_dtype == TTT_DTYPE_FP32))
    return fail(TTT_ERR_UNSUPPORTED, "o_dtype %d with dtype %d: O is dtype, or FP32 with BF16 inputs", d->o_dtype,
                d->dtype);
  const int Hq = d->num_q_heads, Hkv = d->num_kv_heads, D = d->head_dim, p = d->pass_index;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(TTT_ERR_BAD_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d", Hq, Hkv);
  if (D <= 0 || (D & 1)) return fail(TTT_ERR_BAD_SHAPE, "head_dim %d must be positive and even", D);
  const bool bf16 = d->dtype == TTT_DTYPE_BF16;
  if (bf16 ? (D != 128) : (D != 32 && D != 64 && D != 128))
    return fail(TTT_ERR_UNSUPPORTED, "head_dim %d not built for %s here (fp32: 32/64/128; bf16: 128, and 32/64 "
                "through ttt_attn_fwd / ttt_attn_bwd only)", D,
                bf16 ? "bf16" : "fp32");
  if (p < 1 || p > TTT_MAX_PASSES)
    return fail(TTT_ERR_BAD_SHAPE, "pass_index %d outside 1..%d", p, TTT_MAX_PASSES);
  if (!isfinite(d->softmax_scale)) return fail(TTT_ERR_BAD_SHAPE, "softmax_scale is not finite");
  if (!isfinite(d->rope_base) || d->rope_base < 0.f || (d->rope_base > 0.f && d->rope_base <= 1.f))
    return fail(TTT_ERR_BAD_SHAPE, "rope_base %g must be 0 (no RoPE) or > 1", (double)d->rope_base);
  int B, stok, nseq;
  if (d->layout == TTT_LAYOUT_BSHD) {
    if (d->batch < 1 || d->seqlen < 0) return fail(TTT_ERR_BAD_SHAPE, "batch %d / seqlen %d", d->batch, d->seqlen);
    B = d->batch;
    stok = d->seqlen;
    nseq = B;
  } else {
    if (d->seqlen < 0 || d->num_seqs < 1)
      return fail(TTT_ERR_BAD_SHAPE, "THD needs total tokens >= 0 (got %d) and num_seqs >= 1 (got %d)", d->seqlen,
                  d->num_seqs);
    if (!d->cu_seqlens) return fail(TTT_ERR_NULL_ARG, "THD layout needs cu_seqlens");
    B = 1;
    stok = d->seqlen;
    nseq = d->num_seqs;
  }
  if ((int64_t)stok + 128 + 64 * (int64_t)nseq > (int64_t)1 << 30)
    return fail(TTT_ERR_BAD_SHAPE, "too many tokens (%d) or sequences (%d)", stok, nseq);

  ttt::Prob& P = pl.P;
  memset(&P, 0, sizeof P);
  P.layout = d->layout;
  P.B = B;
  P.stok = stok;
  // workspace slots: BSHD one per token; THD each sequence rounded up to 64
  P.spad = ((stok + 63) / 64) * 64 + 64 + (d->layout == TTT_LAYOUT_THD ? 64 * nseq : 0);
  P.nseq = nseq;
  P.cu = d->cu_seqlens;
  P.Hq = Hq;
  P.Hkv = Hkv;
  P.D = D;
  P.p = p;
  P.r = Hq / Hkv;
  P.npos = stok + p - 1;
  P.q_off = 0;
  P.kv_off = 0;
  P.kv_len = stok;
  P.branch = 1;
  if (c) {
    if (c->struct_size != sizeof(ttt_attn_chunk))
      return fail(TTT_ERR_ABI, "chunk struct_size %u != %zu", c->struct_size, sizeof(ttt_attn_chunk));
    if (d->dtype != TTT_DTYPE_BF16) return fail(TTT_ERR_UNSUPPORTED, "ring steps are built for bf16");
    if (c->q_offset < 0 || c->kv_offset < 0 || c->kv_len < 0)
      return fail(TTT_ERR_BAD_SHAPE, "q_offset %lld, kv_offset %lld and kv_len %lld must be >= 0",
                  (long long)c->q_offset, (long long)c->kv_offset, (long long)c->kv_len);
    P.branch = c->with_branch != 0;
    if (d->layout == TTT_LAYOUT_BSHD) {
      if (c->q_offsets || c->kv_offsets || c->kv_cu_seqlens || c->max_position)
        return fail(TTT_ERR_BAD_SHAPE, "BSHD ring steps take q_offset / kv_offset; the THD fields must be NULL / 0");
      if (c->q_offset + stok + p > ((int64_t)1 << 30) || c->kv_offset + c->kv_len > ((int64_t)1 << 30))
        return fail(TTT_ERR_BAD_SHAPE, "positions past 2^30");
      P.q_off = (int)c->q_offset;
      P.kv_off = (int)c->kv_offset;
      P.kv_len = (int)c->kv_len;
      const int rows = stok > P.kv_len ? stok : P.kv_len;
      P.spad = ((rows + 63) / 64) * 64 + 64;
      const int64_t qend = c->q_offset + stok + p - 1, kend = c->kv_offset + c->kv_len;
      P.npos = (int)(qend > kend ? qend : kend);
    } else {
      if (!c->q_offsets || !c->kv_offsets || !c->kv_cu_seqlens)
        return fail(TTT_ERR_NULL_ARG, "THD ring steps need q_offsets, kv_offsets and kv_cu_seqlens");
      if (c->q_offset != 0 || c->kv_offset != 0)
        return fail(TTT_ERR_BAD_SHAPE, "THD ring steps take per-sequence offsets: q_offset and kv_offset must be 0");
      if (c->max_position < 1 || c->max_position > ((int64_t)1 << 30))
        return fail(TTT_ERR_BAD_SHAPE, "max_position %lld outside 1..2^30", (long long)c->max_position);
      if ((int64_t)stok + c->kv_len + 128 + 64 * (int64_t)nseq > (int64_t)1 << 30)
        return fail(TTT_ERR_BAD_SHAPE, "too many query (%d) and key (%lld) rows", stok, (long long)c->kv_len);
      P.kv_len = P.kv_tok = (int)c->kv_len;
      P.kv_cu = c->kv_cu_seqlens;
      P.seg_qoff = c->q_offsets;
      P.seg_kvoff = c->kv_offsets;
      // a sequence's query and key rows share its slots: the longer of the two, rounded up to 64
      P.spad = ((stok + P.kv_len + 63) / 64) * 64 + 64 + 64 * nseq;
      P.npos = (int)c->max_position;
    }
  }
  if (int e = check_slab_offsets(P)) return e;
  if (d->window < 0) return fail(TTT_ERR_BAD_SHAPE, "window %d is negative", d->window);
  if (d->window > 0 && !bf16) return fail(TTT_ERR_UNSUPPORTED, "a sliding window is built for bf16 only");
  P.win = d->window;
  P.scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)D);
  P.scale_log2 = P.scale * ttt::kLog2e;
  const bool thd = d->layout == TTT_LAYOUT_THD;
  auto strides = [&](const int64_t* s, int H, int64_t* out, const char* name, int elem_align) -> int {
    if (s[0] == 0 && s[1] == 0 && s[2] == 0) {
      out[0] = thd ? 0 : (int64_t)stok * H * D;
      out[1] = (int64_t)H * D;
      out[2] = D;
      return 0;
    }
    for (int i = 0; i < 3; ++i) {
      if (s[i] < 0) return fail(TTT_ERR_BAD_SHAPE, "%s stride[%d] = %lld is negative", name, i, (long long)s[i]);
      if (s[i] % elem_align) return fail(TTT_ERR_MISALIGNED, "%s stride[%d] = %lld not a multiple of %d elements",
                                         name, i, (long long)s[i], elem_align);
    }
    if (s[1] > kMaxTokenStride)  // tile loads address 32 rows with 32-bit byte offsets
      return fail(TTT_ERR_BAD_SHAPE, "%s token stride %lld exceeds %lld elements", name, (long long)s[1],
                  (long long)kMaxTokenStride);
    out[0] = thd ? 0 : s[0];
    out[1] = s[1];
    out[2] = s[2];
    return 0;
  };
  int64_t tmp[3];
  const int ea = bf16 ? 8 : 4;
  if (int e = strides(d->q_stride, Hq, tmp, "q", ea)) return e;
  P.qs_b = tmp[0], P.qs_t = tmp[1], P.qs_h = tmp[2];
  if (int e = strides(d->kv_stride, Hkv, tmp, "kv", ea)) return e;
  P.ks_b = tmp[0], P.ks_t = tmp[1], P.ks_h = tmp[2];
  pl.k0s_b = P.ks_b, pl.k0s_t = P.ks_t, pl.k0s_h = P.ks_h;
  if (c) {
    const int64_t* s0 = c->kv0_stride;
    if (s0[0] == 0 && s0[1] == 0 && s0[2] == 0) {
      pl.k0s_b = thd ? 0 : (int64_t)P.kv_len * Hkv * D, pl.k0s_t = (int64_t)Hkv * D, pl.k0s_h = D;
    } else {
      if (int e = strides(s0, Hkv, tmp, "kv0", ea)) return e;
      pl.k0s_b = tmp[0], pl.k0s_t = tmp[1], pl.k0s_h = tmp[2];
    }
  }
  // the kernels read the trunk (pass-1) V with the P.cs_* strides
  P.cs_b = pl.k0s_b, P.cs_t = pl.k0s_t, P.cs_h = pl.k0s_h;
  const bool o_f32 = d->o_dtype == TTT_DTYPE_FP32;
  if (int e = strides(d->o_stride, Hq, tmp, "o", (o_f32 && bf16) ? 8 : ea)) return e;
  P.os_b = tmp[0], P.os_t = tmp[1], P.os_h = tmp[2];
  if (thd) {
    P.lse_b = 0;
    P.lse_h = stok;
  } else {
    P.lse_b = (int64_t)Hq * stok;
    P.lse_h = stok;
  }
  pl.bf16 = bf16;
  pl.o_f32 = o_f32;
  // Stored dS (asked for): ttt_attn_bwd of a bf16 BSHD pass without a window,
  // when its causal 32x32 blocks (2 KB each per head) fit the cap.
  if (d->bwd_mode != TTT_BWD_RECOMPUTE && d->bwd_mode != TTT_BWD_STORED_DS)
    return fail(TTT_ERR_BAD_SHAPE, "bwd_mode %d is neither RECOMPUTE (0) nor STORED_DS (1)", d->bwd_mode);
  pl.ds = false;
  if (for_bwd && bf16 && !thd && !c && d->window == 0 && d->bwd_mode == TTT_BWD_STORED_DS) {
    const int64_t n = (stok + 31) / 32;
    const int64_t tri = n * (n + 1) / 2;
    if ((double)B * Hq * tri * 2048.0 <= (double)TTT_ATTN_STORED_DS_MAX_BYTES) {
      pl.ds = true;
      P.ds_tri = tri;
    }
  }

  // workspace plan
  ttt::WsPlan& w = pl.ws;
  memset(&w, 0, sizeof w);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  const size_t nkv = (size_t)B * Hkv * P.spad * D, nq = (size_t)B * Hq * P.spad * D;
  pl.max_tiles_q = thd ? (stok + ttt::kFwdMinRows - 1) / ttt::kFwdMinRows + nseq + 1 : 0;
  pl.max_tiles_kv = thd ? (P.kv_len + ttt::kBwdBKV - 1) / ttt::kBwdBKV + nseq + 1 : 0;  // kv_len = stok unless a THD ring step
  w.table = take((size_t)2 * P.npos * (D / 2) * sizeof(float));
  if (thd) w.slots = take((size_t)(nseq + 1) * sizeof(int));
  if (bf16) {
    if (thd) w.tiles_q = take((size_t)(pl.max_tiles_q + 1) * 16);
    w.kt = take(nkv * 2);
    if (!for_bwd) {
      w.vt = take(nkv * 2);
    } else {
      if (thd) w.tiles_kv = take((size_t)(pl.max_tiles_kv + 1) * 16);
      w.ktt = take(nkv * 2);
      w.qt = take(nq * 2);
      w.delta = take((size_t)2 * B * Hq * P.spad * 4);  // Delta, then the LSE in log2 units
      w.bnd = take(bound_bytes(P, 1, pl.ds));
      if (pl.ds) w.ds = take((size_t)B * Hq * P.ds_tri * 2048);
    }
  } else {
    w.kt = take(nkv * 4);
    if (for_bwd) {
      w.qt = take(nq * 4);
      w.delta = take((size_t)B * Hq * P.spad * 4);
    }
  }
  w.total = off;
  return TTT_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(TTT_ERR_NULL_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(TTT_ERR_MISALIGNED, "%s (%p) is not 16-byte aligned", name, p);
  return 0;
}

int check_ws(const Plan& pl, const void* ws, size_t ws_bytes) {
  if (pl.ws.total == 0) return 0;
  if (!ws) return fail(TTT_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", pl.ws.total);
  if ((uintptr_t)ws & 255u) return fail(TTT_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);
  if (ws_bytes < pl.ws.total)
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, pl.ws.total);
  return 0;
}

int check_cu_array(const int32_t* dev, int nseq, int64_t total, const char* name, hipStream_t st) {
  std::vector<int32_t> cu(nseq + 1);
  hipError_t e = hipMemcpyAsync(cu.data(), dev, cu.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "reading %s: %s", name, hipGetErrorString(e));
  if (cu[0] != 0) return fail(TTT_ERR_BAD_SHAPE, "%s[0] = %d, expected 0", name, cu[0]);
  for (int s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s]) return fail(TTT_ERR_BAD_SHAPE, "%s decreases at %d (%d > %d)", name, s, cu[s], cu[s + 1]);
  if (cu[nseq] != total)
    return fail(TTT_ERR_BAD_SHAPE, "%s[%d] = %d, expected %lld rows", name, nseq, cu[nseq], (long long)total);
  return 0;
}

// With check_cu_seqlens (THD): cu_seqlens, and a THD ring step's kv_cu_seqlens.
int check_cu(const ttt_attn_desc* d, hipStream_t st, const ttt_attn_chunk* c = nullptr) {
  if (d->layout != TTT_LAYOUT_THD || !d->check_cu_seqlens) return 0;
  if (int e = check_cu_array(d->cu_seqlens, d->num_seqs, d->seqlen, "cu_seqlens", st)) return e;
  if (c) return check_cu_array(c->kv_cu_seqlens, d->num_seqs, c->kv_len, "kv_cu_seqlens", st);
  return 0;
}

// With check_cu_seqlens (THD block drafting): cu_seqlens in whole blocks, and
// the contexts' ctx_cu_seqlens.
int check_block_cu(const ttt_attn_desc* d, const ttt_attn_block* bk, hipStream_t st) {
  if (d->layout != TTT_LAYOUT_THD || !d->check_cu_seqlens) return 0;
  if (int e = check_cu_array(d->cu_seqlens, d->num_seqs, d->seqlen, "cu_seqlens", st)) return e;
  if (int e = check_cu_array(bk->ctx_cu_seqlens, d->num_seqs, bk->ctx_len, "ctx_cu_seqlens", st)) return e;
  std::vector<int32_t> cu(d->num_seqs + 1);
  hipError_t e = hipMemcpyAsync(cu.data(), d->cu_seqlens, cu.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "reading cu_seqlens: %s", hipGetErrorString(e));
  for (int s = 0; s <= d->num_seqs; ++s)
    if (cu[s] % bk->block_size)
      return fail(TTT_ERR_BAD_SHAPE, "cu_seqlens[%d] = %d: every sequence must hold whole blocks of %d", s, cu[s],
                  bk->block_size);
  return 0;
}

int hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return 0;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

}  // namespace

namespace ttt {
void trace(const char* name, int phase, hipStream_t st) {
  if (g_trace_fn) g_trace_fn(g_trace_user, name, phase, (void*)st);
}
}  // namespace ttt

// Runs one launcher between the two trace callbacks.
#define TTT_TRACED(name, call) TTT_TRACED_ON(name, st, call)
#define TTT_TRACED_ON(name, stream_, call) \
  do {                                      \
    ttt::trace(name, 0, stream_);           \
    call;                                   \
    ttt::trace(name, 1, stream_);           \
  } while (0)

namespace {
// Work on the caller's second stream (the descriptor's aux_stream), ordered
// against the call's stream with events: mark(s) records an event at the
// current end of stream s, wait(w, e) makes later work on stream w wait for
// it.  The events are released once they complete.  If an event step fails,
// the side stream is drained from the host so that the ordering still holds.
struct Side {
  hipStream_t side = nullptr;
  hipEvent_t ev[4] = {};
  int nev = 0;
  bool begin(hipStream_t st, hipStream_t aux) {  // the side stream starts after the work on st so far
    if (!aux || aux == st) return false;
    side = aux;
    if (!wait(side, mark(st))) {
      side = nullptr;
      return false;
    }
    return true;
  }
  hipEvent_t mark(hipStream_t s) {
    hipEvent_t e = nullptr;
    if (nev == 4 || hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
    ev[nev++] = e;
    if (hipEventRecord(e, s) != hipSuccess) return nullptr;
    return e;
  }
  bool wait(hipStream_t waiter, hipEvent_t e) {
    if (e && hipStreamWaitEvent(waiter, e, 0) == hipSuccess) return true;
    (void)hipGetLastError();
    if (side) (void)hipStreamSynchronize(side);
    return false;
  }
  ~Side() {
    for (int i = 0; i < nev; ++i) (void)hipEventDestroy(ev[i]);
  }
};
}  // namespace

extern "C" {

void ttt_attn_set_trace_hook(ttt_attn_trace_fn fn, void* user) {
  g_trace_fn = fn;
  g_trace_user = user;
}

int ttt_attn_abi_version(void) { return TTT_ATTN_ABI_VERSION; }

const char* ttt_attn_status_string(int status) {
  switch (status) {
    case TTT_OK: return "ok";
    case TTT_ERR_NULL_ARG: return "null argument";
    case TTT_ERR_BAD_SHAPE: return "bad shape";
    case TTT_ERR_UNSUPPORTED: return "unsupported configuration";
    case TTT_ERR_MISALIGNED: return "misaligned pointer or stride";
    case TTT_ERR_WORKSPACE: return "workspace missing or too small";
    case TTT_ERR_HIP: return "HIP runtime error";
    case TTT_ERR_ABI: return "descriptor ABI mismatch";
    default: return "unknown status";
  }
}

const char* ttt_attn_last_error(void) { return g_last_error.c_str(); }

size_t ttt_attn_workspace_bytes(const ttt_attn_desc* d, int for_bwd) {
  if (padded_head(d)) return padded_ws_bytes(d, for_bwd);
  Plan pl;
  if (make_plan(d, for_bwd, pl) != TTT_OK) return 0;
  return pl.ws.total;
}

}  // extern "C"

namespace {
// Forward of a whole sequence (c = NULL) or of one ring step.
int fwd_impl(const ttt_attn_desc* d, const ttt_attn_chunk* c, const void* q, const void* const* k,
             const void* const* v, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan pl;
  if (int e = make_plan(d, 0, pl, c)) return e;
  ttt::Prob& P = pl.P;
  if (P.stok == 0) return TTT_OK;  // nothing to compute; pointers of empty tensors may be NULL
  if (!k || !v) return fail(TTT_ERR_NULL_ARG, "k or v pointer array is NULL");
  if (int e = check_ptr(q, "q")) return e;
  if (int e = check_ptr(o, "o")) return e;
  if (!lse) return fail(TTT_ERR_NULL_ARG, "lse is NULL");
  if ((uintptr_t)lse & 3u) return fail(TTT_ERR_MISALIGNED, "lse is not 4-byte aligned");
  ttt::PassPtrs kv;
  memset(&kv, 0, sizeof kv);
  const int nptr = P.branch ? P.p : 1;  // a ring step without the branch reads pass 1 only
  for (int i = 0; i < nptr; ++i) {
    // an empty pass-1 key block (kv_len = 0) is never read: its pointers may be NULL
    if (i == 0 && P.kv_len == 0 && !k[0] && !v[0]) continue;
    char nm[16];
    snprintf(nm, sizeof nm, "k[%d]", i);
    if (int e = check_ptr(k[i], nm)) return e;
    snprintf(nm, sizeof nm, "v[%d]", i);
    if (int e = check_ptr(v[i], nm)) return e;
    kv.k[i] = k[i];
    kv.v[i] = v[i];
  }
  if (int e = check_ws(pl, ws, ws_bytes)) return e;
  hipStream_t st = (hipStream_t)stream;
  if (int e = check_cu(d, st, c)) return e;
  (void)hipGetLastError();

  float* cosT = at<float>(ws, pl.ws.table);
  float* sinT = cosT + (size_t)P.npos * (P.D / 2);
  const bool thd = P.layout == TTT_LAYOUT_THD;
  int* slots = thd ? at<int>(ws, pl.ws.slots) : nullptr;
  P.slot_base = slots;
  TTT_TRACED("rope_table", ttt::launch_rope_table(P, cosT, sinT, (double)d->rope_base, st));
  if (!pl.bf16) {
    if (thd) TTT_TRACED("tile_sched", ttt::launch_tile_sched(P, 64, 1, nullptr, 0, slots, st));
    float* kt = at<float>(ws, pl.ws.kt);
    TTT_TRACED("prep_k_f32",
               ttt::launch_prep_rot_f32(P, (const float*)k[0], P.ks_b, P.ks_t, P.ks_h, P.Hkv, 0, cosT, sinT, kt, st));
    TTT_TRACED("fwd_f32", ttt::launch_fwd_f32(P, (const float*)q, kv, kt, cosT, sinT, (float*)o, lse, st));
  } else {
    const int4* tiles = nullptr;
    if (thd) {
      int4* t = at<int4>(ws, pl.ws.tiles_q);
      TTT_TRACED("tile_sched",
                 ttt::launch_tile_sched(P, ttt::fwd_tile_rows(P.r), 1, t, pl.max_tiles_q, slots, st));
      tiles = t;
    }
    _Float16* kt = at<_Float16>(ws, pl.ws.kt);
    _Float16* vt = at<_Float16>(ws, pl.ws.vt);
    // the pass-1 keys: kv_len rows (= the sequence for whole-sequence calls) at positions kv_off + j;
    // rotated K~ rows and V^T in one launch
    ttt::Prob Pk = P;
    if (P.layout == TTT_LAYOUT_BSHD) Pk.stok = P.kv_len;
    ttt::PrepJobs J;
    memset(&J, 0, sizeof J);
    J.n = 2;
    J.j[0] = {(const uint16_t*)k[0], pl.k0s_b, pl.k0s_t, pl.k0s_h, P.Hkv, P.kv_off, 1, 0, kt, nullptr, 0, nullptr, 0};
    J.j[1] = {(const uint16_t*)v[0], pl.k0s_b, pl.k0s_t, pl.k0s_h, P.Hkv, 0, 0, 0, nullptr, (uint16_t*)vt, 0,
              nullptr, 0};  // V^T in fp16: the PV product's operand
    if (P.kv_cu)  // THD ring step: the packed key rows of each sequence, at its own key offset
      for (int j = 0; j < 2; ++j) J.j[j].cu = P.kv_cu, J.j[j].ntok = P.kv_tok, J.j[j].seg_pos = j ? nullptr : P.seg_kvoff;
    TTT_TRACED("prep_kv", ttt::launch_prep_bf16(Pk, J, cosT, sinT, st));
    TTT_TRACED("trunk_fwd",
               ttt::launch_fwd_bf16(P, (const uint16_t*)q, kv, kt, vt, tiles, cosT, sinT, o, pl.o_f32, lse, st));
  }
  return hip_check("ttt_attn_fwd launch");
}
}  // namespace

extern "C" {

int ttt_attn_fwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v, void* o,
                 float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (padded_head(d)) return padded_fwd(d, q, k, v, o, lse, ws, ws_bytes, stream);
  return fwd_impl(d, nullptr, q, k, v, o, lse, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {
// Workspace of the allocation-free forward: a static device array, one copy
// per GPU, held until the process ends.  In host code `scratch` names a host
// stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device (with that device
// current) and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[TTT_ATTN_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TTT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TTT_ERR_HIP, "device %d is past the %d tracked", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(TTT_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}
}  // namespace

extern "C" {

int ttt_attn_fwd_noalloc(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v,
                         void* o, float* lse, void* stream) {
  g_last_error.clear();
  Plan pl;
  if (int e = make_plan(d, 0, pl)) return e;
  if (d->layout == TTT_LAYOUT_THD && d->check_cu_seqlens)
    return fail(TTT_ERR_UNSUPPORTED, "check_cu_seqlens copies to the host and synchronises: not in the "
                                     "allocation-free forward");
  if (pl.ws.total > (size_t)TTT_ATTN_NOALLOC_SCRATCH_BYTES)
    return fail(TTT_ERR_WORKSPACE, "the call needs %zu bytes of workspace; the allocation-free forward's static "
                                   "scratch holds %zu", pl.ws.total, (size_t)TTT_ATTN_NOALLOC_SCRATCH_BYTES);
  if (pl.P.stok == 0) return TTT_OK;
  void* ws = nullptr;
  if (int e = scratch_address(&ws)) return e;
  return fwd_impl(d, nullptr, q, k, v, o, lse, ws, TTT_ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

size_t ttt_attn_chunk_workspace_bytes(const ttt_attn_desc* d, const ttt_attn_chunk* c) {
  g_last_error.clear();
  if (!c) {
    fail(TTT_ERR_NULL_ARG, "chunk is NULL");
    return 0;
  }
  Plan pl;
  if (make_plan(d, 0, pl, c) != TTT_OK) return 0;
  return pl.ws.total;
}

int ttt_attn_fwd_chunk(const ttt_attn_desc* d, const ttt_attn_chunk* c, const void* q, const void* const* k,
                       const void* const* v, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!c) {
    g_last_error.clear();
    return fail(TTT_ERR_NULL_ARG, "chunk is NULL");
  }
  return fwd_impl(d, c, q, k, v, o, lse, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {
// Block-draft plan: the descriptor's rows are the block slots; the context
// and the block keys each get their own staging slabs.
struct BlockPlan {
  Plan pl;
  int64_t cs_b, cs_t, cs_h;  // context K/V strides
  // forward: context K~ / V^T, block K~ / V^T; backward: context K~ / K~^T,
  // block K~ / K~^T (in the same four slots), Q~ rows and Delta
  size_t ctx_kt, ctx_vt, blk_kt, blk_vt, qt, delta, total;
  // THD: workspace slots and the tile lists of the query rows, the context
  // keys and the block keys
  size_t slots, tiles_q, tiles_kv, tiles_kb;
  int max_tiles_q, max_tiles_kv, max_tiles_kb;
};

int make_block_plan(const ttt_attn_desc* d, const ttt_attn_block* bk, BlockPlan& bp, bool for_bwd = false) {
  if (!bk) return fail(TTT_ERR_NULL_ARG, "block descriptor is NULL");
  if (bk->struct_size != sizeof(ttt_attn_block))
    return fail(TTT_ERR_ABI, "block struct_size %u != %zu", bk->struct_size, sizeof(ttt_attn_block));
  Plan& pl = bp.pl;
  if (int e = make_plan(d, 0, pl)) return e;
  ttt::Prob& P = pl.P;
  const bool thd = d->layout == TTT_LAYOUT_THD;
  if (thd && !bk->ctx_cu_seqlens)
    return fail(TTT_ERR_NULL_ARG, "THD block drafting needs ctx_cu_seqlens (the contexts' cu_seqlens)");
  if (!thd && bk->ctx_cu_seqlens)
    return fail(TTT_ERR_BAD_SHAPE, "ctx_cu_seqlens belongs to THD block drafting; BSHD takes it NULL");
  if (!pl.bf16) return fail(TTT_ERR_UNSUPPORTED, "block drafting is built for bf16");
  if (d->pass_index != 1) return fail(TTT_ERR_BAD_SHAPE, "block drafting has no passes: pass_index must be 1");
  if (d->window != 0) return fail(TTT_ERR_UNSUPPORTED, "block drafting takes no sliding window");
  const int bs = bk->block_size;
  if (bs < 1 || bs > 32 || (bs & (bs - 1)))
    return fail(TTT_ERR_UNSUPPORTED, "block_size %d: 1, 2, 4, 8, 16 or 32", bs);
  if (P.stok % bs) return fail(TTT_ERR_BAD_SHAPE, "seqlen %d is not a whole number of blocks of %d", P.stok, bs);
  if (bk->ctx_len < 0 || bk->ctx_len + bs > ((int64_t)1 << 30))
    return fail(TTT_ERR_BAD_SHAPE, "ctx_len %lld outside [0, 2^30 - block_size]", (long long)bk->ctx_len);
  const int ctx = (int)bk->ctx_len;
  P.kv_len = ctx;
  P.branch = 0;
  P.bs_log2 = __builtin_ctz((unsigned)bs);
  P.nblk = P.stok / bs;  // THD: blocks of every sequence, in packed order
  P.anchors = bk->anchors;
  P.cs_b = 0, P.cs_t = 0, P.cs_h = 0;
  P.npos = ctx + bs;                                   // slot positions a + t <= ctx + bs - 1
  // context and block slabs share one slot count: the kernel's V^T row
  // offsets are computed once for both
  if (thd) {
    // a sequence's block rows and context share its slots (the longer of the two, rounded up to 64)
    if ((int64_t)P.stok + ctx + 128 + 64 * (int64_t)P.nseq > (int64_t)1 << 30)
      return fail(TTT_ERR_BAD_SHAPE, "too many block (%d) and context (%d) rows", P.stok, ctx);
    P.kv_cu = bk->ctx_cu_seqlens;
    P.kv_tok = ctx;
    P.spad = ((P.stok + ctx + 63) / 64) * 64 + 64 + 64 * P.nseq;
  } else {
    const int rows_max = ctx > P.stok ? ctx : P.stok;
    P.spad = ((rows_max + 63) / 64) * 64 + 64;
  }
  P.spad_b = P.spad;
  if (int e = check_slab_offsets(P)) return e;
  const int64_t* s0 = bk->ctx_stride;
  const int D = P.D, Hkv = P.Hkv;
  if (s0[0] == 0 && s0[1] == 0 && s0[2] == 0) {
    bp.cs_b = (int64_t)ctx * Hkv * D, bp.cs_t = (int64_t)Hkv * D, bp.cs_h = D;
  } else {
    for (int i = 0; i < 3; ++i) {
      if (s0[i] < 0) return fail(TTT_ERR_BAD_SHAPE, "ctx stride[%d] = %lld is negative", i, (long long)s0[i]);
      if (s0[i] % 8) return fail(TTT_ERR_MISALIGNED, "ctx stride[%d] = %lld not a multiple of 8 elements", i,
                                 (long long)s0[i]);
    }
    if (s0[1] > kMaxTokenStride)
      return fail(TTT_ERR_BAD_SHAPE, "ctx token stride %lld exceeds %lld elements", (long long)s0[1],
                  (long long)kMaxTokenStride);
    bp.cs_b = s0[0], bp.cs_t = s0[1], bp.cs_h = s0[2];
  }
  P.cs_b = bp.cs_b, P.cs_t = bp.cs_t, P.cs_h = bp.cs_h;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at_ = off;
    off = align256(off + bytes);
    return at_;
  };
  memset(&pl.ws, 0, sizeof pl.ws);
  pl.ws.table = take((size_t)2 * P.npos * (D / 2) * sizeof(float));
  bp.slots = bp.tiles_q = bp.tiles_kv = bp.tiles_kb = 0;
  bp.max_tiles_q = bp.max_tiles_kv = bp.max_tiles_kb = 0;
  if (thd) {
    const int nseq = P.nseq;
    bp.max_tiles_q = (P.stok + ttt::kFwdMinRows - 1) / ttt::kFwdMinRows + nseq + 1;
    bp.max_tiles_kv = (ctx + ttt::kBwdBKV - 1) / ttt::kBwdBKV + nseq + 1;
    bp.max_tiles_kb = (P.stok + ttt::kBwdBKV - 1) / ttt::kBwdBKV + nseq + 1;
    bp.slots = take((size_t)(nseq + 1) * sizeof(int));
    bp.tiles_q = take((size_t)(bp.max_tiles_q + 1) * 16);
    if (for_bwd) {
      bp.tiles_kv = take((size_t)(bp.max_tiles_kv + 1) * 16);
      bp.tiles_kb = take((size_t)(bp.max_tiles_kb + 1) * 16);
    }
  }
  const size_t nc = (size_t)P.B * Hkv * P.spad * D, nb = (size_t)P.B * Hkv * P.spad_b * D;
  bp.ctx_kt = take(nc * 2);
  bp.ctx_vt = take(nc * 2);
  bp.blk_kt = take(nb * 2);
  bp.blk_vt = take(nb * 2);
  bp.qt = bp.delta = 0;
  if (for_bwd) {
    bp.qt = take((size_t)P.B * P.Hq * P.spad * D * 2);
    // Delta, the LSE in log2 units, then the row lims
    bp.delta = take((size_t)2 * P.B * P.Hq * P.spad * 4 + (size_t)P.B * P.spad * 4);
    pl.ws.bnd = take(bound_bytes(P, 2));
  }
  bp.total = off;
  pl.ws.total = off;
  return TTT_OK;
}
}  // namespace

extern "C" {

size_t ttt_attn_block_workspace_bytes(const ttt_attn_desc* d, const ttt_attn_block* bk, int for_bwd) {
  g_last_error.clear();
  BlockPlan bp;
  if (make_block_plan(d, bk, bp, for_bwd != 0) != TTT_OK) return 0;
  return bp.total;
}

int ttt_attn_block_bwd(const ttt_attn_desc* d, const ttt_attn_block* bk, const void* q, const void* k_ctx,
                       const void* v_ctx, const void* k_blk, const void* v_blk, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk_ctx, void* dv_ctx, void* dk_blk, void* dv_blk, void* ws,
                       size_t ws_bytes, void* stream) {
  g_last_error.clear();
  BlockPlan bp;
  if (int e = make_block_plan(d, bk, bp, true)) return e;
  Plan& pl = bp.pl;
  ttt::Prob& P = pl.P;
  if (P.stok == 0) return TTT_OK;
  if (!bk->anchors) return fail(TTT_ERR_NULL_ARG, "anchors is NULL");
  if ((uintptr_t)bk->anchors & 3u) return fail(TTT_ERR_MISALIGNED, "anchors is not 4-byte aligned");
  const void* need[] = {q, k_blk, v_blk, o, dout, dq, dk_blk, dv_blk};
  const char* names[] = {"q", "k_blk", "v_blk", "o", "dout", "dq", "dk_blk", "dv_blk"};
  for (int i = 0; i < 8; ++i)
    if (int e = check_ptr(need[i], names[i])) return e;
  if (P.kv_len > 0) {  // an empty context is never read or written: its pointers may be NULL
    const void* cneed[] = {k_ctx, v_ctx, dk_ctx, dv_ctx};
    const char* cnames[] = {"k_ctx", "v_ctx", "dk_ctx", "dv_ctx"};
    for (int i = 0; i < 4; ++i)
      if (int e = check_ptr(cneed[i], cnames[i])) return e;
  }
  if (!lse) return fail(TTT_ERR_NULL_ARG, "lse is NULL");
  if ((uintptr_t)lse & 3u) return fail(TTT_ERR_MISALIGNED, "lse is not 4-byte aligned");
  if (int e = check_ws(pl, ws, ws_bytes)) return e;
  hipStream_t st = (hipStream_t)stream;
  if (int e = check_block_cu(d, bk, st)) return e;
  (void)hipGetLastError();
  float* cosT = at<float>(ws, pl.ws.table);
  float* sinT = cosT + (size_t)P.npos * (P.D / 2);
  _Float16* ckt = at<_Float16>(ws, bp.ctx_kt);
  _Float16* cktt = at<_Float16>(ws, bp.ctx_vt);
  _Float16* bkt = at<_Float16>(ws, bp.blk_kt);
  _Float16* bktt = at<_Float16>(ws, bp.blk_vt);
  _Float16* qt = at<_Float16>(ws, bp.qt);
  float* delta = at<float>(ws, bp.delta);
  const bool thd = P.layout == TTT_LAYOUT_THD;
  int* slots = thd ? at<int>(ws, bp.slots) : nullptr;
  P.slot_base = slots;
  set_bounds(P, at<char>(ws, pl.ws.bnd), 2);
  TTT_TRACED("rope_table", ttt::launch_rope_table(P, cosT, sinT, (double)d->rope_base, st));
  const int4 *tq = nullptr, *tkv = nullptr, *tkb = nullptr;
  if (thd) {  // THD: slots, then the tiles of the query rows, the context keys and the block keys
    int4* a = at<int4>(ws, bp.tiles_q);
    int4* c = at<int4>(ws, bp.tiles_kv);
    int4* k = at<int4>(ws, bp.tiles_kb);
    TTT_TRACED("tile_sched", ttt::launch_tile_sched(P, ttt::dq_tile_rows(P.r), 1, a, bp.max_tiles_q, slots, st));
    ttt::Prob Pkv = P;
    Pkv.cu = P.kv_cu, Pkv.stok = P.kv_tok;
    TTT_TRACED("tile_sched", ttt::launch_tile_sched(Pkv, ttt::kBwdBKV, 0, c, bp.max_tiles_kv, nullptr, st));
    TTT_TRACED("tile_sched", ttt::launch_tile_sched(P, ttt::kBwdBKV, 0, k, bp.max_tiles_kb, nullptr, st));
    tq = a, tkv = c, tkb = k;
  }
  TTT_TRACED("bwd_delta", ttt::launch_delta(P, o, pl.o_f32, dout, false, lse, delta, nullptr, st));
  TTT_TRACED("bwd_dmax", ttt::launch_dmax(P, st));
  ttt::PrepJobs J;
  memset(&J, 0, sizeof J);
  J.n = 1;
  if (P.kv_len > 0) {  // context: K~ rows and K~^T
    ttt::Prob Pc = P;
    Pc.stok = P.kv_len;
    J.j[0] = {(const uint16_t*)k_ctx, bp.cs_b, bp.cs_t, bp.cs_h, P.Hkv, 0, 1, 0, ckt, (uint16_t*)cktt, 0, nullptr, 0};
    if (thd) J.j[0].cu = P.kv_cu, J.j[0].ntok = P.kv_tok;
    TTT_TRACED("prep_ctx_bwd", ttt::launch_prep_bf16(Pc, J, cosT, sinT, st));
  }
  // block keys (K~ rows, K~^T) and queries (Q~ rows) at their slot positions
  J.n = 2;
  J.j[0] = {(const uint16_t*)k_blk, P.ks_b, P.ks_t, P.ks_h, P.Hkv, 0, 1, 0, bkt, (uint16_t*)bktt, 1, nullptr, 0};
  int* lims = (int*)(delta + (size_t)2 * P.B * P.Hq * P.spad);  // per-slot visible context lengths
  J.j[1] = {(const uint16_t*)q, P.qs_b, P.qs_t, P.qs_h, P.Hq, 0, 1, 0, qt, nullptr, 1, lims, 0};
  J.heads_fast = 1;  // mostly row-major outputs (Q~ rows)
  TTT_TRACED("prep_blkq", ttt::launch_prep_bf16(P, J, cosT, sinT, st));
  if (P.kv_len > 0) {
    ttt::Prob Pc = P;  // the context keys' V / dK / dV strides
    Pc.ks_b = bp.cs_b, Pc.ks_t = bp.cs_t, Pc.ks_h = bp.cs_h;
    TTT_TRACED("block_dkdv_ctx", ttt::launch_block_dkdv_bf16(Pc, true, (const uint16_t*)v_ctx, lse,
                                                             (const uint16_t*)dout, ckt, qt, delta, tkv, cosT, sinT,
                                                             dk_ctx, dv_ctx, st));
  }
  TTT_TRACED("block_dkdv_blk", ttt::launch_block_dkdv_bf16(P, false, (const uint16_t*)v_blk, lse,
                                                           (const uint16_t*)dout, bkt, qt, delta, tkb, cosT, sinT,
                                                           dk_blk, dv_blk, st));
  TTT_TRACED("block_dq", ttt::launch_block_dq_bf16(P, (const uint16_t*)v_ctx, (const uint16_t*)v_blk, lse,
                                                   (const uint16_t*)dout, ckt, cktt, bkt, bktt, qt, delta, tq, cosT,
                                                   sinT, (uint16_t*)dq, st));
  return hip_check("ttt_attn_block_bwd launch");
}

int ttt_attn_block_fwd(const ttt_attn_desc* d, const ttt_attn_block* bk, const void* q, const void* k_ctx,
                       const void* v_ctx, const void* k_blk, const void* v_blk, void* o, float* lse, void* ws,
                       size_t ws_bytes, void* stream) {
  g_last_error.clear();
  BlockPlan bp;
  if (int e = make_block_plan(d, bk, bp)) return e;
  Plan& pl = bp.pl;
  ttt::Prob& P = pl.P;
  if (P.stok == 0) return TTT_OK;
  if (!bk->anchors) return fail(TTT_ERR_NULL_ARG, "anchors is NULL");
  if ((uintptr_t)bk->anchors & 3u) return fail(TTT_ERR_MISALIGNED, "anchors is not 4-byte aligned");
  if (int e = check_ptr(q, "q")) return e;
  if (int e = check_ptr(k_blk, "k_blk")) return e;
  if (int e = check_ptr(v_blk, "v_blk")) return e;
  if (int e = check_ptr(o, "o")) return e;
  if (P.kv_len > 0) {  // an empty context is never read: its pointers may be NULL
    if (int e = check_ptr(k_ctx, "k_ctx")) return e;
    if (int e = check_ptr(v_ctx, "v_ctx")) return e;
  }
  if (!lse) return fail(TTT_ERR_NULL_ARG, "lse is NULL");
  if ((uintptr_t)lse & 3u) return fail(TTT_ERR_MISALIGNED, "lse is not 4-byte aligned");
  if (int e = check_ws(pl, ws, ws_bytes)) return e;
  hipStream_t st = (hipStream_t)stream;
  if (int e = check_block_cu(d, bk, st)) return e;
  (void)hipGetLastError();
  float* cosT = at<float>(ws, pl.ws.table);
  float* sinT = cosT + (size_t)P.npos * (P.D / 2);
  _Float16* ckt = at<_Float16>(ws, bp.ctx_kt);
  _Float16* cvt = at<_Float16>(ws, bp.ctx_vt);
  _Float16* bkt = at<_Float16>(ws, bp.blk_kt);
  _Float16* bvt = at<_Float16>(ws, bp.blk_vt);
  const bool thd = P.layout == TTT_LAYOUT_THD;
  int* slots = thd ? at<int>(ws, bp.slots) : nullptr;
  P.slot_base = slots;
  TTT_TRACED("rope_table", ttt::launch_rope_table(P, cosT, sinT, (double)d->rope_base, st));
  const int4* tiles = nullptr;
  if (thd) {  // THD: the slots of each sequence (block rows and context), then the query tiles
    int4* t = at<int4>(ws, bp.tiles_q);
    TTT_TRACED("tile_sched",
               ttt::launch_tile_sched(P, ttt::block_fwd_tile_rows(P.r), 1, t, bp.max_tiles_q, slots, st));
    tiles = t;
  }
  // context: K~ rows at positions j and V^T (kv_len rows; THD: each sequence's own)
  ttt::Prob Pc = P;
  Pc.stok = P.kv_len;
  ttt::PrepJobs J;
  memset(&J, 0, sizeof J);
  J.n = 2;
  J.j[0] = {(const uint16_t*)k_ctx, bp.cs_b, bp.cs_t, bp.cs_h, P.Hkv, 0, 1, 0, ckt, nullptr, 0, nullptr, 0};
  J.j[1] = {(const uint16_t*)v_ctx, bp.cs_b, bp.cs_t, bp.cs_h, P.Hkv, 0, 0, 0, nullptr, (uint16_t*)cvt, 0, nullptr, 0};
  if (thd)
    for (int j = 0; j < 2; ++j) J.j[j].cu = P.kv_cu, J.j[j].ntok = P.kv_tok;
  TTT_TRACED("prep_ctx", ttt::launch_prep_bf16(Pc, J, cosT, sinT, st));
  // block keys: K~ rows at their slot positions and V^T (spad_b slots)
  ttt::Prob Pb = P;
  Pb.spad = P.spad_b;
  J.j[0] = {(const uint16_t*)k_blk, P.ks_b, P.ks_t, P.ks_h, P.Hkv, 0, 1, 0, bkt, nullptr, 1, nullptr, 0};
  J.j[1] = {(const uint16_t*)v_blk, P.ks_b, P.ks_t, P.ks_h, P.Hkv, 0, 0, 0, nullptr, (uint16_t*)bvt, 0, nullptr, 0};
  TTT_TRACED("prep_blk", ttt::launch_prep_bf16(Pb, J, cosT, sinT, st));
  TTT_TRACED("block_fwd", ttt::launch_block_fwd_bf16(P, (const uint16_t*)q, ckt, cvt, bkt, bvt, tiles, cosT, sinT,
                                                     o, pl.o_f32, lse, st));
  return hip_check("ttt_attn_block_fwd launch");
}

}  // extern "C"

namespace {
int make_ce(const ttt_soft_ce_desc* d, ttt::CeProb& C) {
  if (!d) return fail(TTT_ERR_NULL_ARG, "soft-CE descriptor is NULL");
  if (d->struct_size != sizeof(ttt_soft_ce_desc))
    return fail(TTT_ERR_ABI, "soft-CE struct_size %u != %zu", d->struct_size, sizeof(ttt_soft_ce_desc));
  if (d->batch < 1 || d->seqlen < 0 || (int64_t)d->batch * d->seqlen > ((int64_t)1 << 31) - 1)
    return fail(TTT_ERR_BAD_SHAPE, "batch %d / seqlen %d", d->batch, d->seqlen);
  if (d->vocab < 8 || d->vocab % 8)
    return fail(TTT_ERR_BAD_SHAPE, "vocab %d must be a positive multiple of 8", d->vocab);
  if (d->teacher_offset < 0) return fail(TTT_ERR_BAD_SHAPE, "teacher_offset %d is negative", d->teacher_offset);
  if (d->teacher_seqlen < 0 || (int64_t)d->batch * d->teacher_seqlen > ((int64_t)1 << 31) - 1)
    return fail(TTT_ERR_BAD_SHAPE, "teacher_seqlen %d", d->teacher_seqlen);
  if (d->num_groups < 0 || d->num_groups > 64)
    return fail(TTT_ERR_BAD_SHAPE, "num_groups %d outside 0..64", d->num_groups);
  if (((uintptr_t)d->teacher_rows | (uintptr_t)d->groups) & 3u)
    return fail(TTT_ERR_MISALIGNED, "teacher_rows and groups must be 4-byte aligned");
  memset(&C, 0, sizeof C);
  C.B = d->batch, C.S = d->seqlen, C.V = d->vocab, C.offset = d->teacher_offset, C.mask = d->mask;
  C.T = d->teacher_seqlen > 0 ? d->teacher_seqlen : d->seqlen;
  C.trows = d->teacher_rows, C.groups = d->groups;
  C.G = d->num_groups > 0 ? d->num_groups : 1;
  auto st = [&](const int64_t* s, int64_t& sb, int64_t& sr, const char* name, int rows) -> int {
    if (s[0] == 0 && s[1] == 0) {
      sb = (int64_t)rows * d->vocab, sr = d->vocab;
      return 0;
    }
    if (s[0] < 0 || s[1] < d->vocab)
      return fail(TTT_ERR_BAD_SHAPE, "%s strides (%lld, %lld): row stride below the vocab", name, (long long)s[0],
                  (long long)s[1]);
    if (s[0] % 8 || s[1] % 8)
      return fail(TTT_ERR_MISALIGNED, "%s strides (%lld, %lld) not multiples of 8 elements", name, (long long)s[0],
                  (long long)s[1]);
    sb = s[0], sr = s[1];
    return 0;
  };
  if (int e = st(d->student_stride, C.ss_b, C.ss_t, "student", C.S)) return e;
  if (int e = st(d->teacher_stride, C.ts_b, C.ts_t, "teacher", C.T)) return e;
  return TTT_OK;
}
}  // namespace

extern "C" {

size_t ttt_soft_ce_workspace_bytes(const ttt_soft_ce_desc* d) {
  g_last_error.clear();
  ttt::CeProb C;
  if (make_ce(d, C)) return 0;
  return align256((size_t)C.B * C.S * sizeof(float));
}

int ttt_soft_ce_fwd(const ttt_soft_ce_desc* d, const void* student, const void* teacher, float* stats,
                    float* row_lse, float* row_ce, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  ttt::CeProb C;
  if (int e = make_ce(d, C)) return e;
  if (!stats || !row_lse) return fail(TTT_ERR_NULL_ARG, "stats or row_lse is NULL");
  if (((uintptr_t)stats | (uintptr_t)row_lse | (uintptr_t)row_ce) & 3u)
    return fail(TTT_ERR_MISALIGNED, "stats, row_lse and row_ce must be 4-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (C.S > 0) {
    if (int e = check_ptr(student, "student")) return e;
    if (int e = check_ptr(teacher, "teacher")) return e;
    if (!row_ce) {
      const size_t need = (size_t)C.B * C.S * sizeof(float);
      if (!ws) return fail(TTT_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed for row_ce)", need);
      if ((uintptr_t)ws & 255u) return fail(TTT_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);
      if (ws_bytes < need) return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes is smaller than %zu", ws_bytes, need);
      row_ce = (float*)ws;
    }
  }
  (void)hipGetLastError();
  if (C.S == 0) {
    TTT_TRACED("soft_ce_mean", ttt::launch_soft_ce_fwd(C, nullptr, nullptr, row_lse, row_ce, stats, st));
  } else {
    TTT_TRACED("soft_ce_fwd", ttt::launch_soft_ce_fwd(C, (const uint16_t*)student, (const uint16_t*)teacher, row_lse,
                                                      row_ce, stats, st));
  }
  return hip_check("ttt_soft_ce_fwd launch");
}

int ttt_soft_ce_bwd(const ttt_soft_ce_desc* d, const void* student, const void* teacher, const float* row_lse,
                    const float* stats, const float* dloss, void* dstudent, void* stream) {
  g_last_error.clear();
  ttt::CeProb C;
  if (int e = make_ce(d, C)) return e;
  if (C.S == 0) return TTT_OK;
  if (int e = check_ptr(student, "student")) return e;
  if (int e = check_ptr(teacher, "teacher")) return e;
  if (int e = check_ptr(dstudent, "dstudent")) return e;
  if (!row_lse || !stats || !dloss) return fail(TTT_ERR_NULL_ARG, "row_lse, stats or dloss is NULL");
  if (((uintptr_t)row_lse | (uintptr_t)stats | (uintptr_t)dloss) & 3u)
    return fail(TTT_ERR_MISALIGNED, "row_lse, stats and dloss must be 4-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  TTT_TRACED("soft_ce_bwd", ttt::launch_soft_ce_bwd(C, (const uint16_t*)student, (const uint16_t*)teacher, row_lse,
                                                    stats, dloss, (uint16_t*)dstudent, st));
  return hip_check("ttt_soft_ce_bwd launch");
}

int ttt_attn_merge(const ttt_attn_desc* d, const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                   void* o, float* lse, void* stream) {
  g_last_error.clear();
  Plan pl;
  if (int e = make_plan(d, 0, pl)) return e;
  ttt::Prob& P = pl.P;
  if (P.stok == 0) return TTT_OK;
  if (int e = check_ptr(o_a, "o_a")) return e;
  if (int e = check_ptr(o_b, "o_b")) return e;
  if (int e = check_ptr(o, "o")) return e;
  const float* ls[3] = {lse_a, lse_b, lse};
  const char* ln[3] = {"lse_a", "lse_b", "lse"};
  for (int i = 0; i < 3; ++i) {
    if (!ls[i]) return fail(TTT_ERR_NULL_ARG, "%s is NULL", ln[i]);
    if ((uintptr_t)ls[i] & 3u) return fail(TTT_ERR_MISALIGNED, "%s is not 4-byte aligned", ln[i]);
  }
  hipStream_t st = (hipStream_t)stream;
  if (int e = check_cu(d, st)) return e;
  (void)hipGetLastError();
  TTT_TRACED("lse_merge", ttt::launch_merge(P, pl.o_f32, o_a, lse_a, o_b, lse_b, o, lse, st));
  return hip_check("ttt_attn_merge launch");
}

}  // extern "C"

namespace {
int bwd_impl(const ttt_attn_desc* d, const ttt_attn_chunk* c, const void* q, const void* const* k,
             const void* const* v, const void* o, const float* lse, const void* dout, void* dq, void* const* dk,
             void* const* dv, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan pl;
  if (int e = make_plan(d, 1, pl, c)) return e;
  ttt::Prob& P = pl.P;
  if (P.stok == 0) return TTT_OK;  // nothing to compute; pointers of empty tensors may be NULL
  if (!k || !v || !dk || !dv) return fail(TTT_ERR_NULL_ARG, "a k/v/dk/dv pointer array is NULL");
  if (int e = check_ptr(q, "q")) return e;
  if (int e = check_ptr(o, "o")) return e;
  if (int e = check_ptr(dout, "dout")) return e;
  if (int e = check_ptr(dq, "dq")) return e;
  if (!lse) return fail(TTT_ERR_NULL_ARG, "lse is NULL");
  if ((uintptr_t)lse & 3u) return fail(TTT_ERR_MISALIGNED, "lse is not 4-byte aligned");
  ttt::PassPtrs kv;
  ttt::PassGradPtrs g;
  memset(&kv, 0, sizeof kv);
  memset(&g, 0, sizeof g);
  if (c) P.out_f32 = 1;                  // ring-step terms are fp32 (the caller sums them)
  const int nptr = P.branch ? P.p : 1;  // a ring step without the branch touches pass 1 only
  for (int i = 0; i < nptr; ++i) {
    // an empty pass-1 key block (kv_len = 0) is never read or written: its pointers may be NULL
    if (i == 0 && P.kv_len == 0 && !k[0] && !v[0] && !dk[0] && !dv[0]) continue;
    char nm[16];
    snprintf(nm, sizeof nm, "k[%d]", i);
    if (int e = check_ptr(k[i], nm)) return e;
    snprintf(nm, sizeof nm, "v[%d]", i);
    if (int e = check_ptr(v[i], nm)) return e;
    snprintf(nm, sizeof nm, "dk[%d]", i);
    if (int e = check_ptr(dk[i], nm)) return e;
    snprintf(nm, sizeof nm, "dv[%d]", i);
    if (int e = check_ptr(dv[i], nm)) return e;
    kv.k[i] = k[i];
    kv.v[i] = v[i];
    g.dk[i] = dk[i];
    g.dv[i] = dv[i];
  }
  if (int e = check_ws(pl, ws, ws_bytes)) return e;
  hipStream_t st = (hipStream_t)stream;
  if (int e = check_cu(d, st, c)) return e;
  (void)hipGetLastError();

  float* cosT = at<float>(ws, pl.ws.table);
  float* sinT = cosT + (size_t)P.npos * (P.D / 2);
  float* delta = at<float>(ws, pl.ws.delta);
  const bool thd = P.layout == TTT_LAYOUT_THD;
  int* slots = thd ? at<int>(ws, pl.ws.slots) : nullptr;
  P.slot_base = slots;
  TTT_TRACED("rope_table", ttt::launch_rope_table(P, cosT, sinT, (double)d->rope_base, st));
  const int4 *tq = nullptr, *tkv = nullptr;
  if (thd) {
    if (pl.bf16) {
      int4* a = at<int4>(ws, pl.ws.tiles_q);
      int4* b = at<int4>(ws, pl.ws.tiles_kv);
      TTT_TRACED("tile_sched", ttt::launch_tile_sched(P, ttt::dq_tile_rows(P.r), 1, a, pl.max_tiles_q, slots, st));
      ttt::Prob Pkv = P;  // key tiles: a THD ring step's packed key rows, on the slots laid out above
      if (P.kv_cu) Pkv.cu = P.kv_cu, Pkv.stok = P.kv_tok;
      TTT_TRACED("tile_sched", ttt::launch_tile_sched(Pkv, ttt::kBwdBKV, 0, b, pl.max_tiles_kv, nullptr, st));
      tq = a;
      tkv = b;
    } else {
      TTT_TRACED("tile_sched", ttt::launch_tile_sched(P, 64, 1, nullptr, 0, slots, st));
    }
  }
  // bf16: Delta and then the branch gradients (HBM-bound, few registers, no
  // LDS) run on the caller's aux stream when one is given: Delta beside the
  // Q~/K~ rotations, the branch kernel beside the dK/dV kernel (one MFMA wave
  // per SIMD leaves room for one more wave).
  Side sd;
  const bool forked = pl.bf16 && sd.begin(st, (hipStream_t)d->aux_stream);
  const hipStream_t sst = forked ? sd.side : st;
  if (pl.bf16) set_bounds(P, at<char>(ws, pl.ws.bnd), 1, pl.ds);
  if (pl.ds) P.ds = at<_Float16>(ws, pl.ws.ds);
  TTT_TRACED_ON("bwd_delta", sst,
                ttt::launch_delta(P, o, pl.o_f32, dout, !pl.bf16, pl.bf16 ? lse : nullptr, delta, v[0], sst));
  if (pl.bf16) TTT_TRACED_ON("bwd_dmax", sst, ttt::launch_dmax(P, sst));
  const hipEvent_t delta_done = forked ? sd.mark(sd.side) : nullptr;
  if (!pl.bf16) {
    float* kt = at<float>(ws, pl.ws.kt);
    float* qt = at<float>(ws, pl.ws.qt);
    TTT_TRACED("prep_k_f32",
               ttt::launch_prep_rot_f32(P, (const float*)k[0], P.ks_b, P.ks_t, P.ks_h, P.Hkv, 0, cosT, sinT, kt, st));
    TTT_TRACED("prep_q_f32", ttt::launch_prep_rot_f32(P, (const float*)q, P.qs_b, P.qs_t, P.qs_h, P.Hq, P.p - 1, cosT,
                                                      sinT, qt, st));
    ttt::launch_bwd_f32(P, kv, lse, (const float*)dout, kt, qt, delta, cosT, sinT, (float*)dq, g, st);
  } else {
    _Float16* kt = at<_Float16>(ws, pl.ws.kt);
    _Float16* ktt = at<_Float16>(ws, pl.ws.ktt);
    _Float16* qt = at<_Float16>(ws, pl.ws.qt);
    // rotated K~ rows, their transpose K~^T and rotated Q~ rows in one launch
    ttt::PrepJobs J;
    memset(&J, 0, sizeof J);
    J.n = 2;
    // pass-1 keys: kv_len rows at positions kv_off + j; queries at q_off + i + p - 1
    const int krows = (c && P.layout == TTT_LAYOUT_BSHD) ? (P.kv_len > 0 ? P.kv_len : -1) : 0;
    J.j[0] = {(const uint16_t*)k[0], pl.k0s_b, pl.k0s_t, pl.k0s_h, P.Hkv, P.kv_off, 1, 0, kt, (uint16_t*)ktt, 0,
              nullptr, krows};
    J.j[1] = {(const uint16_t*)q, P.qs_b, P.qs_t, P.qs_h, P.Hq, P.q_off + P.p - 1, 1, 0, qt, nullptr, 0, nullptr, 0};
    if (P.kv_cu) {  // THD ring step: per-sequence key rows and offsets
      J.j[0].cu = P.kv_cu, J.j[0].ntok = P.kv_tok, J.j[0].seg_pos = P.seg_kvoff;
      J.j[1].seg_pos = P.seg_qoff;
    }
    J.heads_fast = 1;  // mostly row-major outputs (Q~ rows)
    TTT_TRACED("prep_kq", ttt::launch_prep_bf16(P, J, cosT, sinT, st));
    if (forked) sd.wait(st, delta_done);
    // branch dK/dV of passes 2..p: in the dQ kernel's epilogue when its work
    // item holds every query head of a KV group, else a kernel of their own
    // beside dK/dV on the aux stream
    P.dq_branch = ttt::dq_fuses_branch(P.r) ? 1 : 0;
    const bool branch = P.p > 1 && P.branch && !P.dq_branch;
    if (forked && branch) sd.wait(sd.side, sd.mark(st));  // start the branch kernel with dK/dV, not beside the prologue
    if (branch)
      TTT_TRACED_ON("branch_bwd", sst,
                    ttt::launch_branch_bwd_bf16(P, (const uint16_t*)q, kv, lse, (const uint16_t*)dout, delta, cosT,
                                                sinT, g, sst));
    ttt::Prob Pk = P;  // the pass-1 keys' V / dK / dV strides
    Pk.ks_b = pl.k0s_b, Pk.ks_t = pl.k0s_t, Pk.ks_h = pl.k0s_h;
    TTT_TRACED("trunk_dkdv", ttt::launch_dkdv_bf16(Pk, kv, lse, (const uint16_t*)dout, kt, qt, delta, tkv, cosT,
                                                   sinT, g, st));
    TTT_TRACED(P.ds ? "trunk_dq_ds" : "trunk_dq",
               ttt::launch_dq_bf16(P, (const uint16_t*)q, kv, lse, (const uint16_t*)dout, kt, ktt, qt, delta, tq, cosT,
                                   sinT, (uint16_t*)dq, g, st));
    if (forked && branch) sd.wait(st, sd.mark(sd.side));  // the branch gradients are in
  }
  return hip_check("ttt_attn_bwd launch");
}
}  // namespace

namespace {
// bf16 head_dim 32 / 64 (the pages name no head size; 32, 64 and 128 are the
// boundary's): each head is zero-padded to 128 entries in the workspace with
// element k < D/2 at entry (128/D) k and element D/2 + k at 64 + (128/D) k, so
// that the D = 128 rotate-half pairs and frequencies are exactly the D-dim
// ones and the zero entries add nothing (pad_heads_kernel); the D = 128 path
// then runs on contiguous padded tensors with softmax scale 1/sqrt(D) unless
// one is given, and its outputs are unpadded into the caller's tensors.  Cost:
// the MFMA work of D = 128 plus one pass over every tensor each way.
struct PadRoute {
  ttt_attn_desc d;                 // D = 128, contiguous padded tensors
  int D, S;                        // S: tokens per batch row (BSHD) or all tokens (THD)
  int64_t rows;                    // B*S or T
  int64_t qs[3], ks[3], os[3];     // the caller's element strides of q (and dq), k / v (and dk / dv), o (and dout)
  size_t q, kv, o, dout, dq, dkv, inner, total;  // workspace offsets; kv / dkv: 2p padded tensors
  size_t q_bytes, kv_bytes, o_bytes;
};

int make_pad_route(const ttt_attn_desc* d, int for_bwd, PadRoute& r) {
  if (d->layout != TTT_LAYOUT_BSHD && d->layout != TTT_LAYOUT_THD)
    return fail(TTT_ERR_BAD_SHAPE, "layout %d is neither BSHD (0) nor THD (1)", d->layout);
  const bool thd = d->layout == TTT_LAYOUT_THD;
  r.D = d->head_dim;
  r.d = *d;
  r.d.head_dim = 128;
  if (!(d->softmax_scale > 0.f)) r.d.softmax_scale = 1.0f / sqrtf((float)r.D);
  for (int i = 0; i < 3; ++i) r.d.q_stride[i] = r.d.kv_stride[i] = r.d.o_stride[i] = 0;
  Plan pl;
  if (int e = make_plan(&r.d, for_bwd, pl)) return e;
  const int Hq = d->num_q_heads, Hkv = d->num_kv_heads, D = r.D;
  r.S = d->seqlen;
  r.rows = thd ? (int64_t)d->seqlen : (int64_t)d->batch * d->seqlen;
  auto strides = [&](const int64_t* s, int H, int64_t* out, const char* name) -> int {
    if (s[0] == 0 && s[1] == 0 && s[2] == 0) {
      out[0] = thd ? 0 : (int64_t)r.S * H * D, out[1] = (int64_t)H * D, out[2] = D;
      return 0;
    }
    for (int i = 0; i < 3; ++i)
      if (s[i] < 0) return fail(TTT_ERR_BAD_SHAPE, "%s stride[%d] = %lld is negative", name, i, (long long)s[i]);
    out[0] = thd ? 0 : s[0], out[1] = s[1], out[2] = s[2];
    return 0;
  };
  if (int e = strides(d->q_stride, Hq, r.qs, "q")) return e;
  if (int e = strides(d->kv_stride, Hkv, r.ks, "kv")) return e;
  if (int e = strides(d->o_stride, Hq, r.os, "o")) return e;
  const int p = d->pass_index;
  const size_t osz = d->o_dtype == TTT_DTYPE_FP32 ? 4 : 2;
  r.q_bytes = (size_t)r.rows * Hq * 128 * 2;
  r.kv_bytes = (size_t)r.rows * Hkv * 128 * 2;
  r.o_bytes = (size_t)r.rows * Hq * 128 * osz;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at_ = off;
    off = align256(off + bytes);
    return at_;
  };
  r.q = take(r.q_bytes);
  r.kv = off;
  for (int i = 0; i < 2 * p; ++i) take(r.kv_bytes);
  r.o = take(r.o_bytes);
  r.dout = r.dq = r.dkv = 0;
  if (for_bwd) {
    r.dout = take((size_t)r.rows * Hq * 128 * 2);
    r.dq = take(r.q_bytes);
    r.dkv = off;
    for (int i = 0; i < 2 * p; ++i) take(r.kv_bytes);
  }
  r.inner = off;
  r.total = off + pl.ws.total;
  return TTT_OK;
}

char* kv_slot(void* ws, const PadRoute& r, size_t base, int i) {
  return (char*)ws + base + (size_t)i * align256(r.kv_bytes);
}

size_t padded_ws_bytes(const ttt_attn_desc* d, int for_bwd) {
  PadRoute r;
  if (make_pad_route(d, for_bwd, r) != TTT_OK) return 0;
  return r.total;
}

int padded_fwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v, void* o,
               float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  PadRoute r;
  if (int e = make_pad_route(d, 0, r)) return e;
  if (r.rows == 0) return TTT_OK;
  if (!k || !v) return fail(TTT_ERR_NULL_ARG, "k or v pointer array is NULL");
  if (!q || !o || !lse) return fail(TTT_ERR_NULL_ARG, "q, o or lse is NULL");
  const int p = d->pass_index, Hq = d->num_q_heads, Hkv = d->num_kv_heads;
  for (int i = 0; i < p; ++i)
    if (!k[i] || !v[i]) return fail(TTT_ERR_NULL_ARG, "k[%d] or v[%d] is NULL", i, i);
  if (r.total && (!ws || ((uintptr_t)ws & 255u) || ws_bytes < r.total))
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes at %p: %zu bytes, 256-byte aligned, needed", ws_bytes,
                ws, r.total);
  hipStream_t st = (hipStream_t)stream;
  const bool o32 = d->o_dtype == TTT_DTYPE_FP32;
  char* w = (char*)ws;
  const void* kp[TTT_MAX_PASSES];
  const void* vp[TTT_MAX_PASSES];
  ttt::trace("pad_heads", 0, st);
  ttt::launch_pad_heads(q, false, r.qs[0], r.qs[1], r.qs[2], r.rows, r.S, Hq, r.D, w + r.q, st);
  for (int i = 0; i < p; ++i) {
    kp[i] = kv_slot(ws, r, r.kv, i);
    vp[i] = kv_slot(ws, r, r.kv, p + i);
    ttt::launch_pad_heads(k[i], false, r.ks[0], r.ks[1], r.ks[2], r.rows, r.S, Hkv, r.D, (void*)kp[i], st);
    ttt::launch_pad_heads(v[i], false, r.ks[0], r.ks[1], r.ks[2], r.rows, r.S, Hkv, r.D, (void*)vp[i], st);
  }
  ttt::trace("pad_heads", 1, st);
  if (int e = hip_check("pad_heads launch")) return e;
  if (int e = fwd_impl(&r.d, nullptr, w + r.q, kp, vp, w + r.o, lse, w + r.inner, ws_bytes - r.inner, stream))
    return e;
  ttt::trace("unpad_heads", 0, st);
  ttt::launch_unpad_heads(w + r.o, o32, r.rows, r.S, Hq, r.D, o, r.os[0], r.os[1], r.os[2], st);
  ttt::trace("unpad_heads", 1, st);
  return hip_check("unpad_heads launch");
}

int padded_bwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v, const void* o,
               const float* lse, const void* dout, void* dq, void* const* dk, void* const* dv, void* ws,
               size_t ws_bytes, void* stream) {
  g_last_error.clear();
  PadRoute r;
  if (int e = make_pad_route(d, 1, r)) return e;
  if (r.rows == 0) return TTT_OK;
  if (!k || !v || !dk || !dv) return fail(TTT_ERR_NULL_ARG, "a k/v/dk/dv pointer array is NULL");
  if (!q || !o || !lse || !dout || !dq) return fail(TTT_ERR_NULL_ARG, "q, o, lse, dout or dq is NULL");
  const int p = d->pass_index, Hq = d->num_q_heads, Hkv = d->num_kv_heads;
  for (int i = 0; i < p; ++i)
    if (!k[i] || !v[i] || !dk[i] || !dv[i]) return fail(TTT_ERR_NULL_ARG, "k/v/dk/dv[%d] is NULL", i);
  if (r.total && (!ws || ((uintptr_t)ws & 255u) || ws_bytes < r.total))
    return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes at %p: %zu bytes, 256-byte aligned, needed", ws_bytes,
                ws, r.total);
  hipStream_t st = (hipStream_t)stream;
  const bool o32 = d->o_dtype == TTT_DTYPE_FP32;
  char* w = (char*)ws;
  const void* kp[TTT_MAX_PASSES];
  const void* vp[TTT_MAX_PASSES];
  void* dkp[TTT_MAX_PASSES];
  void* dvp[TTT_MAX_PASSES];
  ttt::trace("pad_heads", 0, st);
  ttt::launch_pad_heads(q, false, r.qs[0], r.qs[1], r.qs[2], r.rows, r.S, Hq, r.D, w + r.q, st);
  ttt::launch_pad_heads(o, o32, r.os[0], r.os[1], r.os[2], r.rows, r.S, Hq, r.D, w + r.o, st);
  ttt::launch_pad_heads(dout, false, r.os[0], r.os[1], r.os[2], r.rows, r.S, Hq, r.D, w + r.dout, st);
  for (int i = 0; i < p; ++i) {
    kp[i] = kv_slot(ws, r, r.kv, i);
    vp[i] = kv_slot(ws, r, r.kv, p + i);
    dkp[i] = kv_slot(ws, r, r.dkv, i);
    dvp[i] = kv_slot(ws, r, r.dkv, p + i);
    ttt::launch_pad_heads(k[i], false, r.ks[0], r.ks[1], r.ks[2], r.rows, r.S, Hkv, r.D, (void*)kp[i], st);
    ttt::launch_pad_heads(v[i], false, r.ks[0], r.ks[1], r.ks[2], r.rows, r.S, Hkv, r.D, (void*)vp[i], st);
  }
  ttt::trace("pad_heads", 1, st);
  if (int e = hip_check("pad_heads launch")) return e;
  if (int e = bwd_impl(&r.d, nullptr, w + r.q, kp, vp, w + r.o, lse, w + r.dout, w + r.dq, dkp, dvp, w + r.inner,
                       ws_bytes - r.inner, stream))
    return e;
  ttt::trace("unpad_heads", 0, st);
  ttt::launch_unpad_heads(w + r.dq, false, r.rows, r.S, Hq, r.D, dq, r.qs[0], r.qs[1], r.qs[2], st);
  for (int i = 0; i < p; ++i) {
    ttt::launch_unpad_heads(dkp[i], false, r.rows, r.S, Hkv, r.D, dk[i], r.ks[0], r.ks[1], r.ks[2], st);
    ttt::launch_unpad_heads(dvp[i], false, r.rows, r.S, Hkv, r.D, dv[i], r.ks[0], r.ks[1], r.ks[2], st);
  }
  ttt::trace("unpad_heads", 1, st);
  return hip_check("unpad_heads launch");
}
}  // namespace

extern "C" {

int ttt_attn_bwd(const ttt_attn_desc* d, const void* q, const void* const* k, const void* const* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* const* dk, void* const* dv, void* ws,
                 size_t ws_bytes, void* stream) {
  if (padded_head(d)) return padded_bwd(d, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream);
  return bwd_impl(d, nullptr, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream);
}

size_t ttt_attn_chunk_bwd_workspace_bytes(const ttt_attn_desc* d, const ttt_attn_chunk* c) {
  g_last_error.clear();
  if (!c) {
    fail(TTT_ERR_NULL_ARG, "chunk is NULL");
    return 0;
  }
  Plan pl;
  if (make_plan(d, 1, pl, c) != TTT_OK) return 0;
  return pl.ws.total;
}

int ttt_attn_bwd_chunk(const ttt_attn_desc* d, const ttt_attn_chunk* c, const void* q, const void* const* k,
                       const void* const* v, const void* o, const float* lse, const void* dout, float* dq,
                       float* const* dk, float* const* dv, void* ws, size_t ws_bytes, void* stream) {
  if (!c) {
    g_last_error.clear();
    return fail(TTT_ERR_NULL_ARG, "chunk is NULL");
  }
  return bwd_impl(d, c, q, k, v, o, lse, dout, dq, (void* const*)dk, (void* const*)dv, ws, ws_bytes, stream);
}

}  // extern "C"
