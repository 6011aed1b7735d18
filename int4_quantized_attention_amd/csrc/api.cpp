// Host side of the rotattn C ABI: validation, workspace layout, RoPE tables,
// P-level thresholds and kernel launches.  See include/rotattn.h.
#include "../../include/rotattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <limits>

#include "kernels.h"

namespace {

using ra::Shape;

Shape to_shape(const rotattn_shape* s) {
  return Shape{s->B, s->H, s->F, s->Hs, s->Ws, s->D, s->Df, s->Dh, s->Dw, s->qk_blk, s->kv_blk};
}
int64_t tokens(const rotattn_shape* s) { return (int64_t)s->F * s->Hs * s->Ws; }
bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// P level thresholds, found independently of any other code base: T[k-1] is the
// smallest binary32 y with 2^y rounding (half to even) to a level >= k.  For k = 1
// the boundary 2^y = 1/2 is a tie that rounds down, so T[0] is the float after -1;
// for k >= 2 the boundary k - 1/2 is never a power of two and T[k-1] is the
// smallest float whose extended-precision exp2 exceeds k - 1/2.
struct Levels {
  float T[16];
  Levels() {
    T[0] = std::nextafter(-1.0f, 0.0f);
    for (int k = 2; k <= 15; ++k) {
      const long double bound = (long double)k - 0.5L;
      float y = (float)std::log2((double)bound);
      while (exp2l((long double)y) <= bound) y = std::nextafter(y, std::numeric_limits<float>::infinity());
      for (;;) {
        const float below = std::nextafter(y, -std::numeric_limits<float>::infinity());
        if (exp2l((long double)below) > bound) y = below;
        else break;
      }
      T[k - 1] = y;
    }
    T[15] = std::numeric_limits<float>::infinity();
  }
};
const Levels& levels() {
  static const Levels lv;
  return lv;
}

rotattn_status launch_status(hipError_t e) { return e == hipSuccess ? ROTATTN_OK : ROTATTN_E_HIP; }

void grid_map(int64_t nqt, int nheads, int& total, int& per_xcd) {
  total = (int)(nqt * nheads);
  per_xcd = (total + 7) / 8;
}

}  // namespace

extern "C" {

rotattn_status rotattn_check_shape(const rotattn_shape* s) {
  if (!s) return ROTATTN_E_NULL;
  if (s->B < 1 || s->H < 1 || s->F < 1 || s->Hs < 1 || s->Ws < 1) return ROTATTN_E_SHAPE;
  if (s->Df < 2 || s->Dh < 2 || s->Dw < 2 || (s->Df | s->Dh | s->Dw) & 1) return ROTATTN_E_SHAPE;
  if (s->Df + s->Dh + s->Dw != s->D) return ROTATTN_E_SHAPE;
  if (s->D != 64 && s->D != 128) return ROTATTN_E_UNSUPPORTED;
  if (!pow2_in(s->qk_blk, 1, 128) || !pow2_in(s->kv_blk, 16, 256)) return ROTATTN_E_UNSUPPORTED;
  const int64_t N = tokens(s);
  if (N > (int64_t)1 << 28) return ROTATTN_E_UNSUPPORTED;
  if ((int64_t)s->B * s->H > 65535) return ROTATTN_E_UNSUPPORTED;
  return ROTATTN_OK;
}

int64_t rotattn_padded_tokens(const rotattn_shape* s) {
  if (!s) return 0;
  const int64_t N = tokens(s);
  return (N + ra::kTokenPad - 1) / ra::kTokenPad * ra::kTokenPad;
}

size_t rotattn_rope_table_floats(const rotattn_shape* s) {
  if (!s) return 0;
  return (size_t)2 * ((size_t)s->F * (s->Df / 2) + (size_t)s->Hs * (s->Dh / 2) + (size_t)s->Ws * (s->Dw / 2));
}

rotattn_status rotattn_build_rope_table(const rotattn_shape* s, rotattn_rot rot, double base, float* host_out) {
  if (!s || !host_out) return ROTATTN_E_NULL;
  const rotattn_status st = rotattn_check_shape(s);
  if (st != ROTATTN_OK) return st;
  if (rot < ROTATTN_ROT_NONE || rot > ROTATTN_ROT_FULL || !(base > 1.0)) return ROTATTN_E_ARG;
  const int npos[3] = {s->F, s->Hs, s->Ws};
  const int dj[3] = {s->Df, s->Dh, s->Dw};
  const double half_sqrt2 = 0.70710678118654752440;  // nearest binary64 to 1/sqrt(2)
  float* out = host_out;
  for (int ax = 0; ax < 3; ++ax) {
    for (int p = 0; p < npos[ax]; ++p) {
      for (int i = 0; i < dj[ax] / 2; ++i) {
        const double theta = std::pow(base, -(2.0 * i) / (double)dj[ax]);
        const double ang = (double)p * theta;
        const double c = std::cos(ang), sn = std::sin(ang);
        if (rot == ROTATTN_ROT_INTERLEAVED) {
          out[0] = (float)((c + sn) * half_sqrt2);
          out[1] = (float)((c - sn) * half_sqrt2);
        } else {
          out[0] = (float)c;
          out[1] = (float)sn;
        }
        out += 2;
      }
    }
  }
  return ROTATTN_OK;
}

// quantisation workspace: K partial sums, Q partial sums (with_q: room for Q
// smoothing), K mean, Q mean, V amax
struct QWs {
  size_t qpart, kmu, qmu, amax, total;
};
static QWs q_ws_parts(const rotattn_shape* s, bool with_q = true) {
  const int64_t N = tokens(s);
  const int64_t BH = (int64_t)s->B * s->H;
  const int64_t nblk = (N + 63) / 64;
  const size_t part = align256((size_t)BH * nblk * s->D * sizeof(double));
  const size_t mu = align256((size_t)BH * s->D * sizeof(float));
  const size_t amax = align256((size_t)BH * s->D * sizeof(uint32_t));
  QWs w;
  w.qpart = part;
  w.kmu = (with_q ? 2 : 1) * part;
  w.qmu = w.kmu + mu;
  w.amax = w.qmu + mu;
  w.total = w.amax + amax;
  return w;
}

size_t rotattn_quantize_qk_workspace(const rotattn_shape* s) {
  if (!s || rotattn_check_shape(s) != ROTATTN_OK) return 0;
  return q_ws_parts(s).total;
}

namespace {
// Variable-length batch: B lengths in [1, N] copied into the kernel arguments.
rotattn_status set_lens(const rotattn_shape* s, const int32_t* seq_lens, int& nlens, int* lens) {
  nlens = 0;
  if (!seq_lens) return ROTATTN_OK;
  if (s->B > ra::kMaxBatch) return ROTATTN_E_UNSUPPORTED;
  const int64_t N = tokens(s);
  for (int b = 0; b < s->B; ++b) {
    if (seq_lens[b] < 1 || seq_lens[b] > N) return ROTATTN_E_ARG;
    lens[b] = seq_lens[b];
  }
  nlens = s->B;
  return ROTATTN_OK;
}

// noalloc: use the library's fixed scratch (workspace is ignored); without Q
// smoothing, so no room is kept for Q partial sums.
rotattn_status quantize_call(const rotattn_shape* s, rotattn_rot rot, rotattn_dtype in_dtype,
                             const void* q, const void* k, const void* v,
                             const float* rope_table, int32_t smooth_k,
                             uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
                             uint8_t* v_codes, float* v_scale, int32_t* v_colsum, bool smooth_q, float* k_bias,
                             const int32_t* seq_lens, void* workspace, size_t workspace_bytes, void* stream,
                             bool noalloc = false) {
  const rotattn_status st = rotattn_check_shape(s);
  if (st != ROTATTN_OK) return st;
  if (!q || !k || !v || !rope_table || !q_codes || !q_scale || !k_codes || !k_scale || !v_codes ||
      !v_scale || (!workspace && !noalloc) || (smooth_q && !k_bias))
    return ROTATTN_E_NULL;
  if (rot < ROTATTN_ROT_NONE || rot > ROTATTN_ROT_FULL) return ROTATTN_E_ARG;
  if (in_dtype < ROTATTN_F32 || in_dtype > ROTATTN_BF16) return ROTATTN_E_ARG;
  const QWs w = q_ws_parts(s, !noalloc);
  if (noalloc) {
    if (w.total > ra::kQuantScratchBytes) return ROTATTN_E_WORKSPACE;
    if (ra::quant_scratch(&workspace) != hipSuccess) return ROTATTN_E_HIP;
    workspace_bytes = ra::kQuantScratchBytes;
  }
  if (workspace_bytes < w.total) return ROTATTN_E_WORKSPACE;
  ra::QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.s = to_shape(s);
  a.Np = rotattn_padded_tokens(s);
  a.rot = (int)rot;
  a.smooth = smooth_k ? 1 : 0;
  a.smooth_q = smooth_q ? 1 : 0;
  a.q = q; a.k = k; a.v = v;
  a.table = rope_table;
  a.qc = q_codes; a.qs = q_scale; a.kc = k_codes; a.ks = k_scale;
  a.vc = v_codes; a.vs = v_scale; a.vcol = v_colsum;
  a.kbias = k_bias;
  const rotattn_status ls = set_lens(s, seq_lens, a.nlens, a.lens);
  if (ls != ROTATTN_OK) return ls;
  a.kpart = (double*)workspace;
  a.qpart = (double*)((char*)workspace + w.qpart);
  a.kmu = (float*)((char*)workspace + w.kmu);
  a.qmu = (float*)((char*)workspace + w.qmu);
  a.vamax = (uint32_t*)((char*)workspace + w.amax);
  return launch_status(ra::launch_quantize(a, (int)in_dtype, (hipStream_t)stream));
}
}  // namespace

rotattn_status rotattn_quantize_qk(const rotattn_shape* s, rotattn_rot rot, rotattn_dtype in_dtype,
                                   const void* q, const void* k, const void* v,
                                   const float* rope_table, int32_t smooth_k,
                                   uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
                                   uint8_t* v_codes, float* v_scale, int32_t* v_colsum,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_call(s, rot, in_dtype, q, k, v, rope_table, smooth_k, q_codes, q_scale, k_codes, k_scale,
                       v_codes, v_scale, v_colsum, false, nullptr, nullptr, workspace, workspace_bytes, stream);
}

rotattn_status rotattn_quantize_qk_ex(const rotattn_shape* s, rotattn_rot rot, rotattn_dtype in_dtype,
                                      const void* q, const void* k, const void* v,
                                      const float* rope_table, const rotattn_quantize_opts* opts,
                                      uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
                                      uint8_t* v_codes, float* v_scale, int32_t* v_colsum,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const rotattn_quantize_opts o = opts ? *opts : rotattn_quantize_opts{1, 0, nullptr, nullptr};
  return quantize_call(s, rot, in_dtype, q, k, v, rope_table, o.smooth_k, q_codes, q_scale, k_codes, k_scale,
                       v_codes, v_scale, v_colsum, o.smooth_q != 0, o.k_bias, o.seq_lens, workspace,
                       workspace_bytes, stream);
}

size_t rotattn_quantize_qk_noalloc_scratch(const rotattn_shape* s) {
  if (!s || rotattn_check_shape(s) != ROTATTN_OK) return 0;
  return q_ws_parts(s, false).total;
}

size_t rotattn_quantize_qk_noalloc_max_scratch(void) { return ra::kQuantScratchBytes; }

rotattn_status rotattn_quantize_qk_noalloc(const rotattn_shape* s, rotattn_rot rot, rotattn_dtype in_dtype,
                                           const void* q, const void* k, const void* v,
                                           const float* rope_table, int32_t smooth_k,
                                           uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
                                           uint8_t* v_codes, float* v_scale, int32_t* v_colsum, void* stream) {
  return quantize_call(s, rot, in_dtype, q, k, v, rope_table, smooth_k, q_codes, q_scale, k_codes, k_scale,
                       v_codes, v_scale, v_colsum, false, nullptr, nullptr, nullptr, 0, stream, true);
}

size_t rotattn_int4_attention_workspace(const rotattn_shape* s) {
  if (!s || rotattn_check_shape(s) != ROTATTN_OK) return 0;
  return ra::attention_workspace_bytes(s->D, s->kv_blk, s->qk_blk, (int64_t)s->B * s->H, rotattn_padded_tokens(s));
}

namespace {
// Both attention entry points: pmax 15 is the method (range-rectified P codes),
// pmax 7 the symmetric baseline of the ablation.
rotattn_status attention_call(const rotattn_shape* s,
                              const uint8_t* q_codes, const float* q_scale,
                              const uint8_t* k_codes, const float* k_scale,
                              const uint8_t* v_codes, const float* v_scale,
                              const int32_t* heads, int32_t n_heads,
                              rotattn_dtype out_dtype, void* out,
                              const rotattn_debug* dbg,
                              void* workspace, size_t workspace_bytes, void* stream, int pmax, int causal,
                              const float* k_bias, const int32_t* seq_lens, uint64_t* skip_stats) {
  const rotattn_status st = rotattn_check_shape(s);
  if (st != ROTATTN_OK) return st;
  if (causal < 0 || (pmax != 15 && pmax != 7)) return ROTATTN_E_ARG;
  if (!q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale || !out || !workspace)
    return ROTATTN_E_NULL;
  // one head's images are addressed through a buffer resource with a 32-bit range
  if (rotattn_int4_attention_workspace(s) / ((size_t)s->B * s->H) > (size_t)INT32_MAX) return ROTATTN_E_UNSUPPORTED;
  if (workspace_bytes < rotattn_int4_attention_workspace(s) || ((uintptr_t)workspace & 15) != 0)
    return ROTATTN_E_WORKSPACE;
  if (out_dtype < ROTATTN_F32 || out_dtype > ROTATTN_BF16) return ROTATTN_E_ARG;
  if (((uintptr_t)skip_stats & 7) != 0) return ROTATTN_E_ARG;
  const int BH = s->B * s->H;
  if (heads) {
    if (n_heads < 0) return ROTATTN_E_ARG;
    for (int i = 0; i < n_heads; ++i)
      if (heads[i] < 0 || heads[i] >= BH) return ROTATTN_E_ARG;
  }
  const int64_t N = tokens(s);
  ra::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.qc = q_codes; a.qs = q_scale; a.kc = k_codes; a.ks = k_scale; a.vc = v_codes; a.vs = v_scale;
  a.img = (uint8_t*)workspace;
  a.img_bytes = (int64_t)workspace_bytes;
  a.out = out;
  a.out_kind = (int)out_dtype;
  a.N = N;
  a.Np = rotattn_padded_tokens(s);
  a.qk_blk = s->qk_blk;
  a.nqt = (int)((N + 127) / 128);
  a.C0 = (float)(1.4426950408889634074 / std::sqrt((double)s->D));
  a.L15 = (float)std::log2((double)pmax);
  a.p_zero = pmax == 15 ? 8 : 0;
  a.causal = causal < N ? causal : 0;  // a block of N or more keys is every key
  a.kbias = k_bias;
  a.stats = (unsigned long long*)skip_stats;
  a.H = s->H;
  const rotattn_status ls = set_lens(s, seq_lens, a.nlens, a.lens);
  if (ls != ROTATTN_OK) return ls;
  std::memcpy(a.T, levels().T, sizeof(a.T));
  hipStream_t hs = (hipStream_t)stream;
  if (dbg) {
    if (!dbg->a_qk || !dbg->p_codes || !dbg->a_pv || !dbg->m || !dbg->l) return ROTATTN_E_NULL;
    if (dbg->bh < 0 || dbg->bh >= BH || dbg->row0 < 0 || dbg->n_rows < 1 ||
        (int64_t)dbg->row0 + dbg->n_rows > (seq_lens ? seq_lens[dbg->bh / s->H] : N))
      return ROTATTN_E_ARG;
    a.dbg_row0 = dbg->row0; a.dbg_n = dbg->n_rows;
    a.dbg_aqk = dbg->a_qk; a.dbg_p = dbg->p_codes; a.dbg_apv = dbg->a_pv; a.dbg_m = dbg->m; a.dbg_l = dbg->l;
    a.nheads = 1;
    a.heads[0] = dbg->bh;
    a.total = a.nqt;
    a.per_xcd = 0;
    return launch_status(ra::launch_attention(a, s->D, s->kv_blk, true, hs));
  }
  const int nh = heads ? n_heads : BH;
  for (int h0 = 0; h0 < nh; h0 += ra::kMaxHeads) {
    const int cnt = nh - h0 < ra::kMaxHeads ? nh - h0 : ra::kMaxHeads;
    a.nheads = cnt;
    for (int i = 0; i < cnt; ++i) a.heads[i] = heads ? heads[h0 + i] : h0 + i;
    grid_map(a.nqt, cnt, a.total, a.per_xcd);
    const hipError_t e = ra::launch_attention(a, s->D, s->kv_blk, false, hs);
    if (e != hipSuccess) return ROTATTN_E_HIP;
  }
  return ROTATTN_OK;
}
}  // namespace

rotattn_status rotattn_int4_attention(const rotattn_shape* s,
                                      const uint8_t* q_codes, const float* q_scale,
                                      const uint8_t* k_codes, const float* k_scale,
                                      const uint8_t* v_codes, const float* v_scale,
                                      const int32_t* heads, int32_t n_heads,
                                      rotattn_dtype out_dtype, void* out,
                                      const rotattn_debug* dbg,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return attention_call(s, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, heads, n_heads, out_dtype, out,
                        dbg, workspace, workspace_bytes, stream, 15, 0, nullptr, nullptr, nullptr);
}

rotattn_status rotattn_int4_attention_symmetric_p(const rotattn_shape* s,
                                                  const uint8_t* q_codes, const float* q_scale,
                                                  const uint8_t* k_codes, const float* k_scale,
                                                  const uint8_t* v_codes, const float* v_scale,
                                                  const int32_t* heads, int32_t n_heads,
                                                  rotattn_dtype out_dtype, void* out,
                                                  const rotattn_debug* dbg,
                                                  void* workspace, size_t workspace_bytes, void* stream) {
  return attention_call(s, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, heads, n_heads, out_dtype, out,
                        dbg, workspace, workspace_bytes, stream, 7, 0, nullptr, nullptr, nullptr);
}

rotattn_status rotattn_int4_attention_ex(const rotattn_shape* s,
                                         const uint8_t* q_codes, const float* q_scale,
                                         const uint8_t* k_codes, const float* k_scale,
                                         const uint8_t* v_codes, const float* v_scale,
                                         const int32_t* heads, int32_t n_heads,
                                         const rotattn_attention_opts* opts,
                                         rotattn_dtype out_dtype, void* out,
                                         const rotattn_debug* dbg,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  const int pmax = opts && opts->p_max ? opts->p_max : 15;
  return attention_call(s, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, heads, n_heads, out_dtype, out,
                        dbg, workspace, workspace_bytes, stream, pmax, opts ? opts->causal_block : 0,
                        opts ? opts->k_bias : nullptr, opts ? opts->seq_lens : nullptr,
                        opts ? opts->skip_stats : nullptr);
}

// the fallback's workspace: RoPE'd fp16 Q [B*H][Np][D], then the K / V^T group images
static size_t fb_q_bytes(const rotattn_shape* s) {
  return align256((size_t)s->B * s->H * rotattn_padded_tokens(s) * s->D * sizeof(uint16_t));
}
static size_t fb_img_bytes(const rotattn_shape* s) {
  return align256((size_t)s->B * s->H * (rotattn_padded_tokens(s) / 64) * ra::fallback_image_bytes(s->D));
}

size_t rotattn_fp16_fallback_workspace(const rotattn_shape* s) {
  if (!s || rotattn_check_shape(s) != ROTATTN_OK) return 0;
  return fb_q_bytes(s) + fb_img_bytes(s);
}

rotattn_status rotattn_fp16_fallback_ex(const rotattn_shape* s, rotattn_dtype in_dtype,
                                        const void* q, const void* k, const void* v,
                                        const float* rope_table,
                                        const int32_t* heads, int32_t n_heads,
                                        const rotattn_fallback_opts* opts,
                                        rotattn_dtype out_dtype, void* out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  const rotattn_status st = rotattn_check_shape(s);
  if (st != ROTATTN_OK) return st;
  const int32_t causal_block = opts ? opts->causal_block : 0;
  if (causal_block < 0) return ROTATTN_E_ARG;
  if (!q || !k || !v || !rope_table || !out || !workspace) return ROTATTN_E_NULL;
  if (in_dtype < ROTATTN_F32 || in_dtype > ROTATTN_BF16) return ROTATTN_E_ARG;
  if (out_dtype < ROTATTN_F32 || out_dtype > ROTATTN_BF16) return ROTATTN_E_ARG;
  // one head's images are addressed through a buffer resource with a 32-bit range
  if (fb_img_bytes(s) / ((size_t)s->B * s->H) > (size_t)INT32_MAX) return ROTATTN_E_UNSUPPORTED;
  if (workspace_bytes < rotattn_fp16_fallback_workspace(s)) return ROTATTN_E_WORKSPACE;
  const int BH = s->B * s->H;
  if (heads) {
    if (n_heads < 0) return ROTATTN_E_ARG;
    for (int i = 0; i < n_heads; ++i)
      if (heads[i] < 0 || heads[i] >= BH) return ROTATTN_E_ARG;
  }
  ra::FbArgs a;
  std::memset(&a, 0, sizeof(a));
  a.s = to_shape(s);
  a.N = tokens(s);
  a.Np = rotattn_padded_tokens(s);
  a.q = q; a.k = k; a.v = v;
  a.table = rope_table;
  a.qr = (_Float16*)workspace;
  a.img = (uint8_t*)workspace + fb_q_bytes(s);
  a.img_bytes = (int64_t)fb_img_bytes(s);
  a.out = out;
  a.out_kind = (int)out_dtype;
  a.nqt = (int)((a.N + 127) / 128);
  a.scale_log2 = (float)(1.4426950408889634074 / std::sqrt((double)s->D));
  a.causal = causal_block < a.N ? causal_block : 0;  // a block of N or more keys is every key
  const rotattn_status ls = set_lens(s, opts ? opts->seq_lens : nullptr, a.nlens, a.lens);
  if (ls != ROTATTN_OK) return ls;
  hipStream_t hs = (hipStream_t)stream;
  const int nh = heads ? n_heads : BH;
  for (int h0 = 0; h0 < nh; h0 += ra::kMaxHeads) {
    const int cnt = nh - h0 < ra::kMaxHeads ? nh - h0 : ra::kMaxHeads;
    a.nheads = cnt;
    for (int i = 0; i < cnt; ++i) a.heads[i] = heads ? heads[h0 + i] : h0 + i;
    grid_map(a.nqt, cnt, a.total, a.per_xcd);
    if (ra::launch_fallback_prep(a, (int)in_dtype, hs) != hipSuccess) return ROTATTN_E_HIP;
    if (ra::launch_fallback(a, hs) != hipSuccess) return ROTATTN_E_HIP;
  }
  return ROTATTN_OK;
}

rotattn_status rotattn_fp16_fallback(const rotattn_shape* s, rotattn_dtype in_dtype,
                                     const void* q, const void* k, const void* v,
                                     const float* rope_table,
                                     const int32_t* heads, int32_t n_heads,
                                     rotattn_dtype out_dtype, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return rotattn_fp16_fallback_ex(s, in_dtype, q, k, v, rope_table, heads, n_heads, nullptr, out_dtype, out,
                                  workspace, workspace_bytes, stream);
}

rotattn_status rotattn_p_level_probe(uint32_t first_bits, int64_t n, uint8_t* out, void* stream) {
  if (!out) return ROTATTN_E_NULL;
  if (n < 0 || (uint64_t)first_bits + (uint64_t)n > ((uint64_t)1 << 32)) return ROTATTN_E_ARG;
  if (n == 0) return ROTATTN_OK;
  return launch_status(ra::launch_level_probe(first_bits, n, out, levels().T, (hipStream_t)stream));
}

const char* rotattn_status_str(rotattn_status st) {
  switch (st) {
    case ROTATTN_OK: return "ok";
    case ROTATTN_E_NULL: return "a required pointer is NULL";
    case ROTATTN_E_SHAPE: return "inconsistent shape";
    case ROTATTN_E_UNSUPPORTED: return "shape or option not supported";
    case ROTATTN_E_WORKSPACE: return "workspace too small";
    case ROTATTN_E_HIP: return "HIP launch failed";
    case ROTATTN_E_ARG: return "bad argument";
  }
  return "unknown status";
}

}  // extern "C"
