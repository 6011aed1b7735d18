/* rotattn.h -- C ABI of the MI355X (gfx950) RotateAttention hot path.
 *
 * RotateAttention (arXiv 2607.02584): mixed-precision INT4 FlashAttention for
 * DiT video models with 3D RoPE.  The problem statement (papernotes.org note,
 * "Key design 1"): Q, K, V of shape [B, H, N = F*Hs*Ws, D] with the head
 * dimension split into frame / height / width RoPE segments, D = Df + Dh + Dw.
 *
 * Three calls, in the order the pages' framework flowchart runs them:
 *   rotattn_quantize_qk    3D RoPE -> RoPE-aware orthogonal rotation -> K smoothing
 *                          -> symmetric per-block INT4 codes (Q, K); per-channel
 *                          INT4 codes of V.
 *   rotattn_int4_attention INT4 Q K^T, online softmax, range-rectified P codes
 *                          round(15 P) - 8 in [-8, 7], INT4 P V, normalisation.
 *   rotattn_fp16_fallback  FP16 FlashAttention for the heads/steps routed to full
 *                          precision ("Key design 3", selective FP16 fallback).
 *
 * Conventions shared by every call
 *   - Plain C, no HIP or torch types.  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream).  All work is enqueued asynchronously on it.
 *   - Ownership: the caller allocates and owns every buffer.  The library never
 *     allocates, frees or synchronises.  Device pointers must be on the current
 *     device; host pointers are read before the call returns.
 *   - Errors: arguments are validated on the host before any launch; a bad
 *     argument returns a status without touching the GPU.  A launch failure
 *     returns ROTATTN_E_HIP.  Nothing is thrown across the ABI.
 *   - Thread safety: no mutable global state; calls are reentrant.  (The P level
 *     threshold table is built once, on first use, with thread-safe static
 *     initialisation and never changes; kernels' LDS limits are set on each call.)
 *     The one exception is rotattn_quantize_qk_noalloc, whose calls share a fixed
 *     per-device scratch array (see there).
 *   - Layouts are C-contiguous.  Token n of a head sits at RoPE position
 *     (f, y, x) with n = (f*Hs + y)*Ws + x.  Code tensors are padded to
 *     Np = rotattn_padded_tokens() tokens; padding codes and scales are zero.
 *   - Supported: D in {64, 128}; Df, Dh, Dw even and summing to D;
 *     qk_blk a power of two in [1, 128] (1 = per-token Q/K scales, the
 *     granularity of the paper.gecl.asia analysis, "Key Insight"); kv_blk a power
 *     of two in [16, 256]; any N >= 1 (see rotattn_check_shape()).
 */
#ifndef ROTATTN_H_
#define ROTATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ROTATTN_OK = 0,
  ROTATTN_E_NULL = 1,        /* a required pointer is NULL                      */
  ROTATTN_E_SHAPE = 2,       /* inconsistent shape (D != Df+Dh+Dw, N < 1, ...)   */
  ROTATTN_E_UNSUPPORTED = 3, /* valid but not implemented (D, block sizes...)    */
  ROTATTN_E_WORKSPACE = 4,   /* workspace too small                              */
  ROTATTN_E_HIP = 5,         /* a HIP launch failed                              */
  ROTATTN_E_ARG = 6          /* other bad argument (head id out of range, ...)   */
} rotattn_status;

typedef enum {
  ROTATTN_ROT_NONE = 0,        /* RoPE only                                       */
  ROTATTN_ROT_INTERLEAVED = 1, /* H2 on channel pairs (2i, 2i+1), pre-multiplied   */
                               /* into the RoPE 2x2 blocks (M' = R M)             */
  ROTATTN_ROT_HALF = 2,        /* per segment: pair channel i with i + Dj/2, H2,  */
                               /* results at (2i, 2i+1)  (Q Pi R)                 */
  ROTATTN_ROT_FULL = 3         /* ablation: after plain RoPE, the orthonormal     */
                               /* D x D Walsh-Hadamard rotation of all channels   */
} rotattn_rot;

typedef enum { ROTATTN_F32 = 0, ROTATTN_F16 = 1, ROTATTN_BF16 = 2 } rotattn_dtype;

/* Problem shape.  N = F*Hs*Ws.  qk_blk: tokens per Q/K scale (one scale covers
 * qk_blk tokens x all D channels).  kv_blk: keys per online-softmax step; the P
 * codes depend on it (the running maximum is updated once per step). */
typedef struct {
  int32_t B, H, F, Hs, Ws, D, Df, Dh, Dw, qk_blk, kv_blk;
} rotattn_shape;

/* Validate a shape for all three calls (no GPU work). */
rotattn_status rotattn_check_shape(const rotattn_shape* s);

/* Tokens per head in every code tensor: N rounded up to a multiple of 256. */
int64_t rotattn_padded_tokens(const rotattn_shape* s);

/* ---- RoPE tables (host, init-time) --------------------------------------------
 * 3D RoPE (Key design 1): axis j in {frame, height, width} owns Dj channels; pair
 * i in [0, Dj/2) of the axis rotates by pos * base^(-2i/Dj).  Layout: frame
 * block [F][Df/2][2], then height [Hs][Dh/2][2], then width [Ws][Dw/2][2].
 * rot = INTERLEAVED stores the fused (alpha, beta) = ((c+s)/sqrt2, (c-s)/sqrt2),
 * i.e. H2 x Rot folded into the RoPE constants ("zero inference overhead");
 * otherwise (cos, sin).  Computed in binary64 (cos, sin of pos*theta), rounded
 * once to binary32.  host_out must hold rotattn_rope_table_floats() floats; the
 * caller copies it to the device for the calls below. */
size_t rotattn_rope_table_floats(const rotattn_shape* s);
rotattn_status rotattn_build_rope_table(const rotattn_shape* s, rotattn_rot rot, double base,
                                        float* host_out);

/* ---- rotattn_quantize_qk --------------------------------------------------------
 * Fused RoPE -> rotation -> smoothing -> INT4 (papernotes note: framework
 * flowchart and Key design 1; SageAttention-style K smoothing).
 *   q, k, v       device [B,H,N,D] of in_dtype.
 *   rope_table    device, from rotattn_build_rope_table(s, rot, ...).
 *   smooth_k      1: subtract from K its per-(b,h) channel mean over all N tokens
 *                 (after RoPE and rotation; softmax-invariant); 0: no smoothing.
 * Outputs (device; code nibbles are two's complement, element 2i in the low
 * nibble of byte i, element 2i+1 in the high nibble):
 *   q_codes, k_codes  u8 [B,H,Np,D/2]   symmetric codes in [-7, 7]
 *   q_scale, k_scale  f32 [B,H,Np/qk_blk]  amax/7 of each qk_blk-token block
 *   v_codes           u8 [B,H,D,Np/2]   V transposed (token pairs per byte),
 *                                       codes in [-7, 7]
 *   v_scale           f32 [B,H,D]       per-channel amax/7 over all N tokens
 *   v_colsum          i32 [B,H,ceil(N/kv_blk),D] or NULL: per kv block sums of V
 *                                       codes, the zero-point term of P~ V for a
 *                                       caller that dequantises P~ V itself
 *                                       (rotattn_int4_attention does not read it:
 *                                       its P operand is P~ + 8)
 * Binary32 op order (bit-reproducible): RoPE u = fma(a,c,-(b*s)), v = fma(a,s,b*c);
 * fused Interleaved o0 = fma(a,al,b*be), o1 = fma(a,be,-(b*al)); Half
 * o0 = (x1+x2)*r, o1 = (x1-x2)*r with r = (float)(1/sqrt2); Full (ablation): plain
 * RoPE, then for stride len = 1, 2, ..., D/2 every pair (x[i], x[i+len]) with
 * i & len == 0 becomes (x[i]+x[i+len], x[i]-x[i+len]), then x * fl(1/sqrt(D));
 * K mean = binary64 sum
 * of in-order 64-token partial sums, in block order, / N, rounded to binary32;
 * code = clamp(rint(x * (7/amax)), -7, 7), scale = amax/7 (IEEE division);
 * amax == 0 gives scale 0 and codes 0.
 * workspace: device, >= rotattn_quantize_qk_workspace(s) bytes, scratch of the call
 * (calls that may run at the same time need workspaces of their own). */
size_t rotattn_quantize_qk_workspace(const rotattn_shape* s);
rotattn_status rotattn_quantize_qk(const rotattn_shape* s, rotattn_rot rot, rotattn_dtype in_dtype,
                                   const void* q, const void* k, const void* v,
                                   const float* rope_table, int32_t smooth_k,
                                   uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
                                   uint8_t* v_codes, float* v_scale, int32_t* v_colsum,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ---- rotattn_quantize_qk_noalloc: for callers that cannot allocate ---------------
 * For code that must not allocate device memory (work under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): rotattn_quantize_qk with
 * the same arguments and results, minus the workspace.  Its scratch (the ordered
 * binary64 partial sums of K, the channel means and the V amax) lives in a fixed
 * device array of rotattn_quantize_qk_noalloc_max_scratch() bytes (64 MiB) that the
 * library holds on every device it runs on until the process ends; the call itself
 * allocates nothing (no hipMalloc, no allocating library routine).  A shape whose
 * scratch, rotattn_quantize_qk_noalloc_scratch(s) (about 8 D bytes per token and
 * head: the Wan-720p-like layer needs 48.5 MB), exceeds it returns
 * ROTATTN_E_WORKSPACE before any launch.  Every call on a device shares that
 * device's array, and each call overwrites it (what must start at zero is cleared
 * by the call's own kernels): calls that overlap on one device, on different
 * streams or threads, race and must be serialised by the caller.  The first call
 * on each device looks up the array's device address (hipGetSymbolAddress) and keeps
 * it; a failed lookup returns ROTATTN_E_HIP. */
size_t rotattn_quantize_qk_noalloc_max_scratch(void);
size_t rotattn_quantize_qk_noalloc_scratch(const rotattn_shape* s);
rotattn_status rotattn_quantize_qk_noalloc(const rotattn_shape* s, rotattn_rot rot, rotattn_dtype in_dtype,
                                           const void* q, const void* k, const void* v,
                                           const float* rope_table, int32_t smooth_k,
                                           uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
                                           uint8_t* v_codes, float* v_scale, int32_t* v_colsum, void* stream);

/* ---- rotattn_quantize_qk_ex: Q smoothing, variable-length batches ----------------
 * rotattn_quantize_qk with options (opts NULL: smooth_k = 1 and nothing else):
 *   smooth_k   as rotattn_quantize_qk.
 *   smooth_q   1: Q smoothing as well, the other reading of the framework's channel
 *              smoothing (papernotes note, Overall framework), as an accuracy
 *              option.  mu_q (the per-(b,h) channel mean of the rotated Q, formed
 *              like the K mean) is subtracted from Q before it is quantised.
 *              Unlike the K mean it does not cancel in softmax: it leaves the
 *              per-key score term dS_j = mu_q . K_j (K_j as quantised: rotated, and
 *              smoothed when smooth_k), written to k_bias.
 *   k_bias     device f32 [B,H,Np], required with smooth_q (ROTATTN_E_NULL
 *              otherwise): the binary64 sum over the channels in order of the
 *              exact products mu_q[d] K_j[d], rounded to binary32; 0 for tokens
 *              that do not exist.  Pass it to rotattn_int4_attention_ex, which
 *              adds it back to every score.
 *   seq_lens   NULL, or host int32 [B] in [1, N]: a variable-length batch in the
 *              padded layout.  Batch element b has seq_lens[b] tokens (at the
 *              positions of the full F x Hs x Ws grid); every mean, amax, scale
 *              block and code uses those only (the means divide by seq_lens[b]),
 *              tokens past them are never read, and their codes, scale blocks,
 *              column sums and k_bias entries are 0.  B > 64 returns
 *              ROTATTN_E_UNSUPPORTED; a length outside [1, N] ROTATTN_E_ARG.
 * The pages name neither option; both are readings stated with the design. */
typedef struct {
  int32_t smooth_k;
  int32_t smooth_q;
  float* k_bias;
  const int32_t* seq_lens;
} rotattn_quantize_opts;

rotattn_status rotattn_quantize_qk_ex(const rotattn_shape* s, rotattn_rot rot, rotattn_dtype in_dtype,
                                      const void* q, const void* k, const void* v,
                                      const float* rope_table, const rotattn_quantize_opts* opts,
                                      uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
                                      uint8_t* v_codes, float* v_scale, int32_t* v_colsum,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- rotattn_int4_attention -----------------------------------------------------
 * INT4 FlashAttention forward (framework flowchart; Key design 2).  For each query
 * row i and online-softmax step s of kv_blk keys:
 *   a_ij = sum_d qc_id kc_jd (exact integer)
 *   c_ij = fl(fl(sq_i sk_j) C0), C0 = fl(log2(e)/sqrt(D)); t_ij = fl(a_ij c_ij)
 *   m_s  = max(m_{s-1}, max_j t_ij)
 *   y_ij = fma(a_ij, c_ij, fl(L15 - m_s)),  L15 = fl(log2 15)
 *   r_ij = round-half-even(2^y_ij) clamped to [0, 15], decided exactly;
 *          P code P~ = r - 8 in [-8, 7]  (fixed scale 15, zero point -8)
 *   l    = 2^(m_{s-1}-m_s) l + sum_j 2^y_ij       (unquantised P)
 *   O_d  = 2^(m_{s-1}-m_s) O_d + sv_d sum_j (P~_ij + 8) vc_jd
 *   out  = O / l.
 * The rotation mode is not needed: an orthogonal R cancels in Q K^T.
 * Work whose result is exactly nothing is skipped: 32-key tile pairs whose every
 * level r is 0 add no P V products, and tiles whose every 2^y is below half an ulp
 * of the running l would not change it.  The output is bit-identical to the dense
 * evaluation, which the debug run performs (it skips nothing and dumps every code).
 *   heads/n_heads  host list of flat head ids b*H + h to compute; NULL = all.  A
 *                  repeated id is computed once per listing, each time writing the
 *                  same values.
 *   out_dtype      F32, F16 or BF16 (round to nearest even); out device [B,H,N,D];
 *                  rows of heads not listed are left untouched.
 *   dbg            NULL in production.  Otherwise a debug run for rows
 *                  [row0, row0+n_rows) of head `bh` only, writing (device):
 *                  a_qk [n_rows][N] i32, p_codes [n_rows][N] i8 (P~),
 *                  a_pv [n_rows][S][D] i32 with S = ceil(N/kv_blk) (per-step
 *                  sum_j (P~+8) vc), m [n_rows] f32, l [n_rows] f32.  The output
 *                  rows are written as well.
 *   workspace      device, >= rotattn_int4_attention_workspace(s) bytes, 16-byte
 *                  aligned: per head and 128-key group (32 keys for kv_blk 16), the
 *                  listed heads' K and V codes restaged as the LDS image of fp6 K
 *                  rows and fp8 V^T rows (36 KiB per 128 keys for D = 128, about
 *                  288 bytes per padded token and head).  Contents need no
 *                  initialisation, and it is scratch of the call (calls that may
 *                  run at the same time need workspaces of their own); a smaller
 *                  size returns ROTATTN_E_WORKSPACE before any launch.  Shapes whose images
 *                  exceed 2^31 bytes per head (N beyond about 6.7 million tokens)
 *                  return ROTATTN_E_UNSUPPORTED. */
typedef struct {
  int32_t bh, row0, n_rows;
  int32_t* a_qk;
  int8_t* p_codes;
  int32_t* a_pv;
  float* m;
  float* l;
} rotattn_debug;

size_t rotattn_int4_attention_workspace(const rotattn_shape* s);
rotattn_status rotattn_int4_attention(const rotattn_shape* s,
                                      const uint8_t* q_codes, const float* q_scale,
                                      const uint8_t* k_codes, const float* k_scale,
                                      const uint8_t* v_codes, const float* v_scale,
                                      const int32_t* heads, int32_t n_heads,
                                      rotattn_dtype out_dtype, void* out,
                                      const rotattn_debug* dbg,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- rotattn_fp16_fallback ------------------------------------------------------
 * Full-precision fallback for sensitive heads / denoising steps (Key design 3):
 * out = softmax(RoPE(Q) RoPE(K)^T / sqrt(D)) V with binary16 MFMA operands and
 * binary32 softmax and accumulation.  RoPE'd Q, K are rounded to binary16.
 *   in_dtype   F32, F16 or BF16 (Q, K after RoPE and V are rounded to binary16).
 *   out_dtype  F32, F16 or BF16.
 *   rope_table plain (cos, sin) table: rotattn_build_rope_table(s, NONE, ...).
 *   heads      as above.
 *   workspace  device, >= rotattn_fp16_fallback_workspace(s) bytes: RoPE'd binary16
 *              Q, then per head and 64-key group the LDS image of K and V^T (36 KiB
 *              per 64 keys for D = 128, 20 KiB for D = 64); scratch of the call.
 *              Shapes whose images exceed 2^31 bytes per head (N beyond about 3.7
 *              million tokens for D = 128) return ROTATTN_E_UNSUPPORTED. */
size_t rotattn_fp16_fallback_workspace(const rotattn_shape* s);
rotattn_status rotattn_fp16_fallback(const rotattn_shape* s, rotattn_dtype in_dtype,
                                     const void* q, const void* k, const void* v,
                                     const float* rope_table,
                                     const int32_t* heads, int32_t n_heads,
                                     rotattn_dtype out_dtype, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---- rotattn_int4_attention_symmetric_p ------------------------------------------
 * Ablation baseline, not the method: the same INT4 attention with the symmetric
 * INT4 P code the pages argue against (papernotes note, Key design 2: a symmetric
 * code round(P / max P * 7) uses only [0, 7], wasting the negative half of INT4).
 * Identical to rotattn_int4_attention except L15 -> fl(log2 7): r_ij = round-half-
 * even(7 P_ij) in [0, 7], the code is r itself (debug p_codes hold r), and
 * l = sum_j 7 P_ij.  Arguments, layouts, workspace and errors as there. */
rotattn_status rotattn_int4_attention_symmetric_p(const rotattn_shape* s,
                                                  const uint8_t* q_codes, const float* q_scale,
                                                  const uint8_t* k_codes, const float* k_scale,
                                                  const uint8_t* v_codes, const float* v_scale,
                                                  const int32_t* heads, int32_t n_heads,
                                                  rotattn_dtype out_dtype, void* out,
                                                  const rotattn_debug* dbg,
                                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---- options: block-causal masks, the P code, the Q-smoothing term ---------------
 * Block-causal attention: the pages name causal as well as bidirectional attention
 * for video DiTs without fixing its granularity (papernotes note, Overall
 * framework).  A causal block size c lets query token i see key j iff j / c <= i / c
 * (integer division), i.e. the keys [0, min(N, (i / c + 1) c)); absent keys take no
 * part in the running maximum, in l or in O.  c = 0 is bidirectional; c = 1
 * token-causal; c = Hs * Ws frame-causal (a frame sees itself and the frames before
 * it); c >= N is bidirectional.  c < 0 returns ROTATTN_E_ARG.
 *   p_max         0 or 15: range-rectified P (the method); 7: the symmetric
 *                 baseline (as rotattn_int4_attention_symmetric_p); other values
 *                 return ROTATTN_E_ARG.
 *   causal_block  c as above.
 *   k_bias        NULL, or device f32 [B,H,Np] from rotattn_quantize_qk_ex with
 *                 smooth_q: every score gains delta_j = fl(k_bias_j * C0) in log2
 *                 units, t_ij = fma(a_ij, c_ij, delta_j), y_ij = fl(t_ij + fl(L15 - m_s)).
 *   seq_lens      NULL, or host int32 [B] in [1, N] (the lengths the codes were made
 *                 with): a row of batch element b sees only its first seq_lens[b]
 *                 keys, and its rows past them are left untouched (debug rows must
 *                 lie below it).  B > 64 returns ROTATTN_E_UNSUPPORTED.
 *   skip_stats    NULL, or device u64 [5], 8-byte aligned, that the run adds its
 *                 counts of the exact skips to (the caller clears it; a kernel
 *                 instance that also counts runs, with the same decisions):
 *                 [0] P V units (one P V MFMA decision: 64 keys x 32 rows, or 32
 *                 keys for kv_blk <= 32), [1] those skipped because every level is
 *                 0, [2] 32 x 32 score tiles, [3] tiles whose exps were skipped as
 *                 below half an ulp of l, [4] units whose levels took the exact
 *                 threshold path.  The counts depend on the data, not on timing.
 * Debug dumps leave the entries of keys a row does not see, and its steps past the
 * query tile's last key, unwritten: fill them first to compare whole arrays.
 * opts NULL is all defaults.  Every other argument, layout, workspace and error as
 * rotattn_int4_attention. */
typedef struct {
  int32_t p_max;
  int32_t causal_block;
  const float* k_bias;
  const int32_t* seq_lens;
  uint64_t* skip_stats;
} rotattn_attention_opts;

rotattn_status rotattn_int4_attention_ex(const rotattn_shape* s,
                                         const uint8_t* q_codes, const float* q_scale,
                                         const uint8_t* k_codes, const float* k_scale,
                                         const uint8_t* v_codes, const float* v_scale,
                                         const int32_t* heads, int32_t n_heads,
                                         const rotattn_attention_opts* opts,
                                         rotattn_dtype out_dtype, void* out,
                                         const rotattn_debug* dbg,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* The FP16 fallback with options (opts NULL: rotattn_fp16_fallback): a causal
 * block c and variable-length batches, both as above (tokens past seq_lens[b] are
 * never read; their output rows are left untouched). */
typedef struct {
  int32_t causal_block;
  const int32_t* seq_lens;
} rotattn_fallback_opts;

rotattn_status rotattn_fp16_fallback_ex(const rotattn_shape* s, rotattn_dtype in_dtype,
                                        const void* q, const void* k, const void* v,
                                        const float* rope_table,
                                        const int32_t* heads, int32_t n_heads,
                                        const rotattn_fallback_opts* opts,
                                        rotattn_dtype out_dtype, void* out,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ---- rotattn_p_level_probe: the P level decision of rotattn_int4_attention -----
 * For tests of the level function (Key design 2: r = round-half-even(15 P), written
 * with y = log2(15 P) as r = round-half-even(2^y) in [0, 15]).  For the binary32
 * exponents y_i whose bit patterns are first_bits + i, i < n, writes (device u8)
 *   out[i] = r_i | (x_i << 4)
 * where r_i is the level as the attention decides it for a key (the hardware-exp2
 * level when its rounding margin is clear, else the exact threshold fix) and x_i
 * the exact threshold fix alone (the attention applies it to every key of a unit
 * with any unclear margin).  Both must equal round-half-even(2^y_i) for every y the
 * attention forms, i.e. y up to L15 + 2^-5.  first_bits + n > 2^32 or n < 0 returns
 * ROTATTN_E_ARG. */
rotattn_status rotattn_p_level_probe(uint32_t first_bits, int64_t n, uint8_t* out, void* stream);

const char* rotattn_status_str(rotattn_status st);

#ifdef __cplusplus
}
#endif
#endif /* ROTATTN_H_ */
