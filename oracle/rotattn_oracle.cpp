// rotattn CPU oracle -- TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, obviously-correct CPU implementation of what the RotateAttention
// hot path computes.  Only the test suite, the smoke check and the benchmark's
// CPU-baseline leg may load it; the product library never does.  It shares no
// code, header, table or constant generator with the GPU library.
//
// Sources (the RotateAttention pages, arXiv 2607.02584):
//   * papernotes.org note, "Key design 1" (RoPE-aware rotation): D = Df + Dh + Dw,
//     orthogonal 2x2 rotations, Interleaved rotation pre-multiplied into the RoPE
//     2x2 blocks (M' = R M), Half rotation QPiR pairing channel d with d + Dj/2.
//   * same note, "Key design 2" (range-rectified P): P = exp(S - m) in (0, 1],
//     code = round(15 P / max P) - 8 in [-8, 7] with fixed scale 15, zero point -8.
//   * same note, "Overall framework" flowchart: S = Q K^T / sqrt(D) on INT4 Q, K;
//     INT4 P V; smoothing of the projected tensors.
//   * arxivdaily abstract: P = exp(QK - max(QK)) is non-negative; fixed scales and
//     zero points; mixed-precision INT4 FlashAttention with FP16 fallback.
//   * the pages name causal as well as bidirectional attention for video DiTs
//     without fixing its granularity: the *_x entry points take a causal block
//     size c (key j visible to query i iff j / c <= i / c; c = 0 bidirectional),
//     and per-element valid lengths for a variable-length batch (seq_lens).
// Readings where the pages are silent (RoPE base, pair layout, block sizes, the
// normaliser, the exact exp) are listed in the design notes and restated at each
// function below.
//
// Build: g++ -O2 -std=c++17 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
// Every floating-point step that decides an integer code is done in IEEE binary32
// with explicit fmaf(), exactly as written; everything else is binary64.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <algorithm>
#include <limits>

namespace {

struct Shape {
  int B, H, F, Hs, Ws, D, Df, Dh, Dw, qk_blk, kv_blk;
  int64_t N() const { return (int64_t)F * Hs * Ws; }
};

Shape unpack(const int32_t* s) {
  return Shape{s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], s[8], s[9], s[10]};
}

constexpr int kMeanBlk = 64;            // tokens per ordered fp64 partial sum of K
constexpr double kInvSqrt2 = 0.70710678118654752440;

// --- 3D RoPE tables (Key design 1: RoPE is block-diagonal in 2x2 rotations) ----
// Axis j in {frame, height, width} owns Dj channels; pair i in [0, Dj/2) rotates by
// pos * theta_{j,i}, theta_{j,i} = base^(-2i/Dj).  Plain table holds (cos, sin);
// the Interleaved table holds the product H2 * Rot folded into (alpha, beta) with
// alpha = (c + s)/sqrt2, beta = (c - s)/sqrt2.  All in binary64, rounded once.
template <class T>
void build_table(const Shape& s, int rot, double base, T* out) {
  const int npos[3] = {s.F, s.Hs, s.Ws};
  const int dj[3] = {s.Df, s.Dh, s.Dw};
  for (int ax = 0; ax < 3; ++ax) {
    for (int p = 0; p < npos[ax]; ++p) {
      for (int i = 0; i < dj[ax] / 2; ++i) {
        double theta = std::pow(base, -(2.0 * i) / (double)dj[ax]);
        double ang = (double)p * theta;
        double c = std::cos(ang), sn = std::sin(ang);
        if (rot == 1) {
          *out++ = (T)((c + sn) * kInvSqrt2);
          *out++ = (T)((c - sn) * kInvSqrt2);
        } else {
          *out++ = (T)c;
          *out++ = (T)sn;
        }
      }
    }
  }
}

int64_t table_entries(const Shape& s) {
  return 2 * ((int64_t)s.F * (s.Df / 2) + (int64_t)s.Hs * (s.Dh / 2) + (int64_t)s.Ws * (s.Dw / 2));
}

inline float fmaT(float a, float b, float c) { return std::fmaf(a, b, c); }
inline double fmaT(double a, double b, double c) { return std::fma(a, b, c); }

// RoPE then the RoPE-aware rotation for one token (Key design 1).
//   rot 0: RoPE only.  rot 1: Interleaved (fused table, H2 on pairs (2i, 2i+1)).
//   rot 2: Half: RoPE, then per segment pair channel o+i with o+Dj/2+i and apply
//          H2, writing the pair to channels (o+2i, o+2i+1)  (the QPiR product).
//   rot 3: Full: RoPE, then the orthonormal D x D Walsh-Hadamard rotation of the
//          whole vector (the dense rotation the pages compare the Half one with,
//          papernotes "Key design 1" cost comparison; an ablation, not the method).
//          Fast Walsh-Hadamard transform: for stride len = 1, 2, 4, ..., D/2, every
//          pair (x[i], x[i+len]) with i & len == 0 becomes (x[i] + x[i+len],
//          x[i] - x[i+len]); then every channel times fl(1/sqrt(D)).
// binary32 op order:  u = fma(a, c, -(b*s)), v = fma(a, s, b*c);
//   fused: o0 = fma(a, al, b*be), o1 = fma(a, be, -(b*al));
//   half:  o0 = (x1 + x2) * r, o1 = (x1 - x2) * r, r = (float)(1/sqrt2).
template <class T>
void rope_rotate_token(const Shape& s, int rot, const T* tab, int64_t n, const T* in, T* out) {
  const int64_t f = n / ((int64_t)s.Hs * s.Ws);
  const int64_t yy = (n / s.Ws) % s.Hs;
  const int64_t xx = n % s.Ws;
  const int64_t pos[3] = {f, yy, xx};
  const int dj[3] = {s.Df, s.Dh, s.Dw};
  const int npos[3] = {s.F, s.Hs, s.Ws};
  const T r = (T)kInvSqrt2;
  std::vector<T> u(s.D);
  const T* axtab = tab;
  int off = 0;
  for (int ax = 0; ax < 3; ++ax) {
    const T* row = axtab + pos[ax] * dj[ax];  // (dj/2) pairs * 2 entries
    for (int i = 0; i < dj[ax] / 2; ++i) {
      const T a = in[off + 2 * i], b = in[off + 2 * i + 1];
      const T t0 = row[2 * i], t1 = row[2 * i + 1];
      if (rot == 1) {
        u[off + 2 * i] = fmaT(a, t0, b * t1);
        u[off + 2 * i + 1] = fmaT(a, t1, -(b * t0));
      } else {
        u[off + 2 * i] = fmaT(a, t0, -(b * t1));
        u[off + 2 * i + 1] = fmaT(a, t1, b * t0);
      }
    }
    if (rot == 2) {
      const int h = dj[ax] / 2;
      for (int i = 0; i < h; ++i) {
        const T x1 = u[off + i], x2 = u[off + h + i];
        out[off + 2 * i] = (x1 + x2) * r;
        out[off + 2 * i + 1] = (x1 - x2) * r;
      }
    } else if (rot != 3) {
      for (int i = 0; i < dj[ax]; ++i) out[off + i] = u[off + i];
    }
    axtab += (int64_t)npos[ax] * dj[ax];
    off += dj[ax];
  }
  if (rot == 3) {
    for (int len = 1; len < s.D; len *= 2)
      for (int i = 0; i < s.D; ++i)
        if ((i & len) == 0) {
          const T a = u[i], b = u[i + len];
          u[i] = a + b;
          u[i + len] = a - b;
        }
    const T rd = (T)(1.0 / std::sqrt((double)s.D));
    for (int i = 0; i < s.D; ++i) out[i] = u[i] * rd;
  }
}

// Symmetric INT4 quantisation of one block of qk_blk tokens x all channels (the
// signed symmetric INT4 quantiser of the papernotes.org note, "Key design 2"; one
// scale per block of tokens generalises the per-token Q/K scales of the
// paper.gecl.asia analysis, "Key Insight").
// amax over the block; amax == 0 -> scale 0, codes 0; else inv = 7/amax (IEEE
// division), code = clamp(rint(x * inv), -7, 7), scale = amax / 7.
void quant_block(const float* x, int64_t count, int8_t* code, float* scale) {
  float amax = 0.f;
  for (int64_t i = 0; i < count; ++i) amax = std::max(amax, std::fabs(x[i]));
  if (amax == 0.f) {
    for (int64_t i = 0; i < count; ++i) code[i] = 0;
    *scale = 0.f;
    return;
  }
  const float inv = 7.0f / amax;
  for (int64_t i = 0; i < count; ++i) {
    float v = std::nearbyintf(x[i] * inv);
    v = std::min(7.f, std::max(-7.f, v));
    code[i] = (int8_t)v;
  }
  *scale = amax / 7.0f;
}

// Thresholds of the range-rectified P code (Key design 2), decided in exact
// arithmetic on the binary32 exponent y' (the log2 of 15 * P):
//   r(y') = round-half-even(2^y') clamped to [0, 15];  code = r - 8.
// r >= k  <=>  y' >= T[k-1], with T[0] the smallest float above -1 (2^-1 = 0.5 is a
// tie that rounds to the even 0) and T[k-1] the smallest float above log2(k - 1/2)
// for k >= 2 (never a tie: k - 1/2 is not a power of two).  log2 is taken in the
// x87 extended format; the smallest float strictly above it is found by stepping.
struct Thresholds {
  float t[15];
  Thresholds() {
    t[0] = std::nextafterf(-1.0f, 1.0f);
    for (int k = 2; k <= 15; ++k) {
      long double L = log2l((long double)k - 0.5L);
      float f = (float)L;
      while (!((long double)f > L)) f = std::nextafterf(f, std::numeric_limits<float>::infinity());
      while ((long double)std::nextafterf(f, -std::numeric_limits<float>::infinity()) > L)
        f = std::nextafterf(f, -std::numeric_limits<float>::infinity());
      t[k - 1] = f;
    }
  }
};
const Thresholds& thresholds() {
  static Thresholds th;
  return th;
}
inline int p_level(float y) {
  const float* t = thresholds().t;
  int r = 0;
  for (int k = 0; k < 15; ++k) r += (y >= t[k]) ? 1 : 0;
  return r;
}

// Keys a query token sees.  cb = 0: all N (bidirectional).  cb > 0: block-causal
// with blocks of cb tokens -- token i sees key j iff j / cb <= i / cb (cb = 1 is
// token-causal, cb = Hs * Ws frame-causal); the pages name causal attention without
// fixing its granularity.
int64_t key_limit(int64_t i, int64_t N, int64_t cb) {
  if (cb <= 0) return N;
  return std::min(N, (i / cb + 1) * cb);
}

// Tokens of batch element b that exist: seq_lens[b] (a variable-length batch in the
// padded [B,H,N,D] layout; tokens past it are padding, read by nothing), else N.
int64_t valid_tokens(const int32_t* seq_lens, int64_t bh, int H, int64_t N) {
  return seq_lens ? (int64_t)seq_lens[bh / H] : N;
}

float c0_of(int D) { return (float)(1.4426950408889634074 / std::sqrt((double)D)); }
float l15() { return (float)std::log2(15.0); }

// float -> binary16 bits, round-half-even (for the fallback oracle's fp16 copy).
uint16_t f32_to_f16_bits(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u));
  const int e = (int)(ax >> 23) - 127;
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  uint32_t mant = (ax & 0x7fffffu) | 0x800000u;
  int shift;  // number of low bits of the 24-bit significand to drop
  uint32_t hexp;
  if (e >= -14) {
    shift = 13;
    hexp = (uint32_t)(e + 15);
  } else {
    if (e < -25) return (uint16_t)sign;
    shift = 13 + (-14 - e);
    hexp = 0;
  }
  uint32_t q = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  uint32_t bits;
  if (hexp == 0) {
    bits = q;  // subnormal (q may carry into the smallest normal, which is fine)
  } else {
    // q holds 1.mmmmmmmmmm (11 bits); a carry to 12 bits bumps the exponent
    if (q >> 11) { q >>= 1; ++hexp; }
    if (hexp >= 31) return (uint16_t)(sign | 0x7c00u);
    bits = (hexp << 10) | (q & 0x3ffu);
  }
  return (uint16_t)(sign | bits);
}
float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ffu;
  float v;
  if (e == 0) v = std::ldexp((float)m, -24);
  else if (e == 31) v = m ? std::numeric_limits<float>::quiet_NaN() : std::numeric_limits<float>::infinity();
  else v = std::ldexp((float)(m | 0x400u), (int)e - 25);
  uint32_t b;
  std::memcpy(&b, &v, 4);
  b |= sign;
  std::memcpy(&v, &b, 4);
  return v;
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
int64_t orc_table_entries(const int32_t* shp) { return table_entries(unpack(shp)); }

void orc_rope_table(const int32_t* shp, int32_t rot, double base, float* out) {
  build_table<float>(unpack(shp), rot, base, out);
}
void orc_rope_table_f64(const int32_t* shp, int32_t rot, double base, double* out) {
  build_table<double>(unpack(shp), rot, base, out);
}

// RoPE + rotation of whole [B,H,N,D] tensors (binary32 spec path).
void orc_rope_rotate(const int32_t* shp, int32_t rot, const float* tab, const float* x, float* out) {
  const Shape s = unpack(shp);
  const int64_t N = s.N(), rows = (int64_t)s.B * s.H * N;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    rope_rotate_token<float>(s, rot, tab, r % N, x + r * s.D, out + r * s.D);
}
// Same in binary64 with a binary64 table (for the orthogonality / invariance pins).
void orc_rope_rotate_f64(const int32_t* shp, int32_t rot, const double* tab, const double* x, double* out) {
  const Shape s = unpack(shp);
  const int64_t N = s.N(), rows = (int64_t)s.B * s.H * N;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    rope_rotate_token<double>(s, rot, tab, r % N, x + r * s.D, out + r * s.D);
}

// ---------------------------------------------------------------------------
// Fused quantisation (the framework flowchart: RoPE -> rotation -> smoothing ->
// INT4).  Inputs are float copies of the caller's tensors [B,H,N,D].
//   Q: RoPE + rotation, then per qk_blk-token block symmetric INT4.
//   K: RoPE + rotation, then (smooth_k) minus the per-(b,h) channel mean mu, then
//      per-block INT4.  mu_d = float( sum over 64-token blocks, in order, of the
//      in-order binary64 sum of the block, divided by N ).
//   V: no RoPE or rotation (its Hadamard is folded into the weights offline); one
//      scale per (b,h,d) channel over all N tokens, and per kv_blk block column
//      sums of the codes.
// Outputs (codes unpacked, one int8 per element):
//   qc, kc [B,H,N,D]; qs, ks [B,H,ceil(N/qk_blk)]; vc [B,H,N,D]; vs [B,H,D];
//   vcol [B,H,ceil(N/kv_blk),D].  Optional (nullable): q_rot, k_rot [B,H,N,D] (K
//   before smoothing), k_mu [B,H,D].
// flags: bit 0 smooths K as above.  Bit 1 smooths Q the same way (the other reading
//   of the framework's channel smoothing): Q' = Q - mu_q with mu_q formed like mu
//   over the rotated Q.  Unlike mu, mu_q does not cancel in softmax: it leaves the
//   per-key term dS_j = mu_q . K_j (K_j as quantised: rotated, and smoothed when
//   bit 0 is set), written to k_bias [B,H,N] as float(binary64 sum over channels in
//   order of the exact products).  The attention adds it back to every score.
//   q_mu [B,H,D] (nullable) receives mu_q.
// seq_lens (nullable, B entries in [1, N]): a variable-length batch.  Batch element b
//   has seq_lens[b] tokens (positions as in the full grid); every statistic, scale
//   block and code uses those tokens only, as if N were seq_lens[b], and the codes,
//   scale blocks, column sums and k_bias entries past it are 0.
void orc_quantize_x(const int32_t* shp, int32_t rot, const float* tab, int32_t flags,
                    const float* q, const float* k, const float* v,
                    int8_t* qc, float* qs, int8_t* kc, float* ks,
                    int8_t* vc, float* vs, int32_t* vcol,
                    float* q_rot, float* k_rot, float* k_mu, float* q_mu, float* k_bias,
                    const int32_t* seq_lens) {
  const int32_t smooth_k = flags & 1, smooth_q = flags & 2;
  const Shape s = unpack(shp);
  const int64_t N = s.N(), D = s.D;
  const int64_t nqb = (N + s.qk_blk - 1) / s.qk_blk;
  const int64_t nkb = (N + s.kv_blk - 1) / s.kv_blk;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < (int64_t)s.B * s.H; ++bh) {
    const int64_t Nb = valid_tokens(seq_lens, bh, s.H, N);
    std::vector<float> qr(N * D), kr(N * D);
    const float* qh = q + bh * N * D;
    const float* kh = k + bh * N * D;
    const float* vh = v + bh * N * D;
    for (int64_t n = 0; n < N; ++n) {
      rope_rotate_token<float>(s, rot, tab, n, qh + n * D, qr.data() + n * D);
      rope_rotate_token<float>(s, rot, tab, n, kh + n * D, kr.data() + n * D);
    }
    if (q_rot) std::memcpy(q_rot + bh * N * D, qr.data(), sizeof(float) * N * D);
    if (k_rot) std::memcpy(k_rot + bh * N * D, kr.data(), sizeof(float) * N * D);
    // channel mean: binary64 sums of 64-token blocks, added in block order, / Nb
    auto channel_mean = [&](const std::vector<float>& x, int64_t d) {
      double total = 0.0;
      for (int64_t b0 = 0; b0 < Nb; b0 += kMeanBlk) {
        double part = 0.0;
        for (int64_t n = b0; n < std::min(Nb, b0 + kMeanBlk); ++n) part += (double)x[n * D + d];
        total += part;
      }
      return (float)(total / (double)Nb);
    };
    if (smooth_k) {
      for (int64_t d = 0; d < D; ++d) {
        const float mu = channel_mean(kr, d);
        if (k_mu) k_mu[bh * D + d] = mu;
        for (int64_t n = 0; n < Nb; ++n) kr[n * D + d] = kr[n * D + d] - mu;
      }
    } else if (k_mu) {
      for (int64_t d = 0; d < D; ++d) k_mu[bh * D + d] = 0.f;
    }
    if (smooth_q) {
      std::vector<float> muq(D);
      for (int64_t d = 0; d < D; ++d) {
        muq[d] = channel_mean(qr, d);
        if (q_mu) q_mu[bh * D + d] = muq[d];
        for (int64_t n = 0; n < Nb; ++n) qr[n * D + d] = qr[n * D + d] - muq[d];
      }
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;  // each product of two binary32 values is exact in binary64
        for (int64_t d = 0; d < D; ++d) acc += (double)muq[d] * (double)kr[n * D + d];
        k_bias[bh * N + n] = n < Nb ? (float)acc : 0.f;
      }
    } else if (q_mu) {
      for (int64_t d = 0; d < D; ++d) q_mu[bh * D + d] = 0.f;
    }
    for (int64_t b = 0; b < nqb; ++b) {
      const int64_t n0 = b * s.qk_blk, full = std::min<int64_t>(s.qk_blk, N - n0);
      const int64_t cnt = std::max<int64_t>(0, std::min<int64_t>(full, Nb - n0));
      std::fill(qc + (bh * N + n0) * D, qc + (bh * N + n0 + full) * D, (int8_t)0);
      std::fill(kc + (bh * N + n0) * D, kc + (bh * N + n0 + full) * D, (int8_t)0);
      quant_block(qr.data() + n0 * D, cnt * D, qc + (bh * N + n0) * D, qs + bh * nqb + b);
      quant_block(kr.data() + n0 * D, cnt * D, kc + (bh * N + n0) * D, ks + bh * nqb + b);
    }
    // V: per-channel scale over all tokens, then per-kv-block column sums.
    for (int64_t d = 0; d < D; ++d) {
      float amax = 0.f;
      for (int64_t n = 0; n < Nb; ++n) amax = std::max(amax, std::fabs(vh[n * D + d]));
      const float inv = amax == 0.f ? 0.f : 7.0f / amax;
      vs[bh * D + d] = amax == 0.f ? 0.f : amax / 7.0f;
      for (int64_t n = 0; n < N; ++n) {
        int8_t c = 0;
        if (amax != 0.f && n < Nb) {
          float t = std::nearbyintf(vh[n * D + d] * inv);
          c = (int8_t)std::min(7.f, std::max(-7.f, t));
        }
        vc[(bh * N + n) * D + d] = c;
      }
      for (int64_t sb = 0; sb < nkb; ++sb) {
        int32_t acc = 0;
        for (int64_t n = sb * s.kv_blk; n < std::min(N, (sb + 1) * s.kv_blk); ++n) acc += vc[(bh * N + n) * D + d];
        vcol[(bh * nkb + sb) * D + d] = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// P-code helpers (Key design 2).
void orc_p_thresholds(float* out15) { std::memcpy(out15, thresholds().t, sizeof(float) * 15); }
void orc_p_levels(const float* y, int64_t n, int8_t* r) {
  for (int64_t i = 0; i < n; ++i) r[i] = (int8_t)p_level(y[i]);
}
float orc_c0(int32_t D) { return c0_of(D); }
float orc_l15() { return l15(); }

// Brute force over every binary32 y with |y| in [lo, hi] (both signs): compare
// the threshold-decided level with rint(exp2((double)y)) (clamped to 15).  binary64
// exp2 is within 1 ulp of 2^y, far closer than any float y to a rounding boundary,
// so this is an independent evaluation of round-half-even(2^y).  Returns the
// number of mismatches; the first mismatch (if any) goes to *first.
int64_t orc_p_level_bruteforce(float lo, float hi, float* first) {
  int64_t bad = 0;
  uint32_t blo, bhi;
  std::memcpy(&blo, &lo, 4);
  std::memcpy(&bhi, &hi, 4);
  for (int sgn = 0; sgn < 2; ++sgn) {
    for (uint32_t b = blo; b <= bhi; ++b) {
      uint32_t bb = b | (sgn ? 0x80000000u : 0u);
      float y;
      std::memcpy(&y, &bb, 4);
      double e = std::exp2((double)y);
      double r = std::nearbyint(e);
      if (r > 15.0) r = 15.0;
      if ((int)r != p_level(y)) {
        if (bad == 0 && first) *first = y;
        ++bad;
      }
    }
  }
  return bad;
}

// ---------------------------------------------------------------------------
// Quantised attention, one query row at a time (framework flowchart + Key design 2).
// For row i of head (b,h), KV steps s of kv_blk keys (keys >= N do not exist):
//   a_ij  = sum_d qc_id kc_jd                          (exact integer)
//   c_ij  = fl(fl(sq_i * sk_j) * C0),  C0 = fl(log2(e)/sqrt(D))
//   t_ij  = fl(a_ij * c_ij)                             (score in log2 units)
//   m_s   = max(m_{s-1}, max_j t_ij),  m_{-1} = -inf    (running row max)
//   y'_ij = fma(a_ij, c_ij, fl(L15 - m_s)),  L15 = fl(log2 15)
//   r_ij  = round-half-even(2^y') clamped to [0,15]  -> code P~ = r - 8 in [-8, 7]
//   p_ij  = 2^y'  (= 15 exp(S - m), binary64; the normaliser uses the unquantised P)
//   l     = 2^(m_{s-1}-m_s) l + sum_j p_ij
//   O_d   = 2^(m_{s-1}-m_s) O_d + sv_d * sum_j r_ij vc_jd      (zero point folded in)
//   out   = O / l.
// Optional dumps: a_qk [rows][N] int32, pcode [rows][N] int8 (P~),
// a_pv [rows][S][D] int32 (per-step sum_j r_ij vc_jd), m_out [rows] f32, l_out.
//
// pmax = 7 gives the symmetric-P baseline the pages argue against (papernotes,
// "Key design 2": code = round(P / max P * 7) in [0, 7], which leaves the negative
// half of INT4 unused): the same steps with L = fl(log2 7) in place of L15, so
// r = round-half-even(7 P) in [0, 7], and the code is r itself (no zero point).
// causal_block: see key_limit(); keys at or beyond the row's limit do not exist for
// it (no score, no code, nothing in m, l or O; their dump entries are not written).
// k_bias (nullable, [B,H,N] binary32): the per-key term dS_j that Q smoothing
// leaves (orc_quantize_x).  With it every score gains delta_j = fl(dS_j * C0):
//   t_ij = fma(a_ij, c_ij, delta_j),  y'_ij = fl(t_ij + fl(L15 - m_s)),
// the rest unchanged.
// seq_lens (nullable): a variable-length batch; a row of batch element b sees only
// the first seq_lens[b] keys (its rows past that are not meaningful to ask for).
void orc_attention_x(const int32_t* shp, const int8_t* qc, const float* qs,
                     const int8_t* kc, const float* ks, const int8_t* vc, const float* vs,
                     const int64_t* rows, int64_t n_rows, double* out,
                     int32_t* a_qk, int8_t* pcode, int32_t* a_pv, float* m_out, double* l_out, int32_t pmax,
                     int32_t causal_block, const float* k_bias, const int32_t* seq_lens) {
  const Shape s = unpack(shp);
  const int64_t N = s.N(), D = s.D;
  const int64_t nqb = (N + s.qk_blk - 1) / s.qk_blk;
  const int64_t S = (N + s.kv_blk - 1) / s.kv_blk;
  const float C0 = c0_of(s.D), L15 = pmax == 7 ? (float)std::log2(7.0) : l15();
  const int zp = pmax == 7 ? 0 : 8;
#pragma omp parallel for schedule(dynamic)
  for (int64_t ri = 0; ri < n_rows; ++ri) {
    const int64_t row = rows[ri];
    const int64_t bh = row / N, i = row % N;
    const int64_t lim = key_limit(i, valid_tokens(seq_lens, bh, s.H, N), causal_block);
    const int8_t* qrow = qc + (bh * N + i) * D;
    const float sq = qs[bh * nqb + i / s.qk_blk];
    std::vector<int32_t> a(s.kv_blk);
    std::vector<float> c(s.kv_blk), tv(s.kv_blk);
    std::vector<double> O(D, 0.0);
    std::vector<int64_t> acc(D);
    float m = -std::numeric_limits<float>::infinity();
    double l = 0.0;
    for (int64_t st = 0; st < S; ++st) {
      const int64_t j0 = st * s.kv_blk, j1 = std::min(lim, j0 + s.kv_blk);
      if (j0 >= lim) {  // a step with no key for this row: nothing changes
        if (a_pv)
          for (int64_t d = 0; d < D; ++d) a_pv[(ri * S + st) * D + d] = 0;
        continue;
      }
      float mnew = m;
      for (int64_t j = j0; j < j1; ++j) {
        const int8_t* krow = kc + (bh * N + j) * D;
        int64_t dot = 0;
        for (int64_t d = 0; d < D; ++d) dot += (int64_t)qrow[d] * krow[d];
        a[j - j0] = (int32_t)dot;
        const float sk = ks[bh * nqb + j / s.qk_blk];
        const float cc = (sq * sk) * C0;
        c[j - j0] = cc;
        const float t = k_bias ? std::fmaf((float)a[j - j0], cc, k_bias[bh * N + j] * C0) : (float)a[j - j0] * cc;
        tv[j - j0] = t;
        mnew = std::max(mnew, t);
        if (a_qk) a_qk[ri * N + j] = a[j - j0];
      }
      const float nm = L15 - mnew;
      const double alpha = std::isinf(m) ? 0.0 : std::exp2((double)m - (double)mnew);
      l *= alpha;
      for (int64_t d = 0; d < D; ++d) O[d] *= alpha;
      std::fill(acc.begin(), acc.end(), 0);
      for (int64_t j = j0; j < j1; ++j) {
        const float y = k_bias ? tv[j - j0] + nm : std::fmaf((float)a[j - j0], c[j - j0], nm);
        const int r = p_level(y);
        if (pcode) pcode[ri * N + j] = (int8_t)(r - zp);
        l += std::exp2((double)y);
        const int8_t* vrow = vc + (bh * N + j) * D;
        for (int64_t d = 0; d < D; ++d) acc[d] += (int64_t)r * vrow[d];
      }
      for (int64_t d = 0; d < D; ++d) {
        if (a_pv) a_pv[(ri * S + st) * D + d] = (int32_t)acc[d];
        O[d] += (double)vs[bh * D + d] * (double)acc[d];
      }
      m = mnew;
    }
    for (int64_t d = 0; d < D; ++d) out[ri * D + d] = O[d] / l;
    if (m_out) m_out[ri] = m;
    if (l_out) l_out[ri] = l;
  }
}

void orc_attention_p(const int32_t* shp, const int8_t* qc, const float* qs,
                     const int8_t* kc, const float* ks, const int8_t* vc, const float* vs,
                     const int64_t* rows, int64_t n_rows, double* out,
                     int32_t* a_qk, int8_t* pcode, int32_t* a_pv, float* m_out, double* l_out, int32_t pmax) {
  orc_attention_x(shp, qc, qs, kc, ks, vc, vs, rows, n_rows, out, a_qk, pcode, a_pv, m_out, l_out, pmax, 0,
                  nullptr, nullptr);
}

void orc_attention(const int32_t* shp, const int8_t* qc, const float* qs,
                   const int8_t* kc, const float* ks, const int8_t* vc, const float* vs,
                   const int64_t* rows, int64_t n_rows, double* out,
                   int32_t* a_qk, int8_t* pcode, int32_t* a_pv, float* m_out, double* l_out) {
  orc_attention_x(shp, qc, qs, kc, ks, vc, vs, rows, n_rows, out, a_qk, pcode, a_pv, m_out, l_out, 15, 0,
                  nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// Unquantised attention in binary64 for the listed rows:
//   out = softmax(RoPE(Q) RoPE(K)^T / sqrt(D)) V, RoPE with a binary64 table.
// (The rotation is orthogonal and cancels in Q K^T, so none is applied.)
void orc_exact_attention_x(const int32_t* shp, const double* tab64_plain,
                           const float* q, const float* k, const float* v,
                           const int64_t* rows, int64_t n_rows, double* out, int32_t causal_block,
                           const int32_t* seq_lens) {
  const Shape s = unpack(shp);
  const int64_t N = s.N(), D = s.D;
  // RoPE every K row of the heads that appear, lazily per head.
  std::vector<int64_t> heads;
  for (int64_t r = 0; r < n_rows; ++r) heads.push_back(rows[r] / N);
  std::sort(heads.begin(), heads.end());
  heads.erase(std::unique(heads.begin(), heads.end()), heads.end());
  for (int64_t bh : heads) {
    std::vector<double> kr(N * D), tmp(D);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      std::vector<double> in(D);
      for (int64_t d = 0; d < D; ++d) in[d] = k[(bh * N + n) * D + d];
      rope_rotate_token<double>(s, 0, tab64_plain, n, in.data(), kr.data() + n * D);
    }
    std::vector<int64_t> mine;
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] / N == bh) mine.push_back(r);
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < (int64_t)mine.size(); ++t) {
      const int64_t r = mine[t], i = rows[r] % N;
      std::vector<double> in(D), qr(D), sc(N);
      const int64_t lim = key_limit(i, valid_tokens(seq_lens, bh, s.H, N), causal_block);
      for (int64_t d = 0; d < D; ++d) in[d] = q[(bh * N + i) * D + d];
      rope_rotate_token<double>(s, 0, tab64_plain, i, in.data(), qr.data());
      double mx = -std::numeric_limits<double>::infinity();
      const double inv = 1.0 / std::sqrt((double)D);
      for (int64_t j = 0; j < lim; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qr[d] * kr[j * D + d];
        sc[j] = dot * inv;
        mx = std::max(mx, sc[j]);
      }
      double den = 0.0;
      std::vector<double> num(D, 0.0);
      for (int64_t j = 0; j < lim; ++j) {
        const double p = std::exp(sc[j] - mx);
        den += p;
        for (int64_t d = 0; d < D; ++d) num[d] += p * (double)v[(bh * N + j) * D + d];
      }
      for (int64_t d = 0; d < D; ++d) out[r * D + d] = num[d] / den;
    }
  }
}

// ---------------------------------------------------------------------------
// Oracle of the FP16 fallback (Key design 3, selective FP16 fallback):
// RoPE in binary32 with the plain table (same op order as above), the RoPE'd Q and
// K rounded to binary16 (round-half-even), then exact binary64 softmax attention
// with V as given.  The fallback kernel also rounds P to binary16 inside; that
// rounding is covered by the tolerance, not mirrored here.
void orc_fallback_attention_x(const int32_t* shp, const float* tab_plain,
                              const float* q, const float* k, const float* v,
                              const int64_t* rows, int64_t n_rows, double* out, int32_t causal_block,
                              const int32_t* seq_lens) {
  const Shape s = unpack(shp);
  const int64_t N = s.N(), D = s.D;
  std::vector<int64_t> heads;
  for (int64_t r = 0; r < n_rows; ++r) heads.push_back(rows[r] / N);
  std::sort(heads.begin(), heads.end());
  heads.erase(std::unique(heads.begin(), heads.end()), heads.end());
  auto to_half = [](float x) { return f16_bits_to_f32(f32_to_f16_bits(x)); };
  for (int64_t bh : heads) {
    std::vector<float> kr(N * D);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      rope_rotate_token<float>(s, 0, tab_plain, n, k + (bh * N + n) * D, kr.data() + n * D);
      for (int64_t d = 0; d < D; ++d) kr[n * D + d] = to_half(kr[n * D + d]);
    }
    std::vector<int64_t> mine;
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] / N == bh) mine.push_back(r);
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < (int64_t)mine.size(); ++t) {
      const int64_t r = mine[t], i = rows[r] % N;
      std::vector<float> qr(D);
      std::vector<double> sc(N);
      const int64_t lim = key_limit(i, valid_tokens(seq_lens, bh, s.H, N), causal_block);
      rope_rotate_token<float>(s, 0, tab_plain, i, q + (bh * N + i) * D, qr.data());
      for (int64_t d = 0; d < D; ++d) qr[d] = to_half(qr[d]);
      double mx = -std::numeric_limits<double>::infinity();
      const double inv = 1.0 / std::sqrt((double)D);
      for (int64_t j = 0; j < lim; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qr[d] * (double)kr[j * D + d];
        sc[j] = dot * inv;
        mx = std::max(mx, sc[j]);
      }
      double den = 0.0;
      std::vector<double> num(D, 0.0);
      for (int64_t j = 0; j < lim; ++j) {
        const double p = std::exp(sc[j] - mx);
        den += p;
        for (int64_t d = 0; d < D; ++d) num[d] += p * (double)v[(bh * N + j) * D + d];
      }
      for (int64_t d = 0; d < D; ++d) out[r * D + d] = num[d] / den;
    }
  }
}

// binary16 round trip (exposed for the pins).
void orc_f32_to_f16(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_bits(x[i]);
}

void orc_exact_attention(const int32_t* shp, const double* tab64_plain, const float* q, const float* k,
                         const float* v, const int64_t* rows, int64_t n_rows, double* out) {
  orc_exact_attention_x(shp, tab64_plain, q, k, v, rows, n_rows, out, 0, nullptr);
}

void orc_fallback_attention(const int32_t* shp, const float* tab_plain, const float* q, const float* k,
                            const float* v, const int64_t* rows, int64_t n_rows, double* out) {
  orc_fallback_attention_x(shp, tab_plain, q, k, v, rows, n_rows, out, 0, nullptr);
}

void orc_quantize(const int32_t* shp, int32_t rot, const float* tab, int32_t smooth_k, const float* q,
                  const float* k, const float* v, int8_t* qc, float* qs, int8_t* kc, float* ks, int8_t* vc,
                  float* vs, int32_t* vcol, float* q_rot, float* k_rot, float* k_mu) {
  orc_quantize_x(shp, rot, tab, smooth_k ? 1 : 0, q, k, v, qc, qs, kc, ks, vc, vs, vcol, q_rot, k_rot, k_mu,
                 nullptr, nullptr, nullptr);
}

}  // extern "C"
