// 3D RoPE + RoPE-aware rotation on a token tile staged in LDS (device code used
// by the quantisation and fallback pre-pass kernels).
#pragma once
#include "common.h"
#include "kernels.h"

namespace ra {

constexpr int kTile = 128;     // tokens per quantisation workgroup
constexpr int kMeanTile = 64;  // tokens per ordered binary64 partial sum of K

// Load a tile of ROWS tokens x D elements into LDS (row stride D+2 elements for
// 16-bit inputs, D+1 for fp32, so that rows fall in different banks); rows at or past
// N are zeros.  256 threads: each issues all of its 16-byte loads before it stores any
// of them (a load-store pair per iteration would wait out one memory latency each).
// Rows past N read row N-1 (N >= 1), so every load stays inside the tensor and none
// sits behind a branch; those values are replaced by zeros.
template <int D, int DT, int ROWS>
RA_DEV void stage_tile(const void* x, int64_t row0, int64_t N, char* lds) {
  constexpr int VPR = DT == 0 ? D / 4 : D / 8;  // 16-byte vectors per row
  static_assert(ROWS * VPR % 256 == 0, "whole passes of 256 threads");
  constexpr int IT = ROWS * VPR / 256;
  const int tid = threadIdx.x;
  const u32x4* src = (const u32x4*)x;
  u32x4 v[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = tid + 256 * i, r = e / VPR, c = e % VPR;
    v[i] = src[min(row0 + r, N - 1) * VPR + c];
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = tid + 256 * i, r = e / VPR, c = e % VPR;
    const u32x4 w = row0 + r < N ? v[i] : u32x4{0u, 0u, 0u, 0u};
    uint32_t* dst = (uint32_t*)lds + r * (DT == 0 ? D + 1 : (D + 2) / 2) + c * 4;
    dst[0] = w[0]; dst[1] = w[1]; dst[2] = w[2]; dst[3] = w[3];
  }
}

template <int D, int DT>
RA_DEV float lds_elem(const char* lds, int r, int c) {
  if (DT == 0) return ((const float*)lds)[r * (D + 1) + c];
  const uint16_t u = ((const uint16_t*)lds)[r * (D + 2) + c];
  if (DT == 1) return (float)__builtin_bit_cast(_Float16, u);
  return __uint_as_float((uint32_t)u << 16);
}

// RoPE (plain) output at channel cc of a token row, binary32 op order
//   u0 = fma(a, c, -(b*s)),  u1 = fma(a, s, b*c).
template <int D, int DT>
RA_DEV float rope_plain(const char* lds, int r, int o, const float* trow, int lc) {
  const int p = lc >> 1;
  const float a = lds_elem<D, DT>(lds, r, o + 2 * p), b = lds_elem<D, DT>(lds, r, o + 2 * p + 1);
  const float t0 = trow[2 * p], t1 = trow[2 * p + 1];
  if ((lc & 1) == 0) {
    const float bs = b * t1;
    return __builtin_fmaf(a, t0, -bs);
  }
  const float bc = b * t0;
  return __builtin_fmaf(a, t1, bc);
}

// Output channel c of RoPE + rotation for token row r at grid position (f, y, x).
template <int D, int DT>
RA_DEV float rope_rot(const char* lds, int r, int c, const Shape& s, int rot, const float* tab,
                      int f, int y, int x) {
  int j, o, dj, pos, toff;
  if (c < s.Df) { j = 0; o = 0; dj = s.Df; pos = f; toff = 0; }
  else if (c < s.Df + s.Dh) { j = 1; o = s.Df; dj = s.Dh; pos = y; toff = s.F * s.Df; }
  else { j = 2; o = s.Df + s.Dh; dj = s.Dw; pos = x; toff = s.F * s.Df + s.Hs * s.Dh; }
  (void)j;
  const float* trow = tab + toff + pos * dj;  // dj/2 pairs x 2 entries
  const int lc = c - o;
  if (rot == 2) {
    const int h = dj >> 1, i = lc >> 1;
    const float x1 = rope_plain<D, DT>(lds, r, o, trow, i);
    const float x2 = rope_plain<D, DT>(lds, r, o, trow, h + i);
    const float rr = 0.70710678118654752440f;
    if ((lc & 1) == 0) { const float sm = x1 + x2; return sm * rr; }
    const float df = x1 - x2;
    return df * rr;
  }
  if (rot == 1) {
    const int p = lc >> 1;
    const float a = lds_elem<D, DT>(lds, r, o + 2 * p), b = lds_elem<D, DT>(lds, r, o + 2 * p + 1);
    const float al = trow[2 * p], be = trow[2 * p + 1];
    if ((lc & 1) == 0) { const float bb = b * be; return __builtin_fmaf(a, al, bb); }
    const float ba = b * al;
    return __builtin_fmaf(a, be, -ba);
  }
  return rope_plain<D, DT>(lds, r, o, trow, lc);
}

// Grid position of token n = (f*Hs + y)*Ws + x.  Token indices stay below 2^29 (the
// shape check bounds N by 2^28, plus the padding), so two 32-bit divisions give it
// exactly; 64-bit divisions cost about a hundred instructions each.
RA_DEV void token_pos(int64_t n, const Shape& s, int& f, int& y, int& x) {
  const uint32_t u = (uint32_t)n, ws = (uint32_t)s.Ws, hs = (uint32_t)s.Hs;
  const uint32_t q = u / ws;  // f*Hs + y
  const uint32_t ff = q / hs;
  x = (int)(u - q * ws);
  y = (int)(q - ff * hs);
  f = (int)ff;
}

// ---- per-thread token slices --------------------------------------------------------
// A thread owns CPT consecutive channels [c0, c0 + CPT) of one token (c0 a multiple
// of CPT, CPT a multiple of 8): it loads them with 16-byte loads, applies RoPE pair by
// pair with one table load per pair, and for the Half rotation exchanges the RoPE
// outputs through an LDS row to pair channel i with i + Dj/2.

template <int DT, int CPT>
RA_DEV void load_slice(const void* base, int64_t n, int D, int c0, float (&x)[CPT]) {
  if (DT == 0) {
    const f32x4* p = (const f32x4*)((const float*)base + n * D + c0);
#pragma unroll
    for (int i = 0; i < CPT / 4; ++i) {
      const f32x4 v = p[i];
      x[4 * i] = v[0]; x[4 * i + 1] = v[1]; x[4 * i + 2] = v[2]; x[4 * i + 3] = v[3];
    }
  } else {
    const u32x4* p = (const u32x4*)((const uint16_t*)base + n * D + c0);
#pragma unroll
    for (int i = 0; i < CPT / 8; ++i) {
      const u32x4 w = p[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = w[e];
        if (DT == 1) {
          x[8 * i + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
          x[8 * i + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
        } else {
          x[8 * i + 2 * e] = __uint_as_float(u << 16);
          x[8 * i + 2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
        }
      }
    }
  }
}

// Offsets (in floats) of a token's rows in the three axis tables, and the first
// global pair index of the height and width segments.
struct SegRows {
  int base0, base1, base2, p1, p2;
};
RA_DEV SegRows seg_rows(const Shape& s, int f, int y, int x) {
  SegRows g;
  g.base0 = f * s.Df;
  g.base1 = s.F * s.Df + y * s.Dh;
  g.base2 = s.F * s.Df + s.Hs * s.Dh + x * s.Dw;
  g.p1 = s.Df / 2;
  g.p2 = (s.Df + s.Dh) / 2;
  return g;
}

// RoPE in place on the slice: pair k is global pair p = c0/2 + k.  ROT 1 uses the
// fused Interleaved table (alpha, beta); otherwise the plain (cos, sin) table.
//   plain: u0 = fma(a, c, -(b*s)), u1 = fma(a, s, b*c)
//   fused: o0 = fma(a, al, b*be),  o1 = fma(a, be, -(b*al))
template <int ROT, int CPT>
RA_DEV void rope_slice(float (&x)[CPT], int c0, const float* tab, const SegRows& g) {
#pragma unroll
  for (int k = 0; k < CPT / 2; ++k) {
    const int p = c0 / 2 + k;
    const int off = p < g.p1 ? g.base0 + 2 * p : (p < g.p2 ? g.base1 + 2 * (p - g.p1) : g.base2 + 2 * (p - g.p2));
    const f32x2 t = *(const f32x2*)(tab + off);
    const float a = x[2 * k], b = x[2 * k + 1];
    if (ROT == 1) {
      const float bb = b * t[1], ba = b * t[0];
      x[2 * k] = __builtin_fmaf(a, t[0], bb);
      x[2 * k + 1] = __builtin_fmaf(a, t[1], -ba);
    } else {
      const float bs = b * t[1], bc = b * t[0];
      x[2 * k] = __builtin_fmaf(a, t[0], -bs);
      x[2 * k + 1] = __builtin_fmaf(a, t[1], bc);
    }
  }
}

// Half rotation of the slice from the token's RoPE outputs U[0..D): output pair
// (o + 2i, o + 2i + 1) = ((x1 + x2) r, (x1 - x2) r), x1 = U[o+i], x2 = U[o+h+i],
// h = Dj/2, r = fl(1/sqrt2).
template <int CPT>
RA_DEV void half_slice(const float* U, int c0, const Shape& s, float (&x)[CPT]) {
  const float r = 0.70710678118654752440f;
#pragma unroll
  for (int k = 0; k < CPT / 2; ++k) {
    const int c = c0 + 2 * k;
    int o, dj;
    if (c < s.Df) { o = 0; dj = s.Df; }
    else if (c < s.Df + s.Dh) { o = s.Df; dj = s.Dh; }
    else { o = s.Df + s.Dh; dj = s.Dw; }
    const int i = (c - o) >> 1;
    const float x1 = U[o + i], x2 = U[o + (dj >> 1) + i];
    const float sm = x1 + x2, df = x1 - x2;
    x[2 * k] = sm * r;
    x[2 * k + 1] = df * r;
  }
}

// Full rotation (ROT 3) of the token's RoPE outputs: the orthonormal D x D
// Walsh-Hadamard transform, stride by stride (1, 2, 4, ..., D/2), every pair
// (x[i], x[i + len]) with i & len == 0 becoming (x[i] + x[i + len], x[i] - x[i + len]),
// then every channel times fl(1/sqrt(D)).  Strides below CPT stay inside the
// thread's slice; larger strides pair the slice with the one of lane ^ (len/CPT)
// (the token's TPT threads are consecutive lanes).  All lanes must call.
template <int D, int CPT>
RA_DEV void hadamard_slice(float (&x)[CPT], int c0) {
#pragma unroll
  for (int len = 1; len < CPT; len *= 2) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if ((i & len) == 0) {
        const float a = x[i], b = x[i + len];
        x[i] = a + b;
        x[i + len] = a - b;
      }
    }
  }
#pragma unroll
  for (int len = CPT; len < D; len *= 2) {
    const bool lower = (c0 & len) == 0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const float o = __shfl_xor(x[i], len / CPT, 64);
      x[i] = lower ? x[i] + o : o - x[i];
    }
  }
  const float rd = D == 128 ? 0.08838834764831844055f : 0.125f;  // fl(1/sqrt(D)), D in {64, 128}
#pragma unroll
  for (int i = 0; i < CPT; ++i) x[i] = x[i] * rd;
}

// RoPE + rotation of one slice; U is this token's LDS row (D + 1 floats, used by
// ROT 2 only).  Contains a workgroup barrier when ROT == 2 (all threads must call);
// ROT 3 exchanges values between the token's lanes (all lanes must call).
template <int DT, int ROT, int CPT, int DD = 0>
RA_DEV void rotated_slice(const void* base, int64_t n, bool valid, int D, int c0, const Shape& s,
                          const float* tab, float* U, float (&x)[CPT]) {
  if (valid) {
    int f, y, xx;
    token_pos(n, s, f, y, xx);
    load_slice<DT, CPT>(base, n, D, c0, x);
    rope_slice<ROT, CPT>(x, c0, tab, seg_rows(s, f, y, xx));
  } else {
#pragma unroll
    for (int i = 0; i < CPT; ++i) x[i] = 0.f;
  }
  if (ROT == 2) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) U[c0 + i] = x[i];
    __syncthreads();
    if (valid) half_slice<CPT>(U, c0, s, x);
  }
  if (ROT == 3) hadamard_slice<DD, CPT>(x, c0);
}

// ---- wave-sliced token tiles ------------------------------------------------------
// A workgroup of four waves takes 64 tokens, one per lane; wave w owns the channel
// slice [w D/4, (w + 1) D/4) of each of them.  The slice start is the same across
// the wave, so what depends on the channel (the RoPE segment of a pair, the Half
// partner of a channel) is one scalar decision per wave, and the per-lane work is
// the arithmetic and one address add per table or LDS access.

// First channel of this wave's slice (a wave-uniform value).
template <int D>
RA_DEV int wave_slice_c0() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * (D / 4);
}

// RoPE in place on a wave slice of token (f, y, x): pair k is global pair p = c0/2 + k,
// whose table entry sits at byte offset Q_j + 8k, Q_j = 4 (row_j - 2 p_j + c0) for the
// segment j of p (row_j: the token's row in segment j's table, p_j: its first pair).
// Every Q_j is >= 0 (segment j's rows start past the 2 p_j floats of the earlier
// segments' first rows).
template <int ROT, int CPT>
RA_DEV void rope_wave_slice(float (&x)[CPT], int c0, const float* tab, const Shape& s, int f, int y, int xx) {
  const uint32_t Q0 = 4u * (uint32_t)(f * s.Df + c0);
  const uint32_t Q1 = 4u * (uint32_t)((s.F - 1) * s.Df + y * s.Dh + c0);
  const uint32_t Q2 = 4u * (uint32_t)((s.F - 1) * s.Df + (s.Hs - 1) * s.Dh + xx * s.Dw + c0);
  const int k1 = s.Df / 2 - c0 / 2, k2 = (s.Df + s.Dh) / 2 - c0 / 2;  // first slice pair of segments 1, 2
#pragma unroll
  for (int k = 0; k < CPT / 2; ++k) {
    const uint32_t Q = k < k1 ? Q0 : (k < k2 ? Q1 : Q2);
    const f32x2 t = *(const f32x2*)((const char*)tab + (size_t)Q + 8 * k);
    const float a = x[2 * k], b = x[2 * k + 1];
    if (ROT == 1) {
      const float bb = b * t[1], ba = b * t[0];
      x[2 * k] = __builtin_fmaf(a, t[0], bb);
      x[2 * k + 1] = __builtin_fmaf(a, t[1], -ba);
    } else {
      const float bs = b * t[1], bc = b * t[0];
      x[2 * k] = __builtin_fmaf(a, t[0], -bs);
      x[2 * k + 1] = __builtin_fmaf(a, t[1], bc);
    }
  }
}

// RoPE + rotation (ROT 0, 1, 2) of this wave's slice of token n, in the lane's
// registers.  U: LDS of 64 token rows of D + 1 floats (ROT 2 exchanges the RoPE
// outputs through it; output pair (c, c + 1) of segment j takes x1 = U[(c + o_j)/2]
// and x2 = U[(c + o_j)/2 + Dj/2], the same pairs as half_slice).  Contains a
// workgroup barrier when ROT == 2 (all threads must call).
template <int DT, int ROT, int D>
RA_DEV void rotated_wave_slice(const void* base, int64_t n, bool valid, int c0, const Shape& s,
                               const float* tab, float* U, int lane, float (&x)[D / 4]) {
  constexpr int CPT = D / 4;
  static_assert(ROT >= 0 && ROT <= 2, "the Full rotation mixes all channels: token-sliced path");
  if (valid) {
    int f, y, xx;
    token_pos(n, s, f, y, xx);
    load_slice<DT, CPT>(base, n, D, c0, x);
    rope_wave_slice<ROT, CPT>(x, c0, tab, s, f, y, xx);
  } else {
#pragma unroll
    for (int i = 0; i < CPT; ++i) x[i] = 0.f;
  }
  if (ROT == 2) {
    float* row = U + lane * (D + 1);
#pragma unroll
    for (int i = 0; i < CPT; ++i) row[c0 + i] = x[i];
    __syncthreads();
    if (valid) {
      const float r = 0.70710678118654752440f;
#pragma unroll
      for (int k = 0; k < CPT / 2; ++k) {
        const int c = c0 + 2 * k;
        const int o = c < s.Df ? 0 : (c < s.Df + s.Dh ? s.Df : s.Df + s.Dh);
        const int h = (c < s.Df ? s.Df : (c < s.Df + s.Dh ? s.Dh : s.Dw)) >> 1;
        const int S = (c + o) >> 1;
        const float x1 = row[S], x2 = row[S + h];
        const float sm = x1 + x2, df = x1 - x2;
        x[2 * k] = sm * r;
        x[2 * k + 1] = df * r;
      }
    }
  }
}

// Maximum of non-negative binary32 values (as their bits, which order like unsigned
// integers) over groups of `width` consecutive lanes (a wave-uniform power of two
// <= 64): quad permutations, the 8- and 16-lane mirrors, a 32-lane swizzle, then
// the two wave halves.  All lanes must be active.
RA_DEV uint32_t group_max_u32(uint32_t v, int width) {
  if (width >= 2) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  if (width >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  if (width >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  if (width >= 16) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  if (width >= 32) v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  if (width >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return v;
}

// The code of v with inv = fl(7/amax), |v| <= amax, as the bits of fl(t + M), t =
// clamp(fl(v inv), -7, 7), M = 1.5 2^23 + 8: in [2^23, 2^24) the ulp is 1, so the sum
// rounds t to an integer, and as M is even, a tie goes to the even integer exactly
// as rint(t) would; the bits are then 0x4B400008 + k for the code k.  Clamping before
// rounding equals clamping after it for |t| < 7.5, which holds whenever inv is finite
// (|fl(v inv)| <= 7 (1 + 2^-24)^2).  The clamp still acts when 7/amax overflows (amax
// below about 2.06e-38): it turns +-inf into +-7 and the NaN of 0 * inf into -7, as
// fmin(7, fmax(-7, .)) does after rounding.  amax = 0 (inv = 0, v = 0) gives k = 0.
RA_DEV uint32_t code_bits(float v, float inv) {
  return __float_as_uint(fminf(7.f, fmaxf(-7.f, v * inv)) + 12582920.0f);
}
// The same without the clamp, for finite inv (then |fl(v inv)| < 7.5).
RA_DEV uint32_t code_bits_finite(float v, float inv) { return __float_as_uint(v * inv + 12582920.0f); }
// The low nibble k + 8 of the bits, in [1, 15], is k in offset binary.
constexpr uint32_t kZeroCodeBits = 0x4B400008u;  // code_bits of a 0 code
RA_DEV int code_of_bits(uint32_t b) { return (int)(b - kZeroCodeBits); }

// Eight code_bits values -> one word of two's-complement nibbles, element e in bits
// [4e, 4e + 4).  sum_e b_e 16^e (mod 2^32) is sum_e (k_e + 8) 16^e plus a constant
// (the 0x4B400000 parts shifted), the offset-binary nibbles carry nothing, and
// flipping each nibble's top bit maps k + 8 to k's two's-complement nibble.
constexpr uint32_t pack_bias() {
  uint32_t c = 0;
  for (int e = 0; e < 8; ++e) c += (kZeroCodeBits - 8u) << (4 * e);
  return c;
}
RA_DEV uint32_t pack8(const uint32_t* b) {
  uint32_t w = b[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) w += b[e] << (4 * e);
  return (w - pack_bias()) ^ 0x88888888u;
}

// code_bits of CNT values sharing inv: the clamp-free form unless 7/amax overflowed.
template <int CNT>
RA_DEV void code_bits_n(const float* v, float inv, uint32_t* b) {
  if (__builtin_expect(__builtin_isinf(inv), 0)) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) b[i] = code_bits(v[i], inv);
  } else {
#pragma unroll
    for (int i = 0; i < CNT; ++i) b[i] = code_bits_finite(v[i], inv);
  }
}

// CPT values (a multiple of 8) -> CPT/8 words of packed codes.
template <int CPT>
RA_DEV void pack_codes(const float (&v)[CPT], float inv, uint32_t (&out)[CPT / 8]) {
  uint32_t b[CPT];
  code_bits_n<CPT>(v, inv, b);
#pragma unroll
  for (int w = 0; w < CPT / 8; ++w) out[w] = pack8(b + 8 * w);
}

}  // namespace ra
