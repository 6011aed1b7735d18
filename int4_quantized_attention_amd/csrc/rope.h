// 3D RoPE + RoPE-aware rotation on a token tile staged in LDS (device code used
// by the quantisation and fallback pre-pass kernels).
#pragma once
#include "common.h"
#include "kernels.h"

namespace ra {

constexpr int kTile = 128;     // tokens per quantisation workgroup
constexpr int kMeanTile = 64;  // tokens per ordered binary64 partial sum of K

// Load a tile of `rows` tokens x D elements into LDS (row stride D+2 elements
// for 16-bit inputs, D+1 for fp32, so that rows fall in different banks).
template <int D, int DT>
RA_DEV void stage_tile(const void* x, int64_t row0, int64_t N, int rows, char* lds) {
  const int tid = threadIdx.x;
  if (DT == 0) {
    float* L = (float*)lds;
    const float4* src = (const float4*)x;
    const int per_row = D / 4;
    for (int e = tid; e < rows * per_row; e += blockDim.x) {
      const int r = e / per_row, c4 = e % per_row;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row0 + r < N) v = src[(row0 + r) * per_row + c4];
      float* dst = L + r * (D + 1) + c4 * 4;
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
  } else {
    uint32_t* L = (uint32_t*)lds;  // 16-bit elements, row stride D+2 = (D+2)/2 dwords
    const uint4* src = (const uint4*)x;
    const int per_row = D / 8;
    for (int e = tid; e < rows * per_row; e += blockDim.x) {
      const int r = e / per_row, c8 = e % per_row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row0 + r < N) v = src[(row0 + r) * per_row + c8];
      uint32_t* dst = L + r * ((D + 2) / 2) + c8 * 4;
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
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

RA_DEV void token_pos(int64_t n, const Shape& s, int& f, int& y, int& x) {
  const int64_t hw = (int64_t)s.Hs * s.Ws;
  f = (int)(n / hw);
  y = (int)((n / s.Ws) % s.Hs);
  x = (int)(n % s.Ws);
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

RA_DEV int quant_code(float v, float inv) {
  float t = __builtin_rintf(v * inv);
  t = fminf(7.f, fmaxf(-7.f, t));
  return (int)t;
}

}  // namespace ra
