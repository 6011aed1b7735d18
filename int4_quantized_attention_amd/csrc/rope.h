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

RA_DEV int quant_code(float v, float inv) {
  float t = __builtin_rintf(v * inv);
  t = fminf(7.f, fmaxf(-7.f, t));
  return (int)t;
}

}  // namespace ra
