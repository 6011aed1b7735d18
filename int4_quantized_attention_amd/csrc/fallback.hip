// K3: FP16 FlashAttention fallback for sensitive heads and denoising steps.
//
// RotateAttention (arXiv 2607.02584), papernotes.org note, "Key design 3"
// (selective FP16 fallback: the first/last denoising steps and the first/last DiT
// blocks keep full-precision attention) and the abstract ("mixed-precision INT4
// FlashAttention ... selective FP16 fallback").
//
// Pre-pass (k3_prep): plain 3D RoPE of Q and K in binary32 (same op order as the
// quantisation kernel) rounded to binary16, and V transposed to [D][Np] binary16.
// Main kernel (k3_attention): one workgroup = 4 waves x 32 query rows, two waves per
// SIMD; S^T = K Q^T on v_mfma_f32_32x32x16_f16, online softmax in binary32 with the
// hardware exp2, P rounded to binary16 and fed straight back as the B operand of
// O^T = V^T P^T; K/V tiles double-buffered in LDS with loads one group ahead.
#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace ra {

constexpr int kFbTile = 64;
constexpr int kFbKV = 64;   // keys per online-softmax step (and per LDS group)
constexpr int kFbBM = 128;  // query rows per workgroup

// grid (Np/64, B*H, 3): z = 0 Q, 1 K (RoPE -> f16), 2 V (transpose -> f16)
template <int D, int DT>
__global__ __launch_bounds__(256) void k3_prep(FbArgs a) {
  extern __shared__ __align__(16) char lds[];
  const Shape s = a.s;
  const int64_t N = a.N, Np = a.Np;
  const int bh = a.heads[blockIdx.y], which = blockIdx.z;
  const int64_t n0 = (int64_t)blockIdx.x * kFbTile;
  const void* src = which == 0 ? a.q : (which == 1 ? a.k : a.v);
  const void* base = (const char*)src + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  const int64_t Nv = valid_len(a.nlens, a.lens, bh, s.H, N);  // tokens that exist
  stage_tile<D, DT>(base, n0, Nv, kFbTile, lds);
  __syncthreads();
  if (which < 2) {
    _Float16* dst = (which == 0 ? a.qr : a.kr) + ((int64_t)bh * Np + n0) * D;
    for (int e = threadIdx.x; e < kFbTile * D; e += blockDim.x) {
      const int r = e / D, c = e % D;
      float v = 0.f;
      if (n0 + r < Nv) {
        int f, y, x;
        token_pos(n0 + r, s, f, y, x);
        v = rope_rot<D, DT>(lds, r, c, s, 0, a.table, f, y, x);
      }
      dst[(int64_t)r * D + c] = (_Float16)v;
    }
  } else {
    _Float16* dst = a.vt + (int64_t)bh * D * Np + n0;
    for (int e = threadIdx.x; e < kFbTile * D; e += blockDim.x) {
      const int c = e / kFbTile, r = e % kFbTile;
      const float v = (n0 + r < Nv) ? lds_elem<D, DT>(lds, r, c) : 0.f;
      dst[(int64_t)c * Np + r] = (_Float16)v;
    }
  }
}

template <int D>
struct FbGeo {
  static constexpr int TG = kFbKV;             // keys per group
  static constexpr int NT = TG / 32;           // 32-key tiles per group
  static constexpr int NDB = D / 32;           // 32-row d blocks of O^T
  static constexpr int KC = D / 16;            // 16-deep chunks of Q K^T (f16 MFMA)
  static constexpr int KROW = D + 8;           // halves
  static constexpr int VROW = TG + 8;          // halves
  static constexpr int KBUF = TG * KROW;       // halves
  static constexpr int VBUF = D * VROW;        // halves
  static constexpr int LDS = 2 * (KBUF + VBUF) * 2;  // bytes
  static constexpr int KU = TG * D / 8;        // 16-byte global units of a K group
  static constexpr int VU = D * TG / 8;
  static constexpr int KUT = (KU + 255) / 256;
  static constexpr int VUT = (VU + 255) / 256;
};

// fields the device helpers need, copied out of the kernel argument block
struct FbCtx {
  const _Float16* kr;
  const _Float16* vt;
  int64_t Np;
  int N;
  int klim;  // keys this lane's query row sees: N, or its block-causal limit
  float scale_log2;
};

template <int D>
RA_DEV void fb_load(const FbCtx& a, int bh, int g, i32x4 (&rk)[FbGeo<D>::KUT], i32x4 (&rv)[FbGeo<D>::VUT]) {
  using G = FbGeo<D>;
  const i32x4* ks = (const i32x4*)(a.kr + ((int64_t)bh * a.Np + (int64_t)g * G::TG) * D);
#pragma unroll
  for (int i = 0; i < G::KUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::KU % 256 == 0 || u < G::KU) rk[i] = ks[u];
  }
#pragma unroll
  for (int i = 0; i < G::VUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::VU % 256 == 0 || u < G::VU) {
      const int d = u / (G::TG / 8), c = u % (G::TG / 8);
      rv[i] = ((const i32x4*)(a.vt + ((int64_t)bh * D + d) * a.Np + (int64_t)g * G::TG))[c];
    }
  }
}

// K rows are permuted inside each 32-key tile so that the S^T accumulator of lane
// half h holds keys 16h..16h+15 of the tile in register order.
template <int D>
RA_DEV void fb_store(_Float16* Kl, _Float16* Vl, const i32x4 (&rk)[FbGeo<D>::KUT], const i32x4 (&rv)[FbGeo<D>::VUT]) {
  using G = FbGeo<D>;
#pragma unroll
  for (int i = 0; i < G::KUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::KU % 256 == 0 || u < G::KU) {
      const int kk = u / (D / 8), c = u % (D / 8);
      const int r = kk & 31, hh = r >> 4, v = r & 15;
      const int row = (kk & ~31) + (v & 3) + 8 * (v >> 2) + 4 * hh;
      *(i32x4*)(Kl + row * G::KROW + 8 * c) = rk[i];
    }
  }
#pragma unroll
  for (int i = 0; i < G::VUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::VU % 256 == 0 || u < G::VU) {
      const int d = u / (G::TG / 8), c = u % (G::TG / 8);
      *(i32x4*)(Vl + d * G::VROW + 8 * c) = rv[i];
    }
  }
}

// MASK: the group holds keys at or past some row's limit; they count as absent
template <int D, bool MASK>
RA_DEV void fb_group(const FbCtx& a, int g, int ngroups, _Float16* lds, i32x4 (&rk)[FbGeo<D>::KUT],
                     i32x4 (&rv)[FbGeo<D>::VUT], const f16x8 (&qop)[FbGeo<D>::KC], int bh,
                     f32x16 (&O)[FbGeo<D>::NDB], float& m, float& l) {
  using G = FbGeo<D>;
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
  const bool odd = g & 1;
  _Float16* const kb_cur = lds + (odd ? G::KBUF : 0);
  _Float16* const kb_nxt = lds + (odd ? 0 : G::KBUF);
  _Float16* const vb_cur = lds + 2 * G::KBUF + (odd ? G::VBUF : 0);
  _Float16* const vb_nxt = lds + 2 * G::KBUF + (odd ? 0 : G::VBUF);
  f32x16 st[G::NT];
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) {
      const f16x8 kop = *(const f16x8*)(kb_cur + (t * 32 + col) * G::KROW + kc * 16 + 8 * h);
      const f32x16 zero = {0};
      st[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, qop[kc], kc == 0 ? zero : st[t], 0, 0, 0);
    }
  }
  if (g + 1 < ngroups) fb_store<D>(kb_nxt, vb_nxt, rk, rv);
  if (g + 2 < ngroups) fb_load<D>(a, bh, g + 2, rk, rv);
  const int j0 = g * G::TG;
  float mloc = -INFINITY;
#pragma unroll
  for (int t = 0; t < G::NT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const bool ok = !MASK || (j0 + t * 32 + 16 * h + v < a.klim);
      mloc = fmaxf(mloc, ok ? st[t][v] : -INFINITY);
    }
  const float sl2 = a.scale_log2;
  const float mnew = fmaxf(m, fmaxf(mloc, __shfl_xor(mloc, 32, 64)) * sl2);
  const float alpha = exp2_hw(m - mnew);
  if (__any(mnew > m)) {
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[db][v] *= alpha;
  }
  l *= alpha;
  m = mnew;
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
    f16x8 pb[2];
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      float p0 = exp2_hw(__builtin_fmaf(st[t][v], sl2, -mnew));
      float p1 = exp2_hw(__builtin_fmaf(st[t][v + 1], sl2, -mnew));
      if (MASK) {
        p0 = (j0 + t * 32 + 16 * h + v < a.klim) ? p0 : 0.f;
        p1 = (j0 + t * 32 + 16 * h + v + 1 < a.klim) ? p1 : 0.f;
      }
      l += p0 + p1;
      pb[v >> 3][v & 7] = (_Float16)p0;
      pb[v >> 3][(v & 7) + 1] = (_Float16)p1;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        const f16x8 vop = *(const f16x8*)(vb_cur + (db * 32 + col) * G::VROW + t * 32 + 16 * h + 8 * q);
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pb[q], O[db], 0, 0, 0);
      }
    }
  }
  lds_barrier();  // the loads of group g+2 stay in flight
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k3_attention(const FbArgs args) {
  using G = FbGeo<D>;
  extern __shared__ __align__(16) _Float16 flds[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  const int L = (int)(blockIdx.x % 8) * args.per_xcd + (int)(blockIdx.x / 8);
  if (L >= args.total) return;
  const int hidx = L / args.nqt;
  // block-causal tiles: the last query tiles see the most keys, so they go first
  const int qt = args.causal > 0 ? args.nqt - 1 - L % args.nqt : L % args.nqt;
  const int bh = args.heads[hidx];
  // tokens of this head that exist: tiles past them have no row and leave at once
  const int Nv = (int)valid_len(args.nlens, args.lens, bh, args.s.H, args.N);
  if (qt * kFbBM >= Nv) return;
  FbCtx a;
  a.kr = args.kr; a.vt = args.vt; a.Np = args.Np; a.N = (int)args.N; a.scale_log2 = args.scale_log2;
  const int N = a.N;  // the layout's tokens per head
  const int qi = qt * kFbBM + w * 32 + col;
  // keys seen: all Nv, or min(Nv, (i / c + 1) c) under block-causal masking (block
  // c); groups wholly below the tile's first row's limit need no per-key test
  const int64_t c = args.causal;
  auto limit = [&](int64_t i) -> int { return c > 0 ? (int)min((int64_t)Nv, (i / c + 1) * c) : Nv; };
  a.klim = limit(qi);
  const int kmax = limit(min(qt * kFbBM + kFbBM - 1, Nv - 1));

  f16x8 qop[G::KC];
  {
    const f16x8* qp = (const f16x8*)(args.qr + ((int64_t)bh * a.Np + qi) * D);
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) qop[kc] = qp[kc * 2 + h];
  }
  float m = -INFINITY, l = 0.f;
  f32x16 O[G::NDB];
#pragma unroll
  for (int db = 0; db < G::NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[db][v] = 0.f;

  const int ngroups = (kmax + G::TG - 1) / G::TG;
  const int nfull = min(limit(qt * kFbBM) / G::TG, ngroups);  // groups no row masks
  i32x4 rk[G::KUT], rv[G::VUT];
  fb_load<D>(a, bh, 0, rk, rv);
  fb_store<D>(flds, flds + 2 * G::KBUF, rk, rv);
  if (ngroups > 1) fb_load<D>(a, bh, 1, rk, rv);
  lds_barrier();
  int g = 0;
  for (; g < nfull; ++g) fb_group<D, false>(a, g, ngroups, flds, rk, rv, qop, bh, O, m, l);
  for (; g < ngroups; ++g) fb_group<D, true>(a, g, ngroups, flds, rk, rv, qop, bh, O, m, l);

  const float lq = l + __shfl_xor(l, 32, 64);
  if (qi < Nv) {
    const float inv = 1.0f / lq;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * h;
        const int64_t off = ((int64_t)bh * N + qi) * D + d0;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = O[db][v4 * 4 + e] * inv;
        store_out4(args.out, args.out_kind, off, o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <int D, int DT>
hipError_t launch_prep_t(const FbArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.Np / kFbTile), a.nheads, 3);
  const size_t lds = (size_t)kFbTile * (DT == 0 ? (D + 1) * 4 : (D + 2) * 2);  // the staged input tile
  k3_prep<D, DT><<<grid, 256, lds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fallback_prep(const FbArgs& a, int dtype, hipStream_t st) {
  if (a.s.D == 128) {
    if (dtype == 0) return launch_prep_t<128, 0>(a, st);
    if (dtype == 1) return launch_prep_t<128, 1>(a, st);
    return launch_prep_t<128, 2>(a, st);
  }
  if (dtype == 0) return launch_prep_t<64, 0>(a, st);
  if (dtype == 1) return launch_prep_t<64, 1>(a, st);
  return launch_prep_t<64, 2>(a, st);
}

template <int D>
hipError_t launch_fb_t(const FbArgs& a, hipStream_t st) {
  using G = FbGeo<D>;
  const hipError_t attr = hipFuncSetAttribute((const void*)k3_attention<D>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
  if (attr != hipSuccess) return attr;
  k3_attention<D><<<8 * a.per_xcd, 256, G::LDS, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fallback(const FbArgs& a, hipStream_t st) {
  if (a.s.D == 128) return launch_fb_t<128>(a, st);
  return launch_fb_t<64>(a, st);
}

}  // namespace ra
