// K3: FP16 FlashAttention fallback for sensitive heads and denoising steps.
//
// RotateAttention (arXiv 2607.02584), papernotes.org note, "Key design 3"
// (selective FP16 fallback: the first/last denoising steps and the first/last DiT
// blocks keep full-precision attention) and the abstract ("mixed-precision INT4
// FlashAttention ... selective FP16 fallback").
//
// Pre-pass (k3_prep): plain 3D RoPE of Q and K in binary32 (same op order as the
// quantisation kernel) rounded to binary16, and V transposed to [D][Np] binary16.
// The pre-pass writes K and V^T of every 64-key group as one image in exactly the
// byte layout the group occupies in LDS (K rows permuted for the S^T register
// layout and padded, then the padded V^T rows).
// Main kernel (k3_attention): one workgroup = 4 waves x 32 query rows, two waves per
// SIMD; S^T = K Q^T on v_mfma_f32_32x32x16_f16, online softmax in binary32 with the
// hardware exp2, P rounded to binary16 and fed straight back as the B operand of
// O^T = V^T P^T; the group images are copied straight from global memory into a
// two-slot LDS ring (buffer_load ... lds), one group ahead.
#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace ra {

constexpr int kFbTile = 64;
constexpr int kFbKV = 64;   // keys per online-softmax step (and per LDS group)
constexpr int kFbBM = 128;  // query rows per workgroup

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
  static constexpr int IMG = ((KBUF + VBUF) * 2 + 4095) / 4096 * 4096;  // bytes of one group's image
  static constexpr int NDMA = IMG / 4096;      // 16-byte copies per thread per group
  static constexpr int LDS = 2 * IMG;          // two ring slots
};

size_t fallback_image_bytes(int D) { return D == 128 ? FbGeo<128>::IMG : FbGeo<64>::IMG; }

// K rows are permuted inside each 32-key tile so that the S^T accumulator of lane
// half h holds keys 16h..16h+15 of the tile in register order: key kk of a group
// sits in image row (kk & ~31) + (v & 3) + 8 (v >> 2) + 4 h, with r = kk & 31,
// h = r >> 4, v = r & 15.
RA_DEV int fb_row_of_key(int kk) {
  const int r = kk & 31, hh = r >> 4, v = r & 15;
  return (kk & ~31) + (v & 3) + 8 * (v >> 2) + 4 * hh;
}

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
  // grid positions of the tile's rows, once per row
  __shared__ int pos[3][kFbTile];
  if (which < 2 && threadIdx.x < kFbTile) {
    int f = 0, y = 0, x = 0;
    if (n0 + threadIdx.x < Nv) token_pos(n0 + threadIdx.x, s, f, y, x);
    pos[0][threadIdx.x] = f;
    pos[1][threadIdx.x] = y;
    pos[2][threadIdx.x] = x;
  }
  stage_tile<D, DT, kFbTile>(base, n0, Nv, lds);
  __syncthreads();
  static_assert(kFbTile == FbGeo<D>::TG, "a pre-pass tile is one key group");
  static_assert(256 % (D / 2) == 0 && 256 % (kFbTile / 2) == 0, "whole rows per pass");
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  // this tile's group image (K and V^T of the 64 keys n0 .. n0+63)
  _Float16* gimg = (_Float16*)(a.img + ((int64_t)bh * (Np / kFbTile) + blockIdx.x) * FbGeo<D>::IMG);
  if (which < 2) {
    // a thread owns the channel pair (c, c + 1) of rows r, r + 256/(D/2), ...: one
    // 4-byte store per row
    // Rows in batches of four: a batch's table loads are all issued before its first
    // store.  Rows past the sequence's end sit at grid position (0, 0, 0) and hold
    // zeros in LDS, so they are computed like the others and their values replaced by
    // zeros.
    _Float16* dst = which == 0 ? a.qr + ((int64_t)bh * Np + n0) * D : nullptr;
    const int c = 2 * (threadIdx.x % (D / 2));
    constexpr int RS = 256 / (D / 2), NR = kFbTile / RS, RB = 4;  // row stride, rows per thread, batch
    static_assert(NR % RB == 0, "whole batches");
#pragma unroll 1
    for (int k0 = 0; k0 < NR; k0 += RB) {
      f16x2 o[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int r = threadIdx.x / (D / 2) + (k0 + k) * RS;
        const int f = pos[0][r], y = pos[1][r], x = pos[2][r];
        float v0 = rope_rot<D, DT>(lds, r, c, s, 0, a.table, f, y, x);
        float v1 = rope_rot<D, DT>(lds, r, c + 1, s, 0, a.table, f, y, x);
        if (n0 + r >= Nv) v0 = v1 = 0.f;
        o[k] = f16x2{(_Float16)v0, (_Float16)v1};
      }
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int r = threadIdx.x / (D / 2) + (k0 + k) * RS;
        if (which == 0) *(f16x2*)(dst + (int64_t)r * D + c) = o[k];
        else *(f16x2*)(gimg + fb_row_of_key(r) * FbGeo<D>::KROW + c) = o[k];
      }
    }
  } else {
    // V^T: a thread owns the token pair (r, r + 1) of channels c, c + 256/32, ...
    _Float16* dst = gimg + FbGeo<D>::KBUF;
    const int r = 2 * (threadIdx.x % (kFbTile / 2));
    for (int c = threadIdx.x / (kFbTile / 2); c < D; c += 256 / (kFbTile / 2)) {
      const float v0 = (n0 + r < Nv) ? lds_elem<D, DT>(lds, r, c) : 0.f;
      const float v1 = (n0 + r + 1 < Nv) ? lds_elem<D, DT>(lds, r + 1, c) : 0.f;
      const f16x2 o = {(_Float16)v0, (_Float16)v1};
      *(f16x2*)(dst + c * FbGeo<D>::VROW + r) = o;
    }
  }
}

// fields the device helpers need, copied out of the kernel argument block
struct FbCtx {
  int64_t Np;
  int N;
  int klim;  // keys this lane's query row sees: N, or its block-causal limit
  float scale_log2;
};

// Copy the image of group g into ring slot buf: wave w copies the w-th quarter of
// the image, one contiguous kilobyte per copy.
template <int D>
RA_DEV void fb_dma(__amdgpu_buffer_rsrc_t r, int g, uint8_t* buf) {
  using G = FbGeo<D>;
  constexpr int WB = G::NDMA * 1024;  // bytes per wave
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  dma_all(std::make_integer_sequence<int, G::NDMA>{}, r, buf + w * WB, 16 * (threadIdx.x & 63), g * G::IMG + w * WB);
}

// Group g on its image in LDS slot cur (K rows, then V^T rows), while the copy of
// group g + 1 into the other slot is in flight.  MASK: the group holds keys at or
// past some row's limit; they count as absent.
template <int D, bool MASK>
RA_DEV void fb_group(const FbCtx& a, int g, const uint8_t* cur, const f16x8 (&qop)[FbGeo<D>::KC],
                     f32x16 (&O)[FbGeo<D>::NDB], float& m, float& l) {
  using G = FbGeo<D>;
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
  const _Float16* const kb_cur = (const _Float16*)cur;
  const _Float16* const vb_cur = kb_cur + G::KBUF;
  f32x16 st[G::NT];
  // the score MFMAs at raised wave priority: while they wait for the matrix pipe the
  // other wave of the SIMD issues its softmax, and each one issues as soon as the
  // pipe frees (1% faster than without)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) {
      const f16x8 kop = *(const f16x8*)(kb_cur + (t * 32 + col) * G::KROW + kc * 16 + 8 * h);
      const f32x16 zero = {0};
      st[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, qop[kc], kc == 0 ? zero : st[t], 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
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
  a.Np = args.Np; a.N = (int)args.N; a.scale_log2 = args.scale_log2;
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
  // the head's group images through a buffer resource that never reaches past the
  // workspace; group 0 in flight, then per group: the copy of group g + 1 into the
  // slot group g - 1 used (free since the last barrier), the group's work, a wait
  // for this wave's copy and one barrier (which covers the other waves' copies)
  const int64_t ngp = a.Np / G::TG;
  const int64_t head0 = (int64_t)bh * ngp * G::IMG;
  const int64_t avail = args.img_bytes - head0;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(args.img + head0), (short)0, (int)(avail < ngp * G::IMG ? (avail > 0 ? avail : 0) : ngp * G::IMG),
      0x00020000);
  uint8_t* const ring = (uint8_t*)flds;
  fb_dma<D>(rsrc, 0, ring);
  wait_vm<0>();
  lds_barrier();
  int g = 0;
  for (; g < nfull; ++g) {
    if (g + 1 < ngroups) fb_dma<D>(rsrc, g + 1, ring + ((g + 1) & 1) * G::IMG);
    fb_group<D, false>(a, g, ring + (g & 1) * G::IMG, qop, O, m, l);
    wait_vm<0>();
    lds_barrier();
  }
  for (; g < ngroups; ++g) {
    if (g + 1 < ngroups) fb_dma<D>(rsrc, g + 1, ring + ((g + 1) & 1) * G::IMG);
    fb_group<D, true>(a, g, ring + (g & 1) * G::IMG, qop, O, m, l);
    wait_vm<0>();
    lds_barrier();
  }

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
