// K3: FP16 FlashAttention fallback for sensitive heads and denoising steps.
//
// RotateAttention (arXiv 2607.02584), papernotes.org note, "Key design 3"
// (selective FP16 fallback: the first/last denoising steps and the first/last DiT
// blocks keep full-precision attention) and the abstract ("mixed-precision INT4
// FlashAttention ... selective FP16 fallback").
//
// Pre-pass (k3_prep): plain 3D RoPE of Q and K in binary32 (same op order as the
// quantisation kernel) rounded to binary16, and V transposed to [D][Np] binary16.
// Main kernel (k3_attention): one workgroup = 4 waves x 32 query rows; S^T = K Q^T
// on v_mfma_f32_32x32x16_f16, online softmax in binary32 with the hardware exp2, P
// rounded to binary16 and fed straight back as the B operand of O^T = V^T P^T.
#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace ra {

constexpr int kFbTile = 64;
constexpr int kFbKV = 64;   // keys per online-softmax step
constexpr int kFbBM = 128;  // query rows per workgroup

// grid (Np/64, B*H, 3): z = 0 Q, 1 K (RoPE -> f16), 2 V (transpose -> f16)
template <int D, int DT>
__global__ __launch_bounds__(256) void k3_prep(FbArgs a) {
  extern __shared__ __align__(16) char lds[];
  const Shape s = a.s;
  const int64_t N = a.N, Np = a.Np;
  const int bh = blockIdx.y, which = blockIdx.z;
  const int64_t n0 = (int64_t)blockIdx.x * kFbTile;
  const void* src = which == 0 ? a.q : (which == 1 ? a.k : a.v);
  const void* base = (const char*)src + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  stage_tile<D, DT>(base, n0, N, kFbTile, lds);
  __syncthreads();
  if (which < 2) {
    _Float16* dst = (which == 0 ? a.qr : a.kr) + ((int64_t)bh * Np + n0) * D;
    for (int e = threadIdx.x; e < kFbTile * D; e += blockDim.x) {
      const int r = e / D, c = e % D;
      float v = 0.f;
      if (n0 + r < N) {
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
      const float v = (n0 + r < N) ? lds_elem<D, DT>(lds, r, c) : 0.f;
      dst[(int64_t)c * Np + r] = (_Float16)v;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k3_attention(const FbArgs a) {
  constexpr int NDB = D / 32, KC = D / 16, NT = kFbKV / 32;
  constexpr int KROW = D + 8;      // halves
  constexpr int VROW = kFbKV + 8;  // halves
  __shared__ __align__(16) _Float16 Kl[kFbKV * KROW];
  __shared__ __align__(16) _Float16 Vl[D * VROW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  const int L = (int)(blockIdx.x % 8) * a.per_xcd + (int)(blockIdx.x / 8);
  if (L >= a.total) return;
  const int hidx = L / a.nqt, qt = L % a.nqt;
  const int bh = a.heads[hidx];
  const int64_t N = a.N, Np = a.Np;
  const int qi = qt * kFbBM + w * 32 + col;

  f16x8 qop[KC];
  {
    const f16x8* qp = (const f16x8*)(a.qr + ((int64_t)bh * Np + qi) * D);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qop[kc] = qp[kc * 2 + h];
  }
  const float sl2 = a.scale_log2;
  float m = -INFINITY, l = 0.f;
  f32x16 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[db][v] = 0.f;

  const int64_t ngroups = (N + kFbKV - 1) / kFbKV;
  for (int64_t g = 0; g < ngroups; ++g) {
    const int64_t j0 = g * kFbKV;
    __syncthreads();
    for (int it = tid; it < kFbKV * (D / 8); it += 256) {
      const int kk = it / (D / 8), c = it % (D / 8);
      const uint4 x = ((const uint4*)(a.kr + ((int64_t)bh * Np + j0 + kk) * D))[c];
      const int r = kk & 31, hh = r >> 4, v = r & 15;
      const int row = (kk & ~31) + (v & 3) + 8 * (v >> 2) + 4 * hh;
      *(uint4*)(Kl + row * KROW + 8 * c) = x;
    }
    for (int it = tid; it < D * (kFbKV / 8); it += 256) {
      const int d = it / (kFbKV / 8), c = it % (kFbKV / 8);
      const uint4 x = ((const uint4*)(a.vt + ((int64_t)bh * D + d) * Np + j0))[c];
      *(uint4*)(Vl + d * VROW + 8 * c) = x;
    }
    __syncthreads();
    f32x16 st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[t][v] = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const f16x8 kop = *(const f16x8*)(Kl + (t * 32 + col) * KROW + kc * 16 + 8 * h);
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, qop[kc], st[t], 0, 0, 0);
      }
    }
    const bool tail = j0 + kFbKV > N;
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t key = j0 + t * 32 + 16 * h + v;
        if (!tail || key < N) mloc = fmaxf(mloc, st[t][v]);
      }
    const float mstep = fmaxf(mloc, __shfl_xor(mloc, 32, 64)) * sl2;
    const float mnew = fmaxf(m, mstep);
    const float alpha = exp2_hw(m - mnew);
    if (__any(mnew > m)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[db][v] *= alpha;
    }
    l *= alpha;
    m = mnew;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f16x8 pb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t key = j0 + t * 32 + 16 * h + v;
        const float p = (!tail || key < N) ? exp2_hw(__builtin_fmaf(st[t][v], sl2, -mnew)) : 0.f;
        l += p;
        pb[v >> 3][v & 7] = (_Float16)p;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f16x8 vop = *(const f16x8*)(Vl + (db * 32 + col) * VROW + t * 32 + 16 * h + 8 * q);
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pb[q], O[db], 0, 0, 0);
        }
      }
    }
  }
  const float lq = l + __shfl_xor(l, 32, 64);
  if (qi < N) {
    const float inv = 1.0f / lq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * h;
        const int64_t off = ((int64_t)bh * N + qi) * D + d0;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = O[db][v4 * 4 + e] * inv;
        if (a.out_f16) {
          *(f16x4*)((_Float16*)a.out + off) = f16x4{(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
        } else {
          *(f32x4*)((float*)a.out + off) = f32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
  }
}

hipError_t launch_fallback_prep(const FbArgs& a, hipStream_t st) {
  const int BH = a.s.B * a.s.H;
  const dim3 grid((unsigned)(a.Np / kFbTile), BH, 3);
  const size_t lds = (size_t)kFbTile * (a.s.D + 2) * 2;
  if (a.s.D == 128) k3_prep<128, 1><<<grid, 256, lds, st>>>(a);
  else k3_prep<64, 1><<<grid, 256, lds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fallback(const FbArgs& a, hipStream_t st) {
  if (a.s.D == 128) k3_attention<128><<<8 * a.per_xcd, 256, 0, st>>>(a);
  else k3_attention<64><<<8 * a.per_xcd, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ra
