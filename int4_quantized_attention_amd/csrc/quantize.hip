// K1: fused 3D RoPE -> RoPE-aware rotation -> K smoothing -> INT4 quantisation.
//
// RotateAttention (arXiv 2607.02584), papernotes.org note: "Overall framework"
// (smoothing, RoPE-aware rotation, INT4 Q/K) and "Key design 1" (3D RoPE split
// D = Df + Dh + Dw; Interleaved rotation fused into the RoPE 2x2 blocks; Half
// rotation Q Pi R pairing channel i with i + Dj/2 inside each segment).
//
// Memory-bound.  Q and K: a thread owns a slice of consecutive channels of one
// token, loads it with 16-byte loads, applies RoPE once per channel pair (one table
// load per pair), exchanges RoPE outputs through LDS only for the Half rotation,
// and writes packed nibbles with 8/16-byte stores.  V is staged through LDS and
// written transposed.  K and V need global statistics (the channel mean of K, the
// channel amax of V), so they are read twice.
#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace ra {

// ---------------------------------------------------------------------------------
// Channel statistics for smoothing: ordered binary64 partial sums of rotated K (and,
// with Q smoothing, of rotated Q) over 64-token blocks.  grid (ceil(N/64), B*H, the
// number of smoothed tensors); z = 0 is K unless only Q is smoothed.  256 threads,
// four per token, each owning D/4 channels.  partial [B*H][nblk][D] f64.
template <int D, int DT, int ROT>
__global__ __launch_bounds__(256) void k1_kstats(QuantArgs a) {
  constexpr int TPT = 4, CPT = D / TPT;
  __shared__ float R[kMeanTile * (D + 1)];  // RoPE outputs (Half), then rotated rows
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int bh = blockIdx.y, blk = blockIdx.x;
  const bool isQ = blockIdx.z + (a.smooth ? 0 : 1) == 1;
  const int64_t Nb = valid_len(a.nlens, a.lens, bh, s.H, N);
  const int64_t n0 = (int64_t)blk * kMeanTile;
  const int lt = threadIdx.x / TPT, c0 = (threadIdx.x % TPT) * CPT;
  const int64_t n = n0 + lt;
  const void* base = (const char*)(isQ ? a.q : a.k) + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  float x[CPT];
  rotated_slice<DT, ROT, CPT, D>(base, n, n < Nb, D, c0, s, a.table, R + lt * (D + 1), x);
  if (ROT == 2) __syncthreads();  // every row of R read before it is overwritten
#pragma unroll
  for (int i = 0; i < CPT; ++i) R[lt * (D + 1) + c0 + i] = x[i];
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    double part = 0.0;
    const int cnt = (int)max((int64_t)0, min((int64_t)kMeanTile, Nb - n0));
    for (int r = 0; r < cnt; ++r) part += (double)R[r * (D + 1) + c];
    const int64_t nblk = (N + kMeanTile - 1) / kMeanTile;
    (isQ ? a.qpart : a.kpart)[((int64_t)bh * nblk + blk) * D + c] = part;
  }
}

// Channel means of K (and Q): binary64 sum of the partials in block order, / N, to
// binary32.  Thread idx: tensor idx / (B*H*D) in the order of k1_kstats' z.  The
// sum is one dependent chain; the loads run eight ahead of it.
__global__ void k1_kmean(QuantArgs a) {
  const int D = a.s.D;
  const int64_t N = (int64_t)a.s.F * a.s.Hs * a.s.Ws;
  const int64_t nblk = (N + kMeanTile - 1) / kMeanTile;
  const int64_t per = (int64_t)a.s.B * a.s.H * D;
  const int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nz = (a.smooth ? 1 : 0) + (a.smooth_q ? 1 : 0);
  if (gidx >= nz * per) return;
  const bool isQ = gidx / per + (a.smooth ? 0 : 1) == 1;
  const int64_t idx = gidx % per;
  const int64_t bh = idx / D, c = idx % D;
  const double* p = (isQ ? a.qpart : a.kpart) + bh * nblk * D + c;
  double total = 0.0;
  int64_t b = 0;
  for (; b + 8 <= nblk; b += 8) {
    double v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(b + i) * D];
#pragma unroll
    for (int i = 0; i < 8; ++i) total += v[i];
  }
  for (; b < nblk; ++b) total += p[b * D];
  // blocks past the valid tokens hold +0.0 partials: adding them changes nothing
  const int64_t Nb = valid_len(a.nlens, a.lens, (int)bh, a.s.H, N);
  (isQ ? a.qmu : a.kmu)[idx] = (float)(total / (double)Nb);
}

__global__ void k1_zero_u32(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// V channel amax over all tokens.  A workgroup takes kVTile tokens of one head:
// thread t owns 8 consecutive channels (one 16-byte load per token for 16-bit
// inputs) of every (256 / (D/8))-th token, the partial maxima meet in LDS, and one
// atomic max per channel on the float bits (non-negative floats order like unsigned
// integers) merges the workgroups.
constexpr int kVTile = 512;
template <int D, int DT>
__global__ __launch_bounds__(256) void k1_vamax(QuantArgs a) {
  constexpr int CG = D / 8, TL = 256 / CG;  // channel groups, tokens in flight
  __shared__ float red[TL][D + 1];
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int bh = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * kVTile;
  const int64_t Nb = valid_len(a.nlens, a.lens, bh, s.H, N);
  const void* base = (const char*)a.v + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  const int cg = threadIdx.x % CG, tl = threadIdx.x / CG;
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.f;
#pragma unroll 4
  for (int r = tl; r < kVTile; r += TL) {
    const int64_t n = n0 + r;
    if (n < Nb) {
      float x[8];
      load_slice<DT, 8>(base, n, D, 8 * cg, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(x[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tl][8 * cg + e] = m[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float r = 0.f;
#pragma unroll
    for (int k = 0; k < TL; ++k) r = fmaxf(r, red[k][threadIdx.x]);
    atomicMax(a.vamax + (int64_t)bh * D + threadIdx.x, __float_as_uint(r));
  }
}

// Q / K quantisation: grid (Np/TOK, B*H, 2 (0 = Q, 1 = K)); 256 threads, TPT per
// token (TOK = 256/TPT tokens per workgroup, a multiple of qk_blk), each owning
// CPT = D/TPT consecutive channels.
template <int D, int DT, int ROT, int TPT>
__global__ __launch_bounds__(256) void k1_quant_qk(QuantArgs a) {
  constexpr int TOK = 256 / TPT, CPT = D / TPT;
  extern __shared__ float U[];  // ROT 2: [TOK][D+1] RoPE outputs
  __shared__ float wred[4];
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int64_t Np = a.Np;
  const int bh = blockIdx.y;
  const bool isK = blockIdx.z == 1;
  const int64_t n0 = (int64_t)blockIdx.x * TOK;
  const void* src = isK ? a.k : a.q;
  const void* base = (const char*)src + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  const int lt = threadIdx.x / TPT, part = threadIdx.x % TPT, c0 = part * CPT;
  const int64_t n = n0 + lt;
  const bool valid = n < valid_len(a.nlens, a.lens, bh, s.H, N);
  float v[CPT];
  rotated_slice<DT, ROT, CPT, D>(base, n, valid, D, c0, s, a.table, U + lt * (D + 1), v);
  if ((isK ? a.smooth : a.smooth_q) && valid) {
    const f32x4* mu = (const f32x4*)((isK ? a.kmu : a.qmu) + (int64_t)bh * D + c0);
#pragma unroll
    for (int i = 0; i < CPT / 4; ++i) {
      const f32x4 m4 = mu[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = v[4 * i + e] - m4[e];
    }
  }
  if (isK && a.smooth_q) {
    // dS_n = mu_q . K_n: binary64, channels in order (the products are exact), as one
    // chain through the token's TPT threads; the last one writes it (0 for tokens
    // that do not exist)
    const float* mq = a.qmu + (int64_t)bh * D + c0;
    double acc = 0.0;
#pragma unroll
    for (int stg = 0; stg < TPT; ++stg) {
      if (part == stg) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) acc = fma((double)mq[i], (double)v[i], acc);
      }
      const double prev = __shfl_up(acc, 1, TPT);
      if (part == stg + 1) acc = prev;
    }
    if (part == TPT - 1) a.kbias[(int64_t)bh * Np + n] = valid ? (float)acc : 0.f;
  }
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) am = fmaxf(am, fabsf(v[i]));
  // reduce over the TPT * qk_blk threads of one scale block (at least one wave)
  am = wave_max(am, 64);
  const int grp = TPT * s.qk_blk;
  if (grp > 64) {
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wred[wid] = am;
    __syncthreads();
    const int wpg = grp / 64;  // waves per block
    const int g0 = (wid / wpg) * wpg;
    am = wred[g0];
    for (int k = 1; k < wpg; ++k) am = fmaxf(am, wred[g0 + k]);
  }
  const float inv = am == 0.f ? 0.f : 7.0f / am;
  uint32_t packed[CPT / 8];
#pragma unroll
  for (int w = 0; w < CPT / 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int code = am == 0.f ? 0 : quant_code(v[w * 8 + e], inv);
      word |= ((uint32_t)code & 0xFu) << (4 * e);
    }
    packed[w] = word;
  }
  uint8_t* codes = (isK ? a.kc : a.qc) + ((int64_t)bh * Np + n) * (D / 2) + c0 / 2;
  if (CPT / 8 == 2) {
    *(u32x2*)codes = u32x2{packed[0], packed[CPT / 8 - 1]};
  } else {
#pragma unroll
    for (int w = 0; w < CPT / 8; w += 4)
      *(u32x4*)(codes + 4 * w) = u32x4{packed[w], packed[w + 1], packed[w + 2], packed[w + 3]};
  }
  if (part == 0 && (lt % s.qk_blk) == 0) {
    float* sc = isK ? a.ks : a.qs;
    sc[(int64_t)bh * (Np / s.qk_blk) + n / s.qk_blk] = am == 0.f ? 0.f : am / 7.0f;
  }
}

// V quantisation into the transposed layout [B,H,D,Np/2] plus per-kv-block
// column sums.  grid (Np/128, B*H); thread -> (channel c, token group g).
template <int D, int DT>
__global__ __launch_bounds__(256) void k1_quant_v(QuantArgs a) {
  extern __shared__ __align__(16) char lds[];
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int64_t Np = a.Np;
  const int bh = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * kTile;
  const void* base = (const char*)a.v + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  const int64_t Nb = valid_len(a.nlens, a.lens, bh, s.H, N);
  stage_tile<D, DT>(base, n0, Nb, kTile, lds);
  __syncthreads();
  constexpr int G = 256 / D, TPG = kTile / G;  // groups, tokens per group
  const int c = threadIdx.x % D, g = threadIdx.x / D;
  const float amax = __uint_as_float(a.vamax[(int64_t)bh * D + c]);
  const float inv = amax == 0.f ? 0.f : 7.0f / amax;
  if (blockIdx.x == 0 && g == 0) a.vs[(int64_t)bh * D + c] = amax == 0.f ? 0.f : amax / 7.0f;
  int codes[TPG];
#pragma unroll
  for (int i = 0; i < TPG; ++i) {
    const int r = g * TPG + i;
    const bool valid = n0 + r < Nb;
    codes[i] = (valid && amax != 0.f) ? quant_code(lds_elem<D, DT>(lds, r, c), inv) : 0;
  }
  uint32_t words[TPG / 8];
#pragma unroll
  for (int w = 0; w < TPG / 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= ((uint32_t)codes[w * 8 + e] & 0xFu) << (4 * e);
    words[w] = word;
  }
  uint4* dst = (uint4*)(a.vc + ((int64_t)bh * D + c) * (Np / 2) + (n0 + g * TPG) / 2);
#pragma unroll
  for (int w = 0; w < TPG / 8; w += 4) dst[w / 4] = make_uint4(words[w], words[w + 1], words[w + 2], words[w + 3]);
  if (a.vcol) {
    // column sums per kv block; 16-token chunk sums first (static indices keep
    // everything in registers), then blocks of kv_blk tokens.
    __shared__ int part[256];
    const int kvb = s.kv_blk;
    const int64_t nkb = (N + kvb - 1) / kvb;
    int chunk[TPG / 16];
#pragma unroll
    for (int ch = 0; ch < TPG / 16; ++ch) {
      int acc = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += codes[ch * 16 + i];
      chunk[ch] = acc;
    }
    if (kvb <= TPG) {
      int acc = 0;
#pragma unroll
      for (int ch = 0; ch < TPG / 16; ++ch) {
        acc += chunk[ch];
        if (((ch + 1) * 16) % kvb == 0) {
          const int64_t sblk = (n0 + g * TPG + (ch + 1) * 16 - kvb) / kvb;
          if (sblk < nkb) a.vcol[((int64_t)bh * nkb + sblk) * D + c] = acc;
          acc = 0;
        }
      }
    } else {
      int acc = 0;
#pragma unroll
      for (int ch = 0; ch < TPG / 16; ++ch) acc += chunk[ch];
      part[threadIdx.x] = acc;
      __syncthreads();
      const int gpb = kvb / TPG;  // groups per block
      if (g % gpb == 0) {
        for (int k = 1; k < gpb; ++k) acc += part[(g + k) * D + c];
        const int64_t sblk = (n0 + g * TPG) / kvb;
        if (sblk < nkb) a.vcol[((int64_t)bh * nkb + sblk) * D + c] = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
template <int D, int DT, int ROT, int TPT>
hipError_t launch_qk(const QuantArgs& a, hipStream_t st) {
  constexpr int TOK = 256 / TPT;
  const size_t lds = ROT == 2 ? (size_t)TOK * (D + 1) * 4 : 0;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k1_quant_qk<D, DT, ROT, TPT>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  k1_quant_qk<D, DT, ROT, TPT><<<dim3((unsigned)(a.Np / TOK), (unsigned)(a.s.B * a.s.H), 2), 256, lds, st>>>(a);
  return hipSuccess;
}

template <int D, int DT, int ROT>
hipError_t launch_rot(const QuantArgs& a, hipStream_t st) {
  const int64_t N = (int64_t)a.s.F * a.s.Hs * a.s.Ws;
  const int BH = a.s.B * a.s.H;
  const int nz = (a.smooth ? 1 : 0) + (a.smooth_q ? 1 : 0);
  if (nz > 0) {
    const int64_t nblk = (N + kMeanTile - 1) / kMeanTile;
    const int64_t nmu = (int64_t)nz * BH * D;
    k1_kstats<D, DT, ROT><<<dim3((unsigned)nblk, BH, nz), 256, 0, st>>>(a);
    k1_kmean<<<(unsigned)((nmu + 255) / 256), 256, 0, st>>>(a);
  }
  // a workgroup covers whole scale blocks: 64 tokens (four threads each) unless
  // qk_blk is 128 (then 128 tokens, two threads each)
  return a.s.qk_blk > 64 ? launch_qk<D, DT, ROT, 2>(a, st) : launch_qk<D, DT, ROT, 4>(a, st);
}

template <int D, int DT>
hipError_t launch_quantize_t(const QuantArgs& a, hipStream_t st) {
  const int BH = a.s.B * a.s.H;
  const size_t in_tile = (size_t)kTile * (DT == 0 ? (D + 1) * 4 : (D + 2) * 2);
  const int64_t nvamax = (int64_t)BH * D;
  if (DT == 0) {
    // fp32 tiles exceed the default 64 KiB of dynamic LDS; gfx950 has 160 KiB
    static const hipError_t attr = hipFuncSetAttribute((const void*)k1_quant_v<D, DT>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)in_tile);
    if (attr != hipSuccess) return attr;
  }
  k1_zero_u32<<<(unsigned)((nvamax + 255) / 256), 256, 0, st>>>(a.vamax, nvamax);
  k1_vamax<D, DT><<<dim3((unsigned)((a.Np + kVTile - 1) / kVTile), BH), 256, 0, st>>>(a);
  hipError_t e;
  if (a.rot == 1) e = launch_rot<D, DT, 1>(a, st);
  else if (a.rot == 2) e = launch_rot<D, DT, 2>(a, st);
  else if (a.rot == 3) e = launch_rot<D, DT, 3>(a, st);
  else e = launch_rot<D, DT, 0>(a, st);
  if (e != hipSuccess) return e;
  k1_quant_v<D, DT><<<dim3((unsigned)(a.Np / kTile), BH), 256, in_tile, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, int dtype, hipStream_t st) {
  if (a.s.D == 128) {
    if (dtype == 0) return launch_quantize_t<128, 0>(a, st);
    if (dtype == 1) return launch_quantize_t<128, 1>(a, st);
    return launch_quantize_t<128, 2>(a, st);
  }
  if (dtype == 0) return launch_quantize_t<64, 0>(a, st);
  if (dtype == 1) return launch_quantize_t<64, 1>(a, st);
  return launch_quantize_t<64, 2>(a, st);
}

}  // namespace ra
