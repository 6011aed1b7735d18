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
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "rope.h"

namespace ra {

// Scratch of rotattn_quantize_qk_noalloc: a fixed device array (each device holds
// its own copy from module load until the process ends), for callers that cannot
// allocate.  Host code never uses the array's name as an address: the device
// address of this device's copy comes from hipGetSymbolAddress, looked up once per
// device and kept.
static __device__ __align__(256) uint8_t scratch[kQuantScratchBytes];

hipError_t quant_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

// V channel amax over all tokens.  A workgroup takes kVTile tokens of one head:
// thread t owns 8 consecutive channels (one 16-byte load per token for 16-bit
// inputs) of every (256 / (D/8))-th token, the partial maxima meet in LDS (red,
// at least (256 / (D/8)) x (D+1) floats), and one atomic max per channel on the
// float bits (non-negative floats order like unsigned integers) merges the
// workgroups.
constexpr int kVTile = 512;
template <int D, int DT>
RA_DEV void vamax_tile(const QuantArgs& a, int bh, int64_t tile, float* red) {
  constexpr int CG = D / 8, TL = 256 / CG;  // channel groups, tokens in flight
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int64_t n0 = tile * kVTile;
  const int64_t Nb = valid_len(a.nlens, a.lens, bh, s.H, N);
  const void* base = (const char*)a.v + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  const int cg = threadIdx.x % CG, tl = threadIdx.x / CG;
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.f;
  // batches of kVB tokens per thread, every load of a batch issued before the first
  // is used; tokens at or past Nb read token Nb - 1 (Nb >= 1) and count as 0
  constexpr int kVB = 8;
  static_assert(kVTile % (TL * kVB) == 0, "whole batches");
  for (int r0 = tl; r0 < kVTile; r0 += TL * kVB) {
    float x[kVB][8];
#pragma unroll
    for (int u = 0; u < kVB; ++u) load_slice<DT, 8>(base, min(n0 + r0 + u * TL, Nb - 1), D, 8 * cg, x[u]);
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const bool ok = n0 + r0 + u * TL < Nb;
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], ok ? fabsf(x[u][e]) : 0.f);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tl * (D + 1) + 8 * cg + e] = m[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float r = 0.f;
#pragma unroll
    for (int k = 0; k < TL; ++k) r = fmaxf(r, red[k * (D + 1) + threadIdx.x]);
    atomicMax(a.vamax + (int64_t)bh * D + threadIdx.x, __float_as_uint(r));
  }
}

// V amax on its own (no smoothing statistics to share a launch with): grid
// (ceil(Np / kVTile), B*H).
template <int D, int DT>
__global__ __launch_bounds__(256) void k1_vamax(QuantArgs a) {
  __shared__ float red[(256 / (D / 8)) * (D + 1)];
  vamax_tile<D, DT>(a, blockIdx.y, blockIdx.x, red);
}

// ---------------------------------------------------------------------------------
// Channel statistics for smoothing: ordered binary64 partial sums of rotated K (and,
// with Q smoothing, of rotated Q) over 64-token blocks.  grid (ceil(N/64), B*H, the
// number of smoothed tensors + 1); z = 0 is K unless only Q is smoothed; the last z
// computes the V amax instead (vamax_tile, the first ceil(Np / kVTile) blocks), so
// that V's pure stream overlaps the statistics' arithmetic.  256 threads, each
// owning D/4 channels of one token: wave slices (lane = token) for ROT 0-2, four
// consecutive lanes per token for the Full rotation.  partial [B*H][nblk][D] f64.
template <int D, int DT, int ROT>
__global__ __launch_bounds__(256) void k1_kstats(QuantArgs a) {
  constexpr int TPT = 4, CPT = D / TPT;
  __shared__ float R[kMeanTile * (D + 1)];  // RoPE outputs (Half), then rotated rows
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int bh = blockIdx.y, blk = blockIdx.x;
  if (blockIdx.z == gridDim.z - 1) {
    static_assert((256 / (D / 8)) * (D + 1) <= kMeanTile * (D + 1), "the V amax fits in R");
    if ((int64_t)blk * kVTile < a.Np) vamax_tile<D, DT>(a, bh, blk, R);
    return;
  }
  const bool isQ = blockIdx.z + (a.smooth ? 0 : 1) == 1;
  const int64_t Nb = valid_len(a.nlens, a.lens, bh, s.H, N);
  const int64_t n0 = (int64_t)blk * kMeanTile;
  static_assert(kMeanTile == 64, "one token per lane");
  const int lt = ROT == 3 ? threadIdx.x / TPT : threadIdx.x & 63;
  const int c0 = ROT == 3 ? (threadIdx.x % TPT) * CPT : wave_slice_c0<D>();
  const int64_t n = n0 + lt;
  const void* base = (const char*)(isQ ? a.q : a.k) + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  float x[CPT];
  if constexpr (ROT == 3) rotated_slice<DT, ROT, CPT, D>(base, n, n < Nb, D, c0, s, a.table, R + lt * (D + 1), x);
  else rotated_wave_slice<DT, ROT, D>(base, n, n < Nb, c0, s, a.table, R, lt, x);
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
// binary32.  One workgroup per (b*H + h, tensor z in the order of k1_kstats' z), run
// by k1_mid; thread c < D owns channel c.  The sum is one dependent chain per
// channel; it runs over chunks of kMeanChunk partial rows staged in LDS (buf,
// kMeanChunk * D doubles), the next chunk's loads in flight (in registers) while the
// current one is summed.
constexpr int kMeanChunk = 32;
template <int D>
RA_DEV void kmean_body(const QuantArgs& a, int bh, int z, double* buf) {
  constexpr int PER = kMeanChunk * D / 256;  // partials each thread stages per chunk
  const int64_t N = (int64_t)a.s.F * a.s.Hs * a.s.Ws;
  const int64_t nblk = (N + kMeanTile - 1) / kMeanTile;
  const bool isQ = z + (a.smooth ? 0 : 1) == 1;
  const double* p = (isQ ? a.qpart : a.kpart) + (int64_t)bh * nblk * D;
  const int tid = threadIdx.x;
  double nxt[PER];
  auto fetch = [&](int64_t b0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i;  // row e / D, channel e % D of the chunk
      nxt[i] = b0 + e / D < nblk ? p[b0 * D + e] : 0.0;
    }
  };
  double total = 0.0;
  fetch(0);
  for (int64_t b0 = 0; b0 < nblk; b0 += kMeanChunk) {
    __syncthreads();  // the previous chunk has been summed
#pragma unroll
    for (int i = 0; i < PER; ++i) buf[tid + 256 * i] = nxt[i];
    __syncthreads();
    if (b0 + kMeanChunk < nblk) fetch(b0 + kMeanChunk);
    if (tid < D) {
      const int rows = (int)min((int64_t)kMeanChunk, nblk - b0);
      for (int r = 0; r < rows; ++r) total += buf[r * D + tid];
    }
  }
  // blocks past the valid tokens hold +0.0 partials: adding them changes nothing
  if (tid < D) {
    const int64_t Nb = valid_len(a.nlens, a.lens, bh, a.s.H, N);
    (isQ ? a.qmu : a.kmu)[(int64_t)bh * D + tid] = (float)(total / (double)Nb);
  }
}

__global__ void k1_zero_u32(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// LDS of one workgroup of the wave-sliced quantiser: the Half exchange rows, the
// scale-block maxima of the four waves, and the hand-on of the dS chain.
template <int D, int ROT>
struct QkwsLds {
  float U[ROT == 2 ? 64 * (D + 1) : 1];
  uint32_t wred[256];
  double dsacc[64];
};

// Q / K quantisation, wave-sliced (ROT 0-2, qk_blk <= 64): one workgroup takes
// tokens 64 blk .. 64 blk + 63 of head bh, of Q or of K; lane = token, wave w =
// channels [w D/4, (w+1) D/4).  A scale block is qk_blk consecutive lanes of all four
// waves: its amax is a lane-group maximum in each wave, then the four waves' values
// through LDS.
template <int D, int DT, int ROT>
RA_DEV void quant_qk_ws_body(const QuantArgs& a, int64_t blk, int bh, bool isK, QkwsLds<D, ROT>& L) {
  constexpr int CPT = D / 4;
  float* const U = L.U;
  uint32_t* const wred = L.wred;
  double* const dsacc = L.dsacc;
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int64_t Np = a.Np;
  const int lane = threadIdx.x & 63;
  const int c0 = wave_slice_c0<D>(), w = c0 / CPT;
  const int64_t n = blk * 64 + lane;
  const void* base = (const char*)(isK ? a.k : a.q) + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  const bool valid = n < valid_len(a.nlens, a.lens, bh, s.H, N);
  // the smoothing mean (and mu_q for the dS chain): the words of the wave's channel
  // slice are the same for every lane, read through the scalar cache (constant
  // address space: nothing writes them during the launch), so they need neither an
  // LDS copy nor a wait ahead of the token loads
  typedef const __attribute__((address_space(4))) float* cfloat_ptr;
  const bool smooth = isK ? a.smooth : a.smooth_q, chain = isK && a.smooth_q;
  const cfloat_ptr mus = (cfloat_ptr)((isK ? a.kmu : a.qmu) + (int64_t)bh * D + c0);
  const cfloat_ptr mqs = (cfloat_ptr)(a.qmu + (int64_t)bh * D + c0);
  float v[CPT];
  rotated_wave_slice<DT, ROT, D>(base, n, valid, c0, s, a.table, U, lane, v);
  if (smooth) {
    // tokens that do not exist are smoothed too: their amax contribution is dropped
    // below and their codes are 0 (inv = 0)
#pragma unroll
    for (int i = 0; i < CPT; ++i) v[i] = v[i] - mus[i];
  }
  if (chain) {
    // dS_n = mu_q . K_n: binary64, channels in order (the products are exact), one
    // chain through the four waves' slices in turn; wave 3 writes it (0 for tokens
    // that do not exist)
    double acc = 0.0;
    for (int stg = 0; stg < 4; ++stg) {
      if (w == stg) {
        if (stg > 0) acc = dsacc[lane];
#pragma unroll
        for (int i = 0; i < CPT; ++i) acc = fma((double)mqs[i], (double)v[i], acc);
        dsacc[lane] = acc;
      }
      __syncthreads();
    }
    if (w == 3) a.kbias[(int64_t)bh * Np + n] = valid ? (float)acc : 0.f;
  }
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) am = fmaxf(am, fabsf(v[i]));
  if (!valid) am = 0.f;
  wred[threadIdx.x] = group_max_u32(__float_as_uint(am), s.qk_blk);
  __syncthreads();
  am = __uint_as_float(max(max(wred[lane], wred[64 + lane]), max(wred[128 + lane], wred[192 + lane])));
  // tokens that do not exist hold zeros; inv = 0 gives them code 0 also where 7/am
  // overflows (0 * inf would give the NaN code)
  const float inv = (am == 0.f || !valid) ? 0.f : 7.0f / am;
  uint32_t packed[CPT / 8];
  pack_codes<CPT>(v, inv, packed);
  uint8_t* codes = (isK ? a.kc : a.qc) + ((int64_t)bh * Np + n) * (D / 2) + c0 / 2;
  if (CPT / 8 == 2) {
    *(u32x2*)codes = u32x2{packed[0], packed[CPT / 8 - 1]};
  } else {
#pragma unroll
    for (int q = 0; q < CPT / 8; q += 4)
      *(u32x4*)(codes + 4 * q) = u32x4{packed[q], packed[q + 1], packed[q + 2], packed[q + 3]};
  }
  if (w == 0 && (lane % s.qk_blk) == 0) {
    float* sc = isK ? a.ks : a.qs;
    sc[(int64_t)bh * (Np / s.qk_blk) + n / s.qk_blk] = am == 0.f ? 0.f : am / 7.0f;
  }
}

// grid (Np/64, B*H, tensors): z = z0 + blockIdx.z, 0 = Q, 1 = K.
template <int D, int DT, int ROT>
__global__ __launch_bounds__(256) void k1_quant_qk_ws(QuantArgs a, int z0) {
  __shared__ QkwsLds<D, ROT> L;
  quant_qk_ws_body<D, DT, ROT>(a, blockIdx.x, blockIdx.y, z0 + (int)blockIdx.z == 1, L);
}

// Q / K quantisation, token-sliced (the Full rotation, and qk_blk = 128): grid
// (Np/TOK, B*H, 2 (0 = Q, 1 = K)); 256 threads, TPT per
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
  // reduce over the TPT * qk_blk threads of one scale block (consecutive lanes, or
  // whole waves)
  const int grp = TPT * s.qk_blk;
  am = wave_max(am, grp < 64 ? grp : 64);
  if (grp > 64) {
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wred[wid] = am;
    __syncthreads();
    const int wpg = grp / 64;  // waves per block
    const int g0 = (wid / wpg) * wpg;
    am = wred[g0];
    for (int k = 1; k < wpg; ++k) am = fmaxf(am, wred[g0 + k]);
  }
  // tokens that do not exist hold zeros; inv = 0 gives them code 0 also where 7/am
  // overflows (0 * inf would give the NaN code)
  const float inv = (am == 0.f || !valid) ? 0.f : 7.0f / am;
  uint32_t packed[CPT / 8];
  pack_codes<CPT>(v, inv, packed);
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
// column sums: one workgroup per kTile tokens (tile) of head bh, LDS lds of
// v_tile_bytes<D, DT>(); thread -> (channel c, token group g).
template <int D, int DT>
constexpr int v_tile_bytes() { return kTile * (DT == 0 ? (D + 1) * 4 : (D + 2) * 2); }
template <int D, int DT>
RA_DEV void quant_v_body(const QuantArgs& a, int64_t tile, int bh, char* lds) {
  const Shape s = a.s;
  const int64_t N = (int64_t)s.F * s.Hs * s.Ws;
  const int64_t Np = a.Np;
  const int64_t n0 = tile * kTile;
  const void* base = (const char*)a.v + (size_t)bh * N * D * (DT == 0 ? 4 : 2);
  const int64_t Nb = valid_len(a.nlens, a.lens, bh, s.H, N);
  constexpr int G = 256 / D, TPG = kTile / G;  // groups, tokens per group
  const int c = threadIdx.x % D, g = threadIdx.x / D;
  const float amax = __uint_as_float(a.vamax[(int64_t)bh * D + c]);  // in flight with the tile
  stage_tile<D, DT, kTile>(base, n0, Nb, lds);
  __syncthreads();
  const float inv = amax == 0.f ? 0.f : 7.0f / amax;
  if (tile == 0 && g == 0) a.vs[(int64_t)bh * D + c] = amax == 0.f ? 0.f : amax / 7.0f;
  float vals[TPG];
#pragma unroll
  for (int i = 0; i < TPG; ++i) vals[i] = lds_elem<D, DT>(lds, g * TPG + i, c);
  uint32_t cb[TPG];
  code_bits_n<TPG>(vals, inv, cb);
  if (n0 + kTile > Nb) {
    // rows past the valid tokens (staged as zeros) take code 0, also where 7/amax
    // overflows and 0 * inf would give the NaN code
#pragma unroll
    for (int i = 0; i < TPG; ++i)
      if (n0 + g * TPG + i >= Nb) cb[i] = kZeroCodeBits;
  }
  uint32_t words[TPG / 8];
#pragma unroll
  for (int w = 0; w < TPG / 8; ++w) words[w] = pack8(cb + 8 * w);
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
      uint32_t acc = 0;  // sum of 16 code bits: the codes' sum plus 16 kZeroCodeBits (mod 2^32)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += cb[ch * 16 + i];
      chunk[ch] = (int)(acc - 16u * kZeroCodeBits);
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
      if (kvb <= kTile) {
        const int gpb = kvb / TPG;  // groups per block
        if (g % gpb == 0) {
          for (int k = 1; k < gpb; ++k) acc += part[(g + k) * D + c];
          const int64_t sblk = (n0 + g * TPG) / kvb;
          if (sblk < nkb) a.vcol[((int64_t)bh * nkb + sblk) * D + c] = acc;
        }
      } else if (g == 0) {
        // a kv block spans several workgroups: each adds its tile's sum (integer
        // atomics, so the result does not depend on their order; cleared first)
        for (int k = 1; k < G; ++k) acc += part[k * D + c];
        const int64_t sblk = n0 / kvb;
        if (sblk < nkb) atomicAdd(a.vcol + ((int64_t)bh * nkb + sblk) * D + c, acc);
      }
    }
  }
}

// The launch between the statistics and the K codes: the channel means (one
// workgroup per head and smoothed tensor, first in dispatch order, so that their
// dependent chains run beside the streams), the V codes (they need the V amax of
// the statistics launch) and, when Q is not smoothed (its codes need no statistics),
// the Q codes.  Per head and 128-token tile the workgroups are: V tile, and with Q
// two 64-token Q blocks, so that the V stream and the Q arithmetic share the CUs.
// One dynamic LDS buffer serves whichever part a workgroup runs.  1-D grid.
template <int D, int DT, int ROT>
constexpr int mid_lds_bytes() {
  constexpr int q = (int)sizeof(QkwsLds<D, ROT>), v = v_tile_bytes<D, DT>(), m = kMeanChunk * D * 8;
  return q > v ? (q > m ? q : m) : (v > m ? v : m);
}
template <int D, int DT, int ROT>
__global__ __launch_bounds__(256) void k1_mid(QuantArgs a, int nmean, int withq) {
  extern __shared__ __align__(16) char lds[];
  const int64_t id = blockIdx.x;
  const int BH = a.s.B * a.s.H;
  if (id < (int64_t)BH * nmean) {
    kmean_body<D>(a, (int)(id % BH), (int)(id / BH), (double*)lds);
    return;
  }
  const int per = withq ? 3 : 1;  // workgroups per head and tile
  const int64_t r = id - (int64_t)BH * nmean, ntile = a.Np / kTile;
  const int bh = (int)(r / (ntile * per));
  const int64_t u = r % (ntile * per), tile = u / per;
  const int j = (int)(u % per);
  if (j == 0) quant_v_body<D, DT>(a, tile, bh, lds);
  else if constexpr (ROT <= 2) quant_qk_ws_body<D, DT, ROT>(a, 2 * tile + (j - 1), bh, false, *(QkwsLds<D, ROT>*)lds);
}

// ---------------------------------------------------------------------------------
template <int D, int DT, int ROT, int TPT>
hipError_t launch_qk(const QuantArgs& a, hipStream_t st) {
  constexpr int TOK = 256 / TPT;
  const size_t lds = ROT == 2 ? (size_t)TOK * (D + 1) * 4 : 0;
  const hipError_t attr = hipFuncSetAttribute((const void*)k1_quant_qk<D, DT, ROT, TPT>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  k1_quant_qk<D, DT, ROT, TPT><<<dim3((unsigned)(a.Np / TOK), (unsigned)(a.s.B * a.s.H), 2), 256, lds, st>>>(a);
  return hipSuccess;
}

// Launch order: clear the V amax (and the column sums when a kv block spans several
// tiles); the statistics (K and Q sums with the V amax, or the V amax alone); k1_mid
// (the means, the V codes, and the Q codes when Q needs no mean); the remaining Q/K
// codes.
template <int D, int DT, int ROT>
hipError_t launch_rot(const QuantArgs& a, hipStream_t st) {
  const int64_t N = (int64_t)a.s.F * a.s.Hs * a.s.Ws;
  const int BH = a.s.B * a.s.H;
  const int nz = (a.smooth ? 1 : 0) + (a.smooth_q ? 1 : 0);
  if (nz > 0) {
    // the statistics, with the V amax as the launch's last z
    const int64_t nblk = (N + kMeanTile - 1) / kMeanTile;
    k1_kstats<D, DT, ROT><<<dim3((unsigned)nblk, BH, nz + 1), 256, 0, st>>>(a);
  } else {
    k1_vamax<D, DT><<<dim3((unsigned)((a.Np + kVTile - 1) / kVTile), BH), 256, 0, st>>>(a);
  }
  // the wave-sliced Q/K kernel takes scale blocks of up to 64 tokens; the Full
  // rotation and qk_blk = 128 use the token-sliced one for both tensors
  const bool ws = ROT <= 2 && a.s.qk_blk <= 64;
  const bool withq = ws && !a.smooth_q;
  constexpr int mid_lds = mid_lds_bytes<D, DT, ROT>();
  const hipError_t attr = hipFuncSetAttribute((const void*)k1_mid<D, DT, ROT>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, mid_lds);
  if (attr != hipSuccess) return attr;
  const int64_t nmid = (int64_t)BH * nz + (int64_t)BH * (a.Np / kTile) * (withq ? 3 : 1);
  k1_mid<D, DT, ROT><<<(unsigned)nmid, 256, mid_lds, st>>>(a, nz, withq ? 1 : 0);
  if (a.s.qk_blk > 64) return launch_qk<D, DT, ROT, 2>(a, st);
  if constexpr (ROT == 3) {
    return launch_qk<D, DT, ROT, 4>(a, st);
  } else {
    k1_quant_qk_ws<D, DT, ROT>
        <<<dim3((unsigned)(a.Np / 64), (unsigned)BH, withq ? 1 : 2), 256, 0, st>>>(a, withq ? 1 : 0);
    return hipSuccess;
  }
}

template <int D, int DT>
hipError_t launch_quantize_t(const QuantArgs& a, hipStream_t st) {
  const int BH = a.s.B * a.s.H;
  const int64_t nvamax = (int64_t)BH * D;
  k1_zero_u32<<<(unsigned)((nvamax + 255) / 256), 256, 0, st>>>(a.vamax, nvamax);  // V amax starts at 0
  if (a.vcol && a.s.kv_blk > kTile) {
    // column sums that several V tiles add into (integer atomics) start at 0
    const int64_t ncol = (int64_t)BH * ((a.s.F * (int64_t)a.s.Hs * a.s.Ws + a.s.kv_blk - 1) / a.s.kv_blk) * D;
    k1_zero_u32<<<(unsigned)((ncol + 255) / 256), 256, 0, st>>>((uint32_t*)a.vcol, ncol);
  }
  hipError_t e;
  if (a.rot == 1) e = launch_rot<D, DT, 1>(a, st);
  else if (a.rot == 2) e = launch_rot<D, DT, 2>(a, st);
  else if (a.rot == 3) e = launch_rot<D, DT, 3>(a, st);
  else e = launch_rot<D, DT, 0>(a, st);
  if (e != hipSuccess) return e;
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
