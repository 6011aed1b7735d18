// K2: INT4 FlashAttention forward with range-rectified P codes (kernels and their
// launch templates; attention_inst.hip instantiates them once per head dimension
// and step size, attention.hip dispatches).
//
// RotateAttention (arXiv 2607.02584), papernotes.org note: framework flowchart
// (INT4 Q K^T -> scores -> range-rectified P -> INT4 P V) and "Key design 2"
// (P = exp(S - m) in (0, 1] with m the running row maximum; code
// round(15 P) - 8 in [-8, 7], fixed scale 15, zero point -8).
//
// gfx950 design
//  * A staging pass (k2_stage) turns each head's INT4 K and V codes into the exact
//    byte image one key group occupies in LDS: K as packed fp6 e2m3 (every code in
//    [-7, 7] is exact in e2m3; 6 bits per value) with rows permuted for the S^T
//    register layout, V^T as fp8 e4m3 (also exact), rows padded so that the LDS
//    reads of consecutive rows hit distinct banks (32 KiB per 128-key group for
//    D = 128; the copy stream is a bound at the margin, so the level thresholds live
//    in a small LDS array of their own).  The main loop copies groups straight from global memory into LDS
//    (buffer_load_dwordx4 ... lds) into a ring of LDS slots and spends no VALU on
//    staging.  A group of 128 keys holds several online-softmax steps (one barrier
//    and one copy per group).
//  * One workgroup = 4 waves x 32 query rows.  Each wave computes S^T = K Q^T on
//    v_mfma_scale_f32_32x32x64_f8f6f4 with fp6 operands (unit scales), which runs
//    at twice the rate of the fp8 and int8 forms.  Products of INT4 values and
//    their sums (|A| <= 49 D < 2^24) are exact in fp32, so the scores arrive as
//    exact integers in float registers.  A lane owns one query row and 16 keys of
//    every 32-key tile; its P levels are already laid out as the B operand of
//    O^T = V^T P^T on the same instruction in its fp8 form, with no LDS round trip.
//    The scores of the next step are issued before the softmax of the current one.
//  * The P level r = round-half-even(2^y) is taken from the hardware exp2: with
//    t = 2^y + 128.5 + 2^-16 the level is byte 2 of t's bits and the low 16 bits
//    carry the rounding margin.  v_exp_f32 is within 1.5 * 2^-24 relative of 2^y,
//    so whenever the margin is above one unit of 2^-16 the level equals the exact
//    one; the (rare) other elements are decided exactly against the 15 thresholds.  The
//    level byte r in [0, 15], read as the fp8 code r * 2^-9 with a B scale of 2^9,
//    is the operand: sum_j (P~_j + 8) v_j = sum_j r_j v_j folds the zero point into
//    the product, and every product and sum is an exact integer in fp32.
//  * Exact skips: a tile pair whose every level is 0 (decided from the exact tile
//    maximum of y) adds exact zeros, so it skips the level packing, the P V MFMA
//    and the V reads; a tile whose every p is below half an ulp of l would not
//    change l, so it also skips the exp.  Both leave every result bit-identical.
//  * The fp32 accumulator holds exact integer sums between moves of the row
//    maximum and is rescaled in place when a maximum in the wave moves.
//  * Two waves per SIMD (<= 256 registers each), so that one wave's MFMAs run
//    under the other's softmax; one barrier per key group.
//  * Workgroup ids are remapped so that the query tiles of a head run on the same
//    XCD and share its L2 for the K/V stream.
#pragma once
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace ra {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;
constexpr float kMagic = 128.5f + 1.0f / 65536.0f;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// minimum of the low 16 bits of three values (v_min3_u16; only the low half of the
// result is meaningful)
RA_DEV uint32_t min3_u16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_min3_u16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// ---- the P level r = round-half-even(2^y) in [0, 15] of an exponent y -------------
// (y = log2(15 P); 2^-1 is the only tie a binary32 y reaches, and it rounds to 0.)
// Fast level: with t = p + kMagic, p the hardware exp2 of y (within 1.5 * 2^-24
// relative of 2^y), the sum lies in [128, 256) where the ulp is 2^-16, so byte 2 of
// t's bits is the nearest integer to p and the low 16 bits are the distance to the
// rounding boundary below.  In units of 2^-16 the computed value exceeds the exact
// 2^y + 0.5 by the 1-unit offset, give or take the exp error (at most 1.5 * 2^-24 *
// 16 = 0.094 units) and the add's rounding (0.5 units), i.e. by 0.406 to 1.594 units:
// it never falls below a boundary the exact value lies above (the offset is larger
// than the 0.594 units of error), and it lies above one the exact value is below (or
// on: the tie 2^y = 0.5 at y = -1) only with a margin of at most 1.594 units, that is
// at most 1 (t sits on the 2^-16 grid, so the margin is a whole number of units).  A
// margin above kMarginMin = 1 therefore makes the fast level the exact one.
// Otherwise the exact level is fixed from y by the two thresholds around the fast
// level (it is within one of the exact level): T[k-1] is the smallest binary32 y
// with level >= k, T[15] = T[16] = +inf.  Every y the attention forms is at most
// L15 plus half an ulp of the running maximum, so p stays below 16 (the maximum
// guard below sends larger ones to the exact path).
constexpr uint32_t kMarginMin = 1;
RA_DEV uint32_t level_bits(float p) { return __float_as_uint(p + kMagic); }
RA_DEV int fast_level(uint32_t t) { return (int)((t >> 16) & 0xFFu); }
RA_DEV bool margin_clear(uint32_t t) { return (t & 0xFFFFu) > kMarginMin; }
RA_DEV int exact_level(float y, int rf, const float* T) {
  const int rh = min(rf, 16);
  const float lo = T[max(rh - 1, 0)], hi = T[rh];
  return rh - ((rh > 0 && y < lo) ? 1 : 0) + ((y >= hi) ? 1 : 0);
}
// The per-key decision as the attention makes it: the fast level when its margin
// is clear, else the exact fix (a pair with any unclear margin fixes every key,
// which leaves clear ones unchanged).
RA_DEV int decide_level(float y, float p, const float* T) {
  const uint32_t t = level_bits(p);
  return margin_clear(t) ? fast_level(t) : exact_level(y, fast_level(t), T);
}

RA_DEV uint32_t pack_b2(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t x = __builtin_amdgcn_perm(b, a, 0x0c0c0602u);
  const uint32_t y = __builtin_amdgcn_perm(d, c, 0x0c0c0602u);
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}

// SM, how a step's K scales vary: 0 one per 16-key unit (qk_blk >= 16); 1 one for
// the whole step (qk_blk >= kv_blk); 2 one per key (qk_blk < 16, per-token scales),
// staged with the group image.  QS: the image also carries the keys' Q-smoothing
// score terms.
template <int D, int KVB, int SM = 0, bool QS = false>
struct Geo {
  // keys per group (staged together; a group holds whole online-softmax steps)
  static constexpr int TG = KVB < 32 ? 32 : (KVB > 128 ? KVB : 128);
  static constexpr int NT = TG / 32;              // 32-key MFMA tiles per group
  static constexpr int TPS = KVB < 32 ? 1 : KVB / 32;  // tiles per online-softmax step
  static constexpr int NSG = NT / TPS;            // steps (tile blocks) per group
  static constexpr int NDB = D / 32;              // 32-row d blocks of O^T
  static constexpr int KC = D / 64;               // 64-deep chunks of Q K^T (fp6 MFMA)
  static constexpr int KB = 3 * D / 4;            // packed fp6 bytes per K row
  static constexpr int KROW = (KB + 16) / 4 % 8 == 0 ? KB + 32 : KB + 16;
  static constexpr int VROW = TG + 16;            // bytes per V^T row (fp8 + pad)
  static constexpr int VOFF = TG * KROW;          // V^T rows start here
  static constexpr int DOFF = VOFF + D * VROW;    // TG floats: per-key score terms (QS)
  static constexpr int SOFF = DOFF + (QS ? 4 * TG : 0);  // TG floats: per-key K scales (SM 2)
  // one group's image, a whole number of 4 KiB copy rounds (K and V^T alone are
  // exactly 32 KiB for D = 128 and 128-key groups)
  static constexpr int IMG = ((SOFF + (SM == 2 ? 4 * TG : 0)) + 4095) / 4096 * 4096;
  static constexpr int NDMA = IMG / 4096;         // 16-byte copies per thread per group
  static constexpr int NB = 4 * IMG <= 81920 ? 4 : 2;  // ring slots (two workgroups per CU)
  static constexpr int LDS = NB * IMG;
  // waves per SIMD of the production kernel: two (<= 256 registers each), one for
  // 256-key steps (eight score tiles live, and 128 KiB or more of LDS per workgroup)
  static constexpr int WPE = KVB > 128 ? 1 : 2;
};
// key (within its 32-key tile) held by K image row rho: row (v&3) + 8(v>>2) + 4h
// holds key 16h + v, so lane half h of the S^T accumulator sees keys 16h..16h+15
RA_DEV int key_of_row(int rho) { return 16 * ((rho >> 2) & 1) + (rho & 3) + 4 * (rho >> 3); }

RA_DEV int nib(uint32_t w, int e) { return (int)((w >> (4 * e)) << 28) >> 28; }  // signed nibble e

// fp8 e4m3 bytes of two integers in [-7, 7] (exact), in the low 16 bits
RA_DEV uint32_t fp8_pair(int c0, int c1) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((float)c0, (float)c1, 0, false) & 0xFFFFu;
}

// fp6 e2m3 code of an integer in [-7, 7]: sign bit 5, exponent bits 4..3 (bias 1),
// mantissa bits 2..0.  Magnitudes 0..7 encode as 00, 08, 10, 14, 18, 1A, 1C, 1E (hex).
RA_DEV uint32_t e2m3(int v) {
  const uint32_t a = (uint32_t)(v < 0 ? -v : v);
  const uint32_t m = (a < 4 ? 0x14100800u >> (8 * a) : 0x1E1C1A18u >> (8 * (a - 4))) & 0xFFu;
  return m | (v < 0 ? 0x20u : 0u);
}

// 32 signed nibbles (code bytes, low nibble first) -> the 32 fp6 values of one MFMA
// operand: value i at bits 6i .. 6i+5 of six little-endian dwords.
RA_DEV void pack_fp6(const u32x4 w, uint32_t (&o)[6]) {
#pragma unroll
  for (int j = 0; j < 6; ++j) o[j] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e2m3(nib(w[i >> 3], i & 7));
    const int b = 6 * i, d = b >> 5, sh = b & 31;
    o[d] |= c << sh;
    if (sh > 26) o[d + 1] |= c >> (32 - sh);
  }
}

// ---- staging: INT4 codes -> per-group LDS images ---------------------------------
// grid (Np / TG, nheads); the image of group g of head bh is at
// img + (bh * (Np / TG) + g) * IMG.
template <int D, int KVB, int SM, bool QS>
__global__ __launch_bounds__(256) void k2_stage(const AttnArgs args) {
  using G = Geo<D, KVB, SM, QS>;
  const int bh = args.heads[blockIdx.y];
  const int g = blockIdx.x;
  const int64_t Np = args.Np;
  const int64_t at = ((int64_t)bh * (Np / G::TG) + g) * G::IMG;
  if (at + G::IMG > args.img_bytes) return;
  uint8_t* img = args.img + at;
  // K: TG rows of D fp6 values.  Chunk c = 2 kc + h (channels 32c .. 32c+31, the
  // operand of lane half h for the kc-th 64-deep MFMA) fills bytes 32c .. 32c+23 of
  // the row (32c+24 .. 32c+31 hold zeros), so that every lane reads its operand with
  // two 16-byte loads straight into the operand's registers.
  // V^T: D rows x TG fp8 e4m3 values.  With steps of 64 or more keys, the 16-key
  // chunks of each 64-key segment are stored in the k order of one 64-deep MFMA:
  // position 32h + 16t' holds keys 32t' + 16h .. +15 (tile t' of the pair, lane
  // half h), so a lane half reads its 32 keys as one contiguous run.
  // Every thread issues all of its 16-byte loads (K: one row chunk; V: 32 keys of
  // one channel) before it converts and stores any of them.
  constexpr int KU = G::TG * D / 32, KIT = (KU + 255) / 256;
  constexpr int VU = D * G::TG / 32, VIT = (VU + 255) / 256;
  u32x4 kw[KIT], vw[VIT];
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (KU % 256 == 0 || u < KU) {
      const int rho = u / (D / 32), c = u % (D / 32);
      const int key = g * G::TG + (rho & ~31) + key_of_row(rho & 31);
      kw[i] = *(const u32x4*)(args.kc + ((int64_t)bh * Np + key) * (D / 2) + 16 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (VU % 256 == 0 || u < VU) {
      const int d = u / (G::TG / 32), c2 = u % (G::TG / 32);
      vw[i] = *(const u32x4*)(args.vc + ((int64_t)bh * D + d) * (Np / 2) + (g * G::TG + 32 * c2) / 2);
    }
  }
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (KU % 256 == 0 || u < KU) {
      const int rho = u / (D / 32), c = u % (D / 32);
      uint32_t o[6];
      pack_fp6(kw[i], o);
      uint8_t* row = img + rho * G::KROW;
      *(i32x4*)(row + 16 * c) = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
      *(u32x2*)(row + D / 2 + 8 * c + 8 * ((rho >> 3) & 1)) = u32x2{o[4], o[5]};
    }
  }
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (VU % 256 == 0 || u < VU) {
      const int d = u / (G::TG / 32), c2 = u % (G::TG / 32);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = 2 * c2 + half;  // 16-key chunk
        i32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = vw[i][2 * half + (q >> 1)];
          const int e0 = 4 * (q & 1);
          o[q] = (int)(fp8_pair(nib(x, e0), nib(x, e0 + 1)) | (fp8_pair(nib(x, e0 + 2), nib(x, e0 + 3)) << 16));
        }
        const int cq = KVB >= 64 ? (c & ~3) | ((c & 1) << 1) | ((c >> 1) & 1) : c;
        *(i32x4*)(img + G::VOFF + d * G::VROW + 16 * cq) = o;
      }
    }
  }
  // Q smoothing: the keys' score terms in log2 units, delta_j = fl(dS_j * C0), in
  // key order (the S^T accumulator holds key 32t + 16h + v of tile t in register v
  // of lane half h)
  if (QS && threadIdx.x < G::TG)
    ((float*)(img + G::DOFF))[threadIdx.x] = args.kbias[(int64_t)bh * Np + g * G::TG + threadIdx.x] * args.C0;
  // per-token K scales (qk_blk < 16), in key order
  if (SM == 2 && threadIdx.x < G::TG) {
    const int sh = __builtin_ctz(args.qk_blk);
    ((float*)(img + G::SOFF))[threadIdx.x] = args.ks[(int64_t)bh * (Np >> sh) + ((g * G::TG + threadIdx.x) >> sh)];
  }
}

// The fields the device helpers need, copied out of the kernel argument block
// (which also holds the head list and stays in the kernarg segment).
struct Ctx {
  const uint8_t* img;
  const float* ks;
  int64_t Np;
  int N, qk_shift;
  int klim;  // keys this lane's query row sees: N, or its block-causal limit
  bool kb;   // per-key score terms staged (Q smoothing)
  float C0, L15;
  float T0;  // the first level threshold: r >= 1 iff y >= T0
  const float* T;  // the 15 level thresholds, then +inf, +inf (LDS)
  int p_zero;
  int dbg_row0, dbg_n;
  int32_t* dbg_aqk;
  int8_t* dbg_p;
  int32_t* dbg_apv;
};

// Per-lane running state of one query row (the lane pair l, l^32 shares a row):
// the output numerator sum_j 2^(m_j - m) r_j v_j in fp32 (m_j the running maximum
// when key j was added), the running maximum m and l = sum_j 2^(y_j + m_j - m).
// Between moves of m the MFMA adds exact integer sums; a move rescales in place.
// What the exact skips saved, counted (wave-uniform) only by the instance that
// reports it: P V units (one MFMA decision each), the units skipped as all-zero,
// score tiles and those whose exps were skipped, and the units that took the
// exact-level path.  The timed instance carries NoCount, whose calls vanish.
struct NoCount {
  RA_DEV void unit(int) {}
  RA_DEV void unit_skip() {}
  RA_DEV void exp_skip() {}
  RA_DEV void fix() {}
};
struct SkipCount {
  uint32_t n_pv = 0, n_pv_skip = 0, n_tile = 0, n_exp_skip = 0, n_fix = 0;
  RA_DEV void unit(int tiles) { n_pv += 1; n_tile += tiles; }
  RA_DEV void unit_skip() { n_pv_skip += 1; }
  RA_DEV void exp_skip() { n_exp_skip += 1; }
  RA_DEV void fix() { n_fix += 1; }
};
template <int NDB, class C>
struct RowState {
  f32x16 acc[NDB];
  float m, l;
  C cnt;
};

// Copy the LDS image of group g into ring slot `buf`: wave w copies the w-th quarter
// of the image, one contiguous kilobyte per copy (dma_all), through a buffer resource
// over the head's images; the lane offset is the only vector operand, the group and
// wave offsets are scalar.
template <int D, int KVB, int SM, bool QS>
RA_DEV void dma_group(__amdgpu_buffer_rsrc_t r, int g, uint8_t* buf) {
  using G = Geo<D, KVB, SM, QS>;
  constexpr int WB = G::NDMA * 1024;  // bytes per wave
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  dma_all(std::make_integer_sequence<int, G::NDMA>{}, r, buf + w * WB, 16 * (threadIdx.x & 63),
          g * G::IMG + w * WB);
}

template <int D, int KVB>
RA_DEV void qk_tiles(const uint8_t* Kl, int tb, const i32x8 (&qop)[Geo<D, KVB>::KC],
                     f32x16 (&st)[Geo<D, KVB>::TPS]) {
  using G = Geo<D, KVB>;
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < G::TPS; ++t) {
    const uint8_t* row = Kl + ((tb + t) * 32 + col) * G::KROW;
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) {
      const int c = 2 * kc + h;
      const i32x4 lo = *(const i32x4*)(row + 16 * c);
      const i32x2 hi = *(const i32x2*)(row + D / 2 + 8 * c + 8 * ((col >> 3) & 1));
      // six dwords of fp6 values (format 2 = e2m3 for both operands); the last two
      // operand dwords are not read by the instruction
      const i32x8 kop = __builtin_shufflevector(lo, __builtin_shufflevector(hi, hi, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5, -1, -1);
      const f32x16 zero = {0};
      st[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop, qop[kc], kc == 0 ? zero : st[t], 2, 2, 0,
                                                               127, 0, 127);
    }
  }
}

// One online-softmax step on tiles tb..tb+TPS-1 of group g (for kv_blk 16, the two
// halves of tile tb as two steps): running max, rescale, the exact skips, P levels,
// P^T operand, P V MFMAs.  MASK: the group holds keys at or past some row's limit (keys >= N,
// or keys a block-causal row does not see); they count as absent.  SM 1: one K scale
// for the whole step, so the maximum needs one multiplication; SM 2 (per-key K scales,
// Sl the group's scales in LDS): without Q smoothing each key's c = fl(fl(sq sk_j) C0)
// is formed for the running maximum, and the scores of the tiles whose exps are
// computed are replaced by their exponents y; the skip tests take a bound of y from
// the tile's maximum of t_j = fl(A_j c_j).
template <int D, int KVB, bool DBG, bool MASK, int SM, class RS>
RA_DEV void softmax_pv(const Ctx& a, int g, int tb, int step0, const uint8_t* Vl, const float* Tl,
                       const float* Sl, float sq, f32x16 (&st)[Geo<D, KVB>::TPS],
                       const float (&ct)[Geo<D, KVB>::TPS], const f32x16 (&sa)[Geo<D, KVB>::TPS],
                       RS& S, bool dbg_row, int dr) {
  using G = Geo<D, KVB>;
  constexpr bool US = SM == 1;
  // per-key scales without Q smoothing (with it, group_iter has already formed the
  // scores t = fma(A, c_j, delta_j) and set c = 1)
  const bool pk = SM == 2 && !a.kb;
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
  const int N = (int)a.N;
  const int j0 = g * G::TG + tb * 32;  // first key of the step's tiles
  const int nsteps = (N + KVB - 1) / KVB;
  constexpr int NSTEP = KVB < 32 ? 2 : 1;
#pragma unroll
  for (int sidx = 0; sidx < NSTEP; ++sidx) {
    const int step = step0 + sidx;
    if (step >= nsteps) break;
    const bool act = (KVB >= 32) || (h == sidx);
    // ---- running maximum (max of the exact integer scores, then times c) -----------
    float imt[G::TPS];  // per tile: the largest score of the lane's present keys
    if (pk) {
      // per-key c: the maximum of t_j = fl(A_j c_j), c_j = fl(fl(sq sk_j) C0), over the
      // lane's present keys.  First a bound from W = max_j fl(A_j sk_j): the three
      // roundings between A_j sq sk_j C0 and t_j, and the one in fl(A_j sk_j), move it
      // by at most a factor (1 +- 2^-24)^4 each way, so t_j <= fl(fl(fl(W sq) C0) f)
      // with f = 1 + 2^-20 for W >= 0 and 1 - 2^-20 for W < 0 (those three roundings
      // taken into account as well: 7 2^-24 < 2^-20); adding 2^-126 covers products
      // that underflow (a c_j of 0 gives t_j = 0).  When no lane's bound exceeds the
      // running maximum, the tile cannot move it and the bound, within about 2^-20 of
      // the exact maximum, stands in for it (here and in the skip tests); otherwise
      // the exact maximum is formed.
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) {
        const float* sk = Sl + 32 * (tb + t) + 16 * h;
        float wm = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          bool ok = act;
          if (MASK) ok = ok && (j0 + t * 32 + 16 * h + v < a.klim);
          wm = fmaxf(wm, ok ? st[t][v] * sk[v] : -INFINITY);
        }
        float im = ((wm * sq) * a.C0) * (wm >= 0.f ? 1.0f + 0x1p-20f : 1.0f - 0x1p-20f) + 0x1p-126f;
        if (__any(im > S.m)) {
          im = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            bool ok = act;
            if (MASK) ok = ok && (j0 + t * 32 + 16 * h + v < a.klim);
            const float c = (sq * sk[v]) * a.C0;
            im = fmaxf(im, ok ? st[t][v] * c : -INFINITY);
          }
        }
        imt[t] = im;
      }
    } else {
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) {
        float im = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          bool ok = act;
          if (MASK) ok = ok && (j0 + t * 32 + 16 * h + v < a.klim);
          im = fmaxf(im, ok ? st[t][v] : -INFINITY);
        }
        imt[t] = im;
      }
    }
    float mloc = -INFINITY;
    if (pk) {
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) mloc = fmaxf(mloc, imt[t]);
    } else if (US) {
      float im = imt[0];
#pragma unroll
      for (int t = 1; t < G::TPS; ++t) im = fmaxf(im, imt[t]);
      if (im != -INFINITY) mloc = im * ct[0];
    } else {
#pragma unroll
      for (int t = 0; t < G::TPS; ++t)
        if (imt[t] != -INFINITY) mloc = fmaxf(mloc, imt[t] * ct[t]);
    }
    const float mnew = fmaxf(S.m, pair_max(mloc));
    const bool moved = __any(mnew > S.m);
    const float alpha = exp2_hw(S.m - mnew);
    if (moved) S.l = S.l * alpha;
    S.m = mnew;
    const bool guard = mnew >= 262144.0f;
    // The level code below forms y = fma(st, c, nm).  With per-key scales the
    // exponents y = fma(A, c_j, L15 - m) of a tile whose exps are needed are formed
    // into st (below, once its pair's skip decision is known), and the code reads
    // them back through c = 1, nm = 0 (exactly y).  The skip tests take a bound: with
    // tmax the largest t_j = fl(A_j c_j) of the tile's present keys, A_j c_j <= t_j +
    // max(|t_j| 2^-24, 2^-150) <= b = fl(fl(tmax + |tmax| 2^-23) + 2^-126) (the inner
    // sum lies at least one ulp above a normal tmax, the outer one covers 0 and
    // subnormals), and y_j = fl(A_j c_j + (L15 - m)) is monotone in A_j c_j, so every
    // exact y_j of the tile is at most fl(b + (L15 - m)).  (No present key: tmax =
    // -inf and the bound is NaN, which no test passes.)
    const float ny = a.L15 - mnew;  // L15 - m, for the per-key exponents
    float nm = ny;
    float cu[G::TPS];
    float ymax[G::TPS];
    if (pk) {
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) {
        ymax[t] = (__builtin_fmaf(fabsf(imt[t]), 0x1p-23f, imt[t]) + 0x1p-126f) + ny;
        cu[t] = 1.0f;
      }
      nm = 0.f;
    } else {
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) {
        cu[t] = ct[t];
        ymax[t] = __builtin_fmaf(imt[t], ct[t], nm);
      }
    }
    // Tiles whose every level is 0: y = fma(A, c, L15 - m) is non-decreasing in the
    // score A (c >= 0), so the largest y of a lane's keys in a tile is fma(max A, c,
    // L15 - m), exactly; when it is below the first threshold in every lane, every
    // exact level of the tile is 0 and its P V products are exact zeros.  (No present
    // key: -inf, or NaN when c = 0; neither compares true.)  The debug run keeps the
    // dense path so that it dumps every code.
    //
    // Tiles whose every p is below half an ulp of l: adding such a p to l (binary32,
    // round to nearest even) returns l unchanged, and l only grows for the rest of
    // the step (the rescale came first), so these additions are exact no-ops and
    // are skipped too.  For l in [2^e, 2^(e+1)) half an ulp is 2^(e-24); the bound
    // on y is e - 24 - 1e-4, so that the hardware exp (within 2^-22 relative of 2^y)
    // stays below it.  While l is 0 (a row's first step) nothing is skipped this way.
    const float ythr = S.l > 0.f ? (float)(__builtin_amdgcn_frexp_expf(S.l) - 25) - 1e-4f : -INFINITY;
    bool ngl[G::TPS];
#pragma unroll
    for (int t = 0; t < G::TPS; ++t) ngl[t] = !DBG && !__any(ymax[t] >= ythr);
    // ---- P levels, P^T operand, level sums, P V: 64 keys (two tiles) per MFMA ---------
    // Fast path: level byte and margin from the hardware exp (level_bits), packed four
    // at a time into the P^T operand.  The level bytes r in [0, 15] are read by the
    // MFMA as fp8 e4m3 codes, whose values are r * 2^-9 (subnormals and the first
    // binade), and the B scale 2^9 makes the products r * v exact; sums stay below
    // 2^24, so the fp32 accumulator adds exact integers.  When some margin in the wave
    // is not clear, every level of the pair is fixed exactly (exact_level) before the
    // one P V MFMA of the pair, so the accumulator only ever adds the exact levels:
    // a pair whose exact levels are all 0 adds exact zeros, which is what makes its
    // skip (above) exact.
    constexpr int PT = G::TPS >= 2 ? 2 : 1;  // tiles per MFMA
#pragma unroll
    for (int pp = 0; pp < G::TPS / PT; ++pp) {
      i32x4 pb[PT];
      bool flag = guard;
      const bool allz = !DBG && !__any(fmaxf(ymax[pp * PT], ymax[pp * PT + PT - 1]) >= a.T0);
      S.cnt.unit(PT);
      if (pk) {
        // per-key scales: the exponents of the pair's tiles whose exps are computed
#pragma unroll
        for (int tp = 0; tp < PT; ++tp) {
          const int t = pp * PT + tp;
          if (allz && ngl[t]) continue;
          const float* sk = Sl + 32 * (tb + t) + 16 * h;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float c = (sq * sk[v]) * a.C0;
            // (with kv_blk 16 the other lane half's keys form the next step: keep them)
            st[t][v] = act ? __builtin_fmaf(st[t][v], c, ny) : st[t][v];
          }
        }
      }
      if (allz) {
        // every level of the pair is 0: the keys enter the normaliser only (same
        // order of additions as the level path); no margin, MFMA, V read or exact
        // path runs.
        // Each path takes L15 - m through an empty asm of its own, so that the
        // compiler can neither merge the two paths' exps nor hoist either set above
        // the branch (where all of them would be computed, and live, at once).
        S.cnt.unit_skip();
        flag = false;
        float nz = nm;
        asm volatile("" : "+v"(nz));
#pragma unroll
        for (int tp = 0; tp < PT; ++tp) {
          const int t = pp * PT + tp;
          // pb is not read on this path (the pair's MFMA is skipped), but the path
          // joins the level path's before the rescale; an empty asm gives pb a value
          // there without the eight moves that a constant would cost
          asm volatile("" : "=v"(pb[tp][0]), "=v"(pb[tp][1]), "=v"(pb[tp][2]), "=v"(pb[tp][3]));
          if (ngl[t]) {  // no p of the tile moves l
            S.cnt.exp_skip();
            continue;
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            bool ok = act;
            if (MASK) ok = ok && (j0 + t * 32 + 16 * h + v < a.klim);
            float p = exp2_hw(__builtin_fmaf(st[t][v], cu[t], nz));
            if (MASK || KVB < 32) p = ok ? p : 0.f;
            S.l += p;
          }
        }
      } else {
      float nl = nm;
      asm volatile("" : "+v"(nl));
#pragma unroll
      for (int tp = 0; tp < PT; ++tp) {
        const int t = pp * PT + tp;
        uint32_t wmin = 0xFFFF;  // low 16 bits: smallest margin (low 16 bits of t) of the tile
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t tt[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * w + e;
            bool ok = act;
            if (MASK) ok = ok && (j0 + t * 32 + 16 * h + v < a.klim);
            const float y = __builtin_fmaf(st[t][v], cu[t], nl);
            float p = exp2_hw(y);
            if (MASK || KVB < 32) p = ok ? p : 0.f;
            S.l += p;
            tt[e] = level_bits(p);
          }
          wmin = min3_u16(wmin, tt[0], tt[1]);
          wmin = min3_u16(wmin, tt[2], tt[3]);
          pb[tp][w] = (int)pack_b2(tt[0], tt[1], tt[2], tt[3]);
        }
        flag = flag || !margin_clear(wmin);
      }
      }  // level path
      if (pp == 0 && moved) {
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
          for (int v = 0; v < 16; ++v) S.acc[db][v] *= alpha;
        }
      }
      if (allz) continue;
      if (DBG || __any(flag)) {
        // exact levels of the whole pair (the debug run always takes this path, so
        // that it dumps the exact code of every key), each fixed from y and the fast
        // level already packed in pb (no second exp)
        S.cnt.fix();
#pragma unroll
        for (int tp = 0; tp < PT; ++tp) {
          const int t = pp * PT + tp;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t rr = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * w + e;
              bool ok = act;
              if (MASK) ok = ok && (j0 + t * 32 + 16 * h + v < a.klim);
              const float y = __builtin_fmaf(st[t][v], cu[t], nm);
              int r = exact_level(y, (int)(((uint32_t)pb[tp][w] >> (8 * e)) & 0xFFu), Tl);
              if (MASK || KVB < 32) r = ok ? r : 0;
              rr |= (uint32_t)r << (8 * e);
              if (DBG && dbg_row && act) {
                const int key = j0 + t * 32 + 16 * h + v;
                if (key < a.klim) {
                  a.dbg_aqk[(int64_t)dr * N + key] = (int32_t)sa[t][v];
                  a.dbg_p[(int64_t)dr * N + key] = (int8_t)(r - a.p_zero);
                }
              }
            }
            pb[tp][w] = (int)rr;
          }
        }
      }
      const i32x8 pop = PT == 2 ? __builtin_shufflevector(pb[0], pb[PT - 1], 0, 1, 2, 3, 4, 5, 6, 7)
                                : __builtin_shufflevector(pb[0], i32x4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
      // this lane half's 32 keys of the pair in the V^T rows (one 16-key chunk,
      // repeated, when a step is a single tile: its P^T half is zero)
      const int voff = PT == 2 ? 32 * (tb + 2 * pp) + 32 * h : 32 * (tb + pp) + 16 * h;
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        const uint8_t* vp = Vl + (db * 32 + col) * G::VROW + voff;
        const i32x4 v0 = *(const i32x4*)vp;
        const i32x4 v1 = PT == 2 ? *(const i32x4*)(vp + 16) : v0;
        const i32x8 vop = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        S.acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop, S.acc[db], 0, 0, 0, 127, 0, 136);
        if (DBG) {
          // this pair's sum_j (P~ + 8) vc (exact integers in fp32), added into the
          // step's entry of the dump (the first pair of the step stores it)
          const f32x16 zero = {0};
          const f32x16 ps = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop, zero, 0, 0, 0, 127, 0, 136);
          // an MFMA reads the operands of every lane: keep it (and its operands) out
          // of the lane-divergent store below
          asm volatile("" ::"v"(ps));
          if (dbg_row) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int d = db * 32 + (v & 3) + 8 * (v >> 2) + 4 * h;
              int32_t* q = a.dbg_apv + ((int64_t)dr * nsteps + step) * D + d;
              *q = (pp == 0 ? 0 : *q) + (int32_t)ps[v];
            }
          }
        }
      }
    }
  }
}

typedef const __attribute__((address_space(4))) float* kscale_ptr;  // read-only: scalar loads

// The work of key group g on its LDS image cur: the K scales of its 16-key units
// (scalar loads, so they never wait behind copies in flight), Q K^T, then each
// online-softmax step's softmax and P V.
template <int D, int KVB, bool DBG, bool MASK, int SM, bool QS, class RS>
RA_DEV void group_compute(const Ctx& a, int g, uint8_t* const cur, const i32x8 (&qop)[Geo<D, KVB>::KC],
                          float sq, int bh, RS& S, bool dbg_row, int dr) {
  using G = Geo<D, KVB, SM, QS>;
  constexpr bool US = SM == 1;
  const int h = (threadIdx.x >> 5) & 1;
  const kscale_ptr ksh = (kscale_ptr)a.ks + (int64_t)bh * (a.Np >> a.qk_shift);
  // The scores of step sg + 1 are issued on the MFMA before the softmax of step sg,
  // so that its latency overlaps that step's VALU work.
  float ct[G::NSG][G::TPS];
  f32x16 st[G::NSG][G::TPS];
#pragma unroll
  for (int sg = 0; sg < G::NSG; ++sg) {
    const int tb = sg * G::TPS;
    if (SM == 2) {
      // per-key scales: c is formed per key (softmax_pv, or the Q-smoothing term below)
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) ct[sg][t] = 1.0f;
    } else if (US) {
      const float c = (sq * ksh[(g * G::TG + 32 * tb) >> a.qk_shift]) * a.C0;
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) ct[sg][t] = c;
    } else {
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) {
        const int k0 = g * G::TG + 32 * (tb + t);
        const float s0 = ksh[k0 >> a.qk_shift], s1 = ksh[(k0 + 16) >> a.qk_shift];
        ct[sg][t] = (sq * (h ? s1 : s0)) * a.C0;
      }
    }
  }
  qk_tiles<D, KVB>(cur, 0, qop, st[0]);
#pragma unroll
  for (int sg = 0; sg < G::NSG; ++sg) {
    const int tb = sg * G::TPS;
    if (sg + 1 < G::NSG) qk_tiles<D, KVB>(cur, tb + G::TPS, qop, st[sg + 1 < G::NSG ? sg + 1 : sg]);
    f32x16 sa[G::TPS];  // the integer scores, kept for the debug dump only
    if (DBG) {
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) sa[t] = st[sg][t];
    }
    const float* Sl = (const float*)(cur + G::SOFF);  // per-key K scales (SM 2)
    if constexpr (QS) {
      // Q smoothing: t = fma(a, c, delta_j) in place; with c = 1 from here on the max
      // is max t and y = fma(t, 1, L15 - m) = fl(t + (L15 - m))
      const float* Dl = (const float*)(cur + G::DOFF) + 32 * tb + 16 * h;
#pragma unroll
      for (int t = 0; t < G::TPS; ++t) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 d4 = *(const f32x4*)(Dl + 32 * t + 4 * v4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c = SM == 2 ? (sq * Sl[32 * (tb + t) + 16 * h + 4 * v4 + e]) * a.C0 : ct[sg][t];
            st[sg][t][4 * v4 + e] = __builtin_fmaf(st[sg][t][4 * v4 + e], c, d4[e]);
          }
        }
        ct[sg][t] = 1.0f;
      }
    }
    const int step0 = KVB < 32 ? 2 * g : g * G::NSG + sg;
    softmax_pv<D, KVB, DBG, MASK, SM>(a, g, tb, step0, cur + G::VOFF, a.T, Sl, sq,
                                      st[sg], ct[sg], DBG ? sa : st[sg], S, dbg_row, dr);
  }
}

// The barrier pipeline (4-wave workgroups; the debug run, and 256-key steps): group g
// in ring slot g % NB.  First the copy of group g + NB - 1 into the slot group g-1
// used (free since the last barrier); then the group's work; then a wait until this
// wave's copy of group g+1 has landed (later copies stay in flight) and one barrier,
// which also covers the other waves' copies.
template <int D, int KVB, bool DBG, bool MASK, int SM, bool QS, int SLOT = -1, class RS>
RA_DEV void group_iter(const Ctx& a, __amdgpu_buffer_rsrc_t rsrc, int g, int ngroups, uint8_t* lds,
                       const i32x8 (&qop)[Geo<D, KVB>::KC], float sq, int bh, RS& S, bool dbg_row, int dr) {
  using G = Geo<D, KVB, SM, QS>;
  // ring slot of this group: a compile-time constant when the caller unrolls the
  // group loop by the slot count (SLOT = g % NB), so LDS addresses stay invariant
  const int slot = SLOT >= 0 ? SLOT : g % G::NB;
  if (g + G::NB - 1 < ngroups)
    dma_group<D, KVB, SM, QS>(rsrc, g + G::NB - 1, lds + ((slot + G::NB - 1) % G::NB) * G::IMG);
  group_compute<D, KVB, DBG, MASK, SM, QS>(a, g, lds + slot * G::IMG, qop, sq, bh, S, dbg_row, dr);
  // copies issued after group g+1's: those of groups g+2 .. min(g+NB-1, ngroups-1)
  const int later = min(g + G::NB - 1, ngroups - 1) - (g + 1);
  if (DBG || later <= 0) wait_vm<0>();
  else if (later == 1) wait_vm<G::NDMA>();
  else wait_vm<2 * G::NDMA>();
  lds_barrier();
}

template <int D, int KVB, bool DBG, int SM, bool QS, bool ST = false>
RA_DEV void k2_body(const AttnArgs& args, uint8_t* lds) {
  using G = Geo<D, KVB, SM, QS>;
  // the P level thresholds (then +inf, +inf) for the exact levels
  __shared__ float Tsh[17];
  constexpr int BM = kBM;  // query rows per workgroup

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  int L;
  if (DBG) {
    L = args.dbg_row0 / BM + blockIdx.x;
  } else {
    L = (int)(blockIdx.x % 8) * args.per_xcd + (int)(blockIdx.x / 8);
    if (L >= args.total) return;
  }
  const int hidx = L / args.nqt;
  // block-causal tiles: the last query tiles see the most keys, so they go first
  const int qt = (!DBG && args.causal > 0) ? args.nqt - 1 - L % args.nqt : L % args.nqt;
  const int bh = args.heads[hidx];
  // tokens of this head that exist (a variable-length batch: tiles past them have
  // no row to write and leave at once, before any copy or barrier)
  const int Nv = (int)valid_len(args.nlens, args.lens, bh, args.H, args.N);
  if (!DBG && qt * BM >= Nv) return;
  Ctx a;
  a.img = args.img; a.ks = args.ks; a.Np = args.Np;
  a.N = (int)args.N; a.qk_shift = __builtin_ctz(args.qk_blk); a.C0 = args.C0; a.L15 = args.L15;
  a.p_zero = args.p_zero;
  a.T0 = args.T[0];
  a.dbg_row0 = args.dbg_row0; a.dbg_n = args.dbg_n;
  a.dbg_aqk = args.dbg_aqk; a.dbg_p = args.dbg_p; a.dbg_apv = args.dbg_apv;
  const int N = a.N;  // the layout's tokens per head
  const int qi = qt * BM + w * 32 + col;
  // Keys seen: all Nv, or under block-causal masking (block c) the keys of the row's
  // own block and every earlier one, min(Nv, (i / c + 1) c).  The tile's groups run
  // up to its last row's limit; groups wholly below its first row's limit need no
  // per-key test.
  const int64_t c = args.causal;
  auto limit = [&](int64_t i) -> int { return c > 0 ? (int)min((int64_t)Nv, (i / c + 1) * c) : Nv; };
  a.klim = limit(qi);
  a.kb = QS;
  a.T = Tsh;
  const int kmax = limit(min(qt * BM + BM - 1, Nv - 1));
  const int ngroups = (kmax + G::TG - 1) / G::TG;
  const int nfull = min(limit(qt * BM) / G::TG, ngroups);  // groups no row masks

  // ---- prologue: groups 0 .. NB-2 in flight ----------------------------------------
  const int64_t ngp = a.Np / G::TG;
  const int64_t head0 = (int64_t)bh * ngp * G::IMG;
  const int64_t avail = args.img_bytes - head0;  // the resource never reaches past the workspace
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.img + head0), (short)0, (int)(avail < ngp * G::IMG ? (avail > 0 ? avail : 0) : ngp * G::IMG),
      0x00020000);
#pragma unroll
  for (int p = 0; p < G::NB - 1; ++p)
    if (p < ngroups) dma_group<D, KVB, SM, QS>(rsrc, p, lds + p * G::IMG);
  if (tid < 17) Tsh[tid] = tid < 15 ? args.T[tid] : INFINITY;

  // ---- Q operand: packed fp6 e2m3 values of the lane's 32 channels per 64-deep chunk
  i32x8 qop[G::KC];
  {
    const u32x4* qp = (const u32x4*)(args.qc + ((int64_t)bh * a.Np + qi) * (D / 2));
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) {
      uint32_t o[6];
      pack_fp6(qp[2 * kc + h], o);
#pragma unroll
      for (int q = 0; q < 8; ++q) qop[kc][q] = q < 6 ? (int)o[q] : 0;
    }
  }
  const float sq = args.qs[(int64_t)bh * (a.Np >> a.qk_shift) + (qi >> a.qk_shift)];

  RowState<G::NDB, std::conditional_t<ST, SkipCount, NoCount>> S;
  S.m = -INFINITY;
  S.l = 0.f;
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
    for (int v = 0; v < 16; ++v) S.acc[db][v] = 0.f;
  }
  const bool dbg_row = DBG && qi >= a.dbg_row0 && qi < a.dbg_row0 + a.dbg_n && qi < Nv;
  const int dr = qi - a.dbg_row0;

  wait_vm<0>();  // the first groups and the Q operand
  lds_barrier();
  int g = 0;
  if (G::NB == 2) {
    for (; g + 2 <= nfull; g += 2) {
      group_iter<D, KVB, DBG, false, SM, QS, 0>(a, rsrc, g, ngroups, lds, qop, sq, bh, S, dbg_row, dr);
      group_iter<D, KVB, DBG, false, SM, QS, 1>(a, rsrc, g + 1, ngroups, lds, qop, sq, bh, S, dbg_row, dr);
    }
  }
  for (; g < nfull; ++g)
    group_iter<D, KVB, DBG, false, SM, QS>(a, rsrc, g, ngroups, lds, qop, sq, bh, S, dbg_row, dr);
  for (; g < ngroups; ++g)
    group_iter<D, KVB, DBG, true, SM, QS>(a, rsrc, g, ngroups, lds, qop, sq, bh, S, dbg_row, dr);

  // ---- epilogue ---------------------------------------------------------------------
  if constexpr (ST) {
    if (lane == 0) {
      atomicAdd(args.stats + 0, (unsigned long long)S.cnt.n_pv);
      atomicAdd(args.stats + 1, (unsigned long long)S.cnt.n_pv_skip);
      atomicAdd(args.stats + 2, (unsigned long long)S.cnt.n_tile);
      atomicAdd(args.stats + 3, (unsigned long long)S.cnt.n_exp_skip);
      atomicAdd(args.stats + 4, (unsigned long long)S.cnt.n_fix);
    }
  }
  const float lq = pair_sum(S.l);
  if (DBG && dbg_row && h == 0) {
    args.dbg_m[dr] = S.m;
    args.dbg_l[dr] = lq;
  }
  if (qi < Nv) {
    const float inv = 1.0f / lq;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * h;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = v4 * 4 + e;
          o[e] = S.acc[db][v] * args.vs[(int64_t)bh * D + d0 + e] * inv;
        }
        const int64_t off = ((int64_t)bh * N + qi) * D + d0;
        store_out4(args.out, args.out_kind, off, o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// The production kernel: two waves per SIMD (<= 256 registers per wave), one for
// 256-key steps.
// ST: the instance that also counts the exact skips (args.stats).
template <int D, int KVB, int SM, bool QS, bool ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Geo<D, KVB, SM>::WPE, Geo<D, KVB, SM>::WPE)))
void k2_attention(const AttnArgs args) {
  extern __shared__ __align__(16) uint8_t lds[];
  k2_body<D, KVB, false, SM, QS, ST>(args, lds);
}

// The debug run (dumps of one head's row range): one wave per SIMD, so that the
// extra dump state fits in registers.
template <int D, int KVB, int SM, bool QS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k2_attention_debug(
    const AttnArgs args) {
  extern __shared__ __align__(16) uint8_t lds[];
  k2_body<D, KVB, true, SM, QS>(args, lds);
}

template <int D, int KVB, int SM, bool QS>
hipError_t launch_t(const AttnArgs& a, bool dbg, hipStream_t st) {
  using G = Geo<D, KVB, SM, QS>;
  // The dynamic LDS limit is raised on every call (for the current device; the
  // setting is idempotent), so the library keeps no state between calls.
  const void* fn = dbg ? (const void*)k2_attention_debug<D, KVB, SM, QS>
                      : a.stats ? (const void*)k2_attention<D, KVB, SM, QS, true>
                                : (const void*)k2_attention<D, KVB, SM, QS, false>;
  const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
  if (attr != hipSuccess) return attr;
  k2_stage<D, KVB, SM, QS><<<dim3((unsigned)(a.Np / G::TG), (unsigned)a.nheads), 256, 0, st>>>(a);
  if (dbg) {
    const int first = a.dbg_row0 / kBM, last = (a.dbg_row0 + a.dbg_n - 1) / kBM;
    k2_attention_debug<D, KVB, SM, QS><<<last - first + 1, 256, G::LDS, st>>>(a);
  } else {
    if (a.stats) k2_attention<D, KVB, SM, QS, true><<<8 * a.per_xcd, 256, G::LDS, st>>>(a);
    else k2_attention<D, KVB, SM, QS, false><<<8 * a.per_xcd, 256, G::LDS, st>>>(a);
  }
  return hipGetLastError();
}

// The scale mode of a call: per-key scales below 16 tokens per block; one scale per
// step when a step of kv_blk >= 32 keys lies inside one K-scale block; else one per
// 16-key unit.
inline int scale_mode(int kv_blk, int qk_blk) {
  if (qk_blk < 16) return 2;
  return (kv_blk >= 32 && qk_blk >= kv_blk) ? 1 : 0;
}

template <int D, int KVB, bool QS>
hipError_t launch_q(const AttnArgs& a, bool dbg, hipStream_t st) {
  switch (scale_mode(KVB, a.qk_blk)) {
    case 2: return launch_t<D, KVB, 2, QS>(a, dbg, st);
    case 1:
      if constexpr (KVB >= 32 && KVB <= 128) return launch_t<D, KVB, 1, QS>(a, dbg, st);
      return hipErrorInvalidValue;
    default: return launch_t<D, KVB, 0, QS>(a, dbg, st);
  }
}

// Q smoothing (per-key score terms) selects the image geometry that carries them.
template <int D, int KVB>
hipError_t launch_s(const AttnArgs& a, bool dbg, hipStream_t st) {
  return a.kbias ? launch_q<D, KVB, true>(a, dbg, st) : launch_q<D, KVB, false>(a, dbg, st);
}

}  // namespace ra
