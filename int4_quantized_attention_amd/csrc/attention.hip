// K2: INT4 FlashAttention forward with range-rectified P codes.
//
// RotateAttention (arXiv 2607.02584), papernotes.org note: framework flowchart
// (INT4 Q K^T -> scores -> range-rectified P -> INT4 P V) and "Key design 2"
// (P = exp(S - m) in (0, 1] with m the running row maximum; code
// round(15 P) - 8 in [-8, 7], fixed scale 15, zero point -8).
//
// gfx950 design
//  * One workgroup = 4 waves x 32 query rows.  Each wave computes S^T = K Q^T on
//    v_mfma_i32_32x32x32_i8, so a lane owns one query row and 16 keys of every
//    32-key tile; its P codes are already laid out as the B operand of the next
//    MFMA, O^T = V^T P^T, with no LDS round trip.
//  * K and V stay INT4 in HBM; the workgroup widens each tile once into LDS as
//    int8 bytes holding 16 c (the nibble moved to the high half of its byte: three
//    bit operations per 8 nibbles).  Both integer products are then 16 times the
//    INT4 ones; the factor is a power of two and is divided out exactly in the
//    score scale and in the output scale.
//  * The P level r = round-half-even(2^y) is taken from the hardware exp2: with
//    t = 2^y + 128.5 + 4*2^-16 the level is byte 2 of t's bits and the low 16 bits
//    carry the rounding margin.  v_exp_f32 is within 1.5 * 2^-24 relative of 2^y,
//    so whenever the margin is above 6/2^16 the level equals the exact one; the
//    (rare) other elements are decided exactly against the 15 thresholds.
//  * The int32 P V accumulator runs across online-softmax steps and is folded
//    into the fp32 output (one fma per element, in a fixed exponent frame) only
//    when a row maximum moves; the next MFMA then restarts it from zero.
//  * Two waves per SIMD (<= 256 registers each), so that one wave's MFMAs run
//    under the other's softmax; one barrier per key group; K and V tiles are
//    double-buffered in LDS and their global loads run one group ahead.
//  * Workgroup ids are remapped so that all query tiles of a head run on the same
//    XCD and share its L2 for the K/V stream.
#include "common.h"
#include "kernels.h"

namespace ra {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;
constexpr float kMagic = 128.5f + 4.0f / 65536.0f;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

RA_DEV uint32_t pack_b2(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t x = __builtin_amdgcn_perm(b, a, 0x0c0c0602u);
  const uint32_t y = __builtin_amdgcn_perm(d, c, 0x0c0c0602u);
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}

// The fields the device helpers need, copied out of the kernel argument block
// (which also holds the head list and stays in the kernarg segment).
struct Ctx {
  const uint8_t* kc;
  const uint8_t* vc;
  const float* ks;
  int64_t Np;
  int N, qk_shift;
  float C0, L15;
  int dbg_row0, dbg_n;
  int32_t* dbg_aqk;
  int8_t* dbg_p;
  int32_t* dbg_apv;
};

template <int D, int KVB>
struct Geo {
  static constexpr int TG = KVB < 32 ? 32 : KVB;  // keys per group (staged together)
  static constexpr int NT = TG / 32;              // 32-key MFMA tiles per group
  static constexpr int NDB = D / 32;              // 32-row d blocks of O^T
  static constexpr int KC = D / 32;               // 32-deep chunks of Q K^T
  static constexpr int KROW = D + 16;             // LDS K row stride (bytes)
  static constexpr int VROW = TG + 16;            // LDS V^T row stride (bytes)
  static constexpr int KBUF = TG * KROW;
  static constexpr int VBUF = D * VROW;
  static constexpr int SKN = TG / 16;             // K scales per group, one per 16 keys
  static constexpr int SOFF = 2 * KBUF + 2 * VBUF;  // two groups of K scales (floats)
  static constexpr int LDS = SOFF + 2 * SKN * 4;    // + 17 floats of level thresholds after it
  static constexpr int KU = TG * D / 16;          // 8-byte global units of a K group
  static constexpr int VU = D * TG / 16;          // 8-byte global units of a V group
  static constexpr int KUT = (KU + 255) / 256;    // per thread
  static constexpr int VUT = (VU + 255) / 256;
};

// Per-lane running state of one query row (the lane pair l, l^32 shares a row).
// Of holds the flushed part of the output numerator in a fixed frame: the sum over
// flushed steps of 2^(m_s - mref) * acc_s, where acc_s is the integer P V sum of a
// step with running maximum m_s.  sigma = 2^(m - mref) for the current maximum, so
// a flush is one fma per element; acc restarts from zero in the next MFMA (fresh).
template <int NDB>
struct RowState {
  f32x16 Of[NDB];
  i32x16 acc[NDB];
  float m, l, mref, sigma;
  bool fresh;
};

template <int D, int KVB>
RA_DEV void load_k(const Ctx& a, int bh, int g, u32x2 (&r)[Geo<D, KVB>::KUT]) {
  using G = Geo<D, KVB>;
  const u32x2* src = (const u32x2*)(a.kc + ((int64_t)bh * a.Np + (int64_t)g * G::TG) * (D / 2));
#pragma unroll
  for (int i = 0; i < G::KUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::KU % 256 == 0 || u < G::KU) r[i] = src[u];
  }
}
template <int D, int KVB>
RA_DEV void load_v(const Ctx& a, int bh, int g, u32x2 (&r)[Geo<D, KVB>::VUT]) {
  using G = Geo<D, KVB>;
#pragma unroll
  for (int i = 0; i < G::VUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::VU % 256 == 0 || u < G::VU) {
      const int d = u / (G::TG / 16), c = u % (G::TG / 16);
      r[i] = ((const u32x2*)(a.vc + ((int64_t)bh * D + d) * (a.Np / 2) + (int64_t)g * (G::TG / 2)))[c];
    }
  }
}
// K rows (sign-extended) are permuted inside each 32-key tile so that the S^T accumulator of lane
// half h holds keys 16h..16h+15 of the tile in register order.
template <int D, int KVB>
RA_DEV void store_k(uint8_t* Kl, const u32x2 (&r)[Geo<D, KVB>::KUT]) {
  using G = Geo<D, KVB>;
#pragma unroll
  for (int i = 0; i < G::KUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::KU % 256 == 0 || u < G::KU) {
      const int kk = u / (D / 16), c = u % (D / 16);
      uint32_t lo0, hi0, lo1, hi1;
      widen_x16(r[i].x, lo0, hi0);
      widen_x16(r[i].y, lo1, hi1);
      const int rr = kk & 31, hh = rr >> 4, v = rr & 15;
      const int row = (kk & ~31) + (v & 3) + 8 * (v >> 2) + 4 * hh;
      *(uint4*)(Kl + row * G::KROW + 16 * c) = make_uint4(lo0, hi0, lo1, hi1);
    }
  }
}
template <int D, int KVB>
RA_DEV void store_v(uint8_t* Vl, const u32x2 (&r)[Geo<D, KVB>::VUT]) {
  using G = Geo<D, KVB>;
#pragma unroll
  for (int i = 0; i < G::VUT; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (G::VU % 256 == 0 || u < G::VU) {
      const int d = u / (G::TG / 16), c = u % (G::TG / 16);
      uint32_t lo0, hi0, lo1, hi1;
      widen_x16(r[i].x, lo0, hi0);
      widen_x16(r[i].y, lo1, hi1);
      *(uint4*)(Vl + d * G::VROW + 16 * c) = make_uint4(lo0, hi0, lo1, hi1);
    }
  }
}

// K scale of the 16-key unit threadIdx.x of group g (threads below TG / 16); staged
// through LDS with the K/V tiles
template <int D, int KVB>
RA_DEV void load_ks(const Ctx& a, int bh, int g, float& rs) {
  using G = Geo<D, KVB>;
  if (threadIdx.x < G::SKN)
    rs = a.ks[(int64_t)bh * (a.Np >> a.qk_shift) + ((g * G::TG + 16 * (int)threadIdx.x) >> a.qk_shift)];
}

template <int D, int KVB>
RA_DEV void qk_tiles(const uint8_t* Kl, const i32x4 (&qop)[Geo<D, KVB>::KC], i32x16 (&st)[Geo<D, KVB>::NT]) {
  using G = Geo<D, KVB>;
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) {
      const i32x4 kop = *(const i32x4*)(Kl + (t * 32 + col) * G::KROW + kc * 32 + 16 * h);
      const i32x16 zero = {0};
      st[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qop[kc], kc == 0 ? zero : st[t], 0, 0, 0);
    }
  }
}

// Online-softmax step(s) of one key group: running max, lazy flush, P levels,
// P^T operand, P V MFMAs.  TAIL: the group holds keys >= N.
template <int D, int KVB, bool DBG, bool TAIL>
RA_DEV void softmax_pv(const Ctx& a, int g, const uint8_t* Vl, const float* Tl,
                       const i32x16 (&st)[Geo<D, KVB>::NT], const float (&sk)[Geo<D, KVB>::NT], float sq,
                       RowState<D / 32>& S, bool dbg_row, int dr) {
  using G = Geo<D, KVB>;
  const int lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
  const int N = (int)a.N;
  const int j0 = g * G::TG;
  const int nsteps = (N + KVB - 1) / KVB;
  // score scale c = (sq sk) C0 of the spec, over 16 for the x16 integer products
  float ct[G::NT];
#pragma unroll
  for (int t = 0; t < G::NT; ++t) ct[t] = ((sq * sk[t]) * a.C0) * 0.0625f;
  constexpr int NSTEP = KVB < 32 ? 2 : 1;
#pragma unroll
  for (int sidx = 0; sidx < NSTEP; ++sidx) {
    const int step = (KVB < 32) ? g * 2 + sidx : g;
    if (step >= nsteps) break;
    const bool act = (KVB >= 32) || (h == sidx);
    // ---- running maximum ---------------------------------------------------------
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < G::NT; ++t) {
      int im = INT32_MIN;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        bool ok = act;
        if (TAIL) ok = ok && (j0 + t * 32 + 16 * h + v < N);
        im = max(im, ok ? st[t][v] : INT32_MIN);
      }
      if (im != INT32_MIN) {
        const float tm = (float)im * ct[t];
        mloc = fmaxf(mloc, tm);
      }
    }
    const float mnew = fmaxf(S.m, pair_max(mloc));
    const float alpha = exp2_hw(S.m - mnew);
    if (DBG || __any(mnew > S.m)) {
      if (!S.fresh) {
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
          for (int v = 0; v < 16; ++v) S.Of[db][v] = __builtin_fmaf((float)S.acc[db][v], S.sigma, S.Of[db][v]);
        }
      }
      S.fresh = true;
      if (g == 0 && sidx == 0) S.mref = mnew;
      if (__any(mnew - S.mref > 64.0f)) {
        // keep sigma far from overflow: move the frame to the current maximum
        const float back = exp2_hw(S.mref - mnew);
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
          for (int v = 0; v < 16; ++v) S.Of[db][v] *= back;
        }
        S.mref = mnew;
      }
      S.sigma = exp2_hw(mnew - S.mref);
    }
    S.l = S.l * alpha;
    S.m = mnew;
    const float nm = a.L15 - mnew;
    const bool guard = mnew >= 262144.0f;
    // ---- P levels, P^T operand, level sums, P V: one 32-key tile at a time --------
#pragma unroll
    for (int t = 0; t < G::NT; ++t) {
      uint32_t tt[16];
      u16x2 wmin = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        bool ok = act;
        if (TAIL) ok = ok && (j0 + t * 32 + 16 * h + v < N);
        const float y = __builtin_fmaf((float)st[t][v], ct[t], nm);
        float p = exp2_hw(y);
        if (TAIL || KVB < 32) p = ok ? p : 0.f;
        S.l += p;
        tt[v] = __float_as_uint(p + kMagic);
        wmin = __builtin_elementwise_min(wmin, __builtin_bit_cast(u16x2, tt[v]));
      }
      if (__any((wmin.x <= 6) || guard)) {
        // A margin is too small somewhere in the wave (rare).  The hardware-exp
        // level r^ is within one of the exact level, which is fixed by the two
        // thresholds around r^ (an LDS table with +inf above the last one).
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float y = __builtin_fmaf((float)st[t][v], ct[t], nm);
          const int rh = min((int)((tt[v] >> 16) & 0xFFu), 16);
          const float lo = Tl[max(rh - 1, 0)], hi = Tl[rh];
          int r = rh - ((rh > 0 && y < lo) ? 1 : 0) + ((y >= hi) ? 1 : 0);
          if (TAIL || KVB < 32) {
            bool ok = act;
            if (TAIL) ok = ok && (j0 + t * 32 + 16 * h + v < N);
            r = ok ? r : 0;
          }
          tt[v] = (tt[v] & 0xFF00FFFFu) | ((uint32_t)r << 16);
        }
      }
      i32x4 pb;
      pb[0] = (int)pack_b2(tt[0], tt[2], tt[4], tt[6]);
      pb[1] = (int)pack_b2(tt[1], tt[3], tt[5], tt[7]);
      pb[2] = (int)pack_b2(tt[8], tt[10], tt[12], tt[14]);
      pb[3] = (int)pack_b2(tt[9], tt[11], tt[13], tt[15]);
      if (t == 0 && S.fresh) {
        const i32x16 zero = {0};
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
          const i32x4 vop = *(const i32x4*)(Vl + (db * 32 + col) * G::VROW + t * 32 + 16 * h);
          S.acc[db] = __builtin_amdgcn_mfma_i32_32x32x32_i8(vop, pb, zero, 0, 0, 0);
        }
        S.fresh = false;
      } else {
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
          const i32x4 vop = *(const i32x4*)(Vl + (db * 32 + col) * G::VROW + t * 32 + 16 * h);
          S.acc[db] = __builtin_amdgcn_mfma_i32_32x32x32_i8(vop, pb, S.acc[db], 0, 0, 0);
        }
      }
      if (DBG && dbg_row && act) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = j0 + t * 32 + 16 * h + v;
          if (key < N) {
            a.dbg_aqk[(int64_t)dr * N + key] = st[t][v] >> 4;
            a.dbg_p[(int64_t)dr * N + key] = (int8_t)((int)((tt[v] >> 16) & 0xFFu) - 8);
          }
        }
      }
    }
    if (DBG && dbg_row) {
      // per-step accumulator sum_j (P~ + 8) vc (the debug run flushes every step)
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int d = db * 32 + (v & 3) + 8 * (v >> 2) + 4 * h;
          a.dbg_apv[((int64_t)dr * nsteps + step) * D + d] = S.acc[db][v] >> 4;
        }
      }
    }
  }
}

// One key group: Q K^T from LDS buffer g&1, widening of the prefetched K/V of
// group g+1 into the other buffer, global loads of group g+2, softmax + P V,
// one barrier.  MFMA/VALU overlap comes from the second wave on each SIMD.
template <int D, int KVB, bool DBG, bool TAIL>
RA_DEV void group_iter(const Ctx& a, int g, int ngroups, uint8_t* lds, u32x2 (&rk)[Geo<D, KVB>::KUT],
                       u32x2 (&rv)[Geo<D, KVB>::VUT], float& rs, const i32x4 (&qop)[Geo<D, KVB>::KC],
                       float sq, int bh, RowState<D / 32>& S, bool dbg_row, int dr) {
  using G = Geo<D, KVB>;
  const bool odd = g & 1;
  uint8_t* const kb_cur = lds + (odd ? G::KBUF : 0);
  uint8_t* const kb_nxt = lds + (odd ? 0 : G::KBUF);
  uint8_t* const vb_cur = lds + 2 * G::KBUF + (odd ? G::VBUF : 0);
  uint8_t* const vb_nxt = lds + 2 * G::KBUF + (odd ? 0 : G::VBUF);
  float* const sb_cur = (float*)(lds + G::SOFF) + (odd ? G::SKN : 0);
  float* const sb_nxt = (float*)(lds + G::SOFF) + (odd ? 0 : G::SKN);
  i32x16 st[G::NT];
  qk_tiles<D, KVB>(kb_cur, qop, st);
  if (g + 1 < ngroups) {
    store_k<D, KVB>(kb_nxt, rk);
    store_v<D, KVB>(vb_nxt, rv);
    if (threadIdx.x < G::SKN) sb_nxt[threadIdx.x] = rs;
  }
  if (g + 2 < ngroups) {
    load_k<D, KVB>(a, bh, g + 2, rk);
    load_v<D, KVB>(a, bh, g + 2, rv);
    load_ks<D, KVB>(a, bh, g + 2, rs);
  }
  float sk[G::NT];
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int t = 0; t < G::NT; ++t) sk[t] = sb_cur[2 * t + h];
  softmax_pv<D, KVB, DBG, TAIL>(a, g, vb_cur, (const float*)(lds + G::LDS), st, sk, sq, S, dbg_row, dr);
  __syncthreads();
}

template <int D, int KVB, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k2_attention(
    const AttnArgs args) {
  using G = Geo<D, KVB>;
  extern __shared__ __align__(16) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  int L;
  if (DBG) {
    L = args.dbg_row0 / kBM + blockIdx.x;
  } else {
    L = (int)(blockIdx.x % 8) * args.per_xcd + (int)(blockIdx.x / 8);
    if (L >= args.total) return;
  }
  const int hidx = L / args.nqt, qt = L % args.nqt;
  const int bh = args.heads[hidx];
  Ctx a;
  a.kc = args.kc; a.vc = args.vc; a.ks = args.ks; a.Np = args.Np;
  a.N = (int)args.N; a.qk_shift = __builtin_ctz(args.qk_blk); a.C0 = args.C0; a.L15 = args.L15;
  a.dbg_row0 = args.dbg_row0; a.dbg_n = args.dbg_n;
  a.dbg_aqk = args.dbg_aqk; a.dbg_p = args.dbg_p; a.dbg_apv = args.dbg_apv;
  const int N = a.N;
  const int qi = qt * kBM + w * 32 + col;

  // ---- Q operand (signed int8) ------------------------------------------------
  i32x4 qop[G::KC];
  {
    const u32x2* qp = (const u32x2*)(args.qc + ((int64_t)bh * a.Np + qi) * (D / 2));
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) {
      const u32x2 x = qp[kc * 2 + h];
      uint32_t lo0, hi0, lo1, hi1;
      widen_signed(x.x, lo0, hi0);
      widen_signed(x.y, lo1, hi1);
      qop[kc] = i32x4{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
    }
  }
  const float sq = args.qs[(int64_t)bh * (a.Np >> a.qk_shift) + (qi >> a.qk_shift)];

  RowState<G::NDB> S;
  S.m = -INFINITY;
  S.l = 0.f;
  S.mref = 0.f;
  S.sigma = 1.f;
  S.fresh = true;
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
    for (int v = 0; v < 16; ++v) { S.Of[db][v] = 0.f; S.acc[db][v] = 0; }
  }
  const bool dbg_row = DBG && qi >= a.dbg_row0 && qi < a.dbg_row0 + a.dbg_n && qi < N;
  const int dr = qi - a.dbg_row0;
  const int ngroups = (N + G::TG - 1) / G::TG;

  if (tid < 17) ((float*)(lds + G::LDS))[tid] = tid < 15 ? args.T[tid] : INFINITY;

  // ---- prologue: group 0 in LDS, group 1 in flight -------------------------------
  u32x2 rk[G::KUT], rv[G::VUT];
  float rs = 0.f;
  load_ks<D, KVB>(a, bh, 0, rs);
  load_k<D, KVB>(a, bh, 0, rk);
  load_v<D, KVB>(a, bh, 0, rv);
  store_k<D, KVB>(lds, rk);
  store_v<D, KVB>(lds + 2 * G::KBUF, rv);
  if (tid < G::SKN) ((float*)(lds + G::SOFF))[tid] = rs;
  if (ngroups > 1) {
    load_k<D, KVB>(a, bh, 1, rk);
    load_v<D, KVB>(a, bh, 1, rv);
    load_ks<D, KVB>(a, bh, 1, rs);
  }
  __syncthreads();
  for (int g = 0; g + 1 < ngroups; ++g)
    group_iter<D, KVB, DBG, false>(a, g, ngroups, lds, rk, rv, rs, qop, sq, bh, S, dbg_row, dr);
  group_iter<D, KVB, DBG, true>(a, ngroups - 1, ngroups, lds, rk, rv, rs, qop, sq, bh, S, dbg_row, dr);

  // ---- epilogue ---------------------------------------------------------------------
  const float lq = pair_sum(S.l);
  const float inv_sigma = 1.0f / S.sigma;
  if (DBG && dbg_row && h == 0) {
    args.dbg_m[dr] = S.m;
    args.dbg_l[dr] = lq;
  }
  if (qi < N) {
    const float inv = 0.0625f / lq;  // also divides out the x16 of the V bytes
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * h;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = v4 * 4 + e;
          const float num = __builtin_fmaf(S.Of[db][v], inv_sigma, (float)S.acc[db][v]);
          o[e] = num * args.vs[(int64_t)bh * D + d0 + e] * inv;
        }
        const int64_t off = ((int64_t)bh * N + qi) * D + d0;
        if (args.out_f16) {
          f16x4 hv = {(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
          *(f16x4*)((_Float16*)args.out + off) = hv;
        } else {
          *(f32x4*)((float*)args.out + off) = f32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
  }
}

template <int D, int KVB>
hipError_t launch_t(const AttnArgs& a, bool dbg, hipStream_t st) {
  using G = Geo<D, KVB>;
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute((const void*)k2_attention<D, KVB, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS + 128);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)k2_attention<D, KVB, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS + 128);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (dbg) {
    const int first = a.dbg_row0 / kBM, last = (a.dbg_row0 + a.dbg_n - 1) / kBM;
    k2_attention<D, KVB, true><<<last - first + 1, 256, G::LDS + 128, st>>>(a);
  } else {
    k2_attention<D, KVB, false><<<8 * a.per_xcd, 256, G::LDS + 128, st>>>(a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_kv(const AttnArgs& a, int kv, bool dbg, hipStream_t st) {
  switch (kv) {
    case 16: return launch_t<D, 16>(a, dbg, st);
    case 32: return launch_t<D, 32>(a, dbg, st);
    case 64: return launch_t<D, 64>(a, dbg, st);
    default: return launch_t<D, 128>(a, dbg, st);
  }
}

hipError_t launch_attention(const AttnArgs& a, int D, int kv_blk, bool dbg, hipStream_t st) {
  if (D == 128) return launch_kv<128>(a, kv_blk, dbg, st);
  return launch_kv<64>(a, kv_blk, dbg, st);
}

}  // namespace ra
