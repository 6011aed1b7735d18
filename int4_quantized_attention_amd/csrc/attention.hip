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
//    offset-binary bytes (code + 8) with three bit operations per 8 nibbles.  The
//    +8 on K is removed exactly by starting the Q K^T accumulation at -8 sum_d q_d;
//    the +8 on V is removed at the end with the per-row sum of the P levels.
//  * The P level r = round-half-even(2^y) is taken from the hardware exp2: with
//    t = 2^y + 128.5 + 4*2^-16 the level is byte 2 of t's bits and the low 16 bits
//    carry the rounding margin.  v_exp_f32 is within 1.5 * 2^-24 relative of 2^y,
//    so whenever the margin is above 6/2^16 the level equals the exact one; the
//    (rare) other elements are decided exactly against the 15 thresholds.
//  * The int32 P V accumulator runs across online-softmax steps and is folded
//    into the fp32 output only when a row maximum moves.
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

RA_DEV float partner(float v) {
  // value of lane l ^ 32
  return __shfl_xor(v, 32, 64);
}

template <int D, int KVB, bool DBG>
__global__ __launch_bounds__(256) void k2_attention(const AttnArgs a) {
  constexpr int TG = KVB < 32 ? 32 : KVB;  // keys staged per group
  constexpr int NT = TG / 32;              // 32-key tiles per group
  constexpr int NDB = D / 32;              // 32-row d blocks of O^T
  constexpr int KC = D / 32;               // 32-deep k chunks of Q K^T
  constexpr int KROW = D + 16;             // LDS K row stride (bytes)
  constexpr int VROW = TG + 16;            // LDS V^T row stride (bytes)
  __shared__ __align__(16) uint8_t Kl[TG * KROW];
  __shared__ __align__(16) uint8_t Vl[D * VROW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  int L;
  if (DBG) {
    L = a.dbg_row0 / kBM + blockIdx.x;
  } else {
    L = (int)(blockIdx.x % 8) * a.per_xcd + (int)(blockIdx.x / 8);
    if (L >= a.total) return;
  }
  const int hidx = L / a.nqt, qt = L % a.nqt;
  const int bh = a.heads[hidx];
  const int64_t N = a.N, Np = a.Np;
  const int qi = qt * kBM + w * 32 + col;

  // ---- Q operand (signed int8), row sum, bias for the offset-binary K ---------
  i32x4 qop[KC];
  int qsum = 0;
  {
    const uint2* qp = (const uint2*)(a.qc + ((int64_t)bh * Np + qi) * (D / 2));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint2 x = qp[kc * 2 + h];
      uint32_t lo0, hi0, lo1, hi1;
      widen_signed(x.x, lo0, hi0);
      widen_signed(x.y, lo1, hi1);
      qop[kc] = i32x4{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
      qsum = __builtin_amdgcn_sdot4((int)lo0, 0x01010101, qsum, false);
      qsum = __builtin_amdgcn_sdot4((int)hi0, 0x01010101, qsum, false);
      qsum = __builtin_amdgcn_sdot4((int)lo1, 0x01010101, qsum, false);
      qsum = __builtin_amdgcn_sdot4((int)hi1, 0x01010101, qsum, false);
    }
  }
  qsum += __shfl_xor(qsum, 32, 64);
  i32x16 cbias;
#pragma unroll
  for (int v = 0; v < 16; ++v) cbias[v] = -8 * qsum;
  const float sq = a.qs[(int64_t)bh * (Np / a.qk_blk) + qi / a.qk_blk];
  const float C0 = a.C0, L15 = a.L15;

  float m = -INFINITY, l = 0.f, Rf = 0.f;
  int Rint = 0;
  f32x16 Of[NDB];
  i32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int v = 0; v < 16; ++v) { Of[db][v] = 0.f; acc[db][v] = 0; }
  }
  const bool dbg_row = DBG && qi >= a.dbg_row0 && qi < a.dbg_row0 + a.dbg_n && qi < N;
  const int dr = qi - a.dbg_row0;
  const int64_t nsteps = (N + KVB - 1) / KVB;

  const int64_t ngroups = (N + TG - 1) / TG;
  for (int64_t g = 0; g < ngroups; ++g) {
    const int64_t j0 = g * TG;
    __syncthreads();
    // ---- stage K (rows permuted so that S^T lane h holds keys 16h..16h+15) ---
    for (int it = tid; it < TG * (D / 16); it += 256) {
      const int kk = it / (D / 16), c = it % (D / 16);
      const uint2 x = ((const uint2*)(a.kc + ((int64_t)bh * Np + j0 + kk) * (D / 2)))[c];
      uint32_t lo0, hi0, lo1, hi1;
      widen_biased(x.x, lo0, hi0);
      widen_biased(x.y, lo1, hi1);
      const int r = kk & 31, hh = r >> 4, v = r & 15;
      const int row = (kk & ~31) + (v & 3) + 8 * (v >> 2) + 4 * hh;
      *(uint4*)(Kl + row * KROW + 16 * c) = make_uint4(lo0, hi0, lo1, hi1);
    }
    // ---- stage V^T ---------------------------------------------------------------
    for (int it = tid; it < D * (TG / 16); it += 256) {
      const int d = it / (TG / 16), c = it % (TG / 16);
      const uint2 x = ((const uint2*)(a.vc + ((int64_t)bh * D + d) * (Np / 2) + j0 / 2))[c];
      uint32_t lo0, hi0, lo1, hi1;
      widen_biased(x.x, lo0, hi0);
      widen_biased(x.y, lo1, hi1);
      *(uint4*)(Vl + d * VROW + 16 * c) = make_uint4(lo0, hi0, lo1, hi1);
    }
    __syncthreads();

    // ---- S^T tiles ---------------------------------------------------------------
    i32x16 st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const i32x4 kop = *(const i32x4*)(Kl + (t * 32 + col) * KROW + kc * 32 + 16 * h);
        st[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qop[kc], kc == 0 ? cbias : st[t], 0, 0, 0);
      }
    }
    float ct[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t key0 = j0 + t * 32 + 16 * h;
      const float sk = a.ks[(int64_t)bh * (Np / a.qk_blk) + key0 / a.qk_blk];
      const float ss = sq * sk;
      ct[t] = ss * C0;
    }

    constexpr int NSTEP = KVB < 32 ? 2 : 1;  // online-softmax steps in this group
#pragma unroll
    for (int sidx = 0; sidx < NSTEP; ++sidx) {
      const int64_t step = (KVB < 32) ? g * 2 + sidx : g;
      if (step >= nsteps) break;
      const bool act = (KVB >= 32) || (h == sidx);
      const bool tail = (j0 + TG > N);
      // ---- row maximum over the step ---------------------------------------------
      float mloc = -INFINITY;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        int im = INT32_MIN;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t key = j0 + t * 32 + 16 * h + v;
          const bool ok = act && (!tail || key < N);
          im = max(im, ok ? st[t][v] : INT32_MIN);
        }
        if (im != INT32_MIN) {
          const float tm = (float)im * ct[t];
          mloc = fmaxf(mloc, tm);
        }
      }
      const float mstep = fmaxf(mloc, partner(mloc));
      const float mnew = fmaxf(m, mstep);
      const float alpha = exp2_hw(m - mnew);
      const bool changed = mnew > m;
      if (DBG || __any(changed)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            Of[db][v] = (Of[db][v] + (float)acc[db][v]) * alpha;
            acc[db][v] = 0;
          }
        }
        Rf = (Rf + (float)Rint) * alpha;
        Rint = 0;
      }
      l = l * alpha;
      m = mnew;
      const float nm = L15 - mnew;
      const bool guard = mnew >= 262144.0f;

      // ---- P levels --------------------------------------------------------------
      uint32_t tt[NT][16];
      u16x2 wmin = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t key = j0 + t * 32 + 16 * h + v;
          const bool ok = act && (!tail || key < N);
          const float af = (float)st[t][v];
          const float y = __builtin_fmaf(af, ct[t], nm);
          const float p = ok ? exp2_hw(y) : 0.f;
          l += p;
          const float tv = p + kMagic;
          tt[t][v] = __float_as_uint(tv);
          wmin = __builtin_elementwise_min(wmin, __builtin_bit_cast(u16x2, tt[t][v]));
        }
      }
      if (__any((wmin.x <= 6) || guard)) {
        // exact decision for the elements whose margin is too small
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t key = j0 + t * 32 + 16 * h + v;
            const bool ok = act && (!tail || key < N);
            const bool flag = ok && (((tt[t][v] & 0xFFFFu) <= 6u) || guard);
            if (__any(flag)) {
              if (flag) {
                const float y = __builtin_fmaf((float)st[t][v], ct[t], nm);
                int r = 0;
#pragma unroll
                for (int k = 0; k < 15; ++k) r += (y >= a.T[k]) ? 1 : 0;
                tt[t][v] = (tt[t][v] & 0xFF00FFFFu) | ((uint32_t)r << 16);
              }
            }
          }
        }
      }
      // ---- pack P^T operand, level sums, P V --------------------------------------
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t* T = tt[t];
        i32x4 pb;
        pb[0] = (int)pack_b2(T[0], T[2], T[4], T[6]);
        pb[1] = (int)pack_b2(T[1], T[3], T[5], T[7]);
        pb[2] = (int)pack_b2(T[8], T[10], T[12], T[14]);
        pb[3] = (int)pack_b2(T[9], T[11], T[13], T[15]);
        Rint = __builtin_amdgcn_sdot4(pb[0], 0x01010101, Rint, false);
        Rint = __builtin_amdgcn_sdot4(pb[1], 0x01010101, Rint, false);
        Rint = __builtin_amdgcn_sdot4(pb[2], 0x01010101, Rint, false);
        Rint = __builtin_amdgcn_sdot4(pb[3], 0x01010101, Rint, false);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const i32x4 vop = *(const i32x4*)(Vl + (db * 32 + col) * VROW + t * 32 + 16 * h);
          acc[db] = __builtin_amdgcn_mfma_i32_32x32x32_i8(vop, pb, acc[db], 0, 0, 0);
        }
        if (DBG && dbg_row && act) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t key = j0 + t * 32 + 16 * h + v;
            if (key < N) {
              a.dbg_aqk[(int64_t)dr * N + key] = st[t][v];
              a.dbg_p[(int64_t)dr * N + key] = (int8_t)((int)((T[v] >> 16) & 0xFFu) - 8);
            }
          }
        }
      }
      if (DBG) {
        // per-step accumulator: sum_j (P~ + 8) vc = acc - 8 * (sum of levels of the row)
        const float rsum = (float)Rint + partner((float)Rint);
        if (dbg_row) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int d = db * 32 + (v & 3) + 8 * (v >> 2) + 4 * h;
              a.dbg_apv[((int64_t)dr * nsteps + step) * D + d] = acc[db][v] - 8 * (int)rsum;
            }
          }
        }
      }
    }
  }
  // ---- epilogue ---------------------------------------------------------------------
  const float lq = l + partner(l);
  const float Rq = (Rf + (float)Rint) + partner(Rf + (float)Rint);
  if (DBG && dbg_row && h == 0) {
    a.dbg_m[dr] = m;
    a.dbg_l[dr] = lq;
  }
  if (qi < N) {
    const float inv = 1.0f / lq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = db * 32 + 8 * v4 + 4 * h;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = v4 * 4 + e;
          const float num = (Of[db][v] + (float)acc[db][v]) - 8.0f * Rq;
          o[e] = num * a.vs[(int64_t)bh * D + d0 + e] * inv;
        }
        const int64_t off = ((int64_t)bh * N + qi) * D + d0;
        if (a.out_f16) {
          f16x4 hv = {(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
          *(f16x4*)((_Float16*)a.out + off) = hv;
        } else {
          *(f32x4*)((float*)a.out + off) = f32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
  }
}

template <int D, int KVB>
hipError_t launch_t(const AttnArgs& a, bool dbg, hipStream_t st) {
  if (dbg) {
    const int first = a.dbg_row0 / kBM, last = (a.dbg_row0 + a.dbg_n - 1) / kBM;
    k2_attention<D, KVB, true><<<last - first + 1, 256, 0, st>>>(a);
  } else {
    k2_attention<D, KVB, false><<<8 * a.per_xcd, 256, 0, st>>>(a);
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
