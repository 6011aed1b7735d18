// K2 entry: dispatch of rotattn_int4_attention over the head dimension and the kv
// step, the attention workspace size, and the probe of the P level decision.  The
// kernels are in attention_impl.h; attention_inst.hip instantiates them.
#include "attention_impl.h"

namespace ra {

// instantiated in attention_inst.hip, one object per (D, kv_blk)
extern template hipError_t launch_s<64, 16>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<64, 32>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<64, 64>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<64, 128>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<64, 256>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<128, 16>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<128, 32>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<128, 64>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<128, 128>(const AttnArgs& a, bool dbg, hipStream_t st);
extern template hipError_t launch_s<128, 256>(const AttnArgs& a, bool dbg, hipStream_t st);

// The P level decision of the attention (decide_level, and exact_level on its own,
// which a pair with any unclear margin applies to every key), for the exponents
// y = the binary32 value of bits first + i, i < n: out[i] = decide | exact << 4.
__global__ __launch_bounds__(256) void k2_level_probe(uint32_t first, int64_t n, uint8_t* out, LevelTable T) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float y = __uint_as_float(first + (uint32_t)i);
    const float p = exp2_hw(y);
    const int r = decide_level(y, p, T.T);
    const int x = exact_level(y, fast_level(level_bits(p)), T.T);
    out[i] = (uint8_t)(r | (x << 4));
  }
}

hipError_t launch_level_probe(uint32_t first, int64_t n, uint8_t* out, const float* thresholds15,
                              hipStream_t st) {
  LevelTable T;
  for (int k = 0; k < 15; ++k) T.T[k] = thresholds15[k];
  T.T[15] = T.T[16] = INFINITY;
  const int64_t blocks = (n + 255) / 256;
  k2_level_probe<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, st>>>(first, n, out, T);
  return hipGetLastError();
}

template <int D, int KVB>
size_t ws_bytes(int qk_blk, int64_t BH, int64_t Np) {
  // the larger geometry of a call with Q smoothing (its images also carry the per-key
  // score terms), so that one workspace size serves both
  const size_t img = scale_mode(KVB, qk_blk) == 2 ? Geo<D, KVB, 2, true>::IMG : Geo<D, KVB, 0, true>::IMG;
  return (size_t)BH * (size_t)(Np / Geo<D, KVB>::TG) * img;
}

template <int D>
size_t ws_bytes_d(int kv_blk, int qk_blk, int64_t BH, int64_t Np) {
  switch (kv_blk) {
    case 16: return ws_bytes<D, 16>(qk_blk, BH, Np);
    case 32: return ws_bytes<D, 32>(qk_blk, BH, Np);
    case 64: return ws_bytes<D, 64>(qk_blk, BH, Np);
    case 128: return ws_bytes<D, 128>(qk_blk, BH, Np);
    default: return ws_bytes<D, 256>(qk_blk, BH, Np);
  }
}

size_t attention_workspace_bytes(int D, int kv_blk, int qk_blk, int64_t BH, int64_t Np) {
  return D == 128 ? ws_bytes_d<128>(kv_blk, qk_blk, BH, Np) : ws_bytes_d<64>(kv_blk, qk_blk, BH, Np);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int kv_blk, bool dbg, hipStream_t st) {
  switch (kv_blk) {
    case 16: return launch_s<D, 16>(a, dbg, st);
    case 32: return launch_s<D, 32>(a, dbg, st);
    case 64: return launch_s<D, 64>(a, dbg, st);
    case 128: return launch_s<D, 128>(a, dbg, st);
    default: return launch_s<D, 256>(a, dbg, st);
  }
}

hipError_t launch_attention(const AttnArgs& a, int D, int kv_blk, bool dbg, hipStream_t st) {
  return D == 128 ? launch_d<128>(a, kv_blk, dbg, st) : launch_d<64>(a, kv_blk, dbg, st);
}

}  // namespace ra
