// Micro-benchmarks of the MI355X (gfx950) rates the kernels are measured against:
// back-to-back MFMA throughput per instruction form, HBM streaming bandwidth, and
// the error of the hardware exp2 (v_exp_f32) that the P-level fast path relies on.
// Built into libkb.so, separate from the product library; driven by kb.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kChains = 4;  // independent accumulators per wave (hide the MFMA latency)

// form: 0 i8 32x32x32, 1 f16 32x32x16, 2 bf16 32x32x16, 3 fp8 e4m3 32x32x64,
// 4 fp6 e2m3 32x32x64, 5 fp4 e2m1 32x32x64 (the last three: the scaled f8f6f4 form)
template <int FORM>
__global__ __launch_bounds__(256) void kb_mfma(float* out, int iters) {
  const int t = threadIdx.x;
  if constexpr (FORM == 0) {
    const i32x4 a = {t, t + 1, t + 2, t + 3};
    i32x16 acc[kChains] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc[c], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][15];
    out[blockIdx.x * 256 + t] = (float)s;
  } else if constexpr (FORM == 1 || FORM == 2) {
    f32x16 acc[kChains] = {};
    if constexpr (FORM == 1) {
      const f16x8 a = {(_Float16)t, 1, 2, 3, 4, 5, 6, 7};
      for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc[c], 0, 0, 0);
      }
    } else {
      const bf16x8 a = {(__bf16)(float)t, 1, 2, 3, 4, 5, 6, 7};
      for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][15];
    out[blockIdx.x * 256 + t] = s;
  } else {
    constexpr int fmt = FORM == 3 ? 0 : (FORM == 4 ? 2 : 4);
    const i32x8 a = {t, 0x11, 0x22, 0x33, 0x44, 0x55, 0x66, 0x77};
    f32x16 acc[kChains] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[c], fmt, fmt, 0, 127, 0, 127);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][15];
    out[blockIdx.x * 256 + t] = s;
  }
}

// streaming copy with 16-byte accesses (grid-stride)
__global__ __launch_bounds__(256) void kb_copy_k(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                 int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

// streaming read: every 16-byte element summed into one float per thread
__global__ __launch_bounds__(256) void kb_read_k(const f32x4* __restrict__ src, int64_t n16, float* out) {
  float s = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const f32x4 v = src[i];
    s += v[0] + v[1] + v[2] + v[3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// out[i] = v_exp_f32 of the binary32 value with bit pattern first + i
__global__ __launch_bounds__(256) void kb_exp2_k(uint32_t first, int64_t n, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = __builtin_amdgcn_exp2f(__uint_as_float(first + (uint32_t)i));
}

}  // namespace

extern "C" {

// Launch the MFMA loop of `form` on `blocks` workgroups of 4 waves, `iters` rounds of
// kChains MFMAs per wave.  out: device float [blocks * 256].  Returns a hipError_t.
int kb_mfma_launch(int form, int blocks, int iters, float* out, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  switch (form) {
    case 0: kb_mfma<0><<<blocks, 256, 0, st>>>(out, iters); break;
    case 1: kb_mfma<1><<<blocks, 256, 0, st>>>(out, iters); break;
    case 2: kb_mfma<2><<<blocks, 256, 0, st>>>(out, iters); break;
    case 3: kb_mfma<3><<<blocks, 256, 0, st>>>(out, iters); break;
    case 4: kb_mfma<4><<<blocks, 256, 0, st>>>(out, iters); break;
    case 5: kb_mfma<5><<<blocks, 256, 0, st>>>(out, iters); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
int kb_mfma_chains(void) { return kChains; }

// bytes a multiple of 16; src, dst device, 16-byte aligned
int kb_copy_launch(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
  kb_copy_k<<<blocks, 256, 0, (hipStream_t)stream>>>((const f32x4*)src, (f32x4*)dst, bytes / 16);
  return (int)hipGetLastError();
}
// out: device float [blocks * 256]
int kb_read_launch(const void* src, int64_t bytes, int blocks, float* out, void* stream) {
  kb_read_k<<<blocks, 256, 0, (hipStream_t)stream>>>((const f32x4*)src, bytes / 16, out);
  return (int)hipGetLastError();
}
// first + n <= 2^32; out: device float [n]
int kb_exp2_launch(uint32_t first, int64_t n, float* out, void* stream) {
  if (n < 0 || (uint64_t)first + (uint64_t)n > ((uint64_t)1 << 32)) return (int)hipErrorInvalidValue;
  const int64_t blocks = (n + 255) / 256;
  kb_exp2_k<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, (hipStream_t)stream>>>(first, n, out);
  return (int)hipGetLastError();
}

}  // extern "C"
