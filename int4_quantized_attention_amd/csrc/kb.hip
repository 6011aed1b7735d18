// Micro-benchmarks of the MI355X (gfx950) rates the kernels are measured against:
// back-to-back MFMA throughput per instruction form, HBM streaming bandwidth, LDS
// read bandwidth alone and feeding f16 MFMAs, and the error of the hardware exp2
// (v_exp_f32) that the P-level fast path relies on.
// Built into libkb.so, separate from the product library; driven by kb.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
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

// LDS reads: each wave reads 16 bytes per lane per ds_read_b128, 8 per round at
// consecutive kilobytes (no bank conflicts), over a 64 KiB buffer (two workgroups per
// CU).  MFMA = 1: each read instead feeds one v_mfma_f32_32x32x16_f16 as its A
// operand (B from registers, four accumulator chains), 1 KiB per 32768 flops, the
// ratio of an attention kernel with 32 query rows per wave.  Per workgroup, lane 0
// of wave 0 records the shader clocks of its loop (s_memtime).
constexpr int kLdsBytes = 65536;
template <int MFMA>
__global__ __launch_bounds__(256) void kb_lds_k(int iters, float* out, unsigned long long* cycles) {
  extern __shared__ __align__(16) uint8_t kb_lds[];
  const int t = threadIdx.x;
  for (int i = t * 16; i < kLdsBytes; i += 256 * 16) {
    const u32x4 v = {(unsigned)i, (unsigned)i + 1u, (unsigned)i + 2u, (unsigned)i + 3u};
    *(u32x4*)(kb_lds + i) = v;
  }
  __syncthreads();
  const unsigned long long c0 = __builtin_readcyclecounter();
  // wave w reads its own 16 KiB quarter, alternating halves from round to round; the
  // memory clobber keeps the compiler from reusing a previous round's values
  const uint8_t* const base = kb_lds + (t >> 6) * 16384 + (t & 63) * 16;
  float r = 0.f;
  if constexpr (MFMA == 0) {
    unsigned acc = 0;
    for (int i = 0; i < iters; ++i) {
      const uint8_t* const p = base + (i & 1) * 8192;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4 v = *(const u32x4*)(p + u * 1024);
        acc = acc + v[0] + v[1];
        acc = acc + v[2] + v[3];
      }
      asm volatile("" ::: "memory");
    }
    r = (float)acc;
  } else {
    const f16x8 b = {(_Float16)t, 1, 2, 3, 4, 5, 6, 7};
    f32x16 acc[kChains] = {};
    for (int i = 0; i < iters; ++i) {
      const uint8_t* const p = base + (i & 1) * 8192;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const f16x8 a = *(const f16x8*)(p + u * 1024);
        acc[u % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[u % kChains], 0, 0, 0);
      }
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][0] + acc[c][15];
  }
  const unsigned long long c1 = __builtin_readcyclecounter();
  out[blockIdx.x * 256 + t] = r;
  if (t == 0) cycles[blockIdx.x] = c1 - c0;
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
// LDS micro-benchmark (mfma 0: reads alone, 1: reads feeding f16 MFMAs) on `blocks`
// workgroups of 4 waves with 64 KiB of LDS each, `iters` rounds of 8 reads per wave.
// out: device float [blocks * 256]; cycles: device u64 [blocks].
int kb_lds_launch(int mfma, int blocks, int iters, float* out, unsigned long long* cycles, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (mfma) kb_lds_k<1><<<blocks, 256, kLdsBytes, st>>>(iters, out, cycles);
  else kb_lds_k<0><<<blocks, 256, kLdsBytes, st>>>(iters, out, cycles);
  return (int)hipGetLastError();
}
int kb_lds_bytes(void) { return kLdsBytes; }

// first + n <= 2^32; out: device float [n]
int kb_exp2_launch(uint32_t first, int64_t n, float* out, void* stream) {
  if (n < 0 || (uint64_t)first + (uint64_t)n > ((uint64_t)1 << 32)) return (int)hipErrorInvalidValue;
  const int64_t blocks = (n + 255) / 256;
  kb_exp2_k<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, (hipStream_t)stream>>>(first, n, out);
  return (int)hipGetLastError();
}

}  // extern "C"
