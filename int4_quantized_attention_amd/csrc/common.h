// Device helpers shared by the rotattn HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define RA_DEV __device__ __forceinline__


namespace ra {

// ---- wave reductions ------------------------------------------------------------
RA_DEV float wave_max(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

RA_DEV float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only: this wave's LDS operations complete
// (lgkmcnt(0)), then s_barrier.  __syncthreads() also waits for every vector
// memory operation in flight (vmcnt(0)), which would drain the global loads a
// pipelined loop issues ahead of time; the kernels that use this barrier wait
// for the loads they need explicitly.  The scheduling fences keep the compiler
// from moving memory operations across it.
RA_DEV void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS copies (buffer_load_dwordx4 ... lds) through a buffer
// resource: copy J moves one contiguous kilobyte (16 bytes per lane) to dst + 1024 J
// from the resource's byte offset soff + 1024 J + the lane's offset; the immediate
// offset applies to the global and the LDS address alike, and reads past the
// resource's range return zero.
template <int J>
RA_DEV void dma_one(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int lane_off, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 4096 * (J >> 2)), 16, lane_off,
                                           soff + 4096 * (J >> 2), 1024 * (J & 3), 0);
}
template <int... J>
RA_DEV void dma_all(std::integer_sequence<int, J...>, __amdgpu_buffer_rsrc_t r, uint8_t* dst, int lane_off,
                    int soff) {
  (dma_one<J>(r, dst, lane_off, soff), ...);
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left unconstrained)
template <int n>
RA_DEV void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// max / sum of a value and the one held by lane l ^ 32 (v_permlane32_swap, no LDS)
RA_DEV float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
RA_DEV float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// tokens of head bh that exist: lens[bh / H] in a variable-length batch, else N
RA_DEV int64_t valid_len(int nlens, const int* lens, int bh, int H, int64_t N) {
  return nlens ? (int64_t)lens[bh / H] : N;
}

// binary32 -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN)
RA_DEV uint16_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// four consecutive output values at element offset off of a binary32, binary16 or
// bfloat16 tensor (kind 0, 1, 2)
RA_DEV void store_out4(void* out, int kind, int64_t off, float o0, float o1, float o2, float o3) {
  if (kind == 1) {
    *(f16x4*)((_Float16*)out + off) = f16x4{(_Float16)o0, (_Float16)o1, (_Float16)o2, (_Float16)o3};
  } else if (kind == 2) {
    const uint32_t w0 = (uint32_t)f32_to_bf16(o0) | ((uint32_t)f32_to_bf16(o1) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(o2) | ((uint32_t)f32_to_bf16(o3) << 16);
    *(u32x2*)((uint16_t*)out + off) = u32x2{w0, w1};
  } else {
    *(f32x4*)((float*)out + off) = f32x4{o0, o1, o2, o3};
  }
}

}  // namespace ra
