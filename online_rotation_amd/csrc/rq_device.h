// rq_device.h -- device-side helpers shared by the gfx950 kernels of the
// rotation + W4A4 library (internal; not part of the C ABI).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Orders this wave's earlier LDS writes before its later LDS reads (the wave
// works alone on its LDS slice, so no workgroup barrier is involved).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Eight fp16 values (one 16-byte load) to fp32, exactly.
__device__ __forceinline__ void h8_to_f32(uint4 raw, float *out) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __half2 h = *reinterpret_cast<const __half2 *>(&w[i]);
    float2 f = __half22float2(h);
    out[2 * i] = f.x;
    out[2 * i + 1] = f.y;
  }
}

// Symmetric INT4 code: clamp(rne(v * inv), -qmax, qmax).  `inv` is the fp32
// reciprocal of the row scale (0 for an all-zero row, giving code 0).
__device__ __forceinline__ int quant_sym(float v, float inv, float qmax) {
  float r = __builtin_rintf(v * inv);
  r = __builtin_amdgcn_fmed3f(r, -qmax, qmax);
  return (int)r;
}

// Asymmetric INT4 code: clamp(rne(v * inv) + zero, 0, 15).
__device__ __forceinline__ int quant_asym(float v, float inv, float zero) {
  float r = __builtin_rintf(v * inv) + zero;
  r = __builtin_amdgcn_fmed3f(r, 0.0f, 15.0f);
  return (int)r;
}

// Pack eight codes (element 2j low nibble, 2j+1 high nibble) into a dword.
__device__ __forceinline__ uint32_t pack8(const int *c) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= (uint32_t)(c[i] & 0xF) << (4 * i);
  return w;
}

// Symmetric per-row scale: fp32(clip * absmax / 7) with the scale's
// reciprocal used for the codes.
__device__ __forceinline__ void sym_scale(float amax, float clip, float &s, float &inv) {
  s = (clip * amax) / 7.0f;
  inv = s > 0.0f ? 1.0f / s : 0.0f;
}

// Asymmetric per-row parameters from the row's min and max.
__device__ __forceinline__ void asym_params(float mn, float mx, float &s, float &inv, int &zero) {
  const float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
  s = (hi - lo) / 15.0f;
  if (s > 0.0f) {
    inv = 1.0f / s;
    float z = __builtin_rintf(-lo / s);
    zero = (int)__builtin_amdgcn_fmed3f(z, 0.0f, 15.0f);
  } else {
    inv = 0.0f;
    zero = 0;
  }
}

}  // namespace rq
