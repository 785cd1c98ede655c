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

// Streaming accesses for data touched once (the quantizers' input rows and
// output codes): nontemporal 16-byte loads and 4- / 16-byte stores.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const void *p) {
  const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(void *p, uint4 v) {
  __builtin_nontemporal_store((v4u32){v.x, v.y, v.z, v.w}, reinterpret_cast<v4u32 *>(p));
}
__device__ __forceinline__ void store_nt(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }

// Orders this wave's earlier LDS writes before its later LDS reads (the wave
// works alone on its LDS slice, so no workgroup barrier is involved).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Wave-wide max / min / inclusive prefix sum on the DPP paths (no LDS
// crossbar round trips): quad and mirror permutations within rows of 16
// lanes, then the row-15 and row-31 broadcasts (gfx9 encodings).  max and
// min return the wave's value in a scalar register.
#define RQ_DPP(old, v, ctrl, rows) __builtin_amdgcn_update_dpp((old), (v), (ctrl), (rows), 0xF, false)
__device__ __forceinline__ float wave_max_dpp(float v) {
  int x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(RQ_DPP(x, x, 0xB1, 0xF)));   // quad_perm [1,0,3,2]
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(RQ_DPP(x, x, 0x4E, 0xF)));   // quad_perm [2,3,0,1]
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(RQ_DPP(x, x, 0x141, 0xF)));  // row_half_mirror
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(RQ_DPP(x, x, 0x140, 0xF)));  // row_mirror: every lane holds its row's max
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(RQ_DPP(x, x, 0x142, 0xA)));  // row_bcast:15 into rows 1, 3
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(RQ_DPP(x, x, 0x143, 0xC)));  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_min_dpp(float v) {
  int x = __float_as_int(v);
  v = fminf(v, __int_as_float(RQ_DPP(x, x, 0xB1, 0xF)));
  x = __float_as_int(v);
  v = fminf(v, __int_as_float(RQ_DPP(x, x, 0x4E, 0xF)));
  x = __float_as_int(v);
  v = fminf(v, __int_as_float(RQ_DPP(x, x, 0x141, 0xF)));
  x = __float_as_int(v);
  v = fminf(v, __int_as_float(RQ_DPP(x, x, 0x140, 0xF)));
  x = __float_as_int(v);
  v = fminf(v, __int_as_float(RQ_DPP(x, x, 0x142, 0xA)));
  x = __float_as_int(v);
  v = fminf(v, __int_as_float(RQ_DPP(x, x, 0x143, 0xC)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// inclusive prefix sum over the lanes; lanes without a source add 0
__device__ __forceinline__ int wave_scan_dpp(int x) {
  x += RQ_DPP(0, x, 0x111, 0xF);  // row_shr:1
  x += RQ_DPP(0, x, 0x112, 0xF);  // row_shr:2
  x += RQ_DPP(0, x, 0x114, 0xF);  // row_shr:4
  x += RQ_DPP(0, x, 0x118, 0xF);  // row_shr:8: every lane holds its row prefix
  x += RQ_DPP(0, x, 0x142, 0xA);  // row_bcast:15 into rows 1, 3
  x += RQ_DPP(0, x, 0x143, 0xC);  // row_bcast:31 into rows 2, 3
  return x;
}
// max over the wave of 32-bit patterns compared as unsigned (for floats
// that are >= 0 this is their max: a NaN, the largest pattern, would
// win); each stage is one DPP max (the identity 0 fills lanes without a
// source), where the float form needs a move and two max per stage
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t x) {
  x = max(x, (uint32_t)RQ_DPP(0, (int)x, 0xB1, 0xF));
  x = max(x, (uint32_t)RQ_DPP(0, (int)x, 0x4E, 0xF));
  x = max(x, (uint32_t)RQ_DPP(0, (int)x, 0x141, 0xF));
  x = max(x, (uint32_t)RQ_DPP(0, (int)x, 0x140, 0xF));
  x = max(x, (uint32_t)RQ_DPP(0, (int)x, 0x142, 0xA));
  x = max(x, (uint32_t)RQ_DPP(0, (int)x, 0x143, 0xC));
  return __builtin_amdgcn_readlane(x, 63);
}
#undef RQ_DPP

// The wave's max / min / sum, in every lane (a scalar register).
// Issue priority for the item done (of n) of a grid-stride loop: level 3
// for the first quarter of the wavefront's items, down to 0 for the last.
// Among waves of equal priority a SIMD issues oldest first, so the
// workgroups placed last on it fall behind and, at equal priority
// throughout, finish the launch alone with their latency exposed; lowering
// the priority of waves that are ahead lets the late ones catch up.
__device__ __forceinline__ void progress_prio(int done, int n) {
  switch (3 - min(3, (4 * done) / max(n, 1))) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

__device__ __forceinline__ float wave_max(float v) { return wave_max_dpp(v); }
__device__ __forceinline__ float wave_min(float v) { return wave_min_dpp(v); }
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_scan_dpp(v), 63); }

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

// Symmetric per-row scale: fp32(clip * absmax / 7), with the product exact in
// fp64 (24 x 24 bits) and the quotient rounded to fp64 and then to fp32, as
// the exact scale is rounded; also the scale's reciprocal used for the codes.
__device__ __forceinline__ void sym_scale(float amax, float clip, float &s, float &inv) {
  s = (float)((double)clip * (double)amax / 7.0);
  inv = s > 0.0f ? 1.0f / s : 0.0f;
}

}  // namespace rq
