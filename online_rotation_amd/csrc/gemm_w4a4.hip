// gemm_w4a4.hip -- INT4 x INT4 GEMM with INT32 accumulation on gfx950 INT8
// matrix cores, with the dequantization epilogue fused (QUIK blog, "QUIK
// quantization" part 4: INT4 operands, INT32 accumulation; part 1: dequantize
// to FP16 and add the FP16 outlier product).
//
// Packed int4 codes are widened to int8 in registers right before the MFMA.
// Signed codes keep the nibble in the high half of each byte ((b << 4) & 0xF0
// and b & 0xF0), unsigned codes in the low half (b & 0x0F, (b >> 4) & 0x0F),
// so every product is scaled by exactly 256 (signed x signed) or 16 (unsigned
// x signed); the scale is shifted out of the INT32 sum exactly.  Both
// operands are widened the same way, so the k order inside an MFMA is
// irrelevant.  Every widened product is at most 128*128 = 2^14 in magnitude
// (signed) or 15*128 (unsigned), so the INT32 sum cannot overflow for the
// K <= 65536 the C ABI accepts.
//
// Tile: 128 (tokens) x 128 (output channels) per 256-thread workgroup, k-step
// 128 codes (64 bytes) staged in LDS with double buffering; each wavefront
// owns a 64 x 64 sub-tile = 2 x 2 MFMA 32x32x32 blocks.
#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {

constexpr int kBM = 128, kBN = 128, kBKB = 64;  // tile rows, cols, k-step bytes
constexpr int kLdsRow = kBKB + 16;              // padded LDS row (bytes)

__device__ __forceinline__ v4i widen_signed(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(w0 & 0xF0F0F0F0u);
  r[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(w1 & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ v4i widen_unsigned(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)(w0 & 0x0F0F0F0Fu);
  r[1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
  r[2] = (int)(w1 & 0x0F0F0F0Fu);
  r[3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
  return r;
}

template <bool XU, int MODE>
__global__ __launch_bounds__(256) void gemm_w4a4(GemmArgs p) {
  __shared__ __align__(16) uint8_t As[2][kBM * kLdsRow];
  __shared__ __align__(16) uint8_t Bs[2][kBN * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t Kb = p.Kb;
  const int nk = (int)((Kb + kBKB - 1) / kBKB);

  uint4 ra[2], rb[2];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256, row = c >> 2, cc = c & 3;
      const int64_t off = (int64_t)kb * kBKB + cc * 16;
      const int64_t gm = m0 + row, gn = n0 + row;
      ra[i] = (gm < p.T && off < Kb) ? *reinterpret_cast<const uint4 *>(p.qx + gm * Kb + off)
                                     : make_uint4(0, 0, 0, 0);
      rb[i] = (gn < p.N && off < Kb) ? *reinterpret_cast<const uint4 *>(p.qw + gn * Kb + off)
                                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256, row = c >> 2, cc = c & 3;
      *reinterpret_cast<uint4 *>(&As[buf][row * kLdsRow + cc * 16]) = ra[i];
      *reinterpret_cast<uint4 *>(&Bs[buf][row * kLdsRow + cc * 16]) = rb[i];
    }
  };

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  gload(0);
  sstore(0);
  __syncthreads();
  const int g = lane >> 5, l32 = lane & 31;
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nk) gload(kb + 1);
    uint32_t aw[2][8], bw[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint8_t *src = &As[buf][(wm * 64 + i * 32 + l32) * kLdsRow + g * 32];
      const uint4 x0 = *reinterpret_cast<const uint4 *>(src);
      const uint4 x1 = *reinterpret_cast<const uint4 *>(src + 16);
      aw[i][0] = x0.x; aw[i][1] = x0.y; aw[i][2] = x0.z; aw[i][3] = x0.w;
      aw[i][4] = x1.x; aw[i][5] = x1.y; aw[i][6] = x1.z; aw[i][7] = x1.w;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t *src = &Bs[buf][(wn * 64 + j * 32 + l32) * kLdsRow + g * 32];
      const uint4 x0 = *reinterpret_cast<const uint4 *>(src);
      const uint4 x1 = *reinterpret_cast<const uint4 *>(src + 16);
      bw[j][0] = x0.x; bw[j][1] = x0.y; bw[j][2] = x0.z; bw[j][3] = x0.w;
      bw[j][4] = x1.x; bw[j][5] = x1.y; bw[j][6] = x1.z; bw[j][7] = x1.w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v4i ao[2], bo[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        ao[i] = XU ? widen_unsigned(aw[i][2 * c], aw[i][2 * c + 1])
                   : widen_signed(aw[i][2 * c], aw[i][2 * c + 1]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bo[j] = widen_signed(bw[j][2 * c], bw[j][2 * c + 1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[i], bo[j], acc[i][j], 0, 0, 0);
    }
    if (kb + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  constexpr int kShift = XU ? 4 : 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t gn = n0 + wn * 64 + j * 32 + l32;
      const int64_t rbase = m0 + wm * 64 + i * 32 + 4 * g;
      if (MODE == 0) {
        int32_t *out = reinterpret_cast<int32_t *>(p.out);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gm = rbase + 8 * (r >> 2) + (r & 3);
          if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = acc[i][j][r] >> kShift;
        }
      } else {
        v16f f;
        const float swn = gn < p.N ? p.sw[gn] : 0.0f;
        const int32_t rsn = (MODE == 2 && p.zx && gn < p.N) ? p.rowsum[gn] : 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gm = rbase + 8 * (r >> 2) + (r & 3);
          int32_t v = acc[i][j][r] >> kShift;
          float sxm = 0.0f;
          if (gm < p.T) {
            sxm = p.sx[gm];
            if (MODE == 2 && p.zx) v -= p.zx[gm] * rsn;
          }
          f[r] = (float)v * sxm * swn;
        }
        if (MODE == 2 && p.n_out > 0) {
          // FP16 outlier product on FP16 matrix cores, fp32 accumulation on
          // top of the dequantized INT4 part.
          const int64_t am = m0 + wm * 64 + i * 32 + l32;
          const int64_t bn = n0 + wn * 64 + j * 32 + l32;
          const __half *arow = p.xo + am * p.n_out;
          const __half *brow = p.wo + bn * p.n_out;
          for (int k0 = 0; k0 < p.n_out; k0 += 16) {
            v8h av, bv;
            uint4 ua = am < p.T ? *reinterpret_cast<const uint4 *>(arow + k0 + g * 8)
                                : make_uint4(0, 0, 0, 0);
            uint4 ub = bn < p.N ? *reinterpret_cast<const uint4 *>(brow + k0 + g * 8)
                                : make_uint4(0, 0, 0, 0);
            __builtin_memcpy(&av, &ua, 16);
            __builtin_memcpy(&bv, &ub, 16);
            f = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, f, 0, 0, 0);
          }
        }
        __half *out = reinterpret_cast<__half *>(p.out);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gm = rbase + 8 * (r >> 2) + (r & 3);
          if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = __float2half_rn(f[r]);
        }
      }
    }
  }
}

hipError_t launch_gemm(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  const dim3 grid((unsigned)((p.N + kBN - 1) / kBN), (unsigned)((p.T + kBM - 1) / kBM));
  const dim3 block(256);
  if (mode == 0) {
    if (x_unsigned) gemm_w4a4<true, 0><<<grid, block, 0, st>>>(p);
    else gemm_w4a4<false, 0><<<grid, block, 0, st>>>(p);
  } else if (mode == 1) {
    gemm_w4a4<false, 1><<<grid, block, 0, st>>>(p);
  } else {
    if (x_unsigned) gemm_w4a4<true, 2><<<grid, block, 0, st>>>(p);
    else gemm_w4a4<false, 2><<<grid, block, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace rq
