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
// Tile: (64*WMB) x (64*WNB) per 256-thread workgroup (2 x 2 wavefronts, each
// owning WMB x WNB MFMA 32x32x32 blocks).  Each k-step of 128 codes (64 bytes
// per row) goes global -> registers -> LDS -> registers:
//   - global loads run kDepth k-steps ahead in a register ring;
//   - LDS holds three k-steps; during step kb a wavefront multiplies the
//     fragments of step kb (already in registers), reads step kb+1's
//     fragments from LDS and stores step kb+2 into LDS;
//   - one workgroup barrier per step: a buffer is read one step after it
//     was stored and overwritten two steps after it was read.
#include "rq_device.h"
#include "rq_kernels.h"
#include "gemm_common.h"


namespace rq {


constexpr int kBKB = 64;              // k-step: 128 codes = 64 bytes per row
constexpr int kDepth = 3;             // global prefetch distance in k-steps

// LDS tile rows are 64 bytes (four 16-byte chunks) with the chunk index
// XOR-swizzled by the row, so that both the cooperative 16-byte stores (four
// lanes per row) and the per-lane 16-byte fragment reads (one row per lane)
// touch distinct banks within every group of 8 or 16 lanes.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kBKB + ((chunk ^ (((row >> 1) ^ (row >> 3)) & 3)) << 4);
}

template <int WMB, int WNB, bool XU, int MODE>
__global__ __launch_bounds__(256) void gemm_w4a4(GemmArgs p, int nt_m, int nt_n) {
  constexpr int BM = 64 * WMB, BN = 64 * WNB;
  constexpr int LA = BM * 4 / 256, LB = BN * 4 / 256;  // 16-byte chunks per thread per k-step
  __shared__ __align__(16) uint8_t As[3][BM * kBKB];
  __shared__ __align__(16) uint8_t Bs[3][BN * kBKB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  int tm, tn;
  map_tile(blockIdx.x, nt_m, nt_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t Kb = p.Kb;
  const int nfull = (int)(Kb / kBKB);               // full 64-byte k-steps
  const int nsteps = nfull + ((Kb % kBKB) ? 1 : 0);  // plus a last 32-byte half step

  // tile bases are uniform; per-thread 32-bit offsets (rows clamped)
  const uint8_t *abase = p.qx + m0 * Kb;
  const uint8_t *bbase = p.qw + n0 * Kb;
  uint32_t aoff[LA], boff[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int c = tid + i * 256;
    aoff[i] = (uint32_t)((min(m0 + (c >> 2), p.T - 1) - m0) * Kb) + (c & 3) * 16;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int c = tid + i * 256;
    boff[i] = (uint32_t)((min(n0 + (c >> 2), p.N - 1) - n0) * Kb) + (c & 3) * 16;
  }
  uint4 ra[kDepth][LA], rb[kDepth][LB];
  auto gload = [&](int slot, int kb) {
    const uint8_t *a = abase + (int64_t)kb * kBKB, *b = bbase + (int64_t)kb * kBKB;
    if (kb < nfull) {
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[slot][i] = *reinterpret_cast<const uint4 *>(a + aoff[i]);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[slot][i] = *reinterpret_cast<const uint4 *>(b + boff[i]);
    } else {  // half step: chunks 0 and 1 are data, 2 and 3 are zero
#pragma unroll
      for (int i = 0; i < LA; ++i)
        ra[slot][i] = ((tid + i * 256) & 2) ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4 *>(a + aoff[i]);
#pragma unroll
      for (int i = 0; i < LB; ++i)
        rb[slot][i] = ((tid + i * 256) & 2) ? make_uint4(0, 0, 0, 0) : *reinterpret_cast<const uint4 *>(b + boff[i]);
    }
  };
  auto sstore = [&](int buf, int slot) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<uint4 *>(&As[buf][lds_off(c >> 2, c & 3)]) = ra[slot][i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<uint4 *>(&Bs[buf][lds_off(c >> 2, c & 3)]) = rb[slot][i];
    }
  };

  v16i acc[WMB][WNB];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int g = lane >> 5, l32 = lane & 31;
  uint4 fa[2][WMB][2], fb[2][WNB][2];  // packed fragments of two k-steps
  auto lread = [&](int f, int buf) {
#pragma unroll
    for (int i = 0; i < WMB; ++i) {
      const int row = wm * 32 * WMB + i * 32 + l32;
      fa[f][i][0] = *reinterpret_cast<const uint4 *>(&As[buf][lds_off(row, 2 * g)]);
      fa[f][i][1] = *reinterpret_cast<const uint4 *>(&As[buf][lds_off(row, 2 * g + 1)]);
    }
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const int row = wn * 32 * WNB + j * 32 + l32;
      fb[f][j][0] = *reinterpret_cast<const uint4 *>(&Bs[buf][lds_off(row, 2 * g)]);
      fb[f][j][1] = *reinterpret_cast<const uint4 *>(&Bs[buf][lds_off(row, 2 * g + 1)]);
    }
  };
  auto compute = [&](int f) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v4i ao[WMB], bo[WNB];
#pragma unroll
      for (int i = 0; i < WMB; ++i) {
        const uint4 &x = fa[f][i][c >> 1];
        const uint32_t w0 = (c & 1) ? x.z : x.x, w1 = (c & 1) ? x.w : x.y;
        ao[i] = XU ? widen_unsigned(w0, w1) : widen_signed(w0, w1);
      }
#pragma unroll
      for (int j = 0; j < WNB; ++j) {
        const uint4 &x = fb[f][j][c >> 1];
        bo[j] = widen_signed((c & 1) ? x.z : x.x, (c & 1) ? x.w : x.y);
      }
#pragma unroll
      for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ao[i], bo[j], acc[i][j], 0, 0, 0);
    }
  };

  // prologue: steps 0 and 1 into LDS, step 0's fragments into registers
#pragma unroll
  for (int s = 0; s < kDepth; ++s)
    if (s < nsteps) gload(s, s);
  sstore(0, 0);
  if (nsteps > 1) sstore(1, 1);
  __syncthreads();
  if (kDepth < nsteps) gload(0, kDepth);
  if (kDepth + 1 < nsteps) gload(1, kDepth + 1);
  lread(0, 0);
  // main loop, unrolled by 6 = lcm(2 fragment sets, 3 LDS buffers, kDepth = 3)
  for (int kb0 = 0; kb0 < nsteps; kb0 += 6) {
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      const int kb = kb0 + s;
      if (kb < nsteps) {
        if (kb + 1 < nsteps) lread((s + 1) & 1, (s + 1) % 3);
        compute(s & 1);
        if (kb + 2 < nsteps) {
          sstore((s + 2) % 3, (s + 2) % kDepth);
          if (kb + 2 + kDepth < nsteps) gload((s + 2) % kDepth, kb + 2 + kDepth);
        }
        __syncthreads();
      }
    }
  }

  // Epilogue.  32x32 accumulator layout: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  constexpr int kShift = XU ? 4 : 8;
  const int64_t row0 = m0 + wm * 32 * WMB, col0 = n0 + wn * 32 * WNB;
#pragma unroll
  for (int i = 0; i < WMB; ++i) {
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const int64_t gn = col0 + 32 * j + l32;
      const int64_t rbase = row0 + 32 * i + 4 * g;
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
          const int64_t am = min(row0 + 32 * i + l32, p.T - 1);
          const int64_t bn = min(col0 + 32 * j + l32, p.N - 1);
          const __half *arow = p.xo + am * p.n_out;
          const __half *brow = p.wo + bn * p.n_out;
          for (int k0 = 0; k0 < p.n_out; k0 += 16) {
            v8h av, bv;
            const uint4 ua = *reinterpret_cast<const uint4 *>(arow + k0 + g * 8);
            const uint4 ub = *reinterpret_cast<const uint4 *>(brow + k0 + g * 8);
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

template <int WMB, int WNB>
static hipError_t launch_tiles(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  constexpr int BM = 64 * WMB, BN = 64 * WNB;
  const int nt_m = (int)((p.T + BM - 1) / BM), nt_n = (int)((p.N + BN - 1) / BN);
  const dim3 grid((unsigned)(nt_m * nt_n)), block(256);
  if (mode == 0) {
    if (x_unsigned) gemm_w4a4<WMB, WNB, true, 0><<<grid, block, 0, st>>>(p, nt_m, nt_n);
    else gemm_w4a4<WMB, WNB, false, 0><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  } else if (mode == 1) {
    gemm_w4a4<WMB, WNB, false, 1><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  } else {
    if (x_unsigned) gemm_w4a4<WMB, WNB, true, 2><<<grid, block, 0, st>>>(p, nt_m, nt_n);
    else gemm_w4a4<WMB, WNB, false, 2><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  }
  return hipGetLastError();
}

// Dispatch: the decode kernel for T <= 32, the register-A kernel for
// T >= 256, this file's LDS-tile kernel otherwise (and whenever K is not a
// multiple of 128 codes).
hipError_t launch_gemm(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  if (gemm_decode_fits(p)) return launch_gemm_decode(p, x_unsigned, mode, st);
  if (gemm_ra_fits(p)) return launch_gemm_ra(p, x_unsigned, mode, st);
  return launch_tiles<2, 2>(p, x_unsigned, mode, st);
}

}  // namespace rq
