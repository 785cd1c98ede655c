// gemm_decode.hip -- the small-T (decode) INT4 x INT4 GEMM with the fused
// dequantization epilogue (QUIK blog, "QUIK quantization" part 4: INT4
// operands, INT32 accumulation; part 1: dequantize, add the FP16 outlier
// product, round once), for T <= 32 on gfx950.
//
// At decode sizes the work is streaming the weight matrix once: 2TNK ops
// against N*K/2 bytes, far below the MFMA ridge.  So the design serves HBM:
//   - a workgroup owns 32 output channels (one 32x32 MFMA block column) and
//     its four wavefronts split K into quarters, so that 4 x N/32 wavefronts
//     stream independent weight ranges with many loads in flight;
//   - both operands go global -> registers -> widened int8 -> MFMA, with a
//     kDcD-step register ring (the activation rows are a few KB, L2-resident;
//     rows past T are clamped onto row T-1 and their outputs dropped);
//   - the four partial INT32 blocks (exact) and the four quarters of the FP16
//     outlier product meet in LDS; wavefront 0 sums them in a fixed order and
//     applies the epilogue.
// A k-step is 128 codes: lane (l32, g) holds dwords [8g, 8g+8) of its row,
// MFMA c of a step takes widened slot 4g + c on both operands.
#include "gemm_common.h"
#include "rq_kernels.h"

namespace rq {

namespace {
constexpr int kDcD = 6;  // load ring depth (k-steps)
}  // namespace

template <bool XU, int MODE>
__global__ __launch_bounds__(256) void gemm_decode(GemmArgs p) {
  __shared__ int32_t red_i[3][16 * 64];   // partial accumulators of waves 1..3
  __shared__ float red_f[3][16 * 64];     // partial outlier products of waves 1..3
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 32, Kb = p.Kb;
  const int nsteps = (int)(Kb >> 6);
  // this wave's k-steps [kbeg, kend)
  const int kbeg = (int)((int64_t)nsteps * wave / 4), kend = (int)((int64_t)nsteps * (wave + 1) / 4);
  const uint8_t *ap = p.qx + min((int64_t)l32, p.T - 1) * Kb + 32 * g;
  const uint8_t *bp = p.qw + min(n0 + l32, p.N - 1) * Kb + 32 * g;
  const int last = max(kend - 1, kbeg);

  v16i acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0;
  uint4 ra[kDcD][2], rb[kDcD][2];
  auto gload = [&](int s, int kb) {
    const int64_t o = (int64_t)kb * 64;
    ra[s][0] = *reinterpret_cast<const uint4 *>(ap + o);
    ra[s][1] = *reinterpret_cast<const uint4 *>(ap + o + 16);
    rb[s][0] = *reinterpret_cast<const uint4 *>(bp + o);
    rb[s][1] = *reinterpret_cast<const uint4 *>(bp + o + 16);
  };
#pragma unroll
  for (int s = 0; s < kDcD; ++s) gload(s, min(kbeg + s, last));
  // Fixed groups of kDcD steps; steps past kend multiply a zeroed operand,
  // so the loop holds no branch (a branch there makes the compiler copy the
  // ring at the back edge and wait for every load in flight).
  for (int kb0 = kbeg; kb0 < kend; kb0 += kDcD) {
#pragma unroll
    for (int u = 0; u < kDcD; ++u) {
      const int kb = kb0 + u;
      const uint32_t live = kb < kend ? 0xFFFFFFFFu : 0u;
      v4i aw[4], bw[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 &wa = ra[u][c >> 1], &wb = rb[u][c >> 1];
        const uint32_t a0 = ((c & 1) ? wa.z : wa.x) & live, a1 = ((c & 1) ? wa.w : wa.y) & live;
        aw[c] = XU ? widen_unsigned(a0, a1) : widen_signed(a0, a1);
        bw[c] = widen_signed((c & 1) ? wb.z : wb.x, (c & 1) ? wb.w : wb.y);
      }
      __builtin_amdgcn_sched_barrier(0);
      gload(u, min(kb + kDcD, last));
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(aw[c], bw[c], acc, 0, 0, 0);
    }
  }

  // FP16 outlier product: this wave's quarter of the n_out columns (whole
  // 16-column MFMA steps), lane (l32, g) supplying halves [k0 + 8g, k0 + 8g + 8)
  v16f fo;
#pragma unroll
  for (int r = 0; r < 16; ++r) fo[r] = 0.0f;
  if (MODE == 2 && p.n_out > 0) {
    const int nk = p.n_out / 16;
    const int k_lo = nk * wave / 4, k_hi = nk * (wave + 1) / 4;
    const __half *xa = p.xo + min((int64_t)l32, p.T - 1) * p.n_out + 8 * g;
    const __half *wb = p.wo + min(n0 + l32, p.N - 1) * p.n_out + 8 * g;
    for (int k = k_lo; k < k_hi; ++k) {
      v8h av, bv;
      const uint4 ta = *reinterpret_cast<const uint4 *>(xa + 16 * k);
      const uint4 tb = *reinterpret_cast<const uint4 *>(wb + 16 * k);
      __builtin_memcpy(&av, &ta, 16);
      __builtin_memcpy(&bv, &tb, 16);
      fo = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, fo, 0, 0, 0);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      red_i[wave - 1][r * 64 + lane] = acc[r];
      red_f[wave - 1][r * 64 + lane] = fo[r];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[r] += red_i[w][r * 64 + lane];
      fo[r] += red_f[w][r * 64 + lane];
    }

  // Epilogue.  32x32 accumulator layout: lane l, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32.
  constexpr int kShift = XU ? 4 : 8;
  const int64_t gn = n0 + l32;
  if (MODE == 0) {
    int32_t *out = reinterpret_cast<int32_t *>(p.out);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t gm = 8 * (r >> 2) + 4 * g + (r & 3);
      if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = acc[r] >> kShift;
    }
    return;
  }
  const int64_t gnc = min(gn, p.N - 1);
  const float swn = p.sw[gnc];
  const int32_t rsn = (MODE == 2 && p.zx) ? p.rowsum[gnc] : 0;
  __half *out = reinterpret_cast<__half *>(p.out);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t gm = 8 * (r >> 2) + 4 * g + (r & 3);
    const int64_t gmc = min(gm, p.T - 1);
    int32_t v = acc[r] >> kShift;
    if (MODE == 2 && p.zx) v -= p.zx[gmc] * rsn;
    const float y = (float)v * p.sx[gmc] * swn + fo[r];
    if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = __float2half_rn(y);
  }
}

bool gemm_decode_fits(const GemmArgs &p) { return p.T <= 32 && p.Kb % 64 == 0 && p.Kb >= 64; }

hipError_t launch_gemm_decode(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  const dim3 grid((unsigned)((p.N + 31) / 32)), block(256);
  if (mode == 0) {
    if (x_unsigned) gemm_decode<true, 0><<<grid, block, 0, st>>>(p);
    else gemm_decode<false, 0><<<grid, block, 0, st>>>(p);
  } else if (mode == 1) {
    gemm_decode<false, 1><<<grid, block, 0, st>>>(p);
  } else {
    if (x_unsigned) gemm_decode<true, 2><<<grid, block, 0, st>>>(p);
    else gemm_decode<false, 2><<<grid, block, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace rq
