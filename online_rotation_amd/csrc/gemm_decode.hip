// gemm_decode.hip -- the small-T (decode) INT4 x INT4 GEMM with the fused
// dequantization epilogue (QUIK blog, "QUIK quantization" part 4: INT4
// operands, INT32 accumulation; part 1: dequantize, add the FP16 outlier
// product, round once), for T <= 32 on gfx950.
//
// At decode sizes the work is streaming the weight matrix once: 2TNK ops
// against N*K/2 bytes, far below the MFMA ridge.  So the design serves HBM:
//   - each wavefront owns 32 output channels (one 32x32 MFMA block column)
//     and streams their weight rows from start to end, one sequential stream
//     per row (splitting K across wavefronts gave every row several
//     concurrent streams and measured 25% slower);
//   - both operands go global -> registers -> widened int8 -> MFMA, with a
//     kDcD-step register ring (the activation rows are a few KB, L2-resident;
//     rows past T are clamped onto row T-1 and their outputs dropped);
//   - the FP16 outlier fragments are all loaded before the ring's prologue,
//     so their latency hides behind the first weight loads.
#include "gemm_common.h"
#include "rq_kernels.h"

namespace rq {

namespace {
constexpr int kDcD = 6;  // load ring depth (k-steps)
}  // namespace

template <bool XU, int MODE>
__global__ __launch_bounds__(256) void gemm_decode(GemmArgs p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 128 + wave * 32, Kb = p.Kb;
  if (n0 >= p.N) return;  // whole wavefront past the last channel
  const int nsteps = (int)(Kb >> 6), last = nsteps - 1;
  const uint8_t *ap = p.qx + min((int64_t)l32, p.T - 1) * Kb + 32 * g;
  const uint8_t *bp = p.qw + min(n0 + l32, p.N - 1) * Kb + 32 * g;

  // FP16 outlier product, lane (l32, g) supplying halves [16k + 8g, 16k + 8g + 8)
  // of its row (A) or column (B); up to kOutK steps per batch of loads
  constexpr int kOutK = 16;
  v16f fo;
#pragma unroll
  for (int r = 0; r < 16; ++r) fo[r] = 0.0f;
  const int nk = MODE == 2 ? p.n_out / 16 : 0;
  const __half *xa = p.xo + min((int64_t)l32, p.T - 1) * p.n_out + 8 * g;
  const __half *wb = p.wo + min(n0 + l32, p.N - 1) * p.n_out + 8 * g;
  uint4 oa[kOutK], ob[kOutK];
  auto oload = [&](int k0) {  // steps past nk are clamped and never multiplied
#pragma unroll
    for (int k = 0; k < kOutK; ++k) {
      const int kk = 16 * min(k0 + k, nk - 1);
      oa[k] = *reinterpret_cast<const uint4 *>(xa + kk);
      ob[k] = *reinterpret_cast<const uint4 *>(wb + kk);
    }
  };
  auto omul = [&](int k0) {
#pragma unroll
    for (int k = 0; k < kOutK; ++k) {
      if (k0 + k < nk) {
        v8h av, bv;
        __builtin_memcpy(&av, &oa[k], 16);
        __builtin_memcpy(&bv, &ob[k], 16);
        fo = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, fo, 0, 0, 0);
      }
    }
  };
  if (nk > 0) oload(0);

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
  for (int s = 0; s < kDcD; ++s) gload(s, min(s, last));
  if (nk > 0) {
    omul(0);
    for (int k0 = kOutK; k0 < nk; k0 += kOutK) {  // more than kOutK*16 outlier columns
      oload(k0);
      omul(k0);
    }
  }
  // Fixed groups of kDcD steps; steps past the end multiply a zeroed
  // operand, so the loop holds no branch (a branch there makes the compiler
  // copy the ring at the back edge and wait for every load in flight).
  for (int kb0 = 0; kb0 < nsteps; kb0 += kDcD) {
#pragma unroll
    for (int u = 0; u < kDcD; ++u) {
      const int kb = kb0 + u;
      const uint32_t live = kb < nsteps ? 0xFFFFFFFFu : 0u;
      v4i aw[4], bw[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 &wa = ra[u][c >> 1], &wq = rb[u][c >> 1];
        const uint32_t a0 = ((c & 1) ? wa.z : wa.x) & live, a1 = ((c & 1) ? wa.w : wa.y) & live;
        aw[c] = XU ? widen_unsigned(a0, a1) : widen_signed(a0, a1);
        bw[c] = widen_signed((c & 1) ? wq.z : wq.x, (c & 1) ? wq.w : wq.y);
      }
      __builtin_amdgcn_sched_barrier(0);
      gload(u, min(kb + kDcD, last));
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(aw[c], bw[c], acc, 0, 0, 0);
    }
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
  const dim3 grid((unsigned)((p.N + 127) / 128)), block(256);
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
