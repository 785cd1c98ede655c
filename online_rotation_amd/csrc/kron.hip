// kron.hip -- FlatQuant's per-token Kronecker transform (FlatQuant article,
// section 2.3: x' = (x * s) (P1 kron P2), evaluated as P1^T . M . P2 on the
// [n1, n2] reshape M of the scaled row) fused with per-token symmetric INT4,
// for n1 = n2 = 64 on gfx950 FP64 matrix cores.
//
// Why FP64: the rotated value feeds a max-based scale that must agree with
// the exact transform to 1e-6.  Two chained 64-term products accumulated in
// fp32 miss that on real rows (measured 1.07e-6); in fp64 the scaled input
// x * s is exact (fp16 x fp32 fits 53 bits), the products are exact and the
// accumulation error is ~1e-15, so x' is the exact value rounded once to
// fp32.  The price is the FP64 rate: 512 MFMAs of 2048 flops per token.
//
// Per token (one wavefront), with A = P1, B = P2 on the activation side and
// A = P1^{-T}, B = P2^{-T}, division by s, on the weight side:
//   Z   = M . B          16 blocks of 16x16, k = 64 in 16 steps of 4
//   Y^T = Z^T . A        the A operand is Z's own accumulator registers
// Z is produced one row block (16 rows) at a time and folded into Y^T at
// once; Y^T's column blocks go in two passes of two (a pass needs only the
// matching column blocks of Z), so two Z blocks are live next to eight of
// Y^T, within 256 registers: two wavefronts per SIMD.
// v_mfma_f64_16x16x4_f64 operands: lane l supplies A[l%16][k_(l/16)] and
// B[k_(l/16)][l%16]; accumulator register r of lane l holds row 4r + l/16,
// column l%16 (measured on gfx950).
//   Z block (bk, bj): step t pairs k = 16kg + t with lane group kg = l/16, so
//   lane (i, kg) reads 16 contiguous fp16 of M row 16bk + i.  B's columns
//   are taken in the order pi(c) = 4(c%4) + c/4 within each block of 16.
//   Y^T block (bj, bi): step (bk, r) uses Z rows 16bk + 4r + kg in lane group
//   kg, which is register r of Z block (bk, bj) in that lane.
// With pi, register r of lane (i, kg) in Y^T block (bj, bi) holds
// Y[16bi + i][16bj + 4kg + r]: four consecutive columns per lane, i.e. one
// 16-bit group of packed nibbles.
// The B operands (entries of B and A in these lane orders) and the channel
// scales live in LDS as per-lane register images, built once per workgroup.
#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {

namespace {
typedef double v4d __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));
constexpr int kImg = 64 * 64;  // entries per image: 64 registers x 64 lanes
// One workgroup of eight wavefronts per CU (two per SIMD): the images are
// built once per CU, not once per four wavefronts.
constexpr int kKronWaves = 8, kKronThreads = 64 * kKronWaves;
}  // namespace

template <bool DIVIDE>
__global__ __launch_bounds__(kKronThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void kron64_mfma(const __half *__restrict__ x, int64_t T, int64_t ldx,
                                                   const float *__restrict__ fa,
                                                   const float *__restrict__ fb,
                                                   const float *__restrict__ chan_scale, float clip,
                                                   uint8_t *__restrict__ q, float *__restrict__ scale,
                                                   int32_t *__restrict__ code_sum) {
  // register v of lane l: double images at [(v / 2) * 128 + 2 l + v % 2],
  // the float image at [(v / 4) * 256 + 4 l + v % 4]
  __shared__ __align__(16) double imgB[kImg];  // v = 4t + bj:         B[16kg + t][16bj + pi(i)]
  __shared__ __align__(16) double imgA[kImg];  // v = 16bk + 4r + bi:  A[16bk + 4r + kg][16bi + i]
  __shared__ __align__(16) float imgS[kImg];   // v = 16bk + t:        s[64(16bk + i) + 16kg + t]
  __shared__ __align__(16) uint8_t qst[kKronWaves][2048];  // a token's packed codes, per wavefront
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, l16 = lane & 15;
  // All 48 loads of a thread first, then the LDS writes, so the loads are in
  // flight together.  Each image is a permutation of its source (4096
  // entries each), so thread t reads source entries e = 512 it + t
  // (coalesced: a wavefront's load covers 256 contiguous bytes) and writes
  // each to its image slot (register v, lane l) from the inverse maps:
  //   B[R][C]:  v = 4 (R % 16) + C / 16,           l = 16 (R / 16) + pi(C % 16)
  //   A[R][C]:  v = 16 (R / 16) + 4 (R / 4 % 4) + C / 16,  l = 16 (R % 4) + C % 16
  //   s[X]:     v = 16 (X / 1024) + X % 16,        l = 16 (X / 16 % 4) + X / 64 % 16
  // (pi is its own inverse).  Gathered in image order instead, the channel
  // scales alone touched 64 cache lines per load instruction, and every
  // workgroup waited several microseconds on the tables.
  constexpr int kIt = kImg / kKronThreads;
  float vb[kIt], va[kIt], vs[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int e = it * kKronThreads + tid;
    vb[it] = fb[e];
    va[it] = fa[e];
    vs[it] = chan_scale ? chan_scale[e] : 1.0f;
  }
  // The first row block of the wavefront's first token is requested right
  // after the tables (loads complete in order, so the image writes below
  // wait for the tables only), and its memory latency runs under the image
  // set-up.  The index is clamped; a wavefront with no token never uses it.
  const int64_t tfirst = (int64_t)blockIdx.x * kKronWaves + wave;
  uint4 xpre[2];
  {
    const __half *src = x + min(tfirst, T - 1) * ldx + 64 * l16 + 16 * kg;
    xpre[0] = *reinterpret_cast<const uint4 *>(src);
    xpre[1] = *reinterpret_cast<const uint4 *>(src + 8);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int e = it * kKronThreads + tid;
    const int R = e >> 6, C = e & 63, c16 = C & 15;
    {
      const int v = 4 * (R & 15) + (C >> 4), l = 16 * (R >> 4) + 4 * (c16 & 3) + (c16 >> 2);
      imgB[(v >> 1) * 128 + 2 * l + (v & 1)] = (double)vb[it];
    }
    {
      const int v = 16 * (R >> 4) + 4 * ((R >> 2) & 3) + (C >> 4), l = 16 * (R & 3) + c16;
      imgA[(v >> 1) * 128 + 2 * l + (v & 1)] = (double)va[it];
    }
    {
      const int v = 16 * (e >> 10) + (e & 15), l = 16 * ((e >> 4) & 3) + ((e >> 6) & 15);
      imgS[(v >> 2) * 256 + 4 * l + (v & 3)] = vs[it];
    }
  }
  __syncthreads();
  const v2d *iB = reinterpret_cast<const v2d *>(imgB);
  const v2d *iA = reinterpret_cast<const v2d *>(imgA);
  const float4 *iS = reinterpret_cast<const float4 *>(imgS);

  // One token: t0 (in range), its first row block already in xpre when pre
  // is set, stores only when live.
  auto token = [&](int64_t t0, bool pre, bool live) {
    const __half *row = x + t0 * ldx;
    // lane (l16, kg) takes M[16bk + l16][16kg .. 16kg + 15]: two 16-byte loads
    // per row block, the next block's in flight while one is worked (the
    // second pass reads the token again, from L2)
    auto xload = [&](int bk, uint4 *xr) {
      const __half *src = row + 64 * (16 * bk + l16) + 16 * kg;
      xr[0] = *reinterpret_cast<const uint4 *>(src);
      xr[1] = *reinterpret_cast<const uint4 *>(src + 8);
    };
    // Two passes over Y's column blocks, bj = 2h and 2h + 1: Y^T[bj][:]
    // needs only Z's column block bj, so a pass computes those two blocks of
    // Z and folds them into its half of Y^T.  Half the accumulators per pass
    // keep the kernel within 256 registers, two wavefronts per SIMD (one
    // pass over all four held 440 and one wavefront per SIMD).
    float yf[2][2][4][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4d y[2][4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) y[a][b] = v4d{0.0, 0.0, 0.0, 0.0};
      uint4 xc[2], xn[2];
      if (h == 0 && pre) {
        xc[0] = xpre[0];
        xc[1] = xpre[1];
      } else {
        xload(0, xc);
      }
#pragma unroll 1
      for (int bk = 0; bk < 4; ++bk) {
        xload(min(bk + 1, 3), xn);
        // Z row block bk, column blocks 2h, 2h + 1 = M[16bk .. 16bk+15][:] . B,
        // each in two partial sums (even and odd steps t): four independent
        // accumulator chains between the dependent FP64 MFMAs, then one add
        v4d z[2], z2[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) z[c] = z2[c] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int tc = 0; tc < 4; ++tc) {
          const float4 sc = iS[(4 * bk + tc) * 64 + lane];
          const float ss[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * tc + e;
            const v2d bb = iB[(2 * t + h) * 64 + lane];  // B entries of column blocks 2h, 2h + 1
            const uint32_t w = (&xc[t >> 3].x)[(t & 7) >> 1];
            const __half hv = __ushort_as_half((unsigned short)((t & 1) ? (w >> 16) : (w & 0xFFFFu)));
            const double xv = (double)__half2float(hv);
            const double av = DIVIDE ? xv / (double)ss[e] : xv * (double)ss[e];
            if (e & 1) {
              z2[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bb.x, z2[0], 0, 0, 0);
              z2[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bb.y, z2[1], 0, 0, 0);
            } else {
              z[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bb.x, z[0], 0, 0, 0);
              z[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bb.y, z[1], 0, 0, 0);
            }
          }
          // one group of four steps at a time: hoisting the operand reads of
          // all sixteen spilled past 256 registers
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) z[c] += z2[c];
        // Y^T[2h + c][:] += Z_bk[:, 2h + c]^T . A_bk
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 16 * bk + 4 * r;
          const v2d a01 = iA[(v >> 1) * 64 + lane], a23 = iA[((v >> 1) + 1) * 64 + lane];
          const double aa[4] = {a01.x, a01.y, a23.x, a23.y};
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
              y[c][bi] = __builtin_amdgcn_mfma_f64_16x16x4f64(z[c][r], aa[bi], y[c][bi], 0, 0, 0);
        }
        xc[0] = xn[0];
        xc[1] = xn[1];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int r = 0; r < 4; ++r) yf[h][c][bi][r] = (float)y[c][bi][r];
    }
    // per-token symmetric INT4 on the fp32-rounded values
    float amax = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(yf[h][c][bi][r]));
    amax = wave_max(amax);
    float s, inv;
    sym_scale(amax, clip, s, inv);
    if (!live) return;
    int csum = 0;
    // the codes go through the wavefront's LDS row, then out in 16-byte stores
    uint8_t *qs = qst[wave];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          const int bj = 2 * h + c;
          uint32_t bits = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cd = quant_sym(yf[h][c][bi][r], inv, 7.0f);
            csum += cd;
            bits |= (uint32_t)(cd & 0xF) << (4 * r);
          }
          // Y[i][j0 .. j0+3], i = 16bi + l16, j0 = 16bj + 4kg: byte (64 i + j0) / 2
          *reinterpret_cast<uint16_t *>(qs + 32 * (16 * bi + l16) + 8 * bj + 2 * kg) = (uint16_t)bits;
        }
    wave_lds_sync();
    {
      const uint4 *src = reinterpret_cast<const uint4 *>(qs);
      uint4 *dst = reinterpret_cast<uint4 *>(q + t0 * 2048);
      const uint4 c0 = src[lane], c1 = src[64 + lane];
      dst[lane] = c0;
      dst[64 + lane] = c1;
    }
    wave_lds_sync();  // the row is free again for the next token
    if (code_sum) csum = wave_sum(csum);
    if (lane == 0) {
      scale[t0] = s;
      if (code_sum) code_sum[t0] = csum;
    }
  };
  // The first token outside the loop, so that no branch stands between the
  // prefetch above and its use (a guarded use lets the compiler sink the
  // prefetch past the barrier); a wavefront past the last token works on
  // that token and stores nothing.
  const int64_t stride = (int64_t)gridDim.x * kKronWaves;
  const int ntok = tfirst < T ? (int)((T - 1 - tfirst) / stride) + 1 : 1;  // for progress_prio
  progress_prio(0, ntok);
  token(min(tfirst, T - 1), true, tfirst < T);
  int done = 1;
  for (int64_t t0 = tfirst + stride; t0 < T; t0 += stride) {
    progress_prio(done++, ntok);
    token(t0, false, true);
  }
}

hipError_t launch_kron64(const void *x, int64_t T, int64_t ldx, const float *fa, const float *fb,
                         const float *chan_scale, bool divide, float clip, uint8_t *q, float *scale,
                         int32_t *code_sum, hipStream_t st) {
  // one workgroup per CU, one token per wavefront at a time
  const int64_t wgs = (T + kKronWaves - 1) / kKronWaves;
  const dim3 g((unsigned)(wgs < 256 ? wgs : 256)), b(kKronThreads);
  const __half *xh = (const __half *)x;
  if (divide)
    kron64_mfma<true><<<g, b, 0, st>>>(xh, T, ldx, fa, fb, chan_scale, clip, q, scale, code_sum);
  else
    kron64_mfma<false><<<g, b, 0, st>>>(xh, T, ldx, fa, fb, chan_scale, clip, q, scale, code_sum);
  return hipGetLastError();
}

}  // namespace rq
