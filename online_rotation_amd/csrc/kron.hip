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
// Z is produced one row block (16 rows) at a time and folded into all of
// Y^T at once, so only four Z blocks are live next to Y^T's sixteen.
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
}  // namespace

template <bool DIVIDE>
__global__ __launch_bounds__(256) void kron64_mfma(const __half *__restrict__ x, int64_t T, int64_t ldx,
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, l16 = lane & 15;
  // all 48 loads of a thread first, then the LDS writes, so the loads are in
  // flight together
  constexpr int kIt = kImg / 256;
  float vb[kIt], va[kIt], vs[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int e = it * 256 + tid;
    const int v = e >> 6, l = e & 63;  // register v of lane l
    const int lk = l >> 4, li = l & 15;
    vb[it] = fb[(16 * lk + (v >> 2)) * 64 + 16 * (v & 3) + 4 * (li & 3) + (li >> 2)];
    va[it] = fa[(16 * (v >> 4) + 4 * ((v >> 2) & 3) + lk) * 64 + 16 * (v & 3) + li];
    vs[it] = chan_scale ? chan_scale[64 * (16 * (v >> 4) + li) + 16 * lk + (v & 15)] : 1.0f;
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int e = it * 256 + tid;
    const int v = e >> 6, l = e & 63;
    imgB[(v >> 1) * 128 + 2 * l + (v & 1)] = (double)vb[it];  // B[16kg + t][16bj + pi(i)], v = 4t + bj
    imgA[(v >> 1) * 128 + 2 * l + (v & 1)] = (double)va[it];  // A[16bk + 4r + kg][16bi + i], v = 16bk + 4r + bi
    imgS[(v >> 2) * 256 + 4 * l + (v & 3)] = vs[it];          // s[64(16bk + i) + 16kg + t], v = 16bk + t
  }
  __syncthreads();
  const v2d *iB = reinterpret_cast<const v2d *>(imgB);
  const v2d *iA = reinterpret_cast<const v2d *>(imgA);
  const float4 *iS = reinterpret_cast<const float4 *>(imgS);

  for (int64_t t0 = (int64_t)blockIdx.x * 4 + wave; t0 < T; t0 += (int64_t)gridDim.x * 4) {
    const __half *row = x + t0 * ldx;
    // lane (l16, kg): M[16bi + l16][16kg .. 16kg + 15] for bi = 0..3
    // lane (l16, kg) needs M[16bk + l16][16kg .. 16kg + 15]: two 16-byte loads per row block
    auto xload = [&](int bk, uint4 *xr) {
      const __half *src = row + 64 * (16 * bk + l16) + 16 * kg;
      xr[0] = *reinterpret_cast<const uint4 *>(src);
      xr[1] = *reinterpret_cast<const uint4 *>(src + 8);
    };
    uint4 xc[2], xn[2];
    xload(0, xc);
    // Y^T block [bj][bi] accumulates over Z's row blocks bk as each is finished
    v4d y[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) y[a][b] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
    for (int bk = 0; bk < 4; ++bk) {
      xload(min(bk + 1, 3), xn);
      // Z row block bk = M[16bk .. 16bk+15][:] . B, column blocks bj
      v4d z[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) z[bj] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int tc = 0; tc < 4; ++tc) {
        const float4 sc = iS[(4 * bk + tc) * 64 + lane];
        const float ss[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * tc + e;
          const v2d b01 = iB[(2 * t) * 64 + lane], b23 = iB[(2 * t + 1) * 64 + lane];
          const double bb[4] = {b01.x, b01.y, b23.x, b23.y};
          const uint32_t w = (&xc[t >> 3].x)[(t & 7) >> 1];
          const __half hv = __ushort_as_half((unsigned short)((t & 1) ? (w >> 16) : (w & 0xFFFFu)));
          const double xv = (double)__half2float(hv);
          const double a = DIVIDE ? xv / (double)ss[e] : xv * (double)ss[e];
#pragma unroll
          for (int bj = 0; bj < 4; ++bj)
            z[bj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb[bj], z[bj], 0, 0, 0);
        }
      }
      // Y^T += Z_bk^T . A_bk
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 16 * bk + 4 * r;
        const v2d a01 = iA[(v >> 1) * 64 + lane], a23 = iA[((v >> 1) + 1) * 64 + lane];
        const double aa[4] = {a01.x, a01.y, a23.x, a23.y};
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
          for (int bi = 0; bi < 4; ++bi)
            y[bj][bi] = __builtin_amdgcn_mfma_f64_16x16x4f64(z[bj][r], aa[bi], y[bj][bi], 0, 0, 0);
      }
      xc[0] = xn[0];
      xc[1] = xn[1];
    }
    // per-token symmetric INT4 on the fp32-rounded values
    float yf[4][4][4];
    float amax = 0.0f;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          yf[bj][bi][r] = (float)y[bj][bi][r];
          amax = fmaxf(amax, fabsf(yf[bj][bi][r]));
        }
    amax = wave_max(amax);
    float s, inv;
    sym_scale(amax, clip, s, inv);
    int csum = 0;
    uint8_t *qrow = q + t0 * 2048;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        uint32_t bits = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = quant_sym(yf[bj][bi][r], inv, 7.0f);
          csum += c;
          bits |= (uint32_t)(c & 0xF) << (4 * r);
        }
        // Y[i][j0 .. j0+3], i = 16bi + l16, j0 = 16bj + 4kg: byte (64 i + j0) / 2
        *reinterpret_cast<uint16_t *>(qrow + 32 * (16 * bi + l16) + 8 * bj + 2 * kg) = (uint16_t)bits;
      }
    if (code_sum) csum = wave_sum(csum);
    if (lane == 0) {
      scale[t0] = s;
      if (code_sum) code_sum[t0] = csum;
    }
  }
}

hipError_t launch_kron64(const void *x, int64_t T, int64_t ldx, const float *fa, const float *fb,
                         const float *chan_scale, bool divide, float clip, uint8_t *q, float *scale,
                         int32_t *code_sum, hipStream_t st) {
  const int64_t wgs = (T + 3) / 4;
  const dim3 g((unsigned)(wgs < 256 ? wgs : 256)), b(256);
  const __half *xh = (const __half *)x;
  if (divide)
    kron64_mfma<true><<<g, b, 0, st>>>(xh, T, ldx, fa, fb, chan_scale, clip, q, scale, code_sum);
  else
    kron64_mfma<false><<<g, b, 0, st>>>(xh, T, ldx, fa, fb, chan_scale, clip, q, scale, code_sum);
  return hipGetLastError();
}

}  // namespace rq
