// clip_search.hip -- QUIK's weight clipping by linear search (QUIK blog,
// "QUIK量化" part 2: before the weights are quantized, a linear search picks
// the clipping threshold).  Per output channel (row of W), every candidate
// ratio c = fp32(k / steps), k = steps, steps - 1, ..., 1, is scored by the
// squared error sum (w - s_c q_c)^2 of symmetric min-max quantization with
// s_c = fp32(c * max|w| / qmax) over the row's normal columns (outlier
// columns keep fp16 and take no part); the first minimum in that order is
// kept, so ties go to the larger ratio.
//
// One workgroup per row (256 threads up to K = 8192, else 1024), grid-stride
// over rows.  Each thread
// keeps its (at most four) 8-column chunks of the row in registers, outlier
// halves zeroed (a zero leaves max|w| and every error term unchanged).  The
// candidates run in batches of four: per value the exact code and the error
// term in fp64, as the scale, code and difference are formed exactly in the
// squared-error definition, then one block reduction of the four sums.
#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {

namespace {

constexpr int kCsChunks = 4;  // 8-column chunks per thread: K <= 8 * 4 * threads
constexpr int kCsBatch = 4;   // candidates per block reduction

// rne(x / s), exactly, for fp16 x (see quant8.hip for the argument)
__device__ __forceinline__ float cs_rne_div(float x, float s, float inv) {
  const float t = x * inv;
  const float c = __builtin_rintf(t);
  const float b = c + __builtin_copysignf(0.5f, t - c);
  const float d = __builtin_fmaf(-b, s, x);
  return __builtin_rintf(b + __builtin_amdgcn_fmed3f(d * 0x1p64f, -0.25f, 0.25f));
}

// The fp32 neighbours lo <= 1/s <= hi; where the two magic-number products
// x*lo and x*hi round to the same integer, it is rne(x / s) (they bracket
// it); elsewhere cs_rne_div decides.
__device__ __forceinline__ void cs_bracket(float s, float inv, float &lo, float &hi) {
  const float e = __builtin_fmaf(-s, inv, 1.0f);
  lo = hi = inv;
  if (e > 0.0f) hi = __uint_as_float(__float_as_uint(inv) + 1u);
  if (e < 0.0f) lo = __uint_as_float(__float_as_uint(inv) - 1u);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

struct CsArgs {
  const __half *w;
  int64_t N, ldw;
  int K, nch;
  const int32_t *oidx;
  int n_out;
  int steps;
  float *clip_out;
};

template <int QMAX, int kCsThreads>
__global__ __launch_bounds__(kCsThreads) void clip_search(CsArgs a) {
  extern __shared__ uint32_t mask[];  // [K / 32] outlier bits
  __shared__ double dred[kCsThreads / 64][kCsBatch];
  __shared__ float fred[kCsThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < a.K / 32; i += kCsThreads) mask[i] = 0u;
  __syncthreads();
  for (int j = tid; j < a.n_out; j += kCsThreads) {
    const int col = a.oidx[j];
    if (col >= 0 && col < a.K) atomicOr(&mask[col >> 5], 1u << (col & 31));
  }
  __syncthreads();
  for (int64_t r = blockIdx.x; r < a.N; r += gridDim.x) {
    const __half *src = a.w + r * a.ldw;
    // the thread's chunks as packed halves, outlier halves zeroed (past the
    // end: all zero)
    uint32_t xp[kCsChunks * 4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kCsChunks; ++i) {
      const int c = tid + kCsThreads * i;
      const uint4 u = *reinterpret_cast<const uint4 *>(src + 8 * min(c, a.nch - 1));
      const uint32_t m = c < a.nch ? (mask[c >> 2] >> (8 * (c & 3))) & 0xFFu : 0xFFu;
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t keep = ((m >> (2 * e)) & 1u ? 0u : 0x0000FFFFu) | ((m >> (2 * e + 1)) & 1u ? 0u : 0xFFFF0000u);
        xp[4 * i + e] = w4[e] & keep;
        const float2 f = __half22float2(*reinterpret_cast<const __half2 *>(&xp[4 * i + e]));
        amax = fmaxf(amax, fmaxf(fabsf(f.x), fabsf(f.y)));
      }
    }
    amax = wave_max(amax);
    if (lane == 0) fred[wave] = amax;
    __syncthreads();
    amax = fred[0];
#pragma unroll
    for (int w = 1; w < kCsThreads / 64; ++w) amax = fmaxf(amax, fred[w]);

    double best = 0.0;
    float best_c = 1.0f;
    bool have = false;
    for (int k0 = a.steps; k0 >= 1; k0 -= kCsBatch) {
      double e[kCsBatch];
      float cb[kCsBatch], sb[kCsBatch], ib[kCsBatch], lb[kCsBatch], hb[kCsBatch];
#pragma unroll
      for (int b = 0; b < kCsBatch; ++b) {
        const int k = max(k0 - b, 1);
        cb[b] = (float)((double)k / (double)a.steps);
        sb[b] = (float)((double)cb[b] * (double)amax / (double)QMAX);
        ib[b] = sb[b] > 0.0f ? 1.0f / sb[b] : 0.0f;
        cs_bracket(sb[b], ib[b], lb[b], hb[b]);
        e[b] = 0.0;
      }
#pragma unroll 2
      for (int j = 0; j < kCsChunks * 4; ++j) {
        const float2 f = __half22float2(*reinterpret_cast<const __half2 *>(&xp[j]));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float xv = h ? f.y : f.x;
#pragma unroll
          for (int b = 0; b < kCsBatch; ++b) {
            const float ma = __builtin_fmaf(xv, lb[b], 12582912.0f), mb = __builtin_fmaf(xv, hb[b], 12582912.0f);
            float r = ma - 12582912.0f;
            if (ma != mb) r = cs_rne_div(xv, sb[b], ib[b]);
            const float q = sb[b] > 0.0f ? __builtin_amdgcn_fmed3f(r, -(float)QMAX, (float)QMAX) : 0.0f;
            const double d = (double)xv - (double)sb[b] * (double)q;
            e[b] = __builtin_fma(d, d, e[b]);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < kCsBatch; ++b) e[b] = wave_sum_f64(e[b]);
      __syncthreads();  // the previous batch's sums are read
      if (lane == 0) {
#pragma unroll
        for (int b = 0; b < kCsBatch; ++b) dred[wave][b] = e[b];
      }
      __syncthreads();
#pragma unroll
      for (int b = 0; b < kCsBatch; ++b) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kCsThreads / 64; ++w) t += dred[w][b];
        if (k0 - b >= 1 && (!have || t < best)) {
          best = t;
          best_c = cb[b];
          have = true;
        }
      }
    }
    if (tid == 0) a.clip_out[r] = best_c;
    __syncthreads();  // fred and dred are free for the next row
  }
}

}  // namespace

hipError_t launch_clip_search(const void *w, int64_t N, int64_t K, int64_t ldw, const int32_t *outlier_idx,
                              int n_out, int bits, int steps, float *clip_out, hipStream_t st) {
  CsArgs a;
  a.w = (const __half *)w;
  a.N = N;
  a.ldw = ldw;
  a.K = (int)K;
  a.nch = (int)(K / 8);
  a.oidx = outlier_idx;
  a.n_out = n_out;
  a.steps = steps;
  a.clip_out = clip_out;
  const size_t lds = (size_t)(K / 32) * 4;
  const bool small = K <= 8 * kCsChunks * 256;  // four chunks per thread at 256 threads
  const dim3 g((unsigned)(N < 4096 ? N : 4096)), b(small ? 256 : 1024);
  if (bits == 8) {
    if (small) clip_search<127, 256><<<g, b, lds, st>>>(a);
    else clip_search<127, 1024><<<g, b, lds, st>>>(a);
  } else {
    if (small) clip_search<7, 256><<<g, b, lds, st>>>(a);
    else clip_search<7, 1024><<<g, b, lds, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace rq
