// quant8.hip -- per-row INT8 quantization of unrotated rows with the QUIK
// outlier split, for the 8-bit down projection (QUIK blog, "QUIK量化" part 3:
// the sensitive down projection is quantized to INT8; experiments, part 1:
// its outlier count grows with the layer's input width; end-to-end speedup:
// more than 600 outliers there).  Activations take per-token asymmetric codes
// in [0, 255] (part 1's form at 8 bits), weights per-channel symmetric codes
// in [-127, 127]; one byte per code.
//
// One workgroup per row, grid-stride over rows.  At start the workgroup turns
// the outlier list into a bit mask, the ascending list of distinct outlier
// columns and, per 8-column chunk, the output offset of its first kept column
// (a block prefix scan), all in LDS.  Per row, each of the 1024 threads loads
// its (at most four) 8-column chunks with 16-byte loads and keeps them for
// both passes: masked fp16 min / max (or |x| max) and the block reduction,
// then codes written byte by byte into an LDS copy of the packed row at their
// compacted positions, and the row stored with 16-byte writes; one thread per
// outlier column copies its value to x_out.  Codes come from two magic-number
// products (recip_bracket below); the exact boundary test runs only where
// they disagree.
#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {

namespace {

constexpr int kQ8Threads = 1024;
constexpr int kQ8MaxChunks = 4;  // 8-column chunks per thread: K <= 32768

// rne(x / s) for s > 0, exactly, whenever |x / s| < 2^22 and x - b s below is
// either 0 or at least 2^-62 in magnitude (true for fp16 x and the scales made
// from fp16 ranges).  c is the integer nearest x * inv, b the half-integer
// between c and its neighbour on the side of x * inv; the sign of x - b s is
// exact in one fma, and zero only at a tie, where rint(b) goes to even.
__device__ __forceinline__ float rne_div(float x, float s, float inv) {
  const float t = x * inv;
  const float c = __builtin_rintf(t);
  const float b = c + __builtin_copysignf(0.5f, t - c);
  const float d = __builtin_fmaf(-b, s, x);
  return __builtin_rintf(b + __builtin_amdgcn_fmed3f(d * 0x1p64f, -0.25f, 0.25f));
}

// The fp32 neighbours lo <= 1/s <= hi (equal when 1/s is exact).  The
// magic-number products x*lo and x*hi, each rounded once to an integer,
// bracket rne(x / s); where they agree that integer is rne(x / s) exactly,
// and only where they differ (x / s within about 2^-23 of a half-integer)
// does rne_div decide.
__device__ __forceinline__ void recip_bracket(float s, float inv, float &lo, float &hi) {
  const float e = __builtin_fmaf(-s, inv, 1.0f);  // sign of 1/s - inv, exact
  lo = hi = inv;
  if (e > 0.0f) hi = __uint_as_float(__float_as_uint(inv) + 1u);
  if (e < 0.0f) lo = __uint_as_float(__float_as_uint(inv) - 1u);
}

// a value every lane of the wavefront holds, into a scalar register
__device__ __forceinline__ float q8_uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

constexpr float kQ8Magic = 12582912.0f;  // 1.5 * 2^23: fma(x, r, kQ8Magic) - kQ8Magic = rne(x * r)

__device__ __forceinline__ float block_reduce(float v, float *red, bool is_max) {
  v = is_max ? wave_max(v) : wave_min(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kQ8Threads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : fminf(r, red[w]);
  return r;
}

struct Q8Args {
  const __half *x;
  int64_t T, ldx;
  int K, nch;              // columns, 8-column chunks (K / 8)
  int kint;                // K - n_out: codes per row
  float clip;
  const float *row_clip;   // per-row clip ratios (symmetric), or null
  const int32_t *oidx;
  int n_out;
  uint8_t *q;              // [T, kint]
  float *scale;
  int32_t *zero;           // asymmetric only
  int32_t *code_sum;       // or null
  __half *x_out;           // [T, n_out] or null
};

template <bool ASYM, bool CSUM>
__global__ __launch_bounds__(kQ8Threads) __attribute__((amdgpu_waves_per_eu(8, 8))) void split_quant8(Q8Args a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t *mask = reinterpret_cast<uint32_t *>(smem);           // [K / 32] outlier bits
  int32_t *cbase = reinterpret_cast<int32_t *>(smem + a.K / 8);  // [K / 8] first kept position per chunk
  uint8_t *row = smem + ((a.K / 8 + a.K / 2 + 15) & ~15);       // [K + 16] bytes: the packed row, a spare slot
  uint16_t *ocol = reinterpret_cast<uint16_t *>(row + a.K + 16);  // [n_out] outlier columns, ascending
  __shared__ float red[2][kQ8Threads / 64];
  __shared__ int ired[kQ8Threads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- outlier mask, then per chunk the output offset of its first kept column
  for (int i = tid; i < a.K / 32; i += kQ8Threads) mask[i] = 0u;
  __syncthreads();
  for (int j = tid; j < a.n_out; j += kQ8Threads) {
    const int col = a.oidx[j];
    if (col >= 0 && col < a.K) atomicOr(&mask[col >> 5], 1u << (col & 31));
  }
  __syncthreads();
  auto cmask = [&](int c) { return (mask[c >> 2] >> (8 * (c & 3))) & 0xFFu; };
  // block exclusive scan of the kept counts over contiguous chunk ranges
  const int cpt = (a.nch + kQ8Threads - 1) / kQ8Threads;
  int kept = 0;
  for (int i = 0; i < cpt; ++i) {
    const int c = tid * cpt + i;
    if (c < a.nch) kept += 8 - __builtin_popcount(cmask(c));
  }
  const int incl = wave_scan_dpp(kept);  // inclusive prefix within the wave
  if (lane == 63) ired[wave] = incl;
  __syncthreads();
  int base = incl - kept;
  for (int w = 0; w < wave; ++w) base += ired[w];
  for (int i = 0; i < cpt; ++i) {
    const int c = tid * cpt + i;
    if (c < a.nch) {
      const uint32_t m = cmask(c);
      cbase[c] = base;
      // the chunk's outliers take ranks 8c - base, 8c - base + 1, ...
      int orank = 8 * c - base;
      for (uint32_t mm = m; mm; mm &= mm - 1u, ++orank)
        if (orank < a.n_out) ocol[orank] = (uint16_t)(8 * c + __builtin_ctz(mm));
      base += 8 - __builtin_popcount(m);
    }
  }
  // distinct outlier columns (duplicates in the list count once)
  int kept_total = 0;
#pragma unroll
  for (int w = 0; w < kQ8Threads / 64; ++w) kept_total += ired[w];
  const int nset = min(a.n_out, a.K - kept_total);
  __syncthreads();

  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const int nrows = (int)((a.T - 1 - blockIdx.x) / gridDim.x) + 1;  // for progress_prio
  int done = 0;
  for (int64_t r = blockIdx.x; r < a.T; r += gridDim.x) {
    progress_prio(done++, nrows);
    const __half *src = a.x + r * a.ldx;
    // the thread's chunks tid + 1024 i, loaded once (past the end: a clamped
    // reload, never used)
    uint4 v[kQ8MaxChunks];
#pragma unroll
    for (int i = 0; i < kQ8MaxChunks; ++i)
      v[i] = load_nt(src + 8 * min(tid + kQ8Threads * i, a.nch - 1));
    // the thread's first outlier column (rank tid in ascending order) is read
    // with the row, an L2 hit once the row is in; column 0 stands in past
    // the list
    const uint16_t og = reinterpret_cast<const uint16_t *>(src)[tid < nset ? ocol[tid] : 0];
    // pass 1: masked min / max of the kept columns (outliers count as 0,
    // which the range [min(x, 0), max(x, 0)] already contains), or |x| max
    h2 mn2 = {0, 0}, mx2 = {0, 0};
#pragma unroll
    for (int i = 0; i < kQ8MaxChunks; ++i) {
      const int c = tid + kQ8Threads * i;
      if (c >= a.nch) continue;
      const uint32_t m = cmask(c);
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // bits 2e, 2e + 1 of m, each sign-extended to a full mask, select the
        // halves that are zeroed
        const uint32_t olo = (uint32_t)((int32_t)(m << (31 - 2 * e)) >> 31);
        const uint32_t ohi = (uint32_t)((int32_t)(m << (30 - 2 * e)) >> 31);
        const uint32_t d = w[e] & ~((olo & 0x0000FFFFu) | (ohi & 0xFFFF0000u));
        h2 h;
        __builtin_memcpy(&h, &d, 4);
        if (!ASYM) h = __builtin_elementwise_abs(h);
        mn2 = __builtin_elementwise_min(mn2, h);
        mx2 = __builtin_elementwise_max(mx2, h);
      }
    }
    float s, inv, zf = 0.0f, lo_c, hi_c;
    if (ASYM) {
      const float mn = block_reduce(fminf((float)mn2[0], (float)mn2[1]), red[0], false);
      const float mx = block_reduce(fmaxf((float)mx2[0], (float)mx2[1]), red[1], true);
      const float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
      // the scale is the exact quotient rounded once to fp32: hi - lo formed
      // exactly in fp64 (fp16 bounds span at most 40 bits; in fp32 the
      // difference rounds when max / |min| exceeds about 2^12), the quotient
      // rounded to fp64 and converted, as a single rounding would be except
      // where the fp64 quotient itself falls on an fp32 midpoint
      s = (float)(((double)hi - (double)lo) / 255.0);
      inv = s > 0.0f ? 1.0f / s : 0.0f;
      if (s > 0.0f) zf = __builtin_amdgcn_fmed3f(rne_div(-lo, s, inv), 0.0f, 255.0f);
      lo_c = 0.0f;
      hi_c = 255.0f;
    } else {
      const float mx = block_reduce(fmaxf((float)mx2[0], (float)mx2[1]), red[1], true);
      const float clip = a.row_clip ? a.row_clip[r] : a.clip;
      s = (float)((double)clip * (double)mx / 127.0);  // the product is exact in fp64
      inv = s > 0.0f ? 1.0f / s : 0.0f;
      lo_c = -127.0f;
      hi_c = 127.0f;
    }
    // pass 2: codes into the LDS row at their compacted positions.  Per
    // value: the two bracket products; where every lane of the wavefront
    // agrees on all eight (all but about 1e-5 of values), the product is the
    // code; else the lanes with a disagreement take the exact test.  The code
    // plus zero point is clamped in the magic-number domain, kQ8Magic + code,
    // whose low byte is the code byte (two's complement for negative
    // symmetric codes), so the float bits go to the LDS row as they are.
    // Outlier positions write their byte to a spare slot past the row
    // instead of branching.  A zero scale needs no select: rlo = rhi = 0 and
    // zf = 0 give code 0.
    float rlo = 0.0f, rhi = 0.0f;
    if (s > 0.0f) recip_bracket(s, inv, rlo, rhi);
    // the row's constants are the same in every lane: scalar registers
    s = q8_uniform(s);
    inv = q8_uniform(inv);
    zf = q8_uniform(zf);
    rlo = q8_uniform(rlo);
    rhi = q8_uniform(rhi);
    const float clo = kQ8Magic + lo_c, chi = kQ8Magic + hi_c;
    auto code_bits = [&](float f) {
      float cv = __builtin_fmaf(f, rlo, kQ8Magic);
      if (cv != __builtin_fmaf(f, rhi, kQ8Magic)) cv = rne_div(f, s, inv) + kQ8Magic;
      return __float_as_uint(__builtin_amdgcn_fmed3f(cv + zf, clo, chi));
    };
    // the outliers, one thread per column in ascending order (the row is in
    // L2 by now): fp16 bits to x_out, and their codes, which the chunks'
    // code sums below include, for the code sum's correction
    int csum = 0;
    for (int j = tid; j < nset; j += kQ8Threads) {
      const uint16_t bits = j == tid ? og : reinterpret_cast<const uint16_t *>(src)[ocol[j]];
      reinterpret_cast<uint16_t *>(a.x_out)[r * a.n_out + j] = bits;
      if (CSUM) {
        const uint32_t cb = code_bits(__half2float(__ushort_as_half(bits))) & 0xFFu;
        csum -= ASYM ? (int)cb : (int)(int8_t)cb;
      }
    }
    const int spare = a.K;
#pragma unroll
    for (int i = 0; i < kQ8MaxChunks; ++i) {
      const int c = tid + kQ8Threads * i;
      if (c >= a.nch) continue;
      const uint32_t m = cmask(c);
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      auto val = [&](int e) {
        const float2 f2 = __half22float2(*reinterpret_cast<const __half2 *>(&w[e >> 1]));
        return (e & 1) ? f2.y : f2.x;
      };
      float cv[8];
      bool split = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cv[e] = __builtin_fmaf(val(e), rlo, kQ8Magic);
        split |= cv[e] != __builtin_fmaf(val(e), rhi, kQ8Magic);
      }
      if (__builtin_amdgcn_ballot_w64(split) != 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (cv[e] != __builtin_fmaf(val(e), rhi, kQ8Magic)) cv[e] = rne_div(val(e), s, inv) + kQ8Magic;
      }
      // value e's byte goes to row[kpos + e - nout] (nout: outliers left of
      // it), an outlier's to the spare slot
      const int kpos = cbase[c];
      int nout = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t b = __float_as_uint(__builtin_amdgcn_fmed3f(cv[e] + zf, clo, chi));
        const int out = (int)((m >> e) & 1u);
        row[out ? spare : kpos + e - nout] = (uint8_t)b;
        nout += out;
        // every column's code enters the sum; the outliers' leave it above
        if (CSUM) csum += ASYM ? (int)(b & 0xFFu) : (int)(int8_t)(b & 0xFFu);
      }
    }
    if (CSUM) {
      const int cs = wave_sum(csum);
      if (lane == 0) ired[wave] = cs;
      __syncthreads();
      if (tid == 0) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < kQ8Threads / 64; ++w) t += ired[w];
        a.code_sum[r] = t;
      }
    }
    if (tid == 0) {
      a.scale[r] = s;
      if (ASYM) a.zero[r] = (int)zf;
    }
    __syncthreads();
    uint8_t *dst = a.q + r * (int64_t)a.kint;
    for (int o = 16 * tid; o < a.kint; o += 16 * kQ8Threads)
      store_nt(dst + o, *reinterpret_cast<const uint4 *>(row + o));
    __syncthreads();
  }
}

}  // namespace

// mask, chunk offsets, the packed row with 16 spare bytes (the slot that
// outlier positions write to), then the outlier columns in ascending order
size_t split8_smem_bytes(int64_t K, int n_out) {
  return (((size_t)(K / 8) + (size_t)(K / 2) + 15) & ~(size_t)15) + (size_t)K + 16 + 2 * (size_t)n_out;
}

hipError_t launch_split8(const void *x, int64_t T, int64_t K, int64_t ldx, bool asym, float clip,
                         const float *row_clip, const int32_t *outlier_idx, int n_out, uint8_t *q,
                         float *scale, int32_t *zero, int32_t *code_sum, void *x_out, hipStream_t st) {
  Q8Args a;
  a.x = (const __half *)x;
  a.T = T;
  a.ldx = ldx;
  a.K = (int)K;
  a.nch = (int)(K / 8);
  a.kint = (int)(K - n_out);
  a.clip = clip;
  a.row_clip = row_clip;
  a.oidx = outlier_idx;
  a.n_out = n_out;
  a.q = q;
  a.scale = scale;
  a.zero = zero;
  a.code_sum = code_sum;
  a.x_out = (__half *)x_out;
  const size_t lds = split8_smem_bytes(K, n_out);
  const dim3 g((unsigned)(T < 1024 ? T : 1024)), b(kQ8Threads);
  void (*k)(Q8Args) = asym ? (code_sum ? split_quant8<true, true> : split_quant8<true, false>)
                            : (code_sum ? split_quant8<false, true> : split_quant8<false, false>);
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k<<<g, b, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace rq
