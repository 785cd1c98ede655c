// rotate_quant.hip -- online transform + per-token INT4 quantization (gfx950).
//
// Kernels:
//   fwht4096_quant   one wavefront per 4096-wide row: Walsh-Hadamard
//                    butterflies ("QuaRot & SpinQuant" blog, section 2) over
//                    the full row or within sequency-ordered Walsh blocks
//                    ("Grouped Sequency-arranged Rotation" abstract), min-max
//                    symmetric INT4 (SpinQuant OpenReview, Q1/A1), packing.
//   rowlds_quant     one workgroup per row, the row staged in LDS: any
//                    power-of-two Hadamard / GSR span, the identity with
//                    QUIK's fp16 outlier split and asymmetric per-token codes
//                    (QUIK blog, "QUIK quantization" parts 1 and 3).
//   kron_quant       FlatQuant's Kronecker affine transform with channel
//                    scaling and clipping (FlatQuant article, section 2.3).
//   kron_inverse_t   fp64 Gauss-Jordan inverse-transpose of a Kronecker
//                    factor, for the weight side of the affine transform.
#include "fwht_common.h"
#include "rq_device.h"
#include "rq_kernels.h"
#include "split_common.h"

namespace rq {

// ---------------------------------------------------------------------------
// fwht4096_quant
//
// Index bits of a 4096-element row are split between the 64 lanes and the 64
// registers of each lane.  Loads are coalesced (lane l, vector v holds
// elements v*512 + l*8 + e), so registers first cover bits {0,1,2,9,10,11};
// one LDS transpose moves bits {3..8} into registers for the remaining
// butterflies, a second transpose brings the row back to the load layout for
// quantization and contiguous packed stores.
//
// LDS word address of element i: bit 2 is flipped by bit 5 and every 512
// elements are padded by 8 words, which makes the 128-bit row accesses and
// the 32-bit transposed accesses free of bank conflicts.
// ---------------------------------------------------------------------------
constexpr int kF4096Waves = 4;
constexpr int kF4096Words = 4096 + 8 * 8;

__device__ __forceinline__ int f4096_addr(int i) {
  return (i ^ (((i >> 5) & 1) << 2)) + ((i >> 9) << 3);
}

// Butterfly along register-index bit `rb` of a[64].
template <int RB>
__device__ __forceinline__ void reg_stage(float *a) {
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (i & (1 << RB)) continue;
    const float u = a[i], w = a[i | (1 << RB)];
    a[i] = u + w;
    a[i | (1 << RB)] = u - w;
  }
}

__device__ __forceinline__ int bitrev(int v, int bits) {
  return (int)(__builtin_bitreverse32((uint32_t)v) >> (32 - bits));
}

template <bool GSR>
__global__ __launch_bounds__(256) void fwht4096_quant(const __half *__restrict__ x, int64_t T,
                                                      int64_t ldx, uint8_t *__restrict__ q,
                                                      float *__restrict__ scale,
                                                      int32_t *__restrict__ code_sum, float clip,
                                                      int span_log2, float norm) {
  __shared__ __align__(16) float lds[kF4096Waves][kF4096Words];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kF4096Waves + wave;
  if (t >= T) return;  // whole wavefront leaves; no workgroup barrier below
  float *L = lds[wave];
  const __half *row = x + t * ldx;

  float a[64];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(row + v * 512 + lane * 8);
    h8_to_f32(raw, a + v * 8);
  }
  // phase 1: idx bits 0,1,2 (register bits 0..2) and 9,10,11 (register bits 3..5)
  if (span_log2 > 0) reg_stage<0>(a);
  if (span_log2 > 1) reg_stage<1>(a);
  if (span_log2 > 2) reg_stage<2>(a);
  if (span_log2 > 9) reg_stage<3>(a);
  if (span_log2 > 10) reg_stage<4>(a);
  if (span_log2 > 11) reg_stage<5>(a);
#pragma unroll
  for (int v = 0; v < 8; ++v) {
#pragma unroll
    for (int e0 = 0; e0 < 8; e0 += 4) {
      const int i = v * 512 + lane * 8 + e0;
      *reinterpret_cast<float4 *>(L + f4096_addr(i)) =
          make_float4(a[v * 8 + e0], a[v * 8 + e0 + 1], a[v * 8 + e0 + 2], a[v * 8 + e0 + 3]);
    }
  }
  wave_lds_sync();
  // phase 2: idx bits 3..8 in registers; lane holds bits {0,1,2} and {9,10,11}
  const int base2 = ((lane >> 3) << 9) | (lane & 7);
#pragma unroll
  for (int r = 0; r < 64; ++r) a[r] = L[f4096_addr(base2 | (r << 3))];
  if (span_log2 > 3) reg_stage<0>(a);
  if (span_log2 > 4) reg_stage<1>(a);
  if (span_log2 > 5) reg_stage<2>(a);
  if (span_log2 > 6) reg_stage<3>(a);
  if (span_log2 > 7) reg_stage<4>(a);
  if (span_log2 > 8) reg_stage<5>(a);
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    a[r] *= norm;
    amax = fmaxf(amax, fabsf(a[r]));
  }
#pragma unroll
  for (int r = 0; r < 64; ++r) L[f4096_addr(base2 | (r << 3))] = a[r];
  amax = wave_max(amax);
  float s, inv;
  sym_scale(amax, clip, s, inv);
  wave_lds_sync();
  // phase 3: back to the load layout (output position j = v*512 + lane*8 + e)
  if (!GSR) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
#pragma unroll
      for (int e0 = 0; e0 < 8; e0 += 4) {
        const float4 f = *reinterpret_cast<const float4 *>(L + f4096_addr(v * 512 + lane * 8 + e0));
        a[v * 8 + e0] = f.x;
        a[v * 8 + e0 + 1] = f.y;
        a[v * 8 + e0 + 2] = f.z;
        a[v * 8 + e0 + 3] = f.w;
      }
    }
  } else {
    // x . Wal_b: the sequency-ordered Walsh block is symmetric and equals the
    // Hadamard block with rows permuted by sigma(s) = bitrev(gray(s)), so
    // output j of a block reads butterfly result sigma(j).
    const int bmask = (1 << span_log2) - 1;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = v * 512 + lane * 8 + e;
        const int s_ = j & bmask;
        const int nat = (j & ~bmask) | bitrev(s_ ^ (s_ >> 1), span_log2);
        a[v * 8 + e] = L[f4096_addr(nat)];
      }
    }
  }
  uint8_t *qrow = q + t * 2048;
  int csum = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    int c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      c[e] = quant_sym(a[v * 8 + e], inv, 7.0f);
      csum += c[e];
    }
    *reinterpret_cast<uint32_t *>(qrow + v * 256 + lane * 4) = pack8(c);
  }
  if (code_sum) csum = wave_sum(csum);
  if (lane == 0) {
    scale[t] = s;
    if (code_sum) code_sum[t] = csum;
  }
}

// ---------------------------------------------------------------------------
// fwht4096_mfma: the same transforms on FP16 matrix cores (fwht_common.h).
// ---------------------------------------------------------------------------
// CLAMP: clip ratio below 1.  At clip 1, |x'| <= amax gives |x' / s| <= 7
// (1 + 2^-22) and the rounded code never leaves [-7, 7], so the clamp is
// dropped; non-finite inputs then leave byte-clean NaN patterns (nibble 0).
template <bool GSR, bool CSUM, bool CLAMP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwht4096_mfma(const __half *__restrict__ x, int64_t T,
                                                     int64_t ldx, uint8_t *__restrict__ q,
                                                     float *__restrict__ scale,
                                                     int32_t *__restrict__ code_sum, float clip,
                                                     int blog2, float norm, int tpw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r32 = lane & 31, g = lane >> 5;
  const int64_t nw = (int64_t)gridDim.x * 4;  // wavefronts in the grid
  const int64_t t0 = (int64_t)blockIdx.x * 4 + wave;

  // Constant operands, staged in LDS once per workgroup: read through
  // lgkmcnt, waiting for them never waits for a token prefetch in flight.
  __shared__ uint4 ltab[GSR ? 8 : 16][64];

  // Each token is read once and its codes written once: both go through
  // nontemporal accesses (measured 13% faster than cached ones on a plain
  // read-8-KB / write-2-KB stream at 2048 tokens).
  // The token goes global -> registers with coalesced 16-byte loads (lane l
  // of load c takes bytes 1024c + 16l: row a = 8c + l/8 of the 64 x 64
  // reshape, 16-byte column l % 8), then through a per-wave LDS stage into
  // the MFMA layout M[a = r32 + 32*rb][b = 16*kc + 8*g + s], s = 0..7, one
  // half (32 rows, loads 4rb .. 4rb + 3) at a time.  Read straight in that
  // layout, each load instruction touched 32 rows 128 bytes apart.  In the
  // stage, column j of row a sits at j ^ ((a >> 1) & 7), so that both the
  // row-wise writes and the 16-lane column reads hit distinct banks.
  __shared__ v4w stage[4][32 * 8];
  auto load = [&](v4w (&raw)[8], int64_t t) {
    const v4w *row = reinterpret_cast<const v4w *>(x + t * ldx);
#pragma unroll
    for (int c = 0; c < 8; ++c) raw[c] = __builtin_nontemporal_load(&row[64 * c + lane]);
  };

  // transform, scale, quantize and (for a wavefront inside the grid's
  // tokens) store token t
  const bool live = t0 < T;
  auto body = [&](const v4w (&raw)[8], int64_t t) {
    const FwhtOut o = fwht_token<GSR, CSUM, CLAMP>(raw, stage[wave], ltab, norm, clip);
    if (!live) return;
    uint8_t *qrow = q + t * 2048;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      __builtin_nontemporal_store(o.code[nb], reinterpret_cast<v4w *>(qrow + 32 * (r32 + 32 * nb) + 16 * g));
    if (lane == 0) {
      if (CSUM) code_sum[t] = o.csum;
      scale[t] = o.s;
    }
  };

  // Tokens t0 + i*nw for i < tpw, tpw being 1 or even.  With P even the next
  // token's loads are in flight while the current one is computed; indices
  // past the end are clamped onto the last row (same inputs, same outputs),
  // so the loop holds no branch.
  // The wavefront's first token is requested first; the operand tables are
  // then computed into LDS (no memory access) and the workgroup meets, so
  // the token's latency runs under the set-up.  A wavefront past the last
  // token works on that token (a clamped index) and stores nothing; with no
  // early exit here the compiler keeps the token's loads ahead of the
  // barrier.
  v4w b0[8], b1[8];
  load(b0, min(t0, T - 1));
  __builtin_amdgcn_sched_barrier(0);
  fwht_make_tables<GSR>(ltab, blog2, threadIdx.x, 256);
  __syncthreads();
  if (tpw == 1) {
    body(b0, min(t0, T - 1));
    return;
  }
  for (int i = 0; i < tpw; i += 2) {
    progress_prio(i, tpw);
    const int64_t ta = min(t0 + i * nw, T - 1), tb = min(t0 + (i + 1) * nw, T - 1),
                  tc = min(t0 + (i + 2) * nw, T - 1);
    load(b1, tb);
    __builtin_amdgcn_sched_barrier(0);
    body(b0, ta);
    __builtin_amdgcn_sched_barrier(0);
    load(b0, tc);
    __builtin_amdgcn_sched_barrier(0);
    body(b1, tb);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// split_quant: no rotation (QUIK), K % 32 == 0, K <= 32768.  Thread t of a
// 256-thread workgroup owns the WPT words of 32 columns that start at column
// 32 WPT t, in every row the workgroup quantizes.
// Once per workgroup: a bit mask of the outlier columns, each word's
// exclusive prefix count (a block scan) and, per word, AND masks that zero
// its outlier halves.  Zeroed outliers leave min(min x, 0), max(max x, 0) and
// the absolute maximum unchanged, so the row reductions test no value.  Per
// row each thread quantizes its values (one fma against a magic number
// shifted by the zero point, one clamp), deletes the outlier nibbles from
// each word's 128-bit code run and ORs the run into a packed row in LDS at
// its compacted nibble offset; the packed row then goes out with coalesced
// stores.
//
// Codes, rounding and the word-level compaction: split_common.h.
// ---------------------------------------------------------------------------
constexpr int kSplitThreads = 256;

template <int WPT>
__global__ __launch_bounds__(kSplitThreads) void split_quant(
    const __half *__restrict__ x, int64_t T, int K, int64_t ldx, int asym, float clip,
    const float *__restrict__ row_clip, const int32_t *__restrict__ outlier_idx, int n_out,
    uint8_t *__restrict__ q, float *__restrict__ scale, int32_t *__restrict__ zero,
    int32_t *__restrict__ code_sum, __half *__restrict__ x_out) {
  constexpr int NW = kSplitThreads * WPT;
  __shared__ uint32_t mask[NW];
  __shared__ int wsum[4];
  __shared__ uint32_t packed[NW * 4 + 1];  // packed codes of one row (+1 spill word)
  __shared__ float redf[8];
  __shared__ int redi[4];
  extern __shared__ uint16_t ocol[];  // [n_out] outlier columns, ascending
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = K / 32;
  const int Kn = K - n_out;

  // A row's 16-byte chunks; inactive words reload the thread's last active
  // word (their keep masks are zero), so the loads hold no branch.  Cached
  // loads: the outlier gather below re-reads the row from L2 (with
  // nontemporal loads it went to HBM and the kernel ran 30% slower).
  auto load_row = [&](uint4 (&u)[WPT][4], int64_t t) {
    const __half *row = x + t * ldx;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const __half *src = row + 32 * min(tid * WPT + j, nw - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) u[j][i] = *reinterpret_cast<const uint4 *>(src + 8 * i);
    }
  };
  // The outlier list's first entries and then the workgroup's first row are
  // requested before the set-up below, so that the row's memory latency runs
  // under it: loads complete in order, so the set-up waits for the list
  // without waiting for the row.  The grid has at most T workgroups, so the
  // row exists; the row loop runs at least once, which keeps the compiler
  // from sinking these loads past the set-up's barriers.
  const int oid0 = tid < n_out ? outlier_idx[tid] : -1;
  __builtin_amdgcn_sched_barrier(0);
  uint4 cur[WPT][4];
  load_row(cur, blockIdx.x);
  __builtin_amdgcn_sched_barrier(0);

  // ---- per-workgroup setup
  for (int i = tid; i < NW; i += kSplitThreads) mask[i] = 0u;
  __syncthreads();
  if (oid0 >= 0 && oid0 < K) atomicOr(&mask[oid0 >> 5], 1u << (oid0 & 31));
  for (int j = tid + kSplitThreads; j < n_out; j += kSplitThreads) {
    const int c = outlier_idx[j];
    if (c >= 0 && c < K) atomicOr(&mask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  uint32_t m[WPT];
  bool active[WPT];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    active[j] = tid * WPT + j < nw;
    m[j] = mask[tid * WPT + j];
    cnt += __popc(m[j]);
  }
  // exclusive prefix of cnt over threads (wave scan + 4 wave totals)
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before[WPT];  // outlier columns left of each word
  before[0] = incl - cnt;
  for (int w = 0; w < wave; ++w) before[0] += wsum[w];
#pragma unroll
  for (int j = 1; j < WPT; ++j) before[j] = before[j - 1] + __popc(m[j - 1]);
  uint32_t keep[WPT][16];  // AND masks zeroing each word's outlier halves
#pragma unroll
  for (int j = 0; j < WPT; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      keep[j][i] = (((m[j] >> (2 * i)) & 1u) ? 0u : 0x0000FFFFu) |
                   (((m[j] >> (2 * i + 1)) & 1u) ? 0u : 0xFFFF0000u);
#pragma unroll
  for (int j = 0; j < WPT; ++j)
    if (!active[j])
#pragma unroll
      for (int i = 0; i < 16; ++i) keep[j][i] = 0u;
  // the outlier columns in ascending order (rank = before + position in word)
  const int nset = min(wsum[0] + wsum[1] + wsum[2] + wsum[3], n_out);
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    uint32_t mo = m[j];
    for (int r = before[j]; mo; ++r, mo &= mo - 1)
      if (r < n_out) ocol[r] = (uint16_t)(32 * (tid * WPT + j) + __ffs(mo) - 1);
  }
  const int nwords = (Kn + 7) / 8;  // packed row words
  for (int i = tid; i < NW * 4 + 1; i += kSplitThreads) packed[i] = 0u;
  __syncthreads();

  // outlier values per thread gathered ahead of the codes: columns ogc
  // (past the list, or with none: column 0, loaded but not stored)
  constexpr int kOg = 4;
  int ogc[kOg];
#pragma unroll
  for (int k = 0; k < kOg; ++k) ogc[k] = nset > 0 ? ocol[min(tid + kSplitThreads * k, nset - 1)] : 0;
  uint4 nxt[WPT][4];
  int64_t t = blockIdx.x;
  // rows of this workgroup, for the issue priority (progress_prio)
  const int nrows = (int)((T - 1 - blockIdx.x) / gridDim.x) + 1;
  int done = 0;
  do {
    progress_prio(done++, nrows);
    const __half *row = x + t * ldx;
    // this row's first kOg * 256 outlier values (L2-resident by now), issued
    // before the next row's loads so that waiting for them leaves those in flight
    unsigned short og[kOg];
#pragma unroll
    for (int k = 0; k < kOg; ++k) og[k] = reinterpret_cast<const unsigned short *>(row)[ogc[k]];
    __builtin_amdgcn_sched_barrier(0);
    // the next row; the last one reloads this row (L2-resident) rather than
    // branch, since a conditional load makes the compiler wait for it below
    const int64_t tn = t + gridDim.x;
    load_row(nxt, tn < T ? tn : t);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t d[WPT][16];
#pragma unroll
    for (int j = 0; j < WPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = cur[j][i];
        d[j][4 * i] = u.x & keep[j][4 * i];
        d[j][4 * i + 1] = u.y & keep[j][4 * i + 1];
        d[j][4 * i + 2] = u.z & keep[j][4 * i + 2];
        d[j][4 * i + 3] = u.w & keep[j][4 * i + 3];
      }
    // per-thread min / max (or absmax) on packed fp16, then the block reduction
    f16x2 mn2 = {0, 0}, mx2 = {0, 0};
#pragma unroll
    for (int j = 0; j < WPT; ++j) word_minmax(d[j], asym, mn2, mx2);
    float mn = fminf((float)mn2.x, (float)mn2.y);
    float mx = fmaxf((float)mx2.x, (float)mx2.y);
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      redf[wave] = mn;
      redf[4 + wave] = mx;
    }
    __syncthreads();
    mn = fminf(fminf(redf[0], redf[1]), fminf(redf[2], redf[3]));
    mx = fmaxf(fmaxf(redf[4], redf[5]), fmaxf(redf[6], redf[7]));
    const RowQuant rqp = row_quant(asym, row_clip ? row_clip[t] : clip, wave_uniform(mn), wave_uniform(mx));
    int csum = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      if (active[j]) csum += quant_word(d[j], m[j], 32 * (tid * WPT + j) - before[j], asym, rqp, packed);
    if (code_sum) {
      csum = wave_sum(csum);
      if (lane == 0) redi[wave] = csum;
    }
    __syncthreads();
    uint8_t *qrow = q + t * (int64_t)(Kn / 2);
    for (int i = tid; i < nwords; i += kSplitThreads) {
      store_nt(reinterpret_cast<uint32_t *>(qrow) + i, packed[i]);
      packed[i] = 0u;
    }
    if (tid == 0) {
      scale[t] = rqp.s;
      if (asym) zero[t] = rqp.zp;
      if (code_sum) code_sum[t] = redi[0] + redi[1] + redi[2] + redi[3];
    }
    // outlier columns keep their fp16 bits
    unsigned short *xo = reinterpret_cast<unsigned short *>(x_out) + t * (int64_t)n_out;
#pragma unroll
    for (int k = 0; k < kOg; ++k) {
      const int r = tid + kSplitThreads * k;
      if (r < nset) xo[r] = og[k];
    }
    for (int r = tid + kSplitThreads * kOg; r < nset; r += kSplitThreads)
      xo[r] = reinterpret_cast<const unsigned short *>(row)[ocol[r]];
    packed[NW * 4] = 0u;
#pragma unroll
    for (int j = 0; j < WPT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[j][i] = nxt[j][i];
    __syncthreads();
    t += gridDim.x;
  } while (t < T);
}

hipError_t launch_split(const void *x, int64_t T, int64_t K, int64_t ldx, bool asym, float clip,
                        const float *row_clip, const int32_t *outlier_idx, int n_out, uint8_t *q,
                        float *scale, int32_t *zero, int32_t *code_sum, void *x_out, hipStream_t st) {
  const int64_t grid = T < 1024 ? T : 1024;
  const int words = (int)(K / 32);
  const dim3 g((unsigned)grid), b(kSplitThreads);
  const __half *xh = (const __half *)x;
  __half *xo = (__half *)x_out;
  const int a = asym ? 1 : 0;
  const size_t lds = (size_t)n_out * sizeof(uint16_t);  // the outlier column list
  void (*k)(const __half *, int64_t, int, int64_t, int, float, const float *, const int32_t *, int, uint8_t *,
            float *, int32_t *, int32_t *, __half *) =
      words <= kSplitThreads ? split_quant<1> : words <= 2 * kSplitThreads ? split_quant<2> : split_quant<4>;
  if (lds > 32 * 1024) {  // beyond what the static arrays leave of the default 64 KB
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k<<<g, b, lds, st>>>(xh, T, (int)K, ldx, a, clip, row_clip, outlier_idx, n_out, q, scale, zero, code_sum, xo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// rowlds_quant: one workgroup (256 threads) per row, grid-stride over rows.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;

struct RowArgs {
  const __half *x;
  int64_t T, K, ldx;
  int span_log2;      // 0: no transform
  int gsr;            // output permutation within each 2^span_log2 block
  float norm;
  float clip;
  uint8_t *q;
  float *scale;
  int32_t *code_sum;
};

__device__ __forceinline__ float block_reduce_max(float v, float *red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ int block_reduce_sum(int v, int *red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Dynamic LDS: vals fp32 [K].
__global__ __launch_bounds__(kRowThreads) void rowlds_quant(RowArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float redf[4];
  __shared__ int redi[4];
  const int K = (int)p.K;
  float *vals = reinterpret_cast<float *>(smem);
  const int tid = threadIdx.x;

  for (int64_t t = blockIdx.x; t < p.T; t += gridDim.x) {
    const __half *row = p.x + t * p.ldx;
    for (int c8 = tid; c8 < K / 8; c8 += kRowThreads) {
      const uint4 raw = *reinterpret_cast<const uint4 *>(row + c8 * 8);
      float f[8];
      h8_to_f32(raw, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) vals[c8 * 8 + i] = f[i];
    }
    __syncthreads();
    for (int lh = 0; lh < p.span_log2; ++lh) {
      const int h = 1 << lh;
      for (int pr = tid; pr < K / 2; pr += kRowThreads) {
        const int i = ((pr >> lh) << (lh + 1)) | (pr & (h - 1));
        const float u = vals[i], w = vals[i + h];
        vals[i] = u + w;
        vals[i + h] = u - w;
      }
      __syncthreads();
    }
    // rotated value of column c; GSR reads its block's transform output in
    // sequency order, sigma(s) = bitrev(gray(s))
    auto value_at = [&](int c) -> float {
      if (p.gsr) {
        const int bm = (1 << p.span_log2) - 1;
        const int s_ = c & bm;
        c = (c & ~bm) | (int)(__builtin_bitreverse32((uint32_t)(s_ ^ (s_ >> 1))) >> (32 - p.span_log2));
      }
      return vals[c] * p.norm;
    };
    float amax = 0.0f;
    for (int c = tid; c < K; c += kRowThreads) amax = fmaxf(amax, fabsf(value_at(c)));
    amax = block_reduce_max(amax, redf);
    float s, inv;
    sym_scale(amax, p.clip, s, inv);
    int csum = 0;
    uint8_t *qrow = p.q + t * (int64_t)(K / 2);
    for (int pb = tid; pb < K / 2; pb += kRowThreads) {
      const int c0 = quant_sym(value_at(2 * pb), inv, 7.0f);
      const int c1 = quant_sym(value_at(2 * pb + 1), inv, 7.0f);
      csum += c0 + c1;
      qrow[pb] = (uint8_t)((c0 & 0xF) | ((c1 & 0xF) << 4));
    }
    if (p.code_sum) csum = block_reduce_sum(csum, redi);
    if (tid == 0) {
      p.scale[t] = s;
      if (p.code_sum) p.code_sum[t] = csum;
    }
    __syncthreads();  // vals is reused by the next row
  }
}

// ---------------------------------------------------------------------------
// kron_quant: per row, M = (x * s) reshaped [n1, n2] (or x / s on the weight
// side), x' = A^T . M . B reshaped back, then symmetric INT4.
// Activations use A = P1, B = P2; the weight side passes A = P1^{-T},
// B = P2^{-T} and divides by s.
// ---------------------------------------------------------------------------
constexpr int kKronPad = 65;

__global__ __launch_bounds__(256) void kron_quant(const __half *__restrict__ x, int64_t T, int64_t ldx,
                                                  int n1, int n2, const float *__restrict__ fa,
                                                  const float *__restrict__ fb,
                                                  const float *__restrict__ chan_scale, int divide,
                                                  float clip, uint8_t *__restrict__ q,
                                                  float *__restrict__ scale,
                                                  int32_t *__restrict__ code_sum) {
  __shared__ float A[64 * kKronPad];
  __shared__ float B[64 * kKronPad];
  __shared__ float M[64 * kKronPad];
  __shared__ float U[64 * kKronPad];
  __shared__ float redf[4];
  __shared__ int redi[4];
  const int tid = threadIdx.x;
  const int K = n1 * n2;
  for (int i = tid; i < n1 * n1; i += 256) A[(i / n1) * kKronPad + i % n1] = fa[i];
  for (int i = tid; i < n2 * n2; i += 256) B[(i / n2) * kKronPad + i % n2] = fb[i];
  __syncthreads();
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const __half *row = x + t * ldx;
    for (int c = tid; c < K; c += 256) {
      float v = __half2float(row[c]);
      if (chan_scale) v = divide ? v / chan_scale[c] : v * chan_scale[c];
      M[(c / n2) * kKronPad + c % n2] = v;
    }
    __syncthreads();
    // U = A^T . M : U[j1][i2] = sum_i1 A[i1][j1] M[i1][i2]
    for (int o = tid; o < K; o += 256) {
      const int j1 = o / n2, i2 = o % n2;
      float acc = 0.0f;
      for (int i1 = 0; i1 < n1; ++i1) acc = fmaf(A[i1 * kKronPad + j1], M[i1 * kKronPad + i2], acc);
      U[j1 * kKronPad + i2] = acc;
    }
    __syncthreads();
    // x' = U . B : x'[j1][j2] = sum_i2 U[j1][i2] B[i2][j2]   (stored in M)
    float amax = 0.0f;
    for (int o = tid; o < K; o += 256) {
      const int j1 = o / n2, j2 = o % n2;
      float acc = 0.0f;
      for (int i2 = 0; i2 < n2; ++i2) acc = fmaf(U[j1 * kKronPad + i2], B[i2 * kKronPad + j2], acc);
      M[j1 * kKronPad + j2] = acc;
      amax = fmaxf(amax, fabsf(acc));
    }
    amax = block_reduce_max(amax, redf);  // includes a barrier after the M writes
    float s, inv;
    sym_scale(amax, clip, s, inv);
    int csum = 0;
    uint8_t *qrow = q + t * (int64_t)(K / 2);
    for (int pb = tid; pb < K / 2; pb += 256) {
      const int o0 = 2 * pb, o1 = 2 * pb + 1;
      const int c0 = quant_sym(M[(o0 / n2) * kKronPad + o0 % n2], inv, 7.0f);
      const int c1 = quant_sym(M[(o1 / n2) * kKronPad + o1 % n2], inv, 7.0f);
      csum += c0 + c1;
      qrow[pb] = (uint8_t)((c0 & 0xF) | ((c1 & 0xF) << 4));
    }
    if (code_sum) csum = block_reduce_sum(csum, redi);
    if (tid == 0) {
      scale[t] = s;
      if (code_sum) code_sum[t] = csum;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// kron_inverse_t: out_k = (P_k^{-1})^T in fp32, P_k fp32 [n_k, n_k], n_k <= 64.
// fp64 Gauss-Jordan elimination with partial pivoting on [P | I]; block k
// handles factor k.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kron_inverse_t(const float *__restrict__ p1, int n1,
                                                      float *__restrict__ o1,
                                                      const float *__restrict__ p2, int n2,
                                                      float *__restrict__ o2) {
  __shared__ double aug[64][129];
  __shared__ int piv;
  const float *P = blockIdx.x == 0 ? p1 : p2;
  float *O = blockIdx.x == 0 ? o1 : o2;
  const int n = blockIdx.x == 0 ? n1 : n2;
  const int tid = threadIdx.x;
  for (int i = tid; i < n * 2 * n; i += 256) {
    const int r = i / (2 * n), c = i % (2 * n);
    aug[r][c] = c < n ? (double)P[r * n + c] : (c - n == r ? 1.0 : 0.0);
  }
  __syncthreads();
  for (int col = 0; col < n; ++col) {
    if (tid == 0) {
      int best = col;
      double bv = fabs(aug[col][col]);
      for (int r = col + 1; r < n; ++r) {
        const double v = fabs(aug[r][col]);
        if (v > bv) {
          bv = v;
          best = r;
        }
      }
      piv = best;
    }
    __syncthreads();
    const int pr = piv;
    if (pr != col) {
      for (int c = tid; c < 2 * n; c += 256) {
        const double tmp = aug[col][c];
        aug[col][c] = aug[pr][c];
        aug[pr][c] = tmp;
      }
    }
    __syncthreads();
    const double d = aug[col][col];
    __syncthreads();
    for (int c = tid; c < 2 * n; c += 256) aug[col][c] /= d;
    __syncthreads();
    for (int i = tid; i < n * 2 * n; i += 256) {
      const int r = i / (2 * n), c = i % (2 * n);
      if (r != col && c != col) aug[r][c] -= aug[r][col] * aug[col][c];
    }
    __syncthreads();
    for (int r = tid; r < n; r += 256)
      if (r != col) aug[r][col] = 0.0;
    __syncthreads();
  }
  // inverse is aug[:, n:2n]; write its transpose
  for (int i = tid; i < n * n; i += 256) {
    const int r = i / n, c = i % n;
    O[r * n + c] = (float)aug[c][n + r];
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
// ---------------------------------------------------------------------------
hipError_t launch_fwht4096(const void *x, int64_t T, int64_t ldx, bool gsr, int span_log2,
                           float norm, float clip, uint8_t *q, float *scale, int32_t *code_sum,
                           hipStream_t st) {
  const int64_t blocks = (T + kF4096Waves - 1) / kF4096Waves;
  const bool had = !gsr && span_log2 == 12, gsr_mfma = gsr && span_log2 >= 3 && span_log2 <= 6;
  if (had || gsr_mfma) {
    // up to 2048 tokens (two wavefronts per SIMD) one token per wavefront;
    // beyond, at most 2048 wavefronts that take an even number of tokens
    // each, the next one's loads in flight while the current one is computed
    // (pairing from 1024 tokens on measured slower at 2048: 8.8 against 7.9 us)
    constexpr int64_t kMaxWaves = 2048;
    const int tpw = T <= kMaxWaves ? 1 : 2 * (int)((T + 2 * kMaxWaves - 1) / (2 * kMaxWaves));
    const dim3 grid((unsigned)(((T + tpw - 1) / tpw + 3) / 4)), block(256);
    const __half *xh = (const __half *)x;
    const int sl = had ? 12 : span_log2;
    const float nm = had ? 1.0f : norm;
    const bool clamp = clip < 1.0f;
#define RQ_FWHT(G, C, L) fwht4096_mfma<G, C, L><<<grid, block, 0, st>>>(xh, T, ldx, q, scale, code_sum, clip, sl, nm, tpw)
    if (had) {
      if (code_sum) {
        if (clamp) RQ_FWHT(false, true, true); else RQ_FWHT(false, true, false);
      } else {
        if (clamp) RQ_FWHT(false, false, true); else RQ_FWHT(false, false, false);
      }
    } else {
      if (code_sum) {
        if (clamp) RQ_FWHT(true, true, true); else RQ_FWHT(true, true, false);
      } else {
        if (clamp) RQ_FWHT(true, false, true); else RQ_FWHT(true, false, false);
      }
    }
#undef RQ_FWHT
    return hipGetLastError();
  }
  if (gsr)
    fwht4096_quant<true><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
        (const __half *)x, T, ldx, q, scale, code_sum, clip, span_log2, norm);
  else
    fwht4096_quant<false><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
        (const __half *)x, T, ldx, q, scale, code_sum, clip, span_log2, norm);
  return hipGetLastError();
}

size_t rowlds_smem_bytes(int64_t K) { return (size_t)K * 4; }

hipError_t launch_rowlds(const void *x, int64_t T, int64_t K, int64_t ldx, int span_log2, bool gsr,
                         float norm, float clip, uint8_t *q, float *scale, int32_t *code_sum,
                         hipStream_t st) {
  RowArgs p;
  p.x = (const __half *)x;
  p.T = T;
  p.K = K;
  p.ldx = ldx;
  p.span_log2 = span_log2;
  p.gsr = gsr ? 1 : 0;
  p.norm = norm;
  p.clip = clip;
  p.q = q;
  p.scale = scale;
  p.code_sum = code_sum;
  const size_t smem = rowlds_smem_bytes(K);
  hipError_t e = hipFuncSetAttribute((const void *)rowlds_quant,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int64_t grid = T < 8192 ? T : 8192;
  rowlds_quant<<<dim3((unsigned)grid), dim3(kRowThreads), smem, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_kron(const void *x, int64_t T, int64_t ldx, int n1, int n2, const float *fa,
                       const float *fb, const float *chan_scale, bool divide, float clip,
                       uint8_t *q, float *scale, int32_t *code_sum, hipStream_t st) {
  if (n1 == 64 && n2 == 64)
    return launch_kron64(x, T, ldx, fa, fb, chan_scale, divide, clip, q, scale, code_sum, st);
  const int64_t grid = T < 8192 ? T : 8192;
  kron_quant<<<dim3((unsigned)grid), dim3(256), 0, st>>>((const __half *)x, T, ldx, n1, n2, fa, fb,
                                                         chan_scale, divide ? 1 : 0, clip, q, scale,
                                                         code_sum);
  return hipGetLastError();
}

hipError_t launch_kron_inverse_t(const float *p1, int n1, float *o1, const float *p2, int n2,
                                 float *o2, hipStream_t st) {
  kron_inverse_t<<<dim3(2), dim3(256), 0, st>>>(p1, n1, o1, p2, n2, o2);
  return hipGetLastError();
}

}  // namespace rq
