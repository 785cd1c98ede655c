// gemm_decode.hip -- the small-T (decode) INT4 x INT4 GEMM with the fused
// dequantization epilogue (QUIK blog, "QUIK quantization" part 4: INT4
// operands, INT32 accumulation; part 1: dequantize, add the FP16 outlier
// product, round once), for T <= 32 on gfx950.
//
// At decode sizes the work is streaming the weight matrix once: 2TNK ops
// against N*K/2 bytes, far below the MFMA ridge.  So both kernels serve HBM:
// each wavefront owns a block of output channels and streams their weight
// rows from start to end, one sequential stream per row (splitting K across
// wavefronts gave every row several concurrent streams and measured 25%
// slower), through a register ring of k-steps.
//   gemm_decode16 (T <= 16, activation stage <= 64 KB): 16 channels per
//     wavefront, the activation rows staged in LDS, FP16 outlier columns as
//     extra ring steps.
//   gemm_decode (the rest): 32 channels per wavefront, activation fragments
//     read from L2 next to the weights, outlier fragments loaded before the
//     ring's prologue.
#include <algorithm>

#include "fwht_common.h"
#include "gemm_common.h"
#include "rq_kernels.h"
#include "split_common.h"

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

// gemm_decode16: T <= 16, activation codes staged in LDS.
//
// Reading the activation fragment of every k-step from L2 next to the weight
// fragment measured ~25% off the weight stream's rate, so here each
// workgroup copies the T activation rows (and, for the outlier product, the
// T rows of x_out) into LDS once, and the register ring carries weight bytes
// only.  One wavefront owns 16 output channels.
// v_mfma_i32_16x16x64_i8 / v_mfma_f32_16x16x32_f16 operands: lane l supplies
// row (A) or column (B) l%16 and k group l/16; register r of lane l holds
// row 4(l/16) + r, column l%16 (measured on gfx950).
// The stream of a wavefront is nsteps INT4 steps followed by n_out/32 FP16
// outlier steps; lane (c, kg) loads bytes [64j + 16kg, 64j + 16kg + 16) of
// its weight row (INT4: codes 128j + 32kg ..; FP16: w_out halves 32j + 8kg ..)
// and the same span of the staged activation row.  Widened dwords (x, y)
// feed INT8 MFMA 0 and (z, w) MFMA 1.  Each step issues both MFMA kinds and
// zeroes the operands of the kind it is not, so the loop has no branch;
// the zero products leave both accumulators (and their summation order)
// exactly as a loop over the live steps alone would.
namespace {
constexpr int kD16 = 8;  // load ring depth (k-steps)
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
// staged row pitches: 16 bytes of padding put the 16 rows a load
// instruction reads on 16 distinct 16-byte LDS bank groups
__host__ __device__ inline uint32_t d16_pitch(int64_t bytes) { return (uint32_t)bytes + 16; }
__host__ __device__ inline size_t d16_lds(int64_t T, int64_t Kb, int64_t n_out) {
  return (size_t)T * d16_pitch(Kb) + (n_out ? (size_t)T * d16_pitch(2 * n_out) : 0);
}
// staged 16-byte chunks
inline int64_t d16_chunks(int64_t T, int64_t Kb, int64_t n_out) { return T * (Kb / 16 + n_out / 8); }
// the stage fits 64 KB of LDS, which four wavefronts load in two groups
inline bool d16_fits(int64_t T, int64_t Kb, int64_t n_out) {
  return T <= 16 && d16_chunks(T, Kb, n_out) <= 4096;
}
// larger stages (up to 32 rows, as two halves of 16 rows per wavefront
// against one weight stream above 16): up to 152 KB of LDS (one workgroup per
// CU), loaded in at most three groups of 8 chunks per thread
constexpr size_t kD16MaxLds2 = 152 * 1024;
inline bool d16_fits2(int64_t T, int64_t Kb, int64_t n_out, int nthr) {
  return T <= 32 && d16_lds(T, Kb, n_out) <= kD16MaxLds2 && d16_chunks(T, Kb, n_out) <= 24 * (int64_t)nthr;
}
// floor(c / d) = umulhi(c, m) with m = ceil(2^32 / d) = floor((2^32 - 1) / d) + 1
// (d >= 2): exact while c * d < 2^32
__device__ inline uint32_t d16_magic(uint32_t d) { return 0xFFFFFFFFu / d + 1; }
}  // namespace

// G = 1, 2: the activation codes (and x_out) are loaded in G groups of 8
// 16-byte chunks per thread.  G = 0: the fused form -- the workgroup
// quantizes the T unrotated fp16 rows of f.x itself (QUIK part 1, with the
// outlier split; the arithmetic of split_common.h, so the codes are those of
// the standalone quantizer) straight into its LDS code rows, one wavefront
// per row, and gathers x_out beside them; the codes never reach HBM.
// The fused staging step (G = 0).  A row of K <= 8192 columns is 4 quarters
// of 64 words (32 columns each); lane l holds word 64q + l of quarter q, so a
// load instruction covers 4 KB of a row.  The T x 4 (row, quarter) chunks
// are dealt round-robin to the wavefronts.  Per workgroup: the outlier bit
// mask, each word's compacted position, AND masks zeroing the outlier halves
// (an LDS table, read per chunk) and the outlier columns in ascending order.
// Pass 1 folds every chunk's min / max into its row (LDS atomics on the bit
// patterns of non-negative floats); pass 2 reloads the chunks (from L2) and
// quantizes them with the row's parameters.  `prologue` issues the weight
// ring's first loads once the setup is done.  LDS: the code rows (pitch pa),
// the x_out rows (pitch po, from xo_base), then the outlier column list.
template <bool ASYM, typename Prologue>
__device__ __forceinline__ void stage_fused(const GemmArgs &p, const FuseArgs &f, uint8_t *xs, uint32_t pa,
                                            uint32_t po, uint32_t xo_base, uint32_t T, int nk, float *sxl,
                                            int *zxl, Prologue prologue) {
  __shared__ uint32_t omask[256];
  __shared__ v4u keepl[16][64];   // [4 quarter + 16-byte chunk][lane]
  __shared__ uint32_t rlo[16], rhi[16];  // per row: bits of -min(min x, 0) and max(max x, 0) (or max |x|)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t nthr = blockDim.x, nwaves = nthr >> 6;
  const int K = f.K, nw = K >> 5, n_out = p.n_out;
  uint16_t *ocol = reinterpret_cast<uint16_t *>(xs + xo_base + (nk ? T * po : 0));

  // chunk c = 4t + q: row t, quarter q of 64 words; quarters past the row are skipped
  const uint32_t nq = (uint32_t)(nw + 63) >> 6, nch = T * nq;
  constexpr int kB = 4;  // chunks per batch
  uint32_t d0[kB][16];   // the first batch, loaded before the setup (it needs none of it)
  {
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t c = min(wave + b * nwaves, nch - 1), t = c / nq, q = c - t * nq;
      const __half *src = f.x + t * f.ldx + 32 * min((int)(64 * q) + lane, nw - 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 u = *reinterpret_cast<const uint4 *>(src + 8 * k);
        d0[b][4 * k] = u.x;
        d0[b][4 * k + 1] = u.y;
        d0[b][4 * k + 2] = u.z;
        d0[b][4 * k + 3] = u.w;
      }
    }
  }
  // the first outlier indices of each thread, loaded beside the rows
  const int oi0 = tid < n_out ? f.oidx[tid] : -1;
  const v4u zero4 = {0u, 0u, 0u, 0u};
  for (uint32_t i = tid; i < T * pa / 16; i += nthr) reinterpret_cast<v4u *>(xs)[i] = zero4;
  for (int i = tid; i < 256; i += nthr) omask[i] = 0u;
  if (tid < 16) rlo[tid] = rhi[tid] = 0u;
  __syncthreads();
  if (oi0 >= 0 && oi0 < K) atomicOr(&omask[oi0 >> 5], 1u << (oi0 & 31));
  for (int j = tid + nthr; j < n_out; j += nthr) {
    const int c = f.oidx[j];
    if (c >= 0 && c < K) atomicOr(&omask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // word 64q + lane: its outlier bits m[q] and the outliers left of it
  uint32_t m[4];
  int before[4], base = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int w = 64 * q + lane;
    m[q] = w < nw ? omask[w] : 0u;
    const int cnt = __popc(m[q]);
    const int incl = wave_scan_dpp(cnt);
    before[q] = base + incl - cnt;
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  const int nset = min(base, n_out);
  if (wave == 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t mo = m[q];
      for (int r = before[q]; mo; ++r, mo &= mo - 1)
        if (r < n_out) ocol[r] = (uint16_t)(32 * (64 * q + lane) + __ffs(mo) - 1);
      // words past the row are zeroed whole
      const uint32_t mk = 64 * q + lane < nw ? m[q] : 0xFFFFFFFFu;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        keepl[4 * q + c][lane] = v4u{keep_mask(mk, 4 * c), keep_mask(mk, 4 * c + 1), keep_mask(mk, 4 * c + 2),
                                     keep_mask(mk, 4 * c + 3)};
    }
  __syncthreads();
  prologue();
  __builtin_amdgcn_sched_barrier(0);

  auto load_chunk = [&](uint32_t c, uint32_t (&d)[16]) {  // raw fp16 pairs of chunk c
    const uint32_t t = c / nq, q = c - t * nq;
    const __half *src = f.x + t * f.ldx + 32 * min((int)(64 * q) + lane, nw - 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 u = *reinterpret_cast<const uint4 *>(src + 8 * k);
      d[4 * k] = u.x;
      d[4 * k + 1] = u.y;
      d[4 * k + 2] = u.z;
      d[4 * k + 3] = u.w;
    }
  };
  auto mask_chunk = [&](uint32_t c, uint32_t (&d)[16]) {  // zero its outlier halves
    const uint32_t q = c - (c / nq) * nq;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const v4u km = keepl[4 * q + k][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * k + e] &= km[e];
    }
  };
  // Chunks go four at a time, their loads issued together; past the end a
  // batch repeats its wave's last chunk and skips its work.
  // pass 1: the rows' min / max
  for (uint32_t c0 = wave; c0 < nch; c0 += kB * nwaves) {
    uint32_t d[kB][16];
    if (c0 == (uint32_t)wave) {
#pragma unroll
      for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) d[b][e] = d0[b][e];
    } else {
#pragma unroll
      for (int b = 0; b < kB; ++b) load_chunk(min(c0 + b * nwaves, nch - 1), d[b]);
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t c = c0 + b * nwaves;
      if (c >= nch) break;
      mask_chunk(c, d[b]);
      f16x2 mn2 = {0, 0}, mx2 = {0, 0};
      word_minmax(d[b], ASYM, mn2, mx2);
      const float mn = wave_min_dpp(fminf((float)mn2.x, (float)mn2.y));
      const float mx = wave_max_dpp(fmaxf((float)mx2.x, (float)mx2.y));
      if (lane == 0) {
        // both >= 0 (0 - v and v + 0 turn a -0 into +0): their bits order as the values
        const uint32_t t = c / nq;
        atomicMax(&rlo[t], __float_as_uint(0.0f - mn));
        atomicMax(&rhi[t], __float_as_uint(mx + 0.0f));
      }
    }
  }
  __syncthreads();
  // pass 2: codes (and the outlier values) with each row's parameters
  for (uint32_t c0 = wave; c0 < nch; c0 += kB * nwaves) {
    uint32_t d[kB][16];
    unsigned short ov[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t c = min(c0 + b * nwaves, nch - 1), t = c / nq, q = c - t * nq;
      if (c0 == (uint32_t)wave) {  // the first batch is still in registers
#pragma unroll
        for (int e = 0; e < 16; ++e) d[b][e] = d0[b][e];
      } else {
        load_chunk(c, d[b]);
      }
      // rank 64q + lane of this row's outliers, loaded beside the chunk
      int oc = 0;  // past the list (or with none): column 0, loaded but not stored
      if (nk && nset > 0) oc = ocol[min((int)(64 * q) + lane, nset - 1)];
      ov[b] = reinterpret_cast<const unsigned short *>(f.x + t * f.ldx)[oc];
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t c = c0 + b * nwaves;
      if (c >= nch) break;
      const uint32_t t = c / nq, q = c - t * nq;
      mask_chunk(c, d[b]);
      const float mn = -__uint_as_float(rlo[t]), mx = __uint_as_float(rhi[t]);
      const RowQuant rq = row_quant(ASYM, f.clip, wave_uniform(mn), wave_uniform(mx));
      if (64 * q + lane < nw) {
        // q is uniform: m[q] and before[q] by selects, not an indexed load
        uint32_t mq = m[0];
        int bq = before[0];
#pragma unroll
        for (int k = 1; k < 4; ++k)
          if (q == (uint32_t)k) {
            mq = m[k];
            bq = before[k];
          }
        quant_word(d[b], mq, 32 * (64 * q + lane) - bq, ASYM, rq, reinterpret_cast<uint32_t *>(xs + t * pa));
      }
      if (q == 0 && lane == 0) {
        sxl[t] = rq.s;
        zxl[t] = rq.zp;
      }
      if (nk) {
        unsigned short *xrow = reinterpret_cast<unsigned short *>(xs + xo_base + t * po);
        const int r = 64 * q + lane;
        if (r < nset) xrow[r] = ov[b];
        if (q == 0) {  // beyond the 64 nq ranks the quarters cover
          const unsigned short *rowh = reinterpret_cast<const unsigned short *>(f.x + t * f.ldx);
          for (int r2 = 64 * (int)nq + lane; r2 < nset; r2 += 64) xrow[r2] = rowh[ocol[r2]];
        }
      }
    }
  }
}

// The rotated fused staging step (G = 0, RG > 0: 1 Walsh-Hadamard, 2 with a
// clip ratio below 1, 3 GSR, 4 GSR clipped), K = 4096: wavefront w takes rows
// w, w + nwaves, ..., each through fwht_token (the standalone quantizer's
// transform and arithmetic, so the codes are its codes), and writes the 2 KB
// of packed codes into its LDS code row and the scale beside it.  The weight
// ring's first loads go out as soon as the first row's loads are issued.
template <int RG, typename Prologue>
__device__ __forceinline__ void stage_rotated(const FuseArgs &f, uint8_t *xs, uint32_t pa, uint32_t T, float *sxl,
                                              Prologue prologue) {
  constexpr bool GSR = RG >= 3, CLAMP = RG == 2 || RG == 4;
  __shared__ uint4 ltab[GSR ? 8 : 16][64];
  __shared__ v4w stage[8][32 * 8];
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, g = lane >> 5;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t nthr = blockDim.x, nwaves = nthr >> 6;
  auto load = [&](v4w (&raw)[8], uint32_t t) {
    const v4w *row = reinterpret_cast<const v4w *>(f.x + (int64_t)t * f.ldx);
#pragma unroll
    for (int c = 0; c < 8; ++c) raw[c] = row[64 * c + lane];
  };
  v4w raw[8];
  load(raw, min(wave, T - 1));
  __builtin_amdgcn_sched_barrier(0);
  prologue();
  __builtin_amdgcn_sched_barrier(0);
  fwht_make_tables<GSR>(ltab, f.gsr_log2, tid, (int)nthr);
  __syncthreads();
  for (uint32_t t = wave; t < T; t += nwaves) {
    if (t != wave) load(raw, t);
    const FwhtOut o = fwht_token<GSR, false, CLAMP>(raw, stage[wave], ltab, f.norm, f.clip);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      *reinterpret_cast<v4w *>(xs + t * pa + 32 * (r32 + 32 * nb) + 16 * g) = o.code[nb];
    if (lane == 0) sxl[t] = o.s;
  }
}

// TH = 2 (17 to 32 rows): each wavefront also multiplies rows
// 16 .. 31 (register r of lane (l16, kg) then token 16 + 4kg + r of the
// second half) against the same weight fragments.
template <bool XU, int MODE, int G, int RG = 0, int TH = 1>
__global__ __launch_bounds__(512) void gemm_decode16(GemmArgs p, FuseArgs f) {
  extern __shared__ __align__(16) uint8_t xs[];
  __shared__ float sxl[16 * TH];  // the rows' scales and zero points (G = 0: made here; else staged)
  __shared__ int zxl[16 * TH];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, l16 = lane & 15;
  const uint32_t nthr = blockDim.x;
  // f.ks wavefronts share each block of 16 channels, each streaming one part
  // of its k-steps (INT4 steps, then outlier steps, each split f.ks ways)
  const int ks = f.ks, cb = (int)(nthr >> 6) / ks;
  const int part = wave / cb, cbk = wave - part * cb;
  const int64_t n0 = ((int64_t)blockIdx.x * cb + cbk) * 16, Kb = p.Kb;
  const int nsteps = (int)(Kb >> 6), last = nsteps - 1;
  const int nk = MODE == 2 ? p.n_out / 32 : 0;  // outlier steps
  const int qs = (nsteps + ks - 1) / ks, qk = (nk + ks - 1) / ks;  // steps per part
  const int j0 = part * qs, o0 = part * qk, L = qs + qk;
  const uint32_t T = (uint32_t)p.T;
  // G = 0 rows have room for all K codes, so that a list with repeated
  // indices (fewer distinct outliers) cannot run a row into the next one
  const uint32_t pa = d16_pitch(G == 0 ? (int64_t)f.K / 2 : Kb), po = d16_pitch(2 * (int64_t)p.n_out);
  const uint32_t xo_base = T * pa;

  // weight stream of this lane: INT4 row, then its outlier row
  const int64_t nrow = min(n0 + l16, p.N - 1);
  const uint8_t *bp = p.qw + nrow * Kb + 16 * kg;
  const uint8_t *wp = nk ? reinterpret_cast<const uint8_t *>(p.wo + nrow * p.n_out) + 16 * kg : bp;
  // the part's local step i, clamped into the stream
  auto src = [&](int i) {
    return i < qs ? bp + 64 * (int64_t)min(j0 + i, last) : wp + 64 * (int64_t)max(min(o0 + i - qs, nk - 1), 0);
  };

  uint4 rb[kD16];
  if constexpr (G == 0 && RG != 0) {
    stage_rotated<RG>(f, xs, pa, T, sxl, [&] {
#pragma unroll
      for (int s = 0; s < kD16; ++s) rb[s] = *reinterpret_cast<const uint4 *>(src(min(s, L - 1)));
    });
  } else if constexpr (G == 0) {
    stage_fused<XU>(p, f, xs, pa, po, xo_base, T, nk, sxl, zxl, [&] {
#pragma unroll
      for (int s = 0; s < kD16; ++s) rb[s] = *reinterpret_cast<const uint4 *>(src(min(s, L - 1)));
    });
  } else {
    // Staging: 16-byte chunks c < na are activation codes (row c / ka), the
    // next no are x_out halves (row (c - na) / ko); 8G per thread.
    const uint32_t ka = (uint32_t)(Kb >> 4), ko = (uint32_t)p.n_out >> 3;
    const uint32_t na = T * ka, no = nk ? T * ko : 0;
    const uint8_t *xo = reinterpret_cast<const uint8_t *>(p.xo);
    // G groups of 8 loads in registers (G fixed at launch: a branch here makes
    // the compiler wait for every load at its join); a lane past the end
    // reloads the last chunk (one shared line per instruction).
    const uint32_t nt = na + no;
    // the rows' scales and zero points, loaded unconditionally (clamped row;
    // without zx a stand-in read, zeroed) and parked in LDS with the codes
    const uint32_t tc = min((uint32_t)tid, T - 1);
    const int32_t *zxp = p.zx ? p.zx : reinterpret_cast<const int32_t *>(p.sx);
    const float vsx = MODE != 0 ? p.sx[tc] : 0.0f;
    const int32_t vzx = MODE == 2 ? zxp[tc] : 0;
    v4u s0[8], s1[8], s2[8];
    auto sload = [&](v4u (&v)[8], int h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = min(nthr * (8 * h + i) + tid, nt - 1);
        v[i] = *reinterpret_cast<const v4u *>(c < na ? p.qx + 16 * (int64_t)c : xo + 16 * (int64_t)(c - na));
      }
    };
    sload(s0, 0);
    if (G >= 2) sload(s1, 1);
    if (G >= 3) sload(s2, 2);
    // Half the weight ring's prologue goes out behind the staging loads, so
    // waiting for the latter below leaves it in flight; the other half once
    // the stage is written.  With the whole ring ahead, the staging loads
    // came back behind more of the launch's first burst of weight requests
    // (whole ring 28.4-29.2 us at the QUIK decode shape, half 27.9-28.9,
    // a quarter or three quarters no better than whole).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kD16 / 2; ++s) rb[s] = *reinterpret_cast<const uint4 *>(src(min(s, L - 1)));
    __builtin_amdgcn_sched_barrier(0);
    {
      const uint32_t ma = d16_magic(ka), mo = nk ? d16_magic(ko) : 0;
      auto sstore = [&](const v4u (&v)[8], int h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t c = nthr * (8 * h + i) + tid;
          if (c < na) {
            const uint32_t r = __umulhi(c, ma);
            *reinterpret_cast<v4u *>(xs + r * pa + 16 * (c - r * ka)) = v[i];
          } else if (c < nt) {
            const uint32_t c2 = c - na, r = __umulhi(c2, mo);
            *reinterpret_cast<v4u *>(xs + xo_base + r * po + 16 * (c2 - r * ko)) = v[i];
          }
        }
      };
      sstore(s0, 0);
      if (G >= 2) sstore(s1, 1);
      if (G >= 3) sstore(s2, 2);
    }
#pragma unroll
    for (int s = kD16 / 2; s < kD16; ++s) rb[s] = *reinterpret_cast<const uint4 *>(src(min(s, L - 1)));
    if (tid < T) {
      sxl[tid] = vsx;
      zxl[tid] = p.zx ? vzx : 0;
    }
  }
  __syncthreads();
  // a wavefront past the last channel leaves (after its share of the
  // staging) unless it must meet the others again to add the parts
  if (ks == 1 && n0 >= p.N) return;

  const uint32_t arow = min((uint32_t)l16, T - 1);
  const uint8_t *xa = xs + arow * pa + 16 * kg;
  const uint8_t *xoa = nk ? xs + xo_base + arow * po + 16 * kg : xa;  // never read unmasked when nk == 0
  // the second half's rows (TH = 2), clamped like the first
  const uint32_t arow2 = min((uint32_t)(16 + l16), T - 1);
  const uint8_t *xa2 = xs + arow2 * pa + 16 * kg;
  const uint8_t *xoa2 = nk ? xs + xo_base + arow2 * po + 16 * kg : xa2;
  // the channel's scale and code sum go out before the weight stream, so the
  // epilogue does not wait on them
  const bool has_zx = G == 0 ? XU : p.zx != nullptr;
  const int64_t gnc = min(n0 + l16, p.N - 1);
  const float swn = MODE != 0 ? p.sw[gnc] : 0.0f;
  const int32_t rsn = (MODE == 2 && has_zx) ? p.rowsum[gnc] : 0;
  v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0}, acc3 = {0, 0, 0, 0};
  v4f fo = {0.0f, 0.0f, 0.0f, 0.0f}, fo2 = {0.0f, 0.0f, 0.0f, 0.0f};
  // Whole ring groups of live INT4 steps first: no masks, no outlier
  // operands (their zero products would leave fo at +0 unchanged) and no
  // x_out reads, so a wavefront issues about half the instructions per step
  // and two wavefronts sharing a SIMD keep pace with the weight stream.  The
  // rest (the group holding the INT4 / outlier boundary, the outlier steps
  // and steps past the end) takes the general step below.
  const int qa = min(qs, nsteps - j0);  // this part's live INT4 steps
  int i0 = 0;
  for (; i0 + kD16 <= qa; i0 += kD16) {
#pragma unroll
    for (int u = 0; u < kD16; ++u) {
      const int i = i0 + u;
      const uint4 wq = rb[u];
      const uint4 wa = *reinterpret_cast<const uint4 *>(xa + 64 * (j0 + i));
      const v4i a0 = XU ? widen_unsigned(wa.x, wa.y) : widen_signed(wa.x, wa.y);
      const v4i a1 = XU ? widen_unsigned(wa.z, wa.w) : widen_signed(wa.z, wa.w);
      const v4i b0 = widen_signed(wq.x, wq.y), b1 = widen_signed(wq.z, wq.w);
      v4i a2, a3;
      if (TH == 2) {
        const uint4 wa2 = *reinterpret_cast<const uint4 *>(xa2 + 64 * (j0 + i));
        a2 = XU ? widen_unsigned(wa2.x, wa2.y) : widen_signed(wa2.x, wa2.y);
        a3 = XU ? widen_unsigned(wa2.z, wa2.w) : widen_signed(wa2.z, wa2.w);
      }
      __builtin_amdgcn_sched_barrier(0);
      rb[u] = *reinterpret_cast<const uint4 *>(src(min(i + kD16, L - 1)));
      acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc1, 0, 0, 0);
      if (TH == 2) {
        acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b0, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, b1, acc3, 0, 0, 0);
      }
    }
  }
  for (; i0 < L; i0 += kD16) {
#pragma unroll
    for (int u = 0; u < kD16; ++u) {
      const int i = i0 + u;
      const uint4 wq = rb[u];
      const uint32_t l4 = (i < qs && j0 + i < nsteps) ? 0xFFFFFFFFu : 0u;
      const uint4 wa = *reinterpret_cast<const uint4 *>(xa + 64 * min(j0 + i, last));
      const v4i a0 = XU ? widen_unsigned(wa.x & l4, wa.y & l4) : widen_signed(wa.x & l4, wa.y & l4);
      const v4i a1 = XU ? widen_unsigned(wa.z & l4, wa.w & l4) : widen_signed(wa.z & l4, wa.w & l4);
      const v4i b0 = widen_signed(wq.x, wq.y), b1 = widen_signed(wq.z, wq.w);
      v4i a2, a3;
      if (TH == 2) {
        const uint4 wa2 = *reinterpret_cast<const uint4 *>(xa2 + 64 * min(j0 + i, last));
        a2 = XU ? widen_unsigned(wa2.x & l4, wa2.y & l4) : widen_signed(wa2.x & l4, wa2.y & l4);
        a3 = XU ? widen_unsigned(wa2.z & l4, wa2.w & l4) : widen_signed(wa2.z & l4, wa2.w & l4);
      }
      v8h ao, bo, ao2;
      if (MODE == 2) {
        const int jo = o0 + i - qs;
        const uint32_t lo = (i >= qs && i < L && jo < nk) ? 0xFFFFFFFFu : 0u;
        const uint4 xv = *reinterpret_cast<const uint4 *>(xoa + 64 * max(min(jo, nk - 1), 0));
        const uint4 am = {xv.x & lo, xv.y & lo, xv.z & lo, xv.w & lo};
        const uint4 bm = {wq.x & lo, wq.y & lo, wq.z & lo, wq.w & lo};
        __builtin_memcpy(&ao, &am, 16);
        __builtin_memcpy(&bo, &bm, 16);
        if (TH == 2) {
          const uint4 xv2 = *reinterpret_cast<const uint4 *>(xoa2 + 64 * max(min(jo, nk - 1), 0));
          const uint4 am2 = {xv2.x & lo, xv2.y & lo, xv2.z & lo, xv2.w & lo};
          __builtin_memcpy(&ao2, &am2, 16);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      rb[u] = *reinterpret_cast<const uint4 *>(src(min(i + kD16, L - 1)));
      acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc1, 0, 0, 0);
      if (MODE == 2) fo = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, bo, fo, 0, 0, 0);
      if (TH == 2) {
        acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b0, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, b1, acc3, 0, 0, 0);
        if (MODE == 2) fo2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao2, bo, fo2, 0, 0, 0);
      }
    }
  }
  if (ks > 1) {
    // the parts' sums meet in LDS (the staged rows are free once every
    // wavefront is past its loop); part 0 adds them in part order
    __syncthreads();
    uint32_t *red = reinterpret_cast<uint32_t *>(xs);
    constexpr int RS = 12 * TH;  // reduction slots per wavefront
    if (part > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        red[(wave * RS + r) * 64 + lane] = (uint32_t)acc0[r];
        red[(wave * RS + 4 + r) * 64 + lane] = (uint32_t)acc1[r];
        red[(wave * RS + 8 + r) * 64 + lane] = __float_as_uint(fo[r]);
        if (TH == 2) {
          red[(wave * RS + 12 + r) * 64 + lane] = (uint32_t)acc2[r];
          red[(wave * RS + 16 + r) * 64 + lane] = (uint32_t)acc3[r];
          red[(wave * RS + 20 + r) * 64 + lane] = __float_as_uint(fo2[r]);
        }
      }
    }
    __syncthreads();
    if (part > 0 || n0 >= p.N) return;
    for (int q = 1; q < ks; ++q) {
      const int w2 = q * cb + cbk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc0[r] += (int)red[(w2 * RS + r) * 64 + lane];
        acc1[r] += (int)red[(w2 * RS + 4 + r) * 64 + lane];
        fo[r] += __uint_as_float(red[(w2 * RS + 8 + r) * 64 + lane]);
        if (TH == 2) {
          acc2[r] += (int)red[(w2 * RS + 12 + r) * 64 + lane];
          acc3[r] += (int)red[(w2 * RS + 16 + r) * 64 + lane];
          fo2[r] += __uint_as_float(red[(w2 * RS + 20 + r) * 64 + lane]);
        }
      }
    }
  }

  // Epilogue: register r of lane (l16, kg) is token 4kg + r, channel n0 + l16.
  constexpr int kShift = XU ? 4 : 8;
  const int64_t gn = n0 + l16;
  if (MODE == 0) {
    int32_t *out = reinterpret_cast<int32_t *>(p.out);
#pragma unroll
    for (int h = 0; h < TH; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gm = 16 * h + 4 * kg + r;
        const int32_t a = h ? acc2[r] + acc3[r] : acc0[r] + acc1[r];
        if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = a >> kShift;
      }
    return;
  }
  __half *out = reinterpret_cast<__half *>(p.out);
#pragma unroll
  for (int h = 0; h < TH; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gm = 16 * h + 4 * kg + r;
      const int64_t gmc = min(gm, p.T - 1);
      int32_t v = (h ? acc2[r] + acc3[r] : acc0[r] + acc1[r]) >> kShift;
      if (MODE == 2 && has_zx) v -= zxl[gmc] * rsn;
      const float y = (float)v * sxl[gmc] * swn + (h ? fo2[r] : fo[r]);
      if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = __float2half_rn(y);
    }
}

// Waves per workgroup (w) and K parts (ks) for N channels of `steps` k-steps
// (INT4 and outlier steps).  One wavefront streams each block of 16 channels
// whole, w sized so that the workgroups spread evenly over the 256 CUs
// (N = 28672 takes 256 of 7; 448 of 4 left 64 CUs with half the work of the
// rest and measured 11% slower).  With fewer than 1024 blocks and long rows
// the blocks' k-steps are split over ks = 2 .. 8 wavefronts of 8-wavefront
// workgroups, towards 2048 weight streams, as long as each part keeps at
// least 32 steps: split into 8-step parts, the 4096-wide rows of N = 11008
// measured 35% slower (every stream a single round trip, 22 MB requested at
// once) and N = 4096 no faster; split in two (35 steps per part), the QUIK
// decode shape (N = 28672) measured 35.1-36.7 against 29-30 us.
static void d16_grid(int64_t N, int64_t steps, int &w, int &ks) {
  const int64_t rb = (N + 15) / 16;
  ks = 1;
  while (rb < 1024 && ks < 8 && rb * ks < 2048 && steps / (2 * ks) >= 32) ks *= 2;
  w = ks > 1 ? 8 : (int)std::min<int64_t>(8, std::max<int64_t>(4, (rb + 255) / 256));
}
constexpr size_t kD16Reduce = 8 * 12 * 64 * 4;  // LDS for adding the parts
constexpr size_t kD16Reduce2 = 8 * 24 * 64 * 4;  // the same with two row halves

// the kernel for (mode, unsigned activations) with G staging groups and TH
// row halves
template <int G, int TH>
static void (*d16_kernel(int mode, bool xu))(GemmArgs, FuseArgs) {
  return mode == 0   ? (xu ? gemm_decode16<true, 0, G, 0, TH> : gemm_decode16<false, 0, G, 0, TH>)
         : mode == 1 ? gemm_decode16<false, 1, G, 0, TH>
                     : (xu ? gemm_decode16<true, 2, G, 0, TH> : gemm_decode16<false, 2, G, 0, TH>);
}

bool gemm_decode_fits(const GemmArgs &p) { return p.T <= 32 && p.Kb % 64 == 0 && p.Kb >= 64; }

hipError_t launch_gemm_decode(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  const int64_t n_out = mode == 2 ? p.n_out : 0;
  if (d16_fits(p.T, p.Kb, n_out)) {
    // w wavefronts (16 channels each) per workgroup, sized so that the
    // channel blocks spread evenly over the 256 CUs: N = 28672 takes 256
    // workgroups of 7 (448 of 4 left 64 CUs with half the work of the rest
    // and measured 11% slower); at least 4, at most 8
    const int64_t rb = (p.N + 15) / 16;
    int w, ks;
    d16_grid(p.N, p.Kb / 64 + n_out / 32, w, ks);
    const int cb = w / ks;
    const dim3 grid((unsigned)((rb + cb - 1) / cb)), block(64 * w);
    const bool g2 = d16_chunks(p.T, p.Kb, n_out) > 8 * 64 * w;
    const size_t lds = std::max(d16_lds(p.T, p.Kb, n_out), ks > 1 ? kD16Reduce : 0);
    void (*k)(GemmArgs, FuseArgs);
    if (g2)
      k = mode == 0   ? (x_unsigned ? gemm_decode16<true, 0, 2> : gemm_decode16<false, 0, 2>)
          : mode == 1 ? gemm_decode16<false, 1, 2>
                      : (x_unsigned ? gemm_decode16<true, 2, 2> : gemm_decode16<false, 2, 2>);
    else
      k = mode == 0   ? (x_unsigned ? gemm_decode16<true, 0, 1> : gemm_decode16<false, 0, 1>)
          : mode == 1 ? gemm_decode16<false, 1, 1>
                      : (x_unsigned ? gemm_decode16<true, 2, 1> : gemm_decode16<false, 2, 1>);
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    FuseArgs f{};
    f.ks = ks;
    k<<<grid, block, lds, st>>>(p, f);
    return hipGetLastError();
  }
  {
    // stages above 64 KB, and 17 to 32 rows (the same streams, each against
    // two halves of 16 rows)
    const int64_t rb = (p.N + 15) / 16;
    int w, ks;
    d16_grid(p.N, p.Kb / 64 + n_out / 32, w, ks);
    const int nthr = 64 * w;
    if (d16_fits2(p.T, p.Kb, n_out, nthr)) {
      const int cb = w / ks;
      const dim3 grid((unsigned)((rb + cb - 1) / cb)), block((unsigned)nthr);
      const int64_t ch = d16_chunks(p.T, p.Kb, n_out);
      const bool two = p.T > 16;
      void (*k)(GemmArgs, FuseArgs) =
          two ? (ch <= 8 * (int64_t)nthr    ? d16_kernel<1, 2>(mode, x_unsigned)
                 : ch <= 16 * (int64_t)nthr ? d16_kernel<2, 2>(mode, x_unsigned)
                                            : d16_kernel<3, 2>(mode, x_unsigned))
              : (ch <= 8 * (int64_t)nthr    ? d16_kernel<1, 1>(mode, x_unsigned)
                 : ch <= 16 * (int64_t)nthr ? d16_kernel<2, 1>(mode, x_unsigned)
                                            : d16_kernel<3, 1>(mode, x_unsigned));
      const size_t lds = std::max(d16_lds(p.T, p.Kb, n_out), ks > 1 ? (two ? kD16Reduce2 : kD16Reduce) : 0);
      if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      FuseArgs f{};
      f.ks = ks;
      k<<<grid, block, lds, st>>>(p, f);
      return hipGetLastError();
    }
  }
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

// Fused decode: the kernel's LDS is the code rows (room for all K codes),
// the x_out rows and the outlier column list.
static size_t fused_lds(int64_t T, int64_t K, int64_t n_out) {
  return (size_t)T * d16_pitch(K / 2) + (n_out ? (size_t)T * d16_pitch(2 * n_out) + 2 * (size_t)n_out : 0);
}

bool decode_fused_rot_fits(const GemmArgs &p, const FuseArgs &f) {
  return p.T >= 1 && p.T <= 16 && f.K == 4096 && p.Kb == 2048 && p.n_out == 0 && f.gsr_log2 >= 0 &&
         f.gsr_log2 <= 6 && f.gsr_log2 != 1 && f.gsr_log2 != 2;
}

hipError_t launch_decode_fused_rot(const GemmArgs &p, const FuseArgs &f0, hipStream_t st) {
  const int64_t rb = (p.N + 15) / 16;
  int w, ks;
  d16_grid(p.N, p.Kb / 64, w, ks);
  FuseArgs f = f0;
  f.ks = ks;
  const int cb = w / ks;
  const dim3 grid((unsigned)((rb + cb - 1) / cb)), block(64 * w);
  const size_t lds = std::max((size_t)p.T * d16_pitch(2048), ks > 1 ? kD16Reduce : 0);
  const bool gsr = f.gsr_log2 != 0, clamp = f.clip < 1.0f;
  void (*k)(GemmArgs, FuseArgs) = gsr ? (clamp ? gemm_decode16<false, 1, 0, 4> : gemm_decode16<false, 1, 0, 3>)
                                      : (clamp ? gemm_decode16<false, 1, 0, 2> : gemm_decode16<false, 1, 0, 1>);
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  k<<<grid, block, lds, st>>>(p, f);
  return hipGetLastError();
}

bool decode_fused_fits(const GemmArgs &p, const FuseArgs &f) {
  return p.T >= 1 && p.T <= 16 && f.K % 32 == 0 && f.K <= 8192 && p.Kb % 64 == 0 && p.Kb >= 64 &&
         2 * p.Kb + p.n_out == f.K && fused_lds(p.T, f.K, p.n_out) <= 96 * 1024;
}

hipError_t launch_decode_fused(const GemmArgs &p, const FuseArgs &f0, bool asym, int mode, hipStream_t st) {
  const int64_t rb = (p.N + 15) / 16;
  int w, ks;
  d16_grid(p.N, p.Kb / 64 + (mode == 2 ? p.n_out / 32 : 0), w, ks);
  FuseArgs f = f0;
  f.ks = ks;
  const int cb = w / ks;
  const dim3 grid((unsigned)((rb + cb - 1) / cb)), block(64 * w);
  const size_t lds = std::max(fused_lds(p.T, f.K, mode == 2 ? p.n_out : 0), ks > 1 ? kD16Reduce : 0);
  void (*k)(GemmArgs, FuseArgs) = mode == 1 ? gemm_decode16<false, 1, 0>
                                  : asym    ? gemm_decode16<true, 2, 0>
                                            : gemm_decode16<false, 2, 0>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k<<<grid, block, lds, st>>>(p, f);
  return hipGetLastError();
}

}  // namespace rq
