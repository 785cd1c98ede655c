// gemm_decode8.hip -- the decode-size (T <= 32) INT8 x INT8 GEMM of QUIK-8B's
// down projection (QUIK blog, "QUIK量化" part 3: the sensitive down
// projection in INT8; the QUIK-8B experiments), with INT32 accumulation
// (part 4) and the fused epilogue: zero-point correction, scales, and the FP16
// outlier product added before the one fp16 rounding (part 1), on gfx950.
//
// At decode sizes the work is one pass over the weight matrix (N * K bytes)
// against a few KB of activations, so the kernel is a weight streamer.  A
// workgroup of 8 wavefronts holds CB blocks of 16 output channels and splits
// each block's K range KS ways (KS * CB = 8): wavefront (ks, cb) streams the
// 16 weight rows of block cb over the ks-th part of the k-steps, one
// sequential stream per row through an 8-step register ring.  KS is chosen so
// that the grid holds about 2048 wavefronts (the down projection, N = 8192,
// has 512 channel blocks: KS = 4), enough bytes in flight to cover the HBM
// latency; the KS partial sums meet in LDS at the end.
//
// Activations are staged in LDS phase by phase: a phase is 8 k-steps (512
// bytes of each token row) of every K part, double-buffered, one barrier per
// phase; each thread loads its share of the next phase while the wavefronts
// multiply the current one.  Unsigned activation codes are stored as u - 128
// (one xor per dword) so that they are int8 MFMA operands; the epilogue adds
// the 128 * rowsum back through the zero-point correction.  The FP16 outlier
// columns follow the INT8 steps in each wavefront's stream (its share of the
// n_out / 32 outlier steps), with x_out staged in LDS once.
//
// v_mfma_i32_16x16x64_i8 / v_mfma_f32_16x16x32_f16: lane l supplies row (A)
// or column (B) l % 16 and k group l / 16 (16 bytes); register r of lane l
// holds row 4 (l / 16) + r, column l % 16.  Tokens are the A rows (NRB blocks
// of 16), channels the B columns.
#include <algorithm>

#include "rq_device.h"
#include "rq_kernels.h"

namespace rq {

namespace {

constexpr int kD8Waves = 8;
constexpr int kD8Ring = 8;                  // weight ring depth = steps per phase
constexpr int kD8Row = kD8Ring * 64 + 16;   // staged bytes per token row and phase (16 of padding)

struct D8Args {
  int ks, cb;        // K parts, channel blocks per workgroup (ks * cb = 8)
  int nsteps;        // 64-code steps of a row
  int qsteps;        // INT8 steps per K part, a multiple of 8
  int nk, qk;        // outlier steps (32 fp16 columns each) in all, per K part
  int nph;           // phases per K part (qsteps / 8)
  uint32_t stage;    // bytes of one phase buffer (ks * T * kD8Row)
  uint32_t xo_base;  // LDS offset of the staged x_out rows
  uint32_t po;       // their pitch
};

__host__ __device__ inline uint32_t d8_po(int n_out) { return (uint32_t)(2 * n_out + 16); }

}  // namespace

template <bool XU, int MODE, int NRB>
__global__ __launch_bounds__(512) void gemm_decode8(GemmArgs p, D8Args d) {
  extern __shared__ __align__(16) uint8_t xs[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wave / d.cb, cbk = wave - ks * d.cb;
  const int kg = lane >> 4, l16 = lane & 15;
  const uint32_t T = (uint32_t)p.T;
  const int64_t n0 = ((int64_t)blockIdx.x * d.cb + cbk) * 16, Kb = p.Kb;
  const int last = d.nsteps - 1;

  // this lane's weight stream: the INT8 steps of its K part, then its outlier steps
  const int64_t nrow = min(n0 + l16, p.N - 1);
  const uint8_t *bp = p.qw + nrow * Kb + 16 * kg;
  const uint8_t *wp = d.nk ? reinterpret_cast<const uint8_t *>(p.wo + nrow * p.n_out) + 16 * kg : bp;
  const int j0 = ks * d.qsteps, o0 = ks * d.qk;
  const int L = d.qsteps + d.qk;
  auto src = [&](int i) {  // local step i, clamped into the stream
    return i < d.qsteps ? bp + 64 * (int64_t)min(j0 + i, last)
                        : wp + 64 * (int64_t)max(min(o0 + i - d.qsteps, d.nk - 1), 0);
  };

  // Stage of phase ph: chunk c (16 bytes) = part q, token row r, chunk cc of
  // the phase's 512 bytes; the activation offset is clamped into the row
  // (steps past the end are staged but masked).
  const uint32_t nch = (uint32_t)d.ks * T * 32;
  auto sload = [&](uint4 (&v)[4], int ph) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = min((uint32_t)(tid + 512 * i), nch - 1);
      const uint32_t q = c / (T * 32), rem = c - q * T * 32, r = rem >> 5, cc = rem & 31;
      const int64_t off = min((int64_t)(q * d.qsteps + ph * kD8Ring) * 64 + 16 * cc, Kb - 16);
      v[i] = *reinterpret_cast<const uint4 *>(p.qx + r * Kb + off);
    }
  };
  auto sstore = [&](const uint4 (&v)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = (uint32_t)(tid + 512 * i);
      if (c < nch) {
        const uint32_t q = c / (T * 32), rem = c - q * T * 32, r = rem >> 5, cc = rem & 31;
        const uint32_t f = XU ? 0x80808080u : 0u;
        const uint4 w = {v[i].x ^ f, v[i].y ^ f, v[i].z ^ f, v[i].w ^ f};
        *reinterpret_cast<uint4 *>(xs + buf * d.stage + (q * T + r) * kD8Row + 16 * cc) = w;
      }
    }
  };

  uint4 rb[kD8Ring];
  {
    uint4 sv[4];
    sload(sv, 0);
    // half the weight ring's prologue ahead of the staging wait, half after
    // the stage is written (as in gemm_decode16)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kD8Ring / 2; ++s) rb[s] = *reinterpret_cast<const uint4 *>(src(min(s, L - 1)));
    __builtin_amdgcn_sched_barrier(0);
    sstore(sv, 0);
#pragma unroll
    for (int s = kD8Ring / 2; s < kD8Ring; ++s) rb[s] = *reinterpret_cast<const uint4 *>(src(min(s, L - 1)));
    // x_out rows, once (the outlier steps read them)
    if (d.nk) {
      const uint32_t ko = (uint32_t)p.n_out / 8, no = T * ko;
      const uint8_t *xo = reinterpret_cast<const uint8_t *>(p.xo);
      for (uint32_t c = tid; c < no; c += 512) {
        const uint32_t r = c / ko, cc = c - r * ko;
        *reinterpret_cast<uint4 *>(xs + d.xo_base + r * d.po + 16 * cc) =
            *reinterpret_cast<const uint4 *>(xo + 16 * (int64_t)c);
      }
    }
  }
  __syncthreads();

  v4i acc[NRB];
  v4f fo[NRB];
#pragma unroll
  for (int b = 0; b < NRB; ++b) {
    acc[b] = v4i{0, 0, 0, 0};
    fo[b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  uint32_t arow[NRB];
#pragma unroll
  for (int b = 0; b < NRB; ++b) arow[b] = min((uint32_t)(l16 + 16 * b), T - 1);

  // INT8 phases: the stage of phase ph + 1 goes out first, then 8 steps on
  // the current stage, then it is stored and the workgroup meets once.
  for (int ph = 0; ph < d.nph; ++ph) {
    uint4 sv[4];
    sload(sv, min(ph + 1, d.nph - 1));
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t *sb = xs + (ph & 1) * d.stage + (uint32_t)ks * T * kD8Row + 16 * kg;
#pragma unroll
    for (int u = 0; u < kD8Ring; ++u) {
      const int i = ph * kD8Ring + u;
      const uint32_t live = j0 + i < d.nsteps ? 0xFFFFFFFFu : 0u;
      const uint4 wq = rb[u];
      v4i a[NRB];
#pragma unroll
      for (int b = 0; b < NRB; ++b) {
        const uint4 x = *reinterpret_cast<const uint4 *>(sb + arow[b] * kD8Row + 64 * u);
        a[b] = v4i{(int)(x.x & live), (int)(x.y & live), (int)(x.z & live), (int)(x.w & live)};
      }
      const v4i bw = {(int)wq.x, (int)wq.y, (int)wq.z, (int)wq.w};
      __builtin_amdgcn_sched_barrier(0);
      rb[u] = *reinterpret_cast<const uint4 *>(src(min(i + kD8Ring, L - 1)));
#pragma unroll
      for (int b = 0; b < NRB; ++b) acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[b], bw, acc[b], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ph + 1 < d.nph) sstore(sv, (ph + 1) & 1);
    __syncthreads();
  }
  // outlier steps of this K part, FP16 on fp32 accumulators; both operands
  // are zeroed past the part's share (a zeroed A alone would still let a
  // non-finite weight half through)
  for (int i0 = d.qsteps; i0 < L; i0 += kD8Ring) {
#pragma unroll
    for (int u = 0; u < kD8Ring; ++u) {
      const int i = i0 + u, jo = o0 + i - d.qsteps;
      const uint32_t live = (i < L && jo < d.nk) ? 0xFFFFFFFFu : 0u;
      const uint4 wq = rb[u];
      const uint4 bm = {wq.x & live, wq.y & live, wq.z & live, wq.w & live};
      v8h bo, ao[NRB];
      __builtin_memcpy(&bo, &bm, 16);
#pragma unroll
      for (int b = 0; b < NRB; ++b) {
        const uint4 x = *reinterpret_cast<const uint4 *>(xs + d.xo_base + arow[b] * d.po + 16 * kg +
                                                         64 * max(min(jo, d.nk - 1), 0));
        const uint4 am = {x.x & live, x.y & live, x.z & live, x.w & live};
        __builtin_memcpy(&ao[b], &am, 16);
      }
      __builtin_amdgcn_sched_barrier(0);
      rb[u] = *reinterpret_cast<const uint4 *>(src(min(i + kD8Ring, L - 1)));
#pragma unroll
      for (int b = 0; b < NRB; ++b) fo[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao[b], bo, fo[b], 0, 0, 0);
    }
  }

  // The K parts' partial sums meet in LDS (the stage buffers are free after
  // the last barrier of the phase loop, and the outlier loop reads only
  // x_out, which lies past them); part 0 adds them in part order.
  constexpr int kVals = 8 * NRB;  // int32 acc + fp32 fo per row block, 4 registers each
  uint32_t *red = reinterpret_cast<uint32_t *>(xs);
  if (d.ks > 1) {
    if (ks > 0) {
#pragma unroll
      for (int b = 0; b < NRB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          red[((wave * kVals) + 8 * b + r) * 64 + lane] = (uint32_t)acc[b][r];
          red[((wave * kVals) + 8 * b + 4 + r) * 64 + lane] = __float_as_uint(fo[b][r]);
        }
    }
    __syncthreads();
    if (ks > 0) return;
    for (int q = 1; q < d.ks; ++q) {
      const int w2 = q * d.cb + cbk;
#pragma unroll
      for (int b = 0; b < NRB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[b][r] += (int)red[((w2 * kVals) + 8 * b + r) * 64 + lane];
          fo[b][r] += __uint_as_float(red[((w2 * kVals) + 8 * b + 4 + r) * 64 + lane]);
        }
    }
  }
  if (n0 >= p.N) return;

  // Epilogue: register r of lane (l16, kg), row block b: token 16 b + 4 kg + r,
  // channel n0 + l16.  Unsigned codes went in as u - 128:
  // sum (u - z) w = acc - (z - 128) rowsum.
  constexpr int kZoff = XU ? 128 : 0;
  const int64_t gn = n0 + l16, gnc = min(gn, p.N - 1);
  const int32_t rsn = (XU || (MODE == 2 && p.zx)) ? p.rowsum[gnc] : 0;
  if (MODE == 0) {
    int32_t *out = reinterpret_cast<int32_t *>(p.out);
#pragma unroll
    for (int b = 0; b < NRB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gm = 16 * b + 4 * kg + r;
        if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = acc[b][r] + kZoff * rsn;
      }
    return;
  }
  const float swn = p.sw[gnc];
  __half *out = reinterpret_cast<__half *>(p.out);
#pragma unroll
  for (int b = 0; b < NRB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gm = 16 * b + 4 * kg + r, gmc = min(gm, p.T - 1);
      int32_t v = acc[b][r];
      if (p.zx) v -= (p.zx[gmc] - kZoff) * rsn;
      else if (kZoff) v += kZoff * rsn;
      const float y = (float)v * p.sx[gmc] * swn + fo[b][r];
      if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = __float2half_rn(y);
    }
}

namespace {

// K parts and LDS bytes for a launch; 0 bytes when it does not fit.
D8Args d8_plan(const GemmArgs &p, int mode, size_t &lds) {
  D8Args d{};
  const int64_t nblk = (p.N + 15) / 16;
  const int64_t T = p.T;
  d.ks = nblk >= 2048 ? 1 : nblk >= 1024 ? 2 : 4;
  while (d.ks > 1 && d.ks * T > 64) d.ks /= 2;  // the stage holds at most 64 token rows per phase
  d.cb = kD8Waves / d.ks;
  d.nsteps = (int)(p.Kb / 64);
  const int per = (d.nsteps + d.ks - 1) / d.ks;
  d.qsteps = (per + kD8Ring - 1) / kD8Ring * kD8Ring;
  d.nph = d.qsteps / kD8Ring;
  const int n_out = mode == 2 ? p.n_out : 0;
  d.nk = n_out / 32;
  d.qk = (d.nk + d.ks - 1) / d.ks;
  d.stage = (uint32_t)(d.ks * T * kD8Row);
  d.po = d8_po(n_out);
  const size_t reduce = (size_t)kD8Waves * 8 * (T > 16 ? 2 : 1) * 64 * 4;
  const size_t stages = std::max<size_t>(2 * (size_t)d.stage, reduce);
  d.xo_base = (uint32_t)((stages + 15) & ~(size_t)15);
  lds = d.xo_base + (d.nk ? (size_t)T * d.po : 0);
  if (lds > 160 * 1024) lds = 0;
  return d;
}

}  // namespace

bool gemm_decode8_fits(const GemmArgs &p, int mode) {
  if (p.T < 1 || p.T > 32 || p.Kb % 64 || p.Kb < 64) return false;
  size_t lds = 0;
  d8_plan(p, mode, lds);
  return lds > 0;
}

hipError_t launch_gemm_decode8(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  size_t lds = 0;
  const D8Args d = d8_plan(p, mode, lds);
  if (lds == 0) return hipErrorInvalidValue;
  const int64_t nblk = (p.N + 15) / 16;
  const dim3 grid((unsigned)((nblk + d.cb - 1) / d.cb)), block(512);
  void (*k)(GemmArgs, D8Args);
  if (p.T > 16)
    k = mode == 0 ? (x_unsigned ? gemm_decode8<true, 0, 2> : gemm_decode8<false, 0, 2>)
                  : (x_unsigned ? gemm_decode8<true, 2, 2> : gemm_decode8<false, 2, 2>);
  else
    k = mode == 0 ? (x_unsigned ? gemm_decode8<true, 0, 1> : gemm_decode8<false, 0, 1>)
                  : (x_unsigned ? gemm_decode8<true, 2, 1> : gemm_decode8<false, 2, 1>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k<<<grid, block, lds, st>>>(p, d);
  return hipGetLastError();
}

}  // namespace rq
