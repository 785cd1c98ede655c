// fwht_common.h -- the 4096-point Walsh-Hadamard and GSR transforms on FP16
// matrix cores with the per-token symmetric INT4 quantizer (internal), shared
// by the standalone quantizer (rotate_quant.hip) and the fused decode form
// (gemm_decode.hip) so that both produce the same codes bit for bit.
#pragma once
#include "rq_device.h"
#include "split_common.h"

namespace rq {

typedef uint32_t v4w __attribute__((ext_vector_type(4)));  // a register vector, not a struct

// ---------------------------------------------------------------------------
// fwht4096_mfma: the same transforms on FP16 matrix cores.
//
// A 4096-wide row viewed as M[a][b] = x[64a + b] (64 x 64).  Since
// H_4096 = H_64 kron H_64, x . H_4096 / 64 = H_64 . M . H_64 / 64, two 64^3
// products; a GSR row with blocks of B <= 64 is the single product M . G,
// G = blockdiag(Wal_B).  Both run on v_mfma_f32_32x32x16_f16:
//   - the fp16 input is exact as an MFMA operand and +-2^k are exact fp16
//     values, so the first product only rounds in its fp32 accumulation;
//   - the second Hadamard product takes its fp32 input as hi + lo fp16
//     (hi rounded to nearest, lo the remainder), 2^-22 relative.  So that lo
//     never falls into fp16 subnormals, the first product is scaled by a
//     per-row power of two chosen from the exponent of max|x| (exact), which
//     puts the largest intermediate just below 2^15; the quantizer divides
//     it out again (exact).
// Constant operands are +-1 sign images (16 bytes per lane) made in the kernel,
// staged in LDS once per workgroup.  Up to 2048 tokens, one wavefront per
// token; beyond, each wavefront takes an even number of tokens and loads the
// next one while it computes the current one.
// Output layout (both cases): accumulator [mb][nb] register r of lane
// (r32, g) holds element 64*(r32 + 32*nb) + 32*mb + 8*(r/4) + 4*g + r%4,
// so four consecutive elements share a lane and a lane pair (l, l+32)
// swaps halves (v_permlane32_swap) into 16 contiguous packed bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v8h as_h8(uint4 u) {
  v8h h;
  __builtin_memcpy(&h, &u, 16);
  return h;
}

__device__ __forceinline__ v16f mfma16(uint4 a, uint4 b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(a), as_h8(b), c, 0, 0, 0);
}

// Split eight fp32 values into fp16 hi (nearest) and lo (remainder) operands.
// hi is one v_cvt_pk_f16_f32 per pair (round to nearest even); the remainder
// f - hi is exact in fp32 and comes from one mixed-precision fma per value
// (the fp16 operand widened inside the fma) that rounds it to fp16 in the
// same instruction.  `neg1` is -1.0 held in a register the compiler cannot
// see through: with a literal -1 the fma folds to a subtraction that needs a
// separate fp16 -> fp32 conversion of hi.
__device__ __forceinline__ void split8(const float *f, uint4 &hi, uint4 &lo, float neg1) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2 ab = __builtin_convertvector((f2){f[2 * j], f[2 * j + 1]}, h2);
    // each remainder rounded to fp16 straight from the fma (v_fma_mixlo /
    // v_fma_mixhi write the two halves of one register)
    h2 lr;
    lr.x = (_Float16)__builtin_fmaf((float)ab.x, neg1, f[2 * j]);
    lr.y = (_Float16)__builtin_fmaf((float)ab.y, neg1, f[2 * j + 1]);
    __builtin_memcpy(&h[j], &ab, 4);
    __builtin_memcpy(&l[j], &lr, 4);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_max_bits(v); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));


// kMagic8 (split_common.h) = 1.5 * 2^23 + 8: fma(v, inv, kMagic8) = kMagic8 +
// rne(v*inv) for |v*inv| < 2^22, so the low nibble of the result's bit
// pattern is the code + 8.

// Stage slot of row a, 16-byte column j (see fwht_token).
__device__ __forceinline__ int fwht_swz(int a, int j) { return a * 8 + (j ^ ((a >> 1) & 7)); }

// Operand images (16 bytes per lane: 8 fp16 values), made in the kernel from
// their formulas (no memory access, so a workgroup's set-up waits on
// nothing; loaded from global tables at kernel start they queued behind the
// tokens' loads and took 1.5 us at the median):
//   Hadamard step 1, B = H_64, operand op = 4 cb + kc of lane (r32, g):
//     column b' = r32 + 32 cb, slot s is row b = 16 kc + 8 g + s; only the
//     sign bits (the kernel ORs in a per-row magnitude);
//   Hadamard step 2, B = H_64 (+-1), operand 8 + (2 nb + rb) 2 + c: column
//     a' = r32 + 32 nb, slot s is row a = 32 rb + 16 c + 8 (s / 4) + 4 g +
//     s % 4, the row the step-1 accumulator register 8 c + s of that lane
//     holds;
//   GSR, A = G^T with G = blockdiag(Wal_B), operand op = 4 mb + kc: output
//     j = r32 + 32 mb, slot s is input b = 16 kc + 8 g + s; G[b][j] =
//     H_B[sigma(b % B)][j % B] inside a block (sigma = bitrev o gray: row
//     sigma(s) of H_B has s sign changes), 0 across blocks.
// H_64[x][y] = (-1)^popcount(x & y).
template <bool GSR>
__device__ __forceinline__ uint4 tab_entry(int op, int l, int blog2) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint32_t v;
    if (GSR) {
      const uint32_t bm = (1u << blog2) - 1u;
      const uint32_t j = (uint32_t)(l & 31) + 32u * (uint32_t)(op >> 2);
      const uint32_t b = 16u * (uint32_t)(op & 3) + 8u * (uint32_t)(l >> 5) + (uint32_t)s;
      const uint32_t bl = b & bm, sig = __builtin_bitreverse32(bl ^ (bl >> 1)) >> (32 - blog2);
      v = (b >> blog2) == (j >> blog2) ? 0x3C00u | ((uint32_t)(__builtin_popcount(sig & j & bm) & 1) << 15) : 0u;
    } else if (op < 8) {
      const uint32_t col = (uint32_t)(l & 31) + 32u * (uint32_t)(op >> 2);
      const uint32_t b = 16u * (uint32_t)(op & 3) + 8u * (uint32_t)(l >> 5) + (uint32_t)s;
      v = (uint32_t)(__builtin_popcount(b & col) & 1) << 15;
    } else {
      const int o = op - 8, nb = o >> 2, rb = (o >> 1) & 1, c = o & 1;
      const uint32_t col = (uint32_t)(l & 31) + 32u * (uint32_t)nb;
      const uint32_t a = 32u * rb + 16u * c + 8u * (uint32_t)(s >> 2) + 4u * (uint32_t)(l >> 5) + (uint32_t)(s & 3);
      v = 0x3C00u | ((uint32_t)(__builtin_popcount(a & col) & 1) << 15);
    }
    w[s >> 1] |= v << (16 * (s & 1));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// All operand images into LDS (8 operands for GSR, 16 for the Hadamard), by
// the nthreads threads of the workgroup.
template <bool GSR>
__device__ __forceinline__ void fwht_make_tables(uint4 (*ltab)[64], int blog2, int tid, int nthreads) {
  constexpr int nop = GSR ? 8 : 16;
  for (int e = tid; e < nop * 64; e += nthreads) ltab[e >> 6][e & 63] = tab_entry<GSR>(e >> 6, e & 63, blog2);
}

struct FwhtOut {
  v4w code[2];
  float s;
  int csum;
};

// One token through the transform and the quantizer: raw holds the token's
// 8 KB as loaded (load c, lane l: bytes 1024c + 16l), st is the wavefront's
// 4 KB LDS stage, ltab the operand tables (fwht_make_tables).  Returns the
// lane's 32 bytes of packed codes (code bytes 32 (r32 + 32 nb) + 16 g, nb =
// 0, 1), the scale and, with CSUM, the token's code sum.
template <bool GSR, bool CSUM, bool CLAMP>
__device__ __forceinline__ FwhtOut fwht_token(const v4w (&raw)[8], v4w *st, const uint4 (*ltab)[64], float norm,
                                            float clip) {
  const int lane = threadIdx.x & 63, r32 = lane & 31, g = lane >> 5;
  FwhtOut out;
  out.csum = 0;
  uint4 mop[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int c = 0; c < 4; ++c) st[fwht_swz(8 * c + (lane >> 3), lane & 7)] = raw[4 * rb + c];
    wave_lds_sync();
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const v4w v = st[fwht_swz(r32, 2 * kc + g)];
      mop[rb][kc] = make_uint4(v.x, v.y, v.z, v.w);
    }
    wave_lds_sync();  // the stage is free again once these reads are done
  }
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  float nrm = norm;

  if (GSR) {
    // C[j][a] = sum_b G[b][j] M[a][b]: A = G^T (table), B = M (column a = lane).
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint4 a = ltab[mb * 4 + kc][lane];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma16(a, mop[nb][kc], acc[mb][nb]);
      }
  } else {
    // per-row scale 2^sx: step-1 operand magnitude 2^(te-15), te = min(38 - e, 30)
    // with e the fp16 exponent field of max|x|, so |P * 2^sx| < 2^15.
    uint32_t mx = 0;
    {
      // max |x| as max(max x, -min x): three-input packed fp16 maximum /
      // minimum over the raw pairs, two chains each (a NaN carries through
      // and, like an infinity, gives exponent field 31)
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      h2 v[32];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) __builtin_memcpy(&v[16 * rb + 4 * kc], &mop[rb][kc], 16);
      h2 hx[2], hn[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        hx[c] = hn[c] = v[16 * c];
#pragma unroll
        for (int i = 1; i < 16; i += 2) {
          const int j = 16 * c + i;
          const int k = i + 1 < 16 ? j + 1 : j;
          hx[c] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(hx[c], v[j]), v[k]);
          hn[c] = __builtin_elementwise_minimum(__builtin_elementwise_minimum(hn[c], v[j]), v[k]);
        }
      }
      const h2 m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(hx[0], hx[1]),
                                                 -__builtin_elementwise_minimum(hn[0], hn[1]));
      uint32_t mb;
      __builtin_memcpy(&mb, &m, 4);
      mx = wave_max_u32(max(mb & 0x7FFFu, (mb >> 16) & 0x7FFFu));
    }
    float neg1 = -1.0f;
    asm volatile("" : "+v"(neg1));
    const int e = (int)((mx >> 10) & 0x1Fu);
    const int te = min(38 - e, 30);
    const uint32_t mag = (uint32_t)te << 10, magd = mag | (mag << 16);
    nrm = __builtin_ldexpf(1.0f, 9 - te);  // undoes 2^(te - 9)
    // step 1: P = M . H_64 * 2^(te-15), lanes <-> column b', registers <-> row a
    v16f p[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[rb][cb][r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        uint4 hb = ltab[cb * 4 + kc][lane];
        hb.x |= magd;
        hb.y |= magd;
        hb.z |= magd;
        hb.w |= magd;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) p[rb][cb] = mfma16(mop[rb][kc], hb, p[rb][cb]);
      }
    }
    // step 2: Y^T[b'][a'] = sum_a P[a][b'] H_64[a][a'] with A = P^T taken
    // straight from the step-1 accumulators.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float f[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) f[s] = p[rb][mb][8 * c + s];
          uint4 hi, lo;
          split8(f, hi, lo, neg1);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const uint4 hb = ltab[8 + (nb * 2 + rb) * 2 + c][lane];
            acc[mb][nb] = mfma16(hi, hb, acc[mb][nb]);
            acc[mb][nb] = mfma16(lo, hb, acc[mb][nb]);
          }
        }
      }
    }
  }

  // per-row symmetric scale from the normalized absmax
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[i][j][r]));
  amax = __uint_as_float(wave_max_bits(__float_as_uint(amax))) * nrm;  // amax >= 0
  float s, inv;
  sym_scale(amax, clip, s, inv);
  const float invn = inv * nrm;
  const float lo_c = kMagic8 - 7.0f, hi_c = kMagic8 + 7.0f;
  float csum = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    uint32_t d[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      uint32_t h[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        uint32_t bits[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float f = __builtin_fmaf(acc[mb][nb][4 * j4 + i], invn, kMagic8);
          if (CLAMP) f = __builtin_amdgcn_fmed3f(f, lo_c, hi_c);
          if (CSUM) csum += f - kMagic8;
          __builtin_memcpy(&bits[i], &f, 4);
        }
        // low byte of bits[i] is code+8 in [1, 15]; pack pairs, then bytes
        const uint32_t p01 = (bits[1] << 4) | bits[0];
        const uint32_t p23 = (bits[3] << 4) | bits[2];
        h[mb] = __builtin_amdgcn_perm(p23, p01, 0x0C0C0400u);
      }
      auto sw = __builtin_amdgcn_permlane32_swap(h[0], h[1], false, false);
      d[j4] = ((uint32_t)sw[0] | ((uint32_t)sw[1] << 16)) ^ 0x88888888u;  // offset -> two's complement
    }
    out.code[nb] = (v4w){d[0], d[1], d[2], d[3]};
  }
  if (CSUM) out.csum = wave_sum((int)csum);
  out.s = s;
  return out;
}


}  // namespace rq
