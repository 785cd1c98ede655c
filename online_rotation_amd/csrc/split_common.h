// split_common.h -- per-token INT4 quantization of unrotated rows with the
// QUIK outlier split (QUIK blog part 1: asymmetric per-token codes, FP16
// outlier columns), shared by the standalone quantizer and the fused decode
// linear so that both produce the same codes bit for bit.
//
// A row is handled in words of 32 columns (16 dwords of fp16 pairs), with the
// outlier halves of each word zeroed beforehand.  Zeroed outliers leave
// min(min x, 0), max(max x, 0) and the absolute maximum unchanged, so the row
// reductions test no value.
//
// Rounding matches rne(x / s) with s = fp32(S), S the exact real scale
// (clip*amax/7 or (hi - lo)/15), and s is formed as the oracle forms it: the
// numerator clip*amax or hi - lo exactly in fp64, the quotient rounded to
// fp64 and then to fp32.  Write the numerator as an integer of m significant
// bits times a power of two.  With fp16 inputs, x / S then lies either
// exactly on a rounding boundary k + 1/2 or at least 2^-(m+1) (and 2^-17)
// from every boundary, while x * inv, with inv within an ulp of 1/s, differs
// from x / S by less than 2^-18.  So for m <= 16 ("narrow" rows, which
// include every row with a zero bound or clip 1) one fma per value is exact
// except at the exact ties, and there x / s falls on the side that the
// rounding of S to s decides; directed_inv moves the reciprocal by at most
// one ulp so that x * inv lands on that same side.  When S == s the ties are
// real and go to even, and when m > 16 ("wide" rows: a large max beside a
// tiny negative min, or clip ratios below 1) a value may lie closer to a
// boundary than the fma resolves; both take rne_quotient, which tests the
// boundary exactly.
#pragma once
#include "rq_device.h"

namespace rq {

// 1.5 * 2^23: fma(v, inv, kMagic0) = kMagic0 + rne(v*inv) for |v*inv| < 2^22,
// the integer in the low mantissa bits
constexpr float kMagic0 = 12582912.0f;
constexpr float kMagic8 = 12582920.0f;  // kMagic0 + 8

// Reciprocal of s nudged to the side of 1/s on which exact ties must land.
// num / den = S (num exact in fp64, den = 7 or 15); `exact` is set when s == S.
__device__ __forceinline__ float directed_inv(float s, float inv, double num, double den, bool &exact) {
  const double r = __builtin_fma(-den, (double)s, num);  // den*(S - s), exact: den*s has <= 28 bits
  const float e = __builtin_fmaf(-s, inv, 1.0f);         // 1/s - inv, sign exact
  exact = r == 0.0;
  uint32_t bits = __float_as_uint(inv);
  if (r > 0.0f && e > 0.0f) ++bits;       // s < S: ties round away from zero, need inv >= 1/s
  else if (r < 0.0f && e < 0.0f) --bits;  // s > S: ties round toward zero, need inv <= 1/s
  return __uint_as_float(bits);
}

// rne(x / s) exactly, for s > 0: the candidate from x * inv, then the sign of
// x - b s (exact in one fma) at the boundary b on that side.
__device__ __forceinline__ float rne_quotient(float x, float s, float inv) {
  const float t = x * inv;
  const float c = __builtin_rintf(t);
  const bool up = t > c;
  const float b = up ? c + 0.5f : c - 0.5f;
  const float d = __builtin_fmaf(-b, s, x);
  if (d == 0.0f) return __builtin_rintf(b);
  return up ? (d > 0.0f ? c + 1.0f : c) : (d < 0.0f ? c - 1.0f : c);
}

// delete nibble `b` (0..31) of the 128-bit value w (w[0] lowest), shifting the
// higher nibbles down by one
__device__ __forceinline__ void del_nibble(uint32_t *w, int b) {
  const int wi = b >> 3, sh = (b & 7) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t hi_in = i < 3 ? (w[i + 1] << 28) : 0u;
    const uint32_t shifted = (w[i] >> 4) | hi_in;
    if (i > wi) {
      w[i] = shifted;
    } else if (i == wi) {
      const uint32_t keep = sh ? ((1u << sh) - 1u) : 0u;
      w[i] = (w[i] & keep) | (shifted & ~keep);
    }
  }
}

// AND mask for dword i of a word whose outlier columns are the bits of m
__device__ __forceinline__ uint32_t keep_mask(uint32_t m, int i) {
  return (((m >> (2 * i)) & 1u) ? 0u : 0x0000FFFFu) | (((m >> (2 * i + 1)) & 1u) ? 0u : 0xFFFF0000u);
}

// Fold 16 dwords of fp16 pairs into running min / max (or |.| max when symmetric).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void word_minmax(const uint32_t *d, bool asym, f16x2 &mn2, f16x2 &mx2) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f16x2 h;
    __builtin_memcpy(&h, &d[i], 4);
    if (!asym) h = __builtin_elementwise_abs(h);
    mn2 = __builtin_elementwise_min(mn2, h);
    mx2 = __builtin_elementwise_max(mx2, h);
  }
}

// A value equal in every lane, marked so for the compiler (the row's
// parameters then live in scalar registers and the rare exact-tie path is a
// scalar branch rather than a per-value select).
__device__ __forceinline__ float wave_uniform(float v) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

// One row's quantizer: scale, zero point and the magic-number form of the codes.
struct RowQuant {
  float s, inv, base, lo_c, hi_c;
  int zp;
  bool exact;  // s == S: exact ties are real ties
  bool wide;   // the numerator of S has more than 16 significant bits
};

// More than 16 significant bits in a finite double: a set bit among the 37
// lowest of its 52 stored fraction bits.
__device__ __forceinline__ bool wide_significand(double v) {
  return (__double_as_longlong(v) & ((1ll << 37) - 1)) != 0;
}

// From the row's min and max (asymmetric: lo = min(mn, 0), hi = max(mx, 0);
// symmetric: mx = max |x|, scale clip * mx / 7).  The numerator is exact in
// fp64 (fp16 bounds span at most 40 bits; clip * mx has at most 35).
__device__ __forceinline__ RowQuant row_quant(bool asym, float clip, float mn, float mx) {
  RowQuant r;
  r.zp = 0;
  r.exact = false;
  r.wide = false;
  if (asym) {
    const float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
    const double range = (double)hi - (double)lo;
    r.s = (float)(range / 15.0);
    r.inv = r.s > 0.0f ? 1.0f / r.s : 0.0f;
    if (r.s > 0.0f) {
      r.inv = directed_inv(r.s, r.inv, range, 15.0, r.exact);
      r.wide = wide_significand(range);
      const float zf = (r.exact || r.wide) ? rne_quotient(-lo, r.s, r.inv)
                                           : __builtin_fmaf(-lo, r.inv, kMagic0) - kMagic0;
      r.zp = (int)__builtin_amdgcn_fmed3f(zf, 0.0f, 15.0f);
    }
    r.base = kMagic0 + (float)r.zp;  // code = clamp(rne(x/s) + zero, 0, 15)
    r.lo_c = kMagic0;
    r.hi_c = kMagic0 + 15.0f;
  } else {
    sym_scale(mx, clip, r.s, r.inv);
    if (r.s > 0.0f) {
      const double num = (double)clip * (double)mx;
      r.inv = directed_inv(r.s, r.inv, num, 7.0, r.exact);
      r.wide = wide_significand(num);
    }
    r.base = kMagic8;  // low nibble = code + 8
    r.lo_c = kMagic8 - 7.0f;
    r.hi_c = kMagic8 + 7.0f;
  }
  return r;
}

// Quantize one word (16 dwords of fp16 pairs, outlier halves zeroed), delete
// the nibbles of its outlier columns m and OR the remaining run of 32 -
// popc(m) codes into the packed row `packed` (32-bit words, LDS) at nibble
// position pos.  Returns the sum of the word's normal-column codes.
__device__ __forceinline__ int quant_word(const uint32_t *d, uint32_t m, int pos, bool asym,
                                          const RowQuant &rq, uint32_t *packed) {
  uint32_t w[4];
  uint32_t nsum = 0;  // sum of the 32 nibbles (outliers, zeroed, included)
  // codes eight at a time: biased code bits whose low byte is the nibble
  // (asymmetric code, or symmetric code + 8), higher bits 0; packed by byte
  // permutes, e = [n0, n2, n4, n6] and o = [n1, n3, n5, n7], nibble k = value k
  auto pack = [&](auto code) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t b[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 f = __half22float2(*reinterpret_cast<const __half2 *>(&d[4 * i + k]));
        b[2 * k] = __float_as_uint(__builtin_amdgcn_fmed3f(code(f.x), rq.lo_c, rq.hi_c));
        b[2 * k + 1] = __float_as_uint(__builtin_amdgcn_fmed3f(code(f.y), rq.lo_c, rq.hi_c));
      }
      const uint32_t e = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[6], b[4], 0x04000C0Cu);
      const uint32_t o = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0400u) | __builtin_amdgcn_perm(b[7], b[5], 0x04000C0Cu);
      const uint32_t wd = (o << 4) | e;
      nsum = __builtin_amdgcn_udot8(wd, 0x11111111u, nsum, false);
      w[i] = asym ? wd : (wd ^ 0x88888888u);  // symmetric: offset-8 nibble -> two's complement
    }
  };
  // Rows with exact ties or a wide numerator (rq.exact, rq.wide, uniform)
  // take the exact quotient, the rest one fma.  The exact path is rare: its
  // loop stays rolled so that it does not set the kernel's register budget.
  if (rq.exact || rq.wide) {
    uint32_t dl[16], q[16];  // a private copy: the rolled loop indexes it
#pragma unroll
    for (int k = 0; k < 16; ++k) dl[k] = d[k];
#pragma unroll 1
    for (int k = 0; k < 16; ++k) {
      const float2 f = __half22float2(*reinterpret_cast<const __half2 *>(&dl[k]));
      const float c0 = __builtin_amdgcn_fmed3f(rne_quotient(f.x, rq.s, rq.inv) + rq.base, rq.lo_c, rq.hi_c);
      const float c1 = __builtin_amdgcn_fmed3f(rne_quotient(f.y, rq.s, rq.inv) + rq.base, rq.lo_c, rq.hi_c);
      q[k] = (__float_as_uint(c0) & 0xFu) | ((__float_as_uint(c1) & 0xFu) << 4);  // byte k%4 of dword k/4
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wd = q[4 * i] | (q[4 * i + 1] << 8) | (q[4 * i + 2] << 16) | (q[4 * i + 3] << 24);
      nsum = __builtin_amdgcn_udot8(wd, 0x11111111u, nsum, false);
      w[i] = asym ? wd : (wd ^ 0x88888888u);
    }
  } else {
    pack([&](float f) { return __builtin_fmaf(f, rq.inv, rq.base); });
  }
  // the run of this word's normal-column codes, outliers deleted
  uint32_t mm = m;
  while (mm) {
    const int b = 31 - __clz(mm);  // highest first, so lower positions stay put
    del_nibble(w, b);
    mm &= ~(1u << b);
  }
  const int cj = __popc(m);
  // place the run (32 - cj nibbles) at nibble position pos
  const int sh = (pos & 7) * 4, w0i = pos >> 3;
  const int nrun = 32 - cj;
  if (nrun < 32) {  // clear the nibbles past the run
    const int wi = nrun >> 3, bi = (nrun & 7) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i > wi) w[i] = 0u;
      else if (i == wi) w[i] &= bi ? ((1u << bi) - 1u) : 0u;
    }
  }
  uint32_t out[5];
  out[0] = w[0] << sh;
#pragma unroll
  for (int i = 1; i < 4; ++i) out[i] = (w[i] << sh) | (sh ? (w[i - 1] >> (32 - sh)) : 0u);
  out[4] = sh ? (w[3] >> (32 - sh)) : 0u;
#pragma unroll
  for (int i = 0; i < 5; ++i)
    if (out[i]) atomicOr(&packed[w0i + i], out[i]);
  // a zeroed outlier's nibble is the zero point (asymmetric) or 8 (symmetric, code 0)
  return asym ? (int)nsum - rq.zp * cj : (int)nsum - 8 * 32;
}

}  // namespace rq
