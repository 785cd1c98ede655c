// kv_quant.hip -- the KV-cache path: R3, a normalized Walsh-Hadamard over the
// channels of each head (SpinQuant OpenReview: the authors' answer on the
// number of rotation matrices, R3 rotates the KV cache before its
// quantization; first reviewer Q2/A2, (W_q R3)(W_k R3)^T = W_q W_k^T),
// then group-wise asymmetric INT4 with one scale and zero point per group of
// channels (FlatQuant article, section 3 quantization setting: KV cache
// group-wise asymmetric, g = 128).
//
// A group of g = 4V channels lives in one lane quad, V consecutive values per
// lane.  The Walsh-Hadamard of natural order factors over the index bits:
// two of its bits select the lane in the quad (DPP quad permutations, no
// LDS), the others are register butterflies within the lane.  The
// transform runs unnormalized in fp32 and is scaled by 1/sqrt(g) once; the
// quad's min / max then give the group's asymmetric scale and zero point
// with the arithmetic of the per-token quantizer (split_common.h), and each
// lane packs its V codes into V/8 dwords.
#include "rq_device.h"
#include "rq_kernels.h"
#include "split_common.h"

namespace rq {

namespace {
// v from lane (lane ^ 1) or (lane ^ 2) of the quad
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
}
}  // namespace

// Group sets: a wavefront takes 16 consecutive groups (one per quad) at a
// time, in a grid-stride loop that loads the next set before it works on the
// current one.  The position (row t0, group column c0) of a set's first group
// is carried from set to set; a quad's own group is c0 + quad, wrapped into
// later rows by a 32-bit reciprocal division.
struct KvArgs {
  const __half *x;
  int64_t ldx;
  uint8_t *q;
  float *scale;
  int32_t *zero;
  int64_t T, total;      // rows, groups (T * gpr)
  int64_t step;          // groups per grid step (16 per wavefront)
  int64_t step_rows;     // step = step_rows * gpr + step_cols
  int32_t step_cols;
  int32_t gpr;           // groups per row
  uint32_t gpr_magic;    // floor((2^32 - 1) / gpr) + 1: n / gpr = umulhi(n, magic) for n * gpr < 2^32
  float norm;            // fp32(1 / sqrt(group))
};

template <int V, bool ROT>
__global__ __launch_bounds__(256) void group_quant(KvArgs a) {
  constexpr int G = 4 * V;   // channels per group
  constexpr int NC = V / 8;  // 16-byte chunks per lane
  const int lane = threadIdx.x & 63, sub = lane & 3, quad = lane >> 2;
  const uint32_t w0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  int64_t gb = (int64_t)w0 * 16;  // first group of the current set
  if (gb >= a.total) return;      // whole wavefront
  int64_t t0 = (uint32_t)gb / (uint32_t)a.gpr;
  int32_t c0 = (int32_t)(gb - t0 * a.gpr);

  // Lane `sub` of a quad holds channels 32c + 8 sub + e (chunk c, element e)
  // of its group: each load instruction reads 64 contiguous bytes per quad;
  // index bits 0-2 and 5.. are in registers, bits 3-4 in the lane.
  auto locate = [&](int64_t gset, int64_t tr, int32_t cc, int64_t &t, int32_t &gc) -> bool {
    const uint32_t n = (uint32_t)cc + quad;
    const uint32_t dq = a.gpr == 1 ? n : __umulhi(n, a.gpr_magic);
    t = tr + dq;
    gc = (int32_t)(n - dq * (uint32_t)a.gpr);
    const bool valid = gset + quad < a.total;
    if (!valid) {  // past the last group: reread it, store nothing
      t = a.T - 1;
      gc = a.gpr - 1;
    }
    return valid;
  };
  auto load = [&](uint4 *r, int64_t t, int32_t gc) {
    const __half *src = a.x + t * a.ldx + (int64_t)gc * G + 8 * sub;
#pragma unroll
    for (int c = 0; c < NC; ++c) r[c] = load_nt(src + 32 * c);
  };

  // Cross-lane butterflies store sigma * value with sigma = (-1)^popcount(sub),
  // each one fma with the partner; fin = sigma / sqrt(group) restores the value.
  const float c1 = (sub & 1) ? -1.0f : 1.0f, c2 = (sub & 2) ? -1.0f : 1.0f;
  const float fin = ROT ? c1 * c2 * a.norm : 1.0f;

  int64_t t;
  int32_t gc;
  bool valid = locate(gb, t0, c0, t, gc);
  uint4 cur[NC];
  load(cur, t, gc);
  for (;;) {
    // the next set, or (past the end) the current one again, an L2 hit:
    // unconditional, so that waiting for the current set never waits for it
    const int64_t gbn = gb + a.step;
    int64_t t0n = t0 + a.step_rows;
    int32_t c0n = c0 + a.step_cols;
    if (c0n >= a.gpr) {
      c0n -= a.gpr;
      ++t0n;
    }
    const bool more = gbn < a.total;
    int64_t tn;
    int32_t gcn;
    const bool validn = more ? locate(gbn, t0n, c0n, tn, gcn) : (tn = t, gcn = gc, false);
    uint4 nxt[NC];
    load(nxt, tn, gcn);

    float v[V];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t w[4] = {cur[c].x, cur[c].y, cur[c].z, cur[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 f = __half22float2(*reinterpret_cast<const __half2 *>(&w[e]));
        v[8 * c + 2 * e] = f.x;
        v[8 * c + 2 * e + 1] = f.y;
      }
    }
    if (ROT) {
      // y_j = sum_i x_i (-1)^popcount(i & j): one butterfly stage per index bit
#pragma unroll
      for (int h = 1; h < V; h <<= 1)
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (!(i & h)) {
            const float p = v[i], r = v[i + h];
            v[i] = p + r;
            v[i + h] = p - r;
          }
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = __builtin_fmaf(quad_xor1(v[i]), c1, v[i]);
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = __builtin_fmaf(quad_xor2(v[i]), c2, v[i]);
    }
    // the group's min and max over the quad (0 included, as the quantizer's
    // range); the stored values times fin are the group's values, so lanes
    // with fin < 0 swap their minimum and maximum
    float mn = 0.0f, mx = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      mn = fminf(mn, v[i]);
      mx = fmaxf(mx, v[i]);
    }
    if (ROT) {
      const float lo = (fin > 0.0f ? mn : mx) * fin, hi = (fin > 0.0f ? mx : mn) * fin;
      mn = lo;
      mx = hi;
    }
    mn = fminf(mn, quad_xor1(mn));
    mx = fmaxf(mx, quad_xor1(mx));
    mn = fminf(mn, quad_xor2(mn));
    mx = fmaxf(mx, quad_xor2(mx));
    const RowQuant rq = row_quant(true, 1.0f, mn, mx);
    // codes eight to a dword, nibble e = channel 32c + 8 sub + e; the byte
    // permutes gather the low bytes (the nibbles) of the magic-biased floats
    uint32_t wd[NC];
    auto pack = [&](auto code) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t b[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) b[k] = __float_as_uint(__builtin_amdgcn_fmed3f(code(v[8 * c + k]), rq.lo_c, rq.hi_c));
        const uint32_t e = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[6], b[4], 0x04000C0Cu);
        const uint32_t o = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0400u) | __builtin_amdgcn_perm(b[7], b[5], 0x04000C0Cu);
        wd[c] = (o << 4) | e;
      }
    };
    if (__builtin_amdgcn_ballot_w64(rq.exact) == 0) {
      const float coef = fin * rq.inv;
      pack([&](float f) { return __builtin_fmaf(f, coef, rq.base); });
    } else {
      // Some group's scale is exact (s equals the real (hi - lo)/15), so its
      // ties x/s = k + 1/2 are real and go to even.  With the two fp32
      // neighbours of 1/s, the magic-number products give the same integer
      // away from a tie and k, k + 1 at it; their sum lies where fp32 steps
      // by 2, so rounding it keeps the even of the two, and one fma halves
      // it and adds the zero point.  Groups with an inexact scale use their
      // directed reciprocal twice.
      float lo_inv = rq.inv, hi_inv = rq.inv;
      if (rq.exact) {
        const float e = __builtin_fmaf(-rq.s, rq.inv, 1.0f);  // sign of 1/s - inv, exact
        if (e > 0.0f) hi_inv = __uint_as_float(__float_as_uint(rq.inv) + 1u);
        if (e < 0.0f) lo_inv = __uint_as_float(__float_as_uint(rq.inv) - 1u);
      }
      const float ca = fin * lo_inv, cb = fin * hi_inv, zf = (float)rq.zp;
      pack([&](float f) {
        return __builtin_fmaf(__builtin_fmaf(f, ca, kMagic0) + __builtin_fmaf(f, cb, kMagic0), 0.5f, zf);
      });
    }
    if (valid) {
      uint32_t *dst = reinterpret_cast<uint32_t *>(a.q + t * (a.gpr * (int64_t)(G / 2)) + (int64_t)gc * (G / 2)) + sub;
#pragma unroll
      for (int c = 0; c < NC; ++c) store_nt(dst + 4 * c, wd[c]);
      if (sub == 0) {
        const int64_t gi = t * a.gpr + gc;
        a.scale[gi] = rq.s;
        a.zero[gi] = rq.zp;
      }
    }
    if (!more) break;
#pragma unroll
    for (int c = 0; c < NC; ++c) cur[c] = nxt[c];
    gb = gbn;
    t0 = t0n;
    c0 = c0n;
    t = tn;
    gc = gcn;
    valid = validn;
  }
}

// grid: two wavefronts per SIMD of the 256 compute units, each with one set
// in flight ahead of the one in work
constexpr int kKvWaves = 256 * 4 * 2;

hipError_t launch_group_quant(const void *x, int64_t T, int64_t K, int64_t ldx, int group, bool rotate,
                              uint8_t *q, float *scale, int32_t *zero, hipStream_t st) {
  KvArgs a;
  a.x = (const __half *)x;
  a.ldx = ldx;
  a.q = q;
  a.scale = scale;
  a.zero = zero;
  a.T = T;
  a.gpr = (int32_t)(K / group);
  a.total = T * a.gpr;
  a.gpr_magic = (uint32_t)(0xFFFFFFFFu / (uint32_t)a.gpr) + 1u;
  a.norm = 1.0f / sqrtf((float)group);
  const int64_t sets = (a.total + 15) / 16;
  const int64_t waves = std::min<int64_t>(sets, kKvWaves);
  const int64_t blocks = (waves + 3) / 4;
  a.step = blocks * 4 * 16;
  a.step_rows = a.step / a.gpr;
  a.step_cols = (int32_t)(a.step - a.step_rows * a.gpr);
  const dim3 g((unsigned)blocks), b(256);
  switch (group * 2 + (rotate ? 1 : 0)) {
    case 64 * 2: group_quant<16, false><<<g, b, 0, st>>>(a); break;
    case 64 * 2 + 1: group_quant<16, true><<<g, b, 0, st>>>(a); break;
    case 128 * 2: group_quant<32, false><<<g, b, 0, st>>>(a); break;
    case 128 * 2 + 1: group_quant<32, true><<<g, b, 0, st>>>(a); break;
    case 256 * 2: group_quant<64, false><<<g, b, 0, st>>>(a); break;
    case 256 * 2 + 1: group_quant<64, true><<<g, b, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rq
