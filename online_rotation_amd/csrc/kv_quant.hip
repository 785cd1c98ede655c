// kv_quant.hip -- the KV-cache path: R3, a normalized Walsh-Hadamard over the
// channels of each head (SpinQuant OpenReview: the authors' answer on the
// number of rotation matrices, R3 rotates the KV cache before its
// quantization; first reviewer Q2/A2, (W_q R3)(W_k R3)^T = W_q W_k^T),
// then group-wise asymmetric INT4 with one scale and zero point per group of
// channels (FlatQuant article, section 3 quantization setting: KV cache
// group-wise asymmetric, g = 128).
//
// A group of g = 4V channels lives in one lane quad, V values per lane.  The
// Walsh-Hadamard of natural order factors over the index bits:
// two of its bits select the lane in the quad (DPP quad permutations, no
// LDS), the others are register butterflies within the lane.  The
// transform runs unnormalized in fp64, where it is exact: every fp16 value
// is an integer multiple of 2^-24 below 2^16, so a signed sum of at most 256
// of them is an integer multiple of 2^-24 below 2^48.  The sums are scaled
// by 1/sqrt(g) and rounded to fp32 once, so each value is within 2^-23
// (relative) of the exact rotation; the quad's min / max then give the
// group's asymmetric scale and zero point with the arithmetic of the
// per-token quantizer (split_common.h), and each lane packs its V codes into
// V/8 dwords.  The keys and values of the same tokens can share one launch:
// per set, the rotated tensor's arithmetic then overlaps the other tensor's
// loads, and the second launch's fixed cost is saved.
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
// the same for an fp64 value, one dword at a time
template <int CTRL>
__device__ __forceinline__ double quad_perm64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
}  // namespace

// Group sets: a wavefront takes 16 consecutive groups (one per quad) at a
// time, in a grid-stride loop.  The position (row t0, group column c0) of a
// set's first group is carried from set to set; a quad's own group is
// c0 + quad, wrapped into later rows by a 32-bit reciprocal division.
struct KvArgs {
  KvTensor ten[2];       // one tensor, or keys and values of the same tokens
  int64_t T, total;      // rows, groups (T * gpr)
  int64_t step;          // groups per grid step (16 per wavefront)
  int64_t step_rows;     // step = step_rows * gpr + step_cols
  int32_t step_cols;
  int32_t gpr;           // groups per row
  uint32_t gpr_magic;    // floor((2^32 - 1) / gpr) + 1: n / gpr = umulhi(n, magic) for n * gpr < 2^32
  int32_t vec_store;     // every code buffer 16-byte aligned: codes leave as 16-byte stores
  double norm;           // fp64(1 / sqrt(group))
};

namespace {

template <int V>
struct KvLane {
  static constexpr int G = 4 * V;   // channels per group
  static constexpr int NC = V / 8;  // 16-byte chunks per lane
  // Rotated groups of 128 or more channels leave the transform with each
  // lane holding V contiguous output channels (see quant); smaller ones
  // keep the loaded layout.
  static constexpr bool kSwapOut = NC >= 4;
  int sub, quad;
  double c1, c2, fin;
  __device__ KvLane(const KvArgs &a) {
    const int lane = threadIdx.x & 63;
    sub = lane & 3;
    quad = lane >> 2;
    c1 = (sub & 1) ? -1.0 : 1.0;
    c2 = (sub & 2) ? -1.0 : 1.0;
    // In the loaded layout the cross-lane butterflies store sigma * value
    // with sigma = (-1)^popcount(sub), each one fma with the partner; fin =
    // sigma / sqrt(group) restores the value.
    fin = kSwapOut ? a.norm : c1 * c2 * a.norm;
  }
  // bit-reversed chunk index (log2(NC) bits): the output position of the
  // lane's chunk c after the exchanging transform
  static __device__ constexpr int chunk_out(int c) {
    int r = 0;
    for (int b = 1, rb = NC >> 1; b < NC; b <<= 1, rb >>= 1)
      if (c & b) r |= rb;
    return r;
  }
  // Row and group column of this quad's group in the set that starts at
  // group gset (row tr, column cc); false past the last group, where the
  // quad rereads the last group and stores nothing.
  __device__ bool locate(const KvArgs &a, int64_t gset, int64_t tr, int32_t cc, int64_t &t, int32_t &gc) const {
    const uint32_t n = (uint32_t)cc + quad;
    const uint32_t dq = a.gpr == 1 ? n : __umulhi(n, a.gpr_magic);
    t = tr + dq;
    gc = (int32_t)(n - dq * (uint32_t)a.gpr);
    const bool valid = gset + quad < a.total;
    if (!valid) {
      t = a.T - 1;
      gc = a.gpr - 1;
    }
    return valid;
  }
  // Lane `sub` of a quad holds channels 32c + 8 sub + e (chunk c, element e)
  // of its group: each load instruction reads 64 contiguous bytes per quad;
  // index bits 0-2 and 5.. are in registers, bits 3-4 in the lane.
  __device__ void load(uint4 *r, const KvTensor &x, int64_t t, int32_t gc) const {
    const __half *src = x.x + t * x.ldx + (int64_t)gc * G + 8 * sub;
#pragma unroll
    for (int c = 0; c < NC; ++c) r[c] = load_nt(src + 32 * c);
  }

  // Transform (ROT), quantize and store one set.
  template <bool ROT>
  __device__ void quant(const KvArgs &a, const uint4 *cur, const KvTensor &o, int64_t t, int32_t gc,
                        bool valid) const {
    // the lane's values as loaded (fp16 pairs) and, rotated, the transform's
    // fp32 results; unrotated values are widened where they are used (the
    // min / max run on the fp16 pairs, the codes' fma takes fp16 operands)
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 hv[V / 2];
    float v[V];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t w[4] = {cur[c].x, cur[c].y, cur[c].z, cur[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) __builtin_memcpy(&hv[4 * c + e], &w[e], 4);
    }
    auto val = [&](int i) -> float { return ROT ? v[i] : (float)hv[i >> 1][i & 1]; };
    if (ROT) {
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = (float)hv[i >> 1][i & 1];
      // y_j = sum_i x_i (-1)^popcount(i & j): one butterfly stage per index
      // bit, in fp64 (exact), then one rounding to fp32
      double d[V];
#pragma unroll
      for (int i = 0; i < V; ++i) d[i] = (double)v[i];
      if (kSwapOut) {
        // In-lane stages first, the two top chunk bits last (h = V/4 with
        // c2, h = V/2 with c1).  In a lane whose quad bit is set, those two
        // write the difference to the lower slot, negated, and the sum to the
        // upper one.  Each cross-lane stage then sends only the upper slots
        // of its bit (the partner's values of the half this lane keeps) and
        // forms both outputs of the kept half, one fma each: half the
        // exchanges of the loaded layout.  Afterwards quad bit 0 selects the
        // top chunk bit of the output index and slot bit V/2 its bit 3;
        // quad bit 1 selects the next chunk bit and slot bit V/4 index bit
        // 4.  So lane sub ends with the V channels from
        // V (2 (sub & 1) + (sub >> 1)) on, chunk c at chunk_out(c).
#pragma unroll
        for (int h = 1; h < V / 4; h <<= 1)
#pragma unroll
          for (int i = 0; i < V; ++i)
            if (!(i & h)) {
              const double p = d[i], r = d[i + h];
              d[i] = p + r;
              d[i + h] = p - r;
            }
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (!(i & (V / 4))) {
            const double p = d[i], r = d[i + V / 4];
            d[i] = __builtin_fma(c2, p, r);
            d[i + V / 4] = __builtin_fma(-c2, r, p);
          }
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
          const double p = d[i], r = d[i + V / 2];
          d[i] = __builtin_fma(c1, p, r);
          d[i + V / 2] = __builtin_fma(-c1, r, p);
        }
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
          const double p = d[i], r = quad_perm64<0xB1>(d[i + V / 2]);  // quad_perm [1,0,3,2]
          d[i] = __builtin_fma(c1, p, r);
          d[i + V / 2] = __builtin_fma(-c1, r, p);
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (!(i & (V / 4))) {
            const double p = d[i], r = quad_perm64<0x4E>(d[i + V / 4]);  // quad_perm [2,3,0,1]
            d[i] = __builtin_fma(c2, p, r);
            d[i + V / 4] = __builtin_fma(-c2, r, p);
          }
      } else {
#pragma unroll
        for (int h = 1; h < V; h <<= 1)
#pragma unroll
          for (int i = 0; i < V; ++i)
            if (!(i & h)) {
              const double p = d[i], r = d[i + h];
              d[i] = p + r;
              d[i + h] = p - r;
            }
#pragma unroll
        for (int i = 0; i < V; ++i) d[i] = __builtin_fma(quad_perm64<0xB1>(d[i]), c1, d[i]);  // quad_perm [1,0,3,2]
#pragma unroll
        for (int i = 0; i < V; ++i) d[i] = __builtin_fma(quad_perm64<0x4E>(d[i]), c2, d[i]);  // quad_perm [2,3,0,1]
      }
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = (float)(d[i] * fin);
    }
    // the group's min and max over the quad (0 included, as the quantizer's range)
    float mn = 0.0f, mx = 0.0f;
    if (ROT) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        mn = fminf(mn, v[i]);
        mx = fmaxf(mx, v[i]);
      }
    } else {
      // three-input packed minimum / maximum (a NaN, which the loaded data
      // never holds, would carry through to the group's scale)
      h2 m0 = hv[0], m1 = hv[0];
#pragma unroll
      for (int i = 1; i < V / 2; ++i) {
        m0 = __builtin_elementwise_minimum(m0, hv[i]);
        m1 = __builtin_elementwise_maximum(m1, hv[i]);
      }
      mn = fminf(fminf((float)m0.x, (float)m0.y), 0.0f);
      mx = fmaxf(fmaxf((float)m1.x, (float)m1.y), 0.0f);
    }
    mn = fminf(mn, quad_xor1(mn));
    mx = fmaxf(mx, quad_xor1(mx));
    mn = fminf(mn, quad_xor2(mn));
    mx = fmaxf(mx, quad_xor2(mx));
    const RowQuant rq = row_quant(true, 1.0f, mn, mx);
    // codes eight to a dword, nibble e = channel 32c + 8 sub + e (loaded
    // layout) or V (2 (sub & 1) + (sub >> 1)) + 8c + e (exchanged layout,
    // from the lane's chunk chunk_out(c)); the byte permutes gather the low
    // bytes (the nibbles) of the magic-biased floats
    constexpr bool SW = ROT && kSwapOut;
    uint32_t wd[NC];
    auto pack = [&](auto code) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int cs = SW ? chunk_out(c) : c;
        uint32_t b[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) b[k] = __float_as_uint(__builtin_amdgcn_fmed3f(code(val(8 * cs + k)), rq.lo_c, rq.hi_c));
        const uint32_t e = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[6], b[4], 0x04000C0Cu);
        const uint32_t od = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0400u) | __builtin_amdgcn_perm(b[7], b[5], 0x04000C0Cu);
        wd[c] = (od << 4) | e;
      }
    };
    if (__builtin_amdgcn_ballot_w64(rq.exact || (!ROT && rq.wide)) == 0) {
      pack([&](float f) { return __builtin_fmaf(f, rq.inv, rq.base); });
    } else if (!ROT && __builtin_amdgcn_ballot_w64(rq.wide) != 0) {
      // Some fp16 group spans a wide range (its hi - lo has more than 16
      // significant bits: a large value beside a tiny one of the other
      // sign), so a value may lie closer to a rounding boundary than one fma
      // resolves: every group of the wavefront takes the exact quotient.
      pack([&](float f) {
        return rq.s > 0.0f ? rne_quotient(f, rq.s, rq.inv) + rq.base : rq.base;
      });
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
      const float zf = (float)rq.zp;
      pack([&](float f) {
        return __builtin_fmaf(__builtin_fmaf(f, lo_inv, kMagic0) + __builtin_fmaf(f, hi_inv, kMagic0), 0.5f, zf);
      });
    }
    uint8_t *gq = o.q + t * (a.gpr * (int64_t)(G / 2)) + (int64_t)gc * (G / 2);
    if (SW) {
      // the lane's V codes are contiguous: V/2 bytes from its position
      uint8_t *lq = gq + (V / 2) * (2 * (sub & 1) + (sub >> 1));
      if (a.vec_store) {
#pragma unroll
        for (int b = 0; b < NC / 4; ++b)
          if (valid) store_nt(reinterpret_cast<uint4 *>(lq) + b, make_uint4(wd[4 * b], wd[4 * b + 1], wd[4 * b + 2], wd[4 * b + 3]));
      } else if (valid) {
#pragma unroll
        for (int c = 0; c < NC; ++c) store_nt(reinterpret_cast<uint32_t *>(lq) + c, wd[c]);
      }
    } else if (NC >= 4 && a.vec_store) {
      // 4 x 4 transposes in the quad (lane s: dword s of chunks 4b..4b+3 ->
      // the four dwords of chunk 4b + s), so each lane stores 16 contiguous
      // bytes and a wavefront's 16 groups leave as whole lines
      const bool o1 = sub & 1, o2 = sub & 2;
#pragma unroll
      for (int b = 0; b < NC / 4; ++b) {
        uint32_t *u = wd + 4 * b;
#pragma unroll
        for (int c = 0; c < 4; c += 2) {
          const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o1 ? u[c] : u[c + 1]), 0xB1, 0xF, 0xF, false);
          if (o1) u[c] = r;
          else u[c + 1] = r;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o2 ? u[c] : u[c + 2]), 0x4E, 0xF, 0xF, false);
          if (o2) u[c] = r;
          else u[c + 2] = r;
        }
        if (valid) store_nt(reinterpret_cast<uint4 *>(gq) + 4 * b + sub, make_uint4(u[0], u[1], u[2], u[3]));
      }
    } else if (valid) {
      uint32_t *dst = reinterpret_cast<uint32_t *>(gq) + sub;
#pragma unroll
      for (int c = 0; c < NC; ++c) store_nt(dst + 4 * c, wd[c]);
    }
    if (valid && sub == 0) {
      const int64_t gi = t * a.gpr + gc;
      o.scale[gi] = rq.s;
      o.zero[gi] = rq.zp;
    }
  }
};

}  // namespace

// One tensor: the next set is loaded before the current one is worked.
template <int V, bool ROT>
__global__ __launch_bounds__(256) void group_quant(KvArgs a) {
  constexpr int NC = V / 8;
  const KvLane<V> L(a);
  const uint32_t w0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  int64_t gb = (int64_t)w0 * 16;  // first group of the current set
  if (gb >= a.total) return;      // whole wavefront
  int64_t t0 = (uint32_t)gb / (uint32_t)a.gpr;
  int32_t c0 = (int32_t)(gb - t0 * a.gpr);

  int64_t t;
  int32_t gc;
  bool valid = L.locate(a, gb, t0, c0, t, gc);
  uint4 cur[NC];
  L.load(cur, a.ten[0], t, gc);
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
    const bool validn = more ? L.locate(a, gbn, t0n, c0n, tn, gcn) : (tn = t, gcn = gc, false);
    uint4 nxt[NC];
    L.load(nxt, a.ten[0], tn, gcn);
    L.template quant<ROT>(a, cur, a.ten[0], t, gc, valid);
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

// Keys and values of the same tokens (same shape): per set the tensor with
// the heavier arithmetic (ten[0], the keys) is worked first while the
// other's data arrives.  The compiler issues the second tensor's loads
// partway through the first one's transform; pinned ahead of the transform
// (a scheduling barrier after each load group) the launch was 6% slower.
template <int V, bool R0, bool R1>
__global__ __launch_bounds__(256) void group_quant_pair(KvArgs a) {
  constexpr int NC = V / 8;
  const KvLane<V> L(a);
  const uint32_t w0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  int64_t gb = (int64_t)w0 * 16;
  if (gb >= a.total) return;
  int64_t t0 = (uint32_t)gb / (uint32_t)a.gpr;
  int32_t c0 = (int32_t)(gb - t0 * a.gpr);
  for (;;) {
    int64_t t;
    int32_t gc;
    const bool valid = L.locate(a, gb, t0, c0, t, gc);
    uint4 k[NC], v[NC];
    L.load(k, a.ten[0], t, gc);
    L.load(v, a.ten[1], t, gc);
    L.template quant<R0>(a, k, a.ten[0], t, gc, valid);
    L.template quant<R1>(a, v, a.ten[1], t, gc, valid);
    gb += a.step;
    if (gb >= a.total) break;
    t0 += a.step_rows;
    c0 += a.step_cols;
    if (c0 >= a.gpr) {
      c0 -= a.gpr;
      ++t0;
    }
  }
}

namespace {
// wavefronts per launch: four per SIMD of the 256 compute units (one set
// each at the 2048 x 4096 shapes); larger inputs loop
constexpr int kKvWaves = 256 * 4 * 4;

KvArgs kv_args(int64_t T, int64_t K, int group, const KvTensor *ten, int nt) {
  KvArgs a{};
  for (int i = 0; i < nt; ++i) a.ten[i] = ten[i];
  if (nt == 1) a.ten[1] = ten[0];
  a.T = T;
  a.gpr = (int32_t)(K / group);
  a.total = T * a.gpr;
  a.gpr_magic = (uint32_t)(0xFFFFFFFFu / (uint32_t)a.gpr) + 1u;
  a.vec_store = 1;
  for (int i = 0; i < nt; ++i)
    if ((uintptr_t)ten[i].q % 16) a.vec_store = 0;
  a.norm = 1.0 / sqrt((double)group);
  return a;
}

int64_t kv_grid(KvArgs &a) {
  const int64_t sets = (a.total + 15) / 16;
  const int64_t waves = std::min<int64_t>(sets, kKvWaves);
  const int64_t blocks = (waves + 3) / 4;
  a.step = blocks * 4 * 16;
  a.step_rows = a.step / a.gpr;
  a.step_cols = (int32_t)(a.step - a.step_rows * a.gpr);
  return blocks;
}
}  // namespace

hipError_t launch_group_quant(const void *x, int64_t T, int64_t K, int64_t ldx, int group, bool rotate,
                              uint8_t *q, float *scale, int32_t *zero, hipStream_t st) {
  const KvTensor ten{(const __half *)x, ldx, q, scale, zero};
  KvArgs a = kv_args(T, K, group, &ten, 1);
  const dim3 g((unsigned)kv_grid(a)), b(256);
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

template <int V>
static void launch_pair_v(const KvArgs &a, bool r0, bool r1, dim3 g, hipStream_t st) {
  const dim3 b(256);
  if (r1) group_quant_pair<V, true, true><<<g, b, 0, st>>>(a);  // r1 implies r0 (rotated tensor first)
  else if (r0) group_quant_pair<V, true, false><<<g, b, 0, st>>>(a);
  else group_quant_pair<V, false, false><<<g, b, 0, st>>>(a);
}

hipError_t launch_group_quant_pair(const KvTensor &k, bool rot_k, const KvTensor &v, bool rot_v, int64_t T,
                                   int64_t K, int group, hipStream_t st) {
  // the rotated tensor first: its arithmetic overlaps the other's loads
  const bool swap = rot_v && !rot_k;
  const KvTensor ten[2] = {swap ? v : k, swap ? k : v};
  KvArgs a = kv_args(T, K, group, ten, 2);
  const bool r0 = swap ? rot_v : rot_k, r1 = swap ? rot_k : rot_v;
  const dim3 g((unsigned)kv_grid(a));
  switch (group) {
    case 64: launch_pair_v<16>(a, r0, r1, g, st); break;
    case 128: launch_pair_v<32>(a, r0, r1, g, st); break;
    case 256: launch_pair_v<64>(a, r0, r1, g, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rq
