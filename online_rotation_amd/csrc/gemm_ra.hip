// gemm_ra.hip -- the large-T INT4 x INT4 GEMM with INT32 accumulation and
// the fused dequantization epilogue (QUIK blog, "QUIK quantization" part 4:
// INT4 operands, INT32 accumulation; part 1: dequantize, then add the FP16
// outlier product before the one fp16 rounding), for gfx950.
//
// Workgroup: 256 threads = 4 wavefronts, one per SIMD; tile 256 tokens x 128
// output channels.  Wavefront w owns tile rows [64w, 64w + 64) against all
// 128 columns: 2 x 4 MFMA 32x32x32 blocks, 128 accumulator registers.  The
// kernel fits two workgroups per CU (256 registers per lane, 48 KB of LDS),
// so that one workgroup's waits are covered by the other's MFMAs whenever a
// CU gets more than one tile.
//
// What sets the design, per 32-code k slice and CU: 32 MFMAs (8 per SIMD).
// Measured on this chip, LDS serves about 136 bytes per clock per CU to
// 16-byte reads, and about four independent VALU instructions issue for free
// beside each MFMA.
//   - A rows belong to one wavefront only, so A goes global -> registers and
//     is widened there (1.5 VALU per MFMA); it never touches LDS.
//   - B columns are shared by all four wavefronts.  Each 16-byte int4 chunk
//     is loaded by one thread, widened once (0.75 VALU per MFMA) and stored
//     as int8, and the wavefronts read MFMA-ready fragments: 16 KB of reads
//     and 4 KB of writes per k slice and CU, about half the LDS rate.
// A k-step is 128 codes (64 bytes per row), four groups of 8 MFMAs.  Global
// loads run ahead in register rings and the B tile goes through 3 or 4 LDS
// buffers, with a barrier every step or every other step (the two schedules
// below), placed so that no fragment read waits on it: every MFMA group's
// fragments are read one group ahead, across step boundaries too.  Every
// step issues the same loads and stores with no branch around them (row
// indices are clamped into the matrices, and loads past the end re-load
// the last step), so the compiler waits only for the load group it needs
// next.
#include "gemm_common.h"
#include "rq_kernels.h"

#include <type_traits>

namespace rq {

namespace {

constexpr int kRaBM = 256, kRaBN = 128;
// Two schedules.  Barrier every other step (int4 codes without zero points
// or outliers): A ring 2 steps deep, B ring 4, B in 4 LDS buffers.  Barrier
// every step (8-bit codes, and the QUIK form, where the other schedule
// measured slower): one ring of 3 steps for both, 3 buffers.  The unroll
// keeps every slot and buffer index static.
constexpr int kRaDA = 2, kRaDB = 4, kRaNB = 4, kRaU4 = 4;
constexpr int kRaD3 = 3, kRaNB3 = 3, kRaU3 = 3;
constexpr int kRaRow = 128;               // LDS bytes per B row and k-step (int8)
constexpr int kRaBuf = kRaBN * kRaRow;    // one buffer: 16 KB
static_assert(kRaNB3 * kRaBuf >= (kRaBM + kRaBN) * 128, "outlier tiles must fit the B buffers");
static_assert(kRaU4 % kRaDA == 0 && kRaU4 % kRaDB == 0 && kRaU4 % kRaNB == 0, "unroll");
static_assert(kRaU3 % kRaD3 == 0 && kRaU3 % kRaNB3 == 0, "unroll");

// Widened slot s (16 bytes) of LDS row r sits at s ^ ((r >> 1) & 7): the 16
// rows that a group of 16 lanes reads (one row per lane) or writes (four
// lanes per row) then fall in distinct banks.
__device__ __forceinline__ int ra_off(int row, int slot) {
  return row * kRaRow + ((slot ^ ((row >> 1) & 7)) << 4);
}

// Tile order within an XCD's contiguous range of positions (the same XCD
// remap as map_tile): groups of G row tiles walked against consecutive column
// tiles.  With 16 or more row tiles (the QUIK shapes, K up to 28672) a group
// of 8 holds 8 row tiles of A, more than an XCD's 4 MB L2, and each round of
// resident workgroups re-fetched them; groups of 4 fetch 20% less there in
// the same time.  Smaller problems keep groups of 8.
__device__ __forceinline__ void ra_map_tile(int bid, int nt_m, int nt_n, int &tm, int &tn) {
  const int nt = nt_m * nt_n;
  int pos = bid;
  if ((nt & 7) == 0) pos = (bid & 7) * (nt >> 3) + (bid >> 3);
  const int G = nt_m >= 16 ? 4 : 8;
  const int group = pos / (G * nt_n);
  const int first = group * G;
  const int gsz = min(G, nt_m - first);
  const int in = pos - group * G * nt_n;
  tm = first + in % gsz;
  tn = in / gsz;
}

__device__ __forceinline__ uint4 ldg16(const uint8_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

}  // namespace

// BITS = 8: the operands are int8 codes (QUIK-8B's down projection), used by
// the MFMAs as they are; a k-step is then 64 codes (still 64 bytes per row),
// two MFMA groups, slot 2g + c in lane group g.  Unsigned activation codes
// (XU) are moved to signed by flipping bit 7 (u - 128), and the epilogue adds
// back 128 * rowsum.
template <bool XU, int MODE, int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_ra(GemmArgs p, int nt_m, int nt_n) {
  constexpr int kGroups = BITS == 8 ? 2 : 4;  // MFMA groups per k-step
  constexpr bool kHalf = BITS == 4 && MODE != 2;  // a barrier every other step
  constexpr int kNB = kHalf ? kRaNB : kRaNB3;
  constexpr int kDA = kHalf ? kRaDA : kRaD3, kDB = kHalf ? kRaDB : kRaD3;
  constexpr int kRaU = kHalf ? kRaU4 : kRaU3;
  __shared__ __align__(16) uint8_t Bs[kNB * kRaBuf];
  // The tile's dequantization vectors (sx, zx per row; sw, rowsum per
  // column), staged in LDS at the start so that the epilogue does not wait on
  // global loads after the k loop (modes 1 and 2).
  __shared__ float s_sx[kRaBM], s_sw[kRaBN];
  __shared__ int32_t s_zx[kRaBM], s_rs[kRaBN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5, l32 = lane & 31;
  int tm, tn;
  ra_map_tile(blockIdx.x, nt_m, nt_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kRaBM, n0 = (int64_t)tn * kRaBN, Kb = p.Kb;
  const int nsteps = (int)(Kb >> 6), last = nsteps - 1;

  // Slot s of a k-step = int4 dwords 2s, 2s+1 (codes 16s .. 16s+15), widened
  // to one 16-byte MFMA operand.  MFMA c of a step takes slot 4g + c in lane
  // group g, on both operands.
  // A: lane (l32, g) loads dwords [8g, 8g+8) of rows 64w + l32 and 64w + 32 + l32.
  const int64_t ar = m0 + wave * 64 + l32;
  const uint8_t *ap0 = p.qx + min(ar, p.T - 1) * Kb + 32 * g;
  const uint8_t *ap1 = p.qx + min(ar + 32, p.T - 1) * Kb + 32 * g;
  // B staging: thread t loads 16-byte chunk q = t & 3 (slots 2q, 2q+1) of tile
  // rows t >> 2 and 64 + (t >> 2).
  const int br = tid >> 2, bq = tid & 3;
  const uint8_t *bp0 = p.qw + min(n0 + br, p.N - 1) * Kb + 16 * bq;
  const uint8_t *bp1 = p.qw + min(n0 + 64 + br, p.N - 1) * Kb + 16 * bq;
  const int ws0 = ra_off(br, BITS == 8 ? bq : 2 * bq), ws1 = ra_off(br, 2 * bq + 1);
  const int ws2 = ra_off(br + 64, BITS == 8 ? bq : 2 * bq), ws3 = ra_off(br + 64, 2 * bq + 1);
  // fragment of block j, MFMA c: row 32j + l32, slot 4g + c.  ((32j + l32) >> 1) & 7
  // does not depend on j, so the offset is j * 32 * kRaRow + rs[c].
  int rs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) rs[c] = l32 * kRaRow + (((kGroups * g + c) ^ ((l32 >> 1) & 7)) << 4);

  // A(k) in A slot k % kDA, B(k) in B slot k % kDB
  uint4 ra[kDA][4], rb[kDB][2];
  auto gload_a = [&](int s, int k) {
    const int64_t o = (int64_t)k * 64;
    ra[s][0] = ldg16(ap0 + o);
    ra[s][1] = ldg16(ap0 + o + 16);
    ra[s][2] = ldg16(ap1 + o);
    ra[s][3] = ldg16(ap1 + o + 16);
  };
  auto gload_b = [&](int s, int k) {
    const int64_t o = (int64_t)k * 64;
    rb[s][0] = ldg16(bp0 + o);
    rb[s][1] = ldg16(bp1 + o);
  };
  // half h of a B staging chunk w, widened, into LDS buffer buf
  auto bstore_w = [&](int buf, const uint4 &w, int h) {
    uint8_t *B = Bs + buf * kRaBuf;
    if (BITS == 8) {
      *reinterpret_cast<uint4 *>(B + (h ? ws2 : ws0)) = w;
    } else {
      *reinterpret_cast<v4i *>(B + (h ? ws2 : ws0)) = widen_signed(w.x, w.y);
      *reinterpret_cast<v4i *>(B + (h ? ws3 : ws1)) = widen_signed(w.z, w.w);
    }
  };
  auto bstore = [&](int buf, int s, int h) { bstore_w(buf, rb[s][h], h); };
  v4i bf[2][4];  // B fragments, double-buffered across MFMA groups
  auto bread = [&](int f, int buf, int c) {
    const uint8_t *B = Bs + buf * kRaBuf;
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[f][j] = *reinterpret_cast<const v4i *>(B + j * 32 * kRaRow + rs[c]);
  };
  auto awiden = [&](int s, int c, v4i *aw) {
    if (BITS == 8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 &w = ra[s][2 * i + c];
        const uint32_t f = XU ? 0x80808080u : 0u;
        aw[i][0] = (int)(w.x ^ f);
        aw[i][1] = (int)(w.y ^ f);
        aw[i][2] = (int)(w.z ^ f);
        aw[i][3] = (int)(w.w ^ f);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 &w = ra[s][2 * i + (c >> 1)];
      const uint32_t w0 = (c & 1) ? w.z : w.x, w1 = (c & 1) ? w.w : w.y;
      aw[i] = XU ? widen_unsigned(w0, w1) : widen_signed(w0, w1);
    }
  };

  v16i acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
  auto mfma8 = [&](const v4i *aw, int f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aw[i], bf[f][j], acc[i][j], 0, 0, 0);
  };

  // The dequantization vectors go out first, unconditionally (clamped
  // indices; a missing zx or rowsum reads a stand-in and is zeroed), so that
  // waiting for B(0) below also covers them.
  constexpr int kZoffS = (BITS == 8 && XU) ? 128 : 0;
  const bool need_zx = MODE == 2 && p.zx;
  const bool need_rs = need_zx || kZoffS;
  float vsx = 0.0f, vsw = 0.0f;
  int32_t vzx = 0, vrs = 0;
  if (MODE != 0) {
    const int64_t sr = min(m0 + tid, p.T - 1), sc = min(n0 + (tid & (kRaBN - 1)), p.N - 1);
    const int32_t *zxp = need_zx ? p.zx : reinterpret_cast<const int32_t *>(p.sx);
    const int32_t *rsp = need_rs ? p.rowsum : reinterpret_cast<const int32_t *>(p.sw);
    vsx = p.sx[sr];
    vzx = zxp[sr];
    vsw = p.sw[sc];
    vrs = rsp[sc];
  }
  // prologue.  Every other step: B(0 .. 3) and A(0 .. 1) in flight; B(0),
  // B(1) into buffers 0, 1 and their slots refilled with B(4), B(5).  Every
  // step: steps 0 .. 2 in flight, B(0) into buffer 0.  Then B(0)'s first
  // fragments.
  if (kHalf) {
#pragma unroll
    for (int s = 0; s < kDB; ++s) gload_b(s, min(s, last));
#pragma unroll
    for (int s = 0; s < kDA; ++s) gload_a(s, min(s, last));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      bstore(k, k, 0);
      bstore(k, k, 1);
      gload_b(k, min(k + kDB, last));
    }
  } else {
#pragma unroll
    for (int s = 0; s < kDA; ++s) {
      gload_a(s, min(s, last));
      gload_b(s, min(s, last));
    }
    bstore(0, 0, 0);
    bstore(0, 0, 1);
  }
  if (MODE != 0) {
    s_sx[tid] = vsx;
    s_zx[tid] = need_zx ? vzx : 0;
    if (tid < kRaBN) {
      s_sw[tid] = vsw;
      s_rs[tid] = need_rs ? vrs : 0;
    }
  }
  __syncthreads();
  bread(0, 0, 0);

  // Barrier every other step.  Step kb: A(kb) in A slot kb % 2, B(kb+2) in
  // B slot (kb+2) % 4 (refilled with B(kb+6) once stored), B(kb) in LDS
  // buffer kb % 4 with MFMA group 0's fragments already in registers,
  // B(kb+1) in buffer (kb+1) % 4.  Each of the four MFMA groups reads the
  // next group's fragments first.  B(kb+2) is stored into buffer (kb+2) % 4
  // during groups 0 and 1, and only odd steps end with a barrier (in group
  // 3, before step kb+1's first fragments are read):
  //   - B(kb+1) is read from step kb's group 3 on; it was stored in step
  //     kb-1, and one of steps kb-1, kb holds a barrier after that store and
  //     before group 3 (kb-1 odd: its own; kb odd: step kb's, ahead of the
  //     read);
  //   - buffer (kb+2) % 4 last held B(kb-2), whose last read is in step
  //     kb-2's group 2; one of steps kb-2, kb-1 ends with a barrier.
  // A barrier every other step lets the wavefronts drift apart for two steps
  // between meetings.  A(kb+2) is requested in step kb's group 3.
  // Barrier every step: A(kb) and B(kb) in load slot kb % 3; B(kb+1), from
  // slot (kb+1) % 3, is stored into buffer (kb+1) % 3 during groups 0 and 1
  // (8-bit: group 0), and every step's group 3 (8-bit: group 1) holds a
  // barrier; buffer (kb+1) % 3 was last read in step kb-2, before step
  // kb-1's barrier.
  auto steps = [&](int kb0, auto tail) {
#pragma unroll
    for (int v = 0; v < kRaU; ++v) {
      const int kb = kb0 + v;
      const int u = v % kDA, us = (v + 1) % kDB;       // A slot of kb; (8-bit) B slot of kb+1
      const int ub = v % kNB, nb = (v + 1) % kNB;      // LDS buffers of steps kb, kb+1
      const int nb2 = (v + 2) % kNB, ub2 = (v + 2) % kDB;  // int4: buffer and B slot of B(kb+2)
      const bool live = !decltype(tail)::value || kb < nsteps;
      v4i aw[2];
      if (BITS == 8) {
        // group 0, then B(kb+1) into its buffer and the barrier; group 1
        // reads step kb+1's first fragments and refills A's load slot
        bread(1, ub, 1);
        __builtin_amdgcn_sched_barrier(0);
        awiden(u, 0, aw);
        if (live) mfma8(aw, 0);
        bstore(nb, us, 0);
        bstore(nb, us, 1);
        __syncthreads();
        awiden(u, 1, aw);
        __builtin_amdgcn_sched_barrier(0);
        gload_a(u, min(kb + kDA, last));
        gload_b(u, min(kb + kDA, last));
        bread(0, nb, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (live) mfma8(aw, 1);
        __builtin_amdgcn_sched_barrier(0);
        if (decltype(tail)::value && kb + 1 >= nsteps) break;
        continue;
      }
      // (sched_barrier: keep each group's fragment reads ahead of its MFMAs;
      // the scheduler otherwise sinks them next to their first use)
      // group 0
      bread(1, ub, 1);
      __builtin_amdgcn_sched_barrier(0);
      awiden(u, 0, aw);
      if (live) mfma8(aw, 0);
      if (kHalf) bstore(nb2, ub2, 0);
      else bstore(nb, us, 0);
      __builtin_amdgcn_sched_barrier(0);
      // group 1
      bread(0, ub, 2);
      __builtin_amdgcn_sched_barrier(0);
      awiden(u, 1, aw);
      if (live) mfma8(aw, 1);
      if (kHalf) {
        bstore(nb2, ub2, 1);
        gload_b(ub2, min(kb + 2 + kDB, last));
      } else {
        bstore(nb, us, 1);
      }
      // group 2
      bread(1, ub, 3);
      __builtin_amdgcn_sched_barrier(0);
      awiden(u, 2, aw);
      if (live) mfma8(aw, 0);
      __builtin_amdgcn_sched_barrier(0);
      // group 3: A(kb) is fully widened after this, so its slot is refilled.
      // The barrier (odd steps) sits here, a whole MFMA group after the last
      // LDS stores of B(kb+2): placed before group 2 it waited for those
      // stores to land with the matrix pipe idle (measured 1-2 us more at
      // T = 2048, K = N = 4096).
      awiden(u, 3, aw);
      __builtin_amdgcn_sched_barrier(0);
      if (!kHalf || (v & 1)) __syncthreads();
      gload_a(u, min(kb + kDA, last));
      if (!kHalf) gload_b(u, min(kb + kDA, last));
      bread(0, nb, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (live) mfma8(aw, 1);
      __builtin_amdgcn_sched_barrier(0);
      // the tail group stops after the last step (a uniform exit, so every
      // wavefront meets the same barriers)
      if (decltype(tail)::value && kb + 1 >= nsteps) break;
    }
  };
  // Whole groups of kRaU steps in the loop; a final partial group outside
  // it, so that no branch sits inside the loop (a branch there makes the
  // compiler copy the load ring at the back edge, waiting for every load in
  // flight).
  int kb0 = 0;
  for (; kb0 + kRaU <= nsteps; kb0 += kRaU) steps(kb0, std::false_type());
  if (kb0 < nsteps) steps(kb0, std::true_type());

  // The epilogue's lane indices are made again here (the lane id from
  // mbcnt) rather than carried across the k loop, where they would hold
  // registers (spilled to scratch when the loop fills the register file).
  const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int etid = wave * 64 + elane, eg = elane >> 5, el32 = elane & 31;
  // Epilogue.  32x32 accumulator layout: lane l, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32 of its block.
  constexpr int kShift = BITS == 8 ? 0 : (XU ? 4 : 8);
  // 8-bit unsigned codes went in as u - 128: sum (u - z) w = acc - (z - 128) rowsum
  constexpr int kZoff = (BITS == 8 && XU) ? 128 : 0;
  const int64_t row0 = m0 + wave * 64, col0 = n0;
  if (MODE == 0) {
    int32_t *out = reinterpret_cast<int32_t *>(p.out);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t gn = col0 + 32 * j + el32;
        const int32_t rsj = kZoff ? p.rowsum[min(gn, p.N - 1)] : 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gm = row0 + 32 * i + 8 * (r >> 2) + 4 * eg + (r & 3);
          if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = (acc[i][j][r] >> kShift) + kZoff * rsj;
        }
      }
    return;
  }
  float swn[4];
  int32_t rsn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    swn[j] = s_sw[32 * j + el32];
    rsn[j] = s_rs[32 * j + el32];
  }
  v16f f[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = wave * 64 + 32 * i + 8 * (r >> 2) + 4 * eg + (r & 3);
      const float sxm = s_sx[lr];
      const int32_t zxm = s_zx[lr] - kZoff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int32_t v = acc[i][j][r] >> kShift;
        if (MODE == 2 || kZoff) v -= zxm * rsn[j];
        f[i][j][r] = (float)v * sxm * swn[j];
      }
    }
  if (MODE == 2 && p.n_out > 0) {
    // FP16 outlier product on FP16 matrix cores, fp32 accumulation on top of
    // the dequantized INT4 part.  x_out (tile rows) and w_out (tile columns)
    // go through the idle B buffers in chunks of 32 columns: 256 x 64 B and
    // 128 x 64 B (at a 128-byte row pitch), loaded with coalesced 16-byte
    // segments (the next chunk into registers while this one is multiplied).
    // 64-column chunks held twice the registers beside the 128 accumulators
    // and spilled 144 bytes per lane; 32-column ones measured 5% faster at
    // the QUIK prefill shape.  Segment s of LDS row r sits at s ^ (r & 7).
    // MFMA step kk of a chunk takes halves [16kk + 8g, 16kk + 8g + 8) of a
    // row in lane group g: segment 2kk + g.
    uint8_t *Xs = Bs, *Ws = Bs + kRaBM * 128;
    const int nch = (p.n_out + 31) / 32;
    // The staging values are named one by one (literal indices): as arrays
    // filled in loops, the compiler moved them into LDS (24 KB per
    // workgroup) before the loops were unrolled.
    auto xo_at = [&](int c, int i) {  // columns past n_out are clamped and never multiplied
      const int idx = etid + 256 * i, row = idx >> 2, col = min(32 * c + 8 * (idx & 3), p.n_out - 8);
      return *reinterpret_cast<const uint4 *>(p.xo + min(m0 + row, p.T - 1) * p.n_out + col);
    };
    auto wo_at = [&](int c, int i) {
      const int idx = etid + 256 * i, row = idx >> 2, col = min(32 * c + 8 * (idx & 3), p.n_out - 8);
      return *reinterpret_cast<const uint4 *>(p.wo + min(n0 + row, p.N - 1) * p.n_out + col);
    };
    auto put = [&](uint8_t *base, int i, const uint4 &v) {
      const int idx = etid + 256 * i, row = idx >> 2, sg = idx & 3;
      *reinterpret_cast<uint4 *>(base + row * 128 + ((sg ^ (row & 7)) << 4)) = v;
    };
    uint4 px0, px1, px2, px3, pw0, pw1;
    auto cload = [&](int c) {
      px0 = xo_at(c, 0);
      px1 = xo_at(c, 1);
      px2 = xo_at(c, 2);
      px3 = xo_at(c, 3);
      pw0 = wo_at(c, 0);
      pw1 = wo_at(c, 1);
    };
    auto cstore = [&]() {
      put(Xs, 0, px0);
      put(Xs, 1, px1);
      put(Xs, 2, px2);
      put(Xs, 3, px3);
      put(Ws, 0, pw0);
      put(Ws, 1, pw1);
    };
    cload(0);
    __syncthreads();  // every wave is done with the B buffers
    for (int c = 0; c < nch; ++c) {
      cstore();
      __syncthreads();
      if (c + 1 < nch) cload(c + 1);
      const int ksteps = min(2, (p.n_out - 32 * c) / 16);
      for (int kk = 0; kk < ksteps; ++kk) {
        v8h av[2], bv[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wave * 64 + 32 * i + el32;
          const uint4 t = *reinterpret_cast<const uint4 *>(Xs + r * 128 + (((2 * kk + eg) ^ (r & 7)) << 4));
          __builtin_memcpy(&av[i], &t, 16);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 32 * j + el32;
          const uint4 t = *reinterpret_cast<const uint4 *>(Ws + r * 128 + (((2 * kk + eg) ^ (r & 7)) << 4));
          __builtin_memcpy(&bv[j], &t, 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            f[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], f[i][j], 0, 0, 0);
      }
      __syncthreads();  // before the next chunk overwrites the tiles
    }
  }
  __half *out = reinterpret_cast<__half *>(p.out);
  if ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0 && (p.ldo & 7) == 0) {
    // Rows of 16-byte aligned outputs leave through LDS: each wavefront
    // stages 32 rows x 128 columns of fp16 (row pitch 272 bytes) in its slice
    // of the idle B buffers, then stores 16 bytes per lane, 4 rows x 256
    // contiguous bytes per instruction (against two 64-byte pieces per 2-byte
    // store instruction written straight from the accumulator layout:
    // measured 1-3 us less at T = 2048, K = N = 4096).
    constexpr int kP = 272;
    __syncthreads();  // every wavefront is done with the B buffers
    uint8_t *W = Bs + wave * (32 * kP);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 8 * (r >> 2) + 4 * eg + (r & 3);
          *reinterpret_cast<__half *>(W + rr * kP + 2 * (32 * j + el32)) = __float2half_rn(f[i][j][r]);
        }
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rr = 4 * it + (elane >> 4), cc = elane & 15;
        const uint4 v = *reinterpret_cast<const uint4 *>(W + rr * kP + 16 * cc);
        const int64_t gm = row0 + 32 * i + rr, gn = col0 + 8 * cc;
        if (gm < p.T) {
          if (gn + 8 <= p.N) {
            *reinterpret_cast<uint4 *>(out + gm * p.ldo + gn) = v;
          } else {  // the last, partial chunk of a row
            const uint16_t h[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                                   (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gn + e < p.N) reinterpret_cast<uint16_t *>(out)[gm * p.ldo + gn + e] = h[e];
          }
        }
      }
      wave_lds_sync();
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gn = col0 + 32 * j + el32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = row0 + 32 * i + 8 * (r >> 2) + 4 * eg + (r & 3);
        if (gm < p.T && gn < p.N) out[gm * p.ldo + gn] = __float2half_rn(f[i][j][r]);
      }
    }
}

bool gemm_ra_fits(const GemmArgs &p) { return p.T >= 256 && p.Kb % 64 == 0 && p.Kb >= 64; }

hipError_t launch_gemm_ra(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  const int nt_m = (int)((p.T + kRaBM - 1) / kRaBM), nt_n = (int)((p.N + kRaBN - 1) / kRaBN);
  const dim3 grid((unsigned)(nt_m * nt_n)), block(256);
  if (mode == 0) {
    if (x_unsigned) gemm_ra<true, 0, 4><<<grid, block, 0, st>>>(p, nt_m, nt_n);
    else gemm_ra<false, 0, 4><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  } else if (mode == 1) {
    gemm_ra<false, 1, 4><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  } else {
    if (x_unsigned) gemm_ra<true, 2, 4><<<grid, block, 0, st>>>(p, nt_m, nt_n);
    else gemm_ra<false, 2, 4><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_ra8(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st) {
  if (p.T <= 32 && gemm_decode8_fits(p, mode)) return launch_gemm_decode8(p, x_unsigned, mode, st);
  const int nt_m = (int)((p.T + kRaBM - 1) / kRaBM), nt_n = (int)((p.N + kRaBN - 1) / kRaBN);
  const dim3 grid((unsigned)(nt_m * nt_n)), block(256);
  if (mode == 0) {
    if (x_unsigned) gemm_ra<true, 0, 8><<<grid, block, 0, st>>>(p, nt_m, nt_n);
    else gemm_ra<false, 0, 8><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  } else if (mode == 1) {
    gemm_ra<false, 1, 8><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  } else {
    if (x_unsigned) gemm_ra<true, 2, 8><<<grid, block, 0, st>>>(p, nt_m, nt_n);
    else gemm_ra<false, 2, 8><<<grid, block, 0, st>>>(p, nt_m, nt_n);
  }
  return hipGetLastError();
}

}  // namespace rq
