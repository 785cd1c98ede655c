// gemm_common.h -- device helpers shared by the INT4 GEMM kernels (internal).
#pragma once

#include "rq_device.h"

namespace rq {

// Int4 -> int8 widening.  Signed codes keep the nibble in the high half of
// each byte (value x16), unsigned codes in the low half (value x1); every
// widened operand pair is built from the same dword indices on both sides,
// so the k order inside an MFMA does not matter.
__device__ __forceinline__ v4i widen_signed(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(w0 & 0xF0F0F0F0u);
  r[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(w1 & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ v4i widen_unsigned(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)(w0 & 0x0F0F0F0Fu);
  r[1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
  r[2] = (int)(w1 & 0x0F0F0F0Fu);
  r[3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
  return r;
}

// Workgroup id -> output tile.  Consecutive ids go round-robin to the 8
// XCDs; remapping gives each XCD a contiguous range of positions, and the
// grouped order walks 8 row-tiles against consecutive column tiles, so the
// workgroups resident on one XCD share rows and columns in its L2.
__device__ __forceinline__ void map_tile(int bid, int nt_m, int nt_n, int &tm, int &tn) {
  const int nt = nt_m * nt_n;
  int pos = bid;
  if ((nt & 7) == 0) pos = (bid & 7) * (nt >> 3) + (bid >> 3);
  constexpr int G = 8;
  const int group = pos / (G * nt_n);
  const int first = group * G;
  const int gsz = min(G, nt_m - first);
  const int in = pos - group * G * nt_n;
  tm = first + in % gsz;
  tn = in / gsz;
}

}  // namespace rq
