// rq_kernels.h -- launchers of the gfx950 kernels (internal; the C ABI in
// rq_api.cpp validates arguments and then calls these).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rq {

struct GemmArgs {
  const uint8_t *qx;     // [T, Kb] packed codes
  const uint8_t *qw;     // [N, Kb] packed codes (signed)
  int64_t T, N, Kb;      // Kb = K / 2 bytes per row
  const float *sx;       // [T]
  const float *sw;       // [N]
  const int32_t *zx;     // [T] or null
  const int32_t *rowsum; // [N] or null
  const __half *xo;      // [T, n_out] or null
  const __half *wo;      // [N, n_out] or null
  int n_out;
  void *out;             // int32 or fp16 [T, ldo]
  int64_t ldo;
};

// The fused decode form (quantizer + linear in one launch): the unrotated
// fp16 rows and their quantizer.
struct FuseArgs {
  const __half *x;       // [T, ldx] fp16 rows
  int64_t ldx;
  int K;                 // columns of x (K - n_out = 2 * GemmArgs::Kb)
  float clip;            // symmetric clip ratio (1 when asymmetric)
  const int32_t *oidx;   // [n_out] outlier columns, or null when n_out == 0
  int gsr_log2;          // rotated form (K = 4096): 0 = Walsh-Hadamard, else GSR block log2
  float norm;            // GSR: 1 / sqrt(block); Walsh-Hadamard: unused
  int ks;                // set by the launcher: wavefronts sharing a channel block's k-steps
};

hipError_t launch_fwht4096(const void *x, int64_t T, int64_t ldx, bool gsr, int span_log2,
                           float norm, float clip, uint8_t *q, float *scale, int32_t *code_sum,
                           hipStream_t st);
size_t rowlds_smem_bytes(int64_t K);
hipError_t launch_rowlds(const void *x, int64_t T, int64_t K, int64_t ldx, int span_log2, bool gsr,
                         float norm, float clip, uint8_t *q, float *scale, int32_t *code_sum,
                         hipStream_t st);
hipError_t launch_split(const void *x, int64_t T, int64_t K, int64_t ldx, bool asym, float clip,
                        const float *row_clip, const int32_t *outlier_idx, int n_out, uint8_t *q,
                        float *scale, int32_t *zero, int32_t *code_sum, void *x_out, hipStream_t st);
hipError_t launch_kron64(const void *x, int64_t T, int64_t ldx, const float *fa, const float *fb,
                         const float *chan_scale, bool divide, float clip, uint8_t *q, float *scale,
                         int32_t *code_sum, hipStream_t st);
hipError_t launch_kron(const void *x, int64_t T, int64_t ldx, int n1, int n2, const float *fa,
                       const float *fb, const float *chan_scale, bool divide, float clip,
                       uint8_t *q, float *scale, int32_t *code_sum, hipStream_t st);
hipError_t launch_kron_inverse_t(const float *p1, int n1, float *o1, const float *p2, int n2,
                                 float *o2, hipStream_t st);
// mode 0: raw int32 accumulator; 1: symmetric fp16 output; 2: mixed fp16 output
bool gemm_decode_fits(const GemmArgs &p);
hipError_t launch_gemm_decode(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st);
// fused decode: p.qx, p.sx, p.zx and p.xo unused; the codes are made in the kernel
bool decode_fused_fits(const GemmArgs &p, const FuseArgs &f);
hipError_t launch_decode_fused(const GemmArgs &p, const FuseArgs &f, bool asym, int mode, hipStream_t st);
// rotated fused decode (K = 4096, symmetric, no outliers): the 4096-point
// Walsh-Hadamard or GSR transform + quantizer per row in the prologue
bool decode_fused_rot_fits(const GemmArgs &p, const FuseArgs &f);
hipError_t launch_decode_fused_rot(const GemmArgs &p, const FuseArgs &f, hipStream_t st);

// kv_quant.hip: per-group Walsh-Hadamard (optional) + group-wise asymmetric INT4
hipError_t launch_group_quant(const void *x, int64_t T, int64_t K, int64_t ldx, int group, bool rotate,
                              uint8_t *q, float *scale, int32_t *zero, hipStream_t st);
// one tensor of the KV quantizer: fp16 input rows and the three outputs
struct KvTensor {
  const __half *x;
  int64_t ldx;
  uint8_t *q;
  float *scale;
  int32_t *zero;
};
// keys and values of the same T tokens in one launch
hipError_t launch_group_quant_pair(const KvTensor &k, bool rot_k, const KvTensor &v, bool rot_v, int64_t T,
                                   int64_t K, int group, hipStream_t st);
bool gemm_ra_fits(const GemmArgs &p);
hipError_t launch_gemm_ra(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st);
// one-byte codes (Kb = K bytes per row); x_unsigned: codes in [0, 255], p.rowsum required;
// T <= 32 goes to gemm_decode8 when its activation stage fits LDS
hipError_t launch_gemm_ra8(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st);
bool gemm_decode8_fits(const GemmArgs &p, int mode);
hipError_t launch_gemm_decode8(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st);
// quant8.hip: unrotated per-row INT8 with the outlier split
size_t split8_smem_bytes(int64_t K, int n_out);
hipError_t launch_split8(const void *x, int64_t T, int64_t K, int64_t ldx, bool asym, float clip,
                         const float *row_clip, const int32_t *outlier_idx, int n_out, uint8_t *q,
                         float *scale, int32_t *zero, int32_t *code_sum, void *x_out, hipStream_t st);
// clip_search.hip: QUIK's per-row weight clip ratio by linear search
hipError_t launch_clip_search(const void *w, int64_t N, int64_t K, int64_t ldw, const int32_t *outlier_idx,
                              int n_out, int bits, int steps, float *clip_out, hipStream_t st);
hipError_t launch_gemm(const GemmArgs &p, bool x_unsigned, int mode, hipStream_t st);

}  // namespace rq
