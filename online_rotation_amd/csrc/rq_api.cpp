// rq_api.cpp -- the C ABI declared in include/rq.h: host-side argument checks,
// then kernel launches on the caller's stream.  Nothing here allocates,
// frees or synchronizes.
#include "../../include/rq.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "rq_kernels.h"

namespace {

// Scratch memory of rq_prepare_weights_noalloc: the KRON factors' inverse
// transposes (at most two 64 x 64 fp32 images, the second at a 256-byte
// offset), in device memory that exists for the life of the process, one copy
// per GPU.  Host code never uses the array's name as an address: each device's
// copy is looked up once with hipGetSymbolAddress and the result is kept.
constexpr int64_t kScratchBytes = 32768;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device id, under g_scratch_mu

thread_local char g_err[512] = "";

rq_status fail(rq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

rq_status ok() {
  g_err[0] = '\0';
  return RQ_OK;
}

rq_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(RQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) {
  int r = 0;
  while ((int64_t(1) << r) < v) ++r;
  return r;
}

constexpr int64_t kMaxK = 65536;
constexpr size_t kMaxLds = 160 * 1024 - 64;
constexpr int kSplitMaxK = 32768;  // the split quantizer: 256 threads x 4 words of 32 columns  // gfx950 LDS per workgroup, minus static reductions

// Checks shared by the activation and weight quantizers.
rq_status check_quant(const void *x, int64_t T, int64_t K, int64_t ldx, const rq_rot_desc *rot,
                      const rq_quant_desc *qd, uint8_t *q, float *scale, void *x_out) {
  if (!rot || !qd) return fail(RQ_EINVAL, "rot and qd descriptors are required");
  if (T < 0 || K <= 0) return fail(RQ_EINVAL, "T must be >= 0 and K > 0 (T=%lld K=%lld)", (long long)T, (long long)K);
  if (K > 32768) return fail(RQ_ESHAPE, "K=%lld exceeds 32768", (long long)K);
  if (K % 8) return fail(RQ_ESHAPE, "K=%lld must be a multiple of 8", (long long)K);
  if (qd->n_out < 0 || qd->n_out >= K) return fail(RQ_EINVAL, "n_out=%d out of range", qd->n_out);
  if (qd->n_out > 0 && !qd->outlier_idx) return fail(RQ_EINVAL, "outlier_idx is NULL with n_out > 0");
  if ((K - qd->n_out) % 64) return fail(RQ_ESHAPE, "K - n_out = %lld is not a multiple of 64", (long long)(K - qd->n_out));
  if (!(qd->clip_ratio > 0.0f && qd->clip_ratio <= 1.0f)) return fail(RQ_EINVAL, "clip_ratio must be in (0, 1]");
  if (qd->asymmetric && qd->clip_ratio != 1.0f) return fail(RQ_EINVAL, "asymmetric quantization takes clip_ratio 1");
  if (qd->bits != 0 && qd->bits != 4 && qd->bits != 8) return fail(RQ_EINVAL, "bits=%d must be 4 or 8", qd->bits);
  if (rot->kind < RQ_ROT_NONE || rot->kind > RQ_ROT_KRON) return fail(RQ_EINVAL, "unknown rotation kind %d", rot->kind);
  if (qd->bits == 8 && rot->kind != RQ_ROT_NONE) return fail(RQ_ESHAPE, "8-bit codes are only supported without a rotation");
  if (qd->row_clip && (rot->kind != RQ_ROT_NONE || qd->asymmetric))
    return fail(RQ_ESHAPE, "per-row clip ratios are only supported for symmetric codes without a rotation");
  if (qd->row_clip && !aligned(qd->row_clip, 4)) return fail(RQ_EALIGN, "row_clip must be 4-byte aligned");
  if (rot->kind != RQ_ROT_NONE && qd->n_out) return fail(RQ_ESHAPE, "outlier split is only supported without a rotation");
  if (rot->kind != RQ_ROT_NONE && qd->asymmetric) return fail(RQ_ESHAPE, "asymmetric codes are only supported without a rotation");
  if (rot->kind == RQ_ROT_HADAMARD && !(pow2(K) && K >= 64)) return fail(RQ_ESHAPE, "HADAMARD needs a power-of-two K >= 64 (K=%lld)", (long long)K);
  if (rot->kind == RQ_ROT_GSR && !(pow2(rot->block) && rot->block >= 2 && rot->block <= 256 && K % rot->block == 0))
    return fail(RQ_ESHAPE, "GSR block %d must be a power of two in [2, 256] dividing K", rot->block);
  if (rot->kind == RQ_ROT_KRON) {
    if (rot->n1 < 1 || rot->n2 < 1 || rot->n1 > 64 || rot->n2 > 64) return fail(RQ_ESHAPE, "KRON factors must be 1..64 wide");
    if ((int64_t)rot->n1 * rot->n2 != K) return fail(RQ_ESHAPE, "KRON needs K == n1*n2");
    if (!rot->p1 || !rot->p2) return fail(RQ_EINVAL, "KRON factors p1/p2 are NULL");
    if (!aligned(rot->p1, 4) || !aligned(rot->p2, 4) || !aligned(rot->chan_scale, 4)) return fail(RQ_EALIGN, "KRON buffers must be 4-byte aligned");
  }
  if (T > 0) {
    if (!x || !q || !scale) return fail(RQ_EINVAL, "x, q and scale are required");
    if (ldx < K || ldx % 8) return fail(RQ_EALIGN, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return fail(RQ_EALIGN, "x and q must be 16-byte aligned, scale 4-byte");
    if (qd->n_out > 0 && (!x_out || !aligned(x_out, 2))) return fail(RQ_EINVAL, "x_out is required when n_out > 0");
    if (qd->n_out > 0 && !aligned(qd->outlier_idx, 4)) return fail(RQ_EALIGN, "outlier_idx must be 4-byte aligned");
  }
  if (rot->kind == RQ_ROT_NONE && (K % 32 || K > kSplitMaxK))
    return fail(RQ_ESHAPE, "without a rotation K must be a multiple of 32 and at most %d (K=%lld)", kSplitMaxK, (long long)K);
  if ((rot->kind == RQ_ROT_HADAMARD || rot->kind == RQ_ROT_GSR) && K != 4096 && rq::rowlds_smem_bytes(K) > kMaxLds)
    return fail(RQ_ESHAPE, "row of K=%lld does not fit in LDS", (long long)K);
  return ok();
}

// Dispatch of the quantizer kernels.  `divide` selects the weight side of the
// affine transform (factors already inverted-transposed, scale divides).
rq_status run_quant(const void *x, int64_t T, int64_t K, int64_t ldx, const rq_rot_desc *rot,
                    const rq_quant_desc *qd, const float *fa, const float *fb, bool divide,
                    uint8_t *q, float *scale, int32_t *zero, int32_t *code_sum, void *x_out,
                    hipStream_t st) {
  if (T == 0) return ok();
  hipError_t e;
  if (rot->kind == RQ_ROT_KRON) {
    e = rq::launch_kron(x, T, ldx, rot->n1, rot->n2, fa, fb, rot->chan_scale, divide,
                        qd->clip_ratio, q, scale, code_sum, st);
    return hip_status(e, "kron_quant launch");
  }
  int span_log2 = 0;
  if (rot->kind == RQ_ROT_HADAMARD) span_log2 = ilog2(K);
  if (rot->kind == RQ_ROT_GSR) span_log2 = ilog2(rot->block);
  const float norm = span_log2 ? (float)(1.0 / sqrt((double)(int64_t(1) << span_log2))) : 1.0f;
  const bool gsr = rot->kind == RQ_ROT_GSR;
  if (K == 4096 && (rot->kind == RQ_ROT_HADAMARD || rot->kind == RQ_ROT_GSR) && !qd->asymmetric && qd->n_out == 0) {
    e = rq::launch_fwht4096(x, T, ldx, gsr, span_log2, norm, qd->clip_ratio, q, scale, code_sum, st);
    return hip_status(e, "fwht4096_quant launch");
  }
  if (rot->kind == RQ_ROT_NONE && qd->bits == 8) {
    e = rq::launch_split8(x, T, K, ldx, qd->asymmetric != 0, qd->clip_ratio, qd->row_clip, qd->outlier_idx,
                          qd->n_out, q, scale, zero, code_sum, x_out, st);
    return hip_status(e, "split_quant8 launch");
  }
  if (rot->kind == RQ_ROT_NONE) {
    e = rq::launch_split(x, T, K, ldx, qd->asymmetric != 0, qd->clip_ratio, qd->row_clip, qd->outlier_idx,
                         qd->n_out, q, scale, zero, code_sum, x_out, st);
    return hip_status(e, "split_quant launch");
  }
  e = rq::launch_rowlds(x, T, K, ldx, span_log2, gsr, norm, qd->clip_ratio, q, scale, code_sum, st);
  return hip_status(e, "rowlds_quant launch");
}

}  // namespace

extern "C" {

int rq_abi_version(void) { return RQ_ABI_VERSION; }

const char *rq_last_error(void) { return g_err; }

const char *rq_status_string(rq_status s) {
  switch (s) {
    case RQ_OK: return "RQ_OK";
    case RQ_EINVAL: return "RQ_EINVAL: invalid argument";
    case RQ_ESHAPE: return "RQ_ESHAPE: unsupported shape";
    case RQ_EALIGN: return "RQ_EALIGN: misaligned pointer or leading dimension";
    case RQ_EHIP: return "RQ_EHIP: HIP runtime error";
  }
  return "unknown rq_status";
}

rq_status rq_rotate_quant(const void *x, int64_t T, int64_t K, int64_t ldx, const rq_rot_desc *rot,
                          const rq_quant_desc *qd, uint8_t *q, float *scale, int32_t *zero,
                          int32_t *code_sum, void *x_out, void *stream) {
  rq_status s = check_quant(x, T, K, ldx, rot, qd, q, scale, x_out);
  if (s != RQ_OK) return s;
  if (T > 0 && qd->asymmetric && (!zero || !aligned(zero, 4))) return fail(RQ_EINVAL, "zero is required for asymmetric codes");
  if (T > 0 && code_sum && !aligned(code_sum, 4)) return fail(RQ_EALIGN, "code_sum must be 4-byte aligned");
  return run_quant(x, T, K, ldx, rot, qd, rot->p1, rot->p2, false, q, scale, zero, code_sum, x_out,
                   (hipStream_t)stream);
}

int64_t rq_prepare_weights_workspace_bytes(const rq_rot_desc *rot) {
  if (!rot || rot->kind != RQ_ROT_KRON) return 0;
  const int64_t a = (int64_t)rot->n1 * rot->n1 * 4, b = (int64_t)rot->n2 * rot->n2 * 4;
  return ((a + 255) / 256) * 256 + b;
}

rq_status rq_prepare_weights_noalloc(const void *w, int64_t N, int64_t K, int64_t ldw, const rq_rot_desc *rot,
                                     const rq_quant_desc *qd, uint8_t *qw, float *sw, int32_t *w_rowsum,
                                     void *w_out, void *stream) {
  if (!rot) return fail(RQ_EINVAL, "rot and qd descriptors are required");
  const int64_t need = rq_prepare_weights_workspace_bytes(rot);
  if (need > kScratchBytes)
    return fail(RQ_ESHAPE, "the transform needs %lld bytes of scratch, above the %lld this entry point holds",
                (long long)need, (long long)kScratchBytes);
  void *ptr = nullptr;
  if (need > 0 && N > 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(RQ_EINVAL, "device id %d is not below %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch_ptr[dev] = nullptr;
        return hip_status(e, "hipGetSymbolAddress(scratch)");
      }
    }
    ptr = g_scratch_ptr[dev];
  }
  return rq_prepare_weights(w, N, K, ldw, rot, qd, qw, sw, w_rowsum, w_out, ptr, need > 0 ? kScratchBytes : 0,
                            stream);
}

rq_status rq_prepare_weights(const void *w, int64_t N, int64_t K, int64_t ldw, const rq_rot_desc *rot,
                             const rq_quant_desc *qd, uint8_t *qw, float *sw, int32_t *w_rowsum,
                             void *w_out, void *workspace, int64_t workspace_bytes, void *stream) {
  rq_status s = check_quant(w, N, K, ldw, rot, qd, qw, sw, w_out);
  if (s != RQ_OK) return s;
  if (qd->asymmetric) return fail(RQ_EINVAL, "weights are quantized symmetrically");
  if (N > 0 && w_rowsum && !aligned(w_rowsum, 4)) return fail(RQ_EALIGN, "w_rowsum must be 4-byte aligned");
  const int64_t need = rq_prepare_weights_workspace_bytes(rot);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return fail(RQ_EINVAL, "KRON weights need a 256-byte aligned workspace of %lld bytes", (long long)need);
  hipStream_t st = (hipStream_t)stream;
  const float *fa = rot->p1, *fb = rot->p2;
  if (rot->kind == RQ_ROT_KRON && N > 0) {
    float *o1 = (float *)workspace;
    float *o2 = (float *)((char *)workspace + ((int64_t)rot->n1 * rot->n1 * 4 + 255) / 256 * 256);
    hipError_t e = rq::launch_kron_inverse_t(rot->p1, rot->n1, o1, rot->p2, rot->n2, o2, st);
    if (e != hipSuccess) return hip_status(e, "kron_inverse_t launch");
    fa = o1;
    fb = o2;
  }
  return run_quant(w, N, K, ldw, rot, qd, fa, fb, true, qw, sw, nullptr, w_rowsum, w_out, st);
}

rq_status rq_search_weight_clip(const void *w, int64_t N, int64_t K, int64_t ldw, const rq_quant_desc *qd,
                                int32_t steps, float *clip_out, void *stream) {
  if (!qd) return fail(RQ_EINVAL, "the quantizer descriptor is required");
  if (qd->asymmetric) return fail(RQ_EINVAL, "weights are quantized symmetrically");
  if (qd->bits != 0 && qd->bits != 4 && qd->bits != 8) return fail(RQ_EINVAL, "bits=%d must be 4 or 8", qd->bits);
  if (steps < 1 || steps > 100000) return fail(RQ_EINVAL, "steps=%d must be in [1, 100000]", steps);
  if (N < 0 || K <= 0) return fail(RQ_EINVAL, "need N >= 0, K > 0");
  if (K % 32 || K > 32768) return fail(RQ_ESHAPE, "K=%lld must be a multiple of 32 and at most 32768", (long long)K);
  if (qd->n_out < 0 || qd->n_out >= K) return fail(RQ_EINVAL, "n_out=%d out of range", qd->n_out);
  if (qd->n_out > 0 && (!qd->outlier_idx || !aligned(qd->outlier_idx, 4))) return fail(RQ_EINVAL, "outlier_idx is required (4-byte aligned) with n_out > 0");
  if (N == 0) return ok();
  if (!w || !aligned(w, 16)) return fail(RQ_EALIGN, "w is required, 16-byte aligned");
  if (ldw < K || ldw % 8) return fail(RQ_EALIGN, "ldw=%lld must be >= K and a multiple of 8", (long long)ldw);
  if (!clip_out || !aligned(clip_out, 4)) return fail(RQ_EALIGN, "clip_out is required, 4-byte aligned");
  return hip_status(rq::launch_clip_search(w, N, K, ldw, qd->outlier_idx, qd->n_out, qd->bits == 8 ? 8 : 4, steps,
                                           clip_out, (hipStream_t)stream), "clip search launch");
}

static rq_status check_gemm(const uint8_t *qx, int64_t T, int64_t K, const uint8_t *qw, int64_t N,
                            const void *out, int64_t ldo, size_t out_elem) {
  if (T < 0 || K <= 0 || N < 1) return fail(RQ_EINVAL, "need T >= 0, K > 0, N >= 1");
  if (K % 64) return fail(RQ_ESHAPE, "K=%lld must be a multiple of 64", (long long)K);
  if (K > kMaxK) return fail(RQ_ESHAPE, "K=%lld exceeds %lld", (long long)K, (long long)kMaxK);
  if ((T + 127) / 128 > 65535 || ((T + 63) / 64) * ((N + 63) / 64) > 2147483647LL)
    return fail(RQ_ESHAPE, "T=%lld, N=%lld exceed the grid limit", (long long)T, (long long)N);
  if (T > 0) {
    if (!qx || !qw || !out) return fail(RQ_EINVAL, "qx, qw and the output are required");
    if (!aligned(qx, 16) || !aligned(qw, 16)) return fail(RQ_EALIGN, "qx and qw must be 16-byte aligned");
    if (!aligned(out, out_elem)) return fail(RQ_EALIGN, "the output must be aligned to its element size");
    if (ldo < N) return fail(RQ_EALIGN, "leading dimension %lld must be >= N=%lld", (long long)ldo, (long long)N);
  }
  return ok();
}

rq_status rq_w4a4_linear(const uint8_t *qx, const float *sx, int64_t T, int64_t K, const uint8_t *qw,
                         const float *sw, int64_t N, void *y, int64_t ldy, void *stream) {
  rq_status s = check_gemm(qx, T, K, qw, N, y, ldy, 2);
  if (s != RQ_OK) return s;
  if (T == 0) return ok();
  if (!sx || !sw || !aligned(sx, 4) || !aligned(sw, 4)) return fail(RQ_EINVAL, "sx and sw are required (4-byte aligned)");
  rq::GemmArgs p{qx, qw, T, N, K / 2, sx, sw, nullptr, nullptr, nullptr, nullptr, 0, y, ldy};
  return hip_status(rq::launch_gemm(p, false, 1, (hipStream_t)stream), "gemm launch");
}

rq_status rq_mixed_outlier_linear(const uint8_t *qx, const float *sx, const int32_t *zx, int64_t T,
                                  int64_t K_int, const uint8_t *qw, const float *sw,
                                  const int32_t *w_rowsum, int64_t N, const void *x_out,
                                  const void *w_out, int32_t n_out, void *y, int64_t ldy,
                                  void *stream) {
  rq_status s = check_gemm(qx, T, K_int, qw, N, y, ldy, 2);
  if (s != RQ_OK) return s;
  if (n_out < 0 || n_out % 32) return fail(RQ_ESHAPE, "n_out=%d must be a non-negative multiple of 32", n_out);
  if (T == 0) return ok();
  if (!sx || !sw || !aligned(sx, 4) || !aligned(sw, 4)) return fail(RQ_EINVAL, "sx and sw are required (4-byte aligned)");
  if (zx && (!w_rowsum || !aligned(zx, 4) || !aligned(w_rowsum, 4))) return fail(RQ_EINVAL, "asymmetric codes need zx and w_rowsum (4-byte aligned)");
  if (n_out > 0 && (!x_out || !w_out || !aligned(x_out, 16) || !aligned(w_out, 16))) return fail(RQ_EINVAL, "x_out and w_out are required (16-byte aligned) when n_out > 0");
  rq::GemmArgs p{qx, qw, T, N, K_int / 2, sx, sw, zx, w_rowsum, (const __half *)x_out,
                 (const __half *)w_out, n_out, y, ldy};
  return hip_status(rq::launch_gemm(p, zx != nullptr, 2, (hipStream_t)stream), "gemm launch");
}

rq_status rq_quant_decode_linear(const void *x, int64_t T, int64_t K, int64_t ldx, const rq_quant_desc *qd,
                                 const uint8_t *qw, const float *sw, const int32_t *w_rowsum, int64_t N,
                                 const void *w_out, void *y, int64_t ldy, void *stream) {
  if (!qd) return fail(RQ_EINVAL, "the quantizer descriptor is required");
  if (T < 0 || K <= 0 || N < 1) return fail(RQ_EINVAL, "need T >= 0, K > 0, N >= 1");
  const int n_out = qd->n_out;
  if (n_out < 0 || n_out >= K || n_out % 32) return fail(RQ_ESHAPE, "n_out=%d must be a multiple of 32 below K", n_out);
  if (n_out > 0 && !qd->outlier_idx) return fail(RQ_EINVAL, "outlier_idx is NULL with n_out > 0");
  if (!(qd->clip_ratio > 0.0f && qd->clip_ratio <= 1.0f)) return fail(RQ_EINVAL, "clip_ratio must be in (0, 1]");
  if (qd->asymmetric && qd->clip_ratio != 1.0f) return fail(RQ_EINVAL, "asymmetric quantization takes clip_ratio 1");
  if (qd->bits != 0 && qd->bits != 4) return fail(RQ_ESHAPE, "the fused decode form takes 4-bit codes");
  if (qd->row_clip) return fail(RQ_ESHAPE, "the fused decode form takes one clip ratio");
  if (T > 16) return fail(RQ_ESHAPE, "the fused decode form takes T <= 16 (T=%lld)", (long long)T);
  if (K % 32 || K > 8192 || (K - n_out) % 128)
    return fail(RQ_ESHAPE, "the fused decode form needs K %% 32 == 0, K <= 8192, (K - n_out) %% 128 == 0 (K=%lld)", (long long)K);
  if (T == 0) return ok();
  if (!x || !aligned(x, 16)) return fail(RQ_EALIGN, "x is required, 16-byte aligned");
  if (ldx < K || ldx % 8) return fail(RQ_EALIGN, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
  if (!qw || !aligned(qw, 16)) return fail(RQ_EALIGN, "qw is required, 16-byte aligned");
  if (!sw || !aligned(sw, 4)) return fail(RQ_EINVAL, "sw is required (4-byte aligned)");
  if (qd->asymmetric && (!w_rowsum || !aligned(w_rowsum, 4))) return fail(RQ_EINVAL, "asymmetric codes need w_rowsum (4-byte aligned)");
  if (n_out > 0 && (!w_out || !aligned(w_out, 16))) return fail(RQ_EINVAL, "w_out is required (16-byte aligned) when n_out > 0");
  if (n_out > 0 && !aligned(qd->outlier_idx, 4)) return fail(RQ_EALIGN, "outlier_idx must be 4-byte aligned");
  if (!y || !aligned(y, 2)) return fail(RQ_EALIGN, "y is required, 2-byte aligned");
  if (ldy < N) return fail(RQ_EALIGN, "leading dimension %lld must be >= N=%lld", (long long)ldy, (long long)N);
  const bool asym = qd->asymmetric != 0;
  const int mode = (asym || n_out > 0) ? 2 : 1;
  rq::GemmArgs p{nullptr, qw, T, N, (K - n_out) / 2, nullptr, sw, nullptr, asym ? w_rowsum : nullptr,
                 nullptr, (const __half *)w_out, n_out, y, ldy};
  rq::FuseArgs f{(const __half *)x, ldx, (int)K, qd->clip_ratio, qd->outlier_idx, 0, 1.0f};
  if (!rq::decode_fused_fits(p, f)) return fail(RQ_ESHAPE, "T=%lld, K=%lld do not fit the fused decode form", (long long)T, (long long)K);
  return hip_status(rq::launch_decode_fused(p, f, asym, mode, (hipStream_t)stream), "fused decode launch");
}

rq_status rq_rotate_quant_decode_linear(const void *x, int64_t T, int64_t K, int64_t ldx, const rq_rot_desc *rot,
                                        const rq_quant_desc *qd, const uint8_t *qw, const float *sw,
                                        const int32_t *w_rowsum, int64_t N, const void *w_out, void *y,
                                        int64_t ldy, void *stream) {
  if (!rot || !qd) return fail(RQ_EINVAL, "rot and qd descriptors are required");
  if (rot->kind == RQ_ROT_NONE)
    return rq_quant_decode_linear(x, T, K, ldx, qd, qw, sw, w_rowsum, N, w_out, y, ldy, stream);
  if (rot->kind != RQ_ROT_HADAMARD && rot->kind != RQ_ROT_GSR)
    return fail(rot->kind == RQ_ROT_KRON ? RQ_ESHAPE : RQ_EINVAL, "the fused decode form takes NONE, HADAMARD or GSR");
  if (T < 0 || K <= 0 || N < 1) return fail(RQ_EINVAL, "need T >= 0, K > 0, N >= 1");
  if (K != 4096) return fail(RQ_ESHAPE, "the rotated fused decode form takes K == 4096 (K=%lld)", (long long)K);
  if (rot->kind == RQ_ROT_GSR && !(pow2(rot->block) && rot->block >= 8 && rot->block <= 64))
    return fail(RQ_ESHAPE, "the rotated fused decode form takes GSR blocks of 8 to 64 (block=%d)", rot->block);
  if (qd->asymmetric || qd->n_out || qd->row_clip || (qd->bits != 0 && qd->bits != 4))
    return fail(RQ_ESHAPE, "the rotated fused decode form takes symmetric 4-bit codes without outliers or row clips");
  if (!(qd->clip_ratio > 0.0f && qd->clip_ratio <= 1.0f)) return fail(RQ_EINVAL, "clip_ratio must be in (0, 1]");
  if (T > 16) return fail(RQ_ESHAPE, "the fused decode form takes T <= 16 (T=%lld)", (long long)T);
  if (T == 0) return ok();
  if (!x || !aligned(x, 16)) return fail(RQ_EALIGN, "x is required, 16-byte aligned");
  if (ldx < K || ldx % 8) return fail(RQ_EALIGN, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
  if (!qw || !aligned(qw, 16)) return fail(RQ_EALIGN, "qw is required, 16-byte aligned");
  if (!sw || !aligned(sw, 4)) return fail(RQ_EINVAL, "sw is required (4-byte aligned)");
  if (!y || !aligned(y, 2)) return fail(RQ_EALIGN, "y is required, 2-byte aligned");
  if (ldy < N) return fail(RQ_EALIGN, "leading dimension %lld must be >= N=%lld", (long long)ldy, (long long)N);
  const int blog2 = rot->kind == RQ_ROT_GSR ? ilog2(rot->block) : 0;
  const float norm = blog2 ? (float)(1.0 / sqrt((double)rot->block)) : 1.0f;
  rq::GemmArgs p{nullptr, qw, T, N, K / 2, nullptr, sw, nullptr, nullptr, nullptr, nullptr, 0, y, ldy};
  rq::FuseArgs f{(const __half *)x, ldx, (int)K, qd->clip_ratio, nullptr, blog2, norm};
  if (!rq::decode_fused_rot_fits(p, f)) return fail(RQ_ESHAPE, "T=%lld does not fit the rotated fused decode form", (long long)T);
  return hip_status(rq::launch_decode_fused_rot(p, f, (hipStream_t)stream), "rotated fused decode launch");
}

static rq_status kv_check_shape(int64_t T, int64_t K, int32_t group) {
  if (T < 0 || K <= 0) return fail(RQ_EINVAL, "need T >= 0, K > 0");
  if (group != 64 && group != 128 && group != 256) return fail(RQ_ESHAPE, "group=%d must be 64, 128 or 256", group);
  if (K % group) return fail(RQ_ESHAPE, "K=%lld must be a multiple of group=%d", (long long)K, group);
  if (K > (int64_t(1) << 21)) return fail(RQ_ESHAPE, "K=%lld is above 2^21 channels", (long long)K);
  if (T > (int64_t(1) << 40) / (K / group)) return fail(RQ_ESHAPE, "T=%lld is too large", (long long)T);
  return RQ_OK;
}

static rq_status kv_check_tensor(const char *what, const void *x, int64_t ldx, int64_t K, const uint8_t *q,
                                 const float *scale, const int32_t *zero) {
  if (!x || !aligned(x, 16)) return fail(RQ_EALIGN, "%sx is required, 16-byte aligned", what);
  if (ldx < K || ldx % 8) return fail(RQ_EALIGN, "%sldx=%lld must be >= K and a multiple of 8", what, (long long)ldx);
  if (!q || !aligned(q, 4)) return fail(RQ_EALIGN, "%sq is required, 4-byte aligned", what);
  if (!scale || !aligned(scale, 4)) return fail(RQ_EALIGN, "%sscale is required, 4-byte aligned", what);
  if (!zero || !aligned(zero, 4)) return fail(RQ_EALIGN, "%szero is required, 4-byte aligned", what);
  return RQ_OK;
}

rq_status rq_kv_rotate_quant(const void *x, int64_t T, int64_t K, int64_t ldx, int32_t group,
                             int32_t rotate, uint8_t *q, float *scale, int32_t *zero, void *stream) {
  if (rq_status st = kv_check_shape(T, K, group)) return st;
  if (T == 0) return ok();
  if (rq_status st = kv_check_tensor("", x, ldx, K, q, scale, zero)) return st;
  return hip_status(rq::launch_group_quant(x, T, K, ldx, group, rotate != 0, q, scale, zero, (hipStream_t)stream),
                    "kv quantizer launch");
}

rq_status rq_kv_cache_quant(const rq_kv_tensor *keys, const rq_kv_tensor *values, int64_t T, int64_t K,
                            int32_t group, void *stream) {
  if (!keys || !values) return fail(RQ_EINVAL, "keys and values descriptors are required");
  if (rq_status st = kv_check_shape(T, K, group)) return st;
  if (T == 0) return ok();
  if (rq_status st = kv_check_tensor("keys: ", keys->x, keys->ldx, K, keys->q, keys->scale, keys->zero)) return st;
  if (rq_status st = kv_check_tensor("values: ", values->x, values->ldx, K, values->q, values->scale, values->zero))
    return st;
  const int64_t G = T * (K / group);
  const uintptr_t kb[3] = {(uintptr_t)keys->q, (uintptr_t)keys->scale, (uintptr_t)keys->zero};
  const uintptr_t vb[3] = {(uintptr_t)values->q, (uintptr_t)values->scale, (uintptr_t)values->zero};
  const uintptr_t len[3] = {(uintptr_t)(T * (K / 2)), (uintptr_t)(G * 4), (uintptr_t)(G * 4)};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      if (kb[i] < vb[j] + len[j] && vb[j] < kb[i] + len[i])
        return fail(RQ_EINVAL, "keys' and values' output buffers overlap");
  const rq::KvTensor k{(const __half *)keys->x, keys->ldx, keys->q, keys->scale, keys->zero};
  const rq::KvTensor v{(const __half *)values->x, values->ldx, values->q, values->scale, values->zero};
  return hip_status(rq::launch_group_quant_pair(k, keys->rotate != 0, v, values->rotate != 0, T, K, group,
                                                (hipStream_t)stream),
                    "kv cache quantizer launch");
}

rq_status rq_w8a8_linear(const uint8_t *qx, const float *sx, const int32_t *zx, int64_t T, int64_t K_int,
                         const uint8_t *qw, const float *sw, const int32_t *w_rowsum, int64_t N,
                         const void *x_out, const void *w_out, int32_t n_out, void *y, int64_t ldy,
                         void *stream) {
  rq_status s = check_gemm(qx, T, K_int, qw, N, y, ldy, 2);
  if (s != RQ_OK) return s;
  if (K_int > 32768) return fail(RQ_ESHAPE, "8-bit K_int=%lld exceeds 32768", (long long)K_int);
  if (n_out < 0 || n_out % 32) return fail(RQ_ESHAPE, "n_out=%d must be a non-negative multiple of 32", n_out);
  if (T == 0) return ok();
  if (!sx || !sw || !aligned(sx, 4) || !aligned(sw, 4)) return fail(RQ_EINVAL, "sx and sw are required (4-byte aligned)");
  if (zx && (!w_rowsum || !aligned(zx, 4) || !aligned(w_rowsum, 4))) return fail(RQ_EINVAL, "asymmetric codes need zx and w_rowsum (4-byte aligned)");
  if (n_out > 0 && (!x_out || !w_out || !aligned(x_out, 16) || !aligned(w_out, 16))) return fail(RQ_EINVAL, "x_out and w_out are required (16-byte aligned) when n_out > 0");
  rq::GemmArgs p{qx, qw, T, N, K_int, sx, sw, zx, w_rowsum, (const __half *)x_out,
                 (const __half *)w_out, n_out, y, ldy};
  return hip_status(rq::launch_gemm_ra8(p, zx != nullptr, 2, (hipStream_t)stream), "gemm launch");
}

rq_status rq_w8a8_gemm_i32(const uint8_t *qx, int32_t x_unsigned, int64_t T, int64_t K, const uint8_t *qw,
                           const int32_t *w_rowsum, int64_t N, int32_t *acc, int64_t ldacc, void *stream) {
  rq_status s = check_gemm(qx, T, K, qw, N, acc, ldacc, 4);
  if (s != RQ_OK) return s;
  if (K > 32768) return fail(RQ_ESHAPE, "8-bit K=%lld exceeds 32768", (long long)K);
  if (T == 0) return ok();
  if (x_unsigned && (!w_rowsum || !aligned(w_rowsum, 4))) return fail(RQ_EINVAL, "unsigned codes need w_rowsum (4-byte aligned)");
  rq::GemmArgs p{qx, qw, T, N, K, nullptr, nullptr, nullptr, x_unsigned ? w_rowsum : nullptr, nullptr, nullptr, 0, acc, ldacc};
  return hip_status(rq::launch_gemm_ra8(p, x_unsigned != 0, 0, (hipStream_t)stream), "gemm launch");
}

rq_status rq_w4a4_gemm_i32(const uint8_t *qx, int32_t x_unsigned, int64_t T, int64_t K, const uint8_t *qw,
                           int64_t N, int32_t *acc, int64_t ldacc, void *stream) {
  rq_status s = check_gemm(qx, T, K, qw, N, acc, ldacc, 4);
  if (s != RQ_OK) return s;
  if (T == 0) return ok();
  rq::GemmArgs p{qx, qw, T, N, K / 2, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, acc, ldacc};
  return hip_status(rq::launch_gemm(p, x_unsigned != 0, 0, (hipStream_t)stream), "gemm launch");
}

}  // extern "C"
