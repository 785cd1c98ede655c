/*
 * rq.h -- C ABI of the online-rotation + W4A4 linear library for MI355X (gfx950).
 *
 * The library computes the quantized linear layer that the rotation-based
 * 4-bit methods share:
 *
 *     Y = dequant( Q(X . R) . Q(W . R^{-T})^T )   [+ X_out . W_out^T]
 *
 * R is an online per-token transform: a normalized Walsh-Hadamard transform
 * ("QuaRot & SpinQuant" blog, section 2), a block-diagonal sequency-ordered
 * Walsh rotation ("Grouped Sequency-arranged Rotation" abstract), or a
 * Kronecker affine transform with channel scaling and clipping (FlatQuant
 * article, section 2.3).  Q is per-token INT4 quantization; the product is an
 * INT4 x INT4 GEMM with INT32 accumulation, then per-token x per-channel
 * dequantization, with QUIK's FP16 outlier columns added (QUIK blog, "QUIK
 * quantization" parts 1 and 4).
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronizes; each call only enqueues
 *     kernels on `stream` (a hipStream_t passed as void*, NULL = default).
 *   - Arguments are checked on the host before anything is launched.  A
 *     failed check returns an error code, launches nothing and writes nothing.
 *     Kernel launch failures return RQ_EHIP.  rq_last_error() then holds a
 *     message (thread-local).  No exception or abort crosses the ABI.
 *   - Matrices are row-major.  fp16 is IEEE binary16.  Packed INT4 rows hold
 *     two codes per byte: element 2j in the low nibble, 2j+1 in the high
 *     nibble.  Symmetric codes are 4-bit two's complement in [-7, 7];
 *     asymmetric codes are unsigned in [0, 15].
 *   - Input matrices must be 16-byte aligned; outputs and fp32/int32
 *     vectors need the alignment of their element type.
 *   - Rounding is round-half-to-even throughout.
 *   - Calls on one stream run in order; the library keeps no state between
 *     calls except the thread-local error string.
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RQ_ABI_VERSION 2

typedef enum {
  RQ_OK = 0,
  RQ_EINVAL = 1, /* null pointer, unknown enum value, negative size, bad ratio */
  RQ_ESHAPE = 2, /* size or transform the library does not support           */
  RQ_EALIGN = 3, /* pointer or leading dimension not aligned / too small       */
  RQ_EHIP = 4    /* a HIP launch or runtime call failed                        */
} rq_status;

typedef enum {
  RQ_ROT_NONE = 0,     /* identity (QUIK: no rotation)                        */
  RQ_ROT_HADAMARD = 1, /* full normalized Walsh-Hadamard over K, natural order */
  RQ_ROT_GSR = 2,      /* blockdiag of sequency-ordered Walsh blocks           */
  RQ_ROT_KRON = 3      /* diag(s) . (P1 kron P2)                               */
} rq_rot_kind;

/* Online transform R, applied to each row on the right: x' = x . R.
 *   HADAMARD  R = H_K, H[i][j] = (-1)^popcount(i&j) / sqrt(K).
 *             K a power of two, 64 <= K <= 32768.
 *   GSR       R = blockdiag(Wal_b, ..., Wal_b), Wal_b row s = the H_b row
 *             with exactly s sign changes.  b = `block`, a power of two,
 *             2 <= b <= 256, K % b == 0, K <= 32768.
 *   KRON      R = diag(chan_scale) . (P1 kron P2) with numpy's Kronecker
 *             index convention; per row, x' reshaped [n1, n2] = P1^T M P2 with
 *             M = (x * chan_scale) reshaped row-major.  K == n1 * n2,
 *             1 <= n1, n2 <= 64.  p1: fp32 [n1, n1], p2: fp32 [n2, n2],
 *             chan_scale: fp32 [K] or NULL (all ones).
 *   NONE      K % 32 == 0, K <= 32768.
 * Rotations (kind != NONE) require n_out == 0 in the quantizer descriptor. */
typedef struct {
  int32_t kind;
  int32_t block;
  int32_t n1, n2;
  const float *p1;
  const float *p2;
  const float *chan_scale;
} rq_rot_desc;

/* Per-row quantizer, at bits = 4 (the default; 0 means 4) or bits = 8.
 *   asymmetric == 0: scale = fp32(clip_ratio * max|x'| / 7),
 *                    code = clamp(rne(x'/scale), -7, 7)
 *                    (SpinQuant OpenReview, first reviewer Q1/A1: min-max onto
 *                    +-(2^{N-1}-1); FlatQuant article section 2.3: clipping).
 *   asymmetric == 1: lo = min(min x, 0), hi = max(max x, 0),
 *                    scale = fp32((hi - lo) / 15), zero = clamp(rne(-lo/scale), 0, 15),
 *                    code = clamp(rne(x/scale) + zero, 0, 15)
 *                    (QUIK blog part 1: asymmetric per-token dynamic).
 *                    clip_ratio must be 1.
 *   A row whose range is 0 gets scale 0, zero 0 and all codes 0.
 *   outlier_idx: device int32 [n_out], the columns kept in fp16 (QUIK blog
 *   parts 1 and 3).  Must be distinct and in [0, K); order does not matter:
 *   outlier columns are emitted in ascending column order, the other K - n_out
 *   columns keep their relative order.  Violating this gives unspecified
 *   values but never an out-of-bounds access.  n_out = 0: no split.
 *   bits == 8 (QUIK-8B, for the sensitive down projection: QUIK blog,
 *   "QUIK量化" part 3; the 8-bit layers take more outliers, experiments part 1
 *   and end-to-end speedup): the same forms with 127 in place of 7 and 255 in
 *   place of 15, one byte per code (signed codes as 8-bit two's complement);
 *   only without a rotation (kind NONE).  Other values of bits: RQ_EINVAL. */
typedef struct {
  int32_t asymmetric;
  float clip_ratio;
  const int32_t *outlier_idx;
  int32_t n_out;
  int32_t bits;
  /* device fp32 [rows] per-row clip ratios in (0, 1], used instead of
   * clip_ratio (symmetric codes without a rotation only; NULL: clip_ratio);
   * rq_search_weight_clip writes them. */
  const float *row_clip;
} rq_quant_desc;

/* rq_rotate_quant -- online transform + per-token INT4 quantization + packing.
 *   x        fp16 [T, ldx] (row t starts at x + t*ldx elements; ldx >= K, ldx % 8 == 0)
 *   q        out uint8 [T, (K - n_out)/2] packed codes (dense rows); at
 *            bits == 8, [T, K - n_out], one byte per code
 *   scale    out fp32 [T]
 *   zero     out int32 [T] (asymmetric only; NULL for symmetric)
 *   code_sum out int32 [T] sum of each row's codes (NULL to skip); the
 *            weight side uses it for the asymmetric zero-point correction
 *   x_out    out fp16 [T, n_out] outlier columns (NULL iff n_out == 0)
 * T == 0 is a no-op.  (K - n_out) must be a positive multiple of 64 (QUIK's
 * 8192 - 256 = 7936 qualifies).  Rows holding Inf or NaN get unspecified
 * codes, scale and zero point (never an out-of-range write). */
rq_status rq_rotate_quant(const void *x, int64_t T, int64_t K, int64_t ldx,
                          const rq_rot_desc *rot, const rq_quant_desc *qd,
                          uint8_t *q, float *scale, int32_t *zero, int32_t *code_sum,
                          void *x_out, void *stream);

/* rq_prepare_weights -- the offline weight side: W' = W . R^{-T}, then
 * per-output-channel symmetric INT4 (FlatQuant article section 3: per-channel
 * symmetric weights; "QuaRot & SpinQuant" blog section 1: the rotation folds
 * into the weights).  For HADAMARD/GSR/NONE, R^{-T} = R.  For KRON,
 * R^{-T} = diag(1/s) . (P1^{-T} kron P2^{-T}); the inverses are computed on
 * the GPU in fp64 (Gauss-Jordan, partial pivoting) into `workspace`.
 *   w        fp16 [N, ldw], qd: symmetric only, clip_ratio as for activations,
 *            outlier_idx/n_out select the fp16 columns (written to w_out [N, n_out])
 *   qw       out uint8 [N, (K - n_out)/2], sw out fp32 [N],
 *   w_rowsum out int32 [N] sum of each row's codes (NULL to skip)
 *   workspace device buffer of rq_prepare_weights_workspace_bytes(rot) bytes
 *            (may be NULL when that is 0).  A singular factor yields
 *            unspecified (non-finite) values, not an error. */
int64_t rq_prepare_weights_workspace_bytes(const rq_rot_desc *rot);
rq_status rq_prepare_weights(const void *w, int64_t N, int64_t K, int64_t ldw,
                             const rq_rot_desc *rot, const rq_quant_desc *qd,
                             uint8_t *qw, float *sw, int32_t *w_rowsum, void *w_out,
                             void *workspace, int64_t workspace_bytes, void *stream);

/* rq_prepare_weights_noalloc -- rq_prepare_weights for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and the same results bit for bit.  The KRON
 * factors' inverse transposes go to a scratch array of 32768 bytes in the
 * library's own device memory, one per GPU, which each GPU keeps until the
 * process ends (its address is looked up on the first call on that device).
 * The call allocates and frees nothing.  Every call on one GPU shares that
 * GPU's scratch array, so calls that may overlap on one GPU (on different
 * streams, or from different threads) race on it: order them.  A transform
 * needing more than 32768 bytes of scratch returns RQ_ESHAPE (none does:
 * KRON factors are at most 64 x 64). */
rq_status rq_prepare_weights_noalloc(const void *w, int64_t N, int64_t K, int64_t ldw,
                                     const rq_rot_desc *rot, const rq_quant_desc *qd,
                                     uint8_t *qw, float *sw, int32_t *w_rowsum, void *w_out,
                                     void *stream);

/* rq_search_weight_clip -- QUIK's weight clipping by linear search (QUIK
 * blog, "QUIK量化" part 2), per output channel.  For each row n of w, the
 * candidate ratios c = fp32(k / steps), k = steps, ..., 1, are scored by
 *   err(c) = sum_k (w[n][k] - s_c * q_c[k])^2 over the normal columns,
 *   s_c = fp32(c * max|w[n][.]| / qmax), q_c = clamp(rne(w / s_c), -qmax, qmax),
 * qmax = 7 (bits 4) or 127 (bits 8), with the error summed in fp64; the
 * first minimum in that order (ties to the larger ratio) goes to
 * clip_out[n].  Pass clip_out as qd->row_clip to rq_prepare_weights.
 *   w        fp16 [N, ldw], ldw >= K, ldw % 8 == 0, 16-byte aligned
 *   qd       symmetric (asymmetric == 0); bits; outlier_idx / n_out select
 *            the fp16 columns, which take no part; clip_ratio, row_clip ignored
 *   steps    1 .. 100000 (100: ratios 0.01 .. 1.00)
 *   clip_out out fp32 [N]
 * K % 32 == 0, K <= 32768.  N == 0 is a no-op. */
rq_status rq_search_weight_clip(const void *w, int64_t N, int64_t K, int64_t ldw,
                                const rq_quant_desc *qd, int32_t steps, float *clip_out,
                                void *stream);

/* rq_w4a4_linear -- y[t][n] = fp16( acc[t][n] * sx[t] * sw[n] ),
 * acc = sum_k qx[t][k] * qw[n][k] in INT32 (QUIK blog part 4), symmetric codes.
 *   qx uint8 [T, K/2], sx fp32 [T], qw uint8 [N, K/2], sw fp32 [N],
 *   y fp16 [T, ldy] (ldy >= N).  K % 64 == 0, 0 < K <= 65536, N >= 1,
 *   ceil(T/128) <= 65535.
 * The scale product is formed in fp32 and rounded once to fp16. */
rq_status rq_w4a4_linear(const uint8_t *qx, const float *sx, int64_t T, int64_t K,
                         const uint8_t *qw, const float *sw, int64_t N,
                         void *y, int64_t ldy, void *stream);

/* rq_mixed_outlier_linear -- QUIK's mixed-precision linear (QUIK blog part 1):
 *   y[t][n] = fp16( (acc[t][n] - zx[t]*w_rowsum[n]) * sx[t] * sw[n]
 *                   + sum_j x_out[t][j] * w_out[n][j] )
 *   qx uint8 [T, K_int/2] asymmetric codes (zx int32 [T]); if zx is NULL the
 *   codes are symmetric and w_rowsum may be NULL.  qw/sw/w_rowsum as written by
 *   rq_prepare_weights.  x_out fp16 [T, n_out], w_out fp16 [N, n_out]
 *   (n_out % 32 == 0, may be 0 with NULL pointers).  The outlier product
 *   accumulates in fp32 on FP16 matrix cores; one fp16 rounding at the end. */
rq_status rq_mixed_outlier_linear(const uint8_t *qx, const float *sx, const int32_t *zx,
                                  int64_t T, int64_t K_int,
                                  const uint8_t *qw, const float *sw, const int32_t *w_rowsum,
                                  int64_t N, const void *x_out, const void *w_out, int32_t n_out,
                                  void *y, int64_t ldy, void *stream);

/* rq_quant_decode_linear -- rq_rotate_quant with rot NONE followed by the
 * linear layer, in one launch, for decode batches: each workgroup quantizes
 * the T activation rows into on-chip memory and streams its weight rows
 * against them, so the activation codes, scales and x_out never reach HBM
 * (operator fusion of the online step to cut memory traffic: FlatQuant
 * article, section 1; SpinQuant OpenReview, latency discussion: fused tensor
 * core kernels).  The codes are those of rq_rotate_quant, and y is that of
 *   qd->asymmetric or qd->n_out > 0:
 *     rq_mixed_outlier_linear(codes, scale, zero or NULL, ..., w_rowsum, x_out, w_out, n_out)
 *   otherwise: rq_w4a4_linear(codes, scale, qw, sw),
 * bit for bit when T * ((K - n_out)/32 + n_out/8) <= 4096 (then the two calls
 * run the same decode kernel); beyond, the fp32 outlier product may differ in
 * its summation order.
 *   x        fp16 [T, ldx], ldx >= K, ldx % 8 == 0, 16-byte aligned
 *   qd       the quantizer of rq_rotate_quant (asymmetric, clip_ratio,
 *            outlier_idx [n_out]); n_out % 32 == 0
 *   qw, sw, w_rowsum (asymmetric only), w_out [N, n_out] (n_out > 0 only):
 *            as written by rq_prepare_weights with the same outlier_idx
 *   y        out fp16 [T, ldy], ldy >= N
 * Shapes: 1 <= T <= 16 (T == 0 is a no-op), K % 32 == 0, K <= 8192,
 * (K - n_out) % 128 == 0, 4-bit codes; otherwise RQ_ESHAPE (use the two calls). */
rq_status rq_quant_decode_linear(const void *x, int64_t T, int64_t K, int64_t ldx,
                                 const rq_quant_desc *qd, const uint8_t *qw, const float *sw,
                                 const int32_t *w_rowsum, int64_t N, const void *w_out,
                                 void *y, int64_t ldy, void *stream);

/* rq_rotate_quant_decode_linear -- rq_rotate_quant followed by the linear
 * layer in one launch for decode batches, with the online transform: each
 * workgroup transforms and quantizes the T activation rows into on-chip
 * memory and streams its weight rows against them (the online transform
 * fused with quantization, FlatQuant article section 2.3; the fused online
 * Hadamard's cost, SpinQuant OpenReview, the authors' answers on inference
 * overhead).
 *   rot NONE      exactly rq_quant_decode_linear (same arguments and limits).
 *   rot HADAMARD  (K == 4096) or GSR (K == 4096, block 8, 16, 32 or 64):
 *                 qd symmetric 4-bit, no outliers, no row clips, clip_ratio
 *                 in (0, 1]; the codes and scales are those of
 *                 rq_rotate_quant(x, rot, qd) and y that of rq_w4a4_linear on
 *                 them, bit for bit.  w_rowsum and w_out are ignored.
 *   x fp16 [T, ldx], ldx >= K, ldx % 8 == 0, 16-byte aligned; qw, sw as
 *   written by rq_prepare_weights with the same rot; y out fp16 [T, ldy].
 * 1 <= T <= 16 (T == 0 is a no-op); other shapes or transforms: RQ_ESHAPE.
 * Every workgroup repeats the transform of all T rows, so the fused form
 * pays off only for the smallest T (measured per T in the design notes). */
rq_status rq_rotate_quant_decode_linear(const void *x, int64_t T, int64_t K, int64_t ldx,
                                        const rq_rot_desc *rot, const rq_quant_desc *qd,
                                        const uint8_t *qw, const float *sw, const int32_t *w_rowsum,
                                        int64_t N, const void *w_out, void *y, int64_t ldy,
                                        void *stream);

/* rq_kv_rotate_quant -- the KV-cache quantizer: R3, a normalized
 * Walsh-Hadamard transform over each head's `group` channels (SpinQuant
 * OpenReview: the authors' answer on the number of rotation matrices, R3
 * rotates the KV cache before its quantization; first reviewer Q2/A2, the
 * rotation of queries and keys cancels in the attention product), then
 * group-wise asymmetric INT4 with one scale and
 * zero point per group (FlatQuant article, section 3: KV cache group-wise
 * asymmetric, group size 128).  For token t and group j of channels
 * [j*group, (j+1)*group):
 *   v        = x[t, group j] . H_group / sqrt(group)   (rotate != 0; else x)
 *   lo, hi   = min(min v, 0), max(max v, 0)
 *   scale    = fp32((hi - lo) / 15),  zero = clamp(rne(-lo / scale), 0, 15)
 *   code     = clamp(rne(v / scale) + zero, 0, 15);  v ~ (code - zero) * scale
 * H_group is the Sylvester Hadamard matrix (natural order).  The signed
 * sums are exact (fp64) and each v is rounded to fp32 once, so with
 * rotate != 0 a code whose v / scale lies within that rounding of a
 * half-integer may differ by one from an exact evaluation; with rotate == 0
 * the result is exact.
 *   x        fp16 [T, ldx], ldx >= K, ldx % 8 == 0, 16-byte aligned
 *   group    64, 128 or 256; K % group == 0, K <= 2^21
 *   q        out uint8 [T, K/2] packed codes, 4-byte aligned (16-byte
 *            aligned: the codes leave in 16-byte stores)
 *   scale    out fp32 [T, K/group];  zero out int32 [T, K/group]
 * T == 0 is a no-op. */
rq_status rq_kv_rotate_quant(const void *x, int64_t T, int64_t K, int64_t ldx, int32_t group,
                             int32_t rotate, uint8_t *q, float *scale, int32_t *zero,
                             void *stream);

/* One tensor of rq_kv_cache_quant: input rows, whether R3 applies, outputs
 * (each as the same-named argument of rq_kv_rotate_quant). */
typedef struct rq_kv_tensor {
  const void *x;  /* fp16 [T, ldx] */
  int64_t ldx;
  int32_t rotate; /* != 0: the per-group Walsh-Hadamard before quantization */
  uint8_t *q;     /* out uint8 [T, K/2] */
  float *scale;   /* out fp32 [T, K/group] */
  int32_t *zero;  /* out int32 [T, K/group] */
} rq_kv_tensor;

/* rq_kv_cache_quant -- the keys and the values of the same T tokens through
 * the KV-cache quantizer in one launch (SpinQuant OpenReview, the authors'
 * answer on the number of rotation matrices: R3 on the keys before the KV
 * cache is quantized; FlatQuant article, section 3: keys and values
 * group-wise asymmetric).  Each tensor's outputs are those of
 * rq_kv_rotate_quant(t->x, T, K, t->ldx, group, t->rotate, t->q, t->scale,
 * t->zero), bit for bit; keys and values take the same shape arguments and
 * limits, their buffers must not overlap.  keys and values are host
 * pointers to descriptors read during the call.  T == 0 is a no-op. */
rq_status rq_kv_cache_quant(const rq_kv_tensor *keys, const rq_kv_tensor *values, int64_t T, int64_t K,
                            int32_t group, void *stream);

/* rq_w8a8_linear -- the 8-bit form of rq_mixed_outlier_linear (QUIK-8B's
 * down projection: QUIK blog, "QUIK量化" part 3 and the QUIK-8B experiments;
 * INT32 accumulation, part 4; the FP16 outlier product added before the one
 * rounding, part 1):
 *   y[t][n] = fp16( (acc[t][n] - zx[t]*w_rowsum[n]) * sx[t] * sw[n]
 *                   + sum_j x_out[t][j] * w_out[n][j] ),
 *   acc = sum_k qx[t][k] * qw[n][k] over K_int one-byte codes.
 *   qx uint8 [T, K_int]: unsigned codes in [0, 255] with zero points zx int32
 *   [T]; zx NULL: signed codes in [-127, 127] (two's complement), w_rowsum
 *   may then be NULL.  qw/sw/w_rowsum as written by rq_prepare_weights with
 *   bits = 8.  x_out fp16 [T, n_out], w_out fp16 [N, n_out] (n_out % 32 == 0,
 *   may be 0 with NULL pointers).  K_int % 64 == 0, 0 < K_int <= 32768. */
rq_status rq_w8a8_linear(const uint8_t *qx, const float *sx, const int32_t *zx, int64_t T,
                         int64_t K_int, const uint8_t *qw, const float *sw,
                         const int32_t *w_rowsum, int64_t N, const void *x_out,
                         const void *w_out, int32_t n_out, void *y, int64_t ldy, void *stream);

/* rq_w8a8_gemm_i32 -- the raw INT32 accumulator of one-byte codes,
 * acc[t][n] = sum_k qx[t][k]*qw[n][k] (the integer product of QUIK-8B's
 * layers: QUIK blog, experiments part 2, on the kernels of "QUIK量化" part 4),
 * for bit-exact tests.  x_unsigned != 0:
 * qx codes are unsigned [0, 255] and w_rowsum (int32 [N], the row sums of qw)
 * is required; otherwise signed.  acc int32 [T, ldacc], ldacc >= N;
 * K % 64 == 0, K <= 32768. */
rq_status rq_w8a8_gemm_i32(const uint8_t *qx, int32_t x_unsigned, int64_t T, int64_t K,
                           const uint8_t *qw, const int32_t *w_rowsum, int64_t N, int32_t *acc,
                           int64_t ldacc, void *stream);

/* rq_w4a4_gemm_i32 -- the raw INT32 accumulator acc[t][n] = sum_k qx[t][k]*qw[n][k]
 * (the INT4 x INT4 product with INT32 accumulation: QUIK blog, "QUIK量化"
 * part 4), for bit-exact tests.  x_unsigned != 0: qx codes are unsigned [0, 15];
 * otherwise signed.  qx uint8 [T, K/2], qw uint8 [N, K/2] (both 16-byte
 * aligned), acc int32 [T, ldacc], ldacc >= N.  K % 64 == 0, 0 < K <= 65536,
 * N >= 1; the same status codes as rq_w4a4_linear.  T == 0 is a no-op. */
rq_status rq_w4a4_gemm_i32(const uint8_t *qx, int32_t x_unsigned, int64_t T, int64_t K,
                           const uint8_t *qw, int64_t N, int32_t *acc, int64_t ldacc,
                           void *stream);

const char *rq_status_string(rq_status s);
const char *rq_last_error(void);
int rq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */
