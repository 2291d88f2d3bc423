/*
 * qopt.h -- C ABI of the block-wise dynamic-tree 8-bit Adam library (libqopt.so),
 * for AMD Instinct MI355X (gfx950).
 *
 * The method: "8-BIT OPTIMIZERS VIA BLOCK-WISE QUANTIZATION", as summarised on the
 * page wiki.neutronadmin.com/news/16836.
 *   - §1 ("when the optimizer meets quantization"): Adam keeps two moments per
 *     parameter, the mean of the gradients and their uncentred variance;
 *     quantization stores values with fewer bits after normalising them into a
 *     range, dequantization maps them back.
 *   - §2 (opening): the optimizer state lives in low precision in GPU memory and is
 *     dequantized to a higher precision for the parameter update, then stored low
 *     precision again.
 *   - §2 "Block-wise Quantization": blocks of 2048 elements, each normalised into
 *     [-1, 1] by its own absolute maximum, with no synchronisation between blocks.
 *   - §2 "Dynamic Quantization": the dynamic-tree code (sign, exponent as a run of
 *     zeros, indicator bit, linear fraction) for the first moment, and its unsigned
 *     variant (sign bit reused as fraction) for the always-positive second moment.
 * fp32 master weights: the DeepSpeed / FSDP mixed-precision page (both keep fp32
 * master parameters for the optimizer step).
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device memory on the current HIP device; everything
 *     else is host memory.  The caller owns every buffer.  The library never
 *     allocates, frees or retains memory and keeps no per-call state, so calls on
 *     different streams are independent.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device work is
 *     enqueued on it and the call returns without synchronising; errors raised by
 *     the device surface when the caller synchronises.  (The bf16-parameter step
 *     and its traffic probe also use one stream of the library's per device, joined
 *     back into `stream`: see qopt_adam8bit_step.)
 *   - Arguments are checked on the host before anything is enqueued; a failed check
 *     returns an error code and enqueues nothing.  n == 0 is a no-op returning
 *     QOPT_OK.  No C++ exception crosses this interface.
 *   - Inputs must be finite.  NaN or infinite inputs give unspecified codes (never
 *     an out-of-bounds access).
 */
#ifndef QOPT_H
#define QOPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Elements per quantization block (§2 "Block-wise Quantization"). */
#define QOPT_BLOCK 2048

/* Return codes. */
typedef enum {
  QOPT_OK = 0,
  QOPT_EINVAL = 1,        /* bad argument: null pointer, negative size, bad value */
  QOPT_EUNSUPPORTED = 2,  /* unknown dtype or codebook kind */
  QOPT_EALIGN = 3,        /* pointer not aligned to its element size */
  QOPT_ELAUNCH = 4,       /* the HIP runtime refused a launch or a device query */
  QOPT_EINTERNAL = 5,     /* codebook construction violated an internal invariant */
  QOPT_ENOSPACE = 6       /* an allocation-free entry point's fixed scratch is too small */
} qopt_status;

/* Codebook kinds (§2 "Dynamic Quantization"). */
typedef enum {
  QOPT_CB_SIGNED = 0,   /* sign bit + 7-bit dynamic-tree magnitude: first moment  */
  QOPT_CB_UNSIGNED = 1  /* 8-bit dynamic-tree magnitude: second moment (>= 0)      */
} qopt_codebook_kind;

/* Element types of parameters and gradients. */
typedef enum { QOPT_F32 = 0, QOPT_BF16 = 1 } qopt_dtype;

#define QOPT_CODEBOOK_MAGIC 0x31424351u /* "QCB1" */
#define QOPT_MAX_BUCKETS 7168
#define QOPT_THRESH_LEN 272

/*
 * A codebook: how a code byte decodes, and the tables that encode a normalised
 * magnitude to its nearest code.  Built on the host by qopt_codebook_build, then
 * copied verbatim to device memory by the caller (sizeof(qopt_codebook) bytes, a
 * multiple of 16, 16-byte aligned) and passed to the device entry points.
 *
 * The code values (§2 "Dynamic Quantization", with these readings where the page is
 * silent): a magnitude bit pattern with e leading zeros, an indicator 1 bit and f
 * fraction bits of integer value j has the value 10^-e * (0.1 + 0.9 * (j+1) / 2^f),
 * rounded to the nearest binary32; the pattern 0 is 0.  Signed codes are
 * sign << 7 | 7-bit pattern (0x80 decodes to -0.0); unsigned codes are the 8-bit
 * pattern.  The code of a normalised magnitude a is the nearest table magnitude,
 * distances measured in binary32, ties to the smaller magnitude.
 *
 * Encoding from the tables: with key = (binary32 bits of a) >> 15 and
 * i = clamp(key - key0, 0, nbuckets - 1), the magnitude index is
 * bucket[i] + (a >= thresh[bucket[i] + 1]).  thresh[k] (k = 1 .. nmag-1) is the
 * least binary32 a whose nearest magnitude index is >= k; entries from nmag on are
 * +infinity.  Every bucket holds at most one threshold, which the builder checks.
 */
typedef struct qopt_codebook {
  uint32_t magic;       /* QOPT_CODEBOOK_MAGIC */
  uint32_t kind;        /* qopt_codebook_kind */
  uint32_t sign_mask;   /* OR-ed into the code of x < 0: 0x80 signed, 0 unsigned */
  uint32_t nmag;        /* number of magnitudes: 128 signed, 256 unsigned */
  uint32_t key0;        /* key of bucket 0 */
  uint32_t nbuckets;    /* buckets in use, <= QOPT_MAX_BUCKETS */
  uint32_t reserved[2];
  float decode[256];                /* value of each code byte, in [-1, 1] */
  float thresh[QOPT_THRESH_LEN];    /* decision thresholds, see above */
  uint8_t bucket[QOPT_MAX_BUCKETS]; /* magnitude index at each bucket start */
} qopt_codebook;

/*
 * Build the codebook of `kind` into *out (host memory).  Pure and thread-safe.
 * Returns QOPT_EUNSUPPORTED for an unknown kind, QOPT_EINVAL for out == NULL.
 */
int qopt_codebook_build(int kind, qopt_codebook* out);

/*
 * Block-wise quantization (§2 "Block-wise Quantization" + "Dynamic Quantization"):
 * for every block b of x_dev (elements [2048 b, min(2048 b + 2048, n)), the last
 * block may be short):
 *   A = max |x_i| over the block;  absmax_dev[b] = A, or 0 when A < 2^-126;
 *   r = 1 / A (binary32, correctly rounded), 0 when A < 2^-126;
 *   codes_dev[i] = nearest code of |x_i| * r, with cb->sign_mask OR-ed in when
 *                  x_i < 0 and A >= 2^-126.
 * x_dev: n fp32 values, 4-byte aligned.  codes_dev: n bytes.  absmax_dev:
 * ceil(n / 2048) fp32 values.  cb_dev: a device copy of qopt_codebook_build's output
 * (signed for values of either sign; unsigned encodes |x|).  Outputs must not
 * overlap the input.
 */
int qopt_quantize_blockwise(const qopt_codebook* cb_dev, const float* x_dev, int64_t n,
                            uint8_t* codes_dev, float* absmax_dev, void* stream);

/*
 * Block-wise dequantization (§1: the inverse map): y_dev[i] =
 * cb->decode[codes_dev[i]] * absmax_dev[i / 2048], one binary32 multiply.
 * Sizes as for qopt_quantize_blockwise.  y_dev may not overlap the inputs.
 */
int qopt_dequantize_blockwise(const qopt_codebook* cb_dev, const uint8_t* codes_dev,
                              const float* absmax_dev, int64_t n, float* y_dev,
                              void* stream);

/*
 * One tensor of a multi-tensor codec call.  All pointers are device memory:
 *   values  n fp32 values (read when quantizing, written when dequantizing),
 *           4-byte aligned;
 *   codes   n code bytes (written when quantizing, read when dequantizing);
 *   absmax  ceil(n / 2048) fp32 block maxima, 4-byte aligned.
 * Blocks restart at element 0 of every tensor.  Tensors whose values are 16-byte
 * aligned and whose codes are 4-byte aligned take the vector path.
 */
typedef struct qopt_codec_tensor {
  float* values;
  uint8_t* codes;
  float* absmax;
  int64_t n;
} qopt_codec_tensor;

/*
 * Multi-tensor forms of qopt_quantize_blockwise / qopt_dequantize_blockwise: the same
 * per-block results for every tensor of the host array `tensors`, in launches of equal
 * block counts with at most 48 tensor pieces and 2^18 blocks each (as for
 * qopt_adam8bit_step; calls of more than 2^18 blocks in launches of at most 2^16)
 * instead of one launch per tensor.  This is the moment codec of optimizer checkpoints (the
 * checkpoint-compression page, ExCP: momentum stored as a codebook plus per-element
 * indices).  Checks: tensors != NULL when ntensors > 0, ntensors >= 0, every n >= 0,
 * non-null pointers for n > 0, alignment as above; tensors with n == 0 are skipped.
 * No tensor may overlap another's buffers.
 */
int qopt_quantize_blockwise_multi(const qopt_codebook* cb_dev, const qopt_codec_tensor* tensors,
                                  int32_t ntensors, void* stream);
int qopt_dequantize_blockwise_multi(const qopt_codebook* cb_dev,
                                    const qopt_codec_tensor* tensors, int32_t ntensors,
                                    void* stream);

/*
 * One parameter tensor of an 8-bit Adam step.  All pointers are device memory:
 *   param    n elements of the step's param dtype, updated in place;
 *   grad     n elements of the step's grad dtype, read only;
 *   m_codes  n bytes, signed codes of the first moment, updated in place;
 *   v_codes  n bytes, unsigned codes of the second moment, updated in place;
 *   m_absmax, v_absmax  ceil(n / 2048) fp32 block maxima, updated in place.
 * Blocks restart at element 0 of every tensor.  Zero-filled state (codes and
 * absmax) is the state before the first step.  Buffers of different tensors, and
 * of one tensor, must not overlap.  Any element alignment is accepted; tensors
 * whose param / grad are 16-byte (fp32) or 8-byte (bf16) aligned and whose code
 * arrays are 4-byte aligned take the vector path.
 */
typedef struct qopt_tensor {
  void* param;
  const void* grad;
  uint8_t* m_codes;
  uint8_t* v_codes;
  float* m_absmax;
  float* v_absmax;
  int64_t n;
} qopt_tensor;

/* Adam hyper-parameters (binary32) and the 1-based step number after increment. */
typedef struct qopt_adam_hparams {
  float lr;
  float beta1;
  float beta2;
  float eps;
  int64_t step;
} qopt_adam_hparams;

/*
 * One fused 8-bit Adam step over `ntensors` tensors (host array `tensors`), all of
 * param dtype `param_dtype` and grad dtype `grad_dtype` (qopt_dtype), sharing `hp`.
 * Per element, binary32, one rounding per operation (the state is dequantized for the
 * update and stored back in 8 bits, §2):
 *   m_prev = decode_m[cm] * Am            v_prev = decode_v[cv] * Av
 *   m = b1 * m_prev + (1 - b1) * g        v = b2 * v_prev + (1 - b2) * (g * g)
 *   p = p - step_size * m / (sqrt(v) * inv_sqrt_bc2 + eps)
 * with step_size = fl32(lr / (1 - b1^t)) and inv_sqrt_bc2 = fl32(1 / sqrt(1 - b2^t))
 * evaluated in binary64 (b^t by square-and-multiply), 1 - b in binary32, correctly
 * rounded sqrt and divide; bf16 parameters are widened and the result rounded to
 * nearest-even.  Then each block of m and v is requantized exactly as
 * qopt_quantize_blockwise does (signed for m, unsigned for v).
 * Checks: tensors != NULL when ntensors > 0, ntensors >= 0, every n >= 0, non-null
 * pointers for n > 0, lr and eps finite, eps >= 0, 0 <= beta < 1, step >= 1.
 * Tensors with n == 0 are skipped.  Large tensor lists are split into several
 * launches of equal block counts (qopt_adam8bit_launch_count), on `stream`; with bf16
 * parameters and more than one launch, every other launch goes on a second stream
 * that the library creates once per device (non-blocking, default priority, kept
 * until the process ends).  That stream first waits for the work enqueued on `stream`
 * before the call, and `stream` waits for its launches before any work enqueued after
 * the call, so the call orders on `stream` as one unit.
 */
int qopt_adam8bit_step(const qopt_tensor* tensors, int32_t ntensors, int param_dtype,
                       int grad_dtype, const qopt_codebook* cb_m_dev,
                       const qopt_codebook* cb_v_dev, const qopt_adam_hparams* hp,
                       void* stream);

/*
 * Number of kernel launches qopt_adam8bit_step enqueues for this tensor list and
 * these dtypes (host only, nothing is launched): the step is split into launches of
 * equal block counts holding at most 48 tensor pieces and 2^18 blocks each.  Same
 * argument checks as qopt_adam8bit_step for the tensors and dtypes; *launches is host
 * memory.
 */
int qopt_adam8bit_launch_count(const qopt_tensor* tensors, int32_t ntensors, int param_dtype,
                               int grad_dtype, int64_t* launches);

/*
 * Measurement aid, not part of the method: moves exactly the bytes one
 * qopt_adam8bit_step moves over these tensors, with the step's launch plan, grid
 * (the step's own workgroups per CU), block order and prefetch, but no arithmetic:
 * parameters, codes and block maxima are written back as read and gradients are read
 * and dropped, so every buffer keeps its contents.  Timing it against the step on the
 * same buffers gives the ceiling of the step's access pattern.  Only blocks on the
 * step's vector path (full blocks of tensors whose pointers allow vector accesses)
 * are moved.  Same argument checks as qopt_adam8bit_step (no codebooks or
 * hyper-parameters); enqueued on `stream` (and, with bf16 parameters, over the second
 * stream as the step's launches are).
 */
int qopt_adam8bit_traffic_probe(const qopt_tensor* tensors, int32_t ntensors, int param_dtype,
                                int grad_dtype, void* stream);

/* Static description of a status code; never NULL. */
const char* qopt_status_string(int status);

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int qopt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QOPT_H */
