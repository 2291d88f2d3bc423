/*
 * qopt_embedding.h -- C ABI of the Stable Embedding layer in libqopt.so, for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer: the 8-bit optimizers summary page (wiki.neutronadmin.com/news/16836),
 * §2 "Stable Embedding Layer": the embedding table is initialised with Xavier
 * uniform, and a layer normalisation follows the lookup so that the output has a
 * variance of about 1.  The YaLM-100B training page (golden-irbis.ru) puts a
 * LayerNorm right after the embedding ("Stabilizations. LayerNorm") and computes
 * every LayerNorm in fp32 ("Stabilizations. BFloat 16"); the kernels here compute
 * in binary32 whatever the storage type.
 *
 * Conventions are those of qopt.h (status codes, dtypes, *_dev pointers in device
 * memory of the current HIP device, caller-owned buffers, host-side argument checks
 * before anything is enqueued, asynchronous work on `stream`).  Tables are row-major
 * [rows, dim]; token indices are int64.
 */
#ifndef QOPT_EMBEDDING_H
#define QOPT_EMBEDDING_H

#include <stddef.h>
#include <stdint.h>

#include "qopt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Rows up to this width (elements) whose width is a multiple of 4 and whose rows are
 * vector-aligned take the register-resident kernels; every other shape takes
 * element-wise kernels with the same arithmetic. */
#define QOPT_EMB_VEC_MAX_DIM 4096

/*
 * Xavier-uniform initialisation (§2 "Stable Embedding Layer").
 *   weight_dev[e] = fl32(a * (2u - 1)), a = fl32(sqrt(6 / (rows + dim))), for every
 *   element e of the row-major [rows, dim] table, where u = (w >> 8) * 2^-24 and w is
 *   word e % 4 of Philox4x32-10 (Salmon et al., SC 2011) applied to the counter
 *   (e / 4 low word, e / 4 high word, 0, 0) with key (seed low word, seed high word).
 *   A bf16 table stores each value rounded to nearest even.
 * weight_dtype: QOPT_F32 or QOPT_BF16.  rows, dim >= 0 (rows * dim == 0 is a no-op).
 * Errors: QOPT_EINVAL (null table with elements, negative sizes), QOPT_EUNSUPPORTED
 * (dtype), QOPT_EALIGN (table not aligned to its element size), QOPT_ELAUNCH.
 */
int qopt_embedding_xavier_init(void* weight_dev, int weight_dtype, int64_t rows, int64_t dim,
                               uint64_t seed, void* stream);

/*
 * Forward: out[t, :] = LayerNorm(weight[idx[t], :]) for t < ntokens, with
 *   mean = sum(x) / dim, var = sum((x - mean)^2) / dim, rstd = 1 / sqrt(var + eps),
 *   out = ((x - mean) * rstd) * gamma + beta, all in binary32 (one rounding per
 *   operation; sums in a fixed order per kernel shape).
 * weight_dev: [rows, dim] of weight_dtype.  idx_dev: [ntokens] int64.
 * gamma_dev, beta_dev: [dim] float.  eps: finite, >= 0.
 * out_dev: [ntokens, dim] of out_dtype (bf16 output is rounded to nearest even).
 * mean_dev, rstd_dev: [ntokens] float, or both NULL; the backward pass needs them.
 * bad_count_dev: int32 device counter or NULL.  An index outside [0, rows) is never
 *   dereferenced: its output row is NaN, its mean and rstd are NaN, and the counter
 *   (if given) is incremented once per such token; the caller zeroes it beforehand.
 * Errors: QOPT_EINVAL (null pointers where data is needed, rows < 1 or dim < 1 with
 * tokens, negative sizes, eps not finite or negative, exactly one of mean/rstd
 * NULL), QOPT_EUNSUPPORTED (dtypes), QOPT_EALIGN (pointers not aligned to their
 * element size), QOPT_ELAUNCH.  ntokens == 0 is a no-op.
 */
int qopt_stable_embedding_forward(const void* weight_dev, int weight_dtype, int64_t rows,
                                  int64_t dim, const int64_t* idx_dev, int64_t ntokens,
                                  const float* gamma_dev, const float* beta_dev, float eps,
                                  void* out_dev, int out_dtype, float* mean_dev,
                                  float* rstd_dev, int32_t* bad_count_dev, void* stream);

/*
 * Workspace the backward pass needs for ntokens tokens of width dim on the current
 * device, in bytes (*bytes; 0 when ntokens == 0).  Errors: QOPT_EINVAL (bytes NULL,
 * negative sizes), QOPT_ELAUNCH (device query).
 */
int qopt_stable_embedding_backward_workspace(int64_t ntokens, int64_t dim, size_t* bytes);

/*
 * Backward of the forward above, for upstream gradient dout:
 *   xhat = (x - mean) * rstd, g = dout * gamma (x = weight[idx[t]], mean and rstd as
 *   saved by the forward), dx = rstd * ((g - sum(g) / dim) - xhat * (sum(g * xhat) / dim)),
 *   dweight[idx[t], :] += dx, dgamma = sum over tokens of dout * xhat,
 *   dbeta = sum over tokens of dout.
 * Vector-path shapes (dim a multiple of 4 up to QOPT_EMB_VEC_MAX_DIM, aligned rows,
 * dweight 16-byte aligned, rows < 2^32 - 1, ntokens < 2^31) group the tokens by row
 * first (a stable radix sort in the workspace): the tokens of a row share x, mean and
 * rstd, so their summed dx is the same map applied to the sum of their dout rows, and
 * each row's gradient is formed once and added to dweight without atomics.  All
 * three results are then reproducible run to run.  Other shapes scatter dx with
 * float atomics (rows shared by several tokens add up in arrival order); dgamma and
 * dbeta are still summed in a fixed order there.
 * dout_dev: [ntokens, dim] of dout_dtype.  dweight_dev: [rows, dim] float, whose
 * existing contents are added to.  dgamma_dev, dbeta_dev: [dim] float (written).
 * workspace_dev: at least qopt_stable_embedding_backward_workspace(ntokens, dim)
 * bytes of device memory, 16-byte aligned; its contents are scratch.
 * Tokens whose index is outside [0, rows) contribute nothing.
 * Errors: as for the forward, plus QOPT_EINVAL for a workspace that is NULL or too
 * small, and QOPT_ELAUNCH if the sort cannot be enqueued.  ntokens == 0 writes zeros
 * to dgamma and dbeta and leaves dweight as it is.
 */
int qopt_stable_embedding_backward(const void* weight_dev, int weight_dtype, int64_t rows,
                                   int64_t dim, const int64_t* idx_dev, int64_t ntokens,
                                   const float* gamma_dev, const float* mean_dev,
                                   const float* rstd_dev, const void* dout_dev, int dout_dtype,
                                   float* dweight_dev, float* dgamma_dev, float* dbeta_dev,
                                   void* workspace_dev, size_t workspace_bytes, void* stream);

/* Bytes of device scratch the allocation-free backward holds per device (64 MiB). */
#define QOPT_EMB_STATIC_SCRATCH_BYTES 67108864

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): qopt_stable_embedding_backward
 * with its workspace in a fixed array of QOPT_EMB_STATIC_SCRATCH_BYTES bytes of device
 * memory that the library holds on each device it runs on until the process ends.
 * Same arguments, checks and results as qopt_stable_embedding_backward without the
 * workspace; the caller still passes every input and output.  The shape's workspace
 * need (qopt_stable_embedding_backward_workspace) must fit the array, or the call
 * returns QOPT_ENOSPACE before enqueueing anything: at width 4096 that allows about
 * 29,000 tokens, at width 1024 about 116,000.  The array's contents are scratch: the
 * kernels write every part they read, so nothing needs clearing between calls.  All
 * calls on one device share that device's array, so calls that overlap in time on
 * one device (on different streams, or from different host threads) race; the caller
 * orders them.  Allocates nothing: no hipMalloc, no library routine that allocates.
 */
int qopt_stable_embedding_backward_noalloc(const void* weight_dev, int weight_dtype,
                                           int64_t rows, int64_t dim, const int64_t* idx_dev,
                                           int64_t ntokens, const float* gamma_dev,
                                           const float* mean_dev, const float* rstd_dev,
                                           const void* dout_dev, int dout_dtype,
                                           float* dweight_dev, float* dgamma_dev,
                                           float* dbeta_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QOPT_EMBEDDING_H */
