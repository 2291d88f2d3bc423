// Stable Embedding layer kernels for gfx950 (include/qopt_embedding.h).
//
// 8-bit optimizers summary page (wiki.neutronadmin.com/news/16836), §2 "Stable
// Embedding Layer": Xavier-uniform initialisation of the table and a layer
// normalisation after the lookup.  YaLM-100B training page (golden-irbis.ru),
// "Stabilizations. LayerNorm" / "Stabilizations. BFloat 16": LayerNorm right after
// the embedding, computed in fp32.
//
// Execution model:
//   - One wavefront per token row.  For rows of up to 4096 elements whose width is
//     a multiple of 4 (the vector path), lane l holds columns s*256 + 4l .. +3 for
//     slices s < S, in registers; row sums are a per-lane sum in slice order followed
//     by a DPP reduction over the 64 lanes (every lane ends with the same bits).
//   - Persistent workgroups walk tokens with a grid stride; gamma and beta are
//     staged in LDS once per workgroup.
//   - Backward (vector path): tokens are sorted by table row and each row's summed
//     upstream gradient gets one LayerNorm backward, written by one wave without
//     atomics (see the grouped backward below); gamma and beta gradients are kept
//     per lane in registers over a wave's rows, written to a workspace slot per
//     workgroup and summed over slots in slot order, so all three gradients are
//     reproducible bit for bit.
//   - Every other shape runs element-wise kernels (one wave per workgroup, columns
//     lane, lane + 64, ...) with the same operations; their table gradient is
//     scattered with float atomics.

#include <hip/hip_runtime.h>
#include <rocprim/device/device_radix_sort.hpp>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "qopt_embedding.h"

namespace {

constexpr int kWave = 64;
constexpr int kVecWaves = 4;  // waves per workgroup in the vector kernels
constexpr int kVecThreads = kWave * kVecWaves;
constexpr int kMaxSlices = QOPT_EMB_VEC_MAX_DIM / 256;
constexpr int kBwdSlotsPerCu = 2;  // backward workgroups (gradient slots) per CU

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// --------------------------------------------------------------- element access

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 pair -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Cache policy, measured on the embed7b shape (each choice timed against the others in
// one process, on the same buffers): table rows read by the forward stay cached, since
// frequent ids reuse them; everything read or written once goes non-temporal, so that
// it does not push those rows out of the caches.  That is the forward's output rows
// (0.192 -> 0.180 ms) and, in the backward, the upstream rows, the table rows and the
// table-gradient rows of each finished run (0.408 -> 0.367 ms).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
  static __device__ __forceinline__ f32x4 load4(const float* p, int64_t i) {
    return *reinterpret_cast<const f32x4*>(p + i);
  }
  static __device__ __forceinline__ f32x4 load4nt(const float* p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i));
  }
  static __device__ __forceinline__ void store4(float* p, int64_t i, f32x4 v) {
    *reinterpret_cast<f32x4*>(p + i) = v;
  }
  static __device__ __forceinline__ void store4nt(float* p, int64_t i, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p + i));
  }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float x) {
    p[i] = static_cast<uint16_t>(f32x2_to_bf16x2(x, 0.0f) & 0xFFFFu);
  }
  static __device__ __forceinline__ f32x4 widen(u32x2 w) {
    return f32x4{bf16_bits_to_f32(w.x & 0xFFFFu), bf16_bits_to_f32(w.x >> 16),
                 bf16_bits_to_f32(w.y & 0xFFFFu), bf16_bits_to_f32(w.y >> 16)};
  }
  static __device__ __forceinline__ f32x4 load4(const uint16_t* p, int64_t i) {
    return widen(*reinterpret_cast<const u32x2*>(p + i));
  }
  static __device__ __forceinline__ f32x4 load4nt(const uint16_t* p, int64_t i) {
    return widen(__builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + i)));
  }
  static __device__ __forceinline__ u32x2 narrow(f32x4 v) {
    u32x2 w;
    w.x = f32x2_to_bf16x2(v.x, v.y);
    w.y = f32x2_to_bf16x2(v.z, v.w);
    return w;
  }
  static __device__ __forceinline__ void store4(uint16_t* p, int64_t i, f32x4 v) {
    *reinterpret_cast<u32x2*>(p + i) = narrow(v);
  }
  static __device__ __forceinline__ void store4nt(uint16_t* p, int64_t i, f32x4 v) {
    __builtin_nontemporal_store(narrow(v), reinterpret_cast<u32x2*>(p + i));
  }
};

// Sum over the 64 lanes, returned to every lane as the same bits.  Four DPP steps
// inside each row of 16 lanes (swap neighbours, swap pairs, mirror the half rows,
// mirror the rows) pair lanes symmetrically, so after them every lane of a row holds
// that row's sum; two row broadcasts then add the rows up into lane 63 as
// (r3 + r2) + (r1 + r0), and lane 63 is read into a scalar register.  Six levels of
// additions, as in a butterfly, with no LDS traffic (a __shfl_xor butterfly compiles
// to six dependent ds_bpermute round trips).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float x) {
  // lanes of rows outside kRowMask read -0.0 (the `old` value), which adds nothing
  return x + __int_as_float(__builtin_amdgcn_update_dpp(static_cast<int>(0x80000000u),
                                                        __float_as_int(x), kCtrl, kRowMask,
                                                        0xF, false));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = dpp_add<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x141, 0xF>(x);  // row_half_mirror
  x = dpp_add<0x140, 0xF>(x);  // row_mirror
  x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ float quiet_nan() { return __uint_as_float(0x7FC00000u); }

// ------------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC 2011): ten rounds; each multiplies words 0 and 2 by two constants, mixes the
// high halves with the other words and the key, and the key advances by two Weyl
// constants between rounds.

struct Words4 {
  uint32_t w[4];
};

__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
    const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return Words4{{c0, c1, c2, c3}};
}

// -------------------------------------------------------------------- kernels

// Xavier uniform: thread i fills elements 4i .. 4i+3 from counter block i.
template <typename WT>
__global__ void __launch_bounds__(256) xavier_kernel(WT* w, uint64_t n, uint64_t nblocks,
                                                     uint32_t k0, uint32_t k1, float a) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t b = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; b < nblocks;
       b += stride) {
    const Words4 r = philox4x32_10(static_cast<uint32_t>(b), static_cast<uint32_t>(b >> 32), 0u,
                                   0u, k0, k1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t e = 4 * b + j;
      if (e < n) {
        const float u = static_cast<float>(r.w[j] >> 8) * 0x1p-24f;  // exact
        const float two_u_minus_1 = (2.0f * u) - 1.0f;                 // exact
        Elem<WT>::store(w, static_cast<int64_t>(e), a * two_u_minus_1);
      }
    }
  }
}

// Stage `dim` floats of src into LDS as S*64 float4 (zeros past dim).
template <int S>
__device__ __forceinline__ void stage4(f32x4* dst, const float* src, int32_t dim) {
  for (int i = threadIdx.x; i < S * kWave; i += blockDim.x) {
    f32x4 v;
    const int c = 4 * i;
    v.x = c + 0 < dim ? src[c + 0] : 0.0f;
    v.y = c + 1 < dim ? src[c + 1] : 0.0f;
    v.z = c + 2 < dim ? src[c + 2] : 0.0f;
    v.w = c + 3 < dim ? src[c + 3] : 0.0f;
    dst[i] = v;
  }
}

template <int S, typename WT, typename OT>
__global__ void __launch_bounds__(kVecThreads)
fwd_vec_kernel(const WT* __restrict__ w, int64_t rows, int32_t dim, const int64_t* __restrict__ idx,
               int64_t ntok, const float* __restrict__ gamma, const float* __restrict__ beta,
               float eps, OT* __restrict__ out, float* __restrict__ mean_out,
               float* __restrict__ rstd_out, int32_t* __restrict__ bad) {
  extern __shared__ f32x4 lds4[];
  f32x4* gam = lds4;
  f32x4* bet = lds4 + S * kWave;
  stage4<S>(gam, gamma, dim);
  stage4<S>(bet, beta, dim);
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kVecWaves;
  const float n_dim = static_cast<float>(dim);
  const int64_t t0 = blockIdx.x * static_cast<int64_t>(kVecWaves) + wave;
  if (t0 >= ntok) return;
  auto row_of = [&](int64_t t) { return t < ntok ? idx[t] : int64_t{0}; };
  auto valid = [&](int64_t r) { return r >= 0 && r < rows; };
  // loads of a token's row, branch-free (an invalid or absent token loads row 0)
  auto load_row = [&](f32x4 (&x)[S], int64_t r) {
    const WT* row = w + (valid(r) ? r : int64_t{0}) * dim;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = s * 256 + 4 * lane;
      x[s] = Elem<WT>::load4(row, c < dim ? c : 0);
    }
  };
  auto process = [&](int64_t t, int64_t r, const f32x4 (&xin)[S]) {
    OT* orow = out + t * dim;
    if (!valid(r)) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int c = s * 256 + 4 * lane;
        if (c < dim) Elem<OT>::store4(orow, c, f32x4{quiet_nan(), quiet_nan(), quiet_nan(), quiet_nan()});
      }
      if (lane == 0) {
        if (mean_out) {
          mean_out[t] = quiet_nan();
          rstd_out[t] = quiet_nan();
        }
        if (bad) atomicAdd(bad, 1);
      }
      return;
    }
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = s * 256 + 4 * lane;
      const f32x4 x = c < dim ? xin[s] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      sum = sum + x.x;
      sum = sum + x.y;
      sum = sum + x.z;
      sum = sum + x.w;
    }
    const float mean = wave_sum(sum) / n_dim;
    float sq = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = s * 256 + 4 * lane;
      if (c < dim) {
        const f32x4 x = xin[s];
        const float d0 = x.x - mean, d1 = x.y - mean, d2 = x.z - mean, d3 = x.w - mean;
        sq = sq + (d0 * d0);
        sq = sq + (d1 * d1);
        sq = sq + (d2 * d2);
        sq = sq + (d3 * d3);
      }
    }
    const float var = wave_sum(sq) / n_dim;
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = s * 256 + 4 * lane;
      if (c < dim) {
        const f32x4 x = xin[s];
        const f32x4 g = gam[s * kWave + lane], b = bet[s * kWave + lane];
        f32x4 y;
        y.x = (((x.x - mean) * rstd) * g.x) + b.x;
        y.y = (((x.y - mean) * rstd) * g.y) + b.y;
        y.z = (((x.z - mean) * rstd) * g.z) + b.z;
        y.w = (((x.w - mean) * rstd) * g.w) + b.w;
        Elem<OT>::store4nt(orow, c, y);
      }
    }
    if (lane == 0 && mean_out) {
      mean_out[t] = mean;
      rstd_out[t] = rstd;
    }
  };
  // two row buffers in turn: the next token's row is in flight while this one is
  // normalised and written (2.5 % faster on the embed7b shape than loading each row
  // when its token comes up)
  f32x4 xa[S], xb[S];
  int64_t ra = row_of(t0);
  int64_t rb = row_of(t0 + stride);
  load_row(xa, ra);
  for (int64_t t = t0; t < ntok; t += 2 * stride) {
    load_row(xb, rb);
    const int64_t rn = row_of(t + 2 * stride);
    process(t, ra, xa);
    if (t + stride >= ntok) break;
    load_row(xa, rn);
    const int64_t rnn = row_of(t + 3 * stride);
    process(t + stride, rb, xb);
    ra = rn;
    rb = rnn;
  }
}

// Element-wise forward: one wave per workgroup, any width and alignment.
template <typename WT, typename OT>
__global__ void __launch_bounds__(kWave)
fwd_elem_kernel(const WT* __restrict__ w, int64_t rows, int64_t dim, const int64_t* __restrict__ idx,
                int64_t ntok, const float* __restrict__ gamma, const float* __restrict__ beta,
                float eps, OT* __restrict__ out, float* __restrict__ mean_out,
                float* __restrict__ rstd_out, int32_t* __restrict__ bad) {
  const int lane = threadIdx.x;
  const float n_dim = static_cast<float>(dim);
  for (int64_t t = blockIdx.x; t < ntok; t += gridDim.x) {
    const int64_t r = idx[t];
    OT* orow = out + t * dim;
    if (r < 0 || r >= rows) {
      for (int64_t c = lane; c < dim; c += kWave) Elem<OT>::store(orow, c, quiet_nan());
      if (lane == 0) {
        if (mean_out) {
          mean_out[t] = quiet_nan();
          rstd_out[t] = quiet_nan();
        }
        if (bad) atomicAdd(bad, 1);
      }
      continue;
    }
    const WT* row = w + r * dim;
    float sum = 0.0f;
    for (int64_t c = lane; c < dim; c += kWave) sum = sum + Elem<WT>::load(row, c);
    const float mean = wave_sum(sum) / n_dim;
    float sq = 0.0f;
    for (int64_t c = lane; c < dim; c += kWave) {
      const float d = Elem<WT>::load(row, c) - mean;
      sq = sq + (d * d);
    }
    const float var = wave_sum(sq) / n_dim;
    const float rstd = 1.0f / sqrtf(var + eps);
    for (int64_t c = lane; c < dim; c += kWave)
      Elem<OT>::store(orow, c, (((Elem<WT>::load(row, c) - mean) * rstd) * gamma[c]) + beta[c]);
    if (lane == 0 && mean_out) {
      mean_out[t] = mean;
      rstd_out[t] = rstd;
    }
  }
}

// ---- grouped backward (vector path)
//
// The tokens that share a row r have the same x, mean and rstd, so their summed
// table gradient is the LayerNorm backward of S_r = sum of their upstream rows:
//   dweight[r] += rstd * ((g - sum(g) / dim) - xhat * (sum(g * xhat) / dim)), g = S_r * gamma,
// and dgamma = sum_r xhat_r * S_r, dbeta = sum_r S_r.  Tokens are sorted by row
// (stable radix sort of (row, token) pairs), the sorted list is cut into chunks of
// kSegChunk tokens, and one wave sums each chunk's runs of equal rows in registers.
// A run that lies inside one chunk is finished by that wave; a run that crosses
// chunk boundaries leaves per-chunk partial sums that a second kernel adds in chunk
// order.  Every row is finished exactly once, by one wave, so dweight is updated
// without atomics and every result is reproducible.

constexpr int kSegChunk = 32;      // sorted tokens per chunk
// chunk workgroups (two waves each) per CU: twice what fits at once, so that workgroups
// whose chunks finish many runs do not hold up the rest
constexpr int kChunkWgPerCu = 8;

// keys[t] = idx[t] for an index in [0, rows), else rows (sorts after every valid row).
__global__ void __launch_bounds__(256) sort_keys_kernel(const int64_t* __restrict__ idx,
                                                        int64_t ntok, uint32_t rows,
                                                        uint32_t* __restrict__ keys,
                                                        int32_t* __restrict__ vals) {
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < ntok;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = idx[t];
    keys[t] = (r >= 0 && r < static_cast<int64_t>(rows)) ? static_cast<uint32_t>(r) : rows;
    vals[t] = static_cast<int32_t>(t);
  }
}

// Per-wave state of the grouped kernels: gamma in LDS, the wave's dgamma / dbeta sums.
template <int S>
struct GroupAcc {
  f32x4 dg[S], db[S];
};

// Finish row k from its summed upstream rows acc (mean / rstd of token t, one of the
// row's tokens): dweight row += the LayerNorm backward of acc; add its dgamma / dbeta
// terms to the wave's sums.  The weight and gradient rows are loaded together.
template <int S, typename WT>
__device__ __forceinline__ void finish_row(const WT* __restrict__ w, int32_t dim, uint32_t k,
                                           int64_t t, const f32x4 (&acc)[S], const f32x4* gam,
                                           const float* __restrict__ mean,
                                           const float* __restrict__ rstd,
                                           float* __restrict__ dweight, int lane,
                                           GroupAcc<S>& ga) {
  const WT* row = w + static_cast<int64_t>(k) * dim;
  const float mu = mean[t], rs = rstd[t];
  const float n_dim = static_cast<float>(dim);
  float* drow = dweight + static_cast<int64_t>(k) * dim;
  f32x4 xs[S], ds[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = s * 256 + 4 * lane < dim ? s * 256 + 4 * lane : 0;
    xs[s] = Elem<WT>::load4nt(row, c);
    ds[s] = Elem<float>::load4nt(drow, c);
  }
  float c1 = 0.0f, c2 = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = s * 256 + 4 * lane;
    if (c < dim) {
      const f32x4 x = xs[s];
      const f32x4 g = gam[s * kWave + lane];
      f32x4 xh, gg;
      xh.x = (x.x - mu) * rs;
      xh.y = (x.y - mu) * rs;
      xh.z = (x.z - mu) * rs;
      xh.w = (x.w - mu) * rs;
      gg.x = acc[s].x * g.x;
      gg.y = acc[s].y * g.y;
      gg.z = acc[s].z * g.z;
      gg.w = acc[s].w * g.w;
      c1 = c1 + gg.x;
      c1 = c1 + gg.y;
      c1 = c1 + gg.z;
      c1 = c1 + gg.w;
      c2 = c2 + (gg.x * xh.x);
      c2 = c2 + (gg.y * xh.y);
      c2 = c2 + (gg.z * xh.z);
      c2 = c2 + (gg.w * xh.w);
      ga.dg[s].x = ga.dg[s].x + (xh.x * acc[s].x);
      ga.dg[s].y = ga.dg[s].y + (xh.y * acc[s].y);
      ga.dg[s].z = ga.dg[s].z + (xh.z * acc[s].z);
      ga.dg[s].w = ga.dg[s].w + (xh.w * acc[s].w);
      ga.db[s] = ga.db[s] + acc[s];
    }
  }
  const float m1 = wave_sum(c1) / n_dim;
  const float m2 = wave_sum(c2) / n_dim;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = s * 256 + 4 * lane;
    if (c < dim) {
      const f32x4 x = xs[s];
      const f32x4 g = gam[s * kWave + lane];
      f32x4 d = ds[s];
      d.x = d.x + (rs * (((acc[s].x * g.x) - m1) - (((x.x - mu) * rs) * m2)));
      d.y = d.y + (rs * (((acc[s].y * g.y) - m1) - (((x.y - mu) * rs) * m2)));
      d.z = d.z + (rs * (((acc[s].z * g.z) - m1) - (((x.z - mu) * rs) * m2)));
      d.w = d.w + (rs * (((acc[s].w * g.w) - m1) - (((x.w - mu) * rs) * m2)));
      Elem<float>::store4nt(drow, c, d);
    }
  }
}

// Combine the workgroup's per-wave dgamma / dbeta sums in wave order and write them
// to workspace slot `slot` ([2][dim] floats).
template <int S>
__device__ __forceinline__ void write_slot(const GroupAcc<S>& ga, f32x4* comb_g, f32x4* comb_b,
                                           float* __restrict__ slots, int64_t slot, int32_t dim,
                                           int wave, int lane) {
  for (int k = 0; k < kVecWaves; ++k) {
    if (wave == k) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int i = s * kWave + lane;
        comb_g[i] = k == 0 ? ga.dg[s] : comb_g[i] + ga.dg[s];
        comb_b[i] = k == 0 ? ga.db[s] : comb_b[i] + ga.db[s];
      }
    }
    __syncthreads();
  }
  float* out = slots + slot * 2 * dim;
  for (int i = threadIdx.x; i < S * kWave; i += kVecThreads) {
    const int c = 4 * i;
    if (c < dim) {
      *reinterpret_cast<f32x4*>(out + c) = comb_g[i];
      *reinterpret_cast<f32x4*>(out + dim + c) = comb_b[i];
    }
  }
}

// Raw 4-element groups of an upstream-gradient row as loaded (fp32 or packed bf16).
template <typename OT> struct Raw4;
template <> struct Raw4<float> {
  typedef f32x4 type;
  static __device__ __forceinline__ type load_nt(const float* p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i));
  }
  static __device__ __forceinline__ f32x4 widen(type v) { return v; }
};
template <> struct Raw4<uint16_t> {
  typedef u32x2 type;
  static __device__ __forceinline__ type load_nt(const uint16_t* p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + i));
  }
  static __device__ __forceinline__ f32x4 widen(type w) {
    return f32x4{bf16_bits_to_f32(w.x & 0xFFFFu), bf16_bits_to_f32(w.x >> 16),
                 bf16_bits_to_f32(w.y & 0xFFFFu), bf16_bits_to_f32(w.y >> 16)};
  }
};

constexpr int kPairThreads = 2 * kWave;  // chunk kernel: two waves share a chunk's columns

// An int the compiler cannot see through.  Addresses derived from it inside a loop
// are redone per iteration (a few cheap ops) instead of being hoisted out of the
// loop as 64-bit offsets per slice, which would pin dozens of registers.
__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Chunk pass: a workgroup of two waves per chunk, walking chunks with a grid stride.
// Wave h owns the slices h, h + 2, ... of every row (SH = S / 2 slices), so a wave
// holds half a row of sums and keeps the next token's upstream row in flight while
// it adds the current one.  The loads and adds of the token loop have no branches
// (a slice past the row's end reads the row's first columns and adds zero) and the
// loads are unconditional, so the compiler waits for exactly the row it adds; with
// a branch per slice it waits for every outstanding load, the prefetched row
// included.  A run that ends in the chunk is finished at once: its weight row and its
// gradient row are loaded together, and the row-wide sums are combined across the two
// waves through LDS, in wave order.  Holding both rows takes up to 254 VGPRs, so 2
// waves per SIMD; that beats loading the gradient row only after the sums at 3.
// parts[chunk][0]: the sum over the chunk's tokens of a run that began in an earlier
// chunk; parts[chunk][1]: of a run that begins in this chunk and goes on past it.
template <int S, typename WT, typename OT>
__global__ void __launch_bounds__(kPairThreads, 2)
group_chunk_kernel(const WT* __restrict__ w, uint32_t rows, int32_t dim,
                   const uint32_t* __restrict__ keys, const int32_t* __restrict__ vals,
                   int64_t ntok, int64_t nchunks, const float* __restrict__ gamma,
                   const float* __restrict__ mean, const float* __restrict__ rstd,
                   const OT* __restrict__ dout, float* __restrict__ dweight,
                   float* __restrict__ parts, float* __restrict__ slots) {
  constexpr int SH = S / 2;
  extern __shared__ f32x4 lds4[];
  f32x4* gam = lds4;
  __shared__ float red[2][2];
  stage4<S>(gam, gamma, dim);
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const float n_dim = static_cast<float>(dim);
  f32x4 dg[SH], db[SH];
#pragma unroll
  for (int i = 0; i < SH; ++i) {
    dg[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    db[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // this lane's first column; slice i of the wave starts 512 columns further on
  const int col0 = h * 256 + 4 * lane;
  auto col = [&](int i) { return col0 + 512 * i; };
  typedef typename Raw4<OT>::type RT;
  auto load_row = [&](RT (&dst)[SH], int64_t t) {
    const int c0 = opaque_int(col0);
    const OT* row = dout + t * dim;
#pragma unroll
    for (int i = 0; i < SH; ++i)
      dst[i] = Raw4<OT>::load_nt(row, c0 + 512 * i < dim ? c0 + 512 * i : 0);
  };
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const int64_t p0 = ch * kSegChunk;
    const int64_t p1 = p0 + kSegChunk < ntok ? p0 + kSegChunk : ntok;
    // the chunk's keys (and its neighbours') and tokens, one per lane
    const int64_t kp = p0 - 1 + lane;
    const uint32_t key_l = (lane < kSegChunk + 2 && kp >= 0 && kp < ntok) ? keys[kp] : 0xFFFFFFFFu;
    const int32_t val_l = (lane < kSegChunk && p0 + lane < ntok) ? vals[p0 + lane] : 0;
    auto key_at = [&](int64_t p) {  // keys[p] for p0 - 1 <= p <= p0 + kSegChunk
      return static_cast<uint32_t>(
          __builtin_amdgcn_readlane(static_cast<int>(key_l), static_cast<int>(p - p0 + 1)));
    };
    auto tok_at = [&](int64_t p) {
      return static_cast<int64_t>(__builtin_amdgcn_readlane(val_l, static_cast<int>(p - p0)));
    };
    const bool head_open = p0 > 0 && key_at(p0 - 1) == key_at(p0);
    f32x4 acc[SH];
#pragma unroll
    for (int i = 0; i < SH; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // two row buffers: token p's row is added from one while token p + 1's is in
    // flight in the other; the loop is unrolled by two so that the buffers swap
    // roles without copies (copying a register whose load is still pending would
    // wait for it)
    RT b0[SH], b1[SH];
#pragma unroll
    for (int i = 0; i < SH; ++i) {
      b0[i] = RT{};
      b1[i] = RT{};
    }
    // The loads are unconditional, so that the compiler can count them and wait for
    // exactly the row it adds: past the chunk's end a step reloads the row it has
    // just used (a cache hit).  Every token position is a valid upstream row.
    load_row(b0, tok_at(p0));
    bool first = true;
    // token p: start loading token p + 1's row into `fill`, add token p's row (in
    // `use`), finish or hand on the run if it ends here; false at the first invalid
    // index (they sort last)
    auto step = [&](int64_t p, const RT (&use)[SH], RT (&fill)[SH]) -> bool {
      const uint32_t k = key_at(p);
      if (k >= rows) return false;
      const int64_t t = tok_at(p);
      load_row(fill, p + 1 < p1 ? tok_at(p + 1) : t);
#pragma unroll
      for (int i = 0; i < SH; ++i) {
        const f32x4 r = Raw4<OT>::widen(use[i]);
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        acc[i] = acc[i] + (col(i) < dim ? r : zero);
      }
      const bool run_ends = p + 1 == ntok || key_at(p + 1) != k;
      if (run_ends || p + 1 == p1) {
        const bool began_here = !(first && head_open);
        if (began_here && run_ends) {
          // finish row k: dweight[k] += LayerNorm backward of acc; gamma / beta terms
          const int c0 = opaque_int(col0);
          const WT* xrow = w + static_cast<int64_t>(k) * dim + c0;
          float* drow = dweight + static_cast<int64_t>(k) * dim + c0;
          const float mu = mean[t], rs = rstd[t];
          f32x4 xs[SH], ds[SH];
#pragma unroll
          for (int i = 0; i < SH; ++i) {
            const int ci = c0 + 512 * i < dim ? 512 * i : 0;
            xs[i] = Elem<WT>::load4nt(xrow, ci);
            ds[i] = Elem<float>::load4nt(drow, ci);
          }
          float c1 = 0.0f, c2 = 0.0f;
#pragma unroll
          for (int i = 0; i < SH; ++i) {
            if (c0 + 512 * i < dim) {
              const f32x4 x = xs[i];
              const f32x4 g = gam[(h + 2 * i) * kWave + lane];
              f32x4 xh, gg;
              xh.x = (x.x - mu) * rs;
              xh.y = (x.y - mu) * rs;
              xh.z = (x.z - mu) * rs;
              xh.w = (x.w - mu) * rs;
              gg.x = acc[i].x * g.x;
              gg.y = acc[i].y * g.y;
              gg.z = acc[i].z * g.z;
              gg.w = acc[i].w * g.w;
              c1 = c1 + gg.x;
              c1 = c1 + gg.y;
              c1 = c1 + gg.z;
              c1 = c1 + gg.w;
              c2 = c2 + (gg.x * xh.x);
              c2 = c2 + (gg.y * xh.y);
              c2 = c2 + (gg.z * xh.z);
              c2 = c2 + (gg.w * xh.w);
              dg[i].x = dg[i].x + (xh.x * acc[i].x);
              dg[i].y = dg[i].y + (xh.y * acc[i].y);
              dg[i].z = dg[i].z + (xh.z * acc[i].z);
              dg[i].w = dg[i].w + (xh.w * acc[i].w);
              db[i] = db[i] + acc[i];
            }
          }
          c1 = wave_sum(c1);
          c2 = wave_sum(c2);
          if (lane == 0) {
            red[h][0] = c1;
            red[h][1] = c2;
          }
          __syncthreads();
          const float m1 = (red[0][0] + red[1][0]) / n_dim;
          const float m2 = (red[0][1] + red[1][1]) / n_dim;
          __syncthreads();
#pragma unroll
          for (int i = 0; i < SH; ++i) {
            if (c0 + 512 * i < dim) {
              const f32x4 x = xs[i];
              const f32x4 g = gam[(h + 2 * i) * kWave + lane];
              f32x4 d = ds[i];
              d.x = d.x + (rs * (((acc[i].x * g.x) - m1) - (((x.x - mu) * rs) * m2)));
              d.y = d.y + (rs * (((acc[i].y * g.y) - m1) - (((x.y - mu) * rs) * m2)));
              d.z = d.z + (rs * (((acc[i].z * g.z) - m1) - (((x.z - mu) * rs) * m2)));
              d.w = d.w + (rs * (((acc[i].w * g.w) - m1) - (((x.w - mu) * rs) * m2)));
              Elem<float>::store4nt(drow, 512 * i, d);
            }
          }
        } else {
          const int c0 = opaque_int(col0);
          float* dst = parts + (ch * 2 + (began_here ? 1 : 0)) * dim + c0;
#pragma unroll
          for (int i = 0; i < SH; ++i)
            if (c0 + 512 * i < dim) *reinterpret_cast<f32x4*>(dst + 512 * i) = acc[i];
        }
#pragma unroll
        for (int i = 0; i < SH; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        first = false;
      }
      return true;
    };
    for (int64_t p = p0; p < p1; p += 2) {
      if (!step(p, b0, b1)) break;
      if (p + 1 >= p1 || !step(p + 1, b1, b0)) break;
    }
  }
  // each wave writes its own columns of the workgroup's slot
  float* out = slots + static_cast<int64_t>(blockIdx.x) * 2 * dim;
#pragma unroll
  for (int i = 0; i < SH; ++i) {
    const int c = col(i);
    if (c < dim) {
      *reinterpret_cast<f32x4*>(out + c) = dg[i];
      *reinterpret_cast<f32x4*>(out + dim + c) = db[i];
    }
  }
}

// Is chunk ch the first chunk of a run that continues past it?  (key of that run in *k)
__device__ __forceinline__ bool span_starts(const uint32_t* __restrict__ keys, uint32_t rows,
                                            int64_t ntok, int64_t ch, uint32_t* k) {
  const int64_t p0 = ch * kSegChunk;
  const int64_t p1 = p0 + kSegChunk;
  if (p1 >= ntok) return false;  // the last chunk has no successor
  *k = keys[p1 - 1];
  if (*k >= rows || keys[p1] != *k) return false;
  return !(keys[p0] == *k && p0 > 0 && keys[p0 - 1] == *k);
}

// Runs that cross chunk boundaries, step 1: one wave per (chunk, 256-column slice)
// adds the following chunks' head partials to the first chunk's tail partial, in
// chunk order, and leaves the run's total in that tail slot.
template <int S>
__global__ void __launch_bounds__(kVecThreads)
group_span_sum_kernel(const uint32_t* __restrict__ keys, uint32_t rows, int32_t dim,
                      int64_t ntok, int64_t nchunks, float* __restrict__ parts) {
  const int lane = threadIdx.x % kWave;
  const int64_t task = blockIdx.x * static_cast<int64_t>(kVecWaves) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t ch = task / S;
  const int s = static_cast<int>(task % S);
  uint32_t k = 0;
  if (ch >= nchunks || !span_starts(keys, rows, ntok, ch, &k)) return;
  // the run ends at the first position past p1 whose key exceeds k (keys are sorted).
  // It lies in [lo, hi], hi being the first position known to be past it; each round
  // the 64 lanes probe 64 evenly spaced keys in [lo, hi) and keep the stretch where
  // the keys pass k, so 2^16 tokens take three rounds of loads.
  int64_t lo = (ch + 1) * kSegChunk, hi = ntok;
  while (lo < hi) {
    const int64_t n = hi - lo;
    const int64_t step = n <= kWave ? 1 : (n + kWave - 1) / kWave;
    int64_t q = lo + (lane + 1) * step - 1;
    q = q < hi - 1 ? q : hi - 1;
    const uint64_t past = __ballot(keys[q] > k);
    const int j = past ? __builtin_ctzll(past) : kWave;
    if (n <= kWave) {
      lo = hi = lo + (j < n ? j : n);
    } else {
      // probe j is the first past k, so the end is in (probe j - 1, probe j]
      const int64_t qlo = lo + static_cast<int64_t>(j) * step;
      const int64_t qj = lo + static_cast<int64_t>(j + 1) * step - 1;
      const int64_t nhi = j == kWave ? hi : (qj < hi - 1 ? qj : hi - 1);
      lo = qlo < hi ? qlo : hi;
      hi = nhi;
    }
  }
  const int64_t last = (lo - 1) / kSegChunk;  // the run's last chunk
  const int c = s * 256 + 4 * lane;
  if (c >= dim) return;
  float* tail = parts + (ch * 2 + 1) * dim + c;
  f32x4 acc = *reinterpret_cast<const f32x4*>(tail);
#pragma unroll 32
  for (int64_t c2 = ch + 1; c2 <= last; ++c2)
    acc = acc + *reinterpret_cast<const f32x4*>(parts + (c2 * 2) * dim + c);
  *reinterpret_cast<f32x4*>(tail) = acc;
}

// Step 2: finish every run that crosses chunk boundaries from its total, one wave per
// run, in a persistent grid whose workgroups keep one gradient slot each.
template <int S, typename WT>
__global__ void __launch_bounds__(kVecThreads)
group_span_finish_kernel(const WT* __restrict__ w, uint32_t rows, int32_t dim,
                         const uint32_t* __restrict__ keys, const int32_t* __restrict__ vals,
                         int64_t ntok, int64_t nchunks, const float* __restrict__ gamma,
                         const float* __restrict__ mean, const float* __restrict__ rstd,
                         float* __restrict__ dweight, const float* __restrict__ parts,
                         float* __restrict__ slots, int64_t slot0) {
  extern __shared__ f32x4 lds4[];
  f32x4* gam = lds4;
  stage4<S>(gam, gamma, dim);
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  GroupAcc<S> ga;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    ga.dg[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    ga.db[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  for (int64_t ch = blockIdx.x * static_cast<int64_t>(kVecWaves) + wave; ch < nchunks;
       ch += static_cast<int64_t>(gridDim.x) * kVecWaves) {
    uint32_t k = 0;
    if (!span_starts(keys, rows, ntok, ch, &k)) continue;
    const float* total = parts + (ch * 2 + 1) * dim;
    f32x4 acc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = s * 256 + 4 * lane;
      acc[s] = c < dim ? *reinterpret_cast<const f32x4*>(total + c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    finish_row<S, WT>(w, dim, k, vals[(ch + 1) * kSegChunk - 1], acc, gam, mean, rstd, dweight,
                      lane, ga);
  }
  f32x4* comb_g = lds4 + S * kWave;
  f32x4* comb_b = lds4 + 2 * S * kWave;
  write_slot<S>(ga, comb_g, comb_b, slots, slot0 + blockIdx.x, dim, wave, lane);
}

// Element-wise backward: one wave per workgroup; the workgroup's slot in the
// workspace accumulates its gamma and beta sums directly (only this wave touches it).
template <typename WT, typename OT>
__global__ void __launch_bounds__(kWave)
bwd_elem_kernel(const WT* __restrict__ w, int64_t rows, int64_t dim, const int64_t* __restrict__ idx,
                int64_t ntok, const float* __restrict__ gamma, const float* __restrict__ mean,
                const float* __restrict__ rstd, const OT* __restrict__ dout,
                float* __restrict__ dweight, float* __restrict__ ws) {
  const int lane = threadIdx.x;
  const float n_dim = static_cast<float>(dim);
  float* slot_g = ws + static_cast<int64_t>(blockIdx.x) * 2 * dim;
  float* slot_b = slot_g + dim;
  for (int64_t c = lane; c < dim; c += kWave) {
    slot_g[c] = 0.0f;
    slot_b[c] = 0.0f;
  }
  for (int64_t t = blockIdx.x; t < ntok; t += gridDim.x) {
    const int64_t r = idx[t];
    if (r < 0 || r >= rows) continue;
    const WT* row = w + r * dim;
    const OT* dyrow = dout + t * dim;
    const float mu = mean[t], rs = rstd[t];
    float c1 = 0.0f, c2 = 0.0f;
    for (int64_t c = lane; c < dim; c += kWave) {
      const float xh = (Elem<WT>::load(row, c) - mu) * rs;
      const float dy = Elem<OT>::load(dyrow, c);
      const float g = dy * gamma[c];
      c1 = c1 + g;
      c2 = c2 + (g * xh);
      slot_g[c] = slot_g[c] + (dy * xh);
      slot_b[c] = slot_b[c] + dy;
    }
    const float m1 = wave_sum(c1) / n_dim;
    const float m2 = wave_sum(c2) / n_dim;
    float* drow = dweight + r * dim;
    for (int64_t c = lane; c < dim; c += kWave) {
      const float xh = (Elem<WT>::load(row, c) - mu) * rs;
      const float g = Elem<OT>::load(dyrow, c) * gamma[c];
      unsafeAtomicAdd(drow + c, rs * ((g - m1) - (xh * m2)));
    }
  }
}

// dgamma[c] and dbeta[c] from the slots, in two deterministic steps.  Step 1:
// workgroup (column block, group g) sums slots [g * per, (g + 1) * per): thread
// (column c, subgroup j) adds the group's slots j, j + 4, ... in order, and the four
// subgroup sums are added in subgroup order into level1[g].  Step 2 does the same over
// the groups: subgroup j adds groups j, j + 4, ... (all its loads issued first), and
// the four subgroup sums are added in subgroup order.
constexpr int kReduceGroups = 64;

__global__ void __launch_bounds__(256) bwd_reduce_step1_kernel(const float* __restrict__ ws,
                                                               int64_t nslots, int64_t per,
                                                               int64_t dim,
                                                               float* __restrict__ level1) {
  __shared__ float part[2][4][64];
  const int col = threadIdx.x % 64;
  const int sub = threadIdx.x / 64;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + col;
  const int64_t g = blockIdx.y;
  const int64_t k0 = g * per;
  const int64_t k1 = k0 + per < nslots ? k0 + per : nslots;
  float a = 0.0f, b = 0.0f;
  if (c < dim) {
    for (int64_t k = k0 + sub; k < k1; k += 4) {
      a = a + ws[(2 * k) * dim + c];
      b = b + ws[(2 * k + 1) * dim + c];
    }
  }
  part[0][sub][col] = a;
  part[1][sub][col] = b;
  __syncthreads();
  if (sub == 0 && c < dim) {
    level1[(2 * g) * dim + c] = ((part[0][0][col] + part[0][1][col]) + part[0][2][col]) + part[0][3][col];
    level1[(2 * g + 1) * dim + c] = ((part[1][0][col] + part[1][1][col]) + part[1][2][col]) + part[1][3][col];
  }
}

__global__ void __launch_bounds__(256) bwd_reduce_step2_kernel(const float* __restrict__ level1,
                                                               int64_t ngroups, int64_t dim,
                                                               float* __restrict__ dgamma,
                                                               float* __restrict__ dbeta) {
  __shared__ float part[2][4][64];
  const int col = threadIdx.x % 64;
  const int sub = threadIdx.x / 64;
  for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64; c0 < dim;
       c0 += static_cast<int64_t>(gridDim.x) * 64) {
    const int64_t c = c0 + col;
    const int64_t cl = c < dim ? c : 0;
    // all of the thread's loads are issued before the first add
    constexpr int kPer = kReduceGroups / 4;
    float va[kPer], vb[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t g = sub + 4 * i < ngroups ? sub + 4 * i : 0;
      va[i] = ngroups > 0 ? level1[(2 * g) * dim + cl] : 0.0f;
      vb[i] = ngroups > 0 ? level1[(2 * g + 1) * dim + cl] : 0.0f;
    }
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (sub + 4 * i < ngroups) {
        a = a + va[i];
        b = b + vb[i];
      }
    }
    part[0][sub][col] = a;
    part[1][sub][col] = b;
    __syncthreads();
    if (sub == 0 && c < dim) {
      dgamma[c] = ((part[0][0][col] + part[0][1][col]) + part[0][2][col]) + part[0][3][col];
      dbeta[c] = ((part[1][0][col] + part[1][1][col]) + part[1][2][col]) + part[1][3][col];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host side

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_cus[kMaxDevices];

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QOPT_ELAUNCH;
  std::call_once(g_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      g_cus[dev] = n;
  });
  if (g_cus[dev] <= 0) return QOPT_ELAUNCH;
  *cus = g_cus[dev];
  return QOPT_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? QOPT_OK : QOPT_ELAUNCH; }

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

size_t dtype_size(int dt) { return dt == QOPT_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == QOPT_F32 || dt == QOPT_BF16; }

// Slices of 256 columns for the vector kernels: the smallest of 2, 4, 8, 16 that
// covers dim (0 if dim is too wide).
int slices_for(int64_t dim) {
  for (int s = 2; s <= kMaxSlices; s *= 2)
    if (dim <= 256 * s) return s;
  return 0;
}

template <typename K>
int persistent_grid(K kernel, int threads, size_t lds, int64_t want, unsigned* grid) {
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != QOPT_OK) return rc;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess ||
      per_cu <= 0)
    return QOPT_ELAUNCH;
  const int64_t resident = static_cast<int64_t>(cus) * per_cu;
  *grid = static_cast<unsigned>(want < resident ? want : resident);
  return QOPT_OK;
}

int64_t bwd_slots(int64_t ntok, int cus) {
  const int64_t cap = static_cast<int64_t>(cus) * kBwdSlotsPerCu;
  return ntok < cap ? ntok : cap;
}

template <int S, typename WT, typename OT>
int launch_fwd_vec(const void* w, int64_t rows, int64_t dim, const int64_t* idx, int64_t ntok,
                   const float* gamma, const float* beta, float eps, void* out, float* mean,
                   float* rstd, int32_t* bad, hipStream_t stream) {
  auto kernel = fwd_vec_kernel<S, WT, OT>;
  const size_t lds = 2 * S * kWave * sizeof(f32x4);
  unsigned grid = 0;
  int rc = persistent_grid(kernel, kVecThreads, lds, (ntok + kVecWaves - 1) / kVecWaves, &grid);
  if (rc != QOPT_OK) return rc;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kVecThreads), lds, stream,
                     static_cast<const WT*>(w), rows, static_cast<int32_t>(dim), idx, ntok, gamma,
                     beta, eps, static_cast<OT*>(out), mean, rstd, bad);
  return launch_status();
}

template <typename WT, typename OT>
int dispatch_fwd(int S, const void* w, int64_t rows, int64_t dim, const int64_t* idx, int64_t ntok,
                 const float* gamma, const float* beta, float eps, void* out, float* mean,
                 float* rstd, int32_t* bad, hipStream_t stream) {
  switch (S) {
    case 2: return launch_fwd_vec<2, WT, OT>(w, rows, dim, idx, ntok, gamma, beta, eps, out, mean, rstd, bad, stream);
    case 4: return launch_fwd_vec<4, WT, OT>(w, rows, dim, idx, ntok, gamma, beta, eps, out, mean, rstd, bad, stream);
    case 8: return launch_fwd_vec<8, WT, OT>(w, rows, dim, idx, ntok, gamma, beta, eps, out, mean, rstd, bad, stream);
    case 16: return launch_fwd_vec<16, WT, OT>(w, rows, dim, idx, ntok, gamma, beta, eps, out, mean, rstd, bad, stream);
    default: break;
  }
  auto kernel = fwd_elem_kernel<WT, OT>;
  unsigned grid = 0;
  int rc = persistent_grid(kernel, kWave, 0, ntok, &grid);
  if (rc != QOPT_OK) return rc;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kWave), 0, stream, static_cast<const WT*>(w), rows,
                     dim, idx, ntok, gamma, beta, eps, static_cast<OT*>(out), mean, rstd, bad);
  return launch_status();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace of the grouped backward: sort keys and values (in and out), the radix
// sort's own storage, the per-chunk partial sums and the dgamma / dbeta slots of the
// two grouped kernels.
struct GroupLayout {
  size_t keys_in = 0, vals_in = 0, keys_out = 0, vals_out = 0, sort_tmp = 0, sort_bytes = 0;
  size_t parts = 0, slots = 0, total = 0;
  int64_t nchunks = 0;
  unsigned grid = 0;        // chunk kernel: two-wave workgroups, persistent
  unsigned span_grid = 0;   // span finish kernel: persistent, one wave per run
};

int group_layout(int64_t ntok, int64_t dim, int cus, GroupLayout* L) {
  L->nchunks = (ntok + kSegChunk - 1) / kSegChunk;
  const int64_t cap = static_cast<int64_t>(cus) * kChunkWgPerCu;
  L->grid = static_cast<unsigned>(L->nchunks < cap ? L->nchunks : cap);
  const int64_t span_want = (L->nchunks + kVecWaves - 1) / kVecWaves;
  L->span_grid = static_cast<unsigned>(span_want < cus ? span_want : cus);
  size_t sb = 0;
  if (rocprim::radix_sort_pairs(nullptr, sb, static_cast<const uint32_t*>(nullptr),
                                static_cast<uint32_t*>(nullptr), static_cast<const int32_t*>(nullptr),
                                static_cast<int32_t*>(nullptr), static_cast<unsigned int>(ntok), 0u,
                                32u, hipStream_t{}) != hipSuccess)
    return QOPT_ELAUNCH;
  const size_t n = static_cast<size_t>(ntok);
  size_t off = 0;
  L->keys_in = off;
  off = align256(off + 4 * n);
  L->vals_in = off;
  off = align256(off + 4 * n);
  L->keys_out = off;
  off = align256(off + 4 * n);
  L->vals_out = off;
  off = align256(off + 4 * n);
  L->sort_tmp = off;
  L->sort_bytes = sb;
  off = align256(off + sb);
  L->parts = off;
  off = align256(off + static_cast<size_t>(L->nchunks) * 2 * static_cast<size_t>(dim) * 4);
  L->slots = off;
  off = align256(off + (static_cast<size_t>(L->grid) + L->span_grid) * 2 *
                            static_cast<size_t>(dim) * 4);
  L->total = off;
  return QOPT_OK;
}

// The grouped path applies to vector-path widths, tables whose row count leaves room
// for the invalid-index key, and token counts the radix sort takes.
bool group_shape_ok(int64_t rows, int64_t dim, int64_t ntok) {
  return dim % 4 == 0 && slices_for(dim) != 0 && rows < 0xFFFFFFFFll && ntok < (int64_t{1} << 31);
}

template <int S, typename WT, typename OT>
int launch_grouped(const void* w, int64_t rows, int64_t dim, const int64_t* idx, int64_t ntok,
                   const float* gamma, const float* mean, const float* rstd, const void* dout,
                   float* dweight, char* ws, const GroupLayout& L, hipStream_t stream) {
  uint32_t* keys_in = reinterpret_cast<uint32_t*>(ws + L.keys_in);
  int32_t* vals_in = reinterpret_cast<int32_t*>(ws + L.vals_in);
  uint32_t* keys = reinterpret_cast<uint32_t*>(ws + L.keys_out);
  int32_t* vals = reinterpret_cast<int32_t*>(ws + L.vals_out);
  float* parts = reinterpret_cast<float*>(ws + L.parts);
  float* slots = reinterpret_cast<float*>(ws + L.slots);
  const int64_t kgrid = (ntok + 255) / 256 < 4096 ? (ntok + 255) / 256 : 4096;
  hipLaunchKernelGGL(sort_keys_kernel, dim3(static_cast<unsigned>(kgrid)), dim3(256), 0, stream,
                     idx, ntok, static_cast<uint32_t>(rows), keys_in, vals_in);
  int rc = launch_status();
  if (rc != QOPT_OK) return rc;
  // Keys lie in [0, rows], so only their low bit-length(rows) bits are sorted: the
  // order is the full sort's (radix sorting is stable) with fewer digit passes.  The
  // workspace was sized for all 32 bits, an upper bound for fewer.
  const unsigned key_bits = 32u - static_cast<unsigned>(__builtin_clz(static_cast<uint32_t>(rows) | 1u));
  size_t need = 0;
  if (rocprim::radix_sort_pairs(nullptr, need, keys_in, keys, vals_in, vals,
                                static_cast<unsigned int>(ntok), 0u, key_bits, stream) != hipSuccess)
    return QOPT_ELAUNCH;
  if (need > L.sort_bytes) return QOPT_EINTERNAL;
  size_t sb = L.sort_bytes;
  if (rocprim::radix_sort_pairs(ws + L.sort_tmp, sb, keys_in, keys, vals_in, vals,
                                static_cast<unsigned int>(ntok), 0u, key_bits, stream) != hipSuccess)
    return QOPT_ELAUNCH;
  const size_t lds = 3 * S * kWave * sizeof(f32x4);
  hipLaunchKernelGGL((group_chunk_kernel<S, WT, OT>), dim3(L.grid), dim3(kPairThreads),
                     S * kWave * sizeof(f32x4), stream, static_cast<const WT*>(w), static_cast<uint32_t>(rows),
                     static_cast<int32_t>(dim), keys, vals, ntok, L.nchunks, gamma, mean, rstd,
                     static_cast<const OT*>(dout), dweight, parts, slots);
  rc = launch_status();
  if (rc != QOPT_OK) return rc;
  const int64_t tasks = L.nchunks * S;
  hipLaunchKernelGGL((group_span_sum_kernel<S>), dim3(static_cast<unsigned>((tasks + kVecWaves - 1) / kVecWaves)),
                     dim3(kVecThreads), 0, stream, keys, static_cast<uint32_t>(rows),
                     static_cast<int32_t>(dim), ntok, L.nchunks, parts);
  rc = launch_status();
  if (rc != QOPT_OK) return rc;
  hipLaunchKernelGGL((group_span_finish_kernel<S, WT>), dim3(L.span_grid), dim3(kVecThreads),
                     lds, stream, static_cast<const WT*>(w), static_cast<uint32_t>(rows),
                     static_cast<int32_t>(dim), keys, vals, ntok, L.nchunks, gamma, mean, rstd,
                     dweight, parts, slots, static_cast<int64_t>(L.grid));
  return launch_status();
}

template <typename WT, typename OT>
int dispatch_bwd(int S, const void* w, int64_t rows, int64_t dim, const int64_t* idx, int64_t ntok,
                 const float* gamma, const float* mean, const float* rstd, const void* dout,
                 float* dweight, char* ws, int cus, float** slots, int64_t* nslots,
                 hipStream_t stream) {
  if (S) {
    GroupLayout L;
    int rc = group_layout(ntok, dim, cus, &L);
    if (rc != QOPT_OK) return rc;
    *slots = reinterpret_cast<float*>(ws + L.slots);
    *nslots = static_cast<int64_t>(L.grid) + L.span_grid;
    switch (S) {
      case 2: return launch_grouped<2, WT, OT>(w, rows, dim, idx, ntok, gamma, mean, rstd, dout, dweight, ws, L, stream);
      case 4: return launch_grouped<4, WT, OT>(w, rows, dim, idx, ntok, gamma, mean, rstd, dout, dweight, ws, L, stream);
      case 8: return launch_grouped<8, WT, OT>(w, rows, dim, idx, ntok, gamma, mean, rstd, dout, dweight, ws, L, stream);
      default: return launch_grouped<16, WT, OT>(w, rows, dim, idx, ntok, gamma, mean, rstd, dout, dweight, ws, L, stream);
    }
  }
  const int64_t cap = static_cast<int64_t>(cus) * kBwdSlotsPerCu;
  const unsigned grid = static_cast<unsigned>(ntok < cap ? ntok : cap);
  *slots = reinterpret_cast<float*>(ws);
  *nslots = grid;
  hipLaunchKernelGGL((bwd_elem_kernel<WT, OT>), dim3(grid), dim3(kWave), 0, stream,
                     static_cast<const WT*>(w), rows, dim, idx, ntok, gamma, mean, rstd,
                     static_cast<const OT*>(dout), dweight, reinterpret_cast<float*>(ws));
  return launch_status();
}

// Workspace bytes for (ntok, dim): the larger of the grouped and element-wise needs.
// Level-1 sums of the dgamma / dbeta reduction sit after the larger of the two paths'
// regions; returns that offset too.
int workspace_need(int64_t ntok, int64_t dim, int cus, size_t* bytes, size_t* level1_off = nullptr) {
  size_t b = static_cast<size_t>(bwd_slots(ntok, cus)) * 2 * static_cast<size_t>(dim) * 4;
  if (dim % 4 == 0 && slices_for(dim) != 0 && ntok < (int64_t{1} << 31)) {
    GroupLayout L;
    int rc = group_layout(ntok, dim, cus, &L);
    if (rc != QOPT_OK) return rc;
    if (L.total > b) b = L.total;
  }
  b = align256(b);
  if (level1_off) *level1_off = b;
  *bytes = b + static_cast<size_t>(kReduceGroups) * 2 * static_cast<size_t>(dim) * 4;
  return QOPT_OK;
}

// Vector path: width a multiple of 4 within the limit, and every row of the table
// and of the token-major arrays aligned for 4-element accesses.
bool vector_ok(int64_t dim, const void* w, int wdt, const void* o, int odt) {
  return dim % 4 == 0 && slices_for(dim) != 0 && aligned(w, 4 * dtype_size(wdt)) &&
         aligned(o, 4 * dtype_size(odt));
}

int check_common(const void* w, int wdt, int64_t rows, int64_t dim, const int64_t* idx,
                 int64_t ntok, const float* gamma, const void* o, int odt) {
  if (rows < 0 || dim < 0 || ntok < 0) return QOPT_EINVAL;
  if (!dtype_ok(wdt) || !dtype_ok(odt)) return QOPT_EUNSUPPORTED;
  if (ntok == 0) return QOPT_OK;
  if (rows < 1 || dim < 1) return QOPT_EINVAL;
  if (!w || !idx || !gamma || !o) return QOPT_EINVAL;
  if (dim > (int64_t{1} << 40) / (rows > ntok ? rows : ntok)) return QOPT_EINVAL;
  if (!aligned(w, dtype_size(wdt)) || !aligned(o, dtype_size(odt)) || !aligned(idx, 8) ||
      !aligned(gamma, 4))
    return QOPT_EALIGN;
  return QOPT_OK;
}

}  // namespace

extern "C" int qopt_embedding_xavier_init(void* weight_dev, int weight_dtype, int64_t rows,
                                          int64_t dim, uint64_t seed, void* stream) {
  if (rows < 0 || dim < 0) return QOPT_EINVAL;
  if (!dtype_ok(weight_dtype)) return QOPT_EUNSUPPORTED;
  if (rows == 0 || dim == 0) return QOPT_OK;
  if (!weight_dev) return QOPT_EINVAL;
  if (dim > (int64_t{1} << 50) / rows) return QOPT_EINVAL;
  if (!aligned(weight_dev, dtype_size(weight_dtype))) return QOPT_EALIGN;
  const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(dim);
  const uint64_t nblocks = (n + 3) / 4;
  const float a = static_cast<float>(std::sqrt(6.0 / (static_cast<double>(rows) + static_cast<double>(dim))));
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != QOPT_OK) return rc;
  const uint64_t want = (nblocks + 255) / 256;
  const uint64_t cap = static_cast<uint64_t>(cus) * 8;
  const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (weight_dtype == QOPT_F32)
    hipLaunchKernelGGL(xavier_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<float*>(weight_dev), n, nblocks, k0, k1, a);
  else
    hipLaunchKernelGGL(xavier_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<uint16_t*>(weight_dev), n, nblocks, k0, k1, a);
  return launch_status();
}

extern "C" int qopt_stable_embedding_forward(const void* weight_dev, int weight_dtype, int64_t rows,
                                             int64_t dim, const int64_t* idx_dev, int64_t ntokens,
                                             const float* gamma_dev, const float* beta_dev,
                                             float eps, void* out_dev, int out_dtype,
                                             float* mean_dev, float* rstd_dev,
                                             int32_t* bad_count_dev, void* stream) {
  int rc = check_common(weight_dev, weight_dtype, rows, dim, idx_dev, ntokens, gamma_dev, out_dev,
                        out_dtype);
  if (rc != QOPT_OK || ntokens == 0) return rc;
  if (!beta_dev) return QOPT_EINVAL;
  if (!std::isfinite(eps) || eps < 0.0f) return QOPT_EINVAL;
  if ((mean_dev == nullptr) != (rstd_dev == nullptr)) return QOPT_EINVAL;
  if (!aligned(beta_dev, 4) || !aligned(mean_dev, 4) || !aligned(rstd_dev, 4) ||
      !aligned(bad_count_dev, 4))
    return QOPT_EALIGN;
  const int S = vector_ok(dim, weight_dev, weight_dtype, out_dev, out_dtype) ? slices_for(dim) : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
#define QOPT_FWD(WT, OT)                                                                          \
  dispatch_fwd<WT, OT>(S, weight_dev, rows, dim, idx_dev, ntokens, gamma_dev, beta_dev, eps,      \
                       out_dev, mean_dev, rstd_dev, bad_count_dev, s)
  if (weight_dtype == QOPT_F32)
    return out_dtype == QOPT_F32 ? QOPT_FWD(float, float) : QOPT_FWD(float, uint16_t);
  return out_dtype == QOPT_F32 ? QOPT_FWD(uint16_t, float) : QOPT_FWD(uint16_t, uint16_t);
#undef QOPT_FWD
}

extern "C" int qopt_stable_embedding_backward_workspace(int64_t ntokens, int64_t dim,
                                                        size_t* bytes) {
  if (!bytes || ntokens < 0 || dim < 0) return QOPT_EINVAL;
  *bytes = 0;
  if (ntokens == 0 || dim == 0) return QOPT_OK;
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != QOPT_OK) return rc;
  return workspace_need(ntokens, dim, cus, bytes);
}

namespace {

// The backward over a caller's workspace; `too_small` is the status returned when the
// workspace cannot hold the shape's need.
int backward_impl(const void* weight_dev, int weight_dtype, int64_t rows, int64_t dim,
                  const int64_t* idx_dev, int64_t ntokens, const float* gamma_dev,
                  const float* mean_dev, const float* rstd_dev, const void* dout_dev,
                  int dout_dtype, float* dweight_dev, float* dgamma_dev, float* dbeta_dev,
                  void* workspace_dev, size_t workspace_bytes, int too_small, void* stream) {
  if (rows < 0 || dim < 0 || ntokens < 0) return QOPT_EINVAL;
  if (!dtype_ok(weight_dtype) || !dtype_ok(dout_dtype)) return QOPT_EUNSUPPORTED;
  if (dim == 0) return ntokens == 0 ? QOPT_OK : QOPT_EINVAL;
  if (!dgamma_dev || !dbeta_dev) return QOPT_EINVAL;
  if (!aligned(dgamma_dev, 4) || !aligned(dbeta_dev, 4)) return QOPT_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc != QOPT_OK) return rc;
  const unsigned rgrid = static_cast<unsigned>(
      (dim + 63) / 64 < static_cast<int64_t>(cus) * 16 ? (dim + 63) / 64 : static_cast<int64_t>(cus) * 16);
  if (ntokens == 0) {
    hipLaunchKernelGGL(bwd_reduce_step2_kernel, dim3(rgrid), dim3(256), 0, s, nullptr, int64_t{0},
                       dim, dgamma_dev, dbeta_dev);
    return launch_status();
  }
  rc = check_common(weight_dev, weight_dtype, rows, dim, idx_dev, ntokens, gamma_dev, dout_dev,
                    dout_dtype);
  if (rc != QOPT_OK) return rc;
  if (!mean_dev || !rstd_dev || !dweight_dev || !workspace_dev) return QOPT_EINVAL;
  if (!aligned(mean_dev, 4) || !aligned(rstd_dev, 4) || !aligned(dweight_dev, 4) ||
      !aligned(workspace_dev, 16))
    return QOPT_EALIGN;
  size_t need = 0, level1_off = 0;
  rc = workspace_need(ntokens, dim, cus, &need, &level1_off);
  if (rc != QOPT_OK) return rc;
  if (workspace_bytes < need) return too_small;
  const bool vec = vector_ok(dim, weight_dev, weight_dtype, dout_dev, dout_dtype) &&
                   group_shape_ok(rows, dim, ntokens) && aligned(dweight_dev, 16);
  const int S = vec ? slices_for(dim) : 0;
  char* ws = static_cast<char*>(workspace_dev);
  float* slots = nullptr;
  int64_t nslots = 0;
#define QOPT_BWD(WT, OT)                                                                          \
  dispatch_bwd<WT, OT>(S, weight_dev, rows, dim, idx_dev, ntokens, gamma_dev, mean_dev, rstd_dev, \
                       dout_dev, dweight_dev, ws, cus, &slots, &nslots, s)
  if (weight_dtype == QOPT_F32)
    rc = dout_dtype == QOPT_F32 ? QOPT_BWD(float, float) : QOPT_BWD(float, uint16_t);
  else
    rc = dout_dtype == QOPT_F32 ? QOPT_BWD(uint16_t, float) : QOPT_BWD(uint16_t, uint16_t);
#undef QOPT_BWD
  if (rc != QOPT_OK) return rc;
  float* level1 = reinterpret_cast<float*>(ws + level1_off);
  const int64_t per = (nslots + kReduceGroups - 1) / kReduceGroups;
  const int64_t ngroups = (nslots + per - 1) / per;
  hipLaunchKernelGGL(bwd_reduce_step1_kernel,
                     dim3(static_cast<unsigned>((dim + 63) / 64), static_cast<unsigned>(ngroups)),
                     dim3(256), 0, s, slots, nslots, per, dim, level1);
  rc = launch_status();
  if (rc != QOPT_OK) return rc;
  hipLaunchKernelGGL(bwd_reduce_step2_kernel, dim3(rgrid), dim3(256), 0, s, level1, ngroups, dim,
                     dgamma_dev, dbeta_dev);
  return launch_status();
}

// Scratch of the allocation-free backward: one fixed array per device, loaded with the
// library's device code.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol); each device's own address is looked up
// once, with that device current, and kept.
__device__ __align__(256) char scratch[QOPT_EMB_STATIC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];

int device_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return QOPT_ELAUNCH;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = p;
  });
  if (g_scratch_ptr[dev] == nullptr) return QOPT_ELAUNCH;
  *ptr = g_scratch_ptr[dev];
  return QOPT_OK;
}

}  // namespace

extern "C" int qopt_stable_embedding_backward(const void* weight_dev, int weight_dtype, int64_t rows,
                                              int64_t dim, const int64_t* idx_dev, int64_t ntokens,
                                              const float* gamma_dev, const float* mean_dev,
                                              const float* rstd_dev, const void* dout_dev,
                                              int dout_dtype, float* dweight_dev, float* dgamma_dev,
                                              float* dbeta_dev, void* workspace_dev,
                                              size_t workspace_bytes, void* stream) {
  return backward_impl(weight_dev, weight_dtype, rows, dim, idx_dev, ntokens, gamma_dev, mean_dev,
                       rstd_dev, dout_dev, dout_dtype, dweight_dev, dgamma_dev, dbeta_dev,
                       workspace_dev, workspace_bytes, QOPT_EINVAL, stream);
}

extern "C" int qopt_stable_embedding_backward_noalloc(const void* weight_dev, int weight_dtype,
                                                      int64_t rows, int64_t dim,
                                                      const int64_t* idx_dev, int64_t ntokens,
                                                      const float* gamma_dev, const float* mean_dev,
                                                      const float* rstd_dev, const void* dout_dev,
                                                      int dout_dtype, float* dweight_dev,
                                                      float* dgamma_dev, float* dbeta_dev,
                                                      void* stream) {
  void* ws = nullptr;
  const int rc = device_scratch(&ws);
  if (rc != QOPT_OK) return rc;
  return backward_impl(weight_dev, weight_dtype, rows, dim, idx_dev, ntokens, gamma_dev, mean_dev,
                       rstd_dev, dout_dev, dout_dtype, dweight_dev, dgamma_dev, dbeta_dev, ws,
                       QOPT_EMB_STATIC_SCRATCH_BYTES, QOPT_ENOSPACE, stream);
}
