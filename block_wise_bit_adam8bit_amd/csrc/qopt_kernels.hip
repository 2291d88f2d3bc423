// Device side of libqopt for gfx950: block-wise quantize, dequantize and the fused
// 8-bit Adam step ("8-BIT OPTIMIZERS VIA BLOCK-WISE QUANTIZATION" summary page:
// §2 opening -- dequantize the 8-bit state, update in higher precision, store 8-bit;
// §2 "Block-wise Quantization" -- 2048-element blocks normalised by their own
// absmax with no synchronisation between blocks; §2 "Dynamic Quantization" -- the
// signed / unsigned dynamic-tree codes).
//
// Execution model (all three kernels):
//   * One wavefront (64 lanes) owns one 2048-element block at a time.  Lane l holds
//     elements s*256 + 4l .. s*256 + 4l + 3 for s = 0..7, so every global access of a
//     slice is one contiguous, fully coalesced wave-wide vector access (16 B per lane
//     for fp32, 8 B for bf16, 4 B for codes).
//   * A block's absmax is a max over the lane's 32 values then a butterfly across the
//     wave: no LDS, no barrier, no other wave involved.
//   * Workgroups of 4 waves are persistent: each stages the codebook(s) into LDS once
//     (the only barrier) and then walks blocks with a grid stride.
//   * Code lookup: decode is one LDS read; encode is one LDS byte read (bucket index
//     from the binary32 bits) plus one LDS threshold read and a compare.
// Floating point: compiled with -ffp-contract=off; '/' and sqrtf are the correctly
// rounded IEEE operations (HIP's default), fp32 denormals are kept.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "qopt.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                       // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kSlices = QOPT_BLOCK / (kWave * 4);  // 8 slices of 4 elements per lane
constexpr int kMaxTensors = 48;                 // tensors per launch (kernarg budget)
constexpr int kRows = static_cast<int>(sizeof(qopt_codebook) / 16);
static_assert(kSlices * kWave * 4 == QOPT_BLOCK, "block layout");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef QOPT_NONTEMPORAL
#define QOPT_NONTEMPORAL 1
#endif

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
#if QOPT_NONTEMPORAL
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
#if QOPT_NONTEMPORAL
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ void stage_codebook(qopt_codebook* dst, const qopt_codebook* src) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int i = threadIdx.x; i < kRows; i += kThreads) d[i] = s[i];
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// Per-codebook encoder parameters kept in registers for the whole kernel.
struct Encoder {
  const qopt_codebook* cb;  // LDS copy
  int32_t key0;
  int32_t last_bucket;
};

__device__ __forceinline__ Encoder make_encoder(const qopt_codebook* lds_cb) {
  Encoder e;
  e.cb = lds_cb;
  e.key0 = static_cast<int32_t>(lds_cb->key0);
  uint32_t nb = lds_cb->nbuckets;
  nb = nb < 1u ? 1u : (nb > QOPT_MAX_BUCKETS ? QOPT_MAX_BUCKETS : nb);
  e.last_bucket = static_cast<int32_t>(nb) - 1;
  return e;
}

// Magnitude index of a >= 0: bucket start index, plus one if a reaches the single
// threshold that may lie inside the bucket.  Indexes stay inside the tables for any
// table contents (bucket bytes <= 255, thresh has >= 257 entries).
__device__ __forceinline__ uint32_t encode_mag(const Encoder& e, float a) {
  int32_t i = static_cast<int32_t>(__float_as_uint(a) >> 15) - e.key0;
  i = i < 0 ? 0 : (i > e.last_bucket ? e.last_bucket : i);
  const uint32_t b = e.cb->bucket[i];
  return b + (a >= e.cb->thresh[b + 1] ? 1u : 0u);
}

// Per-block normalisation: reciprocal, stored absmax and effective sign mask.
struct BlockScale {
  float r;
  float absmax;
  uint32_t sign_mask;
};

__device__ __forceinline__ BlockScale block_scale(float amax, uint32_t sign_mask) {
  BlockScale s;
  const bool ok = amax >= FLT_MIN;  // zero or subnormal blocks store absmax 0, codes 0
  s.r = ok ? 1.0f / amax : 0.0f;
  s.absmax = ok ? amax : 0.0f;
  s.sign_mask = ok ? sign_mask : 0u;
  return s;
}

__device__ __forceinline__ uint32_t encode_signed(const Encoder& e, const BlockScale& s, float x) {
  return encode_mag(e, fabsf(x) * s.r) | (x < 0.0f ? s.sign_mask : 0u);
}

// ---------------------------------------------------------- codec kernels

struct CodecArgs {
  const qopt_codebook* cb;
  const float* x;         // quantize input / dequantize output
  float* y;
  const uint8_t* codes_in;
  uint8_t* codes_out;
  const float* absmax_in;
  float* absmax_out;
  int64_t n;
  uint32_t nblocks;
  uint32_t vector_ok;     // pointers allow the vector path for full blocks
};

__global__ void __launch_bounds__(kThreads)
quantize_kernel(CodecArgs a) {
  __shared__ __align__(16) qopt_codebook cb;
  stage_codebook(&cb, a.cb);
  __syncthreads();
  const Encoder enc = make_encoder(&cb);
  const uint32_t sign_mask = cb.sign_mask;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t stride = gridDim.x * kWaves;

  for (uint32_t blk = blockIdx.x * kWaves + wave; blk < a.nblocks; blk += stride) {
    const int64_t base = static_cast<int64_t>(blk) * QOPT_BLOCK;
    const int64_t rem = a.n - base;
    const int len = rem < QOPT_BLOCK ? static_cast<int>(rem) : QOPT_BLOCK;
    float x[kSlices][4];
    if (len == QOPT_BLOCK && a.vector_ok) {
      const f32x4* src = reinterpret_cast<const f32x4*>(a.x + base);
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        const f32x4 v = ld_stream(src + s * kWave + lane);
        x[s][0] = v.x; x[s][1] = v.y; x[s][2] = v.z; x[s][3] = v.w;
      }
    } else {
#pragma unroll
      for (int s = 0; s < kSlices; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = s * 256 + lane * 4 + j;
          x[s][j] = e < len ? a.x[base + e] : 0.0f;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < kSlices; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(x[s][j]));
    const BlockScale sc = block_scale(wave_max(amax), sign_mask);

    if (len == QOPT_BLOCK && a.vector_ok) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes_out + base);
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w |= encode_signed(enc, sc, x[s][j]) << (8 * j);
        st_stream(dst + s * kWave + lane, w);
      }
    } else {
#pragma unroll
      for (int s = 0; s < kSlices; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = s * 256 + lane * 4 + j;
          if (e < len) a.codes_out[base + e] = static_cast<uint8_t>(encode_signed(enc, sc, x[s][j]));
        }
    }
    if (lane == 0) a.absmax_out[blk] = sc.absmax;
  }
}

__global__ void __launch_bounds__(kThreads)
dequantize_kernel(CodecArgs a) {
  __shared__ __align__(16) qopt_codebook cb;
  stage_codebook(&cb, a.cb);
  __syncthreads();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t stride = gridDim.x * kWaves;

  for (uint32_t blk = blockIdx.x * kWaves + wave; blk < a.nblocks; blk += stride) {
    const int64_t base = static_cast<int64_t>(blk) * QOPT_BLOCK;
    const int64_t rem = a.n - base;
    const int len = rem < QOPT_BLOCK ? static_cast<int>(rem) : QOPT_BLOCK;
    const float A = a.absmax_in[blk];
    if (len == QOPT_BLOCK && a.vector_ok) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.codes_in + base);
      f32x4* dst = reinterpret_cast<f32x4*>(a.y + base);
      uint32_t w[kSlices];
#pragma unroll
      for (int s = 0; s < kSlices; ++s) w[s] = ld_stream(src + s * kWave + lane);
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        f32x4 v;
        v.x = cb.decode[w[s] & 0xFFu] * A;
        v.y = cb.decode[(w[s] >> 8) & 0xFFu] * A;
        v.z = cb.decode[(w[s] >> 16) & 0xFFu] * A;
        v.w = cb.decode[w[s] >> 24] * A;
        st_stream(dst + s * kWave + lane, v);
      }
    } else {
#pragma unroll
      for (int s = 0; s < kSlices; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = s * 256 + lane * 4 + j;
          if (e < len) a.y[base + e] = cb.decode[a.codes_in[base + e]] * A;
        }
    }
  }
}

// ------------------------------------------------------------ Adam kernel

struct AdamScalars {
  float b1, b2, omb1, omb2, eps, step_size, inv_sqrt_bc2;
};

// One launch's work: up to kMaxTensors pieces, each a run of whole blocks of one
// tensor.  Large tensors may be split over several launches so that every launch
// of a step covers the same number of blocks.
struct StepChunk {
  void* param[kMaxTensors];             // tensor base pointers
  const void* grad[kMaxTensors];
  uint8_t* m_codes[kMaxTensors];
  uint8_t* v_codes[kMaxTensors];
  float* m_absmax[kMaxTensors];
  float* v_absmax[kMaxTensors];
  int64_t n[kMaxTensors];                // tensor length
  uint32_t block_lo[kMaxTensors];        // first block of the piece
  uint32_t block_start[kMaxTensors + 1]; // prefix sums of the pieces' block counts
  uint32_t npieces;
  uint64_t vector_ok;                    // bit i: piece i may use the vector path
};

template <typename PT> struct ParamIO;

template <> struct ParamIO<float> {
  __device__ static void load4(const void* p, int64_t base, int idx, float out[4]) {
    const f32x4 v = ld_stream(reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + base) + idx);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  __device__ static void store4(void* p, int64_t base, int idx, const float in[4]) {
    f32x4 v;
    v.x = in[0]; v.y = in[1]; v.z = in[2]; v.w = in[3];
    st_stream(reinterpret_cast<f32x4*>(static_cast<float*>(p) + base) + idx, v);
  }
  __device__ static float load1(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static void store1(void* p, int64_t i, float x) { static_cast<float*>(p)[i] = x; }
};

template <> struct ParamIO<uint16_t> {  // bf16 bit patterns
  __device__ static void load4(const void* p, int64_t base, int idx, float out[4]) {
    const u32x2 v = ld_stream(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + base) + idx);
    out[0] = bf16_to_f32(v.x & 0xFFFFu); out[1] = bf16_to_f32(v.x >> 16);
    out[2] = bf16_to_f32(v.y & 0xFFFFu); out[3] = bf16_to_f32(v.y >> 16);
  }
  __device__ static void store4(void* p, int64_t base, int idx, const float in[4]) {
    u32x2 v;
    v.x = f32_to_bf16_rne(in[0]) | (f32_to_bf16_rne(in[1]) << 16);
    v.y = f32_to_bf16_rne(in[2]) | (f32_to_bf16_rne(in[3]) << 16);
    st_stream(reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p) + base) + idx, v);
  }
  __device__ static float load1(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static void store1(void* p, int64_t i, float x) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16_rne(x));
  }
};

// One element of the update; returns the new parameter, leaves m and v.
__device__ __forceinline__ float adam_element(const AdamScalars& k, float p, float g, float m_prev,
                                              float v_prev, float& m, float& v) {
  m = (k.b1 * m_prev) + (k.omb1 * g);
  v = (k.b2 * v_prev) + (k.omb2 * (g * g));
  const float denom = (sqrtf(v) * k.inv_sqrt_bc2) + k.eps;
  const float u = m / denom;
  return p - (k.step_size * u);
}

template <typename PT, typename GT, bool kVector>
__device__ __forceinline__ void adam_block(const AdamScalars& k, const qopt_codebook& cbm,
                                           const qopt_codebook& cbv, const Encoder& em,
                                           const Encoder& ev, void* param, const void* grad,
                                           uint8_t* cm, uint8_t* cv, float* am, float* av,
                                           int64_t base, int len, int lane) {
  const float Am = *am;
  const float Av = *av;
  float m[kSlices][4], v[kSlices][4];
  float mmax = 0.0f, vmax = 0.0f;

#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    const int idx = s * kWave + lane;
    float p4[4], g4[4];
    uint32_t wm = 0, wv = 0;
    if (kVector) {
      ParamIO<PT>::load4(param, base, idx, p4);
      ParamIO<GT>::load4(grad, base, idx, g4);
      wm = ld_stream(reinterpret_cast<const uint32_t*>(cm + base) + idx);
      wv = ld_stream(reinterpret_cast<const uint32_t*>(cv + base) + idx);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = s * 256 + lane * 4 + j;
        const bool in = e < len;
        p4[j] = in ? ParamIO<PT>::load1(param, base + e) : 0.0f;
        g4[j] = in ? ParamIO<GT>::load1(grad, base + e) : 0.0f;
        wm |= (in ? static_cast<uint32_t>(cm[base + e]) : 0u) << (8 * j);
        wv |= (in ? static_cast<uint32_t>(cv[base + e]) : 0u) << (8 * j);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float m_prev = cbm.decode[(wm >> (8 * j)) & 0xFFu] * Am;
      const float v_prev = cbv.decode[(wv >> (8 * j)) & 0xFFu] * Av;
      p4[j] = adam_element(k, p4[j], g4[j], m_prev, v_prev, m[s][j], v[s][j]);
      if (!kVector && s * 256 + lane * 4 + j >= len) { m[s][j] = 0.0f; v[s][j] = 0.0f; }
      mmax = fmaxf(mmax, fabsf(m[s][j]));
      vmax = fmaxf(vmax, v[s][j]);
    }
    if (kVector) {
      ParamIO<PT>::store4(param, base, idx, p4);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = s * 256 + lane * 4 + j;
        if (e < len) ParamIO<PT>::store1(param, base + e, p4[j]);
      }
    }
  }

  const BlockScale sm = block_scale(wave_max(mmax), cbm.sign_mask);
  const BlockScale sv = block_scale(wave_max(vmax), cbv.sign_mask);

#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    const int idx = s * kWave + lane;
    uint32_t wm = 0, wv = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wm |= encode_signed(em, sm, m[s][j]) << (8 * j);
      wv |= encode_signed(ev, sv, v[s][j]) << (8 * j);
    }
    if (kVector) {
      st_stream(reinterpret_cast<uint32_t*>(cm + base) + idx, wm);
      st_stream(reinterpret_cast<uint32_t*>(cv + base) + idx, wv);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = s * 256 + lane * 4 + j;
        if (e < len) {
          cm[base + e] = static_cast<uint8_t>(wm >> (8 * j));
          cv[base + e] = static_cast<uint8_t>(wv >> (8 * j));
        }
      }
    }
  }
  if (lane == 0) {
    *am = sm.absmax;
    *av = sv.absmax;
  }
}

template <typename PT, typename GT>
__global__ void __launch_bounds__(kThreads)
adam8bit_kernel(StepChunk c, AdamScalars k, const qopt_codebook* cbm_g, const qopt_codebook* cbv_g) {
  __shared__ __align__(16) qopt_codebook cb[2];
  stage_codebook(&cb[0], cbm_g);
  stage_codebook(&cb[1], cbv_g);
  __syncthreads();
  const Encoder em = make_encoder(&cb[0]);
  const Encoder ev = make_encoder(&cb[1]);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t stride = gridDim.x * kWaves;
  const uint32_t total = c.block_start[c.npieces];

  for (uint32_t blk = blockIdx.x * kWaves + wave; blk < total; blk += stride) {
    // piece owning this block: last t with block_start[t] <= blk (wave-uniform)
    uint32_t lo = 0, hi = c.npieces;
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) / 2;
      if (c.block_start[mid] <= blk) lo = mid; else hi = mid;
    }
    const uint32_t t = lo;
    const uint32_t lb = c.block_lo[t] + (blk - c.block_start[t]);
    const int64_t base = static_cast<int64_t>(lb) * QOPT_BLOCK;
    const int64_t rem = c.n[t] - base;
    const int len = rem < QOPT_BLOCK ? static_cast<int>(rem) : QOPT_BLOCK;
    if (len == QOPT_BLOCK && ((c.vector_ok >> t) & 1u)) {
      adam_block<PT, GT, true>(k, cb[0], cb[1], em, ev, c.param[t], c.grad[t], c.m_codes[t],
                               c.v_codes[t], c.m_absmax[t] + lb, c.v_absmax[t] + lb, base, len, lane);
    } else {
      adam_block<PT, GT, false>(k, cb[0], cb[1], em, ev, c.param[t], c.grad[t], c.m_codes[t],
                                c.v_codes[t], c.m_absmax[t] + lb, c.v_absmax[t] + lb, base, len, lane);
    }
  }
}

// ------------------------------------------------------------ host helpers

struct DeviceInfo {
  int cus = 0;
};

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

int current_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QOPT_ELAUNCH;
  std::call_once(g_dev_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      g_dev[dev].cus = n;
  });
  if (g_dev[dev].cus <= 0) return QOPT_ELAUNCH;
  *cus = g_dev[dev].cus;
  return QOPT_OK;
}

// Persistent grid: enough workgroups to fill every CU at the kernel's occupancy,
// never more than there are blocks to hand out.
template <typename K>
int grid_for(K kernel, uint32_t nblocks, unsigned* grid) {
  int cus = 0;
  int rc = current_cus(&cus);
  if (rc != QOPT_OK) return rc;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
      per_cu <= 0)
    return QOPT_ELAUNCH;
  const uint64_t resident = static_cast<uint64_t>(cus) * static_cast<uint64_t>(per_cu);
  const uint64_t wanted = (static_cast<uint64_t>(nblocks) + kWaves - 1) / kWaves;
  *grid = static_cast<unsigned>(wanted < resident ? wanted : resident);
  return QOPT_OK;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launch_status() {
  return hipGetLastError() == hipSuccess ? QOPT_OK : QOPT_ELAUNCH;
}

// b^t in binary64 by square-and-multiply over the bits of t, lowest bit first.
double pow_by_squaring(double b, int64_t t) {
  double result = 1.0;
  double base = b;
  uint64_t e = static_cast<uint64_t>(t);
  while (e) {
    if (e & 1u) result = result * base;
    base = base * base;
    e >>= 1;
  }
  return result;
}

bool finite(float x) { return x == x && x - x == 0.0f; }

// Splits the step into launches of equal block counts (the last may be shorter),
// each holding at most kMaxTensors pieces.  For a given launch count the pieces
// are assigned greedily in tensor order; the count grows until every launch fits.
// emit(chunk, blocks) is called once per launch; returns the first error.
template <typename Emit>
int plan_chunks(const qopt_tensor* tensors, int32_t ntensors, size_t psize, size_t gsize,
                uint64_t nchunks, uint64_t total, Emit&& emit, bool* fits) {
  const uint64_t target = (total + nchunks - 1) / nchunks;
  StepChunk c;
  c.npieces = 0;
  c.vector_ok = 0;
  c.block_start[0] = 0;
  uint64_t blocks = 0;
  *fits = true;
  for (int32_t i = 0; i < ntensors; ++i) {
    const qopt_tensor& t = tensors[i];
    if (t.n == 0) continue;
    const uint64_t nb = (static_cast<uint64_t>(t.n) + QOPT_BLOCK - 1) / QOPT_BLOCK;
    const bool vec = aligned(t.param, 4 * psize) && aligned(t.grad, 4 * gsize) &&
                     aligned(t.m_codes, 4) && aligned(t.v_codes, 4);
    uint64_t lo = 0;
    while (lo < nb) {
      if (c.npieces == static_cast<uint32_t>(kMaxTensors)) {
        *fits = false;
        return QOPT_OK;
      }
      const uint64_t take = (nb - lo < target - blocks) ? nb - lo : target - blocks;
      const uint32_t slot = c.npieces++;
      c.param[slot] = t.param;
      c.grad[slot] = t.grad;
      c.m_codes[slot] = t.m_codes;
      c.v_codes[slot] = t.v_codes;
      c.m_absmax[slot] = t.m_absmax;
      c.v_absmax[slot] = t.v_absmax;
      c.n[slot] = t.n;
      c.block_lo[slot] = static_cast<uint32_t>(lo);
      if (vec) c.vector_ok |= uint64_t{1} << slot;
      blocks += take;
      lo += take;
      c.block_start[slot + 1] = static_cast<uint32_t>(blocks);
      if (blocks == target) {
        const int rc = emit(c, blocks);
        if (rc != QOPT_OK) return rc;
        c.npieces = 0;
        c.vector_ok = 0;
        blocks = 0;
      }
    }
  }
  if (c.npieces > 0) return emit(c, blocks);
  return QOPT_OK;
}

// Number of launches of one step over `tensors` (see plan_chunks).
int count_chunks(const qopt_tensor* tensors, int32_t ntensors, size_t psize, size_t gsize,
                 uint64_t* nchunks_out, uint64_t* total_out) {
  uint64_t total = 0, pieces = 0;
  for (int32_t i = 0; i < ntensors; ++i) {
    if (tensors[i].n == 0) continue;
    const uint64_t nb = (static_cast<uint64_t>(tensors[i].n) + QOPT_BLOCK - 1) / QOPT_BLOCK;
    if (nb > 0xFFFFFFFFull) return QOPT_EINVAL;  // block index of one tensor is 32-bit
    total += nb;
    ++pieces;
  }
  *total_out = total;
  *nchunks_out = 0;
  if (total == 0) return QOPT_OK;
  // launches hold < 2^31 blocks and at most kMaxTensors pieces each
  uint64_t nchunks = (pieces + kMaxTensors - 1) / kMaxTensors;
  const uint64_t by_size = (total + 0x7FFFFFFFull - 1) / 0x7FFFFFFFull;
  if (nchunks < by_size) nchunks = by_size;
  for (;; ++nchunks) {
    bool fits = false;
    plan_chunks(tensors, ntensors, psize, gsize, nchunks, total,
                [](const StepChunk&, uint64_t) { return static_cast<int>(QOPT_OK); }, &fits);
    if (fits) break;
  }
  *nchunks_out = nchunks;
  return QOPT_OK;
}

template <typename PT, typename GT>
int launch_step_chunks(const qopt_tensor* tensors, int32_t ntensors, size_t psize, size_t gsize,
                       const AdamScalars& k, const qopt_codebook* cbm, const qopt_codebook* cbv,
                       hipStream_t stream) {
  auto kernel = adam8bit_kernel<PT, GT>;
  uint64_t nchunks = 0, total = 0;
  int rc = count_chunks(tensors, ntensors, psize, gsize, &nchunks, &total);
  if (rc != QOPT_OK || total == 0) return rc;
  unsigned grid = 0;
  bool fits = true;
  return plan_chunks(
      tensors, ntensors, psize, gsize, nchunks, total,
      [&](const StepChunk& c, uint64_t blocks) {
        int r = grid_for(kernel, static_cast<uint32_t>(blocks), &grid);
        if (r != QOPT_OK) return r;
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream, c, k, cbm, cbv);
        return launch_status();
      },
      &fits);
}

int check_step_tensors(const qopt_tensor* tensors, int32_t ntensors, int param_dtype,
                       int grad_dtype, bool* any) {
  if (ntensors < 0) return QOPT_EINVAL;
  if (ntensors > 0 && tensors == nullptr) return QOPT_EINVAL;
  if ((param_dtype != QOPT_F32 && param_dtype != QOPT_BF16) ||
      (grad_dtype != QOPT_F32 && grad_dtype != QOPT_BF16))
    return QOPT_EUNSUPPORTED;
  const size_t psize = param_dtype == QOPT_F32 ? 4 : 2;
  const size_t gsize = grad_dtype == QOPT_F32 ? 4 : 2;
  *any = false;
  for (int32_t i = 0; i < ntensors; ++i) {
    const qopt_tensor& t = tensors[i];
    if (t.n < 0) return QOPT_EINVAL;
    if (t.n == 0) continue;
    *any = true;
    if (!t.param || !t.grad || !t.m_codes || !t.v_codes || !t.m_absmax || !t.v_absmax)
      return QOPT_EINVAL;
    if (!aligned(t.param, psize) || !aligned(t.grad, gsize) || !aligned(t.m_absmax, 4) ||
        !aligned(t.v_absmax, 4))
      return QOPT_EALIGN;
  }
  return QOPT_OK;
}

}  // namespace

// ------------------------------------------------------------ entry points

extern "C" int qopt_quantize_blockwise(const qopt_codebook* cb_dev, const float* x_dev, int64_t n,
                                       uint8_t* codes_dev, float* absmax_dev, void* stream) {
  if (n < 0) return QOPT_EINVAL;
  if (n == 0) return QOPT_OK;
  if (!cb_dev || !x_dev || !codes_dev || !absmax_dev) return QOPT_EINVAL;
  if (!aligned(cb_dev, 16) || !aligned(x_dev, 4) || !aligned(absmax_dev, 4)) return QOPT_EALIGN;
  const uint64_t nb = (static_cast<uint64_t>(n) + QOPT_BLOCK - 1) / QOPT_BLOCK;
  if (nb > 0xFFFFFFFFull) return QOPT_EINVAL;
  CodecArgs a = {};
  a.cb = cb_dev;
  a.x = x_dev;
  a.codes_out = codes_dev;
  a.absmax_out = absmax_dev;
  a.n = n;
  a.nblocks = static_cast<uint32_t>(nb);
  a.vector_ok = aligned(x_dev, 16) && aligned(codes_dev, 4);
  unsigned grid = 0;
  int rc = grid_for(quantize_kernel, a.nblocks, &grid);
  if (rc != QOPT_OK) return rc;
  hipLaunchKernelGGL(quantize_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return launch_status();
}

extern "C" int qopt_dequantize_blockwise(const qopt_codebook* cb_dev, const uint8_t* codes_dev,
                                         const float* absmax_dev, int64_t n, float* y_dev,
                                         void* stream) {
  if (n < 0) return QOPT_EINVAL;
  if (n == 0) return QOPT_OK;
  if (!cb_dev || !codes_dev || !absmax_dev || !y_dev) return QOPT_EINVAL;
  if (!aligned(cb_dev, 16) || !aligned(y_dev, 4) || !aligned(absmax_dev, 4)) return QOPT_EALIGN;
  const uint64_t nb = (static_cast<uint64_t>(n) + QOPT_BLOCK - 1) / QOPT_BLOCK;
  if (nb > 0xFFFFFFFFull) return QOPT_EINVAL;
  CodecArgs a = {};
  a.cb = cb_dev;
  a.y = y_dev;
  a.codes_in = codes_dev;
  a.absmax_in = absmax_dev;
  a.n = n;
  a.nblocks = static_cast<uint32_t>(nb);
  a.vector_ok = aligned(y_dev, 16) && aligned(codes_dev, 4);
  unsigned grid = 0;
  int rc = grid_for(dequantize_kernel, a.nblocks, &grid);
  if (rc != QOPT_OK) return rc;
  hipLaunchKernelGGL(dequantize_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return launch_status();
}

extern "C" int qopt_adam8bit_step(const qopt_tensor* tensors, int32_t ntensors, int param_dtype,
                                  int grad_dtype, const qopt_codebook* cb_m_dev,
                                  const qopt_codebook* cb_v_dev, const qopt_adam_hparams* hp,
                                  void* stream) {
  if (hp == nullptr) return QOPT_EINVAL;
  bool any = false;
  int rc = check_step_tensors(tensors, ntensors, param_dtype, grad_dtype, &any);
  if (rc != QOPT_OK) return rc;
  if (!finite(hp->lr) || !finite(hp->eps) || hp->eps < 0.0f) return QOPT_EINVAL;
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return QOPT_EINVAL;
  if (hp->step < 1) return QOPT_EINVAL;
  if (!any) return QOPT_OK;
  if (!cb_m_dev || !cb_v_dev) return QOPT_EINVAL;
  if (!aligned(cb_m_dev, 16) || !aligned(cb_v_dev, 16)) return QOPT_EALIGN;
  const size_t psize = param_dtype == QOPT_F32 ? 4 : 2;
  const size_t gsize = grad_dtype == QOPT_F32 ? 4 : 2;

  AdamScalars k;
  k.b1 = hp->beta1;
  k.b2 = hp->beta2;
  k.omb1 = 1.0f - hp->beta1;
  k.omb2 = 1.0f - hp->beta2;
  k.eps = hp->eps;
  const double bc1 = 1.0 - pow_by_squaring(static_cast<double>(hp->beta1), hp->step);
  const double bc2 = 1.0 - pow_by_squaring(static_cast<double>(hp->beta2), hp->step);
  k.step_size = static_cast<float>(static_cast<double>(hp->lr) / bc1);
  k.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (param_dtype == QOPT_F32 && grad_dtype == QOPT_F32)
    return launch_step_chunks<float, float>(tensors, ntensors, psize, gsize, k, cb_m_dev, cb_v_dev, s);
  if (param_dtype == QOPT_F32 && grad_dtype == QOPT_BF16)
    return launch_step_chunks<float, uint16_t>(tensors, ntensors, psize, gsize, k, cb_m_dev, cb_v_dev, s);
  if (param_dtype == QOPT_BF16 && grad_dtype == QOPT_F32)
    return launch_step_chunks<uint16_t, float>(tensors, ntensors, psize, gsize, k, cb_m_dev, cb_v_dev, s);
  return launch_step_chunks<uint16_t, uint16_t>(tensors, ntensors, psize, gsize, k, cb_m_dev, cb_v_dev, s);
}

extern "C" int qopt_adam8bit_launch_count(const qopt_tensor* tensors, int32_t ntensors,
                                          int param_dtype, int grad_dtype, int64_t* launches) {
  if (launches == nullptr) return QOPT_EINVAL;
  bool any = false;
  int rc = check_step_tensors(tensors, ntensors, param_dtype, grad_dtype, &any);
  if (rc != QOPT_OK) return rc;
  uint64_t nchunks = 0, total = 0;
  rc = count_chunks(tensors, ntensors, param_dtype == QOPT_F32 ? 4 : 2,
                    grad_dtype == QOPT_F32 ? 4 : 2, &nchunks, &total);
  if (rc != QOPT_OK) return rc;
  *launches = static_cast<int64_t>(nchunks);
  return QOPT_OK;
}
