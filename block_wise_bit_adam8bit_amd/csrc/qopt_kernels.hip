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
//   * A block's absmax is a max over the lane's 32 values then a DPP reduction across
//     the wave: no LDS, no barrier, no other wave involved.
//   * Workgroups of 4 waves are persistent: each stages the codebook(s) into LDS once
//     (the only barrier) and then walks blocks: the codec with a grid stride, the step
//     in runs of consecutive blocks per wave (StepWalk).
//   * Code lookup: decode is one LDS read; encode is one LDS byte read (bucket index
//     from the binary32 bits) plus one LDS threshold read and a compare.
// Floating point: compiled with -ffp-contract=off; '/' and sqrtf are the correctly
// rounded IEEE operations (HIP's default), fp32 denormals are kept.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "qopt.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                       // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kSlices = QOPT_BLOCK / (kWave * 4);  // 8 slices of 4 elements per lane
constexpr int kMaxTensors = 48;                 // tensors per launch (kernarg budget)
// Where the step keeps a block's second moments until the block maximum is known.
// With fp32 parameters a lane holds its 32 m and 32 v values plus the prefetched
// inputs of the next block in registers: 218-246 VGPRs, 2 waves per SIMD.  With
// bf16 parameters the inputs are smaller and v waits in the wave's own 8 KB of LDS
// instead (written slice by slice after its last use in the update, read back slice
// by slice when encoding), which brings the kernel under 168 VGPRs: 3 waves per
// SIMD, with three 4-wave workgroups (51 KB of LDS each) per CU.
template <typename PT> struct StepShape {
  static constexpr bool kVInLds = false;
  static constexpr int kWavesPerSimd = 2;
};
template <> struct StepShape<uint16_t> {
  static constexpr bool kVInLds = true;
  static constexpr int kWavesPerSimd = 3;
};
// The step's waves walk runs of this many consecutive blocks (run r belongs to wave
// r mod waves) rather than single blocks with a grid stride, so each wave's streams
// are contiguous over the run.  Measured on the Llama-7B set: runs of two 1.1-1.8 %
// faster than single blocks; where the step rolls its loads (step_rolls) runs of four
// are 1.6 % faster than two (one 3.8 % slower, eight 2.4 % slower).
constexpr uint32_t kStepRun = 2;
constexpr uint32_t kStepRunRolled = 4;
constexpr int kRows = static_cast<int>(sizeof(qopt_codebook) / 16);
static_assert(kSlices * kWave * 4 == QOPT_BLOCK, "block layout");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache policy per stream, chosen by measurement on MI355X (each choice compared
// with the others in one process, on the same buffers): the wide streams
// (parameters, gradients, codec values) go non-temporal, and so do the step's
// one-byte code streams; the codec's code streams use ordinary cached accesses
// (non-temporal ones measured 5-17 % slower there, while the step gains about 0.5 %).
#ifndef QOPT_NT_WIDE_LOAD
#define QOPT_NT_WIDE_LOAD 1
#endif
#ifndef QOPT_NT_WIDE_STORE
#define QOPT_NT_WIDE_STORE 1
#endif
#ifndef QOPT_NT_STEP_CODES
#define QOPT_NT_STEP_CODES 1
#endif
#ifndef QOPT_NT_CODEC_CODES
#define QOPT_NT_CODEC_CODES 0
#endif

template <bool kNt, typename T>
__device__ __forceinline__ T ld_policy(const T* p) {
  if constexpr (kNt) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool kNt, typename T>
__device__ __forceinline__ void st_policy(T* p, T v) {
  if constexpr (kNt) __builtin_nontemporal_store(v, p);
  else *p = v;
}
template <typename T> __device__ __forceinline__ T ld_wide(const T* p) {
  return ld_policy<QOPT_NT_WIDE_LOAD != 0>(p);
}
template <typename T> __device__ __forceinline__ void st_wide(T* p, T v) {
  st_policy<QOPT_NT_WIDE_STORE != 0>(p, v);
}
template <typename T> __device__ __forceinline__ T ld_step_code(const T* p) {
  return ld_policy<QOPT_NT_STEP_CODES != 0>(p);
}
template <typename T> __device__ __forceinline__ void st_step_code(T* p, T v) {
  st_policy<QOPT_NT_STEP_CODES != 0>(p, v);
}
template <typename T> __device__ __forceinline__ T ld_codec_code(const T* p) {
  return ld_policy<QOPT_NT_CODEC_CODES != 0>(p);
}
template <typename T> __device__ __forceinline__ void st_codec_code(T* p, T v) {
  st_policy<QOPT_NT_CODEC_CODES != 0>(p, v);
}

// ------------------------------------------------------------------ helpers


__device__ __forceinline__ void stage_codebook(qopt_codebook* dst, const qopt_codebook* src) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int i = threadIdx.x; i < kRows; i += kThreads) d[i] = s[i];
}

// Maximum over the wave of the bit patterns of non-negative floats (magnitudes or
// second moments), as a float, returned to every lane.  For non-negative binary32
// values the order of the bit patterns as unsigned integers is the order of the
// values, and every NaN pattern lies above +inf, so a NaN anywhere in the block makes
// its maximum a NaN, as a maximum over the values that propagates NaN would.  Four
// DPP steps inside each row of 16 lanes (swap neighbours, swap pairs, mirror the half
// rows, mirror the rows), two row broadcasts that carry the row maxima up to lane 63,
// then one read of lane 63 into a scalar register.  No LDS traffic and no waits on it,
// unlike a shuffle-based butterfly.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_max(uint32_t u) {
  // lanes of rows outside kRowMask read 0 (the `old` value), which leaves u unchanged
  return umax(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                     0, static_cast<int>(u), kCtrl, kRowMask, 0xF, false)));
}
__device__ __forceinline__ float wave_max_bits(uint32_t u) {
  u = dpp_max<0xB1, 0xF>(u);   // quad_perm [1,0,3,2]
  u = dpp_max<0x4E, 0xF>(u);   // quad_perm [2,3,0,1]
  u = dpp_max<0x141, 0xF>(u);  // row_half_mirror
  u = dpp_max<0x140, 0xF>(u);  // row_mirror
  u = dpp_max<0x142, 0xA>(u);  // row_bcast:15 into rows 1 and 3
  u = dpp_max<0x143, 0xC>(u);  // row_bcast:31 into rows 2 and 3
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 63)));
}

// Maximum that propagates NaN (v_maximum3_f32 on gfx950, which also folds absolute
// values and a third operand): a block with a NaN in it has a NaN maximum.
__device__ __forceinline__ float max_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950; it
// matches integer nearest-even rounding on every non-NaN binary32 input).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Per-codebook encoder parameters kept in registers for the whole kernel.
struct Encoder {
  const qopt_codebook* cb;  // LDS copy
  uint32_t key0;
  uint32_t last_bucket;
};

__device__ __forceinline__ Encoder make_encoder(const qopt_codebook* lds_cb) {
  Encoder e;
  e.cb = lds_cb;
  e.key0 = lds_cb->key0;
  uint32_t nb = lds_cb->nbuckets;
  nb = nb < 1u ? 1u : (nb > QOPT_MAX_BUCKETS ? QOPT_MAX_BUCKETS : nb);
  e.last_bucket = nb - 1;
  return e;
}

// Magnitude index of a >= 0: bucket start index, plus one if a reaches the single
// threshold that may lie inside the bucket.  The bucket index saturates at 0 below
// bucket 0 and is clamped to the last bucket above it, so every index stays inside
// the tables for any input and any table contents (bucket bytes <= 255, thresh has
// >= 257 entries).
__device__ __forceinline__ uint32_t encode_mag(const Encoder& e, float a) {
  uint32_t i = __builtin_elementwise_sub_sat(__float_as_uint(a) >> 15, e.key0);
  i = i < e.last_bucket ? i : e.last_bucket;
  const uint32_t b = e.cb->bucket[i];
  return b + (a >= e.cb->thresh[b + 1] ? 1u : 0u);
}

// Per-block normalisation: reciprocal, stored absmax and effective sign mask (all
// wave-uniform, held in scalar registers), and whether the block is stored as zero.
struct BlockScale {
  float r;
  float absmax;
  uint32_t sign_mask;
  uint32_t zero;
};

// Zero and subnormal blocks, and blocks whose maximum is NaN, store absmax 0 and
// every code 0.  The kernels branch on `zero` once per block (a scalar branch), so
// the encoder of ordinary blocks carries no test for it.
__device__ __forceinline__ BlockScale block_scale(float amax, uint32_t sign_mask) {
  BlockScale s;
  const bool ok = amax >= FLT_MIN;
  s.r = ok ? 1.0f / amax : 0.0f;
  s.absmax = ok ? amax : 0.0f;
  s.sign_mask = ok ? sign_mask : 0u;
  s.zero = ok ? 0u : 1u;
  return s;
}

// The sign bit is added to the bucket start before the threshold test's carry, so
// the compare feeds one add-with-carry.  This equals (magnitude index | sign bit):
// the magnitude index of a signed table is at most 127 and the sign mask is 0x80,
// or the mask is 0 (an unsigned table, or a zero block).
__device__ __forceinline__ uint32_t encode_signed(const Encoder& e, const BlockScale& s, float x) {
  const float a = fabsf(x) * s.r;
  uint32_t i = __builtin_elementwise_sub_sat(__float_as_uint(a) >> 15, e.key0);
  i = i < e.last_bucket ? i : e.last_bucket;
  const uint32_t b = e.cb->bucket[i];
  const uint32_t sign = x < 0.0f ? s.sign_mask : 0u;
  return (b + sign) + (a >= e.cb->thresh[b + 1] ? 1u : 0u);
}

// Second moments are sums of non-negative terms, so no sign bit is ever set.
__device__ __forceinline__ uint32_t encode_nonneg(const Encoder& e, const BlockScale& s, float x) {
  return encode_mag(e, x * s.r);
}

// ---------------------------------------------------------- codec kernels

// Index of the last piece whose first block is <= blk, by a fixed six-step search
// (kMaxTensors <= 64) written without a loop: a loop here, inside the kernels' block
// loops, measurably slows them even when it rarely runs.
static_assert(kMaxTensors <= 64, "piece search depth");
__device__ __forceinline__ uint32_t piece_of(const uint32_t* block_start, uint32_t npieces,
                                             uint32_t blk) {
  uint32_t t = 0;
#pragma unroll
  for (uint32_t s = 32; s > 0; s >>= 1) {
    const uint32_t probe = t + s;
    if (probe < npieces && block_start[probe] <= blk) t = probe;
  }
  return t;
}

// One codec launch's work: up to kMaxTensors pieces, each a run of whole blocks of
// one tensor (the same plan as the step's, see plan_chunks).
struct CodecChunk {
  float* vals[kMaxTensors];               // quantize: input; dequantize: output
  uint8_t* codes[kMaxTensors];
  float* absmax[kMaxTensors];
  int64_t n[kMaxTensors];
  uint32_t block_lo[kMaxTensors];
  uint32_t block_start[kMaxTensors + 1];
  uint32_t npieces;
  uint64_t vector_ok;                     // bit i: piece i may use the vector path
};

// The piece a wave is working in, held in scalar registers: consecutive blocks of a
// wave usually fall in the same piece, so the piece table is only searched again
// when the grid stride leaves it.
struct CodecPiece {
  float* vals;
  uint8_t* codes;
  float* absmax;
  int64_t n;
  uint32_t begin, end;  // launch-wide block range of the piece
  uint32_t lo;          // the piece's first block within its tensor
  uint32_t vec_ok;
};

__device__ __forceinline__ CodecPiece find_piece(const CodecChunk& c, uint32_t blk) {
  const uint32_t lo = piece_of(c.block_start, c.npieces, blk);
  CodecPiece pc;
  pc.vals = c.vals[lo];
  pc.codes = c.codes[lo];
  pc.absmax = c.absmax[lo];
  pc.n = c.n[lo];
  pc.begin = c.block_start[lo];
  pc.end = c.block_start[lo + 1];
  pc.lo = c.block_lo[lo];
  pc.vec_ok = static_cast<uint32_t>((c.vector_ok >> lo) & 1u);
  return pc;
}

struct CodecRef {
  float* vals;
  uint8_t* codes;
  float* absmax;  // this block's entry
  int64_t base;
  int len;
  uint32_t vec;
};

__device__ __forceinline__ CodecRef block_of(const CodecPiece& pc, uint32_t blk) {
  const uint32_t lb = pc.lo + (blk - pc.begin);
  CodecRef r;
  r.vals = pc.vals;
  r.codes = pc.codes;
  r.absmax = pc.absmax + lb;
  r.base = static_cast<int64_t>(lb) * QOPT_BLOCK;
  const int64_t rem = pc.n - r.base;
  r.len = rem < QOPT_BLOCK ? static_cast<int>(rem) : QOPT_BLOCK;
  r.vec = (r.len == QOPT_BLOCK && pc.vec_ok) ? 1u : 0u;
  return r;
}

// Quantize: each wave walks blocks with a grid stride and keeps the loads of its next
// two blocks in flight (two register sets in turn) while it encodes the current one:
// the block maximum needs the whole block before any code, so a deeper prefetch keeps
// more bytes in flight per wave.
__global__ void __launch_bounds__(kThreads)
quantize_kernel(CodecChunk c, const qopt_codebook* cb_g) {
  __shared__ __align__(16) qopt_codebook cb;
  stage_codebook(&cb, cb_g);
  __syncthreads();
  const Encoder enc = make_encoder(&cb);
  const uint32_t sign_mask = cb.sign_mask;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t stride = gridDim.x * kWaves;
  const uint32_t total = c.block_start[c.npieces];

  uint32_t blk = blockIdx.x * kWaves + wave;
  if (blk >= total) return;
  auto load_vec = [&](const CodecRef& r, f32x4 X[kSlices]) {
    const f32x4* src = reinterpret_cast<const f32x4*>(r.vals + r.base);
#pragma unroll
    for (int s = 0; s < kSlices; ++s) X[s] = ld_wide(src + s * kWave + lane);
  };
  auto process = [&](const CodecRef& cur, const f32x4 X[kSlices]) {
    float x[kSlices][4];
    if (cur.vec) {
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        x[s][0] = X[s].x; x[s][1] = X[s].y; x[s][2] = X[s].z; x[s][3] = X[s].w;
      }
    } else {
#pragma unroll
      for (int s = 0; s < kSlices; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = s * 256 + lane * 4 + j;
          x[s][j] = e < cur.len ? cur.vals[cur.base + e] : 0.0f;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < kSlices; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = max_nan(amax, fabsf(x[s][j]));
    const BlockScale sc = block_scale(wave_max_bits(__float_as_uint(amax)), sign_mask);
    if (cur.vec) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(cur.codes + cur.base);
      if (sc.zero) {
#pragma unroll
        for (int s = 0; s < kSlices; ++s) st_codec_code(dst + s * kWave + lane, 0u);
      } else {
#pragma unroll
        for (int s = 0; s < kSlices; ++s) {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) w |= encode_signed(enc, sc, x[s][j]) << (8 * j);
          st_codec_code(dst + s * kWave + lane, w);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < kSlices; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = s * 256 + lane * 4 + j;
          if (e < cur.len)
            cur.codes[cur.base + e] =
                sc.zero ? 0 : static_cast<uint8_t>(encode_signed(enc, sc, x[s][j]));
        }
    }
    if (lane == 0) *cur.absmax = sc.absmax;
  };
  CodecPiece piece = find_piece(c, blk);
  auto ref_at = [&](uint32_t b) {
    if (b < piece.begin || b >= piece.end) piece = find_piece(c, b);
    return block_of(piece, b);
  };
  // A and B take turns: a block is encoded from one set while the other set's loads
  // and the loads issued right after its own encoding (the block two strides on) are
  // in flight.  Launches hold at most 2^18 blocks, so the indices cannot wrap.
  f32x4 A[kSlices], B[kSlices];
  CodecRef ra = ref_at(blk);
  if (ra.vec) load_vec(ra, A);
  uint32_t bb = blk + stride;
  CodecRef rb = ra;
  if (bb < total) {
    rb = ref_at(bb);
    if (rb.vec) load_vec(rb, B);
  }
  for (;;) {
    process(ra, A);
    if (bb >= total) break;
    const uint32_t na = bb + stride;
    if (na < total) {
      ra = ref_at(na);
      if (ra.vec) load_vec(ra, A);
    }
    process(rb, B);
    if (na >= total) break;
    bb = na + stride;
    if (bb < total) {
      rb = ref_at(bb);
      if (rb.vec) load_vec(rb, B);
    }
  }
}

__global__ void __launch_bounds__(kThreads)
dequantize_kernel(CodecChunk c, const qopt_codebook* cb_g) {
  __shared__ __align__(16) qopt_codebook cb;
  stage_codebook(&cb, cb_g);
  __syncthreads();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t stride = gridDim.x * kWaves;
  const uint32_t total = c.block_start[c.npieces];

  uint32_t blk = blockIdx.x * kWaves + wave;
  if (blk >= total) return;
  CodecPiece piece = find_piece(c, blk);
  for (; blk < total; blk += stride) {
    if (blk >= piece.end) piece = find_piece(c, blk);
    const CodecRef r = block_of(piece, blk);
    const float A = *r.absmax;
    if (r.vec) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(r.codes + r.base);
      f32x4* dst = reinterpret_cast<f32x4*>(r.vals + r.base);
      uint32_t w[kSlices];
#pragma unroll
      for (int s = 0; s < kSlices; ++s) w[s] = ld_codec_code(src + s * kWave + lane);
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        f32x4 v;
        v.x = cb.decode[w[s] & 0xFFu] * A;
        v.y = cb.decode[(w[s] >> 8) & 0xFFu] * A;
        v.z = cb.decode[(w[s] >> 16) & 0xFFu] * A;
        v.w = cb.decode[w[s] >> 24] * A;
        st_wide(dst + s * kWave + lane, v);
      }
    } else {
#pragma unroll
      for (int s = 0; s < kSlices; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = s * 256 + lane * 4 + j;
          if (e < r.len) r.vals[r.base + e] = cb.decode[r.codes[r.base + e]] * A;
        }
    }
  }
}

// ------------------------------------------------------------ Adam kernel

struct AdamScalars {
  float b1, b2, omb1, omb2, eps, step_size, inv_sqrt_bc2;
  // the screened short path for bf16 parameters: its denominator is
  // sqrt(v) * short_a + short_b = (sqrt(v) * inv_sqrt_bc2 + eps) / step_size, so that
  // t = m / denominator; it is taken only where |t| < t_limit
  float short_a, short_b, t_limit;
};

// How bf16 parameters use the screened short path (fp32 parameters never do):
// not at all, or screened, or screened with slices holding a subnormal second
// moment sent to the correctly rounded sequence as well.
enum ScreenMode : int { kNoScreen = 0, kScreen = 1, kScreenSubCheck = 2 };

// Register budget per instantiation: the bf16 kernels of the two rare modes (the
// screen off, or with its subnormal test) need a few more registers than three waves
// per SIMD allow, and run at two waves per SIMD rather than spill.
template <typename PT, int kMode> constexpr int step_waves() {
  return (std::is_same<PT, uint16_t>::value && kMode != kScreen) ? 2
                                                                  : StepShape<PT>::kWavesPerSimd;
}

// Whether the step loads its next block slice by slice while it updates the current
// one (each slice of the next block goes in flight as soon as the same slice of the
// current block is used up), rather than all at once after the update.  The loads are
// then in flight through the whole update as well as the requantization.  It needs
// the registers of two blocks' worth of live inputs in the middle of the update:
// fp32 parameters with bf16 gradients fit at two waves per SIMD (measured 2.3 %
// faster on the Llama-7B set); fp32 gradients would spill, and bf16 parameters need
// their third wave per SIMD more (at two waves with rolling the 20B step ran 7 %
// slower).
template <typename PT, typename GT> constexpr bool step_rolls() {
  return std::is_same<PT, float>::value && std::is_same<GT, uint16_t>::value;
}
template <typename PT, typename GT> constexpr uint32_t step_run() {
  return step_rolls<PT, GT>() ? kStepRunRolled : kStepRun;
}

// The blocks one wave of the step takes, in order: runs of kRun consecutive blocks,
// run r on wave r mod (number of waves), over the largest prefix of the launch in
// which every wave gets the same number of runs; then the remaining blocks one at a
// time, block full + j on wave j mod (number of waves).  Every block is taken exactly
// once, and the launch's last round no longer leaves some waves a whole run behind the
// others.  (All wave-uniform, in scalar registers.)
template <uint32_t kRun> struct StepWalk {
  uint32_t full;     // blocks in whole rounds of runs
  uint32_t stride;   // waves in the grid
  uint32_t wave_id;  // this wave's index in the grid
  __device__ StepWalk(uint32_t total, uint32_t waves, uint32_t id) : stride(waves), wave_id(id) {
    const uint64_t round = static_cast<uint64_t>(waves) * kRun;
    full = static_cast<uint32_t>(total / round * round);
  }
  __device__ uint32_t first() const {
    const uint64_t b = static_cast<uint64_t>(wave_id) * kRun;
    return b < full ? static_cast<uint32_t>(b) : full + wave_id;
  }
  // the block after b, or a value >= every launch's block count (2^32 - 1 at most)
  __device__ uint32_t next(uint32_t b) const {
    uint64_t nb;
    if (b < full) {
      nb = ((b + 1) % kRun) ? uint64_t{b} + 1 : (uint64_t{b / kRun} + stride) * kRun;
      if (nb >= full) nb = uint64_t{full} + wave_id;
    } else {
      nb = uint64_t{b} + stride;
    }
    return nb > 0xFFFFFFFFu ? 0xFFFFFFFFu : static_cast<uint32_t>(nb);
  }
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

// Element types as they sit in memory: fp32, or bf16 bit patterns (uint16_t).
// Four consecutive elements are one vector access: 16 bytes of fp32, 8 of bf16.
template <typename T> struct Vec4T;
template <> struct Vec4T<float> { typedef f32x4 type; };
template <> struct Vec4T<uint16_t> { typedef u32x2 type; };

__device__ __forceinline__ void unpack4(const f32x4& v, float o[4]) {
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void unpack4(const u32x2& v, float o[4]) {
  o[0] = bf16_to_f32(v.x & 0xFFFFu); o[1] = bf16_to_f32(v.x >> 16);
  o[2] = bf16_to_f32(v.y & 0xFFFFu); o[3] = bf16_to_f32(v.y >> 16);
}
__device__ __forceinline__ void pack4(const float in[4], f32x4& v) {
  v.x = in[0]; v.y = in[1]; v.z = in[2]; v.w = in[3];
}
__device__ __forceinline__ void pack4(const float in[4], u32x2& v) {
  v.x = pack_bf16x2(in[0], in[1]);
  v.y = pack_bf16x2(in[2], in[3]);
}

template <typename T> __device__ __forceinline__ float load1(const T* p, int i);
template <> __device__ __forceinline__ float load1<float>(const float* p, int i) { return p[i]; }
template <> __device__ __forceinline__ float load1<uint16_t>(const uint16_t* p, int i) {
  return bf16_to_f32(p[i]);
}
template <typename T> __device__ __forceinline__ void store1(T* p, int i, float x);
template <> __device__ __forceinline__ void store1<float>(float* p, int i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void store1<uint16_t>(uint16_t* p, int i, float x) {
  p[i] = static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// One element of the update; returns the new parameter, leaves m and v.
__device__ __forceinline__ float adam_element(const AdamScalars& k, float p, float g, float m_prev,
                                              float v_prev, float& m, float& v) {
  m = (k.b1 * m_prev) + (k.omb1 * g);
  v = (k.b2 * v_prev) + (k.omb2 * (g * g));
  const float denom = (sqrtf(v) * k.inv_sqrt_bc2) + k.eps;
  const float u = m / denom;
  return p - (k.step_size * u);
}

// Correctly rounded square root for x in {+0} U [2^-96, +inf]: the hardware estimate
// is within one ulp, and a residual test against each neighbour picks the nearest
// binary32.  This is sqrtf's own refinement without its rescaling of tiny inputs and
// its special-case select, which are not needed on that range (checked bit for bit
// against sqrtf on every binary32 in it).
__device__ __forceinline__ float sqrt_rn_unscaled(float x) {
  const float s = __builtin_amdgcn_sqrtf(x);
  const float s_dn = __uint_as_float(__float_as_uint(s) - 1u);
  const float s_up = __uint_as_float(__float_as_uint(s) + 1u);
  const float r_dn = __builtin_fmaf(-s_dn, s, x);
  const float r_up = __builtin_fmaf(-s_up, s, x);
  float r = (r_dn <= 0.0f) ? s_dn : s;
  r = (r_up > 0.0f) ? s_up : r;
  return r;
}

constexpr float kTinyMoment = 0x1p-96f;  // below this, sqrt_rn_unscaled is not exact

// Screen for the bf16 short path.  There t = m * rcp(fma(sq, a, b)) with sq the
// hardware square root of a normal or zero v and a, b the step's scalars folded as
// in AdamScalars.  The hardware square root and reciprocal are each within one ulp
// on those inputs (every normal square-root input, and every normal reciprocal input
// up to 2^126, was checked on the hardware; subnormal square-root inputs flush to
// zero, so they never reach this path).  In units of 2^-24, t is then within 7 of
// the exact m / ((sqrt(v) inv_sqrt_bc2 + eps) / step_size) (square root 2, a 1, the
// fma 1, reciprocal 2, product 1; b's 1 does not add), and the correctly rounded
// sequence's t within 5 of it: they differ by under |t| 2^-20.3.  After both sides
// round p - t to binary32 the sequence's result lies within |t| 2^-20.3 + |pf| 2^-23
// of pf (plus 2^-149 where results are subnormal).  c takes 2^-19 and 2^-22 for the
// two factors (2.5 and 2 times the bound) and adds 2^-126; the sequence's result
// then lies in [pf - c, pf + c], and rounding fp32 -> bf16 is monotone, so if both
// ends give the same bf16 bits so do that result and pf.
__device__ __forceinline__ float screen_width(float pf, float t) {
  return __builtin_fmaf(fabsf(t), 0x1p-19f, __builtin_fmaf(fabsf(pf), 0x1p-22f, 0x1p-126f));
}
// Two elements at once: true where the bf16 bits of the lower ends differ from
// those of the upper ends.  An infinite pf makes one end NaN and the other
// infinite, which differ; a NaN t is caught by the bound on |t| that goes with this
// screen (see update_vec).
__device__ __forceinline__ bool screen_fails_bf16x2(float pf0, float t0, float pf1, float t1) {
  const float c0 = screen_width(pf0, t0);
  const float c1 = screen_width(pf1, t1);
  const uint32_t lo = pack_bf16x2(pf0 - c0, pf1 - c1);
  const uint32_t hi = pack_bf16x2(pf0 + c0, pf1 + c1);
  return lo != hi;
}

// Positive subnormal, as a __builtin_amdgcn_classf mask.
constexpr int kClassPosSubnormal = 0x80;

// Where one block lives, resolved from the launch's piece table (wave-uniform).
struct BlockRef {
  void* param;
  const void* grad;
  uint8_t* cm;
  uint8_t* cv;
  float* am;
  float* av;
  int64_t base;  // first element of the block within its tensor
  int len;       // elements in the block (2048 except a tensor's last block)
  uint32_t vec;  // full block of a tensor whose pointers allow vector accesses
  // (no bool and no tail padding here or in the other loop-carried descriptors:
  // copying padding bytes keeps a private object alive that the compiler then
  // moves to LDS, adding LDS traffic to the block loop)
};

__device__ __forceinline__ BlockRef resolve(const StepChunk& c, uint32_t blk) {
  const uint32_t t = piece_of(c.block_start, c.npieces, blk);
  const uint32_t lb = c.block_lo[t] + (blk - c.block_start[t]);
  BlockRef r;
  r.param = c.param[t];
  r.grad = c.grad[t];
  r.cm = c.m_codes[t];
  r.cv = c.v_codes[t];
  r.am = c.m_absmax[t] + lb;
  r.av = c.v_absmax[t] + lb;
  r.base = static_cast<int64_t>(lb) * QOPT_BLOCK;
  const int64_t rem = c.n[t] - r.base;
  r.len = rem < QOPT_BLOCK ? static_cast<int>(rem) : QOPT_BLOCK;
  r.vec = (r.len == QOPT_BLOCK && ((c.vector_ok >> t) & 1u)) ? 1u : 0u;
  return r;
}

// One lane's vector inputs of one full block: slice s holds elements
// s*256 + 4*lane .. +3.
template <typename PT, typename GT>
struct BlockIn {
  typename Vec4T<PT>::type p[kSlices];
  typename Vec4T<GT>::type g[kSlices];
  uint32_t cm[kSlices];
  uint32_t cv[kSlices];
  float am, av;
};

// The lane index as a value the compiler cannot see through.  Address arithmetic
// derived from it is then redone for each block (a few cheap ops) instead of being
// hoisted out of the block loop, where at three waves per SIMD it would be spilled
// to scratch and reloaded behind a wait for every outstanding load.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

template <typename PT, typename GT>
__device__ __forceinline__ void load_block(BlockIn<PT, GT>& in, const BlockRef& r, int lane) {
  typedef typename Vec4T<PT>::type PV;
  typedef typename Vec4T<GT>::type GV;
  const int l = opaque_lane(lane);
  const PV* p = reinterpret_cast<const PV*>(static_cast<const PT*>(r.param) + r.base) + l;
  const GV* g = reinterpret_cast<const GV*>(static_cast<const GT*>(r.grad) + r.base) + l;
  const uint32_t* cm = reinterpret_cast<const uint32_t*>(r.cm + r.base) + l;
  const uint32_t* cv = reinterpret_cast<const uint32_t*>(r.cv + r.base) + l;
  // Where the block maxima are loaded, measured on the Llama-7B set (fp32 parameters,
  // bf16 gradients) and the 20B set (both bf16): after the streams is 0.8 % faster for
  // the first, before them 0.6 % faster for the second.
  constexpr bool kMaximaFirst =
      std::is_same<PT, uint16_t>::value && std::is_same<GT, uint16_t>::value;
  if constexpr (kMaximaFirst) {
    in.am = *r.am;
    in.av = *r.av;
  }
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    in.p[s] = ld_wide(p + s * kWave);
    in.g[s] = ld_wide(g + s * kWave);
    in.cm[s] = ld_step_code(cm + s * kWave);
    in.cv[s] = ld_step_code(cv + s * kWave);
  }
  if constexpr (!kMaximaFirst) {
    in.am = *r.am;
    in.av = *r.av;
  }
}

// Slice s of a full block's vector inputs (the streams; the block maxima are loaded
// apart).
template <typename PT, typename GT>
__device__ __forceinline__ void load_slice(BlockIn<PT, GT>& in, const BlockRef& r, int lane, int s) {
  typedef typename Vec4T<PT>::type PV;
  typedef typename Vec4T<GT>::type GV;
  const int l = opaque_lane(lane);
  const PV* p = reinterpret_cast<const PV*>(static_cast<const PT*>(r.param) + r.base) + l;
  const GV* g = reinterpret_cast<const GV*>(static_cast<const GT*>(r.grad) + r.base) + l;
  const uint32_t* cm = reinterpret_cast<const uint32_t*>(r.cm + r.base) + l;
  const uint32_t* cv = reinterpret_cast<const uint32_t*>(r.cv + r.base) + l;
  in.p[s] = ld_wide(p + s * kWave);
  in.g[s] = ld_wide(g + s * kWave);
  in.cm[s] = ld_step_code(cm + s * kWave);
  in.cv[s] = ld_step_code(cv + s * kWave);
}

// A wave's second-moment stash in LDS: slice s of lane l at 16 bytes per lane, so
// each slice is one conflict-free 128-bit access across the wave.
__device__ __forceinline__ void stash_v(float* vstash, int s, int lane, const float v4[4]) {
  const f32x4 t = {v4[0], v4[1], v4[2], v4[3]};
  reinterpret_cast<f32x4*>(vstash)[s * kWave + lane] = t;
}
__device__ __forceinline__ void unstash_v(const float* vstash, int s, int lane, float v4[4]) {
  const f32x4 t = reinterpret_cast<const f32x4*>(vstash)[s * kWave + lane];
  v4[0] = t.x; v4[1] = t.y; v4[2] = t.z; v4[3] = t.w;
}

// Update of a full block from prefetched vector inputs; stores p, keeps m and v
// (v in the LDS stash where StepShape says so).  Where the step rolls (step_rolls),
// slice s of block nr is loaded into `in` as soon as slice s of this block is used up.
template <typename PT, typename GT, int kMode>
__device__ __forceinline__ void update_vec(const AdamScalars& k, const qopt_codebook& cbm,
                                           const qopt_codebook& cbv, BlockIn<PT, GT>& in,
                                           const BlockRef& r, const BlockRef& nr, int lane,
                                           float m[kSlices][4], float v[kSlices][4], float* vstash,
                                           float& mmax, float& vmax) {
  typedef typename Vec4T<PT>::type PV;
  PV* pout = reinterpret_cast<PV*>(static_cast<PT*>(r.param) + r.base);
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    float p4[4], g4[4];
    unpack4(in.p[s], p4);
    unpack4(in.g[s], g4);
    constexpr bool kScreened = std::is_same<PT, uint16_t>::value && kMode != kNoScreen;
    // the moments of the slice's 4 elements; where the correctly rounded sequence
    // runs, its square roots skip sqrtf's rescaling of tiny inputs unless some lane of
    // the wave holds a tiny second moment
    uint64_t tiny = 0;  // lanes (as a wave mask) holding 0 < v < 2^-96
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float m_prev = cbm.decode[(in.cm[s] >> (8 * j)) & 0xFFu] * in.am;
      const float v_prev = cbv.decode[(in.cv[s] >> (8 * j)) & 0xFFu] * in.av;
      m[s][j] = (k.b1 * m_prev) + (k.omb1 * g4[j]);
      v[s][j] = (k.b2 * v_prev) + (k.omb2 * (g4[j] * g4[j]));
      // 0 < v < 2^-96 as one unsigned compare on the bits (v is never negative);
      // bf16 parameters take it only on their fallback below
      if constexpr (!kScreened)
        tiny |= __builtin_amdgcn_ballot_w64((__float_as_uint(v[s][j]) - 1u) <
                                            (__float_as_uint(kTinyMoment) - 1u));
    }
    bool exact = true;
    if constexpr (kScreened) {
      // bf16 parameters: the short path (hardware square root and reciprocal, each
      // within one ulp on the inputs that reach it) gives the same bf16 result as
      // the correctly rounded sequence whenever its fp32 result is far enough from
      // a bf16 rounding boundary; lanes where it is not fall back below.  The
      // hardware square root flushes subnormal second moments to zero; unless eps
      // makes that harmless (kMode kScreen), such slices fall back as well.
      uint64_t sub = 0;
      if constexpr (kMode == kScreenSubCheck)
        sub = __builtin_amdgcn_ballot_w64(__builtin_amdgcn_classf(v[s][0], kClassPosSubnormal) |
                                          __builtin_amdgcn_classf(v[s][1], kClassPosSubnormal) |
                                          __builtin_amdgcn_classf(v[s][2], kClassPosSubnormal) |
                                          __builtin_amdgcn_classf(v[s][3], kClassPosSubnormal));
      if (sub == 0) {
        float pf[4], t[4];
        // The short path never forms m / denominator, which the sequence rounds on
        // its own and which may overflow where t does not; where |t| < t_limit
        // (min(step_size, 1) 2^127) neither the sequence's quotient nor its t can
        // overflow.  A NaN t (0/0 with eps = 0) fails the compare too.
        uint64_t unbounded = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sq1 = __builtin_amdgcn_sqrtf(v[s][j]);
          const float denom = __builtin_fmaf(sq1, k.short_a, k.short_b);
          t[j] = m[s][j] * __builtin_amdgcn_rcpf(denom);
          pf[j] = p4[j] - t[j];
          unbounded |= __builtin_amdgcn_ballot_w64(!(fabsf(t[j]) < k.t_limit));
        }
        const uint64_t unsafe =
            unbounded | __builtin_amdgcn_ballot_w64(screen_fails_bf16x2(pf[0], t[0], pf[1], t[1])) |
            __builtin_amdgcn_ballot_w64(screen_fails_bf16x2(pf[2], t[2], pf[3], t[3]));
        if (unsafe == 0) {
          exact = false;
#pragma unroll
          for (int j = 0; j < 4; ++j) p4[j] = pf[j];
        }
      }
      if (exact) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          tiny |= __builtin_amdgcn_ballot_w64((__float_as_uint(v[s][j]) - 1u) <
                                              (__float_as_uint(kTinyMoment) - 1u));
      }
    }
    if (exact) {
      float sq[4];
      if (tiny != 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sq[j] = sqrtf(v[s][j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) sq[j] = sqrt_rn_unscaled(v[s][j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float denom = (sq[j] * k.inv_sqrt_bc2) + k.eps;
        const float u = m[s][j] / denom;
        p4[j] = p4[j] - (k.step_size * u);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mmax = max_nan(mmax, fabsf(m[s][j]));
      vmax = max_nan(vmax, v[s][j]);
    }
    if constexpr (StepShape<PT>::kVInLds) stash_v(vstash, s, lane, v[s]);
    PV pv;
    pack4(p4, pv);
    st_wide(pout + s * kWave + lane, pv);
    if constexpr (step_rolls<PT, GT>()) load_slice(in, nr, lane, s);
  }
}

// Update of a short block, or of a tensor without vector alignment: element-wise
// accesses guarded by the block length; elements past it hold m = v = 0.
template <typename PT, typename GT>
__device__ __forceinline__ void update_scalar(const AdamScalars& k, const qopt_codebook& cbm,
                                              const qopt_codebook& cbv, const BlockRef& r,
                                              int lane, float m[kSlices][4], float v[kSlices][4],
                                              float* vstash, float& mmax, float& vmax) {
  const float Am = *r.am;
  const float Av = *r.av;
  // the block's own base pointers, so that element offsets stay 32-bit
  PT* pb = static_cast<PT*>(r.param) + r.base;
  const GT* gb = static_cast<const GT*>(r.grad) + r.base;
  const uint8_t* cmb = r.cm + r.base;
  const uint8_t* cvb = r.cv + r.base;
#pragma unroll
  for (int s = 0; s < kSlices; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = s * 256 + lane * 4 + j;
      m[s][j] = 0.0f;
      v[s][j] = 0.0f;
      if (e < r.len) {
        const float m_prev = cbm.decode[cmb[e]] * Am;
        const float v_prev = cbv.decode[cvb[e]] * Av;
        const float p = adam_element(k, load1<PT>(pb, e), load1<GT>(gb, e), m_prev, v_prev,
                                     m[s][j], v[s][j]);
        store1<PT>(pb, e, p);
        mmax = max_nan(mmax, fabsf(m[s][j]));
        vmax = max_nan(vmax, v[s][j]);
      }
    }
  if constexpr (StepShape<PT>::kVInLds) {
#pragma unroll
    for (int s = 0; s < kSlices; ++s) stash_v(vstash, s, lane, v[s]);
  }
}

// The codes of one block's m and v (kMasked: ANDed with per-moment masks that zero a
// moment whose block is stored as zero).
template <bool kVInLds, bool kMasked>
__device__ __forceinline__ void encode_block(const Encoder& em, const Encoder& ev,
                                             const BlockScale& sm, const BlockScale& sv,
                                             const BlockRef& r, int lane,
                                             const float m[kSlices][4], const float v[kSlices][4],
                                             const float* vstash) {
  const uint32_t keep_m = sm.zero ? 0u : 0xFFFFFFFFu;
  const uint32_t keep_v = sv.zero ? 0u : 0xFFFFFFFFu;
  uint32_t* cmo = reinterpret_cast<uint32_t*>(r.cm + r.base);
  uint32_t* cvo = reinterpret_cast<uint32_t*>(r.cv + r.base);
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    float vs[4] = {v[s][0], v[s][1], v[s][2], v[s][3]};
    if constexpr (kVInLds) unstash_v(vstash, s, lane, vs);
    uint32_t wm = 0, wv = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wm |= encode_signed(em, sm, m[s][j]) << (8 * j);
      wv |= encode_nonneg(ev, sv, vs[j]) << (8 * j);
    }
    if constexpr (kMasked) {
      wm &= keep_m;
      wv &= keep_v;
    }
    if (r.vec) {
      st_step_code(cmo + s * kWave + lane, wm);
      st_step_code(cvo + s * kWave + lane, wv);
    } else {
      uint8_t* cmb = r.cm + r.base;
      uint8_t* cvb = r.cv + r.base;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = s * 256 + lane * 4 + j;
        if (e < r.len) {
          cmb[e] = static_cast<uint8_t>(wm >> (8 * j));
          cvb[e] = static_cast<uint8_t>(wv >> (8 * j));
        }
      }
    }
  }
}

// Block maxima across the wave, then the codes of m and v and the new maxima.  A
// moment whose block maximum is not normal (rare: zero, subnormal or NaN) keeps its
// codes at 0; such blocks take a copy of the encoder of their own, so that ordinary
// blocks pay nothing for it.
template <bool kVInLds>
__device__ __forceinline__ void requantize(const Encoder& em, const Encoder& ev, uint32_t sign_m,
                                           uint32_t sign_v, const BlockRef& r, int lane,
                                           const float m[kSlices][4], const float v[kSlices][4],
                                           const float* vstash, float mmax, float vmax) {
  const BlockScale sm = block_scale(wave_max_bits(__float_as_uint(mmax)), sign_m);
  const BlockScale sv = block_scale(wave_max_bits(__float_as_uint(vmax)), sign_v);
  if ((sm.zero | sv.zero) == 0)
    encode_block<kVInLds, false>(em, ev, sm, sv, r, lane, m, v, vstash);
  else
    encode_block<kVInLds, true>(em, ev, sm, sv, r, lane, m, v, vstash);
  if (lane == 0) {
    *r.am = sm.absmax;
    *r.av = sv.absmax;
  }
}

// Each wave walks its blocks in StepWalk's order (runs of step_run() consecutive
// blocks, then single blocks for the launch's remainder).  While it requantizes one
// block, the vector inputs of its next block are already in flight: loaded into the
// registers the update no longer needs, slice by slice during the update where the
// step rolls (step_rolls), else all at once after it.
template <typename PT, typename GT, int kMode>
__global__ void __launch_bounds__(kThreads, (step_waves<PT, kMode>()))
adam8bit_kernel(StepChunk c, AdamScalars k, const qopt_codebook* cbm_g, const qopt_codebook* cbv_g) {
  constexpr bool kVInLds = StepShape<PT>::kVInLds;
  __shared__ __align__(16) qopt_codebook cb[2];
  __shared__ __align__(16) float vstash_all[kVInLds ? kWaves * QOPT_BLOCK : 4];
  stage_codebook(&cb[0], cbm_g);
  stage_codebook(&cb[1], cbv_g);
  __syncthreads();
  const Encoder em = make_encoder(&cb[0]);
  const Encoder ev = make_encoder(&cb[1]);
  const uint32_t sign_m = cb[0].sign_mask;
  const uint32_t sign_v = cb[1].sign_mask;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t stride = gridDim.x * kWaves;
  const uint32_t total = c.block_start[c.npieces];
  float* vstash = kVInLds ? vstash_all + wave * QOPT_BLOCK : vstash_all;

  const StepWalk<step_run<PT, GT>()> walk(total, stride, blockIdx.x * kWaves + wave);
  uint32_t blk = walk.first();
  if (blk >= total) return;
  BlockRef cur = resolve(c, blk);
  BlockIn<PT, GT> in;
  if (cur.vec) load_block(in, cur, lane);
  for (;;) {
    float m[kSlices][4], v[kSlices][4];
    float mmax = 0.0f, vmax = 0.0f;
    const uint32_t nblk = walk.next(blk);
    const bool more = nblk < total;
    const BlockRef nxt = more ? resolve(c, nblk) : cur;
    const bool next_vec = more && nxt.vec;
    if (cur.vec) {
      // Rolling steps load the next block's streams during the update; without a next
      // vector block the wave reloads its own block's instead (discarded), so that the
      // update has one shape.
      update_vec<PT, GT, kMode>(k, cb[0], cb[1], in, cur, next_vec ? nxt : cur, lane, m, v, vstash,
                                mmax, vmax);
      if constexpr (step_rolls<PT, GT>()) {
        if (next_vec) {
          in.am = *nxt.am;
          in.av = *nxt.av;
        }
      } else {
        if (next_vec) load_block(in, nxt, lane);
      }
    } else {
      update_scalar<PT, GT>(k, cb[0], cb[1], cur, lane, m, v, vstash, mmax, vmax);
      if (next_vec) load_block(in, nxt, lane);
    }
    // The stash must really go through LDS: without this the compiler may forward
    // the stored values and keep all 32 of them live in registers.
    if constexpr (kVInLds) asm volatile("" ::: "memory");
    requantize<kVInLds>(em, ev, sign_m, sign_v, cur, lane, m, v, vstash, mmax, vmax);
    if (!more) break;
    blk = nblk;
    cur = nxt;
  }
}

// A measurement aid, not part of the method: the step's launch plan, grid, block
// order, prefetch and every load and store of its vector path, with no arithmetic.
// Each block's parameters, codes and block maxima are written back as read, and the
// gradients are read and dropped, so the state is unchanged.  Timed against the step
// on the same buffers it gives the ceiling of the step's access pattern.  Blocks
// that are not on the vector path are skipped.
template <typename PT, typename GT>
__global__ void __launch_bounds__(kThreads) step_traffic_kernel(StepChunk c) {
  typedef typename Vec4T<PT>::type PV;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t stride = gridDim.x * kWaves;
  const uint32_t total = c.block_start[c.npieces];
  const StepWalk<step_run<PT, GT>()> walk(total, stride, blockIdx.x * kWaves + wave);
  uint32_t blk = walk.first();
  if (blk >= total) return;
  BlockRef cur = resolve(c, blk);
  BlockIn<PT, GT> in;
  if (cur.vec) load_block(in, cur, lane);
  for (;;) {
    uint32_t cm[kSlices], cv[kSlices];
    float am = 0.0f, av = 0.0f;
    const uint32_t nblk = walk.next(blk);
    const bool more = nblk < total;
    const BlockRef nxt = more ? resolve(c, nblk) : cur;
    const bool next_vec = more && nxt.vec;
    if (cur.vec) {
      PV* pout = reinterpret_cast<PV*>(static_cast<PT*>(cur.param) + cur.base);
      const BlockRef nr = next_vec ? nxt : cur;
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        asm volatile("" ::"v"(in.g[s]));  // the gradient is waited for, as the step does
        st_wide(pout + s * kWave + lane, in.p[s]);
        cm[s] = in.cm[s];
        cv[s] = in.cv[s];
        if constexpr (step_rolls<PT, GT>()) load_slice(in, nr, lane, s);
      }
      am = in.am;
      av = in.av;
      if constexpr (step_rolls<PT, GT>()) {
        if (next_vec) {
          in.am = *nxt.am;
          in.av = *nxt.av;
        }
      } else {
        if (next_vec) load_block(in, nxt, lane);
      }
    } else if (next_vec) {
      load_block(in, nxt, lane);
    }
    if (cur.vec) {
      uint32_t* cmo = reinterpret_cast<uint32_t*>(cur.cm + cur.base);
      uint32_t* cvo = reinterpret_cast<uint32_t*>(cur.cv + cur.base);
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        st_step_code(cmo + s * kWave + lane, cm[s]);
        st_step_code(cvo + s * kWave + lane, cv[s]);
      }
      if (lane == 0) {
        *cur.am = am;
        *cur.av = av;
      }
    }
    if (!more) break;
    blk = nblk;
    cur = nxt;
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

// A second stream per device, created on first use and kept until the process ends
// (default priority, non-blocking), over which the bf16-parameter step spreads its
// launches (launch_planned).
std::once_flag g_side_once[kMaxDevices];
hipStream_t g_side[kMaxDevices];
int g_side_rc[kMaxDevices];

int side_stream(hipStream_t* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QOPT_ELAUNCH;
  std::call_once(g_side_once[dev], [dev] {
    g_side_rc[dev] = hipStreamCreateWithFlags(&g_side[dev], hipStreamNonBlocking) == hipSuccess
                         ? QOPT_OK
                         : QOPT_ELAUNCH;
  });
  if (g_side_rc[dev] != QOPT_OK) return g_side_rc[dev];
  *out = g_side[dev];
  return QOPT_OK;
}

// Persistent grid: enough workgroups to fill every CU at the kernel's occupancy
// (or at most cap per CU, if cap > 0), never more than there are blocks to hand out.
// Each wave of the kernel takes `run` consecutive blocks at a time.
template <typename K>
int grid_for(K kernel, uint32_t nblocks, int cap, uint32_t run, unsigned* grid) {
  int cus = 0;
  int rc = current_cus(&cus);
  if (rc != QOPT_OK) return rc;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
      per_cu <= 0)
    return QOPT_ELAUNCH;
  if (cap > 0 && per_cu > cap) per_cu = cap;
  const uint64_t resident = static_cast<uint64_t>(cus) * static_cast<uint64_t>(per_cu);
  const uint64_t per_wg = static_cast<uint64_t>(kWaves) * run;
  const uint64_t wanted = (static_cast<uint64_t>(nblocks) + per_wg - 1) / per_wg;
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

// Splits a list of tensors into launches of equal block counts (the last may be
// shorter), each holding at most kMaxTensors pieces; a piece is a run of whole blocks
// of one tensor.  For a given launch count the pieces are assigned greedily in
// tensor order.  size_of(i) gives tensor i's length; fill(chunk, slot, i) writes its
// pointers and length into the slot and says whether it may take the vector path;
// emit(chunk, blocks) is called once per launch.  Returns the first error.
template <typename Chunk, typename SizeOf, typename Fill, typename Emit>
int plan_chunks(int32_t ntensors, const SizeOf& size_of, const Fill& fill, uint64_t nchunks,
                uint64_t total, Emit&& emit, bool* fits) {
  const uint64_t target = (total + nchunks - 1) / nchunks;
  Chunk c;
  c.npieces = 0;
  c.vector_ok = 0;
  c.block_start[0] = 0;
  uint64_t blocks = 0;
  *fits = true;
  for (int32_t i = 0; i < ntensors; ++i) {
    const int64_t n = size_of(i);
    if (n == 0) continue;
    const uint64_t nb = (static_cast<uint64_t>(n) + QOPT_BLOCK - 1) / QOPT_BLOCK;
    uint64_t lo = 0;
    while (lo < nb) {
      if (c.npieces == static_cast<uint32_t>(kMaxTensors)) {
        *fits = false;
        return QOPT_OK;
      }
      const uint64_t take = (nb - lo < target - blocks) ? nb - lo : target - blocks;
      const uint32_t slot = c.npieces++;
      if (fill(c, slot, i)) c.vector_ok |= uint64_t{1} << slot;
      c.block_lo[slot] = static_cast<uint32_t>(lo);
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

// Blocks per launch at most.  Every wave of a launch takes the same number of blocks,
// but waves progress at different rates, so over a long launch they drift apart and
// the blocks in flight spread over an ever wider stretch of memory.  Measured in one
// process on the same buffers, against one launch per 48 tensors: the Llama-7B step
// 1.5 % faster with launches of at most 2^18 blocks (1.1 % at 2^17, 2.6 % slower at
// 2^15, where the launches' ramps and tails start to cost), the 20B bf16 step 2.1 %
// faster (its single launch became 38), the codec on one 6.7e9-value tensor 2-4 %.
constexpr uint64_t kMaxLaunchBlocks = uint64_t{1} << 18;
// The codec's launches are cheaper to start (one codebook to stage, no moments), and
// its long calls gain from shorter launches still: on one 6.7e9-value tensor, launches
// of 2^16 blocks ran quantize 5-6 % and dequantize 2-3 % faster than launches of 2^18
// (two processes).  A call of 2^17 blocks split in two ran 0.8 % slower, so calls of up
// to 2^18 blocks keep the step's bound.
constexpr uint64_t kCodecLongLaunchBlocks = uint64_t{1} << 16;

template <typename Chunk> uint64_t launch_block_cap(uint64_t total);
template <> uint64_t launch_block_cap<StepChunk>(uint64_t) { return kMaxLaunchBlocks; }
template <> uint64_t launch_block_cap<CodecChunk>(uint64_t total) {
  return total > kMaxLaunchBlocks ? kCodecLongLaunchBlocks : kMaxLaunchBlocks;
}

// Launch count of the plan: the smallest count (from the piece and block bounds up)
// whose greedy assignment keeps every launch within kMaxTensors pieces and the block
// bound of launch_block_cap.
template <typename Chunk, typename SizeOf, typename Fill>
int count_chunks(int32_t ntensors, const SizeOf& size_of, const Fill& fill,
                 uint64_t* nchunks_out, uint64_t* total_out) {
  uint64_t total = 0, pieces = 0;
  for (int32_t i = 0; i < ntensors; ++i) {
    const int64_t n = size_of(i);
    if (n == 0) continue;
    const uint64_t nb = (static_cast<uint64_t>(n) + QOPT_BLOCK - 1) / QOPT_BLOCK;
    if (nb > 0xFFFFFFFFull) return QOPT_EINVAL;  // block index of one tensor is 32-bit
    total += nb;
    ++pieces;
  }
  *total_out = total;
  *nchunks_out = 0;
  if (total == 0) return QOPT_OK;
  uint64_t nchunks = (pieces + kMaxTensors - 1) / kMaxTensors;
  const uint64_t cap = launch_block_cap<Chunk>(total);
  const uint64_t by_size = (total + cap - 1) / cap;
  if (nchunks < by_size) nchunks = by_size;
  for (;; ++nchunks) {
    bool fits = false;
    plan_chunks<Chunk>(ntensors, size_of, fill, nchunks, total,
                       [](const Chunk&, uint64_t) { return static_cast<int>(QOPT_OK); }, &fits);
    if (fits) break;
  }
  *nchunks_out = nchunks;
  return QOPT_OK;
}

// Plans and launches `kernel` over the tensors, one launch per chunk of the plan.
// kFork: the launches alternate between `stream` and the device's second stream
// (side_stream), so that each launch's last waves overlap the next launch's first
// ones; the second stream starts after the work queued on `stream` before the call,
// and `stream` waits for the second stream's launches before anything queued after
// the call.  The launches touch disjoint blocks, so their order does not matter.
// Measured in one process on the same buffers: the 20B bf16 step (38 launches)
// 4.8-5.8 % faster (three processes); the fp32-parameter steps 1-1.6 % slower, so they
// keep one stream.
template <typename Chunk, bool kFork = false, typename Kernel, typename SizeOf, typename Fill,
          typename... Args>
int launch_planned(Kernel kernel, int cap, uint32_t run, int32_t ntensors, const SizeOf& size_of,
                   const Fill& fill, hipStream_t stream, Args... args) {
  uint64_t nchunks = 0, total = 0;
  int rc = count_chunks<Chunk>(ntensors, size_of, fill, &nchunks, &total);
  if (rc != QOPT_OK || total == 0) return rc;
  hipStream_t second = stream;
  hipEvent_t before = nullptr, after = nullptr;
  const bool fork = kFork && nchunks > 1;
  if (fork) {
    rc = side_stream(&second);
    if (rc != QOPT_OK) return rc;
    if (hipEventCreateWithFlags(&before, hipEventDisableTiming) != hipSuccess) return QOPT_ELAUNCH;
    if (hipEventCreateWithFlags(&after, hipEventDisableTiming) != hipSuccess) {
      hipEventDestroy(before);
      return QOPT_ELAUNCH;
    }
    if (hipEventRecord(before, stream) != hipSuccess ||
        hipStreamWaitEvent(second, before, 0) != hipSuccess) {
      hipEventDestroy(before);
      hipEventDestroy(after);
      return QOPT_ELAUNCH;
    }
  }
  uint64_t index = 0;
  bool fits = true;
  rc = plan_chunks<Chunk>(
      ntensors, size_of, fill, nchunks, total,
      [&](const Chunk& c, uint64_t blocks) {
        unsigned grid = 0;
        int r = grid_for(kernel, static_cast<uint32_t>(blocks), cap, run, &grid);
        if (r != QOPT_OK) return r;
        hipStream_t s = (index++ & 1) ? second : stream;
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, s, c, args...);
        return launch_status();
      },
      &fits);
  if (fork) {
    // join whatever was enqueued, also after a failed launch
    if (hipEventRecord(after, second) != hipSuccess ||
        hipStreamWaitEvent(stream, after, 0) != hipSuccess)
      rc = QOPT_ELAUNCH;
    hipEventDestroy(before);
    hipEventDestroy(after);
  }
  return rc;
}

// Descriptor fillers of the step and the codec.
struct StepFill {
  const qopt_tensor* t;
  size_t psize, gsize;
  bool operator()(StepChunk& c, uint32_t slot, int32_t i) const {
    const qopt_tensor& x = t[i];
    c.param[slot] = x.param;
    c.grad[slot] = x.grad;
    c.m_codes[slot] = x.m_codes;
    c.v_codes[slot] = x.v_codes;
    c.m_absmax[slot] = x.m_absmax;
    c.v_absmax[slot] = x.v_absmax;
    c.n[slot] = x.n;
    return aligned(x.param, 4 * psize) && aligned(x.grad, 4 * gsize) && aligned(x.m_codes, 4) &&
           aligned(x.v_codes, 4);
  }
};

struct StepSize {
  const qopt_tensor* t;
  int64_t operator()(int32_t i) const { return t[i].n; }
};

struct CodecFill {
  const qopt_codec_tensor* t;
  bool operator()(CodecChunk& c, uint32_t slot, int32_t i) const {
    const qopt_codec_tensor& x = t[i];
    c.vals[slot] = x.values;
    c.codes[slot] = x.codes;
    c.absmax[slot] = x.absmax;
    c.n[slot] = x.n;
    return aligned(x.values, 16) && aligned(x.codes, 4);
  }
};

struct CodecSize {
  const qopt_codec_tensor* t;
  int64_t operator()(int32_t i) const { return t[i].n; }
};

template <typename PT, typename GT, int kMode>
int launch_step_mode(const qopt_tensor* tensors, int32_t ntensors, size_t psize, size_t gsize,
                     const AdamScalars& k, const qopt_codebook* cbm, const qopt_codebook* cbv,
                     hipStream_t stream) {
  return launch_planned<StepChunk, std::is_same<PT, uint16_t>::value>(
      adam8bit_kernel<PT, GT, kMode>, 0, step_run<PT, GT>(), ntensors, StepSize{tensors},
      StepFill{tensors, psize, gsize}, stream, k, cbm, cbv);
}

// mode: a ScreenMode, which only bf16 parameters use.
template <typename PT, typename GT>
int launch_step_chunks(const qopt_tensor* tensors, int32_t ntensors, size_t psize, size_t gsize,
                       const AdamScalars& k, int mode, const qopt_codebook* cbm,
                       const qopt_codebook* cbv, hipStream_t stream) {
  if constexpr (std::is_same<PT, uint16_t>::value) {
    if (mode == kScreen)
      return launch_step_mode<PT, GT, kScreen>(tensors, ntensors, psize, gsize, k, cbm, cbv, stream);
    if (mode == kScreenSubCheck)
      return launch_step_mode<PT, GT, kScreenSubCheck>(tensors, ntensors, psize, gsize, k, cbm, cbv,
                                                       stream);
  }
  return launch_step_mode<PT, GT, kNoScreen>(tensors, ntensors, psize, gsize, k, cbm, cbv, stream);
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

namespace {

int check_codec_tensors(const qopt_codec_tensor* tensors, int32_t ntensors, bool* any) {
  if (ntensors < 0) return QOPT_EINVAL;
  if (ntensors > 0 && tensors == nullptr) return QOPT_EINVAL;
  *any = false;
  for (int32_t i = 0; i < ntensors; ++i) {
    const qopt_codec_tensor& t = tensors[i];
    if (t.n < 0) return QOPT_EINVAL;
    if (t.n == 0) continue;
    *any = true;
    if (!t.values || !t.codes || !t.absmax) return QOPT_EINVAL;
    if (!aligned(t.values, 4) || !aligned(t.absmax, 4)) return QOPT_EALIGN;
  }
  return QOPT_OK;
}

// Quantize, with two blocks in flight per wave, runs best with 2 workgroups per CU
// (8 waves): on 2^28 values, compared in one process, 3.1-3.4 % faster than one block
// in flight at 3 per CU (the previous best), while two in flight at 3 per CU gained
// 0.2 %, three in flight at 2 per CU 2.9 %, and 1 per CU lost 13 %.  Dequantize and
// the step run at full occupancy.
#ifndef QOPT_QUANTIZE_WG_PER_CU
#define QOPT_QUANTIZE_WG_PER_CU 2
#endif
constexpr int kQuantizeWgPerCu = QOPT_QUANTIZE_WG_PER_CU;

template <typename Kernel>
int codec_multi(Kernel kernel, int cap, const qopt_codebook* cb_dev,
                const qopt_codec_tensor* tensors, int32_t ntensors, void* stream) {
  bool any = false;
  int rc = check_codec_tensors(tensors, ntensors, &any);
  if (rc != QOPT_OK || !any) return rc;
  if (!cb_dev) return QOPT_EINVAL;
  if (!aligned(cb_dev, 16)) return QOPT_EALIGN;
  return launch_planned<CodecChunk>(kernel, cap, 1, ntensors, CodecSize{tensors}, CodecFill{tensors},
                                    static_cast<hipStream_t>(stream), cb_dev);
}

}  // namespace

extern "C" int qopt_quantize_blockwise_multi(const qopt_codebook* cb_dev,
                                             const qopt_codec_tensor* tensors, int32_t ntensors,
                                             void* stream) {
  return codec_multi(quantize_kernel, kQuantizeWgPerCu, cb_dev, tensors, ntensors, stream);
}

extern "C" int qopt_dequantize_blockwise_multi(const qopt_codebook* cb_dev,
                                               const qopt_codec_tensor* tensors, int32_t ntensors,
                                               void* stream) {
  return codec_multi(dequantize_kernel, 0, cb_dev, tensors, ntensors, stream);
}

extern "C" int qopt_quantize_blockwise(const qopt_codebook* cb_dev, const float* x_dev, int64_t n,
                                       uint8_t* codes_dev, float* absmax_dev, void* stream) {
  if (n < 0) return QOPT_EINVAL;
  if (n == 0) return QOPT_OK;
  if (!cb_dev || !x_dev || !codes_dev || !absmax_dev) return QOPT_EINVAL;
  if (!aligned(cb_dev, 16) || !aligned(x_dev, 4) || !aligned(absmax_dev, 4)) return QOPT_EALIGN;
  // the kernel only reads `values` when quantizing
  const qopt_codec_tensor t = {const_cast<float*>(x_dev), codes_dev, absmax_dev, n};
  return codec_multi(quantize_kernel, kQuantizeWgPerCu, cb_dev, &t, 1, stream);
}

extern "C" int qopt_dequantize_blockwise(const qopt_codebook* cb_dev, const uint8_t* codes_dev,
                                         const float* absmax_dev, int64_t n, float* y_dev,
                                         void* stream) {
  if (n < 0) return QOPT_EINVAL;
  if (n == 0) return QOPT_OK;
  if (!cb_dev || !codes_dev || !absmax_dev || !y_dev) return QOPT_EINVAL;
  if (!aligned(cb_dev, 16) || !aligned(y_dev, 4) || !aligned(absmax_dev, 4)) return QOPT_EALIGN;
  // the kernel only reads `codes` and `absmax` when dequantizing
  const qopt_codec_tensor t = {y_dev, const_cast<uint8_t*>(codes_dev),
                               const_cast<float*>(absmax_dev), n};
  return codec_multi(dequantize_kernel, 0, cb_dev, &t, 1, stream);
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
  // The bf16 short path's folded scalars, each one rounding of an exact quotient of
  // binary32 values.  Its error bound needs a and b normal (or b zero) and a
  // denominator fma(sq, a, b) that is normal, zero or infinite and at most 2^126
  // when finite (the range where the hardware reciprocal was checked): sq is 0, in
  // [2^-63, 2^64] or infinite, hence a in [2^-63, 2^61] and b at most 2^125.  The
  // step size must be positive and at most 2^20, so that subnormal rounding errors
  // of the sequence's quotient, scaled by it, stay under the bound's 2^-126 floor.
  const double ss = static_cast<double>(k.step_size);
  k.short_a = ss > 0.0 ? static_cast<float>(static_cast<double>(k.inv_sqrt_bc2) / ss) : 0.0f;
  k.short_b = ss > 0.0 ? static_cast<float>(static_cast<double>(k.eps) / ss) : 0.0f;
  k.t_limit = static_cast<float>((ss < 1.0 ? ss : 1.0) * 0x1p127);
  const bool a_ok = k.short_a >= 0x1p-63f && k.short_a <= 0x1p61f;
  const bool b_ok = k.short_b == 0.0f || (k.short_b >= 0x1p-126f && k.short_b <= 0x1p125f);
  const bool screen = ss > 0.0 && ss <= 0x1p20 && a_ok && b_ok;
  // A subnormal v (below 2^-126) has a square root below 2^-63, which the hardware
  // flushes to zero.  With eps >= 2^-39 inv_sqrt_bc2 (so a / b <= 2^39, up to the two
  // roundings of a and b) that moves the denominator by under 2^-63 a / b, about
  // 2^-24 of itself, inside the 2^-23 the error bound allows for the square root.
  // With eps = 0 it makes the denominator 0 and t infinite or NaN, which the bound on
  // |t| rejects.  Only eps in between needs a test for subnormal v.
  const bool sub_check =
      k.eps != 0.0f &&
      !(static_cast<double>(k.eps) >= static_cast<double>(k.inv_sqrt_bc2) * 0x1p-39);
  const int mode = !screen ? kNoScreen : (sub_check ? kScreenSubCheck : kScreen);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (param_dtype == QOPT_F32 && grad_dtype == QOPT_F32)
    return launch_step_chunks<float, float>(tensors, ntensors, psize, gsize, k, mode, cb_m_dev,
                                            cb_v_dev, s);
  if (param_dtype == QOPT_F32 && grad_dtype == QOPT_BF16)
    return launch_step_chunks<float, uint16_t>(tensors, ntensors, psize, gsize, k, mode, cb_m_dev,
                                               cb_v_dev, s);
  if (param_dtype == QOPT_BF16 && grad_dtype == QOPT_F32)
    return launch_step_chunks<uint16_t, float>(tensors, ntensors, psize, gsize, k, mode, cb_m_dev,
                                               cb_v_dev, s);
  return launch_step_chunks<uint16_t, uint16_t>(tensors, ntensors, psize, gsize, k, mode, cb_m_dev,
                                                  cb_v_dev, s);
}

// Workgroups per CU the step itself runs with (its occupancy), so that the traffic
// probe moves the step's bytes with as many waves in flight.
template <typename PT, typename GT>
int step_wg_per_cu(int* per_cu) {
  constexpr int kMode = std::is_same<PT, uint16_t>::value ? kScreen : kNoScreen;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, adam8bit_kernel<PT, GT, kMode>,
                                                   kThreads, 0) != hipSuccess ||
      *per_cu <= 0)
    return QOPT_ELAUNCH;
  return QOPT_OK;
}

template <typename PT, typename GT>
int launch_traffic_probe(const qopt_tensor* tensors, int32_t ntensors, size_t psize, size_t gsize,
                         hipStream_t stream) {
  int per_cu = 0;
  const int rc = step_wg_per_cu<PT, GT>(&per_cu);
  if (rc != QOPT_OK) return rc;
  return launch_planned<StepChunk, std::is_same<PT, uint16_t>::value>(
      step_traffic_kernel<PT, GT>, per_cu, step_run<PT, GT>(), ntensors, StepSize{tensors},
      StepFill{tensors, psize, gsize}, stream);
}

extern "C" int qopt_adam8bit_traffic_probe(const qopt_tensor* tensors, int32_t ntensors,
                                           int param_dtype, int grad_dtype, void* stream) {
  bool any = false;
  const int rc = check_step_tensors(tensors, ntensors, param_dtype, grad_dtype, &any);
  if (rc != QOPT_OK || !any) return rc;
  const size_t psize = param_dtype == QOPT_F32 ? 4 : 2;
  const size_t gsize = grad_dtype == QOPT_F32 ? 4 : 2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (param_dtype == QOPT_F32 && grad_dtype == QOPT_F32)
    return launch_traffic_probe<float, float>(tensors, ntensors, psize, gsize, s);
  if (param_dtype == QOPT_F32 && grad_dtype == QOPT_BF16)
    return launch_traffic_probe<float, uint16_t>(tensors, ntensors, psize, gsize, s);
  if (param_dtype == QOPT_BF16 && grad_dtype == QOPT_F32)
    return launch_traffic_probe<uint16_t, float>(tensors, ntensors, psize, gsize, s);
  return launch_traffic_probe<uint16_t, uint16_t>(tensors, ntensors, psize, gsize, s);
}

extern "C" int qopt_adam8bit_launch_count(const qopt_tensor* tensors, int32_t ntensors,
                                          int param_dtype, int grad_dtype, int64_t* launches) {
  if (launches == nullptr) return QOPT_EINVAL;
  bool any = false;
  int rc = check_step_tensors(tensors, ntensors, param_dtype, grad_dtype, &any);
  if (rc != QOPT_OK) return rc;
  uint64_t nchunks = 0, total = 0;
  rc = count_chunks<StepChunk>(ntensors, StepSize{tensors},
                               StepFill{tensors, param_dtype == QOPT_F32 ? 4u : 2u,
                                        grad_dtype == QOPT_F32 ? 4u : 2u},
                               &nchunks, &total);
  if (rc != QOPT_OK) return rc;
  *launches = static_cast<int64_t>(nchunks);
  return QOPT_OK;
}
