// Measurement aid (include/qopt_probe.h): bytes-only access patterns for the traffic
// of the 8-bit Adam step with fp32 parameters and bf16 gradients.  Not part of the
// method.  Every pattern reads a block's parameters (8 KB), gradients (4 KB) and two
// code streams (2 KB each) and writes the parameters and code streams back unchanged;
// the patterns differ in how waves walk the blocks, in the order of their accesses and
// (the paced patterns) in when they issue them.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "qopt_probe.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;  // waves per workgroup: one per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kSlices = 8;  // 1 KB parameter accesses per block (16 B per lane)
constexpr uint64_t kMaxLaunchBlocks = uint64_t{1} << 18;  // blocks per launch at most

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T> __device__ __forceinline__ T ld(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T> __device__ __forceinline__ void st(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

struct Bufs {
  u32x4* p;   // 512 x 16 B per block
  u32x2* g;   // 512 x 8 B per block
  uint8_t* cm;
  uint8_t* cv;
  uint64_t nblocks;
};

// Code accesses of kCodeBytes bytes per lane: 4 (256 B per wave access, 8 per block
// and stream) or 16 (1 KB per wave access, 2 per block and stream).
template <int kCodeBytes> struct Code;
template <> struct Code<4> {
  typedef uint32_t T;
  static constexpr int kN = 8;
};
template <> struct Code<16> {
  typedef u32x4 T;
  static constexpr int kN = 2;
};

template <int kCodeBytes> struct Block {
  u32x4 p[kSlices];
  u32x2 g[kSlices];
  typename Code<kCodeBytes>::T cm[Code<kCodeBytes>::kN];
  typename Code<kCodeBytes>::T cv[Code<kCodeBytes>::kN];
};

// Loads of block b, stream after stream or slice after slice (the four streams of a
// slice together, as the step issues them).
template <int kCodeBytes, bool kStreamMajor>
__device__ __forceinline__ void load(Block<kCodeBytes>& d, const Bufs& b, uint64_t blk, int lane) {
  typedef typename Code<kCodeBytes>::T C;
  constexpr int kN = Code<kCodeBytes>::kN;
  const u32x4* p = b.p + blk * 512 + lane;
  const u32x2* g = b.g + blk * 512 + lane;
  const C* cm = reinterpret_cast<const C*>(b.cm + blk * 2048) + lane;
  const C* cv = reinterpret_cast<const C*>(b.cv + blk * 2048) + lane;
  if constexpr (kStreamMajor) {
#pragma unroll
    for (int s = 0; s < kSlices; ++s) d.p[s] = ld(p + s * kWave);
#pragma unroll
    for (int s = 0; s < kSlices; ++s) d.g[s] = ld(g + s * kWave);
#pragma unroll
    for (int t = 0; t < kN; ++t) d.cm[t] = ld(cm + t * kWave);
#pragma unroll
    for (int t = 0; t < kN; ++t) d.cv[t] = ld(cv + t * kWave);
  } else {
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
      d.p[s] = ld(p + s * kWave);
      d.g[s] = ld(g + s * kWave);
      if (s < kN) {
        d.cm[s] = ld(cm + s * kWave);
        d.cv[s] = ld(cv + s * kWave);
      }
    }
  }
}

// The block written back: parameters, then m codes, then v codes.  The gradients are
// waited for (as a step would), and the barrier keeps the compiler from dropping the
// store of a value just loaded from the same address.
template <int kCodeBytes>
__device__ __forceinline__ void store(const Block<kCodeBytes>& d, const Bufs& b, uint64_t blk,
                                      int lane) {
  typedef typename Code<kCodeBytes>::T C;
  constexpr int kN = Code<kCodeBytes>::kN;
#pragma unroll
  for (int s = 0; s < kSlices; ++s) asm volatile("" ::"v"(d.g[s]));
  asm volatile("" ::: "memory");
  u32x4* p = b.p + blk * 512 + lane;
  C* cm = reinterpret_cast<C*>(b.cm + blk * 2048) + lane;
  C* cv = reinterpret_cast<C*>(b.cv + blk * 2048) + lane;
#pragma unroll
  for (int s = 0; s < kSlices; ++s) st(p + s * kWave, d.p[s]);
#pragma unroll
  for (int t = 0; t < kN; ++t) st(cm + t * kWave, d.cm[t]);
#pragma unroll
  for (int t = 0; t < kN; ++t) st(cv + t * kWave, d.cv[t]);
}

// Walk: each wave takes runs of kRun consecutive blocks (run r on wave r mod waves)
// with the loads of its next kDepth blocks in flight: a block is written back as
// soon as its loads have arrived, then the loads of the block kDepth places ahead are
// issued into its registers.
template <int kDepth, int kWavesPerSimd, int kRun, int kCodeBytes, bool kStreamMajor>
__global__ void __launch_bounds__(kThreads, kWavesPerSimd) walk_kernel(Bufs b) {
  const int lane = threadIdx.x % kWave;
  const uint64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint64_t nw = static_cast<uint64_t>(gridDim.x) * kWaves;
  const uint64_t n = b.nblocks;
  auto next = [&](uint64_t k) { return ((k + 1) % kRun) ? k + 1 : (k / kRun + nw) * kRun; };
  uint64_t ahead = (static_cast<uint64_t>(blockIdx.x) * kWaves + wave) * kRun;
  if (ahead >= n) return;
  Block<kCodeBytes> buf[kDepth];
  uint64_t blk[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i) {
    blk[i] = ahead;
    if (ahead < n) {
      load<kCodeBytes, kStreamMajor>(buf[i], b, ahead, lane);
      ahead = next(ahead);
    }
  }
  for (;;) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      // blocks are taken in walk order: the first past the end ends the wave
      if (blk[i] >= n) return;
      store<kCodeBytes>(buf[i], b, blk[i], lane);
      blk[i] = ahead;
      if (ahead < n) {
        load<kCodeBytes, kStreamMajor>(buf[i], b, ahead, lane);
        ahead = next(ahead);
      }
    }
  }
}

// Burst: each wave loads kBlocks consecutive blocks, stream by stream across all of
// them, then writes them back; bursts are handed out with a grid stride.
template <int kBlocks, int kWavesPerSimd>
__global__ void __launch_bounds__(kThreads, kWavesPerSimd) burst_kernel(Bufs b) {
  const int lane = threadIdx.x % kWave;
  const uint64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint64_t nw = static_cast<uint64_t>(gridDim.x) * kWaves;
  const uint64_t nbursts = b.nblocks / kBlocks;  // a trailing partial burst is left out
  for (uint64_t k = static_cast<uint64_t>(blockIdx.x) * kWaves + wave; k < nbursts; k += nw) {
    const uint64_t b0 = k * kBlocks;
    u32x4 p[kBlocks][kSlices];
    u32x2 g[kBlocks][kSlices];
    u32x4 cm[kBlocks][2], cv[kBlocks][2];
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int s = 0; s < kSlices; ++s) p[r][s] = ld(b.p + (b0 + r) * 512 + s * kWave + lane);
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int s = 0; s < kSlices; ++s) g[r][s] = ld(b.g + (b0 + r) * 512 + s * kWave + lane);
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        cm[r][t] = ld(reinterpret_cast<const u32x4*>(b.cm + (b0 + r) * 2048) + t * kWave + lane);
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        cv[r][t] = ld(reinterpret_cast<const u32x4*>(b.cv + (b0 + r) * 2048) + t * kWave + lane);
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int s = 0; s < kSlices; ++s) asm volatile("" ::"v"(g[r][s]));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int s = 0; s < kSlices; ++s) st(b.p + (b0 + r) * 512 + s * kWave + lane, p[r][s]);
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        st(reinterpret_cast<u32x4*>(b.cm + (b0 + r) * 2048) + t * kWave + lane, cm[r][t]);
#pragma unroll
    for (int r = 0; r < kBlocks; ++r)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        st(reinterpret_cast<u32x4*>(b.cv + (b0 + r) * 2048) + t * kWave + lane, cv[r][t]);
  }
}

// Paced: every wave moves one block per period of the chip's 100 MHz real-time
// counter.  At the start of each period it writes back the block it loaded in the
// previous period and loads its next block (grid stride), so that all waves issue
// their reads and writes together instead of a steady mix of both.  The period is
// the grid's waves times the bytes of a block over kBytesPerTick; if the memory
// system cannot move a period's bytes in time, waves fall behind the clock and issue
// as soon as they can.  Each wait is bounded (the counter always advances).
struct PacedBlock {
  u32x4 p[kSlices];
  u32x2 g[kSlices];
  uint32_t cm[kSlices], cv[kSlices];
};
__device__ __forceinline__ void paced_load(PacedBlock& x, const Bufs& b, uint64_t k, int lane) {
  const u32x4* pp = b.p + k * 512 + lane;
  const u32x2* gp = b.g + k * 512 + lane;
  const uint32_t* cmp = reinterpret_cast<const uint32_t*>(b.cm + k * 2048) + lane;
  const uint32_t* cvp = reinterpret_cast<const uint32_t*>(b.cv + k * 2048) + lane;
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    x.p[s] = ld(pp + s * kWave);
    x.g[s] = ld(gp + s * kWave);
    x.cm[s] = ld(cmp + s * kWave);
    x.cv[s] = ld(cvp + s * kWave);
  }
}
// Writes back the parameters and codes slice by slice; returns a fold of the gradients
// (so that they are waited for, as a step would).
__device__ __forceinline__ uint32_t paced_store(const PacedBlock& x, const Bufs& b, uint64_t k,
                                                int lane) {
  u32x4* pp = b.p + k * 512 + lane;
  uint32_t* cmp = reinterpret_cast<uint32_t*>(b.cm + k * 2048) + lane;
  uint32_t* cvp = reinterpret_cast<uint32_t*>(b.cv + k * 2048) + lane;
  uint32_t gx = 0;
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    gx ^= x.g[s].x ^ x.g[s].y;
    st(pp + s * kWave, x.p[s]);
    st(cmp + s * kWave, x.cm[s]);
    st(cvp + s * kWave, x.cv[s]);
  }
  return gx;
}
__device__ __forceinline__ uint32_t paced_period(uint32_t ticks) {
  return static_cast<uint32_t>(__builtin_amdgcn_s_memrealtime()) / ticks;
}

template <uint32_t kBytesPerTick>
__global__ void __launch_bounds__(kThreads, 2) paced_kernel(Bufs b) {
  const int lane = threadIdx.x % kWave;
  const uint64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint64_t nw = static_cast<uint64_t>(gridDim.x) * kWaves;
  const uint64_t n = b.nblocks;
  uint64_t blk = static_cast<uint64_t>(blockIdx.x) * kWaves + wave;
  if (blk >= n) return;
  constexpr uint64_t kBlockBytes = 8192 + 4096 + 2 * 2048 + 8192 + 2 * 2048;
  const uint64_t t64 = (nw * kBlockBytes + kBytesPerTick - 1) / kBytesPerTick;
  const uint32_t ticks = static_cast<uint32_t>(t64 < 1 ? 1 : (t64 > 0x7FFFFFFFu ? 0x7FFFFFFFu : t64));
  uint32_t cur = paced_period(ticks);
  uint32_t gx = 0;
  PacedBlock a;
  paced_load(a, b, blk, lane);
  for (;;) {
    const uint64_t next = blk + nw;
    uint32_t p = paced_period(ticks);
    for (int i = 0; i < (1 << 16) && p == cur; ++i) {
      __builtin_amdgcn_s_sleep(1);
      p = paced_period(ticks);
    }
    cur = p;
    gx ^= paced_store(a, b, blk, lane);
    // the fold of this block's gradients is consumed here, so their loads stay (as a
    // step needs them), after this period's stores have been issued
    asm volatile("" ::"v"(gx));
    if (next >= n) break;
    paced_load(a, b, next, lane);
    blk = next;
  }
}

struct Pattern {
  const char* name;
  void (*kernel)(Bufs);
  int waves_per_simd;
};

#define QOPT_WALK(D, W, R, C, SM, NAME) {NAME, walk_kernel<D, W, R, C, SM>, W}
const Pattern kPatterns[] = {
    QOPT_WALK(1, 2, 2, 4, false,
              "walk: 1 block in flight, runs of 2, 2 waves/SIMD, 4 B codes, slice order "
              "(the step's own shape)"),
    QOPT_WALK(1, 2, 8, 4, false,
              "walk: 1 block in flight, runs of 8, 2 waves/SIMD, 4 B codes, slice order"),
    QOPT_WALK(1, 2, 8, 16, true,
              "walk: 1 block in flight, runs of 8, 2 waves/SIMD, 16 B codes, stream order"),
    QOPT_WALK(2, 2, 8, 4, true,
              "walk: 2 blocks in flight, runs of 8, 2 waves/SIMD, 4 B codes, stream order"),
    QOPT_WALK(2, 2, 4, 16, true,
              "walk: 2 blocks in flight, runs of 4, 2 waves/SIMD, 16 B codes, stream order"),
    QOPT_WALK(2, 2, 8, 16, true,
              "walk: 2 blocks in flight, runs of 8, 2 waves/SIMD, 16 B codes, stream order"),
    QOPT_WALK(2, 2, 16, 16, true,
              "walk: 2 blocks in flight, runs of 16, 2 waves/SIMD, 16 B codes, stream order"),
    QOPT_WALK(2, 2, 6, 16, true,
              "walk: 2 blocks in flight, runs of 6, 2 waves/SIMD, 16 B codes, stream order"),
    QOPT_WALK(2, 3, 8, 16, true,
              "walk: 2 blocks in flight, runs of 8, 3 waves/SIMD, 16 B codes, stream order"),
    QOPT_WALK(3, 1, 8, 16, true,
              "walk: 3 blocks in flight, runs of 8, 1 wave/SIMD, 16 B codes, stream order"),
    {"burst: 2 blocks at a time, 1 wave/SIMD, 16 B codes, stream order", burst_kernel<2, 1>, 1},
    {"burst: 4 blocks at a time, 1 wave/SIMD, 16 B codes, stream order", burst_kernel<4, 1>, 1},
    {"paced: 1 block per wave and period, 2 waves/SIMD, 4 B codes, slice order, period for "
     "6.0 TB/s", paced_kernel<60000>, 2},
    {"paced: 1 block per wave and period, 2 waves/SIMD, 4 B codes, slice order, period for "
     "6.4 TB/s", paced_kernel<64000>, 2},
    {"paced: 1 block per wave and period, 2 waves/SIMD, 4 B codes, slice order, period for "
     "6.6 TB/s", paced_kernel<66000>, 2},
    {"paced: 1 block per wave and period, 2 waves/SIMD, 4 B codes, slice order, period for "
     "6.8 TB/s", paced_kernel<68000>, 2},
    {"paced: 1 block per wave and period, 2 waves/SIMD, 4 B codes, slice order, period for "
     "7.0 TB/s", paced_kernel<70000>, 2},
};
#undef QOPT_WALK
constexpr int kNumPatterns = static_cast<int>(sizeof(kPatterns) / sizeof(kPatterns[0]));

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

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

extern "C" int qopt_pattern_probe_count(void) { return kNumPatterns; }

extern "C" const char* qopt_pattern_probe_name(int pattern) {
  return pattern >= 0 && pattern < kNumPatterns ? kPatterns[pattern].name : nullptr;
}

extern "C" int qopt_pattern_probe(int pattern, void* params, void* grads, uint8_t* m_codes,
                                  uint8_t* v_codes, int64_t nblocks, void* stream) {
  if (pattern < 0 || pattern >= kNumPatterns || nblocks < 0) return QOPT_EINVAL;
  if (nblocks == 0) return QOPT_OK;
  if (!params || !grads || !m_codes || !v_codes) return QOPT_EINVAL;
  if (!aligned16(params) || !aligned16(grads) || !aligned16(m_codes) || !aligned16(v_codes))
    return QOPT_EALIGN;
  int cus = 0;
  const int rc = device_cus(&cus);
  if (rc != QOPT_OK) return rc;
  // one 4-wave workgroup per CU per wave and SIMD, as the pattern's registers allow
  const Pattern& pt = kPatterns[pattern];
  const unsigned grid = static_cast<unsigned>(cus * pt.waves_per_simd);
  // launches of equal block counts, at most 2^18 blocks each, as the step plans its own
  const uint64_t total = static_cast<uint64_t>(nblocks);
  const uint64_t nlaunch = (total + kMaxLaunchBlocks - 1) / kMaxLaunchBlocks;
  const uint64_t per = (total + nlaunch - 1) / nlaunch;
  for (uint64_t b0 = 0; b0 < total; b0 += per) {
    const uint64_t nb = total - b0 < per ? total - b0 : per;
    const Bufs b{static_cast<u32x4*>(params) + b0 * 512, static_cast<u32x2*>(grads) + b0 * 512,
                 m_codes + b0 * 2048, v_codes + b0 * 2048, nb};
    hipLaunchKernelGGL(pt.kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       b);
    if (hipGetLastError() != hipSuccess) return QOPT_ELAUNCH;
  }
  return QOPT_OK;
}
