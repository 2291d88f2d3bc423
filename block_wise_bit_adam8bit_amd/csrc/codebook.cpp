// Host side of libqopt: codebook construction, status strings, version.
//
// The dynamic-tree code ("8-BIT OPTIMIZERS VIA BLOCK-WISE QUANTIZATION" summary
// page, §2 "Dynamic Quantization"): reading a magnitude bit pattern from its most
// significant bit, a run of e zero bits is the exponent, the following 1 bit is the
// indicator, and the f bits after it are a linear fraction j.  The signed code
// spends its top bit on the sign and has 7 magnitude bits; the unsigned code (for
// the always-positive second moment) gives that bit to the magnitude, 8 bits.
//
// Readings where the page is silent: the exponent base is 10, the fraction places
// the value on the right end of the j-th of 2^f equal steps of [0.1, 1], so
//     value = 10^-e * (0.1 + 0.9 * (j + 1) / 2^f) = (2^f + 9 (j + 1)) / (10^(e+1) 2^f),
// the all-zero pattern is 0, and each value is stored as the nearest binary32
// (ties to even).  The encoder picks the nearest magnitude by binary32 distances,
// ties to the smaller one; this file turns that rule into exact decision
// thresholds and a bucket index so the kernels need two table reads per value.

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "qopt.h"

namespace {

static_assert(sizeof(qopt_codebook) % 16 == 0, "codebook must be a whole number of 16-byte rows");
static_assert(offsetof(qopt_codebook, decode) % 16 == 0, "decode table alignment");
static_assert(offsetof(qopt_codebook, thresh) % 16 == 0, "threshold table alignment");
static_assert(offsetof(qopt_codebook, bucket) % 16 == 0, "bucket table alignment");

typedef unsigned __int128 u128;

inline uint32_t f32_bits(float x) {
  uint32_t b;
  std::memcpy(&b, &x, 4);
  return b;
}

inline float bits_f32(uint32_t b) {
  float x;
  std::memcpy(&x, &b, 4);
  return x;
}

inline int floor_log2_u64(uint64_t x) { return 63 - __builtin_clzll(x); }

// Nearest binary32 to num / den (num, den > 0, result in the normal range), ties to
// even: scale the quotient into [2^23, 2^24), take integer quotient and remainder,
// round on the remainder.
float ratio_to_f32(uint64_t num, uint64_t den) {
  if (num == 0) return 0.0f;
  int e = floor_log2_u64(num) - floor_log2_u64(den);
  // make e = floor(log2(num / den))
  {
    u128 lhs = num, rhs = den;
    if (e >= 0) rhs <<= e; else lhs <<= -e;
    if (lhs < rhs) --e;
  }
  const int s = 23 - e;  // num / den * 2^s lies in [2^23, 2^24)
  u128 n = num, d = den;
  if (s >= 0) n <<= s; else d <<= -s;
  u128 q = n / d, r = n % d;
  if (2 * r > d || (2 * r == d && (q & 1))) ++q;  // q may reach 2^24: still exact
  return std::ldexp(static_cast<float>(static_cast<uint64_t>(q)), -s);
}

// Magnitude of pattern p (p >= 1) with nb magnitude bits, as num / den.
void pattern_ratio(int nb, uint32_t p, uint64_t* num, uint64_t* den) {
  const int top = 31 - __builtin_clz(p);  // position of the indicator bit
  const int f = top;                      // fraction bits below it
  const int e = nb - 1 - top;             // zero bits above it
  const uint64_t j = p - (1u << f);
  uint64_t pow10 = 1;
  for (int i = 0; i < e + 1; ++i) pow10 *= 10;
  *num = (uint64_t{1} << f) + 9 * (j + 1);
  *den = pow10 << f;
}

// The nearest-magnitude rule on a >= 0: lo = last index with mag[lo] <= a; step up
// to lo + 1 only if that neighbour is strictly nearer in binary32.
int nearest_magnitude(const float* mag, int nmag, float a) {
  int lo = 0;
  int hi = nmag;  // mag[lo] <= a < mag[hi] (mag[nmag] = +inf)
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (mag[mid] <= a) lo = mid; else hi = mid;
  }
  if (lo + 1 < nmag) {
    const float up = mag[lo + 1] - a;
    const float down = a - mag[lo];
    if (up < down) return lo + 1;
  }
  return lo;
}

int build(int kind, qopt_codebook* out) {
  const int nb = (kind == QOPT_CB_SIGNED) ? 7 : 8;
  const int nmag = 1 << nb;
  float mag[256];
  mag[0] = 0.0f;
  for (int p = 1; p < nmag; ++p) {
    uint64_t num, den;
    pattern_ratio(nb, static_cast<uint32_t>(p), &num, &den);
    mag[p] = ratio_to_f32(num, den);
    if (!(mag[p] > mag[p - 1])) return QOPT_EINTERNAL;  // pattern order = value order
  }

  std::memset(out, 0, sizeof(*out));
  out->magic = QOPT_CODEBOOK_MAGIC;
  out->kind = static_cast<uint32_t>(kind);
  out->sign_mask = (kind == QOPT_CB_SIGNED) ? 0x80u : 0u;
  out->nmag = static_cast<uint32_t>(nmag);

  for (int c = 0; c < 256; ++c) {
    if (kind == QOPT_CB_SIGNED) {
      const float v = mag[c & 0x7F];
      out->decode[c] = (c & 0x80) ? -v : v;
    } else {
      out->decode[c] = mag[c];
    }
  }

  // thresh[k]: least binary32 a >= 0 with nearest index >= k.  It lies in
  // (mag[k-1], mag[k]]; the rule is monotone in a, so bisect on bit patterns.
  const float inf = bits_f32(0x7F800000u);
  for (int k = 0; k < QOPT_THRESH_LEN; ++k) out->thresh[k] = inf;
  out->thresh[0] = 0.0f;
  for (int k = 1; k < nmag; ++k) {
    uint32_t lo = f32_bits(mag[k - 1]);  // nearest(lo) == k - 1
    uint32_t hi = f32_bits(mag[k]);      // nearest(hi) == k
    if (nearest_magnitude(mag, nmag, bits_f32(lo)) != k - 1 ||
        nearest_magnitude(mag, nmag, bits_f32(hi)) != k)
      return QOPT_EINTERNAL;
    while (hi - lo > 1) {
      const uint32_t mid = lo + (hi - lo) / 2;
      if (nearest_magnitude(mag, nmag, bits_f32(mid)) >= k) hi = mid; else lo = mid;
    }
    out->thresh[k] = bits_f32(hi);
  }

  // Buckets: key = bits >> 15 (exponent + 8 leading mantissa bits of a >= 0).
  // Bucket 0 starts one key below the first threshold, so everything below it has
  // index 0; the last bucket is the one holding 1.0 and absorbs anything larger.
  const uint32_t key0 = (f32_bits(out->thresh[1]) >> 15) - 1;
  const uint32_t key_last = f32_bits(1.0f) >> 15;
  const uint32_t nbuckets = key_last - key0 + 1;
  if (nbuckets > QOPT_MAX_BUCKETS) return QOPT_EINTERNAL;
  out->key0 = key0;
  out->nbuckets = nbuckets;
  for (uint32_t i = 0; i < nbuckets; ++i) {
    const float start = bits_f32((key0 + i) << 15);
    const float end = (i + 1 < nbuckets) ? bits_f32((key0 + i + 1) << 15) : inf;
    int base = 0;  // thresholds <= start
    int inside = 0;  // thresholds in (start, end)
    for (int k = 1; k < nmag; ++k) {
      if (out->thresh[k] <= start) ++base;
      else if (out->thresh[k] < end) ++inside;
    }
    if (inside > 1 || base > 255) return QOPT_EINTERNAL;
    out->bucket[i] = static_cast<uint8_t>(base);
  }
  // Everything below bucket 0 must encode to 0.
  if (!(out->thresh[1] > bits_f32(key0 << 15))) return QOPT_EINTERNAL;
  return QOPT_OK;
}

}  // namespace

extern "C" int qopt_codebook_build(int kind, qopt_codebook* out) {
  if (out == nullptr) return QOPT_EINVAL;
  if (kind != QOPT_CB_SIGNED && kind != QOPT_CB_UNSIGNED) return QOPT_EUNSUPPORTED;
  return build(kind, out);
}

extern "C" const char* qopt_status_string(int status) {
  switch (status) {
    case QOPT_OK: return "ok";
    case QOPT_EINVAL: return "invalid argument";
    case QOPT_EUNSUPPORTED: return "unsupported dtype or codebook kind";
    case QOPT_EALIGN: return "pointer not aligned to its element size";
    case QOPT_ELAUNCH: return "HIP launch or device query failed";
    case QOPT_EINTERNAL: return "internal invariant violated while building a codebook";
    case QOPT_ENOSPACE:
      return "the request needs more scratch memory than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

extern "C" int qopt_version(void) { return 100; }
