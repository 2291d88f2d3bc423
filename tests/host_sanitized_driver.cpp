// Host code of libqopt under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).
//
// Built by tests/test_host_sanitized.py from the library's own sources, with the
// sanitizers on the host side only, and run without a GPU.  It never calls a device
// entry point past its argument checks, so no HIP runtime call is made.
//
//   host_sanitized_driver CODEBOOKS_OUT TRANSITIONS_SIGNED TRANSITIONS_UNSIGNED
//
// 1. Builds the signed and unsigned codebooks and writes both structs, in that
//    order, to CODEBOOKS_OUT (the test compares them with the shipped library's).
// 2. For every binary32 a in [0, 2), looks a's code index up in the tables the way
//    the kernels do and checks it against the number of transitions <= a (each
//    TRANSITIONS file holds the least binary32 at which the nearest magnitude index
//    becomes k, k = 1 .. nmag-1, as raw little-endian binary32).
// 3. Calls the device entry points with arguments their checks must refuse (or
//    accept as empty work) and checks the status codes.
// 4. Reads launch-plan queries from stdin, one per line,
//    "param_dtype grad_dtype n_1 ... n_k", and prints "status launches" for each.
//
// Exits 0 when every check holds; prints what failed and exits 1 otherwise.

#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <sstream>
#include <string>
#include <vector>

#include "qopt.h"
#include "qopt_embedding.h"

namespace {

int g_failures = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++g_failures;
  }
}

std::vector<float> read_floats(const char* path) {
  std::vector<float> out;
  FILE* f = std::fopen(path, "rb");
  if (!f) return out;
  float x;
  while (std::fread(&x, sizeof x, 1, f) == 1) out.push_back(x);
  std::fclose(f);
  return out;
}

// The kernels' lookup: bucket by the top bits of a, then one threshold compare.
uint32_t table_index(const qopt_codebook& cb, uint32_t bits) {
  int64_t i = static_cast<int64_t>(bits >> 15) - static_cast<int64_t>(cb.key0);
  if (i < 0) i = 0;
  if (i > static_cast<int64_t>(cb.nbuckets) - 1) i = cb.nbuckets - 1;
  const uint32_t b = cb.bucket[i];
  float a;
  std::memcpy(&a, &bits, 4);
  return b + (a >= cb.thresh[b + 1] ? 1u : 0u);
}

void sweep(const qopt_codebook& cb, const std::vector<float>& trans, const char* name) {
  if (trans.size() + 1 != cb.nmag) {
    std::printf("FAIL %s: %zu transitions for %u magnitudes\n", name, trans.size(), cb.nmag);
    ++g_failures;
    return;
  }
  // a runs upward through the bit patterns, so the count of transitions <= a
  // only grows: one pointer walks the sorted transitions.
  size_t below = 0;
  uint64_t bad = 0;
  const uint32_t end = 0x40000000u;  // 2.0f
  for (uint32_t bits = 0; bits < end; ++bits) {
    float a;
    std::memcpy(&a, &bits, 4);
    while (below < trans.size() && trans[below] <= a) ++below;
    const uint32_t got = table_index(cb, bits);
    if (got != below) {
      if (bad < 5) std::printf("FAIL %s: a bits %08x -> index %u, expected %zu\n", name, bits,
                               got, below);
      ++bad;
    }
  }
  if (bad) {
    std::printf("FAIL %s: %" PRIu64 " mismatching binary32 values\n", name, bad);
    ++g_failures;
  }
}

void argument_checks() {
  // pointers below are never dereferenced: every call fails (or finds no work)
  // before any device access
  void* p = reinterpret_cast<void*>(0x1000);
  void* odd = reinterpret_cast<void*>(0x1002);
  auto* pc = static_cast<const qopt_codebook*>(p);
  auto* pf = static_cast<float*>(p);
  auto* pu = static_cast<uint8_t*>(p);

  expect(qopt_codebook_build(0, nullptr), QOPT_EINVAL, "codebook_build(null)");
  qopt_codebook cb;
  expect(qopt_codebook_build(7, &cb), QOPT_EUNSUPPORTED, "codebook_build(kind 7)");

  expect(qopt_quantize_blockwise(nullptr, nullptr, -1, nullptr, nullptr, nullptr), QOPT_EINVAL,
         "quantize n<0");
  expect(qopt_quantize_blockwise(nullptr, nullptr, 0, nullptr, nullptr, nullptr), QOPT_OK,
         "quantize n=0");
  expect(qopt_quantize_blockwise(nullptr, nullptr, 5, nullptr, nullptr, nullptr), QOPT_EINVAL,
         "quantize null");
  expect(qopt_quantize_blockwise(pc, static_cast<const float*>(odd), 5, pu, pf, nullptr),
         QOPT_EALIGN, "quantize misaligned");
  expect(qopt_dequantize_blockwise(nullptr, nullptr, nullptr, -3, nullptr, nullptr), QOPT_EINVAL,
         "dequantize n<0");
  expect(qopt_dequantize_blockwise(nullptr, nullptr, nullptr, 0, nullptr, nullptr), QOPT_OK,
         "dequantize n=0");

  qopt_codec_tensor ct{pf, pu, pf, 10};
  qopt_codec_tensor neg{pf, pu, pf, -1};
  expect(qopt_quantize_blockwise_multi(nullptr, nullptr, 2, nullptr), QOPT_EINVAL,
         "quantize_multi null list");
  expect(qopt_quantize_blockwise_multi(pc, &neg, 1, nullptr), QOPT_EINVAL, "quantize_multi n<0");
  expect(qopt_dequantize_blockwise_multi(nullptr, &ct, 1, nullptr), QOPT_EINVAL,
         "dequantize_multi no codebook");

  const qopt_adam_hparams hp{1e-3f, 0.9f, 0.999f, 1e-8f, 1};
  qopt_tensor t{p, p, pu, pu, pf, pf, 10};
  expect(qopt_adam8bit_step(nullptr, 0, QOPT_F32, QOPT_F32, nullptr, nullptr, &hp, nullptr),
         QOPT_OK, "step no tensors");
  expect(qopt_adam8bit_step(nullptr, 1, QOPT_F32, QOPT_F32, nullptr, nullptr, &hp, nullptr),
         QOPT_EINVAL, "step null list");
  expect(qopt_adam8bit_step(&t, 1, 5, QOPT_F32, pc, pc, &hp, nullptr), QOPT_EUNSUPPORTED,
         "step dtype");
  expect(qopt_adam8bit_step(&t, 1, QOPT_F32, QOPT_F32, pc, pc, nullptr, nullptr), QOPT_EINVAL,
         "step no hparams");
  const qopt_adam_hparams bad_hp[] = {{1e-3f, 0.9f, 0.999f, 1e-8f, 0},
                                      {1e-3f, 1.0f, 0.999f, 1e-8f, 1},
                                      {1e-3f, 0.9f, -0.1f, 1e-8f, 1},
                                      {1e-3f, 0.9f, 0.999f, -1.0f, 1}};
  for (const auto& h : bad_hp)
    expect(qopt_adam8bit_step(&t, 1, QOPT_F32, QOPT_F32, pc, pc, &h, nullptr), QOPT_EINVAL,
           "step bad hparams");
  qopt_tensor mis = t;
  mis.param = odd;
  expect(qopt_adam8bit_step(&mis, 1, QOPT_F32, QOPT_F32, pc, pc, &hp, nullptr), QOPT_EALIGN,
         "step misaligned param");
  int64_t launches = -1;
  expect(qopt_adam8bit_launch_count(&t, 1, QOPT_F32, QOPT_F32, nullptr), QOPT_EINVAL,
         "launch_count null out");
  expect(qopt_adam8bit_launch_count(&t, -1, QOPT_F32, QOPT_F32, &launches), QOPT_EINVAL,
         "launch_count n<0");

  expect(qopt_embedding_xavier_init(nullptr, QOPT_F32, -1, 4, 0, nullptr), QOPT_EINVAL,
         "xavier rows<0");
  expect(qopt_embedding_xavier_init(nullptr, 7, 4, 4, 0, nullptr), QOPT_EUNSUPPORTED,
         "xavier dtype");
  expect(qopt_embedding_xavier_init(nullptr, QOPT_F32, 0, 4, 0, nullptr), QOPT_OK, "xavier empty");
  size_t ws = 99;
  expect(qopt_stable_embedding_backward_workspace(0, 8, &ws), QOPT_OK, "workspace empty");
  if (ws != 0) {
    std::printf("FAIL workspace empty: %zu bytes\n", ws);
    ++g_failures;
  }
  expect(qopt_stable_embedding_backward_workspace(-1, 8, &ws), QOPT_EINVAL, "workspace n<0");
}

// Launch-plan queries: stand-in addresses, 4 KiB-aligned and far apart, never
// dereferenced (the plan only reads sizes and checks alignment).
void plans() {
  std::string line;
  char buf[1 << 16];
  while (std::fgets(buf, sizeof buf, stdin)) {
    line = buf;
    std::istringstream in(line);
    int pdt = 0, gdt = 0;
    if (!(in >> pdt >> gdt)) continue;
    std::vector<qopt_tensor> ts;
    uintptr_t addr = uintptr_t(1) << 40;
    int64_t n = 0;
    while (in >> n) {
      void* a = reinterpret_cast<void*>(addr);
      ts.push_back(qopt_tensor{a, a, static_cast<uint8_t*>(a), static_cast<uint8_t*>(a),
                               static_cast<float*>(a), static_cast<float*>(a), n});
      addr += ((static_cast<uintptr_t>(n < 0 ? 0 : n) + 4095) / 4096) * 4096 * 8 + 4096;
    }
    int64_t launches = -1;
    const int rc = qopt_adam8bit_launch_count(ts.data(), static_cast<int32_t>(ts.size()), pdt,
                                              gdt, &launches);
    std::printf("%d %" PRId64 "\n", rc, launches);
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: %s CODEBOOKS_OUT TRANSITIONS_SIGNED TRANSITIONS_UNSIGNED\n",
                 argv[0]);
    return 2;
  }
  qopt_codebook cbs[2];
  for (int kind = 0; kind < 2; ++kind)
    expect(qopt_codebook_build(kind, &cbs[kind]), QOPT_OK, "codebook_build");
  FILE* f = std::fopen(argv[1], "wb");
  if (!f || std::fwrite(cbs, sizeof cbs, 1, f) != 1) {
    std::printf("FAIL cannot write %s\n", argv[1]);
    return 1;
  }
  std::fclose(f);
  sweep(cbs[0], read_floats(argv[2]), "signed");
  sweep(cbs[1], read_floats(argv[3]), "unsigned");
  argument_checks();
  plans();
  std::printf("checks done, %d failures\n", g_failures);
  return g_failures ? 1 : 0;
}
