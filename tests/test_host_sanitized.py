"""libqopt's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Compiles the library's sources together with tests/host_sanitized_driver.cpp into one
executable. The sanitizers are on its host side only, and every UB report is fatal.
The executable runs without a GPU and makes no device call. Checked here:

- The sanitized codebook builder writes the same bytes as the shipped library's.
- Its tables give, for every binary32 in [0, 2), the code index that the oracle's
  transitions fix.
- The argument checks of every device entry point return their documented statuses.
- The host launch planner gives the shipped library's launch counts on the
  workloads' tensor lists and on seeded random ones.
"""

import ctypes
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle

qopt = pytest.importorskip("block_wise_bit_adam8bit_amd")
from block_wise_bit_adam8bit_amd import _lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_wise_bit_adam8bit_amd", "csrc")
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# each sanitizer flag behind -Xarch_host: the device code is built as usual, unsanitized
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["-std=c++17", "-O2", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
         "-I", os.path.join(ROOT, "include"), *SAN]
DEVICE = ["-x", "hip", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("sanitized")
    units = [(["-x", "c++"], os.path.join(CSRC, "codebook.cpp")),
             (["-x", "c++"], os.path.join(ROOT, "tests", "host_sanitized_driver.cpp")),
             (DEVICE, os.path.join(CSRC, "qopt_kernels.hip")),
             (DEVICE, os.path.join(CSRC, "stable_embedding.hip"))]

    def compile_one(i):
        lang, src = units[i]
        obj = str(d / f"u{i}.o")
        r = subprocess.run([HIPCC, *lang, *FLAGS, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(len(units)) as ex:
        objs = list(ex.map(compile_one, range(len(units))))
    exe = str(d / "host_sanitized_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    for kind, name in ((oracle.SIGNED, "signed"), (oracle.UNSIGNED, "unsigned")):
        oracle.code_transitions(kind).astype("<f4").tofile(str(d / f"transitions_{name}.bin"))
    return exe, d


def _workload_queries():
    import workloads
    lines = []
    for shapes in ("llama7b_shapes", "gpt1p3b_shapes"):
        sizes = [n for _, n in getattr(workloads, shapes)()]
        for pdt in (0, 1):
            for gdt in (0, 1):
                lines.append((pdt, gdt, sizes))
    rng = np.random.default_rng(11)
    for _ in range(40):
        k = int(rng.integers(1, 400))
        # mixed magnitudes: empty, ragged, one block, many blocks
        sizes = (10 ** rng.uniform(0, 9, k)).astype(np.int64)
        sizes[rng.random(k) < 0.1] = 0
        lines.append((int(rng.integers(0, 2)), int(rng.integers(0, 2)), sizes.tolist()))
    lines.append((0, 0, [3] * 1000))
    lines.append((1, 1, [20_000_000_000]))
    lines.append((0, 0, []))
    lines.append((0, 0, [10, -1]))        # negative size: refused
    lines.append((0, 5, [10]))            # unknown grad dtype: refused
    return lines


def _library_launch_count(pdt, gdt, sizes):
    T = _lib.qopt_tensor
    arr = (T * max(len(sizes), 1))()
    off = 1 << 40
    for i, n in enumerate(sizes):
        arr[i] = T(off, off, off, off, off, off, n)   # never dereferenced
        off += ((max(n, 0) + 4095) // 4096) * 4096 * 8 + 4096
    out = ctypes.c_int64(-1)
    rc = qopt.LIB.qopt_adam8bit_launch_count(arr, len(sizes), pdt, gdt, ctypes.byref(out))
    return rc, out.value


def test_host_code_under_sanitizers(driver):
    exe, d = driver
    queries = _workload_queries()
    stdin = "".join(f"{p} {g} {' '.join(map(str, s))}\n" for p, g, s in queries)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    cb_path = d / "codebooks.bin"
    r = subprocess.run([exe, str(cb_path), str(d / "transitions_signed.bin"),
                        str(d / "transitions_unsigned.bin")], input=stdin, capture_output=True,
                       text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    lines = r.stdout.splitlines()
    assert lines[-1] == "checks done, 0 failures"

    # the sanitized builder's bytes are the shipped library's
    raw = cb_path.read_bytes()
    size = ctypes.sizeof(_lib.qopt_codebook)
    assert len(raw) == 2 * size
    for kind in (oracle.SIGNED, oracle.UNSIGNED):
        assert raw[kind * size:(kind + 1) * size] == bytes(qopt.qopt_codebook_build(kind))

    # the sanitized planner's launch counts are the shipped library's
    got = [tuple(int(v) for v in ln.split()) for ln in lines[:-1]]
    want = []
    for p, g, s in queries:
        rc, n = _library_launch_count(p, g, s)
        want.append((rc, n if rc == 0 else -1))
    got = [(rc, n if rc == 0 else -1) for rc, n in got]
    assert got == want
    assert want[0] == (0, 13)                          # the Llama-7B set: thirteen launches
    assert want[-2][0] == qopt.QOPT_EINVAL and want[-1][0] == qopt.QOPT_EUNSUPPORTED


PLANTED = {
    "heap_overflow": ("#include <cstdlib>\n"
                      "int main(int argc, char**) { int* a = (int*)std::malloc(4 * sizeof(int));\n"
                      "  int r = a[argc + 3]; std::free(a); return r == 12345; }\n",
                      "heap-buffer-overflow"),
    "signed_overflow": ("#include <climits>\n"
                        "int main(int argc, char**) { int x = INT_MAX - 1 + argc; return x + argc > 0; }\n",
                        "signed integer overflow"),
}


@pytest.mark.parametrize("case", sorted(PLANTED))
def test_sanitizer_flags_catch_a_planted_error(case, tmp_path):
    """The flags above do instrument host code: a planted heap overflow and a planted
    signed overflow each end the program with the sanitizer's report."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    src, report = PLANTED[case]
    (tmp_path / "planted.cpp").write_text(src)
    exe = str(tmp_path / "planted")
    r = subprocess.run([HIPCC, "-x", "c++", *FLAGS, str(tmp_path / "planted.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]
