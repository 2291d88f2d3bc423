"""ctypes binding of libqopt.so (include/qopt.h): argument marshalling only.

Every step of the quantizer and of the optimizer runs in the library's HIP kernels;
torch only provides device memory and the current stream.  torch is imported before
the library is opened so that libqopt binds to the HIP runtime torch already loaded
(one runtime per process, so torch's streams and pointers are valid for it).
"""

import ctypes
import os
import re

import torch  # noqa: F401  (must be loaded before libqopt.so; see module docstring)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqopt.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "qopt.h")
EMB_HEADER = os.path.join(os.path.dirname(_HERE), "include", "qopt_embedding.h")

QOPT_BLOCK = 2048
(QOPT_OK, QOPT_EINVAL, QOPT_EUNSUPPORTED, QOPT_EALIGN, QOPT_ELAUNCH, QOPT_EINTERNAL,
 QOPT_ENOSPACE) = range(7)
QOPT_CB_SIGNED, QOPT_CB_UNSIGNED = 0, 1
QOPT_F32, QOPT_BF16 = 0, 1
QOPT_CODEBOOK_MAGIC = 0x31424351
QOPT_MAX_BUCKETS = 7168
QOPT_THRESH_LEN = 272
QOPT_EMB_VEC_MAX_DIM = 4096
QOPT_EMB_STATIC_SCRATCH_BYTES = 64 << 20


class QoptError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


class qopt_codebook(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("kind", ctypes.c_uint32),
        ("sign_mask", ctypes.c_uint32),
        ("nmag", ctypes.c_uint32),
        ("key0", ctypes.c_uint32),
        ("nbuckets", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32 * 2),
        ("decode", ctypes.c_float * 256),
        ("thresh", ctypes.c_float * QOPT_THRESH_LEN),
        ("bucket", ctypes.c_uint8 * QOPT_MAX_BUCKETS),
    ]


class qopt_tensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("m_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("m_absmax", ctypes.c_void_p),
        ("v_absmax", ctypes.c_void_p),
        ("n", ctypes.c_int64),
    ]


class qopt_codec_tensor(ctypes.Structure):
    _fields_ = [
        ("values", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("n", ctypes.c_int64),
    ]


class qopt_adam_hparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("step", ctypes.c_int64),
    ]


_SIGNATURES = {
    "qopt_codebook_build": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(qopt_codebook)]),
    "qopt_quantize_blockwise": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "qopt_dequantize_blockwise": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_int64,
                                                 ctypes.c_void_p, ctypes.c_void_p]),
    "qopt_quantize_blockwise_multi": (ctypes.c_int, [ctypes.c_void_p,
                                                     ctypes.POINTER(qopt_codec_tensor),
                                                     ctypes.c_int32, ctypes.c_void_p]),
    "qopt_dequantize_blockwise_multi": (ctypes.c_int, [ctypes.c_void_p,
                                                       ctypes.POINTER(qopt_codec_tensor),
                                                       ctypes.c_int32, ctypes.c_void_p]),
    "qopt_adam8bit_step": (ctypes.c_int, [ctypes.POINTER(qopt_tensor), ctypes.c_int32,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.POINTER(qopt_adam_hparams),
                                          ctypes.c_void_p]),
    "qopt_adam8bit_launch_count": (ctypes.c_int, [ctypes.POINTER(qopt_tensor), ctypes.c_int32,
                                                  ctypes.c_int, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_int64)]),
    "qopt_adam8bit_traffic_probe": (ctypes.c_int, [ctypes.POINTER(qopt_tensor), ctypes.c_int32,
                                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "qopt_embedding_xavier_init": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_uint64,
                                                  ctypes.c_void_p]),
    "qopt_stable_embedding_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                                     ctypes.c_int64, ctypes.c_void_p,
                                                     ctypes.c_int64, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_float,
                                                     ctypes.c_void_p, ctypes.c_int,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_void_p]),
    "qopt_stable_embedding_backward_workspace": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64,
                                                                ctypes.POINTER(ctypes.c_size_t)]),
    "qopt_stable_embedding_backward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                                      ctypes.c_int64, ctypes.c_int64,
                                                      ctypes.c_void_p, ctypes.c_int64,
                                                      ctypes.c_void_p, ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_void_p,
                                                      ctypes.c_int, ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_size_t,
                                                      ctypes.c_void_p]),
    "qopt_stable_embedding_backward_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                                              ctypes.c_int64, ctypes.c_int64,
                                                              ctypes.c_void_p, ctypes.c_int64,
                                                              ctypes.c_void_p, ctypes.c_void_p,
                                                              ctypes.c_void_p, ctypes.c_void_p,
                                                              ctypes.c_int, ctypes.c_void_p,
                                                              ctypes.c_void_p, ctypes.c_void_p,
                                                              ctypes.c_void_p]),
    "qopt_pattern_probe_count": (ctypes.c_int, []),
    "qopt_pattern_probe_name": (ctypes.c_char_p, [ctypes.c_int]),
    "qopt_pattern_probe": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p]),
    "qopt_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qopt_version": (ctypes.c_int, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python block_wise_bit_adam8bit_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def header_constants(paths=(HEADER, EMB_HEADER)):
    """#define values of include/*.h (used by tests to check this mirror)."""
    out = {}
    for path in paths:
        for m in re.finditer(r"#define\s+(QOPT_\w+)\s+(0x[0-9a-fA-F]+|\d+)u?", open(path).read()):
            out[m.group(1)] = int(m.group(2), 0)
    return out


def status_string(status):
    return LIB.qopt_status_string(int(status)).decode()


def check(fn, status):
    if status != QOPT_OK:
        raise QoptError(fn, status)


def stream_handle(device=None):
    """hipStream_t of torch's current stream on ``device`` (as an int)."""
    return torch.cuda.current_stream(device).cuda_stream
