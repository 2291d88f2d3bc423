"""block_wise_bit_adam8bit_amd: block-wise dynamic-tree 8-bit Adam for MI355X.

The compute lives in libqopt.so (HIP kernels for gfx950 behind the C ABI of
include/qopt.h, include/qopt_embedding.h); this package is its thin Python binding
plus a torch optimizer and the Stable Embedding module.
Importing it loads the library and fails with ImportError if it is not built.
"""

from ._lib import (  # noqa: F401
    LIB, LIB_PATH, QOPT_BLOCK, QoptError, status_string,
    QOPT_OK, QOPT_EINVAL, QOPT_EUNSUPPORTED, QOPT_EALIGN, QOPT_ELAUNCH, QOPT_EINTERNAL,
    QOPT_ENOSPACE,
    QOPT_CB_SIGNED, QOPT_CB_UNSIGNED, QOPT_F32, QOPT_BF16,
)
from .functional import (  # noqa: F401
    SIGNED, UNSIGNED, nblocks, codebook, codebook_bytes, qopt_codebook_build,
    qopt_quantize_blockwise, qopt_dequantize_blockwise, qopt_adam8bit_step,
    qopt_adam8bit_launch_count, qopt_adam8bit_traffic_probe, qopt_quantize_blockwise_multi,
    qopt_dequantize_blockwise_multi, make_tensor_array, qopt_pattern_probe,
    qopt_pattern_probe_names,
)
from .checkpoint import (  # noqa: F401
    compress_moments, decompress_moments, compress_moments_multi, decompress_moments_multi,
)
from .optim import Adam8bit  # noqa: F401
from .embedding import (  # noqa: F401
    StableEmbedding, StableEmbeddingFunction, qopt_embedding_xavier_init,
    qopt_stable_embedding_forward, qopt_stable_embedding_backward,
)

__version__ = "0.1.0"
