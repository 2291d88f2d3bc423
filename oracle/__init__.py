"""Plain CPU oracle for block-wise dynamic-tree 8-bit Adam.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``block_wise_bit_adam8bit_amd`` and its HIP library) never calls it,
and this package shares no code, tables or constants with that path.

Source of the method: the Chinese summary page of "8-BIT OPTIMIZERS VIA
BLOCK-WISE QUANTIZATION" (ICLR 2022), wiki.neutronadmin.com/news/16836.  Citations
below use its section headings:

* §1 "when the optimizer meets quantization" -- Adam keeps a first moment (mean of
  the gradients) and a second moment (uncentred variance); quantization maps fp32 to
  fewer bits after normalising into a range, dequantization maps back.
* §2 "three methods" -- the state lives in low precision and is dequantized for the
  update, then stored low precision again.
  - §2 "Block-wise Quantization": blocks of 2048 elements, each normalised into
    [-1, 1] by its own absolute maximum, independently of every other block.
  - §2 "Dynamic Quantization": the dynamic-tree code (sign bit, exponent written as a
    run of zeros, an indicator bit, a linear fraction) and its unsigned variant for
    the always-positive second moment, whose sign bit extends the fraction.

Where the page is silent, the readings are fixed here and listed in each module's
docstring.  Parity status of every function is stated in its docstring: "pinned"
means a ``-m "not gpu"`` test checks it against something other than itself.

The Stable Embedding layer of the same page (§2 "Stable Embedding Layer") has its
own module, ``oracle.embedding``: Xavier-uniform initialisation from a counter-based
generator, and LayerNorm after the lookup, forward and backward, in binary64.

Arithmetic precision: the codes are integers decided by fp32 arithmetic, so every
step that feeds a code decision (the moments, the block absmax, the normalisation)
is evaluated in IEEE binary32, one rounding per operation, in the order written in
``adam8bit.py``.  numpy float32 ufuncs round each operation and never fuse.
"""

from .codebook import (  # noqa: F401
    BLOCK,
    SIGNED,
    UNSIGNED,
    magnitude_rationals,
    magnitudes_f32,
    decode_table,
    round_rational_to_f32,
)
from .blockwise import (  # noqa: F401
    nearest_magnitude_index,
    nearest_magnitude_index_bruteforce,
    quantize_blockwise,
    dequantize_blockwise,
    code_transitions,
)
from .adam8bit import (  # noqa: F401
    adam_scalars,
    adam8bit_step,
    adam8bit_step_multi,
    adam_update_f64,
    bf16_to_f32,
    f32_to_bf16_rne,
)
