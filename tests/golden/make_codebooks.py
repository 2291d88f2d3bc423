"""Write the golden decode tables from the oracle (and nothing else).

    python tests/golden/make_codebooks.py

Each line: code byte, binary32 bit pattern (hex), value.  The values are the
oracle's reading of the dynamic-tree code of the 8-bit optimizers summary page
(§2 "Dynamic Quantization"); the page itself prints no values.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

for kind, name in [(oracle.SIGNED, "codebook_signed.txt"),
                   (oracle.UNSIGNED, "codebook_unsigned.txt")]:
    t = oracle.decode_table(kind)
    with open(os.path.join(HERE, name), "w") as f:
        f.write(f"# {name}: written by make_codebooks.py from oracle.decode_table\n")
        f.write("# code  fp32_bits  value\n")
        for c in range(256):
            f.write(f"0x{c:02x} 0x{int(t.view('uint32')[c]):08x} {float(t[c]):.9g}\n")
