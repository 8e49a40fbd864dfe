"""Source-level rules for the HIP kernels, checked on the CPU.

The ROCm 7.2 device compiler lowers a bit cast whose operand is a subscripted element of a vector
(`__builtin_bit_cast(float, a[1])` with `a` an ext_vector or vector_size type) to a load of the
vector's first element, whatever the subscript. Two reductions once lost three quarters of their
inputs that way (the matrix-core decode kernel's maximum over key groups and the prefill kernel's
FP16 overflow test). The kernels therefore bit-cast whole vectors or named scalars only; this test
keeps any subscripted operand out of the sources.
"""

import pathlib
import re

CSRC = pathlib.Path(__file__).resolve().parents[1] / "paged_kv_cache_pages_amd" / "csrc"
# __builtin_bit_cast(<type>, <name>[...]...) with nothing after the subscripts: the operand is an
# element lvalue.  Expressions such as `x[i] << 16` are prvalues and compile correctly.
PATTERN = re.compile(r"__builtin_bit_cast\(\s*[\w:<> ]+,\s*[\w.]+(\s*\[[^\]]*\])+\s*\)")


def test_no_bit_cast_of_a_subscripted_element():
    sources = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.h"))
    assert sources
    hits = []
    for path in sources:
        for n, line in enumerate(path.read_text().splitlines(), 1):
            if PATTERN.search(line):
                hits.append(f"{path.name}:{n}: {line.strip()}")
    assert not hits, "bit cast of a subscripted element:\n" + "\n".join(hits)


def test_the_rule_catches_the_pattern():
    assert PATTERN.search("x = fmax(__builtin_bit_cast(float, a[0]), __builtin_bit_cast(float, a[1]));")
    assert PATTERN.search("w = __builtin_bit_cast(u16x2, pw[sub][hs][e]);")
    assert not PATTERN.search("const float lo = __builtin_bit_cast(float, x[i] << 16);")
    assert not PATTERN.search("const f2_t a = __builtin_bit_cast(f2_t, swapped);")
