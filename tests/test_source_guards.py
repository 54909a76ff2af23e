"""Source checks of the HIP library that need no GPU.

hipcc (clang) compiles ``__builtin_bit_cast(T, v[i])``, where ``v`` is an
ext-vector value and ``v[i]`` one of its elements, as a read of element 0
for every i: the cast takes the element's address, which is the vector's.
A packed-fp16 scale splat and an fp16 staging rescale written that way both
gave wrong results on the GPU.  The kernels read such an element into a
scalar first; this check keeps the pattern out of the sources.  A host build
of the same cast shows the behaviour: casting the elements of
{0x11111111, 0x22222222, 0x33333333, 0x44444444} returns 0x11111111 four
times, while a copy through a uint32_t returns each element.
"""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "expert_grouped_quantized_amd", "csrc")
# a bit_cast whose whole operand is an indexed element: bit_cast(T, name[...])
ELEMENT_CAST = re.compile(r"__builtin_bit_cast\(\s*[\w:<> ]+,\s*[\w.>-]+\s*\[[^\]]*\]\s*\)")


def _sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip", ".cpp")):
            yield name, open(os.path.join(CSRC, name)).read()


def test_no_bit_cast_of_an_indexed_element():
    hits = []
    for name, text in _sources():
        for no, line in enumerate(text.splitlines(), 1):
            if ELEMENT_CAST.search(line):
                hits.append(f"{name}:{no}: {line.strip()}")
    assert not hits, "bit_cast of an indexed element (read it into a scalar first):\n" + "\n".join(hits)


@pytest.mark.parametrize("line,flagged", [
    ("r = __builtin_bit_cast(f16x2_t, v[w]) * f2;", True),
    ("const f16x2_t t = __builtin_bit_cast(f16x2_t, sc[si >> 1]);", True),
    ("const uint32_t e = v[w]; x = __builtin_bit_cast(f16x2_t, e);", False),
    ("r[j] = __builtin_bit_cast(uint32_t, (t0 + off) * s2);", False),
    ("r[j] = __builtin_bit_cast(uint32_t, c[j] * s2);", False),
])
def test_the_pattern_itself(line, flagged):
    assert bool(ELEMENT_CAST.search(line)) == flagged
