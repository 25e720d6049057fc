"""Host-side checks of source forms that gfx950 code generation got wrong. No
matrix-core product accumulates onto the result of a product of another shape within
the wait states that gfx950 needs between them (the rule and its measurement are in
tests/mfma_chain_check.py; compiles every kernel source to assembly with the library's
own flags, needs hipcc), and no kernel bit-casts one element of a vector."""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from kimi_delta_attention_k1_amd import build as kbuild
from tests.mfma_chain_check import MIN_WAIT, check_asm

SELF_GOOD = """
_Zk:
\tv_mfma_f32_16x16x32_bf16 v[10:13], v[2:5], v[6:9], v[10:13]
\ts_nop 5
\tv_mfma_f32_16x16x16_bf16 v[10:13], v[14:15], v[16:17], v[10:13]
\tv_mfma_f32_16x16x32_bf16 v[20:23], v[2:5], v[6:9], v[20:23]
\tv_mfma_f32_16x16x32_bf16 v[20:23], v[2:5], v[6:9], v[20:23]
\tv_mfma_f32_16x16x16_bf16 v[30:33], v[14:15], v[16:17], 0
\tv_mfma_f32_16x16x32_bf16 v[40:43], v[2:5], v[6:9], v[40:43]
\tv_mfma_f32_16x16x32_bf16 v[44:47], v[2:5], v[6:9], v[44:47]
\tv_mfma_f32_16x16x32_bf16 v[48:51], v[2:5], v[6:9], v[48:51]
\tv_mfma_f32_16x16x16_bf16 v[40:43], v[14:15], v[16:17], v[40:43]
\ts_endpgm
"""

# the forms the probe measured wrong, written as straight-line code and across a loop
SELF_BAD = [
    "_Zk:\n\tv_mfma_f32_16x16x32_bf16 v[10:13], v[2:5], v[6:9], v[10:13]\n"
    "\tv_mfma_f32_16x16x16_bf16 v[10:13], v[14:15], v[16:17], v[10:13]\n\ts_endpgm\n",
    "_Zk:\n\tv_mfma_f32_16x16x16_bf16 v[58:61], v[100:101], v[78:79], v[58:61]\n\tv_add_u32_e32 v1, 0x5800, v1\n"
    "\tv_mfma_f32_16x16x32_bf16 v[58:61], v[90:93], v[70:73], v[58:61]\n\ts_endpgm\n",
    "_Zk:\n\tv_mfma_f32_16x16x32_bf16 v[10:13], v[2:5], v[6:9], v[10:13]\n\ts_nop 3\n"
    "\tv_mfma_f32_16x16x16_bf16 v[10:13], v[14:15], v[16:17], v[10:13]\n\ts_endpgm\n",
    "_Zk:\n.LBB0_1:\n\tv_mfma_f32_16x16x16_bf16 v[10:13], v[14:15], v[16:17], v[10:13]\n\ts_nop 7\n"
    "\tv_mfma_f32_16x16x32_bf16 v[10:13], v[2:5], v[6:9], v[10:13]\n\ts_add_i32 s0, s0, -1\n"
    "\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n",
]


def test_checker_flags_the_measured_forms():
    assert check_asm(SELF_GOOD) == []
    for i, asm in enumerate(SELF_BAD):
        assert check_asm(asm), f"case {i} not flagged"


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [kbuild.hipcc()] + [a for a in kbuild.COMMON if a != "-fPIC"] + [
        "--cuda-device-only", "-S", os.path.join(kbuild.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr[-2000:]}")
    with open(out) as f:
        return f.read()


def test_no_mixed_shape_chain_in_generated_code():
    try:
        kbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        with cf.ThreadPoolExecutor(len(kbuild.SOURCES)) as ex:
            texts = dict(zip(kbuild.SOURCES, ex.map(lambda s: _asm(s, d), kbuild.SOURCES)))
    problems = []
    n_mfma = 0
    for src, asm in texts.items():
        n_mfma += asm.count("v_mfma")
        for fn, reader, writer, wait in check_asm(asm):
            problems.append(f"{src} {fn[:60]}: '{writer}' then '{reader}' after {wait} wait states")
    assert n_mfma > 100  # the kernels were compiled and parsed
    assert not problems, f"mixed-shape MFMA chains closer than {MIN_WAIT} wait states:\n" + "\n".join(problems[:20])


# ROCm 7.2.0's hipcc compiled __builtin_bit_cast(uint16_t, v[r]) on a bf16 vector v to
# element 0 for every r; the kernels reinterpret whole vectors and index the result
_BIT_CAST_OF_ELEMENT = re.compile(r"__builtin_bit_cast\s*\([^,()]+,\s*[A-Za-z_][\w.]*\s*\[")


def test_checker_flags_an_element_bit_cast():
    assert _BIT_CAST_OF_ELEMENT.search("d[0] = __builtin_bit_cast(uint16_t, hi[r]);")
    assert not _BIT_CAST_OF_ELEMENT.search("const i16x4 hb = __builtin_bit_cast(i16x4, hi);")
    assert not _BIT_CAST_OF_ELEMENT.search("x = __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));")


def test_no_bit_cast_of_a_vector_element():
    bad = []
    for src in sorted(os.listdir(kbuild.CSRC)):
        if src.endswith((".hip", ".h")):
            with open(os.path.join(kbuild.CSRC, src)) as f:
                for i, line in enumerate(f, 1):
                    if _BIT_CAST_OF_ELEMENT.search(line):
                        bad.append(f"{src}:{i}: {line.strip()}")
    assert not bad, "bit cast of a vector element:\n" + "\n".join(bad)
