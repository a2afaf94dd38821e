"""Build guards (CPU): properties of the compiled gfx950 code that the
kernels rely on and that a compiler change could break silently.

The FP8 attention kernel issues its LDS DMA from inline asm that writes M0
(the LDS base register the transfer reads) right before each transfer (the
other kernels use the compiler's own LDS-DMA builtin, whose M0 the compiler
manages). That is correct only while no compiler-generated code in the kernel
keeps a value in M0 across the asm, or reads M0 at all. This test compiles
the source to assembly and checks that every instruction naming M0 is one of
the asm's own writes, immediately followed by its wait state and its
transfer, that every LDS DMA has such a write in front of it, and that no
instruction that reads M0 implicitly appears.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mla_long_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# mnemonic prefixes that read M0 without naming it in the text
IMPLICIT_M0 = ("s_movrel", "v_movrel", "s_sendmsg", "ds_gws", "ds_append", "ds_consume",
               "s_set_gpr_idx", "v_interp", "ds_read_addtid", "ds_write_addtid", "buffer_load_lds",
               "s_buffer_load_lds")


def _asm(src, tmp_path):
    """The source's gfx950 assembly, compiled with the library's own flags."""
    import sys
    sys.path.insert(0, ROOT)
    from sparse_mla_long_amd import build
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in build.compile_flags(os.path.basename(src)) if f != "-fPIC"]
    subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(out)],
                   check=True, capture_output=True, text=True)
    return out.read_text().split("\n")


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
@pytest.mark.parametrize("src", ["attention_f8.hip"])
def test_m0_is_written_only_by_the_lds_dma_asm(src, tmp_path):
    lines = [l.split(";")[0].strip() for l in _asm(os.path.join(CSRC, src), tmp_path)]
    code = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    ours = 0
    for i, ins in enumerate(code):
        op = ins.split()[0]
        assert not op.startswith(IMPLICIT_M0), "%s: %s reads M0" % (src, ins)
        if op.startswith("global_load_lds"):
            # every LDS DMA comes right after its M0 write and wait state
            assert code[i - 2].startswith("s_mov_b32 m0,") and code[i - 1] == "s_nop 0", \
                "%s: LDS DMA without its own M0 write: %s" % (src, code[i - 2:i + 1])
        if re.search(r"\bm0\b", ins):
            assert ins.startswith("s_mov_b32 m0,") and code[i + 1] == "s_nop 0" and \
                code[i + 2].startswith("global_load_lds"), "%s: M0 used elsewhere: %s" % (src, ins)
            ours += 1
    assert ours > 0
