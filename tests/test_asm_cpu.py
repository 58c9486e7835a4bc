"""Checks on the gfx950 code the compiler emits for the tile-copy kernels (no GPU needed).

A direct-to-LDS copy takes its LDS base from M0. When the LDS operand reached
the builtin as a pointer to a float vector, the compiler emitted the null LDS
address (M0 = -1) and then dropped every read of the slot as never written;
these tests compile the kernels to assembly and check that every such copy
gets a real base and that no tile kernel spills to scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

import importlib.util as _iu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = _iu.spec_from_file_location(
    "_cabf_build", os.path.join(ROOT, "content_adaptive_block_fractal_amd", "build.py"))
build = _iu.module_from_spec(_spec)
_spec.loader.exec_module(build)

FILES = ["attention_mfma.hip", "attention_pair.hip", "attention_bwd.hip"]


def _have_hipcc() -> bool:
    try:
        return os.path.exists(build._hipcc()) or shutil.which(build._hipcc()) is not None
    except Exception:
        return False


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not _have_hipcc():
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for f in FILES:
        s = str(d / (f + ".s"))
        cmd = [build._hipcc(), *build.FLAGS, "-x", "hip", "-S", "--offload-device-only",
               os.path.join(build.CSRC, f), "-o", s]
        subprocess.run(cmd, check=True, capture_output=True)
        with open(s) as fh:
            out[f] = fh.read()
    return out


def _kernels(text):
    """(name, body) of every kernel in an assembly file: from its symbol to its
    .Lfunc_end label, so every basic block (all exits included) is covered."""
    pat = re.compile(r"^(_Z[^\s:]+):.*?$(.*?)^\.Lfunc_end\d+:", flags=re.M | re.S)
    return [(m.group(1), m.group(2)) for m in pat.finditer(text)]


@pytest.mark.parametrize("f", FILES)
def test_lds_copies_get_a_real_base(assembly, f):
    kernels = _kernels(assembly[f])
    assert kernels, f"{f}: no kernels found in the assembly"
    copies = 0
    for name, body in kernels:
        m0 = None
        for ln in body.splitlines():
            t = ln.strip()
            if re.match(r"^[.\w]+:", t):
                m0 = None           # a label starts a basic block: M0 must be set inside it
            if re.match(r"s_\w+\s+m0,", t):
                m0 = t
            if t.startswith("global_load_lds"):
                copies += 1
                assert m0 is not None, f"{name}: LDS copy without an M0 write in its block"
                assert not re.match(r"s_mov_b32\s+m0,\s*-1\b", m0), f"{name}: null LDS base ({m0})"
    assert copies > 0, f"{f}: no LDS copies found"


@pytest.mark.parametrize("f", FILES)
def test_tile_kernels_do_not_spill(assembly, f):
    text = assembly[f]
    for m in re.finditer(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", text, flags=re.M):
        assert int(m.group(1)) == 0, f"{f}: a kernel uses {m.group(1)} bytes of scratch per lane"
