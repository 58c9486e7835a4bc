"""Checks on the gfx950 code the compiler emits for the tile-copy kernels (no GPU needed).

A direct-to-LDS copy takes its LDS base from M0. When the LDS operand reached
the builtin as a pointer to a float vector, the compiler emitted the null LDS
address (M0 = -1) and then dropped every read of the slot as never written;
these tests compile the kernels to assembly and check that every such copy
gets a real base and that no tile kernel spills to scratch memory.

The tile pipelines keep copies in flight across tiles and wait for them only
at each tile's barrier. An LDS read that the compiler cannot tell apart from
a slot a copy is still filling (two ring slots in one LDS object) makes it
insert a full wait for every copy in flight in the middle of the tile, which
silently takes the prefetch away; the last test checks that every wait on
the copies after a copy is issued is the tile barrier's own.
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


_SCALAR_GLUE = re.compile(r"^(s_waitcnt|s_mov|s_cbranch|s_branch|s_nop|s_and|s_or|s_andn2|s_cselect|s_cmp)")


def _waits_before_barrier(body):
    """Full waits on the memory counter (vmcnt(0)) that follow a tile copy
    (global_load_lds) before the next s_barrier and are not part of that
    barrier's own wait (the barrier within a few scalar instructions, labels
    and branches of the wait)."""
    lines = [ln.strip() for ln in body.splitlines()]
    lines = [t for t in lines if t and not t.startswith(";") and not t.startswith(".") or
             re.match(r"^\.LBB", t)]
    bad, copy_seen = [], False
    for i, t in enumerate(lines):
        if t.startswith("s_barrier"):
            copy_seen = False
        elif t.startswith("global_load_lds"):
            copy_seen = True
        elif copy_seen and t.startswith("s_waitcnt") and "vmcnt(0)" in t:
            ok = False
            for u in lines[i + 1:i + 12]:
                if u.startswith("s_barrier"):
                    ok = True
                    break
                if re.match(r"^\.LBB\w+:", u) or _SCALAR_GLUE.match(u):
                    continue
                break
            if not ok:
                bad.append((i, t, lines[i + 1] if i + 1 < len(lines) else ""))
    return bad


TILE_KERNELS = ("bsa_fwd_mfma", "bwd_dq", "bwd_dkv")


@pytest.mark.parametrize("f", ["attention_mfma.hip", "attention_bwd.hip"])
def test_tile_loops_wait_for_copies_only_at_barriers(assembly, f):
    checked = 0
    for name, body in _kernels(assembly[f]):
        if not any(k in name for k in TILE_KERNELS):
            continue
        checked += 1
        bad = _waits_before_barrier(body)
        assert not bad, f"{name}: waits on the copies in flight inside a tile: {bad[:3]}"
    assert checked > 0
