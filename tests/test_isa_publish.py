"""Build-time check of the in-launch hand-off in fused down+combine, on the AMD
assembly of this repository's own build (gfx950).

The fused kernel publishes its y rows and split-k partial tiles to other
workgroups of the same launch without a release fence: the data are written
with agent-scope relaxed atomic stores, the publishing wave waits until they
have completed (s_waitcnt vmcnt(0)), then bumps a counter; a reader polls the
counter with agent-scope relaxed loads and takes one agent-scope acquire
before it reads.  That is correct only if the compiler emits the stores with
the sc1 bit (agent-scope coherent: written through the XCD's L2) and the
acquire as an L2 invalidate (buffer_inv sc1), the code sequences of the LLVM
AMDGPU memory model for GFX942-class targets.  This test compiles fused.hip
to assembly and checks exactly that, so a compiler or source change that
drops them fails here, on the CPU.  The one-launch backward, which hands its
activation gradient over with a real release, is checked for the L2
write-back that the release implies.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_moe_route_histogram_amd", "csrc")


def _asm(src, tmp_path):
    from combine_moe_route_histogram_amd import build as B
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    flags = [f for f in B.COMMON_FLAGS if f != "-fPIC"]
    r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _functions(asm, name_part):
    """Bodies of the kernels whose mangled name contains name_part."""
    bodies = []
    for m in re.finditer(r"^(_Z\S*" + name_part + r"\S*):", asm, flags=re.M):
        start = m.end()
        end = asm.find("s_endpgm", start)
        assert end > 0
        bodies.append(asm[start:end])
    return bodies


def test_fused_combine_publishes_with_coherent_stores(tmp_path):
    asm = _asm("fused.hip", tmp_path)
    bodies = _functions(asm, "ffn_combine_kernel")
    assert len(bodies) == 2                       # ragged-k and whole-slice instantiations
    for body in bodies:
        stores = re.findall(r"^\s*global_store_dwordx2\b.*$", body, flags=re.M)
        # the y rows and the split-k partials: 8-byte stores, every one agent-coherent
        assert len(stores) >= 32
        assert all(re.search(r"\bsc1\b", s) for s in stores), [s for s in stores if "sc1" not in s][:3]
        # the readers' acquire: invalidate the XCD's L2 (and L1)
        assert re.search(r"^\s*buffer_inv\s+sc1\b", body, flags=re.M)
        # the publish waits for all of its stores before the counter update
        pub = re.search(r"s_waitcnt vmcnt\(0\)(?:(?!s_waitcnt vmcnt).)*?global_atomic_add", body, flags=re.S)
        assert pub, "no vmcnt(0) wait ahead of a counter update"
        # the counters are polled with agent-scope loads
        assert re.search(r"^\s*global_load_dword\b.*\bsc1\b", body, flags=re.M)


def test_one_launch_backward_releases_phase_one(tmp_path):
    asm = _asm("bwd.hip", tmp_path)
    bodies = _functions(asm, "ffn_bwd_kernel")
    assert len(bodies) == 2
    for body in bodies:
        assert re.search(r"^\s*buffer_wbl2\b", body, flags=re.M)     # agent-scope release
        assert re.search(r"^\s*buffer_inv\s+sc1\b", body, flags=re.M)  # agent-scope acquire
