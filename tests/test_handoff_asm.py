"""The cross-workgroup hand-offs carry no release/acquire fence; check the code they rely on.

Two places pass fp32 sums between workgroups within one launch: the contraction slices
of the streaming kernel (k_stream.hip: every slice parks its sums, the last to arrive adds
them) and the split last round of the prefill GEMMs (k_gemm.hip, and k_tiled.hip that serves the
grouped experts: two contraction halves of a tile, the second to arrive adds the first's).  Both use relaxed agent-scope atomics only.
Under the language memory model a relaxed counter orders nothing, so the correctness
argument rests on the code the compiler emits for gfx950, and this file checks exactly
that code (the AMD assembly of this repository's own kernels, built here):

  1. the parked sums are written with stores carrying the sc1 bit (agent-scope atomic
     stores: written through the XCD's L2 to the device coherence point);
  2. between the last of those stores and the arrival counter's atomic add there is an
     ``s_waitcnt`` with ``vmcnt(0)`` (the stores are acknowledged at the coherence point
     before the workgroup counts itself in) and an ``s_barrier`` (every wave has drained
     before thread 0 counts in);
  3. the arrival counter is a returning atomic add (the arrival order comes back);
  4. after it, every load from global memory into registers carries sc1 (agent-scope atomic loads: read
     at the coherence point, never from a stale line of the reader's own L2), and the
     counter is reset with an sc1 store.

With 1-4 a workgroup that sees the final count issues its loads after every slice's
sums are in device-coherent memory, and those loads bypass the non-coherent per-XCD L2.
"""
import os
import re
import subprocess

import pytest

from tensor_mlp_shard_amd import build as B

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "tensor_mlp_shard_amd", "csrc")

pytestmark = pytest.mark.skipif(
    not (os.path.exists("/opt/rocm/bin/hipcc") or __import__("shutil").which("hipcc")),
    reason="hipcc not available")


def _device_asm(src, out_dir):
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [B.hipcc()] + B.HIP_FLAGS + ["--cuda-device-only", "-S", "-x", "hip",
                                       os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _kernels(asm, prefix):
    """{mangled name: list of instruction lines} for the kernels whose names start with prefix."""
    res = {}
    for m in re.finditer(r"^(%s\S*):" % re.escape(prefix), asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        lines = [l.split(";")[0].strip() for l in asm[m.end():end].splitlines()]
        res[m.group(1)] = [l for l in lines if l and not l.startswith(".")]
    return res


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm"))
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(3) as ex:
        ks, kg, kt = ex.map(lambda s: _device_asm(s, d), ["k_stream.hip", "k_gemm.hip", "k_tiled.hip"])
    return {"k_stream": _kernels(ks, "_ZN3tpm8k_stream"), "k_gemm": _kernels(kg, "_ZN3tpm6k_gemm"),
            "k_tiled": _kernels(kt, "_ZN3tpm7k_tiled")}


def _arrival(lines):
    """Index of the arrival counter: the kernel's returning (sc0) global atomic add."""
    idx = [i for i, l in enumerate(lines) if re.match(r"global_atomic_add(_u32)?\s", l) and
           re.search(r"\bsc0\b", l)]
    return idx


def _check_handoff(name, lines, store_op):
    arr = _arrival(lines)
    assert len(arr) == 1, "%s: expected one returning counter atomic, found %d" % (name, len(arr))
    a = arr[0]
    parks = [i for i in range(a) if lines[i].startswith(store_op + " ") and re.search(r"\bsc1\b", lines[i])]
    assert parks, "%s: no sc1 store of the parked sums before the arrival" % name
    last = parks[-1]
    between = lines[last + 1:a]
    assert any(l.startswith("s_waitcnt") and "vmcnt(0)" in l for l in between), \
        "%s: no s_waitcnt vmcnt(0) between the parked stores and the arrival counter" % name
    assert any(l.startswith("s_barrier") for l in between), \
        "%s: no barrier between the parked stores and the arrival counter" % name
    after = lines[a + 1:]
    # loads into registers; the main loop's operand loads into LDS (global_load_lds_*) may be
    # laid out after the hand-off code but never run after it
    loads = [l for l in after if l.startswith("global_load") and not l.startswith("global_load_lds")]
    assert loads, "%s: no load of the parked sums after the arrival" % name
    for l in loads:
        assert re.search(r"\bsc1\b", l), "%s: a load after the arrival without sc1: %s" % (name, l)
    assert any(l.startswith("global_store_dword ") and re.search(r"\bsc1\b", l) for l in after), \
        "%s: no sc1 reset of the arrival counter" % name


def test_stream_slice_handoff(asm):
    ks = asm["k_stream"]
    # the atomic-halves form (last template argument true) has no hand-off: its two halves
    # meet in the output through atomic adds, read only by the next launch
    slices = {n: l for n, l in ks.items() if "Lb0E" in n}
    assert len(slices) >= 10, sorted(ks)
    for name, lines in slices.items():
        _check_handoff(name, lines, "global_store_dword")
    for name, lines in ks.items():
        if "Lb1E" in name:
            assert not _arrival(lines), name
            assert any(re.match(r"global_atomic_add_f32\s", l) for l in lines), name


def test_gemm_split_handoff(asm):
    kg = asm["k_gemm"]
    assert len(kg) >= 5, sorted(kg)
    for name, lines in kg.items():
        _check_handoff(name, lines, "global_store_dwordx2")


def test_tiled_split_handoff(asm):
    kt = asm["k_tiled"]
    assert len(kt) >= 5, sorted(kt)
    for name, lines in kt.items():
        _check_handoff(name, lines, "global_store_dwordx2")
