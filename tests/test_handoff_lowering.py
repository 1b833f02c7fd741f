"""The single-launch decode's hand-off, as the compiler lowers it for gfx950.

Correctness of the fused split-KV decode (pass 1 and the combine in one launch)
rests on the order in which the built code publishes the partial states and
takes the per-(sequence, kv head) counter:

1. every partial row and LSE is stored with an agent-scope store, which gfx950
   code performs as a global store with the `sc1` bit (written through to the
   device coherence point, acknowledged only once there);
2. `s_waitcnt vmcnt(0)` then `s_barrier`: every wave's stores are acknowledged
   before any lane of the workgroup touches the counter;
3. the counter `global_atomic_add`;
4. the workgroup that completes the count acquires with `buffer_inv sc1` before
   it reads the other workgroups' partials.

This test compiles the decode source to gfx950 assembly with the library's
flags and checks that sequence in every fused instantiation, so a toolchain
that lowers any step differently fails here instead of producing wrong values
on the GPU. CPU only (hipcc cross-compiles); about a minute.
"""
import os
import re
import shutil
import subprocess

import pytest

from lse_attention_state_amd import build as mi_build

HIPCC = mi_build.HIPCC
KERNEL = re.compile(
    r"^(_ZN2mi12_GLOBAL__N_123split_kv_partial_kernelILi(\d)ELi(\d)ELi(n1|\d)ELb(\d)ELi(\d+)EE\S*):",
    re.M)


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not available")
    out = tmp_path_factory.mktemp("asm") / "decode.s"
    src = os.path.join(mi_build.CSRC, "decode.hip")
    flags = [f for f in mi_build.CFLAGS if f != "-fPIC"]
    cmd = [HIPCC, *flags, "-x", "hip", "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _bodies(asm):
    """(name, template arguments, instruction list) of every decode kernel."""
    for m in KERNEL.finditer(asm):
        end = asm.index(".Lfunc_end", m.end())
        ins = [l.strip() for l in asm[m.end():end].split("\n")
               if l.startswith("\t") and not l.strip().startswith((";", "."))]
        dt, g, dto, var, pr = m.group(2), m.group(3), m.group(4), m.group(5), m.group(6)
        yield m.group(1), (int(dt), int(g), -1 if dto == "n1" else int(dto), var == "1", int(pr)), ins


def test_fused_decode_publishes_before_the_counter(decode_asm):
    checked = 0
    for name, (dt, g, dto, var, pr), ins in _bodies(decode_asm):
        if dto < 0 or pr != 0:
            continue  # pass 1 only, or one split with prior states in registers: no hand-off
        atom = [i for i, s in enumerate(ins) if s.startswith("global_atomic_add")]
        assert atom, f"{name}: no counter atomic"
        a = atom[0]
        pub = [i for i, s in enumerate(ins[:a])
               if s.startswith("global_store") and re.search(r"\bsc1\b", s)]
        assert pub, f"{name}: partials not stored with sc1 before the counter"
        kinds = {ins[i].split()[0] for i in pub}
        assert "global_store_dwordx2" in kinds and "global_store_dword" in kinds, (name, kinds)
        p = pub[-1]
        waits = [i for i in range(p + 1, a)
                 if ins[i].startswith("s_waitcnt") and "vmcnt(0)" in ins[i]]
        assert waits, f"{name}: no vmcnt(0) between the partial stores and the counter"
        bars = [i for i in range(waits[0] + 1, a) if ins[i] == "s_barrier"]
        assert bars, f"{name}: no barrier between the store wait and the counter"
        late = [ins[i] for i in range(waits[0] + 1, a) if ins[i].startswith("global_store")]
        assert not late, f"{name}: stores after the wait, before the counter: {late}"
        inv = [i for i in range(a + 1, len(ins)) if re.match(r"buffer_inv\b.*\bsc1\b", ins[i])]
        assert inv, f"{name}: no agent-scope acquire (buffer_inv sc1) after the counter"
        checked += 1
    # 2 K/V dtypes x 4 GQA group sizes x 3 output dtypes x (uniform, per-sequence)
    assert checked == 48, checked
