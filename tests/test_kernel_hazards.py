"""Static checks of the compiled gfx950 kernels (CPU only: hipcc cross-compiles).

The K/V direct-to-LDS loads are inline asm, which the compiler's hazard
recognizer cannot see into, so the asm must provide the wait states itself.
This compiles the kernel source to gfx950 assembly with the library's own
flags and checks, in every kernel instance:
  * every SGPR-addressed global_load_lds is preceded by at least 5 wait states
    since the last VALU instruction that wrote one of its SGPR operands (a
    VALU write of an SGPR followed by a vector-memory read of it needs 5);
  * every global_load_lds is preceded by at least 1 wait state since the last
    write of M0 (the LDS-DMA base);
  * device code has no scalar-memory stores, scalar atomics or scalar-cache
    write-backs (s_store*, s_atomic*, s_dcache_wb*);
  * the library's own build uses no scratch: no spilled VGPRs and a zero
    private segment in every instance (a spill reload waits on the same
    vector-memory counter as the K/V prefetch).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = os.path.join(ROOT, "attention_forward_fa2_amd", "csrc", "fa2_fwd_kernel.hip")


def _flags():
    from attention_forward_fa2_amd import build as b
    return [f for f in b.FLAGS if f not in ("-shared", "-fPIC")]


@pytest.fixture(scope="module", params=["normal", "poison", "mf32"])
def kernel_asm(request, tmp_path_factory):
    from attention_forward_fa2_amd import build as b
    out = tmp_path_factory.mktemp("asm") / "k.s"
    extra = {"normal": [], "poison": ["-DFA2_POISON_LDS=1"], "mf32": ["-DFA2_D64_MF=32"]}[request.param]
    cmd = [b.HIPCC, *_flags(), *extra, "--offload-device-only", "-S", KERNEL, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out.read_text()


def _instances(text):
    cur, body = None, []
    for raw in text.splitlines():
        m = re.match(r"^(_Z\S*fa2_fwd_kernel\S*):", raw)
        if m:
            if cur:
                yield cur, body
            cur, body = m.group(1), []
            continue
        line = raw.split(";")[0].strip()
        if cur and line and not line.startswith(".") and not line.endswith(":"):
            body.append(line)
    if cur:
        yield cur, body


def _wait_states(lines):
    """Wait states that the given instructions provide (s_nop N gives N+1)."""
    n = 0
    for x in lines:
        m = re.match(r"s_nop\s+(\d+)", x)
        n += int(m.group(1)) + 1 if m else 1
    return n


def test_kernel_instances_found(kernel_asm):
    names = [n for n, _ in _instances(kernel_asm)]
    assert len(names) == 24, names


def test_sgpr_based_lds_dma_has_5_wait_states_after_valu_sgpr_write(kernel_asm):
    checked = 0
    for name, body in _instances(kernel_asm):
        for i, ins in enumerate(body):
            m = re.match(r"global_load_lds_dwordx4\s+v\d+,\s*s\[(\d+):(\d+)\]", ins)
            if not m:
                continue
            regs = {f"s{m.group(1)}", f"s{m.group(2)}"}
            checked += 1
            for j in range(i - 1, max(-1, i - 40), -1):
                w = re.match(r"(v_\w+)\s+(s\d+|s\[(\d+):(\d+)\])", body[j])
                if not w:
                    continue
                if w.group(3):
                    written = {f"s{r}" for r in range(int(w.group(3)), int(w.group(4)) + 1)}
                else:
                    written = {w.group(2)}
                if written & regs:
                    ws = _wait_states(body[j + 1:i])
                    assert ws >= 5, f"{name}: {body[j]!r} -> {ins!r} with {ws} wait states"
                    break
    assert checked > 0


def test_m0_write_precedes_lds_dma_by_a_wait_state(kernel_asm):
    for name, body in _instances(kernel_asm):
        for i, ins in enumerate(body):
            if not ins.startswith("global_load_lds"):
                continue
            for j in range(i - 1, max(-1, i - 40), -1):
                if re.match(r"s_\w+\s+m0\b", body[j]):
                    assert _wait_states(body[j + 1:i]) >= 1, f"{name}: {body[j]!r} -> {ins!r}"
                    break


def test_no_scalar_cache_writes(kernel_asm):
    bad = [ins for _, body in _instances(kernel_asm) for ins in body
           if re.match(r"s_(store|atomic|dcache_wb|buffer_store|scratch_store)", ins)]
    assert not bad, bad[:5]


def test_library_build_uses_no_scratch(kernel_asm, request):
    if request.node.callspec.params["kernel_asm"] != "normal":
        pytest.skip("only the library's own build is held to this")
    names = re.findall(r"\.name:\s+(_Z\S*fa2_fwd_kernel\S*)", kernel_asm)
    private = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", kernel_asm)
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", kernel_asm)
    assert len(names) == len(private) == len(spills) == 24
    bad = [(n, p, v) for n, p, v in zip(names, private, spills) if int(p) or int(v)]
    assert not bad, bad
