"""Host threads calling the library at once (GPU). The child process below
starts fresh, so the first launches of every kernel instance, including the
per-device opt-in to more than 64 KiB of LDS for the D = 128 full-height
kernel, happen concurrently from 8 threads, each on its own stream. Every
result must equal, bit for bit, the same call made again afterwards from one
thread."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, threading
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import attention_forward_fa2_amd as fa2
from fa2_inputs import make_random, make_packed

dev = torch.device("cuda:0")
def dense(seed, B, H, S, D, H_kv=None):
    q, _, _ = make_random(seed, B, H, S, D)
    _, k, v = make_random(seed + 10, B, H_kv or H, S, D)
    return [torch.from_numpy(x).to(dev) for x in (q, k, v)]
cases = []
for t in range(8):
    kind = t % 4
    if kind == 0:
        cases.append(("fwd", dense(80_000 + t, 1, 4, 700, 128), dict(causal=False)))
    elif kind == 1:
        cases.append(("fwd", dense(80_100 + t, 2, 3, 513, 64), dict(causal=True)))
    elif kind == 2:
        cases.append(("ex", dense(80_200 + t, 1, 6, 400, 64, H_kv=2),
                      dict(window=(50, 20), dropout_p=0.2, seed=t, offset=3)))
    else:
        q, k, v, cu = make_packed(80_300 + t, [300, 0, 129, 64], 4, 2, 128)
        cases.append(("varlen", [torch.from_numpy(x).to(dev) for x in (q, k, v)] + [torch.from_numpy(cu).to(dev)],
                      dict(causal=True)))
torch.cuda.synchronize()

def run(kind, args, kw):
    if kind == "fwd":
        return fa2.forward(*args, **kw)
    if kind == "ex":
        return fa2.forward_ex(*args, **kw)
    return fa2.forward_varlen(*args, max_seqlen=300, **kw)

results = [None] * len(cases)
errors = []
start = threading.Barrier(len(cases))
def worker(i):
    try:
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            start.wait()
            outs = [run(*cases[i]) for _ in range(4)]
        st.synchronize()
        results[i] = [(o.cpu(), l.cpu()) for o, l in outs]
    except Exception as e:  # reported by the main thread
        errors.append(f"thread {i}: {e!r}")
threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
for th in threads: th.start()
for th in threads: th.join(timeout=60)
assert not any(th.is_alive() for th in threads), "a thread did not finish"
assert not errors, errors
for i, c in enumerate(cases):
    o_ref, l_ref = run(*c)
    torch.cuda.synchronize()
    for o, l in results[i]:
        assert torch.equal(o.view(torch.int16), o_ref.cpu().view(torch.int16)), f"case {i}: O differs"
        assert torch.equal(l.view(torch.int32), l_ref.cpu().view(torch.int32)), f"case {i}: LSE differs"
print("THREADS OK", flush=True)
"""


def test_threads_fresh_process():
    print("case: 8 host threads, fresh process", flush=True)
    res = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0 and "THREADS OK" in res.stdout
