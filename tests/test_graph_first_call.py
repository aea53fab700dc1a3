"""Graph capture as the very first use of the library (GPU). In a fresh
process, the first D = 128 full-height launch (which opts the kernel in to more
than 64 KiB of LDS on its first call on a device; the case is checked to use
more than 64 KiB) and the first D = 64 launch
are made inside a HIP graph capture; the replays must equal eager launches made
afterwards, bit for bit."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import attention_forward_fa2_amd as fa2
from fa2_inputs import make_random

dev = torch.device("cuda:0")
# B1 H16 S4096 D128 non-causal is one round of 256 full-height workgroups,
# whose 128 KiB of LDS needs the opt-in; the D = 64 case is causal.
cfg = fa2.fa2_kernel_config(1, 16, 4096, 128, 0)
assert cfg["rows_per_block"] == 256 and cfg["lds_bytes"] > 65536, cfg
cases = [(make_random(49_000, 1, 16, 4096, 128), False), (make_random(49_100, 1, 4, 700, 64), True)]
bufs = []
for (q, k, v), causal in cases:
    t = [torch.from_numpy(x).to(dev) for x in (q, k, v)]
    o = torch.empty_like(t[0]); l = torch.empty(t[0].shape[:3], dtype=torch.float32, device=dev)
    bufs.append((t, o, l, causal))
torch.cuda.synchronize()
side = torch.cuda.Stream()
side.wait_stream(torch.cuda.current_stream())
graph = torch.cuda.CUDAGraph()
with torch.cuda.stream(side):
    with torch.cuda.graph(graph, stream=side):
        for t, o, l, causal in bufs:
            fa2.forward(*t, causal=causal, out=o, lse=l)
torch.cuda.synchronize()
for rep in range(2):
    for t, o, l, causal in bufs:
        o.fill_(float("nan")); l.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    for t, o, l, causal in bufs:
        oe, le = fa2.forward(*t, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), oe.view(torch.int16)), f"replay {rep}: O differs"
        assert torch.equal(l.view(torch.int32), le.view(torch.int32)), f"replay {rep}: LSE differs"
print("GRAPH FIRST CALL OK", flush=True)
"""


def test_first_launches_inside_graph_capture():
    print("case: first D=128 and D=64 launches inside a graph capture, fresh process", flush=True)
    res = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0 and "GRAPH FIRST CALL OK" in res.stdout
