"""The path under HIP graph capture: route -> dispatch -> combine captured once and replayed several
times, with eager work and synchronisations between replays, every replay checked bit for bit against
the eager result of the same calls. The entry points allocate nothing and enqueue no memset, so
every node of the graph is one of the library's kernels."""
import numpy as np
import pytest
import torch

from combine_moe_route_03_amd import _lib as moe
from combine_moe_route_03_amd.workloads import WORKLOADS, Workload, make_inputs
from gpu_util import to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _announce(msg):
    print(f"[gpu] {msg}", flush=True)


CASES = {
    "decode": WORKLOADS["decode"],
    "decode_fp8": WORKLOADS["decode_fp8"],
    # multi-launch layout (more tokens than the one-launch layout takes), fp32
    "mid_f32": Workload("mid_f32", 1500, 512, 64, 4, 8, "f32", "f32", "f32", "f32", "scale"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    w = CASES[name]
    _announce(f"graph capture {name} T={w.T} H={w.H} E={w.E} k={w.k} payload={w.payload}")
    inp = make_inputs(w)
    logits = to_dev(inp["logits"], "f32")
    x = to_dev(inp["x"], w.x_dtype)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    buf = moe.alloc_dispatch_out(w.T, w.H, w.E, w.k, w.N, w.payload)
    ws = moe.alloc_workspace(w.T, w.E, w.k)
    ydt = moe.TORCH_DTYPES[w.y_dtype]
    y = (torch.randn((w.T * w.k, w.H), device="cuda") * 0.5).to(ydt)
    out = torch.empty((w.T, w.H), dtype=moe.TORCH_DTYPES[w.out_dtype], device="cuda")

    def step():
        moe.moe_route_dispatch(logits, x, w.k, w.N, buf, ws, topk_idx=idx, topk_w=wt)
        moe.moe_combine(y, buf.token_row, wt, out)

    outputs = [idx, wt, buf.expert_counts, buf.expert_offsets, buf.rank_counts,
               buf.rank_offsets, buf.token_row, buf.row_token, buf.recv, out]
    if buf.recv_scales is not None:
        outputs.append(buf.recv_scales)

    def snapshot():
        return [t.clone() for t in outputs]

    def clobber():                        # eager work between replays: overwrite every output
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                            # eager reference (and warm-up) on a side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = snapshot()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        clobber()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(want, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}"
