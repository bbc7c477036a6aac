"""HIP-graph capture of the decode step: every replay, with eager work and
synchronizations between replays, must reproduce the eager results."""

import math

import pytest
import torch

import hybrid_sparse_linear_amd as sala
from hybrid_sparse_linear_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    print("[case] decode graph", flush=True)
    B, Hq, Hkv, d, L, H = 2, 16, 2, 128, 64 * 300 + 7, 8
    kc = I.normal((B, Hkv, L, d), 110, 1.0, I.BF16, "cuda")
    vc = I.normal((B, Hkv, L, d), 111, 1.0, I.BF16, "cuda")
    q = I.normal((B, Hq, d), 112, 1.0, I.BF16, "cuda")
    lq, lk, lv = (I.normal((B, H, d), 113 + t, 1.0 / math.sqrt(d), I.BF16, "cuda") for t in range(3))
    s0 = I.normal((B, H, d, d), 116, 1.0 / d, I.F32, "cuda")
    decay = I.slope_decay(H).cuda()
    q4 = q[:, :, None].contiguous()
    idx, kp = sala.sparse_select(q4, kc, topk=16)
    ws_s = torch.zeros(sala.workspace_bytes("sparse_select", dtype=1, B=B, Hq=Hq, Hkv=Hkv, d=d, Nq=1, L=L, block=64,
                                            topk=16, n_init=1, n_local=2), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(sala.workspace_bytes("sparse_decode", dtype=1, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, block=64,
                                            n_sel=19), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lo = torch.empty_like(lq)
    st = s0.clone()

    def step():
        sala.linear_decode(lq, lk, lv, st, decay, out=lo)
        sala.sparse_select(q4, None, k_pooled=kp, L=L, topk=16, idx_out=idx, workspace=ws_s)
        sala.sparse_decode(q, kc, vc, idx[:, :, 0], L=L, out=o, workspace=ws_a)

    # eager reference: three consecutive steps from s0
    st.copy_(s0)
    ref = []
    for _ in range(3):
        step()
        ref.append((o.clone(), lo.clone(), st.clone(), idx.clone()))
    # capture, then replay three times from s0 with eager work in between
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    st.copy_(s0)
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[r][3]), f"replay {r}: indices"
        assert torch.equal(o, ref[r][0]), f"replay {r}: sparse decode output"
        assert torch.equal(lo, ref[r][1]), f"replay {r}: linear decode output"
        assert torch.equal(st, ref[r][2]), f"replay {r}: linear state"
        _ = (q * 2).sum().item()  # eager work between replays
