"""The scan and the decode step captured in a HIP graph (torch.cuda.graph), replayed.

The library enqueues only kernel launches (and, for T == 0, a device copy) on
the caller's stream and allocates nothing, so its calls can be captured:
gdn_scan_noalloc with its static scratch, gdn_scan with a workspace allocated
before the capture, and the in-place decode step.  Each replay, with eager
work and synchronisations between replays, must reproduce the eager results
bit for bit.
"""
import sys

import pytest
import torch

from linear_attention_recurrence_recurrent_amd import (recurrent_step, scan, scan_noalloc,
                                                       scan_workspace_bytes, synth, _desc)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,T,Hk,Hv,dtype", [(1, 70, 2, 4, "bf16"), (8, 40, 16, 32, "f16")])
def test_scan_and_step_replayed_from_a_graph(B, T, Hk, Hv, dtype):
    say("graph capture B=%d T=%d Hk=%d Hv=%d %s" % (B, T, Hk, Hv, dtype))
    ops = {n: t.to(DEV) for n, t in synth.random_operands(B, T, Hk, Hv, 128, 128, dtype=dtype,
                                                          seed=B + T).items()}
    a = (ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"], ops["z"],
         ops["w"])
    step = {n: ops[n][:, :1].contiguous() for n in ("q", "k", "v", "z", "log_decay", "beta")}
    # eager references
    y_ref, s_ref = scan(*a)
    y2_ref, s2_ref = scan_noalloc(*a)
    st_ref = s_ref.clone()
    y1_ref, _ = recurrent_step(step["q"], step["k"], step["v"], step["log_decay"], step["beta"],
                               st_ref, step["z"], ops["w"], inplace=True)
    torch.cuda.synchronize()
    # static buffers, the workspace included, allocated before the capture
    y, s = torch.empty_like(y_ref), torch.empty_like(s_ref)
    y2, s2 = torch.empty_like(y_ref), torch.empty_like(s_ref)
    y1, st = torch.empty_like(y1_ref), torch.empty_like(s_ref)
    dt = {"bf16": 2, "f16": 1}[dtype]
    need = scan_workspace_bytes(_desc(B, T, Hk, Hv, 128, 128, False, dt, dt, True, True, 1e-6,
                                      1e-6))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream's kind of stream
        scan(*a, out=y, state_out=s, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        scan(*a, out=y, state_out=s, workspace=ws)
        scan_noalloc(*a, out=y2, state_out=s2)
        st.copy_(s)
        recurrent_step(step["q"], step["k"], step["v"], step["log_decay"], step["beta"], st,
                       step["z"], ops["w"], inplace=True, out=y1)
    for rep in range(3):
        for t in (y, s, y2, s2, y1, st):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(s, s_ref), "replay %d: gdn_scan" % rep
        assert torch.equal(y2, y2_ref) and torch.equal(s2, s2_ref), "replay %d: noalloc" % rep
        assert torch.equal(y1, y1_ref) and torch.equal(st, st_ref), "replay %d: step" % rep
        # eager work of the program between replays
        scan(*a)
        torch.cuda.synchronize()
