"""GPU: the library's calls captured into a HIP graph and replayed.

Every call enqueues only kernels on the caller's stream (no allocation, no memset, no host
synchronisation), so a step of the path can be captured once and replayed: the bf16 call on
its workspace (whole rounds, the shared-out last round and, when there is no whole round, the
kernel that zeroes its arrival counters; for long sequences the V^T tile prepass), the int8-QK
call (prepass and attention, the same split) and the relative-L1 reduction.  The graph is
replayed several times with eager work and synchronisations in between and with the outputs
cleared before each replay; every replay must reproduce the eager results bit for bit (the
calls are deterministic).
"""
import sys

import numpy as np
import pytest

import datagen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_transformer_attention_amd as dta  # noqa: E402


def announce(msg):
    print(f"[gpu-graph] {msg}", file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# B1 H5 S4000: 80 tiles, all shared out (no whole round: the zeroing kernel runs);
# B2 H24 S4608: 864 tiles, three whole rounds and 96 tiles shared out;
# B1 H2 S33000: V read through V^T tiles written by their prepass kernel.
@pytest.mark.parametrize("B,H,S,D", [(1, 5, 4000, 64), (2, 24, 4608, 128), (1, 2, 33000, 128)])
def test_graph_replay_matches_eager(B, H, S, D):
    announce(f"graph of bf16 + int8-QK + rel-L1, B{B} H{H} S{S} D{D}")
    q = dev(datagen.normal_bf16((B, H, S, D), 1100 + D, 0))
    k = dev(datagen.normal_bf16((B, H, S, D), 1100 + D, 1))
    v = dev(datagen.normal_bf16((B, H, S, D), 1100 + D, 2))
    a = dev(datagen.normal_bf16((1 << 20,), 1100, 3))
    b = dev(datagen.normal_bf16((1 << 20,), 1100, 4))
    ws16 = dta.bf16_workspace(B, H, S, D, "cuda")
    ws8 = dta.int8qk_workspace(B, H, S, D, "cuda")
    wsr = torch.empty(dta.rel_l1_workspace_bytes(a.numel()), dtype=torch.uint8, device="cuda")
    o16 = torch.empty((B, H, S, D), dtype=torch.float32, device="cuda")
    o8 = torch.empty_like(o16)
    r = torch.empty(1, dtype=torch.float32, device="cuda")

    def step():
        dta.attn_fwd_bf16(q, k, v, out=o16, workspace=ws16)
        dta.attn_fwd_int8qk(q, k, v, out=o8, workspace=ws8)
        dta.resid_rel_l1(a, b, out=r, workspace=wsr)

    step()
    torch.cuda.synchronize()
    ref = (o16.clone(), o8.clone(), r.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (o16, o8, r):
            t.fill_(float("nan"))
        ws16.fill_(0xFF)  # the split's counters and slots start as garbage every time
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()  # eager work and a synchronisation between replays
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in (("bf16", o16, ref[0]), ("int8", o8, ref[1]), ("rel-L1", r, ref[2])):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
    announce("  3 replays bit-identical to the eager step")
