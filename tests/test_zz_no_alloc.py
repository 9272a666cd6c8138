"""The allocation-free relative-L1 entry point against the workspace one, through the C ABI.

resid_rel_l1_noalloc keeps its partial sums in the library's static per-GPU array instead of a
caller workspace; it runs the same kernels, so its result must carry the same bits as
resid_rel_l1's on the same input, and stay within relative 1e-4 of the fp64 oracle.  Three calls
in a row shrink the input (all 4096 partial pairs, then 123, then one): a later, smaller call
must not read partial sums a larger call left in the shared array.
"""
import sys

import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_transformer_attention_amd as dta  # noqa: E402

RL1_REL = 1e-4


def announce(msg):
    print(f"[no-alloc] {msg}", file=sys.stderr, flush=True)


def test_rel_l1_noalloc_matches_workspace_call():
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    # first call: 48M elements (the full 4096 partial pairs), drawn on the GPU
    n_big = 48 * 1024 * 1024 + 5
    b_big = torch.randn(n_big, generator=g, device="cuda").to(torch.bfloat16)
    a_big = (b_big.float() + 0.05 * torch.randn(n_big, generator=g, device="cuda")).to(torch.bfloat16)
    announce(f"resid_rel_l1_noalloc n={n_big}")
    want = dta.resid_rel_l1(a_big, b_big)
    dta.resid_rel_l1_noalloc(a_big, b_big, out)
    torch.cuda.synchronize()
    assert out.view(torch.int32).item() == want.view(torch.int32).item(), (out.item(), want.item())
    assert abs(out.item() - 0.05) < 1e-3
    del a_big, b_big
    # then smaller inputs with an oracle value: 1000003 elements (123 pairs), then 7 (one pair)
    for n, seed in ((1000003, 950), (7, 951)):
        a = datagen.normal_bf16((n,), seed, 4)
        b = datagen.normal_bf16((n,), seed, 5)
        ad = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        bd = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
        announce(f"resid_rel_l1_noalloc n={n}")
        dta.resid_rel_l1_noalloc(ad, bd, out)
        torch.cuda.synchronize()
        got = out.item()
        want = dta.resid_rel_l1(ad, bd)
        torch.cuda.synchronize()
        assert out.view(torch.int32).item() == want.view(torch.int32).item(), (got, want.item())
        ref = oracle.rel_l1(datagen.bf16_to_f64(a), datagen.bf16_to_f64(b))
        announce(f"  gpu {got:.8f} oracle {ref:.8f}")
        assert abs(got - ref) <= RL1_REL * ref, (got, ref)
