"""The matrix-core calibration kernel (ditattn_mfma_probe) runs and reports its clocks."""
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_transformer_attention_amd as dta  # noqa: E402


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
@pytest.mark.parametrize("random_operands", [True, False])
def test_mfma_probe_clocks(dtype, random_operands):
    print(f"[calibration] ditattn_mfma_probe {dtype} random={random_operands} iters=200",
          file=sys.stderr, flush=True)
    clocks = dta.mfma_probe(dtype, random_operands, iters=200)
    torch.cuda.synchronize()
    c = clocks.cpu()
    assert c.shape == (dta.MFMA_PROBE_WORKGROUPS, 2)
    assert bool((c[:, 0] > 0).all()) and bool((c[:, 1] > 0).all())
    # 200 x 8 products of at least 16 clocks each per wavefront, two wavefronts per SIMD
    assert bool((c[:, 0] >= 200 * 8 * 16).all())
    ghz = float(c[:, 0].sum()) / float(c[:, 1].sum()) * 0.1
    assert 0.3 < ghz < 3.5, ghz
