"""The allocation-free dynamic-range entry point against the workspace one:
same codes, s and z bit for bit (both run the same kernels; only where the
ranges pass parks its per-workgroup partials differs).  Two calls in a row,
the second on a smaller input, so the second call runs on an array that
still holds the first call's partials."""
import numpy as np
import pytest

from helpers import code_bytes, dev, layer_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_quantization_layernorm_amd as P
    P.lib()
    return P


def _run_both(P, M, K, g, bits, seed):
    c = layer_case(M, K, 64, g, bits, seed=seed, with_weights=False)
    print(f"[no_alloc] M={M} K={K} g={g} bits={bits} seed={seed}", flush=True)
    x = dev(c.x.view(np.int16)).view(torch.float16)
    R = dev(c.R)
    gr, br = dev(c.gamma[c.R]), dev(c.beta[c.R])
    ref = P.rptq_ln_reorder_quant_dynamic(x, R, gr, br, c.bounds, bits)
    rb = P.rptq_codes_row_bytes(c.bounds, bits)
    # outputs pre-filled with a pattern the kernels must overwrite (the code
    # bytes of each row; the tail of the row pitch is not written)
    out = torch.full((M, rb), 0xA5, dtype=torch.uint8, device="cuda")
    s_out = torch.full((g,), -1.0, dtype=torch.float32, device="cuda")
    z_out = torch.full((g,), -7, dtype=torch.int32, device="cuda")
    got = P.rptq_ln_reorder_quant_dynamic_noalloc(x, R, gr, br, c.bounds, bits, out, s_out, z_out)
    torch.cuda.synchronize()
    assert np.array_equal(code_bytes(got[0], c.bounds, bits), code_bytes(ref[0], c.bounds, bits))
    for a, b in zip(got[1:], ref[1:]):
        assert torch.equal(a, b)
    return got


def test_noalloc_matches_workspace_entry_point_twice(P):
    # first call: 8 clusters over 768 channels, 4-bit
    _run_both(P, 1200, 768, 8, 4, seed=11)
    # second call, smaller (fewer rows, channels and clusters, 3-bit)
    _run_both(P, 70, 256, 4, 3, seed=12)


def test_noalloc_rejects_before_any_launch(P):
    # M = 0 is invalid for dynamic ranges; nothing is launched
    x = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    o = torch.zeros((1, 32), dtype=torch.uint8, device="cuda")
    s = torch.zeros(2, dtype=torch.float32, device="cuda")
    z = torch.zeros(2, dtype=torch.int32, device="cuda")
    gm = torch.ones(64, dtype=torch.float32, device="cuda")
    with pytest.raises(P.RptqError):
        P.rptq_ln_reorder_quant_dynamic_noalloc(x, None, gm, gm, np.array([0, 16, 64], np.int32), 4, o, s, z)
