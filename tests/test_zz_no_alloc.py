"""The no-allocation prefill (gdn_prefill_chunked_noalloc) against the
workspace-taking entry point it varies, through the C ABI, on cuda:0.

Both run the same kernels on the same workspace layout (the no-allocation
call uses the library's static device scratch), so the results must be the
same bits. Two calls in a row on one device, the second with a smaller
input, so that the second runs on scratch the first left behind; and a
shape too large for the scratch is refused with no side effects.
"""
import numpy as np
import pytest

import oracle
from gdn_synth import from_torch, small_prefill, to_torch
from tests.parity import TOL, max_error

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_token_amd as g
    g.load_library()
    return g


def _run_both(gdn, d, init):
    q, k, v, a, b = [to_torch(d[n], DEV) for n in ("q", "k", "v", "alpha", "beta")]
    s0 = to_torch(d["S0"], DEV) if init else None
    ref_o, ref_s = gdn.gdn_prefill_chunked(q, k, v, a, b, s0, workspace="auto")
    na_o, na_s = gdn.gdn_prefill_chunked_noalloc(q, k, v, a, b, s0)
    torch.cuda.synchronize()
    return ref_o, ref_s, na_o, na_s


def test_noalloc_matches_workspace_call_twice(gdn):
    # the layer's shapes at T = 4096 (the largest workload that fits the
    # scratch), then a smaller, ragged call with an initial state
    cases = [(1, 4096, 16, 48, 128, False, 400), (1, 1000, 2, 6, 128, True, 401)]
    for B, T, Hk, Hv, D, init, seed in cases:
        d = small_prefill(B, T, Hk, Hv, D, "bf16", seed=seed, init_state=init)
        need = gdn.gdn_prefill_workspace_size(B, T, Hk, Hv, D, D, gdn.GDN_BF16, 0)
        assert 0 < need <= 64 << 20, need
        ref_o, ref_s, na_o, na_s = _run_both(gdn, d, init)
        assert torch.equal(na_o, ref_o), (T, Hv)
        assert torch.equal(na_s, ref_s), (T, Hv)
        o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                      d["S0"] if init else None)
        eo = max_error(from_torch(na_o), o_ref, (0, 2))
        es = max_error(from_torch(na_s), S_ref, (0, 1))
        print(f"[parity] noalloc T={T} Hv={Hv}: out {eo:.3e} state {es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_noalloc_refuses_shapes_beyond_its_scratch(gdn):
    # 262,144 tokens at the layer's heads need a 3.4 GB workspace
    T, Hk, Hv, D = 262144, 16, 48, 128
    assert gdn.gdn_prefill_workspace_size(1, T, Hk, Hv, D, D, gdn.GDN_BF16, 0) > 64 << 20
    lib = gdn.load_library()
    rc = lib.gdn_prefill_chunked_noalloc(None, None, None, None, None, None, None, None, None,
                                         0, 1, T, Hk, Hv, D, D, gdn.GDN_BF16, 1.0, 0, None)
    assert rc == 3  # GDN_ERR_UNSUPPORTED, before any pointer is looked at
