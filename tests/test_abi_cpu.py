"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/gdn.h declares, and rejects invalid calls with the documented
status before any HIP call (so no kernel is ever launched from here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
LIB = os.path.join(ROOT, "gated_deltanet_token_amd", "libgdn.so")

OK, NULLP, SHAPE, UNSUP, MISAL, ALIAS, HIPERR = range(7)
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:gdn_status_t|const char \*|int32_t)\s*(gdn_\w+)\s*\(", text,
                      flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libgdn.so is not built (python -m gated_deltanet_token_amd.build)")
    import gated_deltanet_token_amd as g
    return g.load_library(LIB)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"gdn_prefill_chunked", "gdn_decode_step", "gdn_varlen_prefill", "gdn_decode_multi",
            "gdn_status_string", "gdn_version"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.gdn_version() >= 100


def test_status_strings(lib):
    for s in range(7):
        assert lib.gdn_status_string(s)
    assert b"aligned" in lib.gdn_status_string(MISAL)


# Fake device addresses: every call below must fail validation, so none is
# ever dereferenced or passed to HIP.
A = 1 << 30            # 16-byte aligned base
MB = 1 << 20


def P(i):
    return A + i * 64 * MB  # disjoint, aligned regions


def prefill(lib, q=P(0), k=P(1), v=P(2), a=P(3), b=P(4), s0=P(5), out=P(6), sf=P(7), pre=None,
            every=0, B=1, T=64, Hk=2, Hv=4, Dk=64, Dv=64, dtype=BF16, ws=None, wsb=0, flags=0):
    return lib.gdn_prefill_chunked(q, k, v, a, b, s0, out, sf, pre, every, B, T, Hk, Hv, Dk, Dv,
                                   dtype, 1.0, flags, ws, wsb, None)


def varlen(lib, q=P(0), k=P(1), v=P(2), a=P(3), b=P(4), cu=P(8), N=2, total=64, s0=P(5),
           out=P(6), sf=P(7), pre=None, every=0, Hk=2, Hv=4, Dk=64, Dv=64, dtype=BF16, ws=None,
           wsb=0, flags=0):
    return lib.gdn_varlen_prefill(q, k, v, a, b, cu, N, total, s0, out, sf, pre, every, Hk, Hv, Dk,
                                  Dv, dtype, 1.0, flags, ws, wsb, None)


def decode(lib, q=P(0), k=P(1), v=P(2), a=P(3), b=P(4), s=P(5), out=P(6), B=4, Hk=2, Hv=4,
           Dk=64, Dv=64, dtype=BF16, flags=0):
    return lib.gdn_decode_step(q, k, v, a, b, s, out, B, Hk, Hv, Dk, Dv, dtype, 1.0, flags, None)


def test_prefill_validation(lib):
    assert prefill(lib, q=None) == NULLP
    assert prefill(lib, out=None) == NULLP
    assert prefill(lib, B=0) == SHAPE
    assert prefill(lib, T=-1) == SHAPE
    assert prefill(lib, Hk=3, Hv=4) == SHAPE
    assert prefill(lib, Hk=0) == SHAPE
    assert prefill(lib, Dk=96, Dv=96) == UNSUP
    assert prefill(lib, Dk=64, Dv=128) == UNSUP
    assert prefill(lib, dtype=7) == UNSUP
    assert prefill(lib, q=P(0) + 8) == MISAL
    assert prefill(lib, sf=P(7) + 4) == MISAL
    assert prefill(lib, out=P(2)) == ALIAS            # out on top of v
    assert prefill(lib, out=P(2) + 4096) == ALIAS     # partial overlap
    assert prefill(lib, sf=P(6)) == ALIAS             # final state on top of out
    assert prefill(lib, sf=P(5) + 64) == ALIAS        # partial overlap with initial state
    assert prefill(lib, sf=P(0)) == ALIAS             # final state on top of q
    assert prefill(lib, B=1 << 30, T=1 << 30) == SHAPE  # byte counts overflow
    assert prefill(lib, ws=P(9) + 8, wsb=1 << 20) == MISAL
    assert prefill(lib, ws=P(6), wsb=1 << 20) == ALIAS    # workspace on top of out
    assert prefill(lib, ws=P(7) + 4096, wsb=1 << 20) == ALIAS  # inside the final state


def test_prefix_states_validation(lib):
    assert prefill(lib, pre=P(9), every=0) == SHAPE           # interval required
    assert prefill(lib, pre=P(9), every=-2) == SHAPE
    assert prefill(lib, pre=P(9) + 4, every=1) == MISAL
    assert prefill(lib, pre=P(6), every=1) == ALIAS           # on top of out
    assert prefill(lib, pre=P(7) + 1024, every=1) == ALIAS    # inside the final state
    assert prefill(lib, pre=P(0), every=1) == ALIAS           # on top of q
    assert prefill(lib, pre=P(9), every=1, ws=P(9) + 4096, wsb=1 << 20) == ALIAS  # workspace
    # T < 64 m: no rows, nothing can overlap
    assert prefill(lib, pre=P(6), every=2, q=None, k=None, v=None, a=None, b=None, out=None,
                   sf=None, T=0) == OK
    assert varlen(lib, pre=P(9), every=0) == SHAPE
    assert varlen(lib, pre=P(8), every=1) == ALIAS             # on top of cu_seqlens
    assert varlen(lib, pre=P(5) + 64, every=4) == ALIAS        # N rows always exist


def test_varlen_validation(lib):
    assert varlen(lib, cu=None) == NULLP
    assert varlen(lib, N=0) == SHAPE
    assert varlen(lib, total=-1) == SHAPE
    assert varlen(lib, total=1 << 31) == SHAPE
    assert varlen(lib, cu=P(8) + 4) == MISAL
    assert varlen(lib, out=P(8)) == ALIAS             # out on top of cu_seqlens
    assert varlen(lib, Dk=32, Dv=32) == UNSUP
    assert varlen(lib, ws=P(8), wsb=64) == ALIAS          # workspace on top of cu_seqlens


def test_decode_validation(lib):
    assert decode(lib, s=None) == NULLP
    assert decode(lib, B=0) == SHAPE
    assert decode(lib, Hk=4, Hv=6) == SHAPE
    assert decode(lib, Dk=256, Dv=256) == UNSUP
    assert decode(lib, out=P(5)) == ALIAS             # out on top of the state
    assert decode(lib, s=P(2)) == ALIAS               # state on top of v
    assert decode(lib, v=P(2) + 2) == MISAL


def multi(lib, q=P(0), k=P(1), v=P(2), a=P(3), b=P(4), pool=P(5), ns=8, src=P(8), dst=P(9),
          out=P(6), steps=P(7), B=4, K=3, Hk=2, Hv=4, Dk=64, Dv=64, dtype=BF16, flags=0):
    return lib.gdn_decode_multi(q, k, v, a, b, pool, ns, src, dst, out, steps, B, K, Hk, Hv, Dk,
                                Dv, dtype, 1.0, flags, None)


def test_decode_multi_validation(lib):
    assert multi(lib, pool=None) == NULLP
    assert multi(lib, src=None) == NULLP
    assert multi(lib, dst=None) == NULLP
    assert multi(lib, out=None) == NULLP
    assert multi(lib, B=0) == SHAPE
    assert multi(lib, K=-1) == SHAPE
    assert multi(lib, ns=0) == SHAPE
    assert multi(lib, Hk=3, Hv=4) == SHAPE
    assert multi(lib, Dk=96, Dv=96) == UNSUP
    assert multi(lib, dtype=5) == UNSUP
    assert multi(lib, pool=P(5) + 8) == MISAL
    assert multi(lib, steps=P(7) + 4) == MISAL
    assert multi(lib, src=P(8) + 2) == MISAL
    assert multi(lib, out=P(2)) == ALIAS              # out on top of v
    assert multi(lib, pool=P(0)) == ALIAS             # pool on top of q
    assert multi(lib, src=P(5) + 64) == ALIAS         # slot ids inside the pool
    assert multi(lib, dst=P(7)) == ALIAS              # slot ids inside the step states
    assert multi(lib, steps=P(6)) == ALIAS            # step states on top of out
    assert multi(lib, steps=P(5) + 4096) == ALIAS     # step states inside the pool
    assert multi(lib, B=1 << 24, K=1 << 24) == SHAPE  # step-state bytes overflow
    assert multi(lib, ns=1 << 30, Hv=1 << 20) == SHAPE  # pool bytes overflow


def test_unknown_flags_are_rejected(lib):
    for f in (4, 8, 1 << 31, 7):
        assert prefill(lib, flags=f) == UNSUP
        assert varlen(lib, flags=f) == UNSUP
        assert decode(lib, flags=f) == UNSUP
        assert multi(lib, flags=f) == UNSUP


def test_valid_call_without_device_reports_hip_error(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this checks the no-device path only")
    assert prefill(lib) == HIPERR
    assert b"HIP" in lib.gdn_status_string(HIPERR)
    assert decode(lib) == HIPERR
    assert decode(lib, flags=3) == HIPERR
    assert prefill(lib, flags=3) == HIPERR
    assert multi(lib) == HIPERR
    assert multi(lib, steps=None, K=0, q=None, k=None, v=None, a=None, b=None, out=None) == HIPERR
    assert lib.gdn_prefill_workspace_size(1, 4096, 16, 48, 128, 128, BF16, 0) == 0


def test_workspace_size_rejects_bad_shapes(lib):
    assert lib.gdn_prefill_workspace_size(1, 4096, 16, 47, 128, 128, BF16, 0) == 0
    assert lib.gdn_prefill_workspace_size(0, 4096, 16, 48, 128, 128, BF16, 0) == 0
    assert lib.gdn_prefill_workspace_size(1, 4096, 16, 48, 96, 96, BF16, 0) == 0


def test_empty_prefill_without_final_state_is_a_no_op(lib):
    # T = 0 and nothing to write: succeeds before touching the runtime
    assert prefill(lib, q=None, k=None, v=None, a=None, b=None, out=None, sf=None, T=0) == OK
