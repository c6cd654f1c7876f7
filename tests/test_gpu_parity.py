"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case draws seeded synthetic inputs, runs the library on cuda:0 and
compares with the oracle on the same bits. Metric (per (sequence, value
head) slice, max |x - r| / max |r|) and tolerances (2e-2 for bf16 inputs,
1e-4 for fp32) are in tests/parity.py. The full-size workloads (the
262,144-token prefill and the 64-sequence varlen batch) are checked chain by
chain over every (sequence, value head) pair, each chain run by the oracle
over its full length on host threads and compared as it finishes.
"""
import os

import numpy as np
import pytest

import oracle
from gdn_synth import (SPEC_DECODE, WORKLOADS, from_torch, generate, generate_packed,
                       lengths_for, multi_decode, small_prefill, to_torch)
from tests.parity import TOL, max_error, slice_error

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_token_amd as g
    g.load_library()
    return g


def _t(d, names):
    return [to_torch(d[n], DEV) for n in names]


def _set_path(monkeypatch, path):
    """Prefill path for a test: "fused" or "split" as given; "fused1" is the
    one-pass path with one workgroup per (sequence, value head) chain (the
    path a batch with many chains takes by default)."""
    if path == "fused1":
        monkeypatch.setenv("GDN_PREFILL_PATH", "fused")
        monkeypatch.setenv("GDN_PREFILL_NSPLIT", "1")
    else:
        monkeypatch.setenv("GDN_PREFILL_PATH", path)


def gpu_prefill(gdn, d, use_init=True, scale=1.0, stream=None):
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    s0 = to_torch(d["S0"], DEV) if use_init and d.get("S0") is not None else None
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, s0, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return from_torch(out), from_torch(sf)


def oracle_prefill(d, use_init=True, scale=1.0):
    s0 = d["S0"] if use_init else None
    return oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0, scale)


def check(o, S, o_ref, S_ref, dtype, label, o_axes=(0, 2), s_axes=(0, 1)):
    eo = max_error(o, o_ref, o_axes) if np.asarray(o_ref).size else 0.0
    es = max_error(S, S_ref, s_axes)
    print(f"[parity] {label}: out {eo:.3e}  state {es:.3e}  (tol {TOL[dtype]:.0e})", flush=True)
    assert eo <= TOL[dtype], f"{label}: output error {eo}"
    assert es <= TOL[dtype], f"{label}: state error {es}"
    return eo, es


# ----------------------------------------------------------------- small shapes
SMALL = [
    # B, T, Hk, Hv, D, dtype, init
    (1, 1, 1, 1, 64, "bf16", False),
    (1, 63, 1, 2, 64, "bf16", True),
    (2, 64, 2, 4, 64, "bf16", True),
    (1, 65, 2, 6, 128, "bf16", False),
    (1, 127, 2, 6, 128, "bf16", True),
    (2, 200, 4, 12, 128, "bf16", True),
    (1, 200, 2, 2, 128, "bf16", True),    # Hk == Hv
    (1, 129, 1, 3, 64, "f32", True),
    (1, 100, 2, 4, 128, "f32", True),
]


@pytest.mark.parametrize("B,T,Hk,Hv,D,dtype,init", SMALL)
@pytest.mark.parametrize("nsplit", ["auto", "1", "2", "4", "8"])
@pytest.mark.parametrize("path", ["fused", "split"])
def test_prefill_small(gdn, monkeypatch, B, T, Hk, Hv, D, dtype, init, nsplit, path):
    """Both the single-pass kernel and the two-pass (workspace) path, every
    value-column split, against the oracle."""
    monkeypatch.setenv("GDN_PREFILL_PATH", path)
    if nsplit != "auto":
        monkeypatch.setenv("GDN_PREFILL_NSPLIT", nsplit)
    d = small_prefill(B, T, Hk, Hv, D, dtype, seed=100 + T + D + Hv, init_state=init)
    o, S = gpu_prefill(gdn, d, scale=0.5)
    o_ref, S_ref = oracle_prefill(d, scale=0.5)
    check(o, S, o_ref, S_ref, dtype,
          f"prefill {path} B{B} T{T} Hk{Hk} Hv{Hv} D{D} {dtype} ns={nsplit}")


def test_workspace_path_is_taken_for_small_batches(gdn):
    """48 chains (B=1, the layer's value heads) ask for a workspace; a batch
    with enough chains does not."""
    n = gdn.gdn_prefill_workspace_size(1, 4096, 16, 48, 128, 128, gdn.GDN_BF16, 0)
    # the status word (256 bytes), then T, P and four decay vectors per (chunk, value head)
    assert n == 256 + 64 * 48 * (2 * 64 * 64 * 2 + 4 * 64 * 4)
    assert gdn.gdn_prefill_workspace_size(64, 4096, 16, 48, 128, 128, gdn.GDN_BF16, 0) == 0
    assert gdn.gdn_prefill_workspace_size(2, 130, 16, 48, 128, 128, gdn.GDN_BF16, 1) == \
        256 + (3 + 2) * 48 * (2 * 64 * 64 * 2 + 4 * 64 * 4)


def test_tiny_f32_workload(gdn):
    w = WORKLOADS["tiny_f32"]
    d = generate(w)
    o, S = gpu_prefill(gdn, d)
    o_ref, S_ref = oracle_prefill(d)
    check(o, S, o_ref, S_ref, "f32", w.name)


def test_layer_prefill_4k_workload(gdn):
    w = WORKLOADS["layer_prefill_4k"]
    d = generate(w)
    o, S = gpu_prefill(gdn, d)
    o_ref, S_ref = oracle_prefill(d)
    check(o, S, o_ref, S_ref, "bf16", w.name)


def test_prefill_zero_length_copies_state(gdn):
    d = small_prefill(2, 0, 2, 4, 128, "bf16", seed=5, init_state=True)
    o, S = gpu_prefill(gdn, d)
    assert o.shape == (2, 0, 4, 128)
    np.testing.assert_array_equal(S, d["S0"])
    o, S = gpu_prefill(gdn, d, use_init=False)
    assert not S.any()


def test_prefill_in_place_state(gdn):
    d = small_prefill(1, 150, 2, 4, 128, "bf16", seed=6, init_state=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    s = to_torch(d["S0"], DEV)
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, s, final_state=s)
    torch.cuda.synchronize()
    assert sf.data_ptr() == s.data_ptr()
    o_ref, S_ref = oracle_prefill(d)
    check(from_torch(out), from_torch(s), o_ref, S_ref, "bf16", "in-place state")


def test_prefill_split_invariance(gdn):
    """run(T) == run(T1) then run(T - T1) from its final state (T1 not a
    multiple of 64)."""
    d = small_prefill(1, 300, 2, 6, 128, "bf16", seed=7, init_state=True)
    o, S = gpu_prefill(gdn, d)
    T1 = 101
    d1 = {n: d[n][:, :T1] for n in ("q", "k", "v", "alpha", "beta")}
    d1["S0"] = d["S0"]
    o1, S1 = gpu_prefill(gdn, d1)
    d2 = {n: np.ascontiguousarray(d[n][:, T1:]) for n in ("q", "k", "v", "alpha", "beta")}
    d2["S0"] = S1
    o2, S2 = gpu_prefill(gdn, d2)
    o_ref, S_ref = oracle_prefill(d)
    check(np.concatenate([o1, o2], axis=1), S2, o_ref, S_ref, "bf16", "split at 101")
    check(o, S, o_ref, S_ref, "bf16", "unsplit")


def test_prefill_deterministic(gdn):
    d = small_prefill(1, 333, 2, 6, 128, "bf16", seed=8, init_state=True)
    o1, S1 = gpu_prefill(gdn, d)
    o2, S2 = gpu_prefill(gdn, d)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_prefill_nondefault_stream(gdn):
    d = small_prefill(1, 190, 2, 4, 64, "bf16", seed=9, init_state=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, S = gpu_prefill(gdn, d, stream=s)
    o_ref, S_ref = oracle_prefill(d)
    check(o, S, o_ref, S_ref, "bf16", "side stream")


# ----------------------------------------------------------------- decode
def gpu_decode(gdn, d, scale=1.0):
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    state = to_torch(d["S0"], DEV)
    out = gdn.gdn_decode_step(q, k, v, a, b, state, scale=scale)
    torch.cuda.synchronize()
    return from_torch(out), from_torch(state)


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "bf16"), (128, "f32"), (64, "f32")])
def test_decode_small(gdn, D, dtype):
    d = generate_packed(2, 6, D, dtype, 20 + D, [1] * 5, init_state=True)
    o, S = gpu_decode(gdn, d, scale=0.7)
    o_ref, S_ref = oracle.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], 0.7)
    check(o, S, o_ref, S_ref, dtype, f"decode D{D} {dtype}", o_axes=(0, 1), s_axes=(0, 1))


def _edge_gates(d, case):
    """Gates at the edges of their range: beta = 0 (pure decay of the initial
    state), alpha = beta = 1 (no decay, full overwrite of each key's slot) and
    alpha = 0 on every 37th token (the carried state restarts there). The
    inputs use slow decay (alpha ~ 0.993): at the workloads' decay the exact
    beta = 0 state after 200 tokens, (prod alpha) S0 ~ e^-420 S0, lies below
    the fp32 range, so any fp32 state is 0 against a nonzero fp64 reference."""
    a, b = d["alpha"].copy(), d["beta"].copy()
    if case == "beta0":
        b[...] = 0.0
    elif case == "alpha1_beta1":
        a[...] = 1.0
        b[...] = 1.0
    else:
        a.reshape(-1, a.shape[-1])[::37] = 0.0
    return dict(d, alpha=a, beta=b)


@pytest.mark.parametrize("case", ["beta0", "alpha1_beta1", "alpha0"])
@pytest.mark.parametrize("path", ["fused", "fused1", "split"])
def test_prefill_edge_gates(gdn, monkeypatch, case, path):
    _set_path(monkeypatch, path)
    d = _edge_gates(small_prefill(1, 200, 2, 6, 128, "bf16", seed=71, alpha_shift=-5.0,
                                  init_state=True), case)
    o, S = gpu_prefill(gdn, d)
    o_ref, S_ref = oracle_prefill(d)
    check(o, S, o_ref, S_ref, "bf16", f"edge gates {case} ({path})")


@pytest.mark.parametrize("case", ["beta0", "alpha1_beta1", "alpha0"])
def test_decode_edge_gates(gdn, case):
    d = _edge_gates(generate_packed(2, 6, 128, "bf16", 72, [1] * 40, alpha_shift=-5.0,
                                    init_state=True), case)
    o, S = gpu_decode(gdn, d)
    o_ref, S_ref = oracle.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    check(o, S, o_ref, S_ref, "bf16", f"decode edge gates {case}", o_axes=(0, 1), s_axes=(0, 1))


def test_decode_b256_workload(gdn):
    w = WORKLOADS["decode_b256"]
    d = generate(w)
    o, S = gpu_decode(gdn, d)
    o_ref, S_ref = oracle.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    check(o, S, o_ref, S_ref, "bf16", w.name, o_axes=(0, 1), s_axes=(0, 1))


def test_decode_matches_prefill_T1(gdn):
    d = generate_packed(2, 6, 128, "bf16", 31, [1] * 3, init_state=True)
    o, S = gpu_decode(gdn, d)
    dp = {n: d[n][:, None] for n in ("q", "k", "v", "alpha", "beta")}
    dp["S0"] = d["S0"]
    op, Sp = gpu_prefill(gdn, dp)
    assert max_error(o, op[:, 0], (0, 1)) <= TOL["bf16"]
    assert max_error(S, Sp, (0, 1)) <= TOL["bf16"]  # prefill rounds S to bf16 as an operand


# ------------------------------------------------- K tokens against a slot pool
def gpu_multi(gdn, d, scale=1.0, steps=False):
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    pool = to_torch(d["pool"], DEV)
    src = to_torch(d["src_slot"], DEV)
    dst = to_torch(d["dst_slot"], DEV)
    out, st = gdn.gdn_decode_multi(q, k, v, a, b, pool, src, dst, scale=scale,
                                   want_step_states=steps)
    torch.cuda.synchronize()
    return from_torch(out), from_torch(pool), (from_torch(st) if steps else None)


def check_multi(d, o, pool, st, ref, dtype, label):
    """Outputs and step states per (sequence, head); written slots per
    (slot, head) against the oracle; every other slot bit for bit unchanged."""
    o_ref, pool_ref, st_ref = ref
    B, K = d["q"].shape[:2]
    eo = max_error(o, o_ref, (0, 2)) if K else 0.0
    dst = [int(x) for x in d["dst_slot"] if x >= 0]
    es = max_error(pool[dst], pool_ref[dst], (0, 1)) if dst else 0.0
    et = max_error(st, st_ref, (0, 1, 2)) if st is not None and K else 0.0
    print(f"[parity] {label}: out {eo:.3e} slots {es:.3e} steps {et:.3e} "
          f"(tol {TOL[dtype]:.0e})", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype] and et <= TOL[dtype], label
    keep = sorted(set(range(pool.shape[0])) - set(dst))
    np.testing.assert_array_equal(pool[keep], d["pool"][keep])
    if st is not None and K:
        for b, s in enumerate(d["dst_slot"]):
            if s >= 0:   # the last step state and the written slot are the same registers
                np.testing.assert_array_equal(st[b, K - 1], pool[s])


MULTI = [
    # B, K, Hk, Hv, D, dtype, slot plan
    (3, 1, 1, 2, 64, "bf16", "permute"),
    (4, 4, 2, 6, 128, "bf16", "pairs"),
    (5, 7, 2, 4, 128, "bf16", "inplace"),
    (1, 16, 1, 1, 128, "bf16", "permute"),
    (2, 3, 1, 3, 64, "f32", "permute"),
    (3, 5, 2, 4, 128, "f32", "pairs"),
]


@pytest.mark.parametrize("B,K,Hk,Hv,D,dtype,plan", MULTI)
@pytest.mark.parametrize("steps", [False, True])
def test_decode_multi_small(gdn, B, K, Hk, Hv, D, dtype, plan, steps):
    d = multi_decode(B, K, Hk, Hv, D, dtype, seed=80 + K + D, plan=plan)
    o, pool, st = gpu_multi(gdn, d, 0.8, steps)
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"], 0.8, steps)
    check_multi(d, o, pool, st, ref, dtype, f"multi B{B} K{K} D{D} {dtype} {plan} steps={steps}")


def test_decode_multi_zero_source_and_no_destination(gdn):
    d = multi_decode(4, 3, 2, 4, 128, "bf16", seed=90, plan="permute")
    d["src_slot"][[0, 2]] = -1       # new sequences: zero state
    d["dst_slot"][[1, 2]] = -1       # verification only: nothing written
    o, pool, st = gpu_multi(gdn, d, 1.0, True)
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"], 1.0, True)
    check_multi(d, o, pool, st, ref, "bf16", "multi src<0 / dst<0")


def test_decode_multi_zero_tokens_copies_slots(gdn):
    d = multi_decode(3, 0, 1, 2, 64, "f32", seed=91, plan="permute")
    d["src_slot"][1] = -1
    o, pool, _ = gpu_multi(gdn, d)
    assert o.shape == (3, 0, 2, 64)
    for b in range(3):
        s, t = int(d["src_slot"][b]), int(d["dst_slot"][b])
        np.testing.assert_array_equal(pool[t], d["pool"][s] if s >= 0 else 0.0)


def test_decode_multi_slot_past_pool_gives_nan(gdn):
    d = multi_decode(3, 2, 1, 2, 128, "bf16", seed=92, plan="permute")
    d["dst_slot"][1] = d["pool"].shape[0]          # one past the end
    o, pool, st = gpu_multi(gdn, d, 1.0, True)
    from tests.parity import as_f64
    assert np.isnan(as_f64(o[1])).all() and np.isnan(st[1]).all()
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"], 1.0, True)
    keep_b = [0, 2]
    assert max_error(o[keep_b], ref[0][keep_b], (0, 2)) <= TOL["bf16"]
    written = [int(d["dst_slot"][b]) for b in keep_b]
    assert max_error(pool[written], ref[1][written], (0, 1)) <= TOL["bf16"]
    keep = sorted(set(range(pool.shape[0])) - set(written))
    np.testing.assert_array_equal(pool[keep], d["pool"][keep])


def test_decode_multi_padding_tokens_keep_state(gdn):
    """alpha = 1, beta = 0 is an exact identity step on the GPU as well."""
    d = multi_decode(3, 6, 2, 4, 128, "bf16", seed=93, plan="pairs")
    d["alpha"][:, 2:] = 1.0
    d["beta"][:, 2:] = 0.0
    o, pool, st = gpu_multi(gdn, d, 1.0, True)
    for t in range(2, 6):
        np.testing.assert_array_equal(st[:, t], st[:, 1])
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"], 1.0, True)
    check_multi(d, o, pool, st, ref, "bf16", "multi padding tokens")


def test_decode_multi_K1_matches_decode_step(gdn):
    d = multi_decode(5, 1, 2, 6, 128, "bf16", seed=94, plan="inplace")
    o_m, pool, _ = gpu_multi(gdn, d)
    src = d["src_slot"]
    state = to_torch(d["pool"][src], DEV)
    q, k, v, a, b = (to_torch(np.ascontiguousarray(d[n][:, 0]), DEV)
                     for n in ("q", "k", "v", "alpha", "beta"))
    o_s = from_torch(gdn.gdn_decode_step(q, k, v, a, b, state))
    torch.cuda.synchronize()
    S_s = from_torch(state)
    assert max_error(o_m[:, 0], o_s, (0, 1)) <= 1e-5
    assert max_error(pool[src], S_s, (0, 1)) <= 1e-5


@pytest.mark.parametrize("case", ["beta0", "alpha1_beta1", "alpha0"])
def test_decode_multi_edge_gates(gdn, case):
    """The gate edges through the multi-token path: alpha = 0 restarts the
    state (the kernel's decay scalar cannot carry it), beta = 0 is pure
    decay, alpha = beta = 1 overwrites without decay."""
    d = multi_decode(3, 40, 2, 4, 128, "bf16", seed=95, plan="permute", alpha_shift=-5.0)
    d = _edge_gates(d, case)
    o, pool, st = gpu_multi(gdn, d)
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"])
    check_multi(d, o, pool, st, ref, "bf16", f"multi edge gates {case}")


@pytest.mark.parametrize("alpha_shift", [2.0, -5.0])
def test_decode_multi_many_stages(gdn, alpha_shift):
    """K = 37 spans five LDS stages of 8 tokens; at the workloads' decay the
    running product of alpha leaves the scalar's range and is folded back."""
    d = multi_decode(2, 37, 1, 3, 128, "bf16", seed=96, plan="pairs", alpha_shift=alpha_shift)
    o, pool, st = gpu_multi(gdn, d, 0.9, False)
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"], 0.9)
    check_multi(d, o, pool, st, ref, "bf16", f"multi K=37 alpha_shift={alpha_shift}")
    o2, pool2, st2 = gpu_multi(gdn, d, 0.9, True)   # the per-token-state form
    check_multi(d, o2, pool2, st2, ref[:2] + (oracle.decode_multi(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"], d["src_slot"], d["dst_slot"],
        0.9, True)[2],), "bf16", f"multi K=37 alpha_shift={alpha_shift} steps")


def test_spec_decode_workload(gdn):
    w = SPEC_DECODE
    d = multi_decode(w["B"], w["K"], w["Hk"], w["Hv"], w["D"], w["dtype"], w["seed"],
                     plan=w["plan"])
    o, pool, _ = gpu_multi(gdn, d)
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"])
    check_multi(d, o, pool, None, ref, "bf16", w["name"])


# ----------------------------------------------------------------- varlen
def gpu_varlen(gdn, d, use_init=True):
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    cu = to_torch(d["cu_seqlens"], DEV)
    s0 = to_torch(d["S0"], DEV) if use_init and d["S0"] is not None else None
    out, sf = gdn.gdn_varlen_prefill(q, k, v, a, b, cu, s0)
    torch.cuda.synchronize()
    return out, sf


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "bf16"), (64, "f32")])
@pytest.mark.parametrize("path", ["fused", "fused1", "split"])
def test_varlen_small(gdn, monkeypatch, D, dtype, path):
    _set_path(monkeypatch, path)
    lengths = [5, 1, 70, 0, 129, 64, 200]
    d = generate_packed(2, 6, D, dtype, 40 + D, lengths, init_state=True)
    out, sf = gpu_varlen(gdn, d)
    o_ref, S_ref = oracle.varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                                 d["S0"])
    o = from_torch(out)
    cu = d["cu_seqlens"]
    for n in range(len(lengths)):
        if lengths[n] == 0:
            continue
        e = max_error(o[cu[n]:cu[n + 1]][None], o_ref[cu[n]:cu[n + 1]][None], (0, 2))
        assert e <= TOL[dtype], (n, e)
    check(o[:0], from_torch(sf), o_ref[:0], S_ref, dtype, f"varlen {path} D{D} {dtype} states")


@pytest.mark.parametrize("nseq,Hk", [(300, 2), (37, 3), (2100, 1)])
@pytest.mark.parametrize("path", ["default", "fused1"])
def test_varlen_many_sequences(gdn, monkeypatch, nseq, Hk, path):
    """Many short packed sequences (0 to 200 tokens, slow decay, nonzero
    initial states): the one-pass kernel ranks them by length in each
    workgroup (a sort over more keys than threads; a unit count that is, and
    one that is not, a multiple of 8); past 2,048 sequences it keeps the
    index order. Every chain against the oracle."""
    if path != "default":
        _set_path(monkeypatch, path)
    rng = np.random.default_rng(400 + nseq)
    lengths = [int(x) for x in rng.integers(0, 201, nseq)]
    d = generate_packed(Hk, 3 * Hk, 128, "bf16", 401 + nseq, lengths, alpha_shift=-5.0,
                        init_state=True)
    out, sf = gpu_varlen(gdn, d)
    o_ref, S_ref = oracle.varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                                 d["S0"])
    o = from_torch(out)
    cu = d["cu_seqlens"]
    worst = 0.0
    for n in range(nseq):
        if lengths[n]:
            worst = max(worst, max_error(o[cu[n]:cu[n + 1]][None], o_ref[cu[n]:cu[n + 1]][None],
                                         (0, 2)))
    assert worst <= TOL["bf16"], worst
    check(o[:0], from_torch(sf), o_ref[:0], S_ref, "bf16",
          f"varlen {nseq} sequences Hk={Hk} ({path}), outputs {worst:.3e}")


def test_varlen_matches_per_sequence_prefill(gdn):
    lengths = [77, 300, 64]
    d = generate_packed(2, 6, 128, "bf16", 50, lengths, init_state=True)
    out, sf = gpu_varlen(gdn, d)
    o = from_torch(out)
    S = from_torch(sf)
    cu = d["cu_seqlens"]
    for n in range(len(lengths)):
        dn = {x: np.ascontiguousarray(d[x][cu[n]:cu[n + 1]][None])
              for x in ("q", "k", "v", "alpha", "beta")}
        dn["S0"] = d["S0"][n:n + 1]
        op, Sp = gpu_prefill(gdn, dn)
        np.testing.assert_array_equal(o[cu[n]:cu[n + 1]], op[0])
        np.testing.assert_array_equal(S[n], Sp[0])


# ------------------------------------------------- block-aligned prefix states
SENTINEL = 7.25


def _check_prefix(pre, ref, rows_of, dtype, label):
    """pre: GPU prefix buffer (numpy); ref: oracle list per sequence; rows_of(n, i)
    the row the header assigns to block i of sequence n. Rows no block maps
    to must keep the sentinel."""
    worst = 0.0
    used = set()
    for n, r in enumerate(ref):
        for i in range(r.shape[0]):
            row = rows_of(n, i)
            used.add(row)
            worst = max(worst, max_error(pre[row], r[i], (0,)))
    print(f"[parity] {label}: {len(used)} prefix states, max error {worst:.3e} "
          f"(tol {TOL[dtype]:.0e})", flush=True)
    assert worst <= TOL[dtype], label
    free = sorted(set(range(pre.shape[0])) - used)
    assert np.all(pre[free] == SENTINEL), "rows no block maps to were written"


PREFIX_DENSE = [
    # path, nsplit, dtype, D, every  (kernel reached)
    ("fused", "auto", "bf16", 128, 1),   # prefill_kernel
    ("fused", "8", "bf16", 128, 3),
    ("fused", "1", "bf16", 128, 1),      # fused2_kernel
    ("fused", "1", "bf16", 128, 3),
    ("split", "1", "bf16", 128, 2),      # chain_kernel
    ("split", "4", "bf16", 128, 1),      # chain_db_kernel
    ("split", "2", "bf16", 64, 3),       # chain_db_kernel, D = 64
    ("split", "2", "f32", 64, 1),        # chain_kernel, fp32
    ("fused", "auto", "f32", 128, 2),
]


@pytest.mark.parametrize("path,nsplit,dtype,D,every", PREFIX_DENSE)
def test_prefill_prefix_states(gdn, monkeypatch, path, nsplit, dtype, D, every):
    monkeypatch.setenv("GDN_PREFILL_PATH", path)
    # a call with prefix states never segments: compare with the same path
    monkeypatch.setenv("GDN_PREFILL_SEGMENTS", "0")
    if nsplit != "auto":
        monkeypatch.setenv("GDN_PREFILL_NSPLIT", nsplit)
    B, T, Hk, Hv = 2, 450, 2, 6
    d = small_prefill(B, T, Hk, Hv, D, dtype, seed=110 + every, init_state=True)
    L = 64 * every
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    s0 = to_torch(d["S0"], DEV)
    pre = torch.full((gdn.prefix_state_rows(B, T, every, False), Hv, D, D), SENTINEL,
                     dtype=torch.float32, device=DEV)
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, s0, prefix_states=pre,
                                      prefix_interval=every)
    out0, sf0 = gdn.gdn_prefill_chunked(q, k, v, a, b, s0)
    torch.cuda.synchronize()
    # emitting prefix states leaves the outputs and final states bit for bit
    assert torch.equal(out, out0) and torch.equal(sf, sf0)
    flat = {n: d[n].reshape((-1,) + d[n].shape[2:]) for n in ("q", "k", "v", "alpha", "beta")}
    ref = oracle.prefix_states(flat["q"], flat["k"], flat["v"], flat["alpha"], flat["beta"],
                               [0, T, 2 * T], L, d["S0"])
    _check_prefix(from_torch(pre), ref, lambda n, i: n * (T // L) + i, dtype,
                  f"prefix states {path} ns={nsplit} {dtype} D{D} L={L}")


@pytest.mark.parametrize("path", ["fused", "fused1", "split"])
def test_varlen_prefix_states(gdn, monkeypatch, path):
    _set_path(monkeypatch, path)
    lengths = [300, 64, 1, 640, 127, 128, 0, 257]
    every = 2
    L = 64 * every
    d = generate_packed(2, 6, 128, "bf16", 120, lengths, init_state=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    cu_t = to_torch(d["cu_seqlens"], DEV)
    s0 = to_torch(d["S0"], DEV)
    total, N = int(d["cu_seqlens"][-1]), len(lengths)
    pre = torch.full((gdn.prefix_state_rows(N, total, every, True), 6, 128, 128), SENTINEL,
                     dtype=torch.float32, device=DEV)
    out, sf = gdn.gdn_varlen_prefill(q, k, v, a, b, cu_t, s0, prefix_states=pre,
                                     prefix_interval=every)
    out0, sf0 = gdn.gdn_varlen_prefill(q, k, v, a, b, cu_t, s0)
    torch.cuda.synchronize()
    assert torch.equal(out, out0) and torch.equal(sf, sf0)
    cu = d["cu_seqlens"]
    ref = oracle.prefix_states(d["q"], d["k"], d["v"], d["alpha"], d["beta"], cu, L, d["S0"])
    _check_prefix(from_torch(pre), ref, lambda n, i: int(cu[n]) // L + n + i, "bf16",
                  f"varlen prefix states ({path})")


def test_layer_prefill_4k_prefix_states(gdn):
    """The layer workload with a state every 1024 tokens (16 chunks)."""
    w = WORKLOADS["layer_prefill_4k"]
    d = generate(w)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    pre = torch.full((gdn.prefix_state_rows(1, w.T, 16, False), w.Hv, w.D, w.D), SENTINEL,
                     dtype=torch.float32, device=DEV)
    gdn.gdn_prefill_chunked(q, k, v, a, b, None, prefix_states=pre, prefix_interval=16)
    torch.cuda.synchronize()
    flat = {n: d[n].reshape((-1,) + d[n].shape[2:]) for n in ("q", "k", "v", "alpha", "beta")}
    ref = oracle.prefix_states(flat["q"], flat["k"], flat["v"], flat["alpha"], flat["beta"],
                               [0, w.T], 1024)
    _check_prefix(from_torch(pre), ref, lambda n, i: i, "bf16", f"{w.name} prefix states")


# ------------------------------------------------- input preparation in the kernels
QK, GL = 1, 2   # GDN_QK_L2NORM, GDN_GATE_LOGITS


def _prepared_inputs(gen, flags):
    """Raw q, k (flag 1) and gate logits (flag 2) of a seed, the rest as the
    plain recipe gives them for the same seed (the generator draws the same
    numbers either way)."""
    plain, raw = gen(False), gen(True)
    d = dict(plain)
    if flags & QK:
        d["q"], d["k"] = raw["q"], raw["k"]
    if flags & GL:
        d["alpha"], d["beta"] = raw["alpha"], raw["beta"]
    return d


PREP_DENSE = [
    # path, nsplit, dtype, D, flags
    ("fused", "auto", "bf16", 128, QK | GL),
    ("fused", "2", "bf16", 128, QK),
    ("fused", "1", "bf16", 128, QK | GL),   # fused2_kernel
    ("fused", "1", "bf16", 128, QK),
    ("fused", "auto", "bf16", 128, GL),
    ("split", "1", "bf16", 128, QK | GL),     # chain_kernel
    ("split", "4", "bf16", 128, QK | GL),     # chain_db_kernel
    ("split", "2", "bf16", 64, QK),
    ("split", "2", "f32", 64, QK | GL),
    ("fused", "auto", "f32", 128, QK | GL),
]


@pytest.mark.parametrize("path,nsplit,dtype,D,flags", PREP_DENSE)
def test_prefill_prepared_inputs(gdn, monkeypatch, path, nsplit, dtype, D, flags):
    monkeypatch.setenv("GDN_PREFILL_PATH", path)
    if nsplit != "auto":
        monkeypatch.setenv("GDN_PREFILL_NSPLIT", nsplit)
    d = _prepared_inputs(lambda raw: small_prefill(2, 200, 2, 6, D, dtype, seed=130 + flags,
                                                   init_state=True, raw=raw), flags)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, to_torch(d["S0"], DEV), flags=flags)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                  flags=flags)
    check(from_torch(out), from_torch(sf), o_ref, S_ref, dtype,
          f"prepared inputs flags={flags} {path} ns={nsplit} {dtype} D{D}")


@pytest.mark.parametrize("Hk,Hv", [(2, 2), (2, 4), (2, 6), (1, 4)])
@pytest.mark.parametrize("flags", [0, QK | GL])
@pytest.mark.parametrize("prep", ["grouped", "per_head"])
def test_two_pass_prep_head_groups(gdn, monkeypatch, Hk, Hv, flags, prep):
    """The two-pass prefill (bf16, d = 128, four column slices) with 1 .. 4
    value heads per q/k head: one prep workgroup per q/k head for 2 or 3 of
    them (sharing the K, Q staging and Gram products), one per value head
    otherwise or with GDN_PREP=1."""
    monkeypatch.setenv("GDN_PREFILL_PATH", "split")
    monkeypatch.setenv("GDN_PREFILL_NSPLIT", "4")
    if prep == "per_head":
        monkeypatch.setenv("GDN_PREP", "1")
    d = _prepared_inputs(lambda raw: small_prefill(1, 200, Hk, Hv, 128, "bf16", seed=150 + Hv + flags,
                                                   init_state=True, raw=raw), flags)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, to_torch(d["S0"], DEV), flags=flags)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                  flags=flags)
    check(from_torch(out), from_torch(sf), o_ref, S_ref, "bf16",
          f"two-pass prep {prep} Hk{Hk} Hv{Hv} flags={flags}")


@pytest.mark.parametrize("path", ["fused", "fused1", "split"])
def test_varlen_prepared_inputs_and_zero_rows(gdn, monkeypatch, path):
    """Raw rows of zeros normalise to zero (the 1e-6 under the root): such a
    token writes nothing and reads nothing."""
    _set_path(monkeypatch, path)
    lengths = [150, 1, 64, 300]
    d = generate_packed(2, 6, 128, "bf16", 140, lengths, init_state=True, raw=True)
    d["k"][[3, 70, 71, 400]] = 0
    d["q"][[5, 200]] = 0
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    pre = torch.full((gdn.prefix_state_rows(len(lengths), int(d["cu_seqlens"][-1]), 1, True), 6,
                      128, 128), SENTINEL, dtype=torch.float32, device=DEV)
    out, sf = gdn.gdn_varlen_prefill(q, k, v, a, b, to_torch(d["cu_seqlens"], DEV),
                                     to_torch(d["S0"], DEV), flags=QK | GL, prefix_states=pre,
                                     prefix_interval=1)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                                 d["S0"], flags=QK | GL)
    o = from_torch(out)
    cu = d["cu_seqlens"]
    for n in range(len(lengths)):
        e = max_error(o[cu[n]:cu[n + 1]][None], o_ref[cu[n]:cu[n + 1]][None], (0, 2))
        assert e <= TOL["bf16"], (n, e)
    check(o[:0], from_torch(sf), o_ref[:0], S_ref, "bf16", f"varlen prepared ({path}) states")
    ref = oracle.prefix_states(d["q"], d["k"], d["v"], d["alpha"], d["beta"], cu, 64, d["S0"],
                               flags=QK | GL)
    _check_prefix(from_torch(pre), ref, lambda n, i: int(cu[n]) // 64 + n + i, "bf16",
                  f"varlen prepared prefix states ({path})")


@pytest.mark.parametrize("flags", [QK, GL, QK | GL])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32")])
def test_decode_prepared_inputs(gdn, flags, D, dtype):
    d = _prepared_inputs(lambda raw: generate_packed(2, 6, D, dtype, 150 + flags, [1] * 5,
                                                     init_state=True, raw=raw), flags)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    state = to_torch(d["S0"], DEV)
    out = gdn.gdn_decode_step(q, k, v, a, b, state, scale=0.7, flags=flags)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], 0.7,
                                 flags=flags)
    check(from_torch(out), from_torch(state), o_ref, S_ref, dtype,
          f"decode prepared flags={flags} D{D} {dtype}", o_axes=(0, 1), s_axes=(0, 1))


@pytest.mark.parametrize("steps", [False, True])
def test_decode_multi_prepared_inputs(gdn, steps):
    d = multi_decode(4, 5, 2, 6, 128, "bf16", seed=160, plan="permute", raw=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    pool = to_torch(d["pool"], DEV)
    out, st = gdn.gdn_decode_multi(q, k, v, a, b, pool, to_torch(d["src_slot"], DEV),
                                   to_torch(d["dst_slot"], DEV), flags=QK | GL,
                                   want_step_states=steps)
    torch.cuda.synchronize()
    ref = oracle.decode_multi(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["pool"],
                              d["src_slot"], d["dst_slot"], 1.0, steps, flags=QK | GL)
    check_multi(d, from_torch(out), from_torch(pool), from_torch(st) if steps else None, ref,
                "bf16", f"multi prepared steps={steps}")


def test_layer_prefill_4k_prepared_inputs(gdn):
    """The layer workload from raw q, k and gate logits."""
    w = WORKLOADS["layer_prefill_4k"]
    d = generate(w, raw=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, None, flags=QK | GL)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None,
                                  flags=QK | GL)
    check(from_torch(out), from_torch(sf), o_ref, S_ref, "bf16", f"{w.name} prepared inputs")


# ------------------------------------------------- segmented prefill (few long sequences)
SEG_CASES = [
    # B, T, Hk, Hv, D, segments, init, flags, inner path, alpha shift
    (1, 450, 1, 2, 128, "3", True, 0, "auto", 2.0),
    (2, 700, 2, 4, 128, "2", True, 0, "auto", 2.0),
    (1, 1000, 1, 3, 64, "5", False, 0, "auto", 2.0),
    (1, 640, 2, 6, 128, "4", True, QK | GL, "auto", 2.0),
    (1, 513, 1, 2, 128, "8", True, 0, "fused", 2.0),
    # slow decay (alpha ~ 0.993): the state carried across segments matters,
    # so the segment maps, their scan and the corrections carry the result
    (1, 1300, 1, 2, 128, "6", True, 0, "auto", -5.0),
    (2, 777, 2, 4, 128, "3", False, 0, "auto", -5.0),
    (1, 900, 1, 3, 64, "4", True, 0, "auto", -5.0),
    (1, 1024, 2, 6, 128, "8", True, QK | GL, "auto", -5.0),
    (1, 700, 1, 2, 128, "5", True, 0, "fused", -5.0),
    # one-pass segment passes with one workgroup per chain (identity start,
    # token stride 0 for v)
    (1, 700, 1, 2, 128, "5", True, 0, "fused1", -5.0),
    (1, 640, 2, 6, 128, "4", True, QK | GL, "fused1", 2.0),
]


@pytest.mark.parametrize("B,T,Hk,Hv,D,segs,init,flags,inner,ashift", SEG_CASES)
def test_segmented_prefill(gdn, monkeypatch, B, T, Hk, Hv, D, segs, init, flags, inner, ashift):
    """Segments forced: every segment from zero and from the identity, the
    scan of the segment maps and the corrections, against the oracle."""
    monkeypatch.setenv("GDN_PREFILL_SEGMENTS", segs)
    if inner != "auto":
        _set_path(monkeypatch, inner)
    gen = lambda raw: small_prefill(B, T, Hk, Hv, D, "bf16", seed=170 + T, init_state=init,
                                    raw=raw, alpha_shift=ashift)
    d = _prepared_inputs(gen, flags) if flags else gen(False)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    s0 = to_torch(d["S0"], DEV) if init else None
    n = gdn.gdn_prefill_workspace_size(B, T, Hk, Hv, D, D, gdn.GDN_BF16, 0)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, s0, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                  d["S0"] if init else None, flags=flags)
    check(from_torch(out), from_torch(sf), o_ref, S_ref, "bf16",
          f"segmented P={segs} B{B} T{T} Hv{Hv} D{D} init={init} flags={flags} ({inner}) "
          f"alpha shift {ashift}")


def test_prefill_two_pass_in_place_and_captured(gdn, monkeypatch):
    """The two-pass run of one sequence with the state updated in place
    (initial and final state the same buffer), and the same call captured in
    a graph and replayed: both equal the plain call bit for bit, every
    replay included."""
    monkeypatch.setenv("GDN_PREFILL_SEGMENTS", "0")
    T = 64 * 24 + 9
    d = small_prefill(1, T, 2, 6, 128, "bf16", seed=199, init_state=True, alpha_shift=-5.0)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    n = gdn.gdn_prefill_workspace_size(1, T, 2, 6, 128, 128, gdn.GDN_BF16, 0)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    ref_o, ref_s = gdn.gdn_prefill_chunked(q, k, v, a, b, to_torch(d["S0"], DEV), workspace=ws)
    st = to_torch(d["S0"], DEV)
    out = torch.empty(v.shape, dtype=torch.bfloat16, device=DEV)
    gdn.gdn_prefill_chunked(q, k, v, a, b, st, out=out, final_state=st, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o)
    assert torch.equal(st, ref_s)
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    check(from_torch(out), from_torch(st), o_ref, S_ref, "bf16", "two-pass in place")
    s0_g = to_torch(d["S0"], DEV)
    sf_g = torch.empty_like(s0_g)
    out_g = torch.empty_like(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn.gdn_prefill_chunked(q, k, v, a, b, s0_g, out=out_g, final_state=sf_g, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.zero_()
        sf_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref_o), r
        assert torch.equal(sf_g, ref_s), r


def test_debug_checks_reject_bad_offsets(gdn, monkeypatch):
    """GDN_DEBUG=1: malformed cu_seqlens (not starting at 0, decreasing, not
    ending at total_T) are refused with GDN_ERR_BAD_SHAPE before any kernel
    runs; well-formed ones pass, and the workspace status word reads clean
    after a two-pass call."""
    monkeypatch.setenv("GDN_DEBUG", "1")
    d = generate_packed(2, 6, 128, "bf16", 77, [100, 50, 170], init_state=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    total = int(d["cu_seqlens"][-1])
    for bad in ([5, 100, 150, 320], [0, 150, 100, 320], [0, 100, 150, 300]):
        cu = torch.tensor(bad, dtype=torch.int32, device=DEV)
        with pytest.raises(gdn.GDNError) as ei:
            gdn.gdn_varlen_prefill(q, k, v, a, b, cu, None)
        assert ei.value.status == 2, bad
    assert total == 320
    cu = to_torch(d["cu_seqlens"], DEV)
    out, sf = gdn.gdn_varlen_prefill(q, k, v, a, b, cu, to_torch(d["S0"], DEV))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                                 d["S0"])
    o, c = from_torch(out), d["cu_seqlens"]
    for n in range(3):
        e = max_error(o[c[n]:c[n + 1]][None], o_ref[c[n]:c[n + 1]][None], (0, 2))
        assert e <= TOL["bf16"], (n, e)
    check(o[:0], from_torch(sf), o_ref[:0], S_ref, "bf16", "GDN_DEBUG varlen states")


@pytest.mark.parametrize("D,segs", [(128, "4"), (128, "7"), (64, "5")])
def test_segmented_passes_merged_match_separate(gdn, monkeypatch, D, segs):
    """The two segment passes (from zero, and from the identity with v = 0)
    as one launch over twice the chains, against the same passes launched
    one after the other: both within tolerance of the oracle, and the same
    bits (each value column's arithmetic does not depend on the slicing).
    Both on the double-buffered chain kernel, the one with the merged
    launch (the one-wave-per-SIMD chain groups the keys of an MFMA step
    differently, which changes the last bit of some outputs)."""
    monkeypatch.setenv("GDN_PREFILL_SEGMENTS", segs)
    monkeypatch.setenv("GDN_CHAIN", "db")
    d = small_prefill(1, 1100, 2, 6, D, "bf16", seed=197 + D, alpha_shift=-5.0, init_state=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    s0 = to_torch(d["S0"], DEV)
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    res = {}
    for merge in ("0", "1"):
        monkeypatch.setenv("GDN_PREFILL_SEG_MERGE", merge)
        res[merge] = gdn.gdn_prefill_chunked(q, k, v, a, b, s0)
        torch.cuda.synchronize()
        check(from_torch(res[merge][0]), from_torch(res[merge][1]), o_ref, S_ref, "bf16",
              f"segmented P={segs} D{D} merged={merge}")
    assert torch.equal(res["0"][0], res["1"][0])
    assert torch.equal(res["0"][1], res["1"][1])


@pytest.mark.parametrize("segs", ["3", "4"])
def test_segmented_prefill_without_final_state(gdn, monkeypatch, segs):
    """Segmented with no final state asked for (the scan then writes the last
    state to workspace scratch): outputs bit-equal to those of the same call
    with a final state, and within tolerance of the oracle."""
    monkeypatch.setenv("GDN_PREFILL_SEGMENTS", segs)
    d = small_prefill(1, 900, 1, 2, 128, "bf16", seed=191, alpha_shift=-5.0, init_state=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    s0 = to_torch(d["S0"], DEV)
    n = gdn.gdn_prefill_workspace_size(1, 900, 1, 2, 128, 128, gdn.GDN_BF16, 0)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    out_f, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, s0, workspace=ws)
    out_n, none = gdn.gdn_prefill_chunked(q, k, v, a, b, s0, workspace=ws,
                                          want_final_state=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(out_f, out_n)
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    check(from_torch(out_n), from_torch(sf), o_ref, S_ref, "bf16",
          f"segmented P={segs} without final state")


def test_layer_prefill_4k_tp8_segmented(gdn, monkeypatch):
    """The per-GPU share of the layer at 8-way head-group sharding: few
    enough chains that the segmented path is chosen by itself; its result
    matches the oracle, as does the unsegmented path's."""
    w = WORKLOADS["layer_prefill_4k_tp8"]
    d = generate(w)
    n_seg = gdn.gdn_prefill_workspace_size(1, w.T, w.Hk, w.Hv, w.D, w.D, gdn.GDN_BF16, 0)
    monkeypatch.setenv("GDN_PREFILL_SEGMENTS", "0")
    n_plain = gdn.gdn_prefill_workspace_size(1, w.T, w.Hk, w.Hv, w.D, w.D, gdn.GDN_BF16, 0)
    assert n_seg > n_plain > 0, (n_seg, n_plain)
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    for label in ("unsegmented", "segmented"):
        if label == "segmented":
            monkeypatch.delenv("GDN_PREFILL_SEGMENTS")
        out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, None)
        torch.cuda.synchronize()
        check(from_torch(out), from_torch(sf), o_ref, S_ref, "bf16", f"{w.name} {label}")


def test_tp8_shapes_slow_decay_segmented(gdn, monkeypatch):
    """The TP8 shapes at slow decay and with an initial state, chosen
    segmentation against the oracle; the two paths round differently, which
    shows that the segmented one ran."""
    d = small_prefill(1, 4096, 2, 6, 128, "bf16", seed=180, alpha_shift=-5.0, init_state=True)
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    s0 = to_torch(d["S0"], DEV)
    o_ref, S_ref = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    res = {}
    for label, env in (("unsegmented", "0"), ("segmented", None)):
        if env is None:
            monkeypatch.delenv("GDN_PREFILL_SEGMENTS", raising=False)
        else:
            monkeypatch.setenv("GDN_PREFILL_SEGMENTS", env)
        out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, s0)
        torch.cuda.synchronize()
        res[label] = (from_torch(out), from_torch(sf))
        check(*res[label], o_ref, S_ref, "bf16", f"TP8 shapes slow decay {label}")
    assert not np.array_equal(res["segmented"][1], res["unsegmented"][1])


# ----------------------------------------------------------------- full-size, every chain
def _all_chains_check(d, results, cu, Hv, label):
    """Every (sequence, value head) chain of a packed batch against the fp64
    oracle, on host threads; each chain is compared as soon as it is done, so
    the fp64 outputs are never held whole. `results` maps a path label to the
    GPU's (out [total, Hv, D] as host bf16 bits, final states [N, Hv, D, D])."""
    from concurrent.futures import ThreadPoolExecutor
    N = len(cu) - 1
    worst = {name: [0.0, 0.0] for name in results}

    def work(nh):
        n, h = nh
        s0 = d["S0"][n, h] if d.get("S0") is not None else None
        o_ref, S_ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], int(cu[n]),
                                    int(cu[n + 1]), h, s0)
        errs = {}
        for name, (o, S) in results.items():
            errs[name] = (slice_error(o[int(cu[n]):int(cu[n + 1]), h], o_ref),
                          slice_error(S[n, h], S_ref))
        return errs

    chains = [(n, h) for n in range(N) for h in range(Hv)]
    with ThreadPoolExecutor(oracle.default_threads()) as ex:
        for errs in ex.map(work, chains):
            for name, (eo, es) in errs.items():
                worst[name][0] = max(worst[name][0], eo)
                worst[name][1] = max(worst[name][1], es)
    for name, (eo, es) in worst.items():
        print(f"[parity] {label} ({name}): all {len(chains)} chains: out {eo:.3e} "
              f"state {es:.3e}", flush=True)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (name, eo, es)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_long_prefill_256k_workload_all_chains(gdn):
    """The 262,144-token layer prefill: all 48 value-head chains against the
    oracle over their full length."""
    w = WORKLOADS["long_prefill_256k"]
    d = generate(w)
    flat = {n: d[n].reshape((-1,) + d[n].shape[2:]) for n in ("q", "k", "v", "alpha", "beta")}
    flat["S0"] = None
    q, k, v, a, b = _t(d, ("q", "k", "v", "alpha", "beta"))
    out, sf = gdn.gdn_prefill_chunked(q, k, v, a, b, None)
    torch.cuda.synchronize()
    res = {"default": (from_torch(out.reshape(-1, w.Hv, w.D)), from_torch(sf))}
    del q, k, v, a, b, out, sf
    _all_chains_check(flat, res, np.array([0, w.T]), w.Hv, w.name)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_varlen_64seq_workload_all_chains(gdn, monkeypatch):
    """The 64-sequence packed batch (nonzero initial states): all 3,072
    chains against the oracle, for the default path (one pass: the chains
    fill the chip) and for the two-pass path."""
    w = WORKLOADS["varlen_64seq"]
    d = generate(w)
    res = {}
    for path in ("default", "split"):
        if path == "split":
            monkeypatch.setenv("GDN_PREFILL_PATH", "split")
        out, sf = gpu_varlen(gdn, d)
        res[path] = (from_torch(out), from_torch(sf))
        del out, sf
        torch.cuda.empty_cache()
    monkeypatch.delenv("GDN_PREFILL_PATH", raising=False)
    _all_chains_check(d, res, d["cu_seqlens"], w.Hv, w.name)


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("T,alpha", [(4096, "slow"), (4096, "one"), (65536, "slow")])
def test_layer_shapes_slow_decay_all_chains(gdn, T, alpha):
    """Slow decay at the layer's shapes (16 q/k heads, 48 value heads, d=128)
    on the default path: alpha = exp(-softplus(N(0,1) - 5)) (median ~0.993)
    or alpha = 1, beta = sigmoid(N(0,1) - 2), initial states 0.1 N(0,1). Here
    the state carried across chunks dominates the outputs (at the
    workloads' decay a chunk scales it by ~1e-61), so a wrong carry fails."""
    d = small_prefill(1, T, 16, 48, 128, "bf16", seed=300 + T // 4096 + (alpha == "one"),
                      alpha_shift=-5.0, beta_shift=-2.0, init_state=True)
    if alpha == "one":
        d["alpha"][:] = 1.0
    flat = {n: d[n].reshape((-1,) + d[n].shape[2:]) for n in ("q", "k", "v", "alpha", "beta")}
    flat["S0"] = d["S0"]
    out, sf = gpu_prefill(gdn, d)
    res = {"default": (out.reshape(-1, 48, 128), sf)}
    _all_chains_check(flat, res, np.array([0, T]), 48, f"layer shapes T={T} alpha {alpha}")


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_varlen_layer_shapes_slow_decay_all_chains(gdn):
    """A packed batch at the layer's shapes with slow decay and nonzero
    initial states on the default path: 12 sequences x 48 value heads fill the
    chip, so the single-pass kernel with its longest-first, XCD-balanced order
    runs (ragged and one-token sequences included). Every chain against the
    oracle; the state carried across chunks dominates the outputs."""
    lengths = [4096, 1, 3000, 64, 2500, 700, 130, 1900, 65, 1200, 3333, 10]
    d = generate_packed(16, 48, 128, "bf16", 310, lengths, alpha_shift=-5.0, beta_shift=-2.0,
                        init_state=True)
    out, sf = gpu_varlen(gdn, d)
    res = {"default": (from_torch(out), from_torch(sf))}
    _all_chains_check(d, res, d["cu_seqlens"], 48, "packed layer shapes, slow decay")


def test_slow_decay_stress_diagnostic(gdn):
    """Slow decay (alpha ~ 0.99, small beta) exercises the carried state across
    many chunks, which the workloads' fast decay hides. Diagnostic bound."""
    d = small_prefill(1, 4096, 2, 6, 128, "bf16", seed=60, alpha_shift=-5.0, beta_shift=-2.0,
                      init_state=True)
    o, S = gpu_prefill(gdn, d)
    o_ref, S_ref = oracle_prefill(d)
    check(o, S, o_ref, S_ref, "bf16", "slow-decay stress T=4096")


# ------------------------------------------------- HIP graph capture
def test_graph_capture_replays_match_eager(gdn, monkeypatch):
    """Decode step, K-token decode and prefill (two-pass and segmented)
    captured in one HIP graph (the calls enqueue kernels only: no
    allocation, copy or memset), replayed three times with eager work and
    synchronisations between replays; every replay equals the eager calls
    bit for bit."""
    monkeypatch.setenv("GDN_PREFILL_SEGMENTS", "4")  # the small prefill below segments
    dd = generate_packed(2, 6, 128, "bf16", 190, [1] * 8, init_state=True)
    dq, dk, dv, da, db = _t(dd, ("q", "k", "v", "alpha", "beta"))
    dm = multi_decode(4, 3, 2, 6, 128, "bf16", seed=192, plan="pairs")
    mq, mk, mv, ma, mb = _t(dm, ("q", "k", "v", "alpha", "beta"))
    src, dst = to_torch(dm["src_slot"], DEV), to_torch(dm["dst_slot"], DEV)
    dp = small_prefill(1, 700, 2, 6, 128, "bf16", seed=191, init_state=True)
    pq, pk, pv, pa, pb = _t(dp, ("q", "k", "v", "alpha", "beta"))
    ps0 = to_torch(dp["S0"], DEV)
    nws = gdn.gdn_prefill_workspace_size(1, 700, 2, 6, 128, 128, gdn.GDN_BF16, 0)

    def buffers():
        return dict(state=to_torch(dd["S0"], DEV),
                    d_out=torch.empty(dv.shape, dtype=torch.bfloat16, device=DEV),
                    pool=to_torch(dm["pool"], DEV),
                    m_out=torch.empty(mv.shape, dtype=torch.bfloat16, device=DEV),
                    p_out=torch.empty(pv.shape, dtype=torch.bfloat16, device=DEV),
                    p_sf=torch.empty((1, 6, 128, 128), dtype=torch.float32, device=DEV),
                    ws=torch.empty(nws, dtype=torch.uint8, device=DEV))

    def calls(x):
        gdn.gdn_decode_step(dq, dk, dv, da, db, x["state"], out=x["d_out"])
        gdn.gdn_decode_multi(mq, mk, mv, ma, mb, x["pool"], src, dst, out=x["m_out"])
        gdn.gdn_prefill_chunked(pq, pk, pv, pa, pb, ps0, out=x["p_out"], final_state=x["p_sf"],
                                workspace=x["ws"])

    xg, xe = buffers(), buffers()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(xg)
    torch.cuda.synchronize()
    for r in range(3):
        g.replay()
        calls(xe)
        torch.cuda.synchronize()
        for name in ("state", "d_out", "pool", "m_out", "p_out", "p_sf"):
            assert torch.equal(xg[name], xe[name]), (r, name)
    o_ref, S_ref = oracle.prefill(dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], dp["S0"])
    check(from_torch(xg["p_out"]), from_torch(xg["p_sf"]), o_ref, S_ref, "bf16",
          "graph-captured segmented prefill")
