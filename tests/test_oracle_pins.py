"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test fixes the oracle to something independent of its own code: a
hand-worked example, a closed form of the recurrence for special inputs, an
algebraic invariant, or the literal matrix form of the rule on tiny inputs.
The rule is the gated delta rule used by the Gated DeltaNet layers named in
"The Hybrid Attention in Qwen3.8-27B" (section "Why 27B parameters can carry
262K tokens"): S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T and
o_t = S_t q_t, with value head h reading q/k head h // (Hv / Hk).

Which planted mistake each pin catches:
  hand-worked  : any wrong term, sign or order on a 2x2 case
  decay-only   : alpha taken from the wrong token/head, initial state ignored
  single-token : o from S_{t-1} instead of S_t, S vs S^T, beta dropped, scale
  overwrite    : alpha applied after the write, alpha missing from the erase,
                 a wrong sign in the erase term
  literal form : the rank-1 rewrite of the matrix product
  memory/repeat: overwrite semantics of the delta rule
  linearity    : a hidden non-linearity in (S0, V)
  split        : state hand-over between calls
  chunk mirror : the chunked algebra the GPU evaluates
  slot pool    : src/dst routing, per-token states, padding tokens, K = 0,
                 out-of-range slots (the multi-token decode)
"""
import json
import os

import numpy as np
import pytest

import oracle
from gdn_synth import bf16_bits, bf16_to_f32, small_prefill
from tests.chunk_mirror import chunk_chain

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, T, Hk, Hv, dk, dv, unit_k=True):
    q = rng.standard_normal((T, Hk, dk)).astype(np.float32)
    k = rng.standard_normal((T, Hk, dk)).astype(np.float32)
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, dv)).astype(np.float32)
    alpha = rng.uniform(0.05, 1.0, (T, Hv)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (T, Hv)).astype(np.float32)
    return q, k, v, alpha, beta


def _f64(x):
    return np.asarray(x, np.float64)


# ------------------------------------------------------------ hand-worked
def test_hand_worked_two_tokens():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_two_tokens.json")))
    inp = g["inputs"]
    q = np.array(inp["q"], np.float32)[:, None, :]
    k = np.array(inp["k"], np.float32)[:, None, :]
    v = np.array(inp["v"], np.float32)[:, None, :]
    a = np.array(inp["alpha"], np.float32)[:, None]
    b = np.array(inp["beta"], np.float32)[:, None]
    o, S = oracle.chain(q, k, v, a, b, 0, 2, 0)
    np.testing.assert_array_equal(o, np.array(g["expected"]["o"]))
    np.testing.assert_array_equal(S, np.array(g["expected"]["S_final"]))
    o2, S2 = oracle.chain(q, k, v, a, b, 0, 2, 0, scale=2.0)
    np.testing.assert_array_equal(o2, 2.0 * np.array(g["expected"]["o"]))
    np.testing.assert_array_equal(S2, S)


# ------------------------------------------------------------ closed forms
def test_decay_only_beta_zero():
    """beta = 0: S_T = (prod a) S0 and o_t = (prod_{s<=t} a_s) S0 q_t."""
    rng = np.random.default_rng(1)
    T, Hk, Hv, d = 37, 2, 6, 16
    q, k, v, alpha, _ = _rand_inputs(rng, T, Hk, Hv, d, d)
    beta = np.zeros((T, Hv), np.float32)
    S0 = rng.standard_normal((1, Hv, d, d)).astype(np.float32)
    o, S = oracle.prefill(q[None], k[None], v[None], alpha[None], beta[None], S0)
    for h in range(Hv):
        g = h // (Hv // Hk)
        cp = np.cumprod(_f64(alpha[:, h]))
        exp_o = cp[:, None] * (_f64(q[:, g]) @ _f64(S0[0, h]).T)
        np.testing.assert_allclose(o[0, :, h], exp_o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S[0, h], cp[-1] * _f64(S0[0, h]), rtol=1e-12, atol=1e-300)


def test_single_token_from_zero():
    """T = 1, S0 = 0: S_1 = b v k^T and o = scale * b (k.q) v (q != k)."""
    rng = np.random.default_rng(2)
    Hk, Hv, dk, dv = 3, 6, 8, 12
    q, k, v, alpha, beta = _rand_inputs(rng, 1, Hk, Hv, dk, dv)
    o, S = oracle.prefill(q[None], k[None], v[None], alpha[None], beta[None], None, scale=0.75)
    for h in range(Hv):
        g = h // (Hv // Hk)
        kq = float(_f64(k[0, g]) @ _f64(q[0, g]))
        np.testing.assert_allclose(o[0, 0, h], 0.75 * float(beta[0, h]) * kq * _f64(v[0, h]),
                                   rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S[0, h], float(beta[0, h]) * np.outer(_f64(v[0, h]), _f64(k[0, g])),
                                   rtol=1e-12, atol=1e-14)


def _exact_unit_keys(rng, T, H, d, nnz):
    """Keys with nnz entries of +-1/sqrt(nnz) (nnz a power of 4): norm exactly 1."""
    k = np.zeros((T, H, d), np.float32)
    val = np.float32(1.0 / np.sqrt(nnz))
    for t in range(T):
        for h in range(H):
            idx = rng.choice(d, nnz, replace=False)
            k[t, h, idx] = val * rng.choice([-1.0, 1.0], nnz)
    return k


def test_exact_overwrite_beta_one():
    """beta = 1 and unit k: after the write S_t k_t = v_t, for any alpha and S."""
    rng = np.random.default_rng(3)
    T, Hk, Hv, d = 25, 2, 4, 64
    q, _, v, alpha, _ = _rand_inputs(rng, T, Hk, Hv, d, d)
    k = _exact_unit_keys(rng, T, Hk, d, 16)
    beta = np.ones((T, Hv), np.float32)
    S0 = rng.standard_normal((1, Hv, d, d)).astype(np.float32)
    for t1 in range(1, T + 1):
        _, S = oracle.prefill(q[None, :t1], k[None, :t1], v[None, :t1], alpha[None, :t1],
                              beta[None, :t1], S0)
        for h in range(Hv):
            g = h // (Hv // Hk)
            np.testing.assert_allclose(S[0, h] @ _f64(k[t1 - 1, g]), _f64(v[t1 - 1, h]),
                                       rtol=0, atol=1e-12)


def test_literal_matrix_form():
    """Tiny inputs: the rank-1 token loop equals the literal
    a S (I - b k k^T) + b v k^T evaluated with explicit d x d matrices."""
    rng = np.random.default_rng(4)
    for (T, dk, dv) in [(1, 1, 1), (3, 2, 5), (8, 8, 8), (7, 5, 3)]:
        q, k, v, alpha, beta = _rand_inputs(rng, T, 1, 1, dk, dv, unit_k=False)
        S0 = rng.standard_normal((1, 1, dv, dk)).astype(np.float32)
        o, S = oracle.prefill(q[None], k[None], v[None], alpha[None], beta[None], S0, scale=1.5)
        Sx = _f64(S0[0, 0])
        for t in range(T):
            kt, qt, vt = _f64(k[t, 0]), _f64(q[t, 0]), _f64(v[t, 0])
            a, b = float(alpha[t, 0]), float(beta[t, 0])
            Sx = a * Sx @ (np.eye(dk) - b * np.outer(kt, kt)) + b * np.outer(vt, kt)
            np.testing.assert_allclose(o[0, t, 0], 1.5 * Sx @ qt, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(S[0, 0], Sx, rtol=1e-13, atol=1e-13)


def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_delta_rule_memory_orthonormal_keys():
    """a = b = 1, orthonormal keys, S0 = 0: S_m = sum v_j k_j^T, and a query
    equal to an earlier key returns that key's value."""
    rng = np.random.default_rng(5)
    d, m = 64, 40
    Hrows = (_hadamard(d) / np.sqrt(d)).astype(np.float32)  # entries +-1/8: exact
    order = rng.permutation(d)[:m]
    k = Hrows[order][:, None, :]
    q = k[rng.integers(0, m, m)]  # query: some key (possibly a later one)
    v = rng.standard_normal((m, 1, d)).astype(np.float32)
    ones = np.ones((m, 1), np.float32)
    o, S = oracle.chain(q, k, v, ones, ones, 0, m, 0)
    np.testing.assert_allclose(S, sum(np.outer(_f64(v[j, 0]), _f64(k[j, 0])) for j in range(m)),
                               atol=1e-12)
    for t in range(m):
        j = int(np.where((k[:, 0] == q[t, 0]).all(axis=1))[0][0])
        expect = _f64(v[j, 0]) if j <= t else np.zeros(d)
        np.testing.assert_allclose(o[t], expect, atol=1e-12)


def test_repeated_key_keeps_latest_value():
    rng = np.random.default_rng(6)
    d = 16
    k1 = _exact_unit_keys(rng, 1, 1, d, 4)[0, 0]
    k = np.stack([k1, k1])[:, None, :]
    v = rng.standard_normal((2, 1, d)).astype(np.float32)
    ones = np.ones((2, 1), np.float32)
    _, S = oracle.chain(k, k, v, ones, ones, 0, 2, 0)
    np.testing.assert_allclose(S @ _f64(k1), _f64(v[1, 0]), atol=1e-13)


# ------------------------------------------------------------ invariants
def test_linearity_in_state_and_values():
    rng = np.random.default_rng(7)
    T, Hk, Hv, d = 20, 1, 2, 16
    q, k, _, alpha, beta = _rand_inputs(rng, T, Hk, Hv, d, d)
    v1 = (rng.integers(-64, 64, (T, Hv, d)) / 16).astype(np.float32)
    v2 = (rng.integers(-64, 64, (T, Hv, d)) / 16).astype(np.float32)
    s1 = (rng.integers(-64, 64, (1, Hv, d, d)) / 64).astype(np.float32)
    s2 = (rng.integers(-64, 64, (1, Hv, d, d)) / 64).astype(np.float32)
    oa, Sa = oracle.prefill(q[None], k[None], v1[None], alpha[None], beta[None], s1)
    ob, Sb = oracle.prefill(q[None], k[None], v2[None], alpha[None], beta[None], s2)
    oc, Sc = oracle.prefill(q[None], k[None], (v1 + v2)[None], alpha[None], beta[None], s1 + s2)
    np.testing.assert_allclose(oc, oa + ob, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Sc, Sa + Sb, rtol=1e-11, atol=1e-11)
    oz, Sz = oracle.prefill(q[None], k[None], np.zeros_like(v1)[None], alpha[None], beta[None],
                            None)
    assert not oz.any() and not Sz.any()


@pytest.mark.parametrize("T1", [0, 1, 63, 64, 65, 100])
def test_split_invariance(T1):
    d = small_prefill(1, 130, 2, 4, 32, "bf16", seed=8, init_state=True)
    args = [d[n] for n in ("q", "k", "v", "alpha", "beta")]
    o, S = oracle.prefill(*args, d["S0"])
    oa, Sa = oracle.prefill(*[x[:, :T1] for x in args], d["S0"])
    ob, Sb = oracle.prefill(*[x[:, T1:] for x in args], Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(Sb, S)


def test_zero_length_returns_initial_state():
    d = small_prefill(1, 0, 1, 2, 8, "f32", seed=9, init_state=True)
    o, S = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    assert o.shape == (1, 0, 2, 8)
    np.testing.assert_array_equal(S, d["S0"].astype(np.float64))


def test_bf16_inputs_widen_exactly():
    d = small_prefill(1, 50, 2, 4, 16, "bf16", seed=10, init_state=True)
    o1, S1 = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    f = {n: bf16_to_f32(d[n]) for n in ("q", "k", "v")}
    o2, S2 = oracle.prefill(f["q"], f["k"], f["v"], d["alpha"], d["beta"], d["S0"])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_varlen_equals_per_sequence_and_decode_equals_T1():
    rng = np.random.default_rng(11)
    lengths = [5, 1, 17, 0, 9]
    from gdn_synth import generate_packed
    d = generate_packed(2, 4, 16, "bf16", 12, lengths, init_state=True)
    o, S = oracle.varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"], d["S0"])
    cu = d["cu_seqlens"]
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        on, Sn = oracle.prefill(d["q"][None, sl], d["k"][None, sl], d["v"][None, sl],
                                d["alpha"][None, sl], d["beta"][None, sl], d["S0"][n:n + 1])
        np.testing.assert_array_equal(o[sl], on[0])
        np.testing.assert_array_equal(S[n], Sn[0])
    # decode: one token per sequence == prefill with T = 1
    q, k, v = d["q"][:3], d["k"][:3], d["v"][:3]
    a, b = d["alpha"][:3], d["beta"][:3]
    S0 = np.ascontiguousarray(np.concatenate([d["S0"], d["S0"][:1]])[:3])
    od, Sd = oracle.decode(q, k, v, a, b, S0)
    for i in range(3):
        op, Sp = oracle.prefill(q[None, i:i + 1], k[None, i:i + 1], v[None, i:i + 1],
                                a[None, i:i + 1], b[None, i:i + 1], S0[i:i + 1])
        np.testing.assert_array_equal(od[i], op[0, 0])
        np.testing.assert_array_equal(Sd[i], Sp[0])
    del rng


# ------------------------------------------------------------ chunk algebra
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunk_mirror_matches_oracle(C):
    d = small_prefill(1, 203, 2, 6, 32, "bf16", seed=13, init_state=True)
    o, S = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], scale=0.5)
    for h in range(6):
        g = h // 3
        om, Sm = chunk_chain(d["q"][0, :, g], d["k"][0, :, g], d["v"][0, :, h],
                             d["alpha"][0, :, h], d["beta"][0, :, h], d["S0"][0, h], C=C,
                             scale=0.5)
        np.testing.assert_allclose(om, o[0, :, h], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(Sm, S[0, h], rtol=1e-10, atol=1e-11)


def test_chunk_mirror_slow_decay():
    d = small_prefill(1, 300, 1, 1, 32, "bf16", seed=14, alpha_shift=-5.0, beta_shift=-2.0,
                      init_state=True)
    o, S = oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    om, Sm = chunk_chain(d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0],
                         d["alpha"][0, :, 0], d["beta"][0, :, 0], d["S0"][0, 0], C=64)
    np.testing.assert_allclose(om, o[0, :, 0], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(Sm, S[0, 0], rtol=1e-10, atol=1e-11)


# ------------------------------------------------------------ page facts
def test_state_size_matches_page():
    """48 GDN layers x 48 value heads x 128 x 128 fp32 is the page's ~150 MiB;
    bf16 or fp64 states would be 72 or 288 MiB."""
    g = json.load(open(os.path.join(GOLDEN, "qwen_gdn_layer.json")))["facts"]
    n = g["gdn_layers"]["value"] * g["gdn_v_heads"]["value"] * g["gdn_head_dim"]["value"] ** 2
    approx = g["gdn_state_total_mib_approx"]["value"]
    assert g["gdn_layers"]["value"] * 4 == g["layers_total"]["value"] * 3
    assert abs(n * 4 / 2**20 - approx) / approx < 0.05
    assert abs(n * 2 / 2**20 - approx) / approx > 0.4
    assert abs(n * 8 / 2**20 - approx) / approx > 0.4
    assert g["gdn_v_heads"]["value"] % g["gdn_qk_heads"]["value"] == 0


def test_generator_rounding_is_rne():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3], np.float32)
    # 1 + 2^-8 is halfway between two bf16 values -> ties to even (1.0)
    np.testing.assert_array_equal(bf16_to_f32(bf16_bits(x))[:2], [1.0, 1.0])
    assert bf16_to_f32(bf16_bits(x))[2] == np.float32(1.0078125)
    assert bf16_to_f32(bf16_bits(x))[3] == np.float32(-2.5)


# ------------------------------------------------- K tokens against a slot pool
# The multi-token oracle routes states between pool slots and walks the token
# recurrence. Its pins use closed forms of the recurrence and exact facts of
# the routing, with slot plans in which a transposed src/dst, an off-by-one
# slot, a step state from the wrong token or a write to an unnamed slot fails.
def _multi_inputs(rng, B, K, Hk, Hv, d, nslots):
    q, k, v, alpha, beta = (x.reshape((B, K) + x.shape[1:])
                            for x in _rand_inputs(rng, B * K, Hk, Hv, d, d))
    pool = rng.standard_normal((nslots, Hv, d, d)).astype(np.float32)
    return q, k, v, alpha, beta, pool


def test_multi_decay_only_routes_slots():
    """beta = 0: the state after token t is (prod_{s<=t} a_s) S_src, o_t is
    that state times q_t, the dst slot receives the last one, and every slot
    that is no dst keeps its value bit for bit."""
    rng = np.random.default_rng(41)
    B, K, Hk, Hv, d, ns = 3, 5, 2, 4, 8, 9
    q, k, v, alpha, _, pool = _multi_inputs(rng, B, K, Hk, Hv, d, ns)
    beta = np.zeros((B, K, Hv), np.float32)
    src = np.array([7, 2, 4], np.int32)
    dst = np.array([0, 5, 4], np.int32)          # sequence 2 in place
    o, pool2, steps = oracle.decode_multi(q, k, v, alpha, beta, pool, src, dst, scale=0.5,
                                          want_steps=True)
    for b in range(B):
        for h in range(Hv):
            g = h // (Hv // Hk)
            cp = np.cumprod(_f64(alpha[b, :, h]))
            S0 = _f64(pool[src[b], h])
            for t in range(K):
                np.testing.assert_allclose(steps[b, t, h], cp[t] * S0, rtol=1e-12, atol=1e-300)
                np.testing.assert_allclose(o[b, t, h], 0.5 * cp[t] * (S0 @ _f64(q[b, t, g])),
                                           rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(pool2[dst[b], h], cp[-1] * S0, rtol=1e-12, atol=1e-300)
    for n in set(range(ns)) - set(dst.tolist()):
        np.testing.assert_array_equal(pool2[n], _f64(pool[n]))


def test_multi_zero_source_first_token():
    """src < 0: token 0 starts from S = 0, so o_0 = scale b (k.q) v."""
    rng = np.random.default_rng(42)
    B, K, Hk, Hv, d = 2, 3, 1, 3, 16
    q, k, v, alpha, beta, pool = _multi_inputs(rng, B, K, Hk, Hv, d, 4)
    src = np.array([-1, -1], np.int32)
    dst = np.array([3, 1], np.int32)
    o, _, steps = oracle.decode_multi(q, k, v, alpha, beta, pool, src, dst, scale=1.25,
                                      want_steps=True)
    for b in range(B):
        for h in range(Hv):
            kq = float(_f64(k[b, 0, 0]) @ _f64(q[b, 0, 0]))
            np.testing.assert_allclose(o[b, 0, h], 1.25 * float(beta[b, 0, h]) * kq * _f64(v[b, 0, h]),
                                       rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(steps[b, 0, h],
                                       float(beta[b, 0, h]) * np.outer(_f64(v[b, 0, h]), _f64(k[b, 0, 0])),
                                       rtol=1e-12, atol=1e-14)


def test_multi_identity_padding_tokens():
    """alpha = 1, beta = 0 leaves S unchanged exactly (1*S + 0*k = S), and
    the output of such a token is S q."""
    rng = np.random.default_rng(43)
    B, K, Hk, Hv, d = 2, 6, 2, 4, 8
    q, k, v, alpha, beta, pool = _multi_inputs(rng, B, K, Hk, Hv, d, 4)
    alpha[:, 3:] = 1.0
    beta[:, 3:] = 0.0
    src = np.array([0, 1], np.int32)
    dst = np.array([2, 3], np.int32)
    o, pool2, steps = oracle.decode_multi(q, k, v, alpha, beta, pool, src, dst, want_steps=True)
    for b in range(B):
        for h in range(Hv):
            g = h // (Hv // Hk)
            for t in range(3, K):
                np.testing.assert_array_equal(steps[b, t, h], steps[b, 2, h])
                np.testing.assert_allclose(o[b, t, h], steps[b, 2, h] @ _f64(q[b, t, g]),
                                           rtol=1e-12, atol=1e-14)
            np.testing.assert_array_equal(pool2[dst[b], h], steps[b, 2, h])


def test_multi_overwrite_each_step():
    """beta = 1 and exactly unit keys: after every token S_t k_t = v_t."""
    rng = np.random.default_rng(44)
    B, K, Hk, Hv, d = 2, 4, 2, 4, 64
    q, _, v, alpha, beta, pool = _multi_inputs(rng, B, K, Hk, Hv, d, 5)
    k = _exact_unit_keys(rng, B * K, Hk, d, 16).reshape(B, K, Hk, d)
    beta[...] = 1.0
    src = np.array([4, 1], np.int32)
    dst = np.array([0, 2], np.int32)
    _, _, steps = oracle.decode_multi(q, k, v, alpha, beta, pool, src, dst, want_steps=True)
    for b in range(B):
        for h in range(Hv):
            g = h // (Hv // Hk)
            for t in range(K):
                np.testing.assert_allclose(steps[b, t, h] @ _f64(k[b, t, g]), _f64(v[b, t, h]),
                                           rtol=0, atol=1e-12)


def test_multi_zero_tokens_copies_slot():
    """K = 0: dst receives src (zeros for a negative src); no other slot changes."""
    rng = np.random.default_rng(45)
    q, k, v, alpha, beta, pool = _multi_inputs(rng, 3, 1, 1, 2, 8, 6)
    q, k, v, alpha, beta = (x[:, :0] for x in (q, k, v, alpha, beta))
    src = np.array([5, -1, 0], np.int32)
    dst = np.array([1, 2, -1], np.int32)
    o, pool2, _ = oracle.decode_multi(q, k, v, alpha, beta, pool, src, dst)
    assert o.shape == (3, 0, 2, 8)
    np.testing.assert_array_equal(pool2[1], _f64(pool[5]))
    np.testing.assert_array_equal(pool2[2], 0.0)
    for n in (0, 3, 4, 5):
        np.testing.assert_array_equal(pool2[n], _f64(pool[n]))


def test_multi_slot_out_of_range_is_nan_and_untouched():
    rng = np.random.default_rng(46)
    q, k, v, alpha, beta, pool = _multi_inputs(rng, 2, 2, 1, 2, 8, 3)
    src = np.array([0, 3], np.int32)
    dst = np.array([1, 2], np.int32)
    o, pool2, steps = oracle.decode_multi(q, k, v, alpha, beta, pool, src, dst, want_steps=True)
    assert np.isnan(o[1]).all() and np.isnan(steps[1]).all()
    assert np.isfinite(o[0]).all()
    np.testing.assert_array_equal(pool2[2], _f64(pool[2]))
    np.testing.assert_array_equal(pool2[0], _f64(pool[0]))


# ------------------------------------------------- block-aligned prefix states
def test_prefix_states_decay_only():
    """beta = 0: the state after block i is (prod of alpha over its first
    block * (i + 1) tokens) S0, per sequence of a ragged packed batch."""
    rng = np.random.default_rng(51)
    lens = [7, 20, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, alpha, _ = _rand_inputs(rng, int(cu[-1]), 2, 4, 8, 8)
    alpha = rng.uniform(0.8, 1.0, alpha.shape).astype(np.float32)
    beta = np.zeros_like(alpha)
    S0 = rng.standard_normal((3, 4, 8, 8)).astype(np.float32)
    blk = 6
    pre = oracle.prefix_states(q, k, v, alpha, beta, cu, blk, S0)
    for n, L in enumerate(lens):
        assert pre[n].shape == (L // blk, 4, 8, 8)
        for i in range(L // blk):
            cp = np.prod(_f64(alpha[cu[n]:cu[n] + blk * (i + 1)]), axis=0)
            for h in range(4):
                np.testing.assert_allclose(pre[n][i, h], cp[h] * _f64(S0[n, h]), rtol=1e-12,
                                           atol=1e-300)


def test_prefix_states_overwrite_at_block_ends():
    """beta = 1 and exactly unit keys: each prefix state satisfies S k = v for
    the last token of its block."""
    rng = np.random.default_rng(52)
    T, Hk, Hv, d, blk = 40, 2, 4, 64, 8
    q, _, v, alpha, _ = _rand_inputs(rng, T, Hk, Hv, d, d)
    k = _exact_unit_keys(rng, T, Hk, d, 16)
    beta = np.ones((T, Hv), np.float32)
    pre = oracle.prefix_states(q, k, v, alpha, beta, [0, T], blk)[0]
    assert pre.shape[0] == T // blk
    for i in range(T // blk):
        t = blk * (i + 1) - 1
        for h in range(Hv):
            np.testing.assert_allclose(pre[i, h] @ _f64(k[t, h // (Hv // Hk)]), _f64(v[t, h]),
                                       rtol=0, atol=1e-12)


# ------------------------------------------------- input preparation (flags)
def test_raw_qk_scale_invariance():
    """With q, k L2-normalised by the oracle, scaling any q or k row by a
    positive constant leaves every output and state unchanged (up to the
    1e-6 under the square root); a missing normalisation of either fails."""
    rng = np.random.default_rng(61)
    T, Hk, Hv, d = 30, 2, 4, 16
    q, k, v, alpha, beta = _rand_inputs(rng, T, Hk, Hv, d, d, unit_k=False)
    S0 = rng.standard_normal((1, Hv, d, d)).astype(np.float32)
    o1, S1 = oracle.prefill(q[None], k[None], v[None], alpha[None], beta[None], S0,
                            flags=oracle.QK_L2NORM)
    cq = rng.uniform(0.2, 30.0, (T, Hk, 1)).astype(np.float32)
    ck = rng.uniform(0.2, 30.0, (T, Hk, 1)).astype(np.float32)
    o2, S2 = oracle.prefill((q * cq)[None], (k * ck)[None], v[None], alpha[None], beta[None],
                            S0, flags=oracle.QK_L2NORM)
    np.testing.assert_allclose(o2, o1, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(S2, S1, rtol=1e-5, atol=1e-7)


def test_raw_qk_unit_rows_equal_plain():
    """Rows that already have unit norm come out of the normalisation as
    x / sqrt(1 + 1e-6): the prepared run matches the plain one to ~5e-7."""
    rng = np.random.default_rng(62)
    T, Hk, Hv, d = 20, 1, 2, 64
    q, _, v, alpha, beta = _rand_inputs(rng, T, Hk, Hv, d, d)
    k = _exact_unit_keys(rng, T, Hk, d, 16)
    q = _exact_unit_keys(rng, T, Hk, d, 4)
    o1, S1 = oracle.prefill(q[None], k[None], v[None], alpha[None], beta[None])
    o2, S2 = oracle.prefill(q[None], k[None], v[None], alpha[None], beta[None],
                            flags=oracle.QK_L2NORM)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=5e-6 * np.abs(o1).max())
    np.testing.assert_allclose(S2, S1, rtol=0, atol=5e-6 * np.abs(S1).max())


def test_gate_logits_closed_forms():
    """exp(-softplus(0)) = 1/2 and sigmoid(0) = 1/2: zero logits equal the plain
    run with alpha = beta = 1/2; large logits reach the limits e^-a and e^b."""
    rng = np.random.default_rng(63)
    T, Hk, Hv, d = 12, 1, 2, 8
    q, k, v, _, _ = _rand_inputs(rng, T, Hk, Hv, d, d)
    zero = np.zeros((T, Hv), np.float32)
    half = np.full((T, Hv), 0.5, np.float32)
    o1, S1 = oracle.prefill(q[None], k[None], v[None], zero[None], zero[None],
                            flags=oracle.GATE_LOGITS)
    o2, S2 = oracle.prefill(q[None], k[None], v[None], half[None], half[None])
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(S1, S2, rtol=1e-14, atol=1e-16)
    _, _, _, a, b = oracle.prepare(q, k, v, np.array([40.0, -40.0, 3.0]),
                                   np.array([-40.0, 40.0, -3.0]), oracle.GATE_LOGITS)
    np.testing.assert_allclose(a[0], np.exp(-40.0), rtol=1e-12)
    assert a[1] == 1.0 or abs(a[1] - 1.0) < 1e-15
    np.testing.assert_allclose(a[2], 1.0 / (1.0 + np.exp(3.0)), rtol=1e-14)
    np.testing.assert_allclose(b[0], np.exp(-40.0), rtol=1e-12)
    np.testing.assert_allclose(b[2], 1.0 / (1.0 + np.exp(3.0)), rtol=1e-14)


def test_prepare_matches_the_generator_recipe():
    """The raw inputs of a seed, prepared, give the normalised rows and gates
    the generator stores for the same seed (to its bf16 / fp32 rounding)."""
    from gdn_synth import small_prefill
    plain = small_prefill(1, 300, 2, 6, 128, "bf16", seed=64)
    raw = small_prefill(1, 300, 2, 6, 128, "bf16", seed=64, raw=True)
    q, k, v, a, b = oracle.prepare(raw["q"], raw["k"], raw["v"], raw["alpha"], raw["beta"],
                                   oracle.QK_L2NORM | oracle.GATE_LOGITS)
    np.testing.assert_allclose(q, bf16_to_f32(plain["q"]), rtol=0, atol=4e-3)
    np.testing.assert_allclose(k, bf16_to_f32(plain["k"]), rtol=0, atol=4e-3)
    np.testing.assert_array_equal(v, bf16_to_f32(raw["v"]).astype(np.float64))
    np.testing.assert_allclose(a, plain["alpha"], rtol=2e-7)
    np.testing.assert_allclose(b, plain["beta"], rtol=2e-7)
