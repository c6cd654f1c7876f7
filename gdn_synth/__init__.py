"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module is shared by the tests, the benchmark and the smoke check, and
feeds both the HIP library and the fp64 oracle the very same bits. It holds
none of the mixer's arithmetic: it draws random numbers, shapes them into the
value laws of the workloads below, and rounds to the storage type.

Layer shapes come from "The Hybrid Attention in Qwen3.8-27B" (section
"Grouped-query attention multiplies on top of that": 16 query/key heads, 48
value heads, head dimension 128 on the Gated DeltaNet side); the native
context of 262,144 tokens from its section "Why 27B parameters can carry 262K
tokens". The pages print no inputs, so every value law below is synthetic.

Recipe (fixed so that any block of any workload can be regenerated alone):
  * numpy PCG64; the workload's seed is spawned with SeedSequence into one
    child per (sequence, 4096-token block), plus one child for the lengths
    and one for the initial states;
  * inside a block the draws are, in order: q, k ~ N(0,1) [blk, Hk, D];
    v ~ N(0,1) [blk, Hv, D]; beta logits ~ N(0,1) [blk, Hv]; alpha logits
    ~ N(0,1) [blk, Hv];
  * q and k are L2-normalised in fp32 along the head dimension (x / ||x||,
    no epsilon), then rounded to the storage type; v is rounded directly;
  * beta = sigmoid(logit + beta_shift); alpha = exp(-softplus(logit +
    alpha_shift)), fp32 (the workloads use beta_shift 0; the slow-decay
    stress inputs use alpha_shift -5 and beta_shift -2);
  * initial states, when present, are 0.1 * N(0,1) in fp32;
  * bf16 rounding is round-to-nearest-even of the fp32 value.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_TOKENS = 4096


# ----------------------------------------------------------------- rounding
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs are finite (the generators never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _exp_neg_softplus(x):
    x = x.astype(np.float64)
    sp = np.logaddexp(0.0, x)  # softplus, stable
    return np.exp(-sp).astype(np.float32)


# -------------------------------------------------------------- workloads
@dataclass
class Workload:
    """A named synthetic workload (shapes + value laws + seed)."""
    name: str
    kind: str                    # "prefill", "varlen" or "decode"
    Hk: int
    Hv: int
    D: int
    dtype: str                   # "bf16" or "f32" (type of q, k, v and o)
    seed: int
    B: int = 1                   # prefill batch / decode batch / varlen N
    T: int = 1                   # prefill length (ignored for varlen/decode)
    len_range: tuple = (0, 0)    # varlen: inclusive uniform integer range
    alpha_shift: float = 2.0
    init_state: bool = False
    description: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", "prefill", 1, 1, 64, "f32", 1000, B=1, T=256, alpha_shift=0.0,
        description="tiny single-head gated delta rule: B=1, T=256, Hk=Hv=1, d=64, fp32, "
                    "alpha=exp(-softplus(N(0,1))), zero initial state"),
    "layer_prefill_4k": Workload(
        "layer_prefill_4k", "prefill", 16, 48, 128, "bf16", 1001, B=1, T=4096,
        description="Qwen-card Gated DeltaNet layer prefill: B=1, T=4096, 16 q/k heads, "
                    "48 v heads, d=128, bf16 q/k/v, fp32 alpha/beta/state, zero initial state"),
    "long_prefill_256k": Workload(
        "long_prefill_256k", "prefill", 16, 48, 128, "bf16", 1002, B=1, T=262144,
        description="long-context prefill at the native length: layer shapes, B=1, T=262144"),
    "decode_b256": Workload(
        "decode_b256", "decode", 16, 48, 128, "bf16", 1003, B=256, init_state=True,
        description="batched decode step: B=256, 48 v heads, fp32 128x128 states "
                    "0.1*N(0,1), one token per sequence, in place"),
    "varlen_64seq": Workload(
        "varlen_64seq", "varlen", 16, 48, 128, "bf16", 1004, B=64,
        len_range=(1024, 32768), init_state=True,
        description="varlen packed prefill: 64 sequences, lengths U[1024,32768], "
                    "layer head shapes, initial states 0.1*N(0,1)"),
    "layer_prefill_4k_tp8": Workload(
        "layer_prefill_4k_tp8", "prefill", 2, 6, 128, "bf16", 1006, B=1, T=4096,
        description="one GPU's share of the layer prefill at 8-way head-group sharding: "
                    "B=1, T=4096, 2 q/k heads, 6 v heads, d=128, zero initial state"),
    "long_prefill_256k_tp8": Workload(
        "long_prefill_256k_tp8", "prefill", 2, 6, 128, "bf16", 1007, B=1, T=262144,
        description="the long-context prefill's share at 8-way head-group sharding"),
}


# The multi-token decode workload: B=256 sequences each verifying K=4 tokens
# (three drafted plus one) at the layer's head shapes, two pool slots per
# sequence (read slot 2b, write slot 2b+1, so the pre-verification state is
# kept for rollback).
SPEC_DECODE = dict(name="spec_decode_b256_k4", B=256, K=4, Hk=16, Hv=48, D=128, dtype="bf16",
                   seed=1005, plan="pairs")


def _threads():
    env = os.environ.get("GDN_SYNTH_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(os.cpu_count() or 1, 16))


def _round_store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else x32.astype(np.float32)


def _gen_block(child, n_tok, Hk, Hv, D, dtype, alpha_shift, beta_shift, out, row0, raw=False):
    rng = np.random.Generator(np.random.PCG64(child))
    for name, heads in (("q", Hk), ("k", Hk)):
        x = rng.standard_normal((n_tok, heads, D), dtype=np.float32)
        if not raw:
            nrm = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1,
                                 keepdims=True)).astype(np.float32)
            x = x / nrm
        out[name][row0:row0 + n_tok] = _round_store(x, dtype)
    v = rng.standard_normal((n_tok, Hv, D), dtype=np.float32)
    out["v"][row0:row0 + n_tok] = _round_store(v, dtype)
    bl = rng.standard_normal((n_tok, Hv), dtype=np.float32) + np.float32(beta_shift)
    al = rng.standard_normal((n_tok, Hv), dtype=np.float32) + np.float32(alpha_shift)
    out["beta"][row0:row0 + n_tok] = bl if raw else _sigmoid(bl)
    out["alpha"][row0:row0 + n_tok] = al if raw else _exp_neg_softplus(al)


def lengths_for(w: Workload) -> np.ndarray:
    """Per-sequence token counts of a workload."""
    if w.kind == "prefill":
        return np.full(w.B, w.T, dtype=np.int64)
    if w.kind == "decode":
        return np.ones(w.B, dtype=np.int64)
    ss = np.random.SeedSequence(w.seed)
    len_child = ss.spawn(3)[0]   # the same child generate_packed() reserves
    rng = np.random.Generator(np.random.PCG64(len_child))
    lo, hi = w.len_range
    return rng.integers(lo, hi + 1, size=w.B, dtype=np.int64)


def generate_packed(Hk, Hv, D, dtype, seed, lengths, alpha_shift=2.0, init_state=False,
                    block_tokens=BLOCK_TOKENS, threads=None, beta_shift=0.0, raw=False):
    """Packed tokens of several sequences.

    raw=True draws the same numbers but stores q, k before their L2
    normalisation and alpha, beta as their logits (the inputs of the
    library's in-kernel preparation: alpha = exp(-softplus(a)),
    beta = sigmoid(b)).

    Returns dict: q, k [total,Hk,D]; v [total,Hv,D] (uint16 bf16 bits or
    fp32); alpha, beta [total,Hv] fp32; cu_seqlens [N+1] int32; S0
    [N,Hv,D,D] fp32 or None; lengths [N] int64."""
    lengths = np.asarray(lengths, dtype=np.int64)
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    if total >= 2**31:
        raise ValueError("packed token count must fit int32")
    sdt = np.uint16 if dtype == "bf16" else np.float32
    out = {
        "q": np.empty((total, Hk, D), sdt),
        "k": np.empty((total, Hk, D), sdt),
        "v": np.empty((total, Hv, D), sdt),
        "alpha": np.empty((total, Hv), np.float32),
        "beta": np.empty((total, Hv), np.float32),
    }
    ss = np.random.SeedSequence(seed)
    _len_child, state_child, data_root = ss.spawn(3)
    seq_children = data_root.spawn(max(N, 1))
    jobs = []
    for n in range(N):
        nblk = (int(lengths[n]) + block_tokens - 1) // block_tokens
        blk_children = seq_children[n].spawn(max(nblk, 1))
        for b in range(nblk):
            r0 = int(cu[n]) + b * block_tokens
            nt = min(block_tokens, int(cu[n + 1]) - r0)
            jobs.append((blk_children[b], nt, r0))
    nth = threads or _threads()
    with ThreadPoolExecutor(nth) as ex:
        list(ex.map(lambda j: _gen_block(j[0], j[1], Hk, Hv, D, dtype, alpha_shift, beta_shift,
                                         out, j[2], raw),
                    jobs))
    S0 = None
    if init_state:
        S0 = np.empty((N, Hv, D, D), np.float32)
        st_children = state_child.spawn(max(N, 1))

        def _st(n):
            rng = np.random.Generator(np.random.PCG64(st_children[n]))
            S0[n] = np.float32(0.1) * rng.standard_normal((Hv, D, D), dtype=np.float32)
        with ThreadPoolExecutor(nth) as ex:
            list(ex.map(_st, range(N)))
    out["cu_seqlens"] = cu.astype(np.int32)
    out["S0"] = S0
    out["lengths"] = lengths
    return out


def generate(w: Workload, threads=None, raw=False):
    """Inputs of a named workload.

    prefill: q,k [B,T,Hk,D], v [B,T,Hv,D], alpha,beta [B,T,Hv], S0 [B,Hv,D,D]|None
    decode : q,k [B,Hk,D],   v [B,Hv,D],   alpha,beta [B,Hv],   S0 [B,Hv,D,D]
    varlen : packed layout of generate_packed()."""
    lengths = lengths_for(w)
    d = generate_packed(w.Hk, w.Hv, w.D, w.dtype, w.seed, lengths, w.alpha_shift,
                        w.init_state, threads=threads, raw=raw)
    if w.kind == "prefill":
        for name in ("q", "k", "v", "alpha", "beta"):
            d[name] = d[name].reshape((w.B, w.T) + d[name].shape[1:])
    return d


def small_prefill(B, T, Hk, Hv, D, dtype="bf16", seed=0, alpha_shift=2.0, init_state=False,
                  beta_shift=0.0, raw=False):
    """Prefill inputs of arbitrary shape, same recipe as the workloads."""
    d = generate_packed(Hk, Hv, D, dtype, seed, [T] * B, alpha_shift, init_state,
                        beta_shift=beta_shift, raw=raw)
    for name in ("q", "k", "v", "alpha", "beta"):
        d[name] = d[name].reshape((B, T) + d[name].shape[1:])
    return d


def multi_decode(B, K, Hk, Hv, D, dtype, seed, num_slots=None, plan="permute",
                 alpha_shift=2.0, raw=False):
    """Inputs of a K-tokens-per-sequence decode against a slot pool.

    q, k [B,K,Hk,D]; v [B,K,Hv,D]; alpha, beta [B,K,Hv]: the token recipe of
    generate_packed (each sequence K tokens); pool [num_slots,Hv,D,D] fp32
    0.1*N(0,1); src_slot, dst_slot int32 [B]. Slot plans:
      "permute": 2B distinct slots in random order, src then dst
      "pairs"  : sequence b reads slot 2b and writes slot 2b+1
      "inplace": src = dst = a random permutation of B slots
    num_slots defaults to 2B (B for "inplace")."""
    d = generate_packed(Hk, Hv, D, dtype, seed, [K] * B, alpha_shift, raw=raw)
    for name in ("q", "k", "v", "alpha", "beta"):
        d[name] = d[name].reshape((B, K) + d[name].shape[1:])
    if num_slots is None:
        num_slots = B if plan == "inplace" else 2 * B
    ss = np.random.SeedSequence([seed, 7])
    pool_child, plan_child = ss.spawn(2)
    pool = np.empty((num_slots, Hv, D, D), np.float32)
    kids = pool_child.spawn(max(num_slots, 1))

    def _slot(n):
        rng = np.random.Generator(np.random.PCG64(kids[n]))
        pool[n] = np.float32(0.1) * rng.standard_normal((Hv, D, D), dtype=np.float32)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(_slot, range(num_slots)))
    rng = np.random.Generator(np.random.PCG64(plan_child))
    if plan == "pairs":
        src = 2 * np.arange(B)
        dst = src + 1
    elif plan == "inplace":
        src = rng.permutation(num_slots)[:B]
        dst = src.copy()
    elif plan == "permute":
        perm = rng.permutation(num_slots)[:2 * B]
        src, dst = perm[:B], perm[B:]
    else:
        raise ValueError(f"unknown slot plan {plan!r}")
    d["pool"] = pool
    d["src_slot"] = np.asarray(src, np.int32)
    d["dst_slot"] = np.asarray(dst, np.int32)
    del d["cu_seqlens"], d["S0"], d["lengths"]
    return d


def to_torch(arr: np.ndarray, device):
    """numpy -> torch on `device`; uint16 arrays are bf16 bit patterns."""
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def from_torch(t) -> np.ndarray:
    """torch -> numpy on the host; bf16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
