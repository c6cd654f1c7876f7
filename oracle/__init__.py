"""fp64 CPU oracle for the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark are the only callers. The product path never imports this
package, and this package imports nothing from the product package.

The arithmetic lives in ``gdn_oracle.c`` (a plain token-by-token fp64
recurrence; see its header for the definition and the reading of the pages it
follows), apart from prepare(): the optional input preparation (L2 norms of q
and k rows, gates from logits), written out in fp64 numpy by its definition. This module only builds/loads that library and walks it over
(sequence, value-head) chains with a thread pool. ctypes drops the GIL for
the duration of each call, so the chains run in parallel on the host cores.

Layouts (the same as the HIP library's):
  q, k  [tokens, Hk, Dk]   v  [tokens, Hv, Dv]   alpha, beta [tokens, Hv]
  states [chains, Hv, Dv, Dk]   (S in R^{Dv x Dk}, row-major)
bf16 tensors are passed as numpy uint16 arrays holding the bit patterns.
Value head h reads q/k head h // (Hv // Hk).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2
# input preparation (the library's flags argument)
QK_L2NORM, GATE_LOGITS = 1, 2
L2_EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into liboracle.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fno-fast-math", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        f = lib.gdn_oracle_chain
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_double,
                      ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def default_threads() -> int:
    env = os.environ.get("GDN_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(os.cpu_count() or 1, 16))


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.float64:
        return F64
    raise TypeError(f"q/k/v must be float32, float64 or uint16 (bf16 bits), got {arr.dtype}")


def _widen(x: np.ndarray) -> np.ndarray:
    """Exact fp64 value of fp32 data or of bf16 bit patterns (uint16)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def prepare(q, k, v, alpha, beta, flags):
    """The input preparation the library can do inside its kernels, by its
    definition in fp64 (a plain elementwise/row-wise pass):
      QK_L2NORM  : every q and k row x becomes x / sqrt(sum(x^2) + 1e-6)
      GATE_LOGITS: alpha holds a, beta holds b; alpha = exp(-softplus(a)),
                   beta = 1 / (1 + exp(-b))
    Returns (q, k, v, alpha, beta); prepared arrays are fp64 (v is widened
    exactly alongside prepared q, k), the others are returned unchanged."""
    if flags & QK_L2NORM:
        def l2(x):
            x = _widen(x)
            return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)
        q, k, v = l2(q), l2(k), _widen(v)
    if flags & GATE_LOGITS:
        a = np.asarray(alpha, np.float64)
        b = np.asarray(beta, np.float64)
        alpha = np.exp(-np.logaddexp(0.0, a))
        beta = 1.0 / (1.0 + np.exp(-b))
    return q, k, v, alpha, beta


def chain(q, k, v, alpha, beta, t0: int, t1: int, h: int, S0=None, scale: float = 1.0,
          want_o: bool = True):
    """Run the recurrence for value head ``h`` over packed tokens [t0, t1).

    Returns (o [t1-t0, Dv] fp64 or None, S [Dv, Dk] fp64)."""
    lib = _load()
    for a in (q, k, v, alpha, beta):
        if not a.flags.c_contiguous:
            raise ValueError("oracle inputs must be C-contiguous")
    if q.dtype != k.dtype:
        raise TypeError("q, k must share one dtype")
    if alpha.dtype != beta.dtype or alpha.dtype not in (np.float32, np.float64):
        raise TypeError("alpha, beta must both be float32 or both float64")
    _, Hk, Dk = q.shape
    _, Hv, Dv = v.shape
    g = h // (Hv // Hk)
    T = t1 - t0
    S = np.zeros((Dv, Dk), np.float64) if S0 is None else np.array(S0, np.float64, order="C")
    o = np.empty((max(T, 0), Dv), np.float64) if want_o else None
    if v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(q)
    isz, vsz, asz = q.itemsize, v.itemsize, alpha.itemsize
    rc = lib.gdn_oracle_chain(
        q.ctypes.data + ((t0 * Hk + g) * Dk) * isz,
        k.ctypes.data + ((t0 * Hk + g) * Dk) * isz,
        v.ctypes.data + ((t0 * Hv + h) * Dv) * vsz,
        dt,
        alpha.ctypes.data + (t0 * Hv + h) * asz,
        beta.ctypes.data + (t0 * Hv + h) * asz,
        F64 if alpha.dtype == np.float64 else F32,
        T, Hk * Dk, Hv * Dv, Hv, Dk, Dv, float(scale),
        S.ctypes.data, o.ctypes.data if o is not None else None)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, S


def _flatten_batch(x):
    return x.reshape((-1,) + x.shape[2:])


def prefill(q, k, v, alpha, beta, initial_state=None, scale=1.0, chains=None,
            threads=None, flags=0):
    """Dense-batch prefill: q,k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; alpha,beta [B,T,Hv].

    ``chains`` optionally lists the (b, h) pairs to compute (default: all).
    Returns (o, S): o [B,T,Hv,Dv] fp64 and S [B,Hv,Dv,Dk] fp64; entries of
    chains not computed are NaN."""
    B, T = q.shape[0], q.shape[1]
    Hv, Dv = v.shape[2], v.shape[3]
    Dk = q.shape[3]
    cu = np.arange(B + 1, dtype=np.int64) * T
    o, S = varlen(_flatten_batch(q), _flatten_batch(k), _flatten_batch(v),
                  _flatten_batch(alpha), _flatten_batch(beta), cu, initial_state,
                  scale, chains, threads, flags)
    return o.reshape(B, T, Hv, Dv), S.reshape(B, Hv, Dv, Dk)


def varlen(q, k, v, alpha, beta, cu_seqlens, initial_state=None, scale=1.0,
           chains=None, threads=None, flags=0):
    """Packed prefill: q,k [total,Hk,Dk]; v [total,Hv,Dv]; alpha,beta [total,Hv];
    sequence n spans tokens cu_seqlens[n] .. cu_seqlens[n+1]-1. ``flags``:
    prepare the inputs first (see prepare()).

    Returns (o [total,Hv,Dv] fp64, S [N,Hv,Dv,Dk] fp64); entries of chains not
    listed in ``chains`` are NaN."""
    q, k, v, alpha, beta = prepare(q, k, v, alpha, beta, flags)
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    N = len(cu) - 1
    total, Hv, Dv = v.shape
    Dk = q.shape[2]
    if chains is None:
        chains = [(n, h) for n in range(N) for h in range(Hv)]
    o = np.full((total, Hv, Dv), np.nan)
    S = np.full((N, Hv, Dv, Dk), np.nan)

    def work(nh):
        n, h = nh
        s0 = None if initial_state is None else initial_state[n, h]
        oc, sc = chain(q, k, v, alpha, beta, cu[n], cu[n + 1], h, s0, scale)
        o[cu[n]:cu[n + 1], h, :] = oc
        S[n, h] = sc

    nthreads = threads or default_threads()
    if nthreads == 1 or len(chains) == 1:
        for nh in chains:
            work(nh)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, chains))
    return o, S


def decode(q, k, v, alpha, beta, state, scale=1.0, threads=None, flags=0):
    """One token per sequence: q,k [B,Hk,Dk]; v [B,Hv,Dv]; alpha,beta [B,Hv];
    state [B,Hv,Dv,Dk] fp32 (not modified). Returns (o [B,Hv,Dv], S') in fp64."""
    B = q.shape[0]
    cu = np.arange(B + 1, dtype=np.int64)
    return varlen(q, k, v, alpha, beta, cu, state, scale, None, threads, flags)


def decode_multi(q, k, v, alpha, beta, pool, src_slot, dst_slot, scale=1.0, want_steps=False,
                 threads=None, flags=0):
    """K tokens per sequence against a pool of state slots.

    q,k [B,K,Hk,Dk]; v [B,K,Hv,Dv]; alpha,beta [B,K,Hv] fp32; pool
    [num_slots,Hv,Dv,Dk] (not modified); src_slot, dst_slot: B integers.
    Sequence b starts from pool[src_slot[b]] (zero state when the index is
    negative), runs its K tokens in order, one call of the token recurrence
    per token, and its final state goes to pool[dst_slot[b]] (nowhere when
    that index is negative). A sequence with an index >= num_slots touches no
    slot and gets NaN outputs and step states.

    Returns (o [B,K,Hv,Dv] fp64, pool' [num_slots,Hv,Dv,Dk] fp64,
    steps [B,K,Hv,Dv,Dk] fp64 = the state after each token, or None)."""
    B, K = q.shape[0], q.shape[1]
    Hv, Dv = v.shape[2], v.shape[3]
    Dk = q.shape[3]
    nslots = pool.shape[0]
    q, k, v, alpha, beta = prepare(q, k, v, alpha, beta, flags)
    src = [int(x) for x in np.asarray(src_slot)]
    dst = [int(x) for x in np.asarray(dst_slot)]
    o = np.full((B, K, Hv, Dv), np.nan)
    steps = np.full((B, K, Hv, Dv, Dk), np.nan) if want_steps else None
    out_pool = np.array(pool, np.float64)
    finals = {}

    def work(bh):
        b, h = bh
        if src[b] >= nslots or dst[b] >= nslots:
            return
        S = None if src[b] < 0 else pool[src[b], h]
        for t in range(K):
            ot, S = chain(q[b], k[b], v[b], alpha[b], beta[b], t, t + 1, h, S, scale)
            o[b, t, h] = ot[0]
            if steps is not None:
                steps[b, t, h] = S
        if S is None:
            S = np.zeros((Dv, Dk))
        finals[bh] = S

    pairs = [(b, h) for b in range(B) for h in range(Hv)]
    nthreads = threads or default_threads()
    if nthreads == 1:
        for bh in pairs:
            work(bh)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, pairs))
    for (b, h), S in finals.items():
        if dst[b] >= 0:
            out_pool[dst[b], h] = S
    return o, out_pool, steps


def prefix_states(q, k, v, alpha, beta, cu_seqlens, block, initial_state=None, chains=None,
                  threads=None, flags=0):
    """Block-aligned prefix states of packed sequences: for sequence n and
    value head h, the state after each whole block of ``block`` tokens,
    S_{block * (i + 1)} for i < floor(L_n / block), obtained by running the
    recurrence one block after the other from the initial state.

    q,k [total,Hk,Dk]; v [total,Hv,Dv]; alpha,beta [total,Hv];
    initial_state [N,Hv,Dv,Dk] or None. Returns a list over sequences of
    fp64 arrays [floor(L_n / block), Hv, Dv, Dk] (NaN for chains not listed
    in ``chains``)."""
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    N = len(cu) - 1
    Hv, Dv = v.shape[1], v.shape[2]
    Dk = q.shape[2]
    q, k, v, alpha, beta = prepare(q, k, v, alpha, beta, flags)
    out = [np.full(((cu[n + 1] - cu[n]) // block, Hv, Dv, Dk), np.nan) for n in range(N)]
    if chains is None:
        chains = [(n, h) for n in range(N) for h in range(Hv)]

    def work(nh):
        n, h = nh
        S = None if initial_state is None else initial_state[n, h]
        for i in range(out[n].shape[0]):
            t0 = cu[n] + i * block
            _, S = chain(q, k, v, alpha, beta, t0, t0 + block, h, S, want_o=False)
            out[n][i, h] = S

    nthreads = threads or default_threads()
    if nthreads == 1:
        for nh in chains:
            work(nh)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, chains))
    return out
