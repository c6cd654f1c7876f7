"""Chunk-form mirror of the gated delta rule, numpy fp64 (a test aid).

Not the oracle: it restates, stage by stage, the chunked algebra the HIP
prefill kernel evaluates, so that the algebra itself can be checked against
the token-by-token oracle (they must agree to fp64 rounding) and so that a
kernel's intermediate stages can be compared one by one while debugging.

Derivation (from the recurrence S_t = a_t S_{t-1} + u_t k_t^T with
u_t = b_t (v_t - a_t S_{t-1} k_t), o_t = S_t q_t). Inside a chunk with start
state S, write g_t = sum_{s<=t} ln a_s and gamma_t = e^{g_t}. By induction
S_t = gamma_t S + sum_{j<=t} e^{g_t - g_j} u_j k_j^T. Substituting into u_t:

    (I + A) U = diag(b) V - diag(b gamma) K S^T,
    A_tj = b_t e^{g_t - g_j} (k_t . k_j)   for j < t (zero elsewhere)

so with Tm = (I + A)^{-1} (unit lower triangular):

    U     = Tm diag(b) (V - diag(gamma) K S^T)
    O     = diag(gamma) Q S^T + (Gamma o M_incl o Q K^T) U,  Gamma_tj = e^{g_t-g_j}
    S_end = gamma_C S + U^T diag(e^{g_C - g}) K

Every exponent used is g_t - g_j with t >= j, so each factor is <= 1.
"""
import numpy as np


def bf16_bits_to_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def chunk_chain(q, k, v, alpha, beta, S0=None, C=64, scale=1.0, stages=None):
    """One chain: q,k [T,dk]; v [T,dv]; alpha,beta [T]. Returns (o [T,dv], S)."""
    q = bf16_bits_to_f64(q)
    k = bf16_bits_to_f64(k)
    v = bf16_bits_to_f64(v)
    a = np.asarray(alpha, np.float64)
    b = np.asarray(beta, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    tiny = np.finfo(np.float32).tiny
    for c0 in range(0, T, C):
        c1 = min(c0 + C, T)
        n = c1 - c0
        Qc, Kc, Vc = q[c0:c1], k[c0:c1], v[c0:c1]
        bc = b[c0:c1]
        g = np.cumsum(np.log(np.maximum(a[c0:c1], tiny)))
        gam = np.exp(g)
        diff = g[:, None] - g[None, :]
        lower_strict = np.tril(np.ones((n, n)), -1)
        lower_incl = np.tril(np.ones((n, n)))
        Gam = np.exp(np.where(lower_incl > 0, diff, -np.inf))
        A = (bc[:, None] * Gam * (Kc @ Kc.T)) * lower_strict
        Tm = np.linalg.inv(np.eye(n) + A)
        R = bc[:, None] * (Vc - gam[:, None] * (Kc @ S.T))
        U = Tm @ R
        P = Gam * (Qc @ Kc.T) * lower_incl
        O = gam[:, None] * (Qc @ S.T) + P @ U
        o[c0:c1] = scale * O
        dec = np.exp(g[-1] - g)
        S = gam[-1] * S + U.T @ (dec[:, None] * Kc)
        if stages is not None:
            stages.append(dict(g=g, A=A, T=Tm, R=R, U=U, P=P, O=O, S=S.copy()))
    return o, S
