"""Python binding of libgdn.so, the MI355X Gated DeltaNet token mixer.

Argument marshalling only: each function checks dtypes, devices, shapes and
contiguity of torch tensors, allocates the outputs it is not given, and
calls the C entry point of the same name with raw device pointers and the
current HIP stream. Every step of the computation runs in the library's HIP
kernels; there is no fallback path. If libgdn.so is missing or cannot be
loaded, the first call raises.

The recurrence, per sequence and value head h (q/k head h // (Hv // Hk)):
    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = scale * S_t q_t
States are fp32 [.., Hv, Dv, Dk] (S in R^{Dv x Dk}, row-major).
`flags` (GDN_QK_L2NORM | GDN_GATE_LOGITS) moves the input preparation into
the kernels: raw q/k rows are L2-normalised, alpha/beta are given as logits.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
# input preparation inside the kernels (the `flags` argument)
GDN_QK_L2NORM, GDN_GATE_LOGITS = 1, 2
_STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL_POINTER", 2: "GDN_ERR_BAD_SHAPE",
           3: "GDN_ERR_UNSUPPORTED", 4: "GDN_ERR_MISALIGNED", 5: "GDN_ERR_ALIAS",
           6: "GDN_ERR_HIP"}
EXPORTS = ("gdn_prefill_chunked", "gdn_decode_step", "gdn_varlen_prefill", "gdn_decode_multi",
           "gdn_prefill_workspace_size", "gdn_status_string", "gdn_version",
           "gdn_prefill_chunked_noalloc")

_lib = None


class GDNError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn.so (after torch, so that both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m gated_deltanet_token_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    u32 = ctypes.c_uint32
    sz = ctypes.c_size_t
    lib.gdn_prefill_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32,
                                        i32, i32, i32, ctypes.c_int, f32, u32, vp, sz, vp]
    lib.gdn_prefill_chunked.restype = ctypes.c_int
    lib.gdn_prefill_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64,
                                                i32, i32, i32, i32, ctypes.c_int, f32, u32, vp]
    lib.gdn_prefill_chunked_noalloc.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                    ctypes.c_int, f32, u32, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32,
                                     i32, i32, i32, ctypes.c_int, f32, u32, vp]
    lib.gdn_decode_multi.restype = ctypes.c_int
    lib.gdn_varlen_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp, i32,
                                       i32, i32, i32, i32, ctypes.c_int, f32, u32, vp, sz, vp]
    lib.gdn_varlen_prefill.restype = ctypes.c_int
    lib.gdn_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, ctypes.c_int, i32]
    lib.gdn_prefill_workspace_size.restype = sz
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise GDNError(status, _lib.gdn_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    return stream if stream is not None else torch.cuda.current_stream(device)


def gdn_prefill_workspace_size(num_seqs, tokens, Hk, Hv, Dk, Dv, dtype, packed) -> int:
    """Workspace bytes the prefill calls can use (0: they would not use one)."""
    code = _dtype_code(torch.empty(0, dtype=dtype)) if isinstance(dtype, torch.dtype) else dtype
    return int(load_library().gdn_prefill_workspace_size(num_seqs, tokens, Hk, Hv, Dk, Dv, code,
                                                         int(bool(packed))))


def _workspace(workspace, num_seqs, tokens, Hk, Hv, Dk, Dv, dtype_code, packed, dev, stream):
    """(pointer, bytes, keep-alive) of the workspace argument: None = no
    workspace; "auto" = allocate what the library asks for; a uint8 tensor."""
    if workspace is None:
        return None, 0, None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be None, 'auto' or a tensor")
        n = _lib.gdn_prefill_workspace_size(num_seqs, tokens, Hk, Hv, Dk, Dv, dtype_code,
                                            int(packed))
        if n == 0:
            return None, 0, None
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    workspace.record_stream(stream)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def prefix_state_rows(num_seqs: int, tokens: int, interval: int, packed: bool) -> int:
    """Rows of the prefix_states buffer for blocks of 64 * interval tokens:
    num_seqs * floor(T / L) for a dense batch (tokens = T per sequence),
    floor(total / L) + N for a packed one (tokens = total)."""
    L = 64 * interval
    return tokens // L + num_seqs if packed else num_seqs * (tokens // L)


def _prefix(prefix_states, prefix_interval, rows, Hv, Dv, Dk, dev):
    if prefix_states is None:
        return None, 0
    if int(prefix_interval) < 1:
        raise ValueError("prefix_interval must be >= 1 with prefix_states")
    _need(prefix_states, "prefix_states", torch.float32, (rows, Hv, Dv, Dk), dev)
    return prefix_states, int(prefix_interval)


def gdn_prefill_chunked(q, k, v, alpha, beta, initial_state=None, *, out=None,
                        final_state=None, scale: float = 1.0, want_final_state: bool = True,
                        prefix_states=None, prefix_interval: int = 0, flags: int = 0,
                        workspace="auto", stream=None):
    """Chunked prefill. q,k [B,T,Hk,D]; v [B,T,Hv,D]; alpha,beta [B,T,Hv] fp32;
    initial_state [B,Hv,D,D] fp32 or None. Returns (out, final_state).
    prefix_states: optional fp32 [B * floor(T / L), Hv, D, D] (L = 64 *
    prefix_interval) receiving the state after every whole block of L tokens.
    workspace: "auto" (allocate what the library asks for), None, or a
    device uint8 tensor."""
    lib = load_library()
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, q.shape, dev)
    _need(v, "v", q.dtype, (B, T, Hv, Dv), dev)
    _need(alpha, "alpha", torch.float32, (B, T, Hv), dev)
    _need(beta, "beta", torch.float32, (B, T, Hv), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (B, Hv, Dv, Dk), dev)
    if out is None:
        out = torch.empty((B, T, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (B, T, Hv, Dv), dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (B, Hv, Dv, Dk), dev)
    pre, pint = _prefix(prefix_states, prefix_interval,
                        prefix_state_rows(B, T, max(int(prefix_interval), 1), False), Hv, Dv, Dk,
                        dev)
    st = _stream(dev, stream)
    wp, wb, _keep = _workspace(workspace, B, T, Hk, Hv, Dk, Dv, _dtype_code(q), False, dev, st)
    _check(lib.gdn_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(out),
        _ptr(final_state), _ptr(pre), pint, B, T, Hk, Hv, Dk, Dv, _dtype_code(q), float(scale),
        int(flags), wp, wb, st.cuda_stream))
    return out, final_state


def gdn_prefill_chunked_noalloc(q, k, v, alpha, beta, initial_state=None, *, out=None,
                                final_state=None, scale: float = 1.0,
                                want_final_state: bool = True, prefix_states=None,
                                prefix_interval: int = 0, flags: int = 0, stream=None):
    """gdn_prefill_chunked on the library's static device scratch (no
    workspace argument, nothing allocated by the library; outputs the caller
    does not pass are allocated here by torch, as for the other calls).
    Calls that overlap in time on one device race on that scratch."""
    lib = load_library()
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, q.shape, dev)
    _need(v, "v", q.dtype, (B, T, Hv, Dv), dev)
    _need(alpha, "alpha", torch.float32, (B, T, Hv), dev)
    _need(beta, "beta", torch.float32, (B, T, Hv), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (B, Hv, Dv, Dk), dev)
    if out is None:
        out = torch.empty((B, T, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (B, T, Hv, Dv), dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (B, Hv, Dv, Dk), dev)
    pre, pint = _prefix(prefix_states, prefix_interval,
                        prefix_state_rows(B, T, max(int(prefix_interval), 1), False), Hv, Dv, Dk,
                        dev)
    _check(lib.gdn_prefill_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(out),
        _ptr(final_state), _ptr(pre), pint, B, T, Hk, Hv, Dk, Dv, _dtype_code(q), float(scale),
        int(flags), _stream(dev, stream).cuda_stream))
    return out, final_state


def gdn_varlen_prefill(q, k, v, alpha, beta, cu_seqlens, initial_state=None, *, out=None,
                       final_state=None, scale: float = 1.0, want_final_state: bool = True,
                       prefix_states=None, prefix_interval: int = 0, flags: int = 0,
                       workspace="auto", stream=None):
    """Packed prefill. q,k [total,Hk,D]; v [total,Hv,D]; alpha,beta [total,Hv];
    cu_seqlens int32 [N+1] on the device. Returns (out, final_state [N,Hv,D,D]).
    prefix_states: optional fp32 [floor(total / L) + N, Hv, D, D]; block i of
    sequence n lands in row floor(cu_seqlens[n] / L) + n + i."""
    lib = load_library()
    total, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    dev = q.device
    _need(cu_seqlens, "cu_seqlens", torch.int32, device=dev)
    N = cu_seqlens.shape[0] - 1
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, q.shape, dev)
    _need(v, "v", q.dtype, (total, Hv, Dv), dev)
    _need(alpha, "alpha", torch.float32, (total, Hv), dev)
    _need(beta, "beta", torch.float32, (total, Hv), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, Hv, Dv, Dk), dev)
    if out is None:
        out = torch.empty((total, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (total, Hv, Dv), dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((N, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, Hv, Dv, Dk), dev)
    pre, pint = _prefix(prefix_states, prefix_interval,
                        prefix_state_rows(N, total, max(int(prefix_interval), 1), True), Hv, Dv,
                        Dk, dev)
    st = _stream(dev, stream)
    wp, wb, _keep = _workspace(workspace, N, total, Hk, Hv, Dk, Dv, _dtype_code(q), True, dev, st)
    _check(lib.gdn_varlen_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_seqlens), N, total,
        _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(pre), pint, Hk, Hv, Dk, Dv,
        _dtype_code(q), float(scale), int(flags), wp, wb, st.cuda_stream))
    return out, final_state


def gdn_decode_step(q, k, v, alpha, beta, state, *, out=None, scale: float = 1.0, flags: int = 0,
                    stream=None):
    """One token per sequence; `state` [B,Hv,D,D] fp32 is updated in place.
    q,k [B,Hk,D]; v [B,Hv,D]; alpha,beta [B,Hv]. Returns out [B,Hv,D]."""
    lib = load_library()
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, q.shape, dev)
    _need(v, "v", q.dtype, (B, Hv, Dv), dev)
    _need(alpha, "alpha", torch.float32, (B, Hv), dev)
    _need(beta, "beta", torch.float32, (B, Hv), dev)
    _need(state, "state", torch.float32, (B, Hv, Dv, Dk), dev)
    if out is None:
        out = torch.empty((B, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (B, Hv, Dv), dev)
    _check(lib.gdn_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(out), B, Hk, Hv,
        Dk, Dv, _dtype_code(q), float(scale), int(flags), _stream(dev, stream).cuda_stream))
    return out


def gdn_decode_multi(q, k, v, alpha, beta, state_pool, src_slot, dst_slot, *, out=None,
                     step_states=None, want_step_states: bool = False, scale: float = 1.0,
                     flags: int = 0, stream=None):
    """K tokens per sequence against a pool of state slots.
    q,k [B,K,Hk,D]; v [B,K,Hv,D]; alpha,beta [B,K,Hv] fp32; state_pool
    [num_slots,Hv,D,D] fp32; src_slot, dst_slot int32 [B] on the device
    (negative src = zero state, negative dst = final state not written).
    Returns (out [B,K,Hv,D], step_states [B,K,Hv,D,D] fp32 or None)."""
    lib = load_library()
    B, K, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, q.shape, dev)
    _need(v, "v", q.dtype, (B, K, Hv, Dv), dev)
    _need(alpha, "alpha", torch.float32, (B, K, Hv), dev)
    _need(beta, "beta", torch.float32, (B, K, Hv), dev)
    _need(state_pool, "state_pool", torch.float32, device=dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (Hv, Dv, Dk):
        raise ValueError(f"state_pool must have shape [num_slots, {Hv}, {Dv}, {Dk}], "
                         f"got {tuple(state_pool.shape)}")
    _need(src_slot, "src_slot", torch.int32, (B,), dev)
    _need(dst_slot, "dst_slot", torch.int32, (B,), dev)
    if out is None:
        out = torch.empty((B, K, Hv, Dv), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, (B, K, Hv, Dv), dev)
    if step_states is None and want_step_states:
        step_states = torch.empty((B, K, Hv, Dv, Dk), dtype=torch.float32, device=dev)
    if step_states is not None:
        _need(step_states, "step_states", torch.float32, (B, K, Hv, Dv, Dk), dev)
    _check(lib.gdn_decode_multi(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_pool),
        state_pool.shape[0], _ptr(src_slot), _ptr(dst_slot), _ptr(out), _ptr(step_states), B, K,
        Hk, Hv, Dk, Dv, _dtype_code(q), float(scale), int(flags), _stream(dev, stream).cuda_stream))
    return out, step_states


def gdn_version() -> int:
    return load_library().gdn_version()
