"""ctypes binding of libspecverify (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI of
``include/specverify.h``; this module converts torch tensors to device
pointers, allocates outputs and workspace with torch's caching allocator, and
passes torch's current HIP stream (or the ``stream=`` given).  Outputs and
workspace it allocates are allocated on the stream the call runs on, so the
caching allocator reuses their memory only in that stream's order.  There is
no CPU fallback: when the shared library is missing or fails to load, every
call raises.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARGUMENT, SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_UNSUPPORTED, SV_ERR_HIP = range(5)
SV_F32, SV_BF16 = 0, 1

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


def load() -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libspecverify.so not built: run `python -m draft_token_verification_chain_amd.build` "
                          f"(expected at {LIB_PATH})")
    lib = ctypes.CDLL(LIB_PATH)
    i, p, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.sv_version.restype = i
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_status_string.argtypes = [i]
    for fn in ("sv_chain_workspace_bytes", "sv_greedy_workspace_bytes", "sv_tree_workspace_bytes",
               "sv_tree_sampled_workspace_bytes"):
        getattr(lib, fn).restype = sz
        getattr(lib, fn).argtypes = [i, i, i, i]
    lib.sv_verify_chain.restype = i
    lib.sv_verify_chain.argtypes = [i, i, i, i] + [p] * 9 + [sz, p]
    lib.sv_verify_chain_static.restype = i
    lib.sv_verify_chain_static.argtypes = [i, i, i, i] + [p] * 9
    lib.sv_verify_greedy.restype = i
    lib.sv_verify_greedy.argtypes = [i, i, i, i] + [p] * 5 + [sz, p]
    lib.sv_verify_tree.restype = i
    lib.sv_verify_tree.argtypes = [i, i, i, i, p, p, i, i, p, p, p, p, p, sz, p]
    lib.sv_verify_tree_sampled.restype = i
    lib.sv_verify_tree_sampled.argtypes = [i, i, i, i, p, p, i, i] + [p] * 8 + [sz, p]
    lib.sv_commit_tokens.restype = i
    lib.sv_commit_tokens.argtypes = [i, i, p, p, p, p, i, p, p, p, p]
    lib.sv_set_handoff_polls.restype = i
    lib.sv_set_handoff_polls.argtypes = [i]
    lib.sv_profile_begin.restype = i
    lib.sv_profile_begin.argtypes = [i]
    lib.sv_profile_end.restype = i
    lib.sv_profile_end.argtypes = [p, i]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sv_status_string(int(status)).decode()


def version() -> int:
    return int(load().sv_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name: str, t: torch.Tensor, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context of a call: the given stream, else the current one."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def chain_workspace_bytes(B: int, k: int, V: int, dtype: int) -> int:
    return int(load().sv_chain_workspace_bytes(B, k, V, dtype))


def greedy_workspace_bytes(B: int, k: int, V: int, dtype: int) -> int:
    return int(load().sv_greedy_workspace_bytes(B, k, V, dtype))


def tree_workspace_bytes(B: int, N: int, V: int, dtype: int) -> int:
    return int(load().sv_tree_workspace_bytes(B, N, V, dtype))


def tree_sampled_workspace_bytes(B: int, N: int, V: int, dtype: int) -> int:
    return int(load().sv_tree_sampled_workspace_bytes(B, N, V, dtype))


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def verify_chain(draft_tokens, draft_logits, target_logits, temperature, uniforms, *,
                 accept_prob: bool = True, workspace=None, stream=None, out=None) -> dict:
    """Chain verification with sampling; see ``sv_verify_chain``.

    draft_tokens [B,k] int32, draft_logits [B,k,V], target_logits [B,k+1,V]
    (bf16 or f32, same dtype), temperature [B] f32, uniforms [B,k+1] f32.
    Returns device tensors accepted_len [B], emitted [B,k+1] and accept_prob
    [B,k] (or None).
    """
    lib = load()
    B, k1, V = target_logits.shape
    k = k1 - 1
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    _check_dev("target_logits", target_logits)
    _check_dev("draft_logits", draft_logits, target_logits.dtype, (B, k, V))
    _check_dev("draft_tokens", draft_tokens, torch.int32, (B, k))
    _check_dev("temperature", temperature, torch.float32, (B,))
    _check_dev("uniforms", uniforms, torch.float32, (B, k + 1))
    with _on(stream):
        if out is None:
            out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                       emitted=torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                       accept_prob=torch.empty((B, k), dtype=torch.float32, device=dev) if accept_prob else None)
        ws = _workspace(lib.sv_chain_workspace_bytes(B, k, V, dt), dev, workspace)
    st = lib.sv_verify_chain(B, k, V, dt, _ptr(draft_tokens), _ptr(draft_logits), _ptr(target_logits),
                             _ptr(temperature), _ptr(uniforms), _ptr(out["accepted_len"]), _ptr(out["emitted"]),
                             _ptr(out.get("accept_prob")), _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError("sv_verify_chain", st)
    return out


def verify_chain_static(draft_tokens, draft_logits, target_logits, temperature, uniforms, *,
                        accept_prob: bool = True, stream=None, out=None) -> dict:
    """Chain verification on the library's own device workspace; see
    ``sv_verify_chain_static``.  Same arguments and outputs as verify_chain
    (without a workspace); the library allocates nothing, and calls that
    overlap on one GPU race."""
    lib = load()
    B, k1, V = target_logits.shape
    k = k1 - 1
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    _check_dev("target_logits", target_logits)
    _check_dev("draft_logits", draft_logits, target_logits.dtype, (B, k, V))
    _check_dev("draft_tokens", draft_tokens, torch.int32, (B, k))
    _check_dev("temperature", temperature, torch.float32, (B,))
    _check_dev("uniforms", uniforms, torch.float32, (B, k + 1))
    if out is None:
        with _on(stream):
            out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                       emitted=torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                       accept_prob=torch.empty((B, k), dtype=torch.float32, device=dev) if accept_prob else None)
    st = lib.sv_verify_chain_static(B, k, V, dt, _ptr(draft_tokens), _ptr(draft_logits), _ptr(target_logits),
                                    _ptr(temperature), _ptr(uniforms), _ptr(out["accepted_len"]),
                                    _ptr(out["emitted"]), _ptr(out.get("accept_prob")), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError("sv_verify_chain_static", st)
    return out


def verify_greedy(draft_tokens, target_logits, *, workspace=None, stream=None, out=None) -> dict:
    """Greedy (temperature 0) chain verification; see ``sv_verify_greedy``."""
    lib = load()
    B, k1, V = target_logits.shape
    k = k1 - 1
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    _check_dev("target_logits", target_logits)
    _check_dev("draft_tokens", draft_tokens, torch.int32, (B, k))
    with _on(stream):
        if out is None:
            out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                       emitted=torch.empty((B, k + 1), dtype=torch.int32, device=dev))
        ws = _workspace(lib.sv_greedy_workspace_bytes(B, k, V, dt), dev, workspace)
    st = lib.sv_verify_greedy(B, k, V, dt, _ptr(draft_tokens), _ptr(target_logits), _ptr(out["accepted_len"]),
                              _ptr(out["emitted"]), _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError("sv_verify_greedy", st)
    return out


def verify_tree(node_tokens, parent, max_depth: int, target_logits, *, accepted_nodes: bool = True,
                workspace=None, stream=None, out=None) -> dict:
    """Greedy static-tree verification; see ``sv_verify_tree``.

    node_tokens [B,N] int32, parent [N] (shared) or [B,N] int32, target_logits
    [B,N,V].  Returns accepted_len [B], emitted [B,max_depth+1] and
    accepted_nodes [B,max_depth+1] (or None).
    """
    lib = load()
    B, N, V = target_logits.shape
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    _check_dev("target_logits", target_logits)
    _check_dev("node_tokens", node_tokens, torch.int32, (B, N))
    _check_dev("parent", parent, torch.int32)
    if parent.dim() == 1:
        if parent.shape[0] != N:
            raise ValueError("parent must have N entries")
        stride = 0
    else:
        if parent.shape[0] != B or parent.shape[1] < N:
            raise ValueError("parent must be [N] or [B, >=N]")
        stride = parent.shape[1]
    w = max_depth + 1
    with _on(stream):
        if out is None:
            out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                       emitted=torch.empty((B, w), dtype=torch.int32, device=dev),
                       accepted_nodes=torch.empty((B, w), dtype=torch.int32, device=dev) if accepted_nodes else None)
        ws = _workspace(lib.sv_tree_workspace_bytes(B, N, V, dt), dev, workspace)
    st = lib.sv_verify_tree(B, N, V, dt, _ptr(node_tokens), _ptr(parent), stride, max_depth, _ptr(target_logits),
                            _ptr(out["accepted_len"]), _ptr(out["emitted"]), _ptr(out["accepted_nodes"]),
                            _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError("sv_verify_tree", st)
    return out


def verify_tree_sampled(node_tokens, parent, max_depth: int, draft_logits, target_logits, temperature, uniforms, *,
                        accepted_nodes: bool = True, workspace=None, stream=None, out=None) -> dict:
    """Sampled tree verification (multi-step speculative sampling); see
    ``sv_verify_tree_sampled``.

    node_tokens [B,N] int32, parent [N] (shared) or [B,N] int32, draft_logits
    and target_logits [B,N,V] (same dtype), temperature [B] f32, uniforms
    [B,N] f32.  Returns accepted_len [B], emitted [B,max_depth+1] and
    accepted_nodes [B,max_depth+1] (or None).
    """
    lib = load()
    B, N, V = target_logits.shape
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    _check_dev("target_logits", target_logits)
    _check_dev("draft_logits", draft_logits, target_logits.dtype, (B, N, V))
    _check_dev("node_tokens", node_tokens, torch.int32, (B, N))
    _check_dev("parent", parent, torch.int32)
    _check_dev("temperature", temperature, torch.float32, (B,))
    _check_dev("uniforms", uniforms, torch.float32, (B, N))
    if parent.dim() == 1:
        if parent.shape[0] != N:
            raise ValueError("parent must have N entries")
        stride = 0
    else:
        if parent.shape[0] != B or parent.shape[1] < N:
            raise ValueError("parent must be [N] or [B, >=N]")
        stride = parent.shape[1]
    w = max_depth + 1
    with _on(stream):
        if out is None:
            out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                       emitted=torch.empty((B, w), dtype=torch.int32, device=dev),
                       accepted_nodes=torch.empty((B, w), dtype=torch.int32, device=dev) if accepted_nodes else None)
        ws = _workspace(lib.sv_tree_sampled_workspace_bytes(B, N, V, dt), dev, workspace)
    st = lib.sv_verify_tree_sampled(B, N, V, dt, _ptr(node_tokens), _ptr(parent), stride, max_depth,
                                    _ptr(draft_logits), _ptr(target_logits), _ptr(temperature), _ptr(uniforms),
                                    _ptr(out["accepted_len"]), _ptr(out["emitted"]), _ptr(out["accepted_nodes"]),
                                    _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError("sv_verify_tree_sampled", st)
    return out


def commit_tokens(accepted_len, emitted, seq_len, history=None, *, packed: bool = True, status: bool = True,
                  stream=None, out=None) -> dict:
    """Appends each sequence's committed tokens to its history and advances
    seq_len in place; see ``sv_commit_tokens``.  Returns packed_offsets
    [B+1], packed [B*width] (only the first packed_offsets[B] are written)
    and status [B] (or None for those not requested)."""
    lib = load()
    B, width = emitted.shape
    dev = emitted.device
    _check_dev("accepted_len", accepted_len, torch.int32, (B,))
    _check_dev("emitted", emitted, torch.int32)
    _check_dev("seq_len", seq_len, torch.int32, (B,))
    stride = 0
    if history is not None:
        _check_dev("history", history, torch.int32)
        if history.dim() != 2 or history.shape[0] != B:
            raise ValueError("history must be [B, capacity]")
        stride = history.shape[1]
    if out is None:
        with _on(stream):
            out = dict(packed_offsets=torch.empty(B + 1, dtype=torch.int32, device=dev) if packed else None,
                       packed=torch.empty(max(B * width, 1), dtype=torch.int32, device=dev) if packed else None,
                       status=torch.empty(B, dtype=torch.int32, device=dev) if status else None)
    st = lib.sv_commit_tokens(B, width, _ptr(accepted_len), _ptr(emitted), _ptr(seq_len), _ptr(history), stride,
                              _ptr(out["packed_offsets"]), _ptr(out["packed"]), _ptr(out["status"]), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError("sv_commit_tokens", st)
    return out


def set_handoff_polls(polls: int) -> int:
    """sv_set_handoff_polls: returns the previous value."""
    return int(load().sv_set_handoff_polls(int(polls)))


def profile_begin(max_launches: int) -> None:
    st = load().sv_profile_begin(int(max_launches))
    if st != SV_OK:
        raise SpecVerifyError("sv_profile_begin", st)


def profile_end(max_out: int = 32) -> dict:
    """Per-kernel (launches, total_ms) recorded since profile_begin()."""
    recs = (KernelTime * max_out)()
    n = load().sv_profile_end(recs, max_out)
    if n < 0:
        raise RuntimeError("sv_profile_end failed")
    return {recs[i].name.decode(): (recs[i].launches, recs[i].total_ms) for i in range(n)}
