"""Thin Python binding of libtokengate.so (ctypes over torch device tensors).

Functions carry the names of the C entry points.  They only marshal arguments:
check device / dtype / contiguity, pass raw pointers and the current HIP stream,
and turn a non-zero status into TokenGateError.  Every step of the path runs in
the library's HIP kernels; there is no fallback.  If the library is missing the
import fails loudly.
"""
from __future__ import annotations

import atexit
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtokengate.so")

TG_F32, TG_BF16 = 0, 1
TG_OK = 0


class TokenGateError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m learned_token_pruning_scorer_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    return ctypes.CDLL(LIB_PATH)


_lib = _load()
_p, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_lib.tg_abi_version.restype = _i32
_lib.tg_abi_version.argtypes = []
_lib.tg_status_string.restype = ctypes.c_char_p
_lib.tg_status_string.argtypes = [_i32]
_lib.tg_gate_score.restype = _i32
_lib.tg_gate_score.argtypes = [_i32, _i64, _i32, _i32, _p, _i64, _p, _p, _p, _f32, _p, _p]
_lib.tg_num_kept.restype = _i64
_lib.tg_num_kept.argtypes = [_i64, _i64, _i64, _i64]
_lib.tg_select_workspace_bytes.restype = _sz
_lib.tg_select_workspace_bytes.argtypes = [_i64]
_lib.tg_select_topk.restype = _i32
_lib.tg_select_topk.argtypes = [_i64, _p, _i64, _i64, _i64, _p, _p, _sz, _p]
_lib.tg_select_topk_multi.restype = _i32
_lib.tg_select_topk_multi.argtypes = [_i64, _p, _i64, _i64, ctypes.POINTER(ctypes.c_int64), _i32, _p, _p, _sz, _p]
_lib.tg_select_gather.restype = _i32
_lib.tg_select_gather.argtypes = [_i32, _i64, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p, _sz, _p]
_lib.tg_select_gather_noalloc.restype = _i32
_lib.tg_select_gather_noalloc.argtypes = [_i32, _i64, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p, _p]
_lib.tg_select_check.restype = _i32
_lib.tg_select_check.argtypes = [_p, _sz, _p]
_lib.tg_check_positions.restype = _i32
_lib.tg_check_positions.argtypes = [_p, _i64, _p, _p]
_lib.tg_debug_build.restype = _i32
_lib.tg_debug_build.argtypes = []
_lib.tg_select_random.restype = _i32
_lib.tg_select_random.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_uint64, _p, _p, _sz, _p]
_lib.tg_gather_kept.restype = _i32
_lib.tg_gather_kept.argtypes = [_i32, _i64, _i32, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p]
_lib.tg_gated_attention.restype = _i32
_lib.tg_gated_attention.argtypes = [_i32, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _f32, _p, _p]

_lib.tg_gated_attention_lse.restype = _i32
_lib.tg_gated_attention_lse.argtypes = [_i32, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p]
_lib.tg_gated_attention_split_workspace_bytes.restype = _sz
_lib.tg_gated_attention_split_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, _i32]
_lib.tg_gated_attention_split.restype = _i32
_lib.tg_gated_attention_split.argtypes = [_i32, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _f32, _p, _p, _i32,
                                          _p, _sz, _p]
_lib.tg_gated_attention_backward_workspace_bytes.restype = _sz
_lib.tg_gated_attention_backward_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32]
_lib.tg_gated_attention_backward.restype = _i32
_lib.tg_gated_attention_backward.argtypes = [_i32, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p,
                                             _p, _p, _p, _p, _p, _p, _p, _sz, _p]

_lib.tg_qkv_rope_workspace_bytes.restype = _sz
_lib.tg_qkv_rope_workspace_bytes.argtypes = [_i64, _i32]
_lib.tg_qkv_rope.restype = _i32
_lib.tg_qkv_rope.argtypes = [_i32, _i64, _i32, _p, _i64, _p, _p, _i32, _i32, _i32, _p, _f32, _p, _p, _p, _p, _i64,
                             _i64, _p, _sz, _p]

lib = _lib   # raw ctypes handle (the C ABI itself)


def _check(fn: str, status: int):
    if status != TG_OK:
        raise TokenGateError(fn, status, _lib.tg_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TG_F32
    if t.dtype == torch.bfloat16:
        return TG_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _on_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one device")
    return dev


def tg_abi_version() -> int:
    return int(_lib.tg_abi_version())


def tg_status_string(status: int) -> str:
    return _lib.tg_status_string(status).decode()


def tg_num_kept(n: int, doc_begin: int, doc_end: int, k: int) -> int:
    return int(_lib.tg_num_kept(n, doc_begin, doc_end, k))


def tg_select_workspace_bytes(n: int) -> int:
    return int(_lib.tg_select_workspace_bytes(n))


def tg_gate_score(x, w1, w2, b1=None, b2: float = 0.0, out=None, stream=None):
    """scores[i] = b2 + sum_j w2[j] GELU(b1[j] + x[i,:] . w1[j,:]) -> float32 [n]."""
    dev = _on_gpu(x, w1, w2, b1, out)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [n, d_model] with unit column stride")
    if w1.dtype != x.dtype or w2.dtype != x.dtype or not w1.is_contiguous() or not w2.is_contiguous():
        raise ValueError("w1 and w2 must be contiguous and of x's dtype")
    n, d_model = x.shape
    d_hidden = w1.shape[0]
    if w1.shape != (d_hidden, d_model) or w2.shape != (d_hidden,):
        raise ValueError("shape mismatch between x, w1, w2")
    if b1 is not None and (b1.dtype != torch.float32 or b1.shape != (d_hidden,) or not b1.is_contiguous()):
        raise ValueError("b1 must be float32 [d_hidden]")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=dev)
    _check("tg_gate_score", _lib.tg_gate_score(
        _dtype_code(x), n, d_model, d_hidden, _ptr(x), x.stride(0), _ptr(w1), _ptr(b1), _ptr(w2),
        float(b2), _ptr(out), _stream(dev, stream)))
    return out


# Cached selection workspaces, one per (device, stream): calls that share a workspace must
# not run concurrently, and calls on one stream never do.
_workspaces = {}


def _release_workspaces():
    """Drops the cached device buffers while the runtime is still up (interpreter exit runs
    this before module teardown, so no device memory is released after the HIP runtime)."""
    _workspaces.clear()


atexit.register(_release_workspaces)


def select_workspace(n: int, device, stream=None) -> torch.Tensor:
    """Cached, zero-filled selection workspace for `device` and `stream` (default: the
    device's current stream) with room for n scores."""
    need = tg_select_workspace_bytes(n)
    dev = torch.device(device)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    key = (dev, int(s.cuda_stream))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 16), dtype=torch.uint8, device=dev)
        cur = torch.cuda.current_stream(dev)
        if int(cur.cuda_stream) != int(s.cuda_stream):
            s.wait_stream(cur)   # the zero-fill ran on the current stream
        _workspaces[key] = ws
    return ws


def tg_select_check(workspace, stream=None):
    """Synchronises the stream and raises TokenGateError (TG_ERR_INCOMPLETE) if a selection
    on `workspace` gave up waiting or found it not zero-filled: its outputs are then invalid
    and the workspace must be zero-filled again."""
    dev = _on_gpu(workspace)
    _check("tg_select_check", _lib.tg_select_check(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _stream(dev, stream)))


def tg_select_topk(scores, doc_begin: int, doc_end: int, k: int, out=None, workspace=None, stream=None):
    """Kept positions (int32, ascending): all non-document positions + the best min(k, D) document ones."""
    dev = _on_gpu(scores, out, workspace)
    if scores.dtype != torch.float32 or scores.dim() != 1 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 vector")
    n = scores.shape[0]
    m = tg_num_kept(n, doc_begin, doc_end, k)
    if m < 0:
        raise ValueError("invalid document span or budget")
    if out is None:
        out = torch.empty(m, dtype=torch.int32, device=dev)
    elif out.dtype != torch.int32 or out.numel() < m or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor with room for m entries")
    ws = workspace if workspace is not None else select_workspace(n, dev, stream)
    _check("tg_select_topk", _lib.tg_select_topk(
        n, _ptr(scores), doc_begin, doc_end, k, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(dev, stream)))
    return out[:m]


def tg_select_gather(scores, x, doc_begin: int, doc_end: int, k: int, kept=None, x_kept=None, s_kept=None,
                     workspace=None, stream=None):
    """tg_select_topk and tg_gather_kept in one launch -> (kept int32 [m], x_kept [m, d_model], s_kept [m])."""
    dev = _on_gpu(scores, x, kept, x_kept, s_kept, workspace)
    if scores.dtype != torch.float32 or scores.dim() != 1 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 vector")
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[0] != scores.shape[0]:
        raise ValueError("x must be [n, d_model] with unit column stride, one row per score")
    n, d_model = x.shape
    m = tg_num_kept(n, doc_begin, doc_end, k)
    if m < 0:
        raise ValueError("invalid document span or budget")
    if kept is None:
        kept = torch.empty(max(m, 1), dtype=torch.int32, device=dev)
    elif kept.dtype != torch.int32 or kept.numel() < m or not kept.is_contiguous():
        raise ValueError("kept must be a contiguous int32 tensor with room for m entries")
    if x_kept is None:
        x_kept = torch.empty(max(m, 1), d_model, dtype=x.dtype, device=dev)
    elif x_kept.dtype != x.dtype or x_kept.shape[0] < m or x_kept.shape[1] != d_model or x_kept.stride(1) != 1:
        raise ValueError("x_kept must be [>= m, d_model] of x's dtype")
    if s_kept is None:
        s_kept = torch.empty(max(m, 1), dtype=torch.float32, device=dev)
    elif s_kept.dtype != torch.float32 or s_kept.numel() < m or not s_kept.is_contiguous():
        raise ValueError("s_kept must be a contiguous float32 tensor with room for m entries")
    ws = workspace if workspace is not None else select_workspace(n, dev, stream)
    _check("tg_select_gather", _lib.tg_select_gather(
        _dtype_code(x), n, d_model, _ptr(scores), doc_begin, doc_end, k, _ptr(x), x.stride(0), _ptr(kept),
        _ptr(x_kept), x_kept.stride(0), _ptr(s_kept), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(dev, stream)))
    return kept[:m], x_kept[:m], s_kept[:m]


def tg_select_gather_noalloc(scores, x, doc_begin: int, doc_end: int, k: int, kept, x_kept, s_kept, status=None,
                             stream=None):
    """tg_select_gather on the library's static device scratch (no workspace, nothing allocated
    by the library): outputs kept [>= m] int32, x_kept [>= m, d_model], s_kept [>= m] float32
    and the optional status (one int32: 1 if a wait gave up) are the caller's."""
    dev = _on_gpu(scores, x, kept, x_kept, s_kept, status)
    n, d_model = x.shape
    m = tg_num_kept(n, doc_begin, doc_end, k)
    if m < 0:
        raise ValueError("invalid document span or budget")
    if scores.dtype != torch.float32 or scores.shape != (n,) or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 vector with one entry per row of x")
    if x.stride(1) != 1 or x_kept.dtype != x.dtype or x_kept.shape[0] < m or x_kept.shape[1] != d_model \
            or x_kept.stride(1) != 1:
        raise ValueError("x and x_kept must be [rows, d_model] of one dtype with unit column stride")
    if kept.dtype != torch.int32 or kept.numel() < m or s_kept.dtype != torch.float32 or s_kept.numel() < m:
        raise ValueError("kept (int32) and s_kept (float32) need room for m entries")
    if status is not None and (status.dtype != torch.int32 or status.numel() < 1):
        raise ValueError("status must be an int32 tensor of at least one element")
    _check("tg_select_gather_noalloc", _lib.tg_select_gather_noalloc(
        _dtype_code(x), n, d_model, _ptr(scores), doc_begin, doc_end, k, _ptr(x), x.stride(0), _ptr(kept),
        _ptr(x_kept), x_kept.stride(0), _ptr(s_kept), _ptr(status), _stream(dev, stream)))
    return kept[:m], x_kept[:m], s_kept[:m]


def tg_select_topk_multi(scores, doc_begin: int, doc_end: int, ks, out=None, workspace=None, stream=None):
    """tg_select_topk at each budget in ks (one launch) -> list of int32 kept-position tensors."""
    dev = _on_gpu(scores, out, workspace)
    if scores.dtype != torch.float32 or scores.dim() != 1 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 vector")
    n = scores.shape[0]
    ks = [int(k) for k in ks]
    ms = [tg_num_kept(n, doc_begin, doc_end, k) for k in ks]
    if not ks or min(ms) < 0:
        raise ValueError("invalid document span or budgets")
    total = sum(ms)
    if out is None:
        out = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
    elif out.dtype != torch.int32 or out.numel() < total or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor with room for every kept list")
    ws = workspace if workspace is not None else select_workspace(n, dev, stream)
    karr = (ctypes.c_int64 * len(ks))(*ks)
    _check("tg_select_topk_multi", _lib.tg_select_topk_multi(
        n, _ptr(scores), doc_begin, doc_end, karr, len(ks), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(dev, stream)))
    offs = [0]
    for m in ms:
        offs.append(offs[-1] + m)
    return [out[offs[b]:offs[b + 1]] for b in range(len(ks))]


def tg_select_random(n: int, doc_begin: int, doc_end: int, k: int, seed: int, device="cuda", out=None,
                     workspace=None, stream=None):
    """Random-K selector: non-document positions + a seeded uniform min(k, D)-subset of the document."""
    dev = _on_gpu(out, workspace) or torch.device(device)
    m = tg_num_kept(n, doc_begin, doc_end, k)
    if m < 0:
        raise ValueError("invalid document span or budget")
    if out is None:
        out = torch.empty(max(m, 1), dtype=torch.int32, device=dev)
    elif out.dtype != torch.int32 or out.numel() < m or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor with room for m entries")
    ws = workspace if workspace is not None else select_workspace(n, dev, stream)
    _check("tg_select_random", _lib.tg_select_random(
        n, doc_begin, doc_end, k, seed & 0xFFFFFFFFFFFFFFFF, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(dev, stream)))
    return out[:m]


def tg_gather_kept(x, kept_idx, scores=None, out=None, s_out=None, stream=None):
    """(x[kept_idx], scores[kept_idx]) as new or given tensors."""
    dev = _on_gpu(x, kept_idx, scores, out, s_out)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [n, d_model] with unit column stride")
    if kept_idx.dtype != torch.int32 or not kept_idx.is_contiguous():
        raise ValueError("kept_idx must be contiguous int32")
    n, d_model = x.shape
    m = kept_idx.shape[0]
    if out is None:
        out = torch.empty(m, d_model, dtype=x.dtype, device=dev)
    elif out.dtype != x.dtype or out.shape[0] < m or out.shape[1] != d_model or out.stride(1) != 1:
        raise ValueError("out must be [>= m, d_model] of x's dtype")
    if scores is not None:
        if scores.dtype != torch.float32 or not scores.is_contiguous():
            raise ValueError("scores must be contiguous float32")
        if s_out is None:
            s_out = torch.empty(m, dtype=torch.float32, device=dev)
    _check("tg_gather_kept", _lib.tg_gather_kept(
        _dtype_code(x), n, d_model, _ptr(x), x.stride(0), _ptr(kept_idx), m, _ptr(out), out.stride(0),
        _ptr(scores), _ptr(s_out if scores is not None else None), _stream(dev, stream)))
    return out[:m], (s_out[:m] if scores is not None else None)


def tg_check_positions(pos, out=None, stream=None):
    """Number of positions that break "strictly increasing and non-negative" (a device int32
    tensor of one element; `.item()` synchronises)."""
    dev = _on_gpu(pos, out)
    if pos.dtype != torch.int32 or pos.dim() != 1 or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 vector")
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=dev)
    _check("tg_check_positions", _lib.tg_check_positions(_ptr(pos), pos.shape[0], _ptr(out), _stream(dev, stream)))
    return out


def _check_attention_args(q, k, v, pos, s_kept, gain):
    for t in (q, k, v):
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [m, heads, head_dim]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    m, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (m, hkv, d) or v.shape != (m, hkv, d):
        raise ValueError("k/v shape mismatch")
    if pos is not None and (pos.dtype != torch.int32 or pos.shape != (m,) or not pos.is_contiguous()):
        raise ValueError("pos must be contiguous int32 [m]")
    if (s_kept is None) != (gain is None):
        raise ValueError("s_kept and gain must be given together")
    if s_kept is not None:
        if s_kept.dtype != torch.float32 or s_kept.shape != (m,) or not s_kept.is_contiguous():
            raise ValueError("s_kept must be contiguous float32 [m]")
        if gain.dtype != torch.float32 or gain.shape != (hq,) or not gain.is_contiguous():
            raise ValueError("gain must be contiguous float32 [Hq]")


def tg_gated_attention(q, k, v, pos=None, s_kept=None, gain=None, tau: float = 1.0, out=None, stream=None):
    """Token-gated causal attention; q [m, Hq, d], k/v [m, Hkv, d] -> [m, Hq, d]."""
    dev = _on_gpu(q, k, v, pos, s_kept, gain, out)
    _check_attention_args(q, k, v, pos, s_kept, gain)
    m, hq, d = q.shape
    hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _check("tg_gated_attention", _lib.tg_gated_attention(
        _dtype_code(q), m, hq, hkv, d, _ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(s_kept), _ptr(gain),
        float(tau), _ptr(out), _stream(dev, stream)))
    return out


# ---------------------------------------------------------------------------------------
# numpy <-> torch helpers for the stored tensors of the workloads (bf16 kept as uint16 bits)
# ---------------------------------------------------------------------------------------
def to_device(arr, dtype: str, device="cuda"):
    import numpy as np
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host_bits(t: torch.Tensor):
    """Device tensor -> numpy (bf16 as uint16 bit patterns, float32 as float32)."""
    import numpy as np
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def tg_gated_attention_lse(q, k, v, pos=None, s_kept=None, gain=None, tau: float = 1.0, out=None, lse=None,
                           stream=None):
    """tg_gated_attention that also returns the row log-sum-exp -> (out, lse [m, Hq] float32)."""
    dev = _on_gpu(q, k, v, pos, s_kept, gain, out, lse)
    _check_attention_args(q, k, v, pos, s_kept, gain)
    m, hq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(m, hq, dtype=torch.float32, device=dev)
    _check("tg_gated_attention_lse", _lib.tg_gated_attention_lse(
        _dtype_code(q), m, hq, k.shape[1], d, _ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(s_kept), _ptr(gain),
        float(tau), _ptr(out), _ptr(lse), _stream(dev, stream)))
    return out, lse


def tg_gated_attention_split_workspace_bytes(m: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                             split_tiles: int = 0) -> int:
    return int(_lib.tg_gated_attention_split_workspace_bytes(m, n_q_heads, n_kv_heads, head_dim, split_tiles))


def tg_gated_attention_split(q, k, v, pos=None, s_kept=None, gain=None, tau: float = 1.0, out=None, lse=None,
                             split_tiles: int = 0, workspace=None, stream=None):
    """tg_gated_attention with long query tiles' keys split over workgroups and merged;
    `lse` (a [m, Hq] float32 tensor) is filled when given.  -> out"""
    dev = _on_gpu(q, k, v, pos, s_kept, gain, out, lse, workspace)
    _check_attention_args(q, k, v, pos, s_kept, gain)
    m, hq, d = q.shape
    hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    need = tg_gated_attention_split_workspace_bytes(m, hq, hkv, d, split_tiles)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("tg_gated_attention_split", _lib.tg_gated_attention_split(
        _dtype_code(q), m, hq, hkv, d, _ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(s_kept), _ptr(gain),
        float(tau), _ptr(out), _ptr(lse), int(split_tiles), _ptr(ws), ws.numel() if ws is not None else 0,
        _stream(dev, stream)))
    return out


def tg_gated_attention_backward(q, k, v, pos, s_kept, gain, tau, out, lse, dout, workspace=None, stream=None):
    """Gradients (dq, dk, dv, ds_kept or None, dgain or None, dtau) of sum(out * dout)."""
    dev = _on_gpu(q, k, v, pos, s_kept, gain, out, lse, dout, workspace)
    _check_attention_args(q, k, v, pos, s_kept, gain)
    m, hq, d = q.shape
    hkv = k.shape[1]
    for t in (out, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("out and dout must be shaped and typed like q, contiguous")
    if lse.shape != (m, hq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be float32 [m, Hq]")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty(m, dtype=torch.float32, device=dev) if s_kept is not None else None
    dg = torch.empty(hq, dtype=torch.float32, device=dev) if gain is not None else None
    dtau = torch.empty(1, dtype=torch.float32, device=dev)
    need = int(_lib.tg_gated_attention_backward_workspace_bytes(m, hq, hkv, d))
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check("tg_gated_attention_backward", _lib.tg_gated_attention_backward(
        _dtype_code(q), m, hq, hkv, d, _ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(s_kept), _ptr(gain), float(tau),
        _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ds), _ptr(dg), _ptr(dtau), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(dev, stream)))
    return dq, dk, dv, ds, dg, dtau


def tg_qkv_rope(x_kept, w_qkv, pos, n_q_heads: int, n_kv_heads: int, head_dim: int, rope_theta: float,
                b_qkv=None, q_out=None, k_cache=None, v_cache=None, pos_cache=None, cache_slot0: int = 0,
                workspace=None, stream=None):
    """Kept-row QKV projection + rotary embedding at original positions + KV emission.

    Returns (q_out [m, Hq, d], k_cache, v_cache, pos_cache); caches default to [slot0 + m, Hkv, d]."""
    dev = _on_gpu(x_kept, w_qkv, pos, b_qkv, q_out, k_cache, v_cache, pos_cache, workspace)
    if x_kept.dim() != 2 or x_kept.stride(1) != 1:
        raise ValueError("x_kept must be [m, d_model] with unit column stride")
    m, d_model = x_kept.shape
    n_feat = (n_q_heads + 2 * n_kv_heads) * head_dim
    if w_qkv.shape != (n_feat, d_model) or not w_qkv.is_contiguous() or w_qkv.dtype != x_kept.dtype:
        raise ValueError("w_qkv must be contiguous [(Hq + 2 Hkv) d, d_model] of x_kept's dtype")
    if pos.dtype != torch.int32 or pos.shape != (m,) or not pos.is_contiguous():
        raise ValueError("pos must be contiguous int32 [m]")
    if b_qkv is not None and (b_qkv.dtype != torch.float32 or b_qkv.shape != (n_feat,) or not b_qkv.is_contiguous()):
        raise ValueError("b_qkv must be contiguous float32 [(Hq + 2 Hkv) d]")
    if q_out is None:
        q_out = torch.empty(m, n_q_heads, head_dim, dtype=x_kept.dtype, device=dev)
    cap = cache_slot0 + m
    if k_cache is None:
        k_cache = torch.empty(cap, n_kv_heads, head_dim, dtype=x_kept.dtype, device=dev)
    if v_cache is None:
        v_cache = torch.empty(k_cache.shape, dtype=x_kept.dtype, device=dev)
    if (k_cache.shape != v_cache.shape or k_cache.dim() != 3 or k_cache.shape[1:] != (n_kv_heads, head_dim)
            or not (k_cache.is_contiguous() and v_cache.is_contiguous())):
        raise ValueError("k_cache / v_cache must be contiguous [capacity, Hkv, d]")
    if q_out.shape != (m, n_q_heads, head_dim) or not q_out.is_contiguous():
        raise ValueError("q_out must be contiguous [m, Hq, d]")
    if pos_cache is not None and (pos_cache.dtype != torch.int32 or pos_cache.shape != (k_cache.shape[0],)):
        raise ValueError("pos_cache must be int32 [capacity]")
    need = int(_lib.tg_qkv_rope_workspace_bytes(m, head_dim))
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check("tg_qkv_rope", _lib.tg_qkv_rope(
        _dtype_code(x_kept), m, d_model, _ptr(x_kept), x_kept.stride(0), _ptr(w_qkv), _ptr(b_qkv), n_q_heads,
        n_kv_heads, head_dim, _ptr(pos), float(rope_theta), _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
        _ptr(pos_cache), cache_slot0, k_cache.shape[0], _ptr(ws), ws.numel() * ws.element_size(),
        _stream(dev, stream)))
    return q_out, k_cache, v_cache, pos_cache
