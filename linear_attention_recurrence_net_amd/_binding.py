"""ctypes binding of libgdn.so: argument checks and marshalling only."""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_HEAD, GDN_GATE_KEY = 0, 1
GDN_HEADS_GROUPED, GDN_HEADS_TILED = 0, 1
_HEAD_MAPS = {"grouped": GDN_HEADS_GROUPED, "tiled": GDN_HEADS_TILED,
              GDN_HEADS_GROUPED: GDN_HEADS_GROUPED, GDN_HEADS_TILED: GDN_HEADS_TILED}

EXPORTED = (
    "gdn_forward",
    "gdn_forward_snapshots",
    "gdn_rollback_select",
    "gdn_forward_snapshots_after_rollback",
    "gdn_prefill_workspace_size",
    "gdn_prefill_chunked",
    "gdn_forward_qk_broadcast",
    "gdn_prefill_chunked_qk_broadcast",
    "gdn_prefill_varlen_workspace_size",
    "gdn_prefill_chunked_varlen",
    "gdn_prefill_chunked_snapshots",
    "gdn_prefill_kda_workspace_size",
    "gdn_prefill_chunked_kda",
    "gdn_prefill_workspace_size_ex",
    "gdn_prefill_chunked_ex",
    "gdn_prefill_chunked_ex_after_rollback",
    "gdn_prefill_chunked_ex_noalloc",
    "gdn_prefill_varlen_workspace_size_ex",
    "gdn_prefill_chunked_varlen_ex",
    "gdn_status_str",
)

_lib = None


class GdnError(RuntimeError):
    """A non-zero status returned by libgdn."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m linear_attention_recurrence_net_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.gdn_forward.argtypes = [i32] * 7 + [vp] * 8
    lib.gdn_forward.restype = ctypes.c_int
    lib.gdn_forward_snapshots.argtypes = [i32] * 8 + [vp] * 9
    lib.gdn_forward_snapshots.restype = ctypes.c_int
    lib.gdn_rollback_select.argtypes = [i32] * 5 + [vp] * 4
    lib.gdn_rollback_select.restype = ctypes.c_int
    lib.gdn_prefill_workspace_size.argtypes = [i32] * 6
    lib.gdn_prefill_workspace_size.restype = sz
    lib.gdn_prefill_chunked.argtypes = [i32] * 6 + [vp] * 8 + [sz, vp]
    lib.gdn_prefill_chunked.restype = ctypes.c_int
    lib.gdn_forward_qk_broadcast.argtypes = [i32] * 10 + [vp] * 9
    lib.gdn_forward_snapshots_after_rollback.argtypes = [i32] * 10 + [vp] * 11
    lib.gdn_forward_snapshots_after_rollback.restype = ctypes.c_int
    lib.gdn_forward_qk_broadcast.restype = ctypes.c_int
    lib.gdn_prefill_chunked_qk_broadcast.argtypes = [i32] * 8 + [vp] * 8 + [sz, vp]
    lib.gdn_prefill_chunked_snapshots.argtypes = [i32] * 9 + [vp] * 9 + [sz, vp]
    lib.gdn_prefill_chunked_snapshots.restype = ctypes.c_int
    lib.gdn_prefill_kda_workspace_size.argtypes = [i32] * 6
    lib.gdn_prefill_kda_workspace_size.restype = sz
    lib.gdn_prefill_chunked_kda.argtypes = [i32] * 8 + [vp] * 8 + [sz, vp]
    lib.gdn_prefill_chunked_kda.restype = ctypes.c_int
    lib.gdn_prefill_workspace_size_ex.argtypes = [i32] * 8
    lib.gdn_prefill_workspace_size_ex.restype = sz
    lib.gdn_prefill_chunked_ex.argtypes = [i32] * 11 + [vp] * 9 + [sz, vp]
    lib.gdn_prefill_chunked_ex.restype = ctypes.c_int
    lib.gdn_prefill_chunked_ex_after_rollback.argtypes = [i32] * 11 + [vp] * 10 + [sz, vp, vp]
    lib.gdn_prefill_chunked_ex_after_rollback.restype = ctypes.c_int
    lib.gdn_prefill_chunked_ex_noalloc.argtypes = [i32] * 11 + [vp] * 9
    lib.gdn_prefill_chunked_ex_noalloc.restype = ctypes.c_int
    lib.gdn_prefill_chunked_qk_broadcast.restype = ctypes.c_int
    lib.gdn_prefill_varlen_workspace_size.argtypes = [i32] * 6
    lib.gdn_prefill_varlen_workspace_size.restype = sz
    lib.gdn_prefill_chunked_varlen.argtypes = [i32] * 8 + [vp] * 9 + [sz, vp]
    lib.gdn_prefill_varlen_workspace_size_ex.argtypes = [i32] * 8
    lib.gdn_prefill_varlen_workspace_size_ex.restype = sz
    lib.gdn_prefill_chunked_varlen_ex.argtypes = [i32] * 10 + [vp] * 9 + [sz, vp]
    lib.gdn_prefill_chunked_varlen_ex.restype = ctypes.c_int
    lib.gdn_prefill_chunked_varlen.restype = ctypes.c_int
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise GdnError(fn, status, library().gdn_status_str(status).decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(name: str, t: torch.Tensor, dtypes, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(name: str, t: torch.Tensor, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _qkv_gate(q, k, v, g, beta, shared_qk=False):
    """Check q, k, v, g, beta; with shared_qk, q and k may have H_qk heads
    (a divisor of v's H).  Returns B, T, H, dk, dv, dtype, gate, device (and
    H_qk with shared_qk)."""
    _dev_tensor("q", q, (torch.float32, torch.bfloat16))
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H_qk,d_k]" if shared_qk else "q must be [B,T,H,d_k]")
    B, T, Hq, dk = q.shape
    _dev_tensor("k", k, (q.dtype,), dev)
    _dev_tensor("v", v, (q.dtype,), dev)
    _shape("k", k, (B, T, Hq, dk))
    if v.dim() != 4 or tuple(v.shape[:2]) != (B, T) or (not shared_qk and v.shape[2] != Hq):
        raise ValueError("v must be [B,T,H,d_v]")
    H = v.shape[2]
    if shared_qk and (Hq < 1 or H % Hq != 0):
        raise ValueError(f"v has {H} heads, not a multiple of the {Hq} q/k heads")
    dv = v.shape[3]
    _dev_tensor("g", g, (torch.float32,), dev)
    _dev_tensor("beta", beta, (torch.float32,), dev)
    _shape("beta", beta, (B, T, H))
    if g.dim() == 3:
        _shape("g", g, (B, T, H))
        gate = GDN_GATE_HEAD
    else:
        _shape("g", g, (B, T, H, dk))
        gate = GDN_GATE_KEY
    dt = GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32
    if shared_qk:
        return B, T, H, dk, dv, dt, gate, dev, Hq
    return B, T, H, dk, dv, dt, gate, dev


def gdn_forward(q, k, v, g, beta, state, o=None):
    """Single-slot forward, state [B,H,d_k,d_v] updated in place; returns o.

    g is [B,T,H] (GDA) or [B,T,H,d_k] (KDA) log-gates.
    """
    B, T, H, dk, dv, dt, gate, dev = _qkv_gate(q, k, v, g, beta)
    _dev_tensor("state", state, (torch.float32,), dev)
    _shape("state", state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    st = library().gdn_forward(B, T, H, dk, dv, dt, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                               _ptr(beta), _ptr(state), _ptr(o), _stream_ptr(dev))
    _check("gdn_forward", st)
    return o


def gdn_forward_snapshots(q, k, v, g, beta, state, final_state=None, o=None):
    """Forward with K snapshot slots, state [B,H,K,d_k,d_v]; returns o."""
    B, T, H, dk, dv, dt, gate, dev = _qkv_gate(q, k, v, g, beta)
    _dev_tensor("state", state, (torch.float32,), dev)
    if state.dim() != 5:
        raise ValueError("state must be [B,H,K,d_k,d_v]")
    K = state.shape[2]
    _shape("state", state, (B, H, K, dk, dv))
    if final_state is not None:
        _dev_tensor("final_state", final_state, (torch.float32,), dev)
        _shape("final_state", final_state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    st = library().gdn_forward_snapshots(B, T, H, dk, dv, dt, gate, K, _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(g), _ptr(beta), _ptr(state), _ptr(final_state),
                                         _ptr(o), _stream_ptr(dev))
    _check("gdn_forward_snapshots", st)
    return o


def gdn_rollback_select(accepted, state, err_flag=None):
    """Copy slot accepted[b] to slot 0 for every sequence b (in place).

    err_flag: optional device int32 tensor of one element that the caller
    zeroes; set to 1 when an accepted value is outside 0..K-1.
    """
    _dev_tensor("state", state, (torch.float32,), None)
    dev = state.device
    if state.dim() != 5:
        raise ValueError("state must be [B,H,K,d_k,d_v]")
    B, H, K, dk, dv = state.shape
    _dev_tensor("accepted", accepted, (torch.int32,), dev)
    _shape("accepted", accepted, (B,))
    if err_flag is not None:
        _dev_tensor("err_flag", err_flag, (torch.int32,), dev)
        if err_flag.numel() < 1:
            raise ValueError("err_flag must hold one int32")
    st = library().gdn_rollback_select(B, H, K, dk, dv, _ptr(accepted), _ptr(state),
                                       _ptr(err_flag), _stream_ptr(dev))
    _check("gdn_rollback_select", st)


def gdn_prefill_workspace_size(B: int, T: int, H: int, d_k: int, d_v: int, chunk: int = 64) -> int:
    return int(library().gdn_prefill_workspace_size(B, T, H, d_k, d_v, chunk))


def gdn_prefill_chunked(q, k, v, g, beta, state, o=None, workspace=None, chunk: int = 64):
    """Chunked prefill (GDA, bf16 q/k/v), state [B,H,d_k,d_v] in place; returns o.

    workspace: optional uint8 device tensor of at least
    gdn_prefill_workspace_size(...) bytes; allocated here when omitted.
    """
    B, T, H, dk, dv, dt, gate, dev = _qkv_gate(q, k, v, g, beta)
    _dev_tensor("state", state, (torch.float32,), dev)
    _shape("state", state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    if gate != GDN_GATE_HEAD or dt != GDN_BF16:
        raise GdnError("gdn_prefill_chunked", 3,
                       "chunked prefill supports GDA gates with bfloat16 q/k/v only")
    need = gdn_prefill_workspace_size(B, T, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked(B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _ptr(state), _ptr(o), _ptr(workspace),
                                       workspace.numel(), _stream_ptr(dev))
    _check("gdn_prefill_chunked", st)
    return o


def _head_map(head_map) -> int:
    if head_map not in _HEAD_MAPS:
        raise ValueError(f"head_map must be 'grouped' or 'tiled', got {head_map!r}")
    return _HEAD_MAPS[head_map]


def gdn_forward_qk_broadcast(q, k, v, g, beta, state, head_map="grouped", final_state=None,
                             o=None):
    """Forward with q/k [B,T,H_qk,d_k] shared by the H value heads; returns o.

    head_map 'grouped': value head h reads q/k head h // (H // H_qk);
    'tiled': q/k head h % H_qk.  state is [B,H,d_k,d_v] (one slot, in
    place) or [B,H,K,d_k,d_v] (K snapshot slots, as gdn_forward_snapshots).
    """
    B, T, H, dk, dv, dt, gate, dev, Hq = _qkv_gate(q, k, v, g, beta, shared_qk=True)
    hm = _head_map(head_map)
    _dev_tensor("state", state, (torch.float32,), dev)
    if state.dim() == 4:
        K = 1
        _shape("state", state, (B, H, dk, dv))
    elif state.dim() == 5:
        K = state.shape[2]
        _shape("state", state, (B, H, K, dk, dv))
    else:
        raise ValueError("state must be [B,H,d_k,d_v] or [B,H,K,d_k,d_v]")
    if final_state is not None:
        _dev_tensor("final_state", final_state, (torch.float32,), dev)
        _shape("final_state", final_state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    st = library().gdn_forward_qk_broadcast(B, T, H, Hq, hm, dk, dv, dt, gate, K, _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                            _ptr(final_state), _ptr(o), _stream_ptr(dev))
    _check("gdn_forward_qk_broadcast", st)
    return o


def gdn_forward_snapshots_after_rollback(accepted, q, k, v, g, beta, state, head_map="grouped",
                                         final_state=None, o=None, err_flag=None):
    """gdn_rollback_select(accepted, state, err_flag) followed by
    gdn_forward_qk_broadcast on state [B,H,K,d_k,d_v], in one launch; returns o."""
    B, T, H, dk, dv, dt, gate, dev, Hq = _qkv_gate(q, k, v, g, beta, shared_qk=True)
    hm = _head_map(head_map)
    _dev_tensor("state", state, (torch.float32,), dev)
    if state.dim() != 5:
        raise ValueError("state must be [B,H,K,d_k,d_v]")
    K = state.shape[2]
    _shape("state", state, (B, H, K, dk, dv))
    _dev_tensor("accepted", accepted, (torch.int32,), dev)
    _shape("accepted", accepted, (B,))
    if err_flag is not None:
        _dev_tensor("err_flag", err_flag, (torch.int32,), dev)
        if err_flag.numel() < 1:
            raise ValueError("err_flag must hold one int32")
    if final_state is not None:
        _dev_tensor("final_state", final_state, (torch.float32,), dev)
        _shape("final_state", final_state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    st = library().gdn_forward_snapshots_after_rollback(
        B, T, H, Hq, hm, dk, dv, dt, gate, K, _ptr(accepted), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state), _ptr(final_state), _ptr(o), _ptr(err_flag), _stream_ptr(dev))
    _check("gdn_forward_snapshots_after_rollback", st)
    return o


def gdn_prefill_chunked_qk_broadcast(q, k, v, g, beta, state, head_map="grouped", o=None,
                                     workspace=None, chunk: int = 64):
    """Chunked prefill with q/k [B,T,H_qk,d_k] shared by the H value heads
    (head_map as in gdn_forward_qk_broadcast); state [B,H,d_k,d_v] in place;
    returns o."""
    B, T, H, dk, dv, dt, gate, dev, Hq = _qkv_gate(q, k, v, g, beta, shared_qk=True)
    hm = _head_map(head_map)
    _dev_tensor("state", state, (torch.float32,), dev)
    _shape("state", state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    if gate != GDN_GATE_HEAD or dt != GDN_BF16:
        raise GdnError("gdn_prefill_chunked_qk_broadcast", 3,
                       "chunked prefill supports GDA gates with bfloat16 q/k/v only")
    need = gdn_prefill_workspace_size(B, T, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked_qk_broadcast(
        B, T, H, Hq, hm, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state), _ptr(o), _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    _check("gdn_prefill_chunked_qk_broadcast", st)
    return o


def gdn_prefill_chunked_snapshots(q, k, v, g, beta, state, head_map="grouped", final_state=None,
                                  o=None, workspace=None, chunk: int = 64):
    """Chunked prefill writing state snapshots: state [B,H,K,d_k,d_v] with
    slot 0 the input; slot t <- state after t tokens for 1 <= t <= min(T, K-1);
    for K > 1 the final state goes to final_state [B,H,d_k,d_v] if given
    (K == 1: back to slot 0).  q/k may have H_qk heads as in
    gdn_prefill_chunked_qk_broadcast.  Returns o."""
    B, T, H, dk, dv, dt, gate, dev, Hq = _qkv_gate(q, k, v, g, beta, shared_qk=True)
    hm = _head_map(head_map)
    _dev_tensor("state", state, (torch.float32,), dev)
    if state.dim() != 5:
        raise ValueError("state must be [B,H,K,d_k,d_v]")
    K = state.shape[2]
    _shape("state", state, (B, H, K, dk, dv))
    if final_state is not None:
        _dev_tensor("final_state", final_state, (torch.float32,), dev)
        _shape("final_state", final_state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    if gate != GDN_GATE_HEAD or dt != GDN_BF16:
        raise GdnError("gdn_prefill_chunked_snapshots", 3,
                       "chunked prefill supports GDA gates with bfloat16 q/k/v only")
    need = gdn_prefill_workspace_size(B, T, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked_snapshots(
        B, T, H, Hq, hm, dk, dv, chunk, K, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state), _ptr(final_state), _ptr(o), _ptr(workspace), workspace.numel(),
        _stream_ptr(dev))
    _check("gdn_prefill_chunked_snapshots", st)
    return o


def gdn_prefill_kda_workspace_size(B: int, T: int, H: int, d_k: int, d_v: int,
                                   chunk: int = 64) -> int:
    return int(library().gdn_prefill_kda_workspace_size(B, T, H, d_k, d_v, chunk))


def gdn_prefill_chunked_kda(q, k, v, g, beta, state, head_map="grouped", o=None, workspace=None,
                            chunk: int = 64):
    """Chunked prefill with KDA gates g [B,T,H,d_k] (one log-gate per key
    row); q/k [B,T,H_qk,d_k] as in gdn_prefill_chunked_qk_broadcast; state
    [B,H,d_k,d_v] in place; returns o."""
    B, T, H, dk, dv, dt, gate, dev, Hq = _qkv_gate(q, k, v, g, beta, shared_qk=True)
    hm = _head_map(head_map)
    _dev_tensor("state", state, (torch.float32,), dev)
    _shape("state", state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    if gate != GDN_GATE_KEY or dt != GDN_BF16:
        raise GdnError("gdn_prefill_chunked_kda", 3,
                       "KDA chunked prefill takes g [B,T,H,d_k] and bfloat16 q/k/v")
    need = gdn_prefill_kda_workspace_size(B, T, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked_kda(
        B, T, H, Hq, hm, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state), _ptr(o), _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    _check("gdn_prefill_chunked_kda", st)
    return o


def gdn_prefill_workspace_size_ex(B: int, T: int, H: int, d_k: int, d_v: int, chunk: int = 64,
                                  qkv_dtype: int = GDN_BF16, gate: int = GDN_GATE_HEAD) -> int:
    return int(library().gdn_prefill_workspace_size_ex(B, T, H, d_k, d_v, chunk, qkv_dtype, gate))


def _prefill_ex_args(q, k, v, g, beta, state, head_map, final_state, o):
    """Checks shared by the general prefill entry points; returns the sizes,
    codes and the output tensor (allocated when o is None)."""
    B, T, H, dk, dv, dt, gate, dev, Hq = _qkv_gate(q, k, v, g, beta, shared_qk=True)
    hm = _head_map(head_map)
    _dev_tensor("state", state, (torch.float32,), dev)
    if state.dim() == 4:
        K = 1
        _shape("state", state, (B, H, dk, dv))
    elif state.dim() == 5:
        K = state.shape[2]
        _shape("state", state, (B, H, K, dk, dv))
    else:
        raise ValueError("state must be [B,H,d_k,d_v] or [B,H,K,d_k,d_v]")
    if final_state is not None:
        _dev_tensor("final_state", final_state, (torch.float32,), dev)
        _shape("final_state", final_state, (B, H, dk, dv))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (B, T, H, dv))
    return B, T, H, Hq, hm, dk, dv, dt, gate, K, o, dev


def gdn_prefill_chunked_ex(q, k, v, g, beta, state, head_map="grouped", final_state=None, o=None,
                           workspace=None, chunk: int = 64):
    """The general chunked prefill: q/k/v bfloat16 or float32 (rounded to
    bf16 for the MFMA products), g [B,T,H] (GDA) or [B,T,H,d_k] (KDA),
    q/k with H_qk heads (head_map), state [B,H,d_k,d_v] (in place) or
    [B,H,K,d_k,d_v] (K slots as in gdn_prefill_chunked_snapshots, GDA or KDA),
    final_state for K > 1.  Returns o."""
    B, T, H, Hq, hm, dk, dv, dt, gate, K, o, dev = _prefill_ex_args(q, k, v, g, beta, state, head_map,
                                                                    final_state, o)
    need = gdn_prefill_workspace_size_ex(B, T, H, dk, dv, chunk, dt, gate)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked_ex(
        B, T, H, Hq, hm, dk, dv, chunk, dt, gate, K, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state), _ptr(final_state), _ptr(o), _ptr(workspace), workspace.numel(),
        _stream_ptr(dev))
    _check("gdn_prefill_chunked_ex", st)
    return o


def gdn_prefill_chunked_ex_after_rollback(accepted, q, k, v, g, beta, state, head_map="grouped",
                                          final_state=None, o=None, workspace=None, err_flag=None,
                                          chunk: int = 64):
    """gdn_rollback_select(accepted, state, err_flag) followed by
    gdn_prefill_chunked_ex on state [B,H,K,d_k,d_v], the rollback fused into
    the prefill's chain kernel; returns o."""
    B, T, H, Hq, hm, dk, dv, dt, gate, K, o, dev = _prefill_ex_args(q, k, v, g, beta, state, head_map,
                                                                    final_state, o)
    if state.dim() != 5:
        raise ValueError("state must be [B,H,K,d_k,d_v]")
    _dev_tensor("accepted", accepted, (torch.int32,), dev)
    _shape("accepted", accepted, (B,))
    if err_flag is not None:
        _dev_tensor("err_flag", err_flag, (torch.int32,), dev)
        if err_flag.numel() < 1:
            raise ValueError("err_flag must hold one int32")
    need = gdn_prefill_workspace_size_ex(B, T, H, dk, dv, chunk, dt, gate)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked_ex_after_rollback(
        B, T, H, Hq, hm, dk, dv, chunk, dt, gate, K, _ptr(accepted), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(state), _ptr(final_state), _ptr(o), _ptr(workspace), workspace.numel(),
        _ptr(err_flag), _stream_ptr(dev))
    _check("gdn_prefill_chunked_ex_after_rollback", st)
    return o


def gdn_prefill_chunked_ex_noalloc(q, k, v, g, beta, state, o, head_map="grouped", final_state=None,
                                   chunk: int = 64):
    """gdn_prefill_chunked_ex with the library's fixed scratch array as the
    workspace (for callers that cannot allocate: o must be supplied, and
    nothing is allocated here or in the library).  Returns o."""
    if o is None:
        raise ValueError("o must be supplied: this entry point allocates nothing")
    B, T, H, Hq, hm, dk, dv, dt, gate, K, o, dev = _prefill_ex_args(q, k, v, g, beta, state, head_map,
                                                                    final_state, o)
    st = library().gdn_prefill_chunked_ex_noalloc(
        B, T, H, Hq, hm, dk, dv, chunk, dt, gate, K, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state), _ptr(final_state), _ptr(o), _stream_ptr(dev))
    _check("gdn_prefill_chunked_ex_noalloc", st)
    return o


def gdn_prefill_varlen_workspace_size(N: int, total_T: int, H: int, d_k: int, d_v: int,
                                      chunk: int = 64) -> int:
    return int(library().gdn_prefill_varlen_workspace_size(N, total_T, H, d_k, d_v, chunk))


def gdn_prefill_varlen_workspace_size_ex(N: int, total_T: int, H: int, d_k: int, d_v: int,
                                         chunk: int = 64, qkv_dtype: int = GDN_BF16,
                                         gate: int = GDN_GATE_HEAD) -> int:
    return int(library().gdn_prefill_varlen_workspace_size_ex(N, total_T, H, d_k, d_v, chunk, qkv_dtype,
                                                              gate))


def _varlen_args(fn, cu_seqlens, q, k, v, g, beta, state, head_map, o, bf16_only):
    _dev_tensor("q", q, (torch.bfloat16,) if bf16_only else (torch.bfloat16, torch.float32))
    dev = q.device
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k must be [total,H_qk,d_k] and v [total,H,d_v]")
    # reuse the [B,T,H,d] checks with B = 1
    B, T, H, dk, dv, dt, gate, _, Hq = _qkv_gate(q[None], k[None], v[None], g[None], beta[None],
                                                shared_qk=True)
    if bf16_only and gate != GDN_GATE_HEAD:
        raise GdnError(fn, 3, "this entry point takes GDA gates; gdn_prefill_chunked_varlen_ex takes both")
    hm = _head_map(head_map)
    _dev_tensor("cu_seqlens", cu_seqlens, (torch.int32,), dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be [N+1]")
    N = cu_seqlens.numel() - 1
    _dev_tensor("state", state, (torch.float32,), dev)
    _shape("state", state, (N, H, dk, dv))
    if o is None:
        o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    _dev_tensor("o", o, (torch.float32,), dev)
    _shape("o", o, (T, H, dv))
    return N, T, H, Hq, hm, dk, dv, dt, gate, o, dev


def gdn_prefill_chunked_varlen(cu_seqlens, q, k, v, g, beta, state, head_map="grouped", o=None,
                               workspace=None, chunk: int = 64):
    """Chunked prefill of N packed sequences of different lengths.

    cu_seqlens: device int32 [N+1] token offsets (sequence i is tokens
    cu_seqlens[i]:cu_seqlens[i+1]); q, k [total,H_qk,d_k] bfloat16;
    v [total,H,d_v]; g, beta [total,H]; state [N,H,d_k,d_v] updated in
    place; returns o [total,H,d_v] (rows outside every sequence are left as
    allocated).
    """
    N, T, H, Hq, hm, dk, dv, dt, gate, o, dev = _varlen_args(
        "gdn_prefill_chunked_varlen", cu_seqlens, q, k, v, g, beta, state, head_map, o, True)
    need = gdn_prefill_varlen_workspace_size(N, T, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked_varlen(
        N, T, H, Hq, hm, dk, dv, chunk, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(state), _ptr(o), _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    _check("gdn_prefill_chunked_varlen", st)
    return o


def gdn_prefill_chunked_varlen_ex(cu_seqlens, q, k, v, g, beta, state, head_map="grouped", o=None,
                                  workspace=None, chunk: int = 64):
    """gdn_prefill_chunked_varlen with the gate kind and input type of
    gdn_prefill_chunked_ex: q/k/v bfloat16 or float32, g [total,H] (GDA) or
    [total,H,d_k] (KDA).  Returns o."""
    N, T, H, Hq, hm, dk, dv, dt, gate, o, dev = _varlen_args(
        "gdn_prefill_chunked_varlen_ex", cu_seqlens, q, k, v, g, beta, state, head_map, o, False)
    need = gdn_prefill_varlen_workspace_size_ex(N, T, H, dk, dv, chunk, dt, gate)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, (torch.uint8,), dev)
    st = library().gdn_prefill_chunked_varlen_ex(
        N, T, H, Hq, hm, dk, dv, chunk, dt, gate, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(state), _ptr(o), _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    _check("gdn_prefill_chunked_varlen_ex", st)
    return o
