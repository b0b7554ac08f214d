"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: shapes are read off the tensors, device pointers and
the current HIP stream are passed through, and outputs that the caller does not
supply are allocated with torch (device memory is the only thing torch provides
here). Every step of the layer runs in the HIP kernels of libmoe.so; there is
no fallback: if the library is not built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY names another build of the same library (e.g. a sanitizer build)
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
GATINGS = {"topk_softmax": 0, "softmax_topk": 1, "softmax_topk_scaled": 2}
FILL_ORDERS = {"token": 0, "priority": 1}
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)

_lib = None

_i64, _i32, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "moe_capacity": (_i64, [_i64, _i32, _i32, _f32]),
    "moe_rows_max": (ctypes.c_int, [_i64, _i32, _i32, _f32, ctypes.POINTER(_i64)]),
    "moe_permute_workspace_bytes": (ctypes.c_int, [_i64, _i32, ctypes.POINTER(_sz)]),
    "moe_workspace_bytes": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int,
                                           ctypes.POINTER(_sz)]),
    "moe_route": (ctypes.c_int, [_i64, _i32, _i32, _i32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_gating": (ctypes.c_int, [_i64, _i32, _i32, _i32, ctypes.c_int, _i32, _vp, _vp, _vp, _vp, _vp,
                                        _vp]),
    "moe_permute_priority_workspace_bytes": (ctypes.c_int, [_i64, _i32, ctypes.POINTER(_sz)]),
    "moe_permute_priority": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, ctypes.c_int, _vp, _vp, _vp, _i64,
                                            _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_forward_ex": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _i32, _i32, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _sz, _vp]),
    "moe_permute_noalloc": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp]),
    "moe_permute_noalloc_scratch_bytes": (_sz, []),
    "moe_ffn_workspace_bytes": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int,
                                               ctypes.POINTER(_sz)]),
    "moe_grouped_ffn": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_expert_gate_up": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _vp, _vp,
                                          _vp, _vp, _vp]),
    "moe_expert_down": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _vp, _vp,
                                       _vp, _vp, _sz, _vp]),
    "moe_unpermute_combine": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, ctypes.c_int, _vp, _vp, _vp,
                                             _vp, _vp]),
    "moe_forward": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_expert_choice_workspace_bytes": (ctypes.c_int, [_i64, _i32, ctypes.POINTER(_sz)]),
    "moe_route_expert_choice": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, ctypes.c_int, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _vp, _sz, _vp]),
    "moe_gather_rows": (ctypes.c_int, [_i64, _i32, _i64, ctypes.c_int, _vp, _vp, _vp, _vp]),
    "moe_ffn_rows_workspace_bytes": (ctypes.c_int, [_i64, _i32, _i32, _i32, ctypes.c_int, ctypes.POINTER(_sz)]),
    "moe_grouped_ffn_rows": (ctypes.c_int, [_i64, _i32, _i32, _i32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _sz, _vp]),
    "moe_combine_expert_choice": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, ctypes.c_int, _vp, _vp, _vp, _vp,
                                                 _vp]),
    "moe_forward_expert_choice_workspace_bytes": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32,
                                                                 ctypes.c_int, ctypes.POINTER(_sz)]),
    "moe_forward_expert_choice": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _vp, _vp,
                                                 _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_backward_workspace_bytes": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int,
                                                    ctypes.POINTER(_sz)]),
    "moe_backward": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_backward_ex": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _i32, _i32, _vp, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_backward_expert_choice_workspace_bytes": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32,
                                                                  ctypes.c_int, ctypes.POINTER(_sz)]),
    "moe_backward_expert_choice": (ctypes.c_int, [_i64, _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _vp, _vp,
                                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_clock_probe": (ctypes.c_int, [_vp, _i64, _vp]),
    "moe_wall_clock_khz": (ctypes.c_int, [ctypes.POINTER(_i32)]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sparse_mixture_experts_09_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(fn: str, st: int) -> None:
    if st != MOE_OK:
        raise MoeError(fn, st)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _new(stream, shape, dtype, device):
    """A buffer the wrapper allocates for a call enqueued on `stream`. torch's
    caching allocator ties a block to the stream current at allocation and may
    hand it out again as soon as the tensor is dropped; when the kernels run
    on another stream the block is recorded on that one too, so it is not
    reused before they have finished with it."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None:
        t.record_stream(stream)
    return t


def _new_like(stream, ref):
    return _new(stream, ref.shape, ref.dtype, ref.device)


def moe_capacity(T: int, E: int, k: int, cf: float) -> int:
    return int(lib().moe_capacity(T, E, k, cf))


def moe_rows_max(T: int, E: int, k: int, cf: float) -> int:
    r = _i64()
    _check("moe_rows_max", lib().moe_rows_max(T, E, k, cf, ctypes.byref(r)))
    return int(r.value)


def moe_permute_workspace_bytes(T: int, E: int) -> int:
    b = _sz()
    _check("moe_permute_workspace_bytes", lib().moe_permute_workspace_bytes(T, E, ctypes.byref(b)))
    return int(b.value)


def moe_permute_priority_workspace_bytes(T: int, E: int) -> int:
    b = _sz()
    _check("moe_permute_priority_workspace_bytes",
           lib().moe_permute_priority_workspace_bytes(T, E, ctypes.byref(b)))
    return int(b.value)


def moe_workspace_bytes(T: int, d: int, E: int, k: int, cf: float, F: int, dtype) -> int:
    dt = MOE_BF16 if dtype in (torch.bfloat16, MOE_BF16) else MOE_F32
    b = _sz()
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(T, d, E, k, cf, F, dt, ctypes.byref(b)))
    return int(b.value)


def moe_ffn_workspace_bytes(T: int, d: int, E: int, k: int, cf: float, F: int, dtype) -> int:
    dt = MOE_BF16 if dtype in (torch.bfloat16, MOE_BF16) else MOE_F32
    b = _sz()
    _check("moe_ffn_workspace_bytes", lib().moe_ffn_workspace_bytes(T, d, E, k, cf, F, dt, ctypes.byref(b)))
    return int(b.value)


def _ffn_ws(ws, T, d, E, k, cf, F, dtype, device, stream):
    if ws is None:
        n = moe_ffn_workspace_bytes(T, d, E, k, cf, F, dtype)
        ws = _new(stream, n, torch.uint8, device) if n else None
    return ws


def moe_route(x, w_router, k: int, topk_idx=None, topk_gate=None, logits=None, want_logits=False,
              stream=None, gating: str = "topk_softmax"):
    """Returns (topk_idx [T,k] int32, topk_gate [T,k] fp32, logits [T,E] fp32 or None).
    gating: "topk_softmax" (moe_route), "softmax_topk" or "softmax_topk_scaled"
    (moe_route_gating)."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    if topk_idx is None:
        topk_idx = _new(stream, (T, k), torch.int32, dev)
    if topk_gate is None:
        topk_gate = _new(stream, (T, k), torch.float32, dev)
    if logits is None and want_logits:
        logits = _new(stream, (T, E), torch.float32, dev)
    if gating == "topk_softmax":
        st = lib().moe_route(T, d, E, k, _dt(x), _ptr(x), _ptr(w_router), _ptr(topk_idx), _ptr(topk_gate),
                             _ptr(logits), _stream(stream))
        _check("moe_route", st)
    else:
        st = lib().moe_route_gating(T, d, E, k, _dt(x), GATINGS[gating], _ptr(x), _ptr(w_router),
                                    _ptr(topk_idx), _ptr(topk_gate), _ptr(logits), _stream(stream))
        _check("moe_route_gating", st)
    return topk_idx, topk_gate, logits


def moe_permute(x, topk_idx, E: int, cf: float, stream=None, out=None, score=None, score_stride: int = 1):
    """Returns dict(expert_counts, expert_offsets, slot_row, row_slot, x_perm).
    score: fp32 device tensor of importance scores (token t's score at
    flat index t * score_stride) for Batch Priority Routing (moe_permute_priority);
    None fills in token order (moe_permute)."""
    T, d = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    R_max = moe_rows_max(T, E, k, cf)
    o = out or {}

    def get(name, shape, dtype):
        t = o.get(name)
        return t if t is not None else _new(stream, shape, dtype, dev)

    counts = get("expert_counts", E, torch.int32)
    offsets = get("expert_offsets", E + 1, torch.int32)
    slot_row = get("slot_row", (T, k), torch.int32)
    row_slot = get("row_slot", max(R_max, 1), torch.int32)
    x_perm = get("x_perm", (max(R_max, 1), d), x.dtype)
    if score is None:
        ws = get("ws", max(moe_permute_workspace_bytes(T, E), 16), torch.uint8)
        st = lib().moe_permute(T, d, E, k, cf, _dt(x), _ptr(x), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                               _ptr(slot_row), _ptr(row_slot), _ptr(x_perm), _ptr(ws), ws.numel(),
                               _stream(stream))
        _check("moe_permute", st)
    else:
        if score.dtype != torch.float32:
            raise ValueError("score must be float32")
        ws = get("ws", max(moe_permute_priority_workspace_bytes(T, E), 16), torch.uint8)
        st = lib().moe_permute_priority(T, d, E, k, cf, _dt(x), _ptr(x), _ptr(topk_idx), _ptr(score),
                                        score_stride, _ptr(counts), _ptr(offsets), _ptr(slot_row),
                                        _ptr(row_slot), _ptr(x_perm), _ptr(ws), ws.numel(), _stream(stream))
        _check("moe_permute_priority", st)
    return dict(expert_counts=counts, expert_offsets=offsets, slot_row=slot_row, row_slot=row_slot,
                x_perm=x_perm)


def moe_permute_noalloc(x, topk_idx, E: int, cf: float, out, stream=None):
    """moe_permute without a workspace (the library's static device scratch).
    Every output is caller-supplied in `out` (expert_counts [E], expert_offsets
    [E+1], slot_row [T,k], row_slot [>= R_max], x_perm [>= R_max, d]), so the
    call allocates nothing. Returns `out`."""
    T, d = x.shape
    k = topk_idx.shape[1]
    st = lib().moe_permute_noalloc(T, d, E, k, cf, _dt(x), _ptr(x), _ptr(topk_idx), _ptr(out["expert_counts"]),
                                   _ptr(out["expert_offsets"]), _ptr(out["slot_row"]), _ptr(out["row_slot"]),
                                   _ptr(out["x_perm"]), _stream(stream))
    _check("moe_permute_noalloc", st)
    return out


def moe_permute_noalloc_scratch_bytes() -> int:
    return int(lib().moe_permute_noalloc_scratch_bytes())


def moe_grouped_ffn(x_perm, expert_offsets, w_gate, w_up, w_down, T: int, k: int, cf: float,
                    h=None, out_perm=None, ws=None, stream=None):
    """Returns (h [R_max,F], out_perm [R_max,d]). ws: FFN scratch (allocated
    when None; pass False to run without the split tail)."""
    E, F, d = w_gate.shape
    R_max = moe_rows_max(T, E, k, cf)
    dev = x_perm.device
    if h is None:
        h = _new(stream, (max(R_max, 1), F), x_perm.dtype, dev)
    if out_perm is None:
        out_perm = _new(stream, (max(R_max, 1), d), x_perm.dtype, dev)
    ws = None if ws is False else _ffn_ws(ws, T, d, E, k, cf, F, x_perm.dtype, dev, stream)
    st = lib().moe_grouped_ffn(T, d, E, k, cf, F, _dt(x_perm), _ptr(x_perm), _ptr(expert_offsets),
                               _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(out_perm), _ptr(ws),
                               ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_grouped_ffn", st)
    return h, out_perm


def moe_expert_gate_up(x_perm, expert_offsets, w_gate, w_up, T: int, k: int, cf: float, h=None,
                       stream=None):
    """First grouped GEMM with the SwiGLU epilogue. Returns h [R_max, F]."""
    E, F, d = w_gate.shape
    if h is None:
        h = _new(stream, (max(moe_rows_max(T, E, k, cf), 1), F), x_perm.dtype, x_perm.device)
    st = lib().moe_expert_gate_up(T, d, E, k, cf, F, _dt(x_perm), _ptr(x_perm), _ptr(expert_offsets),
                                  _ptr(w_gate), _ptr(w_up), _ptr(h), _stream(stream))
    _check("moe_expert_gate_up", st)
    return h


def moe_expert_down(h, expert_offsets, w_down, T: int, k: int, cf: float, out_perm=None, ws=None,
                    stream=None):
    """Second grouped GEMM. Returns out_perm [R_max, d]. ws: FFN scratch
    (allocated when None; pass False to run without the split tail)."""
    E, d, F = w_down.shape
    if out_perm is None:
        out_perm = _new(stream, (max(moe_rows_max(T, E, k, cf), 1), d), h.dtype, h.device)
    ws = None if ws is False else _ffn_ws(ws, T, d, E, k, cf, F, h.dtype, h.device, stream)
    st = lib().moe_expert_down(T, d, E, k, cf, F, _dt(h), _ptr(h), _ptr(expert_offsets), _ptr(w_down),
                               _ptr(out_perm), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_expert_down", st)
    return out_perm


def moe_unpermute_combine(out_perm, slot_row, topk_gate, E: int, cf: float, y=None, stream=None):
    T, k = slot_row.shape
    d = out_perm.shape[1]
    if y is None:
        y = _new(stream, (T, d), out_perm.dtype, out_perm.device)
    st = lib().moe_unpermute_combine(T, d, E, k, cf, _dt(out_perm), _ptr(out_perm), _ptr(slot_row),
                                     _ptr(topk_gate), _ptr(y), _stream(stream))
    _check("moe_unpermute_combine", st)
    return y


def moe_forward(x, w_router, w_gate, w_up, w_down, k: int, cf: float, y=None, topk_idx=None,
                topk_gate=None, slot_row=None, ws=None, stream=None, gating: str = "topk_softmax",
                fill_order: str = "token"):
    """The whole layer. Returns y [T, d] (topk_idx / topk_gate / slot_row are
    filled when given). The defaults call moe_forward; another gating or
    fill_order ("priority" = Batch Priority Routing) calls moe_forward_ex."""
    T, d = x.shape
    E, F, _ = w_gate.shape
    if y is None:
        y = _new_like(stream, x)
    if ws is None:
        ws = _new(stream, max(moe_workspace_bytes(T, d, E, k, cf, F, x.dtype), 16), torch.uint8, x.device)
    if gating == "topk_softmax" and fill_order == "token":
        st = lib().moe_forward(T, d, E, k, cf, F, _dt(x), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up),
                               _ptr(w_down), _ptr(y), _ptr(topk_idx), _ptr(topk_gate), _ptr(slot_row),
                               _ptr(ws), ws.numel(), _stream(stream))
        _check("moe_forward", st)
    else:
        st = lib().moe_forward_ex(T, d, E, k, cf, F, _dt(x), GATINGS[gating], FILL_ORDERS[fill_order], _ptr(x),
                                  _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y),
                                  _ptr(topk_idx), _ptr(topk_gate), _ptr(slot_row), _ptr(ws), ws.numel(),
                                  _stream(stream))
        _check("moe_forward_ex", st)
    return y


# ---------------------------------------------------------------------------
# expert choice
# ---------------------------------------------------------------------------

def _size_query(fn, *args) -> int:
    b = _sz()
    _check(fn, getattr(lib(), fn)(*args, ctypes.byref(b)))
    return int(b.value)


def moe_route_expert_choice(x, w_router, k: int, cf: float, stream=None):
    """Scores and per-expert selection. Returns dict(scores [T,E] fp32,
    expert_tokens [E*C] int32, slot [T,E] int32, expert_offsets [E+1] int32, C)."""
    T, d = x.shape
    E = w_router.shape[0]
    C = moe_capacity(T, E, k, cf)
    dev = x.device
    out = dict(scores=_new(stream, (T, E), torch.float32, dev),
               expert_tokens=_new(stream, max(E * C, 1), torch.int32, dev),
               slot=_new(stream, (T, E), torch.int32, dev),
               expert_offsets=_new(stream, E + 1, torch.int32, dev), C=C)
    ws = _new(stream, max(_size_query("moe_route_expert_choice_workspace_bytes", T, E), 16), torch.uint8, dev)
    st = lib().moe_route_expert_choice(T, d, E, k, cf, _dt(x), _ptr(x), _ptr(w_router), _ptr(out["scores"]),
                                       _ptr(out["expert_tokens"]), _ptr(out["slot"]), _ptr(out["expert_offsets"]),
                                       _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_route_expert_choice", st)
    return out


def moe_gather_rows(x, row_token, R: int, x_perm=None, stream=None):
    """x_perm[r] = x[row_token[r]] for r < R."""
    T, d = x.shape
    if x_perm is None:
        x_perm = _new(stream, (max(R, 1), d), x.dtype, x.device)
    _check("moe_gather_rows", lib().moe_gather_rows(T, d, R, _dt(x), _ptr(x), _ptr(row_token), _ptr(x_perm),
                                                    _stream(stream)))
    return x_perm


def moe_grouped_ffn_rows(x_perm, expert_offsets, w_gate, w_up, w_down, R_max: int, h=None, out_perm=None,
                         ws=None, stream=None):
    """Grouped SwiGLU FFN over at most R_max expert-major rows. Returns (h, out_perm)."""
    E, F, d = w_gate.shape
    dev = x_perm.device
    if h is None:
        h = _new(stream, (max(R_max, 1), F), x_perm.dtype, dev)
    if out_perm is None:
        out_perm = _new(stream, (max(R_max, 1), d), x_perm.dtype, dev)
    if ws is None:
        n = _size_query("moe_ffn_rows_workspace_bytes", R_max, d, E, F, _dt(x_perm))
        ws = _new(stream, n, torch.uint8, dev) if n else None
    elif ws is False:
        ws = None
    st = lib().moe_grouped_ffn_rows(R_max, d, E, F, _dt(x_perm), _ptr(x_perm), _ptr(expert_offsets), _ptr(w_gate),
                                    _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(out_perm), _ptr(ws),
                                    ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_grouped_ffn_rows", st)
    return h, out_perm


def moe_combine_expert_choice(out_perm, slot, scores, k: int, cf: float, y=None, stream=None):
    T, E = slot.shape
    d = out_perm.shape[1]
    if y is None:
        y = _new(stream, (T, d), out_perm.dtype, out_perm.device)
    st = lib().moe_combine_expert_choice(T, d, E, k, cf, _dt(out_perm), _ptr(out_perm), _ptr(slot), _ptr(scores),
                                         _ptr(y), _stream(stream))
    _check("moe_combine_expert_choice", st)
    return y


def moe_forward_expert_choice(x, w_router, w_gate, w_up, w_down, k: int, cf: float, y=None, scores=None,
                              slot=None, ws=None, stream=None):
    """The whole expert-choice layer. Returns y [T, d] (scores / slot filled when given)."""
    T, d = x.shape
    E, F, _ = w_gate.shape
    if y is None:
        y = _new_like(stream, x)
    if ws is None:
        n = _size_query("moe_forward_expert_choice_workspace_bytes", T, d, E, k, cf, F, _dt(x))
        ws = _new(stream, max(n, 16), torch.uint8, x.device)
    st = lib().moe_forward_expert_choice(T, d, E, k, cf, F, _dt(x), _ptr(x), _ptr(w_router), _ptr(w_gate),
                                         _ptr(w_up), _ptr(w_down), _ptr(y), _ptr(scores), _ptr(slot), _ptr(ws),
                                         ws.numel(), _stream(stream))
    _check("moe_forward_expert_choice", st)
    return y


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------

def moe_backward(x, w_router, w_gate, w_up, w_down, dy, k: int, cf: float, ws=None, stream=None,
                 gating: str = "topk_softmax", fill_order: str = "token"):
    """Gradients of <dy, y> for the token-choice layer (bf16). Returns dict(dx,
    dw_router, dw_gate, dw_up, dw_down), shaped like x and the weights. The
    defaults call moe_backward; another gating or fill_order calls
    moe_backward_ex."""
    T, d = x.shape
    E, F, _ = w_gate.shape
    out = dict(dx=_new_like(stream, x), dw_router=_new_like(stream, w_router), dw_gate=_new_like(stream, w_gate),
               dw_up=_new_like(stream, w_up), dw_down=_new_like(stream, w_down))
    if ws is None:
        n = _size_query("moe_backward_workspace_bytes", T, d, E, k, cf, F, _dt(x))
        ws = _new(stream, max(n, 16), torch.uint8, x.device)
    ptrs = (_ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(dy), _ptr(out["dx"]),
            _ptr(out["dw_router"]), _ptr(out["dw_gate"]), _ptr(out["dw_up"]), _ptr(out["dw_down"]), _ptr(ws),
            ws.numel(), _stream(stream))
    if gating == "topk_softmax" and fill_order == "token":
        _check("moe_backward", lib().moe_backward(T, d, E, k, cf, F, _dt(x), *ptrs))
    else:
        _check("moe_backward_ex", lib().moe_backward_ex(T, d, E, k, cf, F, _dt(x), GATINGS[gating],
                                                        FILL_ORDERS[fill_order], *ptrs))
    return out


def moe_backward_expert_choice(x, w_router, w_gate, w_up, w_down, dy, k: int, cf: float, ws=None, stream=None):
    """Gradients of <dy, y> for the expert-choice layer. Returns dict(dx,
    dw_router, dw_gate, dw_up, dw_down), shaped like x and the weights."""
    T, d = x.shape
    E, F, _ = w_gate.shape
    out = dict(dx=_new_like(stream, x), dw_router=_new_like(stream, w_router), dw_gate=_new_like(stream, w_gate),
               dw_up=_new_like(stream, w_up), dw_down=_new_like(stream, w_down))
    if ws is None:
        n = _size_query("moe_backward_expert_choice_workspace_bytes", T, d, E, k, cf, F, _dt(x))
        ws = _new(stream, max(n, 16), torch.uint8, x.device)
    _check("moe_backward_expert_choice", lib().moe_backward_expert_choice(
        T, d, E, k, cf, F, _dt(x), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(dy),
        _ptr(out["dx"]), _ptr(out["dw_router"]), _ptr(out["dw_gate"]), _ptr(out["dw_up"]), _ptr(out["dw_down"]),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# measurement aid
# ---------------------------------------------------------------------------

def moe_clock_probe(out, wall_ticks: int, stream=None):
    """Enqueue one clock probe writing {core cycles, wall ticks} into out[0:2]
    (a uint64-sized int64 CUDA tensor of at least 2 elements)."""
    _check("moe_clock_probe", lib().moe_clock_probe(_ptr(out), wall_ticks, _stream(stream)))


def moe_wall_clock_khz() -> int:
    v = _i32()
    _check("moe_wall_clock_khz", lib().moe_wall_clock_khz(ctypes.byref(v)))
    return int(v.value)
