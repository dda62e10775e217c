"""Python binding of the MI355X batch-invariant MoE layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libinvariant_moe.so`` (see include/moe.h for the contract of each call).
PyTorch provides device memory and the stream; there is no CPU or PyTorch
fallback — if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinvariant_moe.so")

F32, BF16, MXFP4 = 0, 1, 2
ROUTE = {"softmax": 0, "sigmoid": 1, "hash": 2}
# flags values selecting the gated activation (MOE_FLAG_GLU_* in moe.h)
GLU = {"swiglu": 0, "clamp": 0x1, "situ": 0x2}
FLAG_W4A8 = 0x4  # moe_layer_forward: routed MXFP4 experts run FP4 x FP8
STAGES = ("routing", "permute", "gate_up_gemm", "down_gemm", "combine")
EXPORTS = ("moe_router_workspace_bytes", "moe_router_topk", "moe_routing_scores", "moe_permute_workspace_bytes",
           "moe_permute", "moe_grouped_swiglu_workspace_bytes", "moe_grouped_swiglu",
           "moe_mx_e4m3_quantize", "moe_grouped_swiglu_w4a8_workspace_bytes",
           "moe_grouped_swiglu_w4a8",
           "moe_combine", "moe_residual_rmsnorm", "moe_combine_rmsnorm",
           "moe_layer_workspace_bytes", "moe_layer_forward",
           "moe_set_stage_events", "moe_status_string", "moe_last_error", "moe_abi_version",
           "moe_build_id", "moe_layer_forward_noalloc", "moe_layer_fused_workspace_bytes",
           "moe_layer_forward_fused")


class MoEError(RuntimeError):
    pass


class _Weights(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p), ("dtype", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libinvariant_moe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        u32 = ctypes.c_uint32
        WP = ctypes.POINTER(_Weights)
        L.moe_router_workspace_bytes.argtypes = [i64, i32, i32]
        L.moe_router_workspace_bytes.restype = sz
        L.moe_router_topk.argtypes = [vp, i32, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, vp, sz, vp]
        L.moe_routing_scores.argtypes = [vp, i64, i32, vp, vp]
        L.moe_permute_workspace_bytes.argtypes = [i64, i32]
        L.moe_permute_workspace_bytes.restype = sz
        L.moe_permute.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
        L.moe_grouped_swiglu_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
        L.moe_grouped_swiglu_workspace_bytes.restype = sz
        L.moe_grouped_swiglu.argtypes = [vp, vp, vp, i64, i32, i32, i32, WP, i32, u32, vp, vp, sz, vp]
        L.moe_combine.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, vp, vp]
        L.moe_mx_e4m3_quantize.argtypes = [vp, vp, i64, i32, vp, vp, vp]
        L.moe_grouped_swiglu_w4a8_workspace_bytes.argtypes = [i64, i32, i32, i32]
        L.moe_grouped_swiglu_w4a8_workspace_bytes.restype = sz
        L.moe_grouped_swiglu_w4a8.argtypes = [vp, vp, vp, i64, i32, i32, i32, WP, u32, vp, vp, sz,
                                              vp]
        f32 = ctypes.c_float
        L.moe_residual_rmsnorm.argtypes = [vp, vp, vp, f32, i64, i32, i32, vp, vp, vp]
        L.moe_combine_rmsnorm.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i64, i32, i32, i32, vp,
                                          vp, vp]
        L.moe_layer_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32]
        L.moe_layer_workspace_bytes.restype = sz
        L.moe_layer_forward.argtypes = [vp, vp, vp, vp, WP, WP, i64, i32, i32, i32, i32, i32, i32,
                                        i32, u32, vp, vp, sz, vp]
        L.moe_layer_forward_noalloc.argtypes = [vp, vp, vp, vp, WP, WP, i64, i32, i32, i32, i32,
                                                i32, i32, i32, u32, vp, vp]
        L.moe_layer_fused_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
        L.moe_layer_fused_workspace_bytes.restype = sz
        L.moe_layer_forward_fused.argtypes = [vp, vp, vp, vp, WP, WP, i64, i32, i32, i32, i32, i32,
                                              i32, i32, u32, vp, vp, sz, vp]
        L.moe_set_stage_events.argtypes = [vp, i32]
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_build_id.restype = ctypes.c_char_p
        for name in ("moe_router_topk", "moe_routing_scores", "moe_permute", "moe_grouped_swiglu", "moe_combine",
                     "moe_residual_rmsnorm", "moe_combine_rmsnorm", "moe_layer_forward",
                     "moe_mx_e4m3_quantize", "moe_grouped_swiglu_w4a8",
                     "moe_layer_forward_noalloc", "moe_layer_forward_fused",
                     "moe_set_stage_events", "moe_abi_version"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def build_id() -> str:
    """Source hash compiled into the loaded library (moe_build_id)."""
    return lib().moe_build_id().decode()


def check_build() -> None:
    """Raise if the loaded library was built from other sources than the ones
    next to it (a stale binary)."""
    from . import _build
    want, got = _build.source_hash(), build_id()
    if want != got:
        raise MoEError(f"{LIB_PATH} was built from other sources (build id {got}, sources "
                       f"{want}): rebuild it with __graft_entry__.build()")


def _check(rc: int) -> None:
    if rc != 0:
        L = lib()
        raise MoEError(f"{L.moe_status_string(rc).decode()}: {L.moe_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoEError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise MoEError("tensors must be contiguous")
    return t.data_ptr()


def _act(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise MoEError(f"activation dtype {t.dtype} not supported (float32 or bfloat16)")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on(stream):
    """Allocation context of a call: buffers (workspaces, outputs) are taken
    from the caching allocator on the stream the kernels run on, so a buffer
    released when the call returns is reused only after that stream's work."""
    return torch.cuda.stream(stream) if stream is not None else _nullctx()


class _nullctx:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


def _allocating(fn):
    """Runs an entry point with the caching allocator on its `stream` argument
    (see _on): the workspace it drops and the outputs it returns belong to the
    stream its kernels were enqueued on."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        b = sig.bind(*args, **kw)
        with _on(b.arguments.get("stream")):
            return fn(*args, **kw)
    return wrapper


@dataclass
class ExpertWeights:
    """Weights of G experts: gate/up [G, I, D], down [G, D, I] (bf16 or fp32 tensors),
    or for MXFP4 uint8 codes [G, I, D/2] / [G, D, I/2] plus uint8 E8M0 scales
    [G, I, D/32] / [G, D, I/32]."""
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    gate_scale: Optional[torch.Tensor] = None
    up_scale: Optional[torch.Tensor] = None
    down_scale: Optional[torch.Tensor] = None

    @property
    def dtype(self) -> int:
        if self.gate_scale is not None:
            return MXFP4
        return _act(self.gate)

    def as_struct(self) -> _Weights:
        return _Weights(_ptr(self.gate), _ptr(self.up), _ptr(self.down), _ptr(self.gate_scale),
                        _ptr(self.up_scale), _ptr(self.down_scale), self.dtype)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


@_allocating
def router_topk(x, w_router, bias, token_ids, E: int, k: int, mode: str, stream=None):
    """Routing: returns (topk_idx [T,k] int32, topk_w [T,k] fp32)."""
    if mode == "hash":
        T, D, dev, act = token_ids.shape[0], 32, token_ids.device, BF16
    else:
        T, D = x.shape
        dev, act = x.device, _act(x)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    L = lib()
    nb = L.moe_router_workspace_bytes(T, E, ROUTE[mode])
    ws = _workspace(nb, dev)
    _check(L.moe_router_topk(_ptr(x) if mode != "hash" else None, act,
                             _ptr(w_router) if mode != "hash" else None, _ptr(bias),
                             _ptr(token_ids), T, D, E, k, ROUTE[mode], _ptr(idx), _ptr(w),
                             _ptr(ws), nb, _stream(stream)))
    return idx, w


@_allocating
def routing_scores(logits, mode: str, out=None, stream=None):
    """Elementwise routing sigmoid (mode "sigmoid") or routing exp ("softmax")."""
    if out is None:
        out = torch.empty_like(logits)
    _check(lib().moe_routing_scores(_ptr(logits), logits.numel(), ROUTE[mode], _ptr(out),
                                    _stream(stream)))
    return out


@_allocating
def permute(topk_idx, E: int, x=None, stream=None):
    """Dispatch: returns (counts [E], offsets [E+1], row_token [T*k], pair_row [T*k],
    x_perm [T*k, D] or None)."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * k, dtype=torch.int32, device=dev)
    pair_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    x_perm = None
    act, D = BF16, 32
    if x is not None:
        act, D = _act(x), x.shape[1]
        x_perm = torch.empty((T * k, D), dtype=x.dtype, device=dev)
    L = lib()
    nb = L.moe_permute_workspace_bytes(T, E)
    ws = _workspace(nb, dev)
    _check(L.moe_permute(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(row_token),
                         _ptr(pair_row), _ptr(x), act, D, _ptr(x_perm), _ptr(ws), nb,
                         _stream(stream)))
    return counts, offsets, row_token, pair_row, x_perm


@_allocating
def grouped_swiglu(x_rows, row_index, expert_offsets, R: int, E: int, weights: ExpertWeights,
                   out=None, stream=None, glu: str = "swiglu"):
    """Expert FFN over grouped rows: out [R, D].  glu: "swiglu", "clamp" or "situ"."""
    D = x_rows.shape[1]
    I = weights.gate.shape[1]
    act = _act(x_rows)
    if out is None:
        out = torch.empty((R, D), dtype=x_rows.dtype, device=x_rows.device)
    L = lib()
    nb = L.moe_grouped_swiglu_workspace_bytes(R, E, D, I, act)
    ws = _workspace(nb, x_rows.device)
    wst = weights.as_struct()
    _check(L.moe_grouped_swiglu(_ptr(x_rows), _ptr(row_index), _ptr(expert_offsets), R, E, D, I,
                                ctypes.byref(wst), act, GLU[glu], _ptr(out), _ptr(ws), nb,
                                _stream(stream)))
    return out


@_allocating
def mx_e4m3_quantize(x, row_index=None, R=None, stream=None):
    """MXFP8 (E4M3 + E8M0 per 32) codes [R, K] and scales [R, K/32] of bf16 rows
    x[row_index[r]] (or x[r])."""
    K = x.shape[1]
    if R is None:
        R = row_index.shape[0] if row_index is not None else x.shape[0]
    codes = torch.empty((R, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().moe_mx_e4m3_quantize(_ptr(x), _ptr(row_index), R, K, _ptr(codes),
                                      _ptr(scales), _stream(stream)))
    return codes, scales


@_allocating
def grouped_swiglu_w4a8(x_rows, row_index, expert_offsets, R: int, E: int,
                        weights: ExpertWeights, out=None, stream=None, glu: str = "swiglu"):
    """Expert FFN over grouped rows with MXFP4 weights and MXFP8 activations:
    out [R, D] bf16."""
    D = x_rows.shape[1]
    I = weights.gate.shape[1]
    if out is None:
        out = torch.empty((R, D), dtype=x_rows.dtype, device=x_rows.device)
    L = lib()
    nb = L.moe_grouped_swiglu_w4a8_workspace_bytes(R, E, D, I)
    ws = _workspace(nb + 256, x_rows.device)
    wp = (ws.data_ptr() + 255) // 256 * 256
    wst = weights.as_struct()
    _check(L.moe_grouped_swiglu_w4a8(_ptr(x_rows), _ptr(row_index), _ptr(expert_offsets), R, E,
                                     D, I, ctypes.byref(wst), GLU[glu], _ptr(out), wp,
                                     ws.numel() - (wp - ws.data_ptr()), _stream(stream)))
    return out


@_allocating
def combine(expert_out, topk_idx, topk_w, pair_row, shared_out, out=None, stream=None):
    """Weighted combine: y [T, D]."""
    T, k = topk_idx.shape
    D = expert_out.shape[1]
    if out is None:
        out = torch.empty((T, D), dtype=expert_out.dtype, device=expert_out.device)
    _check(lib().moe_combine(_ptr(expert_out), _ptr(topk_idx), _ptr(topk_w), _ptr(pair_row),
                             _ptr(shared_out), T, k, D, _act(expert_out), _ptr(out),
                             _stream(stream)))
    return out


@_allocating
def residual_rmsnorm(x, residual, gamma, eps: float, residual_out=None, normed=None,
                     stream=None):
    """h = round(x + residual) -> residual_out, RMSNorm(h) * gamma -> normed.
    residual_out may be residual (in place).  Returns (residual_out, normed)."""
    T, D = x.shape
    if residual_out is None:
        residual_out = torch.empty_like(x)
    if normed is None:
        normed = torch.empty_like(x)
    _check(lib().moe_residual_rmsnorm(_ptr(x), _ptr(residual), _ptr(gamma), eps, T, D, _act(x),
                                      _ptr(residual_out), _ptr(normed), _stream(stream)))
    return residual_out, normed


@_allocating
def combine_rmsnorm(expert_out, topk_idx, topk_w, pair_row, shared_out, residual, gamma,
                    eps: float, residual_out=None, normed=None, stream=None):
    """The combine fused with residual_rmsnorm of its output (same bits as the two
    calls).  Returns (residual_out, normed)."""
    T, k = topk_idx.shape
    D = expert_out.shape[1]
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if normed is None:
        normed = torch.empty_like(residual)
    _check(lib().moe_combine_rmsnorm(_ptr(expert_out), _ptr(topk_idx), _ptr(topk_w),
                                     _ptr(pair_row), _ptr(shared_out), _ptr(residual),
                                     _ptr(gamma), eps, T, k, D, _act(expert_out),
                                     _ptr(residual_out), _ptr(normed), _stream(stream)))
    return residual_out, normed


def layer_workspace_bytes(T, D, E, k, I, I_shared, act, wdtype) -> int:
    return lib().moe_layer_workspace_bytes(T, D, E, k, I, I_shared, act, wdtype)


@_allocating
def layer_forward(x, token_ids, w_router, bias, routed: ExpertWeights,
                  shared: Optional[ExpertWeights], E: int, k: int, mode: str, out=None,
                  workspace=None, stream=None, glu: str = "swiglu", w4a8: bool = False):
    """The whole layer: y [T, D].  glu: the gated activation of every expert FFN;
    w4a8: routed MXFP4 experts on MXFP8 activations (FP4 x FP8 MFMA)."""
    T, D = x.shape
    I = routed.gate.shape[1]
    Is = shared.gate.shape[1] if shared is not None else 0
    act = _act(x)
    L = lib()
    nb = L.moe_layer_workspace_bytes(T, D, E, k, I, Is, act, routed.dtype)
    if workspace is None or workspace.numel() < nb:
        workspace = _workspace(nb + 256, x.device)
    if out is None:
        out = torch.empty((T, D), dtype=x.dtype, device=x.device)
    ws_ptr = (workspace.data_ptr() + 255) // 256 * 256
    ws_bytes = workspace.numel() - (ws_ptr - workspace.data_ptr())
    r = routed.as_struct()
    s = shared.as_struct() if shared is not None else None
    _check(L.moe_layer_forward(_ptr(x), _ptr(token_ids), _ptr(w_router), _ptr(bias),
                               ctypes.byref(r), ctypes.byref(s) if s is not None else None,
                               T, D, E, k, I, Is, ROUTE[mode], act,
                               GLU[glu] | (FLAG_W4A8 if w4a8 else 0), _ptr(out), ws_ptr,
                               ws_bytes, _stream(stream)))
    return out


def fused_workspace(T, D, E, k, I, I_shared, device) -> torch.Tensor:
    """A workspace for layer_forward_fused: zeroed (the task queue's header must
    start at zero), with room to align it to 256 bytes."""
    nb = lib().moe_layer_fused_workspace_bytes(T, D, E, k, I, I_shared)
    return torch.zeros(int(nb) + 256, dtype=torch.uint8, device=device)


def _aligned(ws: torch.Tensor):
    p = (ws.data_ptr() + 255) // 256 * 256
    return p, ws.numel() - (p - ws.data_ptr())


def fused_error(workspace: torch.Tensor) -> int:
    """The sticky error word of a fused workspace (nonzero: a bounded wait gave
    up in some call).  Synchronises with the device."""
    p, _ = _aligned(workspace)
    off = p - workspace.data_ptr()
    return int(workspace[off + 8:off + 12].cpu().view(torch.int32)[0])


@_allocating
def layer_forward_fused(x, token_ids, w_router, bias, routed: ExpertWeights,
                        shared: Optional[ExpertWeights], E: int, k: int, mode: str, out=None,
                        workspace=None, stream=None, glu: str = "swiglu"):
    """The whole layer in one kernel launch (moe_layer_forward_fused): y [T, D],
    bit-identical to layer_forward.  workspace: from fused_workspace (zeroed);
    reuse it across calls on one stream."""
    T, D = x.shape
    I = routed.gate.shape[1]
    Is = shared.gate.shape[1] if shared is not None else 0
    L = lib()
    nb = L.moe_layer_fused_workspace_bytes(T, D, E, k, I, Is)
    if workspace is None or workspace.numel() < nb + 256:
        workspace = fused_workspace(T, D, E, k, I, Is, x.device)
    if out is None:
        out = torch.empty((T, D), dtype=x.dtype, device=x.device)
    ws_ptr, ws_bytes = _aligned(workspace)
    r = routed.as_struct()
    s = shared.as_struct() if shared is not None else None
    _check(L.moe_layer_forward_fused(_ptr(x), _ptr(token_ids), _ptr(w_router), _ptr(bias),
                                     ctypes.byref(r), ctypes.byref(s) if s is not None else None,
                                     T, D, E, k, I, Is, ROUTE[mode], _act(x), GLU[glu],
                                     _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


@_allocating
def layer_forward_noalloc(x, token_ids, w_router, bias, routed: ExpertWeights,
                          shared: Optional[ExpertWeights], E: int, k: int, mode: str, out=None,
                          stream=None, glu: str = "swiglu", w4a8: bool = False):
    """layer_forward on the library's fixed device scratch (no workspace
    argument; moe_layer_forward_noalloc).  Pass `out` to allocate nothing at
    all.  Calls that overlap on one GPU race on the scratch."""
    T, D = x.shape
    I = routed.gate.shape[1]
    Is = shared.gate.shape[1] if shared is not None else 0
    if out is None:
        out = torch.empty((T, D), dtype=x.dtype, device=x.device)
    r = routed.as_struct()
    s = shared.as_struct() if shared is not None else None
    _check(lib().moe_layer_forward_noalloc(
        _ptr(x), _ptr(token_ids), _ptr(w_router), _ptr(bias), ctypes.byref(r),
        ctypes.byref(s) if s is not None else None, T, D, E, k, I, Is, ROUTE[mode], _act(x),
        GLU[glu] | (FLAG_W4A8 if w4a8 else 0), _ptr(out), _stream(stream)))
    return out


def set_stage_events(events) -> None:
    """Record hipEvent_t handles between the stages of later layer_forward calls
    (see moe_set_stage_events); None stops recording."""
    L = lib()
    if events is None:
        _check(L.moe_set_stage_events(None, 0))
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    set_stage_events._keep = arr
    _check(L.moe_set_stage_events(arr, len(events)))


class MoELayer:
    """Device-resident layer weights plus one reusable workspace per stream.

    Calls on one stream run in order and share that stream's workspace; calls
    on different streams use different workspaces, so they may overlap.  A
    workspace that grows is replaced after the old one's stream has finished
    with it (the allocator reuses a block only after its stream's work)."""

    def __init__(self, w_router, bias, routed: ExpertWeights, shared: Optional[ExpertWeights],
                 E: int, k: int, mode: str, glu: str = "swiglu", w4a8: bool = False,
                 fused: bool = False):
        self.w_router, self.bias, self.routed, self.shared = w_router, bias, routed, shared
        self.E, self.k, self.mode, self.glu, self.w4a8 = E, k, mode, glu, w4a8
        self.fused = fused  # one kernel launch per forward (layer_forward_fused)
        self._ws = {}  # stream handle -> workspace allocated on that stream

    def forward(self, x, token_ids=None, out=None, stream=None):
        T, D = x.shape
        I = self.routed.gate.shape[1]
        Is = self.shared.gate.shape[1] if self.shared is not None else 0
        st = stream if stream is not None else torch.cuda.current_stream()
        if self.fused:
            nb = lib().moe_layer_fused_workspace_bytes(T, D, self.E, self.k, I, Is) + 256
        else:
            nb = layer_workspace_bytes(T, D, self.E, self.k, I, Is, _act(x),
                                       self.routed.dtype) + 256
        ws = self._ws.get(st.cuda_stream)
        if ws is None or ws.numel() < nb:
            with _on(st):
                ws = (fused_workspace(T, D, self.E, self.k, I, Is, x.device) if self.fused
                      else _workspace(nb, x.device))
            self._ws[st.cuda_stream] = ws
        if self.fused:
            return layer_forward_fused(x, token_ids, self.w_router, self.bias, self.routed,
                                       self.shared, self.E, self.k, self.mode, out=out,
                                       workspace=ws, stream=st, glu=self.glu)
        return layer_forward(x, token_ids, self.w_router, self.bias, self.routed, self.shared,
                             self.E, self.k, self.mode, out=out, workspace=ws,
                             stream=st, glu=self.glu, w4a8=self.w4a8)
