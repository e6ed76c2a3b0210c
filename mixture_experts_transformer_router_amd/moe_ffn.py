"""ctypes binding of libmoe_ffn.so (argument marshalling only).

Every step of the layer runs in the library's HIP kernels; this module only
turns torch tensors into device pointers and sizes, allocates the output and
workspace with torch (the caching allocator), and passes torch's current HIP
stream.  The entry points keep the C names:

    forward(...)          -> moe_ffn_forward         (GPT-OSS routing, clipped SwiGLU)
    forward_mxfp4(...)    -> moe_ffn_forward_mxfp4   (MXFP4 expert weights)
    forward_grouped(...)  -> moe_ffn_forward_grouped (GLM group-limited routing, shared expert)
    workspace_bytes(...)  -> moe_ffn_workspace_bytes
    each with block=MoeBlock(...) -> the moe_block_* entry point of the same
    layer (RMSNorm in front, residual after) and moe_block_workspace_bytes
    forward_grouped_affine(...) -> moe_block_forward_grouped_affine
                                   (affine group-quantized routed experts)

If the shared library has not been built, loading raises MoeLibraryMissing;
there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ffn.so")
_lib = None

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_CLIPPED_SWIGLU, MOE_ACT_SILU = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
STAGES = ("route", "permute", "gate_up", "down", "combine")

EXPORTED = ("moe_ffn_workspace_bytes", "moe_ffn_forward", "moe_ffn_forward_mxfp4",
            "moe_ffn_forward_grouped", "moe_status_string", "moe_last_error_detail",
            "moe_ffn_profile_enable", "moe_ffn_profile_read", "moe_block_workspace_bytes",
            "moe_block_forward", "moe_block_forward_mxfp4", "moe_block_forward_grouped",
            "moe_block_forward_grouped_affine", "moe_ffn_forward_mxfp4_mxfp8",
            "moe_ffn_workspace_bytes_mxfp8", "moe_mxfp8_quantize", "moe_ffn_forward_mxfp8_mxfp8",
            "moe_ffn_forward_nvfp4", "moe_ffn_mxfp8_h_layout", "moe_ffn_forward_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class MoeBlock(ctypes.Structure):
    """moe_block: RMSNorm scale (device pointer or None), epsilon, residual flag."""
    _fields_ = [("norm_w", ctypes.c_void_p), ("eps", ctypes.c_float), ("residual", ctypes.c_int)]


def make_block(norm_w: Optional[torch.Tensor], eps: float = 1e-5, residual: bool = True) -> MoeBlock:
    """A moe_block for `norm_w` (a device tensor [d], kept alive by the caller)."""
    return MoeBlock(None if norm_w is None else norm_w.data_ptr(), eps, int(bool(residual)))


class AffineExperts(ctypes.Structure):
    """moe_affine_experts: bits, then (codes, scales, biases) device pointers of gate, up, down."""
    _fields_ = [("bits", ctypes.c_int)] + [(f"{w}_{part}", ctypes.c_void_p)
                                          for w in ("gate", "up", "down") for part in ("q", "scales", "biases")]


def make_affine(bits: int, t: dict) -> AffineExperts:
    """moe_affine_experts from device tensors t["w_gate_q"], t["w_gate_qscales"], ... (kept alive by the caller)."""
    vals = [bits]
    for w in ("gate", "up", "down"):
        vals += [t[f"w_{w}_q"].data_ptr(), t[f"w_{w}_qscales"].data_ptr(), t[f"w_{w}_qbiases"].data_ptr()]
    return AffineExperts(*vals)


class RoutingOut(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("sorted_pair", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libmoe_ffn.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MoeLibraryMissing(f"{_LIB_PATH} is not built; run "
                                "`python -m mixture_experts_transformer_router_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    L.moe_ffn_workspace_bytes.restype = _Z
    L.moe_ffn_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I]
    L.moe_ffn_forward.restype = _I
    L.moe_ffn_forward.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F,
                                  _P, _I, _P, _Z, _P, _P]
    L.moe_ffn_forward_noalloc.restype = _I
    L.moe_ffn_forward_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F,
                                          _P, _I, _P, _P]
    L.moe_ffn_forward_mxfp4.restype = _I
    L.moe_ffn_forward_mxfp4.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _I, _I, _I, _I, _I, _F, _F, _P, _P, _Z, _P, _P]
    L.moe_ffn_forward_mxfp4_mxfp8.restype = _I
    L.moe_ffn_forward_mxfp4_mxfp8.argtypes = L.moe_ffn_forward_mxfp4.argtypes
    L.moe_ffn_forward_mxfp8_mxfp8.restype = _I
    L.moe_ffn_forward_mxfp8_mxfp8.argtypes = L.moe_ffn_forward_mxfp4.argtypes
    L.moe_ffn_workspace_bytes_mxfp8.restype = _Z
    L.moe_ffn_workspace_bytes_mxfp8.argtypes = [_I, _I, _I, _I, _I]
    L.moe_ffn_forward_nvfp4.restype = _I
    L.moe_ffn_forward_nvfp4.argtypes = [_P, _P, _P, _P, _P, _F, _P, _P, _P, _F, _P, _P, _P, _F, _P,
                                        _I, _I, _I, _I, _I, _F, _F, _P, _P, _Z, _P, _P]
    L.moe_mxfp8_quantize.restype = _I
    L.moe_mxfp8_quantize.argtypes = [_P, _I, _I, _P, _P, _P]
    L.moe_ffn_forward_grouped.restype = _I
    L.moe_ffn_forward_grouped.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                                          _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _F, _F,
                                          _P, _I, _P, _Z, _P, _P]
    for name in ("moe_ffn_forward", "moe_ffn_forward_mxfp4", "moe_ffn_forward_grouped"):
        blk = getattr(L, name.replace("moe_ffn_", "moe_block_"))
        blk.restype = _I
        blk.argtypes = [_P] + getattr(L, name).argtypes
    L.moe_block_forward_grouped_affine.restype = _I
    L.moe_block_forward_grouped_affine.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                                                   _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _F, _F,
                                                   _P, _P, _Z, _P, _P]
    L.moe_block_workspace_bytes.restype = _Z
    L.moe_block_workspace_bytes.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _I]
    L.moe_ffn_mxfp8_h_layout.restype = _I
    L.moe_ffn_mxfp8_h_layout.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [_I]
    L.moe_last_error_detail.restype = ctypes.c_char_p
    L.moe_last_error_detail.argtypes = []
    L.moe_ffn_profile_enable.restype = _I
    L.moe_ffn_profile_enable.argtypes = [ctypes.c_uint]
    L.moe_ffn_profile_read.restype = _I
    L.moe_ffn_profile_read.argtypes = [_P, _P, _I]
    _lib = L
    return L


def _check(status: int):
    if status != MOE_OK:
        L = load()
        raise MoeError(status, f"{L.moe_status_string(status).decode()}: "
                               f"{L.moe_last_error_detail().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def workspace_bytes(T, d, d_ff, E, k, dtype=MOE_BF16, d_ff_shared=0, block: Optional[MoeBlock] = None,
                    grouped: bool = False) -> int:
    """moe_ffn_workspace_bytes (moe_block_workspace_bytes with `block`); grouped: the
    group-routed layer (implied by a shared expert)."""
    g = int(bool(grouped) or d_ff_shared > 0)
    if block is None:
        n = load().moe_ffn_workspace_bytes(T, d, d_ff, E, k, dtype, g, d_ff_shared)
    else:
        n = load().moe_block_workspace_bytes(ctypes.byref(block), T, d, d_ff, E, k, dtype, g, d_ff_shared)
    if n == ctypes.c_size_t(-1).value:
        raise MoeError(MOE_ERR_UNSUPPORTED, "sizes outside the library's limits")
    return n


def mxfp8_h_layout(T, d, d_ff, E, k):
    """moe_ffn_mxfp8_h_layout: (codes byte offset, scales byte offset, row bytes) of the
    MXFP8 form of h in the workspace of an MXFP8-activation call."""
    co, so, rb = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_int(0)
    _check(load().moe_ffn_mxfp8_h_layout(T, d, d_ff, E, k, ctypes.byref(co), ctypes.byref(so), ctypes.byref(rb)))
    return co.value, so.value, rb.value


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _routing(T, k, E, device, want):
    if not want:
        return None, None
    r = {"topk_idx": torch.empty(T, k, dtype=torch.int32, device=device),
         "topk_w": torch.empty(T, k, dtype=torch.float32, device=device),
         "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=device),
         "sorted_pair": torch.empty(T * k, dtype=torch.int32, device=device)}
    s = RoutingOut(_ptr(r["topk_idx"]), _ptr(r["topk_w"]), _ptr(r["expert_offsets"]), _ptr(r["sorted_pair"]))
    return r, s


def _entry(name: str, block: Optional[MoeBlock]):
    """The plain entry point, or its moe_block_* twin with the block prepended."""
    L = load()
    if block is None:
        return getattr(L, name)
    f = getattr(L, name.replace("moe_ffn_", "moe_block_"))
    return lambda *args: f(ctypes.byref(block), *args)


def forward(x, router_w, router_b, w_gate, b_gate, w_up, b_up, w_down, b_down, k,
            alpha=1.702, limit=7.0, out=None, workspace=None, routing=False, stream=None, block=None):
    """moe_ffn_forward (moe_block_forward with `block`).  Shapes: x [T,d], router_w [E,d],
    w_gate/w_up [E,d_ff,d], w_down [E,d,d_ff], biases [E], [E,d_ff], [E,d] or None."""
    T, d = x.shape
    E, d_ff = w_gate.shape[0], w_gate.shape[1]
    dt = _dt(x)
    out = torch.empty_like(x) if out is None else out
    ws = workspace if workspace is not None else alloc_workspace(
        workspace_bytes(T, d, d_ff, E, k, dt, block=block), x.device)
    r, rs = _routing(T, k, E, x.device, routing)
    st = _entry("moe_ffn_forward", block)(
        _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(w_gate), _ptr(b_gate), _ptr(w_up), _ptr(b_up),
        _ptr(w_down), _ptr(b_down), T, d, d_ff, E, k, alpha, limit, _ptr(out), dt,
        _ptr(ws), ws.numel(), ctypes.byref(rs) if rs is not None else None, _stream(stream))
    _check(st)
    return (out, r) if routing else out


def forward_noalloc(x, router_w, router_b, w_gate, b_gate, w_up, b_up, w_down, b_down, k,
                    alpha=1.702, limit=7.0, out=None, routing=False, stream=None):
    """moe_ffn_forward_noalloc: moe_ffn_forward with the library's own scratch array as
    the workspace (no workspace argument)."""
    T, d = x.shape
    E, d_ff = w_gate.shape[0], w_gate.shape[1]
    out = torch.empty_like(x) if out is None else out
    r, rs = _routing(T, k, E, x.device, routing)
    st = load().moe_ffn_forward_noalloc(
        _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(w_gate), _ptr(b_gate), _ptr(w_up), _ptr(b_up),
        _ptr(w_down), _ptr(b_down), T, d, d_ff, E, k, alpha, limit, _ptr(out), _dt(x),
        ctypes.byref(rs) if rs is not None else None, _stream(stream))
    _check(st)
    return (out, r) if routing else out


def forward_mxfp4(x, router_w, router_b, w_gate_codes, w_gate_scales, b_gate, w_up_codes, w_up_scales,
                  b_up, w_down_codes, w_down_scales, b_down, k, alpha=1.702, limit=7.0, out=None,
                  workspace=None, routing=False, stream=None, block=None):
    """moe_ffn_forward_mxfp4 (moe_block_forward_mxfp4 with `block`).  codes uint8
    [E,rows,cols/2], scales uint8 [E,rows,cols/32]."""
    T, d = x.shape
    E, d_ff = w_gate_codes.shape[0], w_gate_codes.shape[1]
    out = torch.empty_like(x) if out is None else out
    ws = workspace if workspace is not None else alloc_workspace(
        workspace_bytes(T, d, d_ff, E, k, MOE_BF16, block=block), x.device)
    r, rs = _routing(T, k, E, x.device, routing)
    st = _entry("moe_ffn_forward_mxfp4", block)(
        _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(w_gate_codes), _ptr(w_gate_scales), _ptr(b_gate),
        _ptr(w_up_codes), _ptr(w_up_scales), _ptr(b_up), _ptr(w_down_codes), _ptr(w_down_scales), _ptr(b_down),
        T, d, d_ff, E, k, alpha, limit, _ptr(out), _ptr(ws), ws.numel(),
        ctypes.byref(rs) if rs is not None else None, _stream(stream))
    _check(st)
    return (out, r) if routing else out


def workspace_bytes_mxfp8(T, d, d_ff, E, k) -> int:
    n = load().moe_ffn_workspace_bytes_mxfp8(T, d, d_ff, E, k)
    if n == ctypes.c_size_t(-1).value:
        raise MoeError(MOE_ERR_UNSUPPORTED, "sizes outside the library's limits")
    return n


def forward_mxfp4_mxfp8(x, router_w, router_b, w_gate_codes, w_gate_scales, b_gate, w_up_codes, w_up_scales,
                        b_up, w_down_codes, w_down_scales, b_down, k, alpha=1.702, limit=7.0, out=None,
                        workspace=None, routing=False, stream=None, weights="mxfp4"):
    """moe_ffn_forward_mxfp4_mxfp8: the MXFP4 layer with MXFP8 activations on the
    scaled MFMA (weights="mxfp8": moe_ffn_forward_mxfp8_mxfp8, E4M3 weight codes
    [E, rows, cols]).  Arguments as forward_mxfp4 (no block form)."""
    T, d = x.shape
    E, d_ff = w_gate_codes.shape[0], w_gate_codes.shape[1]
    entry = {"mxfp4": "moe_ffn_forward_mxfp4_mxfp8", "mxfp8": "moe_ffn_forward_mxfp8_mxfp8"}[weights]
    out = torch.empty_like(x) if out is None else out
    ws = workspace if workspace is not None else alloc_workspace(
        workspace_bytes_mxfp8(T, d, d_ff, E, k), x.device)
    r, rs = _routing(T, k, E, x.device, routing)
    st = getattr(load(), entry)(
        _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(w_gate_codes), _ptr(w_gate_scales), _ptr(b_gate),
        _ptr(w_up_codes), _ptr(w_up_scales), _ptr(b_up), _ptr(w_down_codes), _ptr(w_down_scales), _ptr(b_down),
        T, d, d_ff, E, k, alpha, limit, _ptr(out), _ptr(ws), ws.numel(),
        ctypes.byref(rs) if rs is not None else None, _stream(stream))
    _check(st)
    return (out, r) if routing else out


def forward_nvfp4(x, router_w, router_b, w_gate_codes, w_gate_scales, w_gate_ts, b_gate, w_up_codes, w_up_scales,
                  w_up_ts, b_up, w_down_codes, w_down_scales, w_down_ts, b_down, k, alpha=1.702, limit=7.0, out=None,
                  workspace=None, routing=False, stream=None):
    """moe_ffn_forward_nvfp4: codes uint8 [E,rows,cols/2], E4M3 scales uint8 [E,rows,cols/16],
    float tensor scales."""
    T, d = x.shape
    E, d_ff = w_gate_codes.shape[0], w_gate_codes.shape[1]
    out = torch.empty_like(x) if out is None else out
    ws = workspace if workspace is not None else alloc_workspace(
        workspace_bytes(T, d, d_ff, E, k, MOE_BF16), x.device)
    r, rs = _routing(T, k, E, x.device, routing)
    st = load().moe_ffn_forward_nvfp4(
        _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(w_gate_codes), _ptr(w_gate_scales), float(w_gate_ts),
        _ptr(b_gate), _ptr(w_up_codes), _ptr(w_up_scales), float(w_up_ts), _ptr(b_up), _ptr(w_down_codes),
        _ptr(w_down_scales), float(w_down_ts), _ptr(b_down), T, d, d_ff, E, k, alpha, limit, _ptr(out), _ptr(ws),
        ws.numel(), ctypes.byref(rs) if rs is not None else None, _stream(stream))
    _check(st)
    return (out, r) if routing else out


def mxfp8_quantize(x, codes=None, scales=None, stream=None):
    """moe_mxfp8_quantize: bf16 [rows, cols] -> (E4M3 codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    rows, cols = x.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device) if scales is None else scales
    _check(load().moe_mxfp8_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def forward_grouped(x, router_w, router_b, w_gate, b_gate, w_up, b_up, w_down, b_down, k,
                    n_group, topk_group, norm_topk_prob, routed_scaling_factor,
                    score=MOE_SCORE_SOFTMAX, act=MOE_ACT_SILU, alpha=1.702, limit=7.0,
                    e_score_bias=None, shared_w_gate=None, shared_w_up=None, shared_w_down=None,
                    out=None, workspace=None, routing=False, stream=None, block=None):
    """moe_ffn_forward_grouped (moe_block_forward_grouped with `block`).  Shared expert
    weights [d_ff_shared, d] x2 and [d, d_ff_shared]."""
    T, d = x.shape
    E, d_ff = w_gate.shape[0], w_gate.shape[1]
    dt = _dt(x)
    Fs = shared_w_gate.shape[0] if shared_w_gate is not None else 0
    out = torch.empty_like(x) if out is None else out
    ws = workspace if workspace is not None else alloc_workspace(
        workspace_bytes(T, d, d_ff, E, k, dt, Fs, block=block, grouped=True), x.device)
    r, rs = _routing(T, k, E, x.device, routing)
    st = _entry("moe_ffn_forward_grouped", block)(
        _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(e_score_bias), _ptr(w_gate), _ptr(b_gate),
        _ptr(w_up), _ptr(b_up), _ptr(w_down), _ptr(b_down), _ptr(shared_w_gate), _ptr(shared_w_up),
        _ptr(shared_w_down), Fs, T, d, d_ff, E, k, n_group, topk_group, int(bool(norm_topk_prob)),
        routed_scaling_factor, score, act, alpha, limit, _ptr(out), dt, _ptr(ws), ws.numel(),
        ctypes.byref(rs) if rs is not None else None, _stream(stream))
    _check(st)
    return (out, r) if routing else out


def forward_grouped_affine(experts: AffineExperts, x, router_w, router_b, k, n_group, topk_group, norm_topk_prob,
                           routed_scaling_factor, d_ff, score=MOE_SCORE_SOFTMAX, act=MOE_ACT_SILU, alpha=1.702,
                           limit=7.0, e_score_bias=None, b_gate=None, b_up=None, b_down=None, shared_w_gate=None,
                           shared_w_up=None, shared_w_down=None, E=None, out=None, workspace=None, routing=False,
                           stream=None, block=None):
    """moe_block_forward_grouped_affine (block None: the plain layer).  `experts` from make_affine."""
    T, d = x.shape
    E = router_w.shape[0] if E is None else E
    Fs = shared_w_gate.shape[0] if shared_w_gate is not None else 0
    out = torch.empty_like(x) if out is None else out
    ws = workspace if workspace is not None else alloc_workspace(
        workspace_bytes(T, d, d_ff, E, k, MOE_BF16, Fs, block=block, grouped=True), x.device)
    r, rs = _routing(T, k, E, x.device, routing)
    st = load().moe_block_forward_grouped_affine(
        ctypes.byref(block) if block is not None else None, ctypes.byref(experts),
        _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(e_score_bias), _ptr(b_gate), _ptr(b_up), _ptr(b_down),
        _ptr(shared_w_gate), _ptr(shared_w_up), _ptr(shared_w_down), Fs, T, d, d_ff, E, k, n_group, topk_group,
        int(bool(norm_topk_prob)), routed_scaling_factor, score, act, alpha, limit, _ptr(out), _ptr(ws),
        ws.numel(), ctypes.byref(rs) if rs is not None else None, _stream(stream))
    _check(st)
    return (out, r) if routing else out


def profile_enable(stage_mask: int):
    _check(load().moe_ffn_profile_enable(stage_mask))


def profile_read():
    """Per stage: (summed milliseconds, number of timed launches) since the last read."""
    ms = (ctypes.c_double * 5)()
    n = (ctypes.c_int * 5)()
    _check(load().moe_ffn_profile_read(ms, n, 5))
    return {STAGES[i]: (ms[i], n[i]) for i in range(5)}


def bind(fn_name: str, *args, block: Optional[MoeBlock] = None):
    """Pre-marshal one call: returns a no-argument callable that invokes the
    named C entry point (its moe_block_* twin with `block`) with the given
    (already converted) arguments and raises on a non-zero status.  Used where
    Python overhead must stay out of a timed loop; the arguments must stay
    alive as long as the callable."""
    L = load()
    f = getattr(L, fn_name if block is None else fn_name.replace("moe_ffn_", "moe_block_"))
    conv = [a.data_ptr() if isinstance(a, torch.Tensor) else a for a in args]
    if block is not None:
        conv = [ctypes.byref(block)] + conv

    def call():
        st = f(*conv)
        if st != MOE_OK:
            _check(st)
    return call


def bound_layer_call(w, t: dict, out: torch.Tensor, workspace: torch.Tensor, stream=None,
                     routing: Optional[RoutingOut] = None):
    """bind() for a workload description `w` and its device tensors `t`
    (a block workload passes t["norm_w"] in a moe_block)."""
    s = _stream(stream)
    rp = ctypes.byref(routing) if routing is not None else None
    g = t.get
    blk = make_block(t["norm_w"], w.norm_eps, True) if getattr(w, "block", False) else None
    if w.weights in ("affine4", "affine8"):
        aff = make_affine(4 if w.weights == "affine4" else 8, t)
        Fs = g("shared_w_gate").shape[0] if g("shared_w_gate") is not None else 0
        L = load()
        args = [ctypes.byref(blk) if blk is not None else None, ctypes.byref(aff)] + [
            a.data_ptr() if isinstance(a, torch.Tensor) else a for a in (
                g("x"), g("router_w"), g("router_b"), None, g("b_gate"), g("b_up"), g("b_down"),
                g("shared_w_gate"), g("shared_w_up"), g("shared_w_down"), Fs, w.T, w.d, w.d_ff, w.E, w.k,
                w.n_group, w.topk_group, int(w.norm_topk_prob), w.routed_scaling_factor,
                MOE_SCORE_SOFTMAX if w.score == "softmax" else MOE_SCORE_SIGMOID,
                MOE_ACT_SILU if w.act == "silu" else MOE_ACT_CLIPPED_SWIGLU, w.alpha, w.limit, out, workspace,
                workspace.numel())] + [rp, s]
        keep = (aff, blk)

        def call():
            st = L.moe_block_forward_grouped_affine(*args)
            if st != MOE_OK:
                _check(st)
        call.keep = keep
        return call
    if w.routing == "grouped":
        Fs = g("shared_w_gate").shape[0] if g("shared_w_gate") is not None else 0
        return bind("moe_ffn_forward_grouped", g("x"), g("router_w"), g("router_b"), None, g("w_gate"),
                    g("b_gate"), g("w_up"), g("b_up"), g("w_down"), g("b_down"), g("shared_w_gate"),
                    g("shared_w_up"), g("shared_w_down"), Fs, w.T, w.d, w.d_ff, w.E, w.k, w.n_group,
                    w.topk_group, int(w.norm_topk_prob), w.routed_scaling_factor,
                    MOE_SCORE_SOFTMAX if w.score == "softmax" else MOE_SCORE_SIGMOID,
                    MOE_ACT_SILU if w.act == "silu" else MOE_ACT_CLIPPED_SWIGLU, w.alpha, w.limit,
                    out, MOE_F32 if w.dtype == "f32" else MOE_BF16, workspace, workspace.numel(), rp, s,
                    block=blk)
    if w.weights in ("mxfp4", "mxfp8") and getattr(w, "act_quant", None) == "mxfp8":
        return bind(f"moe_ffn_forward_{w.weights}_mxfp8", g("x"), g("router_w"), g("router_b"), g("w_gate_codes"),
                    g("w_gate_scales"), g("b_gate"), g("w_up_codes"), g("w_up_scales"), g("b_up"),
                    g("w_down_codes"), g("w_down_scales"), g("b_down"), w.T, w.d, w.d_ff, w.E, w.k,
                    w.alpha, w.limit, out, workspace, workspace.numel(), rp, s)
    if w.weights == "nvfp4":
        return bind("moe_ffn_forward_nvfp4", g("x"), g("router_w"), g("router_b"), g("w_gate_codes"),
                    g("w_gate_scales"), float(t["w_gate_tensor_scale"]), g("b_gate"), g("w_up_codes"),
                    g("w_up_scales"), float(t["w_up_tensor_scale"]), g("b_up"), g("w_down_codes"),
                    g("w_down_scales"), float(t["w_down_tensor_scale"]), g("b_down"), w.T, w.d, w.d_ff, w.E, w.k,
                    w.alpha, w.limit, out, workspace, workspace.numel(), rp, s)
    if w.weights == "mxfp4":
        return bind("moe_ffn_forward_mxfp4", g("x"), g("router_w"), g("router_b"), g("w_gate_codes"),
                    g("w_gate_scales"), g("b_gate"), g("w_up_codes"), g("w_up_scales"), g("b_up"),
                    g("w_down_codes"), g("w_down_scales"), g("b_down"), w.T, w.d, w.d_ff, w.E, w.k,
                    w.alpha, w.limit, out, workspace, workspace.numel(), rp, s, block=blk)
    return bind("moe_ffn_forward", g("x"), g("router_w"), g("router_b"), g("w_gate"), g("b_gate"),
                g("w_up"), g("b_up"), g("w_down"), g("b_down"), w.T, w.d, w.d_ff, w.E, w.k, w.alpha,
                w.limit, out, MOE_F32 if w.dtype == "f32" else MOE_BF16, workspace, workspace.numel(), rp, s,
                block=blk)
