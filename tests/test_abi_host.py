"""The C ABI on the host: the library loads, exports every function that
include/moe_ffn.h declares, and rejects every invalid argument before any HIP
call (the device pointers below are never dereferenced).  CPU only."""
import ctypes
import os
import re

import pytest

from mixture_experts_transformer_router_amd import moe_ffn as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")

FAKE = 0x7f0000000000  # 256-aligned, never dereferenced
FAKE2 = 0x7f1000000000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.lib_path()):
        from mixture_experts_transformer_router_amd import build
        build.build()
    return M.load()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert len(declared) >= 8, declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in moe_ffn.h but not exported"
    assert sorted(declared) == sorted(M.EXPORTED)


def test_status_strings(lib):
    for s, n in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_UNSUPPORTED"),
                 (3, "MOE_ERR_WORKSPACE"), (4, "MOE_ERR_HIP")]:
        assert lib.moe_status_string(s).decode() == n


def test_workspace_bytes(lib):
    n = lib.moe_ffn_workspace_bytes
    assert n(0, 2880, 2880, 32, 4, M.MOE_BF16, 0, 0) == 0
    big = n(8192, 2880, 2880, 32, 4, M.MOE_BF16, 0, 0)
    P = 8192 * 4
    assert big >= 2 * P * 2880 * 2          # hidden activations + expert outputs (bf16)
    assert big < 2 * P * 2880 * 2 + (8 << 20)
    assert n(64, 64, 64, 8, 2, M.MOE_F32, 0, 0) > n(64, 64, 64, 8, 2, M.MOE_BF16, 0, 0)
    # bf16 with T <= 16 also holds the router's 16 partial-logit slices [16][16][E] fp32
    assert n(1, 64, 64, 8, 2, M.MOE_BF16, 0, 0) >= 16 * 16 * 8 * 4 + 2 * (64 + 64) * 2
    assert n(2048, 2048, 1536, 64, 6, M.MOE_BF16, 1, 1536) > n(2048, 2048, 1536, 64, 6, M.MOE_BF16, 1, 0)
    bad = ctypes.c_size_t(-1).value
    assert n(8, 64, 64, 300, 2, M.MOE_BF16, 0, 0) == bad
    assert n(8, 64, 64, 8, 9, M.MOE_BF16, 0, 0) == bad
    assert n(-1, 64, 64, 8, 2, M.MOE_BF16, 0, 0) == bad
    # only a group-routed layer has a shared expert; without one the routing kind does not change the size
    assert n(64, 64, 64, 8, 2, M.MOE_BF16, 0, 64) == bad
    assert n(64, 64, 64, 8, 2, M.MOE_BF16, 1, 0) == n(64, 64, 64, 8, 2, M.MOE_BF16, 0, 0)
    assert n(64, 64, 64, 8, 2, M.MOE_BF16, 1, 64) > n(64, 64, 64, 8, 2, M.MOE_BF16, 1, 0)


def test_mxfp8_h_layout(lib):
    # the MXFP8 codes and scales of h lie inside the workspace, after the bf16 h and y rows
    T, d, F, E, k = 4096, 2880, 2880, 32, 4
    co, so, rb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int()
    assert lib.moe_ffn_mxfp8_h_layout(T, d, F, E, k, ctypes.byref(co), ctypes.byref(so), ctypes.byref(rb)) == M.MOE_OK
    total = lib.moe_ffn_workspace_bytes_mxfp8(T, d, F, E, k)
    assert rb.value == 2944                             # whole 128-element stages
    assert co.value % 256 == 0 and so.value % 256 == 0
    assert co.value >= 2 * T * k * F * 2                # past h and y (bf16)
    assert co.value + T * k * rb.value <= so.value
    assert so.value + T * k * rb.value // 32 <= total
    assert lib.moe_ffn_mxfp8_h_layout(0, d, F, E, k, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_ffn_mxfp8_h_layout(T, d, F, 300, k, None, None, None) == M.MOE_ERR_INVALID_ARG


def _fwd(lib, T=16, d=64, F=64, E=8, k=2, alpha=1.702, limit=7.0, dt=M.MOE_BF16, x=FAKE, wr=FAKE,
         wg=FAKE, wu=FAKE, wd=FAKE, out=FAKE2, ws=None, wsb=None):
    need = lib.moe_ffn_workspace_bytes(max(T, 0), d, F, E, min(k, 16) if k > 0 else 1, dt, 0, 0)
    if ws is None:
        ws = FAKE + (1 << 36)
    if wsb is None:
        wsb = need if need != ctypes.c_size_t(-1).value else 0
    return lib.moe_ffn_forward(x, wr, None, wg, None, wu, None, wd, None, T, d, F, E, k, alpha, limit,
                               out, dt, ws, wsb, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), M.MOE_ERR_INVALID_ARG),
    (dict(k=0), M.MOE_ERR_INVALID_ARG),
    (dict(T=-1), M.MOE_ERR_INVALID_ARG),
    (dict(d=0), M.MOE_ERR_INVALID_ARG),
    (dict(E=0, k=1), M.MOE_ERR_INVALID_ARG),
    (dict(E=300, k=2), M.MOE_ERR_UNSUPPORTED),
    (dict(E=32, k=17), M.MOE_ERR_UNSUPPORTED),
    (dict(d=100), M.MOE_ERR_UNSUPPORTED),
    (dict(F=36), M.MOE_ERR_UNSUPPORTED),
    (dict(limit=0.0), M.MOE_ERR_INVALID_ARG),
    (dict(limit=float("nan")), M.MOE_ERR_INVALID_ARG),
    (dict(alpha=float("inf")), M.MOE_ERR_INVALID_ARG),
    (dict(x=None), M.MOE_ERR_INVALID_ARG),
    (dict(wr=None), M.MOE_ERR_INVALID_ARG),
    (dict(wg=None), M.MOE_ERR_INVALID_ARG),
    (dict(wd=None), M.MOE_ERR_INVALID_ARG),
    (dict(out=None), M.MOE_ERR_INVALID_ARG),
    (dict(dt=7), M.MOE_ERR_INVALID_ARG),
    (dict(out=FAKE), M.MOE_ERR_INVALID_ARG),                       # out aliases x
    (dict(x=FAKE + 8), M.MOE_ERR_INVALID_ARG),                     # 16-byte vector loads
    (dict(wr=FAKE + 4), M.MOE_ERR_INVALID_ARG),
    (dict(wd=FAKE + 2), M.MOE_ERR_INVALID_ARG),
    (dict(out=FAKE2 + 1), M.MOE_ERR_INVALID_ARG),                  # bf16 elements
    (dict(ws=0), M.MOE_ERR_WORKSPACE),
    (dict(wsb=1024), M.MOE_ERR_WORKSPACE),
    (dict(ws=FAKE + (1 << 36) + 64), M.MOE_ERR_WORKSPACE),          # misaligned
    (dict(out=FAKE + (1 << 36) + 512), M.MOE_ERR_INVALID_ARG),      # out inside the workspace
    (dict(T=0), M.MOE_OK),
    (dict(T=0, x=None, out=None, ws=0, wsb=0), M.MOE_OK),
])
def test_forward_argument_checks(lib, kw, status):
    st = _fwd(lib, **kw)
    assert st == status, (st, lib.moe_last_error_detail().decode())
    if status != M.MOE_OK:
        assert len(lib.moe_last_error_detail()) > 0
    else:
        assert lib.moe_last_error_detail() == b""


def _grouped(lib, E=64, k=6, ng=8, tg=4, shared=(None, None, None), Fs=0, score=0, act=1, T=16, d=64, F=64):
    need = lib.moe_ffn_workspace_bytes(T, d, F, E, min(k, 16), M.MOE_BF16, 1, Fs)
    return lib.moe_ffn_forward_grouped(FAKE, FAKE, None, None, FAKE, None, FAKE, None, FAKE, None,
                                       shared[0], shared[1], shared[2], Fs, T, d, F, E, k, ng, tg, 1, 1.8,
                                       score, act, 1.702, 7.0, FAKE2, M.MOE_BF16, FAKE + (1 << 36), need,
                                       None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ng=7), M.MOE_ERR_INVALID_ARG),                  # E % n_group != 0
    (dict(ng=0), M.MOE_ERR_INVALID_ARG),
    (dict(tg=9), M.MOE_ERR_INVALID_ARG),                  # topk_group > n_group
    (dict(tg=0), M.MOE_ERR_INVALID_ARG),
    (dict(tg=1, k=9), M.MOE_ERR_INVALID_ARG),             # k > topk_group * E / n_group
    (dict(E=256, ng=128, tg=4, k=6), M.MOE_ERR_UNSUPPORTED),
    (dict(score=5), M.MOE_ERR_INVALID_ARG),
    (dict(act=3), M.MOE_ERR_INVALID_ARG),
    (dict(shared=(FAKE, None, FAKE), Fs=64), M.MOE_ERR_INVALID_ARG),
    (dict(shared=(FAKE, FAKE, FAKE), Fs=12), M.MOE_ERR_INVALID_ARG),
    (dict(shared=(FAKE, FAKE, FAKE), Fs=0), M.MOE_ERR_INVALID_ARG),
])
def test_grouped_argument_checks(lib, kw, status):
    st = _grouped(lib, **kw)
    assert st == status, (st, lib.moe_last_error_detail().decode())


def test_mxfp4_argument_checks(lib):
    def call(d=64, F=64, codes=FAKE):
        need = lib.moe_ffn_workspace_bytes(16, d, F, 8, 2, M.MOE_BF16, 0, 0)
        return lib.moe_ffn_forward_mxfp4(FAKE, FAKE, None, codes, FAKE, None, FAKE, FAKE, None, FAKE, FAKE,
                                         None, 16, d, F, 8, 2, 1.702, 7.0, FAKE2, FAKE + (1 << 36), need,
                                         None, None)
    assert call(d=48) == M.MOE_ERR_UNSUPPORTED
    assert call(F=40) == M.MOE_ERR_UNSUPPORTED
    assert call(codes=None) == M.MOE_ERR_INVALID_ARG
    assert call(codes=FAKE + 8) == M.MOE_ERR_INVALID_ARG
    assert b"16-byte" in lib.moe_last_error_detail()
    # one expert's codes must stay under 2^32 bytes (32-bit offsets in the kernels)
    assert call(d=65536, F=131072) == M.MOE_ERR_UNSUPPORTED
    assert b"2^32" in lib.moe_last_error_detail()

def test_block_workspace_and_argument_checks(lib):
    n = lib.moe_ffn_workspace_bytes
    nb = lib.moe_block_workspace_bytes
    with_norm = M.MoeBlock(FAKE, 1e-5, 1)
    residual_only = M.MoeBlock(None, 0.0, 1)
    assert nb(None, 64, 256, 128, 8, 2, M.MOE_BF16, 0, 0) == n(64, 256, 128, 8, 2, M.MOE_BF16, 0, 0)
    assert nb(ctypes.byref(residual_only), 64, 256, 128, 8, 2, M.MOE_BF16, 0, 0) == n(64, 256, 128, 8, 2, M.MOE_BF16, 0, 0)
    # the normalised rows: T * d elements more
    assert nb(ctypes.byref(with_norm), 64, 256, 128, 8, 2, M.MOE_BF16, 0, 0) >= n(64, 256, 128, 8, 2, M.MOE_BF16, 0, 0) + 64 * 256 * 2

    def call(block, wsb=None):
        need = nb(ctypes.byref(block), 16, 64, 64, 8, 2, M.MOE_BF16, 0, 0)
        return lib.moe_block_forward(ctypes.byref(block), FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None,
                                     16, 64, 64, 8, 2, 1.702, 7.0, FAKE2, M.MOE_BF16, FAKE + (1 << 36),
                                     need if wsb is None else wsb, None, None)
    assert call(M.MoeBlock(FAKE, -1e-5, 1)) == M.MOE_ERR_INVALID_ARG
    assert b"eps" in lib.moe_last_error_detail()
    assert call(M.MoeBlock(FAKE, float("nan"), 0)) == M.MOE_ERR_INVALID_ARG
    assert call(M.MoeBlock(FAKE, float("inf"), 0)) == M.MOE_ERR_INVALID_ARG
    # the bf16 router reads the norm weight with 16-byte loads
    assert call(M.MoeBlock(FAKE + 2, 1e-5, 1)) == M.MOE_ERR_INVALID_ARG
    assert b"16-byte" in lib.moe_last_error_detail()
    # a workspace sized for the plain layer is too small once the norm needs its rows
    plain = n(16, 64, 64, 8, 2, M.MOE_BF16, 0, 0)
    assert call(M.MoeBlock(FAKE, 1e-5, 1), wsb=plain) == M.MOE_ERR_WORKSPACE
    # T = 0 is a no-op for blocks too
    assert lib.moe_block_forward(ctypes.byref(with_norm), None, None, None, None, None, None, None, None, None,
                                 0, 64, 64, 8, 2, 1.702, 7.0, None, M.MOE_BF16, 0, 0, None, None) == M.MOE_OK


def test_affine_argument_checks(lib):
    def call(bits=4, d=128, F=64, drop=None, experts=True):
        ex = M.AffineExperts(bits, *[FAKE] * 9)
        if drop:
            setattr(ex, drop, None)
        need = lib.moe_ffn_workspace_bytes(16, d, F, 8, 2, M.MOE_BF16, 0, 0)
        return lib.moe_block_forward_grouped_affine(
            None, ctypes.byref(ex) if experts else None, FAKE, FAKE, None, None, None, None, None, None, None,
            None, 0, 16, d, F, 8, 2, 2, 1, 1, 1.0, 0, 1, 1.702, 7.0, FAKE2, FAKE + (1 << 36), need, None, None)
    assert call(experts=False) == M.MOE_ERR_INVALID_ARG
    assert call(bits=5) == M.MOE_ERR_UNSUPPORTED
    assert call(bits=8, d=96) == M.MOE_ERR_UNSUPPORTED       # 8-bit groups of 64
    assert call(bits=4, F=48) == M.MOE_ERR_UNSUPPORTED       # 4-bit groups of 32
    assert call(drop="down_biases") == M.MOE_ERR_INVALID_ARG
    assert b"biases" in lib.moe_last_error_detail()
    assert call(drop="up_q") == M.MOE_ERR_INVALID_ARG


def test_mxfp8_activation_workspace_and_argument_checks(lib):
    nw = lib.moe_ffn_workspace_bytes_mxfp8
    plain = lib.moe_ffn_workspace_bytes(4096, 2880, 2880, 32, 4, M.MOE_BF16, 0, 0)
    need = nw(4096, 2880, 2880, 32, 4)
    # x and h as codes (rows padded to 128 bytes) plus a scale byte per 32
    assert need >= plain + (4096 + 4096 * 4) * 2944 * 33 // 32
    assert nw(0, 64, 64, 8, 2) == 0
    assert nw(8, 64, 64, 300, 2) == ctypes.c_size_t(-1).value

    def call(d=128, F=128, T=16, x=FAKE, scales=FAKE, wsb=None):
        n = nw(T, d, F, 8, 2)
        return lib.moe_ffn_forward_mxfp4_mxfp8(x, FAKE, None, FAKE, scales, None, FAKE, FAKE, None, FAKE, FAKE,
                                               None, T, d, F, 8, 2, 1.702, 7.0, FAKE2, FAKE + (1 << 36),
                                               n if wsb is None else wsb, None, None)
    assert call(d=96) == M.MOE_ERR_UNSUPPORTED                 # whole 64-k MFMA steps
    assert b"64" in lib.moe_last_error_detail()
    assert call(F=160) == M.MOE_ERR_UNSUPPORTED
    assert call(scales=FAKE + 2) == M.MOE_ERR_INVALID_ARG      # 4-byte aligned scale tensors
    assert call(x=FAKE + 8) == M.MOE_ERR_INVALID_ARG           # 16-byte aligned x
    # the MXFP4 layer's workspace is too small for the MXFP8 copies
    assert call(wsb=lib.moe_ffn_workspace_bytes(16, 128, 128, 8, 2, M.MOE_BF16, 0, 0)) == M.MOE_ERR_WORKSPACE
    assert call(T=0) == M.MOE_OK
    # MXFP8 weights: the same checks
    n = nw(16, 96, 128, 8, 2)
    assert lib.moe_ffn_forward_mxfp8_mxfp8(FAKE, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None,
                                           16, 96, 128, 8, 2, 1.702, 7.0, FAKE2, FAKE + (1 << 36), n,
                                           None, None) == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_ffn_forward_mxfp8_mxfp8(FAKE, FAKE, None, None, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None,
                                           16, 128, 128, 8, 2, 1.702, 7.0, FAKE2, FAKE + (1 << 36),
                                           nw(16, 128, 128, 8, 2), None, None) == M.MOE_ERR_INVALID_ARG


def test_mxfp8_quantize_argument_checks(lib):
    q = lib.moe_mxfp8_quantize
    assert q(FAKE, 4, 48, FAKE2, FAKE2 + (1 << 30), None) == M.MOE_ERR_INVALID_ARG      # cols % 32
    assert q(FAKE, -1, 64, FAKE2, FAKE2 + (1 << 30), None) == M.MOE_ERR_INVALID_ARG
    assert q(None, 4, 64, FAKE2, FAKE2 + (1 << 30), None) == M.MOE_ERR_INVALID_ARG
    assert q(FAKE + 8, 4, 64, FAKE2, FAKE2 + (1 << 30), None) == M.MOE_ERR_INVALID_ARG  # alignment
    assert q(FAKE, 4, 64, FAKE + 64, FAKE2, None) == M.MOE_ERR_INVALID_ARG              # codes overlap x
    assert q(None, 0, 64, None, None, None) == M.MOE_OK
    assert q(FAKE, 1 << 20, 1 << 20, FAKE2, FAKE2 + (1 << 44), None) == M.MOE_ERR_UNSUPPORTED



def test_nvfp4_argument_checks(lib):
    def call(d=128, F=128, ts=1.0, codes=FAKE):
        n = lib.moe_ffn_workspace_bytes(16, d, F, 8, 2, M.MOE_BF16, 0, 0)
        return lib.moe_ffn_forward_nvfp4(FAKE, FAKE, None, codes, FAKE, ts, None, FAKE, FAKE, 1.0, None, FAKE, FAKE,
                                         1.0, None, 16, d, F, 8, 2, 1.702, 7.0, FAKE2, FAKE + (1 << 36), n, None, None)
    assert call(ts=float("nan")) == M.MOE_ERR_INVALID_ARG
    assert b"tensor scale" in lib.moe_last_error_detail()
    assert call(ts=float("inf")) == M.MOE_ERR_INVALID_ARG
    assert call(d=48) == M.MOE_ERR_UNSUPPORTED
    assert call(codes=None) == M.MOE_ERR_INVALID_ARG
