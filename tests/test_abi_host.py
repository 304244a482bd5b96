"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

The library loads, exports every function include/moe_latent.h declares, and
rejects bad arguments with the documented codes before touching the device.
"""
import ctypes
import os
import re
import subprocess

import pytest

import synth
from mxfp4_latent_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_latent.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails before any device work


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    return _lib.load()


def test_header_declares_the_five_calls():
    names = _declared()
    for fn in ("moe_route", "moe_permute", "mxfp4_grouped_gemm", "moe_combine_norm_up",
               "shared_expert_ffn", "moe_workspace_bytes", "moe_strerror", "moe_abi_version"):
        assert fn in names
    assert set(names) == set(_lib.EXPORTS)


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for fn in _declared():
        assert fn in exported, fn
        assert hasattr(lib, fn)
    assert lib.moe_abi_version() == 2
    assert b"workspace" in lib.moe_strerror(_lib.MOE_EWORKSPACE)


def _shape(**kw):
    sh = synth.K3_SHAPE
    s = _lib.make_shape(sh.hidden, sh.latent, sh.n_experts, sh.top_k, sh.inter, sh.n_shared, sh.shared_inter)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_workspace_bytes(lib):
    s = _shape()
    for fn in range(8):
        assert lib.moe_workspace_bytes(s, fn, 16) > 0
    assert lib.moe_workspace_bytes(s, 8, 16) == 0
    # the fused combine needs the combine's workspace plus one fp32 per pair
    assert (lib.moe_workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP_REAP, 16)
            >= lib.moe_workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP, 16) + 16 * s.top_k * 4)
    assert lib.moe_workspace_bytes(s, 0, 0) == 0
    bad = _shape(latent=100)
    assert lib.moe_workspace_bytes(bad, 0, 16) == 0
    # grows with the token count
    assert lib.moe_workspace_bytes(s, _lib.MOE_FN_ROUTE, 4096) > lib.moe_workspace_bytes(s, _lib.MOE_FN_ROUTE, 16)


def test_route_validation(lib):
    s = _shape()
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_ROUTE, 16)
    args = [16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]
    bad_T = list(args)
    bad_T[0] = 0
    assert lib.moe_route(s, *bad_T) == _lib.MOE_EINVAL
    nul = list(args)
    nul[1] = None
    assert lib.moe_route(s, *nul) == _lib.MOE_EINVAL
    half = list(args)
    half[4] = None  # w_down without z is an error (and the reverse)
    assert lib.moe_route(s, *half) == _lib.MOE_EINVAL
    mis = list(args)
    mis[1] = FAKE + 2
    assert lib.moe_route(s, *mis) == _lib.MOE_EINVAL
    small = list(args)
    small[10] = ws - 1
    assert lib.moe_route(s, *small) == _lib.MOE_EWORKSPACE
    no_router = list(args)
    no_router[2] = None  # z only: bias, ids, weights and gap must be NULL too
    assert lib.moe_route(s, *no_router) == _lib.MOE_EINVAL
    z_only = [16, FAKE, None, None, FAKE, None, None, FAKE, None, FAKE, ws, None]
    bad_z_only = list(z_only)
    bad_z_only[4] = None
    bad_z_only[7] = None
    assert lib.moe_route(s, *bad_z_only) == _lib.MOE_EINVAL  # neither routing nor z
    assert lib.moe_route(s, *z_only[:10], ws - 1, None) == _lib.MOE_EWORKSPACE
    assert lib.moe_route(None, *args) == _lib.MOE_EINVAL
    assert lib.moe_route(_shape(operand_mode=7), *args) == _lib.MOE_EINVAL
    assert lib.moe_route(_shape(top_k=900), *args) == _lib.MOE_EINVAL
    assert lib.moe_route(_shape(n_experts=2048, top_k=16), *args) == _lib.MOE_ENOTSUP
    assert lib.moe_route(_shape(hidden=7000), *args) == _lib.MOE_ENOTSUP
    assert lib.moe_route(_shape(top_k=33), *args) == _lib.MOE_ENOTSUP


def test_permute_validation(lib):
    s = _shape()
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_PERMUTE, 16)
    assert lib.moe_permute(s, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == _lib.MOE_EINVAL
    assert lib.moe_permute(s, 16, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == _lib.MOE_EINVAL
    assert lib.moe_permute(s, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == _lib.MOE_EWORKSPACE


def test_grouped_gemm_validation(lib):
    s = _shape()
    P = 256
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_GROUPED_GEMM, P)
    G, D = _lib.MOE_OP_GATEUP_SITU, _lib.MOE_OP_DOWN
    f32 = _lib.MOE_DT_F32

    def call(op=G, P_=P, off=FAKE, sp=FAKE, A=FAKE, ar=P // 16, dt=f32, wp=FAKE, wsc=FAKE, w3p=FAKE, w3s=FAKE,
             pw=None, C=FAKE, wsb=ws):
        return lib.mxfp4_grouped_gemm(s, op, P_, off, sp, A, ar, dt, wp, wsc, w3p, w3s, pw, C, FAKE, wsb, None)

    assert call(op=5) == _lib.MOE_EINVAL
    assert call(dt=9) == _lib.MOE_EINVAL
    assert call(P_=0) == _lib.MOE_EINVAL
    assert call(w3p=None) == _lib.MOE_EINVAL           # gate/up needs w3
    assert call(op=D) == _lib.MOE_EINVAL               # down must not get w3
    assert call(op=D, w3p=None, w3s=None, pw=FAKE, sp=None) == _lib.MOE_EINVAL  # weights need sorted_pair
    assert call(pw=FAKE) == _lib.MOE_EINVAL            # no pair weights on gate/up
    assert call(A=FAKE + 4) == _lib.MOE_EINVAL
    assert call(wsc=FAKE + 1) == _lib.MOE_EINVAL
    assert call(wsb=ws - 1) == _lib.MOE_EWORKSPACE
    assert call(op=D, w3p=None, w3s=None, ar=P, wsb=16) == _lib.MOE_EWORKSPACE
    # rows of A: at least one; at least P when A holds the sorted rows itself
    assert call(ar=0) == _lib.MOE_EINVAL
    assert call(sp=None, ar=P - 1) == _lib.MOE_EINVAL
    assert call(op=D, w3p=None, w3s=None, ar=P - 1) == _lib.MOE_EINVAL
    # gathered rows are addressed with 32-bit offsets: A below 2^31 bytes
    lat = s.latent
    big = -(-(1 << 31) // (lat * 4))  # smallest row count with 2^31 bytes or more
    assert call(ar=big) == _lib.MOE_ENOTSUP
    assert call(ar=big - 1, wsb=ws - 1) == _lib.MOE_EWORKSPACE
    # H as bf16 planes: planes input only for down; both forms only on the
    # tiled path without the small-expert split (P >= 8 E) in bf16 operand modes
    GP, BP = _lib.MOE_OP_GATEUP_SITU_BF16X2, _lib.MOE_DT_BF16X2
    assert call(dt=BP) == _lib.MOE_EINVAL
    assert call(op=GP) == _lib.MOE_ENOTSUP                                   # P = 256: decode sizes
    assert call(op=D, w3p=None, w3s=None, ar=P, dt=BP) == _lib.MOE_ENOTSUP
    Pb = 8 * s.n_experts
    wsb_big = lib.moe_workspace_bytes(s, _lib.MOE_FN_GROUPED_GEMM, Pb)
    assert call(op=GP, P_=Pb, wsb=wsb_big - 1) == _lib.MOE_EWORKSPACE      # accepted up to the workspace check
    mx6 = _shape(operand_mode=_lib.MOE_OPND_MX6X3)
    assert lib.mxfp4_grouped_gemm(mx6, GP, Pb, FAKE, FAKE, FAKE, Pb // 16, f32, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                  FAKE, wsb_big, None) == _lib.MOE_ENOTSUP


def test_combine_and_shared_validation(lib):
    s = _shape()
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP, 16)
    assert lib.moe_combine_norm_up(s, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, ws, None) == _lib.MOE_EINVAL
    assert lib.moe_combine_norm_up(s, 16, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ws, None) == _lib.MOE_EINVAL
    assert lib.moe_combine_norm_up(s, 16, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, ws - 1, None) == _lib.MOE_EWORKSPACE
    ws2 = lib.moe_workspace_bytes(s, _lib.MOE_FN_SHARED_FFN, 16)
    assert lib.shared_expert_ffn(s, 16, FAKE, FAKE, FAKE, None, FAKE, 0, FAKE, ws2, None) == _lib.MOE_EINVAL
    assert lib.shared_expert_ffn(s, -1, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ws2, None) == _lib.MOE_EINVAL
    assert lib.shared_expert_ffn(s, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ws2 - 1, None) == _lib.MOE_EWORKSPACE
    none = _shape(n_shared=0)
    assert lib.shared_expert_ffn(none, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ws2, None) == _lib.MOE_EINVAL


def test_no_cpu_fallback_when_library_missing(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load(str(tmp_path / "missing.so"))


def test_reap_saliency_validation(lib):
    s = _shape()
    P = 256
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_REAP_SALIENCY, P)
    assert ws >= P * 4
    args = [P, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ws, None]
    assert lib.moe_reap_saliency(s, -1, *args[1:]) == _lib.MOE_EINVAL
    for i in (1, 2, 5, 6):  # offsets, Y, sal_sum, counts
        a = list(args)
        a[i] = None
        assert lib.moe_reap_saliency(s, *a) == _lib.MOE_EINVAL, i
    for i in (3, 4):  # only one of pair_weight / sorted_pair
        a = list(args)
        a[i] = None
        assert lib.moe_reap_saliency(s, *a) == _lib.MOE_EINVAL, i
    a = list(args)
    a[7] = 2
    assert lib.moe_reap_saliency(s, *a) == _lib.MOE_EINVAL
    a = list(args)
    a[2] = FAKE + 4
    assert lib.moe_reap_saliency(s, *a) == _lib.MOE_EINVAL
    a = list(args)
    a[9] = ws - 1
    assert lib.moe_reap_saliency(s, *a) == _lib.MOE_EWORKSPACE


def test_combine_reap_validation(lib):
    s = _shape()
    T = 16
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP_REAP, T)
    # T, Y, pair_pos, topk_w, gamma, w_up, out, accumulate, offsets, sal_sum, counts, reap_accumulate, ws, bytes
    args = [T, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 0, FAKE, ws, None]
    for i in (8, 9, 10):  # offsets, sal_sum, counts
        a = list(args)
        a[i] = None
        assert lib.moe_combine_norm_up_reap(s, *a) == _lib.MOE_EINVAL, i
    for i, v in ((7, 2), (11, 2), (0, 0)):  # accumulate, reap_accumulate, T
        a = list(args)
        a[i] = v
        assert lib.moe_combine_norm_up_reap(s, *a) == _lib.MOE_EINVAL, i
    a = list(args)
    a[13] = lib.moe_workspace_bytes(s, _lib.MOE_FN_COMBINE_NORM_UP, T)  # the plain combine's is too small
    assert lib.moe_combine_norm_up_reap(s, *a) == _lib.MOE_EWORKSPACE
    wide = _shape(latent=4224)  # a whole row per pass: latent <= 4096
    a = list(args)
    a[13] = lib.moe_workspace_bytes(wide, _lib.MOE_FN_COMBINE_NORM_UP_REAP, T)
    assert lib.moe_combine_norm_up_reap(wide, *a) == _lib.MOE_ENOTSUP


def test_route_capped_validation(lib):
    s = _shape()
    T = 16
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_ROUTE, T)
    # T, x, w_router, bias, w_down, promoted, k_hi, ids, w, z, gap, ws, bytes, stream
    args = [T, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]
    for i, v in ((5, None), (2, None), (6, -1), (0, 0), (3, None)):  # promoted, router, k_hi, T, bias
        a = list(args)
        a[i] = v
        assert lib.moe_route_capped(s, *a) == _lib.MOE_EINVAL, i
    a = list(args)
    a[12] = ws - 1
    assert lib.moe_route_capped(s, *a) == _lib.MOE_EWORKSPACE


def test_route_noalloc_validation(lib):
    """Sizes past the fixed scratch are rejected before any device work."""
    s = _shape()
    assert lib.moe_workspace_bytes(s, _lib.MOE_FN_ROUTE, 64) <= _lib.MOE_ROUTE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_workspace_bytes(s, _lib.MOE_FN_ROUTE, 65) > _lib.MOE_ROUTE_NOALLOC_SCRATCH_BYTES
    args = (FAKE,) * 9 + (None,)
    assert lib.moe_route_noalloc(s, 65, *args) == _lib.MOE_EWORKSPACE
    assert lib.moe_route_noalloc(s, 0, *args) == _lib.MOE_EINVAL
    assert lib.moe_route_noalloc(None, 16, *args) == _lib.MOE_EINVAL


def test_two_bank_validation(lib):
    """The two-bank call checks banks, formats, expert counts and limits before any device work."""
    s = _shape()
    P = 256
    ws = lib.moe_workspace_bytes(s, _lib.MOE_FN_GROUPED_GEMM_TWO_BANK, P)
    assert ws >= lib.moe_workspace_bytes(s, _lib.MOE_FN_GROUPED_GEMM, P)
    G, D = _lib.MOE_OP_GATEUP_SITU, _lib.MOE_OP_DOWN
    f32 = _lib.MOE_DT_F32

    def bank(fmt, n, op=G, bias=True, up=True):
        b = _lib.MoeExpertBank()
        b.format, b.n_experts = fmt, n
        b.packed, b.scale = FAKE, FAKE
        aff = fmt == _lib.MOE_WF_AFFINE2
        b.bias = FAKE if (aff and bias) else None
        if op == G and up:
            b.packed3, b.scale3 = FAKE, FAKE
            b.bias3 = FAKE if (aff and bias) else None
        return b

    def call(ba, bb, op=G, sp=FAKE, ar=P // 16, wsb=ws, shape=s):
        return lib.moe_grouped_gemm_two_bank(shape, op, P, FAKE, sp, FAKE, ar, f32, ctypes.byref(ba),
                                             ctypes.byref(bb), None, FAKE, FAKE, wsb, None)

    M, A2 = _lib.MOE_WF_MXFP4, _lib.MOE_WF_AFFINE2
    assert call(bank(M, 500), bank(A2, 395)) == _lib.MOE_EINVAL          # 895 != 896 experts
    assert call(bank(M, 500), bank(7, 396)) == _lib.MOE_EINVAL           # unknown format
    assert call(bank(M, 500), bank(A2, 396, bias=False)) == _lib.MOE_EINVAL  # affine needs biases
    assert call(bank(M, 500), bank(A2, 396, up=False)) == _lib.MOE_EINVAL    # gate/up needs the up bank
    assert call(bank(M, 500, op=D), bank(A2, 396, op=G), op=D) == _lib.MOE_EINVAL  # down takes no up tensors
    assert call(bank(M, 500), bank(A2, 396), wsb=ws - 1) == _lib.MOE_EWORKSPACE
    assert call(bank(M, 896), bank(A2, 0), wsb=ws - 1) == _lib.MOE_EWORKSPACE   # an empty bank is fine
    mx = _shape(operand_mode=_lib.MOE_OPND_MX6X3)
    assert call(bank(M, 500), bank(A2, 396), shape=mx) == _lib.MOE_ENOTSUP  # bf16 operand modes only
    small_k = _shape(latent=1152, hidden=1152)  # 1152 is not a multiple of 512
    assert call(bank(M, 500), bank(A2, 396), shape=small_k) == _lib.MOE_ENOTSUP
