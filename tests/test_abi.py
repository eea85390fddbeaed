"""CPU-only checks of the C ABI: the library loads, exports every function declared in
include/atma.h, sizes its workspaces, and rejects bad arguments on the host before
launching anything (these calls never reach a kernel, so no GPU is needed)."""
import ctypes

import pytest

g = pytest.importorskip("gated_delta_memory_amd")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
NULL = None


def test_every_declared_symbol_is_exported():
    names = g.header_functions()
    assert len(names) >= 9
    missing = [n for n in names if not hasattr(g.lib, n)]
    assert not missing, missing


def test_status_strings_and_version():
    for s in (0, -1, -2, -3, -4, -5):
        assert g.atma_status_string(s)
    assert g.atma_status_string(42) == "unknown status"
    assert g.atma_version() >= 100


def test_workspace_queries():
    assert g.lib.atma_gdn_fwd_workspace_bytes_dtype(1, 256, 1, 64, 64, 64, g.ATMA_F32) > 0
    # bf16 records are smaller than fp32 ones; a ragged tail still gets a full chunk record
    a = g.lib.atma_gdn_fwd_workspace_bytes_dtype(2, 100, 3, 128, 128, 64, g.ATMA_BF16)
    b = g.lib.atma_gdn_fwd_workspace_bytes_dtype(2, 128, 3, 128, 128, 64, g.ATMA_BF16)
    assert a == b > 0
    assert g.lib.atma_gdn_fwd_workspace_bytes_dtype(1, 256, 1, 96, 64, 64, g.ATMA_BF16) == 0  # unsupported width
    assert g.lib.atma_gdn_fwd_workspace_bytes_dtype(1, 256, 1, 64, 64, 32, g.ATMA_BF16) == 0  # unsupported chunk
    # the six-argument query covers either dtype (the larger need)
    for args in ((1, 256, 1, 64, 64, 64), (2, 100, 3, 128, 128, 64), (1, 70000, 8, 128, 64, 64)):
        both = [g.lib.atma_gdn_fwd_workspace_bytes_dtype(*args, dt) for dt in (g.ATMA_BF16, g.ATMA_F32)]
        assert g.lib.atma_gdn_fwd_workspace_bytes(*args) == max(both) > 0
    assert g.lib.atma_gdn_fwd_workspace_bytes(1, 256, 1, 96, 64, 64) == 0
    assert g.lib.atma_polar_attn_workspace_bytes(1, 1024, 16, 64) == 0
    assert g.lib.atma_polar_attn_decode_workspace_bytes(1, 16, 262144, 64) > 0
    assert g.lib.atma_polar_attn_decode_workspace_bytes(1, 16, 0, 64) == 0


def _gdn(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, init=NULL, o=FAKE, fin=NULL, B=1, T=8, H=1, Dk=64, Dv=64,
             chunk=64, dt=g.ATMA_BF16, ws=FAKE, wsb=1, stream=NULL)
    a.update(over)
    return g.lib.atma_gdn_fwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["init"], a["o"], a["fin"], a["B"],
                              a["T"], a["H"], a["Dk"], a["Dv"], a["chunk"], a["dt"], a["ws"], a["wsb"], a["stream"])


def test_gdn_fwd_validation():
    assert _gdn(q=NULL) == g.ATMA_ERR_NULL
    assert _gdn(o=NULL) == g.ATMA_ERR_NULL
    assert _gdn(T=0) == g.ATMA_ERR_SHAPE
    assert _gdn(B=-1) == g.ATMA_ERR_SHAPE
    assert _gdn(Dk=96) == g.ATMA_ERR_UNSUPPORTED
    assert _gdn(chunk=32) == g.ATMA_ERR_UNSUPPORTED
    assert _gdn(dt=7) == g.ATMA_ERR_UNSUPPORTED
    assert _gdn(B=70000, T=70000) == g.ATMA_ERR_SHAPE          # element count overflow
    assert _gdn(ws=NULL) == g.ATMA_ERR_WORKSPACE
    assert _gdn(wsb=1) == g.ATMA_ERR_WORKSPACE                  # too small
    need = g.lib.atma_gdn_fwd_workspace_bytes_dtype(1, 8, 1, 64, 64, 64, g.ATMA_BF16)
    assert _gdn(wsb=need - 1) == g.ATMA_ERR_WORKSPACE


def _gdnv(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, cu=FAKE, nseq=2, maxT=8, init=NULL, o=FAKE, fin=NULL,
             total=10, H=1, Dk=64, Dv=64, chunk=64, dt=g.ATMA_BF16, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return g.lib.atma_gdn_fwd_varlen(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["cu"], a["nseq"], a["maxT"],
                                     a["init"], a["o"], a["fin"], a["total"], a["H"], a["Dk"], a["Dv"], a["chunk"],
                                     a["dt"], a["ws"], a["wsb"], NULL)


def test_gdn_fwd_varlen_validation():
    assert _gdnv(cu=NULL) == g.ATMA_ERR_NULL
    assert _gdnv(beta=NULL) == g.ATMA_ERR_NULL
    assert _gdnv(nseq=0) == g.ATMA_ERR_SHAPE
    assert _gdnv(maxT=11) == g.ATMA_ERR_SHAPE           # longer than all rows together
    assert _gdnv(total=0) == g.ATMA_ERR_SHAPE
    assert _gdnv(dt=g.ATMA_F32) == g.ATMA_ERR_UNSUPPORTED  # packed batches take the bf16 path
    assert _gdnv(Dk=96) == g.ATMA_ERR_UNSUPPORTED
    assert _gdnv(chunk=32) == g.ATMA_ERR_UNSUPPORTED
    assert _gdnv(ws=NULL) == g.ATMA_ERR_WORKSPACE
    need = g.lib.atma_gdn_fwd_workspace_bytes_dtype(2, 8, 1, 64, 64, 64, g.ATMA_BF16)
    assert _gdnv(wsb=need - 1) == g.ATMA_ERR_WORKSPACE


def test_gdn_decode_validation():
    f = g.lib.atma_gdn_decode_step
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 1, 8, 128, 128, g.ATMA_BF16, NULL) == g.ATMA_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 128, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 100, 128, g.ATMA_BF16, NULL) == g.ATMA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 128, 128, 3, NULL) == g.ATMA_ERR_UNSUPPORTED


def _params(**over):
    p = dict(temp_raw=0x1000, null_slope_raw=0x1000, null_bias=0x1000, mag_beta=0x1000, v_null=0x1000, eps=1e-12)
    p.update(over)
    return g.PolarParams(**p)


def _pfwd(p=None, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, mu=NULL, meff=NULL, B=1, T=16, Hq=4, Hkv=2, D=64, dt=g.ATMA_BF16)
    a.update(over)
    pp = ctypes.byref(p if p is not None else _params()) if p is not False else None
    return g.lib.atma_polar_attn_fwd(a["q"], a["k"], a["v"], pp, a["o"], a["mu"], a["meff"], a["B"], a["T"], a["Hq"],
                                     a["Hkv"], a["D"], a["dt"], NULL, 0, NULL)


def test_polar_fwd_validation():
    assert _pfwd(q=NULL) == g.ATMA_ERR_NULL
    assert _pfwd(p=False) == g.ATMA_ERR_NULL
    assert _pfwd(p=_params(v_null=None)) == g.ATMA_ERR_NULL
    assert _pfwd(p=_params(eps=-1.0)) == g.ATMA_ERR_SHAPE
    assert _pfwd(p=_params(eps=float("nan"))) == g.ATMA_ERR_SHAPE
    assert _pfwd(T=0) == g.ATMA_ERR_SHAPE
    assert _pfwd(Hq=3, Hkv=2) == g.ATMA_ERR_SHAPE
    assert _pfwd(D=96) == g.ATMA_ERR_UNSUPPORTED
    assert _pfwd(dt=g.ATMA_F32) == g.ATMA_ERR_UNSUPPORTED


def _pdec(p=None, **over):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, L=10, Lmax=16, o=FAKE, mu=NULL, B=1, Hq=16, Hkv=16, D=64, dt=g.ATMA_BF16,
             ws=FAKE, wsb=1 << 30)
    a.update(over)
    pp = ctypes.byref(p if p is not None else _params())
    return g.lib.atma_polar_attn_decode(a["q"], a["kc"], a["vc"], a["L"], a["Lmax"], pp, a["o"], a["mu"], a["B"],
                                        a["Hq"], a["Hkv"], a["D"], a["dt"], a["ws"], a["wsb"], NULL)


def test_polar_decode_validation():
    assert _pdec(kc=NULL) == g.ATMA_ERR_NULL
    assert _pdec(L=0) == g.ATMA_ERR_SHAPE
    assert _pdec(L=17) == g.ATMA_ERR_SHAPE            # cache_len > Lmax
    assert _pdec(Hq=16, Hkv=3) == g.ATMA_ERR_SHAPE
    assert _pdec(Hq=48, Hkv=3) == g.ATMA_ERR_UNSUPPORTED   # head layout without a kernel
    assert _pdec(D=96) == g.ATMA_ERR_UNSUPPORTED
    assert _pdec(D=128, Hq=32, Hkv=32) == g.ATMA_ERR_UNSUPPORTED  # 32 kv heads x 128: no kernel
    assert _pdec(ws=NULL) == g.ATMA_ERR_WORKSPACE
    assert _pdec(wsb=16) == g.ATMA_ERR_WORKSPACE


def _pdecv(p=None, **over):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, Lb=10, Lmax=16, o=FAKE, mu=NULL, B=2, Hq=16, Hkv=16, D=64,
             dt=g.ATMA_BF16, ws=FAKE, wsb=1 << 30)
    a.update(over)
    pp = ctypes.byref(p if p is not None else _params())
    return g.lib.atma_polar_attn_decode_varlen(a["q"], a["kc"], a["vc"], a["lens"], a["Lb"], a["Lmax"], pp, a["o"],
                                               a["mu"], a["B"], a["Hq"], a["Hkv"], a["D"], a["dt"], a["ws"], a["wsb"],
                                               NULL)


def test_polar_decode_varlen_validation():
    assert _pdecv(lens=NULL) == g.ATMA_ERR_NULL
    assert _pdecv(o=NULL) == g.ATMA_ERR_NULL
    assert _pdecv(Lb=0) == g.ATMA_ERR_SHAPE
    assert _pdecv(Lb=17) == g.ATMA_ERR_SHAPE           # bound > Lmax
    assert _pdecv(B=0) == g.ATMA_ERR_SHAPE
    assert _pdecv(Hq=16, Hkv=3) == g.ATMA_ERR_SHAPE
    assert _pdecv(D=96) == g.ATMA_ERR_UNSUPPORTED
    assert _pdecv(dt=g.ATMA_F32) == g.ATMA_ERR_UNSUPPORTED
    assert _pdecv(ws=NULL) == g.ATMA_ERR_WORKSPACE
    need = g.lib.atma_polar_attn_decode_workspace_bytes(2, 16, 10, 64)
    assert _pdecv(wsb=need - 1) == g.ATMA_ERR_WORKSPACE


def _pfwdv(p=None, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, nseq=3, maxT=100, o=FAKE, mu=NULL, meff=NULL, total=200, Hq=4, Hkv=2,
             D=64, dt=g.ATMA_BF16)
    a.update(over)
    pp = ctypes.byref(p if p is not None else _params())
    return g.lib.atma_polar_attn_fwd_varlen(a["q"], a["k"], a["v"], a["cu"], a["nseq"], a["maxT"], pp, a["o"],
                                            a["mu"], a["meff"], a["total"], a["Hq"], a["Hkv"], a["D"], a["dt"], NULL)


def test_polar_fwd_varlen_validation():
    assert _pfwdv(cu=NULL) == g.ATMA_ERR_NULL
    assert _pfwdv(v=NULL) == g.ATMA_ERR_NULL
    assert _pfwdv(nseq=0) == g.ATMA_ERR_SHAPE
    assert _pfwdv(maxT=0) == g.ATMA_ERR_SHAPE
    assert _pfwdv(maxT=201) == g.ATMA_ERR_SHAPE          # longer than all rows together
    assert _pfwdv(Hq=4, Hkv=3) == g.ATMA_ERR_SHAPE
    assert _pfwdv(D=96) == g.ATMA_ERR_UNSUPPORTED
    assert _pfwdv(dt=g.ATMA_F32) == g.ATMA_ERR_UNSUPPORTED
    assert _pfwdv(p=_params(v_null=0)) == g.ATMA_ERR_NULL


def test_control_core_validation():
    L = g.lib
    assert L.atma_rope(NULL, FAKE, 1, 8, 1, 64, 0, 10000.0, g.ATMA_BF16, NULL) == g.ATMA_ERR_NULL
    assert L.atma_rope(FAKE, FAKE, 1, 8, 1, 63, 0, 10000.0, g.ATMA_BF16, NULL) == g.ATMA_ERR_UNSUPPORTED
    assert L.atma_rope(FAKE, FAKE, 1, 8, 1, 64, 0, 0.0, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE
    assert L.atma_rope(FAKE, FAKE, 1, 8, 1, 64, -1, 10000.0, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE
    f = L.atma_softmax_attn_fwd
    assert f(FAKE, FAKE, NULL, FAKE, 1, 8, 4, 2, 64, 0.0, g.ATMA_BF16, NULL, 0, NULL) == g.ATMA_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 3, 64, 0.0, g.ATMA_BF16, NULL, 0, NULL) == g.ATMA_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 2, 96, 0.0, g.ATMA_BF16, NULL, 0, NULL) == g.ATMA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 2, 64, -1.0, g.ATMA_BF16, NULL, 0, NULL) == g.ATMA_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 2, 64, 10000.0, g.ATMA_BF16, NULL, 0, NULL) == g.ATMA_ERR_WORKSPACE
    assert L.atma_softmax_attn_workspace_bytes(1, 8, 4, 2, 64, 0.0) == 0
    assert L.atma_softmax_attn_workspace_bytes(1, 8, 4, 2, 64, 10000.0) == 8 * 6 * 64 * 2
    d = L.atma_softmax_attn_decode
    assert d(FAKE, FAKE, FAKE, 9, 8, 0.0, FAKE, 1, 16, 16, 64, g.ATMA_BF16, FAKE, 1 << 30, NULL) == g.ATMA_ERR_SHAPE
    assert d(FAKE, FAKE, FAKE, 8, 8, 0.0, FAKE, 1, 16, 16, 64, g.ATMA_BF16, NULL, 0, NULL) == g.ATMA_ERR_WORKSPACE


def test_polar_train_and_backward_validation():
    pp = ctypes.byref(_params())
    ft = g.lib.atma_polar_attn_fwd_train
    assert ft(FAKE, FAKE, FAKE, pp, FAKE, FAKE, FAKE, NULL, 1, 16, 4, 2, 64, g.ATMA_BF16, NULL) == g.ATMA_ERR_NULL
    assert ft(FAKE, FAKE, FAKE, ctypes.byref(_params(eps=0.0)), FAKE, FAKE, FAKE, FAKE, 1, 16, 4, 2, 64, g.ATMA_BF16,
              NULL) == g.ATMA_ERR_SHAPE  # the backward needs eps > 0
    assert ft(FAKE, FAKE, FAKE, pp, FAKE, FAKE, FAKE, FAKE, 1, 16, 4, 3, 64, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE
    assert ft(FAKE, FAKE, FAKE, pp, FAKE, FAKE, FAKE, FAKE, 1, 16, 4, 2, 96, g.ATMA_BF16, NULL) == g.ATMA_ERR_UNSUPPORTED
    grads = g.PolarParamGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    bad = g.PolarParamGrads(0x1000, 0x1000, None, 0x1000, 0x1000)
    b = g.lib.atma_polar_attn_bwd

    def call(gr=grads, dO=FAKE, B=1, T=16, Hq=4, Hkv=2, D=64, dt=g.ATMA_BF16, ws=FAKE, wsb=1 << 30, p=pp):
        return b(FAKE, FAKE, FAKE, p, FAKE, FAKE, FAKE, dO, FAKE, FAKE, FAKE, ctypes.byref(gr), B, T, Hq, Hkv, D, dt,
                 ws, wsb, NULL)

    assert call(dO=NULL) == g.ATMA_ERR_NULL
    assert call(gr=bad) == g.ATMA_ERR_NULL
    assert call(T=0) == g.ATMA_ERR_SHAPE
    assert call(Hq=4, Hkv=3) == g.ATMA_ERR_SHAPE
    assert call(D=32) == g.ATMA_ERR_UNSUPPORTED
    assert call(dt=g.ATMA_F32) == g.ATMA_ERR_UNSUPPORTED
    assert call(ws=NULL) == g.ATMA_ERR_WORKSPACE
    need = g.lib.atma_polar_attn_bwd_workspace_bytes(1, 16, 4, 2, 64)
    assert need > 0 and call(wsb=need - 1) == g.ATMA_ERR_WORKSPACE
    assert g.lib.atma_polar_attn_bwd_workspace_bytes(1, 16, 4, 2, 96) == 0


def test_gdn_backward_validation():
    f = g.lib.atma_gdn_bwd

    def call(dO=FAKE, B=1, T=16, H=1, Dk=64, Dv=64, chunk=64, dt=g.ATMA_BF16, ws=FAKE, wsb=1 << 30, dq=FAKE):
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, dO, NULL, dq, FAKE, FAKE, FAKE, FAKE, NULL, B, T, H, Dk, Dv,
                 chunk, dt, ws, wsb, NULL)

    assert call(dO=NULL) == g.ATMA_ERR_NULL
    assert call(dq=NULL) == g.ATMA_ERR_NULL
    assert call(T=0) == g.ATMA_ERR_SHAPE
    assert call(Dk=96) == g.ATMA_ERR_UNSUPPORTED
    assert call(chunk=32) == g.ATMA_ERR_UNSUPPORTED
    assert call(dt=3) == g.ATMA_ERR_UNSUPPORTED
    assert call(ws=NULL) == g.ATMA_ERR_WORKSPACE
    need = g.lib.atma_gdn_bwd_workspace_bytes(1, 16, 1, 64, 64, 64, g.ATMA_BF16)
    assert need > 0 and call(wsb=need - 1) == g.ATMA_ERR_WORKSPACE
    assert g.lib.atma_gdn_bwd_workspace_bytes(1, 16, 1, 64, 64, 32, g.ATMA_BF16) == 0


def test_canon_validation():
    c = g.lib.atma_canon
    Y2 = ctypes.c_void_p(0x2000)  # output, distinct from the input
    assert c(NULL, FAKE, NULL, NULL, Y2, 1, 8, 64, 4, 0, 0, 1e-6, g.ATMA_BF16, NULL) == g.ATMA_ERR_NULL
    assert c(FAKE, FAKE, NULL, NULL, Y2, 1, 8, 64, 9, 0, 0, 1e-6, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE   # K > 8
    assert c(FAKE, FAKE, NULL, NULL, Y2, 1, 8, 64, 0, 0, 0, 1e-6, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE
    assert c(FAKE, FAKE, NULL, NULL, Y2, 1, 8, 60, 4, 0, 0, 1e-6, g.ATMA_BF16, NULL) == g.ATMA_ERR_UNSUPPORTED
    assert c(FAKE, FAKE, NULL, NULL, Y2, 1, 8, 64, 4, 0, 3, 1e-6, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE   # C % heads
    assert c(FAKE, FAKE, NULL, NULL, Y2, 1, 8, 96, 4, 0, 1, 1e-6, g.ATMA_BF16, NULL) == g.ATMA_ERR_UNSUPPORTED
    assert c(FAKE, FAKE, NULL, NULL, Y2, 1, 8, 64, 4, 0, 0, 1e-6, g.ATMA_F32, NULL) == g.ATMA_ERR_UNSUPPORTED
    assert c(FAKE, FAKE, NULL, NULL, Y2, 1, 8, 64, 4, 0, 0, 0.0, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE
    assert c(FAKE, FAKE, NULL, NULL, FAKE, 1, 8, 64, 4, 0, 0, 1e-6, g.ATMA_BF16, NULL) == g.ATMA_ERR_SHAPE  # y == x


def test_binding_rejects_host_tensors():
    import torch

    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    a = torch.ones(1, 8, 1)
    with pytest.raises((ValueError, RuntimeError)):
        g.atma_gdn_fwd(q, q, q, a, a, workspace=torch.zeros(1, dtype=torch.uint8), o=q.clone(),
                       final_state=torch.zeros(1, 1, 64, 64))


# ---- the Python binding rejects malformed buffers before reaching the C ABI -------------------
# These run on CPU tensors: the shape and dtype checks come before the device check, so each
# call below raises on the host, naming the offending buffer, and nothing is launched.
import torch  # noqa: E402


def _polar_params(Hq, D):
    return {"temp_raw": torch.zeros(Hq), "null_slope_raw": torch.zeros(Hq), "null_bias": torch.zeros(Hq),
            "mag_beta": torch.zeros(Hq), "v_null": torch.zeros(Hq, D), "eps": 1e-12}


def _raises(fn, match):
    with pytest.raises((ValueError, TypeError), match=match):
        fn()


def test_binding_checks_memory_buffers():
    bf = torch.bfloat16
    B, T, H, D = 2, 8, 2, 64
    q = torch.zeros(B, T, H, D, dtype=bf)
    a = torch.zeros(B, T, H)
    _raises(lambda: g.atma_gdn_fwd(q, q, q, a, a, torch.zeros(B, H, D, D + 1)), "init_state")
    _raises(lambda: g.atma_gdn_fwd(q, q, q, a, a, torch.zeros(B, H, D, D, dtype=torch.float64)), "init_state")
    _raises(lambda: g.atma_gdn_fwd(q, q, q, a, a, o=torch.zeros(B, T, H, D)), "o has dtype")
    _raises(lambda: g.atma_gdn_fwd(q, q, q, a, a, o=torch.zeros(B, T, H, D - 1, dtype=bf)), "o has shape")
    _raises(lambda: g.atma_gdn_fwd(q, q, q, a, a, final_state=torch.zeros(B, H, D, D - 8)), "final_state")
    st = torch.zeros(B, H, D, D)
    qd, ad = torch.zeros(B, H, D, dtype=bf), torch.zeros(B, H)
    _raises(lambda: g.atma_gdn_decode_step(qd, torch.zeros(B, H + 1, D, dtype=bf), qd, ad, ad, st), "k has shape")
    _raises(lambda: g.atma_gdn_decode_step(qd, qd, torch.zeros(B, H, D), ad, ad, st), "v has dtype")
    _raises(lambda: g.atma_gdn_decode_step(qd, qd, qd, torch.zeros(B, H + 1), ad, st), "alpha")
    _raises(lambda: g.atma_gdn_decode_step(qd, qd, qd, ad, torch.zeros(B), st), "beta")
    _raises(lambda: g.atma_gdn_decode_step(qd, qd, qd, ad, ad, st, o=torch.zeros(B, H, 2 * D, dtype=bf)), "o has")
    _raises(lambda: g.atma_gdn_bwd(q, q, q, a, a, torch.zeros(B, T, H, D)), "share a dtype")
    _raises(lambda: g.atma_gdn_bwd(q, q, q, a, a, q, init_state=torch.zeros(B, H, D, 1)), "init_state")
    _raises(lambda: g.atma_gdn_bwd(q, q, q, a, a, q, dS_final=torch.zeros(1, H, D, D)), "dS_final")


def test_binding_checks_polar_buffers():
    bf = torch.bfloat16
    B, T, Hq, Hkv, D = 2, 8, 4, 2, 64
    q, kv = torch.zeros(B, T, Hq, D, dtype=bf), torch.zeros(B, T, Hkv, D, dtype=bf)
    p = _polar_params(Hq, D)
    _raises(lambda: g.atma_polar_attn_fwd(q, kv, kv, _polar_params(Hq - 1, D)), "temp_raw")
    bad = dict(p, v_null=torch.zeros(Hq, D // 2))
    _raises(lambda: g.atma_polar_attn_fwd(q, kv, kv, bad), "v_null")
    _raises(lambda: g.atma_polar_attn_fwd(q, kv, kv, p, o=torch.zeros(B, T, Hq, D)), "o has dtype")
    _raises(lambda: g.atma_polar_attn_fwd(q, kv, kv, p, mu_out=torch.zeros(B, T, Hq)), "mu_out")
    _raises(lambda: g.atma_polar_attn_fwd(q, kv, kv, p, meff_out=torch.zeros(B, Hq, T, dtype=bf)), "meff_out")
    _raises(lambda: g.atma_polar_attn_fwd(q, kv, torch.zeros(B, T, Hkv, D), p), "v has dtype")
    mu, stats, dirn = torch.zeros(B, Hq, T), torch.zeros(B, Hq, T, 4), torch.zeros(B, T, Hq, D)
    _raises(lambda: g.atma_polar_attn_bwd(q, kv, kv, p, mu, stats, dirn, torch.zeros(B, T, Hq, D)), "do has dtype")
    _raises(lambda: g.atma_polar_attn_bwd(q, kv, kv, p, mu.double(), stats, dirn, q), "mu has dtype")
    _raises(lambda: g.atma_polar_attn_bwd(q, kv, kv, p, mu, stats.to(bf), dirn, q), "stats has dtype")
    _raises(lambda: g.atma_polar_attn_bwd(q, kv, kv, p, mu, stats, dirn.to(bf), q), "dir has dtype")
    outs = {"dq": torch.zeros_like(q), "dk": torch.zeros_like(kv), "dv": torch.zeros_like(kv),
            "d_temp_raw": torch.zeros(Hq), "d_null_slope_raw": torch.zeros(Hq), "d_null_bias": torch.zeros(Hq),
            "d_mag_beta": torch.zeros(Hq), "d_v_null": torch.zeros(Hq, D + 1)}
    _raises(lambda: g.atma_polar_attn_bwd(q, kv, kv, p, mu, stats, dirn, q, out=outs), "d_v_null")
    L = 16
    qd, kc = torch.zeros(B, Hq, D, dtype=bf), torch.zeros(B, L, Hkv, D, dtype=bf)
    _raises(lambda: g.atma_polar_attn_decode(qd, kc, torch.zeros(B, L + 1, Hkv, D, dtype=bf), L, p), "v_cache")
    _raises(lambda: g.atma_polar_attn_decode(qd, kc, kc, L, p, o=torch.zeros(B, Hq, D)), "o has dtype")
    _raises(lambda: g.atma_polar_attn_decode(qd, kc, kc, L, p, mu_out=torch.zeros(B, Hq + 1)), "mu_out")
    lens = torch.full((B,), L, dtype=torch.int32)
    _raises(lambda: g.atma_polar_attn_decode_varlen(qd, kc, kc, lens.long(), L, p), "cache_lens")
    _raises(lambda: g.atma_softmax_attn_fwd(q, kv, kv, o=torch.zeros(B, T, Hq, D - 8, dtype=bf)), "o has shape")
    _raises(lambda: g.atma_rope(q, out=torch.zeros(B, T, Hq, D)), "out has dtype")
    x, w = torch.zeros(B, T, 128, dtype=bf), torch.zeros(4, 128)
    _raises(lambda: g.atma_canon(x, w.double()), "w has dtype")
    _raises(lambda: g.atma_canon(x, w, torch.zeros(B, 4, 128, dtype=bf)), "state has shape")
    _raises(lambda: g.atma_canon(x, w, y=torch.zeros(B, T, 128)), "y has dtype")
