"""The C-ABI library without a GPU: it loads, exports every function that
include/ds4q.h declares, and rejects bad arguments on the host with the
documented status codes.  Every call here is chosen so that validation fails
before anything is enqueued (the fake device addresses are never touched)."""
import ctypes
import os
import re

import pytest

import bit_quantized_moe_q2_amd as ds4q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4q.h")

OK, E_INVAL, E_UNSUPPORTED, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ALIAS = 0, -1, -2, -3, -4, -5, -6
BASE = 1 << 40          # fake, 4 KiB-aligned device addresses, never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds4q_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    try:
        return ds4q.load()
    except ImportError as e:      # the build step must have run
        pytest.fail(str(e))


def _layer(**kw):
    a = dict(n_embd=4096, n_ff=2048, n_expert=256, n_expert_used=6, type_gate=ds4q.TYPE_Q2_K,
             type_up=ds4q.TYPE_Q2_K, type_down=ds4q.TYPE_Q2_K, gate=BASE, up=BASE + (1 << 32),
             down=BASE + (2 << 32), flags=0, norm_eps=1e-6)
    a.update(kw)
    return ds4q.MoeLayer(**a)


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "ds4q_moe_decode" in names and "ds4q_dequant" in names and len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    m = re.search(r"#define DS4Q_ABI_VERSION (\d+)", open(HEADER).read())
    assert ds4q.ds4q_abi_version() == int(m.group(1))
    for code in (OK, E_INVAL, E_UNSUPPORTED, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ALIAS, -7, -8):
        assert ds4q.ds4q_strerror(code) != "unknown status"
    assert ds4q.ds4q_strerror(-99) == "unknown status"


def test_dequant_validation(lib):
    f = lib.ds4q_dequant
    src, dst = BASE, BASE + (1 << 32)
    assert f(ds4q.TYPE_IQ2_XXS, src, 4, 256, ds4q.TYPE_F32, dst, None) == E_UNSUPPORTED
    assert f(ds4q.TYPE_Q2_K, src, 4, 256, ds4q.TYPE_F16, dst, None) == E_UNSUPPORTED
    assert f(ds4q.TYPE_Q2_K, src, 4, 200, ds4q.TYPE_F32, dst, None) == E_SHAPE
    assert f(ds4q.TYPE_Q4_1, src, 4, 48, ds4q.TYPE_F32, dst, None) == E_SHAPE
    assert f(ds4q.TYPE_Q2_K, src, -1, 256, ds4q.TYPE_F32, dst, None) == E_SHAPE
    assert f(ds4q.TYPE_Q2_K, src, 0, 256, ds4q.TYPE_F32, dst, None) == OK       # no-op
    assert f(ds4q.TYPE_Q2_K, None, 4, 256, ds4q.TYPE_F32, dst, None) == E_INVAL
    assert f(ds4q.TYPE_Q2_K, src, 4, 256, ds4q.TYPE_F32, dst + 8, None) == E_ALIGN
    assert f(ds4q.TYPE_Q2_K, src + 4, 4, 256, ds4q.TYPE_F32, dst, None) == E_ALIGN
    assert f(ds4q.TYPE_Q2_K, src, 4, 256, ds4q.TYPE_BF16, src + 64, None) == E_ALIAS


def test_matvec_and_route_validation(lib):
    assert lib.ds4q_matvec(ds4q.TYPE_Q2_K, BASE, 8, 300, BASE + (1 << 32), 1,
                           BASE + (2 << 32), None) == E_SHAPE
    assert lib.ds4q_route_workspace_size(10, 256, 9) == 0
    assert lib.ds4q_route_workspace_size(10, 256, 6) > 0
    out = ds4q.RouteOut(BASE, BASE + 4096, 0, 0, 0)
    assert lib.ds4q_route(BASE + (1 << 32), 10, 256, 9, ctypes.byref(out), BASE + (2 << 32),
                          1 << 20, None) == E_INVAL
    assert lib.ds4q_route(BASE + (1 << 32), 65537, 256, 6, ctypes.byref(out), BASE + (2 << 32),
                          1 << 20, None) == E_SHAPE


def test_layer_descriptor_validation(lib):
    ws = lambda L: lib.ds4q_moe_workspace_size(ctypes.byref(L), 1, 0)
    assert ws(_layer()) > 0
    assert ws(_layer(type_gate=ds4q.TYPE_IQ2_XXS, type_up=ds4q.TYPE_IQ2_XXS)) == 0
    assert lib.ds4q_moe_workspace_size(None, 1, 0) == 0
    assert lib.ds4q_moe_workspace_size(ctypes.byref(_layer()), 1, 2) == 0
    x, lg, y, w = BASE + (8 << 32), BASE + (9 << 32), BASE + (10 << 32), BASE + (11 << 32)
    dec = lambda L, T=1: lib.ds4q_moe_decode(ctypes.byref(L), x, lg, T, y, None, w, 1 << 30, None)
    assert dec(_layer(type_gate=ds4q.TYPE_IQ2_XXS, type_up=ds4q.TYPE_IQ2_XXS)) == E_UNSUPPORTED
    assert dec(_layer(type_up=ds4q.TYPE_Q4_1)) == E_UNSUPPORTED        # gate and up share a type
    assert dec(_layer(n_embd=3072)) == E_SHAPE
    assert dec(_layer(n_ff=128)) == E_SHAPE
    assert dec(_layer(n_expert_used=9)) == E_INVAL
    assert dec(_layer(n_expert=2000)) == E_INVAL
    assert dec(_layer(gate=0)) == E_INVAL
    assert dec(_layer(down=BASE + 8)) == E_ALIGN
    assert dec(_layer(flags=0x8)) == E_INVAL
    assert dec(_layer(norm_eps=float("nan"))) == E_INVAL


def test_decode_call_validation(lib):
    L = _layer()
    need = lib.ds4q_moe_workspace_size(ctypes.byref(L), 4, 0)
    assert need > lib.ds4q_moe_workspace_size(ctypes.byref(L), 1, 0) > 0
    x, lg, y, w = BASE + (8 << 32), BASE + (9 << 32), BASE + (10 << 32), BASE + (11 << 32)

    def dec(x=x, lg=lg, T=4, y=y, w=w, wb=need):
        return lib.ds4q_moe_decode(ctypes.byref(L), x, lg, T, y, None, w, wb, None)

    assert dec(T=65) == E_SHAPE
    assert dec(T=-1) == E_SHAPE
    assert dec(T=0) == OK                                   # nothing to do
    assert dec(x=None) == E_INVAL
    assert dec(w=None) == E_WORKSPACE
    assert dec(wb=need - 1) == E_WORKSPACE
    assert dec(x=x + 4) == E_ALIGN
    assert dec(w=w + 16) == E_ALIGN
    assert dec(y=x + 4096 * 4) == E_ALIAS                   # partial overlap of x and y
    assert dec(w=y) == E_ALIAS                              # workspace over the output
    assert dec(lg=y + 64) == E_ALIAS
    ph = lambda p: lib.ds4q_moe_decode_phases(ctypes.byref(L), x, lg, 4, y, None, w, need, p, None)
    assert ph(0) == E_INVAL and ph(8) == E_INVAL and ph(0x17) == E_INVAL
    assert lib.ds4q_moe_decode_phases(ctypes.byref(L), x, lg, 65, y, None, w, need,
                                      ds4q.PHASE_GATEUP, None) == E_SHAPE
    # the allocation-free variant checks its arguments the same way, before
    # it looks up the static scratch on the device
    st = lambda x=x, lg=lg, T=4, y=y: lib.ds4q_moe_decode_static(ctypes.byref(L), x, lg, T, y, None, None)
    assert st(T=65) == E_SHAPE and st(T=-1) == E_SHAPE and st(T=0) == OK
    assert st(x=None) == E_INVAL and st(x=x + 4) == E_ALIGN
    assert st(y=x + 4096 * 4) == E_ALIAS and st(lg=y + 64) == E_ALIAS
    assert lib.ds4q_moe_decode_static(ctypes.byref(_layer(n_expert_used=9)), x, lg, 4, y, None,
                                      None) == E_INVAL


def test_prefill_and_stack_validation(lib):
    L = _layer()
    need = lib.ds4q_moe_workspace_size(ctypes.byref(L), 4096, 1)
    x, lg, y, w = BASE + (8 << 32), BASE + (9 << 32), BASE + (10 << 32), BASE + (11 << 32)
    pre = lambda xt, L=L, T=4096: lib.ds4q_moe_prefill(ctypes.byref(L), x, xt, lg, T, y, None, w,
                                                       need, None)
    assert pre(ds4q.TYPE_F16) == E_UNSUPPORTED
    assert pre(ds4q.TYPE_BF16, _layer(flags=ds4q.F_RMSNORM_INPUT)) == E_INVAL
    assert pre(ds4q.TYPE_BF16, T=65537) == E_SHAPE
    assert lib.ds4q_moe_prefill(ctypes.byref(L), x, ds4q.TYPE_BF16, lg, 4096, y, None, w,
                                need - 256, None) == E_WORKSPACE
    arr = (ds4q.MoeLayer * 2)(_layer(), _layer(n_ff=1024))
    wsd = lib.ds4q_moe_workspace_size(ctypes.byref(L), 1, 0)
    assert lib.ds4q_moe_stack(arr, 2, 0, x, lg, 1, w, wsd, None) == E_SHAPE
    assert lib.ds4q_moe_stack(arr, 2, 2, x, lg, 1, w, wsd, None) == E_INVAL
    assert lib.ds4q_moe_stack(arr, 0, 0, x, lg, 1, w, wsd, None) == OK
    same = (ds4q.MoeLayer * 2)(_layer(), _layer())
    assert lib.ds4q_moe_stack(same, 2, 0, x, x + 64, 1, w, wsd, None) == E_ALIAS


def test_timing_read_empty(lib):
    assert ds4q.ds4q_timing_read() == {}


def test_layer_steering_validation(lib):
    """Steering fields of the layer descriptor (directional-steering section
    of the steering page): alignment, a finite scale, no overlap of the
    direction with the output or the workspace.  NULL switches it off."""
    x, lg, y, w = BASE + (8 << 32), BASE + (9 << 32), BASE + (10 << 32), BASE + (11 << 32)
    dvec = BASE + (12 << 32)

    def dec(L, T=4, y=y):
        need = lib.ds4q_moe_workspace_size(ctypes.byref(L), T, 0)
        return lib.ds4q_moe_decode(ctypes.byref(L), x, lg, T, y, None, w, need, None)

    assert dec(_layer(steer_dir=dvec + 4, steer_scale=1.0)) == E_ALIGN
    assert dec(_layer(steer_dir=dvec, steer_scale=float("nan"))) == E_INVAL
    assert dec(_layer(steer_dir=dvec, steer_scale=float("inf"))) == E_INVAL
    assert dec(_layer(steer_dir=y + 1024, steer_scale=1.0)) == E_ALIAS   # inside y
    assert dec(_layer(steer_dir=w + 256, steer_scale=1.0)) == E_ALIAS    # inside the workspace
    assert dec(_layer(steer_dir=dvec, steer_scale=1.0), T=0) == OK
    assert lib.ds4q_moe_workspace_size(ctypes.byref(_layer(steer_dir=dvec + 4, steer_scale=1.0)), 1, 0) == 0
    bad = (ds4q.MoeLayer * 2)(_layer(), _layer(steer_dir=dvec + 8, steer_scale=1.0))
    assert lib.ds4q_moe_stack(bad, 2, 0, x, lg, 1, w, 1 << 30, None) == E_ALIGN
    # the one-token workspace holds the staged row of the steering tail
    assert (lib.ds4q_moe_workspace_size(ctypes.byref(_layer()), 1, 0)
            >= 4096 * 4 + 6 * 2048 * 4)


def test_layer_imatrix_validation(lib):
    """imatrix accumulators of the layer descriptor: 16-byte alignment, no
    overlap with each other, the output, the workspace or the weights; the
    m-tile paths reserve partial rows in the workspace only when asked."""
    x, lg, y, w = BASE + (8 << 32), BASE + (9 << 32), BASE + (10 << 32), BASE + (11 << 32)
    sa, sb = BASE + (12 << 32), BASE + (13 << 32)

    def pre(L, T=64):
        need = lib.ds4q_moe_workspace_size(ctypes.byref(L), T, 1)
        return lib.ds4q_moe_prefill(ctypes.byref(L), x, ds4q.TYPE_F32, lg, T, y, None, w, need, None)

    assert pre(_layer(imatrix_in=sa + 4)) == E_ALIGN
    assert pre(_layer(imatrix_down=sb + 8)) == E_ALIGN
    assert pre(_layer(imatrix_in=sa, imatrix_down=sa + 4096)) == E_ALIAS     # the two overlap
    assert pre(_layer(imatrix_in=y)) == E_ALIAS                                # over the output
    assert pre(_layer(imatrix_down=w + 1024)) == E_ALIAS                       # inside the workspace
    assert pre(_layer(imatrix_in=BASE + 256)) == E_ALIAS                       # inside the gate tensor
    assert pre(_layer(imatrix_in=sa, imatrix_down=sb), T=0) == OK
    plain = lib.ds4q_moe_workspace_size(ctypes.byref(_layer()), 4096, 1)
    stats = lib.ds4q_moe_workspace_size(ctypes.byref(_layer(imatrix_in=sa)), 4096, 1)
    assert stats - plain >= (256 + 4096 * 6 // 128 + 1) * 4096 * 4
    assert (lib.ds4q_moe_workspace_size(ctypes.byref(_layer(imatrix_in=sa)), 1, 0)
            == lib.ds4q_moe_workspace_size(ctypes.byref(_layer()), 1, 0))


def test_steer_validation(lib):
    f = lib.ds4q_steer
    d, y, o = BASE, BASE + (1 << 30), BASE + (2 << 30)
    assert f(d, 1.0, y, 4, 4096, o, 0x2, None) == E_INVAL          # RMSNORM is not a steering flag
    assert f(d, 1.0, y, -1, 4096, o, 0, None) == E_SHAPE
    assert f(d, 1.0, y, 4, 4098, o, 0, None) == E_SHAPE            # n_embd % 4
    assert f(d, 1.0, y, 4, 0, o, 0, None) == E_SHAPE
    assert f(d, 1.0, y, 0, 4096, o, 0, None) == OK                 # nothing to do
    assert f(None, 1.0, y, 4, 4096, o, 0, None) == E_INVAL
    assert f(d, float("nan"), y, 4, 4096, o, 0, None) == E_INVAL
    assert f(d + 4, 1.0, y, 4, 4096, o, 0, None) == E_ALIGN
    assert f(d, 1.0, y, 4, 4096, d, 0, None) == E_ALIAS            # out over dir
    assert f(d, 1.0, y, 4, 4096, y + 16, 0, None) == E_ALIAS       # out partly over y


def test_codec_validation(lib):
    enc, dec = lib.ds4q_act_encode, lib.ds4q_act_decode
    s, t = BASE, BASE + (1 << 30)
    for f in (enc, dec):
        assert f(s, 1024, 12, t, None) == E_INVAL
        assert f(s, -1, 16, t, None) == E_SHAPE
        assert f(s, 0, 16, t, None) == OK
        assert f(None, 1024, 16, t, None) == E_INVAL
        assert f(s + 8, 1024, 16, t, None) == E_ALIGN
    assert enc(s, 1024, 16, s + 1024, None) == E_ALIAS             # dst inside src
    assert dec(s, 1024, 8, s + 512, None) == E_ALIAS
