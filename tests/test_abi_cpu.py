"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments before launching anything (no GPU is
touched: every call here fails validation on the host)."""
import ctypes as ct
import os
import re
import subprocess

import pytest

import rank_latent_causal_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in ("mla_absorb.h", "kda.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(mla.LIB_PATH), reason="libmla_absorb.so not built")

FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:mla|kda)_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_exactly_the_bound_functions():
    assert declared_functions() == sorted(mla.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ct.CDLL(mla.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T ((?:mla|kda)_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings():
    for s in range(5):
        assert mla.status_string(s).startswith(("MLA_OK", "MLA_ERR"))
    assert "UNKNOWN" in mla.status_string(99)


def test_prefill_workspace_sizes():
    assert mla.prefill_workspace_size(2, 128, 8, 16, 32, mla.DTYPE_F32) == 0
    n = mla.prefill_workspace_size(1, 8192, 96, 128, 512, mla.DTYPE_BF16)
    assert n >= 96 * 512 * 128 * 2 and n % 256 == 0
    with pytest.raises(mla.MLAError):
        mla.prefill_workspace_size(0, 1, 1, 16, 32, mla.DTYPE_BF16)


def test_unified_workspace_size():
    """mla_absorb_workspace_size(is_decode, B, T_or_max_len, H, r, dtype):
    prefill equals the explicit call with the d_q the compiled set pairs
    with r; fp32 needs none; sizes outside the set are rejected."""
    for r, dq in ((32, 16), (256, 64), (512, 128)):
        assert mla.workspace_size(False, 1, 8192, 96, r, mla.DTYPE_BF16) == \
            mla.prefill_workspace_size(1, 8192, 96, dq, r, mla.DTYPE_BF16)
    assert mla.workspace_size(False, 2, 128, 8, 32, mla.DTYPE_F32) == 0
    assert mla.workspace_size(True, 64, 32768, 96, 512, mla.DTYPE_F32) == 0
    for args in ((False, 1, 8, 4, 128, mla.DTYPE_BF16), (False, 0, 8, 4, 512, mla.DTYPE_BF16),
                 (True, 4, 0, 4, 512, mla.DTYPE_BF16), (False, 1, 8, 4, 512, 5)):
        with pytest.raises(mla.MLAError):
            mla.workspace_size(*args)
    # decode with the default split count queries the device: without one the
    # answer is the invalid size, with one it is the explicit call's
    try:
        n = mla.workspace_size(True, 64, 32768, 96, 512, mla.DTYPE_BF16)
    except mla.MLAError:
        return
    assert n == mla.decode_workspace_size(64, 96, 128, 512, 0, mla.DTYPE_BF16)


def test_decode_workspace_sizes_explicit_splits():
    assert mla.decode_workspace_size(64, 96, 128, 512, 256, mla.DTYPE_F32) == 0
    n = mla.decode_workspace_size(64, 96, 128, 512, 256, mla.DTYPE_BF16)
    # q_abs + (G+B) partial rows of r bf16 values + (m, l) in fp32
    assert n >= 64 * 96 * 512 * 2 + (256 + 64) * 96 * (512 * 2 + 2 * 4)
    assert mla.decode_workspace_size(64, 96, 128, 512, 512, mla.DTYPE_BF16) > n
    with pytest.raises(mla.MLAError):
        mla.decode_workspace_size(64, 96, 128, 512, 256, 7)


def _prefill(**kw):
    a = dict(q=FAKE, c=FAKE, w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, B=1, T=8, H=4, dq=128, dv=128,
             r=512, scale=0.1, dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return mla.lib().mla_absorb_prefill(a["q"], a["c"], a["w_uk"], a["w_uv"], a["gate"], a["out"], a["B"],
                                        a["T"], a["H"], a["dq"], a["dv"], a["r"], a["scale"], a["dtype"],
                                        a["ws"], a["wsb"], a["stream"])


def _decode(**kw):
    a = dict(q=FAKE, c=FAKE, cu=FAKE, w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, B=2, H=4, dq=128, dv=128,
             r=512, N=100, scale=0.1, splits=8, dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return mla.lib().mla_absorb_decode(a["q"], a["c"], a["cu"], a["w_uk"], a["w_uv"], a["gate"], a["out"],
                                       a["B"], a["H"], a["dq"], a["dv"], a["r"], a["N"], a["scale"],
                                       a["splits"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), mla.MLA_ERR_INVALID_ARG),
    (dict(out=None), mla.MLA_ERR_INVALID_ARG),
    (dict(c=FAKE + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(B=0), mla.MLA_ERR_INVALID_ARG),
    (dict(T=-3), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=5), mla.MLA_ERR_INVALID_ARG),
    (dict(dq=96, dv=96, r=384), mla.MLA_ERR_UNSUPPORTED),
    (dict(dv=64), mla.MLA_ERR_UNSUPPORTED),
    (dict(dtype=mla.DTYPE_F32, r=2048), mla.MLA_ERR_UNSUPPORTED),
    (dict(ws=None), mla.MLA_ERR_WORKSPACE),
    (dict(wsb=1024), mla.MLA_ERR_WORKSPACE),
    (dict(ws=FAKE + 4), mla.MLA_ERR_WORKSPACE),
])
def test_prefill_rejects(kw, status):
    assert _prefill(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), mla.MLA_ERR_INVALID_ARG),
    (dict(gate=FAKE + 2), mla.MLA_ERR_INVALID_ARG),
    (dict(H=0), mla.MLA_ERR_INVALID_ARG),
    (dict(N=1), mla.MLA_ERR_INVALID_ARG),          # fewer cache rows than sequences
    (dict(scale=float("-inf")), mla.MLA_ERR_INVALID_ARG),
    (dict(N=1 << 31), mla.MLA_ERR_UNSUPPORTED),
    (dict(H=256), mla.MLA_ERR_UNSUPPORTED),
    (dict(dq=64), mla.MLA_ERR_UNSUPPORTED),
    (dict(ws=None), mla.MLA_ERR_WORKSPACE),
    (dict(wsb=4096), mla.MLA_ERR_WORKSPACE),
])
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


def _extend(**kw):
    a = dict(q=FAKE, c=FAKE, w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, B=1, T=8, S=20, H=4, dq=128, dv=128,
             r=512, scale=0.1, dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return mla.lib().mla_absorb_extend(a["q"], a["c"], a["w_uk"], a["w_uv"], a["gate"], a["out"], a["B"],
                                       a["T"], a["S"], a["H"], a["dq"], a["dv"], a["r"], a["scale"],
                                       a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(S=7), mla.MLA_ERR_INVALID_ARG),           # fewer latent rows than queries
    (dict(T=0), mla.MLA_ERR_INVALID_ARG),
    (dict(c=None), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(dq=96, dv=96, r=384), mla.MLA_ERR_UNSUPPORTED),
    (dict(wsb=16), mla.MLA_ERR_WORKSPACE),
])
def test_extend_rejects(kw, status):
    assert _extend(**kw) == status


def test_forward_workspace_sizes():
    n = mla.forward_workspace_size(1, 8192, 1536, 96, 128, 128, 512, mla.DTYPE_BF16)
    rows = 8192
    # c, the query latent, q, gate, the gated core output and the core's W_UK^T
    assert n >= rows * (512 + 1536 + 3 * 96 * 128) * 2 + 96 * 512 * 128 * 2
    with pytest.raises(mla.MLAError):
        mla.forward_workspace_size(1, 8, 64, 8, 16, 16, 32, mla.DTYPE_F32)


def _forward(**kw):
    a = dict(x=FAKE, wkd=FAKE, kvn=FAKE, wqd=FAKE, qn=FAKE, wqu=FAKE, w_uk=FAKE, w_uv=FAKE, wg=FAKE, wo=FAKE,
             y=FAKE, B=1, T=8, D=7168, q_rank=1536, H=96, dq=128, dv=128, r=512, eps=1e-6, scale=0.1,
             dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return mla.lib().mla_gated_forward(a["x"], a["wkd"], a["kvn"], a["wqd"], a["qn"], a["wqu"], a["w_uk"],
                                       a["w_uv"], a["wg"], a["wo"], a["y"], a["B"], a["T"], a["D"], a["q_rank"],
                                       a["H"], a["dq"], a["dv"], a["r"], a["eps"], a["scale"], a["dtype"],
                                       a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mla.MLA_ERR_INVALID_ARG),
    (dict(wo=FAKE + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(T=0), mla.MLA_ERR_INVALID_ARG),
    (dict(eps=-1.0), mla.MLA_ERR_INVALID_ARG),
    (dict(eps=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=mla.DTYPE_F32), mla.MLA_ERR_UNSUPPORTED),
    (dict(D=7000), mla.MLA_ERR_UNSUPPORTED),          # not a multiple of 64
    (dict(q_rank=1500), mla.MLA_ERR_UNSUPPORTED),
    (dict(q_rank=4096), mla.MLA_ERR_UNSUPPORTED),     # beyond one wave's norm row
    (dict(dq=96, dv=96, r=384), mla.MLA_ERR_UNSUPPORTED),
    (dict(ws=None), mla.MLA_ERR_WORKSPACE),
    (dict(wsb=1 << 20), mla.MLA_ERR_WORKSPACE),
])
def test_forward_rejects(kw, status):
    assert _forward(**kw) == status


def _forward_train(**kw):
    a = dict(x=FAKE, wkd=FAKE, kvn=FAKE, wqd=FAKE, qn=FAKE, wqu=FAKE, w_uk=FAKE, w_uv=FAKE, wg=FAKE, wo=FAKE,
             y=FAKE, B=1, T=8, D=7168, q_rank=1536, H=96, dq=128, dv=128, r=512, eps=1e-6, scale=0.1,
             dtype=mla.DTYPE_BF16, st=FAKE, stb=1 << 40, stream=None)
    a.update(kw)
    return mla.lib().mla_gated_forward_train(a["x"], a["wkd"], a["kvn"], a["wqd"], a["qn"], a["wqu"], a["w_uk"],
                                             a["w_uv"], a["wg"], a["wo"], a["y"], a["B"], a["T"], a["D"],
                                             a["q_rank"], a["H"], a["dq"], a["dv"], a["r"], a["eps"], a["scale"],
                                             a["dtype"], a["st"], a["stb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mla.MLA_ERR_INVALID_ARG),
    (dict(y=FAKE + 2), mla.MLA_ERR_INVALID_ARG),
    (dict(B=0), mla.MLA_ERR_INVALID_ARG),
    (dict(eps=-1.0), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=mla.DTYPE_F32), mla.MLA_ERR_UNSUPPORTED),
    (dict(dtype=9), mla.MLA_ERR_INVALID_ARG),
    (dict(D=7000), mla.MLA_ERR_UNSUPPORTED),
    (dict(r=4096, dq=128), mla.MLA_ERR_UNSUPPORTED),
    (dict(st=None), mla.MLA_ERR_WORKSPACE),
    (dict(st=FAKE + 8), mla.MLA_ERR_WORKSPACE),
    (dict(stb=1 << 20), mla.MLA_ERR_WORKSPACE),
])
def test_forward_train_rejects(kw, status):
    assert _forward_train(**kw) == status


def _layer_backward(**kw):
    a = dict(x=FAKE, wkd=FAKE, kvn=FAKE, wqd=FAKE, qn=FAKE, wqu=FAKE, w_uk=FAKE, w_uv=FAKE, wg=FAKE, wo=FAKE,
             dy=FAKE, st=FAKE, stb=1 << 40, dx=FAKE, g=[FAKE] * 9, B=1, T=8, D=7168, q_rank=1536, H=96, dq=128,
             dv=128, r=512, scale=0.1, dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return mla.lib().mla_gated_backward(a["x"], a["wkd"], a["kvn"], a["wqd"], a["qn"], a["wqu"], a["w_uk"],
                                        a["w_uv"], a["wg"], a["wo"], a["dy"], a["st"], a["stb"], a["dx"], *a["g"],
                                        a["B"], a["T"], a["D"], a["q_rank"], a["H"], a["dq"], a["dv"], a["r"],
                                        a["scale"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), mla.MLA_ERR_INVALID_ARG),
    (dict(dx=None), mla.MLA_ERR_INVALID_ARG),
    (dict(g=[FAKE] * 8 + [None]), mla.MLA_ERR_INVALID_ARG),
    (dict(g=[FAKE + 4] + [FAKE] * 8), mla.MLA_ERR_INVALID_ARG),
    (dict(st=None), mla.MLA_ERR_INVALID_ARG),
    (dict(stb=1 << 20), mla.MLA_ERR_INVALID_ARG),
    (dict(T=0), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=mla.DTYPE_F32), mla.MLA_ERR_UNSUPPORTED),
    (dict(q_rank=1500), mla.MLA_ERR_UNSUPPORTED),
    (dict(dq=96, dv=96, r=384), mla.MLA_ERR_UNSUPPORTED),
    (dict(T=1 << 18), mla.MLA_ERR_UNSUPPORTED),       # token-major operands beyond 32-bit offsets
    (dict(ws=None), mla.MLA_ERR_WORKSPACE),
    (dict(wsb=1 << 20), mla.MLA_ERR_WORKSPACE),
    (dict(ws=FAKE + 8), mla.MLA_ERR_WORKSPACE),
])
def test_layer_backward_rejects(kw, status):
    assert _layer_backward(**kw) == status


def test_layer_training_sizes():
    B, T, D, qr, H, dq, dv, r = 1, 8192, 7168, 1536, 96, 128, 128, 512
    n = mla.train_state_size(B, T, qr, H, dq, dv, r, mla.DTYPE_BF16)
    # two copies of each norm's rows, q, gate, the core output, lse and the two 1/rms
    assert n >= T * (2 * (r + qr) + 3 * H * dq) * 2 + T * (H + 2) * 4
    w = mla.layer_backward_workspace_size(B, T, D, qr, H, dq, dv, r, mla.DTYPE_BF16)
    core = mla.backward_workspace_size(B, T, H, dq, dv, r, mla.DTYPE_BF16)
    assert w >= core + T * (H * dv + qr + r) * 2 + D * (H * dv + qr + r) * 2
    for f in (lambda: mla.train_state_size(B, T, qr, H, dq, dv, r, mla.DTYPE_F32),
              lambda: mla.layer_backward_workspace_size(B, 0, D, qr, H, dq, dv, r, mla.DTYPE_BF16)):
        with pytest.raises(mla.MLAError):
            f()


def test_paged_decode_workspace_size():
    n = mla.decode_paged_workspace_size(64, 96, 128, 512, 256, mla.DTYPE_BF16)
    # q_abs, (G+B) partials, then the clamped lengths and tile prefix sums
    # (B + B + 2 int32), which the packed decode holds as well
    assert n >= 64 * 96 * 512 * 2 + (256 + 64) * 96 * (512 * 2 + 2 * 4) + 4 * (2 * 64 + 2)
    assert n == mla.decode_workspace_size(64, 96, 128, 512, 256, mla.DTYPE_BF16)
    with pytest.raises(mla.MLAError):
        mla.decode_paged_workspace_size(64, 96, 128, 512, 256, mla.DTYPE_F32)


def _decode_paged(**kw):
    a = dict(q=FAKE, c=FAKE, bt=FAKE, lens=FAKE, w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, B=2, H=96, dq=128,
             dv=128, r=512, npg=100, ps=64, mp=10, scale=0.1, splits=8, dtype=mla.DTYPE_BF16, ws=FAKE,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return mla.lib().mla_absorb_decode_paged(a["q"], a["c"], a["bt"], a["lens"], a["w_uk"], a["w_uv"], a["gate"],
                                             a["out"], a["B"], a["H"], a["dq"], a["dv"], a["r"], a["npg"], a["ps"],
                                             a["mp"], a["scale"], a["splits"], a["dtype"], a["ws"], a["wsb"],
                                             a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), mla.MLA_ERR_INVALID_ARG),
    (dict(lens=FAKE + 4), mla.MLA_ERR_INVALID_ARG),
    (dict(ps=48), mla.MLA_ERR_INVALID_ARG),       # not a power of two
    (dict(ps=16), mla.MLA_ERR_INVALID_ARG),       # smaller than the 32-row tile
    (dict(ps=(1 << 30) + 1), mla.MLA_ERR_INVALID_ARG),  # above 2^30 and not a power of two
    (dict(ps=2 ** 31 - 1), mla.MLA_ERR_INVALID_ARG),    # the largest int: no unbounded search
    (dict(ps=1 << 30), mla.MLA_ERR_UNSUPPORTED),        # a power of two, but the pool overflows int32 rows
    (dict(npg=0), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=mla.DTYPE_F32), mla.MLA_ERR_UNSUPPORTED),
    (dict(H=200), mla.MLA_ERR_UNSUPPORTED),
    (dict(mp=1 << 26), mla.MLA_ERR_UNSUPPORTED),  # max_pages * page_size beyond int32
    (dict(ws=None), mla.MLA_ERR_WORKSPACE),
    (dict(wsb=4096), mla.MLA_ERR_WORKSPACE),
])
def test_decode_paged_rejects(kw, status):
    assert _decode_paged(**kw) == status


def _extend_paged(**kw):
    a = dict(q=FAKE, c=FAKE, bt=FAKE, w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, B=1, T=8, S=20, H=4, dq=128,
             dv=128, r=512, npg=10, ps=32, mp=4, scale=0.1, dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return mla.lib().mla_absorb_extend_paged(a["q"], a["c"], a["bt"], a["w_uk"], a["w_uv"], a["gate"], a["out"],
                                             a["B"], a["T"], a["S"], a["H"], a["dq"], a["dv"], a["r"], a["npg"],
                                             a["ps"], a["mp"], a["scale"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), mla.MLA_ERR_INVALID_ARG),
    (dict(S=200), mla.MLA_ERR_INVALID_ARG),       # more rows than max_pages * page_size
    (dict(ps=96), mla.MLA_ERR_INVALID_ARG),
    (dict(ps=2 ** 31 - 1), mla.MLA_ERR_INVALID_ARG),
    (dict(S=7), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=mla.DTYPE_F32), mla.MLA_ERR_UNSUPPORTED),
    (dict(dq=96, dv=96, r=384), mla.MLA_ERR_UNSUPPORTED),
    (dict(wsb=16), mla.MLA_ERR_WORKSPACE),
])
def test_extend_paged_rejects(kw, status):
    assert _extend_paged(**kw) == status


def _append(**kw):
    a = dict(c_new=FAKE, c=FAKE, bt=FAKE, pos=FAKE, B=2, r=512, npg=10, ps=64, mp=4, dtype=mla.DTYPE_BF16,
             stream=None)
    a.update(kw)
    return mla.lib().mla_cache_append_paged(a["c_new"], a["c"], a["bt"], a["pos"], a["B"], a["r"], a["npg"],
                                            a["ps"], a["mp"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(pos=None), mla.MLA_ERR_INVALID_ARG),
    (dict(c=FAKE + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(B=0), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=9), mla.MLA_ERR_INVALID_ARG),
    (dict(r=4), mla.MLA_ERR_UNSUPPORTED),          # 8-byte rows: not whole 16-byte chunks
    (dict(npg=1 << 31), mla.MLA_ERR_UNSUPPORTED),
])
def test_cache_append_rejects(kw, status):
    assert _append(**kw) == status


def _varlen(**kw):
    a = dict(q=FAKE, c=FAKE, bt=FAKE, cu=FAKE, lens=FAKE, w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, B=3, Nq=100, H=8,
             dq=128, dv=128, r=512, npg=64, ps=64, mp=8, scale=0.1, dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return mla.lib().mla_absorb_extend_varlen_paged(a["q"], a["c"], a["bt"], a["cu"], a["lens"], a["w_uk"], a["w_uv"],
                                                    a["gate"], a["out"], a["B"], a["Nq"], a["H"], a["dq"], a["dv"],
                                                    a["r"], a["npg"], a["ps"], a["mp"], a["scale"], a["dtype"], a["ws"],
                                                    a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), mla.MLA_ERR_INVALID_ARG),
    (dict(lens=FAKE + 4), mla.MLA_ERR_INVALID_ARG),
    (dict(Nq=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ps=100), mla.MLA_ERR_INVALID_ARG),
    (dict(ps=2 ** 31 - 1), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=mla.DTYPE_F32), mla.MLA_ERR_UNSUPPORTED),
    (dict(dq=96, dv=96, r=384), mla.MLA_ERR_UNSUPPORTED),
    (dict(ws=None), mla.MLA_ERR_WORKSPACE),
    (dict(wsb=1024), mla.MLA_ERR_WORKSPACE),
])
def test_extend_varlen_rejects(kw, status):
    assert _varlen(**kw) == status


def test_varlen_workspace_size():
    n = mla.varlen_workspace_size(4, 1000, 96, 128, 512, mla.DTYPE_BF16)
    assert n >= mla.prefill_workspace_size(1, 1, 96, 128, 512, mla.DTYPE_BF16) + 8 * (1000 // 16 + 4)
    with pytest.raises(mla.MLAError):
        mla.varlen_workspace_size(4, 1000, 96, 128, 512, mla.DTYPE_F32)


def test_kda_workspace_size():
    n = mla.kda_workspace_size(1, 8192, 96, 1, 128, 128)
    # per (batch, value head, 64 positions): W and q e^Gam [64][136], A_hat^T [128][72], Bm [64][72],
    # U^T [128][72] bf16 and the chunk decay [128] fp32
    assert n == 96 * 128 * (((2 * 64 * 136 + 128 * 72 + 64 * 72 + 128 * 72) * 2 + 128 * 4 + 255) // 256 * 256)
    assert mla.kda_workspace_size(2, 65, 4, 2, 16, 16) == 2 * 8 * 2 * mla.kda_workspace_size(1, 64, 1, 1, 16, 16)
    for bad in (dict(K=96, V=96), dict(K=128, V=64), dict(T=0), dict(G=0)):
        kw = dict(B=1, T=64, H=2, G=1, K=128, V=128)
        kw.update(bad)
        with pytest.raises(mla.MLAError):
            mla.kda_workspace_size(**kw)


def _kda(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, o=FAKE, sT=None, B=1, T=100, H=2, G=2, K=128,
             V=128, dtype=mla.DTYPE_BF16, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return mla.lib().kda_chunk_forward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["o"], a["sT"],
                                       a["B"], a["T"], a["H"], a["G"], a["K"], a["V"], a["dtype"], a["ws"],
                                       a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), mla.MLA_ERR_INVALID_ARG),
    (dict(beta=None), mla.MLA_ERR_INVALID_ARG),
    (dict(o=FAKE + 2), mla.MLA_ERR_INVALID_ARG),
    (dict(s0=FAKE + 4), mla.MLA_ERR_INVALID_ARG),
    (dict(sT=FAKE + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(T=0), mla.MLA_ERR_INVALID_ARG),
    (dict(G=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(dtype=mla.DTYPE_F32), mla.MLA_ERR_UNSUPPORTED),
    (dict(dtype=7), mla.MLA_ERR_INVALID_ARG),
    (dict(K=96, V=96), mla.MLA_ERR_UNSUPPORTED),
    (dict(K=128, V=64), mla.MLA_ERR_UNSUPPORTED),
    (dict(T=1 << 21, H=2, G=1), mla.MLA_ERR_UNSUPPORTED),   # one batch's g beyond 32-bit offsets
    (dict(ws=None), mla.MLA_ERR_WORKSPACE),
    (dict(ws=FAKE + 8), mla.MLA_ERR_WORKSPACE),
    (dict(wsb=1 << 12), mla.MLA_ERR_WORKSPACE),     # far below the 653 KB these sizes need
])
def test_kda_rejects(kw, status):
    assert _kda(**kw) == status


def _decode_noalloc(**kw):
    a = dict(q=FAKE, c=FAKE, cu=FAKE, w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, B=2, H=4, dq=128, dv=128,
             r=512, N=100, scale=0.1, splits=8, dtype=mla.DTYPE_BF16, stream=None)
    a.update(kw)
    return mla.lib().mla_absorb_decode_noalloc(a["q"], a["c"], a["cu"], a["w_uk"], a["w_uv"], a["gate"], a["out"],
                                               a["B"], a["H"], a["dq"], a["dv"], a["r"], a["N"], a["scale"],
                                               a["splits"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), mla.MLA_ERR_INVALID_ARG),
    (dict(c=FAKE + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(N=1), mla.MLA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(dq=96, dv=96, r=384), mla.MLA_ERR_UNSUPPORTED),
    # scratch beyond the static buffer: rejected before the buffer is looked up
    (dict(B=300, H=96, N=1000, splits=256), mla.MLA_ERR_WORKSPACE),
    (dict(B=2, H=96, N=1000, splits=1 << 20), mla.MLA_ERR_WORKSPACE),
])
def test_decode_noalloc_rejects(kw, status):
    assert _decode_noalloc(**kw) == status


def test_decode_noalloc_limit_matches_workspace_size():
    """The largest default-split batch the static buffer serves at full width
    is the one whose explicit workspace still fits in it."""
    limit = 64 << 20
    fits = [B for B in range(1, 400) if mla.decode_workspace_size(B, 96, 128, 512, 256, mla.DTYPE_BF16) <= limit]
    assert fits and max(fits) >= 128
    B = max(fits) + 1
    assert _decode_noalloc(B=B, H=96, N=10 * B, splits=256) == mla.MLA_ERR_WORKSPACE
