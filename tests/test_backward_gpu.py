"""GPU parity of the training path: the forward's log-sum-exp and the
backward of the prefill core, through the C ABI, against the oracle.

The backward is fed the oracle's forward output (rounded to bf16) and
log-sum-exp, so the comparison measures the backward alone.  Tolerance (bf16
operands, fp32 accumulation), per gradient tensor (assert_tensor_close):
  * relative Frobenius error ||gpu - oracle|| / ||oracle|| at most 1e-2 for
    the whole tensor, and at most 2e-2 for every token row and every head
    on its own (dq and dgate by row and by head, dc by row, dW_UK and dW_UV
    by head);
  * a slice whose exact norm is below half a typical slice's is held to an
    absolute bar instead: 1% of a typical slice's norm, and 2^-5 of it for
    the query gradient's rows.
The chain rounds q_abs, dol, P, dS, c and the stored da / ol to bf16, each at
most 2^-9 relative, so a term carries about 1% relative error and a long sum
less: measured, whole tensors stay below 5e-3 and slices below 1e-2.  The
query gradient of the first positions is the exception: dS = P (dP - D) is
a difference of two values near 7 at full width, against an exact zero at
t = 0 (one key) and a small difference for the next few rows, so those rows
carry the rounding of D itself (2^-8 |D| per key, not reduced by the small
true value): measured up to 1.9% of a typical row's norm.  One wrong head,
or a few wrong rows, of a large tensor fail the slice bars although they
barely move the whole-tensor error.  The log-sum-exp is
compared at 2e-2 absolute (it is formed from bf16 q_abs).
"""
import sys

import numpy as np
import pytest

import datagen as dg
import oracle
from gpu_util import assert_tensor_close, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

SHAPES = {"toy": (16, 16, 32), "mid": (64, 64, 256), "full": (128, 128, 512)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_causal_amd as mla
    mla.lib()
    return torch


def core_grad_slices(k: str, shape, H: int):
    """Rows (token positions) and heads of each gradient of the core."""
    if k == "dgate":  # [B, T, H*d_v]
        BT, W = shape[0] * shape[1], shape[2]
        return [("row", (BT, W), (0,)), ("head", (BT, H, W // H), (1,))]
    if k == "dq":  # [B, T, H, d_q]
        BT = shape[0] * shape[1]
        return [("row", (BT, shape[2] * shape[3]), (0,)), ("head", (BT, shape[2], shape[3]), (1,))]
    if k == "dc":  # [B, T, r]
        return [("row", (shape[0] * shape[1], shape[2]), (0,))]
    return [("head", None, (0,))]  # dw_uk [H, d_q, r], dw_uv [H, d_v, r]


# the query gradient of the first positions is a small difference (see above)
DQ_NEAR_ZERO = 2.0 ** -5


def _grad_close(got, ref, what, k, H):
    near = {"row": DQ_NEAR_ZERO} if k == "dq" else None
    return assert_tensor_close(got, ref, what, core_grad_slices(k, np.shape(ref), H), near_zero=near)


def _case(B, T, H, shape, seed):
    dq, dv, r = SHAPES[shape]
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.BF16, seed=seed)
    d["scale"] = dq ** -0.5
    dout = dg.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((B, T, H * dv)).astype(np.float32))
    return d, dout


def test_train_forward_lse(o):
    """The training forward's output is the plain forward's, bit for bit, and
    its log-sum-exp matches the oracle's."""
    import torch
    import rank_latent_causal_amd as mla
    for (B, T, H, shape) in [(2, 77, 3, "toy"), (1, 130, 5, "mid"), (2, 70, 9, "full")]:
        d, _ = _case(B, T, H, shape, seed=9000 + T)
        args = [to_dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
        out, lse = mla.mla_absorb_prefill_train(*args, d["scale"])
        ref_out = mla.mla_absorb_prefill(*args, d["scale"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"{shape}: training forward output differs"
        f = dg.as_f32
        want = o.prefill_lse(f(d["q"]), f(d["c"]), f(d["w_uk"]), d["scale"])
        got = lse.cpu().numpy().astype(np.float64)
        err = np.abs(got - want).max()
        assert err <= 2e-2, f"{shape}: lse max err {err:.3g}"


@pytest.mark.parametrize("B,T,H,shape", [
    (2, 100, 3, "toy"),
    (1, 33, 2, "toy"),
    (1, 130, 5, "mid"),
    (2, 70, 9, "full"),
    (1, 200, 8, "full"),
    (1, 64, 96, "full"),
])
def test_backward_parity(o, B, T, H, shape):
    import torch
    import rank_latent_causal_amd as mla
    d, dout = _case(B, T, H, shape, seed=9100 + 7 * T + H)
    f = dg.as_f32
    args64 = [f(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    ref_out = o.prefill(*args64, d["scale"])
    ref_lse = o.prefill_lse(f(d["q"]), f(d["c"]), f(d["w_uk"]), d["scale"])
    want = o.prefill_backward(*args64, f(dout), d["scale"])
    log(f"backward {shape} B={B} T={T} H={H}")
    out_b = dg.f32_to_bf16_bits(ref_out.astype(np.float32))
    g = mla.mla_absorb_prefill_backward(*[to_dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")], to_dev(out_b),
                                        to_dev(ref_lse.astype(np.float32)), to_dev(dout), d["scale"])
    torch.cuda.synchronize()
    for k in ("dgate", "dq", "dc", "dw_uk", "dw_uv"):
        _grad_close(to_host_f64(g[k]), want[k], f"{k} ({shape} B{B} T{T} H{H})", k, H)


def test_backward_workspace_reuse_and_repeat():
    """Two calls on the same inputs give identical bits, also after a larger
    call has left its intermediates in the workspace."""
    import torch
    import rank_latent_causal_amd as mla
    big, dbig = _case(2, 150, 5, "mid", seed=9200)
    small, dsmall = _case(1, 60, 5, "mid", seed=9201)
    ws = torch.empty(mla.backward_workspace_size(2, 150, 5, 64, 64, 256, mla.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")

    def run(d, dout, workspace=None):
        args = [to_dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
        out, lse = mla.mla_absorb_prefill_train(*args, d["scale"])
        return mla.mla_absorb_prefill_backward(*args, out, lse, to_dev(dout), d["scale"], workspace=workspace)

    run(big, dbig, ws)
    a = run(small, dsmall, ws)
    b = run(small, dsmall)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("B,T,H,shape", [(1, 1, 8, "toy"), (1, 33, 3, "full"), (2, 1, 5, "mid")])
def test_backward_poisoned_workspace(o, B, T, H, shape):
    """Every workspace byte set to 0xFF (NaN in bf16 and fp32) before the
    call: a read of a byte the call did not write first shows up as a
    non-finite or wrong gradient.  The last query block holds an odd number
    of rows here, where the staged {lse, D} pairs end mid-copy.  At T = 1 the
    single key's softmax weight is 1 whatever the score, so dq and dW_UK are
    exactly zero in the oracle and rounding noise of P (dP - D) in the
    library: they must be finite and under 2^-7 of the size dq has at the
    same inputs' T = 2; the other gradients meet the usual bar."""
    import torch
    import rank_latent_causal_amd as mla
    d, dout = _case(B, T, H, shape, seed=9300 + T + H)
    dq_, dv_, r_ = SHAPES[shape]
    ws = torch.full((mla.backward_workspace_size(B, T, H, dq_, dv_, r_, mla.DTYPE_BF16),), 255, dtype=torch.uint8,
                    device="cuda")
    f = dg.as_f32
    args64 = [f(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    ref_out = o.prefill(*args64, d["scale"])
    ref_lse = o.prefill_lse(f(d["q"]), f(d["c"]), f(d["w_uk"]), d["scale"])
    want = o.prefill_backward(*args64, f(dout), d["scale"])
    log(f"backward poisoned workspace {shape} B={B} T={T} H={H}")
    out_b = dg.f32_to_bf16_bits(ref_out.astype(np.float32))
    g = mla.mla_absorb_prefill_backward(*[to_dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")], to_dev(out_b),
                                        to_dev(ref_lse.astype(np.float32)), to_dev(dout), d["scale"], workspace=ws)
    torch.cuda.synchronize()
    for k in ("dgate", "dq", "dc", "dw_uk", "dw_uv"):
        got = to_host_f64(g[k])
        assert np.all(np.isfinite(got)), f"{k}: non-finite values"
        if T == 1 and k in ("dq", "dw_uk"):
            assert np.all(want[k] == 0.0), f"oracle {k} at T=1 is not zero"
            continue
        _grad_close(got, want[k], f"{k} ({shape} B{B} T{T} H{H}, poisoned workspace)", k, H)
    if T == 1:
        # the query-side noise against the size of dq one position later
        d2, dout2 = _case(B, 2, H, shape, seed=9300 + T + H)
        want2 = o.prefill_backward(*[f(d2[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")], f(dout2), d2["scale"])
        for k in ("dq", "dw_uk"):
            noise = np.linalg.norm(to_host_f64(g[k]))
            assert noise <= 2.0 ** -7 * np.linalg.norm(want2[k]), f"{k}: T=1 noise {noise:.3g}"
