"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, plus structural invariants that
hold at any size."""
import sys

import numpy as np
import pytest

import datagen as dg
import oracle
from gpu_util import (assert_parity, oracle_decode, oracle_extend, oracle_prefill, run_decode, run_extend,
                      run_prefill, sample_rows, to_dev, to_host_f64)

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
    mla.lib()  # loud failure if the HIP library is missing
    return torch


# ------------------------------------------------------------------ prefill
def test_prefill_toy_f32_workload(o):
    d = dg.workload_inputs("toy_f32")
    log(f"prefill toy_f32 B={d['B']} T={d['T']} H={d['H']}")
    got = to_host_f64(run_prefill(d))
    assert_parity(got, oracle_prefill(o, d), dg.F32, "toy_f32", block=d["d_v"])


@pytest.mark.parametrize("B,T,H,shape", [
    (1, 1, 1, "toy"), (2, 37, 3, "toy"), (3, 100, 5, "toy"),
    (1, 45, 2, "mid"), (2, 97, 9, "mid"), (1, 300, 3, "mid"),
    (1, 33, 1, "full"), (2, 70, 5, "full"), (1, 130, 8, "full"),
])
def test_prefill_bf16_ragged(o, B, T, H, shape):
    dq, dv, r = SHAPES[shape]
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.BF16, seed=1000 + B * 7 + T + H)
    d["scale"] = dq ** -0.5
    log(f"prefill bf16 B={B} T={T} H={H} dq={dq} r={r}")
    got = to_host_f64(run_prefill(d))
    assert_parity(got, oracle_prefill(o, d), dg.BF16, f"prefill {shape} B{B} T{T} H{H}", block=d["d_v"])


@pytest.mark.parametrize("B,T,H,shape", [(1, 40, 4, "full"), (2, 50, 3, "toy")])
def test_prefill_f32_other_shapes(o, B, T, H, shape):
    dq, dv, r = SHAPES[shape]
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=2000 + T)
    log(f"prefill f32 B={B} T={T} H={H} r={r}")
    got = to_host_f64(run_prefill(d, scale=0.3))
    assert_parity(got, oracle_prefill(o, d, scale=0.3), dg.F32, f"prefill f32 {shape}", block=d["d_v"])


def test_prefill_toy_max_workload(o):
    d = dg.workload_inputs("toy_max")
    log("prefill toy_max B=4 T=2048 H=8")
    got = to_host_f64(run_prefill(d))
    assert_parity(got, oracle_prefill(o, d), dg.BF16, "toy_max", block=d["d_v"])


def test_prefill_mid_workload_sampled(o):
    d = dg.workload_inputs("mid")
    log("prefill mid B=4 T=4096 H=32 (sampled rows)")
    got = to_host_f64(run_prefill(d)).reshape(d["B"] * d["T"], -1)
    rows = sample_rows(d["B"], d["T"], 6, seed=5)
    assert_parity(got[rows], oracle_prefill(o, d, rows=rows), dg.BF16, "mid sampled", block=d["d_v"])


def test_prefill_full_workload_sampled(o):
    d = dg.workload_inputs("full_prefill")
    log("prefill full B=1 T=8192 H=96 (sampled rows)")
    got = to_host_f64(run_prefill(d)).reshape(d["B"] * d["T"], -1)
    rows = sample_rows(d["B"], d["T"], 6, seed=6)
    assert_parity(got[rows], oracle_prefill(o, d, rows=rows), dg.BF16, "full sampled", block=d["d_v"])


@pytest.mark.parametrize("B,T,H,shape", [(1, 130, 5, "mid"), (2, 300, 16, "mid"), (2, 70, 9, "full"), (1, 520, 24, "full")])
def test_prefill_deterministic(B, T, H, shape):
    """Repeated calls give the same bits.  Work items go to whichever
    workgroup starts next, so an item lands on a different CU from call to
    call; with other GPU work in between, a read of LDS or registers that
    the item did not write itself (or a missed hazard) shows up here as a
    run-to-run difference."""
    import torch
    dq, dv, r = SHAPES[shape]
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.BF16, seed=4400 + T + H)
    d["scale"] = dq ** -0.5
    log(f"prefill determinism B={B} T={T} H={H} r={r}")
    first = run_prefill(d)
    for rep in range(4):
        torch.randn(1 << 22, device="cuda").sum()  # other work between the calls
        again = run_prefill(d)
        n = int((again != first).sum().item())
        assert n == 0, f"call {rep + 1} differs from call 0 in {n} elements"


@pytest.mark.parametrize("shape", ["mid", "full"])
def test_prefill_poisoned_workspace(shape):
    """The r = 256 / 512 prefill takes its work items from a counter in the
    workspace that the call clears before its kernel starts: a workspace full
    of 0xFF bytes (the counter far out of range), and the same workspace
    reused by a second call, give the bits of a call with a fresh one."""
    import torch
    import rank_latent_causal_amd as mla
    dq, dv, r = SHAPES[shape]
    B, T, H = 2, 200, 12
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.BF16, seed=4700 + r)
    d["scale"] = dq ** -0.5
    log(f"prefill poisoned workspace B={B} T={T} H={H} r={r}")
    args = [to_dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    ref = mla.mla_absorb_prefill(*args, d["scale"])
    n = mla.prefill_workspace_size(B, T, H, dq, r, mla.DTYPE_BF16)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    first = mla.mla_absorb_prefill(*args, d["scale"], workspace=ws)
    second = mla.mla_absorb_prefill(*args, d["scale"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, ref), "poisoned workspace changed the result"
    assert torch.equal(second, ref), "a reused workspace changed the result"


def test_prefill_first_position_closed_form():
    """t = 0 sees only its own latent: out = sigmoid(g) * (c_0 W_UV^T) for any
    q and scale (checked on the GPU output alone, at the full width)."""
    d = dg.prefill_inputs(2, 64, 8, 128, 128, 512, dtype=dg.BF16, seed=3)
    got = to_host_f64(run_prefill(d, scale=5.0))
    c0 = dg.as_f32(d["c"])[:, 0].astype(np.float64)
    wuv = dg.as_f32(d["w_uv"]).astype(np.float64)
    g = dg.as_f32(d["gate"])[:, 0].astype(np.float64)
    ref = np.einsum("bj,hvj->bhv", c0, wuv).reshape(2, -1) / (1 + np.exp(-g))
    assert_parity(got[:, 0], ref, dg.BF16, "t=0 closed form", block=d["d_v"])


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("lens,H,shape,splits", [
    ([1], 4, "toy", 1),
    ([5, 1, 40, 33, 64], 8, "toy", 3),
    ([100, 7, 250], 32, "mid", 0),
    ([31, 32, 33, 1, 200], 96, "full", 4),
    ([300, 1, 129], 96, "full", 0),
    ([1000, 17, 513, 64], 40, "full", 7),
    ([1] * 37 + [45, 2], 96, "full", 3),  # tiles holding dozens of one-row sequences
    ([65, 300], 128, "full", 0),          # the largest head count of one workgroup
    ([300, 77, 1000], 80, "full", 0),     # a partial third group of 32 heads
])
def test_decode_bf16_ragged(o, lens, H, shape, splits):
    dq, dv, r = SHAPES[shape]
    d = dg.decode_inputs(len(lens), H, dq, dv, r, dtype=dg.BF16, seed=3000 + sum(lens), lengths=lens)
    d["scale"] = dq ** -0.5
    log(f"decode bf16 lens={lens} H={H} r={r} splits={splits}")
    got = to_host_f64(run_decode(d, num_splits=splits))
    assert_parity(got, oracle_decode(o, d), dg.BF16, f"decode {shape} {lens}", block=d["d_v"])


def test_decode_f32(o):
    d = dg.decode_inputs(3, 8, 16, 16, 32, dtype=dg.F32, seed=4000, lengths=[9, 1, 130])
    log("decode f32 toy")
    got = to_host_f64(run_decode(d, scale=1.0))
    assert_parity(got, oracle_decode(o, d, scale=1.0), dg.F32, "decode f32", block=d["d_v"])


def test_decode_split_count_invariance():
    d = dg.decode_inputs(4, 96, 128, 128, 512, dtype=dg.BF16, seed=4100, lengths=[700, 3, 1500, 64])
    d["scale"] = 128 ** -0.5
    log("decode split invariance")
    outs = [to_host_f64(run_decode(d, num_splits=s)) for s in (1, 2, 5, 64, 256)]
    for s, x in zip((2, 5, 64, 256), outs[1:]):
        assert_parity(x, outs[0], dg.BF16, f"splits={s} vs 1", block=d["d_v"])


def test_decode_matches_prefill_last_row():
    """Decode over a cache of len rows equals prefill row len - 1, both on the
    GPU (same inputs laid out both ways)."""
    B, T, H = 3, 96, 16
    d = dg.prefill_inputs(B, T, H, 128, 128, 512, dtype=dg.BF16, seed=4200)
    d["scale"] = 128 ** -0.5
    lens = np.array([96, 1, 50])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dd = dict(q=np.stack([d["q"][i, lens[i] - 1] for i in range(B)]),
              c_cache=np.concatenate([d["c"][i, :lens[i]] for i in range(B)]),
              cu_seqlens=cu, w_uk=d["w_uk"], w_uv=d["w_uv"],
              gate=np.stack([d["gate"][i, lens[i] - 1] for i in range(B)]), scale=d["scale"])
    log("decode vs prefill last row")
    pre = to_host_f64(run_prefill(d))
    dec = to_host_f64(run_decode(dd))
    ref = np.stack([pre[i, lens[i] - 1] for i in range(B)])
    assert_parity(dec, ref, dg.BF16, "decode vs prefill last row", block=128)


def test_decode_full_workload_sampled(o):
    d = dg.workload_inputs("full_decode")
    log(f"decode full B=64 total={int(d['cu_seqlens'][-1])} (sampled sequences)")
    got = to_host_f64(run_decode(d))
    seqs = np.array([0, 1, int(np.argmin(d["lengths"])), int(np.argmax(d["lengths"])), 31, 63], dtype=np.int64)
    assert_parity(got[seqs], oracle_decode(o, d, seqs=seqs), dg.BF16, "full decode sampled", block=d["d_v"])


# ------------------------------------------------------------------ edges
@pytest.mark.parametrize("scale", [0.0, 0.35])
def test_prefill_scale_extremes(o, scale):
    """scale 0 (uniform weights over the prefix) and four times the default
    1/sqrt(d_q) (a peakier softmax).  Far larger scales leave the bf16
    regime: q_abs is rounded to bf16 for the MFMA, and a very peaky softmax
    turns that rounding into weight shifts between near-tied keys."""
    d = dg.prefill_inputs(1, 200, 4, 128, 128, 512, dtype=dg.BF16, seed=5100)
    log(f"prefill full width scale={scale}")
    got = to_host_f64(run_prefill(d, scale=scale))
    assert_parity(got, oracle_prefill(o, d, scale=scale), dg.BF16, f"prefill scale={scale}", block=d["d_v"])


def test_prefill_running_max_rescale():
    """Early latent rows shrunk (ramping to full size by position 100) with
    four times the default scale: the running max jumps by more than 8
    (log2 units) after the first tile on most query rows, so the
    accumulator rescale runs, while outputs stay at unit scale."""
    o = oracle.get()
    T = 300
    d = dg.prefill_inputs(1, T, 4, 128, 128, 512, dtype=dg.BF16, seed=5150)
    ramp = np.minimum(1.0, 0.02 + np.arange(T, dtype=np.float32) / 100.0)[None, :, None]
    d["c"] = dg.f32_to_bf16_bits(dg.as_f32(d["c"]) * ramp)
    log("prefill ramped latent (rescale path)")
    got = to_host_f64(run_prefill(d, scale=0.35))
    assert_parity(got, oracle_prefill(o, d, scale=0.35), dg.BF16, "prefill rescale path", block=d["d_v"])


def test_prefill_long_sequence_sampled(o):
    """T well beyond the full workload with a ragged last tile; rows at the
    ends and around tile boundaries."""
    T = 20001
    d = dg.prefill_inputs(1, T, 2, 128, 128, 512, dtype=dg.BF16, seed=5200)
    d["scale"] = 128 ** -0.5
    log(f"prefill long T={T} H=2 (sampled rows)")
    got = to_host_f64(run_prefill(d)).reshape(T, -1)
    rows = np.array([0, 1, 31, 32, 33, 4095, 4096, 9999, 19967, 19968, 19999, 20000], dtype=np.int64)
    assert_parity(got[rows], oracle_prefill(o, d, rows=rows), dg.BF16, "long prefill sampled", block=d["d_v"])


def test_decode_long_sequence(o):
    """One sequence much longer than any range next to a three-row one."""
    d = dg.decode_inputs(2, 8, 128, 128, 512, dtype=dg.BF16, seed=5300, lengths=[150000, 3])
    d["scale"] = 128 ** -0.5
    log("decode long sequence 150000 + 3 rows")
    got = to_host_f64(run_decode(d))
    assert_parity(got, oracle_decode(o, d), dg.BF16, "decode long sequence", block=d["d_v"])


@pytest.mark.parametrize("H,scale", [(32, 0.35), (96, 0.25)])
def test_decode_running_max_rescale(o, H, scale):
    """Cache rows that grow from 2% to full size over each sequence's first
    300 rows, with three to four times the default scale: inside a
    workgroup's range the running max moves by more than 8 (log2 units;
    by 17 to 25 over the first and last sequence) after the first tiles, so
    the accumulator rescale runs, and again after each sequence switch.  At
    H = 96 the factors go from the softmax waves to the other waves; the
    smaller scale there keeps the sharpest of the 96 heads' distributions
    within the per-head bar (bf16 P, 8 significant bits)."""
    lens = [3000, 40, 1500]
    d = dg.decode_inputs(3, H, 128, 128, 512, dtype=dg.BF16, seed=5350, lengths=lens)
    u = np.concatenate([np.arange(n) for n in lens]).astype(np.float32)
    ramp = np.minimum(1.0, 0.02 + u / 300.0)[:, None]
    d["c_cache"] = dg.f32_to_bf16_bits(dg.as_f32(d["c_cache"]) * ramp)
    log(f"decode ramped cache (rescale path) H={H} scale={scale}, 2 splits")
    got = to_host_f64(run_decode(d, scale=scale, num_splits=2))
    assert_parity(got, oracle_decode(o, d, scale=scale), dg.BF16, "decode rescale path", block=d["d_v"])


def test_side_stream_and_workspace_reuse():
    """Calls enqueued on a non-default stream with a caller workspace reused
    across shapes give the same bits as default-stream calls."""
    import torch
    import rank_latent_causal_amd as mla
    from gpu_util import to_dev
    d = dg.prefill_inputs(2, 150, 6, 128, 128, 512, dtype=dg.BF16, seed=5400)
    e = dg.decode_inputs(3, 20, 128, 128, 512, dtype=dg.BF16, seed=5401, lengths=[700, 2, 90])
    P = [to_dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    D = [to_dev(e[k]) for k in ("q", "c_cache", "cu_seqlens", "w_uk", "w_uv", "gate")]
    ref_p = mla.mla_absorb_prefill(*P, 0.1)
    ref_d = mla.mla_absorb_decode(*D, 0.1)
    torch.cuda.synchronize()
    n = max(mla.prefill_workspace_size(2, 150, 6, 128, 512, mla.DTYPE_BF16),
            mla.decode_workspace_size(3, 20, 128, 512, 0, mla.DTYPE_BF16))
    ws = torch.empty(n + 4096, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    log("side stream + shared workspace")
    with torch.cuda.stream(side):
        out_p = mla.mla_absorb_prefill(*P, 0.1, workspace=ws, stream=side)
        out_d = mla.mla_absorb_decode(*D, 0.1, workspace=ws, stream=side)
    side.synchronize()
    assert torch.equal(out_p, ref_p) and torch.equal(out_d, ref_d)


# ------------------------------------------------------------------ chunked prefill
@pytest.mark.parametrize("B,T,S,H,shape", [
    (1, 1, 1, 1, "toy"), (2, 37, 100, 3, "toy"),
    (1, 45, 45, 2, "mid"), (2, 30, 161, 9, "mid"),
    (2, 70, 200, 5, "full"), (1, 33, 1000, 8, "full"), (3, 1, 77, 4, "full"), (1, 130, 131, 8, "full"),
])
def test_extend_bf16_ragged(o, B, T, S, H, shape):
    dq, dv, r = SHAPES[shape]
    d = dg.prefill_inputs(B, S, H, dq, dv, r, dtype=dg.BF16, seed=6000 + B * 7 + T + S + H)
    d["scale"] = dq ** -0.5
    log(f"extend bf16 B={B} T={T} S={S} H={H} r={r}")
    got = to_host_f64(run_extend(d, T))
    assert_parity(got, oracle_extend(o, d, T), dg.BF16, f"extend {shape} B{B} T{T} S{S} H{H}", block=d["d_v"])


def test_extend_f32(o):
    d = dg.prefill_inputs(2, 61, 3, 16, 16, 32, dtype=dg.F32, seed=6100)
    log("extend f32 toy T=20 S=61")
    got = to_host_f64(run_extend(d, 20, scale=0.7))
    assert_parity(got, oracle_extend(o, d, 20, scale=0.7), dg.F32, "extend f32", block=d["d_v"])


def test_extend_without_prefix_is_prefill():
    """S == T runs the prefill path: identical bits."""
    d = dg.prefill_inputs(2, 90, 6, 128, 128, 512, dtype=dg.BF16, seed=6200)
    d["scale"] = 128 ** -0.5
    log("extend S == T vs prefill")
    import torch
    assert torch.equal(run_extend(d, 90), run_prefill(d))


def test_extend_full_width_sampled(o):
    """A 2048-query chunk after 6144 cached positions at the full widths."""
    S, T = 8192, 2048
    d = dg.prefill_inputs(1, S, 96, 128, 128, 512, dtype=dg.BF16, seed=6300)
    d["scale"] = 128 ** -0.5
    log(f"extend full width T={T} S={S} H=96 (sampled rows)")
    got = to_host_f64(run_extend(d, T)).reshape(T, -1)
    rows = sample_rows(1, T, 4, seed=7)
    assert_parity(got[rows], oracle_extend(o, d, T, rows=rows), dg.BF16, "extend full sampled", block=d["d_v"])
