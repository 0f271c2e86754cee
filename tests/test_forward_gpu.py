"""GPU parity of the full Gated MLA layer (mla_gated_forward): projections,
norms, the absorbed core and the output projection through the C ABI,
against the oracle's full-layer forward with bf16 storage of the stage
results, element by element (|gpu - oracle| <= 2e-2 on y)."""
import sys

import numpy as np
import pytest

import datagen as dg
import oracle
from gpu_util import assert_parity, oracle_forward, run_forward, sample_rows, to_host_f64

pytestmark = pytest.mark.gpu

# layer widths: the pages' toy and full K3 sizes, and an intermediate one
WIDTHS = {"toy": dict(D=256, q_rank=64, H=8, d_q=16, d_v=16, r=32),
          "mid": dict(D=1024, q_rank=384, H=32, d_q=64, d_v=64, r=256),
          "full": dict(D=7168, q_rank=1536, H=96, d_q=128, d_v=128, r=512)}


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


def _inputs(B, T, width, seed, eps=1e-6):
    w = WIDTHS[width]
    d = dg.forward_inputs(B, T, dtype=dg.BF16, seed=seed, **w)
    d["eps"] = eps
    d["scale"] = w["d_q"] ** -0.5
    return d


def test_forward_toy_workload(o):
    d = dg.workload_inputs("toy_forward")
    log("forward toy workload B=2 T=128")
    got = to_host_f64(run_forward(d))
    assert_parity(got, oracle_forward(o, d), dg.BF16, "forward toy")


@pytest.mark.parametrize("B,T,width", [(3, 77, "toy"), (1, 1, "toy"), (2, 130, "mid"), (1, 160, "full"),
                                       (2, 45, "full")])
def test_forward_bf16_ragged(o, B, T, width):
    """Row counts that leave partial 128-row GEMM tiles and 32-row attention
    tiles; toy widths also leave partial 128-column tiles (r = 32, q_rank = 64)."""
    d = _inputs(B, T, width, seed=7000 + 10 * B + T)
    log(f"forward {width} B={B} T={T}")
    got = to_host_f64(run_forward(d))
    assert_parity(got, oracle_forward(o, d), dg.BF16, f"forward {width} B{B} T{T}")


def test_forward_eps_and_zero_scale(o):
    """A large eps inside the norms and a zero softmax scale (uniform causal
    attention)."""
    d = _inputs(2, 70, "mid", seed=7100, eps=0.5)
    log("forward mid eps=0.5 scale=0")
    got = to_host_f64(run_forward(d, scale=0.0))
    assert_parity(got, oracle_forward(o, d, scale=0.0), dg.BF16, "forward eps 0.5 scale 0")


def test_forward_full_workload_sampled(o):
    """The whole layer at the full K3 widths, B=1, T=8192: sampled rows (the
    latent of every position is still formed by the oracle)."""
    d = dg.workload_inputs("full_forward")
    log("forward full workload B=1 T=8192 (sampled rows)")
    got = to_host_f64(run_forward(d)).reshape(d["B"] * d["T"], -1)
    rows = sample_rows(d["B"], d["T"], 6, seed=17)
    assert_parity(got[rows], oracle_forward(o, d, rows=rows), dg.BF16, "forward full sampled")


def test_forward_repeatable_and_workspace_reuse():
    """Two calls on the same inputs give identical bits, also when the
    workspace still holds an earlier, larger call's stages."""
    import torch
    import rank_latent_causal_amd as mla
    big = _inputs(2, 200, "mid", seed=7200)
    small = _inputs(1, 50, "mid", seed=7201)
    need = mla.forward_workspace_size(2, 200, 384, 32, 64, 64, 256, mla.DTYPE_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    args = lambda d: [torch.from_numpy(np.ascontiguousarray(d[k]).view(np.int16)).view(torch.bfloat16).cuda()
                      for k in dg.FORWARD_KEYS]
    mla.mla_gated_forward(*args(big), 1e-6, 0.125, workspace=ws)
    a = mla.mla_gated_forward(*args(small), 1e-6, 0.125, workspace=ws)
    b = mla.mla_gated_forward(*args(small), 1e-6, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
