"""mla_absorb_decode_noalloc (the decode call with its scratch in the
library's static per-GPU buffer, for callers that cannot allocate) against
mla_absorb_decode on the same inputs: two calls in a row, the second with
a smaller batch, so the second runs on scratch the first left behind.
Collected last (the module name starts with test_zz)."""
import sys

import numpy as np
import pytest

import datagen as dg
from gpu_util import assert_parity, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_causal_amd as mla
    mla.lib()
    return torch


def _args(d):
    return [to_dev(d[k]) for k in ("q", "c_cache", "cu_seqlens", "w_uk", "w_uv", "gate")]


@pytest.mark.parametrize("splits", [0, 7])
def test_decode_noalloc_matches_decode(splits):
    import torch
    import rank_latent_causal_amd as mla
    big = dg.decode_inputs(6, 96, 128, 128, 512, dtype=dg.BF16, seed=9900 + splits,
                           lengths=[3000, 1, 517, 64, 2048, 33])
    small = dg.decode_inputs(3, 40, 128, 128, 512, dtype=dg.BF16, seed=9901 + splits, lengths=[100, 7, 1])
    for name, d in (("first (6 sequences, H=96)", big), ("second (3 sequences, H=40)", small)):
        log(f"decode noalloc {name}, splits={splits}")
        A = _args(d)
        scale = 128 ** -0.5
        ref = mla.mla_absorb_decode(*A, scale, num_splits=splits)
        out = torch.empty_like(ref)
        got = mla.mla_absorb_decode_noalloc(*A, scale, num_splits=splits, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert_parity(to_host_f64(got), to_host_f64(ref), dg.BF16, f"noalloc vs decode: {name}", block=128)
        # same kernels, same split: the same bits
        assert torch.equal(got, ref), f"{name}: noalloc output differs from mla_absorb_decode"


def test_decode_noalloc_f32():
    """fp32 decode needs no scratch; the call still runs and matches."""
    import torch
    import rank_latent_causal_amd as mla
    d = dg.decode_inputs(3, 8, 16, 16, 32, dtype=dg.F32, seed=9910, lengths=[9, 1, 130])
    A = _args(d)
    ref = mla.mla_absorb_decode(*A, 0.5)
    got = mla.mla_absorb_decode_noalloc(*A, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
