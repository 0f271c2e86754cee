"""GPU parity of the paged latent cache paths: decode and chunked prefill
over shuffled pages (NaN in every slot no sequence owns, so a read past a
sequence's rows would show), and the cache append, through the C ABI against
the oracle's paged functions."""
import sys

import numpy as np
import pytest

import datagen as dg
import oracle
from gpu_util import assert_parity, to_dev, to_host_f64

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


def _paged_decode_case(lens, H, shape, page_size, seed):
    dq, dv, r = SHAPES[shape]
    d = dg.decode_inputs(len(lens), H, dq, dv, r, dtype=dg.BF16, seed=seed, lengths=lens)
    d["scale"] = dq ** -0.5
    lay = dg.paged_layout(d["lengths"], page_size, seed=seed)
    pool = dg.scatter_to_pages(d["c_cache"], d["cu_seqlens"], lay)
    return d, lay, pool


def _run_decode_paged(d, lay, pool, lens=None, num_splits=0):
    import torch
    import rank_latent_causal_amd as mla
    lens = d["lengths"] if lens is None else lens
    out = mla.mla_absorb_decode_paged(to_dev(d["q"]), to_dev(pool), to_dev(lay["block_table"]),
                                      to_dev(np.asarray(lens, dtype=np.int32)), to_dev(d["w_uk"]), to_dev(d["w_uv"]),
                                      to_dev(d["gate"]), d["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return to_host_f64(out)


def _oracle_decode_paged(o, d, lay, pool, lens=None, seqs=None):
    f = dg.as_f32
    lens = d["lengths"] if lens is None else lens
    return o.decode_paged(f(d["q"]), f(pool), lay["block_table"], lens, f(d["w_uk"]), f(d["w_uv"]), f(d["gate"]),
                          d["scale"], seqs=seqs)


@pytest.mark.parametrize("lens,H,shape,page_size,splits", [
    ([1, 31, 32, 33, 100], 8, "toy", 32, 0),
    ([5, 64, 65, 300, 2], 32, "mid", 64, 3),
    ([1, 2, 3], 96, "full", 32, 300),            # more splits than tiles: empty ranges
    ([700, 1, 129, 4000, 64], 96, "full", 256, 0),
    ([1] * 37 + [45, 2], 96, "full", 64, 0),
])
def test_decode_paged_ragged(o, lens, H, shape, page_size, splits):
    d, lay, pool = _paged_decode_case(lens, H, shape, page_size, seed=8000 + sum(lens) % 997)
    log(f"decode paged {shape} H={H} page {page_size} lens {lens[:6]} splits {splits}")
    got = _run_decode_paged(d, lay, pool, num_splits=splits)
    assert_parity(got, _oracle_decode_paged(o, d, lay, pool), dg.BF16, "decode paged", block=d["d_v"])


def test_decode_paged_matches_packed():
    """The paged and packed decode paths agree within the bf16 bar on the
    same rows (their split points differ, so rounding may)."""
    import torch
    import rank_latent_causal_amd as mla
    from gpu_util import run_decode
    d, lay, pool = _paged_decode_case([3000, 17, 2048, 999], 96, "full", 64, seed=8100)
    got = _run_decode_paged(d, lay, pool)
    ref = to_host_f64(run_decode(d))
    assert_parity(got, ref, dg.BF16, "paged vs packed", block=d["d_v"])


def test_decode_paged_lengths_clamped(o):
    """Lengths beyond max_pages * page_size read as that many rows (the
    second sequence fills its pages, so the clamp lands on owned rows)."""
    d, lay, pool = _paged_decode_case([64, 128], 32, "mid", 64, seed=8200)
    cap = lay["max_pages"] * 64
    big = np.array([64, cap + 50], dtype=np.int64)
    got = _run_decode_paged(d, lay, pool, lens=big)
    ref = _oracle_decode_paged(o, d, lay, pool, lens=np.minimum(big, cap))
    assert_parity(got, ref, dg.BF16, "clamped lengths", block=d["d_v"])


def test_decode_paged_full_workload_sampled(o):
    """The full decode workload (64 sequences, lengths U[1024, 32768]) in
    shuffled 64-row pages: every sequence, oracle on a sample of them."""
    d = dg.workload_inputs("full_decode")
    lay = dg.paged_layout(d["lengths"], 64, seed=d["seed"])
    pool = dg.scatter_to_pages(d["c_cache"], d["cu_seqlens"], lay)
    log(f"decode paged full workload: {int(d['cu_seqlens'][-1])} rows in {lay['num_pages']} pages")
    got = _run_decode_paged(d, lay, pool)
    seqs = np.array([0, 1, 17, 31, 40, 63])
    assert_parity(got[seqs], _oracle_decode_paged(o, d, lay, pool, seqs=seqs), dg.BF16, "decode paged full", block=d["d_v"])


@pytest.mark.parametrize("B,T,S,H,shape,page_size", [
    (2, 37, 100, 3, "toy", 32),
    (2, 30, 161, 9, "mid", 64),
    (1, 90, 250, 5, "mid", 32),
    (1, 33, 1000, 8, "full", 128),
    (3, 1, 77, 4, "full", 32),
    (1, 130, 131, 8, "full", 64),
])
def test_extend_paged(o, B, T, S, H, shape, page_size):
    import torch
    import rank_latent_causal_amd as mla
    dq, dv, r = SHAPES[shape]
    d = dg.prefill_inputs(B, S, H, dq, dv, r, dtype=dg.BF16, seed=8300 + S)
    scale = dq ** -0.5
    lay = dg.paged_layout([S] * B, page_size, seed=8300 + S)
    pool = dg.scatter_to_pages(d["c"].reshape(B * S, r), np.arange(B + 1) * S, lay)
    log(f"extend paged {shape} B={B} T={T} S={S} page {page_size}")
    q = np.ascontiguousarray(d["q"][:, S - T:])
    g = np.ascontiguousarray(d["gate"][:, S - T:])
    out = mla.mla_absorb_extend_paged(to_dev(q), to_dev(pool), to_dev(lay["block_table"]), S, to_dev(d["w_uk"]),
                                      to_dev(d["w_uv"]), to_dev(g), scale)
    torch.cuda.synchronize()
    f = dg.as_f32
    ref = o.extend_paged(f(q), f(pool), lay["block_table"], S, f(d["w_uk"]), f(d["w_uv"]), f(g), scale)
    assert_parity(to_host_f64(out), ref, dg.BF16, "extend paged", block=d["d_v"])


def test_cache_append_then_decode(o):
    """Append each sequence's new latent, then decode over the grown
    sequences: the pool changes in exactly those slots (bitwise), and the
    decode matches the oracle's append + paged decode."""
    import torch
    import rank_latent_causal_amd as mla
    lens = np.array([63, 64, 200, 1])
    full = dg.decode_inputs(4, 32, 64, 64, 256, dtype=dg.BF16, seed=8400, lengths=lens + 1)
    full["scale"] = 0.125
    cu = full["cu_seqlens"].astype(np.int64)
    new_rows = np.ascontiguousarray(full["c_cache"][cu[1:] - 1])
    keep = np.ones(cu[-1], bool)
    keep[cu[1:] - 1] = False
    lay = dg.paged_layout(lens + 1, 64, seed=8400)
    pool = dg.scatter_to_pages(full["c_cache"][keep], np.concatenate([[0], np.cumsum(lens)]), lay)
    dev_pool = to_dev(pool)
    bt = to_dev(lay["block_table"])
    mla.mla_cache_append_paged(to_dev(new_rows), dev_pool, bt, to_dev(lens.astype(np.int32)))
    torch.cuda.synchronize()
    after = dev_pool.view(torch.int16).cpu().numpy().view(np.uint16)
    changed = np.any(after != pool, axis=-1)
    assert changed.sum() == 4
    f = dg.as_f32
    want = o.cache_append(f(new_rows), f(pool), lay["block_table"], lens)
    assert np.array_equal(dg.as_f32(after), want, equal_nan=True)
    out = mla.mla_absorb_decode_paged(to_dev(full["q"]), dev_pool, bt, to_dev((lens + 1).astype(np.int32)),
                                      to_dev(full["w_uk"]), to_dev(full["w_uv"]), to_dev(full["gate"]), 0.125)
    torch.cuda.synchronize()
    ref = o.decode_paged(f(full["q"]), want, lay["block_table"], lens + 1, f(full["w_uk"]), f(full["w_uv"]),
                         f(full["gate"]), 0.125)
    assert_parity(to_host_f64(out), ref, dg.BF16, "append then decode", block=full["d_v"])


def _high_word_view(buf, arr: np.ndarray, start: int):
    """Copies an int32 array into a byte buffer at the first 256-aligned
    offset >= start whose device address has bit 31 of its low word set;
    returns (view, next free offset)."""
    import torch
    base = buf.data_ptr()
    off = (start + 255) // 256 * 256
    while ((base + off) & 0xFFFFFFFF) < 0x80000000:
        off = ((base + off) | 0x7FFFFFFF) + 1 - base  # next address with bit 31 set in the low word
        off = max(off, start)
        off = (off + 255) // 256 * 256
    nbytes = arr.nbytes
    view = buf[off:off + nbytes].view(torch.int32).view(arr.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(arr)))
    return view, off + nbytes


def test_paged_tables_at_high_low_word_addresses(o):
    """Regression: block table and lengths whose device addresses have bit 31
    of the low 32-bit word set (a sign-extended address half once made the
    kernels' scalar loads fault)."""
    import torch
    import rank_latent_causal_amd as mla
    d, lay, pool = _paged_decode_case([100, 33, 700], 32, "mid", 64, seed=8500)
    buf = torch.empty((1 << 32) + (1 << 20), dtype=torch.uint8, device="cuda")
    bt, nxt = _high_word_view(buf, lay["block_table"], 0)
    lens, _ = _high_word_view(buf, d["lengths"].astype(np.int32), nxt)
    assert (bt.data_ptr() & 0x80000000) and (lens.data_ptr() & 0x80000000)
    out = mla.mla_absorb_decode_paged(to_dev(d["q"]), to_dev(pool), bt, lens, to_dev(d["w_uk"]), to_dev(d["w_uv"]),
                                      to_dev(d["gate"]), d["scale"])
    torch.cuda.synchronize()
    assert_parity(to_host_f64(out), _oracle_decode_paged(o, d, lay, pool), dg.BF16, "high-address tables", block=d["d_v"])
    del buf


def _varlen_case(S, T, H, shape, page_size, seed):
    """Sequences with cache lengths S and chunk lengths T (T_b <= S_b) in one
    shuffled page pool; returns packed queries, gates, the pool and tables."""
    dq, dv, r = SHAPES[shape]
    parts = [dg.prefill_inputs(1, s_, H, dq, dv, r, dtype=dg.BF16, seed=seed + i) for i, s_ in enumerate(S)]
    rows = np.concatenate([p["c"][0] for p in parts])
    lay = dg.paged_layout(S, page_size, seed=seed)
    pool = dg.scatter_to_pages(rows, np.concatenate([[0], np.cumsum(S)]), lay)
    q = np.ascontiguousarray(np.concatenate([p["q"][0, s_ - t_:] for p, s_, t_ in zip(parts, S, T)]))
    g = np.ascontiguousarray(np.concatenate([p["gate"][0, s_ - t_:] for p, s_, t_ in zip(parts, S, T)]))
    cu_q = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    return dict(q=q, gate=g, pool=pool, lay=lay, cu_q=cu_q, S=np.array(S, dtype=np.int32), w_uk=parts[0]["w_uk"],
                w_uv=parts[0]["w_uv"], scale=dq ** -0.5)


@pytest.mark.parametrize("S,T,H,shape,page_size", [
    ([300, 1000, 5000, 64, 129], [300, 77, 1, 0, 33], 8, "full", 64),
    ([40, 17, 100, 33], [40, 1, 60, 33], 4, "toy", 32),
    ([257, 70, 1], [100, 70, 1], 9, "mid", 128),
    ([4096] * 3 + [2000] * 8, [1] * 3 + [300] * 8, 96, "full", 256),
])
def test_extend_varlen_mixed_batch(o, S, T, H, shape, page_size):
    """One call over a batch mixing prefills (S = T), chunks after a cached
    prefix, decode steps (T = 1) and empty chunks."""
    import torch
    import rank_latent_causal_amd as mla
    v = _varlen_case(S, T, H, shape, page_size, seed=8600 + sum(S) % 991)
    log(f"varlen {shape} H={H} S={S[:5]} T={T[:5]} page {page_size}")
    out = mla.mla_absorb_extend_varlen_paged(to_dev(v["q"]), to_dev(v["pool"]), to_dev(v["lay"]["block_table"]),
                                             to_dev(v["cu_q"]), to_dev(v["S"]), to_dev(v["w_uk"]), to_dev(v["w_uv"]),
                                             to_dev(v["gate"]), v["scale"])
    torch.cuda.synchronize()
    f = dg.as_f32
    ref = o.extend_varlen_paged(f(v["q"]), f(v["pool"]), v["lay"]["block_table"], v["cu_q"], v["S"], f(v["w_uk"]),
                                f(v["w_uv"]), f(v["gate"]), v["scale"])
    assert_parity(to_host_f64(out), ref, dg.BF16, "varlen", block=SHAPES[shape][1])


def test_extend_varlen_clamps_bad_ranges(o):
    """Descriptions that break the preconditions (a query range past Nq, a
    cache length past the table) are clamped on the device: the call stays
    inside its buffers and the well-formed sequences are unaffected."""
    import torch
    import rank_latent_causal_amd as mla
    v = _varlen_case([100, 64], [30, 20], 8, "mid", 64, seed=8700)
    cap = v["lay"]["max_pages"] * 64
    cu_bad = np.array([0, 30, 50 + 1000], dtype=np.int32)  # the last range runs past Nq = 50
    S_bad = np.array([100, cap + 500], dtype=np.int32)
    out = mla.mla_absorb_extend_varlen_paged(to_dev(v["q"]), to_dev(v["pool"]), to_dev(v["lay"]["block_table"]),
                                             to_dev(cu_bad), to_dev(S_bad), to_dev(v["w_uk"]), to_dev(v["w_uv"]),
                                             to_dev(v["gate"]), v["scale"])
    torch.cuda.synchronize()
    f = dg.as_f32
    ref = o.extend_varlen_paged(f(v["q"]), f(v["pool"]), v["lay"]["block_table"], v["cu_q"], v["S"], f(v["w_uk"]),
                                f(v["w_uv"]), f(v["gate"]), v["scale"])
    assert_parity(to_host_f64(out)[:30], ref[:30], dg.BF16, "well-formed sequence next to bad ranges", block=64)
