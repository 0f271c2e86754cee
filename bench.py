"""Benchmark of the absorbed Gated MLA hot path on one MI355X.

One step = one full-width prefill call (B=1, T=8192, H=96, d_q=d_v=128,
r=512, bf16, causal, scale 1/sqrt(d_q)), one chunked-prefill call (the last
2048 of those positions after the 6144 before them) and one full-width decode
call (64 sequences with cache lengths ~ U[1024, 32768], same widths) on
seeded synthetic inputs already resident in HBM.  Each call is bracketed by
HIP events on the stream it runs on.

Printed (one JSON line): prefill TFLOP/s as `value` (causal-triangle
algorithmic FLOPs), chunked-prefill TFLOP/s, decode latent-cache GB/s
(algorithmic bytes), each with a roofline object against MI355X's published
peaks (2.5 PFLOP/s dense bf16 MFMA, 8 TB/s HBM3E, 157.3 TFLOP/s fp32
vector), and the CPU oracle (cpu_baseline): a bounded row sample of the
full prefill, plus the whole decode call and the whole toy and mid-scale
prefill calls.  The smaller prefill workloads (toy fp32, toy-max B=4
T=2048, mid-scale B=4 T=4096 H=32 r=256) are timed whole under their names.
The full-layer forward (projections, norms, core, output projection at the
full K3 widths, B=1, T=8192) is timed separately after the steps and
reported under "forward"; a varlen batch of four chunks over a paged cache
under "extend_varlen"; the backward of the prefill core (with the
log-sum-exp of a training forward run before it) likewise under
"backward"; one training step of the whole layer (training forward, then
the layer backward) under "layer_train"; chunk_kda over B=1, T=8192, H=96,
K=V=128 under "kda".  The decode over a paged cache (the decode workload in
shuffled 64-row pages) runs in each step right after the packed decode and
is reported under "decode_paged".  None of these is part of ms_per_step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import datagen as dg  # noqa: E402

METRIC = "absorbed-MLA prefill TFLOP/s + decode latent-cache GB/s (% of roofline), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs x 2.4 GHz)


def prefill_flops(B, T, H, dq, dv, r):
    """Algorithmic FLOPs of one prefill call: absorb + W_UV products on every
    (b, t, h), and the score and latent-sum products on the causal triangle
    (diagonal included)."""
    pairs = B * H * T * (T + 1) // 2
    return 2 * B * T * H * r * (dq + dv) + 4 * r * pairs


def extend_flops(B, T, S, H, dq, dv, r):
    """Algorithmic FLOPs of one chunked-prefill call: absorb + W_UV on the T
    chunk rows, scores and latent sums over keys 0 .. S-T+t for each row."""
    P = S - T
    pairs = B * H * (T * P + T * (T + 1) // 2)
    return 2 * B * T * H * r * (dq + dv) + 4 * r * pairs


def forward_flops(B, T, D, q_rank, H, dq, dv, r):
    """Algorithmic FLOPs of one full-layer forward: the five projections
    (latent and query down-projections, query up-projection, gate, output
    projection) on every row, plus the core's prefill FLOPs."""
    N = B * T
    return 2 * N * (D * r + D * q_rank + q_rank * H * dq + D * H * dv + H * dv * D) + \
        prefill_flops(B, T, H, dq, dv, r)


def decode_flops(lengths, H, dq, dv, r):
    return int(4 * r * H * int(np.sum(lengths)) + len(lengths) * H * 2 * r * (dq + dv))


def decode_bytes(lengths, H, dq, dv, r, elt=2):
    """Bytes the decode call must move: the latent cache once, both weight
    tensors once, q, gate, out and cu_seqlens."""
    B = len(lengths)
    return int(elt * r * int(np.sum(lengths)) + elt * H * r * (dq + dv) + elt * B * H * (dq + 2 * dv) + 4 * (B + 1))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_full_prefill_full_decode.md")


def kernel_source_hash() -> str:
    """sha256 over the MLA library's HIP sources and its ABI header, in a
    fixed order: the key under which measured HBM traffic is stored.  The
    KDA sources (files named kda*) build separate kernels and are left out."""
    import hashlib
    h = hashlib.sha256()
    files = []
    for d in (os.path.join(ROOT, "rank_latent_causal_amd", "csrc"), os.path.join(ROOT, "include")):
        files += [os.path.join(d, f) for f in sorted(os.listdir(d))
                  if f.endswith((".h", ".hip")) and not f.startswith("kda")]
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the summary was taken on other kernel sources than the current ones."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("traffic-record: "):
                    rec = json.loads(line[len("traffic-record: "):])
                    return rec if rec.get("sources") == kernel_source_hash() else None
    except OSError:
        return None
    return None


KDA_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_full_kda.md")


def kda_source_hash() -> str:
    """sha256 over the sources chunk_kda's kernels are built from (the KDA
    files and the device helpers they include), in a fixed order: the key
    of the KDA traffic record."""
    import hashlib
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "include", "kda.h")] + [
        os.path.join(ROOT, "rank_latent_causal_amd", "csrc", f) for f in ("common.h", "kda_bf16.h", "kda.hip")]
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_kda_traffic():
    """The KDA traffic record (bytes per call) if it was taken from the
    current KDA sources, else None."""
    try:
        with open(KDA_TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("traffic-record: "):
                    rec = json.loads(line[len("traffic-record: "):])
                    return rec if rec.get("sources") == kda_source_hash() else None
    except OSError:
        return None
    return None


def copy_probe(nbytes: int = 1 << 30):
    """One plain device-to-device copy of nbytes: the reference kernel whose
    FETCH_SIZE / WRITE_SIZE readings scale the counters to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# copy probe: {nbytes} bytes device to device", file=sys.stderr, flush=True)


def dev(x):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def cpu_baseline(pre, dec, target_s: float, small: dict):
    """The oracle as it stands, on the host threads OpenMP gives it.

    Headline (value): a sample of query rows of the full-width prefill,
    sized to take about target_s seconds, in TFLOP/s of the same algorithmic
    count.  Also timed, each as a whole call: the full decode workload (all
    64 sequences, GB/s of the same algorithmic bytes) and the prefill
    workloads small enough to finish in seconds (`small`: name -> inputs)."""
    import oracle
    o = oracle.get()
    f = dg.as_f32
    q, c, wk, wv, g = [f(pre[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    B, T, H, dq, dv, r = pre["B"], pre["T"], pre["H"], pre["d_q"], pre["d_v"], pre["r"]

    def row_flops(rows):
        t = rows % T
        return int(np.sum(H * (4 * r * (t + 1) + 2 * r * (dq + dv))))

    def run(n):
        rows = np.array([int((k + 0.5) * B * T / n) for k in range(n)], dtype=np.int64)
        t0 = time.perf_counter()
        o.prefill(q, c, wk, wv, g, pre["scale"], rows=rows)
        return time.perf_counter() - t0, row_flops(rows), rows

    dt, fl, _ = run(64)
    n = int(min(B * T, max(64, 64 * target_s / max(dt, 1e-3))))
    dt, fl, rows = run(n)
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    res = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"{n} query rows (all {H} heads) evenly spaced over the {B}x{T} prefill workload, "
                     f"{fl / 1e9:.1f} GFLOP in {dt:.1f} s"}
    for name, d in small.items():
        args = [f(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
        t0 = time.perf_counter()
        o.prefill(*args, d["scale"])
        sec = time.perf_counter() - t0
        fl = prefill_flops(d["B"], d["T"], d["H"], d["d_q"], d["d_v"], d["r"])
        res[name] = {"value": fl / sec / 1e12, "unit": "TFLOP/s", "seconds": round(sec, 3),
                     "sample": "the whole call"}
    if dec is not None:
        cc = f(dec["c_cache"])
        args = [f(dec["q"]), cc, dec["cu_seqlens"].astype(np.int64), f(dec["w_uk"]), f(dec["w_uv"]),
                f(dec["gate"])]
        t0 = time.perf_counter()
        o.decode(*args, dec["scale"])
        sec = time.perf_counter() - t0
        nb = decode_bytes(dec["lengths"], dec["H"], dec["d_q"], dec["d_v"], dec["r"])
        res["full_decode"] = {"value": nb / sec / 1e9, "unit": "GB/s", "seconds": round(sec, 3),
                              "sample": f"the whole call: all {dec['B']} sequences, "
                                        f"{int(dec['cu_seqlens'][-1])} cache rows"}
        del cc
    return res


def bench_prefill_workload(torch, mla, name, calls, warmup):
    """One named prefill workload (its whole call: the W_UK transpose and the
    prefill kernel for bf16, the fp32 kernel for fp32), timed by HIP events
    around each call on the current stream."""
    d = dg.workload_inputs(name)
    args = [dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    B, T, H, dq, dv, r = d["B"], d["T"], d["H"], d["d_q"], d["d_v"], d["r"]
    bf = d["dtype"] == dg.BF16
    dt = mla.DTYPE_BF16 if bf else mla.DTYPE_F32
    out = torch.empty((B, T, H * dv), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    ws = torch.empty(max(1, mla.prefill_workspace_size(B, T, H, dq, r, dt)), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        mla.mla_absorb_prefill(*args, d["scale"], out=out, workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        mla.mla_absorb_prefill(*args, d["scale"], out=out, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    fl = prefill_flops(B, T, H, dq, dv, r)
    tf = fl / (ms * 1e-3) / 1e12
    if bf:
        kernel = ("mla_prefill_bf16_kernel<16,16,32>" if r == 32 else
                  f"mla_prefill_solo_kernel<{dq},{dv},{r}>") + " (+ W_UK transpose in the same call)"
        roof = {"bound": "mfma", "peak": PEAK_BF16_TFLOPS}
    else:
        kernel = "mla_f32_kernel"
        roof = {"bound": "alu", "peak": PEAK_F32_VALU_TFLOPS}
    roof.update({"achieved": round(tf, 3), "unit": "TFLOP/s", "frac": round(tf / roof["peak"], 5),
                 "traffic": None, "kernel": kernel, "flop_per_launch": fl})
    return {"value": round(tf, 3), "unit": "TFLOP/s", "ms": round(ms, 5), "calls": calls, "seed": d["seed"],
            "workload": f"{name}: B={B}, T={T}, H={H}, d_q=d_v={dq}, r={r}, {d['dtype']}, causal, "
                        f"scale {d['scale']:.4g}",
            "roofline": roof}


def bench_forward(torch, mla, steps, warmup):
    """The whole layer (projections, norms, core, output projection) at the
    full K3 widths, B=1, T=8192, timed on its own after the hot-path steps."""
    fw = dg.WORKLOADS["full_forward"]
    d = dg.workload_inputs("full_forward")
    args = [dev(d[k]) for k in dg.FORWARD_KEYS]
    B, T, D, qr, H, dq, dv, r = (d[k] for k in ("B", "T", "D", "q_rank", "H", "d_q", "d_v", "r"))
    y = torch.empty((B, T, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.forward_workspace_size(B, T, qr, H, dq, dv, r, mla.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(warmup):
        mla.mla_gated_forward(*args, d["eps"], d["scale"], out=y, workspace=ws)
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        mla.mla_gated_forward(*args, d["eps"], d["scale"], out=y, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    f = forward_flops(B, T, D, qr, H, dq, dv, r)
    tf = f / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4), "seed": fw["seed"],
            "workload": f"full_forward: B={B}, T={T}, D={D}, q_rank={qr}, H={H}, d_q=d_v={dq}, r={r}, eps 1e-6",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "flop_per_launch": f}}


def backward_flops(B, T, H, dq, dv, r):
    """Algorithmic FLOPs of one backward of the prefill core: five latent
    products per causal (query, key, head) triple (the recomputed scores,
    dP = dol c^T, da = dS c, and c's key and value gradients), 2 r FLOP
    each, plus the per-row projections (q W_UK, do W_UV, da W_UK^T and the
    two weight gradients)."""
    pairs = B * H * T * (T + 1) // 2
    return 10 * r * pairs + 2 * B * T * H * r * (3 * dq + 2 * dv)


def bench_backward(torch, mla, steps, warmup):
    """The backward of the full-width prefill (B=1, T=8192), its forward
    (with the log-sum-exp) run once before the timed calls."""
    d = dg.workload_inputs("full_prefill")
    args = [dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    B, T, H, dq, dv, r = d["B"], d["T"], d["H"], d["d_q"], d["d_v"], d["r"]
    out, lse = mla.mla_absorb_prefill_train(*args, d["scale"])
    g = torch.Generator(device="cuda").manual_seed(d["seed"])
    dout = torch.randn(out.shape, generator=g, device="cuda").to(torch.bfloat16)
    ws = torch.empty(mla.backward_workspace_size(B, T, H, dq, dv, r, mla.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    for _ in range(max(1, warmup // 4)):
        mla.mla_absorb_prefill_backward(*args, out, lse, dout, d["scale"], workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(1, steps // 4))]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        mla.mla_absorb_prefill_backward(*args, out, lse, dout, d["scale"], workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    f = backward_flops(B, T, H, dq, dv, r)
    tf = f / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4), "calls": len(ev),
            "workload": "backward of full_prefill (B=1, T=8192, H=96, d_q=d_v=128, r=512), dout ~ N(0,1)",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "flop_per_launch": f}}


def layer_train_flops(B, T, D, q_rank, H, dq, dv, r):
    """Algorithmic FLOPs of one training step of the full layer: the forward,
    then the core's backward and, for each of the five projections, its input
    and weight gradients (twice the projection's forward FLOPs; the latent
    and query down-projections' input gradients included, since x needs
    them)."""
    N = B * T
    proj = 2 * N * (D * r + D * q_rank + q_rank * H * dq + D * H * dv + H * dv * D)
    return forward_flops(B, T, D, q_rank, H, dq, dv, r) + 2 * proj + backward_flops(B, T, H, dq, dv, r)


def bench_layer_train(torch, mla, steps, warmup):
    """One training step of the whole layer at the full K3 widths, B=1,
    T=8192: mla_gated_forward_train then mla_gated_backward with dy ~ N(0,1)."""
    fw = dg.WORKLOADS["full_forward"]
    d = dg.workload_inputs("full_forward")
    args = [dev(d[k]) for k in dg.FORWARD_KEYS]
    B, T, D, qr, H, dq, dv, r = (d[k] for k in ("B", "T", "D", "q_rank", "H", "d_q", "d_v", "r"))
    y = torch.empty((B, T, D), dtype=torch.bfloat16, device="cuda")
    state = torch.empty(mla.train_state_size(B, T, qr, H, dq, dv, r, mla.DTYPE_BF16), dtype=torch.uint8,
                        device="cuda")
    ws = torch.empty(mla.layer_backward_workspace_size(B, T, D, qr, H, dq, dv, r, mla.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    g = torch.Generator(device="cuda").manual_seed(fw["seed"])
    dy = torch.randn((B, T, D), generator=g, device="cuda").to(torch.bfloat16)
    grads = None

    def step():
        nonlocal grads
        mla.mla_gated_forward_train(*args, d["eps"], d["scale"], out=y, state=state)
        grads = mla.mla_gated_backward(*args, dy, state, d["scale"], grads=grads, workspace=ws)

    n = max(1, steps // 4)
    for _ in range(max(1, warmup // 4)):
        step()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    torch.cuda.synchronize()
    for a, m, b in ev:
        a.record()
        mla.mla_gated_forward_train(*args, d["eps"], d["scale"], out=y, state=state)
        m.record()
        grads = mla.mla_gated_backward(*args, dy, state, d["scale"], grads=grads, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, _, b in ev]))
    ms_f = float(np.mean([a.elapsed_time(m) for a, m, _ in ev]))
    f = layer_train_flops(B, T, D, qr, H, dq, dv, r)
    tf = f / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4), "ms_forward_train": round(ms_f, 4),
            "ms_backward": round(ms - ms_f, 4), "calls": n, "seed": fw["seed"],
            "workload": f"training step of full_forward: B={B}, T={T}, D={D}, q_rank={qr}, H={H}, d_q=d_v={dq}, "
                        f"r={r}, dy ~ N(0,1)",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "flop_per_launch": f}}


def kda_bytes(B, T, H, G, K, V):
    """Bytes chunk_kda must move: q and k (bf16) per query/key head, v and o
    (bf16), g (fp32) and beta (fp32) per value head, once each."""
    HV = G * H
    return B * T * (2 * H * K * 2 + HV * V * 2 * 2 + HV * K * 4 + HV * 4)


def kda_flops(B, T, H, G, K, V):
    """FLOPs of the step-by-step recurrence: per position and value head the
    decay (K V), the prediction k^T S (2 K V), the write (2 K V) and the
    read-out q^T S (2 K V)."""
    return 7 * B * T * G * H * K * V


def bench_kda(torch, mla, steps, warmup):
    """chunk_kda over the full workload (B=1, T=8192, H=H_V=96, K=V=128), a
    zero initial state, no final state: both kernels of one call."""
    d = dg.workload_inputs("full_kda")
    B, T, H, G, K, V = (d[k] for k in ("B", "T", "H", "G", "K", "V"))
    args = [dev(d[k]) for k in ("q", "k", "v", "g", "beta")]
    out = torch.empty((B, T, G * H, V), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.kda_workspace_size(B, T, H, G, K, V), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        mla.kda_chunk_forward(*args, G=G, out=out, workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        mla.kda_chunk_forward(*args, G=G, out=out, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nb = kda_bytes(B, T, H, G, K, V)
    gbs = nb / (ms * 1e-3) / 1e9
    rec = measured_kda_traffic()
    return {"value": round(gbs, 1), "unit": "GB/s", "ms": round(ms, 4),
            "tflops": round(kda_flops(B, T, H, G, K, V) / (ms * 1e-3) / 1e12, 2), "seed": d["seed"],
            "workload": f"full_kda: B={B}, T={T}, H=H_V={G * H}, K=V={K}, chunks of 64, g in [-5, 0], zero state",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": rec["call_bytes"] if rec else None,
                         "bytes_per_launch": nb, "kernel": "kda_intra + kda_state"}}


def bench_varlen(torch, mla, steps, warmup, page_size=64):
    """A mixed chunk batch at full width in one varlen call over a paged
    cache: chunks of 2048, 1024, 512 and 256 queries after 6144, 3072, 7680
    and 1792 cached positions (H=96, d=128, r=512), pages of 64 rows."""
    S = [8192, 4096, 8192, 2048]
    T = [2048, 1024, 512, 256]
    H, dq, dv, r = 96, 128, 128, 512
    seed = dg.WORKLOADS["full_prefill"]["seed"] + 100
    parts = [dg.prefill_inputs(1, s_, H, dq, dv, r, dtype=dg.BF16, seed=seed + i) for i, s_ in enumerate(S)]
    lay = dg.paged_layout(S, page_size, seed=seed)
    pool = dg.scatter_to_pages(np.concatenate([p["c"][0] for p in parts]), np.concatenate([[0], np.cumsum(S)]), lay)
    q = np.concatenate([p["q"][0, s_ - t_:] for p, s_, t_ in zip(parts, S, T)])
    g = np.concatenate([p["gate"][0, s_ - t_:] for p, s_, t_ in zip(parts, S, T)])
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    args = [dev(q), dev(pool), dev(lay["block_table"]), dev(cu), dev(np.array(S, dtype=np.int32)),
            dev(parts[0]["w_uk"]), dev(parts[0]["w_uv"]), dev(g)]
    scale = dq ** -0.5
    out = torch.empty((int(cu[-1]), H * dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.varlen_workspace_size(len(S), int(cu[-1]), H, dq, r, mla.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        mla.mla_absorb_extend_varlen_paged(*args, scale, out=out, workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        mla.mla_absorb_extend_varlen_paged(*args, scale, out=out, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    f = sum(extend_flops(1, t_, s_, H, dq, dv, r) for s_, t_ in zip(S, T))
    tf = f / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "workload": "varlen chunk batch T=[2048,1024,512,256] after S-T cached of S=[8192,4096,8192,2048], "
                        "H=96, d_q=d_v=128, r=512, 64-row shuffled pages",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "flop_per_launch": f}}


def setup_decode_paged(torch, mla, dec, page_size=64):
    """The full decode workload with its cache in shuffled 64-row pages.
    Returns (launch, report): launch() enqueues one call; report(ms) builds
    the JSON object.  The calls run inside the timed steps, right after the
    packed decode, so both see the same clock state."""
    lay = dg.paged_layout(dec["lengths"], page_size, seed=dec["seed"])
    pool = dg.scatter_to_pages(dec["c_cache"], dec["cu_seqlens"], lay)
    args = [dev(dec["q"]), dev(pool), dev(lay["block_table"]), dev(dec["lengths"].astype(np.int32)),
            dev(dec["w_uk"]), dev(dec["w_uv"]), dev(dec["gate"])]
    B, H, dq, dv, r = dec["B"], dec["H"], dec["d_q"], dec["d_v"], dec["r"]
    out = torch.empty((B, H * dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.decode_paged_workspace_size(B, H, dq, r, 0, mla.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    nbytes = decode_bytes(dec["lengths"], H, dq, dv, r) + 4 * B * lay["max_pages"]

    def launch():
        mla.mla_absorb_decode_paged(*args, dec["scale"], out=out, workspace=ws)

    def report(ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"value": round(gbs, 1), "unit": "GB/s", "ms": round(ms, 4),
                "workload": f"full_decode with the cache in {lay['num_pages']} shuffled pages of {page_size} rows",
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "bytes_per_launch": nbytes}}
    return launch, report


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--which", choices=["both", "prefill", "decode", "forward", "backward", "layer_train", "kda"],
                    default="both",
                    help="both: prefill, chunked prefill and decode, then the full-layer forward and the backward")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's hot path only (got --gpus {args.gpus}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_latent_causal_amd as mla

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    mla.lib()

    pw, dw = dg.WORKLOADS["full_prefill"], dg.WORKLOADS["full_decode"]
    t_gen = time.perf_counter()
    pre = dg.workload_inputs("full_prefill")
    dec = dg.workload_inputs("full_decode")
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f}s; decode cache rows "
          f"{int(dec['cu_seqlens'][-1])}", file=sys.stderr, flush=True)

    P = [dev(pre[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    B, T, H, dq, dv, r = pre["B"], pre["T"], pre["H"], pre["d_q"], pre["d_v"], pre["r"]
    p_out = torch.empty((B, T, H * dv), dtype=torch.bfloat16, device="cuda")
    p_ws = torch.empty(max(1, mla.prefill_workspace_size(B, T, H, dq, r, mla.DTYPE_BF16)), dtype=torch.uint8,
                       device="cuda")
    D = [dev(dec[k]) for k in ("q", "c_cache", "cu_seqlens", "w_uk", "w_uv", "gate")]
    DB = dec["B"]
    # chunked prefill: the last 2048 positions of the prefill workload as a
    # chunk after 6144 cached positions
    XT = 2048
    X = [P[0][:, T - XT:].contiguous(), P[1], P[2], P[3], P[4][:, T - XT:].contiguous()]
    x_out = torch.empty((B, XT, H * dv), dtype=torch.bfloat16, device="cuda")
    d_out = torch.empty((DB, H * dv), dtype=torch.bfloat16, device="cuda")
    d_ws = torch.empty(max(1, mla.decode_workspace_size(DB, H, dq, r, 0, mla.DTYPE_BF16)), dtype=torch.uint8,
                       device="cuda")

    do_pre = args.which in ("both", "prefill")
    do_dec = args.which in ("both", "decode")

    paged = setup_decode_paged(torch, mla, dec) if do_dec else None

    def step(ev):
        if do_pre:
            ev[0].record()
            mla.mla_absorb_prefill(*P, pre["scale"], out=p_out, workspace=p_ws)
            ev[1].record()
        if args.which == "both":
            ev[4].record()
            mla.mla_absorb_extend(*X, pre["scale"], out=x_out, workspace=p_ws)
            ev[5].record()
        if do_dec:
            ev[2].record()
            mla.mla_absorb_decode(*D, dec["scale"], out=d_out, workspace=d_ws)
            ev[3].record()
            ev[6].record()
            paged[0]()
            ev[7].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for _ in range(args.warmup):
        step(warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"# timed {args.steps} steps in {wall:.3f}s", file=sys.stderr, flush=True)

    pf = prefill_flops(B, T, H, dq, dv, r)
    df = decode_flops(dec["lengths"], H, dq, dv, r)
    dbytes = decode_bytes(dec["lengths"], H, dq, dv, r)
    p_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) if do_pre else 0.0
    d_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) if do_dec else 0.0
    p_tflops = pf / (p_ms * 1e-3) / 1e12 if do_pre else None
    d_gbs = dbytes / (d_ms * 1e-3) / 1e9 if do_dec else None

    res = {
        "metric": METRIC,
        "value": round(p_tflops, 2) if do_pre else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(p_ms + d_ms + (float(np.mean([e[4].elapsed_time(e[5]) for e in evs]))
                                           if args.which == "both" else 0.0), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "full_prefill (B=1, T=8192, H=96, d_q=d_v=128, r=512, causal, scale 1/sqrt(128)) + "
                        "full_decode (B=64 queries, cache lengths ~ U[1024,32768], H=96, d_q=d_v=128, r=512)",
            "prefill_seed": pw["seed"], "decode_seed": dw["seed"],
            "decode_cache_rows": int(dec["cu_seqlens"][-1]),
        },
    }
    if do_pre:
        res["roofline"] = {"bound": "mfma", "achieved": round(p_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                           "kernel": "mla_prefill_solo_kernel<128,128,512> (+ W_UK transpose in the same call)", "flop_per_launch": pf,
                           "ms_per_launch": round(p_ms, 4)}
    if do_dec:
        res["decode"] = {"value": round(d_gbs, 1), "unit": "GB/s", "ms": round(d_ms, 4),
                         "tflops": round(df / (d_ms * 1e-3) / 1e12, 2),
                         "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": round(d_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                                      "kernel": "mla_decode_solo<512> + absorb (with the range table) + merge",
                                      "bytes_per_launch": dbytes}}
    traffic = measured_traffic()
    if traffic is not None:
        if do_pre:
            res["roofline"]["traffic"] = traffic["prefill_bytes"]
        if do_dec:
            res["decode"]["roofline"]["traffic"] = traffic["decode_bytes"]
    if args.copy_probe:
        copy_probe()
    if args.which == "both":
        x_ms = float(np.mean([e[4].elapsed_time(e[5]) for e in evs]))
        xf = extend_flops(B, XT, T, H, dq, dv, r)
        x_tf = xf / (x_ms * 1e-3) / 1e12
        res["extend"] = {"value": round(x_tf, 2), "unit": "TFLOP/s", "ms": round(x_ms, 4),
                         "workload": f"chunked prefill: {XT} queries after {T - XT} cached positions "
                                     f"(S={T}), B={B}, H={H}, d_q=d_v={dq}, r={r}",
                         "roofline": {"bound": "mfma", "achieved": round(x_tf, 2), "peak": PEAK_BF16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(x_tf / PEAK_BF16_TFLOPS, 4),
                                      "traffic": None, "flop_per_launch": xf}}
    if do_dec:
        res["decode_paged"] = paged[1](float(np.mean([e[6].elapsed_time(e[7]) for e in evs])))
    if args.which in ("both", "prefill"):
        res["extend_varlen"] = bench_varlen(torch, mla, args.steps, args.warmup)
    if args.which in ("both", "forward"):
        res["forward"] = bench_forward(torch, mla, args.steps, args.warmup)
    if args.which in ("both", "backward"):
        res["backward"] = bench_backward(torch, mla, args.steps, args.warmup)
    if args.which in ("both", "layer_train"):
        res["layer_train"] = bench_layer_train(torch, mla, args.steps, args.warmup)
    if args.which in ("both", "kda"):
        res["kda"] = bench_kda(torch, mla, args.steps, args.warmup)
    if args.which in ("both", "prefill"):
        # the smaller prefill workloads (toy fp32, toy-max, mid-scale): whole
        # calls, each with its roofline object; not part of ms_per_step
        for name, calls in (("toy_f32", 200), ("toy_max", 200), ("mid", max(20, args.steps))):
            res[name] = bench_prefill_workload(torch, mla, name, calls, max(10, args.warmup))
    if not args.no_cpu_baseline and do_pre:
        small = {name: dg.workload_inputs(name) for name in ("toy_f32", "toy_max", "mid")}
        res["cpu_baseline"] = cpu_baseline(pre, dec if do_dec else None, args.cpu_seconds, small)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
