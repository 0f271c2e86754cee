"""Plain CPU oracle for the absorbed Gated MLA layer and chunk_kda's
recurrence (ctypes wrapper).

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package.  The product library never loads
it, and it shares no code with the HIP sources.

The arithmetic lives in ``mla_oracle.c`` (fp64 accumulation, plain loops, one
OpenMP loop over query rows); this module only compiles it with the host C
compiler and marshals numpy arrays.  See the C file's header for the
definition it computes and the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "mla_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-mavx2", "-mfma",
           "-fno-fast-math", "-Wall", "-Wextra"]


LIB_SANITIZED = os.path.join(_HERE, "liboracle_san.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build: any out-of-bounds
# access, use after free, signed overflow, misaligned or null access, or bad
# shift aborts the process (the library must then be loaded into a process
# started with libasan preloaded; see tests/test_oracle_sanitized.py).
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(out_path: str = LIB, mutant: int = 0, quiet: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc; mutant != 0 plants one known mistake;
    sanitize builds it with ASan and UBSan instead of -O3."""
    flags = [f for f in _CFLAGS if f != "-O3"] + ["-O1"] + _SAN_FLAGS if sanitize else list(_CFLAGS)
    cmd = ["gcc", *flags, f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", out_path + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    if not quiet and res.stderr:
        print(res.stderr)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ct.POINTER(ctype))


class Oracle:
    """One loaded build of the oracle (the default one, or a planted mutant)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} not built; call oracle.build()")
        self.path = path
        self.lib = ct.CDLL(path)
        L = self.lib
        fp, dp, i64p = ct.POINTER(ct.c_float), ct.POINTER(ct.c_double), ct.POINTER(ct.c_int64)
        I, I64, D = ct.c_int, ct.c_int64, ct.c_double
        L.oracle_mutant.restype = I
        L.oracle_prefill.argtypes = [fp, fp, fp, fp, fp, I, I, I, I, I, I, D, i64p, I64, dp, I]
        L.oracle_extend.argtypes = [fp, fp, fp, fp, fp, I, I, I, I, I, I, I, D, i64p, I64, dp, I]
        L.oracle_decode.argtypes = [fp, fp, i64p, fp, fp, fp, I, I, I, I, I, D, i64p, I64, dp, I]
        L.oracle_prefill_decompressed.argtypes = [fp, fp, fp, fp, fp, I, I, I, I, I, I, D, dp, I]
        L.oracle_prefill_attn.argtypes = [fp, fp, fp, I, I, I, I, I, D, dp]
        L.oracle_round_bf16.argtypes = [dp, I64, dp]
        L.oracle_decode_paged.argtypes = [fp, fp, I64, I, i64p, I, i64p, fp, fp, fp, I, I, I, I, I, D, i64p, I64,
                                          dp, I]
        L.oracle_extend_paged.argtypes = [fp, fp, I64, I, i64p, I, fp, fp, fp, I, I, I, I, I, I, I, D, i64p, I64,
                                          dp, I]
        L.oracle_cache_append.argtypes = [fp, fp, I64, I, i64p, I, i64p, I, I]
        L.oracle_prefill_backward.argtypes = [fp] * 6 + [I] * 6 + [D] + [dp] * 5 + [I]
        L.oracle_prefill_lse.argtypes = [fp, fp, fp, I, I, I, I, I, D, dp, I]
        L.oracle_forward_backward.argtypes = [fp] * 11 + [I] * 8 + [D, D] + [dp] * 10 + [I]
        L.oracle_kda.argtypes = [fp] * 6 + [I] * 6 + [dp, dp, I]
        L.oracle_extend_varlen_paged.argtypes = [fp, fp, I64, I, i64p, I, i64p, i64p, fp, fp, fp, I, I, I, I, I, D,
                                                 dp, I]
        L.oracle_forward.argtypes = [fp] * 10 + [I] * 8 + [D, D, I, i64p, I64] + [dp] * 5 + [I]
        for f in ("oracle_prefill", "oracle_extend", "oracle_decode", "oracle_prefill_decompressed",
                  "oracle_prefill_attn", "oracle_round_bf16", "oracle_forward", "oracle_decode_paged",
                  "oracle_extend_paged", "oracle_cache_append", "oracle_prefill_backward",
                  "oracle_prefill_lse", "oracle_extend_varlen_paged", "oracle_forward_backward", "oracle_kda"):
            getattr(L, f).restype = I

    @property
    def mutant(self) -> int:
        return self.lib.oracle_mutant()

    @staticmethod
    def _check(rc: int, what: str) -> None:
        if rc != 0:
            raise ValueError(f"{what} failed with code {rc}")

    def prefill(self, q, c, w_uk, w_uv, gate, scale: float, rows=None, threads: int = 0) -> np.ndarray:
        """Prefill.  rows: flattened b*T+t indices (None: all).  Returns
        [B,T,H*dv] for all rows, else [len(rows), H*dv] (float64)."""
        q, c, w_uk, w_uv, gate = map(_f32, (q, c, w_uk, w_uv, gate))
        B, T, H, dq = q.shape
        r = c.shape[-1]
        dv = w_uv.shape[1]
        assert c.shape == (B, T, r) and w_uk.shape == (H, dq, r) and w_uv.shape == (H, dv, r)
        assert gate.shape == (B, T, H * dv)
        if rows is None:
            out = np.empty((B, T, H * dv), dtype=np.float64)
            rp, n = None, B * T
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            out = np.empty((rows.shape[0], H * dv), dtype=np.float64)
            rp, n = _ptr(rows, ct.c_int64), rows.shape[0]
        self._check(self.lib.oracle_prefill(
            _ptr(q, ct.c_float), _ptr(c, ct.c_float), _ptr(w_uk, ct.c_float), _ptr(w_uv, ct.c_float),
            _ptr(gate, ct.c_float), B, T, H, dq, dv, r, float(scale), rp, n,
            _ptr(out, ct.c_double), threads), "oracle_prefill")
        return out

    def extend(self, q, c, w_uk, w_uv, gate, scale: float, rows=None, threads: int = 0) -> np.ndarray:
        """Chunked prefill: q [B,T,H,dq] are the last T positions of sequences
        whose latent is c [B,S,r] (S >= T); query t attends to keys
        0 .. S-T+t.  rows as for prefill.  Returns [B,T,H*dv] or
        [len(rows), H*dv] (float64)."""
        q, c, w_uk, w_uv, gate = map(_f32, (q, c, w_uk, w_uv, gate))
        B, T, H, dq = q.shape
        S, r = c.shape[1], c.shape[2]
        dv = w_uv.shape[1]
        assert c.shape == (B, S, r) and S >= T and w_uk.shape == (H, dq, r) and w_uv.shape == (H, dv, r)
        assert gate.shape == (B, T, H * dv)
        if rows is None:
            out = np.empty((B, T, H * dv), dtype=np.float64)
            rp, n = None, B * T
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            out = np.empty((rows.shape[0], H * dv), dtype=np.float64)
            rp, n = _ptr(rows, ct.c_int64), rows.shape[0]
        self._check(self.lib.oracle_extend(
            _ptr(q, ct.c_float), _ptr(c, ct.c_float), _ptr(w_uk, ct.c_float), _ptr(w_uv, ct.c_float),
            _ptr(gate, ct.c_float), B, T, S, H, dq, dv, r, float(scale), rp, n,
            _ptr(out, ct.c_double), threads), "oracle_extend")
        return out

    def decode(self, q, c_cache, cu_seqlens, w_uk, w_uv, gate, scale: float, seqs=None,
               threads: int = 0) -> np.ndarray:
        """Decode.  Returns [B, H*dv] (or [len(seqs), H*dv]) float64."""
        q, c_cache, w_uk, w_uv, gate = map(_f32, (q, c_cache, w_uk, w_uv, gate))
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        B, H, dq = q.shape
        r = c_cache.shape[-1]
        dv = w_uv.shape[1]
        assert cu.shape == (B + 1,) and c_cache.shape == (int(cu[-1]), r)
        assert gate.shape == (B, H * dv)
        if seqs is None:
            sp, n = None, B
        else:
            seqs = np.ascontiguousarray(seqs, dtype=np.int64)
            sp, n = _ptr(seqs, ct.c_int64), seqs.shape[0]
        out = np.empty((n, H * dv), dtype=np.float64)
        self._check(self.lib.oracle_decode(
            _ptr(q, ct.c_float), _ptr(c_cache, ct.c_float), _ptr(cu, ct.c_int64),
            _ptr(w_uk, ct.c_float), _ptr(w_uv, ct.c_float), _ptr(gate, ct.c_float),
            B, H, dq, dv, r, float(scale), sp, n, _ptr(out, ct.c_double), threads), "oracle_decode")
        return out

    def prefill_decompressed(self, q, c, w_uk, w_uv, gate, scale: float, threads: int = 0) -> np.ndarray:
        q, c, w_uk, w_uv, gate = map(_f32, (q, c, w_uk, w_uv, gate))
        B, T, H, dq = q.shape
        r = c.shape[-1]
        dv = w_uv.shape[1]
        out = np.empty((B, T, H * dv), dtype=np.float64)
        self._check(self.lib.oracle_prefill_decompressed(
            _ptr(q, ct.c_float), _ptr(c, ct.c_float), _ptr(w_uk, ct.c_float), _ptr(w_uv, ct.c_float),
            _ptr(gate, ct.c_float), B, T, H, dq, dv, r, float(scale), _ptr(out, ct.c_double), threads),
            "oracle_prefill_decompressed")
        return out

    def attn(self, q, c, w_uk, scale: float) -> np.ndarray:
        """Attention weights [B,H,T,T] (tiny shapes only)."""
        q, c, w_uk = map(_f32, (q, c, w_uk))
        B, T, H, dq = q.shape
        r = c.shape[-1]
        out = np.empty((B, H, T, T), dtype=np.float64)
        self._check(self.lib.oracle_prefill_attn(
            _ptr(q, ct.c_float), _ptr(c, ct.c_float), _ptr(w_uk, ct.c_float), B, T, H, dq, r,
            float(scale), _ptr(out, ct.c_double)), "oracle_prefill_attn")
        return out

    def decode_paged(self, q, pages, block_table, seq_lens, w_uk, w_uv, gate, scale: float, seqs=None,
                     threads: int = 0) -> np.ndarray:
        """Decode against a paged cache: pages [num_pages, page_size, r],
        block_table [B, max_pages], seq_lens [B].  Returns [B, H*dv] (or
        [len(seqs), H*dv]) float64."""
        q, pages, w_uk, w_uv, gate = map(_f32, (q, pages, w_uk, w_uv, gate))
        bt = np.ascontiguousarray(block_table, dtype=np.int64)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int64)
        B, H, dq = q.shape
        npg, ps, r = pages.shape
        dv = w_uv.shape[1]
        assert bt.shape[0] == B and lens.shape == (B,) and gate.shape == (B, H * dv)
        if seqs is None:
            sp, n = None, B
        else:
            seqs = np.ascontiguousarray(seqs, dtype=np.int64)
            sp, n = _ptr(seqs, ct.c_int64), seqs.shape[0]
        out = np.empty((n, H * dv), dtype=np.float64)
        self._check(self.lib.oracle_decode_paged(
            _ptr(q, ct.c_float), _ptr(pages, ct.c_float), npg, ps, _ptr(bt, ct.c_int64), bt.shape[1],
            _ptr(lens, ct.c_int64), _ptr(w_uk, ct.c_float), _ptr(w_uv, ct.c_float), _ptr(gate, ct.c_float),
            B, H, dq, dv, r, float(scale), sp, n, _ptr(out, ct.c_double), threads), "oracle_decode_paged")
        return out

    def extend_paged(self, q, pages, block_table, S: int, w_uk, w_uv, gate, scale: float, rows=None,
                     threads: int = 0) -> np.ndarray:
        """Chunked prefill against a paged cache holding S rows per
        sequence.  Returns [B,T,H*dv] or [len(rows), H*dv] (float64)."""
        q, pages, w_uk, w_uv, gate = map(_f32, (q, pages, w_uk, w_uv, gate))
        bt = np.ascontiguousarray(block_table, dtype=np.int64)
        B, T, H, dq = q.shape
        npg, ps, r = pages.shape
        dv = w_uv.shape[1]
        assert bt.shape[0] == B and gate.shape == (B, T, H * dv)
        if rows is None:
            out = np.empty((B, T, H * dv), dtype=np.float64)
            rp, n = None, B * T
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            out = np.empty((rows.shape[0], H * dv), dtype=np.float64)
            rp, n = _ptr(rows, ct.c_int64), rows.shape[0]
        self._check(self.lib.oracle_extend_paged(
            _ptr(q, ct.c_float), _ptr(pages, ct.c_float), npg, ps, _ptr(bt, ct.c_int64), bt.shape[1],
            _ptr(w_uk, ct.c_float), _ptr(w_uv, ct.c_float), _ptr(gate, ct.c_float), B, T, int(S), H, dq, dv, r,
            float(scale), rp, n, _ptr(out, ct.c_double), threads), "oracle_extend_paged")
        return out

    def extend_varlen_paged(self, q, pages, block_table, cu_q, seq_lens, w_uk, w_uv, gate, scale: float,
                            threads: int = 0) -> np.ndarray:
        """Varlen chunked prefill: q [Nq,H,dq] packed by cu_q [B+1], seq_lens
        [B] cache rows per sequence (the chunk is the last T_b of them).
        Returns [Nq, H*dv] float64."""
        q, pages, w_uk, w_uv, gate = map(_f32, (q, pages, w_uk, w_uv, gate))
        bt = np.ascontiguousarray(block_table, dtype=np.int64)
        cu = np.ascontiguousarray(cu_q, dtype=np.int64)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int64)
        Nq, H, dq = q.shape
        npg, ps, r = pages.shape
        dv = w_uv.shape[1]
        B = lens.shape[0]
        assert cu.shape == (B + 1,) and cu[-1] == Nq and bt.shape[0] == B and gate.shape == (Nq, H * dv)
        out = np.zeros((Nq, H * dv), dtype=np.float64)
        self._check(self.lib.oracle_extend_varlen_paged(
            _ptr(q, ct.c_float), _ptr(pages, ct.c_float), npg, ps, _ptr(bt, ct.c_int64), bt.shape[1],
            _ptr(cu, ct.c_int64), _ptr(lens, ct.c_int64), _ptr(w_uk, ct.c_float), _ptr(w_uv, ct.c_float),
            _ptr(gate, ct.c_float), B, H, dq, dv, r, float(scale), _ptr(out, ct.c_double), threads),
            "oracle_extend_varlen_paged")
        return out

    def cache_append(self, c_new, pages, block_table, positions) -> np.ndarray:
        """Returns a copy of pages [num_pages, page_size, r] (float32) with
        row c_new[i] written at position positions[i] of sequence i."""
        c_new = _f32(c_new)
        pages = np.array(pages, dtype=np.float32, order="C", copy=True)
        bt = np.ascontiguousarray(block_table, dtype=np.int64)
        pos = np.ascontiguousarray(positions, dtype=np.int64)
        npg, ps, r = pages.shape
        B = c_new.shape[0]
        assert c_new.shape == (B, r) and bt.shape[0] == B and pos.shape == (B,)
        self._check(self.lib.oracle_cache_append(
            _ptr(c_new, ct.c_float), _ptr(pages, ct.c_float), npg, ps, _ptr(bt, ct.c_int64), bt.shape[1],
            _ptr(pos, ct.c_int64), B, r), "oracle_cache_append")
        return pages

    def prefill_backward(self, q, c, w_uk, w_uv, gate, dout, scale: float, threads: int = 0) -> dict:
        """Gradients of the prefill core given dout [B,T,H*dv]: dict with dq
        [B,T,H,dq], dc [B,T,r], dw_uk [H,dq,r], dw_uv [H,dv,r], dgate
        [B,T,H*dv] (float64)."""
        q, c, w_uk, w_uv, gate, dout = map(_f32, (q, c, w_uk, w_uv, gate, dout))
        B, T, H, dq = q.shape
        r = c.shape[-1]
        dv = w_uv.shape[1]
        assert c.shape == (B, T, r) and w_uk.shape == (H, dq, r) and w_uv.shape == (H, dv, r)
        assert gate.shape == (B, T, H * dv) and dout.shape == gate.shape
        g = dict(dq=np.empty((B, T, H, dq)), dc=np.empty((B, T, r)), dw_uk=np.empty((H, dq, r)),
                 dw_uv=np.empty((H, dv, r)), dgate=np.empty((B, T, H * dv)))
        self._check(self.lib.oracle_prefill_backward(
            *[_ptr(a, ct.c_float) for a in (q, c, w_uk, w_uv, gate, dout)], B, T, H, dq, dv, r, float(scale),
            *[_ptr(g[k], ct.c_double) for k in ("dq", "dc", "dw_uk", "dw_uv", "dgate")], threads),
            "oracle_prefill_backward")
        return g

    def prefill_lse(self, q, c, w_uk, scale: float, threads: int = 0) -> np.ndarray:
        """Natural-log log-sum-exp of each causal score row, [B, H, T]."""
        q, c, w_uk = map(_f32, (q, c, w_uk))
        B, T, H, dq = q.shape
        r = c.shape[-1]
        out = np.empty((B, H, T), dtype=np.float64)
        self._check(self.lib.oracle_prefill_lse(_ptr(q, ct.c_float), _ptr(c, ct.c_float), _ptr(w_uk, ct.c_float),
                                                B, T, H, dq, r, float(scale), _ptr(out, ct.c_double), threads),
                    "oracle_prefill_lse")
        return out

    GRAD_KEYS = ("dx", "dw_kv_down", "dkv_norm", "dw_q_down", "dq_norm", "dw_q_up", "dw_uk", "dw_uv", "dw_gate",
                 "dw_o")

    def forward_backward(self, x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o, dy,
                         eps: float, scale: float, threads: int = 0) -> dict:
        """Gradients of the full layer given dy [B,T,D] (stage results of
        the forward stored as float32): dict keyed by GRAD_KEYS, float64."""
        x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o, dy = map(
            _f32, (x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o, dy))
        B, T, D = x.shape
        r = w_kv_down.shape[0]
        q_rank = w_q_down.shape[0]
        H, dq, _ = w_uk.shape
        dv = w_uv.shape[1]
        assert dy.shape == x.shape
        shapes = dict(dx=x.shape, dw_kv_down=w_kv_down.shape, dkv_norm=kv_norm.shape, dw_q_down=w_q_down.shape,
                      dq_norm=q_norm.shape, dw_q_up=w_q_up.shape, dw_uk=w_uk.shape, dw_uv=w_uv.shape,
                      dw_gate=w_gate.shape, dw_o=w_o.shape)
        g = {k: np.empty(shapes[k], dtype=np.float64) for k in self.GRAD_KEYS}
        self._check(self.lib.oracle_forward_backward(
            *[_ptr(a, ct.c_float) for a in (x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate,
                                             w_o, dy)],
            B, T, D, q_rank, H, dq, dv, r, float(eps), float(scale), *[_ptr(g[k], ct.c_double) for k in self.GRAD_KEYS],
            threads), "oracle_forward_backward")
        return g

    def kda(self, q, k, v, g, beta, s0=None, G: int = 1, threads: int = 0):
        """chunk_kda's recurrence: returns (o [B,T,G*H,V], final state
        [B,G*H,K,V]), float64; q, k [B,T,H,K], v [B,T,G*H,V], g [B,T,G*H,K],
        beta [B,T,G*H], s0 [B,G*H,K,V] or None (zero state)."""
        q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
        B, T, H, K = q.shape
        V = v.shape[3]
        HV = G * H
        assert k.shape == q.shape and v.shape == (B, T, HV, V) and g.shape == (B, T, HV, K)
        assert beta.shape == (B, T, HV)
        s0p = None
        if s0 is not None:
            s0 = _f32(s0)
            assert s0.shape == (B, HV, K, V)
            s0p = _ptr(s0, ct.c_float)
        o = np.empty((B, T, HV, V), dtype=np.float64)
        st = np.empty((B, HV, K, V), dtype=np.float64)
        self._check(self.lib.oracle_kda(_ptr(q, ct.c_float), _ptr(k, ct.c_float), _ptr(v, ct.c_float),
                                        _ptr(g, ct.c_float), _ptr(beta, ct.c_float), s0p, B, T, H, G, K, V,
                                        _ptr(o, ct.c_double), _ptr(st, ct.c_double), threads), "oracle_kda")
        return o, st

    def round_bf16(self, v) -> np.ndarray:
        """Nearest bf16 value of each element (ties to even), as float64."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty_like(v)
        self._check(self.lib.oracle_round_bf16(_ptr(v, ct.c_double), v.size, _ptr(out, ct.c_double)),
                    "oracle_round_bf16")
        return out

    STAGE_F32 = 0
    STAGE_BF16 = 1

    def forward(self, x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o,
                eps: float, scale: float, stage: int = 0, rows=None, stages: bool = False,
                threads: int = 0):
        """Full Gated MLA forward: x [B,T,D] -> y [B,T,D] (rows None) or
        [len(rows), D] (float64).  stage: STAGE_F32 / STAGE_BF16, the
        storage type of the stage results.  stages=True also returns a dict
        with c [B*T,r], q [n,H*dq], gate [n,H*dv] and o [n,H*dv] as stored."""
        x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o = map(
            _f32, (x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o))
        B, T, D = x.shape
        r = w_kv_down.shape[0]
        q_rank = w_q_down.shape[0]
        H, dq, _ = w_uk.shape
        dv = w_uv.shape[1]
        assert w_kv_down.shape == (r, D) and kv_norm.shape == (r,)
        assert w_q_down.shape == (q_rank, D) and q_norm.shape == (q_rank,)
        assert w_q_up.shape == (H * dq, q_rank) and w_uk.shape == (H, dq, r) and w_uv.shape == (H, dv, r)
        assert w_gate.shape == (H * dv, D) and w_o.shape == (D, H * dv)
        if rows is None:
            rp, n = None, B * T
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            rp, n = _ptr(rows, ct.c_int64), rows.shape[0]
        y = np.empty((n, D), dtype=np.float64)
        st = dict(c=np.empty((B * T, r)), q=np.empty((n, H * dq)), gate=np.empty((n, H * dv)),
                  o=np.empty((n, H * dv))) if stages else None
        sp = [(_ptr(st[k], ct.c_double) if stages else None) for k in ("c", "q", "gate", "o")]
        self._check(self.lib.oracle_forward(
            *[_ptr(a, ct.c_float) for a in (x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv,
                                             w_gate, w_o)],
            B, T, D, q_rank, H, dq, dv, r, float(eps), float(scale), int(stage), rp, n,
            _ptr(y, ct.c_double), *sp, threads), "oracle_forward")
        if rows is None:
            y = y.reshape(B, T, D)
        return (y, st) if stages else y


_default = None


def get() -> Oracle:
    """The default (non-mutant) oracle, built on first use if missing.  With
    ORACLE_SANITIZE=1 in the environment, the ASan/UBSan build instead."""
    global _default
    if _default is None:
        san = os.environ.get("ORACLE_SANITIZE") == "1"
        path = LIB_SANITIZED if san else LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
            build(path, sanitize=san)
        _default = Oracle(path)
    return _default


def build_mutant(mutant: int, directory: str | None = None) -> Oracle:
    """Build and load a planted-mistake variant into a scratch directory."""
    directory = directory or tempfile.mkdtemp(prefix="oracle_mut_")
    path = os.path.join(directory, f"liboracle_mut{mutant}.so")
    build(path, mutant=mutant)
    return Oracle(path)
