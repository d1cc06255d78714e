"""One decode or prefill step through the HIP library (C ABI via the ctypes binding) and
through the CPU oracle on the same seeded inputs, with the comparisons the parity tests make.

A step is: copy_blocks for the copy-on-write pairs, reshape_and_cache of the new tokens (one per
sequence at position ctx - 1 for decode, the newest q_len for prefill), then the attention over
ctx tokens. Cache writes and copies are compared bit for bit over the whole pools; attention
within the stated tolerance.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import paged_kv_cache_384_amd as pa
from paged_kv_cache_384_amd import workloads as wl
from _helpers import NAN_BITS, to_storage

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
U = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
MANT_BITS = {"f32": 23, "f16": 10, "bf16": 7}
MIN_NORMAL_EXP = {"f32": -126, "f16": -14, "bf16": -126}


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output type at each exact value: the error that
    storing the exact result in that type already makes (nearest-even rounding)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, MIN_NORMAL_EXP[dtype]), MIN_NORMAL_EXP[dtype])
    return np.ldexp(1.0, (e - MANT_BITS[dtype] - 1).astype(np.int64))


def excess_error(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """Largest |got - ref| beyond the output type's own rounding of ref. The tolerance bounds
    the arithmetic; a 16-bit output of magnitude 4 or more cannot be nearer than 2^-7 (bf16) to
    an exact value that falls between two representable ones, whatever the arithmetic."""
    if np.size(ref) == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) - half_ulp(ref, dtype)))


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def poison_tails(batch, k_pool, v_pool):
    """NaN into the slots at or past ctx of each sequence's last block (through the oracle's
    own writer), except in blocks that are copy-on-write sources: their tail slots are copied
    into the sharers' private blocks this step, so they hold ordinary values."""
    cfg = batch.cfg
    B = cfg.block_size
    sources = set(batch.copy_pairs[:, 0].tolist())
    seqs, poss = [], []
    for s in range(cfg.num_seqs):
        n = int(batch.context_lens[s])
        nb = -(-n // B)
        if nb == 0 or int(batch.block_tables[s, nb - 1]) in sources:
            continue
        for p in range(n, nb * B):
            seqs.append(s)
            poss.append(p)
    if not seqs:
        return k_pool, v_pool
    T = len(seqs)
    nan = np.full((T, cfg.num_kv_heads, cfg.head_dim), NAN_BITS[cfg.dtype],
                  dtype=k_pool.dtype)
    return oracle.reshape_and_cache_ref(
        k_pool, v_pool, nan, nan, batch.block_tables, np.array(seqs, np.int32),
        np.array(poss, np.int32), dtype=cfg.dtype, num_kv_heads=cfg.num_kv_heads,
        block_size=B, head_dim=cfg.head_dim)


def same_bits(a: np.ndarray, b: np.ndarray, dtype: str) -> bool:
    return np.array_equal(a.view(U[dtype]), b.view(U[dtype]))


class Prepared:
    """A batch, its seeded values as host storage arrays (pools with poisoned tails) and the
    same on the GPU."""

    def __init__(self, cfg, *, device_values=False, poison=True, value_seed=0):
        dev = torch.device("cuda:0")
        self.cfg = cfg
        self.batch = batch = wl.build_batch(cfg)
        vals = wl.make_values(batch, device=dev if device_values else "cpu", seed=value_seed)
        kp = to_storage(vals["k_pool"])
        vp = to_storage(vals["v_pool"])
        if poison:
            kp, vp = poison_tails(batch, kp, vp)
        self.kp, self.vp = kp, vp
        self.q = to_storage(vals["query"])
        self.key = to_storage(vals["key"])
        self.val = to_storage(vals["value"])
        self.dt = cfg.dtype
        tdt = vals["query"].dtype

        def up(a):
            return (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt)
                    if self.dt == "bf16" else torch.from_numpy(np.ascontiguousarray(a))).to(dev)

        self.kp_d, self.vp_d = up(kp), up(vp)
        self.q_d, self.key_d, self.val_d = up(self.q), up(self.key), up(self.val)
        self.bt_d = torch.from_numpy(batch.block_tables).to(dev)
        self.ctx_d = torch.from_numpy(batch.context_lens).to(dev)
        self.seq_d = torch.from_numpy(batch.token_seq).to(dev)
        self.pos_d = torch.from_numpy(batch.token_pos).to(dev)
        self.qs_d = torch.from_numpy(batch.query_start).to(dev)
        self.pairs_d = torch.from_numpy(batch.copy_pairs.reshape(-1)).to(dev)
        self.kw = dict(dtype=self.dt, num_kv_heads=cfg.num_kv_heads, block_size=cfg.block_size,
                       head_dim=cfg.head_dim)

    def write_cache(self, check_pools=True):
        """Copy-on-write copies, then the new tokens into their slots, on both sides."""
        batch, dt, kw = self.batch, self.dt, self.kw
        if batch.copy_pairs.shape[0]:
            pa.pa_copy_blocks(self.kp_d, self.vp_d, self.pairs_d, head_dim=self.cfg.head_dim)
            torch.cuda.synchronize()
            self.kp, self.vp = oracle.copy_blocks_ref(self.kp, self.vp, batch.copy_pairs, **kw)
            if check_pools:
                assert same_bits(to_storage(self.kp_d), self.kp, dt), "copy_blocks: key pool differs"
                assert same_bits(to_storage(self.vp_d), self.vp, dt), "copy_blocks: value pool differs"
        pa.pa_reshape_and_cache(self.kp_d, self.vp_d, self.key_d, self.val_d, self.bt_d,
                                self.seq_d, self.pos_d)
        torch.cuda.synchronize()
        self.kp, self.vp = oracle.reshape_and_cache_ref(
            self.kp, self.vp, self.key, self.val, batch.block_tables, batch.token_seq,
            batch.token_pos, **kw)
        if check_pools:
            assert same_bits(to_storage(self.kp_d), self.kp, dt), "reshape_and_cache: key pool differs"
            assert same_bits(to_storage(self.vp_d), self.vp, dt), "reshape_and_cache: value pool differs"


def run_step(cfg, *, partition_size=0, sample=None, device_values=False, poison=True,
             check_pools=True, value_seed=0, shared_blocks=None, twin=False):
    """Run one step on the GPU and check it against the oracle.

    sample: None = every (seq, head) through the oracle; else a list of sequence ids whose
    outputs (all heads) the oracle computes.
    shared_blocks: the read-policy flag passed to pa_decode (None = whether the batch's tables
    share blocks).
    twin: the batch is laid out contiguously; also run pa_decode_contiguous (no table) and
    require it to give pa_decode's output bit for bit.
    Returns a dict of measured errors.
    """
    t0 = time.time()
    P = Prepared(cfg, device_values=device_values, poison=poison, value_seed=value_seed)
    batch, dt = P.batch, P.dt
    res = {"prep_s": time.time() - t0}
    # 1. copy-on-write copies, 2. new tokens into their slots
    P.write_cache(check_pools)
    # 3. attention
    out_d = torch.full_like(P.q_d, float("nan"))
    if shared_blocks is None:
        shared_blocks = batch.shares_blocks
    pa.pa_decode(out_d, P.q_d, P.kp_d, P.vp_d, P.bt_d, P.ctx_d, cfg.scale, batch.max_context_len,
                 partition_size, shared_blocks=shared_blocks)
    torch.cuda.synchronize()
    if twin:
        out2_d = torch.full_like(P.q_d, float("nan"))
        pa.pa_decode_contiguous(out2_d, P.q_d, P.kp_d, P.vp_d, P.ctx_d, cfg.scale,
                                batch.max_context_len, batch.max_blocks_per_seq, partition_size)
        torch.cuda.synchronize()
        assert same_bits(to_storage(out2_d), to_storage(out_d), dt), "contiguous twin differs"
    out = to_storage(out_d)
    seqs = list(range(cfg.num_seqs)) if sample is None else list(sample)
    t1 = time.time()
    ref = oracle.paged_decode_ref(P.q, P.kp, P.vp, batch.block_tables, batch.context_lens,
                                  cfg.scale, seqs=seqs, **P.kw)
    res["oracle_s"] = time.time() - t1
    got = oracle.to_f64(out[seqs], dt)
    assert np.isfinite(got).all(), "non-finite output"
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    res["max_abs_err"] = err
    res["excess_err"] = excess = excess_error(got, ref, dt)
    res["max_abs_out"] = float(np.abs(ref).max()) if ref.size else 0.0
    assert excess <= TOL[dt], (f"{cfg.name}: max abs error {err} ({excess} beyond the output "
                               f"rounding) > {TOL[dt]}")
    return res


def run_prefill(cfg, *, rows=None, device_values=False, poison=True, check_pools=True,
                value_seed=0, max_query_len=None, max_context_len=None, prepared=None):
    """One prefill step on the GPU (cache writes of every new token, then pa_prefill) checked
    against the oracle.

    rows: None = every query row through the oracle; else a dict seq -> list of query indices j.
    max_query_len: passed to pa_prefill (default: the batch's largest q_len); queries at or past
    it must be left untouched (NaN in the output buffer).
    max_context_len: passed to pa_prefill (default: the batch's longest context); longer
    contexts are truncated to it, on both sides.
    Returns a dict of measured errors.
    """
    t0 = time.time()
    P = prepared or Prepared(cfg, device_values=device_values, poison=poison,
                             value_seed=value_seed)
    batch, dt = P.batch, P.dt
    res = {"prep_s": time.time() - t0}
    P.write_cache(check_pools)
    mql = batch.max_query_len if max_query_len is None else max_query_len
    mcl = batch.max_context_len if max_context_len is None else max_context_len
    out_d = torch.full_like(P.q_d, float("nan"))
    pa.pa_prefill(out_d, P.q_d, P.kp_d, P.vp_d, P.bt_d, P.qs_d, P.ctx_d, cfg.scale, mql, mcl)
    torch.cuda.synchronize()
    out = to_storage(out_d)
    qs = batch.query_start
    ql = batch.query_lens
    if rows is None:
        rows = {s: list(range(min(int(ql[s]), mql))) for s in range(cfg.num_seqs)}
    rows = {s: [j for j in js if j < mql] for s, js in rows.items()}
    t1 = time.time()
    ctx_ref = np.minimum(batch.context_lens, mcl)
    ref = oracle.paged_prefill_ref(P.q, P.kp, P.vp, batch.block_tables, qs, ctx_ref, cfg.scale,
                                   seqs=sorted(rows), rows=rows, **P.kw)
    res["oracle_s"] = time.time() - t1
    err, excess, mx, n = 0.0, -1.0, 0.0, 0
    for (s, j), r in ref.items():
        got = oracle.to_f64(out[int(qs[s]) + j], dt)
        assert np.isfinite(got).all(), f"non-finite output at seq {s} query {j}"
        err = max(err, float(np.abs(got - r).max()))
        excess = max(excess, excess_error(got, r, dt))
        mx = max(mx, float(np.abs(r).max()))
        n += 1
    # rows past max_query_len are not computed
    skipped = [int(qs[s]) + j for s in range(cfg.num_seqs) for j in range(mql, int(ql[s]))]
    if skipped:
        assert np.isnan(oracle.to_f64(out[skipped], dt)).all(), "rows past max_query_len written"
    res.update(max_abs_err=err, excess_err=excess, max_abs_out=mx, rows=n)
    assert excess <= TOL[dt], (f"{cfg.name}: max abs error {err} ({excess} beyond the output "
                               f"rounding) > {TOL[dt]}")
    return res
