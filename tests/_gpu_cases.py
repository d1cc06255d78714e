"""One decode or prefill step through the HIP library (C ABI via the ctypes binding) and
through the CPU oracle on the same seeded inputs, with the comparisons the parity tests make.

A step is: copy_blocks for the copy-on-write pairs, reshape_and_cache of the new tokens (one per
sequence at position ctx - 1 for decode, the newest q_len for prefill), then the attention over
ctx tokens. Cache writes and copies are compared bit for bit over the whole pools; attention
within the stated tolerance.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

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
# unit roundoff of the 16-bit types the prefill kernel rounds its softmax weights to
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# fp32 slack on each weight: score products summed in fp32, the exponent's fma and exp2, and the
# rescaling when the running maximum moves (a few 2^-24 each; for unit-scale inputs at d <= 128
# the score sum's worst case is about 2^-14 relative on a weight)
WEIGHT_SLACK = 2.0 ** -12
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output type at each exact value: the error that
    storing the exact result in that type already makes (nearest-even rounding)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, MIN_NORMAL_EXP[dtype]), MIN_NORMAL_EXP[dtype])
    return np.ldexp(1.0, (e - MANT_BITS[dtype] - 1).astype(np.int64))


def parity_bar(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element bar on |out - oracle|: the stated tolerance (1e-5 fp32, 1e-2 fp16/bf16).
    Only where half a unit in the last place of the output type at the exact value reaches the
    tolerance itself (bf16 from |o| = 4, fp16 from 32, fp32 from 256) can no output meet it,
    since the exact value may sit halfway between two representable ones; there the bar is the
    tolerance plus that half unit."""
    h = half_ulp(ref, dtype)
    return np.where(h >= TOL[dtype], TOL[dtype] + h, TOL[dtype])


def prefill_bound(ref: np.ndarray, m2: np.ndarray, seen, vmax: float, dtype: str) -> np.ndarray:
    """Per-element bound on |out - oracle| that the prefill kernel's documented arithmetic
    guarantees.

    The kernel rounds every softmax weight p_t (at most 2^8, at least one of them >= 1, since
    the running maximum is always one of the scores) to the input type and divides by the sum
    of the same rounded weights, so its result is an exact weighted mean with perturbed weights:
        o~ - o = sum_t e_t (v_t - o) / sum_t p~_t,   |e_t| <= u p_t + tau,
    with u the type's unit roundoff (widened by the fp32 slack on each weight) and tau the
    absolute error below the type's normal range (fp16 subnormal spacing 2^-24, halved; none
    for bf16, whose range is fp32's). Hence, with w the exact weights, M2 = sum_t w_t v_t^2 (from
    the oracle) and sum_t w_t |v_t - o| <= sqrt(M2 - o^2):
        |o~ - o| <= u / (1 - u) * sqrt(M2 - o^2) + n * tau * 2 vmax / (1 - u)
    for n seen tokens and |v| <= vmax. The fp32 sums of the products add at most
    (ceil(n/32) + 4) * 2^-23 * sqrt(M2) (one rounding per 32-token matrix step, doubled), and
    storing the result in the output type adds half a unit in the last place at |o| plus all
    of that.
    seen: tokens each row attends to (broadcast against ref)."""
    u = UNIT_ROUNDOFF[dtype] + WEIGHT_SLACK
    tau = {"f16": 2.0 ** -25, "bf16": 0.0}[dtype]
    n = np.asarray(seen, dtype=np.float64)
    spread = np.sqrt(np.maximum(m2 - ref * ref, 0.0))
    acc = (np.ceil(n / 32.0) + 4.0) * 2.0 ** -23
    arith = (u * spread + n * tau * 2.0 * vmax) / (1.0 - u) + acc * np.sqrt(np.maximum(m2, 0.0))
    return arith + half_ulp(np.abs(ref) + arith, dtype)


def excess_error(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """Largest |got - ref| beyond the output type's own rounding of ref (reported beside the
    plain error; not a pass criterion)."""
    if np.size(ref) == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) - half_ulp(ref, dtype)))


def check_attention(got: np.ndarray, ref: np.ndarray, dtype: str, where: str) -> dict:
    """Assert |got - ref| <= parity_bar element by element; return the measured figures."""
    if np.size(ref) == 0:
        return {"max_abs_err": 0.0, "max_err_over_bar": 0.0, "allowance_elems": 0,
                "max_abs_out": 0.0}
    assert np.isfinite(got).all(), f"{where}: non-finite output"
    err = np.abs(got - ref)
    bar = parity_bar(ref, dtype)
    worst = int(np.argmax(err / bar))
    res = {"max_abs_err": float(err.max()), "max_err_over_bar": float((err / bar).max()),
           "allowance_elems": int((bar > TOL[dtype]).sum()),
           "max_abs_out": float(np.abs(ref).max())}
    assert (err <= bar).all(), (
        f"{where}: |out - oracle| = {err.flat[worst]:.4g} > bar {bar.flat[worst]:.4g} at "
        f"|o| = {abs(ref.flat[worst]):.4g} (max abs error {res['max_abs_err']:.4g})")
    return res


def merge_stats(parts):
    """Combine check_attention / prefill figures of several chunks (max of maxima, sums of
    counts)."""
    out = {}
    for p in parts:
        for k, v in p.items():
            if k in ("allowance_elems", "rows", "bound_over_tol_elems", "elements"):
                out[k] = out.get(k, 0) + v
            else:
                out[k] = max(out.get(k, v), v)
    return out


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
    res.update(check_decode(P, out, seqs, cfg.name))
    res["oracle_s"] = time.time() - t1
    return res


def _chunks(items, weights, n):
    """Split items into at most n lists of similar total weight (heaviest first)."""
    order = sorted(range(len(items)), key=lambda i: -weights[i])
    bins = [[] for _ in range(max(1, min(n, len(items))))]
    load = [0] * len(bins)
    for i in order:
        k = load.index(min(load))
        bins[k].append(items[i])
        load[k] += weights[i] + 1
    return [sorted(b) for b in bins if b]


def check_decode(P, out, seqs, where):
    """Oracle outputs of the given sequences (every query head), computed in worker threads
    over groups of sequences, compared with the kernel's stored outputs ``out`` element by
    element against parity_bar."""
    batch, dt = P.batch, P.dt
    if not len(seqs):
        return {"max_abs_err": 0.0, "max_err_over_bar": 0.0, "allowance_elems": 0,
                "max_abs_out": 0.0, "excess_err": 0.0}

    def work(group):
        ref = oracle.paged_decode_ref(P.q, P.kp, P.vp, batch.block_tables, batch.context_lens,
                                      P.cfg.scale, seqs=group, **P.kw)
        got = oracle.to_f64(out[group], dt)
        r = check_attention(got, ref, dt, f"{where} (seqs {group[:4]}...)")
        r["excess_err"] = excess_error(got, ref, dt)
        return r

    groups = _chunks(list(seqs), [int(batch.context_lens[s]) for s in seqs], 4 * WORKERS)
    with ThreadPoolExecutor(WORKERS) as ex:
        return merge_stats(list(ex.map(work, groups)))


def pool_abs_max(pool: np.ndarray, dtype: str) -> float:
    """Largest finite |element| of a stored pool (NaN poison ignored), in slices."""
    flat = pool.reshape(-1)
    top = 0.0
    step = 1 << 24
    for i in range(0, flat.size, step):
        x = np.abs(oracle.to_f64(flat[i:i + step], dtype))
        x = x[np.isfinite(x)]
        if x.size:
            top = max(top, float(x.max()))
    return top


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
    res.update(check_prefill(P, out, rows, ctx_ref, cfg.name))
    res["oracle_s"] = time.time() - t1
    # rows past max_query_len are not computed
    skipped = [int(qs[s]) + j for s in range(cfg.num_seqs) for j in range(mql, int(ql[s]))]
    if skipped:
        assert np.isnan(oracle.to_f64(out[skipped], dt)).all(), "rows past max_query_len written"
    return res


def check_prefill(P, out, rows, ctx_ref, where):
    """Oracle rows (dict seq -> query indices j) against the kernel's stored prefill output
    ``out``, element by element: the stated bar (parity_bar) and the bound the kernel's
    arithmetic guarantees (prefill_bound). Sequences are computed in worker threads."""
    batch, dt = P.batch, P.dt
    qs, ql = batch.query_start, batch.query_lens
    vmax = pool_abs_max(P.vp, dt)

    def work(s):
        js = rows[s]
        if not js:
            return {"rows": 0}
        ref = oracle.paged_prefill_ref(P.q, P.kp, P.vp, batch.block_tables, qs, ctx_ref,
                                       P.cfg.scale, seqs=[s], rows={s: js}, moments=True, **P.kw)
        o = np.stack([ref[(s, j)][0] for j in js])
        m2 = np.stack([ref[(s, j)][1] for j in js])
        got = oracle.to_f64(out[int(qs[s]) + np.asarray(js)], dt)
        r = check_attention(got, o, dt, f"{where} seq {s}")
        seen = np.maximum(int(ctx_ref[s]) - int(ql[s]) + np.asarray(js) + 1, 0)
        bound = prefill_bound(o, m2, seen[:, None, None], vmax, dt)
        err = np.abs(got - o)
        worst = np.unravel_index(int(np.argmax(err / bound)), err.shape)
        assert (err <= bound).all(), (
            f"{where} seq {s} query {js[worst[0]]}: |out - oracle| = {err[worst]:.4g} > "
            f"arithmetic bound {bound[worst]:.4g}")
        r.update(rows=len(js), max_err_over_bound=float((err / bound).max()),
                 bound_over_tol_elems=int((bound > TOL[dt]).sum()), elements=int(err.size),
                 excess_err=excess_error(got, o, dt))
        return r

    seqs = sorted(rows)
    order = sorted(seqs, key=lambda s: -len(rows[s]) * int(ctx_ref[s]))
    with ThreadPoolExecutor(WORKERS) as ex:
        return merge_stats(list(ex.map(work, order)))
