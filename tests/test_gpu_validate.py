"""pa_validate_tables and pa_validate_writes through the C ABI: the violation count of corrupted
tables, lengths and query ranges, and of cache writes and copy pairs that would race, equals a
count made on the host from the rule include/pa.h states, and a valid batch counts zero. The
count is cleared by the call itself (checked by calling twice)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_384_amd as pa
from paged_kv_cache_384_amd import workloads as wl
from _gpu_cases import log

pytestmark = pytest.mark.gpu


def host_count(tables, ctx, max_ctx, B, NB, qs=None):
    n_bad = 0
    for s in range(len(ctx)):
        n = int(ctx[s])
        n_bad += n < 0 or n > max_ctx
        used = min(max(n, 0), max_ctx)
        for j in range((used + B - 1) // B):
            n_bad += not (0 <= int(tables[s, j]) < NB)
        if qs is not None:
            if s == 0:
                n_bad += int(qs[0]) != 0
            q = int(qs[s + 1]) - int(qs[s])
            n_bad += q < 0 or q > max(n, 0)
    return n_bad


def run(kp, tables, ctx, max_ctx, d, qs=None):
    dev = kp.device
    v = torch.full((1,), 12345, dtype=torch.int32, device=dev)
    args = dict(head_dim=d, query_start=None if qs is None else torch.from_numpy(qs).to(dev))
    bt_d = torch.from_numpy(np.ascontiguousarray(tables)).to(dev)
    ctx_d = torch.from_numpy(np.ascontiguousarray(ctx)).to(dev)
    pa.pa_validate_tables(kp, bt_d, ctx_d, max_ctx, v, **args)
    first = int(v.item())
    pa.pa_validate_tables(kp, bt_d, ctx_d, max_ctx, v, **args)
    assert int(v.item()) == first  # cleared by the call, not accumulated
    return first


def test_validate_decode_tables():
    cfg = wl.DecodeConfig("val_f16", "f16", num_seqs=6, num_q_heads=4, num_kv_heads=2,
                          head_dim=64, block_size=16, ctx=("uniform", 40, 300), seed=31)
    b = wl.build_batch(cfg)
    NB, B, W = b.num_blocks, cfg.block_size, b.max_blocks_per_seq
    kp = torch.zeros((NB, cfg.num_kv_heads, B * cfg.head_dim), dtype=torch.float16,
                     device="cuda:0")
    tables, ctx = b.block_tables.copy(), b.context_lens.copy()
    max_ctx = int(b.max_context_len)
    assert run(kp, tables, ctx, max_ctx, cfg.head_dim) == 0
    # corrupt: used entries out of the pool, an unused entry (not counted), a length above the
    # bound and a negative length
    nb0 = (int(ctx[0]) + B - 1) // B
    tables[0, 0] = -1
    tables[1, (int(ctx[1]) - 1) // B] = NB
    unused = (int(ctx[2]) + B - 1) // B
    if unused < W:
        tables[2, unused] = -7
    ctx[3] = max_ctx + 5
    ctx[4] = -3
    tables[5, :] = NB + 100  # every used entry of sequence 5
    want = host_count(tables, ctx, max_ctx, B, NB)
    got = run(kp, tables, ctx, max_ctx, cfg.head_dim)
    log(f"[validate] decode tables: {got} violations (host count {want}, seq 0 uses {nb0} blocks)")
    assert got == want and got >= 4


def test_validate_query_ranges():
    cfg = wl.DecodeConfig("val_q_bf16", "bf16", num_seqs=5, num_q_heads=2, num_kv_heads=2,
                          head_dim=128, block_size=32, ctx=("uniform", 50, 400),
                          new_tokens=("uniform", 1, 40), seed=32)
    b = wl.build_batch(cfg)
    NB, B = b.num_blocks, cfg.block_size
    kp = torch.zeros((NB, cfg.num_kv_heads, B * cfg.head_dim), dtype=torch.bfloat16,
                     device="cuda:0")
    tables, ctx = b.block_tables.copy(), b.context_lens.copy()
    qs = b.query_start.astype(np.int32).copy()
    max_ctx = int(b.max_context_len)
    assert run(kp, tables, ctx, max_ctx, cfg.head_dim, qs) == 0
    ctx[1] = int(qs[2] - qs[1]) - 1          # q_len > n
    qs[3] = qs[2] - 1                        # decreasing: q_len of seq 2 < 0 (and seq 3 grows)
    bad_qs0 = qs.copy()
    bad_qs0[0] = 1                           # query_start[0] != 0
    for q in (qs, bad_qs0):
        want = host_count(tables, ctx, max_ctx, B, NB, q)
        got = run(kp, tables, ctx, max_ctx, cfg.head_dim, q)
        log(f"[validate] query ranges: {got} violations (host count {want})")
        assert got == want and got >= 2


def test_validate_empty_batch_writes_zero():
    kp = torch.zeros((4, 1, 16 * 64), dtype=torch.float16, device="cuda:0")
    v = torch.full((1,), 7, dtype=torch.int32, device="cuda:0")
    bt = torch.zeros((0, 1), dtype=torch.int32, device="cuda:0")
    ctx = torch.zeros((0,), dtype=torch.int32, device="cuda:0")
    pa.pa_validate_tables(kp, bt, ctx, 16, v, head_dim=64)
    assert int(v.item()) == 0


# ---- pa_validate_writes: the write-race contract of cache writes and copy-on-write copies ----

def host_write_count(tables, seq, pos, pairs, B, NB):
    """The rule include/pa.h states for pa_validate_writes, counted on the host."""
    S, W = tables.shape
    bad = 0
    seen = set()
    for n in range(len(seq)):
        s, p = int(seq[n]), int(pos[n])
        if p < 0 or p >= W * B or s < 0 or s >= S:
            continue                                   # a token the cache write skips
        blk = int(tables[s, p // B])
        if not 0 <= blk < NB:
            bad += 1
            blk = min(max(blk, 0), NB - 1)             # where the clamped write lands
        slot = blk * B + p % B
        bad += slot in seen
        seen.add(slot)
    valid = [(int(a), int(b)) for a, b in np.asarray(pairs).reshape(-1, 2)
             if 0 <= a < NB and 0 <= b < NB]
    sources = {a for a, _ in valid}
    dests = set()
    for _, b in valid:
        bad += b in dests
        bad += b in sources
        dests.add(b)
    return bad


def run_writes(kp, d, tables, seq, pos, pairs):
    dev = kp.device
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    v = torch.full((1,), 12345, dtype=torch.int32, device=dev)
    kw = dict(head_dim=d, block_tables=t(tables), token_seq=t(seq), token_pos=t(pos),
              src_dst=t(np.asarray(pairs).reshape(-1)) if len(pairs) else None)
    pa.pa_validate_writes(kp, v, **kw)
    first = int(v.item())
    pa.pa_validate_writes(kp, v, **kw)
    assert int(v.item()) == first  # cleared by the call, not accumulated
    return first


def test_validate_writes_of_a_copy_on_write_step():
    """A valid shared-prefix decode step (copies, then one new token per sequence) counts zero;
    then single corruptions, each counted as the rule says."""
    cfg = wl.DecodeConfig("valw_f16", "f16", num_seqs=12, num_q_heads=4, num_kv_heads=4,
                          head_dim=128, ctx=("shared_prefix", 44, 1, 70, 4), seed=33)
    b = wl.build_batch(cfg)
    NB, B = b.num_blocks, cfg.block_size
    kp = torch.zeros((NB, cfg.num_kv_heads, B * cfg.head_dim), dtype=torch.float16,
                     device="cuda:0")
    tables, seq, pos = b.block_tables.copy(), b.token_seq.copy(), b.token_pos.copy()
    pairs = b.copy_pairs.copy()
    assert len(pairs) > 0 and run_writes(kp, 128, tables, seq, pos, pairs) == 0
    cases = {}
    s2 = seq.copy(); p2 = pos.copy()
    s2[3], p2[3] = s2[2], p2[2]                         # two tokens on one slot
    cases["same slot"] = (tables, s2, p2, pairs)
    t2 = tables.copy()
    last = lambda s: int(pos[s]) // B
    t2[5, last(5)] = -4                                 # an entry below the pool
    t2[6, last(6)] = NB + 9                             # and one above it
    cases["ids outside the pool"] = (t2, seq, pos, pairs)
    t3 = tables.copy()
    t3[7, last(7)] = t3[8, last(8)]                     # two sequences writing one block
    p3 = pos.copy()
    p3[7] = (int(pos[7]) // B) * B + int(pos[8]) % B    # ... at the same offset
    cases["shared block"] = (t3, seq, p3, pairs)
    sk = seq.copy(); pk = pos.copy()
    sk[1], pk[1] = sk[0], -1                            # skipped duplicates are not counted
    sk[4] = cfg.num_seqs + 3
    cases["skipped tokens"] = (tables, sk, pk, pairs)
    q1 = pairs.copy(); q1[1, 1] = q1[0, 1]              # a destination written twice
    cases["destination twice"] = (tables, seq, pos, q1)
    q2 = pairs.copy(); q2[2, 1] = q2[0, 0]              # a destination another pair reads
    cases["destination read"] = (tables, seq, pos, q2)
    q3 = pairs.copy(); q3[1] = (q3[1, 1], q3[1, 1])     # a block copied onto itself
    cases["self copy"] = (tables, seq, pos, q3)
    q4 = pairs.copy(); q4[0] = (NB, q4[1, 1])           # out of the pool: skipped, not counted
    cases["skipped pair"] = (tables, seq, pos, q4)
    for name, (t, s, p, q) in cases.items():
        want = host_write_count(t, s, p, q, B, NB)
        got = run_writes(kp, 128, t, s, p, q)
        log(f"[validate writes] {name}: {got} (host count {want})")
        assert got == want, name
        assert (got == 0) == (name in ("skipped tokens", "skipped pair")), name


def test_validate_writes_many_tokens_and_pairs():
    """A prefill-sized write set (several thousand tokens over many 256-item tiles) and hundreds
    of copy pairs, with collisions planted at random, including triples."""
    rng = np.random.default_rng(34)
    S, W, B, NB = 40, 64, 16, 3000
    tables = rng.permutation(NB)[:S * W].reshape(S, W).astype(np.int32)
    seq = np.repeat(np.arange(S), 150).astype(np.int32)
    pos = np.tile(np.arange(150), S).astype(np.int32)
    order = rng.permutation(len(seq))
    seq, pos = seq[order], pos[order]
    kp = torch.zeros((NB, 1, B * 64), dtype=torch.float16, device="cuda:0")
    pairs = np.stack([rng.permutation(NB)[:700], rng.permutation(NB)[:700]], 1).astype(np.int32)
    # distinct destinations that are no source, apart from what is planted below
    pool = np.setdiff1d(np.arange(NB), pairs[:, 0])
    pairs[:, 1] = rng.permutation(pool)[:700]
    assert run_writes(kp, 64, tables, seq, pos, pairs) == 0
    for k in rng.choice(len(seq), 40, replace=False):  # duplicate some tokens' slots
        j = int(rng.integers(len(seq)))
        seq[k], pos[k] = seq[j], pos[j]
    tables[rng.integers(S), rng.integers(W)] = NB + 1
    for k in rng.choice(700, 30, replace=False):
        j = int(rng.integers(700))
        pairs[k, 1] = pairs[j, int(rng.integers(2))]
    want = host_write_count(tables, seq, pos, pairs, B, NB)
    got = run_writes(kp, 64, tables, seq, pos, pairs)
    log(f"[validate writes] {len(seq)} tokens, {len(pairs)} pairs: {got} (host count {want})")
    assert got == want and got > 40


def test_validate_writes_nothing_to_check():
    kp = torch.zeros((4, 1, 16 * 64), dtype=torch.float16, device="cuda:0")
    v = torch.full((1,), 7, dtype=torch.int32, device="cuda:0")
    pa.pa_validate_writes(kp, v, head_dim=64)
    assert int(v.item()) == 0
