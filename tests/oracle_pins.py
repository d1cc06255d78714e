"""Checks that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError when the oracle
disagrees with: a library routine (torch's scaled_dot_product_attention, torch's dtype
conversions), a closed form, an invariance the pages state (paging, block size and sharing do
not change the result), brute-force enumeration, or the layout properties the library's header
promises. ``tests/test_oracle.py`` runs them; ``tests/test_oracle_mutations.py`` plants mistakes
in the oracle and checks that some pin catches each one.

Pages cited by title and section:
  "PagedAttention" (newikis.com), "수학적 공식": dense causal attention and its blocked form.
  "PagedAttention 심층 분석" (ryotta.opik.net), §2/§3: paging does not change results; blocked
  partial sums; block-table lookup pseudocode; §4 copy-on-write.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from _helpers import NAN_BITS, random_storage, to_storage

ESZ = {"f32": 4, "f16": 2, "bf16": 2}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _widen_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 tensor of stored elements via torch's own dtype conversion (not the oracle's)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.float64)


def make_case(rng, *, dtype="f32", S=3, Hq=4, Hkv=2, d=64, B=16, ctx=(1, 17, 40),
              num_blocks=None, poison=True):
    """Random contiguous K/V per sequence, written into scattered pool blocks.

    The pool is first filled with unrelated values (NaN when ``poison``); every position
    0..ctx-1 of each sequence is then written through ``reshape_and_cache_ref``.
    Returns a dict with the stored arrays and the ground-truth contiguous K/V.
    """
    import oracle
    ctx = np.asarray(ctx, dtype=np.int32)
    nbs = [-(-int(c) // B) for c in ctx]
    NB = num_blocks or (sum(nbs) + 3)
    order = rng.permutation(NB)
    poison_block = int(order[-1])
    maxb = max(max(nbs), 1) + 2
    tables = np.full((S, maxb), poison_block, dtype=np.int32)
    k = 0
    for s in range(S):
        tables[s, :nbs[s]] = order[k:k + nbs[s]]
        k += nbs[s]
    shape = (NB, Hkv, B * d)
    k_pool = random_storage(rng, shape, dtype)
    v_pool = random_storage(rng, shape, dtype)
    if poison:
        k_pool[...] = NAN_BITS[dtype]
        v_pool[...] = NAN_BITS[dtype]
    Ks = [random_storage(rng, (int(c), Hkv, d), dtype) for c in ctx]
    Vs = [random_storage(rng, (int(c), Hkv, d), dtype) for c in ctx]
    tok_seq = np.concatenate([np.full(int(c), s, np.int32) for s, c in enumerate(ctx)])
    tok_pos = np.concatenate([np.arange(int(c), dtype=np.int32) for c in ctx])
    if tok_seq.size:
        key = np.concatenate(Ks)
        val = np.concatenate(Vs)
        k_pool, v_pool = oracle.reshape_and_cache_ref(
            k_pool, v_pool, key, val, tables, tok_seq, tok_pos, dtype=dtype,
            num_kv_heads=Hkv, block_size=B, head_dim=d)
    q = random_storage(rng, (S, Hq, d), dtype)
    return dict(dtype=dtype, S=S, Hq=Hq, Hkv=Hkv, d=d, B=B, ctx=ctx, tables=tables,
                k_pool=k_pool, v_pool=v_pool, q=q, K=Ks, V=Vs, NB=NB,
                poison_block=poison_block, scale=np.float32(1.0 / math.sqrt(d)))


def decode(oracle, c, **over):
    args = dict(dtype=c["dtype"], num_kv_heads=c["Hkv"], block_size=c["B"], head_dim=c["d"])
    args.update(over)
    return oracle.paged_decode_ref(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"],
                                   c["scale"], **args)


# ---------------------------------------------------------------------------------------------
# dtype widening
# ---------------------------------------------------------------------------------------------

def pin_widening(oracle):
    rng = np.random.default_rng(11)
    bits16 = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    for dtype, arr in (("bf16", bits16), ("f16", bits16.view(np.float16)),
                       ("f32", rng.standard_normal(999).astype(np.float32) * 1e3)):
        mine = oracle.to_f64(arr, dtype)
        ref = _widen_torch(arr, dtype).numpy()
        both_nan = np.isnan(mine) & np.isnan(ref)
        assert np.array_equal(mine[~both_nan], ref[~both_nan]), dtype
        assert np.array_equal(np.isnan(mine), np.isnan(ref)), dtype


# ---------------------------------------------------------------------------------------------
# layout properties promised by the header
# ---------------------------------------------------------------------------------------------

LAYOUT_CASES = [(3, 16, 64, 4), (3, 16, 64, 2), (2, 16, 128, 2), (2, 16, 128, 4), (2, 8, 64, 2)]


def pin_layout(oracle):
    for Hkv, B, d, esz in LAYOUT_CASES:
        NB = 4
        kw = dict(num_kv_heads=Hkv, block_size=B, head_dim=d)
        b = np.arange(NB)[:, None, None, None]
        h = np.arange(Hkv)[None, :, None, None]
        t = np.arange(B)[None, None, :, None]
        i = np.arange(d)[None, None, None, :]
        ko = np.broadcast_to(oracle.k_offset(b, h, t, i, esz=esz, **kw), (NB, Hkv, B, d))
        vo = np.broadcast_to(oracle.v_offset(b, h, t, i, **kw), (NB, Hkv, B, d))
        total = NB * Hkv * B * d
        for off in (ko, vo):
            # a bijection onto the pool
            assert np.array_equal(np.sort(off.reshape(-1)), np.arange(total))
            # each (block, head) tile is one contiguous run, in (block, head) order
            for bb in range(NB):
                for hh in range(Hkv):
                    tile = np.sort(off[bb, hh].reshape(-1))
                    start = (bb * Hkv + hh) * B * d
                    assert np.array_equal(tile, np.arange(start, start + B * d))
        # value rows: a token's d elements are contiguous and in order
        assert np.array_equal(vo[..., 1:] - vo[..., :-1], np.ones_like(vo[..., 1:]))
        # key chunk rows: with W = 64 bytes of elements, chunk c of a tile holds slot 0..B-1's
        # W elements back to back: B*64 contiguous bytes, slot t at byte t*64 of the row
        W = 64 // esz
        for c in range(d // W):
            rows = ko[..., c * W:(c + 1) * W]                      # [NB, Hkv, B, W]
            row_start = rows[:, :, 0, 0]
            expect = (row_start[:, :, None, None] + np.arange(B)[:, None] * W
                      + np.arange(W)[None, :])
            assert np.array_equal(rows, expect)
            tile_start = (np.arange(NB)[:, None] * Hkv + np.arange(Hkv)[None, :]) * B * d
            assert np.array_equal(row_start, tile_start + c * B * W)


# ---------------------------------------------------------------------------------------------
# slot computation and cache writes
# ---------------------------------------------------------------------------------------------

def pin_slot_enumeration(oracle):
    rng = np.random.default_rng(3)
    for B in (1, 4, 16):
        table = rng.permutation(50)[:9]
        enumerated = [int(b) * B + o for b in table for o in range(B)]
        for pos in range(len(table) * B):
            assert oracle.slot_of(table, pos, B) == enumerated[pos]


def pin_cache_round_trip(oracle):
    """Tokens written through the block table come back, bit for bit, through the gather."""
    rng = np.random.default_rng(5)
    for dtype in ("f32", "f16", "bf16"):
        c = make_case(rng, dtype=dtype, S=3, Hq=2, Hkv=2, d=64, ctx=(1, 16, 45))
        for s in range(c["S"]):
            K, V = oracle.gather_sequence_kv(c["k_pool"], c["v_pool"], c["tables"][s],
                                             c["ctx"][s], dtype=dtype, num_kv_heads=c["Hkv"],
                                             block_size=c["B"], head_dim=c["d"])
            assert np.array_equal(K, _widen_torch(c["K"][s], dtype).numpy())
            assert np.array_equal(V, _widen_torch(c["V"][s], dtype).numpy())


def pin_cache_write_footprint(oracle):
    """A write changes exactly the new tokens' elements and copies their bits (NaN payloads
    included); a negative position writes nothing."""
    rng = np.random.default_rng(6)
    for dtype in ("f16", "bf16", "f32"):
        Hkv, d, B, NB = 3, 64, 16, 10
        k_pool = random_storage(rng, (NB, Hkv, B * d), dtype)
        v_pool = random_storage(rng, (NB, Hkv, B * d), dtype)
        tables = rng.permutation(NB)[:8].reshape(2, 4).astype(np.int32)
        key = random_storage(rng, (3, Hkv, d), dtype)
        val = random_storage(rng, (3, Hkv, d), dtype)
        key.reshape(-1)[5] = NAN_BITS[dtype]
        seq = np.array([0, 1, 1], np.int32)
        pos = np.array([17, 63, -1], np.int32)
        k2, v2 = oracle.reshape_and_cache_ref(k_pool, v_pool, key, val, tables, seq, pos,
                                              dtype=dtype, num_kv_heads=Hkv, block_size=B,
                                              head_dim=d)
        u = {2: np.uint16, 4: np.uint32}[ESZ[dtype]]
        for before, after, src in ((k_pool, k2, key), (v_pool, v2, val)):
            diff = before.view(u) != after.view(u)
            # at most the 2 written tokens' Hkv*d elements change
            assert diff.sum() <= 2 * Hkv * d
            changed_vals = np.sort(after.view(u)[diff])
            written = np.sort(src[:2].view(u).reshape(-1))
            # every changed element now holds a value from the written tokens
            assert np.isin(changed_vals, written).all()
            # and every written element is found in the pool
            assert np.isin(written, after.view(u)).all()


def pin_copy_blocks(oracle):
    rng = np.random.default_rng(8)
    c = make_case(rng, dtype="f16", S=2, Hq=2, Hkv=2, d=64, ctx=(40, 21), poison=False)
    src = int(c["tables"][1, 1])                          # seq 1's last (partial) block
    free = sorted(set(range(c["NB"])) - set(c["tables"].reshape(-1).tolist()))
    dst = free[0]
    k2, v2 = oracle.copy_blocks_ref(c["k_pool"], c["v_pool"], [[src, dst]], dtype="f16",
                                    num_kv_heads=2, block_size=16, head_dim=64)
    u = np.uint16
    # block-granular: only block dst changed, and it now equals block src
    for before, after in ((c["k_pool"], k2), (c["v_pool"], v2)):
        changed_blocks = np.nonzero((before.view(u) != after.view(u)).any(axis=(1, 2)))[0]
        assert set(changed_blocks.tolist()) <= {dst}
        assert np.array_equal(after.view(u)[dst], before.view(u)[src])
    # remapping the table entry to the copy leaves attention unchanged
    c2 = dict(c, k_pool=k2, v_pool=v2, tables=c["tables"].copy())
    c2["tables"][1, 1] = dst
    assert np.array_equal(decode(oracle, c), decode(oracle, c2))


# ---------------------------------------------------------------------------------------------
# attention against a library routine
# ---------------------------------------------------------------------------------------------

def _sdpa(c):
    """torch scaled_dot_product_attention in float64 over each sequence's contiguous K/V."""
    outs = []
    scale = float(c["scale"])
    for s in range(c["S"]):
        q = _widen_torch(c["q"][s], c["dtype"])[None, :, None, :]          # [1, Hq, 1, d]
        if int(c["ctx"][s]) == 0:
            outs.append(torch.zeros(c["Hq"], c["d"], dtype=torch.float64))
            continue
        K = _widen_torch(c["K"][s], c["dtype"]).permute(1, 0, 2)[None]     # [1, Hkv, n, d]
        V = _widen_torch(c["V"][s], c["dtype"]).permute(1, 0, 2)[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            q, K.contiguous(), V.contiguous(), scale=scale,
            enable_gqa=c["Hq"] != c["Hkv"])
        outs.append(o[0, :, 0, :])
    return torch.stack(outs).numpy()


def pin_sdpa(oracle):
    rng = np.random.default_rng(21)
    cases = [
        dict(dtype="f32", S=3, Hq=4, Hkv=4, d=64, ctx=(1, 17, 200)),
        dict(dtype="f16", S=4, Hq=6, Hkv=2, d=128, ctx=(16, 15, 33, 100)),
        dict(dtype="bf16", S=3, Hq=8, Hkv=2, d=128, ctx=(48, 5, 129)),
        dict(dtype="f16", S=2, Hq=3, Hkv=3, d=64, B=8, ctx=(9, 70)),
    ]
    for kw in cases:
        c = make_case(rng, **kw)
        mine = decode(oracle, c)
        ref = _sdpa(c)
        assert np.abs(mine - ref).max() <= 1e-12, kw


# ---------------------------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------------------------

def pin_closed_forms(oracle):
    rng = np.random.default_rng(31)
    # a two-token case worked by hand: q.k = (1, 0) with scale 1 gives weights e:1
    d = 64
    c = make_case(rng, dtype="f32", S=1, Hq=1, Hkv=1, d=d, ctx=(2,), poison=False)
    q = np.zeros((1, 1, d), np.float32); q[0, 0, 0] = 1
    K = np.zeros((2, 1, d), np.float32); K[0, 0, 0] = 1; K[1, 0, 1] = 1
    V = np.zeros((2, 1, d), np.float32); V[0, 0, :2] = (1, 2); V[1, 0, :2] = (3, 4)
    kp, vp = oracle.reshape_and_cache_ref(c["k_pool"], c["v_pool"], K, V, c["tables"],
                                          np.zeros(2, np.int32), np.arange(2, dtype=np.int32),
                                          dtype="f32", num_kv_heads=1, block_size=16,
                                          head_dim=d)
    o = oracle.paged_decode_ref(q, kp, vp, c["tables"], c["ctx"], 1.0, dtype="f32",
                                num_kv_heads=1, block_size=16, head_dim=d)[0, 0]
    e = math.e
    assert abs(o[0] - (e * 1 + 3) / (e + 1)) < 1e-15
    assert abs(o[1] - (e * 2 + 4) / (e + 1)) < 1e-15
    assert np.all(o[2:] == 0)

    for dtype in ("f32", "bf16"):
        # identical keys: every weight equal, output = mean of the values
        c = make_case(rng, dtype=dtype, S=2, Hq=2, Hkv=2, d=64, ctx=(37, 5), poison=False)
        for s in range(2):
            n = int(c["ctx"][s])
            K = np.broadcast_to(c["K"][s][:1], c["K"][s].shape).copy()
            tok = np.arange(n, dtype=np.int32)
            kp, _ = oracle.reshape_and_cache_ref(c["k_pool"], c["v_pool"], K, c["V"][s],
                                                 c["tables"], np.full(n, s, np.int32), tok,
                                                 dtype=dtype, num_kv_heads=2, block_size=16,
                                                 head_dim=64)
            c["k_pool"] = kp
            c["K"][s] = K
        o = decode(oracle, c)
        for s in range(2):
            mean = _widen_torch(c["V"][s], dtype).numpy().mean(axis=0)       # [Hkv, d]
            assert np.abs(o[s] - mean).max() < 1e-13
        # scale 0: uniform weights again
        c = make_case(rng, dtype=dtype, S=2, Hq=4, Hkv=2, d=64, ctx=(33, 70), poison=False)
        o = oracle.paged_decode_ref(c["q"], c["k_pool"], c["v_pool"], c["tables"], c["ctx"],
                                    0.0, dtype=dtype, num_kv_heads=2, block_size=16,
                                    head_dim=64)
        for s in range(2):
            mean = _widen_torch(c["V"][s], dtype).numpy().mean(axis=0)
            assert np.abs(o[s] - np.repeat(mean, 2, axis=0)).max() < 1e-13
        # one token: the output is that token's value exactly
        c = make_case(rng, dtype=dtype, S=2, Hq=2, Hkv=2, d=64, ctx=(1, 1))
        o = decode(oracle, c)
        for s in range(2):
            assert np.array_equal(o[s], _widen_torch(c["V"][s][0], dtype).numpy())
        # a dominant key: output -> that token's value
        c = make_case(rng, dtype="f32", S=1, Hq=1, Hkv=1, d=64, ctx=(50,), poison=False)
        qv = c["q"][0, 0].astype(np.float64)
        K = c["K"][0].copy()
        K[23, 0] = (qv * 40.0 / (qv @ qv) * math.sqrt(64)).astype(np.float32)
        kp, _ = oracle.reshape_and_cache_ref(c["k_pool"], c["v_pool"], K, c["V"][0],
                                             c["tables"], np.zeros(50, np.int32),
                                             np.arange(50, dtype=np.int32), dtype="f32",
                                             num_kv_heads=1, block_size=16, head_dim=64)
        c["k_pool"] = kp
        o = decode(oracle, c)[0, 0]
        assert np.abs(o - c["V"][0][23, 0]).max() < 1e-6
    # convexity: each output coordinate lies between the smallest and largest value
    c = make_case(rng, dtype="f16", S=3, Hq=4, Hkv=4, d=64, ctx=(3, 64, 77))
    o = decode(oracle, c)
    for s in range(3):
        V = _widen_torch(c["V"][s], "f16").numpy()
        assert np.all(o[s] <= V.max(axis=0) + 1e-12) and np.all(o[s] >= V.min(axis=0) - 1e-12)
    # no context: zeros
    c = make_case(rng, dtype="f32", S=2, Hq=2, Hkv=2, d=64, ctx=(0, 3))
    o = decode(oracle, c)
    assert np.all(o[0] == 0) and np.all(np.isfinite(o[1]))


# ---------------------------------------------------------------------------------------------
# invariances the pages state
# ---------------------------------------------------------------------------------------------

def pin_paging_invariance(oracle):
    """Renumbering physical blocks (pool and tables together) changes nothing, bit for bit."""
    rng = np.random.default_rng(41)
    c = make_case(rng, dtype="bf16", S=3, Hq=4, Hkv=2, d=128, ctx=(60, 7, 129))
    base = decode(oracle, c)
    for _ in range(3):
        perm = rng.permutation(c["NB"])             # old id b -> new id perm[b]
        k2 = np.empty_like(c["k_pool"]); k2[perm] = c["k_pool"]
        v2 = np.empty_like(c["v_pool"]); v2[perm] = c["v_pool"]
        c2 = dict(c, k_pool=k2, v_pool=v2, tables=perm[c["tables"]].astype(np.int32))
        assert np.array_equal(decode(oracle, c2), base)


def pin_block_size_invariance(oracle):
    """The same logical tokens stored with B = 1, 4, 8, 16 give the same result."""
    rng = np.random.default_rng(43)
    outs = []
    ctx = (1, 31, 90)
    c0 = make_case(rng, dtype="f16", S=3, Hq=4, Hkv=2, d=64, B=16, ctx=ctx)
    for B in (1, 4, 8, 16):
        c = make_case(np.random.default_rng(1000 + B), dtype="f16", S=3, Hq=4, Hkv=2, d=64,
                      B=B, ctx=ctx)
        # overwrite with the same logical K/V and q as c0
        tok_seq = np.concatenate([np.full(n, s, np.int32) for s, n in enumerate(ctx)])
        tok_pos = np.concatenate([np.arange(n, dtype=np.int32) for n in ctx])
        kp, vp = oracle.reshape_and_cache_ref(c["k_pool"], c["v_pool"], np.concatenate(c0["K"]),
                                              np.concatenate(c0["V"]), c["tables"], tok_seq,
                                              tok_pos, dtype="f16", num_kv_heads=2,
                                              block_size=B, head_dim=64)
        c.update(k_pool=kp, v_pool=vp, q=c0["q"])
        outs.append(decode(oracle, c))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def pin_sharing_invariance(oracle):
    """Two sequences whose tables point at one shared prefix give the same result as when the
    prefix is duplicated into separate blocks."""
    rng = np.random.default_rng(47)
    c = make_case(rng, dtype="f16", S=2, Hq=2, Hkv=2, d=64, ctx=(50, 50), num_blocks=16,
                  poison=False)
    shared = c["tables"].copy()
    shared[1, :3] = shared[0, :3]                    # seq 1 reads seq 0's first three blocks
    c_shared = dict(c, tables=shared)
    out_shared = decode(oracle, c_shared)
    used = set(shared[:, :4].reshape(-1).tolist())
    free = [b for b in range(c["NB"]) if b not in used][:3]
    pairs = [[int(shared[0, j]), free[j]] for j in range(3)]
    kp, vp = oracle.copy_blocks_ref(c["k_pool"], c["v_pool"], pairs, dtype="f16",
                                    num_kv_heads=2, block_size=16, head_dim=64)
    copied = shared.copy()
    copied[1, :3] = free
    out_copied = decode(oracle, dict(c, k_pool=kp, v_pool=vp, tables=copied))
    assert np.array_equal(out_shared, out_copied)


def pin_poison_ignored(oracle):
    """Slots past ctx and table entries past the last block are never read: NaN there leaves
    the result finite and unchanged."""
    rng = np.random.default_rng(53)
    c = make_case(rng, dtype="f16", S=3, Hq=2, Hkv=2, d=64, ctx=(3, 16, 17), poison=True)
    out = decode(oracle, c)
    assert np.isfinite(out).all()
    c2 = dict(c, k_pool=c["k_pool"].copy(), v_pool=c["v_pool"].copy())
    # replace every NaN by 0: result unchanged
    for name in ("k_pool", "v_pool"):
        a = c2[name].view(np.float16)
        a[np.isnan(a)] = 0
    assert np.array_equal(decode(oracle, c2), out)


# ---------------------------------------------------------------------------------------------
# the second form (block loop) and the split merge against the first
# ---------------------------------------------------------------------------------------------

def pin_blocked_form(oracle):
    """[wiki]'s blocked form (per-block weight vectors over one common denominator, block
    outputs summed) equals the dense form: only the grouping of the sums differs ([anal] §3)."""
    rng = np.random.default_rng(61)
    for B, ctx in ((16, (1, 16, 17, 300)), (8, (9, 40, 2, 64))):
        c = make_case(rng, dtype="bf16", S=4, Hq=4, Hkv=2, d=128, B=B, ctx=ctx)
        ref = decode(oracle, c)
        q64 = _widen_torch(c["q"], "bf16").numpy()
        for s in range(c["S"]):
            for h in range(c["Hq"]):
                o = oracle.blocked_form_ref(q64[s, h], c["k_pool"], c["v_pool"], c["tables"][s],
                                            c["ctx"][s], c["scale"], h // 2, dtype="bf16",
                                            num_kv_heads=2, block_size=B, head_dim=128)
                assert np.abs(o - ref[s, h]).max() <= 1e-13


def pin_split_merge(oracle):
    rng = np.random.default_rng(67)
    c = make_case(rng, dtype="f32", S=1, Hq=1, Hkv=1, d=64, ctx=(1000,), poison=False)
    K = _widen_torch(c["K"][0][:, 0], "f32").numpy()
    V = _widen_torch(c["V"][0][:, 0], "f32").numpy()
    q = _widen_torch(c["q"][0, 0], "f32").numpy()
    whole = decode(oracle, c)[0, 0]
    for part in (16, 100, 512, 999, 1000, 4096):
        states = oracle.partition_states_ref(q, K, V, c["scale"], part)
        assert len(states) == -(-1000 // part)
        assert np.abs(oracle.merge_partition_states_ref(states) - whole).max() <= 1e-13


# ---------------------------------------------------------------------------------------------
# prefill: every query token of a prompt (or of a chunk of one) attends causally
# ---------------------------------------------------------------------------------------------

def _prefill_case(rng, *, q_lens, **kw):
    """A decode case whose sequences also carry q_lens new query tokens each (their newest)."""
    c = make_case(rng, **kw)
    q_lens = np.asarray(q_lens, np.int32)
    qs = np.zeros(c["S"] + 1, np.int32)
    qs[1:] = np.cumsum(q_lens)
    c["qs"] = qs
    c["Q"] = random_storage(rng, (int(qs[-1]), c["Hq"], c["d"]), c["dtype"])
    return c


def _prefill(oracle, c, **over):
    args = dict(dtype=c["dtype"], num_kv_heads=c["Hkv"], block_size=c["B"], head_dim=c["d"])
    args.update(over)
    return oracle.paged_prefill_ref(c["Q"], c["k_pool"], c["v_pool"], c["tables"], c["qs"],
                                    c["ctx"], c["scale"], **args)


def pin_prefill_sdpa(oracle):
    """Against torch's scaled_dot_product_attention in float64 with an explicit causal mask
    (query j of a chunk of q_len at the end of ctx tokens sees tokens 0 .. ctx - q_len + j)."""
    rng = np.random.default_rng(71)
    cases = [
        dict(dtype="f32", S=2, Hq=4, Hkv=4, d=64, ctx=(40, 17), q_lens=(40, 17)),
        dict(dtype="bf16", S=3, Hq=8, Hkv=2, d=128, ctx=(33, 70, 16), q_lens=(33, 9, 1)),
        dict(dtype="f16", S=2, Hq=6, Hkv=3, d=64, B=8, ctx=(50, 23), q_lens=(20, 23)),
        dict(dtype="bf16", S=1, Hq=4, Hkv=1, d=128, B=32, ctx=(100,), q_lens=(64,)),
    ]
    for kw in cases:
        c = _prefill_case(rng, **kw)
        mine = _prefill(oracle, c)
        scale = float(c["scale"])
        for s in range(c["S"]):
            n = int(c["ctx"][s])
            ql = int(c["qs"][s + 1] - c["qs"][s])
            q = _widen_torch(c["Q"][c["qs"][s]:c["qs"][s + 1]], c["dtype"]).permute(1, 0, 2)[None]
            K = _widen_torch(c["K"][s], c["dtype"]).permute(1, 0, 2)[None].contiguous()
            V = _widen_torch(c["V"][s], c["dtype"]).permute(1, 0, 2)[None].contiguous()
            mask = (torch.arange(n)[None, :] <= (n - ql + torch.arange(ql))[:, None])
            o = torch.nn.functional.scaled_dot_product_attention(
                q, K, V, attn_mask=mask, scale=scale, enable_gqa=c["Hq"] != c["Hkv"])[0]
            for j in range(ql):
                assert np.abs(mine[(s, j)] - o[:, j, :].numpy()).max() <= 1e-12, (kw, s, j)


def pin_prefill_decode_and_chunks(oracle):
    """One query per sequence is a decode step; a prompt taken in two chunks (the second chunk's
    queries over the whole context) gives the whole prompt's rows exactly."""
    rng = np.random.default_rng(73)
    c = _prefill_case(rng, dtype="bf16", S=3, Hq=4, Hkv=2, d=64, ctx=(30, 1, 65),
                      q_lens=(1, 1, 1))
    c["q"] = c["Q"]  # one query row per sequence
    dec = decode(oracle, c)
    pre = _prefill(oracle, c)
    for s in range(3):
        assert np.array_equal(pre[(s, 0)], dec[s])
    n, n1 = 45, 19
    whole = _prefill_case(np.random.default_rng(75), dtype="f16", S=1, Hq=4, Hkv=2, d=64,
                          ctx=(n,), q_lens=(n,))
    full = _prefill(oracle, whole)
    tail = dict(whole)
    tail["Q"] = whole["Q"][n1:]
    tail["qs"] = np.array([0, n - n1], np.int32)
    part = _prefill(oracle, tail)
    for j in range(n - n1):
        assert np.array_equal(part[(0, j)], full[(0, n1 + j)])
    # the first query of a whole prompt sees only itself: its output is its own value row
    v0 = oracle.to_f64(whole["V"][0][0], "f16")
    for h in range(4):
        assert np.array_equal(full[(0, 0)][h], v0[h // 2])


def pin_prefill_longer_than_context(oracle):
    """A chunk longer than its context (q_len > ctx, outside the callers' contract): its first
    q_len - ctx queries sit at negative positions and see no token, giving zero rows; the others
    are the rows of the same queries with q_len = ctx."""
    rng = np.random.default_rng(79)
    n, extra = 10, 6
    c = _prefill_case(rng, dtype="f16", S=1, Hq=4, Hkv=2, d=64, ctx=(n,), q_lens=(n + extra,))
    out = _prefill(oracle, c)
    for j in range(extra):
        assert np.array_equal(out[(0, j)], np.zeros((4, 64))), j
    fit = dict(c)
    fit["Q"] = c["Q"][extra:]
    fit["qs"] = np.array([0, n], np.int32)
    ref = _prefill(oracle, fit)
    for j in range(n):
        assert np.array_equal(out[(0, extra + j)], ref[(0, j)])


def pin_swap_blocks(oracle):
    """Swapping blocks into another pool changes exactly the destination blocks, each becoming
    a bit copy of its source block in both pools; swapping out and back in restores the blocks;
    within one pool it is the copy-on-write copy."""
    rng = np.random.default_rng(77)
    kw = dict(dtype="bf16", num_kv_heads=2, block_size=16, head_dim=64)
    shape = (2, 16 * 64)
    gk, gv = (random_storage(rng, (12,) + shape, "bf16") for _ in range(2))
    hk, hv = (random_storage(rng, (7,) + shape, "bf16") for _ in range(2))
    pairs = np.array([[3, 6], [11, 0], [4, 2]], np.int32)
    ok, ov = oracle.swap_blocks_ref(hk, hv, gk, gv, pairs, **kw)
    changed = sorted(set(range(7)) - {b for b in range(7) if np.array_equal(ok[b], hk[b])
                                        and np.array_equal(ov[b], hv[b])})
    assert changed == [0, 2, 6]
    for src, dst in pairs:
        assert np.array_equal(ok[dst], gk[src]) and np.array_equal(ov[dst], gv[src])
    back_k, back_v = oracle.swap_blocks_ref(np.zeros_like(gk), np.zeros_like(gv), ok, ov,
                                            pairs[:, ::-1], **kw)
    for src, _ in pairs:
        assert np.array_equal(back_k[src], gk[src]) and np.array_equal(back_v[src], gv[src])
    within = oracle.swap_blocks_ref(gk, gv, gk, gv, np.array([[1, 5]], np.int32), **kw)
    cow = oracle.copy_blocks_ref(gk, gv, np.array([[1, 5]], np.int32), **kw)
    assert all(np.array_equal(a, b) for a, b in zip(within, cow))


def pin_causal_moments(oracle):
    """The second moment the prefill rounding bound uses, against brute force: each weight
    computed on its own with math.exp, then sum w v^2; and the bound it gives on the mean
    absolute deviation (sum w |v - o| <= sqrt(M2 - o^2)) holds."""
    rng = np.random.default_rng(83)
    n, d, r = 7, 5, 9
    Q = rng.standard_normal((r, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d)) * 3
    last = np.array([-1, 0, 1, 2, 3, 4, 5, 6, 6])
    O, M2 = oracle.causal_rows(Q, K, V, last, 0.7, moments=True)
    for i in range(r):
        if last[i] < 0:
            assert not O[i].any() and not M2[i].any()
            continue
        zs = [0.7 * sum(Q[i, k] * K[t, k] for k in range(d)) for t in range(last[i] + 1)]
        es = [math.exp(z) for z in zs]
        w = [e / sum(es) for e in es]
        for e in range(d):
            o = sum(w[t] * V[t, e] for t in range(len(w)))
            m2 = sum(w[t] * V[t, e] ** 2 for t in range(len(w)))
            mad = sum(w[t] * abs(V[t, e] - o) for t in range(len(w)))
            assert abs(O[i, e] - o) <= 1e-12 and abs(M2[i, e] - m2) <= 1e-12
            assert mad <= math.sqrt(max(m2 - o * o, 0.0)) + 1e-12
    # one visible token: the mean is that value and the spread is zero
    assert np.allclose(M2[1], V[0] ** 2, rtol=0, atol=1e-12)


ALL_PINS = [pin_widening, pin_layout, pin_slot_enumeration, pin_cache_round_trip,
            pin_cache_write_footprint, pin_copy_blocks, pin_sdpa, pin_closed_forms,
            pin_paging_invariance, pin_block_size_invariance, pin_sharing_invariance,
            pin_poison_ignored, pin_blocked_form, pin_split_merge, pin_prefill_sdpa,
            pin_prefill_decode_and_chunks, pin_prefill_longer_than_context, pin_swap_blocks, pin_causal_moments]
