"""Plant plausible mistakes in the oracle (on the CPU, through monkeypatch) and check that at
least one pin fails for each: the pins are strong enough to catch a dropped term, a wrong sign
or index, or a swapped operand."""
import numpy as np
import pytest

import oracle
import oracle.paged_attention as pa_mod
from oracle_pins import ALL_PINS

_orig = {name: getattr(pa_mod, name) for name in dir(pa_mod) if not name.startswith("__")}


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(pa_mod, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def m_exp_sign(mp):
    def f(q, K, V, scale):
        if K.shape[0] == 0:
            return np.zeros(V.shape[1])
        z = scale * (K @ q)
        w = np.exp(-(z - z.max()))
        return (w @ V) / w.sum()
    _patch(mp, "attention_one_query", f)


def m_denominator(mp):
    def f(q, K, V, scale):
        if K.shape[0] == 0:
            return np.zeros(V.shape[1])
        z = scale * (K @ q)
        w = np.exp(z - z.max())
        return (w @ V) / (w.sum() + 1.0)
    _patch(mp, "attention_one_query", f)


def m_keys_as_values(mp):
    def f(q, K, V, scale):
        if K.shape[0] == 0:
            return np.zeros(V.shape[1])
        z = scale * (K @ q)
        w = np.exp(z - z.max())
        return (w @ K) / w.sum()
    _patch(mp, "attention_one_query", f)


def m_no_scale(mp):
    orig = _orig["attention_one_query"]
    _patch(mp, "attention_one_query", lambda q, K, V, scale: orig(q, K, V, 1.0))


def m_scale_twice(mp):
    orig = _orig["attention_one_query"]
    _patch(mp, "attention_one_query", lambda q, K, V, scale: orig(q, K, V, scale * scale))


def m_head_modulo(mp):
    def f(query, k_pool, v_pool, block_tables, context_lens, scale, *, dtype, num_kv_heads,
          block_size, head_dim, seqs=None, heads=None):
        q64 = pa_mod.to_f64(query, dtype)
        S, Hq, d = q64.shape
        scale64 = float(np.float32(scale))
        seqs = range(S) if seqs is None else list(seqs)
        heads = range(Hq) if heads is None else list(heads)
        out = np.zeros((len(seqs), len(heads), d))
        for n, s in enumerate(seqs):
            K, V = pa_mod.gather_sequence_kv(k_pool, v_pool, block_tables[s], int(context_lens[s]),
                                             dtype=dtype, num_kv_heads=num_kv_heads,
                                             block_size=block_size, head_dim=head_dim)
            for m, h in enumerate(heads):
                g = h % num_kv_heads
                out[n, m] = pa_mod.attention_one_query(q64[s, h], K[:, g], V[:, g], scale64)
        return out
    _patch(mp, "paged_decode_ref", f)


def _gather_with(block_of, slot_of):
    def f(k_pool, v_pool, row, ctx, *, dtype, num_kv_heads, block_size, head_dim):
        t = np.arange(int(ctx))
        phys = np.asarray(row)[block_of(t, block_size)]
        return pa_mod.token_kv(k_pool, v_pool, phys, slot_of(t, block_size), dtype=dtype,
                               num_kv_heads=num_kv_heads, block_size=block_size,
                               head_dim=head_dim)
    return f


def m_gather_block_index(mp):
    _patch(mp, "gather_sequence_kv", _gather_with(lambda t, B: t % B, lambda t, B: t % B))


def m_gather_slot_index(mp):
    _patch(mp, "gather_sequence_kv", _gather_with(lambda t, B: t // B, lambda t, B: (t + 1) % B))


def m_gather_one_past(mp):
    orig = _orig["gather_sequence_kv"]

    def f(k_pool, v_pool, row, ctx, **kw):
        n = int(ctx)
        return orig(k_pool, v_pool, row, n + 1 if n % kw["block_size"] else n, **kw)
    _patch(mp, "gather_sequence_kv", f)


def m_k_offset_swapped(mp):
    def f(b, h, t, i, *, num_kv_heads, block_size, head_dim, esz):
        W = 64 // esz
        tile = block_size * head_dim
        return ((np.asarray(b, dtype=np.int64) * num_kv_heads + h) * tile
                + (np.asarray(i) // W) * (block_size * W) + np.asarray(i) % W * block_size
                + np.asarray(t))
    _patch(mp, "k_offset", f)


def m_v_offset_transposed(mp):
    def f(b, h, t, i, *, num_kv_heads, block_size, head_dim):
        return ((np.asarray(b, dtype=np.int64) * num_kv_heads + h) * block_size * head_dim
                + np.asarray(i) * block_size + np.asarray(t))
    _patch(mp, "v_offset", f)


def m_slot_swapped(mp):
    _patch(mp, "slot_of", lambda row, pos, B: int(row[pos % B]) * B + pos // B)


def m_copy_only_keys(mp):
    def f(k_pool, v_pool, pairs, *, dtype, num_kv_heads, block_size, head_dim):
        k2, _ = _orig["copy_blocks_ref"](k_pool, v_pool, pairs, dtype=dtype,
                                         num_kv_heads=num_kv_heads, block_size=block_size,
                                         head_dim=head_dim)
        return k2, np.array(v_pool, copy=True)
    _patch(mp, "copy_blocks_ref", f)


def m_merge_no_rescale_l(mp):
    def f(states):
        M = max(m for m, _, _ in states)
        num = sum(np.exp(m - M) * acc for m, _, acc in states)
        den = sum(l for _, l, _ in states)
        return num / den
    _patch(mp, "merge_partition_states_ref", f)


def m_blocked_per_block_denominator(mp):
    """Each block's weight vector divided by its own block's sum (a misreading of the blocked
    denominator) instead of the sum over all blocks."""
    def f(q, k_pool, v_pool, row, ctx, scale, g, *, dtype, num_kv_heads, block_size, head_dim):
        scale64 = float(np.float32(scale))
        out = np.zeros(head_dim)
        for j in range(-(-int(ctx) // block_size)):
            valid = min(block_size, int(ctx) - j * block_size)
            K, V = pa_mod.token_kv(k_pool, v_pool, np.full(valid, int(row[j])), np.arange(valid),
                                   dtype=dtype, num_kv_heads=num_kv_heads,
                                   block_size=block_size, head_dim=head_dim)
            z = scale64 * (K[:, g] @ q)
            e = np.exp(z - z.max())
            out = out + V[:, g].T @ (e / e.sum())
        return out
    _patch(mp, "blocked_form_ref", f)


def _causal_with(mp, *, strict=False, scale_factor=1.0):
    """causal_rows with the query's own token masked out (strict) or the scale changed."""
    orig = _orig["causal_rows"]

    def f(Q, K, V, last, scale, moments=False):
        last = np.asarray(last) - (1 if strict else 0)
        return orig(Q, K, V, last, scale * scale_factor, moments)
    _patch(mp, "causal_rows", f)


def m_causal_excludes_self(mp):
    _causal_with(mp, strict=True)


def m_causal_wrong_scale(mp):
    _causal_with(mp, scale_factor=0.125)


def m_moments_first_moment(mp):
    """The prefill bound's second moment computed as sum w |v| (a first moment) instead."""
    orig = _orig["causal_rows"]

    def f(Q, K, V, last, scale, moments=False):
        if not moments:
            return orig(Q, K, V, last, scale)
        O, _ = orig(Q, K, V, last, scale, True)
        _, M1 = orig(Q, K, np.sqrt(np.abs(V)), last, scale, True)
        return O, M1
    _patch(mp, "causal_rows", f)


def m_bf16_shift(mp):
    orig = _orig["to_f64"]

    def f(a, dtype):
        if dtype == "bf16":
            bits = np.asarray(a).view(np.uint16).astype(np.uint32) << np.uint32(15)
            return bits.view(np.float32).astype(np.float64)
        return orig(a, dtype)
    _patch(mp, "to_f64", f)


def _prefill_with(mp, limit):
    """paged_prefill_ref with the last visible token of query j (chunk of q_len at the end of
    ctx tokens) given by limit(ctx, q_len, j) instead of ctx - q_len + j."""
    def f(query, k_pool, v_pool, block_tables, query_start, context_lens, scale, *, dtype,
          num_kv_heads, block_size, head_dim, seqs=None, rows=None):
        q64 = pa_mod.to_f64(query, dtype)
        T, Hq, d = q64.shape
        G = Hq // num_kv_heads
        scale64 = float(np.float32(scale))
        out = {}
        for s in (range(len(context_lens)) if seqs is None else seqs):
            ctx = int(context_lens[s])
            q0, q1 = int(query_start[s]), int(query_start[s + 1])
            K, V = pa_mod.gather_sequence_kv(k_pool, v_pool, block_tables[s], ctx, dtype=dtype,
                                             num_kv_heads=num_kv_heads, block_size=block_size,
                                             head_dim=head_dim)
            for j in range(q1 - q0):
                p = limit(ctx, q1 - q0, j)
                out[(s, j)] = np.stack([pa_mod.attention_one_query(
                    q64[q0 + j, h], K[:p + 1, h // G], V[:p + 1, h // G], scale64)
                    for h in range(Hq)])
        return out
    _patch(mp, "paged_prefill_ref", f)


def m_prefill_sees_next_token(mp):
    _prefill_with(mp, lambda ctx, ql, j: min(ctx - ql + j + 1, ctx - 1))


def m_prefill_ignores_chunk_offset(mp):
    _prefill_with(mp, lambda ctx, ql, j: j)


def m_swap_reads_destination_pool(mp):
    def f(dst_k, dst_v, src_k, src_v, pairs, **kw):
        return _orig["swap_blocks_ref"](dst_k, dst_v, dst_k, dst_v, pairs, **kw)
    _patch(mp, "swap_blocks_ref", f)


MUTATIONS = [m_exp_sign, m_denominator, m_keys_as_values, m_no_scale, m_scale_twice,
             m_head_modulo, m_gather_block_index, m_gather_slot_index, m_gather_one_past,
             m_k_offset_swapped, m_v_offset_transposed, m_slot_swapped, m_copy_only_keys,
             m_merge_no_rescale_l, m_blocked_per_block_denominator, m_bf16_shift, m_prefill_sees_next_token,
             m_prefill_ignores_chunk_offset, m_swap_reads_destination_pool,
             m_moments_first_moment, m_causal_excludes_self, m_causal_wrong_scale]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m.__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(oracle)
        except Exception as e:  # an assertion, or a crash the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught {mutation.__name__}"
