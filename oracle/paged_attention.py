"""CPU oracle for the paged KV-cache attention path (decode, prefill, cache writes, block copies).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this module. It shares no code with the HIP library (no kernels,
headers, helpers, constants or layout tables) and imports nothing from it; the library never
imports it.

Everything is plain numpy in float64. Stored fp32 / fp16 / bf16 values are widened exactly to
float64 before any arithmetic. Nothing is blocked, fused or reordered beyond what the cited
definitions state.

Sources, cited by page title and section (the same four pages throughout):
  [wiki]  "PagedAttention" (newikis.com/ko/PagedAttention), section "수학적 공식" (mathematical
          formulation): the dense causal attention of one query token i (weights a_ij, output
          o_i summed over t = 1..i) and its blocked form (K_j, V_j of B tokens each; A_ij,
          o_i summed over the first ceil(i/B) blocks).
  [anal]  "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net), §2 (KV blocks of
          B tokens in scattered physical memory, on-demand allocation), §3 (the block-wise
          kernel gives the same result as ordinary attention, only partial sums are blocked;
          a logical block is found through the sequence's block table), §4 (copy-on-write of a
          shared block).
  [blog]  "PagedAttention 논문 쉽게 읽기" (iplexlaw.co.kr), §2: a token is written into the free
          slot of its sequence's last block; ②: copy-on-write of a shared last block.
  [dev]   "추론 엔진에서의 메모리 가상화: PagedAttention과 메모리 단편화의 제거" (molayo1419.me):
          two preallocated pools key_cache / value_cache; copy-on-write allocates a fresh block,
          copies the old contents, remaps the writer's table entry.

Readings where the pages leave a step open (each is listed with its reason in the design notes):
  * The query of the decode step is the sequence's newest token, so it attends to all
    ``ctx`` cached tokens, itself included (the dense formula sums t = 1..i).
  * The blocked formula's last block K_j runs past token i; those slots are excluded (weight 0),
    as the dense formula, which stops at t = i, requires.
  * The blocked denominator sums exp over every score of blocks 1..ceil(i/B) (all entries), which
    is the dense denominator.
  * The scale is the caller's float32 ``scale`` (1/sqrt(d) in every workload), widened exactly.
  * Grouped-query attention (not on the pages): query head h reads KV head h // (Hq / Hkv).
  * ctx = 0 gives a zero output.
  * Prefill (several query tokens of one sequence at once): the q_len queries are the
    sequence's newest tokens, already written to the cache, so query j sits at position
    ctx - q_len + j and the dense formula for that position applies unchanged (each query
    attends to itself and everything before it, nothing after).

The physical pool layout is the library's choice, fixed by its header; ``k_offset`` and
``v_offset`` below restate it from that description and are pinned by layout properties in
the tests (a bijection, contiguous 4 KiB tiles, 1 KiB key chunk rows), and against the library
only through parity.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------------------------
# Stored dtypes
# ---------------------------------------------------------------------------------------------

_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
_ESZ = {"f32": 4, "f16": 2, "bf16": 2}


def storage_dtype(dtype: str):
    """numpy array dtype holding stored elements (bf16 is held as its 16 raw bits)."""
    return _STORAGE[dtype]


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored fp32 / fp16 / bf16 elements to float64.

    bf16 is the upper half of an IEEE binary32, so its 16 bits shifted left by 16 are the
    binary32 of the same value.
    """
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float32, copy=False).astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):     # signalling-NaN bit patterns stay NaN
            return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------------------------
# Physical pool layout (the library's documented index functions, restated independently)
# ---------------------------------------------------------------------------------------------

def k_offset(b, h, t, i, *, num_kv_heads: int, block_size: int, head_dim: int, esz: int):
    """Element offset of key (physical block b, KV head h, slot t, dim i) in the key pool.

    The (b, h) tile of block_size*head_dim elements starts at (b*Hkv + h)*B*d. Inside it the
    head dimension is cut into 64-byte chunks of W = 64/esz elements; chunk c holds, for slot
    0..B-1 in turn, that slot's W elements, so element (t, i) sits at (i//W)*B*W + t*W + i%W.
    """
    W = 64 // esz
    tile = block_size * head_dim
    return ((np.asarray(b, dtype=np.int64) * num_kv_heads + h) * tile
            + (np.asarray(i) // W) * (block_size * W) + np.asarray(t) * W + np.asarray(i) % W)


def v_offset(b, h, t, i, *, num_kv_heads: int, block_size: int, head_dim: int):
    """Element offset of value (b, h, t, i) in the value pool: tile (b*Hkv + h), row t, column i."""
    return ((np.asarray(b, dtype=np.int64) * num_kv_heads + h) * block_size
            + np.asarray(t)) * head_dim + np.asarray(i)


def _flat(pool: np.ndarray) -> np.ndarray:
    return pool.reshape(-1)


def token_kv(k_pool, v_pool, blocks, slots, *, dtype, num_kv_heads, block_size, head_dim):
    """Keys and values of the given (physical block, slot) pairs: two float64 [n, Hkv, d]."""
    esz = _ESZ[dtype]
    b = np.asarray(blocks, dtype=np.int64)[:, None, None]
    t = np.asarray(slots, dtype=np.int64)[:, None, None]
    h = np.arange(num_kv_heads)[None, :, None]
    i = np.arange(head_dim)[None, None, :]
    ko = k_offset(b, h, t, i, num_kv_heads=num_kv_heads, block_size=block_size,
                  head_dim=head_dim, esz=esz)
    vo = v_offset(b, h, t, i, num_kv_heads=num_kv_heads, block_size=block_size,
                  head_dim=head_dim)
    return to_f64(_flat(k_pool)[ko], dtype), to_f64(_flat(v_pool)[vo], dtype)


def gather_sequence_kv(k_pool, v_pool, block_table_row, ctx, *, dtype, num_kv_heads,
                       block_size, head_dim):
    """Logical keys/values of one sequence's first ``ctx`` tokens through its block table.

    Token t (0-based) lives in logical block t // B, which the table maps to a physical block,
    at slot t % B ([anal] §2 and the lookup pseudocode; [wiki] blocked K_j, V_j).
    Returns two float64 arrays [ctx, Hkv, d].
    """
    t = np.arange(int(ctx))
    phys = np.asarray(block_table_row)[t // block_size]
    return token_kv(k_pool, v_pool, phys, t % block_size, dtype=dtype,
                    num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim)


# ---------------------------------------------------------------------------------------------
# Attention: the plain definition
# ---------------------------------------------------------------------------------------------

def attention_one_query(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) weighted sum of the rows of V, in float64 ([wiki] dense form).

    q [d], K [n, d], V [n, d]. Subtracting the maximum score before exp leaves the weights
    unchanged and keeps exp finite. n = 0 gives zeros.
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def paged_decode_ref(query, k_pool, v_pool, block_tables, context_lens, scale, *, dtype,
                     num_kv_heads, block_size, head_dim, seqs=None, heads=None):
    """Decode attention of every (sequence, query head) over its paged KV cache.

    query: stored [S, Hq, d]; pools: stored, any shape with NB*Hkv*B*d elements in the library
    layout; block_tables int [S, maxb]; context_lens int [S]; scale: the caller's float32.
    ``seqs`` / ``heads`` select a subset (for sampled checks at full size).
    Returns float64 [len(seqs), len(heads), d].
    """
    q64 = to_f64(query, dtype)
    S, Hq, d = q64.shape
    G = Hq // num_kv_heads
    scale64 = float(np.float32(scale))
    seqs = range(S) if seqs is None else list(seqs)
    heads = range(Hq) if heads is None else list(heads)
    out = np.zeros((len(seqs), len(heads), d))
    for n, s in enumerate(seqs):
        ctx = int(context_lens[s])
        K, V = gather_sequence_kv(k_pool, v_pool, block_tables[s], ctx, dtype=dtype,
                                  num_kv_heads=num_kv_heads, block_size=block_size,
                                  head_dim=head_dim)
        for m, h in enumerate(heads):
            g = h // G
            out[n, m] = attention_one_query(q64[s, h], K[:, g, :], V[:, g, :], scale64)
    return out


def causal_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, last: np.ndarray, scale: float,
                moments: bool = False):
    """The dense causal form for several query rows at once ([wiki] dense form for a general
    query token i: it attends to tokens 1..i and to nothing after).

    Q [r, d]; K, V [n, d]; row r attends to tokens 0..last[r] (last[r] < 0: no token, a zero
    row). Returns O [r, d], and with ``moments`` also M2 [r, d] = sum_t w_t v_t^2, the second
    moment of the values under the row's softmax weights w (what a rounding bound on a weighted
    mean needs: sum_t w_t |v_t - o| <= sqrt(M2 - o^2)).
    """
    r, d = Q.shape
    O = np.zeros((r, d))
    M2 = np.zeros((r, d))
    if r and K.shape[0]:
        Z = scale * (Q @ K.T)
        visible = np.arange(K.shape[0])[None, :] <= np.asarray(last)[:, None]
        Z = np.where(visible, Z, -np.inf)
        seen = visible.any(axis=1)
        top = np.where(seen, Z.max(axis=1, initial=-np.inf), 0.0)
        W = np.exp(Z - top[:, None])                # exp(-inf) = 0 outside the causal range
        den = W.sum(axis=1)
        den = np.where(seen, den, 1.0)
        O = (W @ V) / den[:, None]
        if moments:
            M2 = (W @ (V * V)) / den[:, None]
    return (O, M2) if moments else O


def paged_prefill_ref(query, k_pool, v_pool, block_tables, query_start, context_lens, scale, *,
                      dtype, num_kv_heads, block_size, head_dim, seqs=None, rows=None,
                      moments=False):
    """Causal attention of every query token over its sequence's paged KV cache ([wiki] dense
    form for a general query i: token i attends to tokens 1..i; the blocked form sums over the
    first ceil(i/B) blocks).

    Sequence s's queries are rows query_start[s] .. query_start[s+1]-1 of ``query`` (stored
    [T, Hq, d]); they are its newest q_len = query_start[s+1] - query_start[s] tokens, so query j
    sits at position p = ctx - q_len + j (0-based) and attends to tokens 0..p of the cache
    (q_len = 1 is a decode step, q_len = ctx a whole prompt; a negative p, q_len > ctx, sees no
    token and gives a zero row, as an empty context does). ``seqs`` selects sequences, ``rows``
    (a dict seq -> list of j) selects queries within them. Returns a dict (s, j) -> float64
    [Hq, d]; with ``moments`` a dict (s, j) -> (o, M2), M2 as in ``causal_rows``.
    """
    q64 = to_f64(query, dtype)
    T, Hq, d = q64.shape
    G = Hq // num_kv_heads
    scale64 = float(np.float32(scale))
    S = len(context_lens)
    seqs = range(S) if seqs is None else list(seqs)
    out = {}
    for s in seqs:
        ctx = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        q_len = q1 - q0
        K, V = gather_sequence_kv(k_pool, v_pool, block_tables[s], ctx, dtype=dtype,
                                  num_kv_heads=num_kv_heads, block_size=block_size,
                                  head_dim=head_dim)
        js = np.asarray(range(q_len) if rows is None else rows[s], dtype=np.int64)
        if js.size == 0:
            continue
        last = ctx - q_len + js                     # position of query j
        o = np.zeros((js.size, Hq, d))
        m2 = np.zeros((js.size, Hq, d))
        for h in range(Hq):
            g = h // G
            res = causal_rows(q64[q0 + js, h], K[:, g, :], V[:, g, :], last, scale64, moments)
            if moments:
                o[:, h], m2[:, h] = res
            else:
                o[:, h] = res
        for n, j in enumerate(js.tolist()):
            out[(s, j)] = (o[n], m2[n]) if moments else o[n]
    return out


# ---------------------------------------------------------------------------------------------
# The blocked form (a second form, used to check the first)
# ---------------------------------------------------------------------------------------------

def blocked_form_ref(q, k_pool, v_pool, block_table_row, ctx, scale, g, *, dtype,
                     num_kv_heads, block_size, head_dim):
    """One query head over one sequence in [wiki]'s blocked form: with K_j, V_j the keys and
    values of logical block j (the physical block the table names), the weight vector of block
    j is exp(scale * K_j q) divided by the sum of every entry of every block's vector, and the
    output is the sum over blocks of V_j^T times that vector.

    Every block's exponentials are taken relative to one common constant (the largest score of
    the sequence), which cancels in the ratio and keeps them finite. Slots at or past ``ctx`` in
    the last block are not part of K_j, V_j. q: float64 [d]. Returns float64 [d].
    """
    scale64 = float(np.float32(scale))
    num_blocks = -(-int(ctx) // block_size)
    if num_blocks == 0:
        return np.zeros(head_dim)
    scores, values = [], []
    for j in range(num_blocks):
        valid = min(block_size, int(ctx) - j * block_size)
        K, V = token_kv(k_pool, v_pool, np.full(valid, int(block_table_row[j])),
                        np.arange(valid), dtype=dtype, num_kv_heads=num_kv_heads,
                        block_size=block_size, head_dim=head_dim)
        scores.append(scale64 * (K[:, g, :] @ q))
        values.append(V[:, g, :])
    shift = max(float(z.max()) for z in scores)
    vectors = [np.exp(z - shift) for z in scores]
    denominator = sum(float(e.sum()) for e in vectors)
    return sum(V.T @ e for V, e in zip(values, vectors)) / denominator


# ---------------------------------------------------------------------------------------------
# Split over context partitions and the merge of their states
# ---------------------------------------------------------------------------------------------

def partition_states_ref(q, K, V, scale, partition_tokens):
    """Softmax state (m, l, acc) of each run of ``partition_tokens`` consecutive tokens.

    m = max score in the run, l = sum of exp(score - m), acc = sum of exp(score - m) * v.
    q [d], K/V [n, d] float64.
    """
    scale64 = float(np.float32(scale))
    states = []
    for start in range(0, K.shape[0], partition_tokens):
        z = scale64 * (K[start:start + partition_tokens] @ q)
        m = float(z.max())
        w = np.exp(z - m)
        states.append((m, float(w.sum()), w @ V[start:start + partition_tokens]))
    return states


def merge_partition_states_ref(states):
    """Combine partition states: with M the largest m, o = sum e^(m_p-M) acc_p / sum e^(m_p-M) l_p.

    Exact because every partial sum only needs rescaling to a common maximum ([anal] §3: the
    blocked computation differs from ordinary attention only in how partial sums are grouped).
    """
    M = max(m for m, _, _ in states)
    num = sum(np.exp(m - M) * acc for m, _, acc in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den


# ---------------------------------------------------------------------------------------------
# Cache writes and block copies
# ---------------------------------------------------------------------------------------------

def slot_of(block_table_row, pos: int, block_size: int) -> int:
    """Physical slot of token position ``pos``: the table's block for pos // B, offset pos % B."""
    return int(block_table_row[pos // block_size]) * block_size + pos % block_size


def reshape_and_cache_ref(k_pool, v_pool, key, value, block_tables, token_seq, token_pos, *,
                          dtype, num_kv_heads, block_size, head_dim):
    """Copies of the pools with each new token's key/value written into its slot.

    Token n belongs to sequence token_seq[n] at position token_pos[n] (negative = skip). Its
    slot is the one ``slot_of`` names ([blog] §2: the token goes into its block's free slot).
    Elements are copied bit for bit. key/value: stored [T, Hkv, d].
    """
    esz = _ESZ[dtype]
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    kf, vf = _flat(k_out), _flat(v_out)
    key = np.asarray(key)
    value = np.asarray(value)
    i = np.arange(head_dim)
    for n in range(len(token_seq)):
        pos = int(token_pos[n])
        if pos < 0:
            continue
        slot = slot_of(block_tables[int(token_seq[n])], pos, block_size)
        b, t = slot // block_size, slot % block_size
        for h in range(num_kv_heads):
            kf[k_offset(b, h, t, i, num_kv_heads=num_kv_heads, block_size=block_size,
                        head_dim=head_dim, esz=esz)] = key[n, h]
            vf[v_offset(b, h, t, i, num_kv_heads=num_kv_heads, block_size=block_size,
                        head_dim=head_dim)] = value[n, h]
    return k_out, v_out


def copy_blocks_ref(k_pool, v_pool, pairs, *, dtype, num_kv_heads, block_size, head_dim):
    """Copies of the pools where, for each (src, dst) pair, block dst receives all of block
    src's key and value elements (every KV head, every slot), bit for bit ([dev] and [anal] §4:
    the copy-on-write duplicate of a shared block)."""
    esz = _ESZ[dtype]
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    kf, vf = _flat(k_out), _flat(v_out)
    h = np.arange(num_kv_heads)[:, None, None]
    t = np.arange(block_size)[None, :, None]
    i = np.arange(head_dim)[None, None, :]
    kw = dict(num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim)
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        kf[k_offset(dst, h, t, i, esz=esz, **kw)] = kf[k_offset(src, h, t, i, esz=esz, **kw)]
        vf[v_offset(dst, h, t, i, **kw)] = vf[v_offset(src, h, t, i, **kw)]
    return k_out, v_out


def swap_blocks_ref(dst_k, dst_v, src_k, src_v, pairs, *, dtype, num_kv_heads, block_size,
                    head_dim):
    """Copies of the destination pools where, for each (src, dst) pair, destination block dst
    receives all of source block src's key and value elements (every KV head, every slot), bit
    for bit ([anal] §6: a preempted sequence's blocks are swapped out to a CPU block pool and
    back in, block by block)."""
    esz = _ESZ[dtype]
    k_out = np.array(dst_k, copy=True)
    v_out = np.array(dst_v, copy=True)
    kf, vf = _flat(k_out), _flat(v_out)
    ksf, vsf = _flat(np.asarray(src_k)), _flat(np.asarray(src_v))
    h = np.arange(num_kv_heads)[:, None, None]
    t = np.arange(block_size)[None, :, None]
    i = np.arange(head_dim)[None, None, :]
    kw = dict(num_kv_heads=num_kv_heads, block_size=block_size, head_dim=head_dim)
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        kf[k_offset(dst, h, t, i, esz=esz, **kw)] = ksf[k_offset(src, h, t, i, esz=esz, **kw)]
        vf[v_offset(dst, h, t, i, **kw)] = vsf[v_offset(src, h, t, i, **kw)]
    return k_out, v_out
