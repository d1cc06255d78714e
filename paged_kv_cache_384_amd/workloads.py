"""Seeded synthetic inputs for the paged attention path (decode and prefill): configurations, a
host block manager and value generators.

This module is shared by the tests, the benchmark and the smoke check. It holds none of the
path's arithmetic: no attention, no slot computation, no pool layout. It only

* draws per-sequence context lengths from the distributions the workloads name,
* hands out physical block ids through a host block manager (a seeded free list, reference
  counts and copy-on-write bookkeeping), producing block tables and copy pairs, and
* fills query / new-token / pool tensors with N(0,1) draws rounded to the storage dtype.

Pool tensors have shape ``[num_blocks, num_kv_heads, block_size * head_dim]``: one opaque tile
per (physical block, KV head). How a tile orders its elements is the library's business and is
not used here.

Sources for the block manager, cited by page title and section:
  * "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net), "핵심 개념" and §2:
    fixed-size KV blocks, a block table from logical to physical blocks, allocation on demand
    so that only a sequence's last block is partly empty; §4: blocks shared with a reference
    count, copied only when a sharer writes into a block whose count exceeds one.
  * "추론 엔진에서의 메모리 가상화: PagedAttention과 메모리 단편화의 제거" (molayo1419.me), block
    manager and copy-on-write sections: allocation is host-side integer bookkeeping over two
    preallocated pools; the worked example with shared blocks #10/#11 (count 2) and a fresh
    block #45 for the branch that writes.
  * "PagedAttention 논문 쉽게 읽기" (iplexlaw.co.kr), §2: a new token goes into the free slot of
    the last block, and a new block is appended to the table only when that block is full.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "DecodeConfig", "CONFIGS", "PREFILL_CONFIGS", "BlockManager", "PoolExhausted", "DecodeBatch", "build_batch",
    "make_values", "config", "element_size", "kv_bytes_per_token",
]

_ESZ = {"f32": 4, "f16": 2, "bf16": 2}


def element_size(dtype: str) -> int:
    """Bytes per stored element for the dtype names used throughout ('f32', 'f16', 'bf16')."""
    return _ESZ[dtype]


def kv_bytes_per_token(num_layers: int, hidden: int, esz: int) -> int:
    """K and V bytes one token occupies across all layers of a model (both caches)."""
    return 2 * num_layers * hidden * esz


@dataclass(frozen=True)
class DecodeConfig:
    """One synthetic decode workload.

    ``ctx`` names the context-length distribution:
      ("fixed", (n_0, n_1, ...))              the given lengths, one per sequence
      ("uniform", lo, hi)                     integers, both ends inclusive
      ("lognormal", median, sigma, lo, hi)    round(exp(N(ln median, sigma^2))), clipped
      ("shared_prefix", prompt, lo, hi, n)    ``num_seqs // n`` prompts of ``prompt`` tokens,
                                              each shared by ``n`` samples whose own suffixes
                                              are uniform in [lo, hi]
    ``num_blocks`` = 0 sizes the pool as ceil(pool_slack * blocks in use) + 1 (the extra block is
    the poison block that unused table entries point at).
    ``placement``: "shuffled" hands physical blocks out in a seeded random order; "contiguous"
    gives sequence s the span of physical blocks [s * W, s * W + ceil(ctx / B)) with W the
    table width (the layout of a cache that is not paged; the pool is S * W + 1 blocks).
    ``new_tokens`` names how many of each context's tokens are new this step (written to the
    cache and used as queries; they are always the newest):
      ("one",)               one per sequence (a decode step)
      ("all",)               the whole context (a prompt's prefill)
      ("uniform", lo, hi)    integers in [lo, hi], capped at the context (a prefill chunk on
                             top of tokens cached earlier)
    """
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int = 16
    ctx: tuple = ("uniform", 1, 200)
    num_blocks: int = 0
    pool_slack: float = 1.25
    seed: int = 0
    partition_size: int = 0
    description: str = ""
    placement: str = "shuffled"
    new_tokens: tuple = ("one",)

    @property
    def esz(self) -> int:
        return element_size(self.dtype)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_ctx_bound(self) -> int:
        """Largest context the distribution can produce (sizes the block-table width)."""
        kind = self.ctx[0]
        if kind == "fixed":
            return max(int(n) for n in self.ctx[1]) if len(self.ctx[1]) else 0
        if kind == "uniform":
            return int(self.ctx[2])
        if kind == "lognormal":
            return int(self.ctx[4])
        if kind == "shared_prefix":
            return int(self.ctx[1]) + int(self.ctx[3])
        raise ValueError(kind)


CONFIGS: dict[str, DecodeConfig] = {
    "tiny_fp32": DecodeConfig(
        "tiny_fp32", "f32", num_seqs=4, num_q_heads=4, num_kv_heads=4, head_dim=64,
        ctx=("uniform", 1, 200), num_blocks=64, seed=1,
        description="Tiny fp32 decode: 4 seqs, 4 heads, d=64, B=16, ctx U[1,200], "
                    "64 physical blocks in a seeded random order"),
    "opt13b_fp16": DecodeConfig(
        "opt13b_fp16", "f16", num_seqs=64, num_q_heads=40, num_kv_heads=40, head_dim=128,
        ctx=("uniform", 128, 2048), num_blocks=8192, seed=2,
        description="OPT-13B-shape decode fp16: 64 seqs, 40 heads (MHA), d=128, B=16, "
                    "ctx U[128,2048], 8192-block pool in shuffled order, one new token per seq"),
    "gqa_bf16": DecodeConfig(
        "gqa_bf16", "bf16", num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
        ctx=("lognormal", 1024, 0.75, 16, 4096), seed=3,
        description="GQA decode bf16: 256 seqs, 32 q heads over 8 KV heads, d=128, B=16, "
                    "ctx lognormal (median 1024, sigma 0.75) clipped to [16,4096]"),
    "cow_fp16": DecodeConfig(
        "cow_fp16", "f16", num_seqs=256, num_q_heads=40, num_kv_heads=40, head_dim=128,
        ctx=("shared_prefix", 520, 1, 256, 8), seed=4,
        description="Shared-prefix / copy-on-write fp16: 32 prompts x 8 samples, 40 heads, "
                    "d=128, B=16, 520-token shared prompt (32 full blocks + an 8-token partial "
                    "block duplicated by copy-on-write), suffixes U[1,256]"),
    "long_bf16": DecodeConfig(
        "long_bf16", "bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
        ctx=("uniform", 16384, 32768), seed=5, partition_size=512,
        description="Long-context split-K bf16: 8 seqs, 32 q heads over 8 KV heads, d=128, "
                    "B=16, ctx U[16384,32768], 512-token partitions"),
}


# Prefill workloads (many new tokens per sequence): the attention becomes two dense products per
# key/value tile, so these are measured in FLOP/s on the matrix cores rather than in HBM bytes.
PREFILL_CONFIGS: dict[str, DecodeConfig] = {
    "prefill_bf16": DecodeConfig(
        "prefill_bf16", "bf16", num_seqs=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        ctx=("uniform", 512, 4096), new_tokens=("all",), seed=6,
        description="GQA prompt prefill bf16: 16 prompts of U[512,4096] tokens, 32 q heads "
                    "over 8 KV heads, d=128, B=16, every prompt token a query"),
    "chunked_fp16": DecodeConfig(
        "chunked_fp16", "f16", num_seqs=32, num_q_heads=40, num_kv_heads=40, head_dim=128,
        ctx=("uniform", 512, 4096), new_tokens=("uniform", 128, 512), seed=7,
        description="OPT-13B-shape chunked prefill fp16: 32 seqs with contexts U[512,4096], "
                    "of which the newest U[128,512] tokens are this step's queries, 40 heads, "
                    "d=128, B=16"),
}


def config(name: str, **overrides) -> DecodeConfig:
    """A named configuration, optionally with fields replaced (for smaller parity cases)."""
    cfg = CONFIGS[name] if name in CONFIGS else PREFILL_CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


class PoolExhausted(RuntimeError):
    """Raised when the free list is empty."""


class BlockManager:
    """Host-side allocator of physical KV blocks for building block tables.

    The free list is a seeded permutation of the physical ids, so logically consecutive blocks
    land at scattered physical places. Each sequence owns a block table (a Python list of
    physical ids) and a token count. Reference counts track how many tables point at a block.
    """

    def __init__(self, num_blocks: int, block_size: int, rng: np.random.Generator | None = None,
                 order: np.ndarray | None = None):
        if order is None:
            order = (rng.permutation(num_blocks) if rng is not None
                     else np.arange(num_blocks))
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        # pop() takes from the end, so reverse to hand ids out in ``order``'s order
        self._free = [int(b) for b in order[::-1]]
        self.ref = np.zeros(num_blocks, dtype=np.int64)
        self.tables: list[list[int]] = []
        self.lengths: list[int] = []
        self.copies: list[tuple[int, int]] = []

    # -- allocation ---------------------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def take(self, block: int | None = None) -> int:
        """Pop a free block (or remove the given id from the free list) with count 1."""
        if block is None:
            if not self._free:
                raise PoolExhausted("no free physical block left")
            b = self._free.pop()
        else:
            self._free.remove(block)
            b = block
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self._free.append(b)

    def new_sequence(self) -> int:
        self.tables.append([])
        self.lengths.append(0)
        return len(self.tables) - 1

    def blocks_needed(self, num_tokens: int) -> int:
        return -(-num_tokens // self.block_size)

    def append_tokens(self, seq: int, n: int) -> None:
        """Make room for ``n`` more tokens of ``seq``, one token at a time.

        A token goes into the last block's free slot; when that block is full a new block is
        appended; when the last block is partly full but shared (count > 1), this sequence gets
        a private copy first (recorded as a (src, dst) copy pair) and the shared count drops.
        """
        table = self.tables[seq]
        for _ in range(n):
            filled = self.lengths[seq] % self.block_size
            if filled == 0:
                table.append(self.take())
            elif self.ref[table[-1]] > 1:
                src = table[-1]
                dst = self.take()
                self.copies.append((src, dst))
                table[-1] = dst
                self.ref[src] -= 1
            self.lengths[seq] += 1

    def fork(self, seq: int) -> int:
        """A new sequence sharing every block of ``seq`` (counts incremented)."""
        child = self.new_sequence()
        self.tables[child] = list(self.tables[seq])
        self.lengths[child] = self.lengths[seq]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def free_sequence(self, seq: int) -> None:
        for b in self.tables[seq]:
            self._release(b)
        self.tables[seq] = []
        self.lengths[seq] = 0

    def swap_out(self, seq: int, cpu: "BlockManager") -> tuple[int, np.ndarray]:
        """Move a sequence's blocks to the CPU block pool ``cpu`` ([anal] §6: a preempted
        sequence's blocks are evicted to CPU memory, all of them or none). Every GPU block gets
        a free CPU block and is released here; the sequence continues in ``cpu`` under the
        returned id. Returns (cpu sequence id, (gpu block, cpu block) copy pairs). Raises
        PoolExhausted, changing nothing, when the CPU pool cannot take every block, and
        ValueError for a sequence with shared blocks (those stay resident)."""
        t = self.tables[seq]
        if any(self.ref[b] != 1 for b in t):
            raise ValueError("a sequence with shared blocks is not swapped out")
        if cpu.num_free < len(t):
            raise PoolExhausted("the CPU block pool cannot take the whole sequence")
        cs = cpu.new_sequence()
        pairs = [(b, cpu.take()) for b in t]
        cpu.tables[cs] = [c for _, c in pairs]
        cpu.lengths[cs] = self.lengths[seq]
        self.free_sequence(seq)
        return cs, np.array(pairs, dtype=np.int32).reshape(-1, 2)

    def swap_in(self, cpu: "BlockManager", cpu_seq: int) -> tuple[int, np.ndarray]:
        """Bring a swapped-out sequence back: fresh GPU blocks for all of its CPU blocks (or
        PoolExhausted, changing nothing). Returns (gpu sequence id, (cpu block, gpu block)
        copy pairs); the CPU blocks are released."""
        t = cpu.tables[cpu_seq]
        if self.num_free < len(t):
            raise PoolExhausted("not enough free GPU blocks to swap the sequence in")
        gs = self.new_sequence()
        pairs = [(c, self.take()) for c in t]
        self.tables[gs] = [g for _, g in pairs]
        self.lengths[gs] = cpu.lengths[cpu_seq]
        cpu.free_sequence(cpu_seq)
        return gs, np.array(pairs, dtype=np.int32).reshape(-1, 2)

    def wasted_slots(self, seq: int) -> int:
        """Allocated but unfilled token slots of ``seq`` (only its last block can have any)."""
        return len(self.tables[seq]) * self.block_size - self.lengths[seq]


@dataclass
class DecodeBatch:
    """Host-side (numpy) structure of one decode step of a configuration."""
    cfg: DecodeConfig
    context_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray        # int32 [S, max_blocks_per_seq]; unused entries = poison id
    num_blocks: int
    poison_block: int               # physical block that no sequence owns
    copy_pairs: np.ndarray          # int32 [P, 2] (src, dst) copy-on-write pairs
    token_seq: np.ndarray           # int32 [T] sequence of each new token (grouped by sequence)
    token_pos: np.ndarray           # int32 [T] position of each new token (ctx - q_len .. ctx - 1)
    ref_counts: np.ndarray          # int64 [NB]
    wasted_slots: np.ndarray        # int64 [S]
    query_lens: np.ndarray          # int32 [S] new tokens (queries) per sequence
    extra: dict = field(default_factory=dict)

    @property
    def query_start(self) -> np.ndarray:
        """int32 [S + 1]: sequence s's new tokens are rows query_start[s] .. query_start[s+1]-1."""
        return np.concatenate([[0], np.cumsum(self.query_lens, dtype=np.int64)]).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.query_lens.size else 0

    def attention_flops(self) -> int:
        """Multiply-adds x 2 of the two products of causal attention over every new token:
        query j of a sequence with n cached tokens and q new ones sees n - q + j + 1 tokens, and
        each seen token costs d multiply-adds for its score and d for its share of the output,
        per query head."""
        c = self.cfg
        n = self.context_lens.astype(np.int64)
        q = self.query_lens.astype(np.int64)
        seen = q * (n - q) + q * (q + 1) // 2  # sum over j of (n - q + j + 1)
        return int(seen.sum()) * 4 * c.head_dim * c.num_q_heads

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def shares_blocks(self) -> bool:
        """Whether some physical block is referenced by more than one sequence's table."""
        return bool((self.ref_counts > 1).any())

    def block_counts(self) -> tuple:
        """(distinct physical blocks the tables reference, blocks the same contexts would take
        if no block were shared): the block-count saving of prefix sharing for this batch."""
        B = self.cfg.block_size
        nb = (self.context_lens.astype(np.int64) + B - 1) // B
        used = [self.block_tables[s, :nb[s]] for s in range(self.cfg.num_seqs)]
        distinct = int(np.unique(np.concatenate(used)).size) if used else 0
        return distinct, int(nb.sum())

    def kv_bytes(self) -> int:
        """K plus V bytes the attention must read: every context token, every KV head."""
        c = self.cfg
        return int(self.context_lens.astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * c.esz

    def unique_kv_bytes(self) -> int:
        """K plus V bytes of the distinct (physical block, slot) pairs the attention reads: what
        must come from HBM at least once when sequences share blocks (equal to kv_bytes when
        none are shared)."""
        c = self.cfg
        B = c.block_size
        used = {}
        for s in range(c.num_seqs):
            n = int(self.context_lens[s])
            for j in range(-(-n // B)):
                b = int(self.block_tables[s, j])
                used[b] = max(used.get(b, 0), min(B, n - j * B))
        return sum(used.values()) * c.num_kv_heads * c.head_dim * 2 * c.esz


def _draw_context_lens(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.ctx[0]
    if kind == "fixed":
        lens = np.asarray(cfg.ctx[1], dtype=np.int64)
        if lens.shape != (cfg.num_seqs,):
            raise ValueError("one fixed length per sequence")
        return lens
    if kind == "uniform":
        lo, hi = cfg.ctx[1], cfg.ctx[2]
        return rng.integers(lo, hi + 1, size=cfg.num_seqs).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = cfg.ctx[1:]
        x = np.exp(rng.normal(math.log(median), sigma, size=cfg.num_seqs))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    raise ValueError(kind)


def build_batch(cfg: DecodeConfig) -> DecodeBatch:
    """Draw context lengths and build block tables through the block manager.

    Every sequence's context includes its newest token (written this step at ``ctx - 1``);
    the blocks it occupies are handed out in seeded random physical order.
    """
    rng = np.random.default_rng(cfg.seed)
    B = cfg.block_size
    kind = cfg.ctx[0]
    if kind == "shared_prefix":
        prompt, lo, hi, n = cfg.ctx[1:]
        num_prompts = cfg.num_seqs // n
        suffix = rng.integers(lo, hi + 1, size=(num_prompts, n)).astype(np.int64)
        ctx = (prompt + suffix).reshape(-1)
        pb = -(-prompt // B)
        cow_per_prompt = (n - 1) if prompt % B else 0
        blocks_needed = (num_prompts * (pb + cow_per_prompt)
                         + int(sum(-(-int(c) // B) - pb for c in ctx)))
    else:
        ctx = _draw_context_lens(cfg, rng)
        suffix = None
        blocks_needed = int(sum(-(-int(c) // B) for c in ctx))
    maxb = max(1, -(-cfg.max_ctx_bound // B))
    if cfg.placement == "contiguous":
        if kind == "shared_prefix":
            raise ValueError("a contiguous cache cannot share blocks")
        S = cfg.num_seqs
        nb_pool = S * maxb + 1
        # hand-out order: the poison block (the last id) first, then each sequence's own span
        spans = [np.arange(s * maxb, s * maxb + -(-int(c) // B)) for s, c in enumerate(ctx)]
        used = np.concatenate([np.array([nb_pool - 1])] + spans)
        rest = np.setdiff1d(np.arange(nb_pool), used)
        bm = BlockManager(nb_pool, B, order=np.concatenate([used, rest]))
    else:
        nb_pool = cfg.num_blocks or int(math.ceil(cfg.pool_slack * blocks_needed)) + 1
        if nb_pool < blocks_needed + 1:
            raise PoolExhausted(f"pool of {nb_pool} blocks cannot hold {blocks_needed} + poison")
        bm = BlockManager(nb_pool, B, rng=rng)
    poison = bm.take()
    if kind == "shared_prefix":
        prompt, lo, hi, n = cfg.ctx[1:]
        seqs = []
        for p in range(cfg.num_seqs // n):
            root = bm.new_sequence()
            bm.append_tokens(root, prompt)
            children = [bm.fork(root) for _ in range(n)]
            bm.free_sequence(root)
            for i, c in enumerate(children):
                bm.append_tokens(c, int(suffix[p, i]))
            seqs.extend(children)
    else:
        seqs = []
        for c in ctx:
            s = bm.new_sequence()
            bm.append_tokens(s, int(c))
            seqs.append(s)
    S = cfg.num_seqs
    tables = np.full((S, maxb), poison, dtype=np.int32)
    for i, s in enumerate(seqs):
        t = bm.tables[s]
        tables[i, :len(t)] = t
    lens = np.array([bm.lengths[s] for s in seqs], dtype=np.int32)
    assert np.array_equal(lens, np.asarray(ctx, dtype=np.int32))
    ref = bm.ref.copy()
    ref[poison] = 0
    pairs = np.array(bm.copies, dtype=np.int32).reshape(-1, 2)
    waste = np.array([bm.wasted_slots(s) for s in seqs], dtype=np.int64)
    qlens = _draw_query_lens(cfg, lens)
    token_seq = np.repeat(np.arange(S, dtype=np.int32), qlens)
    token_pos = np.concatenate([np.arange(int(n) - int(q), int(n), dtype=np.int32)
                                for n, q in zip(lens, qlens)] or [np.zeros(0, np.int32)])
    return DecodeBatch(
        cfg=cfg, context_lens=lens, block_tables=tables, num_blocks=nb_pool,
        poison_block=int(poison), copy_pairs=pairs, token_seq=token_seq,
        token_pos=token_pos.astype(np.int32), ref_counts=ref, wasted_slots=waste,
        query_lens=qlens)


def _draw_query_lens(cfg: DecodeConfig, lens: np.ndarray) -> np.ndarray:
    """New tokens per sequence (from a generator of its own, so the rest of the batch does not
    depend on the choice)."""
    kind = cfg.new_tokens[0]
    if kind == "one":
        # one per sequence even at ctx = 0 (its cache write has position -1 and is skipped)
        return np.ones(len(lens), dtype=np.int32)
    if kind == "all":
        return lens.astype(np.int32)
    if kind == "uniform":
        lo, hi = cfg.new_tokens[1:]
        rng = np.random.default_rng([cfg.seed, 101])
        q = rng.integers(lo, hi + 1, size=len(lens))
        return np.minimum(q, lens).astype(np.int32)
    raise ValueError(kind)


def _torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def make_values(batch: DecodeBatch, device="cpu", seed: int | None = None, poison_nan=True):
    """N(0,1) query, new-token key/value and pool contents, rounded (nearest-even) to the dtype.

    Returns a dict of torch tensors on ``device``:
      query [T, Hq, d], key/value [T, Hkv, d], k_pool/v_pool [NB, Hkv, B*d], with T the number
      of new tokens (one per sequence in a decode step, so query is then [S, Hq, d]).
    With ``poison_nan`` the poison block (where every unused table entry points) is NaN, so a
    read past a sequence's last block shows up in the result.
    """
    import torch
    cfg = batch.cfg
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 1000003 + (0 if seed is None else seed))
    tdt = _torch_dtype(cfg.dtype)
    S, Hq, Hkv, d, B = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    T = int(batch.token_seq.shape[0])
    NB = batch.num_blocks

    def draw(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(tdt)

    out = {
        "query": draw(T, Hq, d),
        "key": draw(T, Hkv, d),
        "value": draw(T, Hkv, d),
    }
    for name in ("k_pool", "v_pool"):
        pool = torch.empty(NB, Hkv, B * d, device=device, dtype=tdt)
        # fill in slabs to bound the float32 temporary
        step = max(1, (1 << 26) // (Hkv * B * d))
        for b0 in range(0, NB, step):
            b1 = min(NB, b0 + step)
            pool[b0:b1] = draw(b1 - b0, Hkv, B * d)
        if poison_nan:
            pool[batch.poison_block] = float("nan")
        out[name] = pool
    return out
