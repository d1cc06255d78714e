"""Seeded random sweep of small decode and prefill steps against the oracle, through the C ABI:
dtypes, head dims, block sizes, head groupings (including group sizes 3 and 8), context-length
mixes and partition sizes drawn together, so combinations the hand-written cases do not name are
covered too. The draw is fixed (one seed), so every run checks the same cases."""
import numpy as np
import pytest

from paged_kv_cache_384_amd import workloads as wl
from _gpu_cases import log, run_prefill, run_step

pytestmark = pytest.mark.gpu


def _decode_cases(n=64, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = str(rng.choice(["f32", "f16", "bf16"]))
        d = int(rng.choice([64, 128]))
        B = int(rng.choice([8, 16, 32]))
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        S = int(rng.integers(1, 9))
        hi = int(rng.choice([40, 300, 1500, 3000]))
        q = max(16, B)
        part = int(rng.choice([0, q, 2 * q, 256, 512, 1024, 2048]))
        if rng.random() < 0.25 and S >= 2:
            ctx = ("shared_prefix", int(rng.integers(1, 200)), 1, int(rng.integers(2, 120)), 2)
            S = S // 2 * 2
        else:
            ctx = ("uniform", 1, hi)
        cfg = wl.DecodeConfig(f"rd{i}_{dt}_d{d}_b{B}_{g * hkv}q{hkv}kv", dt, num_seqs=S,
                              num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, block_size=B,
                              ctx=ctx, seed=1000 + i)
        out.append((cfg, part))
    return out


def _prefill_cases(n=32, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = str(rng.choice(["f16", "bf16"]))
        d = int(rng.choice([64, 128]))
        B = int(rng.choice([8, 16, 32]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 3, 4]))
        S = int(rng.integers(1, 5))
        lo = int(rng.integers(1, 200))
        hi = lo + int(rng.integers(0, 500))
        new = ("all",) if rng.random() < 0.4 else ("uniform", 1, int(rng.integers(2, 300)))
        cfg = wl.DecodeConfig(f"rp{i}_{dt}_d{d}_b{B}_{g * hkv}q{hkv}kv", dt, num_seqs=S,
                              num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, block_size=B,
                              ctx=("uniform", lo, hi), new_tokens=new, seed=2000 + i)
        out.append(cfg)
    return out


DECODE = _decode_cases()
PREFILL = _prefill_cases()


@pytest.mark.parametrize("cfg,part", DECODE, ids=[f"{c.name}_p{p}" for c, p in DECODE])
def test_random_decode(cfg, part):
    log(f"[random] decode {cfg.name} S={cfg.num_seqs} ctx={cfg.ctx} partition={part}")
    r = run_step(cfg, partition_size=part)
    log(f"    max_abs_err={r['max_abs_err']:.3g}")


@pytest.mark.parametrize("cfg", PREFILL, ids=[c.name for c in PREFILL])
def test_random_prefill(cfg):
    log(f"[random] prefill {cfg.name} S={cfg.num_seqs} ctx={cfg.ctx} new={cfg.new_tokens}")
    r = run_prefill(cfg)
    log(f"    rows={r['rows']} max_abs_err={r['max_abs_err']:.3g}")
