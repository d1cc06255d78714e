"""The five decode workloads at full size, in the launch configuration bench.py times (the
workload's partition setting, library defaults otherwise). Cache writes and copy-on-write copies
are compared bit for bit over the whole pools; attention outputs of every sequence and every
query head are compared with the oracle element by element."""
import pytest

from paged_kv_cache_384_amd import workloads as wl
from _gpu_cases import log, run_step

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.mark.parametrize("name", ["tiny_fp32", "opt13b_fp16", "gqa_bf16", "cow_fp16", "long_bf16"])
def test_full_size(name):
    cfg = wl.CONFIGS[name]
    log(f"[full] {name} partition={cfg.partition_size}: every sequence and head")
    r = run_step(cfg, partition_size=cfg.partition_size, device_values=name != "tiny_fp32")
    log(f"    max_abs_err={r['max_abs_err']:.3g} max err/bar={r['max_err_over_bar']:.3g} "
        f"allowance elements={r['allowance_elems']} max|o|={r['max_abs_out']:.3g} "
        f"oracle {r['oracle_s']:.1f}s prep {r['prep_s']:.1f}s")


@pytest.mark.parametrize("name", ["opt13b_fp16", "gqa_bf16", "long_bf16"])
def test_kv_head_shard(name):
    """One GPU's share of the batch when its KV heads are split 8 ways (what bench.py
    --kv-head-shards 8 times): the same sequences, tables and pool with 1/8 of the heads, so far
    fewer workgroups than the whole batch launches."""
    from dataclasses import replace
    full = wl.CONFIGS[name]
    cfg = replace(full, name=f"{name}_kvshard8", num_q_heads=full.num_q_heads // 8,
                  num_kv_heads=full.num_kv_heads // 8)
    log(f"[full] {cfg.name}: {cfg.num_q_heads} query heads over {cfg.num_kv_heads} KV heads")
    r = run_step(cfg, partition_size=cfg.partition_size, device_values=True)
    log(f"    max_abs_err={r['max_abs_err']:.3g} max err/bar={r['max_err_over_bar']:.3g}")
