"""The five workloads at full size, in the launch configuration bench.py times (the workload's
partition setting, library defaults otherwise). Cache writes and copy-on-write copies are
compared bit for bit over the whole pools; attention outputs are compared with the oracle on a
sample of sequences (every query head of each), including the longest and shortest contexts."""
import numpy as np
import pytest

from paged_kv_cache_384_amd import workloads as wl
from _gpu_cases import log, run_step

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def sample_for(name):
    b = wl.build_batch(wl.CONFIGS[name])
    lens = b.context_lens
    S = len(lens)
    if S <= 8:
        return list(range(S)) if name != "long_bf16" else [int(np.argmax(lens)), int(np.argmin(lens))]
    picks = {0, S - 1, int(np.argmax(lens)), int(np.argmin(lens)), S // 2}
    if name == "cow_fp16":
        picks |= set(range(8))       # all samples of prompt 0 (7 copies + the in-place sharer)
    return sorted(picks)


@pytest.mark.parametrize("name", ["tiny_fp32", "opt13b_fp16", "gqa_bf16", "cow_fp16", "long_bf16"])
def test_full_size(name):
    cfg = wl.CONFIGS[name]
    seqs = sample_for(name)
    log(f"[full] {name} partition={cfg.partition_size} sampled seqs={seqs}")
    r = run_step(cfg, partition_size=cfg.partition_size, sample=seqs,
                 device_values=name != "tiny_fp32")
    log(f"    max_abs_err={r['max_abs_err']:.3g} max|o|={r['max_abs_out']:.3g} "
        f"oracle {r['oracle_s']:.1f}s prep {r['prep_s']:.1f}s")
