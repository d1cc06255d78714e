"""The decode step captured in a HIP graph, as bench.py times it: copy-on-write copies, the cache
write and both decode stages recorded once, then replayed several times with eager work and
synchronisations in between. Every replay must reproduce the eager step bit for bit (the
kernels are deterministic and the step is idempotent: it rewrites the same slots with the same
values), and the eager step itself matches the CPU oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_384_amd as pa
from paged_kv_cache_384_amd import workloads as wl
from _gpu_cases import log, run_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over", [
    ("cow_fp16", dict(num_seqs=16, num_q_heads=8, num_kv_heads=8,
                      ctx=("shared_prefix", 40, 1, 600, 4))),
    ("gqa_bf16", dict(num_seqs=12, num_q_heads=16, num_kv_heads=4,
                      ctx=("lognormal", 400, 0.75, 1, 2000))),
], ids=["cow_fp16", "gqa_bf16"])
def test_graph_replay_matches_eager(name, over):
    cfg = wl.config(name, **over)
    log(f"[graph] {name} {over}: eager step against the oracle")
    run_step(cfg, partition_size=64)

    dev = torch.device("cuda:0")
    batch = wl.build_batch(cfg)
    vals = wl.make_values(batch, device=dev, seed=3, poison_nan=False)
    bt = torch.from_numpy(batch.block_tables).to(dev)
    ctx = torch.from_numpy(batch.context_lens).to(dev)
    tseq = torch.from_numpy(batch.token_seq).to(dev)
    tpos = torch.from_numpy(batch.token_pos).to(dev)
    pairs = torch.from_numpy(batch.copy_pairs.reshape(-1)).to(dev)
    part = 64
    shared = batch.shares_blocks
    ws_bytes = pa.pa_decode_workspace_bytes(vals["k_pool"], cfg.num_seqs, cfg.num_q_heads,
                                            cfg.head_dim, batch.max_context_len, part,
                                            shared_blocks=shared)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty_like(vals["query"])

    def step(o):
        if batch.copy_pairs.shape[0]:
            pa.pa_copy_blocks(vals["k_pool"], vals["v_pool"], pairs, head_dim=cfg.head_dim)
        pa.pa_reshape_and_cache(vals["k_pool"], vals["v_pool"], vals["key"], vals["value"], bt,
                                tseq, tpos)
        pa.pa_decode(o, vals["query"], vals["k_pool"], vals["v_pool"], bt, ctx, cfg.scale,
                     batch.max_context_len, part, ws, shared_blocks=shared)

    step(out)
    torch.cuda.synchronize()
    eager = out.clone()
    k_eager, v_eager = vals["k_pool"].clone(), vals["v_pool"].clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    other = torch.empty_like(out)
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[graph] {name} replay {r}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} output"
        assert torch.equal(vals["k_pool"], k_eager) and torch.equal(vals["v_pool"], v_eager)
        # eager work between replays, on the same buffers and workspace
        step(other)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16))
    assert np.isfinite(eager.float().cpu().numpy()).all()


def test_prefill_graph_replay_matches_eager():
    """A prefill step (cache write of every new token, then pa_prefill) captured once and
    replayed with eager work in between reproduces the eager step bit for bit; the eager step
    matches the oracle (the same inputs as the small prefill parity case)."""
    from _gpu_cases import Prepared, run_prefill
    cfg = wl.DecodeConfig("graph_prefill", "bf16", num_seqs=4, num_q_heads=8, num_kv_heads=2,
                          head_dim=128, block_size=16, ctx=("uniform", 100, 600),
                          new_tokens=("uniform", 1, 300), seed=21)
    P = Prepared(cfg, poison=False)
    log("[graph] prefill: eager step against the oracle")
    run_prefill(cfg, prepared=P)
    b = P.batch
    out = torch.empty_like(P.q_d)

    def step(o):
        pa.pa_reshape_and_cache(P.kp_d, P.vp_d, P.key_d, P.val_d, P.bt_d, P.seq_d, P.pos_d)
        pa.pa_prefill(o, P.q_d, P.kp_d, P.vp_d, P.bt_d, P.qs_d, P.ctx_d, cfg.scale,
                      b.max_query_len, b.max_context_len)

    step(out)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    other = torch.empty_like(out)
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[graph] prefill replay {r}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} output"
        step(other)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16))
