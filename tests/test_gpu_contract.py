"""Behaviour include/pa.h defines at the edges of the callers' contract, through the C ABI:
cache writes of tokens outside the table are skipped, copy pairs naming a block outside the pool
are skipped, and decode truncates contexts longer than max_context_len. Each kernel checks these
cases itself before touching the table or a pool, so they are ordinary launches; the expected
pools and outputs come from the oracle on the valid part of the input."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_384_amd as pa
from paged_kv_cache_384_amd import workloads as wl
from _gpu_cases import Prepared, check_attention, log, same_bits
from _helpers import to_storage

pytestmark = pytest.mark.gpu


def test_cache_write_skips_tokens_outside_the_table():
    """Tokens whose sequence is outside [0, num_seqs) or whose position is negative or at or past
    max_blocks_per_seq * B change nothing; the other tokens are written as usual."""
    cfg = wl.DecodeConfig("skip_bf16", "bf16", num_seqs=5, num_q_heads=4, num_kv_heads=2,
                          head_dim=128, ctx=("uniform", 10, 200), seed=43)
    P = Prepared(cfg, poison=False)
    b = P.batch
    W, B = b.max_blocks_per_seq, cfg.block_size
    seq = b.token_seq.copy()
    pos = b.token_pos.copy()
    seq[0], seq[1] = -1, cfg.num_seqs      # sequence out of range
    pos[2], pos[3] = W * B, -5             # position past the table / negative
    log(f"[contract] cache write: seq {seq.tolist()} pos {pos.tolist()}")
    dev = P.kp_d.device
    pa.pa_reshape_and_cache(P.kp_d, P.vp_d, P.key_d, P.val_d, P.bt_d,
                            torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev))
    torch.cuda.synchronize()
    keep = [n for n in range(len(seq)) if 0 <= seq[n] < cfg.num_seqs and 0 <= pos[n] < W * B]
    assert keep == [4]
    kp, vp = oracle.reshape_and_cache_ref(P.kp, P.vp, P.key[keep], P.val[keep], b.block_tables,
                                          seq[keep], pos[keep], **P.kw)
    assert same_bits(to_storage(P.kp_d), kp, cfg.dtype)
    assert same_bits(to_storage(P.vp_d), vp, cfg.dtype)


def test_copy_skips_pairs_outside_the_pool():
    cfg = wl.DecodeConfig("copyskip_f16", "f16", num_seqs=4, num_q_heads=4, num_kv_heads=4,
                          head_dim=64, ctx=("uniform", 10, 100), seed=44)
    P = Prepared(cfg, poison=False)
    NB = P.batch.num_blocks
    pairs = np.array([[1, 2], [-1, 3], [4, NB], [NB + 7, 5], [6, 0]], np.int32)
    log(f"[contract] copy pairs {pairs.tolist()} (pool of {NB} blocks)")
    pa.pa_copy_blocks(P.kp_d, P.vp_d, torch.from_numpy(pairs.reshape(-1)).to(P.kp_d.device),
                      head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    valid = pairs[[0, 4]]
    kp, vp = oracle.copy_blocks_ref(P.kp, P.vp, valid, **P.kw)
    assert same_bits(to_storage(P.kp_d), kp, cfg.dtype)
    assert same_bits(to_storage(P.vp_d), vp, cfg.dtype)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_truncates_to_max_context_len(dt):
    """Contexts longer than max_context_len are read up to it: the output equals the oracle's
    over the truncated contexts (the new token's own slot then lies past the cut and is
    ignored)."""
    cfg = wl.DecodeConfig(f"trunc_{dt}", dt, num_seqs=4, num_q_heads=8, num_kv_heads=2,
                          head_dim=128, ctx=("fixed", (700, 300, 1200, 513)), seed=45)
    P = Prepared(cfg)
    P.write_cache(check_pools=False)
    b = P.batch
    mcl = 512
    out_d = torch.full_like(P.q_d, float("nan"))
    for part in (0, 128):
        pa.pa_decode(out_d, P.q_d, P.kp_d, P.vp_d, P.bt_d, P.ctx_d, cfg.scale, mcl, part)
        torch.cuda.synchronize()
        got = oracle.to_f64(to_storage(out_d), dt)
        ref = oracle.paged_decode_ref(P.q, P.kp, P.vp, b.block_tables,
                                      np.minimum(b.context_lens, mcl), cfg.scale, **P.kw)
        r = check_attention(got, ref, dt, f"truncated decode, partition {part}")
        log(f"[contract] decode max_context_len={mcl} partition={part}: "
            f"error {r['max_abs_err']:.3g}")
