"""pa_measure_tile_read (the bandwidth reference bench.py sets beside the attention kernel)
through the C ABI: each wavefront's XOR of the words it read equals the same fold made on the
host, so the reference really reads the tiles it is given, in full, from both pools."""
import numpy as np
import pytest
import torch

import paged_kv_cache_384_amd as pa
from _gpu_cases import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tile_bytes,num_tiles", [(4096, 1000), (1024, 33), (8192, 64)])
def test_tile_read_folds(tile_bytes, num_tiles):
    rng = np.random.default_rng(tile_bytes + num_tiles)
    pool_tiles = num_tiles + 17
    a = rng.integers(0, 2 ** 32, size=pool_tiles * tile_bytes // 4, dtype=np.uint64).astype(np.uint32)
    b = rng.integers(0, 2 ** 32, size=pool_tiles * tile_bytes // 4, dtype=np.uint64).astype(np.uint32)
    order = rng.permutation(pool_tiles)[:num_tiles].astype(np.int32)
    dev = torch.device("cuda:0")
    ta = torch.from_numpy(a.view(np.int32)).to(dev)
    tb = torch.from_numpy(b.view(np.int32)).to(dev)
    tt = torch.from_numpy(order).to(dev)
    sink = pa.pa_measure_tile_read(ta, tb, tt, tile_bytes)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    words = tile_bytes // 4
    A = a.reshape(pool_tiles, words)
    B = b.reshape(pool_tiles, words)
    want = []
    for w in range(0, num_tiles, 32):
        ids = order[w:w + 32]
        want.append(np.bitwise_xor.reduce(np.concatenate([A[ids].ravel(), B[ids].ravel()])))
    log(f"[measure] {num_tiles} tiles of {tile_bytes} B: {len(want)} wavefront folds")
    assert np.array_equal(got[:len(want)], np.array(want, dtype=np.uint32))
