"""The C ABI without a GPU: the library loads, exports every function include/pa.h declares,
and rejects bad arguments on the host before making any HIP call. CPU only."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_384_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH = range(7)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pa.library_path):
        pytest.skip("libpa.so not built")
    if _gpu_visible():
        # these cases pass made-up device addresses; if a check were missing the call would
        # launch with them, so they only run where no GPU can execute a launch
        pytest.skip("host-validation cases run only where no GPU is visible")
    return pa.lib()


def desc(dtype=1, nb=64, hkv=4, d=128, b=16, flags=0):
    return pa.CacheDesc(dtype, nb, hkv, d, b, flags)


P = ctypes.c_void_p
GOOD = P(0x10000)          # aligned, never dereferenced: every case below fails validation first
ODD = P(0x10001)


def test_every_declared_function_is_exported(L):
    declared = header_functions()
    assert set(declared) == set(pa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version_and_status_strings(L):
    assert L.pa_abi_version() == pa.ABI_VERSION
    for s in range(7):
        assert pa.pa_status_string(s)
    assert pa.pa_status_string(99) == "unknown status"


def decode(L, d=None, *, S=2, Hq=4, maxb=8, max_ctx=100, part=0, ws=None, ws_bytes=0,
           ptrs=None):
    d = desc() if d is None else d
    p = ptrs or {}
    return L.pa_decode(ctypes.byref(d) if d is not False else None,
                       p.get("k", GOOD), p.get("v", GOOD), p.get("out", GOOD), p.get("q", GOOD),
                       p.get("bt", GOOD), maxb, p.get("ctx", GOOD), S, Hq, 0.1, max_ctx, part,
                       ws or P(0), ws_bytes, P(0))


def test_decode_validation(L):
    assert decode(L, False) == NULL
    assert decode(L, desc(dtype=7)) == UNSUP
    assert decode(L, desc(d=96)) == UNSUP
    assert decode(L, desc(b=4)) == UNSUP
    assert decode(L, desc(b=64)) == UNSUP
    assert decode(L, desc(b=32), part=16) == SHAPE       # partitions are whole blocks
    assert decode(L, desc(b=8), part=8) == SHAPE         # and whole 16-token groups
    assert decode(L, desc(flags=2)) == UNSUP              # unknown flag bit
    assert decode(L, desc(flags=0x80000000)) == UNSUP
    assert decode(L, desc(nb=0)) == SHAPE
    assert decode(L, desc(hkv=0)) == SHAPE
    assert decode(L, Hq=6) == SHAPE                      # 6 % 4 != 0
    assert decode(L, S=-1) == SHAPE
    assert decode(L, part=24) == SHAPE                   # not a multiple of 16
    assert decode(L, part=4096) == SHAPE                 # above the maximum
    assert decode(L, max_ctx=8 * 16 + 1) == SHAPE        # longer than the table can address
    assert decode(L, max_ctx=-1) == SHAPE
    assert decode(L, maxb=0) == SHAPE
    for k in ("k", "v", "out", "q", "bt", "ctx"):
        assert decode(L, ptrs={k: P(0)}) == NULL, k
    for k in ("k", "v", "out", "q"):
        assert decode(L, ptrs={k: ODD}) == ALIGN, k
    assert decode(L, ptrs={"bt": P(0x10002)}) == ALIGN
    # more than one partition needs a workspace of the advertised size
    need = L.pa_decode_workspace_bytes(ctypes.byref(desc()), 2, 4, 100, 32)
    assert need == 2 * 4 * 4 * (128 + 2) * 4
    assert decode(L, part=32) == WS
    assert decode(L, part=32, ws=GOOD, ws_bytes=need - 1) == WS
    # nothing to do: no pointer is needed and nothing is launched
    assert decode(L, S=0, ptrs={k: P(0) for k in ("k", "v", "out", "q", "bt", "ctx")}) == OK


def test_stage_entry_points_share_validation(L):
    for fn in (L.pa_decode_attention, L.pa_decode_reduce):
        assert fn(None, GOOD, GOOD, GOOD, GOOD, GOOD, 8, GOOD, 2, 4, 0.1, 100, 0, P(0), 0,
                  P(0)) == NULL
        assert fn(ctypes.byref(desc()), GOOD, GOOD, GOOD, GOOD, GOOD, 8, GOOD, 2, 4, 0.1, 100,
                  32, P(0), 0, P(0)) == WS


def test_static_decode_validation(L):
    """pa_decode_static makes pa_decode's checks, and refuses sizes whose partition states
    exceed its fixed array (PA_ERR_WORKSPACE), all before any HIP call."""
    def ds(d=None, *, S=2, Hq=4, maxb=8, max_ctx=100, part=0, ptrs=None):
        d = desc() if d is None else d
        p = ptrs or {}
        return L.pa_decode_static(ctypes.byref(d) if d is not False else None,
                                  p.get("k", GOOD), p.get("v", GOOD), p.get("out", GOOD),
                                  p.get("q", GOOD), p.get("bt", GOOD), maxb, p.get("ctx", GOOD),
                                  S, Hq, 0.1, max_ctx, part, P(0))
    assert ds(False) == NULL
    assert ds(desc(d=96)) == UNSUP
    assert ds(Hq=6) == SHAPE
    assert ds(part=24) == SHAPE
    assert ds(max_ctx=8 * 16 + 1) == SHAPE
    for k in ("k", "v", "out", "q", "bt", "ctx"):
        assert ds(ptrs={k: P(0)}) == NULL, k
    assert ds(ptrs={"q": ODD}) == ALIGN
    assert ds(S=0, ptrs={k: P(0) for k in ("k", "v", "out", "q", "bt", "ctx")}) == OK
    # 2 x 64 heads x 513 partitions of (128 + 2) floats = 34 145 280 bytes > 32 MiB
    big = dict(S=2, Hq=64, maxb=1024, max_ctx=8200, part=16)
    d8 = desc(hkv=8, nb=4096)
    assert L.pa_decode_workspace_bytes(ctypes.byref(d8), 2, 64, 8200, 16) > pa.STATIC_WORKSPACE_BYTES
    assert ds(d8, **big) == WS
    # at 32-token partitions the same batch needs half that: it passes every host check (so
    # it is not run here, where it would launch)
    assert L.pa_decode_workspace_bytes(ctypes.byref(d8), 2, 64, 8200, 32) <= pa.STATIC_WORKSPACE_BYTES


def test_contiguous_twin_validation(L):
    def dc(d=None, *, S=2, maxb=8, max_ctx=100, ptrs=None):
        d = desc() if d is None else d
        p = ptrs or {}
        return L.pa_decode_contiguous(ctypes.byref(d) if d is not False else None,
                                      p.get("k", GOOD), p.get("v", GOOD), p.get("out", GOOD),
                                      p.get("q", GOOD), maxb, p.get("ctx", GOOD), S, 4, 0.1,
                                      max_ctx, 0, P(0), 0, P(0))
    assert dc(False) == NULL
    assert dc(desc(flags=1)) == UNSUP                    # contiguous sequences share nothing
    assert dc(desc(nb=15), maxb=8) == SHAPE              # 2 sequences x 8 blocks > 15
    assert dc(max_ctx=8 * 16 + 1) == SHAPE
    for k in ("k", "v", "out", "q", "ctx"):
        assert dc(ptrs={k: P(0)}) == NULL, k
    assert dc(ptrs={"q": ODD}) == ALIGN
    assert dc(S=0, ptrs={k: P(0) for k in ("k", "v", "out", "q", "ctx")}) == OK


def test_workspace_bytes(L):
    # block sizes 8 and 32: the default partition rounds a short context up to whole
    # 16-token groups and whole blocks
    # (4 query heads per KV head: default partitions of 1024 tokens)
    for b, ctx, parts in ((8, 100, 1), (32, 100, 1), (32, 4096, 4)):
        n = L.pa_decode_workspace_bytes(ctypes.byref(desc(dtype=2, hkv=8, d=128, b=b)), 4, 32,
                                        ctx, 0)
        assert n == (0 if parts == 1 else 4 * 32 * parts * 130 * 4), (b, ctx)
    d = desc(dtype=2, hkv=8, d=128)
    # longest context fits the default partition: no workspace
    assert L.pa_decode_workspace_bytes(ctypes.byref(d), 256, 32, 1024, 0) == 0
    # workgroups of 4 query heads: ceil(4096 / 1024) = 4 states of (d + 2) floats per (seq, head)
    assert L.pa_decode_workspace_bytes(ctypes.byref(d), 256, 32, 4096, 0) == 256 * 32 * 4 * 130 * 4
    assert L.pa_decode_workspace_bytes(ctypes.byref(d), 8, 32, 32768, 512) == 8 * 32 * 64 * 130 * 4
    # single-head workgroups (MHA): 512-token default partitions
    m = desc(dtype=1, hkv=40, d=128)
    assert L.pa_decode_workspace_bytes(ctypes.byref(m), 64, 40, 512, 0) == 0
    assert L.pa_decode_workspace_bytes(ctypes.byref(m), 64, 40, 2048, 0) == 64 * 40 * 4 * 130 * 4
    assert L.pa_decode_workspace_bytes(ctypes.byref(d), 4, 33, 100, 0) == ctypes.c_size_t(-1).value


def test_cache_write_validation(L):
    def rc(d=None, *, T=3, S=2, maxb=4, ptrs=None):
        d = desc() if d is None else d
        p = ptrs or {}
        return L.pa_reshape_and_cache(ctypes.byref(d) if d is not False else None,
                                      p.get("kc", GOOD), p.get("vc", GOOD), p.get("k", GOOD),
                                      p.get("v", GOOD), p.get("bt", GOOD), S, maxb,
                                      p.get("seq", GOOD), p.get("pos", GOOD), T, P(0))
    assert rc(False) == NULL
    assert rc(desc(dtype=5)) == UNSUP
    assert rc(desc(flags=4)) == UNSUP
    assert rc(T=-1) == SHAPE
    assert rc(S=0) == SHAPE
    assert rc(maxb=0) == SHAPE
    for k in ("kc", "vc", "k", "v", "bt", "seq", "pos"):
        assert rc(ptrs={k: P(0)}) == NULL, k
    for k in ("kc", "vc", "k", "v"):
        assert rc(ptrs={k: ODD}) == ALIGN, k
    assert rc(ptrs={"pos": P(0x10002)}) == ALIGN
    assert rc(T=0, ptrs={k: P(0) for k in ("kc", "vc", "k", "v", "bt", "seq", "pos")}) == OK


def test_copy_validation(L):
    d = desc()
    assert L.pa_copy_blocks(None, GOOD, GOOD, GOOD, 3, P(0)) == NULL
    assert L.pa_copy_blocks(ctypes.byref(desc(d=32)), GOOD, GOOD, GOOD, 3, P(0)) == UNSUP
    assert L.pa_copy_blocks(ctypes.byref(d), GOOD, GOOD, GOOD, -1, P(0)) == SHAPE
    assert L.pa_copy_blocks(ctypes.byref(d), P(0), GOOD, GOOD, 3, P(0)) == NULL
    assert L.pa_copy_blocks(ctypes.byref(d), GOOD, ODD, GOOD, 3, P(0)) == ALIGN
    assert L.pa_copy_blocks(ctypes.byref(d), P(0), P(0), P(0), 0, P(0)) == OK


def test_binding_names_match_c_names():
    for name in pa.EXPORTED_SYMBOLS:
        if name != "pa_decode_workspace_bytes":
            assert callable(getattr(pa, name)), name


def test_library_exports_the_abi_and_imports_only_long_standing_hip_symbols():
    """Only the functions pa.h declares are exported as code (the other dynamic symbols are the
    kernel handles the HIP runtime registers), and every HIP symbol the library imports carries
    the hip_4.2 version: the HIP runtime loaded in a process may be an older one than the
    toolchain that built the library (torch ships its own), so a newer symbol would keep the
    library from loading."""
    import shutil
    import subprocess
    if not os.path.exists(pa.library_path) or shutil.which("nm") is None:
        pytest.skip("libpa.so not built or nm missing")
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines()
                if ln.split() and ln.split()[-2] in ("T", "W")}
    assert exported == set(header_functions()), sorted(exported ^ set(header_functions()))[:10]
    out = subprocess.run(["nm", "-D", "--undefined-only", pa.library_path], capture_output=True,
                         text=True, check=True).stdout
    hip = [ln.split()[-1] for ln in out.splitlines() if "hip" in ln.lower()]
    assert hip and all(sym.endswith("@hip_4.2") for sym in hip), hip


def test_swap_validation(L):
    """Both pools of one shape apart from the block count; pointers checked before anything
    runs (the pointer query that follows needs a GPU, so only failures before it run here)."""
    def sw(dd, ss, pairs, n, dk=GOOD):
        return L.pa_swap_blocks(ctypes.byref(dd), dk, GOOD, ctypes.byref(ss), GOOD, GOOD,
                                pairs, n, P(0))
    assert sw(desc(), desc(d=64), GOOD, 2) == SHAPE            # head_dim differs
    assert sw(desc(), desc(b=32), GOOD, 2) == SHAPE            # block size differs
    assert sw(desc(), desc(dtype=2), GOOD, 2) == SHAPE         # dtype differs
    assert sw(desc(), desc(flags=8), GOOD, 2) == UNSUP
    assert sw(desc(), desc(), P(0), 2) == NULL
    assert sw(desc(), desc(), GOOD, 2, dk=P(0)) == NULL
    assert sw(desc(), desc(), GOOD, -1) == SHAPE
    assert sw(desc(), desc(), GOOD, 2, dk=ODD) == ALIGN
    assert sw(desc(), desc(), P(0x10002), 2) == ALIGN
    assert sw(desc(), desc(), P(0), 0) == OK


def test_prefill_validation(L):
    """16-bit pools only; sizes, pointers and alignment checked before the launch."""
    def pf(d=None, *, S=2, Hq=4, maxb=8, mql=100, max_ctx=100, ptrs=None, scale=0.1):
        d = desc() if d is None else d
        p = ptrs or {}
        return L.pa_prefill(ctypes.byref(d) if d is not False else None, p.get("k", GOOD),
                            p.get("v", GOOD), p.get("out", GOOD), p.get("q", GOOD),
                            p.get("bt", GOOD), maxb, p.get("qs", GOOD), p.get("ctx", GOOD), S, Hq,
                            scale, mql, max_ctx, P(0))
    assert pf(False) == NULL
    assert pf(desc(dtype=0)) == UNSUP                    # fp32 has no matrix-core prefill
    assert pf(desc(d=96)) == UNSUP
    assert pf(desc(b=64)) == UNSUP
    assert pf(desc(flags=2)) == UNSUP
    assert pf(Hq=6) == SHAPE                             # not a multiple of 4 KV heads
    assert pf(Hq=0) == SHAPE
    assert pf(S=-1) == SHAPE
    assert pf(mql=-1) == SHAPE
    assert pf(max_ctx=8 * 16 + 1) == SHAPE               # longer than the table
    assert pf(maxb=0) == SHAPE
    for bad in (0.0, -0.1, float("nan"), float("inf")):
        assert pf(scale=bad) == SHAPE, bad
    assert pf(S=1 << 20, Hq=1 << 10, mql=1 << 12) == SHAPE  # grid past 2^32 work-items
    for k in ("k", "v", "out", "q", "bt", "qs", "ctx"):
        assert pf(ptrs={k: P(0)}) == NULL, k
    for k in ("k", "v", "out", "q"):
        assert pf(ptrs={k: P(0x10008)}) == ALIGN, k
    for k in ("bt", "qs", "ctx"):
        assert pf(ptrs={k: P(0x10002)}) == ALIGN, k
    none = {k: P(0) for k in ("k", "v", "out", "q", "bt", "qs", "ctx")}
    assert pf(S=0, ptrs=none) == OK
    assert pf(mql=0, ptrs=none) == OK
    assert pf(desc(dtype=2, d=64, b=8), S=0, max_ctx=64, ptrs=none) == OK
    assert pf(desc(dtype=2, d=64, b=8), S=0, max_ctx=65, ptrs=none) == SHAPE


def test_validate_tables_validation(L):
    """Sizes, pointers and alignment checked before the launch; query_start may be NULL."""
    def vt(d=None, *, S=2, maxb=8, max_ctx=100, ptrs=None):
        d = desc() if d is None else d
        p = ptrs or {}
        return L.pa_validate_tables(ctypes.byref(d) if d is not False else None,
                                    p.get("bt", GOOD), S, maxb, p.get("ctx", GOOD),
                                    p.get("qs", GOOD), max_ctx, p.get("out", GOOD), P(0))
    assert vt(False) == NULL
    assert vt(desc(d=96)) == UNSUP
    assert vt(desc(b=64)) == UNSUP
    assert vt(S=-1) == SHAPE
    assert vt(maxb=0) == SHAPE
    assert vt(max_ctx=-1) == SHAPE
    assert vt(max_ctx=8 * 16 + 1) == SHAPE               # longer than the table
    assert vt(S=1 << 24, maxb=1 << 8, max_ctx=16) == SHAPE  # count could overflow int32
    for k in ("bt", "ctx", "out"):
        assert vt(ptrs={k: P(0)}) == NULL, k
    assert vt(S=0, ptrs={"bt": P(0), "ctx": P(0), "qs": P(0), "out": P(0)}) == NULL
    for k in ("bt", "ctx", "qs", "out"):
        assert vt(ptrs={k: P(0x10002)}) == ALIGN, k


def test_binding_rejects_host_tensors_and_bad_shapes():
    """The Python binding checks placement and shapes before any call reaches the library."""
    import torch
    if not os.path.exists(pa.library_path):
        pytest.skip("libpa.so not built")
    q = torch.zeros(10, 4, 128, dtype=torch.bfloat16)
    pool = torch.zeros(8, 2, 16 * 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    qs = torch.tensor([0, 4, 10], dtype=torch.int32)
    ctx = torch.tensor([4, 6], dtype=torch.int32)
    with pytest.raises(ValueError, match="on the GPU"):
        pa.pa_prefill(torch.empty_like(q), q, pool, pool, bt, qs, ctx, 0.1, 6, 64)
    with pytest.raises(ValueError, match="out must match"):
        pa.pa_prefill(torch.empty(9, 4, 128, dtype=torch.bfloat16), q, pool, pool, bt, qs, ctx,
                      0.1, 6, 64)
    with pytest.raises(ValueError, match="query_start"):
        pa.pa_prefill(torch.empty_like(q), q, pool, pool, bt, qs[:2], ctx, 0.1, 6, 64)
    with pytest.raises(ValueError, match="pools must be"):
        pa.pa_prefill(torch.empty_like(q), q, pool[:, :, :100], pool, bt, qs, ctx, 0.1, 6, 64)
    with pytest.raises(ValueError, match="on the GPU"):
        pa.pa_decode(torch.empty(2, 4, 128, dtype=torch.bfloat16),
                     torch.zeros(2, 4, 128, dtype=torch.bfloat16), pool, pool, bt, ctx, 0.1, 64)


MAX_WGS = ((1 << 32) - 1) // 256   # 256-thread workgroups in a grid of at most 2^32 - 1 items


def test_grids_stay_below_2_32_work_items(L):
    """Every launch's grid (256-thread workgroups) is bounded by 2^32 - 1 work-items on the host:
    one workgroup past the limit gives PA_ERR_SHAPE; at the limit the shape checks pass (a NULL
    pointer then stops the call before it could launch)."""
    one = desc(hkv=1)
    # decode: one workgroup per (KV head, sequence, head group, partition)
    assert decode(L, one, S=MAX_WGS + 1, Hq=1) == SHAPE
    assert decode(L, one, S=MAX_WGS, Hq=1, ptrs={"k": P(0)}) == NULL
    # the merge: one workgroup or wavefront per (sequence, query head) when contexts split
    d8 = desc(hkv=8, dtype=2)
    S = 1 << 19                # 16 S attention workgroups fit, 32 S merged heads do not
    assert decode(L, d8, S=S, Hq=32, maxb=128, max_ctx=2048, ptrs={"k": P(0)}) == SHAPE
    assert decode(L, d8, S=S - 1, Hq=32, maxb=128, max_ctx=2048, ptrs={"k": P(0)}) == NULL
    # cache writes: one thread per 16-byte piece (16 pieces per token at d = 128 fp16, Hkv = 1)
    T = 16 * MAX_WGS
    args = lambda t, k: (ctypes.byref(one), GOOD, GOOD, k, GOOD, GOOD, 2, 4, GOOD, GOOD, t, P(0))
    assert L.pa_reshape_and_cache(*args(T + 16, GOOD)) == SHAPE
    assert L.pa_reshape_and_cache(*args(T, P(0))) == NULL
    # copies: one workgroup per 32 KiB chunk of a block (Hkv = 8: one chunk per pair)
    assert L.pa_copy_blocks(ctypes.byref(desc(hkv=8)), GOOD, GOOD, GOOD, MAX_WGS + 1, P(0)) == SHAPE
    assert L.pa_copy_blocks(ctypes.byref(desc(hkv=8)), P(0), GOOD, GOOD, MAX_WGS, P(0)) == NULL
    # prefill: one workgroup per (sequence, KV head) unit and query head, units rounded up to 8
    pq = lambda S, k: L.pa_prefill(ctypes.byref(one), k, GOOD, GOOD, GOOD, GOOD, 8, GOOD, GOOD,
                                   S, 1, 0.1, 128, 100, P(0))
    assert pq(MAX_WGS - 7 + 8, GOOD) == SHAPE
    assert pq(MAX_WGS - 7, P(0)) == NULL
    # table validation: one workgroup per sequence
    vt = lambda S: L.pa_validate_tables(ctypes.byref(desc()), GOOD, S, 1, GOOD, P(0), 16, GOOD,
                                        P(0))
    assert vt(MAX_WGS + 1) == SHAPE


def test_validate_writes_validation(L):
    """Sizes, pointers and alignment checked before any launch; token and pair arrays may be NULL
    when there are none."""
    def vw(d=None, *, S=2, maxb=4, T=3, npairs=2, ptrs=None):
        d = desc() if d is None else d
        p = ptrs or {}
        return L.pa_validate_writes(ctypes.byref(d) if d is not False else None,
                                    p.get("bt", GOOD), S, maxb, p.get("seq", GOOD),
                                    p.get("pos", GOOD), T, p.get("pairs", GOOD), npairs,
                                    p.get("out", GOOD), P(0))
    assert vw(False) == NULL
    assert vw(desc(d=96)) == UNSUP
    assert vw(desc(b=4)) == UNSUP
    assert vw(T=-1) == SHAPE
    assert vw(npairs=-1) == SHAPE
    assert vw(T=1 << 29, npairs=1 << 29) == SHAPE           # the count could overflow
    assert vw(S=0) == SHAPE
    assert vw(maxb=0) == SHAPE
    assert vw(maxb=1 << 27, ptrs={"out": P(0)}) == SHAPE     # positions past int32 (B = 16)
    for k in ("bt", "seq", "pos", "pairs", "out"):
        assert vw(ptrs={k: P(0)}) == NULL, k
    for k in ("bt", "seq", "pos", "pairs", "out"):
        assert vw(ptrs={k: P(0x10002)}) == ALIGN, k
    # nothing to compare: only the count's pointer is needed (a launch follows, so stop it there)
    none = {k: P(0) for k in ("bt", "seq", "pos", "pairs", "out")}
    assert vw(T=0, npairs=0, S=0, maxb=0, ptrs=none) == NULL


def test_measure_tile_read_validation(L):
    """Sizes, pointers and alignment checked before the launch."""
    def mt(n=64, tb=4096, ptrs=None):
        p = ptrs or {}
        return L.pa_measure_tile_read(p.get("a", GOOD), p.get("b", GOOD), p.get("t", GOOD), n,
                                      tb, p.get("s", GOOD), P(0))
    assert mt(n=-1) == SHAPE
    for tb in (0, 1000, 1536, 65536 + 1024):
        assert mt(tb=tb) == SHAPE, tb
    for k in ("a", "b", "t", "s"):
        assert mt(ptrs={k: P(0)}) == NULL, k
    assert mt(ptrs={"a": ODD}) == ALIGN
    assert mt(ptrs={"t": P(0x10002)}) == ALIGN
    assert mt(n=0, ptrs={k: P(0) for k in "abts"}) == OK
