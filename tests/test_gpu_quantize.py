"""GPU parity of tq_quantize against the CPU oracle (through the C ABI).

Inputs are the seeded synthetic workloads; the oracle quantizes the same
arrays in float64. Codes and sign bits must be bit-exact except within 1e-6
of a decision boundary (fewer than 1e-5 of all coordinates), norms to 1e-6.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotation_amd as m
    m.lib()
    return m


def _run(tq, spec, x, fmt, n_rows, rows=None, seg=(1, 1, 0), dtype="f32"):
    import torch
    oq, dq = gc.quantizers(spec)
    cache = tq.Cache.empty(dq, n_rows, fmt)
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    dr = None if rows is None else torch.from_numpy(np.asarray(rows, np.int64)).cuda()
    tq.tq_quantize(dq, fmt, xt, cache, dst_rows=dr, seg_len=seg[0], seg_stride=seg[1], seg_offset=seg[2])
    torch.cuda.synchronize()
    return oq, dq, cache


def _check(tq, spec, x, fmt, n_rows, rows, dtype="f32", seg=None, pass_rows=True):
    oq, dq, cache = _run(tq, spec, x, fmt, n_rows, rows if pass_rows else None,
                         seg if seg else (1, 1, 0), dtype)
    qv = oracle.quantize(x.astype(np.float64), oq)
    got = gc.select_rows(gc.read_cache(cache, dq), np.asarray(rows))
    return gc.compare_records(x.astype(np.float64), oq, qv, got)


@pytest.mark.parametrize("fmt_name", ["TQ_TOKEN_MAJOR", "TQ_BLOCK32"])
def test_tiny_workload_fp32(tq, fmt_name):
    # d = 128, 4096 iid N(0,1) fp32 keys, 3 bits (2 + 1), seed 0
    wl = synth.workload("tiny")
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_kv_slab(wl, "K", 0, 0, 0, 4096)
    stats = _check(tq, spec, x, getattr(tq, fmt_name), 4096, np.arange(4096), pass_rows=False,
                   seg=(4096, 4096, 0))
    print(stats)


@pytest.mark.parametrize("fmt_name", ["TQ_TOKEN_MAJOR", "TQ_BLOCK32"])
def test_bf16_outliers_4bit_ragged(tq, fmt_name):
    # 1000 vectors (not a multiple of the 64-vector tile), bf16 with x10 outlier channels
    wl = synth.workload("llama8b_decode")
    spec = synth.draw_quantizer(wl, "V")
    x = synth.draw_kv_slab(wl, "V", 0, 3, 100, 1100)
    x[17] = 0.0  # a zero vector
    _check(tq, spec, x, getattr(tq, fmt_name), 1024, np.arange(1000), dtype="bf16")


@pytest.mark.parametrize("name", ["mixed_3p5", "mixed_2p5"])
@pytest.mark.parametrize("fmt_name", ["TQ_TOKEN_MAJOR", "TQ_BLOCK32"])
def test_two_group_fractional_bits(tq, name, fmt_name):
    wl = synth.workload(name)
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_kv_slab(wl, "K", 2, 5, 0, 333)
    _check(tq, spec, x, getattr(tq, fmt_name), 352, np.arange(333), dtype="bf16")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_every_bit_width_d64(tq, m):
    wl = synth.workload("llama8b_decode", d=64, groups=((64, m),), n_outliers=0)
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_kv_slab(wl, "K", 0, 0, 0, 256)
    _check(tq, spec, x, tq.TQ_TOKEN_MAJOR, 256, np.arange(256), dtype="bf16")


# Tile path (more than SMALL_MAX vectors) with bf16 rows of d a multiple of 8
# and d <= 128: the half-precision MFMA variants (bf16 rotation in three parts,
# fp16 sketch product in two parts) must meet the same record rule. Rows given
# by segments take the transposed variant for both formats; an explicit row
# list takes it for token-major records only.
@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("fmt_name", ["TQ_TOKEN_MAJOR", "TQ_BLOCK32"])
@pytest.mark.parametrize("by_segments", [True, False])
def test_tile_path_d64_every_bit_width(tq, m, fmt_name, by_segments):
    wl = synth.workload("llama8b_decode", d=64, groups=((64, m),), n_outliers=0)
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_kv_slab(wl, "K", 0, 1, 0, 1500)
    _check(tq, spec, x, getattr(tq, fmt_name), 1536, np.arange(1500), dtype="bf16",
           seg=(1500, 1536, 0), pass_rows=not by_segments)


@pytest.mark.parametrize("name", ["mixed_3p5", "mixed_2p5"])
def test_tile_path_two_groups(tq, name):
    wl = synth.workload(name)
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_kv_slab(wl, "K", 1, 2, 0, 1300)
    for fmt in (tq.TQ_TOKEN_MAJOR, tq.TQ_BLOCK32):
        _check(tq, spec, x, fmt, 1312, np.arange(1300), dtype="bf16", seg=(1300, 1312, 0), pass_rows=False)


@pytest.mark.parametrize("scale_exp", [-40, -20, 20, 40])
def test_tile_path_input_scale(tq, scale_exp):
    # inputs scaled by a power of two (exact in bf16): far from unit norm the
    # scaled fp16 residual parts must neither overflow nor lose their bits
    wl = synth.workload("llama8b_decode")
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_kv_slab(wl, "K", 0, 5, 0, 700) * np.float32(2.0 ** scale_exp)
    x[3] = 0.0
    x[4, :] = 0.0
    x[4, 7] = np.float32(2.0 ** scale_exp)  # a one-hot vector
    for fmt in (tq.TQ_TOKEN_MAJOR, tq.TQ_BLOCK32):
        _check(tq, spec, x, fmt, 704, np.arange(700), dtype="bf16", seg=(700, 704, 0), pass_rows=False)


# d = 128 with one group (bf16, at least one 64-vector tile) takes the
# pipelined tile path, whose workgroups keep three tiles in flight: enough
# vectors that every workgroup runs several tiles (more than 3 x 256), a
# ragged last tile, segments whose block pairs are partly covered, every code
# width, both formats, and MSE-only block records.
@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("fmt_name,mse_only", [("TQ_TOKEN_MAJOR", False), ("TQ_BLOCK32", False),
                                                ("TQ_BLOCK32", True)])
def test_pipelined_path_many_tiles_per_workgroup(tq, m, fmt_name, mse_only):
    import torch
    wl = synth.workload("llama8b_decode", groups=((128, m),))
    spec = synth.draw_quantizer(wl, "V")
    seg_len, cap, offset = 4100, 4224, 29
    n_vec = 64 * 256 * 3 + 64 * 40 + 37
    n_seg = (n_vec + seg_len - 1) // seg_len
    x = np.concatenate([synth.draw_kv_slab(wl, "V", 0, h, 0, seg_len) for h in range(n_seg)])[:n_vec]
    x[5] = 0.0  # a zero vector
    i = np.arange(n_vec)
    rows = (i // seg_len) * cap + offset + i % seg_len
    oq, dq = gc.quantizers(spec, mse_only=mse_only)
    fmt = getattr(tq, fmt_name)
    cache = tq.Cache.empty(dq, n_seg * cap, fmt)
    cache.codes.fill_(-1)
    if cache.signs is not None and cache.signs.numel():
        cache.signs.fill_(-1)
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    tq.tq_quantize(dq, fmt, xt, cache, seg_len=seg_len, seg_stride=cap, seg_offset=offset)
    torch.cuda.synchronize()
    qv = oracle.quantize(x.astype(np.float64), oq)
    got_all = gc.read_cache(cache, dq)
    gc.compare_records(x.astype(np.float64), oq, qv, gc.select_rows(got_all, rows))
    # rows outside the segments keep every bit (block records share words
    # with them)
    untouched = np.setdiff1d(np.arange(n_seg * cap), rows)
    assert np.all(got_all[0][0][untouched] == 2 ** m - 1)
    if not mse_only:
        assert np.all(got_all[1][0][untouched])


@pytest.mark.parametrize("seg_len,offset,n_vec", [(1000, 5, 2000), (777, 37, 777), (600, 32, 1800), (520, 63, 1040)])
def test_tile_path_block_segments_partial_pairs(tq, seg_len, offset, n_vec):
    # block records by segments whose first and last 64-row block pairs are
    # partly covered: the transposed path merges those words bit by bit into a
    # cache pre-filled with ones; rows outside the segments keep every bit
    import torch
    wl = synth.workload("llama8b_decode")
    spec = synth.draw_quantizer(wl, "V")
    cap = 1152
    n_seg = (n_vec + seg_len - 1) // seg_len
    x = synth.draw_kv_slab(wl, "V", 1, 3, 0, n_vec)
    i = np.arange(n_vec)
    rows = (i // seg_len) * cap + offset + i % seg_len
    oq, dq = gc.quantizers(spec)
    qv = oracle.quantize(x.astype(np.float64), oq)
    cache = tq.Cache.empty(dq, n_seg * cap, tq.TQ_BLOCK32)
    cache.codes.fill_(-1)
    cache.signs.fill_(-1)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    tq.tq_quantize(dq, tq.TQ_BLOCK32, xt, cache, seg_len=seg_len, seg_stride=cap, seg_offset=offset)
    torch.cuda.synchronize()
    got_all = gc.read_cache(cache, dq)
    gc.compare_records(x.astype(np.float64), oq, qv, gc.select_rows(got_all, rows))
    untouched = np.setdiff1d(np.arange(n_seg * cap), rows)
    L = 2 ** dq.mse_bits[0] - 1
    assert np.all(got_all[0][0][untouched] == L) and np.all(got_all[1][0][untouched])


def test_d200_unit_vectors(tq):
    # nearest-neighbour database shape: d = 200, L2-normalised mixture vectors, 4 bits
    wl = synth.workload("nn_search")
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_mixture_vectors(wl, 500, "db")
    for fmt in (tq.TQ_TOKEN_MAJOR, tq.TQ_BLOCK32):
        _check(tq, spec, x, fmt, 512, np.arange(500))


def test_scattered_rows_and_partial_blocks(tq):
    # rows given explicitly in a random order: every block is partial and is
    # updated in place; rows not written keep their previous contents
    import torch
    wl = synth.workload("llama8b_decode")
    spec = synth.draw_quantizer(wl, "V")
    x = synth.draw_kv_slab(wl, "V", 0, 1, 0, 200)
    rows = np.random.default_rng(0).permutation(256)[:200]
    oq, dq = gc.quantizers(spec)
    cache = tq.Cache.empty(dq, 256, tq.TQ_BLOCK32)
    # pre-fill with ones: untouched bits must stay, written fields must be replaced
    cache.codes.fill_(-1)
    cache.signs.fill_(-1)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    tq.tq_quantize(dq, tq.TQ_BLOCK32, xt, cache, dst_rows=torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    got_all = gc.read_cache(cache, dq)
    qv = oracle.quantize(x.astype(np.float64), oq)
    gc.compare_records(x.astype(np.float64), oq, qv, gc.select_rows(got_all, rows))
    untouched = np.setdiff1d(np.arange(256), rows)
    L = 2 ** dq.mse_bits[0] - 1
    assert np.all(got_all[0][0][untouched] == L) and np.all(got_all[1][0][untouched])


def test_append_rows_by_segments(tq):
    # one new token per (batch, head) slice: vector i -> row i * capacity + 777
    wl = synth.workload("llama8b_decode")
    spec = synth.draw_quantizer(wl, "K")
    x = np.stack([synth.draw_kv_slab(wl, "K", 0, h, 777, 778)[0] for h in range(8)])
    cap = 1024
    rows = np.arange(8) * cap + 777
    for fmt in (tq.TQ_TOKEN_MAJOR, tq.TQ_BLOCK32):
        _check(tq, spec, x, fmt, 8 * cap, rows, dtype="bf16", seg=(1, cap, 777), pass_rows=False)


@pytest.mark.parametrize("seg_len,offset,n_vec", [(150, 45, 677), (32, 0, 96), (7, 30, 40), (300, 1, 300)])
def test_segments_partial_blocks_keep_other_rows(tq, seg_len, offset, n_vec):
    # segments of seg_len rows at offset within 256-row slices (the last one
    # ragged), over a cache pre-filled with ones: block records are merged
    # word by word, rows outside the segments keep every bit
    import torch
    wl = synth.workload("llama8b_decode")
    spec = synth.draw_quantizer(wl, "V")
    cap = 512
    n_seg = (n_vec + seg_len - 1) // seg_len
    x = synth.draw_kv_slab(wl, "V", 0, 2, 0, n_vec)
    i = np.arange(n_vec)
    rows = (i // seg_len) * cap + offset + i % seg_len
    oq, dq = gc.quantizers(spec)
    qv = oracle.quantize(x.astype(np.float64), oq)
    for fmt in (tq.TQ_BLOCK32, tq.TQ_TOKEN_MAJOR):
        cache = tq.Cache.empty(dq, n_seg * cap, fmt)
        cache.codes.fill_(-1)
        cache.signs.fill_(-1)
        xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
        tq.tq_quantize(dq, fmt, xt, cache, seg_len=seg_len, seg_stride=cap, seg_offset=offset)
        torch.cuda.synchronize()
        got_all = gc.read_cache(cache, dq)
        gc.compare_records(x.astype(np.float64), oq, qv, gc.select_rows(got_all, rows))
        untouched = np.setdiff1d(np.arange(n_seg * cap), rows)
        L = 2 ** dq.mse_bits[0] - 1
        assert np.all(got_all[0][0][untouched] == L) and np.all(got_all[1][0][untouched])


def test_empty_call_is_noop(tq):
    import torch
    wl = synth.workload("tiny")
    spec = synth.draw_quantizer(wl, "K")
    oq, dq = gc.quantizers(spec)
    cache = tq.Cache.empty(dq, 64, tq.TQ_TOKEN_MAJOR)
    tq.tq_quantize(dq, tq.TQ_TOKEN_MAJOR, torch.zeros((0, 128), device="cuda"), cache)
    torch.cuda.synchronize()
    assert int(cache.codes.abs().sum()) == 0


# Calls with at most SMALL_MAX vectors take the one-workgroup-per-vector path.
SMALL_MAX = 512
SMALL_CASES = [
    # name, overrides, kind, format, dtype, n_vec
    ("llama8b_decode", {}, "K", "TQ_TOKEN_MAJOR", "bf16", 1),
    ("llama8b_decode", {}, "V", "TQ_BLOCK32", "bf16", 64),
    ("mixed_3p5", {}, "K", "TQ_TOKEN_MAJOR", "bf16", 17),
    ("mixed_3p5", {}, "V", "TQ_BLOCK32", "bf16", 17),
    ("mixed_2p5", {}, "V", "TQ_BLOCK32", "bf16", 5),
    ("tiny", {}, "K", "TQ_BLOCK32", "f32", 40),
    ("llama8b_decode", dict(d=64, groups=((64, 1),), n_outliers=0), "K", "TQ_TOKEN_MAJOR", "bf16", 33),
    ("llama8b_decode", dict(d=64, groups=((64, 4),), n_outliers=0), "V", "TQ_BLOCK32", "bf16", 33),
    ("tiny", dict(d=100, groups=((100, 2),)), "K", "TQ_TOKEN_MAJOR", "f32", 9),
    ("tiny", dict(d=120, groups=((120, 3),)), "K", "TQ_BLOCK32", "f32", 9),
]


@pytest.mark.parametrize("name,over,kind,fmt_name,dtype,n_vec", SMALL_CASES)
def test_few_vectors_path(tq, name, over, kind, fmt_name, dtype, n_vec):
    # a handful of vectors, one per 32-row block or packed into a block,
    # into a cache pre-filled with ones: the records of the written rows
    # against the oracle, every bit of the other rows kept
    import torch
    wl = synth.workload(name, **over)
    spec = synth.draw_quantizer(wl, kind)
    x = synth.draw_kv_slab(wl, kind, 1, 0, 0, n_vec).copy()
    x[n_vec // 2] = 0.0  # a zero vector
    rows = np.random.default_rng(n_vec).permutation(128)[:n_vec] * (3 if n_vec < 40 else 1)
    n_rows = 384
    oq, dq = gc.quantizers(spec)
    fmt = getattr(tq, fmt_name)
    cache = tq.Cache.empty(dq, n_rows, fmt)
    cache.codes.fill_(-1)
    cache.signs.fill_(-1)
    xt = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    tq.tq_quantize(dq, fmt, xt, cache, dst_rows=torch.from_numpy(rows.astype(np.int64)).cuda())
    torch.cuda.synchronize()
    got_all = gc.read_cache(cache, dq)
    qv = oracle.quantize(x.astype(np.float64), oq)
    gc.compare_records(x.astype(np.float64), oq, qv, gc.select_rows(got_all, rows))
    untouched = np.setdiff1d(np.arange(n_rows), rows)
    for g in range(len(dq.mse_bits)):
        assert np.all(got_all[0][g][untouched] == 2 ** dq.mse_bits[g] - 1)
        assert np.all(got_all[1][g][untouched])


def test_few_vectors_unaligned_rows(tq):
    # fp32 rows with a stride of d + 1 floats (no 16-byte loads), by segments
    import torch
    wl = synth.workload("tiny")
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_kv_slab(wl, "K", 0, 0, 0, 12)
    xs = torch.zeros((12, 129), device="cuda")
    xs[:, :128] = torch.from_numpy(x).cuda()
    oq, dq = gc.quantizers(spec)
    for fmt in (tq.TQ_TOKEN_MAJOR, tq.TQ_BLOCK32):
        cache = tq.Cache.empty(dq, 12 * 64, fmt)
        tq.tq_quantize(dq, fmt, xs[:, :128], cache, seg_len=1, seg_stride=64, seg_offset=37)
        torch.cuda.synchronize()
        qv = oracle.quantize(x.astype(np.float64), oq)
        gc.compare_records(x.astype(np.float64), oq, qv,
                           gc.select_rows(gc.read_cache(cache, dq), np.arange(12) * 64 + 37))


def test_few_vectors_agree_with_tiles(tq):
    # the same SMALL_MAX vectors through the few-vector path (one call) and the
    # tile path (inside a call with one vector more): equal records up to the
    # boundary rule
    import torch
    wl = synth.workload("llama8b_decode")
    spec = synth.draw_quantizer(wl, "K")
    n = SMALL_MAX
    x = synth.draw_kv_slab(wl, "K", 0, 4, 0, n + 1)
    oq, dq = gc.quantizers(spec)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    a = tq.Cache.empty(dq, n + 32, tq.TQ_TOKEN_MAJOR)
    b = tq.Cache.empty(dq, n + 32, tq.TQ_TOKEN_MAJOR)
    tq.tq_quantize(dq, tq.TQ_TOKEN_MAJOR, xt[:n], a, seg_len=n, seg_stride=n)
    tq.tq_quantize(dq, tq.TQ_TOKEN_MAJOR, xt, b, seg_len=n + 1, seg_stride=n + 1)
    torch.cuda.synchronize()
    ca, cb = (c.codes.cpu().numpy().reshape(n + 32, -1)[:n] for c in (a, b))
    sa, sb = (c.signs.cpu().numpy().reshape(n + 32, -1)[:n] for c in (a, b))
    na, nb = (c.norms.cpu().numpy().reshape(n + 32, -1)[:n] for c in (a, b))
    assert np.mean(np.all(ca == cb, axis=1) & np.all(sa == sb, axis=1)) >= 0.95
    # norms n to 1e-6 relative, residual norms gamma to 2e-6 n (the record rule)
    assert np.all(np.abs(na[:, 0] - nb[:, 0]) <= 1e-6 * nb[:, 0])
    assert np.all(np.abs(na[:, 1] - nb[:, 1]) <= 2e-6 * nb[:, 0])


# MSE-only records (stage one alone): codes and norms, no sign words; the
# tile path (more than SMALL_MAX vectors) and the few-vector path, both formats,
# scattered rows (partial 32-row blocks) into a cache pre-filled with ones.
MSE_ONLY_CASES = [
    # name, kind, format, dtype, n_vec
    ("llama8b_decode", "V", "TQ_BLOCK32", "bf16", 600),
    ("llama8b_decode", "V", "TQ_BLOCK32", "bf16", 300),
    ("llama8b_decode", "V", "TQ_BLOCK32", "bf16", 1),
    ("mixed_3p5", "V", "TQ_BLOCK32", "bf16", 17),
    ("mixed_3p5", "V", "TQ_TOKEN_MAJOR", "bf16", 700),
    ("tiny", "K", "TQ_TOKEN_MAJOR", "f32", 40),
    ("tiny", "K", "TQ_BLOCK32", "f32", 129),
    ("tiny", "K", "TQ_BLOCK32", "f32", 1029),
]


@pytest.mark.parametrize("name,kind,fmt_name,dtype,n_vec", MSE_ONLY_CASES)
def test_mse_only_records(tq, name, kind, fmt_name, dtype, n_vec):
    import torch
    wl = synth.workload(name)
    spec = synth.draw_quantizer(wl, kind)
    x = synth.draw_kv_slab(wl, kind, 0, 1, 0, n_vec).copy()
    x[n_vec // 2] = 0.0
    n_rows = 32 * ((3 * n_vec + 31) // 32 + 1)
    rows = np.random.default_rng(n_vec + 5).permutation(n_rows)[:n_vec]
    oq, dq = gc.quantizers(spec, mse_only=True)
    fmt = getattr(tq, fmt_name)
    cache = tq.Cache.empty(dq, n_rows, fmt)
    assert cache.signs.numel() == 0
    cache.codes.fill_(-1)
    xt = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    tq.tq_quantize(dq, fmt, xt, cache, dst_rows=torch.from_numpy(rows.astype(np.int64)).cuda())
    torch.cuda.synchronize()
    got_all = gc.read_cache(cache, dq)
    qv = oracle.quantize(x.astype(np.float64), oq)
    print(gc.compare_records(x.astype(np.float64), oq, qv, gc.select_rows(got_all, rows)))
    untouched = np.setdiff1d(np.arange(n_rows), rows)
    for g in range(len(dq.mse_bits)):
        assert np.all(got_all[0][g][untouched] == 2 ** dq.mse_bits[g] - 1)


# fp16 norm storage: codes and signs as in the float32 layout, the norms
# within one float16 unit of the oracle's (both round to nearest even)
F16_CASES = [
    # name, kind, format, dtype, n_vec, mse_only
    ("llama8b_decode", "K", "TQ_TOKEN_MAJOR", "bf16", 1, False),
    ("llama8b_decode", "V", "TQ_BLOCK32", "bf16", 300, False),
    ("llama8b_decode", "V", "TQ_BLOCK32", "bf16", 600, False),
    ("mixed_3p5", "K", "TQ_TOKEN_MAJOR", "bf16", 700, False),
    ("mixed_3p5", "V", "TQ_BLOCK32", "bf16", 17, True),
    ("tiny", "K", "TQ_BLOCK32", "f32", 129, True),
]


@pytest.mark.parametrize("name,kind,fmt_name,dtype,n_vec,mse_only", F16_CASES)
def test_fp16_norm_records(tq, name, kind, fmt_name, dtype, n_vec, mse_only):
    import torch
    wl = synth.workload(name)
    spec = synth.draw_quantizer(wl, kind)
    x = synth.draw_kv_slab(wl, kind, 1, 1, 0, n_vec).copy()
    x[n_vec // 2] = 0.0
    n_rows = 32 * ((3 * n_vec + 31) // 32 + 1)
    rows = np.random.default_rng(n_vec + 9).permutation(n_rows)[:n_vec]
    oq, dq = gc.quantizers(spec, mse_only=mse_only, norm_f16=True)
    fmt = getattr(tq, fmt_name)
    cache = tq.Cache.empty(dq, n_rows, fmt)
    assert cache.norms.dtype == torch.float16
    cache.norms.fill_(7.0)
    xt = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    tq.tq_quantize(dq, fmt, xt, cache, dst_rows=torch.from_numpy(rows.astype(np.int64)).cuda())
    torch.cuda.synchronize()
    got_all = gc.read_cache(cache, dq)
    qv = oracle.quantize(x.astype(np.float64), oq)
    print(gc.compare_records(x.astype(np.float64), oq, qv, gc.select_rows(got_all, rows)))
    untouched = np.setdiff1d(np.arange(n_rows), rows)
    for g in range(len(dq.mse_bits)):
        assert np.all(got_all[2][g][untouched] == 7.0) and np.all(got_all[3][g][untouched] == 7.0)
