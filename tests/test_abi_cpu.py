"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every function include/turboquant.h declares; the C++ Lloyd-Max
codebook agrees with the independent numpy/scipy oracle; record sizes; the
sketch folding; and argument validation, which must reject bad calls before
any HIP call is made (the device pointers passed here are never touched)."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "turboquant.h")


@pytest.fixture(scope="module")
def tq():
    import kv_cache_vector_rotation_amd as m
    if not os.path.exists(m.LIB_PATH):
        from kv_cache_vector_rotation_amd import build
        build.build()
    m.lib()
    return m


def test_header_symbols_exported(tq):
    text = open(HEADER).read()
    declared = sorted(set(re.findall(r"^\s*(?:tq_status|int|const char\*)\s+(tq_\w+)\s*\(", text, re.M)))
    assert len(declared) == 16
    lib = C.CDLL(tq.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(tq.SYMBOLS) == declared
    version = int(re.search(r"#define TQ_ABI_VERSION (\d+)", text).group(1))
    assert tq.tq_abi_version() == version


@pytest.mark.parametrize("d", [3, 8, 64, 128, 200, 1024])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_codebook_matches_oracle(tq, d, m):
    c, t, mse = tq.tq_build_codebook(d, m)
    ref = oracle.lloyd_max(d, m)
    assert np.max(np.abs(c - ref.centroids)) <= 1e-10 / math.sqrt(d)
    assert np.max(np.abs(t - ref.boundaries)) <= 1e-10 / math.sqrt(d)
    assert abs(mse - ref.mse_per_coord) <= 1e-13
    assert np.array_equal(c, -c[::-1])
    assert np.array_equal(t, 0.5 * (c[:-1] + c[1:]))


def test_codebook_errors(tq):
    for d, m in [(2, 2), (128, 0), (128, 5), (-1, 1)]:
        with pytest.raises(tq.TQError) as e:
            tq.tq_build_codebook(d, m)
        assert e.value.status == tq.TQ_ERR_INVALID
    with pytest.raises(tq.TQError) as e:
        tq.tq_build_codebook(128, 3, max_iter=1)
    assert e.value.status == tq.TQ_ERR_NOCONVERGE
    lib = tq.lib()
    c = (C.c_double * 8)()
    assert lib.tq_build_codebook(128, 3, 0, 0.0, c, None, None) == tq.TQ_ERR_INVALID
    assert lib.tq_build_codebook(128, 3, 0, -1.0, c, c, None) == tq.TQ_ERR_INVALID


@pytest.mark.parametrize("dims,bits", [([128], [2]), ([128], [3]), ([64, 64], [3, 2]),
                                       ([64, 64], [2, 1]), ([200], [3]), ([40, 24], [4, 1])])
def test_record_layout(tq, dims, bits):
    info = tq.tq_record_layout(tq.make_layout(dims, bits))
    cw, sw, nf, bcw, bsw = oracle.record_words(dims, bits)
    assert (info.code_words, info.sign_words, info.norm_floats, info.block_code_words,
            info.block_sign_words) == (cw, sw, nf, bcw, bsw)
    assert info.record_bits == 8 * oracle.record_bytes(dims, bits)


def test_layout_validation(tq):
    bad = [([2], [2]), ([300], [2]), ([128], [0]), ([128], [5]), ([64, 2], [2, 2])]
    for dims, bits in bad:
        with pytest.raises(tq.TQError):
            tq.tq_record_layout(tq.make_layout(dims, bits))
    l = tq.make_layout([64, 64], [2, 2])
    l.d = 100
    with pytest.raises(tq.TQError):
        tq.tq_record_layout(l)


def test_fold_sketch(tq):
    rng = np.random.default_rng(1)
    rot = rng.standard_normal((48, 48)).astype(np.float32)
    sk = rng.standard_normal((48, 48)).astype(np.float32)
    got = tq.tq_fold_sketch(rot, sk)
    ref = (sk.astype(np.float64) @ rot.astype(np.float64).T).astype(np.float32)
    assert np.array_equal(got, ref)


# ---- validation of device entry points (nothing is dereferenced) ----
FAKE = 1 << 20  # a 16-byte aligned address that is never accessed


def _fake_quantizer(tq, dims=(128,), bits=(3,)):
    q = tq.tq_quantizer()
    q.layout = tq.make_layout(dims, bits)
    q.rot = q.sketch = q.sketch_rot = q.centroids = q.boundaries = FAKE
    return q


def _fake_cache(tq, n_rows):
    c = tq.tq_cache()
    c.codes = c.signs = c.norms = FAKE
    c.n_rows = n_rows
    return c


def test_quantize_validation(tq):
    lib = tq.lib()
    q = _fake_quantizer(tq)
    cache = _fake_cache(tq, 1024)
    rows = tq.tq_rows()
    rows.dst_rows, rows.seg_len, rows.seg_stride, rows.seg_offset = None, 1024, 1024, 0
    call = lambda **kw: lib.tq_quantize(C.byref(kw.get("q", q)), kw.get("fmt", 0), kw.get("x", FAKE),
                                        kw.get("dt", 0), kw.get("n", 100), kw.get("stride", 128),
                                        C.byref(kw.get("rows", rows)), C.byref(kw.get("cache", cache)),
                                        None)
    assert call(n=-1) == tq.TQ_ERR_INVALID
    assert call(fmt=7) == tq.TQ_ERR_INVALID
    assert call(dt=9) == tq.TQ_ERR_INVALID
    assert call(stride=127) == tq.TQ_ERR_INVALID
    assert call(n=1025) == tq.TQ_ERR_INVALID                 # rows beyond the cache
    assert call(x=FAKE + 2) == tq.TQ_ERR_INVALID             # misaligned input
    assert call(n=0) == tq.TQ_OK                              # no-op, nothing launched
    small = _fake_cache(tq, 1000)
    assert call(fmt=1, cache=small) == tq.TQ_ERR_INVALID      # block records need 32-row blocks
    overlap = tq.tq_rows()
    overlap.dst_rows, overlap.seg_len, overlap.seg_stride, overlap.seg_offset = None, 10, 5, 0
    assert call(rows=overlap) == tq.TQ_ERR_INVALID
    bad_q = _fake_quantizer(tq)
    bad_q.rot = None
    assert call(q=bad_q) == tq.TQ_ERR_INVALID
    mis = _fake_quantizer(tq)
    mis.centroids = FAKE + 4
    assert call(q=mis) == tq.TQ_ERR_INVALID
    split = _fake_quantizer(tq, dims=(72, 56), bits=(3, 2))
    assert call(q=split) == tq.TQ_ERR_UNSUPPORTED            # group edge not a multiple of 16
    odd = _fake_quantizer(tq, dims=(100,), bits=(3,))
    assert call(q=odd, fmt=1, stride=100) == tq.TQ_ERR_UNSUPPORTED


def test_decode_validation(tq):
    lib = tq.lib()
    kq, vq = _fake_quantizer(tq), _fake_quantizer(tq)
    kc = _fake_cache(tq, 2 * 8 * 1024)
    vc = _fake_cache(tq, 2 * 8 * 1024)

    def call(shape, **kw):
        return lib.tq_attn_decode(C.byref(kw.get("kq", kq)), kw.get("vq", C.byref(vq)), C.byref(shape),
                                  kw.get("q", FAKE), kw.get("dt", 1), C.byref(kw.get("kc", kc)),
                                  C.byref(kw.get("vc", vc)), kw.get("logits", None), kw.get("out", FAKE),
                                  kw.get("ws", FAKE), kw.get("wsb", 1 << 40), None)

    good = tq.decode_shape(2, 32, 8, 1000, 1024, 0.088)
    for bad in [tq.decode_shape(2, 30, 8, 1000, 1024, 0.1), tq.decode_shape(2, 32, 8, 0, 1024, 0.1),
                tq.decode_shape(2, 32, 8, 1025, 1024, 0.1), tq.decode_shape(2, 32, 8, 1000, 1000, 0.1),
                tq.decode_shape(0, 32, 8, 1000, 1024, 0.1), tq.decode_shape(2, 32, 8, 1000, 1024, math.inf),
                tq.decode_shape(2, 32, 8, 1000, 1024, 0.1, n_split=-1)]:
        assert call(bad) == tq.TQ_ERR_INVALID
    assert call(good, dt=5) == tq.TQ_ERR_INVALID
    assert call(good, out=None) == tq.TQ_ERR_INVALID                       # V given, no output
    assert call(good, vq=None, out=FAKE, logits=FAKE) == tq.TQ_ERR_INVALID  # logits-only with out
    assert call(good, vq=None, out=None) == tq.TQ_ERR_INVALID              # logits-only without logits
    assert call(good, kc=_fake_cache(tq, 100)) == tq.TQ_ERR_INVALID        # cache too small
    assert call(good, q=FAKE + 8) == tq.TQ_ERR_INVALID
    assert call(good, wsb=10) == tq.TQ_ERR_WORKSPACE
    other = _fake_quantizer(tq, bits=(2,))
    assert call(good, vq=C.byref(other)) == tq.TQ_ERR_UNSUPPORTED          # K and V layouts differ
    d64 = _fake_quantizer(tq, dims=(64,), bits=(3,))
    assert call(good, kq=d64, vq=C.byref(_fake_quantizer(tq, dims=(64,), bits=(3,)))) == tq.TQ_ERR_UNSUPPORTED
    # the workspace query agrees with what the call requires
    need = C.c_size_t()
    assert lib.tq_attn_decode_workspace_bytes(C.byref(kq), C.byref(vq), C.byref(good), C.byref(need)) == 0
    assert call(good, wsb=need.value - 1) == tq.TQ_ERR_WORKSPACE


def test_decode_scratch_validation(tq):
    # the static-workspace decode validates like tq_attn_decode and rejects
    # shapes whose workspace exceeds its 16 MiB array, before any HIP call
    lib = tq.lib()
    kq, vq = _fake_quantizer(tq), _fake_quantizer(tq)
    kc = _fake_cache(tq, 2 * 8 * 1024)
    vc = _fake_cache(tq, 2 * 8 * 1024)

    def call(shape, **kw):
        return lib.tq_attn_decode_scratch(C.byref(kq), kw.get("vq", C.byref(vq)), C.byref(shape),
                                          kw.get("q", FAKE), kw.get("dt", 1), C.byref(kw.get("kc", kc)),
                                          C.byref(vc), kw.get("logits", None), kw.get("out", FAKE), None)

    good = tq.decode_shape(2, 32, 8, 1000, 1024, 0.088)
    assert call(tq.decode_shape(2, 30, 8, 1000, 1024, 0.1)) == tq.TQ_ERR_INVALID
    assert call(good, dt=5) == tq.TQ_ERR_INVALID
    assert call(good, out=None) == tq.TQ_ERR_INVALID
    assert call(good, q=FAKE + 8) == tq.TQ_ERR_INVALID
    assert call(good, kc=_fake_cache(tq, 100)) == tq.TQ_ERR_INVALID
    big = tq.decode_shape(2, 32, 8, 131072, 131072, 0.088, n_split=1024)
    need = C.c_size_t()
    assert lib.tq_attn_decode_workspace_bytes(C.byref(kq), C.byref(vq), C.byref(big), C.byref(need)) == 0
    assert need.value > 16 << 20
    assert call(big) == tq.TQ_ERR_WORKSPACE


def test_phase_mask_validation(tq):
    lib = tq.lib()
    kq, vq = _fake_quantizer(tq), _fake_quantizer(tq)
    kc, vc = _fake_cache(tq, 8 * 1024), _fake_cache(tq, 8 * 1024)
    shape = tq.decode_shape(1, 32, 8, 1000, 1024, 0.088)
    for mask in (0, 8, 15):
        assert lib.tq_attn_decode_phases(mask, C.byref(kq), C.byref(vq), C.byref(shape), FAKE, 1,
                                         C.byref(kc), C.byref(vc), None, FAKE, FAKE, 10, None) == tq.TQ_ERR_INVALID
    # a valid mask reaches the workspace check
    assert lib.tq_attn_decode_phases(2, C.byref(kq), C.byref(vq), C.byref(shape), FAKE, 1, C.byref(kc),
                                     C.byref(vc), None, FAKE, FAKE, 10, None) == tq.TQ_ERR_WORKSPACE


def test_decode_append_validation(tq):
    # every error is found before any launch (no GPU here)
    lib = tq.lib()
    kq, vq = _fake_quantizer(tq), _fake_quantizer(tq)
    kc, vc = _fake_cache(tq, 8 * 1024), _fake_cache(tq, 8 * 1024)
    shape = tq.decode_shape(1, 32, 8, 1000, 1024, 0.088)
    need = C.c_size_t()
    assert lib.tq_attn_decode_workspace_bytes(C.byref(kq), C.byref(vq), C.byref(shape), C.byref(need)) == 0

    def app(n_vec=8, stride=128, dtype=1, x=FAKE, seg=(1, 1024, 999)):
        a = tq.tq_append()
        a.x, a.dtype, a.n_vec, a.x_row_stride = x, dtype, n_vec, stride
        a.rows.dst_rows = None
        a.rows.seg_len, a.rows.seg_stride, a.rows.seg_offset = seg
        return a

    def call(k_new, v_new, vq_=C.byref(vq), wsb=need.value):
        return lib.tq_attn_decode_append(C.byref(kq), vq_, C.byref(shape),
                                         C.byref(k_new) if k_new is not None else None,
                                         C.byref(v_new) if v_new is not None else None, FAKE, 1,
                                         C.byref(kc), C.byref(vc), None, FAKE, FAKE, wsb, None)

    assert call(app(), app(), wsb=need.value - 1) == tq.TQ_ERR_WORKSPACE  # decode checks first
    assert call(app(dtype=7), app()) == tq.TQ_ERR_INVALID                  # bad K dtype
    assert call(app(), app(stride=64)) == tq.TQ_ERR_INVALID                # V row stride < d
    assert call(app(seg=(1, 1024, 1024)), app()) == tq.TQ_ERR_INVALID      # K rows past the cache
    assert call(app(n_vec=-1), None) == tq.TQ_ERR_INVALID
    assert lib.tq_attn_decode_append(C.byref(kq), None, C.byref(shape), None, C.byref(app()), FAKE, 1,
                                     C.byref(kc), None, FAKE, None, FAKE, need.value, None) == tq.TQ_ERR_INVALID


def test_bf16_baseline_validation(tq):
    # the uncompressed baseline: sizing and every argument error before any launch
    lib = tq.lib()
    shape = tq.decode_shape(2, 32, 8, 1000, 1024, 0.088)
    need = C.c_size_t()
    assert lib.tq_attn_decode_bf16_workspace_bytes(C.byref(shape), 128, C.byref(need)) == 0
    # 2 * 32 heads x n_split x (2 + 128) floats, n_split for about 512 workgroups
    n_split = min(512 // 16, (32 + 3) // 4)
    assert need.value == 2 * 32 * n_split * 130 * 4
    assert lib.tq_attn_decode_bf16_workspace_bytes(C.byref(shape), 64, C.byref(need)) == tq.TQ_ERR_UNSUPPORTED

    def call(shape=shape, d=128, q=FAKE, dt=1, k=FAKE, v=FAKE, out=FAKE, ws=FAKE, wsb=need.value):
        return lib.tq_attn_decode_bf16(C.byref(shape), d, q, dt, k, v, None, out, ws, wsb, None)

    assert call(wsb=need.value - 1) == tq.TQ_ERR_WORKSPACE
    assert call(dt=7) == tq.TQ_ERR_INVALID
    assert call(out=None) == tq.TQ_ERR_INVALID
    assert call(k=FAKE + 2) == tq.TQ_ERR_INVALID  # misaligned
    assert call(d=64) == tq.TQ_ERR_UNSUPPORTED
    assert call(shape=tq.decode_shape(2, 30, 8, 1000, 1024, 0.088)) == tq.TQ_ERR_INVALID  # heads not a multiple
    assert call(shape=tq.decode_shape(2, 32, 8, 1000, 1000, 0.088)) == tq.TQ_ERR_INVALID  # capacity % 32


def test_search_validation(tq):
    # nearest-neighbour search: sizing and argument errors before any launch
    lib = tq.lib()
    q = _fake_quantizer(tq, dims=(200,), bits=(3,))
    db = _fake_cache(tq, 1000)
    need = C.c_size_t()
    assert lib.tq_search_workspace_bytes(C.byref(q), 1000, 50, 10, C.byref(need)) == 0
    # prepared queries (50 x 4 x 200 fp16: the rotated and the sketched query,
    # each as a high part and a scaled low part; rounded up to 256 B), the
    # codebook scale (256 B) and two [50][slices][10] lists; 63 tiles of 16
    # rows give 16 slices of 4 tiles
    qprep = (50 * 4 * 200 * 2 + 255) // 256 * 256
    assert need.value == qprep + 256 + 2 * 50 * 16 * 10 * 4
    for args in ((0, 50, 10), (1000, 0, 10), (1000, 50, 0), (1000, 50, 11)):
        assert lib.tq_search_workspace_bytes(C.byref(q), *args, C.byref(need)) == tq.TQ_ERR_INVALID
    assert lib.tq_search_workspace_bytes(C.byref(q), 1000, 50, 10, C.byref(need)) == 0

    def call(qz=q, db=db, n_db=1000, x=FAKE, dt=0, n_q=50, k=10, oi=FAKE, os_=FAKE, ws=FAKE, wsb=need.value):
        return lib.tq_search(C.byref(qz), C.byref(db), n_db, x, dt, n_q, k, oi, os_, ws, wsb, None)

    assert call(wsb=need.value - 1) == tq.TQ_ERR_WORKSPACE
    assert call(dt=5) == tq.TQ_ERR_INVALID
    assert call(k=11) == tq.TQ_ERR_INVALID
    assert call(x=None) == tq.TQ_ERR_INVALID
    assert call(oi=FAKE + 4) == tq.TQ_ERR_INVALID  # misaligned int64 output
    assert call(n_db=1001) == tq.TQ_ERR_INVALID  # more rows than the cache holds
    two = _fake_quantizer(tq, dims=(64, 64), bits=(3, 2))
    assert call(qz=two) == tq.TQ_ERR_UNSUPPORTED
    four = _fake_quantizer(tq, dims=(128,), bits=(4,))
    n4 = C.c_size_t()
    assert lib.tq_search_workspace_bytes(C.byref(four), 1000, 50, 10, C.byref(n4)) == 0
    assert call(qz=four, wsb=n4.value) == tq.TQ_ERR_UNSUPPORTED
    odd = _fake_quantizer(tq, dims=(96,), bits=(3,))
    assert call(qz=odd) == tq.TQ_ERR_UNSUPPORTED


def test_query_token_chunks_validation(tq):
    # n_q_tokens = T: the workspace holds T prepared queries and partials per
    # head; T past n_ctx is rejected; the bf16 baseline takes T = 1 only
    lib = tq.lib()
    q = _fake_quantizer(tq)
    need1, needT = C.c_size_t(), C.c_size_t()
    s1 = tq.decode_shape(1, 8, 2, 1000, 1024, 0.088, n_split=4)
    sT = tq.decode_shape(1, 8, 2, 1000, 1024, 0.088, n_split=4, n_q_tokens=16)
    assert lib.tq_attn_decode_workspace_bytes(C.byref(q), C.byref(q), C.byref(s1), C.byref(need1)) == 0
    assert lib.tq_attn_decode_workspace_bytes(C.byref(q), C.byref(q), C.byref(sT), C.byref(needT)) == 0
    per_head = lambda heads: (heads * 4 * 128 * 2 + 255) // 256 * 256 + 256 + (heads * 4 * 258 * 4 + 255) // 256 * 256
    assert need1.value == per_head(8) and needT.value == per_head(8 * 16)
    bad = tq.decode_shape(1, 8, 2, 10, 32, 0.088, n_q_tokens=11)
    assert lib.tq_attn_decode_workspace_bytes(C.byref(q), C.byref(q), C.byref(bad), C.byref(needT)) == \
        tq.TQ_ERR_INVALID
    nb = C.c_size_t()
    assert lib.tq_attn_decode_bf16_workspace_bytes(C.byref(sT), 128, C.byref(nb)) == tq.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("dims,bits", [([128], [3]), ([64, 64], [3, 2]), ([200], [4])])
def test_mse_only_record_layout(tq, dims, bits):
    # stage-one records: no sign words, m_g bits per channel plus the norms
    info = tq.tq_record_layout(tq.make_layout(dims, bits, mse_only=True))
    assert (info.code_words, info.sign_words, info.norm_floats, info.block_code_words,
            info.block_sign_words) == oracle.record_words(dims, bits, mse_only=True)
    assert info.record_bits == 8 * oracle.record_bytes(dims, bits, mse_only=True)
    l = tq.make_layout(dims, bits)
    l.mse_only = 2
    with pytest.raises(tq.TQError):
        tq.tq_record_layout(l)


def test_mse_only_decode_and_search_validation(tq):
    # MSE-only V is decoded (its sign pointer may be NULL); MSE-only K and an
    # MSE-only search database are refused
    lib = tq.lib()
    kq = _fake_quantizer(tq)
    vq_m = _fake_quantizer(tq)
    vq_m.layout = tq.make_layout((128,), (3,), mse_only=True)
    kc = _fake_cache(tq, 2 * 8 * 1024)
    vc = _fake_cache(tq, 2 * 8 * 1024)
    vc.signs = None
    shape = tq.decode_shape(2, 32, 8, 1000, 1024, 0.088)
    need = C.c_size_t()
    assert lib.tq_attn_decode_workspace_bytes(C.byref(kq), C.byref(vq_m), C.byref(shape), C.byref(need)) == 0

    def call(kq=kq, vq=vq_m, vc=vc, wsb=need.value):
        # a workspace one byte short: validation passes up to the size check
        return lib.tq_attn_decode(C.byref(kq), C.byref(vq), C.byref(shape), FAKE, 1, C.byref(kc), C.byref(vc),
                                  None, FAKE, FAKE, wsb, None)

    assert call(wsb=need.value - 1) == tq.TQ_ERR_WORKSPACE        # V without signs accepted
    full_v = _fake_quantizer(tq)
    assert call(vq=full_v, wsb=need.value - 1) == tq.TQ_ERR_INVALID   # its signs are required
    assert call(kq=vq_m, vq=full_v) == tq.TQ_ERR_UNSUPPORTED         # MSE-only K
    q = _fake_quantizer(tq, dims=(200,), bits=(3,))
    q.layout = tq.make_layout((200,), (3,), mse_only=True)
    db = _fake_cache(tq, 1000)
    assert lib.tq_search_workspace_bytes(C.byref(q), 1000, 50, 10, C.byref(need)) == 0
    assert lib.tq_search(C.byref(q), C.byref(db), 1000, FAKE, 0, 50, 10, FAKE, FAKE, FAKE, need.value,
                         None) == tq.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("mse_only", [False, True])
def test_norm_f16_record_layout(tq, mse_only):
    info = tq.tq_record_layout(tq.make_layout([64, 64], [3, 2], mse_only=mse_only, norm_f16=True))
    assert info.norm_floats == 4
    assert info.record_bits == 8 * oracle.record_bytes([64, 64], [3, 2], mse_only=mse_only, norm_f16=True)
    l = tq.make_layout([128], [3])
    l.norm_f16 = 3
    with pytest.raises(tq.TQError):
        tq.tq_record_layout(l)
