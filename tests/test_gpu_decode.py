"""GPU parity of tq_attn_decode against the CPU oracle (through the C ABI).

The compressed caches are written by the oracle (its own codes, signs and
norms, packed by its own packers) and uploaded, so the device and the oracle
decode the identical cache. Logits and outputs must agree within 2e-3
normwise per (batch, head): max |got - ref| <= 2e-3 max |ref|.
"""
import math

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


def _oracle_side(wl, n_ctx, cap, with_v=True, v_mse=False, k_f16=False, v_f16=False):
    """Quantize the K (and V) streams with the oracle, return oracle quantizers,
    specs, per-(b,h) dequantized caches and packed arrays (v_mse: MSE-only V
    records; k_f16, v_f16: fp16 norms)."""
    ks, vs = synth.draw_quantizer(wl, "K"), synth.draw_quantizer(wl, "V")
    okq = oracle.Quantizer.from_spec(ks, norm_f16=k_f16)
    ovq = oracle.Quantizer.from_spec(vs, mse_only=v_mse, norm_f16=v_f16)
    B, H = wl.batch, wl.n_kv_heads
    dims = [g.dim for g in ks.groups]
    bits = [g.mse_bits for g in ks.groups]
    kx = np.concatenate([synth.draw_kv_slab(wl, "K", b, h, 0, n_ctx) for b in range(B) for h in range(H)])
    qk = oracle.quantize(kx, okq)
    k_t = oracle.dequantize(qk.idx, qk.bits, qk.norm, qk.gamma, okq).reshape(B, H, n_ctx, wl.d)
    rows = np.concatenate([(b * H + h) * cap + np.arange(n_ctx) for b in range(B) for h in range(H)])
    karr = gc.oracle_cache_arrays(qk, dims, bits, 0, B * H * cap, rows, norm_f16=k_f16)
    out = dict(ks=ks, vs=vs, k_t=k_t, karr=karr, dims=dims, bits=bits, v_mse=v_mse, k_f16=k_f16, v_f16=v_f16)
    if with_v:
        # block records need whole blocks: quantize up to the block boundary
        nb = ((n_ctx + 31) // 32) * 32
        vx = np.concatenate([synth.draw_kv_slab(wl, "V", b, h, 0, nb) for b in range(B) for h in range(H)])
        qvv = oracle.quantize(vx, ovq)
        v_full = oracle.dequantize(qvv.idx, qvv.bits, qvv.norm, qvv.gamma, ovq).reshape(B, H, nb, wl.d)
        vrows = np.concatenate([(b * H + h) * cap + np.arange(nb) for b in range(B) for h in range(H)])
        out["varr"] = gc.oracle_cache_arrays(qvv, dims, bits, 1, B * H * cap, vrows, v_mse, v_f16)
        out["v_t"] = v_full[:, :, :n_ctx]
    return out


def _device_decode(tq, wl, o, n_ctx, cap, with_v=True, want_logits=True, n_split=0, q=None):
    import torch
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm,
                                 norm_f16=o["k_f16"])
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm,
                                 mse_only=o["v_mse"], norm_f16=o["v_f16"])
    B, H = wl.batch, wl.n_kv_heads
    kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, B * H * cap, o["karr"])
    vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, B * H * cap, o["varr"]) if with_v else None
    if q is None:
        q = synth.draw_queries(wl)
    qt = torch.from_numpy(q).cuda()
    if wl.dtype == "bf16":
        qt = qt.to(torch.bfloat16)
    shape = tq.decode_shape(B, wl.n_q_heads, H, n_ctx, cap, wl.scale, n_split)
    logits = torch.full((B, wl.n_q_heads, n_ctx), float("nan"), device="cuda") if want_logits else None
    out = torch.full((B, wl.n_q_heads, wl.d), float("nan"), device="cuda") if with_v else None
    tq.tq_attn_decode(kq, vq if with_v else None, shape, qt, kc, vc, logits=logits, out=out)
    torch.cuda.synchronize()
    return (None if logits is None else logits.cpu().numpy().astype(np.float64),
            None if out is None else out.cpu().numpy().astype(np.float64), q)


def _reference(wl, o, q, with_v=True):
    B = wl.batch
    lg, ot = [], []
    for b in range(B):
        l, out = oracle.attention_decode(q[b].astype(np.float64), o["k_t"][b],
                                         o["v_t"][b] if with_v else None, wl.scale)
        lg.append(l)
        ot.append(out)
    return np.stack(lg), (np.stack(ot) if with_v else None)


def test_tiny_logits_only(tq):
    # 64 fp32 queries x 4096 fp32 keys, 3 bits, raw inner products (scale 1)
    wl = synth.workload("tiny")
    o = _oracle_side(wl, 4096, 4096, with_v=False)
    got, _, q = _device_decode(tq, wl, o, 4096, 4096, with_v=False)
    ref, _ = _reference(wl, o, q, with_v=False)
    ok, worst = gc.normwise_close(got, ref)
    print("tiny logits worst", worst)
    assert ok, worst


CASES = [
    # name, overrides, n_ctx, cap
    ("llama8b_decode", dict(batch=2, n_q_heads=8, n_kv_heads=2), 1000, 1024),
    ("llama8b_decode", dict(batch=1, n_q_heads=8, n_kv_heads=1), 1, 32),
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=2), 33, 64),
    ("llama8b_decode", dict(batch=1, n_q_heads=16, n_kv_heads=2), 2048, 2048),
    ("llama70b_long", dict(batch=2, n_q_heads=16, n_kv_heads=2), 1500, 1536),
    ("llama70b_long", dict(batch=1, n_q_heads=40, n_kv_heads=2), 300, 320),
    ("mixed_3p5", dict(batch=2, n_q_heads=8, n_kv_heads=2), 777, 800),
    ("mixed_2p5", dict(batch=2, n_q_heads=8, n_kv_heads=2), 777, 800),
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=1, groups=((128, 1),)), 500, 512),
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=1, groups=((128, 4),)), 500, 512),
]


@pytest.mark.parametrize("name,over,n_ctx,cap", CASES)
def test_decode_matches_oracle(tq, name, over, n_ctx, cap):
    wl = synth.workload(name, **over)
    o = _oracle_side(wl, n_ctx, cap)
    lg, out, q = _device_decode(tq, wl, o, n_ctx, cap)
    rl, ro = _reference(wl, o, q)
    ok_l, wl_ = gc.normwise_close(lg, rl)
    ok_o, wo = gc.normwise_close(out, ro)
    print(name, over, n_ctx, "logits", wl_, "out", wo)
    assert ok_l and ok_o, (wl_, wo)


def test_split_count_does_not_change_result(tq):
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=8, n_kv_heads=2)
    o = _oracle_side(wl, 3000, 3008)
    outs = []
    for ns in (1, 3, 7, 0, 16):
        _, out, q = _device_decode(tq, wl, o, 3000, 3008, want_logits=False, n_split=ns)
        outs.append(out)
    _, ro = _reference(wl, o, q)
    for out in outs:
        ok, err = gc.normwise_close(out, ro)
        print("  vs oracle", err, flush=True)
        assert ok, err
    # the softmax reference is an integer in the log2 domain and the softmax
    # argument sits on a fixed fp32 grid, so a token's fp16 weight is the same
    # whatever the split (up to a power of two); only the order of the fp32
    # sums changes (observed ~3e-7)
    for out in outs[1:]:
        ok, err = gc.normwise_close(out, outs[0], tol=5e-6)
        print("  vs one split", err, flush=True)
        assert ok, err


def test_gqa_equals_repeated_heads(tq):
    # G query heads sharing one KV head give the same outputs as the same
    # queries each against its own copy of that KV head
    import torch
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=4, n_kv_heads=1)
    o = _oracle_side(wl, 200, 224)
    _, out_gqa, q = _device_decode(tq, wl, o, 200, 224, want_logits=False)
    wl4 = synth.workload("llama8b_decode", batch=1, n_q_heads=4, n_kv_heads=4)
    o4 = dict(o)
    kc, ks_, kn = o["karr"]
    vc, vs_, vn = o["varr"]
    o4["karr"] = (np.tile(kc, 4), np.tile(ks_, 4), np.tile(kn, 4))
    o4["varr"] = (np.tile(vc, 4), np.tile(vs_, 4), np.tile(vn, 4))
    _, out_mha, _ = _device_decode(tq, wl4, o4, 200, 224, want_logits=False, q=q)
    assert np.max(np.abs(out_gqa - out_mha)) <= 1e-5 * np.max(np.abs(out_gqa))


def test_single_token_returns_its_value(tq):
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=4, n_kv_heads=1)
    o = _oracle_side(wl, 1, 32)
    _, out, _ = _device_decode(tq, wl, o, 1, 32, want_logits=False)
    ref = np.repeat(o["v_t"][0, :, 0], 4, axis=0)
    assert gc.normwise_close(out[0], ref)[0]


@pytest.mark.parametrize("n_ctx,cap,n_new", [(1000, 1024, 1), (64, 64, 1), (700, 768, 40), (1500, 1536, 300)])
def test_append_step_equals_separate_calls(tq, n_ctx, cap, n_new):
    # one launch for the K/V appends and the query preparation, then the
    # decode: the same caches and the same results, bit for bit, as
    # tq_quantize (K), tq_quantize (V) and tq_attn_decode in a row; one new
    # token per head, and 40 and 300 (several tiles, ragged blocks). Two
    # steps in a row on one workspace, with different tokens.
    import torch
    wl = synth.workload("llama8b_decode", batch=2, n_q_heads=8, n_kv_heads=2)
    o = _oracle_side(wl, n_ctx, cap)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm)
    B, H = wl.batch, wl.n_kv_heads
    t0 = n_ctx - n_new  # the appended tokens [t0, n_ctx) of every (batch, kv head)
    kx = np.concatenate([synth.draw_kv_slab(wl, "K", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    vx = np.concatenate([synth.draw_kv_slab(wl, "V", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(B, wl.n_q_heads, H, n_ctx, cap, wl.scale)
    ws = torch.zeros(tq.tq_attn_decode_workspace_bytes(kq, vq, shape), dtype=torch.uint8, device="cuda")
    for sign in (1.0, -1.0):
        kx_t = torch.from_numpy(sign * kx).cuda().to(torch.bfloat16)
        vx_t = torch.from_numpy(sign * vx).cuda().to(torch.bfloat16)
        results = []
        for fused in (False, True):
            kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, B * H * cap, o["karr"])
            vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, B * H * cap, o["varr"])
            logits = torch.full((B, wl.n_q_heads, n_ctx), float("nan"), device="cuda")
            out = torch.full((B, wl.n_q_heads, wl.d), float("nan"), device="cuda")
            if fused:
                tq.tq_attn_decode_append(kq, vq, shape, q, kc, vc,
                                         k_new=tq.append_spec(kx_t, seg_len=n_new, seg_stride=cap, seg_offset=t0),
                                         v_new=tq.append_spec(vx_t, seg_len=n_new, seg_stride=cap, seg_offset=t0),
                                         logits=logits, out=out, workspace=ws)
            else:
                tq.tq_quantize(kq, tq.TQ_TOKEN_MAJOR, kx_t, kc, seg_len=n_new, seg_stride=cap, seg_offset=t0)
                tq.tq_quantize(vq, tq.TQ_BLOCK32, vx_t, vc, seg_len=n_new, seg_stride=cap, seg_offset=t0)
                tq.tq_attn_decode(kq, vq, shape, q, kc, vc, logits=logits, out=out)
            torch.cuda.synchronize()
            results.append([x.cpu().numpy() for x in (kc.codes, kc.signs, kc.norms, vc.codes, vc.signs,
                                                      vc.norms, logits, out)])
        for a, b in zip(*results):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # and the step (of the second, negated tokens) agrees with the oracle
    kt, vt = o["k_t"].copy(), o["v_t"].copy()
    okq, ovq = oracle.Quantizer.from_spec(o["ks"]), oracle.Quantizer.from_spec(o["vs"])
    for arr, x, qz in ((kt, kx, okq), (vt, vx, ovq)):
        # (the appended inputs went through bf16)
        xb = torch.from_numpy(-x).to(torch.bfloat16).to(torch.float64).numpy()
        qv = oracle.quantize(xb, qz)
        arr[:, :, t0:n_ctx] = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz).reshape(B, H, n_new, wl.d)
    q64 = synth.draw_queries(wl)
    for b in range(B):
        rl, ro = oracle.attention_decode(q64[b].astype(np.float64), kt[b], vt[b], wl.scale)
        assert gc.normwise_close(results[1][6][b].astype(np.float64), rl)[0]
        assert gc.normwise_close(results[1][7][b].astype(np.float64), ro)[0]


def test_append_step_in_a_captured_graph(tq):
    # the fused step captured in a graph replays to the eager results, every
    # time (eager work and synchronizations between the replays)
    import torch
    wl = synth.workload("llama8b_decode", batch=2, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap, n_new = 1000, 1024, 1
    o = _oracle_side(wl, n_ctx, cap)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm)
    B, H = wl.batch, wl.n_kv_heads
    t0 = n_ctx - n_new
    kx = np.concatenate([synth.draw_kv_slab(wl, "K", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    vx = np.concatenate([synth.draw_kv_slab(wl, "V", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    kx_t = torch.from_numpy(kx).cuda().to(torch.bfloat16)
    vx_t = torch.from_numpy(vx).cuda().to(torch.bfloat16)
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(B, wl.n_q_heads, H, n_ctx, cap, wl.scale)
    ws = torch.zeros(tq.tq_attn_decode_workspace_bytes(kq, vq, shape), dtype=torch.uint8, device="cuda")
    kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, B * H * cap, o["karr"])
    vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, B * H * cap, o["varr"])
    logits = torch.zeros((B, wl.n_q_heads, n_ctx), device="cuda")
    out = torch.zeros((B, wl.n_q_heads, wl.d), device="cuda")
    k_app = tq.append_spec(kx_t, seg_len=n_new, seg_stride=cap, seg_offset=t0)
    v_app = tq.append_spec(vx_t, seg_len=n_new, seg_stride=cap, seg_offset=t0)

    def step():
        tq.tq_attn_decode_append(kq, vq, shape, q, kc, vc, k_new=k_app, v_new=v_app, logits=logits, out=out,
                                 workspace=ws, stream=torch.cuda.current_stream())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (kc.codes, kc.signs, kc.norms, vc.codes, vc.signs, vc.norms, logits, out)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        logits.fill_(float("nan"))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (kc.codes, kc.signs, kc.norms, vc.codes, vc.signs, vc.norms, logits, out)
        for a, b in zip(ref, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


# A chunk of T query tokens attended causally (n_q_tokens = T): q and out
# are [batch, T, n_q_heads, d], logits [batch, n_q_heads, T, n_ctx].
CHUNK_CASES = [
    # name, overrides, n_ctx, cap, T
    ("llama8b_decode", dict(batch=2, n_q_heads=8, n_kv_heads=2), 1000, 1024, 16),
    ("llama8b_decode", dict(batch=1, n_q_heads=8, n_kv_heads=2), 300, 320, 3),
    ("llama8b_decode", dict(batch=2, n_q_heads=2, n_kv_heads=2), 500, 512, 2),   # 2 columns per KV head
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=1), 40, 64, 40),    # the whole context
    ("mixed_3p5", dict(batch=1, n_q_heads=8, n_kv_heads=2), 777, 800, 8),
    ("llama70b_long", dict(batch=1, n_q_heads=16, n_kv_heads=2), 2000, 2048, 33),
    # widths 1 and 4 bits per code, a ragged context, three column blocks
    ("llama8b_decode", dict(batch=1, n_q_heads=8, n_kv_heads=2, groups=((128, 1),)), 333, 352, 12),
    ("llama8b_decode", dict(batch=1, n_q_heads=8, n_kv_heads=2, groups=((128, 4),), n_outliers=0), 450, 480, 9),
]


def _chunk_queries(wl, T, seed=21):
    q = synth.standard_normal(synth.rng_for(wl.seed, seed, T), (wl.batch, T, wl.n_q_heads, wl.d))
    return synth.to_bf16_exact(q) if wl.dtype == "bf16" else q


@pytest.mark.parametrize("name,over,n_ctx,cap,T", CHUNK_CASES)
def test_causal_chunk_matches_oracle(tq, name, over, n_ctx, cap, T):
    import torch
    wl = synth.workload(name, **over)
    o = _oracle_side(wl, n_ctx, cap)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm)
    B, H = wl.batch, wl.n_kv_heads
    kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, B * H * cap, o["karr"])
    vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, B * H * cap, o["varr"])
    q = _chunk_queries(wl, T)
    qt = torch.from_numpy(q).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(B, wl.n_q_heads, H, n_ctx, cap, wl.scale, n_q_tokens=T)
    logits = torch.full((B, wl.n_q_heads, T, n_ctx), float("nan"), device="cuda")
    out = torch.full((B, T, wl.n_q_heads, wl.d), float("nan"), device="cuda")
    tq.tq_attn_decode(kq, vq, shape, qt, kc, vc, logits=logits, out=out)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy().astype(np.float64)
    ot = out.cpu().numpy().astype(np.float64)
    worst_l = worst_o = 0.0
    for b in range(B):
        rl, ro = oracle.attention_prefill(q[b].astype(np.float64), o["k_t"][b], o["v_t"][b], wl.scale)
        for i in range(T):
            lim = n_ctx - T + i + 1
            assert np.all(np.isneginf(lg[b, :, i, lim:]))
            ok, w = gc.normwise_close(lg[b, :, i, :lim], rl[:, i, :lim])
            assert ok, ("logits", b, i, w)
            worst_l = max(worst_l, w)
        ok, w = gc.normwise_close(ot[b], ro)
        assert ok, ("out", b, w)
        worst_o = max(worst_o, w)
    print(name, over, n_ctx, T, "logits", worst_l, "out", worst_o)


@pytest.mark.parametrize("v_mse,f16", [(True, False), (False, True), (True, True)])
def test_causal_chunk_record_variants(tq, v_mse, f16):
    # a chunk of 16 query tokens per head (64 columns per KV head: the
    # decode-once chunk kernel) over MSE-only V records and / or fp16 norms
    import torch
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap, T = 600, 640, 16
    o = _oracle_side(wl, n_ctx, cap, v_mse=v_mse, k_f16=f16, v_f16=f16)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm, norm_f16=f16)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm,
                                 mse_only=v_mse, norm_f16=f16)
    kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, 2 * cap, o["karr"])
    vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, 2 * cap, o["varr"])
    q = _chunk_queries(wl, T)
    qt = torch.from_numpy(q).cuda().to(torch.bfloat16)
    out = torch.full((1, T, 8, 128), float("nan"), device="cuda")
    tq.tq_attn_decode(kq, vq, tq.decode_shape(1, 8, 2, n_ctx, cap, wl.scale, n_q_tokens=T), qt, kc, vc, out=out)
    torch.cuda.synchronize()
    _, ro = oracle.attention_prefill(q[0].astype(np.float64), o["k_t"][0], o["v_t"][0], wl.scale)
    ok, w = gc.normwise_close(out[0].cpu().numpy().astype(np.float64), ro)
    print("chunk variants", v_mse, f16, "out", w)
    assert ok, w


def test_causal_chunk_split_count_and_logits_only(tq):
    # the chunk kernel's result does not depend on the split count beyond
    # fp32 summation order, and a logits-only call gives the same logits
    import torch
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap, T = 900, 928, 10
    o = _oracle_side(wl, n_ctx, cap)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm)
    kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, 2 * cap, o["karr"])
    vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, 2 * cap, o["varr"])
    qt = torch.from_numpy(_chunk_queries(wl, T)).cuda().to(torch.bfloat16)
    outs, lgs = [], []
    for n_split in (1, 5, 29):
        shape = tq.decode_shape(1, 8, 2, n_ctx, cap, wl.scale, n_q_tokens=T, n_split=n_split)
        lg = torch.full((1, 8, T, n_ctx), float("nan"), device="cuda")
        out = torch.empty((1, T, 8, 128), device="cuda")
        tq.tq_attn_decode(kq, vq, shape, qt, kc, vc, logits=lg, out=out)
        outs.append(out.cpu().numpy())
        lgs.append(lg.cpu().numpy())
    lg_only = torch.full((1, 8, T, n_ctx), float("nan"), device="cuda")
    tq.tq_attn_decode(kq, None, tq.decode_shape(1, 8, 2, n_ctx, cap, wl.scale, n_q_tokens=T), qt, kc, None,
                      logits=lg_only)
    torch.cuda.synchronize()
    for o2 in outs[1:]:
        assert np.max(np.abs(o2 - outs[0])) <= 5e-5 * np.max(np.abs(outs[0]))
    for l2 in lgs[1:]:
        assert np.array_equal(np.isnan(l2), np.isnan(lgs[0]))
        fin = np.isfinite(lgs[0])
        assert np.array_equal(l2[fin], lgs[0][fin])
    fin = np.isfinite(lgs[0])
    assert np.array_equal(lg_only.cpu().numpy()[fin], lgs[0][fin])


def test_causal_chunk_last_token_equals_decode(tq):
    # the chunk's last token attends to the whole context, like a decode step
    import torch
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap, T = 700, 704, 6
    o = _oracle_side(wl, n_ctx, cap)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm)
    kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, 2 * cap, o["karr"])
    vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, 2 * cap, o["varr"])
    q = torch.from_numpy(_chunk_queries(wl, T)).cuda().to(torch.bfloat16)
    out = torch.empty((1, T, 8, 128), device="cuda")
    tq.tq_attn_decode(kq, vq, tq.decode_shape(1, 8, 2, n_ctx, cap, wl.scale, n_q_tokens=T), q, kc, vc, out=out)
    out1 = torch.empty((1, 8, 128), device="cuda")
    tq.tq_attn_decode(kq, vq, tq.decode_shape(1, 8, 2, n_ctx, cap, wl.scale), q[:, -1].contiguous(), kc, vc,
                      out=out1)
    torch.cuda.synchronize()
    a, b1 = out[0, -1].cpu().numpy(), out1[0].cpu().numpy()
    # (the decode of a 4-head group carries each softmax weight as an fp16
    # part and its remainder; the chunk's 24 columns take the weights as
    # plain fp16, 2^-11 relative, so the two agree to that rounding)
    assert np.max(np.abs(a - b1)) <= 5e-4 * np.max(np.abs(b1))


def test_causal_chunk_append_step_equals_separate_calls(tq):
    # a prefill chunk through tq_attn_decode_append (append T tokens of K and
    # V, prepare T x 8 queries, attend causally) against tq_quantize twice and
    # tq_attn_decode: bit for bit
    import torch
    wl = synth.workload("llama8b_decode", batch=2, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap, T = 900, 1024, 24
    o = _oracle_side(wl, n_ctx, cap)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm)
    B, H = 2, 2
    t0 = n_ctx - T
    kx = np.concatenate([synth.draw_kv_slab(wl, "K", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    vx = np.concatenate([synth.draw_kv_slab(wl, "V", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    kx_t = torch.from_numpy(-kx).cuda().to(torch.bfloat16)
    vx_t = torch.from_numpy(-vx).cuda().to(torch.bfloat16)
    q = torch.from_numpy(_chunk_queries(wl, T)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(B, 8, H, n_ctx, cap, wl.scale, n_q_tokens=T)
    res = []
    for fused in (False, True):
        kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, B * H * cap, o["karr"])
        vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, B * H * cap, o["varr"])
        out = torch.full((B, T, 8, 128), float("nan"), device="cuda")
        if fused:
            tq.tq_attn_decode_append(kq, vq, shape, q, kc, vc,
                                     k_new=tq.append_spec(kx_t, seg_len=T, seg_stride=cap, seg_offset=t0),
                                     v_new=tq.append_spec(vx_t, seg_len=T, seg_stride=cap, seg_offset=t0),
                                     out=out)
        else:
            tq.tq_quantize(kq, tq.TQ_TOKEN_MAJOR, kx_t, kc, seg_len=T, seg_stride=cap, seg_offset=t0)
            tq.tq_quantize(vq, tq.TQ_BLOCK32, vx_t, vc, seg_len=T, seg_stride=cap, seg_offset=t0)
            tq.tq_attn_decode(kq, vq, shape, q, kc, vc, out=out)
        torch.cuda.synchronize()
        res.append((kc.codes.cpu(), vc.codes.cpu(), out.cpu()))
    for x, y in zip(res[0], res[1]):
        assert torch.equal(x, y)


def _paged_arrays(tq, o, B, H, cap, n_pblocks, table):
    """Scatter the contiguous oracle caches of _oracle_side into a paged
    layout: logical block j of batch b -> physical block table[b, j]."""
    import kv_cache_vector_rotation_amd as m
    cw, sw, nf, bcw, bsw = oracle.record_words(o["dims"], o["bits"], o["v_mse"])
    kc, ks_, kn = (a.reshape(B * H * cap, -1) for a in o["karr"])
    vc, vs_, vn = o["varr"]
    vc = vc.reshape(B * H * cap // 32, bcw)
    vs_ = vs_.reshape(B * H * cap // 32, bsw)
    vn = vn.reshape(B * H * cap, nf)
    rows = n_pblocks * H * 32
    pk = [np.zeros((rows, a.shape[1]), a.dtype) for a in (kc, ks_, kn)]
    pv = [np.zeros((n_pblocks * H, bcw), vc.dtype), np.zeros((n_pblocks * H, bsw), vs_.dtype),
          np.zeros((rows, nf), vn.dtype)]
    for b in range(B):
        for j in range(cap // 32):
            p = table[b, j]
            for h in range(H):
                src = (b * H + h) * cap + 32 * j
                dst = (p * H + h) * 32
                for a, t in zip((kc, ks_, kn), pk):
                    t[dst:dst + 32] = a[src:src + 32]
                pv[0][p * H + h] = vc[src // 32]
                pv[1][p * H + h] = vs_[src // 32]
                pv[2][dst:dst + 32] = vn[src:src + 32]
    return tuple(a.ravel() for a in pk), tuple(a.ravel() for a in pv), rows


def _paged_setup(tq, wl, n_ctx, cap, seed=3, v_mse=False, f16=False):
    B, H = wl.batch, wl.n_kv_heads
    o = _oracle_side(wl, n_ctx, cap, v_mse=v_mse, k_f16=f16, v_f16=f16)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm, norm_f16=f16)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm,
                                 mse_only=v_mse, norm_f16=f16)
    mb = cap // 32
    n_pblocks = B * mb + 5  # a few physical blocks that no sequence uses
    table = np.random.default_rng(seed).permutation(n_pblocks)[:B * mb].reshape(B, mb).astype(np.int32)
    parr_k, parr_v, rows = _paged_arrays(tq, o, B, H, cap, n_pblocks, table)
    kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, rows, parr_k)
    vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, rows, parr_v)
    return o, kq, vq, kc, vc, table


@pytest.mark.parametrize("v_mse,f16", [(False, False), (True, True)])
def test_paged_cache_equals_contiguous(tq, v_mse, f16):
    # the same records in a block-table layout give the same outputs and
    # logits, bit for bit, as the contiguous cache (also with MSE-only V
    # records and fp16 norms)
    import torch
    wl = synth.workload("llama8b_decode", batch=3, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap = 1000, 1024
    o, kq, vq, kc, vc, table = _paged_setup(tq, wl, n_ctx, cap, v_mse=v_mse, f16=f16)
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(3, 8, 2, n_ctx, cap, wl.scale)
    res = []
    for paged in (False, True):
        lg = torch.full((3, 8, n_ctx), float("nan"), device="cuda")
        out = torch.full((3, 8, 128), float("nan"), device="cuda")
        if paged:
            tq.tq_attn_decode_paged(kq, vq, shape, torch.from_numpy(table).cuda(), q, kc, vc, logits=lg, out=out)
        else:
            kc0 = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, 3 * 2 * cap, o["karr"])
            vc0 = gc.to_device_cache(vq, tq.TQ_BLOCK32, 3 * 2 * cap, o["varr"])
            tq.tq_attn_decode(kq, vq, shape, q, kc0, vc0, logits=lg, out=out)
        torch.cuda.synchronize()
        res.append((lg.cpu(), out.cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("T", [1, 5])
def test_paged_cache_per_sequence_lengths(tq, T):
    # sequences of 1000, 517 and 33 tokens in one call (and a causal chunk of
    # T tokens at the end of each), against the oracle on each sequence's
    # own prefix
    import torch
    wl = synth.workload("llama8b_decode", batch=3, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap = 1000, 1024
    lens = np.array([1000, 517, 33], np.int32)
    o, kq, vq, kc, vc, table = _paged_setup(tq, wl, n_ctx, cap, seed=5)
    q = _chunk_queries(wl, T)
    qt = torch.from_numpy(q).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(3, 8, 2, n_ctx, cap, wl.scale, n_q_tokens=T)
    lg = torch.full((3, 8, T, n_ctx), float("nan"), device="cuda")
    out = torch.full((3, T, 8, 128), float("nan"), device="cuda")
    tq.tq_attn_decode_paged(kq, vq, shape, torch.from_numpy(table).cuda(), qt, kc, vc,
                            seq_lens=torch.from_numpy(lens).cuda(), logits=lg, out=out)
    torch.cuda.synchronize()
    lgn, otn = lg.cpu().numpy().astype(np.float64), out.cpu().numpy().astype(np.float64)
    for b in range(3):
        n = int(lens[b])
        rl, ro = oracle.attention_prefill(q[b].astype(np.float64), o["k_t"][b][:, :n], o["v_t"][b][:, :n],
                                          wl.scale)
        assert gc.normwise_close(otn[b], ro)[0], b
        for i in range(T):
            lim = n - T + i + 1
            assert gc.normwise_close(lgn[b, :, i, :lim], rl[:, i, :lim])[0], (b, i)
        assert np.all(np.isnan(lgn[b, :, :, n:]))  # past the sequence: not written


def test_paged_sequence_shorter_than_chunk(tq):
    # a chunk of 5 query tokens over sequences of 3 and 40 tokens: in the
    # first sequence two query tokens see no key (zero output, -inf logits)
    import torch
    wl = synth.workload("llama8b_decode", batch=3, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap, T = 1000, 1024, 5
    lens = np.array([3, 40, 1000], np.int32)
    o, kq, vq, kc, vc, table = _paged_setup(tq, wl, n_ctx, cap, seed=9)
    q = _chunk_queries(wl, T)
    qt = torch.from_numpy(q).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(3, 8, 2, n_ctx, cap, wl.scale, n_q_tokens=T)
    lg = torch.full((3, 8, T, n_ctx), float("nan"), device="cuda")
    out = torch.full((3, T, 8, 128), float("nan"), device="cuda")
    print("paged chunk T=5 over sequences of 3, 40, 1000 tokens", flush=True)
    tq.tq_attn_decode_paged(kq, vq, shape, torch.from_numpy(table).cuda(), qt, kc, vc,
                            seq_lens=torch.from_numpy(lens).cuda(), logits=lg, out=out)
    torch.cuda.synchronize()
    lgn, otn = lg.cpu().numpy().astype(np.float64), out.cpu().numpy().astype(np.float64)
    for b in range(3):
        n = int(lens[b])
        rl, ro = oracle.attention_prefill(q[b].astype(np.float64), o["k_t"][b][:, :n], o["v_t"][b][:, :n],
                                          wl.scale)
        for i in range(T):
            lim = n - T + i + 1
            if lim <= 0:
                assert np.all(otn[b, i] == 0.0), (b, i)
                assert np.all(np.isneginf(lgn[b, :, i, :n])), (b, i)
            else:
                assert gc.normwise_close(otn[b, i], ro[i])[0], (b, i)
                assert gc.normwise_close(lgn[b, :, i, :lim], rl[:, i, :lim])[0], (b, i)


# MSE-only V records (codes and norms, no sign words; the values are
# dequantized as n Pi^T c[idx]) under two-stage K: the packed layout (at most
# 4 query heads per KV head), 16-head blocks, two groups, ragged lengths.
MSE_V_CASES = [
    ("llama8b_decode", dict(batch=2, n_q_heads=8, n_kv_heads=2), 1000, 1024),
    ("llama8b_decode", dict(batch=1, n_q_heads=16, n_kv_heads=2), 2048, 2048),
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=1), 33, 64),
    ("mixed_3p5", dict(batch=2, n_q_heads=8, n_kv_heads=2), 777, 800),
    ("mixed_2p5", dict(batch=1, n_q_heads=40, n_kv_heads=2), 300, 320),
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=1, groups=((128, 4),)), 500, 512),
]


@pytest.mark.parametrize("name,over,n_ctx,cap", MSE_V_CASES)
def test_mse_only_v_matches_oracle(tq, name, over, n_ctx, cap):
    wl = synth.workload(name, **over)
    o = _oracle_side(wl, n_ctx, cap, v_mse=True)
    lg, out, q = _device_decode(tq, wl, o, n_ctx, cap)
    rl, ro = _reference(wl, o, q)
    ok_l, wl_ = gc.normwise_close(lg, rl)
    ok_o, wo = gc.normwise_close(out, ro)
    print(name, over, n_ctx, "logits", wl_, "out", wo)
    assert ok_l and ok_o, (wl_, wo)


def test_mse_only_v_append_step(tq):
    # fused K/V append + decode with MSE-only V: the same cache and results,
    # bit for bit, as tq_quantize (K), tq_quantize (V) and tq_attn_decode
    import torch
    wl = synth.workload("llama8b_decode", batch=2, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap, n_new = 700, 768, 40
    o = _oracle_side(wl, n_ctx, cap, v_mse=True)
    kq = tq.Quantizer.from_parts(o["ks"].rotations, o["ks"].sketches, o["bits"], perm=o["ks"].perm)
    vq = tq.Quantizer.from_parts(o["vs"].rotations, o["vs"].sketches, o["bits"], perm=o["vs"].perm,
                                 mse_only=True)
    B, H = wl.batch, wl.n_kv_heads
    t0 = n_ctx - n_new
    kx = np.concatenate([synth.draw_kv_slab(wl, "K", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    vx = np.concatenate([synth.draw_kv_slab(wl, "V", b, h, t0, n_ctx) for b in range(B) for h in range(H)])
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(B, wl.n_q_heads, H, n_ctx, cap, wl.scale)
    kx_t = torch.from_numpy(-kx).cuda().to(torch.bfloat16)
    vx_t = torch.from_numpy(-vx).cuda().to(torch.bfloat16)
    results = []
    for fused in (False, True):
        kc = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, B * H * cap, o["karr"])
        vc = gc.to_device_cache(vq, tq.TQ_BLOCK32, B * H * cap, o["varr"])
        logits = torch.full((B, wl.n_q_heads, n_ctx), float("nan"), device="cuda")
        out = torch.full((B, wl.n_q_heads, wl.d), float("nan"), device="cuda")
        if fused:
            tq.tq_attn_decode_append(kq, vq, shape, q, kc, vc,
                                     k_new=tq.append_spec(kx_t, seg_len=n_new, seg_stride=cap, seg_offset=t0),
                                     v_new=tq.append_spec(vx_t, seg_len=n_new, seg_stride=cap, seg_offset=t0),
                                     logits=logits, out=out)
        else:
            tq.tq_quantize(kq, tq.TQ_TOKEN_MAJOR, kx_t, kc, seg_len=n_new, seg_stride=cap, seg_offset=t0)
            tq.tq_quantize(vq, tq.TQ_BLOCK32, vx_t, vc, seg_len=n_new, seg_stride=cap, seg_offset=t0)
            tq.tq_attn_decode(kq, vq, shape, q, kc, vc, logits=logits, out=out)
        torch.cuda.synchronize()
        results.append([x.cpu().numpy() for x in (kc.codes, kc.signs, kc.norms, vc.codes, vc.norms,
                                                  logits, out)])
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    kt, vt = o["k_t"].copy(), o["v_t"].copy()
    okq, ovq = oracle.Quantizer.from_spec(o["ks"]), oracle.Quantizer.from_spec(o["vs"], mse_only=True)
    for arr, x, qz in ((kt, kx, okq), (vt, vx, ovq)):
        xb = torch.from_numpy(-x).to(torch.bfloat16).to(torch.float64).numpy()
        qv = oracle.quantize(xb, qz)
        arr[:, :, t0:n_ctx] = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz).reshape(B, H, n_new, wl.d)
    q64 = synth.draw_queries(wl)
    for b in range(B):
        rl, ro = oracle.attention_decode(q64[b].astype(np.float64), kt[b], vt[b], wl.scale)
        assert gc.normwise_close(results[1][5][b].astype(np.float64), rl)[0]
        assert gc.normwise_close(results[1][6][b].astype(np.float64), ro)[0]


# fp16 norms in the K and/or V records (the oracle dequantizes with the same
# stored float16 values): packed and 16-head blocks, two groups, MSE-only V,
# logits only, ragged lengths.
F16_CASES = [
    # name, overrides, n_ctx, cap, k_f16, v_f16, v_mse, with_v
    ("llama8b_decode", dict(batch=2, n_q_heads=8, n_kv_heads=2), 1000, 1024, True, True, False, True),
    ("llama8b_decode", dict(batch=1, n_q_heads=16, n_kv_heads=2), 2048, 2048, True, False, False, True),
    ("mixed_3p5", dict(batch=2, n_q_heads=8, n_kv_heads=2), 777, 800, False, True, False, True),
    ("mixed_2p5", dict(batch=1, n_q_heads=40, n_kv_heads=2), 300, 320, True, True, True, True),
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=1), 33, 64, True, True, True, True),
    ("tiny", {}, 4096, 4096, True, False, False, False),
]


@pytest.mark.parametrize("name,over,n_ctx,cap,k_f16,v_f16,v_mse,with_v", F16_CASES)
def test_fp16_norms_match_oracle(tq, name, over, n_ctx, cap, k_f16, v_f16, v_mse, with_v):
    wl = synth.workload(name, **over)
    o = _oracle_side(wl, n_ctx, cap, with_v=with_v, v_mse=v_mse, k_f16=k_f16, v_f16=v_f16)
    lg, out, q = _device_decode(tq, wl, o, n_ctx, cap, with_v=with_v)
    rl, ro = _reference(wl, o, q, with_v=with_v)
    ok_l, wl_ = gc.normwise_close(lg, rl)
    ok_o, wo = gc.normwise_close(out, ro) if with_v else (True, 0.0)
    print(name, over, n_ctx, k_f16, v_f16, v_mse, "logits", wl_, "out", wo)
    assert ok_l and ok_o, (wl_, wo)


@pytest.mark.parametrize("v_mse", [False, True])
def test_fp16_norm_reads_equal_float32_layout(tq, v_mse):
    # records whose norms are float16 numbers, stored once as float16 and once
    # as float32: the decode must give identical logits and outputs (the
    # float16 read path only changes where the values come from)
    import torch
    wl = synth.workload("llama8b_decode", batch=2, n_q_heads=8, n_kv_heads=2)
    n_ctx, cap = 3000, 3008
    o = _oracle_side(wl, n_ctx, cap, v_mse=v_mse, k_f16=True, v_f16=True)
    q = synth.draw_queries(wl)
    res = []
    for f16 in (True, False):
        o2 = dict(o, k_f16=f16, v_f16=f16)
        if not f16:
            o2["karr"] = (o["karr"][0], o["karr"][1], o["karr"][2].astype(np.float32))
            o2["varr"] = (o["varr"][0], o["varr"][1], o["varr"][2].astype(np.float32))
        lg, out, _ = _device_decode(tq, wl, o2, n_ctx, cap, q=q)
        res.append((lg, out))
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])
