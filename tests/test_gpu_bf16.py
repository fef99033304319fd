"""GPU parity of tq_attn_decode_bf16, the uncompressed baseline decode,
against the CPU oracle (through the C ABI).

The caches hold the synthetic bf16 tokens themselves, so the oracle's
attention over those exact values (float64) is the reference. Rows of the
cache past n_ctx are filled with NaN: the kernel must ignore them. Logits and
outputs must agree within 2e-3 normwise per (batch, head), as for the
compressed decode.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def tq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotation_amd as m
    m.lib()
    return m


def _close(got, ref, tol=TOL):
    err = np.max(np.abs(got - ref), axis=-1)
    scale = np.max(np.abs(ref), axis=-1)
    worst = float(np.max(err / np.maximum(scale, 1e-30)))
    return worst <= tol, worst


def _device_caches(wl, n_ctx, cap, pairs=None):
    """bf16 K [B*H*cap, d] (token-major) and V [B*H*cap/32, d, 32] (channel-major
    inside 32-row blocks) on the device, holding the synthetic tokens of the
    (b, h) pairs in `pairs` (all pairs when None) and NaN past n_ctx; other
    pairs hold seeded random values no expected value depends on. Returns
    (k, v, {(b, h): (K slab, V slab)})."""
    import torch
    B, H, d = wl.batch, wl.n_kv_heads, wl.d
    g = torch.Generator(device="cuda").manual_seed(11)
    k = torch.randn((B * H * cap, d), generator=g, device="cuda").to(torch.bfloat16)
    vt = torch.randn((B * H * cap, d), generator=g, device="cuda").to(torch.bfloat16)
    slabs = {}
    for b in range(B):
        for h in range(H):
            r0 = (b * H + h) * cap
            k[r0 + n_ctx:r0 + cap] = float("nan")
            vt[r0 + n_ctx:r0 + cap] = float("nan")
            if pairs is not None and (b, h) not in pairs:
                continue
            ks = synth.draw_kv_slab(wl, "K", b, h, 0, n_ctx)
            vs = synth.draw_kv_slab(wl, "V", b, h, 0, n_ctx)
            k[r0:r0 + n_ctx] = torch.from_numpy(ks).cuda().to(torch.bfloat16)
            vt[r0:r0 + n_ctx] = torch.from_numpy(vs).cuda().to(torch.bfloat16)
            slabs[(b, h)] = (ks.astype(np.float64), vs.astype(np.float64))
    v = vt.reshape(B * H * cap // 32, 32, d).transpose(1, 2).contiguous()
    return k, v, slabs


def _run(tq, wl, k, v, n_ctx, cap, q=None, n_split=0, want_logits=True, q_f32=False):
    import torch
    B = wl.batch
    if q is None:
        q = synth.draw_queries(wl)
    qt = torch.from_numpy(q).cuda()
    if not q_f32:
        qt = qt.to(torch.bfloat16)
    shape = tq.decode_shape(B, wl.n_q_heads, wl.n_kv_heads, n_ctx, cap, wl.scale, n_split)
    logits = torch.full((B, wl.n_q_heads, n_ctx), float("nan"), device="cuda") if want_logits else None
    out = torch.full((B, wl.n_q_heads, wl.d), float("nan"), device="cuda")
    tq.tq_attn_decode_bf16(shape, qt, k, v, out, logits=logits)
    torch.cuda.synchronize()
    return (None if logits is None else logits.cpu().numpy().astype(np.float64),
            out.cpu().numpy().astype(np.float64), q)


def _reference(wl, slabs, q, b, h):
    """Oracle logits [G, n_ctx] and outputs [G, d] of the query heads of kv head h."""
    G = wl.n_q_heads // wl.n_kv_heads
    ks, vs = slabs[(b, h)]
    return oracle.attention_decode(q[b, h * G:(h + 1) * G].astype(np.float64), ks[None], vs[None], wl.scale)


def _check(wl, slabs, q, lg, out):
    G = wl.n_q_heads // wl.n_kv_heads
    worst_l = worst_o = 0.0
    for (b, h) in slabs:
        rl, ro = _reference(wl, slabs, q, b, h)
        sl = slice(h * G, (h + 1) * G)
        if lg is not None:
            ok, w = _close(lg[b, sl], rl)
            assert ok, ("logits", b, h, w)
            worst_l = max(worst_l, w)
        ok, w = _close(out[b, sl], ro)
        assert ok, ("out", b, h, w)
        worst_o = max(worst_o, w)
    return worst_l, worst_o


CASES = [
    # name, overrides, n_ctx, cap
    ("llama8b_decode", dict(batch=2, n_q_heads=8, n_kv_heads=2), 1000, 1024),
    ("llama8b_decode", dict(batch=1, n_q_heads=8, n_kv_heads=1), 1, 32),
    ("llama8b_decode", dict(batch=1, n_q_heads=4, n_kv_heads=2), 33, 64),
    ("llama8b_decode", dict(batch=1, n_q_heads=16, n_kv_heads=2), 2048, 2048),
    ("llama8b_decode", dict(batch=2, n_q_heads=64, n_kv_heads=2), 777, 800),
    ("llama70b_long", dict(batch=1, n_q_heads=40, n_kv_heads=2), 300, 320),
    ("llama70b_long", dict(batch=2, n_q_heads=4, n_kv_heads=4), 5000, 5024),
]


@pytest.mark.parametrize("name,over,n_ctx,cap", CASES)
def test_bf16_decode_matches_oracle(tq, name, over, n_ctx, cap):
    wl = synth.workload(name, **over)
    k, v, slabs = _device_caches(wl, n_ctx, cap)
    lg, out, q = _run(tq, wl, k, v, n_ctx, cap)
    wl_, wo = _check(wl, slabs, q, lg, out)
    print(name, over, n_ctx, "logits", wl_, "out", wo)


def test_bf16_decode_f32_queries(tq):
    # fp32 queries (not rounded to bf16), 64 heads over one KV head (four
    # blocks of 16 heads), scale 1; the cache holds bf16-exact tokens
    wl = synth.workload("tiny", dtype="bf16")
    qf = synth.draw_queries(synth.workload("tiny"))
    k, v, slabs = _device_caches(wl, 4000, 4096)
    lg, out, _ = _run(tq, wl, k, v, 4000, 4096, q=qf, q_f32=True)
    _check(wl, slabs, qf, lg, out)


def test_bf16_split_count_does_not_change_result(tq):
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=8, n_kv_heads=2)
    k, v, slabs = _device_caches(wl, 3000, 3008)
    outs = []
    for ns in (1, 3, 7, 0, 16):
        _, out, q = _run(tq, wl, k, v, 3000, 3008, n_split=ns, want_logits=False)
        _check(wl, slabs, q, None, out)
        outs.append(out)
    # integer log2 softmax reference: a token's weight is the same whatever
    # the split (up to a power of two); only the order of fp32 sums changes
    for out in outs[1:]:
        assert _close(out, outs[0], tol=5e-5)[0]


def test_bf16_single_token_returns_its_value(tq):
    wl = synth.workload("llama8b_decode", batch=1, n_q_heads=4, n_kv_heads=1)
    k, v, slabs = _device_caches(wl, 1, 32)
    _, out, _ = _run(tq, wl, k, v, 1, 32, want_logits=False)
    ref = np.repeat(slabs[(0, 0)][1][:1], 4, axis=0)
    # the weight 2^(l - ceil l) enters the value product as bf16 hi + lo parts
    # (relative error below 2^-17)
    assert np.max(np.abs(out[0] - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_bf16_full_size_llama8b(tq):
    # the launch bench.py times: batch 1, 32 query heads over 8 KV heads,
    # 32768 tokens, default split count; every logit and output
    wl = synth.workload("llama8b_decode")
    n = wl.n_ctx
    k, v, slabs = _device_caches(wl, n, n)
    lg, out, q = _run(tq, wl, k, v, n, n)
    print("llama8b full size", _check(wl, slabs, q, lg, out))


def test_bf16_full_size_batch16_sampled(tq):
    # batch 16 x 8 KV heads x 32768 tokens (1 GiB each of bf16 K and V): sampled pairs
    wl = synth.workload("mixed_3p5")
    n = wl.n_ctx
    pairs = {(0, 0), (15, 7), (9, 3)}
    k, v, slabs = _device_caches(wl, n, n, pairs=pairs)
    lg, out, q = _run(tq, wl, k, v, n, n)
    print("batch16 sampled", _check(wl, slabs, q, lg, out))
