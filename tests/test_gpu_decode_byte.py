"""GPU parity of the byte-table split-K kernel (one quantizer group whose
code width m divides 8: m = 1, 2, 4) against the CPU oracle, through the C
ABI. Covers both column packings (at most 4 query heads per KV head in
quads; larger groups in blocks of 8 heads, the last block partial), m = 1,
2, 4, MSE-only V records, fp16 norms, a one-token context, logits only,
split-count invariance and the paged layout. The device decodes the
oracle's own records; logits and outputs must agree within 2e-3 normwise
per (batch, head)."""
import numpy as np
import pytest

import synth
from tests import gpu_common as gc
from tests.test_gpu_decode import _device_decode, _oracle_side, _paged_setup, _reference

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotation_amd as m
    m.lib()
    return m


BYTE_CASES = [
    # overrides of llama70b_long (3 bits unless groups say otherwise), n_ctx, cap, v_mse, f16, with_v
    (dict(batch=2, n_q_heads=8, n_kv_heads=2), 1000, 1024, False, False, True),        # quads, G = 4
    (dict(batch=1, n_q_heads=6, n_kv_heads=2), 300, 320, False, False, True),          # G = 3
    (dict(batch=1, n_q_heads=16, n_kv_heads=2), 4113, 4128, False, False, True),       # G = 8, ragged
    (dict(batch=1, n_q_heads=24, n_kv_heads=2), 700, 704, False, False, True),         # G = 12: 8 + 4
    (dict(batch=1, n_q_heads=2, n_kv_heads=2), 100, 128, False, False, True),          # G = 1
    (dict(batch=1, n_q_heads=16, n_kv_heads=2, groups=((128, 1),)), 1000, 1024, False, False, True),
    (dict(batch=1, n_q_heads=16, n_kv_heads=2, groups=((128, 4),)), 1000, 1024, False, False, True),
    (dict(batch=1, n_q_heads=8, n_kv_heads=2, groups=((128, 1),)), 777, 800, False, False, True),
    (dict(batch=1, n_q_heads=16, n_kv_heads=2), 1000, 1024, True, False, True),         # MSE-only V
    (dict(batch=1, n_q_heads=8, n_kv_heads=2), 1000, 1024, True, True, True),           # + fp16 norms
    (dict(batch=2, n_q_heads=16, n_kv_heads=2), 999, 1024, False, True, True),          # fp16 norms
    (dict(batch=1, n_q_heads=16, n_kv_heads=2), 1, 32, False, False, True),             # one token
    (dict(batch=1, n_q_heads=8, n_kv_heads=2), 500, 512, False, False, False),          # logits only
]


@pytest.mark.parametrize("over,n_ctx,cap,v_mse,f16,with_v", BYTE_CASES)
def test_byte_kernel_matches_oracle(tq, over, n_ctx, cap, v_mse, f16, with_v):
    wl = synth.workload("llama70b_long", **over)
    print("byte kernel case", over, n_ctx, v_mse, f16, with_v, flush=True)
    o = _oracle_side(wl, n_ctx, cap, with_v=with_v, v_mse=v_mse, k_f16=f16, v_f16=f16)
    lg, out, q = _device_decode(tq, wl, o, n_ctx, cap, with_v=with_v)
    rl, ro = _reference(wl, o, q, with_v=with_v)
    ok_l, el = gc.normwise_close(lg, rl)
    print("  logits", el, flush=True)
    assert ok_l, el
    if with_v:
        ok_o, eo = gc.normwise_close(out, ro)
        print("  out", eo, flush=True)
        assert ok_o, eo


def test_byte_kernel_split_count_invariance(tq):
    # the integer log2 softmax reference, with the softmax argument held on a
    # fixed fp32 grid (offset into [64, 128)), makes every split's weights the
    # same power-of-two multiples, so only the fp32 summation order changes
    # (observed ~4e-7; a weight whose fp16 rounding depended on the split
    # would move the output by up to 2^-11 of its share)
    wl = synth.workload("llama70b_long", batch=1, n_q_heads=16, n_kv_heads=2)
    o = _oracle_side(wl, 3000, 3008)
    outs = []
    for ns in (1, 3, 7, 0, 12):
        print("byte kernel n_split", ns, flush=True)
        _, out, q = _device_decode(tq, wl, o, 3000, 3008, want_logits=False, n_split=ns)
        outs.append(out)
    _, ro = _reference(wl, o, q)
    for out in outs:
        ok, err = gc.normwise_close(out, ro)
        print("  vs oracle", err, flush=True)
        assert ok, err
    for out in outs[1:]:
        ok, err = gc.normwise_close(out, outs[0], tol=5e-6)
        print("  vs one split", err, flush=True)
        assert ok, err


@pytest.mark.parametrize("G", [4, 8])
def test_byte_kernel_paged_equals_contiguous(tq, G):
    import torch
    wl = synth.workload("llama70b_long", batch=3, n_q_heads=2 * G, n_kv_heads=2)
    n_ctx, cap = 1000, 1024
    o, kq, vq, kc, vc, table = _paged_setup(tq, wl, n_ctx, cap)
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(3, 2 * G, 2, n_ctx, cap, wl.scale)
    res = []
    for paged in (False, True):
        print("byte kernel paged", paged, "G", G, flush=True)
        lg = torch.full((3, 2 * G, n_ctx), float("nan"), device="cuda")
        out = torch.full((3, 2 * G, 128), float("nan"), device="cuda")
        if paged:
            tq.tq_attn_decode_paged(kq, vq, shape, torch.from_numpy(table).cuda(), q, kc, vc, logits=lg, out=out)
        else:
            kc2 = gc.to_device_cache(kq, tq.TQ_TOKEN_MAJOR, 3 * 2 * cap, o["karr"])
            vc2 = gc.to_device_cache(vq, tq.TQ_BLOCK32, 3 * 2 * cap, o["varr"])
            tq.tq_attn_decode(kq, vq, shape, q, kc2, vc2, logits=lg, out=out)
        torch.cuda.synchronize()
        res.append((lg.cpu(), out.cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    _, ro = _reference(wl, o, synth.draw_queries(wl))
    assert gc.normwise_close(res[0][1].numpy().astype(np.float64), ro)[0]


@pytest.mark.parametrize("name,over,n_ctx,cap", [
    ("llama70b_long", dict(batch=1, n_q_heads=16, n_kv_heads=2), 1500, 1536),            # byte kernel, 8-head blocks
    ("llama70b_long", dict(batch=1, n_q_heads=8, n_kv_heads=2), 777, 800),               # byte kernel, quads
    ("llama8b_decode", dict(batch=1, n_q_heads=8, n_kv_heads=2), 1000, 1024),            # general kernel, packed
    ("mixed_3p5", dict(batch=1, n_q_heads=8, n_kv_heads=2), 999, 1024),                  # two groups, packed
])
def test_peaked_softmax(tq, name, over, n_ctx, cap):
    # queries scaled by 32 (a power of two, so bf16 queries stay exact):
    # log2-domain logits spread over ~100 units, so the
    # running reference jumps by more than the fixed grid's 32-unit window
    # and most weights underflow; outputs still follow the oracle, and the
    # split count still changes them by fp32 summation order only
    wl = synth.workload(name, **over)
    o = _oracle_side(wl, n_ctx, cap)
    q = (synth.draw_queries(wl) * 32.0).astype(np.float32)
    outs = []
    for ns in (1, 0, 7):
        print("peaked", name, over, "n_split", ns, flush=True)
        lg, out, q2 = _device_decode(tq, wl, o, n_ctx, cap, n_split=ns, q=q)
        outs.append((lg, out))
    rl, ro = _reference(wl, o, q2)
    ok_l, el = gc.normwise_close(outs[0][0], rl)
    ok_o, eo = gc.normwise_close(outs[0][1], ro)
    print("  logits", el, "out", eo, flush=True)
    assert ok_l, el
    assert ok_o, eo
    for lg, out in outs[1:]:
        ok, err = gc.normwise_close(out, outs[0][1], tol=5e-5)
        print("  vs one split", err, flush=True)
        assert ok, err
        # (logits far below the running reference sit on a finer fp32 grid
        # whose rounding depends on the reference: equal to ~1e-6)
        ok, err = gc.normwise_close(lg, outs[0][0], tol=1e-5)
        assert ok, err
