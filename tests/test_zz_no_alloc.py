"""tq_attn_decode_scratch (decode with the library's static device workspace,
for callers that cannot allocate) against tq_attn_decode with a caller
workspace, through the C ABI: two calls in a row on the same GPU, the second
with a smaller shape, each giving results identical to the workspace call
(the same kernels run on the same inputs; only the workspace address
differs)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotation_amd as m
    m.lib()
    return m


def _case(tq, batch, hq, hkv, n_ctx, want_logits):
    import torch
    wl = synth.workload("llama8b_decode", batch=batch, n_q_heads=hq, n_kv_heads=hkv, n_ctx=n_ctx)
    cap = wl.capacity
    ks, vs = synth.draw_quantizer(wl, "K"), synth.draw_quantizer(wl, "V")
    bits = [g.mse_bits for g in ks.groups]
    kq = tq.Quantizer.from_parts(ks.rotations, ks.sketches, bits, perm=ks.perm)
    vq = tq.Quantizer.from_parts(vs.rotations, vs.sketches, bits, perm=vs.perm)
    n_rows = batch * hkv * cap
    kc = tq.Cache.empty(kq, n_rows, tq.TQ_TOKEN_MAJOR)
    vc = tq.Cache.empty(vq, n_rows, tq.TQ_BLOCK32)
    for b in range(batch):
        for h in range(hkv):
            r0 = (b * hkv + h) * cap
            for side, qz, cache, fmt in (("K", kq, kc, tq.TQ_TOKEN_MAJOR), ("V", vq, vc, tq.TQ_BLOCK32)):
                x = torch.from_numpy(synth.draw_kv_slab(wl, side, b, h, 0, cap)).cuda().to(torch.bfloat16)
                tq.tq_quantize(qz, fmt, x, cache, seg_len=cap, seg_stride=cap, seg_offset=r0)
    q = torch.from_numpy(synth.draw_queries(wl)).cuda().to(torch.bfloat16)
    shape = tq.decode_shape(batch, hq, hkv, n_ctx, cap, wl.scale)
    res = []
    for fn in ("workspace", "scratch"):
        out = torch.full((batch, hq, wl.d), float("nan"), device="cuda")
        logits = torch.full((batch, hq, n_ctx), float("nan"), device="cuda") if want_logits else None
        if fn == "workspace":
            tq.tq_attn_decode(kq, vq, shape, q, kc, vc, logits=logits, out=out)
        else:
            tq.tq_attn_decode_scratch(kq, vq, shape, q, kc, vc, logits=logits, out=out)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), None if logits is None else logits.cpu().numpy()))
    (o_ws, l_ws), (o_sc, l_sc) = res
    assert np.all(np.isfinite(o_ws))
    np.testing.assert_array_equal(o_sc, o_ws)
    if want_logits:
        np.testing.assert_array_equal(l_sc, l_ws)


def test_scratch_decode_two_calls_second_smaller(tq):
    print("no-alloc decode: B=2, 32 q / 8 kv heads, 3000 tokens, with logits", flush=True)
    _case(tq, 2, 32, 8, 3000, True)
    print("no-alloc decode: B=1, 8 q / 2 kv heads, 500 tokens, no logits", flush=True)
    _case(tq, 1, 8, 2, 500, False)
