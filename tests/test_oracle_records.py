"""Pins of the oracle's record packers and byte accounting.

The packers are checked against words derived by hand from the format
definition (tests/golden/records_hand.json) and against an unpacker written
here independently from the same definition. The byte accounting is checked
against the figures of the winningdata.io article: its memory table
("Os numeros que importam": 4-bit ~0.125x and 3-bit ~0.09x of FP32, norms
not counted) and its KV sizing example ("O problema"), whose product is
garbled on the page; with 8 KV heads (the GQA shape of a 70B model) the
formula gives the ~42 GB it states.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "records_hand.json")))


def _hex(ws):
    return [int(w, 16) for w in ws]


def test_token_major_hand_words_one_group():
    g = GOLD["token_major_one_group"]
    idx = np.zeros((1, 32), np.int64)
    for j, v in g["codes_nonzero"].items():
        idx[0, int(j)] = v
    bits = np.zeros((1, 32), bool)
    bits[0, g["signs_set"]] = True
    c, s, n = oracle.pack_token_major([idx], [bits], [np.array([g["norm"]])],
                                      [np.array([g["gamma"]])], g["dims"], g["mse_bits"])
    assert c[0].tolist() == _hex(g["expect_code_words"])
    assert s[0].tolist() == _hex(g["expect_sign_words"])
    assert n[0].tolist() == [2.5, 0.75]


def test_token_major_hand_words_two_groups():
    g = GOLD["token_major_two_groups"]
    i0 = np.zeros((1, 32), np.int64)
    i1 = np.zeros((1, 32), np.int64)
    for j, v in g["group0_codes_nonzero"].items():
        i0[0, int(j)] = v
    for j, v in g["group1_codes_nonzero"].items():
        i1[0, int(j)] = v
    b0 = np.zeros((1, 32), bool)
    b1 = np.zeros((1, 32), bool)
    b1[0, g["group1_signs_set"]] = True
    one = [np.ones(1), np.ones(1)]
    c, s, n = oracle.pack_token_major([i0, i1], [b0, b1], one, one, g["dims"], g["mse_bits"])
    assert c[0].tolist() == _hex(g["expect_code_words"])
    assert s[0].tolist() == _hex(g["expect_sign_words"])
    assert n.shape == (1, 4)


def test_block32_hand_words():
    g = GOLD["block32_one_group"]
    idx = np.zeros((32, 32), np.int64)
    bits = np.zeros((32, 32), bool)
    for e in g["entries"]:
        idx[e["slot"], e["channel"]] = e["code"]
        bits[e["slot"], e["channel"]] = bool(e["sign"])
    z = np.zeros(32)
    c, s, n = oracle.pack_block32([idx], [bits], [z], [z], g["dims"], g["mse_bits"])
    assert c.shape == (1, 64) and s.shape == (1, 32) and n.shape == (32, 2)
    expect_c = np.zeros(64, np.uint32)
    for k, v in g["expect_code_words_nonzero"].items():
        expect_c[int(k)] = int(v, 16)
    expect_s = np.zeros(32, np.uint32)
    for k, v in g["expect_sign_words_nonzero"].items():
        expect_s[int(k)] = int(v, 16)
    assert np.array_equal(c[0], expect_c) and np.array_equal(s[0], expect_s)


def _bit(words, pos):
    return (int(words[pos // 32]) >> (pos % 32)) & 1


def _unpack_token_major(c_row, s_row, dims, mse_bits):
    codes, signs, cw, sw = [], [], 0, 0
    for d, m in zip(dims, mse_bits):
        w = c_row[cw:]
        codes.append([sum(_bit(w, m * j + p) << p for p in range(m)) for j in range(d)])
        signs.append([_bit(s_row[sw:], j) for j in range(d)])
        cw += (m * d + 31) // 32
        sw += (d + 31) // 32
    return codes, signs


def _unpack_block32(c_blk, s_blk, dims, mse_bits, slot):
    o, s = slot // 8, slot % 8
    codes, signs, cw, sw = [], [], 0, 0
    for d, m in zip(dims, mse_bits):
        codes.append([sum(_bit(c_blk[cw:], 8 * m * (o * d + j) + m * s + p) << p for p in range(m))
                      for j in range(d)])
        signs.append([_bit(s_blk[sw:], 8 * (o * d + j) + s) for j in range(d)])
        cw += m * d
        sw += d
    return codes, signs


@pytest.mark.parametrize("dims,bits", [([128], [3]), ([64, 64], [3, 2]), ([64, 64], [2, 1]),
                                       ([200], [3]), ([40, 24], [4, 1])])
def test_round_trip_independent_unpacker(dims, bits):
    rng = np.random.default_rng(sum(dims) + sum(bits))
    n = 64
    idx = [rng.integers(0, 2 ** m, size=(n, d)) for d, m in zip(dims, bits)]
    sg = [rng.random((n, d)) < 0.5 for d in dims]
    nm = [rng.random(n).astype(np.float32) for _ in dims]
    c, s, norms = oracle.pack_token_major(idx, sg, nm, nm, dims, bits)
    cw, sw, nf, bcw, bsw = oracle.record_words(dims, bits)
    assert c.shape == (n, cw) and s.shape == (n, sw) and norms.shape == (n, nf)
    for r in (0, 17, 63):
        codes, signs = _unpack_token_major(c[r], s[r], dims, bits)
        for g in range(len(dims)):
            assert codes[g] == idx[g][r].tolist() and signs[g] == sg[g][r].astype(int).tolist()
    if all(d % 8 == 0 for d in dims):
        cb, sb, nb = oracle.pack_block32(idx, sg, nm, nm, dims, bits)
        assert cb.shape == (n // 32, bcw) and sb.shape == (n // 32, bsw)
        for r in (0, 9, 31, 40, 63):
            codes, signs = _unpack_block32(cb[r // 32], sb[r // 32], dims, bits, r % 32)
            for g in range(len(dims)):
                assert codes[g] == idx[g][r].tolist() and signs[g] == sg[g][r].astype(int).tolist()
        assert np.array_equal(nb, norms)


def test_bytes_per_token():
    # 3 bits = 2 + 1 and 4 bits = 3 + 1 per channel plus two float32 norms per group
    assert oracle.record_bytes([128], [2]) == 56
    assert oracle.record_bytes([128], [3]) == 72
    assert oracle.record_bytes([64, 64], [3, 2]) == 72      # 3.5 bits per channel
    assert oracle.record_bytes([64, 64], [2, 1]) == 56      # 2.5 bits per channel
    assert oracle.record_bytes([200], [3]) == 108
    # memory relative to FP32 with norms not counted: 4/32 and 3/32 of FP32
    fp32 = 128 * 4
    assert oracle.record_bytes([128], [3], include_norms=False) / fp32 == 0.125
    assert abs(oracle.record_bytes([128], [2], include_norms=False) / fp32 - 0.09375) < 1e-12


def test_kv_sizing_example():
    # K and V x 80 layers x 8 KV heads x d=128 x 128K tokens x 2 bytes (FP16)
    fp16_bytes = 2 * 80 * 8 * 128 * 128 * 1024 * 2
    assert fp16_bytes == 42_949_672_960
    assert 41e9 < fp16_bytes < 43e9
    # the same cache in 3-bit records (norms included) is 56/256 of that
    assert fp16_bytes * oracle.record_bytes([128], [2]) / 256 == 2 * 80 * 8 * 128 * 1024 * 56
