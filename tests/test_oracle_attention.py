"""Pins of the oracle's paged decode attention (MXFP8 K/V, GQA): a
hand-worked example, closed forms (one token, zero query), invariants
(token order, slots past the length, head grouping) and the cache layout
against the packed-weight layout written independently for the GEMMs."""

import math
import os

import numpy as np
import pytest

from oracle import attention as att
from oracle import fp8, layout, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attention_worked_example.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = np.array([float(t) for t in v.split()])
    return vals


def _bf16(rng, shape, std=1.0):
    return fp8.to_bf16((rng.standard_normal(shape) * std).astype(np.float32).astype(np.float64))


def test_worked_example():
    g = _golden()
    D = 32
    q = np.zeros((2, 2, D))
    k = np.zeros((2, 3, 1, D))
    v = np.zeros((2, 3, 1, D))
    q[0, 0, 0] = 256.0
    k[0, 0, 0, 1] = 256.0
    k[0, 1, 0, 0] = 256.0
    k[0, 2, 0, 0] = 1000.0
    v[0, 0, 0, 2], v[0, 0, 0, 5] = 300.5, 256.0
    v[0, 1, 0, 3], v[0, 1, 0, 4] = 448.0, 17.0
    v[0, 2, 0, 0] = 1000.0
    q[1] = 5.0
    k[1, 0, 0, 0] = 7.0
    v[1, 0, 0, 7], v[1, 0, 0, 8] = 100.0, 3.0
    o = att.decode_attention(q, k, v, [2, 1], sm_scale=math.log(3.0) / 65536.0)
    np.testing.assert_allclose(o[0, 0, 2:6], g["seq0_head0_dims_2_3_4_5"], rtol=1e-15, atol=1e-13)
    np.testing.assert_allclose(o[0, 1, 2:6], g["seq0_head1_dims_2_3_4_5"], rtol=1e-15, atol=1e-13)
    for h in range(2):
        np.testing.assert_array_equal(o[1, h, 7:9], g["seq1_dims_7_8"])
        assert np.all(np.delete(o[1, h], [7, 8]) == 0.0)
    assert np.all(np.delete(o[0, 0], [2, 3, 4, 5]) == 0.0)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    q = _bf16(rng, (2, 8, 128))
    k = _bf16(rng, (2, 5, 2, 128))
    v = _bf16(rng, (2, 5, 2, 128))
    o = att.decode_attention(q, k, v, [1, 1])
    vd = att.dequantize_vectors(*att.quantize_vectors(v[:, 0]))
    for h in range(8):
        np.testing.assert_allclose(o[:, h], vd[:, h // 4], rtol=1e-14)


def test_zero_query_averages_the_values():
    rng = np.random.default_rng(2)
    T = 37
    q = np.zeros((1, 4, 64))
    k = _bf16(rng, (1, T + 3, 1, 64))
    v = _bf16(rng, (1, T + 3, 1, 64))
    o = att.decode_attention(q, k, v, [T])
    vd = att.dequantize_vectors(*att.quantize_vectors(v[0, :T, 0]))
    np.testing.assert_allclose(o[0], np.broadcast_to(vd.mean(axis=0), (4, 64)), rtol=1e-12)


def test_token_order_and_slots_past_the_length():
    rng = np.random.default_rng(3)
    T = 29
    q = _bf16(rng, (1, 4, 64))
    k = _bf16(rng, (1, 40, 2, 64))
    v = _bf16(rng, (1, 40, 2, 64))
    o = att.decode_attention(q, k, v, [T])
    perm = np.concatenate([rng.permutation(T), np.arange(T, 40)])
    o2 = att.decode_attention(q, k[:, perm], v[:, perm], [T])
    np.testing.assert_allclose(o, o2, rtol=1e-12)
    k3, v3 = k.copy(), v.copy()
    k3[:, T:] = 1e4
    v3[:, T:] = -1e4
    np.testing.assert_array_equal(att.decode_attention(q, k3, v3, [T]), o)


def test_query_heads_read_their_group():
    """Head h attends over KV head h // G only: moving the other KV heads
    changes nothing for it."""
    rng = np.random.default_rng(4)
    q = _bf16(rng, (1, 6, 32))
    k = _bf16(rng, (1, 9, 3, 32))
    v = _bf16(rng, (1, 9, 3, 32))
    o = att.decode_attention(q, k, v, [9])
    for g in range(3):
        k2, v2 = k.copy(), v.copy()
        others = [x for x in range(3) if x != g]
        k2[:, :, others] *= -3.0
        v2[:, :, others] += 1.0
        o2 = att.decode_attention(q, k2, v2, [9])
        np.testing.assert_array_equal(o2[0, 2 * g:2 * g + 2], o[0, 2 * g:2 * g + 2])


def test_k_page_matches_the_packed_weight_layout():
    """A K page's first 2048 bytes are the packed-weight tile of its 16 slots
    (tokens as rows); its scale bytes follow the lane order of the matrix
    instruction's scale operand (lane l: slot l % 16, block l // 16)."""
    rng = np.random.default_rng(5)
    x = _bf16(rng, (16, 1, 128), 2.0)
    c, s = att.quantize_vectors(x)
    pg = att.pack_pages(c, s, np.arange(16), 1, "k")[0, 0]
    np.testing.assert_array_equal(pg[:2048], layout.pack_codes(c[:, 0]))
    for l in range(64):
        assert pg[2048 + l] == s[l % 16, 0, l // 16]


def test_v_page_layout():
    """V page bytes at hand-computed offsets: lane (d % 16) + 16 (r // 4),
    byte 4 (d // 16) + r % 4 of its 32; scales at 2048 + 16 (r // 4) + 4 b + r % 4."""
    rng = np.random.default_rng(6)
    x = _bf16(rng, (5, 2, 128), 2.0)
    c, s = att.quantize_vectors(x)
    slots = np.array([3, 17, 18, 31, 40])
    pg = att.pack_pages(c, s, slots, 3, "v")
    # (slot, dim) -> byte, worked out by hand
    hand = {(3, 0): 32 * 0 + 0 + 3, (3, 17): 32 * 1 + 4 + 3, (1, 77): 32 * 13 + 16 + 1,
            (2, 126): 32 * 14 + 28 + 2, (15, 127): 32 * 63 + 28 + 3, (8, 40): 32 * 40 + 8 + 0}
    for t, sl in enumerate(slots):
        p, r = divmod(int(sl), 16)
        for h in range(2):
            for (rr, dim), off in hand.items():
                if rr == r:
                    assert pg[p, h, off] == c[t, h, dim]
            for dim in range(128):
                assert pg[p, h, 32 * (dim % 16 + 16 * (r // 4)) + 4 * (dim // 16) + r % 4] == c[t, h, dim]
            for b in range(4):
                assert pg[p, h, 2048 + 16 * (r // 4) + 4 * b + r % 4] == s[t, h, b]
    # slot 3, block 2 and slot 13, block 1, by hand
    assert pg[0, 0, 2048 + 0 + 8 + 3] == s[0, 0, 2]
    assert pg[2, 1, 2048 + 32 + 0 + 0] == s[4, 1, 0]  # slot 40 = page 2, slot 8, block 0
    # slot 37 (page 2, slot 5) was never written
    assert np.all(pg[2, :, [32 * (d % 16 + 16) + 4 * (d // 16) + 1 for d in range(128)]] == 0)
    # every byte of a page is some (slot, dim) exactly once
    seen = {32 * (d % 16 + 16 * (r // 4)) + 4 * (d // 16) + r % 4 for r in range(16) for d in range(128)}
    assert seen == set(range(2048))


def test_quantize_vectors_is_the_activation_quantizer():
    rng = np.random.default_rng(7)
    x = _bf16(rng, (3, 4, 64))
    c, s = att.quantize_vectors(x)
    c2, s2 = quant.quantize_act(x.reshape(12, 64), "mx")
    np.testing.assert_array_equal(c.reshape(12, 64), c2)
    np.testing.assert_array_equal(s.reshape(12, 2), s2)
