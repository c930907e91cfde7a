"""GPU parity of the paged decode attention over an MXFP8 K/V cache: the
cache writer byte for byte against the oracle's layout, and the decode
against the oracle's float64 attention (ragged lengths, shuffled pages, GQA
groups of 1, 4 and 16, split sequences), plus edge cases."""

import numpy as np
import pytest
import torch

import swiglu_decode_amd as sgd
import synth
from oracle import attention as att
from synth import bf16_to_f64
from tests.gpu_util import assert_close, dev, note

pytestmark = pytest.mark.gpu


def _slots(inp):
    """Slot of every (sequence, token) in sequence order, and the flat token list."""
    lens, pages = inp["lens"], inp["pages"]
    slots, idx = [], []
    for b, T in enumerate(lens):
        t = np.arange(T)
        slots.append(pages[b, t // 16] * 16 + t % 16)
        idx.append(np.stack([np.full(T, b), t], axis=1))
    return np.concatenate(slots).astype(np.int32), np.concatenate(idx)


def _build(inp, Hkv, d):
    slots, idx = _slots(inp)
    kf = inp["k"][idx[:, 0], idx[:, 1]].contiguous()  # [n, Hkv, 128]
    vf = inp["v"][idx[:, 0], idx[:, 1]].contiguous()
    kc = sgd.kv_cache_alloc(inp["n_pages"], Hkv, d)
    vc = sgd.kv_cache_alloc(inp["n_pages"], Hkv, d)
    st = torch.from_numpy(slots).to(d)
    sgd.kv_cache_write("k", kf.to(d), st, kc, inp["n_pages"])
    sgd.kv_cache_write("v", vf.to(d), st, vc, inp["n_pages"])
    return kc, vc, slots, kf, vf


def test_kv_cache_write_bit_exact():
    d = dev()
    note("paged K/V cache write vs oracle layout")
    Hkv = 3
    inp = synth.attention_inputs(4, 6, Hkv, 1, 70, 2001, extra_pages=5)
    kc, vc, slots, kf, vf = _build(inp, Hkv, d)
    torch.cuda.synchronize()
    for kind, x, cache in (("k", kf, kc), ("v", vf, vc)):
        c, s = att.quantize_vectors(bf16_to_f64(x))
        want = att.pack_pages(c, s, slots, inp["n_pages"], kind).reshape(-1)
        got = cache.cpu().numpy()
        assert got.size == want.size
        np.testing.assert_array_equal(got, want, err_msg=f"{kind} cache bytes")


@pytest.mark.parametrize("B,Hq,Hkv,lo,hi", [(5, 8, 2, 1, 200), (3, 16, 1, 1, 40), (4, 4, 4, 15, 17),
                                            (8, 32, 8, 1, 2000), (2, 32, 8, 3000, 5000),
                                            # one split each: the largest batch taken in order of
                                            # length, and one past it (dispatch order)
                                            (256, 4, 2, 1, 100), (300, 8, 2, 1, 64)])
def test_decode_attention_parity(B, Hq, Hkv, lo, hi):
    d = dev()
    note(f"paged decode attention B={B} Hq={Hq} Hkv={Hkv} lengths {lo}..{hi}")
    inp = synth.attention_inputs(B, Hq, Hkv, lo, hi, 2100 + B + Hq, extra_pages=3)
    kc, vc, _, _, _ = _build(inp, Hkv, d)
    out = sgd.paged_decode_attention(inp["q"].to(d), kc, vc, inp["n_pages"], torch.from_numpy(inp["pages"]).to(d),
                                     torch.from_numpy(inp["lens"]).to(d), Hkv)
    out2 = sgd.paged_decode_attention(inp["q"].to(d), kc, vc, inp["n_pages"], torch.from_numpy(inp["pages"]).to(d),
                                      torch.from_numpy(inp["lens"]).to(d), Hkv)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "not deterministic"
    want = att.decode_attention(bf16_to_f64(inp["q"]), bf16_to_f64(inp["k"]), bf16_to_f64(inp["v"]), inp["lens"])
    got = out.float().cpu().numpy().astype(np.float64)
    assert_close(got.reshape(B * Hq, -1), want.reshape(B * Hq, -1), f"decode attention B={B} Hq={Hq} Hkv={Hkv}")
    # every head of every sequence, not only in aggregate
    for b in range(B):
        for h in range(Hq):
            rf = np.linalg.norm(got[b, h] - want[b, h]) / np.linalg.norm(want[b, h])
            assert rf <= 1e-2, (b, h, rf)


@pytest.mark.parametrize("sm_scale", [0.02, 0.5])
def test_decode_attention_custom_scale(sm_scale):
    """A softmax scale other than 1/sqrt(head_dim): flat (0.02) and sharp
    (0.5, a few tokens carry most of the weight) distributions."""
    d = dev()
    note(f"paged decode attention sm_scale={sm_scale}")
    B, Hq, Hkv = 6, 16, 4
    inp = synth.attention_inputs(B, Hq, Hkv, 1, 600, 2500, extra_pages=2)
    kc, vc, _, _, _ = _build(inp, Hkv, d)
    out = sgd.paged_decode_attention(inp["q"].to(d), kc, vc, inp["n_pages"], torch.from_numpy(inp["pages"]).to(d),
                                     torch.from_numpy(inp["lens"]).to(d), Hkv, sm_scale=sm_scale)
    torch.cuda.synchronize()
    want = att.decode_attention(bf16_to_f64(inp["q"]), bf16_to_f64(inp["k"]), bf16_to_f64(inp["v"]), inp["lens"],
                                sm_scale=sm_scale)
    got = out.float().cpu().numpy().astype(np.float64)
    assert_close(got.reshape(B * Hq, -1), want.reshape(B * Hq, -1), f"decode attention sm_scale={sm_scale}")


def test_decode_attention_edges():
    """A length of 0 gives zeros; a table entry outside the cache is harmless
    for the other sequences; a one-token sequence returns its dequantized V."""
    d = dev()
    note("paged decode attention edge cases")
    Hkv, Hq = 2, 4
    inp = synth.attention_inputs(3, Hq, Hkv, 1, 30, 2200)
    kc, vc, _, _, _ = _build(inp, Hkv, d)
    lens = inp["lens"].copy()
    lens[0] = 0
    lens[2] = 1
    pages = inp["pages"].copy()
    pages[0, :] = 10 ** 6  # never read: length 0
    out = sgd.paged_decode_attention(inp["q"].to(d), kc, vc, inp["n_pages"], torch.from_numpy(pages).to(d),
                                     torch.from_numpy(lens).to(d), Hkv)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(got[0] == 0.0)
    vd = att.dequantize_vectors(*att.quantize_vectors(bf16_to_f64(inp["v"][2, 0])))  # [Hkv, 128]
    for h in range(Hq):
        np.testing.assert_allclose(got[2, h], vd[h // 2], rtol=2 ** -8, atol=1e-30)
    want = att.decode_attention(bf16_to_f64(inp["q"][1:2]), bf16_to_f64(inp["k"][1:2]), bf16_to_f64(inp["v"][1:2]),
                                lens[1:2])
    assert_close(got[1], want[0], "decode attention middle sequence")


def test_decode_attention_graph_replays():
    d = dev()
    note("paged decode attention under graph replay")
    Hkv, Hq = 8, 32
    inp = synth.attention_inputs(16, Hq, Hkv, 100, 900, 2300)
    kc, vc, _, _, _ = _build(inp, Hkv, d)
    q = inp["q"].to(d)
    pages = torch.from_numpy(inp["pages"]).to(d)
    lens = torch.from_numpy(inp["lens"]).to(d)
    out = torch.empty((16, Hq, 128), dtype=torch.bfloat16, device=d)
    ws = sgd.Workspace(d)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sgd.paged_decode_attention(q, kc, vc, inp["n_pages"], pages, lens, Hkv, out=out, workspace=ws)
        s.synchronize()
        want = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            sgd.paged_decode_attention(q, kc, vc, inp["n_pages"], pages, lens, Hkv, out=out, workspace=ws)
        for i in range(5):
            out.fill_(float("nan"))
            s.synchronize()
            g.replay()
            s.synchronize()
            assert torch.equal(out, want), f"replay {i}"


@pytest.mark.parametrize("ties", [False, True])
def test_decode_attention_full_batch(ties):
    """The benchmarked shape (batch 64, 32 query heads over 8 KV heads,
    lengths 256..4096): one split per sequence, workgroups taken in order of
    length.  With `ties`, most lengths are cut to one value (equal lengths are
    ordered by index).  Sampled sequences (the longest, the shortest and every
    eighth) against the oracle; the whole output is deterministic."""
    d = dev()
    B, Hq, Hkv = 64, 32, 8
    note(f"paged decode attention B={B} Hq={Hq} Hkv={Hkv} lengths 256..4096 ties={ties}")
    inp = synth.attention_inputs(B, Hq, Hkv, 256, 4096, 2400)
    kc, vc, _, _, _ = _build(inp, Hkv, d)
    lens = inp["lens"].copy()
    if ties:
        lens = np.minimum(lens, 1000).astype(np.int32)
    q, pages, lt = inp["q"].to(d), torch.from_numpy(inp["pages"]).to(d), torch.from_numpy(lens).to(d)
    out = sgd.paged_decode_attention(q, kc, vc, inp["n_pages"], pages, lt, Hkv)
    out2 = sgd.paged_decode_attention(q, kc, vc, inp["n_pages"], pages, lt, Hkv)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "not deterministic"
    got = out.float().cpu().numpy().astype(np.float64)
    sample = sorted({int(np.argmax(lens)), int(np.argmin(lens))} | set(range(0, B, 8)))
    for b in sample:
        T = int(lens[b])
        want = att.decode_attention(bf16_to_f64(inp["q"][b:b + 1]), bf16_to_f64(inp["k"][b:b + 1, :T]),
                                    bf16_to_f64(inp["v"][b:b + 1, :T]), lens[b:b + 1])[0]
        assert_close(got[b], want, f"decode attention sequence {b} (length {T})")
        for h in range(Hq):
            rf = np.linalg.norm(got[b, h] - want[h]) / np.linalg.norm(want[h])
            assert rf <= 1e-2, (b, h, rf)
