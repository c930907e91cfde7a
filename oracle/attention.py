"""Paged decode attention over an MXFP8 KV cache, stated plainly in float64.

TEST INFRASTRUCTURE ONLY (see the package header): imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product.

Source: fish.audio blog "Cómo hicimos que nuestra API de texto a voz sea
gratuita: la ingeniería de inferencia detrás de S2.1 Pro", section "Qué hay
en código abierto" (an MXFP8 FlashAttention whose modes include paged decode
with native GQA through a stride-0 K/V broadcast: every query head of a group
reads its group's K/V, nothing is copied per head) and section "Resultados de
benchmark del kernel" (the decode-attention measurement).  The pages name the
operation and its formats but not its arithmetic; the readings taken here:

* K and V are cached per token and per KV head, each head_dim vector
  quantized on its own in 1x32 MX blocks along head_dim (OCP MX: E4M3
  elements, E8M0 scale; ``oracle.quant`` with fmt "mx"), the way a decode
  step appends one token to the cache;
* the query vector is quantized the same way (the fp8 QK^T product);
* query head h of Hq reads KV head h // G, G = Hq / Hkv;
* s_t = sm_scale * <q', k'_t> for the sequence's tokens t < T, p = softmax(s),
  o = sum_t p_t v'_t, with primes the dequantized values; sm_scale defaults
  to 1/sqrt(head_dim).

``page_bytes`` and ``pack_pages`` state the library's paged cache layout
(written from its prose definition in swiglu_decode.h) for bit-exact checks
of the GPU's cache writes.
"""

import numpy as np

from .quant import dequantize_act, quantize_act

PAGE = 16  # token slots per page
HEAD_DIM = 128


def quantize_vectors(x):
    """MX-quantize the last axis of x [..., D]: (codes uint8 [..., D],
    E8M0 scales uint8 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    c, s = quantize_act(x.reshape(-1, D), "mx")
    return c.reshape(x.shape), s.reshape(x.shape[:-1] + (D // 32,))


def dequantize_vectors(codes, scales):
    D = codes.shape[-1]
    return dequantize_act(codes.reshape(-1, D), scales.reshape(-1, D // 32), "mx").reshape(codes.shape)


def decode_attention(q, k, v, seq_lens, sm_scale=None):
    """o [B, Hq, D] for queries q [B, Hq, D], cached keys and values
    k, v [B, Tmax, Hkv, D] (float64 holding bf16 values; slots t >= T of a
    sequence are ignored) and lengths seq_lens [B] (each >= 1)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    qd = dequantize_vectors(*quantize_vectors(q))
    kd = dequantize_vectors(*quantize_vectors(k))
    vd = dequantize_vectors(*quantize_vectors(v))
    o = np.zeros((B, Hq, D))
    for b in range(B):
        T = int(seq_lens[b])
        for h in range(Hq):
            g = h // G
            s = sm_scale * (kd[b, :T, g] @ qd[b, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            o[b, h] = p @ vd[b, :T, g]
    return o


# ---------------------------------------------------------------------------
# Paged cache layout (per physical page and KV head, 2112 bytes for D = 128)
# ---------------------------------------------------------------------------
# K: bytes 0..2047 hold the page's 16 token slots as a 16 x 128 operand tile:
#    lane l = r + 16 q (slot r, q = 0..3) has dims 16q..16q+15 at bytes
#    16l..16l+15 and dims 64+16q..64+16q+15 at bytes 1024+16l..1024+16l+15;
#    bytes 2048 + l: the E8M0 scale of slot l % 16, 32-dim block l // 16.
# V: bytes 0..2047: lane l = (d % 16) + 16 (r // 4) holds bytes 32 l..32 l+31:
#    byte 32 l + 4 n + (r % 4) is the code of slot r, dim d = 16 n + d % 16
#    (n = 0..7), i.e. per lane and 16-dim block n one dword of four
#    consecutive slots; byte 2048 + 16 (r // 4) + 4 b + r % 4: the scale of
#    slot r, block b (lane group r // 4 reads its 16 scale bytes at once).
def page_bytes(D=HEAD_DIM):
    return D * PAGE + PAGE * (D // 32)


def _k_tile(codes, scales):
    """codes [16, 128], scales [16, 4] -> 2112 bytes (K layout)."""
    out = np.zeros(page_bytes(), dtype=np.uint8)
    for l in range(64):
        r, q = l % 16, l // 16
        out[16 * l:16 * l + 16] = codes[r, 16 * q:16 * q + 16]
        out[1024 + 16 * l:1024 + 16 * l + 16] = codes[r, 64 + 16 * q:64 + 16 * q + 16]
        out[2048 + l] = scales[r, q]
    return out


def _v_tile(codes, scales):
    """codes [16, 128], scales [16, 4] -> 2112 bytes (V layout)."""
    out = np.zeros(page_bytes(), dtype=np.uint8)
    for r in range(16):
        for d in range(HEAD_DIM):
            lane = d % 16 + 16 * (r // 4)
            out[32 * lane + 4 * (d // 16) + r % 4] = codes[r, d]
        for b in range(4):
            out[2048 + 16 * (r // 4) + 4 * b + r % 4] = scales[r, b]
    return out


def pack_pages(codes, scales, slots, n_pages, kind):
    """Cache bytes [n_pages, Hkv, 2112] holding token n's codes [n, Hkv, 128]
    and scales [n, Hkv, 4] at slot slots[n] = page * 16 + offset (kind "k" or
    "v"); slots no token names are zero."""
    n, Hkv, D = codes.shape
    assert D == HEAD_DIM
    tok = np.zeros((n_pages, Hkv, PAGE, D), dtype=np.uint8)
    sc = np.zeros((n_pages, Hkv, PAGE, D // 32), dtype=np.uint8)
    for t in range(n):
        p, r = divmod(int(slots[t]), PAGE)
        tok[p, :, r] = codes[t]
        sc[p, :, r] = scales[t]
    tile = _k_tile if kind == "k" else _v_tile
    out = np.zeros((n_pages, Hkv, page_bytes()), dtype=np.uint8)
    for p in range(n_pages):
        for h in range(Hkv):
            out[p, h] = tile(tok[p, h], sc[p, h])
    return out
