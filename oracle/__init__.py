"""CPU oracle for the decode-shape FP8 SwiGLU MLP.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU statement of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``swiglu_decode_amd``) never imports, calls or
falls back to anything here, and nothing here imports the product path.

Sources the definitions follow:

* Fish Audio, X post "We Made Our Best Voice Model Free. Here's the GPU Math
  Behind It.", section "Custom kernels for the shapes TTS actually uses":
  the SwiGLU MLP (activation, gate multiplication, down projection), 128x128
  block-scaled FP8 and 1x32 MX microscaling with OCP UE8M0 scales.
* fish.audio blog "Cómo hicimos que nuestra API de texto a voz sea
  gratuita: la ingeniería de inferencia detrás de S2.1 Pro", sections
  "Estrategia de cuantización FP8" (the two scale granularities), "Resultados
  de benchmark del kernel" (activation quantization with UE8M0 packing; the
  SwiGLU result re-quantized as the down GEMM's activation) and "Qué hay en
  código abierto" (1x128 activation groups times 128x128 weight blocks).
* The format names the pages use point to two public specifications: the OCP
  8-bit Floating Point Specification (OFP8, E4M3 element) and the OCP
  Microscaling Formats (MX) v1.0 specification (E8M0 shared scale).

Modules:

* ``fp8``    -- E4M3 decode table, RNE saturating encoder, UE8M0 codec, bf16.
* ``quant``  -- block-128 and MX-32 scale derivation, quantize, dequantize.
* ``layout`` -- the packed (pre-shuffled) weight layout, written from its
  prose definition, for bit-exact comparison of packed buffers.
* ``ref``    -- fp64 scaled GEMM, SwiGLU MLP, RMSNorm, decode stack, output
  head, error metrics.
* ``attention`` -- paged decode attention over an MXFP8 K/V cache with GQA
  (fish.audio blog, section "Qué hay en código abierto"), and the paged
  cache layout.

Parity notes: every function is pinned by tests under ``tests/`` against
closed forms, invariants, brute force or an independent library
implementation; see each module's header.
"""

from . import fp8, quant, layout, ref, attention  # noqa: F401
