"""CPU oracle for native low-bit MLA decode (QuantMLA C4R4 / C2R4).

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct
definition that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The library under ``bit_mla_kv_quant_amd/`` never imports it and
shares no code with it: the layout, the quantizer, the protected-set rule and
the attention here are written independently from the pages.

Sources (cited by page title and section only):
  * "QuantMLA: Function-Aligned Dual-Path Quantization for Low-Bit MLA KV
    Caching" -- cited as [QuantMLA <section>]; the paperlayer.ai summary and the
    signal-papers full text carry the same section numbering.
  * "DeepSeek MLA: low-rank KV cache and inference efficiency" (weigao.cc,
    Chinese) -- cited as [MLA blog <section>].

Arithmetic conventions:
  * the quantizer and the dequantizer run op-for-op in IEEE float32 (numpy
    float32 scalars/arrays), with bf16 storage via round-to-nearest-even;
  * attention runs in float64 over the bf16 values each token contributes.

Modules:
  quant       -- bf16 rounding, per-token group quantizer, dequantizer
  layout      -- packed page byte layout (pack / unpack), prot-buffer rows
  attention   -- protected set, effective rows, fp64 softmax attention,
                 partial (m, s, o) triples and their merge
  accounting  -- persistent-cache byte accounting and cache-schema counts

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, library routines or the pages' printed
numbers.  The paper's own kernel outputs are not available, so agreement with
them is "parity unpinned" (no code, weights or data are published with the
pages).
"""

from . import quant, layout, attention, accounting  # noqa: F401
