"""Native low-bit MLA decode (QuantMLA C4R4 / C2R4) for AMD MI355X (gfx950).

The compute lives in ``libmla_lowbit.so`` (hand-written HIP, C ABI declared in
``include/mla_lowbit.h``).  ``bit_mla_kv_quant_amd.ops`` is a thin ctypes
binding over it and raises if the library is not built; there is no CPU
fallback.  ``bit_mla_kv_quant_amd.synth`` draws seeded synthetic workloads.
"""
