"""Persistent KV-cache byte accounting and cache-schema counts (oracle).

[QuantMLA App. C.5]: with d_c = 512, d_r = 64 and 64-token pages the packed
C4R4 page takes 20,480 bytes (320 per token and layer); each request and layer
adds a 132 x 576 x 2 = 152,064-byte BF16 protection buffer; reverse page
mappings take 8 bytes per physical page; a BF16 page takes 64 x 1,152 =
73,728 bytes.  The per-layer allocation formula for a request of length L is
missing from the extracted text; the reading taken (pages = ceil(L / 64),
reverse maps counted on the packed side only) is

    packed(L) = ceil(L/64) * (page_bytes + 8) + 152,064
    bf16(L)   = ceil(L/64) * 73,728

which yields the printed ratios 3.22x at 4K and 3.59x at 128K
[QuantMLA §4.4, App. C.5].  Model weights, shared page tables, allocator
overhead and workspaces are excluded, as on the pages.

[MLA blog §1]: MHA with 128 heads of 128 dims caches 2*128*128 = 32,768
elements per token and layer; MLA caches d_c + d_R = 576, about 56.9x fewer.
[MLA blog §5]: MLA cache bytes = layers * tokens * batch * (d_c + d_R) *
bytes_per_element.
"""

import math

PAPER_C4R4_PAGE = 20480      # [QuantMLA App. C.5]
REVERSE_MAP_BYTES = 8        # per physical page
PROT_BYTES = 132 * 576 * 2   # 152,064
BF16_PAGE = 64 * (512 + 64) * 2   # 73,728


def pages(L, page_tokens=64):
    return -(-int(L) // page_tokens)


def packed_bytes(L, page_bytes=PAPER_C4R4_PAGE):
    return pages(L) * (page_bytes + REVERSE_MAP_BYTES) + PROT_BYTES


def bf16_bytes(L):
    return pages(L) * BF16_PAGE


def compression(L, page_bytes=PAPER_C4R4_PAGE):
    return bf16_bytes(L) / packed_bytes(L, page_bytes)


def mha_elements(n_heads, head_dim):
    """K and V for every head: 2 * heads * head_dim elements per token and layer."""
    return 2 * n_heads * head_dim


def mla_elements(d_c, d_r):
    return d_c + d_r


def mla_cache_bytes(layers, tokens, batch, d_c, d_r, bytes_per_elem):
    return layers * tokens * batch * (d_c + d_r) * bytes_per_elem


def mha_cache_bytes(layers, tokens, batch, n_heads, head_dim, bytes_per_elem):
    return layers * tokens * batch * mha_elements(n_heads, head_dim) * bytes_per_elem


def gib(nbytes):
    return nbytes / float(1 << 30)


def gb(nbytes):
    return nbytes / 1e9


def ceil_div(a, b):
    return -(-a // b)


__all__ = [n for n in dir() if not n.startswith("_") and n != "math"]
