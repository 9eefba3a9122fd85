"""Packed page byte layout and BF16 protection-buffer rows (oracle).

[MLA blog §6]: a paged MLA cache keeps, per page of block_tokens tokens, the
latent c_KV[block_tokens, d_c] and the RoPE key k_R[block_tokens, d_R]; a
logical-to-physical block map locates pages.
[QuantMLA App. C.5]: pages hold 64 tokens; the fused writer quantizes, packs
integer codes and inserts them at the token's mapped slot; a packed copy of
every token is kept; each request and layer also owns a fixed BF16 protection
buffer of 132 rows of 576 values (4 sink + 128 recent tokens).

The pages do not print a byte layout (their 20,480-byte C4R4 page cannot hold
bf16 scale+zero for all nine groups; see the accounting module).  The layout
below is this library's own, written out here independently of the HIP code.

One physical page (P = 64 token slots), structure-of-arrays, all region
offsets multiples of 256 bytes:

  region   C4R4                         C2R4
  codes_c  [4 blk][64 tok][64 B]        [2 blk][64 tok][64 B]
           blk = content dims 128*blk..   blk = content dims 256*blk..
           byte k: dims 2k (bits 0-3),    little-endian 32-bit word k holds
                   2k+1 (bits 4-7)        dims 16k..16k+15: dim 16k+2m at
                                          bits 2m..2m+1 and dim 16k+2m+1 at
                                          bits 16+2m..17+2m (m = 0..7), so
                                          each pair of neighbouring dims sits
                                          16 bits apart
  codes_r  [64 tok][32 B]  byte k: RoPE dims 2k (bits 0-3), 2k+1 (bits 4-7)
  meta_c   [64 tok][8 grp][2] bf16 (scale, zero), little endian
  meta_r   [64 tok][2] bf16 (scale, zero); format C4R4F (content as C4R4):
           [64 tok][2] fp32 (scale, zero), little endian

  page bytes: C4R4 16384+2048+2048+256 = 20736 ; C2R4 8192+2048+2048+256 = 12544 ;
              C4R4F 16384+2048+2048+512 = 20992

A slot index is page_id * 64 + offset.

Protection-buffer rows (per sequence slot, [132][576] bf16, row = [c | k_R]):
token i < 4 uses row i; token i >= 4 uses row 4 + (i mod 128).  Any 128
consecutive positions land on distinct rows, so the ring always holds the 128
most recent tokens and a new token replaces exactly the one leaving the window.
"""

import numpy as np

from .quant import D_C, D_R, F32_ROPE, FORMATS, N_GROUPS_C

PAGE_TOKENS = 64
N_SINK = 4
N_RECENT = 128
PROT_ROWS = N_SINK + N_RECENT   # 132


def _regions(fmt):
    cbytes = FORMATS[fmt][0] * D_C // 8               # content code bytes per token
    codes_c = PAGE_TOKENS * cbytes
    codes_r = PAGE_TOKENS * 32
    meta_c = PAGE_TOKENS * N_GROUPS_C * 4
    meta_r = PAGE_TOKENS * (8 if fmt in F32_ROPE else 4)   # (scale, zero) fp32 or bf16
    off_r = codes_c
    off_mc = off_r + codes_r
    off_mr = off_mc + meta_c
    total = off_mr + meta_r
    return {"cbytes": cbytes, "off_c": 0, "off_r": off_r, "off_mc": off_mc,
            "off_mr": off_mr, "page_bytes": total}


def page_bytes(fmt):
    return _regions(fmt)["page_bytes"]


def pack_content(codes_c, fmt):
    """codes_c uint8 [T,512] -> per-token packed content bytes [T, n_blk, 64]."""
    q = np.asarray(codes_c, dtype=np.uint8)
    T = q.shape[0]
    if FORMATS[fmt][0] == 4:
        # blk b covers dims 128b..128b+127; byte k = dims 2k (lo), 2k+1 (hi)
        q = q.reshape(T, 4, 64, 2)
        return (q[..., 0] | (q[..., 1] << 4)).astype(np.uint8)
    # C2R4: blk b covers dims 256b..256b+255 as 16 words of 16 dims; within a
    # word, dim 2m goes to bits 2m and dim 2m+1 to bits 16+2m
    q = q.reshape(T, 2, 16, 8, 2).astype(np.uint32)
    shift_even = (2 * np.arange(8, dtype=np.uint32))
    words = ((q[..., 0] << shift_even) | (q[..., 1] << (shift_even + 16))).sum(axis=-1)
    return words.astype("<u4").view(np.uint8).reshape(T, 2, 64)


def unpack_content(packed, fmt):
    """Inverse of pack_content: [T, n_blk, 64] bytes -> codes [T,512]."""
    p = np.asarray(packed, dtype=np.uint8)
    T = p.shape[0]
    if FORMATS[fmt][0] == 4:
        return np.stack([p & 0xF, p >> 4], axis=-1).reshape(T, D_C).astype(np.uint8)
    words = np.ascontiguousarray(p).view("<u4").reshape(T, 2, 16, 1).astype(np.uint32)
    shift_even = (2 * np.arange(8, dtype=np.uint32))
    even = (words >> shift_even) & 3
    odd = (words >> (shift_even + 16)) & 3
    return np.stack([even, odd], axis=-1).reshape(T, D_C).astype(np.uint8)


def pack_rope(codes_r):
    """codes_r uint8 [T,64] -> [T,32] bytes; byte k = dims 2k (lo), 2k+1 (hi)."""
    q = np.asarray(codes_r, dtype=np.uint8).reshape(-1, 32, 2)
    return (q[..., 0] | (q[..., 1] << 4)).astype(np.uint8)


def unpack_rope(packed):
    p = np.asarray(packed, dtype=np.uint8)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[0], D_R).astype(np.uint8)


def write_tokens(pages, slots, qt, fmt):
    """Insert quantized tokens into a page pool.

    pages : uint8 [num_pages, page_bytes] (modified in place)
    slots : int64 [T], slot = page_id*64 + offset
    qt    : output of quant.quantize_tokens
    """
    R = _regions(fmt)
    slots = np.asarray(slots, dtype=np.int64)
    pc = pack_content(qt["codes_c"], fmt)          # [T, nblk, 64]
    pr = pack_rope(qt["codes_r"])                  # [T, 32]
    nblk = pc.shape[1]
    for t, slot in enumerate(slots):
        pg, off = divmod(int(slot), PAGE_TOKENS)
        page = pages[pg]
        for b in range(nblk):
            base = R["off_c"] + (b * PAGE_TOKENS + off) * 64
            page[base:base + 64] = pc[t, b]
        base = R["off_r"] + off * 32
        page[base:base + 32] = pr[t]
        meta = np.stack([qt["scale"][t, :N_GROUPS_C], qt["zero"][t, :N_GROUPS_C]], axis=1)
        base = R["off_mc"] + off * N_GROUPS_C * 4
        page[base:base + N_GROUPS_C * 4] = meta.astype("<u2").reshape(-1).view(np.uint8)
        if fmt in F32_ROPE:
            mr = np.array([qt["scale_r32"][t], qt["zero_r32"][t]], dtype="<f4")
            base = R["off_mr"] + off * 8
            page[base:base + 8] = mr.view(np.uint8)
        else:
            mr = np.array([qt["scale"][t, N_GROUPS_C], qt["zero"][t, N_GROUPS_C]], dtype="<u2")
            base = R["off_mr"] + off * 4
            page[base:base + 4] = mr.view(np.uint8)


def read_page(page, fmt):
    """Decode one page's 64 slots -> dict like quantize_tokens' output (T=64)."""
    R = _regions(fmt)
    page = np.asarray(page, dtype=np.uint8)
    nblk = R["cbytes"] // 64
    pc = page[R["off_c"]:R["off_c"] + nblk * PAGE_TOKENS * 64].reshape(nblk, PAGE_TOKENS, 64)
    pc = pc.transpose(1, 0, 2)                                  # [tok, blk, 64]
    pr = page[R["off_r"]:R["off_r"] + PAGE_TOKENS * 32].reshape(PAGE_TOKENS, 32)
    mc = page[R["off_mc"]:R["off_mc"] + PAGE_TOKENS * N_GROUPS_C * 4].copy().view("<u2")
    mc = mc.reshape(PAGE_TOKENS, N_GROUPS_C, 2)
    out = {"codes_c": unpack_content(pc, fmt), "codes_r": unpack_rope(pr)}
    if fmt in F32_ROPE:
        mr32 = page[R["off_mr"]:R["off_mr"] + PAGE_TOKENS * 8].copy().view("<f4").reshape(PAGE_TOKENS, 2)
        out["scale_r32"] = mr32[:, 0].astype(np.float32)
        out["zero_r32"] = mr32[:, 1].astype(np.float32)
        mr = np.zeros((PAGE_TOKENS, 2), np.uint16)
    else:
        mr = page[R["off_mr"]:R["off_mr"] + PAGE_TOKENS * 4].copy().view("<u2").reshape(PAGE_TOKENS, 2)
    out["scale"] = np.concatenate([mc[:, :, 0], mr[:, :1]], axis=1).astype(np.uint16)
    out["zero"] = np.concatenate([mc[:, :, 1], mr[:, 1:]], axis=1).astype(np.uint16)
    return out


def prot_row(i):
    """Protection-buffer row of zero-based token position i (scalar or array)."""
    i = np.asarray(i, dtype=np.int64)
    return np.where(i < N_SINK, i, N_SINK + (i % N_RECENT))
