"""Helpers for the GPU parity tests: move a drawn workload to the device,
fill the cache through kv_quant_append, and build the oracle's expectations.
The oracle never sees anything the GPU produced except to compare with."""

import numpy as np
import torch

from oracle import attention, layout, quant


def dev():
    return torch.device("cuda:0")


def t_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev())


def t_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev())


def t_i64(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int64)).to(dev())


class GpuCache:
    """Device-side page pool + protection buffers for one drawn workload."""

    def __init__(self, d, fmt=None, seq_slots=None):
        from bit_mla_kv_quant_amd import ops
        self.ops = ops
        self.d = d
        self.fmt = fmt or d.wl.fmt
        self.pb = ops.mla_lb_page_bytes(self.fmt)
        self.pages = torch.zeros((d.num_pages, self.pb), dtype=torch.uint8, device=dev())
        B = d.B
        self.seq_slot_np = np.arange(B, dtype=np.int32) if seq_slots is None else np.asarray(seq_slots, np.int32)
        nslots = int(self.seq_slot_np.max()) + 1
        self.prot = torch.zeros((nslots, 132, 576), dtype=torch.int16, device=dev())
        self.seq_slot = t_i32(self.seq_slot_np)
        self.block_table = t_i32(d.block_table)
        self.lens = d.lens.astype(np.int64).copy()

    def append(self, b_list, positions_list, new_lens):
        """Append tokens: for each b in b_list, positions (array) with the
        sequence length after the call new_lens[k]."""
        d = self.d
        lat, kr, slots, ss, pos, nl = [], [], [], [], [], []
        for b, P, n in zip(b_list, positions_list, new_lens):
            P = np.asarray(P, dtype=np.int64)
            lat.append(d.c[b][P])
            kr.append(d.kr[b][P])
            slots.append(d.slots(b, P))
            ss.append(np.full(len(P), self.seq_slot_np[b], np.int32))
            pos.append(P.astype(np.int32))
            nl.append(np.full(len(P), n, np.int32))
        lat = np.concatenate(lat)
        if lat.shape[0] == 0:
            return
        self.ops.kv_quant_append(
            self.fmt, t_bf16(lat), t_bf16(np.concatenate(kr)), t_i64(np.concatenate(slots)),
            t_i32(np.concatenate(ss)), t_i32(np.concatenate(pos)), t_i32(np.concatenate(nl)),
            self.pages, self.prot)

    def fill(self, chunk_tokens=1 << 20):
        """Append every sequence's first lens[b] tokens (prompt-style bulk insert)."""
        B = self.d.B
        pending = []
        count = 0
        for b in range(B):
            L = int(self.lens[b])
            pending.append((b, np.arange(L), L))
            count += L
            if count >= chunk_tokens:
                self.append(*zip(*pending))
                pending, count = [], 0
        if pending:
            self.append(*zip(*pending))

    def decode(self, lens=None, num_splits=0, max_seq_len=None, scale=None):
        d = self.d
        lens = self.lens if lens is None else np.asarray(lens)
        msl = int(lens.max()) if max_seq_len is None else max_seq_len
        out, lse = self.ops.mla_decode_lowbit(
            self.fmt, t_bf16(d.q_lat), t_bf16(d.q_rope), self.pages, self.prot, self.seq_slot,
            self.block_table, t_i32(lens), msl, d.scale if scale is None else scale,
            num_splits=num_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

    def decode_mq(self, lens=None, num_splits=0, max_seq_len=None):
        """mla_decode_lowbit_mq over the drawn query rows: [B, queries, H, ...]."""
        d = self.d
        nq, H = d.wl.queries, d.H
        lens = self.lens if lens is None else np.asarray(lens)
        msl = int(lens.max()) if max_seq_len is None else max_seq_len
        ql = t_bf16(d.q_lat).view(d.B, nq, H, 512)
        qr = t_bf16(d.q_rope).view(d.B, nq, H, 64)
        out, lse = self.ops.mla_decode_lowbit_mq(
            self.fmt, ql, qr, self.pages, self.prot, self.seq_slot, self.block_table,
            t_i32(lens), msl, d.scale, num_splits=num_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

    def fused_step(self, lens, num_splits=0, max_seq_len=None):
        """mla_decode_lowbit_append: store token lens[b]-1 of each sequence
        (lens[b] > 0) and decode over lens[b] tokens, in one call."""
        d = self.d
        lens = np.asarray(lens, dtype=np.int64)
        msl = int(lens.max()) if max_seq_len is None else max_seq_len
        # an empty sequence appends nothing: its row is never read
        lat = np.stack([d.c[b][L - 1] if L > 0 else np.zeros(512, np.uint16)
                        for b, L in enumerate(lens)])
        kr = np.stack([d.kr[b][L - 1] if L > 0 else np.zeros(64, np.uint16)
                       for b, L in enumerate(lens)])
        out, lse = self.ops.mla_decode_lowbit_append(
            self.fmt, t_bf16(lat), t_bf16(kr), t_bf16(d.q_lat), t_bf16(d.q_rope), self.pages,
            self.prot, self.seq_slot, self.block_table, t_i32(lens), msl, d.scale,
            num_splits=num_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

    def clone(self):
        """A second cache holding the same bytes (same workload)."""
        other = GpuCache.__new__(GpuCache)
        other.__dict__.update(self.__dict__)
        other.pages = self.pages.clone()
        other.prot = self.prot.clone()
        other.lens = self.lens.copy()
        return other


def oracle_decode(d, b, L, fmt=None):
    return attention.decode_sequence(d.c[b][:L], d.kr[b][:L], d.q_lat[b], d.q_rope[b],
                                     fmt or d.wl.fmt, d.scale)


def oracle_decode_mq(d, b, L, fmt=None):
    nq, H = d.wl.queries, d.H
    return attention.decode_multi(d.c[b][:L], d.kr[b][:L], d.q_lat[b].reshape(nq, H, 512),
                                  d.q_rope[b].reshape(nq, H, 64), fmt or d.wl.fmt, d.scale)


def oracle_page(d, pid, lens, fmt=None):
    """Bytes of physical page pid as the oracle writes it (zero where unused)."""
    fmt = fmt or d.wl.fmt
    page = np.zeros((1, layout.page_bytes(fmt)), np.uint8)
    hit = np.argwhere(d.block_table == pid)
    for b, blk in hit:
        L = int(lens[b])
        P = np.arange(64 * blk, min(64 * blk + 64, L))
        if len(P) == 0:
            continue
        qt = quant.quantize_tokens(d.c[b][P], d.kr[b][P], fmt)
        layout.write_tokens(page, P % 64, qt, fmt)
    return page[0]


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
