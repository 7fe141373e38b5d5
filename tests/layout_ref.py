"""Independent reader of the packed layout described in include/moe_decode.h.

Written from the header's description only (no library code), so that the
library's packer and its GPU generator can be checked against it. Used by
tests only."""

from __future__ import annotations

import numpy as np

GROUP = 64


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


def row_bytes(bits: int, cols: int) -> int:
    return 4 * ((cols + 9) // 10) if bits == 3 else cols * bits // 8


def codes_bytes(bits: int, rows: int, cols: int) -> int:
    return _align(row_bytes(bits, cols) * rows)


def matrix_bytes(bits: int, rows: int, cols: int) -> int:
    return codes_bytes(bits, rows, cols) + _align(rows * (cols // GROUP) * 4)


def unpack(bits: int, rows: int, cols: int, buf: np.ndarray):
    """-> codes uint8 [rows, cols], scale bits uint16 [rows, cols/64], bias bits uint16."""
    buf = np.asarray(buf, dtype=np.uint8)
    rb = row_bytes(bits, cols)
    raw = buf[: rb * rows].reshape(rows, rb)
    if bits == 8:
        codes = raw.copy()
    elif bits == 4:
        codes = np.stack([raw & 15, raw >> 4], axis=-1).reshape(rows, cols)
    elif bits == 2:
        codes = np.stack([(raw >> s) & 3 for s in (0, 2, 4, 6)], axis=-1).reshape(rows, cols)
    elif bits == 6:
        # unit of 16 codes in dwords A, B, C; code c = j + 8h in half h:
        # j 0,1 / 3,4 / 6,7: 6 bits at A / B / C bit 6*(j mod 3); j 2 / 5: low
        # nibble at A / B bit 12, high 2 bits at C bit 12 / 14
        w = raw.view(np.uint32).reshape(rows, cols // 16, 3).astype(np.uint64)
        codes = np.zeros((rows, cols // 16, 16), dtype=np.uint8)

        def field(word, bit, n):
            return (w[..., word] >> np.uint64(bit)) & np.uint64((1 << n) - 1)

        for c in range(16):
            h, j = 16 * (c // 8), c % 8
            if j in (2, 5):
                v = field(j // 3, h + 12, 4) | (field(2, h + 12 + 2 * (j // 5), 2) << np.uint64(4))
            else:
                v = field(j // 3, h + 6 * (j % 3), 6)
            codes[..., c] = v.astype(np.uint8)
        codes = codes.reshape(rows, cols)
    elif bits == 3:
        # 10 codes per dword: slot l < 5 at bit 3l, slot l >= 5 at bit 16 + 3(l - 5)
        w = raw.view(np.uint32).astype(np.uint64)
        j = np.arange(cols)
        l = j % 10
        pos = np.where(l < 5, 3 * l, 16 + 3 * (l - 5)).astype(np.uint64)
        codes = ((w[:, j // 10] >> pos) & np.uint64(7)).astype(np.uint8)
        # spare bits (15 and 31) must be zero
        assert np.all(w & np.uint64(0x80008000) == 0)
    else:
        raise ValueError(bits)
    sb = buf[codes_bytes(bits, rows, cols): codes_bytes(bits, rows, cols) + rows * (cols // GROUP) * 4]
    sb = sb.view(np.uint32).reshape(rows, cols // GROUP)
    return codes, (sb & 0xFFFF).astype(np.uint16), (sb >> 16).astype(np.uint16)


def layer_offsets(hidden, n_experts, inter, shared_inter, router_bits, expert_bits, shared_bits, **_):
    """Offsets of the layer block parts, as the header describes them."""
    off = {}
    o = 0
    off["router"] = o
    o += _align(n_experts * hidden * 2) if router_bits == 16 else matrix_bytes(router_bits, n_experts, hidden)
    off["gatevec"] = o
    o += _align(hidden * 2)
    off["shared"] = o
    g = matrix_bytes(shared_bits, shared_inter, hidden)
    off["shared_up"], off["shared_down"] = g, 2 * g
    o += 2 * g + matrix_bytes(shared_bits, hidden, shared_inter)
    off["expert0"] = o
    g = matrix_bytes(expert_bits, inter, hidden)
    off["expert_up"], off["expert_down"] = g, 2 * g
    off["expert_stride"] = 2 * g + matrix_bytes(expert_bits, hidden, inter)
    o += off["expert_stride"] * n_experts
    off["total_bytes"] = o
    return off


def unpack_ffn(buf: np.ndarray, bits: int, hidden: int, inter: int):
    """gate/up/down (codes, scale bits, bias bits) of one expert block."""
    g = matrix_bytes(bits, inter, hidden)
    return {
        "gate": unpack(bits, inter, hidden, buf[:g]),
        "up": unpack(bits, inter, hidden, buf[g:2 * g]),
        "down": unpack(bits, hidden, inter, buf[2 * g:]),
    }
