"""Plain reference of the state-snapshot file: CRC-32C and the byte layout.

TEST INFRASTRUCTURE ONLY (imported by tests/, never by the product package);
shares no code with the library's C++ snapshot writer / reader.

CRC-32C is computed bit by bit from its definition (the Castagnoli polynomial
0x1EDC6F41, processed reflected as 0x82F63B78, initial value and final xor
0xFFFFFFFF); the published check values pin it (tests).  The file layout is
the one gdn_snapshot.h documents: a 128-byte little-endian header (magic,
version, key, position, the state layout, region sizes, payload size, the
payload's and the header's CRC-32C) followed by, per GDN layer, the window
bytes then the state bytes of the slot.  The page ("Kapitsa 源码拆解 05",
disk-cache integrity section) fixes the principle: header and payload each
carry a CRC-32C, and the reader checks identity and both checksums.
"""
from __future__ import annotations

import struct

MAGIC = b"GDNSTAT1"
HEADER = 128


def crc32c(data: bytes, crc: int = 0) -> int:
    c = crc ^ 0xFFFFFFFF
    for byte in data:
        c ^= byte
        for _ in range(8):
            c = (c >> 1) ^ (0x82F63B78 if c & 1 else 0)
    return c ^ 0xFFFFFFFF


def build_file(key, position, layout, payload: bytes) -> bytes:
    """layout: (layers, C, W, Hk, Hv, dk, dv, window_bytes, state_bytes)."""
    nl, C, W, Hk, Hv, dk, dv, win, st = layout
    assert len(payload) == nl * (win + st)
    h = bytearray(HEADER)
    struct.pack_into("<8sIIQq9iIqqqI", h, 0, MAGIC, 1, HEADER, key, position,
                     nl, C, W, Hk, Hv, dk, dv, 1, 2, 0, win, st, len(payload), crc32c(payload))
    struct.pack_into("<I", h, 100, crc32c(bytes(h[:100])))
    return bytes(h) + payload


def parse_file(blob: bytes):
    """Returns (fields dict, payload) or raises ValueError for a damaged file."""
    if len(blob) < HEADER or blob[:8] != MAGIC:
        raise ValueError("not a snapshot")
    (magic, version, hbytes, key, position, nl, C, W, Hk, Hv, dk, dv, sdt, wdt, _z, win, st,
     payload_bytes, payload_crc) = struct.unpack_from("<8sIIQq9iIqqqI", blob, 0)
    (header_crc,) = struct.unpack_from("<I", blob, 100)
    if version != 1 or hbytes != HEADER or header_crc != crc32c(blob[:100]):
        raise ValueError("bad header")
    payload = blob[HEADER:]
    if len(payload) != payload_bytes or crc32c(payload) != payload_crc:
        raise ValueError("bad payload")
    return dict(key=key, position=position, num_linear_layers=nl, conv_channels=C,
                conv_width=W, num_k_heads=Hk, num_v_heads=Hv, head_k_dim=dk, head_v_dim=dv,
                window_bytes=win, state_bytes=st, payload_bytes=payload_bytes,
                payload_crc=payload_crc), payload
