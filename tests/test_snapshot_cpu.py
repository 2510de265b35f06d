"""State-snapshot files on the host (no GPU): the CRC-32C of the oracle and of
the library against published check values and each other, and the
library's reader against files built by the oracle's writer, intact and
damaged ("Kapitsa 源码拆解 05", disk-cache integrity: header and payload each
carry a CRC-32C; the reader checks identity and both checksums)."""
import os
import random

import pytest

import hybrid_linear_attention_slot_amd as gdn
from oracle.snapshot import HEADER, build_file, crc32c, parse_file

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "crc32c_check_values.txt")
VECTORS = {
    "ascii_123456789": b"123456789",
    "zeros_32": bytes(32),
    "ones_32": bytes([0xFF] * 32),
    "incrementing_32": bytes(range(32)),
    "decrementing_32": bytes(range(31, -1, -1)),
}


def golden():
    out = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, val = line.split()
            out[name] = int(val, 16)
    return out


def test_crc32c_check_values():
    g = golden()
    assert set(g) == set(VECTORS)
    for name, data in VECTORS.items():
        assert crc32c(data) == g[name], name           # the oracle
        assert gdn.gdn_crc32c(data) == g[name], name   # the library


def test_library_crc_matches_oracle_on_random_data_and_chains():
    rng = random.Random(3)
    for n in (0, 1, 7, 8, 9, 63, 64, 1000, 4099):
        data = bytes(rng.getrandbits(8) for _ in range(n))
        assert gdn.gdn_crc32c(data) == crc32c(data)
        cut = n // 3
        assert gdn.gdn_crc32c(data[cut:], gdn.gdn_crc32c(data[:cut])) == crc32c(data)


LAYOUT = (3, 64, 4, 1, 2, 16, 16, 3 * 64 * 2, 2 * 16 * 16 * 4)  # 3 GDN layers, C1 geometry


def payload(seed):
    rng = random.Random(seed)
    return bytes(rng.getrandbits(8) for _ in range(LAYOUT[0] * (LAYOUT[7] + LAYOUT[8])))


def test_reader_accepts_oracle_files(tmp_path):
    p = tmp_path / "s.bin"
    blob = build_file(0x1234, 800, LAYOUT, payload(1))
    p.write_bytes(blob)
    info = gdn.gdn_snapshot_read_info(str(p))
    fields, _ = parse_file(blob)
    for k, v in fields.items():
        assert info[k] == v, k
    assert info["payload_bytes"] == len(blob) - HEADER


@pytest.mark.parametrize("where", ["magic", "version", "key", "layout", "header_crc",
                                   "payload_first", "payload_last", "payload_crc"])
def test_reader_rejects_a_flipped_byte(tmp_path, where):
    blob = bytearray(build_file(7, 16, LAYOUT, payload(2)))
    off = {"magic": 0, "version": 8, "key": 16, "layout": 36, "header_crc": 100,
           "payload_first": HEADER, "payload_last": len(blob) - 1, "payload_crc": 96}[where]
    blob[off] ^= 0x01
    p = tmp_path / "s.bin"
    p.write_bytes(bytes(blob))
    with pytest.raises(ValueError):
        parse_file(bytes(blob))
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_snapshot_read_info(str(p))
    assert e.value.code == gdn.GDN_ECORRUPT


def test_reader_rejects_truncated_and_extended_files(tmp_path):
    blob = build_file(7, 16, LAYOUT, payload(3))
    for bad in (blob[:-1], blob[:HEADER], blob[:50], blob + b"\0"):
        p = tmp_path / "s.bin"
        p.write_bytes(bad)
        with pytest.raises(gdn.GdnError) as e:
            gdn.gdn_snapshot_read_info(str(p))
        assert e.value.code == gdn.GDN_ECORRUPT
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_snapshot_read_info(str(tmp_path / "missing.bin"))
    assert e.value.code == gdn.GDN_EIO


def test_reader_rejects_a_consistent_header_that_states_a_huge_payload(tmp_path):
    """A header with a valid checksum whose payload size does not match the
    file: rejected from the header and the file size alone (the reader must
    not try to allocate the stated 2^62 bytes)."""
    import struct
    blob = bytearray(build_file(7, 16, LAYOUT, payload(4)))
    struct.pack_into("<q", blob, 88, 1 << 62)
    struct.pack_into("<I", blob, 100, crc32c(bytes(blob[:100])))
    p = tmp_path / "s.bin"
    p.write_bytes(bytes(blob))
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_snapshot_read_info(str(p))
    assert e.value.code == gdn.GDN_ECORRUPT
    assert "truncated" in str(e.value)
