"""Sharded-state checkpoint files on the host (no GPU): CRC32C pinned to the
published iSCSI test vectors (RFC 3720, appendix B.4) and to a bit-at-a-time
reference, and save / load of host-resident shard state with every error path
(truncation, corruption, bad magic, capacity, inconsistent sizes)."""
import ctypes
import os

import numpy as np
import pytest

import sharded_state_amd as ss
from sharded_state_amd import _native as N


def _crc(b):
    buf = ctypes.create_string_buffer(bytes(b), len(b))
    return N.lib().fsdp_crc32c(buf, len(b))


def _crc_bitwise(data):
    crc = 0xFFFFFFFF
    for byte in data:
        crc ^= byte
        for _ in range(8):
            crc = (crc >> 1) ^ (0x82F63B78 if crc & 1 else 0)
    return crc ^ 0xFFFFFFFF


def test_crc32c_published_vectors():
    assert _crc(b"123456789") == 0xE3069283
    assert _crc(bytes(32)) == 0x8A9136AA
    assert _crc(bytes([0xFF] * 32)) == 0x62A8AB43
    assert _crc(bytes(range(32))) == 0x46DD794E
    assert _crc(bytes(range(31, -1, -1))) == 0x113FDB5C


def test_crc32c_matches_bitwise_reference_on_every_length():
    rng = np.random.default_rng(0)
    for n in list(range(0, 40)) + [63, 64, 65, 1000, 4099]:
        data = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
        want = _crc_bitwise(data) if n else 0
        assert _crc(data) == want, n


def _state(S, seed):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(S) * s).astype(np.float32) for s in (0.02, 1e-3, 1e-6)]


def _crc_table_ref(data):
    """CRC32C with a byte table derived from the bitwise definition (fast
    enough in Python for a few MB)."""
    table = []
    for i in range(256):
        c = i
        for _ in range(8):
            c = (c >> 1) ^ (0x82F63B78 if c & 1 else 0)
        table.append(c)
    crc = 0xFFFFFFFF
    for byte in data:
        crc = (crc >> 8) ^ table[(crc ^ byte) & 0xFF]
    return crc ^ 0xFFFFFFFF


def test_crc32c_multi_lane_path_on_large_buffers():
    """Buffers of 64 KiB and more take three interleaved hardware chains whose
    registers are combined with the zero-bytes map; lengths on both sides of
    the switch, with lane tails of every residue, must give the plain CRC."""
    rng = np.random.default_rng(5)
    assert _crc_table_ref(b"123456789") == 0xE3069283
    for n in (65535, 65536, 65537, 65536 + 23, 3 * 65536 + 7, 200003, (1 << 20) + 5):
        data = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
        assert _crc(data) == _crc_table_ref(data), n


def test_host_round_trip(tmp_path):
    numels = [1000 * 999, 999, 1]
    P, Pp, S = ss.fsdp_layout(numels, 2)
    p, m, v = _state(S, 1)
    path = ss.shard_path(str(tmp_path / "unit"), 1)
    ss.save_shard(path, numels, 2, 1, p, m, v, step=7, hp=ss.AdamWHP(lr=3e-4, weight_decay=0.1))
    assert os.path.exists(path) and not os.path.exists(path + ".tmp")
    info, sizes = ss.shard_info(path)
    assert sizes == numels
    assert (info["world"], info["rank"], info["numel"], info["padded_numel"], info["shard_numel"]) == (2, 1, P, Pp, S)
    assert info["step"] == 7 and abs(info["hp"].lr - np.float32(3e-4)) == 0 and info["hp"].weight_decay == np.float32(0.1)
    q = [np.empty(S, np.float32) for _ in range(3)]
    ss.load_shard(path, *q)
    for a, b in zip((p, m, v), q):
        assert a.tobytes() == b.tobytes()
    # payload starts at a 4096-aligned offset after the header and size table
    raw = open(path, "rb").read()
    assert len(raw) == 4096 + 3 * 4 * S


def _save(tmp_path, S=5003):
    numels = [S * 2 - 1]
    p, m, v = _state(S, 2)
    path = str(tmp_path / "u-shard0")
    ss.save_shard(path, numels, 2, 0, p, m, v, step=1, hp=ss.AdamWHP())
    return path, S


def _load_code(path, S):
    q = [np.empty(S, np.float32) for _ in range(3)]
    try:
        ss.load_shard(path, *q)
        return 0
    except ss.FsdpError as e:
        return e.code


def test_corruption_is_detected(tmp_path):
    path, S = _save(tmp_path)
    raw = bytearray(open(path, "rb").read())
    for where in (4096 + 5, len(raw) - 1, 256 + 3):          # payload, last byte, size table
        bad = bytearray(raw)
        bad[where] ^= 0x10
        open(path, "wb").write(bad)
        assert _load_code(path, S) == N.E_FORMAT, where
    open(path, "wb").write(raw[:-100])                          # truncated payload
    assert _load_code(path, S) == N.E_FORMAT
    open(path, "wb").write(raw[:100])                           # truncated header
    assert _load_code(path, S) == N.E_FORMAT
    bad = bytearray(raw)
    bad[0:8] = b"NOTSHARD"
    open(path, "wb").write(bad)
    assert _load_code(path, S) == N.E_FORMAT
    open(path, "wb").write(raw)
    assert _load_code(path, S) == 0
    assert _load_code(str(tmp_path / "missing"), S) == N.E_IO


def test_argument_errors(tmp_path):
    path, S = _save(tmp_path)
    small = [np.empty(S - 1, np.float32) for _ in range(3)]
    with pytest.raises(ss.FsdpError) as e:
        ss.load_shard(path, *small)
    assert e.value.code == N.E_SIZE
    L = N.lib()
    info = N.CkptInfo(2, 2, 10, 10, 5, N.F32, N.F32, 1, N.AdamWHP(), 1)        # rank out of range
    assert L.fsdp_save_shard(str(tmp_path / "x").encode(), ctypes.byref(info), N.i64_array([10]),
                             None, None, None, 0, None) == N.E_INVAL
    info = N.CkptInfo(2, 0, 10, 12, 5, N.F32, N.F32, 1, N.AdamWHP(), 1)        # padded / shard inconsistent
    assert L.fsdp_save_shard(str(tmp_path / "x").encode(), ctypes.byref(info), N.i64_array([10]),
                             None, None, None, 0, None) == N.E_SIZE
    info = N.CkptInfo(2, 0, 10, 10, 5, N.F32, N.F32, 1, N.AdamWHP(), 1)
    assert L.fsdp_save_shard(str(tmp_path / "x").encode(), ctypes.byref(info), N.i64_array([9]),
                             None, None, None, 0, None) == N.E_SIZE                # sizes do not sum to numel
    assert L.fsdp_save_shard(str(tmp_path / "no" / "dir" / "x").encode(), ctypes.byref(info),
                             N.i64_array([10]), None, None, None, 0, None) in (N.E_INVAL, N.E_IO)


def test_every_header_and_table_byte_is_checked(tmp_path):
    """A flipped bit anywhere in the 256-byte header (its own checksum covers
    it) or the size table makes the file unreadable, never a silently different
    step, hyper-parameter or size; bytes of the unused gap between the table and
    the 4096-aligned payload change nothing.  Runs through both the header query
    and the load."""
    path, S = _save(tmp_path, S=2053)
    raw = bytearray(open(path, "rb").read())
    table_end = 256 + 8 * 1
    for where in list(range(0, table_end)) + [table_end, 1000, 4095]:
        for bit in (0x01, 0x80):
            bad = bytearray(raw)
            bad[where] ^= bit
            open(path, "wb").write(bad)
            code = _load_code(path, S)
            if where < table_end:
                assert code == N.E_FORMAT, (where, bit)
                with pytest.raises(ss.FsdpError) as e:
                    ss.shard_info(path)
                assert e.value.code == N.E_FORMAT
            else:
                assert code == 0, (where, bit)      # padding before the payload is not data
    open(path, "wb").write(raw)
    assert _load_code(path, S) == 0


def test_payload_flips_and_truncations_at_every_boundary(tmp_path):
    """Payload flips (first, middle and last byte of each of the three state
    shards) fail the payload checksum; a file cut at any length short of the
    whole, or with bytes appended, fails before anything is read into the
    destinations' full size."""
    path, S = _save(tmp_path, S=1031)
    raw = bytes(open(path, "rb").read())
    sb = 4 * S
    for k in range(3):
        for off in (0, sb // 2, sb - 1):
            bad = bytearray(raw)
            bad[4096 + k * sb + off] ^= 0x04
            open(path, "wb").write(bad)
            assert _load_code(path, S) == N.E_FORMAT, (k, off)
    cuts = sorted(set(list(range(0, 300, 7)) + [255, 256, 257, 263, 264, 265, 4095, 4096, 4097, 4096 + sb,
                                                  4096 + 2 * sb + 1, len(raw) - 8, len(raw) - 1]))
    for n in cuts:
        open(path, "wb").write(raw[:n])
        assert _load_code(path, S) == N.E_FORMAT, n
    open(path, "wb").write(raw + b"\0" * 8)
    assert _load_code(path, S) == N.E_FORMAT
    open(path, "wb").write(raw)
    assert _load_code(path, S) == 0


def test_a_consistently_forged_header_cannot_make_the_reader_allocate(tmp_path):
    """A header rewritten with a huge tensor count and a matching header
    checksum still fails: the table must lie inside the file."""
    import struct
    path, S = _save(tmp_path, S=515)
    raw = bytearray(open(path, "rb").read())
    # n_tensors sits after the five hyper-parameter floats; recompute the header's checksum
    off = 8 + 4 + 4 + 4 + 4 + 8 * 3 + 4 + 4 + 8 + 4 * 5
    for n in (1 << 30, (1 << 31) - 1):
        bad = bytearray(raw)
        bad[off:off + 4] = struct.pack("<i", n)
        bad[112:116] = b"\0\0\0\0"
        bad[112:116] = struct.pack("<I", _crc(bytes(bad[:256])))
        open(path, "wb").write(bad)
        assert _load_code(path, S) == N.E_FORMAT, n
        assert "payload layout" in N.lib().fsdp_last_error().decode()


def test_large_shard_read_in_parts(tmp_path):
    """A state shard of several 4 MB parts is read and checksummed by several
    workers whose registers are folded in file order: the round trip is exact,
    the whole-file checksum equals the plain CRC32C of the payload bytes, and a
    flipped byte in any part (first, a middle one, the last) is caught."""
    S = 3 * (1 << 20) + 517                       # 12 MB of fp32 per state buffer: three parts and a tail
    numels = [2 * S - 1]
    p, m, v = _state(S, 9)
    path = str(tmp_path / "big-shard1")
    ss.save_shard(path, numels, 2, 1, p, m, v, step=3, hp=ss.AdamWHP())
    raw = bytes(open(path, "rb").read())
    payload = raw[4096:]
    assert payload == p.tobytes() + m.tobytes() + v.tobytes()
    import struct
    assert struct.unpack("<I", raw[108:112])[0] == _crc(payload)    # crc_payload field
    q = [np.empty(S, np.float32) for _ in range(3)]
    ss.load_shard(path, *q)
    for a, b in zip((p, m, v), q):
        assert a.tobytes() == b.tobytes()
    sb = 4 * S
    for off in (0, 5 << 20, sb + (9 << 20), 3 * sb - 1):
        bad = bytearray(raw)
        bad[4096 + off] ^= 0x20
        open(path, "wb").write(bad)
        assert _load_code(path, S) == N.E_FORMAT, off
    open(path, "wb").write(raw)
    assert _load_code(path, S) == 0
