"""Host-side (numpy) model of the FP6 operand-tile layout of include/rotw4a4.h.

Test plumbing, not method arithmetic: it converts integer codes to the tile
bytes the HIP path reads and writes, and back, so that tests can compare tiles
with the oracle's integer codes. The E2M3 code of an integer is found by
decoding all 64 six-bit patterns with the OCP FP6 E2M3 definition (sign bit 5,
exponent bits 4..3 with bias 1, mantissa bits 2..0, subnormals at exponent 0)
and picking the one whose value is that integer.
"""
import numpy as np

TILE = 1536
PLANE1 = 1024


def e2m3_value(code: int) -> float:
    s = -1.0 if code & 32 else 1.0
    e = (code >> 3) & 3
    m = code & 7
    if e == 0:
        return s * (m / 8.0)                       # 2^(1 - bias) * 0.m, bias 1
    return s * (2.0 ** (e - 1)) * (1.0 + m / 8.0)


def _encode_table():
    enc = {}
    for c in range(64):
        v = e2m3_value(c)
        if v == int(v) and -7 <= v <= 7 and int(v) not in enc and not (v == 0 and c & 32):
            enc[int(v)] = c
    return enc


ENC = _encode_table()          # integer -> E2M3 code (positive zero for 0)


def rows_padded(R: int) -> int:
    return (R + 255) // 256 * 256


def tiles_size(R: int, K: int) -> int:
    return rows_padded(R) * K * 3 // 4


def _lane_index(R: int, K: int):
    """for every (row, k): byte offset of its lane's two planes and its field index e"""
    KT = K // 64
    rows, ks = np.meshgrid(np.arange(R), np.arange(K), indexing="ij")
    t = (rows // 32) * KT + ks // 64
    lane = 32 * ((ks % 64) // 32) + rows % 32
    return t * TILE, lane, ks % 32


def _lane_bytes_offsets(tbase, lane):
    """byte offsets of the 24 bytes of a lane's 192-bit string: 16 in plane 0, 8 in plane 1"""
    j = np.arange(24)
    return np.where(j < 16, tbase[..., None] + lane[..., None] * 16 + j,
                    tbase[..., None] + PLANE1 + lane[..., None] * 8 + (j - 16))


def tile(q: np.ndarray) -> np.ndarray:
    """int codes [R][K] in [-7, 7] -> tile bytes (uint8, tiles_size(R, K))."""
    R, K = q.shape
    assert K % 64 == 0
    Rp = rows_padded(R)
    qp = np.zeros((Rp, K), np.int64)
    qp[:R] = q
    f = np.vectorize(ENC.__getitem__)(qp).astype(np.uint64)
    tbase, lane, e = _lane_index(Rp, K)
    # one 192-bit string per (tile, lane) = three uint64 words; field e at bit 6e
    slot = (tbase // TILE) * 64 + lane
    words = np.zeros((slot.max() + 1, 3), np.uint64)
    b = (6 * e).ravel()
    w = b // 64
    sh = (b % 64).astype(np.uint64)
    v = f.ravel()
    sl = slot.ravel()
    np.bitwise_or.at(words, (sl, w), v << sh)
    spill = (b % 64) > 58
    np.bitwise_or.at(words, (sl[spill], w[spill] + 1), v[spill] >> (np.uint64(64) - sh[spill]))
    lane_bytes = words.view(np.uint8).reshape(-1, 24)                # little-endian 192 bits
    out = np.zeros(Rp * K * 3 // 4, np.uint8)
    nslots = lane_bytes.shape[0]
    st = np.arange(nslots)
    offs = _lane_bytes_offsets((st // 64) * TILE, st % 64)
    out[offs.ravel()] = lane_bytes.ravel()
    return out


def untile(b: np.ndarray, R: int, K: int) -> np.ndarray:
    """tile bytes -> int codes [R][K] (rows below R only)."""
    DEC = {c: int(e2m3_value(c)) for c in range(64) if e2m3_value(c) == int(e2m3_value(c))}
    b = np.asarray(b, np.uint8)[: tiles_size(R, K)]
    nslots = len(b) // TILE * 64
    st = np.arange(nslots)
    offs = _lane_bytes_offsets((st // 64) * TILE, st % 64)
    words = b[offs].copy().view(np.uint64).reshape(-1, 3)           # [slot][3]
    tbase, lane, e = _lane_index(R, K)
    sl = (tbase // TILE) * 64 + lane
    bit = 6 * e
    w = bit // 64
    sh = (bit % 64).astype(np.uint64)
    v = words[sl, w] >> sh
    spill = (bit % 64) > 58
    nxt = words[sl, np.minimum(w + 1, 2)] << (np.uint64(64) - np.where(spill, sh, np.uint64(1)))
    v = np.where(spill, v | nxt, v)
    codes = (v & np.uint64(63)).astype(np.int64)
    lut = np.zeros(64, np.int64)
    valid = np.zeros(64, bool)
    for c, val in DEC.items():
        lut[c] = val
        valid[c] = True
    assert valid[codes].all(), "tile holds a six-bit pattern that is not an integer in [-7, 7]"
    return lut[codes]
