"""Compressed scale format (CSF) of the NVFP4 block scales.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "Step-5-Preview-NVFP4-Local", sections "Modifications" (item 1) and
"Format". The E4M3 block scales of a routed-expert matrix form a tensor
[E, R, C] (one byte per 16 weights; R = 1536, C = 256 for gate and up,
R = 4096, C = 96 for down). The page keeps them in three tensors, restated
here as this module uses them:

* `fixed`, bytes [E, R/16, 16 * (1 + C/2)]. Rows come in slabs of 16; a
  slab holds its 16 per-row bases first, then, row after row, that row's C
  4-bit codes packed in pairs (the even column in bits 0..3).
* `exceptions`, 32-bit words: the low 24 bits give a position row * C + col
  inside one expert, the top 8 bits the byte stored there; the words of an
  expert are contiguous and in position order.
* `starts`, int64 [E + 1]: the words of expert e are those from starts[e] up
  to, not including, starts[e + 1].

Decoding: the byte at a position listed among its expert's exceptions is
the byte stored with it; every other byte equals its row's base plus its
code (at most base + 15). Encoding chooses, per row, the smallest base in
0 .. 240 for which the 16 consecutive values from the base on contain as
many of the row's bytes as any other choice; bytes outside that range
become exceptions.

Reading where the page is silent: a position held by an exception keeps
code 0 in the fixed tensor (the decoder never uses it). Rows and columns of
an exception position are counted within the expert.
"""
import numpy as np

MAX_BASE = 240          # the last window is [240, 255]
WINDOW = 16


def row_bases(rows):
    """Base of every row of a [N, C] uint8 array: the lowest b in 0..240 whose
    window [b, b + 15] holds the most bytes of the row."""
    rows = np.asarray(rows, dtype=np.uint8)
    n, c = rows.shape
    out = np.empty(n, dtype=np.uint8)
    step = max(1, (1 << 22) // 256)             # rows per histogram block
    for r0 in range(0, n, step):
        blk = rows[r0:r0 + step].astype(np.int64)
        m = blk.shape[0]
        # hist[i, v] = how many bytes of row i equal v
        hist = np.bincount((np.arange(m)[:, None] * 256 + blk).ravel(),
                           minlength=m * 256).reshape(m, 256)
        cs = np.concatenate([np.zeros((m, 1), np.int64), np.cumsum(hist, axis=1)], axis=1)
        # covered[i, b] = bytes of row i in [b, b + 15], b = 0..240
        covered = cs[:, WINDOW:WINDOW + MAX_BASE + 1] - cs[:, 0:MAX_BASE + 1]
        out[r0:r0 + m] = np.argmax(covered, axis=1)      # first maximum = lowest base
    return out


def encode(scales):
    """scales uint8 [E, R, C] (R % 16 == 0, C even) -> (fixed, exceptions, starts)."""
    s = np.asarray(scales, dtype=np.uint8)
    E, R, C = s.shape
    assert R % 16 == 0 and C % 2 == 0 and R * C < (1 << 24)
    base = row_bases(s.reshape(E * R, C)).reshape(E, R)
    d = s.astype(np.int16) - base[:, :, None].astype(np.int16)
    inside = (d >= 0) & (d < WINDOW)
    codes = np.where(inside, d, 0).astype(np.uint8)
    packed = (codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)).astype(np.uint8)   # [E, R, C/2]
    slabs = R // 16
    fixed = np.empty((E, slabs, 16 * (1 + C // 2)), dtype=np.uint8)
    fixed[:, :, :16] = base.reshape(E, slabs, 16)
    fixed[:, :, 16:] = packed.reshape(E, slabs, 16 * (C // 2))
    exc, starts = [], [0]
    for e in range(E):
        pos = np.flatnonzero(~inside[e].ravel())                 # row-major order
        val = s[e].ravel()[pos].astype(np.uint32)
        exc.append(pos.astype(np.uint32) | (val << 24))
        starts.append(starts[-1] + pos.size)
    exceptions = np.concatenate(exc) if exc else np.zeros(0, np.uint32)
    return fixed, exceptions.astype(np.uint32), np.asarray(starts, dtype=np.int64)


def decode(fixed, exceptions, starts, R, C):
    """The scale bytes uint8 [E, R, C] the three tensors encode."""
    fixed = np.asarray(fixed, dtype=np.uint8)
    E = fixed.shape[0]
    slabs = R // 16
    assert fixed.shape == (E, slabs, 16 * (1 + C // 2))
    base = fixed[:, :, :16].reshape(E, R)
    packed = fixed[:, :, 16:].reshape(E, R, C // 2)
    codes = np.empty((E, R, C), dtype=np.uint8)
    codes[:, :, 0::2] = packed & 0xF
    codes[:, :, 1::2] = packed >> 4
    out = (base[:, :, None].astype(np.uint16) + codes).astype(np.uint8)
    exceptions = np.asarray(exceptions, dtype=np.uint32)
    for e in range(E):
        x = exceptions[int(starts[e]):int(starts[e + 1])]
        pos = (x & 0xFFFFFF).astype(np.int64)
        assert np.all(pos < R * C)
        flat = out[e].reshape(-1)
        flat[pos] = (x >> 24).astype(np.uint8)
    return out


def row_starts(exceptions, starts, E, R, C):
    """int32 [E, R+1]: entry [e, r] is the index of expert e's first
    exception at a position >= r * C (the expert's exceptions in stored
    order, which is ascending position), so row r's exceptions are
    [entry[e, r], entry[e, r+1]). A reader that keeps scales compressed
    uses it to find a row's exceptions without scanning the expert's list."""
    exceptions = np.asarray(exceptions, dtype=np.uint32)
    out = np.empty((E, R + 1), dtype=np.int32)
    for e in range(E):
        lo, hi = int(starts[e]), int(starts[e + 1])
        pos = (exceptions[lo:hi] & 0xFFFFFF).astype(np.int64)
        assert np.all(np.diff(pos) > 0), "exceptions of an expert must be in ascending position"
        out[e] = lo + np.searchsorted(pos, np.arange(R + 1, dtype=np.int64) * C, side="left")
    return out


def fixed_bytes(E, R, C):
    """Bytes of the fixed tensor: E * R/16 slabs of 16 * (1 + C/2)."""
    return E * (R // 16) * 16 * (1 + C // 2)
