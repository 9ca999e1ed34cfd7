"""Dropout of the attention probabilities with a counter-based random mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GS] section 1 computes the operator without dropout, and section 6 adds that
with training dropout the backward recomputation has to reproduce the very
mask the forward drew, together with its scaling.  A counter-based generator
makes that possible without storing the mask: the random bits of element
(b, h, i, j) are a pure function of a seed and the element's coordinates.

Generator: Philox4x32-10 as defined by Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011), section 4: a 128-bit
counter (four 32-bit words) and a 64-bit key (two words) go through ten
rounds; each round multiplies counter words 0 and 2 by the constants
0xD2511F53 and 0xCD9E8D57 into 64-bit products, and the new counter is
(hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); between
rounds the key is bumped by the Weyl constants 0x9E3779B9 and 0xBB67AE85
(all arithmetic mod 2^32).

The mask layout is a convention of this library (the pages fix none; it is
stated the same way in the C header):

* key     = (seed mod 2^32, seed div 2^32)
* counter = (i, j div 64, b*H + h, (j div 4) mod 4)
* the output words x0..x3 hold 16 bytes; key j takes byte (j mod 4) of word
  ((j div 16) mod 4), i.e. (x_w >> 8*(j mod 4)) & 0xff
* element (i, j) is kept iff that byte < T, where T = keep_256 in 1..256 is
  the number of byte values kept (keep probability T/256); kept
  probabilities are multiplied by 256/T, so that the expectation of the
  dropped output is the undropped output.

Reading: dropout acts on the normalised probabilities P (after the softmax,
before the product with V); the denominator l and the log-sum-exp are those
of the undropped softmax, which is what the backward needs to rebuild P.
"""

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32_10(counter, key):
    """Philox4x32-10 on arrays: counter [..., 4] and key [..., 2] (uint32,
    broadcastable).  Returns the four output words [..., 4] as uint32."""
    counter = np.asarray(counter, dtype=np.uint32)
    key = np.asarray(key, dtype=np.uint32)
    c0, c1, c2, c3 = (counter[..., n] for n in range(4))
    k0, k1 = key[..., 0], key[..., 1]
    with np.errstate(over="ignore"):
        for rnd in range(10):
            p0 = c0.astype(np.uint64) * _M0
            p1 = c2.astype(np.uint64) * _M1
            hi0, lo0 = (p0 >> _SH).astype(np.uint32), (p0 & _LO).astype(np.uint32)
            hi1, lo1 = (p1 >> _SH).astype(np.uint32), (p1 & _LO).astype(np.uint32)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            if rnd < 9:
                k0 = (k0 + _W0).astype(np.uint32)
                k1 = (k1 + _W1).astype(np.uint32)
    return np.stack(np.broadcast_arrays(c0, c1, c2, c3), axis=-1)


def seed_key(seed):
    """The Philox key (two words) of a 64-bit seed."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)


def dropout_bytes(bh, row_ids, nk, seed):
    """The random byte of every element (i, j), i in ``row_ids``, j < nk, of
    head ``bh`` = b*H + h: uint8 [len(row_ids), nk]."""
    rows = np.asarray(row_ids, dtype=np.int64).reshape(-1)
    j = np.arange(nk, dtype=np.int64)
    ctr = np.zeros((rows.size, nk, 4), dtype=np.uint32)
    ctr[..., 0] = rows[:, None]
    ctr[..., 1] = (j >> 6)[None, :]
    ctr[..., 2] = int(bh)
    ctr[..., 3] = ((j >> 2) & 3)[None, :]
    words = philox4x32_10(ctr, seed_key(seed))          # [R, nk, 4]
    w = np.take_along_axis(words, ((j >> 4) & 3)[None, :, None].repeat(rows.size, 0), axis=2)[..., 0]
    return ((w >> (8 * (j & 3)).astype(np.uint32)[None, :]) & 0xFF).astype(np.uint8)


def keep_mask(bh, row_ids, nk, seed, keep_256):
    """Boolean [len(row_ids), nk]: True where element (i, j) is kept."""
    t = int(keep_256)
    if not 1 <= t <= 256:
        raise ValueError("keep_256 must lie in 1..256")
    return dropout_bytes(bh, row_ids, nk, seed).astype(np.int64) < t


def keep_scale(keep_256):
    """Factor applied to kept probabilities: 256 / keep_256."""
    return 256.0 / float(keep_256)
