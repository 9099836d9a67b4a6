"""Per-target digests of CSR interaction lists, formed in numpy from copied
lists (test helper).  A target's digest is its entry count and the sum
(mod 2^64) of h(s) over its sources s, h(s) the (s+1)-th output of SplitMix64
(S. Vigna) seeded with 0: order-independent, so that lists too large to hold
twice can be compared target by target with the oracle's digest-mode walk."""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix_h(src: np.ndarray) -> np.ndarray:
    z = (src.astype(np.uint64) + np.uint64(1)) * _GAMMA
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def csr_digests(off: np.ndarray, src: np.ndarray, chunk: int = 1 << 26):
    """(count, hash) per target of the CSR list (off [n+1], src [off[n]])."""
    off = np.asarray(off, dtype=np.int64)
    cnt = np.diff(off).astype(np.uint64)
    pref = np.zeros(off.shape[0], dtype=np.uint64)  # hash prefix sums at every offset
    carry = np.uint64(0)
    with np.errstate(over="ignore"):
        for c0 in range(0, int(off[-1]), chunk):
            h = splitmix_h(src[c0:c0 + chunk])
            cs = np.cumsum(h, dtype=np.uint64) + carry
            lo, hi = np.searchsorted(off, [c0 + 1, c0 + h.shape[0]], side="left")[0], \
                np.searchsorted(off, c0 + h.shape[0], side="right")
            sel = slice(lo, hi)
            pref[sel] = cs[off[sel] - c0 - 1]
            carry = cs[-1]
        return cnt, pref[1:] - pref[:-1]
