"""Independent formulation of the range coder with unbounded Python integers.

Test-only. The oracle's coder keeps a 32-bit window of the low end of the code
interval and pushes carries back into the bytes already written. This version
keeps the whole low end as one integer (scaled by 2^(32+8k) after k byte
shifts), so it needs no window and no carry handling. The interval widths are
identical in both formulations, because the width never depends on the low
end. If the two agree byte for byte, the oracle's carry and flush logic is
right.

It also returns every nested interval, so a test can check that the value of
the emitted bytes lies inside all of them.
"""

from __future__ import annotations

import math

TOP = 1 << 24


def encode(symbols, cdf):
    """Return (bytes, intervals, shifts_per_symbol)."""
    lo = 0
    width = (1 << 32) - 1
    k = 0
    intervals = []
    shifts = []
    for s in symbols:
        r = width >> 16
        lo += r * cdf[s]
        width = r * (cdf[s + 1] - cdf[s])
        n = 0
        while width < TOP:
            lo <<= 8
            width <<= 8
            k += 1
            n += 1
        shifts.append(n)
        intervals.append((lo, width, k))
    # Smallest multiple of 2^24 at the final scale that is >= lo.
    v = -(-lo // TOP) * TOP
    assert v < (1 << (32 + 8 * k)), "code value escaped [0, 1)"
    full = v.to_bytes(4 + k, "big")
    out = full[: k + 1]
    if out and out[-1] == 0 and len(out) == k + 1:
        out = out[:k]
    return bytes(out), intervals, shifts, v, k


def value_in_all_intervals(v, k, intervals):
    for lo, width, ki in intervals:
        scale = 1 << (8 * (k - ki))
        if not (lo * scale <= v < (lo + width) * scale):
            return False
    return True


def information_bits(symbols, cdf):
    """I_q = sum of -log2(freq(s) / 2^16) over the stream."""
    return sum(-math.log2((cdf[s + 1] - cdf[s]) / 65536.0) for s in symbols)
