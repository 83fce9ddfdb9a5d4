"""Host-side check of the tagged-maximum rule that the 8-wave epilogue of
the readout with in-place bias uses, written out here in numpy.

Each lane sees its row's ids in tiles of 32, holding 16 of them per tile at
positions 8q + jj (q, jj in 0..3).  A rounded sum widened to fp32 has 16
zero low bits; the rule puts 31 - position there, takes the signed integer
maximum over the tile, compares the tile's maximum with its tag cleared
against the running one (strictly, so a later tile never wins a tie), and
asks for the exact compare-and-select pass whenever the lane's final
maximum is not above +0.  Claim: when no exact pass is asked for, the
result is the first maximum under real-number comparison (-0 equal to +0).
Checked on random lanes drawn to make ties, signed zeros, infinities,
subnormals and all-negative lanes common."""
import numpy as np

POS = [8 * q + jj for q in range(4) for jj in range(4)]


def _f32(bits16):
    return (np.asarray(bits16, np.uint32) << 16).view(np.float32)


def _first_max(vals16):
    v = _f32(vals16).astype(np.float64)
    return int(np.argmax(v == v.max()))


def _tagged(vals16, n_valid):
    """vals16[t, k]: bf16 bits of the lane's k-th id of tile t (position
    POS[k]); ids from n_valid on are past V (masked)."""
    T = vals16.shape[0]
    best = np.int32(np.uint32(0xFF800000).view(np.int32))   # -inf
    bidx = 0
    for t in range(T):
        m = np.iinfo(np.int32).min
        for k in range(16):
            if t * 16 + k >= n_valid:
                continue
            tagged = np.int64((int(vals16[t, k]) << 16) | (31 - POS[k]))
            tagged = int(np.int64(tagged).astype(np.uint32).view(np.int32))
            m = max(m, tagged)
        mv = int(np.uint32(np.int64(m) & 0xFFFF0000).view(np.int32))
        if mv > best:
            best = mv
            bidx = t * 16 + POS.index(31 - (int(np.int64(m) & 0xFFFF)))
    return best, bidx


def test_tagged_maximum_is_first_maximum_unless_flagged():
    g = np.random.Generator(np.random.PCG64(2024))
    special = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x8001, 0x3F80, 0xBF80,
                        0x7F7F, 0xFF7F], np.uint16)
    flagged = exact = 0
    for trial in range(3000):
        T = int(g.integers(1, 5))
        kind = trial % 4
        if kind == 0:      # few distinct values: many ties
            vals = g.choice(np.array([0x3F80, 0x4000, 0x3F00, 0xBF80], np.uint16), size=(T, 16))
        elif kind == 1:    # special values
            vals = g.choice(special, size=(T, 16))
        elif kind == 2:    # all negative
            vals = (0x8000 | g.integers(0x0001, 0x7F80, size=(T, 16))).astype(np.uint16)
        else:              # anything finite or infinite, no NaN
            vals = g.integers(0, 0x10000, size=(T, 16)).astype(np.uint16)
            nan = ((vals & 0x7F80) == 0x7F80) & ((vals & 0x007F) != 0)
            vals[nan] = 0x7F80
        n_valid = int(g.integers(1, T * 16 + 1))
        best, bidx = _tagged(vals, n_valid)
        # ids in ascending order: tile, then position
        order = sorted(range(n_valid), key=lambda i: (i // 16, POS[i % 16]))
        seq = [vals[i // 16, i % 16] for i in order]
        want_k = order[_first_max(seq)]
        if best <= 0:
            flagged += 1
            continue
        exact += 1
        assert bidx == want_k, (trial, vals, n_valid, bidx, want_k)
        # and the kept value is that id's value
        assert best == int(np.uint32(int(vals[want_k // 16, want_k % 16]) << 16).view(np.int32))
    assert flagged > 300 and exact > 1000, (flagged, exact)


def test_every_non_positive_maximum_is_flagged():
    """Lanes whose true maximum is +0, -0, negative or -inf always ask for
    the exact pass (the tag orders those wrongly)."""
    g = np.random.Generator(np.random.PCG64(7))
    for trial in range(2000):
        T = int(g.integers(1, 4))
        vals = (0x8000 | g.integers(0, 0x7F81, size=(T, 16))).astype(np.uint16)
        if trial % 3 == 0:
            vals[g.integers(0, T), g.integers(0, 16)] = 0x0000
        best, _ = _tagged(vals, T * 16)
        assert best <= 0
