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
subnormals and all-negative lanes common.

The second mode, which the kernel switches a workgroup to when a lane's
maximum after its first tile is not positive, first maps each half to a
16-bit integer that orders as the value does; the claim there is the first
maximum of any sign, with only NaN left to the exact pass."""
import numpy as np

POS = [8 * q + jj for q in range(4) for jj in range(4)]


def _f32(bits16):
    return (np.asarray(bits16, np.uint32) << 16).view(np.float32)


def _first_max(vals16):
    v = _f32(vals16).astype(np.float64)
    return int(np.argmax(v == v.max()))


def _ord16(bits16):
    """The order-preserving map of the negative-logit mode, one 16-bit half:
    sign and magnitude become the two's complement integer +-magnitude, kept
    as its 16-bit pattern."""
    b = int(bits16)
    mag = b & 0x7FFF
    return (-mag if b & 0x8000 else mag) & 0xFFFF


def _unord_hi(word):
    """Inverse map from the high half of a word (low half zero) back to the
    bf16 pattern, in the high half."""
    o = int(np.uint32(word).view(np.int32)) >> 16
    h = (0x8000 | -o) if o < 0 else o
    return (h << 16) & 0xFFFFFFFF


def _tagged(vals16, n_valid, ord_mode=False):
    """vals16[t, k]: bf16 bits of the lane's k-th id of tile t (position
    POS[k]); ids from n_valid on are past V (masked).  With ord_mode the
    halves go through the order-preserving map first and the running best
    starts at the int32 minimum."""
    T = vals16.shape[0]
    best = np.iinfo(np.int32).min if ord_mode else \
        np.int32(np.uint32(0xFF800000).view(np.int32))   # -inf
    bidx = 0
    for t in range(T):
        m = np.iinfo(np.int32).min
        for k in range(16):
            if t * 16 + k >= n_valid:
                continue
            h = _ord16(vals16[t, k]) if ord_mode else int(vals16[t, k])
            tagged = np.int64((h << 16) | (31 - POS[k]))
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


def test_order_map_orders_every_pattern_as_its_value():
    """Over all 65536 bf16 patterns: the mapped 16-bit integers order as the
    values do (-0 and +0 equal), a NaN with the sign clear maps above +inf
    and one with the sign set below -inf, and the inverse gives back the
    pattern (+0 for -0)."""
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):      # NaN patterns widen to NaN
        vals = _f32(pats).astype(np.float64)
    mapped = np.array([_ord16(p) for p in pats], np.uint16).view(np.int16).astype(np.int64)
    fin = ~np.isnan(vals)
    order = np.argsort(vals[fin], kind="stable")
    mv = mapped[fin][order]
    vv = vals[fin][order]
    assert np.all(np.diff(mv) >= 0)
    assert np.array_equal(np.diff(mv) == 0, np.diff(vv) == 0)
    pos_nan = np.isnan(vals) & (pats < 0x8000)
    neg_nan = np.isnan(vals) & (pats >= 0x8000)
    assert mapped[pos_nan].min() > mapped[pats == 0x7F80][0]
    assert mapped[neg_nan].max() < mapped[pats == 0xFF80][0]
    for p in range(65536):
        back = _unord_hi((_ord16(p) << 16) & 0xFFFFFFFF) >> 16
        assert back == (0 if p == 0x8000 else p), hex(p)


def test_mapped_tagged_maximum_is_first_maximum_of_any_sign():
    """The negative-logit mode: with mapped halves the tagged rule gives the
    first maximum for every lane without NaN, all-negative lanes, -inf and
    signed-zero ties included; after the inverse map the kept value is the
    winner's (+0 for -0), so the check after the range flags only NaN."""
    g = np.random.Generator(np.random.PCG64(2025))
    special = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x8001, 0x3F80, 0xBF80,
                        0x7F7F, 0xFF7F], np.uint16)
    for trial in range(3000):
        T = int(g.integers(1, 5))
        kind = trial % 4
        if kind == 0:
            vals = g.choice(np.array([0xBF80, 0xC000, 0xBF00, 0x8000, 0x0000], np.uint16),
                            size=(T, 16))
        elif kind == 1:
            vals = g.choice(special, size=(T, 16))
        elif kind == 2:
            vals = (0x8000 | g.integers(0x0000, 0x7F81, size=(T, 16))).astype(np.uint16)
        else:
            vals = g.integers(0, 0x10000, size=(T, 16)).astype(np.uint16)
            nan = ((vals & 0x7F80) == 0x7F80) & ((vals & 0x007F) != 0)
            vals[nan] = 0xFF80
        n_valid = int(g.integers(1, T * 16 + 1))
        best, bidx = _tagged(vals, n_valid, ord_mode=True)
        order = sorted(range(n_valid), key=lambda i: (i // 16, POS[i % 16]))
        seq = [vals[i // 16, i % 16] for i in order]
        want_k = order[_first_max(seq)]
        assert bidx == want_k, (trial, vals, n_valid, bidx, want_k)
        kept = _unord_hi(int(np.int32(best).view(np.uint32))) >> 16
        w = int(vals[want_k // 16, want_k % 16])
        assert kept == (0 if w == 0x8000 else w)
        assert (kept & 0x7FFF) <= 0x7F80          # no NaN: no exact pass asked for
