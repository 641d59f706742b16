"""Pins for the oracle's formats, relayout and reconstruction.

Sources ("mlx-iqk" package description, page 1):
  * "Format" section, stream tables for IQ2_KS / IQ2_K / IQ1_S_R4 and the two
    reconstruction formulas, every step in float32;
  * "Format" section, row budgets 2 + 70n/256, 76n/256, 2 + 6n/32 bytes and
    the IQ1_S_R4 wire in whole four-row groups;
  * introduction: bits per weight 2.1875 (+16-bit row scale), 2.375,
    1.5 (+16-bit row scale); the relayout changes no reconstructed value and
    no stored byte budget.

Pins used here, none of which re-types the oracle's own formula:
  * hand-assembled wire blocks with hand-computed literal outputs;
  * byte budgets and bits per weight as literals;
  * relayout = a bit permutation (single-bit tracing) and exact round trips;
  * two independent decoders (wire and streams) agree field by field;
  * exact closed forms: for small-integer tables and fp16 scales every
    float32 product is exact, so the expected value is the exact product
    (checked to be representable) and the sign of zero follows IEEE's XOR
    rule;
  * the order of the two float32 multiplies: each product of two float32 is
    exact in double, so one correctly rounded float32 conversion per step
    gives the IEEE result of (d*s)*v, which differs from d*(s*v) on some of
    the sampled cases.
"""
import os

import numpy as np
import pytest

import oracle
import synth

KS, K, R4 = oracle.IQ2_KS, oracle.IQ2_K, oracle.IQ1_S_R4


# --------------------------------------------------------------------------
# sizes (P2)
# --------------------------------------------------------------------------

def test_row_budgets_and_bits_per_weight():
    # the pages' budgets and bits per weight (tests/golden/format_budgets.txt, cited there)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "format_budgets.txt")
    members = {"IQ2_KS": KS, "IQ2_K": K, "IQ1_S_R4": R4}
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(rows) == 12
    for name, n, rb, scale_bits, bpw in rows:
        fmt, n, rb = members[name], int(n), int(rb)
        assert oracle.row_bytes(fmt, n) == rb
        assert (rb * 8 - int(scale_bits)) / n == float(bpw)
    # invalid shapes are refused
    assert oracle.row_bytes(KS, 100) == -1
    assert oracle.tensor_bytes(R4, 6, 256) == -1
    # a routed gate/up expert (2048 rows x 4096) in each member
    assert oracle.tensor_bytes(KS, 2048, 4096) == 2_297_856
    assert oracle.tensor_bytes(K, 2048, 4096) == 2_490_368
    assert oracle.tensor_bytes(R4, 2048, 4096) == 1_576_960


# --------------------------------------------------------------------------
# hand-computed blocks (P1)
# --------------------------------------------------------------------------

def _f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_iq2ks_hand_block_all_same():
    # one row, n = 256: d = 0.5, scale index bits all zero (-> -16 under the
    # offset-16 reading), alphabet bit 1 everywhere, every code 3
    wire = np.zeros(72, np.uint8)
    wire[0:2] = [0x00, 0x38]            # fp16 0.5
    wire[2:4] = [0xFF, 0x00]            # extra: alphabet bits 0-7 set, high scale bits clear
    wire[4:8] = 0x00                    # low scale nibbles
    wire[8:72] = 0xFF                   # all codes 3
    values = np.array([1, 2, 3, 4, 5, 6, 7, 13], np.float32)
    s = oracle.pack(KS, wire, 1, 256)
    w = oracle.dequant(KS, s, 1, 256, values)
    assert np.all(w == -104.0)          # (0.5 * -16) * 13


def test_iq2ks_hand_block_single_code_position():
    # d = 1, every sub-block's 5-bit raw scale = 17 (-> si = 1), alphabet 0,
    # every code 0 except block weight j = 128*1 + 32*2 + 5 = 197 (code 2)
    wire = np.zeros(72, np.uint8)
    wire[0:2] = [0x00, 0x3C]            # fp16 1.0
    wire[2:4] = [0x00, 0xFF]            # extra: high scale bits of all 8 sub-blocks
    wire[4:8] = 0x11                    # low nibbles 1
    wire[8 + 32 + 5] = 0b10 << 4        # qs byte 32h + l, bits 2p (h=1, p=2, l=5)
    values = np.array([10, 20, 30, 40, 50, 60, 70, 80], np.float32)
    s = oracle.pack(KS, wire, 1, 256)
    expected_streams = np.zeros(72, np.uint8)
    expected_streams[49] = 0x08         # weight 197 -> qs byte 49, bits 2..3
    expected_streams[64:68] = 0x11      # scl plane
    expected_streams[68] = 0xFF         # sch plane
    expected_streams[69] = 0x00         # sex plane
    expected_streams[70:72] = [0x00, 0x3C]
    assert np.array_equal(s, expected_streams)
    w = oracle.dequant(KS, s, 1, 256, values)
    exp = np.full(256, 10.0, np.float32)
    exp[197] = 30.0
    assert np.array_equal(w[0], exp)


def test_iq2ks_zero_scale_keeps_ieee_sign():
    # raw scale 16 -> si = 0: (d * +0.0) * v has the sign of d times the sign of v
    wire = np.zeros(72, np.uint8)
    wire[0:2] = [0x00, 0x3C]            # +1.0
    wire[2:4] = [0x00, 0xFF]            # high bits set, low nibbles 0 -> raw 16
    values = np.array([-3, 2, 5, -7, 1, 1, 1, 1], np.float32)
    wire[8:72] = 0b11100100             # codes 0,1,2,3 in each byte
    w = oracle.dequant(KS, oracle.pack(KS, wire, 1, 256), 1, 256, values)
    assert np.all(w == 0.0)
    # weight 128h + 32p + l has code p: signs of values[p]
    p = (np.arange(256) % 128) // 32
    expect_neg = np.array([True, False, False, True])[p]
    assert np.array_equal(np.signbit(w[0]), expect_neg)


def test_iq2k_hand_blocks():
    # one row, n = 512 (two 76-byte blocks)
    wire = np.zeros(152, np.uint8)
    # block 0: d = 1.0, all alphabet bits 1, scales 0x98 (even sub-block nibble 8 -> 0, odd 9 -> 1),
    # codes all 1
    wire[0:2] = [0x00, 0x3C]
    wire[2:4] = [0xFF, 0xFF]
    wire[4:12] = 0x98
    wire[12:76] = 0x55
    # block 1: d = -2.0, alphabet 0, scales 0x0F (even nibble 15 -> 7, odd 0 -> -8), codes all 2
    wire[76:78] = [0x00, 0xC0]
    wire[78:80] = [0x00, 0x00]
    wire[80:88] = 0x0F
    wire[88:152] = 0xAA
    values = np.array([1, 2, 3, 4, 5, 6, 7, 8], np.float32)
    w = oracle.dequant(K, oracle.pack(K, wire, 1, 512), 1, 512, values)[0]
    sb = np.arange(512) // 16
    exp = np.empty(512, np.float32)
    b0 = np.arange(512) < 256
    exp[b0 & (sb % 2 == 0)] = 0.0       # (1 * 0) * 6
    exp[b0 & (sb % 2 == 1)] = 6.0       # (1 * 1) * 6
    exp[~b0 & (sb % 2 == 0)] = -42.0    # (-2 * 7) * 3
    exp[~b0 & (sb % 2 == 1)] = 48.0     # (-2 * -8) * 3
    assert np.array_equal(w, exp)
    assert not np.any(np.signbit(w[b0 & (sb % 2 == 0)]))


def test_iq2k_hand_block_stream_bytes():
    # one row, n = 256 (one 76-byte wire block {d, extra, scales[8], qs[64]});
    # the canonical streams are qs (64) | scl (8) | sex (2) | dv (2), each
    # field at the position the stream table and the LSB-first reading give
    wire = np.zeros(76, np.uint8)
    wire[0:2] = [0x00, 0x3C]            # d = 1.0
    wire[2:4] = [0x01, 0x80]            # extra: alphabet 1 for sub-blocks 0 and 15
    wire[4:12] = 0x88                   # scale nibbles 8 (-> 0) ...
    wire[4] = 0x21                      # ... sub-block 0: 1 (-> -7), sub-block 1: 2 (-> -6)
    wire[11] = 0xF3                     # sub-block 14: 3 (-> -5), sub-block 15: 15 (-> 7)
    wire[12 + 0] = 0x01                 # weight 0 (h=0, p=0, l=0): code 1
    wire[12 + 5] = 0x08                 # weight 37 (h=0, p=1, l=5): code 2 at bits 2..3
    wire[12 + 63] = 0xC0                # weight 255 (h=1, p=3, l=31): code 3 at bits 6..7
    s = oracle.pack(K, wire, 1, 256)
    expected = np.zeros(76, np.uint8)
    expected[0] = 0x01                  # weight 0 -> qs byte 0, bits 0..1
    expected[9] = 0x08                  # weight 37 -> qs byte 9, bits 2..3
    expected[63] = 0xC0                 # weight 255 -> qs byte 63, bits 6..7
    expected[64:72] = [0x21, 0x88, 0x88, 0x88, 0x88, 0x88, 0x88, 0xF3]  # scl: sub-block s at byte s/2, low nibble first
    expected[72:74] = [0x01, 0x80]      # sex: bit s of the plane
    expected[74:76] = [0x00, 0x3C]      # dv
    assert np.array_equal(s, expected)
    assert np.array_equal(oracle.unpack(K, s, 1, 256), wire)
    values = np.array([1, 2, 3, 4, 5, 6, 7, 8], np.float32)
    w = oracle.dequant(K, s, 1, 256, values)[0]
    exp = np.zeros(256, np.float32)
    exp[0:16] = -35.0                   # (1 * -7) * values[4 + 0]
    exp[0] = -42.0                      # (1 * -7) * values[4 + 1]
    exp[16:32] = -6.0                   # (1 * -6) * values[0]
    exp[224:240] = -5.0                 # (1 * -5) * values[0]
    exp[240:256] = 35.0                 # (1 * 7) * values[4 + 0]
    exp[255] = 56.0                     # (1 * 7) * values[4 + 3]
    assert np.array_equal(w, exp)


def test_iq1s_r4_hand_group():
    # four rows, n = 32 (one block of four 8-weight groups)
    grid = np.zeros((2048, 8), np.int8)
    grid[0x123] = [1, -1, 0, 1, -1, 0, 1, -1]
    grid[0x7FF] = -1
    wire = np.zeros(4 * 8, np.uint8)    # 4 x 2 + 24 = 32 bytes
    wire[0:8] = [0x00, 0x3C, 0x00, 0x40, 0x00, 0x38, 0x00, 0xBC]   # d = 1, 2, 0.5, -1
    qs = wire[8:24]
    qh = wire[24:32]
    for j in range(4):
        qs[4 * j + 0] = 0x23            # row 0: index 0x123 in every group
        qs[4 * j + 1] = 0xFF            # row 1: index 0x7FF
        qs[4 * j + 2] = 0x00            # row 2: index 0
        qs[4 * j + 3] = j               # row 3: index j
    qh[0:2] = [0x49, 0x32]              # row 0: 0x3249 = hi bits 1,1,1,1; ls 3; sign 0
    qh[2:4] = [0xFF, 0x8F]              # row 1: 0x8FFF = hi bits 7,7,7,7; ls 0; sign 1
    qh[4:6] = [0x00, 0xF0]              # row 2: 0xF000 = ls 7; sign 1
    qh[6:8] = [0x00, 0x10]              # row 3: 0x1000 = ls 1; sign 0
    s = oracle.pack(R4, wire, 4, 32)
    w = oracle.dequant(R4, s, 4, 32, None, grid)
    row0 = np.tile(np.array([7.875, -6.125, 0.875, 7.875, -6.125, 0.875, 7.875, -6.125], np.float32), 4)
    assert np.array_equal(w[0], row0)                       # (1*7) * (g + 1/8)
    assert np.array_equal(w[1], np.full(32, -2.25, np.float32))    # (2*1) * (-1 - 1/8)
    assert np.array_equal(w[2], np.full(32, -0.9375, np.float32))  # (0.5*15) * (0 - 1/8)
    assert np.array_equal(w[3], np.full(32, -0.375, np.float32))   # (-1*3) * (0 + 1/8)
    # streams: per-row qs bytes, then qh words, then dv
    assert np.array_equal(s[0:4], [0x23] * 4)
    assert np.array_equal(s[12:16], [0, 1, 2, 3])
    assert np.array_equal(s[16:18], [0x49, 0x32])
    assert np.array_equal(s[24:32], wire[0:8])


# --------------------------------------------------------------------------
# relayout is a permutation (P3)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,rows,n", [(KS, 4, 256), (K, 4, 256), (R4, 4, 256), (R4, 8, 64)])
def test_relayout_single_bit_tracing(fmt, rows, n):
    nbytes = rows * oracle.row_bytes(fmt, n)
    base = synth.random_bytes(nbytes, 5)
    s0 = np.unpackbits(oracle.pack(fmt, base, rows, n))
    seen = np.zeros(nbytes * 8, bool)
    for bit in range(nbytes * 8):
        w = base.copy()
        w[bit // 8] ^= np.uint8(1 << (bit % 8))
        diff = np.flatnonzero(np.unpackbits(oracle.pack(fmt, w, rows, n)) != s0)
        assert diff.size == 1, f"wire bit {bit} moved {diff.size} stream bits"
        assert not seen[diff[0]]
        seen[diff[0]] = True
    assert seen.all()


@pytest.mark.parametrize("fmt,rows,n", [(KS, 6, 512), (K, 5, 768), (R4, 12, 96), (R4, 4, 4096), (K, 2, 4096)])
def test_relayout_round_trips(fmt, rows, n):
    nbytes = rows * oracle.row_bytes(fmt, n)
    w = synth.random_bytes(nbytes, 21)
    s = oracle.pack(fmt, w, rows, n)
    assert s.size == w.size
    assert np.array_equal(oracle.unpack(fmt, s, rows, n), w)
    s2 = synth.random_bytes(nbytes, 22)
    assert np.array_equal(oracle.pack(fmt, oracle.unpack(fmt, s2, rows, n), rows, n), s2)


@pytest.mark.parametrize("fmt,rows,n", [(KS, 8, 512), (K, 8, 512), (R4, 8, 256)])
def test_two_decoders_agree(fmt, rows, n):
    w = synth.wire(fmt, rows, n, 31)
    fw = oracle.decode_wire(fmt, w, rows, n)
    fs = oracle.decode_streams(fmt, oracle.pack(fmt, w, rows, n), rows, n)
    assert np.array_equal(fw, fs)
    # every field stays inside its stated range
    if fmt == KS:
        assert fw["a"].min() >= -16 and fw["a"].max() <= 15
    if fmt == K:
        assert fw["a"].min() >= -8 and fw["a"].max() <= 7
    if fmt == R4:
        assert fw["c"].max() <= 2047 and fw["a"].max() <= 7
    assert set(np.unique(fw["b"])) <= {0, 1}


def test_uniform_bytes_give_uniform_fields():
    # the synthetic recipe: uniform random wire bytes => uniform fields
    rows, n = 64, 4096
    f = oracle.decode_wire(KS, synth.wire(KS, rows, n, 7), rows, n)
    si = f["a"][:, ::32].ravel()
    counts = np.bincount(si + 16, minlength=32)
    assert counts.min() > 0.7 * counts.mean()
    codes = np.bincount(f["c"].ravel(), minlength=4)
    assert codes.min() > 0.95 * codes.mean()


# --------------------------------------------------------------------------
# exact closed forms (P4)
# --------------------------------------------------------------------------

D_CASES = [0x3C00, 0x3555, 0x0001, 0x03FF, 0xBC00, 0x0000, 0x8000, 0x7BFF, 0x2E66]


def _half_exact(h):
    """exact value of an fp16 bit pattern as a double, from the IEEE
    definition (normal: (1024+m) * 2^(e-25); subnormal: m * 2^-24)"""
    h = np.asarray(h, np.int64)
    sgn = np.where(h >> 15, -1.0, 1.0)
    e = (h >> 10) & 31
    m = h & 1023
    mag = np.where(e == 0, m * 2.0**-24, (1024 + m) * np.exp2(e.astype(np.float64) - 25))
    return sgn * mag


def _expect_bits(exact: np.ndarray, neg_zero: np.ndarray) -> np.ndarray:
    """float32 bits of values that are exactly representable (checked), with
    IEEE's sign-XOR rule deciding the sign of zero results"""
    v = exact.astype(np.float32)
    assert np.array_equal(v.astype(np.float64), exact), "closed form is not exact in float32"
    bits = v.view(np.uint32).copy()
    z = exact == 0
    bits[z] = np.where(neg_zero[z], 0x80000000, 0).astype(np.uint32)
    return bits


def _rows_by_scale(cells, per_row, sb, n):
    """lay cells (d, a, b, c) out as rows of n weights, one d per row, one
    cell per sb-weight sub-block"""
    by_d = {}
    for c in cells:
        by_d.setdefault(c[0], []).append(c)
    rows = []
    for cl in by_d.values():
        for i in range(0, len(cl), per_row):
            chunk = cl[i:i + per_row]
            rows.append(chunk + [chunk[-1]] * (per_row - len(chunk)))
    f = np.zeros((len(rows), n), oracle.FIELD_DTYPE)
    for r, chunk in enumerate(rows):
        for j, cell in enumerate(chunk):
            f[r, j * sb:(j + 1) * sb] = cell
    return f


@pytest.mark.parametrize("fmt", [KS, K])
def test_two_bit_reconstruction_exhaustive_fields(fmt):
    # every (scale index, alphabet, code) against scales that are normal,
    # subnormal, negative, +-0 and the largest finite fp16.  With an integer
    # table every float32 step is exact, so the expected value is the exact
    # product d * si * v.
    sis = range(-16, 16) if fmt == KS else range(-8, 8)
    sb = 32 if fmt == KS else 16
    n = 256
    values = np.array([-31, -13, 1, 17, -26, -8, 0, 22], np.float32)
    cells = [(d, si, a, c) for d in D_CASES for si in sis for a in (0, 1) for c in range(4)]
    f = _rows_by_scale(cells, n // sb, sb, n)
    got = oracle.weight_rows(fmt, f, values).view(np.uint32)
    d = _half_exact(f["d"])
    si = f["a"].astype(np.float64)
    v = values[4 * f["b"] + f["c"]].astype(np.float64)
    neg = (f["d"] >> 15).astype(bool) ^ (si < 0) ^ np.signbit(v)
    assert np.array_equal(got, _expect_bits(d * si * v, neg))


def test_iq1s_reconstruction_exhaustive_fields():
    # every grid index x ls x shift sign x position, ternary grid: exact products
    rng = np.random.default_rng(3)
    grid = rng.integers(-1, 2, size=(2048, 8)).astype(np.int8)
    n = 256
    cells = [(d, ls, sg, idx) for d in (0x3C00, 0x0001, 0xBC00, 0x8000, 0x2E66)
             for ls in range(8) for sg in (0, 1) for idx in range(2048)]
    # one 32-weight block per (d, ls, sign) and four 8-weight groups of indices
    blocks = []
    for i in range(0, len(cells), 4):
        blocks.append(cells[i:i + 4])
    by_d = {}
    for b in blocks:
        by_d.setdefault(b[0][0], []).append(b)
    rows = []
    for bl in by_d.values():
        for i in range(0, len(bl), n // 32):
            chunk = bl[i:i + n // 32]
            rows.append(chunk + [chunk[-1]] * (n // 32 - len(chunk)))
    rows += [rows[-1]] * ((-len(rows)) % 4)
    f = np.zeros((len(rows), n), oracle.FIELD_DTYPE)
    for r, chunk in enumerate(rows):
        for b, grp in enumerate(chunk):
            for j, (d, ls, sg, idx) in enumerate(grp):
                f[r, 32 * b + 8 * j:32 * b + 8 * j + 8] = (d, grp[0][1], grp[0][2], idx)
    got = oracle.weight_rows(R4, f, None, grid).view(np.uint32)
    d = _half_exact(f["d"])
    ls = f["a"].astype(np.float64)
    g = grid[f["c"], np.arange(n)[None, :] % 8].astype(np.float64)
    t = g + np.where(f["b"] == 1, -0.125, 0.125)
    neg = (f["d"] >> 15).astype(bool) ^ (t < 0)
    assert np.array_equal(got, _expect_bits(d * (2 * ls + 1) * t, neg))


def _f32(x: float) -> np.float32:
    """one correctly rounded conversion of an exact double to float32"""
    return np.float32(x)


def test_float32_step_order_with_general_tables():
    # random float32 table entries and random fp16 scales: the products are
    # no longer exact, so the result depends on the order of the two float32
    # multiplies.  Expected: round((round(d*si)) * v), each product exact in double.
    rng = np.random.default_rng(9)
    rows, n = 64, 256
    values = (rng.standard_normal(8) * 3).astype(np.float32)
    w_wire = synth.wire(KS, rows, n, 17, sigma=0.37)
    s = oracle.pack(KS, w_wire, rows, n)
    f = oracle.decode_streams(KS, s, rows, n)
    got = oracle.dequant(KS, s, rows, n, values)
    differs = 0
    for r in range(rows):
        d = np.float32(np.uint16(f[r, 0]["d"]).view(np.float16))
        for k in range(0, n, 7):
            si = float(f[r, k]["a"])
            v = float(values[4 * f[r, k]["b"] + f[r, k]["c"]])
            dl = _f32(float(d) * si)
            exp = _f32(float(dl) * v)
            other = _f32(float(d) * float(_f32(si * v)))
            differs += int(exp.view(np.uint32) != other.view(np.uint32))
            assert got[r, k].view(np.uint32) == exp.view(np.uint32)
    assert differs > 0, "sample does not discriminate the multiply order"


def test_iq1s_step_order_with_general_grid():
    rng = np.random.default_rng(10)
    rows, n = 8, 256
    grid = rng.integers(-128, 128, size=(2048, 8)).astype(np.int8)
    w_wire = synth.wire(R4, rows, n, 18, sigma=0.37)
    s = oracle.pack(R4, w_wire, rows, n)
    f = oracle.decode_streams(R4, s, rows, n)
    got = oracle.dequant(R4, s, rows, n, None, grid)
    for r in range(rows):
        d = np.float32(np.uint16(f[r, 0]["d"]).view(np.float16))
        for k in range(n):
            ls, sg, idx = int(f[r, k]["a"]), int(f[r, k]["b"]), int(f[r, k]["c"])
            sc = _f32(float(d) * (2 * ls + 1))
            t = float(grid[idx, k % 8]) + (-0.125 if sg else 0.125)   # exact
            exp = _f32(float(sc) * t)
            assert got[r, k].view(np.uint32) == exp.view(np.uint32)


def test_dequant_casts_are_one_rne_of_the_f32_chain():
    rows, n = 16, 512
    values = synth.values_table(4)
    for fmt in (KS, K):
        s = oracle.pack(fmt, synth.wire(fmt, rows, n, 40 + fmt), rows, n)
        w32 = oracle.dequant(fmt, s, rows, n, values, None, oracle.F32)
        w16 = oracle.dequant(fmt, s, rows, n, values, None, oracle.F16)
        wb = oracle.dequant(fmt, s, rows, n, values, None, oracle.BF16)
        assert np.array_equal(w16.ravel(), w32.ravel().astype(np.float16).view(np.uint16))
        import torch
        ref = torch.from_numpy(w32.ravel().copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(wb.ravel(), ref)
