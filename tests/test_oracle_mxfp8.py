"""Pins of the MXFP8 oracle (CPU): the E4M3 code table, rounding, saturation,
the block-scale rule, the error bound, and the MX GEMM on exact inputs.

Each pin is fixed by the OCP MX / OCP FP8 definitions or by arithmetic, not by
re-running the oracle's own formulas."""
import numpy as np

from oracle import moe_oracle as om
from oracle import mxfp8_oracle as mo


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_e4m3_known_values():
    d = mo.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x30, 0x38, 0x3C, 0x40, 0x77, 0x7E,
                                 0x80, 0xB8, 0xFE], dtype=np.uint8))
    assert d.tolist() == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 0.5, 1.0, 1.5, 2.0,
                          1.875 * 2 ** 7, 448.0, -0.0, -1.0, -448.0]
    assert np.signbit(d[10])
    assert np.isnan(mo.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_table_structure():
    pos = mo.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    # 127 distinct non-negative values in increasing code order; 126 positive
    assert np.all(np.diff(pos) > 0)
    assert (pos > 0).sum() == 126
    # each binade [2^e, 2^(e+1)) above the subnormals holds 8 values spaced 2^(e-3)
    for e in range(-6, 9):
        vals = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(vals) == (7 if e == 8 else 8)
        assert np.allclose(np.diff(vals), 2.0 ** (e - 3))


def test_e4m3_encode_roundtrip_every_code():
    c = _finite_codes()
    assert np.array_equal(mo.e4m3_encode(mo.e4m3_decode(c)), c)


def test_e4m3_ties_to_even_at_every_midpoint():
    pos = mo.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448 ascending
    mids = (pos[:-1] + pos[1:]) / 2
    got = mo.e4m3_encode(mids)
    lo = np.arange(0x7E, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)  # even mantissa wins
    assert np.array_equal(got, want)
    # just off the midpoint, the nearer neighbour wins
    assert np.array_equal(mo.e4m3_encode(mids * (1 - 1e-9)), lo)
    assert np.array_equal(mo.e4m3_encode(mids * (1 + 1e-9)), lo + 1)


def test_e4m3_saturates():
    got = mo.e4m3_encode(np.array([448.0, 460.0, 464.0, 500.0, 1e9, -1e9, -470.0]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_mx_scale_rule():
    # amax = 1.0 -> s = -8; amax = 300 -> s = 0; amax just below 2 -> s = -8
    for amax, s in [(1.0, -8), (300.0, 0), (1.999, -8), (2.0, -7), (2.0 ** -130, -127),
                    (2.0 ** 200, 127)]:
        v = np.zeros((1, 32))
        v[0, 5] = -amax
        v[0, 9] = amax / 3
        _, sc = mo.mx_quantize(v)
        assert int(sc[0, 0]) == s + 127, (amax, int(sc[0, 0]) - 127)
    # all-zero block
    q, sc = mo.mx_quantize(np.zeros((2, 64)))
    assert np.all(q == 0) and np.all(sc == 0)
    # the largest element lands in [256, 512) before saturation, i.e. code >= 0x78
    rng = np.random.default_rng(3)
    v = rng.standard_normal((50, 256)) * np.exp2(rng.integers(-20, 20, size=(50, 1)))
    q, sc = mo.mx_quantize(v)
    qb = q.reshape(50, 8, 32) & 0x7F
    assert np.all(qb.max(axis=-1) >= 0x78)


def test_mx_error_bound():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-10, 10, size=(64, 1)))
    q, sc = mo.mx_quantize(v)
    d = mo.mx_dequantize(q, sc)
    X = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    y = np.abs(v) / X
    err = np.abs(d - v)
    normal = (y >= 2.0 ** -6) & (y <= 448)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(v[normal]) * (1 + 1e-12))
    assert np.all(err[y < 2.0 ** -6] <= 2.0 ** -10 * X[y < 2.0 ** -6] * (1 + 1e-12))
    # saturated elements: only those above 448 X, clipped to 448 X
    sat = y > 448
    assert np.allclose(np.abs(d[sat]), 448 * X[sat])


def test_mx_quantize_idempotent_on_representable_values():
    rng = np.random.default_rng(5)
    q0 = rng.integers(0, 256, size=(20, 96)).astype(np.uint8)
    q0[(q0 & 0x7F) == 0x7F] = 0x38
    q0[:, ::32] = 0x7E  # each block holds a max-magnitude element: scale is kept
    s0 = rng.integers(100, 150, size=(20, 3)).astype(np.uint8)
    q, s = mo.mx_quantize(mo.mx_dequantize(q0, s0))
    assert np.array_equal(s, s0)
    assert np.array_equal(mo.e4m3_decode(q), mo.e4m3_decode(q0))  # +0 / -0 aside


def test_mx_gemm_matches_matmul_on_exact_inputs():
    rng = np.random.default_rng(6)
    # E4M3 values with unit scales (s = 0 needs amax in [256, 512): set one 256)
    a = mo.e4m3_decode(rng.integers(0, 0x70, size=(16, 64)).astype(np.uint8)) * \
        rng.choice([-1, 1], size=(16, 64))
    a[:, 0] = 256.0
    a[:, 32] = -256.0
    w = mo.e4m3_decode(rng.integers(0, 0x70, size=(24, 64)).astype(np.uint8))
    w[:, 0] = 256.0
    w[:, 32] = 256.0
    aq, asc = mo.mx_quantize(a)
    wq, wsc = mo.mx_quantize(w)
    assert np.all(asc == 127) and np.all(wsc == 127)
    assert np.array_equal(mo.mx_gemm(aq, asc, wq, wsc), a @ w.T)


def test_pack_weights_layout():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((3, 64, 40))  # [n, K, N]
    q, s = mo.pack_weights(w)
    assert q.shape == (3, 40, 64) and s.shape == (3, 40, 2)
    q1, s1 = mo.mx_quantize(w[1][:, 7])
    assert np.array_equal(q[1, 7], q1) and np.array_equal(s[1, 7], s1)


def test_round_bf16():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0 ** -130, 3.0e38])
    got = mo.round_bf16(v)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2.0 ** -6
    assert got[3] == np.float32(-2.0 ** -130).astype(np.float64) or got[3] == -2.0 ** -130


def test_expert_ffn_mxfp8_close_to_plain_ffn():
    # the quantized FFN stays within the format's error of the plain one
    rng = np.random.default_rng(8)
    M, D, I, n = 48, 64, 64, 3
    x = rng.standard_normal((M, D))
    wgu = rng.standard_normal((n, D, 2 * I)) * 0.05
    wd = rng.standard_normal((n, I, D)) * 0.05
    off = np.array([0, 10, 10, 48])
    r = mo.expert_ffn_mxfp8(x, off, wgu, wd)
    y_ref = om.expert_ffn(x, off, wgu, wd)
    rel = np.linalg.norm(r["y"] - y_ref) / np.linalg.norm(y_ref)
    assert 1e-3 < rel < 0.08
    # segments with no rows give no output rows; H and Y shapes
    assert r["h"].shape == (M, I) and r["y"].shape == (M, D)
    # the H handed to GEMM 2 is bf16 (its low 16 bits are zero)
    hb = r["h"].astype(np.float32).view(np.uint32)
    assert np.all(hb & 0xFFFF == 0)
