"""Pins of the MXFP4 weight format: the oracle's dequantisation against the format's
definition (OCP Microscaling Formats (MX) v1.0: FP4 E2M1 elements, E8M0 block scale of 32
elements) and the generator's quantisation against hand-computed and brute-force nearest
values."""
import numpy as np

import gen
import oracle


def _bitfield_value(code):
    """E2M1 value from its fields: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0;
    exponent 0 is subnormal (0.5 * mantissa)."""
    sign = -1.0 if code & 8 else 1.0
    exp, man = (code >> 1) & 3, code & 1
    mag = 0.5 * man if exp == 0 else 2.0 ** (exp - 1) * (1.0 + 0.5 * man)
    return sign * mag


def test_all_sixteen_codes_and_nibble_order():
    codes = np.zeros((1, 16), dtype=np.uint8)
    for j in range(16):  # element 2j = code j (low nibble), element 2j+1 = code 15-j (high)
        codes[0, j] = j | ((15 - j) << 4)
    vals = oracle.mxfp4_dequant(codes, np.full((1, 1), 127, dtype=np.uint8))[0]
    for j in range(16):
        assert vals[2 * j] == _bitfield_value(j)
        assert vals[2 * j + 1] == _bitfield_value(15 - j)
    assert sorted(set(abs(v) for v in vals)) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_scale_is_a_power_of_two_per_block():
    codes = np.full((1, 64), 0x22, dtype=np.uint8)  # 128 elements, all code 2 = 1.0
    scales = np.array([[0, 1, 127, 254]], dtype=np.uint8)
    vals = oracle.mxfp4_dequant(codes, scales)[0]
    for b, s in enumerate((0, 1, 127, 254)):
        assert np.all(vals[32 * b:32 * (b + 1)] == 2.0 ** (s - 127))


def test_hand_quantised_block_ties_and_saturation():
    """Block with max |v| = 7 * 2^-8: shared exponent floor(log2 7) - 2 - 8 = -8.  Scaled
    values and their E2M1 codes by hand: ties go to the even code (mantissa 0), 7 saturates
    to 6, -0.3 rounds to -0.5."""
    X = 2.0 ** -8
    scaled = [6, -3, 0.5, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 7, -0.3]
    want = [6, -3, 0.5, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6, -0.5]
    v = np.zeros(32, dtype=np.float32)
    v[:len(scaled)] = np.array(scaled, dtype=np.float32) * np.float32(X)
    codes, scale = gen.mxfp4_block(v)
    assert scale == 127 - 8
    got = oracle.mxfp4_dequant(codes[None, :], np.array([[scale]], dtype=np.uint8))[0]
    np.testing.assert_array_equal(got[:len(want)], np.array(want) * X)
    assert np.all(got[len(want):] == 0)


def test_random_blocks_round_to_a_nearest_grid_value():
    """Brute force over random blocks: the shared exponent puts max |v| / X in [4, 8); every
    element dequantises to a nearest point of the scaled E2M1 grid (saturating beyond 6X),
    ties to the even code."""
    r = np.random.default_rng(5)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    even = np.array([True, False, True, False, True, False, True, False])
    for _ in range(400):
        v = (r.standard_normal(32) * r.choice([1e-3, 0.02, 1.0, 30.0])).astype(np.float32)
        codes, s = gen.mxfp4_block(v)
        X = 2.0 ** (s - 127)
        assert 4.0 <= np.max(np.abs(v)) / X < 8.0
        got = oracle.mxfp4_dequant(codes[None, :], np.array([[s]], dtype=np.uint8))[0]
        for vi, gi in zip(v.astype(np.float64), got):
            a = min(abs(vi) / X, 6.0)
            dist = np.abs(grid - a)
            best = np.nonzero(dist == dist.min())[0]
            pick = best[0] if len(best) == 1 else best[even[best]][0]
            assert abs(gi) == grid[pick] * X
            assert gi == 0.0 or np.sign(gi) == np.sign(vi)


def test_all_zero_block():
    codes, s = gen.mxfp4_block(np.zeros(32, dtype=np.float32))
    assert s == 0 and np.all(codes == 0)


def test_tiled_entry_layout():
    """An MXFP4 entry written for the library holds every block of every matrix where the
    documented tiled layout puts it (16-row x 128-element tiles; strips whose last tile is
    short when K is not a multiple of 128), and nothing else: each byte is written once."""
    from gen import configs
    from gen.arena import fill_entries_ptr
    for d, f in ((320, 192), (256, 128)):
        w = configs.Workload("mx_layout", seed=31, T=1, d=d, E=2, k=1, f=f, dtype=gen.MXFP4)
        nbytes = w.entry_elems
        buf = np.full(nbytes, 0xA5, dtype=np.uint8)
        fill_entries_ptr(w, [(0, 1)], buf.ctypes.data, nbytes)
        fd = f * d
        seen = np.zeros(nbytes, dtype=np.int64)
        mats = configs.gen_expert(w, 0, 1)
        for mi, ((codes, scales), (R, K)) in enumerate(zip(mats, ((f, d), (f, d), (d, f)))):
            cbase, sbase = mi * fd // 2, 3 * fd // 2 + mi * fd // 32
            for r in range(R):
                for b in range(K // 32):
                    co = cbase + 8 * K * (r // 16) + 1024 * (b // 4) + 16 * (16 * (b % 4) + r % 16)
                    so = sbase + K // 2 * (r // 16) + 64 * (b // 4) + 16 * (b % 4) + r % 16
                    assert np.array_equal(buf[co:co + 16], codes[r, 16 * b:16 * b + 16]), (mi, r, b)
                    assert buf[so] == scales[r, b], (mi, r, b)
                    seen[co:co + 16] += 1
                    seen[so] += 1
        assert np.all(seen == 1)
