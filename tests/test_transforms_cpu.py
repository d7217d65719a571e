"""CPU checks of the bit-level transforms the kernels use (restated here in
Python from their definitions; the GPU parity tests check the kernels).

* int4 limbs: X in [-2^22, 2^22] -> six balanced base-16 digits via
  Y = (X + 0x888888) ^ 0x888888 (each nibble the digit's 4-bit two's complement);
* int8 limbs: three balanced base-256 digits via Y = (X + 0x808080) ^ 0x808080;
* int4 weights -> int8 bytes for the integer matrix cores: each nibble n becomes
  ((n ^ 8) + 0x78) ^ 0x80 within its byte, then the low- and high-nibble bytes are
  interleaved with two byte permutes (v_perm_b32 semantics: selector k < 4 takes
  byte k of the second source, 4..7 byte k - 4 of the first)."""
import numpy as np


def signed(v, bits):
    v &= (1 << bits) - 1
    return v - (1 << bits) if v >= 1 << (bits - 1) else v


def test_int4_limb_digits_reconstruct_x():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.integers(-(1 << 22), (1 << 22) + 1, 20000), [-(1 << 22), 1 << 22, 0, -1, 1]])
    for x in xs.tolist():
        y = ((x + 0x888888) & 0xFFFFFFFF) ^ 0x888888
        digits = [signed(y >> (4 * l), 4) for l in range(6)]
        assert all(-8 <= d <= 7 for d in digits)
        assert sum(d * 16 ** l for l, d in enumerate(digits)) == x


def test_int8_limb_digits_reconstruct_x():
    rng = np.random.default_rng(2)
    xs = np.concatenate([rng.integers(-(1 << 22), (1 << 22) + 1, 20000), [-(1 << 22), 1 << 22, 0, -1, 1]])
    for x in xs.tolist():
        y = ((x + 0x808080) & 0xFFFFFFFF) ^ 0x808080
        digits = [signed(y >> (8 * l), 8) for l in range(3)]
        assert all(-128 <= d <= 127 for d in digits)
        assert sum(d * 256 ** l for l, d in enumerate(digits)) == x
        # |sum of 32 products with int8 weights| per digit <= 32 * 128 * 128 = 2^19
        assert max(abs(d) for d in digits) * 128 * 32 <= 1 << 19


def perm(s0, s1, sel):
    b = [(s1 >> (8 * i)) & 0xFF for i in range(4)] + [(s0 >> (8 * i)) & 0xFF for i in range(4)]
    return sum(b[(sel >> (8 * i)) & 0xFF] << (8 * i) for i in range(4))


def nib_to_i8(w):
    m = 0xFFFFFFFF
    lo = w & 0x0F0F0F0F
    hi = (w >> 4) & 0x0F0F0F0F
    lo = (((lo ^ 0x08080808) + 0x78787878) & m) ^ 0x80808080
    hi = (((hi ^ 0x08080808) + 0x78787878) & m) ^ 0x80808080
    return perm(hi, lo, 0x05010400), perm(hi, lo, 0x07030602)


def test_nibbles_to_int8_bytes():
    rng = np.random.default_rng(3)
    words = rng.integers(0, 1 << 32, 20000, dtype=np.uint64).tolist() + [0, 0xFFFFFFFF, 0x88888888, 0x77777777]
    for w in words:
        expect = []
        for j in range(4):
            byte = (w >> (8 * j)) & 0xFF
            expect += [signed(byte & 0xF, 4), signed(byte >> 4, 4)]  # element 2j low nibble, 2j+1 high
        got = [signed(o >> (8 * i), 8) for o in nib_to_i8(w) for i in range(4)]
        assert got == expect


def block_fixed_point(v: np.ndarray):
    """The kernels' block fixed point of one fp32 group: sh = min(22 - E, 149) with
    max|v| < 2^E, X = rint(v * 2^sh) (ties to even), factor f = 2^-sh."""
    m = float(np.max(np.abs(v)))
    E = int(np.frexp(np.float32(m))[1])
    sh = min(22 - E, 149)
    X = np.rint(np.ldexp(v.astype(np.float64), sh))
    return X, sh


def test_block_fixed_point_across_the_fp32_range():
    """|X| <= 2^22 for every group scale from the largest fp32 values to the
    subnormals; a group of subnormals is held exactly (the shift stops at 149);
    each element is kept to within half a step of 2^(E-22) <= 2^-22 of the
    group maximum."""
    rng = np.random.default_rng(4)
    for e in list(range(-149, 128, 7)) + [127, -126, -127, -140, -149]:
        v = (rng.uniform(-1, 1, 32) * 2.0 ** e).astype(np.float32)
        if not np.isfinite(v).all() or np.max(np.abs(v)) == 0:
            continue
        X, sh = block_fixed_point(v)
        assert np.max(np.abs(X)) <= 2 ** 22
        back = np.ldexp(X, -sh)
        m = float(np.max(np.abs(v)))
        assert np.max(np.abs(back - v.astype(np.float64))) <= m * 2.0 ** -22
        if m < 2.0 ** -127:  # shift 149: subnormals are multiples of 2^-149, held exactly
            assert np.array_equal(back, v.astype(np.float64))


def test_group_factor_order_keeps_tiny_contributions():
    """A group's contribution T * s * 2^-sh: multiplying the fp16 scale by 2^-sh
    first underflows for tiny activations, applying the power of two last does
    not (the kernels' order)."""
    T = np.float32(1234567.0)
    s = np.float32(0.0137)
    f = np.float32(2.0 ** -140)
    exact = float(T) * float(s) * 2.0 ** -140
    late = np.float32(T * s) * f
    early = T * np.float32(s * f)
    assert abs(float(late) - exact) <= exact * 2.0 ** -23
    assert abs(float(early) - exact) > exact * 2.0 ** -10
