"""The input encodings both sides share (CPU only): float32 -> bf16 and
float32 -> OCP fp8 E4M3 codes, round to nearest even, pinned by values the
formats fix, not by re-deriving the encoders."""

import numpy as np

import workloads


def test_e4m3_codes_of_values_the_format_fixes():
    # OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities,
    # 0x7F is NaN, so the largest finite code 0x7E is 1.75 * 2^8 = 448; the
    # smallest subnormal 0x01 is 2^-9, the smallest normal 0x08 is 2^-6
    vals = np.array([0.0, 1.0, 1.5, -2.0, 448.0, 2.0 ** -9, 2.0 ** -6, 0.875 * 2.0 ** -6, 240.0],
                    np.float32)
    want = np.array([0x00, 0x38, 0x3C, 0xC0, 0x7E, 0x01, 0x08, 0x07, 0x77], np.uint8)
    np.testing.assert_array_equal(workloads.f32_to_e4m3_bits(vals), want)
    np.testing.assert_array_equal(workloads.e4m3_bits_to_f32(want), vals)


def test_e4m3_rounds_to_nearest_even_and_saturates():
    # halfway between 1.0 (mantissa 000) and 1.125 (001) -> 1.0 (even);
    # halfway between 1.125 (001) and 1.25 (010) -> 1.25; just above -> up;
    # halfway between 0 and the smallest subnormal -> 0; beyond 448 -> 448
    vals = np.array([1.0625, 1.1875, 1.0626, 2.0 ** -10, -2.0 ** -10 * 1.01, 1000.0, -500.0],
                    np.float32)
    got = workloads.e4m3_bits_to_f32(workloads.f32_to_e4m3_bits(vals))
    np.testing.assert_array_equal(got, np.array([1.0, 1.25, 1.125, 0.0, -2.0 ** -9, 448.0, -448.0],
                                                np.float32))


def test_e4m3_every_code_decodes_and_reencodes_to_itself():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = workloads.e4m3_bits_to_f32(codes)
    back = workloads.f32_to_e4m3_bits(vals)
    # -0 encodes as +0; every other code is its own round trip
    np.testing.assert_array_equal(np.where(codes == 0x80, 0, back), np.where(codes == 0x80, 0, codes))
    # values grow with the code inside each sign
    pos = vals[codes < 0x80]
    assert np.all(np.diff(pos) > 0)


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1 (even); 1 + 3 * 2^-8 -> 1 + 2^-6
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -3.0, 65280.0], np.float32)
    got = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(vals))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0 + 2.0 ** -6, -3.0, 65280.0], np.float32))


def test_fp8_workload_draws_fp8_score_operands_and_bf16_values():
    w = workloads.make("dflash_r")
    w8 = workloads.Workload("dflash_r-fp8", w.seqlens, w.C, w.r, w.kind, w.depth_or_block, w.hq,
                            w.hkv, w.d, "fp8", False, w.seed, anchors=w.anchors)
    raw = workloads.draw(w8, 64, 16)
    for name, arr in raw.items():
        assert arr.dtype == (np.uint8 if name in workloads.FP8_TENSORS else np.uint16), name
    # the fp8 draws are the bf16 workload's N(0, 1) values, encoded differently
    rb = workloads.draw(w, 64, 16, names=["q"])
    qf = workloads.as_f32(w8, raw["q"])
    qb = workloads.as_f32(w, rb["q"])
    # element by element within the E4M3 half-ulp (2^-4 relative) plus the
    # bf16 one, or the subnormal step near zero
    assert np.all(np.abs(qf - qb) <= (2.0 ** -4 + 2.0 ** -8) * np.abs(qb) + 2.0 ** -10)
