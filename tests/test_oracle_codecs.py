"""Pins of the oracle's codecs against the pages' printed sizes, format specs,
closed forms and library routines (torch's bf16 / float8_e4m3fn conversions)."""
import numpy as np
import pytest
import torch

from oracle import codecs as K
from synth import configs as C, gen


# ------------------------------------------------------------------ Q8_0 ---
def test_q8_0_hand_block():
    """A block whose scale is exactly 1: codes are the inputs rounded half away
    from zero (2.5 -> 3, -2.5 -> -3, 0.5 -> 1, 126.5 -> 127), d stored as fp16 1.0."""
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [127, -2.5, 2.5, 0.5, -0.5, 126.5, 1.49, -1.51]
    b = K.q8_0_encode(x).reshape(34)
    assert b[0] == 0x00 and b[1] == 0x3C                      # fp16 1.0 little-endian
    q = b[2:].view(np.int8)
    assert list(q[:8]) == [127, -3, 3, 1, -1, 127, 1, -2]
    assert not q[8:].any()
    np.testing.assert_array_equal(K.q8_0_decode(b[None], 1, 32)[0, :8],
                                  [127, -3, 3, 1, -1, 127, 1, -2])


def test_q8_0_zero_block_and_layout():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    b = K.q8_0_encode(x)
    assert b.shape == (2, 68)
    assert not b[0].any() and not b[1, :34].any()            # zero blocks: d = 0, q = 0
    d = b[1, 34:36].copy().view(np.float16)[0]
    assert d == np.float16(np.float32(1.0) / np.float32(127))


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-3])
def test_q8_0_roundtrip_is_identity_on_codes(std):
    """encode(decode(B)) == B: the block maximum decodes to d16 * 127 exactly,
    so re-encoding recovers d16 and every code."""
    w = gen.normal((64, 4096), seed=7, idx=int(std * 1e4), std=std)
    w[3, :32] = 0.0
    b = K.q8_0_encode(w)
    again = K.q8_0_encode(K.q8_0_decode(b, 64, 4096).astype(np.float32))
    np.testing.assert_array_equal(b, again)


def test_q8_0_two_encoders_agree():
    """The generator's encoder and the oracle's encoder are separate code; they
    must produce identical bytes, including constructed half-way cases."""
    w = gen.normal((128, 1024), seed=11, idx=0, std=0.02)
    w[0, :32] = np.arange(32, dtype=np.float32) - 16.5        # many .5 ratios
    w[1, :32] = (np.arange(32, dtype=np.float32) - 15) * np.float32(0.5)
    np.testing.assert_array_equal(gen.to_q8_0(w), K.q8_0_encode(w))


def test_q8_0_accuracy_band():
    """Relative RMSE of Q8_0 on Gaussian weights sits next to the printed
    0.00544127 of the real checkpoint (graysoft.dev page, "Conversion result")."""
    w = gen.normal((256, 7168), seed=13, idx=0, std=0.02)
    d = K.q8_0_decode(K.q8_0_encode(w), 256, 7168)
    rel = np.sqrt(np.mean((d - w) ** 2)) / np.sqrt(np.mean(w.astype(np.float64) ** 2))
    assert 0.0045 < rel < 0.0065


def test_q8_0_size_pins_printed_file():
    """34 bytes per 32 weights reproduces the printed Q8_0 conversion
    (graysoft.dev page, "Conversion result": 2,249,289,601 parameters,
    38 Q8_0 + 24 F32 tensors, 2,390,153,888 output bytes, 4,498,585,858 BF16
    source bytes) for that card's 64-query / 16-KV, head-dim-64 geometry
    ("Architecture metadata"); the remainder is file header."""
    H, inter, V, R = 7168, 14336, 163840, 256
    q8 = [H * 5 * H]
    for _ in range(5):
        q8 += [64 * 64 * H, 16 * 64 * H, 16 * 64 * H, H * 64 * 64, inter * H, inter * H, H * inter]
    q8 += [V * R, V * R]
    f32 = [H, H, 64, 64] * 5 + [H, H, H + R, 1]
    assert len(q8) == 38 and len(f32) == 24
    params = sum(q8) + sum(f32)
    assert params == 2_249_289_601
    q8_bytes = sum(q8) // K.Q8_BLOCK * K.Q8_BYTES
    data = q8_bytes + 4 * sum(f32)
    header = 2_390_153_888 - data
    assert 0 < header < 65536                       # 7,324 bytes of GGUF header
    assert 0 < 4_498_585_858 - 2 * params < 65536   # safetensors header
    assert round(100 * 2_390_153_888 / 4_498_585_858, 2) == 53.13


# ------------------------------------------------------------------ FP8 ----
def test_fp8_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([K.e4m3fn_value(int(c)) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_fp8_spec_values():
    v = K.e4m3fn_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest finite
    assert v(0x01) == 2.0 ** -9                             # smallest subnormal
    assert v(0x08) == 2.0 ** -6                             # smallest normal
    assert v(0x38) == 1.0
    vals = [v(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))       # codes ordered by value


def test_fp8_encode_roundtrip_and_vs_torch():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = K._E4M3_TABLE[finite]
    np.testing.assert_array_equal(K.e4m3fn_encode(vals), finite)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(60)
    pos = K._E4M3_TABLE[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)    # exact ties
    x = np.concatenate([x, mids, -mids, np.float32([600, -1e4, 0.0])])
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(K.e4m3fn_encode(x), ref)


def test_fp8_per_channel_scale_factors_out():
    w = gen.normal((32, 256), seed=17, idx=0, std=0.02)
    codes, s = gen.to_fp8_e4m3_per_channel(w)
    x = np.random.default_rng(1).standard_normal(256)
    full = K.fp8_decode(codes, s) @ x
    unit = K.fp8_decode(codes, np.ones_like(s)) @ x
    np.testing.assert_allclose(full, s.astype(np.float64) * unit, rtol=1e-13)
    assert np.abs(K.fp8_decode(codes, s)).max(axis=1) == pytest.approx(np.abs(w).max(axis=1), rel=0.07)


# ------------------------------------------------------------------ bf16 ---
def test_bf16_decode_all_codes_vs_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = K.bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_rne_vs_torch_and_generator():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000).astype(np.float32)
    ties = (np.arange(1, 2001, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(K.bf16_encode(x), ref)
    np.testing.assert_array_equal(gen.to_bf16_bits(x), ref)


# ---------------------------------------------------------------- MXFP4 ----
def test_e2m1_values_are_the_mx_element_set():
    """FP4 E2M1 as the OCP MX format defines it: the 8 magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit; codes ordered by value."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [K.e2m1_value(c) for c in range(8)] == mags
    assert [K.e2m1_value(c | 8) for c in range(8)] == [-m for m in mags]


def test_e8m0_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([K.e8m0_value(int(c)) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127


def test_mxfp4_hand_block_layout():
    """amax 3 -> shared exponent floor(log2 3) - 2 = -1 (code 126, X = 0.5);
    element 2i in the low nibble of byte 1 + i."""
    w = np.zeros((1, 64), np.float32)
    w[0, :8] = [3.0, -0.5, 0.25, 1.0, 0.0, -3.0, 2.0, 0.75]
    b = K.mxfp4_encode(w)
    assert b.shape == (1, 34)
    assert b[0, 0] == 126
    # x / X = 6, -1, 0.5, 2, 0, -6, 4, 1.5 -> codes 7, 0xA, 1, 4, 0, 0xF, 6, 3
    assert list(b[0, 1:5]) == [0xA7, 0x41, 0xF0, 0x36]
    assert b[0, 17] == 0 and not b[0, 18:].any()         # all-zero block: exponent -127
    np.testing.assert_array_equal(K.mxfp4_decode(b, 1, 64)[0, :8], w[0, :8])


def test_mxfp4_rounding_ties_and_saturation():
    """Nearest element, ties to the even code, saturation at 6 (block amax in
    [4, 8) gives X = 1, so x / X = x)."""
    cases = [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0),
             (5.01, 6.0), (0.2, 0.0), (0.26, 0.5), (7.9, 6.0), (-2.5, -2.0), (-5.0, -4.0), (-7.0, -6.0)]
    w = np.zeros((len(cases), 32), np.float32)
    for i, (x, _) in enumerate(cases):
        w[i, 0] = x
        w[i, 1] = 7.99 if abs(x) < 4 else 0.0           # pins the block amax inside [4, 8)
    d = K.mxfp4_decode(K.mxfp4_encode(w), len(cases), 32)
    assert list(d[:, 0]) == [want for _, want in cases]


def test_mxfp4_scales_and_roundtrip():
    """Scaling a block by 2^k moves only its scale code; decoding then
    re-encoding is the identity on blocks."""
    w = gen.normal((64, 256), seed=21, idx=0, std=0.02)
    b = K.mxfp4_encode(w)
    b2 = K.mxfp4_encode(w * np.float32(8.0))
    np.testing.assert_array_equal(b2[:, 1:17], b[:, 1:17])
    assert np.all(b2.reshape(64, 8, 17)[:, :, 0] == b.reshape(64, 8, 17)[:, :, 0] + 3)
    d = K.mxfp4_decode(b, 64, 256)
    np.testing.assert_array_equal(K.mxfp4_encode(d.astype(np.float32)), b)


def test_weight_snr_matches_the_printed_table():
    """Weight SNR of the codecs on Gaussian weights sits at the values the
    huggingface.co "Kimi-K3-DSpark-NVFP4" page prints in "Detail" (measured
    there on the trained drafter): MXFP4 19.0 dB, FP8 31.5 dB.  A scale
    exponent off by one moves MXFP4 by 1.5 dB or more."""
    w = gen.normal((256, 7168), seed=13, idx=0, std=0.02)
    w64 = w.astype(np.float64)

    def snr(d):
        return 10 * np.log10(np.sum(w64 ** 2) / np.sum((d - w64) ** 2))

    mx = snr(K.mxfp4_decode(K.mxfp4_encode(w), 256, 7168))
    codes, s = gen.to_fp8_e4m3_per_channel(w)
    f8 = snr(K.fp8_decode(codes, s))
    assert 18.5 < mx < 19.5, mx
    assert 31.0 < f8 < 32.0, f8


def test_mxfp4_two_encoders_agree():
    w = gen.normal((96, 1024), seed=23, idx=0, std=0.02)
    w[0, :32] = np.arange(32, dtype=np.float32) * np.float32(0.25)   # ties on every grid
    w[1, :32] = -(np.arange(32, dtype=np.float32) - 3) * np.float32(0.125)
    w[2, :32] = 0.0
    np.testing.assert_array_equal(gen.to_mxfp4(w), K.mxfp4_encode(w))
