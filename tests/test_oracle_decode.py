"""Pins for the oracle's row decoders against library routines and the
OCP FP8 definition's landmark values."""
import numpy as np
import torch

from oracle import bf16_decode, decode_rows, e4m3fn_decode


def test_e4m3fn_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_landmarks():
    # largest finite, smallest normal, smallest subnormal, one, negative zero
    assert e4m3fn_decode(np.uint8(0x7E)) == 448.0
    assert e4m3fn_decode(np.uint8(0x08)) == 2.0 ** -6
    assert e4m3fn_decode(np.uint8(0x01)) == 2.0 ** -9
    assert e4m3fn_decode(np.uint8(0x38)) == 1.0
    z = e4m3fn_decode(np.uint8(0x80))
    assert z == 0.0 and np.signbit(z)


def test_bf16_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    special = np.array([0x0000, 0x8000, 0x3F80, 0x0001, 0x7F7F, 0xFF7F], dtype=np.uint16)
    bits = np.concatenate([bits, special])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = bf16_decode(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert bf16_decode(np.uint16(0x3F80)) == 1.0


def test_decode_rows_fp8_scale():
    codes = np.array([[0x38, 0xB8, 0x7E]], dtype=np.uint8)
    out = decode_rows(codes, np.array([0.25], dtype=np.float32), "fp8")
    assert out.tolist() == [[0.25, -0.25, 112.0]]


def test_decode_rows_f32_exact():
    x = np.array([[1.0, np.float32(0.1), -3.5]], dtype=np.float32)
    assert np.array_equal(decode_rows(x, None, "f32"), x.astype(np.float64))
