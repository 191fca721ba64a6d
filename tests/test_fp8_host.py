"""The kernels' FP8 E4M3 -> fp16 conversion, emulated bit for bit on the CPU.

The kernels place a byte's 7 magnitude bits at bits 7..13 of an fp16 (which
then reads as (1 + f/8) 2^(e-15), or f 2^-17 for e = 0), multiply by 2^8 in
fp16 and put the sign at bit 15.  Every finite E4M3 value must come out
exactly, including the subnormals (f 2^-9), whose intermediate is an fp16
subnormal.
"""
import numpy as np

import oracle


def kernel_conversion(b):
    b = np.asarray(b, np.uint16)
    mag = ((b & 0x7F) << 7).astype(np.uint16).view(np.float16)
    scaled = (mag * np.float16(256.0)).astype(np.float16).view(np.uint16)
    return (scaled | ((b & 0x80) << 8)).astype(np.uint16).view(np.float16)


def test_every_finite_e4m3_byte_converts_exactly():
    b = np.arange(256, dtype=np.uint8)
    ref = oracle.fp8_e4m3_to_float64(b)
    ok = ~np.isnan(ref)
    got = kernel_conversion(b).astype(np.float64)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_two_bytes_per_word_layout():
    """The packed form: bytes 0 and 1 of a 32-bit word go to the low and the
    high fp16 of the result (bits 7..14 and 23..30 before the scaling)."""
    w = np.uint32(0x0000B83C)          # byte 0 = 0x3C (1.5), byte 1 = 0xB8 (-1.0)
    mag = np.uint32(((w & 0x7F) << 7) | ((w & 0x7F00) << 15))
    pair = np.array([mag], np.uint32).view(np.float16) * np.float16(256.0)
    bits = pair.view(np.uint32)[0] | np.uint32(((w & 0x80) << 8) | ((w & 0x8000) << 16))
    lo, hi = np.array([bits], np.uint32).view(np.float16)
    assert (float(lo), float(hi)) == (1.5, -1.0)
