"""Pins for the oracle's q8_0 codec (CPU only)."""
import math
import struct

import numpy as np
import pytest

import oracle
import synth


def f32(v: float) -> float:
    """Round a Python float to the nearest float32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def f16_bits(v: float) -> int:
    return struct.unpack("<H", struct.pack("<e", v))[0]


def scalar_encode_block(xs):
    """Independent scalar q8_0 encode: every float32 operation done in float64 and rounded
    once to float32 (exact for * and correctly rounded for / since 53 >= 2*24 + 2)."""
    xs = [f32(v) for v in xs]
    amax = max(abs(v) for v in xs)
    d = f32(amax / 127.0)
    inv = f32(1.0 / d) if d != 0.0 else 0.0
    qs = []
    for v in xs:
        p = f32(v * inv)
        r = math.floor(abs(p) + 0.5)
        qs.append(int(math.copysign(r, p)) if r else 0)
    return f16_bits(d), qs


def test_tie_vector_rounds_half_away_from_zero():
    blk = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5] + [0.0] * 24
    d16, q = oracle.q8_0_encode(np.array(blk, np.float32))
    assert float(d16[0]) == 1.0
    assert list(q[0, :8]) == [127, 3, -3, 1, -1, 2, -2, 127]
    assert np.all(q[0, 8:] == 0)


def test_zero_block_and_amax_maps_to_127():
    d16, q = oracle.q8_0_encode(np.zeros(64, np.float32))
    assert np.all(d16 == 0) and np.all(q == 0)
    x = synth.normal(7, (4, 96))
    d16, q = oracle.q8_0_encode(x)
    xb = x.reshape(4, 3, 32)
    am = np.argmax(np.abs(xb), axis=-1)
    qa = np.take_along_axis(q, am[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(qa) == 127)
    assert np.all(np.sign(qa) == np.sign(np.take_along_axis(xb, am[..., None], -1)[..., 0]))


@pytest.mark.parametrize("seed,scale", [(1, 0.02), (2, 1.0), (3, 1e-6), (4, 3e-9), (5, 2e4)])
def test_matches_scalar_rederivation(seed, scale):
    x = synth.uniform(seed, (40, 32), -1.0, 1.0) * np.float32(scale)
    # plant exact ties: make element 1 of a few blocks land on k + 1/2 after scaling
    d16, q = oracle.q8_0_encode(x)
    for r in range(x.shape[0]):
        bits, qs = scalar_encode_block(x[r].tolist())
        assert int(d16[r, 0].view(np.uint16)) == bits
        assert list(q[r, 0]) == qs


def test_subnormal_scale_blocks():
    x = np.full(32, 3e-5, np.float32)      # d = amax/127 ~ 1e-6: an fp16 subnormal
    x[3] = -1.3e-4
    d16, q = oracle.q8_0_encode(x)
    bits, qs = scalar_encode_block(x.tolist())
    assert int(d16[0].view(np.uint16)) == bits
    assert bits & 0x7C00 == 0 and bits != 0          # fp16 subnormal scale
    assert list(q[0]) == qs


def test_round_trip_bound_and_idempotence():
    x = synth.normal(11, (64, 256), scale=0.7)
    d16, q = oracle.q8_0_encode(x)
    xh = oracle.q8_0_decode(d16, q)
    xb = x.reshape(64, 8, 32).astype(np.float64)
    d = (np.max(np.abs(xb), axis=-1) / 127.0)
    dh = d16.astype(np.float64)
    bound = d / 2 + 127 * np.abs(d - dh) + 4 * np.abs(xb).max(-1) * 2.0 ** -23
    err = np.abs(xh.reshape(64, 8, 32) - xb).max(-1)
    assert np.all(err <= bound)
    d2, q2 = oracle.q8_0_encode(xh)
    assert np.array_equal(d2.view(np.uint16), d16.view(np.uint16))
    assert np.array_equal(q2, q)


def test_interchange_bytes_layout_and_padding():
    x = synth.normal(13, (3, 50))               # K = 50 -> padded to 64 (2 blocks)
    b = oracle.q8_0_encode_bytes(x)
    assert b.shape == (3, 68)
    d16, q = oracle.q8_0_encode(x)
    # block 0 of row 1: little-endian fp16 scale then 32 signed bytes
    assert int(b[1, 0]) | (int(b[1, 1]) << 8) == int(d16[1, 0].view(np.uint16))
    assert np.array_equal(b[1, 2:34].view(np.int8), q[1, 0])
    # padding values quantise to 0 and do not change the second block's scale
    assert np.all(q[:, 1, 18:] == 0)
    xp = np.concatenate([x, np.zeros((3, 14), np.float32)], axis=1)
    d16p, _ = oracle.q8_0_encode(xp)
    assert np.array_equal(d16p.view(np.uint16), d16.view(np.uint16))
    back = oracle.q8_0_decode_bytes(b, 50)
    assert back.shape == (3, 50)
    assert np.array_equal(back, oracle.q8_0_decode(d16, q)[:, :50])
