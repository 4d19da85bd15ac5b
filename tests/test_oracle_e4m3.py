"""Pins for the oracle's OCP E4M3 codec: the format's printed points and torch's own cast."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_points.json")


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def test_decode_spec_points():
    d = json.load(open(GOLDEN))
    for code, val in d["decode"]:
        got = float(e4m3.decode(int(code, 16)))
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == val and np.signbit(got) == np.signbit(val), code


def test_encode_spec_points():
    d = json.load(open(GOLDEN))
    for val, code in d["encode"]:
        assert int(e4m3.encode(np.float32(val))) == int(code, 16), (val, code)


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = e4m3.decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_encode_matches_torch_sweep():
    # every finite value, every midpoint between neighbours, and one float32 ulp either side
    vals = np.unique(e4m3.decode(np.arange(0x7F)))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    cands = [vals.astype(np.float32), mids,
             np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))]
    rng = np.random.default_rng(0)
    cands.append(rng.uniform(-448, 448, 200000).astype(np.float32))
    cands.append((rng.standard_normal(200000) * 0.01).astype(np.float32))
    x = np.concatenate(cands)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3.encode(x)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_encode_saturates():
    x = np.array([448.0, 463.9, 464.0, 500.0, 1e6, 3e38], dtype=np.float32)
    assert np.all(e4m3.encode(x) == 0x7E)
    assert np.all(e4m3.encode(-x) == 0xFE)


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(e4m3.decode(codes).astype(np.float32)), codes)
