"""The device's e4m3fn codec (the fp8 cache's format), bit for bit against the oracle's.

Inputs: every finite code value of both signs, the midpoint between each pair of neighbouring
codes (a tie: round to the even code) and values just above and below each midpoint, values
beyond the largest code (saturation at 448), zeros of both signs, NaN, and a seeded spread of
magnitudes from far below the smallest subnormal to above the range.  The expected codes are the
oracle's round-to-nearest-even quantiser (already pinned against torch's float8_e4m3fn on the CPU).
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_compress_amd import api
from oracle import numerics

pytestmark = pytest.mark.gpu


def code_values():
    """fp64 value of each of the 256 codes (NaN for 0x7F / 0xFF)."""
    v = np.empty(256)
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        if (c & 0x7F) == 0x7F:
            v[c] = np.nan
            continue
        mag = (1 + m / 8) * 2.0 ** (e - 7) if e else m * 2.0 ** -9
        v[c] = -mag if c & 0x80 else mag
    return v


def oracle_code(x):
    """Code of the oracle's quantised value of fp32 x (NaN -> 0x7F / 0xFF)."""
    vals = code_values()
    out = np.empty(len(x), dtype=np.uint8)
    for i, xi in enumerate(np.asarray(x, dtype=np.float64)):
        neg = np.signbit(xi)
        if np.isnan(xi):
            out[i] = 0xFF if neg else 0x7F
            continue
        q = float(numerics.e4m3_quantise(np.array([xi]))[0])
        mag = abs(q)
        c = int(np.nonzero(vals[:127] == mag)[0][0])
        out[i] = c | (0x80 if neg else 0)
    return out


def run(fn, x, out_dtype):
    xs = torch.as_tensor(x).cuda()
    out = torch.empty(len(x), dtype=out_dtype, device="cuda")
    st = getattr(api.lib(), fn)(api._ptr(xs), api._ptr(out), len(x), api._stream(None))
    assert st == 0, api.STATUS.get(st, st)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_encode_every_code_tie_and_edge():
    vals = code_values()
    finite = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))          # 0 .. 448, 127 magnitudes
    mids = (finite[1:] + finite[:-1]) / 2
    xs = [finite, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
          np.nextafter(mids.astype(np.float32), np.float32(0)), [448.0, 449.0, 464.0, 465.0, 480.0, 1e6, 3e38],
          [2.0 ** -10, 2.0 ** -11, 2.0 ** -9 * 0.5000001, 1e-30, 2.0 ** -126]]
    pos = np.concatenate([np.asarray(a, dtype=np.float64) for a in xs]).astype(np.float32)
    g = np.random.default_rng(0)
    spread = (g.choice([-1.0, 1.0], 4096) * 2.0 ** g.uniform(-14, 10, 4096)).astype(np.float32)
    x = np.concatenate([pos, -pos, spread, np.array([0.0, -0.0, np.nan, -np.nan], np.float32)])
    got = run("mla_fp8_e4m3_encode", x, torch.uint8)
    want = oracle_code(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]
    # ties went to the even code (mantissa bit 0 clear), both signs
    tie_codes = got[len(finite):len(finite) + len(mids)]
    assert np.all((tie_codes & 1) == 0)


def test_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = run("mla_fp8_e4m3_decode", codes, torch.float32).astype(np.float64)
    want = code_values()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))      # -0 stays -0
    # the round trip of every finite code is the identity
    back = run("mla_fp8_e4m3_encode", got[~nan].astype(np.float32), torch.uint8)
    assert np.array_equal(back, codes[~nan])
