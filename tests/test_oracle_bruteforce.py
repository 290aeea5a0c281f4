"""P5: the vectorised oracle against a scalar brute force on tiny shapes (CPU only).

The brute force below is written from the method's definition with plain Python loops and the
math module only -- no numpy linear algebra and none of the oracle's helpers -- so that a
transposed operand, a wrong slice or a dropped term in either implementation shows up as a
mismatch.  Both use the same readings (adjacent-pair RoPE, sigma = 1/sqrt(d_n + d_r), decode
token appended before it attends).
"""
import math
import random

import numpy as np
import pytest

import oracle
from oracle import Dims


def lin(Wrows, x):
    return [sum(Wrows[o][i] * x[i] for i in range(len(x))) for o in range(len(Wrows))]


def bf_norm(v, g, eps):
    ms = sum(t * t for t in v) / len(v)
    return [v[i] / math.sqrt(ms + eps) * g[i] for i in range(len(v))]


def bf_rope(u, p, base):
    out = list(u)
    d = len(u)
    for i in range(d // 2):
        a = p * base ** (-2.0 * i / d)
        out[2 * i] = u[2 * i] * math.cos(a) - u[2 * i + 1] * math.sin(a)
        out[2 * i + 1] = u[2 * i] * math.sin(a) + u[2 * i + 1] * math.cos(a)
    return out


def bf_row(d, W, x, p):
    a = lin(W["kv_a_proj"], x)
    lat = bf_norm(a[: d.kv_lora_rank], W["kv_a_norm"], d.rms_eps)
    return lat + bf_rope(a[d.kv_lora_rank:], p, d.rope_theta)


def bf_query(d, W, x, p):
    if d.q_lora_rank:
        q = lin(W["q_b_proj"], bf_norm(lin(W["q_a_proj"], x), W["q_a_norm"], d.rms_eps))
    else:
        q = lin(W["q_proj"], x)
    w = d.qk_nope + d.qk_rope
    heads = []
    for h in range(d.heads):
        qh = q[h * w:(h + 1) * w]
        heads.append(qh[: d.qk_nope] + bf_rope(qh[d.qk_nope:], p, d.rope_theta))
    return heads


def bf_attend(d, W, qheads, rows):
    out = []
    blk = d.qk_nope + d.v_head
    for h in range(d.heads):
        Wk = W["kv_b_proj"][h * blk: h * blk + d.qk_nope]
        Wv = W["kv_b_proj"][h * blk + d.qk_nope:(h + 1) * blk]
        scores, values = [], []
        for r in rows:
            lat, kpe = r[: d.kv_lora_rank], r[d.kv_lora_rank:]
            key = lin(Wk, lat) + list(kpe)
            scores.append(d.sigma * sum(qheads[h][i] * key[i] for i in range(len(key))))
            values.append(lin(Wv, lat))
        m = max(scores)
        e = [math.exp(s - m) for s in scores]
        z = sum(e)
        out.append([sum(e[t] / z * values[t][j] for t in range(len(rows))) for j in range(d.v_head)])
    return out


def rand_w(d, rnd):
    def mat(r, c):
        return [[rnd.gauss(0, 0.3) for _ in range(c)] for _ in range(r)]
    W = {}
    if d.q_lora_rank:
        W["q_a_proj"] = mat(d.q_lora_rank, d.hidden)
        W["q_a_norm"] = [1 + rnd.gauss(0, 0.2) for _ in range(d.q_lora_rank)]
        W["q_b_proj"] = mat(d.heads * (d.qk_nope + d.qk_rope), d.q_lora_rank)
    else:
        W["q_proj"] = mat(d.heads * (d.qk_nope + d.qk_rope), d.hidden)
    W["kv_a_proj"] = mat(d.kv_lora_rank + d.qk_rope, d.hidden)
    W["kv_a_norm"] = [1 + rnd.gauss(0, 0.2) for _ in range(d.kv_lora_rank)]
    W["kv_b_proj"] = mat(d.heads * (d.qk_nope + d.v_head), d.kv_lora_rank)
    return W


def as_np(W):
    return {k: np.array(v, dtype=np.float64) for k, v in W.items()}


CASES = [Dims(12, 2, 6, 8, 4, 4, 4), Dims(10, 3, 0, 6, 2, 4, 5, rope_theta=50.0), Dims(9, 1, 5, 4, 3, 2, 2, softmax_scale=0.7)]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("ctx", [1, 2, 7])
def test_p5_decode_matches_brute_force(case, ctx):
    d = CASES[case]
    rnd = random.Random(100 * case + ctx)
    W = rand_w(d, rnd)
    xs = [[rnd.gauss(0, 1) for _ in range(d.hidden)] for _ in range(ctx)]
    rows = [bf_row(d, W, xs[t], t) for t in range(ctx)]
    ref = bf_attend(d, W, bf_query(d, W, xs[-1], ctx - 1), rows)
    Wn = as_np(W)
    hist = oracle.kv_rows(d, Wn, np.array(xs[:-1]).reshape(ctx - 1, d.hidden), np.arange(ctx - 1)) if ctx > 1 \
        else np.zeros((0, d.row_width))
    got, new_row = oracle.decode_one(d, Wn, np.array(xs[-1]), hist, "f32")
    # the oracle rounds the new row to the f32 cache format; compare its rows unrounded first
    np.testing.assert_allclose(oracle.kv_rows(d, Wn, np.array(xs), np.arange(ctx)), np.array(rows), rtol=1e-12, atol=1e-13)
    rows32 = [list(np.float32(r).astype(np.float64)) for r in rows[-1:]]
    ref32 = bf_attend(d, W, bf_query(d, W, xs[-1], ctx - 1), rows[:-1] + rows32)
    np.testing.assert_allclose(got, np.array(ref32), rtol=1e-11, atol=1e-13)
    assert np.max(np.abs(np.array(ref32) - np.array(ref))) < 1e-5   # rounding one row moves little


@pytest.mark.parametrize("case", range(len(CASES)))
def test_p5_prefill_matches_brute_force(case):
    d = CASES[case]
    rnd = random.Random(7 + case)
    W = rand_w(d, rnd)
    n = 6
    xs = [[rnd.gauss(0, 1) for _ in range(d.hidden)] for _ in range(n)]
    rows = [[float(np.float32(v)) for v in bf_row(d, W, xs[t], t)] for t in range(n)]
    got, _ = oracle.prefill_chunk(d, as_np(W), np.array(xs), 0, np.zeros((0, d.row_width)), "f32")
    for i in range(n):
        ref = bf_attend(d, W, bf_query(d, W, xs[i], i), rows[: i + 1])
        np.testing.assert_allclose(got[i], np.array(ref), rtol=1e-10, atol=1e-12)
