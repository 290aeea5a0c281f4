"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the property it checks.  A plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, normalising the wrong slice, rotating the wrong
pairs) fails at least one of them; the scalar brute force in test_oracle_bruteforce.py covers
the rest of the wiring.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Dims

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mtrt_dimensions.json")


def dims_236b(**kw):
    return Dims(5120, 128, 1536, 512, 128, 64, 128, **kw)


SHAPES = {
    "tiny": Dims(256, 4, 96, 64, 32, 16, 32),
    "lite": Dims(2048, 16, 0, 512, 128, 64, 128),
    "dsv2": dims_236b(),
}


def rand_weights(d, seed, gamma_random=False):
    g = np.random.default_rng(seed)
    H = d.heads

    def gain(n):
        return 1.0 + 0.1 * g.standard_normal(n) if gamma_random else np.ones(n)

    W = {}
    if d.q_lora_rank:
        W["q_a_proj"] = 0.02 * g.standard_normal((d.q_lora_rank, d.hidden))
        W["q_a_norm"] = gain(d.q_lora_rank)
        W["q_b_proj"] = 0.02 * g.standard_normal((H * (d.qk_nope + d.qk_rope), d.q_lora_rank))
    else:
        W["q_proj"] = 0.02 * g.standard_normal((H * (d.qk_nope + d.qk_rope), d.hidden))
    W["kv_a_proj"] = 0.02 * g.standard_normal((d.kv_lora_rank + d.qk_rope, d.hidden))
    W["kv_a_norm"] = gain(d.kv_lora_rank)
    W["kv_b_proj"] = 0.02 * g.standard_normal((H * (d.qk_nope + d.v_head), d.kv_lora_rank))
    return W


# ---------------------------------------------------------------- P1: cache geometry (page table)
def test_p1_cache_geometry_matches_page_table():
    g = json.load(open(GOLDEN))
    d = Dims(g["hidden_size"], g["num_heads"], g["q_lora_rank"], g["kv_lora_rank"],
             g["k_nope_per_head"], g["qk_rope_head_dim"], g["v_per_head"])
    assert d.qk_nope + d.qk_rope == g["query_head_dim"]
    # Values cached per token: the width of the rows the oracle's compression produces.
    small = Dims(64, d.heads, 0, d.kv_lora_rank, d.qk_nope, d.qk_rope, d.v_head)
    W = {"kv_a_proj": np.random.default_rng(0).standard_normal((d.kv_lora_rank + d.qk_rope, 64)),
         "kv_a_norm": np.ones(d.kv_lora_rank)}
    rows = oracle.kv_rows(small, W, np.ones((3, 64)), np.arange(3))
    assert rows.shape == (3, g["mla_values_per_token_per_layer"]) and d.row_width == rows.shape[1]
    # Values an uncompressed cache would hold: what decompression yields per token, all heads.
    kvb = {"kv_b_proj": np.zeros((d.heads * (d.qk_nope + d.v_head), 1))}
    per_token = sum(w.shape[0] for h in range(d.heads) for w in oracle.head_weights(d, kvb, h))
    assert per_token == g["mha_values_per_token_per_layer"] == d.mha_width
    assert d.row_width * 2 == 1152            # bf16 bytes per cached token
    assert d.row_width * 1 + 4 == 580         # e4m3 codes + one fp32 scale


# ---------------------------------------------------------------- P6: RoPE
def test_p6_rope_closed_forms():
    d = 64
    u = np.random.default_rng(1).standard_normal((5, d))
    np.testing.assert_array_equal(oracle.rope(u, np.zeros(5), 10000.0), u)           # position 0
    r = oracle.rope(u, np.arange(5) * 977, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(u, axis=1), rtol=1e-14)
    for i in (0, 1, 17, 31):
        e = np.zeros(d)
        e[2 * i] = 1.0
        p = 131071
        th = 10000.0 ** (-2.0 * i / d)
        out = oracle.rope(e, np.array(p), 10000.0)
        exp = np.zeros(d)
        exp[2 * i], exp[2 * i + 1] = math.cos(p * th), math.sin(p * th)
        np.testing.assert_allclose(out, exp, atol=1e-12)
        e2 = np.zeros(d)
        e2[2 * i + 1] = 1.0        # the odd partner rotates to (-sin, cos)
        out2 = oracle.rope(e2, np.array(p), 10000.0)
        exp2 = np.zeros(d)
        exp2[2 * i], exp2[2 * i + 1] = -math.sin(p * th), math.cos(p * th)
        np.testing.assert_allclose(out2, exp2, atol=1e-12)


def test_p6_rope_relative_position():
    g = np.random.default_rng(2)
    q, k = g.standard_normal(64), g.standard_normal(64)
    dots = [oracle.rope(q, np.array(m), 1e4) @ oracle.rope(k, np.array(m - 37), 1e4) for m in (37, 100, 5000, 131072)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


# YaRN (the pages name YaRN as the route to the 128K context but give no constants; the pins
# below fix what the method guarantees whatever the constants).
YARN = dict(factor=40.0, original=4096, beta_fast=32.0, beta_slow=1.0)


def test_p6_yarn_off_is_plain_rope():
    g = np.random.default_rng(4)
    u = g.standard_normal((3, 64))
    pos = np.array([5, 4000, 131071])
    for factor in (0.0, 1.0, 0.5):
        np.testing.assert_array_equal(oracle.rope(u, pos, 1e4, factor=factor, original=4096, beta_fast=32.0,
                                                  beta_slow=1.0), oracle.rope(u, pos, 1e4))


def test_p6_yarn_by_parts_limits():
    """Fast pairs (many turns over the original context) keep their rotation; slow pairs (under
    beta_slow turns) are position-interpolated: at position s * p they turn as plain RoPE at p."""
    d, s = 64, YARN["factor"]
    f = 1e4 ** (-2.0 * np.arange(d // 2) / d)
    turns = YARN["original"] * f / (2 * math.pi)
    fast, slow = np.where(turns >= 32.0)[0], np.where(turns <= 1.0)[0]
    assert len(fast) >= 10 and len(slow) >= 4 and 0 in fast and d // 2 - 1 in slow
    g = np.random.default_rng(5)
    u = g.standard_normal(d)
    for p in (1, 777, 50000):
        y = oracle.rope(u, np.array(p), 1e4, **YARN)
        plain = oracle.rope(u, np.array(p), 1e4)
        stretched = oracle.rope(u, np.array(p * s), 1e4, **YARN)
        for i in fast:
            np.testing.assert_allclose(y[2 * i:2 * i + 2], plain[2 * i:2 * i + 2], rtol=0, atol=1e-12)
        for i in slow:
            np.testing.assert_allclose(stretched[2 * i:2 * i + 2], plain[2 * i:2 * i + 2], rtol=0, atol=1e-9)
    fy = oracle.rope_frequencies(d, 1e4, **YARN)
    assert np.all(np.diff(fy) < 0)                      # still strictly slower towards the last pair
    assert np.all(fy <= f) and np.all(fy >= f / s)      # between position interpolation and none


def test_p6_yarn_ramp_interior_by_hand():
    """Inside the ramp the frequency is linear in the turn count r: for d = 4 and base 100 the
    pairs turn at f = 1 and f = 0.1; with an original context of 170 pi, pair 1 makes r = 8.5
    turns, halfway from beta_slow = 1 to beta_fast = 16 (g = 1/2), so at factor s = 4 it turns
    at (1/2)(0.1 / 4) + (1/2)(0.1) = 0.0625; with 95 pi it makes 4.75 turns (g = 1/4) and turns
    at (3/4)(0.1 / 4) + (1/4)(0.1) = 0.04375.  Pair 0 (85 and 47.5 turns, above beta_fast)
    keeps f = 1.  (A ramp running the other way, or over the pair index, gives other values.)"""
    kw = dict(factor=4.0, beta_fast=16.0, beta_slow=1.0)
    np.testing.assert_allclose(oracle.rope_frequencies(4, 100.0, original=170 * math.pi, **kw), [1.0, 0.0625],
                               rtol=1e-12)
    np.testing.assert_allclose(oracle.rope_frequencies(4, 100.0, original=95 * math.pi, **kw), [1.0, 0.04375],
                               rtol=1e-12)


def test_p6_yarn_relative_position_and_mscale():
    g = np.random.default_rng(6)
    q, k = g.standard_normal(64), g.standard_normal(64)
    dots = [oracle.rope(q, np.array(m), 1e4, **YARN) @ oracle.rope(k, np.array(m - 37), 1e4, **YARN)
            for m in (37, 100, 5000, 131072)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)
    m = 1.3
    scaled = oracle.rope(q, np.array(900), 1e4, mscale=m, **YARN) @ oracle.rope(k, np.array(11), 1e4, mscale=m, **YARN)
    plain = oracle.rope(q, np.array(900), 1e4, **YARN) @ oracle.rope(k, np.array(11), 1e4, **YARN)
    np.testing.assert_allclose(scaled, m * m * plain, rtol=1e-12)


# ---------------------------------------------------------------- P7: RMSNorm
def test_p7_rmsnorm_closed_form():
    g = np.random.default_rng(3)
    c = g.standard_normal((7, 512)) * np.array([[1e-3], [1e-2], [0.1], [1], [3], [10], [100]])
    eps = 1e-6
    ch = oracle.rms_norm(c, np.ones(512), eps)
    ms = np.mean(c * c, axis=1)
    np.testing.assert_allclose(np.mean(ch * ch, axis=1), 1.0 / (1.0 + eps / ms), rtol=1e-13)
    gam = g.standard_normal(512)
    np.testing.assert_allclose(oracle.rms_norm(c, gam, eps), ch * gam, rtol=1e-13)
    # scale invariance up to eps: doubling the input leaves a large-norm row unchanged
    np.testing.assert_allclose(oracle.rms_norm(2 * c[4:], np.ones(512), 0.0), oracle.rms_norm(c[4:], np.ones(512), 0.0), rtol=1e-13)


# ---------------------------------------------------------------- compression layout
def test_compress_split_and_norm_slice():
    """kv_a output is [latent | k_pe]; only the latent is normalised; only k_pe is rotated."""
    d = Dims(12, 2, 0, 8, 4, 4, 4)
    W = {"kv_a_proj": np.eye(12), "kv_a_norm": np.ones(8)}
    x = np.random.default_rng(4).standard_normal((3, 12)) * 5
    pos = np.array([0, 3, 11])
    rows = oracle.kv_rows(d, W, x, pos)
    np.testing.assert_allclose(rows[:, :8], x[:, :8] / np.sqrt(np.mean(x[:, :8] ** 2, axis=1, keepdims=True) + 1e-6), rtol=1e-13)
    np.testing.assert_allclose(rows[0, 8:], x[0, 8:], rtol=1e-15)                        # position 0
    np.testing.assert_allclose(np.linalg.norm(rows[:, 8:], axis=1), np.linalg.norm(x[:, 8:], axis=1), rtol=1e-13)
    assert not np.allclose(rows[1:, 8:], x[1:, 8:])


# ---------------------------------------------------------------- P2: absorbed == explicit
@pytest.mark.parametrize("name", list(SHAPES))
def test_p2_absorbed_equals_explicit(name):
    d = SHAPES[name]
    W = rand_weights(d, 5, gamma_random=True)
    g = np.random.default_rng(6)
    n = 37
    x = g.standard_normal((n, d.hidden))
    rows = oracle.kv_rows(d, W, x, np.arange(n))
    qn, qp = oracle.queries(d, W, x[-2:], np.array([n - 2, n - 1]))
    heads = range(d.heads) if d.heads <= 16 else [0, 1, 63, 127]
    a = oracle.attend_explicit(d, W, qn, qp, rows, heads=heads)
    b = oracle.attend_absorbed(d, W, qn, qp, rows, heads=heads)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.sqrt(np.mean(a * a))


# ---------------------------------------------------------------- P3: softmax normalisation
def test_p3_probabilities_sum_to_one():
    d = SHAPES["tiny"]
    W = rand_weights(d, 7)
    x = np.random.default_rng(8).standard_normal((50, d.hidden)) * 3
    rows = oracle.kv_rows(d, W, x, np.arange(50))
    qn, qp = oracle.queries(d, W, x, np.arange(50))
    _, p = oracle.attend_explicit(d, W, qn, qp, rows, return_probs=True, causal_limit=np.arange(50) + 1)
    np.testing.assert_allclose(p.sum(axis=2), 1.0, atol=1e-14)
    hidden = np.broadcast_to((np.arange(50)[None, :] > np.arange(50)[:, None])[:, None, :], p.shape)
    assert np.all(p[hidden] == 0) and np.all(p[~hidden] > 0)


def test_p3_constant_latent_returns_its_value():
    """If every cached latent is the same c, each head outputs W_UV^h c whatever the scores."""
    d = SHAPES["tiny"]
    W = rand_weights(d, 9)
    g = np.random.default_rng(10)
    c = g.standard_normal(d.kv_lora_rank)
    rows = np.concatenate([np.tile(c, (29, 1)), g.standard_normal((29, d.qk_rope)) * 4], axis=1)
    qn, qp = g.standard_normal((3, d.heads, d.qk_nope)) * 5, g.standard_normal((3, d.heads, d.qk_rope)) * 5
    out = oracle.attend_explicit(d, W, qn, qp, rows)
    for h in range(d.heads):
        np.testing.assert_allclose(out[:, h], np.tile(oracle.head_weights(d, W, h)[1] @ c, (3, 1)), rtol=1e-12)


# ---------------------------------------------------------------- P4: length-1 context
def test_p4_single_row_context_returns_its_v():
    d = SHAPES["tiny"]
    W = rand_weights(d, 11)
    x = np.random.default_rng(12).standard_normal(d.hidden)
    out, row = oracle.decode_one(d, W, x, np.zeros((0, d.row_width)), "f32")
    for h in range(d.heads):
        np.testing.assert_allclose(out[h], oracle.head_weights(d, W, h)[1] @ row[: d.kv_lora_rank], rtol=1e-13)


# ---------------------------------------------------------------- scores: a peaked softmax selects
def test_peaked_scores_select_the_matching_key():
    d = Dims(8, 1, 0, 8, 4, 4, 4, softmax_scale=1.0)
    W = {"kv_b_proj": np.vstack([np.eye(4, 8), np.eye(4, 8, 4)])}  # k_nope = c[:4], v = c[4:]
    g = np.random.default_rng(13)
    rows = g.standard_normal((6, 12))
    qn = 60.0 * rows[3, :4][None, None, :] / np.linalg.norm(rows[3, :4])
    qp = np.zeros((1, 1, 4))
    out = oracle.attend_explicit(d, W, qn, qp, rows)
    np.testing.assert_allclose(out[0, 0], rows[3, 4:8], atol=1e-6)
    # the shared RoPE key contributes with a + sign: a q_pe aligned with row 1's k_pe selects it
    out2 = oracle.attend_explicit(d, W, np.zeros((1, 1, 4)), 60.0 * rows[1, 8:][None, None, :] / np.linalg.norm(rows[1, 8:]), rows)
    np.testing.assert_allclose(out2[0, 0], rows[1, 4:8], atol=1e-6)


# ---------------------------------------------------------------- output projection (o_proj reading)
def test_output_projection_selects_head_major_inputs():
    """A 0/1 o_proj that picks input j_i for output i returns head j_i // d_v's entry j_i % d_v
    (heads side by side in head order): a transposed weight, or heads interleaved feature-major,
    picks other entries (the selection is not an involution and rows differ from columns)."""
    d = Dims(10, 3, 0, 8, 4, 4, 4)                      # H * d_v = 12 inputs, 10 outputs
    o = np.array([[[100 * h + j + 0.5 for j in range(d.v_head)] for h in range(d.heads)]], dtype=np.float64)
    pick = np.random.default_rng(31).permutation(d.heads * d.v_head)[: d.hidden]
    w = np.zeros((d.hidden, d.heads * d.v_head))
    w[np.arange(d.hidden), pick] = 1.0
    out = oracle.output_projection(d, {"o_proj": w}, o)
    assert out.shape == (1, d.hidden)
    np.testing.assert_array_equal(out[0], [100 * (j // d.v_head) + j % d.v_head + 0.5 for j in pick])


def test_output_projection_brute_force():
    """Against a scalar triple loop (output i = sum over heads h and features j of
    o_proj[i][h d_v + j] o[h][j]) on a small random case, two tokens at once."""
    d = Dims(6, 3, 0, 8, 4, 4, 5)
    g = np.random.default_rng(32)
    o = g.standard_normal((2, d.heads, d.v_head))
    w = g.standard_normal((d.hidden, d.heads * d.v_head))
    want = np.zeros((2, d.hidden))
    for t in range(2):
        for i in range(d.hidden):
            for h in range(d.heads):
                for j in range(d.v_head):
                    want[t, i] += w[i, h * d.v_head + j] * o[t, h, j]
    np.testing.assert_allclose(oracle.output_projection(d, {"o_proj": w}, o), want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- P10 / P11: causality and chunking
def test_p10_causality():
    d = SHAPES["tiny"]
    W = rand_weights(d, 14, gamma_random=True)
    x = np.random.default_rng(15).standard_normal((20, d.hidden))
    out, _ = oracle.prefill_chunk(d, W, x, 0, np.zeros((0, d.row_width)), "f32")
    x2 = x.copy()
    x2[12:] += 3.0
    out2, _ = oracle.prefill_chunk(d, W, x2, 0, np.zeros((0, d.row_width)), "f32")
    np.testing.assert_array_equal(out[:12], out2[:12])
    assert not np.allclose(out[12:], out2[12:])


@pytest.mark.parametrize("chunk", [1, 3, 8])
def test_p11_chunked_equals_whole_and_matches_decode(chunk):
    d = SHAPES["tiny"]
    W = rand_weights(d, 16, gamma_random=True)
    x = np.random.default_rng(17).standard_normal((16, d.hidden))
    whole, whole_rows = oracle.prefill_chunk(d, W, x, 0, np.zeros((0, d.row_width)), "f32")
    rows = np.zeros((0, d.row_width))
    outs = []
    for s in range(0, 16, chunk):
        o, r = oracle.prefill_chunk(d, W, x[s:s + chunk], s, rows, "f32")
        outs.append(o)
        rows = np.concatenate([rows, r])
    np.testing.assert_allclose(np.concatenate(outs), whole, rtol=1e-9, atol=1e-12)
    dec, _ = oracle.decode_one(d, W, x[-1], whole_rows[:-1], "f32")
    np.testing.assert_allclose(dec, whole[-1], rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- P13: bf16 rounding
def test_p13_bf16_matches_torch():
    g = np.random.default_rng(18)
    x = np.concatenate([g.standard_normal(100000) * 10 ** g.uniform(-30, 30, 100000),
                        [0.0, -0.0, 1.0, 1e-40, -3e-39]]).astype(np.float32)
    bits = g.integers(0, 2 ** 31, 5000).astype(np.uint32)
    ties = ((bits & 0x7F7F0000) | 0x00008000).view(np.float32)     # exactly halfway cases
    ties = ties[np.abs(ties) < 1e38]          # keep clear of rounding up to infinity
    for arr in (x, ties):
        ref = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(oracle.bf16_round(arr.astype(np.float64)), ref)


# ---------------------------------------------------------------- P12: e4m3 codec
def test_p12_e4m3_code_roundtrip_and_library():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    vals = oracle.e4m3_decode_codes(codes)
    np.testing.assert_array_equal(oracle.e4m3_quantise(vals), vals)
    np.testing.assert_array_equal(oracle.e4m3_encode_values(vals), codes)
    assert np.max(vals) == 448.0 and np.min(vals[vals > 0]) == 2.0 ** -9
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(lib, vals)


def test_p12_e4m3_rounding_and_saturation():
    g = np.random.default_rng(19)
    v = (g.standard_normal(200000) * 10 ** g.uniform(-4, 2.6, 200000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    q = oracle.e4m3_quantise(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(q, ref)
    # error within half a step of the local e4m3 spacing
    a = np.abs(v.astype(np.float64))
    step = np.ldexp(1.0, np.maximum(np.frexp(a)[1] - 1, -6) - 3)
    assert np.all(np.abs(q - v) <= step / 2)
    np.testing.assert_array_equal(oracle.e4m3_quantise(np.array([449.0, 470.0, 1e9, -500.0])), [448.0, 448.0, 448.0, -448.0])


def test_fp8_store_scale():
    g = np.random.default_rng(20)
    rows = g.standard_normal((50, 576)) * 10 ** g.uniform(-3, 3, (50, 1))
    vals, codes, scale = oracle.fp8_store(rows)
    amax = np.max(np.abs(rows.astype(np.float32)), axis=1)
    np.testing.assert_allclose(scale, amax / 448.0, rtol=1e-7)
    assert np.all(np.max(np.abs(oracle.e4m3_decode_codes(codes)), axis=1) == 448.0)
    np.testing.assert_allclose(np.max(np.abs(vals), axis=1), amax, rtol=1e-6)
    rel = np.abs(vals - rows) / amax[:, None]
    assert np.max(rel) <= 2.0 ** -4 * 1.0001       # at most half a step of the top binade
    z_vals, z_codes, z_scale = oracle.fp8_store(np.zeros((1, 576)))
    assert z_scale[0] == 1.0 and np.all(z_codes == 0) and np.all(z_vals == 0)


def test_batched_absorbed_reference_matches_explicit():
    """The full-size decode tests' all-heads reference (the absorbed form with the heads batched,
    tests/mla_ref.py) equals the explicit oracle on random rows and queries (tiny and Lite shapes,
    every head)."""
    from mla_latent_kv_compress_amd import inputs
    from mla_latent_kv_compress_amd.configs import LITE, TINY
    from mla_ref import absorbed_all_heads, oracle_dims, oracle_weights, rel_err

    class _Layer:
        pass

    for shape, act in ((TINY, "f32"), (LITE, "bf16")):
        layer = _Layer()
        layer.shape, layer.act = shape, act
        layer.w_host = inputs.make_weights(shape, act, 3)
        d, W = oracle_dims(shape), oracle_weights(layer)
        g = np.random.default_rng(1)
        rows = g.standard_normal((300, d.row_width))
        qn, qp = g.standard_normal((d.heads, d.qk_nope)), g.standard_normal((d.heads, d.qk_rope))
        got = absorbed_all_heads(layer, rows, qn, qp)
        ref = oracle.attend_explicit(d, W, qn[None], qp[None], rows)[0]
        assert rel_err(got, ref) < 1e-12
