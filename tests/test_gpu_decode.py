"""GPU parity of mla_compress_append and mla_decode against the fp64 oracle (small shapes).

Sizes are chosen so the oracle finishes in seconds while spanning several 64-token pages, a
ragged last page and the degenerate length-1 context.  Error metric: max|gpu - oracle| /
rms(oracle) with the oracle rounding rows to the cache format; bars 1e-5 (fp32), 2e-2 (bf16),
6e-2 (fp8 cache).  Cache placement and paging are compared bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_compress_amd import api
from mla_latent_kv_compress_amd.configs import DSV2, LITE, TINY, Workload, WORKLOADS
from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer, slots_for
from mla_ref import (TOL, bf16_half_quantum, bf16_out_ok, decode_reference, history_rows, oracle_dims, oracle_weights,
                     rel_err)
from oracle.numerics import e4m3_decode_codes

pytestmark = pytest.mark.gpu


def wl(shape, act, cache, B, **kw):
    return Workload("test", shape, act, cache, decode_batch=B, **kw)


def log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- compress / append
@pytest.mark.parametrize("shape,act,cache", [(TINY, "f32", "f32"), (DSV2, "bf16", "bf16"), (DSV2, "bf16", "fp8"),
                                             (LITE, "bf16", "bf16")])
def test_compress_rows_and_placement(shape, act, cache):
    log(f"compress {shape.hidden_size} {act}/{cache}")
    layer = Layer(shape, act, cache, seed=3)
    nb = 4
    c = layer.new_cache(nb, fill=0xA5)
    if c.scale is not None:
        c.scale.fill_(-7.0)
    T = 70
    g = np.random.default_rng(5)
    from mla_latent_kv_compress_amd import inputs
    x = inputs.history_hidden(shape, 0, 0, T, act, seed=3)
    pos = g.integers(0, 100000, T)
    slots = g.permutation(nb * 64)[:T].astype(np.int64)
    slots[3] = -1                         # skipped
    slots[7] = nb * 64 + 5                # beyond the pool: skipped
    from mla_latent_kv_compress_amd.workload import to_device
    layer.append(c, to_device(x, act, "cuda"), pos, slots)
    torch.cuda.synchronize()
    d, W = oracle_dims(shape), oracle_weights(layer)
    rows64 = oracle.kv_rows(d, W, x.astype(np.float64), pos)          # before the storage rounding
    vals, codes, scale = oracle.store_rows(rows64, cache)
    data = c.data.view(torch.uint8).cpu().numpy().reshape(nb * 64, -1)
    written = np.zeros(nb * 64, bool)
    ok = slots >= 0
    ok &= slots < nb * 64
    written[slots[ok]] = True
    sentinel = np.full(data.shape[1], 0xA5, np.uint8)
    assert np.all(data[~written] == sentinel), "untouched slots must keep their bytes"
    rows = c.data.float().cpu().numpy().reshape(nb * 64, -1) if cache != "fp8" else None
    idx = np.nonzero(ok)[0]
    if cache == "f32":
        np.testing.assert_allclose(rows[slots[idx]], vals[idx], rtol=2e-6, atol=1e-6)
    elif cache == "bf16":
        # Every stored value is the nearest bf16 value (ties to even) of some value within fp32
        # arithmetic error of the fp64 row (2^-18 of the row's rms; measured at most 2^-20):
        # values differ from the oracle's rounding only next to a rounding boundary.
        got = rows[slots[idx]]
        v64 = rows64[idx]
        rms = np.sqrt(np.mean(v64 * v64, axis=1, keepdims=True))
        assert np.all(np.abs(got - v64) <= bf16_half_quantum(v64) + 2.0 ** -18 * rms)
        assert np.mean(got == vals[idx]) > 0.999          # measured: 0.03% differ
    else:
        # Codes differ from the oracle's only where the scaled value (the fp32 row over the fp32
        # scale, the precision both sides decide in) lies within fp32 error of the boundary
        # between the two codes: 448 2^-20 in scaled units (measured at most 7.1e-5).
        gc = data[slots[idx]]
        oc = codes[idx]
        sc = c.scale.cpu().numpy().reshape(-1)
        np.testing.assert_allclose(sc[slots[idx]], scale[idx], rtol=2e-6)
        assert np.all(sc[~written] == -7.0)
        mis = gc != oc
        assert mis.mean() < 1e-3, mis.mean()               # measured: 0.002%
        scaled = (rows64[idx].astype(np.float32) / scale[idx].reshape(-1, 1)).astype(np.float64)
        mid = (e4m3_decode_codes(gc) + e4m3_decode_codes(oc)) / 2
        assert np.all(np.abs(scaled - mid)[mis] <= 448.0 * 2.0 ** -20)


# ---------------------------------------------------------------- decode parity
CASES = {
    "tiny_f32": (TINY, "f32", "f32", [128]),
    "tiny_ragged": (TINY, "f32", "f32", [0, 63, 64, 200]),
    "dsv2_bf16": (DSV2, "bf16", "bf16", [0, 70, 300]),
    "dsv2_fp8": (DSV2, "bf16", "fp8", [0, 70, 300]),
    "lite_bf16": (LITE, "bf16", "bf16", [1, 127, 450]),
    "lite_fp8": (LITE, "bf16", "fp8", [5, 200]),
    "dsv2_fp8_long": (DSV2, "bf16", "fp8", [31, 1000, 2047]),
    # 32 and 48 heads: the narrow instance with two live head tiles, and a partial 64-head group
    "lite32_bf16": (dataclasses.replace(LITE, num_heads=32), "bf16", "bf16", [2, 97, 333]),
    "lite32_fp8": (dataclasses.replace(LITE, num_heads=32), "bf16", "fp8", [40, 255]),
    "lite48_bf16": (dataclasses.replace(LITE, num_heads=48), "bf16", "bf16", [9, 190]),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("splits", [1, 3])
def test_decode_matches_oracle(case, splits):
    shape, act, cache, lengths = CASES[case]
    log(f"decode {case} splits={splits}")
    layer = Layer(shape, act, cache, seed=1)
    batch = DecodeBatch(layer, wl(shape, act, cache, len(lengths)), seed=1, lengths=lengths)
    out = batch.run(num_splits=splits).float().cpu().numpy()
    for b in range(len(lengths)):
        ref = decode_reference(layer, batch, b, seed=1)
        e = rel_err(out[b], ref)
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
        assert e <= TOL[cache if cache == "fp8" else act], (b, e)


@pytest.mark.parametrize("heads,splits", [(16, 16), (32, 8), (32, 20)])
def test_narrow_heads_many_splits(heads, splits):
    """The narrow-head instances (one or two live 16-head tiles) with more splits than stages:
    short contexts leave most splits empty, and above four splits the merge runs first."""
    shape = dataclasses.replace(LITE, num_heads=heads)
    lengths = [1, 70, 300]
    log(f"narrow heads {heads}, splits {splits}")
    layer = Layer(shape, "bf16", "bf16", seed=7)
    batch = DecodeBatch(layer, wl(shape, "bf16", "bf16", len(lengths)), seed=7, lengths=lengths)
    out = batch.run(num_splits=splits).float().cpu().numpy()
    for b in range(len(lengths)):
        e = rel_err(out[b], decode_reference(layer, batch, b, seed=7))
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
        assert e <= TOL["bf16"], (b, e)


@pytest.mark.parametrize("B", [100, 140])
def test_decode_large_batches(B):
    """100 sequences: the decode projections run as 128-row weight-streaming tiles (rows 64..127
    in the second half of each tile, rows 100..127 past the batch).  140 sequences: beyond those
    tiles, the general front (tiled GEMMs, separate norm and row kernels, query packing).
    Compared with the oracle on sequences from every 64-row block and the last one."""
    lengths = [int(x) for x in np.random.default_rng(12).integers(0, 160, B)]
    log(f"decode {B} sequences")
    layer = Layer(DSV2, "bf16", "bf16", seed=12)
    batch = DecodeBatch(layer, wl(DSV2, "bf16", "bf16", len(lengths)), seed=12, lengths=lengths)
    out = batch.run(num_splits=2).float().cpu().numpy()
    assert np.isfinite(out).all()
    for b in sorted({0, 31, 63, 64, 77, B - 1} | ({128, 133} if B > 128 else set())):
        e = rel_err(out[b], decode_reference(layer, batch, b, seed=12))
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
        assert e <= TOL["bf16"], (b, e)


@pytest.mark.parametrize("variant", ["peaked", "gamma"])
def test_decode_variants(variant):
    """A peaked softmax (4x the default scale: exercises the reference-max bookkeeping far from a
    flat softmax, and scales every score's rounding error by 4) and random norm gains, both at
    the bf16 bar."""
    log(f"decode variant {variant}")
    mult = 4.0 if variant == "peaked" else 1.0
    kw = dict(softmax_scale=mult / np.sqrt(192.0)) if variant == "peaked" else dict(gamma="random")
    layer = Layer(DSV2, "bf16", "bf16", seed=2, **kw)
    lengths = [150, 400]
    batch = DecodeBatch(layer, wl(layer.shape, "bf16", "bf16", 2), seed=2, lengths=lengths)
    out = batch.run(num_splits=2).float().cpu().numpy()
    for b in range(2):
        e = rel_err(out[b], decode_reference(layer, batch, b, seed=2))
        log(f"  seq {b}: rel err {e:.2e}")
        assert e <= TOL["bf16"], (b, e)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_decode_per_head_query_scales(cache):
    """Heads whose queries differ in magnitude by powers of two: the q_nope rows of head h in
    q_b_proj are scaled by 2^(h mod 6 - 3), so the absorbed latent queries of neighbouring heads
    span 2^-3 .. 2^2 of the default (the largest as sharp as the peaked variant).  On the fp8
    cache every head's latent query enters the fp8 products with its own power-of-two block
    scale, which a lane-to-head mix-up of those scales would break; on the bf16 cache the same
    spread checks the bf16 products.  Bars as for every other case."""
    from mla_latent_kv_compress_amd.workload import to_device
    log(f"decode per-head query scales ({cache} cache)")
    layer = Layer(DSV2, "bf16", cache, seed=4)
    s = layer.shape
    w = layer.w_host["q_b_proj"].reshape(s.num_heads, s.qk_head_dim, -1).copy()
    for h in range(s.num_heads):
        w[h, :s.qk_nope_head_dim] *= np.float32(2.0 ** ((h % 6) - 3))     # exact in bf16
    layer.w_host["q_b_proj"] = w.reshape(s.num_heads * s.qk_head_dim, -1)
    layer.w["q_b_proj"] = to_device(layer.w_host["q_b_proj"], "bf16", "cuda")
    layer.w_struct = api.make_weights(layer.w)
    lengths = [90, 333]
    batch = DecodeBatch(layer, wl(s, "bf16", cache, 2), seed=4, lengths=lengths)
    out = batch.run(num_splits=2).float().cpu().numpy()
    for b in range(2):
        e = rel_err(out[b], decode_reference(layer, batch, b, seed=4))
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
        assert e <= TOL[cache], (b, e)


@pytest.mark.parametrize("shape,B,splits", [
    (DSV2, 40, 4),     # 128 heads x 2 row blocks of 32 = 256 (head, rows) blocks: all 128 columns per work-group
    (DSV2, 20, 4),     # 128 blocks: the columns cut over 2 work-groups
    (LITE, 5, 4),      # 16 blocks: the columns cut over 4 work-groups
    (DSV2, 32, 0),     # the library's own choice for 32 sequences of 128 heads: 4 splits
    (LITE, 40, 8),     # eight splits (merged by a first kernel, then projected), 16 heads x 2 row blocks
    (DSV2, 20, 8),     # the same with 128 heads
])
def test_four_split_merge(shape, B, splits):
    """The merge + W_UV kernel's four-split instance in each of its three column forms, the
    automatic split count at B = 32 (which picks four), and eight splits (merged by a first kernel;
    many of these short sequences leave some splits empty)."""
    lengths = [int(x) for x in np.random.default_rng(13).integers(0, 260, B)]
    if splits == 0:
        lengths[1] = 700          # a block table of 11 pages: room for 4 splits of whole stages
    log(f"decode four-split merge: H {shape.num_heads}, B {B}, splits {splits}")
    layer = Layer(shape, "bf16", "bf16", seed=13)
    batch = DecodeBatch(layer, wl(shape, "bf16", "bf16", B), seed=13, lengths=lengths)
    if splits == 0:
        assert api.decode_num_splits(layer.cfg, B, batch.table.shape[1]) == 4
    out = batch.run(num_splits=splits).float().cpu().numpy()
    assert np.isfinite(out).all()
    for b in sorted({0, 1, B // 2, B - 1}):
        e = rel_err(out[b], decode_reference(layer, batch, b, seed=13))
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
        assert e <= TOL["bf16"], (b, e)


@pytest.mark.parametrize("splits", [1, 2, 7])
def test_constant_latent_returns_its_value(splits):
    """When every cached row holds the same latent c (the RoPE keys differ, so the softmax weights
    do), every head's output is W_UV^h c whatever the weights: the softmax normalisation and the
    split merge are checked without the oracle's attention.  The new token's own row carries c,
    since the history is filled with the latent the decode step computes for it."""
    log(f"decode constant latent, splits {splits}")
    from mla_latent_kv_compress_amd.workload import to_device
    layer = Layer(DSV2, "bf16", "bf16", seed=11, softmax_scale=4.0 / np.sqrt(192.0))
    lengths = [0, 1, 63, 700]
    batch = DecodeBatch(layer, wl(DSV2, "bf16", "bf16", len(lengths)), seed=11, lengths=lengths, history=False)
    d, W = oracle_dims(DSV2), oracle_weights(layer)
    g = np.random.default_rng(11)
    data = batch.cache.data.view(-1, d.row_width)
    want = []
    for b, L in enumerate(lengths):
        new_row = oracle.cache_rows(d, W, batch.x_host[b].astype(np.float64)[None], np.array([L]), "bf16")[0][0]
        c = new_row[: d.kv_lora_rank]
        rows = np.empty((L, d.row_width))
        rows[:, : d.kv_lora_rank] = c
        rows[:, d.kv_lora_rank:] = inputs_bf16(g.standard_normal((L, d.qk_rope)) * 2.0)
        if L:
            slots = slots_for(batch.table[b], np.arange(L))
            data[torch.as_tensor(slots, device="cuda")] = to_device(rows.astype(np.float32), "bf16", "cuda")
        want.append(np.stack([oracle.head_weights(d, W, h)[1] @ c for h in range(d.heads)]))
    out = batch.run(num_splits=splits).float().cpu().numpy()
    for b in range(len(lengths)):
        # The value product weighs the (equal) latents with bf16 probabilities p (1 + e_t),
        # |e_t| <= 2^-8, against the fp32 sum of the p: the result is W_UV^h c times a weighted
        # mean of (1 + e_t), so each head may be off by 2^-8 of its own largest value; 1e-3 of the
        # rms covers the fp16 split state and the accumulation.
        err = np.max(np.abs(out[b] - want[b]), axis=1)
        rms = np.sqrt(np.mean(want[b] ** 2))
        bound = 2.0 ** -8 * np.max(np.abs(want[b]), axis=1) + 1e-3 * rms
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {rel_err(out[b], want[b]):.2e}, "
            f"worst head at {np.max(err / bound):.2f} of its bound")
        assert np.all(err <= bound), (b, float(np.max(err / bound)))


def inputs_bf16(x):
    from mla_latent_kv_compress_amd import inputs
    return inputs.to_dtype_values(np.asarray(x, dtype=np.float32), "bf16").astype(np.float64)


def _loud_history(cache, factor, seed=4):
    """One sequence of 300 cached tokens whose token 250 has its hidden state scaled by `factor`
    (its k_pe is not normalized, so its scores grow with the factor).  Returns the layer, the
    batch, the oracle's cache rows and the new token's scores against every row, per head, in
    log2 units."""
    from mla_latent_kv_compress_amd import inputs
    from mla_latent_kv_compress_amd.workload import to_device
    layer = Layer(DSV2, "bf16", cache, seed=seed)
    L, loud = 300, 250
    batch = DecodeBatch(layer, wl(DSV2, "bf16", cache, 1), seed=seed, lengths=[L], history=False)
    x = inputs.history_hidden(DSV2, 0, 0, L, "bf16", seed=seed).copy()
    x[loud] = inputs.to_dtype_values(x[loud] * factor, "bf16")
    pos = np.arange(L)
    layer.append(batch.cache, to_device(x, "bf16", "cuda"), pos, slots_for(batch.table[0], pos))
    d, W = oracle_dims(DSV2), oracle_weights(layer)
    rows = oracle.cache_rows(d, W, x.astype(np.float64), pos, cache)[0]
    xn = batch.x_host[0].astype(np.float64)
    new_row = oracle.cache_rows(d, W, xn[None], np.array([L]), cache)[0]
    allrows = np.concatenate([rows, new_row])
    qn, qp = oracle.queries(d, W, xn[None], np.array([L]))
    c, kpe = allrows[:, : d.kv_lora_rank], allrows[:, d.kv_lora_rank:]
    s2 = np.empty((d.heads, L + 1))
    for h in range(d.heads):
        w_uk, _ = oracle.head_weights(d, W, h)
        s2[h] = d.sigma * (qn[0, h] @ (c @ w_uk.T).T + qp[0, h] @ kpe.T) / np.log(2)
    return layer, batch, rows, s2, loud


def _loud_compare(cache, layer, batch, rows, s2, loud, splits_list):
    """Compare every head with the oracle; every output must be finite."""
    ref = decode_reference(layer, batch, 0, hist_rows=rows)
    for splits in splits_list:
        out = batch.run(num_splits=splits).float().cpu().numpy()[0]
        assert np.isfinite(out).all()
        e = rel_err(out, ref)
        log(f"  splits {splits}: all {len(ref)} heads, rel err {e:.2e}")
        assert e <= TOL["fp8" if cache == "fp8" else "bf16"], e


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_decode_loud_token_restart(cache):
    """One history token far louder than the rest forces the reference-max restart.

    Its hidden state is scaled 300x, so for some heads its score exceeds the maximum of the
    first stage of its split by more than 64 (log2 units, a factor 2^64 in probability), which
    makes the decode work-group drop what it accumulated and redo the split against the exact
    maxima.  The oracle's own scores confirm that the condition is met.
    """
    log(f"decode loud token ({cache} cache)")
    layer, batch, rows, s2, loud = _loud_history(cache, 300.0)
    assert np.any(s2[:, loud] > s2[:, :32].max(axis=1) + 64), "the loud token must outgrow the first stage"
    _loud_compare(cache, layer, batch, rows, s2, loud, (1, 2))


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_decode_loud_token_within_slack(cache):
    """A loud token (hidden state scaled 30x) that outgrows the first stage's maximum by up to
    about 56 log2 units: within the slack of 64, so no restart, and the heads it dominates
    accumulate weights up to ~2^56 against the first stage's reference.  Their unnormalized
    partial state O runs far past the fp16 range (65504); the split's state is stored with a
    per-head power-of-two scale, so the result must still match.  (One split: the first stage is
    the first 32 tokens.)"""
    log(f"decode loud token within the slack ({cache} cache)")
    layer, batch, rows, s2, loud = _loud_history(cache, 30.0)
    over = s2[:, loud] - s2[:, :32].max(axis=1)
    log(f"  largest excess over the first stage {over.max():.1f} log2 units")
    assert 24 <= over.max() <= 62, over.max()
    _loud_compare(cache, layer, batch, rows, s2, loud, (1,))


@pytest.mark.parametrize("cache,lengths,splits,ranked", [
    # 8 x 20 x 2 = 320 work-groups, more than 8 splits: not ranked (short pieces everywhere)
    ("bf16", [33, 2000, 64, 1200, 0, 640, 3100, 257], 20, False),
    ("fp8", [33, 2000, 64, 1200, 0, 640, 3100, 257], 20, False),
    # 20 sequences (not a multiple of the 8 XCDs), 8 splits: 320 work-groups, ranked, the head
    # groups of each (sequence, split) paired on one XCD
    ("bf16", [int(x) for x in np.random.default_rng(9).integers(0, 700, 20)], 8, True),
    ("fp8", [int(x) for x in np.random.default_rng(9).integers(0, 700, 20)], 8, True),
    # 21 sequences x 7 splits = 147 (sequence, split) units, padded to 152 by work-groups that
    # leave at once; ranked (294 working work-groups)
    ("bf16", [int(x) for x in np.random.default_rng(10).integers(0, 700, 21)], 7, True),
])
def test_ragged_batch(cache, lengths, splits, ranked):
    """Ragged lengths over more work-groups than one round.  With at most 8 splits the sequences
    are ranked by length on the GPU and dispatched longest first; every sequence must still get
    its own result.  (Which of these cases the planner ranks is checked on the CPU, in the host
    planning test.)"""
    log(f"decode ragged ({cache} cache, B {len(lengths)}, {splits} splits, ranked {ranked})")
    layer = Layer(DSV2, "bf16", cache, seed=5)
    batch = DecodeBatch(layer, wl(DSV2, "bf16", cache, len(lengths)), seed=5, lengths=lengths)
    out = batch.run(num_splits=splits).float().cpu().numpy()
    for b in range(len(lengths)):
        e = rel_err(out[b], decode_reference(layer, batch, b, seed=5))
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
        assert e <= TOL[cache if cache == "fp8" else "bf16"], (b, e)


# YaRN-scaled RoPE (the pages give no constants; these exercise every branch of the ramp: with
# an original context of 1024 the 32 pairs split into kept, interpolated and mixed ones).
YARN_DSV2 = dataclasses.replace(DSV2, rope_factor=8.0, rope_original_max_position=1024, rope_beta_fast=32.0,
                                rope_beta_slow=1.0, rope_mscale=1.1)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_decode_yarn_rope(cache):
    lengths = [100, 2047, 3000]
    log(f"decode with YaRN RoPE ({cache} cache)")
    layer = Layer(YARN_DSV2, "bf16", cache, seed=6)
    batch = DecodeBatch(layer, wl(YARN_DSV2, "bf16", cache, len(lengths)), seed=6, lengths=lengths)
    out = batch.run(num_splits=3).float().cpu().numpy()
    for b in range(len(lengths)):
        e = rel_err(out[b], decode_reference(layer, batch, b, seed=6))
        log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
        assert e <= TOL[cache if cache == "fp8" else "bf16"], (b, e)


def test_bf16_output():
    log("decode bf16 output")
    layer = Layer(DSV2, "bf16", "bf16", seed=1, out_dtype="bf16")
    lengths = [70, 300]
    batch = DecodeBatch(layer, wl(DSV2, "bf16", "bf16", 2), seed=1, lengths=lengths)
    out = batch.run(num_splits=2)
    assert out.dtype == torch.bfloat16
    out = out.float().cpu().numpy()
    for b in range(2):
        assert bf16_out_ok(out[b], decode_reference(layer, batch, b, seed=1), TOL["bf16"])


def test_split_counts_and_paging_is_bitwise_invariant():
    log("splits / paging")
    layer = Layer(DSV2, "bf16", "bf16", seed=4)
    lengths = [1000, 333, 64]
    w = wl(DSV2, "bf16", "bf16", 3)
    shuffled = DecodeBatch(layer, w, seed=4, lengths=lengths)
    ident = DecodeBatch(layer, w, seed=4, lengths=lengths, shuffle=False)
    refs = [decode_reference(layer, shuffled, b, seed=4) for b in range(3)]
    for s in (1, 2, 7, 16, 64, 1024):             # 1024: the largest count, nearly every split empty
        out = shuffled.run(num_splits=s).float().cpu().numpy()
        errs = [rel_err(out[b], refs[b]) for b in range(3)]
        log(f"  splits {s}: {max(errs):.2e}")
        assert max(errs) <= TOL["bf16"]
    a = shuffled.run(num_splits=7)
    b = ident.run(num_splits=7)
    assert torch.equal(a, b), "physical page order must not change any bit"
    assert torch.equal(a, shuffled.run(num_splits=7)), "repeat runs must be bitwise identical"


def test_fp32_paging_invariance_and_tail_pages():
    log("tiny paging")
    layer = Layer(TINY, "f32", "f32", seed=6)
    w = wl(TINY, "f32", "f32", 2)
    a = DecodeBatch(layer, w, seed=6, lengths=[128, 65]).run(num_splits=2)
    b = DecodeBatch(layer, w, seed=6, lengths=[128, 65], shuffle=False).run(num_splits=2)
    assert torch.equal(a, b)
