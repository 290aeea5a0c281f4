"""GPU parity of the output projection (o_proj on the attention output) against the fp64 oracle.

The weights carry o_proj [hidden, H * v_head_dim] (seeded N(0, 0.02^2)); mla_decode and
mla_prefill then return [tokens, hidden].  The reference is the oracle's per-head output mapped
by its output_projection.  Cases cover each route of the product: the fp32 path (direct, no K
split), the bf16 path with the attention output in fp32 entering the skinny product as a bf16
hi + lo pair (K split 4 at the 236B shape, 8 at Lite, then the split sum), the bf16 path past the
skinny kernel's 128 rows (attention output in bf16, generic product), bf16 output, the fp8 cache,
and prefill (generic product; fp32 and bf16 outputs).
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_compress_amd import api, inputs
from mla_latent_kv_compress_amd.configs import DSV2, LITE, TINY, Workload
from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer, build_history, to_device
from mla_ref import TOL, bf16_out_ok, decode_reference, history_rows, oracle_dims, oracle_weights, rel_err

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def projected(layer, heads_out):
    return oracle.output_projection(oracle_dims(layer.shape), oracle_weights(layer), heads_out)


DECODE = {
    # name: shape, act, cache, out dtype, history lengths, splits, sequences checked
    "tiny_f32": (TINY, "f32", "f32", "f32", [127, 3, 64], 2, None),
    "dsv2_bf16": (DSV2, "bf16", "bf16", "f32", [700, 64, 1, 300], 2, None),
    "dsv2_bf16_out": (DSV2, "bf16", "bf16", "bf16", [200, 90], 0, None),
    "dsv2_fp8": (DSV2, "bf16", "fp8", "f32", [500, 129, 33], 0, None),
    "lite_bf16": (LITE, "bf16", "bf16", "f32", [400, 65, 5], 0, None),
    "dsv2_bf16_b160": (DSV2, "bf16", "bf16", "f32", [40] * 159 + [300], 1, [0, 77, 159]),
}


@pytest.mark.parametrize("case", list(DECODE))
def test_decode_with_output_projection(case):
    shape, act, cache, out_dt, lengths, splits, check = DECODE[case]
    log(f"decode + o_proj {case}")
    layer = Layer(shape, act, cache, seed=21, out_dtype=out_dt, o_proj=True)
    wl = Workload("t", shape, act, cache, decode_batch=len(lengths))
    batch = DecodeBatch(layer, wl, seed=21, lengths=lengths)
    out = batch.run(num_splits=splits).float().cpu().numpy()
    assert out.shape == (len(lengths), shape.hidden_size)
    bar = TOL["fp8" if cache == "fp8" else act]
    for b in (range(len(lengths)) if check is None else check):
        ref = projected(layer, decode_reference(layer, batch, b, seed=21))
        e = rel_err(out[b], ref)
        log(f"  seq {b} (ctx {lengths[b] + 1}): rel err {e:.2e}")
        if out_dt == "bf16":
            assert bf16_out_ok(out[b], ref, bar), (b, e)
        else:
            assert e <= bar, (b, e)


def test_decode_output_projection_is_the_per_head_output_projected():
    """The same batch with and without o_proj: the projected output equals o_proj applied (in
    fp64 on the host) to the library's own per-head output, to the bf16 bar (the two runs differ
    only in the product after the attention)."""
    log("decode with vs without o_proj")
    layer_o = Layer(DSV2, "bf16", "bf16", seed=22, o_proj=True)
    wl = Workload("t", DSV2, "bf16", "bf16", decode_batch=3)
    batch = DecodeBatch(layer_o, wl, seed=22, lengths=[250, 31, 129])
    plain_w = {k: v for k, v in layer_o.w.items() if k != "o_proj"}
    heads = api.decode(layer_o.cfg, plain_w, batch.x, batch.ctx_t, batch.table_t, batch.cache, num_splits=2)
    assert heads.shape == (3, DSV2.num_heads, DSV2.v_head_dim)
    # (the decode appended the new tokens; the second call rewrites the same rows with the same values)
    proj = batch.run(num_splits=2).float().cpu().numpy()
    want = projected(layer_o, heads.float().cpu().numpy().astype(np.float64))
    for b in range(3):
        e = rel_err(proj[b], want[b])
        log(f"  seq {b}: {e:.2e}")
        assert e <= 1e-2, (b, e)


PREFILL = {
    "tiny_f32": (TINY, "f32", "f32", "f32", [0, 64], [70, 33]),
    "dsv2_bf16": (DSV2, "bf16", "bf16", "f32", [0, 100], [130, 64]),
    "dsv2_bf16_out": (DSV2, "bf16", "bf16", "bf16", [0], [96]),
    "dsv2_fp8": (DSV2, "bf16", "fp8", "f32", [64], [100]),
}


@pytest.mark.parametrize("case", list(PREFILL))
def test_prefill_with_output_projection(case):
    shape, act, cache, out_dt, starts, lens = PREFILL[case]
    log(f"prefill + o_proj {case}")
    layer = Layer(shape, act, cache, seed=23, out_dtype=out_dt, o_proj=True)
    ctx = np.array(starts) + np.array(lens)
    table, nb = inputs.block_table(ctx, 23)
    kv = layer.new_cache(nb)
    build_history(layer, kv, table, np.array(starts), 23)
    x = np.concatenate([inputs.history_hidden(shape, s, starts[s], lens[s], act, 23) for s in range(len(lens))])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = api.prefill(layer.cfg, layer.w, to_device(x, act, "cuda"), torch.as_tensor(cu, device="cuda"),
                      torch.as_tensor(np.array(starts, dtype=np.int32), device="cuda"),
                      torch.as_tensor(table, device="cuda"), kv, int(max(lens)), int(ctx.max()))
    out = out.float().cpu().numpy()
    assert out.shape == (int(sum(lens)), shape.hidden_size)
    d, W = oracle_dims(shape), oracle_weights(layer)
    bar = TOL["fp8" if cache == "fp8" else act]
    for s in range(len(lens)):
        prior = history_rows(layer, s, starts[s], 23)
        xs = x[cu[s]:cu[s + 1]].astype(np.float64)
        heads, _ = oracle.prefill_chunk(d, W, xs, starts[s], prior, cache)
        ref = oracle.output_projection(d, W, heads)
        got = out[cu[s]:cu[s + 1]]
        errs = [rel_err(got[i], ref[i]) for i in range(len(ref))]
        log(f"  seq {s}: worst rel err {max(errs):.2e}")
        if out_dt == "bf16":
            assert all(bf16_out_ok(got[i], ref[i], bar) for i in range(len(ref)))
        else:
            assert max(errs) <= bar
