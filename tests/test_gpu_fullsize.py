"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Each decode workload runs over its whole batch and paged cache at its real shape with the split
count the bench uses (seed 0, eager launch, fp32 output); the oracle then recomputes a seeded
sample of sequences one at a time (all heads; at long contexts the explicit form on a fixed head
subset, whose explicit form over every head would take minutes on the host, and every head in
the weight-absorbed fp64 form, checked against the explicit one on that subset first) and every
other output is checked to be finite.
The mixed fp8 workload's chunked prefill (4 prompts x 4096 tokens in chunks of 1024) is checked
on sampled rows of every chunk; the oracle chains the chunks itself, each chunk's stored rows
becoming the next one's prior context.
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_compress_amd import api, inputs
from mla_latent_kv_compress_amd.configs import WORKLOADS
from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer, PrefillBatch
from mla_ref import (TOL, absorbed_all_heads, decode_reference, decode_rows_and_queries, oracle_dims, oracle_weights,
                     rel_err)

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def picks(batch, count, seed=99):
    """`count` sequences drawn without replacement, plus the shortest and longest when ragged."""
    B = len(batch.hist)
    out = list(np.random.default_rng(seed).choice(B, size=min(count, B), replace=False))
    if len(set(batch.hist.tolist())) > 1:
        out += [int(np.argmin(batch.hist)), int(np.argmax(batch.hist))]
    return sorted(set(int(b) for b in out))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,count,heads", [
    ("lite_bf16", 3, None),
    ("dsv2_bf16", 2, None),
    ("dsv2_128k", 4, [0, 61, 127]),
    ("dsv2_mixed_fp8", 3, [0, 61, 127]),
])
def test_fullsize_decode(name, count, heads):
    wl = WORKLOADS[name]
    log(f"full-size decode {name}: building the cache")
    layer = Layer(wl.shape, wl.act_dtype, wl.cache_dtype, out_dtype="f32")
    batch = DecodeBatch(layer, wl)
    B, max_blocks = batch.table.shape
    splits = wl.num_splits or api.decode_num_splits(layer.cfg, B, max_blocks)
    ws = torch.empty(api.decode_workspace_size(layer.cfg, B, max_blocks, splits), dtype=torch.uint8, device="cuda")
    log(f"  B={B} max ctx={int(batch.ctx.max())} splits={splits}: decoding")
    out = batch.run(num_splits=splits, workspace=ws).float().cpu().numpy()
    assert np.isfinite(out).all()
    bar = TOL["fp8" if wl.cache_dtype == "fp8" else wl.act_dtype]
    d, W = oracle_dims(layer.shape), oracle_weights(layer)
    for b in picks(batch, count):
        if heads is None:
            ref = decode_reference(layer, batch, b)
            e = rel_err(out[b], ref)
            log(f"  seq {b} ctx {int(batch.ctx[b])}: rel err {e:.2e}")
            assert e <= bar, (name, b, e)
            continue
        # Long contexts: the explicit oracle on the sampled heads, and every head against the
        # absorbed form, itself checked against the explicit oracle on those heads first
        rows, q_nope, q_pe = decode_rows_and_queries(layer, batch, b)
        ref = oracle.attend_explicit(d, W, q_nope[None], q_pe[None], rows, heads=heads)[0]
        ref_all = absorbed_all_heads(layer, rows, q_nope, q_pe)
        assert rel_err(ref_all[heads], ref) <= 1e-9, (name, b)
        e = rel_err(out[b][heads], ref)
        e_all = rel_err(out[b], ref_all)
        log(f"  seq {b} ctx {int(batch.ctx[b])}: rel err {e:.2e} (heads {heads}), {e_all:.2e} (all heads)")
        assert e <= bar, (name, b, e)
        assert e_all <= bar, (name, b, e_all)


@pytest.mark.timeout(900)
def test_fullsize_chunked_prefill_fp8():
    wl = WORKLOADS["dsv2_mixed_fp8"]
    log("full-size chunked prefill dsv2_mixed_fp8")
    layer = Layer(wl.shape, wl.act_dtype, wl.cache_dtype, out_dtype="f32")
    pb = PrefillBatch(layer, wl.prefill_seqs, wl.prefill_len, wl.prefill_chunk)
    ws = torch.empty(pb.workspace_size(), dtype=torch.uint8, device="cuda")
    outs = []
    for k in range(pb.num_chunks):
        outs.append(pb.run_chunk(k, workspace=ws).float().cpu().numpy())
        assert np.isfinite(outs[-1]).all()
    d, W = oracle_dims(layer.shape), oracle_weights(layer)
    n = pb.chunk
    for s in (0, pb.S - 1):
        prompt = pb.prompts[s].astype(np.float64)
        prior = np.empty((0, d.row_width))
        for k in range(pb.num_chunks):
            c0 = k * n
            rows = sorted({0, (37 * (k + 1) + 11 * s) % n, n - 1})
            ref, new_rows = oracle.prefill_chunk(d, W, prompt[c0:c0 + n], c0, prior, layer.cache_dtype,
                                                 query_rows=rows)
            prior = np.concatenate([prior, new_rows])
            for j, r in enumerate(rows):
                e = rel_err(outs[k][s * n + r], ref[j])
                log(f"  seq {s} chunk {k} row {r} (position {c0 + r}): rel err {e:.2e}")
                assert e <= TOL["fp8"], (s, k, r, e)
