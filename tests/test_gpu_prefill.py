"""GPU parity of mla_prefill (causal chunked prefill, explicit form) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_compress_amd import api, inputs
from mla_latent_kv_compress_amd.configs import DSV2, LITE, TINY, Workload
from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer, build_history, to_device
from mla_ref import TOL, bf16_out_ok, history_rows, oracle_dims, oracle_weights, rel_err, token_err

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


class Prefill:
    """S sequences: `starts[s]` tokens already cached, then one chunk of `lens[s]` tokens."""

    def __init__(self, layer, starts, lens, seed=0, shuffle=True):
        self.layer, self.starts, self.lens, self.seed = layer, list(starts), list(lens), seed
        ctx = np.array(starts) + np.array(lens)
        self.table, nb = inputs.block_table(ctx, seed, shuffle=shuffle)
        self.cache = layer.new_cache(nb)
        build_history(layer, self.cache, self.table, np.array(starts), seed)
        self.max_q, self.max_ctx = int(max(lens)), int(ctx.max())
        self.table_t = torch.as_tensor(self.table, device="cuda")

    def chunk_hidden(self, s, start, n):
        return inputs.history_hidden(self.layer.shape, s, start, n, self.layer.act, self.seed)

    def run(self, starts=None, lens=None):
        starts = self.starts if starts is None else starts
        lens = self.lens if lens is None else lens
        x = np.concatenate([self.chunk_hidden(s, starts[s], lens[s]) for s in range(len(lens))])
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        out = api.prefill(self.layer.cfg, self.layer.w, to_device(x, self.layer.act, "cuda"),
                          torch.as_tensor(cu, device="cuda"),
                          torch.as_tensor(np.array(starts, dtype=np.int32), device="cuda"), self.table_t,
                          self.cache, int(max(lens)), int(max(np.array(starts) + np.array(lens))))
        return out.float().cpu().numpy(), cu

    def reference(self, s, rows=None, heads=None):
        layer = self.layer
        d, W = oracle_dims(layer.shape), oracle_weights(layer)
        prior = history_rows(layer, s, self.starts[s], self.seed)
        x = self.chunk_hidden(s, self.starts[s], self.lens[s]).astype(np.float64)
        out, _ = oracle.prefill_chunk(d, W, x, self.starts[s], prior, layer.cache_dtype, heads=heads, query_rows=rows)
        return out


CASES = {
    "tiny_f32": (TINY, "f32", "f32", [0, 64, 7], [5, 70, 64]),
    "dsv2_bf16": (DSV2, "bf16", "bf16", [0, 50], [100, 64]),
    "dsv2_fp8": (DSV2, "bf16", "fp8", [0, 130], [70, 33]),
    "lite_bf16": (LITE, "bf16", "bf16", [0, 1], [129, 64]),
    # several 128-query tiles and 64-key tiles with ragged tails, cached history before the chunk
    "dsv2_bf16_tiles": (DSV2, "bf16", "bf16", [300, 0, 1000], [300, 257, 130]),
    "dsv2_fp8_tiles": (DSV2, "bf16", "fp8", [64, 0], [200, 129]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_matches_oracle(case):
    shape, act, cache, starts, lens = CASES[case]
    log(f"prefill {case}")
    layer = Layer(shape, act, cache, seed=7)
    pf = Prefill(layer, starts, lens, seed=7)
    out, cu = pf.run()
    for s in range(len(lens)):
        ref = pf.reference(s)
        e = token_err(out[cu[s]:cu[s + 1]], ref)
        log(f"  seq {s} start {starts[s]} len {lens[s]}: rel err {e:.2e}")
        assert e <= TOL[cache if cache == "fp8" else act], (s, e)


def test_prefill_yarn_rope():
    """Prefill parity with YaRN-scaled RoPE (constants as in the decode test); rope_mscale m
    scales the RoPE part of every score by m^2, at the plain bf16 bar."""
    import dataclasses
    m = 1.1
    shape = dataclasses.replace(DSV2, rope_factor=8.0, rope_original_max_position=1024, rope_beta_fast=32.0,
                                rope_beta_slow=1.0, rope_mscale=m)
    log("prefill with YaRN RoPE")
    layer = Layer(shape, "bf16", "bf16", seed=7)
    pf = Prefill(layer, [0, 1500], [300, 200], seed=7)
    out, cu = pf.run()
    for s in range(2):
        e = token_err(out[cu[s]:cu[s + 1]], pf.reference(s))
        log(f"  seq {s}: rel err {e:.2e}")
        assert e <= TOL["bf16"], (s, e)


def test_chunked_equals_whole_and_last_row_equals_decode():
    log("prefill chunking")
    layer = Layer(DSV2, "bf16", "bf16", seed=8)
    n = 192
    whole = Prefill(layer, [0], [n], seed=8)
    out_whole, _ = whole.run()
    chunked = Prefill(layer, [0], [n], seed=8)
    parts = [chunked.run(starts=[s], lens=[64])[0] for s in range(0, n, 64)]
    e = token_err(np.concatenate(parts), out_whole)
    log(f"  chunked vs whole: {e:.2e}")
    assert e <= 1e-2
    # decode of the last token over the same history equals the last prefill row
    dec = DecodeBatch(layer, Workload("t", DSV2, "bf16", "bf16", decode_batch=1), seed=8, lengths=[n - 1],
                      history=True)
    x_last = inputs.history_hidden(DSV2, 0, n - 1, 1, "bf16", 8)
    dec.x.copy_(to_device(x_last, "bf16", "cuda"))
    out_dec = dec.run(num_splits=2).float().cpu().numpy()
    e2 = rel_err(out_dec[0], out_whole[-1])
    log(f"  decode vs prefill last row: {e2:.2e}")
    assert e2 <= 2e-2


def test_prefill_bf16_output():
    log("prefill bf16 output")
    layer = Layer(DSV2, "bf16", "bf16", seed=7, out_dtype="bf16")
    pf = Prefill(layer, [0, 50], [100, 64], seed=7)
    out, cu = pf.run()
    for s in range(2):
        ref = pf.reference(s)
        got = out[cu[s]:cu[s + 1]]
        assert all(bf16_out_ok(got[i], ref[i], TOL["bf16"]) for i in range(len(ref)))


@pytest.mark.parametrize("shape,act,n,cut", [(TINY, "f32", 80, 50), (DSV2, "bf16", 300, 200)])
def test_prefill_causality(shape, act, n, cut):
    """Changing later tokens of a chunk leaves earlier rows bit-identical."""
    log(f"prefill causality ({act})")
    layer = Layer(shape, act, act, seed=9)
    pf = Prefill(layer, [0], [n], seed=9)
    out1, _ = pf.run()
    orig = pf.chunk_hidden

    def perturbed(s, start, n):
        x = orig(s, start, n).copy()
        x[cut - start:] += 1.0
        return x
    pf.chunk_hidden = perturbed
    out2, _ = pf.run()
    assert np.array_equal(out1[:cut], out2[:cut])
    assert not np.allclose(out1[cut:], out2[cut:])


@pytest.mark.parametrize("cache,o_proj", [("bf16", False), ("fp8", True)])
def test_prefill_key_blocks(cache, o_proj):
    """The context decompressed in key blocks of 128 positions (the running softmax state carried
    from block to block: nine blocks here, some past a sequence's causal range) meets the oracle's
    bar and agrees with the one-block result to 5e-3: the decompression then runs with 128 rows
    per launch instead of 1130, on other GEMM tiles whose fp32 sums may round a few keys and
    values to the neighbouring fp16 value (2^-11 relative), while a dropped block or a lost row
    sum would move the output by far more."""
    log(f"prefill key blocks ({cache}, o_proj {o_proj})")
    layer = Layer(DSV2, "bf16", cache, seed=12, o_proj=o_proj)
    pf = Prefill(layer, [300, 0, 1000], [300, 257, 130], seed=12)
    whole, cu = pf.run()
    layer.cfg.prefill_key_block = 128
    try:
        blocks, _ = pf.run()                     # (appends the same rows again)
    finally:
        layer.cfg.prefill_key_block = 0
    d, W = oracle_dims(DSV2), oracle_weights(layer)
    for s in range(3):
        got = blocks[cu[s]:cu[s + 1]]
        e1 = token_err(got, whole[cu[s]:cu[s + 1]])
        ref = pf.reference(s)
        if o_proj:
            ref = oracle.output_projection(d, W, ref)
        e2 = token_err(got, ref)
        log(f"  seq {s}: vs one block {e1:.2e}, vs oracle {e2:.2e}")
        assert e1 <= 5e-3, (s, e1)
        assert e2 <= TOL[cache], (s, e2)
