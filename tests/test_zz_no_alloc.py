"""mla_decode_noalloc (the decode step on the library's static per-GPU workspace) against
mla_decode with a caller workspace: identical outputs on two calls in a row, the second smaller
than the first, both within the oracle's bar; a request beyond the static array is refused
before anything runs."""
import numpy as np
import pytest
import torch

from mla_latent_kv_compress_amd import api
from mla_latent_kv_compress_amd.configs import DSV2, Workload
from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer
from mla_ref import TOL, decode_reference, rel_err

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def test_noalloc_matches_workspace_decode_twice():
    layer = Layer(DSV2, "bf16", "bf16", seed=21)
    for B, lengths, splits in ((6, [700, 33, 0, 257, 1500, 64], 0), (2, [100, 5], 3)):
        log(f"no-alloc decode: B {B}, lengths {lengths}, splits {splits}")
        batch = DecodeBatch(layer, Workload("t", DSV2, "bf16", "bf16", decode_batch=B), seed=21, lengths=lengths)
        # the new token's row is appended by each call (same bytes both times), so the two
        # calls see identical caches
        want = batch.run(num_splits=splits).clone()
        got = api.decode_noalloc(layer.cfg, layer.w, batch.x, batch.ctx_t, batch.table_t, batch.cache,
                                 num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(got, want), float((got - want).abs().max())
        out = got.float().cpu().numpy()
        for b in (0, B - 1):
            e = rel_err(out[b], decode_reference(layer, batch, b, seed=21))
            log(f"  seq {b} ctx {lengths[b] + 1}: rel err {e:.2e}")
            assert e <= TOL["bf16"]


def test_noalloc_refuses_beyond_the_scratch():
    layer = Layer(DSV2, "bf16", "bf16", seed=21)
    B, max_blocks = 128, 513                       # 115 MB of workspace: more than the 64 MiB array
    assert api.decode_workspace_size(layer.cfg, B, max_blocks, 2) > 64 << 20
    x = torch.zeros((B, DSV2.hidden_size), dtype=torch.bfloat16, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    table = torch.zeros((B, max_blocks), dtype=torch.int32, device="cuda")
    cache = layer.new_cache(1)
    with pytest.raises(api.MLAError) as e:
        api.decode_noalloc(layer.cfg, layer.w, x, ctx, table, cache, num_splits=2)
    assert e.value.status == 3
