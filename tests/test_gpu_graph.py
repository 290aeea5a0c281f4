"""A decode step captured in a HIP graph replays to the eager result, every replay."""
import numpy as np
import pytest
import torch

from mla_latent_kv_compress_amd import api
from mla_latent_kv_compress_amd.configs import DSV2, TINY, Workload
from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,act,cache,o_proj", [(DSV2, "bf16", "bf16", False), (DSV2, "bf16", "fp8", False),
                                                    (TINY, "f32", "f32", False), (DSV2, "bf16", "bf16", True)])
def test_graph_replays_match_eager(shape, act, cache, o_proj):
    print(f"graph replay {act}/{cache} o_proj {o_proj}", flush=True)
    layer = Layer(shape, act, cache, seed=11, o_proj=o_proj)
    batch = DecodeBatch(layer, Workload("g", shape, act, cache, decode_batch=3), seed=11, lengths=[70, 300, 1])
    splits = 3
    B, mb = batch.table.shape
    ws = torch.empty(api.decode_workspace_size(layer.cfg, B, mb, splits), dtype=torch.uint8, device="cuda")
    out = torch.empty(api.out_shape(layer.cfg, layer.w, B), dtype=torch.float32, device="cuda")
    ref = batch.run(num_splits=splits, out=torch.empty_like(out), workspace=ws).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        batch.run(num_splits=splits, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        batch.run(num_splits=splits, out=out, workspace=ws)
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        scratch.mul_(1.0001).add_(0.5)            # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"
