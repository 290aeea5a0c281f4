"""Device-side set-up of a workload from the seeded inputs: weights, paged cache, batch.

The history cache is built by the library itself (mla_compress_append over each sequence's
seeded history hidden states), then decode or prefill calls run on top of it.  This module
does index bookkeeping and host-to-device copies only.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

from . import api, inputs
from .configs import PAGE_SIZE


def to_device(x32, act_dtype, device):
    return torch.from_numpy(np.ascontiguousarray(x32)).to(device=device, dtype=api.TORCH_ACT[act_dtype])


def slots_for(table_row, positions):
    """Cache slot (page * 64 + row) of each position of one sequence."""
    positions = np.asarray(positions, dtype=np.int64)
    return table_row[positions // PAGE_SIZE].astype(np.int64) * PAGE_SIZE + positions % PAGE_SIZE


class Layer:
    """Weights of one MLA layer on the device (plus the float32 host copy they came from)."""

    def __init__(self, shape, act_dtype, cache_dtype, seed=0, device="cuda", gamma="one", softmax_scale=None,
                 out_dtype="f32", o_proj=False):
        if softmax_scale is not None:
            from dataclasses import replace
            shape = replace(shape, softmax_scale=softmax_scale)
        self.shape, self.act, self.cache_dtype, self.device = shape, act_dtype, cache_dtype, device
        self.cfg = api.make_config(shape, act_dtype, cache_dtype, out_dtype)
        self.w_host = inputs.make_weights(shape, act_dtype, seed, gamma=gamma, o_proj=o_proj)
        self.w = {k: to_device(v, act_dtype, device) for k, v in self.w_host.items()}
        self.w_struct = api.make_weights(self.w)

    def new_cache(self, num_blocks, fill=None):
        return api.Cache(self.shape, self.cache_dtype, num_blocks, self.device, fill=fill)

    def append(self, cache, hidden_dev, positions, slots, workspace=None):
        pos = torch.as_tensor(np.asarray(positions, dtype=np.int32), device=self.device)
        sl = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=self.device)
        return api.compress_append(self.cfg, self.w, hidden_dev, pos, sl, cache, workspace=workspace)


def build_history(layer, cache, table, lengths, seed=0, chunk=8192, threads=None):
    """Compress each sequence's seeded history (positions 0..L-1) into the paged cache."""
    shape, act = layer.shape, layer.act
    threads = threads or min(16, os.cpu_count() or 1)
    jobs = [(b, int(L)) for b, L in enumerate(lengths) if L > 0]

    def gen(job):
        b, L = job
        return b, L, inputs.history_hidden(shape, b, 0, L, act, seed)

    ws = None
    with ThreadPoolExecutor(threads) as ex:
        # jobs go to the pool a window at a time so that at most `threads` histories are held
        done = (r for i in range(0, len(jobs), threads) for r in ex.map(gen, jobs[i:i + threads]))
        for b, L, hid in done:
            for s in range(0, L, chunk):
                n = min(chunk, L - s)
                pos = np.arange(s, s + n)
                need = api.lib().mla_compress_append_workspace_size(api.ctypes.byref(layer.cfg), n)
                if ws is None or ws.numel() < need:
                    ws = torch.empty(need, dtype=torch.uint8, device=layer.device)
                layer.append(cache, to_device(hid[s:s + n], act, layer.device), pos, slots_for(table[b], pos),
                             workspace=ws)
    torch.cuda.synchronize()


class DecodeBatch:
    """A decode step's inputs: history in the cache, new-token hidden states, block table."""

    def __init__(self, layer, workload, seed=0, shuffle=True, spare_blocks=0, history=True, lengths=None):
        self.layer, self.wl = layer, workload
        self.hist = (inputs.history_lengths(workload, seed) if lengths is None
                     else np.asarray(lengths, dtype=np.int64))
        self.ctx = self.hist + 1
        self.table, self.num_blocks = inputs.block_table(self.ctx, seed, shuffle=shuffle, spare_blocks=spare_blocks)
        self.cache = layer.new_cache(self.num_blocks)
        if history:
            build_history(layer, self.cache, self.table, self.hist, seed)
        self.x_host = inputs.decode_hidden(layer.shape, len(self.hist), layer.act, seed)
        self.x = to_device(self.x_host, layer.act, layer.device)
        self.ctx_t = torch.as_tensor(self.ctx.astype(np.int32), device=layer.device)
        self.table_t = torch.as_tensor(self.table, device=layer.device)

    def run(self, num_splits=None, out=None, workspace=None, stream=None, attn_events=None):
        s = self.wl.num_splits if num_splits is None else num_splits
        return api.decode(self.layer.cfg, self.layer.w, self.x, self.ctx_t, self.table_t, self.cache,
                          num_splits=s, out=out, workspace=workspace, stream=stream,
                          weights_struct=self.layer.w_struct, attn_events=attn_events)


class PrefillBatch:
    """Chunked prefill of S prompts of `length` tokens each, in chunks of `chunk` tokens.

    The prompts are the seeded prefill hidden states (inputs.prefill_hidden); every sequence
    starts empty and chunk k of every sequence goes into one mla_prefill call.
    """

    def __init__(self, layer, num_seqs, length, chunk, seed=0, shuffle=True):
        self.layer, self.S, self.length, self.chunk, self.seed = layer, num_seqs, length, chunk, seed
        self.table, self.num_blocks = inputs.block_table(np.full(num_seqs, length), seed, shuffle=shuffle)
        self.cache = layer.new_cache(self.num_blocks)
        self.table_t = torch.as_tensor(self.table, device=layer.device)
        self.prompts = [inputs.prefill_hidden(layer.shape, s, length, layer.act, seed) for s in range(num_seqs)]
        self.num_chunks = (length + chunk - 1) // chunk
        self._dev = []
        for k in range(self.num_chunks):
            c0, c1 = k * chunk, min(length, (k + 1) * chunk)
            x = np.concatenate([p[c0:c1] for p in self.prompts])
            cu = np.arange(num_seqs + 1, dtype=np.int32) * (c1 - c0)
            self._dev.append((to_device(x, layer.act, layer.device), torch.as_tensor(cu, device=layer.device),
                              torch.full((num_seqs,), c0, dtype=torch.int32, device=layer.device), c1 - c0, c1))

    def workspace_size(self):
        k = self.num_chunks - 1
        _, _, _, n, c1 = self._dev[k]
        return api.prefill_workspace_size(self.layer.cfg, self.S, self.S * n, n, c1)

    def run_chunk(self, k, out=None, workspace=None, stream=None):
        x, cu, start, n, c1 = self._dev[k]
        return api.prefill(self.layer.cfg, self.layer.w, x, cu, start, self.table_t, self.cache, n, c1,
                           out=out, workspace=workspace, stream=stream)
