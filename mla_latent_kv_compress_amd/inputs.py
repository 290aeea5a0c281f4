"""Seeded synthetic inputs shared by the GPU tests, the bench and the oracle checks.

This module draws random numbers and lays out page tables; it holds none of the method's
arithmetic.  Every array is produced by numpy's PCG64 generator seeded with (seed, stream), so
any part (one sequence's history, one chunk) can be regenerated alone.  Values that feed a
bf16 computation are rounded once to bf16 (torch's conversion) and returned as float32 arrays
holding those exact values; both sides consume the same numbers.

Distributions: projection weights N(0, 0.02^2); norm gains 1 (or 1 + N(0, 0.1^2) in the gain
variant); hidden states N(0, 1); page order a uniform random permutation of the block pool;
ragged history lengths uniform integers.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import PAGE_SIZE

STREAM_WEIGHTS = 0
STREAM_DECODE_X = 1
STREAM_PAGES = 2
STREAM_LENGTHS = 3
STREAM_GAMMA = 5
STREAM_OPROJ = 6
STREAM_HISTORY = 1000        # + sequence index
STREAM_PREFILL = 500000      # + sequence index
HISTORY_BLOCK = 4096         # history hidden states are drawn in blocks of this many tokens


def rng(seed, *stream):
    return np.random.default_rng([int(seed), *[int(s) for s in stream]])


def to_dtype_values(x32, dtype):
    """float32 array holding the values x32 takes in `dtype` ("f32" or "bf16")."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        import torch
        return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def make_weights(shape, act_dtype, seed=0, gamma="one", o_proj=False):
    """Weights in (out, in) layout as float32 arrays of act_dtype values, keyed by name; with
    o_proj also the output projection [hidden, H * v_head_dim] (from a stream of its own, so the
    other weights do not depend on whether it is drawn)."""
    g = rng(seed, STREAM_WEIGHTS)
    gg = rng(seed, STREAM_GAMMA)
    out = {}
    for name, shp in shape.weight_shapes():
        if name.endswith("_norm"):
            if gamma == "one":
                v = np.ones(shp, dtype=np.float32)
            else:
                v = (1.0 + 0.1 * gg.standard_normal(shp, dtype=np.float32)).astype(np.float32)
        else:
            v = g.standard_normal(shp, dtype=np.float32) * np.float32(0.02)
        out[name] = to_dtype_values(v, act_dtype)
    if o_proj:
        v = rng(seed, STREAM_OPROJ).standard_normal((shape.hidden_size, shape.num_heads * shape.v_head_dim),
                                                    dtype=np.float32) * np.float32(0.02)
        out["o_proj"] = to_dtype_values(v, act_dtype)
    return out


def history_lengths(workload, seed=0):
    """Cached tokens per decode sequence (before the decode token)."""
    B = workload.decode_batch
    if workload.history_range is None:
        return np.full(B, workload.history, dtype=np.int64)
    lo, hi = workload.history_range
    return rng(seed, STREAM_LENGTHS).integers(lo, hi, endpoint=True, size=B).astype(np.int64)


def block_table(token_counts, seed=0, page=PAGE_SIZE, spare_blocks=0, shuffle=True):
    """Paged layout for sequences holding token_counts[i] tokens.

    Returns (table int32 [S, max_blocks], num_blocks).  Logical block j of sequence i lives at
    physical block table[i, j]; physical blocks are a random permutation of the pool, assigned
    in (sequence, logical block) order.  Unused table entries are -1.
    """
    counts = np.asarray(token_counts, dtype=np.int64)
    nblk = (counts + page - 1) // page
    total = int(nblk.sum()) + int(spare_blocks)
    perm = rng(seed, STREAM_PAGES).permutation(total) if shuffle else np.arange(total)
    table = np.full((len(counts), max(int(nblk.max()), 1)), -1, dtype=np.int32)
    k = 0
    for i, n in enumerate(nblk):
        table[i, :n] = perm[k:k + n]
        k += n
    return table, total


def decode_hidden(shape, batch, act_dtype, seed=0):
    """Hidden states [batch, D] of the decode tokens."""
    x = rng(seed, STREAM_DECODE_X).standard_normal((batch, shape.hidden_size), dtype=np.float32)
    return to_dtype_values(x, act_dtype)


def history_hidden(shape, seq, start, count, act_dtype, seed=0):
    """Hidden states [count, D] of positions start .. start+count-1 of sequence `seq`'s history.

    Drawn in blocks of HISTORY_BLOCK tokens from stream (STREAM_HISTORY + seq, block index), so
    any range can be regenerated without drawing the rest.
    """
    D = shape.hidden_size
    out = np.empty((count, D), dtype=np.float32)
    pos = start
    while pos < start + count:
        blk = pos // HISTORY_BLOCK
        lo = blk * HISTORY_BLOCK
        take = min(start + count, lo + HISTORY_BLOCK) - pos
        block = rng(seed, STREAM_HISTORY + seq, blk).standard_normal((HISTORY_BLOCK, D), dtype=np.float32)
        out[pos - start:pos - start + take] = block[pos - lo:pos - lo + take]
        pos += take
    return to_dtype_values(out, act_dtype)


def history_hidden_many(shape, seqs_counts, act_dtype, seed=0, threads=None):
    """history_hidden for several (seq, count) pairs in a thread pool (numpy drops the GIL)."""
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda sc: history_hidden(shape, sc[0], 0, sc[1], act_dtype, seed), seqs_counts))


def prefill_hidden(shape, seq, length, act_dtype, seed=0):
    """Prompt hidden states [length, D] of prefill sequence `seq`."""
    x = rng(seed, STREAM_PREFILL + seq).standard_normal((length, shape.hidden_size), dtype=np.float32)
    return to_dtype_values(x, act_dtype)
