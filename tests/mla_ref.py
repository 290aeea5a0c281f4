"""Glue between the seeded workloads and the fp64 oracle (test-side only).

The oracle consumes exactly the values the GPU receives: the float32 arrays the input
generator produced (already rounded to the activation dtype), upcast to fp64.  History rows
are recomputed by the oracle from the regenerated history hidden states.
"""
import numpy as np

import oracle
from mla_latent_kv_compress_amd import inputs


def oracle_dims(shape):
    return oracle.Dims(shape.hidden_size, shape.num_heads, shape.q_lora_rank, shape.kv_lora_rank,
                       shape.qk_nope_head_dim, shape.qk_rope_head_dim, shape.v_head_dim, shape.rope_theta,
                       shape.rms_eps, shape.softmax_scale, shape.rope_factor, shape.rope_original_max_position,
                       shape.rope_beta_fast, shape.rope_beta_slow, shape.rope_mscale)


def oracle_weights(layer):
    return {k: v.astype(np.float64) for k, v in layer.w_host.items()}


def history_rows(layer, seq, length, seed=0, chunk=16384):
    """Stored cache rows (fp64 values) of positions 0..length-1 of history sequence `seq`."""
    d, W = oracle_dims(layer.shape), oracle_weights(layer)
    out = np.empty((length, d.row_width))
    for s in range(0, length, chunk):
        n = min(chunk, length - s)
        x = inputs.history_hidden(layer.shape, seq, s, n, layer.act, seed).astype(np.float64)
        out[s:s + n] = oracle.cache_rows(d, W, x, np.arange(s, s + n), layer.cache_dtype)[0]
    return out


def decode_rows_and_queries(layer, batch, seq, seed=0):
    """The oracle's stored rows of sequence `seq` after its decode token is appended, and that
    token's queries (the first steps of oracle.decode_one)."""
    d, W = oracle_dims(layer.shape), oracle_weights(layer)
    L = int(batch.hist[seq])
    x = batch.x_host[seq].astype(np.float64)
    new_row, _, _ = oracle.cache_rows(d, W, x[None, :], np.array([L]), layer.cache_dtype)
    rows = np.concatenate([history_rows(layer, seq, L, seed), new_row], axis=0)
    q_nope, q_pe = oracle.queries(d, W, x[None, :], np.array([L]))
    return rows, q_nope[0], q_pe[0]


def absorbed_all_heads(layer, rows, q_nope, q_pe):
    """All heads of one decode token in the weight-absorbed form, fp64, the heads batched into
    three matrix products (oracle.attend_absorbed computes the same head by head, too slowly for
    131072 rows): Q^h = [W_UK^h^T q_nope^h | q_pe^h], p^h = softmax(sigma Q^h . rows),
    o^h = W_UV^h (p^h . rows[:, :d_c]).  A test checks it against the explicit oracle on sampled
    heads before using it."""
    d, W = oracle_dims(layer.shape), oracle_weights(layer)
    dc = d.kv_lora_rank
    blk = W["kv_b_proj"].reshape(d.heads, d.qk_nope + d.v_head, dc)
    w_uk, w_uv = blk[:, : d.qk_nope], blk[:, d.qk_nope:]                # [H, d_n, d_c], [H, d_v, d_c]
    q_hat = np.concatenate([np.einsum("hn,hnc->hc", q_nope, w_uk), q_pe], axis=1)   # [H, d_c + d_r]
    p = oracle.softmax(d.sigma * (q_hat @ rows.T), axis=1)                # [H, n]
    o_lat = p @ rows[:, :dc]                                             # [H, d_c]
    return np.einsum("hvc,hc->hv", w_uv, o_lat)


def decode_reference(layer, batch, seq, heads=None, seed=0, hist_rows=None):
    d, W = oracle_dims(layer.shape), oracle_weights(layer)
    L = int(batch.hist[seq])
    rows = history_rows(layer, seq, L, seed) if hist_rows is None else hist_rows
    out, _ = oracle.decode_one(d, W, batch.x_host[seq].astype(np.float64), rows, layer.cache_dtype, heads=heads)
    return out


def rel_err(got, ref):
    """max |got - ref| / rms(ref) over one token's output [H, d_v] (or any array)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref * ref)))


def token_err(got, ref):
    """Worst per-token rel_err over the leading (token) axis."""
    return max(rel_err(got[i], ref[i]) for i in range(len(ref)))


def bf16_half_quantum(x):
    """Half the spacing of bfloat16 values around each x: the most a round-to-nearest store of x
    in bf16 can move it (x = m 2^e with 0.5 <= |m| < 1 has quantum 2^(e - 8))."""
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e - 9, -134))


def bf16_out_ok(got, ref, bar):
    """A bf16 output within the bar, plus the format's own rounding of each value: |got - ref| <=
    bar * rms(ref) + half a bf16 quantum of ref (the store of an exact result could move it that
    far; the computation's error is what the bar bounds)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return bool(np.all(np.abs(got - ref) <= bar * rms + bf16_half_quantum(ref)))


# Error bars: max|err| / rms(out) per output token, fp32 output.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
