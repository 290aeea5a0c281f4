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


def bf16_out_ok(got, ref, bar):
    """A bf16 output may add its own rounding (half an ulp, <= 2^-8 of the value) to the bar."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return bool(np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + bar * rms))


# Error bars: max|err| / rms(out) per output token, fp32 output.
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
