"""Plain fp64 definition of Multi-head Latent Attention (MLA) over a latent KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, in the pages' order ([MTRT], sections "MLA 的两个核心部件" and
"源码里的压缩全流程"):

  query      q = q_b_proj(q_a_layernorm(q_a_proj(x)))   (or q = q_proj(x) with no query
             compression); per head q = [q_nope (d_n) | q_pe (d_r)], RoPE on q_pe only.
  compress   a = kv_a_proj_with_mqa(x) = [latent c (d_c) | k_pe (d_r)]; the latent is
             RMS-normalised (kv_a_layernorm), k_pe is rotated by RoPE; the cache row is
             [c_hat | k_pe_hat] -- d_c + d_r values per token per layer, shared by all heads
             ([MTRT], FAQ Q2 and the table in "省了多少").
  decompress kv_b_proj maps the latent back to per-head [k_nope (d_n) | v (d_v)].
  attend     k_h = [k_nope_h | k_pe] (the one k_pe is broadcast to every head); scores are
             sigma * q_h . k_h, softmax over the context, o_h = sum p * v_h.

Weights use the (out, in) layout of a linear layer.  Readings where the pages are silent
(listed with reasons in the design notes): sigma = 1/sqrt(d_n + d_r); RMSNorm is
x / sqrt(mean(x^2) + eps) * gamma; RoPE rotates adjacent pairs (2i, 2i+1) with
theta_i = base^(-2i/d_r) and the phase taken in fp64; q_b_proj rows of head h are
[nope | rope]; kv_b_proj rows of head h are [k_nope | v]; a decode token is appended to
the cache before it attends, so it attends to itself.
"""
from dataclasses import dataclass
import math

import numpy as np

from .numerics import store_rows


@dataclass(frozen=True)
class Dims:
    hidden: int
    heads: int
    q_lora_rank: int          # 0: no query compression (a single q_proj)
    kv_lora_rank: int         # d_c
    qk_nope: int              # d_n
    qk_rope: int              # d_r
    v_head: int               # d_v
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    softmax_scale: float = 0.0   # 0: 1/sqrt(d_n + d_r)
    # YaRN context extension of the rotary embedding (rope_factor <= 1: plain RoPE).  The pages
    # name YaRN as how the 128K context is reached but give no constants.
    rope_factor: float = 0.0
    rope_original_max_position: int = 0
    rope_beta_fast: float = 0.0
    rope_beta_slow: float = 0.0
    rope_mscale: float = 0.0     # 0: 1

    @property
    def rope_args(self):
        """Keyword arguments of rope() for this layer."""
        return dict(factor=self.rope_factor, original=self.rope_original_max_position,
                    beta_fast=self.rope_beta_fast, beta_slow=self.rope_beta_slow,
                    mscale=self.rope_mscale or 1.0)

    @property
    def sigma(self):
        if self.softmax_scale:
            return float(self.softmax_scale)
        return 1.0 / math.sqrt(self.qk_nope + self.qk_rope)

    @property
    def row_width(self):
        """Values cached per token per layer: latent plus the shared RoPE key."""
        return self.kv_lora_rank + self.qk_rope

    @property
    def mha_width(self):
        """Values an uncompressed multi-head cache would hold per token per layer."""
        return self.heads * (self.qk_nope + self.v_head)


def rms_norm(v, gamma, eps):
    """RMSNorm over the last axis: v / sqrt(mean(v^2) + eps) * gamma."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * gamma


def rope_frequencies(d, theta, factor=0.0, original=0, beta_fast=0.0, beta_slow=0.0):
    """Angular frequency of each pair i < d/2.

    Plain RoPE: f_i = theta**(-2i/d).  With factor s > 1, YaRN's interpolation "by parts"
    (Peng et al., "YaRN: Efficient Context Window Extension of Large Language Models", the
    ramp over the number of turns a dimension makes across the original context): a pair whose
    wavelength 2 pi / f_i fits r = original * f_i / (2 pi) times into the original context keeps
    its frequency when r >= beta_fast, is slowed by the factor (f_i / s, i.e. plain position
    interpolation) when r <= beta_slow, and in between takes (1 - g) f_i / s + g f_i with
    g = (r - beta_slow) / (beta_fast - beta_slow).
    """
    f = float(theta) ** (-2.0 * np.arange(d // 2) / d)
    if factor <= 1.0:
        return f
    turns = original * f / (2.0 * np.pi)
    g = np.clip((turns - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return (1.0 - g) * (f / factor) + g * f


def rope(u, pos, theta, factor=0.0, original=0, beta_fast=0.0, beta_slow=0.0, mscale=1.0):
    """Rotary embedding of the last axis (even length d) at integer positions pos.

    Pair i = (u[2i], u[2i+1]) is rotated by the angle pos * f_i (rope_frequencies), and scaled
    by mscale (1 for the plain rotation).  pos broadcasts against u.shape[:-1].  The angle is
    formed in fp64.
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    freq = rope_frequencies(d, theta, factor, original, beta_fast, beta_slow)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    cos, sin = mscale * np.cos(ang), mscale * np.sin(ang)
    even, odd = u[..., 0::2], u[..., 1::2]
    out = np.empty(np.broadcast_shapes(u.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = even * cos - odd * sin
    out[..., 1::2] = even * sin + odd * cos
    return out


def kv_rows(dims, W, x, pos):
    """Cache rows [T, d_c + d_r] for hidden states x [T, D] at positions pos [T], before rounding.

    [MTRT], "源码里的压缩全流程", steps "KV 压缩" (the split: latent first, then k_pe) and
    "KV 解压" (kv_a_layernorm acts on the latent only); RoPE acts on k_pe only.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    a = x @ W["kv_a_proj"].T
    c = a[:, : dims.kv_lora_rank]
    k_pe = a[:, dims.kv_lora_rank:]
    c_hat = rms_norm(c, W["kv_a_norm"], dims.rms_eps)
    k_hat = rope(k_pe, np.asarray(pos), dims.rope_theta, **dims.rope_args)
    return np.concatenate([c_hat, k_hat], axis=1)


def cache_rows(dims, W, x, pos, cache_dtype):
    """kv_rows followed by the storage rounding of the cache format (values, codes, scale)."""
    return store_rows(kv_rows(dims, W, x, pos), cache_dtype)


def queries(dims, W, x, pos):
    """Per-head queries for x [T, D] at positions pos [T]: (q_nope [T,H,d_n], q_pe [T,H,d_r]).

    [MTRT], "源码里的压缩全流程", step "Query 低秩分解" (1536-rank path with its own
    RMSNorm) and step "拼回完整 Q / K" (RoPE acts on q_pe only).
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    if dims.q_lora_rank > 0:
        cq = rms_norm(x @ W["q_a_proj"].T, W["q_a_norm"], dims.rms_eps)
        q = cq @ W["q_b_proj"].T
    else:
        q = x @ W["q_proj"].T
    q = q.reshape(x.shape[0], dims.heads, dims.qk_nope + dims.qk_rope)
    q_nope = q[..., : dims.qk_nope]
    q_pe = rope(q[..., dims.qk_nope:], np.asarray(pos)[:, None], dims.rope_theta, **dims.rope_args)
    return q_nope, q_pe


def head_weights(dims, W, h):
    """(W_UK^h [d_n, d_c], W_UV^h [d_v, d_c]): head h's slices of kv_b_proj."""
    blk = W["kv_b_proj"][h * (dims.qk_nope + dims.v_head):(h + 1) * (dims.qk_nope + dims.v_head)]
    return blk[: dims.qk_nope], blk[dims.qk_nope:]


def softmax(s, axis=-1):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def attend_explicit(dims, W, q_nope, q_pe, rows, heads=None, return_probs=False, causal_limit=None):
    """Explicit (decompressing) attention of queries against cached rows.

    q_nope [Q, H, d_n], q_pe [Q, H, d_r]; rows [n, d_c + d_r] are the stored cache rows.
    causal_limit [Q]: query i sees rows [0, causal_limit[i]) (None: every row).
    heads: iterable of head indices to evaluate (None: all).  Returns O [Q, len(heads), d_v]
    (and the probabilities [Q, len(heads), n] if asked).

    Per head h: k_nope = W_UK^h c, v = W_UV^h c for every cached latent c ([MTRT],
    "源码里的压缩全流程", step "KV 解压"); k = [k_nope | k_pe] with the shared k_pe
    (FAQ Q2); softmax(sigma * q . k) weights the v.
    """
    rows = np.asarray(rows, dtype=np.float64)
    c = rows[:, : dims.kv_lora_rank]
    k_pe = rows[:, dims.kv_lora_rank:]
    nq, n = q_nope.shape[0], rows.shape[0]
    heads = list(range(dims.heads)) if heads is None else list(heads)
    mask = None
    if causal_limit is not None:
        mask = np.arange(n)[None, :] >= np.asarray(causal_limit)[:, None]   # [Q, n] True = hidden
    out = np.empty((nq, len(heads), dims.v_head))
    probs = np.empty((nq, len(heads), n)) if return_probs else None
    for j, h in enumerate(heads):
        w_uk, w_uv = head_weights(dims, W, h)
        k_nope = c @ w_uk.T                    # [n, d_n]
        v = c @ w_uv.T                         # [n, d_v]
        s = dims.sigma * (q_nope[:, h] @ k_nope.T + q_pe[:, h] @ k_pe.T)   # [Q, n]
        if mask is not None:
            s = np.where(mask, -np.inf, s)
        p = softmax(s, axis=1)
        out[:, j] = p @ v
        if return_probs:
            probs[:, j] = p
    return (out, probs) if return_probs else out


def attend_absorbed(dims, W, q_nope, q_pe, rows, heads=None):
    """Second fp64 path, weight-absorbed: used only to pin the identity with attend_explicit.

    q_lat = W_UK^h^T q_nope scores the latent directly; the probability-weighted latent is
    mapped to the output by W_UV^h.  Equal to the explicit form because kv_b_proj is linear.
    """
    rows = np.asarray(rows, dtype=np.float64)
    heads = list(range(dims.heads)) if heads is None else list(heads)
    out = np.empty((q_nope.shape[0], len(heads), dims.v_head))
    for j, h in enumerate(heads):
        w_uk, w_uv = head_weights(dims, W, h)
        q_hat = np.concatenate([q_nope[:, h] @ w_uk, q_pe[:, h]], axis=1)   # [Q, d_c + d_r]
        p = softmax(dims.sigma * (q_hat @ rows.T), axis=1)
        out[:, j] = (p @ rows[:, : dims.kv_lora_rank]) @ w_uv.T
    return out


def decode_one(dims, W, x_new, history_rows, cache_dtype, heads=None):
    """One decode step of one sequence.

    x_new [D] is the new token's hidden state; history_rows [L, d_c + d_r] are the stored rows
    of positions 0..L-1.  The new token (position L) is compressed, rounded to the cache format
    and appended, then attends over all L + 1 rows.  Returns (O [H', d_v], stored new row).
    """
    L = history_rows.shape[0]
    new_row, _, _ = cache_rows(dims, W, x_new[None, :], np.array([L]), cache_dtype)
    rows = np.concatenate([history_rows, new_row], axis=0)
    q_nope, q_pe = queries(dims, W, x_new[None, :], np.array([L]))
    return attend_explicit(dims, W, q_nope, q_pe, rows, heads=heads)[0], new_row[0]


def prefill_chunk(dims, W, x, start_pos, prior_rows, cache_dtype, heads=None, query_rows=None):
    """Causal prefill of one chunk of one sequence.

    x [n, D] are the chunk's hidden states at positions start_pos .. start_pos + n - 1;
    prior_rows [start_pos, d_c + d_r] are the stored rows of the earlier positions.  The chunk's
    rows are rounded and appended first, then query i attends to positions <= start_pos + i.
    query_rows: optional subset of chunk rows to evaluate.  Returns (O [n', H', d_v], new rows).
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    n = x.shape[0]
    pos = start_pos + np.arange(n)
    new_rows, _, _ = cache_rows(dims, W, x, pos, cache_dtype)
    rows = np.concatenate([prior_rows, new_rows], axis=0) if start_pos else new_rows
    sel = np.arange(n) if query_rows is None else np.asarray(query_rows)
    q_nope, q_pe = queries(dims, W, x[sel], pos[sel])
    out = attend_explicit(dims, W, q_nope, q_pe, rows, heads=heads, causal_limit=pos[sel] + 1)
    return out, new_rows


def output_projection(dims, W, o):
    """The attention output taken back to the model width: the last step of the forward flow.

    [MTRT], section "MLA 的两个核心部件": the flow ends with the attention result passed on as
    the layer's output.  The pages name no output projection; the reading taken is a linear
    layer o_proj of (out, in) layout [hidden, H * d_v] applied to the heads' outputs laid side by
    side in head order (head h fills inputs h * d_v .. h * d_v + d_v - 1), as the input
    projections are laid out.  o: [..., H, d_v]  ->  [..., hidden].
    """
    o = np.asarray(o, dtype=np.float64)
    flat = o.reshape(o.shape[:-2] + (dims.heads * dims.v_head,))
    return flat @ np.asarray(W["o_proj"], dtype=np.float64).T
