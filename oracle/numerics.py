"""Storage rounding used by the oracle: fp32, bf16 and OCP fp8 e4m3 (with a per-token scale).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU library imports this.

The cache format is part of what the method stores ([MTRT], section "源码里的压缩全流程",
step "写入缓存": what is written is the latent plus k_pe), so the oracle rounds exactly once,
where a row is written to the cache.  The pages name fp8 quantisation without a format
([HOTDRY-OPT], the deployment section on vLLM/SGLang); the reading taken here is the OCP e4m3
("e4m3fn") encoding with one fp32 scale per token:

    s    = amax(|row|) / 448          (fp32 arithmetic; amax == 0 gives s = 1)
    code = e4m3(RNE(row / s))         (fp32 division, round to nearest even, saturate at +-448)
    value = s * code

Every function here works elementwise on numpy arrays and returns float64 arrays holding the
exactly representable stored value.
"""
import numpy as np

E4M3_MAX = 448.0


def fp32_round(x):
    """Round to the nearest float32 (numpy's cast is round-to-nearest-even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even; returned as fp64.

    bfloat16 keeps 8 significant bits (7 stored + the implicit one) and float32's exponent
    range, so the quantum of a normal value x = m * 2**e (0.5 <= |m| < 1) is 2**(e - 8); below
    the smallest normal (2**-126) the quantum stays at the subnormal step 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_round expects finite values")
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)  # np.rint rounds half to even
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise OverflowError("value outside the bfloat16 range")
    return r


def e4m3_quantise(v):
    """Nearest e4m3fn value to v (ties to even), saturating at +-448. Returns float64 values.

    e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; normal magnitudes run
    from 2**-6 to 448 = 1.75 * 2**8 (the all-ones pattern is NaN, so 480 does not exist);
    subnormals are multiples of 2**-9.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                      # a = m * 2**e with 0.5 <= m < 1, so floor(log2 a) = e - 1
    exp = np.maximum(e - 1, -6)             # below 2**-6 the step stays at the subnormal 2**-9
    quantum = np.ldexp(1.0, exp - 3)        # 3 mantissa bits
    r = np.rint(a / quantum) * quantum      # a / quantum is exact (power-of-two divisor)
    r = np.minimum(r, E4M3_MAX)
    return np.where(v < 0, -r, r)


def e4m3_encode_values(r):
    """Byte codes of values that are already exact e4m3 values (as returned by e4m3_quantise)."""
    r = np.asarray(r, dtype=np.float64)
    sign = (np.signbit(r)).astype(np.uint8) << 7
    a = np.abs(r)
    codes = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    codes[sub] = np.rint(a[sub] * 512.0).astype(np.uint8)      # exponent field 0, value m * 2**-9
    nrm = ~sub
    _, e = np.frexp(a[nrm])
    ex = e - 1                                                  # unbiased exponent, -6 .. 8
    mant = np.rint((a[nrm] / np.ldexp(1.0, ex) - 1.0) * 8.0).astype(np.int64)
    codes[nrm] = (((ex + 7) << 3) | mant).astype(np.uint8)
    return codes | sign


def e4m3_decode_codes(codes):
    """Values of e4m3fn byte codes; the two NaN codes (0x7F, 0xFF) decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def fp8_store(rows):
    """Per-token e4m3 storage of rows [T, W]: returns (stored values fp64, codes uint8, scale fp32).

    The scale and the division are taken in float32 from the float32 row, i.e. in the precision
    the kernel makes the same decision in, so the integer codes are comparable.
    """
    r32 = np.asarray(rows, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(r32), axis=-1, keepdims=True).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    scaled = (r32 / scale).astype(np.float32)
    qv = e4m3_quantise(scaled.astype(np.float64))
    codes = e4m3_encode_values(qv)
    values = qv * scale.astype(np.float64)
    return values, codes, scale[..., 0]


def store_rows(rows, cache_dtype):
    """Round cache rows to their storage format. cache_dtype is 'f32', 'bf16' or 'fp8'.

    Returns (values fp64, codes or None, scale or None).
    """
    if cache_dtype == "f32":
        return fp32_round(rows), None, None
    if cache_dtype == "bf16":
        return bf16_round(rows), None, None
    if cache_dtype == "fp8":
        return fp8_store(rows)
    raise ValueError(f"unknown cache dtype {cache_dtype!r}")
