"""C ABI checks that need no GPU: symbols, struct layout, host-side validation, workspace sizes.

Every call here fails validation (or is a pure size query) and returns before any HIP call,
so nothing runs on a device.
"""
import ctypes
import os
import re
import subprocess

import pytest

from mla_latent_kv_compress_amd import api
from mla_latent_kv_compress_amd.configs import DSV2, LITE, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(api.LIB_PATH), reason="libmla.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) == 13
    L = api.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in api.SIGNATURES, f"binding lacks {n}"
    nm = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (mla_[a-z0-9_]+)$", nm, flags=re.M))
    assert exported == set(names)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mla.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(mla_config), '
                   'offsetof(mla_config, rope_theta), offsetof(mla_config, cache_dtype), sizeof(mla_weights), '
                   'sizeof(mla_cache), offsetof(mla_cache, num_blocks)); return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(api.MlaConfig), api.MlaConfig.rope_theta.offset, api.MlaConfig.cache_dtype.offset,
            ctypes.sizeof(api.MlaWeights), ctypes.sizeof(api.MlaCache), api.MlaCache.num_blocks.offset]
    assert got == want


def cfg(shape=DSV2, act="bf16", cache="bf16", **kw):
    c = api.make_config(shape, act, cache)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_status_strings():
    L = api.lib()
    assert L.mla_status_string(0) == b"ok"
    for s in range(1, 5):
        assert L.mla_status_string(s) not in (b"ok", b"unknown status")
    assert L.mla_status_string(99) == b"unknown status"


@pytest.mark.parametrize("bad,code", [
    (dict(page_size=32), 1), (dict(qk_rope_head_dim=63), 1), (dict(num_heads=0), 1),
    (dict(act_dtype=7), 1), (dict(cache_dtype=9), 1), (dict(rope_theta=0.0), 1), (dict(rms_eps=-1.0), 1),
    (dict(softmax_scale=float("nan")), 1), (dict(kv_lora_rank=256), 2), (dict(num_heads=24), 2),
    (dict(act_dtype=api.F32, cache_dtype=api.BF16), 2),
    # YaRN: a factor above 1 needs the original context length and beta_fast > beta_slow >= 0
    (dict(rope_factor=8.0), 1), (dict(rope_factor=8.0, rope_original_max_position=4096, rope_beta_fast=1.0,
                                      rope_beta_slow=32.0), 1),
    (dict(rope_factor=8.0, rope_original_max_position=4096, rope_beta_fast=32.0, rope_beta_slow=-1.0), 1),
    (dict(rope_mscale=-1.0), 1), (dict(rope_factor=float("inf")), 1),
    (dict(prefill_key_block=-64), 1),
])
def test_config_validation(bad, code):
    L = api.lib()
    c = cfg(**bad)
    assert L.mla_decode_workspace_size(ctypes.byref(c), 4, 8, 0) == 0
    w = api.MlaWeights(*([ctypes.c_void_p(16)] * 6))
    cache = api.MlaCache(ctypes.c_void_p(16), ctypes.c_void_p(16), 8)
    one = ctypes.c_void_p(16)
    st = L.mla_decode(ctypes.byref(c), ctypes.byref(w), one, one, one, 8, ctypes.byref(cache), 4, 0, one, 1 << 30,
                      one, None)
    assert st == code


def test_argument_validation_returns_before_any_launch():
    L = api.lib()
    c = cfg()
    one = ctypes.c_void_p(16)
    w = api.MlaWeights(*([one] * 6))
    cache = api.MlaCache(one, None, 8)
    ws_need = L.mla_decode_workspace_size(ctypes.byref(c), 4, 8, 0)
    assert ws_need > 0
    args = lambda **k: dict(dict(hidden=one, ctx=one, bt=one, mb=8, B=4, S=0, ws=one, wsb=ws_need, out=one), **k)

    def call(**k):
        a = args(**k)
        return L.mla_decode(ctypes.byref(c), ctypes.byref(w), a["hidden"], a["ctx"], a["bt"], a["mb"],
                            ctypes.byref(cache), a["B"], a["S"], a["ws"], a["wsb"], a["out"], None)
    assert call(hidden=None) == 1
    assert call(ctx=None) == 1
    assert call(out=None) == 1
    assert call(B=0) == 1
    assert call(mb=0) == 1
    assert call(S=-1) == 1
    assert call(S=2000) == 1
    assert call(ws=None) == 3
    assert call(wsb=ws_need - 1) == 3
    # fp8 cache without scales
    c8 = cfg(cache="fp8")
    assert L.mla_decode(ctypes.byref(c8), ctypes.byref(w), one, one, one, 8, ctypes.byref(cache), 4, 0, one,
                        1 << 40, one, None) == 1
    # missing query weights
    w2 = api.MlaWeights(None, None, one, one, one, one)
    assert L.mla_decode(ctypes.byref(c), ctypes.byref(w2), one, one, one, 8, ctypes.byref(cache), 4, 0, one,
                        1 << 40, one, None) == 1
    # compress: negative count, missing slots; zero tokens is a no-op
    assert L.mla_compress_append(ctypes.byref(c), ctypes.byref(w), one, one, one, ctypes.byref(cache), -1, one,
                                 1 << 30, None) == 1
    assert L.mla_compress_append(ctypes.byref(c), ctypes.byref(w), one, one, None, ctypes.byref(cache), 3, one,
                                 1 << 30, None) == 1
    assert L.mla_compress_append(ctypes.byref(c), ctypes.byref(w), one, one, one, ctypes.byref(cache), 0, None,
                                 0, None) == 0
    # stream read: byte count not a multiple of 16, misaligned or null source, unknown mode;
    # 0 bytes no-op
    assert L.mla_stream_read(one, 24, one, 0, None) == 1
    assert L.mla_stream_read(ctypes.c_void_p(8), 32, one, 1, None) == 1
    assert L.mla_stream_read(None, 32, one, 0, None) == 1
    assert L.mla_stream_read(one, 32, one, 2, None) == 1
    assert L.mla_stream_read(one, 32, one, -1, None) == 1
    assert L.mla_stream_read(None, 0, None, 1, None) == 0
    # prefill: max_ctx beyond the block table, chunk longer than the context
    assert L.mla_prefill(ctypes.byref(c), ctypes.byref(w), one, one, one, one, 2, ctypes.byref(cache), 1, 64, 64,
                         129, one, 1 << 40, one, None) == 1
    assert L.mla_prefill(ctypes.byref(c), ctypes.byref(w), one, one, one, one, 2, ctypes.byref(cache), 1, 64, 100,
                         64, one, 1 << 40, one, None) == 1


def test_workspace_sizes_and_splits():
    L = api.lib()
    for shape, act, cache in [(TINY, "f32", "f32"), (LITE, "bf16", "bf16"), (DSV2, "bf16", "fp8")]:
        c = cfg(shape, act, cache)
        a = L.mla_decode_workspace_size(ctypes.byref(c), 8, 16, 1)
        b = L.mla_decode_workspace_size(ctypes.byref(c), 8, 16, 4)
        assert 0 < a < b
        assert L.mla_decode_workspace_size(ctypes.byref(c), 16, 16, 4) > b
        assert L.mla_prefill_workspace_size(ctypes.byref(c), 2, 100, 60, 128) > 0
        # a long chunk (kv_a and q_a as K-split partials of the 256 x 256-tile kernel; Lite has
        # no query LoRA)
        assert L.mla_prefill_workspace_size(ctypes.byref(c), 4, 4096, 1024, 4096) > 0
        assert L.mla_compress_append_workspace_size(ctypes.byref(c), 10) > 0
        s = L.mla_decode_num_splits(ctypes.byref(c), 4, 2049)
        assert 1 <= s <= 64
    c = cfg()
    assert L.mla_decode_num_splits(ctypes.byref(c), 64, 129) * 64 * 2 >= 256   # fills 256 CUs


def test_prefill_workspace_bounded_by_the_key_block():
    """The prefill workspace holds one key block of decompressed keys and values per sequence:
    with the library's choice it stays near 2 GiB of them however long the context (plus the
    running softmax state), and an explicit block bounds it further."""
    L = api.lib()
    c = cfg()
    size = lambda cc, ctx: L.mla_prefill_workspace_size(ctypes.byref(cc), 4, 4096, 1024, ctx)
    whole = size(c, 4096)
    assert size(c, 8192) > whole                          # two blocks' worth fits under the budget
    assert size(c, 131072) < 3 * 2 ** 30                  # 128K: blocks, not the whole context
    assert size(c, 131072) == size(c, 65536)              # bounded by the block, not the context
    c.prefill_key_block = 1024
    assert size(c, 131072) < whole


def test_decode_split_choice_for_the_workloads():
    """Splits the library picks: enough 64-head work-groups (two head groups at 128 heads) for one
    round over 256 CUs; a batch that fills a round by itself with block tables of 4096+ tokens gets
    two rounds, since its lengths may be ragged and the work-groups go longest first."""
    L = api.lib()
    bf16, fp8 = cfg(DSV2, "bf16", "bf16"), cfg(DSV2, "bf16", "fp8")
    assert L.mla_decode_num_splits(ctypes.byref(bf16), 64, 129) == 2            # 64 x 8193 tokens
    assert L.mla_decode_num_splits(ctypes.byref(bf16), 4, 2049) == 32           # 4 x 131072 tokens
    assert L.mla_decode_num_splits(ctypes.byref(fp8), 128, 512) == 2            # ragged 512..32768
    assert L.mla_decode_num_splits(ctypes.byref(fp8), 128, 32) == 1             # short contexts: one round
    lite = cfg(LITE, "bf16", "bf16")
    assert L.mla_decode_num_splits(ctypes.byref(lite), 32, 65) == 8             # 16 heads: one group
