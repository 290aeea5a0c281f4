"""The HIP-free validation and planning unit (mla_plan.cpp), built with a plain host compiler
under AddressSanitizer and UndefinedBehaviorSanitizer and driven by tests/host/plan_driver.cpp:
configuration and argument statuses, workspace regions (aligned, disjoint, inside the size), the
decode split choice and which ragged batches are ranked longest first.  CPU only."""
import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_compress_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = tmp_path_factory.mktemp("plan") / "plan_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "plan_driver.cpp"), os.path.join(CSRC, "mla_plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return str(exe)


def run(driver, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver, *map(str, args)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_validation_and_regions_under_sanitizers(driver):
    out = run(driver, "check")
    assert "FAIL" not in out, out
    assert out.strip().endswith("0 failures")


def ctx_blocks(lengths):
    return max((L + 1 + 63) // 64 for L in lengths)


@pytest.mark.parametrize("B,max_len,splits,ranked", [
    (8, 3100, 20, False),      # more than 8 splits: not ranked
    (20, 700, 8, True),        # 20 x 8 x 2 = 320 work-groups > 256, 8 splits: ranked
    (21, 700, 7, True),        # 294 working work-groups: ranked
    (64, 8192, 2, False),      # the 236B workload: one round (256 work-groups)
    (128, 32768, 2, True),     # the mixed workload's ragged batch
])
def test_ranking_rule(driver, B, max_len, splits, ranked):
    plan = json.loads(run(driver, "decode", 128, B, ctx_blocks([max_len]), splits))
    assert plan["ordered"] is ranked
    assert plan["cq_pair"] is True
    assert plan["hidden_pair"] is False              # (a query LoRA: the grouped front instead)


def test_auto_splits(driver):
    # 32 sequences x 2 head groups = 64 work-groups: 4 splits fill 256 CUs (room for them)
    assert json.loads(run(driver, "decode", 128, 32, 11, 0))["splits"] == 4
    # the 236B workload: 64 x 2 x 2 = 256
    assert json.loads(run(driver, "decode", 128, 64, 129, 0))["splits"] == 2
    # a short block table caps the count at half its pages
    assert json.loads(run(driver, "decode", 128, 32, 5, 0))["splits"] == 2


def test_prefill_plan(driver):
    assert json.loads(run(driver, "prefill", 4, 4096, 1024, 4096))["q16"] is True
