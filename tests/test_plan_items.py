"""Host-side check of the forward plan's work items (no GPU).

Builds tests/plan_items_check.cpp with the library's host planner sources
(plan.cpp, mask_spec.cpp) using g++, and runs it: for fixed and random mask
specs, lengths, tile heights and split caps, the items of each query block,
taken in order, must hold exactly the block's in-place tiles and gathered
keys, cut on whole tiles, with consistent partial slots, merge lists and a
heaviest-first order; the backward plan's key-block items likewise hold
each key block's query tiles exactly.  The split is a rearrangement of work, so the fp64
oracle is not involved; the GPU parity tests then check the merged results.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "block_sparse_masked_spec_amd", "csrc")


SOURCES = [os.path.join(HERE, "plan_items_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "mask_spec.cpp")]


def build_and_run(tmp_path, name, flags, env=None):
    exe = str(tmp_path / name)
    build = subprocess.run(["g++", "-std=c++20", "-Wall", *flags, "-o", exe, *SOURCES],
                           capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                         env={**os.environ, **(env or {})})
    assert run.returncode == 0 and run.stdout.startswith("ok"), run.stdout[-2000:] + run.stderr[-4000:]
    assert int(run.stdout.split()[1]) >= 1200


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_split_items_cover_each_block_exactly(tmp_path):
    build_and_run(tmp_path, "plan_items_check", ["-O1"])


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_parser_and_planner_under_address_and_ub_sanitizers(tmp_path):
    """The same program (plan coverage plus 20000 fuzzed specs through the
    parser) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
    host: any out-of-bounds access, leak, overflow or other undefined
    behaviour in the parser or planner aborts it."""
    build_and_run(tmp_path, "plan_items_check_asan",
                  ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined"],
                  env={"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
