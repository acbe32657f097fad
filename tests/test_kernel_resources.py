"""Register and scratch budgets of the kernels, from the compiler's
kernel-resource-usage remarks that the build records
(token_level_top_amd/_build/resource_usage.json). No GPU needed.

A kernel that starts to spill after an edit still passes every parity test;
it only runs slower (the decode split kernel lost 4 % to a 12-byte spill).
These checks make such a change visible at build time:
  * the streaming kernels (decode split-K, decode scores, sparse gathers and
    their combines, pass 1, the KV projection, selection, staging) use no
    scratch at all;
  * the pass-2 score kernels run four waves per SIMD where their launcher asks
    for it, which at 128 VGPRs costs them a few spilled loop-invariant values
    (reloaded in the trim path and, for FP8, once per tile); three waves
    without the spill measured slower, so the spill is bounded here instead;
  * the occupancy each hot kernel is tuned for still holds.
"""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RES = os.path.join(ROOT, "token_level_top_amd", "_build", "resource_usage.json")

NO_SCRATCH = {"decode_split_kernel", "decode_score_kernel", "rows_attn_kernel", "combine_kernel",
              "attn_fwd_pipe_kernel", "kv_project_dma_kernel", "kv_project_kernel", "select_collect_kernel",
              "select_hist_kernel", "select_final_kernel", "block_select_kernel", "prep_kv_kernel",
              "widen_fp8_kernel", "fill_u32_kernel", "probe_gather_kernel", "probe_mfma_kernel", "probe_stream_kernel"}
BOUNDED_SCRATCH = {"score_stream_kernel": 48, "block_score_kernel": 48, "attn_fwd_kernel": 48}


def _parse(name):
    m = re.match(r"_ZN3hs2\d+([a-z_0-9]+?)([IE].*)", name)  # kernel names are lower case
    if not m:
        return None, []
    args = m.group(2)
    return m.group(1), [int(x) for x in re.findall(r"L[ib](\d+)E", args)] if args.startswith("I") else []


@pytest.fixture(scope="module")
def res():
    if not os.path.exists(RES):
        pytest.skip("library not built (run __graft_entry__.build())")
    with open(RES) as f:
        return json.load(f)


def test_every_kernel_family_is_recorded(res):
    fams = {_parse(k)[0] for k in res}
    assert NO_SCRATCH | set(BOUNDED_SCRATCH) <= fams, sorted((NO_SCRATCH | set(BOUNDED_SCRATCH)) - fams)


def test_streaming_kernels_use_no_scratch(res):
    bad = [(k, v["scratch"]) for k, v in res.items() if _parse(k)[0] in NO_SCRATCH and v["scratch"] != 0]
    assert not bad, bad


def test_score_kernels_spill_at_most_a_few_values(res):
    bad = [(k, v["scratch"]) for k, v in res.items()
           if _parse(k)[0] in BOUNDED_SCRATCH and v["scratch"] > BOUNDED_SCRATCH[_parse(k)[0]]]
    assert not bad, bad


def test_hot_kernel_occupancy(res):
    seen = 0
    for k, v in res.items():
        fam, args = _parse(k)
        if fam == "decode_split_kernel":
            assert v["occupancy"] >= 2, (k, v)      # two 4-wave workgroups per CU
        elif fam == "attn_fwd_pipe_kernel":
            assert v["occupancy"] >= 2, (k, v)      # 8-wave workgroups, two waves per SIMD
        elif fam == "kv_project_dma_kernel":
            assert v["occupancy"] == 2, (k, v)      # 8 waves, 128 KiB of LDS: one workgroup per CU
        elif fam == "score_stream_kernel" and args[0] == 16 and args[2] in (1, 2):
            assert v["occupancy"] == 4, (k, v)      # 16 heads, bf16 / FP8 cache: four waves per SIMD
        else:
            continue
        seen += 1
    assert seen > 0
