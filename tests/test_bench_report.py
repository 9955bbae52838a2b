"""bench.py's report helpers on the CPU: the suite's markdown summary is built
from a suite dict alone, and every section it writes shows up."""

import json

import bench


def _entry(us, nbytes=1 << 20, **extra):
    e = bench.rate(nbytes, us)
    e.update(splits=1, layers=1, tokens_per_s_per_layer=123.0, query_tokens_per_s_per_layer=456.0)
    e.update(extra)
    return e


def _suite():
    S = {}
    S["fp32 5 requests (37..511 tokens), one layer"] = _entry(10.5, splits=32)
    S["bf16 256 mixed-length requests, 32 layers"] = _entry(
        51.0, full_step_us=1800.0, full_step_fused_us=1700.0, full_step_append_layers_us=1690.0,
        longest_first=dict(bench.rate(1 << 20, 49.0), tokens_per_s_per_layer=1.0, full_step_append_layers_us=1600.0),
        swap_500MiB=dict(out_ms=9.6, in_ms=9.4, out_GiB_s=50.9, in_GiB_s=51.8, bytes=524288000))
    S["bf16 prefix sharing, 64 branches (COW), one layer"] = _entry(38.8, full_step_us=175.0)
    S["bf16 168 x 1025 tokens, 24 layers"] = _entry(62.0, full_step_us=1560.0)
    for B in (8, 16, 32, 64):
        S[f"bf16 32 x 4096 tokens, block size {B}"] = _entry(86.0 + B / 64)
    S["bf16 verification, 32 x 4096 tokens, T = 16 query tokens"] = _entry(110.0, splits=2)
    S["bf16 prompt chunk, 8 x 4096 tokens, T = 512 query tokens"] = _entry(
        400.0, TFLOP_s=640.0, frac_bf16_mfma_peak=0.256)
    S["bf16 re-prefill attention, one 4000-token request in 512-token chunks"] = dict(
        us_per_layer=520.0, chunks=8, TFLOP_s=250.0, frac_bf16_mfma_peak=0.1, ms_for_32_layers=16.6)
    return S


def test_suite_markdown_has_every_section():
    S = json.loads(json.dumps(_suite()))  # as read back from the JSON file
    md = bench.suite_markdown(S, "python3 bench.py --suite x.json")
    for needle in ("python3 bench.py --suite x.json", "| bf16 256 mixed-length requests, 32 layers | 51.000 |",
                   "issued longest first | 49.000 |", "| bf16 verification, 32 x 4096 tokens, T = 16 query tokens |",
                   "| 640.0 | 25.6 % |", "| 16 | 86.250 |", "## Block swap", "| out (pool -> host) | 9.6 | 50.9 |",
                   "## Swap or recompute", "| 520.0 | 8 | 250.0 | 10.0 % | 16.6 |"):
        assert needle in md, needle
    assert md.endswith("\n")


def test_suite_markdown_without_the_optional_parts():
    S = _suite()
    del S["bf16 256 mixed-length requests, 32 layers"]["longest_first"]
    del S["bf16 256 mixed-length requests, 32 layers"]["swap_500MiB"]
    del S["bf16 re-prefill attention, one 4000-token request in 512-token chunks"]
    md = bench.suite_markdown(S, "cmd")
    assert "longest first" not in md and "## Block swap" not in md and "## Swap or recompute" not in md
