"""Pins of the acceptance-rate model used for Sparse-to-Dense's I/O
argument (bench.py): the closed form of the expected tokens per round
against an explicit sum over accepted-prefix lengths, its limits, and the
per-token accounting."""
import pytest

import bench


@pytest.mark.parametrize("gamma", [1, 3, 5, 8])
@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.7, 0.95])
def test_expected_tokens_is_the_sum_over_prefix_lengths(alpha, gamma):
    probs = [alpha ** k * (1 - alpha) for k in range(gamma)] + [alpha ** gamma]
    assert sum(probs) == pytest.approx(1.0)
    want = sum((k + 1) * p for k, p in enumerate(probs))
    assert bench.expected_tokens(alpha, gamma) == pytest.approx(want, rel=1e-12)


def test_limits():
    assert bench.expected_tokens(0.0, 5) == 1.0          # only the bonus token
    assert bench.expected_tokens(1.0, 5) == 6.0          # every draft accepted
    assert bench.expected_tokens(0.999999, 5) == pytest.approx(6.0, rel=1e-5)


def test_per_token_accounting():
    r = bench.io_model(0.0, 4, draft_us=2.0, verify_us=10.0, dense_us=8.0, draft_bytes=100,
                       verify_bytes=1000, dense_bytes=900)
    # one token per round: 4 drafts + one verification per token
    assert r["tokens_per_round"] == 1.0
    assert r["kv_bytes_per_token"] == 1400 and r["attn_us_per_token"] == 18.0
    assert r["attn_speedup"] == pytest.approx(8.0 / 18.0, abs=1e-3)
    r = bench.io_model(1.0, 4, 2.0, 10.0, 8.0, 100, 1000, 900)
    assert r["tokens_per_round"] == 5.0 and r["kv_bytes_per_token"] == 280


@pytest.mark.parametrize("gamma", [1, 3, 5, 8])
def test_break_even_alpha_balances_the_round(gamma):
    draft_us, verify_us, dense_us = 3.0, 12.0, 10.0
    a = bench.break_even_alpha(gamma, draft_us, verify_us, dense_us)
    need = (gamma * draft_us + verify_us) / dense_us
    if need > gamma + 1:
        assert a is None
        return
    assert dense_us * bench.expected_tokens(a, gamma) == pytest.approx(gamma * draft_us + verify_us,
                                                                       rel=1e-3)
    r = bench.io_model(a, gamma, draft_us, verify_us, dense_us, 1, 1, 1)
    assert r["attn_speedup"] == pytest.approx(1.0, abs=2e-3)


def test_break_even_alpha_limits():
    assert bench.break_even_alpha(4, 1.0, 5.0, 20.0) == 0.0      # pays even with no acceptance
    assert bench.break_even_alpha(2, 10.0, 10.0, 5.0) is None    # 30 us > 3 tokens x 5 us
    # cheaper drafts (a smaller kept fraction) break even at a lower rate
    assert bench.break_even_alpha(5, 2.0, 20.0, 19.0) < bench.break_even_alpha(5, 6.0, 20.0, 19.0)


def test_bench_refuses_more_than_one_gpu():
    """The library has no multi-GPU path: the bench exits with a message
    (status 2) before it touches a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
