"""Host-side checks of bench.py: the one-GPU refusal, and the algorithmic
costs per launch that the roofline divides by.  Per token at the 380M-shape
layer (every tensor read or written once at its stored width) they are route
2,064 B, combine 16,400 B, chunk 24,672 B and 3.77 MFLOP, projections 10.5
MFLOP, with two choices of this design counted as they are: the dispatch
writes no gathered copy of x (the projection's loads gather the rows), so it
moves 292 B (index arrays and gates) instead of 6,296; and the chunk stage
also counts writing the final recurrent states, 40 slots x 4 heads x 128 x
256 x 4 B over 16,384 tokens = 1,280 B (and as much again for reading them
when the step is given entering states; the timed step starts from zeros).
The layer bounds (unfused design, every stage at its peak) are 96.4, 34.3,
60.6 and 34.3 M tokens/s for the 380M, 1.3B, 16-memory and long-context
shapes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stage_costs_per_token():
    import bench
    from mixture_memories_recurrence_amd import synth
    cfg = synth.CONFIGS["l380m"]
    NT = cfg.B * cfg.T
    c = bench.stage_costs(cfg)
    per_tok = {k: v["bytes"] / NT for k, v in c.items()}
    # weights are shared by the batch: a fraction of a byte per token at this size
    assert per_tok["route"] == pytest.approx(2064, abs=1)
    assert per_tok["dispatch"] == pytest.approx(292, abs=0.01)
    assert per_tok["combine"] == pytest.approx(16400, abs=0.01)
    assert per_tok["chunk"] == pytest.approx(24672 + 1280, abs=0.01)
    c_in = bench.stage_costs(cfg, state_in=True)
    assert c_in["chunk"]["bytes"] / NT == pytest.approx(24672 + 2560, abs=0.01)
    assert c["chunk"]["flops"] / NT / 1e6 == pytest.approx(3.77, abs=0.01)
    assert c["project"]["flops"] / NT / 1e6 == pytest.approx(10.5, abs=0.05)


@pytest.mark.parametrize("name,mtok", [("l380m", 96.4), ("l1b3", 34.3), ("m16", 60.6), ("long32k", 34.3)])
def test_layer_bound(name, mtok):
    import bench
    from mixture_memories_recurrence_amd import synth
    tok_s, us = bench.layer_bound(synth.CONFIGS[name])
    assert tok_s / 1e6 == pytest.approx(mtok, abs=0.05)
    if name == "l380m":  # route 2,064 B, dispatch 6,296 B, combine 16,400 B, chunk 24,672 B per token at 8 TB/s
        NT = 16384
        assert us["route"] == pytest.approx(2064 * NT / 8e12 * 1e6, rel=1e-9)
        assert us["dispatch"] == pytest.approx(6296 * NT / 8e12 * 1e6, rel=1e-9)
        assert us["combine"] == pytest.approx(16400 * NT / 8e12 * 1e6, rel=1e-9)
        assert us["chunk"] == pytest.approx(24672 * NT / 8e12 * 1e6, rel=1e-9)


def test_clock_warmup_runs_whole_groups_for_the_time_asked(monkeypatch):
    """bench.ramp runs the line's own step untimed, in groups of four with a
    device synchronisation after each group, until the time asked has passed;
    with no time asked it runs nothing."""
    import time
    import torch
    import bench
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    calls = []
    assert bench.ramp(lambda: calls.append(1), 0) == 0
    assert calls == []
    t0 = time.perf_counter()
    n = bench.ramp(lambda: calls.append(1), 0.05)
    assert time.perf_counter() - t0 >= 0.05
    assert n == len(calls) and n >= 4 and n % 4 == 0
