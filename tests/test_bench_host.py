"""Host-side checks of bench.py: the one-GPU refusal, and the algorithmic
costs per launch that the roofline divides by.  Per token at the 380M-shape
layer (every tensor read or written once at its stored width) they are route
2,064 B, combine 16,400 B, chunk 24,672 B and 3.77 MFLOP, projections 10.5
MFLOP, with two choices of this design counted as they are: the dispatch
writes no gathered copy of x (the projection's loads gather the rows), so it
moves 292 B (index arrays and gates) instead of 6,296; and the chunk stage
also counts reading and writing the recurrent states, 2 x 40 slots x 4 heads
x 128 x 256 x 4 B over 16,384 tokens = 2,560 B."""
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
    assert per_tok["chunk"] == pytest.approx(24672 + 2560, abs=0.01)
    assert c["chunk"]["flops"] / NT / 1e6 == pytest.approx(3.77, abs=0.01)
    assert c["project"]["flops"] / NT / 1e6 == pytest.approx(10.5, abs=0.05)
