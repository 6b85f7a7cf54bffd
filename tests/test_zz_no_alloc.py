"""mom_dispatch_noalloc (the dispatch with the library's fixed scratch, for
callers that cannot allocate) against mom_dispatch through the C ABI: the
same outputs bit for bit, on two calls in a row, the second with a smaller
input.  The first call's count array (16 memories x 24 sequences x 64 counts
of 64 positions = 24576 counts) takes the separate scan launch, the second's
(4 x 3 x 11 = 132) the scan inside the scatter, and the second call finds the
first call's counts and offsets still in the array."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mixture_memories_recurrence_amd import mom, synth  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(B, T, M, K, H, seed):
    cfg = synth.LayerConfig(B, T, 64, H, 128, 256, M, K, "bf16")
    rng = np.random.default_rng(seed)
    NT = B * T
    idx = np.argsort(rng.random((NT, M)), axis=1)[:, :K].astype(np.int32)  # K distinct memories per token
    x = synth.round_bf16(rng.standard_normal((NT, cfg.D)).astype(np.float32))
    alpha = rng.uniform(0.9, 1.0, (NT, H, M + 1)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (NT, H, M + 1)).astype(np.float32)
    return cfg, dict(idx=torch.from_numpy(idx).cuda(), x=torch.from_numpy(x).to(torch.bfloat16).cuda(),
                     alpha=torch.from_numpy(alpha).cuda(), beta=torch.from_numpy(beta).cuda())


def _outputs(cfg):
    B, T, M, K, H = cfg.B, cfg.T, cfg.M, cfg.K, cfg.H
    NT, N = B * T, B * T * (K + 1)
    i32 = dict(dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    return dict(seg_off=torch.full(((M + 1) * B + 1,), -1, **i32), perm=torch.full((N,), -1, **i32),
                inv=torch.full((NT, K), -1, **i32), x_packed=torch.zeros(NT * K, cfg.D, dtype=torch.bfloat16,
                                                                        device="cuda"),
                alpha_p=torch.full((N, H), float("nan"), **f32), beta_p=torch.full((N, H), float("nan"), **f32))


def _run(cfg, inp, noalloc):
    d = mom.dims_of(cfg)
    o = _outputs(cfg)
    args = (d, inp["idx"], inp["x"], inp["alpha"], inp["beta"], o["seg_off"], o["perm"], o["inv"], o["x_packed"],
            o["alpha_p"], o["beta_p"])
    if noalloc:
        mom.mom_dispatch_noalloc(*args)
    else:
        ws = torch.empty(max(mom.mom_workspace_bytes(d, mom.WS_DISPATCH), 256), dtype=torch.uint8, device="cuda")
        mom.mom_dispatch(*args, ws)
    torch.cuda.synchronize()
    return o


def test_dispatch_noalloc_equals_dispatch_twice_shrinking():
    for B, T, M, K, H, seed in ((24, 4096, 16, 4, 4, 1), (3, 700, 4, 2, 2, 2)):
        cfg, inp = _case(B, T, M, K, H, seed)
        print("noalloc dispatch B=%d T=%d M=%d K=%d H=%d" % (B, T, M, K, H), flush=True)
        ref = _run(cfg, inp, noalloc=False)
        got = _run(cfg, inp, noalloc=True)
        for name in ref:
            assert torch.equal(got[name], ref[name]), name
        # the permutation is a bijection onto the rows
        assert torch.equal(torch.sort(got["perm"][: B * T * K].long()).values.cpu(),
                           torch.sort(ref["perm"][: B * T * K].long()).values.cpu())


def test_dispatch_noalloc_too_large_is_refused():
    cfg = synth.LayerConfig(64, 65 * 256, 64, 1, 128, 256, 16, 4, "bf16")
    d = mom.dims_of(cfg)
    fake = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(mom.MomError, match="fixed scratch"):
        mom.mom_dispatch_noalloc(d, fake, fake, fake, fake, fake, fake, fake, None, fake, fake)
