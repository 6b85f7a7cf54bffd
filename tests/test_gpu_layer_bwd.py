"""GPU parity of the layer's gradients (combine, recurrence, dispatch gathers,
router weights with the top-k choice held fixed) against the fp64 checker's
composition (oracle.layer_bwd), through the C ABI.  Tolerance as for the
recurrence's gradients (tests/test_gpu_bwd.py): rel-L2 <= 5e-3 and max-abs <=
5e-3 * max|reference| per gradient tensor."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
from mixture_memories_recurrence_amd import mom, synth  # noqa: E402
from oracle import oracle  # noqa: E402
from parity import log, to_gpu  # noqa: E402
from test_gpu_bwd import assert_grad  # noqa: E402

pytestmark = pytest.mark.gpu


def small(name, B, T):
    import dataclasses
    return dataclasses.replace(synth.CONFIGS[name], B=B, T=T)


@pytest.mark.parametrize("name,B,T,rule", [("l380m", 2, 300, "gdn"), ("l380m", 2, 300, "gla"), ("m16", 2, 200, "gdn"),
                                           ("l1b3", 1, 257, "gdn")])
def test_layer_bwd_reduced(name, B, T, rule):
    """Whole-layer gradients at reduced length (ragged last chunks), from
    non-zero entering states, with final-state gradients."""
    cfg = small(name, B, T)
    inp = synth.make_layer_inputs(cfg, seed=21)
    NT = B * T
    rng = np.random.default_rng(22)
    dout = rng.standard_normal((NT, cfg.H, cfg.dv)).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, cfg.M + 1, cfg.H, cfg.dk, cfg.dv))).astype(np.float32)
    dS = rng.standard_normal(S0.shape).astype(np.float32)
    layer = mom.MomLayer(cfg, inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"], rule=rule)
    x = torch.from_numpy(inp["x"]).to(torch.bfloat16).cuda()
    log("layer_bwd", name, B, T, rule)
    _, _, b = layer.forward(x, to_gpu(inp["alpha"]), to_gpu(inp["beta"]), state_in=to_gpu(S0))
    g = layer.backward(x, to_gpu(dout), b, dstate_out=to_gpu(dS), state_in=to_gpu(S0))
    torch.cuda.synchronize()
    dims = (B, T, cfg.D, cfg.H, cfg.dk, cfg.dv, cfg.M, cfg.K)
    ref = oracle.layer_bwd(dims, inp["x"], inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"], inp["alpha"],
                           inp["beta"], dout, state0=S0, dstate=dS, rule=rule)
    assert np.array_equal(b["idx"].cpu().numpy(), ref["idx"])
    f = lambda t: t.float().cpu().numpy()
    for name_g, rn in (("d_alpha", "d_alpha"), ("d_beta", "d_beta"), ("dq", "dq"), ("dk", "dk_rows"),
                       ("dv", "dv_rows"), ("dx_router", "dx_router"), ("dw_r", "dw_r"), ("dbias", "dbias"),
                       ("dstate_in", "dstate0")):
        assert_grad(name_g, f(g[name_g]), ref[rn])


@pytest.mark.parametrize("rule,train", [("gdn", False), ("gla", False), ("gdn", True)])
def test_layer_bwd_tiny_f32(rule, train):
    """The float32 layer's gradients (the row-by-row reverse sweep for the
    recurrence), from non-zero entering states with final-state gradients,
    after a plain forward and after a training forward, to the float32
    tolerance (1e-5, relative to each tensor's largest value for max-abs)."""
    from test_gpu_bwd import GRAD_REL_F32
    cfg = synth.CONFIGS["tiny_f32"]
    B, T = cfg.B, cfg.T
    inp = synth.make_layer_inputs(cfg, seed=25)
    NT = B * T
    rng = np.random.default_rng(26)
    dout = rng.standard_normal((NT, cfg.H, cfg.dv)).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, cfg.M + 1, cfg.H, cfg.dk, cfg.dv))).astype(np.float32)
    dS = rng.standard_normal(S0.shape).astype(np.float32)
    layer = mom.MomLayer(cfg, inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"], rule=rule)
    x = to_gpu(inp["x"])
    log("layer_bwd f32", rule, "train" if train else "")
    _, _, b = layer.forward(x, to_gpu(inp["alpha"]), to_gpu(inp["beta"]), state_in=to_gpu(S0), train=train)
    g = layer.backward(x, to_gpu(dout), b, dstate_out=to_gpu(dS), state_in=to_gpu(S0))
    torch.cuda.synchronize()
    dims = (B, T, cfg.D, cfg.H, cfg.dk, cfg.dv, cfg.M, cfg.K)
    ref = oracle.layer_bwd(dims, inp["x"], inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"], inp["alpha"],
                           inp["beta"], dout, state0=S0, dstate=dS, rule=rule)
    assert np.array_equal(b["idx"].cpu().numpy(), ref["idx"])
    f = lambda t: t.float().cpu().numpy()
    for name_g, rn in (("d_alpha", "d_alpha"), ("d_beta", "d_beta"), ("dq", "dq"), ("dk", "dk_rows"),
                       ("dv", "dv_rows"), ("dx_router", "dx_router"), ("dw_r", "dw_r"), ("dbias", "dbias"),
                       ("dstate_in", "dstate0")):
        assert_grad(name_g, f(g[name_g]), ref[rn], GRAD_REL_F32)


def test_combine_route_dispatch_bwd_full_size():
    """At the 380M shape (8 x 2048 tokens), the three gather / router gradient
    entry points on the GPU's own forward results, against the checker's
    functions on the same values."""
    cfg = synth.CONFIGS["l380m"]
    inp = synth.make_layer_inputs(cfg, seed=23)
    layer = mom.MomLayer(cfg, inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"])
    x = torch.from_numpy(inp["x"]).to(torch.bfloat16).cuda()
    log("combine / route / dispatch bwd, full size")
    _, _, b = layer.forward(x, to_gpu(inp["alpha"]), to_gpu(inp["beta"]))
    NT, N, NR, H = b["NT"], b["N"], b["NR"], cfg.H
    rng = np.random.default_rng(24)
    dout = rng.standard_normal((NT, H, cfg.dv)).astype(np.float32)
    d = b["dims"]
    d_o = torch.full((N, H, cfg.dv), float("nan"), device="cuda")
    dw = torch.empty(NT, cfg.K, device="cuda")
    mom.mom_combine_bwd(d, NT, b["inv"], b["w"], b["o"], to_gpu(dout), d_o, d_o[NR:], dw)
    dap = rng.standard_normal((N, H)).astype(np.float32)
    dbp = rng.standard_normal((N, H)).astype(np.float32)
    dqr = rng.standard_normal((N, H, cfg.dk)).astype(np.float32)
    da = torch.empty(NT, H, cfg.M + 1, device="cuda")
    db = torch.empty_like(da)
    dq = torch.empty(NT, H, cfg.dk, device="cuda")
    mom.mom_dispatch_bwd(d, b["idx"], b["inv"], to_gpu(dap), to_gpu(dbp), to_gpu(dqr), da, db, dq)
    dx = torch.empty(NT, cfg.D, device="cuda")
    dwr = torch.empty(cfg.M, cfg.D, device="cuda")
    dbias = torch.empty(cfg.M, device="cuda")
    ws = torch.empty(mom.mom_workspace_bytes(d, mom.WS_ROUTE_BWD), dtype=torch.uint8, device="cuda")
    mom.mom_route_bwd(d, x, layer.w_r, b["idx"], b["w"], dw, dx, dwr, dbias, ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    idx, inv, w, o = b["idx"].cpu().numpy(), b["inv"].cpu().numpy(), f(b["w"]), f(b["o"])
    d_r, d_s, dw_ref = oracle.combine_bwd(inv, w, o, dout, n_rows=N)
    d_r[NR:] = d_s
    assert_grad("combine d_o", f(d_o), d_r)
    assert_grad("combine dw", f(dw), dw_ref)
    da_ref, db_ref, dq_ref = oracle.dispatch_bwd(idx, inv, cfg.M, dap, dbp, dqr)
    assert np.array_equal(f(da), da_ref.astype(np.float32)) and np.array_equal(f(db), db_ref.astype(np.float32))
    assert_grad("dispatch dq", f(dq), dq_ref)
    xr = f(x)
    dx_ref, dwr_ref, db_ref2 = oracle.route_bwd(xr, f(layer.w_r), idx, w, f(dw))
    assert_grad("router dx", f(dx), dx_ref)
    assert_grad("router dw_r", f(dwr), dwr_ref)
    assert_grad("router dbias", f(dbias), db_ref2)


@pytest.mark.parametrize("M,K,D,NT", [(64, 8, 192, 700), (5, 2, 320, 513), (16, 4, 1024, 300)])
def test_route_bwd_shapes(M, K, D, NT):
    """mom_route_bwd alone over random selections and upstream gradients: many
    memories (sums kept in LDS), column counts that are not a multiple of 256,
    and token counts that leave a partial tile."""
    rng = np.random.default_rng(M + K + D)
    x = rng.standard_normal((NT, D)).astype(np.float32)
    w_r = (rng.standard_normal((M, D)) / np.sqrt(D)).astype(np.float32)
    idx = np.stack([rng.permutation(M)[:K] for _ in range(NT)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (NT, K)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    dw = rng.standard_normal((NT, K)).astype(np.float32)
    cfg = synth.LayerConfig(1, NT, D, 2, 64, 64, M, K, "bf16")
    d = mom.dims_of(cfg)
    xb, wb = to_gpu(x, torch.bfloat16), to_gpu(w_r, torch.bfloat16)
    dx = torch.empty(NT, D, device="cuda")
    dwr = torch.empty(M, D, device="cuda")
    db = torch.empty(M, device="cuda")
    ws = torch.empty(mom.mom_workspace_bytes(d, mom.WS_ROUTE_BWD), dtype=torch.uint8, device="cuda")
    log("route_bwd", M, K, D, NT)
    mom.mom_route_bwd(d, xb, wb, to_gpu(idx), to_gpu(w), to_gpu(dw), dx, dwr, db, ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    dx_ref, dwr_ref, db_ref = oracle.route_bwd(f(xb), f(wb), idx, w, dw)
    assert_grad("router dx", f(dx), dx_ref)
    assert_grad("router dw_r", f(dwr), dwr_ref)
    assert_grad("router dbias", f(db), db_ref)


@pytest.mark.parametrize("name,B,T,rule,overlap", [("l380m", 8, 2048, "gdn", True), ("l380m", 8, 2048, "gdn", False),
                                                   ("l380m", 2, 300, "gla", True), ("m16", 2, 200, "gdn", True)])
def test_layer_train_forward_saved_backward(name, B, T, rule, overlap):
    """A training step (forward with train=True, then backward reading what it
    kept) gives the plain forward's outputs and the recompute backward's
    gradients bit for bit, on one stream and on two; the next backward after it
    recomputes and agrees too."""
    cfg = small(name, B, T)
    inp = synth.make_layer_inputs(cfg, seed=23)
    NT = B * T
    rng = np.random.default_rng(24)
    dout = to_gpu(rng.standard_normal((NT, cfg.H, cfg.dv)).astype(np.float32))
    S0 = to_gpu((0.1 * rng.standard_normal((B, cfg.M + 1, cfg.H, cfg.dk, cfg.dv))).astype(np.float32))
    dS = to_gpu(rng.standard_normal(tuple(S0.shape)).astype(np.float32))
    layer = mom.MomLayer(cfg, inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"], rule=rule)
    x = torch.from_numpy(inp["x"]).to(torch.bfloat16).cuda()
    a, c = to_gpu(inp["alpha"]), to_gpu(inp["beta"])
    log("layer train/saved", name, B, T, rule, "overlap" if overlap else "serial")
    res = []
    for train, backwards in ((False, 1), (True, 2)):
        st = torch.empty_like(S0)
        out, _, b = layer.forward(x, a, c, state_in=S0, state_out=st, overlap=overlap, train=train)
        r = dict(out=out.clone(), st=st)
        # the training forward left its factors for the backward (two workspaces when on two streams)
        assert b["saved"] == (("split" if overlap else "all") if train else None)
        for i in range(backwards):
            g = layer.backward(x, dout, b, dstate_out=dS, state_in=S0)
            r.update({"%s%d" % (k, i): v.clone() for k, v in g.items()})
        torch.cuda.synchronize()
        res.append(r)
    ref, got = res
    for k in got:
        base = k[:-1] + "0" if k[-1] == "1" else k
        assert torch.equal(got[k], ref[base]), k
