"""The C ABI without a GPU: the library loads, exports every function the header
declares, sizes its workspace, and rejects bad arguments before any launch."""
import ctypes
import dataclasses
import os
import re
import subprocess

import pytest

torch = pytest.importorskip("torch")
from mixture_memories_recurrence_amd import mom  # noqa: E402
from mixture_memories_recurrence_amd.synth import CONFIGS  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mom.h")

needs_lib = pytest.mark.skipif(not os.path.exists(mom.LIB_PATH), reason="libmom.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:mom_status|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(mom.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", mom.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for f in declared_functions():
        assert f in exported, f
    L = mom.lib()
    for f in declared_functions():
        assert getattr(L, f) is not None


def _dims(**kw):
    d = mom.dims_of(CONFIGS["l380m"])
    for k, v in kw.items():
        setattr(d, k, v)
    return d


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: every call below fails validation
ODD = ctypes.c_void_p(0x10004)


@needs_lib
@pytest.mark.parametrize("field,value,status", [
    ("dk", 96, -3), ("dv", 32, -3), ("dv", 192, -3), ("dv", 1152, -3), ("chunk", 32, -3), ("D", 1000, -3),
    ("M", 65, -3), ("topk", 9, -3), ("topk", 0, -2), ("B", 0, -2), ("T", -1, -2), ("dtype", 7, -3), ("topk", 5, -2)])
def test_bad_dims_are_rejected(field, value, status):
    d = _dims(**{field: value})
    if field == "topk" and value == 9:
        d.M = 16          # topk <= M, but above the supported 8
    L = mom.lib()
    assert L.mom_route(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, None) == status
    assert L.mom_workspace_bytes(ctypes.byref(d), 0) == 0


@needs_lib
def test_chunk_lengths_per_storage():
    """Float32 storage takes chunks of 16, 32 or 64 rows; half precision (the
    matrix-core path) only 64; other lengths are refused."""
    L = mom.lib()
    for dtype, chunk, ok in [(mom.DTYPE_F32, 16, True), (mom.DTYPE_F32, 32, True), (mom.DTYPE_F32, 64, True),
                             (mom.DTYPE_F32, 48, False), (mom.DTYPE_F32, 128, False), (mom.DTYPE_F32, 8, False),
                             (mom.DTYPE_BF16, 16, False), (mom.DTYPE_BF16, 32, False), (mom.DTYPE_BF16, 64, True)]:
        d = _dims(dtype=dtype, chunk=chunk)
        assert (L.mom_workspace_bytes(ctypes.byref(d), 0) > 0) == ok, (dtype, chunk)
        if not ok:
            assert L.mom_route(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, None) == -3


@needs_lib
def test_wide_values_only_outside_decode():
    """A value width that is a multiple of 128 above 256 passes the shared
    checks (the chunk recurrence takes it) but gdn_decode_step rejects it."""
    d = _dims(dv=768)
    L = mom.lib()
    assert L.mom_workspace_bytes(ctypes.byref(d), 0) > 0
    assert L.gdn_decode_step(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -3


@needs_lib
def test_null_and_alignment_are_rejected():
    L = mom.lib()
    d = _dims()
    assert L.mom_route(None, FAKE, FAKE, None, FAKE, FAKE, None) == -1
    assert L.mom_route(ctypes.byref(d), None, FAKE, None, FAKE, FAKE, None) == -1
    assert L.mom_route(ctypes.byref(d), ODD, FAKE, None, FAKE, FAKE, None) == -4
    assert L.mom_combine(ctypes.byref(d), 4, None, FAKE, FAKE, FAKE, None, None) == -1
    assert L.mom_combine(ctypes.byref(d), -1, None, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert L.mom_project(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ODD, None) == -4
    assert L.gdn_decode_step(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == -1
    # chunk: n_state smaller than the segments with identity slots
    assert L.gdn_chunk_fwd(ctypes.byref(d), 10, 10, 10, 3, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                           FAKE, FAKE, None, 0, None) == -2


@needs_lib
def test_dispatch_workspace_is_checked():
    L = mom.lib()
    d = _dims()
    need = L.mom_workspace_bytes(ctypes.byref(d), 0)
    n = d.M * d.B * -(-d.T // 64)  # counts of every 64 positions, then their scan
    assert need >= (-(-n // 64) * 64 + n) * 4 and need % 256 == 0
    args = [FAKE] * 10
    assert L.mom_dispatch(ctypes.byref(d), *args, None, need, None) == -5
    assert L.mom_dispatch(ctypes.byref(d), *args, FAKE, need - 1, None) == -5


@needs_lib
def test_status_strings():
    L = mom.lib()
    for s in range(-6, 1):
        assert L.mom_status_string(s).decode()
    assert L.mom_status_string(-99).decode() == "unknown status"


@needs_lib
def test_chunk_workspace_sizes():
    L = mom.lib()
    d = _dims()
    n_seg, n_rows = (d.M + 1) * d.B, d.B * d.T * (d.topk + 1)
    need = L.gdn_chunk_workspace_bytes(ctypes.byref(d), n_seg, n_rows)
    n_chunks = n_rows // 64 + n_seg
    assert need >= n_chunks * d.H * (64 * 64 * 2 * 2 + 64 * 4) and need % 256 == 0
    assert L.mom_workspace_bytes(ctypes.byref(d), 1) == need
    assert L.gdn_chunk_workspace_bytes(ctypes.byref(d), -1, n_rows) == 0
    # missing workspace is refused before any launch
    assert L.gdn_chunk_fwd(ctypes.byref(d), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, FAKE, FAKE, FAKE,
                           FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == -5
    d32 = _dims(dtype=0)
    assert L.gdn_chunk_workspace_bytes(ctypes.byref(d32), n_seg, n_rows) == 0


@needs_lib
def test_decode_combined_checks():
    """The decode step with the combine folded in needs the router weights and
    takes the value widths gdn_decode_step takes."""
    L = mom.lib()
    d = _dims()
    for f in (L.gdn_decode_step_combined, L.gla_decode_step_combined):
        assert f(ctypes.byref(d), 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
        assert f(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -1
        assert f(ctypes.byref(_dims(dv=768)), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 None) == -3
        assert f(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 0


@needs_lib
def test_route_count_checks():
    """The one-pass route and histogram needs the dispatch workspace (for one
    position per sequence and for whole sequences), and the counted dispatch
    validates like mom_dispatch / mom_dispatch_part, all before any launch."""
    L = mom.lib()
    for d in (_dims(T=1), _dims()):
        need = L.mom_workspace_bytes(ctypes.byref(d), 0)
        assert L.mom_route_count(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, need - 1, None) == -5
        assert L.mom_route_count(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == -5
        assert L.mom_route_count(ctypes.byref(d), None, FAKE, None, FAKE, FAKE, FAKE, need, None) == -1
        args = [FAKE] * 10
        assert L.mom_dispatch_counted(ctypes.byref(d), *args, None, need, None) == -5
        assert L.mom_dispatch_counted(ctypes.byref(d), *args, FAKE, need - 1, None) == -5
        assert L.mom_dispatch_counted_part(ctypes.byref(d), *args, FAKE, need, 3, None) == -2
        assert L.mom_dispatch_counted_part(ctypes.byref(d), *args, None, need, 2, None) == -5
    assert L.mom_route_count(ctypes.byref(_dims(topk=0)), FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None) == -2


@needs_lib
def test_chunk_bwd_checks():
    """The gradient entry points: workspace size (half storage: forward factors, X
    (half), and two half states per chunk and head; float32: the state entering
    every chunk, checkpoints every 8 rows per block, and the column blocks'
    partial sums), and the usual refusals, all before any launch."""
    L = mom.lib()
    d = _dims()
    n_seg, n_rows = (d.M + 1) * d.B, d.B * d.T * (d.topk + 1)
    need = L.gdn_chunk_bwd_workspace_bytes(ctypes.byref(d), n_seg, n_rows)
    n_chunks = n_rows // 64 + n_seg
    per = 64 * 64 * 2 * 2 + 64 * 4 * 2 + 64 * 64 * 2 + 2 * d.dk * d.dv * 2
    assert need >= n_chunks * d.H * per and need % 256 == 0
    assert need > L.gdn_chunk_workspace_bytes(ctypes.byref(d), n_seg, n_rows)
    args = [FAKE] * 5 + [None, FAKE, None] + [FAKE] * 6  # q..beta, state_in, d_o, dstate_out, outputs
    for f in (L.gdn_chunk_bwd, L.gla_chunk_bwd, L.gdn_chunk_bwd_saved, L.gla_chunk_bwd_saved):
        # no workspace, a short one, a missing output, float32 storage
        assert f(ctypes.byref(d), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *args, None, 0, None) == -5
        assert f(ctypes.byref(d), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *args, FAKE, need - 1,
                 None) == -5
        bad = list(args)
        bad[8] = None  # dq
        assert f(ctypes.byref(d), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *bad, FAKE, need, None) == -1
        d32 = _dims(dtype=0)
        need32 = L.gdn_chunk_bwd_workspace_bytes(ctypes.byref(d32), n_seg, n_rows)
        assert f(ctypes.byref(d32), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *args, FAKE, need32 - 1,
                 None) == -5
    a256 = lambda b: (b + 255) // 256 * 256
    nb = d.dv // 64
    need32 = a256(n_chunks * d.H * d.dk * d.dv * 4) + a256(n_seg * d.H * nb * 8 * d.dk * 64 * 4) + \
        2 * a256(nb * n_rows * d.H * d.dk * 4) + 2 * a256(nb * n_rows * d.H * 4)
    assert L.gdn_chunk_bwd_workspace_bytes(ctypes.byref(_dims(dtype=0)), n_seg, n_rows) == need32
    fargs = [FAKE] * 5 + [None, FAKE, FAKE]  # q..beta, state_in, state_out, o
    for f in (L.gdn_chunk_fwd_train, L.gla_chunk_fwd_train):
        # the training forward needs the gradient workspace, not the forward's
        small = L.gdn_chunk_workspace_bytes(ctypes.byref(d), n_seg, n_rows)
        assert f(ctypes.byref(d), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *fargs, None, 0, None) == -5
        assert f(ctypes.byref(d), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *fargs, FAKE, small,
                 None) == -5
        for i in (6, 7):  # state_out, o
            bad = list(fargs)
            bad[i] = None
            assert f(ctypes.byref(d), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *bad, FAKE, need,
                     None) == -1
        assert f(ctypes.byref(_dims(dtype=0)), n_seg, n_rows, d.B * d.T, n_seg, FAKE, None, None, *fargs, FAKE,
                 need32 - 1, None) == -5


@needs_lib
def test_dispatch_noalloc_checks_before_any_launch():
    """The allocation-free dispatch validates like mom_dispatch and rejects
    sizes past its fixed scratch (M*B*ceil(T/64) <= 32768 counts, and as many
    scanned offsets) with
    MOM_ERR_TOO_LARGE, all before any HIP call (so without a GPU)."""
    L = mom.lib()
    f = lambda d, *p: L.mom_dispatch_noalloc(ctypes.byref(d), *p, None)
    ok = [FAKE] * 10
    assert L.mom_dispatch_noalloc(None, *ok, None) == -1
    assert f(_dims(), None, *ok[1:]) == -1                  # idx
    assert f(_dims(), FAKE, None, FAKE, *ok[3:]) == -1      # beta
    assert f(_dims(), FAKE, FAKE, FAKE, FAKE, ODD, *ok[5:]) == -4   # seg_off misaligned
    assert f(_dims(topk=0), *ok) == -2
    # 16 memories x 32 sequences x 65 counts of 64 positions = 33280 counts > 32768
    big = _dims(M=16, topk=4, B=32, T=65 * 64)
    assert f(big, *ok) == -7
    assert L.mom_status_string(-7).decode().startswith("sizes exceed")
    # exactly at the limit passes the size check (then needs a GPU, not called here)
    assert L.mom_workspace_bytes(ctypes.byref(_dims(M=16, topk=4, B=32, T=64 * 64)), 0) == 65536 * 4


@needs_lib
def test_chunk_workspace_reserves_the_scan_only_for_few_long_segments():
    """gdn_chunk_fwd's workspace: the per-chunk factors (T and P half, the
    decays float32, per (chunk, head)), plus the long-segment scan's groups,
    maps and entering states only when the walk would run at most 8 blocks
    over long segments (one long sequence with 4 heads, two with 2), not for
    any call the layer makes at its configurations."""
    L = mom.lib()
    a256 = lambda b: (b + 255) // 256 * 256

    def factors(n_seg, n_rows, H):
        nch = n_rows // 64 + n_seg
        return 2 * a256(nch * H * 64 * 64 * 2) + a256(nch * H * 2 * 64 * 4)

    for name, n_seg, scan, H in (("l380m", 40, False, None), ("l380m", 8, False, None), ("long32k", 5, False, None),
                                 ("long32k", 1, False, None), ("long32k", 1, True, 4), ("long32k", 2, True, 2)):
        c = CONFIGS[name] if H is None else dataclasses.replace(CONFIGS[name], H=H)
        d = mom.dims_of(c)
        N = c.B * c.T * (c.K + 1)
        got = L.gdn_chunk_workspace_bytes(ctypes.byref(d), n_seg, N)
        if scan:
            n_groups = N // (8 * 64) + n_seg
            extra = a256((n_groups + 1) * 4) * 2 + a256((n_seg + 1) * 4) + \
                a256(n_groups * c.H * c.dk * (c.dv + c.dk) * 4) + a256(n_groups * c.H * c.dk * c.dv * 4)
            assert got == factors(n_seg, N, c.H) + extra, (name, n_seg)
        else:
            assert got == factors(n_seg, N, c.H), (name, n_seg)
