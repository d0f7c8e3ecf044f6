"""A decode step captured into a HIP graph (through torch.cuda.graph) and
replayed: kv_append + paged_decode (plan, partition and reduce kernels) and
paged_decode_noalloc launch nothing the capture cannot hold (no memset, copy or
host synchronisation).  Each replay, with eager work and a synchronisation
between replays, must equal the eager step bit for bit."""
import numpy as np
import pytest

import harness
import workloads as wl
from tests.oracle_ref import TOL, expected, parity_error

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("dt,Hq,Hkv,D,lens,P", [
    (wl.BF16, 32, 8, 128, [3000, 64, 1, 2049, 700], 256),     # matrix-core kernel, several partitions
    (wl.F16, 8, 8, 128, [900, 17, 300], 0),                   # vector kernel
    (wl.F32, 4, 4, 16, [25], 0),                              # the tiny shape
])
def test_captured_step_replays_equal_eager(dt, Hq, Hkv, D, lens, P, noalloc):
    w = wl.custom(91, lens, Hq, Hkv, D, dt)
    prep = harness.prepare(w, partition_tokens=P)
    out = torch.empty_like(prep.q)
    need = prep.pool.workspace_bytes(w.B, w.H_q, prep.max_len)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")

    def step():
        prep.append_step()
        if noalloc:
            prep.pool.decode_noalloc(prep.q, prep.tables, prep.lens, prep.max_len, w.scale, out=out)
        else:
            prep.decode(out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    out_dt = wl.BF16 if dt == wl.E4M3 else dt
    assert parity_error(harness.out_to_f64(eager), expected(w), out_dt) <= TOL[dt]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.empty_like(out)
    for i in range(4):
        out.fill_(float("nan"))                                   # eager work between replays
        prep.decode(out=other, workspace=ws)                      # an eager call on the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), eager.view(torch.uint8)), f"replay {i} differs"
        assert torch.equal(other.view(torch.uint8), eager.view(torch.uint8))
    del g
    prep.pool.close()
