"""dlrm_forward_noalloc (the workspace in the library's static device array)
against dlrm_forward with a caller-owned workspace, through the C ABI.

Both run the same kernels on the same inputs, so the bar is bit-identical
outputs; the oracle checks the no-allocation result too (1e-5 absolute on the
sigmoid outputs).  Two calls in a row share the array, the second with a
smaller batch; a request beyond the array is refused before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import dlrm_embedding_interaction_amd as dl
import dlrm_inputs as di
import oracle

pytestmark = pytest.mark.gpu


def _noalloc(model, dense, indices, offsets, out):
    L = dl.load()
    b, dp, ip, nn_, op, ib = model.forward_args(dense, indices, offsets)
    return L.dlrm_forward_noalloc(ctypes.byref(model._desc), b, dp, ip, nn_, op, ib, out.data_ptr(),
                                  dl._stream(out.device))


def _head(inp, B):
    """The first B samples of a one-index-per-bag workload, on the GPU."""
    return ([i[:B].contiguous() for i in inp.indices], [o[:B].contiguous() for o in inp.offsets],
            inp.dense[:B].contiguous())


@pytest.mark.parametrize("name", ["page4", "manytable"])
@pytest.mark.parametrize("pack", [False, True])
@pytest.mark.parametrize("itype", [torch.int64, torch.int32])
def test_noalloc_matches_forward_twice_second_smaller(name, pack, itype, orc):
    """pack=False takes the layered path, whose workspace is the static array;
    pack=True the single launch (page4) or, at 32 tables, the path choice of
    dlrm_forward.  Batch 2048, then 700 on the same array."""
    w = di.get(name)
    cpu = di.make_inputs(w)
    g = cpu.to("cuda")
    m = dl.Model.from_inputs(g, pack=pack)
    for B in (2048, 700):
        idx, off, dense = _head(g, B)
        idx = [i.to(itype) for i in idx]
        off = [o.to(itype) for o in off]
        ref = m.forward(dense, idx, off, path="auto").clone()
        out = torch.full((B,), -1.0, device="cuda")
        rc = _noalloc(m, dense, idx, off, out)
        assert rc == dl.DLRM_OK, dl.load().dlrm_status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, pack, B)
        want = oracle.forward_inputs(di.subset(cpu, torch.arange(B)), oracle=orc)
        assert np.abs(out.cpu().double().numpy() - want).max() <= 1e-5


def test_noalloc_refuses_a_workspace_beyond_its_array():
    L = dl.load()
    w = di.custom("noalloc_big", 40000, 13, 3, 500, 64, 1, (13, 64), hidden_top=(1024,), cfg_id=26)
    g = di.make_inputs(w, device="cuda")
    m = dl.Model.from_inputs(g, pack=False)
    assert m.workspace_bytes(w.batch) > L.dlrm_forward_noalloc_max_bytes()
    out = torch.full((w.batch,), -1.0, device="cuda")
    assert _noalloc(m, g.dense, g.indices, g.offsets, out) == dl.DLRM_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == -1.0)
    # a batch that fits the array runs and matches dlrm_forward
    B = 1000
    idx, off, dense = _head(g, B)
    ref = m.forward(dense, idx, off).clone()
    small = torch.full((B,), -1.0, device="cuda")
    assert _noalloc(m, dense, idx, off, small) == dl.DLRM_OK
    torch.cuda.synchronize()
    assert torch.equal(small, ref)
