"""gla_fwd_noalloc (the forward that allocates nothing, its workspace a fixed
device array in the library) against gla_fwd: identical outputs, bit for bit,
on two calls in a row whose second problem is smaller, both sequence-split so
that the scratch is really used; and both within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from ssm_recurrence_amd import binding as gb
from ssm_recurrence_amd.inputs import small_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate,dtype", [("vector", torch.bfloat16), ("scalar", torch.float32)])
def test_noalloc_forward_matches_gla_fwd(gate, dtype):
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    # (T, H, split, document lengths): the second call smaller than the first
    for T, H, split, lens in ((2048, 4, 8, [700, 1348]), (700, 2, 3, [100, 600])):
        case = small_case(seed=T + H, B=2, T=T, H=H, d=128, gate=gate, dtype=dtype, lengths=lens)
        prob = gb.problem_of(case.q, case.v, case.g, gate, 64, split)
        need = gb.workspace_size(prob, False)
        assert 0 < need <= gb.load().gla_fwd_noalloc_max_scratch()
        c = case.to("cuda")
        print("noalloc", gate, dtype, "T", T, "H", H, "split", split, "scratch bytes", need, flush=True)
        o1, h1 = gb.fwd(c.q, c.k, c.v, c.g, c.h0, c.segment_ids, gate=gate, split=split)
        o2, h2 = gb.fwd_noalloc(c.q, c.k, c.v, c.g, c.h0, c.segment_ids, gate=gate, split=split)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), "o differs from gla_fwd"
        assert torch.equal(h1, h2), "hT differs from gla_fwd"
        ro, rh = oracle.fwd(case.q, case.k, case.v, case.g, case.h0, case.segment_ids, gate=gate)
        for got, ref in ((o2, ro), (h2, rh)):
            a = got.float().cpu().numpy().astype(np.float64)
            assert np.all(np.isfinite(a))
            assert np.max(np.abs(a - ref)) / np.max(np.abs(ref)) <= tol
