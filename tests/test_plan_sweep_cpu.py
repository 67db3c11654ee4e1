"""The plan sweep's enumeration (rmsnorm_row_normalisation_amd/plan_sweep.py)
on the CPU: every candidate is a plan the library accepts, and the policy's
plan of every operation is among the candidates, so a sweep always times the
policy against every alternative it could have picked."""
import pytest
import torch

import rmsnorm_row_normalisation_amd as ks
from rmsnorm_row_normalisation_amd import plan_sweep

DTYPES = [torch.bfloat16, torch.float16, torch.float32]


@pytest.mark.parametrize("op", plan_sweep.OPS)
@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_candidates_cover_the_policy(op, dtype):
    for hidden in (64, 1000, 1024, 4096, 8192, 16384):
        cands = plan_sweep.candidates(op, dtype, hidden)
        if not cands:       # rows past the vector path: the policy takes the generic one
            assert ks.get_plan(op, dtype, hidden, 64).path != 0, (op, dtype, hidden)
            continue
        names = {plan_sweep.plan_name(p) for p in cands}
        assert len(names) == len(cands)
        for p in cands:
            assert plan_sweep.accepted(op, dtype, hidden, p)
        for rows in (1, 64, 2048, 32768):
            pol = ks.get_plan(op, dtype, hidden, rows, compute_units=256)
            if pol.path != 0:
                continue
            assert plan_sweep.plan_name(pol) in names, (op, dtype, hidden, rows, pol.as_dict())


def test_rejects_and_names():
    bad = ks.Plan(path=0, threads_per_row=64, vectors_per_thread=8, elems_per_access=8, rows_per_block=4,
                  block_threads=256, load_nt=1, store_nt=1, weight_lds=1)
    assert not plan_sweep.accepted("rms_norm_backward", torch.bfloat16, 4096, bad)
    assert plan_sweep.accepted("rms_norm", torch.bfloat16, 4096, bad)
    assert plan_sweep.plan_name(bad) == "64x8/256 nt11 lds1"
    assert plan_sweep.candidates("rms_norm", torch.bfloat16, 4095) == []     # odd row bytes: no vector plan
