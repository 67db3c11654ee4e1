"""ks_softmax_noalloc (softmax for callers that cannot allocate: its split
plans keep their per-chunk statistics in the library's static device array)
against ks_softmax_ws (the same contract with a caller workspace), through the
C ABI on cuda:0.

Both calls run the same plan and kernels, so their outputs must be identical
bit for bit; each is also held to the softmax bar against the CPU oracle
(within 1 ulp of bf16/fp16, >= 99.9% bit-identical on large cases).  Two calls
in a row share the array: the second, smaller call leaves statistics of the
first beyond its own range, which it must not read.
"""
import pytest
import torch

import oracle
import rmsnorm_row_normalisation_amd as ks
import workloads
from compare import check_normalised
from gpu_cases import require_gpu, say
from rmsnorm_row_normalisation_amd import binding as b

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _pair(x_cpu: torch.Tensor, stream: torch.cuda.Stream):
    """(ks_softmax_noalloc output, ks_softmax_ws output) for one batch, on one stream."""
    rows, hidden = x_cpu.shape
    code = ks.KS_DTYPE[x_cpu.dtype]
    x = x_cpu.cuda()
    y_static = torch.full_like(x, float("nan"))
    y_ws = torch.full_like(x, float("nan"))
    need = b.ks_softmax_workspace_size(rows, hidden, code)
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    st = b.ks_softmax_noalloc(y_static.data_ptr(), x.data_ptr(), rows, hidden, code, stream.cuda_stream)
    assert st == b.KS_SUCCESS, b.lib().ks_status_string(st)
    st = b.ks_softmax_ws(y_ws.data_ptr(), x.data_ptr(), rows, hidden, code, ws.data_ptr(), need, stream.cuda_stream)
    assert st == b.KS_SUCCESS, b.lib().ks_status_string(st)
    stream.synchronize()
    return y_static.cpu(), y_ws.cpu(), need


@pytest.mark.parametrize("first, second", [
    (((8, 65536), "float16", 31), ((2, 32768), "bfloat16", 32)),     # split, then a smaller split
    (((4, 128256), "float32", 33), ((1, 8192), "float32", 34)),      # vocabulary rows, then one row
    (((64, 131072), "bfloat16", 35), ((16, 1024), "bfloat16", 36)),  # split, then a one-pass plan
])
def test_noalloc_matches_workspace_entry(first, second):
    stream = torch.cuda.Stream()
    needs = []
    for shape, dtype, seed in (first, second):
        x = workloads.random_case(shape, dtype, seed)["x"]
        say("softmax_noalloc", shape, dtype, "seed", seed)
        got, want, need = _pair(x, stream)
        needs.append(need)
        assert need <= b.KS_NOALLOC_SCRATCH_BYTES
        assert torch.equal(got.view(torch.int16 if got.element_size() == 2 else torch.int32),
                           want.view(torch.int16 if want.element_size() == 2 else torch.int32))
        check_normalised(got, oracle.softmax(x), 0.999 if x.numel() >= 20000 else None)
    assert needs[0] > 0 and needs[1] < needs[0]



def test_noalloc_under_graph_capture():
    """The use it exists for: captured into a HIP graph (no allocation inside the
    capture), replayed several times with eager calls and synchronisations in
    between; every replay gives the eager result bit for bit."""
    x = workloads.random_case((4, 65536), "float16", 37)["x"].cuda()
    rows, hidden = x.shape
    code = ks.KS_DTYPE[x.dtype]
    assert b.ks_softmax_workspace_size(rows, hidden, code) > 0          # a split plan: the array is used
    stream = torch.cuda.Stream()
    want = torch.empty_like(x)
    with torch.cuda.stream(stream):
        assert b.ks_softmax_noalloc(want.data_ptr(), x.data_ptr(), rows, hidden, code, stream.cuda_stream) == 0
    stream.synchronize()
    out = torch.full_like(x, float("nan"))
    other_in = workloads.random_case((2, 32768), "bfloat16", 38)["x"].cuda()
    other_out = torch.empty_like(other_in)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            st = b.ks_softmax_noalloc(out.data_ptr(), x.data_ptr(), rows, hidden, code, stream.cuda_stream)
    assert st == 0
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("noalloc graph replay", rep)
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))
        # eager work on the same array between replays (another shape, another dtype)
        assert b.ks_softmax_noalloc(other_out.data_ptr(), other_in.data_ptr(), 2, 32768, ks.KS_DTYPE[other_in.dtype],
                                    torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
    check_normalised(out.cpu(), oracle.softmax(x.cpu()), 0.999)
