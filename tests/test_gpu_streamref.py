"""The benchmark's reference streams (libks_streamref.so) on the GPU: each
kernel writes exactly what its source says, so the ceilings and the wave
timeline measured with them are timings of the work they claim to do.

Every row kernel's wave-wide scale is 1 / sqrt(1 + s) for a non-negative s,
converted to an integer and or-ed with 1: always 1, so the row layouts store
each piece with its first word xor 1.
"""
import pytest
import torch

import bench
from gpu_cases import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def ref():
    return bench.StreamRef()


def _words(n_bytes: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-2**31, 2**31 - 1, (n_bytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)


def _flip_first_word(w: torch.Tensor) -> torch.Tensor:
    out = w.clone().view(-1, 4)
    out[:, 0] ^= 1
    return out.view(-1)


def _run(rc: int, what: str) -> None:
    assert rc == 0, f"{what} returned {rc}"
    torch.cuda.synchronize()


def test_write_copy_read(ref):
    n = 64 << 10
    src_h = _words(n, 1)
    src = src_h.cuda()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    say("streamref read / write / copy", n)
    _run(ref.h.ksref_read(src.data_ptr(), n, sink.data_ptr(), None, None, None), "ksref_read")
    off = torch.arange(0, n, 16, dtype=torch.int64)    # each piece's byte offset, the pattern write_one stores
    want = torch.stack([off, off ^ 0x55555555, ~off & 0xFFFFFFFF, torch.full_like(off, 0x3F800000)], 1)
    for policy in (0, 1, 2):
        dst = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
        _run(ref.h.ksref_write(dst.data_ptr(), n, policy, None, None, None), f"ksref_write {policy}")
        got = dst.cpu().view(-1, 4).to(torch.int64) & 0xFFFFFFFF
        assert torch.equal(got, want), f"write policy {policy}"
        dst.zero_()
        _run(ref.h.ksref_copy(src.data_ptr(), dst.data_ptr(), n, policy, None, None, None), f"ksref_copy {policy}")
        assert torch.equal(dst.cpu(), _flip_first_word(src_h)), f"copy policy {policy}"


@pytest.mark.parametrize("pieces", [1, 2, 4, 8])
def test_row_layouts(ref, pieces):
    n = 256 << 10
    x_h, r_h = _words(n, 10 + pieces), _words(n, 20 + pieces)
    x, y = x_h.cuda(), torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    say("streamref rows / in place", pieces)
    _run(ref.h.ksref_copy_rows(x.data_ptr(), y.data_ptr(), n, pieces, None, None, None), "ksref_copy_rows")
    assert torch.equal(y.cpu(), _flip_first_word(x_h))
    if pieces == 4:
        return                         # ksref_inplace4 has 1, 2 and 8 pieces
    r = r_h.cuda()
    _run(ref.h.ksref_inplace4(x.data_ptr(), r.data_ptr(), n, pieces, None, None, None), "ksref_inplace4")
    assert torch.equal(r.cpu(), x_h ^ r_h)
    assert torch.equal(x.cpu(), _flip_first_word(x_h))


@pytest.mark.parametrize("layout", [0, 1, 2])
@pytest.mark.parametrize("policy", [1, 2])
def test_timeline(ref, layout, policy):
    n = 256 << 10                      # 8 workgroups, 32 waves of one 8 KiB row
    waves = n // 8192
    x_h, y_h = _words(n, 30 + layout), _words(n, 40 + layout)
    x, y = x_h.cuda(), y_h.cuda()
    stamps = torch.zeros(waves, 8, dtype=torch.int64, device="cuda")
    say("streamref timeline", layout, policy)
    _run(ref.h.ksref_timeline(x.data_ptr(), y.data_ptr(), n, layout, policy, stamps.data_ptr(),
                              stamps.numel() * 8, None, None, None), "ksref_timeline")
    if layout == 0:
        assert torch.equal(x.cpu(), x_h) and torch.equal(y.cpu(), _flip_first_word(x_h))
    elif layout == 1:
        assert torch.equal(y.cpu(), x_h ^ y_h) and torch.equal(x.cpu(), _flip_first_word(x_h))
    else:
        assert torch.equal(x.cpu(), x_h) and torch.equal(y.cpu(), y_h)
    st = stamps.cpu()
    times = st[:, :6]
    assert bool((times > 0).all())
    assert bool((times[:, 1:] >= times[:, :-1]).all()), "a wave's stamps must not go back in time"
    assert bool((st[:, 7] >= 0).all() and (st[:, 7] < 64).all())        # XCD ids
    khz = bench.ctypes.c_int(0)
    assert ref.h.ksref_wall_clock_khz(bench.ctypes.byref(khz)) == 0 and khz.value > 0
    span_us = float(times[:, 5].max() - times[:, 0].min()) * 1e3 / khz.value
    assert span_us < 10000.0, "a 256 KiB kernel spans milliseconds: the clock or the stamps are wrong"


def test_empty_and_spin(ref):
    say("streamref empty / spin")
    _run(ref.h.ksref_empty(512, None, None, None), "ksref_empty")
    _run(ref.h.ksref_spin(10, None), "ksref_spin")
