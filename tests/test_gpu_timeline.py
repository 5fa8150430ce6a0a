"""GPU test of the instrumented timing build (libpk_gemm_rs_timeline.so: the
library's sources compiled with PK_TIMELINE): with a phase record attached,
its outputs must be bitwise those of the product library, and the record
must hold a plausible placement and increasing phase times for every
workgroup."""
import numpy as np
import pytest
import torch

from gemm_reduce_scatter_amd import binding as pk
from gemm_reduce_scatter_amd import inputs as gen
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _native():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pk.load()
    yield
    pk.use_library(pk.LIB_NAME)
    torch.cuda.synchronize()


@pytest.mark.parametrize("config", [1, 6])
def test_timing_build_is_bitwise_the_library(config):
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=71)
    ref = H.Share(w, "f32")
    pk.use_library(pk.LIB_NAME)
    H.run(ref, A, B, peers, config=config)
    got = H.Share(w, "f32")
    tl = torch.zeros(pk.TIMELINE_BYTES // 8, dtype=torch.int64, device=DEV)
    try:
        pk.use_library(pk.TIMELINE_LIB_NAME)
        H.run(got, A, B, peers, config=config, timeline=tl)
        torch.cuda.synchronize()
    finally:
        pk.use_library(pk.LIB_NAME)
    assert torch.equal(got.send.view(torch.int16), ref.send.view(torch.int16))
    assert torch.equal(got.out.view(torch.int32), ref.out.view(torch.int32))
    assert torch.equal(got.flags, ref.flags)
    t = tl.cpu().numpy().view(np.uint64).reshape(pk.TIMELINE_WORKGROUPS, pk.TIMELINE_SLOTS)
    live = np.nonzero(t[:, 1])[0]
    assert live.size > 0 and np.array_equal(live, np.arange(live.size))   # one row per workgroup
    for b in live:
        xcc, hw = int(t[b, 0]) >> 32, int(t[b, 0]) & 0xFFFFFFFF
        assert xcc < 8 and ((hw >> 8) & 15) < 16
        marks = [int(m) for m in t[b, 2:] if m]
        assert marks, b
        clocks = [int(t[b, 1])] + [m & ((1 << 56) - 1) for m in marks]
        assert all(x <= y for x, y in zip(clocks, clocks[1:])), b
        assert all(1 <= (m >> 56) <= 4 for m in marks)
    # the product library ignores the record
    tl2 = torch.zeros_like(tl)
    H.run(ref, A, B, peers, config=config, timeline=tl2)
    torch.cuda.synchronize()
    assert int(tl2.abs().max()) == 0
