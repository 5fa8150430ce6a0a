"""GPU tests of the all-gather + GEMM against the oracle, through the C ABI.

C = A_gathered * B, where tiles of other ranks' rows wait for the ready words
of the A chunks they read.  Integer-valued inputs give products exact in
fp32 and in bf16, so C must match the oracle bit for bit; real-valued inputs
must meet the same bound as the fused share.
"""
import numpy as np
import pytest
import torch

import oracle.gemm_rs_oracle as orc
from gemm_reduce_scatter_amd import binding as pk
from gemm_reduce_scatter_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _native():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pk.load()
    yield
    torch.cuda.synchronize()


def _inputs(M, N, K, integer, seed):
    w = gen.Workload("ag", P=1, rank=0, M=M, N=N, K=K, chunk_rows=0,
                     ab_dist="int" if integer else "normal_sqrtk", peer_dist="int",
                     out_dtype="bf16")
    A, B, _ = gen.make_inputs(w, DEV, seed=seed, integer=integer)
    return A, B


def _run(A, B, ready, P, rank, chunk_rows, expected=1, spin=1 << 16, order=1, **kw):
    M, K = A.shape
    N = B.shape[1]
    C = torch.full((M, N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pk.pk_ag_gemm(A, ready, B, C, err, M, N, K, P, rank, chunk_rows, expected, spin, order, **kw)
    return C, err


@pytest.mark.parametrize("shape", [(2048, 768, 512, 8, 3, 64), (1024, 1032, 200, 4, 0, 128),
                                   (960, 256, 96, 4, 3, 240)],
                         ids=["p8", "ragged_nk", "ragged_m"])
@pytest.mark.parametrize("order", [0, 1, 2])
def test_ag_gemm_integer_exact(shape, order):
    M, N, K, P, rank, cr = shape
    A, B = _inputs(M, N, K, True, 30)
    ready = torch.ones((P, (M // P) // cr), dtype=torch.int32, device=DEV)
    C, err = _run(A, B, ready, P, rank, cr, order=order)
    torch.cuda.synchronize()
    want, want_err = orc.ag_gemm(gen.bf16_bits(A), gen.bf16_bits(B),
                                 ready.cpu().numpy().view(np.uint32), P, rank, cr, 1)
    assert int(err.item()) == want_err == 0
    assert np.array_equal(gen.bf16_bits(C), orc.f64_to_bf16_bits(want))


def test_ag_gemm_real_within_bound():
    M, N, K, P, rank, cr = 2048, 1024, 1024, 8, 5, 128
    A, B = _inputs(M, N, K, False, 31)
    ready = torch.full((P, (M // P) // cr), 7, dtype=torch.int32, device=DEV)
    C, err = _run(A, B, ready, P, rank, cr, expected=7)
    torch.cuda.synchronize()
    want, _ = orc.ag_gemm(gen.bf16_bits(A), gen.bf16_bits(B),
                          ready.cpu().numpy().view(np.uint32), P, rank, cr, 7)
    got = orc.bf16_bits_to_f64(gen.bf16_bits(C))
    mag = orc.local_partial_abs(gen.bf16_bits(A), gen.bf16_bits(B))
    tol = orc.error_bound(mag, K, True, want)
    assert int(err.item()) == 0
    assert np.all(np.abs(got - want) <= tol)
    # bf16 C against the oracle rounded once to bf16 (the rounding alone is
    # about 1.1e-3 relative, above the 1e-3 budget), as for a bf16 shard
    assert orc.rel_frobenius(got, orc.bf16_bits_to_f64(orc.f64_to_bf16_bits(want))) <= 1e-3


def test_ag_gemm_waits_for_chunks_produced_concurrently():
    """The other ranks' rows are copied into the gathered buffer and their
    ready words set, rank by rank in ring order, on a second stream while the
    kernel runs; it leaves 32 CUs for those copies."""
    M, N, K, P, rank, cr = 2048, 1024, 768, 8, 2, 64
    S = M // P
    src, B = _inputs(M, N, K, True, 32)
    A = torch.zeros_like(src)
    A[rank * S:(rank + 1) * S] = src[rank * S:(rank + 1) * S]
    ready = torch.zeros((P, S // cr), dtype=torch.int32, device=DEV)
    C = torch.full((M, N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    torch.cuda.synchronize()
    s_gemm, s_copy = torch.cuda.Stream(), torch.cuda.Stream()
    pk.pk_ag_gemm(A, ready, B, C, err, M, N, K, P, rank, cr, 1, 1 << 16, 1,
                  max_workgroups=max(cus - 32, 1), stream=s_gemm)
    with torch.cuda.stream(s_copy):
        for i in range(1, P):
            p = (rank + i) % P
            A[p * S:(p + 1) * S].copy_(src[p * S:(p + 1) * S])
            ready[p].fill_(1)          # a later kernel on this stream: the rows are written
    torch.cuda.synchronize()
    want, _ = orc.ag_gemm(gen.bf16_bits(src), gen.bf16_bits(B),
                          np.ones((P, S // cr), np.uint32), P, rank, cr, 1)
    assert int(err.item()) == 0
    assert np.array_equal(gen.bf16_bits(C), orc.f64_to_bf16_bits(want))


def test_ag_gemm_gives_up_on_missing_chunks():
    M, N, K, P, rank, cr = 1024, 512, 256, 4, 1, 64
    A, B = _inputs(M, N, K, True, 33)
    ready = torch.ones((P, (M // P) // cr), dtype=torch.int32, device=DEV)
    ready[3, 2] = 0                                    # one chunk of rank 3 never arrives
    C, err = _run(A, B, ready, P, rank, cr, spin=4)
    torch.cuda.synchronize()
    want, want_err = orc.ag_gemm(gen.bf16_bits(A), gen.bf16_bits(B),
                                 ready.cpu().numpy().view(np.uint32), P, rank, cr, 1)
    assert int(err.item()) == want_err == 1
    # every tile is still computed, from the rows as they are
    assert np.array_equal(gen.bf16_bits(C), orc.f64_to_bf16_bits(want))


def test_ag_gemm_rejects_bad_arguments():
    A, B = _inputs(1024, 512, 256, True, 34)
    ready = torch.ones((4, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(pk.PkError):
        _run(A, B, ready, 4, 4, 64)                    # rank outside [0, P)
    with pytest.raises(pk.PkError):
        _run(A, B, ready, 4, 0, 64, spin=0)
    with pytest.raises(ValueError):
        _run(A, B, ready[:1], 4, 0, 64)                # a_ready too short
