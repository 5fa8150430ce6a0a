"""GPU test of pk_gemm_rs_intercu_reduce_static, the entry point that keeps
the reduction role's workspace in the library's static device array instead
of taking it from the caller.

Its outputs (send buffers, owned shard, flags, error word) must equal those
of pk_gemm_rs_intercu_reduce with a caller-provided workspace, bit for bit,
on two calls in a row whose second is smaller than the first (the array
keeps the first call's contents), in both the background mode and with
dedicated reduction workgroups; the integer twin also matches the oracle.
"""
import numpy as np
import pytest
import torch

import oracle.gemm_rs_oracle as orc
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
    torch.cuda.synchronize()


# Tile configuration 1 (256 x 256) throughout: the background mode runs only
# that one, and the smaller second shape would otherwise pick another.
def _with_workspace(w, A, B, peers, n_comm, order):
    share = H.Share(w, w.out_dtype)
    presum = torch.full((w.S, w.N), float("nan"), dtype=torch.float32, device=DEV)
    pieces = torch.zeros(pk.pk_reduce_piece_words(w.M, w.N, w.P), dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    call = pk.BoundInterCUReduce(A, B, peers, share.send, share.out, share.flags, presum, pieces,
                                 err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, order,
                                 1 if w.out_dtype == "bf16" else 0, 1, n_comm, config=1)
    call()
    assert call.check() == 0
    return share


def _static(w, A, B, peers, n_comm, order):
    share = H.Share(w, w.out_dtype)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    call = pk.BoundInterCUReduceStatic(A, B, peers, share.send, share.out, share.flags, err,
                                       w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, order,
                                       1 if w.out_dtype == "bf16" else 0, 0, n_comm, config=1)
    call()
    assert call.check() == 0
    return share


def _same(a, b):
    assert torch.equal(a.send.view(torch.int16), b.send.view(torch.int16)), "send buffers differ"
    word = torch.int32 if a.out_dtype == "f32" else torch.int16
    assert torch.equal(a.out.view(word), b.out.view(word)), "owned shard differs"
    assert torch.equal(a.flags, b.flags), "flags differ"
    assert a.canaries_intact() and b.canaries_intact()


@pytest.mark.parametrize("n_comm", [0, 32])
def test_static_workspace_matches_caller_workspace(n_comm):
    big = gen.WORKLOADS["comm_dominant"]                      # (M/P) x N = 512 x 4096
    small = big.with_(M=2048, N=1024, K=256, chunk_rows=64,   # 256 x 1024, integer twin
                      ab_dist="int", peer_dist="int")
    for i, (w, integer) in enumerate(((big, False), (small, True))):
        print(f"[static n_comm={n_comm}] call {i + 1}: M={w.M} N={w.N} K={w.K}", flush=True)
        A, B, peers = gen.make_inputs(w, DEV, seed=90 + i, integer=integer)
        for order in (w.tile_order, 2):
            ref = _with_workspace(w, A, B, peers, n_comm, order)
            got = _static(w, A, B, peers, n_comm, order)
            _same(got, ref)
        if integer:
            res = orc.gemm_rs_oracle(gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers),
                                     w.P, w.rank, w.chunk_rows)
            H.compare_exact(res, got)


def test_static_workspace_rejects_what_it_cannot_hold():
    max_sums, max_pieces, nbytes = pk.pk_static_workspace_limits()
    assert max_sums == 1 << 22 and max_pieces == 1 << 16
    assert nbytes == 4 * (max_sums + max_pieces)
    w = gen.WORKLOADS["comm_dominant"].with_(M=16384, N=4096, K=8)   # (M/P) x N = 2^23
    A, B, peers = gen.make_inputs(w, DEV, seed=99)
    share = H.Share(w, "f32")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(pk.PkError) as e:
        pk.pk_gemm_rs_intercu_reduce_static(A, B, peers, share.send, share.out, share.flags, err,
                                            w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, 0, 0, 0,
                                            32)
    assert e.value.code == -8
    torch.cuda.synchronize()
    assert int(share.flags.abs().max()) == 0 and int(err.item()) == 0
