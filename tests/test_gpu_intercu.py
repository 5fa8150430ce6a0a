"""GPU tests of the inter-CU schedule (communicator workgroups) through the C ABI.

One launch must leave send buffers, the owned shard and the flags bit for bit
as the staged share does, and its communicator workgroups must have moved
every chunk into the staging buffers (the oracle's consume_chunks says what
they hold).  On integer-valued inputs every output is also compared with the
oracle's own share (gemm_rs_oracle), and the moved chunks with the oracle's
send bits, so no part of the check rests on the HIP path alone.
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


def _staging(w, chunk_rows):
    n = (w.P - 1) * (w.S // chunk_rows)
    dest = torch.full((w.P - 1, w.S, w.N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    status = torch.full((n,), 7, dtype=torch.int32, device=DEV)
    return dest, status


def _check(w, ref, share, dest_before, dest, status, expected, chunk_rows, res=None):
    """`res`: the oracle's share of integer-valued inputs; then send, out,
    flags and the moved chunks are compared with it as well."""
    assert torch.equal(share.send.view(torch.int16), ref.send.view(torch.int16))
    word = torch.int32 if share.out_dtype == "f32" else torch.int16
    assert torch.equal(share.out.view(word), ref.out.view(word))
    assert torch.equal(share.flags, ref.flags)
    n = (w.P - 1) * (w.S // chunk_rows)
    ready = share.flags[:n].cpu().numpy().view(np.uint32).reshape(w.P - 1, -1)
    sent = gen.bf16_bits(share.send) if res is None else res.send_bits
    if res is not None:
        H.compare_exact(res, share)
        assert np.array_equal(ready, res.ready)
    want_dest, want_status = orc.consume_chunks(ready, sent, dest_before, chunk_rows, expected)
    assert np.array_equal(status.cpu().numpy().reshape(w.P - 1, -1), want_status)
    assert np.array_equal(gen.bf16_bits(dest), want_dest)
    return want_status


def _oracle(w, A, B, peers, ready_before=None):
    return orc.gemm_rs_oracle(gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers), w.P,
                              w.rank, w.chunk_rows, ready_before=ready_before)


@pytest.mark.parametrize("n_comm", [8, 32])
def test_intercu_integer_twin_against_oracle(n_comm):
    """Comm-dominant shape, integer twin: send, out, flags and every moved
    chunk equal the oracle's, over two calls on one flags buffer."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=45, integer=True)
    ref = H.Share(w, "f32")
    share = H.Share(w, "f32")
    dest, status = _staging(w, w.chunk_rows)
    call = pk.BoundInterCU(A, B, peers, share.send, share.out, share.flags, dest, status, w.M,
                           w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0, 1, n_comm)
    ready = None
    for n in (1, 2):
        H.run(ref, A, B, peers)
        res = _oracle(w, A, B, peers, ready)
        before = gen.bf16_bits(dest)
        call()
        assert np.all(call.check() == 0)
        _check(w, ref, share, before, dest, status, n, w.chunk_rows, res)
        ready = res.ready
        call.next()
    assert share.canaries_intact()


@pytest.mark.parametrize("n_comm", [8, 32])
def test_intercu_comm_dominant_matches_staged(n_comm):
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=41)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers)
    share = H.Share(w, "f32")
    dest, status = _staging(w, w.chunk_rows)
    before = gen.bf16_bits(dest)
    pk.pk_gemm_rs_intercu(A, B, peers, share.send, share.out, share.flags, dest, status, w.M,
                          w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0, 1, n_comm)
    torch.cuda.synchronize()
    st = _check(w, ref, share, before, dest, status, 1, w.chunk_rows)
    assert np.all(st == 0)
    assert share.canaries_intact()


@pytest.mark.parametrize("order", [0, 1, 2])
def test_intercu_whole_tiles_bf16(order):
    w = gen.Workload("icu", P=4, rank=1, M=4096, N=1280, K=512, chunk_rows=256,
                     ab_dist="int", peer_dist="int", out_dtype="bf16")
    A, B, peers = gen.make_inputs(w, DEV, seed=42, integer=True)
    ref = H.Share(w, "bf16")
    H.run(ref, A, B, peers, tile_order=order, owned_split=-1)
    share = H.Share(w, "bf16")
    dest, status = _staging(w, w.chunk_rows)
    before = gen.bf16_bits(dest)
    pk.pk_gemm_rs_intercu(A, B, peers, share.send, share.out, share.flags, dest, status, w.M,
                          w.N, w.K, w.P, w.rank, w.chunk_rows, order, 1, 1, 16,
                          owned_split=-1)
    torch.cuda.synchronize()
    st = _check(w, ref, share, before, dest, status, 1, w.chunk_rows, _oracle(w, A, B, peers))
    assert np.all(st == 0)


def test_intercu_repeated_calls_and_a_wrong_epoch():
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=43)
    ref = H.Share(w, "f32")
    share = H.Share(w, "f32")
    dest, status = _staging(w, w.chunk_rows)
    call = pk.BoundInterCU(A, B, peers, share.send, share.out, share.flags, dest, status, w.M,
                           w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0, 1, 16)
    for n in (1, 2):
        H.run(ref, A, B, peers)
        before = gen.bf16_bits(dest)
        call()
        torch.cuda.synchronize()
        st = _check(w, ref, share, before, dest, status, n, w.chunk_rows)
        assert np.all(st == 0), n
        call.next()
    # a call told to move call 5 while the words reach 3: every chunk given up
    H.run(ref, A, B, peers)
    dest2, status2 = _staging(w, w.chunk_rows)
    before = gen.bf16_bits(dest2)
    pk.pk_gemm_rs_intercu(A, B, peers, share.send, share.out, share.flags, dest2, status2, w.M,
                          w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0, 5, 16,
                          spin_limit=4)
    torch.cuda.synchronize()
    st = _check(w, ref, share, before, dest2, status2, 5, w.chunk_rows)
    assert np.all(st == 1)
    with pytest.raises(pk.IncompleteError):
        pk.BoundInterCU(A, B, peers, share.send, share.out, share.flags, dest2, status2, w.M,
                        w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0, 5, 16).check()


def test_intercu_rejects_bad_arguments():
    w = gen.WORKLOADS["tiny"]
    A, B, peers = gen.make_inputs(w, DEV, seed=44)
    share = H.Share(w, "f32")
    dest, status = _staging(w, w.chunk_rows)
    with pytest.raises(pk.PkError):
        pk.pk_gemm_rs_intercu(A, B, peers, share.send, share.out, share.flags, dest, status,
                              w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, 0, 0, 1, 0)
    with pytest.raises(ValueError):
        pk.pk_gemm_rs_intercu(A, B, peers, share.send, share.out, share.flags, dest[:0], status,
                              w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, 0, 0, 1, 8)
