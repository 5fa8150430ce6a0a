"""GPU tests of the chunk consumer (the step after the share) against the oracle.

The consumer waits on each chunk's ready word and copies the chunk from the
send buffers into staging buffers; the oracle's consume_chunks says what the
staging buffers and status words must hold.  Every test bounds the waits
with spin_limit, so a chunk that is never signalled ends as a time-out.
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
W = gen.Workload("consume", P=8, rank=3, M=2048, N=1024, K=256, chunk_rows=64,
                 ab_dist="int", peer_dist="int", out_dtype="f32")
N_CHUNKS = (W.P - 1) * (W.S // W.chunk_rows)


@pytest.fixture(scope="module", autouse=True)
def _native():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pk.load()
    yield
    torch.cuda.synchronize()


def _staging():
    dest = torch.full((W.P - 1, W.S, W.N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    status = torch.full((N_CHUNKS,), 7, dtype=torch.int32, device=DEV)
    observed = torch.full((N_CHUNKS,), -1, dtype=torch.int64, device=DEV)
    return dest, status, observed


def _check(share, dest_before, dest, status, expected):
    ready = share.flags[:N_CHUNKS].cpu().numpy().view(np.uint32).reshape(W.P - 1, -1)
    want_dest, want_status = orc.consume_chunks(ready, gen.bf16_bits(share.send),
                                                dest_before, W.chunk_rows, expected)
    assert np.array_equal(status.cpu().numpy().reshape(W.P - 1, -1), want_status)
    assert np.array_equal(gen.bf16_bits(dest), want_dest)
    return want_status


def _produce(share, calls=1, **opts):
    A, B, peers = gen.make_inputs(W, DEV, seed=3, integer=True)
    for _ in range(calls):
        H.run(share, A, B, peers, **opts)
    return A, B, peers


def test_consume_after_the_producer():
    share = H.Share(W, "f32")
    _produce(share)
    dest, status, observed = _staging()
    before = gen.bf16_bits(dest)
    flags_before = share.flags.clone()
    pk.pk_rs_consume(share.flags, share.send, dest, W.M, W.N, W.P, W.chunk_rows, 1, status,
                     observed)
    torch.cuda.synchronize()
    st = _check(share, before, dest, status, 1)
    assert np.all(st == 0)
    assert torch.all(observed > 0)
    assert torch.equal(share.flags, flags_before)          # the consumer writes no flag


@pytest.mark.parametrize("config", [0, 1])
def test_consume_concurrently_with_the_producer(config):
    """Producer and consumer on two streams at once; the producer leaves 16
    CUs to the consumer.  Every chunk must be seen after its word rose.
    Configuration 0 lets the library choose (64 x 64 tiles here); 1 runs the
    gathered rows (P = 8, S = 256: 8 row groups x 4 column tiles), whose
    arrivals follow a workgroup-scope release: eight runs on fresh,
    poison-filled buffers with different inputs, so that a chunk read before
    its rows were visible would show poison or another run's values."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    opts = {"config": config} if config else {}
    for rep in range(8 if config else 1):
        share = H.Share(W, "f32")
        dest, status, observed = _staging()
        before = gen.bf16_bits(dest)
        clock = torch.zeros(N_CHUNKS, dtype=torch.int64, device=DEV)
        A, B, peers = gen.make_inputs(W, DEV, seed=3 + 10 * rep, integer=True)
        torch.cuda.synchronize()
        s_prod, s_cons = torch.cuda.Stream(), torch.cuda.Stream()
        H.run(share, A, B, peers, stream=s_prod, max_workgroups=max(cus - 16, 1),
              ready_clock=clock, **opts)
        pk.pk_rs_consume(share.flags, share.send, dest, W.M, W.N, W.P, W.chunk_rows, 1, status,
                         observed, spin_limit=1 << 16, max_workgroups=16, stream=s_cons)
        torch.cuda.synchronize()
        st = _check(share, before, dest, status, 1)
        assert np.all(st == 0), rep
        assert torch.all(clock > 0)
        assert torch.all(observed >= clock)


def test_consume_times_out_on_unsignalled_chunks():
    share = H.Share(W, "f32")                  # flags zero: nothing was produced
    dest, status, observed = _staging()
    before = gen.bf16_bits(dest)
    pk.pk_rs_consume(share.flags, share.send, dest, W.M, W.N, W.P, W.chunk_rows, 1, status,
                     observed, spin_limit=4)
    torch.cuda.synchronize()
    st = _check(share, before, dest, status, 1)
    assert np.all(st == 1)
    assert torch.all(observed == 0)


def test_consume_waits_for_the_requested_call():
    share = H.Share(W, "f32")
    _produce(share, calls=2)                   # ready words at 2
    for expected, spin in ((2, 1 << 16), (3, 4), (1, 4)):
        dest, status, observed = _staging()
        before = gen.bf16_bits(dest)
        pk.pk_rs_consume(share.flags, share.send, dest, W.M, W.N, W.P, W.chunk_rows, expected,
                         status, observed, spin_limit=spin)
        torch.cuda.synchronize()
        st = _check(share, before, dest, status, expected)
        assert np.all(st == (1 if expected == 3 else 0)), expected


def test_consume_rejects_bad_arguments():
    share = H.Share(W, "f32")
    dest, status, _ = _staging()
    with pytest.raises(pk.PkError):
        pk.pk_rs_consume(share.flags, share.send, dest, W.M, W.N, W.P, 100, 1, status)   # chunk
    with pytest.raises(pk.PkError):
        pk.pk_rs_consume(share.flags, share.send, dest, W.M, W.N, W.P, W.chunk_rows, 1, status,
                         spin_limit=0)
    with pytest.raises(ValueError):
        pk.pk_rs_consume(share.flags, share.send, dest[:2], W.M, W.N, W.P, W.chunk_rows, 1,
                         status)
