"""GPU tests of the inter-CU schedule's reduction role through the C ABI.

Dedicated workgroups sum the owned shard's staged peer partials into an fp32
workspace while the rest run the share; the owned items add their local
partial to it.  The summation order is the fused epilogue's, so send
buffers, the owned shard and the flags must equal the staged share's bit for
bit, the workspace must hold the oracle's peer sum (exactly on integer
inputs), and the piece words and the error word must be what the oracle's
intercu_reduce says.
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


def _side(w):
    """presum (NaN-filled), piece words, error word."""
    presum = torch.full((w.S, w.N), float("nan"), dtype=torch.float32, device=DEV)
    pieces = torch.zeros(pk.pk_reduce_piece_words(w.M, w.N, w.P), dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    return presum, pieces, err


def _peer_sum_f32(peers):
    """The fused epilogue's peer sum: fp32, ascending slots, from +0."""
    t = torch.zeros(peers.shape[1:], dtype=torch.float32, device=peers.device)
    for j in range(peers.shape[0]):
        t = t + peers[j].float()
    return t


def _same(share, ref):
    assert torch.equal(share.send.view(torch.int16), ref.send.view(torch.int16))
    word = torch.int32 if share.out_dtype == "f32" else torch.int16
    assert torch.equal(share.out.view(word), ref.out.view(word))
    assert torch.equal(share.flags, ref.flags)


def _check_side(w, peers, presum, pieces, err, pieces_before, expected, exact, peer_ready=None):
    want, want_pieces, want_err = orc.intercu_reduce(
        gen.bf16_bits(peers), pieces_before, expected, w.chunk_rows,
        None if peer_ready is None else peer_ready.cpu().numpy().view(np.uint32))
    got = presum.cpu().numpy().astype(np.float64)
    if exact:
        assert np.array_equal(got, want)
    else:
        # seven bf16 terms summed in fp32: within the recursive-summation bound
        mag = np.abs(orc.bf16_bits_to_f64(gen.bf16_bits(peers))).sum(axis=0)
        n = peers.shape[0]
        u = 2.0 ** -24
        assert np.all(np.abs(got - want) <= n * u / (1 - n * u) * mag)
    assert torch.equal(presum, _peer_sum_f32(peers))
    shape = want_pieces.shape
    assert np.array_equal(pieces.cpu().numpy().view(np.uint32).reshape(shape), want_pieces)
    assert int(err.item()) == want_err
    return want_pieces


@pytest.mark.parametrize("n_comm", [8, 32])
def test_reduce_comm_dominant_matches_staged(n_comm):
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=51)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers)
    share = H.Share(w, "f32")
    presum, pieces, err = _side(w)
    before = np.zeros(pk.pk_reduce_piece_words(w.M, w.N, w.P), np.uint32).reshape(
        -(-w.S // 64), -(-w.N // 64))
    pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags, presum, pieces,
                                 err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0,
                                 1, n_comm)
    torch.cuda.synchronize()
    _same(share, ref)
    _check_side(w, peers, presum, pieces, err, before, 1, exact=False)
    assert share.canaries_intact()


def test_reduce_in_place_fp32_out_and_repeated_calls():
    """presum is out itself; three calls in a row raise the piece words to 3."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=52)
    ref = H.Share(w, "f32")
    share = H.Share(w, "f32")
    _, pieces, err = _side(w)
    call = pk.BoundInterCUReduce(A, B, peers, share.send, share.out, share.flags, share.out,
                                 pieces, err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows,
                                 w.tile_order, 0, 1, 32)
    for n in (1, 2, 3):
        H.run(ref, A, B, peers)
        call()
        torch.cuda.synchronize()
        _same(share, ref)
        assert np.all(pieces.cpu().numpy() == n) and int(err.item()) == 0
        call.next()
    assert share.canaries_intact()


SHAPES = [
    # whole tiles (bf16 out), ragged N and K, every order
    gen.Workload("red_a", P=4, rank=1, M=4096, N=1032, K=200, chunk_rows=256,
                 ab_dist="int", peer_dist="int", out_dtype="bf16"),
    # P = 2 under the owned split of configuration 1 (one peer slot), fp32 out
    gen.Workload("red_b", P=2, rank=1, M=1024, N=2048, K=320, chunk_rows=128,
                 ab_dist="int", peer_dist="int", out_dtype="f32"),
    # a shard height that is not a multiple of 64 (ragged pieces)
    gen.Workload("red_c", P=8, rank=6, M=8 * 160, N=512, K=96, chunk_rows=80,
                 ab_dist="int", peer_dist="int", out_dtype="f32"),
]


OPTS = {"red_b": dict(config=1, owned_split=1)}


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("order", [0, 1, 2])
def test_reduce_integer_exact_against_oracle(w, order):
    A, B, peers = gen.make_inputs(w, DEV, seed=53, integer=True)
    share = H.Share(w, w.out_dtype)
    presum, pieces, err = _side(w)
    pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags, presum, pieces,
                                 err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, order,
                                 1 if w.out_dtype == "bf16" else 0, 1, 16,
                                 **OPTS.get(w.name, {}))
    torch.cuda.synchronize()
    res = orc.gemm_rs_oracle(gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers), w.P,
                             w.rank, w.chunk_rows)
    assert np.array_equal(gen.bf16_bits(share.send), res.send_bits)
    if w.out_dtype == "bf16":
        assert np.array_equal(gen.bf16_bits(share.out), orc.f64_to_bf16_bits(res.out))
    else:
        assert np.array_equal(share.out.cpu().numpy().astype(np.float64), res.out)
    assert np.array_equal(share.flags.cpu().numpy().view(np.uint32),
                          res.flags)
    before = np.zeros((-(-w.S // 64), -(-w.N // 64)), np.uint32)
    _check_side(w, peers, presum, pieces, err, before, 1, exact=True)
    assert share.canaries_intact()


def test_reduce_waits_for_incoming_chunks():
    """peer_ready given: every word at `expected` lets the sums through; one
    word a call behind is given up (error bit 2) and its rows summed as they
    are, which here are already the staged values.  In the second call the
    piece words already stand at `expected` and the workspace holds the sums,
    so the compute side does not wait and the outcome does not depend on
    how long the reduction side waited."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=54)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers)
    n_chunks = w.S // w.chunk_rows
    ready = torch.full((w.P - 1, n_chunks), 3, dtype=torch.int32, device=DEV)
    before = np.zeros((-(-w.S // 64), -(-w.N // 64)), np.uint32)
    for late in (False, True):
        share = H.Share(w, "f32")
        presum, pieces, err = _side(w)
        if late:
            ready[4, 2] = 2
            presum.copy_(_peer_sum_f32(peers))
            pieces.fill_(3)
        else:
            pieces.fill_(2)
        call = pk.BoundInterCUReduce(A, B, peers, share.send, share.out, share.flags, presum,
                                     pieces, err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows,
                                     w.tile_order, 0, 3, 32, spin_limit=8 if late else 1 << 16,
                                     peer_ready=ready)
        call()
        if late:
            # an incoming chunk given up: the binding's check refuses the results
            with pytest.raises(pk.IncompleteError):
                call.check()
        else:
            assert call.check() == 0
        _same(share, ref)
        _check_side(w, peers, presum, pieces, err, before + (3 if late else 2), 3, exact=False,
                    peer_ready=ready)
        assert int(err.item()) == (2 if late else 0)


def test_reduce_with_chunks_arriving_during_the_launch():
    """The peer partials are copied in and their ready words raised, slot by
    slot, on a second stream while the kernel runs on all but 32 CUs."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=55)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers)
    staged = torch.zeros_like(peers)
    ready = torch.zeros((w.P - 1, w.S // w.chunk_rows), dtype=torch.int32, device=DEV)
    share = H.Share(w, "f32")
    presum, pieces, err = _side(w)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    torch.cuda.synchronize()
    s_main, s_copy = torch.cuda.Stream(), torch.cuda.Stream()
    pk.pk_gemm_rs_intercu_reduce(A, B, staged, share.send, share.out, share.flags, presum, pieces,
                                 err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0,
                                 1, 32, peer_ready=ready, max_workgroups=max(cus - 64, 8),
                                 stream=s_main)
    with torch.cuda.stream(s_copy):
        for j in range(w.P - 1):
            staged[j].copy_(peers[j])
            ready[j].fill_(1)          # a later kernel on this stream: the slot is written
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    _same(share, ref)
    assert torch.equal(presum, _peer_sum_f32(peers))


def test_reduce_piece_wait_gives_up():
    """Compute workgroups told to wait for call 5 while the pieces reach 1
    give up (error bit 1) and sum their staged peers themselves: with presum
    NaN-filled when the launch starts, the results are still the staged
    share's, bit for bit, and the binding's check accepts them."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=56)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers)
    presum, pieces, err = _side(w)
    share = H.Share(w, "f32")
    call = pk.BoundInterCUReduce(A, B, peers, share.send, share.out, share.flags, presum, pieces,
                                 err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0,
                                 5, 32, spin_limit=4)
    call()
    assert call.check() == 1
    _same(share, ref)
    before = np.zeros((-(-w.S // 64), -(-w.N // 64)), np.uint32)
    _check_side(w, peers, presum, pieces, err, before, 5, exact=False)


def test_reduce_rejects_bad_arguments():
    w = gen.WORKLOADS["tiny"]
    A, B, peers = gen.make_inputs(w, DEV, seed=57)
    share = H.Share(w, "f32")
    presum, pieces, err = _side(w)
    with pytest.raises(pk.PkError):      # no reduction workgroups, and P = 2 has no background reduction
        pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags, presum,
                                     pieces, err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, 0, 0,
                                     1, 0)
    with pytest.raises(ValueError):      # workspace too small
        pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags,
                                     presum[:1], pieces, err, w.M, w.N, w.K, w.P, w.rank,
                                     w.chunk_rows, 0, 0, 1, 8)
    with pytest.raises(ValueError):      # piece words missing
        pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags, presum,
                                     pieces[:0], err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows,
                                     0, 0, 1, 8)
    # a bf16 out cannot hold the fp32 sums: presum starting at out's address
    # (a float buffer whose first half is the bf16 out) is refused by the library
    both = torch.zeros((w.S, w.N), dtype=torch.float32, device=DEV)
    out16 = both.view(torch.bfloat16).view(-1)[:w.S * w.N].view(w.S, w.N)
    with pytest.raises(pk.PkError) as e:
        pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, out16, share.flags, both, pieces,
                                     err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, 0, 1, 1, 8)
    assert e.value.code == -1


# --- reduction in the background of the main loops (no communicator CUs) ---
# num_comm_cus = 0: every workgroup multiplies one whole tile; while the send
# tiles' workgroups (and each owned tile's own) multiply, each sums the peer
# partials of one owned sub-tile into presum and raises its pieces; the owned
# tiles then add their local partial.  Outputs are the staged share's, bit
# for bit.


@pytest.mark.parametrize("order", [0, 1, 2])
def test_background_reduce_matches_staged(order):
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=61 + order)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers, tile_order=order)
    share = H.Share(w, "f32")
    presum, pieces, err = _side(w)
    before = np.zeros((-(-w.S // 64), -(-w.N // 64)), np.uint32)
    pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags, presum, pieces,
                                 err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, order, 0, 1, 0)
    torch.cuda.synchronize()
    _same(share, ref)
    _check_side(w, peers, presum, pieces, err, before, 1, exact=False)
    assert share.canaries_intact()


def test_background_reduce_integer_exact_repeated():
    """Integer inputs give the oracle's results exactly on each of three
    calls, and the piece and ready words count the calls."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=64, integer=True)
    res = orc.gemm_rs_oracle(gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers), w.P,
                             w.rank, w.chunk_rows)
    share = H.Share(w, "f32")
    presum, pieces, err = _side(w)
    call = pk.BoundInterCUReduce(A, B, peers, share.send, share.out, share.flags, presum,
                                 pieces, err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows,
                                 w.tile_order, 0, 1, 0)
    half = (w.P - 1) * (w.S // w.chunk_rows)   # ready words, then the counters' lines
    for n in (1, 2, 3):
        call()
        assert call.check() == 0
        assert np.array_equal(gen.bf16_bits(share.send), res.send_bits)
        assert np.array_equal(share.out.cpu().numpy().astype(np.float64), res.out)
        assert int(share.flags[:half].min()) == n and int(share.flags[:half].max()) == n
        assert int(share.flags[half:].abs().max()) == 0
        assert np.all(pieces.cpu().numpy() == n) and int(err.item()) == 0
        call.next()
    assert share.canaries_intact()


def test_background_reduce_incoming_chunk_waits():
    """peer_ready given: all words at `expected` pass; one word a call behind
    is given up after a few polls (error bit 2) and the sub-tiles whose rows
    it covers are summed from the staged partials as they are (here already
    complete), so the outputs stay the staged share's.  The piece waits share
    the short spin limit, so in that call the piece words already stand at
    `expected` and presum already holds the sums: the owned tiles do not
    wait, and the outcome does not depend on how long the chunk waits took."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=65)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers)
    ready = torch.full((w.P - 1, w.S // w.chunk_rows), 1, dtype=torch.int32, device=DEV)
    for late in (False, True):
        if late:
            ready[3, 1] = 0
        share = H.Share(w, "f32")
        presum, pieces, err = _side(w)
        if late:
            presum.copy_(_peer_sum_f32(peers))
            pieces.fill_(1)
        pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags, presum,
                                     pieces, err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows,
                                     w.tile_order, 0, 1, 0, spin_limit=8 if late else 1 << 16,
                                     peer_ready=ready)
        torch.cuda.synchronize()
        _same(share, ref)
        assert torch.equal(presum, _peer_sum_f32(peers))
        assert np.all(pieces.cpu().numpy() == (2 if late else 1))
        assert int(err.item()) == (2 if late else 0)


def test_background_reduce_piece_wait_gives_up():
    """Owned tiles told to wait for call 5 while the pieces reach 1 give up
    (error bit 1) and sum their staged peers themselves: presum is NaN-filled
    when the launch starts, yet the results are the staged share's."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=66)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers)
    presum, pieces, err = _side(w)
    share = H.Share(w, "f32")
    pk.pk_gemm_rs_intercu_reduce(A, B, peers, share.send, share.out, share.flags, presum, pieces,
                                 err, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, w.tile_order, 0,
                                 5, 0, spin_limit=4)
    torch.cuda.synchronize()
    _same(share, ref)
    assert np.all(pieces.cpu().numpy() == 1)
    assert int(err.item()) == 1


def test_background_reduce_rejects_what_it_cannot_run():
    """P other than 8, the owned split turned off, or a grid that cannot hold
    every tile at once: PK_ERR_CONFIG, nothing launched."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=67)
    share = H.Share(w, "f32")
    presum, pieces, err = _side(w)
    args = (A, B, peers, share.send, share.out, share.flags, presum, pieces, err, w.M, w.N, w.K,
            w.P, w.rank, w.chunk_rows, w.tile_order, 0, 1, 0)
    for kw in (dict(owned_split=-1), dict(max_workgroups=128), dict(config=2)):
        with pytest.raises(pk.PkError) as e:
            pk.pk_gemm_rs_intercu_reduce(*args, **kw)
        assert e.value.code == -5
    # presum may not be out itself here: a send tile's workgroup that started
    # late would store its bare peer sum over a finished owned tile
    with pytest.raises(pk.PkError) as e:
        pk.pk_gemm_rs_intercu_reduce(*args[:6], share.out, *args[7:])
    assert e.value.code == -1
    w4 = gen.WORKLOADS["comm_dominant"].with_(P=4, rank=1)
    A4, B4, p4 = gen.make_inputs(w4, DEV, seed=68)
    s4 = H.Share(w4, "f32")
    pr4, pc4, er4 = _side(w4)
    with pytest.raises(pk.PkError) as e:
        pk.pk_gemm_rs_intercu_reduce(A4, B4, p4, s4.send, s4.out, s4.flags, pr4, pc4, er4, w4.M,
                                     w4.N, w4.K, w4.P, w4.rank, w4.chunk_rows, 0, 0, 1, 0)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert int(share.flags.abs().max()) == 0 and int(pieces.abs().max()) == 0
