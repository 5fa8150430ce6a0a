"""GPU tests of the atomic push variant against the oracle, through the C ABI.

Every tile of the rank's partial is added with fp32 atomics into the owners'
accumulators.  Integer-valued inputs are exact in fp32, so every word must
match the oracle; with the owned accumulator pre-filled with the fp32 peer
sum in slot order, the push result must equal the staged variant bit for bit.
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


SHAPES = [
    gen.Workload("push_a", P=4, rank=2, M=1024, N=768, K=320, chunk_rows=64,
                 ab_dist="int", peer_dist="int", out_dtype="f32"),
    gen.Workload("push_b", P=8, rank=5, M=2048, N=1032, K=200, chunk_rows=128,
                 ab_dist="int", peer_dist="int", out_dtype="f32"),   # ragged N, K tails
]


def _flags(w):
    return torch.zeros(pk.pk_flags_words(w.P, w.M, w.chunk_rows), dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("order", [0, 1, 2])
def test_push_integer_exact(w, order):
    A, B, _ = gen.make_inputs(w, DEV, seed=11, integer=True)
    g = torch.Generator(device=DEV).manual_seed(12)
    before = torch.randint(-64, 65, (w.P, w.S, w.N), generator=g, device=DEV).float()
    accum = before.clone()
    flags = _flags(w)
    pk.pk_gemm_rs_push(A, B, accum, flags, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, order)
    torch.cuda.synchronize()
    C = orc.local_partial(gen.bf16_bits(A), gen.bf16_bits(B))
    want, ready, counters = orc.push_share(C, before.cpu().numpy().astype(np.float64), w.P,
                                           w.rank, w.chunk_rows)
    assert np.array_equal(accum.cpu().numpy().astype(np.float64), want)
    assert np.array_equal(flags.cpu().numpy().view(np.uint32), orc.flag_words(ready, counters))


@pytest.mark.parametrize("integer", [True, False])
def test_push_equals_staged_bitwise(integer):
    """Owned accumulator pre-filled with the fp32 peer sum in slot order, the
    others with zeros: push(owned) == staged out and bf16(push(d)) == send."""
    w = gen.Workload("push_vs_staged", P=8, rank=3, M=2048, N=1024, K=384, chunk_rows=128,
                     ab_dist="int" if integer else "normal_sqrtk",
                     peer_dist="int" if integer else "normal", out_dtype="f32")
    A, B, peers = gen.make_inputs(w, DEV, seed=13, integer=integer)
    share = H.Share(w, "f32")
    H.run(share, A, B, peers)
    accum = torch.zeros((w.P, w.S, w.N), dtype=torch.float32, device=DEV)
    t = torch.zeros((w.S, w.N), dtype=torch.float32, device=DEV)
    for j in range(w.P - 1):                   # ascending slot order, from +0
        t = t + peers[j].float()
    accum[w.rank] = t
    flags = _flags(w)
    pk.pk_gemm_rs_push(A, B, accum, flags, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, 0)
    torch.cuda.synchronize()
    assert torch.equal(accum[w.rank].view(torch.int32), share.out.view(torch.int32))
    for d in range(w.P):
        if d == w.rank:
            continue
        slot = orc.slot_of_dest(d, w.rank)
        assert torch.equal(accum[d].to(torch.bfloat16).view(torch.int16),
                           share.send[slot].view(torch.int16)), d
    assert torch.equal(flags, share.flags)


def test_push_virtual_ranks_sum_into_shared_accumulators():
    """P ranks on one GPU push into the same accumulators, one after another
    and then all at once on separate streams; integer inputs make the sum
    independent of the order of the adds."""
    P, M, N, K = 4, 1024, 512, 256
    ws = [gen.Workload(f"vr{r}", P=P, rank=r, M=M, N=N, K=K, chunk_rows=64, ab_dist="int",
                       peer_dist="int", out_dtype="f32") for r in range(P)]
    ins = [gen.make_inputs(w, DEV, seed=20 + r, integer=True)[:2] for r, w in enumerate(ws)]
    full = sum(orc.local_partial(gen.bf16_bits(A), gen.bf16_bits(B)) for A, B in ins)
    want = full.reshape(P, M // P, N)
    for concurrent in (False, True):
        accum = torch.zeros((P, M // P, N), dtype=torch.float32, device=DEV)
        flags = [_flags(w) for w in ws]
        streams = [torch.cuda.Stream() for _ in ws] if concurrent else [None] * P
        torch.cuda.synchronize()
        for w, (A, B), f, s in zip(ws, ins, flags, streams):
            pk.pk_gemm_rs_push(A, B, accum, f, M, N, K, P, w.rank, w.chunk_rows, 2,
                               max_workgroups=64 if concurrent else 0, stream=s)
        torch.cuda.synchronize()
        assert np.array_equal(accum.cpu().numpy().astype(np.float64), want), concurrent


def test_push_rejects_bad_options():
    w = SHAPES[0]
    A, B, _ = gen.make_inputs(w, DEV, seed=1, integer=True)
    accum = torch.zeros((w.P, w.S, w.N), dtype=torch.float32, device=DEV)
    with pytest.raises(pk.PkError):
        pk.pk_gemm_rs_push(A, B, accum, _flags(w), w.M, w.N, w.K, w.P, w.rank, w.chunk_rows, 5)
    with pytest.raises(ValueError):
        pk.pk_gemm_rs_push(A, B, accum[:1], _flags(w), w.M, w.N, w.K, w.P, w.rank,
                           w.chunk_rows, 0)
    with pytest.raises(ValueError):
        pk.pk_gemm_rs_push(A, B, accum.to(torch.bfloat16), _flags(w), w.M, w.N, w.K, w.P,
                           w.rank, w.chunk_rows, 0)
