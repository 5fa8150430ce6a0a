"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Small and medium shapes compare every element; the 32768-wide workloads
compare sampled elements (each its own fp64 dot product in the oracle) plus
every flag word, and check invariance across tile orders and chunk sizes on
the full buffers.  Integer-valued twins must match bit for bit; real-valued
inputs must meet: relative Frobenius error <= 1e-3 and every element within
max(2 bf16 ulp, the float32 accumulation bound) of the oracle.
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
    pk.load()          # raises if the HIP library is not built
    yield
    torch.cuda.synchronize()


def _run_and_check(w, out_dtype, integer, seed=0, order=None, chunk_rows=None, **opts):
    A, B, peers = gen.make_inputs(w, DEV, seed=seed, integer=integer)
    share = H.Share(w, out_dtype, chunk_rows=chunk_rows)
    H.run(share, A, B, peers, tile_order=order, **opts)
    torch.cuda.synchronize()
    res = H.oracle_for(w, A, B, peers, chunk_rows=share.chunk_rows)
    if integer:
        H.compare_exact(res, share)
        return None
    mag = orc.local_partial_abs(gen.bf16_bits(A), gen.bf16_bits(B))
    return H.compare_real(res, mag, share, n_terms=w.K + w.P)


# ---------------------------------------------------------------- small / medium

def test_tiny_real():
    stats = _run_and_check(gen.WORKLOADS["tiny"], "f32", integer=False)
    print("tiny", stats)


def test_tiny_integer_twin_bit_exact():
    _run_and_check(gen.WORKLOADS["tiny"], "f32", integer=True)


MED = gen.Workload("medium", P=4, rank=1, M=1024, N=512, K=192, chunk_rows=64,
                   ab_dist="normal_sqrtk", peer_dist="normal", out_dtype="f32")


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("order", [0, 1, 2])
def test_medium_integer_every_config_and_order(config, order):
    _run_and_check(MED, "f32", integer=True, order=order, config=config)


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_medium_real_every_config(config, out_dtype):
    _run_and_check(MED, out_dtype, integer=False, config=config)


# shards of 200 rows, N = 328, K = 136: ragged row tiles in every shard,
# a ragged last column tile and a partial last K step for every config.
RAGGED = gen.Workload("ragged", P=3, rank=2, M=600, N=328, K=136, chunk_rows=40,
                      ab_dist="uniform1", peer_dist="uniform8", out_dtype="f32")


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("integer", [True, False])
def test_ragged_tails(config, integer):
    _run_and_check(RAGGED, "bf16", integer=integer, config=config)
    _run_and_check(RAGGED.with_(rank=0), "f32", integer=integer, config=config, order=2)


# The owned split: owned tiles of configuration 1 cut into 64 x 128 sub-tiles
# whose peer partials are read ahead; P = 8, 4 and 2 use 7, 3 and 1 slots.
SPLIT8 = gen.Workload("split8", P=8, rank=5, M=4096, N=768, K=200, chunk_rows=64,
                      ab_dist="normal_sqrtk", peer_dist="normal", out_dtype="f32")
SPLIT4 = gen.Workload("split4", P=4, rank=1, M=1200, N=328, K=136, chunk_rows=60,
                      ab_dist="uniform1", peer_dist="uniform8", out_dtype="f32")
SPLIT2 = gen.Workload("split2", P=2, rank=1, M=520, N=264, K=64, chunk_rows=52,
                      ab_dist="uniform1", peer_dist="uniform8", out_dtype="f32")
# P = 8 in one round: SPLIT8 (S = 512) and GATHER8 (S = 96: three row groups, a
# ragged last column tile, a partial last K step) take the gathered rows;
# ONE8 (S = 200, not a multiple of 32) takes the sub-tiles with the spare
# workgroups.
GATHER8 = gen.Workload("gather8", P=8, rank=2, M=768, N=1000, K=136, chunk_rows=32,
                       ab_dist="uniform1", peer_dist="uniform8", out_dtype="f32")
ONE8 = gen.Workload("one8", P=8, rank=6, M=1600, N=1000, K=136, chunk_rows=40,
                    ab_dist="uniform1", peer_dist="uniform8", out_dtype="f32")
# gathered rows with one k16 step of K (a single partial stage)
GATHER8K8 = gen.Workload("gather8k8", P=8, rank=0, M=1024, N=264, K=8, chunk_rows=64,
                         ab_dist="uniform1", peer_dist="uniform8", out_dtype="f32")
SPLITS = [SPLIT8, SPLIT4, SPLIT2, GATHER8, ONE8, GATHER8K8]


@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("w", SPLITS, ids=lambda w: w.name)
def test_owned_split_integer(w, order):
    _run_and_check(w, "f32", integer=True, order=order, config=1, owned_split=1)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("w", SPLITS, ids=lambda w: w.name)
def test_owned_split_real(w, out_dtype):
    _run_and_check(w, out_dtype, integer=False, order=2, config=1, owned_split=1)


@pytest.mark.parametrize("chunk_rows", [2, 4, 96])
def test_gathered_rows_chunk_sizes(chunk_rows):
    # chunks of 2 rows: a row group's 224 send rows touch 113 chunks, past the
    # 64 arrivals a wave issues at once
    _run_and_check(GATHER8, "f32", integer=True, chunk_rows=chunk_rows, config=1, owned_split=1)


def _random_cases(n, seed=20261203):
    """Seeded shapes drawn over the planner's choices: P = 2, 4 or 8 (P = 8
    with S a multiple of 32 takes the gathered rows, otherwise the sub-tiles),
    ragged N and K, any chunk size that divides S, every order, the default or
    a forced configuration and owned split."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        P = int(rng.choice([2, 4, 8, 8, 8]))
        S = int(rng.choice([32, 64, 96, 104, 160, 200, 256, 288, 320]))
        divs = [d for d in range(1, S + 1) if S % d == 0]
        chunk = int(rng.choice(divs))
        N = 8 * int(rng.integers(1, 140))
        K = 8 * int(rng.integers(0, 40))
        opts = {}
        cfg = int(rng.choice([0, 1, 1, 1, 4, 6]))
        if cfg:
            opts["config"] = cfg
        # configuration 6 rejects a forced split it cannot run
        split = int(rng.choice([0, -1] if cfg == 6 else [0, 1, 1, -1]))
        if split:
            opts["owned_split"] = split
        w = gen.Workload(f"rand{i}", P=P, rank=int(rng.integers(0, P)), M=P * S, N=N, K=K,
                         chunk_rows=chunk, ab_dist="uniform1", peer_dist="uniform8",
                         out_dtype=str(rng.choice(["f32", "bf16"])))
        cases.append((w, int(rng.integers(0, 3)), opts))
    return cases


def _random_gather_cases(n, seed=31):
    """Seeded shapes that take the gathered rows (P = 8, S a multiple of 32,
    configuration 1 with the owned split, every (row group, column tile) item
    on a workgroup of its own)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        S = 32 * int(rng.integers(1, 21))
        tn_max = max(1, min(5, 256 // (S // 32)))
        N = 8 * int(rng.integers(1, 32 * tn_max + 1))
        divs = [d for d in range(1, S + 1) if S % d == 0]
        w = gen.Workload(f"rgather{i}", P=8, rank=int(rng.integers(0, 8)), M=8 * S, N=N,
                         K=8 * int(rng.integers(0, 48)), chunk_rows=int(rng.choice(divs)),
                         ab_dist="uniform1", peer_dist="uniform8",
                         out_dtype=str(rng.choice(["f32", "bf16"])))
        cases.append((w, int(rng.integers(0, 3)), {"config": 1, "owned_split": 1}))
    return cases


RANDOM_CASES = _random_cases(16) + _random_gather_cases(8)


@pytest.mark.parametrize("w,order,opts", RANDOM_CASES, ids=lambda c: getattr(c, "name", None))
def test_random_shapes_integer_exact(w, order, opts):
    print(w, order, opts, flush=True)
    _run_and_check(w, w.out_dtype, integer=True, order=order, **opts)


@pytest.mark.parametrize("w,order,opts", RANDOM_CASES[::2], ids=lambda c: getattr(c, "name", None))
def test_random_shapes_real(w, order, opts):
    print(w, order, opts, flush=True)
    print(_run_and_check(w, w.out_dtype, integer=False, seed=7, order=order, **opts))


@pytest.mark.parametrize("w", [SPLIT8, GATHER8, ONE8], ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_owned_split_matches_whole_tiles_bitwise(w, out_dtype):
    # whole tiles, the P = 8 one-round schedule (gathered rows or sub-tiles),
    # and the multi-round walk of sub-tiles (a grid of 7 workgroups)
    A, B, peers = gen.make_inputs(w, DEV, seed=11)
    outs = []
    for split, grid in ((-1, 0), (1, 0), (1, 7)):
        share = H.Share(w, out_dtype)
        H.run(share, A, B, peers, config=1, owned_split=split, max_workgroups=grid)
        torch.cuda.synchronize()
        assert torch.equal(share.flags.cpu(), torch.from_numpy(
            H.expected_flags(w, w.chunk_rows).view(np.int32)))
        outs.append((share.send.view(torch.int16).clone(),
                     share.out.view(torch.int16 if out_dtype == "bf16" else torch.int32).clone()))
    for o in outs[1:]:
        assert torch.equal(outs[0][0], o[0]) and torch.equal(outs[0][1], o[1])


@pytest.mark.parametrize("chunk_rows", [8, 40, 200])
def test_chunk_sizes_ragged(chunk_rows):
    _run_and_check(RAGGED, "f32", integer=True, chunk_rows=chunk_rows)


@pytest.mark.parametrize("P,rank,M", [(4, 2, 256), (8, 5, 512)])   # P = 8: gathered rows
def test_k_zero_gives_peer_sum(P, rank, M):
    w = gen.Workload("k0", P=P, rank=rank, M=M, N=64, K=0, chunk_rows=16,
                     ab_dist="uniform1", peer_dist="int", out_dtype="f32")
    A = torch.empty((w.M, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((0, w.N), dtype=torch.bfloat16, device=DEV)
    _, _, peers = gen.make_inputs(w.with_(K=8), DEV, seed=4, integer=True)
    share = H.Share(w, "f32")
    H.run(share, A, B, peers)
    torch.cuda.synchronize()
    send, out, _, flags = H.host(share)
    expect = orc.bf16_bits_to_f64(gen.bf16_bits(peers)).sum(axis=0)
    assert np.array_equal(out, expect)
    assert np.all(send == 0)                       # +0.0 everywhere
    assert np.array_equal(flags, H.expected_flags(w, w.chunk_rows))


def test_p1_is_plain_gemm():
    w = gen.Workload("p1", P=1, rank=0, M=320, N=192, K=96, chunk_rows=64,
                     ab_dist="uniform1", peer_dist="int", out_dtype="f32")
    _run_and_check(w, "f32", integer=True)
    _run_and_check(w, "bf16", integer=False)


def test_empty_m_and_n_are_no_ops():
    w = gen.Workload("empty", P=2, rank=1, M=0, N=64, K=64, chunk_rows=0,
                     ab_dist="uniform1", peer_dist="int", out_dtype="f32")
    z = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    assert pk.pk_gemm_rs_local(z, z, z, z, torch.empty(0, device=DEV), None, 0, 64, 64, 2, 1, 0, 0) == 0
    assert pk.pk_gemm_rs_local(z, z, z, z, torch.empty(0, device=DEV), None, 64, 0, 64, 2, 1, 32, 0) == 0
    torch.cuda.synchronize()
    del w


def test_invalid_arguments_raise_before_launch():
    w = gen.WORKLOADS["tiny"]
    A, B, peers = gen.make_inputs(w, DEV, seed=0)
    share = H.Share(w, "f32")
    with pytest.raises(pk.PkError):
        pk.pk_gemm_rs_local(A, B, peers, share.send, share.out, share.flags,
                            w.M, w.N, w.K, w.P, 5, w.chunk_rows, 0)
    with pytest.raises(pk.PkError):
        pk.pk_gemm_rs_local(A, B, peers, share.send, share.out, share.flags,
                            w.M, w.N, w.K, w.P, 0, 48, 0)
    torch.cuda.synchronize()
    assert share.canaries_intact()
    assert torch.all(share.flags == 0)             # nothing ran


@pytest.mark.parametrize("kind", ["row_lo", "row_hi", "col"])
def test_placement_probes(kind):
    w = gen.Workload("probe", P=8, rank=5, M=8192, N=520, K=16, chunk_rows=128,
                     ab_dist="int", peer_dist="int", out_dtype="f32")
    A, B, peers = gen.make_probe_inputs(w, kind, DEV)
    share = H.Share(w, "bf16")
    H.run(share, A, B, peers, tile_order=2)
    torch.cuda.synchronize()
    res = H.oracle_for(w, A, B, peers)
    H.compare_exact(res, share)


def test_gemm_only_mode():
    w = gen.Workload("gemm", P=8, rank=0, M=1024, N=768, K=256, chunk_rows=128,
                     ab_dist="int", peer_dist="int", out_dtype="bf16")
    A, B, _ = gen.make_inputs(w, DEV, seed=9, integer=True)
    out = torch.full((w.M, w.N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    pk.pk_gemm_rs_local_ex(A, B, None, None, out, None, w.M, w.N, w.K, w.P, 0, 0, 0, 1,
                           gemm_only=True)
    torch.cuda.synchronize()
    C = orc.local_partial(gen.bf16_bits(A), gen.bf16_bits(B))
    assert np.array_equal(gen.bf16_bits(out), orc.f64_to_bf16_bits(C))


# ---------------------------------------------------------------- comm-dominant, full size

CD = gen.WORKLOADS["comm_dominant"]


def test_comm_dominant_real_full():
    stats = _run_and_check(CD, "f32", integer=False)
    print("comm_dominant", stats)


def test_comm_dominant_integer_full():
    _run_and_check(CD, "f32", integer=True, order=1)


def test_outputs_invariant_across_orders_chunks_and_runs():
    A, B, peers = gen.make_inputs(CD, DEV, seed=5)
    ref = None
    for chunk in (64, 128, 256, 512):
        for order in (0, 1, 2):
            for grid, split, sig, pol in ((0, 0, 0, 0), (37, 0, 1, 1), (0, -1, 3, 2),
                                          (100, 1, 1000, 1)):
                share = H.Share(CD, "f32", chunk_rows=chunk)
                H.run(share, A, B, peers, tile_order=order, max_workgroups=grid,
                      owned_split=split, signal_batch=sig, store_policy=pol)
                torch.cuda.synchronize()
                assert torch.equal(share.flags.cpu(), torch.from_numpy(
                    H.expected_flags(CD, chunk).view(np.int32)))
                cur = (share.send.view(torch.int16).clone(), share.out.clone())
                if ref is None:
                    ref = cur
                else:
                    assert torch.equal(cur[0], ref[0]), (chunk, order, grid, split)
                    assert torch.equal(cur[1].view(torch.int32), ref[1].view(torch.int32))
    # repeat calls on the same buffers, flags never cleared: each call raises
    # every ready word by one and leaves the counters at zero
    share = H.Share(CD, "f32")
    for n in range(1, 4):
        H.run(share, A, B, peers, owned_split=(0, -1, 1)[n - 1])
        torch.cuda.synchronize()
        assert torch.equal(share.flags.cpu(), torch.from_numpy(
            H.expected_flags(CD, CD.chunk_rows, calls=n).view(np.int32)))
    assert torch.equal(share.send.view(torch.int16), ref[0])
    assert torch.equal(share.out.view(torch.int32), ref[1].view(torch.int32))


@pytest.mark.parametrize("order", [0, 1, 2])
def test_two_per_cu_schedule(order):
    """Configuration 6 at P = 8 runs the owned split with two workgroups per
    CU (send tiles on the first half of the grid, owned sub-tiles then send
    tiles on the second): bitwise the share of configuration 1, and the
    oracle's on the integer twin."""
    w = gen.WORKLOADS["comm_dominant"]
    A, B, peers = gen.make_inputs(w, DEV, seed=81 + order)
    ref = H.Share(w, "f32")
    H.run(ref, A, B, peers, tile_order=order, config=1)
    got = H.Share(w, "f32")
    H.run(got, A, B, peers, tile_order=order, config=6)
    torch.cuda.synchronize()
    assert torch.equal(got.send.view(torch.int16), ref.send.view(torch.int16))
    assert torch.equal(got.out.view(torch.int32), ref.out.view(torch.int32))
    assert torch.equal(got.flags, ref.flags) and got.canaries_intact()
    Ai, Bi, Pi = gen.make_inputs(w, DEV, seed=91 + order, integer=True)
    sh = H.Share(w, "f32")
    H.run(sh, Ai, Bi, Pi, tile_order=order, config=6)
    torch.cuda.synchronize()
    H.compare_exact(orc.gemm_rs_oracle(gen.bf16_bits(Ai), gen.bf16_bits(Bi), gen.bf16_bits(Pi),
                                       w.P, w.rank, w.chunk_rows), sh)


def test_bound_call_relaunches_the_same_share():
    w = gen.Workload("bound", P=4, rank=2, M=1024, N=768, K=320, chunk_rows=64,
                     ab_dist="int", peer_dist="int", out_dtype="f32")
    A, B, peers = gen.make_inputs(w, DEV, seed=21, integer=True)
    share = H.Share(w, "f32")
    call = pk.BoundCall(A, B, peers, share.send, share.out, share.flags, w.M, w.N, w.K, w.P,
                        w.rank, w.chunk_rows, 2, 0, owned_split=1)
    ready = None
    for n in (1, 2):
        call()
        torch.cuda.synchronize()
        res = orc.gemm_rs_oracle(gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers), w.P,
                                 w.rank, w.chunk_rows, ready_before=ready)
        H.compare_exact(res, share)   # integer inputs: every output and flag exact
        assert np.array_equal(share.flags.cpu().numpy().view(np.uint32),
                              H.expected_flags(w, w.chunk_rows, calls=n))
        ready = res.ready
    with pytest.raises(ValueError):
        pk.BoundCall(A, B, peers, share.send, share.out[:10], share.flags, w.M, w.N, w.K, w.P,
                     w.rank, w.chunk_rows, 2, 0)


def test_virtual_ranks_reduce_scatter_on_one_gpu():
    """All P ranks on one GPU: each rank's send slots feed the others' peers.

    The concatenated shards must equal the sum over ranks of their partials
    (each sent partial rounded to bf16 once), which for integer inputs is the
    exact stacked GEMM [A_1..A_P][B_1;..;B_P]."""
    P = 4
    w = gen.Workload("vr", P=P, rank=0, M=1024, N=384, K=128, chunk_rows=64,
                     ab_dist="int", peer_dist="int", out_dtype="f32")
    As, Bs = [], []
    for q in range(P):
        A, B, _ = gen.make_inputs(w, DEV, seed=100 + 10 * q, integer=True)
        As.append(A)
        Bs.append(B)
    zero = torch.zeros((P - 1, w.S, w.N), dtype=torch.bfloat16, device=DEV)
    sends = []
    for q in range(P):
        sh = H.Share(w.with_(rank=q), "f32")
        H.run(sh, As[q], Bs[q], zero, tile_order=q % 3)
        sends.append(sh.send.clone())
    outs = []
    for r in range(P):
        peers = torch.stack([sends[q][r if r < q else r - 1] for q in range(P) if q != r])
        sh = H.Share(w.with_(rank=r), "f32")
        H.run(sh, As[r], Bs[r], peers.contiguous(), tile_order=(r + 1) % 3)
        outs.append(sh.out.clone())
    torch.cuda.synchronize()
    full = torch.cat(outs).cpu().numpy().astype(np.float64)
    Acat = np.concatenate([gen.bf16_bits(a) for a in As], axis=1)
    Bcat = np.concatenate([gen.bf16_bits(b) for b in Bs], axis=0)
    assert np.array_equal(full, orc.local_partial(Acat, Bcat))


# ---------------------------------------------------------------- 32768 workloads
# (compared with the oracle at stratified positions and on complete tiles in
# test_gpu_full_size.py)


def test_large_k_sweep_invariance():
    """The 12 schedule points of the large-K workload give identical bits."""
    w = gen.WORKLOADS["large_k"]
    A, B, peers = gen.make_inputs(w, DEV, seed=2)
    ref = None
    for chunk in w.sweep_chunk_rows:
        share = H.Share(w, "bf16", chunk_rows=chunk)
        for order in (0, 1, 2):
            share.reset_flags()
            H.run(share, A, B, peers, tile_order=order)
            torch.cuda.synchronize()
            assert np.array_equal(share.flags.cpu().numpy().view(np.uint32),
                                  H.expected_flags(w, chunk))
            if ref is None:
                ref = (share.send.view(torch.int16).clone(), share.out.view(torch.int16).clone())
            else:
                assert torch.equal(share.send.view(torch.int16), ref[0]), (chunk, order)
                assert torch.equal(share.out.view(torch.int16), ref[1]), (chunk, order)
        del share
