"""Full-size GPU parity through the C ABI.

* The three 32768-wide workloads, real-valued and integer twin, compared with
  the oracle at stratified positions (4 in every 256 x 256 tile of every
  shard, 1 in every 64 x 128 sub-tile of the owned shard, plus shard, chunk
  and tile edges: about 82k positions, every tile met) and on complete tiles
  (the last row tile and the last column tile of every shard, and owned
  tiles), so a fault confined to one tile or to high row and column indices
  cannot pass.
* The reduce-scatter as a whole: all P = 8 ranks simulated on one GPU, each
  rank's send chunks fed to the others as their peer partials.  The owner's
  result is the sum of every rank's partial for its shard ("ParallelKittens:
  Systematic and Practical Simplification of Multi-GPU AI Kernels", section 3
  "Scheduling Analysis"): at the comm-dominant shape checked in full against
  the oracle run for every rank and against the stacked GEMM
  [A_1 .. A_P][B_1; ..; B_P]; at the near-threshold shape at stratified
  positions of every shard.

With PK_PARITY_RECORD set, each check appends its statistics (strict 2-ulp
count, elements that needed the rounding bound, exact-match fraction of the
send values, largest error relative to the bound) as a JSON line to that
file.
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


def _edge_tiles(w, tile=256):
    """(shard, row tile, column tile): the last row tile of every shard at the
    first and last column tile, its first row tile at the last column tile,
    and an interior owned tile."""
    tm, tn = -(-w.S // tile), -(-w.N // tile)
    tiles = []
    for d in range(w.P):
        tiles += [(d, tm - 1, 0), (d, tm - 1, tn - 1), (d, 0, tn - 1)]
    tiles.append((w.rank, tm // 2, tn // 2))
    return tiles


@pytest.mark.parametrize("integer", [False, True], ids=["real", "integer_twin"])
@pytest.mark.parametrize("name", ["near_threshold", "compute_bound", "large_k"])
def test_large_workload_stratified(name, integer):
    w = gen.WORKLOADS[name]
    kind = "integer twin" if integer else "real"
    print(f"[{name} {kind}] generating", flush=True)
    A, B, peers = gen.make_inputs(w, DEV, seed=1 if integer else 0, integer=integer)
    share = H.Share(w, w.out_dtype)
    print(f"[{name} {kind}] running", flush=True)
    H.run(share, A, B, peers)
    torch.cuda.synchronize()
    assert np.array_equal(share.flags.cpu().numpy().view(np.uint32),
                          H.expected_flags(w, w.chunk_rows))
    assert share.canaries_intact()
    rows, cols = H.stratified_positions(w, seed=10 + integer)
    print(f"[{name} {kind}] checking {rows.size} positions", flush=True)
    st = H.check_positions(w, A, B, peers, share, rows, cols, integer)
    H.check_tiles(w, A, B, peers, share, _edge_tiles(w), integer)
    st["complete_tiles"] = len(_edge_tiles(w))
    H.record(f"{name} {kind}", st)
    del A, B, peers, share
    torch.cuda.empty_cache()


def _virtual_ranks(w, seed, orders=(0, 1, 2)):
    """Run all P ranks on one GPU: every rank sends (zero peers), then every
    rank reduces with the others' send chunks as its peers.  Returns the
    operands, the send buffers and the owned shards, all on the device."""
    P = w.P
    ops = [gen.make_operands(w, DEV, seed=seed + 10 * q, integer=True) for q in range(P)]
    zero = torch.zeros((P - 1, w.S, w.N), dtype=torch.bfloat16, device=DEV)
    sends = []
    for q in range(P):
        sh = H.Share(w.with_(rank=q), w.out_dtype)
        H.run(sh, ops[q][0], ops[q][1], zero, tile_order=orders[q % len(orders)])
        sends.append(sh.send.clone())
        del sh
    del zero
    outs = []
    for r in range(P):
        peers = torch.stack([sends[q][r if r < q else r - 1] for q in range(P) if q != r])
        sh = H.Share(w.with_(rank=r), w.out_dtype)
        H.run(sh, ops[r][0], ops[r][1], peers, tile_order=orders[(r + 1) % len(orders)])
        torch.cuda.synchronize()
        assert np.array_equal(sh.flags.cpu().numpy().view(np.uint32),
                              H.expected_flags(w, w.chunk_rows))
        assert sh.canaries_intact()
        outs.append(sh.out.clone())
        del sh, peers
    torch.cuda.synchronize()
    return ops, sends, outs


def test_virtual_ranks_comm_dominant_shape_in_full():
    """P = 8 ranks at M = N = 4096, K = 512, integer twin, fp32 out: every
    send buffer and every owned shard equals the oracle's, and the
    concatenated shards equal the stacked GEMM wherever no rank's partial
    needed rounding to bf16 on its way to the owner."""
    w = gen.WORKLOADS["comm_dominant"].with_(ab_dist="int", peer_dist="int")
    P, S = w.P, w.S
    ops, sends, outs = _virtual_ranks(w, seed=300)
    Cs = [orc.local_partial(gen.bf16_bits(A), gen.bf16_bits(B)) for A, B in ops]
    zeros = np.zeros((P - 1, S, w.N))
    sent = []
    for q in range(P):
        res = orc.reduce_scatter_share(Cs[q], zeros, P, q, w.chunk_rows)
        assert np.array_equal(gen.bf16_bits(sends[q]), res.send_bits), f"rank {q} send"
        sent.append(res.send_bits)
    full = []
    for r in range(P):
        peers = np.stack([orc.bf16_bits_to_f64(sent[q][orc.slot_of_dest(r, q)])
                          for q in range(P) if q != r])
        res = orc.reduce_scatter_share(Cs[r], peers, P, r, w.chunk_rows)
        got = outs[r].cpu().numpy().astype(np.float64)
        assert np.array_equal(got, res.out), f"rank {r} owned shard"
        full.append(got)
    full = np.concatenate(full)
    stacked = orc.local_partial(np.concatenate([gen.bf16_bits(A) for A, _ in ops], axis=1),
                                np.concatenate([gen.bf16_bits(B) for _, B in ops], axis=0))
    exact = np.all(np.stack([np.abs(C) <= 256 for C in Cs]), axis=0)   # bf16 holds them
    assert exact.mean() > 0.99
    assert np.array_equal(full[exact], stacked[exact])
    H.record("virtual ranks comm_dominant shape (full)",
             dict(elements=int(full.size), stacked_identity_elements=int(exact.sum())))


def test_virtual_ranks_near_threshold_shape_sampled():
    """P = 8 ranks at M = N = 32768, K = 2048, integer twin, bf16 out: at
    stratified positions of every shard the owner's value is
    bf16(C_r + sum over the other ranks q, in slot order, of bf16(C_q))."""
    w = gen.WORKLOADS["near_threshold"].with_(ab_dist="int", peer_dist="int")
    P, S = w.P, w.S
    print("[virtual ranks near_threshold] running 16 calls", flush=True)
    ops, sends, outs = _virtual_ranks(w, seed=400)
    del sends
    torch.cuda.empty_cache()
    checked = 0
    for r in range(P):
        rows, cols = H.stratified_positions(w, seed=50 + r, per_tile=2, ranks=[r])
        # every rank's partial at these positions
        parts = []
        for q in range(P):
            v, _ = orc.partial_elements(H._gather_rows(ops[q][0], rows),
                                        H._gather_cols(ops[q][1], cols))
            parts.append(v)
        peer_bits = np.stack([orc.f64_to_bf16_bits(parts[q]) for q in range(P) if q != r])
        val, _ = orc.owned_elements(parts[r], np.zeros_like(parts[r]), peer_bits)
        lr = torch.from_numpy(rows - r * S).to(DEV)
        got = gen.bf16_bits(outs[r][lr, torch.from_numpy(cols).to(DEV)])
        assert np.array_equal(got, orc.f64_to_bf16_bits(val)), f"rank {r}"
        checked += rows.size
        print(f"[virtual ranks near_threshold] rank {r}: {rows.size} positions exact", flush=True)
    H.record("virtual ranks near_threshold shape (stratified)", dict(positions=checked))
