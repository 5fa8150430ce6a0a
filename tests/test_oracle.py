"""Pins for the fp64 oracle: closed forms, brute force, identities, special
cases and library routines other than the oracle's own.  CPU only.

Each pin is written so that a plausible slip in the oracle (a dropped term, a
wrong sign, a swapped slot, a transposed operand, a double rounding) fails at
least one of them; ``test_planted_mistakes_are_caught`` plants such slips in
the oracle and checks that the pins notice.
"""
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle.gemm_rs_oracle as orc
from gemm_reduce_scatter_amd import inputs as gen
from gemm_reduce_scatter_amd import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 format

def _bits_from_f32(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0] >> 16


def test_bf16_decode_closed_forms():
    cases = {0x0000: 0.0, 0x3F80: 1.0, 0x4000: 2.0, 0xC000: -2.0, 0x3F81: 1.0 + 2 ** -7,
             0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0x4380: 256.0, 0xBF00: -0.5}
    got = orc.bf16_bits_to_f64(np.array(list(cases), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(cases.values())))
    assert np.isinf(orc.bf16_bits_to_f64(np.array([0x7F80], np.uint16)))[0]
    assert np.signbit(orc.bf16_bits_to_f64(np.array([0x8000], np.uint16)))[0]


def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_round_trip_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = orc.bf16_bits_to_f64(bits)
    finite = ~np.isnan(vals)
    assert np.array_equal(orc.f64_to_bf16_bits(vals[finite]), bits[finite])


def test_bf16_encode_vs_torch_on_float32():
    # torch's float32 -> bfloat16 conversion rounds to nearest even; for
    # float32 inputs rounding from float64 must agree with it exactly.
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),    # subnormal range
        (rng.uniform(-3.3e38, 3.3e38, 20000)).astype(np.float32),   # near overflow
        # exact ties: low 16 bits 0x8000
        ((rng.integers(0, 2 ** 15, 20000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f64_to_bf16_bits(x.astype(np.float64)), ref)


def test_bf16_encode_ties_and_no_double_rounding():
    # halfway between 1 and 1+2^-7 -> even (1.0)
    assert orc.f64_to_bf16_bits(np.array([1 + 2 ** -8]))[0] == 0x3F80
    # halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6
    assert orc.f64_to_bf16_bits(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82
    # just above the tie: must round up.  Rounding to float32 first would land
    # exactly on the tie and then go to even (0x3F80): a double rounding.
    assert orc.f64_to_bf16_bits(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81
    assert orc.f64_to_bf16_bits(np.array([-(1 + 2 ** -8 + 2 ** -40)]))[0] == 0xBF81
    # overflow: the tie above the largest finite value rounds to infinity
    big = (2 - 2 ** -8) * 2.0 ** 127
    assert orc.f64_to_bf16_bits(np.array([big]))[0] == 0x7F80
    assert orc.f64_to_bf16_bits(np.array([np.nextafter(big, 0)]))[0] == 0x7F7F
    assert orc.f64_to_bf16_bits(np.array([-0.0]))[0] == 0x8000
    assert orc.f64_to_bf16_bits(np.array([2.0 ** -134]))[0] == 0x0000      # tie -> even 0
    assert orc.f64_to_bf16_bits(np.array([3 * 2.0 ** -134]))[0] == 0x0002  # tie -> even 2
    assert orc.f64_to_bf16_bits(np.array([np.nan]))[0] == 0x7FC0


def test_ulp_closed_forms():
    assert orc.ulp_bf16(np.array([1.0]))[0] == 2 ** -7
    assert orc.ulp_bf16(np.array([1.99]))[0] == 2 ** -7
    assert orc.ulp_bf16(np.array([256.0]))[0] == 2.0
    assert orc.ulp_bf16(np.array([-3.0]))[0] == 2 ** -6
    assert orc.ulp_bf16(np.array([0.0]))[0] == 2.0 ** -133
    assert orc.ulp_bf16(np.array([2.0 ** -130]))[0] == 2.0 ** -133


# ---------------------------------------------------------------- the GEMM

def _bits(a: np.ndarray) -> np.ndarray:
    """bf16 bits of small integer-valued float arrays (exact)."""
    return np.array([_bits_from_f32(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def test_local_partial_brute_force_integers():
    rng = np.random.default_rng(7)
    A = rng.integers(-3, 4, (5, 7))
    B = rng.integers(-3, 4, (7, 3))
    C = orc.local_partial(_bits(A), _bits(B))
    for i in range(5):
        for n in range(3):
            s = 0
            for k in range(7):
                s += int(A[i, k]) * int(B[k, n])
            assert C[i, n] == s


def test_local_partial_nonsquare_orientation():
    # A is 2 x 3, B is 3 x 4: a transposed operand would not even conform,
    # and the row/column roles are pinned by a hand-computed product.
    A = np.array([[1, 0, 2], [0, 1, 0]])
    B = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [-1, 0, 1, 0]])
    C = orc.local_partial(_bits(A), _bits(B))
    assert np.array_equal(C, np.array([[-1, 2, 5, 4], [5, 6, 7, 8]]))


def test_local_partial_real_values_vs_exact_rational():
    # Products of bf16 numbers are exact in float64; sums of 4 such products
    # with magnitudes near 1 are exact too, so fractions.Fraction pins it.
    from fractions import Fraction
    rng = np.random.default_rng(3)
    A = rng.standard_normal((3, 4)).astype(np.float32)
    B = rng.standard_normal((4, 2)).astype(np.float32)
    Ab = torch.from_numpy(A).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    Bb = torch.from_numpy(B).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    Af = orc.bf16_bits_to_f64(Ab)
    Bf = orc.bf16_bits_to_f64(Bb)
    C = orc.local_partial(Ab, Bb)
    for i in range(3):
        for n in range(2):
            exact = sum(Fraction(float(Af[i, k])) * Fraction(float(Bf[k, n])) for k in range(4))
            assert C[i, n] == float(exact)


def test_empty_inner_dimension():
    C = orc.local_partial(np.zeros((4, 0), np.uint16), np.zeros((0, 3), np.uint16))
    assert C.shape == (4, 3) and not np.any(C)


# ---------------------------------------------------------------- reduce-scatter

def _int_mats(rng, M, K, N):
    return rng.integers(-2, 3, (M, K)), rng.integers(-2, 3, (K, N))


def _virtual_ranks(As, Bs, P, chunk_rows):
    """Run the oracle for every rank, feeding each rank the other ranks' sends."""
    M = As[0].shape[0]
    S = M // P
    Cs = [orc.local_partial(_bits(As[q]), _bits(Bs[q])) for q in range(P)]
    # sends[q][d] = what rank q sends to rank d (bf16 bits)
    sends = []
    for q in range(P):
        r = orc.reduce_scatter_share(Cs[q], np.zeros((P - 1, S, Cs[q].shape[1])), P, q, chunk_rows)
        sends.append({orc.dest_of_slot(j, q): r.send_bits[j] for j in range(P - 1)})
    outs = []
    for r in range(P):
        peers = np.stack([orc.bf16_bits_to_f64(sends[q][r]) for q in range(P) if q != r]) \
            if P > 1 else np.zeros((0, S, Cs[r].shape[1]))
        outs.append(orc.reduce_scatter_share(Cs[r], peers, P, r, chunk_rows))
    return outs


@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_concatenated_shards_equal_stacked_gemm(P):
    # sum_p A_p B_p = [A_1 .. A_P] [B_1; ..; B_P]: one textbook GEMM with K' = P K,
    # evaluated here with Python integers.
    rng = np.random.default_rng(11 + P)
    M, K, N = 4 * P, 3, 5
    As, Bs = zip(*[_int_mats(rng, M, K, N) for _ in range(P)])
    outs = _virtual_ranks(As, Bs, P, chunk_rows=2)
    full = np.concatenate([o.out for o in outs], axis=0)
    Acat = np.concatenate(As, axis=1)
    Bcat = np.concatenate(Bs, axis=0)
    expect = np.array([[sum(int(Acat[i, k]) * int(Bcat[k, n]) for k in range(P * K))
                        for n in range(N)] for i in range(M)])
    assert np.array_equal(full, expect)


def test_each_rank_keeps_only_its_shard():
    # Rank r's output must not depend on other shards' rows of its own partial.
    rng = np.random.default_rng(5)
    P, M, K, N = 4, 8, 3, 4
    S = M // P
    A, B = _int_mats(rng, M, K, N)
    C = orc.local_partial(_bits(A), _bits(B))
    for r in range(P):
        res = orc.reduce_scatter_share(C, np.zeros((P - 1, S, N)), P, r, 1)
        C2 = C.copy()
        C2[np.arange(M) // S != r] += 1000.0
        res2 = orc.reduce_scatter_share(C2, np.zeros((P - 1, S, N)), P, r, 1)
        assert np.array_equal(res.out, res2.out)
        assert np.array_equal(res.out, C[r * S:(r + 1) * S])


def test_p1_reduces_to_gemm():
    rng = np.random.default_rng(9)
    A, B = _int_mats(rng, 6, 4, 5)
    res = orc.gemm_rs_oracle(_bits(A), _bits(B), np.zeros((0, 6, 5), np.uint16), 1, 0, 3)
    assert res.send_bits.shape == (0, 6, 5)
    assert np.array_equal(res.out, A @ B)
    assert res.flags.size == 0


def test_owned_sum_adds_every_peer_once():
    P, S, N = 4, 2, 3
    C = np.zeros((P * S, N))
    peers = np.stack([np.full((S, N), 10.0 ** j) for j in range(P - 1)])
    for rank in range(P):
        res = orc.reduce_scatter_share(C, peers, P, rank, 1)
        assert np.all(res.out == 111.0)


def test_send_slots_skip_self_in_rank_order():
    P, S, N = 4, 2, 2
    C = np.repeat(np.arange(P * S, dtype=np.float64)[:, None], N, axis=1)
    for rank in range(P):
        res = orc.reduce_scatter_share(C, np.zeros((P - 1, S, N)), P, rank, 1)
        dests = [d for d in range(P) if d != rank]
        for j, d in enumerate(dests):
            got = orc.bf16_bits_to_f64(res.send_bits[j])
            assert np.array_equal(got[:, 0], np.arange(d * S, (d + 1) * S))
        assert np.array_equal(res.out[:, 0], np.arange(rank * S, (rank + 1) * S))


@pytest.mark.parametrize("kind", ["row_lo", "row_hi", "col"])
def test_placement_probes(kind):
    w = gen.Workload("probe", P=4, rank=2, M=1024, N=40, K=8, chunk_rows=64,
                     ab_dist="int", peer_dist="int", out_dtype="f32")
    A, B, peers = gen.make_probe_inputs(w, kind)
    res = orc.gemm_rs_oracle(gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers),
                             w.P, w.rank, w.chunk_rows)
    S = w.S
    for j in range(w.P - 1):
        d = j if j < w.rank else j + 1
        vals = orc.bf16_bits_to_f64(res.send_bits[j])
        rows = np.arange(d * S, (d + 1) * S)[:, None]
        cols = np.arange(w.N)[None, :]
        if kind == "row_lo":
            exp = np.broadcast_to(rows % 256, vals.shape)
        elif kind == "row_hi":
            exp = np.broadcast_to((rows // 256) % 256, vals.shape)
        else:
            exp = np.broadcast_to(cols % 256, vals.shape)
        assert np.array_equal(vals, exp)


def test_identity_rows_copy_b_into_every_send_chunk():
    # A = [I; I; ...] (K = S) makes every destination's rows equal B exactly.
    P, rank, S, N = 4, 1, 8, 16
    A = np.concatenate([np.eye(S)] * P, axis=0)
    rng = np.random.default_rng(2)
    Bf = rng.standard_normal((S, N)).astype(np.float32)
    Bb = torch.from_numpy(Bf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    res = orc.gemm_rs_oracle(_bits(A), Bb, np.zeros((P - 1, S, N), np.uint16), P, rank, 4)
    for j in range(P - 1):
        assert np.array_equal(res.send_bits[j], Bb)


def test_flags_closed_form():
    rng = np.random.default_rng(4)
    A, B = _int_mats(rng, 64, 4, 8)
    res = orc.gemm_rs_oracle(_bits(A), _bits(B), np.zeros((3, 16, 8), np.uint16), 4, 3, 4)
    assert res.ready.shape == (3, 4) and np.all(res.ready == 1)
    assert res.counters.shape == (3, 4) and np.all(res.counters == 0)
    # device order: 12 ready words, then 12 counters, one per 32-word line
    assert np.array_equal(res.flags, np.array([1] * 12 + [0] * (12 * 32), np.uint32))
    res.counters[1, 2] = 5   # a counter sits at the start of its own line
    assert res.flags[12 + 32 * 6] == 5 and res.flags.sum() == 12 + 5


def test_ready_words_count_calls():
    """Signal adds one per call (ParallelKittens summary page, "The Eight PK
    Primitives": signal adds to a counter, wait waits for it to reach a value)."""
    rng = np.random.default_rng(5)
    A, B = _int_mats(rng, 64, 4, 8)
    peers = np.zeros((3, 16, 8), np.uint16)
    before = np.array([[0, 1, 2, 7], [5, 5, 5, 5], [0xFFFFFFFF, 0, 3, 9]], np.uint32)
    res = orc.gemm_rs_oracle(_bits(A), _bits(B), peers, 4, 3, 4, ready_before=before)
    assert np.array_equal(res.ready, np.array([[1, 2, 3, 8], [6, 6, 6, 6], [0, 1, 4, 10]],
                                              np.uint32))
    assert np.all(res.counters == 0)
    with pytest.raises(ValueError):
        orc.gemm_rs_oracle(_bits(A), _bits(B), peers, 4, 3, 4, ready_before=before[:2])


def test_bad_arguments_rejected():
    C = np.zeros((8, 2))
    with pytest.raises(ValueError):
        orc.reduce_scatter_share(C, np.zeros((2, 2, 2)), 3, 0, 1)     # M % P
    with pytest.raises(ValueError):
        orc.reduce_scatter_share(C, np.zeros((3, 2, 2)), 4, 4, 1)     # rank
    with pytest.raises(ValueError):
        orc.reduce_scatter_share(C, np.zeros((3, 2, 2)), 4, 0, 3)     # chunk
    with pytest.raises(ValueError):
        orc.slot_of_dest(1, 1)


# ---------------------------------------------------------------- sampled path

def test_sampled_elements_match_full_oracle():
    w = gen.WORKLOADS["tiny"].with_(P=4, rank=1, M=64, N=48, K=40, chunk_rows=4)
    A, B, peers = gen.make_inputs(w, seed=3)
    Ab, Bb, Pb = gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers)
    full = orc.gemm_rs_oracle(Ab, Bb, Pb, w.P, w.rank, w.chunk_rows)
    rows = np.arange(w.M).repeat(w.N)
    cols = np.tile(np.arange(w.N), w.M)
    kind, val, mag = orc.gemm_rs_elements(Ab, Bb, Pb, w.P, w.rank, rows, cols)
    S = w.S
    own = (rows // S) == w.rank
    assert np.array_equal(kind.astype(bool), own)
    np.testing.assert_allclose(val[own], full.out.ravel(), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(val[~own], full.C.ravel()[~own], rtol=1e-14, atol=1e-14)
    assert np.all(mag >= np.abs(val) - 1e-12)


# ---------------------------------------------------------------- tolerance

def test_error_bound_covers_float32_sequential_accumulation():
    # A float32 loop (round to nearest after every add) must land inside the
    # bound; this checks the bound's derivation, not the kernel.
    rng = np.random.default_rng(8)
    K = 4096
    a = (rng.standard_normal((64, K)) / math.sqrt(K)).astype(np.float32)
    b = (rng.standard_normal((K, 16)) / math.sqrt(K)).astype(np.float32)
    ab = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bb = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    af = orc.bf16_bits_to_f64(ab).astype(np.float32)
    bf = orc.bf16_bits_to_f64(bb).astype(np.float32)
    acc = np.zeros((64, 16), np.float32)
    for k in range(K):
        acc = acc + af[:, k:k + 1] * bf[k:k + 1, :]
    ref = orc.local_partial(ab, bb)
    mag = orc.local_partial_abs(ab, bb)
    tol = orc.error_bound(mag, K, bf16_out=False, ref=ref)
    assert np.all(np.abs(acc.astype(np.float64) - ref) <= tol)
    # and the bf16-rounded result against the bf16 tolerance
    acc_b = orc.bf16_bits_to_f64(orc.f64_to_bf16_bits(acc.astype(np.float64)))
    tolb = orc.error_bound(mag, K, bf16_out=True, ref=ref)
    assert np.all(np.abs(acc_b - ref) <= tolb)


def test_error_bound_closed_forms():
    # Where the Higham term and the half-ulp term are exact rationals the
    # tolerance has a closed form.  n u = 4096 * 2**-23 = 2**-11, so
    # gamma_4096 = 2**-11 / (1 - 2**-11) = 1/2047 exactly.
    g = 1.0 / 2047.0
    one = np.array([1.0])
    # the Higham term dominates: tolerance = gamma * mag
    t = orc.error_bound(np.array([1000.0]), 4096, bf16_out=False, ref=one)
    assert t[0] == pytest.approx(1000.0 * g, rel=1e-15)
    # the 2-ulp floor dominates: 2 * 2**-7 at |ref| = 1, 2 * 2**-4 at |ref| = 12
    t = orc.error_bound(np.array([1.0, 1.0]), 4096, bf16_out=False, ref=np.array([1.0, -12.0]))
    assert t[0] == 2.0 ** -6 and t[1] == 2.0 ** -3
    # a bf16 result adds half a bf16 ulp at |ref| + gamma * mag:
    # 1 + 1000/2047 = 1.4885.. lies in [1, 2), ulp 2**-7
    t = orc.error_bound(np.array([1000.0]), 4096, bf16_out=True, ref=one)
    assert t[0] == pytest.approx(1000.0 * g + 2.0 ** -8, rel=1e-15)
    # no terms: no rounding error, only the 2-ulp floor
    t = orc.error_bound(np.array([5.0]), 0, bf16_out=False, ref=np.array([3.0]))
    assert t[0] == 2.0 * 2.0 ** -6
    # n = 2**10 terms: gamma = 2**-13 / (1 - 2**-13) = 1/8191
    t = orc.error_bound(np.array([8191.0 * 64]), 1024, bf16_out=False, ref=one)
    assert t[0] == pytest.approx(64.0, rel=1e-15)


def test_local_partial_abs_by_hand():
    # Mixed signs: |A|.|B| differs from |A.B| wherever terms cancel.
    A = np.array([[1.0, -2.0], [-0.5, 3.0]])
    B = np.array([[3.0, -1.0], [4.0, 0.25]])
    T = orc.local_partial_abs(_bits(A), _bits(B))
    assert np.array_equal(T, np.array([[11.0, 1.5], [13.5, 1.25]]))
    C = orc.local_partial(_bits(A), _bits(B))
    assert np.array_equal(C, np.array([[-5.0, -1.5], [10.5, 1.25]]))
    # invariants: |A.B| <= |A|.|B|, with equality for non-negative operands
    rng = np.random.default_rng(4)
    Ar = rng.integers(-3, 4, (6, 5)).astype(float)
    Br = rng.integers(-3, 4, (5, 7)).astype(float)
    Tr = orc.local_partial_abs(_bits(Ar), _bits(Br))
    assert np.all(np.abs(orc.local_partial(_bits(Ar), _bits(Br))) <= Tr)
    assert np.array_equal(Tr, np.abs(Ar) @ np.abs(Br))
    assert np.array_equal(orc.local_partial_abs(_bits(np.abs(Ar)), _bits(np.abs(Br))),
                          orc.local_partial(_bits(np.abs(Ar)), _bits(np.abs(Br))))


def test_partial_and_owned_elements_match_the_full_share():
    # the paired-position functions against the full product (local_partial,
    # pinned above) and the full share (reduce_scatter_share)
    w = gen.WORKLOADS["tiny"].with_(P=4, rank=1, M=32, N=24, K=40, chunk_rows=4)
    A, B, peers = gen.make_inputs(w, seed=6)
    Ab, Bb, Pb = gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers)
    full = orc.gemm_rs_oracle(Ab, Bb, Pb, w.P, w.rank, w.chunk_rows)
    T = orc.local_partial_abs(Ab, Bb)
    rng = np.random.default_rng(2)
    rows = rng.integers(0, w.M, 300)
    cols = rng.integers(0, w.N, 300)
    val, mag = orc.partial_elements(Ab[rows], Bb[:, cols])
    np.testing.assert_allclose(val, full.C[rows, cols], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(mag, T[rows, cols], rtol=1e-13, atol=0)
    S = w.S
    own = (rows // S) == w.rank
    lr, lc = rows[own] - w.rank * S, cols[own]
    ov, om = orc.owned_elements(val[own], mag[own], Pb[:, lr, lc])
    np.testing.assert_allclose(ov, full.out[lr, lc], rtol=1e-13, atol=1e-13)
    pabs = np.sum(np.abs(orc.bf16_bits_to_f64(Pb)), axis=0)
    np.testing.assert_allclose(om, T[rows[own], lc] + pabs[lr, lc], rtol=1e-13, atol=0)
    # integer twin: exact
    Ai, Bi, Pi = gen.make_inputs(w, seed=7, integer=True)
    Ab, Bb, Pb = gen.bf16_bits(Ai), gen.bf16_bits(Bi), gen.bf16_bits(Pi)
    full = orc.gemm_rs_oracle(Ab, Bb, Pb, w.P, w.rank, w.chunk_rows)
    val, _ = orc.partial_elements(Ab[rows], Bb[:, cols])
    assert np.array_equal(val, full.C[rows, cols])
    ov, _ = orc.owned_elements(val[own], mag[own], Pb[:, lr, lc])
    assert np.array_equal(ov, full.out[lr, lc])
    with pytest.raises(ValueError):
        orc.partial_elements(Ab[rows[:3]], Bb[:, cols[:4]])


def test_sampled_magnitudes_are_abs_products_plus_peer_magnitudes():
    w = gen.WORKLOADS["tiny"].with_(P=4, rank=2, M=32, N=16, K=24, chunk_rows=4)
    A, B, peers = gen.make_inputs(w, seed=5)
    Ab, Bb, Pb = gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers)
    rows = np.arange(w.M).repeat(w.N)
    cols = np.tile(np.arange(w.N), w.M)
    _, _, mag = orc.gemm_rs_elements(Ab, Bb, Pb, w.P, w.rank, rows, cols)
    want = orc.local_partial_abs(Ab, Bb)
    S = w.S
    want[w.rank * S:(w.rank + 1) * S] += np.sum(np.abs(orc.bf16_bits_to_f64(Pb)), axis=0)
    np.testing.assert_allclose(mag.reshape(w.M, w.N), want, rtol=1e-14, atol=0)


def test_rel_frobenius():
    assert orc.rel_frobenius(np.array([3.0, 4.0]), np.array([3.0, 4.0])) == 0.0
    assert orc.rel_frobenius(np.array([3.0, 4.0]), np.array([0.0, 5.0])) == pytest.approx(
        math.sqrt(9 + 1) / 5)


# ---------------------------------------------------------------- page numbers

def _table3():
    rows = []
    with open(os.path.join(GOLDEN, "table3_gemm_vs_gemm_rs.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, g, fz, pct, mk = line.split()
            rows.append((int(k), float(g), float(fz), float(pct), mk))
    return rows


def _kv(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split()
            d[k] = float(v)
    return d


def test_exposed_fraction_reproduces_table3():
    for K, g, fz, pct, mk in _table3():
        frac = 100.0 * metrics.exposed_fraction(fz, g)
        if mk == "lt":
            assert frac < pct
        else:
            assert round(frac) == pct


def test_overlap_bound_and_throughput_reproduce_pages():
    d = _kv("overlap_bound.txt")
    k = metrics.overlap_threshold_k(d["s_bytes"], d["R_flops"], d["B_bytes"])
    assert math.floor(k) == d["k_floor"] and round(k) == d["k_round"]
    t = metrics.tflops(32768, 32768, 4096, d["fused_ms_k4096"] * 1e-3)
    assert round(t, 1) == d["fused_tflops_k4096"]
    # the tile sides cancel: per-tile compute == per-tile transfer at K*
    for m, n in [(128, 128), (256, 64)]:
        assert metrics.tile_compute_seconds(m, n, k, d["R_flops"]) == pytest.approx(
            metrics.tile_transfer_seconds(m, n, d["s_bytes"], d["B_bytes"]))


# ---------------------------------------------------------------- planted mistakes

def _run_pins():
    """The pins above that exercise the reduce-scatter definition."""
    test_concatenated_shards_equal_stacked_gemm(3)
    test_send_slots_skip_self_in_rank_order()
    test_owned_sum_adds_every_peer_once()
    test_local_partial_brute_force_integers()
    test_local_partial_nonsquare_orientation()
    test_bf16_encode_ties_and_no_double_rounding()
    test_bf16_decode_closed_forms()
    test_local_partial_real_values_vs_exact_rational()
    for kind in ("row_lo", "row_hi", "col"):
        test_placement_probes(kind)
    test_error_bound_closed_forms()
    test_local_partial_abs_by_hand()


def test_pins_pass_on_the_real_oracle():
    _run_pins()


@pytest.mark.parametrize("mistake", ["slot_ring_relative", "slot_no_skip", "drop_last_peer",
                                     "peer_sign", "transposed_b", "double_rounding",
                                     "own_rows_shift", "decode_truncates", "gamma_too_loose",
                                     "mag_from_raw_bits"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    if mistake == "slot_ring_relative":
        # another plausible convention (slots ordered from rank+1 around the
        # ring) applied on the sending side only
        real = orc.reduce_scatter_share

        def bad(C, peers, P, rank, chunk_rows):
            monkeypatch.setattr(orc, "slot_of_dest", lambda d, r: (d - r - 1) % P)
            return real(C, peers, P, rank, chunk_rows)
        monkeypatch.setattr(orc, "reduce_scatter_share", bad)
    elif mistake == "slot_no_skip":
        monkeypatch.setattr(orc, "slot_of_dest", lambda d, r: d - 1 if d > 0 else 0)
    elif mistake == "drop_last_peer":
        real = orc.reduce_scatter_share

        def bad(C, peers, P, rank, chunk_rows):
            p = np.array(peers, dtype=np.float64, copy=True)
            if p.shape[0] > 0:
                p[-1] = 0.0
            return real(C, p, P, rank, chunk_rows)
        monkeypatch.setattr(orc, "reduce_scatter_share", bad)
    elif mistake == "peer_sign":
        real = orc.reduce_scatter_share

        def bad(C, peers, P, rank, chunk_rows):
            return real(C, -np.asarray(peers, dtype=np.float64), P, rank, chunk_rows)
        monkeypatch.setattr(orc, "reduce_scatter_share", bad)
    elif mistake == "transposed_b":
        real = orc.local_partial

        def bad(A_bits, B_bits):
            B = np.asarray(B_bits)
            B = B.T if B.shape[0] == B.shape[1] else B[::-1]
            return real(A_bits, np.ascontiguousarray(B))
        monkeypatch.setattr(orc, "local_partial", bad)
    elif mistake == "double_rounding":
        real = orc.f64_to_bf16_bits
        monkeypatch.setattr(orc, "f64_to_bf16_bits",
                            lambda x: real(np.asarray(x, np.float64).astype(np.float32).astype(np.float64)))
    elif mistake == "own_rows_shift":
        real = orc.reduce_scatter_share

        def bad(C, peers, P, rank, chunk_rows):
            return real(np.roll(C, 1, axis=0), peers, P, rank, chunk_rows)
        monkeypatch.setattr(orc, "reduce_scatter_share", bad)
    elif mistake == "decode_truncates":
        real = orc.bf16_bits_to_f64
        monkeypatch.setattr(orc, "bf16_bits_to_f64", lambda b: np.trunc(real(b)))
    elif mistake == "gamma_too_loose":
        # a unit roundoff 1024 times too large (2**-13): every real-valued
        # elementwise check would pass almost anything
        real = orc.error_bound
        monkeypatch.setattr(orc, "error_bound",
                            lambda mag, n, bf16_out, ref, u=2.0 ** -23: real(mag, n, bf16_out, ref,
                                                                            u=u * 1024))
    elif mistake == "mag_from_raw_bits":
        # magnitudes taken from the bf16 bit patterns as integers, not decoded
        def bad(A_bits, B_bits):
            return np.asarray(A_bits, np.float64) @ np.asarray(B_bits, np.float64)
        monkeypatch.setattr(orc, "local_partial_abs", bad)
    with pytest.raises((AssertionError, IndexError)):
        _run_pins()


def test_consume_chunks_by_hand():
    """Worked example: 2 slots x 3 chunks of 2 rows; waits for call 5."""
    send = np.arange(2 * 6 * 4, dtype=np.uint16).reshape(2, 6, 4)
    dest = np.full_like(send, 0xFFFF)
    ready = np.array([[5, 4, 6], [0xFFFFFFFF, 5, 7]], np.uint32)
    got, status = orc.consume_chunks(ready, send, dest, 2, 5)
    assert np.array_equal(status, np.array([[0, 1, 0], [1, 0, 0]], np.int32))
    want = dest.copy()
    want[0, 0:2] = send[0, 0:2]
    want[0, 4:6] = send[0, 4:6]
    want[1, 2:4] = send[1, 2:4]
    want[1, 4:6] = send[1, 4:6]
    assert np.array_equal(got, want)
    assert np.all(dest == 0xFFFF)            # the input is not modified


def test_consume_chunks_wraps_at_2_32():
    send = np.ones((1, 2, 8), np.uint16)
    dest = np.zeros_like(send)
    # expected 0xFFFFFFFF: a word that has wrapped to 1 is two calls past it
    got, status = orc.consume_chunks(np.array([[1, 0xFFFFFFFE]], np.uint32), send, dest, 1,
                                     0xFFFFFFFF)
    assert np.array_equal(status, np.array([[0, 1]], np.int32))
    assert np.array_equal(got[0, 0], send[0, 0]) and np.all(got[0, 1] == 0)
    with pytest.raises(ValueError):
        orc.consume_chunks(np.zeros((1, 3), np.uint32), send, dest, 1, 0)


def test_push_share_matches_the_staged_share():
    """Owner's accumulator pre-filled with the peers' sum: the push result on
    the owned shard is the staged owned sum, the other owners get C's rows."""
    rng = np.random.default_rng(6)
    P, rank, M, K, N, cr = 4, 1, 32, 6, 8, 4
    S = M // P
    A, B = _int_mats(rng, M, K, N)
    peers = rng.integers(-8, 9, (P - 1, S, N)).astype(np.float64)
    C = A.astype(np.float64) @ B.astype(np.float64)
    staged = orc.reduce_scatter_share(C, peers, P, rank, cr)
    before = np.zeros((P, S, N))
    before[rank] = peers.sum(axis=0)
    acc, ready, counters = orc.push_share(C, before, P, rank, cr)
    assert np.array_equal(acc[rank], staged.out)
    for d in range(P):
        if d != rank:
            assert np.array_equal(acc[d], C[d * S:(d + 1) * S])
    assert np.array_equal(ready, staged.ready) and np.array_equal(counters, staged.counters)


def test_push_from_every_rank_gives_the_full_sum():
    """P ranks pushing into shared accumulators: accumulator d ends with
    sum_p A_p . B_p restricted to shard d (the reduce-scatter's definition)."""
    rng = np.random.default_rng(7)
    P, M, K, N = 3, 12, 5, 4
    S = M // P
    acc = np.zeros((P, S, N))
    full = np.zeros((M, N))
    for r in range(P):
        A, B = _int_mats(rng, M, K, N)
        C = A.astype(np.float64) @ B.astype(np.float64)
        full += C
        acc, _, _ = orc.push_share(C, acc, P, r, 2)
    for d in range(P):
        assert np.array_equal(acc[d], full[d * S:(d + 1) * S])
    with pytest.raises(ValueError):
        orc.push_share(np.zeros((12, 4)), np.zeros((2, 4, 4)), 3, 0, 2)


def test_ag_gemm_is_the_gathered_product():
    """Each rank's row block of C is that rank's A rows times B (block rows of
    a product), and only other ranks' late chunks count as errors."""
    rng = np.random.default_rng(8)
    P, rank, S, K, N, cr = 4, 2, 6, 5, 7, 3
    blocks = [rng.integers(-2, 3, (S, K)) for _ in range(P)]
    B = rng.integers(-2, 3, (K, N))
    A = np.concatenate(blocks)
    ready = np.full((P, S // cr), 3, np.uint32)
    C, err = orc.ag_gemm(_bits(A), _bits(B), ready, P, rank, cr, 3)
    assert err == 0
    for p in range(P):
        assert np.array_equal(C[p * S:(p + 1) * S], blocks[p].astype(np.float64) @ B)
    ready[rank, 0] = 0                    # this rank's own words are never waited on
    assert orc.ag_gemm(_bits(A), _bits(B), ready, P, rank, cr, 3)[1] == 0
    ready[0, 1] = 2                       # another rank's chunk one call behind
    assert orc.ag_gemm(_bits(A), _bits(B), ready, P, rank, cr, 3)[1] == 1



def test_intercu_reduce_by_hand():
    """Two slots of known bf16 values: the workspace holds their sum, every
    piece word rises by one, and only late words set error bits."""
    S, N = 130, 72                                   # ragged: 3 x 2 pieces of 64 x 64
    peers = np.zeros((2, S, N))
    peers[0] = 1.5
    peers[1, :, :8] = -0.25
    peers[1, 128:, 64:] = 40.0
    presum, pieces, err = orc.intercu_reduce(_bits(peers), np.zeros((3, 2), np.uint32), 1, 65)
    want = np.full((S, N), 1.5)
    want[:, :8] = 1.25
    want[128:, 64:] = 41.5
    assert np.array_equal(presum, want) and err == 0
    assert np.array_equal(pieces, np.ones((3, 2), np.uint32))
    # piece words raised to 4 while the compute side waits for 5: bit 1
    assert orc.intercu_reduce(_bits(peers), np.full((3, 2), 3, np.uint32), 5, 65)[2] == 1
    # an incoming chunk one call behind: bit 2; wrap-around counts as arrived
    ready = np.full((2, 2), 7, np.uint32)
    assert orc.intercu_reduce(_bits(peers), np.full((3, 2), 6, np.uint32), 7, 65, ready)[2] == 0
    ready[1, 0] = 6
    assert orc.intercu_reduce(_bits(peers), np.full((3, 2), 6, np.uint32), 7, 65, ready)[2] == 2
    wrap = np.full((3, 2), 0xFFFFFFFF, np.uint32)
    p, w, e = orc.intercu_reduce(_bits(peers), wrap, 0, 65, np.zeros((2, 2), np.uint32))
    assert np.all(w == 0) and e == 0
    with pytest.raises(ValueError):
        orc.intercu_reduce(_bits(peers), np.zeros((2, 2), np.uint32), 1, 65)


def test_intercu_reduce_plus_local_partial_is_the_owned_shard():
    """presum + the rank's own rows of C equals the staged share's out: the
    reduction role only moves where the peer sum is taken."""
    rng = np.random.default_rng(9)
    P, rank, S, K, N = 4, 1, 64, 16, 64
    A = rng.integers(-2, 3, (P * S, K))
    B = rng.integers(-2, 3, (K, N))
    peers = rng.integers(-8, 9, (P - 1, S, N))
    C = orc.local_partial(_bits(A), _bits(B))
    share = orc.reduce_scatter_share(C, orc.bf16_bits_to_f64(_bits(peers)), P, rank, 32)
    presum, _, _ = orc.intercu_reduce(_bits(peers), np.zeros((1, 1), np.uint32), 1, 32)
    assert np.array_equal(presum + C[rank * S:(rank + 1) * S], share.out)
