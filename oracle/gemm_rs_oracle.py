"""Plain fp64 CPU oracle for one rank's share of a fused GEMM + reduce-scatter.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library; it takes plain numpy arrays of bf16 bit
patterns (``uint16``) and returns numpy arrays.

What it computes, and where the pages define it
-----------------------------------------------
Sources are three web pages, cited by title and section:

[PK]  "ParallelKittens: Systematic and Practical Simplification of Multi-GPU AI
      Kernels" (paper summary page), section 3 "Technical Approach":
      "Scheduling Analysis" (the fused GEMM + reduce-scatter example: every
      GPU produces a partial of each output tile and the GPU owning that
      tile's shard ends with the sum of all partials) and "The Eight PK
      Primitives" (store_add_async adds a tile into the owner's buffer;
      signal adds to a barrier word, wait spins until it reaches a value).
[PKN] "ParallelKittens: Three Principles and Eight Primitives for Multi-GPU
      Kernels" (reading notes), section 3 "Principle 2": the M x N x K
      GEMM + reduce-scatter on P GPUs with bf16 elements (s = 2 bytes).
[SYN] "Syncopate: Efficient Multi-GPU AI Kernels via Automatic Chunk-Centric
      Compute-Communication Overlap", section 5.1 "Communication Schedule
      Abstraction": a chunk is a logical block of one or more tiles that is
      communicated as a unit.

Definition implemented (one rank ``rank`` of ``P``; S = M / P):

    C          = A . B                       (this rank's local partial, M x N)
    send[j]    = bf16_rne(C[d*S:(d+1)*S, :])  for every destination d != rank,
                                              slot j = d if d < rank else d - 1
    out        = C[rank*S:(rank+1)*S, :] + sum_j peers[j]   (j ascending)
    ready[j,c] = ready_before[j,c] + 1,       for every slot j and chunk c
    counter[j,c] = 0

The pages fix the mathematics (the owner ends with the sum over all ranks of
their partials for its shard) but not the buffer layout, the rounding mode of
the bf16 send copy, or the flag words; the readings taken here are:

* shards are contiguous row blocks and rank r owns rows [r*S, (r+1)*S);
* send buffers are bf16, rounded to nearest-even directly from the exact
  (fp64) value -- no intermediate fp32 rounding;
* slots skip the calling rank and are in ascending rank order;
* chunk c of a slot is rows [c*chunk_rows, (c+1)*chunk_rows) of that slot, at
  full width N;
* the owned shard sums the staged peer partials in ascending slot order;
* a chunk's ready word counts the times it was published: the pages' signal
  primitive ("The Eight PK Primitives" in the ParallelKittens summary page)
  atomically adds a value to a barrier counter and wait spins until the
  counter reaches an expected value, so each call adds exactly 1 to every
  chunk's ready word (from zero for fresh flags) and leaves its arrival
  counter back at 0.

Everything is computed in fp64.  The matrix product is a library primitive
(numpy ``matmul`` in float64); every other step is written out here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Words per arrival counter in the flags buffer: the pages fix what a counter
# does, not where it lives; the device keeps each on a 128-byte line of its own.
COUNTER_LINE_WORDS = 32


def flag_words(ready: np.ndarray, counters: np.ndarray) -> np.ndarray:
    """Flag words in device order: all ready words (slot-major), then each
    arrival counter at the start of a COUNTER_LINE_WORDS line of its own (the
    other words of the line zero)."""
    lines = np.zeros((counters.size, COUNTER_LINE_WORDS), np.uint32)
    lines[:, 0] = counters.ravel()
    return np.concatenate([ready.ravel().astype(np.uint32), lines.ravel()])

__all__ = [
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "ulp_bf16",
    "slot_of_dest",
    "dest_of_slot",
    "local_partial",
    "local_partial_abs",
    "reduce_scatter_share",
    "flag_words",
    "gemm_rs_oracle",
    "gemm_rs_elements",
    "partial_elements",
    "owned_elements",
    "error_bound",
    "OracleResult",
    "consume_chunks",
    "push_share",
    "ag_gemm",
]

# ---------------------------------------------------------------------------
# bf16 <-> fp64, from the IEEE-754 binary format definition.
# bf16 = 1 sign bit, 8 exponent bits (bias 127), 7 stored fraction bits: the
# top 16 bits of an IEEE binary32.  Smallest normal 2**-126, subnormal
# spacing 2**-133, largest finite (2 - 2**-7) * 2**127.
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64.

    A bf16 pattern is the high half of the binary32 with the same value, so
    shifting it up 16 bits and reinterpreting as float32 is exact; float32 ->
    float64 is exact too.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (float64 result).

    For |x| in [2**E, 2**(E+1)) the spacing is 2**(E-7); below the smallest
    normal 2**-126 it is the subnormal spacing 2**-133.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)                   # a = m * 2**e, m in [0.5, 1)
    E = np.where(a > 0, e - 1, -126)
    E = np.maximum(E, -126)
    return np.ldexp(np.ones_like(a), (E - 7).astype(np.int64))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16, round-to-nearest-even, return uint16 bits.

    Rounds once, directly from the float64 value: the result is the bf16
    number nearest to x, ties going to the one whose last stored fraction bit
    is 0.  Values whose rounded magnitude reaches 2**128 become infinity (the
    IEEE overflow rule for round-to-nearest); NaN maps to the quiet NaN 0x7FC0
    with the input's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    q = ulp_bf16(a)                       # power of two: a / q is exact
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(a / q) * q            # numpy rint: ties to even integer
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    v = np.copysign(r, x)                 # keeps the sign of zero
    # v is a bf16 value, hence exactly a float32; its top half is the pattern.
    with np.errstate(invalid="ignore"):
        f32 = v.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        sign = (np.signbit(x).astype(np.uint16) << np.uint16(15))
        bits = np.where(nan, np.uint16(0x7FC0) | sign, bits).astype(np.uint16)
    return bits


# ---------------------------------------------------------------------------
# Slot / chunk bookkeeping (the readings listed in the module docstring).
# ---------------------------------------------------------------------------


def slot_of_dest(dest: int, rank: int) -> int:
    """Send slot that holds the rows destined to rank ``dest`` (dest != rank)."""
    if dest == rank:
        raise ValueError("the owned shard has no send slot")
    return dest if dest < rank else dest - 1


def dest_of_slot(slot: int, rank: int) -> int:
    """Inverse of :func:`slot_of_dest`."""
    return slot if slot < rank else slot + 1


# ---------------------------------------------------------------------------
# The local partial and the reduce-scatter share.
# ---------------------------------------------------------------------------


def local_partial(A_bits: np.ndarray, B_bits: np.ndarray) -> np.ndarray:
    """C = A . B in float64 (library matmul), from bf16 bit patterns.

    [PKN] section 3: the local M x N x K GEMM whose output tiles are then sent
    to their owners.  Products of two bf16 numbers are exact in float64; the
    sums carry float64 rounding only.
    """
    A = bf16_bits_to_f64(A_bits)
    B = bf16_bits_to_f64(B_bits)
    if A.shape[1] != B.shape[0]:
        raise ValueError("inner dimensions differ")
    if A.shape[1] == 0:
        return np.zeros((A.shape[0], B.shape[1]), dtype=np.float64)
    return A @ B


def local_partial_abs(A_bits: np.ndarray, B_bits: np.ndarray) -> np.ndarray:
    """T = |A| . |B| in float64, the magnitude that scales rounding error."""
    A = np.abs(bf16_bits_to_f64(A_bits))
    B = np.abs(bf16_bits_to_f64(B_bits))
    if A.shape[1] == 0:
        return np.zeros((A.shape[0], B.shape[1]), dtype=np.float64)
    return A @ B


@dataclass
class OracleResult:
    send_bits: np.ndarray      # uint16 [P-1, S, N]   bf16 send buffers
    out: np.ndarray            # float64 [S, N]       owned shard, exact sum
    ready: np.ndarray          # uint32 [P-1, S/chunk_rows]
    counters: np.ndarray       # uint32 [P-1, S/chunk_rows]
    C: np.ndarray              # float64 [M, N]       local partial

    @property
    def flags(self) -> np.ndarray:
        """Flag words in device order (flag_words)."""
        return flag_words(self.ready, self.counters)

    def out_bf16_bits(self) -> np.ndarray:
        return f64_to_bf16_bits(self.out)

    def out_f32(self) -> np.ndarray:
        """The owned shard rounded once to float32 (nearest-even)."""
        return self.out.astype(np.float32)


def reduce_scatter_share(C: np.ndarray, peers: np.ndarray, P: int, rank: int,
                         chunk_rows: int, ready_before=None) -> OracleResult:
    """Reduce-scatter share of rank ``rank`` given its local partial C.

    [PK] "Scheduling Analysis": each output row block goes to the rank that
    owns it; the owner adds every rank's partial for its shard.  ``peers``
    (float64 [P-1, S, N]) are the partials that the other ranks sent to this
    rank, slot j coming from rank dest_of_slot(j).  [SYN] 5.1: each slot is
    split into chunks of ``chunk_rows`` full-width rows, each a unit whose
    readiness is signalled once per call: its ready word goes up by one from
    ``ready_before`` (uint32 [P-1, S/chunk_rows], zeros when None).
    """
    M, N = C.shape
    if P < 1 or not (0 <= rank < P):
        raise ValueError("need P >= 1 and 0 <= rank < P")
    if M % P:
        raise ValueError("M must be a multiple of P")
    S = M // P
    if chunk_rows <= 0 or (S % chunk_rows):
        raise ValueError("chunk_rows must divide the shard height")
    peers = np.asarray(peers, dtype=np.float64)
    if peers.shape != (P - 1, S, N):
        raise ValueError(f"peers must have shape {(P - 1, S, N)}")

    send = np.empty((P - 1, S, N), dtype=np.uint16)
    for d in range(P):
        if d == rank:
            continue
        send[slot_of_dest(d, rank)] = f64_to_bf16_bits(C[d * S:(d + 1) * S, :])

    out = C[rank * S:(rank + 1) * S, :].copy()
    for j in range(P - 1):                # ascending slot order
        out = out + peers[j]

    n_chunks = S // chunk_rows
    if ready_before is None:
        ready_before = np.zeros((P - 1, n_chunks), dtype=np.uint32)
    ready_before = np.asarray(ready_before, dtype=np.uint32)
    if ready_before.shape != (P - 1, n_chunks):
        raise ValueError(f"ready_before must have shape {(P - 1, n_chunks)}")
    ready = ready_before + np.uint32(1)    # uint32 arithmetic wraps like the device word
    counters = np.zeros((P - 1, n_chunks), dtype=np.uint32)
    return OracleResult(send_bits=send, out=out, ready=ready, counters=counters, C=C)


def gemm_rs_oracle(A_bits: np.ndarray, B_bits: np.ndarray, peer_bits: np.ndarray,
                   P: int, rank: int, chunk_rows: int, ready_before=None) -> OracleResult:
    """Whole share from bf16 inputs: local partial, send copies, owned sum, flags."""
    C = local_partial(A_bits, B_bits)
    peers = bf16_bits_to_f64(peer_bits)
    return reduce_scatter_share(C, peers, P, rank, chunk_rows, ready_before)


def partial_elements(A_rows_bits: np.ndarray, B_cols_bits: np.ndarray):
    """C at paired positions: element i is row i of ``A_rows_bits`` [n, K]
    (bf16 bits) dotted with column i of ``B_cols_bits`` [K, n].

    [PKN] section 3: one element of the local partial C = A . B, each its own
    fp64 dot product (the products of two bf16 numbers are exact in fp64).
    Returns (value, |A|.|B|) per position.
    """
    A = bf16_bits_to_f64(np.asarray(A_rows_bits))
    B = bf16_bits_to_f64(np.asarray(B_cols_bits)).T
    if A.shape != B.shape:
        raise ValueError("need A rows [n, K] and B columns [K, n]")
    return np.einsum("ik,ik->i", A, B), np.einsum("ik,ik->i", np.abs(A), np.abs(B))


def owned_elements(c_val: np.ndarray, c_mag: np.ndarray, peer_bits_at: np.ndarray):
    """Owned-shard values at sampled positions: [PK] "Scheduling Analysis",
    the owner's result is its own partial plus every peer's, here
    C + sum_j peers[j] in ascending slot order (fp64).  ``peer_bits_at`` is
    [P-1, n], the bf16 bits of each slot at the positions.  Returns
    (value, |A|.|B| + sum_j |peer_j|)."""
    val = np.array(c_val, dtype=np.float64, copy=True)
    mag = np.array(c_mag, dtype=np.float64, copy=True)
    for j in range(np.asarray(peer_bits_at).shape[0]):
        pv = bf16_bits_to_f64(np.asarray(peer_bits_at)[j])
        val = val + pv
        mag = mag + np.abs(pv)
    return val, mag


def gemm_rs_elements(A_bits: np.ndarray, B_bits: np.ndarray, peer_bits, P: int,
                     rank: int, rows: np.ndarray, cols: np.ndarray):
    """Expected values at the output positions (rows[i], cols[i]) only.

    For problems too large for the full product: each requested element of C
    is its own fp64 dot product of one row of A and one column of B.  ``rows``
    are global row indices in [0, M).  Returns ``(kind, value, mag)`` where
    kind is 1 for rows in the owned shard (value = exact owned sum) and 0 for
    rows that are sent (value = exact C, to be rounded by the caller), and mag
    is |A|.|B| + sum_j |peer_j| at that position (for the rounding bound).
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    M = A_bits.shape[0]
    S = M // P
    A = bf16_bits_to_f64(np.asarray(A_bits)[rows, :])            # [n, K]
    Bc = bf16_bits_to_f64(np.asarray(B_bits)[:, cols]).T          # [n, K]
    val = np.einsum("ik,ik->i", A, Bc)
    mag = np.einsum("ik,ik->i", np.abs(A), np.abs(Bc))
    owned = (rows // S) == rank
    kind = owned.astype(np.int64)
    if np.any(owned):
        lr = rows[owned] - rank * S
        lc = cols[owned]
        acc = val[owned]
        amag = mag[owned]
        for j in range(P - 1):
            pv = bf16_bits_to_f64(peer_bits[j][lr, lc])
            acc = acc + pv
            amag = amag + np.abs(pv)
        val = val.copy()
        mag = mag.copy()
        val[owned] = acc
        mag[owned] = amag
    return kind, val, mag


# ---------------------------------------------------------------------------
# Rounding bound for a float32-accumulating implementation.
# ---------------------------------------------------------------------------


def error_bound(mag: np.ndarray, n_terms: int, bf16_out: bool, ref: np.ndarray,
                u: float = 2.0 ** -23) -> np.ndarray:
    """Per-element tolerance for a float32 evaluation of the same sums.

    A sum of n_terms products evaluated in a working precision with unit
    roundoff u, in any order, differs from the exact value by at most
    gamma_n * sum|terms| with gamma_n = n*u / (1 - n*u) (Higham, "Accuracy and
    Stability of Numerical Algorithms", 2nd ed., section 3.1).  The rounding
    of a matrix core's internal sums is not published; u = 2**-23 is the unit
    roundoff of a 24-bit significand under chopping (round toward zero), the
    weakest rounding that keeps each operation's relative error below one ulp
    (Higham section 2.1: u = 2**(1-t) for chopping, 2**-t for round to
    nearest with t = 24), so the bound holds under either.  The tolerance is
    the larger of that bound and 2 bf16 ulps of the reference; a bf16-stored
    result adds half a bf16 ulp for its final rounding.
    """
    n = float(n_terms)
    gamma = n * u / (1.0 - n * u)
    tol = gamma * np.asarray(mag, dtype=np.float64)
    if bf16_out:
        tol = tol + 0.5 * ulp_bf16(np.abs(ref) + tol)
    return np.maximum(tol, 2.0 * ulp_bf16(ref))


def rel_frobenius(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_F / ||ref||_F (0 when both vanish)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = math.sqrt(float(np.sum(ref * ref)))
    num = math.sqrt(float(np.sum((a - ref) ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


def consume_chunks(ready: np.ndarray, send_bits: np.ndarray, dest_bits: np.ndarray,
                   chunk_rows: int, expected: int):
    """The chunk consumer (the step after the share): what dest and the status
    words hold after one pass.

    [PK] "The Eight PK Primitives": wait spins on a counter until it reaches an
    expected value; [SYN] 5.1: a chunk moves as one unit.  ``ready`` (uint32
    [P-1, C]) are the producer's ready words, ``send_bits`` / ``dest_bits``
    (uint16 [P-1, S, N]) the send buffers and the staging buffers before the
    pass.  A chunk whose ready word has reached ``expected`` -- compared as a
    signed 32-bit distance, the reading taken here so that counts may wrap --
    is copied and gets status 0; any other chunk is left alone and gets
    status 1 (timed out).  Returns (dest_bits after, status int32 [P-1, C]).
    """
    ready = np.asarray(ready, dtype=np.uint32)
    dest = np.array(dest_bits, dtype=np.uint16, copy=True)
    n_slots, C = ready.shape
    if send_bits.shape[0] != n_slots or dest.shape != send_bits.shape:
        raise ValueError("ready, send and dest disagree on the number of slots")
    if send_bits.shape[1] != C * chunk_rows:
        raise ValueError("chunks do not tile the shard")
    status = np.ones((n_slots, C), dtype=np.int32)
    for j in range(n_slots):
        for c in range(C):
            distance = (int(ready[j, c]) - (expected & 0xFFFFFFFF)) & 0xFFFFFFFF
            if distance >= 1 << 31:        # as a signed 32-bit value
                distance -= 1 << 32
            if distance >= 0:
                rows = slice(c * chunk_rows, (c + 1) * chunk_rows)
                dest[j, rows] = send_bits[j, rows]
                status[j, c] = 0
    return dest, status


def push_share(C: np.ndarray, accum_before: np.ndarray, P: int, rank: int, chunk_rows: int,
               ready_before=None):
    """Atomic push variant: what one rank's share leaves in the owners'
    accumulators.

    [PK] "The Eight PK Primitives": store_add_async adds a tile atomically
    into a peer's buffer; [PK] "Scheduling Analysis": each output tile goes to
    the rank that owns its rows.  ``accum_before`` (float64 [P, S, N]) holds
    the owners' accumulators before the call; every owner d (this rank
    included) receives this rank's partial rows of shard d once:
    accum[d] = accum_before[d] + C[d*S:(d+1)*S], exact in fp64.  Ready words
    and counters as in reduce_scatter_share: each of the P-1 other owners'
    chunks is signalled once.  Returns (accum float64 [P, S, N], ready,
    counters).
    """
    M, N = C.shape
    if P < 1 or not (0 <= rank < P) or M % P:
        raise ValueError("need P >= 1, 0 <= rank < P and P dividing M")
    S = M // P
    accum_before = np.asarray(accum_before, dtype=np.float64)
    if accum_before.shape != (P, S, N):
        raise ValueError(f"accum_before must have shape {(P, S, N)}")
    accum = accum_before.copy()
    for d in range(P):
        accum[d] = accum[d] + C[d * S:(d + 1) * S, :]
    if chunk_rows <= 0 or S % chunk_rows:
        raise ValueError("chunk_rows must divide the shard height")
    n_chunks = S // chunk_rows
    if ready_before is None:
        ready_before = np.zeros((P - 1, n_chunks), dtype=np.uint32)
    ready = np.asarray(ready_before, dtype=np.uint32) + np.uint32(1)
    counters = np.zeros((P - 1, n_chunks), dtype=np.uint32)
    return accum, ready, counters


def ag_gemm(A_bits: np.ndarray, B_bits: np.ndarray, ready: np.ndarray, P: int, rank: int,
            chunk_rows: int, expected: int):
    """All-gather + GEMM, the step before the share in a tensor-parallel MLP.

    [PK] "Data and Tensor Parallelism: AG+GEMM, GEMM+RS, and GEMM+AR": the
    rows of A are gathered from the P ranks (rank p owns rows [p*S, (p+1)*S))
    and multiplied by this rank's B.  ``A_bits`` (uint16 [M, K]) is the
    gathered buffer, ``ready`` (uint32 [P, S/chunk_rows]) the arrival words of
    its chunks.  Returns (C float64 [M, N] = A . B exactly, error) where error
    is 1 when some chunk of another rank's rows has not reached ``expected``
    (signed 32-bit distance): every chunk is read by some tile, whose wait then
    gives up.
    """
    A_bits = np.asarray(A_bits)
    M = A_bits.shape[0]
    if P < 1 or not (0 <= rank < P) or M % P:
        raise ValueError("need P >= 1, 0 <= rank < P and P dividing M")
    S = M // P
    if S and (chunk_rows <= 0 or S % chunk_rows):
        raise ValueError("chunk_rows must divide the shard height")
    C = local_partial(A_bits, B_bits)
    ready = np.asarray(ready, dtype=np.uint32)
    error = 0
    for p in range(P):
        if p == rank:
            continue
        for c in range(ready.shape[1]):
            d = (int(ready[p, c]) - (expected & 0xFFFFFFFF)) & 0xFFFFFFFF
            if d >= 1 << 31:
                error = 1
    return C, error



def _behind(word: int, expected: int) -> bool:
    """True when ``word`` has not reached ``expected`` as a signed 32-bit
    distance (the reading of the pages' wait taken throughout, so counts may
    wrap)."""
    d = (int(word) - (expected & 0xFFFFFFFF)) & 0xFFFFFFFF
    return d >= 1 << 31


def intercu_reduce(peer_bits: np.ndarray, piece_before: np.ndarray, expected: int,
                   chunk_rows: int, peer_ready=None):
    """Inter-CU schedule, reduction role: what the reduction workgroups leave
    beside the share itself (which is the staged share's, reduce_scatter_share).

    [PK] "Scheduling Analysis": with inter-SM overlapping whole SMs do the
    communication side while the rest compute; here they do the owner-side
    reduction of the staged peer partials, and the owned-shard value is that
    peer sum plus the local partial.  [PK] "The Eight PK Primitives": signal
    adds to a counter and wait spins until it reaches a value.

    ``peer_bits`` (uint16 [P-1, S, N]) are the staged peer partials,
    ``piece_before`` (uint32 [ceil(S/64), ceil(N/64)]) the piece words before
    the call (a 64 x 64 piece of the owned shard each, the interface's
    layout), ``peer_ready`` None or the incoming chunk words (uint32
    [P-1, S/chunk_rows]).  Returns
      presum  float64 [S, N]: sum over slots of the peer partials (exact);
      pieces  uint32: piece_before + 1 (every piece is summed once per call);
      error   int: bit 2 when an incoming chunk word has not reached
              ``expected`` (the rows are then summed as they are), bit 1 when
              a raised piece word is still behind ``expected`` (the owned
              item covering it then gives up waiting).
    """
    peers = bf16_bits_to_f64(np.asarray(peer_bits))
    n_slots, S, N = peers.shape
    presum = np.zeros((S, N), dtype=np.float64)
    for j in range(n_slots):
        presum = presum + peers[j]
    piece_before = np.asarray(piece_before, dtype=np.uint32)
    if piece_before.shape != (-(-S // 64), -(-N // 64)):
        raise ValueError("one piece word per 64 x 64 block of the shard")
    pieces = piece_before + np.uint32(1)
    error = 0
    if peer_ready is not None:
        peer_ready = np.asarray(peer_ready, dtype=np.uint32)
        if chunk_rows <= 0 or S % chunk_rows or peer_ready.shape != (n_slots, S // chunk_rows):
            raise ValueError("one incoming word per slot and chunk")
        if any(_behind(w, expected) for w in peer_ready.ravel()):
            error |= 2
    if any(_behind(w, expected) for w in pieces.ravel()):
        error |= 1
    return presum, pieces, error
