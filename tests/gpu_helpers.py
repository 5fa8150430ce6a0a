"""Helpers shared by the GPU parity tests: buffer set-up with poison and
canaries, one call through the C ABI, comparisons against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle.gemm_rs_oracle as orc
from gemm_reduce_scatter_amd import binding as pk
from gemm_reduce_scatter_amd import inputs as gen

GUARD = 4096          # canary elements after every output buffer
POISON_BF16 = -1      # 0xFFFF: a NaN pattern
CANARY_U16 = 0x5A5A
CANARY_F32 = 1234.5


class Share:
    """Device buffers of one call, each followed by a canary region."""

    def __init__(self, w: gen.Workload, out_dtype: str, device="cuda", chunk_rows=None):
        self.w = w
        self.chunk_rows = w.chunk_rows if chunk_rows is None else chunk_rows
        S, N, P = w.S, w.N, w.P
        n_send = max(P - 1, 0) * S * N
        self._send = torch.full((n_send + GUARD,), POISON_BF16, dtype=torch.int16, device=device)
        self._send[n_send:] = CANARY_U16
        self.send = self._send[:n_send].view(torch.bfloat16).view(max(P - 1, 0), S, N)
        self.out_dtype = out_dtype
        n_out = S * N
        if out_dtype == "f32":
            self._out = torch.full((n_out + GUARD,), float("nan"), dtype=torch.float32, device=device)
            self._out[n_out:] = CANARY_F32
            self.out = self._out[:n_out].view(S, N)
        else:
            self._out = torch.full((n_out + GUARD,), POISON_BF16, dtype=torch.int16, device=device)
            self._out[n_out:] = CANARY_U16
            self.out = self._out[:n_out].view(torch.bfloat16).view(S, N)
        nf = pk.pk_flags_words(P, w.M, self.chunk_rows) if S > 0 else 0
        self._flags = torch.zeros((nf + GUARD,), dtype=torch.int32, device=device)
        self._flags[nf:] = 0x13579BD
        self.flags = self._flags[:nf]
        self.n_flags = nf

    def reset_flags(self):
        self.flags.zero_()

    def canaries_intact(self) -> bool:
        ok = bool(torch.all(self._send[self._send.numel() - GUARD:] == CANARY_U16))
        if self.out_dtype == "f32":
            ok &= bool(torch.all(self._out[self._out.numel() - GUARD:] == CANARY_F32))
        else:
            ok &= bool(torch.all(self._out[self._out.numel() - GUARD:] == CANARY_U16))
        ok &= bool(torch.all(self._flags[self._flags.numel() - GUARD:] == 0x13579BD))
        return ok


def run(share: Share, A, B, peers, tile_order=None, stream=None, **opts):
    w = share.w
    order = w.tile_order if tile_order is None else tile_order
    out_bf16 = 1 if share.out_dtype == "bf16" else 0
    send = share.send if w.P > 1 else None
    flags = share.flags if share.n_flags > 0 else None
    pk_peers = peers if w.P > 1 else None
    if opts:
        pk.pk_gemm_rs_local_ex(A, B, pk_peers, send, share.out, flags, w.M, w.N, w.K, w.P, w.rank,
                               share.chunk_rows, order, out_bf16, stream=stream, **opts)
    elif out_bf16:
        pk.pk_gemm_rs_local_bf16out(A, B, pk_peers, send, share.out, flags, w.M, w.N, w.K, w.P,
                                    w.rank, share.chunk_rows, order, stream=stream)
    else:
        pk.pk_gemm_rs_local(A, B, pk_peers, send, share.out, flags, w.M, w.N, w.K, w.P, w.rank,
                            share.chunk_rows, order, stream=stream)


def host(share: Share):
    """(send bits [P-1,S,N] uint16, out float64 [S,N], out bits or None, flags uint32)."""
    send = gen.bf16_bits(share.send) if share.w.P > 1 else np.zeros((0, share.w.S, share.w.N), np.uint16)
    if share.out_dtype == "f32":
        out = share.out.cpu().numpy().astype(np.float64)
        out_bits = None
    else:
        out_bits = gen.bf16_bits(share.out)
        out = orc.bf16_bits_to_f64(out_bits)
    flags = share.flags.cpu().numpy().view(np.uint32)
    return send, out, out_bits, flags


def expected_flags(w: gen.Workload, chunk_rows: int, calls: int = 1) -> np.ndarray:
    """Closed form after `calls` calls on zeroed flags: every ready word equals
    `calls` (one signal per chunk per call), every counter 0."""
    if w.S == 0 or w.P == 1:
        return np.zeros(0, np.uint32)
    n = (w.P - 1) * (w.S // chunk_rows)
    return np.concatenate([np.full(n, calls, np.uint32), np.zeros(n, np.uint32)])


def compare_real(res: orc.OracleResult, mag_C, share: Share, n_terms: int):
    """Real-valued inputs: tolerance checks of out and send; returns stats."""
    send, out, _, flags = host(share)
    w = share.w
    S = w.S
    want = res.flags if (w.S > 0 and w.P > 1) else np.zeros(0, np.uint32)
    assert np.array_equal(flags, want), "flags"
    bf16_out = share.out_dtype == "bf16"
    # owned shard
    own_mag = mag_C[w.rank * S:(w.rank + 1) * S]
    tol = orc.error_bound(own_mag + res.peer_abs, n_terms, bf16_out, res.out)
    err = np.abs(out - res.out)
    assert np.all(np.isfinite(out)), "non-finite output"
    bad = err > tol
    assert not np.any(bad), f"{int(bad.sum())} owned elements out of tolerance, max err {err.max()}"
    # A bf16 shard is compared with the oracle's shard rounded once to bf16:
    # bf16 rounding alone is ~1.3e-3 relative (RMS), above the 1e-3 budget.
    ref_frob = orc.bf16_bits_to_f64(res.out_bf16_bits()) if bf16_out else res.out
    rel = orc.rel_frobenius(out, ref_frob)
    assert rel <= 1e-3, rel
    strict = int(np.sum(err > 2.0 * orc.ulp_bf16(res.out)))
    # send buffers: bf16 of the fp32 accumulation vs the exact value
    exact_match = 1.0
    if w.P > 1:
        ref = np.concatenate([res.C[d * S:(d + 1) * S] for d in range(w.P) if d != w.rank])
        mg = np.concatenate([mag_C[d * S:(d + 1) * S] for d in range(w.P) if d != w.rank])
        got = orc.bf16_bits_to_f64(send.reshape(-1, w.N))
        tols = orc.error_bound(mg, n_terms, True, ref)
        e = np.abs(got - ref)
        assert np.all(np.isfinite(got)), "non-finite send value"
        assert not np.any(e > tols), f"{int((e > tols).sum())} send elements out of tolerance"
        exact_match = float(np.mean(send.reshape(-1, w.N) == res.send_bits.reshape(-1, w.N)))
        assert exact_match > 0.9, exact_match
    assert share.canaries_intact()
    return dict(rel_frobenius=rel, strict_2ulp_fails=strict, send_exact_fraction=exact_match)


def compare_exact(res: orc.OracleResult, share: Share):
    """Integer-valued inputs: every output bit must match the oracle."""
    send, out, out_bits, flags = host(share)
    w = share.w
    want = res.flags if (w.S > 0 and w.P > 1) else np.zeros(0, np.uint32)
    assert np.array_equal(flags, want), "flags"
    if w.P > 1:
        assert np.array_equal(send, res.send_bits), "send buffers differ"
    if share.out_dtype == "f32":
        assert np.array_equal(out, res.out), "out differs"
    else:
        assert np.array_equal(out_bits, res.out_bf16_bits()), "out differs"
    assert share.canaries_intact(), "canary overwritten"


def oracle_for(w: gen.Workload, A, B, peers, chunk_rows=None):
    res = orc.gemm_rs_oracle(gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers),
                             w.P, w.rank, w.chunk_rows if chunk_rows is None else chunk_rows)
    res.peer_abs = np.sum(np.abs(orc.bf16_bits_to_f64(gen.bf16_bits(peers))), axis=0) \
        if w.P > 1 else 0.0
    return res
