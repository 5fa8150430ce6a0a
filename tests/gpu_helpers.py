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
    `calls` (one signal per chunk per call), every counter (one per 32-word
    line) 0."""
    if w.S == 0 or w.P == 1:
        return np.zeros(0, np.uint32)
    n = (w.P - 1) * (w.S // chunk_rows)
    return np.concatenate([np.full(n, calls, np.uint32), np.zeros(32 * n, np.uint32)])


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
        # within 1 bf16 ulp of the oracle's rounding wherever the fp32
        # rounding bound stays below half an ulp
        rv = orc.bf16_bits_to_f64(res.send_bits.reshape(-1, w.N))
        tight = n_terms * 2.0 ** -23 / (1 - n_terms * 2.0 ** -23) * mg <= 0.5 * orc.ulp_bf16(ref)
        d = np.abs(got - rv)
        assert np.all(d[tight] <= orc.ulp_bf16(rv[tight])), "send values beyond 1 ulp"
        exact_match = float(np.mean(send.reshape(-1, w.N) == res.send_bits.reshape(-1, w.N)))
        assert exact_match > 0.999, exact_match
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


# ---------------------------------------------------------------- full-size checks
# For shapes whose full product is too large for the host, the GPU outputs are
# compared with the oracle at positions chosen so that every tile meets it:
# a few points in every 256 x 256 tile of every shard, one in every 64 x 128
# sub-tile of the owned shard, and the shard, chunk and tile edges.

def stratified_positions(w: gen.Workload, seed: int, per_tile: int = 4, tile: int = 256,
                         sub=(64, 128), ranks=None):
    """Global (rows, cols) with `per_tile` random points in every tile x tile
    block of every shard in `ranks` (default all), one in every `sub` block of
    the owned shard (when it is among them), plus shard/chunk/tile edges."""
    rng = np.random.default_rng(seed)
    S, N = w.S, w.N
    ranks = range(w.P) if ranks is None else ranks
    rows, cols = [], []

    def blocks(d, bm, bn, k):
        tm, tn = -(-S // bm), -(-N // bn)
        t = np.repeat(np.arange(tm), tn * k)
        u = np.tile(np.repeat(np.arange(tn), k), tm)
        r0, c0 = t * bm, u * bn
        rh, ch = np.minimum(bm, S - r0), np.minimum(bn, N - c0)
        rows.append(d * S + r0 + (rng.random(t.size) * rh).astype(np.int64))
        cols.append(c0 + (rng.random(u.size) * ch).astype(np.int64))

    for d in ranks:
        blocks(d, tile, tile, per_tile)
        if d == w.rank:
            blocks(d, sub[0], sub[1], 1)
        edge_r = [r for r in (0, 1, w.chunk_rows - 1, w.chunk_rows, S - 2, S - 1) if 0 <= r < S]
        edge_c = [c for c in (0, 7, 8, 127, 128, 255, 256, N - 9, N - 8, N - 1) if 0 <= c < N]
        for r in edge_r:
            rows.append(np.full(len(edge_c), d * S + r, np.int64))
            cols.append(np.array(edge_c, np.int64))
    return np.concatenate(rows), np.concatenate(cols)


def _gather_rows(A, rows):
    return gen.bf16_bits(A.index_select(0, torch.from_numpy(rows).to(A.device)))


def _gather_cols(B, cols):
    return gen.bf16_bits(B.index_select(1, torch.from_numpy(cols).to(B.device)).contiguous())


def check_positions(w: gen.Workload, A, B, peers, share: Share, rows, cols, integer: bool,
                    chunk: int = 4096):
    """Send buffers and owned shard at (rows, cols) against the oracle's
    paired-position functions.  Integer inputs: every bit.  Real inputs: send
    values within 1 bf16 ulp of the oracle's rounding wherever the fp32
    rounding bound is below half an ulp (else within that bound), owned
    values within error_bound and the Frobenius budget; every owned element
    beyond a strict 2 ulp must be one whose Higham term exceeds 2 ulp.
    Returns the statistics."""
    S = w.S
    bf16_out = share.out_dtype == "bf16"
    n_terms = w.K + w.P
    st = dict(points=int(rows.size), send_points=0, owned_points=0, send_exact=0,
              send_1ulp=0, send_floor=0, owned_strict_2ulp=0, owned_floor=0,
              max_err_over_tol=0.0, max_err_over_gamma24=0.0)
    g24 = n_terms * 2.0 ** -24 / (1 - n_terms * 2.0 ** -24)
    got_all, ref_all = [], []
    for i0 in range(0, rows.size, chunk):
        r = rows[i0:i0 + chunk]
        c = cols[i0:i0 + chunk]
        val, mag = orc.partial_elements(_gather_rows(A, r), _gather_cols(B, c))
        shard = r // S
        lr = r - shard * S
        own = shard == w.rank
        dev = share.out.device
        lr_t = torch.from_numpy(lr).to(dev)
        c_t = torch.from_numpy(c).to(dev)
        # send slots
        snd = ~own
        if np.any(snd):
            slot = np.where(shard[snd] < w.rank, shard[snd], shard[snd] - 1)
            s_t = torch.from_numpy(snd).to(dev)
            got = gen.bf16_bits(share.send[torch.from_numpy(slot).to(dev), lr_t[s_t], c_t[s_t]])
            ref = orc.f64_to_bf16_bits(val[snd])
            st["send_points"] += int(snd.sum())
            st["send_exact"] += int(np.sum(got == ref))
            if integer:
                assert np.array_equal(got, ref), "send values differ on integer inputs"
            else:
                gv, rv = orc.bf16_bits_to_f64(got), orc.bf16_bits_to_f64(ref)
                assert np.all(np.isfinite(gv)), "non-finite send value"
                gamma_mag = n_terms * 2.0 ** -23 / (1 - n_terms * 2.0 ** -23) * mag[snd]
                tight = gamma_mag <= 0.5 * orc.ulp_bf16(val[snd])
                d = np.abs(gv - rv)
                assert np.all(d[tight] <= orc.ulp_bf16(rv[tight])), \
                    f"{int(np.sum(d[tight] > orc.ulp_bf16(rv[tight])))} send values beyond 1 ulp"
                tol = orc.error_bound(mag[snd], n_terms, True, val[snd])
                assert np.all(np.abs(gv - val[snd]) <= tol), "send values beyond the rounding bound"
                st["send_1ulp"] += int(np.sum((d > 0) & tight))
                st["send_floor"] += int(np.sum(~tight))
                st["send_max_ulps"] = max(st.get("send_max_ulps", 0.0),
                                          float(np.max(d / orc.ulp_bf16(rv))))
        if np.any(own):
            o_t = torch.from_numpy(own).to(dev)
            pbits = gen.bf16_bits(peers[:, lr_t[o_t], c_t[o_t]])
            ov, om = orc.owned_elements(val[own], mag[own], pbits)
            if bf16_out:
                gbits = gen.bf16_bits(share.out[lr_t[o_t], c_t[o_t]])
                got = orc.bf16_bits_to_f64(gbits)
            else:
                got = share.out[lr_t[o_t], c_t[o_t]].cpu().numpy().astype(np.float64)
            st["owned_points"] += int(own.sum())
            if integer:
                want = orc.bf16_bits_to_f64(orc.f64_to_bf16_bits(ov)) if bf16_out else ov
                assert np.array_equal(got, want), "owned values differ on integer inputs"
            else:
                assert np.all(np.isfinite(got)), "non-finite owned value"
                tol = orc.error_bound(om, n_terms, bf16_out, ov)
                err = np.abs(got - ov)
                assert np.all(err <= tol), f"{int(np.sum(err > tol))} owned values out of tolerance"
                two = 2.0 * orc.ulp_bf16(ov)
                strict = err > two
                floor = tol > two
                assert not np.any(strict & ~floor), "beyond 2 ulp where the bound is 2 ulp"
                st["owned_strict_2ulp"] += int(strict.sum())
                st["owned_floor"] += int(floor.sum())
                st["max_err_over_tol"] = max(st["max_err_over_tol"], float(np.max(err / tol)))
                # against the bound with float32's unit roundoff (2**-24)
                # and without the 2-ulp floor: below 1 means the results also
                # meet that tighter reading
                st["max_err_over_gamma24"] = max(
                    st["max_err_over_gamma24"],
                    float(np.max(err / (g24 * om + (0.5 * orc.ulp_bf16(ov) if bf16_out else 0.0)))))
                got_all.append(got)
                ref_all.append(orc.bf16_bits_to_f64(orc.f64_to_bf16_bits(ov)) if bf16_out else ov)
    if got_all:
        st["owned_rel_frobenius"] = orc.rel_frobenius(np.concatenate(got_all),
                                                      np.concatenate(ref_all))
        assert st["owned_rel_frobenius"] <= 1e-3
    if st["send_points"]:
        st["send_exact_fraction"] = st["send_exact"] / st["send_points"]
        assert st["send_exact_fraction"] > 0.999, st["send_exact_fraction"]
    return st


def check_tiles(w: gen.Workload, A, B, peers, share: Share, tiles, integer: bool, tile: int = 256):
    """Complete tile x tile blocks (shard d, row tile t, column tile u) of the
    send buffers or the owned shard against the oracle's product of the
    block's rows of A and columns of B (local_partial), plus the peers for
    the owned shard."""
    S, N = w.S, w.N
    n_terms = w.K + w.P
    bf16_out = share.out_dtype == "bf16"
    for d, t, u in tiles:
        lr = np.arange(t * tile, min((t + 1) * tile, S))
        cc = np.arange(u * tile, min((u + 1) * tile, N))
        Ab = _gather_rows(A, d * S + lr)
        Bb = _gather_cols(B, cc)
        C = orc.local_partial(Ab, Bb)
        lr_t = torch.from_numpy(lr).to(share.out.device)
        cc_t = torch.from_numpy(cc).to(share.out.device)
        if d != w.rank:
            slot = d if d < w.rank else d - 1
            got = gen.bf16_bits(share.send[slot].index_select(0, lr_t).index_select(1, cc_t))
            ref = orc.f64_to_bf16_bits(C)
            if integer:
                assert np.array_equal(got, ref), ("send tile", d, t, u)
            else:
                T = orc.local_partial_abs(Ab, Bb)
                tol = orc.error_bound(T, n_terms, True, C)
                assert np.all(np.abs(orc.bf16_bits_to_f64(got) - C) <= tol), ("send tile", d, t, u)
        else:
            pb = gen.bf16_bits(peers.index_select(1, lr_t).index_select(2, cc_t))
            T = orc.local_partial_abs(Ab, Bb)
            ov, om = orc.owned_elements(C.ravel(), T.ravel(), pb.reshape(pb.shape[0], -1))
            blk = share.out.index_select(0, lr_t).index_select(1, cc_t)
            got = (orc.bf16_bits_to_f64(gen.bf16_bits(blk)) if bf16_out
                   else blk.cpu().numpy().astype(np.float64)).ravel()
            if integer:
                want = orc.bf16_bits_to_f64(orc.f64_to_bf16_bits(ov)) if bf16_out else ov
                assert np.array_equal(got, want), ("owned tile", t, u)
            else:
                tol = orc.error_bound(om, n_terms, bf16_out, ov)
                assert np.all(np.abs(got - ov) <= tol), ("owned tile", t, u)


def record(name: str, stats: dict):
    """Print the statistics; with PK_PARITY_RECORD set, also append them as
    one JSON line to that file."""
    import json
    import os
    line = json.dumps(dict(name=name, **stats), sort_keys=True)
    print(line, flush=True)
    path = os.environ.get("PK_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
