"""Host-side checks of the C ABI that need no GPU: the library loads and
exports what the header declares, argument validation, the tile walk and
the chunk arrival counts."""
import ctypes
import os
import re

import numpy as np
import pytest

from gemm_reduce_scatter_amd import binding as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pk_gemm_rs.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pk_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pk.load()
    names = _declared_functions()
    assert "pk_gemm_rs_local" in names and "pk_gemm_rs_local_bf16out" in names
    for n in names:
        assert hasattr(lib, n), n
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr)


def test_version_and_strerror():
    assert pk.pk_version() >= 100
    for code in range(-7, 1):
        assert pk.pk_strerror(code)
    assert pk.pk_strerror(-99) == "unknown error"


def test_flags_words():
    # ready words, then one 32-word line per arrival counter
    assert pk.pk_flags_words(8, 4096, 128) == 33 * 7 * 4
    assert pk.pk_flags_words(8, 32768, 256) == 33 * 7 * 16
    assert pk.pk_flags_words(2, 256, 64) == 33 * 1 * 2
    assert pk.pk_flags_words(1, 256, 64) == 0
    assert pk.pk_flags_words(4, 0, 0) == 0
    with pytest.raises(pk.PkError):
        pk.pk_flags_words(3, 256, 64)       # M % P
    with pytest.raises(pk.PkError):
        pk.pk_flags_words(2, 256, 48)       # chunk does not divide S
    with pytest.raises(pk.PkError):
        pk.pk_flags_words(0, 256, 64)


# Fake but aligned addresses: pk_validate never dereferences them.
GOOD = dict(A=0x10000, B=0x20000, peer_partials=0x30000, send_bufs=0x40000, out=0x50000,
            flags=0x60000)


def _v(**kw):
    args = dict(GOOD)
    args.update(dict(M=256, N=256, K=128, P=2, rank=0, chunk_rows=64, tile_order=0))
    args.update(kw)
    return pk.pk_validate(args["A"], args["B"], args["peer_partials"], args["send_bufs"],
                          args["out"], args["flags"], args["M"], args["N"], args["K"], args["P"],
                          args["rank"], args["chunk_rows"], args["tile_order"],
                          args.get("out_bf16", 0), args.get("config", 0),
                          args.get("max_workgroups", 0), args.get("group_n", 0),
                          args.get("gemm_only", False), args.get("owned_split", 0),
                          store_policy=args.get("store_policy", 0))


def test_validate_accepts_good_arguments():
    assert _v() == 0
    assert _v(out_bf16=1) == 0
    assert _v(P=1, rank=0, peer_partials=None, send_bufs=None, flags=None) == 0
    assert _v(M=0, A=None, B=None, out=None) == 0
    assert _v(K=0, A=None, B=None) == 0
    assert _v(gemm_only=True, peer_partials=None, send_bufs=None, flags=None) == 0
    for cfg in range(1, pk.pk_config_count() + 1):
        assert _v(config=cfg) == 0
    for pol in (0, 1, 2):
        assert _v(store_policy=pol) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), -1), (dict(B=0x20008), -1), (dict(out=None), -1), (dict(flags=None), -1),
    (dict(send_bufs=None), -1), (dict(peer_partials=0x30001), -1), (dict(flags=0x60002), -1),
    (dict(M=255), -2), (dict(N=12), -2), (dict(K=12), -2), (dict(chunk_rows=48), -2),
    (dict(chunk_rows=0), -2), (dict(M=-2), -2), (dict(out_bf16=2), -2),
    (dict(P=0), -3), (dict(rank=2), -3), (dict(rank=-1), -3), (dict(P=65, M=65 * 64), -3),
    (dict(tile_order=3), -4), (dict(tile_order=-1), -4),
    (dict(config=99), -5), (dict(max_workgroups=-1), -5), (dict(owned_split=2), -5),
    (dict(store_policy=3), -5), (dict(store_policy=-1), -5),
])
def test_validate_rejects(kw, code):
    assert _v(**kw) == code


def test_binding_rejects_short_buffers():
    """The binding refuses buffers smaller than a call reads or writes."""
    import torch
    M, N, K, P, cr = 512, 256, 64, 4, 64
    S = M // P
    bf = torch.bfloat16

    def bufs(out_rows, out_dtype=bf, peers_rows=S):
        return (torch.empty(M, K, dtype=bf), torch.empty(K, N, dtype=bf),
                torch.empty(P - 1, peers_rows, N, dtype=bf), torch.empty(P - 1, S, N, dtype=bf),
                torch.empty(out_rows, N, dtype=out_dtype),
                torch.zeros(pk.pk_flags_words(P, M, cr), dtype=torch.int32))

    pk._check_sizes(*bufs(S), M, N, K, P, cr, 1)
    pk._check_sizes(*bufs(S, torch.float32), M, N, K, P, cr, 0)
    pk._check_sizes(*bufs(M), M, N, K, P, cr, 1, gemm_only=True)
    with pytest.raises(ValueError, match="out"):
        pk._check_sizes(*bufs(S), M, N, K, P, cr, 1, gemm_only=True)   # gemm-only writes M rows
    with pytest.raises(ValueError, match="out"):
        pk._check_sizes(*bufs(S), M, N, K, P, cr, 0)                   # fp32 out in a bf16 buffer
    with pytest.raises(ValueError, match="peer_partials"):
        pk._check_sizes(*bufs(S, peers_rows=S - 1), M, N, K, P, cr, 1)
    z = torch.empty(0, dtype=bf)
    pk._check_sizes(z, z, z, z, z, None, 0, 64, 64, 2, 0, 0)   # empty calls touch nothing


def test_config_table():
    n = pk.pk_config_count()
    assert n >= 3
    for i in range(1, n + 1):
        c = pk.pk_config_info(i)
        assert c["BM"] % c["WM"] == 0 and c["BN"] % c["WN"] == 0
        assert c["threads"] == 64 * (c["BM"] // c["WM"]) * (c["BN"] // c["WN"])
    with pytest.raises(pk.PkError):
        pk.pk_config_info(0)


def test_select_config_for_the_workloads():
    """The pick is the largest tile that still gives every CU (256) a tile."""
    big = pk.pk_config_info(pk.pk_select_config(32768, 32768, 4096, 8))
    assert big["BM"] == 256 and big["BN"] == 256
    for M, N, K, P in ((4096, 4096, 512, 8), (256, 256, 128, 2), (2048, 1024, 64, 4)):
        c = pk.pk_config_info(pk.pk_select_config(M, N, K, P))
        tiles = P * -(-(M // P) // c["BM"]) * -(-N // c["BN"])
        smaller = [pk.pk_config_info(i) for i in range(1, pk.pk_config_count() + 1)]
        if tiles < 256:      # only the smallest tile may leave CUs idle
            assert c["BM"] * c["BN"] == min(x["BM"] * x["BN"] for x in smaller)


# ---------------------------------------------------------------- tile walk

def _tiles(M, N, P, cfg):
    c = pk.pk_config_info(cfg)
    S = M // P
    Tm = -(-S // c["BM"])
    Tn = -(-N // c["BN"])
    return Tm, Tn


@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("shape", [(256, 256, 2, 0, 3), (4096, 4096, 8, 3, 2), (600, 200, 3, 1, 3),
                                   (8192, 1024, 8, 7, 1)])
@pytest.mark.parametrize("group_n", [0, 1, 3])
def test_tile_walk_is_a_permutation(order, shape, group_n):
    M, N, P, rank, cfg = shape
    Tm, Tn = _tiles(M, N, P, cfg)
    w = pk.pk_tile_walk(M, N, P, rank, cfg, order, group_n)
    assert w.shape == (P * Tm * Tn, 4)
    keys = {tuple(r) for r in w.tolist()}
    assert keys == {(d, t, u, -1) for d in range(P) for t in range(Tm) for u in range(Tn)}


def test_tile_orders_follow_their_definitions():
    M, N, P, rank, cfg = 4096, 4096, 8, 3, 2
    Tm, Tn = _tiles(M, N, P, cfg)
    per = Tm * Tn
    # group_n = Tn: plain chunk-major order inside a shard
    rm = pk.pk_tile_walk(M, N, P, rank, cfg, 0, group_n=Tn)
    assert list(rm[:, 0]) == [d for d in range(P) for _ in range(per)]
    # inside a shard: chunk-major (row tile outer, column tile inner)
    assert [tuple(x) for x in rm[:per, 1:3]] == [(t, u) for t in range(Tm) for u in range(Tn)]
    of = pk.pk_tile_walk(M, N, P, rank, cfg, 1, group_n=Tn)
    assert list(of[:, 0]) == [(rank + i) % P for i in range(P) for _ in range(per)]
    rr = pk.pk_tile_walk(M, N, P, rank, cfg, 2, group_n=Tn)
    assert list(rr[:P, 0]) == [(rank + 1 + i) % P for i in range(P)]
    assert rr[P - 1, 0] == rank                    # owned shard last in each round
    assert all(len(set(rr[i * P:(i + 1) * P, 0])) == P for i in range(per))
    assert np.array_equal(rr[::P, 1:3], rm[:per, 1:3])


def test_grouped_walk_visits_column_groups():
    M, N, P, rank, cfg = 8192, 2048, 2, 0, 2    # Tm = 32, Tn = 16
    Tm, Tn = _tiles(M, N, P, cfg)
    w = pk.pk_tile_walk(M, N, P, rank, cfg, 0, group_n=4)
    first = w[:Tm * 4]
    assert set(first[:, 2]) == {0, 1, 2, 3} and set(first[:, 1]) == set(range(Tm))


OWNED_R = 8          # owned sub-tiles per whole tile of configuration 1


@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("shape", [(4096, 4096, 8, 3), (2048, 768, 4, 0), (600, 520, 2, 1)])
def test_owned_split_walk_covers_every_item_once(order, shape):
    M, N, P, rank = shape
    Tm, Tn = _tiles(M, N, P, 1)
    w = pk.pk_tile_walk(M, N, P, rank, 1, order, 0, owned_split=1)
    assert w.shape == ((P - 1 + OWNED_R) * Tm * Tn, 4)
    keys = [tuple(r) for r in w.tolist()]
    assert len(set(keys)) == len(keys)
    want = {(d, t, u, -1) for d in range(P) if d != rank for t in range(Tm) for u in range(Tn)}
    want |= {(rank, t, u, q) for t in range(Tm) for u in range(Tn) for q in range(OWNED_R)}
    assert set(keys) == want


def test_owned_split_walk_pairs_send_tiles_with_owned_sub_tiles():
    """Under the split the walk is a list of pairs: send tile s (tile order,
    owned shard skipped) followed by owned sub-tile s (owned order)."""
    M, N, P, rank = 4096, 4096, 8, 3
    Tm, Tn = _tiles(M, N, P, 1)
    per = Tm * Tn
    whole = {o: pk.pk_tile_walk(M, N, P, rank, 1, o) for o in (0, 1, 2)}
    for order in (0, 1, 2):
        w = pk.pk_tile_walk(M, N, P, rank, 1, order, owned_split=1)
        sends = w[w[:, 3] < 0]
        owned = w[w[:, 3] >= 0]
        # send tiles keep the whole-tile order with the owned shard removed
        ref = whole[order][whole[order][:, 0] != rank]
        if order == 1:       # owned-first lists rank+1, ..., rank+P-1
            assert list(sends[::per, 0]) == [(rank + 1 + k) % P for k in range(P - 1)]
        else:
            assert np.array_equal(sends[:, :3], ref[:, :3])
        # owned sub-tiles: owned tile j // R, sub-tile j % R, in the owned shard's
        # order under this tile order (its column groups may differ by order)
        own_ref = whole[order][whole[order][:, 0] == rank]
        assert list(owned[:, 3]) == [j % OWNED_R for j in range(OWNED_R * per)]
        assert np.array_equal(owned[:, 1:3], np.repeat(own_ref[:, 1:3], OWNED_R, axis=0))
        # pairing: item 2s is send tile s, item 2s+1 its owned sub-tile
        n_pairs = min(len(sends), len(owned))
        assert np.array_equal(w[0:2 * n_pairs:2], sends[:n_pairs])
        assert np.array_equal(w[1:2 * n_pairs:2], owned[:n_pairs])
    rr = pk.pk_tile_walk(M, N, P, rank, 1, 2, owned_split=1)
    s_rr = rr[rr[:, 3] < 0]
    assert list(s_rr[:P - 1, 0]) == [(rank + 1 + j) % P for j in range(P - 1)]
    with pytest.raises(pk.PkError):
        pk.pk_tile_walk(M, N, P, rank, 2, 0, owned_split=1)          # configuration 1 only


# ---------------------------------------------------------------- chunk arrivals

@pytest.mark.parametrize("M,N,P,chunk,cfg", [(4096, 4096, 8, 128, 2), (256, 256, 2, 64, 3),
                                             (32768, 32768, 8, 1024, 1), (600, 200, 3, 8, 3),
                                             (600, 200, 3, 200, 2), (2400, 520, 3, 40, 1)])
def test_chunk_arrivals_count_overlapping_tiles(M, N, P, chunk, cfg):
    c = pk.pk_config_info(cfg)
    S = M // P
    Tm, Tn = _tiles(M, N, P, cfg)
    for ci in range(S // chunk):
        lo, hi = ci * chunk, (ci + 1) * chunk       # shard-local rows
        n = sum(1 for t in range(Tm)
                if max(lo, t * c["BM"]) < min(hi, min((t + 1) * c["BM"], S))) * Tn
        assert pk.pk_chunk_arrivals(M, N, P, chunk, cfg, ci) == n


def test_reduce_piece_words():
    assert pk.pk_reduce_piece_words(4096, 4096, 8) == 8 * 64
    assert pk.pk_reduce_piece_words(32768, 32768, 8) == 64 * 512
    assert pk.pk_reduce_piece_words(8 * 130, 72, 8) == 3 * 2        # ragged rows and columns
    assert pk.pk_reduce_piece_words(0, 64, 2) == 0
    with pytest.raises(pk.PkError):
        pk.pk_reduce_piece_words(100, 64, 3)
    with pytest.raises(pk.PkError):
        pk.pk_reduce_piece_words(128, 64, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(P=1, rank=0), -3), (dict(n_comm=0), -5), (dict(n_comm=-1), -5), (dict(n_comm=2000), -5),
    (dict(spin=0), -5),
    (dict(presum=0x70004), -1), (dict(presum=None), -1), (dict(piece_ready=None), -1),
    (dict(piece_ready=0x80002), -1), (dict(error=None), -1), (dict(peer_ready=0x90001), -1),
    (dict(out_bf16=1, presum=0x50000), -1), (dict(M=255), -2), (dict(tile_order=5), -4),
])
def test_intercu_reduce_rejects_before_any_hip_call(kw, code):
    """Argument errors come back before the entry point touches the device
    (fake but aligned pointers; a good call would launch)."""
    import ctypes
    lib = pk.load()
    a = dict(A=0x10000, B=0x20000, peers=0x30000, peer_ready=None, send=0x40000, out=0x50000,
             flags=0x60000, presum=0x70000, piece_ready=0x80000, error=0x90000, M=256, N=256,
             K=128, P=2, rank=0, chunk_rows=64, tile_order=0, out_bf16=0, expected=1, n_comm=8,
             spin=16)
    a.update(kw)
    vp = ctypes.c_void_p
    rc = lib.pk_gemm_rs_intercu_reduce(
        vp(a["A"]), vp(a["B"]), vp(a["peers"]), vp(a["peer_ready"]), vp(a["send"]),
        vp(a["out"]), vp(a["flags"]), vp(a["presum"]), vp(a["piece_ready"]), vp(a["error"]),
        a["M"], a["N"], a["K"], a["P"], a["rank"], a["chunk_rows"], a["tile_order"],
        a["out_bf16"], ctypes.c_uint32(a["expected"]), a["n_comm"], a["spin"], None, None)
    assert rc == code


# Gathered-row schedule (P = 8, S a multiple of 32): each row group of 256
# tile rows holds 224 send rows in slot order and 32 owned rows.
GATHER_SHAPES = [(4096, 4096, 8, 3, 128), (4096, 768, 8, 5, 64), (768, 1000, 8, 2, 32),
                 (1536, 328, 8, 0, 96), (256, 256, 8, 7, 32)]


@pytest.mark.parametrize("M,N,P,rank,cr", GATHER_SHAPES)
def test_gathered_rows_cover_every_row_once_in_slot_order(M, N, P, rank, cr):
    S = M // P
    groups = [pk.pk_gather_rows(P, rank, M, g) for g in range(S // 32)]
    assert sorted(np.concatenate(groups).tolist()) == list(range(M))
    send = []
    for g, r in enumerate(groups):
        for h in range(2):
            # tile rows 112..127 of each half: owned rows 32 g + 16 h ..
            assert (r[128 * h + 112:128 * h + 128] == rank * S + 32 * g + 16 * h + np.arange(16)).all()
            # the epilogue stores 16-row blocks of send rows: consecutive rows of one shard
            for b in range(7):
                blk = r[128 * h + 16 * b:128 * h + 16 * b + 16]
                assert (np.diff(blk) == 1).all() and blk[0] // S == blk[-1] // S != rank
            send.extend(r[128 * h:128 * h + 112].tolist())
    # all send rows, shard by shard in slot order (the owner skipped)
    assert send == [d * S + i for d in range(P) if d != rank for i in range(S)]


@pytest.mark.parametrize("M,N,P,rank,cr", GATHER_SHAPES)
def test_gathered_arrivals_are_what_the_work_items_make(M, N, P, rank, cr):
    exp, made = pk.pk_gather_arrivals(M, N, P, cr)
    assert exp.shape == (P - 1, M // P // cr)
    assert (exp > 0).all() and (exp == made).all()


def _gather_random_shapes(n, seed=5):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        S = 32 * int(rng.integers(1, 40))
        divs = [d for d in range(1, S + 1) if S % d == 0]
        out.append((8 * S, 8 * int(rng.integers(1, 200)), 8, int(rng.integers(0, 8)),
                    int(rng.choice(divs))))
    return out


@pytest.mark.parametrize("M,N,P,rank,cr", _gather_random_shapes(12))
def test_gathered_arrivals_brute_force(M, N, P, rank, cr):
    """Arrivals counted from the row lists themselves: a chunk waits for one
    arrival per column tile from every row group whose rows hold one of its
    rows."""
    S, Tn = M // P, -(-N // 256)
    want = np.zeros((P - 1, S // cr), np.int64)
    for g in range(S // 32):
        rows = pk.pk_gather_rows(P, rank, M, g)
        shard, lrow = rows // S, rows % S
        send = shard != rank
        slot = np.where(shard[send] < rank, shard[send], shard[send] - 1)
        for d, c in set(zip(slot.tolist(), (lrow[send] // cr).tolist())):
            want[d, c] += Tn
    exp, made = pk.pk_gather_arrivals(M, N, P, cr)
    assert np.array_equal(exp, want) and np.array_equal(made, want)


def test_gathered_arrivals_hand_counted():
    # S = 512, 16 column tiles, chunks of 128 rows: send rows 0..223 are group 0,
    # 224..447 group 1, 448..671 group 2, ...
    exp, _ = pk.pk_gather_arrivals(4096, 4096, 8, 128)
    assert exp[0, 0] == 16          # rows 0..127 of slot 0: group 0
    assert exp[0, 1] == 32          # rows 128..255: groups 0 and 1
    assert exp[0, 3] == 32          # rows 384..511: groups 1 and 2
    assert exp[1, 0] == 16          # send rows 512..639: group 2
    assert exp[6, 3] == 16          # send rows 3456..3583: group 15 only
    rows = pk.pk_gather_rows(8, 3, 4096, 0)
    assert rows[0] == 0 and rows[111] == 111 and rows[112] == 3 * 512 and rows[128] == 112
    assert rows[240] == 3 * 512 + 16


def test_gathered_rows_reject_shapes_that_do_not_fit():
    with pytest.raises(pk.PkError):
        pk.pk_gather_rows(4, 0, 1024, 0)          # P != 8
    with pytest.raises(pk.PkError):
        pk.pk_gather_rows(8, 0, 8 * 200, 0)       # S % 32
    with pytest.raises(pk.PkError):
        pk.pk_gather_rows(8, 0, 4096, 16)         # group past S / 32
    with pytest.raises(pk.PkError):
        pk.pk_gather_arrivals(8 * 200, 512, 8, 40)
