"""ctypes binding of libpk_gemm_rs.so (declared in include/pk_gemm_rs.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, a negative return code becomes a
:class:`PkError`.  Every step of the computation runs in the HIP library; if
the library is missing this module raises instead of computing anything
itself.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libpk_gemm_rs.so"
_lib = None

ROW_MAJOR, OWNED_FIRST, DEST_ROUND_ROBIN = 0, 1, 2


class PkError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} (code {code})")
        self.code = code


class IncompleteError(RuntimeError):
    """A launch that waits on other workgroups gave some wait up (a grid that
    was not resident at once); ``words`` holds the status or error words."""

    def __init__(self, what: str, words):
        super().__init__(what)
        self.words = words


def read_words(words, stream=None):
    """Wait until `stream` (default: torch's current stream) has reached the
    end of the calls issued so far, then return the int32 status or error
    words as a numpy array."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    s.synchronize()
    return words.detach().cpu().numpy().view(np.int32).copy()


class _Options(ctypes.Structure):
    _fields_ = [("config", ctypes.c_int), ("max_workgroups", ctypes.c_int),
                ("group_n", ctypes.c_int), ("gemm_only", ctypes.c_int),
                ("owned_split", ctypes.c_int), ("signal_batch", ctypes.c_int),
                ("ready_clock", ctypes.c_void_p), ("store_policy", ctypes.c_int),
                ("timeline", ctypes.c_void_p)]


TIMELINE_LIB_NAME = "libpk_gemm_rs_timeline.so"


def lib_path(name: str = LIB_NAME) -> str:
    return os.path.join(_HERE, name)


def load():
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(lib_path())
    return _lib


def use_library(name: str = LIB_NAME):
    """Make every call below go to the library `name` in the package
    directory: LIB_NAME (the product) or TIMELINE_LIB_NAME (the same sources
    built with the phase recorder, for timing studies).  Returns it."""
    global _lib
    _lib = _open(lib_path(name))
    return _lib


def _open(path: str):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    u32p = ctypes.POINTER(ctypes.c_uint32)
    main = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32]
    lib.pk_gemm_rs_local.argtypes = main + [vp]
    lib.pk_gemm_rs_local_bf16out.argtypes = main + [vp]
    lib.pk_gemm_rs_local_ex.argtypes = main + [i32, ctypes.POINTER(_Options), vp]
    for f in ("pk_gemm_rs_local", "pk_gemm_rs_local_bf16out", "pk_gemm_rs_local_ex"):
        getattr(lib, f).restype = i32
    lib.pk_flags_words.argtypes = [i32, i64, i32]
    lib.pk_flags_words.restype = i64
    lib.pk_validate.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32,
                                ctypes.POINTER(_Options)]
    lib.pk_validate.restype = i32
    lib.pk_config_count.argtypes = []
    lib.pk_config_count.restype = i32
    ip = ctypes.POINTER(i32)
    lib.pk_config_info.argtypes = [i32, ip, ip, ip, ip, ip, ip]
    lib.pk_config_info.restype = i32
    lib.pk_select_config.argtypes = [i64, i64, i64, i32]
    lib.pk_select_config.restype = i32
    lib.pk_tile_walk.argtypes = [i64, i64, i32, i32, i32, i32, i32, i32,
                                 ctypes.POINTER(ctypes.c_int32), i64]
    lib.pk_tile_walk.restype = i64
    lib.pk_chunk_arrivals.argtypes = [i64, i64, i32, i32, i32, i32]
    lib.pk_chunk_arrivals.restype = i64
    lib.pk_gather_rows.argtypes = [i32, i32, i64, i32, ctypes.POINTER(ctypes.c_int64)]
    lib.pk_gather_rows.restype = i32
    lib.pk_gather_arrivals.argtypes = [i64, i64, i32, i32, ctypes.POINTER(ctypes.c_uint32),
                                       ctypes.POINTER(ctypes.c_uint32)]
    lib.pk_gather_arrivals.restype = i32
    lib.pk_strerror.argtypes = [i32]
    lib.pk_strerror.restype = ctypes.c_char_p
    lib.pk_version.argtypes = []
    lib.pk_version.restype = i32
    lib.pk_rs_consume.argtypes = [vp, vp, vp, i64, i64, i32, i32, ctypes.c_uint32, i32, vp, vp,
                                  i32, vp]
    lib.pk_rs_consume.restype = i32
    lib.pk_gemm_rs_push.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32,
                                    ctypes.POINTER(_Options), vp]
    lib.pk_gemm_rs_push.restype = i32
    lib.pk_ag_gemm.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32,
                               ctypes.c_uint32, i32, i32, ctypes.POINTER(_Options), vp]
    lib.pk_ag_gemm.restype = i32
    lib.pk_gemm_rs_intercu.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                       i32, i32, i32, ctypes.c_uint32, i32, i32,
                                       ctypes.POINTER(_Options), vp]
    lib.pk_gemm_rs_intercu.restype = i32
    lib.pk_gemm_rs_intercu_reduce.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                              i64, i32, i32, i32, i32, i32, ctypes.c_uint32,
                                              i32, i32, ctypes.POINTER(_Options), vp]
    lib.pk_gemm_rs_intercu_reduce.restype = i32
    lib.pk_reduce_piece_words.argtypes = [i64, i64, i32]
    lib.pk_reduce_piece_words.restype = i64
    lib.pk_gemm_rs_intercu_reduce_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                                     i64, i32, i32, i32, i32, i32,
                                                     ctypes.c_uint32, i32, i32,
                                                     ctypes.POINTER(_Options), vp]
    lib.pk_gemm_rs_intercu_reduce_static.restype = i32
    lib.pk_static_workspace_limits.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.pk_static_workspace_limits.restype = i64
    del u32p
    return lib


def pk_strerror(code: int) -> str:
    return load().pk_strerror(int(code)).decode()


def _check(code: int) -> int:
    if code < 0:
        raise PkError(code, pk_strerror(code))
    return code


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _opts(config=0, max_workgroups=0, group_n=0, gemm_only=False, owned_split=0,
          signal_batch=0, ready_clock=None, store_policy=0, timeline=None):
    if timeline is not None and (timeline.numel() * timeline.element_size() < TIMELINE_BYTES
                                 or not timeline.is_contiguous()):
        raise ValueError(f"timeline must be a contiguous buffer of {TIMELINE_BYTES} bytes")
    return _Options(int(config), int(max_workgroups), int(group_n), 1 if gemm_only else 0,
                    int(owned_split), int(signal_batch),
                    None if ready_clock is None else ready_clock.data_ptr(), int(store_policy),
                    None if timeline is None else timeline.data_ptr())


# Phase record of the instrumented timing build: 2048 workgroups x 32 uint64.
TIMELINE_WORKGROUPS, TIMELINE_SLOTS = 2048, 32
TIMELINE_BYTES = TIMELINE_WORKGROUPS * TIMELINE_SLOTS * 8


def _check_tensors(A, B, peer_partials, send_bufs, out, flags):
    import torch
    for name, t in (("A", A), ("B", B), ("peer_partials", peer_partials),
                    ("send_bufs", send_bufs), ("out", out), ("flags", flags)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in (("A", A), ("B", B), ("peer_partials", peer_partials), ("send_bufs", send_bufs)):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    if flags is not None and flags.dtype not in (torch.int32, torch.uint32):
        raise ValueError("flags must be a 32-bit integer tensor")


def _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows,
                 out_bf16, gemm_only=False):
    """Reject buffers smaller than the kernel reads or writes for these sizes.

    The library sees plain pointers and cannot check this itself.  Argument
    errors it does detect (M not a multiple of P, bad chunk_rows, ...) are left
    to it, so this check only runs on sizes it would accept.
    """
    M, N, K, P = int(M), int(N), int(K), int(P)
    if P < 1 or M <= 0 or N <= 0 or K < 0 or M % P:
        return                    # rejected by the library, or a no-op touching no buffer
    S = M // P
    need = [("A", A, 2 * M * K), ("B", B, 2 * K * N),
            ("out", out, 2 * M * N if gemm_only else (2 if out_bf16 else 4) * S * N)]
    if not gemm_only:
        need += [("peer_partials", peer_partials, 2 * (P - 1) * S * N),
                 ("send_bufs", send_bufs, 2 * (P - 1) * S * N)]
        words = load().pk_flags_words(P, M, int(chunk_rows))
        if words >= 0:
            need.append(("flags", flags, 4 * words))
    for name, t, nbytes in need:
        if t is not None and t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, "
                             f"the call needs {nbytes}")


def pk_gemm_rs_local(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank,
                     chunk_rows, tile_order, stream=None) -> int:
    """Fused share with a float32 ``out``; asynchronous on ``stream``."""
    _check_tensors(A, B, peer_partials, send_bufs, out, flags)
    _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows, 0)
    return _check(load().pk_gemm_rs_local(
        _ptr(A), _ptr(B), _ptr(peer_partials), _ptr(send_bufs), _ptr(out), _ptr(flags),
        int(M), int(N), int(K), int(P), int(rank), int(chunk_rows), int(tile_order),
        _stream(stream)))


def pk_gemm_rs_local_bf16out(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank,
                             chunk_rows, tile_order, stream=None) -> int:
    """Fused share with a bf16 ``out``; asynchronous on ``stream``."""
    _check_tensors(A, B, peer_partials, send_bufs, out, flags)
    _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows, 1)
    return _check(load().pk_gemm_rs_local_bf16out(
        _ptr(A), _ptr(B), _ptr(peer_partials), _ptr(send_bufs), _ptr(out), _ptr(flags),
        int(M), int(N), int(K), int(P), int(rank), int(chunk_rows), int(tile_order),
        _stream(stream)))


def pk_gemm_rs_local_ex(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank,
                        chunk_rows, tile_order, out_bf16, config=0, max_workgroups=0,
                        group_n=0, gemm_only=False, owned_split=0, signal_batch=0,
                        ready_clock=None, store_policy=0, timeline=None, stream=None) -> int:
    """Fused share with explicit tile configuration / grid / grouping options.

    ready_clock: None or a device int64 tensor of (P-1)*S/chunk_rows words that
    receives the device clock at which each chunk's ready word rose.
    timeline: None or a device buffer of TIMELINE_BYTES, filled only by the
    instrumented timing build (see use_library)."""
    _check_tensors(A, B, peer_partials, send_bufs, out, flags)
    _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows, out_bf16,
                 gemm_only)
    _check_clock(ready_clock, M, P, chunk_rows, gemm_only)
    o = _opts(config, max_workgroups, group_n, gemm_only, owned_split, signal_batch, ready_clock,
              store_policy, timeline)
    return _check(load().pk_gemm_rs_local_ex(
        _ptr(A), _ptr(B), _ptr(peer_partials), _ptr(send_bufs), _ptr(out), _ptr(flags),
        int(M), int(N), int(K), int(P), int(rank), int(chunk_rows), int(tile_order),
        int(out_bf16), ctypes.byref(o), _stream(stream)))


def _chunks(M, P, chunk_rows) -> int:
    M, P, chunk_rows = int(M), int(P), int(chunk_rows)
    if P < 2 or M <= 0 or chunk_rows <= 0 or M % P or (M // P) % chunk_rows:
        return 0
    return (P - 1) * ((M // P) // chunk_rows)


def _check_clock(ready_clock, M, P, chunk_rows, gemm_only=False):
    import torch
    if ready_clock is None:
        return
    if gemm_only:
        raise ValueError("ready_clock needs the fused share (gemm_only off)")
    if not ready_clock.is_cuda or not ready_clock.is_contiguous() or \
            ready_clock.dtype not in (torch.int64, torch.uint64):
        raise ValueError("ready_clock must be a contiguous 64-bit device tensor")
    if ready_clock.numel() < _chunks(M, P, chunk_rows):
        raise ValueError("ready_clock needs one word per chunk")


def pk_gemm_rs_push(A, B, accum, flags, M, N, K, P, rank, chunk_rows, tile_order, config=0,
                    max_workgroups=0, group_n=0, signal_batch=0, ready_clock=None,
                    stream=None) -> int:
    """Atomic push variant: accum[d] += this rank's partial rows of shard d for
    every owner d (fp32 atomics); see pk_gemm_rs.h."""
    import torch
    _check_tensors(A, B, None, None, accum, flags)
    if accum.dtype != torch.float32:
        raise ValueError("accum must be float32")
    M_, N_, K_, P_ = int(M), int(N), int(K), int(P)
    if P_ >= 1 and M_ > 0 and N_ > 0 and K_ >= 0 and M_ % P_ == 0:
        need = [("A", A, 2 * M_ * K_), ("B", B, 2 * K_ * N_), ("accum", accum, 4 * M_ * N_)]
        words = load().pk_flags_words(P_, M_, int(chunk_rows))
        if words >= 0:
            need.append(("flags", flags, 4 * words))
        for name, t, nbytes in need:
            if t is not None and t.numel() * t.element_size() < nbytes:
                raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, "
                                 f"the call needs {nbytes}")
    _check_clock(ready_clock, M, P, chunk_rows)
    o = _opts(config, max_workgroups, group_n, False, 0, signal_batch, ready_clock)
    return _check(load().pk_gemm_rs_push(
        _ptr(A), _ptr(B), _ptr(accum), _ptr(flags), M_, N_, K_, P_, int(rank), int(chunk_rows),
        int(tile_order), ctypes.byref(o), _stream(stream)))


class BoundPush:
    """pk_gemm_rs_push with its arguments checked and marshalled once; calling
    the object launches it again (see BoundCall)."""

    def __init__(self, A, B, accum, flags, M, N, K, P, rank, chunk_rows, tile_order, config=0,
                 max_workgroups=0, group_n=0, signal_batch=0, stream=None):
        import torch
        _check_tensors(A, B, None, None, accum, flags)
        if accum.dtype != torch.float32 or accum.numel() < int(M) * int(N):
            raise ValueError("accum must be float32 [P][S][N]")
        self._keep = (A, B, accum, flags)
        self._opts = _opts(config, max_workgroups, group_n, False, 0, signal_batch)
        self._fn = load().pk_gemm_rs_push
        self._args = (_ptr(A), _ptr(B), _ptr(accum), _ptr(flags), int(M), int(N), int(K),
                      int(P), int(rank), int(chunk_rows), int(tile_order),
                      ctypes.byref(self._opts), _stream(stream))

    def __call__(self) -> int:
        return _check(self._fn(*self._args))


def _ag_args(A, a_ready, B, C, error, M, N, K, P, rank, chunk_rows):
    import torch
    for name, t in (("A", A), ("B", B), ("C", C), ("a_ready", a_ready), ("error", error)):
        if t is None:
            if int(P) > 1 and name in ("a_ready", "error"):
                raise ValueError(f"{name} is required when P > 1")
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    for name, t in (("A", A), ("B", B), ("C", C)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    M_, N_, K_, P_ = int(M), int(N), int(K), int(P)
    if P_ >= 1 and M_ > 0 and N_ > 0 and K_ >= 0 and M_ % P_ == 0:
        need = [("A", A, 2 * M_ * K_), ("B", B, 2 * K_ * N_), ("C", C, 2 * M_ * N_)]
        S = M_ // P_
        if P_ > 1 and int(chunk_rows) > 0 and S % int(chunk_rows) == 0:
            need.append(("a_ready", a_ready, 4 * P_ * (S // int(chunk_rows))))
        for name, t, nbytes in need:
            if t is not None and t.numel() * t.element_size() < nbytes:
                raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, "
                                 f"the call needs {nbytes}")


def pk_ag_gemm(A, a_ready, B, C, error, M, N, K, P, rank, chunk_rows, expected,
               spin_limit=1 << 16, tile_order=1, config=0, max_workgroups=0, group_n=0,
               store_policy=0, stream=None) -> int:
    """All-gather + GEMM: C = A_gathered * B, each tile of another rank's rows
    waiting for its A chunks' ready words (see pk_gemm_rs.h)."""
    _ag_args(A, a_ready, B, C, error, M, N, K, P, rank, chunk_rows)
    o = _opts(config, max_workgroups, group_n, store_policy=store_policy)
    return _check(load().pk_ag_gemm(
        _ptr(A), _ptr(a_ready), _ptr(B), _ptr(C), _ptr(error), int(M), int(N), int(K), int(P),
        int(rank), int(chunk_rows), ctypes.c_uint32(int(expected) & 0xFFFFFFFF),
        int(spin_limit), int(tile_order), ctypes.byref(o), _stream(stream)))


class BoundAgGemm:
    """pk_ag_gemm with its arguments checked and marshalled once (see BoundCall)."""

    def __init__(self, A, a_ready, B, C, error, M, N, K, P, rank, chunk_rows, expected,
                 spin_limit=1 << 16, tile_order=1, config=0, max_workgroups=0, group_n=0,
                 store_policy=0, stream=None):
        _ag_args(A, a_ready, B, C, error, M, N, K, P, rank, chunk_rows)
        self._keep = (A, a_ready, B, C, error)
        self._opts = _opts(config, max_workgroups, group_n, store_policy=store_policy)
        self._fn = load().pk_ag_gemm
        self._args = (_ptr(A), _ptr(a_ready), _ptr(B), _ptr(C), _ptr(error), int(M), int(N),
                      int(K), int(P), int(rank), int(chunk_rows),
                      ctypes.c_uint32(int(expected) & 0xFFFFFFFF), int(spin_limit),
                      int(tile_order), ctypes.byref(self._opts), _stream(stream))

    def __call__(self) -> int:
        return _check(self._fn(*self._args))


class BoundInterCU:
    """pk_gemm_rs_intercu with its arguments checked and marshalled once;
    calling the object launches call `expected` (the value the call raises
    the ready words to), which the caller advances between launches with
    next()."""

    def __init__(self, A, B, peer_partials, send_bufs, out, flags, dest, status, M, N, K, P,
                 rank, chunk_rows, tile_order, out_bf16, expected, num_comm_cus,
                 spin_limit=1 << 16, config=0, max_workgroups=0, group_n=0, owned_split=0,
                 signal_batch=0, store_policy=0, stream=None):
        import torch
        _check_tensors(A, B, peer_partials, send_bufs, out, flags)
        _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows,
                     out_bf16)
        for name, t in (("dest", dest), ("status", status)):
            if t is None or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous device tensor")
        n = _chunks(M, P, chunk_rows)
        if n > 0:
            need = 2 * (int(P) - 1) * (int(M) // int(P)) * int(N)
            if dest.numel() * dest.element_size() < need:
                raise ValueError("dest is smaller than the send buffers")
            if status.dtype != torch.int32 or status.numel() < n:
                raise ValueError("status must be int32 with one word per chunk")
        self._keep = (A, B, peer_partials, send_bufs, out, flags, dest, status)
        self._opts = _opts(config, max_workgroups, group_n, False, owned_split, signal_batch,
                           store_policy=store_policy)
        self._fn = load().pk_gemm_rs_intercu
        self._head = (_ptr(A), _ptr(B), _ptr(peer_partials), _ptr(send_bufs), _ptr(out),
                      _ptr(flags), _ptr(dest), _ptr(status), int(M), int(N), int(K), int(P),
                      int(rank), int(chunk_rows), int(tile_order), int(out_bf16))
        self._tail = (int(num_comm_cus), int(spin_limit), ctypes.byref(self._opts),
                      _stream(stream))
        self.expected = int(expected)

    def next(self):
        self.expected += 1

    def __call__(self) -> int:
        return _check(self._fn(*self._head, ctypes.c_uint32(self.expected & 0xFFFFFFFF),
                               *self._tail))

    def check(self, stream=None):
        """After the launches so far: the per-chunk status words; raises
        IncompleteError when a chunk was given up (its dest rows are not
        valid; send_bufs, out and flags always are)."""
        st = read_words(self._keep[7], stream)
        if np.any(st != 0):
            raise IncompleteError(f"{int(np.count_nonzero(st))} chunks were not moved", st)
        return st


def pk_gemm_rs_intercu(A, B, peer_partials, send_bufs, out, flags, dest, status, M, N, K, P,
                       rank, chunk_rows, tile_order, out_bf16, expected, num_comm_cus,
                       spin_limit=1 << 16, stream=None, **opts) -> int:
    """Fused share plus the move of every send chunk into dest by dedicated
    communicator workgroups, in one launch (see pk_gemm_rs.h)."""
    return BoundInterCU(A, B, peer_partials, send_bufs, out, flags, dest, status, M, N, K, P,
                        rank, chunk_rows, tile_order, out_bf16, expected, num_comm_cus,
                        spin_limit, stream=stream, **opts)()


def pk_reduce_piece_words(M, N, P) -> int:
    return _check(load().pk_reduce_piece_words(int(M), int(N), int(P)))


class BoundInterCUReduce:
    """pk_gemm_rs_intercu_reduce with its arguments checked and marshalled
    once; calling the object launches call `expected` (the value it raises
    the piece words to, and waits for on peer_ready), which the caller
    advances between launches with next()."""

    def __init__(self, A, B, peer_partials, send_bufs, out, flags, presum, piece_ready, error,
                 M, N, K, P, rank, chunk_rows, tile_order, out_bf16, expected, num_comm_cus,
                 spin_limit=1 << 16, peer_ready=None, config=0, max_workgroups=0, group_n=0,
                 owned_split=0, signal_batch=0, store_policy=0, stream=None):
        import torch
        _check_tensors(A, B, peer_partials, send_bufs, out, flags)
        _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows,
                     out_bf16)
        for name, t in (("presum", presum), ("piece_ready", piece_ready), ("error", error),
                        ("peer_ready", peer_ready)):
            if t is None:
                if name != "peer_ready":
                    raise ValueError(f"{name} is required")
                continue
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous device tensor")
        if presum.dtype != torch.float32:
            raise ValueError("presum must be float32")
        for name, t in (("piece_ready", piece_ready), ("error", error), ("peer_ready", peer_ready)):
            if t is not None and t.dtype not in (torch.int32, torch.uint32):
                raise ValueError(f"{name} must be a 32-bit integer tensor")
        M_, N_, P_ = int(M), int(N), int(P)
        if P_ >= 1 and M_ > 0 and N_ > 0 and M_ % P_ == 0:
            S = M_ // P_
            if presum.numel() < S * N_:
                raise ValueError(f"presum holds {presum.numel()} floats, needs {S * N_}")
            words = load().pk_reduce_piece_words(M_, N_, P_)
            if words >= 0 and piece_ready.numel() < words:
                raise ValueError(f"piece_ready holds {piece_ready.numel()} words, needs {words}")
            if error.numel() < 1:
                raise ValueError("error needs one word")
            n = _chunks(M, P, chunk_rows)
            if peer_ready is not None and n > 0 and peer_ready.numel() < n:
                raise ValueError("peer_ready needs one word per incoming chunk")
        self._keep = (A, B, peer_partials, send_bufs, out, flags, presum, piece_ready, error,
                      peer_ready)
        self._opts = _opts(config, max_workgroups, group_n, False, owned_split, signal_batch,
                           store_policy=store_policy)
        self._fn = load().pk_gemm_rs_intercu_reduce
        self._head = (_ptr(A), _ptr(B), _ptr(peer_partials), _ptr(peer_ready), _ptr(send_bufs),
                      _ptr(out), _ptr(flags), _ptr(presum), _ptr(piece_ready), _ptr(error),
                      M_, N_, int(K), P_, int(rank), int(chunk_rows), int(tile_order),
                      int(out_bf16))
        self._tail = (int(num_comm_cus), int(spin_limit), ctypes.byref(self._opts),
                      _stream(stream))
        self.expected = int(expected)

    def next(self):
        self.expected += 1

    def __call__(self) -> int:
        return _check(self._fn(*self._head, ctypes.c_uint32(self.expected & 0xFFFFFFFF),
                               *self._tail))

    def check(self, stream=None) -> int:
        """After the launches so far: the error word, or IncompleteError when
        it says `out` is not valid (pk_gemm_rs.h: bit 2, an incoming chunk
        given up; any bit when presum is out itself).  Bit 1 alone with a
        separate presum only reports that owned items summed their peers
        themselves."""
        presum, out, error = self._keep[6], self._keep[4], self._keep[8]
        return _check_reduce_error(read_words(error, stream)[0], presum.data_ptr() == out.data_ptr())


def _check_reduce_error(e: int, presum_is_out: bool) -> int:
    if (e & 2) or (e != 0 and presum_is_out):
        raise IncompleteError(f"reduction role gave up waits (error word {e}): out is not valid",
                              np.array([e], np.int32))
    return int(e)


class BoundInterCUReduceStatic:
    """pk_gemm_rs_intercu_reduce_static (workspace in the library's static
    device array) with its arguments checked and marshalled once; calling the
    object launches with `expected` for the incoming chunk words."""

    def __init__(self, A, B, peer_partials, send_bufs, out, flags, error, M, N, K, P, rank,
                 chunk_rows, tile_order, out_bf16, expected=0, num_comm_cus=0,
                 spin_limit=1 << 16, peer_ready=None, config=0, max_workgroups=0, group_n=0,
                 owned_split=0, signal_batch=0, store_policy=0, stream=None):
        import torch
        _check_tensors(A, B, peer_partials, send_bufs, out, flags)
        _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows,
                     out_bf16)
        for name, t in (("error", error), ("peer_ready", peer_ready)):
            if t is None:
                if name == "error":
                    raise ValueError("error is required")
                continue
            if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.int32,
                                                                          torch.uint32):
                raise ValueError(f"{name} must be a contiguous 32-bit integer device tensor")
        if error.numel() < 1:
            raise ValueError("error needs one word")
        n = _chunks(M, P, chunk_rows)
        if peer_ready is not None and n > 0 and peer_ready.numel() < n:
            raise ValueError("peer_ready needs one word per incoming chunk")
        self._keep = (A, B, peer_partials, send_bufs, out, flags, error, peer_ready)
        self._opts = _opts(config, max_workgroups, group_n, False, owned_split, signal_batch,
                           store_policy=store_policy)
        self._fn = load().pk_gemm_rs_intercu_reduce_static
        self._head = (_ptr(A), _ptr(B), _ptr(peer_partials), _ptr(peer_ready), _ptr(send_bufs),
                      _ptr(out), _ptr(flags), _ptr(error), int(M), int(N), int(K), int(P),
                      int(rank), int(chunk_rows), int(tile_order), int(out_bf16))
        self._tail = (int(num_comm_cus), int(spin_limit), ctypes.byref(self._opts),
                      _stream(stream))
        self.expected = int(expected)

    def __call__(self) -> int:
        return _check(self._fn(*self._head, ctypes.c_uint32(self.expected & 0xFFFFFFFF),
                               *self._tail))

    def check(self, stream=None) -> int:
        """The error word after the launches so far (see BoundInterCUReduce.check)."""
        return _check_reduce_error(read_words(self._keep[6], stream)[0], False)


def pk_gemm_rs_intercu_reduce_static(A, B, peer_partials, send_bufs, out, flags, error, M, N, K,
                                     P, rank, chunk_rows, tile_order, out_bf16, expected=0,
                                     num_comm_cus=0, spin_limit=1 << 16, peer_ready=None,
                                     stream=None, **opts) -> int:
    """The reduction role with its workspace in the library's static device
    array, for callers that cannot allocate (see pk_gemm_rs.h)."""
    return BoundInterCUReduceStatic(A, B, peer_partials, send_bufs, out, flags, error, M, N, K,
                                    P, rank, chunk_rows, tile_order, out_bf16, expected,
                                    num_comm_cus, spin_limit, peer_ready, stream=stream,
                                    **opts)()


def pk_static_workspace_limits():
    """(max (M/P)*N, max piece words, bytes per GPU) of the static workspace."""
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    nbytes = load().pk_static_workspace_limits(ctypes.byref(a), ctypes.byref(b))
    return int(a.value), int(b.value), int(nbytes)


def pk_gemm_rs_intercu_reduce(A, B, peer_partials, send_bufs, out, flags, presum, piece_ready,
                              error, M, N, K, P, rank, chunk_rows, tile_order, out_bf16,
                              expected, num_comm_cus, spin_limit=1 << 16, peer_ready=None,
                              stream=None, **opts) -> int:
    """Fused share whose owned-shard peer sum is done by dedicated reduction
    workgroups in the same launch (see pk_gemm_rs.h)."""
    return BoundInterCUReduce(A, B, peer_partials, send_bufs, out, flags, presum, piece_ready,
                              error, M, N, K, P, rank, chunk_rows, tile_order, out_bf16,
                              expected, num_comm_cus, spin_limit, peer_ready, stream=stream,
                              **opts)()


def pk_rs_consume(flags, send_bufs, dest, M, N, P, chunk_rows, expected, status,
                  observed=None, spin_limit=1 << 16, max_workgroups=0, stream=None) -> int:
    """Chunk consumer: wait for each chunk's ready word to reach `expected`,
    then copy the chunk from send_bufs to dest (see pk_gemm_rs.h)."""
    import torch
    for name, t in (("flags", flags), ("send_bufs", send_bufs), ("dest", dest),
                    ("status", status), ("observed", observed)):
        if t is None:
            if name != "observed":
                raise ValueError(f"{name} is required")
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    n = _chunks(M, P, chunk_rows)
    if n > 0:
        S = int(M) // int(P)
        need = 2 * (int(P) - 1) * S * int(N)
        for name, t in (("send_bufs", send_bufs), ("dest", dest)):
            if t.numel() * t.element_size() < need:
                raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {need}")
        if flags.numel() * flags.element_size() < 4 * n:
            raise ValueError("flags is shorter than the ready words")
        if status.dtype != torch.int32 or status.numel() < n:
            raise ValueError("status must be int32 with one word per chunk")
        if observed is not None and (observed.element_size() != 8 or observed.numel() < n):
            raise ValueError("observed must be 64-bit with one word per chunk")
    return _check(load().pk_rs_consume(
        _ptr(flags), _ptr(send_bufs), _ptr(dest), int(M), int(N), int(P), int(chunk_rows),
        ctypes.c_uint32(int(expected) & 0xFFFFFFFF), int(spin_limit), _ptr(status),
        _ptr(observed), int(max_workgroups), _stream(stream)))


class BoundCall:
    """pk_gemm_rs_local_ex with its tensors checked and its arguments marshalled
    once.  Calling the object launches the share again on ``stream`` (fixed at
    construction; None = torch's current stream at that time) with the same
    buffers, so a loop of launches pays only the foreign call.  The tensors
    must stay alive and unmoved while the object is used."""

    def __init__(self, A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank,
                 chunk_rows, tile_order, out_bf16, config=0, max_workgroups=0, group_n=0,
                 gemm_only=False, owned_split=0, signal_batch=0, ready_clock=None,
                 store_policy=0, timeline=None, stream=None):
        _check_tensors(A, B, peer_partials, send_bufs, out, flags)
        _check_sizes(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, chunk_rows,
                     out_bf16, gemm_only)
        _check_clock(ready_clock, M, P, chunk_rows, gemm_only)
        self._keep = (A, B, peer_partials, send_bufs, out, flags, ready_clock, timeline)
        self._opts = _opts(config, max_workgroups, group_n, gemm_only, owned_split, signal_batch,
                           ready_clock, store_policy, timeline)
        self._fn = load().pk_gemm_rs_local_ex
        self._args = (_ptr(A), _ptr(B), _ptr(peer_partials), _ptr(send_bufs), _ptr(out),
                      _ptr(flags), int(M), int(N), int(K), int(P), int(rank), int(chunk_rows),
                      int(tile_order), int(out_bf16), ctypes.byref(self._opts), _stream(stream))
        code = load().pk_validate(*self._args[:14], ctypes.byref(self._opts))
        _check(code)

    def __call__(self) -> int:
        return _check(self._fn(*self._args))


def pk_flags_words(P, M, chunk_rows) -> int:
    return _check(load().pk_flags_words(int(P), int(M), int(chunk_rows)))


def pk_validate(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                tile_order, out_bf16=0, config=0, max_workgroups=0, group_n=0,
                gemm_only=False, owned_split=0, signal_batch=0, store_policy=0) -> int:
    """Return code the library would give these arguments (no HIP call).

    Pointer arguments are plain integers (addresses) or None."""
    o = _opts(config, max_workgroups, group_n, gemm_only, owned_split, signal_batch,
              store_policy=store_policy)
    v = [None if p is None else ctypes.c_void_p(int(p)) for p in
         (A, B, peer_partials, send_bufs, out, flags)]
    return load().pk_validate(*v, int(M), int(N), int(K), int(P), int(rank), int(chunk_rows),
                              int(tile_order), int(out_bf16), ctypes.byref(o))


def pk_config_count() -> int:
    return load().pk_config_count()


def pk_config_info(cfg_id: int) -> dict:
    vals = [ctypes.c_int() for _ in range(6)]
    _check(load().pk_config_info(int(cfg_id), *[ctypes.byref(v) for v in vals]))
    return dict(zip(("BM", "BN", "BK", "WM", "WN", "threads"), (v.value for v in vals)))


def pk_select_config(M, N, K, P) -> int:
    return _check(load().pk_select_config(int(M), int(N), int(K), int(P)))


def pk_tile_walk(M, N, P, rank, config, tile_order, group_n=0, owned_split=0) -> np.ndarray:
    """The work walk as an int32 array [total, 4] of (shard, row tile, column tile,
    sub-tile); sub-tile is -1 for whole tiles."""
    lib = load()
    total = _check(lib.pk_tile_walk(int(M), int(N), int(P), int(rank), int(config),
                                    int(tile_order), int(group_n), int(owned_split), None, 0))
    buf = np.zeros((max(total, 1), 4), dtype=np.int32)
    _check(lib.pk_tile_walk(int(M), int(N), int(P), int(rank), int(config), int(tile_order),
                            int(group_n), int(owned_split),
                            buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(total)))
    return buf[:total]


def pk_chunk_arrivals(M, N, P, chunk_rows, config, c) -> int:
    return _check(load().pk_chunk_arrivals(int(M), int(N), int(P), int(chunk_rows),
                                           int(config), int(c)))


def pk_gather_rows(P, rank, M, g) -> np.ndarray:
    """Rows of A that tile rows 0..255 of row group g read under the
    gathered-row schedule (int64 [256])."""
    rows = np.zeros(256, dtype=np.int64)
    _check(load().pk_gather_rows(int(P), int(rank), int(M), int(g),
                                 rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return rows


def pk_gather_arrivals(M, N, P, chunk_rows):
    """(expected, made): arrivals each chunk of each send slot waits for under
    the gathered-row schedule and the arrivals its work items make, both
    uint32 [P-1][S/chunk_rows]."""
    n = (P - 1) * (M // P // chunk_rows) if P > 1 and chunk_rows > 0 else 0
    exp = np.zeros(max(n, 1), dtype=np.uint32)
    made = np.zeros(max(n, 1), dtype=np.uint32)
    _check(load().pk_gather_arrivals(int(M), int(N), int(P), int(chunk_rows),
                                     exp.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                     made.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))))
    shape = (P - 1, M // P // chunk_rows)
    return exp[:n].reshape(shape), made[:n].reshape(shape)


def pk_version() -> int:
    return load().pk_version()
