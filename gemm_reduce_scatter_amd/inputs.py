"""Seeded synthetic inputs and the workload table.

This module only draws numbers and names shapes: it holds none of the
method's arithmetic and imports neither the HIP library nor the oracle, so
both sides of every parity check can be fed the same bytes from here.

Recipe (the pages measure on synthetic bf16 matrices only, so the
distributions below stand in for them):

* every tensor is drawn with its own ``torch.Generator`` seeded from
  ``seed`` (A: seed, B: seed + 1, peer slot j: seed + 2 + j) on the device
  that will hold it; the same (seed, device kind) always gives the same bytes;
* real-valued tensors are drawn in float32, scaled in float32 and rounded to
  bf16 (round to nearest even) by torch;
* ``int`` twins draw A and B uniformly from {-2..2} and peers from {-8..8};
  every sum of such products stays an exact float32 integer, so float32 and
  float64 evaluation agree bit for bit.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

# Tile-order codes understood by the library (0 row-major, 1 owned-first,
# 2 destination round-robin).
ROW_MAJOR, OWNED_FIRST, DEST_ROUND_ROBIN = 0, 1, 2
TILE_ORDER_NAMES = {ROW_MAJOR: "row-major", OWNED_FIRST: "owned-first",
                    DEST_ROUND_ROBIN: "dest-round-robin"}


@dataclass(frozen=True)
class Workload:
    name: str
    P: int
    rank: int
    M: int
    N: int
    K: int
    chunk_rows: int
    ab_dist: str            # "uniform1", "uniform1_sqrtk", "normal_sqrtk", "int"
    peer_dist: str          # "uniform8", "normal", "int"
    out_dtype: str          # "f32" or "bf16"
    tile_order: int = ROW_MAJOR
    sweep_chunk_rows: tuple = field(default_factory=tuple)

    @property
    def S(self) -> int:
        return self.M // self.P

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def algorithmic_bytes(self) -> int:
        """A + B read once, send written once, peers read once, out written once."""
        s_out = 4 if self.out_dtype == "f32" else 2
        ab = 2 * (self.M * self.K + self.K * self.N)
        send = 2 * (self.P - 1) * self.S * self.N
        peers = 2 * (self.P - 1) * self.S * self.N
        out = s_out * self.S * self.N
        return ab + send + peers + out

    def epilogue_bytes(self) -> int:
        s_out = 4 if self.out_dtype == "f32" else 2
        return 4 * (self.P - 1) * self.S * self.N + s_out * self.S * self.N

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: one rank of a P-way tensor-parallel GEMM + reduce-scatter.
WORKLOADS = {
    "tiny": Workload("tiny", P=2, rank=0, M=256, N=256, K=128, chunk_rows=64,
                     ab_dist="uniform1", peer_dist="uniform8", out_dtype="f32"),
    "comm_dominant": Workload("comm_dominant", P=8, rank=3, M=4096, N=4096, K=512,
                              chunk_rows=128, ab_dist="normal_sqrtk", peer_dist="normal",
                              out_dtype="f32"),
    # dest-round-robin measured fastest of the three orders on these two shares
    # (by about 1 % at every chunk size); the large-K share is swept
    "near_threshold": Workload("near_threshold", P=8, rank=0, M=32768, N=32768, K=2048,
                               chunk_rows=256, ab_dist="normal_sqrtk", peer_dist="normal",
                               out_dtype="bf16", tile_order=DEST_ROUND_ROBIN),
    "compute_bound": Workload("compute_bound", P=8, rank=5, M=32768, N=32768, K=4096,
                              chunk_rows=512, ab_dist="uniform1_sqrtk", peer_dist="normal",
                              out_dtype="bf16", tile_order=DEST_ROUND_ROBIN),
    "large_k": Workload("large_k", P=8, rank=7, M=32768, N=32768, K=8192,
                        chunk_rows=512, ab_dist="normal_sqrtk", peer_dist="normal",
                        out_dtype="bf16", sweep_chunk_rows=(128, 256, 512, 1024)),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _draw(shape, dist: str, K: int, device, seed: int) -> torch.Tensor:
    g = _gen(device, seed)
    if dist == "int5":                    # {-2..2}
        return torch.randint(-2, 3, shape, generator=g, device=device,
                             dtype=torch.int32).to(torch.bfloat16)
    if dist == "int17":                   # {-8..8}
        return torch.randint(-8, 9, shape, generator=g, device=device,
                             dtype=torch.int32).to(torch.bfloat16)
    if dist in ("uniform1", "uniform1_sqrtk", "uniform8"):
        x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        x = x * 2.0 - 1.0
        if dist == "uniform8":
            x = x * 8.0
        elif dist == "uniform1_sqrtk":
            x = x * torch.tensor(1.0 / math.sqrt(K), dtype=torch.float32)
        return x.to(torch.bfloat16)
    if dist in ("normal", "normal_sqrtk"):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if dist == "normal_sqrtk":
            x = x * torch.tensor(1.0 / math.sqrt(K), dtype=torch.float32)
        return x.to(torch.bfloat16)
    raise ValueError(f"unknown distribution {dist!r}")


def make_operands(w: Workload, device="cpu", seed: int = 0, integer: bool = False):
    """A [M,K] and B [K,N] only: the same bytes make_inputs draws for them."""
    ab = "int5" if integer else w.ab_dist
    if ab == "int":
        ab = "int5"
    return _draw((w.M, w.K), ab, w.K, device, seed), _draw((w.K, w.N), ab, w.K, device, seed + 1)


def make_inputs(w: Workload, device="cpu", seed: int = 0, integer: bool = False):
    """A [M,K], B [K,N], peers [P-1,S,N] as bf16 tensors on ``device``."""
    pd = "int17" if integer else w.peer_dist
    if pd == "int":
        pd = "int17"
    A, B = make_operands(w, device, seed, integer)
    peers = torch.empty((max(w.P - 1, 0), w.S, w.N), dtype=torch.bfloat16, device=device)
    for j in range(w.P - 1):
        peers[j] = _draw((w.S, w.N), pd, w.K, device, seed + 2 + j)
    return A, B, peers


def make_probe_inputs(w: Workload, kind: str, device="cpu"):
    """Index-encoding inputs: every element of C names its row or column.

    kind "row_lo": C[i][n] = i mod 256; "row_hi": C[i][n] = (i // 256) mod 256;
    "col": C[i][n] = n mod 256.  All values are exact small integers in bf16,
    peers are zero.
    """
    A = torch.zeros((w.M, w.K), dtype=torch.float32)
    B = torch.zeros((w.K, w.N), dtype=torch.float32)
    rows = torch.arange(w.M, dtype=torch.int64)
    cols = torch.arange(w.N, dtype=torch.int64)
    if kind == "row_lo":
        A[:, 0] = (rows % 256).to(torch.float32)
        B[0, :] = 1.0
    elif kind == "row_hi":
        A[:, 0] = ((rows // 256) % 256).to(torch.float32)
        B[0, :] = 1.0
    elif kind == "col":
        A[:, 0] = 1.0
        B[0, :] = (cols % 256).to(torch.float32)
    else:
        raise ValueError(kind)
    peers = torch.zeros((max(w.P - 1, 0), w.S, w.N), dtype=torch.bfloat16)
    return (A.to(torch.bfloat16).to(device), B.to(torch.bfloat16).to(device),
            peers.to(device))


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def f32_array(t: torch.Tensor):
    return t.detach().to("cpu").contiguous().numpy()
