// Tile walk and chunk bookkeeping for the fused GEMM + reduce-scatter share.
//
// Shared by the device kernel and the host-side validator/planner (plain
// inline C++, no HIP types).  The output M x N is split into P row shards of
// S = M / P rows; every shard is tiled on its own, so a tile never straddles
// two shards and every shard has the same tile grid:
//
//   Tm = ceil(S / BM) row tiles,  Tn = ceil(N / BN) column tiles,
//   tile (d, t, u) covers shard-local rows [t*BM, min((t+1)*BM, S)) of
//   shard d and columns [u*BN, min((u+1)*BN, N)).
//
// Chunks follow Syncopate section 5.1 ("Communication Schedule
// Abstraction"): a chunk is a logical block of one or more tiles moved as one
// unit; here chunk c of a destination is shard-local rows
// [c*chunk_rows, (c+1)*chunk_rows) at full width.  A chunk's ready word is
// raised by the last tile that writes into it, so the number of arrivals a
// chunk waits for is (row tiles overlapping it) x Tn.
//
// Owned split: the owned shard may be tiled finer than the send shards.
// Every owned tile is then cut into R = Rm x Rn sub-tiles of (BM/Rm) x
// (BN/Rn), each its own work item, so that the heavy owned epilogue (it
// reads P-1 staged partials per element) is spread over many workgroups
// instead of falling on the few that hold whole owned tiles.  R = 1 keeps
// whole tiles.  Under the split the walk is a list of pairs: position s
// holds send tile s (in the tile order, owned shard skipped) and owned
// sub-tile s (in the owned shard's own order), either of which may be
// missing past the end of its list; the workgroup that runs the pair reads
// the sub-tile's peer partials while it multiplies the send tile.
//
// Tile orders (the order work items are handed out; results never depend on
// it, Syncopate section 5.2 "Tile-Scheduler Swizzling" reorders waves the same
// way without moving data):
//   0 row-major:        shards 0 .. P-1, each shard chunk-major;
//   1 owned-first:      shards rank, rank+1, ..., rank+P-1 (mod P);
//   2 dest-round-robin: position s takes tile s/P of shard (rank+1+s) mod P,
//                       so consecutive tiles go to different destinations
//                       and the owned shard comes last in every round.
// Under the owned split the order applies to the send tiles (owned-first
// then lists shards rank+1, ..., rank+P-1, each owned sub-tile riding with
// its send tile).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define PK_HD __host__ __device__ __forceinline__
#else
#define PK_HD inline
#endif

namespace pk {

enum TileOrder : int { kRowMajor = 0, kOwnedFirst = 1, kDestRoundRobin = 2 };

struct TileCoord {
  int shard;   // owning rank of the tile's rows
  int t;       // shard-local row-tile index
  int u;       // column-tile index
  int sub;     // -1: the whole tile; else owned sub-tile index in [0, Rm*Rn)
};

struct Grid {
  int P, rank, S, N, BM, BN, Tm, Tn, order, group_n;
  int Rm, Rn;  // owned split (1 x 1: none)
  PK_HD long long tiles_per_shard() const { return (long long)Tm * Tn; }
  PK_HD int R() const { return Rm * Rn; }
  PK_HD long long total() const { return tiles_per_shard() * (P - 1 + R()); }
};

PK_HD int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Position i (0 <= i < Tm*Tn) of the walk inside one shard.  Column tiles are
// visited in groups of `group_n`: inside a group, all row tiles of a group of
// columns before the next group.  group_n == Tn gives plain row-major
// (chunk-major) order; smaller groups keep the A and B panels that run side
// by side small enough to stay in cache.
PK_HD void intra_shard(const Grid& g, long long i, int& t, int& u) {
  const int gn = g.group_n <= 0 || g.group_n > g.Tn ? g.Tn : g.group_n;
  const long long per_group = (long long)g.Tm * gn;
  const long long grp = i / per_group;
  const long long r = i - grp * per_group;
  const int u0 = (int)grp * gn;
  const int width = (g.Tn - u0) < gn ? (g.Tn - u0) : gn;   // last group may be narrow
  t = (int)(r / width);
  u = u0 + (int)(r - (long long)t * width);
}

// Whole tile at walk position s (0 <= s < P*Tm*Tn) when there is no owned
// split.
PK_HD TileCoord tile_at(const Grid& g, long long s) {
  TileCoord c;
  const long long per = g.tiles_per_shard();
  long long i;
  if (g.order == kDestRoundRobin) {
    c.shard = (int)((g.rank + 1 + s % g.P) % g.P);
    i = s / g.P;
  } else if (g.order == kOwnedFirst) {
    c.shard = (int)((g.rank + s / per) % g.P);
    i = s % per;
  } else {
    c.shard = (int)(s / per);
    i = s % per;
  }
  intra_shard(g, i, c.t, c.u);
  c.sub = -1;
  return c;
}

// Owned sub-tile j of the owned shard under the split (0 <= j < R*Tm*Tn).
PK_HD TileCoord owned_item(const Grid& g, long long j) {
  TileCoord c;
  const int R = g.R();
  const long long i = j / R;
  c.shard = g.rank;
  c.sub = (int)(j - i * R);
  intra_shard(g, i, c.t, c.u);
  return c;
}

// Send tile i (0 <= i < (P-1)*Tm*Tn) in the tile order, the owned shard
// skipped.
PK_HD TileCoord send_item(const Grid& g, long long i) {
  TileCoord c;
  const long long per = g.tiles_per_shard();
  long long k, r;
  if (g.order == kDestRoundRobin) {
    k = i % (g.P - 1);
    r = i / (g.P - 1);
    c.shard = (int)((g.rank + 1 + k) % g.P);
  } else {
    k = i / per;
    r = i - k * per;
    if (g.order == kOwnedFirst) c.shard = (int)((g.rank + 1 + k) % g.P);
    else c.shard = k < g.rank ? (int)k : (int)k + 1;
  }
  c.sub = -1;
  intra_shard(g, r, c.t, c.u);
  return c;
}

// Under the split: the pair at walk position s (0 <= s < pairs()).
PK_HD long long split_sends(const Grid& g) { return g.tiles_per_shard() * (g.P - 1); }
PK_HD long long split_owned(const Grid& g) { return g.tiles_per_shard() * g.R(); }
PK_HD long long split_pairs(const Grid& g) {
  return split_sends(g) > split_owned(g) ? split_sends(g) : split_owned(g);
}

// Send slot of destination d (d != rank): ranks in ascending order, skipping
// the caller.
PK_HD int slot_of(int d, int rank) { return d < rank ? d : d - 1; }

// Chunks [c_first, c_last] touched by shard-local row tile t.
PK_HD void chunks_of_row_tile(int t, int BM, int S, int chunk_rows, int& c_first, int& c_last) {
  const long long r0 = (long long)t * BM;
  long long r1 = r0 + BM;
  if (r1 > S) r1 = S;
  c_first = (int)(r0 / chunk_rows);
  c_last = (int)((r1 - 1) / chunk_rows);
}

// Number of tile arrivals chunk c waits for.
PK_HD unsigned expected_arrivals(int c, int BM, int chunk_rows, int Tn) {
  const long long r0 = (long long)c * chunk_rows;
  const long long r1 = r0 + chunk_rows - 1;
  return (unsigned)((r1 / BM - r0 / BM + 1) * (long long)Tn);
}

// Gathered-row tiles (P = 8, S a multiple of 32; configuration 1's 256 x 256
// tile).  Instead of whole tiles of one shard, the M rows are cut into S/32
// row groups of 256: group g holds send rows 224 g .. 224 g + 223 (the P-1
// send shards' rows one after another in slot order) and owned rows
// 32 g .. 32 g + 31.  Tile rows 112 .. 127 of each 128-row half h are owned
// rows 32 g + 16 h .. + 15, the others send rows 224 g + 112 h + r.  Each
// row group x column tile is one work item, (S/32) * Tn of them, and each
// holds both send rows and a slice of the owned shard, so no work item is all
// owned rows.  A 16-row block of send rows that starts at a multiple of 16
// never straddles two shards (S is a multiple of 32).
constexpr int kGatherRows = 256, kGatherSendRows = 224, kGatherOwnedRows = 32;

PK_HD bool gather_fits(int P, long long S) { return P == 8 && S > 0 && S % kGatherOwnedRows == 0; }
PK_HD int gather_groups(long long S) { return (int)(S / kGatherOwnedRows); }

// Send row sr (0 <= sr < (P-1) S, slot order) -> its slot and shard-local row.
PK_HD void gather_send_row(int sr, int S, int& slot, int& lrow) {
  slot = sr / S;
  lrow = sr - slot * S;
}

// Row of the whole M x K operand A that tile row tr (0 .. 255) of row group g
// reads.
PK_HD long long gather_row(int rank, int S, int g, int tr) {
  const int h = tr >> 7, r = tr & 127;
  if (r >= 112) return (long long)rank * S + kGatherOwnedRows * g + 16 * h + (r - 112);
  int slot, lrow;
  gather_send_row(kGatherSendRows * g + 112 * h + r, S, slot, lrow);
  return (long long)(slot < rank ? slot : slot + 1) * S + lrow;
}

// Arrivals chunk c of send slot d waits for under the gathered rows: Tn from
// every row group whose send rows touch the chunk.
PK_HD unsigned gather_expected_arrivals(int d, int c, int S, int chunk_rows, int Tn) {
  const long long r0 = (long long)d * S + (long long)c * chunk_rows;
  const long long end = (long long)(c + 1) * chunk_rows < S ? (long long)(c + 1) * chunk_rows : S;
  const long long r1 = (long long)d * S + end - 1;
  return (unsigned)((r1 / kGatherSendRows - r0 / kGatherSendRows + 1) * (long long)Tn);
}

// The (slot, chunk) pairs row group g's send rows touch, in order, through
// visit(slot, chunk); returns how many.
template <class Visit>
PK_HD int gather_chunks(int g, int P, int S, int chunk_rows, const Visit& visit) {
  const int sr0 = kGatherSendRows * g, sr1 = sr0 + kGatherSendRows - 1;
  int n = 0;
  for (int d = sr0 / S; d <= sr1 / S && d < P - 1; ++d) {
    const int lo = sr0 > d * S ? sr0 - d * S : 0;
    const int hi = sr1 < (d + 1) * S - 1 ? sr1 - d * S : S - 1;
    for (int c = lo / chunk_rows; c <= hi / chunk_rows; ++c, ++n) visit(d, c);
  }
  return n;
}

}  // namespace pk
