// libpk_gemm_rs: one GPU's share of a tile-fused bf16 GEMM + reduce-scatter
// for MI355X (gfx950, CDNA4).
//
// What is computed is stated in include/pk_gemm_rs.h.  The design follows
// the intra-SM overlap of the fused GEMM + reduce-scatter in "ParallelKittens:
// Systematic and Practical Simplification of Multi-GPU AI Kernels" (section 3,
// "Scheduling Analysis"): the workgroup that produces an output tile also
// ships it, so there are no dedicated communication CUs.  Differences from
// that design, for gfx950 and a single GPU:
//  * the owner does not receive atomic adds; it sums the staged peer partials
//    in a fixed order and stores once (deterministic, no atomics on data);
//  * tiles for other ranks go to per-destination chunked send buffers, and
//    the last tile of a chunk raises its ready word (chunks as in Syncopate,
//    section 5.1);
//  * the main loop is bf16 MFMA (v_mfma_f32_32x32x16_bf16) on 64-wide
//    wavefronts fed from LDS, double buffered;
//  * one persistent workgroup per CU slot walks the tile order; consecutive
//    walk positions go to the same XCD so tiles that share A/B panels share
//    that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pk_gemm_rs.h"
#include "pk_plan.h"

namespace pk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Tile configurations.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int FM = WM / 32, FN = WN / 32;   // 32x32 MFMA blocks per wave
  static constexpr int KCH = BK / 8;                 // 16-byte chunks per LDS row
  static constexpr int A_CHUNKS = BM * KCH;          // per stage
  static constexpr int B_CHUNKS = BN * KCH;
  static constexpr int A_PER_THREAD = A_CHUNKS / THREADS;
  static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);       // 8x8 element blocks
  static constexpr int B_PER_THREAD = (B_BLOCKS + THREADS - 1) / THREADS;
  static constexpr int STAGE_CHUNKS = A_CHUNKS + B_CHUNKS;
  static constexpr int LDS_MAIN = 2 * STAGE_CHUNKS * 16;     // bytes
  static constexpr int EPI_STRIDE = WN + 8;                  // floats per staged row
  static constexpr int LDS_EPI = WAVES * 32 * EPI_STRIDE * 4;
  static constexpr int LDS = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
  static_assert(A_CHUNKS % THREADS == 0, "A tile must split evenly over threads");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
};

// id 1..3; the table in pk_config_info mirrors these.
using Cfg1 = Cfg<256, 256, 128, 128>;
using Cfg2 = Cfg<128, 128, 64, 64>;
using Cfg3 = Cfg<64, 64, 32, 32>;

struct KArgs {
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* peers;
  uint16_t* send;
  void* out;
  uint32_t* flags;
  long long M, N, K;
  int P, rank, S, chunk_rows, n_chunks;
  int out_bf16, gemm_only;
  Grid g;
  long long total_tiles;
};

// LDS swizzle: 16-byte chunk c of row r lives at chunk c ^ swz(r), so 16
// consecutive rows read at one logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// One output tile: main loop + fused epilogue.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void load_a(const KArgs& a, const TileCoord& tc, int k0, int tid,
                                       u32x4 (&ra)[C::A_PER_THREAD]) {
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const int idx = tid + i * C::THREADS;
    const int r = idx / C::KCH, c = idx % C::KCH;
    const int lr = tc.t * C::BM + r;               // shard-local row
    const int k = k0 + c * 8;
    const bool ok = (lr < a.S) && (k < a.K);
    const uint16_t* p = a.A + ((long long)tc.shard * a.S + lr) * a.K + k;
    ra[i] = ok ? load16(p) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <class C>
__device__ __forceinline__ void load_b(const KArgs& a, const TileCoord& tc, int k0, int tid,
                                       u32x4 (&rb)[C::B_PER_THREAD][8]) {
#pragma unroll
  for (int i = 0; i < C::B_PER_THREAD; ++i) {
    const int b = tid + i * C::THREADS;
    const int kb = b / (C::BN / 8), nb = b % (C::BN / 8);
    const long long n = (long long)tc.u * C::BN + nb * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = k0 + kb * 8 + r;
      const bool ok = (b < C::B_BLOCKS) && (k < a.K) && (n < a.N);
      rb[i][r] = ok ? load16(a.B + (long long)k * a.N + n) : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <class C>
__device__ __forceinline__ void store_a(u32x4* lds_a, int tid, const u32x4 (&ra)[C::A_PER_THREAD]) {
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const int idx = tid + i * C::THREADS;
    const int r = idx / C::KCH, c = idx % C::KCH;
    lds_a[r * C::KCH + (c ^ swz(r))] = ra[i];
  }
}

// B arrives as 8 k-rows x 8 n-columns per thread and is stored transposed
// (n-major, k contiguous) so that each MFMA lane reads its 8 k-values of one
// column with a single 16-byte LDS read.
template <class C>
__device__ __forceinline__ void store_b(u32x4* lds_b, int tid, const u32x4 (&rb)[C::B_PER_THREAD][8]) {
#pragma unroll
  for (int i = 0; i < C::B_PER_THREAD; ++i) {
    const int b = tid + i * C::THREADS;
    if (b < C::B_BLOCKS) {
      const int kb = b / (C::BN / 8), nb = b % (C::BN / 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = j >> 1;
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = rb[i][2 * p][q], hi = rb[i][2 * p + 1][q];
          o[p] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int n = nb * 8 + j;
        lds_b[n * C::KCH + (kb ^ swz(n))] = o;
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void mma_stage(const u32x4* lds_a, const u32x4* lds_b, int wm, int wn,
                                          int lane, f32x16 (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int kk = 0; kk < C::BK / 16; ++kk) {
    const int ch = kk * 2 + (lane >> 5);
    bf16x8 af[C::FM], bf[C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int r = wm * C::WM + fm * 32 + (lane & 31);
      af[fm] = __builtin_bit_cast(bf16x8, lds_a[r * C::KCH + (ch ^ swz(r))]);
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int n = wn * C::WN + fn * 32 + (lane & 31);
      bf[fn] = __builtin_bit_cast(bf16x8, lds_b[n * C::KCH + (ch ^ swz(n))]);
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
  }
}

// Epilogue for 8 consecutive columns of one row of the tile.
__device__ __forceinline__ void emit8(const KArgs& a, const TileCoord& tc, int lr, long long col,
                                      const float (&v)[8]) {
  if (a.gemm_only) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((long long)tc.shard * a.S + lr) * a.N + col;
    *reinterpret_cast<u32x4*>(dst) = o;
    return;
  }
  if (tc.shard != a.rank) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
    const int slot = slot_of(tc.shard, a.rank);
    uint16_t* dst = a.send + ((long long)slot * a.S + lr) * a.N + col;
    *reinterpret_cast<u32x4*>(dst) = o;
    return;
  }
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = v[e];
  const long long base = (long long)lr * a.N + col;
  const long long slot_stride = (long long)a.S * a.N;
  for (int j = 0; j < a.P - 1; ++j) {          // ascending slot order
    const u32x4 pv = load16(a.peers + j * slot_stride + base);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      s[2 * p] += bf16lo(pv[p]);
      s[2 * p + 1] += bf16hi(pv[p]);
    }
  }
  if (a.out_bf16) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = pack_bf16x2(s[2 * p], s[2 * p + 1]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + base) = o;
  } else {
    float* dst = reinterpret_cast<float*>(a.out) + base;
    *reinterpret_cast<f32x4*>(dst) = f32x4{s[0], s[1], s[2], s[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{s[4], s[5], s[6], s[7]};
  }
}

// Ready-word protocol for one finished send tile.  Every thread has already
// made its stores visible device-wide (release fence) and the workgroup has
// met at a barrier.  One thread then adds an arrival to each chunk the tile
// touches; the arrival that completes a chunk (acquire-release on the
// counter) publishes the ready word with a release store and resets the
// counter for the next launch.
__device__ __forceinline__ void signal_chunks(const KArgs& a, const TileCoord& tc, int BM) {
  int c0, c1;
  chunks_of_row_tile(tc.t, BM, a.S, a.chunk_rows, c0, c1);
  const int slot = slot_of(tc.shard, a.rank);
  uint32_t* ready = a.flags;
  uint32_t* counters = a.flags + (long long)(a.P - 1) * a.n_chunks;
  for (int c = c0; c <= c1; ++c) {
    const int idx = slot * a.n_chunks + c;
    const uint32_t want = expected_arrivals(c, BM, a.chunk_rows, a.g.Tn);
    const uint32_t old = __hip_atomic_fetch_add(&counters[idx], 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == want) {
      __hip_atomic_store(&ready[idx], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&counters[idx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <class C>
__global__ void __launch_bounds__(C::THREADS) gemm_rs_kernel(KArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];
  u32x4* lds = reinterpret_cast<u32x4*>(smem);
  float* lds_f = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of walk positions.
  const int G = gridDim.x;
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (w & 7) * (G >> 3) + (w >> 3);

  const int nk = (int)((a.K + C::BK - 1) / C::BK);

  for (long long s = w; s < a.total_tiles; s += G) {
    const TileCoord tc = tile_at(a.g, s);

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 ra[C::A_PER_THREAD];
    u32x4 rb[C::B_PER_THREAD][8];
    if (nk > 0) {
      load_a<C>(a, tc, 0, tid, ra);
      load_b<C>(a, tc, 0, tid, rb);
      store_a<C>(lds, tid, ra);
      store_b<C>(lds + C::A_CHUNKS, tid, rb);
    }
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int cur = ks & 1;
      const bool more = ks + 1 < nk;
      if (more) {
        load_a<C>(a, tc, (ks + 1) * C::BK, tid, ra);
        load_b<C>(a, tc, (ks + 1) * C::BK, tid, rb);
      }
      const u32x4* st = lds + cur * C::STAGE_CHUNKS;
      mma_stage<C>(st, st + C::A_CHUNKS, wm, wn, lane, acc);
      if (more) {
        u32x4* nx = lds + (cur ^ 1) * C::STAGE_CHUNKS;
        store_a<C>(nx, tid, ra);
        store_b<C>(nx + C::A_CHUNKS, tid, rb);
      }
      __syncthreads();
    }

    // Epilogue: re-lay each 32-row stripe of the wave tile through LDS so
    // that every lane owns 8 consecutive columns of one row (16-byte global
    // accesses), then send, sum or store.
    float* stage = lds_f + wave * 32 * C::EPI_STRIDE;
    constexpr int LPR = C::WN / 8;                 // lanes per staged row
    constexpr int ROWS_PER_IT = 64 / LPR;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          stage[row * C::EPI_STRIDE + fn * 32 + (lane & 31)] = acc[fm][fn][r];
        }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 32 / ROWS_PER_IT; ++it) {
        const int rr = it * ROWS_PER_IT + lane / LPR;
        const int c8 = lane % LPR;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8 + 4);
        const float v[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        const int lr = tc.t * C::BM + wm * C::WM + fm * 32 + rr;
        const long long col = (long long)tc.u * C::BN + wn * C::WN + c8 * 8;
        if (lr < a.S && col < a.N) emit8(a, tc, lr, col, v);
      }
      __syncthreads();
    }

    if (!a.gemm_only && tc.shard != a.rank) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) signal_chunks(a, tc, C::BM);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: configuration table, validation, launch.
// ---------------------------------------------------------------------------
struct CfgInfo {
  int BM, BN, BK, WM, WN, threads;
};
static const CfgInfo kCfgs[] = {
    {Cfg1::BM, Cfg1::BN, Cfg1::BK, Cfg1::WM, Cfg1::WN, Cfg1::THREADS},
    {Cfg2::BM, Cfg2::BN, Cfg2::BK, Cfg2::WM, Cfg2::WN, Cfg2::THREADS},
    {Cfg3::BM, Cfg3::BN, Cfg3::BK, Cfg3::WM, Cfg3::WN, Cfg3::THREADS},
};
static constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
static constexpr int kAssumedCUs = 256;   // MI355X; used only for the static pick

static int default_group_n(const CfgInfo& c, int Tn) {
  (void)c;
  return Tn;
}

static int select_config(long long M, long long N, long long K, int P) {
  (void)K;
  const long long S = P > 0 ? M / P : 0;
  for (int i = 0; i < kNumCfgs; ++i) {
    const CfgInfo& c = kCfgs[i];
    if (S < c.BM || N < c.BN) continue;
    const long long tiles = (long long)P * ((S + c.BM - 1) / c.BM) * ((N + c.BN - 1) / c.BN);
    if (tiles >= 4LL * kAssumedCUs) return i + 1;
  }
  return kNumCfgs;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int validate(const void* A, const void* B, const void* peers, const void* send,
                    const void* out, const uint32_t* flags, long long M, long long N,
                    long long K, int P, int rank, int chunk_rows, int tile_order, int out_bf16,
                    const pk_options* o) {
  if (P < 1 || P > 64 || rank < 0 || rank >= P) return PK_ERR_RANK;
  if (tile_order < 0 || tile_order > 2) return PK_ERR_TILE_ORDER;
  if (M < 0 || N < 0 || K < 0) return PK_ERR_SHAPE;
  if (M % P != 0 || N % 8 != 0 || K % 8 != 0) return PK_ERR_SHAPE;
  if (out_bf16 != 0 && out_bf16 != 1) return PK_ERR_SHAPE;
  const long long S = M / P;
  const bool gemm_only = o && o->gemm_only;
  if (!gemm_only) {
    if (chunk_rows <= 0) {
      if (!(S == 0 && chunk_rows == 0)) return PK_ERR_SHAPE;
    } else if (S % chunk_rows != 0) {
      return PK_ERR_SHAPE;
    }
  }
  if (M > (1LL << 31) || N > (1LL << 31) || K > (1LL << 31)) return PK_ERR_TOO_LARGE;
  if (o && (o->config < 0 || o->config > kNumCfgs)) return PK_ERR_CONFIG;
  if (o && (o->max_workgroups < 0 || o->group_n < 0)) return PK_ERR_CONFIG;
  if (M == 0 || N == 0) return PK_OK;     // nothing to write
  auto need = [](const void* p) { return p != nullptr && aligned16(p); };
  if (!need(out)) return PK_ERR_POINTER;
  if (K > 0 && (!need(A) || !need(B))) return PK_ERR_POINTER;
  if (!gemm_only && P > 1) {
    if (!need(peers) || !need(send) || flags == nullptr ||
        (reinterpret_cast<uintptr_t>(flags) & 3u))
      return PK_ERR_POINTER;
  }
  return PK_OK;
}

template <class C>
static int occupancy_of(int dev) {
  static int occ[64];
  static std::once_flag once[64];
  if (dev < 0 || dev >= 64) return 1;
  std::call_once(once[dev], [&] {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, gemm_rs_kernel<C>, C::THREADS, 0) !=
            hipSuccess ||
        blocks < 1)
      blocks = 1;
    occ[dev] = blocks;
  });
  return occ[dev];
}

static int cu_count(int dev) {
  static int cus[64];
  static std::once_flag once[64];
  if (dev < 0 || dev >= 64) return kAssumedCUs;
  std::call_once(once[dev], [&] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = kAssumedCUs;
    cus[dev] = n;
  });
  return cus[dev];
}

template <class C>
static int launch(KArgs& a, const pk_options* o, hipStream_t stream) {
  a.g.BM = C::BM;
  a.g.BN = C::BN;
  a.g.Tm = a.S > 0 ? ceil_div(a.S, C::BM) : 0;
  a.g.Tn = ceil_div(a.N, C::BN);
  a.g.group_n = (o && o->group_n > 0) ? o->group_n : default_group_n(kCfgs[0], a.g.Tn);
  a.total_tiles = a.g.total();
  if (a.total_tiles == 0) return PK_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PK_ERR_LAUNCH;
  long long grid = (long long)cu_count(dev) * occupancy_of<C>(dev);
  if (o && o->max_workgroups > 0 && o->max_workgroups < grid) grid = o->max_workgroups;
  if (grid > a.total_tiles) grid = a.total_tiles;
  hipLaunchKernelGGL(gemm_rs_kernel<C>, dim3((unsigned)grid), dim3(C::THREADS), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_LAUNCH;
}

static int run(const void* A, const void* B, const void* peers, void* send, void* out,
               uint32_t* flags, long long M, long long N, long long K, int P, int rank,
               int chunk_rows, int tile_order, int out_bf16, const pk_options* o, void* stream) {
  const int v = validate(A, B, peers, send, out, flags, M, N, K, P, rank, chunk_rows, tile_order,
                         out_bf16, o);
  if (v != PK_OK) return v;
  if (M == 0 || N == 0) return PK_OK;
  KArgs a;
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.peers = static_cast<const uint16_t*>(peers);
  a.send = static_cast<uint16_t*>(send);
  a.out = out;
  a.flags = flags;
  a.M = M;
  a.N = N;
  a.K = K;
  a.gemm_only = (o && o->gemm_only) ? 1 : 0;
  if (a.gemm_only) {
    // One shard covering every row, nothing sent.
    a.P = 1;
    a.rank = 0;
    a.S = (int)M;
    a.chunk_rows = 1;
    a.n_chunks = 0;
    a.out_bf16 = 1;
  } else {
    a.P = P;
    a.rank = rank;
    a.S = (int)(M / P);
    a.chunk_rows = chunk_rows > 0 ? chunk_rows : 1;
    a.n_chunks = chunk_rows > 0 ? (int)(a.S / chunk_rows) : 0;
    a.out_bf16 = out_bf16;
  }
  a.g.P = a.P;
  a.g.rank = a.rank;
  a.g.S = a.S;
  a.g.N = (int)N;
  a.g.order = tile_order;
  const int cfg = (o && o->config > 0) ? o->config : select_config(M, N, K, a.P);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (cfg) {
    case 1: return launch<Cfg1>(a, o, s);
    case 2: return launch<Cfg2>(a, o, s);
    case 3: return launch<Cfg3>(a, o, s);
    default: return PK_ERR_CONFIG;
  }
}

}  // namespace pk

// ---------------------------------------------------------------------------
// C ABI.
// ---------------------------------------------------------------------------
extern "C" {

int pk_gemm_rs_local(const void* A, const void* B, const void* peer_partials, void* send_bufs,
                     void* out, uint32_t* flags, int64_t M, int64_t N, int64_t K, int P,
                     int rank, int chunk_rows, int tile_order, void* stream) {
  return pk::run(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                 tile_order, 0, nullptr, stream);
}

int pk_gemm_rs_local_bf16out(const void* A, const void* B, const void* peer_partials,
                             void* send_bufs, void* out, uint32_t* flags, int64_t M, int64_t N,
                             int64_t K, int P, int rank, int chunk_rows, int tile_order,
                             void* stream) {
  return pk::run(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                 tile_order, 1, nullptr, stream);
}

int pk_gemm_rs_local_ex(const void* A, const void* B, const void* peer_partials, void* send_bufs,
                        void* out, uint32_t* flags, int64_t M, int64_t N, int64_t K, int P,
                        int rank, int chunk_rows, int tile_order, int out_bf16,
                        const pk_options* opts, void* stream) {
  return pk::run(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                 tile_order, out_bf16, opts, stream);
}

int64_t pk_flags_words(int P, int64_t M, int chunk_rows) {
  if (P < 1 || P > 64) return PK_ERR_RANK;
  if (M < 0 || M % P != 0) return PK_ERR_SHAPE;
  const int64_t S = M / P;
  if (S == 0) return 0;
  if (chunk_rows <= 0 || S % chunk_rows != 0) return PK_ERR_SHAPE;
  return 2 * (int64_t)(P - 1) * (S / chunk_rows);
}

int pk_validate(const void* A, const void* B, const void* peer_partials, const void* send_bufs,
                const void* out, const uint32_t* flags, int64_t M, int64_t N, int64_t K, int P,
                int rank, int chunk_rows, int tile_order, int out_bf16, const pk_options* opts) {
  return pk::validate(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                      tile_order, out_bf16, opts);
}

int pk_config_count(void) { return pk::kNumCfgs; }

int pk_config_info(int id, int* BM, int* BN, int* BK, int* WM, int* WN, int* threads) {
  if (id < 1 || id > pk::kNumCfgs) return PK_ERR_CONFIG;
  const pk::CfgInfo& c = pk::kCfgs[id - 1];
  if (BM) *BM = c.BM;
  if (BN) *BN = c.BN;
  if (BK) *BK = c.BK;
  if (WM) *WM = c.WM;
  if (WN) *WN = c.WN;
  if (threads) *threads = c.threads;
  return PK_OK;
}

int pk_select_config(int64_t M, int64_t N, int64_t K, int P) {
  if (P < 1) return PK_ERR_RANK;
  return pk::select_config(M, N, K, P);
}

int64_t pk_tile_walk(int64_t M, int64_t N, int P, int rank, int config, int tile_order,
                     int group_n, int32_t* out3, int64_t cap) {
  if (P < 1 || P > 64 || rank < 0 || rank >= P) return PK_ERR_RANK;
  if (tile_order < 0 || tile_order > 2) return PK_ERR_TILE_ORDER;
  if (M < 0 || N < 0 || M % P != 0) return PK_ERR_SHAPE;
  if (config < 1 || config > pk::kNumCfgs) return PK_ERR_CONFIG;
  const pk::CfgInfo& c = pk::kCfgs[config - 1];
  pk::Grid g;
  g.P = P;
  g.rank = rank;
  g.S = (int)(M / P);
  g.N = (int)N;
  g.BM = c.BM;
  g.BN = c.BN;
  g.Tm = g.S > 0 ? pk::ceil_div(g.S, c.BM) : 0;
  g.Tn = pk::ceil_div(N, c.BN);
  g.order = tile_order;
  g.group_n = group_n > 0 ? group_n : pk::default_group_n(c, g.Tn);
  const long long total = g.total();
  for (long long s = 0; s < total && s < cap; ++s) {
    const pk::TileCoord tc = pk::tile_at(g, s);
    out3[3 * s] = tc.shard;
    out3[3 * s + 1] = tc.t;
    out3[3 * s + 2] = tc.u;
  }
  return total;
}

int64_t pk_chunk_arrivals(int64_t M, int64_t N, int P, int chunk_rows, int config, int c) {
  if (P < 1 || P > 64) return PK_ERR_RANK;
  if (M < 0 || M % P != 0 || N < 0) return PK_ERR_SHAPE;
  if (config < 1 || config > pk::kNumCfgs) return PK_ERR_CONFIG;
  const int64_t S = M / P;
  if (chunk_rows <= 0 || S % chunk_rows != 0 || c < 0 || c >= S / chunk_rows) return PK_ERR_SHAPE;
  const pk::CfgInfo& cf = pk::kCfgs[config - 1];
  return pk::expected_arrivals(c, cf.BM, chunk_rows, pk::ceil_div(N, cf.BN));
}

const char* pk_strerror(int code) {
  switch (code) {
    case PK_OK: return "ok";
    case PK_ERR_POINTER: return "null or misaligned pointer";
    case PK_ERR_SHAPE: return "unsupported shape (M % P, N % 8, K % 8, chunk_rows must divide M/P)";
    case PK_ERR_RANK: return "P must be in [1, 64] and rank in [0, P)";
    case PK_ERR_TILE_ORDER: return "tile_order must be 0 (row-major), 1 (owned-first) or 2 (dest-round-robin)";
    case PK_ERR_CONFIG: return "unknown tile configuration or option";
    case PK_ERR_LAUNCH: return "HIP launch failed";
    case PK_ERR_TOO_LARGE: return "dimension exceeds 2^31";
    default: return "unknown error";
  }
}

int pk_version(void) { return 100; }

}  // extern "C"
