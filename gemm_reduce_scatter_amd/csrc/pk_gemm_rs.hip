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
//  * operand tiles move global -> LDS by buffer loads that write LDS
//    directly (no register staging); lanes outside the matrix read zero
//    through the buffer range check, which also covers ragged tiles and a
//    partial last K step;
//  * the main loop is bf16 MFMA (v_mfma_f32_32x32x16_bf16) on 64-wide
//    wavefronts.  A is read from LDS with 16-byte reads; B stays n-major in
//    LDS as it is in memory and is read with the CDNA4 transposing LDS read
//    (ds_read_b64_tr_b16), which hands each lane the k-run of one column;
//  * one persistent workgroup per CU slot walks the tile order; consecutive
//    walk positions go to the same XCD so tiles that share A/B panels share
//    that XCD's L2.
// The same kernel template runs the library's other entry points through its
// Mode: a plain GEMM (the standalone reference), the pages' atomic push
// epilogue, and the all-gather + GEMM whose tiles wait for their A chunks;
// the inter-CU schedule is the fused mode with communicator workgroups at
// the front of the grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "pk_chunk_move.h"
#include "pk_gemm_rs.h"
#include "pk_plan.h"

namespace pk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define PK_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// Tile configurations.  Four waves (256 threads) per workgroup in a
// WAVES_M x WAVES_N arrangement; each wave owns a WM x WN block of 32x32
// MFMA accumulators.  STAGES-deep ring of LDS operand buffers of BK k each.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int STAGES_, int OCC_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int OCC = OCC_;   // workgroups meant to share a CU
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;   // 32x32 MFMA blocks per wave
  static constexpr int KK = BK / 16;                 // k16 MFMA steps per stage
  // LDS operand layout, per stage:
  //   A: BM rows of BK k (A_CPR chunks of 16 bytes), chunk c of row r stored
  //      at chunk c ^ swz_a(r);
  //   B: BK k-rows of BN n (B_CPR chunks), chunk c of k-row k stored at
  //      chunk c ^ swz_b(k).
  static constexpr int A_CPR = BK / 8;
  static constexpr int A_RPL = 64 / A_CPR;            // A rows per 64-lane load
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int B_CPR = BN / 8;                // 16-byte chunks per B row
  static constexpr int B_RPL = 64 / B_CPR;            // B rows per 64-lane load
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;   // 1 KiB per wave load
  static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
  static constexpr int LOADS = A_LOADS + B_LOADS;          // per wave per stage
  static constexpr int EPI_STRIDE = WN + 8;                // floats per staged row
  static constexpr int LDS_EPI = WAVES * 16 * EPI_STRIDE * 4;  // 16-row half stripes
  // Stage buffers are separate LDS arrays (the compiler then knows that reads
  // of one stage never alias the DMA into another); the epilogue staging
  // area reuses stage 0.
  static constexpr int LDS0 = STAGE_BYTES > LDS_EPI ? STAGE_BYTES : LDS_EPI;
  static constexpr int LDS = LDS0 + (STAGES - 1) * STAGE_BYTES;
  static_assert(WAVES == 4, "four waves per workgroup");
  static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
  static_assert(STAGES >= 2 && STAGES <= 4, "2..4 stages");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
  static_assert(A_LOADS >= 1 && A_BYTES % (1024 * WAVES) == 0, "A stage splits over the waves");
  static_assert(B_LOADS >= 1 && B_BYTES % (1024 * WAVES) == 0, "B stage splits over the waves");
  static_assert(B_CPR >= 8 && B_CPR <= 64, "B row is 8..64 chunks");
  static_assert(LDS * OCC <= 160 * 1024, "fits the 160 KiB LDS of a CU");
};

// id 1..6; the table in pk_config_info mirrors these.
using Cfg1 = Cfg<256, 256, 2, 2, 32, 4>;
using Cfg2 = Cfg<128, 128, 2, 2, 64, 2>;
using Cfg3 = Cfg<64, 64, 2, 2, 64, 2>;
using Cfg4 = Cfg<256, 128, 2, 2, 32, 4>;
using Cfg5 = Cfg<256, 256, 2, 2, 64, 2>;
// Two workgroups per CU: 72 KiB of LDS and at most 256 registers per lane
// each (128 accumulators), so one workgroup's stores and latency-bound steps
// overlap the other's MFMAs.
using Cfg6 = Cfg<256, 128, 2, 2, 32, 3, 2>;
// Owned sub-tiles when the owned shard is split: 64 x 128, eight per Cfg1
// tile, four per Cfg6 tile (with that configuration's LDS budget).
using CfgOwned = Cfg<64, 128, 2, 2, 64, 4>;
using CfgOwned3 = Cfg<64, 128, 2, 2, 64, 3, 2>;
template <class C>
struct OwnedOf {
  using type = CfgOwned;
};
template <>
struct OwnedOf<Cfg6> {
  using type = CfgOwned3;
};

struct KArgs {
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* peers;
  uint16_t* send;
  void* out;
  uint32_t* flags;
  long long M;
  int N, K;            // N <= 2^24, K <= 2^22 (validated)
  int P, rank, S, chunk_rows, n_chunks;
  int out_bf16;
  int store_nt;        // output stores carry the non-temporal hint (store16)
  int sig_batch;       // send tiles per ready-word release (>= 1)
  uint64_t* ready_clock;   // null, or [P-1][n_chunks]: device clock when a ready word rose
  // all-gather + GEMM: ready words [P][n_chunks] of the gathered A rows, the
  // value that means "arrived", polls per word before giving up, and the
  // word set to 1 when a wait gave up
  const uint32_t* wait_ready;
  uint32_t wait_expected;
  int spin_limit;
  int32_t* wait_error;
  // communicator workgroups (inter-CU schedule): the first n_comm of the
  // grid move finished send chunks instead of computing tiles
  int n_comm;
  pkm::MoveArgs mv;
  // reduction role of the communicators: the fp32 peer sum of the owned
  // shard [S][N], its counting words per 64 x 64 piece ([ceil(S/64)][piece_cols]),
  // and null or the ready words [P-1][n_chunks] of the incoming peer chunks
  // (those wait for wait_expected)
  float* presum;
  uint32_t* piece_ready;
  int piece_cols;
  uint32_t piece_expected;   // the value a piece word reaches in this call
  const uint32_t* peer_ready;
  Grid g;
  long long total_tiles;
  uint64_t* timeline;   // null, or the phase record of an instrumented build
};

// Instrumented timing build (compiled with -DPK_TIMELINE, a library of its
// own; the product library has no trace of it): thread 0 of every workgroup
// writes into timeline[blockIdx][kTlSlots] its hardware placement (slot 0:
// XCC id << 32 | the HW_ID register: CU, SE, SIMD), the 100 MHz wall clock at
// its start (slot 1) and, in later slots, (kind << 56) | clock at each phase
// boundary: 1 first stage landed, 2 main loop done, 3 epilogue done, 4 ready
// words raised.  Nothing else changes: the results are bitwise the product
// library's.
constexpr int kTlSlots = 32;
constexpr long long kTimelineWorkgroups = 2048;   // the record holds this many workgroups
#ifdef PK_TIMELINE
__device__ __forceinline__ int& tl_slot() {
  __shared__ int n;
  return n;
}
__device__ __forceinline__ void tl_start(const KArgs& a) {
  if (a.timeline && threadIdx.x == 0) {
    tl_slot() = 2;
    const uint64_t hw = (uint64_t)__builtin_amdgcn_s_getreg((31 << 11) | 4) |
                        ((uint64_t)__builtin_amdgcn_s_getreg((3 << 11) | 20) << 32);
    a.timeline[(long long)blockIdx.x * kTlSlots] = hw;
    a.timeline[(long long)blockIdx.x * kTlSlots + 1] = wall_clock64();
  }
}
__device__ __forceinline__ void tl_mark(const KArgs& a, uint64_t kind) {
  if (a.timeline && threadIdx.x == 0) {
    int& n = tl_slot();
    if (n < kTlSlots) a.timeline[(long long)blockIdx.x * kTlSlots + n] = (kind << 56) | wall_clock64();
    ++n;
  }
}
#define PK_TL_START(a) tl_start(a)
#define PK_MARK(a, kind) tl_mark(a, kind)
#else
#define PK_TL_START(a) ((void)0)
#define PK_MARK(a, kind) ((void)0)
#endif

// LDS swizzles.  A: the 16 rows a 16-lane group reads at one logical chunk
// land in 16 distinct 16-byte bank groups, and so do the 8 rows of each
// 8-lane quarter; the swizzle depends on r % 16 only, so it is the same for
// every 32-row fragment and every load of a lane.  B: the four k-rows a
// transposing read touches (k % 4 = 0..3) land in distinct bank groups for
// both the 16- and the 32-lane halves of the read.
template <int BK>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (BK == 64) return (r ^ ((r >> 3) & 1)) & 7;   // 128-byte rows
  else return ((r >> 1) ^ (r >> 3)) & 3;                     // 64-byte rows
}
template <int CPR>
__device__ __forceinline__ int swz_b(int k) {
  const int j = k & 3;
  return (((j & 1) << 2) + (j >> 1) * 10) & (CPR - 1);
}

// Buffer descriptor over `bytes` bytes from `base` (at most 2^31).  A load
// whose vector + scalar offset reaches `bytes` reads zero without touching
// memory; lanes outside the matrix get a vector offset of 2^31 for that.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes = 0x80000000u) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr uint32_t kOffNone = 0x80000000u;

// 16 bytes per lane from r + voff + soff into LDS at dst + 16 * lane.  soff is
// wave-uniform; voff of a lane outside the matrix is kOffNone.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, PK_LDS void* dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (int)voff, (int)soff, 0, 0);
}

// Staged peer partials are read exactly once: non-temporal loads (nt), so
// they stream past the caches instead of evicting the A and B panels that
// the main loops of the other workgroups reuse.
constexpr int kAuxStream = 2;   // cache-policy bits of a buffer load: nt

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 16-byte store of output data (send chunks, the owned shard, GEMM-only C,
// the reduction workspace), written through the L2 to memory (sc0 sc1), so a
// device-scope release has few dirty lines to write back.  `nt` marks it as
// streaming data as well: that keeps gigabytes of send chunks from evicting
// the A and B panels other workgroups reuse, but costs time when the call's
// streams are small enough to stay in the last-level cache (a runtime choice
// per call, KArgs::store_nt).  The compiler does not see the store, so the
// wait states a following write of its data registers needs are issued here.
__device__ __forceinline__ void store16(void* p, u32x4 v, bool nt) {
  if (nt)
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\ts_nop 1" ::"v"(p), "v"(v)
                 : "memory");
  else
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 1" ::"v"(p), "v"(v)
                 : "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt with vmcnt = N (0..63) and the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wave-local ordering of LDS writes before LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Operand staging: one stage (BK k) of the A row panel and the B column
// panel of a tile, global -> LDS.
// ---------------------------------------------------------------------------
template <class C>
struct Loader {
  // per-lane constants
  uint32_t a_off;      // byte offset of this lane's A chunk for load 0 at k0 = 0
  int a_row;           // row of load 0 relative to the tile
  int a_kc;            // k offset (elements) of this lane's A chunk
  uint32_t b_off;      // byte offset of this lane's B chunk for load 0 at k0 = 0
  int b_k;             // k-row of load 0
  int b_nc;            // n offset (elements) of this lane's B chunk
  // per item: the vector offsets above, or kOffNone for rows past the shard
  // (A load q) and columns past N (B)
  uint32_t a_vo[C::A_LOADS];
  uint32_t b_vo;

  __device__ __forceinline__ void init(const KArgs& a, int wave, int lane) {
    // A: load q of wave w covers LDS rows (q*WAVES + w)*A_RPL .. +A_RPL-1;
    // lane i fills row +i/A_CPR, physical chunk i%A_CPR, which holds logical
    // chunk (i%A_CPR)^swz_a.  swz_a depends on the row mod 16, the same for
    // every q.
    a_row = wave * C::A_RPL + lane / C::A_CPR;
    a_kc = 8 * ((lane % C::A_CPR) ^ swz_a<C::BK>(a_row));
    a_off = (uint32_t)(a_row * a.K + a_kc) * 2u;
    // B: load q of wave w covers k-rows (q*WAVES + w)*B_RPL .. +B_RPL-1.
    b_k = wave * C::B_RPL + lane / C::B_CPR;
    b_nc = 8 * ((lane % C::B_CPR) ^ swz_b<C::B_CPR>(b_k));
    b_off = (uint32_t)(b_k * a.N + b_nc) * 2u;
  }

  __device__ __forceinline__ void bind(const KArgs& a, int rows_valid, int col0) {
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q)
      a_vo[q] = a_row + q * C::WAVES * C::A_RPL < rows_valid ? a_off : kOffNone;
    b_vo = col0 + b_nc < a.N ? b_off : kOffNone;
  }

  // Gathered rows: the A row of load q is tile row a_row + q*WAVES*A_RPL of
  // row group g, at its own row of A (gather_row); the stage descriptor then
  // starts at row 0 and the loads take no row step.  A load covers one block
  // of 16 tile rows, which are 16 consecutive rows of A, so the block's first
  // row is worked out once per wave (scalar) and each lane adds its offset.
  __device__ __forceinline__ void bind_gather(const KArgs& a, int g, int col0, int wave, int lane) {
    static_assert(C::A_RPL == 16, "a load covers one 16-row block");
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q) {
      const long long r0 = gather_row(a.rank, a.S, g, (q * C::WAVES + wave) * C::A_RPL);
      a_vo[q] = (uint32_t)((r0 + lane / C::A_CPR) * a.K + a_kc) * 2u;
    }
    b_vo = col0 + b_nc < a.N ? b_off : kOffNone;
  }

  // Per-stage descriptors: A rows from row0, B columns from col0, both at k0.
  struct Stage {
    __amdgpu_buffer_rsrc_t ra, rb;
    int k0;
  };
  __device__ __forceinline__ Stage stage(const KArgs& a, long long row0, int col0,
                                         int k0) const {
    Stage st;
    st.ra = make_rsrc(a.A + row0 * a.K + k0);
    // B's rows k0 .. K-1 only: the rows past K of a stage (all of them past
    // the end of K) fall outside the range and read zero.
    const long long rem = (long long)(a.K - k0) * a.N * 2;
    st.rb = make_rsrc(a.B + (long long)k0 * a.N + col0,
                      rem <= 0 ? 0u : rem >= 0x80000000LL ? 0x80000000u : (uint32_t)rem);
    st.k0 = k0;
    return st;
  }

  // Issue loads [Q0, Q1) of this wave's A loads followed by its B loads
  // (numbered 0 .. LOADS-1) of one stage into `dst`.  The per-load step is a
  // scalar offset.  Lanes outside the matrix load zeros: rows past the shard
  // and columns past N through their vector offsets (bind), B's k-rows past
  // K through the stage descriptor's range, and A's k-columns past K
  // (which the range of a row-strided A cannot cut off) through one compare
  // per call, shared by all A loads of the lane.
  template <int Q0, int Q1, bool GA = false>
  __device__ __forceinline__ void issue(const KArgs& a, const Stage& st,
                                        unsigned char* dst, int wave) const {
    const bool a_k_ok = st.k0 + a_kc < a.K;
#pragma unroll
    for (int q = Q0; q < Q1; ++q) {
      if (q < C::A_LOADS) {
        const uint32_t soff = GA ? 0u : (uint32_t)(q * C::WAVES * C::A_RPL) * (uint32_t)a.K * 2u;
        dma16(st.ra, (PK_LDS void*)(dst + (q * C::WAVES + wave) * 1024),
              a_k_ok ? a_vo[q] : kOffNone, soff);
      } else {
        const int qb = q - C::A_LOADS;
        const uint32_t soff = (uint32_t)(qb * C::WAVES * C::B_RPL) * (uint32_t)a.N * 2u;
        dma16(st.rb, (PK_LDS void*)(dst + C::A_BYTES + (qb * C::WAVES + wave) * 1024), b_vo,
              soff);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one LDS stage.
// ---------------------------------------------------------------------------
template <class C>
struct Reader {
  uint32_t a_base;            // this lane's A row (fragment 0) byte offset in a stage
  uint32_t a_x[C::KK];        // swizzled chunk byte offset for k16 step kk
  uint32_t b_base[C::FN];     // this lane's B address part for fragment fn (row + chunk)

  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    const int r = wm * C::WM + (lane & 31);
    a_base = (uint32_t)r * (uint32_t)(C::BK * 2);
    const int sa = swz_a<C::BK>(r);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) a_x[kk] = (uint32_t)(((2 * kk + (lane >> 5)) ^ sa) << 4);
    // Transposing B read: 16-lane group g reads k-rows kbase + 0..3 (one per
    // lane quad j) at columns nbase + 4i .. +3 (lane i of the quad); after
    // the transpose lane t of the group holds rows kbase + 0..3 of column
    // nbase + t.  MFMA 32x32x16 wants lane L to hold k = 8*(L/32) + 0..7 of
    // column L%32: group g gets nbase = 16*(g&1), kbase = 8*(g>>1), and a
    // second read at kbase + 4 gives k + 4..7.
    const int g = lane >> 4, t = lane & 15, i = t & 3, j = t >> 2;
    const int krow = 8 * (g >> 1) + j;
    const int sb = swz_b<C::B_CPR>(krow);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int n = wn * C::WN + fn * 32 + 16 * (g & 1) + 4 * i;
      b_base[fn] = (uint32_t)C::A_BYTES + (uint32_t)krow * (uint32_t)(C::BN * 2) +
                   (uint32_t)((((n >> 3) ^ sb) << 4) + ((n & 4) << 1));
    }
  }

  struct Frags {
    bf16x8 a[C::FM], b[C::FN];
  };

  __device__ __forceinline__ void read(const unsigned char* st, int kk, Frags& f) const {
    // In the order the MFMAs (fm outer, fn inner) first use them: A0, all of
    // B, then A1 .. A(FM-1), so the reads issued last are needed last.
    f.a[0] = *reinterpret_cast<const bf16x8*>(st + a_base + a_x[kk]);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const unsigned char* p = st + b_base[fn] + kk * 16 * (C::BN * 2);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PK_LDS s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PK_LDS s16x4*)(p + 4 * C::BN * 2));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      f.b[fn] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
    }
#pragma unroll
    for (int fm = 1; fm < C::FM; ++fm)
      f.a[fm] = *reinterpret_cast<const bf16x8*>(st + a_base + fm * 32 * (C::BK * 2) + a_x[kk]);
  }

  __device__ __forceinline__ static void mfma(const Frags& f, f32x16 (&acc)[C::FM][C::FN]) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[fm], f.b[fn], acc[fm][fn], 0, 0, 0);
  }
};

// Issue order of one k16 step, for the compiler's scheduler: MFMA i is
// followed by fragment read i of the next step (while there are any) and
// load i of the stage ahead (while there are any).  A wave issues in order
// and a 32x32x16 MFMA holds the issue port for many cycles, so reads and
// loads placed after the whole MFMA group would start late.
template <int I, int N, int NR, int NV>
__device__ __forceinline__ void step_pattern() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // MFMA
    if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    // global loads evenly spaced: after MFMAs 0, N/NV, 2N/NV, ...
    if constexpr (NV > 0 && (I * NV) % N < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    step_pattern<I + 1, N, NR, NV>();
  }
}

// One stage of the main loop: MFMA over `cur` in KK k16 steps while a share
// of the loads of the stage STAGES-1 ahead (into `nxt`) is issued during each
// step, spaced out among its MFMAs so that the four waves never queue many
// loads at once.  Fragments run one step ahead: step kk multiplies the fragments read
// during step kk-1.  The last step first waits for this wave's loads of the
// next stage, meets the other waves at the barrier (after which every wave
// has finished reading `cur` and the next stage is complete), reads the
// next stage's first fragments from `nbuf` and only then multiplies, so the
// LDS latency at the stage boundary hides behind that step's MFMAs and the
// barrier behind the previous step's.  A stage past K loads zeros (every
// lane fails the k bound), so the loop body has no branches, the number of
// loads in flight is fixed, and the accumulators stay in place across
// iterations.  `bg` gets one hook per step (step STG*KK + kk of the trip) to
// issue background loads; it issues BG::LOADS_PER_STEP of them.
template <class C, int STG, int KKI, class BG, bool GA = false>
__device__ __forceinline__ void stage_steps(const KArgs& a, const Loader<C>& ld,
                                            const typename Loader<C>::Stage& ns,
                                            const Reader<C>& rd, const unsigned char* cur,
                                            unsigned char* nxt, const unsigned char* nbuf,
                                            int wave, f32x16 (&acc)[C::FM][C::FN],
                                            typename Reader<C>::Frags (&f)[2], BG& bg) {
  if constexpr (KKI < C::KK) {
    constexpr int QP = (C::LOADS + C::KK - 1) / C::KK;   // loads issued per k16 step
    constexpr int Q0 = KKI * QP < C::LOADS ? KKI * QP : C::LOADS;
    constexpr int Q1 = (KKI + 1) * QP < C::LOADS ? (KKI + 1) * QP : C::LOADS;
    // With three or more stages the last step's loads wait until after the
    // barrier, so every step spreads its loads over its MFMAs.
    constexpr bool LATE = KKI + 1 == C::KK && C::STAGES >= 3;
    if constexpr (!LATE) ld.template issue<Q0, Q1, GA>(a, ns, nxt, wave);
    bg.template step<STG * C::KK + KKI>(a);
    if constexpr (KKI + 1 < C::KK) {
      rd.read(cur, KKI + 1, f[(KKI + 1) & 1]);
    } else {
      // Every read of `cur` has returned (its fragments feed the MFMAs of
      // this and the previous step), so the barrier also ends all use of it.
      // Loads complete in issue order; younger than the next stage's are
      // the stages after it issued so far (all but this step's share of the
      // newest one when it comes late) and the background loads issued
      // since its last share: those of the last STAGES - 2 stages, which may
      // stay in flight.
      wait_vm<(C::STAGES - 2) * C::LOADS - (LATE ? Q1 - Q0 : 0) +
              (C::STAGES - 2) * C::KK * BG::LOADS_PER_STEP>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // `nxt` was last read in the stage before this one, before the
      // previous barrier.
      if constexpr (LATE) ld.template issue<Q0, Q1, GA>(a, ns, nxt, wave);
      rd.read(nbuf, 0, f[(KKI + 1) & 1]);
    }
    Reader<C>::mfma(f[KKI & 1], acc);
    step_pattern<0, C::FM * C::FN, C::FM + 2 * C::FN, (KKI + 1 < C::KK || LATE) ? Q1 - Q0 : 0>();
    __builtin_amdgcn_sched_barrier(0);
    stage_steps<C, STG, KKI + 1, BG, GA>(a, ld, ns, rd, cur, nxt, nbuf, wave, acc, f, bg);
  }
}

template <class C, int STG, class BG, bool GA = false>
__device__ __forceinline__ void main_stage(const KArgs& a, const Loader<C>& ld,
                                           const typename Loader<C>::Stage& ns,
                                           const Reader<C>& rd, const unsigned char* cur,
                                           unsigned char* nxt, const unsigned char* nbuf,
                                           int wave, f32x16 (&acc)[C::FM][C::FN],
                                           typename Reader<C>::Frags (&f)[2], BG& bg) {
  static_assert(C::KK % 2 == 0, "the next stage's first fragments land in f[0]");
  stage_steps<C, STG, 0, BG, GA>(a, ld, ns, rd, cur, nxt, nbuf, wave, acc, f, bg);
}

// No background work.
struct NoBackground {
  static constexpr int LOADS_PER_STEP = 0;
  template <int I>
  __device__ __forceinline__ void step(const KArgs&) {}
  __device__ __forceinline__ void end_trip() {}
  __device__ __forceinline__ void finish(const KArgs&) {}
};

// Stage buffer I of the ring (compile-time, so every LDS access names one
// array).
template <int I>
__device__ __forceinline__ unsigned char* pick(unsigned char* b0, unsigned char* b1,
                                               unsigned char* b2, unsigned char* b3) {
  if constexpr (I == 0) return b0;
  else if constexpr (I == 1) return b1;
  else if constexpr (I == 2) return b2;
  else return b3;
}

// Ready-word protocol (the pages' signal primitive, per chunk).  A caller
// has made the stores of one or more finished send tiles visible at device
// scope with a release fence; for each tile it then adds one arrival to
// every chunk the tile touches (signal_chunk, one per pair).  Each arrival is relaxed: the data it vouches
// for was released before it.  The arrival that completes a chunk acquires
// (so the other workgroups' released stores happen before what follows),
// adds one to the ready word with release (the pages' signal adds to a
// counter and their wait waits for it to reach a value: call n of a flags
// buffer raises its ready words to n, and nothing has to clear them between
// calls) and resets the counter for the next launch.
// Each chunk's arrival counter has a 128-byte line of its own (counter idx
// at word kCounterStride * idx of the counter area): the arrivals of one
// launch at different chunks then do not queue behind each other at one line
// (measured 2-3 us of the comm-dominant share with all counters in one line).
constexpr int kCounterStride = 32;
__device__ __forceinline__ uint32_t* chunk_counter(const KArgs& a, int idx) {
  return a.flags + (long long)(a.P - 1) * a.n_chunks + (long long)kCounterStride * idx;
}
// One arrival at chunk idx; returns the count before it.
__device__ __forceinline__ uint32_t arrive_chunk(const KArgs& a, int idx) {
  return __hip_atomic_fetch_add(chunk_counter(a, idx), 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
// The arrival that completed chunk idx: acquire, raise the ready word, reset
// the counter.
__device__ __forceinline__ void complete_chunk(const KArgs& a, int idx) {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __hip_atomic_fetch_add(&a.flags[idx], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(chunk_counter(a, idx), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a.ready_clock) a.ready_clock[idx] = wall_clock64();
}
__device__ __forceinline__ void signal_chunk(const KArgs& a, int idx, uint32_t want) {
  if (arrive_chunk(a, idx) + 1u == want) complete_chunk(a, idx);
}

// Arrivals of a batch of finished send tiles, spread over the lanes of one
// wave: the batch's (tile, chunk) pairs are numbered in walk order and lane
// l takes pairs l, l+64, ..., so the arrivals of up to 64 pairs travel in
// one vector atomic instead of one after another.  `tile_of(k2, tc)` gives
// the send tile of round k2 (false for an owned item).
template <class TileOf>
__device__ __forceinline__ void signal_batch(const KArgs& a, long long fk, long long k, int BM,
                                             int lane, const TileOf& tile_of) {
  for (int base = 0;; base += 64) {
    int n = 0, idx = -1;
    uint32_t want = 0;
    for (long long k2 = fk; k2 <= k; ++k2) {
      TileCoord tc;
      if (!tile_of(k2, tc)) continue;
      int c0, c1;
      chunks_of_row_tile(tc.t, BM, a.S, a.chunk_rows, c0, c1);
      const int slot = slot_of(tc.shard, a.rank);
      for (int c = c0; c <= c1; ++c, ++n) {
        if (n == base + lane) {
          idx = slot * a.n_chunks + c;
          want = expected_arrivals(c, BM, a.chunk_rows, a.g.Tn);
        }
      }
    }
    if (idx >= 0) signal_chunk(a, idx, want);
    if (n <= base + 64) break;
  }
}

// kFused: staged reduce-scatter (send chunks + owner-side sum of the staged
// peer partials); kGemmOnly: plain GEMM; kPush: every tile added with fp32
// atomics into the accumulator of the rank that owns its rows; kAgGemm:
// all-gather + GEMM, a tile of another rank's rows first waits for the
// ready words of the A chunks it reads.
// kFusedReduce: kFused whose owned items add their local partial to the peer
// sum that the communicator workgroups wrote into presum.
enum Mode : int { kFused = 0, kGemmOnly = 1, kPush = 2, kAgGemm = 3, kFusedReduce = 4 };
constexpr bool staged_mode(int m) { return m == kFused || m == kFusedReduce; }

// ---------------------------------------------------------------------------
// Epilogue of one work item.  Each wave re-lays its accumulators, one 16-row
// half of a 32-row stripe at a time, through LDS so that every lane owns 8
// consecutive columns of one row (16-byte global accesses), then sends, sums
// or stores.  `lrow0` is the shard-local row and `col0` the column of the
// item's first element.
//
// Lane segments: for stripe fm, half h and pass it, a lane owns row
// lrow0 + wm*WM + 32 fm + 16 h + it*RPI + lane/LPR, columns
// col0 + wn*WN + 8 (lane%LPR) .. +7.
// ---------------------------------------------------------------------------
template <class C>
struct Seg {
  static constexpr int LPR = C::WN / 8;        // lanes per staged row
  static constexpr int RPI = 64 / LPR;         // rows per pass
  static constexpr int PASSES = 16 / RPI;
  static constexpr int COUNT = C::FM * 2 * PASSES;   // segments per lane
  __device__ __forceinline__ static int row(int wm, int lane, int fm, int h, int it) {
    return wm * C::WM + fm * 32 + 16 * h + it * RPI + lane / LPR;
  }
  __device__ __forceinline__ static int col(int wn, int lane) {
    return wn * C::WN + (lane % LPR) * 8;
  }
};

// The owned shard's value is (sum_j peer_j) + C: the staged peer partials
// added in ascending slot order starting from 0, then the local partial.
// The sum comes from one of three sources, all with that order:
//  kPeersDirect   - loaded in the epilogue, GS slots at a time;
//  kPeersPrefetch - every slot of every segment read into registers before
//                   the item's main loop (GS = P-1);
//  kPeersPresum   - summed in the background while the workgroup multiplied
//                   a send tile just before this item (PresumStream);
//  kPeersReduced  - summed by the communicator workgroups into presum (fp32),
//                   read once its pieces' words have risen (reduce_units).
// kSendOnly marks a send tile under the owned split, which is never owned
// (the owned shard is cut into sub-tiles of their own): its epilogue has no
// owned branch.
enum PeerSource : int {
  kPeersDirect = 0,
  kPeersPrefetch = 1,
  kPeersPresum = 2,
  kPeersReduced = 3,
  kSendOnly = 4
};

__device__ __forceinline__ void add_bf16x8(float (&t)[8], u32x4 v) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    t[2 * p] += bf16lo(v[p]);
    t[2 * p + 1] += bf16hi(v[p]);
  }
}

// As add_bf16x8 when `ok`, else adds +0 (the sums start at +0 and never
// hold -0, so this leaves them unchanged).
__device__ __forceinline__ void add_bf16x8_if(float (&t)[8], u32x4 v, bool ok) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    t[2 * p] += ok ? bf16lo(v[p]) : 0.0f;
    t[2 * p + 1] += ok ? bf16hi(v[p]) : 0.0f;
  }
}

// Peer partials of every segment of an owned item, read into registers
// before the main loop so the loads overlap it (GS = P-1 slots).
template <class C, int GS>
struct PeerPrefetch {
  u32x4 v[Seg<C>::COUNT][GS];
  __device__ __forceinline__ void load(const KArgs& a, int lrow0, int col0, int wm, int wn,
                                       int lane) {
    const long long slot_stride = (long long)a.S * a.N;
    const int col = col0 + Seg<C>::col(wn, lane);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int it = 0; it < Seg<C>::PASSES; ++it) {
          const int lr = lrow0 + Seg<C>::row(wm, lane, fm, h, it);
          const bool ok = lr < a.S && col < a.N;
          const long long base = ok ? (long long)lr * a.N + col : 0;   // row 0 stays in bounds
          const int sg = (fm * 2 + h) * Seg<C>::PASSES + it;
#pragma unroll
          for (int jj = 0; jj < GS; ++jj) v[sg][jj] = load16(a.peers + jj * slot_stride + base);
        }
  }
};

// The peer sums of SEGS segments of 8 owned elements per lane (GS = P-1
// slots), accumulated by a workgroup while it multiplies a tile whose main
// loop has STEPS k16 steps per trip.  Load g (g = trip*STEPS + step) reads
// slot g/SEGS of segment g%SEGS; each segment keeps two loads in flight and
// adds one when it issues the load two slots later, 2*SEGS steps after it
// was issued, so a load has that many steps of MFMA to land in.  The loads go
// through a buffer descriptor over the peer partials: slots past P-2 get an
// offset past its range and read zeros, which add nothing (the sums start at
// +0 and never hold -0).  finish() adds the last loads and any slots a short
// K left unread.  Byte offsets are 32-bit: the owned split requires the peer
// partials to span less than 2^31 bytes.
template <int SEGS_, int GS, int STEPS>
struct PeerStream {
  static constexpr int SEGS = SEGS_;
  static constexpr int SPT = STEPS / SEGS;              // slots per trip
  static constexpr int LOADS_PER_STEP = 1;
  static_assert(STEPS % SEGS == 0, "whole segments per trip");
  float v[SEGS][8];
  u32x4 q[2][SEGS];   // slot n of a segment lands in q[n & 1]: two loads in flight
  uint32_t off[SEGS];          // byte offset of each segment in slot 0
  uint32_t slot_bytes;
  __amdgpu_buffer_rsrc_t rsrc;
  int trip;

  // Segment sg at shard-local row lr, column col (outside the shard: row 0,
  // whose sums are never stored).
  __device__ __forceinline__ void set(const KArgs& a, int sg, int lr, int col) {
    const bool ok = lr < a.S && col < a.N;
    off[sg] = ok ? ((uint32_t)lr * (uint32_t)a.N + (uint32_t)col) * 2u : 0u;
  }
  __device__ __forceinline__ void start(const KArgs& a) {
    rsrc = make_rsrc(a.peers);
    slot_bytes = (uint32_t)a.S * (uint32_t)a.N * 2u;
#pragma unroll
    for (int sg = 0; sg < SEGS; ++sg) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[sg][e] = 0.0f;
      q[0][sg] = u32x4{0u, 0u, 0u, 0u};
      q[1][sg] = u32x4{0u, 0u, 0u, 0u};
    }
    trip = 0;
  }

  __device__ __forceinline__ u32x4 load(uint32_t off_b, int slot) const {
    const uint32_t o = slot < GS ? off_b + (uint32_t)slot * slot_bytes : kOffNone;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, o, 0, kAuxStream));
  }

  template <int I>
  __device__ __forceinline__ void step(const KArgs&) {
    constexpr int sg = I % SEGS, so = I / SEGS;
    static_assert(SPT % 2 == 0, "a step's slot parity is the same every trip");
    add_bf16x8(v[sg], q[so & 1][sg]);                    // slot n-2, or zeros
    q[so & 1][sg] = load(off[sg], trip * SPT + so);
  }
  __device__ __forceinline__ void end_trip() { ++trip; }
  __device__ __forceinline__ void finish(const KArgs&) {
#pragma unroll
    for (int sg = 0; sg < SEGS; ++sg) {
      add_bf16x8(v[sg], q[0][sg]);
      add_bf16x8(v[sg], q[1][sg]);
    }
    for (int slot = trip * SPT; slot < GS; ++slot)
#pragma unroll
      for (int sg = 0; sg < SEGS; ++sg) add_bf16x8(v[sg], load(off[sg], slot));
  }
};

// The segments of an owned sub-tile of configuration CO, in its epilogue's
// order (Seg<CO>).
template <class CO, int GS, int STEPS>
struct PresumStream : PeerStream<Seg<CO>::COUNT, GS, STEPS> {
  using SG = Seg<CO>;
  __device__ __forceinline__ void init(const KArgs& a, int lrow0, int col0, int wm, int wn,
                                       int lane) {
    this->start(a);
    const int col = col0 + SG::col(wn, lane);
#pragma unroll
    for (int fm = 0; fm < CO::FM; ++fm)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int it = 0; it < SG::PASSES; ++it)
          this->set(a, (fm * 2 + h) * SG::PASSES + it, lrow0 + SG::row(wm, lane, fm, h, it), col);
  }
};

// The owned half stripe of a gathered-row tile of configuration C (16 owned
// rows x WN columns per wave, from shard-local row olr), in the order of
// gather_epilogue: pass it covers rows olr + it*RPI + lane/LPR.
template <class C, int GS, int STEPS>
struct GatherStream : PeerStream<Seg<C>::PASSES, GS, STEPS> {
  using SG = Seg<C>;
  __device__ __forceinline__ void init(const KArgs& a, int olr, int col0, int wn, int lane) {
    this->start(a);
    const int col = col0 + SG::col(wn, lane);
#pragma unroll
    for (int it = 0; it < SG::PASSES; ++it)
      this->set(a, it, olr + it * SG::RPI + lane / SG::LPR, col);
  }
};

struct NoPeers {};

__device__ __forceinline__ void store_out(const KArgs& a, long long base, const float (&s)[8]) {
  if (a.out_bf16) {
    const u32x4 o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]),
                     pack_bf16x2(s[6], s[7])};
    store16(reinterpret_cast<uint16_t*>(a.out) + base, o, a.store_nt);
  } else {
    float* dst = reinterpret_cast<float*>(a.out) + base;
    store16(dst, u32x4{__float_as_uint(s[0]), __float_as_uint(s[1]), __float_as_uint(s[2]),
                       __float_as_uint(s[3])}, a.store_nt);
    store16(dst + 4, u32x4{__float_as_uint(s[4]), __float_as_uint(s[5]), __float_as_uint(s[6]),
                           __float_as_uint(s[7])}, a.store_nt);
  }
}

template <class C, int MODE, int GS, int SRC, class PV>
__device__ __forceinline__ void epilogue(const KArgs& a, int shard, int lrow0, int col0,
                                         float* lds_f, int wave, int wm, int wn, int lane,
                                         f32x16 (&acc)[C::FM][C::FN], const PV& pv) {
  using SG = Seg<C>;
  float* stage = lds_f + wave * 16 * C::EPI_STRIDE;
  constexpr int LPR = SG::LPR, RPI = SG::RPI, PASSES = SG::PASSES;
  // owned segments summed together: 4 for small wave tiles, 2 when the
  // accumulators take a large part of the register file, 1 when two
  // workgroups share the CU's registers
  constexpr int BATCH = SRC != kPeersDirect ? PASSES
                        : C::OCC > 1        ? 1
                        : (C::FM * C::FN >= 4 ? 2 : (PASSES < 4 ? PASSES : 4));
  static_assert(PASSES % BATCH == 0, "batches tile the passes");
  const bool owned = SRC != kSendOnly && staged_mode(MODE) && shard == a.rank;
  const int c8 = lane % LPR;
  const long long col = (long long)col0 + SG::col(wn, lane);
  const bool col_ok = col < a.N;
  const long long slot_stride = (long long)a.S * a.N;
  const int slot = staged_mode(MODE) && !owned ? slot_of(shard, a.rank) : 0;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // accumulator registers 8h .. 8h+7 hold rows 16h .. 16h+15 of the stripe
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) - 16 * h;
          stage[row * C::EPI_STRIDE + fn * 32 + (lane & 31)] = acc[fm][fn][r];
        }
      wave_lds_sync();
      if (MODE == kPush) {
        // out holds the P owners' fp32 accumulators, [P][S][N]
        float* accum = reinterpret_cast<float*>(a.out) + (long long)shard * slot_stride;
#pragma unroll
        for (int it = 0; it < PASSES; ++it) {
          const int rr = it * RPI + lane / LPR;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8 + 4);
          const int lr = lrow0 + SG::row(wm, lane, fm, h, it);
          if (lr < a.S && col_ok) {
            float* dst = accum + (long long)lr * a.N + col;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              __hip_atomic_fetch_add(dst + e, x0[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_fetch_add(dst + 4 + e, x1[e], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      } else if (SRC == kSendOnly || !owned) {
#pragma unroll
        for (int it = 0; it < PASSES; ++it) {
          const int rr = it * RPI + lane / LPR;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8 + 4);
          const int lr = lrow0 + SG::row(wm, lane, fm, h, it);
          if (lr < a.S && col_ok) {
            const u32x4 o = {pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                             pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
            uint16_t* dst;
            if (MODE == kGemmOnly || MODE == kAgGemm)
              dst = reinterpret_cast<uint16_t*>(a.out) + ((long long)shard * a.S + lr) * a.N + col;
            else
              dst = a.send + (slot * (long long)a.S + lr) * a.N + col;
            store16(dst, o, a.store_nt);
          }
        }
      } else if constexpr (SRC != kSendOnly) {
#pragma unroll
        for (int it0 = 0; it0 < PASSES; it0 += BATCH) {
          float t[BATCH][8];     // peer sums
          bool ok[BATCH];
          long long base[BATCH];
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            const int lr = lrow0 + SG::row(wm, lane, fm, h, it0 + b);
            ok[b] = lr < a.S && col_ok;
            base[b] = ok[b] ? (long long)lr * a.N + col : 0;   // row 0 stays in bounds
            const int sg = (fm * 2 + h) * PASSES + it0 + b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if constexpr (SRC == kPeersPresum) t[b][e] = pv.v[sg][e];
              else t[b][e] = 0.0f;
            }
            if constexpr (SRC == kPeersReduced) {
              const float* ps = a.presum + base[b];
              const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ps));
              const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ps + 4));
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                t[b][e] = __uint_as_float(lo[e]);
                t[b][4 + e] = __uint_as_float(hi[e]);
              }
            }
            if constexpr (SRC == kPeersPrefetch) {
#pragma unroll
              for (int jj = 0; jj < GS; ++jj) add_bf16x8(t[b], pv.v[sg][jj]);
            }
          }
          if constexpr (SRC == kPeersDirect) {
            // ascending slot order; GS slots' loads are in flight together
            for (int j0 = 0; j0 < a.P - 1; j0 += GS) {
              u32x4 q[BATCH][GS];
#pragma unroll
              for (int b = 0; b < BATCH; ++b)
#pragma unroll
                for (int jj = 0; jj < GS; ++jj)
                  q[b][jj] = load16(a.peers + (j0 + jj) * slot_stride + base[b]);
#pragma unroll
              for (int b = 0; b < BATCH; ++b)
#pragma unroll
                for (int jj = 0; jj < GS; ++jj) add_bf16x8(t[b], q[b][jj]);
            }
          }
#pragma unroll
          for (int b = 0; b < BATCH; ++b) {
            const int rr = (it0 + b) * RPI + lane / LPR;
            float* st8 = stage + rr * C::EPI_STRIDE + c8 * 8;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(st8);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(st8 + 4);
            float s8[8] = {t[b][0] + x0[0], t[b][1] + x0[1], t[b][2] + x0[2], t[b][3] + x0[3],
                           t[b][4] + x1[0], t[b][5] + x1[1], t[b][6] + x1[2], t[b][7] + x1[3]};
            if (a.out_bf16) {
              if (ok[b]) store_out(a, base[b], s8);
            } else {
              // fp32: the sums go back over the lane's staged values ...
              *reinterpret_cast<f32x4*>(st8) = f32x4{s8[0], s8[1], s8[2], s8[3]};
              *reinterpret_cast<f32x4*>(st8 + 4) = f32x4{s8[4], s8[5], s8[6], s8[7]};
            }
          }
          if (!a.out_bf16) {
            // ... and leave as two dense halves of each row's run of 8*LPR
            // floats: lane c8 stores floats 4 c8 .. 4 c8 + 3, then 4 LPR +
            // 4 c8 .., so every store instruction writes whole runs of 16 LPR
            // bytes instead of every other 16 bytes (half-written lines would
            // each be written through twice)
            wave_lds_sync();
            float* out32 = reinterpret_cast<float*>(a.out);
            const long long colr = (long long)col0 + wn * C::WN;
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
              const int rr = (it0 + b) * RPI + lane / LPR;
              const int lr = lrow0 + SG::row(wm, lane, fm, h, it0 + b);
              const float* row = stage + rr * C::EPI_STRIDE;
#pragma unroll
              for (int half = 0; half < 2; ++half) {
                const int c = half * 4 * LPR + 4 * c8;
                const f32x4 y = *reinterpret_cast<const f32x4*>(row + c);
                if (lr < a.S && colr + c < a.N)
                  store16(out32 + (long long)lr * a.N + colr + c,
                          u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                                __float_as_uint(y[3])},
                          a.store_nt);
              }
            }
          }
        }
      }
      wave_lds_sync();
    }
  }
}

// Epilogue of a gathered-row tile of row group g (configuration C, 256 rows:
// gather_row).  PART 0: the send half stripes, bf16 into the send slot of
// their rows' shard (16 rows that start at a multiple of 16 never straddle
// two shards); PART 1: the wave's owned half stripe (fm = FM-1, h = 1), out
// = peer sum (`ps`, ascending slot order from +0) + C, as the owned epilogue
// adds it.
template <class C, int PART, class PS>
__device__ __forceinline__ void gather_epilogue(const KArgs& a, int g, int col0, float* lds_f,
                                                int wave, int wm, int wn, int lane,
                                                f32x16 (&acc)[C::FM][C::FN], const PS& ps) {
  using SG = Seg<C>;
  static_assert(C::BM == kGatherRows && C::WAVES_M == 2, "two 128-row halves of gathered rows");
  float* stage = lds_f + wave * 16 * C::EPI_STRIDE;
  constexpr int LPR = SG::LPR, RPI = SG::RPI, PASSES = SG::PASSES;
  const int c8 = lane % LPR;
  const long long col = (long long)col0 + SG::col(wn, lane);
  const bool col_ok = col < a.N;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool owned_hs = fm == C::FM - 1 && h == 1;
      if (owned_hs != (PART == 1)) continue;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) - 16 * h;
          stage[row * C::EPI_STRIDE + fn * 32 + (lane & 31)] = acc[fm][fn][r];
        }
      wave_lds_sync();
      if constexpr (PART == 0) {
        int slot, lrow;
        gather_send_row(kGatherSendRows * g + 112 * wm + 32 * fm + 16 * h, a.S, slot, lrow);
#pragma unroll
        for (int it = 0; it < PASSES; ++it) {
          const int rr = it * RPI + lane / LPR;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(stage + rr * C::EPI_STRIDE + c8 * 8 + 4);
          if (col_ok) {
            const u32x4 o = {pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                             pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
            store16(a.send + (slot * (long long)a.S + lrow + rr) * a.N + col, o, a.store_nt);
          }
        }
      } else {
        const int olr = kGatherOwnedRows * g + 16 * wm;
#pragma unroll
        for (int it = 0; it < PASSES; ++it) {
          const int rr = it * RPI + lane / LPR;
          float* st8 = stage + rr * C::EPI_STRIDE + c8 * 8;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(st8);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(st8 + 4);
          float s8[8] = {ps.v[it][0] + x0[0], ps.v[it][1] + x0[1], ps.v[it][2] + x0[2],
                         ps.v[it][3] + x0[3], ps.v[it][4] + x1[0], ps.v[it][5] + x1[1],
                         ps.v[it][6] + x1[2], ps.v[it][7] + x1[3]};
          if (a.out_bf16) {
            if (col_ok) store_out(a, (long long)(olr + rr) * a.N + col, s8);
          } else {
            *reinterpret_cast<f32x4*>(st8) = f32x4{s8[0], s8[1], s8[2], s8[3]};
            *reinterpret_cast<f32x4*>(st8 + 4) = f32x4{s8[4], s8[5], s8[6], s8[7]};
          }
        }
        if (!a.out_bf16) {
          // fp32: dense halves of each row's run of 8*LPR floats, as in the
          // owned epilogue
          wave_lds_sync();
          float* out32 = reinterpret_cast<float*>(a.out);
          const long long colr = (long long)col0 + wn * C::WN;
#pragma unroll
          for (int it = 0; it < PASSES; ++it) {
            const int rr = it * RPI + lane / LPR;
            const float* row = stage + rr * C::EPI_STRIDE;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int c = half * 4 * LPR + 4 * c8;
              const f32x4 y = *reinterpret_cast<const f32x4*>(row + c);
              if (colr + c < a.N)
                store16(out32 + (long long)(olr + rr) * a.N + colr + c,
                        u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                              __float_as_uint(y[3])},
                        a.store_nt);
            }
          }
        }
      }
      wave_lds_sync();
    }
  }
}

// Release of a gathered-row tile of row group g, whose stores every thread has
// waited for and met the others at a barrier after: wave 0 releases and adds
// the tile's arrivals at every chunk its send rows touch, one (slot, chunk)
// pair per lane.  Wave 0 meets the other waves at one more barrier as soon as
// its first 64 arrivals are issued, so the stores the others go on to issue
// queue behind those arrivals rather than ahead of them (measured 3 % of the
// comm-dominant share); it looks at what they returned after the barrier.
// Pairs past the first 64 (chunks of a few rows only) follow one per lane.
// Every wave of the workgroup calls it.
// The send rows were stored with store16, which writes through the L2 at
// system scope (sc0 sc1), and every wave has waited for its stores to complete
// before the barrier ahead of this call: they are already visible beyond the
// L2, so the release only has to keep the arrivals behind them, which a
// workgroup-scope release does (a wait, no writeback of the L2, measured 1 us
// of the comm-dominant share).  The arrival that completes a chunk still
// acquires and raises the ready word with a device-scope release.
__device__ __forceinline__ void gather_release(const KArgs& a, int g, int wave, int lane) {
  if (wave != 0) {
    __builtin_amdgcn_s_barrier();
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  int idx = -1, n = 0;
  uint32_t want = 0;
  gather_chunks(g, a.P, a.S, a.chunk_rows, [&](int d, int c) {
    if (n++ == lane) {
      idx = d * a.n_chunks + c;
      want = gather_expected_arrivals(d, c, a.S, a.chunk_rows, a.g.Tn);
    }
  });
  const uint32_t old = idx >= 0 ? arrive_chunk(a, idx) : 0u;
  __builtin_amdgcn_s_barrier();
  if (idx >= 0 && old + 1u == want) complete_chunk(a, idx);
  if (n > 64) {
    int m = 0;
    gather_chunks(g, a.P, a.S, a.chunk_rows, [&](int d, int c) {
      if (m >= 64 && m % 64 == lane)
        signal_chunk(a, d * a.n_chunks + c,
                     gather_expected_arrivals(d, c, a.S, a.chunk_rows, a.g.Tn));
      ++m;
    });
  }
}

// All-gather + GEMM: before a tile of rank tc.shard's rows reads A, one
// thread waits (the pages' wait primitive) until the ready word of every A
// chunk the tile's rows touch has reached wait_expected, a signed 32-bit
// distance so counts may wrap, polling each at most spin_limit times; every
// wave then acquires, so the loads of the tile see the chunk data.  A wait
// that gives up sets *wait_error and the tile is computed from whatever the
// rows hold, so a missing producer ends the kernel instead of hanging it.
__device__ __forceinline__ void wait_rows(const KArgs& a, const TileCoord& tc, int BM, int tid) {
  if (tid == 0) {
    int c0, c1;
    chunks_of_row_tile(tc.t, BM, a.S, a.chunk_rows, c0, c1);
    bool all = true;
    for (int c = c0; c <= c1; ++c) {
      const uint32_t* w = a.wait_ready + (long long)tc.shard * a.n_chunks + c;
      int polls = 0;
      while ((int32_t)(__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                       a.wait_expected) < 0) {
        if (++polls >= a.spin_limit) {
          all = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (!all) __hip_atomic_store(a.wait_error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Reduction role of the inter-CU schedule.  The peer sum of the owned shard
// is written into presum by the communicator workgroups in pieces of
// kPiece x kPiece elements; a piece's word rises by one per call once its
// sums are visible at device scope (the counting convention of the ready
// words).
constexpr int kPiece = 64;

// Wave 0 polls `n` words (word q at `at(q)`), lane l taking q = l, l+64, ...,
// until each reaches wait_expected (a signed 32-bit distance) or spin_limit
// polls; a word given up ORs `bit` into *wait_error.  Every wave then
// acquires at device scope.
template <class At>
__device__ __forceinline__ bool wait_words(const KArgs& a, int n, int bit, uint32_t expected,
                                           int wave, int lane, const At& at) {
  __shared__ int all_arrived;
  if (wave == 0) {
    bool ok = true;
    for (int q = lane; q < n; q += 64) {
      const uint32_t* w = at(q);
      int polls = 0;
      while ((int32_t)(__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                       expected) < 0) {
        if (++polls >= a.spin_limit) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (!ok) __hip_atomic_fetch_or(a.wait_error, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool all = __builtin_amdgcn_ballot_w64(!ok) == 0;
    if (lane == 0) all_arrived = all ? 1 : 0;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const bool all = all_arrived != 0;
  __syncthreads();   // every wave has read the verdict before the next wait writes it
  return all;
}

// An owned item of `rows` x `cols` at (lrow0, col0) waits for the words of
// the pieces it covers before its epilogue reads presum; false (the same in
// every wave) when a word was given up.
__device__ __forceinline__ bool wait_pieces(const KArgs& a, int lrow0, int col0, int rows,
                                            int cols, int wave, int lane) {
  const int r1 = lrow0 + rows < a.S ? lrow0 + rows : a.S;
  const int c1 = col0 + cols < a.N ? col0 + cols : a.N;
  const int pr0 = lrow0 / kPiece, pc0 = col0 / kPiece;
  const int npc = (c1 - 1) / kPiece - pc0 + 1;
  const int n = ((r1 - 1) / kPiece - pr0 + 1) * npc;
  return wait_words(a, n, 1, a.piece_expected, wave, lane, [&](int q) {
    return a.piece_ready + (long long)(pr0 + q / npc) * a.piece_cols + pc0 + q % npc;
  });
}

// LDS of the kernel: a ring of up to four stage buffers shared by the tile
// configurations it runs; buffer 0 also holds the epilogue staging area.
template <class C1, class C2>
struct LdsPlan {
  static constexpr int mx(int x, int y) { return x > y ? x : y; }
  static constexpr int B0 = mx(C1::LDS0, C2::LDS0);
  static constexpr int BS = mx(C1::STAGE_BYTES, C2::STAGE_BYTES);
  static constexpr int ST = mx(C1::STAGES, C2::STAGES);
  static constexpr int B2 = ST > 2 ? BS : 16;
  static constexpr int B3 = ST > 3 ? BS : 16;
  static_assert((B0 + BS + B2 + B3) * C1::OCC <= 160 * 1024, "fits the 160 KiB LDS of a CU");
};

// Main loop of one work item: a tile of configuration C whose first row is
// shard-local row `lrow0` of shard `shard` and whose first column is `col0`,
// multiplied into `acc`.  `bg` runs in the background of the main loop; an
// owned item that takes its peer sum by prefetch (SRC kPeersPrefetch) reads
// it into `pf`.  On return every stage load has landed and every wave has
// passed a barrier, so the ring may be refilled.  With GA the tile is a
// gathered-row tile: `lrow0` is its row group and `shard` is unused.
// The first stages (0 .. S-2) of a work item into the ring b0, b1, ... as
// main_part issues them; a caller that issues them early (before the previous
// item's epilogue, so their latency hides behind its stores) then runs
// main_part with PRE.
// An item's coordinates are the same in every lane, but the compiler cannot
// always prove it (an item chosen after a wait whose result went through LDS,
// say); read from the first lane they stay in scalar registers, and so do
// the buffer descriptors built from them (a descriptor taken for divergent
// costs a loop over the lanes around every load that uses it).
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <class C>
__device__ __forceinline__ void issue_prologue(const KArgs& a, int shard, int lrow0, int col0,
                                               unsigned char* b0, unsigned char* b1,
                                               unsigned char* b2, int wave, int lane) {
  constexpr int S = C::STAGES, NQ = C::LOADS;
  shard = uniform_int(shard);
  lrow0 = uniform_int(lrow0);
  col0 = uniform_int(col0);
  const long long row0 = (long long)shard * a.S + lrow0;
  Loader<C> ld;
  ld.init(a, wave, lane);
  ld.bind(a, a.S - lrow0, col0);
  if ((a.K + C::BK - 1) / C::BK > 0) {
    ld.template issue<0, NQ>(a, ld.stage(a, row0, col0, 0), b0, wave);
    if constexpr (S > 2) ld.template issue<0, NQ>(a, ld.stage(a, row0, col0, C::BK), b1, wave);
    if constexpr (S > 3) ld.template issue<0, NQ>(a, ld.stage(a, row0, col0, 2 * C::BK), b2, wave);
  }
}

template <class C, int GS, int SRC, class BG, class PFT, bool PRE = false, bool GA = false>
__device__ __forceinline__ void main_part(const KArgs& a, int shard, int lrow0, int col0,
                                          unsigned char* b0, unsigned char* b1,
                                          unsigned char* b2, unsigned char* b3, int wave,
                                          int lane, BG& bg, PFT& pf,
                                          f32x16 (&acc)[C::FM][C::FN]) {
  constexpr int S = C::STAGES;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  shard = uniform_int(shard);
  lrow0 = uniform_int(lrow0);
  col0 = uniform_int(col0);
  // GA (gathered rows): lrow0 is the row group and every A row of the tile
  // carries its own row of A
  const long long row0 = GA ? 0 : (long long)shard * a.S + lrow0;
  Loader<C> ld;
  ld.init(a, wave, lane);
  if constexpr (GA) ld.bind_gather(a, lrow0, col0, wave, lane);
  else ld.bind(a, a.S - lrow0, col0);
  const int nk = (a.K + C::BK - 1) / C::BK;

  // prologue: stages 0 .. S-2 (already issued by the caller with PRE).  The
  // loads go out first; zeroing the accumulators (one instruction per
  // register, some 256 per lane) and the reader's set-up then run while
  // they are in flight instead of delaying them.
  constexpr int NQ = C::LOADS;
  if (!PRE && nk > 0) {
    ld.template issue<0, NQ, GA>(a, ld.stage(a, row0, col0, 0), b0, wave);
    if constexpr (S > 2) ld.template issue<0, NQ, GA>(a, ld.stage(a, row0, col0, C::BK), b1, wave);
    if constexpr (S > 3) ld.template issue<0, NQ, GA>(a, ld.stage(a, row0, col0, 2 * C::BK), b2, wave);
  }
  __builtin_amdgcn_sched_barrier(0);
  Reader<C> rd;
  rd.init(wm, wn, lane);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  if (nk > 0) {
    // Loads complete in issue order, so this leaves stages 1 .. S-2 in
    // flight; older stores of the previous item are retired too (with PRE,
    // the stores issued after the prologue as well: the wait is only longer).
    wait_vm<(S - 2) * NQ>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    PK_MARK(a, 1);
  }
  typename Reader<C>::Frags f[2];
  if (nk > 0) rd.read(b0, 0, f[0]);
  // Owned sub-items read their peer partials now; the loads must land by the
  // end of the first step, one stage of MFMA later.
  if constexpr (SRC == kPeersPrefetch) pf.load(a, lrow0, col0, wm, wn, lane);
  if (nk > 0) {
    // S steps per trip, step I multiplies buffer I and fills buffer
    // (I + S - 1) % S with the stage S-1 ahead.  A last partial trip
    // multiplies stages of zeros, which leaves the accumulators unchanged
    // (they never hold -0).
    for (int kq = 0; kq < nk; kq += S) {
#define PK_STEP(I)                                                                           \
  main_stage<C, (I), BG, GA>(a, ld, ld.stage(a, row0, col0, (kq + (I) + S - 1) * C::BK), rd, \
                             pick<(I)>(b0, b1, b2, b3), pick<((I) + S - 1) % S>(b0, b1, b2, b3), \
                             pick<((I) + 1) % S>(b0, b1, b2, b3), wave, acc, f, bg)
      PK_STEP(0);
      PK_STEP(1);
      if constexpr (S > 2) PK_STEP(2);
      if constexpr (S > 3) PK_STEP(3);
#undef PK_STEP
      bg.end_trip();
    }
    wait_vm0();        // loads of stages past the end (zeros) into the staging area
    __syncthreads();
  }
  bg.finish(a);
  PK_MARK(a, 2);
}

// One work item: its main loop (main_part), then its epilogue.  An owned
// item takes its peer sum from source SRC (`pv` for kPeersPresum).
template <class C, int MODE, int GS, int SRC, class BG, class PV, bool PRE = false>
__device__ __forceinline__ void process(const KArgs& a, int shard, int lrow0, int col0,
                                        unsigned char* b0, unsigned char* b1, unsigned char* b2,
                                        unsigned char* b3, int tid, int wave, int lane, BG& bg,
                                        const PV& pv) {
  (void)tid;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  using PFT = typename std::conditional<SRC == kPeersPrefetch, PeerPrefetch<C, GS>, NoPeers>::type;
  PFT pf;
  f32x16 acc[C::FM][C::FN];
  main_part<C, GS, SRC, BG, PFT, PRE>(a, shard, lrow0, col0, b0, b1, b2, b3, wave, lane, bg, pf,
                                      acc);
  using PVT = typename std::conditional<SRC == kPeersPrefetch, PFT, PV>::type;
  const PVT* src;
  if constexpr (SRC == kPeersPrefetch) src = &pf;
  else src = &pv;
  if constexpr (SRC == kPeersReduced) {
    // An owned item reads the communicators' sums once their pieces have
    // risen; if a wait gives up (a reduction workgroup that never ran, on a
    // device shared with other work), it sums its staged peers itself, so
    // `out` is right either way and the error word tells the caller.
    if (shard == a.rank && !wait_pieces(a, lrow0, col0, C::BM, C::BN, wave, lane)) {
      epilogue<C, MODE, GS, kPeersDirect, PVT>(a, shard, lrow0, col0, reinterpret_cast<float*>(b0),
                                               wave, wm, wn, lane, acc, *src);
      return;
    }
  }
  epilogue<C, MODE, GS, SRC, PVT>(a, shard, lrow0, col0, reinterpret_cast<float*>(b0), wave, wm,
                                  wn, lane, acc, *src);
  PK_MARK(a, 3);
}

// The persistent kernel: workgroup w takes walk positions w, w+G, w+2G, ...
// Whole tiles use configuration CS.  Under the owned split (CO != CS) a
// position holds a send tile and an owned CO sub-tile: the workgroup
// multiplies the send tile while it sums the sub-tile's peer partials in the
// background, sends, then multiplies the sub-tile and adds that sum.
// Positions past the end of one list hold only the other (a lone sub-tile
// reads its peer partials ahead into registers).
// Communicator workgroup r of nc: the owned items of the walk (the same
// sub-tiles or whole tiles the compute workgroups take, in the owned
// shard's walk order of this launch's grid), items r, r+nc, ...
// For each: wait for the incoming chunks its rows touch (when peer_ready is
// given; a word given up ORs 2 into *wait_error and the rows are summed as
// they are), sum its staged peer partials in ascending slot order from +0
// in fp32 (GS slots' loads in flight per element group), store the sums
// into presum, release, and raise the words of its pieces.
template <int GS, int THREADS>
__device__ __forceinline__ void reduce_units(const KArgs& a, int r, int nc, int tid, int wave,
                                             int lane) {
  const Grid& g = a.g;
  const int R = g.Rm * g.Rn;
  const int ur = g.BM / g.Rm, uc = g.BN / g.Rn;
  const long long n_units = (long long)R * g.Tm * g.Tn;
  const long long slot_stride = (long long)a.S * a.N;
  constexpr int U = 4;   // element groups (8 columns) per thread in flight
  for (long long j = r; j < n_units; j += nc) {
    const long long i = j / R;
    const int sub = (int)(j - i * R);
    int t, u;
    intra_shard(g, i, t, u);
    const int r0 = t * g.BM + (sub / g.Rn) * ur;
    const int c0 = u * g.BN + (sub % g.Rn) * uc;
    const int nr = ur < a.S - r0 ? ur : a.S - r0;
    const int ncol = uc < a.N - c0 ? uc : a.N - c0;
    if (a.peer_ready) {
      const int ch0 = r0 / a.chunk_rows, nch = (r0 + nr - 1) / a.chunk_rows - ch0 + 1;
      wait_words(a, (a.P - 1) * nch, 2, a.wait_expected, wave, lane, [&](int q) {
        return a.peer_ready + (long long)(q / nch) * a.n_chunks + ch0 + q % nch;
      });
    }
    const int gpr = ncol / 8;
    const int ng = nr * gpr;
    for (int g0 = tid; g0 < ng; g0 += U * THREADS) {
      float acc[U][8];
      long long base[U];
      bool ok[U];
#pragma unroll
      for (int b = 0; b < U; ++b) {
        const int gi = g0 + b * THREADS;
        ok[b] = gi < ng;
        const int rr = ok[b] ? gi / gpr : 0;
        base[b] = ok[b] ? (long long)(r0 + rr) * a.N + c0 + (gi - rr * gpr) * 8 : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[b][e] = 0.0f;
      }
      for (int j0 = 0; j0 < a.P - 1; j0 += GS) {
        u32x4 q[U][GS];
#pragma unroll
        for (int b = 0; b < U; ++b)
#pragma unroll
          for (int jj = 0; jj < GS; ++jj)
            q[b][jj] = load16(a.peers + (j0 + jj) * slot_stride + base[b]);
#pragma unroll
        for (int b = 0; b < U; ++b)
#pragma unroll
          for (int jj = 0; jj < GS; ++jj) add_bf16x8(acc[b], q[b][jj]);
      }
#pragma unroll
      for (int b = 0; b < U; ++b) {
        if (!ok[b]) continue;
        float* dst = a.presum + base[b];
        store16(dst, u32x4{__float_as_uint(acc[b][0]), __float_as_uint(acc[b][1]),
                           __float_as_uint(acc[b][2]), __float_as_uint(acc[b][3])}, a.store_nt);
        store16(dst + 4, u32x4{__float_as_uint(acc[b][4]), __float_as_uint(acc[b][5]),
                               __float_as_uint(acc[b][6]), __float_as_uint(acc[b][7])},
                a.store_nt);
      }
    }
    wait_vm0();   // this thread's sums have reached the cache
    __syncthreads();
    if (wave == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // ... and memory
      const int npc = (ncol + kPiece - 1) / kPiece;
      const int n = (nr + kPiece - 1) / kPiece * npc;
      for (int q = lane; q < n; q += 64)
        __hip_atomic_fetch_add(a.piece_ready + (long long)(r0 / kPiece + q / npc) * a.piece_cols +
                                   c0 / kPiece + q % npc,
                               1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <class CS, class CO, int MODE, int GS, int ONE = 0>
__global__ void __launch_bounds__(CS::THREADS)
    __attribute__((amdgpu_waves_per_eu(CS::OCC * CS::WAVES / 4))) pk_gemm_rs_fused(KArgs a) {
  using L = LdsPlan<CS, CO>;
  constexpr bool SPLIT = !__is_same(CS, CO);
  static_assert(CS::THREADS == CO::THREADS, "one workgroup size");
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[L::B0];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[L::BS];
  __shared__ __attribute__((aligned(1024))) unsigned char lds2[L::B2];
  __shared__ __attribute__((aligned(1024))) unsigned char lds3[L::B3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  PK_TL_START(a);

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of walk positions.
  // Inter-CU schedule (the pages' communication workers): the first n_comm
  // workgroups, a multiple of 8 so the XCD of a compute workgroup is still
  // blockIdx & 7, move finished send chunks into the staging buffers while
  // the rest compute.  All of them are resident at once (the host sizes the
  // grid to the device), and every wait they make is bounded.
  if (a.n_comm > 0 && (int)blockIdx.x < a.n_comm) {
    if constexpr (MODE == kFusedReduce)
      reduce_units<GS, CS::THREADS>(a, blockIdx.x, a.n_comm, tid, wave, lane);
    else
      pkm::move_chunks<CS::THREADS>(a.mv, blockIdx.x, a.n_comm, tid,
                                    reinterpret_cast<int*>(lds0));
    return;
  }
  const int G = gridDim.x - a.n_comm;
  int w = blockIdx.x - a.n_comm;
  if ((G & 7) == 0) w = (w & 7) * (G >> 3) + (w >> 3);

  // Round k covers walk positions kG .. kG+G-1.  Without the split the
  // position a workgroup takes moves by one every round, so work that recurs
  // at a fixed stride of the walk (the owned tiles of the round-robin order,
  // one in every P positions) rotates over the workgroups instead of falling
  // on the same G/P of them; an XCD's positions in a round stay contiguous.
  const auto pos = [&](long long k) -> long long {
    return k * G + (SPLIT ? w : (int)((w + k) % G));
  };

  NoBackground nobg;
  NoPeers nopv;
  // Finished send tiles are signalled in batches: one device-scope release
  // (an L2 writeback on this multi-XCD part, several microseconds) covers up
  // to a.sig_batch tiles.  Rounds fk .. k hold the tiles not yet signalled.
  long long fk = 0;
  int npend = 0;
  const long long n_send = SPLIT ? split_sends(a.g) : 0;
  const long long n_own = SPLIT ? split_owned(a.g) : 0;
  // Release the pending send tiles of rounds fk .. k and raise their chunks.
  const auto flush = [&](long long k) {
    wait_vm0();            // this thread's stores have reached the cache
    __syncthreads();
    if (wave == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // ... and the whole cache, memory
      signal_batch(a, fk, k, CS::BM, lane, [&](long long k2, TileCoord& tc) {
        const long long s2 = pos(k2);
        if constexpr (SPLIT) {
          if (s2 >= n_send) return false;
          tc = send_item(a.g, s2);
          return true;
        } else {
          tc = tile_at(a.g, s2);
          return tc.shard != a.rank;
        }
      });
    }
    fk = k + 1;
    npend = 0;
    PK_MARK(a, 4);
  };
  if constexpr (MODE == kFusedReduce && SPLIT && GS == 7) {
    if (a.n_comm == 0) {
      // Reduction in the background of the main loops (no communicator
      // workgroups): one whole tile per workgroup, P = 8 and sub-tiles of an
      // eighth of a tile (the host checks both and that the grid holds every
      // tile).  Workgroup w < n_send multiplies send tile w; workgroup
      // n_send + t multiplies owned tile t.  While it multiplies, each sums
      // the staged peer partials of one owned sub-tile (PresumStream): send
      // tile w sub-tile w % 7 of owned tile w / 7, owned tile t its own
      // sub-tile 7.  It stores that sum into presum, releases it, and raises
      // the sub-tile's piece words; then a send tile is sent and signalled,
      // and an owned tile waits for the pieces of its eight sub-tiles and
      // stores out = presum + C.  The sums and their order are the fused
      // epilogue's, so every output is the staged share's, bit for bit.
      constexpr int R = 8;
      const int wm = wave / CO::WAVES_N, wn = wave % CO::WAVES_N;
      const long long n_tiles = a.g.tiles_per_shard();
      if (w >= n_send + n_tiles) return;
      const bool is_send = w < n_send;
      const long long oi = is_send ? w / (R - 1) : w - n_send;
      const int osub = is_send ? (int)(w % (R - 1)) : R - 1;
      int ot, ou;
      intra_shard(a.g, oi, ot, ou);
      const int olr = ot * CS::BM + (osub / a.g.Rn) * CO::BM;
      const int oc = ou * CS::BN + (osub % a.g.Rn) * CO::BN;
      int shard = a.rank, lrow0 = ot * CS::BM, col0 = ou * CS::BN;
      if (is_send) {
        const TileCoord st = send_item(a.g, w);
        shard = st.shard;
        lrow0 = st.t * CS::BM;
        col0 = st.u * CS::BN;
      }
      const int nr = CO::BM < a.S - olr ? CO::BM : a.S - olr;
      const int ncol = CO::BN < a.N - oc ? CO::BN : a.N - oc;
      if (a.peer_ready && nr > 0 && ncol > 0) {
        // the incoming chunks the sub-tile's rows touch must have arrived
        const int ch0 = olr / a.chunk_rows, nch = (olr + nr - 1) / a.chunk_rows - ch0 + 1;
        wait_words(a, (a.P - 1) * nch, 2, a.wait_expected, wave, lane, [&](int q) {
          return a.peer_ready + (long long)(q / nch) * a.n_chunks + ch0 + q % nch;
        });
      }
      PresumStream<CO, GS, CS::STAGES * CS::KK> ps;
      ps.init(a, olr, oc, wm, wn, lane);
      f32x16 acc[CS::FM][CS::FN];
      main_part<CS, GS, kPeersDirect>(a, shard, lrow0, col0, lds0, lds1, lds2, lds3, wave, lane,
                                      ps, nopv, acc);
      using SG = Seg<CO>;
      const int pc = oc + SG::col(wn, lane);
#pragma unroll
      for (int fm = 0; fm < CO::FM; ++fm)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int it = 0; it < SG::PASSES; ++it) {
            const int pr = olr + SG::row(wm, lane, fm, h, it);
            const int sg = (fm * 2 + h) * SG::PASSES + it;
            if (pr < a.S && pc < a.N) {
              float* dst = a.presum + (long long)pr * a.N + pc;
              store16(dst, u32x4{__float_as_uint(ps.v[sg][0]), __float_as_uint(ps.v[sg][1]),
                                 __float_as_uint(ps.v[sg][2]), __float_as_uint(ps.v[sg][3])},
                      a.store_nt);
              store16(dst + 4, u32x4{__float_as_uint(ps.v[sg][4]), __float_as_uint(ps.v[sg][5]),
                                     __float_as_uint(ps.v[sg][6]), __float_as_uint(ps.v[sg][7])},
                      a.store_nt);
            }
          }
      wait_vm0();   // this thread's sums have reached the cache
      __syncthreads();
      if (wave == 0 && nr > 0 && ncol > 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // ... and memory
        const int npc = (ncol + kPiece - 1) / kPiece;
        const int n = (nr + kPiece - 1) / kPiece * npc;
        for (int q = lane; q < n; q += 64)
          __hip_atomic_fetch_add(a.piece_ready + (long long)(olr / kPiece + q / npc) * a.piece_cols +
                                     oc / kPiece + q % npc,
                                 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (is_send) {
        epilogue<CS, MODE, GS, kSendOnly, NoPeers>(a, shard, lrow0, col0,
                                                   reinterpret_cast<float*>(lds0), wave, wm, wn,
                                                   lane, acc, nopv);
        flush(0);
      } else if (wait_pieces(a, lrow0, col0, CS::BM, CS::BN, wave, lane)) {
        epilogue<CS, MODE, GS, kPeersReduced, NoPeers>(a, shard, lrow0, col0,
                                                       reinterpret_cast<float*>(lds0), wave, wm,
                                                       wn, lane, acc, nopv);
      } else {
        // a sub-tile's sums never rose (its workgroup was not resident):
        // the owned tile sums its staged peers itself
        epilogue<CS, MODE, GS, kPeersDirect, NoPeers>(a, shard, lrow0, col0,
                                                      reinterpret_cast<float*>(lds0), wave, wm,
                                                      wn, lane, acc, nopv);
      }
      return;
    }
  }
  if constexpr (ONE == 2) {
    static_assert(MODE == kFused && SPLIT && GS == 7 && CS::OCC == 2, "the two-per-CU schedule");
    // Two workgroups share each CU (the host launches this instance only
    // when the work fits): the first half of the grid, dispatched first, one
    // per CU, and the second half beside it.  A first-half workgroup
    // multiplies send tile j and sends it; the one beside it first takes
    // owned sub-tile j (its peers read ahead into registers: mostly memory
    // traffic, little MFMA), then multiplies send tile half + j and sends it.
    // So while one workgroup of a CU multiplies, the other is reading peers
    // or storing, and no workgroup waits for its own stores before its next
    // loads.  Within each half the positions of one XCD are contiguous.
    const int half = (int)(gridDim.x / 2);
    const int b = blockIdx.x;
    const bool first = b < half;
    const int bb = first ? b : b - half;
    const int j = (half & 7) == 0 ? (bb & 7) * (half >> 3) + (bb >> 3) : bb;
    if (first) {
      if (j < n_send) {
        w = j;   // the walk position flush() signals
        const TileCoord st = send_item(a.g, w);
        process<CS, MODE, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0, lds1,
                                            lds2, lds3, tid, wave, lane, nobg, nopv);
        flush(0);
      }
    } else {
      if (j < n_own) {
        const TileCoord ot = owned_item(a.g, j);
        const int sm = ot.sub / a.g.Rn, sn = ot.sub - sm * a.g.Rn;
        process<CO, MODE, GS, kPeersPrefetch>(a, ot.shard, ot.t * CS::BM + sm * CO::BM,
                                              ot.u * CS::BN + sn * CO::BN, lds0, lds1, lds2,
                                              lds3, tid, wave, lane, nobg, nopv);
      }
      if (half + j < n_send) {
        __syncthreads();   // the staging area is the send tile's first stage
        w = half + j;
        const TileCoord st = send_item(a.g, w);
        process<CS, MODE, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0, lds1,
                                            lds2, lds3, tid, wave, lane, nobg, nopv);
        flush(0);
      }
    }
    return;
  } else if constexpr (ONE == 3) {
    static_assert(MODE == kFused && GS == 7 && !SPLIT && CS::BM == kGatherRows &&
                      CS::WAVES_M == 2 && Seg<CS>::PASSES * 2 * CS::FM == Seg<CS>::COUNT,
                  "the gathered-row schedule");
    // Gathered-row tiles in one round (P = 8; the host launches this
    // instance only when every work item has a workgroup of its own): work
    // item (g, u) multiplies the 256 rows of row group g (224 send rows, 32
    // owned rows) by column tile u while its waves sum their owned half
    // stripes' peer partials in the background, stores the send rows,
    // releases them once and adds its arrivals, then stores the owned rows.
    const int wm = wave / CS::WAVES_N, wn = wave % CS::WAVES_N;
    if (w >= (long long)gather_groups(a.S) * a.g.Tn) return;
    Grid gg = a.g;
    gg.Tm = gather_groups(a.S);
    int grp, u;
    intra_shard(gg, w, grp, u);
    const int col0 = u * CS::BN;
    GatherStream<CS, GS, CS::STAGES * CS::KK> ps;
    ps.init(a, kGatherOwnedRows * grp + 16 * wm, col0, wn, lane);
    f32x16 acc[CS::FM][CS::FN];
    NoPeers nopf;
    main_part<CS, GS, kSendOnly, decltype(ps), NoPeers, false, true>(
        a, 0, grp, col0, lds0, lds1, lds2, lds3, wave, lane, ps, nopf, acc);
    float* stage = reinterpret_cast<float*>(lds0);
    gather_epilogue<CS, 0>(a, grp, col0, stage, wave, wm, wn, lane, acc, ps);
    PK_MARK(a, 3);
    // The send rows are released and signalled before the owned rows are
    // stored, so the release waits for none of those stores and the other
    // waves store theirs while wave 0 signals.
    wait_vm0();   // this thread's stores have reached the cache
    __syncthreads();
    gather_release(a, grp, wave, lane);
    PK_MARK(a, 4);
    gather_epilogue<CS, 1>(a, grp, col0, stage, wave, wm, wn, lane, acc, ps);
    PK_MARK(a, 3);
    return;
  } else if constexpr (ONE == 1) {
    static_assert(MODE == kFused && SPLIT && GS == 7, "the one-round schedule");
    {
      // The owned split in one round with workgroups to spare: G - n_send of
      // them hold no send tile (the host launches this instance only then).
      // Every fourth send tile's workgroup only sends; its owned sub-tile
      // goes to the spare workgroups, which take their own sub-tile and then
      // those, round robin, each with its peers read ahead into registers.
      // The other send tiles' workgroups pair their tile with their own
      // sub-tile as in the walk below.  A paired workgroup is the longest
      // chain (send tile, then sub-tile); a spare one otherwise finishes
      // after a third of it.  A quarter of the sub-tiles fills the spare
      // workgroups without making them the longest: fewer relieved
      // workgroups leave more long chains, and more overload the spare ones.
      const int wm = wave / CO::WAVES_N, wn = wave % CO::WAVES_N;
      const long long spare = G - n_send;
      const long long n_relieved = (n_send + 3) / 4;   // send tiles 0, 4, 8, ...
      const auto owned_ahead = [&](long long j) {
        const TileCoord ot = owned_item(a.g, j);
        const int sm = ot.sub / a.g.Rn, sn = ot.sub - sm * a.g.Rn;
        process<CO, MODE, GS, kPeersPrefetch>(a, ot.shard, ot.t * CS::BM + sm * CO::BM,
                                              ot.u * CS::BN + sn * CO::BN, lds0, lds1, lds2,
                                              lds3, tid, wave, lane, nobg, nopv);
      };
      if (w < n_send) {
        const TileCoord st = send_item(a.g, w);
        if ((w & 3) == 0) {
          process<CS, MODE, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0,
                                              lds1, lds2, lds3, tid, wave, lane, nobg, nopv);
          flush(0);
        } else {
          const TileCoord ot = owned_item(a.g, w);
          const int sm = ot.sub / a.g.Rn, sn = ot.sub - sm * a.g.Rn;
          const int olr = ot.t * CS::BM + sm * CO::BM, oc = ot.u * CS::BN + sn * CO::BN;
          PresumStream<CO, GS, CS::STAGES * CS::KK> ps;
          ps.init(a, olr, oc, wm, wn, lane);
          {
            f32x16 acc[CS::FM][CS::FN];
            NoPeers nopf;
            main_part<CS, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0, lds1,
                                         lds2, lds3, wave, lane, ps, nopf, acc);
            // The sub-tile's first stages go into lds1 .. lds3 (its ring
            // starts at lds1) while the send tile is re-laid in lds0 and
            // stored, so their latency hides behind the stores; its ready
            // words are raised after the sub-tile, with one wait and one
            // release for both.
            issue_prologue<CO>(a, ot.shard, olr, oc, lds1, lds2, lds3, wave, lane);
            epilogue<CS, MODE, GS, kSendOnly, NoPeers>(a, st.shard, st.t * CS::BM, st.u * CS::BN,
                                                       reinterpret_cast<float*>(lds0), wave, wm,
                                                       wn, lane, acc, nopv);
            PK_MARK(a, 3);
          }
          // The send tile's stores were issued before the sub-tile's main
          // loop: release them and raise its ready words once that loop is
          // done, so the release does not also wait for the sub-tile's own
          // stores (which need none); wave 0 releases while the others start
          // the sub-tile's epilogue.
          {
            f32x16 acc[CO::FM][CO::FN];
            NoPeers nopf;
            main_part<CO, GS, kPeersPresum, NoBackground, NoPeers, true>(
                a, ot.shard, olr, oc, lds1, lds2, lds3, lds0, wave, lane, nobg, nopf, acc);
            flush(0);
            epilogue<CO, MODE, GS, kPeersPresum, decltype(ps)>(
                a, ot.shard, olr, oc, reinterpret_cast<float*>(lds1), wave, wm, wn, lane, acc, ps);
            PK_MARK(a, 3);
          }
        }
      } else {
        if (w < n_own) owned_ahead(w);
        for (long long i = w - n_send; i < n_relieved; i += spare) {
          __syncthreads();   // the staging area is the next item's first stage
          owned_ahead(4 * i);
        }
      }
      return;
    }
  } else {   // the walk, round by round
  for (long long k = 0, s = pos(0); s < a.total_tiles; s = pos(++k)) {
    const bool last = pos(k + 1) >= a.total_tiles;
    if constexpr (!SPLIT) {
      const TileCoord tc = tile_at(a.g, s);
      if constexpr (MODE == kAgGemm) {
        if (tc.shard != a.rank) wait_rows(a, tc, CS::BM, tid);
      }
      constexpr int SRC = MODE == kFusedReduce ? kPeersReduced : kPeersDirect;
      process<CS, MODE, GS, SRC>(a, tc.shard, tc.t * CS::BM, tc.u * CS::BN, lds0, lds1, lds2,
                                 lds3, tid, wave, lane, nobg, nopv);
      constexpr bool SIGNALS = staged_mode(MODE) || MODE == kPush;
      if (SIGNALS && tc.shard != a.rank) ++npend;
      if (SIGNALS && npend > 0 && (npend >= a.sig_batch || last)) flush(k);
    } else if constexpr (MODE == kFusedReduce) {
      // the owned sub-tile's peer sum comes from the communicators
      if (s < n_send) {
        const TileCoord st = send_item(a.g, s);
        process<CS, MODE, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0,
                                            lds1, lds2, lds3, tid, wave, lane, nobg, nopv);
        if (++npend >= a.sig_batch || last) flush(k);
      }
      if (s < n_own) {
        if (s < n_send) __syncthreads();   // the staging area is the sub-tile's first stage
        const TileCoord ot = owned_item(a.g, s);
        const int sm = ot.sub / a.g.Rn, sn = ot.sub - sm * a.g.Rn;
        process<CO, MODE, GS, kPeersReduced>(a, ot.shard, ot.t * CS::BM + sm * CO::BM,
                                             ot.u * CS::BN + sn * CO::BN, lds0, lds1, lds2,
                                             lds3, tid, wave, lane, nobg, nopv);
        if (npend > 0 && last) flush(k);
      }
    } else {
      const int wm = wave / CO::WAVES_N, wn = wave % CO::WAVES_N;
      if (s < n_send) {
        const TileCoord st = send_item(a.g, s);
        // A send tile's batch is released before the owned sub-tile that
        // rides with it, so the wait covers only send stores and the ready
        // words rise a sub-tile earlier.  A quarter of the workgroups take
        // the pair the other way round (the sub-tile first, its peers read
        // into registers, then the send tile): their send tiles are written
        // later than the rest, which spreads the burst of send stores that
        // otherwise leaves every CU at once (P = 8; with fewer peer slots the
        // sub-tile's own work is small and the extra code path would spill).
        if (GS == 7 && s < n_own && (w & 3) == 0) {
          const TileCoord ot = owned_item(a.g, s);
          const int sm = ot.sub / a.g.Rn, sn = ot.sub - sm * a.g.Rn;
          process<CO, MODE, GS, kPeersPrefetch>(a, ot.shard, ot.t * CS::BM + sm * CO::BM,
                                                ot.u * CS::BN + sn * CO::BN, lds0, lds1, lds2,
                                                lds3, tid, wave, lane, nobg, nopv);
          __syncthreads();   // the staging area is the send tile's first stage
          process<CS, MODE, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0,
                                              lds1, lds2, lds3, tid, wave, lane, nobg, nopv);
          if (++npend >= a.sig_batch || last) flush(k);
        } else if (s < n_own) {
          const TileCoord ot = owned_item(a.g, s);
          const int sm = ot.sub / a.g.Rn, sn = ot.sub - sm * a.g.Rn;
          const int olr = ot.t * CS::BM + sm * CO::BM, oc = ot.u * CS::BN + sn * CO::BN;
          PresumStream<CO, GS, CS::STAGES * CS::KK> ps;
          ps.init(a, olr, oc, wm, wn, lane);
          process<CS, MODE, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0,
                                              lds1, lds2, lds3, tid, wave, lane, ps, nopv);
          if (++npend >= a.sig_batch || last) flush(k);
          __syncthreads();   // the staging area is the sub-tile's first stage
          process<CO, MODE, GS, kPeersPresum>(a, ot.shard, olr, oc, lds0, lds1, lds2, lds3, tid,
                                              wave, lane, nobg, ps);
        } else {
          process<CS, MODE, GS, kSendOnly>(a, st.shard, st.t * CS::BM, st.u * CS::BN, lds0,
                                              lds1, lds2, lds3, tid, wave, lane, nobg, nopv);
          if (++npend >= a.sig_batch || last) flush(k);
        }
      } else {
        const TileCoord ot = owned_item(a.g, s);
        const int sm = ot.sub / a.g.Rn, sn = ot.sub - sm * a.g.Rn;
        process<CO, MODE, GS, kPeersPrefetch>(a, ot.shard, ot.t * CS::BM + sm * CO::BM,
                                              ot.u * CS::BN + sn * CO::BN, lds0, lds1, lds2,
                                              lds3, tid, wave, lane, nobg, nopv);
        if (npend > 0 && last) flush(k);
      }
    }
    __syncthreads();   // the staging area is the next item's first stage
  }
  }   // the walk
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
    {Cfg4::BM, Cfg4::BN, Cfg4::BK, Cfg4::WM, Cfg4::WN, Cfg4::THREADS},
    {Cfg5::BM, Cfg5::BN, Cfg5::BK, Cfg5::WM, Cfg5::WN, Cfg5::THREADS},
    {Cfg6::BM, Cfg6::BN, Cfg6::BK, Cfg6::WM, Cfg6::WN, Cfg6::THREADS},
};
static constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
static constexpr int kAssumedCUs = 256;   // MI355X; used only for the static pick
static constexpr int kDefaultSignalBatch = 8;

// Column tiles per locality group.  Row-major and owned-first: with 256
// workgroups in flight and 32 per XCD, groups of 8 columns give every XCD a
// 4 x 8 block of tiles at a time.  Dest-round-robin hands an XCD's 32
// positions to 8 shards, 4 consecutive tiles each: groups of 32 columns put
// the 8 XCDs of a round on one row tile of every shard, so each A panel of
// the round is shared by all of them (measured 0.6-2 % faster on the
// 32768-wide shares than groups of 8).
static int default_group_n(const CfgInfo& c, int Tn, int order) {
  (void)c;
  const int gn = order == kDestRoundRobin ? 32 : 8;
  return Tn < gn ? Tn : gn;
}

static int select_config(long long M, long long N, long long K, int P) {
  (void)K;
  const long long S = P > 0 ? M / P : 0;
  static const int order[] = {1, 4, 2, 3};   // largest tile first
  for (int id : order) {
    const CfgInfo& c = kCfgs[id - 1];
    if (S < c.BM || N < c.BN) continue;
    const long long tiles = (long long)P * ((S + c.BM - 1) / c.BM) * ((N + c.BN - 1) / c.BN);
    if (tiles >= kAssumedCUs) return id;
  }
  return 3;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Buffer-load offsets are 32-bit: an A row panel (256 rows x K) and 64 rows of
// B must each stay below 2^31 bytes.
static constexpr long long kMaxK = 1LL << 22;
static constexpr long long kMaxN = 1LL << 24;

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
  if (M > (1LL << 31) || N > kMaxN || K > kMaxK) return PK_ERR_TOO_LARGE;
  if (o && (o->config < 0 || o->config > kNumCfgs)) return PK_ERR_CONFIG;
  if (o && (o->max_workgroups < 0 || o->group_n < 0)) return PK_ERR_CONFIG;
  if (o && (o->owned_split < -1 || o->owned_split > 1)) return PK_ERR_CONFIG;
  if (o && o->signal_batch < 0) return PK_ERR_CONFIG;
  if (o && (o->store_policy < 0 || o->store_policy > 2)) return PK_ERR_CONFIG;
  if (o && o->ready_clock && (reinterpret_cast<uintptr_t>(o->ready_clock) & 7u))
    return PK_ERR_POINTER;
  if (o && o->timeline && (reinterpret_cast<uintptr_t>(o->timeline) & 7u)) return PK_ERR_POINTER;
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

// Arguments of the atomic push variant: `out` is the owners' fp32
// accumulators [P][S][N]; no peers or send buffers; gemm_only and the owned
// split do not apply.
static int validate_push(const void* A, const void* B, const void* accum, const uint32_t* flags,
                         long long M, long long N, long long K, int P, int rank, int chunk_rows,
                         int tile_order, const pk_options* o) {
  if (o && (o->gemm_only != 0 || o->owned_split == 1)) return PK_ERR_CONFIG;
  // the shape, rank, order and option checks of the staged variant; its
  // pointer checks ask for peers and send buffers, so they are redone here
  const int v = validate(A, B, nullptr, nullptr, accum, flags, M, N, K, P, rank, chunk_rows,
                         tile_order, 0, o);
  if (v != PK_OK && v != PK_ERR_POINTER) return v;
  if (M == 0 || N == 0) return PK_OK;
  auto a16 = [](const void* p) { return p != nullptr && aligned16(p); };
  if (!a16(accum) || (K > 0 && (!a16(A) || !a16(B)))) return PK_ERR_POINTER;
  if (P > 1 && (flags == nullptr || (reinterpret_cast<uintptr_t>(flags) & 3u)))
    return PK_ERR_POINTER;
  if (o && o->ready_clock && (reinterpret_cast<uintptr_t>(o->ready_clock) & 7u))
    return PK_ERR_POINTER;
  return PK_OK;
}

// Resident workgroups per CU of one kernel instance, asked once per device.
template <class CS, class CO, int MODE, int GS, int ONE = 0>
static int occupancy_of(int dev) {
  static int occ[64];
  static std::once_flag once[64];
  if (dev < 0 || dev >= 64) return 1;
  std::call_once(once[dev], [&] {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, pk_gemm_rs_fused<CS, CO, MODE, GS, ONE>, CS::THREADS, 0) != hipSuccess ||
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

template <class CS, class CO, int MODE, int GS>
static int launch_as(KArgs& a, const pk_options* o, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PK_ERR_LAUNCH;
  // communicator workgroups come on top of the compute grid and take its
  // place on the device, so that every workgroup is resident at once
  long long grid = (long long)cu_count(dev) * occupancy_of<CS, CO, MODE, GS>(dev) - a.n_comm;
  if (grid < 1) return PK_ERR_CONFIG;
  if (o && o->max_workgroups > 0 && o->max_workgroups < grid) grid = o->max_workgroups;
  // ... and holds every whole tile on its own resident workgroup (the owned
  // tiles wait for sums that the send tiles' workgroups produce)
  if (MODE == kFusedReduce && a.n_comm == 0 && grid < (long long)a.P * a.g.tiles_per_shard())
    return PK_ERR_CONFIG;
  if (grid > a.total_tiles) grid = a.total_tiles;
  if (a.timeline && grid + a.n_comm > kTimelineWorkgroups) return PK_ERR_CONFIG;
  if constexpr (MODE == kFused && __is_same(CS, Cfg1) && __is_same(CO, CfgOwned) && GS == 7) {
    // The owned split at P = 8 with a workgroup for every gathered-row work
    // item (S a multiple of 32, 32-bit row offsets into A): the gathered-row
    // schedule, which needs no sub-tiles.
    const long long items = (long long)gather_groups(a.S) * a.g.Tn;
    if (gather_fits(a.P, a.S) && a.n_comm == 0 && items <= grid &&
        a.M * (long long)a.K * 2 <= (1LL << 31)) {
      hipLaunchKernelGGL((pk_gemm_rs_fused<CS, CS, MODE, GS, 3>), dim3((unsigned)items),
                         dim3(CS::THREADS), 0, stream, a);
      return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_LAUNCH;
    }
  }
  if constexpr (MODE == kFused && !__is_same(CS, CO) && GS == 7) {
    // the owned split in one round with workgroups to spare: its own schedule
    const long long n_send = split_sends(a.g), n_own = split_owned(a.g);
    if (n_send <= grid && n_own <= grid && n_own > n_send) {
      hipLaunchKernelGGL((pk_gemm_rs_fused<CS, CO, MODE, GS, 1>),
                         dim3((unsigned)(grid + a.n_comm)), dim3(CS::THREADS), 0, stream, a);
      return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_LAUNCH;
    }
  }
  hipLaunchKernelGGL((pk_gemm_rs_fused<CS, CO, MODE, GS>), dim3((unsigned)(grid + a.n_comm)),
                     dim3(CS::THREADS), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_LAUNCH;
}

// The owned split in the two-per-CU schedule (configuration 6, P = 8): the
// grid of two workgroups per CU; its first half holds a send tile each, its
// second half every owned sub-tile and the remaining send tiles.  Returns
// PK_ERR_CONFIG (nothing launched) when the work does not fit that grid.
static int launch_two(KArgs& a, const pk_options* o, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PK_ERR_LAUNCH;
  long long grid = (long long)cu_count(dev) * occupancy_of<Cfg6, CfgOwned3, kFused, 7, 2>(dev);
  if (o && o->max_workgroups > 0 && o->max_workgroups < grid) grid = o->max_workgroups;
  grid &= ~1LL;
  const long long half = grid / 2;
  const long long n_send = split_sends(a.g), n_own = split_owned(a.g);
  if (half < 1 || n_own > half || n_send > grid) return PK_ERR_CONFIG;
  if (a.timeline && grid > kTimelineWorkgroups) return PK_ERR_CONFIG;
  hipLaunchKernelGGL((pk_gemm_rs_fused<Cfg6, CfgOwned3, kFused, 7, 2>), dim3((unsigned)grid),
                     dim3(Cfg6::THREADS), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_LAUNCH;
}

// Owned split of configuration `cfg` for a call: on request, or by default
// when the whole-tile walk gives fewer than two tiles per CU (the owned
// tiles then sit on the critical path).  Available for configuration 1 with
// P - 1 in {1, 3, 7} (all peer slots of a segment in one batch) and peer
// partials spanning less than 2^31 bytes (32-bit buffer offsets).
static bool use_owned_split(int cfg, int P, long long S, long long N, long long whole_tiles,
                            const pk_options* o) {
  const int req = o ? o->owned_split : 0;
  const bool able = cfg == 1 && (P == 2 || P == 4 || P == 8) &&
                    2LL * (P - 1) * S * N < (1LL << 31) - 16;
  if (req < 0 || !able) return false;
  if (req > 0) return true;
  return whole_tiles < 2LL * kAssumedCUs;
}

// Staged modes: the peer slots summed per batch of loads are 7 for P = 8
// (and 15, 22, ...), else 3 or 1; the owned split is compiled for
// configuration 1 with P - 1 in {1, 3, 7}.
template <class C, int MODE>
static int launch_staged(KArgs& a, bool split, const pk_options* o, hipStream_t stream) {
  if constexpr (__is_same(C, Cfg1)) {
    if (split) {
      switch (a.P - 1) {
        case 7: return launch_as<C, CfgOwned, MODE, 7>(a, o, stream);
        case 3: return launch_as<C, CfgOwned, MODE, 3>(a, o, stream);
        default: return launch_as<C, CfgOwned, MODE, 1>(a, o, stream);
      }
    }
  }
  const int np = a.P - 1;
  if (np > 0 && np % 7 == 0) return launch_as<C, C, MODE, 7>(a, o, stream);
  if (np > 0 && np % 3 == 0) return launch_as<C, C, MODE, 3>(a, o, stream);
  return launch_as<C, C, MODE, 1>(a, o, stream);
}

template <class C>
static int launch(KArgs& a, int mode, int cfg, const pk_options* o, hipStream_t stream) {
  const bool gemm_only = mode == kGemmOnly;
  a.g.BM = C::BM;
  a.g.BN = C::BN;
  a.g.Tm = a.S > 0 ? ceil_div(a.S, C::BM) : 0;
  a.g.Tn = ceil_div(a.N, C::BN);
  a.g.group_n = (o && o->group_n > 0) ? o->group_n : default_group_n(kCfgs[0], a.g.Tn, a.g.order);
  a.g.Rm = a.g.Rn = 1;
  if constexpr (C::OCC == 2) {
    // Two workgroups per CU: the plain GEMM and the staged share, the latter
    // with the owned split in the two-per-CU schedule at P = 8 unless the
    // split is turned off or the work does not fit it (then whole tiles).
    if (mode != kGemmOnly && mode != kFused) return PK_ERR_CONFIG;
    if (mode == kFused && a.P == 8 && !(o && o->owned_split < 0)) {
      KArgs t = a;
      t.g.Rm = C::BM / OwnedOf<C>::type::BM;
      t.g.Rn = C::BN / OwnedOf<C>::type::BN;
      t.total_tiles = split_pairs(t.g);
      if (t.total_tiles == 0) return PK_OK;
      if (2LL * (a.P - 1) * a.S * a.N < (1LL << 31) - 16) {
        const int r = launch_two(t, o, stream);
        if (r != PK_ERR_CONFIG) return r;
      }
    }
    if (o && o->owned_split > 0) return PK_ERR_CONFIG;
    a.total_tiles = a.g.total();
    if (a.total_tiles == 0) return PK_OK;
    if (gemm_only) return launch_as<C, C, kGemmOnly, 1>(a, o, stream);
    return launch_staged<C, kFused>(a, false, o, stream);
  } else {
  const bool split = staged_mode(mode) && use_owned_split(cfg, a.P, a.S, a.N, a.g.total(), o);
  if (split) {
    a.g.Rm = C::BM / CfgOwned::BM;
    a.g.Rn = C::BN / CfgOwned::BN;
  }
  a.total_tiles = split ? split_pairs(a.g) : a.g.total();
  if (a.total_tiles == 0) return PK_OK;
  // The reduction in the background of the main loops (reduction role with
  // no communicator workgroups) runs configuration 1's owned split at P = 8.
  if (mode == kFusedReduce && a.n_comm == 0 &&
      (!split || !__is_same(C, Cfg1) || a.P != 8 || a.g.R() != 8))
    return PK_ERR_CONFIG;
  if (gemm_only) return launch_as<C, C, kGemmOnly, 1>(a, o, stream);
  if (mode == kPush) return launch_as<C, C, kPush, 1>(a, o, stream);
  if (mode == kAgGemm) return launch_as<C, C, kAgGemm, 1>(a, o, stream);
  if (mode == kFusedReduce) return launch_staged<C, kFusedReduce>(a, split, o, stream);
  return launch_staged<C, kFused>(a, split, o, stream);
  }
}

// Reduction role of the communicators (pk_gemm_rs_intercu_reduce).
struct RedArgs {
  float* presum;
  uint32_t* piece_ready;
  const uint32_t* peer_ready;
  int32_t* error;
  uint32_t expected;         // incoming chunk words
  uint32_t piece_expected;   // piece words
  int spin_limit;
};

// Output stores stream past the caches (nt) unless the call's stored bytes
// fit well inside the 256 MB last-level cache, where the non-temporal hint
// only slows them (pk_options.store_policy overrides).
static constexpr long long kStreamStoreBytes = 64LL << 20;
static int store_nt_for(const pk_options* o, long long stored_bytes) {
  const int policy = o ? o->store_policy : 0;
  if (policy == 1) return 1;
  if (policy == 2) return 0;
  return stored_bytes > kStreamStoreBytes ? 1 : 0;
}

static int run(const void* A, const void* B, const void* peers, void* send, void* out,
               uint32_t* flags, long long M, long long N, long long K, int P, int rank,
               int chunk_rows, int tile_order, int out_bf16, const pk_options* o, void* stream,
               bool push = false, int n_comm = 0, const pkm::MoveArgs* mv = nullptr,
               const RedArgs* red = nullptr) {
  const int v = push ? validate_push(A, B, out, flags, M, N, K, P, rank, chunk_rows, tile_order, o)
                     : validate(A, B, peers, send, out, flags, M, N, K, P, rank, chunk_rows,
                                tile_order, out_bf16, o);
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
  a.N = (int)N;
  a.K = (int)K;
  const bool gemm_only = !push && o && o->gemm_only;
  const int mode = push ? kPush : gemm_only ? kGemmOnly : red ? kFusedReduce : kFused;
  if (gemm_only) {
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
  a.store_nt = store_nt_for(
      o, gemm_only ? 2LL * M * N
                   : (long long)a.S * N * (2LL * (a.P - 1) + (out_bf16 ? 2 : 4)));
  a.sig_batch = (o && o->signal_batch > 0) ? o->signal_batch : kDefaultSignalBatch;
  a.ready_clock = o ? o->ready_clock : nullptr;
  a.timeline = o ? o->timeline : nullptr;
  a.wait_ready = nullptr;
  a.wait_expected = 0;
  a.spin_limit = 1;
  a.wait_error = nullptr;
  a.n_comm = 0;
  a.mv = pkm::MoveArgs{};
  a.presum = nullptr;
  a.piece_ready = nullptr;
  a.piece_cols = 0;
  a.piece_expected = 0;
  a.peer_ready = nullptr;
  if (mv) {
    a.n_comm = n_comm;
    a.mv = *mv;
  }
  if (red) {
    a.n_comm = n_comm;
    a.presum = red->presum;
    a.piece_ready = red->piece_ready;
    a.piece_cols = ceil_div(N, kPiece);
    a.peer_ready = red->peer_ready;
    a.wait_expected = red->expected;
    a.piece_expected = red->piece_expected;
    a.spin_limit = red->spin_limit;
    a.wait_error = red->error;
  }
  const int cfg = (o && o->config > 0) ? o->config : select_config(M, N, K, a.P);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (cfg) {
    case 1: return launch<Cfg1>(a, mode, cfg, o, s);
    case 2: return launch<Cfg2>(a, mode, cfg, o, s);
    case 3: return launch<Cfg3>(a, mode, cfg, o, s);
    case 4: return launch<Cfg4>(a, mode, cfg, o, s);
    case 5: return launch<Cfg5>(a, mode, cfg, o, s);
    case 6: return launch<Cfg6>(a, mode, cfg, o, s);
    default: return PK_ERR_CONFIG;
  }
}

// All-gather + GEMM: C [M][N] bf16 = A [M][K] (gathered rows) * B [K][N].
static int run_ag(const void* A, const uint32_t* a_ready, const void* B, void* Cout,
                  int32_t* error, long long M, long long N, long long K, int P, int rank,
                  int chunk_rows, uint32_t expected, int spin_limit, int tile_order,
                  const pk_options* o, void* stream) {
  if (P < 1 || P > 64 || rank < 0 || rank >= P) return PK_ERR_RANK;
  if (tile_order < 0 || tile_order > 2) return PK_ERR_TILE_ORDER;
  if (M < 0 || N < 0 || K < 0 || M % P != 0 || N % 8 != 0 || K % 8 != 0) return PK_ERR_SHAPE;
  const long long S = M / P;
  if (S > 0 && (chunk_rows <= 0 || S % chunk_rows != 0)) return PK_ERR_SHAPE;
  if (M > (1LL << 31) || N > kMaxN || K > kMaxK) return PK_ERR_TOO_LARGE;
  if (spin_limit < 1) return PK_ERR_CONFIG;
  if (o && (o->config < 0 || o->config > kNumCfgs || o->max_workgroups < 0 || o->group_n < 0 ||
            o->gemm_only != 0 || o->owned_split == 1 || o->signal_batch < 0 ||
            o->store_policy < 0 || o->store_policy > 2))
    return PK_ERR_CONFIG;
  if (M == 0 || N == 0) return PK_OK;
  if (!aligned16(Cout) || (K > 0 && (!aligned16(A) || !aligned16(B)))) return PK_ERR_POINTER;
  if (P > 1 && (a_ready == nullptr || (reinterpret_cast<uintptr_t>(a_ready) & 3u) ||
                error == nullptr || (reinterpret_cast<uintptr_t>(error) & 3u)))
    return PK_ERR_POINTER;
  KArgs a{};
  a.timeline = o ? o->timeline : nullptr;
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.out = Cout;
  a.M = M;
  a.N = (int)N;
  a.K = (int)K;
  a.P = P;
  a.rank = rank;
  a.S = (int)S;
  a.chunk_rows = chunk_rows > 0 ? chunk_rows : 1;
  a.n_chunks = chunk_rows > 0 ? (int)(S / chunk_rows) : 0;
  a.out_bf16 = 1;
  a.store_nt = store_nt_for(o, 2LL * M * N);
  a.sig_batch = 1;
  a.wait_ready = a_ready;
  a.wait_expected = expected;
  a.spin_limit = spin_limit;
  a.wait_error = error;
  a.g.P = P;
  a.g.rank = rank;
  a.g.S = (int)S;
  a.g.N = (int)N;
  a.g.order = tile_order;
  const int cfg = (o && o->config > 0) ? o->config : select_config(M, N, K, P);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (cfg) {
    case 1: return launch<Cfg1>(a, kAgGemm, cfg, o, s);
    case 2: return launch<Cfg2>(a, kAgGemm, cfg, o, s);
    case 3: return launch<Cfg3>(a, kAgGemm, cfg, o, s);
    case 4: return launch<Cfg4>(a, kAgGemm, cfg, o, s);
    case 5: return launch<Cfg5>(a, kAgGemm, cfg, o, s);
    case 6: return launch<Cfg6>(a, kAgGemm, cfg, o, s);
    default: return PK_ERR_CONFIG;
  }
}

// Arguments of the reduction role that both of its entry points check (the
// workspace pointers are checked by the caller).
static int validate_reduce(const void* A, const void* B, const void* peers, const uint32_t* peer_ready,
                           const void* send, const void* out, const uint32_t* flags,
                           const int32_t* error, long long M, long long N, long long K, int P,
                           int rank, int chunk_rows, int tile_order, int out_bf16, int num_comm_cus,
                           int spin_limit, const pk_options* o) {
  if (P < 2) return PK_ERR_RANK;
  if (num_comm_cus < 0 || num_comm_cus > 1024 || spin_limit < 1) return PK_ERR_CONFIG;
  if (o && o->gemm_only) return PK_ERR_CONFIG;
  const int v = validate(A, B, peers, send, out, flags, M, N, K, P, rank, chunk_rows, tile_order,
                         out_bf16, o);
  if (v != PK_OK) return v;
  if (M == 0 || N == 0) return PK_OK;
  auto a4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (error == nullptr || !a4(error) || !a4(peer_ready)) return PK_ERR_POINTER;
  return PK_OK;
}

// Workspace of pk_gemm_rs_intercu_reduce_static, for callers that cannot
// allocate: the fp32 peer sum of the owned shard (at most kScratchSums
// elements, 16 MiB) followed by the piece words (at most kScratchPieces).
// One copy per GPU, held until the process ends; calls on one GPU share it.
constexpr long long kScratchSums = 1LL << 22;
constexpr long long kScratchPieces = 1LL << 16;
__device__ __align__(256) unsigned char scratch[(kScratchSums + kScratchPieces) * 4];

// The device address of this GPU's copy of `scratch`, looked up once per
// device with that device current (host code must never pass the array's
// name itself to a kernel: on the host it is only a stand-in).
static unsigned char* scratch_ptr(int dev) {
  static unsigned char* ptr[64];
  static hipError_t err[64];
  static std::once_flag once[64];
  if (dev < 0 || dev >= 64) return nullptr;
  std::call_once(once[dev], [&] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    ptr[dev] = err[dev] == hipSuccess ? static_cast<unsigned char*>(p) : nullptr;
  });
  return ptr[dev];
}

// Sets n words to v (a kernel, not a memset, so the call can be captured in a
// graph).
__global__ void __launch_bounds__(256) fill_words(uint32_t* p, long long n, uint32_t v) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += gridDim.x * 256LL) p[i] = v;
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

int pk_gemm_rs_push(const void* A, const void* B, float* accum, uint32_t* flags, int64_t M,
                    int64_t N, int64_t K, int P, int rank, int chunk_rows, int tile_order,
                    const pk_options* opts, void* stream) {
  return pk::run(A, B, nullptr, nullptr, accum, flags, M, N, K, P, rank, chunk_rows, tile_order,
                 0, opts, stream, true);
}

int pk_gemm_rs_intercu(const void* A, const void* B, const void* peer_partials, void* send_bufs,
                       void* out, uint32_t* flags, void* dest, int32_t* status, int64_t M,
                       int64_t N, int64_t K, int P, int rank, int chunk_rows, int tile_order,
                       int out_bf16, uint32_t expected, int num_comm_cus, int spin_limit,
                       const pk_options* opts, void* stream) {
  if (P < 2) return PK_ERR_RANK;
  if (num_comm_cus < 1 || num_comm_cus > 1024 || spin_limit < 1) return PK_ERR_CONFIG;
  if (opts && opts->gemm_only) return PK_ERR_CONFIG;
  const int v = pk::validate(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank,
                             chunk_rows, tile_order, out_bf16, opts);
  if (v != PK_OK) return v;
  if (M == 0 || N == 0) return PK_OK;
  if (!pk::aligned16(dest) || status == nullptr || (reinterpret_cast<uintptr_t>(status) & 3u))
    return PK_ERR_POINTER;
  const long long S = M / P, C = S / chunk_rows;
  pkm::MoveArgs mv{};
  mv.ready = flags;
  mv.src = static_cast<const pkm::u32x4*>(send_bufs);
  mv.dst = static_cast<pkm::u32x4*>(dest);
  mv.status = status;
  mv.observed = nullptr;
  mv.units_per_chunk = (long long)chunk_rows * N / 8;
  mv.units_per_slot = S * N / 8;
  mv.C = (int)C;
  mv.items = (int)((P - 1) * C);
  mv.expected = expected;
  mv.spin_limit = spin_limit;
  const int n_comm = (num_comm_cus + 7) / 8 * 8;   // whole XCD rounds
  return pk::run(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                 tile_order, out_bf16, opts, stream, false, n_comm, &mv);
}

int pk_gemm_rs_intercu_reduce(const void* A, const void* B, const void* peer_partials,
                              const uint32_t* peer_ready, void* send_bufs, void* out,
                              uint32_t* flags, float* presum, uint32_t* piece_ready,
                              int32_t* error, int64_t M, int64_t N, int64_t K, int P, int rank,
                              int chunk_rows, int tile_order, int out_bf16, uint32_t expected,
                              int num_comm_cus, int spin_limit, const pk_options* opts,
                              void* stream) {
  const int v = pk::validate_reduce(A, B, peer_partials, peer_ready, send_bufs, out, flags, error,
                                    M, N, K, P, rank, chunk_rows, tile_order, out_bf16,
                                    num_comm_cus, spin_limit, opts);
  if (v != PK_OK || M == 0 || N == 0) return v;
  auto a4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (presum == nullptr || !pk::aligned16(presum) || piece_ready == nullptr || !a4(piece_ready))
    return PK_ERR_POINTER;
  // presum may be the fp32 out itself with communicator workgroups (each
  // element is read, then written, by one thread); not with a bf16 out, and
  // not in the background mode, where a late send tile's workgroup would
  // write its bare peer sum over an owned tile that already stored out
  if (static_cast<const void*>(presum) == out && (out_bf16 || num_comm_cus == 0))
    return PK_ERR_POINTER;
  pk::RedArgs red{presum, piece_ready, peer_ready, error, expected, expected, spin_limit};
  const int n_comm = (num_comm_cus + 7) / 8 * 8;   // whole XCD rounds
  return pk::run(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                 tile_order, out_bf16, opts, stream, false, n_comm, nullptr, &red);
}

int pk_gemm_rs_intercu_reduce_static(const void* A, const void* B, const void* peer_partials,
                                     const uint32_t* peer_ready, void* send_bufs, void* out,
                                     uint32_t* flags, int32_t* error, int64_t M, int64_t N,
                                     int64_t K, int P, int rank, int chunk_rows, int tile_order,
                                     int out_bf16, uint32_t expected, int num_comm_cus,
                                     int spin_limit, const pk_options* opts, void* stream) {
  const int v = pk::validate_reduce(A, B, peer_partials, peer_ready, send_bufs, out, flags, error,
                                    M, N, K, P, rank, chunk_rows, tile_order, out_bf16,
                                    num_comm_cus, spin_limit, opts);
  if (v != PK_OK || M == 0 || N == 0) return v;
  const long long S = M / P;
  const long long pieces = ((S + pk::kPiece - 1) / pk::kPiece) * ((N + pk::kPiece - 1) / pk::kPiece);
  if (S * N > pk::kScratchSums || pieces > pk::kScratchPieces) return PK_ERR_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PK_ERR_LAUNCH;
  unsigned char* ws = pk::scratch_ptr(dev);
  if (ws == nullptr) return PK_ERR_LAUNCH;
  float* presum = reinterpret_cast<float*>(ws);
  uint32_t* piece_ready = reinterpret_cast<uint32_t*>(ws + pk::kScratchSums * 4);
  // the words keep the last call's counts: start this call's from zero
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned blocks = (unsigned)((pieces + 255) / 256);
  hipLaunchKernelGGL(pk::fill_words, dim3(blocks), dim3(256), 0, s, piece_ready, pieces, 0u);
  if (hipGetLastError() != hipSuccess) return PK_ERR_LAUNCH;
  pk::RedArgs red{presum, piece_ready, peer_ready, error, expected, 1u, spin_limit};
  const int n_comm = (num_comm_cus + 7) / 8 * 8;   // whole XCD rounds
  return pk::run(A, B, peer_partials, send_bufs, out, flags, M, N, K, P, rank, chunk_rows,
                 tile_order, out_bf16, opts, stream, false, n_comm, nullptr, &red);
}

int64_t pk_static_workspace_limits(int64_t* max_sum_elements, int64_t* max_piece_words) {
  if (max_sum_elements) *max_sum_elements = pk::kScratchSums;
  if (max_piece_words) *max_piece_words = pk::kScratchPieces;
  return (pk::kScratchSums + pk::kScratchPieces) * 4;
}

int64_t pk_reduce_piece_words(int64_t M, int64_t N, int P) {
  if (P < 1 || P > 64) return PK_ERR_RANK;
  if (M < 0 || N < 0 || M % P != 0) return PK_ERR_SHAPE;
  const int64_t S = M / P;
  return ((S + pk::kPiece - 1) / pk::kPiece) * ((N + pk::kPiece - 1) / pk::kPiece);
}

int pk_ag_gemm(const void* A, const uint32_t* a_ready, const void* B, void* C, int32_t* error,
               int64_t M, int64_t N, int64_t K, int P, int rank, int chunk_rows,
               uint32_t expected, int spin_limit, int tile_order, const pk_options* opts,
               void* stream) {
  return pk::run_ag(A, a_ready, B, C, error, M, N, K, P, rank, chunk_rows, expected, spin_limit,
                    tile_order, opts, stream);
}

int64_t pk_flags_words(int P, int64_t M, int chunk_rows) {
  if (P < 1 || P > 64) return PK_ERR_RANK;
  if (M < 0 || M % P != 0) return PK_ERR_SHAPE;
  const int64_t S = M / P;
  if (S == 0) return 0;
  if (chunk_rows <= 0 || S % chunk_rows != 0) return PK_ERR_SHAPE;
  return (1 + pk::kCounterStride) * (int64_t)(P - 1) * (S / chunk_rows);
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
                     int group_n, int owned_split, int32_t* out4, int64_t cap) {
  if (P < 1 || P > 64 || rank < 0 || rank >= P) return PK_ERR_RANK;
  if (tile_order < 0 || tile_order > 2) return PK_ERR_TILE_ORDER;
  if (M < 0 || N < 0 || M % P != 0) return PK_ERR_SHAPE;
  if (config < 1 || config > pk::kNumCfgs) return PK_ERR_CONFIG;
  if (owned_split < 0 || (owned_split > 0 && config != 1 && config != 6)) return PK_ERR_CONFIG;
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
  g.group_n = group_n > 0 ? group_n : pk::default_group_n(c, g.Tn, tile_order);
  g.Rm = owned_split ? c.BM / pk::CfgOwned::BM : 1;
  g.Rn = owned_split ? c.BN / pk::CfgOwned::BN : 1;
  const long long total = g.total();
  long long n = 0;
  auto put = [&](const pk::TileCoord& tc) {
    if (n < cap) {
      out4[4 * n] = tc.shard;
      out4[4 * n + 1] = tc.t;
      out4[4 * n + 2] = tc.u;
      out4[4 * n + 3] = tc.sub;
    }
    ++n;
  };
  if (!owned_split) {
    for (long long s = 0; s < total; ++s) put(pk::tile_at(g, s));
  } else {
    // pairs in walk order: the send tile, then its owned sub-tile
    const long long pairs = pk::split_pairs(g);
    for (long long s = 0; s < pairs; ++s) {
      if (s < pk::split_sends(g)) put(pk::send_item(g, s));
      if (s < pk::split_owned(g)) put(pk::owned_item(g, s));
    }
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

int pk_gather_rows(int P, int rank, int64_t M, int g, int64_t* rows) {
  if (P < 1 || P > 64 || rank < 0 || rank >= P) return PK_ERR_RANK;
  if (M <= 0 || M % P != 0 || !rows) return PK_ERR_SHAPE;
  const int64_t S = M / P;
  if (!pk::gather_fits(P, S) || S >= (1LL << 31) || g < 0 || g >= pk::gather_groups(S))
    return PK_ERR_CONFIG;
  for (int tr = 0; tr < pk::kGatherRows; ++tr) rows[tr] = pk::gather_row(rank, (int)S, g, tr);
  return PK_OK;
}

int pk_gather_arrivals(int64_t M, int64_t N, int P, int chunk_rows, uint32_t* expected,
                       uint32_t* made) {
  if (P < 1 || P > 64) return PK_ERR_RANK;
  if (M <= 0 || M % P != 0 || N <= 0 || !expected || !made) return PK_ERR_SHAPE;
  const int64_t S = M / P;
  if (!pk::gather_fits(P, S) || S >= (1LL << 31)) return PK_ERR_CONFIG;
  if (chunk_rows <= 0 || S % chunk_rows != 0) return PK_ERR_SHAPE;
  const int n_chunks = (int)(S / chunk_rows), Tn = pk::ceil_div(N, pk::Cfg1::BN);
  for (int64_t i = 0; i < (int64_t)(P - 1) * n_chunks; ++i) {
    expected[i] = pk::gather_expected_arrivals((int)(i / n_chunks), (int)(i % n_chunks), (int)S,
                                               chunk_rows, Tn);
    made[i] = 0;
  }
  for (int g = 0; g < pk::gather_groups(S); ++g)
    pk::gather_chunks(g, P, (int)S, chunk_rows,
                      [&](int d, int c) { made[(int64_t)d * n_chunks + c] += (uint32_t)Tn; });
  return PK_OK;
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
    case PK_ERR_SCRATCH: return "shape needs more than the static workspace holds (pk_static_workspace_limits)";
    default: return "unknown error";
  }
}

int pk_version(void) { return 100; }

}  // extern "C"
