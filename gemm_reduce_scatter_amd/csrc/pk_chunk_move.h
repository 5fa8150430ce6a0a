// Moving finished send chunks: the transfer half of the reduce-scatter.
//
// Shared by the standalone chunk consumer (pk_consume.hip) and the
// communicator workgroups of the fused kernel (pk_gemm_rs.hip).  A chunk of
// send slot j is rows [c*chunk_rows, (c+1)*chunk_rows) of send_bufs[j]; once
// its ready word has reached the producer call being moved (the pages' wait
// primitive, "The Eight PK Primitives" of the ParallelKittens summary page;
// Syncopate section 5.1 chunks), it is copied into dest[j], the staging
// buffer of the rank that owns those rows in a multi-GPU run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct MoveArgs {
  const uint32_t* ready;       // [P-1][C] ready words of the producer's flags
  const u32x4* src;            // send_bufs, bf16 [P-1][S][N] as 16-byte units
  u32x4* dst;                  // dest, same layout
  int32_t* status;             // [P-1][C]: 0 moved, 1 gave up
  uint64_t* observed;          // [P-1][C] or null: device clock when the word was seen
  long long units_per_chunk;   // chunk_rows * N / 8
  long long units_per_slot;    // S * N / 8
  int C, items;                // chunks per slot, (P-1) * C
  uint32_t expected;
  int spin_limit;
};

constexpr int kUnroll = 8;

// Workgroup `w` of `G` moves items w, w+G, ... (item i = slot i / C, chunk
// i % C, the order the row-major walk completes chunks).  One thread polls
// the item's word with relaxed loads and short sleeps, at most spin_limit
// times (a signed 32-bit distance, so counts may wrap); on success every wave
// acquires at device scope and the workgroup copies the chunk with kUnroll
// non-temporal 16-byte loads in flight per thread.  A chunk given up keeps
// its dest rows and gets status 1, so a producer that never signals ends the
// mover instead of hanging it.  `ok_sh` is one int of LDS.
template <int THREADS>
__device__ __forceinline__ void move_chunks(const MoveArgs& a, int w, int G, int tid,
                                            int* ok_sh) {
  for (int item = w; item < a.items; item += G) {
    if (tid == 0) {
      int polls = 0;
      bool ok = false;
      for (;;) {
        const uint32_t v = __hip_atomic_load(&a.ready[item], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if ((int32_t)(v - a.expected) >= 0) {
          ok = true;
          break;
        }
        if (++polls >= a.spin_limit) break;
        __builtin_amdgcn_s_sleep(2);
      }
      const uint64_t t = wall_clock64();
      a.status[item] = ok ? 0 : 1;
      if (a.observed) a.observed[item] = ok ? t : 0;
      *ok_sh = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = *ok_sh != 0;
    if (ok) {
      // The producer raised the word with a device-scope release; this
      // acquire makes its send stores visible to the loads below.
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const int j = item / a.C, c = item - j * a.C;
      const long long base = (long long)j * a.units_per_slot + (long long)c * a.units_per_chunk;
      const u32x4* s = a.src + base;
      u32x4* d = a.dst + base;
      long long u = tid;
      for (; u + (kUnroll - 1) * THREADS < a.units_per_chunk; u += kUnroll * THREADS) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int r = 0; r < kUnroll; ++r) v[r] = __builtin_nontemporal_load(s + u + r * THREADS);
#pragma unroll
        for (int r = 0; r < kUnroll; ++r) __builtin_nontemporal_store(v[r], d + u + r * THREADS);
      }
      for (; u < a.units_per_chunk; u += THREADS) d[u] = s[u];
    }
    __syncthreads();   // ok_sh is rewritten by the next item
  }
}

}  // namespace pkm
