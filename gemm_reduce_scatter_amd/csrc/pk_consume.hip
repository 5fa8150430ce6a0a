// Chunk consumer: the transfer half of the reduce-scatter, the step that
// follows the fused share.  One GPU stands in for the links: a chunk whose
// ready word has reached the producer call being consumed is copied from the
// producer's send buffer into a destination staging buffer, which in a
// multi-GPU run is the buffer of the rank that owns those rows.
//
// Sources: the pages' wait primitive ("ParallelKittens: Systematic and
// Practical Simplification of Multi-GPU AI Kernels", "The Eight PK
// Primitives": wait spins on a counter until it reaches an expected value)
// and Syncopate's chunk ("Syncopate: Efficient Multi-GPU AI Kernels via
// Automatic Chunk-Centric Compute-Communication Overlap", section 5.1: a
// chunk is moved as one unit once the tiles that form it are produced).
//
// Work layout: item i is (slot j, chunk c) with i = j * C + c, C = S /
// chunk_rows, the order in which the row-major tile walk completes chunks.
// Workgroup w takes items w, w+G, ....  One thread polls the item's ready
// word with relaxed loads and a short sleep between polls, at most
// spin_limit times; on success every wave acquires at device scope and the
// workgroup copies the chunk (chunk_rows x N bf16) with 16-byte loads and
// stores.  On time-out the chunk is left alone and its status says so, so
// a dead producer ends the kernel instead of hanging it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pk_gemm_rs.h"

namespace pkc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CArgs {
  const uint32_t* ready;   // [P-1][C] ready words of the producer's flags
  const u32x4* src;        // send_bufs, bf16 [P-1][S][N] as 16-byte units
  u32x4* dst;              // dest, same layout
  int32_t* status;         // [P-1][C]
  uint64_t* observed;      // [P-1][C] or null
  long long units_per_chunk;   // chunk_rows * N / 8
  long long units_per_slot;    // S * N / 8
  int C, items;
  uint32_t expected;
  int spin_limit;
};

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kThreads) pk_rs_consume_kernel(CArgs a) {
  __shared__ int ok_sh;
  const int tid = threadIdx.x;
  for (int item = blockIdx.x; item < a.items; item += gridDim.x) {
    if (tid == 0) {
      int polls = 0;
      bool ok = false;
      for (;;) {
        const uint32_t v = __hip_atomic_load(&a.ready[item], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        // counts wrap at 2^32: compare as a signed distance
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
      ok_sh = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = ok_sh != 0;
    if (ok) {
      // The producer raised the word with a device-scope release; this
      // acquire makes its send stores visible to the loads below.
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const int j = item / a.C, c = item - j * a.C;
      const long long base = (long long)j * a.units_per_slot + (long long)c * a.units_per_chunk;
      const u32x4* s = a.src + base;
      u32x4* d = a.dst + base;
      // kUnroll loads in flight per thread before their stores: the copy is
      // bound by bytes in flight per CU, not by instructions
      long long u = tid;
      for (; u + (kUnroll - 1) * kThreads < a.units_per_chunk; u += kUnroll * kThreads) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int r = 0; r < kUnroll; ++r) v[r] = __builtin_nontemporal_load(s + u + r * kThreads);
#pragma unroll
        for (int r = 0; r < kUnroll; ++r) __builtin_nontemporal_store(v[r], d + u + r * kThreads);
      }
      for (; u < a.units_per_chunk; u += kThreads) d[u] = s[u];
    }
    __syncthreads();   // ok_sh is rewritten by the next item
  }
}

}  // namespace pkc

extern "C" int pk_rs_consume(const uint32_t* flags, const void* send_bufs, void* dest,
                             int64_t M, int64_t N, int P, int chunk_rows, uint32_t expected,
                             int spin_limit, int32_t* status, uint64_t* observed,
                             int max_workgroups, void* stream) {
  if (P < 2 || P > 64) return PK_ERR_RANK;
  if (M <= 0 || N <= 0 || M % P != 0 || N % 8 != 0 || chunk_rows <= 0) return PK_ERR_SHAPE;
  const long long S = M / P;
  if (S % chunk_rows != 0) return PK_ERR_SHAPE;
  if (spin_limit < 1 || max_workgroups < 0) return PK_ERR_CONFIG;
  const long long C = S / chunk_rows;
  const long long items = (long long)(P - 1) * C;
  if (items > (1LL << 30) || S * N > (1LL << 40)) return PK_ERR_TOO_LARGE;
  auto a16 = [](const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!a16(send_bufs) || !a16(dest) || flags == nullptr || status == nullptr ||
      (reinterpret_cast<uintptr_t>(flags) & 3u) || (reinterpret_cast<uintptr_t>(status) & 3u) ||
      (observed && (reinterpret_cast<uintptr_t>(observed) & 7u)))
    return PK_ERR_POINTER;
  pkc::CArgs a;
  a.ready = flags;
  a.src = static_cast<const pkc::u32x4*>(send_bufs);
  a.dst = static_cast<pkc::u32x4*>(dest);
  a.status = status;
  a.observed = observed;
  a.units_per_chunk = (long long)chunk_rows * N / 8;
  a.units_per_slot = S * N / 8;
  a.C = (int)C;
  a.items = (int)items;
  a.expected = expected;
  a.spin_limit = spin_limit;
  long long grid = max_workgroups > 0 ? max_workgroups : 32;
  if (grid > items) grid = items;
  hipLaunchKernelGGL(pkc::pk_rs_consume_kernel, dim3((unsigned)grid), dim3(pkc::kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? PK_OK : PK_ERR_LAUNCH;
}
