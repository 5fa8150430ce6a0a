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
// The per-chunk wait and copy are move_chunks (pk_chunk_move.h), which the
// fused kernel's communicator workgroups run as well.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pk_chunk_move.h"
#include "pk_gemm_rs.h"

namespace pkc {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) pk_rs_consume_kernel(pkm::MoveArgs a) {
  __shared__ int ok_sh;
  pkm::move_chunks<kThreads>(a, blockIdx.x, gridDim.x, threadIdx.x, &ok_sh);
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
  pkm::MoveArgs a;
  a.ready = flags;
  a.src = static_cast<const pkm::u32x4*>(send_bufs);
  a.dst = static_cast<pkm::u32x4*>(dest);
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
