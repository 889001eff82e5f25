// The launch order of the halo gather-GEMM's tiles, from the per-tile work
// estimates that the kernel-map kernel writes with each tile's plan
// (halo_plan.h).
#include "common.h"
#include "launch.h"

namespace trsc {
namespace {

// The launch order of the tiles: a counting sort by decreasing cost in one
// workgroup (bucket b holds cost kHaloMaxCost - b). Tiles of equal cost are
// placed by atomics, in no fixed order: the order only schedules the
// gather-GEMM's workgroups, each of which computes its own rows the same way
// wherever it runs.
constexpr int kOrderThreads = 1024;
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderBuckets = 1024;
static_assert(kHaloMaxCost < kOrderBuckets && kOrderBuckets == kOrderThreads, "cost buckets");
__global__ __launch_bounds__(kOrderThreads) void halo_order(const uint16_t* __restrict__ costs, int64_t tiles,
                                                            int32_t* __restrict__ order) {
  __shared__ uint32_t cnt[kOrderBuckets];
  __shared__ uint32_t wsum[kOrderWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  cnt[tid] = 0u;
  __syncthreads();
  for (int64_t t = tid; t < tiles; t += kOrderThreads) atomicAdd(&cnt[kHaloMaxCost - int(costs[t])], 1u);
  __syncthreads();
  {  // exclusive scan of the bucket counts
    const uint32_t own = cnt[tid];
    uint32_t x = own;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    cnt[tid] = before + x - own;
  }
  __syncthreads();
  for (int64_t t = tid; t < tiles; t += kOrderThreads)
    order[atomicAdd(&cnt[kHaloMaxCost - int(costs[t])], 1u)] = int32_t(t);
}

}  // namespace

hipError_t launch_halo_order(const uint16_t* costs, int64_t tiles, int32_t* order, hipStream_t st) {
  if (tiles <= 0) return hipSuccess;
  halo_order<<<1, kOrderThreads, 0, st>>>(costs, tiles, order);
  return hipGetLastError();
}

}  // namespace trsc
