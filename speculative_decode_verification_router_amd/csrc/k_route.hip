// Routing kernels: per-token combine, RMSNorm, router and top-k (arithmetic
// in route_core.h), and the grouping of (token, slot) pairs by expert.
//
// A routing block of 16 wavefronts handles `ntok` tokens: one token per
// block on the small-batch path (the whole block on one token's latency
// chain), sixteen on the large-batch path (router weights shared by the
// tile).  Large batches are then grouped by a separate kernel: a ballot-based
// one on one block for up to 16384 pairs, else a stable counting sort
// (per-thread histogram over contiguous pair ranges, an exclusive scan in
// (expert, thread) order, and a scatter that keeps ascending pair order
// inside every expert segment).
#include "route_core.h"

namespace mv {

namespace {

// kLogits: blocks (token, expert group), the groups of a token adjacent.
__host__ __device__ inline int route_groups(const RouteArgs &a) {
  return a.mode == kLogits ? (a.E + kRouteGroup - 1) / kRouteGroup : 1;
}

template <typename T>
__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a, CombineArgs c, int ntok) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = route_groups(a);
  const int t0 = blockIdx.x / G * ntok;
  route_block<T>(a, c, t0, min(ntok, a.T - t0), ntok, smem, blockIdx.x % G);
}

__global__ __launch_bounds__(kRouteThreads) void k_group(RouteArgs a) {
  __shared__ int cnt_lds[kRouteWaves * kWave], run_lds[kRouteWaves * kWave];
  const GroupOut o{a.seg, a.tile_start, a.rows, a.tile_info};
  group_pairs(a.ids, a.T, a.E, a.S, a.k, a.nslot, a.tile_m, o, cnt_lds, run_lds, kRouteWaves);
}

__global__ __launch_bounds__(256) void k_permute_large(RouteArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int E = p.E, S = p.S, k = p.k, T = p.T;
  const int stride = E + 2;  // u16 per thread row; odd dword stride avoids bank conflicts
  uint16_t *hist = reinterpret_cast<uint16_t *>(smem);               // [256][E+2]
  int *segl = reinterpret_cast<int *>(smem + 256 * stride * 2 + 16);  // [E+S+1]
  int *cnt = segl + (E + S + 1);                                      // [E]

  const int np = T * k;
  const int cp = (np + 255) / 256;
  const int p0 = min(np, tid * cp), p1 = min(np, p0 + cp);

  for (int e = 0; e < E; ++e) hist[tid * stride + e] = 0;
  for (int q = p0; q < p1; ++q) {
    const int e = min(max(p.ids[q], 0), E - 1);  // ids are always in range; clamp defensively
    hist[tid * stride + e] = hist[tid * stride + e] + 1;
  }
  __syncthreads();
  if (tid < E) {
    int s = 0;
    for (int i = 0; i < 256; ++i) s += hist[i * stride + tid];
    cnt[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, tiles = 0;
    for (int e = 0; e < E + S; ++e) {
      const int c = e < E ? cnt[e] : T;
      segl[e] = off;
      p.seg[e] = off;
      p.tile_start[e] = tiles;
      off += c;
      tiles += (c + p.tile_m - 1) / p.tile_m;
    }
    segl[E + S] = off;
    p.seg[E + S] = off;
    p.tile_start[E + S] = tiles;
  }
  __syncthreads();
  if (tid < E) {  // per expert: exclusive scan over threads (offsets within the segment)
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int c = hist[i * stride + tid];
      hist[i * stride + tid] = static_cast<uint16_t>(run);
      run += c;
    }
  }
  __syncthreads();
  for (int q = p0; q < p1; ++q) {
    const int e = min(max(p.ids[q], 0), E - 1);
    const int pos = segl[e] + hist[tid * stride + e];
    hist[tid * stride + e] = hist[tid * stride + e] + 1;
    p.rows[pos] = (q / k) * p.nslot + (q % k);
  }
  for (int j = tid; j < S * T; j += 256) {
    const int s = j / T, t = j % T;
    p.rows[segl[E + s] + t] = t * p.nslot + k + s;
  }
  // tile table: one thread per expert segment
  if (tid < E + S) {
    const int c = segl[tid + 1] - segl[tid];
    const int first = p.tile_start[tid];
    for (int j = 0; j * p.tile_m < c; ++j)
      p.tile_info[first + j] = make_int4(tid, segl[tid] + j * p.tile_m, min(p.tile_m, c - j * p.tile_m), 0);
  }
}

__global__ void k_copy_status(const unsigned *word, int32_t *status) {
  status[0] = static_cast<int32_t>(ld_agent(word));
}

}  // namespace

hipError_t launch_copy_status(const unsigned *word, int32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(1), 0, s, word, status);
  return hipGetLastError();
}

hipError_t launch_route(int dtype, const RouteArgs &a, const CombineArgs &c, int ntok, hipStream_t s) {
  const size_t smem = route_smem(ntok, a.d, dtype == 1 ? 2 : 4).total;
  const void *k = dtype == 1 ? reinterpret_cast<const void *>(k_route<bf16_t>)
                             : reinterpret_cast<const void *>(k_route<float>);
  if (smem > 48 * 1024)
    (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (a.mode == kLogits && ntok != 1) return hipErrorInvalidValue;
  const dim3 grid((a.T + ntok - 1) / ntok * route_groups(a));
  if (dtype == 1)
    hipLaunchKernelGGL(k_route<bf16_t>, grid, dim3(kRouteThreads), smem, s, a, c, ntok);
  else
    hipLaunchKernelGGL(k_route<float>, grid, dim3(kRouteThreads), smem, s, a, c, ntok);
  return hipGetLastError();
}

hipError_t launch_permute(const RouteArgs &a, hipStream_t s) {
  if (a.T * a.k <= 16 * 1024) {
    hipLaunchKernelGGL(k_group, dim3(1), dim3(kRouteThreads), 0, s, a);
  } else {
    const size_t smem =
        256 * static_cast<size_t>(a.E + 2) * 2 + 16 + 4 * static_cast<size_t>(2 * a.E + a.S + 1);
    hipLaunchKernelGGL(k_permute_large, dim3(1), dim3(256), smem, s, a);
  }
  return hipGetLastError();
}

}  // namespace mv
