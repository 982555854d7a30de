// Grouped expert FFN kernels (routed experts and the always-on shared ones).
//
// Up to 128 rows a block is one 16-row tile and one slice pair (the tile
// parts of expert_core.h), with the tile's activation rows staged in LDS as
// the MFMA A operand.  Small batches skip the separate grouping kernel: every gate/up block groups
// the T*k routed pairs itself (one wavefront, a few ballots per expert) and
// block (0, 0) also writes the grouping for the down kernel.
#include "expert_core.h"

namespace mv {

namespace {

// Grouping of a small batch, built in LDS by every gate/up block.
struct Grouping {
  int cnt[kThreads], run[kThreads];
  int seg[kMaxExperts + 1];
  int tile_start[kMaxExperts + 1];
  int rows[kSmallT * kMaxSlots];
};

// Tile `tile` of the grouping: from the global table (large batches) or,
// for small batches, by grouping the pairs in this block.
__device__ bool block_tile(const ExpertArgs &p, int tile, TileInfo &ti, Grouping &g, bool write_global) {
  const int ne = p.E + p.S;
  if (!p.group_in_block) {
    if (tile >= p.tile_start[ne]) return false;
    const int4 v = p.tile_info[tile];
    ti.e = v.x;
    ti.r0 = v.y;
    ti.m = v.z;
    return true;
  }
  const GroupOut lds{g.seg, g.tile_start, g.rows, nullptr};
  group_pairs(p.ids, p.T, p.E, p.S, p.k, p.nslot, kTileM, lds, g.cnt, g.run, kThreads / kWave);
  __syncthreads();
  if (write_global) {  // the grouping of record, for the down kernel
    for (int i = threadIdx.x; i <= ne; i += blockDim.x) {
      p.seg[i] = g.seg[i];
      p.tile_start[i] = g.tile_start[i];
    }
    for (int i = threadIdx.x; i < p.T * p.nslot; i += blockDim.x) p.rows[i] = g.rows[i];
    for (int e = threadIdx.x; e < ne; e += blockDim.x) {
      const int c = g.seg[e + 1] - g.seg[e];
      for (int j = 0; j * kTileM < c; ++j)
        p.tile_info[g.tile_start[e] + j] =
            make_int4(e, g.seg[e] + j * kTileM, min(kTileM, c - j * kTileM), 0);
    }
  }
  if (tile >= g.tile_start[ne]) return false;
  int e = 0;
  while (e + 1 < ne && g.tile_start[e + 1] <= tile) ++e;
  ti.e = e;
  ti.r0 = g.seg[e] + (tile - g.tile_start[e]) * kTileM;
  ti.m = min(kTileM, g.seg[e + 1] - ti.r0);
  return true;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_gate_up(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ Grouping g;
  __shared__ float up_acc[2][64][4];
  constexpr int VN = Vec<T>::N;
  TileInfo ti;
  if (!block_tile(p, blockIdx.y, ti, g, p.group_in_block && blockIdx.x == 0 && blockIdx.y == 0))
    return;
  GateUpPart<T> part;
  part.begin(p, ti, blockIdx.x, threadIdx.x);  // first weights in flight while x is staged

  const int d = p.d, nvec = d / VN, lda = d + VN;
  const int *rows = p.group_in_block ? g.rows : p.rows;
  T *A = reinterpret_cast<T *>(smem);
  const T *x = static_cast<const T *>(p.x);
  for (int it = threadIdx.x; it < kTileM * nvec; it += blockDim.x) {
    const int rr = it / nvec, c = it - rr * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < ti.m) v = ld16(x + static_cast<size_t>(rows[ti.r0 + rr] / p.nslot) * d + c * VN);
    st16(A + rr * lda + c * VN, v);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  part.finish(p, ti, A + (lane & 15) * lda + (lane >> 4) * VN, up_acc, threadIdx.x);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_down(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float half_acc[2][64][4];
  constexpr int VN = Vec<T>::N;
  if (blockIdx.y >= p.tile_start[p.E + p.S]) return;
  const int4 tv = p.tile_info[blockIdx.y];
  const TileInfo ti{tv.x, tv.y, tv.z};
  DownPart<T> part;
  part.begin(p, ti, blockIdx.x, threadIdx.x);  // first weights in flight while a is staged
  stage_a_tile<T>(p, ti, reinterpret_cast<T *>(smem), threadIdx.x, blockDim.x);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  part.finish(p, ti, reinterpret_cast<const T *>(smem) + (lane & 15) * (p.F + VN) + (lane >> 4) * VN, half_acc,
              threadIdx.x);
}

// ------------------------------------------------------------ medium batches
//
// Tiles of up to MT * 16 rows of one expert and one wavefront per 16 output
// columns, with no LDS: each wavefront reads its A fragments from global
// memory (they stay in L2) next to its weight stream, so every weight row is
// read once per tile instead of once per 16 rows.  Loads run one batch of
// kMidWin windows ahead of the MFMAs.  Per-row arithmetic is the 16-row
// kernels': gate and up each one MFMA chain over K in window order; down two
// chains over the K halves, added low half first.
constexpr int kMidWin = 2;

// acc[c][i] += A_i * B_c over windows [w_lo, w_hi) for NB weight streams.
template <typename T, int MT, int NB>
__device__ __forceinline__ void mid_chain(f32x4_t (*acc)[MT], const T *const *ar, const T *const *b,
                                          int w_lo, int w_hi) {
  constexpr int WIN = 4 * Vec<T>::N, U = kMidWin;
  uint4 qb[2][NB][U], qa[2][MT][U];
  auto load = [&](int buf, int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = min(w0 + u, w_hi - 1);
#pragma unroll
      for (int c = 0; c < NB; ++c) qb[buf][c][u] = ld16(b[c] + w * WIN);
#pragma unroll
      for (int i = 0; i < MT; ++i) qa[buf][i][u] = ld16(ar[i] + w * WIN);
    }
  };
  if (w_lo >= w_hi) return;
  load(0, w_lo);
  int buf = 0;
  for (int w0 = w_lo; w0 < w_hi; w0 += U, buf ^= 1) {
    if (w0 + U < w_hi) load(buf ^ 1, w0 + U);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (w0 + u < w_hi) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int c = 0; c < NB; ++c) mfma16(acc[c][i], qa[buf][i][u], qb[buf][c][u], T());
      }
  }
}

template <typename T, int MT>
__global__ __launch_bounds__(kThreads) void k_gate_up_mid(ExpertArgs p) {
  constexpr int VN = Vec<T>::N, WIN = 4 * VN;
  if (blockIdx.y >= p.tile_start[p.E + p.S]) return;
  const int4 tv = p.tile_info[blockIdx.y];
  const int e = tv.x, r0 = tv.y, m = tv.z;
  const int d = p.d, F = p.F;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int f0 = (blockIdx.x * (kThreads / kWave) + wv) * 16;
  if (f0 >= F) return;  // no block-wide synchronisation below
  const int r = lane & 15, koff = (lane >> 4) * VN;
  const T *W = expert_base<T>(p, e, static_cast<size_t>(2) * F * d);
  const T *b[2] = {W + static_cast<size_t>(f0 + r) * d + koff, W + static_cast<size_t>(F + f0 + r) * d + koff};
  const T *x = static_cast<const T *>(p.x);
  const T *ar[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = i * 16 + r;
    const int pair = p.rows[r0 + (row < m ? row : 0)];
    ar[i] = x + static_cast<size_t>(pair / p.nslot) * d + koff;
  }
  f32x4_t acc[2][MT];  // [gate | up][tile]
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    acc[0][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[1][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  mid_chain<T, MT, 2>(acc, ar, b, 0, d / WIN);
  T *aout = static_cast<T *>(p.a_out);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = i * 16 + (lane >> 4) * 4 + j;
      if (row < m) {
        const float gv = acc[0][i][j], uv = acc[1][i][j];
        aout[static_cast<size_t>(r0 + row) * F + f0 + r] = from_f32<T>(gv / (1.0f + expf(-gv)) * uv);
      }
    }
  }
}

template <typename T, int MT>
__global__ __launch_bounds__(kThreads) void k_down_mid(ExpertArgs p) {
  constexpr int VN = Vec<T>::N, WIN = 4 * VN;
  if (blockIdx.y >= p.tile_start[p.E + p.S]) return;
  const int4 tv = p.tile_info[blockIdx.y];
  const int e = tv.x, r0 = tv.y, m = tv.z;
  const int d = p.d, F = p.F;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * (kThreads / kWave) + wv) * 16;
  if (n0 >= d) return;
  const int r = lane & 15, koff = (lane >> 4) * VN;
  const T *b[1] = {expert_base<T>(p, e, static_cast<size_t>(d) * F) + static_cast<size_t>(n0 + r) * F + koff};
  const T *a = static_cast<const T *>(p.a);
  const T *ar[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = i * 16 + r;
    ar[i] = a + static_cast<size_t>(r0 + (row < m ? row : 0)) * F + koff;
  }
  f32x4_t lo[1][MT], hi[1][MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    lo[0][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    hi[0][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int nwin = F / WIN;
  mid_chain<T, MT, 1>(lo, ar, b, 0, nwin / 2);
  mid_chain<T, MT, 1>(hi, ar, b, nwin / 2, nwin);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = i * 16 + (lane >> 4) * 4 + j;
      if (row < m) {
        const int pair = p.rows[r0 + row];
        const int tok = pair / p.nslot, s = pair - tok * p.nslot;
        const float w = s < p.k ? p.gates[tok * p.k + s] : 1.0f;
        p.slots[static_cast<size_t>(pair) * d + n0 + r] = w * (lo[0][i][j] + hi[0][i][j]);
      }
    }
  }
}

template <typename KernelT>
void allow_lds(KernelT kernel, size_t bytes) {
  if (bytes > 48 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

}  // namespace

hipError_t launch_gate_up(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.F + 31) / 32, max_tiles);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t smem = kTileM * (a.d + 16 / es) * es;
  if (dtype == 1) {
    allow_lds(k_gate_up<bf16_t>, smem);
    hipLaunchKernelGGL(k_gate_up<bf16_t>, grid, dim3(kThreads), smem, s, a);
  } else {
    allow_lds(k_gate_up<float>, smem);
    hipLaunchKernelGGL(k_gate_up<float>, grid, dim3(kThreads), smem, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_down(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.d + 31) / 32, max_tiles);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t smem = kTileM * (a.F + 16 / es) * es;
  if (dtype == 1) {
    allow_lds(k_down<bf16_t>, smem);
    hipLaunchKernelGGL(k_down<bf16_t>, grid, dim3(kThreads), smem, s, a);
  } else {
    allow_lds(k_down<float>, smem);
    hipLaunchKernelGGL(k_down<float>, grid, dim3(kThreads), smem, s, a);
  }
  return hipGetLastError();
}

}  // namespace mv

namespace mv {

hipError_t launch_gate_up_mid(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.F + 63) / 64, max_tiles);
  if (dtype == 1)
    hipLaunchKernelGGL((k_gate_up_mid<bf16_t, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_gate_up_mid<float, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_mid(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.d + 63) / 64, max_tiles);
  if (dtype == 1)
    hipLaunchKernelGGL((k_down_mid<bf16_t, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_down_mid<float, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mv
