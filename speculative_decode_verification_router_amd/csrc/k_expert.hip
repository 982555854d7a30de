// Grouped expert FFN kernels (routed experts and the always-on shared ones).
//
// Both kernels work on "tiles" of up to 16 rows of one expert's segment of
// the sorted (token, slot) pair list.  The A operand (activation rows) is
// staged in LDS; the weights are streamed from HBM once per tile straight
// into MFMA operand registers (16-byte loads, several K-windows in flight per
// lane).  Each wavefront owns 16 output columns over the full K.
//
//   gate/up:  g = x W_gate^T, u = x W_up^T (fp32), a = round(SiLU(g) * u)
//   down:     y = a W_down^T (fp32); slot[pair] = w_pair * y
// where w_pair is the softmax gate of the routed pair, or 1 for a shared
// expert (architecture paragraph of "Jina AI Releases jina-ocr-v1, a 3.4B
// MoE Document Parser With Built-In Speculative Decoding", ainewsfeed.tech:
// two shared experts beside 64 routed ones).
#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

namespace {

constexpr int kWaves = 4;   // wavefronts per block, 16 columns each
constexpr int kUnroll = 8;  // K-windows whose loads are issued together

struct TileInfo {
  int e, r0, m;
};

__device__ __forceinline__ bool find_tile(const ExpertArgs &p, int tile, TileInfo &ti) {
  const int ne = p.E + p.S;
  if (tile >= p.tile_start[ne]) return false;
  int e = 0;
  while (e + 1 < ne && p.tile_start[e + 1] <= tile) ++e;
  ti.e = e;
  ti.r0 = p.seg[e] + (tile - p.tile_start[e]) * kTileM;
  ti.m = min(kTileM, p.seg[e + 1] - ti.r0);
  return true;
}

// acc += A[16 x K] * B[K x 16] where lane l reads A row (l % 16) from `a`
// (LDS) and B column (l % 16) from `b` (global), both at K offset
// (l / 16) * VN inside each window of 4*VN elements.
template <typename T>
__device__ __forceinline__ void mfma_rowpanel(f32x4_t &acc, const T *a, const T *b, int nwin) {
  constexpr int W = 4 * Vec<T>::N;
  for (int w0 = 0; w0 < nwin; w0 += kUnroll) {
    uint4 bq[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (w0 + u < nwin) bq[u] = ld16(b + (w0 + u) * W);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (w0 + u < nwin) mfma16(acc, ld16(a + (w0 + u) * W), bq[u], T());
  }
}

template <typename T>
__device__ __forceinline__ void mfma_rowpanel2(f32x4_t &acc0, f32x4_t &acc1, const T *a,
                                               const T *b0, const T *b1, int nwin) {
  constexpr int W = 4 * Vec<T>::N;
  for (int w0 = 0; w0 < nwin; w0 += kUnroll) {
    uint4 q0[kUnroll], q1[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (w0 + u < nwin) {
        q0[u] = ld16(b0 + (w0 + u) * W);
        q1[u] = ld16(b1 + (w0 + u) * W);
      }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (w0 + u < nwin) {
        const uint4 av = ld16(a + (w0 + u) * W);
        mfma16(acc0, av, q0[u], T());
        mfma16(acc1, av, q1[u], T());
      }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_gate_up(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int VN = Vec<T>::N;
  TileInfo ti;
  if (!find_tile(p, blockIdx.y, ti)) return;
  const int d = p.d, F = p.F, nvec = d / VN, lda = d + VN;
  T *A = reinterpret_cast<T *>(smem);
  const T *x = static_cast<const T *>(p.x);
  for (int i = threadIdx.x; i < kTileM * nvec; i += blockDim.x) {
    const int r = i / nvec, c = i - r * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < ti.m) {
      const int tok = p.rows[ti.r0 + r] / p.nslot;
      v = ld16(x + static_cast<size_t>(tok) * d + c * VN);
    }
    st16(A + r * lda + c * VN, v);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int f0 = (blockIdx.x * kWaves + wv) * 16;
  if (f0 >= F) return;
  const size_t expert_elems = static_cast<size_t>(2) * F * d;
  const T *W = ti.e < p.E
                   ? static_cast<const T *>(p.w_routed) + static_cast<size_t>(ti.e) * expert_elems
                   : static_cast<const T *>(p.w_shared) + static_cast<size_t>(ti.e - p.E) * expert_elems;
  const int koff = (lane >> 4) * VN;
  const T *bg = W + static_cast<size_t>(f0 + (lane & 15)) * d + koff;
  const T *bu = bg + static_cast<size_t>(F) * d;
  const T *ar = A + (lane & 15) * lda + koff;

  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  mfma_rowpanel2<T>(accg, accu, ar, bg, bu, d / (4 * VN));

  T *aout = static_cast<T *>(p.a_out);
  const int col = f0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (lane >> 4) * 4 + i;
    if (r < ti.m) {
      const float g = accg[i], u = accu[i];
      aout[static_cast<size_t>(ti.r0 + r) * F + col] = from_f32<T>(g / (1.0f + expf(-g)) * u);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_down(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int VN = Vec<T>::N;
  TileInfo ti;
  if (!find_tile(p, blockIdx.y, ti)) return;
  const int d = p.d, F = p.F, nvec = F / VN, lda = F + VN;
  T *A = reinterpret_cast<T *>(smem);
  const T *a = static_cast<const T *>(p.a);
  for (int i = threadIdx.x; i < kTileM * nvec; i += blockDim.x) {
    const int r = i / nvec, c = i - r * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < ti.m) v = ld16(a + static_cast<size_t>(ti.r0 + r) * F + c * VN);
    st16(A + r * lda + c * VN, v);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * kWaves + wv) * 16;
  if (n0 >= d) return;
  const size_t expert_elems = static_cast<size_t>(d) * F;
  const T *W = ti.e < p.E
                   ? static_cast<const T *>(p.w_routed) + static_cast<size_t>(ti.e) * expert_elems
                   : static_cast<const T *>(p.w_shared) + static_cast<size_t>(ti.e - p.E) * expert_elems;
  const int koff = (lane >> 4) * VN;
  const T *b = W + static_cast<size_t>(n0 + (lane & 15)) * F + koff;
  const T *ar = A + (lane & 15) * lda + koff;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  mfma_rowpanel<T>(acc, ar, b, F / (4 * VN));

  const int col = n0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (lane >> 4) * 4 + i;
    if (r < ti.m) {
      const int pair = p.rows[ti.r0 + r];
      const int tok = pair / p.nslot, s = pair - tok * p.nslot;
      const float w = s < p.k ? p.gates[tok * p.k + s] : 1.0f;
      p.slots[static_cast<size_t>(pair) * d + col] = w * acc[i];
    }
  }
}

template <typename KernelT>
void allow_big_lds(KernelT kernel, size_t bytes) {
  if (bytes > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

}  // namespace

hipError_t launch_gate_up(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.F + 16 * kWaves - 1) / (16 * kWaves), max_tiles);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t smem = kTileM * (a.d + 16 / es) * es;
  if (dtype == 1) {
    allow_big_lds(k_gate_up<bf16_t>, smem);
    hipLaunchKernelGGL(k_gate_up<bf16_t>, grid, dim3(64 * kWaves), smem, s, a);
  } else {
    allow_big_lds(k_gate_up<float>, smem);
    hipLaunchKernelGGL(k_gate_up<float>, grid, dim3(64 * kWaves), smem, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_down(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.d + 16 * kWaves - 1) / (16 * kWaves), max_tiles);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t smem = kTileM * (a.F + 16 / es) * es;
  if (dtype == 1) {
    allow_big_lds(k_down<bf16_t>, smem);
    hipLaunchKernelGGL(k_down<bf16_t>, grid, dim3(64 * kWaves), smem, s, a);
  } else {
    allow_big_lds(k_down<float>, smem);
    hipLaunchKernelGGL(k_down<float>, grid, dim3(64 * kWaves), smem, s, a);
  }
  return hipGetLastError();
}

}  // namespace mv
