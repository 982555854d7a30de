// LM head with a fused greedy argmax, and the speculative accept rule.
//
// The verify step needs only the decoder's own greedy choice at every
// position (FastMTP paragraph of "Jina AI Releases jina-ocr-v1, a 3.4B MoE
// Document Parser With Built-In Speculative Decoding", ainewsfeed.tech), so
// the logits z = x_f W_lm^T are reduced on the fly and never stored.  Each
// wavefront streams 16 vocabulary rows per slice into MFMA operands, keeps a
// running (value, id) maximum per token packed into a 64-bit key that orders
// by value and then by lower id, and one 64-bit atomicMax per token and block
// folds the blocks together; the result does not depend on block order.
#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

namespace {

constexpr int kLmWaves = 4;
constexpr int kLmSlices = 4;   // 16-row vocabulary slices per wavefront
constexpr int kLmUnroll = 8;

template <typename T>
__global__ __launch_bounds__(256) void k_lm_argmax(LmArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int VN = Vec<T>::N, WIN = 4 * VN;
  const int r0 = blockIdx.y * kTileM;
  const int m = min(kTileM, p.T - r0);
  const int d = p.d, nvec = d / VN, lda = d + VN;
  T *A = reinterpret_cast<T *>(smem);
  __shared__ unsigned long long red[kLmWaves][kTileM];

  const T *xf = static_cast<const T *>(p.xf);
  for (int i = threadIdx.x; i < kTileM * nvec; i += blockDim.x) {
    const int r = i / nvec, c = i - r * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < m) v = ld16(xf + static_cast<size_t>(r0 + r) * d + c * VN);
    st16(A + r * lda + c * VN, v);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int koff = (lane >> 4) * VN;
  const T *ar = A + (lane & 15) * lda + koff;
  const int nwin = d / WIN;
  uint64_t best[4] = {0ull, 0ull, 0ull, 0ull};
  const int vbase = (blockIdx.x * kLmWaves + wv) * 16 * kLmSlices;
  for (int sl = 0; sl < kLmSlices; ++sl) {
    const int v0 = vbase + sl * 16;
    if (v0 >= p.V) break;
    const int v = v0 + (lane & 15);
    const T *b = static_cast<const T *>(p.w) + static_cast<size_t>(min(v, p.V - 1)) * d + koff;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int w0 = 0; w0 < nwin; w0 += kLmUnroll) {
      uint4 q[kLmUnroll];
#pragma unroll
      for (int u = 0; u < kLmUnroll; ++u)
        if (w0 + u < nwin) q[u] = ld16(b + (w0 + u) * WIN);
#pragma unroll
      for (int u = 0; u < kLmUnroll; ++u)
        if (w0 + u < nwin) mfma16(acc, ld16(ar + (w0 + u) * WIN), q[u], T());
    }
    if (v < p.V) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t key = argmax_key(acc[i], static_cast<uint32_t>(v));
        best[i] = key > best[i] ? key : best[i];
      }
    }
  }
  // maximum over the 16 lanes that share rows 4*(lane/16)..+3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint64_t other = shfl_xor_u64(best[i], o);
      best[i] = other > best[i] ? other : best[i];
    }
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][(lane >> 4) * 4 + i] = best[i];
  }
  __syncthreads();
  if (threadIdx.x < m) {
    uint64_t k = 0ull;
#pragma unroll
    for (int w = 0; w < kLmWaves; ++w) k = red[w][threadIdx.x] > k ? red[w][threadIdx.x] : k;
    if (k != 0ull) atomicMax(p.argkey + r0 + threadIdx.x, static_cast<unsigned long long>(k));
  }
}

// One thread per sequence.  n = first j < K with drafts[j] != argmax[j]
// (else K); committed = argmax[0..n], -1 after; n_committed = n + 1.
__global__ __launch_bounds__(256) void k_accept(AcceptArgs p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.B) return;
  const int K = p.K, base = b * (K + 1);
  for (int j = 0; j <= K; ++j) {
    const int g = p.argkey ? static_cast<int>(key_index(p.argkey[base + j])) : p.argmax_in[base + j];
    if (p.argmax_out) p.argmax_out[base + j] = g;
  }
  const int *g = p.argkey ? p.argmax_out : p.argmax_in;
  int n = 0;
  while (n < K && p.drafts[b * K + n] == g[base + n]) ++n;
  for (int j = 0; j <= K; ++j) p.committed[base + j] = j <= n ? g[base + j] : -1;
  p.n_acc[b] = n;
  p.n_com[b] = n + 1;
}

}  // namespace

hipError_t launch_lm_argmax(int dtype, const LmArgs &a, hipStream_t s) {
  const int rows_per_block = 16 * kLmSlices * kLmWaves;
  const dim3 grid((a.V + rows_per_block - 1) / rows_per_block, (a.T + kTileM - 1) / kTileM);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t smem = kTileM * (a.d + 16 / es) * es;
  if (smem > 65536) {
    const void *k = dtype == 1 ? reinterpret_cast<const void *>(k_lm_argmax<bf16_t>)
                               : reinterpret_cast<const void *>(k_lm_argmax<float>);
    (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  }
  if (dtype == 1)
    hipLaunchKernelGGL(k_lm_argmax<bf16_t>, grid, dim3(64 * kLmWaves), smem, s, a);
  else
    hipLaunchKernelGGL(k_lm_argmax<float>, grid, dim3(64 * kLmWaves), smem, s, a);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_accept, dim3((a.B + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mv
