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
#include "lm_core.h"

namespace mv {

namespace {

}  // namespace

namespace {

template <typename T>
__global__ __launch_bounds__(256) void k_lm_argmax(LmArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int VN = Vec<T>::N;
  const int r0 = blockIdx.y * kTileM;
  const int m = min(kTileM, p.T - r0);
  const int d = p.d, nvec = d / VN, lda = d + VN;
  T *A = reinterpret_cast<T *>(smem);  // rows [0, m) of x_f, then a zero row
  __shared__ unsigned long long red[kLmWaves][kTileM];

  LmStream<T> ls;
  ls.begin(p, blockIdx.x, threadIdx.x);  // weights requested before x_f is staged
  const T *xf = static_cast<const T *>(p.xf);
  for (int i = threadIdx.x; i < (m + 1) * nvec; i += blockDim.x) {
    const int r = i / nvec, c = i - r * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < m) v = ld16(xf + static_cast<size_t>(r0 + r) * d + c * VN);
    st16(A + r * lda + c * VN, v);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int arow = (lane & 15) < m ? (lane & 15) : m;
  ls.finish(p, r0, m, A + arow * lda + (lane >> 4) * VN, red, threadIdx.x);
  lm_block_done(p, gridDim.x * gridDim.y);
}

// Up to 128 rows: every block takes all rows of its 16*MT-row group, so the
// LM head is streamed once per group instead of once per 16 rows.  x_f is
// staged through LDS in K-slabs of four windows, double-buffered: the next
// slab's rows and weights are loaded while the current one is multiplied.
// Eight wavefronts of two 16-row vocabulary slices each; per (row, vocab id)
// the arithmetic is the 16-row kernel's (one MFMA chain over K in order).
constexpr int kLmMidWaves = 8;
constexpr int kLmMidSlices = 2;
constexpr int kLmSlabWin = 4;

template <typename T, int MT>
__global__ __launch_bounds__(64 * kLmMidWaves) void k_lm_argmax_mid(LmArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int VN = Vec<T>::N, WIN = 4 * VN, KS = kLmSlabWin * WIN, LDA = KS + VN;
  constexpr int ROWS = 16 * MT, CPR = KS / VN;  // 16-byte chunks per row and slab
  constexpr int NT = 64 * kLmMidWaves;
  constexpr int PER = (ROWS * CPR + NT - 1) / NT;
  __shared__ unsigned long long red[kLmMidWaves][ROWS];
  T *A = reinterpret_cast<T *>(smem);  // [2][ROWS][LDA]
  const int rbase = blockIdx.y * ROWS;
  const int m = min(ROWS, p.T - rbase);
  const int d = p.d, nslab = d / KS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, koff = (lane >> 4) * VN;
  const T *xf = static_cast<const T *>(p.xf);

  uint4 st[PER];
  auto load_slab = [&](int s) {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int it = threadIdx.x + c * NT, row = it / CPR, ch = it - row * CPR;
      st[c] = make_uint4(0, 0, 0, 0);
      if (it < ROWS * CPR && row < m) st[c] = ld16(xf + static_cast<size_t>(rbase + row) * d + s * KS + ch * VN);
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int it = threadIdx.x + c * NT, row = it / CPR, ch = it - row * CPR;
      if (it < ROWS * CPR) st16(A + (buf * ROWS + row) * LDA + ch * VN, st[c]);
    }
  };

  const int vbase = (blockIdx.x * kLmMidWaves + wv) * 16 * kLmMidSlices;
  const T *b[kLmMidSlices];
#pragma unroll
  for (int j = 0; j < kLmMidSlices; ++j)
    b[j] = static_cast<const T *>(p.w) + static_cast<size_t>(min(vbase + j * 16 + r, p.V - 1)) * d + koff;
  uint4 q[kLmMidSlices][kLmSlabWin], qn[kLmMidSlices][kLmSlabWin];
  auto load_w = [&](uint4 (&dst)[kLmMidSlices][kLmSlabWin], int s) {
#pragma unroll
    for (int j = 0; j < kLmMidSlices; ++j)
#pragma unroll
      for (int u = 0; u < kLmSlabWin; ++u) dst[j][u] = ld16(b[j] + s * KS + u * WIN);
  };

  f32x4_t acc[MT][kLmMidSlices];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < kLmMidSlices; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_w(q, 0);
  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int s = 0; s < nslab; ++s) {
    const bool more = s + 1 < nslab;
    if (more) {
      load_w(qn, s + 1);
      load_slab(s + 1);
    }
    const T *As = A + (s & 1) * ROWS * LDA + r * LDA + koff;
#pragma unroll
    for (int u = 0; u < kLmSlabWin; ++u) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const uint4 a = ld16(As + i * 16 * LDA + u * WIN);
#pragma unroll
        for (int j = 0; j < kLmMidSlices; ++j) mfma16(acc[i][j], a, q[j][u], T());
      }
    }
    if (more) store_slab((s + 1) & 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int j = 0; j < kLmMidSlices; ++j)
#pragma unroll
        for (int u = 0; u < kLmSlabWin; ++u) q[j][u] = qn[j][u];
    }
  }

  // per row: best key over this wavefront's columns, then over the 16 lanes
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint64_t best = 0ull;
#pragma unroll
      for (int j = 0; j < kLmMidSlices; ++j) {
        const int v = vbase + j * 16 + r;
        if (v < p.V) {
          const uint64_t key = argmax_key(acc[i][j][jj], static_cast<uint32_t>(v));
          best = key > best ? key : best;
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const uint64_t other = shfl_xor_u64(best, o);
        best = other > best ? other : best;
      }
      if (r == 0) red[wv][i * 16 + (lane >> 4) * 4 + jj] = best;
    }
  }
  __syncthreads();
  for (int row = threadIdx.x; row < m; row += NT) {
    uint64_t k = 0ull;
#pragma unroll
    for (int w = 0; w < kLmMidWaves; ++w) k = red[w][row] > k ? red[w][row] : k;
    if (k != 0ull) atomicMax(p.argkey + rbase + row, static_cast<unsigned long long>(k));
  }
  lm_block_done(p, gridDim.x * gridDim.y);
}

// One thread per sequence.
__global__ __launch_bounds__(256) void k_accept(AcceptArgs p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < p.B) accept_sequence(p, b, false);
}

}  // namespace

template <typename T, int MT>
hipError_t launch_lm_mid(const LmArgs &a, hipStream_t s) {
  constexpr int VN = Vec<T>::N, KS = kLmSlabWin * 4 * VN;
  const size_t smem = 2 * static_cast<size_t>(16 * MT) * (KS + VN) * sizeof(T);
  const int rows_per_block = 16 * kLmMidSlices * kLmMidWaves;
  const dim3 grid((a.V + rows_per_block - 1) / rows_per_block, (a.T + 16 * MT - 1) / (16 * MT));
  if (smem > 48 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k_lm_argmax_mid<T, MT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  hipLaunchKernelGGL((k_lm_argmax_mid<T, MT>), grid, dim3(64 * kLmMidWaves), smem, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_lm_rows(const LmArgs &a, hipStream_t s) {
  if (a.T <= 32) return launch_lm_mid<T, 2>(a, s);
  if (a.T <= 64) return launch_lm_mid<T, 4>(a, s);
  return launch_lm_mid<T, 8>(a, s);
}

hipError_t launch_lm_argmax(int dtype, const LmArgs &a, hipStream_t s) {
  const int es = dtype == 1 ? 2 : 4;
  // K-slabs of four 16-byte windows per lane group need d to be a multiple of them
  const bool slabs = a.d % (kLmSlabWin * 4 * (16 / es)) == 0;
  if (a.T > kTileM && slabs) return dtype == 1 ? launch_lm_rows<bf16_t>(a, s) : launch_lm_rows<float>(a, s);
  const int rows_per_block = 16 * kLmSlices * kLmWaves;
  const dim3 grid((a.V + rows_per_block - 1) / rows_per_block, (a.T + kTileM - 1) / kTileM);
  const size_t rows = (a.T < kTileM ? a.T : kTileM) + 1;  // the largest tile's rows and a zero row
  const size_t smem = rows * (a.d + 16 / es) * es;
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
