// LM-head building block: one vocabulary block against up to 16 x_f rows.
#pragma once

#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

constexpr int kLmWaves = 4;
constexpr int kLmSlices = 4;   // 16-row vocabulary slices per wavefront
constexpr int kLmUnroll = 16;
constexpr int kLmRowsPerBlock = 16 * kLmSlices * kLmWaves;

// Vocabulary block `vblk` (kLmRowsPerBlock rows: kLmWaves wavefronts of
// kLmSlices 16-row slices) of the LM head against up to 16 x_f rows staged
// in LDS (A, row stride lda, rows >= m zero), by 256 threads with local
// index tid: per row the best (value, ~id) key of the block is folded into
// argkey[rbase + row] with one atomicMax (one block barrier inside).
template <typename T>
__device__ __forceinline__ void lm_rows_block(const LmArgs &p, int vblk, int rbase, int m, const T *A, int lda,
                                              unsigned long long (*red)[kTileM], int tid) {
  constexpr int VN = Vec<T>::N, WIN = 4 * VN;
  const int lane = tid & 63, wv = tid >> 6;
  const int koff = (lane >> 4) * VN;
  const T *ar = A + (lane & 15) * lda + koff;
  const int nwin = p.d / WIN;
  uint64_t best[4] = {0ull, 0ull, 0ull, 0ull};
  const int vbase = (vblk * kLmWaves + wv) * 16 * kLmSlices;
  for (int sl = 0; sl < kLmSlices; ++sl) {
    const int v0 = vbase + sl * 16;
    if (v0 >= p.V) break;
    const int v = v0 + (lane & 15);
    const T *b = static_cast<const T *>(p.w) + static_cast<size_t>(min(v, p.V - 1)) * p.d + koff;
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
  if (tid < m) {
    uint64_t k = 0ull;
#pragma unroll
    for (int w = 0; w < kLmWaves; ++w) k = red[w][tid] > k ? red[w][tid] : k;
    if (k != 0ull) atomicMax(p.argkey + rbase + tid, static_cast<unsigned long long>(k));
  }
}

}  // namespace mv
