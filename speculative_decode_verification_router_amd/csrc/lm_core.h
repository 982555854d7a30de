// LM-head building block: one vocabulary block against up to 16 x_f rows.
#pragma once

#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

constexpr int kLmWaves = 4;
constexpr int kLmSlices = 4;   // 16-row vocabulary slices per wavefront
constexpr int kLmUnroll = 10;  // K-windows per weight batch; two batches in flight
constexpr int kLmRowsPerBlock = 16 * kLmSlices * kLmWaves;

// Vocabulary block `vblk` (kLmRowsPerBlock rows: kLmWaves wavefronts of
// kLmSlices 16-row slices) of the LM head against up to 16 x_f rows.  Each
// wavefront streams its slices' weight rows as one sequence of batches of
// kLmUnroll windows, the next batch requested before the current one is
// multiplied; begin() requests the first batch, so a kernel can issue it
// before it stages the x_f rows.  kGlobal: the weight loads go through a
// global-space pointer (gld16), for callers whose arguments come from device
// memory; elsewhere the compiler already knows the space, and the plain form
// schedules better.
template <typename T, bool kGlobal = false>
struct LmStream {
  static constexpr int VN = Vec<T>::N, WIN = 4 * VN;
  int vbase, nwin, bps, nb, koff;
  uint4 qa[kLmUnroll], qb[kLmUnroll];

  __device__ __forceinline__ const T *row(const LmArgs &p, int slice) const {
    const int v = min(vbase + slice * 16 + static_cast<int>(threadIdx.x & 15), p.V - 1);
    return static_cast<const T *>(p.w) + static_cast<size_t>(v) * p.d + koff;
  }
  // batch g: slice g / bps, windows from (g % bps) * kLmUnroll
  __device__ __forceinline__ void load(const LmArgs &p, uint4 *q, int g) const {
    const int slice = g / bps, w0 = (g - slice * bps) * kLmUnroll;
    const T *b = row(p, slice);
#pragma unroll
    for (int u = 0; u < kLmUnroll; ++u)
      if (w0 + u < nwin) q[u] = kGlobal ? gld16(b + (w0 + u) * WIN) : ld16(b + (w0 + u) * WIN);
  }
  __device__ __forceinline__ void begin(const LmArgs &p, int vblk, int tid) {
    const int lane = tid & 63, wv = tid >> 6;
    koff = (lane >> 4) * VN;
    nwin = p.d / WIN;
    bps = (nwin + kLmUnroll - 1) / kLmUnroll;
    nb = kLmSlices * bps;
    vbase = (vblk * kLmWaves + wv) * 16 * kLmSlices;
    load(p, qa, 0);
  }
  // MFMAs of batch g; after the last batch of a slice its logits are folded
  // into the running (value, ~id) maximum of each of this lane's rows
  __device__ __forceinline__ void step(const LmArgs &p, const uint4 *q, int g, const T *arow, f32x4_t &acc,
                                       uint64_t *best) const {
    const int slice = g / bps, w0 = (g - slice * bps) * kLmUnroll;
#pragma unroll
    for (int u = 0; u < kLmUnroll; ++u)
      if (w0 + u < nwin) mfma16(acc, ld16(arow + (w0 + u) * WIN), q[u], T());
    if (w0 + kLmUnroll >= nwin) {
      const int v = vbase + slice * 16 + static_cast<int>(threadIdx.x & 15);
      if (v < p.V) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t key = argmax_key(acc[i], static_cast<uint32_t>(v));
          best[i] = key > best[i] ? key : best[i];
        }
      }
      acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  // arow: this lane's x_f row in LDS (row (lane % 16), or a zero row past
  // the m rows), at its K offset.  Per row the best key of the block is
  // folded into argkey[rbase + row] with one atomicMax (one block barrier).
  __device__ void finish(const LmArgs &p, int rbase, int m, const T *arow, unsigned long long (*red)[kTileM],
                         int tid) {
    const int lane = tid & 63, wv = tid >> 6;
    uint64_t best[4] = {0ull, 0ull, 0ull, 0ull};
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < nb; g += 2) {
      if (g + 1 < nb) load(p, qb, g + 1);
      step(p, qa, g, arow, acc, best);
      if (g + 2 < nb) load(p, qa, g + 2);
      if (g + 1 < nb) step(p, qb, g + 1, arow, acc, best);
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
};

// Accept rule for sequence b: n = first j < K with drafts[j] != argmax[j]
// (else K); committed = argmax[0..n], -1 after; n_committed = n + 1.  With
// `coherent` the keys are read with agent-scope loads (keys folded by other
// blocks of the same launch).
__device__ inline void accept_sequence(const AcceptArgs &p, int b, bool coherent) {
  const int K = p.K, base = b * (K + 1);
  for (int j = 0; j <= K; ++j) {
    int g;
    if (p.argkey) {
      const unsigned long long key =
          coherent ? ld_agent(p.argkey + base + j)
                   : p.argkey[base + j];
      g = static_cast<int>(key_index(key));
    } else {
      g = p.argmax_in[base + j];
    }
    if (p.argmax_out) p.argmax_out[base + j] = g;
  }
  const int *g = p.argkey ? p.argmax_out : p.argmax_in;
  int n = 0;
  while (n < K && p.drafts[b * K + n] == g[base + n]) ++n;
  for (int j = 0; j <= K; ++j) p.committed[base + j] = j <= n ? g[base + j] : -1;
  p.n_acc[b] = n;
  p.n_com[b] = n + 1;
}

// After a block's atomicMax: wait for it to complete, count the block, and
// in the last of n_blocks blocks to finish run the accept rule over every
// sequence.  The key updates are device-scope atomics and the last block
// reads the keys with agent-scope loads, so no cache write-back is needed.
__device__ inline void lm_block_done(const LmArgs &p, unsigned n_blocks) {
  if (!p.done) return;
  __shared__ int last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    last = add_agent(p.done, 1u) == n_blocks - 1;
  __syncthreads();
  if (!last) return;
  for (int b = threadIdx.x; b < p.accept.B; b += blockDim.x) accept_sequence(p.accept, b, true);
}

}  // namespace mv
