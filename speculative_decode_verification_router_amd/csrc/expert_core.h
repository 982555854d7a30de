// Expert-tile building blocks: 256 threads (local index tid, four wavefronts)
// work on one tile of up to 16 rows of one expert's segment of the sorted
// pair list, streaming weight rows from HBM straight into MFMA B-operand
// registers with 16-byte loads, eight K-windows in flight per wavefront.
//
//   gate/up: a slice pair is two 16-column slices of F; per slice one
//            wavefront streams the gate rows and one the up rows over the
//            full K = d; a = round(SiLU(g) * u) after an LDS exchange.
//   down:    a slice pair is two 16-column slices of d; per slice two
//            wavefronts split K = F in halves, added in a fixed order through
//            LDS; slot[pair] = w_pair * y.
// w_pair is the softmax gate of the routed pair, or 1 for a shared expert
// (architecture paragraph of "Jina AI Releases jina-ocr-v1, a 3.4B MoE
// Document Parser With Built-In Speculative Decoding", ainewsfeed.tech: two
// shared experts beside 64 routed ones).
#pragma once

#include "route_core.h"

namespace mv {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kUnroll = 8;       // K-windows whose loads are issued together
constexpr int kUnrollFused = 20;  // the same in the fused small-batch launch (fewer, longer batches)

struct TileInfo {
  int e, r0, m;
  int j = 0;  // the tile's index among its expert's tiles
};

template <typename T>
__device__ __forceinline__ const T *expert_base(const void *w_routed, const void *w_shared, int E, int e,
                                               size_t elems) {
  return e < E ? static_cast<const T *>(w_routed) + static_cast<size_t>(e) * elems
               : static_cast<const T *>(w_shared) + static_cast<size_t>(e - E) * elems;
}
template <typename T>
__device__ __forceinline__ const T *expert_base(const ExpertArgs &p, int e, size_t elems) {
  return expert_base<T>(p.w_routed, p.w_shared, p.E, e, elems);
}

// Weight loads of windows [w0, min(w0 + U, w_hi)) into registers.
template <typename T, int U = kUnroll>
__device__ __forceinline__ void load_batch(uint4 *q, const T *b, int w0, int w_hi) {
  constexpr int W = 4 * Vec<T>::N;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (w0 + u < w_hi) q[u] = gld16(b + (w0 + u) * W);
}

// U MFMAs over windows [w0, min(w0 + U, w_hi)), branch-free for a full batch.
template <typename T, int U>
__device__ __forceinline__ void mfma_batch(f32x4_t &acc, const T *a, const uint4 *q, int w0, int w_hi) {
  constexpr int W = 4 * Vec<T>::N;
  if (w0 + U <= w_hi) {
#pragma unroll
    for (int u = 0; u < U; ++u) mfma16(acc, ld16(a + (w0 + u) * W), q[u], T());
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (w0 + u < w_hi) mfma16(acc, ld16(a + (w0 + u) * W), q[u], T());
  }
}

// acc += A[16 x K] * B[K x 16] over windows [w_lo, w_hi), the first batch of
// weights already in `q`: lane l reads A row (l % 16) from `a` (LDS) and B
// column (l % 16) from `b` (global), both at K offset (l / 16) * VN inside
// each window of 4*VN elements.
//
// Batches of up to kUnroll windows (w_lo and w_hi the same in every lane of
// the wavefront): each later batch lives in registers of its own iteration,
// so that no weight register is carried from one batch to the next (a
// carried batch is copied as a whole, which waits for all of its loads before
// the first MFMA), and a full batch is branch-free, each MFMA waiting for its
// own load only.  Longer batches (the fused small-batch launch) keep one wait
// per batch: there the per-window form needs more registers than three
// blocks per compute unit leave, and measured slower.
template <typename T, int U = kUnroll>
__device__ __forceinline__ void mfma_panel(f32x4_t &acc, const T *a, const T *b, int w_lo, int w_hi,
                                           uint4 *q) {
  constexpr int W = 4 * Vec<T>::N;
  if constexpr (U > kUnroll) {
    for (int w0 = w_lo; w0 < w_hi; w0 += U) {
      if (w0 != w_lo) load_batch<T, U>(q, b, w0, w_hi);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (w0 + u < w_hi) mfma16(acc, ld16(a + (w0 + u) * W), q[u], T());
    }
    return;
  }
  if (w_lo >= w_hi) return;
  mfma_batch<T, U>(acc, a, q, w_lo, w_hi);
  for (int w0 = w_lo + U; w0 < w_hi; w0 += U) {
    uint4 r[U];
    if (w0 + U <= w_hi) {  // a full batch: loads and MFMAs in one branch-free block
#pragma unroll
      for (int u = 0; u < U; ++u) r[u] = gld16(b + (w0 + u) * W);
      __builtin_amdgcn_sched_barrier(0);  // every load of the batch in flight before the first MFMA
#pragma unroll
      for (int u = 0; u < U; ++u) mfma16(acc, ld16(a + (w0 + u) * W), r[u], T());
    } else {
      load_batch<T, U>(r, b, w0, w_hi);
      mfma_batch<T, U>(acc, a, r, w0, w_hi);
    }
  }
}

// The same MFMAs in the same order with two weight batches in flight: batch
// i + 1 is requested before the MFMAs of batch i (q0 holds the first batch).
template <typename T, int U>
__device__ __forceinline__ void mfma_panel2(f32x4_t &acc, const T *a, const T *b, int w_lo, int w_hi,
                                            uint4 *q0, uint4 *q1) {
  auto mma = [&](const uint4 *q, int w0) { mfma_batch<T, U>(acc, a, q, w0, w_hi); };
  for (int w0 = w_lo; w0 < w_hi; w0 += 2 * U) {
    if (w0 + U < w_hi) load_batch<T, U>(q1, b, w0 + U, w_hi);
    mma(q0, w0);
    if (w0 + U < w_hi) {
      if (w0 + 2 * U < w_hi) load_batch<T, U>(q0, b, w0 + 2 * U, w_hi);
      mma(q1, w0 + U);
    }
  }
}

// The tile's a rows (zero-filled past m) into LDS, row stride F + one vector.
// kCoherent: a was written by other blocks of the same launch (write-through
// stores), so it is read with agent-scope loads, which no stale cache line
// can answer.
template <typename T, bool kCoherent = false>
__device__ __forceinline__ void stage_a_tile(const ExpertArgs &p, const TileInfo &ti, T *A, int tid, int nthreads) {
  constexpr int VN = Vec<T>::N;
  const int F = p.F, nvec = F / VN, lda = F + VN;
  const T *a = static_cast<const T *>(p.a);
  for (int it = tid; it < kTileM * nvec; it += nthreads) {
    const int rr = it / nvec, c = it - rr * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < ti.m) {
      const T *src = a + static_cast<size_t>(ti.r0 + rr) * F + c * VN;
      if constexpr (kCoherent) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(src);
        v.x = ld_agent(q);
        v.y = ld_agent(q + 1);
        v.z = ld_agent(q + 2);
        v.w = ld_agent(q + 3);
      } else {
        v = ld16(src);
      }
    }
    st16(A + rr * lda + c * VN, v);
  }
}

// Write-through store of one value per lane, the lanes of a pair holding
// adjacent columns (bf16: the even lane stores both as one 32-bit word; both
// lanes of the pair must call this).
__device__ __forceinline__ void store_through(float *p, float v, int) {
  st_agent(p, v);
}
__device__ __forceinline__ void store_through(bf16_t *p, float v, int lane) {
  const uint32_t mine = f32_to_bf16(v), other = __shfl_xor(mine, 1);
  if (!(lane & 1))
    st_agent(reinterpret_cast<uint32_t *>(p), mine | (other << 16));
}

// gate/up of slice pair `pair` of a tile.  begin() issues the first weight
// batch; finish() runs the MFMAs with this lane's A row at `arow` (LDS),
// exchanges the up accumulators and writes a (one block barrier inside).
// DB: two weight batches in flight (U more registers).
// ks / ns (begin): this block takes part ks of ns equal parts of the K
// windows, for partial gate and up outputs (finish_partial) that the reader
// adds up before the SiLU.
template <typename T, int U = kUnroll, bool DB = false>
struct GateUpPart {
  const T *b;
  int f0, which, slice, w_lo, w_hi;
  uint4 q[U];
  uint4 q2[DB ? U : 1];  // second weight buffer (DB: two batches in flight)
  __device__ __forceinline__ void begin(const ExpertArgs &p, const TileInfo &ti, int pair, int tid, int ks = 0,
                                        int ns = 1) {
    constexpr int VN = Vec<T>::N;
    const int lane = tid & 63, wv = tid >> 6;
    slice = wv >> 1;
    which = wv & 1;  // 0 gate rows, 1 up rows
    f0 = (pair * 2 + slice) * 16;
    const int d = p.d, F = p.F, r = lane & 15, koff = (lane >> 4) * VN;
    const int nwin = d / (4 * VN);
    w_lo = f0 < F ? ks * nwin / ns : 0;
    w_hi = f0 < F ? (ks + 1) * nwin / ns : 0;
    if constexpr (U <= kUnroll) {  // the same in every lane: scalar branches in the stream
      w_lo = __builtin_amdgcn_readfirstlane(w_lo);
      w_hi = __builtin_amdgcn_readfirstlane(w_hi);
    }
    const T *W = expert_base<T>(p, ti.e, static_cast<size_t>(2) * F * d);
    b = W + static_cast<size_t>(which * F + min(f0, F - 16) + r) * d + koff;
    load_batch<T, U>(q, b, w_lo, w_hi);
  }
  // The raw gate (which = 0) or up (which = 1) accumulators of rows [0, m):
  // out[row * 2F + which * F + f0 + column] for tile row `row` (ti.r0 + row
  // of the batch), out already offset to this block's K part.
  __device__ __forceinline__ void finish_partial(const ExpertArgs &p, const TileInfo &ti, const T *arow, float *out,
                                                 int tid) {
    const int lane = tid & 63, F = p.F;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    mfma_panel<T, U>(acc, arow, b, w_lo, w_hi, q);
    if (f0 >= F) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < ti.m) out[static_cast<size_t>(ti.r0 + row) * 2 * F + which * F + f0 + (lane & 15)] = acc[i];
    }
  }
  // kThrough: a is written with write-through stores (read by other blocks
  // of the same launch).
  template <bool kThrough = false>
  __device__ __forceinline__ void finish(const ExpertArgs &p, const TileInfo &ti, const T *arow,
                                         float (*up_acc)[64][4], int tid) {
    const int lane = tid & 63, F = p.F;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DB) mfma_panel2<T, U>(acc, arow, b, w_lo, w_hi, q, q2);
    else mfma_panel<T, U>(acc, arow, b, w_lo, w_hi, q);
    if (which == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) up_acc[slice][lane][i] = acc[i];
    }
    __syncthreads();
    if (which == 1 || f0 >= F) return;
    T *aout = static_cast<T *>(p.a_out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < ti.m) {
        const float gv = acc[i], uv = up_acc[slice][lane][i];
        const float v = gv / (1.0f + expf(-gv)) * uv;
        T *dst = aout + static_cast<size_t>(ti.r0 + row) * F + f0 + (lane & 15);
        if constexpr (kThrough) store_through(dst, v, lane);
        else *dst = from_f32<T>(v);
      }
    }
  }
};

// down of slice pair `pair` of a tile; same split as GateUpPart.  The down
// weights are p.w_routed / p.w_shared unless given.  ks / ns: this block
// takes part ks of ns equal parts of the K windows (its two halves split
// that part), for a partial output that the reader adds up.
template <typename T, int U = kUnroll>
struct DownPart {
  const T *b;
  int n0, half, slice, w_lo, w_hi;
  uint4 q[U];
  __device__ __forceinline__ void begin(const ExpertArgs &p, const TileInfo &ti, int pair, int tid,
                                        const void *w_routed = nullptr, const void *w_shared = nullptr,
                                        int ks = 0, int ns = 1) {
    constexpr int VN = Vec<T>::N;
    const int lane = tid & 63, wv = tid >> 6;
    slice = wv >> 1;
    half = wv & 1;
    n0 = (pair * 2 + slice) * 16;
    const int d = p.d, F = p.F, r = lane & 15, koff = (lane >> 4) * VN;
    const int nwin = F / (4 * VN), k0 = ks * nwin / ns, k1 = (ks + 1) * nwin / ns;
    w_lo = n0 < d ? k0 + half * (k1 - k0) / 2 : 0;
    w_hi = n0 < d ? k0 + (half + 1) * (k1 - k0) / 2 : 0;
    if constexpr (U <= kUnroll) {  // the same in every lane: scalar branches in the stream
      w_lo = __builtin_amdgcn_readfirstlane(w_lo);
      w_hi = __builtin_amdgcn_readfirstlane(w_hi);
    }
    const T *W = w_routed ? expert_base<T>(w_routed, w_shared, p.E, ti.e, static_cast<size_t>(d) * F)
                          : expert_base<T>(p, ti.e, static_cast<size_t>(d) * F);
    b = W + static_cast<size_t>(min(n0, d - 16) + r) * F + koff;
    load_batch<T, U>(q, b, w_lo, w_hi);
  }
  // tile_rows[row]: the pair id (t*nslot + slot) of tile row `row`; gates:
  // [T, k] softmax gates of the routed pairs.  kThrough: the slots are
  // written through (read by later blocks of the same launch).  out_off:
  // offset (floats) of this block's output from p.slots.
  template <bool kThrough = false>
  __device__ __forceinline__ void finish(const ExpertArgs &p, const TileInfo &ti, const T *arow,
                                         float (*half_acc)[64][4], int tid, const int *tile_rows,
                                         const float *gates, size_t out_off = 0) {
    const int lane = tid & 63, d = p.d;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    mfma_panel<T, U>(acc, arow, b, w_lo, w_hi, q);
    if (half == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) half_acc[slice][lane][i] = acc[i];
    }
    __syncthreads();
    if (half == 1 || n0 >= d) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < ti.m) {
        const int pair = tile_rows[row];
        const int tok = pair / p.nslot, s = pair - tok * p.nslot;
        const float w = s < p.k ? gates[tok * p.k + s] : 1.0f;
        float *dst = p.slots + out_off + static_cast<size_t>(pair) * d + n0 + (lane & 15);
        const float v = w * (acc[i] + half_acc[slice][lane][i]);
        if constexpr (kThrough) st_agent(dst, v);
        else *dst = v;
      }
    }
  }
};

}  // namespace mv
