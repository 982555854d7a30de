// Grouped expert GEMMs for large batches, where the expert FFN is bound by
// the matrix cores rather than by weight streaming (bf16 only).
//
// An expert segment of the sorted pair list is cut into tiles of kGBM rows.
// A block computes a kGBM x kGBN output tile of one expert with eight
// wavefronts (a 4 x 2 grid of 64 x 128 bands, as 32x32 MFMA tiles; two
// wavefronts per SIMD): A rows and B rows are staged through LDS in K-steps of kGBK, with the global loads of the next
// kStages steps in flight in registers while the current step is multiplied
// (v_mfma_f32_32x32x16_bf16, which on gfx950 sustains nearly twice the rate
// of the 16x16x32 form; one MFMA chain per output element over K in order).
//
//   gate/up: B rows = 128 gate rows and the 128 matching up rows of
//            W_gate_up, a = round(SiLU(g) * u) in the epilogue (SwiGLU experts).
//   down:    B rows = 256 rows of W_down; slot[pair] = w_pair * y.
//
// Blocks are numbered so that the hardware's round-robin dispatch over the
// eight XCDs gives each XCD one contiguous run of the work list ordered by
// (expert, column block, row tile): the blocks running together on one XCD
// share an expert's weight columns and activation rows in that XCD's L2.
#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

namespace {

#ifndef MV_GEMM_BN
#define MV_GEMM_BN 256
#define MV_GEMM_BK 64
#define MV_GEMM_PAD 8
#endif
#ifndef MV_GEMM_WAVES_M
#define MV_GEMM_WAVES_M 4
#endif
constexpr int kGBM = 256;             // rows per tile
constexpr int kGBN = MV_GEMM_BN;      // B rows per block
constexpr int kGBK = MV_GEMM_BK;      // K per LDS stage
// LDS row stride in elements: 144 bytes, nine 16-byte units, so the eight
// rows one 16-byte read serves per cycle fall in distinct bank groups (the
// rows are read 32 lanes deep by the MFMA fragments)
constexpr int kGLd = kGBK + MV_GEMM_PAD;
constexpr int kGWavesM = MV_GEMM_WAVES_M;  // wavefront grid: kGWavesM x kGWavesN bands
constexpr int kGWavesN = kGBN / 128;
constexpr int kGWaveM = kGBM / kGWavesM;  // rows per wavefront
constexpr int kGMT = kGWaveM / 32;        // 32-row MFMA tiles per wavefront
constexpr int kGThreads = 64 * kGWavesM * kGWavesN;
constexpr int kGWaveN = kGBN / kGWavesN;  // B rows per wavefront
constexpr int kGChunks = kGBK / 8;    // 16-byte chunks per row and K-step
constexpr int kGroupTiles = 1;        // row tiles walked together per expert (1 beat 2, 3, 4 and 8)
constexpr int kXcds = 8;

struct GemmSmem {
  bf16_t a[2][kGBM * kGLd];
  bf16_t b[2][kGBN * kGLd];
};

// Work item of this block: the row tile and column block, or false.  Items
// of one expert are walked in groups of kGroupTiles row tiles, column block
// by column block, so the blocks in flight on an XCD share operands (with one
// row tile per group: a row tile's activations across its column blocks).
__device__ bool gemm_item(const int *tile_start, int ne, int nb_count, int &tile, int &nb) {
  const int total = tile_start[ne] * nb_count;
  const int q = (total + kXcds - 1) / kXcds;
  const int x = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
  if (i >= q) return false;
  const int item = x * q + i;
  if (item >= total) return false;
  int lo = 0, hi = ne - 1;  // last expert whose first item is <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] * nb_count <= item) lo = mid; else hi = mid - 1;
  }
  const int nt = tile_start[lo + 1] - tile_start[lo];
  const int j = item - tile_start[lo] * nb_count;
  const int g = j / (kGroupTiles * nb_count), w = j - g * kGroupTiles * nb_count;
  const int in_group = min(kGroupTiles, nt - g * kGroupTiles);
  nb = w / in_group;
  tile = tile_start[lo] + g * kGroupTiles + (w - nb * in_group);
  return true;
}

// Global -> registers -> LDS copy of a [ROWS x kGBK] tile, kGChunks threads
// per row; kStages steps are in flight in registers, one slot per step.
#ifndef MV_GEMM_STAGES
#define MV_GEMM_STAGES 2
#endif
constexpr int kStages = MV_GEMM_STAGES;

template <int ROWS>
struct Stager {
  static constexpr int PER = ROWS * kGChunks / kGThreads;
  const bf16_t *src[PER];
  const bf16_t *alt[PER];  // source of K >= split (two operands laid end to end)
  int split = 1 << 30;
  uint4 reg[kStages][PER];
  __device__ __forceinline__ static int row(int j) { return threadIdx.x / kGChunks + j * (kGThreads / kGChunks); }
  __device__ __forceinline__ static int col() { return (threadIdx.x % kGChunks) * 8; }
  __device__ __forceinline__ void load(int slot, int k0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) reg[slot][j] = ld16(k0 < split ? src[j] + k0 : alt[j] + (k0 - split));
  }
  __device__ __forceinline__ void store(int slot, bf16_t *lds) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) st16(lds + row(j) * kGLd + col(), reg[slot][j]);
  }
};

// Per wavefront: a kGWaveM x kGWaveN output band as kGMT x (kGWaveN / 32) tiles of 32x32.
typedef f32x16_t GemmAcc[kGMT][kGWaveN / 32];

// MFMAs of one K-step from LDS buffer `cur`; the fragments of the next
// 16-deep slice are read while the current one is multiplied.
__device__ __forceinline__ void gemm_step(const GemmSmem &sm, int cur, GemmAcc &acc) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv % kGWavesM, wn = wv / kGWavesM;
  const bf16_t *as = sm.a[cur] + (wm * kGWaveM + (lane & 31)) * kGLd + (lane >> 5) * 8;
  const bf16_t *bs = sm.b[cur] + (wn * kGWaveN + (lane & 31)) * kGLd + (lane >> 5) * 8;
  uint4 af[2][kGMT], bfr[2][kGWaveN / 32];
#pragma unroll
  for (int i = 0; i < kGMT; ++i) af[0][i] = ld16(as + i * 32 * kGLd);
#pragma unroll
  for (int j = 0; j < kGWaveN / 32; ++j) bfr[0][j] = ld16(bs + j * 32 * kGLd);
#pragma unroll
  for (int u = 0; u < kGBK / 16; ++u) {
    const int c = u & 1;
    if (u + 1 < kGBK / 16) {
#pragma unroll
      for (int i = 0; i < kGMT; ++i) af[c ^ 1][i] = ld16(as + i * 32 * kGLd + (u + 1) * 16);
#pragma unroll
      for (int j = 0; j < kGWaveN / 32; ++j) bfr[c ^ 1][j] = ld16(bs + j * 32 * kGLd + (u + 1) * 16);
    }
#pragma unroll
    for (int i = 0; i < kGMT; ++i)
#pragma unroll
      for (int j = 0; j < kGWaveN / 32; ++j) mfma32(acc[i][j], af[c][i], bfr[c][j]);
  }
}

// Row (within the block tile) of element q of this lane's tile i, and the
// B row of its column in tile j.
__device__ __forceinline__ int gemm_row(int i, int q) {
  const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) % kGWavesM;
  return wm * kGWaveM + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
}
__device__ __forceinline__ int gemm_col(int j) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) / kGWavesM;
  return wn * kGWaveN + j * 32 + (lane & 31);
}

// acc[i][j] += A band rows x B rows over K = nk * kGBK.  Step ks: its
// registers go to LDS buffer ks % 2, one block barrier, the loads of step
// ks + kStages reuse the freed registers, then the MFMAs of step ks.  Loads
// past the end re-read the last step, so every load is unconditional.  With
// NK (= nk) known at compile time the loop is fully unrolled, which lets the
// compiler's wait counts keep kStages steps in flight; NK = 0 is the rolled
// loop for other widths.
template <int NK>
__device__ __forceinline__ void gemm_mainloop(GemmSmem &sm, Stager<kGBM> &A, Stager<kGBN> &B, int nk,
                                              GemmAcc &acc) {
  if (NK > 0) nk = NK;
#pragma unroll
  for (int s = 0; s < kStages; ++s) {
    A.load(s, min(s, nk - 1) * kGBK);
    B.load(s, min(s, nk - 1) * kGBK);
  }
  if (NK > 0) {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int slot = ks % kStages, cur = ks & 1;
      A.store(slot, sm.a[cur]);
      B.store(slot, sm.b[cur]);
      __syncthreads();
      if (ks + kStages < NK) {
        A.load(slot, (ks + kStages) * kGBK);
        B.load(slot, (ks + kStages) * kGBK);
      }
      gemm_step(sm, cur, acc);
    }
    return;
  }
  for (int ks0 = 0; ks0 < nk; ks0 += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      const int ks = ks0 + s;
      const int cur = ks & 1;
      A.store(s, sm.a[cur]);
      B.store(s, sm.b[cur]);
      __syncthreads();
      A.load(s, min(ks + kStages, nk - 1) * kGBK);
      B.load(s, min(ks + kStages, nk - 1) * kGBK);
      if (ks < nk) gemm_step(sm, cur, acc);
    }
  }
}

__device__ __forceinline__ const bf16_t *expert_w(const ExpertArgs &p, int e, size_t elems) {
  return e < p.E ? static_cast<const bf16_t *>(p.w_routed) + static_cast<size_t>(e) * elems
                 : static_cast<const bf16_t *>(p.w_shared) + static_cast<size_t>(e - p.E) * elems;
}

template <int NK>
__global__ __launch_bounds__(kGThreads) void k_gemm_gate_up(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GemmSmem &sm = *reinterpret_cast<GemmSmem *>(smem_raw);
  const int ne = p.E + p.S, d = p.d, F = p.F;
  int tile, nb;
  if (!gemm_item(p.tile_start, ne, F / (kGBN / 2), tile, nb)) return;  // kGBN/2 columns of a
  const int4 tv = p.tile_info[tile];
  const int e = tv.x, r0 = tv.y, m = tv.z;
  const int n0 = nb * (kGBN / 2);
  const int c8 = Stager<kGBM>::col();
  Stager<kGBM> A;
  Stager<kGBN> B;
  const bf16_t *x = static_cast<const bf16_t *>(p.x);
#pragma unroll
  for (int j = 0; j < Stager<kGBM>::PER; ++j) {
    const int row = Stager<kGBM>::row(j);
    const int pair = p.rows[r0 + (row < m ? row : 0)];
    A.src[j] = x + static_cast<size_t>(pair / p.nslot) * d + c8;
  }
  const bf16_t *W = expert_w(p, e, static_cast<size_t>(2) * F * d);
#pragma unroll
  for (int j = 0; j < Stager<kGBN>::PER; ++j) {
    // B rows in runs of 64: gate columns c..c+63, then the matching up rows,
    // so each wavefront's band holds both halves of its 64 columns
    const int br = Stager<kGBN>::row(j), run = br / 64;
    const int c = (run / 2) * 64 + br % 64;
    const int wrow = run % 2 ? F + n0 + c : n0 + c;
    B.src[j] = W + static_cast<size_t>(wrow) * d + c8;
  }
  GemmAcc acc;
#pragma unroll
  for (int i = 0; i < kGMT; ++i)
#pragma unroll
    for (int j = 0; j < kGWaveN / 32; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  gemm_mainloop<NK>(sm, A, B, d / kGBK, acc);

  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) / kGWavesM;
  bf16_t *aout = static_cast<bf16_t *>(p.a_out);
#pragma unroll
  for (int i = 0; i < kGMT; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = gemm_row(i, q);
      if (row >= m) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // tiles 0, 1 gate; 2, 3 up
        // SiLU with the hardware exp2 and reciprocal (about 1 ulp each; the
        // product is rounded to bf16)
        const float gv = acc[i][j][q], uv = acc[i][j + 2][q];
        const float sg = gv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gv));
        aout[static_cast<size_t>(r0 + row) * F + n0 + wn * 64 + j * 32 + (lane & 31)] = f32_to_bf16(sg * uv);
      }
    }
}

// Routed experts only (the shared ones go through k_gemm_down_shared).
template <int NK>
__global__ __launch_bounds__(kGThreads) void k_gemm_down(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GemmSmem &sm = *reinterpret_cast<GemmSmem *>(smem_raw);
  const int ne = p.E, d = p.d, F = p.F;
  int tile, nb;
  if (!gemm_item(p.tile_start, ne, d / kGBN, tile, nb)) return;
  const int4 tv = p.tile_info[tile];
  const int e = tv.x, r0 = tv.y, m = tv.z;
  const int n0 = nb * kGBN;
  const int c8 = Stager<kGBM>::col();
  Stager<kGBM> A;
  Stager<kGBN> B;
  const bf16_t *a = static_cast<const bf16_t *>(p.a);
#pragma unroll
  for (int j = 0; j < Stager<kGBM>::PER; ++j) {
    const int row = Stager<kGBM>::row(j);
    A.src[j] = a + static_cast<size_t>(r0 + (row < m ? row : 0)) * F + c8;
  }
  const bf16_t *W = expert_w(p, e, static_cast<size_t>(d) * F);
#pragma unroll
  for (int j = 0; j < Stager<kGBN>::PER; ++j)
    B.src[j] = W + static_cast<size_t>(n0 + Stager<kGBN>::row(j)) * F + c8;
  GemmAcc acc;
#pragma unroll
  for (int i = 0; i < kGMT; ++i)
#pragma unroll
    for (int j = 0; j < kGWaveN / 32; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  gemm_mainloop<NK>(sm, A, B, F / kGBK, acc);

  // the pair ids and gates of kEpi row tiles of this lane are read before
  // their first store: loads and stores share one memory counter, so a gate
  // read between stores would wait for all of them to complete
  constexpr int kEpi = kGMT < 2 ? kGMT : 2;
#pragma unroll
  for (int i0 = 0; i0 < kGMT; i0 += kEpi) {
    int pr[kEpi][16];
    float gw[kEpi][16];
#pragma unroll
    for (int i = 0; i < kEpi; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) pr[i][q] = p.rows[r0 + min(gemm_row(i0 + i, q), m - 1)];
#pragma unroll
    for (int i = 0; i < kEpi; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int tok = pr[i][q] / p.nslot, s = pr[i][q] - tok * p.nslot;
        gw[i][q] = s < p.k ? p.gates[tok * p.k + s] : 1.0f;
      }
#pragma unroll
    for (int i = 0; i < kEpi; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = gemm_row(i0 + i, q);
        if (row >= m) continue;
        const int pair = pr[i][q];
        const float w = gw[i][q];
        float *dst = p.slots + static_cast<size_t>(pair) * d + n0;
#pragma unroll
        for (int j = 0; j < kGWaveN / 32; ++j) dst[gemm_col(j)] = w * acc[i0 + i][j][q];
      }
  }
}

// Shared experts' down projection over every token, with the combine in
// the epilogue: K runs over the S shared experts laid end to end (their a
// rows and W_down columns), y = ((slot_0 + ... + slot_{k-1}) + shared) in
// that order, h_dst = round(h_src + y).  Row tiles of kGBM tokens.  KT > 0
// fixes top_k at compile time (0: p.k, up to kMaxTopK).
template <int NK, int KT>
__global__ __launch_bounds__(kGThreads) void k_gemm_down_shared(ExpertArgs p, CombineArgs c) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GemmSmem &sm = *reinterpret_cast<GemmSmem *>(smem_raw);
  const int d = p.d, F = p.F, T = p.T;
  const int nb_count = d / kGBN, nmt = (T + kGBM - 1) / kGBM;
  const int total = nmt * nb_count, q = (total + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, i0 = blockIdx.x / kXcds;
  if (i0 >= q || xcd * q + i0 >= total) return;
  const int item = xcd * q + i0;
  const int g = item / (kGroupTiles * nb_count), w = item - g * kGroupTiles * nb_count;
  const int in_group = min(kGroupTiles, nmt - g * kGroupTiles);
  const int nb = w / in_group, mt = g * kGroupTiles + (w - nb * in_group);
  const int t0 = mt * kGBM, n0 = nb * kGBN;
  const int c8 = Stager<kGBM>::col();
  const int S = p.S;
  const bf16_t *a = static_cast<const bf16_t *>(p.a);
  const bf16_t *W = static_cast<const bf16_t *>(p.w_shared);
  const int seg0 = S > 0 ? p.seg[p.E] : 0, seg1 = S > 1 ? p.seg[p.E + 1] : 0;
  Stager<kGBM> A;
  Stager<kGBN> B;
  A.split = B.split = F;
#pragma unroll
  for (int j = 0; j < Stager<kGBM>::PER; ++j) {
    const int t = min(t0 + Stager<kGBM>::row(j), T - 1);
    A.src[j] = a + static_cast<size_t>(seg0 + t) * F + c8;
    A.alt[j] = a + static_cast<size_t>(seg1 + t) * F + c8;
  }
#pragma unroll
  for (int j = 0; j < Stager<kGBN>::PER; ++j) {
    const size_t r = static_cast<size_t>(n0 + Stager<kGBN>::row(j)) * F + c8;
    B.src[j] = W + r;
    B.alt[j] = W + static_cast<size_t>(d) * F + r;
  }
  GemmAcc acc;
#pragma unroll
  for (int i = 0; i < kGMT; ++i)
#pragma unroll
    for (int j = 0; j < kGWaveN / 32; ++j)
#pragma unroll
      for (int qq = 0; qq < 16; ++qq) acc[i][j][qq] = 0.f;
  if (S > 0) gemm_mainloop<NK>(sm, A, B, S * F / kGBK, acc);

  // Epilogue through LDS, in kGMT rounds: in round r every wavefront stages
  // its 32-row MFMA tile r (block rows wm*64 + r*32 .. +31; 128 rows in all),
  // then each wavefront takes whole staged rows, lane l columns 4l .. 4l+3,
  // so the slot and residual loads and the stores run along rows in 16- and
  // 8-byte pieces, kRowsInFlight rows per lane loaded before any is stored.
  constexpr int NJ = kGWaveN / 32;
  constexpr int kStLd = kGBN + 4;             // fp32 row stride of the staged rows
  constexpr int kStaged = kGWavesM * 32;      // rows staged per round
  constexpr int kWaves = kGThreads / kWave;
  constexpr int kRowsInFlight = KT > 0 ? 4 : 2;  // up to kMaxTopK slot loads per row otherwise
  constexpr int KS = KT > 0 ? KT : kMaxTopK;  // slot loads per row
  static_assert(kStaged * kStLd * 4 <= static_cast<int>(sizeof(GemmSmem)), "staged rows fit the LDS");
  static_assert(kGBN == 4 * kWave, "one lane per 4 columns");
  const int k = KT > 0 ? KT : p.k;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, wm = wv % kGWavesM;
  float *stage = reinterpret_cast<float *>(smem_raw);
  const bf16_t *hs = static_cast<const bf16_t *>(c.h_src);
  bf16_t *hd = static_cast<bf16_t *>(c.h_dst);
#pragma unroll
  for (int r = 0; r < kGMT; ++r) {
    __syncthreads();  // the K loop's last LDS reads, or the previous round's, are done
#pragma unroll
    for (int qq = 0; qq < 16; ++qq)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        stage[(wm * 32 + (qq >> 2) * 8 + (lane >> 5) * 4 + (qq & 3)) * kStLd + gemm_col(j)] = acc[r][j][qq];
    __syncthreads();
    for (int u0 = 0; u0 < kStaged / kWaves; u0 += kRowsInFlight) {
      float4 sv[kRowsInFlight][KS];
      uint2 hv[kRowsInFlight];
      int tr[kRowsInFlight];
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int sr = wv + (u0 + u) * kWaves;  // staged row: block row (sr/32)*64 + r*32 + sr%32
        tr[u] = t0 + (sr / 32) * kGWaveM + r * 32 + sr % 32;
        const size_t t = static_cast<size_t>(min(tr[u], T - 1));
        const float *sp = p.slots + t * p.nslot * d + n0 + lane * 4;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          sv[u][s] = *reinterpret_cast<const float4 *>(sp + static_cast<size_t>(min(s, k - 1)) * d);
        hv[u] = ld8(hs + t * d + n0 + lane * 4);
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        if (tr[u] >= T) continue;
        const int sr = wv + (u0 + u) * kWaves;
        const float4 sh = *reinterpret_cast<const float4 *>(stage + sr * kStLd + lane * 4);
        float y[4] = {0.f, 0.f, 0.f, 0.f}, hf[4], o[4];
#pragma unroll
        for (int s = 0; s < KS; ++s)
          if (s < k) {
            y[0] += sv[u][s].x; y[1] += sv[u][s].y; y[2] += sv[u][s].z; y[3] += sv[u][s].w;
          }
        y[0] += sh.x; y[1] += sh.y; y[2] += sh.z; y[3] += sh.w;
        unpack8(hv[u], hf, bf16_t());
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = round_to<bf16_t>(hf[e] + y[e]);
        const size_t off = static_cast<size_t>(tr[u]) * d + n0 + lane * 4;
        st8(hd + off, pack8(o, bf16_t()));
        if (c.y_moe) *reinterpret_cast<float4 *>(c.y_moe + off) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
  }
}

}  // namespace

int gemm_tile_rows() { return kGBM; }


template <typename KernelT>
hipError_t launch_gemm(KernelT kernel, int items, const ExpertArgs &a, hipStream_t s) {
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            sizeof(GemmSmem));
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kGThreads), sizeof(GemmSmem), s, a);
  return hipGetLastError();
}

// Unrolled K loops for the widths d = 1280 and F = 896.
constexpr int kNkD = 1280 / kGBK, kNkF = 896 / kGBK;

hipError_t launch_gemm_gate_up(const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const int items = max_tiles * (a.F / (kGBN / 2));
  return a.d == kNkD * kGBK ? launch_gemm(k_gemm_gate_up<kNkD>, items, a, s)
                            : launch_gemm(k_gemm_gate_up<0>, items, a, s);
}

hipError_t launch_gemm_down(const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const int items = max_tiles * (a.d / kGBN);
  return a.F == kNkF * kGBK ? launch_gemm(k_gemm_down<kNkF>, items, a, s)
                            : launch_gemm(k_gemm_down<0>, items, a, s);
}

hipError_t launch_gemm_down_shared(const ExpertArgs &a, const CombineArgs &c, hipStream_t s) {
  const int items = (a.T + kGBM - 1) / kGBM * (a.d / kGBN);
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  const bool unrolled = a.S == 2 && a.F == kNkF * kGBK && a.k == 6;
  const void *k = unrolled ? reinterpret_cast<const void *>(k_gemm_down_shared<2 * kNkF, 6>)
                           : reinterpret_cast<const void *>(k_gemm_down_shared<0, 0>);
  (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(GemmSmem));
  if (unrolled)
    hipLaunchKernelGGL((k_gemm_down_shared<2 * kNkF, 6>), dim3(grid), dim3(kGThreads), sizeof(GemmSmem), s, a, c);
  else
    hipLaunchKernelGGL((k_gemm_down_shared<0, 0>), dim3(grid), dim3(kGThreads), sizeof(GemmSmem), s, a, c);
  return hipGetLastError();
}

}  // namespace mv
