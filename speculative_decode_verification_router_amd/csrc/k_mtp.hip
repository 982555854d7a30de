// Kernels of the FastMTP draft block: one dense block whose parameters are
// shared by every draft position, fed by the decoder's last hidden state and
// the token that follows it, drafting through the decoder's own LM head
// (FastMTP paragraph of "Jina AI Releases jina-ocr-v1, a 3.4B MoE Document
// Parser With Built-In Speculative Decoding", ainewsfeed.tech).  One draft
// position is five launches:
//
//   k_mtp_proj    z = u W_proj^T on 16-row tiles; each block builds the tile's
//                 u = [R(RMSNorm(h) * g_h) ; R(RMSNorm(E[t]) * g_e)] in LDS
//                 itself (t: the input token, or the previous draft read from
//                 the LM head's argmax key), and block (0, 0) records the
//                 previous draft and clears the key buffer this position's
//                 LM head will fold into
//   k_mtp_ffn_gu  g = x Wg^T, u = x Wu^T, x = R(RMSNorm(R(z)) * g_ffn) built
//                 in LDS by each block
//   k_mtp_ffn_dn  y = a W_down^T, a = R(SiLU(g) * u) formed while staged
//   k_mtp_out     h2 = R(R(z) + y) (the next position's h), x_o = R(RMSNorm(h2) * g_out)
//   (LM head)     the verify step's k_lm_argmax on x_o
//
// Up to kMtpFoldMaxB sequences the output kernel's work runs in the LM
// head's blocks (k_mtp_lm), so a position is four launches.
//
// and k_mtp_last reads the last draft.  Above kMtpFusedMaxB sequences the
// norms run in row kernels instead (k_mtp_in, k_mtp_mid; see below).  The
// argmax keys alternate between two buffers by position parity, so a
// projection reads the previous position's keys while its block (0, 0)
// clears the other buffer.  The weight streams are the expert-tile parts of
// expert_core.h with kUnrollFused windows per batch.  The projection, the
// FFN down and (up to kMtpFusedMaxB sequences) the FFN gate/up split K into
// kMtpSplit parts, one block each (their grids are small otherwise), and
// write fp32 partials that their readers add in part order: the FFN's norm
// (z), the FFN down while it forms a = R(SiLU(g) * u) (g, u), the output
// kernel (z, y).  Above kMtpFusedMaxB sequences the gate/up writes a itself:
// there the down blocks of two or more 16-row tiles would each form a whole
// tile's a from the partials.
// A row's sum of squares is taken per 16-byte chunk in order, then over the
// chunks as in the verify step's RMSNorm.
#include "expert_core.h"
#include "lm_core.h"

namespace mv {

namespace {

constexpr int kRowThreads = 256;
constexpr int kDenseU = kUnrollFused;

// Chunks each thread loads before it uses any of them.
constexpr int kChunksInFlight = 8;
// Up to this many chunks per thread a tile's rows are read once, kept in
// registers between their norm and its use.
constexpr int kOnePassChunks = 8;

// 1/rms of rows [0, m) of a tile, rows given by val(row, chunk, out[VN]),
// into inv[row]; part: LDS of m * d / VN floats.  Synchronises the block.
template <int VN, typename F>
__device__ __forceinline__ void tile_inv_rms(int m, int d, float eps, float *part, float *inv, F val) {
  const int nvec = d / VN, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int it0 = tid; it0 < m * nvec; it0 += kChunksInFlight * blockDim.x) {
    float v[kChunksInFlight][VN];
#pragma unroll
    for (int u = 0; u < kChunksInFlight; ++u) {
      const int it = it0 + u * static_cast<int>(blockDim.x), r = it / nvec;
      if (it < m * nvec) val(r, it - r * nvec, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kChunksInFlight; ++u) {
      const int it = it0 + u * static_cast<int>(blockDim.x);
      float s = v[u][0] * v[u][0];
#pragma unroll
      for (int i = 1; i < VN; ++i) s = __builtin_fmaf(v[u][i], v[u][i], s);
      if (it < m * nvec) part[it] = s;
    }
  }
  __syncthreads();
  for (int r = w; r < m; r += blockDim.x / kWave) {
    float acc = 0.f;
    for (int ch = lane; ch < nvec; ch += kWave) acc += part[r * nvec + ch];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) inv[r] = 1.0f / sqrtf(acc / static_cast<float>(d) + eps);
  }
  __syncthreads();
}

// tile_inv_rms's sums and reduction for rows [0, m) whose chunks a thread
// holds in registers: chunk it = threadIdx.x + u * kRowThreads in v[u]
// (it < n = m * nvec).  Synchronises the block.
template <int VN>
__device__ __forceinline__ void one_pass_inv(int m, int nvec, int d, float eps, float *part, float *inv,
                                             const float (*v)[VN], int n) {
  const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
  for (int u = 0; u < kOnePassChunks; ++u) {
    const int it = tid + u * kRowThreads;
    float s = v[u][0] * v[u][0];
#pragma unroll
    for (int i = 1; i < VN; ++i) s = __builtin_fmaf(v[u][i], v[u][i], s);
    if (it < n) part[it] = s;
  }
  __syncthreads();
  for (int r = tid >> 6; r < m; r += kRowThreads / kWave) {
    float acc = 0.f;
    for (int ch = lane; ch < nvec; ch += kWave) acc += part[r * nvec + ch];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) inv[r] = 1.0f / sqrtf(acc / static_cast<float>(d) + eps);
  }
  __syncthreads();
}

// VN fp32 values at p (16-byte aligned).
template <int VN>
__device__ __forceinline__ void ld_vec(const float *p, float *v) {
  ld_f32<4>(p, v);
  if constexpr (VN == 8) ld_f32<4>(p + 4, v + 4);
}

// VN values of a K-split output: the kMtpSplit partials at p, `stride`
// floats apart, added in part order.
template <int VN>
__device__ __forceinline__ void ld_parts(const float *p, size_t stride, float *v) {
  float q[kMtpSplit][VN];
#pragma unroll
  for (int s = 0; s < kMtpSplit; ++s) ld_vec<VN>(p + s * stride, q[s]);
#pragma unroll
  for (int i = 0; i < VN; ++i) {
    float t = q[0][i];
#pragma unroll
    for (int s = 1; s < kMtpSplit; ++s) t += q[s][i];
    v[i] = t;
  }
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_proj(ExpertArgs p, MtpArgs a, int step) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float inv[2][kTileM];
  __shared__ int tok[kTileM], rows[kTileM];
  __shared__ float half_acc[2][64][4];
  constexpr int VN = Vec<T>::N;
  const int d = a.d, nvec = d / VN, lda = 2 * d + VN, tid = threadIdx.x, lane = tid & 63;
  const int r0 = blockIdx.y * kTileM, m = min(kTileM, a.B - r0);
  T *A = reinterpret_cast<T *>(smem);
  float *part = reinterpret_cast<float *>(smem + static_cast<size_t>(kTileM) * lda * sizeof(T));
  const TileInfo ti{0, r0, m};
  DownPart<T, kDenseU> part_w;
  part_w.begin(p, ti, blockIdx.x, tid, nullptr, nullptr, blockIdx.z, kMtpSplit);  // in flight while u is built

  const unsigned long long *key_prev = a.argkey + static_cast<size_t>((step - 1) & 1) * a.B;
  if (tid < kTileM) {
    rows[tid] = r0 + tid;
    if (tid < m) {
      const int b = r0 + tid;
      const int t = step == 0 ? a.tokens[b] : static_cast<int>(key_index(key_prev[b]));
      tok[tid] = min(max(t, 0), a.V - 1);
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
    unsigned long long *key_cur = a.argkey + static_cast<size_t>(step & 1) * a.B;
    for (int b = tid; b < a.B; b += blockDim.x) {
      if (step > 0) a.drafts[static_cast<size_t>(b) * a.K + step - 1] = static_cast<int>(key_index(key_prev[b]));
      key_cur[b] = 0ull;
    }
  }
  __syncthreads();
  const T *h = static_cast<const T *>(step == 0 ? a.h_in : a.h_cur);
  const T *emb = static_cast<const T *>(a.embed);
  auto hv = [&](int r, int ch, float *v) { unpack(ld16(h + static_cast<size_t>(r0 + r) * d + ch * VN), v, T()); };
  auto ev = [&](int r, int ch, float *v) { unpack(ld16(emb + static_cast<size_t>(tok[r]) * d + ch * VN), v, T()); };
  const T *gh = static_cast<const T *>(a.norm_h), *ge = static_cast<const T *>(a.norm_e);
  const int nu = m * 2 * nvec;
  if (nu <= kOnePassChunks * kRowThreads) {
    // One pass: the 2m rows [h rows | E rows] (row q: h row q, or E row q - m)
    // and their gamma chunks are loaded once; the chunk sums, the per-row
    // reduction and u are tile_inv_rms's and the loop below's arithmetic.
    float v[kOnePassChunks][VN];
    uint4 gq[kOnePassChunks];
#pragma unroll
    for (int u = 0; u < kOnePassChunks; ++u) {
      const int it = tid + u * kRowThreads, q = it / nvec, ch = it - q * nvec;
      if (it < nu) {
        if (q >= m) ev(q - m, ch, v[u]); else hv(q, ch, v[u]);
        gq[u] = ld16((q >= m ? ge : gh) + ch * VN);
      }
    }
    float *inv_all = inv[0];  // inv[0][r] and inv[1][r] follow each other: row q at inv_all[q < m ? q : kTileM + q - m]
#pragma unroll
    for (int u = 0; u < kOnePassChunks; ++u) {
      const int it = tid + u * kRowThreads;
      float sq = v[u][0] * v[u][0];
#pragma unroll
      for (int i = 1; i < VN; ++i) sq = __builtin_fmaf(v[u][i], v[u][i], sq);
      if (it < nu) part[it] = sq;
    }
    __syncthreads();
    for (int q = tid >> 6; q < 2 * m; q += kRowThreads / kWave) {
      float acc = 0.f;
      for (int ch = lane; ch < nvec; ch += kWave) acc += part[q * nvec + ch];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
      if (lane == 0) inv_all[q < m ? q : kTileM + q - m] = 1.0f / sqrtf(acc / static_cast<float>(d) + a.eps);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kOnePassChunks; ++u) {
      const int it = tid + u * kRowThreads, q = it / nvec, ch = it - q * nvec;
      if (it >= nu) break;
      const int half = q >= m, r = q - half * m;
      float g[VN], o[VN];
      unpack(gq[u], g, T());
      const float sc = inv[half][r];
#pragma unroll
      for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[u][i] * sc) * g[i]);
      st16(A + r * lda + (half * nvec + ch) * VN, pack(o, T()));
    }
    __syncthreads();
    part_w.finish(p, ti, A + (lane & 15) * lda + (lane >> 4) * VN, half_acc, tid, rows, nullptr,
                  static_cast<size_t>(blockIdx.z) * a.B * d);
    return;
  }
  tile_inv_rms<VN>(m, d, a.eps, part, inv[0], hv);
  tile_inv_rms<VN>(m, d, a.eps, part, inv[1], ev);
  // u = [R(RMSNorm(h) * g_h) ; R(RMSNorm(E[t]) * g_e)] for rows [0, m) only: an
  // MFMA output row depends on its own A row alone
  for (int it0 = tid; it0 < nu; it0 += kChunksInFlight * blockDim.x) {
    float v[kChunksInFlight][VN];
    uint4 gq[kChunksInFlight];
#pragma unroll
    for (int u = 0; u < kChunksInFlight; ++u) {
      const int it = it0 + u * static_cast<int>(blockDim.x), r = it / (2 * nvec), c = it - r * 2 * nvec;
      const int half = c >= nvec, ch = c - half * nvec;
      if (it < nu) {
        if (half) ev(r, ch, v[u]); else hv(r, ch, v[u]);
        gq[u] = ld16((half ? ge : gh) + ch * VN);
      }
    }
#pragma unroll
    for (int u = 0; u < kChunksInFlight; ++u) {
      const int it = it0 + u * static_cast<int>(blockDim.x), r = it / (2 * nvec), c = it - r * 2 * nvec;
      if (it >= nu) break;
      float g[VN], o[VN];
      unpack(gq[u], g, T());
      const float sc = inv[c >= nvec][r];
#pragma unroll
      for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[u][i] * sc) * g[i]);
      st16(A + r * lda + c * VN, pack(o, T()));
    }
  }
  __syncthreads();
  part_w.finish(p, ti, A + (lane & 15) * lda + (lane >> 4) * VN, half_acc, tid, rows, nullptr,
                static_cast<size_t>(blockIdx.z) * a.B * d);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_ffn_gu(ExpertArgs p, MtpArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float inv[kTileM];
  constexpr int VN = Vec<T>::N;
  const int d = a.d, nvec = d / VN, lda = d + VN, tid = threadIdx.x, lane = tid & 63;
  const int r0 = blockIdx.y * kTileM, m = min(kTileM, a.B - r0);
  T *A = reinterpret_cast<T *>(smem);
  float *part = reinterpret_cast<float *>(smem + static_cast<size_t>(kTileM) * lda * sizeof(T));
  const TileInfo ti{0, r0, m};
  GateUpPart<T, kDenseU> part_w;
  part_w.begin(p, ti, blockIdx.x, tid, blockIdx.z, kMtpSplit);
  auto h1v = [&](int r, int ch, float *v) {  // h1 = R(z)
    ld_parts<VN>(a.acc + static_cast<size_t>(r0 + r) * d + ch * VN, static_cast<size_t>(a.B) * d, v);
#pragma unroll
    for (int i = 0; i < VN; ++i) v[i] = round_to<T>(v[i]);
  };
  const T *gf = static_cast<const T *>(a.norm_ffn);
  const int nx = m * nvec;
  if (nx <= kOnePassChunks * kRowThreads) {  // one pass, as in k_mtp_proj
    float v[kOnePassChunks][VN];
    uint4 gq[kOnePassChunks];
#pragma unroll
    for (int u = 0; u < kOnePassChunks; ++u) {
      const int it = tid + u * kRowThreads, r = it / nvec, ch = it - r * nvec;
      if (it < nx) {
        h1v(r, ch, v[u]);
        gq[u] = ld16(gf + ch * VN);
      }
    }
    one_pass_inv<VN>(m, nvec, d, a.eps, part, inv, v, nx);
#pragma unroll
    for (int u = 0; u < kOnePassChunks; ++u) {
      const int it = tid + u * kRowThreads, r = it / nvec;
      if (it >= nx) break;
      float g[VN], o[VN];
      unpack(gq[u], g, T());
#pragma unroll
      for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[u][i] * inv[r]) * g[i]);
      st16(A + r * lda + (it - r * nvec) * VN, pack(o, T()));
    }
    __syncthreads();
    part_w.finish_partial(p, ti, A + (lane & 15) * lda + (lane >> 4) * VN,
                          a.gu + static_cast<size_t>(blockIdx.z) * a.B * 2 * p.F, tid);
    return;
  }
  tile_inv_rms<VN>(m, d, a.eps, part, inv, h1v);
  // x = R(RMSNorm(h1) * g_ffn) for rows [0, m) (as in k_mtp_proj)
  for (int it0 = tid; it0 < nx; it0 += kChunksInFlight * blockDim.x) {
    float v[kChunksInFlight][VN];
    uint4 gq[kChunksInFlight];
#pragma unroll
    for (int u = 0; u < kChunksInFlight; ++u) {
      const int it = it0 + u * static_cast<int>(blockDim.x), r = it / nvec, ch = it - r * nvec;
      if (it < nx) {
        h1v(r, ch, v[u]);
        gq[u] = ld16(gf + ch * VN);
      }
    }
#pragma unroll
    for (int u = 0; u < kChunksInFlight; ++u) {
      const int it = it0 + u * static_cast<int>(blockDim.x), r = it / nvec;
      if (it >= nx) break;
      float g[VN], o[VN];
      unpack(gq[u], g, T());
#pragma unroll
      for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[u][i] * inv[r]) * g[i]);
      st16(A + r * lda + (it - r * nvec) * VN, pack(o, T()));
    }
  }
  __syncthreads();
  part_w.finish_partial(p, ti, A + (lane & 15) * lda + (lane >> 4) * VN,
                        a.gu + static_cast<size_t>(blockIdx.z) * a.B * 2 * p.F, tid);
}

// A dense projection of a 16-row tile of the rows at p.a (width p.F): the
// projection or the FFN down above kMtpFusedMaxB sequences; or (kFromGu) the
// FFN down whose tile a = R(SiLU(g) * u) is formed from the gate/up partials
// as it is staged.
template <typename T, bool kFromGu>
__global__ __launch_bounds__(kRowThreads) void k_mtp_ffn_dn(ExpertArgs p, MtpArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int rows[kTileM];
  __shared__ float half_acc[2][64][4];
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63, r0 = blockIdx.y * kTileM;
  const TileInfo ti{0, r0, min(kTileM, a.B - r0)};
  DownPart<T, kDenseU> part_w;
  part_w.begin(p, ti, blockIdx.x, threadIdx.x, nullptr, nullptr, blockIdx.z, kMtpSplit);
  if (threadIdx.x < kTileM) rows[threadIdx.x] = r0 + threadIdx.x;
  if constexpr (kFromGu) {  // a = R(SiLU(g) * u) of rows [0, m), zero rows past m
    const int F = p.F, nv = F / VN, ldf = F + VN;
    const size_t part_stride = static_cast<size_t>(a.B) * 2 * F;
    T *A = reinterpret_cast<T *>(smem);
    for (int it = threadIdx.x; it < kTileM * nv; it += blockDim.x) {
      const int rr = it / nv, c = it - rr * nv;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < ti.m) {
        const float *gp = a.gu + static_cast<size_t>(r0 + rr) * 2 * F + c * VN;
        float g[VN], u[VN], o[VN];
        ld_parts<VN>(gp, part_stride, g);
        ld_parts<VN>(gp + F, part_stride, u);
#pragma unroll
        for (int i = 0; i < VN; ++i) o[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
        v = pack(o, T());
      }
      st16(A + rr * ldf + c * VN, v);
    }
  } else {
    stage_a_tile<T>(p, ti, reinterpret_cast<T *>(smem), threadIdx.x, blockDim.x);
  }
  __syncthreads();
  part_w.finish(p, ti, reinterpret_cast<const T *>(smem) + (lane & 15) * (p.F + VN) + (lane >> 4) * VN, half_acc,
                threadIdx.x, rows, nullptr, static_cast<size_t>(blockIdx.z) * a.B * a.d);
}

// Larger batches (more than kMtpFusedMaxB sequences) normalise in row
// kernels, one block per sequence, and the projection and gate/up read their
// tiles from global memory: with 16 rows per tile the in-block norms of the
// fused kernels would run four rows after one another per wavefront.

// u = [R(RMSNorm(h) * g_h) ; R(RMSNorm(E[t]) * g_e)] of sequence blockIdx.x,
// with the token and key handling of k_mtp_proj.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_in(MtpArgs a, int step) {
  constexpr int VN = Vec<T>::N;
  __shared__ float part[kMtpMaxD / 4];
  __shared__ float inv[2];
  __shared__ int tok;
  const int b = blockIdx.x, d = a.d;
  if (threadIdx.x == 0) {
    const unsigned long long *key_prev = a.argkey + static_cast<size_t>((step - 1) & 1) * a.B;
    int t = a.tokens[b];
    if (step > 0) {
      t = static_cast<int>(key_index(key_prev[b]));
      a.drafts[static_cast<size_t>(b) * a.K + step - 1] = t;
    }
    a.argkey[static_cast<size_t>(step & 1) * a.B + b] = 0ull;
    tok = min(max(t, 0), a.V - 1);
  }
  __syncthreads();
  const T *h = static_cast<const T *>(step == 0 ? a.h_in : a.h_cur) + static_cast<size_t>(b) * d;
  const T *e = static_cast<const T *>(a.embed) + static_cast<size_t>(tok) * d;
  T *u = static_cast<T *>(a.u) + static_cast<size_t>(b) * 2 * d;
  auto hv = [&](int, int ch, float *v) { unpack(ld16(h + ch * VN), v, T()); };
  auto ev = [&](int, int ch, float *v) { unpack(ld16(e + ch * VN), v, T()); };
  tile_inv_rms<VN>(1, d, a.eps, part, inv, hv);
  tile_inv_rms<VN>(1, d, a.eps, part, inv + 1, ev);
  const T *gh = static_cast<const T *>(a.norm_h), *ge = static_cast<const T *>(a.norm_e);
  for (int c = threadIdx.x; c < 2 * (d / VN); c += blockDim.x) {
    const int half = c >= d / VN, ch = c - half * (d / VN);
    float v[VN], g[VN], o[VN];
    if (half) ev(0, ch, v); else hv(0, ch, v);
    unpack(ld16((half ? ge : gh) + ch * VN), g, T());
#pragma unroll
    for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[i] * inv[half]) * g[i]);
    st16(u + c * VN, pack(o, T()));
  }
}

// x = R(RMSNorm(R(z)) * g_ffn) of sequence blockIdx.x.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_mid(MtpArgs a) {
  constexpr int VN = Vec<T>::N;
  __shared__ float part[kMtpMaxD / 4];
  __shared__ float inv;
  const int b = blockIdx.x, d = a.d;
  const float *z = a.acc + static_cast<size_t>(b) * d;
  auto h1v = [&](int, int ch, float *v) {
    ld_parts<VN>(z + ch * VN, static_cast<size_t>(a.B) * d, v);
#pragma unroll
    for (int i = 0; i < VN; ++i) v[i] = round_to<T>(v[i]);
  };
  tile_inv_rms<VN>(1, d, a.eps, part, &inv, h1v);
  const T *gf = static_cast<const T *>(a.norm_ffn);
  T *x = static_cast<T *>(a.x) + static_cast<size_t>(b) * d;
  for (int ch = threadIdx.x; ch < d / VN; ch += blockDim.x) {
    float v[VN], g[VN], o[VN];
    h1v(0, ch, v);
    unpack(ld16(gf + ch * VN), g, T());
#pragma unroll
    for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[i] * inv) * g[i]);
    st16(x + ch * VN, pack(o, T()));
  }
}

// The FFN gate/up of a 16-row tile of x (global).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_dense_gu(ExpertArgs p, MtpArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float up_acc[2][64][4];
  constexpr int VN = Vec<T>::N;
  const int d = a.d, nvec = d / VN, lda = d + VN, lane = threadIdx.x & 63;
  const int r0 = blockIdx.y * kTileM, m = min(kTileM, a.B - r0);
  const TileInfo ti{0, r0, m};
  GateUpPart<T, kDenseU> part_w;
  part_w.begin(p, ti, blockIdx.x, threadIdx.x);
  T *A = reinterpret_cast<T *>(smem);
  const T *x = static_cast<const T *>(a.x);
  for (int it = threadIdx.x; it < m * nvec; it += blockDim.x) {  // rows [0, m), as in k_mtp_proj
    const int r = it / nvec, ch = it - r * nvec;
    st16(A + r * lda + ch * VN, ld16(x + static_cast<size_t>(r0 + r) * d + ch * VN));
  }
  __syncthreads();
  part_w.template finish<false>(p, ti, A + (lane & 15) * lda + (lane >> 4) * VN, up_acc, threadIdx.x);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_out(MtpArgs a, int last) {
  constexpr int VN = Vec<T>::N;
  __shared__ float part[kMtpMaxD / 4];
  __shared__ float inv;
  const int b = blockIdx.x, d = a.d;
  const float *z = a.acc + static_cast<size_t>(b) * d, *y = a.acc2 + static_cast<size_t>(b) * d;
  auto hv = [&](int, int ch, float *v) {  // h2 = R(R(z) + y)
    float q[VN];
    ld_parts<VN>(z + ch * VN, static_cast<size_t>(a.B) * d, v);
    ld_parts<VN>(y + ch * VN, static_cast<size_t>(a.B) * d, q);
#pragma unroll
    for (int i = 0; i < VN; ++i) v[i] = round_to<T>(round_to<T>(v[i]) + q[i]);
  };
  T *hc = static_cast<T *>(a.h_cur) + static_cast<size_t>(b) * d;
  T *ho = last && a.h_out ? static_cast<T *>(a.h_out) + static_cast<size_t>(b) * d : nullptr;
  for (int ch = threadIdx.x; ch < d / VN; ch += blockDim.x) {
    float v[VN];
    hv(0, ch, v);
    const uint4 pk = pack(v, T());
    st16(hc + ch * VN, pk);
    if (ho) st16(ho + ch * VN, pk);
  }
  tile_inv_rms<VN>(1, d, a.eps, part, &inv, hv);
  const T *go = static_cast<const T *>(a.norm_out);
  T *xo = static_cast<T *>(a.xo) + static_cast<size_t>(b) * d;
  for (int ch = threadIdx.x; ch < d / VN; ch += blockDim.x) {
    float v[VN], g[VN], o[VN];
    hv(0, ch, v);
    unpack(ld16(go + ch * VN), g, T());
#pragma unroll
    for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[i] * inv) * g[i]);
    st16(xo + ch * VN, pack(o, T()));
  }
}

// The LM head of a draft position up to kMtpFoldMaxB sequences with the
// output kernel folded in: each block requests its first weights, then forms
// the rows' x_o = R(RMSNorm(h2) * g_out), h2 = R(R(z) + y) from the
// projection's and the FFN's partials (the arithmetic of k_mtp_out, row for
// row), and block 0 also writes h2, the next position's input (and, after
// the last position, h_out).  The keys fold into p.argkey.
template <typename T>
__global__ __launch_bounds__(64 * kLmWaves) void k_mtp_lm(LmArgs p, MtpArgs a, int last) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ unsigned long long red[kLmWaves][kTileM];
  __shared__ float inv[kMtpFoldMaxB];
  constexpr int VN = Vec<T>::N;
  const int m = a.B, d = a.d, nvec = d / VN, lda = d + VN, tid = threadIdx.x, lane = tid & 63;
  T *A = reinterpret_cast<T *>(smem);  // rows [0, m) of x_o, then a zero row
  float *part = reinterpret_cast<float *>(smem + static_cast<size_t>(m + 1) * lda * sizeof(T));
  LmStream<T> ls;
  ls.begin(p, blockIdx.x, tid);  // weights requested before x_o is formed
  const size_t stride = static_cast<size_t>(a.B) * d;
  auto hv = [&](int r, int ch, float *v) {  // h2 = R(R(z) + y)
    float q[VN];
    ld_parts<VN>(a.acc + static_cast<size_t>(r) * d + ch * VN, stride, v);
    ld_parts<VN>(a.acc2 + static_cast<size_t>(r) * d + ch * VN, stride, q);
#pragma unroll
    for (int i = 0; i < VN; ++i) v[i] = round_to<T>(round_to<T>(v[i]) + q[i]);
  };
  const T *go = static_cast<const T *>(a.norm_out);
  T *hc = static_cast<T *>(a.h_cur), *ho = last && a.h_out ? static_cast<T *>(a.h_out) : nullptr;
  static_assert(64 * kLmWaves == kRowThreads, "the LM head's blocks have kRowThreads threads");
  if (m * nvec <= kOnePassChunks * kRowThreads) {  // one pass, as in k_mtp_proj
    const int n = m * nvec;
    float v[kOnePassChunks][VN];
    uint4 gq[kOnePassChunks];
#pragma unroll
    for (int u = 0; u < kOnePassChunks; ++u) {
      const int it = tid + u * kRowThreads, r = it / nvec, ch = it - r * nvec;
      if (it < n) {
        hv(r, ch, v[u]);
        gq[u] = ld16(go + ch * VN);
      }
    }
    one_pass_inv<VN>(m, nvec, d, a.eps, part, inv, v, n);
#pragma unroll
    for (int u = 0; u < kOnePassChunks; ++u) {
      const int it = tid + u * kRowThreads, r = it / nvec, ch = it - r * nvec;
      if (it >= n) break;
      if (blockIdx.x == 0) {
        const uint4 pk = pack(v[u], T());
        st16(hc + static_cast<size_t>(r) * d + ch * VN, pk);
        if (ho) st16(ho + static_cast<size_t>(r) * d + ch * VN, pk);
      }
      float g[VN], o[VN];
      unpack(gq[u], g, T());
#pragma unroll
      for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[u][i] * inv[r]) * g[i]);
      st16(A + r * lda + ch * VN, pack(o, T()));
    }
    for (int ch = tid; ch < nvec; ch += kRowThreads) st16(A + m * lda + ch * VN, make_uint4(0, 0, 0, 0));
    __syncthreads();
    const int arow = (lane & 15) < m ? (lane & 15) : m;
    ls.finish(p, 0, m, A + arow * lda + (lane >> 4) * VN, red, tid);
    return;
  }
  tile_inv_rms<VN>(m, d, a.eps, part, inv, hv);
  for (int it = tid; it < (m + 1) * nvec; it += blockDim.x) {
    const int r = it / nvec, ch = it - r * nvec;
    uint4 xo = make_uint4(0, 0, 0, 0);
    if (r < m) {
      float v[VN], g[VN], o[VN];
      hv(r, ch, v);
      if (blockIdx.x == 0) {
        const uint4 pk = pack(v, T());
        st16(hc + static_cast<size_t>(r) * d + ch * VN, pk);
        if (ho) st16(ho + static_cast<size_t>(r) * d + ch * VN, pk);
      }
      unpack(ld16(go + ch * VN), g, T());
#pragma unroll
      for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[i] * inv[r]) * g[i]);
      xo = pack(o, T());
    }
    st16(A + r * lda + ch * VN, xo);
  }
  __syncthreads();
  const int arow = (lane & 15) < m ? (lane & 15) : m;
  ls.finish(p, 0, m, A + arow * lda + (lane >> 4) * VN, red, tid);
}

__global__ void k_mtp_last(MtpArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  const unsigned long long *key = a.argkey + static_cast<size_t>((a.K - 1) & 1) * a.B;
  if (b < a.B) a.drafts[static_cast<size_t>(b) * a.K + a.K - 1] = static_cast<int>(key_index(key[b]));
}

template <typename KernelT>
void set_lds(KernelT kernel, size_t bytes) {
  if (bytes > 48 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(bytes));
}

}  // namespace

size_t mtp_proj_lds(int d, int es) {  // the tile and its rows' chunk sums
  return static_cast<size_t>(kTileM) * (2 * d + 16 / es) * es + static_cast<size_t>(kTileM) * (d / (16 / es)) * 4;
}
static size_t mtp_gu_lds(int d, int es) {
  return static_cast<size_t>(kTileM) * (d + 16 / es) * es + static_cast<size_t>(kTileM) * (d / (16 / es)) * 4;
}
size_t mtp_ffn_lds(int d, int F, int es) {
  const size_t gu = mtp_gu_lds(d, es);
  const size_t dn = static_cast<size_t>(kTileM) * (F + 16 / es) * es;
  return gu > dn ? gu : dn;
}

hipError_t launch_mtp_position(int dtype, const ExpertArgs &proj, const ExpertArgs &gu, const ExpertArgs &dn,
                               const MtpArgs &a, int step, hipStream_t s) {
  const int ntiles = (a.B + kTileM - 1) / kTileM, es = dtype == 1 ? 2 : 4;
  const bool fused = a.B <= kMtpFusedMaxB;
  const dim3 g_proj((a.d + 31) / 32, ntiles, kMtpSplit), g_gu((gu.F + 31) / 32, ntiles, fused ? kMtpSplit : 1),
      g_dn((a.d + 31) / 32, ntiles, kMtpSplit);
  const size_t l_proj = mtp_proj_lds(a.d, es);
  const size_t l_gu = mtp_gu_lds(a.d, es);
  const size_t l_dn = static_cast<size_t>(kTileM) * (dn.F + 16 / es) * es;
  const int last = step == a.K - 1;
  ExpertArgs proj_u = proj;  // the row-kernel path's projection reads u from global
  proj_u.a = a.u;
  if (dtype == 1) {
    set_lds(k_mtp_proj<bf16_t>, l_proj);
    set_lds(k_mtp_ffn_gu<bf16_t>, l_gu);
    set_lds(k_mtp_dense_gu<bf16_t>, l_gu);
    set_lds(k_mtp_ffn_dn<bf16_t, false>, l_proj > l_dn ? l_proj : l_dn);
    set_lds(k_mtp_ffn_dn<bf16_t, true>, l_dn);
    if (fused) {
      hipLaunchKernelGGL(k_mtp_proj<bf16_t>, g_proj, dim3(kRowThreads), l_proj, s, proj, a, step);
      hipLaunchKernelGGL(k_mtp_ffn_gu<bf16_t>, g_gu, dim3(kRowThreads), l_gu, s, gu, a);
    } else {
      hipLaunchKernelGGL(k_mtp_in<bf16_t>, dim3(a.B), dim3(kRowThreads), 0, s, a, step);
      hipLaunchKernelGGL((k_mtp_ffn_dn<bf16_t, false>), g_proj, dim3(kRowThreads), l_proj, s, proj_u, a);
      hipLaunchKernelGGL(k_mtp_mid<bf16_t>, dim3(a.B), dim3(kRowThreads), 0, s, a);
      hipLaunchKernelGGL(k_mtp_dense_gu<bf16_t>, g_gu, dim3(kRowThreads), l_gu, s, gu, a);
    }
    if (fused)
      hipLaunchKernelGGL((k_mtp_ffn_dn<bf16_t, true>), g_dn, dim3(kRowThreads), l_dn, s, dn, a);
    else
      hipLaunchKernelGGL((k_mtp_ffn_dn<bf16_t, false>), g_dn, dim3(kRowThreads), l_dn, s, dn, a);
    if (a.B > kMtpFoldMaxB)  // otherwise the LM head forms h2 and x_o (k_mtp_lm)
      hipLaunchKernelGGL(k_mtp_out<bf16_t>, dim3(a.B), dim3(kRowThreads), 0, s, a, last);
  } else {
    set_lds(k_mtp_proj<float>, l_proj);
    set_lds(k_mtp_ffn_gu<float>, l_gu);
    set_lds(k_mtp_dense_gu<float>, l_gu);
    set_lds(k_mtp_ffn_dn<float, false>, l_proj > l_dn ? l_proj : l_dn);
    set_lds(k_mtp_ffn_dn<float, true>, l_dn);
    if (fused) {
      hipLaunchKernelGGL(k_mtp_proj<float>, g_proj, dim3(kRowThreads), l_proj, s, proj, a, step);
      hipLaunchKernelGGL(k_mtp_ffn_gu<float>, g_gu, dim3(kRowThreads), l_gu, s, gu, a);
    } else {
      hipLaunchKernelGGL(k_mtp_in<float>, dim3(a.B), dim3(kRowThreads), 0, s, a, step);
      hipLaunchKernelGGL((k_mtp_ffn_dn<float, false>), g_proj, dim3(kRowThreads), l_proj, s, proj_u, a);
      hipLaunchKernelGGL(k_mtp_mid<float>, dim3(a.B), dim3(kRowThreads), 0, s, a);
      hipLaunchKernelGGL(k_mtp_dense_gu<float>, g_gu, dim3(kRowThreads), l_gu, s, gu, a);
    }
    if (fused)
      hipLaunchKernelGGL((k_mtp_ffn_dn<float, true>), g_dn, dim3(kRowThreads), l_dn, s, dn, a);
    else
      hipLaunchKernelGGL((k_mtp_ffn_dn<float, false>), g_dn, dim3(kRowThreads), l_dn, s, dn, a);
    if (a.B > kMtpFoldMaxB)  // otherwise the LM head forms h2 and x_o (k_mtp_lm)
      hipLaunchKernelGGL(k_mtp_out<float>, dim3(a.B), dim3(kRowThreads), 0, s, a, last);
  }
  return hipGetLastError();
}

hipError_t launch_mtp_lm(int dtype, const LmArgs &la, const MtpArgs &a, int step, hipStream_t s) {
  if (a.B > kMtpFoldMaxB) return launch_lm_argmax(dtype, la, s);
  if (la.T != a.B || la.d != a.d || la.done) return hipErrorInvalidValue;
  const int es = dtype == 1 ? 2 : 4, last = step == a.K - 1;
  const dim3 grid((la.V + kLmRowsPerBlock - 1) / kLmRowsPerBlock);
  const size_t smem = static_cast<size_t>(a.B + 1) * (a.d + 16 / es) * es +
                      static_cast<size_t>(a.B) * (a.d / (16 / es)) * 4;
  if (dtype == 1) {
    set_lds(k_mtp_lm<bf16_t>, smem);
    hipLaunchKernelGGL(k_mtp_lm<bf16_t>, grid, dim3(64 * kLmWaves), smem, s, la, a, last);
  } else {
    set_lds(k_mtp_lm<float>, smem);
    hipLaunchKernelGGL(k_mtp_lm<float>, grid, dim3(64 * kLmWaves), smem, s, la, a, last);
  }
  return hipGetLastError();
}

hipError_t launch_mtp_last(const MtpArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_mtp_last, dim3((a.B + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mv
