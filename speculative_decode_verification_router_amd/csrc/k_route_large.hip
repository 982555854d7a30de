// Routing and grouping for large batches (bf16, the compute-bound path).
//
// k_route_large: 16 tokens per block of eight wavefronts.  Each wavefront
// requests its router-weight fragments first, then RMSNorm with the canonical
// sum of squares (route_core.h), the router logits x W_r^T on the matrix
// cores (v_mfma_f32_32x32x16_bf16; the products of bf16 values are exact and
// the sums fp32, in the instruction's order; four K quarters added in order),
// top-k by rank as in route_core.h, and the block's per-expert pair counts.
//
// k_scatter: the stable grouping of the (token, slot) pairs by expert from
// those counts.  Each block takes the same 16 tokens: the counts of the
// blocks before it give each expert's offset, a ballot match ranks its own
// pairs, so every expert segment keeps ascending pair order.  Block 0 also
// writes the segment and tile tables.  Routing follows the architecture
// paragraph of "Jina AI Releases jina-ocr-v1, a 3.4B MoE Document Parser With
// Built-In Speculative Decoding" (ainewsfeed.tech): 64 routed experts, top-6,
// two shared experts.
#include "route_core.h"

namespace mv {

namespace {

constexpr int kRLTok = 16;       // tokens per routing block
constexpr int kRLThreads = 512;  // 8 wavefronts: 2 expert halves x 4 K quarters
// K windows per quarter prefetched into registers (half a quarter at d = 1280;
// the rest is read in the MFMA loop): 110 VGPRs, so two blocks share a CU
constexpr int kRLQuarterWin = 10;
constexpr int kScatterThreads = 256;
constexpr int kScatterBatch = 32;  // count loads in flight per thread (16.9 -> 14.5 us over 8)

struct RLSmem {
  size_t x, p, lg, key, inv, sel, g, total;
};
__host__ __device__ inline RLSmem rl_smem(int d) {
  const int nvec = d / 8;
  RLSmem s;
  s.x = 0;                                                         // [17][d + 8] bf16: rows, then a zero row
  s.p = s.x + static_cast<size_t>(kRLTok + 1) * (d + 8) * 2;       // [16][nvec] fp32 chunk partials
  // [4][16][64] fp32 logit quarters, over the partials: those are read
  // before the block barriers that precede the logits
  s.lg = s.p;
  const size_t p_bytes = static_cast<size_t>(kRLTok) * nvec * 4, lg_bytes = static_cast<size_t>(4) * kRLTok * 64 * 4;
  s.key = s.lg + (p_bytes > lg_bytes ? p_bytes : lg_bytes);        // [16][64] top-k keys
  s.inv = s.key + static_cast<size_t>(kRLTok) * 64 * 8;            // [16]
  s.sel = s.inv + kRLTok * 4;                                      // [16][kMaxTopK]
  s.g = s.sel + kRLTok * kMaxTopK * 4;                             // [d] gamma, bf16
  s.total = s.g + static_cast<size_t>(d) * 2;
  return s;
}

__global__ __launch_bounds__(kRLThreads) void k_route_large(RouteArgs a, const bf16_t *h, int *blk_cnt) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int cnt[64];
  const int d = a.d, nvec = d / 8, ld = d + 8;
  const RLSmem L = rl_smem(d);
  bf16_t *xl = reinterpret_cast<bf16_t *>(smem + L.x);
  float *pl = reinterpret_cast<float *>(smem + L.p);
  float *lg = reinterpret_cast<float *>(smem + L.lg);
  float *inv = reinterpret_cast<float *>(smem + L.inv);
  float *sel = reinterpret_cast<float *>(smem + L.sel);
  uint64_t *keys = reinterpret_cast<uint64_t *>(smem + L.key);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int t0 = blockIdx.x * kRLTok, nt = min(kRLTok, a.T - t0);

  if (tid < 64) cnt[tid] = 0;
  if (a.status && blockIdx.x == 0 && tid == 0) *a.status = 0u;  // first launch of a call
  // router weights first: wavefront w takes experts 32*(w&1) .. +31 over K
  // quarter w>>1, its fragments requested before the rows are read
  const int nwin = d / 16, quarter = wv >> 1;
  const int w_lo = quarter * nwin / 4, w_hi = (quarter + 1) * nwin / 4;
  const int e_r = min(32 * (wv & 1) + (lane & 31), a.E - 1);
  const bf16_t *wr = static_cast<const bf16_t *>(a.router_w) + static_cast<size_t>(e_r) * d + (lane >> 5) * 8;
  uint4 b[kRLQuarterWin];
#pragma unroll
  for (int u = 0; u < kRLQuarterWin; ++u) b[u] = ld16(wr + min(w_lo + u, w_hi - 1) * 16);
  // gamma to LDS, requested with the rows (read by the x pass below, which
  // also stores x_out: a global gamma load there would wait for those stores)
  const bf16_t *gam = static_cast<const bf16_t *>(a.gamma);
  bf16_t *gl = reinterpret_cast<bf16_t *>(smem + L.g);
  uint4 gv = make_uint4(0, 0, 0, 0);
  if (tid < nvec) gv = ld16(gam + tid * 8);
  // rows, chunk partial sums of squares; rows nt..16 are zero (row 16 feeds
  // the MFMA tile's rows 16..31).  kRowLoads loads per thread cover all
  // 17 rows in one round trip for d <= 1280.
  constexpr int kRowLoads = 6;
  for (int it0 = tid; it0 < (kRLTok + 1) * nvec; it0 += kRowLoads * kRLThreads) {
    uint4 v[kRowLoads];
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
      const int it = it0 + u * kRLThreads, r = it / nvec, ch = it - r * nvec;
      v[u] = make_uint4(0, 0, 0, 0);
      if (it < (kRLTok + 1) * nvec && r < nt) v[u] = ld16(h + static_cast<size_t>(t0 + r) * d + ch * 8);
    }
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
      const int it = it0 + u * kRLThreads, r = it / nvec, ch = it - r * nvec;
      if (it >= (kRLTok + 1) * nvec) break;
      if (r < nt) {
        float f[8];
        unpack(v[u], f, bf16_t());
        float s = f[0] * f[0];  // route_block's order: first square, then fused multiply-adds
#pragma unroll
        for (int i = 1; i < 8; ++i) s = __builtin_fmaf(f[i], f[i], s);
        pl[r * nvec + ch] = s;
      }
      st16(xl + r * ld + ch * 8, v[u]);
    }
  }
  if (tid < nvec) st16(gl + tid * 8, gv);
  __syncthreads();
  for (int r = wv; r < nt; r += kRLThreads / kWave) {
    float acc = 0.f;
    for (int ch = lane; ch < nvec; ch += kWave) acc += pl[r * nvec + ch];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) inv[r] = 1.0f / sqrtf(acc / static_cast<float>(d) + a.eps);
  }
  __syncthreads();
  bf16_t *xo = static_cast<bf16_t *>(a.x_out);
  for (int it = tid; it < nt * nvec; it += blockDim.x) {
    const int r = it / nvec, ch = it - r * nvec;
    float hv[8], g[8], x[8];
    unpack(ld16(xl + r * ld + ch * 8), hv, bf16_t());
    unpack(ld16(gl + ch * 8), g, bf16_t());
    const float s = inv[r];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = round_to<bf16_t>((hv[i] * s) * g[i]);
    const uint4 pk = pack(x, bf16_t());
    st16(xl + r * ld + ch * 8, pk);
    st16(xo + static_cast<size_t>(t0 + r) * d + ch * 8, pk);
  }
  __syncthreads();

  {  // logits of this wavefront's experts over its K quarter; rows < 16 kept
    const bf16_t *xr = xl + min(lane & 31, kRLTok) * ld + (lane >> 5) * 8;
    f32x16_t acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll
    for (int u = 0; u < kRLQuarterWin; ++u)
      if (w_lo + u < w_hi) mfma32(acc, ld16(xr + (w_lo + u) * 16), b[u]);
    for (int w = w_lo + kRLQuarterWin; w < w_hi; ++w) mfma32(acc, ld16(xr + w * 16), ld16(wr + w * 16));
    float *dst = lg + quarter * kRLTok * 64;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
      if (row < kRLTok) dst[row * 64 + 32 * (wv & 1) + (lane & 31)] = acc[q];
    }
  }
  __syncthreads();
  for (int i = tid; i < nt * 64; i += blockDim.x) {
    const int r = i / 64, e = i % 64;
    const float bias = (a.router_b && e < a.E) ? a.router_b[e] : 0.f;
    const float *q = lg + r * 64 + e;
    lg[r * 64 + e] = (((q[0] + q[kRLTok * 64]) + q[2 * kRLTok * 64]) + q[3 * kRLTok * 64]) + bias;
  }
  __syncthreads();
  for (int r = wv; r < nt; r += kRLThreads / kWave)
    select_top_k(lg + r * 64, keys + r * 64, sel + r * kMaxTopK, a.E, a.k, a.ids + (t0 + r) * a.k,
                 a.gates + (t0 + r) * a.k, cnt);
  __syncthreads();
  if (tid < 64) blk_cnt[blockIdx.x * 64 + tid] = cnt[tid];
}

__global__ __launch_bounds__(kScatterThreads) void k_scatter(RouteArgs a, const int *blk_cnt, int nblk) {
  __shared__ int part_tot[4][64], part_before[4][64];
  __shared__ int seg_e[64], base_e[64], first_run[64];
  __shared__ int ends[2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E, S = a.S, k = a.k, T = a.T, tm = a.tile_m;
  {  // per expert: all pairs, and pairs in the blocks before this one
    const int e = tid & 63, part = tid >> 6;
    const int b0 = part * nblk / 4, b1 = (part + 1) * nblk / 4;
    int tot = 0, before = 0;
    for (int b = b0; b < b1; b += kScatterBatch) {
      int c[kScatterBatch];  // loads in flight per thread
#pragma unroll
      for (int u = 0; u < kScatterBatch; ++u) c[u] = b + u < b1 ? blk_cnt[(b + u) * 64 + e] : 0;
#pragma unroll
      for (int u = 0; u < kScatterBatch; ++u) {
        tot += c[u];
        before += b + u < static_cast<int>(blockIdx.x) ? c[u] : 0;
      }
    }
    part_tot[part][e] = tot;
    part_before[part][e] = before;
  }
  __syncthreads();
  if (wv == 0) {
    const int cnt = lane < E ? part_tot[0][lane] + part_tot[1][lane] + part_tot[2][lane] + part_tot[3][lane] : 0;
    const int before = part_before[0][lane] + part_before[1][lane] + part_before[2][lane] + part_before[3][lane];
    const int tiles = (cnt + tm - 1) / tm;
    int sc = cnt, st = tiles;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int vc = __shfl_up(sc, off), vt = __shfl_up(st, off);
      if (lane >= off) { sc += vc; st += vt; }
    }
    const int seg = sc - cnt, tile0 = st - tiles;
    const int routed_total = __builtin_amdgcn_readlane(sc, kWave - 1);
    const int routed_tiles = __builtin_amdgcn_readlane(st, kWave - 1);
    seg_e[lane] = seg;
    base_e[lane] = seg + before;
    if (lane == 0) {
      ends[0] = routed_total;
      ends[1] = routed_tiles;
    }
    if (blockIdx.x == 0) {
      const int shared_tiles = (T + tm - 1) / tm;
      if (lane < E) {
        a.seg[lane] = seg;
        a.tile_start[lane] = tile0;
        for (int j = 0; j < tiles; ++j)
          a.tile_info[tile0 + j] = make_int4(lane, seg + j * tm, min(tm, cnt - j * tm), 0);
      }
      if (lane <= S) {
        a.seg[E + lane] = routed_total + lane * T;
        a.tile_start[E + lane] = routed_tiles + lane * shared_tiles;
      }
      for (int j = lane; j < S * shared_tiles; j += kWave) {
        const int s = j / shared_tiles, i = j % shared_tiles;
        a.tile_info[routed_tiles + j] = make_int4(E + s, routed_total + s * T + i * tm, min(tm, T - i * tm), 0);
      }
    }
  }
  __syncthreads();
  // this block's pairs: wavefront w ranks pairs [64w, 64w + 64) of the block
  const int t0 = blockIdx.x * kRLTok, nt = min(kRLTok, T - t0);
  const int np = nt * k, p0 = t0 * k;
  const int nw = (np + kWave - 1) / kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  __shared__ int run_cnt[4][64];
  if (wv < nw) {
    run_cnt[wv][lane] = 0;
    __builtin_amdgcn_wave_barrier();
    const int q = wv * kWave + lane;
    const int e_q = q < np ? a.ids[p0 + q] : 0;
    const uint64_t m = match_lanes(e_q, q < np);
    if (q < np && (m & below) == 0) run_cnt[wv][e_q] = __popcll(m);
  }
  __syncthreads();
  if (wv < nw) {
    const int q = wv * kWave + lane;
    const int e_q = q < np ? a.ids[p0 + q] : 0;
    const uint64_t m = match_lanes(e_q, q < np);
    int off = base_e[e_q];
    for (int v = 0; v < wv; ++v) off += run_cnt[v][e_q];
    if (q < np) a.rows[off + __popcll(m & below)] = ((p0 + q) / k) * a.nslot + (p0 + q) % k;
  }
  const int routed_total = ends[0];
  for (int j = tid; j < S * nt; j += blockDim.x) {
    const int s = j / nt, t = t0 + j % nt;
    a.rows[routed_total + s * T + t] = t * a.nslot + k + s;
  }
}

}  // namespace

int route_large_blocks(int T) { return (T + kRLTok - 1) / kRLTok; }

hipError_t launch_route_large(const RouteArgs &a, const void *h, int *blk_cnt, hipStream_t s) {
  const size_t smem = rl_smem(a.d).total;
  if (smem > 48 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k_route_large),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  const int nblk = route_large_blocks(a.T);
  hipLaunchKernelGGL(k_route_large, dim3(nblk), dim3(kRLThreads), smem, s, a, static_cast<const bf16_t *>(h),
                     blk_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scatter, dim3(nblk), dim3(kScatterThreads), 0, s, a, static_cast<const int *>(blk_cnt), nblk);
  return hipGetLastError();
}

}  // namespace mv
