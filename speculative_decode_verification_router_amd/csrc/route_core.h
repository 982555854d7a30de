// Per-token routing core.  Every routing kernel runs this code, with one or
// sixteen tokens per block, so a token's results do not depend on the batch
// it is in.  Canonical arithmetic (chunk = one 16-byte vector: 8 bf16 or 4
// fp32 elements of a row):
//   combine   h' = round(h + y),  y = sum of the token's slots in slot order
//             (routed slots in selection order, then the shared ones)
//   sumsq     chunk partial p_c = sequential sum of h'^2 over chunk c (the
//             first square, then one fused multiply-add per element); lane l
//             of one wavefront sums p_c for c = l, l+64, ... in order; then a
//             xor butterfly (32, 16, 8, 4, 2, 1); lane 0's value
//   RMSNorm   x = round((h' * (sumsq/d + eps)^-1/2) * gamma)
//   router    16 lanes per expert: lane q sums, in one fp32 FMA chain, the
//             chunks c = q, q+16, ... of x * W_r[e]; xor butterfly (1, 2, 4,
//             8); lane q = 0's value, + optional bias
//   top-k     experts ordered by (logit desc, id asc); gates = softmax over
//             the k selected logits, denominator summed in rank order
// Routing follows the architecture paragraph of "Jina AI Releases jina-ocr-v1,
// a 3.4B MoE Document Parser With Built-In Speculative Decoding"
// (ainewsfeed.tech): 64 routed experts, top-6, two shared experts.
#pragma once

#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

constexpr int kRouteThreads = 1024;  // 16 wavefronts: wavefront w owns experts 4w..4w+3
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRouterChunks = 10;    // router chunks per lane held in registers (d <= 1280 bf16)

// Router weights of one wavefront's four experts (e = e_base + (lane >> 4)):
// lane q = lane & 15 holds the chunks c = q, q+16, ... of its expert's row.
template <typename T>
__device__ __forceinline__ void router_preload(uint4 *wq, const T *w_router, int E, int e_base, int d) {
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63, q = lane & 15;
  const int e = min(e_base + (lane >> 4), E - 1);
  const T *wr = w_router + static_cast<size_t>(e) * d;
  const int nvec = d / VN;
#pragma unroll
  for (int i = 0; i < kRouterChunks; ++i)
    if (q + 16 * i < nvec) wq[i] = gld16(wr + (q + 16 * i) * VN);
}

// Router logit (without bias) of expert e_base + lane / 16 for the x row at
// xr (LDS), the same value in all 16 lanes of the expert.
template <typename T>
__device__ __forceinline__ float router_dot(const uint4 *wq, const T *xr, int d, const T *w_router, int E,
                                            int e_base) {
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63, q = lane & 15;
  const int e = e_base + (lane >> 4);
  const int nvec = d / VN;
  const T *wr = w_router + static_cast<size_t>(min(e, E - 1)) * d;
  float acc = 0.f;
  auto accumulate = [&](const uint4 &wv, int c) {
    float w[VN], x[VN];
    unpack(wv, w, T());
    unpack(ld16(xr + c * VN), x, T());
#pragma unroll
    for (int j = 0; j < VN; ++j) acc = __builtin_fmaf(x[j], w[j], acc);
  };
#pragma unroll
  for (int i = 0; i < kRouterChunks; ++i)
    if (q + 16 * i < nvec) accumulate(wq[i], q + 16 * i);
  for (int c = q + 16 * kRouterChunks; c < nvec; c += 16) accumulate(gld16(wr + c * VN), c);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o);
  return acc;
}

// Router logits of tokens [0, nt) of the x rows in LDS (x_lds[t*ldx + j]).
// kThrough: the logits are written through (read by other blocks of the
// same launch).
template <typename T, bool kThrough = false>
__device__ __forceinline__ void router_rows(const uint4 *wq, const T *x_lds, int ldx, int nt, int d,
                                            const T *w_router, const float *bias, int E, int e_base,
                                            float *lg) {
  const int lane = threadIdx.x & 63, q = lane & 15;
  const int e = e_base + (lane >> 4);
  const float b = (bias && e < E) ? bias[e] : 0.f;
  for (int t = 0; t < nt; ++t) {
    const float acc = router_dot<T>(wq, x_lds + t * ldx, d, w_router, E, e_base);
    if (q == 0 && e < 64) {
      if constexpr (kThrough) st_agent(lg + t * 64 + e, acc + b);
      else lg[t * 64 + e] = acc + b;
    }
  }
}

// Top-k of one token's logits on one wavefront: lane e's rank
// is the number of experts ordered before it by (logit desc, id asc).  Each
// lane's (logit, id) key goes to LDS once (lanes >= E write 0, below every
// real key) and every lane counts the keys above its own, two per read.
// key_lds: 64 keys, 16-byte aligned; sel_lds: kMaxTopK floats.  logit: lane
// e's logit (lanes >= E: any value).  cnt_lds (LDS, optional): 1 is added to
// the count of every chosen expert.
__device__ __forceinline__ void select_top_k_of(float logit, uint64_t *key_lds, float *sel_lds, int E, int k,
                                                int *ids, float *gates, int *cnt_lds = nullptr) {
  const int lane = threadIdx.x & 63;
  const uint64_t mine = lane < E ? argmax_key(logit, static_cast<uint32_t>(lane)) : 0ull;
  key_lds[lane] = mine;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint4 *kv = reinterpret_cast<const uint4 *>(key_lds);
  int rank = 0;
#pragma unroll
  for (int j = 0; j < kWave / 2; ++j) {
    const uint4 two = kv[j];
    rank += ((static_cast<uint64_t>(two.y) << 32 | two.x) > mine) +
            ((static_cast<uint64_t>(two.w) << 32 | two.z) > mine);
  }
  const bool chosen = lane < E && rank < k;
  const uint64_t top = __ballot(chosen && rank == 0);
  const float vmax = __shfl(logit, static_cast<int>(__builtin_ctzll(top)));
  const float ex = expf(logit - vmax);
  if (chosen) {
    sel_lds[rank] = ex;
    ids[rank] = lane;
    if (cnt_lds) atomicAdd(cnt_lds + lane, 1);  // pairs per expert, counted in LDS
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // denominator in rank order; every entry is read, a surplus one adds -0
  float v[kMaxTopK];
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) v[s] = sel_lds[s];
  float den = 0.f + v[0];
#pragma unroll
  for (int s = 1; s < kMaxTopK; ++s) den += s < k ? v[s] : -0.f;
  if (chosen) gates[rank] = ex / den;
}

// select_top_k_of on lg_row[0..64).  kCoherent: the logits were written by
// other blocks of the same launch and are read with agent-scope loads.
template <bool kCoherent = false>
__device__ __forceinline__ void select_top_k(const float *lg_row, uint64_t *key_lds, float *sel_lds, int E,
                                             int k, int *ids, float *gates, int *cnt_lds = nullptr) {
  const int lane = threadIdx.x & 63;
  const float logit = kCoherent ? ld_agent(lg_row + lane)
                                : lg_row[lane];
  select_top_k_of(logit, key_lds, sel_lds, E, k, ids, gates, cnt_lds);
}

// LDS layout of a routing block holding `ntok` token rows.
struct RouteSmem {
  size_t h, g, p, lg, key, inv, sel, total;
};
__host__ __device__ inline RouteSmem route_smem(int ntok, int d, int elem_bytes) {
  const int vn = 16 / elem_bytes, nvec = d / vn;
  RouteSmem s;
  s.h = 0;                                                        // [ntok][d + vn] storage T
  s.g = s.h + static_cast<size_t>(ntok) * (d + vn) * elem_bytes;  // [d] gamma, storage T
  s.p = s.g + static_cast<size_t>(d) * elem_bytes;                // [ntok][nvec] fp32 partials
  s.lg = s.p + static_cast<size_t>(ntok) * nvec * 4;              // [ntok][64] logits
  s.key = s.lg + static_cast<size_t>(ntok) * 64 * 4;              // [ntok][64] top-k keys
  s.inv = s.key + static_cast<size_t>(ntok) * 64 * 8;             // [ntok]
  s.sel = s.inv + static_cast<size_t>(ntok) * 4;                  // [ntok][kMaxTopK]
  s.total = s.sel + static_cast<size_t>(ntok) * kMaxTopK * 4;
  return s;
}

// Routes tokens [t0, t0 + nt) (nt <= ntok) with one block of kRouteThreads.
// In kLogits mode the block takes expert group `eg` (experts kRouteGroup*eg
// onwards) of one token and writes only their logits; group 0 also writes
// h_dst and x_out.
template <typename T>
__device__ void route_block(const RouteArgs &a, const CombineArgs &c, int t0, int nt, int ntok,
                            unsigned char *smem, int eg = 0) {
  constexpr int VN = Vec<T>::N;
  const int d = a.d, nvec = d / VN, ld = d + VN;
  const RouteSmem L = route_smem(ntok, d, sizeof(T));
  T *hl = reinterpret_cast<T *>(smem + L.h);
  float *pl = reinterpret_cast<float *>(smem + L.p);
  float *lg = reinterpret_cast<float *>(smem + L.lg);
  float *inv = reinterpret_cast<float *>(smem + L.inv);
  float *sel = reinterpret_cast<float *>(smem + L.sel);
  uint64_t *keys = reinterpret_cast<uint64_t *>(smem + L.key);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // Every load of the first phase is requested before any is used, so the
  // block waits on one memory round trip: the router weights, gamma, the rows
  // and all of their slots.
  const bool logits_only = a.mode == kLogits;
  const int e_blk = logits_only ? kRouteGroup * eg : 0;                  // first expert of this block
  const int n_blk = logits_only ? kRouteGroup : 64;                      // experts of this block
  const bool router_wave = 4 * wv < n_blk && e_blk + 4 * wv < a.E;       // four experts per wavefront
  const bool writer = eg == 0;                                           // h_dst and x_out
  if (logits_only && blockIdx.x == 0)
    for (int i = tid; i < a.n_tile_done; i += blockDim.x) a.tile_done[i * kDoneStride] = 0u;
  if (a.status && blockIdx.x == 0 && tid == 0) *a.status = 0u;  // first launch of a call
  uint4 wq[kRouterChunks];
  if ((a.mode == kRoute || logits_only) && router_wave)
    router_preload<T>(wq, static_cast<const T *>(a.router_w), a.E, e_blk + 4 * wv, d);
  T *gl = reinterpret_cast<T *>(smem + L.g);
  uint4 gv = make_uint4(0, 0, 0, 0);
  if (a.mode != kCombine && tid < nvec) gv = ld16(static_cast<const T *>(a.gamma) + tid * VN);

  // combine (or plain load) of the rows: two adjacent lanes per chunk, HV
  // elements each.  The lower lane's running sum of squares is handed to the
  // upper one, which continues it, so each chunk partial keeps the sequential
  // order over the chunk's VN elements.
  constexpr int HV = VN / 2;
  constexpr int kSlotBatch = 8;  // slot loads in flight per lane
  const T *hs = static_cast<const T *>(c.h_src);
  for (int it = tid; it < nt * nvec * 2; it += blockDim.x) {
    const int r = it / (2 * nvec), hc = it - r * 2 * nvec, ch = hc >> 1, half = hc & 1;
    const int t = t0 + r;
    const int col = ch * VN + half * HV;
    const T *hrow = hs + static_cast<size_t>(t) * d + col;
    float h[HV];
    if (c.slots) {
      // slot loads first, index clamped so every load is unconditional; a
      // surplus slot adds -0, which leaves every sum unchanged
      const float *sp = c.slots + static_cast<size_t>(t) * a.nslot * d + col;
      float v[kSlotBatch][HV], y[HV];
#pragma unroll
      for (int s = 0; s < kSlotBatch; ++s)
        ld_f32<HV>(sp + static_cast<size_t>(min(s, a.nslot - 1)) * d, v[s]);
      const uint2 hq = ld8(hrow);
#pragma unroll
      for (int i = 0; i < HV; ++i) y[i] = 0.f + v[0][i];  // nslot >= 1 whenever slots are combined
#pragma unroll
      for (int s = 1; s < kSlotBatch; ++s)
#pragma unroll
        for (int i = 0; i < HV; ++i) y[i] += s < a.nslot ? v[s][i] : -0.f;
      for (int s0 = kSlotBatch; s0 < a.nslot; s0 += kSlotBatch) {
#pragma unroll
        for (int s = 0; s < kSlotBatch; ++s)
          ld_f32<HV>(sp + static_cast<size_t>(min(s0 + s, a.nslot - 1)) * d, v[s]);
#pragma unroll
        for (int s = 0; s < kSlotBatch; ++s)
#pragma unroll
          for (int i = 0; i < HV; ++i) y[i] += s0 + s < a.nslot ? v[s][i] : -0.f;
      }
      unpack8(hq, h, T());
#pragma unroll
      for (int i = 0; i < HV; ++i) h[i] = round_to<T>(h[i] + y[i]);
      if (c.y_moe) st_f32<HV>(c.y_moe + static_cast<size_t>(t) * d + col, y);
    } else {
      unpack8(ld8(hrow), h, T());
    }
    float p = h[0] * h[0];
#pragma unroll
    for (int i = 1; i < HV; ++i) p = __builtin_fmaf(h[i], h[i], p);
    const float lower = __shfl_xor(p, 1);
    if (half) {
      p = lower;
#pragma unroll
      for (int i = 0; i < HV; ++i) p = __builtin_fmaf(h[i], h[i], p);
      pl[r * nvec + ch] = p;
    }
    const uint2 pk = pack8(h, T());
    st8(hl + r * ld + col, pk);
    if (c.slots && c.h_dst && writer) st8(static_cast<T *>(c.h_dst) + static_cast<size_t>(t) * d + col, pk);
  }
  if (a.mode == kCombine) return;
  if (tid < nvec) st16(gl + tid * VN, gv);
  __syncthreads();

  // per-token sum of squares (wavefront r handles token r) and 1/rms
  for (int r = wv; r < nt; r += blockDim.x / kWave) {
    float acc = 0.f;
    for (int ch = lane; ch < nvec; ch += kWave) acc += pl[r * nvec + ch];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) inv[r] = 1.0f / sqrtf(acc / static_cast<float>(d) + a.eps);
  }
  __syncthreads();

  // x = round(h * inv * gamma): to LDS (router operand) and to x_out
  T *xo = static_cast<T *>(a.x_out);
  for (int it = tid; it < nt * nvec; it += blockDim.x) {
    const int r = it / nvec, ch = it % nvec;
    float hv[VN], g[VN], x[VN];
    unpack(ld16(hl + r * ld + ch * VN), hv, T());
    unpack(ld16(gl + ch * VN), g, T());
    const float s = inv[r];
#pragma unroll
    for (int i = 0; i < VN; ++i) x[i] = round_to<T>((hv[i] * s) * g[i]);
    const uint4 pk = pack(x, T());
    st16(hl + r * ld + ch * VN, pk);
    if (writer) st16(xo + static_cast<size_t>(t0 + r) * d + ch * VN, pk);
  }
  if (a.mode == kFinal) {
    if (tid < nt) a.argkey[t0 + tid] = 0ull;
    if (a.done && blockIdx.x == 0 && tid == 0) *a.done = 0u;
    return;
  }
  __syncthreads();

  if (logits_only) {
    if (router_wave)
      router_rows<T>(wq, hl, ld, nt, d, static_cast<const T *>(a.router_w), a.router_b, a.E, e_blk + 4 * wv,
                     a.logits + static_cast<size_t>(t0) * 64);
    return;
  }
  if (router_wave)
    router_rows<T>(wq, hl, ld, nt, d, static_cast<const T *>(a.router_w), a.router_b, a.E, 4 * wv, lg);
  __syncthreads();
  for (int r = wv; r < nt; r += blockDim.x / kWave)
    select_top_k(lg + r * 64, keys + r * 64, sel + r * kMaxTopK, a.E, a.k, a.ids + (t0 + r) * a.k,
                 a.gates + (t0 + r) * a.k);
}

// Routing of one token inside the fused small-batch expert launch: a block of
// 256 threads takes token t's combine and RMSNorm and the logits of expert
// group eg.  The arithmetic is route_block's in kLogits mode, with one thread
// per 16-byte chunk (its sum of squares is the same sequential sum).  x and
// the logits, which other blocks of the launch read, are written through.
// In the fused expert launch the logits are stored once x has completed, and
// the readers take them as they land (their buffer was filled with
// kLogitUnset before the launch).  In the one-launch step (kInLaunch), once x
// and the logits have completed the block adds 1 to every copy of the
// routing counter (done[i * stride], i < copies).  Group 0 also writes h_dst,
// which only later launches read.
// kInLaunch: h_src and the slots were written by other blocks of the same
// launch (agent-scope loads) and h_dst is read by later blocks of it
// (write-through).  kFinal: route_block's kFinal mode (final norm, x_f to
// a.x_out, argkey[t] cleared), no router.
template <typename T, bool kInLaunch = false, bool kFinal = false>
__device__ void route_fused(const RouteArgs &a, const CombineArgs &c, int t, int eg, unsigned char *smem,
                            unsigned *done, int copies, int stride) {
  constexpr int VN = Vec<T>::N;
  constexpr int kSlotBatch = 8;
  const int d = a.d, nvec = d / VN;
  const RouteSmem L = route_smem(1, d, sizeof(T));
  T *hl = reinterpret_cast<T *>(smem + L.h);
  T *gl = reinterpret_cast<T *>(smem + L.g);
  float *pl = reinterpret_cast<float *>(smem + L.p);
  float *inv = reinterpret_cast<float *>(smem + L.inv);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e_blk = kRouteGroup * eg;
  const bool router_wave = !kFinal && 4 * wv < kRouteGroup && e_blk + 4 * wv < a.E;
  const bool writer = eg == 0;
  auto slot4 = [](const float *p, float *o) {
    if constexpr (kInLaunch) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = ld_agent(p + i);
    } else {
      ld_f32<4>(p, o);
    }
  };

  uint4 wq[kRouterChunks];
  if (router_wave) router_preload<T>(wq, static_cast<const T *>(a.router_w), a.E, e_blk + 4 * wv, d);
  const T *hs = static_cast<const T *>(c.h_src);
  for (int ch = tid; ch < nvec; ch += blockDim.x) {
    const uint4 gv = ld16(static_cast<const T *>(a.gamma) + ch * VN);
    const T *hrow = hs + static_cast<size_t>(t) * d + ch * VN;
    float h[VN];
    if (c.slots) {
      const float *sp = c.slots + static_cast<size_t>(t) * a.nslot * d + ch * VN;
      float v[kSlotBatch][VN], y[VN];
#pragma unroll
      for (int s = 0; s < kSlotBatch; ++s)
#pragma unroll
        for (int i = 0; i < VN; i += 4) slot4(sp + static_cast<size_t>(min(s, a.nslot - 1)) * d + i, v[s] + i);
      const uint4 hq = kInLaunch ? ld16_agent(hrow) : ld16(hrow);
#pragma unroll
      for (int i = 0; i < VN; ++i) y[i] = 0.f + v[0][i];
#pragma unroll
      for (int s = 1; s < kSlotBatch; ++s)
#pragma unroll
        for (int i = 0; i < VN; ++i) y[i] += s < a.nslot ? v[s][i] : -0.f;
      for (int s0 = kSlotBatch; s0 < a.nslot; s0 += kSlotBatch) {
#pragma unroll
        for (int s = 0; s < kSlotBatch; ++s)
#pragma unroll
          for (int i = 0; i < VN; i += 4)
            slot4(sp + static_cast<size_t>(min(s0 + s, a.nslot - 1)) * d + i, v[s] + i);
#pragma unroll
        for (int s = 0; s < kSlotBatch; ++s)
#pragma unroll
          for (int i = 0; i < VN; ++i) y[i] += s0 + s < a.nslot ? v[s][i] : -0.f;
      }
      unpack(hq, h, T());
#pragma unroll
      for (int i = 0; i < VN; ++i) h[i] = round_to<T>(h[i] + y[i]);
    } else {
      unpack(kInLaunch ? ld16_agent(hrow) : ld16(hrow), h, T());
    }
    float p = h[0] * h[0];
#pragma unroll
    for (int i = 1; i < VN; ++i) p = __builtin_fmaf(h[i], h[i], p);
    pl[ch] = p;
    const uint4 pk = pack(h, T());
    st16(hl + ch * VN, pk);
    st16(gl + ch * VN, gv);
    if (c.slots && c.h_dst && writer) {
      T *hd = static_cast<T *>(c.h_dst) + static_cast<size_t>(t) * d + ch * VN;
      if constexpr (kInLaunch) st16_through(hd, pk);
      else st16(hd, pk);
    }
  }
  __syncthreads();
  if (wv == 0) {  // sum of squares and 1/rms, in route_block's order
    float acc = 0.f;
    for (int ch = lane; ch < nvec; ch += kWave) acc += pl[ch];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) inv[0] = 1.0f / sqrtf(acc / static_cast<float>(d) + a.eps);
  }
  __syncthreads();
  T *xo = static_cast<T *>(a.x_out) + static_cast<size_t>(t) * d;
  for (int ch = tid; ch < nvec; ch += blockDim.x) {
    float hv[VN], g[VN], x[VN];
    unpack(ld16(hl + ch * VN), hv, T());
    unpack(ld16(gl + ch * VN), g, T());
    const float sc = inv[0];
#pragma unroll
    for (int i = 0; i < VN; ++i) x[i] = round_to<T>((hv[i] * sc) * g[i]);
    const uint4 pk = pack(x, T());
    st16(hl + ch * VN, pk);
    if (writer) {
      uint32_t *q = reinterpret_cast<uint32_t *>(xo + ch * VN);
      st_agent(q, pk.x);
      st_agent(q + 1, pk.y);
      st_agent(q + 2, pk.z);
      st_agent(q + 3, pk.w);
    }
  }
  if constexpr (kFinal) {
    if (tid == 0) st_agent(a.argkey + t, 0ull);
  } else if constexpr (!kInLaunch) {
    // the fused launch's readers take the logits as they land, so x must
    // have completed before any logit is stored; the wait overlaps the
    // router's dot products
    __syncthreads();
    const int e = e_blk + 4 * wv + (lane >> 4);
    float lg = 0.f;
    if (router_wave) {
      lg = router_dot<T>(wq, hl, d, static_cast<const T *>(a.router_w), a.E, e_blk + 4 * wv);
      lg += (a.router_b && e < a.E) ? a.router_b[e] : 0.f;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's x has completed
    __syncthreads();
    if (router_wave && (lane & 15) == 0 && e < 64)
      st_agent(a.logits + static_cast<size_t>(t) * 64 + e, lg);
    return;
  } else {
    __syncthreads();
    if (router_wave)
      router_rows<T, true>(wq, hl, 0, 1, d, static_cast<const T *>(a.router_w), a.router_b, a.E, e_blk + 4 * wv,
                           a.logits + static_cast<size_t>(t) * 64);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's x and logits have completed
  __syncthreads();
  if (tid < copies)
    add_agent(done + static_cast<size_t>(tid) * stride, 1u);
}

// ---------------------------------------------------------------- grouping

// Where the grouping of (token, slot) pairs by expert is written.
struct GroupOut {
  int *seg;         // [E+S+1] first row of each expert segment
  int *tile_start;  // [E+S+1] first tile of each expert
  int *rows;        // [T*nslot] pair id (t*nslot + slot) of each sorted row
  int4 *tile_info;  // [tiles] (expert, first row, rows, 0), or null
};

// Lanes of this wavefront whose value equals this lane's (values < 128),
// from seven ballots over the bits of the value.
__device__ __forceinline__ uint64_t match_lanes(int v, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const bool bit = (v >> b) & 1;
    const uint64_t on = __ballot(valid && bit);
    m &= bit ? on : ~on;
  }
  return valid ? m : 0ull;
}

// Stable grouping of the T*k routed pairs by expert with the block's first
// `nw` wavefronts, each taking a contiguous run of pairs 64 at a time: a
// pair's same-expert lanes give its rank among the earlier pairs of its
// expert in the run and, for the first of them, the run's count; per-expert
// offsets of the runs follow in wavefront order, so every expert segment
// keeps ascending pair order.  Shared expert s gets segment E + s holding
// every token.  Every thread of the block must call this (it synchronises
// the block).  Requires E <= 64, nw * 64 <= blockDim.x and `cnt_lds`,
// `run_lds` in LDS with nw * 64 ints each.  `ids` and every output may be in
// global memory or in LDS.
__device__ inline void group_pairs(const int *ids, int T, int E, int S, int k, int nslot, int tile_m,
                                   const GroupOut &o, int *cnt_lds, int *run_lds, int nw) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int np = T * k;
  nw = max(1, min(nw, (np + kWave - 1) / kWave));  // no idle runs for small batches
  const bool mine = w < nw;
  const int per = ((np + nw - 1) / nw + kWave - 1) / kWave * kWave;
  const int p0 = mine ? min(np, w * per) : 0, p1 = mine ? min(np, p0 + per) : 0;
  const uint64_t below = (1ull << lane) - 1ull;
  if (mine) cnt_lds[w * kWave + lane] = 0;
  __syncthreads();
  for (int base = p0; base < p1; base += kWave) {
    const int q = base + lane;
    const int e_q = q < p1 ? ids[q] : 0;
    const uint64_t m = match_lanes(e_q, q < p1);
    if (q < p1 && (m & below) == 0) cnt_lds[w * kWave + e_q] += __popcll(m);  // first lane of its expert
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  const int shared_tiles = (T + tile_m - 1) / tile_m;
  __shared__ int routed_end[2];
  if (w == 0) {
    // per expert (lane): offsets of the runs, then scans over the experts
    int cnt = 0;
    for (int v = 0; v < nw; ++v) {
      const int c = lane < E ? cnt_lds[v * kWave + lane] : 0;
      run_lds[v * kWave + lane] = cnt;
      cnt += c;
    }
    const int tiles = (cnt + tile_m - 1) / tile_m;
    int sc = cnt, st = tiles;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int vc = __shfl_up(sc, off), vt = __shfl_up(st, off);
      if (lane >= off) { sc += vc; st += vt; }
    }
    const int seg_e = sc - cnt, tile_e = st - tiles;
    const int routed_total = __builtin_amdgcn_readlane(sc, kWave - 1);
    const int routed_tiles = __builtin_amdgcn_readlane(st, kWave - 1);
    if (lane < E) {
      o.seg[lane] = seg_e;
      o.tile_start[lane] = tile_e;
    }
    if (lane <= S) {
      o.seg[E + lane] = routed_total + lane * T;
      o.tile_start[E + lane] = routed_tiles + lane * shared_tiles;
    }
    for (int v = 0; v < nw; ++v) run_lds[v * kWave + lane] += seg_e;  // next free row per run
    if (o.tile_info && lane < E)
      for (int j = 0; j < tiles; ++j)
        o.tile_info[tile_e + j] = make_int4(lane, seg_e + j * tile_m, min(tile_m, cnt - j * tile_m), 0);
    if (lane == 0) {
      routed_end[0] = routed_total;
      routed_end[1] = routed_tiles;
    }
  }
  __syncthreads();
  // scatter the routed pairs
  for (int base = p0; base < p1; base += kWave) {
    const int q = base + lane;
    const int e_q = q < p1 ? ids[q] : 0;
    const uint64_t m = match_lanes(e_q, q < p1);
    if (q < p1) o.rows[run_lds[w * kWave + e_q] + __popcll(m & below)] = (q / k) * nslot + (q % k);
    __builtin_amdgcn_wave_barrier();
    if (q < p1 && (m & below) == 0) run_lds[w * kWave + e_q] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  const int routed_total = routed_end[0], routed_tiles = routed_end[1];
  for (int j = threadIdx.x; j < S * T; j += blockDim.x) {
    const int s = j / T, t = j % T;
    o.rows[routed_total + s * T + t] = t * nslot + k + s;
  }
  if (o.tile_info)
    for (int j = threadIdx.x; j < S * shared_tiles; j += blockDim.x) {
      const int s = j / shared_tiles, i = j % shared_tiles;
      o.tile_info[routed_tiles + j] =
          make_int4(E + s, routed_total + s * T + i * tile_m, min(tile_m, T - i * tile_m), 0);
    }
}

}  // namespace mv
