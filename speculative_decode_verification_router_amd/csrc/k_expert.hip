// Grouped expert FFN kernels (routed experts and the always-on shared ones).
//
// Up to 128 rows a block is one 16-row tile and one slice pair (the tile
// parts of expert_core.h), with the tile's activation rows staged in LDS as
// the MFMA A operand.  Small batches skip the separate grouping kernel: every
// wavefront of a gate/up block finds its block's tile from the routing
// itself, and the blocks of the first slice pair write the grouping for the
// down kernel, each its own tile's entry.  Batches of up to 8 rows routed to
// logits run gate/up and down in one launch (k_ffn_small), taking the top-k
// in every block.
#include "expert_core.h"
#include "lm_core.h"

namespace mv {

namespace {

// Tile `y` of the grouping table.  The entry is requested together with the
// tile count, one round trip: the table holds an entry for every block of the
// grid, and the test reads both, so neither load waits for the other.
__device__ __forceinline__ bool table_tile(const ExpertArgs &p, int y, TileInfo &ti) {
  const int4 v = p.tile_info[y];
  const int n = p.tile_start[p.E + p.S];
  if (y >= n || v.z <= 0) return false;
  ti.e = v.x;
  ti.r0 = v.y;
  ti.m = v.z;
  return true;
}

// Small batches: every wavefront finds tile `y` of the grouping on its own,
// with no block barrier, so the weights of the tile can be requested right
// after the routing is read.  Per-expert pair counts by LDS atomics (lane e
// reads expert e's count), an exclusive scan over the expert lanes gives the
// segments and first tiles (shared expert s: segment T*k + s*T), a ballot
// finds the expert whose tiles hold y, and the tile's rows are that expert's
// pairs ranked by ballots in ascending pair order: the stable grouping.
struct alignas(16) SmallTiles {
  int cnt[kThreads / kWave][kWave];
  int rows[kThreads / kWave][kTileM];  // pair id (t*nslot + slot) of each tile row
  // top-k from router logits (T <= kLogitsMaxT)
  int ids[kLogitsMaxT * kMaxTopK];
  float gates[kLogitsMaxT * kMaxTopK];
  uint64_t keys[kThreads / kWave][kWave];
  float sel[kThreads / kWave][kMaxTopK];
};
// id loads per lane for up to kSmallT rows, and for the logits-routed batches
constexpr int kIdLoads = (kSmallT * kMaxTopK + kWave - 1) / kWave;
constexpr int kIdLoadsLogits = (kLogitsMaxT * kMaxTopK + kWave - 1) / kWave;

// Top-k of every row from the router logits: wavefront w takes rows w, w+4,
// ...; ids and gates go to LDS, and with write_record also to ids_out and
// gates_out.  Synchronises the block.
__device__ void small_top_k(const ExpertArgs &p, SmallTiles &st, bool write_record) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1), k = p.k;
  for (int t = w; t < p.T; t += kThreads / kWave)
    select_top_k<true>(p.logits + static_cast<size_t>(t) * 64, st.keys[w], st.sel[w], p.E, k, st.ids + t * k,
                       st.gates + t * k);
  __syncthreads();
  if (write_record && w == 0)
    for (int i = lane; i < p.T * k; i += kWave) {
      p.ids_out[i] = st.ids[i];
      p.gates_out[i] = st.gates[i];
    }
}

// Wavefront w reads the logits of rows w, w+4, ... (agent-scope loads) until
// none of the first E holds kLogitUnset, at most spin_limit polls (a wait
// that gives up records 1 in *err and goes on); with `select` it then takes
// their top-k as small_top_k does.  Synchronises the block.
__device__ void small_top_k_poll(const ExpertArgs &p, SmallTiles &st, bool select, bool write_record) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1), k = p.k;
  for (int t = w; t < p.T; t += kThreads / kWave) {
    const float *row = p.logits + static_cast<size_t>(t) * 64 + lane;
    float v = 0.f;
    for (int polls = 0;; ++polls) {
      v = ld_agent(row);
      if (!__ballot(lane < p.E && __float_as_uint(v) == kLogitUnset)) break;
      if (polls >= p.spin_limit) {
        if (lane == 0) st_agent(p.err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(64);
    }
    if (select) select_top_k_of(v, st.keys[w], st.sel[w], p.E, k, st.ids + t * k, st.gates + t * k);
  }
  __syncthreads();
  if (select && write_record && w == 0)
    for (int i = lane; i < p.T * k; i += kWave) {
      p.ids_out[i] = st.ids[i];
      p.gates_out[i] = st.gates[i];
    }
}

// routed_only: y counts routed tiles only.  NL: id loads per lane (T*k <= 64*NL).
template <int NL>
__device__ bool small_tile(const ExpertArgs &p, const int *ids, int y, TileInfo &ti, SmallTiles &st,
                           bool write_record, bool routed_only = false) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int E = p.E, S = p.S, k = p.k, T = p.T, np = T * k, ne = E + S;
  const uint64_t below = (1ull << lane) - 1ull;
  int v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) v[i] = ids[min(i * kWave + lane, np - 1)];
  int *cnt = st.cnt[w];
  cnt[lane] = 0;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    v[i] = min(max(v[i], 0), E - 1);  // ids are always in range; clamp defensively
    if (i * kWave + lane < np) atomicAdd(&cnt[v[i]], 1);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c = lane < E ? cnt[lane] : 0;
  const int tiles = (c + kTileM - 1) / kTileM;
  int sc = c, stl = tiles;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int vc = __shfl_up(sc, off), vt = __shfl_up(stl, off);
    if (lane >= off) { sc += vc; stl += vt; }
  }
  const int seg_e = sc - c, first_e = stl - tiles;
  const int routed_tiles = __builtin_amdgcn_readlane(stl, kWave - 1);
  const int shared_tiles = (T + kTileM - 1) / kTileM;
  if (write_record) {  // segment and tile tables of record, for the down kernel
    if (lane < E) {
      p.seg[lane] = seg_e;
      p.tile_start[lane] = first_e;
    }
    if (lane <= S) {
      p.seg[E + lane] = np + lane * T;
      p.tile_start[E + lane] = routed_tiles + lane * shared_tiles;
    }
  }
  if (y >= routed_tiles + (routed_only ? 0 : S * shared_tiles)) return false;
  int *rows = st.rows[w];
  if (y < routed_tiles) {
    const uint64_t hit = __ballot(lane < E && y >= first_e && y < first_e + tiles);
    const int e = static_cast<int>(__builtin_ctzll(hit));
    const int j = y - __builtin_amdgcn_readlane(first_e, e);
    ti.e = e;
    ti.r0 = __builtin_amdgcn_readlane(seg_e, e) + j * kTileM;
    ti.m = min(kTileM, __builtin_amdgcn_readlane(c, e) - j * kTileM);
    ti.j = j;
    int run = 0;  // pairs of expert e before this batch of 64
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = i * kWave + lane;
      const bool mine = q < np && v[i] == e;
      const uint64_t m = __ballot(mine);
      const int rr = run + __popcll(m & below) - j * kTileM;
      if (mine && rr >= 0 && rr < kTileM) rows[rr] = (q / k) * p.nslot + (q % k);
      run += __popcll(m);
    }
  } else {
    const int s = (y - routed_tiles) / shared_tiles, j = y - routed_tiles - s * shared_tiles;
    ti.e = E + s;
    ti.r0 = np + s * T + j * kTileM;
    ti.m = min(kTileM, T - j * kTileM);
    ti.j = j;
    if (lane < ti.m) rows[lane] = (j * kTileM + lane) * p.nslot + k + s;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return true;
}

// U: K-windows per weight batch.
template <typename T, int U = kUnroll>
__global__ __launch_bounds__(kThreads) void k_gate_up(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SmallTiles st;
  __shared__ float up_acc[2][64][4];
  constexpr int VN = Vec<T>::N;
  TileInfo ti;
  const bool small = p.group_in_block != 0;
  const bool first = blockIdx.x == 0 && blockIdx.y == 0;
  if (small ? !small_tile<kIdLoads>(p, p.ids, blockIdx.y, ti, st, first && threadIdx.x < kWave)
            : !table_tile(p, blockIdx.y, ti))
    return;
  // Slot pair of this block.  Blocks go to the eight XCDs round-robin in
  // launch order, so with gridDim.x slot pairs per tile, slot pair x of an
  // expert's tile j would land on an XCD shifted by gridDim.x * j (mod 8)
  // from its first tile's, and read the same weight slice through another
  // L2.  Rotating the slot pairs by that shift keeps every slice of an
  // expert on one XCD (but the few that wrap).
  const int shift = small ? static_cast<int>((gridDim.x * ti.j) & 7u) : 0;
  const int pair = (static_cast<int>(blockIdx.x) + shift) % static_cast<int>(gridDim.x);
  GateUpPart<T, U, true> part;  // two weight batches in flight (the x tile's LDS, not registers, bounds occupancy)
  part.begin(p, ti, pair, threadIdx.x);  // first weights in flight while x is staged

  const int d = p.d, nvec = d / VN, lda = d + VN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (small && blockIdx.x == 0 && w == 0) {  // this tile's entry of the grouping of record
    if (lane < ti.m) p.rows[ti.r0 + lane] = st.rows[0][lane];
    if (lane == 0) p.tile_info[blockIdx.y] = make_int4(ti.e, ti.r0, ti.m, 0);
  }
  T *A = reinterpret_cast<T *>(smem);
  const T *x = static_cast<const T *>(p.x);
  for (int it = threadIdx.x; it < kTileM * nvec; it += blockDim.x) {
    const int rr = it / nvec, c = it - rr * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < ti.m) {
      const int pair = small ? st.rows[w][rr] : p.rows[ti.r0 + rr];
      v = ld16(x + static_cast<size_t>(pair / p.nslot) * d + c * VN);
    }
    st16(A + rr * lda + c * VN, v);
  }
  __syncthreads();
  part.finish(p, ti, A + (lane & 15) * lda + (lane >> 4) * VN, up_acc, threadIdx.x);
}

template <typename T, int U = kUnroll>
__global__ __launch_bounds__(kThreads) void k_down(ExpertArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float half_acc[2][64][4];
  constexpr int VN = Vec<T>::N;
  TileInfo ti;
  if (!table_tile(p, blockIdx.y, ti)) return;
  DownPart<T, U> part;
  part.begin(p, ti, blockIdx.x, threadIdx.x);  // first weights in flight while a is staged
  stage_a_tile<T>(p, ti, reinterpret_cast<T *>(smem), threadIdx.x, blockDim.x);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  part.finish(p, ti, reinterpret_cast<const T *>(smem) + (lane & 15) * (p.F + VN) + (lane >> 4) * VN, half_acc,
              threadIdx.x, p.rows + ti.r0, p.gates);
}

// ------------------------------------------- gate/up and down in one launch
//
// Batches routed to logits (up to kLogitsMaxT rows) run a layer's gate/up
// and down in one launch.  The grid holds the gate/up blocks first, then the
// down blocks, each tile-major with the shared experts' tiles first (they
// need no routing); every other block takes the top-k and finds its tile
// itself.  A gate/up block writes its SiLU products with write-through
// stores and, once they have completed, counts itself on its tile's counter.
// A down block waits, without requesting anything else, until every gate/up
// block of its tile has counted; then it requests its weights and reads the
// products with agent-scope loads.  Every wait is for blocks of lower index
// (routing blocks, then gate/up blocks), which in-order dispatch places on
// the chip before the waiter, so with every waiter also resident the waits
// end.  Should a launch be starved (say, preempted), the waits are bounded:
// the result of that call is then wrong, and its status word says so.

// Thread 0 waits until *ctr >= target, for at most `limit` polls (about a
// microsecond each); a wait that gives up records 1 in *err (the call's
// status word, read back with mv_step_status) and the block goes on.  The
// caller synchronises the block afterwards.
__device__ __forceinline__ void wait_count(const unsigned *ctr, unsigned target, unsigned *err, int limit) {
  if (threadIdx.x != 0) return;
  unsigned n = 0;
  int polls = 0;
  while ((n = ld_agent(ctr)) < target && polls++ < limit)
    __builtin_amdgcn_s_sleep(64);
  if (n < target) st_agent(err, 1u);
}

// n_route > 0: the launch also routes this layer (ra, ca): its first n_route
// blocks (token, expert group) run route_fused, and the other blocks wait
// for them (shared gate/up blocks after requesting their first weights) by
// reading the logits until every one has landed (the one-launch step: on
// the routing counter).
// Block `vb` of the launch (blockIdx.x of k_ffn_small, or a virtual block of
// the one-launch step); kInLaunch: the one-launch step, where the routing's
// sources were written by blocks of the same launch and the slots are read by
// later blocks of it.
template <typename T, bool kInLaunch>
__device__ void ffn_small_block(const ExpertArgs &p, const RouteArgs &ra, const CombineArgs &ca, int max_tiles,
                                int n_route, int vb, unsigned char *smem, SmallTiles &st, float (*xacc)[64][4]) {
  constexpr int VN = Vec<T>::N;
  const int d = p.d, F = p.F, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (vb == 0) {  // the next launch's counters (this launch's were cleared before it started) and logits
    for (int i = tid; i < p.n_done; i += blockDim.x) p.done_next[static_cast<size_t>(i) * kDoneStride] = 0u;
    if (p.logits_next)
      for (int i = tid; i < p.T * 64; i += blockDim.x) p.logits_next[i] = __uint_as_float(kLogitUnset);
  }
  if (vb < n_route) {
    const int G = (p.E + kRouteGroup - 1) / kRouteGroup;
    route_fused<T, kInLaunch>(ra, ca, vb / G, vb % G, smem, p.route_done, kRouteCopies, kDoneStride);
    return;
  }
  const unsigned *route_ctr = p.route_done + static_cast<size_t>(vb % kRouteCopies) * kDoneStride;
  const int sp_gu = (F + 31) / 32, sp_dn = (d + 31) / 32;
  const int b0 = vb - n_route;
  const bool gu = b0 < sp_gu * max_tiles;
  const int b = gu ? b0 : b0 - sp_gu * max_tiles;
  const int sp = gu ? sp_gu : sp_dn, y = b / sp, pair = b - y * sp;
  // tiles [0, n_sh) are the shared experts' (all rows, no routing needed, so
  // their weights are requested at once); routed tiles follow
  const int shared_tiles = (p.T + kTileM - 1) / kTileM, n_sh = p.S * shared_tiles;
  const bool shared = y < n_sh;
  TileInfo ti;
  if (shared) {
    const int s = y / shared_tiles, j = y - s * shared_tiles;
    ti.e = p.E + s;
    ti.r0 = p.T * p.k + s * p.T + j * kTileM;
    ti.m = min(kTileM, p.T - j * kTileM);
    if (lane < ti.m) st.rows[w][lane] = (j * kTileM + lane) * p.nslot + p.k + s;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    const bool record = gu && y == n_sh && pair == 0;  // writes ids and gates of record
    if (n_route && !kInLaunch) {
      small_top_k_poll(p, st, true, record);
    } else {
      if (n_route) {
        wait_count(route_ctr, n_route, p.err, p.spin_limit);
        __syncthreads();
      }
      small_top_k(p, st, record);
    }
    if (!small_tile<kIdLoadsLogits>(p, st.ids, y - n_sh, ti, st, false, true)) return;
  }
  // LDS tile: rows [0, R) hold the tile's rows (R = min(T, 16) >= m), row R
  // is zero and stands in for the MFMA rows past m
  const int R = min(p.T, kTileM);
  T *A = reinterpret_cast<T *>(smem);
  const int arow = (lane & 15) < ti.m ? (lane & 15) : R;

  if (gu) {
    GateUpPart<T, kUnrollFused> part;
    part.begin(p, ti, pair, tid);
    if (shared && n_route) {  // x is written by this launch's routing blocks
      if constexpr (kInLaunch) {
        wait_count(route_ctr, n_route, p.err, p.spin_limit);
        __syncthreads();
      } else {
        small_top_k_poll(p, st, false, false);  // a row's logits land after its x
      }
    }
    const int nvec = d / VN, lda = d + VN;
    const T *x = static_cast<const T *>(p.x);
    for (int it = tid; it < (R + 1) * nvec; it += blockDim.x) {
      const int rr = it / nvec, c = it - rr * nvec;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < ti.m) {
        const T *src = x + static_cast<size_t>(st.rows[w][rr] / p.nslot) * d + c * VN;
        if (n_route) {
          const uint32_t *q = reinterpret_cast<const uint32_t *>(src);
          v.x = ld_agent(q);
          v.y = ld_agent(q + 1);
          v.z = ld_agent(q + 2);
          v.w = ld_agent(q + 3);
        } else {
          v = ld16(src);
        }
      }
      if (rr < ti.m || rr == R) st16(A + rr * lda + c * VN, v);
    }
    __syncthreads();
    part.template finish<true>(p, ti, A + arow * lda + (lane >> 4) * VN, xacc, tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's products have completed
    __syncthreads();
    if (tid == 0)
      add_agent(p.tile_done + y * kDoneStride, 1u);
    return;
  }

  // no weight requests before the tile is ready: the wait takes no bandwidth
  wait_count(p.tile_done + y * kDoneStride, static_cast<unsigned>(sp_gu), p.err, p.spin_limit);
  __syncthreads();
  DownPart<T, kUnrollFused> part;
  part.begin(p, ti, pair, tid, p.w_routed_down, p.w_shared_down);
  {  // the tile's products (agent-scope loads: written by this launch) and the zero row
    const int nvec = F / VN, lda = F + VN;
    const T *a = static_cast<const T *>(p.a);
    for (int it = tid; it < (R + 1) * nvec; it += blockDim.x) {
      const int rr = it / nvec, c = it - rr * nvec;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < ti.m) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(a + static_cast<size_t>(ti.r0 + rr) * F + c * VN);
        v.x = ld_agent(q);
        v.y = ld_agent(q + 1);
        v.z = ld_agent(q + 2);
        v.w = ld_agent(q + 3);
      }
      if (rr < ti.m || rr == R) st16(A + rr * lda + c * VN, v);
    }
  }
  __syncthreads();
  part.template finish<kInLaunch>(p, ti, A + arow * (F + VN) + (lane >> 4) * VN, xacc, tid, st.rows[w], st.gates);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_ffn_small(ExpertArgs p, RouteArgs ra, CombineArgs ca, int max_tiles,
                                                        int n_route) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SmallTiles st;
  __shared__ float xacc[2][64][4];
  ffn_small_block<T, false>(p, ra, ca, max_tiles, n_route, static_cast<int>(blockIdx.x), smem, st, xacc);
}

// ------------------------------------------------- one-launch verify step
//
// The verify step of a batch routed to logits as one launch.  Its launches
// become virtual blocks, numbered in launch order: per layer the fused
// launch's blocks (routing, gate/up, down; layer 0 routes inside it too),
// then one final-norm block per token, then the LM head's blocks, whose last
// one applies the accept rule.  Every wait is for virtual blocks of lower
// number: a layer's routing for every expert block of the previous layer
// (which also keeps each buffer the layers share from being overwritten while
// it is read), its expert blocks as in the fused launch, the final norm for
// the last layer, the LM head for the final norm.  Data another block of the
// launch reads is written through and read with agent-scope loads.  Per
// virtual block the arithmetic is that of the block it stands for
// (route_fused is route_block's in both modes), so results are bit-identical
// to the launches.
// One block: every layer's arguments from the shared ones and the layer's
// pointers; all blocks: the counters and the status word cleared.
__global__ __launch_bounds__(256) void k_one_launch_setup(OneLaunchArgs a, OneLaunchDev *dev, unsigned *status) {
  const size_t n = one_launch_counter_words(a.L, a.max_tiles);
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    a.ctr[i] = 0u;
  if (blockIdx.x != 0) return;
  if (threadIdx.x == 0) *status = 0u;
  const int l = threadIdx.x;
  if (l < a.L) {
    const StepLayer &sl = a.layer[l];
    unsigned *set = a.ctr + static_cast<size_t>(l) * a.set_lines * kDoneStride;
    OneLaunchLayer ly;
    ly.e = a.e;
    ly.e.w_routed = sl.gu;
    ly.e.w_shared = sl.sgu;
    ly.e.w_routed_down = sl.down;
    ly.e.w_shared_down = sl.sdown;
    ly.e.ids_out = sl.ids;
    ly.e.tile_done = set;
    ly.e.route_done = set + static_cast<size_t>(a.max_tiles) * kDoneStride;
    ly.r = a.r;
    ly.r.gamma = sl.norm;
    ly.r.router_w = sl.router;
    ly.r.router_b = sl.bias;
    ly.c = CombineArgs{sl.h_src, sl.h_dst, l ? a.slots : nullptr, nullptr};
    dev->layer[l] = ly;
  }
  if (threadIdx.x == 0) {
    dev->f = a.f;
    dev->fc = CombineArgs{a.h_last, a.h_final, a.slots, nullptr};
    dev->lm = a.lm;
  }
}

// Virtual blocks of the one-launch step.
template <typename T>
__device__ __forceinline__ void one_launch_layer_block(const OneLaunchLayer &ly, int max_tiles, int n_route,
                                                                int local, unsigned char *smem, SmallTiles &st,
                                                                float (*xacc)[64][4]) {
  ffn_small_block<T, true>(ly.e, ly.r, ly.c, max_tiles, n_route, local, smem, st, xacc);
}
template <typename T>
__device__ __forceinline__ void one_launch_final_block(const OneLaunchDev *dev, int t, unsigned char *smem,
                                                                unsigned *final_ctr) {
  route_fused<T, true, true>(dev->f, dev->fc, t, 0, smem, final_ctr, 1, kDoneStride);
}
template <typename T>
__device__ __forceinline__ void one_launch_lm_block(const LmArgs &p, int vblk, int n_lm, const unsigned *ready,
                                                             unsigned *err, int spin_limit, unsigned char *smem,
                                                             unsigned long long (*red)[kTileM]) {
  constexpr int VN = Vec<T>::N;
  const int tid = threadIdx.x, T_ = p.T, d = p.d;
  LmStream<T, true> ls;  // p is read from device memory
  ls.begin(p, vblk, tid);  // weights requested before x_f is ready
  wait_count(ready, static_cast<unsigned>(T_), err, spin_limit);
  __syncthreads();
  const int nvec = d / VN, lda = d + VN;
  T *A = reinterpret_cast<T *>(smem);  // rows [0, T) of x_f, then a zero row
  const T *xf = static_cast<const T *>(p.xf);
  for (int i = tid; i < (T_ + 1) * nvec; i += blockDim.x) {
    const int rr = i / nvec, cc = i - rr * nvec;
    st16(A + rr * lda + cc * VN,
         rr < T_ ? ld16_agent(xf + static_cast<size_t>(rr) * d + cc * VN) : make_uint4(0, 0, 0, 0));
  }
  __syncthreads();
  const int lane = tid & 63;
  const int arow = (lane & 15) < T_ ? (lane & 15) : T_;
  ls.finish(p, 0, T_, A + arow * lda + (lane >> 4) * VN, red, tid);
  lm_block_done(p, static_cast<unsigned>(n_lm));
}

// The step kernel: one hardware block per virtual block, in virtual-block
// order.  The hardware hands a launch's blocks out in increasing order and
// every wait is for lower-numbered blocks, so the lowest unfinished block has
// been dispatched and has every input (the fused launch's argument): the
// launch cannot deadlock, and its waits are bounded as in the fused launch.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_one_launch(const OneLaunchDev *__restrict__ dev, int L, int T_,
                                                       int n_route, int n_expert, int max_tiles, int n_lm,
                                                       int set_lines, unsigned *ctr, unsigned *err, int spin_limit) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SmallTiles st;
  __shared__ float xacc[2][64][4];
  __shared__ unsigned long long red[kLmWaves][kTileM];
  const int per_layer = n_route + n_expert;
  const int n_layers_vb = L * per_layer;
  unsigned *final_ctr = ctr + static_cast<size_t>(L) * set_lines * kDoneStride;
  const int vb = static_cast<int>(blockIdx.x);
  if (vb < n_layers_vb) {
    const int l = vb / per_layer, local = vb - l * per_layer;
    unsigned *done_l = ctr + (static_cast<size_t>(l) * set_lines + max_tiles + kRouteCopies) * kDoneStride;
    if (local < n_route && l > 0) {  // the previous layer's expert blocks have finished
      wait_count(done_l - static_cast<size_t>(set_lines) * kDoneStride, static_cast<unsigned>(n_expert), err,
                 spin_limit);
      __syncthreads();
    }
    one_launch_layer_block<T>(dev->layer[l], max_tiles, n_route, local, smem, st, xacc);
    if (local >= n_route) {  // count this expert block of layer l
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // its slots have completed
      __syncthreads();
      if (threadIdx.x == 0) add_agent(done_l, 1u);
    }
    return;
  }
  if (vb < n_layers_vb + T_) {  // final combine and norm of one token
    wait_count(final_ctr - static_cast<size_t>(set_lines - max_tiles - kRouteCopies) * kDoneStride,
               static_cast<unsigned>(n_expert), err, spin_limit);
    __syncthreads();
    one_launch_final_block<T>(dev, vb - n_layers_vb, smem, final_ctr);
    return;
  }
  one_launch_lm_block<T>(dev->lm, vb - n_layers_vb - T_, n_lm, final_ctr, err, spin_limit, smem, red);
}

// ------------------------------------------------------------ medium batches
//
// Tiles of up to MT * 16 rows of one expert and one wavefront per
// kMidSlices 16-column slices of the output: the block stages the tile's A
// rows through LDS one batch of kMidWin windows at a time and each
// wavefront uses its A fragments for all of its slices, so every weight row
// is read once per tile instead of once per 16 rows.  Loads run one batch
// ahead of the MFMAs.  Per-row arithmetic is the 16-row
// kernels': gate and up each one MFMA chain over K in window order; down two
// chains over the K halves, added low half first.
constexpr int kMidWin = 2;
constexpr int kMidSlices = 2;  // 16-column weight slices per wavefront, sharing its A fragments

// acc[c][i] += A_i * B_c over windows [w_lo, w_hi) for NB weight streams.
// The block's 16 * MT A rows are staged through LDS one batch of kMidWin
// windows at a time: thread t loads 16 bytes of row t / 4 per window (srow:
// that row at this thread's 16-byte part) and every wavefront reads its
// fragments there, so a window costs one A load per lane instead of MT.
// Every wavefront of the block must call this with the same window range
// (one barrier per batch).
template <typename T, int MT>
constexpr int mid_lds_bytes() {
  return 2 * kMidWin * 16 * MT * (4 * Vec<T>::N * static_cast<int>(sizeof(T)) + 16);
}
template <typename T, int MT, int NB>
__device__ __forceinline__ void mid_chain(f32x4_t (*acc)[MT], const T *srow, const T *const *b, int w_lo,
                                          int w_hi, unsigned char *lds) {
  constexpr int WIN = 4 * Vec<T>::N, U = kMidWin;
  constexpr int RS = WIN * static_cast<int>(sizeof(T)) + 16;  // LDS row stride: one 16-byte pad
  constexpr int SLAB = 16 * MT * RS, BUF = U * SLAB;            // one window, one batch
  static_assert(16 * MT * 4 == kThreads, "one A row part per thread and window");
  const int tid = threadIdx.x, lane = tid & 63;
  unsigned char *wr = lds + (tid >> 2) * RS + (tid & 3) * 16;
  const unsigned char *rd = lds + (lane & 15) * RS + (lane >> 4) * 16;
  uint4 qb[2][NB][U], sa[U];
  // A parts first: staging them then waits for those loads only
  auto load = [&](int buf, int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) sa[u] = ld16(srow + min(w0 + u, w_hi - 1) * WIN);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = min(w0 + u, w_hi - 1);
#pragma unroll
      for (int c = 0; c < NB; ++c) qb[buf][c][u] = ld16(b[c] + w * WIN);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u) st16(wr + buf * BUF + u * SLAB, sa[u]);
  };
  // batch at w0 in buffer `buf` (registers and LDS), the next one requested
  // into the other buffer first; two batches per iteration keep `buf` a
  // compile-time index, so that both register buffers stay in registers
  auto step = [&](int buf, int w0) {
    const bool more = w0 + U < w_hi;
    if (more) load(buf ^ 1, w0 + U);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (w0 + u < w_hi) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const uint4 a = ld16(rd + buf * BUF + u * SLAB + i * 16 * RS);
#pragma unroll
          for (int c = 0; c < NB; ++c) mfma16(acc[c][i], a, qb[buf][c][u], T());
        }
      }
    if (more) stage(buf ^ 1);
    __syncthreads();  // the other buffer is staged; this one is free again
  };
  if (w_lo >= w_hi) return;
  load(0, w_lo);
  stage(0);
  __syncthreads();
  for (int w0 = w_lo; w0 < w_hi; w0 += 2 * U) {
    step(0, w0);
    if (w0 + U < w_hi) step(1, w0 + U);
  }
}

template <typename T, int MT>
__global__ __launch_bounds__(kThreads) void k_gate_up_mid(ExpertArgs p) {
  constexpr int VN = Vec<T>::N, WIN = 4 * VN;
  TileInfo ti;
  if (!table_tile(p, blockIdx.y, ti)) return;
  const int e = ti.e, r0 = ti.r0, m = ti.m;
  const int d = p.d, F = p.F;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __shared__ __align__(16) unsigned char lds[mid_lds_bytes<T, MT>()];
  const int f0 = (blockIdx.x * (kThreads / kWave) + wv) * 16 * kMidSlices;
  // a wavefront past F (F % 64 == 0: all of its slices are) streams the last
  // slices again for the block's barriers and stores nothing
  const int fw = min(f0, F - 16 * kMidSlices);
  const int r = lane & 15, koff = (lane >> 4) * VN;
  const T *W = expert_base<T>(p, e, static_cast<size_t>(2) * F * d);
  const T *b[2 * kMidSlices];  // [slice][gate | up]
#pragma unroll
  for (int c = 0; c < kMidSlices; ++c) {
    b[2 * c] = W + static_cast<size_t>(fw + 16 * c + r) * d + koff;
    b[2 * c + 1] = W + static_cast<size_t>(F + fw + 16 * c + r) * d + koff;
  }
  const T *x = static_cast<const T *>(p.x);
  const int srow_i = threadIdx.x >> 2;  // this thread's staging row and part
  const int spair = p.rows[r0 + (srow_i < m ? srow_i : 0)];
  const T *srow = x + static_cast<size_t>(spair / p.nslot) * d + (threadIdx.x & 3) * VN;
  f32x4_t acc[2 * kMidSlices][MT];  // [slice][gate | up][tile]
#pragma unroll
  for (int c = 0; c < 2 * kMidSlices; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[c][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  mid_chain<T, MT, 2 * kMidSlices>(acc, srow, b, 0, d / WIN, lds);
  if (f0 >= F) return;
  T *aout = static_cast<T *>(p.a_out);
#pragma unroll
  for (int c = 0; c < kMidSlices; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = i * 16 + (lane >> 4) * 4 + j;
        if (row < m) {
          const float gv = acc[2 * c][i][j], uv = acc[2 * c + 1][i][j];
          aout[static_cast<size_t>(r0 + row) * F + f0 + 16 * c + r] = from_f32<T>(gv / (1.0f + expf(-gv)) * uv);
        }
      }
    }
}

template <typename T, int MT>
__global__ __launch_bounds__(kThreads) void k_down_mid(ExpertArgs p) {
  constexpr int VN = Vec<T>::N, WIN = 4 * VN;
  TileInfo ti;
  if (!table_tile(p, blockIdx.y, ti)) return;
  const int e = ti.e, r0 = ti.r0, m = ti.m;
  const int d = p.d, F = p.F;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __shared__ __align__(16) unsigned char lds[mid_lds_bytes<T, MT>()];
  const int n0 = (blockIdx.x * (kThreads / kWave) + wv) * 16 * kMidSlices;
  const int nw = min(n0, d - 16 * kMidSlices);  // past d (d % 64 == 0): the last slices again, no stores
  const int r = lane & 15, koff = (lane >> 4) * VN;
  const T *b[kMidSlices];
#pragma unroll
  for (int c = 0; c < kMidSlices; ++c)
    b[c] = expert_base<T>(p, e, static_cast<size_t>(d) * F) + static_cast<size_t>(nw + 16 * c + r) * F + koff;
  const T *a = static_cast<const T *>(p.a);
  const int srow_i = threadIdx.x >> 2;  // this thread's staging row and part
  const T *srow = a + static_cast<size_t>(r0 + (srow_i < m ? srow_i : 0)) * F + (threadIdx.x & 3) * VN;
  f32x4_t lo[kMidSlices][MT], hi[kMidSlices][MT];
#pragma unroll
  for (int c = 0; c < kMidSlices; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      lo[c][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      hi[c][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  const int nwin = F / WIN;
  mid_chain<T, MT, kMidSlices>(lo, srow, b, 0, nwin / 2, lds);
  mid_chain<T, MT, kMidSlices>(hi, srow, b, nwin / 2, nwin, lds);
  if (n0 >= d) return;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = i * 16 + (lane >> 4) * 4 + j;
      if (row < m) {
        const int pair = p.rows[r0 + row];
        const int tok = pair / p.nslot, s = pair - tok * p.nslot;
        const float w = s < p.k ? p.gates[tok * p.k + s] : 1.0f;
#pragma unroll
        for (int c = 0; c < kMidSlices; ++c)
          p.slots[static_cast<size_t>(pair) * d + n0 + 16 * c + r] = w * (lo[c][i][j] + hi[c][i][j]);
      }
    }
  }
}

template <typename KernelT>
void allow_lds(KernelT kernel, size_t bytes) {
  if (bytes > 48 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

template <int U>
hipError_t launch_gate_up_u(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.F + 31) / 32, max_tiles);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t smem = kTileM * (a.d + 16 / es) * es;
  if (dtype == 1) {
    allow_lds(k_gate_up<bf16_t, U>, smem);
    hipLaunchKernelGGL((k_gate_up<bf16_t, U>), grid, dim3(kThreads), smem, s, a);
  } else {
    allow_lds(k_gate_up<float, U>, smem);
    hipLaunchKernelGGL((k_gate_up<float, U>), grid, dim3(kThreads), smem, s, a);
  }
  return hipGetLastError();
}

template <int U>
hipError_t launch_down_u(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.d + 31) / 32, max_tiles);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t smem = kTileM * (a.F + 16 / es) * es;
  if (dtype == 1) {
    allow_lds(k_down<bf16_t, U>, smem);
    hipLaunchKernelGGL((k_down<bf16_t, U>), grid, dim3(kThreads), smem, s, a);
  } else {
    allow_lds(k_down<float, U>, smem);
    hipLaunchKernelGGL((k_down<float, U>), grid, dim3(kThreads), smem, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  return launch_gate_up_u<kUnroll>(dtype, a, max_tiles, s);
}

hipError_t launch_down(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  return launch_down_u<kUnroll>(dtype, a, max_tiles, s);
}

hipError_t launch_ffn_small(int dtype, const ExpertArgs &a, const RouteArgs *ra, const CombineArgs *ca, int max_tiles,
                            hipStream_t s) {
  if (!a.logits || a.T > kLogitsMaxT || !a.tile_done || !a.route_done || !a.done_next || !a.err ||
      !a.w_routed_down)
    return hipErrorInvalidValue;
  if (ra && (ra->mode != kLogits || ra->logits != a.logits)) return hipErrorInvalidValue;
  const int n_route = ra ? a.T * ((a.E + kRouteGroup - 1) / kRouteGroup) : 0;
  const dim3 grid(n_route + ((a.F + 31) / 32 + (a.d + 31) / 32) * max_tiles);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t rows = (a.T < kTileM ? a.T : kTileM) + 1;  // the tile's rows and a zero row
  size_t smem = rows * ((a.d > a.F ? a.d : a.F) + 16 / es) * es;
  if (ra) {
    const size_t route = route_smem(1, a.d, static_cast<int>(es)).total;
    smem = smem > route ? smem : route;
  }
  const RouteArgs r0 = ra ? *ra : RouteArgs{};
  const CombineArgs c0 = ca ? *ca : CombineArgs{};
  if (dtype == 1) {
    allow_lds(k_ffn_small<bf16_t>, smem);
    hipLaunchKernelGGL(k_ffn_small<bf16_t>, grid, dim3(kThreads), smem, s, a, r0, c0, max_tiles, n_route);
  } else {
    allow_lds(k_ffn_small<float>, smem);
    hipLaunchKernelGGL(k_ffn_small<float>, grid, dim3(kThreads), smem, s, a, r0, c0, max_tiles, n_route);
  }
  return hipGetLastError();
}

size_t one_launch_smem(int dtype, int T, int d, int F) {
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t rows = (T < kTileM ? T : kTileM) + 1;
  size_t smem = rows * ((d > F ? d : F) + 16 / es) * es;  // fused expert blocks and the LM head's x_f rows
  const size_t route = route_smem(1, d, static_cast<int>(es)).total;
  return smem > route ? smem : route;
}

hipError_t launch_one_launch(int dtype, const OneLaunchArgs &a, OneLaunchDev *dev, unsigned *status, size_t smem,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_one_launch_setup, dim3(16), dim3(256), 0, s, a, dev, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_expert = ((a.e.F + 31) / 32 + (a.e.d + 31) / 32) * a.max_tiles;
  const int T = a.e.T, total = a.L * (a.n_route + n_expert) + T + a.n_lm;
  if (dtype == 1) {
    allow_lds(k_one_launch<bf16_t>, smem);
    hipLaunchKernelGGL(k_one_launch<bf16_t>, dim3(total), dim3(kThreads), smem, s, dev, a.L, T, a.n_route, n_expert,
                       a.max_tiles, a.n_lm, a.set_lines, a.ctr, a.e.err, a.e.spin_limit);
  } else {
    allow_lds(k_one_launch<float>, smem);
    hipLaunchKernelGGL(k_one_launch<float>, dim3(total), dim3(kThreads), smem, s, dev, a.L, T, a.n_route, n_expert,
                       a.max_tiles, a.n_lm, a.set_lines, a.ctr, a.e.err, a.e.spin_limit);
  }
  return hipGetLastError();
}

}  // namespace mv

namespace mv {

hipError_t launch_gate_up_mid(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.F + 64 * kMidSlices - 1) / (64 * kMidSlices), max_tiles);
  if (dtype == 1)
    hipLaunchKernelGGL((k_gate_up_mid<bf16_t, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_gate_up_mid<float, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_mid(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s) {
  const dim3 grid((a.d + 64 * kMidSlices - 1) / (64 * kMidSlices), max_tiles);
  if (dtype == 1)
    hipLaunchKernelGGL((k_down_mid<bf16_t, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_down_mid<float, kMidTiles>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mv
