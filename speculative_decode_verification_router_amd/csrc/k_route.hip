// Per-token prologue of each MoE layer and the expert permutation.
//
// One wavefront per token row:
//   combine   h = round(h + sum_s slot[t, s])   (previous layer's experts,
//             routed slots in selection order, then the shared ones)
//   RMSNorm   x = round((h * (mean(h^2) + eps)^-1/2) * gamma)
//   router    l = x W_r^T (+ b), fp32
//   top-k     experts ordered by (logit desc, id asc); gates = softmax over
//             the k selected logits
// The routing follows the architecture paragraph of "Jina AI Releases
// jina-ocr-v1, a 3.4B MoE Document Parser With Built-In Speculative Decoding"
// (ainewsfeed.tech): 64 routed experts, top-6, two shared experts.
//
// The permutation is a stable counting sort of the T*k (token, slot) pairs
// by expert: a per-thread histogram over contiguous pair ranges, a scan in
// (expert, thread) order, then a scatter that keeps ascending pair order
// inside every expert segment.  Shared experts get one segment each holding
// every token.
#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

namespace {

// Sums the 64 per-lane partial vectors acc[0..63] across the wavefront so
// that lane e ends up with the full sum for entry e (recursive halving: each
// step trades the half a lane does not keep with its partner).
template <int N>
__device__ __forceinline__ void halve(float *acc, int lane) {
  const bool upper = (lane & N) != 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float send = upper ? acc[i] : acc[i + N];
    const float keep = upper ? acc[i + N] : acc[i];
    acc[i] = keep + __shfl_xor(send, N);
  }
}

__device__ __forceinline__ float transpose_reduce64(float *acc, int lane) {
  halve<32>(acc, lane);
  halve<16>(acc, lane);
  halve<8>(acc, lane);
  halve<4>(acc, lane);
  halve<2>(acc, lane);
  halve<1>(acc, lane);
  return acc[0];
}

// Stable counting sort of the routed pairs by expert; one block of 256.
__device__ void permute_block(const PrologueArgs &p, unsigned char *smem) {
  const int tid = threadIdx.x;
  const int E = p.E, S = p.S, k = p.k, T = p.T;
  const int stride = E + 2;  // u16 per thread row; odd dword stride avoids bank conflicts
  uint16_t *hist = reinterpret_cast<uint16_t *>(smem);            // [256][E+2]
  int *segl = reinterpret_cast<int *>(smem + 256 * stride * 2 + 16);  // [E+S+1]
  int *cnt = segl + (E + S + 1);                                   // [E]

  const int np = T * k;
  const int cp = (np + 255) / 256;
  const int p0 = min(np, tid * cp), p1 = min(np, p0 + cp);

  for (int e = 0; e < E; ++e) hist[tid * stride + e] = 0;
  for (int q = p0; q < p1; ++q) {
    const int e = min(max(p.ids[q], 0), E - 1);  // ids are always in range; clamp defensively
    hist[tid * stride + e] = hist[tid * stride + e] + 1;
  }
  __syncthreads();
  if (tid < E) {
    int s = 0;
    for (int i = 0; i < 256; ++i) s += hist[i * stride + tid];
    cnt[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, tiles = 0;
    for (int e = 0; e < E + S; ++e) {
      const int c = e < E ? cnt[e] : T;
      segl[e] = off;
      p.seg[e] = off;
      p.tile_start[e] = tiles;
      off += c;
      tiles += (c + p.tile_m - 1) / p.tile_m;
    }
    segl[E + S] = off;
    p.seg[E + S] = off;
    p.tile_start[E + S] = tiles;
  }
  __syncthreads();
  if (tid < E) {  // per expert: exclusive scan over threads (offsets within the segment)
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int c = hist[i * stride + tid];
      hist[i * stride + tid] = static_cast<uint16_t>(run);
      run += c;
    }
  }
  __syncthreads();
  for (int q = p0; q < p1; ++q) {
    const int e = min(max(p.ids[q], 0), E - 1);
    const int pos = segl[e] + hist[tid * stride + e];
    hist[tid * stride + e] = hist[tid * stride + e] + 1;
    p.rows[pos] = (q / k) * p.nslot + (q % k);
  }
  for (int j = tid; j < S * T; j += 256) {
    const int s = j / T, t = j % T;
    p.rows[segl[E + s] + t] = t * p.nslot + k + s;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_prologue(PrologueArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kPrologueTokens + wv;
  const int d = p.d, nvec = d / VN;
  float *row = reinterpret_cast<float *>(smem) + wv * d;

  if (t < p.T) {
    const T *src = static_cast<const T *>(p.h_src) + static_cast<size_t>(t) * d;
    T *dst = p.h_dst ? static_cast<T *>(p.h_dst) + static_cast<size_t>(t) * d : nullptr;
    float ss = 0.f;
    for (int c = lane; c < nvec; c += kWave) {
      float h[VN];
      unpack(ld16(src + c * VN), h, T());
      if (p.slots) {
        float y[VN];
#pragma unroll
        for (int i = 0; i < VN; ++i) y[i] = 0.f;
        for (int s = 0; s < p.nslot; ++s) {
          const float *sp = p.slots + (static_cast<size_t>(t) * p.nslot + s) * d + c * VN;
#pragma unroll
          for (int q = 0; q < VN; q += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(sp + q);
            y[q] += v.x; y[q + 1] += v.y; y[q + 2] += v.z; y[q + 3] += v.w;
          }
        }
        if (p.y_moe) {
          float *yp = p.y_moe + static_cast<size_t>(t) * d + c * VN;
#pragma unroll
          for (int q = 0; q < VN; q += 4)
            *reinterpret_cast<float4 *>(yp + q) = make_float4(y[q], y[q + 1], y[q + 2], y[q + 3]);
        }
#pragma unroll
        for (int i = 0; i < VN; ++i) h[i] = round_to<T>(h[i] + y[i]);
      }
      if (dst) st16(dst + c * VN, pack(h, T()));
#pragma unroll
      for (int i = 0; i < VN; ++i) {
        row[c * VN + i] = h[i];
        ss += h[i] * h[i];
      }
    }
    if (p.mode != kCombine) {
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + p.eps);
      const T *gam = static_cast<const T *>(p.gamma);
      T *xo = static_cast<T *>(p.x_out) + static_cast<size_t>(t) * d;
      for (int c = lane; c < nvec; c += kWave) {
        float g[VN], x[VN];
        unpack(ld16(gam + c * VN), g, T());
#pragma unroll
        for (int i = 0; i < VN; ++i) x[i] = round_to<T>((row[c * VN + i] * inv) * g[i]);
        st16(xo + c * VN, pack(x, T()));
#pragma unroll
        for (int i = 0; i < VN; ++i) row[c * VN + i] = x[i];
      }
      if (p.mode == kFinal && lane == 0) p.argkey[t] = 0ull;
    }
    if (p.mode == kRoute) {
      // router logits: lane-partial dot products for all experts, then a
      // transpose-reduction leaving expert `lane`'s logit on lane `lane`.
      float acc[64];
#pragma unroll
      for (int e = 0; e < 64; ++e) acc[e] = 0.f;
      const T *wr = static_cast<const T *>(p.router_w);
      for (int c = lane; c < nvec; c += kWave) {
        float x[VN];
#pragma unroll
        for (int i = 0; i < VN; ++i) x[i] = row[c * VN + i];
#pragma unroll
        for (int e0 = 0; e0 < 64; e0 += 16) {
          uint4 q[16];
#pragma unroll
          for (int e = 0; e < 16; ++e)
            q[e] = (e0 + e < p.E) ? ld16(wr + static_cast<size_t>(e0 + e) * d + c * VN)
                                  : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float w[VN];
            unpack(q[e], w, T());
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[e0 + e] += x[i] * w[i];
          }
        }
      }
      float logit = transpose_reduce64(acc, lane);
      if (p.router_b && lane < p.E) logit += p.router_b[lane];
      uint64_t key = lane < p.E ? argmax_key(logit, static_cast<uint32_t>(lane)) : 0ull;

      float vsel[8];
      int isel[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        vsel[s] = 0.f;
        isel[s] = 0;
        if (s < p.k) {
          uint64_t m = key;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) {
            const uint64_t other = shfl_xor_u64(m, o);
            m = other > m ? other : m;
          }
          const int e = static_cast<int>(key_index(m));
          vsel[s] = __shfl(logit, e);
          isel[s] = e;
          if (lane == e) key = 0ull;
        }
      }
      if (lane == 0) {
        float ex[8], den = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          ex[s] = s < p.k ? expf(vsel[s] - vsel[0]) : 0.f;
          den += ex[s];
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          if (s < p.k) {
            p.ids[t * p.k + s] = isel[s];
            p.gates[t * p.k + s] = ex[s] / den;
          }
        }
      }
    }
  }
  if (p.mode == kRoute && gridDim.x == 1) {
    __syncthreads();
    permute_block(p, smem);
  }
}

__global__ __launch_bounds__(256) void k_permute(PrologueArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  permute_block(p, smem);
}

size_t permute_smem(const PrologueArgs &a) {
  return 256 * static_cast<size_t>(a.E + 2) * 2 + 16 + 4 * static_cast<size_t>(2 * a.E + a.S + 1);
}

}  // namespace

hipError_t launch_prologue(int dtype, const PrologueArgs &a, hipStream_t s) {
  const int grid = (a.T + kPrologueTokens - 1) / kPrologueTokens;
  size_t smem = static_cast<size_t>(kPrologueTokens) * a.d * sizeof(float);
  if (a.mode == kRoute && grid == 1) smem = smem > permute_smem(a) ? smem : permute_smem(a);
  if (dtype == 1)
    hipLaunchKernelGGL(k_prologue<bf16_t>, dim3(grid), dim3(256), smem, s, a);
  else
    hipLaunchKernelGGL(k_prologue<float>, dim3(grid), dim3(256), smem, s, a);
  return hipGetLastError();
}

hipError_t launch_permute(const PrologueArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(256), permute_smem(a), s, a);
  return hipGetLastError();
}

}  // namespace mv
