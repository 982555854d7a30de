// Row kernels of the FastMTP draft block: one dense block whose parameters
// are shared by every draft position, fed by the decoder's last hidden state
// and the token that follows it, drafting through the decoder's own LM head
// (FastMTP paragraph of "Jina AI Releases jina-ocr-v1, a 3.4B MoE Document
// Parser With Built-In Speculative Decoding", ainewsfeed.tech).  The
// projection and the dense SwiGLU FFN run on the 16-row expert-tile kernels
// (k_gate_up, k_down) with a one-expert tile table; the LM head is the
// verify step's.  These kernels do the per-row work in between, one block of
// 256 threads per sequence:
//
//   k_mtp_in    token (the input token, or the previous draft from the LM
//               head's argmax key, which it also records and clears),
//               u = [R(RMSNorm(h) * g_h) ; R(RMSNorm(E[t]) * g_e)]
//   k_mtp_mid   h1 = R(z), x = R(RMSNorm(h1) * g_ffn)       (z = u W_proj^T)
//   k_mtp_out   h2 = R(h1 + y), x_o = R(RMSNorm(h2) * g_out) (y = FFN(x))
//   k_mtp_last  the last draft from the LM head's argmax key
//
// The sum of squares of a row is taken per 16-byte chunk in order, then over
// the chunks as in the verify step's RMSNorm.
#include "mv_common.h"
#include "mv_internal.h"

namespace mv {

namespace {

constexpr int kRowThreads = 256;

// 1/rms of a row of d values produced by `val(chunk, out)` (VN values per
// chunk), computed by the whole block; `part` is LDS of d / VN floats.
template <int VN, typename F>
__device__ __forceinline__ float block_inv_rms(int d, float eps, float *part, float *inv, F val) {
  const int nvec = d / VN, tid = threadIdx.x, lane = tid & 63;
  for (int ch = tid; ch < nvec; ch += blockDim.x) {
    float v[VN];
    val(ch, v);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VN; ++i) s += v[i] * v[i];
    part[ch] = s;
  }
  __syncthreads();
  if (tid < kWave) {
    float acc = 0.f;
    for (int ch = lane; ch < nvec; ch += kWave) acc += part[ch];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) *inv = 1.0f / sqrtf(acc / static_cast<float>(d) + eps);
  }
  __syncthreads();
  return *inv;
}

// dst[0..d) = R((v * inv) * gamma), v from `val`.
template <typename T, typename F>
__device__ __forceinline__ void store_normed(int d, float inv, const T *gamma, T *dst, F val) {
  constexpr int VN = Vec<T>::N;
  for (int ch = threadIdx.x; ch < d / VN; ch += blockDim.x) {
    float v[VN], g[VN], o[VN];
    val(ch, v);
    unpack(ld16(gamma + ch * VN), g, T());
#pragma unroll
    for (int i = 0; i < VN; ++i) o[i] = round_to<T>((v[i] * inv) * g[i]);
    st16(dst + ch * VN, pack(o, T()));
  }
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_in(MtpArgs a, int step) {
  constexpr int VN = Vec<T>::N;
  __shared__ float part[kMtpMaxD / 4];
  __shared__ float inv[2];
  __shared__ int tok;
  const int b = blockIdx.x, d = a.d;
  if (threadIdx.x == 0) {
    int t;
    if (step == 0) {
      t = a.tokens[b];
    } else {
      t = static_cast<int>(key_index(a.argkey[b]));
      a.drafts[static_cast<size_t>(b) * a.K + step - 1] = t;
    }
    a.argkey[b] = 0ull;  // for this step's LM head
    tok = min(max(t, 0), a.V - 1);
    a.rows[b] = b;  // the one-expert tile table of the dense kernels
    if (b == 0) {
      const int ntiles = (a.B + kTileM - 1) / kTileM;
      a.tile_start[0] = 0;
      a.tile_start[1] = ntiles;
      for (int y = 0; y < ntiles; ++y) a.tile_info[y] = make_int4(0, y * kTileM, min(kTileM, a.B - y * kTileM), 0);
    }
  }
  __syncthreads();
  const T *h = static_cast<const T *>(step == 0 ? a.h_in : a.h_cur) + static_cast<size_t>(b) * d;
  const T *e = static_cast<const T *>(a.embed) + static_cast<size_t>(tok) * d;
  T *u = static_cast<T *>(a.u) + static_cast<size_t>(b) * 2 * d;
  auto hv = [&](int ch, float *v) { unpack(ld16(h + ch * VN), v, T()); };
  auto ev = [&](int ch, float *v) { unpack(ld16(e + ch * VN), v, T()); };
  const float ih = block_inv_rms<VN>(d, a.eps, part, inv, hv);
  store_normed<T>(d, ih, static_cast<const T *>(a.norm_h), u, hv);
  const float ie = block_inv_rms<VN>(d, a.eps, part, inv + 1, ev);
  store_normed<T>(d, ie, static_cast<const T *>(a.norm_e), u + d, ev);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_mid(MtpArgs a) {
  constexpr int VN = Vec<T>::N;
  __shared__ float part[kMtpMaxD / 4];
  __shared__ float inv;
  const int b = blockIdx.x, d = a.d;
  const float *z = a.acc + static_cast<size_t>(b) * d;
  T *h1 = static_cast<T *>(a.h1) + static_cast<size_t>(b) * d;
  auto hv = [&](int ch, float *v) {  // h1 = R(z), recomputed from z on each pass
    float q[VN];
    ld_f32<4>(z + ch * VN, q);
    if (VN == 8) ld_f32<4>(z + ch * VN + 4, q + 4);
#pragma unroll
    for (int i = 0; i < VN; ++i) v[i] = round_to<T>(q[i]);
  };
  for (int ch = threadIdx.x; ch < d / VN; ch += blockDim.x) {
    float v[VN];
    hv(ch, v);
    st16(h1 + ch * VN, pack(v, T()));
  }
  const float ix = block_inv_rms<VN>(d, a.eps, part, &inv, hv);
  store_normed<T>(d, ix, static_cast<const T *>(a.norm_ffn), static_cast<T *>(a.x) + static_cast<size_t>(b) * d, hv);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_mtp_out(MtpArgs a, int last) {
  constexpr int VN = Vec<T>::N;
  __shared__ float part[kMtpMaxD / 4];
  __shared__ float inv;
  const int b = blockIdx.x, d = a.d;
  const float *y = a.acc + static_cast<size_t>(b) * d;
  const T *h1 = static_cast<const T *>(a.h1) + static_cast<size_t>(b) * d;
  auto hv = [&](int ch, float *v) {  // h2 = R(h1 + y)
    float q[VN];
    ld_f32<4>(y + ch * VN, q);
    if (VN == 8) ld_f32<4>(y + ch * VN + 4, q + 4);
    unpack(ld16(h1 + ch * VN), v, T());
#pragma unroll
    for (int i = 0; i < VN; ++i) v[i] = round_to<T>(v[i] + q[i]);
  };
  T *hc = static_cast<T *>(a.h_cur) + static_cast<size_t>(b) * d;
  T *ho = last && a.h_out ? static_cast<T *>(a.h_out) + static_cast<size_t>(b) * d : nullptr;
  for (int ch = threadIdx.x; ch < d / VN; ch += blockDim.x) {
    float v[VN];
    hv(ch, v);
    const uint4 pk = pack(v, T());
    st16(hc + ch * VN, pk);
    if (ho) st16(ho + ch * VN, pk);
  }
  const float io = block_inv_rms<VN>(d, a.eps, part, &inv, hv);
  store_normed<T>(d, io, static_cast<const T *>(a.norm_out), static_cast<T *>(a.xo) + static_cast<size_t>(b) * d, hv);
}

__global__ void k_mtp_last(MtpArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < a.B) a.drafts[static_cast<size_t>(b) * a.K + a.K - 1] = static_cast<int>(key_index(a.argkey[b]));
}

template <typename KernelT>
hipError_t launch_rows(KernelT kernel, const MtpArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(kernel, dim3(a.B), dim3(kRowThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mtp_in(int dtype, const MtpArgs &a, int step, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(k_mtp_in<bf16_t>, dim3(a.B), dim3(kRowThreads), 0, s, a, step);
  else
    hipLaunchKernelGGL(k_mtp_in<float>, dim3(a.B), dim3(kRowThreads), 0, s, a, step);
  return hipGetLastError();
}

hipError_t launch_mtp_mid(int dtype, const MtpArgs &a, hipStream_t s) {
  return dtype == 1 ? launch_rows(k_mtp_mid<bf16_t>, a, s) : launch_rows(k_mtp_mid<float>, a, s);
}

hipError_t launch_mtp_out(int dtype, const MtpArgs &a, int last, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(k_mtp_out<bf16_t>, dim3(a.B), dim3(kRowThreads), 0, s, a, last);
  else
    hipLaunchKernelGGL(k_mtp_out<float>, dim3(a.B), dim3(kRowThreads), 0, s, a, last);
  return hipGetLastError();
}

hipError_t launch_mtp_last(const MtpArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_mtp_last, dim3((a.B + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mv
