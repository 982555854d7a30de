// Host-side interface between the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mv {

// Rows of one expert tile of the grouped expert kernels.
constexpr int kTileM = 16;

enum PrologueMode {
  kRoute = 0,    // [combine] -> RMSNorm -> router -> top-k (+ permute if one block)
  kFinal = 1,    // combine -> final RMSNorm -> x_f; clears the argmax keys
  kCombine = 2,  // combine only: h_out = h + y
};

struct PrologueArgs {
  int T, d, E, S, k, nslot, mode, tile_m;
  float eps;
  const void *h_src;       // [T, d] residual input
  void *h_dst;             // [T, d] (h_src + y) or copy of h_src; may be null
  const float *slots;      // [T*nslot, d] previous layer's expert outputs; null: no combine
  float *y_moe;            // [T, d] fp32 sum of slots (optional)
  const void *gamma;       // [d]
  void *x_out;             // [T, d]
  const void *router_w;    // [E, d]
  const float *router_b;   // [E] or null
  int *ids;                // [T, k]
  float *gates;            // [T, k]
  unsigned long long *argkey;  // [T], cleared in kFinal mode
  int *seg;                // [E+S+1] row offset of each expert segment
  int *tile_start;         // [E+S+1] first tile of each expert
  int *rows;               // [T*nslot] pair id of each sorted row
};

struct ExpertArgs {
  int T, d, F, E, S, k, nslot;
  const void *x;           // [T, d] normalised layer input
  const void *a;           // [T*nslot, F] SwiGLU products, sorted-row order
  void *a_out;
  const void *w_routed;    // this layer's routed block: [E, 2F, d] or [E, d, F]
  const void *w_shared;    // this layer's shared block: [S, 2F, d] or [S, d, F]
  const int *seg, *tile_start, *rows;
  const float *gates;      // [T, k]
  float *slots;            // [T*nslot, d]
};

struct LmArgs {
  int T, d, V;
  const void *xf;          // [T, d]
  const void *w;           // [V, d]
  unsigned long long *argkey;  // [T]
};

struct AcceptArgs {
  int B, K;
  const unsigned long long *argkey;  // [B*(K+1)] packed keys, or null
  const int *argmax_in;              // used when argkey is null
  int *argmax_out;                   // may be null
  const int *drafts;                 // [B, K]
  int *n_acc, *committed, *n_com;
};

// dtype-dispatched launchers (dtype: 0 fp32, 1 bf16); return the launch error.
hipError_t launch_prologue(int dtype, const PrologueArgs &a, hipStream_t s);
hipError_t launch_permute(const PrologueArgs &a, hipStream_t s);
hipError_t launch_gate_up(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_down(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_lm_argmax(int dtype, const LmArgs &a, hipStream_t s);
hipError_t launch_accept(const AcceptArgs &a, hipStream_t s);

// Tokens handled by one prologue block (one wavefront per token).
constexpr int kPrologueTokens = 4;

}  // namespace mv
