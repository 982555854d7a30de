// Host-side interface between the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mv {

// Rows of one expert tile of the grouped expert kernels, and tokens of one
// routing tile.
constexpr int kTileM = 16;
// Up to this many token rows a step takes the small-batch path: every gate/up
// block finds its tile from the routing itself instead of a separate
// grouping kernel.
constexpr int kSmallT = 128;
// Batches of more than kMidMinT rows: expert tiles of up to kMidRows rows,
// each weight row streamed once per tile (up to kMidMinT rows, 16-row tiles
// with more wavefronts in flight stream faster).
constexpr int kMidMinT = 128;
// bf16 batches of more than kLargeMinT rows: LDS-tiled MFMA GEMMs.
constexpr int kLargeMinT = 512;
constexpr int kMidTiles = 4;
constexpr int kMidRows = 16 * kMidTiles;
// Largest expert count (routed + shared) and slots per token supported.
constexpr int kMaxExperts = 64 + 4;
constexpr int kMaxSlots = 8 + 4;
constexpr int kMaxTopK = 8;

enum RouteMode {
  kRoute = 0,    // RMSNorm -> router -> top-k (-> permutation)
  kFinal = 1,    // final RMSNorm -> x_f; clears the argmax keys
  kCombine = 2,  // combine only
  kLogits = 3,   // RMSNorm -> router logits of one group of experts per block;
                 // the top-k is left to the small-batch gate/up kernel
};
// Experts per routing block in kLogits mode, and the largest batch that
// routes that way (every gate/up block then takes the top-k of all rows).
constexpr int kRouteGroup = 16;
constexpr int kLogitsMaxT = 8;  // measured: at 16 rows separate launches are 18% faster
// Per-tile counters of the fused expert launch, one per 256-byte line so
// that polls of different tiles do not meet in one memory channel.
constexpr int kDoneStride = 64;
// Copies of a layer's routing counter in the one-launch step, so that its
// many waiting blocks spread their polls over that many lines (the fused
// expert launch's blocks read the logits themselves as they land).
constexpr int kRouteCopies = 32;
// Polls (about a microsecond each) a fused-launch wait makes before it gives
// up and records the timeout in the call's status word.
constexpr int kSpinLimitDefault = 1 << 18;
// Bit pattern of a router logit not yet written: a negative NaN with every
// payload bit set, which the routing arithmetic does not produce unless an
// input holds it.  A fused launch that routes its own layer reads the logits
// as they land; the launch before it fills their buffer with this pattern.
constexpr uint32_t kLogitUnset = 0xffffffffu;

struct RouteArgs {
  int T, d, E, S, k, nslot, mode;
  int tile_m;               // rows per expert tile of the grouping
  float eps;
  const void *gamma;        // [d]
  void *x_out;              // [T, d]
  const void *router_w;     // [E, d]
  const float *router_b;    // [E] or null
  int *ids;                 // [T, k]
  float *gates;             // [T, k]
  int *seg, *tile_start, *rows;
  int4 *tile_info;          // [max tiles] (expert, first row, rows, 0) per 16-row tile
  unsigned long long *argkey;  // kFinal: cleared
  unsigned *done;           // kFinal: cleared (the LM head's block count)
  float *logits;            // kLogits: [T, 64] fp32 router logits
  unsigned *tile_done;      // kLogits: counters [i * kDoneStride], i < n_tile_done, cleared for the fused expert launch
  int n_tile_done;
  unsigned *status;         // if set: block 0 clears the call's status word (first launch of a call)
};

// Combine of the previous layer's expert slots into the hidden state.
struct CombineArgs {
  const void *h_src;        // [T, d] residual input
  void *h_dst;              // [T, d] h_src + y (may alias h_src)
  const float *slots;       // [T*nslot, d]; null: no combine (h_dst unused)
  float *y_moe;             // [T, d] optional
};

struct ExpertArgs {
  int T, d, F, E, S, k, nslot;
  const void *x;           // [T, d] normalised layer input
  const void *a;           // [T*nslot, F] SwiGLU products, sorted-row order
  void *a_out;
  const void *w_routed;    // this layer's routed block: [E, 2F, d] or [E, d, F]
  const void *w_shared;    // this layer's shared block: [S, 2F, d] or [S, d, F]
  const int *ids;          // [T, k] routing (grouped in-block on the small path)
  int group_in_block;      // small path: gate/up groups the pairs (block (0,0) writes them)
  int *seg, *tile_start, *rows;
  int4 *tile_info;         // [max tiles] (expert, first row, rows, 0)
  const float *gates;      // [T, k]
  float *slots;            // [T*nslot, d]
  // kLogits routing (T <= kLogitsMaxT): the gate/up kernel takes the top-k of
  // these logits itself, and its block (0, 0) writes ids_out and gates_out
  const float *logits;     // [T, 64] or null
  int *ids_out;            // [T, k]
  float *gates_out;        // [T, k] (the down kernel's gates)
  const void *w_routed_down;  // fused launch: this layer's down blocks ([E, d, F] and [S, d, F])
  const void *w_shared_down;
  // fused launch: this launch's counters, one per 256-byte line (cleared
  // before it starts), and the next launch's, which it clears
  unsigned *tile_done;     // [tile * kDoneStride]: gate/up blocks done per tile
  unsigned *route_done;    // [copy * kDoneStride]: routing blocks done, kRouteCopies copies (one-launch step)
  unsigned *done_next;     // [i * kDoneStride], i < n_done
  int n_done;
  unsigned *err;           // the call's status word: set to 1 if a fused launch's wait gave up
  int spin_limit;          // polls before a fused launch's wait gives up
  // fused launch: the next layer's logits buffer ([T, 64]), which block 0
  // fills with kLogitUnset (null: none)
  float *logits_next;
};

struct AcceptArgs {
  int B, K;
  const unsigned long long *argkey;  // [B*(K+1)] packed keys, or null
  const int *argmax_in;              // used when argkey is null
  int *argmax_out;                   // may be null
  const int *drafts;                 // [B, K]
  int *n_acc, *committed, *n_com;
};

struct LmArgs {
  int T, d, V;
  const void *xf;          // [T, d]
  const void *w;           // [V, d]
  unsigned long long *argkey;  // [T]
  unsigned *done;          // if set: blocks finished (zeroed beforehand); the last one runs `accept`
  AcceptArgs accept;
};

// FastMTP draft block (k_mtp.hip).  Buffers are [B, ...] rows in the
// config dtype unless noted.
constexpr int kMtpMaxD = 4096;
// The projection and the FFN's gate/up and down split K into this many
// parts, one block each (enough blocks to stream from most of the chip);
// their readers add the fp32 partial outputs in part order.
constexpr int kMtpSplit = 2;
struct MtpArgs {
  int B, K, d, V;
  float eps;
  const int *tokens;             // [B] input tokens (position 0)
  unsigned long long *argkey;    // [2, B] LM-head argmax keys, by position parity
  int *drafts;                   // [B, K]
  const void *h_in;              // [B, d] position 0's hidden state
  void *h_cur;                   // [B, d] the block's output, next position's input
  void *h_out;                   // [B, d] or null: the last position's output
  const void *embed;             // [V, d]
  const void *norm_h, *norm_e, *norm_ffn, *norm_out;  // [d]
  float *acc;                    // [kMtpSplit, B, d] fp32 projection output z, partial over K
  float *acc2;                   // [kMtpSplit, B, d] fp32 FFN output y, partial over K
  float *gu;                     // [kMtpSplit, B, 2F] fp32 FFN gate and up, partial over K
  void *xo;                      // [B, d] LM-head input
  void *u;                       // [B, 2d] projection input (row-kernel path)
  void *x;                       // [B, d] FFN input (row-kernel path)
};
// Up to this many sequences the projection and gate/up kernels normalise
// their tiles themselves (at most one row per wavefront).
constexpr int kMtpFusedMaxB = 4;
// Up to this many sequences the LM head's blocks form the position's output
// rows themselves (at 4 each block's extra rows cost more than the launch).
constexpr int kMtpFoldMaxB = 3;
// Dynamic LDS of the projection and FFN kernels, bytes (es: element size).
size_t mtp_proj_lds(int d, int es);
size_t mtp_ffn_lds(int d, int F, int es);
// The launches of one draft position before its LM head; proj, gu and
// dn are one-expert arguments (E = 1, k = 0, nslot = 1) of the projection
// (F = 2d, slots = acc), the FFN gate/up (a_out) and the FFN down (slots = acc2).
hipError_t launch_mtp_position(int dtype, const ExpertArgs &proj, const ExpertArgs &gu, const ExpertArgs &dn,
                               const MtpArgs &a, int step, hipStream_t s);
hipError_t launch_mtp_last(const MtpArgs &a, hipStream_t s);
// The LM head of draft position `step` (la: keys of this position, no block
// counter); up to kMtpFoldMaxB sequences it also forms h2 and x_o, which
// launch_mtp_position then leaves to it.
hipError_t launch_mtp_lm(int dtype, const LmArgs &la, const MtpArgs &a, int step, hipStream_t s);

// One-launch verify step for batches routed to logits (k_expert.hip): the
// step's launches become the blocks of one launch.
// Per-layer pointers, and the arguments every layer shares (the per-layer
// fields of e and r are replaced from `layer`).
constexpr int kOneLaunchMaxLayers = 16;
struct StepLayer {
  const void *gu, *down, *sgu, *sdown, *norm, *router;
  const float *bias;
  int *ids;            // [T, k] top-k ids of record
  const void *h_src;   // the combine's residual input (layer 0: h_in, no combine)
  void *h_dst;         // the combine's output (layers >= 1)
};
struct OneLaunchArgs {
  ExpertArgs e;        // fused-launch arguments (n_done = 0: the counters are cleared before the launch)
  RouteArgs r;         // kLogits routing
  RouteArgs f;         // final norm: gamma, x_out (x_f), argkey
  LmArgs lm;           // LM head with the accept rule (done: its block counter)
  const float *slots;
  const void *h_last;  // residual input of the final combine
  void *h_final;       // its output (h_out)
  unsigned *ctr;       // counter lines: per layer [tiles | routing copies | experts done], then the final norm's and the LM head's
  int L, max_tiles, n_route, n_lm, set_lines;
  StepLayer layer[kOneLaunchMaxLayers];
};
// Counter words the one-launch step uses for L layers at max_tiles tiles.
__host__ __device__ inline size_t one_launch_counter_words(int L, int max_tiles) {
  return (static_cast<size_t>(L) * (max_tiles + kRouteCopies + 1) + 2) * kDoneStride;
}
// The arguments of every virtual block, written into the workspace by the
// setup kernel and read in place by the step kernel.
struct OneLaunchLayer {
  ExpertArgs e;
  RouteArgs r;
  CombineArgs c;
};
struct OneLaunchDev {
  OneLaunchLayer layer[kOneLaunchMaxLayers];
  RouteArgs f;
  CombineArgs fc;
  LmArgs lm;
};
size_t one_launch_smem(int dtype, int T, int d, int F);
// Setup (arguments into dev, counters and status word cleared), then the step.
hipError_t launch_one_launch(int dtype, const OneLaunchArgs &a, OneLaunchDev *dev, unsigned *status, size_t smem,
                             hipStream_t s);

// dtype-dispatched launchers (dtype: 0 fp32, 1 bf16); return the launch error.
hipError_t launch_route(int dtype, const RouteArgs &a, const CombineArgs &c, int ntok, hipStream_t s);
hipError_t launch_permute(const RouteArgs &a, hipStream_t s);
hipError_t launch_gate_up(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_down(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s);
// ra / ca: also route this layer inside the launch (kLogits), or null.
hipError_t launch_ffn_small(int dtype, const ExpertArgs &a, const RouteArgs *ra, const CombineArgs *ca, int max_tiles,
                            hipStream_t s);
hipError_t launch_gate_up_mid(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_down_mid(int dtype, const ExpertArgs &a, int max_tiles, hipStream_t s);
int gemm_tile_rows();
hipError_t launch_gemm_gate_up(const ExpertArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_gemm_down(const ExpertArgs &a, int max_tiles, hipStream_t s);
hipError_t launch_gemm_down_shared(const ExpertArgs &a, const CombineArgs &c, hipStream_t s);
int route_large_blocks(int T);
hipError_t launch_route_large(const RouteArgs &a, const void *h, int *blk_cnt, hipStream_t s);
hipError_t launch_lm_argmax(int dtype, const LmArgs &a, hipStream_t s);
hipError_t launch_accept(const AcceptArgs &a, hipStream_t s);
// status[0] = *word (int32), one thread.
hipError_t launch_copy_status(const unsigned *word, int32_t *status, hipStream_t s);

}  // namespace mv
