// Internal interfaces between the C-ABI host code and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/megamoe.h"

namespace mm {

// Route numbering.  A token has K = Kr + S slots: its Kr routed top-k
// choices, then S (0 or 1) shared-expert slots; route r = i*K + k.  Experts
// 0 .. Er-1 are the routed ones, expert Er + s is shared expert s, which
// every active token visits with gate weight 1.
//
// Wavefront-to-route mapping shared by the count and scatter kernels: one
// wave owns floor(64/K) consecutive tokens (its lanes hold (token, slot)
// pairs, lane = t*K + k; the remaining lanes idle).
inline int tokens_per_wave(int K) { return 64 / K; }
inline int64_t dispatch_waves(int64_t T, int K) { return (T + tokens_per_wave(K) - 1) / tokens_per_wave(K); }
constexpr int kDispatchWavesPerBlock = 4;

struct DispatchArgs {
  const int32_t* topk_ids;   // [T][Kr]
  const int8_t* active;      // [T] x_active_mask (0: token inactive), or null (all active)
  const void* x;             // bf16 [T][H]
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E+1]
  int32_t* pool_src;         // [P]
  int32_t* route_to_pool;    // [T*K]
  void* x_pool;              // [P][H]
  float* x_pool_scale;       // [P] (A8W8)
  uint8_t* x_pool_mx;        // [P][H/32] E8M0 (MX use cases)
  int32_t* wave_base;        // ws: [waves][E]
  uint32_t* err;             // ws: device error word (mm_device_error bits)
  int64_t T, H, P;
  int E, K, block_m, usecase;
  int Er, Kr;                // routed experts and routed top-k (E = Er + S, K = Kr + S)
};

// Tile configurations of the grouped GEMMs (compile-time instances).
enum TileCfg : int {
  TILE_M64_N128 = 0,   // weight-streaming regime: few rows per expert
  TILE_M128_N256 = 1,  // compute regime
  TILE_M256_N256 = 2,  // compute regime, many rows per expert
  TILE_COUNT = 3
};
inline int tile_bm(int t) { return t == TILE_M64_N128 ? 64 : t == TILE_M128_N256 ? 128 : 256; }
inline int tile_bn(int t) { return t == TILE_M64_N128 ? 128 : 256; }

struct GemmArgs {
  const uint8_t* A;          // pool rows [P][Kdim]
  const uint8_t* B;          // prepared weights [E][N][Kdim]
  const int32_t* offsets;    // [E+1]
  const int32_t* counts;     // [E]
  const int32_t* pool_src;   // [P]
  int64_t P;                 // pool capacity (rows)
  int64_t routes;            // T*K
  uint32_t* err;             // device error word (mm_device_error bits)
  int E, N, Kdim, I, H, K;
  int Kr;                    // routed slots per token (slots Kr .. K-1: shared experts, gate weight 1)
  int gate_up_group;
  int group_m;               // M-blocks per tile group of an expert (0: all of them)
  // Linear1 (mode 0)
  const float* x_scale;      // [P] (A8W8)
  const float* w_scale;      // [E][N] formula order (A8W8)
  void* a_out;               // [P][I] bf16 (A16W16)
  float* a_stage;            // [P][I] f32 (A8W8)
  // Linear2 (mode 1)
  const float* a_scale;      // [P] (A8W8)
  const float* topk_w;       // [T][Kr]
  void* contrib;             // [T*K][H] float32 (A16W16) or bf16 (A8W8)
  // debug (mode 2: raw int32 accumulators)
  int32_t* raw_out;
  // MX use cases: E8M0 scales of the A rows [rows][Kdim/32] (a_mx_rows rows),
  // of the prepared B rows (formula order, [E][N][Kdim/32]); Linear1 writes
  // A's codes to a_out and their E8M0 scales to out_mx [P][I/32]
  const uint8_t* a_mx;
  int64_t a_mx_rows;
  const uint8_t* b_mx;
  uint8_t* out_mx;
  // Linear1 of the fused kernel: A row p of a tile is the token row
  // a_route[p] / K of A (a_rows token rows) instead of pool row p
  const int32_t* a_route;    // [P] route i*K+k of pool row p (-1: padding), or null
  int64_t a_rows;            // T when a_route is set
  // split tail tiles (partial accumulators of K pieces, their ready flags)
  uint32_t* partials;        // [kSplitSlots][BM*BN] words
  uint32_t* split_flags;     // [kSplitSlots], zero between calls
  int max_split;             // largest K split of a tail tile (<= 1: none)
  float clamp;               // Linear1: H clamped to [-clamp, clamp] before SwiGLU (+inf: none)
  uint32_t spin_limit;       // polls before a wait for a partial gives up
  // The fused kernel's dependency schedule (null: none).  Linear1 adds one
  // to dep_done[b] for each finished tile of M-block b, once its stores are
  // complete; Linear2 waits for dep_wait[b] >= dep_target before the first
  // copy of a tile of M-block b.
  uint32_t* dep_done;
  const uint32_t* dep_wait;
  uint32_t dep_target;
  // the fused kernel's per-XCD tile counters [8], zero at the start (null:
  // each workgroup takes every G-th tile of its XCD's slice)
  uint32_t* claim;
  int steal;                 // with claim: take other XCDs' tiles once this XCD's are done
};

struct RequantArgs {
  const float* a_stage;      // [P][I]
  const int32_t* offsets;    // [E+1]
  const int32_t* counts;     // [E]
  void* a_pool;              // [P][I] codes
  float* a_scale;            // [P]
  int64_t P;
  int E, I, usecase;
};

struct CombineArgs {
  const void* contrib;         // [T*K][H] float32, or bf16 when slot_bf16
  const int32_t* route_to_pool;// [T*K]
  void* y;                     // [T][H]
  int64_t T;
  int H, K, y_f32, slot_bf16;
};

// Control words at the start of the workspace, cleared by the pre-pass of
// every call: [1] is the device error word (mm_device_error bits); the fused
// kernel's grid barriers use [0], [2] and [16..47]; [kSplitFlag0 ..] are the
// ready flags of split tail tiles (each flag is reset by its consumer, so
// they are zero again when a GEMM ends).
constexpr int kSplitSlots = 512;
constexpr int kSplitFlag0 = 64;
// [kClockWord0, +8): the fused kernel's clock sample, four 64-bit words:
// shader-clock counter at start and end, 100 MHz counter at start and end
constexpr int kClockWord0 = 48;
constexpr int kCtlWords = kSplitFlag0 + kSplitSlots;

// Everything the fused persistent kernel needs: the arguments of each phase.
struct MegaArgs {
  DispatchArgs d;
  GemmArgs l1, l2;
  RequantArgs rq;
  CombineArgs cb;
  uint32_t* ctl;             // [kCtlWords]
  int64_t nwaves;            // dispatch waves
  // Linear1 reads the token rows in place (l1.a_route set): A8W8 codes and
  // scales of the T tokens are made here, no pool rows are gathered
  void* x_tok;               // [T][H] codes (A8W8, MX)
  void* x_tok_scale;         // float [T] (A8W8) or E8M0 [T][H/32] (MX)
  int l1_by_token;
  uint32_t spin_limit;       // polls before a grid barrier gives up
  // the routed experts' counts for the caller (expert_token_nums [Er]);
  // d.counts is the workspace's own [E] array (shared experts included)
  int32_t* counts_out;
  // counters of the dependency schedule, cleared by the pre-pass: per
  // M-block finished Linear1 tiles [0, dep_blocks), then requantised rows
  // [dep_blocks, 2 * dep_blocks), then the tile counters of Linear1 and
  // Linear2 (8 each)
  uint32_t* dep;
  int64_t dep_blocks;
  int no_dep;                // 1: grid barriers instead of the dependency schedule
  int static_tiles;          // 1: no tile counters (each workgroup every G-th tile)
};

// launchers (return hipError_t of the launch)
// clears counts[0..E) and ctl words [ctl_first, ctl_first + ctl_n)
hipError_t launch_zero(int32_t* counts, int E, uint32_t* ctl, int ctl_first, int ctl_n, hipStream_t s);
hipError_t launch_mega_prep(const MegaArgs& a, MegaArgs* dev_args, hipStream_t s);
hipError_t launch_mega(int usecase, int tile, bool exact_l1, const MegaArgs* dev_args, int grid, bool coop,
                       hipStream_t s);
int mega_grid(int tile, int num_cus);
hipError_t launch_count(const DispatchArgs& a, hipStream_t s);
hipError_t launch_scatter(const DispatchArgs& a, hipStream_t s);
hipError_t launch_gather(const DispatchArgs& a, hipStream_t s);
// esz: bytes per weight (2, 1), or 0 for e2m1 (two per byte)
hipError_t launch_prepare(const void* w1, const void* w2, void* w1o, void* w2o, int E, int H, int I,
                          int esz, int group, hipStream_t s);
// exact_l1: e4m3 Linear1 on bf16 MFMA with exact widening (else on the e4m3 MFMA)
hipError_t launch_gemm(int mode, int usecase, int tile, bool exact_l1, const GemmArgs& a, int grid, hipStream_t s);
int gemm_grid(int tile, int64_t P, int N, int num_cus);
hipError_t launch_requant(const RequantArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace mm
