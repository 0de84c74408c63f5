// Grouped expert GEMMs on CDNA4 MFMA with fused epilogues.
//
// Linear1 (mode 0): per expert e, H_e = X_e . W1[e] over the BLOCK_M-padded
//   pool rows of e (operator page, Expert Compute step 1), then SwiGLU in the
//   epilogue (step 2: A = SiLU(H[:, :I]) * H[:, I:]).  The prepared W1 rows
//   interleave 32 gate columns with the 32 matching up columns, so every lane
//   holds a gate accumulator and its up partner.  A16W16 stores A in bf16;
//   A8W8 dequantises (C * s^W1) * s^X, stores A in float32 and records the
//   row amax for the per-row requantisation (step 3).
// Linear2 (mode 1): Y_e = A_e . W2[e] (A8W8: (D * s^W2) * s^A), times the
//   route's gate weight G[i,k]; the weighted row is written to the route's
//   float32 combine slot i*K+k (Token Combine sums the slots in order).
// Mode 2 stores the raw int32 accumulators (A8W8-INT exactness checks).
//
// Tiling: one 256-thread workgroup per BLOCK_M x 256 output tile, 4 waves,
// each wave a grid of 32x32 MFMA blocks.  K advances 128 bytes per stage
// (64 bf16 or 128 int8/e4m3); the A and B stages are double-buffered in LDS
// with a register prefetch of the next stage from HBM.  Every LDS row is
// padded to 144 bytes so the 16-byte fragment reads of 32 consecutive rows
// hit distinct banks.  The grid is persistent: workgroups stride over the
// tile list (expert M-blocks x N-blocks), whose length is read on the device
// from the dispatch offsets, so no host synchronisation is needed.
#include "mm_device.hpp"
#include "mm_internal.hpp"

namespace mm {

constexpr int kBN = 256;
constexpr int kRowBytes = 128;          // K bytes per stage row
constexpr int kMaxExperts = 1024;

// Workgroup shapes: 4 waves (one per SIMD), WM along M x WN along N; a wave's
// N range must hold whole 64-row gate/up groups (WTN >= 64).
template <int BM> struct TileShape;
template <> struct TileShape<64> { static constexpr int WM = 1, WN = 4; };
template <> struct TileShape<128> { static constexpr int WM = 2, WN = 4; };
template <int BM> constexpr int threads_of() { return 64 * TileShape<BM>::WM * TileShape<BM>::WN; }
constexpr int kStages = 3;   // LDS ring slots

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS fragment read outside the compiler's view: the compiler would otherwise
// wait for every in-flight LDS-DMA before any LDS read it cannot disambiguate.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <int N>
__device__ __forceinline__ void lgkm_wait() { asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N)); }
__device__ __forceinline__ void tie(u32x4& v) { asm volatile("" : "+v"(v)); }
// wait until at most VM of this wave's LDS-DMA loads are in flight and all its
// LDS reads returned, then the workgroup barrier
template <int VM>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// Loads of one K-stage straight into LDS slot kb % S: instruction i of wave wv
// moves DMA group g = wv + NW*i (8 rows); groups below BM/8 are A rows.
// The tile bases become buffer descriptors here (reads past a tile return
// zero); the descriptor type cannot appear in a signature the host pass sees.
template <int D, int NW, int BM, int STAGE, int S>
__device__ __forceinline__ void issue_stage(uint8_t* lds, const uint8_t* abase, int abytes, const uint8_t* bbase,
                                            int bbytes, const uint32_t* doff, int wv, int kb) {
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, abytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc((void*)bbase, (short)0, bbytes, 0x00020000);
  const int slot = kb % S;
  const int koff = __builtin_amdgcn_readfirstlane(kb * kRowBytes);   // scalar offset of stage kb
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int g = wv + NW * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(g < BM / 8 ? ar : br, (lds_ptr_t)(lds + slot * STAGE + g * 1024), 16,
                                             doff[i], koff, 0, 0);
  }
}

// 16 e4m3 -> 16 bf16 (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ void widen_e4m3(const u32x4& w, u32x4& lo, u32x4& hi) {
#define CVT(x, hi_) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((x), 1.0f, (hi_)))
  lo = u32x4{CVT(w[0], false), CVT(w[0], true), CVT(w[1], false), CVT(w[1], true)};
  hi = u32x4{CVT(w[2], false), CVT(w[2], true), CVT(w[3], false), CVT(w[3], true)};
#undef CVT
}

// Mainloop data layout.  A stage holds BLOCK_M A rows then 256 B rows of 128
// K-bytes (eight 16-byte chunks) each, filled by buffer loads straight into
// LDS: one wave instruction moves 8 rows (64 lanes x 16 bytes, lane i -> byte
// 16*i of the group).  Chunk c of row r sits at position c ^ ((r / 2) % 8):
// LDS serves a 16-byte read of 16 lanes per pass over 64 banks, and 16
// consecutive rows at one chunk then hit 16 distinct bank groups.  A lane's
// MFMA operand covers chunks 4h..4h+3 of its row (h = lane / 32), the same
// chunks for A and B, so every product pairs equal k.
//
// Pipeline per stage k (three LDS slots): wait for stage k's loads and a
// barrier; issue the loads of stage k+2 into the slot stage k-1 used; read
// stage k's fragments and run its MFMAs chunk by chunk as the reads land.
// Two waves per SIMD overlap one wave's reads with the other's MFMAs.
//
// Epilogue: the accumulators go through the (then idle) LDS ring as a
// float32 tile, so each output row leaves as one contiguous store.
template <int UC, int BM, int MODE, bool WIDEN>
__global__ __launch_bounds__(threads_of<BM>()) __attribute__((amdgpu_waves_per_eu(threads_of<BM>() / 256, threads_of<BM>() / 256)))
void k_gemm(GemmArgs a) {
  constexpr int WM = TileShape<BM>::WM, WN = TileShape<BM>::WN, S = kStages;
  constexpr int NT = threads_of<BM>(), NW = NT / 64;
  constexpr int WTM = BM / WM, WTN = kBN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int ROWS = BM + kBN;
  constexpr int STAGE = ROWS * kRowBytes;
  constexpr int GROUPS = ROWS / 8;
  static_assert(GROUPS % NW == 0, "DMA groups must split evenly over the waves");
  constexpr int D = GROUPS / NW;                           // DMA instructions per wave per stage
  static_assert(2 * D <= 63, "vmcnt range");
  constexpr int ESZ = (UC == UC_BF16) ? 2 : 1;
  constexpr int NFR = MB + NB;                             // fragment reads per chunk index
  // epilogue tile in LDS (float32): Linear1 keeps the 128 SwiGLU columns,
  // Linear2 / raw keep all 256; pitch = 8 (mod 16) floats keeps the two lane
  // halves of an accumulator write in different bank halves
  constexpr int OCOLS = (MODE == 0) ? kBN / 2 : kBN;
  constexpr int OPITCH = OCOLS + 8;
  static_assert(BM * OPITCH * 4 + 3 * BM * 4 <= S * STAGE, "epilogue tile fits the ring");
  typedef typename Acc<UC>::type AccT;

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int32_t off_s[kMaxExperts + 1];
  __shared__ int32_t cnt_s[kMaxExperts];

  const int t = threadIdx.x, l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(t / 64);
  const int h = l / 32, lr = l % 32;
  const int wm = wv / WN, wn = wv % WN;

  for (int e = t; e <= a.E; e += NT) off_s[e] = a.offsets[e];
  for (int e = t; e < a.E; e += NT) cnt_s[e] = a.counts[e];
  __syncthreads();

  const int kbytes = a.Kdim * ESZ;
  const int nk = kbytes / kRowBytes;
  const int n_tiles = a.N / kBN;
  const int total = (off_s[a.E] / BM) * n_tiles;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;

  // per-lane LDS addresses of the four fragment chunks (stage slot added per stage)
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t cpos = (uint32_t)(((4 * h + q) ^ ((lr >> 1) & 7)) << 4);
    aoff[q] = lds_base + (uint32_t)(wm * WTM + lr) * kRowBytes + cpos;
    boff[q] = lds_base + (uint32_t)(BM + wn * WTN + lr) * kRowBytes + cpos;
  }
  // per-lane byte offsets of the DMA rows inside their tile: row r = 8g + l/8
  // lands its logical chunk (l%8) ^ ((r/2)%8) at position l%8
  uint32_t doff[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int g = wv + NW * i;
    const int r = 8 * g + l / 8;
    doff[i] = (uint32_t)((r < BM ? r : r - BM) * kbytes + (((l & 7) ^ ((r >> 1) & 7)) << 4));
  }
  float* otile = reinterpret_cast<float*>(lds);               // epilogue tile [BM][OPITCH]
  float* orow = reinterpret_cast<float*>(lds) + BM * OPITCH;  // per-row s^X (Linear1) / s^A (Linear2) [BM]
  float* ogw = orow + BM;                                      // per-row gate weight [BM]
  int32_t* oroute = reinterpret_cast<int32_t*>(ogw + BM);     // per-row route i*K+k [BM]

  // Tile order: expert-major, then N-block, then M-block, so tiles that run
  // together share weight tiles (same expert and N-block) and activation
  // tiles (same M-block).  Workgroup w runs on XCD w % 8 (round-robin
  // dispatch); each XCD walks its own contiguous slice of the list so the
  // sharing happens inside one L2.
  const int nxcd = gridDim.x >= 8 ? 8 : 1;
  const int xcd = blockIdx.x % nxcd, wgx = blockIdx.x / nxcd, per_x = gridDim.x / nxcd;
  const int slice = (total + nxcd - 1) / nxcd;
  const int t_beg = xcd * slice, t_end = min(total, t_beg + slice);
  const bool in_grid = (int)blockIdx.x < per_x * nxcd;   // a tail beyond a multiple of 8 stays idle
  for (int tile = t_beg + wgx; in_grid && tile < t_end; tile += per_x) {
    // expert of this tile: the largest e with (off[e] / BM) * n_tiles <= tile
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((off_s[mid] / BM) * n_tiles <= tile) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int mb0 = off_s[e] / BM, nmb = (off_s[e + 1] - off_s[e]) / BM;
    const int local = tile - mb0 * n_tiles;
    const int nblk = local / nmb, mblk = mb0 + local % nmb;
    const int row0 = mblk * BM, n0 = nblk * kBN;
    const int valid = min(BM, off_s[e] + cnt_s[e] - row0);
    const uint8_t* abase = a.A + (int64_t)row0 * kbytes;
    const uint8_t* bbase = a.B + ((int64_t)e * a.N + n0) * kbytes;

#define MM_ISSUE(kb_) issue_stage<D, NW, BM, STAGE, S>(lds, abase, BM * kbytes, bbase, kBN * kbytes, doff, wv, (kb_))
    AccT acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

    // every wave is done with the previous tile's LDS use and stores
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < nk) MM_ISSUE(st);
    for (int kb = 0; kb < nk; ++kb) {
      // stage kb landed for every wave; everyone is done with stage kb-1's slot
      if (kb + 1 < nk) vm_barrier<D>(); else vm_barrier<0>();
      if (kb + S - 1 < nk) MM_ISSUE(kb + S - 1);
      const uint32_t so = (uint32_t)((kb % S) * STAGE);
      u32x4 fa[MB][4], fb[NB][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (MB > 0) fa[0][q] = ds_read16<0>(aoff[q] + so);
        if constexpr (MB > 1) fa[1][q] = ds_read16<4096>(aoff[q] + so);
        if constexpr (NB > 0) fb[0][q] = ds_read16<0>(boff[q] + so);
        if constexpr (NB > 1) fb[1][q] = ds_read16<4096>(boff[q] + so);
        if constexpr (NB > 2) fb[2][q] = ds_read16<8192>(boff[q] + so);
        if constexpr (NB > 3) fb[3][q] = ds_read16<12288>(boff[q] + so);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // chunk q has landed once at most NFR*(3-q) reads are outstanding
        if (q == 0) lgkm_wait<(NFR * 3 > 15 ? 15 : NFR * 3)>();
        else if (q == 1) lgkm_wait<(NFR * 2 > 15 ? 15 : NFR * 2)>();
        else if (q == 2) lgkm_wait<NFR>();
        else lgkm_wait<0>();
#pragma unroll
        for (int i = 0; i < MB; ++i) tie(fa[i][q]);
#pragma unroll
        for (int j = 0; j < NB; ++j) tie(fb[j][q]);
        if constexpr (UC == UC_FP8 && !WIDEN) {
          if (q & 1) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
              for (int j = 0; j < NB; ++j) mfma_fp8(acc[i][j], fa[i][q - 1], fa[i][q], fb[j][q - 1], fb[j][q]);
          }
        } else if constexpr (WIDEN) {
          u32x4 alo[MB], ahi[MB], blo[NB], bhi[NB];
#pragma unroll
          for (int i = 0; i < MB; ++i) widen_e4m3(fa[i][q], alo[i], ahi[i]);
#pragma unroll
          for (int j = 0; j < NB; ++j) widen_e4m3(fb[j][q], blo[j], bhi[j]);
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              mfma_bf16(acc[i][j], alo[i], blo[j]);
              mfma_bf16(acc[i][j], ahi[i], bhi[j]);
            }
        } else {
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              if constexpr (UC == UC_BF16) mfma_bf16(acc[i][j], fa[i][q], fb[j][q]);
              else mfma_i8(acc[i][j], fa[i][q], fb[j][q]);
            }
        }
      }
    }
#undef MM_ISSUE
    // ------------------------------------------------------------ epilogue
    // all waves are done reading the ring: it becomes the output tile
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (MODE == 0 && UC != UC_BF16) {
      for (int r = t; r < BM; r += NT) orow[r] = r < valid ? a.x_scale[row0 + r] : 0.0f;
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int rb = wm * WTM + i * 32 + 4 * h;
      if constexpr (MODE == 0) {
        // gate/up pair j -> 32 output columns
#pragma unroll
        for (int j = 0; j < NB / 2; ++j) {
          const int oc = wn * (WTN / 2) + j * 32 + lr;
          float gs = 1.0f, us = 1.0f;
          if constexpr (UC != UC_BF16) {
            const int col = n0 / 2 + oc;
            gs = a.w_scale[(int64_t)e * 2 * a.I + col];
            us = a.w_scale[(int64_t)e * 2 * a.I + a.I + col];
          }
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = rb + 8 * (q / 4) + (q % 4);
            float g = acc_to_f32(acc[i][2 * j][q]);
            float u = acc_to_f32(acc[i][2 * j + 1][q]);
            if constexpr (UC != UC_BF16) {
              const float sx = orow[r];
              g = (g * gs) * sx;
              u = (u * us) * sx;
            }
            otile[r * OPITCH + oc] = silu(g) * u;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int oc = wn * WTN + j * 32 + lr;
          float ws = 1.0f;
          if constexpr (MODE == 1 && UC != UC_BF16) ws = a.w_scale[(int64_t)e * a.H + n0 + oc];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = rb + 8 * (q / 4) + (q % 4);
            if constexpr (MODE == 2) reinterpret_cast<int32_t*>(otile)[r * OPITCH + oc] = acc[i][j][q];
            else otile[r * OPITCH + oc] = acc_to_f32(acc[i][j][q]) * ws;
          }
        }
      }
    }
    if constexpr (MODE == 1) {
      // per-row route, A8W8 row scale s^A and the route's gate weight G[i,k]
      for (int r = t; r < BM; r += NT) {
        if (r < valid) {
          const int64_t p = (int64_t)row0 + r;
          const int32_t route = a.pool_src[p];
          oroute[r] = route;
          ogw[r] = a.topk_w[route];
          orow[r] = (UC != UC_BF16) ? a.a_scale[p] : 1.0f;
        }
      }
    }
    __syncthreads();
    // cooperative row-major pass: 16-byte column chunks, one row per group of
    // CPR consecutive threads (BM * CPR is a multiple of the thread count, so
    // every thread runs the same number of trips)
    constexpr int CPR = OCOLS / 4;                       // float4 chunks per row
    static_assert((BM * CPR) % NT == 0 && CPR <= 64 && 64 % CPR == 0, "row groups stay inside a wave");
    for (int idx = t; idx < BM * CPR; idx += NT) {
      const int r = idx / CPR, c4 = idx % CPR;
      const bool ok = r < valid;
      const int64_t p = (int64_t)row0 + r;
      const f32x4 v = *reinterpret_cast<const f32x4*>(otile + r * OPITCH + c4 * 4);
      if constexpr (MODE == 0) {
        const int col = n0 / 2 + c4 * 4;
        if constexpr (UC == UC_BF16) {
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          if (ok) *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.a_out) + p * a.I + col) = o;
        } else {
          if (ok) *reinterpret_cast<f32x4*>(a.a_stage + p * a.I + col) = v;
          // row amax of this tile's columns; the row's tiles combine by atomicMax
          float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
          for (int o = CPR / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          if (ok && c4 == 0) atomicMax(&a.a_amax[p], __float_as_uint(m));
        }
      } else if constexpr (MODE == 1) {
        // contribution of route i*K+k: ((D * s^W2) * s^A) * G[i,k]
        const float rs = orow[r], gw = ogw[r];
        f32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = (UC != UC_BF16) ? (v[c] * rs) * gw : v[c] * gw;
        if (ok) *reinterpret_cast<f32x4*>(a.contrib + (int64_t)oroute[r] * a.H + n0 + c4 * 4) = o;
      } else {
        const int n = n0 + c4 * 4;
        int col = n;
        if (a.gate_up_group > 0) {
          const int g2 = 2 * a.gate_up_group;
          const int qq = n / g2, m = n % g2;
          col = (m < a.gate_up_group) ? qq * a.gate_up_group + m : a.I + qq * a.gate_up_group + (m - a.gate_up_group);
        }
        if (ok) *reinterpret_cast<i32x4*>(a.raw_out + p * a.N + col) = __builtin_bit_cast(i32x4, v);
      }
    }
  }
}

template <int UC, int BM, int MODE>
static hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t s) {
  // e4m3 Linear1 runs on bf16 MFMA with exact e4m3 -> bf16 widening: the
  // e4m3 MFMAs round inside their dot products, and the per-row e4m3
  // requantisation that follows Linear1 would turn that rounding into code
  // changes.  Linear2 keeps the e4m3 MFMA (nothing is quantised after it).
  constexpr bool WIDEN = (UC == UC_FP8) && (MODE == 0);
  constexpr size_t lds = (size_t)kStages * (BM + kBN) * kRowBytes;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)k_gemm<UC, BM, MODE, WIDEN>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemm<UC, BM, MODE, WIDEN>), dim3(grid), dim3(threads_of<BM>()), lds, s, a);
  return hipGetLastError();
}

template <int UC, int MODE>
static hipError_t launch_bm(int tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tile) {
    case TILE_M64_N256: return launch_one<UC, 64, MODE>(a, grid, s);
    default: return launch_one<UC, 128, MODE>(a, grid, s);
  }
}

template <int MODE>
static hipError_t launch_uc(int usecase, int tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (usecase) {
    case UC_BF16: return launch_bm<UC_BF16, MODE>(tile, a, grid, s);
    case UC_FP8: return launch_bm<UC_FP8, MODE>(tile, a, grid, s);
    default: return launch_bm<UC_I8, MODE>(tile, a, grid, s);
  }
}

hipError_t launch_gemm(int mode, int usecase, int tile, const GemmArgs& a, int grid, hipStream_t s) {
  if (mode == 0) return launch_uc<0>(usecase, tile, a, grid, s);
  if (mode == 1) return launch_uc<1>(usecase, tile, a, grid, s);
  if (usecase != UC_I8) return hipErrorInvalidValue;
  return launch_bm<UC_I8, 2>(tile, a, grid, s);
}

int gemm_grid(int tile, int64_t P, int N, int num_cus) {
  const int64_t tiles = (P / tile_bm(tile)) * (int64_t)(N / kBN);
  int64_t g = num_cus;   // one resident workgroup per CU (LDS bound)
  if (tiles < g) g = tiles;
  return (int)(g < 1 ? 1 : g);
}

// ---------------------------------------------------------------------------
// per-row requantisation of A (A8W8): s^A = max(amax/Qmax, 1e-8), IEEE f32
// ---------------------------------------------------------------------------
template <int UC>
__global__ __launch_bounds__(256) void k_requant(RequantArgs a) {
  __shared__ int32_t off_s[kMaxExperts + 1];
  __shared__ int32_t cnt_s[kMaxExperts];
  for (int e = threadIdx.x; e <= a.E; e += 256) off_s[e] = a.offsets[e];
  for (int e = threadIdx.x; e < a.E; e += 256) cnt_s[e] = a.counts[e];
  __syncthreads();
  const int w = threadIdx.x / 64, l = lane_id();
  const int64_t p = (int64_t)blockIdx.x * 4 + w;
  if (p >= off_s[a.E]) return;
  // padding rows (past the expert's count) carry no route
  int lo = 0, hi = a.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off_s[mid] <= p) lo = mid; else hi = mid;
  }
  if (p >= (int64_t)off_s[lo] + cnt_s[lo]) return;
  const float qmax = (UC == UC_I8) ? 127.0f : 448.0f;
  const float s = fmaxf(__uint_as_float(a.a_amax[p]) / qmax, 1e-8f);
  const float4* src = reinterpret_cast<const float4*>(a.a_stage + p * a.I);
  uint2* dst = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.a_pool) + p * a.I);
  for (int c = l; c < a.I / 8; c += 64) {
    const float4 v0 = src[2 * c], v1 = src[2 * c + 1];
    const float f[8] = {v0.x / s, v0.y / s, v0.z / s, v0.w / s, v1.x / s, v1.y / s, v1.z / s, v1.w / s};
    uint32_t o[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if constexpr (UC == UC_I8) {
        o[q] = (uint32_t)(f32_to_i8sym(f[4 * q]) & 0xff) | ((uint32_t)(f32_to_i8sym(f[4 * q + 1]) & 0xff) << 8) |
               ((uint32_t)(f32_to_i8sym(f[4 * q + 2]) & 0xff) << 16) | ((uint32_t)(f32_to_i8sym(f[4 * q + 3]) & 0xff) << 24);
      } else {
        o[q] = f32x2_to_e4m3x2(f[4 * q], f[4 * q + 1]) | (f32x2_to_e4m3x2(f[4 * q + 2], f[4 * q + 3]) << 16);
      }
    }
    dst[c] = make_uint2(o[0], o[1]);
  }
  if (l == 0) a.a_scale[p] = s;
}

hipError_t launch_requant(const RequantArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.P + 3) / 4));
  if (a.usecase == UC_I8) hipLaunchKernelGGL(k_requant<UC_I8>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_requant<UC_FP8>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token Combine: y_i = sum_{k=0..K-1} slot[i*K+k] in slot order, float32;
// masked routes (route_to_pool < 0) contribute nothing.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int64_t i = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= a.H) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int k = 0; k < a.K; ++k) {
    const int64_t r = i * a.K + k;
    if (a.route_to_pool[r] < 0) continue;
    const float4* src = reinterpret_cast<const float4*>(a.contrib + r * a.H + c);
    const float4 v0 = src[0], v1 = src[1];
    acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
    acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
  }
  if (a.y_f32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.y) + i * a.H + c);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + i * a.H + c) = o;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.T, (unsigned)((a.H + 2047) / 2048));
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm
