// Device-side bodies of the grouped expert GEMMs on CDNA4 MFMA with fused
// epilogues, the A8W8 requantisation and Token Combine, shared by the
// stand-alone kernels and the fused persistent kernel.
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
// Tiling: one workgroup per BLOCK_M x 256 output tile; each wave owns a
// 64 x 64 grid of 32x32 MFMA blocks.  K advances 128
// bytes per stage (64 bf16 or 128 int8/e4m3).  Stages are copied from HBM
// straight into a three-slot LDS ring by buffer loads (no register staging),
// in a bank-conflict-free swizzled order; the fragment reads of the next
// stage are interleaved with the MFMAs of the current one.  The grid is
// persistent: workgroups stride over the tile list (expert M-blocks x
// N-blocks), whose length is read on the device from the dispatch offsets,
// so no host synchronisation is needed.
#pragma once
#include "mm_device.hpp"
#include "mm_internal.hpp"

#include <type_traits>

namespace mm {

constexpr int kBN = 256;
constexpr int kRowBytes = 128;          // K bytes per stage row
constexpr int kMaxExperts = 1024;

// Workgroup shapes: WM waves along M x WN along N, one workgroup per CU (the
// LDS ring fills it): four waves (one per SIMD) for 64-row tiles, eight (two
// per SIMD) for 128-row tiles.  A wave's N range must hold whole 64-row
// gate/up groups (WTN >= 64).
template <int BM> struct TileShape;
template <> struct TileShape<64> { static constexpr int WM = 1, WN = 4; };
template <> struct TileShape<128> { static constexpr int WM = 2, WN = 4; };
template <int BM> constexpr int threads_of() { return 64 * TileShape<BM>::WM * TileShape<BM>::WN; }
// LDS ring slots: a 256-row tile's stage is 64 KB, so only two fit
template <int BM> constexpr int stages_of() { return BM >= 256 ? 2 : 3; }
constexpr int kLdsMax = 152 * 1024;   // dynamic LDS left beside the expert tables
// Epilogue: the float32 output tile goes through LDS in NPASS row bands
// (Linear1 keeps the 128 SwiGLU columns, Linear2 / raw all 256), plus three
// per-row arrays.  The pitch is 8 (mod 16) floats so the two lane halves of
// an accumulator write land in different bank halves.
template <int MODE> constexpr int ocols_of() { return MODE == 0 ? 128 : 256; }
template <int BM, int MODE> constexpr int epi_bytes(int npass) { return (BM / npass) * (ocols_of<MODE>() + 8) * 4 + 3 * BM * 4; }
template <int BM, int MODE> constexpr int epi_passes() {
  return epi_bytes<BM, MODE>(1) <= kLdsMax ? 1 : epi_bytes<BM, MODE>(2) <= kLdsMax ? 2 : 4;
}
template <int BM, int MODE> constexpr int lds_bytes_of() {
  const int ring = stages_of<BM>() * (BM + 256) * 128;
  const int epi = epi_bytes<BM, MODE>(epi_passes<BM, MODE>());
  return ring > epi ? ring : epi;
}

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

// One LDS-DMA instruction of stage kb: instruction i of wave wv moves the
// 8-row group g = wv + NW*i into slot kb % S (groups below BM/8 are A rows).
// voff is the lane's byte offset inside its group; the group's row offset
// and the stage's K offset are wave-uniform and go in the scalar offset.
// The tile bases become buffer descriptors here: the descriptor type cannot
// appear in a signature the host pass sees.
template <int NW, int BM, int STAGE, int S>
__device__ __forceinline__ void dma_one(uint8_t* lds, const uint8_t* abase, int abytes, const uint8_t* bbase,
                                        int bbytes, uint32_t voff, int wv, int kbytes, int i, int kb) {
  const bool is_a = i < BM / (8 * NW);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(is_a ? abase : bbase), (short)0, is_a ? abytes : bbytes, 0x00020000);
  const int rows = is_a ? 8 * NW * i : 8 * NW * i - BM;
  const int soff = __builtin_amdgcn_readfirstlane(rows * kbytes + kb * kRowBytes);
  const int g = wv + NW * i;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds + (kb % S) * STAGE + g * 1024), 16, voff, soff, 0, 0);
}

// The fragments of one K-stage held in registers: four 16-byte chunks of
// the wave's MB A blocks and NB B blocks.
template <int MB, int NB>
struct Frags {
  u32x4 a[MB][4];
  u32x4 b[NB][4];
};

// Fragment read r of a stage (r = chunk * (MB + NB) + block; A blocks first),
// 32 rows apart inside the wave's rows.  Only called with r known at compile
// time after unrolling, so every branch folds away.
template <int MB, int NB>
__device__ __forceinline__ void read_frag(Frags<MB, NB>& f, int r, const uint32_t* aoff, const uint32_t* boff,
                                          uint32_t so) {
  const int q = r / (MB + NB), x = r % (MB + NB);
  if (x < MB) {
    const uint32_t ad = aoff[q] + so;
    if (x == 0) f.a[0][q] = ds_read16<0>(ad);
    if constexpr (MB > 1) if (x == 1) f.a[1][q] = ds_read16<4096>(ad);
    if constexpr (MB > 2) if (x == 2) f.a[2][q] = ds_read16<8192>(ad);
    if constexpr (MB > 3) if (x == 3) f.a[3][q] = ds_read16<12288>(ad);
  } else {
    const uint32_t ad = boff[q] + so;
    const int y = x - MB;
    if (y == 0) f.b[0][q] = ds_read16<0>(ad);
    if constexpr (NB > 1) if (y == 1) f.b[1][q] = ds_read16<4096>(ad);
    if constexpr (NB > 2) if (y == 2) f.b[2][q] = ds_read16<8192>(ad);
    if constexpr (NB > 3) if (y == 3) f.b[3][q] = ds_read16<12288>(ad);
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
// Epilogue: the accumulators go through the (then idle) LDS ring as a
// float32 tile, so each output row leaves as one contiguous store.
// The argument block with every field forced into scalar registers: the
// fused kernel loads its arguments from memory, and a tile base the compiler
// cannot prove uniform would turn each buffer load into a loop over lanes.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>((hi << 32) | lo);
}

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ GemmArgs uniform_args(const GemmArgs& in) {
  GemmArgs a = in;
  a.A = uniform_ptr(in.A);
  a.B = uniform_ptr(in.B);
  a.offsets = uniform_ptr(in.offsets);
  a.counts = uniform_ptr(in.counts);
  a.pool_src = uniform_ptr(in.pool_src);
  a.x_scale = uniform_ptr(in.x_scale);
  a.w_scale = uniform_ptr(in.w_scale);
  a.a_out = uniform_ptr(in.a_out);
  a.a_stage = uniform_ptr(in.a_stage);
  a.a_amax = uniform_ptr(in.a_amax);
  a.a_scale = uniform_ptr(in.a_scale);
  a.topk_w = uniform_ptr(in.topk_w);
  a.contrib = uniform_ptr(in.contrib);
  a.raw_out = uniform_ptr(in.raw_out);
  a.err = uniform_ptr(in.err);
  a.E = uniform_int(in.E);
  a.N = uniform_int(in.N);
  a.Kdim = uniform_int(in.Kdim);
  a.I = uniform_int(in.I);
  a.H = uniform_int(in.H);
  a.K = uniform_int(in.K);
  a.gate_up_group = uniform_int(in.gate_up_group);
  return a;
}

template <int UC, int BM, int MODE, bool WIDEN>
__device__ __forceinline__ void gemm_tiles(const GemmArgs& args, uint8_t* lds, int32_t* off_s, int32_t* cnt_s) {
  const GemmArgs a = uniform_args(args);
  constexpr int WM = TileShape<BM>::WM, WN = TileShape<BM>::WN, S = stages_of<BM>();
  constexpr int NT = threads_of<BM>(), NW = NT / 64;
  constexpr int WTM = BM / WM, WTN = kBN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int ROWS = BM + kBN;
  constexpr int STAGE = ROWS * kRowBytes;
  constexpr int GROUPS = ROWS / 8;
  static_assert(GROUPS % NW == 0, "DMA groups must split evenly over the waves");
  constexpr int D = GROUPS / NW;                           // DMA instructions per wave per stage
  static_assert((S - 1) * D <= 63, "vmcnt range");
  constexpr int ESZ = (UC == UC_BF16) ? 2 : 1;
  constexpr int NFR = MB + NB;                             // fragment reads per chunk index
  // MFMA phases of a stage: one chunk each, or two for e4m3 MFMAs (K = 64)
  constexpr int CPP = (UC == UC_FP8 && !WIDEN) ? 2 : 1;
  constexpr int NPH = 4 / CPP;
  constexpr int RPP = NFR * CPP;                           // fragment reads per phase
  constexpr int MPP = MB * NB * (WIDEN ? 2 : 1);           // MFMAs per phase
  // phase 0 may start once only the reads of the later phases are in flight
  constexpr int P0WAIT = (4 * NFR - RPP) > 15 ? 15 : (4 * NFR - RPP);
  static_assert(BM % (8 * NW) == 0, "A rows fill whole DMA instructions");
  constexpr int OCOLS = ocols_of<MODE>();
  constexpr int OPITCH = OCOLS + 8;
  constexpr int NPASS = epi_passes<BM, MODE>(), EPR = BM / NPASS;   // epilogue row bands
  static_assert(epi_bytes<BM, MODE>(NPASS) <= kLdsMax && EPR % 32 == 0, "epilogue band fits LDS");
  typedef typename Acc<UC>::type AccT;


  const int t = threadIdx.x, l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(t / 64);
  const int h = l / 32, lr = l % 32;
  const int wm = wv / WN, wn = wv % WN;

  for (int e = t; e <= a.E; e += NT) off_s[e] = a.offsets[e];
  for (int e = t; e < a.E; e += NT) cnt_s[e] = a.counts[e];
  __syncthreads();
  // The offsets must describe a padded pool inside P rows: multiples of
  // BLOCK_M, each expert's block range holding its count.  Anything else
  // (offsets the caller made up) runs no tile and raises
  // MM_DEVERR_BAD_OFFSETS instead of addressing outside the pool.
  bool bad = false;
  for (int e = t; e < a.E; e += NT)
    bad |= off_s[e] < 0 || off_s[e] % BM != 0 || cnt_s[e] < 0 || (int64_t)off_s[e] + cnt_s[e] > off_s[e + 1];
  if (t == 0) bad |= off_s[a.E] % BM != 0 || off_s[a.E] > a.P;
  const bool offsets_ok = __syncthreads_or(bad) == 0;
  if (!offsets_ok && t == 0 && a.err) atomicOr(a.err, (uint32_t)MM_DEVERR_BAD_OFFSETS);

  const int kbytes = a.Kdim * ESZ;
  const int nk = kbytes / kRowBytes;
  const int n_tiles = a.N / kBN;
  const int total = offsets_ok ? (off_s[a.E] / BM) * n_tiles : 0;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;

  // per-lane LDS addresses of the four fragment chunks (stage slot added per stage)
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t cpos = (uint32_t)(((4 * h + q) ^ ((lr >> 1) & 7)) << 4);
    aoff[q] = lds_base + (uint32_t)(wm * WTM + lr) * kRowBytes + cpos;
    boff[q] = lds_base + (uint32_t)(BM + wn * WTN + lr) * kRowBytes + cpos;
  }
  // per-lane byte offset of the DMA rows: group g covers rows 8g .. 8g+7, lane
  // l row 8g + l/8, and lands its logical chunk (l%8) ^ ((row/2)%8) at
  // position l%8.  With NW even, g and wv have the same parity, so the
  // swizzle and the in-group offset are the same for all of a wave's groups.
  static_assert(NW % 2 == 0, "DMA swizzle assumes an even wave count");
  const uint32_t voff =
      (uint32_t)((8 * wv + l / 8) * kbytes + (((l & 7) ^ ((4 * (wv & 1) + l / 16) & 7)) << 4));
  float* otile = reinterpret_cast<float*>(lds);                // epilogue band [EPR][OPITCH]
  float* orow = reinterpret_cast<float*>(lds) + EPR * OPITCH;  // per-row s^X (Linear1) / s^A (Linear2) [BM]
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

    const int abytes = BM * kbytes, bbytes = kBN * kbytes;
#define MM_DMA(i_, kb_) dma_one<NW, BM, STAGE, S>(lds, abase, abytes, bbase, bbytes, voff, wv, kbytes, (i_), (kb_))
    AccT acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

    Frags<MB, NB> f;
    // MFMA mi of phase p (chunks CPP*p .. CPP*p + CPP-1 of the stage in f)
    u32x4 wa_lo[MB], wa_hi[MB], wb_lo, wb_hi;   // e4m3 -> bf16 widened operands
    auto mfma_at = [&](int p, int mi) {
      if constexpr (UC == UC_FP8 && !WIDEN) {
        const int i = mi / NB, j = mi % NB, q0 = 2 * p;
        mfma_fp8(acc[i][j], f.a[i][q0], f.a[i][q0 + 1], f.b[j][q0], f.b[j][q0 + 1]);
      } else if constexpr (WIDEN) {
        // B block j outer, so one widened B fragment is live at a time
        const int j = mi / (2 * MB), i = (mi % (2 * MB)) / 2, hi = mi % 2;
        if (mi == 0) {
#pragma unroll
          for (int x = 0; x < MB; ++x) widen_e4m3(f.a[x][p], wa_lo[x], wa_hi[x]);
        }
        if (mi % (2 * MB) == 0) widen_e4m3(f.b[j][p], wb_lo, wb_hi);
        if (hi) mfma_bf16(acc[i][j], wa_hi[i], wb_hi);
        else mfma_bf16(acc[i][j], wa_lo[i], wb_lo);
      } else {
        const int i = mi / NB, j = mi % NB;
        if constexpr (UC == UC_BF16) mfma_bf16(acc[i][j], f.a[i][p], f.b[j][p]);
        else mfma_i8(acc[i][j], f.a[i][p], f.b[j][p]);
      }
    };
    auto tie_chunks = [&](int c0, int c1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < c0 || q >= c1) continue;
#pragma unroll
        for (int i = 0; i < MB; ++i) tie(f.a[i][q]);
#pragma unroll
        for (int j = 0; j < NB; ++j) tie(f.b[j][q]);
      }
    };

    // One K-stage kb.  Phase 0 runs on fragments read during the previous
    // stage.  Then a barrier: stage kb+1 has landed for every wave and every
    // wave is done reading stage kb, so stage kb's slot takes stage kb+S.
    // Phases 1.. run with those DMA issues and the reads of stage kb+1 spread
    // between their MFMAs: a phase's fragment registers are read again as
    // soon as that phase's MFMAs are issued; the last phase's at the end.
    // Scheduling barriers keep this order.
    auto step = [&](int kb, auto refill_tag, auto more_tag, auto vm_tag) {
      constexpr bool REFILL = decltype(refill_tag)::value, MORE = decltype(more_tag)::value;
      constexpr int VM = decltype(vm_tag)::value;   // this wave's DMA loads still allowed in flight
      lgkm_wait<P0WAIT>();
      tie_chunks(0, CPP);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < MPP; ++mi) mfma_at(0, mi);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MORE) {
        vm_barrier<VM>();
      } else {
        lgkm_wait<0>();
      }
      tie_chunks(CPP, 4);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t so = (uint32_t)(((kb + 1) % S) * STAGE);
#ifndef MM_DMA_SPAN
#define MM_DMA_SPAN 0
#endif
      // MFMAs after the barrier over which the DMA issues are spread
      constexpr int NMR = MM_DMA_SPAN == 0 ? (NPH - 1) * MPP : (MM_DMA_SPAN < (NPH - 1) * MPP ? MM_DMA_SPAN : (NPH - 1) * MPP);
      int dm = 0;
#pragma unroll
      for (int p = 1; p < NPH; ++p) {
        int rd = 0;
#pragma unroll
        for (int mi = 0; mi < MPP; ++mi) {
          mfma_at(p, mi);
          if constexpr (REFILL) {
            const int m = (p - 1) * MPP + mi;
            const int target = m < NMR ? ((m + 1) * D + NMR - 1) / NMR : D;
#pragma unroll
            for (int x = 0; x < D; ++x)
              if (x >= dm && x < target) MM_DMA(x, kb + S);
            dm = target < D ? target : D;
          }
          if constexpr (MORE) {
            const int target = ((mi + 1) * RPP + MPP - 1) / MPP;
#pragma unroll
            for (int r = 0; r < RPP; ++r)
              if (r >= rd && r < target) read_frag(f, (p - 1) * RPP + r, aoff, boff, so);
            rd = target < RPP ? target : RPP;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (MORE) {
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_frag(f, (NPH - 1) * RPP + r, aoff, boff, so);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // every wave is done with the previous tile's LDS use and stores
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int st = 0; st < S; ++st)
      if (st < nk) {
#pragma unroll
        for (int x = 0; x < D; ++x) MM_DMA(x, st);
      }
    // stage 0 landed for every wave (the later stages may still be in flight)
    if constexpr (S == 3) {
      if (nk >= 3) vm_barrier<2 * D>(); else if (nk == 2) vm_barrier<D>(); else vm_barrier<0>();
    } else {
      if (nk >= 2) vm_barrier<D>(); else vm_barrier<0>();
    }
#pragma unroll
    for (int r = 0; r < 4 * NFR; ++r) read_frag(f, r, aoff, boff, 0u);
    // Every barrier below has a compile-time DMA count: stage kb+S refills
    // while kb + S < nk, and the last stages drain the ring.
    const std::integral_constant<bool, true> yes;
    const std::integral_constant<bool, false> no;
    const std::integral_constant<int, D> vm_d;
    const std::integral_constant<int, 0> vm_0;
    if constexpr (S == 3) {
      if (nk >= 3) {
        for (int kb = 0; kb < nk - 3; ++kb) step(kb, yes, yes, vm_d);
        step(nk - 3, no, yes, vm_d);
      }
    } else {
      for (int kb = 0; kb < nk - 2; ++kb) step(kb, yes, yes, vm_0);
    }
    if (nk >= 2) step(nk - 2, no, yes, vm_0);
    step(nk - 1, no, no, vm_0);
#undef MM_DMA
    // ------------------------------------------------------------ epilogue
    // all waves are done reading the ring: it becomes the output band
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (MODE == 0 && UC != UC_BF16) {
      for (int r = t; r < BM; r += NT) orow[r] = r < valid ? a.x_scale[row0 + r] : 0.0f;
    }
    if constexpr (MODE == 1) {
      // per-row route, A8W8 row scale s^A and the route's gate weight G[i,k]
      for (int r = t; r < BM; r += NT) {
        if (r < valid) {
          const int64_t p = (int64_t)row0 + r;
          int32_t route = a.pool_src[p];
          if (route < 0 || route >= a.routes) route = -1;   // not a route of this call: row left out
          oroute[r] = route;
          ogw[r] = route >= 0 ? a.topk_w[route] : 0.0f;
          orow[r] = (UC != UC_BF16) ? a.a_scale[p] : 1.0f;
        }
      }
    }
    if constexpr (MODE != 2) __syncthreads();
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const int rlo = pass * EPR;   // rows rlo .. rlo + EPR - 1 of the tile
      if (pass > 0) __syncthreads();   // the previous band has left LDS
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if ((wm * WTM + i * 32) / EPR != pass) continue;
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
              otile[(r - rlo) * OPITCH + oc] = silu(g) * u;
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
              if constexpr (MODE == 2) reinterpret_cast<int32_t*>(otile)[(r - rlo) * OPITCH + oc] = acc[i][j][q];
              else otile[(r - rlo) * OPITCH + oc] = acc_to_f32(acc[i][j][q]) * ws;
            }
          }
        }
      }
      __syncthreads();
      // cooperative row-major pass over the band: 16-byte column chunks, one
      // row per group of CPR consecutive threads (EPR * CPR is a multiple of
      // the thread count, so every thread runs the same number of trips)
      constexpr int CPR = OCOLS / 4;                     // float4 chunks per row
      static_assert((EPR * CPR) % NT == 0 && CPR <= 64 && 64 % CPR == 0, "row groups stay inside a wave");
      for (int idx = t; idx < EPR * CPR; idx += NT) {
        const int rr = idx / CPR, c4 = idx % CPR;
        const int r = rlo + rr;
        const bool ok = r < valid;
        const int64_t p = (int64_t)row0 + r;
        const f32x4 v = *reinterpret_cast<const f32x4*>(otile + rr * OPITCH + c4 * 4);
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
          if (ok && oroute[r] >= 0) *reinterpret_cast<f32x4*>(a.contrib + (int64_t)oroute[r] * a.H + n0 + c4 * 4) = o;
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
  __syncthreads();   // the block is done with LDS
}

// ---------------------------------------------------------------------------
// per-row requantisation of A (A8W8): s^A = max(amax/Qmax, 1e-8), IEEE f32.
// One wave per pool row p; rows past their expert's count (padding) carry no
// route and are skipped.  off_s / cnt_s: the dispatch offsets and counts.
// ---------------------------------------------------------------------------
template <int UC>
__device__ __forceinline__ void requant_row(const RequantArgs& a, int64_t p, const int32_t* off_s, const int32_t* cnt_s) {
  const int l = lane_id();
  if (p >= off_s[a.E] || p >= a.P) return;
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

// ---------------------------------------------------------------------------
// Token Combine: y_i = sum_{k=0..K-1} slot[i*K+k] in slot order, float32;
// masked routes (route_to_pool < 0) contribute nothing.  One thread makes 8
// consecutive columns c .. c+7 of token i.
// ---------------------------------------------------------------------------
// U work items idx0, idx0 + stride, ... (item = token idx / (H/8), columns
// 8 * (idx % (H/8)) ..) at once, so a thread keeps U loads in flight; the
// K contributions of each element are still added in slot order.
template <int U>
__device__ __forceinline__ void combine_8u(const CombineArgs& a, int64_t idx0, int64_t stride, int64_t work) {
  const int64_t nch = a.H / 8;
  float acc[U][8];
  int64_t tok[U];
  int col[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t idx = idx0 + u * stride;
    tok[u] = idx < work ? idx / nch : -1;
    col[u] = (int)(idx % nch) * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[u][c] = 0.0f;
  }
  for (int k = 0; k < a.K; ++k) {
    float4 v[U][2];
    bool on[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = tok[u] * a.K + k;
      on[u] = tok[u] >= 0 && a.route_to_pool[r] >= 0;
      if (on[u]) {
        const float4* src = reinterpret_cast<const float4*>(a.contrib + r * a.H + col[u]);
        v[u][0] = src[0];
        v[u][1] = src[1];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!on[u]) continue;
      acc[u][0] += v[u][0].x; acc[u][1] += v[u][0].y; acc[u][2] += v[u][0].z; acc[u][3] += v[u][0].w;
      acc[u][4] += v[u][1].x; acc[u][5] += v[u][1].y; acc[u][6] += v[u][1].z; acc[u][7] += v[u][1].w;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (tok[u] < 0) continue;
    if (a.y_f32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.y) + tok[u] * a.H + col[u]);
      dst[0] = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
      dst[1] = make_float4(acc[u][4], acc[u][5], acc[u][6], acc[u][7]);
    } else {
      uint4 o;
      o.x = pack_bf16x2(acc[u][0], acc[u][1]);
      o.y = pack_bf16x2(acc[u][2], acc[u][3]);
      o.z = pack_bf16x2(acc[u][4], acc[u][5]);
      o.w = pack_bf16x2(acc[u][6], acc[u][7]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + tok[u] * a.H + col[u]) = o;
    }
  }
}

__device__ __forceinline__ void combine_8(const CombineArgs& a, int64_t i, int c) {
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

}  // namespace mm
