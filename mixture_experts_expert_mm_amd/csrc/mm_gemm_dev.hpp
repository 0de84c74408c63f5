// Device-side bodies of the grouped expert GEMMs on CDNA4 MFMA with fused
// epilogues, the A8W8 requantisation and Token Combine, shared by the
// stand-alone kernels and the fused persistent kernel.
//
// Linear1 (mode 0): per expert e, H_e = X_e . W1[e] over the BLOCK_M-padded
//   pool rows of e (operator page, Expert Compute step 1), then SwiGLU in the
//   epilogue (step 2: A = SiLU(H[:, :I]) * H[:, I:]).  The prepared W1 rows
//   interleave 32 gate columns with the 32 matching up columns, so every lane
//   holds a gate accumulator and its up partner.  A16W16 stores A in bf16;
//   A8W8 dequantises (C * s^W1) * s^X and stores A in float32 for the
//   per-row requantisation (step 3), which finds the row amax itself.
// Linear2 (mode 1): Y_e = A_e . W2[e] (A8W8: (D * s^W2) * s^A), times the
//   route's gate weight G[i,k]; the weighted row is written to the route's
//   float32 combine slot i*K+k (Token Combine sums the slots in order).
// Mode 2 stores the raw int32 accumulators (A8W8-INT exactness checks).
//
// Tiling: one workgroup per BLOCK_M x BN output tile (128 x 256 or 64 x 128);
// each wave owns a 64 x 64 grid of 32x32 MFMA blocks.  K advances 128
// bytes per stage (64 bf16 or 128 int8/e4m3).  Stages are copied from HBM
// straight into a ring of LDS slots by buffer loads (no register staging),
// in a bank-conflict-free swizzled order; the fragment reads of the next
// stage are interleaved with the MFMAs of the current one.  The grid is
// persistent: workgroups stride over the tile list (expert M-blocks x
// N-blocks), whose length is read on the device from the dispatch offsets,
// so no host synchronisation is needed.
#pragma once
#include "mm_device.hpp"
#include "mm_internal.hpp"

#include <type_traits>
#include <utility>

namespace mm {

constexpr int kMaxExperts = 1024;

// Tile shapes (BLOCK_M x BN, WM waves along M x WN along N, S LDS ring
// slots of RB K-bytes per row), one workgroup per CU:
//  * 128 x 256, eight waves (two per SIMD), three slots of 128 K-bytes (the
//    LDS holds no more), for the compute regime;
//  * 256 x 256, four waves (one per SIMD) of 128 x 128, two slots of 64 KiB,
//    for many rows per expert: per K-stage a wave reads 256 rows for
//    2 * 128 * 128 products (128 rows for 2 * 64 * 64 at 128 x 256), which
//    halves the LDS reads, copies and barriers per MFMA.  Its 256
//    accumulator registers take the whole AGPR file of the wave (one wave
//    per SIMD has 512 registers); not for the MX use cases (eight scale
//    rows of 64 per stage, one per wave, need eight waves);
//  * 64 x 128, four waves (one per SIMD), for the weight-streaming regime
//    (few rows per expert): narrow tiles make four times as many tiles out
//    of the same weights, so the last round of tiles leaves fewer CUs idle,
//    and the small stages leave room for six slots, five stages (120 KiB)
//    in flight per CU to cover the HBM latency.
// A wave's N range must hold whole 64-row gate/up groups (WTN >= 64).
template <int BM> struct TileShape;
template <> struct TileShape<64> { static constexpr int WM = 2, WN = 2, BN = 128, S = 6, RB = 128; };
template <> struct TileShape<128> { static constexpr int WM = 2, WN = 4, BN = 256, S = 3, RB = 128; };
template <> struct TileShape<256> { static constexpr int WM = 2, WN = 2, BN = 256, S = 2, RB = 128; };
template <int BM> constexpr int threads_of() { return 64 * TileShape<BM>::WM * TileShape<BM>::WN; }
// The LDS ring of a use case: A rows of RBA bytes per stage (128 K-values
// of 1 byte, 64 of bf16), B rows of RBB bytes (64 for e2m1 weights: the same
// 128 K-values at half a byte each).  The MX use cases also ring one E8M0
// word per A and B row per stage (the four scales of its 128 K-values), 64
// rows per wave (BM + BN rows used); the e2m1 ring's smaller stages leave
// room for more slots.
template <int UC, int BM> struct Ring {
  static constexpr int BN = TileShape<BM>::BN;
  static constexpr int RBA = 128;
  static constexpr int RBB = UC == UC_MX4 ? 64 : 128;
  static constexpr int S = UC == UC_MX4 ? (BM == 64 ? 8 : 4) : TileShape<BM>::S;
  static constexpr int STAGE = BM * RBA + BN * RBB;
  static constexpr int SCALE_STAGE = is_mx(UC) ? threads_of<BM>() * 4 : 0;
};
// Experts the LDS copies of the offsets and counts hold (the MX rings leave
// room for 512).
template <int UC> constexpr int max_experts() { return is_mx(UC) ? 512 : 1024; }
// Per-row data of a tile for its epilogue, two tiles' worth (the next tile's
// is written while the current one is still being stored): 16 bytes a row.
struct RowInfo {
  float gw;        // Linear2: gate weight G[i,k]
  float rs;        // s^X (Linear1, A8W8) or s^A (Linear2, A8W8) of the row
  int32_t route;   // Linear2: route i*K+k of the row (-1: no store)
  float pad;
};
// LDS: the data ring, the row data, the scale ring
template <int UC, int BM> constexpr int lds_bytes_of() {
  return Ring<UC, BM>::S * (Ring<UC, BM>::STAGE + Ring<UC, BM>::SCALE_STAGE) + 2 * BM * (int)sizeof(RowInfo);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS fragment read outside the compiler's view: the compiler would otherwise
// wait for every in-flight LDS-DMA before any LDS read it cannot disambiguate.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t ds_read4(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read8(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
// LDS stores outside the compiler's view (for the same reason as the reads)
template <int OFF>
__device__ __forceinline__ void ds_write2(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b16 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void ds_write2hi(uint32_t addr, uint32_t v) {   // bits 16-31 of v
  asm volatile("ds_write_b16_d16_hi %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void ds_write4(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_wait() { asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N)); }
__device__ __forceinline__ void tie(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(u32x2& v) { asm volatile("" : "+v"(v)); }
// wait until at most VM of this wave's LDS-DMA loads are in flight and all its
// LDS reads returned, then the workgroup barrier
template <int VM>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// One LDS-DMA instruction of stage kb: instruction i of wave wv moves the
// group g = wv + NW*i of RPI = 1024 / RB rows into slot kb % S (groups
// below BM / RPI are A rows).  voff is the lane's byte offset inside its
// group; the group's row offset and the stage's K offset are wave-uniform
// and go in the scalar offset.  The tile bases become buffer descriptors
// here: the descriptor type cannot appear in a signature the host pass sees.
// A rows take the lane's offset voff_a: its row-in-group offset, or, when
// read by token (by_tok), its token row's offset (the group's row offset then
// stays out of the scalar offset); a lane whose row is past the tile's valid
// rows gets an offset beyond the descriptor's range, which loads zeros
// without a memory access.
constexpr uint32_t kOffRange = 0x7fff0000u;   // past any A descriptor's range (< 2^31 bytes)

// A rows take RBA bytes of each K-stage and B rows RBB (half as many for
// e2m1 weights, so a B group moves twice the rows); instruction i < DA of a
// wave moves A rows, the others B rows.  Each instruction fills 1 KiB of the
// stage, so group g lands at byte g*1024 either way.
template <int NW, int BM, int STAGE, int S, int RBA, int RBB>
__device__ __forceinline__ void dma_one(uint8_t* lds, const uint8_t* abase, int abytes, const uint8_t* bbase,
                                        int bbytes, uint32_t voff_b, int wv, int kbytes_a, int kbytes_b, int i, int kb,
                                        int kbase, bool by_tok, uint32_t voff_a) {
  constexpr int RPIA = 1024 / RBA, RPIB = 1024 / RBB;
  constexpr int DA = BM / (RPIA * NW);
  const bool is_a = i < DA;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(is_a ? abase : bbase), (short)0, is_a ? abytes : bbytes, 0x00020000);
  const int soff = is_a ? __builtin_amdgcn_readfirstlane((by_tok ? 0 : RPIA * NW * i) * kbytes_a + (kb + kbase) * RBA)
                        : __builtin_amdgcn_readfirstlane(RPIB * NW * (i - DA) * kbytes_b + (kb + kbase) * RBB);
  const int g = wv + NW * i;
  const uint32_t vo = is_a ? voff_a : voff_b;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds + (kb % S) * STAGE + g * 1024), 16, vo, soff, 0, 0);
}

// The fragments of one K-stage held in registers: NQ 16-byte chunks of the
// wave's MB A blocks and NQB of its NB B blocks.
template <int MB, int NB, int NQ, int NQB = NQ>
struct Frags {
  u32x4 a[MB][NQ];
  u32x4 b[NB][NQB];
};

// Fragment read r of a stage (r = chunk * (MB + NB) + block; A blocks first),
// 32 rows (BOFF bytes) apart inside the wave's rows.  Only called with r
// known at compile time after unrolling, so every branch folds away.
template <int BOFF, int MB, int NB, int NQ>
__device__ __forceinline__ void read_frag(Frags<MB, NB, NQ>& f, int r, const uint32_t* aoff, const uint32_t* boff,
                                          uint32_t so) {
  const int q = r / (MB + NB), x = r % (MB + NB);
  if (x < MB) {
    const uint32_t ad = aoff[q] + so;
    if (x == 0) f.a[0][q] = ds_read16<0>(ad);
    if constexpr (MB > 1) if (x == 1) f.a[1][q] = ds_read16<BOFF>(ad);
    if constexpr (MB > 2) if (x == 2) f.a[2][q] = ds_read16<2 * BOFF>(ad);
    if constexpr (MB > 3) if (x == 3) f.a[3][q] = ds_read16<3 * BOFF>(ad);
  } else {
    const uint32_t ad = boff[q] + so;
    const int y = x - MB;
    if (y == 0) f.b[0][q] = ds_read16<0>(ad);
    if constexpr (NB > 1) if (y == 1) f.b[1][q] = ds_read16<BOFF>(ad);
    if constexpr (NB > 2) if (y == 2) f.b[2][q] = ds_read16<2 * BOFF>(ad);
    if constexpr (NB > 3) if (y == 3) f.b[3][q] = ds_read16<3 * BOFF>(ad);
  }
}

// Fragment read r of a stage for the MX MFMAs (K = 64 per instruction):
// phase p = r / RPP reads A chunks 2p, 2p+1 of each A block, then B chunk
// CPB*p .. CPB*p + CPB-1 of each B block (two e4m3 chunks, or one e2m1
// chunk: 32 values in 16 bytes).  BOFFA / BOFFB: 32 rows apart.
template <int BOFFA, int BOFFB, int MB, int NB, int NQ, int NQB>
__device__ __forceinline__ void read_frag_mx(Frags<MB, NB, NQ, NQB>& f, int r, const uint32_t* aoff,
                                             const uint32_t* boff, uint32_t so) {
  constexpr int CPB = NQB / 2;
  constexpr int RPP = 2 * MB + CPB * NB;
  const int p = r / RPP, x = r % RPP;
  if (x < 2 * MB) {
    const int q = 2 * p + x / MB, i = x % MB;
    const uint32_t ad = aoff[q] + so;
    if (i == 0) f.a[0][q] = ds_read16<0>(ad);
    if constexpr (MB > 1) if (i == 1) f.a[1][q] = ds_read16<BOFFA>(ad);
    if constexpr (MB > 2) if (i == 2) f.a[2][q] = ds_read16<2 * BOFFA>(ad);
    if constexpr (MB > 3) if (i == 3) f.a[3][q] = ds_read16<3 * BOFFA>(ad);
  } else {
    const int y = x - 2 * MB, q = CPB * p + y / NB, j = y % NB;
    const uint32_t ad = boff[q] + so;
    if (j == 0) f.b[0][q] = ds_read16<0>(ad);
    if constexpr (NB > 1) if (j == 1) f.b[1][q] = ds_read16<BOFFB>(ad);
    if constexpr (NB > 2) if (j == 2) f.b[2][q] = ds_read16<2 * BOFFB>(ad);
    if constexpr (NB > 3) if (j == 3) f.b[3][q] = ds_read16<3 * BOFFB>(ad);
  }
}

// 16 e4m3 times an MX scale 2^k -> 16 bf16 (exact: e4m3 values times a
// power of two within the float range are bf16 values)
__device__ __forceinline__ void widen_e4m3_scaled(const u32x4& w, float s, u32x4& lo, u32x4& hi) {
#define CVT(x, hi_) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((x), s, (hi_)))
  lo = u32x4{CVT(w[0], false), CVT(w[0], true), CVT(w[1], false), CVT(w[1], true)};
  hi = u32x4{CVT(w[2], false), CVT(w[2], true), CVT(w[3], false), CVT(w[3], true)};
#undef CVT
}
// 32 e2m1 (16 bytes, the even K in the low nibble) times 2^k -> four
// operands of 8 bf16 in K order (exact)
__device__ __forceinline__ void widen_e2m1_scaled(const u32x4& w, float s, u32x4* o) {
#define CVT(x, b_) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((x), s, (b_)))
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = u32x4{CVT(w[d], 0), CVT(w[d], 1), CVT(w[d], 2), CVT(w[d], 3)};
#undef CVT
}

// 16 e4m3 -> 16 bf16 (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ void widen_e4m3(const u32x4& w, u32x4& lo, u32x4& hi) {
#define CVT(x, hi_) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((x), 1.0f, (hi_)))
  lo = u32x4{CVT(w[0], false), CVT(w[0], true), CVT(w[1], false), CVT(w[1], true)};
  hi = u32x4{CVT(w[2], false), CVT(w[2], true), CVT(w[3], false), CVT(w[3], true)};
#undef CVT
}

// Mainloop data layout.  A stage holds BLOCK_M A rows then BN B rows of RB
// K-bytes (CH = RB/16 chunks of 16 bytes) each, filled by buffer loads
// straight into LDS: one wave instruction moves 1 KiB = 1024/RB rows (64
// lanes x 16 bytes, lane i -> byte 16*i of the group).  Chunk c of row r
// sits at position c ^ ((r / (16/CH)) % CH): LDS serves a 16-byte read of 16
// lanes per pass over 64 banks (16 groups of 16 bytes), and 16 consecutive
// rows at one chunk then hit 16 distinct bank groups.  A lane's MFMA operand
// covers chunks NQ*h .. NQ*h+NQ-1 of its row (h = lane / 32, NQ = CH/2),
// the same chunks for A and B, so every product pairs equal k.
//
// Tiles run back to back: once a tile's last MFMAs are issued the ring is
// free, so the first stages of the workgroup's next tile are issued at once
// and the finished tile's epilogue (stores straight from the accumulators:
// lanes 0-31 and 32-63 each write 32 consecutive columns of one row) runs
// while they are in flight.

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

// The same pointer typed as global memory: after the round trip through an
// integer the compiler no longer knows the address space and would use flat
// instructions.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gp(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

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
  a.a_scale = uniform_ptr(in.a_scale);
  a.topk_w = uniform_ptr(in.topk_w);
  a.contrib = uniform_ptr(in.contrib);
  a.raw_out = uniform_ptr(in.raw_out);
  a.a_mx = uniform_ptr(in.a_mx);
  a.a_mx_rows = (int64_t)uniform_int((int)in.a_mx_rows);   // < 2^31 (checked by the host)
  a.b_mx = uniform_ptr(in.b_mx);
  a.out_mx = uniform_ptr(in.out_mx);
  a.err = uniform_ptr(in.err);
  a.E = uniform_int(in.E);
  a.N = uniform_int(in.N);
  a.Kdim = uniform_int(in.Kdim);
  a.I = uniform_int(in.I);
  a.H = uniform_int(in.H);
  a.K = uniform_int(in.K);
  a.Kr = uniform_int(in.Kr);
  a.gate_up_group = uniform_int(in.gate_up_group);
  a.group_m = uniform_int(in.group_m);
  a.a_route = uniform_ptr(in.a_route);
  a.a_rows = (int64_t)uniform_int((int)in.a_rows);   // < 2^31 (checked by the host)
  a.partials = uniform_ptr(in.partials);
  a.dep_done = uniform_ptr(in.dep_done);
  a.dep_wait = uniform_ptr(in.dep_wait);
  a.dep_target = (uint32_t)uniform_int((int)in.dep_target);
  a.claim = uniform_ptr(in.claim);
  a.steal = uniform_int(in.steal);
  a.split_flags = uniform_ptr(in.split_flags);
  a.max_split = uniform_int(in.max_split);
  a.clamp = __builtin_bit_cast(float, uniform_int(__builtin_bit_cast(int, in.clamp)));
  a.spin_limit = (uint32_t)uniform_int((int)in.spin_limit);
  return a;
}

// One item of the workgroup's work list: a tile, or a K piece of a split
// tail tile, resolved.
enum TileRole : int { kRoleFull = 0, kRoleReduce = 1, kRoleProduce = 2 };
struct TileRef {
  int e, row0, n0, valid;
  const uint8_t* abase;   // first A row of the tile
  const uint8_t* bbase;   // first B row (prepared weights) of the tile
  int kbase, nkl;         // K stages kbase .. kbase + nkl - 1
  uint32_t aoa[8];        // per lane: byte offsets of its A rows' chunks (A read by token)
  uint32_t sc;            // MX: per lane, byte offset of the scale row it moves (or one past the range)
  int role;               // TileRole: whole tile, or piece 0 (adds the others' partials), or a later piece
  int slot;               // partial slot of a piece (piece 0: the later pieces use slot + 1 ..)
};

constexpr int kMinSplitStages = 4;   // shortest K piece of a split tile

// K pieces per tail tile.  A slice of n tiles on G workgroups runs n / G full
// rounds and then `tail` tiles; split in c pieces they take ceil(tail*c/G)
// rounds of 1/c of a tile.  c divides G (the pieces of one tile run in the
// same round) and tail*c <= 2G (two partial slots per workgroup).  Depends
// only on the arguments, so every launch shape that has the same grid splits
// the same way.
__device__ __forceinline__ int split_factor(int tail, int G, int nk, int max_split, int grid) {
  if (max_split < 2 || tail <= 0 || 2 * grid > kSplitSlots) return 1;
  int best = 1;
  for (int c = 2; c <= 8 && c <= max_split; c *= 2) {
    if (G % c != 0 || nk / c < kMinSplitStages || tail * c > 2 * G) continue;
    const int rc = (tail * c + G - 1) / G, rb = (tail * best + G - 1) / G;
    if (rc * best < rb * c) best = c;
  }
  return best;
}

// Copies issued after MFMA slot g (from 0) when DT copies spread evenly over
// `slots` MFMAs.
constexpr int dma_after(int g, int dt, int slots) { return ((g + 1) * dt + slots - 1) / slots < dt ? ((g + 1) * dt + slots - 1) / slots : dt; }

// An accumulator element as a 32-bit word and back.  The element is passed
// by value: a bit cast applied directly to a vector element expression was
// compiled into a read of element 0.
__device__ __forceinline__ uint32_t word_of(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t word_of(int32_t x) { return (uint32_t)x; }
template <typename E> __device__ __forceinline__ E from_word(uint32_t w);
template <> __device__ __forceinline__ float from_word<float>(uint32_t w) { return __uint_as_float(w); }
template <> __device__ __forceinline__ int32_t from_word<int32_t>(uint32_t w) { return (int32_t)w; }

__device__ __forceinline__ bool poll_flag(uint32_t* p, uint32_t spin_limit) {
  uint32_t polls = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
    if (++polls > spin_limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

// Tile order: expert-major; inside an expert, groups of group_m M-blocks
// (0: all of them), and in a group N-block-major, M-block fastest.  With
// group_m = 8 the 32 workgroups of an XCD run 8 M-blocks x 4 N-blocks of one
// expert at a time and per K-stage read 8 activation and 4 weight stages
// (the fewest bytes for 32 tiles when activation rows come from the pool);
// without groups they read one weight stage and up to 32 activation stages.
// Tiles are counted inside an XCD's slice of M-blocks [mb_beg, mb_end): an
// expert's M-blocks clipped to the slice, times the N-blocks.  The expert of
// a tile is the largest e with (clip(off[e] / BM) - mb_beg) * n_tiles <= tile.
template <int BM>
__device__ __forceinline__ TileRef resolve_tile(const GemmArgs& a, const int32_t* off_s, const int32_t* cnt_s,
                                               int tile, int n_tiles, int kbytes, int kbytes_b, int mb_beg,
                                               int mb_end) {
  auto first_mb = [&](int e) { return min(max(off_s[e] / BM, mb_beg), mb_end); };
  int lo = 0, hi = a.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((first_mb(mid) - mb_beg) * n_tiles <= tile) lo = mid; else hi = mid;
  }
  // every field is wave-uniform; saying so keeps them in scalar registers
  // (a tile base the compiler cannot prove uniform would turn each buffer
  // load into a loop over lanes)
  TileRef r;
  r.e = uniform_int(lo);
  const int mb0 = first_mb(lo), nmb = first_mb(lo + 1) - mb0;
  const int local = tile - (mb0 - mb_beg) * n_tiles;
  const int GM = a.group_m > 0 ? a.group_m : nmb;   // M-blocks per group (0: the whole expert)
  const int g = local / (GM * n_tiles), gm = min(GM, nmb - g * GM);
  const int idx = local - g * GM * n_tiles;
  const int nblk = idx / gm, mblk = mb0 + g * GM + idx % gm;
  r.row0 = uniform_int(mblk * BM);
  r.n0 = uniform_int(nblk * TileShape<BM>::BN);
  r.valid = uniform_int(min(BM, off_s[lo] + cnt_s[lo] - r.row0));
  r.abase = uniform_ptr(a.a_route ? a.A : a.A + (int64_t)r.row0 * kbytes);
  r.bbase = uniform_ptr(a.B + ((int64_t)r.e * a.N + r.n0) * kbytes_b);
  return r;
}

template <int UC, int BM, int MODE, bool WIDEN>
__device__ __forceinline__ void gemm_tiles(const GemmArgs& args, uint8_t* lds, int32_t* off_s, int32_t* cnt_s) {
  const GemmArgs a = uniform_args(args);
  constexpr bool MX = is_mx(UC), B4 = UC == UC_MX4;
  // MX on the scaled MX MFMA, or (MXW, Linear1's exact mode) on the bf16
  // MFMA after widening each e4m3 / e2m1 value times its block scale to bf16
  constexpr bool MXI = MX && !WIDEN, MXW = MX && WIDEN;
  constexpr int WM = TileShape<BM>::WM, WN = TileShape<BM>::WN, S = Ring<UC, BM>::S;
  constexpr int NT = threads_of<BM>(), NW = NT / 64;
  constexpr int BN = TileShape<BM>::BN, RB = Ring<UC, BM>::RBA, RBB = Ring<UC, BM>::RBB;
  constexpr int CH = RB / 16, NQ = CH / 2;                 // A: chunks per row; per lane and block
  constexpr int CHB = RBB / 16, NQB = CHB / 2;             // B: the same
  constexpr int RPI = 1024 / RB, RPIB = 1024 / RBB;        // rows per DMA instruction
  constexpr int RPS = 16 / CH, RPSB = 16 / CHB;            // rows per swizzle step
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int STAGE = Ring<UC, BM>::STAGE;
  constexpr int SSTAGE = Ring<UC, BM>::SCALE_STAGE;
  constexpr int GA = BM / RPI, GB = BN / RPIB, GROUPS = GA + GB;
  static_assert(GROUPS % NW == 0 && GA % NW == 0, "DMA groups must split evenly over the waves");
  constexpr int D = GROUPS / NW;                           // data DMA instructions per wave per stage
  // MX: one scale DMA instruction per wave and stage, 64 rows' E8M0 words:
  // waves 0 .. BM/64-1 the A rows, the next BN/64 the B rows, the others
  // none (their loads read zeros into the unused rest of the scale slot).
  // No lane is masked off, so the step stays free of branches.
  constexpr int DT = D + (MX ? 1 : 0);                     // DMA instructions per wave per stage
  static_assert(!MX || (BM % 64 == 0 && BN % 64 == 0 && (BM + BN) / 64 <= NW), "scale rows per wave");
  static_assert((S - 1) * DT <= 63, "vmcnt range");
  constexpr int ESZ = (UC == UC_BF16) ? 2 : 1;
  constexpr int NFR = MB + NB;                             // fragment reads per chunk index
  // MFMA phases of a stage: one chunk each, or two for e4m3 / MX MFMAs (K = 64)
  constexpr int CPP = ((UC == UC_FP8 && !WIDEN) || MX) ? 2 : 1;
  constexpr int NPH = NQ / CPP;
  static_assert(NPH >= 2, "a stage needs MFMA phases after its barrier to hide the refill and the reads");
  static_assert(!MX || NPH == 2, "MX phases select scale bytes 0 and 2");
  constexpr int RPP = MX ? 2 * MB + (NQB / 2) * NB : NFR * CPP;   // fragment reads per phase
  constexpr int NSR = MX ? MB + NB : 0;                    // scale-word reads per stage (before the fragments)
  constexpr int MPP = MB * NB * (MXW ? 4 : WIDEN ? 2 : 1); // MFMAs per phase
  // phase 0 may start once only the reads of the later phases are in flight
  constexpr int P0WAIT = (NPH - 1) * RPP > 15 ? 15 : (NPH - 1) * RPP;
  static_assert(BM % (RPI * NW) == 0, "A rows fill whole DMA instructions");
  static_assert(MODE != 0 || NB % 2 == 0, "Linear1 waves hold whole gate/up pairs");
  typedef typename Acc<UC>::type AccT;
  typedef std::conditional_t<UC == UC_I8, int32_t, float> AccE;   // one accumulator element

  const int t = threadIdx.x, l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(t / 64);
  const int h = l / 32, lr = l % 32;
  const int wm = wv / WN, wn = wv % WN;

  for (int e = t; e <= a.E; e += NT) off_s[e] = gp(a.offsets)[e];
  for (int e = t; e < a.E; e += NT) cnt_s[e] = gp(a.counts)[e];
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

  const int kbytes = a.Kdim * ESZ;                         // A bytes per row
  const int kbytes_b = B4 ? a.Kdim / 2 : kbytes;           // B bytes per row
  const int nk = kbytes / RB;
  const int n_tiles = a.N / BN;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  RowInfo* rowinfo = reinterpret_cast<RowInfo*>(lds + S * STAGE);   // [2][BM]
  const uint32_t rowinfo_base = lds_base + (uint32_t)(S * STAGE);
  // MX scale ring: per slot, BM A words then BN B words
  uint8_t* const scl = lds + S * STAGE + 2 * BM * (int)sizeof(RowInfo);
  const uint32_t scl_base = lds_base + (uint32_t)(S * STAGE + 2 * BM * (int)sizeof(RowInfo));

  // per-lane LDS addresses of the NQ fragment chunks (stage slot added per
  // stage); the wave's first rows are a multiple of 16, the swizzle period.
  // Chunk q of lane half h is the row's 16-byte chunk NQ*h + q, except for
  // the MX MFMAs, whose block scales follow the instruction's K layout: in
  // an e4m3 operand, bytes 0-15 of both lane halves form K-block 0 and bytes
  // 16-31 K-block 1 (scaled by lane half 0's and 1's scale); in an e2m1
  // operand each lane half holds one K-block.  So lane half h takes chunks
  // 2q + h: phase p's blocks are then the stage's MX groups 2p and 2p+1.
  uint32_t aoff[NQ], boff[NQB];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = MXI ? 2 * q + h : NQ * h + q;
    aoff[q] = lds_base + (uint32_t)(wm * WTM + lr) * RB + (uint32_t)((c ^ ((lr / RPS) % CH)) << 4);
  }
#pragma unroll
  for (int q = 0; q < NQB; ++q) {
    const int c = MXI ? 2 * q + h : NQB * h + q;
    boff[q] = lds_base + (uint32_t)(BM * RB) + (uint32_t)(wn * WTN + lr) * RBB + (uint32_t)((c ^ ((lr / RPSB) % CHB)) << 4);
  }
  // MX: the lane's A-row and B-row scale words (slot added per stage)
  const uint32_t asc_rd = scl_base + (uint32_t)(wm * WTM + lr) * 4;
  const uint32_t bsc_rd = scl_base + (uint32_t)(BM + wn * WTN + lr) * 4;
  // per-lane byte offset of the DMA rows: group g covers rows RPI*g ..
  // RPI*g + RPI-1, lane l row RPI*g + l/CH, and lands its logical chunk
  // (l%CH) ^ swizzle(row) at position l%CH.  The swizzle of a lane's row is
  // the same in all of a wave's groups g = wv + NW*i: their row offsets
  // differ by RPI*NW*i, a multiple of the swizzle period RPS*CH (needs NW
  // even when CH = 8).  B rows alike with their own width.
  static_assert((RPI * NW / RPS) % CH == 0, "DMA swizzle must repeat across a wave's groups");
  static_assert((RPIB * NW / RPSB) % CHB == 0, "DMA swizzle must repeat across a wave's groups");
  const uint32_t vchunk = (uint32_t)(((l % CH) ^ (((RPI * wv + l / CH) / RPS) % CH)) << 4);
  const uint32_t voff = (uint32_t)((RPI * wv + l / CH) * kbytes) + vchunk;
  const uint32_t vchunk_b = (uint32_t)(((l % CHB) ^ (((RPIB * wv + l / CHB) / RPSB) % CHB)) << 4);
  const uint32_t voff_b = (uint32_t)((RPIB * wv + l / CHB) * kbytes_b) + vchunk_b;
  // A read by token: the A buffer is the T token rows, each lane's rows come
  // from the route of their pool row (padding rows read token 0, unused)
  const bool by_tok = MODE == 0 && a.a_route != nullptr;   // only Linear1 reads token rows in place
  constexpr int DA = BM / (RPI * NW);                      // A instructions per wave and stage
  static_assert(DA <= 8, "per-lane A row offsets of at most eight instructions");
  const int abytes = by_tok ? (int)(a.a_rows * kbytes) : BM * kbytes, bbytes = BN * kbytes_b;
  // MX scale rows: a_mx [a_mx_rows][G], b_mx [E][N][G] bytes, G = Kdim / 32
  const int gbytes = a.Kdim / kMxGroup;
  const int asc_bytes = MX ? (int)(a.a_mx_rows * gbytes) : 0;
  const int bsc_bytes = MX ? a.E * a.N * gbytes : 0;
  // One DMA instruction x of stage kb of tile tr: x < D data, x = D the
  // wave's 64 scale rows (lane l: row 64*wv + l of the slot, A rows then B
  // rows), each lane's word landing at its row's word.
  const bool scale_a = wv < BM / 64;
  // (each field read on its own: a select between the two fields' addresses
  // would put a copy of the arguments in scratch memory)
  const void* const scale_src = scale_a ? (const void*)uniform_ptr(a.a_mx) : (const void*)uniform_ptr(a.b_mx);
  const int scale_bytes = uniform_int(scale_a ? asc_bytes : bsc_bytes);
  auto dma_x = [&](const TileRef& tr, int x, int kb) {
    if (x < D) {
      dma_one<NW, BM, STAGE, S, RB, RBB>(lds, tr.abase, abytes, tr.bbase, bbytes, voff_b, wv, kbytes, kbytes_b, x, kb,
                                         tr.kbase, by_tok,
                                         by_tok ? tr.aoa[x < DA ? x : 0]
                                                : (RPI * (wv + NW * x) + l / CH < tr.valid ? voff : kOffRange));
    } else if constexpr (MX) {
      const int soff = __builtin_amdgcn_readfirstlane((kb + tr.kbase) * 4);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)scale_src, (short)0, scale_bytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(scl + (kb % S) * SSTAGE + 64 * wv * 4), 4, tr.sc, soff,
                                               0, 0);
    }
  };
#define MM_DMA(tr_, i_, kb_) dma_x((tr_), (i_), (kb_))

  // Per-row epilogue data of a tile, thread t holding row t: loaded into
  // registers when the tile's stages go out (the loads that need the route
  // once the tile's first stage has landed, by then the route has arrived),
  // written to rowinfo[buf] when the tile's mainloop is done.  No wait for
  // row data holds back the tile's stages.
  static_assert(BM <= NT, "one row per thread");
  // A8W8: the per-output-channel scales of the lane's columns ride along
  // (loaded with the row data, before the tile's copies; the epilogue reads
  // them without a wait)
  constexpr bool COLS = UC != UC_BF16 && !MX && MODE != 2;
  constexpr int NCS = COLS ? NB : 1;
  struct RowRegs {
    int32_t route;
    float gw, rs;
    float cs0[NCS], cs1[MODE == 0 ? NCS : 1];   // cs1: Linear1's up columns
  };
  auto row_blank = [&]() {
    RowRegs rr;
    rr.route = -1;
    rr.gw = 0.0f;
    rr.rs = 1.0f;
#pragma unroll
    for (int j = 0; j < NCS; ++j) rr.cs0[j] = 1.0f;
#pragma unroll
    for (int j = 0; j < (MODE == 0 ? NCS : 1); ++j) rr.cs1[j] = 1.0f;
    return rr;
  };
  auto row_first = [&](const TileRef& tr) {
    RowRegs rr = row_blank();
#pragma unroll
    for (int j = 0; j < NCS; ++j) {
      if constexpr (MODE == 0 && COLS) {
        if (j < NB / 2) {
          const int col = tr.n0 / 2 + wn * (WTN / 2) + j * 32 + lr;
          rr.cs0[j] = gp(a.w_scale)[(int64_t)tr.e * 2 * a.I + col];           // gate column
          rr.cs1[j] = gp(a.w_scale)[(int64_t)tr.e * 2 * a.I + a.I + col];     // up column
        }
      }
      if constexpr (MODE == 1 && COLS) rr.cs0[j] = gp(a.w_scale)[(int64_t)tr.e * a.H + tr.n0 + wn * WTN + j * 32 + lr];
    }
    if (t < tr.valid) {
      const int64_t p = (int64_t)tr.row0 + t;
      if constexpr (MODE == 0 && UC != UC_BF16 && !MX) {
        if (by_tok) rr.route = gp(a.a_route)[p];
        else rr.rs = gp(a.x_scale)[p];
      }
      if constexpr (MODE == 1) {
        rr.route = gp(a.pool_src)[p];
        if constexpr (UC != UC_BF16 && !MX) rr.rs = gp(a.a_scale)[p];
      }
    }
    return rr;
  };
  auto row_second = [&](RowRegs& rr) {
    // the tile's first stage has landed, so have the column scales (issued
    // before it): taken here, at a wait the compiler sees as complete
#pragma unroll
    for (int j = 0; j < NCS; ++j) asm volatile("" : "+v"(rr.cs0[j]));
    if constexpr (MODE == 0) {
#pragma unroll
      for (int j = 0; j < NCS; ++j) asm volatile("" : "+v"(rr.cs1[j]));
    }
    if constexpr (MODE == 0 && UC != UC_BF16 && !MX) {
      if (by_tok) rr.rs = rr.route >= 0 ? gp(a.x_scale)[rr.route / a.K] : 1.0f;
    }
    if constexpr (MODE == 1) {
      if (rr.route < 0 || rr.route >= a.routes) rr.route = -1;   // not a route of this call: row left out
      // routed slot k < Kr: G[i,k]; a shared-expert slot: weight 1
      const int slot = rr.route >= 0 ? rr.route % a.K : 0;
      rr.gw = rr.route < 0 ? 0.0f : slot < a.Kr ? gp(a.topk_w)[(rr.route / a.K) * a.Kr + slot] : 1.0f;
    }
  };
  auto row_commit = [&](const RowRegs& rr, int buf) {
    if (t < BM) rowinfo[buf * BM + t] = RowInfo{rr.gw, rr.rs, MODE == 1 ? rr.route : -1, 0.0f};
  };
  // The first S stages of tile `tr`, after its row data loads.
  // Between tiles the first stage goes out before the finished tile's
  // epilogue and the others after it: the epilogue's stores, counted with
  // the loads in order, then complete with stage 0 and do not hold up the
  // next tile's first wait.
  auto start_first = [&](const TileRef& tr) {
    const RowRegs rr = row_first(tr);
#pragma unroll
    for (int x = 0; x < DT; ++x) MM_DMA(tr, x, 0);
    return rr;
  };
  auto start_rest = [&](const TileRef& tr) {
#pragma unroll
    for (int st = 1; st < S; ++st)
      if (st < tr.nkl) {
#pragma unroll
        for (int x = 0; x < DT; ++x) MM_DMA(tr, x, st);
      }
  };
  auto start_tile = [&](const TileRef& tr) {
    const RowRegs rr = start_first(tr);
    start_rest(tr);
    return rr;
  };

  // Workgroup w runs on XCD w % 8 (round-robin dispatch); each XCD walks the
  // tiles of its own contiguous slice of M-blocks, all their N-blocks, so the
  // sharing happens inside one L2 and every tile of an M-block runs on the
  // same XCD (measured: bf16 16K tokens 1.5% faster than equal tile counts).
  const int nxcd = gridDim.x >= 8 ? 8 : 1;
  const int xcd = blockIdx.x % nxcd, wgx = blockIdx.x / nxcd, per_x = gridDim.x / nxcd;
  const int n_mb = offsets_ok ? off_s[a.E] / BM : 0;
  const int mb_slice = (n_mb + nxcd - 1) / nxcd;
  const int mb_beg = min(n_mb, xcd * mb_slice), mb_end = min(n_mb, mb_beg + mb_slice);
  const int t_beg = 0, t_end = (mb_end - mb_beg) * n_tiles;
  const bool in_grid = (int)blockIdx.x < per_x * nxcd;   // a tail beyond a multiple of 8 stays idle

  // Work list of this workgroup: the slice's full rounds of tiles round
  // robin, then its tail tiles (fewer than one per workgroup) split along K
  // into sk pieces each, so that the last round ends sooner.  Piece p of the
  // tail goes to workgroup p % G; piece 0 of a tile adds the partial sums of
  // the tile's later pieces (in piece order) and runs the epilogue.
  const int n_s = in_grid ? max(0, t_end - t_beg) : 0;
  const int full = n_s / per_x, tail = n_s - full * per_x;
  // no K split at 256 x 256 (its accumulators fill the register file; a
  // loop that adds partial sums into them would spill them)
  constexpr bool CAN_SPLIT = BM != 256;
  // Dynamic tiles (the fused kernel, a.claim set; smaller tiles only with
  // at least 8 tiles per workgroup, where the last round matters little):
  // the workgroups of an XCD take the slice's tiles in order from a counter
  // of their XCD, each claiming its next tile when it starts the current
  // one, so a workgroup that runs faster takes more tiles.  A workgroup
  // whose XCD's slice is exhausted goes on claiming from the next XCDs'
  // counters (a.steal), so a faster XCD takes tiles of a slower one.  Item j
  // of XCD x is tile j of x's slice, whole (no K split).
  const bool dyn = a.claim != nullptr && in_grid && (BM == 256 || n_s >= 8 * per_x);
  const int sk = CAN_SPLIT && !dyn ? split_factor(tail, per_x, nk, a.max_split, (int)gridDim.x) : 1;
  const int pieces = tail * sk;
  const int n_items = full + (pieces > wgx ? (pieces - wgx + per_x - 1) / per_x : 0);
  __shared__ int32_t claim_s[2];
  int cx = xcd, cx_beg = mb_beg, cx_end = mb_end, cx_ns = n_s;   // the XCD whose tiles are being claimed
  auto set_cx = [&](int x) {
    cx = x;
    cx_beg = min(n_mb, x * mb_slice);
    cx_end = min(n_mb, cx_beg + mb_slice);
    cx_ns = (cx_end - cx_beg) * n_tiles;
  };
  // thread 0: the claim v of XCD x, moved on to the next XCDs while their
  // slices are exhausted; into claim_s (x = -1: none left)
  auto settle_claim = [&](uint32_t v) {
    int x = cx, left = a.steal ? nxcd - 1 : 0;
    const auto ns_of = [&](int y) {
      const int b = min(n_mb, y * mb_slice);
      return (min(n_mb, b + mb_slice) - b) * n_tiles;
    };
    while ((int)v >= ns_of(x) && left > 0) {
      x = (x + 1) % nxcd;
      --left;
      v = __hip_atomic_fetch_add(a.claim + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    claim_s[0] = (int)v;
    claim_s[1] = (int)v < ns_of(x) ? x : -1;
  };
  auto make_item = [&](int j) {
    TileRef r;
    if (dyn || j < full) {
      r = resolve_tile<BM>(a, off_s, cnt_s, t_beg + (dyn ? j : wgx + j * per_x), n_tiles, kbytes, kbytes_b,
                           dyn ? cx_beg : mb_beg, dyn ? cx_end : mb_end);
      r.kbase = 0;
      r.nkl = nk;
      r.role = kRoleFull;
      r.slot = 0;
    } else {
      const int p = wgx + (j - full) * per_x, sub = p % sk;
      r = resolve_tile<BM>(a, off_s, cnt_s, t_beg + full * per_x + p / sk, n_tiles, kbytes, kbytes_b, mb_beg,
                           mb_end);
      r.kbase = uniform_int(sub * nk / sk);
      r.nkl = uniform_int((sub + 1) * nk / sk - sub * nk / sk);
      r.role = sk == 1 ? kRoleFull : (sub == 0 ? kRoleReduce : kRoleProduce);
      r.slot = uniform_int(xcd * 2 * per_x + p);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) r.aoa[x] = 0;
    if (by_tok) {
      // every route load first, then the offsets: one round trip, and no
      // branch between the loads (a route < 0, a padding row, reads zeros).
      // The lane id is laundered so that the row addresses are not computed
      // ahead of the tile loop and kept live through the mainloop.
      int lm = l;
      asm volatile("" : "+v"(lm));
      int32_t route[DA];
#pragma unroll
      for (int x = 0; x < DA; ++x) route[x] = gp(a.a_route)[(int64_t)r.row0 + RPI * (wv + NW * x) + lm / CH];
#pragma unroll
      for (int x = 0; x < DA; ++x) {
        const uint32_t tok = (uint32_t)max(route[x], 0) / (uint32_t)a.K;
        r.aoa[x] = route[x] >= 0 ? tok * (uint32_t)kbytes + vchunk : kOffRange;
      }
    }   // (pool rows: the offsets follow from the valid count when the copies go out)
    r.sc = 0;
    if constexpr (MX) {
      // A-scale waves: tile row 64*wv + l (its token row when A is read by
      // token); past the valid rows an offset beyond the range (the word
      // reads as zero; the row's data is zero too).  B-scale waves: column
      // n0 + 64*(wv - BM/64) + l in formula order (Linear1's prepared rows
      // interleave gate and up columns in groups of gate_up_group).  Other
      // waves: beyond the range.
      if (scale_a) {
        const int row = 64 * wv + l;
        if (by_tok) {
          const int32_t route = gp(a.a_route)[(int64_t)r.row0 + row];
          r.sc = route >= 0 ? ((uint32_t)max(route, 0) / (uint32_t)a.K) * (uint32_t)gbytes : kOffRange;
        } else {
          r.sc = row < r.valid ? (uint32_t)((r.row0 + row) * gbytes) : kOffRange;
        }
      } else if (wv < (BM + BN) / 64) {
        int n = r.n0 + 64 * (wv - BM / 64) + l;
        if (MODE == 0 && a.gate_up_group > 0) {
          const int g2 = 2 * a.gate_up_group, qq = n / g2, m = n % g2;
          n = m < a.gate_up_group ? qq * a.gate_up_group + m : a.I + qq * a.gate_up_group + (m - a.gate_up_group);
        }
        r.sc = (uint32_t)(((int64_t)r.e * a.N + n) * gbytes);
      } else {
        r.sc = kOffRange;
      }
    }
    return r;
  };

  // Dependency schedule of the fused kernel.  Linear2: before the first
  // copy of a tile of M-block b, wait until dep_wait[b] >= dep_target; one
  // wave-wide load reads the counters of 64 blocks, and blocks seen complete
  // are not polled again.  Linear1: a tile counts for its M-block once its
  // stores are complete (pend_mb, below).
  int dw_base = 0, pend_mb = -1;
  uint64_t dw_mask = 0;
  auto dep_ready = [&](int mb) {
    if constexpr (MODE != 1) return;
    if (a.dep_wait == nullptr || dw_base == 0x40000000) return;
    if (mb >= dw_base && mb < dw_base + 64 && ((dw_mask >> (mb - dw_base)) & 1u)) return;
    if (mb < dw_base || mb >= dw_base + 64) dw_base = mb;
    uint32_t polls = 0;
    for (;;) {
      const int q = dw_base + l;
      const uint32_t v = q < n_mb ? __hip_atomic_load(a.dep_wait + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      dw_mask = __ballot(v >= a.dep_target);
      if ((dw_mask >> (mb - dw_base)) & 1u) break;
      if (++polls > a.spin_limit) {   // gives up: flagged, and no later wait of this wave polls
        if (l == 0 && a.err) atomicOr(a.err, (uint32_t)MM_DEVERR_BARRIER_TIMEOUT);
        dw_base = 0x40000000;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    asm volatile("" ::: "memory");
  };

  int item = 0;
  bool have = item < n_items;
  if (dyn) {
    if (t == 0) settle_claim(__hip_atomic_fetch_add(a.claim + xcd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(claim_s[0]);
    const int x = __builtin_amdgcn_readfirstlane(claim_s[1]);
    have = x >= 0;
    if (have) set_cx(x);
  }
  TileRef cur{};
  RowRegs rr_cur = row_blank();
  int buf = 0;
  if (have) {
    cur = make_item(item);
    dep_ready(cur.row0 / BM);
    rr_cur = start_tile(cur);
  }
  // thread 0: the claim for the item after this one, made when this item
  // starts (at 256 x 256, whose next item is settled after the epilogue,
  // when its epilogue starts: nothing held through the main loop)
  uint32_t claim_v = 0;
  while (have) {
    if (BM != 256 && dyn && t == 0)
      claim_v = __hip_atomic_fetch_add(a.claim + cx, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    AccT acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

    Frags<MB, NB, NQ, NQB> f;
    // MX: the scale words of the A rows and B columns of the stage being
    // computed (shifted so that byte p is the lane's group of phase p) and
    // of the next stage (being read)
    uint32_t sa_c[MX ? MB : 1], sb_c[MX ? NB : 1], sa_n[MX ? MB : 1], sb_n[MX ? NB : 1];
    // MXW: the block scales of phases 0 and 1 as floats (lane half h, phase
    // p: the stage's K-group 2h + p); a zero E8M0 byte (2^-127, all-zero or
    // tiny groups) widens as 0
    float saf[MXW ? MB : 1][2], sbf[MXW ? NB : 1][2];
    auto read_scales = [&](uint32_t ss) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < MB; ++i) sa_n[i] = ds_read4<0>(asc_rd + ss + (uint32_t)(i * 32 * 4));
#pragma unroll
        for (int j = 0; j < NB; ++j) sb_n[j] = ds_read4<0>(bsc_rd + ss + (uint32_t)(j * 32 * 4));
      }
    };
    // after the wait for the stage's first reads: its scale words.  Lane half
    // h supplies the scale of K-block h, which in phase p is the stage's
    // group 2p + h: byte 2p of the word shifted down by 8h bits.
    auto take_scales = [&]() {
      if constexpr (MXI) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          tie(sa_n[i]);
          sa_c[i] = sa_n[i] >> (8 * h);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          tie(sb_n[j]);
          sb_c[j] = sb_n[j] >> (8 * h);
        }
      } else if constexpr (MXW) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          tie(sa_n[i]);
#pragma unroll
          for (int p = 0; p < 2; ++p) saf[i][p] = __uint_as_float(((sa_n[i] >> (8 * (2 * h + p))) & 0xffu) << 23);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          tie(sb_n[j]);
#pragma unroll
          for (int p = 0; p < 2; ++p) sbf[j][p] = __uint_as_float(((sb_n[j] >> (8 * (2 * h + p))) & 0xffu) << 23);
        }
      }
    };
    // all fragment reads of a stage, slot offset so (scale words first)
    auto read_stage = [&](uint32_t so) {
      if constexpr (MX) {
        read_scales((so / STAGE) * SSTAGE);
#pragma unroll
        for (int r = 0; r < NPH * RPP; ++r) read_frag_mx<32 * RB, 32 * RBB>(f, r, aoff, boff, so);
      } else {
#pragma unroll
        for (int r = 0; r < NQ * NFR; ++r) read_frag<32 * RB>(f, r, aoff, boff, so);
      }
    };
    auto read_one = [&](int r, uint32_t so) {
      if constexpr (MX) read_frag_mx<32 * RB, 32 * RBB>(f, r, aoff, boff, so);
      else read_frag<32 * RB>(f, r, aoff, boff, so);
    };
    // MFMA mi of phase p (chunks CPP*p .. CPP*p + CPP-1 of the stage in f)
    u32x4 wa_lo[MB], wa_hi[MB], wb_lo, wb_hi;   // e4m3 -> bf16 widened operands
    u32x4 wax[MXW ? MB : 1][4], wbx[4];          // MXW: the phase's 32 K-values as four bf16 operands
    auto mfma_at = [&](int p, int mi) {
      if constexpr (MXW) {
        // B block j outer; t: the four 8-value parts of the phase's K range
        const int j = mi / (4 * MB), i = (mi % (4 * MB)) / 4, t = mi % 4;
        if (mi == 0) {
#pragma unroll
          for (int x = 0; x < MB; ++x) {
            widen_e4m3_scaled(f.a[x][2 * p], saf[x][p], wax[x][0], wax[x][1]);
            widen_e4m3_scaled(f.a[x][2 * p + 1], saf[x][p], wax[x][2], wax[x][3]);
          }
        }
        if (mi % (4 * MB) == 0) {
          if constexpr (B4) {
            widen_e2m1_scaled(f.b[j][p], sbf[j][p], wbx);
          } else {
            widen_e4m3_scaled(f.b[j][2 * p], sbf[j][p], wbx[0], wbx[1]);
            widen_e4m3_scaled(f.b[j][2 * p + 1], sbf[j][p], wbx[2], wbx[3]);
          }
        }
        mfma_bf16(acc[i][j], wax[i][t], wbx[t]);
      } else if constexpr (MX) {
        const int i = mi / NB, j = mi % NB, q0 = 2 * p;
        const int qb0 = B4 ? p : q0, qb1 = B4 ? p : q0 + 1;
        if (p == 0) mfma_mx<0, B4>(acc[i][j], f.a[i][q0], f.a[i][q0 + 1], f.b[j][qb0], f.b[j][qb1], sa_c[i], sb_c[j]);
        else mfma_mx<2, B4>(acc[i][j], f.a[i][q0], f.a[i][q0 + 1], f.b[j][qb0], f.b[j][qb1], sa_c[i], sb_c[j]);
      } else if constexpr (UC == UC_FP8 && !WIDEN) {
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
    // the fragment registers of phases p0 .. p1-1 (reads completed)
    auto tie_phases = [&](int p0, int p1) {
      constexpr int CPB = NQB / NPH;   // B chunks per phase
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q < p0 * CPP || q >= p1 * CPP) continue;
#pragma unroll
        for (int i = 0; i < MB; ++i) tie(f.a[i][q]);
      }
#pragma unroll
      for (int q = 0; q < NQB; ++q) {
        if (q < p0 * CPB || q >= p1 * CPB) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) tie(f.b[j][q]);
      }
    };

    // One K-stage kb.  Phase 0 runs on fragments read during the previous
    // stage.  In the steady state (a refilling step) a first barrier after
    // M0 of its MFMAs: every wave is then done reading stage kb (those reads
    // were issued during the previous step), so stage kb's slot takes stage
    // kb+S, its copies spread evenly over all the step's later MFMAs (the
    // copy engine sees a steady demand, and each copy has most of a step to
    // land).  After phase 0 a barrier: stage kb+1 has landed for every wave
    // (stage kb+S's first D0 copies may be in flight).  Phases 1.. run with
    // the other copies and the reads of stage kb+1 spread between their
    // MFMAs: a phase's fragment registers are read again as soon as that
    // phase's MFMAs are issued; the last phase's at the end.  Scheduling
    // barriers keep this order.
    constexpr int M0 = MPP >= 8 ? MPP / 4 : 1;              // phase-0 MFMAs before the first barrier
    constexpr int SLOTS = (MPP - M0) + (NPH - 1) * MPP;     // MFMAs the refill spreads over
    constexpr int D0 = dma_after(MPP - M0 - 1, DT, SLOTS);  // copies issued in phase 0
    auto step = [&](int kb, auto refill_tag, auto more_tag, auto vm_tag) {
      constexpr bool REFILL = decltype(refill_tag)::value, MORE = decltype(more_tag)::value;
      constexpr int VM = decltype(vm_tag)::value;   // this wave's loads of later stages in flight
      static_assert(!REFILL || MORE, "a refilling step has a next stage");
      lgkm_wait<P0WAIT>();
      take_scales();
      tie_phases(0, 1);
      __builtin_amdgcn_sched_barrier(0);
      int dm = 0;
      if constexpr (REFILL) {
#pragma unroll
        for (int mi = 0; mi < M0; ++mi) mfma_at(0, mi);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        tie_phases(1, NPH);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = M0; mi < MPP; ++mi) {
          mfma_at(0, mi);
          const int target = dma_after(mi - M0, DT, SLOTS);
#pragma unroll
          for (int x = 0; x < DT; ++x)
            if (x >= dm && x < target) MM_DMA(cur, x, kb + S);
          dm = target;
          __builtin_amdgcn_sched_barrier(0);
        }
        vm_barrier<VM + D0>();
      } else {
#pragma unroll
        for (int mi = 0; mi < MPP; ++mi) mfma_at(0, mi);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MORE) {
          vm_barrier<VM>();
        } else {
          lgkm_wait<0>();
        }
        tie_phases(1, NPH);
      }
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t so = (uint32_t)(((kb + 1) % S) * STAGE);
      if constexpr (MORE) read_scales((uint32_t)(((kb + 1) % S) * SSTAGE));   // ahead of stage kb+1's fragments
#pragma unroll
      for (int p = 1; p < NPH; ++p) {
        int rd = 0;
#pragma unroll
        for (int mi = 0; mi < MPP; ++mi) {
          mfma_at(p, mi);
          if constexpr (REFILL) {
            const int target = dma_after((MPP - M0) + (p - 1) * MPP + mi, DT, SLOTS);
#pragma unroll
            for (int x = 0; x < DT; ++x)
              if (x >= dm && x < target) MM_DMA(cur, x, kb + S);
            dm = target;
          }
          if constexpr (MORE) {
            const int target = ((mi + 1) * RPP + MPP - 1) / MPP;
#pragma unroll
            for (int r = 0; r < RPP; ++r)
              if (r >= rd && r < target) read_one((p - 1) * RPP + r, so);
            rd = target < RPP ? target : RPP;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (MORE) {
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_one((NPH - 1) * RPP + r, so);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // stage 0 landed for every wave: the tile's other min(nk, S) - 1 stages
    // may still be in flight (the previous tile's epilogue stores, issued
    // between stage 0 and them, complete before them)
    const int nkl = cur.nkl;
    static_for<S>([&](auto cc) {
      constexpr int c = S - 1 - decltype(cc)::value;   // S-1, ..., 0
      if (min(nkl, S) - 1 == c) vm_barrier<c * DT>();
    });
    row_second(rr_cur);
    read_stage(0u);
    // Every barrier below has a compile-time DMA count.  At step kb's barrier
    // stage kb+1 must have landed while stages kb+2 .. min(nk-1, kb+S-1) may
    // be in flight; stage kb+S refills while kb + S < nk, and the last S
    // steps drain the ring.
    const std::integral_constant<bool, true> yes;
    const std::integral_constant<bool, false> no;
    for (int kb = 0; kb < nkl - S; ++kb) step(kb, yes, yes, std::integral_constant<int, (S - 2) * DT>{});
    static_for<S - 1>([&](auto jj) {
      constexpr int j = S - decltype(jj)::value;   // S, ..., 2 steps before the end
      if (nkl >= j) step(nkl - j, no, yes, std::integral_constant<int, (j - 2) * DT>{});
    });
    step(nkl - 1, no, no, std::integral_constant<int, 0>{});

    // ------------------------------------------------ next tile, epilogue
    // this tile's row data goes to LDS; every wave is done reading the ring
    row_commit(rr_cur, buf);
    // dynamic tiles with the next tile's first stage ahead of the epilogue:
    // the next item is settled here (after the epilogue at 256 x 256)
    if (BM != 256 && dyn && t == 0) settle_claim(claim_v);
    // (a one-stage tile's wait did not cover the stores of the tile before:
    // with the dependency schedule they are waited for here)
    if (MODE == 0 && a.dep_done != nullptr && cur.nkl < 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // Every wave has waited for this tile's last stage, so the stores of the
    // tile before it, issued earlier, are complete: that tile counts for its
    // M-block now (in-order completion of vector memory operations)
    if (MODE == 0 && a.dep_done != nullptr) {
      if (t == 0 && pend_mb >= 0)
        __hip_atomic_fetch_add(a.dep_done + pend_mb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pend_mb = cur.role != kRoleProduce ? cur.row0 / BM : -1;
    }
    int nitem = item + 1;
    bool nhave = !dyn && nitem < n_items;   // dynamic tiles: known after the row-data barrier, or the epilogue
    TileRef nxt{};
    bool early_dyn = false;   // the next dynamic item's TileRef is made here (not after the epilogue)
    if (BM == 256 && dyn && t == 0)
      claim_v = __hip_atomic_fetch_add(a.claim + cx, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (BM != 256 && dyn) {
      nitem = __builtin_amdgcn_readfirstlane(claim_s[0]);
      const int x = __builtin_amdgcn_readfirstlane(claim_s[1]);
      nhave = x >= 0;
      if (nhave) set_cx(x);
      early_dyn = true;
    }
    RowRegs rr_nxt = row_blank();
    // A K piece of a split tile: a later piece hands its partial sums to
    // piece 0 through its slot and moves on; piece 0 adds them in piece
    // order.  Both finish this exchange before the next item's stages go out
    // (the waits for the exchange would otherwise wait for those too).
    if (CAN_SPLIT && cur.role != kRoleFull) {
      // Slots [slot, slot + sk) as one buffer.  Only rows below the tile's
      // valid count are exchanged: word group v of block (i, j) holds rows
      // rb0 + 32i + 8v .. + 3 of one column; a group past the valid rows gets
      // an offset beyond the descriptor's range, so its store is dropped and
      // its load returns zeros, neither touching memory.  (The epilogue never
      // stores those rows, and their A rows are zero in every piece.)
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.partials + (size_t)cur.slot * (BM * BN)), (short)0, 8 * BM * BN * 4, 0x00020000);
      const uint32_t lane_bytes = (uint32_t)(((wv * MB * NB) * 64 + l) * 16 * 4);   // [wave][block][lane][16] words
      const int rb0 = wm * WTM + 4 * h;
      uint32_t vo[MB][4];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) vo[i][v] = rb0 + i * 32 + 8 * v < cur.valid ? lane_bytes : kOffRange;
      if (cur.role == kRoleProduce) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              __builtin_amdgcn_raw_buffer_store_b128(
                  u32x4{word_of(acc[i][j][4 * v]), word_of(acc[i][j][4 * v + 1]), word_of(acc[i][j][4 * v + 2]),
                        word_of(acc[i][j][4 * v + 3])},
                  prs, vo[i][v], ((i * NB + j) * 64 * 16 + 4 * v) * 4, 0);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the partial sums are in L2
        __syncthreads();
        if (t == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          __hip_atomic_store(&a.split_flags[cur.slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        __shared__ int32_t ready;
        if (t == 0) {
          bool ok = true;
          for (int q = 1; q < sk; ++q) ok = ok && poll_flag(&a.split_flags[cur.slot + q], a.spin_limit);
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          if (!ok && a.err) atomicOr(a.err, (uint32_t)MM_DEVERR_BARRIER_TIMEOUT);
          ready = ok ? 1 : 0;
        }
        __syncthreads();
        if (ready) {
          for (int q = 1; q < sk; ++q) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
              for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
                      prs, vo[i][v], (q * (BM * BN) + (i * NB + j) * 64 * 16 + 4 * v) * 4, 0);
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[i][j][4 * v + e] += from_word<AccE>(w[e]);
                }
          }
        }
        __syncthreads();   // every partial has been read: the flags go back to zero
        if (t == 0)
          for (int q = 1; q < sk; ++q)
            __hip_atomic_store(&a.split_flags[cur.slot + q], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // The next item's first stage goes out now, ahead of this tile's
    // epilogue, where the epilogue keeps its values in registers.  At
    // 256 x 256 the accumulators fill the register file and the epilogue
    // reloads spilled values, and each reload waits for every load in
    // flight: there the next item's stages all go out after the epilogue.
    constexpr bool EARLY_FIRST = BM != 256;
    // Epilogue staging (Linear1 without MX, Linear2): one 32-row block of a
    // wave's outputs at a time, OESZ bytes an element, rows OPITCH bytes
    // apart (padded so that the two lane halves, 4 rows apart, write other
    // banks), in the ring slots the next item's copies leave alone.
    constexpr int OESZ = MODE == 1 ? (UC == UC_BF16 ? 4 : 2) : (UC == UC_BF16 ? 2 : 4);
    constexpr int OCOLS = MODE == 1 ? WTN : WTN / 2;           // output columns of a wave
    constexpr int OPITCH = OCOLS * OESZ + (OESZ == 4 ? 32 : 16);
    constexpr int OREG = 32 * OPITCH;                           // one wave's staging bytes
    constexpr int CPR = OCOLS * OESZ / 16;                      // 16-byte pieces per staged row
    constexpr int CPL = 32 * CPR / 64;                          // pieces per lane
    constexpr bool STAGED = MODE == 0 || MODE == 1;
    static_assert(!STAGED || ((EARLY_FIRST ? STAGE : 0) + NW * OREG <= S * STAGE && 64 % CPR == 0 && CPL >= 1),
                  "epilogue staging fits the free ring slots");
    const uint32_t stg_base = lds_base + (uint32_t)(EARLY_FIRST ? STAGE : 0);
    if (nhave) {
      nxt = make_item(nitem);
      if (EARLY_FIRST) {
        dep_ready(nxt.row0 / BM);
        rr_nxt = start_first(nxt);
      }
    }
    if (cur.role != kRoleProduce) {   // a later piece has no epilogue
      // The lane's coordinates again, from a lane id the compiler cannot
      // trace: nothing the epilogue derives from them is computed ahead of
      // the tile loop and kept live (or spilled) through the mainloop.
      int le = l;
      asm volatile("" : "+v"(le));
      const int h = le / 32, lr = le % 32;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int rb = wm * WTM + i * 32 + 4 * h;   // this lane's rows: rb + 8*(q/4) + q%4
        // row data of the 16 rows, read outside the compiler's view (it would
        // otherwise wait for the next tile's LDS copies first): Linear2 needs
        // the whole entry, A8W8 Linear1 only s^X
        u32x2 ri[MODE == 1 ? 16 : 1];   // Linear2: G[i,k] and s^A of the row
        uint32_t sxr[(MODE == 0 && UC != UC_BF16 && !MX) ? 16 : 1];
        if constexpr (MODE == 1 || (MODE == 0 && UC != UC_BF16 && !MX)) {
          const uint32_t ad = rowinfo_base + (uint32_t)((buf * BM + rb) * (int)sizeof(RowInfo));
          static_for<16>([&](auto qc) {
            constexpr int q = qc, OFF = (8 * (q / 4) + (q % 4)) * (int)sizeof(RowInfo);
            if constexpr (MODE == 1) ri[q] = ds_read8<OFF>(ad);
            else sxr[q] = ds_read4<OFF + 4>(ad);
          });
          lgkm_wait<0>();
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            if constexpr (MODE == 1) tie(ri[q]);
            else tie(sxr[q]);
          }
        }
        if constexpr (MODE == 0 && MX) {
          // SwiGLU into LDS (float32, the MFMA layout: one column per lane),
          // then Q_MX of each row's group of 32 A columns (the wave's 32
          // output columns) from a lane pair: lanes 2r and 2r+1 take row r,
          // 16 columns each; the group's amax is the larger of the two
          // halves' maxima; exponent floor(log2 amax) - 8, codes
          // e4m3(v * 2^-exponent), 16 codes a lane in one store
          static_assert(OCOLS == kMxGroup && OESZ == 4, "one MX group of A columns per wave and row");
          const uint32_t wst = stg_base + (uint32_t)(wv * OREG);
          const uint32_t wlane = wst + (uint32_t)((4 * h) * OPITCH + lr * 4);
          static_for<16>([&](auto qc) {
            constexpr int q = qc, OFF = (8 * (q / 4) + (q % 4)) * OPITCH;
            const float g = __builtin_amdgcn_fmed3f(acc_to_f32(acc[i][0][q]), -a.clamp, a.clamp);
            const float u = __builtin_amdgcn_fmed3f(acc_to_f32(acc[i][1][q]), -a.clamp, a.clamp);
            ds_write4<OFF>(wlane, __float_as_uint(silu(g) * u));
          });
          lgkm_wait<0>();
          const int row = le / 2, half = le % 2;
          u32x4 w[4];
          const uint32_t rd = wst + (uint32_t)(row * OPITCH + half * 64);
          static_for<4>([&](auto kc) {
            constexpr int k = kc;
            w[k] = ds_read16<16 * k>(rd);
          });
          lgkm_wait<0>();
          float m = 0.0f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            tie(w[k]);
#pragma unroll
            for (int c = 0; c < 4; ++c) m = fmaxf(m, fabsf(__uint_as_float(w[k][c])));
          }
          m = fmaxf(m, __shfl_xor(m, 1, 64));
          const int x = mx_shared_exp_e4m3(m);
          const float inv = mx_inv_scale(x);
          u32x4 codes;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            codes[k] = f32x2_to_e4m3x2(__uint_as_float(w[k][0]) * inv, __uint_as_float(w[k][1]) * inv) |
                       (f32x2_to_e4m3x2(__uint_as_float(w[k][2]) * inv, __uint_as_float(w[k][3]) * inv) << 16);
          // the tile's rows as buffers whose ranges end at its last valid
          // row: stores to rows past it are dropped without a branch
          const int gpr = a.I / kMxGroup;   // scale bytes per row
          const int trow = wm * WTM + i * 32 + row;
          const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
              static_cast<uint8_t*>(a.a_out) + (int64_t)cur.row0 * a.I + cur.n0 / 2, (short)0, cur.valid * a.I,
              0x00020000);
          const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
              a.out_mx + (int64_t)cur.row0 * gpr + cur.n0 / 2 / kMxGroup, (short)0, cur.valid * gpr, 0x00020000);
          __builtin_amdgcn_raw_buffer_store_b128(codes, ors, trow * a.I + wn * kMxGroup + half * 16, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(x + 127), srs, half == 0 ? trow * gpr + wn : (int)kOffRange,
                                               0, 0);
        } else if constexpr (MODE == 0 || MODE == 1) {
          // The wave's 32-row block i goes through LDS: each lane writes its
          // 16 rows x NB column values (one column per lane, the MFMA
          // layout), then reads back 16-byte pieces of rows and stores them
          // whole (8 bf16 or 4 float32 a lane and instruction instead of one
          // element).
          const uint32_t wst = stg_base + (uint32_t)(wv * OREG);   // this wave's staging block
          const uint32_t wlane = wst + (uint32_t)((4 * h) * OPITCH + lr * OESZ);
          // output value of accumulator q of column block j (constant q, j)
          auto value = [&](const int q, const int j) -> float {
            float o;
            if constexpr (MODE == 0) {
              // SwiGLU of the gate column (block 2j) and its up partner (2j+1)
              float g = acc_to_f32(acc[i][2 * j][q]);
              float u = acc_to_f32(acc[i][2 * j + 1][q]);
              if constexpr (UC != UC_BF16) {
                const float sx = __uint_as_float(sxr[q]);
                g = (g * rr_cur.cs0[j]) * sx;
                u = (u * rr_cur.cs1[j]) * sx;
              }
              // the operator's activation_clamp (+inf: none; identity on finite H)
              g = __builtin_amdgcn_fmed3f(g, -a.clamp, a.clamp);
              u = __builtin_amdgcn_fmed3f(u, -a.clamp, a.clamp);
              o = silu(g) * u;
            } else {
              // contribution of route i*K+k: ((D * s^W2) * s^A) * G[i,k]
              // (MX: the MFMA applied the block scales; A16W16: D * G)
              const float gw = __uint_as_float(ri[q][0]);
              const float rs = __uint_as_float(ri[q][1]);
              float v = acc_to_f32(acc[i][j][q]);
              if constexpr (COLS) v *= rr_cur.cs0[j];
              o = (UC != UC_BF16 && !MX) ? (v * rs) * gw : v * gw;
            }
            return o;
          };
          // rows q and q + 1 (q even) are adjacent: bf16 pairs share one
          // conversion, the high half stored by ds_write_b16_d16_hi; the
          // offsets are the instructions' immediates
          static_for<8>([&](auto qp) {
            constexpr int q = 2 * qp;
            static_for<OCOLS / 32>([&](auto jc) {
              constexpr int j = jc, OFF = (8 * (q / 4) + (q % 4)) * OPITCH + j * 32 * OESZ;
              static_assert(OFF + OPITCH < 65536, "LDS offsets fit the immediate");
              const float o0 = value(q, j), o1 = value(q + 1, j);
              if constexpr (OESZ == 2) {
                const uint32_t pk = pack_bf16x2(o0, o1);
                ds_write2<OFF>(wlane, pk);
                ds_write2hi<OFF + OPITCH>(wlane, pk);
              } else {
                ds_write4<OFF>(wlane, __float_as_uint(o0));
                ds_write4<OFF + OPITCH>(wlane, __float_as_uint(o1));
              }
            });
          });
          lgkm_wait<0>();
          // read back: lane le takes 16-byte piece ch of staged rows
          // le / CPR + (64 / CPR) * k
          const int ch = le % CPR, r0 = le / CPR;
          u32x4 pv[CPL];
          uint32_t prt[MODE == 1 ? CPL : 1];
          const uint32_t rd = wst + (uint32_t)(r0 * OPITCH + ch * 16);
          const uint32_t rdi = rowinfo_base + (uint32_t)((buf * BM + wm * WTM + i * 32 + r0) * (int)sizeof(RowInfo));
          static_for<CPL>([&](auto kc) {
            constexpr int k = kc;
            pv[k] = ds_read16<(64 / CPR) * k * OPITCH>(rd);
            if constexpr (MODE == 1) prt[k] = ds_read4<8 + (64 / CPR) * k * (int)sizeof(RowInfo)>(rdi);
          });
          lgkm_wait<0>();
#pragma unroll
          for (int k = 0; k < CPL; ++k) {
            tie(pv[k]);
            if constexpr (MODE == 1) tie(prt[k]);
          }
          if constexpr (MODE == 0) {
            // the tile's rows of A as one buffer whose range ends at its last
            // valid row: stores to rows past it are dropped without a branch
            // (offsets stay 32-bit: BLOCK_M * I * 4 < 2^31)
            uint8_t* const obase =
                (UC == UC_BF16 ? static_cast<uint8_t*>(a.a_out) : reinterpret_cast<uint8_t*>(a.a_stage)) +
                ((int64_t)cur.row0 * a.I + cur.n0 / 2) * OESZ;
            const __amdgpu_buffer_rsrc_t ors =
                __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, cur.valid * a.I * OESZ, 0x00020000);
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
              const int row = wm * WTM + i * 32 + r0 + (64 / CPR) * k;
              __builtin_amdgcn_raw_buffer_store_b128(pv[k], ors, (row * a.I + wn * (WTN / 2)) * OESZ + ch * 16, 0, 0);
            }
          } else {
            // each row into its route's combine slot (rows without a route: none)
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
              const int32_t route = (int32_t)prt[k];
              if (route >= 0) {
                uint8_t* const dst = static_cast<uint8_t*>(a.contrib) +
                                     ((uint64_t)(uint32_t)route * (uint32_t)a.H + (uint32_t)(cur.n0 + wn * WTN)) * OESZ +
                                     ch * 16;
                *gp(reinterpret_cast<u32x4*>(dst)) = pv[k];
              }
            }
          }
        } else {
          int32_t* const rbase = a.raw_out + (int64_t)cur.row0 * a.N;
          int lane_row = rb;
          asm volatile("" : "+v"(lane_row));   // keeps the row offsets inside the tile loop
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int n = cur.n0 + wn * WTN + j * 32 + lr;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int r = rb + 8 * (q / 4) + (q % 4);
              int col = n;
              if (a.gate_up_group > 0) {
                const int g2 = 2 * a.gate_up_group;
                const int qq = n / g2, m = n % g2;
                col = (m < a.gate_up_group) ? qq * a.gate_up_group + m : a.I + qq * a.gate_up_group + (m - a.gate_up_group);
              }
              // int32 accumulators as they are, float32 ones as their bit patterns
              if (r < cur.valid) gp(rbase)[(lane_row + 8 * (q / 4) + (q % 4)) * a.N + col] = (int32_t)word_of(acc[i][j][q]);
            }
          }
        }
      }
    }
    // every wave is done reading its staging block before the copies
    // overwrite the slots
    if (BM == 256 && dyn && t == 0) settle_claim(claim_v);
    if constexpr (STAGED) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (dyn) __syncthreads();
    if (dyn && !early_dyn) {
      nitem = __builtin_amdgcn_readfirstlane(claim_s[0]);
      const int x = __builtin_amdgcn_readfirstlane(claim_s[1]);
      nhave = x >= 0;
      if (nhave) {
        set_cx(x);
        nxt = make_item(nitem);
      }
    }
    if (nhave) {
      if (!EARLY_FIRST) {
        dep_ready(nxt.row0 / BM);
        rr_nxt = start_first(nxt);
      }
      start_rest(nxt);
    }
    item = nitem;
    have = nhave;
    cur = nxt;
    rr_cur = rr_nxt;
    buf ^= 1;
  }
#undef MM_DMA
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();   // the block is done with LDS
  if (MODE == 0 && a.dep_done != nullptr && t == 0 && pend_mb >= 0)
    __hip_atomic_fetch_add(a.dep_done + pend_mb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// per-row requantisation of A (A8W8): s^A = max(amax/Qmax, 1e-8), IEEE f32.
// One wave per pool row; rows past their expert's count (padding) carry no
// route and are skipped.  off_s / cnt_s: the dispatch offsets and counts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool requant_row_live(const RequantArgs& a, int64_t p, const int32_t* off_s, const int32_t* cnt_s) {
  if (p >= off_s[a.E] || p >= a.P) return false;
  int lo = 0, hi = a.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off_s[mid] <= p) lo = mid; else hi = mid;
  }
  return p < (int64_t)off_s[lo] + cnt_s[lo];
}

template <int UC>
__device__ __forceinline__ uint2 requant_codes8(const float4& v0, const float4& v1, float s) {
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
  return make_uint2(o[0], o[1]);
}

__device__ __forceinline__ float amax4(const float4& v, float m) {
  return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Rows p0, p0 + pstride, ... (U of them) by one wave.  Rows of up to RC
// float8 chunks per lane (I <= 64*8*RC) stay in registers between the amax
// (exact: a max) and the codes, with the loads of all U rows in flight at
// once; longer rows are read twice, one at a time.
template <int UC, int U, int RC = 8>
__device__ __forceinline__ void requant_rows(const RequantArgs& a, int64_t p0, int64_t pstride, const int32_t* off_s,
                                             const int32_t* cnt_s) {
  constexpr int kRequantRegChunks = RC;
  const int l = lane_id();
  const int nch = a.I / 8;
  const float qmax = (UC == UC_I8) ? 127.0f : 448.0f;
  bool live[U];
#pragma unroll
  for (int u = 0; u < U; ++u) live[u] = requant_row_live(a, p0 + u * pstride, off_s, cnt_s);
  if (nch <= 64 * kRequantRegChunks) {
    // registers cleared first, then loads that only fill them: no branch
    // writes a register a load in flight targets, so every load of the U
    // rows is issued before the first wait
    float4 keep[U][2 * kRequantRegChunks];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2 * kRequantRegChunks; ++j) keep[u][j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float4* src = reinterpret_cast<const float4*>(a.a_stage + (p0 + u * pstride) * a.I);
#pragma unroll
      for (int j = 0; j < kRequantRegChunks; ++j) {
        const int c = j * 64 + l;
        if (live[u] && c < nch) {
          keep[u][2 * j] = src[2 * c];
          keep[u][2 * j + 1] = src[2 * c + 1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live[u]) continue;
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 2 * kRequantRegChunks; ++j) m = amax4(keep[u][j], m);
      const float s = fmaxf(wave_max(m) / qmax, 1e-8f);
      const int64_t p = p0 + u * pstride;
      uint2* dst = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.a_pool) + p * a.I);
#pragma unroll
      for (int j = 0; j < kRequantRegChunks; ++j) {
        const int c = j * 64 + l;
        if (c < nch) dst[c] = requant_codes8<UC>(keep[u][2 * j], keep[u][2 * j + 1], s);
      }
      if (l == 0) a.a_scale[p] = s;
    }
  } else {
    for (int u = 0; u < U; ++u) {
      if (!live[u]) continue;
      const int64_t p = p0 + u * pstride;
      const float4* src = reinterpret_cast<const float4*>(a.a_stage + p * a.I);
      float m = 0.0f;
      for (int c = l; c < a.I / 4; c += 64) m = amax4(src[c], m);
      const float s = fmaxf(wave_max(m) / qmax, 1e-8f);
      uint2* dst = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.a_pool) + p * a.I);
      for (int c = l; c < nch; c += 64) dst[c] = requant_codes8<UC>(src[2 * c], src[2 * c + 1], s);
      if (l == 0) a.a_scale[p] = s;
    }
  }
}

// The fused kernel's requantisation with four waves per CU (one per SIMD):
// rows p0 + k * pstride below `used`, RU at a time, the next RU rows' loads
// issued before this batch's maxima, codes and stores, so that a wave alone
// on its SIMD keeps loads in flight while it computes.  Each load and store
// is a buffer access whose descriptor covers its row only when the row is
// live (padding rows and rows past `used`: no memory access, loads read 0),
// so every batch issues the same instructions and the waits between them
// have fixed counts.  The same arithmetic as requant_rows (bit for bit).
// I <= 2048: four chunks of 8 values per lane.
template <int UC, int RU>
__device__ __forceinline__ void requant_stream(const RequantArgs& a, int64_t p0, int64_t pstride, int64_t used,
                                               const int32_t* off_s, const int32_t* cnt_s) {
  constexpr int RC = 4;
  if (p0 >= used) return;
  const int l = lane_id();
  const int nch = a.I / 8;
  const float qmax = (UC == UC_I8) ? 127.0f : 448.0f;
  float4 buf[2][RU][2 * RC];
  bool live[2][RU];
  // (the row is the wave's: its base and range go to scalar registers, or
  // the compiler would loop over the lanes for each access)
  auto row_rsrc = [&](const void* base, int64_t p, int64_t elem_bytes, bool on) {
    const uint8_t* b = static_cast<const uint8_t*>(base) + (on ? p : 0) * elem_bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(b), (short)0,
                                             uniform_int(on ? (int)elem_bytes : 0), 0x00020000);
  };
  auto load = [&](auto bt, int64_t p) {
    constexpr int b = decltype(bt)::value;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int64_t pu = p + u * pstride;
      live[b][u] = requant_row_live(a, pu, off_s, cnt_s);
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.a_stage, pu, (int64_t)a.I * 4, live[b][u]);
#pragma unroll
      for (int j = 0; j < RC; ++j) {
        const int c = j * 64 + l;
        const int off = c < nch ? c * 32 : (int)kOffRange;
        buf[b][u][2 * j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        buf[b][u][2 * j + 1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
      }
    }
  };
  auto process = [&](auto bt, int64_t p) {
    constexpr int b = decltype(bt)::value;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 2 * RC; ++j) m = amax4(buf[b][u][j], m);
      const float sc = fmaxf(wave_max(m) / qmax, 1e-8f);
      const int64_t pu = p + u * pstride;
      const __amdgpu_buffer_rsrc_t ro = row_rsrc(a.a_pool, pu, a.I, live[b][u]);
#pragma unroll
      for (int j = 0; j < RC; ++j) {
        const int c = j * 64 + l;
        const uint2 q = requant_codes8<UC>(buf[b][u][2 * j], buf[b][u][2 * j + 1], sc);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{q.x, q.y}, ro, c < nch ? c * 8 : (int)kOffRange, 0, 0);
      }
      const __amdgpu_buffer_rsrc_t rsc = row_rsrc(a.a_scale, pu, 4, live[b][u]);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rsc, l == 0 ? 0 : (int)kOffRange, 0, 0);
    }
  };
  const std::integral_constant<int, 0> b0;
  const std::integral_constant<int, 1> b1;
  const int64_t step = (int64_t)RU * pstride;
  int64_t p = p0;
  load(b0, p);
  for (;;) {
    load(b1, p + step);   // the next batch (past `used`: nothing is read)
    process(b0, p);
    p += step;
    if (p >= used) break;
    load(b0, p + step);
    process(b1, p);
    p += step;
    if (p >= used) break;
  }
}

// The fused kernel's requantisation under its dependency schedule: the rows
// of this workgroup's XCD slice (the M-blocks its Linear1 and Linear2 tiles
// cover, as gemm_tiles cuts them), wave wx of the slice's WX waves taking
// rows wx, wx + WX, ..., two at a time with the next two rows' loads in
// flight (as requant_stream, the same arithmetic).  A row is loaded once all
// Linear1 tiles of its M-block are counted (dep_l1[b] >= l1_target); every
// row of the slice (padding rows too) counts once in dep_rq[b] when its
// stores are complete: two batches later, when the loads of a batch issued
// after them have landed (in-order completion), or at the end.  I <= 2048.
template <int UC, int BM, int NW>
__device__ __forceinline__ void requant_dep(const RequantArgs& a, const int32_t* off_s, const int32_t* cnt_s,
                                            const uint32_t* dep_l1, uint32_t l1_target, uint32_t* dep_rq,
                                            uint32_t spin_limit, uint32_t* err) {
  constexpr int RC = 4, RU = 2;
  constexpr int nxcd = 8;
  const int xcd = blockIdx.x % nxcd, per_x = gridDim.x / nxcd;
  if ((int)blockIdx.x >= per_x * nxcd) return;
  const int n_mb = off_s[a.E] / BM;
  const int mb_slice = (n_mb + nxcd - 1) / nxcd;
  const int mb_beg = min(n_mb, xcd * mb_slice), mb_end = min(n_mb, mb_beg + mb_slice);
  const int64_t WX = (int64_t)per_x * NW, step = RU * WX;
  const int64_t wx = (int64_t)(blockIdx.x / nxcd) * NW + __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int64_t r_beg = (int64_t)mb_beg * BM + wx, r_end = (int64_t)mb_end * BM;
  const int64_t nbat = r_end > r_beg ? (r_end - r_beg + step - 1) / step : 0;
  if (nbat == 0) return;
  const int l = lane_id();
  const int nch = a.I / 8;
  const float qmax = (UC == UC_I8) ? 127.0f : 448.0f;
  float4 buf[2][RU][2 * RC];
  bool live[2][RU];
  int dw_base = 0;
  uint64_t dw_mask = 0;
  auto l1_ready = [&](int mb) {
    if (dw_base == 0x40000000) return;
    if (mb >= dw_base && mb < dw_base + 64 && ((dw_mask >> (mb - dw_base)) & 1u)) return;
    if (mb < dw_base || mb >= dw_base + 64) dw_base = mb;
    uint32_t polls = 0;
    for (;;) {
      const int q = dw_base + l;
      const uint32_t v = q < n_mb ? __hip_atomic_load(dep_l1 + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      dw_mask = __ballot(v >= l1_target);
      if ((dw_mask >> (mb - dw_base)) & 1u) break;
      if (++polls > spin_limit) {   // gives up: flagged, and no later wait of this wave polls
        if (l == 0 && err) atomicOr(err, (uint32_t)MM_DEVERR_BARRIER_TIMEOUT);
        dw_base = 0x40000000;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    asm volatile("" ::: "memory");
  };
  auto row_rsrc = [&](const void* base, int64_t p, int64_t elem_bytes, bool on) {
    const uint8_t* b = static_cast<const uint8_t*>(base) + (on ? p : 0) * elem_bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(b), (short)0,
                                             uniform_int(on ? (int)elem_bytes : 0), 0x00020000);
  };
  auto load = [&](auto bt, int64_t j) {
    constexpr int b = decltype(bt)::value;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int64_t pu = r_beg + j * step + u * WX;
      const bool in = pu < r_end;
      if (in) l1_ready((int)(pu / BM));
      live[b][u] = in && requant_row_live(a, pu, off_s, cnt_s);
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.a_stage, pu, (int64_t)a.I * 4, live[b][u]);
#pragma unroll
      for (int c8 = 0; c8 < RC; ++c8) {
        const int c = c8 * 64 + l;
        const int off = c < nch ? c * 32 : (int)kOffRange;
        buf[b][u][2 * c8] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        buf[b][u][2 * c8 + 1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
      }
    }
  };
  auto process = [&](auto bt, int64_t j) {
    constexpr int b = decltype(bt)::value;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      float m = 0.0f;
#pragma unroll
      for (int c8 = 0; c8 < 2 * RC; ++c8) m = amax4(buf[b][u][c8], m);
      const float sc = fmaxf(wave_max(m) / qmax, 1e-8f);
      const int64_t pu = r_beg + j * step + u * WX;
      const __amdgpu_buffer_rsrc_t ro = row_rsrc(a.a_pool, pu, a.I, live[b][u]);
#pragma unroll
      for (int c8 = 0; c8 < RC; ++c8) {
        const int c = c8 * 64 + l;
        const uint2 q = requant_codes8<UC>(buf[b][u][2 * c8], buf[b][u][2 * c8 + 1], sc);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{q.x, q.y}, ro, c < nch ? c * 8 : (int)kOffRange, 0, 0);
      }
      const __amdgpu_buffer_rsrc_t rsc = row_rsrc(a.a_scale, pu, 4, live[b][u]);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rsc, l == 0 ? 0 : (int)kOffRange, 0, 0);
    }
  };
  auto publish = [&](int64_t j) {
    asm volatile("" ::: "memory");
    if (j < 0 || j >= nbat || l != 0) return;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int64_t pu = r_beg + j * step + u * WX;
      if (pu < r_end) __hip_atomic_fetch_add(dep_rq + pu / BM, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  const std::integral_constant<int, 0> b0;
  const std::integral_constant<int, 1> b1;
  load(b0, 0);
  for (int64_t j = 0;;) {
    load(b1, j + 1);   // the next batch (past the slice: nothing is read)
    process(b0, j);
    publish(j - 2);
    if (++j >= nbat) break;
    load(b0, j + 1);
    process(b1, j);
    publish(j - 2);
    if (++j >= nbat) break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  publish(nbat - 2);
  publish(nbat - 1);
}

// ---------------------------------------------------------------------------
// Token Combine: y_i = sum_{k=0..K-1} slot[i*K+k] in slot order, float32;
// masked routes (route_to_pool < 0) contribute nothing.  One thread makes 8
// consecutive columns c .. c+7 of token i.  Slots are float32, or bf16 for
// the A8W8 use cases.

// U work items idx0, idx0 + stride, ... at once (item = token idx / (H/8),
// columns 8 * (idx % (H/8)) .. +7).  For each group of up to 8 routes of a
// token the route indices are loaded together and then all the slot rows
// together, so a thread keeps 8U slot loads in flight; the additions still
// run in slot order and a masked route adds nothing.  BF16: the slots are
// bf16 (the A8W8 use cases), else float32.
template <int U, bool BF16>
__device__ __forceinline__ void combine_items(const CombineArgs& a, int64_t idx0, int64_t stride, int64_t work) {
  constexpr int KC = 8;
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
  // The route-index loads are unconditional (a clamped, in-bounds index)
  // and a slot load only fills a register cleared beforehand, so no branch
  // of the unrolled loops writes a register a load in flight still targets
  // (which would make the compiler wait for every load in turn).
  for (int k0 = 0; k0 < a.K; k0 += KC) {
    bool on[U][KC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tu = tok[u] >= 0 ? tok[u] : 0;
      int32_t pi[KC];
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) pi[kk] = a.route_to_pool[tu * a.K + min(k0 + kk, a.K - 1)];
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) on[u][kk] = tok[u] >= 0 && k0 + kk < a.K && pi[kk] >= 0;
    }
    if constexpr (BF16) {
      uint4 w[U][KC];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          w[u][kk] = make_uint4(0u, 0u, 0u, 0u);
          if (on[u][kk])
            w[u][kk] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.contrib) +
                                                       (tok[u] * a.K + k0 + kk) * a.H + col[u]);
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          if (!on[u][kk]) continue;
          const uint32_t ww[4] = {w[u][kk].x, w[u][kk].y, w[u][kk].z, w[u][kk].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[u][2 * q] += bf16_bits_to_f32(ww[q] & 0xffffu);
            acc[u][2 * q + 1] += bf16_bits_to_f32(ww[q] >> 16);
          }
        }
    } else {
      float4 v[U][KC][2];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          v[u][kk][0] = v[u][kk][1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (on[u][kk]) {
            const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.contrib) +
                                                                (tok[u] * a.K + k0 + kk) * a.H + col[u]);
            v[u][kk][0] = src[0];
            v[u][kk][1] = src[1];
          }
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          if (!on[u][kk]) continue;
          const float4 v0 = v[u][kk][0], v1 = v[u][kk][1];
          acc[u][0] += v0.x; acc[u][1] += v0.y; acc[u][2] += v0.z; acc[u][3] += v0.w;
          acc[u][4] += v1.x; acc[u][5] += v1.y; acc[u][6] += v1.z; acc[u][7] += v1.w;
        }
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

// Token Combine of the fused kernel through LDS: the slot rows arrive by
// LDS-DMA (no registers hold loads in flight, so a workgroup of few waves
// still keeps three units of 8 slot-row segments in flight), then each thread
// sums its columns in slot order exactly as combine_items does (masked
// routes add nothing) and stores them.  A unit is one token's columns
// [seg * NT * CPT, +NT * CPT) of its K <= 8 slots (slots past K and columns
// past H are loaded beyond the descriptors' ranges: zeros, no memory
// access), plus the token's route_to_pool entries, which every wave loads
// into its own corner.  Thread t reads only the bytes its own wave loaded, so
// the waves need no barrier; the waits are fixed vmcnt counts (every unit
// issues the same copies and stores per wave, out-of-range ones included).
template <int NT, bool BF16>
struct CombineLds {
  static constexpr int NW = NT / 64, CPT = BF16 ? 8 : 4, ESZ = BF16 ? 2 : 4;
  static constexpr int KMAX = 8;
  static constexpr int SLOT_BYTES = NT * 16;                   // one slot row segment
  static constexpr int UNIT = KMAX * SLOT_BYTES + NW * 256;   // + the waves' route_to_pool corners
  static constexpr int NBUF = NT <= 256 ? 3 : 2;
  static constexpr int BYTES = NBUF * UNIT;
  static constexpr int DT = KMAX + 1;                          // DMA instructions per wave and unit
  static constexpr int YS = BF16 ? 2 : 1;                      // y stores per wave and unit
};

template <int NT, bool BF16>
__device__ __forceinline__ void combine_lds(const CombineArgs& a, uint8_t* lds) {
  typedef CombineLds<NT, BF16> C;
  constexpr int NW = C::NW, CPT = C::CPT, ESZ = C::ESZ, NBUF = C::NBUF, DT = C::DT, YS = C::YS;
  const int t = threadIdx.x, l = t % 64;
  const int wv = __builtin_amdgcn_readfirstlane(t / 64);
  const int K = a.K, H = a.H;
  const int SEG = NT * CPT;
  const int nseg = (H + SEG - 1) / SEG;
  const int64_t units = a.T * nseg, G = gridDim.x;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  const int ysz = a.y_f32 ? 4 : 2;
  // unit j's copies into buffer b (past the last unit: every copy beyond range)
  auto issue = [&](int64_t j, int b) {
    const bool on = j < units;
    const int64_t i = on ? j / nseg : 0;
    const int seg = on ? (int)(j % nseg) : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(static_cast<const uint8_t*>(a.contrib) + i * K * (int64_t)H * ESZ), (short)0,
        on ? K * H * ESZ : 0, 0x00020000);
    const int col = seg * SEG + (wv * 64 + l) * CPT;
    uint8_t* const ub = lds + b * C::UNIT;
#pragma unroll
    for (int k = 0; k < C::KMAX; ++k) {
      const int off = (k < K && col < H) ? (k * H + col) * ESZ : (int)kOffRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(ub + k * C::SLOT_BYTES + wv * 1024), 16, off, 0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(reinterpret_cast<const uint8_t*>(a.route_to_pool) + i * K * 4), (short)0, on ? K * 4 : 0,
        0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t)(ub + C::KMAX * C::SLOT_BYTES + wv * 256), 4, l * 4, 0, 0,
                                             0);
  };
  // sum and store unit j from buffer b; VM: this wave's later copies and
  // stores still allowed in flight when unit j's copies have landed
  auto finish = [&](int64_t j, int b, auto vm_tag) {
    constexpr int VM = decltype(vm_tag)::value;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VM) : "memory");
    const int64_t i = j / nseg;
    const int seg = (int)(j % nseg);
    const uint32_t ub = lds_base + (uint32_t)(b * C::UNIT);
    uint32_t pi[C::KMAX];
    u32x4 v[C::KMAX];
#pragma unroll
    for (int k = 0; k < C::KMAX; ++k) pi[k] = ds_read4<0>(ub + (uint32_t)(C::KMAX * C::SLOT_BYTES + wv * 256 + k * 4));
#pragma unroll
    for (int k = 0; k < C::KMAX; ++k) v[k] = ds_read16<0>(ub + (uint32_t)(k * C::SLOT_BYTES + t * 16));
    lgkm_wait<0>();
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int k = 0; k < C::KMAX; ++k) {
      tie(pi[k]);
      tie(v[k]);
      if (k < K && (int32_t)pi[k] >= 0) {
        if constexpr (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += bf16_bits_to_f32(v[k][q] & 0xffffu);
            acc[2 * q + 1] += bf16_bits_to_f32(v[k][q] >> 16);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(v[k][q]);
        }
      }
    }
    const int col = seg * SEG + t * CPT;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(static_cast<uint8_t*>(a.y) + i * (int64_t)H * ysz), (short)0, H * ysz, 0x00020000);
    const int yo = col < H ? col * ysz : (int)kOffRange;
    if constexpr (BF16) {
      if (a.y_f32) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])},
            ry, yo, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]), __float_as_uint(acc[7])},
            ry, yo == (int)kOffRange ? yo : yo + 16, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])},
                                               ry, yo, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, ry, (int)kOffRange, 0, 0);   // keeps YS fixed
      }
    } else {
      if (a.y_f32)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])},
            ry, yo, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])}, ry, yo,
                                              0, 0);
    }
  };
  const int64_t j0 = blockIdx.x;
  if (j0 >= units) return;
  // copies of the first NBUF - 1 units, then per unit: the copies of the
  // unit NBUF - 1 ahead, then the wait for this unit's (the first units see
  // fewer later stores, so their counts are their own).  Copies past the
  // last unit still write zeros into LDS: every exit waits for them.
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b) issue(j0 + b * G, b);
  int64_t j = j0;
  issue(j + (NBUF - 1) * G, NBUF - 1);
  finish(j, 0, std::integral_constant<int, (NBUF - 1) * DT>{});
  j += G;
  if (j < units) {
    issue(j + (NBUF - 1) * G, 0);
    finish(j, 1, std::integral_constant<int, (NBUF - 1) * DT + YS>{});
    j += G;
    int b = 2 % NBUF;
    for (; j < units; j += G) {
      issue(j + (NBUF - 1) * G, (b + NBUF - 1) % NBUF);
      finish(j, b, std::integral_constant<int, (NBUF - 1) * (DT + YS)>{});
      b = (b + 1) % NBUF;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace mm
