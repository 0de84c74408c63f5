// The fused persistent kernel of mega_moe: every step of the routed-expert
// path in one launch.  One workgroup per compute unit, the whole grid
// resident at once; the phases run in order, separated by grid-wide
// barriers:
//   count + claim | prefix + scatter | gather | Linear1 + SwiGLU |
//   (A8W8) requantisation | Linear2 + gate | combine
// When Linear1 reads the token rows in place there is no gather phase and
// the A8W8 token quantisation runs beside the count; a small batch is
// dispatched whole by one block in the first phase (no prefix + scatter
// phase).  Each phase computes
// exactly what the three-call path's kernels compute, so the results are
// bitwise those of that path.  The counters it relies on (expert counts, A8W8 row
// amax, barrier arrivals, error word) are cleared by a small pre-pass.
#include "mm_dispatch_dev.hpp"
#include "mm_gemm_dev.hpp"

namespace mm {

// Grid-wide barrier, hierarchical over the XCDs.  Control words (cleared by
// the pre-pass): ctl[0] XCDs released, ctl[1] error word, ctl[2] workgroups
// registered, ctl[16 + x] arrivals on XCD x, ctl[32 + x] workgroups on XCD x.
//
// Every workgroup registers its XCD at kernel start.  At barrier n each wave
// waits for its own stores to complete (be in L2), then the workgroup
// barrier (which alone does not wait for them); thread 0 adds one arrival
// for its XCD, and the last workgroup of an XCD to arrive writes that XCD's
// L2 back (one device-scope release per XCD, not one per workgroup) and
// releases the XCD; every workgroup then waits for all active XCDs and
// acquires.  Polls
// are relaxed device-scope loads with a sleep between them.  After spin_limit
// polls a wait gives up: it sets MM_DEVERR_BARRIER_TIMEOUT and the block
// leaves the kernel, so no phase runs on data another block may not have
// finished; blocks waiting for it time out at their next barrier.
struct BarState {
  uint32_t xcd, wg_in_xcd, active_xcds;
};

__device__ __forceinline__ uint32_t xcc_id() {
  // hardware register XCC_ID (20), bits 3:0: the XCD this wave runs on
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u;
}

__device__ __forceinline__ bool poll_until(uint32_t* p, uint32_t target, uint32_t spin_limit) {
  uint32_t polls = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (++polls > spin_limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

__device__ __forceinline__ void barrier_register(uint32_t* ctl, BarState& bs) {
  bs = BarState{xcc_id(), 0u, 0u};
  if (threadIdx.x == 0) {
    // ctl[3] != 0: some workgroup does not run on XCD blockIdx % 8, so the
    // GEMMs' per-XCD slices do not share an L2 and the dependency schedule
    // is off (grid barriers between the phases instead)
    if (gridDim.x % 8 != 0 || blockIdx.x % 8 != bs.xcd) {
      __hip_atomic_fetch_or(&ctl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
    __hip_atomic_fetch_add(&ctl[32 + bs.xcd], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&ctl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ bool grid_barrier(uint32_t* ctl, uint32_t n, uint32_t spin_limit, BarState& bs, int32_t* ok_lds) {
  // s_waitcnt vmcnt(0): the write-back below covers only stores already in
  // L2, and a wave's stores may still be in flight at the workgroup barrier
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (threadIdx.x == 0) {
    bool ok = true;
    if (bs.wg_in_xcd == 0) {   // first barrier: wait for every registration, then read them
      ok = poll_until(&ctl[2], gridDim.x, spin_limit);
      bs.wg_in_xcd = __hip_atomic_load(&ctl[32 + bs.xcd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int x = 0; x < 16; ++x)
        bs.active_xcds += __hip_atomic_load(&ctl[32 + x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > 0 ? 1u : 0u;
    }
    if (ok) {
      const uint32_t before = __hip_atomic_fetch_add(&ctl[16 + bs.xcd], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (before + 1 == n * bs.wg_in_xcd) {   // last of its XCD
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      ok = poll_until(&ctl[0], n * bs.active_xcds, spin_limit);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (!ok) __hip_atomic_fetch_or(&ctl[1], (uint32_t)MM_DEVERR_BARRIER_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *ok_lds = ok ? 1 : 0;
  }
  __syncthreads();
  return *ok_lds != 0;
}

template <int UC, int BM>
constexpr int mega_lds_bytes() {
  return lds_bytes_of<UC, BM>();
}

template <int UC, int BM, bool WIDEN>
__global__ __launch_bounds__(threads_of<BM>()) __attribute__((amdgpu_waves_per_eu(threads_of<BM>() / 256, threads_of<BM>() / 256)))
void k_mega(const MegaArgs* mp) {
  // The arguments sit in device memory (written by the pre-pass) rather than
  // in the kernel-argument segment, so each phase loads the fields it uses
  // where it uses them instead of holding all of them in scalar registers
  // for the whole kernel.
  const MegaArgs& m = *mp;
  constexpr int NT = threads_of<BM>(), NW = NT / 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int MAXE = max_experts<UC>();
  __shared__ int32_t off_s[MAXE + 1];
  __shared__ int32_t cnt_s[MAXE];
  __shared__ int32_t wsum[NW];
  __shared__ int32_t dst[64];
  __shared__ float red[NW];
  __shared__ int32_t ok;
  static_assert((MAXE + 1 + (int64_t)NW * MAXE) * 4 <= mega_lds_bytes<UC, BM>(), "dispatch scratch fits");
  int32_t* smem = reinterpret_cast<int32_t*>(lds);
  const int t = threadIdx.x;
  uint32_t* const ctl = m.ctl;
  const uint32_t spin = m.spin_limit;
  const int64_t nwaves = m.nwaves;
  // clock sample of this run: shader-clock counter and the constant 100 MHz
  // counter, read by workgroup 0 when it starts and when it is done
  if (blockIdx.x == 0 && t == 0) {
    uint64_t* clk = reinterpret_cast<uint64_t*>(ctl + kClockWord0);
    clk[0] = __builtin_amdgcn_s_memtime();
    clk[2] = __builtin_amdgcn_s_memrealtime();
  }
  BarState bs;
  barrier_register(ctl, bs);
  uint32_t nb = 0;
  const int64_t nvb = (nwaves + NW - 1) / NW;   // virtual dispatch blocks of NW waves

  // count + claim (each phase copies the arguments it needs into registers).
  // When Linear1 reads the token rows in place, A8W8 quantises each token
  // once (one wave per token) into a [T][H] buffer: that needs no routing,
  // so it runs here too, beside the count.  A small batch (at most
  // kOneBlockRoutes routes per thread of a block) is dispatched whole by
  // block 0 here, which saves the prefix + scatter phase and its barrier.
  constexpr int kOneBlockRoutes = 16;
  const bool one_block = m.d.T * m.d.K <= (int64_t)kOneBlockRoutes * NT;
  {
    const DispatchArgs d = m.d;
    if (one_block) {
      if (blockIdx.x == 0) dispatch_one_block<NT, kOneBlockRoutes>(d, smem, off_s, wsum);
    } else {
      for (int64_t vb = blockIdx.x; vb < nvb; vb += gridDim.x) count_block<NW>(d, vb, nwaves, smem);
    }
  }
  if constexpr (UC != UC_BF16) {
    if (m.l1_by_token) {
      DispatchArgs d = m.d;
      d.x_pool = m.x_tok;
      if constexpr (is_mx(UC)) d.x_pool_mx = static_cast<uint8_t*>(m.x_tok_scale);
      else d.x_pool_scale = static_cast<float*>(m.x_tok_scale);
      // token i to wave i / G of block i % G: a short batch spreads over all CUs
      const int64_t nwv = (int64_t)gridDim.x * NW;
      for (int64_t tok = (int64_t)(t / 64) * gridDim.x + blockIdx.x; tok < d.T; tok += nwv) quant_token_wave<UC>(d, tok);
    }
  }
  if (!grid_barrier(ctl, ++nb, spin, bs, &ok)) return;
  // Dependency schedule (every workgroup reads the same word, so all take
  // the same barriers): with each workgroup on XCD blockIdx % 8, the tiles
  // of an M-block, its requantisation and its Linear2 tiles all run on one
  // XCD, which shares one L2.  Linear1 counts finished tiles per M-block,
  // the requantisation waits for them and counts rows, Linear2 waits for
  // those: no grid barrier between Linear1, the requantisation and Linear2.
  // Completion is published once the stores are complete (in L2); consumers
  // poll with device-scope loads and read the data through L2 (this kernel
  // has not read those lines before, so no stale copies sit in L1).
  constexpr bool kA8W8 = UC == UC_FP8 || UC == UC_I8;
  const bool dep = !m.no_dep && gridDim.x >= 8 && (!kA8W8 || m.rq.I <= 2048) &&
                   __hip_atomic_load(&ctl[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
  // the counts are final: the routed experts' ones go to the caller
  if (blockIdx.x == 0)
    for (int e = t; e < m.d.Er; e += NT) m.counts_out[e] = m.d.counts[e];

  // padded prefix (every block, into LDS) + scatter
  if (!one_block) {
    const DispatchArgs d = m.d;
    padded_prefix<NT>(d, d.counts, off_s, wsum);
    if (blockIdx.x == 0)
      for (int e = t; e <= d.E; e += NT) d.offsets[e] = off_s[e];
    for (int64_t vb = blockIdx.x; vb < nvb; vb += gridDim.x) scatter_block<NW>(d, vb, nvb, nwaves, off_s, smem);
    if (!grid_barrier(ctl, ++nb, spin, bs, &ok)) return;
  }

  // gather (+ A8W8 activation quantisation) of the pool rows, one token per
  // block at a time, unless Linear1 reads the token rows in place
  if (!m.l1_by_token) {
    const DispatchArgs d = m.d;
    for (int64_t tok = blockIdx.x; tok < d.T; tok += gridDim.x) gather_token<UC, NT>(d, tok, dst, red);
    if (!grid_barrier(ctl, ++nb, spin, bs, &ok)) return;
  }

  // Linear1 + SwiGLU (gemm_tiles leaves the offsets and counts in off_s / cnt_s)
  constexpr int BN = TileShape<BM>::BN;
  {
    GemmArgs g = m.l1;
    if (dep) g.dep_done = m.dep;
    if (!m.static_tiles) g.claim = m.dep + 2 * m.dep_blocks;
    g.steal = !dep && m.static_tiles == 0;   // the dependency schedule needs every tile on its own XCD
    gemm_tiles<UC, BM, 0, WIDEN>(g, lds, off_s, cnt_s);
  }
  if (!dep && !grid_barrier(ctl, ++nb, spin, bs, &ok)) return;

  if constexpr (kA8W8) {
    if (dep) {
      requant_dep<UC, BM, NW>(m.rq, off_s, cnt_s, m.dep, (uint32_t)(m.l1.N / BN), m.dep + m.dep_blocks, spin,
                              m.l1.err);
      __syncthreads();   // (gemm_tiles rewrites off_s / cnt_s, with the same values)
    } else {
      // per-row requantisation of A, one wave per pool row (two rows at a
      // time when I <= 2048; with four waves per CU, two rows while the next
      // two load); MX quantised A in the Linear1 epilogue
      const RequantArgs r = m.rq;
      const int64_t used = off_s[r.E], nwv = (int64_t)gridDim.x * NW;
      const int64_t p0 = (int64_t)blockIdx.x * NW + t / 64;
      if (r.I <= 2048) {
        if constexpr (NW >= 8) {
          for (int64_t p = p0; p < used; p += 2 * nwv) requant_rows<UC, 2, 4>(r, p, nwv, off_s, cnt_s);
        } else {
          requant_stream<UC, 2>(r, p0, nwv, used, off_s, cnt_s);   // one wave per SIMD: loads ahead of the math
        }
      } else {
        for (int64_t p = p0; p < used; p += nwv) requant_rows<UC, 1>(r, p, 0, off_s, cnt_s);
      }
      if (!grid_barrier(ctl, ++nb, spin, bs, &ok)) return;
    }
  }

  // Linear2 + gate weight into the combine slots
  {
    GemmArgs g = m.l2;
    if (!m.static_tiles) g.claim = m.dep + 2 * m.dep_blocks + 8;
    g.steal = !dep && m.static_tiles == 0;
    if (dep) {
      g.dep_wait = kA8W8 ? m.dep + m.dep_blocks : m.dep;
      g.dep_target = kA8W8 ? (uint32_t)BM : (uint32_t)(m.l1.N / BN);
    }
    gemm_tiles<UC, BM, 1, false>(g, lds, off_s, cnt_s);
  }
  if (!grid_barrier(ctl, ++nb, spin, bs, &ok)) return;

  // combine: up to 8 slots a token through LDS (the ring is free now);
  // otherwise 8 columns of one token per item, two items per thread at a
  // time with bf16 slots (A8W8), one with float32 slots, twice that with
  // four waves per CU (the same loads in flight per CU)
  const CombineArgs c = m.cb;
  static_assert(CombineLds<NT, UC != UC_BF16>::BYTES <= mega_lds_bytes<UC, BM>(), "combine buffers fit the ring");
  if (c.K <= CombineLds<NT, UC != UC_BF16>::KMAX) {
    combine_lds<NT, UC != UC_BF16>(c, lds);
  } else {
    const int64_t work = c.T * (c.H / 8), stride = (int64_t)gridDim.x * NT;
    constexpr int CU = (UC == UC_BF16 ? 1 : 2) * (NW >= 8 ? 1 : 2);
    for (int64_t idx = (int64_t)blockIdx.x * NT + t; idx < work; idx += CU * stride)
      combine_items<CU, UC != UC_BF16>(c, idx, stride, work);
  }
  __syncthreads();
  if (blockIdx.x == 0 && t == 0) {
    uint64_t* clk = reinterpret_cast<uint64_t*>(ctl + kClockWord0);
    clk[1] = __builtin_amdgcn_s_memtime();
    clk[3] = __builtin_amdgcn_s_memrealtime();
  }
}

// Pre-pass: clears the counters the fused kernel accumulates into (expert
// counts, control words) and stores the kernel's arguments in the workspace.
__global__ __launch_bounds__(256) void k_mega_prep(MegaArgs m, MegaArgs* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < m.d.E; j += stride) m.d.counts[j] = 0;
  for (int64_t j = i; j < kCtlWords; j += stride) m.ctl[j] = 0u;
  for (int64_t j = i; j < 2 * m.dep_blocks + 16; j += stride) m.dep[j] = 0u;
  constexpr int words = (int)(sizeof(MegaArgs) / 4);
  static_assert(sizeof(MegaArgs) % 4 == 0, "argument block copies as words");
  if (blockIdx.x == 0) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&m);
    for (int w = threadIdx.x; w < words; w += blockDim.x) reinterpret_cast<uint32_t*>(out)[w] = src[w];
  }
}

// The grid barriers need every workgroup of the grid resident at once.  The
// grid is one workgroup per CU and the kernel's LDS use admits one per CU,
// which the occupancy query confirms here.  By default the launch is an
// ordinary one: work of other streams that holds CUs only delays the late
// workgroups, which the barriers wait for (bounded).  A plan made with
// MM_COOPERATIVE=1 launches cooperatively: the runtime then starts the grid
// only once all of it can be resident, at some microseconds per call.
template <int UC, int BM, bool WIDEN>
static hipError_t launch_mega_one(const MegaArgs* dev_args, int grid, bool cooperative, hipStream_t s) {
  constexpr size_t lds = (size_t)mega_lds_bytes<UC, BM>();
  static int per_cu = -1;
  if (per_cu < 0) {
    hipError_t err = hipFuncSetAttribute((const void*)k_mega<UC, BM, WIDEN>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    int n = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_mega<UC, BM, WIDEN>, threads_of<BM>(), lds);
    if (err != hipSuccess) return err;
    per_cu = n;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  if (per_cu < 1 || grid > per_cu * cus) return hipErrorCooperativeLaunchTooLarge;
  if (cooperative) {
    // the runtime starts the grid only when all of it can be resident
    const MegaArgs* arg = dev_args;
    void* params[] = {(void*)&arg};
    return hipLaunchCooperativeKernel((const void*)k_mega<UC, BM, WIDEN>, dim3(grid), dim3(threads_of<BM>()), params,
                                      (unsigned)lds, s);
  }
  hipLaunchKernelGGL((k_mega<UC, BM, WIDEN>), dim3(grid), dim3(threads_of<BM>()), lds, s, dev_args);
  return hipGetLastError();
}

template <int UC, bool WIDEN = false>
static hipError_t launch_mega_bm(int tile, const MegaArgs* a, int grid, bool coop, hipStream_t s) {
  switch (tile) {
    case TILE_M64_N128: return launch_mega_one<UC, 64, WIDEN>(a, grid, coop, s);
    case TILE_M256_N256:
      if constexpr (is_mx(UC)) return hipErrorInvalidValue;   // the plan keeps MX at 128
      else return launch_mega_one<UC, 256, WIDEN>(a, grid, coop, s);
    default: return launch_mega_one<UC, 128, WIDEN>(a, grid, coop, s);
  }
}

hipError_t launch_mega_prep(const MegaArgs& a, MegaArgs* dev_args, hipStream_t s) {
  int grid = (a.d.E + 255) / 256;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_mega_prep, dim3(grid), dim3(256), 0, s, a, dev_args);
  return hipGetLastError();
}

hipError_t launch_mega(int usecase, int tile, bool exact_l1, const MegaArgs* dev_args, int grid, bool coop,
                       hipStream_t s) {
  switch (usecase) {
    case UC_BF16: return launch_mega_bm<UC_BF16>(tile, dev_args, grid, coop, s);
    case UC_FP8:
      return exact_l1 ? launch_mega_bm<UC_FP8, true>(tile, dev_args, grid, coop, s)
                      : launch_mega_bm<UC_FP8>(tile, dev_args, grid, coop, s);
    case UC_MX8:
      return exact_l1 ? launch_mega_bm<UC_MX8, true>(tile, dev_args, grid, coop, s)
                      : launch_mega_bm<UC_MX8>(tile, dev_args, grid, coop, s);
    case UC_MX4:
      return exact_l1 ? launch_mega_bm<UC_MX4, true>(tile, dev_args, grid, coop, s)
                      : launch_mega_bm<UC_MX4>(tile, dev_args, grid, coop, s);
    default: return launch_mega_bm<UC_I8>(tile, dev_args, grid, coop, s);
  }
}

int mega_grid(int /*tile*/, int num_cus) { return num_cus; }   // one resident workgroup per CU

}  // namespace mm
