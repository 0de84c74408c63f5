// Stand-alone kernels of the three-call path: grouped GEMMs, A8W8
// requantisation, Token Combine (thin wrappers over mm_gemm_dev.hpp).
#include "mm_gemm_dev.hpp"

namespace mm {

template <int UC, int BM, int MODE, bool WIDEN>
__global__ __launch_bounds__(threads_of<BM>()) __attribute__((amdgpu_waves_per_eu(threads_of<BM>() / 256, threads_of<BM>() / 256)))
void k_gemm(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int32_t off_s[max_experts<UC>() + 1];
  __shared__ int32_t cnt_s[max_experts<UC>()];
  gemm_tiles<UC, BM, MODE, WIDEN>(a, lds, off_s, cnt_s);
}

template <int UC, int BM, int MODE, bool WIDEN>
static hipError_t launch_one(const GemmArgs& a, int grid, hipStream_t s) {
  constexpr size_t lds = (size_t)lds_bytes_of<UC, BM>();
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

template <int UC, int MODE, bool WIDEN = false>
static hipError_t launch_bm(int tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tile) {
    case TILE_M64_N128: return launch_one<UC, 64, MODE, WIDEN>(a, grid, s);
    case TILE_M256_N256:
      if constexpr (is_mx(UC)) return hipErrorInvalidValue;   // the plan keeps MX at 128
      else return launch_one<UC, 256, MODE, WIDEN>(a, grid, s);
    default: return launch_one<UC, 128, MODE, WIDEN>(a, grid, s);
  }
}

// e4m3 Linear1 either on the e4m3 MFMA, or (exact_l1) on the bf16 MFMA after
// an exact e4m3 -> bf16 widening: the e4m3 MFMAs round inside their dot
// products, and the per-row requantisation after Linear1 can turn that into
// code changes, which move Y visibly when I is small.  Linear2 always keeps
// the e4m3 MFMA (nothing is quantised after it).
template <int MODE>
static hipError_t launch_uc(int usecase, int tile, bool exact_l1, const GemmArgs& a, int grid, hipStream_t s) {
  switch (usecase) {
    case UC_BF16: return launch_bm<UC_BF16, MODE>(tile, a, grid, s);
    case UC_FP8:
      if (MODE == 0 && exact_l1) return launch_bm<UC_FP8, MODE, MODE == 0>(tile, a, grid, s);
      return launch_bm<UC_FP8, MODE>(tile, a, grid, s);
    case UC_MX8:
      if (MODE == 0 && exact_l1) return launch_bm<UC_MX8, MODE, MODE == 0>(tile, a, grid, s);
      return launch_bm<UC_MX8, MODE>(tile, a, grid, s);
    case UC_MX4:
      if (MODE == 0 && exact_l1) return launch_bm<UC_MX4, MODE, MODE == 0>(tile, a, grid, s);
      return launch_bm<UC_MX4, MODE>(tile, a, grid, s);
    default: return launch_bm<UC_I8, MODE>(tile, a, grid, s);
  }
}

hipError_t launch_gemm(int mode, int usecase, int tile, bool exact_l1, const GemmArgs& a, int grid, hipStream_t s) {
  if (mode == 0) return launch_uc<0>(usecase, tile, exact_l1, a, grid, s);
  if (mode == 1) return launch_uc<1>(usecase, tile, exact_l1, a, grid, s);
  if (usecase == UC_FP8) return exact_l1 ? launch_bm<UC_FP8, 2, true>(tile, a, grid, s) : launch_bm<UC_FP8, 2>(tile, a, grid, s);
  if (usecase != UC_I8) return hipErrorInvalidValue;
  return launch_bm<UC_I8, 2>(tile, a, grid, s);
}

// One resident workgroup per CU (LDS bound), the fused kernel's grid too:
// the tail split depends on the grid, so both paths split alike and their
// results agree bit for bit.
int gemm_grid(int /*tile*/, int64_t /*P*/, int /*N*/, int num_cus) { return num_cus < 1 ? 1 : num_cus; }

template <int UC>
__global__ __launch_bounds__(256) void k_requant(RequantArgs a) {
  __shared__ int32_t off_s[kMaxExperts + 1];
  __shared__ int32_t cnt_s[kMaxExperts];
  for (int e = threadIdx.x; e <= a.E; e += 256) off_s[e] = a.offsets[e];
  for (int e = threadIdx.x; e < a.E; e += 256) cnt_s[e] = a.counts[e];
  __syncthreads();
  requant_rows<UC, 1>(a, (int64_t)blockIdx.x * 4 + threadIdx.x / 64, 0, off_s, cnt_s);
}

hipError_t launch_requant(const RequantArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.P + 3) / 4));
  if (a.usecase == UC_I8) hipLaunchKernelGGL(k_requant<UC_I8>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_requant<UC_FP8>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int64_t work = a.T * (a.H / 8), idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a.slot_bf16) combine_items<1, true>(a, idx, 0, work);
  else combine_items<1, false>(a, idx, 0, work);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.T * (a.H / 8) + 255) / 256));
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm
