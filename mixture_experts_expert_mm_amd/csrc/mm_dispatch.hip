// EP Dispatch kernels of the three-call path (thin wrappers over the
// device bodies shared with the fused kernel), the per-call counter reset
// and the one-time weight relayout.
#include "mm_dispatch_dev.hpp"

namespace mm {

// ---------------------------------------------------------------------------
// reset of the per-call counters and control words
// ---------------------------------------------------------------------------
__global__ void k_zero(int32_t* __restrict__ counts, int E, uint32_t* __restrict__ ctl, int ctl_first, int ctl_n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (counts)
    for (int64_t j = i; j < E; j += stride) counts[j] = 0;
  if (ctl)
    for (int64_t j = i; j < ctl_n; j += stride) ctl[ctl_first + j] = 0u;
}

__global__ __launch_bounds__(256) void k_count(DispatchArgs a, int64_t nwaves) {
  extern __shared__ int32_t smem[];
  count_block<kDispatchWavesPerBlock>(a, blockIdx.x, nwaves, smem);
}

__global__ __launch_bounds__(256) void k_scatter(DispatchArgs a, int64_t nwaves) {
  extern __shared__ int32_t smem[];
  int32_t* off = smem;                     // [E+1]
  int32_t* run = smem + a.E + 1;           // [4][E]
  __shared__ int32_t wsum[kDispatchWavesPerBlock];
  padded_prefix<256>(a, a.counts, off, wsum);
  if (blockIdx.x == 0)
    for (int e = threadIdx.x; e <= a.E; e += 256) a.offsets[e] = off[e];
  scatter_block<kDispatchWavesPerBlock>(a, blockIdx.x, gridDim.x, nwaves, off, run);
}

template <int UC>
__global__ __launch_bounds__(256) void k_gather(DispatchArgs a) {
  __shared__ int32_t dst[64];
  __shared__ float red[4];
  gather_token<UC, 256>(a, blockIdx.x, dst, red);
}

// ---------------------------------------------------------------------------
// one-time weight relayout (K-contiguous rows, gate/up interleave for W1)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ in, T* __restrict__ out,
                                                   int rows_in, int cols_in, int inter, int group) {
  // in [E][rows_in][cols_in] -> out [E][cols_in][rows_in]; out row n takes
  // in column c(n) (gate/up interleave when group > 0, identity otherwise)
  __shared__ T tile[64][65];
  const int e = blockIdx.z;
  const int n0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const T* src = in + (int64_t)e * rows_in * cols_in;
  T* dstp = out + (int64_t)e * rows_in * cols_in;
  const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
  for (int r = ty; r < 64; r += 4) {
    const int n = n0 + tx, row = r0 + r;
    if (n < cols_in && row < rows_in) {
      int c = n;
      if (group > 0) {
        const int q = n / (2 * group), m = n % (2 * group);
        c = (m < group) ? q * group + m : inter + q * group + (m - group);
      }
      tile[r][tx] = src[(int64_t)row * cols_in + c];
    }
  }
  __syncthreads();
  for (int j = ty; j < 64; j += 4) {
    const int n = n0 + j, row = r0 + tx;
    if (n < cols_in && row < rows_in) dstp[(int64_t)n * rows_in + row] = tile[tx][j];
  }
}

// e2m1 weights, two per byte: in [E][rows_in][cols_in/2] (packed along the
// columns) -> out [E][cols_in][rows_in/2] (packed along the rows), with the
// gate/up interleave c(n) of the output rows when group > 0.  One output
// byte per thread: values (2b, n) and (2b+1, n), the even one in the low
// nibble.
__global__ __launch_bounds__(256) void k_transpose_e2m1(const uint8_t* __restrict__ in, uint8_t* __restrict__ out,
                                                         int rows_in, int cols_in, int inter, int group) {
  const int e = blockIdx.z;
  const int64_t per_e = (int64_t)rows_in * cols_in / 2;
  const uint8_t* src = in + e * per_e;
  uint8_t* dstp = out + e * per_e;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // output byte of expert e
  if (idx >= per_e) return;
  const int n = (int)(idx / (rows_in / 2)), b = (int)(idx % (rows_in / 2));
  int c = n;
  if (group > 0) {
    const int q = n / (2 * group), m = n % (2 * group);
    c = (m < group) ? q * group + m : inter + q * group + (m - group);
  }
  const int r0 = 2 * b, r1 = 2 * b + 1;
  const uint32_t v0 = (src[(int64_t)r0 * (cols_in / 2) + c / 2] >> ((c & 1) * 4)) & 0xFu;
  const uint32_t v1 = (src[(int64_t)r1 * (cols_in / 2) + c / 2] >> ((c & 1) * 4)) & 0xFu;
  dstp[idx] = (uint8_t)(v0 | (v1 << 4));
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_zero(int32_t* counts, int E, uint32_t* ctl, int ctl_first, int ctl_n, hipStream_t s) {
  int grid = ((E > ctl_n ? E : ctl_n) + 255) / 256;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_zero, dim3(grid), dim3(256), 0, s, counts, E, ctl, ctl_first, ctl_n);
  return hipGetLastError();
}

hipError_t launch_count(const DispatchArgs& a, hipStream_t s) {
  const int64_t nw = dispatch_waves(a.T, a.K);
  const int grid = (int)((nw + kDispatchWavesPerBlock - 1) / kDispatchWavesPerBlock);
  const size_t lds = sizeof(int32_t) * kDispatchWavesPerBlock * a.E;
  hipLaunchKernelGGL(k_count, dim3(grid), dim3(256), lds, s, a, nw);
  return hipGetLastError();
}

hipError_t launch_scatter(const DispatchArgs& a, hipStream_t s) {
  const int64_t nw = dispatch_waves(a.T, a.K);
  const int grid = (int)((nw + kDispatchWavesPerBlock - 1) / kDispatchWavesPerBlock);
  const size_t lds = sizeof(int32_t) * ((a.E + 1) + kDispatchWavesPerBlock * a.E);
  hipLaunchKernelGGL(k_scatter, dim3(grid), dim3(256), lds, s, a, nw);
  return hipGetLastError();
}

hipError_t launch_gather(const DispatchArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.T);
  switch (a.usecase) {
    case UC_BF16: hipLaunchKernelGGL(k_gather<UC_BF16>, grid, dim3(256), 0, s, a); break;
    case UC_FP8: hipLaunchKernelGGL(k_gather<UC_FP8>, grid, dim3(256), 0, s, a); break;
    case UC_MX8:
    case UC_MX4: hipLaunchKernelGGL(k_gather<UC_MX8>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_gather<UC_I8>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_prepare(const void* w1, const void* w2, void* w1o, void* w2o, int E, int H, int I,
                          int esz, int group, hipStream_t s) {
  const dim3 g1((2 * I + 63) / 64, (H + 63) / 64, E), g2((H + 63) / 64, (I + 63) / 64, E);
  if (esz == 0) {   // e2m1: W1 [E][H][2I] -> [E][2I][H], W2 [E][I][H] -> [E][H][I], nibbles
    const unsigned b1 = (unsigned)(((int64_t)H * 2 * I / 2 + 255) / 256), b2 = (unsigned)(((int64_t)I * H / 2 + 255) / 256);
    hipLaunchKernelGGL(k_transpose_e2m1, dim3(b1, 1, E), dim3(256), 0, s, (const uint8_t*)w1, (uint8_t*)w1o, H, 2 * I, I, group);
    hipLaunchKernelGGL(k_transpose_e2m1, dim3(b2, 1, E), dim3(256), 0, s, (const uint8_t*)w2, (uint8_t*)w2o, I, H, 0, 0);
  } else if (esz == 2) {
    hipLaunchKernelGGL(k_transpose<uint16_t>, g1, dim3(256), 0, s, (const uint16_t*)w1, (uint16_t*)w1o, H, 2 * I, I, group);
    hipLaunchKernelGGL(k_transpose<uint16_t>, g2, dim3(256), 0, s, (const uint16_t*)w2, (uint16_t*)w2o, I, H, 0, 0);
  } else {
    hipLaunchKernelGGL(k_transpose<uint8_t>, g1, dim3(256), 0, s, (const uint8_t*)w1, (uint8_t*)w1o, H, 2 * I, I, group);
    hipLaunchKernelGGL(k_transpose<uint8_t>, g2, dim3(256), 0, s, (const uint8_t*)w2, (uint8_t*)w2o, I, H, 0, 0);
  }
  return hipGetLastError();
}

}  // namespace mm
