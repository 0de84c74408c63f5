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
constexpr int kLdsRow = 144;            // padded LDS row pitch
constexpr int kMaxExperts = 1024;

// waves of a workgroup: WM along M x WN along N (a wave's N range must hold
// whole 64-row gate/up groups, so WTN >= 64)
template <int BM> struct WaveGrid;
template <> struct WaveGrid<32> { static constexpr int WM = 1, WN = 4; };
template <> struct WaveGrid<64> { static constexpr int WM = 2, WN = 4; };
template <> struct WaveGrid<128> { static constexpr int WM = 2, WN = 4; };
template <> struct WaveGrid<256> { static constexpr int WM = 2, WN = 4; };
template <int BM> constexpr int threads_of() { return 64 * WaveGrid<BM>::WM * WaveGrid<BM>::WN; }

template <int UC, int BM, int MODE, bool WIDEN>
__global__ __launch_bounds__(threads_of<BM>()) __attribute__((amdgpu_waves_per_eu(threads_of<BM>() / 256, threads_of<BM>() / 256)))
void k_gemm(GemmArgs a) {
  constexpr int WM = WaveGrid<BM>::WM, WN = WaveGrid<BM>::WN;
  constexpr int NT = threads_of<BM>();
  constexpr int WTM = BM / WM, WTN = kBN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int ROWS = BM + kBN;
  // global bytes per row per stage: 128, or 64 e4m3 widened to 128 bytes of bf16
  constexpr int GB = WIDEN ? 64 : kRowBytes;
  constexpr int GCH = GB / 16;                             // 16-byte global chunks per row
  constexpr int CH = (ROWS * GCH + NT - 1) / NT;           // chunks per thread per stage
  constexpr int STAGE = ROWS * kLdsRow;
  constexpr int ESZ = (UC == UC_BF16) ? 2 : 1;
  constexpr bool MF_BF16 = (UC == UC_BF16) || WIDEN;       // MFMA operand type
  typedef typename Acc<UC>::type AccT;

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int32_t off_s[kMaxExperts + 1];
  __shared__ int32_t cnt_s[kMaxExperts];

  const int t = threadIdx.x, w = t / 64, l = lane_id();
  const int h = l / 32, lr = l % 32;
  const int wm = w / WN, wn = w % WN;

  for (int e = t; e <= a.E; e += NT) off_s[e] = a.offsets[e];
  for (int e = t; e < a.E; e += NT) cnt_s[e] = a.counts[e];
  __syncthreads();

  const int64_t kbytes = (int64_t)a.Kdim * ESZ;
  const int nk = (int)(kbytes / GB);
  const int n_tiles = a.N / kBN;
  const int total = (off_s[a.E] / BM) * n_tiles;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mblk = tile / n_tiles, nblk = tile % n_tiles;
    const int row0 = mblk * BM, n0 = nblk * kBN;
    // expert of this M-block: the largest e with off[e] <= row0
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off_s[mid] <= row0) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int valid = min(BM, off_s[e] + cnt_s[e] - row0);

    // Global chunk addresses: the A and B tile origins are wave-uniform (scalar
    // bases); each thread keeps 32-bit offsets.  Chunk j of thread t is chunk
    // c = t + NT*j of the stage; rows [0, BM) are A rows, the rest B rows.
    const uint8_t* abase = a.A + (int64_t)row0 * kbytes;
    const uint8_t* bbase = a.B + ((int64_t)e * a.N + n0) * kbytes;
    uint32_t goff[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = min(t + NT * j, ROWS * GCH - 1);
      const int row = c / GCH, col = c % GCH;
      goff[j] = (uint32_t)((row < BM ? row : row - BM) * kbytes + col * 16);
    }
    u32x4 stg[CH];
    auto load_stage = [&](int kb) {
      const uint8_t* ab = abase + (int64_t)kb * GB;
      const uint8_t* bb = bbase + (int64_t)kb * GB;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = t + NT * j;
        if (CH * NT == ROWS * GCH || c < ROWS * GCH) {
          // rows of chunk j are all A rows or all B rows when NT divides BM*GCH
          const bool is_a = (BM * GCH) % NT == 0 ? (j < BM * GCH / NT) : (c / GCH < BM);
          stg[j] = *reinterpret_cast<const u32x4*>((is_a ? ab : bb) + goff[j]);
        }
      }
    };
    auto store_stage = [&](int buf) {
      uint8_t* base = lds + buf * STAGE;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = t + NT * j;
        if (CH * NT != ROWS * GCH && c >= ROWS * GCH) continue;
        if constexpr (WIDEN) {
          // 16 e4m3 -> 16 bf16 (exact: every e4m3 value is a bf16 value)
          const u32x4 wv = stg[j];
          uint32_t o[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[q], 1.0f, false));
            o[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv[q], 1.0f, true));
          }
          uint8_t* d = base + (c / GCH) * kLdsRow + (c % GCH) * 32;
          *reinterpret_cast<u32x4*>(d) = u32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<u32x4*>(d + 16) = u32x4{o[4], o[5], o[6], o[7]};
        } else {
          *reinterpret_cast<u32x4*>(base + (c / GCH) * kLdsRow + (c % GCH) * 16) = stg[j];
        }
      }
    };

    AccT acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kb = 0; kb < nk; ++kb) {
      const int cur = kb & 1;
      if (kb + 1 < nk) load_stage(kb + 1);
      const uint8_t* As = lds + cur * STAGE + (wm * WTM + lr) * kLdsRow + h * 64;
      const uint8_t* Bs = lds + cur * STAGE + (BM + wn * WTN + lr) * kLdsRow + h * 64;
      if constexpr (UC == UC_FP8 && !WIDEN) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          u32x4 af[MB][2], bfr[NB][2];
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            af[i][0] = *reinterpret_cast<const u32x4*>(As + i * 32 * kLdsRow + s * 32);
            af[i][1] = *reinterpret_cast<const u32x4*>(As + i * 32 * kLdsRow + s * 32 + 16);
          }
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            bfr[j][0] = *reinterpret_cast<const u32x4*>(Bs + j * 32 * kLdsRow + s * 32);
            bfr[j][1] = *reinterpret_cast<const u32x4*>(Bs + j * 32 * kLdsRow + s * 32 + 16);
          }
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) mfma_fp8(acc[i][j], af[i][0], af[i][1], bfr[j][0], bfr[j][1]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 af[MB], bfr[NB];
#pragma unroll
          for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const u32x4*>(As + i * 32 * kLdsRow + s * 16);
#pragma unroll
          for (int j = 0; j < NB; ++j) bfr[j] = *reinterpret_cast<const u32x4*>(Bs + j * 32 * kLdsRow + s * 16);
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              if constexpr (MF_BF16) mfma_bf16(acc[i][j], af[i], bfr[j]);
              else mfma_i8(acc[i][j], af[i], bfr[j]);
            }
        }
      }
      if (kb + 1 < nk) store_stage(cur ^ 1);
      __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
    if constexpr (MODE == 0) {
      // blocks alternate gate (even) / up (odd); pair j covers 32 output columns
      const int colbase = (n0 + wn * WTN) / 2;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int rl = wm * WTM + i * 32 + 8 * (q / 4) + 4 * h + (q % 4);
          const bool ok = rl < valid;
          const int64_t p = (int64_t)row0 + rl;
          float rmax = 0.0f;
          float sx = 1.0f;
          if constexpr (UC != UC_BF16) sx = ok ? a.x_scale[p] : 0.0f;
#pragma unroll
          for (int j = 0; j < NB / 2; ++j) {
            const int col = colbase + j * 32 + lr;
            float g = acc_to_f32(acc[i][2 * j][q]);
            float u = acc_to_f32(acc[i][2 * j + 1][q]);
            if constexpr (UC != UC_BF16) {
              const float* ws = a.w_scale + (int64_t)e * 2 * a.I;
              g = (g * ws[col]) * sx;
              u = (u * ws[a.I + col]) * sx;
            }
            const float av = silu(g) * u;
            if constexpr (UC == UC_BF16) {
              if (ok) static_cast<uint16_t*>(a.a_out)[p * a.I + col] = f32_to_bf16_bits(av);
            } else {
              if (ok) a.a_stage[p * a.I + col] = av;
              rmax = fmaxf(rmax, fabsf(av));
            }
          }
          if constexpr (UC != UC_BF16) {
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o, 64));
            if (ok && lr == 0) atomicMax(&a.a_amax[p], __float_as_uint(rmax));
          }
        }
      }
    } else if constexpr (MODE == 1) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int rl = wm * WTM + i * 32 + 8 * (q / 4) + 4 * h + (q % 4);
          if (rl >= valid) continue;
          const int64_t p = (int64_t)row0 + rl;
          const int32_t r = a.pool_src[p];
          float rs = 1.0f;
          if constexpr (UC != UC_BF16) rs = a.a_scale[p];
          const float gw = a.topk_w[r];
          float* dst = a.contrib + (int64_t)r * a.H;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int col = n0 + wn * WTN + j * 32 + lr;
            float v = acc_to_f32(acc[i][j][q]);
            if constexpr (UC != UC_BF16) v = (v * a.w_scale[(int64_t)e * a.H + col]) * rs;
            dst[col] = v * gw;
          }
        }
      }
    } else {
      // raw accumulators, formula column order
#pragma unroll
      for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int rl = wm * WTM + i * 32 + 8 * (q / 4) + 4 * h + (q % 4);
          if (rl >= valid) continue;
          const int64_t p = (int64_t)row0 + rl;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int n = n0 + wn * WTN + j * 32 + lr;
            int col = n;
            if (a.gate_up_group > 0) {
              const int g2 = 2 * a.gate_up_group;
              const int qq = n / g2, m = n % g2;
              col = (m < a.gate_up_group) ? qq * a.gate_up_group + m : a.I + qq * a.gate_up_group + (m - a.gate_up_group);
            }
            if constexpr (UC == UC_I8) a.raw_out[p * a.N + col] = acc[i][j][q];
          }
        }
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
  constexpr size_t lds = 2 * (size_t)(BM + kBN) * kLdsRow;
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
    case TILE_M32_N256: return launch_one<UC, 32, MODE>(a, grid, s);
    case TILE_M64_N256: return launch_one<UC, 64, MODE>(a, grid, s);
    case TILE_M128_N256: return launch_one<UC, 128, MODE>(a, grid, s);
    default: return launch_one<UC, 256, MODE>(a, grid, s);
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
