// Device-side bodies of EP Dispatch, shared by the stand-alone dispatch
// kernels and the fused persistent kernel: route read, count + claim,
// padded prefix, scatter, gather (+ per-token activation quantisation).
//
// Count -> Prefix Sum -> Scatter follows the DeepEP "Metadata System" notes
// (sections 3.2-3.5): routes are counted in LDS, each wavefront claims its
// range inside an expert with one global atomic per expert it touches (the
// returned old value is the wave's base inside that expert), and the final
// slot of a route is the wave base plus its rank among the lanes of the
// same expert (ballot + popcount).  Pool rows of expert e start at the
// padded prefix off[e] (a multiple of BLOCK_M).
#pragma once
#include "mm_device.hpp"
#include "mm_internal.hpp"

namespace mm {

// Expert of route (tok, slot): a routed slot (slot < Kr) reads topk_ids, a
// shared-expert slot names expert Er + (slot - Kr).  -1 for masked routes
// (id < 0), ids >= Er (which also raise MM_DEVERR_BAD_EXPERT) and every
// slot of a token whose x_active_mask entry is 0 (the token takes part in
// nothing, so its output row is 0).
__device__ __forceinline__ int route_expert(const DispatchArgs& a, int64_t tok, int slot) {
  if (a.active && a.active[tok] == 0) return -1;
  if (slot >= a.Kr) return a.Er + (slot - a.Kr);
  const int e = a.topk_ids[tok * a.Kr + slot];
  if (e >= a.Er && a.err) atomicOr(a.err, (uint32_t)MM_DEVERR_BAD_EXPERT);
  return (e >= 0 && e < a.Er) ? e : -1;
}

// Route of lane l of global wave gw: token gw*tpw + l/K, slot l%K.  Returns
// the expert id (route_expert), or -1 for idle lanes and skipped routes.
__device__ __forceinline__ int read_route(const DispatchArgs& a, int64_t gw, int l, int64_t* route) {
  const int tpw = 64 / a.K;
  const int64_t tok = gw * tpw + l / a.K;
  const int slot = l % a.K;
  *route = -1;
  if (l >= tpw * a.K || tok >= a.T) return -1;
  *route = tok * a.K + slot;
  return route_expert(a, tok, slot);
}

// Count + claim for dispatch waves vb*NW .. vb*NW+NW-1, one per wave of the
// block: LDS histogram per wave (smem: NW * E ints), then one global atomic
// per (wave, expert) with a nonzero count.
template <int NW>
__device__ __forceinline__ void count_block(const DispatchArgs& a, int64_t vb, int64_t nwaves, int32_t* smem) {
  const int w = threadIdx.x / 64, l = lane_id();
  int32_t* hist = smem + w * a.E;
  const int64_t gw = vb * NW + w;
  for (int e = l; e < a.E; e += 64) hist[e] = 0;
  __syncthreads();
  int64_t route;
  const int e = (gw < nwaves) ? read_route(a, gw, l, &route) : -1;
  if (e >= 0) atomicAdd(&hist[e], 1);
  __syncthreads();
  if (gw < nwaves) {
    for (int ex = l; ex < a.E; ex += 64) {
      const int c = hist[ex];
      if (c > 0) a.wave_base[gw * a.E + ex] = atomicAdd(&a.counts[ex], c);
    }
  }
  __syncthreads();
}

// Block-wide exclusive scan of the BLOCK_M-padded counts cnt[0..E-1] (the
// global counts, or an LDS copy) into off[0..E] (wsum: NT/64 ints of LDS).
template <int NT>
__device__ __forceinline__ void padded_prefix(const DispatchArgs& a, const int32_t* cnt, int32_t* off, int32_t* wsum) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, w = t / 64, l = lane_id();
  const int per = (a.E + NT - 1) / NT;
  const int e0 = t * per;
  int local = 0;
  for (int j = 0; j < per; ++j) {
    const int e = e0 + j;
    if (e < a.E) local += (cnt[e] + a.block_m - 1) / a.block_m * a.block_m;
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (l >= o) incl += v;
  }
  if (l == 63) wsum[w] = incl;
  __syncthreads();
  int excl = incl - local;
  for (int ww = 0; ww < w; ++ww) excl += wsum[ww];
  for (int j = 0; j < per; ++j) {
    const int e = e0 + j;
    if (e < a.E) {
      off[e] = excl;
      excl += (cnt[e] + a.block_m - 1) / a.block_m * a.block_m;
    }
  }
  if (t == 0) {
    int total = 0;
    for (int ww = 0; ww < NW; ++ww) total += wsum[ww];
    off[a.E] = total;
  }
  __syncthreads();
}

// The whole dispatch of a small batch (at most MAXR * NT routes) by one
// block, with no grid-wide step between count and scatter.  Thread t takes
// routes t, t + NT, ...; a route's rank inside its expert is the old value
// of an LDS atomic add on that expert's count (hist: E ints of LDS).  Then,
// as in the multi-block path: the padded prefix, counts and offsets out,
// pool_src / route_to_pool, and pool_src = -1 on every expert's padding
// rows.  The order of the routes inside an expert is arbitrary here as it
// is with the per-wave claims; every later step computes a route's result
// from its own row alone, so the output does not depend on that order.
template <int NT, int MAXR>
__device__ __forceinline__ void dispatch_one_block(const DispatchArgs& a, int32_t* hist, int32_t* off, int32_t* wsum) {
  const int t = threadIdx.x;
  const int64_t R = a.T * a.K;
  for (int e = t; e < a.E; e += NT) hist[e] = 0;
  __syncthreads();
  int ex[MAXR], rk[MAXR];
  // registers set first and loads that only fill them: every load goes out
  // before the first wait
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const int64_t r = t + (int64_t)NT * j;
    ex[j] = r < R ? route_expert(a, r / a.K, (int)(r % a.K)) : -1;
  }
#pragma unroll
  for (int j = 0; j < MAXR; ++j) rk[j] = ex[j] >= 0 ? atomicAdd(&hist[ex[j]], 1) : 0;
  __syncthreads();
  padded_prefix<NT>(a, hist, off, wsum);
  for (int e = t; e < a.E; e += NT) a.counts[e] = hist[e];
  for (int e = t; e <= a.E; e += NT) a.offsets[e] = off[e];
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const int64_t r = t + (int64_t)NT * j;
    if (r < R) {
      const int32_t p = ex[j] >= 0 ? off[ex[j]] + rk[j] : -1;
      a.route_to_pool[r] = p;
      if (p >= 0) a.pool_src[p] = (int32_t)r;
    }
  }
  for (int e = 0; e < a.E; ++e)
    for (int64_t p = (int64_t)off[e] + hist[e] + t; p < off[e + 1]; p += NT) a.pool_src[p] = -1;
  __syncthreads();
}

// Scatter for dispatch waves vb*NW.. (off: the padded prefix in LDS; run:
// NW * E ints of LDS).  Virtual block vb of nvb also marks the padding rows
// of experts vb, vb + nvb, ... with pool_src = -1.
template <int NW>
__device__ __forceinline__ void scatter_block(const DispatchArgs& a, int64_t vb, int64_t nvb, int64_t nwaves, const int32_t* off,
                              int32_t* run) {
  constexpr int NT = NW * 64;
  const int t = threadIdx.x, w = t / 64, l = lane_id();
  for (int64_t e = vb; e < a.E; e += nvb) {
    const int64_t p0 = (int64_t)off[e] + a.counts[e], p1 = off[e + 1];
    for (int64_t p = p0 + t; p < p1; p += NT) a.pool_src[p] = -1;
  }
  const int64_t gw = vb * NW + w;
  if (gw < nwaves) {
    int32_t* myrun = run + w * a.E;
    // running pool position per expert: padded prefix + the wave's claimed
    // base (entries of experts this wave does not touch are never read)
    for (int e = l; e < a.E; e += 64) myrun[e] = off[e] + a.wave_base[gw * a.E + e];
    __builtin_amdgcn_wave_barrier();
    int64_t route;
    const int e = read_route(a, gw, l, &route);
    int32_t p = -1;
    uint64_t act = ballot(e >= 0);
    while (act) {
      const int leader = __ffsll((unsigned long long)act) - 1;
      const int le = __shfl(e, leader, 64);
      const uint64_t m = ballot(e == le);
      const int base = myrun[le];
      if (e == le) p = base + __popcll(m & lanemask_lt());
      __builtin_amdgcn_wave_barrier();
      if (l == leader) myrun[le] = base + __popcll(m);
      __builtin_amdgcn_wave_barrier();
      act &= ~m;
    }
    if (route >= 0) {
      a.route_to_pool[route] = p;
      if (p >= 0) a.pool_src[p] = (int32_t)route;
    }
  }
  __syncthreads();
}

// A8W8 activation quantisation: s_i = max(max|x_i| / Qmax, 1e-8) and
// q = round(x_i / s_i) in IEEE float32 (correctly rounded division), int8
// ties-to-even clamped to [-127,127] or e4m3fn ties-to-even saturated to
// +-448.
constexpr int kMaxHidden = 16384;

// The 8 codes of 8 bf16 activations (one 16-byte chunk) at scale s.
template <int UC>
__device__ __forceinline__ uint2 codes8_of_bf16(const uint4& v, float s) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float f0 = bf16_bits_to_f32(wv[2 * q] & 0xffffu) / s;
    const float f1 = bf16_bits_to_f32(wv[2 * q] >> 16) / s;
    const float f2 = bf16_bits_to_f32(wv[2 * q + 1] & 0xffffu) / s;
    const float f3 = bf16_bits_to_f32(wv[2 * q + 1] >> 16) / s;
    if constexpr (UC == UC_I8) {
      o[q] = (uint32_t)(f32_to_i8sym(f0) & 0xff) | ((uint32_t)(f32_to_i8sym(f1) & 0xff) << 8) |
             ((uint32_t)(f32_to_i8sym(f2) & 0xff) << 16) | ((uint32_t)(f32_to_i8sym(f3) & 0xff) << 24);
    } else {
      o[q] = f32x2_to_e4m3x2(f0, f1) | (f32x2_to_e4m3x2(f2, f3) << 16);
    }
  }
  return make_uint2(o[0], o[1]);
}

// MX-FP8 codes of 8 bf16 activations: e4m3(x * 2^-X), exact scaling by the
// group's element multiplier inv = 2^-X (saturating at +-448, ties to even).
__device__ __forceinline__ uint2 mx_codes8_of_bf16(const uint4& v, float inv) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float f0 = bf16_bits_to_f32(wv[2 * q] & 0xffffu) * inv;
    const float f1 = bf16_bits_to_f32(wv[2 * q] >> 16) * inv;
    const float f2 = bf16_bits_to_f32(wv[2 * q + 1] & 0xffffu) * inv;
    const float f3 = bf16_bits_to_f32(wv[2 * q + 1] >> 16) * inv;
    o[q] = f32x2_to_e4m3x2(f0, f1) | (f32x2_to_e4m3x2(f2, f3) << 16);
  }
  return make_uint2(o[0], o[1]);
}

__device__ __forceinline__ float amax8_of_bf16(const uint4& v, float m) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(wv[q] & 0xffffu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(wv[q] >> 16)));
  }
  return m;
}

// A8W8 quantisation of token i by one wave into row i of a [T][H] code
// buffer (x_pool, x_pool_scale indexed by token): the fused kernel's step
// for a Linear1 that reads token rows in place.  A block runs one token per
// wave, so the loads of several tokens are in flight without block
// barriers.  Rows of up to 64 * kTokRegChunks chunks stay in registers
// between the amax and the codes; longer rows are read twice.  Same
// arithmetic, so the same codes and scale, as the block gather below.
template <int UC>
__device__ __forceinline__ void quant_token_wave(const DispatchArgs& a, int64_t i) {
  constexpr int kTokRegChunks = 16;   // H <= 64 * 16 * 8 = 8192
  const int l = lane_id();
  const int nchunk = (int)(a.H / 8);
  const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + i * a.H);
  uint2* dst = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.x_pool) + i * a.H);
  if constexpr (is_mx(UC)) {
    // Q_MX per group of 32: chunk c (8 values) belongs to group c / 4, the
    // four chunks of a group sit in four neighbouring lanes (c = j*64 + l)
    uint8_t* const sc = a.x_pool_mx + i * (a.H / kMxGroup);
    for (int j0 = 0; j0 < nchunk; j0 += 64 * kTokRegChunks) {
      uint4 v[kTokRegChunks];
#pragma unroll
      for (int j = 0; j < kTokRegChunks; ++j) v[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int j = 0; j < kTokRegChunks; ++j) {
        const int c = j0 + j * 64 + l;
        if (c < nchunk) v[j] = xr[c];
      }
#pragma unroll
      for (int j = 0; j < kTokRegChunks; ++j) {
        const int c = j0 + j * 64 + l;
        float m = amax8_of_bf16(v[j], 0.0f);
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        const int x = mx_shared_exp_e4m3(m);
        if (c < nchunk) {
          dst[c] = mx_codes8_of_bf16(v[j], mx_inv_scale(x));
          if ((l & 3) == 0) sc[c / 4] = (uint8_t)(x + 127);
        }
      }
    }
    return;
  }
  const float qmax = (UC == UC_I8) ? 127.0f : 448.0f;
  float m = 0.0f;
  if (nchunk <= 64 * kTokRegChunks) {
    // registers cleared first, then loads that only fill them, then the
    // amax (a cleared chunk adds |0|): every load is issued before the first
    // wait
    uint4 v[kTokRegChunks];
#pragma unroll
    for (int j = 0; j < kTokRegChunks; ++j) v[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < kTokRegChunks; ++j) {
      const int c = j * 64 + l;
      if (c < nchunk) v[j] = xr[c];
    }
#pragma unroll
    for (int j = 0; j < kTokRegChunks; ++j) m = amax8_of_bf16(v[j], m);
    const float s = fmaxf(wave_max(m) / qmax, 1e-8f);
#pragma unroll
    for (int j = 0; j < kTokRegChunks; ++j) {
      const int c = j * 64 + l;
      if (c < nchunk) dst[c] = codes8_of_bf16<UC>(v[j], s);
    }
    if (l == 0) a.x_pool_scale[i] = s;
  } else {
    for (int c = l; c < nchunk; c += 64) m = amax8_of_bf16(xr[c], m);
    const float s = fmaxf(wave_max(m) / qmax, 1e-8f);
    for (int c = l; c < nchunk; c += 64) dst[c] = codes8_of_bf16<UC>(xr[c], s);
    if (l == 0) a.x_pool_scale[i] = s;
  }
}

// Gather of token i by the whole block: reads x_i once, writes its K pool
// rows (A8W8: their codes and scales) (dst: 64 ints of LDS, red: NT/64
// floats of LDS).
template <int UC, int NT>
__device__ __forceinline__ void gather_token(const DispatchArgs& a, int64_t i, int32_t* dst, float* red) {
  constexpr int NW = NT / 64, MAXC = kMaxHidden / 8 / NT;
  const int t = threadIdx.x;
  const int nrows = a.K;
  if (t < nrows) dst[t] = a.route_to_pool[i * a.K + t];
  const int nchunk = (int)(a.H / 8);
  const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + i * a.H);
  if constexpr (is_mx(UC)) {
    // Q_MX per group of 32 (four neighbouring threads' chunks), the codes and
    // E8M0 byte written to each of the token's pool rows
    __syncthreads();
    const int gpr = (int)(a.H / kMxGroup);
    for (int c0 = 0; c0 < nchunk; c0 += NT) {
      const int c = c0 + t;
      const uint4 v = c < nchunk ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
      float m = amax8_of_bf16(v, 0.0f);
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      const int x = mx_shared_exp_e4m3(m);
      if (c < nchunk) {
        const uint2 ov = mx_codes8_of_bf16(v, mx_inv_scale(x));
        for (int k = 0; k < nrows; ++k) {
          const int p = dst[k];
          if (p < 0) continue;
          reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.x_pool) + (int64_t)p * a.H)[c] = ov;
          if ((t & 3) == 0) a.x_pool_mx[(int64_t)p * gpr + c / 4] = (uint8_t)(x + 127);
        }
      }
    }
  } else if constexpr (UC == UC_BF16) {
    __syncthreads();
    for (int c = t; c < nchunk; c += NT) {
      const uint4 v = xr[c];
      for (int k = 0; k < nrows; ++k) {
        const int p = dst[k];
        if (p >= 0) reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.x_pool) + (int64_t)p * a.H)[c] = v;
      }
    }
  } else {
    uint4 v[MAXC];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) v[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int c = t + j * NT;
      if (c < nchunk) v[j] = xr[c];
    }
#pragma unroll
    for (int j = 0; j < MAXC; ++j) m = amax8_of_bf16(v[j], m);
    m = wave_max(m);
    if (lane_id() == 0) red[t / 64] = m;
    __syncthreads();
    float amax = red[0];
    for (int ww = 1; ww < NW; ++ww) amax = fmaxf(amax, red[ww]);
    const float qmax = (UC == UC_I8) ? 127.0f : 448.0f;
    const float s = fmaxf(amax / qmax, 1e-8f);
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int c = t + j * NT;
      if (c < nchunk) {
        const uint2 ov = codes8_of_bf16<UC>(v[j], s);
        for (int k = 0; k < nrows; ++k) {
          const int p = dst[k];
          if (p >= 0) reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.x_pool) + (int64_t)p * a.H)[c] = ov;
        }
      }
    }
    if (t < nrows && dst[t] >= 0) a.x_pool_scale[dst[t]] = s;
  }
  __syncthreads();   // dst / red are reused by the next token
}

}  // namespace mm
