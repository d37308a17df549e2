// NVFP4 codec kernels for gfx950: domain amax, block-scale + element encode
// (row mode and transposed column mode, optionally behind the 16-point random
// Hadamard transform), and decode.
//
// Format and recipe: E2M1 elements with one FP8 (E4M3FN) scale per 16
// elements and an FP32 tensor scale (neurohive.io LongLive-2.0 summary, NVFP4
// paragraph; tailorednewshub.com "LongLive-2.0: Infraestructura paralela NVFP4
// para video largo", section "Entrenamiento NVFP4").  The KV cache uses one
// tensor scale per block of eight frames (hyper.ai LongLive-2.0 summary,
// section "方法"), which these kernels express as row "domains".
//
// All kernels are bound by HBM traffic.  One thread owns one 16-element block
// at a time: it reads 32 B (bf16) or 64 B (float32) with 16-byte vector loads,
// so a wavefront touches 2-4 KiB of contiguous memory per iteration, and
// writes the block's 8 code bytes as one 8-byte store.
#include "device.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMaxGrid = 4096;  // 256 CUs x 16 workgroups

inline uint32_t grid_for(int64_t work_items) {
  int64_t g = (work_items + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  return (uint32_t)(g < kMaxGrid ? g : kMaxGrid);
}

__global__ void zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Workgroup max of non-negative values, folded into *dst with one atomic.
// Non-negative float32 values order like their bit patterns, so an unsigned
// integer max is exact and independent of arrival order.
__device__ __forceinline__ void workgroup_atomic_max(float m, float* dst) {
  __shared__ float part[kThreads / 64];
  m = wave_max(m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = part[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) t = fmaxf(t, part[w]);
    if (t > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(t));
  }
}

// ---------------------------------------------------------------------------
// Step 1: amax of each row domain (gridDim.y = number of domains).
template <int DT, bool RHT>
__global__ __launch_bounds__(kThreads) void amax_rows_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, int64_t rpd,
    float* __restrict__ amax, uint32_t mask) {
  const int64_t r0 = (int64_t)blockIdx.y * rpd;
  const int64_t r1 = rows < r0 + rpd ? rows : r0 + rpd;
  const uint32_t bpr = (uint32_t)(cols / kBlock);
  const uint32_t nblk = (uint32_t)((r1 - r0) * bpr);
  const bool contig = (ld == cols);
  const int64_t base = r0 * ld;
  float m = 0.0f;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < nblk; i += gridDim.x * kThreads) {
    int64_t off;
    if (contig) {
      off = (int64_t)i * kBlock;
    } else {
      const uint32_t r = i / bpr, cb = i - r * bpr;
      off = (int64_t)r * ld + (int64_t)cb * kBlock;
    }
    float v[16];
    load16<DT>(x, base + off, v);
    if constexpr (RHT) rht16(v, mask);
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  workgroup_atomic_max(m, amax + blockIdx.y);
}

// Step 1 for the RHT along axis 0: blocks are 16 consecutive rows of one
// column; lanes take consecutive columns so every load is coalesced.
template <int DT>
__global__ __launch_bounds__(kThreads) void amax_cols_rht_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    float* __restrict__ amax, uint32_t mask) {
  const uint32_t nbc = (uint32_t)(rows / kBlock);
  const uint32_t ncols = (uint32_t)cols;
  const uint32_t nblk = nbc * ncols;
  float m = 0.0f;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < nblk; i += gridDim.x * kThreads) {
    const uint32_t j = i / ncols, c = i - j * ncols;
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = load1<DT>(x, (int64_t)(kBlock * j + t) * ld + c);
    rht16(v, mask);
#pragma unroll
    for (int t = 0; t < 16; ++t) m = fmaxf(m, fabsf(v[t]));
  }
  workgroup_atomic_max(m, amax);
}

// ---------------------------------------------------------------------------
// Steps 2-6, axis 1: block i of the (row-major) output is elements
// [16*(i % bpr), +16) of row i / bpr; its codes are bytes [8i, 8i+8) and its
// scale is byte i of the contiguous outputs.
template <int DT, bool RHT>
__global__ __launch_bounds__(kThreads) void encode_rows_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, int64_t rpd,
    const float* __restrict__ amax, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint32_t mask) {
  const uint32_t bpr = (uint32_t)(cols / kBlock);
  const uint32_t nblk = (uint32_t)(rows * bpr);
  const bool contig = (ld == cols);
  const bool one_domain = (rpd >= rows);
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < nblk; i += gridDim.x * kThreads) {
    uint32_t r = 0, cb = i;
    if (!contig || !one_domain) {
      r = i / bpr;
      cb = i - r * bpr;
    }
    const uint32_t dom = one_domain ? 0u : r / (uint32_t)rpd;
    const float S = amax[dom] / kGlobalMax;
    if (cb == 0 && (one_domain ? i == 0 : (int64_t)r == (int64_t)dom * rpd)) tscale[dom] = S;
    float v[16];
    load16<DT>(x, contig ? (int64_t)i * kBlock : (int64_t)r * ld + (int64_t)cb * kBlock, v);
    if constexpr (RHT) rht16(v, mask);
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
    float rcp;
    const uint32_t sig = block_scale(a, S, rcp);
    const u32x2_t w = encode16(v, rcp);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(codes) + i);
    scales[i] = (uint8_t)sig;
  }
}

// Steps 2-6, axis 0: blocks run down the columns of x [rows][ld]; the output
// is the transpose, [cols][rows/2] codes and [cols][rows/16] scales.
template <int DT, bool RHT>
__global__ __launch_bounds__(kThreads) void encode_cols_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tscale, uint32_t mask) {
  const uint32_t nbc = (uint32_t)(rows / kBlock);
  const uint32_t ncols = (uint32_t)cols;
  const uint32_t nblk = nbc * ncols;
  const float S = amax[0] / kGlobalMax;
  if (blockIdx.x == 0 && threadIdx.x == 0) tscale[0] = S;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < nblk; i += gridDim.x * kThreads) {
    const uint32_t j = i / ncols, c = i - j * ncols;
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = load1<DT>(x, (int64_t)(kBlock * j + t) * ld + c);
    if constexpr (RHT) rht16(v, mask);
    float a = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) a = fmaxf(a, fabsf(v[t]));
    float rcp;
    const uint32_t sig = block_scale(a, S, rcp);
    const u32x2_t w = encode16(v, rcp);
    const int64_t ob = (int64_t)c * nbc + j;  // block index in the transposed output
    reinterpret_cast<u32x2_t*>(codes)[ob] = w;
    scales[ob] = (uint8_t)sig;
  }
}

// ---------------------------------------------------------------------------
// Step 7: x' = f32(e2m1 * s_b) * S, then float32 or bf16 (RNE) out.
template <int OUT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ ts, int64_t rows, int64_t k, int64_t rpd, void* __restrict__ out) {
  const uint32_t bpr = (uint32_t)(k / kBlock);
  const uint32_t nblk = (uint32_t)(rows * bpr);
  const bool one_domain = (rpd >= rows);
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < nblk; i += gridDim.x * kThreads) {
    const uint32_t dom = one_domain ? 0u : (i / bpr) / (uint32_t)rpd;
    const float S = ts[dom];
    const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(codes) + i);
    const float sf = e4m3_to_f32(scales[i]);
    float o[16];
    decode8_f32(w.x, o);
    decode8_f32(w.y, o + 8);
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = (o[e] * sf) * S;
    if constexpr (OUT == 0) {
      float4_t* dst = reinterpret_cast<float4_t*>(out) + (int64_t)i * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_nontemporal_store(float4_t{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]}, dst + q);
    } else {
      uint32_t p[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) p[q] = f32_to_bf16_rne(o[2 * q]) | (f32_to_bf16_rne(o[2 * q + 1]) << 16);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(out) + (int64_t)i * 2;
      __builtin_nontemporal_store(u32x4_t{p[0], p[1], p[2], p[3]}, dst);
      __builtin_nontemporal_store(u32x4_t{p[4], p[5], p[6], p[7]}, dst + 1);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_amax_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                            int64_t rpd, float* amax, bool rht, uint32_t mask, hipStream_t s) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  const int64_t ndom = (rows + rpd - 1) / rpd;
  hipError_t e = launch_zero(amax, ndom, s);
  if (e != hipSuccess) return e;
  const dim3 grid(grid_for(rpd * (cols / kBlock)), (unsigned)ndom);
  if (dt == 0) {
    if (rht) amax_rows_kernel<0, true><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, amax, mask);
    else amax_rows_kernel<0, false><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, amax, mask);
  } else {
    if (rht) amax_rows_kernel<1, true><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, amax, mask);
    else amax_rows_kernel<1, false><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, amax, mask);
  }
  return hipGetLastError();
}

hipError_t launch_amax_cols_rht(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                float* amax, uint32_t mask, hipStream_t s) {
  hipError_t e = launch_zero(amax, 1, s);
  if (e != hipSuccess) return e;
  const unsigned grid = grid_for((rows / kBlock) * cols);
  if (dt == 0) amax_cols_rht_kernel<0><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, amax, mask);
  else amax_cols_rht_kernel<1><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, amax, mask);
  return hipGetLastError();
}

hipError_t launch_encode_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int64_t rpd, const float* amax, QOut out, bool rht, uint32_t mask,
                              hipStream_t s) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  const unsigned grid = grid_for(rows * (cols / kBlock));
#define NVFP4_ENC_ROWS(D, R) \
  encode_rows_kernel<D, R><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, amax, out.codes, out.scales, out.tscale, mask)
  if (dt == 0) { if (rht) NVFP4_ENC_ROWS(0, true); else NVFP4_ENC_ROWS(0, false); }
  else { if (rht) NVFP4_ENC_ROWS(1, true); else NVFP4_ENC_ROWS(1, false); }
#undef NVFP4_ENC_ROWS
  return hipGetLastError();
}

hipError_t launch_encode_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              const float* amax, QOut out, bool rht, uint32_t mask, hipStream_t s) {
  const unsigned grid = grid_for((rows / kBlock) * cols);
#define NVFP4_ENC_COLS(D, R) \
  encode_cols_kernel<D, R><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, amax, out.codes, out.scales, out.tscale, mask)
  if (dt == 0) { if (rht) NVFP4_ENC_COLS(0, true); else NVFP4_ENC_COLS(0, false); }
  else { if (rht) NVFP4_ENC_COLS(1, true); else NVFP4_ENC_COLS(1, false); }
#undef NVFP4_ENC_COLS
  return hipGetLastError();
}

hipError_t launch_dequant(QOut in, int64_t rows, int64_t k, int64_t rpd, void* out, int out_dt,
                          hipStream_t s) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  const unsigned grid = grid_for(rows * (k / kBlock));
  if (out_dt == 0) dequant_kernel<0><<<grid, kThreads, 0, s>>>(in.codes, in.scales, in.tscale, rows, k, rpd, out);
  else dequant_kernel<1><<<grid, kThreads, 0, s>>>(in.codes, in.scales, in.tscale, rows, k, rpd, out);
  return hipGetLastError();
}

}  // namespace nvfp4
