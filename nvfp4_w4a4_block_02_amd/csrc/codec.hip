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
// Every kernel here is bound by HBM traffic, so the design rules are:
//   * 16-byte vector loads, coalesced across the wavefront; several blocks in
//     flight per thread;
//   * the domain amax is reduced without same-address atomics: each
//     workgroup of the amax pass writes one partial maximum, and every
//     workgroup of the encode pass reduces its domain's partials (at most
//     kMaxParts floats, an L2 hit) before it starts;
//   * column mode (blocks running down the columns, output stored
//     transposed) goes through an LDS tile so that both the reads and the
//     8-byte code writes stay coalesced.
#include "device.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

__host__ __device__ inline uint32_t cdiv(int64_t a, int64_t b) { return (uint32_t)((a + b - 1) / b); }

__global__ void zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Max over the workgroup; the result is valid in every thread.
__device__ __forceinline__ float workgroup_max(float m) {
  __shared__ float part[kThreads / 64];
  m = wave_max(m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // `part` may still be read by a previous call
  if (lane == 0) part[wave] = m;
  __syncthreads();
  float t = part[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) t = fmaxf(t, part[w]);
  return t;
}

// Domain amax from `nparts` partial maxima (nparts <= kMaxParts).
__device__ __forceinline__ float reduce_parts(const float* __restrict__ parts, int nparts) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += kThreads) m = fmaxf(m, parts[i]);
  return workgroup_max(m);
}

// ---------------------------------------------------------------------------
// Step 1, row layout: partial amax of each row domain.  Grid (P, ndom); the
// workgroup (x, d) writes parts[d * P + x].  Two 16-element blocks per
// iteration keep four 16-byte loads in flight per thread (bf16).
template <int DT, bool RHT>
__global__ __launch_bounds__(kThreads) void amax_rows_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, int64_t rpd,
    float* __restrict__ parts, uint32_t mask) {
  const int64_t r0 = (int64_t)blockIdx.y * rpd;
  const int64_t r1 = rows < r0 + rpd ? rows : r0 + rpd;
  const uint32_t bpr = (uint32_t)(cols / kBlock);
  const uint32_t nblk = (uint32_t)((r1 - r0) * bpr);
  const bool contig = (ld == cols);
  const int64_t base = r0 * ld;
  const uint32_t stride = gridDim.x * kThreads;
  auto offset = [&](uint32_t i) -> int64_t {
    if (contig) return base + (int64_t)i * kBlock;
    const uint32_t r = i / bpr, cb = i - r * bpr;
    return base + (int64_t)r * ld + (int64_t)cb * kBlock;
  };
  float m = 0.0f;
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < nblk; i += 2 * stride) {
    float v[16], w[16];
    load16<DT>(x, offset(i), v);
    load16<DT>(x, offset(i + stride), w);
    if constexpr (RHT) { rht16(v, mask); rht16(w, mask); }
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, fmaxf(fabsf(v[j]), fabsf(w[j])));
  }
  if (i < nblk) {
    float v[16];
    load16<DT>(x, offset(i), v);
    if constexpr (RHT) rht16(v, mask);
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  m = workgroup_max(m);
  if (threadIdx.x == 0) parts[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// ---------------------------------------------------------------------------
// Steps 2-6, row layout (axis 1).  Grid (G, ndom).  Block i of domain d is
// global block gi = d * rpd * bpr + i: elements [16 * (gi % bpr), +16) of row
// gi / bpr; its codes are bytes [8 gi, 8 gi + 8) and its scale is byte gi of
// the contiguous outputs.  `parts` holds `nparts` partial maxima per domain.
template <int DT, bool RHT>
__global__ __launch_bounds__(kThreads) void encode_rows_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, int64_t rpd,
    const float* __restrict__ parts, int nparts, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tscale, uint32_t mask) {
  const uint32_t d = blockIdx.y;
  const float A = reduce_parts(parts + (int64_t)d * nparts, nparts);
  const float S = A / kGlobalMax;
  if (blockIdx.x == 0 && threadIdx.x == 0) tscale[d] = S;
  const int64_t r0 = (int64_t)d * rpd;
  const int64_t r1 = rows < r0 + rpd ? rows : r0 + rpd;
  const uint32_t bpr = (uint32_t)(cols / kBlock);
  const uint32_t nblk = (uint32_t)((r1 - r0) * bpr);
  const int64_t gbase = r0 * bpr;  // first global block of the domain
  const bool contig = (ld == cols);
  const uint32_t stride = gridDim.x * kThreads;
  auto encode_one = [&](uint32_t i, const float (&vin)[16]) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = vin[j];
    if constexpr (RHT) rht16(v, mask);
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
    float rcp;
    const uint32_t sig = block_scale(a, S, rcp);
    const u32x2_t w = encode16(v, rcp);
    const int64_t gi = gbase + i;
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(codes) + gi);
    scales[gi] = (uint8_t)sig;
  };
  auto offset = [&](uint32_t i) -> int64_t {
    if (contig) return r0 * ld + (int64_t)i * kBlock;
    const uint32_t r = i / bpr, cb = i - r * bpr;
    return (r0 + r) * ld + (int64_t)cb * kBlock;
  };
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < nblk; i += 2 * stride) {
    float v[16], w[16];
    load16<DT>(x, offset(i), v);
    load16<DT>(x, offset(i + stride), w);
    encode_one(i, v);
    encode_one(i + stride, w);
  }
  if (i < nblk) {
    float v[16];
    load16<DT>(x, offset(i), v);
    encode_one(i, v);
  }
}

// ---------------------------------------------------------------------------
// Column layout (axis 0): x is [rows][ld], 16-element blocks run down the
// columns and the NVFP4 output is the transpose ([cols][rows/2] codes,
// [cols][rows/16] scales).  One tile = 128 rows (8 blocks) x 64 columns:
//   1. coalesced 16-byte loads of the tile into LDS (as float32);
//   2. thread t transforms/encodes blocks (column t % 64, block t / 64 and
//      t / 64 + 4), reading a column of LDS (conflict-free: consecutive lanes,
//      consecutive words);
//   3. the 8-byte codes and the scale bytes are staged in LDS and written so
//      that consecutive lanes fill consecutive bytes of an output row.
// AMAX_ONLY: step 1 of the recipe for the transformed tensor (no output but
// one partial max per workgroup).
constexpr int kTR = 128;  // tile rows (reduction dim)
constexpr int kTC = 64;   // tile columns

template <int DT, bool RHT, bool AMAX_ONLY>
__global__ __launch_bounds__(kThreads) void cols_tile_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ parts_in, int nparts_in, float* __restrict__ parts_out,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ tscale,
    uint32_t mask) {
  __shared__ float tile[kTR][kTC + 1];
  __shared__ u32x2_t ocodes[kTC][kTR / 16];
  __shared__ uint8_t oscale[kTC][kTR / 16];
  float S = 0.0f;
  if constexpr (!AMAX_ONLY) {
    S = reduce_parts(parts_in, nparts_in) / kGlobalMax;
    if (blockIdx.x == 0 && threadIdx.x == 0) tscale[0] = S;
  }
  const int64_t nbc = rows / kBlock;               // blocks per column = per output row
  const uint32_t ntr = cdiv(rows, kTR), ntc = cdiv(cols, kTC);
  const uint32_t ntiles = ntr * ntc;
  const int t = threadIdx.x;
  constexpr int kEpc = 16 / (DT == 0 ? 4 : 2);     // elements per 16-byte chunk
  constexpr int kCpr = kTC / kEpc;                 // chunks per tile row
  const bool vec_ok = (cols % kEpc) == 0;          // every chunk fully inside or outside
  float m = 0.0f;
  for (uint32_t tl = blockIdx.x; tl < ntiles; tl += gridDim.x) {
    const int64_t tr = tl / ntc, tc = tl - tr * ntc;
    const int64_t k0 = tr * kTR, c0 = tc * kTC;
    const int nrow = (int)(rows - k0 < kTR ? rows - k0 : kTR);  // multiple of 16
    __syncthreads();  // previous tile's LDS reads are done
    for (int q = t; q < kTR * kCpr; q += kThreads) {
      const int r = q / kCpr, ch = q - r * kCpr;
      const int64_t c = c0 + (int64_t)ch * kEpc;
      float v[kEpc];
      if (r < nrow && c + kEpc <= cols && vec_ok) {
        const int64_t off = (k0 + r) * ld + c;
        if constexpr (DT == 0) {
          const float4_t u = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(static_cast<const float*>(x) + off));
          v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
        } else {
          const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(x) + off));
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kEpc; ++j)
          v[j] = (r < nrow && c + j < cols) ? load1<DT>(x, (k0 + r) * ld + c + j) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < kEpc; ++j) tile[r][ch * kEpc + j] = v[j];
    }
    __syncthreads();
    const int cc = t & (kTC - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jb = (t >> 6) + 4 * h;  // block within the tile
      if (16 * jb >= nrow || c0 + cc >= cols) continue;
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = tile[16 * jb + i][cc];
      if constexpr (RHT) rht16(v, mask);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
      if constexpr (AMAX_ONLY) {
        m = fmaxf(m, a);
      } else {
        float rcp;
        const uint32_t sig = block_scale(a, S, rcp);
        ocodes[cc][jb] = encode16(v, rcp);
        oscale[cc][jb] = (uint8_t)sig;
      }
    }
    if constexpr (!AMAX_ONLY) {
      __syncthreads();
      const int nb = nrow / 16;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = t + kThreads * h;  // (output row, block) pair
        const int orow = p >> 3, b = p & 7;
        if (b < nb && c0 + orow < cols) {
          const int64_t ob = (c0 + orow) * nbc + k0 / 16 + b;  // block index in the output
          reinterpret_cast<u32x2_t*>(codes)[ob] = ocodes[orow][b];
          scales[ob] = oscale[orow][b];
        }
      }
    }
  }
  if constexpr (AMAX_ONLY) {
    m = workgroup_max(m);
    if (threadIdx.x == 0) parts_out[blockIdx.x] = m;
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

__global__ __launch_bounds__(kThreads) void reduce_parts_kernel(const float* __restrict__ parts, int nparts,
                                                                 float* __restrict__ amax) {
  const float m = reduce_parts(parts + (int64_t)blockIdx.x * nparts, nparts);
  if (threadIdx.x == 0) amax[blockIdx.x] = m;
}

// Partial-max workgroups for `nblk` 16-element blocks: about 8 blocks per
// thread, capped at kMaxParts.
inline uint32_t parts_for(int64_t nblk) {
  int64_t p = (nblk + 8 * kThreads - 1) / (8 * kThreads);
  if (p < 1) p = 1;
  return (uint32_t)(p < kMaxParts ? p : kMaxParts);
}

// Encode workgroups per domain: two blocks per thread per iteration, at most
// 256 CUs x 8 workgroups over all domains.
inline uint32_t encode_grid(int64_t nblk, int64_t ndom) {
  int64_t g = (nblk + 2 * kThreads - 1) / (2 * kThreads);
  const int64_t cap = (2048 + ndom - 1) / ndom;
  if (g > cap) g = cap;
  return (uint32_t)(g < 1 ? 1 : g);
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_reduce_parts(const float* parts, uint32_t nparts, int64_t ndom, float* amax, hipStream_t s) {
  reduce_parts_kernel<<<(unsigned)ndom, kThreads, 0, s>>>(parts, (int)nparts, amax);
  return hipGetLastError();
}

uint32_t amax_parts_rows(int64_t rows, int64_t cols, int64_t rpd) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  return parts_for(rpd * (cols / kBlock));
}

uint32_t amax_parts_cols(int64_t rows, int64_t cols) {
  const int64_t tiles = (int64_t)cdiv(rows, kTR) * cdiv(cols, kTC);
  return (uint32_t)(tiles < kMaxParts ? (tiles < 1 ? 1 : tiles) : kMaxParts);
}

hipError_t launch_amax_parts_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  int64_t rpd, float* parts, uint32_t nparts, bool rht, uint32_t mask,
                                  hipStream_t s) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  const dim3 grid(nparts, (unsigned)((rows + rpd - 1) / rpd));
#define NVFP4_AMAX(D, R) amax_rows_kernel<D, R><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, parts, mask)
  if (dt == 0) { if (rht) NVFP4_AMAX(0, true); else NVFP4_AMAX(0, false); }
  else { if (rht) NVFP4_AMAX(1, true); else NVFP4_AMAX(1, false); }
#undef NVFP4_AMAX
  return hipGetLastError();
}

hipError_t launch_amax_parts_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  float* parts, uint32_t nparts, bool rht, uint32_t mask, hipStream_t s) {
#define NVFP4_CAMAX(D, R)                                                                        \
  cols_tile_kernel<D, R, true><<<nparts, kThreads, 0, s>>>(x, rows, cols, ld, nullptr, 0, parts, \
                                                            nullptr, nullptr, nullptr, mask)
  if (dt == 0) { if (rht) NVFP4_CAMAX(0, true); else NVFP4_CAMAX(0, false); }
  else { if (rht) NVFP4_CAMAX(1, true); else NVFP4_CAMAX(1, false); }
#undef NVFP4_CAMAX
  return hipGetLastError();
}

hipError_t launch_encode_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int64_t rpd, const float* parts, uint32_t nparts, QOut out, bool rht,
                              uint32_t mask, hipStream_t s) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  const int64_t ndom = (rows + rpd - 1) / rpd;
  const dim3 grid(encode_grid(rpd * (cols / kBlock), ndom), (unsigned)ndom);
#define NVFP4_ENC_ROWS(D, R)                                                                       \
  encode_rows_kernel<D, R><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, parts, (int)nparts,  \
                                                     out.codes, out.scales, out.tscale, mask)
  if (dt == 0) { if (rht) NVFP4_ENC_ROWS(0, true); else NVFP4_ENC_ROWS(0, false); }
  else { if (rht) NVFP4_ENC_ROWS(1, true); else NVFP4_ENC_ROWS(1, false); }
#undef NVFP4_ENC_ROWS
  return hipGetLastError();
}

hipError_t launch_encode_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              const float* parts, uint32_t nparts, QOut out, bool rht, uint32_t mask,
                              hipStream_t s) {
  const int64_t tiles = (int64_t)cdiv(rows, kTR) * cdiv(cols, kTC);
  const unsigned grid = (unsigned)(tiles < 2048 ? tiles : 2048);
#define NVFP4_ENC_COLS(D, R)                                                                     \
  cols_tile_kernel<D, R, false><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, parts, (int)nparts, \
                                                          nullptr, out.codes, out.scales,        \
                                                          out.tscale, mask)
  if (dt == 0) { if (rht) NVFP4_ENC_COLS(0, true); else NVFP4_ENC_COLS(0, false); }
  else { if (rht) NVFP4_ENC_COLS(1, true); else NVFP4_ENC_COLS(1, false); }
#undef NVFP4_ENC_COLS
  return hipGetLastError();
}

hipError_t launch_dequant(QOut in, int64_t rows, int64_t k, int64_t rpd, void* out, int out_dt,
                          hipStream_t s) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  int64_t g = (rows * (k / kBlock) + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(g < 4096 ? (g < 1 ? 1 : g) : 4096);
  if (out_dt == 0) dequant_kernel<0><<<grid, kThreads, 0, s>>>(in.codes, in.scales, in.tscale, rows, k, rpd, out);
  else dequant_kernel<1><<<grid, kThreads, 0, s>>>(in.codes, in.scales, in.tscale, rows, k, rpd, out);
  return hipGetLastError();
}

}  // namespace nvfp4
