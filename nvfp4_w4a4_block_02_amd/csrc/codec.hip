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
//     transposed): each thread loads a 4-column chunk from 16 consecutive
//     rows, i.e. four whole blocks, straight into registers; only the
//     encoded output is staged in LDS, so that the transposed code and
//     scale writes stay contiguous.
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
//
// FO6: Four Over Six encoder (tailorednewshub.com, "Inferencia W4A4 NVFP4":
// adaptive scale selection for the KV cache).  Each block is encoded twice,
// with the scale mapping its maximum to 6 and to 4, and the candidate with
// the strictly smaller squared decode error (block_sq_error) is stored;
// ties keep the core recipe.
template <int DT, bool RHT, bool FO6>
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
    uint32_t sig = block_scale(a, S, rcp);
    u32x2_t w = encode16(v, rcp);
    if constexpr (FO6) {
      float rcp4;
      const uint32_t sig4 = block_scale<4>(a, S, rcp4);
      const u32x2_t w4 = encode16(v, rcp4);
      if (block_sq_error(v, w4, sig4, S) < block_sq_error(v, w, sig, S)) {
        sig = sig4;
        w = w4;
      }
    }
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
// [cols][rows/16] scales).  One tile = kColRB row blocks (128 rows) x 128
// columns.  Thread t owns column chunk t % 32 (4 consecutive columns) of row
// block t / 32: it loads the chunk from each of the block's 16 rows (8-byte
// loads for bf16, 16-byte for float32; a wavefront reads two 256- or
// 512-byte row segments per load), so it holds four complete column blocks
// in registers — no transpose through LDS is needed to compute them.  Only
// the encoded output goes through LDS, so that every column's codes (64
// bytes) and scales (8 bytes) of the tile are written contiguously.
// AMAX_ONLY: step 1 of the recipe for the (transformed) tensor, one partial
// maximum per workgroup.
constexpr int kColRB = 8;                       // row blocks per tile
constexpr int kColCH = kThreads / kColRB;       // column chunks per tile
constexpr int kColCPC = 4;                      // columns per chunk
constexpr int kColTC = kColCH * kColCPC;        // tile columns
constexpr int kColTR = kColRB * kBlock;         // tile rows

template <int DT>
struct ColChunk;
template <>
struct ColChunk<1> { u32x2_t v; };   // 4 bf16
template <>
struct ColChunk<0> { float4_t v; };  // 4 float32

template <int DT>
__device__ __forceinline__ float chunk_elem(const ColChunk<DT>& c, int j) {
  if constexpr (DT == 1) {
    const uint32_t w = (j < 2) ? c.v.x : c.v.y;
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    return j == 0 ? c.v.x : j == 1 ? c.v.y : j == 2 ? c.v.z : c.v.w;
  }
}

//
// The output rows may be longer than `rows` (out_k >= rows, a multiple of
// 16): the blocks past `rows` get zero codes and zero scales, which decode to
// 0 and add nothing to a GEMM over the padded reduction dimension.
template <int DT, bool RHT, bool AMAX_ONLY>
__global__ __launch_bounds__(kThreads) void cols_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ parts_in, int nparts_in, float* __restrict__ parts_out,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ tscale,
    uint32_t mask, int64_t out_k) {
  // Output staging, row-block major with one column of padding so that both
  // the per-thread writes and the per-column reads spread over the banks.
  __shared__ u32x2_t ocodes[AMAX_ONLY ? 1 : kColRB][kColTC + 1];
  __shared__ uint8_t oscale[AMAX_ONLY ? 1 : kColRB][kColTC + 4];
  float S = 0.0f;
  if constexpr (!AMAX_ONLY) {
    S = reduce_parts(parts_in, nparts_in) / kGlobalMax;
    if (blockIdx.x == 0 && threadIdx.x == 0) tscale[0] = S;
  }
  const int64_t nbc = out_k / kBlock;              // blocks per output row (>= rows / 16)
  const uint32_t ntr = cdiv(rows, kColTR), ntc = cdiv(cols, kColTC);
  const uint32_t ntiles = ntr * ntc;
  const int t = threadIdx.x, q = t % kColCH, rb = t / kColCH;
  float m = 0.0f;
  for (uint32_t tl = blockIdx.x; tl < ntiles; tl += gridDim.x) {
    const int64_t tr = tl / ntc, tc = tl - tr * ntc;
    const int64_t k0 = tr * kColTR, c0 = tc * kColTC;
    const int nb = (int)((rows - k0) / kBlock < kColRB ? (rows - k0) / kBlock : kColRB);  // row blocks present
    const int64_t r0 = k0 + (int64_t)rb * kBlock;
    const int64_t cq = c0 + (int64_t)q * kColCPC;
    const bool active = rb < nb && cq < cols;
    ColChunk<DT> raw[kBlock];
    if (active) {
      if (cq + kColCPC <= cols) {
#pragma unroll
        for (int i = 0; i < kBlock; ++i) {
          const int64_t off = (r0 + i) * ld + cq;
          if constexpr (DT == 1)
            raw[i].v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(x) + off));
          else
            raw[i].v = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(static_cast<const float*>(x) + off));
        }
      } else {  // right edge: columns past `cols` read as 0 (their blocks are skipped)
#pragma unroll
        for (int i = 0; i < kBlock; ++i) {
          const int64_t off = (r0 + i) * ld + cq;
          float e[kColCPC];
#pragma unroll
          for (int j = 0; j < kColCPC; ++j) e[j] = cq + j < cols ? load1<DT>(x, off + j) : 0.0f;
          if constexpr (DT == 1) {
            raw[i].v = u32x2_t{(__float_as_uint(e[0]) >> 16) | (__float_as_uint(e[1]) & 0xFFFF0000u),
                               (__float_as_uint(e[2]) >> 16) | (__float_as_uint(e[3]) & 0xFFFF0000u)};
          } else {
            raw[i].v = float4_t{e[0], e[1], e[2], e[3]};
          }
        }
      }
    }
    if constexpr (!AMAX_ONLY) __syncthreads();  // the previous tile's output is written out
    if (active) {
#pragma unroll
      for (int j = 0; j < kColCPC; ++j) {
        if (cq + j >= cols) break;
        float v[kBlock];
#pragma unroll
        for (int i = 0; i < kBlock; ++i) v[i] = chunk_elem<DT>(raw[i], j);
        if constexpr (RHT) rht16(v, mask);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < kBlock; ++i) a = fmaxf(a, fabsf(v[i]));
        if constexpr (AMAX_ONLY) {
          m = fmaxf(m, a);
        } else {
          float rcp;
          const uint32_t sig = block_scale(a, S, rcp);
          ocodes[rb][q * kColCPC + j] = encode16(v, rcp);
          oscale[rb][q * kColCPC + j] = (uint8_t)sig;
        }
      }
    }
    if constexpr (!AMAX_ONLY) {
      __syncthreads();
      // Consecutive threads write consecutive blocks of one output row.
#pragma unroll
      for (int h = 0; h < kColTC * kColRB / kThreads; ++h) {
        const int p = t + kThreads * h;
        const int col = p / kColRB, b = p % kColRB;
        if (b < nb && c0 + col < cols) {
          const int64_t ob = (c0 + col) * nbc + k0 / kBlock + b;  // block index in the output
          reinterpret_cast<u32x2_t*>(codes)[ob] = ocodes[b][col];
          scales[ob] = oscale[b][col];
        }
      }
    }
  }
  if constexpr (AMAX_ONLY) {
    m = workgroup_max(m);
    if (threadIdx.x == 0) parts_out[blockIdx.x] = m;
  } else {
    // Zero blocks of the padded reduction dimension.
    const int64_t nb_in = rows / kBlock, npad = nbc - nb_in;
    const int64_t total = npad * cols;
    for (int64_t p = (int64_t)blockIdx.x * kThreads + t; p < total; p += (int64_t)gridDim.x * kThreads) {
      const int64_t orow = p / npad, ob = orow * nbc + nb_in + (p - orow * npad);
      reinterpret_cast<u32x2_t*>(codes)[ob] = u32x2_t{0u, 0u};
      scales[ob] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// Step 7: x' = f32(e2m1 * s_b) * S, then float32 or bf16 (RNE) out.  The
// unit of work is one 16-byte piece of output — 8 bf16 (one code dword) or 4
// float32 (one code half-word) — so that consecutive lanes store consecutive
// 16 bytes (one contiguous 1 KiB per wavefront store) and load consecutive
// code bytes.  Four units are in flight per thread.
template <int OUT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ ts, int64_t rows, int64_t k, int64_t rpd, void* __restrict__ out) {
  constexpr int E = OUT == 1 ? 8 : 4;                  // elements per unit
  const uint64_t nunits = (uint64_t)rows * (uint64_t)k / E;
  const uint64_t upd = (uint64_t)(rpd < rows ? rpd : rows) * (uint64_t)k / E;  // units per domain
  const bool one_domain = (rpd >= rows);
  const bool narrow = nunits <= 0xFFFFFFFFull;  // 32-bit domain division suffices
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  // Tensor scale of unit u's domain.  A thread's units rise monotonically and
  // a domain spans millions of units, so the division runs only when u
  // leaves the cached range.
  uint64_t dlo = 0, dhi = one_domain ? ~0ull : 0;
  float S = one_domain ? ts[0] : 0.0f;
  auto tscale = [&](uint64_t u) {
    if (u >= dhi) {
      const uint64_t d = narrow ? (uint64_t)((uint32_t)u / (uint32_t)upd) : u / upd;
      dlo = d * upd;
      dhi = dlo + upd;
      S = ts[d];
    }
    return S;
  };
  auto load = [&](uint64_t u, uint32_t& w, uint32_t& sb) {
    if constexpr (OUT == 1) w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes) + u);
    else w = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(codes) + u);
    sb = scales[u * E / kBlock];
  };
  // P = e2m1 * f32(s_b) is exact; one rounding for P * S, then RNE to bf16.
  auto store = [&](uint64_t u, uint32_t w, uint32_t sb, float St) {
    const float sf = e4m3_to_f32(sb);
    if constexpr (OUT == 1) {
      float o[8];
      decode8_f32(w, o);
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t v = {(__bf16)((o[2 * q] * sf) * St), (__bf16)((o[2 * q + 1] * sf) * St)};
        p[q] = __builtin_bit_cast(uint32_t, v);
      }
      __builtin_nontemporal_store(u32x4_t{p[0], p[1], p[2], p[3]}, reinterpret_cast<u32x4_t*>(out) + u);
    } else {
      const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
      const float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
      __builtin_nontemporal_store(float4_t{(a.x * sf) * St, (a.y * sf) * St, (b.x * sf) * St, (b.y * sf) * St},
                                  reinterpret_cast<float4_t*>(out) + u);
    }
  };
  uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + 3 * stride < nunits; u += 4 * stride) {
    // the four units' loads first, then their arithmetic and stores
    uint32_t w[4], sb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) load(u + j * stride, w[j], sb[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) store(u + j * stride, w[j], sb[j], tscale(u + j * stride));
  }
  for (; u < nunits; u += stride) {
    uint32_t w, sb;
    load(u, w, sb);
    store(u, w, sb, tscale(u));
  }
}

__global__ __launch_bounds__(kThreads) void reduce_parts_kernel(const float* __restrict__ parts, int nparts,
                                                                 float* __restrict__ amax) {
  const float m = reduce_parts(parts + (int64_t)blockIdx.x * nparts, nparts);
  if (threadIdx.x == 0) amax[blockIdx.x] = m;
}

// Partial-max workgroups for `nblk` 16-element blocks: about 4 blocks per
// thread (enough workgroups to keep HBM busy on small tensors), capped at
// kMaxParts.
inline uint32_t parts_for(int64_t nblk) {
  int64_t p = (nblk + 4 * kThreads - 1) / (4 * kThreads);
  if (p < 1) p = 1;
  return (uint32_t)(p < kMaxParts ? p : kMaxParts);
}

// Encode workgroups per domain: two blocks per thread per iteration, at most
// 256 CUs x 16 workgroups over all domains.
inline uint32_t encode_grid(int64_t nblk, int64_t ndom) {
  int64_t g = (nblk + 2 * kThreads - 1) / (2 * kThreads);
  const int64_t cap = (4096 + ndom - 1) / ndom;
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
  const int64_t tiles = (int64_t)cdiv(rows, kColTR) * cdiv(cols, kColTC);
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
  cols_kernel<D, R, true><<<nparts, kThreads, 0, s>>>(x, rows, cols, ld, nullptr, 0, parts, \
                                                            nullptr, nullptr, nullptr, mask, rows)
  if (dt == 0) { if (rht) NVFP4_CAMAX(0, true); else NVFP4_CAMAX(0, false); }
  else { if (rht) NVFP4_CAMAX(1, true); else NVFP4_CAMAX(1, false); }
#undef NVFP4_CAMAX
  return hipGetLastError();
}

hipError_t launch_encode_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int64_t rpd, const float* parts, uint32_t nparts, QOut out, bool rht,
                              uint32_t mask, hipStream_t s, bool four_over_six) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  const int64_t ndom = (rows + rpd - 1) / rpd;
  const dim3 grid(encode_grid(rpd * (cols / kBlock), ndom), (unsigned)ndom);
#define NVFP4_ENC_ROWS(D, R, F)                                                                       \
  encode_rows_kernel<D, R, F><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, rpd, parts, (int)nparts,  \
                                                        out.codes, out.scales, out.tscale, mask)
  if (four_over_six) {  // no RHT variant: the KV cache is quantized without it
    if (rht) return hipErrorInvalidValue;
    if (dt == 0) NVFP4_ENC_ROWS(0, false, true); else NVFP4_ENC_ROWS(1, false, true);
  } else if (dt == 0) {
    if (rht) NVFP4_ENC_ROWS(0, true, false); else NVFP4_ENC_ROWS(0, false, false);
  } else {
    if (rht) NVFP4_ENC_ROWS(1, true, false); else NVFP4_ENC_ROWS(1, false, false);
  }
#undef NVFP4_ENC_ROWS
  return hipGetLastError();
}

hipError_t launch_encode_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              const float* parts, uint32_t nparts, QOut out, bool rht, uint32_t mask,
                              hipStream_t s, int64_t out_k) {
  if (out_k < rows) out_k = rows;
  // Same grid as the amax pass: at most kMaxParts workgroups, so that a
  // tensor of many tiles gives every workgroup the same number of them.
  const int64_t tiles = (int64_t)cdiv(rows, kColTR) * cdiv(cols, kColTC);
  const unsigned grid = (unsigned)(tiles < (int64_t)kMaxParts ? tiles : kMaxParts);
#define NVFP4_ENC_COLS(D, R)                                                                     \
  cols_kernel<D, R, false><<<grid, kThreads, 0, s>>>(x, rows, cols, ld, parts, (int)nparts, \
                                                          nullptr, out.codes, out.scales,        \
                                                          out.tscale, mask, out_k)
  if (dt == 0) { if (rht) NVFP4_ENC_COLS(0, true); else NVFP4_ENC_COLS(0, false); }
  else { if (rht) NVFP4_ENC_COLS(1, true); else NVFP4_ENC_COLS(1, false); }
#undef NVFP4_ENC_COLS
  return hipGetLastError();
}

hipError_t launch_dequant(QOut in, int64_t rows, int64_t k, int64_t rpd, void* out, int out_dt,
                          hipStream_t s) {
  if (rpd <= 0 || rpd > rows) rpd = rows;
  const int64_t units = rows * k / (out_dt == 0 ? 4 : 8);
  int64_t g = (units + 4 * kThreads - 1) / (4 * kThreads);
  const unsigned grid = (unsigned)(g < 4096 ? (g < 1 ? 1 : g) : 4096);
  if (out_dt == 0) dequant_kernel<0><<<grid, kThreads, 0, s>>>(in.codes, in.scales, in.tscale, rows, k, rpd, out);
  else dequant_kernel<1><<<grid, kThreads, 0, s>>>(in.codes, in.scales, in.tscale, rows, k, rpd, out);
  return hipGetLastError();
}

}  // namespace nvfp4
