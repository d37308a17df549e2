// Block-scaled NVFP4 x NVFP4 GEMM for gfx950 (W4A4 linear layers:
// tailorednewshub.com "LongLive-2.0: Infraestructura paralela NVFP4 para video
// largo", section "Inferencia W4A4 NVFP4"; format from neurohive.io
// LongLive-2.0 summary, NVFP4 paragraph).
//
//   C[m][n] = epi( S_A * S_B * sum_k P_A[m][k] * P_B[n][k] ),
//   P = e2m1(code) * f32(s_b)  for the 16-element block of k.
//
// Why fp16 MFMA.  The product of an E2M1 value (2 significant bits) and an
// E4M3 scale (4 significant bits) needs up to 6 significant bits, so the
// decoded operand fits neither FP8/FP6/FP4 nor the E8M0-per-32 scaling of the
// gfx950 f8f6f4 MFMAs; it is exact in fp16 (|P| <= 2688, smallest 2^-10).
// Each operand fragment is therefore decoded in registers — E2M1 -> fp16 with
// v_cvt_scalef32_pk_f16_fp4 (scale 1.0), then one packed fp16 multiply by the
// block scale — and fed to v_mfma_f32_32x32x16_f16, which accumulates the
// exact products in float32.  The tensor scales are applied in the epilogue.
//
// Work split.  A workgroup of 4 wavefronts computes a (2*WM) x (2*WN) tile;
// each wavefront a WM x WN sub-tile made of FA x FB 32x32 MFMA fragments.
// K advances 128 elements (8 NVFP4 blocks, 64 bytes of codes per row) at a
// time.  Within a K-tile, lanes 0-31 own k in [0, 64) and lanes 32-63 own
// k in [64, 128) of their row (A) or column (B): a lane loads its 32 code
// bytes and 4 scale bytes with two 16-byte and one 4-byte load per fragment,
// and MFMA step s (0..7) consumes code dword s.  The MFMA reduction runs over
// any k as long as A and B use the same assignment, which they do.
#include "device.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = 128;  // K elements per main-loop iteration

__device__ __forceinline__ half8_t decode8(uint32_t codes, half2_t sig2) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sig2;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sig2;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sig2;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sig2;
  half8_t r;
  r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
  r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  return r;
}

// Four E4M3 bytes -> four fp16 broadcast pairs (exact: every E4M3 value is an
// fp16 value).
__device__ __forceinline__ void scales_to_h2(uint32_t sw, half2_t (&s2)[4]) {
  const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
  const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
  s2[0] = half2_t{lo.x, lo.x};
  s2[1] = half2_t{lo.y, lo.y};
  s2[2] = half2_t{hi.x, hi.x};
  s2[3] = half2_t{hi.y, hi.y};
}

__device__ __forceinline__ float gelu_tanh(float h) {
  const float c = 0.7978845608028654f;  // sqrt(2 / pi)
  return 0.5f * h * (1.0f + tanhf(c * (h + 0.044715f * h * h * h)));
}

template <int FA, int FB>
struct Tile {
  uint4 a[FA][2];
  uint4 b[FB][2];
  uint32_t sa[FA];
  uint32_t sb[FB];
};

template <int FA, int FB>
__device__ __forceinline__ void load_tile_fast(Tile<FA, FB>& t, const uint8_t* const (&pa)[FA],
                                               const uint8_t* const (&psa)[FA],
                                               const uint8_t* const (&pb)[FB],
                                               const uint8_t* const (&psb)[FB], int kt) {
#pragma unroll
  for (int f = 0; f < FA; ++f) {
    const uint4* p = reinterpret_cast<const uint4*>(pa[f] + kt / 2);
    t.a[f][0] = p[0];
    t.a[f][1] = p[1];
    t.sa[f] = *reinterpret_cast<const uint32_t*>(psa[f] + kt / 16);
  }
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    const uint4* p = reinterpret_cast<const uint4*>(pb[f] + kt / 2);
    t.b[f][0] = p[0];
    t.b[f][1] = p[1];
    t.sb[f] = *reinterpret_cast<const uint32_t*>(psb[f] + kt / 16);
  }
}

// Generic K: any K % 16 == 0.  Code dwords and scale bytes past K read as 0
// (decoding to +0), so the partial last K-tile needs no other special case.
template <int FA, int FB>
__device__ __forceinline__ void load_tile_checked(Tile<FA, FB>& t, const uint8_t* const (&pa)[FA],
                                                  const uint8_t* const (&psa)[FA],
                                                  const uint8_t* const (&pb)[FB],
                                                  const uint8_t* const (&psb)[FB], int kt, int K,
                                                  int hh) {
  // `row` arguments already point at this lane's first code byte / scale byte
  // of the tile (k = kt + 64 * hh).
  const int kl = kt + 64 * hh;
  auto ld_codes = [&](const uint8_t* row, uint4 (&dst)[2]) {
    uint32_t w[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k0 = kl + 8 * s;
      w[s] = (k0 < K) ? *reinterpret_cast<const uint32_t*>(row + 4 * s) : 0u;
    }
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  };
  auto ld_scales = [&](const uint8_t* row) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k0 = kl + 16 * q;
      if (k0 < K) v |= (uint32_t)row[q] << (8 * q);
    }
    return v;
  };
#pragma unroll
  for (int f = 0; f < FA; ++f) {
    ld_codes(pa[f] + kt / 2, t.a[f]);
    t.sa[f] = ld_scales(psa[f] + kt / 16);
  }
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    ld_codes(pb[f] + kt / 2, t.b[f]);
    t.sb[f] = ld_scales(psb[f] + kt / 16);
  }
}

__device__ __forceinline__ uint32_t dword_of(const uint4 (&c)[2], int s) {
  const uint4 q = c[s >> 2];
  switch (s & 3) {
    case 0: return q.x;
    case 1: return q.y;
    case 2: return q.z;
    default: return q.w;
  }
}

template <int FA, int FB>
__device__ __forceinline__ void compute_tile(const Tile<FA, FB>& t, float16_t (&acc)[FA][FB]) {
  half2_t sa2[FA][4], sb2[FB][4];
#pragma unroll
  for (int f = 0; f < FA; ++f) scales_to_h2(t.sa[f], sa2[f]);
#pragma unroll
  for (int f = 0; f < FB; ++f) scales_to_h2(t.sb[f], sb2[f]);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    half8_t av[FA], bv[FB];
#pragma unroll
    for (int f = 0; f < FA; ++f) av[f] = decode8(dword_of(t.a[f], s), sa2[f][s >> 1]);
#pragma unroll
    for (int f = 0; f < FB; ++f) bv[f] = decode8(dword_of(t.b[f], s), sb2[f][s >> 1]);
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
      for (int j = 0; j < FB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
  }
}

template <int FA, int FB, int OUT, int EPI, bool FAST>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    void* __restrict__ c, int64_t ldc, int M, int N, int K, float* __restrict__ amax_out) {
  constexpr int WM = 32 * FA, WN = 32 * FB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int m0 = blockIdx.y * (2 * WM) + (wave >> 1) * WM;
  const int n0 = blockIdx.x * (2 * WN) + (wave & 1) * WN;
  const int64_t cpitch = K / 2, spitch = K / 16;

  const uint8_t* pa[FA];
  const uint8_t* psa[FA];
  const uint8_t* pb[FB];
  const uint8_t* psb[FB];
#pragma unroll
  for (int f = 0; f < FA; ++f) {
    const int row = min(m0 + 32 * f + li, M - 1);  // clamp: rows past M are computed, never stored
    pa[f] = ac + (int64_t)row * cpitch + 32 * hh;
    psa[f] = as + (int64_t)row * spitch + 4 * hh;
  }
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    const int col = min(n0 + 32 * f + li, N - 1);
    pb[f] = bc + (int64_t)col * cpitch + 32 * hh;
    psb[f] = bs + (int64_t)col * spitch + 4 * hh;
  }

  float16_t acc[FA][FB];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if constexpr (FAST) {
    // Ping-pong between two register tiles so the loads of the next K-tile
    // are in flight while the current one is decoded and multiplied.
    Tile<FA, FB> t0, t1;
    load_tile_fast(t0, pa, psa, pb, psb, 0);
    int kt = 0;
    for (; kt + 2 * kKT <= K; kt += 2 * kKT) {
      load_tile_fast(t1, pa, psa, pb, psb, kt + kKT);
      compute_tile(t0, acc);
      if (kt + 2 * kKT < K) load_tile_fast(t0, pa, psa, pb, psb, kt + 2 * kKT);
      compute_tile(t1, acc);
    }
    if (kt < K) compute_tile(t0, acc);  // odd number of K-tiles
  } else {
    Tile<FA, FB> cur;
    for (int kt = 0; kt < K; kt += kKT) {
      load_tile_checked(cur, pa, psa, pb, psb, kt, K, hh);
      compute_tile(cur, acc);
    }
  }

  // Epilogue: tensor scales, optional GELU, store, optional amax.
  const float sab = ats[0] * bts[0];
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < FA; ++i) {
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      const int col = n0 + 32 * j + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + 32 * i + (r >> 2) * 8 + hh * 4 + (r & 3);
        float v = acc[i][j][r] * sab;
        if constexpr (EPI == 1) v = gelu_tanh(v);
        if (row < M && col < N) {
          if constexpr (OUT == 0) {
            static_cast<float*>(c)[(int64_t)row * ldc + col] = v;
          } else {
            const uint32_t hb = f32_to_bf16_rne(v);
            static_cast<uint16_t*>(c)[(int64_t)row * ldc + col] = (uint16_t)hb;
            v = bf16_to_f32(hb);
          }
          mx = fmaxf(mx, fabsf(v));
        }
      }
    }
  }
  if (amax_out != nullptr) {
    mx = wave_max(mx);
    if (lane == 0 && mx > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(mx));
  }
}

template <int FA, int FB>
hipError_t launch_tiles(QOut a, QOut b, int m, int n, int k, void* c, int c_dt, int64_t ldc,
                        int epi, float* amax_out, bool fast, hipStream_t s) {
  const dim3 grid((unsigned)((n + 64 * FB - 1) / (64 * FB)), (unsigned)((m + 64 * FA - 1) / (64 * FA)));
#define NVFP4_GEMM_LAUNCH(OUT, EPI, FASTV)                                                  \
  gemm_kernel<FA, FB, OUT, EPI, FASTV><<<grid, kThreads, 0, s>>>(                           \
      a.codes, a.scales, a.tscale, b.codes, b.scales, b.tscale, c, ldc, m, n, k, amax_out)
#define NVFP4_GEMM_EPI(OUT, FASTV)                 \
  if (epi == 1) NVFP4_GEMM_LAUNCH(OUT, 1, FASTV); \
  else NVFP4_GEMM_LAUNCH(OUT, 0, FASTV);
  if (fast) {
    if (c_dt == 0) { NVFP4_GEMM_EPI(0, true) } else { NVFP4_GEMM_EPI(1, true) }
  } else {
    if (c_dt == 0) { NVFP4_GEMM_EPI(0, false) } else { NVFP4_GEMM_EPI(1, false) }
  }
#undef NVFP4_GEMM_EPI
#undef NVFP4_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(QOut a, QOut b, int64_t m, int64_t n, int64_t k, void* c, int c_dt,
                       int64_t ldc, int epilogue, float* amax_out, hipStream_t s) {
  if (amax_out != nullptr) {
    hipError_t e = launch_zero(amax_out, 1, s);
    if (e != hipSuccess) return e;
  }
  const bool fast = (k % kKT == 0) && ((uintptr_t)a.codes % 16 == 0) && ((uintptr_t)b.codes % 16 == 0) &&
                    ((uintptr_t)a.scales % 4 == 0) && ((uintptr_t)b.scales % 4 == 0);
  return launch_tiles<2, 4>(a, b, (int)m, (int)n, (int)k, c, c_dt, ldc, epilogue, amax_out, fast, s);
}

}  // namespace nvfp4
