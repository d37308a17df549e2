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
// Work split.  A workgroup of 4 wavefronts (2 x 2) computes a
// (64 FA) x (64 FB) tile; each wavefront a (32 FA) x (32 FB) sub-tile made of
// FA x FB 32x32 MFMA fragments.  K advances 128 elements (8 NVFP4 blocks, 64
// code bytes per row) per tile.  Within a K-tile, lanes 0-31 own k in
// [0, 64) and lanes 32-63 own k in [64, 128) of their row (A) or column (B);
// MFMA step s (0..7) consumes code dword s of the lane, so each step covers
// k = {8s..8s+7} and {64+8s..64+8s+7}.  The MFMA reduction runs over any k as
// long as A and B use the same assignment, which they do.
//
// Main kernel (K >= 512, K % 256 == 0): a 3-stage LDS ring of codes and a
// 2-slot ring of scales (four K-tiles per slot) fed by direct global->LDS
// loads (global_load_lds_dwordx4).  Every K-tile is read
// from memory once per workgroup; its LDS image is laid out in the order the
// consuming lanes read it (fragment, 16-byte half, lane), so the ds_reads are
// contiguous and conflict-free.  One barrier per K-tile; the loads of tile
// t+3 are spread over the MFMA steps of tile t, and the decode of step s+1 is
// interleaved with the MFMAs of step s.  bf16 outputs of whole wavefront
// sub-tiles leave through the (then free) LDS ring, transposed into rows, as
// 16-byte stores; the tensor scales are read during the first tile's wait.
//
// Fallback kernel (any other K % 16 == 0): the same fragments loaded straight
// into registers with bounds checks; code bytes past K read as 0.
#include <cmath>
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace nvfp4 {
namespace {

typedef __attribute__((address_space(1))) const void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

constexpr int kKT = 128;    // K elements per tile
constexpr int kStages = 3;  // LDS ring depth
constexpr int kOutRegion = 20736;  // LDS bytes per wavefront for the staged bf16 epilogue

// The four converts come first and the multiplies after them: a multiply that
// directly follows the convert it reads stalls the wavefront (a packed fp16
// multiply issued right behind its convert ran ~20% slower in isolation).
__device__ __forceinline__ half8_t decode8(uint32_t codes, half2_t sig2) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  p0 = p0 * sig2;
  p1 = p1 * sig2;
  p2 = p2 * sig2;
  p3 = p3 * sig2;
  half8_t r;
  r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
  r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  return r;
}

// Byte q (0..3) of four E4M3 scale bytes as an fp16 broadcast pair (exact:
// every E4M3 value is an fp16 value).
__device__ __forceinline__ half2_t scale_h2(uint32_t sw, int q) {
  const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
  const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
  const _Float16 v = q == 0 ? lo.x : q == 1 ? lo.y : q == 2 ? hi.x : hi.y;
  return half2_t{v, v};
}

// GELU, tanh form: g(h) = 0.5 h (1 + tanh(u)), u = sqrt(2/pi) (h + 0.044715 h^3).
// Evaluated through the identity 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)) as
// g = h / (1 + 2^(-2u log2 e)) with the hardware exp2 and reciprocal: a few
// float32 ulp, no cancellation in either tail (g -> h for large h, g -> -0
// for large negative h, where 2^(...) overflows to +inf and 1/inf = 0).
__device__ __forceinline__ float gelu_tanh(float h) {
  const float k = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float w = k * (h + 0.044715f * (h * h * h));
  return h * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(w));
}

// One K-tile of this lane's fragments: 32 code bytes and 4 scale bytes each.
template <int FA, int FB>
struct Frags {
  u32x4_t a[FA][2];
  u32x4_t b[FB][2];
  uint32_t sa[FA];
  uint32_t sb[FB];
};

template <int FA, int FB>
__device__ __forceinline__ void decode_step(const Frags<FA, FB>& t, int s, half8_t (&A)[FA], half8_t (&B)[FB]) {
#pragma unroll
  for (int f = 0; f < FA; ++f) A[f] = decode8(t.a[f][s >> 2][s & 3], scale_h2(t.sa[f], s >> 1));
#pragma unroll
  for (int f = 0; f < FB; ++f) B[f] = decode8(t.b[f][s >> 2][s & 3], scale_h2(t.sb[f], s >> 1));
}

template <int FA, int FB>
__device__ __forceinline__ void mfma_step(const half8_t (&A)[FA], const half8_t (&B)[FB], float16_t (&acc)[FA][FB]) {
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], acc[i][j], 0, 0, 0);
}

// Ask the scheduler to alternate one MFMA with the decode VALU work of the
// next step.
template <int FA, int FB>
__device__ __forceinline__ void interleave_hint() {
  constexpr int nv = (8 * (FA + FB) + FA * FB - 1) / (FA * FB);
#pragma unroll
  for (int i = 0; i < FA * FB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
  }
}

// All 8 MFMA steps of one K-tile; the decode of step s+1 overlaps step s.
template <int FA, int FB>
__device__ __forceinline__ void compute_tile(const Frags<FA, FB>& t, float16_t (&acc)[FA][FB]) {
  half8_t A0[FA], B0[FB], A1[FA], B1[FB];
  decode_step(t, 0, A0, B0);
#pragma unroll
  for (int s = 0; s < 8; s += 2) {
    mfma_step(A0, B0, acc);
    decode_step(t, s + 1, A1, B1);
    interleave_hint<FA, FB>();
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(A1, B1, acc);
    if (s + 2 < 8) decode_step(t, s + 2, A0, B0);
    interleave_hint<FA, FB>();
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue: tensor scales, optional GELU, store, optional amax of the stored
// values.  MFMA 32x32 output layout: lane l, accumulator r holds row
// (r / 4) * 8 + (l / 32) * 4 + r % 4, column l % 32 of the fragment.
//
// A sub-tile wholly inside C takes a branch-free path: one base address per
// lane, the row offsets (uniform multiples of ldc) added per accumulator row
// and the column fragments as immediate store offsets; edge sub-tiles check
// every element.  Both store the same values.
// This lane's index in its wavefront from mbcnt, for epilogues that should
// not keep the thread id in a register through the K loop.
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// l: this lane's index in its wavefront (li = l % 32, hh = l / 32).
template <int FA, int FB, int OUT, int EPI, bool WHOLE = false>
__device__ __forceinline__ void store_tile(const float16_t (&acc)[FA][FB], float sab, int m0, int n0, int l, int li,
                                           int hh, int M, int N, void* __restrict__ c, int64_t ldc,
                                           float* __restrict__ amax_out) {
  using T = typename std::conditional<OUT == 0, float, uint16_t>::type;
  float mx = 0.0f;
  if (WHOLE || (m0 + 32 * FA <= M && n0 + 32 * FB <= N)) {
    T* const base = static_cast<T*>(c) + (int64_t)(m0 + hh * 4) * ldc + n0 + li;
#pragma unroll
    for (int i = 0; i < FA; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        T* const p = base + (int64_t)(32 * i + (r >> 2) * 8 + (r & 3)) * ldc;
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          float v = acc[i][j][r] * sab;
          if constexpr (EPI == 1) v = gelu_tanh(v);
          if constexpr (OUT == 0) {
            p[32 * j] = v;
          } else {
            const uint32_t hb = f32_to_bf16_rne(v);
            p[32 * j] = (uint16_t)hb;
            v = bf16_to_f32(hb);
          }
          mx = fmaxf(mx, fabsf(v));
        }
      }
    }
    if (amax_out != nullptr) {
      mx = wave_max(mx);
      if (l == 0 && mx > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(mx));
    }
    return;
  }
  if constexpr (WHOLE) return;
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
    if (l == 0 && mx > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(mx));
  }
}


// Workgroup -> output tile.  Workgroups are dealt round-robin to the 8 XCDs,
// each with its own L2.  Tiles are put in "band" order (bands of `band` tile
// columns, row-major inside a band) and every XCD gets one contiguous run of
// that order, so the ~32 tiles an XCD runs at once form a compact block of
// A rows and B columns that its L2 can hold; `band` is chosen on the host to
// make that block roughly square in bytes.  A bijection for any tile count.
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int band, int& tm, int& tn) {
  const int ntiles = tiles_m * tiles_n;
  const int id = blockIdx.x;
  const int x = id % 8, local = id / 8, q = ntiles / 8, r = ntiles % 8;
  const int t = x * q + (x < r ? x : r) + local;  // position in band order
  const int full = tiles_n / band;                 // bands of full width
  const int per_band = band * tiles_m;
  const int b = t / per_band;
  int n0, w, loc;
  if (b < full) {
    n0 = b * band;
    w = band;
    loc = t - b * per_band;
  } else {  // the last, narrower band
    n0 = full * band;
    w = tiles_n - n0;
    loc = t - full * per_band;
  }
  tm = loc / w;
  tn = n0 + (loc - tm * w);
}

// Fragments of one K-tile straight from global memory, bounds-checked along
// K.  This lane owns k in [kt + 64 hh, kt + 64 hh + 64) of its rows: code
// dword s covers k0 = kt + 64 hh + 8 s (valid iff k0 < K, since K % 16 == 0)
// and scale byte q covers k0 = kt + 64 hh + 16 q; past K both read as 0, and
// a zero code decodes to 0.
template <int FA, int FB>
__device__ __forceinline__ void load_frags_checked(Frags<FA, FB>& fr, const uint8_t* const (&pa)[FA],
                                                   const uint8_t* const (&psa)[FA], const uint8_t* const (&pb)[FB],
                                                   const uint8_t* const (&psb)[FB], int kt, int hh, int K) {
  const int kl = kt + 64 * hh;
  auto ld_codes = [&](const uint8_t* row, u32x4_t (&dst)[2]) {
    uint32_t w[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) w[s] = (kl + 8 * s < K) ? *reinterpret_cast<const uint32_t*>(row + 4 * s) : 0u;
    dst[0] = u32x4_t{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4_t{w[4], w[5], w[6], w[7]};
  };
  auto ld_scales = [&](const uint8_t* row) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (kl + 16 * q < K) v |= (uint32_t)row[q] << (8 * q);
    return v;
  };
#pragma unroll
  for (int f = 0; f < FA; ++f) {
    ld_codes(pa[f] + kt / 2, fr.a[f]);
    fr.sa[f] = ld_scales(psa[f] + kt / 16);
  }
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    ld_codes(pb[f] + kt / 2, fr.b[f]);
    fr.sb[f] = ld_scales(psb[f] + kt / 16);
  }
}

// ---------------------------------------------------------------------------
// Main kernel: K >= 512, K % 256 == 0 (code and scale rows 16-byte aligned,
// an even number of K-tiles); every K-tile goes through the LDS pipeline.
//
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14): wait until at most N vector-memory
// operations of this wave are outstanding / until all LDS reads are done.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Per MFMA of one step: one MFMA, its share of the next step's decode, and
// (for the first NVM MFMAs) one of the global->LDS loads issued in the step.
// Each step is closed by sched_barrier(0): the interleave is solved per step,
// which keeps the schedule and makes compilation take seconds instead of the
// many minutes the solver needs for a whole unrolled tile.
template <int FA, int FB, int NVM>
__device__ __forceinline__ void step_schedule() {
  constexpr int nv = (8 * (FA + FB) + FA * FB - 1) / (FA * FB);
#pragma unroll
  for (int i = 0; i < FA * FB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);  // VALU
    if (i < NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
  }
}

// Read this wave's fragments of one K-tile from its LDS stage (codes) and
// from the scale ring: `ss` points at the tile's scale bytes inside its
// 4-tile group (fragment j's 32 rows at 1024 j, 32 bytes per row, 8 per
// tile), `so` is this lane's row and k-half offset there.
template <int FA, int FB>
__device__ __forceinline__ void read_stage(Frags<FA, FB>& fr, const uint8_t* st, const uint8_t* ss, int so, int wy,
                                           int wx, int l, int off_b) {
  constexpr int NFA = 2 * FA;
#pragma unroll
  for (int f = 0; f < FA; ++f) {
    const int fj = wy * FA + f;
    fr.a[f][0] = *reinterpret_cast<const u32x4_t*>(st + (2 * fj) * 1024 + 16 * l);
    fr.a[f][1] = *reinterpret_cast<const u32x4_t*>(st + (2 * fj + 1) * 1024 + 16 * l);
    fr.sa[f] = *reinterpret_cast<const uint32_t*>(ss + fj * 1024 + so);
  }
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    const int fj = wx * FB + f;
    fr.b[f][0] = *reinterpret_cast<const u32x4_t*>(st + off_b + (2 * fj) * 1024 + 16 * l);
    fr.b[f][1] = *reinterpret_cast<const u32x4_t*>(st + off_b + (2 * fj + 1) * 1024 + 16 * l);
    fr.sb[f] = *reinterpret_cast<const uint32_t*>(ss + (NFA + fj) * 1024 + so);
  }
}

// bf16 epilogue through LDS for a wavefront's whole (32 FA) x (32 FB)
// sub-tile inside C: the accumulators are scaled (optionally GELU'd), rounded
// to bf16 and written to the wavefront's LDS region in row-major order, then
// read back 16 bytes per lane and stored row-contiguously, so that every
// global store writes whole 16-byte pieces of rows (one instruction covers
// 64 x 16 bytes) instead of one bf16 per lane.  IC fragment rows per pass
// keep the region within kOutRegion bytes.  The row pitch is padded by 16
// bytes so that the two row groups a 2-byte LDS store touches (rows r and
// r + 4) fall in different banks.
template <int FA, int FB, int EPI, bool CHECKED = false>
__device__ __forceinline__ void store_tile_staged(const float16_t (&acc)[FA][FB], float sab, int m0, int n0, int l,
                                                  int li, int hh, uint8_t* lds, uint16_t* __restrict__ c,
                                                  int64_t ldc, float* __restrict__ amax_out, int M = 0, int N = 0) {
  constexpr int COLS = 32 * FB, PITCH = 2 * COLS + 16;
  constexpr int IC = (FA * 32 * PITCH <= kOutRegion) ? FA : 2;  // fragment rows per pass
  static_assert(FA % IC == 0 && IC * 32 * PITCH <= kOutRegion, "staging region");
  constexpr int LPR = COLS / 8;   // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;   // rows per read instruction
  static_assert(64 % LPR == 0 && (IC * 32) % RPI == 0, "whole rows per read instruction");
  float mx = 0.0f;
#pragma unroll
  for (int i0 = 0; i0 < FA; i0 += IC) {
#pragma unroll
    for (int i = i0; i < i0 + IC; ++i) {
#pragma unroll
      for (int j = 0; j < FB; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * (i - i0) + (r >> 2) * 8 + hh * 4 + (r & 3);
          float v = acc[i][j][r] * sab;
          if constexpr (EPI == 1) v = gelu_tanh(v);
          const uint32_t hb = f32_to_bf16_rne(v);
          mx = fmaxf(mx, fabsf(bf16_to_f32(hb)));
          *reinterpret_cast<uint16_t*>(lds + row * PITCH + 2 * (32 * j + li)) = (uint16_t)hb;
        }
      }
    }
    wait_lgkmcnt0();
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < IC * 32 / RPI; ++it) {
      const int row = it * RPI + l / LPR, seg = l % LPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + row * PITCH + 16 * seg);
      if (!CHECKED || (m0 + 32 * i0 + row < M && n0 + 8 * seg < N))
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(c + (int64_t)(m0 + 32 * i0 + row) * ldc + n0 + 8 * seg));
    }
    if (i0 + IC < FA) {
      wait_lgkmcnt0();
      __builtin_amdgcn_wave_barrier();
    }
  }
  if (amax_out != nullptr) {
    mx = wave_max(mx);
    if (l == 0 && mx > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(mx));
  }
}


// The code ring holds three K-tiles.  Every tile body issues CPW code loads
// (this wave's share of one future tile); near the end of K they are clamped
// to the last tile and land in a stage that is never read again.  Scales
// travel separately, four K-tiles at a time: one 16-byte load per lane
// brings 32 bytes of scales for each of a fragment's 32 rows (1 KiB per
// fragment), into a double-buffered scale ring.  Four-byte scale loads per
// tile cost ~18% of the attention-projection GEMM (timing variants without
// them, or with them all on one cache line); this takes four times fewer
// scale load instructions and half the cache-line accesses.  Scale group g
// (tiles 4g .. 4g+3, shifted back to end at the last tile when K / 128 is
// not a multiple of 4) is issued in body 4g - 3 and first read at the start
// of body 4g - 1, the same two-body lead as the codes.  Tile body t:
//   1. wait for this wave's loads of tile t+1 (and of scale group (t+1)/4)
//      and for its LDS reads of tile t (already in registers), then one
//      barrier: tile t+1 is complete in LDS and every wave is done reading
//      stage t % 3;
//   2. issue the LDS reads of tile t+1 (consumed at the end of the body), and
//      when t % 4 == 1 the loads of scale group (t+3)/4;
//   3. 8 MFMA steps on tile t, each overlapped with the decode of the next
//      step and the code loads of tile t+3 into stage t % 3.
template <int FA, int FB, int OUT, int EPI, int EDGE>
__global__ __launch_bounds__(256) void gemm_lds_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    void* __restrict__ c, int64_t ldc, int M, int N, int K, float* __restrict__ amax_out, int band) {
  constexpr int NFA = 2 * FA, NFB = 2 * FB;                  // fragments per workgroup
  constexpr int NFR = NFA + NFB;
  constexpr int OFF_B = NFA * 2048;
  constexpr int STAGE = OFF_B + NFB * 2048;                  // codes of one K-tile
  constexpr int SGROUP = NFR * 1024;                          // scales of one 4-tile group
  constexpr int SRING = kStages * STAGE;                      // offset of the scale ring
  static_assert((FA + FB) % 2 == 0, "load slots assume FA + FB even");
  constexpr int CPW = FA + FB;        // 16-byte code loads per wave per tile
  constexpr int SPW = NFR / 4;        // 16-byte scale loads per wave per 4-tile group
  static_assert(NFR % 4 == 0, "scale loads are dealt evenly over the 4 waves");
  constexpr int LPS = (CPW + 7) / 8;  // code loads issued per MFMA step (8 steps per tile)
  static_assert(3 * CPW + SPW < 64, "three tiles of loads must fit the vmcnt counter");
  constexpr bool kStaged = OUT == 1 && (FB == 2 || FB == 4);  // bf16 epilogue through LDS
  constexpr int SMEM = kStaged && 4 * kOutRegion > SRING + 2 * SGROUP ? 4 * kOutRegion : SRING + 2 * SGROUP;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS destinations in SGPRs
  const int li = l & 31, hh = l >> 5;
  const int tiles_n = (N + 64 * FB - 1) / (64 * FB);
  const int tiles_m = (M + 64 * FA - 1) / (64 * FA);
  int tm, tn;
  tile_of(tiles_m, tiles_n, band, tm, tn);
  const int mwg = tm * 64 * FA, nwg = tn * 64 * FB;
  const int64_t cpitch = K / 2, spitch = K / 16;

  // Load slots: code loads (2 per fragment per tile) and scale loads (1 per
  // fragment per 4-tile group) dealt round-robin over the 4 waves.  Lane l of
  // a code load fetches the 16-byte half q of row (32 f + l % 32), k-half
  // l / 32; lane l of a scale load fetches bytes 16 (l % 2) .. 16 (l % 2) + 15
  // of the group's 32 scale bytes of row (32 f + l / 2); rows past M / N are
  // clamped (computed, never stored).  The address of a load is a uniform
  // base (the operand, advanced per K-tile) plus a 32-bit lane offset (the
  // host takes this path only for operands below 2^31 bytes), so it goes out
  // with a scalar base and the LDS destination is uniform too: no per-load
  // 64-bit vector arithmetic.
  const uint8_t* base[CPW + SPW];
  uint32_t off[CPW + SPW];
  int dst[CPW + SPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int i = wave + 4 * j;  // 0 .. 2 (NFA + NFB) - 1
    const bool isA = i < 2 * NFA;
    const int ii = isA ? i : i - 2 * NFA, f = ii >> 1, q = ii & 1;
    const int row = isA ? min(mwg + 32 * f + li, M - 1) : min(nwg + 32 * f + li, N - 1);
    base[j] = isA ? ac : bc;
    off[j] = (uint32_t)row * (uint32_t)cpitch + 32 * hh + 16 * q;
    dst[j] = (isA ? 0 : OFF_B) + (2 * f + q) * 1024;
  }
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int i = wave + 4 * j;  // 0 .. NFR - 1
    const bool isA = i < NFA;
    const int f = isA ? i : i - NFA;
    const int row = isA ? min(mwg + 32 * f + (l >> 1), M - 1) : min(nwg + 32 * f + (l >> 1), N - 1);
    base[CPW + j] = isA ? as : bs;
    off[CPW + j] = (uint32_t)row * (uint32_t)spitch + 16 * (l & 1);
    dst[CPW + j] = i * 1024;
  }
  const int nt = K / kKT;       // >= 4 on this path
  const int ng = (nt + 3) / 4;  // scale groups
  // First tile of scale group g (the last group is shifted back so that its
  // 32 bytes per row stay inside the row).
  auto gstart = [&](int g) { return min(4 * g, nt - 4); };
  // Code load j of tile `tile` into the stage at `st`.
  auto load = [&](int j, int tile, uint8_t* st) {
    if (j < CPW)
      __builtin_amdgcn_global_load_lds((gvoid_t*)(base[j] + (int64_t)tile * (kKT / 2) + off[j]), (lvoid_t*)(st + dst[j]),
                                       16, 0, 0);
  };
  // The scale loads of group g (clamped to the last group) into ring slot g % 2.
  auto load_scales = [&](int g) {
    const int64_t b0 = (int64_t)gstart(min(g, ng - 1)) * (kKT / 16);
    uint8_t* const sl = smem + SRING + (g & 1) * SGROUP;
#pragma unroll
    for (int j = 0; j < SPW; ++j)
      __builtin_amdgcn_global_load_lds((gvoid_t*)(base[CPW + j] + b0 + off[CPW + j]), (lvoid_t*)(sl + dst[CPW + j]), 16,
                                       0, 0);
  };
  // Scale bytes of tile u in the ring, and this lane's offset within a fragment.
  auto sbase = [&](int u) -> const uint8_t* {
    const int g = u >> 2;
    return smem + SRING + (g & 1) * SGROUP + 8 * (u - gstart(g));
  };
  const int so = 32 * li + 4 * hh;

  const int wy = wave >> 1, wx = wave & 1;
  float16_t acc[FA][FB];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  load_scales(0);
#pragma unroll
  for (int t = 0; t < kStages; ++t) {
#pragma unroll
    for (int j = 0; j < CPW; ++j) load(j, min(t, nt - 1), smem + t * STAGE);
  }
  // The tensor scales, read now so that their latency hides under the wait
  // for the first tile instead of delaying the epilogue.
  float sab = ats[0] * bts[0];
  asm volatile("" : "+v"(sab));
  wait_vmcnt<2 * CPW>();  // scale group 0 and tile 0 landed (this wave's part)
  __builtin_amdgcn_s_barrier();

  Frags<FA, FB> F0, F1;
  half8_t A0[FA], B0[FB], A1[FA], B1[FB];
  read_stage(F0, smem, sbase(0), so, wy, wx, l, OFF_B);
  decode_step(F0, 0, A0, B0);

  auto body = [&](int t, const Frags<FA, FB>& cur, Frags<FA, FB>& nxt) {
    // Outstanding loads allowed: those body t-1 issued (codes of tile t+2,
    // plus a scale group when t - 1 = 1 mod 4).
    if ((t & 3) == 2) wait_vmcnt<CPW + SPW>();
    else wait_vmcnt<CPW>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    // (in the last body the next tile does not exist: its decode is never
    // used, and its scale bytes are read at the last tile's, in bounds)
    read_stage(nxt, smem + ((t + 1) % kStages) * STAGE, sbase(min(t + 1, nt - 1)), so, wy, wx, l, OFF_B);
    if ((t & 3) == 1) load_scales((t + 3) >> 2);
    uint8_t* const ist = smem + (t % kStages) * STAGE;
    const int tl = min(t + kStages, nt - 1);
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      mfma_step(A0, B0, acc);
#pragma unroll
      for (int q = 0; q < LPS; ++q) load(s * LPS + q, tl, ist);
      decode_step(cur, s + 1, A1, B1);
      step_schedule<FA, FB, LPS>();
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(A1, B1, acc);
#pragma unroll
      for (int q = 0; q < LPS; ++q) load((s + 1) * LPS + q, tl, ist);
      if (s + 2 < 8) decode_step(cur, s + 2, A0, B0);
      else decode_step(nxt, 0, A0, B0);
      step_schedule<FA, FB, LPS>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int t = 0;
  for (; t + 2 <= nt; t += 2) {
    body(t, F0, F1);
    body(t + 1, F1, F0);
  }
  if (t < nt) body(t, F0, F1);
  wait_vmcnt<0>();  // no load into LDS may be in flight when the workgroup ends

  const int m0 = mwg + wy * 32 * FA, n0 = nwg + wx * 32 * FB;
  {
  // The instances without a second epilogue path recompute the lane index
  // here: kept through the K loop it is spilled to scratch (the loop uses
  // all 256 VGPRs) and its reload waits behind the tile's stores.
  const int le = EDGE != 0 ? lane_id() : l, li = le & 31, hh = le >> 5;
  if constexpr (kStaged) {
    // Every wave has finished with the LDS ring (its loads landed, its reads
    // done) before any wave overwrites it with output.
    __syncthreads();
    static_assert(4 * kOutRegion <= SMEM, "the staging regions reuse the LDS rings");
    if constexpr (EDGE != 0) {
      // the host checked ldc % 8, the alignment of C and N % 8: edge tiles
      // (EDGE 2) store only their rows below M and 8-column pieces below N
      store_tile_staged<FA, FB, EPI, EDGE == 2>(acc, sab, m0, n0, le, li, hh, smem + wave * kOutRegion,
                                                static_cast<uint16_t*>(c), ldc, amax_out, M, N);
      return;
    }
    const bool whole = m0 + 32 * FA <= M && n0 + 32 * FB <= N && ldc % 8 == 0 && ((uintptr_t)c & 15) == 0;
    if (whole) {
      store_tile_staged<FA, FB, EPI>(acc, sab, m0, n0, le, li, hh, smem + wave * kOutRegion, static_cast<uint16_t*>(c),
                                     ldc, amax_out);
      return;
    }
  }
  if constexpr (!kStaged || EDGE == 0)
    store_tile<FA, FB, OUT, EPI, EDGE == 1>(acc, sab, m0, n0, le, li, hh, M, N, c, ldc, amax_out);
  }
}

// ---------------------------------------------------------------------------
// Fallback kernel: K < 512, K % 256 != 0 or misaligned operands (fragments
// straight from global memory, bounds-checked along K).
template <int FA, int FB, int OUT, int EPI>
__global__ __launch_bounds__(256) void gemm_checked_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    void* __restrict__ c, int64_t ldc, int M, int N, int K, float* __restrict__ amax_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int m0 = blockIdx.y * (64 * FA) + (wave >> 1) * 32 * FA;
  const int n0 = blockIdx.x * (64 * FB) + (wave & 1) * 32 * FB;
  const int64_t cpitch = K / 2, spitch = K / 16;
  const uint8_t* pa[FA];
  const uint8_t* psa[FA];
  const uint8_t* pb[FB];
  const uint8_t* psb[FB];
#pragma unroll
  for (int f = 0; f < FA; ++f) {
    const int row = min(m0 + 32 * f + li, M - 1);
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
  for (int kt = 0; kt < K; kt += kKT) {
    Frags<FA, FB> fr;
    load_frags_checked(fr, pa, psa, pb, psb, kt, hh, K);
    compute_tile(fr, acc);
  }
  store_tile<FA, FB, OUT, EPI>(acc, ats[0] * bts[0], m0, n0, lane, li, hh, M, N, c, ldc, amax_out);
}

struct Args {
  QOut a, b;
  int m, n, k;
  void* c;
  int64_t ldc;
  float* amax;
};

// Band width for tile_of: the ~32 tiles one XCD runs at once (32 CUs) span
// about sqrt(32 tileM / tileN) band columns, which balances the A and B
// bytes they touch.
inline int band_for(int tiles_m, int tiles_n, int tile_m, int tile_n) {
  const int ntiles = tiles_m * tiles_n;
  int conc = (ntiles + 7) / 8;
  if (conc > 32) conc = 32;
  int w = (int)std::lround(std::sqrt((double)conc * tile_m / tile_n));
  if (w < 1) w = 1;
  if (w > tiles_n) w = tiles_n;
  return w;
}

template <int FA, int FB, int OUT, int EPI>
void launch_lds(const Args& g, hipStream_t s) {
  const int tiles_m = (g.m + 64 * FA - 1) / (64 * FA), tiles_n = (g.n + 64 * FB - 1) / (64 * FB);
  const int band = band_for(tiles_m, tiles_n, 64 * FA, 64 * FB);
  // Instances without the branch between two epilogue paths when the launch
  // allows it: with the branch, all accumulators are copied to vector
  // registers ahead of it, which spills in the 4x4 kernels.  Float32 output
  // (4x4): a launch of whole tiles only (no tile reaches past M or N) needs
  // no edge path (EDGE 1).  bf16 output staged through LDS (FB 2 or 4):
  // with ldc % 8 == 0, C 16-byte aligned and N % 8 == 0 the staged path
  // stores edge tiles too, checking rows and 8-column pieces (EDGE 2; EDGE 1
  // without the checks when every tile is whole).
  const bool whole = g.m % (64 * FA) == 0 && g.n % (64 * FB) == 0;
  auto go = [&](auto edge) {
    gemm_lds_kernel<FA, FB, OUT, EPI, decltype(edge)::value><<<tiles_m * tiles_n, 256, 0, s>>>(
        g.a.codes, g.a.scales, g.a.tscale, g.b.codes, g.b.scales, g.b.tscale, g.c, g.ldc, g.m, g.n, g.k, g.amax, band);
  };
  if constexpr (OUT == 0 && FA * FB >= 16) {
    if (whole) return go(std::integral_constant<int, 1>());
  }
  if constexpr (OUT == 1 && (FB == 2 || FB == 4)) {
    if (g.ldc % 8 == 0 && ((uintptr_t)g.c & 15) == 0 && g.n % 8 == 0)
      return whole ? go(std::integral_constant<int, 1>()) : go(std::integral_constant<int, 2>());
  }
  go(std::integral_constant<int, 0>());
}

template <int OUT, int EPI>
void launch_lds_tiles(int fa, int fb, const Args& g, hipStream_t s) {
  if (fa == 1 && fb == 1) launch_lds<1, 1, OUT, EPI>(g, s);
  else if (fa == 4 && fb == 4) launch_lds<4, 4, OUT, EPI>(g, s);
  else if (fa == 3 && fb == 3) launch_lds<3, 3, OUT, EPI>(g, s);
  else if (fa == 4 && fb == 2) launch_lds<4, 2, OUT, EPI>(g, s);
  else launch_lds<2, 4, OUT, EPI>(g, s);
}

template <int OUT, int EPI>
void launch_checked(const Args& g, hipStream_t s) {
  const dim3 grid((unsigned)((g.n + 255) / 256), (unsigned)((g.m + 127) / 128));
  gemm_checked_kernel<2, 4, OUT, EPI><<<grid, 256, 0, s>>>(g.a.codes, g.a.scales, g.a.tscale, g.b.codes,
                                                           g.b.scales, g.b.tscale, g.c, g.ldc, g.m, g.n, g.k, g.amax);
}

// Tile shape by a small cost model: rounds of 256 workgroups (one per CU) x
// MFMA work per workgroup / relative efficiency of the shape (bigger
// fragments amortize the decode over more MFMAs).  The 64 x 64 tile (one
// fragment per wavefront) decodes the most per MFMA but spreads a small
// output over many CUs, which is what a latency-bound problem needs.
struct Cand { int fa, fb; double eff; };
constexpr Cand kCands[] = {{2, 4, 1.0}, {4, 2, 1.0}, {3, 3, 1.05}, {4, 4, 1.15}, {1, 1, 0.45}};

double tile_cost(int64_t m, int64_t n, const Cand& cd) {
  const int64_t tiles = ((m + 64 * cd.fa - 1) / (64 * cd.fa)) * ((n + 64 * cd.fb - 1) / (64 * cd.fb));
  return (double)((tiles + 255) / 256) * cd.fa * cd.fb / cd.eff;
}

Cand pick_tiles(int64_t m, int64_t n) {
  Cand best = kCands[0];
  double bc = 1e300;
  for (const Cand& cd : kCands) {
    const double c = tile_cost(m, n, cd);
    if (c < bc - 1e-9) { bc = c; best = cd; }
  }
  return best;
}

}  // namespace

bool gemm_tiles_supported(int fa, int fb) {
  return (fa == 2 && fb == 4) || (fa == 4 && fb == 2) || (fa == 3 && fb == 3) || (fa == 4 && fb == 4) ||
         (fa == 1 && fb == 1);
}

hipError_t launch_gemm(QOut a, QOut b, int64_t m, int64_t n, int64_t k, void* c, int c_dt,
                       int64_t ldc, int epilogue, float* amax_out, int tile_fa, int tile_fb, hipStream_t s) {
  if (amax_out != nullptr) {
    hipError_t e = launch_zero(amax_out, 1, s);
    if (e != hipSuccess) return e;
  }
  const Args g{a, b, (int)m, (int)n, (int)k, c, ldc, amax_out};
  // LDS path: K >= 512 (one scale group of four K-tiles) and K % 256 == 0,
  // so every code and scale row, and every scale group's first byte, is
  // 16-byte aligned as the direct-to-LDS 16-byte loads need.
  const bool lds_path = (k >= 4 * kKT) && (k % 256 == 0) && ((uintptr_t)a.codes % 16 == 0) &&
                        ((uintptr_t)b.codes % 16 == 0) && ((uintptr_t)a.scales % 16 == 0) && ((uintptr_t)b.scales % 16 == 0) &&
                        m * (k / 2) < ((int64_t)1 << 31) && n * (k / 2) < ((int64_t)1 << 31);  // 32-bit load offsets
  if (lds_path) {
    auto run = [&](int fa, int fb, const Args& ar) {
      if (c_dt == 0) { if (epilogue == 1) launch_lds_tiles<0, 1>(fa, fb, ar, s); else launch_lds_tiles<0, 0>(fa, fb, ar, s); }
      else { if (epilogue == 1) launch_lds_tiles<1, 1>(fa, fb, ar, s); else launch_lds_tiles<1, 0>(fa, fb, ar, s); }
    };
    if (gemm_tiles_supported(tile_fa, tile_fb)) {
      run(tile_fa, tile_fb, g);
      return hipGetLastError();
    }
    const Cand cd = pick_tiles(m, n);
    // A last row of tiles that is mostly empty can cost a whole extra round
    // of workgroups (10560 rows in 256-row tiles: 41 full tile rows and one
    // of 64 rows, 10 rounds of 256 tiles where 9 hold the work).  When the
    // cost model says so, the full tile rows run as one launch and the
    // remaining rows as a second launch with tiles fitted to them.  Every
    // output element is the same whatever tile computes it, so the split
    // changes no value.
    const int64_t tm = 64 * cd.fa, full = m / tm, rem = m - full * tm;
    if (rem > 0 && full > 0) {
      const Cand rc = pick_tiles(rem, n);
      if (tile_cost(full * tm, n, cd) + tile_cost(rem, n, rc) < 0.95 * tile_cost(m, n, cd)) {
        const int64_t m1 = full * tm;
        Args top = g, bottom = g;
        top.m = (int)m1;
        bottom.m = (int)rem;
        bottom.a.codes = a.codes + m1 * (k / 2);
        bottom.a.scales = a.scales + m1 * (k / 16);
        bottom.c = static_cast<uint8_t*>(c) + m1 * ldc * (c_dt == 0 ? 4 : 2);
        run(cd.fa, cd.fb, top);
        run(rc.fa, rc.fb, bottom);
        return hipGetLastError();
      }
    }
    run(cd.fa, cd.fb, g);
  } else {
    if (c_dt == 0) { if (epilogue == 1) launch_checked<0, 1>(g, s); else launch_checked<0, 0>(g, s); }
    else { if (epilogue == 1) launch_checked<1, 1>(g, s); else launch_checked<1, 0>(g, s); }
  }
  return hipGetLastError();
}

}  // namespace nvfp4
