// Frame-causal window attention that reads the NVFP4 KV cache directly.
//
// The cache (3 sink + 9 local latent frames: 171host.com "LongLive 2.0
// 技术拆解", section 2.2) is held in NVFP4 with one tensor scale per block of
// 8 frames (hyper.ai LongLive-2.0 summary, "方法"; tailorednewshub.com
// "LongLive-2.0: Infraestructura paralela NVFP4 para video largo", section
// "Inferencia W4A4 NVFP4").  Instead of rebuilding a bf16 copy of the window
// and running attention over it, every K/V tile is decoded into LDS inside the
// attention loop, so the cache is read once per workgroup at 4.5 bits per
// element and the bf16 window is never written.
//
//   O[q, h, :] = sum_j softmax_j(Q[q,h,:] . K[j,h,:] / sqrt(128)) V[j,h,:]
//   over the keys j of frames 0 .. frame(q)   (frame-level causal mask)
//
// with K, V = e2m1(code) * s_b * S exactly as the codec defines them.
//
// Arithmetic.  A decoded element e2m1 * s_b has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in fp16; both products run on
// v_mfma_f32_32x32x16_f16 with float32 accumulation:
//   * S^T = K Q^T.  Q (bf16) enters as fp16 after a power-of-two scale per
//     query row that puts the row maximum in [2^14, 2^15): every bf16 value
//     within 2^-29 of the row maximum converts exactly, and smaller ones move
//     the dot product by less than float32 accumulation does.  The row scale,
//     the K tensor scale of the tile's frame block and log2(e)/sqrt(128) are
//     one float32 factor per lane applied to the accumulator.
//   * Softmax in base 2 with a running maximum per query.  The maximum is only
//     moved when the new tile exceeds it by more than 8 (a factor 256), so the
//     accumulator is rescaled rarely; probabilities stay <= 256 and go to fp16
//     (11 significant bits).
//   * O^T = V^T P^T.  The accumulator is kept in units of one V tensor scale and
//     rescaled by the ratio when a key block with another frame-block scale
//     arrives (once per frame-block boundary).
//
// Work split.  A workgroup of 4 wavefronts owns 128 queries of one head.
// Wavefront w takes queries 64*(w&1) .. +63 (two 32-query MFMA columns) and
// the key block of parity w>>1 in every 64-key tile, so each wavefront runs
// 16 + 16 MFMAs per tile and the two parities are merged once at the end.
// Lanes own queries: in the transposed products each lane holds one query
// column, so the row maximum, row sum and rescales are per-lane scalars and
// the probabilities feed the second MFMA from the registers they were
// computed in (the key order inside an MFMA step is permuted to match, see
// decode_v).  Tiles are double-buffered in LDS: while tile t is consumed, the
// raw codes of tile t+1 (loaded one iteration earlier) are decoded into the
// other buffer; one barrier per tile.
#include <cmath>

#include "device.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kD = 128;                  // head_dim
constexpr int kQT = 128;                 // queries per workgroup
constexpr int kKT = 64;                  // keys per tile
constexpr int kKRow = 2 * kD + 16;       // bytes per decoded K row (fp16, padded)
constexpr int kVRow = 2 * kKT + 16;      // bytes per decoded V^T row (fp16, padded)
constexpr int kKBuf = kKT * kKRow;       // 17408
constexpr int kVBuf = kD * kVRow;        // 18432
constexpr int kBuf = kKBuf + kVBuf;
constexpr int kLds = 2 * kBuf;           // 71680
constexpr float kMInit = -1.0e30f;       // finite: exp2(kMInit - m) = 0, exp2(0) = 1
constexpr float kLazy = 8.0f;            // rescale threshold (log2 units)
constexpr float kLog2eRsqrtD = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)

// Raw codes of one tile held by a lane between its load and its decode.
struct Raw {
  u32x4_t kc;       // 32 K codes: key (lane & 63), d in [32 * wave, +32)
  uint32_t ks;      // their two E4M3 block scales (low 16 bits)
  uint32_t vc[4];   // 8 V codes (d in [8 * dc, +8)) of keys 4 * kg + r
  uint32_t vs[4];   // the V block scale of each of those keys
};

struct Geo {
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int heads, h, nkeys;
};

__device__ __forceinline__ half8_t decode8(uint32_t codes, half2_t sig2) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sig2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sig2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sig2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sig2;
  half8_t r;
  r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
  r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  return r;
}

__device__ __forceinline__ void load_raw(const Geo& g, int key0, int tid, Raw& r) {
  const int wave = tid >> 6;
  {
    const int key = min(key0 + (tid & 63), g.nkeys - 1);
    const uint32_t row = (uint32_t)key * (uint32_t)g.heads + (uint32_t)g.h;
    r.kc = *reinterpret_cast<const u32x4_t*>(g.kc + row * 64u + 16u * wave);
    r.ks = *reinterpret_cast<const uint16_t*>(g.ks + row * 8u + 2u * wave);
  }
  const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = min(key0 + 4 * kg + i, g.nkeys - 1);
    const uint32_t row = (uint32_t)key * (uint32_t)g.heads + (uint32_t)g.h;
    r.vc[i] = *reinterpret_cast<const uint32_t*>(g.vc + row * 64u + 4u * dc);
    r.vs[i] = g.vs[row * 8u + (dc >> 1)];
  }
}

// K tile, row-major: K_lds[key][d], fp16, row pitch kKRow.
__device__ __forceinline__ void decode_k(const Raw& r, uint8_t* buf, int tid) {
  const int wave = tid >> 6, key = tid & 63;
  const half2_t s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.ks, 1.0f, false);
  const half2_t s0 = {s.x, s.x}, s1 = {s.y, s.y};
  uint8_t* dst = buf + key * kKRow + 64 * wave;
  *reinterpret_cast<half8_t*>(dst + 0) = decode8(r.kc[0], s0);
  *reinterpret_cast<half8_t*>(dst + 16) = decode8(r.kc[1], s0);
  *reinterpret_cast<half8_t*>(dst + 32) = decode8(r.kc[2], s1);
  *reinterpret_cast<half8_t*>(dst + 48) = decode8(r.kc[3], s1);
}

// Code byte B of the interleaved key pairs: d = 2B (lo) and d = 2B + 1 (hi)
// for keys (0, 1) and (2, 3), one 8-byte LDS write per d.
template <int B>
__device__ __forceinline__ void v_byte(uint32_t lo01, uint32_t hi01, uint32_t lo23, uint32_t hi23, half2_t s01,
                                       half2_t s23, uint8_t* dst) {
  const half2_t e01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo01, 1.0f, B) * s01;
  const half2_t e23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo23, 1.0f, B) * s23;
  const half2_t o01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi01, 1.0f, B) * s01;
  const half2_t o23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi23, 1.0f, B) * s23;
  u32x2_t we, wo;
  we[0] = __builtin_bit_cast(uint32_t, e01); we[1] = __builtin_bit_cast(uint32_t, e23);
  wo[0] = __builtin_bit_cast(uint32_t, o01); wo[1] = __builtin_bit_cast(uint32_t, o23);
  *reinterpret_cast<u32x2_t*>(dst + (2 * B) * kVRow) = we;
  *reinterpret_cast<u32x2_t*>(dst + (2 * B + 1) * kVRow) = wo;
}

// V tile, transposed: Vt_lds[d][key'], fp16, row pitch kVRow.  key' permutes
// the key offset o (0..63) by swapping its bits 2 and 3: the second MFMA's
// k-step u of key block b then reads, in lane half hf, the 8 keys
// 32b + 16u + {0,1,2,3,8,9,10,11} + 4hf contiguously — exactly the keys whose
// probabilities that lane holds from the first MFMA's output layout.
// Each lane decodes 4 consecutive keys x 8 d and writes one 8-byte group of 4
// keys per d; the two nibble streams of a key pair are interleaved first so
// that one conversion yields the pair (key0, key1) at the same d.
__device__ __forceinline__ void decode_v(const Raw& r, uint8_t* buf, int tid) {
  const int kg = tid & 15, dc = tid >> 4;
  const int kgp = (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);
  const uint32_t m = 0x0F0F0F0Fu;
  const uint32_t lo01 = (r.vc[0] & m) | ((r.vc[1] << 4) & ~m);
  const uint32_t hi01 = ((r.vc[0] >> 4) & m) | (r.vc[1] & ~m);
  const uint32_t lo23 = (r.vc[2] & m) | ((r.vc[3] << 4) & ~m);
  const uint32_t hi23 = ((r.vc[2] >> 4) & m) | (r.vc[3] & ~m);
  const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.vs[0] | (r.vs[1] << 8), 1.0f, false);
  const half2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.vs[2] | (r.vs[3] << 8), 1.0f, false);
  uint8_t* dst = buf + kKBuf + (8 * dc) * kVRow + 8 * kgp;
  v_byte<0>(lo01, hi01, lo23, hi23, s01, s23, dst);
  v_byte<1>(lo01, hi01, lo23, hi23, s01, s23, dst);
  v_byte<2>(lo01, hi01, lo23, hi23, s01, s23, dst);
  v_byte<3>(lo01, hi01, lo23, hi23, s01, s23, dst);
}

// Per-query-column state of a wavefront (two 32-query columns g = 0, 1).
struct State {
  float16_t acc[2][4];   // O^T: column g, d block db (32 d), in units of svref
  float m[2];            // running maximum (base 2), equal in lanes c and c + 32
  float l[2];            // partial row sum over this lane's keys
  float svref;           // V tensor scale the accumulator is expressed in (0: none yet)
};

template <int G>
__device__ __forceinline__ void softmax_col(float16_t& s, float c, bool masked, int key_base, int hf, int lim,
                                            State& st, half8_t& p0, half8_t& p1) {
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = s[i] * c;
    if (masked) {
      const int key = key_base + 8 * (i >> 2) + 4 * hf + (i & 3);
      v = key < lim ? v : -INFINITY;
    }
    s[i] = v;
    mt = fmaxf(mt, v);
  }
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mnew = fmaxf(st.m[G], mt);
  const bool need = mnew > st.m[G] + kLazy;
  if (__ballot(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m[G] - mnew) : 1.0f;
    st.m[G] = need ? mnew : st.m[G];
    st.l[G] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[G][db][i] *= alpha;
  }
  const float mref = st.m[G];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float p = __builtin_amdgcn_exp2f(s[i] - mref);
    sum += p;
    if (i < 8) p0[i] = (_Float16)p; else p1[i - 8] = (_Float16)p;
  }
  st.l[G] += sum;
}

// Merge the partner wavefront's partial (other key parity) for column G and
// write the 32 queries x 128 d of that column.
template <int G, bool F32OUT>
__device__ __forceinline__ void finish_col(const State& st, const float* part, int lane, int64_t qrow, bool valid,
                                           void* __restrict__ out) {
  const int hf = lane >> 5;
  const float m1 = part[64 * 64 + lane], l1 = part[64 * 64 + 64 + lane], sv1 = part[64 * 64 + 128 + lane];
  const float l0 = st.l[G] + __shfl_xor(st.l[G], 32, 64);
  const float m0 = st.m[G];
  const float M = fmaxf(m0, m1);
  const float e0 = __builtin_amdgcn_exp2f(m0 - M), e1 = __builtin_amdgcn_exp2f(m1 - M);
  const float inv = 1.0f / (l0 * e0 + l1 * e1);
  const float a0 = st.svref * e0 * inv, a1 = sv1 * e1 * inv;
  if (!valid) return;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * i4 + r;
        v[r] = st.acc[G][db][i] * a0 + part[(db * 16 + i) * 64 + lane] * a1;
      }
      const int d = 32 * db + 8 * i4 + 4 * hf;
      if constexpr (F32OUT) {
        float4_t w = {v[0], v[1], v[2], v[3]};
        *reinterpret_cast<float4_t*>(static_cast<float*>(out) + qrow * kD + d) = w;
      } else {
        u32x2_t w;
        w[0] = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
        w[1] = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + qrow * kD + d) = w;
      }
    }
  }
}

// Store column G of this wavefront's partial for the partner to merge.
template <int G>
__device__ __forceinline__ void stash_col(const State& st, float* part, int lane) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[(db * 16 + i) * 64 + lane] = st.acc[G][db][i];
  part[64 * 64 + lane] = st.m[G];
  part[64 * 64 + 64 + lane] = st.l[G] + __shfl_xor(st.l[G], 32, 64);
  part[64 * 64 + 128 + lane] = st.svref;
}

template <bool F32OUT>
__global__ __launch_bounds__(256) void kv_attention_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks,
    const float* __restrict__ kts, const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs,
    const float* __restrict__ vts, void* __restrict__ out, int nq, int tokens, int heads, int frames,
    int q_frames, int fb_keys, int qtiles) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave & 1, kp = wave >> 1;
  const int c = lane & 31, hf = lane >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of (head, query tile) so the heads it reads stay in its L2.
  const int n = gridDim.x, w = blockIdx.x;
  const int per = n >> 3, rem = n & 7, x = w & 7;
  const int id = x * per + min(x, rem) + (w >> 3);
  const int h = id / qtiles, qt = id - h * qtiles;

  const int nkeys = frames * tokens;
  const int q0 = qt * kQT;
  const int qlast = min(q0 + kQT, nq) - 1;
  const int first_frame = frames - q_frames;
  const int kmin = (first_frame + q0 / tokens + 1) * tokens;      // every query sees keys < kmin
  const int kmax = (first_frame + qlast / tokens + 1) * tokens;   // no query sees keys >= kmax
  const int nt = (kmax + kKT - 1) / kKT;

  Geo geo{kc, ks, vc, vs, heads, h, nkeys};

  // Queries of this lane (two columns), converted to fp16 with a per-row
  // power-of-two scale; d of MFMA step s is 16s + 8hf + j.
  half8_t qf[2][8];
  float cq[2];
  int lim[2];
  int64_t qrow[2];
  bool qvalid[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int qi = q0 + 64 * qh + 32 * g + c;
    qvalid[g] = qi < nq;
    qrow[g] = (int64_t)qi * heads + h;
    lim[g] = qvalid[g] ? (first_frame + qi / tokens + 1) * tokens : kmax;
    u32x4_t raw[8];
    float mx = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      raw[s] = qvalid[g] ? *reinterpret_cast<const u32x4_t*>(q + qrow[g] * kD + 16 * s + 8 * hf) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mx = fmaxf(mx, fabsf(bf16_to_f32(raw[s][j] & 0xFFFFu)));
        mx = fmaxf(mx, fabsf(bf16_to_f32(raw[s][j] >> 16)));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    int e = 0;
    if (mx > 0.0f) {
      int E;
      (void)frexpf(mx, &E);             // mx = f * 2^E, f in [0.5, 1)
      e = min(max(15 - E, -126), 126);  // mx * 2^e in [2^14, 2^15) unless clamped
    }
    const float sc = ldexpf(1.0f, e);
    cq[g] = ldexpf(kLog2eRsqrtD, -e);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qf[g][s][2 * j] = (_Float16)(bf16_to_f32(raw[s][j] & 0xFFFFu) * sc);
        qf[g][s][2 * j + 1] = (_Float16)(bf16_to_f32(raw[s][j] >> 16) * sc);
      }
  }

  State st;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    st.m[g] = kMInit;
    st.l[g] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[g][db][i] = 0.0f;
  }
  st.svref = 0.0f;

  Raw raw;
  load_raw(geo, 0, tid, raw);
  decode_k(raw, smem, tid);
  decode_v(raw, smem, tid);
  if (nt > 1) load_raw(geo, kKT, tid, raw);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    uint8_t* buf = smem + (t & 1) * kBuf;
    const int kbase = t * kKT + 32 * kp;
    if (kbase < kmax) {
      const int fb = kbase / fb_keys;
      const float skt = kts[fb], svt = vts[fb];
      float16_t sacc[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) { sacc[0][i] = 0.0f; sacc[1][i] = 0.0f; }
      const uint8_t* ka = buf + (32 * kp + c) * kKRow + 16 * hf;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const half8_t a = *reinterpret_cast<const half8_t*>(ka + 32 * s);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[0][s], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[1][s], sacc[1], 0, 0, 0);
      }
      const bool masked = kbase + 32 > kmin;
      half8_t pb[2][2];
      softmax_col<0>(sacc[0], cq[0] * skt, masked, kbase, hf, lim[0], st, pb[0][0], pb[0][1]);
      softmax_col<1>(sacc[1], cq[1] * skt, masked, kbase, hf, lim[1], st, pb[1][0], pb[1][1]);
      if (svt != 0.0f) {
        if (st.svref == 0.0f) {
          st.svref = svt;
        } else if (svt != st.svref) {
          const float ratio = st.svref / svt;
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) st.acc[g][db][i] *= ratio;
          st.svref = svt;
        }
        const uint8_t* va = buf + kKBuf + c * kVRow + 2 * (32 * kp + 8 * hf);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const half8_t a = *reinterpret_cast<const half8_t*>(va + (32 * db) * kVRow + 32 * u);
            st.acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[0][u], st.acc[0][db], 0, 0, 0);
            st.acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[1][u], st.acc[1][db], 0, 0, 0);
          }
      }
    }
    if (t + 1 < nt) {
      uint8_t* nbuf = smem + ((t + 1) & 1) * kBuf;
      decode_k(raw, nbuf, tid);
      decode_v(raw, nbuf, tid);
      if (t + 2 < nt) load_raw(geo, (t + 2) * kKT, tid, raw);
    }
    __syncthreads();
  }

  // Merge the two key parities: wavefront (qh, kp) finishes column g = kp and
  // hands column 1 - kp to its partner.  The loop's last barrier freed LDS.
  float* parts = reinterpret_cast<float*>(smem);
  constexpr int kPart = 64 * 64 + 3 * 64;   // floats per (qh, g) region
  if (kp == 0) stash_col<1>(st, parts + (qh * 2 + 1) * kPart, lane);
  else stash_col<0>(st, parts + (qh * 2 + 0) * kPart, lane);
  __syncthreads();
  if (kp == 0) finish_col<0, F32OUT>(st, parts + (qh * 2 + 0) * kPart, lane, qrow[0], qvalid[0], out);
  else finish_col<1, F32OUT>(st, parts + (qh * 2 + 1) * kPart, lane, qrow[1], qvalid[1], out);
}

static_assert(4 * (64 * 64 + 3 * 64) * 4 <= kLds, "merge regions must fit in LDS");

}  // namespace

hipError_t launch_kv_attention(const uint16_t* q, QOut k, QOut v, void* out, int out_f32, int64_t nq, int64_t tokens,
                               int64_t heads, int64_t frames, int64_t q_frames, int64_t frame_block,
                               hipStream_t s) {
  const int qtiles = (int)((nq + kQT - 1) / kQT);
  const int grid = qtiles * (int)heads;
  const int fb_keys = (int)(frame_block * tokens);
  if (out_f32)
    kv_attention_kernel<true><<<grid, 256, 0, s>>>(q, k.codes, k.scales, k.tscale, v.codes, v.scales, v.tscale, out,
                                                   (int)nq, (int)tokens, (int)heads, (int)frames, (int)q_frames,
                                                   fb_keys, qtiles);
  else
    kv_attention_kernel<false><<<grid, 256, 0, s>>>(q, k.codes, k.scales, k.tscale, v.codes, v.scales, v.tscale,
                                                    out, (int)nq, (int)tokens, (int)heads, (int)frames,
                                                    (int)q_frames, fb_keys, qtiles);
  return hipGetLastError();
}

}  // namespace nvfp4
