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
//   O[q, h, :] = sum_j softmax_j(Q[q,h,:] . K[j,h,:] / sqrt(D)) V[j,h,:]
//   over the keys j of frames 0 .. frame(q)   (frame-level causal mask)
//
// with K, V = e2m1(code) * s_b * S exactly as the codec defines them, for a
// head dimension D of 64 or 128 (one kernel instance each).
//
// Arithmetic.  A decoded element e2m1 * s_b has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in fp16; both products run on
// v_mfma_f32_32x32x16_f16 with float32 accumulation:
//   * S^T = K Q^T.  Q (bf16) enters as fp16 after a power-of-two scale per
//     query row that puts the row maximum in [2^14, 2^15): every bf16 value
//     within 2^-29 of the row maximum converts exactly, and smaller ones move
//     the dot product by less than float32 accumulation does.  The row scale,
//     the K tensor scale of the tile's frame block and log2(e)/sqrt(D) are
//     one float32 factor per lane applied to the accumulator.
//   * Softmax in base 2 with a running maximum per query.  The maximum is only
//     moved when the new tile exceeds it by more than 8 (a factor 256), so the
//     accumulator is rescaled rarely; probabilities stay <= 256 and go to fp16
//     (11 significant bits above 2^-14; below, fp16 subnormals round to a
//     multiple of 2^-24, which only matters when the keys weighted below
//     about 2^-24 of the largest carry the output).
//   * O^T = V^T P^T.  The accumulator is kept in units of one V tensor scale and
//     rescaled by the ratio when a key block with another frame-block scale
//     arrives (once per frame-block boundary).
//
// Work split.  A workgroup of 4 wavefronts owns 128 queries of one head;
// wavefront w takes queries 32w .. 32w+31 (one 32-query MFMA column) over all
// keys, so each wavefront runs D/8 + D/8 MFMAs per 64-key tile.  Two workgroups
// share a CU, so the two wavefronts on a SIMD come from different workgroups
// and their MFMA and VALU work interleaves.  Lanes own queries: in the
// transposed products each lane holds one query column, so the row maximum,
// row sum and rescales are per-lane scalars and the probabilities feed the
// second MFMA from the registers they were computed in (the key order inside
// an MFMA step is permuted to match, see decode_v).  Tiles are double-buffered
// in LDS and the loop is software-pipelined by one tile on the K side: the
// scores of tile t+1 are computed while tile t's softmax runs, and tile t's
// P V product overlaps the decode of the next tiles (raw codes loaded one
// iteration earlier); one barrier per tile.
//
// Key tiles follow the frame blocks: the tiles of frame block b start at its
// first key, so no tile mixes two tensor scales.  When a frame block is not a
// whole number of tiles, its last tile is partial and its keys past the
// block end are masked (they belong to the next block's first tile); when it
// is (e.g. 8 frames of 880 tokens), tile t simply starts at key 64 t.
#include <cmath>
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kQT = 128;                 // queries per workgroup
constexpr int kKT = 64;                  // keys per tile
constexpr int kVRow = 2 * kKT + 16;      // bytes per decoded V^T row (fp16, padded)
constexpr float kMInit = -1.0e30f;       // finite: exp2(kMInit - m) = 0, exp2(0) = 1
constexpr float kLazy = 8.0f;            // rescale threshold (log2 units)

// Sizes that follow the head dimension D (64 or 128).  Lane duties: in the
// K decode lane (key, wave) owns d in [D/4 * wave, +D/4) (D/8 code bytes);
// in the V decode lane (kg, dc) owns 4 keys x D/16 elements (D/32 code bytes
// per key).
template <int D>
struct Dim {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  static constexpr int kKRow = 2 * D + 16;     // bytes per decoded K row (fp16, padded)
  static constexpr int kKBuf = kKT * kKRow;    // 17408 at D = 128
  static constexpr int kVBuf = D * kVRow;      // 18432 at D = 128
  static constexpr int kBuf = kKBuf + kVBuf;
  static constexpr int kLds = 2 * kBuf;        // 71680 at D = 128
  static constexpr int kSteps = D / 16;        // k-steps of the score MFMA
  static constexpr int kDB = D / 32;           // 32-wide d blocks of the output
  static constexpr int kRow = D / 2;           // code bytes per cache row
  static constexpr int kKW = D / 32;           // 32-bit code words per lane of a K tile
  using KWords = std::conditional_t<D == 128, u32x4_t, u32x2_t>;
  static constexpr int kVB = D / 32;           // code bytes per key per lane of a V tile
  // log2(e) / sqrt(D)
  static constexpr float kLog2eRsqrtD = 1.4426950408889634f * (D == 64 ? 0.125f : 0.08838834764831845f);
};

// Raw codes of one tile held by a lane between its load and its decode.
template <int D>
struct Raw {
  typename Dim<D>::KWords kc;   // D/4 K codes: key (lane & 63), d in [D/4 * wave, +D/4)
  uint32_t ks;                  // their E4M3 block scales (low D/64 bytes)
  uint32_t vc[4];               // D/16 V codes (d in [D/16 * dc, +D/16)) of keys 4 * kg + r
  uint32_t vs[4];               // the V block scale of each of those keys
};

struct Geo {
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int heads, h, nkeys;
  // byte offsets of this lane's code loads from the first code row of a tile
  // (scale offsets are these >> 3: a row has D/2 code bytes and D/16 scale
  // bytes, 8 code bytes per scale byte)
  uint32_t okc, ovc[4];
};

template <int D>
__device__ __forceinline__ void init_geo(Geo& g, int tid) {
  const uint32_t rb = (uint32_t)g.heads * Dim<D>::kRow;   // code bytes between consecutive keys
  g.okc = (uint32_t)(tid & 63) * rb + (uint32_t)(4 * Dim<D>::kKW) * (uint32_t)(tid >> 6);
  const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) g.ovc[i] = (uint32_t)(4 * kg + i) * rb + (uint32_t)Dim<D>::kVB * (uint32_t)dc;
}

// The lane's V code bytes of one key at p (D/32 bytes).
template <int D>
__device__ __forceinline__ uint32_t load_vbytes(const uint8_t* p) {
  if constexpr (D == 128) return *reinterpret_cast<const uint32_t*>(p);
  else return *reinterpret_cast<const uint16_t*>(p);
}
// The K block scales of one lane (D/64 bytes) at p.
template <int D>
__device__ __forceinline__ uint32_t load_kscales(const uint8_t* p) {
  if constexpr (D == 128) return *reinterpret_cast<const uint16_t*>(p);
  else return *p;
}

// Raw codes of K tile key0 (D/8 code bytes + D/64 scale bytes per lane).
template <int D>
__device__ __forceinline__ void load_raw_k(const Geo& g, int key0, int tid, Raw<D>& r) {
  constexpr uint32_t kRow = Dim<D>::kRow;
  if (key0 + kKT <= g.nkeys) {
    const uint32_t row0 = (uint32_t)key0 * (uint32_t)g.heads + (uint32_t)g.h;
    r.kc = *reinterpret_cast<const typename Dim<D>::KWords*>(g.kc + (size_t)row0 * kRow + g.okc);
    r.ks = load_kscales<D>(g.ks + (size_t)row0 * (kRow / 8) + (g.okc >> 3));
    return;
  }
  // last, partial tile: rows past the end re-read the last key (masked)
  const int key = min(key0 + (tid & 63), g.nkeys - 1);
  const uint32_t row = (uint32_t)key * (uint32_t)g.heads + (uint32_t)g.h;
  const uint32_t wave = (uint32_t)(tid >> 6);
  r.kc = *reinterpret_cast<const typename Dim<D>::KWords*>(g.kc + row * kRow + (D / 8) * wave);
  r.ks = load_kscales<D>(g.ks + row * (kRow / 8) + (D / 64) * wave);
}

// Raw codes of V tile key0 (4 keys x D/16 elements per lane).
template <int D>
__device__ __forceinline__ void load_raw_v(const Geo& g, int key0, int tid, Raw<D>& r) {
  constexpr uint32_t kRow = Dim<D>::kRow;
  if (key0 + kKT <= g.nkeys) {
    const uint32_t row0 = (uint32_t)key0 * (uint32_t)g.heads + (uint32_t)g.h;
    const uint8_t* vcb = g.vc + (size_t)row0 * kRow;
    const uint8_t* vsb = g.vs + (size_t)row0 * (kRow / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.vc[i] = load_vbytes<D>(vcb + g.ovc[i]);
      r.vs[i] = vsb[g.ovc[i] >> 3];
    }
    return;
  }
  const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = min(key0 + 4 * kg + i, g.nkeys - 1);
    const uint32_t row = (uint32_t)key * (uint32_t)g.heads + (uint32_t)g.h;
    r.vc[i] = load_vbytes<D>(g.vc + row * kRow + (uint32_t)Dim<D>::kVB * dc);
    r.vs[i] = g.vs[row * (kRow / 8) + (dc >> (D == 128 ? 1 : 2))];   // 16 elements per scale
  }
}

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

// K tile, row-major: K_lds[key][d], fp16, row pitch kKRow.  Code word w
// (8 elements) takes block scale w / 2.
template <int D>
__device__ __forceinline__ void decode_k(const Raw<D>& r, uint8_t* buf, int tid) {
  const int wave = tid >> 6, key = tid & 63;
  const half2_t s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.ks, 1.0f, false);
  const half2_t s0 = {s.x, s.x}, s1 = {s.y, s.y};
  uint8_t* dst = buf + key * Dim<D>::kKRow + Dim<D>::kRow * wave;
#pragma unroll
  for (int w = 0; w < Dim<D>::kKW; ++w)
    *reinterpret_cast<half8_t*>(dst + 16 * w) = decode8(r.kc[w], w < 2 ? s0 : s1);
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

// V tile, transposed: Vt_lds[d][key'], fp16, row pitch kVRow, after the K
// tile in the buffer.  key' permutes
// the key offset o (0..63) by swapping its bits 2 and 3: the second MFMA's
// k-step u of key block b then reads, in lane half hf, the 8 keys
// 32b + 16u + {0,1,2,3,8,9,10,11} + 4hf contiguously — exactly the keys whose
// probabilities that lane holds from the first MFMA's output layout.
// Each lane decodes 4 consecutive keys x D/16 d and writes one 8-byte group of
// 4 keys per d; the two nibble streams of a key pair are interleaved first so
// that one conversion yields the pair (key0, key1) at the same d.
template <int D>
__device__ __forceinline__ void decode_v(const Raw<D>& r, uint8_t* buf, int tid) {
  const int kg = tid & 15, dc = tid >> 4;
  const int kgp = (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);
  const uint32_t m = 0x0F0F0F0Fu;
  const uint32_t lo01 = (r.vc[0] & m) | ((r.vc[1] << 4) & ~m);
  const uint32_t hi01 = ((r.vc[0] >> 4) & m) | (r.vc[1] & ~m);
  const uint32_t lo23 = (r.vc[2] & m) | ((r.vc[3] << 4) & ~m);
  const uint32_t hi23 = ((r.vc[2] >> 4) & m) | (r.vc[3] & ~m);
  const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.vs[0] | (r.vs[1] << 8), 1.0f, false);
  const half2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.vs[2] | (r.vs[3] << 8), 1.0f, false);
  uint8_t* dst = buf + Dim<D>::kKBuf + (2 * Dim<D>::kVB * dc) * kVRow + 8 * kgp;
  v_byte<0>(lo01, hi01, lo23, hi23, s01, s23, dst);
  v_byte<1>(lo01, hi01, lo23, hi23, s01, s23, dst);
  if constexpr (Dim<D>::kVB == 4) {
    v_byte<2>(lo01, hi01, lo23, hi23, s01, s23, dst);
    v_byte<3>(lo01, hi01, lo23, hi23, s01, s23, dst);
  }
}

// Softmax and output state of one wavefront (32 queries, one per lane column).
template <int D>
struct State {
  float16_t acc[Dim<D>::kDB];   // O^T for d block db (32 d), in units of svref
  float m;            // running maximum of the scaled scores (base 2), equal in lanes c and c + 32
  float l;            // partial row sum over this lane's keys
  float svref;        // V tensor scale the accumulator is expressed in (0: none yet)
};

// S^T = K Q^T for one 64-key tile (two 32-key blocks) of the wavefront's 32
// queries; kbuf holds the decoded K tile.
template <int D>
__device__ __forceinline__ void qk_tile(const uint8_t* kbuf, int c, int hf, const half8_t (&qf)[Dim<D>::kSteps],
                                        float16_t (&sacc)[2]) {
  constexpr int kKRow = Dim<D>::kKRow;
#pragma unroll
  for (int i = 0; i < 16; ++i) { sacc[0][i] = 0.0f; sacc[1][i] = 0.0f; }
  const uint8_t* ka = kbuf + c * kKRow + 16 * hf;
#pragma unroll
  for (int s = 0; s < Dim<D>::kSteps; ++s) {
    const half8_t a0 = *reinterpret_cast<const half8_t*>(ka + 32 * s);
    const half8_t a1 = *reinterpret_cast<const half8_t*>(ka + 32 * kKRow + 32 * s);
    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qf[s], sacc[0], 0, 0, 0);
    sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, qf[s], sacc[1], 0, 0, 0);
  }
}

// Online softmax of one tile's scores (the tile lies in one frame block: sk is
// its K tensor scale).  Produces the fp16 probabilities and returns the factor
// the accumulator must be multiplied by before they are added (1 unless the
// running maximum moved).  MASK: apply the per-query key limit.
template <bool MASK, int D>
__device__ __forceinline__ float softmax_tile(float16_t (&sacc)[2], int key0, int hf, float cq, int lim, float sk,
                                              State<D>& st, half8_t (&pb)[2][2]) {
  // Scaled scores s = raw * cs, rounded to float32 first and the maximum
  // taken over those same values, so the maximum's exponent is exactly 0 at
  // any magnitude (an fma against a rounded maximum would leave a residual
  // of up to half an ulp of it: beyond 2^24 enough to overflow or flush every
  // probability).  Contraction of s - m into an fma is therefore off here.
  // Masked keys become -inf.
#pragma clang fp contract(off)
  const float cs = cq * sk;
  const int rel = lim - key0 - 4 * hf;   // key offset limit of this lane's elements
  float mt = -INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = sacc[b][i] * cs;
      if (MASK) v = (32 * b + 8 * (i >> 2) + (i & 3)) < rel ? v : -INFINITY;
      sacc[b][i] = v;
      mt = fmaxf(mt, v);
    }
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));   // the pair of lanes holding one query
  const float mnew = fmaxf(st.m, mt);
  const bool need = mnew > st.m + kLazy;
  const float alpha = need ? __builtin_amdgcn_exp2f(st.m - mnew) : 1.0f;
  st.m = need ? mnew : st.m;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pb[0][i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(sacc[0][i] - st.m);
    pb[1][i >> 3][i & 7] = (_Float16)__builtin_amdgcn_exp2f(sacc[1][i] - st.m);
  }
  // Row sum of the rounded probabilities, the values the numerator uses:
  // fp16 pairs dotted with (1, 1) into float32 accumulators.
  const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
  float sa = 0.0f, sb = 0.0f;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sa = __builtin_amdgcn_fdot2(half2_t{pb[0][u][2 * k], pb[0][u][2 * k + 1]}, one2, sa, false);
      sb = __builtin_amdgcn_fdot2(half2_t{pb[1][u][2 * k], pb[1][u][2 * k + 1]}, one2, sb, false);
    }
  st.l = st.l * alpha + (sa + sb);
  // materialize the probabilities here, ahead of the rescale branch, so they
  // are computed alongside the next tile's score MFMAs
  __asm__ volatile("" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]));
  return alpha;
}

template <int D>
__device__ __forceinline__ void rescale(State<D>& st, float f) {
  if (__ballot(f != 1.0f)) {
#pragma unroll
    for (int db = 0; db < Dim<D>::kDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[db][i] *= f;
  }
}

// O^T += V^T P^T for one tile; vbuf holds the decoded, transposed V tile.
template <int D>
__device__ __forceinline__ void pv_tile(const uint8_t* vbuf, int c, int hf, const half8_t (&pb)[2][2], State<D>& st) {
  const uint8_t* va = vbuf + c * kVRow + 16 * hf;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < Dim<D>::kDB; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const half8_t a = *reinterpret_cast<const half8_t*>(va + (32 * db) * kVRow + 64 * b + 32 * u);
        st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[b][u], st.acc[db], 0, 0, 0);
      }
}

// First key of key tile t with `tpb` tiles per frame block of fb_keys keys.
__device__ __forceinline__ int tile_key0(int t, int tpb, int fb_keys) {
  if (tpb * kKT == fb_keys) return t * kKT;   // blocks of whole tiles
  const int b = t / tpb;
  return b * fb_keys + (t - b * tpb) * kKT;
}

struct Ctx {
  uint8_t* smem;
  int nt, c, hf, tid, lim, fb_keys, tpb;   // tpb: key tiles per frame block
  float cq;
  const float* kts;
  const float* vts;
};

// Loop iteration t (software-pipelined by one tile on the K side): the scores
// of tile t+1 are computed while tile t's softmax runs, and tile t's P V
// product overlaps the decode of K tile t+2 and V tile t+1 (raw codes loaded
// one iteration earlier), after which K t+3 and V t+2 are loaded.  Buffers:
// K and V tile u live in buffer u & 1; a tile is decoded one iteration after
// the buffer's previous tile was last read, with one barrier per iteration.
template <bool MASK, int D>
__device__ __forceinline__ void step(const Ctx& x, int t, const half8_t (&qf)[Dim<D>::kSteps], const Geo& geo,
                                     Raw<D>& raw, float16_t (&scur)[2], State<D>& st) {
  constexpr int kBuf = Dim<D>::kBuf;
  // VALU instructions placed after each MFMA of the score product: the
  // softmax work of a tile does not depend on D, the MFMA count does
  constexpr int kVpm = 5 * 128 / D;
  uint8_t* b0 = x.smem + (t & 1) * kBuf;        // K t+2 (write), V t (read)
  uint8_t* b1 = x.smem + ((t + 1) & 1) * kBuf;  // K t+1 (read), V t+1 (write)
  const int key0 = tile_key0(t, x.tpb, x.fb_keys);
  const int fb = key0 / x.fb_keys;
  // A new V tensor scale (once per frame block): re-express the accumulator
  // in it.  An all-zero V frame block (scale 0) decodes to zeros and keeps
  // the unit.
  const float sv = x.vts[fb];
  if (sv != 0.0f && sv != st.svref) {
    if (st.svref != 0.0f) rescale(st, st.svref / sv);
    st.svref = sv;
  }
  // Region 1: scores of tile t+1 (MFMA) under the softmax of tile t (VALU).
  // On the last tile the scores are computed from a stale buffer and unused.
  float16_t snext[2];
  qk_tile<D>(b1, x.c, x.hf, qf, snext);
  half8_t pb[2][2];
  // keys past the query's limit or past the frame block's end take no part
  const float f = softmax_tile<MASK, D>(scur, key0, x.hf, x.cq, min(x.lim, (fb + 1) * x.fb_keys), x.kts[fb], st, pb);
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int s = 0; s < Dim<D>::kSteps; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kVpm, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kVpm, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  rescale(st, f);
  // Region 2: P V of tile t (MFMA) under the decode of K t+2 and V t+1 (VALU
  // and LDS writes).  Buffers past the last tile are rewritten harmlessly.
  pv_tile<D>(b0 + Dim<D>::kKBuf, x.c, x.hf, pb, st);
  decode_k<D>(raw, b0, x.tid);
  decode_v<D>(raw, b1, x.tid);
#pragma unroll
  for (int s = 0; s < D / 8; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (t + 3 < x.nt) load_raw_k(geo, tile_key0(t + 3, x.tpb, x.fb_keys), x.tid, raw);
  if (t + 2 < x.nt) load_raw_v(geo, tile_key0(t + 2, x.tpb, x.fb_keys), x.tid, raw);
  __syncthreads();
  scur[0] = snext[0];
  scur[1] = snext[1];
}

template <bool F32OUT, int D>
__global__ __launch_bounds__(256, 2) void kv_attention_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks,
    const float* __restrict__ kts, const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs,
    const float* __restrict__ vts, void* __restrict__ out, int nq, int tokens, int heads, int frames,
    int q_frames, int fb_keys, int qtiles) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Dim<D>::kLds];
  constexpr int kSteps = Dim<D>::kSteps;
  constexpr int kBuf = Dim<D>::kBuf;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hf = lane >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of (head, query tile) so the heads it reads stay in its L2.
  const int n = gridDim.x, w = blockIdx.x;
  const int per = n >> 3, rem = n & 7, x = w & 7;
  const int id = x * per + min(x, rem) + (w >> 3);
  const int h = id / qtiles, qt = id - h * qtiles;

  const int nkeys = frames * tokens;
  const int q0 = qt * kQT;
  const int first_frame = frames - q_frames;
  const int qlast = min(q0 + kQT, nq) - 1;
  const int kmax = (first_frame + qlast / tokens + 1) * tokens;   // no query of the group sees keys >= kmax
  const int tpb = (fb_keys + kKT - 1) / kKT;                      // key tiles per frame block
  const int nt = (kmax / fb_keys) * tpb + (kmax % fb_keys + kKT - 1) / kKT;
  // this wavefront's first query sees keys < kmin_w: tiles below need no mask
  const int qw = min(q0 + 32 * wave, nq - 1);
  const int kmin_w = (first_frame + qw / tokens + 1) * tokens;

  Geo geo{kc, ks, vc, vs, heads, h, nkeys, 0u, {0u, 0u, 0u, 0u}};
  init_geo<D>(geo, tid);

  // The lane's query, converted to fp16 with a per-row power-of-two scale;
  // d of MFMA step s is 16s + 8hf + j.
  const int qi = q0 + 32 * wave + c;
  const bool qvalid = qi < nq;
  const int64_t qrow = (int64_t)qi * heads + h;
  const int lim = qvalid ? (first_frame + qi / tokens + 1) * tokens : kmax;
  half8_t qf[kSteps];
  float cq;
  {
    u32x4_t raw[kSteps];
    float mx = 0.0f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      raw[s] = qvalid ? *reinterpret_cast<const u32x4_t*>(q + qrow * D + 16 * s + 8 * hf) : u32x4_t{0, 0, 0, 0};
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
    cq = ldexpf(Dim<D>::kLog2eRsqrtD, -e);
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qf[s][2 * j] = (_Float16)(bf16_to_f32(raw[s][j] & 0xFFFFu) * sc);
        qf[s][2 * j + 1] = (_Float16)(bf16_to_f32(raw[s][j] >> 16) * sc);
      }
  }

  State<D> st;
  st.m = kMInit;
  st.l = 0.0f;
  st.svref = 0.0f;
#pragma unroll
  for (int db = 0; db < Dim<D>::kDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.acc[db][i] = 0.0f;

  // Prologue: K and V tile 0 and K tile 1 decoded, the scores of tile 0
  // computed, raw codes of K tile 2 and V tile 1 in flight.
  Raw<D> raw;
  load_raw_k<D>(geo, 0, tid, raw);
  load_raw_v<D>(geo, 0, tid, raw);
  decode_k<D>(raw, smem, tid);
  decode_v<D>(raw, smem, tid);
  if (nt > 1) {
    load_raw_k<D>(geo, tile_key0(1, tpb, fb_keys), tid, raw);
    decode_k<D>(raw, smem + kBuf, tid);
  }
  if (nt > 2) load_raw_k<D>(geo, tile_key0(2, tpb, fb_keys), tid, raw);
  if (nt > 1) load_raw_v<D>(geo, tile_key0(1, tpb, fb_keys), tid, raw);
  __syncthreads();
  float16_t scur[2];
  qk_tile<D>(smem, c, hf, qf, scur);
  __syncthreads();   // K tile 0 is read: its buffer is rewritten in the first iteration

  // Tiles wholly below this wavefront's first query limit need no mask; the
  // two kinds run in two loops (one copy of the tile code each).
  const Ctx cx{smem, nt, c, hf, tid, lim, fb_keys, tpb, cq, kts, vts};
  // Tiles wholly below the first query limit are unmasked; with partial
  // block-end tiles only those before the first one (the first block's tiles
  // start at 64 t, so "wholly below" is the same test there).
  int nt_plain = min(kmin_w / kKT, nt);
  if (tpb * kKT != fb_keys) nt_plain = min(nt_plain, tpb - 1);
  int t = 0;
  for (; t < nt_plain; ++t) step<false, D>(cx, t, qf, geo, raw, scur, st);
  for (; t < nt; ++t) step<true, D>(cx, t, qf, geo, raw, scur, st);

  const float l = st.l + __shfl_xor(st.l, 32, 64);
  const float a = st.svref / l;
  if (!qvalid) return;
#pragma unroll
  for (int db = 0; db < Dim<D>::kDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * db + 8 * i4 + 4 * hf;
      const float v0 = st.acc[db][4 * i4] * a, v1 = st.acc[db][4 * i4 + 1] * a;
      const float v2 = st.acc[db][4 * i4 + 2] * a, v3 = st.acc[db][4 * i4 + 3] * a;
      if constexpr (F32OUT) {
        float4_t wv = {v0, v1, v2, v3};
        *reinterpret_cast<float4_t*>(static_cast<float*>(out) + qrow * D + d) = wv;
      } else {
        u32x2_t wv;
        wv[0] = f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16);
        wv[1] = f32_to_bf16_rne(v2) | (f32_to_bf16_rne(v3) << 16);
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + qrow * D + d) = wv;
      }
    }
}

template <int D>
void launch_dim(const uint16_t* q, QOut k, QOut v, void* out, int out_f32, int nq, int tokens, int heads,
                int frames, int q_frames, int fb_keys, int qtiles, hipStream_t s) {
  const int grid = qtiles * heads;
  if (out_f32)
    kv_attention_kernel<true, D><<<grid, 256, 0, s>>>(q, k.codes, k.scales, k.tscale, v.codes, v.scales, v.tscale,
                                                      out, nq, tokens, heads, frames, q_frames, fb_keys, qtiles);
  else
    kv_attention_kernel<false, D><<<grid, 256, 0, s>>>(q, k.codes, k.scales, k.tscale, v.codes, v.scales,
                                                       v.tscale, out, nq, tokens, heads, frames, q_frames, fb_keys,
                                                       qtiles);
}

}  // namespace

hipError_t launch_kv_attention(const uint16_t* q, QOut k, QOut v, void* out, int out_f32, int64_t nq, int64_t tokens,
                               int64_t heads, int64_t head_dim, int64_t frames, int64_t q_frames,
                               int64_t frame_block, hipStream_t s) {
  const int qtiles = (int)((nq + kQT - 1) / kQT);
  const int fb_keys = (int)(frame_block * tokens);
  if (head_dim == 64)
    launch_dim<64>(q, k, v, out, out_f32, (int)nq, (int)tokens, (int)heads, (int)frames, (int)q_frames, fb_keys,
                   qtiles, s);
  else if (head_dim == 128)
    launch_dim<128>(q, k, v, out, out_f32, (int)nq, (int)tokens, (int)heads, (int)frames, (int)q_frames, fb_keys,
                    qtiles, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace nvfp4
