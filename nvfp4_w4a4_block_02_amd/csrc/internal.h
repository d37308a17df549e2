// Internal launch interface between the C ABI layer (api.hip) and the kernel
// files.  Arguments are validated by the caller; these functions only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

struct QOut {            // device pointers of an NVFP4 output / input
  uint8_t* codes;
  uint8_t* scales;
  float* tscale;
};

// Zero `n` floats (a fill kernel rather than hipMemsetAsync, so the sequence
// stays valid inside captured graphs).
hipError_t launch_zero(float* p, int64_t n, hipStream_t s);

// Partial maxima: the amax pass writes one float per workgroup and domain;
// consumers reduce at most kMaxParts of them per domain.
constexpr uint32_t kMaxParts = 1024;

// Number of partials the amax passes below use for a problem.
uint32_t amax_parts_rows(int64_t rows, int64_t cols, int64_t rows_per_domain);
uint32_t amax_parts_cols(int64_t rows, int64_t cols);

// Step 1: partial amax per domain, row layout (also used for axis 0 without
// the transform, where the amax does not depend on the block direction);
// parts[d * nparts + w].
hipError_t launch_amax_parts_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  int64_t rows_per_domain, float* parts, uint32_t nparts, bool rht,
                                  uint32_t mask, hipStream_t s);
// Step 1 for blocks running down the columns (one domain), needed with the RHT.
hipError_t launch_amax_parts_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  float* parts, uint32_t nparts, bool rht, uint32_t mask, hipStream_t s);
// Reduce `nparts` partials per domain into amax[ndom].
hipError_t launch_reduce_parts(const float* parts, uint32_t nparts, int64_t ndom, float* amax, hipStream_t s);

// Steps 2-6 from per-domain partial maxima (nparts = 1: final amax values).
// four_over_six: Four Over Six block-scale selection (not combined with rht).
hipError_t launch_encode_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int64_t rows_per_domain, const float* parts, uint32_t nparts, QOut out,
                              bool rht, uint32_t mask, hipStream_t s, bool four_over_six = false);
// out_k: length of the output rows (>= rows; blocks past rows are zeroed).
hipError_t launch_encode_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              const float* parts, uint32_t nparts, QOut out, bool rht, uint32_t mask,
                              hipStream_t s, int64_t out_k = 0);

// Step 7.
hipError_t launch_dequant(QOut in, int64_t rows, int64_t k, int64_t rows_per_domain, void* out,
                          int out_dt, hipStream_t s);

// Block-scaled GEMM; tile_fa/tile_fb = 0 picks the tile shape by cost model.
hipError_t launch_gemm(QOut a, QOut b, int64_t m, int64_t n, int64_t k, void* c, int c_dt,
                       int64_t ldc, int epilogue, float* amax_out, int tile_fa, int tile_fb, hipStream_t s);
bool gemm_tiles_supported(int tile_fa, int tile_fb);

// Frame-causal window attention over an NVFP4 KV cache (head_dim 128).
hipError_t launch_kv_attention(const uint16_t* q, QOut k, QOut v, void* out, int out_f32, int64_t nq,
                               int64_t tokens, int64_t heads, int64_t frames, int64_t q_frames,
                               int64_t frame_block, hipStream_t s);

}  // namespace nvfp4
