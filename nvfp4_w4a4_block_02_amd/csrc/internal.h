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

// Workgroups of a pass over row domains (the amax pass, which writes one
// partial maximum per workgroup, or the encode pass): every domain but the
// last has rows_per_domain rows and gets `full` workgroups, the last
// (possibly shorter) one gets `last`, on one flat grid of
// (ndom - 1) * full + last workgroups.  The partial maxima of domain d are
// parts[d * full + x], x < (d + 1 < ndom ? full : last).  Final per-domain
// amax values are the case full = last = 1.
struct DomGrid {
  uint32_t full, last, ndom;
  __host__ __device__ inline void locate(uint32_t g, uint32_t& d, uint32_t& x, uint32_t& n) const {
    d = g / full;
    if (d >= ndom) d = ndom - 1;
    x = g - d * full;
    n = d + 1 < ndom ? full : last;
  }
};

// Partial-maximum grids the amax passes below use for a problem.
DomGrid amax_grid_rows(int64_t rows, int64_t cols, int64_t rows_per_domain);
DomGrid amax_grid_cols(int64_t rows, int64_t cols);

// Step 1: partial amax per domain, row layout (also used for axis 0 without
// the transform when cols % 16 == 0, where the amax does not depend on the
// block direction).
hipError_t launch_amax_parts_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  int64_t rows_per_domain, float* parts, DomGrid pg, bool rht,
                                  uint32_t mask, hipStream_t s);
// Step 1 for blocks running down the columns (one domain).
hipError_t launch_amax_parts_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  float* parts, DomGrid pg, bool rht, uint32_t mask, hipStream_t s);
// Reduce the partials of every domain into amax[ndom].
hipError_t launch_reduce_parts(const float* parts, DomGrid pg, float* amax, hipStream_t s);

// Steps 2-6 from per-domain partial maxima laid out as `pg` says.
// four_over_six: Four Over Six block-scale selection (not combined with rht).
// pg_is_amax_grid: `pg` is the grid of the amax pass that just read this
// same tensor (not final per-domain values), which the encode may reuse.
hipError_t launch_encode_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int64_t rows_per_domain, const float* parts, DomGrid pg, QOut out,
                              bool rht, uint32_t mask, hipStream_t s, bool four_over_six = false,
                              bool pg_is_amax_grid = false);
// out_k: length of the output rows (>= rows; blocks past rows are zeroed).
hipError_t launch_encode_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              const float* parts, DomGrid pg, QOut out, bool rht, uint32_t mask,
                              hipStream_t s, int64_t out_k = 0);

// K and V of one cache (bf16, contiguous, same shape) on one launch per
// pass: the amax pass writes each tensor's partial maxima as the one-tensor
// pass would, K's at parts[0, total(pg)) and V's right after them; the
// encode pass reads them back from there.
hipError_t launch_kv_pair_amax(const void* k, const void* v, int64_t rows, int64_t cols, int64_t rows_per_domain,
                               float* parts, DomGrid pg, hipStream_t s);
hipError_t launch_kv_pair_encode(const void* k, const void* v, int64_t rows, int64_t cols,
                                 int64_t rows_per_domain, const float* parts, DomGrid pg, QOut k_out,
                                 QOut v_out, bool four_over_six, hipStream_t s);

// Step 7 for K and V of one cache (same shape) on one launch, bf16 out.
hipError_t launch_kv_pair_dequant(QOut k_in, QOut v_in, int64_t rows, int64_t k, int64_t rows_per_domain,
                                  void* k_out, void* v_out, hipStream_t s);

// Step 7.
hipError_t launch_dequant(QOut in, int64_t rows, int64_t k, int64_t rows_per_domain, void* out,
                          int out_dt, hipStream_t s);

// Block-scaled GEMM; tile_fa/tile_fb = 0 picks the tile shape by cost model.
hipError_t launch_gemm(QOut a, QOut b, int64_t m, int64_t n, int64_t k, void* c, int c_dt,
                       int64_t ldc, int epilogue, float* amax_out, int tile_fa, int tile_fb, hipStream_t s);
bool gemm_tiles_supported(int tile_fa, int tile_fb);

// Frame-causal window attention over an NVFP4 KV cache (head_dim 64 or 128;
// other values return hipErrorInvalidValue without a launch).
hipError_t launch_kv_attention(const uint16_t* q, QOut k, QOut v, void* out, int out_f32, int64_t nq,
                               int64_t tokens, int64_t heads, int64_t head_dim, int64_t frames,
                               int64_t q_frames, int64_t frame_block, hipStream_t s);

}  // namespace nvfp4
