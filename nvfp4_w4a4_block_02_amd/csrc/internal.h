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

// Step 1: per-domain amax, axis-1 blocks (or plain magnitudes when !rht).
hipError_t launch_amax_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                            int64_t rows_per_domain, float* amax, bool rht, uint32_t mask,
                            hipStream_t s);
// Step 1 for RHT along axis 0 (blocks run down columns).
hipError_t launch_amax_cols_rht(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                float* amax, uint32_t mask, hipStream_t s);

// Steps 2-6.
hipError_t launch_encode_rows(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int64_t rows_per_domain, const float* amax, QOut out, bool rht,
                              uint32_t mask, hipStream_t s);
hipError_t launch_encode_cols(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              const float* amax, QOut out, bool rht, uint32_t mask, hipStream_t s);

// Step 7.
hipError_t launch_dequant(QOut in, int64_t rows, int64_t k, int64_t rows_per_domain, void* out,
                          int out_dt, hipStream_t s);

// Block-scaled GEMM.
hipError_t launch_gemm(QOut a, QOut b, int64_t m, int64_t n, int64_t k, void* c, int c_dt,
                       int64_t ldc, int epilogue, float* amax_out, hipStream_t s);

}  // namespace nvfp4
