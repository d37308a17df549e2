// C ABI of libnvfp4.so: argument validation (host only, before any HIP call)
// and kernel launches on the caller's stream.  See include/nvfp4.h for the
// contract of every entry point.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "internal.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int64_t kMaxBlocks = (int64_t)1 << 31;  // kernels index 16-element blocks with 32 bits

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int dt) { return dt == NVFP4_F32 || dt == NVFP4_BF16; }

int64_t elem_size(int dt) { return dt == NVFP4_F32 ? 4 : 2; }

// Rows stay 16-byte aligned when ld * elem_size is a multiple of 16.
bool ld_ok(int64_t ld, int dt) { return ld % (16 / elem_size(dt)) == 0; }

// a * b for non-negative sizes, saturated at INT64_MAX instead of
// overflowing, so that absurd arguments fail the size limits below.
int64_t mul_sat(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

int from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP; }

bool tensor_ok(const nvfp4_tensor* t) {
  return t && t->codes && t->scales && t->tscale && aligned16(t->codes) && aligned16(t->scales) &&
         aligned16(t->tscale) && t->rows >= 0 && t->k >= 0 && t->k % 16 == 0;
}

int64_t ndomains(int64_t rows, int64_t rpd) {
  if (rpd <= 0 || rpd > rows) return rows > 0 ? 1 : 0;
  return (rows + rpd - 1) / rpd;
}

nvfp4::QOut qout(const nvfp4_tensor* t) { return nvfp4::QOut{t->codes, t->scales, t->tscale}; }

// Shared checks of a dense input and its NVFP4 output for axis 0 or 1.
int check_dense_to_q(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld, int axis,
                     const nvfp4_tensor* out) {
  if (!x || !valid_dtype(dt) || rows < 0 || cols < 0 || ld < cols || !aligned16(x) || !ld_ok(ld, dt))
    return NVFP4_EINVAL;
  if (!tensor_ok(out)) return NVFP4_EINVAL;
  if (axis == 1) {
    if (cols % 16 != 0 || out->rows != rows || out->k != cols) return NVFP4_EINVAL;
  } else if (axis == 0) {
    if (rows % 16 != 0 || out->rows != cols || out->k < rows) return NVFP4_EINVAL;
  } else {
    return NVFP4_EINVAL;
  }
  if (mul_sat(rows / 16 + 1, cols + 1) > kMaxBlocks || mul_sat(rows, cols / 16 + 1) > kMaxBlocks ||
      mul_sat(out->k / 16 + 1, out->rows + 1) > kMaxBlocks)
    return NVFP4_EUNSUPPORTED;
  return NVFP4_OK;
}

// Scratch of nvfp4_quantize_noalloc: the amax pass's partial maxima of its
// one scaling domain (at most kMaxParts floats), in a device array that each
// GPU holds until the process ends, so that the call allocates nothing.  The
// array's host-side name is not a device address: kernels get the address
// hipGetSymbolAddress returns for the device, looked up once per device and
// cached here.
constexpr size_t kScratchFloats = nvfp4::kMaxParts;  // 4 KiB
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 256;
std::atomic<float*> g_scratch[kMaxDevices];

// Device address of `scratch` on the device that runs `stream` (the current
// device for the NULL stream); nullptr if HIP cannot provide it.  The first
// call for a device looks the address up with that device current.
float* scratch_on(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || addr == nullptr) return nullptr;
  g_scratch[dev].store(static_cast<float*>(addr), std::memory_order_release);
  return static_cast<float*>(addr);
}

}  // namespace

extern "C" {

int nvfp4_version(void) { return kVersion; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument";
    case NVFP4_EUNSUPPORTED: return "unsupported problem size";
    case NVFP4_EWORKSPACE: return "workspace too small";
    case NVFP4_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t nvfp4_workspace_bytes(int op, int64_t rows, int64_t cols) {
  // The amax passes keep at most kMaxParts partial maxima per scaling domain.
  const int64_t per_domain = (int64_t)nvfp4::kMaxParts * 4;
  switch (op) {
    case NVFP4_OP_QUANTIZE:
    case NVFP4_OP_RHT16:
    case NVFP4_OP_AMAX:
      return (size_t)(op == NVFP4_OP_AMAX ? mul_sat(ndomains(rows, cols), per_domain) : per_domain);
    case NVFP4_OP_GEMM:
      return 0;
    case NVFP4_OP_KV_QUANT:
      return (size_t)mul_sat(ndomains(rows, cols), per_domain);
    case NVFP4_OP_KV_QUANT_PAIR:
      return (size_t)mul_sat(2, mul_sat(ndomains(rows, cols), per_domain));
    default:
      return 0;
  }
}

int nvfp4_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
               int64_t rows_per_domain, float* amax, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !amax || !valid_dtype(dtype) || rows < 0 || cols < 0 || cols % 16 != 0 || ld < cols ||
      !aligned16(x) || !ld_ok(ld, dtype) || rows_per_domain < 0)
    return NVFP4_EINVAL;
  if (!ws || !aligned16(ws)) return NVFP4_EINVAL;
  if (ws_bytes < nvfp4_workspace_bytes(NVFP4_OP_AMAX, rows, rows_per_domain)) return NVFP4_EWORKSPACE;
  if (mul_sat(rows, cols / 16) >= kMaxBlocks) return NVFP4_EUNSUPPORTED;
  if (rows == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nd = ndomains(rows, rows_per_domain);
  if (cols == 0) return from_hip(nvfp4::launch_zero(amax, nd, s));
  float* parts = static_cast<float*>(ws);
  const nvfp4::DomGrid pg = nvfp4::amax_grid_rows(rows, cols, rows_per_domain);  // pg.ndom == nd
  if (nvfp4::launch_amax_parts_rows(x, dtype, rows, cols, ld, rows_per_domain, parts, pg, false, 0, s) != hipSuccess)
    return NVFP4_EHIP;
  return from_hip(nvfp4::launch_reduce_parts(parts, pg, amax, s));
}

int nvfp4_encode(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                 int64_t rows_per_domain, const float* amax, const nvfp4_tensor* out, void* stream) {
  if (!amax || rows_per_domain < 0) return NVFP4_EINVAL;
  int st = check_dense_to_q(x, dtype, rows, cols, ld, axis, out);
  if (st != NVFP4_OK) return st;
  if (axis == 0 && rows_per_domain != 0) return NVFP4_EINVAL;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  // one final amax value per domain
  const nvfp4::DomGrid given{1, 1, (uint32_t)ndomains(rows, rows_per_domain)};
  if (axis == 1)
    return from_hip(nvfp4::launch_encode_rows(x, dtype, rows, cols, ld, rows_per_domain, amax, given, qout(out),
                                              false, 0, s));
  return from_hip(nvfp4::launch_encode_cols(x, dtype, rows, cols, ld, amax, given, qout(out), false, 0, s, out->k));
}

static int quantize_impl(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                         bool rht, uint32_t mask, const nvfp4_tensor* out, void* ws, size_t ws_bytes,
                         void* stream) {
  int st = check_dense_to_q(x, dtype, rows, cols, ld, axis, out);
  if (st != NVFP4_OK) return st;
  if (rht && mask > 0xFFFFu) return NVFP4_EINVAL;
  if (!ws || !aligned16(ws)) return NVFP4_EINVAL;
  if (ws_bytes < nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, rows, cols)) return NVFP4_EWORKSPACE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  float* parts = static_cast<float*>(ws);
  hipError_t e;
  nvfp4::DomGrid pg;
  if (axis == 1 || (!rht && cols % 16 == 0)) {
    // Without the transform the amax does not depend on the block direction,
    // and the row pass covers every column when they fill whole 16-element
    // pieces.  Axis 0 accepts any column count: then the column pass, which
    // handles the right edge, takes the amax.
    pg = nvfp4::amax_grid_rows(rows, cols, 0);
    e = nvfp4::launch_amax_parts_rows(x, dtype, rows, cols, ld, 0, parts, pg, rht, mask, s);
  } else {
    pg = nvfp4::amax_grid_cols(rows, cols);
    e = nvfp4::launch_amax_parts_cols(x, dtype, rows, cols, ld, parts, pg, rht, mask, s);
  }
  if (e != hipSuccess) return NVFP4_EHIP;
  if (axis == 1)
    e = nvfp4::launch_encode_rows(x, dtype, rows, cols, ld, 0, parts, pg, qout(out), rht, mask, s, false, true);
  else e = nvfp4::launch_encode_cols(x, dtype, rows, cols, ld, parts, pg, qout(out), rht, mask, s, out->k);
  return from_hip(e);
}

int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                   const nvfp4_tensor* out, void* ws, size_t ws_bytes, void* stream) {
  return quantize_impl(x, dtype, rows, cols, ld, axis, false, 0, out, ws, ws_bytes, stream);
}

int rht16_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                   uint32_t sign_mask, const nvfp4_tensor* out, void* ws, size_t ws_bytes, void* stream) {
  return quantize_impl(x, dtype, rows, cols, ld, axis, true, sign_mask, out, ws, ws_bytes, stream);
}

int nvfp4_quantize_noalloc(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
                           const nvfp4_tensor* out, void* stream) {
  int st = check_dense_to_q(x, dtype, rows, cols, ld, axis, out);
  if (st != NVFP4_OK) return st;
  if (nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, rows, cols) > sizeof(scratch)) return NVFP4_EWORKSPACE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  float* ws = scratch_on(static_cast<hipStream_t>(stream));
  if (ws == nullptr) return NVFP4_EHIP;
  return quantize_impl(x, dtype, rows, cols, ld, axis, false, 0, out, ws, sizeof(scratch), stream);
}

// Host checks of a GEMM call (nothing launched).
static int check_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, const void* c, int c_dtype, int64_t ldc,
                      int epilogue, const float* amax_out) {
  if (!tensor_ok(a) || !tensor_ok(b) || !c || !valid_dtype(c_dtype)) return NVFP4_EINVAL;
  if (a->k != b->k || ldc < b->rows || !aligned16(c)) return NVFP4_EINVAL;
  if (epilogue != NVFP4_EPI_NONE && epilogue != NVFP4_EPI_GELU_TANH) return NVFP4_EINVAL;
  if (amax_out && ((uintptr_t)amax_out & 3u)) return NVFP4_EINVAL;
  if (a->rows >= ((int64_t)1 << 31) || b->rows >= ((int64_t)1 << 31) || a->k >= ((int64_t)1 << 31))
    return NVFP4_EUNSUPPORTED;
  return NVFP4_OK;
}

static int gemm_impl(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int c_dtype, int64_t ldc,
                     int epilogue, float* amax_out, int tile_fa, int tile_fb, void* stream) {
  const int st = check_gemm(a, b, c, c_dtype, ldc, epilogue, amax_out);
  if (st != NVFP4_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (a->rows == 0 || b->rows == 0) {
    return amax_out ? from_hip(nvfp4::launch_zero(amax_out, 1, s)) : NVFP4_OK;
  }
  return from_hip(nvfp4::launch_gemm(qout(a), qout(b), a->rows, b->rows, a->k, c, c_dtype, ldc, epilogue,
                                     amax_out, tile_fa, tile_fb, s));
}

int nvfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int c_dtype, int64_t ldc,
               int epilogue, float* amax_out, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  return gemm_impl(a, b, c, c_dtype, ldc, epilogue, amax_out, 0, 0, stream);
}

int nvfp4_gemm_tiled(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int c_dtype, int64_t ldc,
                     int epilogue, float* amax_out, int tile_fa, int tile_fb, void* stream) {
  if (!nvfp4::gemm_tiles_supported(tile_fa, tile_fb)) return NVFP4_EINVAL;
  return gemm_impl(a, b, c, c_dtype, ldc, epilogue, amax_out, tile_fa, tile_fb, stream);
}

int nvfp4_linear(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, const nvfp4_tensor* w,
                 const nvfp4_tensor* xq, void* c, int c_dtype, int64_t ldc, int epilogue, float* amax_out,
                 void* ws, size_t ws_bytes, void* stream) {
  // Every check of both steps first, so that a bad argument launches nothing.
  int st = check_dense_to_q(x, dtype, rows, cols, ld, 1, xq);
  if (st != NVFP4_OK) return st;
  if (!ws || !aligned16(ws)) return NVFP4_EINVAL;
  if (ws_bytes < nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, rows, cols)) return NVFP4_EWORKSPACE;
  st = check_gemm(xq, w, c, c_dtype, ldc, epilogue, amax_out);
  if (st != NVFP4_OK) return st;
  st = quantize_impl(x, dtype, rows, cols, ld, 1, false, 0, xq, ws, ws_bytes, stream);
  if (st != NVFP4_OK) return st;
  return gemm_impl(xq, w, c, c_dtype, ldc, epilogue, amax_out, 0, 0, stream);
}

static int kv_quant_impl(const void* kv, int64_t frames, int64_t tokens, int64_t heads, int64_t head_dim,
                         int64_t frame_block, const nvfp4_tensor* out, void* ws, size_t ws_bytes, void* stream,
                         bool four_over_six) {
  if (!kv || !aligned16(kv) || frames < 0 || tokens < 0 || heads < 0 || head_dim < 0 || head_dim % 16 != 0 ||
      frame_block <= 0)
    return NVFP4_EINVAL;
  const int64_t rows = mul_sat(mul_sat(frames, tokens), heads);
  if (rows == INT64_MAX || mul_sat(rows, head_dim / 16 + 1) >= kMaxBlocks) return NVFP4_EUNSUPPORTED;
  if (!tensor_ok(out) || out->rows != rows || out->k != head_dim) return NVFP4_EINVAL;
  if (!ws || !aligned16(ws)) return NVFP4_EINVAL;
  if (ws_bytes < nvfp4_workspace_bytes(NVFP4_OP_KV_QUANT, frames, frame_block)) return NVFP4_EWORKSPACE;
  if (rows == 0 || head_dim == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t rpd = (frame_block < frames ? frame_block : frames) * tokens * heads;  // <= rows
  float* parts = static_cast<float*>(ws);
  const nvfp4::DomGrid pg = nvfp4::amax_grid_rows(rows, head_dim, rpd);
  if (nvfp4::launch_amax_parts_rows(kv, NVFP4_BF16, rows, head_dim, head_dim, rpd, parts, pg, false, 0, s) !=
      hipSuccess)
    return NVFP4_EHIP;
  return from_hip(nvfp4::launch_encode_rows(kv, NVFP4_BF16, rows, head_dim, head_dim, rpd, parts, pg,
                                            qout(out), false, 0, s, four_over_six, true));
}

int nvfp4_kv_quant(const void* kv, int64_t frames, int64_t tokens, int64_t heads, int64_t head_dim,
                   int64_t frame_block, const nvfp4_tensor* out, void* ws, size_t ws_bytes, void* stream) {
  return kv_quant_impl(kv, frames, tokens, heads, head_dim, frame_block, out, ws, ws_bytes, stream, false);
}

int nvfp4_kv_quant_4over6(const void* kv, int64_t frames, int64_t tokens, int64_t heads, int64_t head_dim,
                          int64_t frame_block, const nvfp4_tensor* out, void* ws, size_t ws_bytes, void* stream) {
  return kv_quant_impl(kv, frames, tokens, heads, head_dim, frame_block, out, ws, ws_bytes, stream, true);
}

int nvfp4_kv_quant_pair(const void* k, const void* v, int64_t frames, int64_t tokens, int64_t heads,
                        int64_t head_dim, int64_t frame_block, int four_over_six, const nvfp4_tensor* k_out,
                        const nvfp4_tensor* v_out, void* ws, size_t ws_bytes, void* stream) {
  if (!k || !v || !aligned16(k) || !aligned16(v) || frames < 0 || tokens < 0 || heads < 0 || head_dim < 0 ||
      head_dim % 16 != 0 || frame_block <= 0 || (four_over_six != 0 && four_over_six != 1))
    return NVFP4_EINVAL;
  const int64_t rows = mul_sat(mul_sat(frames, tokens), heads);
  if (rows == INT64_MAX || mul_sat(rows, head_dim / 16 + 1) >= kMaxBlocks) return NVFP4_EUNSUPPORTED;
  if (!tensor_ok(k_out) || k_out->rows != rows || k_out->k != head_dim) return NVFP4_EINVAL;
  if (!tensor_ok(v_out) || v_out->rows != rows || v_out->k != head_dim) return NVFP4_EINVAL;
  if (!ws || !aligned16(ws)) return NVFP4_EINVAL;
  if (ws_bytes < nvfp4_workspace_bytes(NVFP4_OP_KV_QUANT_PAIR, frames, frame_block)) return NVFP4_EWORKSPACE;
  if (rows == 0 || head_dim == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t rpd = (frame_block < frames ? frame_block : frames) * tokens * heads;  // <= rows
  float* parts = static_cast<float*>(ws);
  const nvfp4::DomGrid pg = nvfp4::amax_grid_rows(rows, head_dim, rpd);
  if (nvfp4::launch_kv_pair_amax(k, v, rows, head_dim, rpd, parts, pg, s) != hipSuccess) return NVFP4_EHIP;
  return from_hip(nvfp4::launch_kv_pair_encode(k, v, rows, head_dim, rpd, parts, pg, qout(k_out), qout(v_out),
                                               four_over_six == 1, s));
}

int nvfp4_kv_dequant(const nvfp4_tensor* in, int64_t frames, int64_t tokens, int64_t heads, int64_t head_dim,
                     int64_t frame_block, void* out, void* stream) {
  if (!tensor_ok(in) || !out || !aligned16(out) || frames < 0 || tokens < 0 || heads < 0 || frame_block <= 0)
    return NVFP4_EINVAL;
  const int64_t rows = mul_sat(mul_sat(frames, tokens), heads);
  if (rows == INT64_MAX || mul_sat(rows, head_dim / 16 + 1) >= kMaxBlocks) return NVFP4_EUNSUPPORTED;
  if (in->rows != rows || in->k != head_dim) return NVFP4_EINVAL;
  if (rows == 0 || head_dim == 0) return NVFP4_OK;
  const int64_t rpd = (frame_block < frames ? frame_block : frames) * tokens * heads;  // <= rows
  return from_hip(nvfp4::launch_dequant(qout(in), rows, head_dim, rpd, out, NVFP4_BF16, (hipStream_t)stream));
}

int nvfp4_kv_dequant_pair(const nvfp4_tensor* k_in, const nvfp4_tensor* v_in, int64_t frames, int64_t tokens,
                          int64_t heads, int64_t head_dim, int64_t frame_block, void* k_out, void* v_out,
                          void* stream) {
  if (!tensor_ok(k_in) || !tensor_ok(v_in) || !k_out || !v_out || !aligned16(k_out) || !aligned16(v_out) ||
      frames < 0 || tokens < 0 || heads < 0 || frame_block <= 0)
    return NVFP4_EINVAL;
  const int64_t rows = mul_sat(mul_sat(frames, tokens), heads);
  if (rows == INT64_MAX || mul_sat(rows, head_dim / 16 + 1) >= kMaxBlocks) return NVFP4_EUNSUPPORTED;
  if (k_in->rows != rows || k_in->k != head_dim || v_in->rows != rows || v_in->k != head_dim) return NVFP4_EINVAL;
  if (rows == 0 || head_dim == 0) return NVFP4_OK;
  const int64_t rpd = (frame_block < frames ? frame_block : frames) * tokens * heads;  // <= rows
  return from_hip(nvfp4::launch_kv_pair_dequant(qout(k_in), qout(v_in), rows, head_dim, rpd, k_out, v_out,
                                                (hipStream_t)stream));
}

int nvfp4_kv_attention(const void* q, int64_t q_frames, const nvfp4_tensor* k, const nvfp4_tensor* v,
                       int64_t frames, int64_t tokens, int64_t heads, int64_t head_dim, int64_t frame_block,
                       void* out, int out_dtype, void* stream) {
  if (!q || !out || !aligned16(q) || !aligned16(out) || !valid_dtype(out_dtype) || frames < 0 || tokens < 0 ||
      heads < 0 || head_dim < 0 || head_dim % 16 != 0 || frame_block <= 0 || q_frames < 0 || q_frames > frames)
    return NVFP4_EINVAL;
  const int64_t rows = mul_sat(mul_sat(frames, tokens), heads);
  // 32-bit offsets: code bytes of the cache and the workgroup count
  if (mul_sat(rows, head_dim / 2) >= ((int64_t)1 << 31)) return NVFP4_EUNSUPPORTED;
  if (!tensor_ok(k) || !tensor_ok(v) || k->rows != rows || v->rows != rows || k->k != head_dim ||
      v->k != head_dim)
    return NVFP4_EINVAL;
  const int64_t nq = q_frames * tokens;  // <= rows
  if (nq == 0 || heads == 0) return NVFP4_OK;
  if (head_dim != 64 && head_dim != 128) return NVFP4_EUNSUPPORTED;
  if (((nq + 127) / 128) * heads >= ((int64_t)1 << 31)) return NVFP4_EUNSUPPORTED;
  // One frame block covers the whole window when frame_block >= frames (as
  // in nvfp4_kv_dequant); the kernel then sees at most frames * tokens keys
  // per block.
  const int64_t fb = frame_block < frames ? frame_block : frames;
  return from_hip(nvfp4::launch_kv_attention(static_cast<const uint16_t*>(q), qout(k), qout(v), out,
                                             out_dtype == NVFP4_F32, nq, tokens, heads, head_dim, frames,
                                             q_frames, fb, (hipStream_t)stream));
}

int nvfp4_dequantize(const nvfp4_tensor* in, int64_t rows_per_domain, void* out, int dtype, void* stream) {
  if (!tensor_ok(in) || !out || !aligned16(out) || !valid_dtype(dtype) || rows_per_domain < 0)
    return NVFP4_EINVAL;
  if (mul_sat(in->rows, in->k / 16 + 1) >= kMaxBlocks) return NVFP4_EUNSUPPORTED;
  if (in->rows == 0 || in->k == 0) return NVFP4_OK;
  return from_hip(nvfp4::launch_dequant(qout(in), in->rows, in->k, rows_per_domain, out, dtype,
                                        (hipStream_t)stream));
}

}  // extern "C"
