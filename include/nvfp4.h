/*
 * nvfp4.h — C ABI of the MI355X (gfx950) NVFP4 W4A4 library (libnvfp4.so).
 *
 * Format (what every entry point reads or writes).  NVFP4 stores each element
 * as a 4-bit E2M1 code (sign, 2 exponent bits, 1 mantissa bit; magnitudes
 * 0, .5, 1, 1.5, 2, 3, 4, 6), one FP8 block scale per 16 consecutive elements
 * and one FP32 scale per tensor — neurohive.io, "LongLive-2.0: NVIDIA научила
 * модель генерировать длинное видео в реальном времени с квантованием NVFP4",
 * section "Ключевые компоненты LongLive-2.0" (NVFP4 paragraph), and
 * tailorednewshub.com, "LongLive-2.0: Infraestructura paralela NVFP4 para
 * video largo", section "Entrenamiento NVFP4" (FP8 block / FP32 tensor
 * scale).  Readings where the pages are silent, fixed by this library:
 *
 *   - the FP8 block scale is OCP E4M3FN (bias 7, max 448, no infinities);
 *   - domain amax A, tensor scale S = A / 2688 (2688 = 6 * 448);
 *   - block scale s_b = E4M3_RNE_satfinite((max|x| over the block / 6) / S);
 *   - element code = sign(x) | E2M1_RNE_satfinite(|x| * (1 / (f32(s_b) * S)));
 *     a negative value that rounds to zero keeps its sign (code 0x8);
 *   - all scale arithmetic is IEEE float32 with correctly rounded division;
 *   - decode: x' = f32(e2m1 * s_b) * S (the first product is exact).
 *
 * Memory layout of an NVFP4 tensor of `rows` x `k` (blocks run along k):
 *   codes  [rows][k/2] bytes, byte j = code[2j] | code[2j+1] << 4;
 *   scales [rows][k/16] E4M3FN bytes, row-major, no swizzle;
 *   tscale one float32 S per scaling domain (1 for a plain tensor).
 * Storage is 4.5 bits per element, i.e. 3.56x smaller than bf16 (the pages
 * report about 3.6x for the NVFP4 KV cache: tailorednewshub.com, section
 * "Inferencia W4A4 NVFP4").
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller owns every buffer (inputs, outputs, workspace).
 *     The library never allocates or frees memory.  Apart from the 4 KiB
 *     per-GPU scratch array of nvfp4_quantize_noalloc it keeps no mutable
 *     global state, so concurrent calls on different streams are safe as
 *     long as their buffers do not overlap.
 *   - Pointers named x / c / out / codes / scales / tscale / amax / ws are
 *     DEVICE pointers; the nvfp4_tensor structs themselves live in HOST memory
 *     and are read before the call returns.
 *   - Asynchrony: every call enqueues its kernels on `stream` (a hipStream_t;
 *     NULL = the default stream) and returns without synchronizing.  Results
 *     are visible after the caller synchronizes that stream.
 *   - Errors: argument problems are detected on the host before any HIP call
 *     and return NVFP4_EINVAL (null pointer, k % 16 != 0, ld < cols,
 *     misalignment, mismatched operands, unknown dtype/flag); a workspace that
 *     is too small returns NVFP4_EWORKSPACE; problems beyond the kernels'
 *     32-bit indexing (2^31 16-element blocks per tensor; GEMM dimensions of
 *     2^31 or more) return NVFP4_EUNSUPPORTED, as do shapes whose size
 *     products overflow 64 bits; a failed launch returns NVFP4_EHIP.
 *     Zero-sized problems return NVFP4_OK without launching.
 *   - Inputs must be finite.  Non-finite inputs give unspecified codes; there
 *     is no check on the device.  Tensors whose amax is below about 2^-100
 *     (where 1/(s_b * S) overflows float32) also give unspecified codes.
 *   - Alignment: device pointers must be 16-byte aligned; the leading
 *     dimension of an input (in elements) must keep every row 16-byte aligned
 *     (bf16: ld % 8 == 0; float32: ld % 4 == 0).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NVFP4_OK            0
#define NVFP4_EINVAL       -1
#define NVFP4_EUNSUPPORTED -2
#define NVFP4_EWORKSPACE   -3
#define NVFP4_EHIP         -4

/* Element types of dense (non-NVFP4) tensors. */
#define NVFP4_F32  0
#define NVFP4_BF16 1

/* GEMM epilogues. */
#define NVFP4_EPI_NONE      0
#define NVFP4_EPI_GELU_TANH 1

/* Workspace queries (nvfp4_workspace_bytes `op`). */
#define NVFP4_OP_QUANTIZE 0
#define NVFP4_OP_RHT16    1
#define NVFP4_OP_GEMM     2
#define NVFP4_OP_KV_QUANT 3
#define NVFP4_OP_AMAX     4
#define NVFP4_OP_KV_QUANT_PAIR 5

/* An NVFP4 tensor (host struct holding device pointers), layout above. */
typedef struct {
  uint8_t *codes;   /* device, [rows][k/2]                      */
  uint8_t *scales;  /* device, [rows][k/16] E4M3FN               */
  float   *tscale;  /* device, [n_domains] float32 tensor scales */
  int64_t  rows;
  int64_t  k;       /* multiple of 16                            */
} nvfp4_tensor;

/* Library version (major * 10000 + minor * 100 + patch). */
int nvfp4_version(void);

/* Human-readable text of a status code (static string, never NULL). */
const char *nvfp4_status_string(int status);

/* Bytes of device workspace `op` needs for a rows x cols problem (for
 * NVFP4_OP_KV_QUANT and NVFP4_OP_KV_QUANT_PAIR: rows = frames,
 * cols = frame_block; for NVFP4_OP_AMAX:
 * cols = rows_per_domain).  The workspace holds the partial maxima of the
 * amax pass (4 KiB per scaling domain); it must be 16-byte aligned and its
 * contents on entry do not matter.  Calls that share a workspace must not
 * overlap in time. */
size_t nvfp4_workspace_bytes(int op, int64_t rows, int64_t cols);

/*
 * Domain amax (step 1 of the recipe): the FP32 tensor scale of NVFP4 is
 * derived from the largest magnitude of its scaling domain (neurohive.io NVFP4
 * paragraph: a per-tensor scale beside the 16-element block scales; hyper.ai
 * LongLive-2.0 summary, "方法": one domain per 8-frame block of the KV cache).
 * amax[d] = max |x| over the rows of domain d, where domain d is rows [d*rows_per_domain, (d+1)*rows_per_domain)
 * (the last domain may be shorter; rows_per_domain = 0 means one domain).
 * x: device [rows][ld] of `dtype`.  amax: device float32
 * [ceil(rows/rows_per_domain)], overwritten.  The maximum is exact and does
 * not depend on thread scheduling (partial maxima, no atomics).
 * ws: >= nvfp4_workspace_bytes(NVFP4_OP_AMAX, rows, rows_per_domain).
 */
int nvfp4_amax(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
               int64_t rows_per_domain, float *amax, void *ws, size_t ws_bytes, void *stream);

/*
 * Encode (steps 2-6) given each domain's amax: writes codes, block scales
 * and tscale[d] = amax[d] / 2688 — the E2M1 elements with one FP8 scale per
 * 16 elements and one FP32 scale per domain of the NVFP4 format (neurohive.io
 * NVFP4 paragraph; tailorednewshub.com, "Entrenamiento NVFP4").  Split from
 * nvfp4_quantize so that a caller holding the amax already (the GEMM
 * epilogue's max |H|, a weight quantized along both dims) skips its pass.
 *   axis = 1: blocks run along cols (x is [rows][cols], K-contiguous); the
 *             output is rows x cols.
 *   axis = 0: blocks run along rows (x's reduction dim is dim 0, as for a
 *             weight gradient); the output is stored transposed, cols x
 *             out->k, and rows_per_domain must be 0.  out->k may exceed rows
 *             (a multiple of 16): the blocks past rows get zero codes and
 *             zero scales, which decode to 0 and leave a GEMM over the padded
 *             reduction dimension unchanged (nvfp4_gemm runs its fastest path
 *             when K >= 512 and K % 256 == 0).
 * `out` must describe the output shape exactly (for axis 1: rows x cols);
 * out->tscale needs one float per domain.
 */
int nvfp4_encode(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 int axis, int64_t rows_per_domain, const float *amax,
                 const nvfp4_tensor *out, void *stream);

/*
 * Quantize a whole tensor (one domain): nvfp4_amax into the workspace, then
 * nvfp4_encode.  ws: device, >= nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, ...).
 * This is the activation (and offline weight) quantizer of the W4A4 linear
 * layers (tailorednewshub.com, section "Inferencia W4A4 NVFP4").
 */
int nvfp4_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                   int axis, const nvfp4_tensor *out, void *ws, size_t ws_bytes,
                   void *stream);

/*
 * nvfp4_quantize without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The amax pass's partial maxima go to a
 * 4 KiB device array inside the library instead, one per GPU, held until the
 * process ends; its device address is looked up once per device, on the
 * first call for the device that runs `stream`, and no call allocates.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams) race, and the caller must serialize them.
 * Nothing in the array needs clearing (each call writes every partial it
 * reads).  The array holds the partial maxima of every tensor
 * nvfp4_quantize accepts (at most 1024 floats), so no valid size is refused
 * for lack of room (that check returns NVFP4_EWORKSPACE); NVFP4_EHIP if the
 * array's address cannot be obtained.  Arguments, results and the other
 * errors as nvfp4_quantize.
 */
int nvfp4_quantize_noalloc(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                           int axis, const nvfp4_tensor *out, void *stream);

/*
 * Random Hadamard transform then quantize (gradient path: the pages apply an
 * RHT before quantizing weight gradients — neurohive.io NVFP4 paragraph;
 * tailorednewshub.com, "Entrenamiento NVFP4").  Every 16-element block v
 * along `axis` becomes v' = (1/4) * H16 * diag(d) * v, with H16 the Sylvester
 * Hadamard matrix and d_j = -1 iff bit j of sign_mask is set (one mask for
 * the whole tensor), evaluated in float32 as: sign flip, butterfly stages of
 * stride 1, 2, 4, 8 ((a, b) -> (a + b, a - b)), multiply by 0.25.  The amax
 * and all scales are those of the transformed tensor.  Axis and layout as in
 * nvfp4_encode.  ws: >= nvfp4_workspace_bytes(NVFP4_OP_RHT16, ...).
 */
int rht16_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                   int axis, uint32_t sign_mask, const nvfp4_tensor *out,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * Block-scaled W4A4 GEMM (tailorednewshub.com, "Inferencia W4A4 NVFP4": FP4
 * GEMMs replace BF16 GEMMs):
 *   c[m][n] = epi( S_A * S_B * sum_k P_A[m][k] * P_B[n][k] ),
 *   P = e2m1(code) * f32(s_b)  (decoded exactly), float32 accumulation.
 * a: M x K (a->rows = M), b: N x K (b->rows = N, a linear layer's weight),
 * both with one tscale.  c: device [M][ldc] of c_dtype (float32 or bf16,
 * round-to-nearest-even), ldc >= N.  epilogue: NVFP4_EPI_NONE or
 * NVFP4_EPI_GELU_TANH (0.5 h (1 + tanh(0.79788456 (h + 0.044715 h^3))),
 * float32).  amax_out: NULL, or a device float that receives max |c| over the
 * stored values (it is reset by the call), so that c can be re-quantized with
 * nvfp4_encode without another pass over it.  ws may be NULL
 * (nvfp4_workspace_bytes(NVFP4_OP_GEMM, ...) is 0).  The tile shape is
 * chosen per problem; when the last row of tiles is mostly empty, the call
 * may run the full tile rows and the remaining rows as two kernels on
 * `stream` (same values as one kernel; the amax covers both).
 */
int nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype,
               int64_t ldc, int epilogue, float *amax_out, void *ws, size_t ws_bytes,
               void *stream);

/*
 * nvfp4_gemm with an explicit tile shape instead of the built-in choice (the
 * same W4A4 GEMM: tailorednewshub.com, "Inferencia W4A4 NVFP4").
 * tile_fa x tile_fb is the number of 32x32 MFMA fragments per wavefront
 * along M x N (a workgroup covers 64*tile_fa x 64*tile_fb outputs); the
 * supported shapes are 2x4, 4x2, 3x3, 4x4 and 1x1, used when K >= 512 and
 * K % 256 == 0 (other K always take the bounds-checked 2x4 kernel).  Every
 * shape accumulates each output element in the same order, so results are
 * bit-identical across shapes.  Unsupported shapes return NVFP4_EINVAL.
 * Intended for tuning and testing.
 */
int nvfp4_gemm_tiled(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype,
                     int64_t ldc, int epilogue, float *amax_out, int tile_fa, int tile_fb,
                     void *stream);

/*
 * One W4A4 linear layer in one call (tailorednewshub.com, "Inferencia W4A4
 * NVFP4": the activations are quantized to NVFP4 on the fly and the layer's
 * GEMM runs on NVFP4 weights): the activation quantize of x [rows, cols]
 * (float32 or bf16, blocks along cols, i.e. nvfp4_quantize with axis 1)
 * into xq, then c = epi(xq @ w^T) (nvfp4_gemm with a = xq, b = w).  The
 * results and the codes left in xq are those of the two calls; every
 * argument of both is checked before anything is launched (xq must be
 * rows x cols, w must have k = cols).  ws: >= nvfp4_workspace_bytes(
 * NVFP4_OP_QUANTIZE, rows, cols).  One host call instead of two, for
 * latency-bound small layers.
 */
int nvfp4_linear(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 const nvfp4_tensor *w, const nvfp4_tensor *xq, void *c, int c_dtype,
                 int64_t ldc, int epilogue, float *amax_out, void *ws, size_t ws_bytes,
                 void *stream);

/*
 * KV-cache quantization in frame blocks (hyper.ai summary of the LongLive-2.0
 * paper, section "方法": the KV cache is quantized per block of eight frames).
 * kv: device bf16 [frames][tokens][heads][head_dim], contiguous.  One tscale
 * per frame block (frames [b*frame_block, (b+1)*frame_block), the last block
 * may be partial) over all its tokens and heads; 16-element blocks along
 * head_dim.  out: rows = frames*tokens*heads, k = head_dim, tscale holds
 * ceil(frames/frame_block) floats.
 * ws: >= nvfp4_workspace_bytes(NVFP4_OP_KV_QUANT, frames, frame_block).
 */
int nvfp4_kv_quant(const void *kv, int64_t frames, int64_t tokens, int64_t heads,
                   int64_t head_dim, int64_t frame_block, const nvfp4_tensor *out,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * nvfp4_kv_quant with the Four Over Six encoder (tailorednewshub.com,
 * "Inferencia W4A4 NVFP4": the NVFP4 KV cache uses adaptive scale selection
 * under that name; the pages give nothing beyond the name).  Reading
 * implemented: same format, tensor scales and decode as nvfp4_kv_quant; for
 * every 16-element block two candidates are encoded, one whose scale maps the
 * block maximum to 6 (the core recipe) and one mapping it to 4
 * (s_b = E4M3((max|x| / 4) / S)), and the stored one is the candidate with
 * the strictly smaller squared decode error
 * E = sum_i (x_i - f32(e2m1_i * s_b) * S)^2, each operation a separately
 * rounded float32 operation summed from element 0 to 15 (ties keep the core
 * recipe).  Arguments, layout, workspace and errors as nvfp4_kv_quant.
 */
int nvfp4_kv_quant_4over6(const void *kv, int64_t frames, int64_t tokens, int64_t heads,
                          int64_t head_dim, int64_t frame_block, const nvfp4_tensor *out,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * K and V of one cache in one call (the pages quantize both halves of the KV
 * cache in 8-frame blocks: hyper.ai summary, section "方法"): the same codes,
 * block scales and tensor scales as nvfp4_kv_quant (four_over_six = 0) or
 * nvfp4_kv_quant_4over6 (four_over_six = 1) called on k into k_out and on v
 * into v_out, with the amax pass of both tensors in one launch and the encode
 * pass of both in another (two launches instead of four).  k and v: device
 * bf16 [frames][tokens][heads][head_dim], contiguous, same shape; k_out and
 * v_out must not overlap.
 * ws: >= nvfp4_workspace_bytes(NVFP4_OP_KV_QUANT_PAIR, frames, frame_block)
 * (twice the one-tensor workspace).  Other values of four_over_six return
 * NVFP4_EINVAL; errors otherwise as nvfp4_kv_quant.
 */
int nvfp4_kv_quant_pair(const void *k, const void *v, int64_t frames, int64_t tokens,
                        int64_t heads, int64_t head_dim, int64_t frame_block, int four_over_six,
                        const nvfp4_tensor *k_out, const nvfp4_tensor *v_out, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * KV-cache dequantization of the whole window to bf16 (the pages rebuild the
 * cache with a parallel dequant kernel for window attention: hyper.ai
 * summary, section "方法").  out: device bf16 [frames][tokens][heads][head_dim].
 */
int nvfp4_kv_dequant(const nvfp4_tensor *in, int64_t frames, int64_t tokens, int64_t heads,
                     int64_t head_dim, int64_t frame_block, void *out, void *stream);

/*
 * K and V of one cache decoded in one launch (the pages' dequant of the
 * NVFP4 KV window: hyper.ai summary, section "方法"): the same bf16 values as
 * nvfp4_kv_dequant on k_in into k_out and on v_in into v_out.  Both inputs
 * describe [frames][tokens][heads][head_dim] with the same frame_block.
 */
int nvfp4_kv_dequant_pair(const nvfp4_tensor *k_in, const nvfp4_tensor *v_in, int64_t frames,
                          int64_t tokens, int64_t heads, int64_t head_dim, int64_t frame_block,
                          void *k_out, void *v_out, void *stream);

/*
 * Frame-causal window attention that reads the NVFP4 KV cache directly (the
 * consumer of the cache: 9 local latent frames plus 3 sink frames kept in the
 * cache, 171host.com "LongLive 2.0 技术拆解", section 2.2; NVFP4 cache in
 * 8-frame blocks, hyper.ai LongLive-2.0 summary, "方法").  K and V tiles are
 * decoded in on-chip memory inside the attention loop; no bf16 copy of the
 * window is written.
 *
 *   q    device bf16 [q_frames * tokens][heads][head_dim], contiguous: the
 *        queries of the last q_frames frames of the window (the chunk being
 *        generated);
 *   k, v NVFP4 caches as written by nvfp4_kv_quant / nvfp4_kv_quant_4over6
 *        (rows = frames * tokens * heads, k = head_dim, one tensor scale per
 *        frame block);
 *   out  device [q_frames * tokens][heads][head_dim], out_dtype NVFP4_F32 or
 *        NVFP4_BF16 (round-to-nearest-even), contiguous.
 *
 * Query i sits in window frame f = frames - q_frames + i / tokens and attends
 * to every key of frames 0..f (its own frame included, no later frame):
 *   out[i][h] = sum_j softmax_j(q[i][h] . K[j][h] / sqrt(head_dim)) V[j][h],
 * K, V = e2m1 * s_b * S exactly.  Products run on fp16 MFMA with float32
 * accumulation (decoded elements are exact in fp16; q enters with a per-row
 * power-of-two scale); probabilities are rounded to fp16.  Results agree with
 * an exact computation to about 2^-10 of sum_j p_j |V_j| / sum_j p_j per
 * element (plus the bf16 rounding of the output), except where the output is
 * carried by keys weighted below about 2^-24 of the largest (fp16's
 * subnormal range): there the error can reach 2^-25 sum_j |V_j| / L over
 * those keys, L = sum_j p_j / max_j p_j.
 *
 * Frame blocks may hold any number of keys (frame_block * tokens); a
 * frame_block >= frames means one block over the whole window, as in
 * nvfp4_kv_dequant.  Limits: head_dim must be 64 or 128 (else
 * NVFP4_EUNSUPPORTED); 1 <= q_frames <= frames; the cache's code bytes
 * (frames * tokens * heads * head_dim / 2) below 2^31.  A non-finite value anywhere in the keys a
 * workgroup of 128 queries scans can propagate to its outputs.  No workspace.
 */
int nvfp4_kv_attention(const void *q, int64_t q_frames, const nvfp4_tensor *k, const nvfp4_tensor *v,
                       int64_t frames, int64_t tokens, int64_t heads, int64_t head_dim,
                       int64_t frame_block, void *out, int out_dtype, void *stream);

/*
 * Plain dequantization, the format's decode x' = f32(e2m1 * s_b) * S
 * (neurohive.io NVFP4 paragraph: E2M1 values, FP8 block and FP32 tensor
 * scales; the same decode the KV dequantizer applies, hyper.ai LongLive-2.0
 * summary, "方法"), float32 or bf16 (round-to-nearest-even) output
 * [rows][k], contiguous; rows_per_domain as in nvfp4_amax (0 = one domain).
 */
int nvfp4_dequantize(const nvfp4_tensor *in, int64_t rows_per_domain, void *out,
                     int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
