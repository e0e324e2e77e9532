/*
 * moe_nvfp4.h -- C-ABI of libmoe_nvfp4.so: one MoE layer's NVFP4 routed-expert
 * computation on an AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on four pages of the vLLM API reference:
 *   [expert_tp]      vllm.models.muse_spark.nvidia.specialized_decode.runtime.expert_tp
 *   [flashinfer_ops] vllm.models.muse_spark.nvidia.specialized_decode.runtime.flashinfer_ops
 *   [runner]         vllm.models.muse_spark.nvidia.muse_moe_runner
 *   [model]          vllm.models.muse_spark.nvidia.model
 * A layer runs, on one stream, in this order:
 *   moe_route -> nvfp4_quant -> moe_experts_fwd -> moe_finalize
 * (moe_route_quant is the first two in one launch)
 * (the model page, "_prepared_nvfp4_forward", prepares the quantized input and
 * the routing; the runner page, "MuseSparkTrtLlmNvFp4Experts.apply_routed", runs
 * the experts up to the GEMM2 rows and hands them to "MusePostExpertFinalize").
 *
 * Conventions for every call
 *   - Pointers named in the comments as "device" point to device memory of the
 *     current HIP device; the caller allocates, owns and frees all of it. The
 *     library allocates, frees and synchronizes nothing: a call validates its
 *     arguments on the host, enqueues its kernels on `stream` (a hipStream_t,
 *     NULL = the default stream) and returns. Nothing is read back to the host,
 *     so every call can be captured into a HIP graph.
 *   - Device pointers must be 16-byte aligned.
 *   - Return 0 on success or a negative MOE_E* code. Validation happens before
 *     any launch, so a refused call leaves no partial work. moe_last_error()
 *     returns the calling thread's message for its last failed call.
 *   - Sizes are in elements unless named *_bytes or *_stride_bytes.
 *   - bf16 values are passed as their uint16 bit patterns; e4m3 scales as
 *     bytes (OCP float8 e4m3fn: bias 7, max 448, 0x7F/0xFF NaN).
 *
 * NVFP4 as this library stores it (the expert_tp page, "StockNvfp4"): two e2m1
 * codes per byte, element 2j in the low nibble of byte j; one e4m3 scale per 16
 * consecutive elements of a row; plus one fp32 global scale per tensor.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_NVFP4_ABI_VERSION 8

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null pointer, bad size, stride or alignment */
#define MOE_EUNSUPPORTED (-2) /* a shape the kernels do not take (divisibility, limits) */
#define MOE_ELAUNCH (-3)      /* a HIP launch failed */

/* Limits of this build. */
#define MOE_MAX_EXPERTS 1024  /* E and E_local */
#define MOE_MAX_TOPK 32
#define MOE_MAX_HIDDEN 16384  /* H, and I in moe_experts_fwd */

int moe_abi_version(void);
const char* moe_last_error(void);

/* ------------------------------------------------------------------ sizing
 * rows_max: the padded permuted rows a routing of T tokens x K routes over
 * E_local experts can need with tile m:
 *   (min(E_local, T*K) + (T*K - min(E_local, T*K)) / m) * m
 * -- the bound of the flashinfer_ops page, "gemm2_rows", without that op's
 * 128 KiB floor. Returns -1 for invalid arguments. */
int64_t moe_rows_max(int T, int K, int E_local, int tile_m);

/* The int32 routing-metadata buffer written by moe_route and read by
 * moe_experts_fwd / moe_finalize. Fields are indices into the buffer (int32
 * units); every field starts at a multiple of 64. Contents after moe_route:
 *   num_tiles       [1]          tiles holding routes (sum over experts of ceil(count/m))
 *   total_rows      [1]          num_tiles * m
 *   expert_offsets  [E_local+1]  first permuted row of each local expert; last = total_rows
 *   expert_counts   [E_local]    routes per local expert
 *   exp2perm        [T*K]        permuted row of route t*K+k, or -1 (padding token
 *                                or expert not local: "not served here")
 *   perm2tok        [rows_max]   token of each permuted row; -1 for padding rows
 *                                and for every row >= total_rows
 *   tile_expert     [rows_max/m] local expert of each tile; -1 beyond num_tiles
 *   sync_status     [1]          0; moe_experts_fwd sets 1 if one of its waits
 *                                gave up: its intermediate and rows are then NOT
 *                                valid, and neither is anything computed from them
 *                                (a caller that cannot rule this out reads the word
 *                                after the stream completes and drops the results)
 *   sub_sync        [256*subs_max] (subs_max = rows_max/16): two counters per
 *                                16-row tile s, at 256*s and 256*s + 1 (1 KB
 *                                apart, so that the polls on different tiles
 *                                spread over memory channels), set to 0 by
 *                                moe_route; moe_experts_fwd's one-launch form
 *                                uses them and leaves them at 0 again. The
 *                                other words are not used.
 *   tok_sync        [32*T]       three counters per token t, at 32*t .. 32*t + 2
 *                                (128 bytes apart), set to 0 by moe_route; the
 *                                one-launch form of moe_experts_finalize uses them
 *                                and leaves them at 0 again. The other words are
 *                                not used.
 *   fin_part        [128*T]      that form's working space: per token, the fp32
 *                                partial sums of squares its workgroups exchange
 *   perm_counts     [ceil(T*K/512) * E_local]  moe_route's working space when it
 *                                routes more than 8 tokens and 512 routes: per chunk of 512
 *                                routes, the routes of each expert, then the
 *                                chunk's first row in each expert
 *   queue           [16]         (inside the first 64 words) the work queues of
 *                                moe_experts_fwd's register-tiled form: 8 per-XCD
 *                                item counters and an exit counter, set to 0 by
 *                                moe_route; that form leaves them at 0 again
 * Order (the counting-sort reading of the flashinfer_ops page's metadata,
 * "FlashInferOps.slot"): experts ascending, routes of one expert in ascending
 * t*K+k, each expert's rows padded to a multiple of m. */
typedef struct moe_meta_layout {
    int64_t num_tiles;
    int64_t total_rows;
    int64_t expert_offsets;
    int64_t expert_counts;
    int64_t exp2perm;
    int64_t perm2tok;
    int64_t tile_expert;
    int64_t total_ints; /* buffer length in int32 */
    int64_t rows_max;
    int64_t tiles_max;
    int64_t sync_status;
    int64_t sub_sync;
    int64_t subs_max;
    int64_t perm_counts;
    int64_t tok_sync;
    int64_t fin_part;
    int64_t queue;
} moe_meta_layout;

int moe_meta_layout_get(int T, int K, int E_local, int tile_m, moe_meta_layout* out);

/* ------------------------------------------------------------------ routing
 * Top-k routing of MuseSpark1x (the runner page, "validate_deployment": sigmoid
 * scores, plus an expert bias, sum-renormalized, no expert groups; the model
 * page, "MuseSpark1xMoE": router_score_division_eps 1e-15, renormalize,
 * e_score_correction_bias; "_prepared_nvfp4_forward": padding tokens route
 * nowhere), then the permutation metadata above.
 *   s_e   = sigmoid(logit_e), by a fixed fp32 algorithm (Cody-Waite range
 *           reduction, degree-7 Taylor polynomial, no fused multiply-add)
 *   key_e = s_e + bias_e; the K largest keys, ties to the lower expert index,
 *           listed by key descending
 *   w_k   = s_{e_k} / (sum_k s_{e_k} + 1e-15) * route_scale, fp32, sum over k in order
 * The bias takes part in the selection only.
 *   logits       device fp32 [T, E], row stride logits_row_stride (>= E), finite
 *   expert_bias  device fp32 [E] or NULL (zeros)
 *   is_padding   device uint8 [T] or NULL; nonzero: the token's ids are -1, weights 0
 *   topk_ids     device int32 [T, K] out: global expert ids
 *   topk_weights device fp32 [T, K] out
 *   meta         device int32 [layout.total_ints] out (moe_meta_layout_get with
 *                the same T, K, local_num_experts, tile_m)
 * tile_m must be a multiple of 16, at most 256. Experts outside
 * [local_expert_offset, local_expert_offset + local_num_experts) are not served
 * here (exp2perm -1), as on an expert-parallel rank. */
int moe_route(const float* logits, int64_t logits_row_stride, const float* expert_bias,
              const uint8_t* is_padding, int T, int E, int K, float route_scale, int tile_m,
              int local_expert_offset, int local_num_experts, int32_t* topk_ids,
              float* topk_weights, int32_t* meta, void* stream);

/* ------------------------------------------------------------------ router
 * The router's linear layer (the model page, "MuseSpark1xMoE": GateLinear from
 * the router input to the E local experts, no bias, fp32 parameters and
 * output; the model's router output multiplier is folded into the weight as it
 * loads, "_load_router_weight"; the router input is fp32 on the decode path,
 * "wants_fp32_router_input"):
 *   logits[t, e] = fp32( sum_d x[t, d] * w_router[e, d] )
 * the products exact and the sum accumulated in fp64, rounded once to fp32.
 *   x         device fp32 [T, D], row stride x_row_stride elements (>= D, % 4 == 0)
 *   w_router  device fp32 [E, D], contiguous
 *   logits    device fp32 [T, E] out, contiguous
 * D % 4 == 0, E <= MOE_MAX_EXPERTS. One launch on `stream`. */
int moe_router_logits(const float* x, int64_t x_row_stride, const float* w_router, int T, int D,
                      int E, float* logits, void* stream);

/* The full routing chain (the model page, "_route_topk_and_pool": the router,
 * then "_compute_routing" on its logits): moe_router_logits into `logits`,
 * then moe_route(logits, E, ...) with the remaining arguments, on `stream`; the
 * same outputs as those two calls, bit for bit. Every check of both calls runs
 * before the first launch. */
int moe_router_route(const float* x, int64_t x_row_stride, const float* w_router, int D,
                     const float* expert_bias, const uint8_t* is_padding, int T, int E, int K,
                     float route_scale, int tile_m, int local_expert_offset, int local_num_experts,
                     float* logits, int32_t* topk_ids, float* topk_weights, int32_t* meta,
                     void* stream);

/* ------------------------------------------------------------------ quantizer
 * NVFP4 quantization of the expert input with one global scale, scales in the
 * plain row-major layout (the model page, "_prepared_nvfp4_forward":
 * scaled_fp4_quant(x, global_scale, is_sf_swizzled_layout=False)). Per block of
 * 16 values of a row, with every step one correctly rounded fp32 operation:
 *   amax = max |x_i|;  s = (amax * gscale) / 6;  sf = e4m3(s)   (nearest even, saturating)
 *   d = decode(sf);  code_i = 0 if d == 0, else e2m1(x_i * (gscale / d))
 *   (e2m1: nearest even, saturating to 6; the sign bit follows the product)
 *   x       device bf16 [T, H], row stride x_row_stride elements (>= H)
 *   gscale  device fp32 [1]: the input global scale (a1_gscale = 1 / a13)
 *   codes   device uint8 [T, H/2] out;  sf device uint8 [T, H/16] out
 * These two arrays are moe_experts_fwd's activation input as they are.
 * H % 16 == 0. */
int nvfp4_quant(const uint16_t* x, int64_t x_row_stride, const float* gscale, int T, int H,
                uint8_t* codes, uint8_t* sf, void* stream);

/* ------------------------------------------------------------------ norm + quantizer
 * The pre-expert RMSNorm run inside the NVFP4 input quantizer (the model page,
 * "MuseSpark1xMoE": pre_expert_norm with a weight, a zero-centred gain and
 * rms_norm_eps; "norm_fuses_into_nvfp4_quant": the weight applies after
 * normalizing; "_prepared_nvfp4_forward": norm_quant_trtllm_nvfp4(pooled,
 * num_tokens, weight, eps, gain_center, global_scale)). Per row of H values:
 *   s  = sum_j x_j^2 in fp64;  ms = fp32(s / H);  r = 1 / sqrt(ms + eps)  (fp32)
 *   y_j = (x_j * r) * gamma_j,  gamma_j = fp32(norm_weight_j) + gain_center
 * each fp32 step one correctly rounded operation; y (fp32, not rounded to bf16)
 * is then quantized exactly as nvfp4_quant quantizes x.
 *   x            device bf16 [T, H], row stride x_row_stride elements (>= H)
 *   norm_weight  device bf16 [H] or NULL (ones)
 *   eps          in (0, 1]
 *   gscale       device fp32 [1]: the input global scale
 *   codes, sf    as nvfp4_quant: device uint8 [T, H/2] and [T, H/16] out
 * H % 16 == 0, H <= MOE_MAX_HIDDEN. One launch on `stream`. */
int nvfp4_norm_quant(const uint16_t* x, int64_t x_row_stride, const uint16_t* norm_weight,
                     float gain_center, float eps, const float* gscale, int T, int H,
                     uint8_t* codes, uint8_t* sf, void* stream);

/* ------------------------------------------------------------------ routing + quantizer
 * moe_route and nvfp4_quant in one launch: the same outputs as moe_route(...)
 * followed by nvfp4_quant(x, x_row_stride, gscale, T, H, codes, sf) on the
 * same stream, bit for bit (the quantizer does not depend on the routing, so
 * its workgroups run beside the routing ones). Arguments and checks are those
 * of the two calls; H is the quantizer's row length. */
int moe_route_quant(const float* logits, int64_t logits_row_stride, const float* expert_bias,
                    const uint8_t* is_padding, int T, int E, int K, float route_scale,
                    int tile_m, int local_expert_offset, int local_num_experts,
                    int32_t* topk_ids, float* topk_weights, int32_t* meta, const uint16_t* x,
                    int64_t x_row_stride, const float* gscale, int H, uint8_t* codes,
                    uint8_t* sf, void* stream);

/* ------------------------------------------------------------------ weights
 * The converted weight layout the expert kernels read. The property the pages
 * require of it (the expert_tp page, module docstring, "slice_views"): an
 * expert-TP slice of the converted weights -- intermediate columns
 * [r I', (r+1) I') -- is, byte for byte, the converted layout of the slice, so
 * slices are views. This library's layout has it for I' % 64 == 0:
 *   An NVFP4 matrix of N rows and K columns (N % 32 == 0, K % 64 == 0) is stored
 *   per expert as [N/32 row pairs][K/64 k-tiles]; a row pair is two groups of 16
 *   rows (half h = 0, 1), and a k-tile of a pair holds its 32 rows x 64 columns
 *   as 1024 code bytes (array *_codes) and 128 scale bytes (array *_sf). The
 *   tile has 64 slots s = q*16 + n, one per 16-column block q of row n, holding
 *   that block of both halves: element k (k < 64, i = k % 16, q = k / 16) of row
 *   n of half h is nibble (i & 1) of code byte (s*2 + h)*8 + i/2, and the block's
 *   scale is scale byte s*2 + h.
 *   (Lane s of a 64-wide wave reads one 16-byte slot and its 2 scale bytes: a
 *   whole 16-element block of both halves, its operands for two 16x16x32 MFMA
 *   steps with the lane's K indices 16q + 8j + [0, 8), j = 0, 1.)
 *   w13 [E, 2I, H] (N = 2I, K = H): converted row 32c + w is gate row 16c + w for
 *   w < 16 and up row I + 16c + (w - 16) otherwise (the gated interleave): pair c
 *   is the gate (half 0) and up (half 1) rows of intermediates [16c, 16c + 16),
 *   so slice r is pairs [rI'/16, (r+1)I'/16).
 *   w2 [E, H, I] (N = H, K = I): pair c is output columns [32c, 32c + 32); slice
 *   r is k-tiles [rI'/64, (r+1)I'/64) of every pair.
 * moe_pack_w13 / moe_pack_w2 convert from the logical layout (the expert_tp
 * page, "StockNvfp4": codes [E, N, K/2], scales [E, N, K/16], row-major; w13
 * rows [0, I) gate = w1, [I, 2I) up = w3) into this one. Device buffers, no
 * overlap; the outputs have the same byte counts as the inputs. */
int moe_pack_w13(const uint8_t* codes, const uint8_t* sf, int E, int I, int H, uint8_t* out_codes,
                 uint8_t* out_sf, void* stream);
int moe_pack_w2(const uint8_t* codes, const uint8_t* sf, int E, int H, int I, uint8_t* out_codes,
                uint8_t* out_sf, void* stream);

/* Converted experts as the expert kernels take them: base pointers and byte
 * strides, so that an expert-TP slice is passed as a view with no copy
 * (the expert_tp page, "TpExperts", "slice_views").
 *   w13, w13_sf: expert e, row pair c at base + e*expert_stride + c*pair_stride
 *                (k-tiles of a pair contiguous: 1024 / 128 bytes each)
 *   w2, w2_sf:   likewise; for slice r of tp of a full-width w2 the base moves
 *                by r*(I'/64) k-tiles and pair_stride stays the full width's
 *   g1_alphas, g1_scale_c, g2_alphas: device fp32 [E_local], the folded scalars
 *     (the runner page, "process_weights_after_loading": g1_alphas = a13*w1_gs,
 *     g1_scale_c = a13*w3_gs/a2, g2_alphas = a2*w2_gs; the expert_tp page: they
 *     do not depend on the slice). */
typedef struct moe_nvfp4_weights {
    const uint8_t* w13;
    const uint8_t* w13_sf;
    const uint8_t* w2;
    const uint8_t* w2_sf;
    int64_t w13_expert_stride_bytes;
    int64_t w13_pair_stride_bytes;
    int64_t w13_sf_expert_stride_bytes;
    int64_t w13_sf_pair_stride_bytes;
    int64_t w2_expert_stride_bytes;
    int64_t w2_pair_stride_bytes;
    int64_t w2_sf_expert_stride_bytes;
    int64_t w2_sf_pair_stride_bytes;
    const float* g1_alphas;
    const float* g1_scale_c;
    const float* g2_alphas;
} moe_nvfp4_weights;

/* Host-only check of a converted-weight descriptor for E_local experts of H x I
 * (I: the full intermediate width the descriptor spans), and for tp > 1 of its
 * cut into tp intermediate slices -- why the weights cannot be cut tp ways, as
 * the expert_tp page's "unsupported" and "shape_of" state it: tp must divide I,
 * and the slice I/tp and H must be multiples of 64 and 128 (the scale tile's
 * k-width and row count), so that every slice is a byte view of the converted
 * layout (moe_experts_fwd on the view). Checks every pointer for NULL and
 * 16-byte alignment and every stride against the shape, as moe_experts_fwd
 * does before a launch. Reads no device memory and launches nothing.
 * Returns MOE_OK, MOE_EINVAL (NULL, alignment, strides) or MOE_EUNSUPPORTED
 * (shape, limits, the tp cut), with the reason in moe_last_error(). */
int moe_validate_weights(const moe_nvfp4_weights* w, int E_local, int H, int I, int tp);

/* The device buffers one layer call reads and writes besides its inputs and
 * its output (the flashinfer_ops page: buffers are sized once, "gemm2_rows"
 * bounds the routed rows), as byte offsets into one caller-owned allocation,
 * each a multiple of 256:
 *   meta          int32 [moe_meta_layout_get(T, K, E_local, tile_m).total_ints]
 *   topk_ids      int32 [T, K];  topk_weights fp32 [T, K]
 *   a_codes       uint8 [T, H/2];  a_sf uint8 [T, H/16]   (the quantized input)
 *   inter_codes   uint8 [rows_max, (I/tp)/2];  inter_sf uint8 [rows_max, (I/tp)/16]
 *   rows          bf16 [tp, rows_max, H]   (one GEMM2 partial per expert-TP slice)
 * rows_max = moe_rows_max(T, K, E_local, tile_m). Returns total_bytes and
 * fills *layout when it is not NULL; -1 for invalid arguments (the reason in
 * moe_last_error()). Host only: reads and launches nothing. */
typedef struct moe_workspace_layout {
    int64_t meta;
    int64_t topk_ids;
    int64_t topk_weights;
    int64_t a_codes;
    int64_t a_sf;
    int64_t inter_codes;
    int64_t inter_sf;
    int64_t rows;
    int64_t total_bytes;
} moe_workspace_layout;

int64_t moe_workspace_bytes(int T, int K, int E_local, int H, int I, int tile_m, int tp,
                            moe_workspace_layout* layout);

/* ------------------------------------------------------------------ experts
 * The routed experts up to the GEMM2 rows, as the op with do_finalize=False
 * computes them (the runner page, "MuseSparkTrtLlmNvFp4Experts.apply_routed";
 * the flashinfer_ops page, "routed_experts_from_metadata"). For every permuted
 * row p that holds a route (token t = perm2tok[p], expert e of its tile):
 *   acc1[n]  = sum_h dq(a[t, h]) * dq(w13[e, n, h])      n < 2I, fp32 accumulate
 *   g = acc1_gate * g1_alphas[e];  u = acc1_up * g1_scale_c[e];  h = silu(g) * u
 *   (inter_codes[p], inter_sf[p]) = NVFP4 of h along I with global scale 1
 *   acc2[n]  = sum_i dq(h[i]) * dq(w2[e, n, i])           n < H
 *   rows[p, n] = bf16(acc2[n] * g2_alphas[e])             nearest even
 * dq(.) = e2m1 code * e4m3 scale of its block; every such value is exact in
 * f16, the MFMA operand type, and the accumulation is fp32. Padding rows are
 * not written.
 *   a_codes, a_sf  device [T, H/2], [T, H/16]: the NVFP4 input, row-major, as
 *                  nvfp4_quant writes it
 *   meta           moe_route's metadata for the same T, K, E_local, tile_m (in/out:
 *                  the sync words, see below)
 *   w              converted experts (host struct; pointers in it are device)
 *   inter_codes, inter_sf  device [rows_max, I/2], [rows_max, I/16] out: the
 *                  requantized intermediate, row-major (GEMM2's input)
 *   rows           device bf16 [rows_max, rows_stride] out, rows_stride >= H
 * Launches on `stream`: with few routes per expert and H % 256 == 0,
 * I % 256 == 0, 9*H and 9*I <= 40960, one launch in which each 16-row tile's
 * GEMM2 workgroups fetch their weights at once and wait, on the tile's
 * counters in meta's sub_sync, for its GEMM1 workgroups to publish the
 * intermediate; otherwise two (GEMM1 with the SwiGLU/requant epilogue, then
 * GEMM2). The counters must be 0 on entry (moe_route leaves them so, and every
 * call returns them to 0), so calls that share one meta buffer must not run
 * concurrently. Every wait is bounded: a wait that gives up sets
 * meta[sync_status] to 1.
 * H % 64 == 0, I % 64 == 0, H and I <= MOE_MAX_HIDDEN, tile_m % 16 == 0. */
int moe_experts_fwd(const uint8_t* a_codes, const uint8_t* a_sf, int32_t* meta,
                    const moe_nvfp4_weights* w, int T, int K, int E_local, int H, int I,
                    int tile_m, uint8_t* inter_codes, uint8_t* inter_sf, uint16_t* rows,
                    int64_t rows_stride, void* stream);

/* ------------------------------------------------------------------ experts + finalize
 * moe_experts_fwd followed by moe_finalize, with the same results bit for bit:
 * the expert step writes its GEMM2 rows as partial n_partials - 1, at
 *   rows + (n_partials - 1) * partial_stride
 * (partials 0 .. n_partials - 2, the other expert-TP slices, were written by
 * earlier calls), then every token's output is finalized from all n_partials
 * partials as moe_finalize(rows, rows_stride, n_partials, partial_stride,
 * meta + exp2perm, topk_weights, norm_weight, gain_center, eps,
 * weight_before_norm, T, K, H, out) computes it (the runner page,
 * "MusePostExpertFinalize"; the flashinfer_ops page's module docstring: the
 * tail kernel finalizes).
 * Where moe_experts_fwd runs in one launch, the finalize runs in that launch
 * too: the workgroup that publishes a token's last route row finalizes the
 * token, counting arrivals on meta's tok_sync (moe_route leaves them at 0 and
 * the call returns them to 0; calls that share one meta buffer must not run
 * concurrently). Otherwise moe_finalize is launched after the expert step.
 * Arguments and checks are those of the two calls. */
int moe_experts_finalize(const uint8_t* a_codes, const uint8_t* a_sf, int32_t* meta,
                         const moe_nvfp4_weights* w, int T, int K, int E_local, int H, int I,
                         int tile_m, uint8_t* inter_codes, uint8_t* inter_sf, uint16_t* rows,
                         int64_t rows_stride, int n_partials, int64_t partial_stride,
                         const float* topk_weights, const uint16_t* norm_weight, float gain_center,
                         float eps, int weight_before_norm, uint16_t* out, void* stream);

/* ------------------------------------------------------------------ experts, no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): moe_experts_fwd with
 * the requantized intermediate kept in the library's own static device memory
 * instead of caller buffers -- the same kernels and the same rows, bit for bit.
 * The caller passes inputs and outputs only (a_codes, a_sf, meta, w, rows as in
 * moe_experts_fwd).
 *   - The static intermediate holds at most MOE_NOALLOC_SCRATCH_BYTES: calls whose
 *     rows_max * I/2 (rounded up to 256) + rows_max * I/16 bytes exceed it return
 *     MOE_EUNSUPPORTED before any launch. Every GPU the library runs on holds
 *     that much for the life of the process.
 *   - All calls on one GPU share that memory and it keeps the last call's
 *     contents (nothing in it needs to start at zero). Calls that overlap on one
 *     GPU -- on different streams, or from different threads -- race; serialize
 *     them (as calls sharing one meta buffer must be already).
 *   - No hipMalloc, hipFree or allocating library routine is called. The first
 *     call on a device looks the memory's address up once (hipGetSymbolAddress,
 *     with that device current). */
#define MOE_NOALLOC_SCRATCH_BYTES (64LL << 20)

int moe_experts_fwd_noalloc(const uint8_t* a_codes, const uint8_t* a_sf, int32_t* meta,
                            const moe_nvfp4_weights* w, int T, int K, int E_local, int H, int I,
                            int tile_m, uint16_t* rows, int64_t rows_stride, void* stream);

/* ------------------------------------------------------------------ experts, W4A16
 * The W4A16 variant of the routed experts: bf16 activations, not quantized,
 * against the same converted NVFP4 weights (the runner page,
 * "MuseSparkModelOptNvFp4FusedMoE": route-major W4A16 GEMMs with SwiGLU;
 * "_process_hopper_marlin_weights": GEMM1 applies the gate's weight global
 * scale to both halves of w13, "keeping the SiLU gate input exact", and GEMM2's
 * global scale carries the up/gate ratio). For every permuted row p that holds
 * a route (token t = perm2tok[p], expert e of its tile):
 *   acc1[n]    = sum_h x[t, h] * dq(w13[e, n, h])           n < 2I, fp32 accumulate
 *   inter[p,i] = bf16(silu(acc1_gate * s13[e]) * (acc1_up * s13[e]))   nearest even
 *   rows[p, n] = bf16(sum_i inter[p, i] * dq(w2[e, n, i]) * s2[e])
 * with s13 = w->g1_alphas (the gate's global scale) and s2 = w->g2_alphas
 * (w2's global scale times up/gate, formed by the caller); w->g1_scale_c is
 * not read. Products of bf16 and NVFP4 values are exact in fp32.
 *   x       device bf16 [T, H], row stride x_row_stride elements (>= H, % 8 == 0)
 *   meta    moe_route's metadata for the same T, K, E_local, tile_m; its sync
 *           words are used and left at 0, and sync_status reports a wait that
 *           gave up, as in moe_experts_fwd
 *   inter   device bf16 [rows_max, I] out: the intermediate, permuted row order
 *   rows    device bf16 [rows_max, rows_stride] out, as moe_experts_fwd
 * One launch on `stream` where H and I are multiples of 256 and T*K >= 128
 * (GEMM2's workgroups wait for GEMM1's through the sync words), else two.
 * H % 64 == 0, I % 64 == 0, both <= MOE_MAX_HIDDEN. */
int moe_experts_fwd_w4a16(const uint16_t* x, int64_t x_row_stride, int32_t* meta,
                          const moe_nvfp4_weights* w, int T, int K, int E_local, int H, int I,
                          int tile_m, uint16_t* inter, uint16_t* rows, int64_t rows_stride,
                          void* stream);

/* ------------------------------------------------------------------ experts, BF16 layers
 * The routed experts of the BF16 layers (the flashinfer_ops page,
 * "routed_experts_bf16", "bf16_arguments": the same routing on the router
 * logits, bf16 w13 and w2, unfinalized rows; the runner page,
 * "MuseSparkUnquantizedFusedMoE"). The routing is moe_route's; this call runs
 * the GEMMs on its metadata. For every permuted row p that holds a route:
 *   acc1[n]    = sum_h x[t, h] * w13[e, n, h]         n < 2I (gate rows first), fp32 accumulate
 *   inter[p,i] = bf16(silu(acc1_gate[i]) * acc1_up[i])
 *   rows[p, n] = bf16(sum_i inter[p, i] * w2[e, n, i])
 *   x      device bf16 [T, H], row stride x_row_stride elements (>= H, % 8 == 0)
 *   meta   moe_route's metadata for the same T, K, E_local, tile_m; its sync
 *          words are used as by moe_experts_fwd_w4a16
 *   w13    device bf16 [E_local, 2I, H], w2 device bf16 [E_local, H, I], contiguous
 *   inter  device bf16 [rows_max, I] out;  rows as moe_experts_fwd
 * One launch on `stream` where H and I are multiples of 256, else two.
 * H % 64 == 0, I % 64 == 0, both <= MOE_MAX_HIDDEN. */
int moe_experts_fwd_bf16(const uint16_t* x, int64_t x_row_stride, int32_t* meta,
                         const uint16_t* w13, const uint16_t* w2, int T, int K, int E_local, int H,
                         int I, int tile_m, uint16_t* inter, uint16_t* rows, int64_t rows_stride,
                         void* stream);

/* ------------------------------------------------------------------ finalize
 * Post-expert finalize (the runner page, "MusePostExpertFinalize",
 * "_finalize_native", "_finalize_chunk", "_effective_weight"): for each token t
 *   r_k = route k's GEMM2 row, rows[exp2perm[t,k]] (zero if the index is -1);
 *         with n_partials > 1 the partials are summed in fp32 and rounded once
 *         to bf16 before the norm (tensor-parallel K-partials; the expert_tp
 *         page, "probe_rel_l2"; the runner page, "_finalize_chunk")
 *   gamma = fp32(norm_weight) + gain_center         (norm_weight NULL: ones)
 *   weight_before_norm: y = z / sqrt(mean(z^2) + eps), z = gamma * r
 *   otherwise:          y = gamma * (r / sqrt(mean(r^2) + eps))
 *   out[t] = bf16(sum_k topk_weights[t,k] * y_k)    fp32, k ascending
 *   rows          device bf16, partial q's row p at rows + q*partial_stride + p*rows_stride
 *   exp2perm      device int32 [T, K] (the meta buffer's field)
 *   topk_weights  device fp32 [T, K]
 *   norm_weight   device bf16 [H] or NULL
 *   out           device bf16 [T, H]
 * H % 8 == 0, H <= MOE_MAX_HIDDEN, 1 <= n_partials <= 16. */
int moe_finalize(const uint16_t* rows, int64_t rows_stride, int n_partials,
                 int64_t partial_stride, const int32_t* exp2perm, const float* topk_weights,
                 const uint16_t* norm_weight, float gain_center, float eps,
                 int weight_before_norm, int T, int K, int H, uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
