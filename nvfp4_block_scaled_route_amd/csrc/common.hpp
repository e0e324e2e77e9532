// Shared device helpers and host error plumbing of libmoe_nvfp4 (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ host side
int fail(int code, const char* fmt, ...);          // sets the thread's message, returns code
int quant_check(const uint16_t* x, int64_t x_row_stride, const float* gscale, int T, int H,
                uint8_t* codes, uint8_t* sf, const char* name);   // nvfp4_quant's validation
int check_launch(const char* what);                // MOE_ELAUNCH on a pending launch error
// moe_route's validation (shared with moe_router_route, which runs it before
// its first launch)
int moe_route_check(int T, int E, int K, int tile_m, int local_expert_offset, int local_num_experts,
                    int64_t logits_row_stride, const float* logits, const int32_t* topk_ids,
                    const float* topk_weights, const int32_t* meta, const char* name);
// the converted-weight descriptor's pointers, alignment and strides for H x I
// experts (g1_scale_c checked when need_scale_c): shared by the expert calls
// and moe_validate_weights
int check_weights(const moe_nvfp4_weights* w, int H, int I, bool need_scale_c, const char* name);
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
moe_meta_layout meta_layout(int T, int K, int E_local, int tile_m);
// int32 words between the sync counters of consecutive 16-row tiles in the
// metadata (1 KB): tiles' counters on distinct cache lines and memory channels,
// so that the polls of many workgroups do not all queue on one channel.
constexpr int kSubSyncStride = 256;
// int32 words between the arrival counters of consecutive tokens (128 bytes:
// one counter a cache line) -- moe_experts_finalize's one-launch form
constexpr int kTokSyncStride = 32;
// words a token's finalize exchanges between its workgroups: 16 waves x 8 routes
constexpr int kFinPartWords = 128;
// the tiled expert step's work queues in the metadata header: words
// [kQueueOffset, kQueueOffset + kXcds) count the items taken from each XCD's
// queue, word kQueueOffset + kXcds the workgroups that have finished
constexpr int kQueueOffset = 16;
constexpr int kQueueWords = 16;
// converted weight layout: code and scale bytes per row pair and k-tile
constexpr int kSlotBytes = 1024, kSlotSfBytes = 128;

// ------------------------------------------------------------------ codecs
// e2m1: nearest value of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code,
// saturating at 6; the sign bit follows the input (NaN encodes to +0). Each
// threshold is a midpoint of the grid; >= where the upper neighbour has the
// even code, > where the lower one has.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    if (!(v == v)) return 0u;
    const float a = __builtin_fabsf(v);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// e4m3fn (bias 7, subnormals m * 2^-9, max 448): nearest even, saturating to
// +-448; NaN encodes to 0x7F. Works on the fp32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    if (!(v == v)) return 0x7Fu;
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = __builtin_fabsf(v);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {                       // below 2^-6: the subnormal grid
        code = (uint32_t)__builtin_rintf(a * 512.0f); // exact scaling, ties to even
    } else {
        const uint32_t ab = __float_as_uint(a);
        uint32_t e = (ab >> 23) - 120u;               // biased e4m3 exponent, 1 .. 15
        uint32_t m = (ab >> 20) & 7u;
        const uint32_t rem = ab & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
        if (m == 8u) { m = 0u; ++e; }
        code = (e << 3) | m;
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return code | sign;
}

// e4m3fn byte -> fp32 (exact; NaN codes are not decoded).
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float mag = e == 0u ? (float)m * 0.001953125f
                              : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -mag : mag;
}

// The NVFP4 block scale and the element multiplier of one 16-value block:
// s = (amax * gscale) / 6 -> e4m3 byte; r = gscale / decode(byte) (0 when the
// scale decodes to 0). One correctly rounded fp32 operation per step.
struct BlockScale {
    uint32_t byte;
    float r;
};
__device__ __forceinline__ BlockScale nvfp4_block_scale(float amax, float gscale) {
#pragma clang fp contract(off)
    const float s = __fdiv_rn(__fmul_rn(amax, gscale), 6.0f);
    BlockScale out;
    out.byte = e4m3_encode(s);
    const float d = e4m3_decode(out.byte);
    out.r = d == 0.0f ? 0.0f : __fdiv_rn(gscale, d);
    return out;
}

// The e2m1 code of one element given its block's multiplier (code 0 when the
// block scale is 0).
__device__ __forceinline__ uint32_t nvfp4_code(float x, const BlockScale& bs) {
    return bs.r == 0.0f ? 0u : e2m1_encode(__fmul_rn(x, bs.r));
}

// The same for 8 consecutive elements, packed (element 0 in the low nibble).
// The hardware pack conversion at scale 1 (no scaling) rounds to nearest, ties
// to the even code, saturates at 6 and keeps the sign: it gives e2m1_encode's
// code for every non-NaN f32 (checked over all 2^32 patterns on gfx950).
// kNan: NaN products take code 0 as in e2m1_encode; without it the caller
// guarantees that there are none.
template <bool kNan>
__device__ __forceinline__ uint32_t nvfp4_codes8(const float* v, const BlockScale& bs) {
    float p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        p[k] = __fmul_rn(v[k], bs.r);
        if (kNan) p[k] = p[k] == p[k] ? p[k] : 0.0f;
    }
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[0], p[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[2], p[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[4], p[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[6], p[7], 1.0f, 3);
    return bs.r == 0.0f ? 0u : w;
}

// ------------------------------------------------------------------ sigmoid
// s(l) = 1 / (1 + exp(-l)). exp by Cody and Waite's range reduction
// x = n ln2 + r, with ln2 split so that n * ln2_hi is exact, and the degree-7
// Taylor polynomial of e^r in Horner form; every step is a separate, correctly
// rounded fp32 operation (no fused multiply-add). exp(x) for x > 80 gives a
// sigmoid of 0, for x < -20 a sigmoid of 1 (e^x is below half an ulp of 1).
__device__ __forceinline__ float sigmoid32(float l) {
#pragma clang fp contract(off)
    const float x = -l;
    if (x > 80.0f) return 0.0f;
    if (x < -20.0f) return 1.0f;
    const float n = __builtin_rintf(__fmul_rn(x, 1.4426950408889634f));
    float r = __fsub_rn(x, __fmul_rn(n, 0.693359375f));
    r = __fsub_rn(r, __fmul_rn(n, (float)(0.6931471805599453 - 0.693359375)));
    float p = (float)(1.0 / 5040.0);
    p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 720.0));
    p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 120.0));
    p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 24.0));
    p = __fadd_rn(__fmul_rn(p, r), (float)(1.0 / 6.0));
    p = __fadd_rn(__fmul_rn(p, r), 0.5f);
    p = __fadd_rn(__fmul_rn(p, r), 1.0f);
    p = __fadd_rn(__fmul_rn(p, r), 1.0f);
    const float e = __builtin_ldexpf(p, (int)n);
    return __fdiv_rn(1.0f, __fadd_rn(1.0f, e));
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {   // nearest even
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return 0x7FC0u;   // NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two finite values -> packed bf16 (a in the low half) with the hardware pack
// conversion: the same bits as f32_to_bf16 for every non-NaN f32 (checked over
// all 2^32 patterns on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_pack(float a, float b) {
    const floatx2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ------------------------------------------------------------------ NVFP4 quantizer block
// One 16-value block (row t, block b) of a bf16 matrix -> 8 code bytes and its
// e4m3 scale byte, in nvfp4_quant's layout (row-major codes and scales).
__device__ __forceinline__ void quantize_block16(const uint16_t* __restrict__ x, int64_t x_row_stride,
                                                 float gscale, int H, int t, int b,
                                                 uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ sf) {
    const uint4* src = reinterpret_cast<const uint4*>(x + t * x_row_stride + b * 16);
    const uint4 p0 = src[0], p1 = src[1];
    const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        amax = fmaxf(amax, fmaxf(__builtin_fabsf(v[2 * i]), __builtin_fabsf(v[2 * i + 1])));
    }
    const BlockScale bs = nvfp4_block_scale(amax, gscale);
    const uint32_t lo = nvfp4_codes8<true>(v, bs), hi = nvfp4_codes8<true>(v + 8, bs);
    *reinterpret_cast<uint2*>(codes + (int64_t)t * (H >> 1) + b * 8) = make_uint2(lo, hi);
    sf[(int64_t)t * (H >> 4) + b] = (uint8_t)bs.byte;
}

// ------------------------------------------------------------------ NVFP4 -> f16 operands
// 8 e2m1 codes (a u32, element 0 in the low nibble) times one e4m3 scale -> the
// 8 exact f16 products. The hardware pack-convert applies only the exponent of
// its scale operand, so it runs at scale 1 and the e4m3 scale (exact in f16)
// multiplies after it; every product e2m1 * e4m3 has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in f16. `scale` holds the f16 scale
// in both halves.
__device__ __forceinline__ half8 nvfp4x8_to_f16(uint32_t codes, half2v scale) {
    const half2v v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * scale;
    const half2v v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * scale;
    const half2v v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * scale;
    const half2v v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * scale;
    half8 out;
    out[0] = v0[0]; out[1] = v0[1]; out[2] = v1[0]; out[3] = v1[1];
    out[4] = v2[0]; out[5] = v2[1]; out[6] = v3[0]; out[7] = v3[1];
    return out;
}

// Two e4m3 bytes (bits 0-7 and 8-15) -> two exact f16 values (the hardware
// OCP e4m3 -> f16 conversion; scale 1 leaves the values unchanged).
__device__ __forceinline__ half2v e4m3x2_to_f16(uint32_t two_bytes) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_bytes, 1.0f, false);
}

__device__ __forceinline__ half2v splat_lo(half2v v) { half2v r = {v[0], v[0]}; return r; }
__device__ __forceinline__ half2v splat_hi(half2v v) { half2v r = {v[1], v[1]}; return r; }

// ------------------------------------------------------------------ wave reductions
// Cross-lane moves by DPP (no LDS traffic, no wait counter). Controls of the
// gfx9 encoding: quad_perm, row_shr:n, row_mirror, row_half_mirror,
// row_bcast:15, row_bcast:31.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int ctrl, int row_mask = 0xF, int bank_mask = 0xF, bool bound_ctrl = true>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, ctrl, row_mask, bank_mask, bound_ctrl);
}
template <int ctrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, true));
}

// Sum over the 64 lanes in a fixed order (every lane of a 16-lane row forms the
// same row sum: pairs within quads, quads, halves, then the four rows in
// order), so the result is deterministic. Uniform result.
__device__ __forceinline__ float wave_sum(float v) {
    v = __fadd_rn(v, dpp_f<kDppQuadXor1>(v));
    v = __fadd_rn(v, dpp_f<kDppQuadXor2>(v));
    v = __fadd_rn(v, dpp_f<kDppRowHalfMirror>(v));
    v = __fadd_rn(v, dpp_f<kDppRowMirror>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return __fadd_rn(__fadd_rn(r0, r1), __fadd_rn(r2, r3));
}

// Inclusive prefix sum over the 64 lanes (integers: exact in any order).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += dpp_i<kDppRowShr1>(v);
    v += dpp_i<kDppRowShr2>(v);
    v += dpp_i<kDppRowShr4>(v);
    v += dpp_i<kDppRowShr8>(v);
    v += dpp_i<kDppRowBcast15, 0xA>(v);     // rows 1, 3 += last lane of rows 0, 2
    v += dpp_i<kDppRowBcast31, 0xC>(v);     // rows 2, 3 += lane 31
    return v;
}

// LDS writes of this wave are seen by its later LDS reads (a wave's LDS
// operations complete in order); this keeps the compiler from moving them.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max16(float v) {      // max over 16-lane rows
    v = fmaxf(v, __shfl_xor(v, 8));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 1));
    return v;
}

}  // namespace moe
