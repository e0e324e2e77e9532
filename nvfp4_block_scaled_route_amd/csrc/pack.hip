// moe_pack_w13 / moe_pack_w2: logical NVFP4 expert weights -> the converted
// layout the expert kernels read (moe_nvfp4.h, "weights"). Run once at load,
// like the weight conversion of the runner page,
// "MuseSparkModelOptNvFp4FusedMoE.process_weights_after_loading".
//
// Both layouts keep a 16-element block of a row in 8 consecutive bytes (element
// 2j in the low nibble of byte j), so the conversion moves whole blocks: one
// thread writes one converted 8-byte half-slot, and for the scales one byte.
#include "common.hpp"

namespace moe {

// converted row -> logical row (w13: the gated interleave; w2: identity)
__device__ __forceinline__ int64_t logical_row(int64_t rho, int interleave_half) {
    if (interleave_half == 0) return rho;
    const int64_t c = rho >> 5, w = rho & 31;
    return w < 16 ? 16 * c + w : interleave_half + 16 * c + (w - 16);
}

// Tile index (e, pair, k-tile) and position (slot, half) of one converted item.
struct TilePos {
    int64_t e, row;
    int c, q;
};
__device__ __forceinline__ TilePos tile_pos(int64_t tile, int item, int N, int K,
                                            int interleave_half) {
    const int tiles_k = K / 64, pairs = N / 32;
    const int h = item & 1, s = item >> 1, n = s & 15;
    TilePos t;
    t.q = s >> 4;
    t.e = tile / ((int64_t)pairs * tiles_k);
    const int64_t rem = tile - t.e * pairs * tiles_k;
    const int64_t p = rem / tiles_k;
    t.c = (int)(rem - p * tiles_k);
    t.row = logical_row(p * 32 + h * 16 + n, interleave_half);
    return t;
}

// out_codes: E * (N/32) * (K/64) tiles of 1024 bytes; thread -> one 8-byte half-slot
__global__ void __launch_bounds__(256) pack_codes_kernel(const uint8_t* __restrict__ in, int E,
                                                         int N, int K, int interleave_half,
                                                         uint2* __restrict__ out) {
    const int64_t total = (int64_t)E * N * K / 16;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const TilePos t = tile_pos(i >> 7, (int)(i & 127), N, K, interleave_half);
    const uint8_t* src = in + (t.e * N + t.row) * (int64_t)(K / 2) + t.c * 32 + t.q * 8;
    out[i] = *reinterpret_cast<const uint2*>(src);
}

// out_sf: E * (N/32) * (K/64) tiles of 128 bytes; thread -> one byte
__global__ void __launch_bounds__(256) pack_scales_kernel(const uint8_t* __restrict__ in, int E,
                                                          int N, int K, int interleave_half,
                                                          uint8_t* __restrict__ out) {
    const int64_t total = (int64_t)E * N * K / 16;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const TilePos t = tile_pos(i >> 7, (int)(i & 127), N, K, interleave_half);
    out[i] = in[(t.e * N + t.row) * (int64_t)(K / 16) + t.c * 4 + t.q];
}

static int pack(const char* name, const uint8_t* codes, const uint8_t* sf, int E, int N, int K,
                int interleave_half, uint8_t* out_codes, uint8_t* out_sf, void* stream) {
    if (E < 0 || N < 0 || K < 0) return fail(MOE_EINVAL, "%s: negative size", name);
    if (N % 32 || K % 64)
        return fail(MOE_EUNSUPPORTED, "%s: rows %d must be a multiple of 32 and columns %d of 64",
                    name, N, K);
    if ((int64_t)E * N * K == 0) return MOE_OK;
    if (!codes || !sf || !out_codes || !out_sf) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    if (!aligned16(codes) || !aligned16(sf) || !aligned16(out_codes) || !aligned16(out_sf))
        return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    const int64_t items = (int64_t)E * N * K / 16;
    if ((items + 255) / 256 > 0x7FFFFFFF) return fail(MOE_EUNSUPPORTED, "%s: too large", name);
    const dim3 grid((unsigned)((items + 255) / 256));
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(pack_codes_kernel, grid, dim3(256), 0, s, codes, E, N, K, interleave_half,
                       reinterpret_cast<uint2*>(out_codes));
    int rc = check_launch(name);
    if (rc) return rc;
    hipLaunchKernelGGL(pack_scales_kernel, grid, dim3(256), 0, s, sf, E, N, K, interleave_half,
                       out_sf);
    return check_launch(name);
}

}  // namespace moe

extern "C" int moe_pack_w13(const uint8_t* codes, const uint8_t* sf, int E, int I, int H,
                            uint8_t* out_codes, uint8_t* out_sf, void* stream) {
    if (I % 16) return moe::fail(MOE_EUNSUPPORTED, "moe_pack_w13: I=%d is not a multiple of 16", I);
    return moe::pack("moe_pack_w13", codes, sf, E, 2 * I, H, I, out_codes, out_sf, stream);
}

extern "C" int moe_pack_w2(const uint8_t* codes, const uint8_t* sf, int E, int H, int I,
                           uint8_t* out_codes, uint8_t* out_sf, void* stream) {
    return moe::pack("moe_pack_w2", codes, sf, E, H, I, 0, out_codes, out_sf, stream);
}
