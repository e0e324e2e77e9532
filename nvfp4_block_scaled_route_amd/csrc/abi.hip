// Host-side plumbing of the C-ABI: error state, sizing, the metadata layout.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

namespace moe {

static thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

static int64_t align64(int64_t n) { return (n + 63) / 64 * 64; }

moe_meta_layout meta_layout(int T, int K, int E_local, int tile_m) {
    moe_meta_layout L;
    const int64_t R = (int64_t)T * K;
    const int64_t filled = R < E_local ? R : E_local;
    L.rows_max = (filled + (R - filled) / tile_m) * tile_m;
    L.tiles_max = L.rows_max / tile_m;
    L.num_tiles = 0;
    L.total_rows = 1;
    int64_t off = 64;
    L.expert_offsets = off; off += align64(E_local + 1);
    L.expert_counts = off;  off += align64(E_local);
    L.exp2perm = off;       off += align64(R);
    L.perm2tok = off;       off += align64(L.rows_max);
    L.tile_expert = off;    off += align64(L.tiles_max);
    L.sync_status = 2;
    L.queue = kQueueOffset;
    L.subs_max = L.rows_max / 16;
    L.sub_sync = off;       off += align64(kSubSyncStride * L.subs_max);
    L.tok_sync = off;       off += align64(kTokSyncStride * (int64_t)T);
    L.fin_part = off;       off += align64(kFinPartWords * (int64_t)T);
    L.perm_counts = off;    off += align64(((R + 511) / 512) * E_local);
    L.total_ints = off;
    return L;
}

int check_weights(const moe_nvfp4_weights* w, int H, int I, bool need_scale_c, const char* name) {
    if (!w) return fail(MOE_EINVAL, "%s: NULL weights", name);
    if (!w->w13 || !w->w13_sf || !w->w2 || !w->w2_sf || !w->g1_alphas || !w->g2_alphas ||
        (need_scale_c && !w->g1_scale_c))
        return fail(MOE_EINVAL, "%s: NULL weight pointer", name);
    const void* ptrs[] = {w->w13, w->w13_sf, w->w2, w->w2_sf, w->g1_alphas, w->g2_alphas};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return fail(MOE_EINVAL, "%s: weight pointers must be 16-byte aligned", name);
    if (need_scale_c && !aligned16(w->g1_scale_c))
        return fail(MOE_EINVAL, "%s: weight pointers must be 16-byte aligned", name);
    const int64_t kt1 = H / 64, kt2 = I / 64;
    if (w->w13_pair_stride_bytes < kt1 * kSlotBytes || w->w13_sf_pair_stride_bytes < kt1 * kSlotSfBytes ||
        w->w2_pair_stride_bytes < kt2 * kSlotBytes || w->w2_sf_pair_stride_bytes < kt2 * kSlotSfBytes ||
        (w->w13_pair_stride_bytes | w->w13_sf_pair_stride_bytes | w->w2_pair_stride_bytes |
         w->w2_sf_pair_stride_bytes) % 16)
        return fail(MOE_EINVAL, "%s: pair strides too small or not multiples of 16", name);
    if (w->w13_expert_stride_bytes < (int64_t)(I / 16) * w->w13_pair_stride_bytes ||
        w->w13_sf_expert_stride_bytes < (int64_t)(I / 16) * w->w13_sf_pair_stride_bytes ||
        w->w2_expert_stride_bytes < (int64_t)(H / 32) * w->w2_pair_stride_bytes ||
        w->w2_sf_expert_stride_bytes < (int64_t)(H / 32) * w->w2_sf_pair_stride_bytes ||
        (w->w13_expert_stride_bytes | w->w13_sf_expert_stride_bytes | w->w2_expert_stride_bytes |
         w->w2_sf_expert_stride_bytes) % 16)
        return fail(MOE_EINVAL, "%s: expert strides too small or not multiples of 16", name);
    return MOE_OK;
}

static int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_NVFP4_ABI_VERSION; }

const char* moe_last_error(void) { return moe::g_error; }

int64_t moe_rows_max(int T, int K, int E_local, int tile_m) {
    if (T < 0 || K < 1 || E_local < 1 || tile_m < 1) return -1;
    return moe::meta_layout(T, K, E_local, tile_m).rows_max;
}

int moe_meta_layout_get(int T, int K, int E_local, int tile_m, moe_meta_layout* out) {
    if (!out) return moe::fail(MOE_EINVAL, "moe_meta_layout_get: out is NULL");
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E_local < 1 || E_local > MOE_MAX_EXPERTS)
        return moe::fail(MOE_EINVAL, "moe_meta_layout_get: T=%d K=%d E_local=%d out of range", T, K,
                         E_local);
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return moe::fail(MOE_EUNSUPPORTED, "moe_meta_layout_get: tile_m=%d must be a multiple of 16 in [16, 256]",
                         tile_m);
    *out = moe::meta_layout(T, K, E_local, tile_m);
    return MOE_OK;
}

int moe_validate_weights(const moe_nvfp4_weights* w, int E_local, int H, int I, int tp) {
    using namespace moe;
    const char* name = "moe_validate_weights";
    if (E_local < 1 || E_local > MOE_MAX_EXPERTS)
        return fail(MOE_EINVAL, "%s: E_local=%d out of range", name, E_local);
    if (H < 64 || H % 64 || I < 64 || I % 64 || H > MOE_MAX_HIDDEN || I > MOE_MAX_HIDDEN)
        return fail(MOE_EUNSUPPORTED, "%s: H=%d and I=%d must be multiples of 64 up to %d", name, H, I,
                    MOE_MAX_HIDDEN);
    if (tp < 1) return fail(MOE_EINVAL, "%s: tp=%d must be at least 1", name, tp);
    if (tp > 1) {
        if (I % tp) return fail(MOE_EUNSUPPORTED, "%s: intermediate %d does not split %d ways", name, I, tp);
        if ((I / tp) % 64 || H % 128)
            return fail(MOE_EUNSUPPORTED, "%s: intermediate slice %d and hidden %d must be multiples of 64 and 128",
                        name, I / tp, H);
    }
    return check_weights(w, H, I, true, name);
}

int64_t moe_workspace_bytes(int T, int K, int E_local, int H, int I, int tile_m, int tp,
                            moe_workspace_layout* layout) {
    using namespace moe;
    const char* name = "moe_workspace_bytes";
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E_local < 1 || E_local > MOE_MAX_EXPERTS || tp < 1) {
        fail(MOE_EINVAL, "%s: T=%d K=%d E_local=%d tp=%d out of range", name, T, K, E_local, tp);
        return -1;
    }
    if (tile_m < 16 || tile_m > 256 || tile_m % 16 || H < 16 || H % 16 || I % tp || (I / tp) < 16 ||
        (I / tp) % 16) {
        fail(MOE_EUNSUPPORTED, "%s: tile_m=%d H=%d I=%d tp=%d not supported", name, tile_m, H, I, tp);
        return -1;
    }
    const moe_meta_layout L = meta_layout(T, K, E_local, tile_m);
    const int64_t R = (int64_t)T * K, Is = I / tp;
    moe_workspace_layout w;
    int64_t off = 0;
    w.meta = off;         off += align256(4 * L.total_ints);
    w.topk_ids = off;     off += align256(4 * R);
    w.topk_weights = off; off += align256(4 * R);
    w.a_codes = off;      off += align256((int64_t)T * (H / 2));
    w.a_sf = off;         off += align256((int64_t)T * (H / 16));
    w.inter_codes = off;  off += align256(L.rows_max * (Is / 2));
    w.inter_sf = off;     off += align256(L.rows_max * (Is / 16));
    w.rows = off;         off += align256((int64_t)tp * L.rows_max * H * 2);
    w.total_bytes = off;
    if (layout) *layout = w;
    return off;
}

}  // extern "C"
