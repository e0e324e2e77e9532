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
    L.subs_max = L.rows_max / 16;
    L.sub_sync = off;       off += align64(kSubSyncStride * L.subs_max);
    L.perm_counts = off;    off += align64(((R + 511) / 512) * E_local);
    L.total_ints = off;
    return L;
}

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

}  // extern "C"
