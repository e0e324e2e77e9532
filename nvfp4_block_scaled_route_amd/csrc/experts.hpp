// Arguments shared by the expert kernels (moe_experts_fwd): the streaming
// kernels for few routes per expert (experts.hip) and the tiled kernels for
// many (experts_tiled.hip).
#pragma once
#include "common.hpp"

namespace moe {

struct ExpArgs {
    const uint8_t* a_codes;
    const uint8_t* a_sf;
    const int32_t* meta;
    moe_meta_layout L;
    moe_nvfp4_weights w;
    int T, E_local, H, I, tile_m;
    uint8_t* inter_codes;
    uint8_t* inter_sf;
    uint16_t* rows;
    int64_t rows_stride;
    int32_t* sync;       // meta's sub_sync: per 16-row tile (kSubSyncStride apart), GEMM1 workgroups done, GEMM2 copies done
    int32_t* status;     // meta's sync_status
    int32_t* queue;      // meta's queue words (the register-tiled form's work queues)
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediates (gfx9 encoding): at most n vector-memory loads in
// flight, the other counters unconstrained; and-ed with lgkmcnt_zero(): no
// LDS reads in flight either
__host__ __device__ constexpr int vmcnt_at_most(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}
__host__ __device__ constexpr int lgkmcnt_zero() { return ~(15 << 8); }

__device__ __forceinline__ u32x4 buffer_desc(const void* base) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    // raw buffer (stride 0) with no range limit; gfx9 data-format word
    return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xFFFFu, 0x7FFFFFFFu, 0x00020000u};
}

// Expert weights are read once per call: non-temporal loads keep them from
// displacing what is read again (metadata, activations, intermediate, rows) in
// the L2 and Infinity Cache. Measured on decode_b8: expert step 31.3 -> 29.4 us,
// whole layer 45.3 -> 42.5 us.
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t load_stream2(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS load: lane l's 16 bytes at base + voff + soff land at LDS
// address lds + 16 l. The compiler does not see it: a wait for it is the
// caller's (vmcnt, which it shares with the loads issued around it). The LDS
// address goes to the instruction in M0 as an input operand, so the compiler
// writes M0 itself right before it and knows the register is taken (the
// instruction only reads M0). Inline assembly rather than the compiler's
// direct-to-LDS builtin: the compiler takes that builtin for an LDS write of
// unknown extent and makes every later LDS read wait for it, which would
// serialize the double-buffered stages of the tiled kernels.
__device__ __forceinline__ void lds_copy16(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}

// The same load, agent-coherent (sc1): it returns what another XCD wrote with
// agent-coherent stores, not a line its own L2 may still hold.
__device__ __forceinline__ void lds_copy16_sc1(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen sc1 lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}

// A bounded wait for a counter another workgroup of the same launch adds to
// (agent-coherent polls, a sleep between them): after kSpinMax polls it gives
// up and sets the status word to 1, so no wait can hang the launch.
constexpr uint32_t kSpinMax = 1u << 20;

__device__ __forceinline__ void wait_ready(int32_t* ready, int target, int32_t* status) {
    for (uint32_t it = 0;; ++it) {
        if (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
        if (it >= kSpinMax) {
            __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(8);
    }
}

// The unit's 16-row tile: expert (-1: no unit) and the lane's row token.
struct RowTile {
    int e;
    int row0;
    int tok;                // token of row n (lane & 15), -1 for a padding row
    uint32_t vmask;         // bit m: row m holds a route
};

__device__ __forceinline__ RowTile row_tile(const ExpArgs& a, int sub, int n) {
    RowTile r;
    const int per_tile = a.tile_m >> 4;
    const int t = (int)((uint32_t)sub / (uint32_t)per_tile);
    // Both metadata loads go out before any decision: the tile index is clamped
    // so that they stay in bounds for units past the last tile.
    const int tc = min(t, (int)a.L.tiles_max - 1);
    r.row0 = tc * a.tile_m + (sub - t * per_tile) * 16;
    const int e = a.meta[a.L.tile_expert + tc];
    int tok = a.meta[a.L.perm2tok + r.row0 + n];
    if (tok >= a.T) tok = -1;
    r.tok = tok;
    r.vmask = (uint32_t)(__ballot(tok >= 0) & 0xFFFFull);
    r.e = (t < a.L.tiles_max && e >= 0 && e < a.E_local && r.vmask) ? e : -1;
    return r;
}

// GEMM2: lane (q, n) holds rows 4q + i of output columns 32c + n and 32c + 16 + n.
// kPublish: the rows are read by other workgroups of the same launch (the
// finalize in the launch), so they are written with agent-coherent stores.
template <bool kPublish = false>
__device__ __forceinline__ void gemm2_epilogue(const ExpArgs& a, const RowTile& rt, int e, int c, int n, int q,
                                               const floatx4& acc0, const floatx4& acc1) {
    const float alpha = a.w.g2_alphas[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        if ((rt.vmask >> m) & 1u) {
            uint16_t* out = a.rows + (int64_t)(rt.row0 + m) * a.rows_stride + c * 32 + n;
            const uint16_t v0 = (uint16_t)f32_to_bf16(acc0[i] * alpha), v1 = (uint16_t)f32_to_bf16(acc1[i] * alpha);
            if (kPublish) {
                __hip_atomic_store(out, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(out + 16, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                out[0] = v0;
                out[16] = v1;
            }
        }
    }
}

// The tiled path: 128-row blocks of one expert (tile_m % 128 == 0), K in whole
// 4-k-tile stages (H % 256 == 0, I % 256 == 0), activation code offsets below
// 2^31 bytes.
bool tiled_shape_ok(int T, int H, int I, int tile_m);
// Both GEMMs in one launch of persistent workgroups taking work items from
// per-XCD queues (meta's queue words), GEMM2's items waiting on per-block
// counters (meta's sub_sync) for GEMM1's. Returns MOE_OK or an error code.
int launch_tiled(const ExpArgs& a, hipStream_t s);

}  // namespace moe
