// The expert GEMMs for many routes per expert (prefill): LDS-tiled MFMA.
//   the runner page, "MuseSparkTrtLlmNvFp4Experts.apply_routed"; the
//   flashinfer_ops page, "routed_experts_from_metadata" -- same arithmetic as
//   the streaming kernels in experts.hip (GEMM1 + SwiGLU + requant, GEMM2).
//
// With hundreds of routes per expert the GEMMs are bound by the matrix cores,
// not by the weight stream, and every operand element must serve many MFMAs.
// A workgroup computes a 128 x 128 output block (128 permuted rows of one
// expert x 128 weight rows = 4 row pairs) over K in 64-wide k-tiles:
//   * four waves, 2 x 2, each compute 64 x 64 with v_mfma_f32_32x32x16_f16;
//   * the weight operand B goes through LDS: the 256 threads load one k-tile
//     of it as NVFP4 (16 code bytes + the scale word each), decode it once to
//     exact f16 and store it (double buffered, rows padded to 144 bytes), and
//     every wave reads its fragments from there;
//   * the activation operand A goes straight to registers: each wave gathers
//     its own 64 rows in MFMA lane order (a lane's 32 elements of a k-tile are
//     two whole NVFP4 blocks of its row: the MFMA K index is permuted on both
//     operands to make it so) and decodes them itself, so A costs no LDS
//     traffic and no LDS latency sits before the MFMAs;
//   * the raw loads run 4 k-tiles ahead in registers, so HBM latency is hidden
//     behind 4 k-tiles of MFMA work; one barrier per k-tile.
// Blocks are mapped so that consecutive row blocks with the same column block
// -- usually rows of one expert, sharing its weights -- run on the same XCD
// (workgroups are dealt to the 8 XCDs round robin) and meet in its L2.
// GEMM1's epilogue (SwiGLU, 16-wide amax, e4m3 scale, codes) and GEMM2's
// (bf16 rows) work from the MFMA accumulators; rows without a route are
// neither read from global memory as routes nor written.
#include "experts.hpp"

namespace moe {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kLdsRow = kTK + 8;            // halves per LDS row
constexpr int kTiledThreads = 256;
constexpr int kAhead = 4;                   // k-tiles loaded ahead in registers
constexpr int kXcds = 8;

// One thread's raw operands of one k-tile: its A rows (each lane holds 32 of
// K = 64: blocks 2h and 2h + 1 of its row, h = lane / 32) and one B slot
// (block q of row n of both halves of a pair). Scales are loaded as aligned
// 32-bit words (in bounds: the 4 block scales of a row's k-tile; the scales of
// an even/odd slot pair) and the thread's 16 bits are shifted out where they
// are used: a 16-bit load would be widened with a mask that the compiler
// hoists to the top of the loop, where it makes every wave wait for all loads
// in flight.
struct TileRegs {
    uint4 a[2];       // A, row tiles 0 and 1: 32 elements each (2 blocks)
    uint32_t asf[2];  // the rows' 4 block scales of the k-tile
    uint4 b;          // B slot
    uint32_t bsf;     // scales of slots 2 (slot / 2), 2 (slot / 2) + 1
};

struct TilePtrs {
    const uint8_t* ac[2];   // k-tile c at +32 c
    const uint8_t* as[2];   // +4 c
    const uint8_t* bc;      // +1024 c
    const uint8_t* bs;      // +128 c
};

// The six loads of a k-tile always issue in this order and by themselves
// (prologue and loop alike), so that every use waits only for the loads issued
// before it: vmcnt drains in issue order.
__device__ __forceinline__ void tile_load(TileRegs& r, const TilePtrs& p, int c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        r.a[i] = *reinterpret_cast<const uint4*>(p.ac[i] + c * 32);
        __builtin_amdgcn_sched_barrier(0);
        r.asf[i] = *reinterpret_cast<const uint32_t*>(p.as[i] + c * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
    r.b = *reinterpret_cast<const uint4*>(p.bc + (int64_t)c * kSlotBytes);
    __builtin_amdgcn_sched_barrier(0);
    r.bsf = *reinterpret_cast<const uint32_t*>(p.bs + (int64_t)c * kSlotSfBytes);
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void store_half8(_Float16* dst, const half8& v) {
    *reinterpret_cast<half8*>(dst) = v;
}

// Decode one thread's B slot of a k-tile into LDS. The MFMA's K index is
// permuted on both operands: lane (h, r) of a K = 16 step s takes elements
// 32h + 8s + [0, 8) of the k-tile (the A lane's own two blocks), so element j of
// block q lives at LDS column 32 (q % 2) + 16 (j / 8) + 8 (q / 2) + j % 8.
__device__ __forceinline__ void store_b(const TileRegs& r, _Float16 (*Bs)[kLdsRow], int bp, int slot) {
    const half2v sb = e4m3x2_to_f16(r.bsf >> (16 * (slot & 1)));
    const half2v sb0 = splat_lo(sb), sb1 = splat_hi(sb);
    const int q = slot >> 4, n = slot & 15;
    const int col = 32 * (q & 1) + 8 * (q >> 1);
    _Float16* b0 = &Bs[bp * 32 + n][col];
    _Float16* b1 = &Bs[bp * 32 + 16 + n][col];
    store_half8(b0, nvfp4x8_to_f16(r.b.x, sb0));
    store_half8(b0 + 16, nvfp4x8_to_f16(r.b.y, sb0));
    store_half8(b1, nvfp4x8_to_f16(r.b.z, sb1));
    store_half8(b1 + 16, nvfp4x8_to_f16(r.b.w, sb1));
}

// The wave's 64 x 64 block over one k-tile: A decoded from the lane's own
// registers, B fragments from LDS, 4 steps of K = 16, 2 x 2 MFMA tiles.
__device__ __forceinline__ void tile_mfma(const TileRegs& r, const _Float16 (*Bs)[kLdsRow], int wn,
                                          int lane, floatx16 acc[2][2]) {
    const int rr = lane & 31, h = lane >> 5;
    half8 bf[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bf[s][j] = *reinterpret_cast<const half8*>(&Bs[wn * 64 + j * 32 + rr][s * 16 + 8 * h]);
    half2v sa[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const half2v sc = e4m3x2_to_f16(r.asf[i] >> (16 * h));
        sa[i][0] = splat_lo(sc);
        sa[i][1] = splat_hi(sc);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        half8 af[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t w = s == 0 ? r.a[i].x : s == 1 ? r.a[i].y : s == 2 ? r.a[i].z : r.a[i].w;
            af[i] = nvfp4x8_to_f16(w, sa[i][s >> 1]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[s][j], acc[i][j], 0, 0, 0);
    }
}

template <int MODE>   // 1: GEMM1 + SwiGLU + requant, 2: GEMM2
__global__ void __launch_bounds__(kTiledThreads) tiled_kernel(ExpArgs a, int nx, int ny) {
    // the two LDS buffers are separate objects, so that the stores of the next
    // k-tile provably do not alias the fragment reads of this one
    __shared__ _Float16 Bs0[kTN][kLdsRow], Bs1[kTN][kLdsRow];
    __shared__ int s_valid[kTM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware block order: consecutive ids run on one XCD
    const int per_xcd = (int)gridDim.x / kXcds;
    const int id = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (id >= nx * ny) return;
    const int bx = id % nx, by = id / nx;
    const int row0 = bx * kTM;
    const int e = a.meta[a.L.tile_expert + row0 / a.tile_m];
    if (e < 0 || e >= a.E_local) return;

    const int K = MODE == 1 ? a.H : a.I;
    const int KT = K >> 6;
    const int h = lane >> 5, rr = lane & 31;
    const int bp = tid >> 6, slot = tid & 63;
    const int pair = by * 4 + bp;
    TilePtrs p;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = wm * 64 + i * 32 + rr;       // this lane's A row of row tile i
        int tok = a.meta[a.L.perm2tok + row0 + m];
        if (tok >= a.T) tok = -1;
        if (wn == 0 && h == 0) s_valid[m] = tok >= 0;
        if (MODE == 1) {
            const int64_t t = tok >= 0 ? tok : 0;   // rows without a route read a stand-in row
            p.ac[i] = a.a_codes + t * (a.H >> 1) + h * 16;
            p.as[i] = a.a_sf + t * (a.H >> 4);
        } else {
            const int64_t row = row0 + m;
            p.ac[i] = a.inter_codes + row * (a.I >> 1) + h * 16;
            p.as[i] = a.inter_sf + row * (a.I >> 4);
        }
    }
    if (MODE == 1) {
        p.bc = a.w.w13 + e * a.w.w13_expert_stride_bytes + pair * a.w.w13_pair_stride_bytes + slot * 16;
        p.bs = a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + pair * a.w.w13_sf_pair_stride_bytes + (slot >> 1) * 4;
    } else {
        p.bc = a.w.w2 + e * a.w.w2_expert_stride_bytes + pair * a.w.w2_pair_stride_bytes + slot * 16;
        p.bs = a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + pair * a.w.w2_sf_pair_stride_bytes + (slot >> 1) * 4;
    }

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.0f;

    // ring slot k % kAhead holds k-tile k; k-tile 0's B is decoded into buffer 0
    TileRegs ring[kAhead];
#pragma unroll
    for (int d = 0; d < kAhead; ++d) tile_load(ring[d], p, d);
    store_b(ring[0], Bs0, bp, slot);
    __syncthreads();

    // iteration c: MFMAs of k-tile c (A from ring slot c, B from buffer c & 1),
    // B of k-tile c + 1 into the other buffer, ring slot c reloaded with k-tile
    // c + kAhead. Branch-free, one scheduling region per k-tile: past the end
    // the ring reloads the last k-tile (in bounds, unused) and the last
    // iteration decodes into the buffer nobody reads again. KT % kAhead == 0.
    for (int c0 = 0; c0 < KT; c0 += kAhead) {
#pragma unroll
        for (int d = 0; d < kAhead; ++d) {
            const int c = c0 + d;
            _Float16 (*Bcur)[kLdsRow] = (d & 1) ? Bs1 : Bs0;     // kAhead is even
            _Float16 (*Bnxt)[kLdsRow] = (d & 1) ? Bs0 : Bs1;
            tile_mfma(ring[d], Bcur, wn, lane, acc);
            store_b(ring[(d + 1) % kAhead], Bnxt, bp, slot);
            tile_load(ring[d], p, min(c + kAhead, KT - 1));
            __syncthreads();
        }
    }

    // epilogue: lane l of a 32 x 32 tile holds column l % 32, rows 8(x/4) + 4(l/32) + x%4
    const int n = lane & 31;
    if (MODE == 1) {
        const float ga = a.w.g1_alphas[e], uc = a.w.g1_scale_c[e];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int pr = by * 4 + wn * 2 + j;          // pair = intermediates [16 pr, 16 pr + 16)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int m = wm * 64 + i * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
                    const float g = acc[i][j][x] * ga;                       // gate: lanes n < 16
                    const float u = __shfl_xor(acc[i][j][x], 16) * uc;       // up from lane n + 16
                    const float hv = g / (1.0f + expf(-g)) * u;
                    const float amax = wave_max16(__builtin_fabsf(hv));
                    const BlockScale bsc = nvfp4_block_scale(amax, 1.0f);
                    const uint32_t code = nvfp4_code(hv, bsc);
                    uint32_t b = code | (__shfl_xor(code, 1) << 4);
                    b = b | (__shfl_xor(b, 2) << 8);
                    b = b | (__shfl_xor(b, 4) << 16);
                    if (n < 16 && s_valid[m]) {
                        const int64_t row = row0 + m;
                        if ((n & 7) == 0)
                            *reinterpret_cast<uint32_t*>(a.inter_codes + row * (a.I >> 1) + pr * 8 + (n >> 1)) = b;
                        if (n == 0) a.inter_sf[row * (a.I >> 4) + pr] = (uint8_t)bsc.byte;
                    }
                }
            }
        }
    } else {
        const float alpha = a.w.g2_alphas[e];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = (by * 4 + wn * 2 + j) * 32 + n;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int m = wm * 64 + i * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
                    if (s_valid[m])
                        a.rows[(int64_t)(row0 + m) * a.rows_stride + col] =
                            (uint16_t)f32_to_bf16(acc[i][j][x] * alpha);
                }
            }
        }
    }
}

bool tiled_shape_ok(int H, int I, int tile_m) {
    return tile_m % kTM == 0 && H % 256 == 0 && I % 256 == 0;
}

void launch_tiled(const ExpArgs& a, hipStream_t s) {
    const int nx = (int)(a.L.rows_max / kTM);
    const int ny1 = 2 * a.I / kTN, ny2 = a.H / kTN;
    auto grid = [](int blocks) { return dim3((unsigned)((blocks + kXcds - 1) / kXcds * kXcds)); };
    hipLaunchKernelGGL(tiled_kernel<1>, grid(nx * ny1), dim3(kTiledThreads), 0, s, a, nx, ny1);
    hipLaunchKernelGGL(tiled_kernel<2>, grid(nx * ny2), dim3(kTiledThreads), 0, s, a, nx, ny2);
}

}  // namespace moe
