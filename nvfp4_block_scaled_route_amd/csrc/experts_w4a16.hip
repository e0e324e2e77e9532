// moe_experts_fwd_w4a16: the W4A16 variant of the routed experts -- bf16
// activations against the same converted NVFP4 weights (the runner page,
// "MuseSparkModelOptNvFp4FusedMoE": route-major W4A16 GEMMs with SwiGLU;
// "_process_hopper_marlin_weights": one global scale, the gate's, for both
// halves of w13, and the up side's ratio up/gate folded into GEMM2's scale).
//
//   GEMM1  acc1 = x(t) . dq(w13[e])^T         x: the bf16 input row of token t
//   act    h = bf16(silu(acc_gate * s13[e]) * (acc_up * s13[e]))
//   GEMM2  rows = bf16(h . dq(w2[e])^T * s2[e])
//
// Operands: a bf16 activation times an NVFP4 weight (e2m1 * e4m3: at most 6
// significant bits, between 2^-10 and 2688) is exact in fp32, so both GEMMs run
// v_mfma_f32_16x16x32_bf16. The weight decode is exact too: 8 codes to fp32 at
// scale 1, times the e4m3 block scale in fp32 (the hardware conversion applies
// only its scale operand's exponent), then packed to bf16 (exact: 6 bits).
// The K index is permuted as in the W4A4 kernels: lane (q, n) takes 16-element
// block q of every 64-wide k-tile, for row n of both operands, so the weight
// slot of the converted layout is again one 16-byte load; the activation block
// is 32 bytes of row n.
//
// Decode is bound by the weight stream; one wave is one unit (16 routed rows x
// one gate/up pair for GEMM1, 16 rows x 32 output columns for GEMM2) over all of
// K through a D-stage register pipeline, activations read from the cache (they
// are 64 times smaller than the weights at decode).
#include "experts.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kW16Threads = 256;   // 4 independent waves per workgroup
constexpr int kCacheSc1 = 16;      // buffer-instruction cache policy: agent-coherent (sc1)

struct W16Args {
    const uint16_t* x;          // GEMM1: bf16 [T, x_row_stride]; GEMM2: the intermediate
    int64_t x_row_stride;
    ExpArgs e;                  // metadata, weights (g1_alphas = s13, g2_alphas = s2), shape, rows
    uint16_t* inter;            // bf16 [rows_max, I]
};

// A lane's weight operands of one k-tile: 16 elements (block q) of its row in
// both halves (half 0, half 1), as they arrive from memory.
template <bool kBf16> struct WSlot;
template <> struct WSlot<false> {   // NVFP4: the converted layout's 16-byte slot and its 2 scale bytes
    uint4 w;         // half 0 elements 0-7, 8-15, half 1 elements 0-7, 8-15
    uint32_t wsf;    // e4m3 scales of half 0 (bits 0-7) and half 1 (bits 8-15)
};
template <> struct WSlot<true> {    // bf16: 32 bytes of each half's row
    uint4 h0a, h0b, h1a, h1b;
};

template <bool kBf16>
struct W16Stage {
    WSlot<kBf16> w;
    uint4 a0, a1;    // bf16 activation elements 0-7 and 8-15 of the lane's block
};

// NVFP4: p0 = the lane's slot, p1 = its scale bytes (k-tile c at + 1024 c, + 128 c).
// bf16: p0, p1 = the lane's block in the half-0 and half-1 rows (k-tile c at + 128 c).
struct W16Streams {
    const uint8_t* p0;
    const uint8_t* p1;
    const uint16_t* a;          // k-tile c at + 64 c elements
};

template <bool kBf16>
__device__ __forceinline__ void w16_load_w(W16Stage<kBf16>& st, const W16Streams& p, int c) {
    if constexpr (kBf16) {
        // plain loads: on the bf16 rows (two 32-byte pieces of two rows a lane)
        // the non-temporal hint measured slower (decode_b8 95 vs 91 us)
        const uint4* r0 = reinterpret_cast<const uint4*>(p.p0 + (int64_t)c * 128);
        const uint4* r1 = reinterpret_cast<const uint4*>(p.p1 + (int64_t)c * 128);
        st.w.h0a = r0[0];
        st.w.h0b = r0[1];
        st.w.h1a = r1[0];
        st.w.h1b = r1[1];
    } else {
        st.w.w = load_stream16(p.p0 + (int64_t)c * kSlotBytes);
        st.w.wsf = load_stream2(p.p1 + (int64_t)c * kSlotSfBytes);
    }
}

template <bool kBf16>
__device__ __forceinline__ void w16_load(W16Stage<kBf16>& st, const W16Streams& p, int c) {
    w16_load_w<kBf16>(st, p, c);
    const uint4* a = reinterpret_cast<const uint4*>(p.a + c * 64);
    st.a0 = a[0];
    st.a1 = a[1];
}

// 8 e2m1 codes times one fp32 block scale -> 8 exact bf16 values.
template <int B>
__device__ __forceinline__ void fp4x2_to_bf16(uint32_t codes, float s, bf16x8& out) {
    const floatx2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, B);
    out[2 * B] = (__bf16)__fmul_rn(f[0], s);
    out[2 * B + 1] = (__bf16)__fmul_rn(f[1], s);
}

__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t codes, float s) {
    bf16x8 out;
    fp4x2_to_bf16<0>(codes, s, out);
    fp4x2_to_bf16<1>(codes, s, out);
    fp4x2_to_bf16<2>(codes, s, out);
    fp4x2_to_bf16<3>(codes, s, out);
    return out;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

template <bool kBf16>
__device__ __forceinline__ void w16_use(const W16Stage<kBf16>& st, floatx4& acc0, floatx4& acc1) {
    const bf16x8 a0 = as_bf16x8(st.a0), a1 = as_bf16x8(st.a1);
    bf16x8 w0a, w0b, w1a, w1b;
    if constexpr (kBf16) {
        w0a = as_bf16x8(st.w.h0a); w0b = as_bf16x8(st.w.h0b);
        w1a = as_bf16x8(st.w.h1a); w1b = as_bf16x8(st.w.h1b);
    } else {
        const floatx2 s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(st.w.wsf, 1.0f, false);
        w0a = fp4x8_to_bf16(st.w.w.x, s[0]); w0b = fp4x8_to_bf16(st.w.w.y, s[0]);
        w1a = fp4x8_to_bf16(st.w.w.z, s[1]); w1b = fp4x8_to_bf16(st.w.w.w, s[1]);
    }
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, w0a, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, w1a, acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, w0b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, w1b, acc1, 0, 0, 0);
}

// All KT k-tiles through a D-deep pipeline (KT % D == 0); loads of a stage
// issue together and in stage order (vmcnt drains in issue order).
template <bool kBf16, int D>
__device__ __forceinline__ void w16_stream(const W16Streams& p, int KT, floatx4& acc0, floatx4& acc1) {
    W16Stage<kBf16> st[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        w16_load<kBf16>(st[d], p, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    int c0 = 0;
    for (; c0 + D < KT; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            w16_use<kBf16>(st[d], acc0, acc1);
            w16_load<kBf16>(st[d], p, c0 + D + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        w16_use<kBf16>(st[d], acc0, acc1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// GEMM1 epilogue: lane (q, n) holds rows 4q + i of intermediate 16j + n.
// kPub: GEMM2 workgroups of the same launch read the intermediate, so it is
// written with agent-coherent stores.
template <bool kBf16, bool kPub = false>
__device__ __forceinline__ void w16_gemm1_epilogue(const W16Args& a, const RowTile& rt, int ex, int j, int n, int q,
                                                   const floatx4& acc_g, const floatx4& acc_u) {
    const ExpArgs& e = a.e;
    const float s13 = kBf16 ? 1.0f : e.w.g1_alphas[ex];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        const float g = __fmul_rn(acc_g[i], s13);
        const float u = __fmul_rn(acc_u[i], s13);
        // silu(g) = g * sigmoid(g) with sigmoid from e^-|g| (never overflows): a
        // bf16 intermediate keeps the tiny values of strongly negative gates,
        // which g / (1 + e^-g) would flush to zero once e^-g overflows
        const float eg = expf(-__builtin_fabsf(g));
        const float sig = __fdiv_rn(g >= 0.0f ? 1.0f : eg, __fadd_rn(1.0f, eg));
        const float h = __fmul_rn(__fmul_rn(g, sig), u);
        if ((rt.vmask >> m) & 1u) {
            uint16_t* dst = a.inter + (int64_t)(rt.row0 + m) * e.I + j * 16 + n;
            if (kPub) __hip_atomic_store(dst, (uint16_t)f32_to_bf16(h), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = (uint16_t)f32_to_bf16(h);
        }
    }
}

// GEMM1 unit (16 routed rows, intermediate pair j); lane (q, n) ends with rows
// 4q + i of intermediate 16j + n, gate and up. bf16 weights: w13 [E, 2I, H],
// gate rows first; no global scales.
template <bool kBf16, int D>
__global__ void __launch_bounds__(kW16Threads) w16_gemm1_kernel(W16Args a) {
    const ExpArgs& e = a.e;
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * (kW16Threads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n1 = e.I >> 4;
    const int sub = (int)(unit / n1), j = (int)(unit - sub * n1);
    const RowTile rt = row_tile(e, sub, n);
    if (rt.e < 0) return;
    const int ex = rt.e;
    W16Streams p;
    if constexpr (kBf16) {
        const uint8_t* w13 = e.w.w13 + ex * e.w.w13_expert_stride_bytes;
        p.p0 = w13 + ((int64_t)(16 * j + n) * e.H + 16 * q) * 2;
        p.p1 = w13 + ((int64_t)(e.I + 16 * j + n) * e.H + 16 * q) * 2;
    } else {
        p.p0 = e.w.w13 + ex * e.w.w13_expert_stride_bytes + j * e.w.w13_pair_stride_bytes + lane * 16;
        p.p1 = e.w.w13_sf + ex * e.w.w13_sf_expert_stride_bytes + j * e.w.w13_sf_pair_stride_bytes + lane * 2;
    }
    const int64_t tok = rt.tok >= 0 ? rt.tok : 0;   // padding rows read token 0's row, never written
    p.a = a.x + tok * a.x_row_stride + q * 16;
    floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
    w16_stream<kBf16, D>(p, e.H >> 6, acc_g, acc_u);
    w16_gemm1_epilogue<kBf16>(a, rt, ex, j, n, q, acc_g, acc_u);
}

// GEMM2 epilogue: lane (q, n) holds rows 4q + i of columns 32c + n and 32c + 16 + n.
template <bool kBf16>
__device__ __forceinline__ void w16_gemm2_epilogue(const ExpArgs& e, const RowTile& rt, int ex, int c, int n, int q,
                                                   const floatx4& acc0, const floatx4& acc1) {
    const float alpha = kBf16 ? 1.0f : e.w.g2_alphas[ex];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        if ((rt.vmask >> m) & 1u) {
            uint16_t* out = e.rows + (int64_t)(rt.row0 + m) * e.rows_stride + c * 32 + n;
            out[0] = (uint16_t)f32_to_bf16(__fmul_rn(acc0[i], alpha));
            out[16] = (uint16_t)f32_to_bf16(__fmul_rn(acc1[i], alpha));
        }
    }
}

// GEMM2 unit (16 routed rows, output pair c: columns 32c + n and 32c + 16 + n)
// on the bf16 intermediate. bf16 weights: w2 [E, H, I]; no global scale.
template <bool kBf16, int D>
__global__ void __launch_bounds__(kW16Threads) w16_gemm2_kernel(W16Args a) {
    const ExpArgs& e = a.e;
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * (kW16Threads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n2 = e.H >> 5;
    const int sub = (int)(unit / n2), c = (int)(unit - sub * n2);
    const RowTile rt = row_tile(e, sub, n);
    if (rt.e < 0) return;
    const int ex = rt.e;
    W16Streams p;
    if constexpr (kBf16) {
        const uint8_t* w2 = e.w.w2 + ex * e.w.w2_expert_stride_bytes;
        p.p0 = w2 + ((int64_t)(32 * c + n) * e.I + 16 * q) * 2;
        p.p1 = w2 + ((int64_t)(32 * c + 16 + n) * e.I + 16 * q) * 2;
    } else {
        p.p0 = e.w.w2 + ex * e.w.w2_expert_stride_bytes + c * e.w.w2_pair_stride_bytes + lane * 16;
        p.p1 = e.w.w2_sf + ex * e.w.w2_sf_expert_stride_bytes + c * e.w.w2_sf_pair_stride_bytes + lane * 2;
    }
    p.a = a.inter + (int64_t)(rt.row0 + n) * e.I + q * 16;
    floatx4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    w16_stream<kBf16, D>(p, e.I >> 6, acc0, acc1);
    w16_gemm2_epilogue<kBf16>(e, rt, ex, c, n, q, acc0, acc1);
}

// ---------------------------------------------------------------- four units per workgroup
// A workgroup's four waves take four units of one 16-row tile and share its
// activation rows through LDS, staged 256 columns (4 k-tiles, 8 KB of bf16) at
// a time in two buffers: while the waves run chunk c from one buffer, the
// workgroup's loads of chunk c + 1 are in flight and land in the other, one
// barrier a chunk. Without it every wave read its rows' 32-byte blocks from the
// cache itself -- 16 rows x 2 KB per k-tile per wave beside its weight slot.
// Rows are 528 bytes apart in LDS (256 bf16 + 16 bytes): a k-tile's 16-byte
// reads by 16 lanes of one q (16 rows, one column) then fall on 16 distinct
// groups of 4 banks. The weights stream through a register pipeline of D
// stages (whole chunks) across the chunks.
constexpr int kW16Chunk = 256;                  // columns per LDS chunk
constexpr int kW16RowBytes = kW16Chunk * 2 + 16;
constexpr int kW16BufBytes = 16 * kW16RowBytes;

// 16 bytes of a staged row: plain, or agent-coherent (sc1: the row was
// published by another XCD in this launch) through a buffer load on `base`.
template <bool kCoh>
__device__ __forceinline__ u32x4 w16_row16(const uint16_t* base, const uint16_t* p) {
    if constexpr (kCoh) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
        return __builtin_amdgcn_raw_buffer_load_b128(r, (int)((p - base) * 2), 0, kCacheSc1);
    } else {
        return *reinterpret_cast<const u32x4*>(p);
    }
}

// The chunk loop of w16_wg_run once chunk 0 is in LDS and the first D weight
// k-tiles are in flight in st: s0, s1 hold this thread's 32 bytes of chunk 1.
template <bool kBf16, int D, bool kCoh>
__device__ __forceinline__ void w16_wg_loop(W16Stage<kBf16> (&st)[D], const W16Streams& p, const uint16_t* base,
                                            const uint16_t* srow, int KT, uint8_t* lds, u32x4 s0, u32x4 s1,
                                            floatx4& acc0, floatx4& acc1) {
    constexpr int CK = kW16Chunk / 64;          // k-tiles per chunk
    constexpr int H = D / CK;                   // chunks per pass over the pipeline
    const int lane = threadIdx.x & 63, t = threadIdx.x;
    const int NC = KT / CK;
    uint8_t* wpos = lds + (t >> 4) * kW16RowBytes + (t & 15) * 32;
    const uint8_t* rpos = lds + (lane & 15) * kW16RowBytes + (lane >> 4) * 32;
    const uint16_t* src = srow + (t & 15) * 16;
    for (int c0 = 0; c0 < NC; c0 += H) {
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int c = c0 + h;
            const uint8_t* buf = rpos + (c & 1) * kW16BufBytes;
#pragma unroll
            for (int d = 0; d < CK; ++d) {
                W16Stage<kBf16>& sd = st[CK * h + d];
                sd.a0 = *reinterpret_cast<const uint4*>(buf + d * 128);
                sd.a1 = *reinterpret_cast<const uint4*>(buf + d * 128 + 16);
                w16_use<kBf16>(sd, acc0, acc1);
                if (CK * c + d + D < KT) w16_load_w<kBf16>(sd, p, CK * c + d + D);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (c + 1 < NC) {
                u32x4* nxt = reinterpret_cast<u32x4*>(wpos + ((c + 1) & 1) * kW16BufBytes);
                nxt[0] = s0;
                nxt[1] = s1;
            }
            __syncthreads();
            if (c + 2 < NC) {
                s0 = w16_row16<kCoh>(base, src + (c + 2) * kW16Chunk);
                s1 = w16_row16<kCoh>(base, src + (c + 2) * kW16Chunk + 8);
            }
        }
    }
}

// Runs all KT k-tiles (KT % D == 0): the weights stream D k-tiles ahead (4,
// one chunk, or 8, two), the activations one chunk ahead. srow: the bf16 row
// this thread stages (row threadIdx.x / 16 of the tile), 32 bytes at column
// 16 (threadIdx.x % 16) of each chunk.
template <bool kBf16, int D>
__device__ __forceinline__ void w16_wg_run(const W16Streams& p, const uint16_t* srow, int KT, uint8_t* lds,
                                           floatx4& acc0, floatx4& acc1) {
    constexpr int CK = kW16Chunk / 64;
    static_assert(D % CK == 0, "the pipeline holds whole chunks");
    const int t = threadIdx.x;
    const int NC = KT / CK;
    uint8_t* wpos = lds + (t >> 4) * kW16RowBytes + (t & 15) * 32;
    const uint16_t* src = srow + (t & 15) * 16;
    W16Stage<kBf16> st[D];
    // chunk 0's rows, then the first weights and chunk 1's rows go out before
    // chunk 0 is stored, so that their latencies overlap
    const u32x4 f0 = w16_row16<false>(srow, src), f1 = w16_row16<false>(srow, src + 8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        w16_load_w<kBf16>(st[d], p, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 s0 = f0, s1 = f1;
    if (NC > 1) {
        s0 = w16_row16<false>(srow, src + kW16Chunk);
        s1 = w16_row16<false>(srow, src + kW16Chunk + 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    reinterpret_cast<u32x4*>(wpos)[0] = f0;
    reinterpret_cast<u32x4*>(wpos)[1] = f1;
    __syncthreads();
    w16_wg_loop<kBf16, D, false>(st, p, srow, srow, KT, lds, s0, s1, acc0, acc1);
}

// GEMM1: the 4 units of a workgroup are intermediate pairs of one tile (I/16
// % 4 == 0); thread t stages the input row of the tile's row t / 16 (gathered
// by token; a padding row stages token 0's row, which feeds no written
// output).
template <bool kBf16, int D>
__global__ void __launch_bounds__(kW16Threads) w16_wg_gemm1_kernel(W16Args a) {
    __shared__ __align__(16) uint8_t lds[2 * kW16BufBytes];
    const ExpArgs& e = a.e;
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * (kW16Threads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n1 = e.I >> 4;
    const int sub = (int)(unit / n1), j = (int)(unit - sub * n1);
    const RowTile rt = row_tile(e, sub, n);     // one tile for the whole workgroup
    if (rt.e < 0) return;
    const int ex = rt.e;
    W16Streams p;
    if constexpr (kBf16) {
        const uint8_t* w13 = e.w.w13 + ex * e.w.w13_expert_stride_bytes;
        p.p0 = w13 + ((int64_t)(16 * j + n) * e.H + 16 * q) * 2;
        p.p1 = w13 + ((int64_t)(e.I + 16 * j + n) * e.H + 16 * q) * 2;
    } else {
        p.p0 = e.w.w13 + ex * e.w.w13_expert_stride_bytes + j * e.w.w13_pair_stride_bytes + lane * 16;
        p.p1 = e.w.w13_sf + ex * e.w.w13_sf_expert_stride_bytes + j * e.w.w13_sf_pair_stride_bytes + lane * 2;
    }
    int tok = e.meta[e.L.perm2tok + rt.row0 + (threadIdx.x >> 4)];
    if (tok < 0 || tok >= e.T) tok = 0;
    floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
    w16_wg_run<kBf16, D>(p, a.x + (int64_t)tok * a.x_row_stride, e.H >> 6, lds, acc_g, acc_u);
    w16_gemm1_epilogue<kBf16>(a, rt, ex, j, n, q, acc_g, acc_u);
}

// GEMM2: the 4 units of a workgroup are output pairs of one tile (H/32 % 4 ==
// 0); the tile's 16 intermediate rows are consecutive.
template <bool kBf16, int D>
__global__ void __launch_bounds__(kW16Threads) w16_wg_gemm2_kernel(W16Args a) {
    __shared__ __align__(16) uint8_t lds[2 * kW16BufBytes];
    const ExpArgs& e = a.e;
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * (kW16Threads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n2 = e.H >> 5;
    const int sub = (int)(unit / n2), c = (int)(unit - sub * n2);
    const RowTile rt = row_tile(e, sub, n);
    if (rt.e < 0) return;
    const int ex = rt.e;
    W16Streams p;
    if constexpr (kBf16) {
        const uint8_t* w2 = e.w.w2 + ex * e.w.w2_expert_stride_bytes;
        p.p0 = w2 + ((int64_t)(32 * c + n) * e.I + 16 * q) * 2;
        p.p1 = w2 + ((int64_t)(32 * c + 16 + n) * e.I + 16 * q) * 2;
    } else {
        p.p0 = e.w.w2 + ex * e.w.w2_expert_stride_bytes + c * e.w.w2_pair_stride_bytes + lane * 16;
        p.p1 = e.w.w2_sf + ex * e.w.w2_sf_expert_stride_bytes + c * e.w.w2_sf_pair_stride_bytes + lane * 2;
    }
    floatx4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    w16_wg_run<kBf16, D>(p, a.inter + (int64_t)(rt.row0 + (threadIdx.x >> 4)) * e.I, e.I >> 6, lds,
                              acc0, acc1);
    w16_gemm2_epilogue<kBf16>(e, rt, ex, c, n, q, acc0, acc1);
}

// Both GEMMs in one launch (H and I multiples of 256; for W4A16, 128 routes or
// more -- w16_launch): workgroups [0, g1_blocks)
// are w16_wg_gemm1_kernel's, the rest w16_wg_gemm2_kernel's, as in the W4A4
// one-launch kernel (experts.hip). A GEMM1 workgroup writes its part of the
// bf16 intermediate with agent-coherent stores, waits until they have
// completed and adds 1 to its tile's ready counter (meta's sub_sync). A GEMM2
// workgroup issues its first weight k-tiles, waits (bounded, sync_status 1 if
// it gives up) until all I/64 GEMM1 workgroups of its tile have added theirs,
// counts itself on the tile's done counter -- the last of the tile's H/128
// returns both counters to 0 -- and stages the intermediate with agent-coherent
// loads. Workgroups are dispatched in index order, so every GEMM1 workgroup
// has been dispatched before a GEMM2 workgroup waits, and GEMM1 waits for
// nothing.
template <bool kBf16>
__global__ void __launch_bounds__(kW16Threads) w16_fused_kernel(W16Args a, uint32_t g1_blocks) {
    constexpr int D = 4;
    __shared__ __align__(16) uint8_t lds[2 * kW16BufBytes];
    const ExpArgs& e = a.e;
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (blockIdx.x < g1_blocks) {
        const uint32_t unit = blockIdx.x * (kW16Threads / 64) + wave;
        const uint32_t n1 = e.I >> 4;
        const int sub = (int)(unit / n1), j = (int)(unit - sub * n1);
        const RowTile rt = row_tile(e, sub, n);     // one tile for the whole workgroup
        if (rt.e < 0) return;
        const int ex = rt.e;
        W16Streams p;
        if constexpr (kBf16) {
            const uint8_t* w13 = e.w.w13 + ex * e.w.w13_expert_stride_bytes;
            p.p0 = w13 + ((int64_t)(16 * j + n) * e.H + 16 * q) * 2;
            p.p1 = w13 + ((int64_t)(e.I + 16 * j + n) * e.H + 16 * q) * 2;
        } else {
            p.p0 = e.w.w13 + ex * e.w.w13_expert_stride_bytes + j * e.w.w13_pair_stride_bytes + lane * 16;
            p.p1 = e.w.w13_sf + ex * e.w.w13_sf_expert_stride_bytes + j * e.w.w13_sf_pair_stride_bytes + lane * 2;
        }
        int tok = e.meta[e.L.perm2tok + rt.row0 + (threadIdx.x >> 4)];
        if (tok < 0 || tok >= e.T) tok = 0;
        floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
        w16_wg_run<kBf16, D>(p, a.x + (int64_t)tok * a.x_row_stride, e.H >> 6, lds, acc_g, acc_u);
        w16_gemm1_epilogue<kBf16, true>(a, rt, ex, j, n, q, acc_g, acc_u);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores have completed
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(e.sync + kSubSyncStride * sub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const uint32_t unit = (blockIdx.x - g1_blocks) * (kW16Threads / 64) + wave;
    const uint32_t n2 = e.H >> 5;
    const int sub = (int)(unit / n2), c = (int)(unit - sub * n2);
    const RowTile rt = row_tile(e, sub, n);
    if (rt.e < 0) return;
    const int ex = rt.e;
    W16Streams p;
    if constexpr (kBf16) {
        const uint8_t* w2 = e.w.w2 + ex * e.w.w2_expert_stride_bytes;
        p.p0 = w2 + ((int64_t)(32 * c + n) * e.I + 16 * q) * 2;
        p.p1 = w2 + ((int64_t)(32 * c + 16 + n) * e.I + 16 * q) * 2;
    } else {
        p.p0 = e.w.w2 + ex * e.w.w2_expert_stride_bytes + c * e.w.w2_pair_stride_bytes + lane * 16;
        p.p1 = e.w.w2_sf + ex * e.w.w2_sf_expert_stride_bytes + c * e.w.w2_sf_pair_stride_bytes + lane * 2;
    }
    W16Stage<kBf16> st[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        w16_load_w<kBf16>(st[d], p, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    int32_t* ready = e.sync + kSubSyncStride * sub;
    if (wave == 0) wait_ready(ready, e.I >> 6, e.status);
    __syncthreads();
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(ready + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (e.H >> 7) - 1) {
        __hip_atomic_store(ready, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ready + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the tile's intermediate rows, staged as in w16_wg_run but agent-coherent
    const int t = threadIdx.x;
    const int KT = e.I >> 6, NC = KT / (kW16Chunk / 64);
    const uint16_t* srow = a.inter + (int64_t)(rt.row0 + (t >> 4)) * e.I;
    const uint16_t* src = srow + (t & 15) * 16;
    const u32x4 f0 = w16_row16<true>(a.inter, src), f1 = w16_row16<true>(a.inter, src + 8);
    u32x4 s0 = f0, s1 = f1;
    if (NC > 1) {
        s0 = w16_row16<true>(a.inter, src + kW16Chunk);
        s1 = w16_row16<true>(a.inter, src + kW16Chunk + 8);
    }
    uint8_t* wpos = lds + (t >> 4) * kW16RowBytes + (t & 15) * 32;
    reinterpret_cast<u32x4*>(wpos)[0] = f0;
    reinterpret_cast<u32x4*>(wpos)[1] = f1;
    __syncthreads();
    floatx4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    w16_wg_loop<kBf16, D, true>(st, p, a.inter, srow, KT, lds, s0, s1, acc0, acc1);
    w16_gemm2_epilogue<kBf16>(e, rt, ex, c, n, q, acc0, acc1);
}

static int w16_depth(int kt, int cap) {
    for (int d = cap; d > 1; d >>= 1)
        if (kt % d == 0) return d;
    return 1;
}

// The checks both variants share; then the two launches. kBf16 stages hold 4x
// the weight bytes of NVFP4 ones, so their pipeline is at most 2 deep (8 KB in
// flight per wave either way).
template <bool kBf16>
static int w16_launch(const char* name, const uint16_t* x, int64_t x_row_stride, int32_t* meta,
                      const moe_nvfp4_weights& w, int T, int K, int E_local, int H, int I, int tile_m,
                      uint16_t* inter, uint16_t* rows, int64_t rows_stride, hipStream_t s) {
    if (x_row_stride < H || x_row_stride % 8)
        return fail(MOE_EINVAL, "%s: x row stride must be >= H and a multiple of 8", name);
    if (rows_stride < H || rows_stride % 8)
        return fail(MOE_EINVAL, "%s: rows_stride must be >= H and a multiple of 8", name);
    W16Args a;
    a.x = x; a.x_row_stride = x_row_stride; a.inter = inter;
    a.e.meta = meta; a.e.L = meta_layout(T, K, E_local, tile_m);
    a.e.w = w; a.e.T = T; a.e.E_local = E_local; a.e.H = H; a.e.I = I; a.e.tile_m = tile_m;
    a.e.rows = rows; a.e.rows_stride = rows_stride;
    a.e.a_codes = nullptr; a.e.a_sf = nullptr; a.e.inter_codes = nullptr; a.e.inter_sf = nullptr;
    a.e.sync = meta + a.e.L.sub_sync; a.e.status = meta + a.e.L.sync_status;
    if (a.e.L.rows_max == 0) return MOE_OK;
    const int64_t subs = a.e.L.rows_max / 16;
    const int64_t units1 = subs * (I / 16), units2 = subs * (H / 32);
    if (units1 > 0x7FFFFFFF || units2 > 0x7FFFFFFF) return fail(MOE_EUNSUPPORTED, "%s: too many work units", name);
    const int wpb = kW16Threads / 64;
    const dim3 g1((unsigned)((units1 + wpb - 1) / wpb)), g2((unsigned)((units2 + wpb - 1) / wpb)), b(kW16Threads);
    const int cap = kBf16 ? 2 : 4;
    // both workgroup forms in one launch where they both apply (and the
    // intermediate's byte offsets fit the coherent loads' 32 bits) and the
    // weight stream is long enough for the hand-over's fixed cost (the
    // intermediate's agent-coherent stores completing, the polls) to pay.
    // Measured, back to back: BF16 at decode_b8 84.7 -> 81.1 us, W4A16 at
    // decode_b64_zipf (512 routes) 132.7 -> 126.5 us, but W4A16 at decode_b8
    // (64 routes, 112 MB of weights) 28.0 -> 28.8 us
    const bool one_launch = kBf16 || (int64_t)T * K >= 128;
    if (one_launch && H % kW16Chunk == 0 && I % kW16Chunk == 0 && a.e.L.rows_max * I * 2 < (1ll << 31)) {
        hipLaunchKernelGGL((w16_fused_kernel<kBf16>), dim3(g1.x + g2.x), b, 0, s, a, g1.x);
        return check_launch(name);
    }
    // the workgroup forms where the shape allows: whole 256-column chunks, and
    // for GEMM2 four output pairs in one tile (H % 128 == 0). The weights
    // stream one chunk (4 k-tiles) ahead: 8 measured no faster, and neither did
    // 8 waves a workgroup sharing one tile's rows.
    if (H % kW16Chunk == 0) {
        hipLaunchKernelGGL((w16_wg_gemm1_kernel<kBf16, 4>), g1, b, 0, s, a);
    } else {
        switch (w16_depth(H / 64, cap)) {
            case 4: hipLaunchKernelGGL((w16_gemm1_kernel<kBf16, 4>), g1, b, 0, s, a); break;
            case 2: hipLaunchKernelGGL((w16_gemm1_kernel<kBf16, 2>), g1, b, 0, s, a); break;
            default: hipLaunchKernelGGL((w16_gemm1_kernel<kBf16, 1>), g1, b, 0, s, a); break;
        }
    }
    int rc = check_launch(name);
    if (rc) return rc;
    if (I % kW16Chunk == 0 && H % 128 == 0) {
        hipLaunchKernelGGL((w16_wg_gemm2_kernel<kBf16, 4>), g2, b, 0, s, a);
    } else {
        switch (w16_depth(I / 64, cap)) {
            case 4: hipLaunchKernelGGL((w16_gemm2_kernel<kBf16, 4>), g2, b, 0, s, a); break;
            case 2: hipLaunchKernelGGL((w16_gemm2_kernel<kBf16, 2>), g2, b, 0, s, a); break;
            default: hipLaunchKernelGGL((w16_gemm2_kernel<kBf16, 1>), g2, b, 0, s, a); break;
        }
    }
    return check_launch(name);
}

static int w16_shape_check(const char* name, int T, int K, int E_local, int H, int I, int tile_m) {
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E_local < 1 || E_local > MOE_MAX_EXPERTS)
        return fail(MOE_EINVAL, "%s: T=%d K=%d E_local=%d out of range", name, T, K, E_local);
    if (H < 64 || H % 64 || I < 64 || I % 64 || H > MOE_MAX_HIDDEN || I > MOE_MAX_HIDDEN)
        return fail(MOE_EUNSUPPORTED, "%s: H=%d and I=%d must be multiples of 64 up to %d", name, H, I,
                    MOE_MAX_HIDDEN);
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return fail(MOE_EUNSUPPORTED, "%s: tile_m=%d must be a multiple of 16 in [16, 256]", name, tile_m);
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_experts_fwd_w4a16(const uint16_t* x, int64_t x_row_stride, int32_t* meta,
                                     const moe_nvfp4_weights* w, int T, int K, int E_local, int H, int I,
                                     int tile_m, uint16_t* inter, uint16_t* rows, int64_t rows_stride,
                                     void* stream) {
    using namespace moe;
    const char* name = "moe_experts_fwd_w4a16";
    int rc = w16_shape_check(name, T, K, E_local, H, I, tile_m);
    if (rc) return rc;
    if (!w || !meta) return fail(MOE_EINVAL, "%s: NULL weights or meta", name);
    if (T == 0) return MOE_OK;
    if (!x || !inter || !rows) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    const void* ptrs[] = {x, meta, inter, rows};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    if (int rc = check_weights(w, H, I, false, name)) return rc;
    return w16_launch<false>(name, x, x_row_stride, meta, *w, T, K, E_local, H, I, tile_m, inter, rows,
                             rows_stride, (hipStream_t)stream);
}

extern "C" int moe_experts_fwd_bf16(const uint16_t* x, int64_t x_row_stride, int32_t* meta,
                                    const uint16_t* w13, const uint16_t* w2, int T, int K, int E_local, int H,
                                    int I, int tile_m, uint16_t* inter, uint16_t* rows, int64_t rows_stride,
                                    void* stream) {
    using namespace moe;
    const char* name = "moe_experts_fwd_bf16";
    int rc = w16_shape_check(name, T, K, E_local, H, I, tile_m);
    if (rc) return rc;
    if (!meta) return fail(MOE_EINVAL, "%s: NULL meta", name);
    if (T == 0) return MOE_OK;
    if (!x || !w13 || !w2 || !inter || !rows) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    const void* ptrs[] = {x, meta, w13, w2, inter, rows};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    moe_nvfp4_weights w = {};
    w.w13 = reinterpret_cast<const uint8_t*>(w13);
    w.w2 = reinterpret_cast<const uint8_t*>(w2);
    w.w13_expert_stride_bytes = (int64_t)2 * I * H * 2;
    w.w2_expert_stride_bytes = (int64_t)H * I * 2;
    return w16_launch<true>(name, x, x_row_stride, meta, w, T, K, E_local, H, I, tile_m, inter, rows, rows_stride,
                            (hipStream_t)stream);
}
