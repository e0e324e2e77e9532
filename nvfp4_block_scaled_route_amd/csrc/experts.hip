// moe_experts_fwd: the routed experts up to the GEMM2 rows -- the runner page,
// "MuseSparkTrtLlmNvFp4Experts.apply_routed" (TRT-LLM-gen op, do_finalize=False);
// the flashinfer_ops page, "routed_experts_from_metadata".
//
//   GEMM1  acc1 = A(t) . w13[e]^T       A: NVFP4 input row of token t
//   act    h = silu(acc_gate * g1_alphas[e]) * (acc_up * g1_scale_c[e]),
//          requantized to NVFP4 along I with global scale 1 (the intermediate's
//          global scale is folded into g1_scale_c: the runner page,
//          "process_weights_after_loading")
//   GEMM2  rows = bf16(hq . w2[e]^T * g2_alphas[e])
//
// Operands: every NVFP4 element e2m1 * e4m3 is exact in f16, so both GEMMs run
// v_mfma_f32_16x16x32_f16 with fp32 accumulation; both operands are decoded in
// registers from their codes (a pack-convert of 8 codes and one packed multiply
// by the block's e4m3 scale). Each lane of a wave owns whole 16-element blocks
// of K (lane (q, n) takes block q of every 64-wide k-tile, for row n of both
// operands), so one scale byte per operand and k-tile serves a lane, and the
// weight layout puts a lane's block of both row halves in one 16-byte slot.
//
// Decode is bound by the weight stream, so the kernels are built to keep HBM
// busy: one wave is one work unit, computes all of K on its own and writes its
// results itself -- no workgroup barrier, no cross-wave reduction. Units:
//   GEMM1 (16 routed rows, intermediate pair j): the 16 gate and 16 up weight
//     rows of intermediates [16j, 16j + 16) over K = H, so the SwiGLU and the
//     16-wide NVFP4 block of the requant complete in the wave;
//   GEMM2 (16 routed rows, output pair c): 32 output columns over K = I.
// A wave streams its unit's k-tiles through a D-stage register pipeline: the
// loads of k-tile c + D (16-byte weight slot, 2 weight scale bytes, 8 activation
// code bytes, 1 activation scale byte) are issued right after k-tile c is
// consumed, so D k-tiles of every wave are in flight at all times.
// Units are numbered row tile major; a unit finds its expert in the tile's
// metadata entry, which is -1 for every tile past the routed ones, so those
// waves exit at once. The expert kernels never read expert counts: a 16-row
// tile's padding rows have token -1 and are neither read nor written.
//
// Where the shape allows, a workgroup's four waves take four units of one tile
// and share one copy of the tile's 16 activation rows in LDS, brought in by
// direct-to-LDS loads issued ahead of the weight pipeline: a wave's k-tile then
// requests only its 16-byte weight slot and 2 scale bytes from memory, not 16
// rows x (8 code bytes + 1 scale byte) spread over 32 cache lines, which leaves
// a CU's memory requests to the weights.
#include <mutex>

#include "experts.hpp"
#include "finalize.hpp"

namespace moe {

constexpr int kThreads = 256;              // 4 independent waves per workgroup
constexpr int kWavesPerBlock = kThreads / 64;

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One k-tile's operands of one lane.
struct Stage {
    uint4 w;        // weight slot: half 0 elements 0-7, 8-15, half 1 elements 0-7, 8-15
    uint32_t wsf;   // scale bytes of half 0 (bits 0-7) and half 1 (bits 8-15)
    uint2 a;        // activation block: elements 0-7, 8-15
    uint32_t asf;   // its scale byte
};

// Per-lane operand pointers of one unit; k-tile c is at +c * {1024, 128, 32, 4}.
// A lane whose activation row holds no route reads an in-bounds stand-in row:
// row m of an MFMA product depends on row m of A only, and such rows are never
// written, so their values do not matter (and nothing has to wait to mask them).
struct Streams {
    const uint8_t* wc;
    const uint8_t* ws;
    const uint8_t* ac;
    const uint8_t* as;
};

__device__ __forceinline__ void load_w(Stage& st, const Streams& p, int c) {
    st.w = load_stream16(p.wc + (int64_t)c * kSlotBytes);
    st.wsf = load_stream2(p.ws + (int64_t)c * kSlotSfBytes);
}

__device__ __forceinline__ void load_stage(Stage& st, const Streams& p, int c) {
    load_w(st, p, c);
    st.a = *reinterpret_cast<const uint2*>(p.ac + c * 32);
    st.asf = p.as[c * 4];
}

// acc0 += A . half0^T, acc1 += A . half1^T over one k-tile (two MFMA steps).
__device__ __forceinline__ void use_stage(const Stage& st, floatx4& acc0, floatx4& acc1) {
    const half2v ws = e4m3x2_to_f16(st.wsf);
    const half2v as = splat_lo(e4m3x2_to_f16(st.asf));
    const half2v s0 = splat_lo(ws), s1 = splat_hi(ws);
    {
        const half8 a = nvfp4x8_to_f16(st.a.x, as);
        acc0 = mfma16(a, nvfp4x8_to_f16(st.w.x, s0), acc0);
        acc1 = mfma16(a, nvfp4x8_to_f16(st.w.z, s1), acc1);
    }
    {
        const half8 a = nvfp4x8_to_f16(st.a.y, as);
        acc0 = mfma16(a, nvfp4x8_to_f16(st.w.y, s0), acc0);
        acc1 = mfma16(a, nvfp4x8_to_f16(st.w.w, s1), acc1);
    }
}

// All KT k-tiles of one unit through a D-deep pipeline (KT % D == 0, KT >= D).
template <int D>
__device__ __forceinline__ void stream_unit(const Streams& p, int KT, floatx4& acc0, floatx4& acc1) {
    Stage st[D];
    // Every stage's four loads issue together and in stage order, here and in
    // the loop, so that consuming stage d waits only for the loads issued before
    // it: vmcnt drains in issue order.
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_stage(st[d], p, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int c0 = 0; c0 + D < KT; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            use_stage(st[d], acc0, acc1);
            load_stage(st[d], p, c0 + D + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        use_stage(st[d], acc0, acc1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------- epilogues
// Agent-coherent stores (sc1): visible to agent-coherent loads on every XCD
// once they have completed, without a write-back of the writer's L2.
__device__ __forceinline__ void store_u32_sc1(uint8_t* p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_u8_sc1(uint8_t* p, uint8_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// GEMM1: lane (q, n) holds rows 4q + i of intermediate 16j + n. kPublish: the
// intermediate is handed to GEMM2 workgroups of the same launch, so it is
// written with agent-coherent stores.
template <bool kPublish = false>
__device__ __forceinline__ void gemm1_epilogue(const ExpArgs& a, const RowTile& rt, int e, int j, int n, int q,
                                               const floatx4& acc_g, const floatx4& acc_u) {
    const float ga = a.w.g1_alphas[e], uc = a.w.g1_scale_c[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        const float g = acc_g[i] * ga;
        const float u = acc_u[i] * uc;
        const float h = g / (1.0f + expf(-g)) * u;
        const float amax = wave_max16(__builtin_fabsf(h));
        const BlockScale bs = nvfp4_block_scale(amax, 1.0f);
        const uint32_t code = nvfp4_code(h, bs);
        uint32_t b = code | (__shfl_xor(code, 1) << 4);      // even n: byte n/2
        b = b | (__shfl_xor(b, 2) << 8);                      // n % 4 == 0: 2 bytes
        b = b | (__shfl_xor(b, 4) << 16);                     // n % 8 == 0: 4 bytes
        if ((rt.vmask >> m) & 1u) {
            const int64_t row = rt.row0 + m;
            uint8_t* cp = a.inter_codes + row * (a.I >> 1) + j * 8 + (n >> 1);
            uint8_t* sp = a.inter_sf + row * (a.I >> 4) + j;
            if (kPublish) {
                if ((n & 7) == 0) store_u32_sc1(cp, b);
                if (n == 0) store_u8_sc1(sp, (uint8_t)bs.byte);
            } else {
                if ((n & 7) == 0) *reinterpret_cast<uint32_t*>(cp) = b;
                if (n == 0) *sp = (uint8_t)bs.byte;
            }
        }
    }
}

// ---------------------------------------------------------------- one unit per wave
// Activation rows read by every wave from global memory: the kernels for the
// shapes the workgroup kernels below do not take.
template <int D>
__global__ void __launch_bounds__(kThreads) gemm1_kernel(ExpArgs a) {
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n1 = a.I >> 4;
    const int sub = (int)(unit / n1), j = (int)(unit - sub * n1);
    const RowTile rt = row_tile(a, sub, n);
    if (rt.e < 0) return;
    const int e = rt.e;
    Streams p;
    p.wc = a.w.w13 + e * a.w.w13_expert_stride_bytes + j * a.w.w13_pair_stride_bytes + lane * 16;
    p.ws = a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + j * a.w.w13_sf_pair_stride_bytes + lane * 2;
    const int64_t tok = rt.tok >= 0 ? rt.tok : 0;
    p.ac = a.a_codes + tok * (a.H >> 1) + q * 8;
    p.as = a.a_sf + tok * (a.H >> 4) + q;
    floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
    stream_unit<D>(p, a.H >> 6, acc_g, acc_u);
    gemm1_epilogue(a, rt, e, j, n, q, acc_g, acc_u);
}

template <int D>
__global__ void __launch_bounds__(kThreads) gemm2_kernel(ExpArgs a) {
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n2 = a.H >> 5;
    const int sub = (int)(unit / n2), c = (int)(unit - sub * n2);
    const RowTile rt = row_tile(a, sub, n);
    if (rt.e < 0) return;
    const int e = rt.e;
    Streams p;
    p.wc = a.w.w2 + e * a.w.w2_expert_stride_bytes + c * a.w.w2_pair_stride_bytes + lane * 16;
    p.ws = a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + c * a.w.w2_sf_pair_stride_bytes + lane * 2;
    const int64_t row = rt.row0 + n;   // the intermediate is in permuted row order
    p.ac = a.inter_codes + row * (a.I >> 1) + q * 8;
    p.as = a.inter_sf + row * (a.I >> 4) + q;
    floatx4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    stream_unit<D>(p, a.I >> 6, acc0, acc1);
    gemm2_epilogue(a, rt, e, c, n, q, acc0, acc1);
}

// ---------------------------------------------------------------- four units per workgroup
// The tile's 16 activation rows (K values each: K/2 code bytes, K/16 scale
// bytes) in LDS as 16-byte chunks, chunk-major: code chunk k of row r at
// 16 (16 k + r), scale chunk k of row r at 16 (K/2 + 16 k + r). A k-tile's
// reads (row n, 8 code bytes at 32c + 8q and scale byte 4c + q for lane
// (q, n)) then fall on distinct banks.
__host__ __device__ constexpr int tile_lds_bytes(int K) { return 8 * K + K; }

// Issue the copy of the tile: chunk x of each region goes to LDS unit x, so
// one direct-to-LDS load moves 64 consecutive units, lane l taking row l % 16
// (a lane of a 16-row MFMA tile, whose row base `cbase`/`sbase` it holds).
// The four waves take every fourth load.
// kCoherent: agent-coherent loads (a tile another XCD published in this launch).
template <bool kCoherent = false>
__device__ __forceinline__ void copy_tile(uint8_t* lds, int K, int wave, int lane, u32x4 crsrc, uint32_t cbase,
                                          u32x4 srsrc, uint32_t sbase) {
    const int code_chunks = K >> 1, sf_chunks = K >> 4;   // 16 rows x (K/32) and 16 rows x (K/256)
    const uint32_t l0 = lds_addr(lds);
    const uint32_t k = (uint32_t)(lane >> 4);
    for (int x0 = wave * 64; x0 < code_chunks; x0 += kThreads) {
        const uint32_t l = __builtin_amdgcn_readfirstlane(l0 + x0 * 16), v = cbase + ((x0 >> 4) + k) * 16;
        if (kCoherent) lds_copy16_sc1(crsrc, l, v, 0);
        else lds_copy16(crsrc, l, v, 0);
    }
    for (int x0 = wave * 64; x0 < sf_chunks; x0 += kThreads)
        if (x0 + lane < sf_chunks) {
            const uint32_t l = __builtin_amdgcn_readfirstlane(l0 + (code_chunks + x0) * 16);
            const uint32_t v = sbase + ((x0 >> 4) + k) * 16;
            if (kCoherent) lds_copy16_sc1(srsrc, l, v, 0);
            else lds_copy16(srsrc, l, v, 0);
        }
}

// A wave's loads of the copy issued by copy_tile: wait for those with all D
// weight k-tiles (2 loads each) requested after them still in flight, then
// for the other waves' copies.
template <int D>
__device__ __forceinline__ void copy_wait() {
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(2 * D));
    __syncthreads();
}

// Only the weights go through the D-deep register pipeline; the activation
// of k-tile c comes from the LDS copy (lc, ls: the lane's row and position
// in the chunk-major layout), read one k-tile ahead. As in stream_unit, the
// steady-state loop has no branches, so the compiler's waits count the
// pipeline exactly.
__device__ __forceinline__ void lds_act(uint2& a, uint32_t& s, const uint8_t* lc, const uint8_t* ls, int c) {
    a = *reinterpret_cast<const uint2*>(lc + c * 512);   // code chunk 2c + q/2 of the lane's row
    s = ls[(c >> 2) * 256 + (c & 3) * 4];                  // byte 4c + q: scale chunk c/4
}

template <int D>
__device__ __forceinline__ void preload_w(Stage (&st)[D], const Streams& p) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_w(st[d], p, d);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The k-tiles of a unit whose first D weight k-tiles are in flight in st and
// whose tile is in LDS.
template <int D>
__device__ __forceinline__ void stream_lds_run(Stage (&st)[D], const Streams& p, const uint8_t* lc,
                                               const uint8_t* ls, int KT, floatx4& acc0, floatx4& acc1) {
    uint2 na;
    uint32_t ns;
    lds_act(na, ns, lc, ls, 0);
    int c0 = 0;
    for (; c0 + D < KT; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            st[d].a = na;
            st[d].asf = ns;
            lds_act(na, ns, lc, ls, c0 + d + 1);
            use_stage(st[d], acc0, acc1);
            load_w(st[d], p, c0 + D + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        st[d].a = na;
        st[d].asf = ns;
        if (d + 1 < D) lds_act(na, ns, lc, ls, c0 + d + 1);
        use_stage(st[d], acc0, acc1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
__device__ __forceinline__ void stream_lds(const Streams& p, const uint8_t* lc, const uint8_t* ls, int KT,
                                           floatx4& acc0, floatx4& acc1) {
    Stage st[D];
    preload_w<D>(st, p);
    copy_wait<D>();
    stream_lds_run<D>(st, p, lc, ls, KT, acc0, acc1);
}

// GEMM1 units 4b .. 4b + 3: intermediate pairs of one tile (I/16 % 4 == 0).
// The 16 activation rows are gathered by token; a padding row reads token 0's
// row, which only feeds an output row that is never written.
template <int D>
__global__ void __launch_bounds__(kThreads) gemm1_wg_kernel(ExpArgs a) {
    extern __shared__ __align__(16) uint8_t tile_lds[];
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n1 = a.I >> 4;
    const uint32_t unit = blockIdx.x * kWavesPerBlock + wave;
    const int sub = (int)(unit / n1), j = (int)(unit - sub * n1);
    const RowTile rt = row_tile(a, sub, n);   // one tile for the whole workgroup
    if (rt.e < 0) return;
    const int e = rt.e;
    const uint32_t tok = rt.tok >= 0 ? (uint32_t)rt.tok : 0u;
    copy_tile(tile_lds, a.H, wave, lane, buffer_desc(a.a_codes), tok * (uint32_t)(a.H >> 1), buffer_desc(a.a_sf),
              tok * (uint32_t)(a.H >> 4));
    Streams p;
    p.wc = a.w.w13 + e * a.w.w13_expert_stride_bytes + j * a.w.w13_pair_stride_bytes + lane * 16;
    p.ws = a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + j * a.w.w13_sf_pair_stride_bytes + lane * 2;
    const uint8_t* lc = tile_lds + ((q >> 1) * 16 + n) * 16 + (q & 1) * 8;
    const uint8_t* ls = tile_lds + (a.H >> 1) * 16 + n * 16 + q;
    floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
    stream_lds<D>(p, lc, ls, a.H >> 6, acc_g, acc_u);
    gemm1_epilogue(a, rt, e, j, n, q, acc_g, acc_u);
}

// GEMM2 units 4b .. 4b + 3: output pairs of one tile (H/32 % 4 == 0); the
// tile's 16 intermediate rows are consecutive.
template <int D>
__global__ void __launch_bounds__(kThreads) gemm2_wg_kernel(ExpArgs a) {
    extern __shared__ __align__(16) uint8_t tile_lds[];
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n2 = a.H >> 5;
    const uint32_t unit = blockIdx.x * kWavesPerBlock + wave;
    const int sub = (int)(unit / n2), c = (int)(unit - sub * n2);
    const RowTile rt = row_tile(a, sub, n);   // one tile for the whole workgroup
    if (rt.e < 0) return;
    const int e = rt.e;
    const uint32_t row = (uint32_t)(rt.row0 + n);
    copy_tile(tile_lds, a.I, wave, lane, buffer_desc(a.inter_codes), row * (uint32_t)(a.I >> 1),
              buffer_desc(a.inter_sf), row * (uint32_t)(a.I >> 4));
    Streams p;
    p.wc = a.w.w2 + e * a.w.w2_expert_stride_bytes + c * a.w.w2_pair_stride_bytes + lane * 16;
    p.ws = a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + c * a.w.w2_sf_pair_stride_bytes + lane * 2;
    const uint8_t* lc = tile_lds + ((q >> 1) * 16 + n) * 16 + (q & 1) * 8;
    const uint8_t* ls = tile_lds + (a.I >> 1) * 16 + n * 16 + q;
    floatx4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    stream_lds<D>(p, lc, ls, a.I >> 6, acc0, acc1);
    gemm2_epilogue(a, rt, e, c, n, q, acc0, acc1);
}

// ---------------------------------------------------------------- both GEMMs in one launch
// Workgroups [0, g1_blocks) are GEMM1's, as in gemm1_wg_kernel; the rest are
// GEMM2's, as in gemm2_wg_kernel, except that a GEMM2 workgroup issues the
// loads of its first D2 weight k-tiles at once and only then waits for its
// 16-row tile's intermediate. The weights of both GEMMs thus stream from HBM
// together, and what is left after GEMM1's stream ends is the hand-over of the
// small intermediate and GEMM2's MFMAs on weights already in registers.
//
// Hand-over between XCDs, each with its own L2: a GEMM1 workgroup writes its
// part of the intermediate with agent-coherent stores, waits until they have
// completed, and adds 1 to the tile's ready counter. A GEMM2 workgroup polls
// that counter until all I/64 GEMM1 workgroups of the tile have added theirs,
// then copies the tile with agent-coherent loads. Nothing handed over passes
// through plain stores, so no L2 write-back or invalidation is needed.
//
// Forward progress: workgroups are dispatched in index order, so every GEMM1
// workgroup has been dispatched before a GEMM2 workgroup can wait, and GEMM1
// workgroups wait for nothing. The wait is bounded all the same: after
// kSpinMax polls it gives up and sets the status word to 1.
//
// Reset: after its copy each GEMM2 workgroup counts itself on the tile's done
// counter; the last of the tile's H/128 returns both counters to 0, so the next
// call on the same metadata starts from 0.

// A GEMM2 unit whose D = KT weight k-tiles are all held in st (I = 256: two
// output pairs a wave, run one after the other, share the wave's metadata
// loads, wait and copy).
template <int D>
__device__ __forceinline__ void run_held(const Stage (&st)[D], const uint8_t* lc, const uint8_t* ls, floatx4& acc0,
                                         floatx4& acc1) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        Stage x = st[d];
        lds_act(x.a, x.asf, lc, ls, d);
        use_stage(x, acc0, acc1);
    }
}

// ---------------------------------------------------------------- the finalize in the launch
// moe_experts_finalize's one-launch form (K <= 8). GEMM2 workgroups write their
// rows with agent-coherent stores, wait until they have completed, and count
// themselves on the arrival counter (word 0) of each token in their 16 rows.
// The grid ends with F = fin_threads(H, T, n_partials) / 256 finalizer workgroups per token:
// finalizer f plays moe_finalize's threads [256 f, 256 f + 256) (finalize.hpp),
// so the arithmetic and its order are moe_finalize's. It waits until every
// GEMM2 workgroup of every tile holding one of the token's served routes has
// arrived (served routes x the H >> (6 + P2) workgroups of a tile), reads its
// columns of the routes' rows (agent-coherent loads) once and keeps them in
// registers, and forms its waves' sums of squares. With F > 1 the token's
// finalizers exchange those through meta's fin_part (agent-coherent stores,
// then word 1 of the token's counters counts them), each runs the same
// 16-lane tree on all of them, and the last to pass (word 2) returns the
// token's counters to 0. A token with no served route gets zero rows at once.
// Finalizers are dispatched after every GEMM workgroup, so what they wait for
// is already running; their waits are bounded as GEMM2's are (sync_status 1
// if one gives up).
struct FinFuse {
    FinArgs f;             // rows: partial 0 (this launch writes partial n_partials - 1)
    int32_t* tok_sync;     // meta's tok_sync
    int32_t* fin_part;     // meta's fin_part
    uint32_t fin_block0;   // the first finalizer workgroup
    int F;                 // finalizer workgroups per token
};

// LDS of a finalizer workgroup
struct FinLds {
    float s_part[kFinBatch][kFinMaxWaves];
    float s_inv[MOE_MAX_TOPK];
};

// A GEMM2 workgroup's rows are complete: count it on each of its tokens.
__device__ __forceinline__ void arrive(const FinFuse& fin, const RowTile& rt, int wave, int lane) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's rows have completed
    __syncthreads();
    if (wave == 0 && lane < 16 && ((rt.vmask >> lane) & 1u))
        __hip_atomic_fetch_add(fin.tok_sync + (int64_t)rt.tok * kTokSyncStride, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

template <int W, int P2>
__device__ void finalizer(const ExpArgs& a, const FinFuse& fin, uint8_t* lds) {
    FinLds& l = *reinterpret_cast<FinLds*>(lds);
    const FinArgs& f = fin.f;
    const uint32_t x = blockIdx.x - fin.fin_block0;
    const int t = (int)(x / (uint32_t)fin.F), part = (int)(x - (uint32_t)t * fin.F);
    const int tid = threadIdx.x, lane = tid & 63;
    const int nthreads_v = fin_threads(f.H, f.T, f.n_partials), nwaves_v = nthreads_v >> 6, ngroups = f.H / W;
    const int vt = part * kThreads + tid;              // moe_finalize's thread this one plays
    const bool wave_on = (vt & ~63) < nthreads_v;      // uniform over the wave
    int32_t* cnt = fin.tok_sync + (int64_t)t * kTokSyncStride;
    // what does not depend on the GEMM2 rows is read before the wait
    int perm[kFinBatch];
    float wk[kFinBatch];
    int served = 0;
#pragma unroll
    for (int kk = 0; kk < kFinBatch; ++kk) {
        perm[kk] = kk < f.K ? f.exp2perm[(int64_t)t * f.K + kk] : -1;
        wk[kk] = kk < f.K ? f.weights[(int64_t)t * f.K + kk] : 0.0f;
        served += perm[kk] >= 0;
    }
    float g[W];
    if (vt < ngroups) gamma_cols<W>(f, vt, g);
    if (served == 0) {                                 // no served route: zero columns
        if (vt < ngroups) {
            Cols<W> z;
#pragma unroll
            for (int i = 0; i < W / 2; ++i) z.w[i] = 0u;
            store_cols<W>(f.out + (int64_t)t * f.H + W * vt, z);
        }
        return;
    }
    if (tid == 0) {
        wait_ready(cnt, served * (a.H >> (6 + P2)), a.status);
        if (fin.F == 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    Cols<W> raw[kFinBatch];
#pragma unroll
    for (int kk = 0; kk < kFinBatch; ++kk) {
#pragma unroll
        for (int i = 0; i < W / 2; ++i) raw[kk].w[i] = 0u;
        if (perm[kk] >= 0 && vt < ngroups) raw[kk] = load_row_coherent<W>(f, perm[kk], vt);
    }
    // sums of squares: the thread's W columns, then its wave
    float ss[kFinBatch];
#pragma unroll
    for (int kk = 0; kk < kFinBatch; ++kk) {
        ss[kk] = 0.0f;
        if (vt < ngroups) {
            float v[W];
            unpack<W>(raw[kk], v);
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const float z = f.weight_before_norm ? __fmul_rn(g[i], v[i]) : v[i];
                ss[kk] = __fadd_rn(ss[kk], __fmul_rn(z, z));
            }
        }
        if (wave_on) ss[kk] = wave_sum(ss[kk]);
    }
    if (fin.F == 1) {
        if (wave_on && lane == 0)
#pragma unroll
            for (int kk = 0; kk < kFinBatch; ++kk) l.s_part[kk][vt >> 6] = ss[kk];
        __syncthreads();
    } else {
        int32_t* pp = fin.fin_part + (int64_t)t * kFinPartWords;
        if (wave_on && lane == 0)
#pragma unroll
            for (int kk = 0; kk < kFinBatch; ++kk)
                __hip_atomic_store(pp + (vt >> 6) * kFinBatch + kk, __float_as_int(ss[kk]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_fetch_add(cnt + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_ready(cnt + 1, fin.F, a.status);
        }
        __syncthreads();
        if (tid < kFinBatch * kFinMaxWaves) {
            const int k = tid >> 4, w = tid & 15;
            l.s_part[k][w] = w < nwaves_v ? __int_as_float(__hip_atomic_load(pp + w * kFinBatch + k, __ATOMIC_RELAXED,
                                                                              __HIP_MEMORY_SCOPE_AGENT))
                                          : 0.0f;
        }
        __syncthreads();
        if (tid == 0 &&
            __hip_atomic_fetch_add(cnt + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == fin.F - 1) {
            __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(cnt + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(cnt + 2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    fin_inv_tree(f, 0, tid, kThreads, nwaves_v, l.s_part, l.s_inv);
    __syncthreads();
    // weighted sum over the routes, k ascending, from the held rows
    if (vt < ngroups) {
        float acc[W];
#pragma unroll
        for (int i = 0; i < W; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < kFinBatch; ++kk) {
            if (kk >= f.K || perm[kk] < 0) continue;   // a missing row normalizes to zero
            const float inv = l.s_inv[kk];
            float v[W];
            unpack<W>(raw[kk], v);
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const float y = f.weight_before_norm ? __fmul_rn(__fmul_rn(g[i], v[i]), inv)
                                                     : __fmul_rn(g[i], __fmul_rn(v[i], inv));
                acc[i] = __fadd_rn(acc[i], __fmul_rn(y, wk[kk]));
            }
        }
        store_cols<W>(f.out + (int64_t)t * f.H + W * vt, pack<W>(acc));
    }
}

template <int D1, int D2, int P2, bool kFin>
__global__ void __launch_bounds__(kThreads) experts_fused_kernel(ExpArgs a, uint32_t g1_blocks, FinFuse fin) {
    extern __shared__ __align__(16) uint8_t tile_lds[];
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* lc = tile_lds + ((q >> 1) * 16 + n) * 16 + (q & 1) * 8;
    if (kFin && blockIdx.x >= fin.fin_block0) {
        if (fin_w(fin.f.H, fin.f.T, fin.f.n_partials) == 2) finalizer<2, P2>(a, fin, tile_lds);
        else finalizer<4, P2>(a, fin, tile_lds);        // W = 8 launches no finalizer workgroups
        return;
    }
    if (blockIdx.x < g1_blocks) {
        const uint32_t n1 = a.I >> 4;
        const uint32_t unit = blockIdx.x * kWavesPerBlock + wave;
        const int sub = (int)(unit / n1), j = (int)(unit - sub * n1);
        const RowTile rt = row_tile(a, sub, n);
        if (rt.e < 0) return;
        const int e = rt.e;
        const uint32_t tok = rt.tok >= 0 ? (uint32_t)rt.tok : 0u;
        copy_tile(tile_lds, a.H, wave, lane, buffer_desc(a.a_codes), tok * (uint32_t)(a.H >> 1),
                  buffer_desc(a.a_sf), tok * (uint32_t)(a.H >> 4));
        Streams p;
        p.wc = a.w.w13 + e * a.w.w13_expert_stride_bytes + j * a.w.w13_pair_stride_bytes + lane * 16;
        p.ws = a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + j * a.w.w13_sf_pair_stride_bytes + lane * 2;
        const uint8_t* ls = tile_lds + (a.H >> 1) * 16 + n * 16 + q;
        floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
        stream_lds<D1>(p, lc, ls, a.H >> 6, acc_g, acc_u);
        gemm1_epilogue<true>(a, rt, e, j, n, q, acc_g, acc_u);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores have completed
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(a.sync + kSubSyncStride * sub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const uint32_t n2 = (a.H >> 5) / P2;        // GEMM2 units a tile
    const uint32_t unit = (blockIdx.x - g1_blocks) * kWavesPerBlock + wave;
    const int sub = (int)(unit / n2), c = (int)(unit - sub * n2) * P2;   // first output pair
    const RowTile rt = row_tile(a, sub, n);
    if (rt.e < 0) return;
    const int e = rt.e;
    Streams p, p1;
    p.wc = a.w.w2 + e * a.w.w2_expert_stride_bytes + c * a.w.w2_pair_stride_bytes + lane * 16;
    p.ws = a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + c * a.w.w2_sf_pair_stride_bytes + lane * 2;
    p1.wc = p.wc + a.w.w2_pair_stride_bytes;
    p1.ws = p.ws + a.w.w2_sf_pair_stride_bytes;
    Stage st[D2], st1[P2 == 2 ? D2 : 1];
    preload_w<D2>(st, p);
    if constexpr (P2 == 2) preload_w<D2>(st1, p1);
    int32_t* ready = a.sync + kSubSyncStride * sub;
    if (wave == 0) wait_ready(ready, a.I >> 6, a.status);
    __syncthreads();
    const uint32_t row = (uint32_t)(rt.row0 + n);
    copy_tile<true>(tile_lds, a.I, wave, lane, buffer_desc(a.inter_codes), row * (uint32_t)(a.I >> 1),
                    buffer_desc(a.inter_sf), row * (uint32_t)(a.I >> 4));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // this wave's part of the copy has landed
    __syncthreads();
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(ready + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (a.H >> (6 + P2)) - 1) {
        __hip_atomic_store(ready, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ready + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint8_t* ls = tile_lds + (a.I >> 1) * 16 + n * 16 + q;
    floatx4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    if constexpr (P2 == 2) {
        run_held<D2>(st, lc, ls, acc0, acc1);
        gemm2_epilogue<kFin>(a, rt, e, c, n, q, acc0, acc1);
        acc0 = floatx4{0, 0, 0, 0};
        acc1 = floatx4{0, 0, 0, 0};
        run_held<D2>(st1, lc, ls, acc0, acc1);
        gemm2_epilogue<kFin>(a, rt, e, c + 1, n, q, acc0, acc1);
    } else {
        stream_lds_run<D2>(st, p, lc, ls, a.I >> 6, acc0, acc1);
        gemm2_epilogue<kFin>(a, rt, e, c, n, q, acc0, acc1);
    }
    if constexpr (kFin) arrive(fin, rt, wave, lane);
}

// ---------------------------------------------------------------- launch
static int pipeline_depth(int kt) {
    const int depths[] = {8, 6, 4, 3, 2, 1};
    for (int d : depths)
        if (kt % d == 0) return d;
    return 1;
}

// Deepest pipelines of the workgroup kernels, as measured on the decode
// shapes: GEMM1 gains nothing past 8 k-tiles (16 was slower), GEMM2 (12 k-tiles
// at I = 768) a little from holding all of them.
constexpr int kWgDepth1 = 8, kWgDepth2 = 16;

// The workgroup kernels' LDS: at most 40 KB keeps 4 workgroups on a CU.
constexpr int kMaxTileLds = 40 * 1024;

#define MOE_LAUNCH_DEPTHS(kernel)                                                                  \
    static void launch_##kernel(int d, dim3 grid, unsigned lds, hipStream_t s, const ExpArgs& a) { \
        switch (d) {                                                                               \
            case 8: hipLaunchKernelGGL(kernel<8>, grid, dim3(kThreads), lds, s, a); break;        \
            case 6: hipLaunchKernelGGL(kernel<6>, grid, dim3(kThreads), lds, s, a); break;        \
            case 4: hipLaunchKernelGGL(kernel<4>, grid, dim3(kThreads), lds, s, a); break;        \
            case 3: hipLaunchKernelGGL(kernel<3>, grid, dim3(kThreads), lds, s, a); break;        \
            case 2: hipLaunchKernelGGL(kernel<2>, grid, dim3(kThreads), lds, s, a); break;        \
            default: hipLaunchKernelGGL(kernel<1>, grid, dim3(kThreads), lds, s, a); break;       \
        }                                                                                          \
    }
MOE_LAUNCH_DEPTHS(gemm1_kernel)
MOE_LAUNCH_DEPTHS(gemm2_kernel)
#undef MOE_LAUNCH_DEPTHS

// The workgroup kernels hold only weights in their pipeline (5 registers a
// k-tile), so they go deeper.
static int wg_depth(int kt, int cap) {
    const int depths[] = {16, 12, 8, 6, 4, 3, 2, 1};
    for (int d : depths)
        if (d <= cap && kt % d == 0) return d;
    return 1;
}

#define MOE_LAUNCH_WG(kernel)                                                                      \
    static void launch_##kernel(int d, dim3 grid, unsigned lds, hipStream_t s, const ExpArgs& a) { \
        switch (d) {                                                                               \
            case 16: hipLaunchKernelGGL(kernel<16>, grid, dim3(kThreads), lds, s, a); break;      \
            case 12: hipLaunchKernelGGL(kernel<12>, grid, dim3(kThreads), lds, s, a); break;      \
            case 8: hipLaunchKernelGGL(kernel<8>, grid, dim3(kThreads), lds, s, a); break;        \
            case 6: hipLaunchKernelGGL(kernel<6>, grid, dim3(kThreads), lds, s, a); break;        \
            case 4: hipLaunchKernelGGL(kernel<4>, grid, dim3(kThreads), lds, s, a); break;        \
            case 3: hipLaunchKernelGGL(kernel<3>, grid, dim3(kThreads), lds, s, a); break;        \
            case 2: hipLaunchKernelGGL(kernel<2>, grid, dim3(kThreads), lds, s, a); break;        \
            default: hipLaunchKernelGGL(kernel<1>, grid, dim3(kThreads), lds, s, a); break;       \
        }                                                                                          \
    }
MOE_LAUNCH_WG(gemm1_wg_kernel)
MOE_LAUNCH_WG(gemm2_wg_kernel)
#undef MOE_LAUNCH_WG

// The one-launch form holds GEMM2's first D2 weight k-tiles in registers
// while it waits: 8 where that divides I/64, else 4. Up to 8 k-tiles (40
// registers) the kernel stays within five waves per SIMD, so that on decode
// shapes every workgroup is resident from the start; 12 (all of I = 768) cost
// a wave per SIMD and were slower, and 6 measured no better than 4.
static int fused_depth2(int kt2) { return kt2 % 8 == 0 ? 8 : 4; }

template <bool kFin>
static void launch_fused(int d1, int d2, bool two_pairs, dim3 grid, unsigned lds, hipStream_t s,
                         const ExpArgs& a, uint32_t g1_blocks, const FinFuse& fin) {
#define MOE_FUSED(D1, D2, P2) \
    hipLaunchKernelGGL((experts_fused_kernel<D1, D2, P2, kFin>), grid, dim3(kThreads), lds, s, a, g1_blocks, fin)
    if (two_pairs) {
        if (d1 == 8) MOE_FUSED(8, 4, 2);
        else MOE_FUSED(4, 4, 2);
    } else if (d1 == 8) {
        if (d2 == 8) MOE_FUSED(8, 8, 1);
        else MOE_FUSED(8, 4, 1);
    } else {
        if (d2 == 8) MOE_FUSED(4, 8, 1);
        else MOE_FUSED(4, 4, 1);
    }
#undef MOE_FUSED
}

static int experts_shape_check(const char* name, int T, int K, int E_local, int H, int I, int tile_m) {
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E_local < 1 || E_local > MOE_MAX_EXPERTS)
        return fail(MOE_EINVAL, "%s: T=%d K=%d E_local=%d out of range", name, T, K, E_local);
    if (H < 64 || H % 64 || I < 64 || I % 64)
        return fail(MOE_EUNSUPPORTED, "%s: H=%d and I=%d must be multiples of 64", name, H, I);
    if (H > MOE_MAX_HIDDEN || I > MOE_MAX_HIDDEN)
        return fail(MOE_EUNSUPPORTED, "%s: H=%d or I=%d above %d", name, H, I, MOE_MAX_HIDDEN);
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return fail(MOE_EUNSUPPORTED, "%s: tile_m=%d must be a multiple of 16 in [16, 256]", name, tile_m);
    return MOE_OK;
}

// moe_experts_fwd with its checks; the intermediate at inter_codes / inter_sf.
// fin (moe_experts_finalize): the finalize of the rows too -- in the same launch
// where the one-launch form applies, else by moe_finalize after the GEMMs.
static int experts_fwd(const char* name, const uint8_t* a_codes, const uint8_t* a_sf, int32_t* meta,
                       const moe_nvfp4_weights* w, int T, int K, int E_local, int H, int I, int tile_m,
                       uint8_t* inter_codes, uint8_t* inter_sf, uint16_t* rows, int64_t rows_stride,
                       void* stream, const FinArgs* fin = nullptr) {
    if (int rc = experts_shape_check(name, T, K, E_local, H, I, tile_m)) return rc;
    if (!w || !meta) return fail(MOE_EINVAL, "%s: NULL weights or meta", name);
    if (T == 0) return MOE_OK;
    if (!a_codes || !a_sf || !inter_codes || !inter_sf || !rows) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    const void* ptrs[] = {a_codes, a_sf, meta, inter_codes, inter_sf, rows};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    if (int rc = check_weights(w, H, I, true, name)) return rc;
    const int64_t kt1 = H / 64, kt2 = I / 64;
    if (rows_stride < H || rows_stride % 8)
        return fail(MOE_EINVAL, "%s: rows_stride must be >= H and a multiple of 8", name);
    ExpArgs args;
    args.a_codes = a_codes; args.a_sf = a_sf; args.meta = meta;
    args.L = meta_layout(T, K, E_local, tile_m);
    args.w = *w; args.T = T; args.E_local = E_local; args.H = H; args.I = I; args.tile_m = tile_m;
    args.inter_codes = inter_codes; args.inter_sf = inter_sf; args.rows = rows;
    args.rows_stride = rows_stride;
    args.sync = meta + args.L.sub_sync;
    args.status = meta + args.L.sync_status;
    args.queue = meta + args.L.queue;
    if (args.L.rows_max == 0) return MOE_OK;
    const int64_t subs = args.L.rows_max / 16;             // 16-row tiles, routed or not
    const int64_t units1 = subs * (I / 16), units2 = subs * (H / 32);
    const int64_t grid1 = (units1 + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid2 = (units2 + kWavesPerBlock - 1) / kWavesPerBlock;
    if (units1 > 0x7FFFFFFF || units2 > 0x7FFFFFFF)   // unit indices are 32-bit in the kernels
        return fail(MOE_EUNSUPPORTED, "%s: too many work units", name);
    hipStream_t s = (hipStream_t)stream;
    // Many routes per expert (on average a quarter of a 128-row block or more):
    // the GEMMs are MFMA-bound and take the register-tiled kernels.
    auto finalize_after = [&](int rc) {
        if (rc || !fin) return rc;
        return moe_finalize(fin->rows, fin->rows_stride, fin->n_partials, fin->partial_stride, fin->exp2perm,
                            fin->weights, fin->norm_weight, fin->gain_center, fin->eps, fin->weight_before_norm,
                            fin->T, fin->K, fin->H, fin->out, stream);
    };
    if (tiled_shape_ok(T, H, I, tile_m) && (int64_t)T * K >= (int64_t)32 * E_local) {
        if (int rc = launch_tiled(args, s)) return rc;
        return finalize_after(check_launch("moe_experts_fwd (tiled)"));
    }
    // Workgroups of four units sharing one LDS copy of their tile's activation
    // where the shape allows: whole 16-byte scale chunks (K % 256 == 0), at
    // most 40 KB of LDS, GEMM2's four output pairs in one tile (H % 128 == 0),
    // 32-bit row offsets into the activation.
    const int d1 = pipeline_depth((int)kt1), d2 = pipeline_depth((int)kt2);
    const bool wg1 = H % 256 == 0 && tile_lds_bytes(H) <= kMaxTileLds && (int64_t)T * (H / 2) < (1ll << 31);
    const bool wg2 = I % 256 == 0 && H % 128 == 0 && tile_lds_bytes(I) <= kMaxTileLds &&
                     args.L.rows_max * (I / 2) < (1ll << 31);
    // Both workgroup forms: one launch, GEMM2's weights streamed beside GEMM1's
    // (pipeline depths dividing H/64 and I/64, both multiples of 4).
    if (wg1 && wg2 && grid1 + grid2 <= 0x7FFFFFFF) {
        const unsigned lds = (unsigned)(tile_lds_bytes(H) > tile_lds_bytes(I) ? tile_lds_bytes(H) : tile_lds_bytes(I));
        const int f1 = kt1 % 8 == 0 ? 8 : 4;
        const int f2 = fused_depth2((int)kt2);
        // I = 256: a GEMM2 wave holds all 4 k-tiles of two output pairs (H % 256 == 0)
        const bool two_pairs = kt2 == 4 && H % 256 == 0;
        const int64_t g2 = two_pairs ? grid2 / 2 : grid2;
        FinFuse ff{};
        if (fin && K <= kFinBatch && fin_w(H, T, fin->n_partials) <= 4) {
            ff.f = *fin;
            ff.tok_sync = meta + args.L.tok_sync;
            ff.fin_part = meta + args.L.fin_part;
            ff.fin_block0 = (uint32_t)(grid1 + g2);
            ff.F = (fin_threads(H, T, fin->n_partials) + kThreads - 1) / kThreads;
            const unsigned lds_f = (unsigned)sizeof(FinLds) > lds ? (unsigned)sizeof(FinLds) : lds;
            launch_fused<true>(f1, f2, two_pairs, dim3((unsigned)(grid1 + g2 + (int64_t)T * ff.F)), lds_f, s, args,
                               (uint32_t)grid1, ff);
            return check_launch("moe_experts_finalize (GEMM1 + GEMM2 + finalize)");
        }
        launch_fused<false>(f1, f2, two_pairs, dim3((unsigned)(grid1 + g2)), lds, s, args, (uint32_t)grid1, ff);
        return finalize_after(check_launch("moe_experts_fwd (GEMM1 + GEMM2)"));
    }
    if (wg1) launch_gemm1_wg_kernel(wg_depth((int)kt1, kWgDepth1), dim3((unsigned)grid1), (unsigned)tile_lds_bytes(H), s, args);
    else launch_gemm1_kernel(d1, dim3((unsigned)grid1), 0, s, args);
    int rc = check_launch("moe_experts_fwd (GEMM1)");
    if (rc) return rc;
    if (wg2) launch_gemm2_wg_kernel(wg_depth((int)kt2, kWgDepth2), dim3((unsigned)grid2), (unsigned)tile_lds_bytes(I), s, args);
    else launch_gemm2_kernel(d2, dim3((unsigned)grid2), 0, s, args);
    return finalize_after(check_launch("moe_experts_fwd (GEMM2)"));
}

// ---------------------------------------------------------------- the intermediate in static memory
// moe_experts_fwd_noalloc keeps the requantized intermediate (GEMM1's output,
// GEMM2's input: nothing outside the call reads it) in this array instead of
// caller memory, so that a caller that cannot allocate device memory needs
// none beyond its inputs and outputs. Every GPU the library runs on holds its
// own copy for the life of the process; calls on one GPU share it.
constexpr int64_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t* g_scratch_ptr[kMaxScratchDevices];   // device address of `scratch` on each GPU

// The device address of the current GPU's scratch, looked up once per GPU
// (with that GPU current) on its first call. The array's name is only a host
// stand-in: kernels and copies take this address.
static int scratch_base(const char* name, uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_ELAUNCH, "%s: hipGetDevice failed: %s", name, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(MOE_EUNSUPPORTED, "%s: device %d beyond the %d this build tracks", name, dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ELAUNCH, "%s: hipGetSymbolAddress(scratch) failed: %s", name, hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace moe

extern "C" int moe_experts_fwd(const uint8_t* a_codes, const uint8_t* a_sf, int32_t* meta,
                               const moe_nvfp4_weights* w, int T, int K, int E_local, int H,
                               int I, int tile_m, uint8_t* inter_codes, uint8_t* inter_sf,
                               uint16_t* rows, int64_t rows_stride, void* stream) {
    return moe::experts_fwd("moe_experts_fwd", a_codes, a_sf, meta, w, T, K, E_local, H, I, tile_m,
                            inter_codes, inter_sf, rows, rows_stride, stream);
}

extern "C" int moe_experts_finalize(const uint8_t* a_codes, const uint8_t* a_sf, int32_t* meta,
                                    const moe_nvfp4_weights* w, int T, int K, int E_local, int H, int I,
                                    int tile_m, uint8_t* inter_codes, uint8_t* inter_sf, uint16_t* rows,
                                    int64_t rows_stride, int n_partials, int64_t partial_stride,
                                    const float* topk_weights, const uint16_t* norm_weight, float gain_center,
                                    float eps, int weight_before_norm, uint16_t* out, void* stream) {
    using namespace moe;
    const char* name = "moe_experts_finalize";
    if (int rc = experts_shape_check(name, T, K, E_local, H, I, tile_m)) return rc;
    if (n_partials < 1 || n_partials > 16)
        return fail(MOE_EUNSUPPORTED, "%s: n_partials=%d outside [1, 16]", name, n_partials);
    if (T == 0) return MOE_OK;
    if (!rows || !topk_weights || !out || !meta) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    if (!aligned16(topk_weights) || !aligned16(out) || (norm_weight && !aligned16(norm_weight)))
        return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    if (n_partials > 1 && (partial_stride % 8 || partial_stride < 0))
        return fail(MOE_EINVAL, "%s: partial_stride must be a non-negative multiple of 8", name);
    const moe_meta_layout L = meta_layout(T, K, E_local, tile_m);
    FinArgs f;
    f.rows = rows; f.rows_stride = rows_stride; f.n_partials = n_partials; f.partial_stride = partial_stride;
    f.exp2perm = meta + L.exp2perm; f.weights = topk_weights; f.norm_weight = norm_weight;
    f.gain_center = gain_center; f.eps = eps; f.weight_before_norm = weight_before_norm ? 1 : 0;
    f.T = T; f.K = K; f.H = H; f.out = out;
    return experts_fwd(name, a_codes, a_sf, meta, w, T, K, E_local, H, I, tile_m, inter_codes, inter_sf,
                       rows + (int64_t)(n_partials - 1) * partial_stride, rows_stride, stream, &f);
}

extern "C" int moe_experts_fwd_noalloc(const uint8_t* a_codes, const uint8_t* a_sf, int32_t* meta,
                                       const moe_nvfp4_weights* w, int T, int K, int E_local, int H,
                                       int I, int tile_m, uint16_t* rows, int64_t rows_stride,
                                       void* stream) {
    using namespace moe;
    const char* name = "moe_experts_fwd_noalloc";
    if (int rc = experts_shape_check(name, T, K, E_local, H, I, tile_m)) return rc;
    const moe_meta_layout L = meta_layout(T, K, E_local, tile_m);
    const int64_t codes_bytes = (L.rows_max * (I / 2) + 255) / 256 * 256;
    const int64_t need = codes_bytes + L.rows_max * (I / 16);
    if (need > kScratchBytes)
        return fail(MOE_EUNSUPPORTED,
                    "%s: the intermediate of %lld rows x %d needs %lld bytes, above the %lld of static scratch",
                    name, (long long)L.rows_max, I, (long long)need, (long long)kScratchBytes);
    if (!w || !meta) return fail(MOE_EINVAL, "%s: NULL weights or meta", name);
    if (T == 0 || L.rows_max == 0) return MOE_OK;
    uint8_t* base = nullptr;
    if (int rc = scratch_base(name, &base)) return rc;
    return experts_fwd(name, a_codes, a_sf, meta, w, T, K, E_local, H, I, tile_m, base, base + codes_bytes, rows,
                       rows_stride, stream);
}
