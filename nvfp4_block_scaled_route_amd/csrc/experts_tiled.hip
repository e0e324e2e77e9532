// The expert GEMMs for many routes per expert (prefill): register-tiled MFMA.
//   the runner page, "MuseSparkTrtLlmNvFp4Experts.apply_routed"; the
//   flashinfer_ops page, "routed_experts_from_metadata" -- same arithmetic as
//   the streaming kernels in experts.hip (GEMM1 + SwiGLU + requant, GEMM2).
//
// With hundreds of routes per expert the GEMMs are bound by the matrix cores,
// not by the weight stream. gfx950 has no MFMA for 16-element blocks under e4m3
// scales, so both operands are decoded to exact f16 (one VALU instruction per
// element) and multiplied with v_mfma_f32_32x32x16_f16. The decode is the cost
// to amortize: every decoded element must feed as many MFMAs as possible.
//
// A workgroup takes one 128-row block of one expert and 4 column blocks of 128;
// each of its 4 waves computes one 128 x 128 output block over K in 64-wide
// k-tiles with 4 x 4 accumulators (the 256 accumulators fill the AGPR file: one
// wave per SIMD):
//   * the MFMA K index is permuted on both operands so that over the 4 K-steps
//     of a k-tile a lane (r, h) of a 32 x 32 x 16 MFMA holds two whole NVFP4
//     blocks of its row (column), blocks 2h and 2h + 1, each under one scale;
//     a decoded A fragment then feeds 4 MFMAs and a decoded B fragment 4:
//     4 VALU instructions per 32-cycle MFMA, which run beside the matrix pipe;
//   * the weights (B) go straight from global memory to registers in MFMA lane
//     order (whole pair tiles of the converted layout: full cache lines), two
//     k-tiles ahead;
//   * the activation rows (A) are shared by the 4 waves: the workgroup copies 4
//     k-tiles of its 128 rows at a time (128 bytes of codes per row: whole cache
//     lines) with direct global-to-LDS loads into a double-buffered LDS stage,
//     one barrier per stage, and each wave reads its fragments from there. A
//     row's 16-byte chunks are stored XOR-swizzled by the row's low 3 bits, so
//     the fragment reads of 8 consecutive rows hit 8 different bank groups.
//     (Gathered straight into registers, every A load touched 32 cache lines
//     for 32 bytes each, and the weight stream evicted them before the next
//     k-tile could use the rest.)
//   * row tiles with no route are skipped (an expert's rows are padded to the
//     block size): a block runs with 1 to 4 row tiles.
// Workgroups are mapped to the routed row blocks only (their count is read from
// the routing metadata), split into 8 equal contiguous chunks, one per XCD
// (workgroups are dealt to the 8 XCDs round robin), row block major: the
// column groups of a row block, and the row blocks of one expert, run on the
// same XCD at about the same time and share the A rows and the weights in its L2.
//
// GEMM1's columns are arranged so that a lane holds the gate and the up value of
// the same intermediate in two accumulators (column tiles 2t and 2t + 1 take the
// gate and the up halves of the same two pairs), so SwiGLU is lane-local; the
// 16-wide amax and the packing of the codes use DPP moves within 16-lane rows.
// GEMM2 writes bf16 rows. Rows without a route are not written.
#include "experts.hpp"

namespace moe {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kCT = 4;                      // 32-column MFMA tiles per wave
constexpr int kBlockRows = 128;             // rows per block (4 row tiles of 32)
constexpr int kWaves = 4;                   // waves (column blocks) per workgroup
constexpr int kStage = 4;                   // k-tiles per A stage in LDS
constexpr int kAhead = 2;                   // weight k-tiles loaded ahead in registers
constexpr int kXcds = 8;
constexpr int kARowBytes = 32 * kStage;     // codes of one row in a stage
constexpr int kASfBytes = 4 * kStage;       // block scales of one row in a stage

// LDS: two A stages (codes, swizzled; block scales)
struct ALds {
    uint8_t codes[2][kBlockRows * kARowBytes];
    uint8_t sf[2][kBlockRows * kASfBytes];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
    // raw buffer (stride 0) with no range limit; gfx9 data-format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// One lane's raw weight operands of one k-tile: blocks 2h and 2h + 1 of each
// column tile's column (8 bytes each, 256 bytes apart in the pair tile) and the
// u32 words holding their scales. In GEMM1 column tiles 2t and 2t + 1 are the
// two halves of the same pairs, whose scale bytes share words: kSW word pairs.
template <int MODE>
struct BRaw {
    static constexpr int kSW = MODE == 1 ? kCT / 2 : kCT;
    static constexpr int kLoads = 2 * kCT + 2 * kSW;
    uint2 b[kCT][2];
    uint32_t bsf[kSW][2];
};

// One lane's raw activation operands of one k-tile: the 32 codes (blocks 2h,
// 2h + 1) of each row tile's row and the row's 4 block scales of the k-tile.
template <int RT>
struct ARaw {
    uint4 a[RT];
    uint32_t asf[RT];
};

struct BSrc {
    __amdgpu_buffer_rsrc_t b, bs;   // k-tile c at + 1024 c, + 128 c
    uint32_t b_off, bs_off;         // per lane
    int b_step, bs_step;            // from one pair to the next
};

// The weight loads of a k-tile always issue in this order and by themselves
// (prologue and loop alike), so that every use waits only for the loads issued
// before it: vmcnt drains in issue order.
template <int MODE>
__device__ __forceinline__ void b_load(BRaw<MODE>& r, const BSrc& p, int c) {
#pragma unroll
    for (int j = 0; j < kCT; ++j) {
        // GEMM1: tile j = 2t + g is half g of pairs 2t + lane / 16;
        // GEMM2: tile j is pair j
        const int so = c * kSlotBytes + (MODE == 1 ? (j >> 1) * 2 : j) * p.b_step;
        const int o = (int)p.b_off + (MODE == 1 ? (j & 1) * 8 : 0);
        __builtin_amdgcn_sched_barrier(0);
        const u32x2 v0 = __builtin_amdgcn_raw_buffer_load_b64(p.b, o, so, 0);
        __builtin_amdgcn_sched_barrier(0);
        const u32x2 v1 = __builtin_amdgcn_raw_buffer_load_b64(p.b, o + 256, so, 0);
        r.b[j][0] = make_uint2(v0[0], v0[1]);
        r.b[j][1] = make_uint2(v1[0], v1[1]);
    }
#pragma unroll
    for (int t = 0; t < BRaw<MODE>::kSW; ++t) {
        const int so = c * kSlotSfBytes + t * (MODE == 1 ? 2 : 1) * p.bs_step;
        __builtin_amdgcn_sched_barrier(0);
        r.bsf[t][0] = __builtin_amdgcn_raw_buffer_load_b32(p.bs, (int)p.bs_off, so, 0);
        __builtin_amdgcn_sched_barrier(0);
        r.bsf[t][1] = __builtin_amdgcn_raw_buffer_load_b32(p.bs, (int)p.bs_off + 32, so, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// The workgroup's copy of A stage g into LDS buffer g & 1. Codes: wave w's
// load q covers rows 32q + 8w + [0, 8) (1 KB, lane l at byte 16 l): lane l
// fetches chunk (l % 8) ^ (row % 8) of row 32q + 8w + l / 8. Scales: waves 0
// and 1, lane l fetches the 16 scale bytes of row 64w + l.
//
// The copies are written as inline assembly on purpose: the compiler treats
// its own direct-to-LDS loads as LDS writes of unknown extent and waits for
// all of them (vmcnt(0), the weight prefetch included) before every LDS read,
// which would serialize the stage pipeline. Here the stage's own vmcnt wait
// and barrier order the copies against the reads. M0 holds the LDS address.
struct ASrc {
    u32x4 a, as;                    // buffer descriptors
    uint32_t a_off[4];              // per lane and load q: row start + chunk
    uint32_t as_off;                // per lane: row start (waves 0, 1)
};

__device__ __forceinline__ u32x4 buffer_desc(const void* base) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    // raw buffer (stride 0) with no range limit; gfx9 data-format word
    return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xFFFFu, 0x7FFFFFFFu, 0x00020000u};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void lds_copy16(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

__device__ __forceinline__ void a_stage_load(ALds& lds, const ASrc& p, int wave, int g) {
    const int buf = g & 1;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        lds_copy16(p.a, __builtin_amdgcn_readfirstlane(lds_addr(&lds.codes[buf][(32 * q + 8 * wave) * kARowBytes])),
                   p.a_off[q], (uint32_t)(g * kARowBytes));
    if (wave < 2)
        lds_copy16(p.as, __builtin_amdgcn_readfirstlane(lds_addr(&lds.sf[buf][64 * wave * kASfBytes])), p.as_off,
                   (uint32_t)(g * kASfBytes));
}

// A fragments of k-tile c of a stage: lane (nn, h) of row tile i reads the 16
// bytes of chunk 2c + h of row 32 i + nn (swizzled), and its 4 block scales.
template <int RT>
__device__ __forceinline__ void a_read(ARaw<RT>& r, const ALds& lds, int buf, int c, int nn, int h) {
    const int pos = ((2 * c + h) ^ (nn & 7)) * 16;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        r.a[i] = *reinterpret_cast<const uint4*>(&lds.codes[buf][(32 * i + nn) * kARowBytes + pos]);
        r.asf[i] = *reinterpret_cast<const uint32_t*>(&lds.sf[buf][(32 * i + nn) * kASfBytes + 4 * c]);
    }
}

// The MFMAs of one k-tile. K-step s takes, in lane (r, h), the elements
// 32 h + 8 s + [0, 8) of the k-tile: u32 word s of the lane's 16 code bytes,
// under the scale of block 2h + s / 2. The fragments of step s + 1 are decoded
// while the MFMAs of step s run: one MFMA, then 4 or 5 VALU instructions.
template <int RT>
struct Frags {
    half8 a[RT], b[kCT];
};

template <int MODE, int RT>
__device__ __forceinline__ void decode_step(const ARaw<RT>& ar, const BRaw<MODE>& br, const half2v (&sa)[RT],
                                            const half2v (&sb)[kCT], int s, Frags<RT>& f) {
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const uint32_t w = s == 0 ? ar.a[i].x : s == 1 ? ar.a[i].y : s == 2 ? ar.a[i].z : ar.a[i].w;
        f.a[i] = nvfp4x8_to_f16(w, s < 2 ? splat_lo(sa[i]) : splat_hi(sa[i]));
    }
#pragma unroll
    for (int j = 0; j < kCT; ++j) {
        const uint32_t w = s == 0 ? br.b[j][0].x : s == 1 ? br.b[j][0].y : s == 2 ? br.b[j][1].x : br.b[j][1].y;
        f.b[j] = nvfp4x8_to_f16(w, s < 2 ? splat_lo(sb[j]) : splat_hi(sb[j]));
    }
}

template <int MODE, int RT>
__device__ __forceinline__ void tile_mfma(const ARaw<RT>& ar, const BRaw<MODE>& br, int h,
                                          const uint32_t (&sel)[2], floatx16 (&acc)[RT][kCT]) {
    half2v sa[RT], sb[kCT];
#pragma unroll
    for (int i = 0; i < RT; ++i) sa[i] = e4m3x2_to_f16(ar.asf[i] >> (16 * h));
#pragma unroll
    for (int j = 0; j < kCT; ++j) {
        const int t = MODE == 1 ? j >> 1 : j;
        sb[j] = e4m3x2_to_f16(__builtin_amdgcn_perm(br.bsf[t][1], br.bsf[t][0], sel[MODE == 1 ? j & 1 : 0]));
    }
    Frags<RT> f[2];
    decode_step(ar, br, sa, sb, 0, f[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (s < 3) decode_step(ar, br, sa, sb, s + 1, f[(s + 1) & 1]);
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < kCT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f[s & 1].a[i], f[s & 1].b[j], acc[i][j], 0, 0, 0);
        if (s < 3) {
#pragma unroll
            for (int k = 0; k < RT * kCT; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 8 * (RT + kCT) / (RT * kCT) + 1, 0);   // VALU
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// s_waitcnt immediate (gfx9 encoding): at most n vector-memory loads in
// flight, the other counters unconstrained
__host__ __device__ constexpr int vmcnt_at_most(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// max over 16-lane rows by DPP (exact in any order)
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    return v;
}

// lane i of each 16-lane row receives lane i + n (0 past the row's end)
template <int n>
__device__ __forceinline__ uint32_t row_shl(uint32_t v) {
    return (uint32_t)dpp_i<0x100 + n>((int)v);
}

// lane i of each 16-lane row receives lane x of the row
template <int x>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + x, 0xF, 0xF, false));
}

// GEMM1 epilogue of one gate tile and its up tile: rows m0 + [0, 32), lane l
// holds intermediate col0 + l % 32 of rows m0 + 8(x/4) + 4(l/32) + x%4 in
// element x. The 16 intermediates of a block sit in one 16-lane row, so the
// amax is a row max; the block scale of element x is computed by lane x of the
// row (one scale per lane, then broadcast back), and the codes are packed 8 to
// a word by shifting within the row.
__device__ __forceinline__ void swiglu_quant_tile(const floatx16& gacc, const floatx16& uacc, float ga, float uc,
                                                  int lane, uint32_t vrow, const ExpArgs& a, int m0, int col0) {
    const int n = lane & 15, h = lane >> 5;
    const int col = col0 + (lane & 31);
    float hv[16];
    float amax_t = 0.0f;        // lane n: amax of element n's block
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        const float g = gacc[x] * ga;
        const float u = uacc[x] * uc;
        hv[x] = g / (1.0f + expf(-g)) * u;
        const float am = row16_max(__builtin_fabsf(hv[x]));
        amax_t = n == x ? am : amax_t;
    }
    const BlockScale bs = nvfp4_block_scale(amax_t, 1.0f);
    {   // lane n writes the scale byte of element n's row
        const int64_t row = m0 + 8 * (n >> 2) + 4 * h + (n & 3);
        if ((vrow >> n) & 1u) a.inter_sf[row * (a.I >> 4) + (col >> 4)] = (uint8_t)bs.byte;
    }
#define MOE_CODE(x)                                                                        \
    {                                                                                      \
        const float r = row_bcast<x>(bs.r);                                                \
        uint32_t b = r == 0.0f ? 0u : e2m1_encode(__fmul_rn(hv[x], r));                     \
        b |= row_shl<1>(b) << 4;                                                           \
        b |= row_shl<2>(b) << 8;                                                           \
        b |= row_shl<4>(b) << 16;                                                          \
        const int64_t row = m0 + 8 * (x >> 2) + 4 * h + (x & 3);                          \
        if (((vrow >> x) & 1u) && (n & 7) == 0)                                            \
            *reinterpret_cast<uint32_t*>(a.inter_codes + row * (a.I >> 1) + (col >> 1)) = b; \
    }
    MOE_CODE(0) MOE_CODE(1) MOE_CODE(2) MOE_CODE(3) MOE_CODE(4) MOE_CODE(5) MOE_CODE(6) MOE_CODE(7)
    MOE_CODE(8) MOE_CODE(9) MOE_CODE(10) MOE_CODE(11) MOE_CODE(12) MOE_CODE(13) MOE_CODE(14) MOE_CODE(15)
#undef MOE_CODE
}

// GEMM2 epilogue of one tile: bf16 rows m0 + [0, 32), columns col0 + [0, 32).
__device__ __forceinline__ void bf16_tile(const floatx16& acc, float alpha, int lane, uint32_t vrow,
                                          const ExpArgs& a, int m0, int col0) {
    const int h = lane >> 5;
    uint16_t* out = a.rows + (int64_t)m0 * a.rows_stride + col0 + (lane & 31);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        const int m = 8 * (x >> 2) + 4 * h + (x & 3);
        if ((vrow >> x) & 1u) out[(int64_t)m * a.rows_stride] = (uint16_t)f32_to_bf16(acc[x] * alpha);
    }
}

// One wave's block: rows [row0, row0 + 32 RT) of expert e, column block cb
// (computed but not stored when store is false: a column group past the end).
// vrows[i]: bit x is set when the row this lane holds in element x of row tile
// i's accumulators has a route.
template <int MODE, int RT>
__device__ __forceinline__ void run_block(const ExpArgs& a, ALds& lds, const ASrc& ap, int e, int row0, int cb,
                                          bool store, int wave, int lane, const uint32_t (&vrows)[4]) {
    const int h = lane >> 5, nn = lane & 31, n = lane & 15, hh = (lane >> 4) & 1;
    const int K = MODE == 1 ? a.H : a.I;
    const int NS = K / (64 * kStage);

    BSrc p;
    if (MODE == 1) {
        const int pair0 = cb * kCT;                                 // 4 pairs: 64 intermediates
        p.b = buffer_rsrc(a.w.w13 + e * a.w.w13_expert_stride_bytes + pair0 * a.w.w13_pair_stride_bytes);
        p.bs = buffer_rsrc(a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + pair0 * a.w.w13_sf_pair_stride_bytes);
        p.b_step = (int)a.w.w13_pair_stride_bytes;
        p.bs_step = (int)a.w.w13_sf_pair_stride_bytes;
        // column nn of tile 2t + g: pair 2t + nn / 16, half g, row n
        p.b_off = hh * (uint32_t)p.b_step + (uint32_t)(2 * h * 16 + n) * 16;
        p.bs_off = hh * (uint32_t)p.bs_step + 64 * h + 4 * (n >> 1);
    } else {
        const int pair0 = cb * kCT;                                 // 4 pairs: 128 output columns
        p.b = buffer_rsrc(a.w.w2 + e * a.w.w2_expert_stride_bytes + pair0 * a.w.w2_pair_stride_bytes);
        p.bs = buffer_rsrc(a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + pair0 * a.w.w2_sf_pair_stride_bytes);
        p.b_step = (int)a.w.w2_pair_stride_bytes;
        p.bs_step = (int)a.w.w2_sf_pair_stride_bytes;
        // column nn of tile j: pair j, half nn / 16, row n
        p.b_off = (uint32_t)((2 * h * 16 + n) * 2 + hh) * 8;
        p.bs_off = 64 * h + 4 * (n >> 1);
    }
    // byte selectors of the two block scales (block 2h from the first word,
    // 2h + 1 from the second): for half g = 0, 1 (GEMM1), the lane's half (GEMM2)
    uint32_t sel[2];
    {
        const uint32_t b0 = MODE == 1 ? 2 * (n & 1) : 2 * (n & 1) + hh;
        sel[0] = 0x0c0c0000u | ((4 + b0) << 8) | b0;
        sel[1] = sel[0] + 0x0101u;
    }

    floatx16 acc[RT][kCT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < kCT; ++j)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.0f;

    // prologue: A stage 0, weights for k-tiles 0 .. kAhead - 1
    a_stage_load(lds, ap, wave, 0);
    BRaw<MODE> ring[kAhead];
#pragma unroll
    for (int d = 0; d < kAhead; ++d) b_load(ring[d], p, d);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kAhead * BRaw<MODE>::kLoads));
    __syncthreads();

    // stage g (buffer g % 2): A stage g + 1 is copied into the other buffer
    // (read by nobody since the last barrier; in the last stage a harmless copy
    // of the last stage); k-tiles 4g .. 4g + 3 run, the weights of k-tile
    // c + kAhead load into ring slot c % kAhead (past the end: the last k-tile
    // again, unused); then every wave's copies have landed (vmcnt: only the
    // weight loads issued after them may still be in flight) and a barrier
    // publishes them.
    const int KT = NS * kStage;
    for (int g = 0; g < NS; ++g) {
        const int buf = g & 1;
        a_stage_load(lds, ap, wave, min(g + 1, NS - 1));
        ARaw<RT> ar[2];
        a_read(ar[0], lds, buf, 0, nn, h);
#pragma unroll
        for (int c = 0; c < kStage; ++c) {
            if (c + 1 < kStage) a_read(ar[(c + 1) & 1], lds, buf, c + 1, nn, h);
            tile_mfma(ar[c & 1], ring[c % kAhead], h, sel, acc);
            b_load(ring[c % kAhead], p, min(kStage * g + c + kAhead, KT - 1));
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kAhead * BRaw<MODE>::kLoads));
        __syncthreads();
    }

    if (!store) return;
    // epilogue, one 32 x 32 tile (GEMM1: a gate tile and its up tile) at a time
    if (MODE == 1) {
        const float ga = a.w.g1_alphas[e], uc = a.w.g1_scale_c[e];
#define MOE_EPI1(i, t)                                                                          \
    if (RT > i) swiglu_quant_tile(acc[RT > i ? i : 0][2 * t], acc[RT > i ? i : 0][2 * t + 1], ga, uc, lane, \
                                  vrows[i], a, row0 + 32 * i, 64 * cb + 32 * t)
        MOE_EPI1(0, 0); MOE_EPI1(0, 1); MOE_EPI1(1, 0); MOE_EPI1(1, 1);
        MOE_EPI1(2, 0); MOE_EPI1(2, 1); MOE_EPI1(3, 0); MOE_EPI1(3, 1);
#undef MOE_EPI1
    } else {
        const float alpha = a.w.g2_alphas[e];
#define MOE_EPI2(i, j) \
    if (RT > i) bf16_tile(acc[RT > i ? i : 0][j], alpha, lane, vrows[i], a, row0 + 32 * i, 128 * cb + 32 * j)
        MOE_EPI2(0, 0); MOE_EPI2(0, 1); MOE_EPI2(0, 2); MOE_EPI2(0, 3);
        MOE_EPI2(1, 0); MOE_EPI2(1, 1); MOE_EPI2(1, 2); MOE_EPI2(1, 3);
        MOE_EPI2(2, 0); MOE_EPI2(2, 1); MOE_EPI2(2, 2); MOE_EPI2(2, 3);
        MOE_EPI2(3, 0); MOE_EPI2(3, 1); MOE_EPI2(3, 2); MOE_EPI2(3, 3);
#undef MOE_EPI2
    }
}

template <int MODE>   // 1: GEMM1 + SwiGLU + requant, 2: GEMM2
__global__ void __launch_bounds__(64 * kWaves) tiled_kernel(ExpArgs a, int ncg, int ncb) {
    __shared__ ALds lds;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // work items: (routed row block, column group), row block major, in 8
    // equal contiguous chunks, chunk x on XCD x
    const int items = a.meta[a.L.num_tiles] * (a.tile_m / kBlockRows) * ncg;
    const int per_xcd = (items + kXcds - 1) / kXcds;
    const int slot = (int)(blockIdx.x / kXcds);
    if (slot >= per_xcd) return;
    const int item = (int)(blockIdx.x % kXcds) * per_xcd + slot;
    if (item >= items) return;
    const int bx = item / ncg, cg = item % ncg;
    const int row0 = bx * kBlockRows;
    const int e = a.meta[a.L.tile_expert + row0 / a.tile_m];
    if (e < 0 || e >= a.E_local) return;                     // uniform over the workgroup
    int cb = cg * kWaves + wave;
    const bool store = cb < ncb;
    cb = min(cb, ncb - 1);

    const int nn = lane & 31, h = lane >> 5;
    // the rows this lane holds in the accumulators: element x of row tile i is
    // row 32 i + 8(x/4) + 4h + x%4
    uint32_t vrows[4];
    int rt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = a.meta[a.L.perm2tok + row0 + 32 * i + nn];
        const uint32_t m = (uint32_t)__ballot(t >= 0 && t < a.T);   // bit r: row 32 i + r
        if (m != 0u) rt = i + 1;
        uint32_t v = 0;
#pragma unroll
        for (int x = 0; x < 16; ++x) v |= ((m >> (8 * (x >> 2) + 4 * h + (x & 3))) & 1u) << x;
        vrows[i] = v;
    }

    // the A stage copies of this lane (rows without a route copy token row 0)
    ASrc ap;
    {
        const int l8 = lane >> 3, c16 = lane & 7;
        if (MODE == 1) {
            ap.a = buffer_desc(a.a_codes);
            ap.as = buffer_desc(a.a_sf);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 32 * q + 8 * wave + l8;
                int t = a.meta[a.L.perm2tok + row0 + r];
                t = (t >= 0 && t < a.T) ? t : 0;
                ap.a_off[q] = (uint32_t)t * (uint32_t)(a.H >> 1) + ((c16 ^ (r & 7)) * 16);
            }
            int t = a.meta[a.L.perm2tok + row0 + ((64 * wave + lane) & (kBlockRows - 1))];
            t = (t >= 0 && t < a.T) ? t : 0;
            ap.as_off = (uint32_t)t * (uint32_t)(a.H >> 4);
        } else {
            ap.a = buffer_desc(a.inter_codes + (int64_t)row0 * (a.I >> 1));
            ap.as = buffer_desc(a.inter_sf + (int64_t)row0 * (a.I >> 4));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 32 * q + 8 * wave + l8;
                ap.a_off[q] = (uint32_t)r * (uint32_t)(a.I >> 1) + ((c16 ^ (r & 7)) * 16);
            }
            ap.as_off = (uint32_t)((64 * wave + lane) & (kBlockRows - 1)) * (uint32_t)(a.I >> 4);
        }
    }

    switch (rt) {
        case 1: run_block<MODE, 1>(a, lds, ap, e, row0, cb, store, wave, lane, vrows); break;
        case 2: run_block<MODE, 2>(a, lds, ap, e, row0, cb, store, wave, lane, vrows); break;
        case 3: run_block<MODE, 3>(a, lds, ap, e, row0, cb, store, wave, lane, vrows); break;
        case 4: run_block<MODE, 4>(a, lds, ap, e, row0, cb, store, wave, lane, vrows); break;
        default: break;
    }
}

bool tiled_shape_ok(int T, int H, int I, int tile_m) {
    // whole row blocks; K = H and K = I in whole A stages (4 k-tiles); 32-bit
    // per-lane offsets into the activation codes
    return tile_m % kBlockRows == 0 && H % (64 * kStage) == 0 && I % (64 * kStage) == 0 &&
           (int64_t)T * (H / 2) < ((int64_t)1 << 31);
}

void launch_tiled(const ExpArgs& a, hipStream_t s) {
    // grids cover every row block that routing can fill; the kernels take the
    // routed ones from the metadata
    const int nx = (int)(a.L.rows_max / kBlockRows);
    const int ncb1 = a.I / 64, ncb2 = a.H / 128;
    const int ncg1 = (ncb1 + kWaves - 1) / kWaves, ncg2 = (ncb2 + kWaves - 1) / kWaves;
    auto grid = [](int64_t items) { return dim3((unsigned)((items + kXcds - 1) / kXcds * kXcds)); };
    hipLaunchKernelGGL(tiled_kernel<1>, grid((int64_t)nx * ncg1), dim3(64 * kWaves), 0, s, a, ncg1, ncb1);
    hipLaunchKernelGGL(tiled_kernel<2>, grid((int64_t)nx * ncg2), dim3(64 * kWaves), 0, s, a, ncg2, ncb2);
}

}  // namespace moe
