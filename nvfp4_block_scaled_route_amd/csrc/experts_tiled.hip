// The expert GEMMs for many routes per expert (prefill): register-tiled MFMA.
//   the runner page, "MuseSparkTrtLlmNvFp4Experts.apply_routed"; the
//   flashinfer_ops page, "routed_experts_from_metadata" -- same arithmetic as
//   the streaming kernels in experts.hip (GEMM1 + SwiGLU + requant, GEMM2).
//
// With hundreds of routes per expert the GEMMs are bound by the matrix cores,
// not by the weight stream. gfx950 has no MFMA for 16-element blocks under e4m3
// scales, so both operands are decoded to exact f16 (one VALU instruction per
// element) and multiplied with v_mfma_f32_32x32x16_f16. The decode is the cost
// to amortize, and the matrix pipe has to be kept busy while it runs.
//
// Two workgroups share a CU (two waves per SIMD: while one waits at a barrier,
// on memory or in its epilogue, the other issues MFMAs). A workgroup takes one
// 128-row block of one expert and 4 column blocks; each of its 4 waves computes
// one 128 x 64 output block over K in 64-wide k-tiles with 4 x 2 accumulators
// (128 accumulator registers, half of a wave's share at two waves a SIMD):
//   * the MFMA K index is permuted on both operands so that over the 4 K-steps
//     of a k-tile a lane (r, h) of a 32 x 32 x 16 MFMA holds two whole NVFP4
//     blocks of its row (column), blocks 2h and 2h + 1, each under one scale;
//   * the weights (B) go straight from global memory to registers in MFMA lane
//     order (whole pair tiles of the converted layout: full cache lines), two
//     k-tiles ahead; each wave decodes its own columns (2 fragments a K-step,
//     each feeding RT MFMAs);
//   * the activation rows (A): the workgroup copies 4 k-tiles of its routed
//     rows at a time (128 bytes of codes per row: whole cache lines) with
//     direct global-to-LDS loads into a double-buffered raw stage (one row's
//     16-byte chunks XOR-swizzled, chunk_swizzle). In blocks of 3 or 4 routed
//     row tiles A is decoded once per workgroup: during k-tile c every thread
//     decodes its share of k-tile c + 1 into a double-buffered f16 tile in MFMA
//     fragment order, from which each wave reads its A fragments with 16-byte
//     LDS reads (64 lanes, 1 KB contiguous: no bank conflicts); one barrier per
//     k-tile publishes the decoded tile. In blocks of 1 or 2, each wave decodes
//     its own A fragments from the raw stage (one barrier per stage);
//   * row tiles with no route are skipped (an expert's rows are padded to the
//     block size): a block runs with 1 to 4 row tiles and copies and decodes
//     only those.
// One persistent workgroup per half CU takes work items -- (routed row block,
// column group) of GEMM1, then of GEMM2 -- from 8 queues, one per XCD: the
// routed row blocks (their count is read from the routing metadata) are split
// into 8 equal contiguous chunks, and queue x holds chunk x's GEMM1 items, then
// its GEMM2 items, each expert's run of blocks in the chunk column group major:
// the items that read one weight column group (one per block of the expert)
// follow one another, and those that read one block's rows are as many items
// apart as the expert has blocks there (2 to 3 here), so both are read while
// the XCD's L2 still holds them. A workgroup takes from its own XCD's queue
// (workgroups are dealt to the 8 XCDs round robin); when that queue is empty it
// takes from the others, so that no XCD idles while another still has work
// (items differ in length: a block runs 1 to 4 row tiles).
//
// GEMM1's columns are arranged so that a lane holds the gate and the up value of
// the same intermediate in two accumulators (column tiles 0 and 1 take the gate
// and the up halves of the same two pairs), so SwiGLU is lane-local. The
// epilogues then transpose each 32 x 32 tile through LDS so that a lane holds
// one whole 16-wide block of one row: the requantization (amax, e4m3 scale,
// codes) and the bf16 packing are lane-local and the stores are 8 or 32
// contiguous bytes. Rows without a route are not written.
#include <atomic>

#include "experts.hpp"

namespace moe {

constexpr int kMaxDevices = 64;             // devices whose CU count is cached

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kCT = 2;                      // 32-column MFMA tiles per wave
constexpr int kBlockRows = 128;             // rows per block (4 row tiles of 32)
constexpr int kWaves = 4;                   // waves (column blocks) per workgroup
constexpr int kWgPerCu = 2;                 // workgroups a CU holds at once
constexpr int kStage = 4;                   // k-tiles per raw A stage in LDS
constexpr int kXcds = 8;
constexpr int kARowBytes = 32 * kStage;     // codes of one row in a stage
constexpr int kASfBytes = 4 * kStage;       // block scales of one row in a stage
constexpr int kSlabStride = 36;             // floats per row of an epilogue slab
constexpr int kAhBytes = 4 * 4 * 64 * 16;   // decoded A of one k-tile: [row tile][K-step][lane] 16 bytes

// The LDS position (16-byte unit within its 128-byte row) of chunk k of row r:
// rows r and r + 1 fall in different halves of the 64 banks, so the 8
// positions of the rows r % 2 == const must differ over 16 consecutive rows.
__device__ __forceinline__ int chunk_swizzle(int k, int r) { return k ^ (r & 7) ^ ((r >> 3) & 1); }

// LDS of a workgroup (68 KB: two fit a CU): the raw A stages (codes, swizzled;
// block scales), which the epilogue's tile transposes reuse once the k-loop is
// done, and the two decoded f16 A k-tiles.
struct ALds {
    union {
        struct {
            alignas(16) uint8_t codes[2][kBlockRows * kARowBytes];
            alignas(16) uint8_t sf[2][kBlockRows * kASfBytes];
        } raw;
        float slab[kWaves][2][32 * kSlabStride];   // per wave, two: the epilogue's tile transposes
    } u;
    alignas(16) uint8_t ah[2][kAhBytes];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
    // raw buffer (stride 0) with no range limit; gfx9 data-format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// One lane's raw weight operands of one k-tile: blocks 2h and 2h + 1 of each
// column tile's column (8 bytes each, 256 bytes apart in the pair tile) and the
// u32 words holding their scales. In GEMM1 column tiles 0 and 1 are the two
// halves of the same pairs, whose scale bytes share words: kSW word pairs.
template <int MODE>
struct BRaw {
    static constexpr int kSW = MODE == 1 ? kCT / 2 : kCT;
    static constexpr int kLoads = 2 * kCT + 2 * kSW;
    uint2 b[kCT][2];
    uint32_t bsf[kSW][2];
};

struct BSrc {
    __amdgpu_buffer_rsrc_t b, bs;   // k-tile c at + 1024 c, + 128 c
    uint32_t b_off, bs_off;         // per lane
    int b_step, bs_step;            // from one pair to the next
};

// The weight loads of a k-tile in three parts, each issued as soon as the
// slot's previous contents are consumed (vmcnt drains in issue order, so a
// wait for one part never waits for a part issued later): the scale words
// (consumed by k-tile c - 1's last region), blocks 2h (words 0, 1: consumed
// by step 1) and blocks 2h + 1 (words 2, 3: consumed by step 3).
template <int MODE>
__device__ __forceinline__ void b_load_sf(BRaw<MODE>& r, const BSrc& p, int c) {
#pragma unroll
    for (int t = 0; t < BRaw<MODE>::kSW; ++t) {
        const int so = c * kSlotSfBytes + t * (MODE == 1 ? 2 : 1) * p.bs_step;
        r.bsf[t][0] = __builtin_amdgcn_raw_buffer_load_b32(p.bs, (int)p.bs_off, so, 0);
        r.bsf[t][1] = __builtin_amdgcn_raw_buffer_load_b32(p.bs, (int)p.bs_off + 32, so, 0);
    }
}

template <int MODE, int PART>
__device__ __forceinline__ void b_load_half(BRaw<MODE>& r, const BSrc& p, int c) {
#pragma unroll
    for (int j = 0; j < kCT; ++j) {
        const int so = c * kSlotBytes + (MODE == 1 ? (j >> 1) * 2 : j) * p.b_step;
        const int o = (int)p.b_off + (MODE == 1 ? (j & 1) * 8 : 0) + 256 * PART;
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(p.b, o, so, 0);
        r.b[j][PART] = make_uint2(v[0], v[1]);
    }
}

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

// The workgroup's copy of raw A stage g into LDS buffer g & 1, the rows of
// its RT routed row tiles only. Codes: wave w's load q covers rows
// 32q + 8w + [0, 8) (1 KB, lane l at byte 16 l): lane l fetches the chunk of
// row 32q + 8w + l / 8 whose swizzled position is l % 8 (the swizzle is an
// involution). Scales: waves 0 and 1, lane l fetches the 16 scale bytes of
// row 64w + l.
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

// kCoherent: agent-coherent copies (an intermediate other workgroups of the
// same launch published).
template <int RT, bool kCoherent>
__device__ __forceinline__ void a_stage_load(ALds& lds, const ASrc& p, int wave, int g) {
    const int buf = g & 1;
#pragma unroll
    for (int q = 0; q < RT; ++q) {
        const uint32_t l =
            __builtin_amdgcn_readfirstlane(lds_addr(&lds.u.raw.codes[buf][(32 * q + 8 * wave) * kARowBytes]));
        if (kCoherent) lds_copy16_sc1(p.a, l, p.a_off[q], (uint32_t)(g * kARowBytes));
        else lds_copy16(p.a, l, p.a_off[q], (uint32_t)(g * kARowBytes));
    }
    if (wave < (RT + 1) / 2) {
        const uint32_t l = __builtin_amdgcn_readfirstlane(lds_addr(&lds.u.raw.sf[buf][64 * wave * kASfBytes]));
        if (kCoherent) lds_copy16_sc1(p.as, l, p.as_off, (uint32_t)(g * kASfBytes));
        else lds_copy16(p.as, l, p.as_off, (uint32_t)(g * kASfBytes));
    }
}

// The workgroup's decode of A k-tile c (from raw stage c / 4) into the f16 tile
// ah[c % 2]: thread (wave w, lane l = 32 h + nn) makes the fragments (row tile
// i, K-step w, lane l) for i < RT -- u32 word w of chunk 2 (c % 4) + h of row
// 32 i + nn (8 codes: elements 32 h + 8 w + [0, 8) of the k-tile) under the
// scale of block 2h + w / 2 -- and stores each at ((4 i + w) 64 + l) 16: the
// 16 bytes lane l of a wave reads for K-step w of row tile i.
template <int RT>
struct ADec {
    uint32_t w[RT];
    uint32_t sf[RT];
};

template <int RT>
__device__ __forceinline__ void adec_read(ADec<RT>& r, const ALds& lds, int c, int wave, int nn, int h) {
    const int buf = (c / kStage) & 1, cc = c % kStage;
    const int pos = chunk_swizzle(2 * cc + h, nn) * 16 + 4 * wave;   // rows 32 i + nn: same low bits
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int row = 32 * i + nn;
        r.w[i] = *reinterpret_cast<const uint32_t*>(&lds.u.raw.codes[buf][row * kARowBytes + pos]);
        r.sf[i] = lds.u.raw.sf[buf][row * kASfBytes + 4 * cc + 2 * h + (wave >> 1)];
    }
}

template <int RT, int I0, int I1>
__device__ __forceinline__ void adec_write(const ADec<RT>& r, ALds& lds, int c, int wave, int lane) {
#pragma unroll
    for (int i = I0; i < (I1 < RT ? I1 : RT); ++i) {
        const half8 v = nvfp4x8_to_f16(r.w[i], splat_lo(e4m3x2_to_f16(r.sf[i])));
        *reinterpret_cast<half8*>(&lds.ah[c & 1][((4 * i + wave) * 64 + lane) * 16]) = v;
    }
}

// A fragments of K-step s of k-tile c, one 16-byte read per row tile.
template <int RT>
__device__ __forceinline__ void a_frags(half8 (&fa)[RT], const ALds& lds, int c, int s, int lane) {
#pragma unroll
    for (int i = 0; i < RT; ++i) fa[i] = *reinterpret_cast<const half8*>(&lds.ah[c & 1][((4 * i + s) * 64 + lane) * 16]);
}

// B fragments of K-step s: lane (r, h) takes u32 word s of its 16 code bytes
// (elements 32 h + 8 s + [0, 8) of the k-tile) under the scale of block
// 2h + s / 2.
template <int MODE>
__device__ __forceinline__ void b_frags(half8 (&fb)[kCT], const BRaw<MODE>& br, const half2v (&sb)[kCT], int s) {
#pragma unroll
    for (int j = 0; j < kCT; ++j) {
        const uint32_t w = s == 0 ? br.b[j][0].x : s == 1 ? br.b[j][0].y : s == 2 ? br.b[j][1].x : br.b[j][1].y;
        fb[j] = nvfp4x8_to_f16(w, s < 2 ? splat_lo(sb[j]) : splat_hi(sb[j]));
    }
}

// The weight block scales of one k-tile as f16 pairs (block 2h, block 2h + 1).
template <int MODE>
__device__ __forceinline__ void b_scales(const BRaw<MODE>& br, const uint32_t (&sel)[2], half2v (&sb)[kCT]) {
#pragma unroll
    for (int j = 0; j < kCT; ++j) {
        const int t = MODE == 1 ? j >> 1 : j;
        sb[j] = e4m3x2_to_f16(__builtin_amdgcn_perm(br.bsf[t][1], br.bsf[t][0], sel[MODE == 1 ? j & 1 : 0]));
    }
}

// Keeps a step's B decode in the region where it is written: without it the
// compiler sinks the VALU work next to its first use, into the following
// region, where it no longer overlaps the MFMAs. (The A fragments' LDS reads
// stay in their region by the region's scheduling barrier; their wait falls
// at the first MFMA that uses them.)
__device__ __forceinline__ void pin(half8 (&fb)[kCT]) {
#pragma unroll
    for (int j = 0; j < kCT; ++j) asm volatile("" : "+v"(fb[j]));
}

template <int RT>
__device__ __forceinline__ void step_mfma(const half8 (&fa)[RT], const half8 (&fb)[kCT], floatx16 (&acc)[RT][kCT]) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < kCT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// Scheduling of one K-step region: each of its RT x kCT MFMAs followed by its
// share of the region's VALU work (NV instructions) and memory instructions
// (NM: vector-memory and LDS reads and writes).
template <int RT, int NV, int NM>
__device__ __forceinline__ void interleave() {
    constexpr int kM = RT * kCT;
    constexpr int kV = (NV + kM - 1) / kM, kMem = (NM + kM - 1) / kM;
#pragma unroll
    for (int k = 0; k < kM; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);                 // VALU
        if (kMem > 0) __builtin_amdgcn_sched_group_barrier(0x020 | 0x100 | 0x200, kMem, 0);   // VMEM, DS
    }
    __builtin_amdgcn_sched_barrier(0);
}

// The epilogues transpose each 32 x 32 tile through a private LDS slab of the
// wave (rows padded to 36 floats: the 16-byte reads of 8 consecutive rows fall
// in 8 different bank groups), so that lane L then holds the 16 consecutive
// columns 16 (L % 2) + [0, 16) of row L / 2: one whole NVFP4 block (GEMM1) or
// 32 contiguous bytes of a bf16 row (GEMM2), with all arithmetic lane-local.
// A wave's LDS instructions execute in order, so its later reads see its
// earlier writes (those of other lanes included) without a wait; this only
// keeps the compiler from reordering them. The two slabs of a wave alternate
// between tiles, so a tile's writes never meet the previous tile's reads.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// lane l holds column l % 32 of rows 8(x/4) + 4(l/32) + x%4 in element x
__device__ __forceinline__ void slab_store(float* slab, const float (&v)[16], int lane) {
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int x = 0; x < 16; ++x) slab[(8 * (x >> 2) + 4 * h + (x & 3)) * kSlabStride + n] = v[x];
}

__device__ __forceinline__ void slab_load_row16(const float* slab, float (&v)[16], int lane) {
    const float4* src = reinterpret_cast<const float4*>(slab + (lane >> 1) * kSlabStride + 16 * (lane & 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 t = src[q];
        v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
}

// silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (each about
// 1 ulp): a third of the instructions of the correctly rounded expf and
// division, which dominate this epilogue. Saturates correctly: e^-g overflows
// to inf for g < -88 (silu -> -0) and underflows to 0 for large g (silu -> g).
__device__ __forceinline__ float silu_fast(float g) {
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// GEMM1 epilogue of one gate tile and its up tile (rows m0 + [0, 32),
// intermediates col0 + [0, 32)): SwiGLU lane-local in the MFMA layout, then
// per lane one block: amax, e4m3 scale, 16 codes, 8 code bytes and the scale
// byte stored when its row has a route (bit r of vmask).
template <bool kPub>
__device__ __forceinline__ void swiglu_quant_tile(const floatx16& gacc, const floatx16& uacc, float ga, float uc,
                                                  int lane, uint32_t vmask, const ExpArgs& a, int m0, int col0,
                                                  float* slab) {
    float hv[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        const float g = gacc[x] * ga;
        const float u = uacc[x] * uc;
        hv[x] = silu_fast(g) * u;
    }
    slab_store(slab, hv, lane);
    lds_order();
    float v[16];
    slab_load_row16(slab, v, lane);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, __builtin_fabsf(v[k]));
    const BlockScale bs = nvfp4_block_scale(amax, 1.0f);
    // finite values: products of finite accumulators
    const uint32_t w0 = nvfp4_codes8<false>(v, bs), w1 = nvfp4_codes8<false>(v + 8, bs);
    const int r = lane >> 1;
    if ((vmask >> r) & 1u) {
        const int64_t row = m0 + r;
        const int col = col0 + 16 * (lane & 1);
        uint8_t* cp = a.inter_codes + row * (a.I >> 1) + (col >> 1);
        uint8_t* sp = a.inter_sf + row * (a.I >> 4) + (col >> 4);
        if (kPub) {        // read by GEMM2 workgroups of the same launch: agent-coherent stores
            __hip_atomic_store(reinterpret_cast<uint64_t*>(cp), (uint64_t)w0 | ((uint64_t)w1 << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sp, (uint8_t)bs.byte, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            *reinterpret_cast<uint2*>(cp) = make_uint2(w0, w1);
            *sp = (uint8_t)bs.byte;
        }
    }
}

// GEMM2 epilogue of one tile: bf16 rows m0 + [0, 32), columns col0 + [0, 32);
// lane L stores 32 contiguous bytes of row L / 2.
__device__ __forceinline__ void bf16_tile(const floatx16& acc, float alpha, int lane, uint32_t vmask,
                                          const ExpArgs& a, int m0, int col0, float* slab) {
    float o[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) o[x] = acc[x] * alpha;
    slab_store(slab, o, lane);
    lds_order();
    float v[16];
    slab_load_row16(slab, v, lane);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = bf16x2_pack(v[2 * k], v[2 * k + 1]);   // finite sums
    const int r = lane >> 1;
    if ((vmask >> r) & 1u) {
        uint4* dst = reinterpret_cast<uint4*>(a.rows + (int64_t)(m0 + r) * a.rows_stride + col0 + 16 * (lane & 1));
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
}

// A wave's k-loop state.
template <int MODE, int RT>
struct KState {
    floatx16 acc[RT][kCT];
    BRaw<MODE> ring[2];             // weight k-tile c in slot c % 2
    half8 fa[2][RT], fb[2][kCT];    // fragments of the current and the next K-step
    half2v sb[kCT];                 // the current k-tile's weight block scales
};

struct KPos {
    int KT, NS;                     // k-tiles, raw stages
    int wave, lane, nn, h;
};

// One k-tile c (position CC in its raw stage g; weight ring slot c % 2): 4
// K-step regions of RT x 2 MFMAs. While the MFMAs of step s run, the fragments
// of step s + 1 are read and decoded (in the last region those of step 0 of
// k-tile c + 1), the workgroup decodes the A of k-tile c + 1 (regions 0 to 2)
// and the weights of k-tile c + 2 load into the slot k-tile c has finished
// with. The barrier after region 2 publishes the A of k-tile c + 1 (and frees
// ah[c % 2], whose last reads were issued before it); once a stage (CC == 2)
// it also waits for raw stage g + 1, copied during k-tile 4g - 2, and frees raw
// buffer g % 2 for stage g + 2 (raw stage g was last read by the decode of
// k-tile 4g + 3). Past the end the copies repeat the last stage and the weight
// loads the last k-tile.
template <int MODE, int RT, bool kCoh, int CC>
__device__ __forceinline__ void ktile(KState<MODE, RT>& st, ALds& lds, const ASrc& ap, const BSrc& p,
                                      const uint32_t (&sel)[2], const KPos& k, int c) {
    constexpr int SLOT = CC & 1, NXT = SLOT ^ 1;
    // weight loads issued between one stage copy (k-tile 4g - 2, region 3) and
    // the barrier that waits for it (k-tile 4g + 2, after region 2): 4 k-tiles'
    // worth
    constexpr int kAfterCopy = 4 * BRaw<MODE>::kLoads;
    static_assert(kAfterCopy <= 63, "vmcnt range");
    constexpr int kVB = 8 * kCT;                                    // VALU of one step's B fragments
    constexpr int kVA = 9;                                          // VALU of one decoded A fragment
    const int cn = min(c + 2, k.KT - 1);
    ADec<RT> ad;
    // region 0: the raw A of k-tile c + 1 read; the weight scales of k-tile
    // c + 2 load into slot SLOT
    a_frags(st.fa[1], lds, c, 1, k.lane);
    b_frags(st.fb[1], st.ring[SLOT], st.sb, 1);
    b_load_sf(st.ring[SLOT], p, cn);
    adec_read(ad, lds, c + 1, k.wave, k.nn, k.h);
    step_mfma(st.fa[0], st.fb[0], st.acc);
    pin(st.fb[1]);
    interleave<RT, kVB, RT + 2 * BRaw<MODE>::kSW + 2 * RT>();
    // region 1: half of it decoded; blocks 2h of k-tile c + 2 load
    a_frags(st.fa[0], lds, c, 2, k.lane);
    b_frags(st.fb[0], st.ring[SLOT], st.sb, 2);
    b_load_half<MODE, 0>(st.ring[SLOT], p, cn);
    adec_write<RT, 0, (RT + 1) / 2>(ad, lds, c + 1, k.wave, k.lane);
    step_mfma(st.fa[1], st.fb[1], st.acc);
    pin(st.fb[0]);
    interleave<RT, kVB + kVA * ((RT + 1) / 2), RT + kCT + (RT + 1) / 2>();
    // region 2: the rest decoded
    a_frags(st.fa[1], lds, c, 3, k.lane);
    b_frags(st.fb[1], st.ring[SLOT], st.sb, 3);
    adec_write<RT, (RT + 1) / 2, RT>(ad, lds, c + 1, k.wave, k.lane);
    step_mfma(st.fa[0], st.fb[0], st.acc);
    pin(st.fb[1]);
    interleave<RT, kVB + kVA * (RT / 2), RT + RT / 2>();
    // every wave's part of the A of k-tile c + 1 written (and its reads of
    // ah[c % 2] done); once a stage, its copy of raw stage g + 1 landed
    if (CC == 2) __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kAfterCopy) & lgkmcnt_zero());
    else __builtin_amdgcn_s_waitcnt(lgkmcnt_zero());
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // region 3: step 0 of k-tile c + 1 read and decoded; blocks 2h + 1 of
    // k-tile c + 2 load into slot SLOT. The copy of raw stage g + 2 (into raw
    // buffer g % 2) issues with the weight loads it will be waited for with:
    // vmcnt drains in order, so a copy issued earlier would hold up the next
    // wait for the weights by a memory latency
    if (CC == 2) a_stage_load<RT, kCoh>(lds, ap, k.wave, min(c / kStage + 2, k.NS - 1));
    b_load_half<MODE, 1>(st.ring[SLOT], p, cn);
    half2v sb1[kCT];
    b_scales(st.ring[NXT], sel, sb1);
    a_frags(st.fa[0], lds, c + 1, 0, k.lane);
    b_frags(st.fb[0], st.ring[NXT], sb1, 0);
    step_mfma(st.fa[1], st.fb[1], st.acc);
    pin(st.fb[0]);
    interleave<RT, kVB + 4 * kCT, RT + kCT>();
#pragma unroll
    for (int j = 0; j < kCT; ++j) st.sb[j] = sb1[j];
}

// Blocks of one or two row tiles: each wave decodes its own A fragments from
// the raw stage -- RT of them a K-step, no more than it decodes for B -- which
// saves the decoded tile's LDS traffic and leaves one barrier per raw stage
// instead of one per k-tile.
template <int RT>
struct ARaw {
    uint4 a[RT];                    // codes of chunk 2 (c % 4) + h of rows 32 i + nn
    uint32_t asf[RT];               // their 4 block scales of k-tile c
};

template <int RT>
__device__ __forceinline__ void a_read(ARaw<RT>& r, const ALds& lds, int c, int nn, int h) {
    const int buf = (c / kStage) & 1, cc = c % kStage;
    const int pos = chunk_swizzle(2 * cc + h, nn) * 16;       // rows 32 i + nn: same low bits
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        r.a[i] = *reinterpret_cast<const uint4*>(&lds.u.raw.codes[buf][(32 * i + nn) * kARowBytes + pos]);
        r.asf[i] = *reinterpret_cast<const uint32_t*>(&lds.u.raw.sf[buf][(32 * i + nn) * kASfBytes + 4 * cc]);
    }
}

template <int RT>
__device__ __forceinline__ void a_own_frags(half8 (&fa)[RT], const ARaw<RT>& ar, const half2v (&sa)[RT], int s) {
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const uint32_t w = s == 0 ? ar.a[i].x : s == 1 ? ar.a[i].y : s == 2 ? ar.a[i].z : ar.a[i].w;
        fa[i] = nvfp4x8_to_f16(w, s < 2 ? splat_lo(sa[i]) : splat_hi(sa[i]));
    }
}

template <int RT>
__device__ __forceinline__ void a_scales(const ARaw<RT>& ar, int h, half2v (&sa)[RT]) {
#pragma unroll
    for (int i = 0; i < RT; ++i) sa[i] = e4m3x2_to_f16(ar.asf[i] >> (16 * h));
}

template <int RT>
__device__ __forceinline__ void pin_own(half8 (&fa)[RT], half8 (&fb)[kCT]) {
#pragma unroll
    for (int i = 0; i < RT; ++i) asm volatile("" : "+v"(fa[i]));
    pin(fb);
}

template <int MODE, int RT>
struct KStateOwn {
    floatx16 acc[RT][kCT];
    BRaw<MODE> ring[2];             // weight k-tile c in slot c % 2
    ARaw<RT> ar[2];                 // raw A of k-tile c in slot c % 2
    half8 fa[2][RT], fb[2][kCT];    // fragments of the current and the next K-step
    half2v sa[RT], sb[kCT];         // the current k-tile's block scales
};

// One k-tile c of the own-decode form: 4 K-step regions; while the MFMAs of
// step s run the wave decodes the fragments of step s + 1 (in the last region
// those of step 0 of k-tile c + 1), the weights of k-tile c + 2 load into ring
// slot c % 2 and the raw A of k-tile c + 2 is read into A slot c % 2. A barrier in
// k-tile 4g + 2 publishes raw stage g + 1 (copied during k-tile 4g - 2) and
// frees raw buffer g % 2 for stage g + 2: every read of stage g was issued by
// then (the raw A of k-tile c is read during k-tile c - 2).
template <int MODE, int RT, bool kCoh, int CC>
__device__ __forceinline__ void ktile_own(KStateOwn<MODE, RT>& st, ALds& lds, const ASrc& ap, const BSrc& p,
                                          const uint32_t (&sel)[2], const KPos& k, int c) {
    constexpr int d = CC & 1, SLOT = d, NXT = d ^ 1;
    constexpr int kAfterCopy = 4 * BRaw<MODE>::kLoads;
    static_assert(kAfterCopy <= 63, "vmcnt range");
    constexpr int kV = 8 * (RT + kCT);                              // VALU of one step's fragments
    const int cn = min(c + 2, k.KT - 1);
    // region 0
    a_own_frags(st.fa[1], st.ar[d], st.sa, 1);
    b_frags(st.fb[1], st.ring[SLOT], st.sb, 1);
    b_load_sf(st.ring[SLOT], p, cn);
    step_mfma(st.fa[0], st.fb[0], st.acc);
    pin_own(st.fa[1], st.fb[1]);
    interleave<RT, kV, 2 * BRaw<MODE>::kSW>();
    // region 1
    a_own_frags(st.fa[0], st.ar[d], st.sa, 2);
    b_frags(st.fb[0], st.ring[SLOT], st.sb, 2);
    b_load_half<MODE, 0>(st.ring[SLOT], p, cn);
    step_mfma(st.fa[1], st.fb[1], st.acc);
    pin_own(st.fa[0], st.fb[0]);
    interleave<RT, kV, kCT>();
    if (CC == 2) {
        // every wave: its reads of stage g done, its copy of stage g + 1 landed
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kAfterCopy) & lgkmcnt_zero());
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    }
    // region 2
    a_own_frags(st.fa[1], st.ar[d], st.sa, 3);
    b_frags(st.fb[1], st.ring[SLOT], st.sb, 3);
    step_mfma(st.fa[0], st.fb[0], st.acc);
    pin_own(st.fa[1], st.fb[1]);
    interleave<RT, kV, 0>();
    // region 3: step 0 of k-tile c + 1; the copy of raw stage g + 2 (into raw
    // buffer g % 2, free since the barrier) issues with the weight loads it
    // will be waited for with
    half2v sa1[RT], sb1[kCT];
    a_scales(st.ar[d ^ 1], k.h, sa1);
    b_scales(st.ring[NXT], sel, sb1);
    a_own_frags(st.fa[0], st.ar[d ^ 1], sa1, 0);
    b_frags(st.fb[0], st.ring[NXT], sb1, 0);
    if (CC == 2) a_stage_load<RT, kCoh>(lds, ap, k.wave, min(c / kStage + 2, k.NS - 1));
    b_load_half<MODE, 1>(st.ring[SLOT], p, cn);
    a_read(st.ar[d], lds, cn, k.nn, k.h);
    step_mfma(st.fa[1], st.fb[1], st.acc);
    pin_own(st.fa[0], st.fb[0]);
    interleave<RT, kV + 2 * (RT + kCT), kCT + 2 * RT>();
#pragma unroll
    for (int i = 0; i < RT; ++i) st.sa[i] = sa1[i];
#pragma unroll
    for (int j = 0; j < kCT; ++j) st.sb[j] = sb1[j];
}

// The epilogue of a wave's block, one 32 x 32 tile (GEMM1: a gate tile and
// its up tile) at a time, the wave's two slabs alternating.
template <int MODE, int RT, bool kPub>
__device__ __forceinline__ void epilogue(const floatx16 (&acc)[RT][kCT], const ExpArgs& a, ALds& lds, int e, int row0,
                                         int cb, int wave, int lane, const uint32_t (&vmask)[4]) {
    if (MODE == 1) {
        const float ga = a.w.g1_alphas[e], uc = a.w.g1_scale_c[e];
#define MOE_EPI1(i)                                                                                          \
    if (RT > i) swiglu_quant_tile<kPub>(acc[RT > i ? i : 0][0], acc[RT > i ? i : 0][1], ga, uc, lane, vmask[i], a, \
                                        row0 + 32 * i, 32 * cb, lds.u.slab[wave][i & 1])
        MOE_EPI1(0); MOE_EPI1(1); MOE_EPI1(2); MOE_EPI1(3);
#undef MOE_EPI1
    } else {
        const float alpha = a.w.g2_alphas[e];
#define MOE_EPI2(i, j) \
    if (RT > i) bf16_tile(acc[RT > i ? i : 0][j], alpha, lane, vmask[i], a, row0 + 32 * i, 64 * cb + 32 * j, \
                          lds.u.slab[wave][j])
        MOE_EPI2(0, 0); MOE_EPI2(0, 1); MOE_EPI2(1, 0); MOE_EPI2(1, 1);
        MOE_EPI2(2, 0); MOE_EPI2(2, 1); MOE_EPI2(3, 0); MOE_EPI2(3, 1);
#undef MOE_EPI2
    }
}

// One wave's block: rows [row0, row0 + 32 RT) of expert e, column block cb
// (computed but not stored when store is false: a column group past the end).
// vmask[i]: bit r is set when row 32 i + r of the block has a route.
// The k-loop runs at wave priority 1, the prologue, epilogue and item start at
// 0: while the CU's other workgroup is outside its k-loop, the instruction
// arbiter serves this one's MFMAs and decode first (prefill_t4096 1113.5 ->
// 1108.3 us a launch, three alternations on one box; the reverse, the
// epilogue first, measured 1115.7 us).
template <int MODE, int RT, bool kPub>
__device__ __forceinline__ void run_block(const ExpArgs& a, ALds& lds, const ASrc& ap, int e, int row0, int cb,
                                          bool store, int wave, int lane, const uint32_t (&vmask)[4]) {
    const int h = lane >> 5, nn = lane & 31, n = lane & 15, hh = (lane >> 4) & 1;
    const int K = MODE == 1 ? a.H : a.I;
    const int NS = K / (64 * kStage);
    constexpr bool kCoh = kPub && MODE == 2;

    BSrc p;
    if (MODE == 1) {
        const int pair0 = cb * kCT;                                 // 2 pairs: 32 intermediates
        p.b = buffer_rsrc(a.w.w13 + e * a.w.w13_expert_stride_bytes + pair0 * a.w.w13_pair_stride_bytes);
        p.bs = buffer_rsrc(a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + pair0 * a.w.w13_sf_pair_stride_bytes);
        p.b_step = (int)a.w.w13_pair_stride_bytes;
        p.bs_step = (int)a.w.w13_sf_pair_stride_bytes;
        // column nn of tile g: pair nn / 16, half g, row n
        p.b_off = hh * (uint32_t)p.b_step + (uint32_t)(2 * h * 16 + n) * 16;
        p.bs_off = hh * (uint32_t)p.bs_step + 64 * h + 4 * (n >> 1);
    } else {
        const int pair0 = cb * kCT;                                 // 2 pairs: 64 output columns
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

    KPos k;
    k.KT = NS * kStage;
    k.NS = NS;
    k.wave = wave;
    k.lane = lane;
    k.nn = nn;
    k.h = h;
    if constexpr (RT <= 2) {
        KStateOwn<MODE, RT> st;
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < kCT; ++j)
#pragma unroll
                for (int x = 0; x < 16; ++x) st.acc[i][j][x] = 0.0f;
        // Prologue: raw stages 0 and 1, weight k-tiles 0 and 1, the raw A of
        // k-tiles 0 and 1, the fragments of step 0.
        a_stage_load<RT, kCoh>(lds, ap, wave, 0);
        a_stage_load<RT, kCoh>(lds, ap, wave, min(1, NS - 1));
        b_load(st.ring[0], p, 0);
        b_load(st.ring[1], p, min(1, k.KT - 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
        __syncthreads();
        a_read(st.ar[0], lds, 0, nn, h);
        a_read(st.ar[1], lds, min(1, k.KT - 1), nn, h);
        a_scales(st.ar[0], h, st.sa);
        b_scales(st.ring[0], sel, st.sb);
        a_own_frags(st.fa[0], st.ar[0], st.sa, 0);
        b_frags(st.fb[0], st.ring[0], st.sb, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        for (int c0 = 0; c0 < k.KT; c0 += kStage) {
            ktile_own<MODE, RT, kCoh, 0>(st, lds, ap, p, sel, k, c0);
            ktile_own<MODE, RT, kCoh, 1>(st, lds, ap, p, sel, k, c0 + 1);
            ktile_own<MODE, RT, kCoh, 2>(st, lds, ap, p, sel, k, c0 + 2);
            ktile_own<MODE, RT, kCoh, 3>(st, lds, ap, p, sel, k, c0 + 3);
        }
        __builtin_amdgcn_s_setprio(0);
        // the epilogue's slabs reuse the raw stages: every wave's copies landed
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
        __syncthreads();
        if (store) epilogue<MODE, RT, kPub>(st.acc, a, lds, e, row0, cb, wave, lane, vmask);
    } else {
        KState<MODE, RT> st;
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < kCT; ++j)
#pragma unroll
                for (int x = 0; x < 16; ++x) st.acc[i][j][x] = 0.0f;
        // Prologue: raw stages 0 and 1, weight k-tiles 0 and 1, the A of
        // k-tile 0 decoded, the fragments of its step 0.
        a_stage_load<RT, kCoh>(lds, ap, wave, 0);
        a_stage_load<RT, kCoh>(lds, ap, wave, min(1, NS - 1));
        b_load(st.ring[0], p, 0);
        b_load(st.ring[1], p, min(1, k.KT - 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
        __syncthreads();
        {
            ADec<RT> ad;
            adec_read(ad, lds, 0, wave, nn, h);
            adec_write<RT, 0, RT>(ad, lds, 0, wave, lane);
        }
        __builtin_amdgcn_s_waitcnt(lgkmcnt_zero());
        __syncthreads();
        b_scales(st.ring[0], sel, st.sb);
        a_frags(st.fa[0], lds, 0, 0, lane);
        b_frags(st.fb[0], st.ring[0], st.sb, 0);
        __builtin_amdgcn_sched_barrier(0);
        // k-tiles four at a time (one raw stage)
        __builtin_amdgcn_s_setprio(1);
        for (int c0 = 0; c0 < k.KT; c0 += kStage) {
            ktile<MODE, RT, kCoh, 0>(st, lds, ap, p, sel, k, c0);
            ktile<MODE, RT, kCoh, 1>(st, lds, ap, p, sel, k, c0 + 1);
            ktile<MODE, RT, kCoh, 2>(st, lds, ap, p, sel, k, c0 + 2);
            ktile<MODE, RT, kCoh, 3>(st, lds, ap, p, sel, k, c0 + 3);
        }
        __builtin_amdgcn_s_setprio(0);
        // the epilogue's slabs reuse the raw stages: every wave's copies landed
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
        __syncthreads();
        if (store) epilogue<MODE, RT, kPub>(st.acc, a, lds, e, row0, cb, wave, lane, vmask);
    }
}

// The work queues (meta's queue words): queue x holds the GEMM1 items of the
// row blocks [x bpx, (x + 1) bpx), ncg1 a block, then their GEMM2 items.
// Position v of a queue's GEMM1 (or GEMM2) items names a cell by item_cell.
struct Queues {
    int32_t* q;             // items taken from each queue; q[kXcds]: workgroups finished
    int nblocks, bpx, ncg1, ncg2, home;
};

__device__ __forceinline__ int queue_blocks(const Queues& Q, int x) {
    return min(max(Q.nblocks - x * Q.bpx, 0), Q.bpx);
}

// Thread 0: the next item, x << 24 | its position in queue x; -1 when every
// queue is empty. From the home queue while it lasts; then from the queue
// with the most items left, by one read of all the counters (8 loads in
// flight at once) and an increment of the chosen one, again while a chosen
// queue turns out to be empty. *done (in LDS, so that no register stays live
// across items) holds the queues this workgroup found empty. A counter passes
// its item count by at most one per workgroup; the last workgroup out resets
// them.
__device__ __forceinline__ int take_item(const Queues& Q, uint32_t* done) {
    uint32_t d = *done;
    int item = -1;
    const int ni = Q.ncg1 + Q.ncg2;
    if (!((d >> Q.home) & 1u)) {
        const int v = __hip_atomic_fetch_add(Q.q + Q.home, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v < queue_blocks(Q, Q.home) * ni) item = (Q.home << 24) | v;
        else d |= 1u << Q.home;
    }
    while (item < 0 && d != (1u << kXcds) - 1) {
        int left[kXcds];
#pragma unroll
        for (int x = 0; x < kXcds; ++x)
            left[x] = ((d >> x) & 1u) ? 0
                      : queue_blocks(Q, x) * ni - __hip_atomic_load(Q.q + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int best = -1, most = 0;
#pragma unroll
        for (int x = 0; x < kXcds; ++x) {
            if (left[x] > most) { most = left[x]; best = x; }
            if (left[x] <= 0) d |= 1u << x;
        }
        if (best < 0) break;
        const int v = __hip_atomic_fetch_add(Q.q + best, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v < queue_blocks(Q, best) * ni) item = (best << 24) | v;
        else d |= 1u << best;
    }
    *done = d;
    return item;
}

// The cell (row block *bx, column group *cg) at position v of one GEMM's items
// of the chunk [b0, b0 + nb): v / ncg names a block, whose expert's blocks in
// the chunk, [gs, ge), hold the positions [(gs - b0) ncg, (ge - b0) ncg); those
// go column group major. Every block below the routed count belongs to an
// expert whose padded rows start and end on block boundaries.
__device__ __forceinline__ void item_cell(const ExpArgs& a, int b0, int nb, int v, int ncg, int* bx, int* cg) {
    const int bm = b0 + v / ncg;
    const int e = __builtin_amdgcn_readfirstlane(a.meta[a.L.tile_expert + bm * kBlockRows / a.tile_m]);
    const int gs = max(__builtin_amdgcn_readfirstlane(a.meta[a.L.expert_offsets + e]) / kBlockRows, b0);
    const int ge = min(__builtin_amdgcn_readfirstlane(a.meta[a.L.expert_offsets + e + 1]) / kBlockRows, b0 + nb);
    const int g = ge - gs, u = v - (gs - b0) * ncg;
    *bx = gs + u % g;
    *cg = u / g;
}

// One work item of GEMM MODE (1: GEMM1 + SwiGLU + requant, 2: GEMM2): row
// block bx, column group cg. GEMM1 publishes its part of a row block's
// intermediate with agent-coherent stores and counts itself on the block's
// ready counter; GEMM2 waits for all GEMM1 items of its block, copies the
// intermediate with agent-coherent loads, and the block's last GEMM2 item
// returns the counters to 0. Thread 0 takes the workgroup's next item into
// *s_next as soon as this one waits for nothing more (a GEMM1 item at once, a
// GEMM2 item once its block's intermediate is ready): a workgroup then never
// holds an item that another one waits for while it waits itself.
template <int MODE>
__device__ __forceinline__ void tiled_item(const ExpArgs& a, ALds& lds, int bx, int cg, int ncg, int ncb, int ncg1,
                                           const Queues& Q, uint32_t* done, int* s_next) {
    // the lane index through an empty asm: the per-lane offsets derived from it
    // are recomputed for every item rather than kept live across the item loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (MODE == 1 && threadIdx.x == 0) *s_next = take_item(Q, done);

    const int row0 = bx * kBlockRows;
    const int e = a.meta[a.L.tile_expert + row0 / a.tile_m];
    if (e < 0 || e >= a.E_local) {                            // uniform over the workgroup
        if (MODE == 2 && threadIdx.x == 0) *s_next = take_item(Q, done);
        return;
    }
    int cb = cg * kWaves + wave;
    const bool store = cb < ncb;
    cb = min(cb, ncb - 1);

    const int nn = lane & 31;
    // bit r of vmask[i]: row 32 i + r of the block has a route
    uint32_t vmask[4];
    int rt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = a.meta[a.L.perm2tok + row0 + 32 * i + nn];
        vmask[i] = (uint32_t)__ballot(t >= 0 && t < a.T);
        if (vmask[i] != 0u) rt = i + 1;
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
                ap.a_off[q] = (uint32_t)t * (uint32_t)(a.H >> 1) + chunk_swizzle(c16, r) * 16;
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
                ap.a_off[q] = (uint32_t)r * (uint32_t)(a.I >> 1) + chunk_swizzle(c16, r) * 16;
            }
            ap.as_off = (uint32_t)((64 * wave + lane) & (kBlockRows - 1)) * (uint32_t)(a.I >> 4);
        }
    }

    if (rt == 0) {                                        // uniform: a block of padding only
        if (MODE == 2 && threadIdx.x == 0) *s_next = take_item(Q, done);
        return;
    }
    // the block's two counters: meta's sub_sync of its first 16-row tile
    if (MODE == 2) {
        if (threadIdx.x == 0) {
            wait_ready(a.sync + (int64_t)kSubSyncStride * (bx * (kBlockRows / 16)), ncg1, a.status);
            *s_next = take_item(Q, done);
        }
        __syncthreads();
    }
    switch (rt) {
        case 1: run_block<MODE, 1, true>(a, lds, ap, e, row0, cb, store, wave, lane, vmask); break;
        case 2: run_block<MODE, 2, true>(a, lds, ap, e, row0, cb, store, wave, lane, vmask); break;
        case 3: run_block<MODE, 3, true>(a, lds, ap, e, row0, cb, store, wave, lane, vmask); break;
        default: run_block<MODE, 4, true>(a, lds, ap, e, row0, cb, store, wave, lane, vmask); break;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores (GEMM1) or copies (GEMM2) are done
    __syncthreads();
    int32_t* cnt = a.sync + (int64_t)kSubSyncStride * (bx * (kBlockRows / 16));
    if (threadIdx.x == 0) {
        if (MODE == 1) {
            __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (__hip_atomic_fetch_add(cnt + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ncg - 1) {
            __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(cnt + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// A pointer into the kernel argument segment (constant address space: its
// loads are scalar).
template <typename T>
using KernArg = const T __attribute__((address_space(4)))*;

// Both GEMMs in one launch, persistent workgroups (two a CU) looping over the
// queues' items. A GEMM2 item only waits for GEMM1 items that running
// workgroups have taken (a queue yields all its GEMM1 items before any GEMM2
// item, and a workgroup holds a taken item only while its current one waits
// for nothing), so every wait ends. The last workgroup out returns the queue
// counters to 0 for the next call on the same routing.
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kWgPerCu)))
tiled_fused_kernel(ExpArgs a, int ncg1, int ncb1, int ncg2, int ncb2) {
    __shared__ ALds lds;
    __shared__ int s_next;
    __shared__ uint32_t s_done;
    Queues Q;
    Q.q = a.queue;
    Q.nblocks = __builtin_amdgcn_readfirstlane(a.meta[a.L.num_tiles]) * (a.tile_m / kBlockRows);
    Q.bpx = (Q.nblocks + kXcds - 1) / kXcds;
    Q.ncg1 = ncg1;
    Q.ncg2 = ncg2;
    Q.home = (int)(blockIdx.x & (kXcds - 1));
    if (threadIdx.x == 0) {
        s_done = 0;
        s_next = take_item(Q, &s_done);
    }
    __syncthreads();
    int it = __builtin_amdgcn_readfirstlane(s_next);
    while (it >= 0) {
        __syncthreads();                                  // every thread has read s_next
        // the arguments are read again from the kernel argument segment for
        // every item (an empty asm hides the pointer's value): left to
        // itself the compiler keeps every field live in registers across the
        // loop, which spills the k-loop's registers
        KernArg<ExpArgs> pa = (KernArg<ExpArgs>)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(pa));
        const ExpArgs& ai = *(const ExpArgs*)pa;
        const int x = it >> 24, v = it & 0xFFFFFF;
        const int nb = queue_blocks(Q, x), n1 = nb * ncg1, b0 = x * Q.bpx;
        int bx, cg;
        if (v < n1) {
            item_cell(ai, b0, nb, v, ncg1, &bx, &cg);
            tiled_item<1>(ai, lds, bx, cg, ncg1, ncb1, ncg1, Q, &s_done, &s_next);
        } else {
            item_cell(ai, b0, nb, v - n1, ncg2, &bx, &cg);
            tiled_item<2>(ai, lds, bx, cg, ncg2, ncb2, ncg1, Q, &s_done, &s_next);
        }
        __syncthreads();
        it = __builtin_amdgcn_readfirstlane(s_next);
    }
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(Q.q + kXcds, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
        for (int y = 0; y <= kXcds; ++y) __hip_atomic_store(Q.q + y, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

bool tiled_shape_ok(int T, int H, int I, int tile_m) {
    // whole row blocks; K = H and K = I in whole A stages (4 k-tiles); 32-bit
    // per-lane offsets into the activation codes
    return tile_m % kBlockRows == 0 && H % (64 * kStage) == 0 && I % (64 * kStage) == 0 &&
           (int64_t)T * (H / 2) < ((int64_t)1 << 31);
}

int launch_tiled(const ExpArgs& a, hipStream_t s) {
    // the routed row blocks are read from the metadata on the device; the
    // queues' item indices are 24-bit
    const int nx = (int)(a.L.rows_max / kBlockRows);
    const int ncb1 = a.I / 32, ncb2 = a.H / 64;    // column blocks of one wave
    const int ncg1 = (ncb1 + kWaves - 1) / kWaves, ncg2 = (ncb2 + kWaves - 1) / kWaves;
    if ((int64_t)((nx + kXcds - 1) / kXcds) * (ncg1 + ncg2) >= (1 << 24))
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: too many row blocks for the work queues");
    // the device's compute-unit count, read once per device (racing first
    // calls store the same value)
    static std::atomic<int> s_cus[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(MOE_ELAUNCH, "moe_experts_fwd: no current device");
    int cus = dev < kMaxDevices ? s_cus[dev].load(std::memory_order_relaxed) : 0;
    if (cus < 1) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            return fail(MOE_ELAUNCH, "moe_experts_fwd: cannot read the device's compute unit count");
        if (dev < kMaxDevices) s_cus[dev].store(cus, std::memory_order_relaxed);
    }
    // two workgroups per CU (each wave takes half of a SIMD's registers), a
    // multiple of the 8 XCDs
    const int grid = (kWgPerCu * cus + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(tiled_fused_kernel, dim3((unsigned)grid), dim3(64 * kWaves), 0, s, a, ncg1, ncb1, ncg2, ncb2);
    return MOE_OK;
}

}  // namespace moe
