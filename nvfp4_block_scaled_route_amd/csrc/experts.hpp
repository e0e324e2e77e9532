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
};

constexpr int kSlotBytes = 1024, kSlotSfBytes = 128;   // converted layout: per pair and k-tile

// The tiled path: 128-row blocks of one expert (tile_m % 128 == 0), K in whole
// 4-k-tile stages (H % 256 == 0, I % 256 == 0), activation code offsets below
// 2^31 bytes.
bool tiled_shape_ok(int T, int H, int I, int tile_m);
void launch_tiled(const ExpArgs& a, hipStream_t s);

}  // namespace moe
