// Internal declarations shared by the planner, the kernels and the C ABI.
#pragma once

#include <cstdint>
#include <vector>

#include "bfz.h"

namespace bfz {

constexpr int kTileDim = BFZ_TILE_DIM;
constexpr int kTileElems = BFZ_TILE_ELEMS;
// Weights one pack / unpack launch can address: their base pointers travel
// as kernel arguments (no per-call device copies), so a shard touching
// more weights than this is covered by several launches.
constexpr int kSegWeights = 64;

// One row of the device lookup table: where a slot's tile sits in its
// row-major weight.  24 bytes.
struct TileEntry {
    int64_t base;         // offset of the tile's element (0, 0): (e H + 128 i) W + 128 j
    int32_t ld;           // W, the weight's row stride
    int32_t scale_index;  // (e hb + i) wb + j, its cell of the scale grid
    int16_t valid_rows;   // 1..128 (0 in a padding slot)
    int16_t valid_cols;   // 1..128 (0 in a padding slot)
    int16_t local;        // weight index minus the launch segment's first weight; -1: padding
    int16_t reserved;
};
static_assert(sizeof(TileEntry) == 24, "TileEntry layout");

// A run of consecutive slots whose weights fit one launch.
struct Segment {
    int64_t slot0, n_slots;
    int32_t weight0, n_weights;
};

struct PackArgs {
    const float* src[kSegWeights];
};

struct UnpackArgs {
    uint8_t* codes[kSegWeights];
    float* scale[kSegWeights];
};

struct TransposeArgs {
    uint8_t* codes[kSegWeights];  // W^T, row-major [E, W, H]
    float* scale[kSegWeights];    // [E, W, ceil(H / 128)]
    int32_t rows[kSegWeights];    // H of each weight
};

// What the step kernels need of one step: the FP32 scalars, rounded once
// from double, the options, and the state layout.
struct StepScalars {
    float b1, c1, b2, c2, step_size, sbc2, eps, decay;
    int32_t has_decay;
    int32_t pow2;          // power-of-two tile scales
    int64_t state_stride;  // floats from one tile of master / m / v to the next
};

// Kernel launchers (kernels.hip).  They return a hipError_t value as int.
int launch_pack(const TileEntry* d_entries, int64_t n_slots, float* dst, int64_t dst_stride,
                const PackArgs& args, void* stream);
int launch_unpack(const TileEntry* d_entries, int64_t n_slots, const uint8_t* codes,
                  const float* scale_inv, const UnpackArgs& args, void* stream);
int launch_step(float* master, const float* grad, float* m, float* v, uint8_t* codes,
                float* scale_inv, int64_t n_tiles, const StepScalars& s, void* stream);
int launch_fold_step(const TileEntry* d_entries, int64_t n_slots, const PackArgs& grads,
                     float* master, float* m, float* v, uint8_t* codes, float* scale_inv,
                     const StepScalars& s, void* stream);
int launch_fold_step_unfold(const TileEntry* d_entries, int64_t n_slots, const PackArgs& grads,
                            const UnpackArgs& outs, float* master, float* m, float* v,
                            uint8_t* codes, float* scale_inv, const StepScalars& s, void* stream);
int launch_fold_step_unfold_t(const TileEntry* d_entries, int64_t n_slots, const PackArgs& grads,
                              const UnpackArgs& outs, const TransposeArgs& touts, float* master,
                              float* m, float* v, uint8_t* codes, float* scale_inv,
                              const StepScalars& s, void* stream);
// order: the launch's workgroup -> slot map (a permutation of [0, n_slots)).
int launch_transpose_pow2(const TileEntry* d_entries, const int32_t* order, int64_t n_slots,
                          const uint8_t* codes, const float* scale_inv, const TransposeArgs& args,
                          void* stream);
int launch_encode(const float* in, uint8_t* out, int64_t n, void* stream);
const char* hip_error_string(int err);

// Error reporting (abi.cpp): records the message for bfz_last_error().
int fail(int code, const char* fmt, ...);

}  // namespace bfz

struct bfz_plan {
    int32_t n_weights = 0, D = 1, rank = 0;
    int64_t total = 0, quota = 0, owned = 0, first = 0;
    std::vector<int64_t> dims;               // n_weights x {E, H, W}
    std::vector<int64_t> table;              // quota x {weight, e, i, j, rows, cols}
    std::vector<bfz::TileEntry> entries;     // quota rows, segment-relative `local`
    std::vector<bfz::Segment> segments;
    // The transpose's launch order: within each segment, a permutation of
    // its slots (segment-relative) -- workgroup b of the segment's launch
    // takes slot transpose_order[slot0 + b].  Padding slots: identity.
    std::vector<int32_t> transpose_order;
    bfz::TileEntry* d_entries = nullptr;     // device copy of entries, then of transpose_order
    int32_t* d_transpose_order = nullptr;    // inside the same allocation
    int device = -1;
};
