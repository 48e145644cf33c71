// CDNA4 (gfx950) kernels of the shard step: fold, fused AdamW + E4M3
// requantization, unfold.  All three are HBM-streaming kernels -- no
// contraction, so no MFMA -- built around one 128x128 tile per workgroup.
//
// Floating point: every element operation is one IEEE binary32 operation
// in the order the update defines (no contraction into FMA: the file
// pragma and -ffp-contract=off; sqrtf and '/' are the correctly rounded
// HIP defaults), so results do not depend on instruction scheduling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "bfz_internal.h"

#pragma clang fp contract(off)

namespace bfz {
namespace {

constexpr int kThreads = 256;  // transpose / encode: 4 wave64s per workgroup
constexpr int kUnpackThreads = 1024;  // unfold: one 16-byte piece per thread

// ---------------------------------------------------------------------
// E4M3 (OCP E4M3FN) rounding of a binary32 value: nearest value, ties to
// even, saturating at +-448, sign kept.  Pure integer work on the bits.
// Normal range (|y| >= 2^-6): drop 20 mantissa bits with round-half-even
// (the carry may step into the exponent, which is the right answer), then
// re-bias the exponent from 127 to 7.  Below 2^-6 the E4M3 values are the
// multiples of 2^-9, so the code is |y| * 2^9 rounded half-even (exact
// scaling; 8 rounds up into the smallest normal, code 0x08, correctly).
// ---------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t mag = bits & 0x7FFFFFFFu;
    uint32_t code;
    if (mag >= 0x43E00000u) {                 // |y| >= 448 (and Inf): saturate
        code = 0x7Eu;
    } else if (mag >= 0x3C800000u) {          // 2^-6 <= |y| < 448
        const uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);
        code = (r >> 20) - ((127u - 7u) << 3);
    } else {                                  // |y| < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
    }
    return code | sign;
}

// Power-of-two tile scale: the smallest 2^T with 448 * 2^T >= amax (amax
// finite, > 0), T clamped to >= -149 (the smallest binary32 power of two).
// With amax = (1 + f) 2^e and 448 = 1.75 * 2^8: T = e - 8 when 1 + f <= 1.75,
// else e - 7.  Exact integer work on the bits.
__device__ __forceinline__ float pow2_scale(float amax) {
    const uint32_t b = __float_as_uint(amax);
    int e;
    uint32_t mant;
    if (b >= 0x00800000u) {
        e = (int)(b >> 23) - 127;
        mant = b & 0x7FFFFFu;
    } else {  // subnormal amax = b * 2^-149
        const int lead = 31 - __clz(b);
        e = lead - 149;
        mant = (b << (23 - lead)) & 0x7FFFFFu;
    }
    int T = e - 8 + (mant > 0x600000u ? 1 : 0);
    if (T < -149) T = -149;
    return T >= -126 ? __uint_as_float((uint32_t)(T + 127) << 23) : __uint_as_float(1u << (T + 149));
}

// AdamW of one element, the update of the Int8AdamW step (lpnh.cn essay,
// section 4.3): moments, bias-corrected denominator, step, then decay of
// the updated value.
__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v,
                                           const StepScalars& s) {
    const float mm = s.b1 * m + s.c1 * g;
    const float vv = s.b2 * v + s.c2 * (g * g);
    const float den = sqrtf(vv) / s.sbc2 + s.eps;
    float pp = p - s.step_size * (mm / den);
    if (s.has_decay) pp = pp - s.decay * pp;
    m = mm;
    v = vv;
    p = pp;
}

// Non-temporal (streaming) 16-byte accesses: every byte of the step is
// touched exactly once, so keeping it in the caches only evicts the other
// streams.  The builtins take clang vector types.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 load_stream(const f32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }

// A tile's blocks in the shard arrays (master, m, v, a tile-major gradient:
// 64 KiB each; codes: 16 KiB) are accessed through buffer instructions,
// whose cache-policy operand can carry sc1 (device scope) beside nt.  On
// this part each XCD has its own L2, so a device-scope store is written
// through the L2 as it is made instead of staying there dirty until
// evicted; non-temporal loads and nt + sc1 stores measured 1-2.6% faster
// for every step kernel than non-temporal global loads and stores, and the
// fold's nt + sc1 block stores up to 2% faster (the same values land in
// memory).  The descriptor spans exactly the block: an
// offset past it would read zero or be dropped, never touch other memory.
constexpr int kPolicyLoad = 2;        // nt
constexpr int kPolicyStore = 2 | 16;  // nt sc1
constexpr uint32_t kRawBufferFlags = 0x00020000u;  // descriptor word 3 of a raw dword buffer

struct TileBlock {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ TileBlock(const void* base, int bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                              kRawBufferFlags)) {}
    __device__ __forceinline__ f32x4 load(int i) const {  // float4 i of the block
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, kPolicyLoad));
    }
    __device__ __forceinline__ void store(int i, const f32x4& v) const {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, i * 16, 0, kPolicyStore);
    }
    __device__ __forceinline__ void store_word(int i, uint32_t w) const {  // 32-bit word i
        __builtin_amdgcn_raw_buffer_store_b32(w, r, i * 4, 0, kPolicyStore);
    }
};

__device__ __forceinline__ float abs_max4(float a, const f32x4& x) {
    return fmaxf(fmaxf(a, fmaxf(fabsf(x.x), fabsf(x.y))), fmaxf(fabsf(x.z), fabsf(x.w)));
}

__device__ __forceinline__ uint32_t pack_codes(const f32x4& x, float scale) {
    return e4m3_code(x.x / scale) | (e4m3_code(x.y / scale) << 8) |
           (e4m3_code(x.z / scale) << 16) | (e4m3_code(x.w / scale) << 24);
}

// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  The streaming kernels map them to tiles in runs of R consecutive
// tiles per XCD, dealt round-robin: workgroup b = 8 j + x (XCD x) takes tile
// 8 R (j / R) + R x + j % R, and the last n % (8 R) tiles keep their own
// index.  The workgroups in flight then cover one compact window of
// consecutive tiles (dispatch order), while each XCD's L2 sees R
// neighbouring tiles -- whose row-major rows share DRAM pages -- back to
// back.  Bijective for any n_tiles.  R per kernel, measured on MI355X
// against one contiguous eighth of the shard per XCD (the earlier order),
// each A/B in one process on one box:
//   step kernels, R = 4: one-kernel step 2.01B-element shard 9.75 -> 9.58 ms,
//     dense 3.92 -> 3.88, MoE 1.71 -> 1.69, ragged 0.366 -> 0.359 (R = 2
//     within 0.5% of 4; 8 and 16 slower);
//   fold (pack_kernel, whole-tile workgroups at the time), R = 2: dense
//     1.034 -> 1.023 ms, 2.01B 2.527 -> 2.477, ragged unchanged (longer
//     runs up to 2% slower on the large shards); with quarter-tile
//     workgroups the unit is a quarter tile and R = 64 (16 tiles; 8 to
//     32 tiles within 1.5%, 1 and 2 tiles 5-10% slower);
//   unfold (unpack_kernel, 256-thread workgroups at the time), R = 32 (a
//     whole tile row of a 4096-wide weight per XCD): dense 0.280 -> 0.268
//     ms, 2.01B 0.688 -> 0.657, ragged 0.0468 -> 0.0451 (R = 2..16 in
//     between, 64 slightly slower); the 1024-thread form keeps R = 32
//     (8 to 64 within 1%).
// The transpose keeps plain order (below).
template <int64_t R>
__device__ __forceinline__ int64_t run_tile(int64_t b, int64_t n_tiles) {
    const int64_t full = n_tiles / (8 * R) * (8 * R);
    if (b >= full) return b;
    const int64_t x = b % 8, j = b / 8;
    return (j / R) * (8 * R) + x * R + j % R;
}
constexpr int64_t kStepRun = 4, kPackRun = 64, kUnpackRun = 32;
__device__ __forceinline__ int64_t step_tile_of(int64_t b, int64_t n_tiles) {
    return run_tile<kStepRun>(b, n_tiles);
}

// One 1024-thread workgroup (16 wave64s) owns one tile: each thread holds
// 4 float4 of it (float4 i = k * 1024 + thread, k < 4, i.e. rows
// 32 k + thread / 32, columns 4 (thread % 32) .. +3).  The source issues a
// thread's 16 16-byte loads (master, grad, m, v) ahead of the arithmetic
// and leaves their final order to the compiler's scheduler, which
// interleaves part of them with the math (forcing all of them first, or an
// explicit pipeline one to three float4 ahead, measured 1-8% slower).  The
// update runs in registers, then master/m/v go back out, and the new master
// values stay in VGPRs.  The tile amax: lane shuffles within each
// wave, then the 16 wave maxima through LDS (one barrier).  Then the
// register-held values are quantized and stored as one 32-bit word of 4
// codes per float4.  HBM sees each input once and each output once.  The
// launch reserves enough LDS that one tile is in flight per CU, which keeps
// the DRAM access windows compact (measured faster than 2-4 tiles per CU).
constexpr int kStepThreads = 1024;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kStepVec = kTileElems / 4 / kStepThreads;  // float4 per thread per array
constexpr int kStepLdsBytes = 96 * 1024;                 // > half of the 160 KiB per CU

// A gradient source has two phases per float4 k: load(k, spare) issues
// the memory reads, finish(k, raw) turns what they returned into the
// float4.  step_tile places every load of the tile before the first finish
// (the compiler then schedules them), so the lane shuffles of misaligned
// rows do not make the wave wait for all its outstanding reads once per
// float4.  A lane with nothing to read (outside the weight's edge, or a
// padding slot) reads `spare` instead -- a 16-byte block of the same tile
// that the wave reads anyway -- and finish() discards it: lane-divergent
// branches around those loads would make the compiler wait for every
// outstanding read where they join.

// Gradient of a tile already folded into the tile-major shard.
struct TileMajorGrad {
    TileBlock tile;
    typedef f32x4 Raw;
    __device__ __forceinline__ Raw load(int k, const f32x4*) const {
        return tile.load(k * kStepThreads + threadIdx.x);
    }
    __device__ __forceinline__ f32x4 finish(int, const Raw& r) const { return r; }
};

// Gradient read straight from the weight's row-major tensor (the fold done
// on the fly): row 32 k + thread / 32, four columns from 4 (thread % 32).
// Outside the weight's edge, and in padding slots (origin == nullptr), the
// gradient is +0.0 -- exactly what the fold would have stored there.  Two
// sources, chosen per tile (uniform over the workgroup, so neither load
// phase holds a branch): RowMajorGrad for rows on 16-byte boundaries
// (W % 4 == 0, 16-byte aligned weight) and padding slots,
// ShiftedRowMajorGrad for rows that start off a 16-byte boundary.
struct RowMajorGrad {
    const float* origin;  // the tile's element (0, 0) in its weight; nullptr: padding
    int32_t ld;
    int16_t rows, cols;
    typedef f32x4 Raw;
    __device__ __forceinline__ bool lane_ok(int k, int c) const {
        return origin != nullptr && k * 32 + (int)(threadIdx.x >> 5) < rows && c < cols;
    }
    // W % 4 == 0 makes the tile's valid width a multiple of 4: each float4
    // lies wholly inside or wholly outside it
    __device__ __forceinline__ Raw load(int k, const f32x4* spare) const {
        const int r = k * 32 + (threadIdx.x >> 5), c = 4 * (threadIdx.x & 31);
        // formed for every lane; a lane outside the weight (or in a padding
        // slot, origin null) never dereferences it: the select hands it
        // `spare`.  (Forming it inside the select instead changed the whole
        // kernel's schedule and measured 2% slower.)
        const f32x4* q = reinterpret_cast<const f32x4*>(origin + (int64_t)r * ld + c);
        return load_stream(lane_ok(k, c) ? q : spare);
    }
    __device__ __forceinline__ f32x4 finish(int k, const Raw& x) const {
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        return lane_ok(k, 4 * (threadIdx.x & 31)) ? x : zero;
    }
};

// A row that starts a floats past a 16-byte boundary (a = 1..3: odd W or an
// offset weight): lane l loads the aligned block holding row elements
// c - a .. c - a + 3 and takes the a elements it lacks from its right
// neighbour's block (a 32-lane shuffle); the row's last lane also loads the
// block after.  A block is read only if it holds an element of the row's
// valid part; an aligned 16-byte block never crosses a page, so every read
// stays in mapped memory.
struct ShiftedRowMajorGrad {
    const float* origin;
    int32_t ld;
    int16_t rows, cols;
    struct Raw {
        f32x4 f, g;  // the block under the lane, and the one after (last lane)
    };
    __device__ __forceinline__ Raw load(int k, const f32x4* spare) const {
        const int r = k * 32 + (threadIdx.x >> 5), c = 4 * (threadIdx.x & 31);
        const bool row_ok = r < rows;
        const float* row = origin + (int64_t)(row_ok ? r : 0) * ld;
        const int a = (int)((reinterpret_cast<uintptr_t>(row) >> 2) & 3u);
        const f32x4* blk = reinterpret_cast<const f32x4*>(row - a) + (c >> 2);
        const bool last = (threadIdx.x & 31) == 31;
        Raw x;
        x.f = load_stream(row_ok && c - a < cols ? blk : spare);
        // the extra block is the last lane's alone: a masked load (giving
        // every lane the spare read instead measured 3% slower on ragged
        // weights)
        x.g = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (row_ok && last && a > 0 && kTileDim - a < cols) x.g = load_stream(blk + 1);
        return x;
    }
    // Both rows of a wave run the shuffle unconditionally (32-lane segments).
    __device__ __forceinline__ f32x4 finish(int k, const Raw& x) const {
        const int r = k * 32 + (threadIdx.x >> 5), c = 4 * (threadIdx.x & 31);
        const bool row_ok = r < rows;
        const float* row = origin + (int64_t)(row_ok ? r : 0) * ld;
        const int a = (int)((reinterpret_cast<uintptr_t>(row) >> 2) & 3u);
        const bool last = (threadIdx.x & 31) == 31;
        // g's last float is never selected below (a <= 3); keep it live to
        // here, or its register is reused while the load into it is still
        // in flight, which makes the wave wait right after issuing it
        __asm__ volatile("" : : "v"(x.g[3]));
        const f32x4 f = x.f;
        f32x4 n;
#pragma unroll
        for (int l = 0; l < 4; ++l) n[l] = __shfl_down(f[l], 1, 32);
        if (last) n = x.g;
        f32x4 y;
        y[0] = a == 0 ? f[0] : a == 1 ? f[1] : a == 2 ? f[2] : f[3];
        y[1] = a == 0 ? f[1] : a == 1 ? f[2] : a == 2 ? f[3] : n[0];
        y[2] = a == 0 ? f[2] : a == 1 ? f[3] : a == 2 ? n[0] : n[1];
        y[3] = a == 0 ? f[3] : a == 1 ? n[0] : a == 2 ? n[1] : n[2];
#pragma unroll
        for (int l = 0; l < 4; ++l)
            if (!row_ok || c + l >= cols) y[l] = 0.0f;
        return y;
    }
};

// The gradient source of slot entry t in the launch's weights: calls
// f(source) with RowMajorGrad or ShiftedRowMajorGrad (padding slots take
// the former with no origin).
template <class F>
__device__ __forceinline__ void with_row_major_grad(const TileEntry& t, const PackArgs& grads,
                                                    F&& f) {
    if (t.local < 0) {
        f(RowMajorGrad{nullptr, t.ld, t.valid_rows, t.valid_cols});
        return;
    }
    const float* w = grads.src[t.local];
    if (((t.ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(w) & 15u) == 0))
        f(RowMajorGrad{w + t.base, t.ld, t.valid_rows, t.valid_cols});
    else
        f(ShiftedRowMajorGrad{w + t.base, t.ld, t.valid_rows, t.valid_cols});
}

// Where a tile's codes and scale go besides the tile-major shard: straight
// into the row-major FP8 weight and its scale grid (the unfold done in the
// same pass).  origin == nullptr: nowhere else.  Thread t's word of 4 codes
// for float4 k belongs at row 32 k + t / 32, columns 4 (t % 32) .. +3.
struct RowMajorCodes {
    uint8_t* origin;      // the tile's element (0, 0) in the FP8 weight
    float* scale_cell;    // its cell of the scale grid
    int32_t ld;
    int16_t rows, cols;
    bool vec;             // W % 4 == 0 and the weight is 4-byte aligned
    // Rows off a 4-byte boundary store bytes, through the cache: the L2
    // merges them, and building aligned words with a lane shuffle (as the
    // unfold and transpose kernels do) measured 1.5% slower here.
    __device__ __forceinline__ void put(int k, uint32_t word) const {
        const int r = k * 32 + (threadIdx.x >> 5), c = 4 * (threadIdx.x & 31);
        if (origin == nullptr || r >= rows) return;
        uint8_t* q = origin + (int64_t)r * ld + c;
        if (vec && c + 4 <= cols) {
            store_stream(reinterpret_cast<uint32_t*>(q), word);
            return;
        }
#pragma unroll
        for (int l = 0; l < 4; ++l)
            if (c + l < cols) q[l] = (uint8_t)(word >> (8 * l));
    }
};

template <class GradFn, class Out = RowMajorCodes>
__device__ __forceinline__ float step_tile(int64_t tile, float* __restrict__ master,
                                           float* __restrict__ mom1, float* __restrict__ mom2,
                                           uint32_t* __restrict__ codes,
                                           float* __restrict__ scale_inv, const StepScalars& s,
                                           const GradFn& grad_at, float* wave_amax,
                                           const Out& out = Out{}) {
    // master / m / v tiles sit state_stride floats apart (16384: separate
    // arrays; 49152: one [master | m | v] block per tile); codes are tile-major
    const int64_t base = tile * (kTileElems / 4);
    const int64_t sbase = tile * (s.state_stride / 4);
    f32x4* P = reinterpret_cast<f32x4*>(master) + sbase;
    f32x4* M = reinterpret_cast<f32x4*>(mom1) + sbase;
    f32x4* V = reinterpret_cast<f32x4*>(mom2) + sbase;
    const TileBlock bP(P, kTileElems * 4), bM(M, kTileElems * 4), bV(V, kTileElems * 4);

    f32x4 p[kStepVec], g[kStepVec], m[kStepVec], v[kStepVec];
    typename GradFn::Raw graw[kStepVec];
#pragma unroll
    for (int k = 0; k < kStepVec; ++k) {
        const int i = k * kStepThreads + threadIdx.x;
        p[k] = bP.load(i);
        graw[k] = grad_at.load(k, P + i);
        m[k] = bM.load(i);
        v[k] = bV.load(i);
    }
#pragma unroll
    for (int k = 0; k < kStepVec; ++k) g[k] = grad_at.finish(k, graw[k]);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < kStepVec; ++k) {
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            float pl = p[k][l], ml = m[k][l], vl = v[k][l];
            adamw_elem(pl, g[k][l], ml, vl, s);
            p[k][l] = pl;
            m[k][l] = ml;
            v[k][l] = vl;
        }
        amax = abs_max4(amax, p[k]);
    }
    // master, then m, then v: in the interleaved layout the workgroup writes
    // its [master | m | v] block front to back (measured 0.6-2.8% faster
    // than storing each float4's three values as it is done, and than the
    // order m, v, master)
#pragma unroll
    for (int k = 0; k < kStepVec; ++k) bP.store(k * kStepThreads + threadIdx.x, p[k]);
#pragma unroll
    for (int k = 0; k < kStepVec; ++k) bM.store(k * kStepThreads + threadIdx.x, m[k]);
#pragma unroll
    for (int k = 0; k < kStepVec; ++k) bV.store(k * kStepThreads + threadIdx.x, v[k]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = wave_amax[0];
#pragma unroll
    for (int w = 1; w < kStepWaves; ++w) amax = fmaxf(amax, wave_amax[w]);

    // scale_inv = amax / 448 (or its power-of-two form); an all-zero tile
    // takes 1 and codes 0.  A nonzero amax of at most 224 * 2^-149 rounds
    // amax / 448 to zero: such a tile takes 2^-149, the smallest positive
    // binary32, so no code comes from a division by zero.
    const bool zero = amax == 0.0f;
    const float plain = amax / 448.0f;
    const float scale = zero ? 1.0f
                             : (s.pow2 ? pow2_scale(amax) : (plain == 0.0f ? 0x1p-149f : plain));
    if (threadIdx.x == 0) {
        if (scale_inv) scale_inv[tile] = scale;
        if (out.scale_cell) *out.scale_cell = scale;
    }
    const TileBlock C(codes ? codes + base : nullptr, kTileElems);
#pragma unroll
    for (int k = 0; k < kStepVec; ++k) {
        const uint32_t word = zero ? 0u : pack_codes(p[k], scale);
        if (codes) C.store_word(k * kStepThreads + threadIdx.x, word);
        out.put(k, word);
    }
    return scale;
}

__global__ __launch_bounds__(kStepThreads) void step_kernel(
    float* __restrict__ master, const float* __restrict__ grad, float* __restrict__ mom1,
    float* __restrict__ mom2, uint32_t* __restrict__ codes, float* __restrict__ scale_inv,
    StepScalars s, int64_t n_tiles) {
    extern __shared__ float wave_amax[];
    const int64_t tile = step_tile_of(blockIdx.x, n_tiles);
    const TileMajorGrad g{TileBlock(grad + tile * kTileElems, kTileElems * 4)};
    step_tile(tile, master, mom1, mom2, codes, scale_inv, s, g, wave_amax);
}

// The same step, with the gradient fold fused in: slot s of this launch
// reads its gradient from the row-major weight its table entry names.
// master/m/v/codes/scale_inv and entries point at the launch's first slot.
__global__ __launch_bounds__(kStepThreads) void fold_step_kernel(
    const TileEntry* __restrict__ entries, PackArgs grads, float* __restrict__ master,
    float* __restrict__ mom1, float* __restrict__ mom2, uint32_t* __restrict__ codes,
    float* __restrict__ scale_inv, StepScalars s, int64_t n_slots) {
    extern __shared__ float wave_amax[];
    const int64_t slot = step_tile_of(blockIdx.x, n_slots);
    const TileEntry t = entries[slot];
    with_row_major_grad(t, grads, [&](const auto& g) {
        step_tile(slot, master, mom1, mom2, codes, scale_inv, s, g, wave_amax);
    });
}

// Fold, step and unfold in one pass: as fold_step_kernel, and each owned
// tile's codes and scale also land in the row-major FP8 weight and scale
// grid its entry names.  codes / scale_inv may be null (row-major only).
__global__ __launch_bounds__(kStepThreads) void fold_step_unfold_kernel(
    const TileEntry* __restrict__ entries, PackArgs grads, UnpackArgs outs,
    float* __restrict__ master, float* __restrict__ mom1, float* __restrict__ mom2,
    uint32_t* __restrict__ codes, float* __restrict__ scale_inv, StepScalars s, int64_t n_slots) {
    extern __shared__ float wave_amax[];
    const int64_t slot = step_tile_of(blockIdx.x, n_slots);
    const TileEntry t = entries[slot];
    RowMajorCodes out{nullptr, nullptr, t.ld, t.valid_rows, t.valid_cols, false};
    if (t.local >= 0) {
        uint8_t* d = outs.codes[t.local];
        out.origin = d + t.base;
        out.scale_cell = outs.scale[t.local] + t.scale_index;
        out.vec = ((t.ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(d) & 3u) == 0);
    }
    with_row_major_grad(t, grads, [&](const auto& g) {
        step_tile(slot, master, mom1, mom2, codes, scale_inv, s, g, wave_amax, out);
    });
}

// Fold: one 1024-thread workgroup per quarter slot.  Unit u covers float4
// group k = u % 4 of slot u / 4 in the step kernels' thread layout: thread t
// moves float4 column t % 32 of row 32 k + t / 32, so a wave covers two
// 512-byte tile rows per instruction on both sides.  Units run in runs of
// 64 (16 tiles) per XCD.  Whole-tile workgroups (four float4 per thread, all
// loaded before the stores) hold four times the bytes in flight per
// workgroup and measured 3-7% slower: dense shard 1.023 -> 0.992 ms,
// 2.01B-element shard 2.485 -> 2.397, MoE 0.448 -> 0.420, ragged 0.099 ->
// 0.094 (one process, five repeats; half-tile units in between).
// Streaming loads, and the block's stores at device scope as in the step
// kernels.  Outside the weight's edge, and in padding slots, the tile gets
// +0.0.  Slot s is written at dst + s * dst_stride.
__global__ __launch_bounds__(kStepThreads) void pack_kernel(const TileEntry* __restrict__ entries,
                                                            float* __restrict__ dst, int64_t dst_stride,
                                                            PackArgs args) {
    const int64_t u = run_tile<kPackRun>(blockIdx.x, gridDim.x);
    const int64_t slot = u / kStepVec;
    const int k = (int)(u % kStepVec);
    const TileEntry t = entries[slot];
    f32x4* out = reinterpret_cast<f32x4*>(dst + slot * dst_stride);
    const TileBlock block(out, kTileElems * 4);
    const int i = k * kStepThreads + threadIdx.x;
    // a lane with nothing to read loads its own (not yet written) output float4
    with_row_major_grad(t, args, [&](const auto& src) {
        const auto raw = src.load(k, out + i);
        block.store(i, src.finish(k, raw));
    });
}

// Unfold of codes and scales: one 1024-thread workgroup per owned slot, in
// runs of 32 tiles per XCD (run_tile; plain order measured 5.6% slower on
// the dense shard than one contiguous eighth per XCD, itself 4% slower than
// this).  Thread t moves one 16-byte piece: the 16 codes of column block
// t % 8 in row t / 8.  (A 256-thread workgroup moving four pieces per
// thread, all loaded before the first store, holds more bytes in flight per
// CU and measured 4-7% slower on full tiles of 4096- and 11008-wide
// weights; so did two or four tiles per workgroup.)  A row of a full-width
// tile goes out as one 16-byte store per lane when it starts on a
// 16-byte boundary, as 4-byte words when on a 4-byte boundary, and otherwise
// as aligned words built from the lane's codes and its left neighbour's last
// word (a shuffle within the row's 8 lanes), with bytes only for the row's
// two partial end words.  The word stores are ordinary cached stores: such a
// row shares its end cache lines with the neighbouring tiles, and the L2
// merges the halves (streaming stores of partial lines measured about 1.6x
// slower).  Ragged-width tiles use the widest store each lane's piece allows.
__global__ __launch_bounds__(kUnpackThreads) void unpack_kernel(
    const TileEntry* __restrict__ entries, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale_inv, UnpackArgs args) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t slot = run_tile<kUnpackRun>(blockIdx.x, gridDim.x);
    const TileEntry t = entries[slot];
    if (t.local < 0) return;
    const u32x4* in = reinterpret_cast<const u32x4*>(codes + slot * kTileElems);
    uint8_t* dst = args.codes[t.local] + t.base;
    const int c16 = threadIdx.x & 7;
    const int r = threadIdx.x >> 3;
    const int col = 16 * c16;
    const bool full = t.valid_cols == kTileDim;
    // the tile always holds 128 rows (padding included), so the load is in bounds
    const u32x4 x = __builtin_nontemporal_load(in + r * 8 + c16);
    if (r < t.valid_rows) {  // the same for the 8 lanes of a row
        const uint32_t o[4] = {x[0], x[1], x[2], x[3]};
        uint8_t* row = dst + (int64_t)r * t.ld + col;
        const uintptr_t seg = reinterpret_cast<uintptr_t>(row) - (uintptr_t)col;
        const int b = (int)(seg & 3u);
        const uint32_t prev = (uint32_t)__shfl_up((int)o[3], 1, 8);
        const uintptr_t at = reinterpret_cast<uintptr_t>(row);
        if (full && (seg & 15u) == 0) {
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(row));
        } else if (full && b == 0) {
            uint32_t* rw = reinterpret_cast<uint32_t*>(row);
#pragma unroll
            for (int q = 0; q < 4; ++q) rw[q] = o[q];
        } else if (full) {
            // word q holds row bytes col - b + 4q .. +3
            uint32_t* rw = reinterpret_cast<uint32_t*>(row - b);
            uint32_t wv[4];
            wv[0] = __builtin_amdgcn_alignbyte(o[0], prev, (uint32_t)(4 - b));
#pragma unroll
            for (int q = 1; q < 4; ++q) wv[q] = __builtin_amdgcn_alignbyte(o[q], o[q - 1], (uint32_t)(4 - b));
            if (c16 == 0) {
                for (int l = b; l < 4; ++l) row[l - b] = (uint8_t)(wv[0] >> (8 * l));
            } else {
                rw[0] = wv[0];
            }
#pragma unroll
            for (int q = 1; q < 4; ++q) rw[q] = wv[q];
            if (c16 == 7)
                for (int l = 0; l < b; ++l) row[16 - b + l] = (uint8_t)(o[3] >> (8 * (4 - b + l)));
        } else if (col + 16 <= t.valid_cols && (at & 15u) == 0) {
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(row));
        } else if (col + 16 <= t.valid_cols && (at & 3u) == 0) {
            uint32_t* rw = reinterpret_cast<uint32_t*>(row);
#pragma unroll
            for (int q = 0; q < 4; ++q) rw[q] = o[q];
        } else {
            for (int l = 0; l < 16 && col + l < t.valid_cols; ++l) row[l] = (uint8_t)(o[l >> 2] >> (8 * (l & 3)));
        }
    }
    if (threadIdx.x == 0) args.scale[t.local][t.scale_index] = scale_inv[slot];
}

// ---------------------------------------------------------------------
// Scaling-aware transpose of power-of-two-quantized tiles: exponent edits.
// ---------------------------------------------------------------------

// Doublings the E4M3 magnitude code `mag` (1..126) can take and stay within
// 448: a normal code (E, M) has 15 - E of them (14 - E when M = 7, since
// 1.875 * 2 > 1.75); subnormals M * 2^-9 have 17 (M = 1), 16 (M = 2, 3) or
// 15 (M = 4..7).
__device__ __forceinline__ int e4m3_headroom(uint32_t mag) {
    if (mag >= 8u) return ((mag & 7u) == 7u ? 14 : 15) - (int)(mag >> 3);
    return mag == 1u ? 17 : (mag < 4u ? 16 : 15);
}

// The code of the same value on a scale 2^d times finer: d doublings.  A
// subnormal doubles by shifting its 3-bit significand left until it turns
// normal (code 8 = 2^-6 is exactly 4 * 2^-9 doubled); a normal doubles by
// adding 1 to its exponent field (+8).  Exact while within 448, which the
// caller's headroom guarantees.
__device__ __forceinline__ uint32_t e4m3_scale_up(uint32_t code, int d) {
    const uint32_t sign = code & 0x80u;
    uint32_t mag = code & 0x7Fu;
    if (mag == 0u) return code;
    if (mag < 8u) {
        const int sh = min(d, 4 - (32 - __clz(mag)));
        mag <<= sh;
        d -= sh;
    }
    return sign | (mag + ((uint32_t)d << 3));
}

// binary32 exponent of a power of two (normal or subnormal).
__device__ __forceinline__ int pow2_exponent(float s) {
    const uint32_t b = __float_as_uint(s);
    return b >= 0x00800000u ? (int)(b >> 23) - 127 : (31 - __clz(b)) - 149;
}

__device__ __forceinline__ float pow2_value(int T) {
    return T >= -126 ? __uint_as_float((uint32_t)(T + 127) << 23) : __uint_as_float(1u << (T + 149));
}

// Largest of the 16 bytes of four words whose bytes are below 0x80 (E4M3
// magnitudes with the sign masked off).
__device__ __forceinline__ uint32_t byte_max16(const uint32_t a[4]) {
    uint32_t m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        m[q] = max(max(a[q] & 0xFFu, (a[q] >> 8) & 0xFFu), max((a[q] >> 16) & 0xFFu, a[q] >> 24));
    return max(max(m[0], m[1]), max(m[2], m[3]));
}

// The 8-entry byte table c -> e4m3_scale_up(c, d) for the subnormal codes
// c = 0..7, d = 0..17, as two words (entries 0-3 in lo, 4-7 in hi).  A code
// c takes s = 4 - bitlength(c) doublings as a left shift (3 for c = 1, 2 for
// c = 2, 3, 1 for c = 4..7) and the rest as +8 each; no entry exceeds 142,
// so the per-byte sums never carry.
__device__ __forceinline__ void subnormal_table(int d, uint32_t& lo, uint32_t& hi) {
    hi = d >= 1 ? 0x0E0C0A08u + (uint32_t)(d - 1) * 0x08080808u : 0x07060504u;
    lo = d >= 2 ? 0x0C080000u + (uint32_t)(d - 2) * 0x08080800u : (d == 1 ? 0x06040200u : 0x03020100u);
    if (d == 2) lo |= 0x0400u;  // c = 1 is still subnormal after two doublings
}

// One lane's part of W^T row c of a tile: the lane holds bytes 16 k2 .. +15
// of the row (tile rows 16 k2 .. +15 of column c) in v, 8 lanes per row.
// The group's largest magnitude code (valid rows only; an 8-lane shuffle
// reduction) gives the headroom d (clamped so 2^(T - d) >= 2^-149), lane 0
// writes the group scale, and every code is moved up d binades.  A normal
// code moves by adding 8d to its byte -- one add per 32-bit word, which
// cannot carry out of a byte since the headroom keeps every code <= 126;
// subnormal codes (rare: magnitudes under 2^-6 of the scale) are looked up,
// four bytes at a time, in a byte table indexed by their 3-bit value; a
// lane on a ragged edge goes byte by byte.  All 8 lanes of the row must
// call it (shuffles).  An all-zero group: scale 1, codes 0.
__device__ __forceinline__ void wt_row(const uint32_t v[4], int c, int k2, int T, const TileEntry& t,
                                       uint8_t* wt, float* wt_scale, int64_t H, int64_t W,
                                       int64_t hb, int64_t e, int64_t i, int64_t j) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int r0 = 16 * k2;
    const int nvalid = max(0, min(16, (int)t.valid_rows - r0));
    uint32_t a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = v[q] & 0x7F7F7F7Fu;
    uint32_t mx = 0;
    if (nvalid == 16) {
        mx = byte_max16(a);
    } else {
        for (int l = 0; l < nvalid; ++l) mx = max(mx, (v[l >> 2] >> (8 * (l & 3))) & 0x7Fu);
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 4, 64));
    if (c >= t.valid_cols) return;
    int d = mx == 0u ? 0 : e4m3_headroom(mx);
    if (T - d < -149) d = T + 149;
    const int64_t out_row = e * W + kTileDim * j + c;
    if (k2 == 0) wt_scale[out_row * hb + i] = mx == 0u ? 1.0f : pow2_value(T - d);
    if (nvalid == 0) return;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (mx != 0u && nvalid == 16) {
        // per byte: bit 7 of nf set for a normal code (exponent field != 0),
        // bit 7 of sub for a nonzero code that is not normal
        uint32_t nf[4], sub[4];
        const uint32_t inc = (uint32_t)d << 3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            nf[q] = ((a[q] & 0x78787878u) + 0x78787878u) & 0x80808080u;
            sub[q] = ((a[q] + 0x7F7F7F7Fu) & 0x80808080u) & ~nf[q];
            o[q] = v[q] + (nf[q] >> 7) * inc;
        }
        if ((sub[0] | sub[1] | sub[2] | sub[3]) != 0u) {
            uint32_t lo, hi;
            subnormal_table(d, lo, hi);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t looked = __builtin_amdgcn_perm(hi, lo, v[q] & 0x07070707u) | (v[q] & 0x80808080u);
                const uint32_t bytes = sub[q] | (sub[q] - (sub[q] >> 7));  // 0xFF where sub
                o[q] = (looked & bytes) | (o[q] & ~bytes);
            }
        }
    } else if (mx != 0u) {
        for (int l = 0; l < nvalid; ++l)
            o[l >> 2] |= e4m3_scale_up((v[l >> 2] >> (8 * (l & 3))) & 0xFFu, d) << (8 * (l & 3));
    }
    uint8_t* q = wt + out_row * H + kTileDim * i + r0;
    // The row's 128-byte segment starts b bytes past a 4-byte boundary
    // (odd H).  A full-height tile then stores aligned words built from
    // this lane's codes and the last word of its left neighbour in the
    // row (a shuffle within the 8 lanes); only the segment's first and
    // last partial words go byte by byte.  Off a 16-byte boundary the
    // stores are cached, so the L2 can merge the segment's end lines
    // with the neighbouring tiles' pieces.  Ragged tiles store bytes.
    const uintptr_t seg = reinterpret_cast<uintptr_t>(q) - (uintptr_t)r0;
    const int b = (int)(seg & 3u);
    const uint32_t prev = (uint32_t)__shfl_up((int)o[3], 1, 8);
    if (t.valid_rows == kTileDim && (seg & 15u) == 0) {
        const u32x4 y = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(q));
    } else if (t.valid_rows == kTileDim && b == 0) {
        uint32_t* qw = reinterpret_cast<uint32_t*>(q);
#pragma unroll
        for (int k = 0; k < 4; ++k) qw[k] = o[k];
    } else if (t.valid_rows == kTileDim) {
        // word k holds segment bytes r0 - b + 4k .. +3
        uint32_t* qw = reinterpret_cast<uint32_t*>(q - b);
        uint32_t wv[4];
        wv[0] = __builtin_amdgcn_alignbyte(o[0], prev, (uint32_t)(4 - b));
#pragma unroll
        for (int k = 1; k < 4; ++k) wv[k] = __builtin_amdgcn_alignbyte(o[k], o[k - 1], (uint32_t)(4 - b));
        if (k2 == 0) {
            for (int l = b; l < 4; ++l) q[l - b] = (uint8_t)(wv[0] >> (8 * l));
        } else {
            qw[0] = wv[0];
        }
#pragma unroll
        for (int k = 1; k < 4; ++k) qw[k] = wv[k];
        if (k2 == 7)
            for (int l = 0; l < b; ++l) q[16 - b + l] = (uint8_t)(o[3] >> (8 * (4 - b + l)));
    } else {
        for (int l = 0; l < nvalid; ++l) q[l] = (uint8_t)(o[l >> 2] >> (8 * (l & 3)));
    }
}

// wt_row for a full tile whose W^T row segments all start on a 16-byte
// boundary (W^T rows of a multiple of 16 bytes, 16-byte aligned weight;
// decided once per tile): no ragged edge, no alignment cases, no
// neighbour's word; the row's address comes in from the caller.  The same
// group scale and exponent edit as wt_row, byte for byte (measured 0.6-1.1%
// faster than wt_row on the dense, 2.01B-element and MoE shards).
__device__ __forceinline__ void wt_row_full(const uint32_t v[4], int k2, int T, uint8_t* seg,
                                            float* scale_cell) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    uint32_t a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = v[q] & 0x7F7F7F7Fu;
    uint32_t mx = byte_max16(a);
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 4, 64));
    int d = mx == 0u ? 0 : e4m3_headroom(mx);
    if (T - d < -149) d = T + 149;
    if (k2 == 0) *scale_cell = mx == 0u ? 1.0f : pow2_value(T - d);
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (mx != 0u) {
        uint32_t nf[4], sub[4];
        const uint32_t inc = (uint32_t)d << 3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            nf[q] = ((a[q] & 0x78787878u) + 0x78787878u) & 0x80808080u;
            sub[q] = ((a[q] + 0x7F7F7F7Fu) & 0x80808080u) & ~nf[q];
            o[q] = v[q] + (nf[q] >> 7) * inc;
        }
        if ((sub[0] | sub[1] | sub[2] | sub[3]) != 0u) {
            uint32_t lo, hi;
            subnormal_table(d, lo, hi);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t looked = __builtin_amdgcn_perm(hi, lo, v[q] & 0x07070707u) | (v[q] & 0x80808080u);
                const uint32_t bytes = sub[q] | (sub[q] - (sub[q] >> 7));
                o[q] = (looked & bytes) | (o[q] & ~bytes);
            }
        }
    }
    const u32x4 y = {o[0], o[1], o[2], o[3]};
    __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(seg + 16 * k2));
}

// One 256-thread workgroup per owned slot.
//  1. Thread t reads rows 4(t / 8) .. +3, bytes 16(t % 8) .. +15 of the tile
//     (four 16-byte loads), transposes each 4x4-byte block with byte
//     permutes and writes the 16 resulting words to LDS as words of W^T
//     rows: W^T row c (= tile column c) holds bytes r = 0..127 (= tile rows)
//     in 32 words.  Word w of row c sits at c * 32 + ((w + 4 (c / 16)) % 32):
//     the rotation keeps each aligned group of four words together and puts
//     exactly two lanes of a wave on every bank in step 1.
//  2. Eight consecutive lanes own one W^T row, 16 bytes (one aligned 16-byte
//     LDS read) each, so a wave stores eight contiguous 128-byte row
//     segments (wt_row: group scale, exponent edit, store).
__global__ __launch_bounds__(kThreads) void transpose_pow2_kernel(
    const TileEntry* __restrict__ entries, const int32_t* __restrict__ order,
    const uint8_t* __restrict__ codes, const float* __restrict__ scale_inv, TransposeArgs args) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ uint32_t tile_t[kTileDim * 32];
    // The plan's transpose order: tile columns dealt to XCDs (see the
    // planner).  Plain order was 1.5-7% faster than one contiguous eighth
    // of the shard per XCD and 1-7% faster than runs of 2 to 8 consecutive
    // tiles per XCD (run_tile) on the dense and 2.01B-element shards; the
    // column dealing is faster still where tile rows do not hold a multiple
    // of 8 tiles.
    const int64_t slot = order[blockIdx.x];
    const TileEntry t = entries[slot];
    if (t.local < 0) return;
    {
        const u32x4* in = reinterpret_cast<const u32x4*>(codes + slot * kTileElems);
        const int cx = threadIdx.x & 7, rq = threadIdx.x >> 3;
        u32x4 w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = __builtin_nontemporal_load(in + (4 * rq + k) * 8 + cx);
        const int rot = (rq + 4 * cx) & 31;
#pragma unroll
        for (int wq = 0; wq < 4; ++wq) {
            // rows 0, 1 (and 2, 3) interleaved byte by byte, then the columns
            const uint32_t x01lo = __builtin_amdgcn_perm(w[1][wq], w[0][wq], 0x05010400u);
            const uint32_t x01hi = __builtin_amdgcn_perm(w[1][wq], w[0][wq], 0x07030602u);
            const uint32_t x23lo = __builtin_amdgcn_perm(w[3][wq], w[2][wq], 0x05010400u);
            const uint32_t x23hi = __builtin_amdgcn_perm(w[3][wq], w[2][wq], 0x07030602u);
            const uint32_t col[4] = {__builtin_amdgcn_perm(x23lo, x01lo, 0x05040100u),
                                     __builtin_amdgcn_perm(x23lo, x01lo, 0x07060302u),
                                     __builtin_amdgcn_perm(x23hi, x01hi, 0x05040100u),
                                     __builtin_amdgcn_perm(x23hi, x01hi, 0x07060302u)};
#pragma unroll
            for (int l = 0; l < 4; ++l) tile_t[(16 * cx + 4 * wq + l) * 32 + rot] = col[l];
        }
    }
    __syncthreads();

    const int T = pow2_exponent(scale_inv[slot]);
    const int64_t H = args.rows[t.local], W = t.ld;
    const int64_t hb = (H + kTileDim - 1) / kTileDim, wb = (W + kTileDim - 1) / kTileDim;
    const int64_t j = t.scale_index % wb, ei = t.scale_index / wb;
    const int64_t i = ei % hb, e = ei / hb;
    const int k2 = threadIdx.x & 7;        // 16-byte chunk of the row: rows 16 k2 .. +15
    uint8_t* wt = args.codes[t.local];
    if (t.valid_rows == kTileDim && t.valid_cols == kTileDim && (H & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(wt) & 15u) == 0) {
        uint8_t* base = wt + (e * W + kTileDim * j) * H + kTileDim * i;
        float* sbase = args.scale[t.local] + (e * W + kTileDim * j) * hb + i;
#pragma unroll
        for (int mr = 0; mr < 4; ++mr) {
            const int c = (threadIdx.x >> 3) + 32 * mr;  // W^T row within the tile
            const u32x4 vv = *reinterpret_cast<const u32x4*>(&tile_t[c * 32 + ((4 * k2 + 4 * (c >> 4)) & 31)]);
            const uint32_t v[4] = {vv[0], vv[1], vv[2], vv[3]};
            wt_row_full(v, k2, T, base + (int64_t)c * H, sbase + (int64_t)c * hb);
        }
        return;
    }
#pragma unroll
    for (int mr = 0; mr < 4; ++mr) {
        const int c = (threadIdx.x >> 3) + 32 * mr;  // W^T row within the tile
        const u32x4 vv = *reinterpret_cast<const u32x4*>(&tile_t[c * 32 + ((4 * k2 + 4 * (c >> 4)) & 31)]);
        const uint32_t v[4] = {vv[0], vv[1], vv[2], vv[3]};
        wt_row(v, c, k2, T, t, wt, args.scale[t.local], H, W, hb, e, i, j);
    }
}

// Sink of the step's code words for the fused transposed copy: each word
// goes to the row-major FP8 weight (as RowMajorCodes) and into an LDS copy
// of the tile's codes, row r word w (columns 4w .. 4w + 3) at
// r * 32 + ((w + r / 4) % 32); that rotation puts two lanes of a wave on
// each bank both here and in the 4x4-block reads that follow.
struct StagedCodes {
    RowMajorCodes rm;
    float* scale_cell;   // the row-major scale-grid cell (step_tile writes it)
    uint32_t* tile_rm;   // LDS, 4096 words
    __device__ __forceinline__ void put(int k, uint32_t word) const {
        rm.put(k, word);
        const int r = k * 32 + (threadIdx.x >> 5), w = threadIdx.x & 31;
        tile_rm[r * 32 + ((w + (r >> 2)) & 31)] = word;
    }
};

// Fold, power-of-two step, unfold and the transposed copy in one pass: as
// fold_step_unfold_kernel, and each owned tile's codes also leave as W^T
// (row-major [E, W, H]) with one power-of-two scale per 128-element group
// of a W^T row, by exponent edits of the codes the step just produced --
// the scaling-aware transpose without reading the codes back.
//  1. the step (step_tile); its code words also go to LDS (StagedCodes);
//  2. thread t transposes the 4x4-byte block of tile rows 4 (t % 32) .. +3,
//     column word t / 32, into W^T-row words laid out as in
//     transpose_pow2_kernel (two lanes per bank on both sides);
//  3. 8 lanes per W^T row, the 1024 threads covering the tile's 128 columns
//     at once: wt_row.
__global__ __launch_bounds__(kStepThreads) void fold_step_unfold_t_kernel(
    const TileEntry* __restrict__ entries, PackArgs grads, UnpackArgs outs, TransposeArgs touts,
    float* __restrict__ master, float* __restrict__ mom1, float* __restrict__ mom2,
    uint32_t* __restrict__ codes, float* __restrict__ scale_inv, StepScalars s, int64_t n_slots) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    extern __shared__ float smem[];
    float* wave_amax = smem;                                       // kStepWaves floats
    uint32_t* tile_rm = reinterpret_cast<uint32_t*>(smem + 64);    // 16 KiB, codes by rows
    uint32_t* tile_t = tile_rm + kTileElems / 4;                   // 16 KiB, codes by W^T rows
    const int64_t slot = step_tile_of(blockIdx.x, n_slots);
    const TileEntry t = entries[slot];
    StagedCodes out{RowMajorCodes{nullptr, nullptr, t.ld, t.valid_rows, t.valid_cols, false}, nullptr,
                    tile_rm};
    if (t.local >= 0) {
        uint8_t* d = outs.codes[t.local];
        out.rm.origin = d + t.base;
        out.rm.vec = ((t.ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(d) & 3u) == 0);
        out.scale_cell = outs.scale[t.local] + t.scale_index;
    }
    float scale = 0.0f;
    with_row_major_grad(t, grads, [&](const auto& g) {
        scale = step_tile(slot, master, mom1, mom2, codes, scale_inv, s, g, wave_amax, out);
    });
    __syncthreads();
    {
        const int rq = threadIdx.x & 31, bc = threadIdx.x >> 5;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = tile_rm[(4 * rq + j) * 32 + ((bc + rq) & 31)];
        const uint32_t x01lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
        const uint32_t x01hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
        const uint32_t x23lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
        const uint32_t x23hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
        const uint32_t col[4] = {__builtin_amdgcn_perm(x23lo, x01lo, 0x05040100u),
                                 __builtin_amdgcn_perm(x23lo, x01lo, 0x07060302u),
                                 __builtin_amdgcn_perm(x23hi, x01hi, 0x05040100u),
                                 __builtin_amdgcn_perm(x23hi, x01hi, 0x07060302u)};
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int c = 4 * bc + l;
            tile_t[c * 32 + ((rq + 4 * (c >> 4)) & 31)] = col[l];
        }
    }
    __syncthreads();
    if (t.local < 0) return;
    const int T = pow2_exponent(scale);
    const int64_t H = touts.rows[t.local], W = t.ld;
    const int64_t hb = (H + kTileDim - 1) / kTileDim, wb = (W + kTileDim - 1) / kTileDim;
    const int64_t j = t.scale_index % wb, ei = t.scale_index / wb;
    const int64_t i = ei % hb, e = ei / hb;
    const int c = threadIdx.x >> 3, k2 = threadIdx.x & 7;
    const u32x4 vv = *reinterpret_cast<const u32x4*>(&tile_t[c * 32 + ((4 * k2 + 4 * (c >> 4)) & 31)]);
    const uint32_t v[4] = {vv[0], vv[1], vv[2], vv[3]};
    wt_row(v, c, k2, T, t, touts.codes[t.local], touts.scale[t.local], H, W, hb, e, i, j);
}

__global__ __launch_bounds__(kThreads) void encode_kernel(const float* __restrict__ in,
                                                          uint8_t* __restrict__ out, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        out[i] = (uint8_t)e4m3_code(in[i]);
}

}  // namespace

namespace {

// The dynamic-LDS limit is a per-device function attribute: set it once per
// kernel on each device the step runs on (devices 0-63 remember it in a bit
// mask; a device past 63 sets it on every launch, which is harmless).
hipError_t reserve_lds(const void* kernel, std::atomic<uint64_t>& ready) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
    if (!bit || !(ready.load(std::memory_order_acquire) & bit)) {
        err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kStepLdsBytes);
        if (err != hipSuccess) return err;
        ready.fetch_or(bit, std::memory_order_release);
    }
    return hipSuccess;
}

std::atomic<uint64_t> g_step_lds{0}, g_fold_step_lds{0}, g_fold_step_unfold_lds{0},
    g_fold_step_unfold_t_lds{0};

}  // namespace

int launch_step(float* master, const float* grad, float* m, float* v, uint8_t* codes,
                float* scale_inv, int64_t n_tiles, const StepScalars& s, void* stream) {
    if (n_tiles == 0) return hipSuccess;
    hipError_t err = reserve_lds(reinterpret_cast<const void*>(step_kernel), g_step_lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(step_kernel, dim3((uint32_t)n_tiles), dim3(kStepThreads), kStepLdsBytes,
                       (hipStream_t)stream, master, grad, m, v,
                       reinterpret_cast<uint32_t*>(codes), scale_inv, s, n_tiles);
    return hipGetLastError();
}

int launch_fold_step(const TileEntry* d_entries, int64_t n_slots, const PackArgs& grads,
                     float* master, float* m, float* v, uint8_t* codes, float* scale_inv,
                     const StepScalars& s, void* stream) {
    if (n_slots == 0) return hipSuccess;
    hipError_t err = reserve_lds(reinterpret_cast<const void*>(fold_step_kernel), g_fold_step_lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(fold_step_kernel, dim3((uint32_t)n_slots), dim3(kStepThreads),
                       kStepLdsBytes, (hipStream_t)stream, d_entries, grads, master, m, v,
                       reinterpret_cast<uint32_t*>(codes), scale_inv, s, n_slots);
    return hipGetLastError();
}

int launch_fold_step_unfold(const TileEntry* d_entries, int64_t n_slots, const PackArgs& grads,
                            const UnpackArgs& outs, float* master, float* m, float* v,
                            uint8_t* codes, float* scale_inv, const StepScalars& s, void* stream) {
    if (n_slots == 0) return hipSuccess;
    hipError_t err = reserve_lds(reinterpret_cast<const void*>(fold_step_unfold_kernel),
                                 g_fold_step_unfold_lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(fold_step_unfold_kernel, dim3((uint32_t)n_slots), dim3(kStepThreads),
                       kStepLdsBytes, (hipStream_t)stream, d_entries, grads, outs, master, m, v,
                       reinterpret_cast<uint32_t*>(codes), scale_inv, s, n_slots);
    return hipGetLastError();
}

int launch_pack(const TileEntry* d_entries, int64_t n_slots, float* dst, int64_t dst_stride,
                const PackArgs& args, void* stream) {
    // four 1024-thread workgroups per slot, and a launch counts its
    // work-items in 32 bits: at most 2^20 - 1 slots a launch
    constexpr int64_t kMaxSlots = (int64_t(1) << 32) / (kStepVec * kStepThreads) - 1;
    for (int64_t s0 = 0; s0 < n_slots; s0 += kMaxSlots) {
        const int64_t n = std::min(kMaxSlots, n_slots - s0);
        hipLaunchKernelGGL(pack_kernel, dim3((uint32_t)(kStepVec * n)), dim3(kStepThreads), 0,
                           (hipStream_t)stream, d_entries + s0, dst + s0 * dst_stride, dst_stride,
                           args);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

int launch_unpack(const TileEntry* d_entries, int64_t n_slots, const uint8_t* codes,
                  const float* scale_inv, const UnpackArgs& args, void* stream) {
    if (n_slots == 0) return hipSuccess;
    hipLaunchKernelGGL(unpack_kernel, dim3((uint32_t)n_slots), dim3(kUnpackThreads), 0,
                       (hipStream_t)stream, d_entries, codes, scale_inv, args);
    return hipGetLastError();
}

int launch_fold_step_unfold_t(const TileEntry* d_entries, int64_t n_slots, const PackArgs& grads,
                              const UnpackArgs& outs, const TransposeArgs& touts, float* master,
                              float* m, float* v, uint8_t* codes, float* scale_inv,
                              const StepScalars& s, void* stream) {
    if (n_slots == 0) return hipSuccess;
    hipError_t err = reserve_lds(reinterpret_cast<const void*>(fold_step_unfold_t_kernel),
                                 g_fold_step_unfold_t_lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(fold_step_unfold_t_kernel, dim3((uint32_t)n_slots), dim3(kStepThreads),
                       kStepLdsBytes, (hipStream_t)stream, d_entries, grads, outs, touts, master, m, v,
                       reinterpret_cast<uint32_t*>(codes), scale_inv, s, n_slots);
    return hipGetLastError();
}

int launch_transpose_pow2(const TileEntry* d_entries, const int32_t* order, int64_t n_slots,
                          const uint8_t* codes, const float* scale_inv, const TransposeArgs& args,
                          void* stream) {
    if (n_slots == 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_pow2_kernel, dim3((uint32_t)n_slots), dim3(kThreads), 0,
                       (hipStream_t)stream, d_entries, order, codes, scale_inv, args);
    return hipGetLastError();
}

int launch_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(encode_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, in, out, n);
    return hipGetLastError();
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace bfz
