// CPU build of the library's planner and C ABI (plan.cpp, abi.cpp) for
// AddressSanitizer / UndefinedBehaviorSanitizer runs -- no GPU involved.
//
//  * The few HIP runtime calls the host code makes (device query, malloc,
//    memcpy, free, error strings) are served from host memory here.
//  * Every kernel launch is replaced by a host loop that reads and writes
//    exactly the elements the kernel reaches through the uploaded tile table
//    (base, ld, local, valid extent, scale_index).  Weights, grids and
//    shards are allocated at their exact sizes, so a table entry that points
//    outside a weight, or a segment that overruns the shard, is a sanitizer
//    report.
//  * Each launch segment is recorded: the segments of one call must tile the
//    shard's slots exactly once, with at most 64 weights each.
//  * Results of the layout calls are compared with direct loops over the
//    weights (fold, unfold, transposed placement), and error paths are
//    driven with bad arguments.
// Exit status 0 when every check passes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "bfz.h"
#include "bfz_internal.h"

// ---- the HIP runtime calls of the host code, on host memory ----------------
static int g_device = 0;        // the "current device" the host code sees
static int g_device_count = 1;  // 0: a host with no HIP device
extern "C" {
hipError_t hipGetDeviceCount(int* n) {
    *n = g_device_count;
    return g_device_count > 0 ? hipSuccess : hipErrorNoDevice;
}
hipError_t hipGetDevice(int* d) {
    if (g_device_count == 0) return hipErrorNoDevice;
    *d = g_device;
    return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipMalloc(void** p, size_t n) {
    *p = std::malloc(n);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
    std::free(p);
    return hipSuccess;
}
hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) {
    std::memcpy(d, s, n);
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "host stand-in error"; }
}

static int g_failures = 0;
#define CHECK(cond, ...)                                             \
    do {                                                             \
        if (!(cond)) {                                               \
            std::fprintf(stderr, "CHECK failed at line %d: ", __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                       \
            std::fprintf(stderr, "\n");                              \
            ++g_failures;                                            \
        }                                                            \
    } while (0)

// ---- launches as host loops over the table --------------------------------
namespace {
struct Call {
    const bfz::TileEntry* entries;
    int64_t n_slots;
};
std::vector<Call> g_calls;
int g_fail_launch = 0;  // nonzero: the next launch reports this HIP error

int record(const bfz::TileEntry* e, int64_t n) {
    g_calls.push_back({e, n});
    for (int64_t s = 0; s < n; ++s)
        CHECK(e[s].local >= -1 && e[s].local < bfz::kSegWeights, "slot %lld: local %d outside one launch's weights",
              (long long)s, int(e[s].local));
    if (g_fail_launch) {
        int err = g_fail_launch;
        g_fail_launch = 0;
        return err;
    }
    return 0;
}
}  // namespace

namespace bfz {

int launch_pack(const TileEntry* e, int64_t n, float* dst, int64_t dst_stride, const PackArgs& args,
                void*) {
    if (int err = record(e, n)) return err;
    for (int64_t s = 0; s < n; ++s) {
        const TileEntry& t = e[s];
        float* tile = dst + s * dst_stride;
        for (int a = 0; a < kTileDim; ++a)
            for (int b = 0; b < kTileDim; ++b)
                tile[a * kTileDim + b] = (t.local >= 0 && a < t.valid_rows && b < t.valid_cols)
                                             ? args.src[t.local][t.base + (int64_t)a * t.ld + b]
                                             : 0.0f;
    }
    return 0;
}

int launch_unpack(const TileEntry* e, int64_t n, const uint8_t* codes, const float* scale_inv,
                  const UnpackArgs& args, void*) {
    if (int err = record(e, n)) return err;
    for (int64_t s = 0; s < n; ++s) {
        const TileEntry& t = e[s];
        if (t.local < 0) continue;
        for (int a = 0; a < t.valid_rows; ++a)
            for (int b = 0; b < t.valid_cols; ++b)
                args.codes[t.local][t.base + (int64_t)a * t.ld + b] = codes[s * kTileElems + a * kTileDim + b];
        args.scale[t.local][t.scale_index] = scale_inv[s];
    }
    return 0;
}

// The step's arithmetic is not what is checked here: each element of every
// array is read and written once (p += g, m += p, v = m - g, code = low byte
// of p's bits, scale_inv = 1), so the sanitizer sees the kernel's extents
// and a result that depends on every array's placement.  master / m / v
// tiles sit `stride` floats apart, gradient and code tiles 16384.
static void touch_tile(float* p, const float* g, float* m, float* v, uint8_t* codes, float* sc,
                       int64_t s, int64_t stride) {
    for (int k = 0; k < kTileElems; ++k) {
        const int64_t i = s * stride + k, j = s * kTileElems + k;
        const float gi = g ? g[j] : 0.0f;
        p[i] += gi;
        m[i] += p[i];
        v[i] = m[i] - gi;
        if (codes) {
            uint32_t bits;
            std::memcpy(&bits, &p[i], 4);
            codes[j] = uint8_t(bits);
        }
    }
    if (sc) sc[s] = 1.0f;
}

int launch_step(float* master, const float* grad, float* m, float* v, uint8_t* codes,
                float* scale_inv, int64_t n_tiles, const StepScalars& st, void*) {
    g_calls.push_back({nullptr, n_tiles});
    for (int64_t s = 0; s < n_tiles; ++s)
        touch_tile(master, grad, m, v, codes, scale_inv, s, st.state_stride);
    return 0;
}

static void fold_grad(const TileEntry& t, const float* src, std::vector<float>& tile) {
    tile.assign(kTileElems, 0.0f);
    if (t.local < 0) return;
    for (int a = 0; a < t.valid_rows; ++a)
        for (int b = 0; b < t.valid_cols; ++b) tile[a * kTileDim + b] = src[t.base + (int64_t)a * t.ld + b];
}

int launch_fold_step(const TileEntry* e, int64_t n, const PackArgs& grads, float* master, float* m,
                     float* v, uint8_t* codes, float* scale_inv, const StepScalars& st, void*) {
    if (int err = record(e, n)) return err;
    std::vector<float> g;
    for (int64_t s = 0; s < n; ++s) {
        fold_grad(e[s], e[s].local >= 0 ? grads.src[e[s].local] : nullptr, g);
        for (int k = 0; k < kTileElems; ++k) master[s * st.state_stride + k] += g[k];
        touch_tile(master, nullptr, m, v, codes, scale_inv, s, st.state_stride);
    }
    return 0;
}

int launch_fold_step_unfold(const TileEntry* e, int64_t n, const PackArgs& grads,
                            const UnpackArgs& outs, float* master, float* m, float* v,
                            uint8_t* codes, float* scale_inv, const StepScalars& st, void*) {
    if (int err = record(e, n)) return err;
    std::vector<float> g;
    for (int64_t s = 0; s < n; ++s) {
        const TileEntry& t = e[s];
        fold_grad(t, t.local >= 0 ? grads.src[t.local] : nullptr, g);
        for (int k = 0; k < kTileElems; ++k) master[s * st.state_stride + k] += g[k];
        touch_tile(master, nullptr, m, v, codes, scale_inv, s, st.state_stride);
        if (t.local < 0) continue;
        for (int a = 0; a < t.valid_rows; ++a)
            for (int b = 0; b < t.valid_cols; ++b) {
                uint32_t bits;
                std::memcpy(&bits, &master[s * st.state_stride + a * kTileDim + b], 4);
                outs.codes[t.local][t.base + (int64_t)a * t.ld + b] = uint8_t(bits);
            }
        outs.scale[t.local][t.scale_index] = 1.0f;
    }
    return 0;
}

int launch_fold_step_unfold_t(const TileEntry* e, int64_t n, const PackArgs& grads,
                              const UnpackArgs& outs, const TransposeArgs& touts, float* master,
                              float* m, float* v, uint8_t* codes, float* scale_inv,
                              const StepScalars& s, void* stream) {
    // the step and row-major output as launch_fold_step_unfold (which records
    // the segment), then the transposed placement from the tile's codes
    // (low bytes of the updated master)
    if (int err = launch_fold_step_unfold(e, n, grads, outs, master, m, v, codes, scale_inv, s, stream))
        return err;
    for (int64_t sl = 0; sl < n; ++sl) {
        const TileEntry& t = e[sl];
        if (t.local < 0) continue;
        const int64_t H = touts.rows[t.local], W = t.ld;
        const int64_t hb = (H + kTileDim - 1) / kTileDim, wb = (W + kTileDim - 1) / kTileDim;
        const int64_t j = t.scale_index % wb, ei = t.scale_index / wb, i = ei % hb, ex = ei / hb;
        for (int c = 0; c < t.valid_cols; ++c) {
            const int64_t out_row = ex * W + kTileDim * j + c;
            for (int r = 0; r < t.valid_rows; ++r) {
                uint32_t bits;
                std::memcpy(&bits, &master[sl * s.state_stride + r * kTileDim + c], 4);
                touts.codes[t.local][out_row * H + kTileDim * i + r] = uint8_t(bits);
            }
            touts.scale[t.local][out_row * hb + i] = 1.0f;
        }
    }
    return 0;
}

int launch_transpose_pow2(const TileEntry* e, const int32_t* order, int64_t n, const uint8_t* codes,
                          const float* scale_inv, const TransposeArgs& args, void*) {
    if (int err = record(e, n)) return err;
    // the launch order must be a permutation of the segment's slots: each
    // workgroup takes one slot, every slot once
    std::vector<char> seen(size_t(n), 0);
    for (int64_t b = 0; b < n; ++b) {
        CHECK(order[b] >= 0 && order[b] < n && !seen[size_t(order[b])],
              "transpose order: workgroup %lld takes slot %d of %lld", (long long)b, order[b], (long long)n);
        if (order[b] >= 0 && order[b] < n) seen[size_t(order[b])] = 1;
    }
    for (int64_t b = 0; b < n; ++b) {
        const int64_t s = order[b];
        if (s < 0 || s >= n) continue;
        const TileEntry& t = e[s];
        if (t.local < 0) continue;
        const int64_t H = args.rows[t.local], W = t.ld;
        const int64_t hb = (H + kTileDim - 1) / kTileDim, wb = (W + kTileDim - 1) / kTileDim;
        const int64_t j = t.scale_index % wb, ei = t.scale_index / wb, i = ei % hb, ex = ei / hb;
        for (int c = 0; c < t.valid_cols; ++c) {
            const int64_t out_row = ex * W + kTileDim * j + c;
            for (int r = 0; r < t.valid_rows; ++r)
                args.codes[t.local][out_row * H + kTileDim * i + r] = codes[s * kTileElems + r * kTileDim + c];
            args.scale[t.local][out_row * hb + i] = scale_inv[s];
        }
    }
    return 0;
}

int launch_encode(const float* in, uint8_t* out, int64_t n, void*) {
    g_calls.push_back({nullptr, n});
    for (int64_t i = 0; i < n; ++i) out[i] = in[i] < 0.0f ? 0x80 : 0x00;
    return 0;
}

const char* hip_error_string(int) { return "host stand-in launch error"; }

}  // namespace bfz

// ---- helpers -----------------------------------------------------------------
namespace {

using bfz::kTileElems;

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return g_rng;
}
int64_t uniform(int64_t lo, int64_t hi) { return lo + int64_t(next_u64() % uint64_t(hi - lo + 1)); }

// Buffers allocated at their exact size (no slack for the sanitizer to hide in).
template <class T>
T* exact(int64_t n) {
    return static_cast<T*>(std::malloc(size_t(n > 0 ? n : 1) * sizeof(T)));
}

struct Tile {
    int64_t p, e, i, j, rows, cols;
};

std::vector<Tile> enumerate(const std::vector<int64_t>& dims) {
    std::vector<Tile> out;
    for (size_t p = 0; p < dims.size() / 3; ++p) {
        const int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
        const int64_t hb = (H + 127) / 128, wb = (W + 127) / 128;
        for (int64_t e = 0; e < E; ++e)
            for (int64_t i = 0; i < hb; ++i)
                for (int64_t j = 0; j < wb; ++j)
                    out.push_back({int64_t(p), e, i, j, std::min<int64_t>(128, H - 128 * i),
                                   std::min<int64_t>(128, W - 128 * j)});
    }
    return out;
}

// The recorded segments of one call tile [0, q) of the plan's table in order.
void check_segments(const bfz_plan* plan, int64_t q, bool skip_padding_segments, const char* what) {
    int64_t next = 0;
    for (const Call& c : g_calls) {
        const int64_t first = c.entries - plan->d_entries;
        CHECK(first == next || (skip_padding_segments && first > next), "%s: segment starts at %lld, expected %lld",
              what, (long long)first, (long long)next);
        CHECK(c.n_slots > 0 && first + c.n_slots <= q, "%s: segment [%lld, +%lld) outside [0, %lld)", what,
              (long long)first, (long long)c.n_slots, (long long)q);
        next = first + c.n_slots;
    }
    if (!skip_padding_segments) CHECK(next == q, "%s: segments end at %lld of %lld", what, (long long)next, (long long)q);
    g_calls.clear();
}

void run_plan_case(const std::vector<int64_t>& dims, int32_t D) {
    const int32_t n = int32_t(dims.size() / 3);
    const std::vector<Tile> all = enumerate(dims);
    const int64_t T = int64_t(all.size());
    int64_t seen = 0;
    for (int32_t rank = 0; rank < D; ++rank) {
        bfz_plan* plan = nullptr;
        CHECK(bfz_plan_create(dims.data(), n, D, rank, &plan) == BFZ_OK, "plan_create: %s", bfz_last_error());
        if (!plan) return;
        const int64_t q = bfz_plan_shard_tiles(plan), owned = bfz_plan_owned_tiles(plan);
        CHECK(q == (T + D - 1) / D && bfz_plan_total_tiles(plan) == T, "quota");
        std::vector<int64_t> table(size_t(6 * q));
        CHECK(bfz_plan_table(plan, table.data()) == BFZ_OK, "plan_table");
        for (int64_t s = 0; s < q; ++s) {
            int64_t row[6];
            CHECK(bfz_plan_tile(plan, s, row) == BFZ_OK, "plan_tile");
            CHECK(std::memcmp(row, &table[size_t(6 * s)], sizeof row) == 0, "tile vs table");
            if (s < owned) {
                const Tile& w = all[size_t(seen + s)];
                CHECK(row[0] == w.p && row[1] == w.e && row[2] == w.i && row[3] == w.j && row[4] == w.rows &&
                          row[5] == w.cols,
                      "slot %lld of rank %d is not tile %lld", (long long)s, rank, (long long)(seen + s));
            } else {
                CHECK(row[0] == -1, "padding slot");
            }
        }
        int64_t bad[6];
        CHECK(bfz_plan_tile(plan, q, bad) == BFZ_EINVAL && bfz_plan_tile(plan, -1, bad) == BFZ_EINVAL,
              "plan_tile range");
        seen += owned;

        // created with a device visible, the plan already holds its device
        // table: uploading again changes nothing
        CHECK(bfz_plan_upload(plan) == BFZ_OK, "upload on the same device: %s", bfz_last_error());
        {   // a plan created on a host without a device is host-only: its
            // device calls report a state error until bfz_plan_upload
            g_device_count = 0;
            bfz_plan* host_only = nullptr;
            CHECK(bfz_plan_create(dims.data(), n, D, rank, &host_only) == BFZ_OK, "host-only plan: %s",
                  bfz_last_error());
            g_device_count = 1;
            std::vector<const float*> nul(size_t(n), nullptr);
            float* tiny_dst = exact<float>(kTileElems * (q > 0 ? q : 1));
            CHECK(pack_shard(host_only, nul.data(), tiny_dst, nullptr) == BFZ_ESTATE &&
                      std::strstr(bfz_last_error(), "no device table"),
                  "pack with a host-only plan");
            CHECK(bfz_plan_upload(host_only) == BFZ_OK, "upload of a host-only plan: %s", bfz_last_error());
            CHECK(bfz_plan_upload(host_only) == BFZ_OK, "second upload on the same device");
            std::free(tiny_dst);
            bfz_plan_destroy(host_only);
        }

        // exact-size weights, FP8 weights, scale grids and transposes
        std::vector<float*> wts(size_t(n), nullptr), grads(size_t(n), nullptr);
        std::vector<uint8_t*> w8(size_t(n), nullptr), wt8(size_t(n), nullptr);
        std::vector<float*> grid(size_t(n), nullptr), tgrid(size_t(n), nullptr);
        std::vector<bool> touched(size_t(n), false);
        for (int64_t s = 0; s < owned; ++s) touched[size_t(table[size_t(6 * s)])] = true;
        for (int32_t p = 0; p < n; ++p) {
            if (!touched[size_t(p)]) continue;  // weights this rank does not touch stay NULL
            const int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
            const int64_t hb = (H + 127) / 128, wb = (W + 127) / 128;
            wts[size_t(p)] = exact<float>(E * H * W);
            grads[size_t(p)] = exact<float>(E * H * W);
            for (int64_t k = 0; k < E * H * W; ++k) {
                wts[size_t(p)][k] = float(p * 1000003 + k);
                grads[size_t(p)][k] = 0.0f;
            }
            w8[size_t(p)] = exact<uint8_t>(E * H * W);
            wt8[size_t(p)] = exact<uint8_t>(E * W * H);
            grid[size_t(p)] = exact<float>(E * hb * wb);
            tgrid[size_t(p)] = exact<float>(E * W * hb);
        }
        const int64_t ne = q * kTileElems;
        float* shard = exact<float>(ne);
        float* m = exact<float>(ne);
        float* v = exact<float>(ne);
        uint8_t* codes = exact<uint8_t>(ne);
        float* sc = exact<float>(q);
        for (int64_t k = 0; k < ne; ++k) m[k] = v[k] = 0.0f;

        // fold against a direct loop
        g_calls.clear();
        CHECK(pack_shard(plan, const_cast<const float* const*>(wts.data()), shard, nullptr) == BFZ_OK, "pack: %s",
              bfz_last_error());
        check_segments(plan, q, false, "pack_shard");
        for (int64_t s = 0; s < q; ++s) {
            const int64_t* r = &table[size_t(6 * s)];
            for (int a = 0; a < 128; ++a)
                for (int b = 0; b < 128; ++b) {
                    float want = 0.0f;
                    if (r[0] >= 0 && a < r[4] && b < r[5]) {
                        const int64_t H = dims[3 * r[0] + 1], W = dims[3 * r[0] + 2];
                        want = wts[size_t(r[0])][(r[1] * H + 128 * r[2] + a) * W + 128 * r[3] + b];
                    }
                    CHECK(shard[s * kTileElems + a * 128 + b] == want, "fold slot %lld (%d, %d)", (long long)s, a, b);
                }
        }
        // unfold of codes = low byte of the folded value: the FP8 weight then
        // holds the low byte of every owned element
        for (int64_t k = 0; k < ne; ++k) {
            uint32_t bits;
            std::memcpy(&bits, &shard[k], 4);
            codes[k] = uint8_t(bits);
        }
        for (int64_t s = 0; s < q; ++s) sc[s] = float(s + 1);
        CHECK(unpack_fp8(plan, codes, sc, w8.data(), grid.data(), nullptr) == BFZ_OK, "unpack: %s", bfz_last_error());
        check_segments(plan, q, true, "unpack_fp8");
        for (int64_t s = 0; s < owned; ++s) {
            const int64_t* r = &table[size_t(6 * s)];
            const int64_t H = dims[3 * r[0] + 1], W = dims[3 * r[0] + 2];
            const int64_t hb = (H + 127) / 128, wb = (W + 127) / 128;
            for (int64_t a = 0; a < r[4]; ++a)
                for (int64_t b = 0; b < r[5]; ++b) {
                    const int64_t k = (r[1] * H + 128 * r[2] + a) * W + 128 * r[3] + b;
                    uint32_t bits;
                    std::memcpy(&bits, &wts[size_t(r[0])][k], 4);
                    CHECK(w8[size_t(r[0])][k] == uint8_t(bits), "unfold element");
                }
            CHECK(grid[size_t(r[0])][(r[1] * hb + r[2]) * wb + r[3]] == float(s + 1), "scale grid cell");
        }
        // transposed placement
        CHECK(bfz_transpose_pow2(plan, codes, sc, wt8.data(), tgrid.data(), nullptr) == BFZ_OK, "transpose: %s",
              bfz_last_error());
        check_segments(plan, q, true, "bfz_transpose_pow2");
        for (int64_t s = 0; s < owned; ++s) {
            const int64_t* r = &table[size_t(6 * s)];
            const int64_t H = dims[3 * r[0] + 1], W = dims[3 * r[0] + 2];
            for (int64_t a = 0; a < r[4]; ++a)
                for (int64_t b = 0; b < r[5]; ++b)
                    CHECK(wt8[size_t(r[0])][(r[1] * W + 128 * r[3] + b) * H + 128 * r[2] + a] ==
                              w8[size_t(r[0])][(r[1] * H + 128 * r[2] + a) * W + 128 * r[3] + b],
                          "transposed element");
        }
        // the step entry points reach every slot of the shard; the
        // hyper-parameters (exactly the six-field, 48-byte struct) and
        // the options sit in heap blocks of their exact size, so reading past
        // either is a sanitizer report
        bfz_adamw* hpp = exact<bfz_adamw>(1);
        *hpp = bfz_adamw{1e-4, 0.9, 0.95, 1e-8, 0.1, 1};
        const bfz_adamw& hp = *hpp;
        bfz_step_options* opt = exact<bfz_step_options>(1);
        *opt = bfz_step_options{0, 0, 0};
        g_calls.clear();
        CHECK(adamw_fp8_step(shard, shard, m, v, codes, sc, q, &hp, nullptr) == BFZ_OK, "step: %s", bfz_last_error());
        CHECK(adamw_fp8_step_ex(shard, shard, m, v, codes, sc, q, &hp, opt, nullptr) == BFZ_OK, "step ex: %s",
              bfz_last_error());
        CHECK(adamw_fp8_step_ex(shard, shard, m, v, codes, sc, q, &hp, nullptr, nullptr) == BFZ_OK,
              "step ex, no options: %s", bfz_last_error());
        g_calls.clear();
        CHECK(fold_adamw_fp8_step(plan, const_cast<const float* const*>(grads.data()), shard, m, v, codes, sc, &hp,
                                  nullptr, nullptr) == BFZ_OK,
              "fold step: %s", bfz_last_error());
        check_segments(plan, q, false, "fold_adamw_fp8_step");
        CHECK(fold_adamw_fp8_step_unpack(plan, const_cast<const float* const*>(grads.data()), shard, m, v, codes, sc,
                                         w8.data(), grid.data(), &hp, opt, nullptr) == BFZ_OK,
              "one-kernel step: %s", bfz_last_error());
        check_segments(plan, q, false, "fold_adamw_fp8_step_unpack");
        CHECK(fold_adamw_fp8_step_unpack(plan, const_cast<const float* const*>(grads.data()), shard, m, v, nullptr,
                                         nullptr, w8.data(), grid.data(), &hp, nullptr, nullptr) == BFZ_OK,
              "one-kernel step without tile-major codes: %s", bfz_last_error());
        check_segments(plan, q, false, "fold_adamw_fp8_step_unpack (row-major only)");
        CHECK(fold_adamw_fp8_step_unpack_t(plan, const_cast<const float* const*>(grads.data()), shard, m, v,
                                           codes, sc, w8.data(), grid.data(), wt8.data(), tgrid.data(), &hp, opt,
                                           nullptr) == BFZ_EINVAL,
              "transposed copy without power-of-two scales");
        CHECK(fold_adamw_fp8_step_unpack_t(plan, const_cast<const float* const*>(grads.data()), shard, m, v,
                                           codes, sc, w8.data(), grid.data(), wt8.data(), tgrid.data(), &hp,
                                           nullptr, nullptr) == BFZ_EINVAL,
              "transposed copy without options");
        g_calls.clear();
        opt->scale_pow2 = 1;
        CHECK(fold_adamw_fp8_step_unpack_t(plan, const_cast<const float* const*>(grads.data()), shard, m, v,
                                           codes, sc, w8.data(), grid.data(), wt8.data(), tgrid.data(), &hp, opt,
                                           nullptr) == BFZ_OK,
              "one-kernel step with the transposed copy: %s", bfz_last_error());
        check_segments(plan, q, false, "fold_adamw_fp8_step_unpack_t");
        std::free(hpp);
        std::free(opt);

        // a launch failure surfaces as BFZ_EHIP with a message
        if (q > 0) {
            g_fail_launch = int(hipErrorLaunchFailure);
            CHECK(pack_shard(plan, const_cast<const float* const*>(wts.data()), shard, nullptr) == BFZ_EHIP &&
                      std::strlen(bfz_last_error()) > 0,
                  "launch failure");
            g_fail_launch = 0;
            g_calls.clear();
        }
        for (int32_t p = 0; p < n; ++p) {
            std::free(wts[size_t(p)]);
            std::free(grads[size_t(p)]);
            std::free(w8[size_t(p)]);
            std::free(wt8[size_t(p)]);
            std::free(grid[size_t(p)]);
            std::free(tgrid[size_t(p)]);
        }
        std::free(shard);
        std::free(m);
        std::free(v);
        std::free(codes);
        std::free(sc);
        bfz_plan_destroy(plan);
    }
    CHECK(seen == T, "ranks own %lld of %lld tiles", (long long)seen, (long long)T);
}

// The interleaved state layout (state_stride 49152: one [master | m | v]
// block per tile, allocated at its exact size) against three separate
// arrays: the same folds and steps must leave bit-identical state, codes,
// scales and row-major outputs in every route, so a launch segment given
// the wrong state offset shows up -- and any access past the block buffer
// is a sanitizer report.
void run_layout_case(const std::vector<int64_t>& dims, int32_t D) {
    const int32_t n = int32_t(dims.size() / 3);
    constexpr int64_t S = 3 * kTileElems;
    for (int32_t rank = 0; rank < D; ++rank) {
        bfz_plan* plan = nullptr;
        CHECK(bfz_plan_create(dims.data(), n, D, rank, &plan) == BFZ_OK, "plan_create: %s", bfz_last_error());
        if (!plan) return;
        const int64_t q = bfz_plan_shard_tiles(plan), ne = q * kTileElems;
        const size_t nw = size_t(n);
        std::vector<float*> w(nw), gr(nw);
        std::vector<uint8_t*> w8a(nw), w8b(nw), wta(nw), wtb(nw);
        std::vector<float*> ga(nw), gb(nw), tga(nw), tgb(nw);
        for (int32_t p = 0; p < n; ++p) {
            const int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
            const int64_t cells = E * ((H + 127) / 128) * ((W + 127) / 128), tcells = E * W * ((H + 127) / 128);
            w[size_t(p)] = exact<float>(E * H * W);
            gr[size_t(p)] = exact<float>(E * H * W);
            for (int64_t k = 0; k < E * H * W; ++k) {
                w[size_t(p)][k] = float(p + 1) + float(k % 1021) * 0.25f;
                gr[size_t(p)][k] = float(k % 7) - 3.0f;
            }
            for (auto* v8 : {&w8a, &w8b, &wta, &wtb}) {
                (*v8)[size_t(p)] = exact<uint8_t>(E * H * W);
                std::memset((*v8)[size_t(p)], 0, size_t(E * H * W));
            }
            for (auto* vg : {&ga, &gb}) {
                (*vg)[size_t(p)] = exact<float>(cells);
                std::memset((*vg)[size_t(p)], 0, size_t(cells) * 4);
            }
            for (auto* vg : {&tga, &tgb}) {
                (*vg)[size_t(p)] = exact<float>(tcells);
                std::memset((*vg)[size_t(p)], 0, size_t(tcells) * 4);
            }
        }
        const float* const* wc = const_cast<const float* const*>(w.data());
        const float* const* gc = const_cast<const float* const*>(gr.data());
        float* P = exact<float>(ne);
        float* M = exact<float>(ne);
        float* V = exact<float>(ne);
        float* state = exact<float>(q * S);
        float* grad = exact<float>(ne);
        uint8_t* ca = exact<uint8_t>(ne);
        uint8_t* cb = exact<uint8_t>(ne);
        float* sa = exact<float>(q);
        float* sb = exact<float>(q);
        // fold master, m and v (the same weights, so m = v = master to start)
        for (float* x : {P, M, V}) CHECK(pack_shard(plan, wc, x, nullptr) == BFZ_OK, "pack: %s", bfz_last_error());
        for (int64_t off : {int64_t(0), int64_t(kTileElems), int64_t(2 * kTileElems)})
            CHECK(pack_shard_strided(plan, wc, state + off, S, nullptr) == BFZ_OK, "pack strided: %s",
                  bfz_last_error());
        CHECK(pack_shard(plan, gc, grad, nullptr) == BFZ_OK, "pack grad");
        g_calls.clear();
        const bfz_adamw hp{1e-4, 0.9, 0.95, 1e-8, 0.1, 1};
        bfz_step_options hs{0, 0, 0};
        bfz_step_options hi{0, 0, S};
        float *Pi = state, *Mi = state + kTileElems, *Vi = state + 2 * kTileElems;
        CHECK(adamw_fp8_step(P, grad, M, V, ca, sa, q, &hp, nullptr) == BFZ_OK, "step");
        CHECK(adamw_fp8_step_ex(Pi, grad, Mi, Vi, cb, sb, q, &hp, &hi, nullptr) == BFZ_OK, "step interleaved: %s",
              bfz_last_error());
        CHECK(fold_adamw_fp8_step(plan, gc, P, M, V, ca, sa, &hp, &hs, nullptr) == BFZ_OK, "fold step");
        CHECK(fold_adamw_fp8_step(plan, gc, Pi, Mi, Vi, cb, sb, &hp, &hi, nullptr) == BFZ_OK,
              "fold step interleaved");
        CHECK(fold_adamw_fp8_step_unpack(plan, gc, P, M, V, ca, sa, w8a.data(), ga.data(), &hp, &hs, nullptr) ==
                  BFZ_OK,
              "one-kernel step");
        CHECK(fold_adamw_fp8_step_unpack(plan, gc, Pi, Mi, Vi, cb, sb, w8b.data(), gb.data(), &hp, &hi, nullptr) ==
                  BFZ_OK,
              "one-kernel step interleaved");
        hs.scale_pow2 = hi.scale_pow2 = 1;
        CHECK(fold_adamw_fp8_step_unpack_t(plan, gc, P, M, V, ca, sa, w8a.data(), ga.data(), wta.data(),
                                           tga.data(), &hp, &hs, nullptr) == BFZ_OK,
              "transposed-copy step");
        CHECK(fold_adamw_fp8_step_unpack_t(plan, gc, Pi, Mi, Vi, cb, sb, w8b.data(), gb.data(), wtb.data(),
                                           tgb.data(), &hp, &hi, nullptr) == BFZ_OK,
              "transposed-copy step interleaved");
        g_calls.clear();
        for (int64_t sl = 0; sl < q; ++sl) {
            CHECK(std::memcmp(P + sl * kTileElems, Pi + sl * S, kTileElems * 4) == 0 &&
                      std::memcmp(M + sl * kTileElems, Mi + sl * S, kTileElems * 4) == 0 &&
                      std::memcmp(V + sl * kTileElems, Vi + sl * S, kTileElems * 4) == 0,
                  "rank %d slot %lld: interleaved state differs from separate arrays", rank, (long long)sl);
        }
        CHECK(std::memcmp(ca, cb, size_t(ne)) == 0 && std::memcmp(sa, sb, size_t(q) * 4) == 0, "codes / scales");
        for (int32_t p = 0; p < n; ++p) {
            const int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
            const int64_t cells = E * ((H + 127) / 128) * ((W + 127) / 128), tcells = E * W * ((H + 127) / 128);
            CHECK(std::memcmp(w8a[size_t(p)], w8b[size_t(p)], size_t(E * H * W)) == 0 &&
                      std::memcmp(wta[size_t(p)], wtb[size_t(p)], size_t(E * H * W)) == 0 &&
                      std::memcmp(ga[size_t(p)], gb[size_t(p)], size_t(cells) * 4) == 0 &&
                      std::memcmp(tga[size_t(p)], tgb[size_t(p)], size_t(tcells) * 4) == 0,
                  "row-major outputs of weight %d", p);
            for (auto* v : {&w8a, &w8b, &wta, &wtb}) std::free((*v)[size_t(p)]);
            for (auto* v : {&ga, &gb, &tga, &tgb}) std::free((*v)[size_t(p)]);
            std::free(w[size_t(p)]);
            std::free(gr[size_t(p)]);
        }
        for (void* x : {(void*)P, (void*)M, (void*)V, (void*)state, (void*)grad, (void*)ca, (void*)cb, (void*)sa,
                        (void*)sb})
            std::free(x);
        bfz_plan_destroy(plan);
    }
}

void run_error_paths() {
    const int64_t dims[] = {1, 200, 130};
    bfz_plan* plan = nullptr;
    CHECK(bfz_plan_create(nullptr, 1, 1, 0, &plan) == BFZ_EINVAL, "null dims");
    CHECK(bfz_plan_create(dims, 1, 0, 0, &plan) == BFZ_EINVAL, "D = 0");
    CHECK(bfz_plan_create(dims, 1, 2, 2, &plan) == BFZ_EINVAL, "rank = D");
    CHECK(bfz_plan_create(dims, 1, 2, -1, &plan) == BFZ_EINVAL, "rank < 0");
    CHECK(bfz_plan_create(dims, -1, 1, 0, &plan) == BFZ_EINVAL, "n_params < 0");
    const int64_t zero_dim[] = {1, 0, 5};
    CHECK(bfz_plan_create(zero_dim, 1, 1, 0, &plan) == BFZ_EINVAL, "H = 0");
    CHECK(bfz_plan_create(dims, 1, 1, 0, nullptr) == BFZ_EINVAL, "null out");
    CHECK(bfz_plan_upload(nullptr) == BFZ_EINVAL, "upload null");
    bfz_plan_destroy(nullptr);
    int32_t bop[1];
    int64_t be[2];
    CHECK(bfz_paramwise_split(dims, 1, 0, bop, be) == BFZ_EINVAL, "paramwise D = 0");
    CHECK(bfz_paramwise_split(dims, 1, 2, nullptr, be) == BFZ_EINVAL, "paramwise null");
    CHECK(bfz_paramwise_split(dims, 1, 2, bop, be) == BFZ_OK && be[bop[0]] == 200 * 130, "paramwise");

    CHECK(bfz_plan_create(dims, 1, 1, 0, &plan) == BFZ_OK && plan, "plan");
    {   // the plan belongs to the device it was created (uploaded) on
        const int64_t qq = bfz_plan_shard_tiles(plan);
        float* d = exact<float>(qq * kTileElems);
        float* wv = exact<float>(200 * 130);
        const float* ws[1] = {wv};
        g_device = 1;
        CHECK(pack_shard(plan, ws, d, nullptr) == BFZ_ESTATE && std::strstr(bfz_last_error(), "device"),
              "plan used with another device current");
        CHECK(bfz_plan_upload(plan) == BFZ_EINVAL, "upload to a second device");
        g_device = 0;
        std::free(d);
        std::free(wv);
    }
    const int64_t q = bfz_plan_shard_tiles(plan), ne = q * kTileElems;
    float* a = exact<float>(ne + 4);
    uint8_t* c = exact<uint8_t>(ne + 16);
    float* s = exact<float>(q + 1);
    float* w = exact<float>(200 * 130 + 1);
    uint8_t* w8 = exact<uint8_t>(200 * 130 + 1);
    float* g = exact<float>(2 * 2 + 1);
    const bfz_adamw hp{1e-4, 0.9, 0.95, 1e-8, 0.1, 1};
    const float* src[1] = {w};
    const float* src_odd[1] = {reinterpret_cast<const float*>(reinterpret_cast<const char*>(w) + 2)};
    uint8_t* d8[1] = {w8};
    float* dg[1] = {g};
    float* dg_odd[1] = {reinterpret_cast<float*>(reinterpret_cast<char*>(g) + 1)};
    const float* srcnull[1] = {nullptr};
    CHECK(pack_shard(nullptr, src, a, nullptr) == BFZ_EINVAL, "pack null plan");
    CHECK(pack_shard(plan, srcnull, a, nullptr) == BFZ_EINVAL, "pack null weight");
    CHECK(pack_shard(plan, src, a + 1, nullptr) == BFZ_EALIGN, "pack misaligned dst");
    CHECK(pack_shard(plan, src_odd, a, nullptr) == BFZ_EALIGN, "pack weight not 4-byte aligned");
    CHECK(unpack_fp8(plan, c + 1, s, d8, dg, nullptr) == BFZ_EALIGN, "unpack misaligned codes");
    CHECK(unpack_fp8(plan, c, s, d8, dg_odd, nullptr) == BFZ_EALIGN, "unpack misaligned grid");
    CHECK(adamw_fp8_step(a, a, a, a, c, s, -1, &hp, nullptr) == BFZ_EINVAL, "n_tiles < 0");
    CHECK(adamw_fp8_step(a + 1, a, a, a, c, s, q, &hp, nullptr) == BFZ_EALIGN, "misaligned master");
    CHECK(adamw_fp8_step(a, a, a, a, c + 4, s, q, &hp, nullptr) == BFZ_EALIGN, "misaligned codes");
    CHECK(adamw_fp8_step(a, a, a, a, c, s, q, nullptr, nullptr) == BFZ_EINVAL, "null hp");
    bfz_adamw bad = hp;
    bad.step = 0;
    CHECK(adamw_fp8_step(a, a, a, a, c, s, q, &bad, nullptr) == BFZ_EINVAL, "step 0");
    bad = hp;
    bad.beta1 = 1.0;
    CHECK(adamw_fp8_step(a, a, a, a, c, s, q, &bad, nullptr) == BFZ_EINVAL, "beta1 = 1");
    bad = hp;
    bad.lr = std::nan("");
    CHECK(fold_adamw_fp8_step(plan, src, a, a, a, c, s, &bad, nullptr, nullptr) == BFZ_EINVAL, "NaN lr");
    bad = hp;
    bad.eps = -1.0;
    CHECK(fold_adamw_fp8_step(plan, src, a, a, a, c, s, &bad, nullptr, nullptr) == BFZ_EINVAL, "eps < 0");
    bad.eps = 0.0;
    CHECK(adamw_fp8_step(a, a, a, a, c, s, q, &bad, nullptr) == BFZ_EINVAL && std::strstr(bfz_last_error(), "eps > 0"),
          "eps = 0");
    CHECK(fold_adamw_fp8_step_unpack(plan, src, a, a, a, c, nullptr, d8, dg, &hp, nullptr, nullptr) == BFZ_EINVAL,
          "codes without scale_inv");
    CHECK(fold_adamw_fp8_step_unpack(plan, src, a, a, a, nullptr, nullptr, d8, dg_odd, &hp, nullptr, nullptr) ==
              BFZ_EALIGN,
          "misaligned scale grid");
    CHECK(bfz_e4m3_encode(nullptr, c, 4, nullptr) == BFZ_EINVAL && bfz_e4m3_encode(a, c, -1, nullptr) == BFZ_EINVAL,
          "encode args");
    const bfz_step_options reserved{0, 1, 0};
    CHECK(adamw_fp8_step_ex(a, a, a, a, c, s, q, &hp, &reserved, nullptr) == BFZ_EINVAL &&
              std::strstr(bfz_last_error(), "reserved"),
          "reserved option field");
    for (int64_t stride : {int64_t(-16384), int64_t(16383), int64_t(16386), (int64_t(1) << 26) + 4}) {
        const bfz_step_options so{0, 0, stride};
        CHECK(adamw_fp8_step_ex(a, a, a, a, c, s, q, &hp, &so, nullptr) == BFZ_EINVAL &&
                  std::strstr(bfz_last_error(), "state_stride"),
              "bad state_stride %lld", (long long)stride);
        CHECK(pack_shard_strided(plan, src, a, stride, nullptr) == BFZ_EINVAL, "bad dst_stride %lld",
              (long long)stride);
    }
    CHECK(std::strlen(bfz_last_error()) > 0, "message");
    std::free(a);
    std::free(c);
    std::free(s);
    std::free(w);
    std::free(w8);
    std::free(g);
    bfz_plan_destroy(plan);
}

}  // namespace

int main() {
    run_error_paths();
    // ragged weights, several experts, more ranks than tiles
    for (int trial = 0; trial < 12; ++trial) {
        std::vector<int64_t> dims;
        const int n = int(uniform(1, 5));
        for (int p = 0; p < n; ++p) {
            dims.push_back(uniform(1, 3));
            dims.push_back(uniform(1, 400));
            dims.push_back(uniform(1, 400));
        }
        run_plan_case(dims, int32_t(uniform(1, 9)));
    }
    // more weights than one launch addresses: several segments
    std::vector<int64_t> many;
    for (int p = 0; p < 150; ++p) {
        many.push_back(1);
        many.push_back(uniform(1, 140));
        many.push_back(uniform(1, 140));
    }
    run_plan_case(many, 3);
    // tall weights over several ranks: ownership cut inside tile columns,
    // tile-row counts that are not multiples of 4
    run_plan_case({1, 1100, 300, 2, 700, 520}, 3);
    run_plan_case({1, 2000, 130, 1, 129, 4000}, 5);
    // tile rows of 8 and 16 tiles (kept in fold order by the transpose's
    // launch order) beside rows of 3 and 11 (dealt down their columns)
    run_plan_case({1, 300, 1024, 2, 260, 2048, 1, 500, 300, 1, 200, 1400}, 2);
    // both state layouts, one weight and several segments
    run_layout_case({2, 300, 200, 1, 129, 257}, 2);
    run_layout_case(many, 3);
    if (g_failures) {
        std::fprintf(stderr, "%d checks failed\n", g_failures);
        return 1;
    }
    std::printf("host driver: all checks passed\n");
    return 0;
}
