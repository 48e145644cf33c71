// Host planner: the block-wise split of one rank and its lookup table.
//
// "A ZeRO Optimizer Design for Blockwise FP8 Quantization", section
// "Block-wise split": weights are cut at 128x128 units (each quantized
// dimension padded to a multiple of 128), and a lookup table records, for
// every unit in the flat buffer, its weight and its real extent, so the
// optimizer can walk the 1-D buffer.  Section "Parameter layout transform"
// fixes the unit order within a weight (expert, tile row, tile column).
// Dealing units to ranks: equal quota q = ceil(T / D), rank r takes the
// contiguous global range [r q, min((r + 1) q, T)), short shards padded to q
// (the page pads param-wise buckets to the largest one, section
// "Param-wise split"; contiguity keeps the rank's slice one range of the
// flat buffer, so one collective moves it).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <limits>
#include <memory>
#include <new>

#include "bfz_internal.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The plan's tables, once the arguments are known to be valid (may throw
// std::bad_alloc, which bfz_plan_create turns into an error code).
int build_plan(const int64_t* dims, int32_t n_weights, int32_t D, int32_t rank, int64_t total,
               bfz_plan** out);

// Copies the table and the transpose order to the current device, one
// allocation (the plan has no device copy yet).
int upload_table(bfz_plan* plan, int dev, const char* where) {
    using namespace bfz;
    const size_t n = plan->entries.size();
    const size_t bytes = std::max<size_t>(1, n * sizeof(TileEntry) + n * sizeof(int32_t));
    static_assert(sizeof(TileEntry) % alignof(int32_t) == 0, "order array alignment");
    TileEntry* d = nullptr;
    hipError_t err = hipMalloc(reinterpret_cast<void**>(&d), bytes);
    if (err != hipSuccess) return fail(BFZ_EHIP, "%s: hipMalloc: %s", where, hipGetErrorString(err));
    int32_t* d_order = reinterpret_cast<int32_t*>(d + n);
    if (n) {
        err = hipMemcpy(d, plan->entries.data(), n * sizeof(TileEntry), hipMemcpyHostToDevice);
        if (err == hipSuccess)
            err = hipMemcpy(d_order, plan->transpose_order.data(), n * sizeof(int32_t),
                            hipMemcpyHostToDevice);
        if (err != hipSuccess) {
            (void)hipFree(d);
            return fail(BFZ_EHIP, "%s: hipMemcpy: %s", where, hipGetErrorString(err));
        }
    }
    plan->d_entries = d;
    plan->d_transpose_order = d_order;
    plan->device = dev;
    return BFZ_OK;
}

}  // namespace

extern "C" int bfz_plan_create(const int64_t* dims, int32_t n_weights, int32_t D, int32_t rank,
                               bfz_plan** out) {
    using namespace bfz;
    if (!dims || !out) return fail(BFZ_EINVAL, "bfz_plan_create: null pointer");
    *out = nullptr;
    if (n_weights < 1) return fail(BFZ_EINVAL, "bfz_plan_create: n_params must be >= 1");
    if (D < 1 || rank < 0 || rank >= D)
        return fail(BFZ_EINVAL, "bfz_plan_create: need D >= 1 and 0 <= rank < D (got D=%d rank=%d)",
                    D, rank);
    const int64_t kMaxDim = std::numeric_limits<int32_t>::max();
    int64_t total = 0;
    for (int32_t p = 0; p < n_weights; ++p) {
        int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
        if (E < 1 || H < 1 || W < 1 || H > kMaxDim || W > kMaxDim)
            return fail(BFZ_EINVAL, "bfz_plan_create: weight %d has bad dims {%lld, %lld, %lld}", p,
                        (long long)E, (long long)H, (long long)W);
        int64_t grid = ceil_div(H, kTileDim) * ceil_div(W, kTileDim);
        // a tile's cell in its weight's scale grid is a 32-bit index
        if (E > int64_t(INT32_MAX) / grid)
            return fail(BFZ_EINVAL, "bfz_plan_create: weight %d has more than 2^31 - 1 tiles", p);
        total += E * grid;
    }
    // A shard beyond 2^31 - 1 tiles (3.5e13 elements) is far past any one
    // GPU's memory; refusing it keeps the host table (80 B per slot) sane.
    if (ceil_div(total, D) > int64_t(INT32_MAX))
        return fail(BFZ_EINVAL, "bfz_plan_create: %lld tiles over %d ranks is more than 2^31 - 1 per rank",
                    (long long)total, D);
    int rc;
    try {
        rc = build_plan(dims, n_weights, D, rank, total, out);
    } catch (const std::bad_alloc&) {
        return fail(BFZ_EINVAL, "bfz_plan_create: out of host memory");
    }
    if (rc) return rc;
    // The device copy goes to the current device when the process sees one;
    // without a device the plan stays host-only (queries work, device calls
    // report BFZ_ESTATE).
    int count = 0, dev = -1;
    if (hipGetDeviceCount(&count) == hipSuccess && count > 0 && hipGetDevice(&dev) == hipSuccess) {
        rc = upload_table(*out, dev, "bfz_plan_create");
        if (rc) {
            delete *out;
            *out = nullptr;
            return rc;
        }
    }
    return BFZ_OK;
}

namespace {

// The transpose's launch order.  The dispatcher deals workgroups to the 8
// XCDs round-robin (b on XCD b % 8), and the tiles of one tile column write
// neighbouring pieces of the same W^T rows and group-scale rows, so each
// segment's slots are dealt to XCDs by tile column: queue x holds the slots
// with j % 8 == x, and position 8 k + x of the order takes the k-th slot of
// queue x (the queues' remainders, beyond the shortest, follow in slot
// order).  Inside a queue the slots stay in fold order (along tile rows),
// except for weights whose tile rows hold a number of tiles that is not a
// multiple of 8, which go down their tile columns (column-major).  With 8 |
// tiles per row, plain order already deals by column; the order changes
// the other weights.  Measured against plain order (one process, one box):
// dense-LLM shard 0.3135 -> 0.3003 ms, ragged 0.0459 -> 0.0405 ms, the
// 4096x4096 and MoE shards unchanged; going down the columns for every
// weight was 2.5% slower on the 4096x4096 shard.
void build_transpose_order(bfz_plan* plan) {
    using namespace bfz;
    const int64_t q = plan->quota;
    plan->transpose_order.resize(size_t(q));
    for (const Segment& seg : plan->segments) {
        int32_t* ord = plan->transpose_order.data() + seg.slot0;
        const int32_t n = int32_t(seg.n_slots);
        if (seg.n_weights == 0) {  // padding: never launched
            for (int32_t r = 0; r < n; ++r) ord[r] = r;
            continue;
        }
        const int64_t* row = &plan->table[size_t(6 * seg.slot0)];
        std::vector<int32_t> queue[8];
        for (int32_t r = 0; r < n; ++r) queue[row[6 * r + 3] % 8].push_back(r);
        for (auto& qx : queue) {
            std::stable_sort(qx.begin(), qx.end(), [&](int32_t a, int32_t b) {
                const int64_t* ta = row + 6 * a;
                const int64_t* tb = row + 6 * b;
                if (ta[0] != tb[0]) return ta[0] < tb[0];  // weight
                if (ta[1] != tb[1]) return ta[1] < tb[1];  // expert
                const int64_t W = plan->dims[size_t(3 * ta[0] + 2)];
                if ((W + kTileDim - 1) / kTileDim % 8 == 0) return false;  // fold order kept
                if (ta[3] != tb[3]) return ta[3] < tb[3];  // column-major: j, then i
                return ta[2] < tb[2];
            });
        }
        size_t shortest = queue[0].size();
        for (const auto& qx : queue) shortest = std::min(shortest, qx.size());
        int32_t pos = 0;
        for (size_t k = 0; k < shortest; ++k)
            for (const auto& qx : queue) ord[pos++] = qx[k];
        std::vector<int32_t> rest;
        for (const auto& qx : queue) rest.insert(rest.end(), qx.begin() + ptrdiff_t(shortest), qx.end());
        std::sort(rest.begin(), rest.end());
        for (int32_t r : rest) ord[pos++] = r;
    }
}

int build_plan(const int64_t* dims, int32_t n_weights, int32_t D, int32_t rank, int64_t total,
               bfz_plan** out) {
    using namespace bfz;
    std::unique_ptr<bfz_plan> plan(new bfz_plan);
    plan->n_weights = n_weights;
    plan->D = D;
    plan->rank = rank;
    plan->dims.assign(dims, dims + 3 * n_weights);
    plan->total = total;
    plan->quota = ceil_div(total, D);
    plan->first = int64_t(rank) * plan->quota;
    int64_t last = std::min(plan->first + plan->quota, total);
    plan->owned = last > plan->first ? last - plan->first : 0;

    const int64_t q = plan->quota;
    plan->table.assign(6 * q, 0);
    plan->entries.assign(q, TileEntry{0, 0, 0, 0, 0, -1, 0});
    for (int64_t s = 0; s < q; ++s) plan->table[6 * s] = -1;

    // Walk the owned global range weight by weight; within a weight, the
    // global index g maps to (expert, tile row, tile col) by division.
    int64_t weight_first = 0;  // global index of weight p's first tile
    std::vector<int32_t> slot_weight(q, -1);
    for (int32_t p = 0; p < n_weights && weight_first < last; ++p) {
        int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
        int64_t hb = ceil_div(H, kTileDim), wb = ceil_div(W, kTileDim);
        int64_t n = E * hb * wb;
        int64_t lo = std::max(weight_first, plan->first), hi = std::min(weight_first + n, last);
        for (int64_t g = lo; g < hi; ++g) {
            int64_t local = g - weight_first;
            int64_t e = local / (hb * wb), rem = local % (hb * wb);
            int64_t i = rem / wb, j = rem % wb;
            int64_t s = g - plan->first;
            int64_t rows = std::min<int64_t>(kTileDim, H - kTileDim * i);
            int64_t cols = std::min<int64_t>(kTileDim, W - kTileDim * j);
            int64_t* row = &plan->table[6 * s];
            row[0] = p; row[1] = e; row[2] = i; row[3] = j; row[4] = rows; row[5] = cols;
            TileEntry& t = plan->entries[s];
            t.base = (e * H + kTileDim * i) * W + kTileDim * j;
            t.ld = int32_t(W);
            t.scale_index = int32_t((e * hb + i) * wb + j);
            t.valid_rows = int16_t(rows);
            t.valid_cols = int16_t(cols);
            slot_weight[s] = p;
        }
        weight_first += n;
    }

    // Cut the slots into launch segments of at most kSegWeights weights.
    int64_t s = 0;
    while (s < plan->owned) {
        Segment seg{s, 0, slot_weight[s], 0};
        int64_t e = s;
        while (e < plan->owned && slot_weight[e] - seg.weight0 < kSegWeights) ++e;
        seg.n_slots = e - s;
        seg.n_weights = slot_weight[e - 1] - seg.weight0 + 1;
        for (int64_t k = s; k < e; ++k)
            plan->entries[k].local = int16_t(slot_weight[k] - seg.weight0);
        plan->segments.push_back(seg);
        s = e;
    }
    if (plan->owned < q) {  // padding slots ride in a segment of their own
        plan->segments.push_back(Segment{plan->owned, q - plan->owned, 0, 0});
    }
    build_transpose_order(plan.get());
    *out = plan.release();
    return BFZ_OK;
}

}  // namespace

// "Param-wise split" (the alternative the page rejects, kept to compare
// padding): weights sorted by size, largest first, each dealt to the bucket
// with the fewest elements so far; every bucket is then padded to the
// largest.  Ties: equal sizes keep their declared order, equal buckets go to
// the lower index.
extern "C" int bfz_paramwise_split(const int64_t* dims, int32_t n_weights, int32_t D,
                                   int32_t* bucket_of_weight, int64_t* bucket_elems) {
    using namespace bfz;
    if (!dims || !bucket_of_weight || !bucket_elems)
        return fail(BFZ_EINVAL, "bfz_paramwise_split: null pointer");
    if (n_weights < 1 || D < 1)
        return fail(BFZ_EINVAL, "bfz_paramwise_split: need n_params >= 1 and D >= 1");
    std::vector<std::pair<int64_t, int32_t>> order;
    try {
        order.resize(n_weights);
    } catch (const std::bad_alloc&) {
        return fail(BFZ_EINVAL, "bfz_paramwise_split: out of host memory");
    }
    // every bucket's sum stays below 2^62 when the total does
    int64_t total = 0;
    for (int32_t p = 0; p < n_weights; ++p) {
        const int64_t E = dims[3 * p], H = dims[3 * p + 1], W = dims[3 * p + 2];
        if (E < 1 || H < 1 || W < 1 || H > (int64_t(1) << 31) || W > (int64_t(1) << 31) ||
            E > (int64_t(1) << 62) / (H * W))
            return fail(BFZ_EINVAL, "bfz_paramwise_split: weight %d has bad dims", p);
        order[p] = {E * H * W, p};
        if (order[p].first > (int64_t(1) << 62) - total)
            return fail(BFZ_EINVAL, "bfz_paramwise_split: more than 2^62 elements in all");
        total += order[p].first;
    }
    std::stable_sort(order.begin(), order.end(),
                     [](const auto& a, const auto& b) { return a.first > b.first; });
    std::fill(bucket_elems, bucket_elems + D, int64_t(0));
    for (const auto& [size, p] : order) {
        const int32_t b = int32_t(std::min_element(bucket_elems, bucket_elems + D) - bucket_elems);
        bucket_of_weight[p] = b;
        bucket_elems[b] += size;
    }
    return BFZ_OK;
}

extern "C" void bfz_plan_destroy(bfz_plan* plan) {
    if (!plan) return;
    if (plan->d_entries) {
        int prev = -1;
        (void)hipGetDevice(&prev);
        if (plan->device >= 0) (void)hipSetDevice(plan->device);
        (void)hipFree(plan->d_entries);
        if (prev >= 0) (void)hipSetDevice(prev);
    }
    delete plan;
}

extern "C" int bfz_plan_upload(bfz_plan* plan) {
    using namespace bfz;
    if (!plan) return fail(BFZ_EINVAL, "bfz_plan_upload: null plan");
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(BFZ_EHIP, "bfz_plan_upload: %s", hipGetErrorString(err));
    if (plan->d_entries) {
        if (plan->device == dev) return BFZ_OK;
        return fail(BFZ_EINVAL, "bfz_plan_upload: plan already on device %d", plan->device);
    }
    return upload_table(plan, dev, "bfz_plan_upload");
}

extern "C" int64_t bfz_plan_shard_tiles(const bfz_plan* plan) { return plan ? plan->quota : -1; }
extern "C" int64_t bfz_plan_owned_tiles(const bfz_plan* plan) { return plan ? plan->owned : -1; }
extern "C" int64_t bfz_plan_total_tiles(const bfz_plan* plan) { return plan ? plan->total : -1; }

extern "C" int bfz_plan_table(const bfz_plan* plan, int64_t* out) {
    if (!plan || !out) return bfz::fail(BFZ_EINVAL, "bfz_plan_table: null pointer");
    std::copy(plan->table.begin(), plan->table.end(), out);
    return BFZ_OK;
}

extern "C" int bfz_plan_tile(const bfz_plan* plan, int64_t slot, int64_t out[6]) {
    if (!plan || !out) return bfz::fail(BFZ_EINVAL, "bfz_plan_tile: null pointer");
    if (slot < 0 || slot >= plan->quota)
        return bfz::fail(BFZ_EINVAL, "bfz_plan_tile: slot %lld outside [0, %lld)", (long long)slot,
                         (long long)plan->quota);
    std::copy(&plan->table[6 * slot], &plan->table[6 * slot] + 6, out);
    return BFZ_OK;
}
