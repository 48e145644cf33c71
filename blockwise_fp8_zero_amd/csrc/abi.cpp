// The C ABI: argument checks, per-step scalars, launches, error strings.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "bfz_internal.h"

namespace bfz {
namespace {

thread_local char g_last_error[512] = "";

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_fail(const char* where, int err) {
    return fail(BFZ_EHIP, "%s: %s", where, hip_error_string(err));
}

// One tile per 1024-thread workgroup, and a launch's work-item count is a
// 32-bit number: at most this many tiles per launch.
constexpr int64_t kMaxLaunchTiles = (int64_t(1) << 32) / 1024 - 1;

// The plan's tile table lives on the device it was uploaded to: a call made
// with another device current would hand that device a foreign pointer.
int check_plan(const bfz_plan* plan, const char* where) {
    if (!plan->d_entries)
        return fail(BFZ_ESTATE, "%s: plan has no device table (no HIP device was visible when it "
                    "was created; see bfz_plan_upload)", where);
    for (const Segment& seg : plan->segments)
        if (seg.n_slots > kMaxLaunchTiles)
            return fail(BFZ_EINVAL, "%s: %lld slots in one launch segment, more than %lld", where,
                        (long long)seg.n_slots, (long long)kMaxLaunchTiles);
    int dev = -1;
    const hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(where, err);
    if (dev != plan->device)
        return fail(BFZ_ESTATE, "%s: plan uploaded to device %d, but device %d is current", where,
                    plan->device, dev);
    return BFZ_OK;
}

// Owned slots reference only weights whose pointer must then be non-null.
int check_weights(const bfz_plan* plan, const void* const* ptrs, const char* where) {
    for (const Segment& seg : plan->segments)
        for (int32_t w = seg.weight0; w < seg.weight0 + seg.n_weights; ++w)
            if (!ptrs[w])
                return fail(BFZ_EINVAL, "%s: pointer of weight %d is NULL but the rank owns its tiles",
                            where, w);
    return BFZ_OK;
}

}  // namespace

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

}  // namespace bfz

using namespace bfz;

extern "C" const char* bfz_last_error(void) { return g_last_error; }

namespace {

// Tiles of a strided shard array (master, m, v) sit `stride` floats apart:
// at least a tile, whole float4 (16-byte aligned tiles), and at most 2^26
// so that slot * stride stays far inside 64 bits.
constexpr int64_t kMaxStateStride = int64_t(1) << 26;

bool valid_stride(int64_t stride) {
    return stride >= kTileElems && stride <= kMaxStateStride && stride % 4 == 0;
}

int fold(const bfz_plan* plan, const float* const* src, float* dst, int64_t dst_stride,
         void* stream, const char* where) {
    if (!plan || !src || !dst) return fail(BFZ_EINVAL, "%s: null pointer", where);
    if (!valid_stride(dst_stride))
        return fail(BFZ_EINVAL, "%s: dst_stride %lld is not a multiple of 4 in [16384, 2^26]", where,
                    (long long)dst_stride);
    int rc = check_plan(plan, where);
    if (rc) return rc;
    if (!aligned(dst, 16)) return fail(BFZ_EALIGN, "%s: dst must be 16-byte aligned", where);
    rc = check_weights(plan, reinterpret_cast<const void* const*>(src), where);
    if (rc) return rc;
    for (int32_t w = 0; w < plan->n_weights; ++w)
        if (src[w] && !aligned(src[w], 4))
            return fail(BFZ_EALIGN, "%s: weight %d must be 4-byte aligned", where, w);
    for (const Segment& seg : plan->segments) {
        PackArgs args{};
        for (int32_t k = 0; k < seg.n_weights; ++k) args.src[k] = src[seg.weight0 + k];
        int err = launch_pack(plan->d_entries + seg.slot0, seg.n_slots, dst + seg.slot0 * dst_stride,
                              dst_stride, args, stream);
        if (err != hipSuccess) return hip_fail(where, err);
    }
    return BFZ_OK;
}

}  // namespace

extern "C" int pack_shard(const bfz_plan* plan, const float* const* src, float* dst, void* stream) {
    return fold(plan, src, dst, kTileElems, stream, "pack_shard");
}

extern "C" int pack_shard_strided(const bfz_plan* plan, const float* const* src, float* dst,
                                  int64_t dst_stride, void* stream) {
    return fold(plan, src, dst, dst_stride, stream, "pack_shard_strided");
}

extern "C" int unpack_fp8(const bfz_plan* plan, const uint8_t* codes, const float* scale_inv,
                          uint8_t* const* dst_fp8, float* const* dst_scale, void* stream) {
    if (!plan || !codes || !scale_inv || !dst_fp8 || !dst_scale)
        return fail(BFZ_EINVAL, "unpack_fp8: null pointer");
    int rc = check_plan(plan, "unpack_fp8");
    if (rc) return rc;
    if (!aligned(codes, 16)) return fail(BFZ_EALIGN, "unpack_fp8: codes must be 16-byte aligned");
    if (!aligned(scale_inv, 4)) return fail(BFZ_EALIGN, "unpack_fp8: scale_inv must be 4-byte aligned");
    rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_fp8), "unpack_fp8");
    if (rc) return rc;
    rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_scale), "unpack_fp8 (scale)");
    if (rc) return rc;
    for (int32_t w = 0; w < plan->n_weights; ++w)
        if (dst_scale[w] && !aligned(dst_scale[w], 4))
            return fail(BFZ_EALIGN, "unpack_fp8: scale grid %d must be 4-byte aligned", w);
    for (const Segment& seg : plan->segments) {
        if (seg.n_weights == 0) continue;  // padding slots carry nothing back
        UnpackArgs args{};
        for (int32_t k = 0; k < seg.n_weights; ++k) {
            args.codes[k] = dst_fp8[seg.weight0 + k];
            args.scale[k] = dst_scale[seg.weight0 + k];
        }
        int err = launch_unpack(plan->d_entries + seg.slot0, seg.n_slots,
                                codes + seg.slot0 * kTileElems, scale_inv + seg.slot0, args, stream);
        if (err != hipSuccess) return hip_fail("unpack_fp8", err);
    }
    return BFZ_OK;
}

namespace {

// The step's scalars, formed in double and rounded to binary32 once each:
// the bias corrections 1 - beta^t enter as lr / (1 - beta1^t) and
// sqrt(1 - beta2^t), as in the Int8AdamW step (lpnh.cn essay, section 4.3).
// opts may be NULL (every option 0).  eps must be positive: it keeps the
// denominator of an all-zero slot (every padding slot) away from 0 / 0.
int make_scalars(const bfz_adamw* hp, const bfz_step_options* opts, StepScalars* s,
                 const char* where) {
    const bfz_step_options none{};
    if (!opts) opts = &none;
    if (opts->reserved != 0) return fail(BFZ_EINVAL, "%s: bfz_step_options.reserved must be 0", where);
    s->state_stride = opts->state_stride == 0 ? kTileElems : opts->state_stride;
    if (!valid_stride(s->state_stride))
        return fail(BFZ_EINVAL, "%s: state_stride %lld is not 0 or a multiple of 4 in [16384, 2^26]",
                    where, (long long)opts->state_stride);
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps, wd = hp->weight_decay;
    if (!std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(wd) || !(eps > 0.0) ||
        !(b1 >= 0.0 && b1 < 1.0) || !(b2 >= 0.0 && b2 < 1.0) || hp->step < 1)
        return fail(BFZ_EINVAL,
                    "%s: need finite lr/eps/weight_decay, eps > 0, 0 <= beta < 1, step >= 1", where);
    const double t = double(hp->step);
    s->b1 = float(b1);
    s->c1 = float(1.0 - b1);
    s->b2 = float(b2);
    s->c2 = float(1.0 - b2);
    s->step_size = float(lr / (1.0 - std::pow(b1, t)));
    s->sbc2 = float(std::sqrt(1.0 - std::pow(b2, t)));
    s->eps = float(eps);
    s->decay = float(lr * wd);
    s->has_decay = wd != 0.0;
    s->pow2 = opts->scale_pow2 != 0;
    return BFZ_OK;
}

int check_state(float* master, float* m, float* v, uint8_t* codes, float* scale_inv,
                const char* where) {
    if (!aligned(master, 16) || !aligned(m, 16) || !aligned(v, 16) || !aligned(codes, 16))
        return fail(BFZ_EALIGN, "%s: master, grad, m, v and codes must be 16-byte aligned", where);
    if (!aligned(scale_inv, 4)) return fail(BFZ_EALIGN, "%s: scale_inv must be 4-byte aligned", where);
    return BFZ_OK;
}

int step_tiles(float* master, const float* grad, float* m, float* v, uint8_t* codes,
               float* scale_inv, int64_t n_tiles, const bfz_adamw* hp,
               const bfz_step_options* opts, void* stream, const char* where) {
    if (!master || !grad || !m || !v || !codes || !scale_inv || !hp)
        return fail(BFZ_EINVAL, "%s: null pointer", where);
    if (n_tiles < 0 || n_tiles > kMaxLaunchTiles)
        return fail(BFZ_EINVAL, "%s: n_tiles %lld outside [0, %lld]", where, (long long)n_tiles,
                    (long long)kMaxLaunchTiles);
    if (!aligned(grad, 16))
        return fail(BFZ_EALIGN, "%s: master, grad, m, v and codes must be 16-byte aligned", where);
    int rc = check_state(master, m, v, codes, scale_inv, where);
    if (rc) return rc;
    StepScalars s;
    rc = make_scalars(hp, opts, &s, where);
    if (rc) return rc;
    int err = launch_step(master, grad, m, v, codes, scale_inv, n_tiles, s, stream);
    if (err != hipSuccess) return hip_fail(where, err);
    return BFZ_OK;
}

}  // namespace

extern "C" int adamw_fp8_step(float* master, const float* grad, float* m, float* v,
                              uint8_t* codes, float* scale_inv, int64_t n_tiles,
                              const bfz_adamw* hp, void* stream) {
    return step_tiles(master, grad, m, v, codes, scale_inv, n_tiles, hp, nullptr, stream,
                      "adamw_fp8_step");
}

extern "C" int adamw_fp8_step_ex(float* master, const float* grad, float* m, float* v,
                                 uint8_t* codes, float* scale_inv, int64_t n_tiles,
                                 const bfz_adamw* hp, const bfz_step_options* opts,
                                 void* stream) {
    return step_tiles(master, grad, m, v, codes, scale_inv, n_tiles, hp, opts, stream,
                      "adamw_fp8_step_ex");
}

extern "C" int fold_adamw_fp8_step(const bfz_plan* plan, const float* const* grad, float* master,
                                   float* m, float* v, uint8_t* codes, float* scale_inv,
                                   const bfz_adamw* hp, const bfz_step_options* opts,
                                   void* stream) {
    if (!plan || !grad || !master || !m || !v || !codes || !scale_inv || !hp)
        return fail(BFZ_EINVAL, "fold_adamw_fp8_step: null pointer");
    int rc = check_plan(plan, "fold_adamw_fp8_step");
    if (rc) return rc;
    rc = check_weights(plan, reinterpret_cast<const void* const*>(grad), "fold_adamw_fp8_step");
    if (rc) return rc;
    for (int32_t w = 0; w < plan->n_weights; ++w)
        if (grad[w] && !aligned(grad[w], 4))
            return fail(BFZ_EALIGN, "fold_adamw_fp8_step: gradient %d must be 4-byte aligned", w);
    rc = check_state(master, m, v, codes, scale_inv, "fold_adamw_fp8_step");
    if (rc) return rc;
    StepScalars s;
    rc = make_scalars(hp, opts, &s, "fold_adamw_fp8_step");
    if (rc) return rc;
    for (const Segment& seg : plan->segments) {
        PackArgs args{};
        for (int32_t k = 0; k < seg.n_weights; ++k) args.src[k] = grad[seg.weight0 + k];
        const int64_t off = seg.slot0 * kTileElems, soff = seg.slot0 * s.state_stride;
        int err = launch_fold_step(plan->d_entries + seg.slot0, seg.n_slots, args, master + soff,
                                   m + soff, v + soff, codes + off, scale_inv + seg.slot0, s, stream);
        if (err != hipSuccess) return hip_fail("fold_adamw_fp8_step", err);
    }
    return BFZ_OK;
}

extern "C" int fold_adamw_fp8_step_unpack(const bfz_plan* plan, const float* const* grad,
                                          float* master, float* m, float* v, uint8_t* codes,
                                          float* scale_inv, uint8_t* const* dst_fp8,
                                          float* const* dst_scale, const bfz_adamw* hp,
                                          const bfz_step_options* opts, void* stream) {
    const char* where = "fold_adamw_fp8_step_unpack";
    if (!plan || !grad || !master || !m || !v || !dst_fp8 || !dst_scale || !hp)
        return fail(BFZ_EINVAL, "%s: null pointer", where);
    if (!codes != !scale_inv)
        return fail(BFZ_EINVAL, "%s: codes and scale_inv must be both given or both NULL", where);
    int rc = check_plan(plan, where);
    if (rc) return rc;
    rc = check_weights(plan, reinterpret_cast<const void* const*>(grad), where);
    if (!rc) rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_fp8), where);
    if (!rc) rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_scale), where);
    if (rc) return rc;
    for (int32_t w = 0; w < plan->n_weights; ++w) {
        if (grad[w] && !aligned(grad[w], 4))
            return fail(BFZ_EALIGN, "%s: gradient %d must be 4-byte aligned", where, w);
        if (dst_scale[w] && !aligned(dst_scale[w], 4))
            return fail(BFZ_EALIGN, "%s: scale grid %d must be 4-byte aligned", where, w);
    }
    if (!aligned(master, 16) || !aligned(m, 16) || !aligned(v, 16) || (codes && !aligned(codes, 16)))
        return fail(BFZ_EALIGN, "%s: master, m, v and codes must be 16-byte aligned", where);
    if (scale_inv && !aligned(scale_inv, 4))
        return fail(BFZ_EALIGN, "%s: scale_inv must be 4-byte aligned", where);
    StepScalars s;
    rc = make_scalars(hp, opts, &s, where);
    if (rc) return rc;
    for (const Segment& seg : plan->segments) {
        PackArgs in{};
        UnpackArgs out{};
        for (int32_t k = 0; k < seg.n_weights; ++k) {
            in.src[k] = grad[seg.weight0 + k];
            out.codes[k] = dst_fp8[seg.weight0 + k];
            out.scale[k] = dst_scale[seg.weight0 + k];
        }
        const int64_t off = seg.slot0 * kTileElems, soff = seg.slot0 * s.state_stride;
        int err = launch_fold_step_unfold(plan->d_entries + seg.slot0, seg.n_slots, in, out,
                                          master + soff, m + soff, v + soff,
                                          codes ? codes + off : nullptr,
                                          scale_inv ? scale_inv + seg.slot0 : nullptr, s, stream);
        if (err != hipSuccess) return hip_fail(where, err);
    }
    return BFZ_OK;
}

extern "C" int fold_adamw_fp8_step_unpack_t(const bfz_plan* plan, const float* const* grad,
                                            float* master, float* m, float* v, uint8_t* codes,
                                            float* scale_inv, uint8_t* const* dst_fp8,
                                            float* const* dst_scale, uint8_t* const* dst_t,
                                            float* const* dst_t_scale, const bfz_adamw* hp,
                                            const bfz_step_options* opts, void* stream) {
    const char* where = "fold_adamw_fp8_step_unpack_t";
    if (!plan || !grad || !master || !m || !v || !dst_fp8 || !dst_scale || !dst_t || !dst_t_scale ||
        !hp)
        return fail(BFZ_EINVAL, "%s: null pointer", where);
    if (!codes != !scale_inv)
        return fail(BFZ_EINVAL, "%s: codes and scale_inv must be both given or both NULL", where);
    if (!opts || !opts->scale_pow2)
        return fail(BFZ_EINVAL, "%s: the transposed copy needs power-of-two scales "
                    "(bfz_step_options.scale_pow2)", where);
    int rc = check_plan(plan, where);
    if (rc) return rc;
    rc = check_weights(plan, reinterpret_cast<const void* const*>(grad), where);
    if (!rc) rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_fp8), where);
    if (!rc) rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_scale), where);
    if (!rc) rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_t), where);
    if (!rc) rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_t_scale), where);
    if (rc) return rc;
    for (int32_t w = 0; w < plan->n_weights; ++w) {
        if (grad[w] && !aligned(grad[w], 4))
            return fail(BFZ_EALIGN, "%s: gradient %d must be 4-byte aligned", where, w);
        if (dst_scale[w] && !aligned(dst_scale[w], 4))
            return fail(BFZ_EALIGN, "%s: scale grid %d must be 4-byte aligned", where, w);
        if (dst_t_scale[w] && !aligned(dst_t_scale[w], 4))
            return fail(BFZ_EALIGN, "%s: transposed scale grid %d must be 4-byte aligned", where, w);
    }
    if (!aligned(master, 16) || !aligned(m, 16) || !aligned(v, 16) || (codes && !aligned(codes, 16)))
        return fail(BFZ_EALIGN, "%s: master, m, v and codes must be 16-byte aligned", where);
    if (scale_inv && !aligned(scale_inv, 4))
        return fail(BFZ_EALIGN, "%s: scale_inv must be 4-byte aligned", where);
    StepScalars s;
    rc = make_scalars(hp, opts, &s, where);
    if (rc) return rc;
    for (const Segment& seg : plan->segments) {
        PackArgs in{};
        UnpackArgs out{};
        TransposeArgs tout{};
        for (int32_t k = 0; k < seg.n_weights; ++k) {
            in.src[k] = grad[seg.weight0 + k];
            out.codes[k] = dst_fp8[seg.weight0 + k];
            out.scale[k] = dst_scale[seg.weight0 + k];
            tout.codes[k] = dst_t[seg.weight0 + k];
            tout.scale[k] = dst_t_scale[seg.weight0 + k];
            tout.rows[k] = int32_t(plan->dims[3 * (seg.weight0 + k) + 1]);
        }
        const int64_t off = seg.slot0 * kTileElems, soff = seg.slot0 * s.state_stride;
        int err = launch_fold_step_unfold_t(plan->d_entries + seg.slot0, seg.n_slots, in, out, tout,
                                            master + soff, m + soff, v + soff,
                                            codes ? codes + off : nullptr,
                                            scale_inv ? scale_inv + seg.slot0 : nullptr, s, stream);
        if (err != hipSuccess) return hip_fail(where, err);
    }
    return BFZ_OK;
}

extern "C" int bfz_transpose_pow2(const bfz_plan* plan, const uint8_t* codes,
                                  const float* scale_inv, uint8_t* const* dst_t,
                                  float* const* dst_t_scale, void* stream) {
    const char* where = "bfz_transpose_pow2";
    if (!plan || !codes || !scale_inv || !dst_t || !dst_t_scale)
        return fail(BFZ_EINVAL, "%s: null pointer", where);
    int rc = check_plan(plan, where);
    if (rc) return rc;
    if (!aligned(codes, 16)) return fail(BFZ_EALIGN, "%s: codes must be 16-byte aligned", where);
    if (!aligned(scale_inv, 4)) return fail(BFZ_EALIGN, "%s: scale_inv must be 4-byte aligned", where);
    rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_t), where);
    if (!rc) rc = check_weights(plan, reinterpret_cast<const void* const*>(dst_t_scale), where);
    if (rc) return rc;
    for (int32_t w = 0; w < plan->n_weights; ++w)
        if (dst_t_scale[w] && !aligned(dst_t_scale[w], 4))
            return fail(BFZ_EALIGN, "%s: scale grid %d must be 4-byte aligned", where, w);
    for (const Segment& seg : plan->segments) {
        if (seg.n_weights == 0) continue;
        TransposeArgs args{};
        for (int32_t k = 0; k < seg.n_weights; ++k) {
            args.codes[k] = dst_t[seg.weight0 + k];
            args.scale[k] = dst_t_scale[seg.weight0 + k];
            args.rows[k] = int32_t(plan->dims[3 * (seg.weight0 + k) + 1]);
        }
        int err = launch_transpose_pow2(plan->d_entries + seg.slot0,
                                        plan->d_transpose_order + seg.slot0, seg.n_slots,
                                        codes + seg.slot0 * kTileElems, scale_inv + seg.slot0,
                                        args, stream);
        if (err != hipSuccess) return hip_fail(where, err);
    }
    return BFZ_OK;
}

extern "C" int bfz_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (!in || !out) return fail(BFZ_EINVAL, "bfz_e4m3_encode: null pointer");
    if (n < 0) return fail(BFZ_EINVAL, "bfz_e4m3_encode: n < 0");
    int err = launch_encode(in, out, n, stream);
    if (err != hipSuccess) return hip_fail("bfz_e4m3_encode", err);
    return BFZ_OK;
}
