// Seeded synthetic inputs for the shard-step tests and benchmark.
//
// This module holds none of the optimizer's or the quantizer's arithmetic:
// it only draws values.  One source serves both sides: the host functions
// feed the CPU oracle and the device kernel fills full-size GPU buffers,
// and because every floating-point step below is a single IEEE-754 binary64
// add, subtract, multiply or divide (no fused multiply-add, no library
// transcendental), the two produce bit-identical float32 values.
//
// Counter-based draws: value k of a stream is a pure function of
// (stream key, k), so any slice of any tensor can be regenerated alone.
//   * Hash: the SplitMix64 output function (Steele, Lea and Flood, "Fast
//     splittable pseudorandom number generators", OOPSLA 2014), applied to
//     key + (j + 1) * golden-gamma.
//   * Uniform: top 53 bits, offset by half a step, so u lies in (0, 1).
//   * Normal: Box-Muller, z = sqrt(-2 ln u1) cos(2 pi u2), with ln, cos,
//     exp and sqrt written below from their series / Newton definitions.
//   * Student-t with 3 degrees of freedom: z0 / sqrt((z1^2+z2^2+z3^2)/3).
#include <hip/hip_runtime.h>

#include <cstdint>

#pragma clang fp contract(off)

extern "C" {
struct synth_recipe {
    uint64_t key;          // stream key of this tensor
    int32_t kind;          // SYNTH_NORMAL, SYNTH_T3, SYNTH_T3_SQUARED, SYNTH_EXPERT_LOGU, SYNTH_ZERO
    int32_t reserved;
    double scale;          // sigma of the normal / multiplier of the t draw
    double logu_lo;        // kind SYNTH_EXPERT_LOGU: per-expert factor 10^U(lo, hi)
    double logu_hi;
    uint64_t expert_key;   // stream of per-expert factors (shared by an expert's tensors)
    double zero_tile_prob; // > 0: 128x128 tiles drawn with this probability are all zero
    uint64_t zero_key;     // stream of those draws (shared by the tensors of one weight)
    int64_t H, W;          // shape of one expert: element (e, r, c) has index (e H + r) W + c
};
}

enum { SYNTH_NORMAL = 0, SYNTH_T3 = 1, SYNTH_T3_SQUARED = 2, SYNTH_EXPERT_LOGU = 3, SYNTH_ZERO = 4 };

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr double kLn2 = 0.6931471805599453;
constexpr double kLn10 = 2.302585092994046;
constexpr double kTwoPi = 6.283185307179586;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__host__ __device__ inline double uniform(uint64_t key, uint64_t j) {
    uint64_t z = mix64(key + (j + 1) * kGamma);
    return ((double)(z >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

__host__ __device__ inline double bits_to_double(uint64_t b) {
    union { uint64_t u; double d; } x;
    x.u = b;
    return x.d;
}

__host__ __device__ inline uint64_t double_to_bits(double d) {
    union { uint64_t u; double d; } x;
    x.d = d;
    return x.u;
}

// ln x for a normal x > 0: x = m 2^e with m in [sqrt(1/2), sqrt(2)), then
// ln m = 2 artanh(s), s = (m-1)/(m+1), as its odd power series.
__host__ __device__ inline double ln_pos(double x) {
    uint64_t b = double_to_bits(x);
    int64_t e = (int64_t)((b >> 52) & 0x7FF) - 1023;
    double m = bits_to_double((b & 0xFFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
    if (m > 1.4142135623730951) {
        m = m * 0.5;
        e = e + 1;
    }
    double s = (m - 1.0) / (m + 1.0);
    double s2 = s * s;
    double poly = 1.0 / 23.0;
    poly = poly * s2 + 1.0 / 21.0;
    poly = poly * s2 + 1.0 / 19.0;
    poly = poly * s2 + 1.0 / 17.0;
    poly = poly * s2 + 1.0 / 15.0;
    poly = poly * s2 + 1.0 / 13.0;
    poly = poly * s2 + 1.0 / 11.0;
    poly = poly * s2 + 1.0 / 9.0;
    poly = poly * s2 + 1.0 / 7.0;
    poly = poly * s2 + 1.0 / 5.0;
    poly = poly * s2 + 1.0 / 3.0;
    poly = poly * s2 + 1.0;
    return (double)e * kLn2 + 2.0 * s * poly;
}

// 1/n! for n = 0..22: 1/n! = (1/(n-1)!) / n, one correctly rounded division
// per step, evaluated once at compile time into a table (a recursive
// constexpr call in a plain expression is not guaranteed to fold, and the
// host build did evaluate it at run time, ~20 divisions per use).
struct InvFactTable {
    double v[23];
    constexpr InvFactTable() : v() {
        v[0] = 1.0;
        v[1] = 1.0;
        for (int n = 2; n < 23; ++n) v[n] = v[n - 1] / (double)n;
    }
};
constexpr InvFactTable kInvFact{};
__host__ __device__ constexpr double inv_fact(int n) { return kInvFact.v[n]; }

// exp x for |x| < 700: x = k ln2 + r, |r| <= ln2/2, Taylor series of e^r
// (Horner form, degree 22).
__host__ __device__ inline double exp_small(double x) {
    double kf = x / kLn2;
    int64_t k = (int64_t)(kf < 0.0 ? kf - 0.5 : kf + 0.5);
    double r = x - (double)k * kLn2;
    double sum = inv_fact(22);
#pragma unroll
    for (int n = 21; n >= 0; --n) sum = sum * r + inv_fact(n);
    return sum * bits_to_double((uint64_t)(k + 1023) << 52);
}

// Newton's iteration for sqrt a, a > 0, from the exponent-halved guess.
__host__ __device__ inline double sqrt_pos(double a) {
    uint64_t b = double_to_bits(a);
    int64_t e = (int64_t)((b >> 52) & 0x7FF) - 1023;
    double y = bits_to_double((uint64_t)((e / 2) + 1023) << 52);
    for (int n = 0; n < 7; ++n) y = 0.5 * (y + a / y);
    return y;
}

// cos(2 pi u), u in [0, 1): reduce to the nearest quarter turn, then the
// Taylor series of sin / cos on [-pi/4, pi/4] (Horner form, to x^18 / x^19).
__host__ __device__ inline double cos_turns(double u) {
    int64_t n = (int64_t)(4.0 * u + 0.5);
    double x = (u - 0.25 * (double)n) * kTwoPi;
    double x2 = x * x;
    double c = inv_fact(18), s = -inv_fact(19);
#pragma unroll
    for (int k = 8; k >= 0; --k) {
        const double sign = (k & 1) ? -1.0 : 1.0;
        c = c * x2 + sign * inv_fact(2 * k);
        s = s * x2 + sign * inv_fact(2 * k + 1);
    }
    s = s * x;
    switch (n & 3) {
        case 0: return c;
        case 1: return -s;
        case 2: return -c;
        default: return s;
    }
}

__host__ __device__ inline double normal(uint64_t key, uint64_t j) {
    double u1 = uniform(key, 2 * j), u2 = uniform(key, 2 * j + 1);
    return sqrt_pos(-2.0 * ln_pos(u1)) * cos_turns(u2);
}

__host__ __device__ inline double student_t3(uint64_t key, uint64_t j) {
    double z0 = normal(key, 4 * j), z1 = normal(key, 4 * j + 1);
    double z2 = normal(key, 4 * j + 2), z3 = normal(key, 4 * j + 3);
    double chi = (z1 * z1 + z2 * z2 + z3 * z3) / 3.0;
    return z0 / sqrt_pos(chi);
}

// Whether the 128x128 tile (e, ti, tj) of the tensor is drawn all zero.
__host__ __device__ inline bool zero_tile(const synth_recipe& r, int64_t e, int64_t ti, int64_t tj) {
    const int64_t wb = (r.W + 127) / 128, hb = (r.H + 127) / 128;
    return uniform(r.zero_key, (uint64_t)((e * hb + ti) * wb + tj)) < r.zero_tile_prob;
}

// Value k ignoring the zero tiles.
__host__ __device__ inline float value_raw(const synth_recipe& r, int64_t k) {
    const int64_t per_expert = r.H * r.W;
    double v;
    switch (r.kind) {
        case SYNTH_NORMAL: v = r.scale * normal(r.key, (uint64_t)k); break;
        case SYNTH_T3: v = r.scale * student_t3(r.key, (uint64_t)k); break;
        case SYNTH_T3_SQUARED: {
            double t = r.scale * student_t3(r.key, (uint64_t)k);
            v = t * t;
            break;
        }
        case SYNTH_EXPERT_LOGU: {
            int64_t e = k / per_expert;
            double u = uniform(r.expert_key, (uint64_t)e);
            double lg = r.logu_lo + (r.logu_hi - r.logu_lo) * u;
            v = exp_small(lg * kLn10) * normal(r.key, (uint64_t)k);
            break;
        }
        default: v = 0.0; break;
    }
    return (float)v;
}

__host__ __device__ inline float value_at(const synth_recipe& r, int64_t k) {
    if (r.zero_tile_prob > 0.0) {
        const int64_t per_expert = r.H * r.W;
        const int64_t e = k / per_expert, rem = k - e * per_expert;
        const int64_t row = rem / r.W, col = rem - row * r.W;
        if (zero_tile(r, e, row / 128, col / 128)) return 0.0f;
    }
    return value_raw(r, k);
}

__global__ void fill_kernel(float* __restrict__ out, int64_t lo, int64_t n, synth_recipe r) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride)
        out[t] = value_at(r, lo + t);
}

}  // namespace

extern "C" {

uint64_t synth_key(uint64_t seed, uint64_t config, uint64_t array, uint64_t param, uint64_t step) {
    uint64_t h = mix64(seed + kGamma);
    h = mix64(h + config + kGamma);
    h = mix64(h + array + kGamma);
    h = mix64(h + param + kGamma);
    return mix64(h + step + kGamma);
}

double synth_uniform(uint64_t key, uint64_t j) { return uniform(key, j); }
double synth_normal(uint64_t key, uint64_t j) { return normal(key, j); }
double synth_student_t3(uint64_t key, uint64_t j) { return student_t3(key, j); }
double synth_ln(double x) { return ln_pos(x); }
double synth_exp(double x) { return exp_small(x); }
double synth_sqrt(double x) { return sqrt_pos(x); }
double synth_cos_turns(double u) { return cos_turns(u); }

// Host: out[k - lo] = value k, k in [lo, hi).
int synth_fill_host(float* out, int64_t lo, int64_t hi, const synth_recipe* r) {
    if (!out || !r || lo < 0 || hi < lo || r->H < 1 || r->W < 1) return -1;
    for (int64_t k = lo; k < hi; ++k) out[k - lo] = value_at(*r, k);
    return 0;
}

// Host: the rectangle rows [r0, r0+nr) x cols [c0, c0+nc) of expert e,
// row-major into out (nr x nc).
int synth_fill_rect_host(float* out, int64_t e, int64_t r0, int64_t nr, int64_t c0, int64_t nc,
                         const synth_recipe* r) {
    if (!out || !r || e < 0 || r0 < 0 || c0 < 0 || nr < 0 || nc < 0 || r0 + nr > r->H ||
        c0 + nc > r->W)
        return -1;
    // a rectangle inside one tile (the oracle's per-slot draws) decides the
    // tile's zero draw once
    const bool one_tile = nr > 0 && nc > 0 && r0 / 128 == (r0 + nr - 1) / 128 &&
                          c0 / 128 == (c0 + nc - 1) / 128;
    if (one_tile && r->zero_tile_prob > 0.0) {
        const bool zero = zero_tile(*r, e, r0 / 128, c0 / 128);
        for (int64_t a = 0; a < nr; ++a)
            for (int64_t b = 0; b < nc; ++b)
                out[a * nc + b] = zero ? 0.0f : value_raw(*r, (e * r->H + r0 + a) * r->W + c0 + b);
        return 0;
    }
    for (int64_t a = 0; a < nr; ++a)
        for (int64_t b = 0; b < nc; ++b)
            out[a * nc + b] = value_at(*r, (e * r->H + r0 + a) * r->W + c0 + b);
    return 0;
}

// Device: out[k - lo] = value k, k in [lo, hi), on the given stream.
int synth_fill_device(float* out, int64_t lo, int64_t hi, const synth_recipe* r, void* stream) {
    if (!out || !r || lo < 0 || hi < lo || r->H < 1 || r->W < 1) return -1;
    int64_t n = hi - lo;
    if (n == 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       out, lo, n, *r);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
