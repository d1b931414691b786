/*
 * synth.c -- seeded, counter-based synthetic input generator.
 *
 * This module only makes input bits.  It holds none of the MoE layer's
 * arithmetic: no gate, no routing, no FFN, no activation quantiser.  Both
 * sides of every parity check (the fp64 CPU oracle and the HIP path) are fed
 * the identical arrays it writes, so it is the only code they share.
 *
 * Generator definition
 *   mix64(z)     : the SplitMix64 output function (Steele, Lea and Flood,
 *                  "Fast splittable pseudorandom number generators",
 *                  OOPSLA 2014): two xor-shift-multiply rounds and a final
 *                  xor-shift.
 *   key          : mix64 chain over (seed, tensor id, sub-stream id); the
 *                  sub-stream is the expert id for per-expert weights, so one
 *                  expert can be regenerated alone.
 *   draw(key, i) : mix64(key + (i + 1) * 0x9E3779B97F4A7C15) -- the i-th
 *                  64-bit word of the stream, independent of every other.
 *   uniform      : (draw >> 11) * 2^-53 in [0, 1).
 *   normal       : Box-Muller on the pair (2p, 2p+1): u1 = ((w >> 11) + 1)
 *                  * 2^-53 in (0, 1], u2 uniform, r = sqrt(-2 ln u1); element
 *                  2p gets r cos(2 pi u2), element 2p+1 gets r sin(2 pi u2).
 *   storage      : value in double -> float (round to nearest even) -> for
 *                  bf16 tensors, the upper 16 bits after round-to-nearest-even
 *                  on the float bits.
 *
 * Because every element is a pure function of (seed, tensor, sub, index),
 * the result does not depend on the number of threads or on chunking.
 *
 * FP8 weights (e4m3 with one fp32 scale per 128x128 block) are made here as
 * stored layer weights: the block's float values v are drawn as above, then
 * a = max|v| over the block, scale = a / 448 (rounded to float), and each
 * code is the OCP e4m3fn value nearest v * (448 / a) (ties to even
 * mantissa, saturated at 448).  With pow2 set the block scale is instead the
 * smallest power of two 2^e >= a / 448 and the codes are the e4m3 values
 * nearest v * 2^-e (the weights of the power-of-two-scale FP8 variant).
 * This is weight preparation only; the layer's activation quantiser lives
 * separately in the oracle and in the kernels.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint32_t tensor, uint32_t sub)
{
    uint64_t k = mix64(seed ^ GOLDEN);
    k = mix64(k + ((uint64_t)tensor + 1) * GOLDEN);
    k = mix64(k + ((uint64_t)sub + 1) * 0xD1B54A32D192ED03ULL);
    return k;
}

static inline uint64_t draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GOLDEN);
}

static inline double unit53(uint64_t w)
{
    return (double)(w >> 11) * 0x1.0p-53;
}

/* Both normals of pair p. */
static inline void normal_pair(uint64_t key, uint64_t p, double *z0, double *z1)
{
    double u1 = (double)((draw(key, 2 * p) >> 11) + 1) * 0x1.0p-53;
    double u2 = unit53(draw(key, 2 * p + 1));
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925 * u2;
    *z0 = r * cos(a);
    *z1 = r * sin(a);
}

static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) /* NaN */
        return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Normal values (std * z) as float, elements [0, n) of the stream. */
void synth_normal_f32(float *out, int64_t n, uint64_t seed, uint32_t tensor,
                      uint32_t sub, double std)
{
    uint64_t key = stream_key(seed, tensor, sub);
    int64_t npair = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npair; ++p) {
        double z0, z1;
        normal_pair(key, (uint64_t)p, &z0, &z1);
        out[2 * p] = (float)(std * z0);
        if (2 * p + 1 < n)
            out[2 * p + 1] = (float)(std * z1);
    }
}

/* Same stream as synth_normal_f32, stored as bf16 bits. */
void synth_normal_bf16(uint16_t *out, int64_t n, uint64_t seed, uint32_t tensor,
                       uint32_t sub, double std)
{
    uint64_t key = stream_key(seed, tensor, sub);
    int64_t npair = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npair; ++p) {
        double z0, z1;
        normal_pair(key, (uint64_t)p, &z0, &z1);
        out[2 * p] = f32_to_bf16_rne((float)(std * z0));
        if (2 * p + 1 < n)
            out[2 * p + 1] = f32_to_bf16_rne((float)(std * z1));
    }
}

/* Uniform values lo + (hi - lo) * u as float. */
void synth_uniform_f32(float *out, int64_t n, uint64_t seed, uint32_t tensor,
                       uint32_t sub, double lo, double hi)
{
    uint64_t key = stream_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(lo + (hi - lo) * unit53(draw(key, (uint64_t)i)));
}

/* Raw 64-bit words of a stream (used for seeded integer test inputs). */
void synth_words(uint64_t *out, int64_t n, uint64_t seed, uint32_t tensor,
                 uint32_t sub)
{
    uint64_t key = stream_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = draw(key, (uint64_t)i);
}

/* ---- e4m3 weight preparation (generator-side encoder) ------------------ */

/* Nearest OCP e4m3fn code to float v, ties to even mantissa, saturated at
 * +-448.  Normal range (|v| >= 2^-6): round the 23-bit float mantissa to 3
 * bits on the float's bit pattern; a carry moves into the exponent field as
 * it should.  Below 2^-6 the code is the subnormal count |v| * 2^9 rounded
 * to nearest even (8 there is the smallest normal, code 0x08). */
static uint8_t e4m3_encode_gen(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    uint8_t s = (uint8_t)((u >> 24) & 0x80);
    u &= 0x7FFFFFFFu;
    float a;
    memcpy(&a, &u, 4);
    if (!(a < 448.0f))
        return s | 0x7E;
    int e = (int)(u >> 23) - 127;
    if (e >= -6) {
        uint32_t m = u & 0x7FFFFFu;
        uint32_t code = ((uint32_t)(e + 7) << 3) | (m >> 20);
        uint32_t rem = m & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (code & 1u)))
            code += 1;
        if (code > 0x7Eu)
            code = 0x7E;
        return s | (uint8_t)code;
    }
    double sub = rint((double)a * 512.0); /* exact scaling; rint is RNE */
    return s | (uint8_t)sub;
}

/* Matrix [rows, cols] (rows, cols multiples of 128) drawn like
 * synth_normal_f32 (element r*cols + c of the stream), then stored as e4m3
 * codes q[rows*cols] with block scales s[(rows/128) * (cols/128)]. */
/* Power-of-two block scale for a block with max |v| = amax > 0: the
 * smallest 2^e not below amax / 448, e in [-126, 127]. */
static int gen_pow2_exponent(float amax)
{
    double r = (double)amax / 448.0;
    int e = (int)ceil(log2(r));
    while (e > -126 && ldexp(1.0, e - 1) >= r)
        --e;
    while (ldexp(1.0, e) < r)
        ++e;
    if (e < -126)
        e = -126;
    if (e > 127)
        e = 127;
    return e;
}

void synth_normal_e4m3_blocks(uint8_t *q, float *s, int64_t rows, int64_t cols,
                              uint64_t seed, uint32_t tensor, uint32_t sub,
                              double std, int pow2)
{
    uint64_t key = stream_key(seed, tensor, sub);
    int64_t rb = rows / 128, cb = cols / 128;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < rb * cb; ++b) {
        int64_t r0 = (b / cb) * 128, c0 = (b % cb) * 128;
        static __thread float blk[128 * 128];
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            for (int j = 0; j < 128; j += 2) {
                uint64_t idx = (uint64_t)((r0 + i) * cols + c0 + j);
                double z0, z1;
                normal_pair(key, idx >> 1, &z0, &z1); /* cols even: j, j+1 pair */
                float v0 = (float)(std * z0), v1 = (float)(std * z1);
                blk[i * 128 + j] = v0;
                blk[i * 128 + j + 1] = v1;
                float a0 = fabsf(v0), a1 = fabsf(v1);
                if (a0 > amax) amax = a0;
                if (a1 > amax) amax = a1;
            }
        }
        float scale = 1.0f, inv = 0.0f;
        if (amax > 0.0f && pow2) {
            int e = gen_pow2_exponent(amax);
            scale = (float)ldexp(1.0, e);
            inv = (float)ldexp(1.0, -e);
        } else if (amax > 0.0f) {
            scale = (float)((double)amax / 448.0);
            inv = (float)(448.0 / (double)amax);
        }
        s[b] = scale;
        for (int i = 0; i < 128; ++i)
            for (int j = 0; j < 128; ++j)
                q[(r0 + i) * cols + c0 + j] = e4m3_encode_gen(blk[i * 128 + j] * inv);
    }
}
