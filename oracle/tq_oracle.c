/*
 * tq_oracle.c -- plain, slow, obviously correct CPU reference for the
 * packed-ternary x q8_K matrix-vector / small-batch matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg.  It shares no code, header or table with the
 * GPU library.
 *
 * Every function follows the plain definition of what the method computes,
 * with no slot masking, no u-then-correct trick and no repacked layout:
 *
 *   pq2_0 decode   "how i made a 27b ternary model 3.8x faster..." (page 1),
 *                  section "what's running": 2-bit code u = w + 1, four per
 *                  byte, one fp16 scale per 128 weights.  Bit order inside a
 *                  byte: weight k of a group sits in byte k>>2 at bits
 *                  2*(k&3)..+1, low bits first, the order in which the pages'
 *                  packer ("the layout") shifts code s by 2*s.
 *   ptq1_0 decode  page 1, "the detour that lost", and the ciot README
 *                  (page 2), ptq1_0 paragraph: trit k of byte b is
 *                  floor(3 * ((b * 3^k) mod 256) / 256), weight = trit - 1.
 *                  Block: fp16 d then 26 bytes; weight k is trit k%5 of byte
 *                  k/5 (the two trits past 128 are padding).
 *   q8_K           page 2 intro: 256 int8 values, one float scale and 16
 *                  partial sums per block.  Scale d = max|x| / 127 in fp32,
 *                  q = round-to-nearest-even(x / d), partial sums over 16
 *                  consecutive values.
 *   group dot      page 1, "the trick with 4 and 16": integer dot per 128
 *                  weights, exact in int32, float scales applied afterwards.
 *   float output   y = sum over groups of d_w * d_x * I, every term exact in
 *                  fp64, summed in ascending group order in fp64, rounded to
 *                  fp32 once (the pages only say the float math "can round
 *                  differently"; this is the reading that makes the result a
 *                  well-defined function of the inputs).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off (no -ffast-math:
 * the q8_K rounding must be IEEE).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define TQO_FMT_PQ2_0 1
#define TQO_FMT_PTQ1_0 2
#define TQO_GROUP 128
#define TQO_QBLOCK 256

/* IEEE 754 binary16 -> binary32, written out from the format's definition:
 * sign, 5-bit exponent (bias 15), 10-bit fraction; subnormals, inf, NaN. */
float tqo_half_to_float(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    float v;
    if (expo == 0) {
        v = ldexpf((float)frac, -24); /* 0.frac * 2^-14 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(frac | 0x400), expo - 25); /* 1.frac * 2^(e-15) */
    }
    return sign ? -v : v;
}

static float block_scale(const uint8_t *blk)
{
    const uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8)); /* little-endian fp16 */
    return tqo_half_to_float(h);
}

/* Decode one 34-byte pq2_0 block into w[128] in {-1, 0, 1} (and 2 for the
 * unused code 3, decoded literally as u - 1).  Returns the number of codes
 * equal to 3. */
int tqo_decode_pq2_block(const uint8_t *blk, int8_t *w, float *d)
{
    const uint8_t *qs = blk + 2;
    int bad = 0;
    for (int k = 0; k < TQO_GROUP; ++k) {
        const int u = (qs[k >> 2] >> (2 * (k & 3))) & 3;
        if (u == 3)
            ++bad;
        w[k] = (int8_t)(u - 1);
    }
    *d = block_scale(blk);
    return bad;
}

/* Decode one 28-byte ptq1_0 block into w[128] in {-1, 0, 1}. */
int tqo_decode_ptq1_block(const uint8_t *blk, int8_t *w, float *d)
{
    static const int pow3[5] = {1, 3, 9, 27, 81};
    const uint8_t *qs = blk + 2;
    for (int k = 0; k < TQO_GROUP; ++k) {
        const int b = qs[k / 5];
        const int j = k % 5;
        const int v = (b * pow3[j]) % 256;  /* b * 3^j mod 256 */
        const int trit = (3 * v) / 256;     /* floor(3 v / 256) in {0,1,2} */
        w[k] = (int8_t)(trit - 1);
    }
    *d = block_scale(blk);
    return 0;
}

static int block_bytes(int fmt)
{
    return fmt == TQO_FMT_PQ2_0 ? 34 : (fmt == TQO_FMT_PTQ1_0 ? 28 : 0);
}

static int decode_block(int fmt, const uint8_t *blk, int8_t *w, float *d)
{
    return fmt == TQO_FMT_PQ2_0 ? tqo_decode_pq2_block(blk, w, d) : tqo_decode_ptq1_block(blk, w, d);
}

/* Decode rows [r0, r1) of a canonical matrix into w[(r - r0) * cols + k] and
 * d[(r - r0) * (cols/128) + g].  Returns the count of invalid codes. */
int64_t tqo_decode_rows(int fmt, const uint8_t *W, int64_t cols, int64_t r0, int64_t r1, int8_t *w, float *d)
{
    const int bb = block_bytes(fmt);
    const int64_t G = cols / TQO_GROUP;
    int64_t bad = 0;
    if (!bb)
        return -1;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t g = 0; g < G; ++g)
            bad += decode_block(fmt, W + (r * G + g) * bb, w + (r - r0) * cols + g * TQO_GROUP, d + (r - r0) * G + g);
    return bad;
}

/* q8_K quantization of one token's activations x[cols] (cols % 256 == 0).
 * Per block of 256: amax = max |x|; d = amax / 127 (fp32 division);
 * if d == 0 every q is 0, else q = rint(x / d) (fp32 division, ties to even)
 * clamped to [-127, 127]; bsums[j] = sum of q over values 16j .. 16j+15. */
void tqo_quantize_q8k(const float *x, int64_t cols, int8_t *q, float *d, int16_t *bsums)
{
    for (int64_t b = 0; b < cols / TQO_QBLOCK; ++b) {
        const float *xb = x + b * TQO_QBLOCK;
        int8_t *qb = q + b * TQO_QBLOCK;
        float amax = 0.0f;
        for (int i = 0; i < TQO_QBLOCK; ++i) {
            const float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        const volatile float dv = amax / 127.0f; /* keep the fp32 rounding explicit */
        const float db = dv;
        d[b] = db;
        for (int i = 0; i < TQO_QBLOCK; ++i) {
            int v = 0;
            if (db != 0.0f) {
                const volatile float ratio = xb[i] / db;
                float r = rintf(ratio);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                v = (int)r;
            }
            qb[i] = (int8_t)v;
        }
        for (int j = 0; j < TQO_QBLOCK / 16; ++j) {
            int s = 0;
            for (int i = 0; i < 16; ++i)
                s += qb[16 * j + i];
            bsums[b * (TQO_QBLOCK / 16) + j] = (int16_t)s;
        }
    }
}

/* Quantize tokens [t0, t1) of x[tokens][cols]. */
void tqo_quantize_rows(const float *x, int64_t cols, int64_t t0, int64_t t1, int8_t *q, float *d, int16_t *bsums)
{
    for (int64_t t = t0; t < t1; ++t)
        tqo_quantize_q8k(x + t * cols, cols, q + t * cols, d + t * (cols / TQO_QBLOCK), bsums + t * (cols / 16));
}

/* Exact integer group dots I[t][r][g] = sum_{k<128} w[r][128g+k] * q[t][128g+k]
 * for rows [r0, r1) and every token; written to I[t][r - r0][g] with row
 * stride (r1 - r0).  Accumulated in int64; returns 1 if any value would not
 * fit int32, else 0. */
int tqo_group_dots(int fmt, const uint8_t *W, int64_t cols, int64_t tokens, const int8_t *q, int64_t r0, int64_t r1, int32_t *I)
{
    const int bb = block_bytes(fmt);
    const int64_t G = cols / TQO_GROUP;
    const int64_t nr = r1 - r0;
    int overflow = 0;
    int8_t w[TQO_GROUP];
    float dw;
    if (!bb)
        return -1;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t g = 0; g < G; ++g) {
            decode_block(fmt, W + (r * G + g) * bb, w, &dw);
            for (int64_t t = 0; t < tokens; ++t) {
                const int8_t *qt = q + t * cols + g * TQO_GROUP;
                int64_t s = 0;
                for (int k = 0; k < TQO_GROUP; ++k)
                    s += (int64_t)w[k] * (int64_t)qt[k];
                if (s > INT32_MAX || s < INT32_MIN)
                    overflow = 1;
                I[(t * nr + (r - r0)) * G + g] = (int32_t)s;
            }
        }
    }
    return overflow;
}

/* Float output y[t][r] for rows [r0, r1), written at y[t * ystride + (r - r0)]:
 *   y = fl32( sum_g  (double)d_w[r][g] * (double)d_x[t][g/2] * (double)I[t][r][g] )
 * with the product exact in fp64 and the sum taken in ascending g in fp64.
 * If mag is non-null, mag[t * ystride + (r - r0)] = sum_g |term_g| (fp64), the
 * magnitude against which a zero output is judged. */
int tqo_matmul(int fmt, const uint8_t *W, int64_t cols, int64_t tokens, const int8_t *q, const float *dx, int64_t r0, int64_t r1,
               float *y, double *mag, int64_t ystride)
{
    const int bb = block_bytes(fmt);
    const int64_t G = cols / TQO_GROUP;
    const int64_t B = cols / TQO_QBLOCK;
    int8_t w[TQO_GROUP];
    float dw;
    if (!bb)
        return -1;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t t = 0; t < tokens; ++t) {
            double acc = 0.0, m = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                decode_block(fmt, W + (r * G + g) * bb, w, &dw);
                const int8_t *qt = q + t * cols + g * TQO_GROUP;
                int64_t s = 0;
                for (int k = 0; k < TQO_GROUP; ++k)
                    s += (int64_t)w[k] * (int64_t)qt[k];
                const double term = ((double)dw * (double)dx[t * B + g / 2]) * (double)s;
                acc += term;
                m += fabs(term);
            }
            y[t * ystride + (r - r0)] = (float)acc;
            if (mag)
                mag[t * ystride + (r - r0)] = m;
        }
    }
    return 0;
}
