/*
 * VBQ CPU ORACLE -- test infrastructure only.
 *
 * This file is the plain, slow, obviously-correct CPU statement of what the
 * VBQ decode path computes.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the GPU library never links,
 * includes or calls it, and it includes nothing from the GPU library.
 *
 * What it follows:
 *   - "Variable Bit-width Quantization" (mlsanity.com page, Abstract): every
 *     contiguous group of 64 weights carries its own bit-width from
 *     {1, 2, 4, 8}; the recipe is stored as packed low-bit codes and decode
 *     multiplies by the dequantized weights ("fused dequantize-and-multiply").
 *   - The pages give no dequant rule, scale format, bit order or byte layout.
 *     The build fixes them (readings, not page facts):
 *       * one fp16 scale s per group, code q in [0, 2^b - 1],
 *         w = s * (q - (2^b - 1) / 2)          (symmetric, no zero level);
 *       * groups run along K (the reduction axis);
 *       * the packed layout "VBQ1" described next.
 *
 * Packed layout VBQ1 (all integers little-endian):
 *   header, 256 bytes at offset 0:
 *     u32 magic 0x31514256, u32 version 1, u32 N, u32 K, u32 G = K/64,
 *     u32 S = 32 (groups per K-slice), u32 nS = ceil(G/32), u32 row_pad = 128,
 *     u64 off_row_off, off_slice_off, off_wmap, off_scales, off_codes,
 *     u64 total_bytes, u64 code_bytes (sum of 8*b over groups),
 *     u64 code_bytes_padded (128 * row_off[N]); the rest is zero.
 *   sections, each at a 256-byte aligned offset, in this order:
 *     row_off   u32[N+1]   start of row n's code record, in 128-byte units
 *     slice_off u32[N][nS] byte offset of slice t inside row n's record
 *     wmap      u32[N][nS][2] two bit planes: bit i (group 32t+i) of plane 0
 *                           is bit 0 of log2(b), of plane 1 is bit 1; bits of
 *                           groups past G are zero
 *     scales    u16[N][G]  fp16 bit patterns, natural group order
 *     codes     row records, each padded with zero bytes to a 128 multiple
 *   row record: slices t = 0..nS-1 in order; inside a slice the groups are
 *   bucketed by width (all 1-bit groups, then 2-, 4-, 8-bit), ascending g
 *   inside a bucket; a b-bit group takes 8*b bytes.
 *   group encoding: the 64 codes are split into halves H0 = codes 0..31 and
 *   H1 = codes 32..63; each half is packed LSB-first into a string of 2*b
 *   16-bit units (code j of the half at bit j*b); 32-bit word d of the group
 *   (d = 0..2b-1) is H0 unit d in its low 16 bits and H1 unit d in its high
 *   16 bits.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define VBQO_OK 0
#define VBQO_ERR_SHAPE (-1)
#define VBQO_ERR_BITS (-2)
#define VBQO_ERR_CODE (-3)
#define VBQO_ERR_LAYOUT (-4)
#define VBQO_ERR_SIZE (-5)

#define MAGIC 0x31514256u

/* ---- fp16 <-> double, written from the IEEE 754 binary16 definition ---- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double vbqo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even; overflow gives inf. */
uint16_t vbqo_f64_to_f16_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(a))
        return (uint16_t)(sign | 0x7c00);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1; /* a in [2^E, 2^(E+1)) */
    if (E < -14)
        E = -14; /* subnormal range shares the 2^-24 quantum */
    double quantum = ldexp(1.0, E - 10);
    double n = a / quantum; /* exact: scaling by a power of two */
    double r = floor(n);
    double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    double rounded = r * quantum;
    if (rounded > 65504.0)
        return (uint16_t)(sign | 0x7c00);
    /* rebuild the bit pattern from the rounded value */
    if (rounded < ldexp(1.0, -14)) {
        return (uint16_t)(sign | (uint16_t)(rounded / ldexp(1.0, -24)));
    }
    int e2;
    frexp(rounded, &e2);
    int E2 = e2 - 1;
    uint16_t frac_bits = (uint16_t)(rounded / ldexp(1.0, E2 - 10) - 1024.0);
    return (uint16_t)(sign | ((E2 + 15) << 10) | frac_bits);
}

/* ---- layout arithmetic ---- */

static uint64_t align256(uint64_t x) { return (x + 255u) & ~(uint64_t)255u; }

static int valid_width(int b) { return b == 1 || b == 2 || b == 4 || b == 8; }

static int log2_width(int b) { return b == 1 ? 0 : b == 2 ? 1 : b == 4 ? 2 : 3; }

static int check_shape(int N, int K)
{
    if (N < 1 || K < 64 || (K % 64) != 0)
        return VBQO_ERR_SHAPE;
    return VBQO_OK;
}

/*
 * Header fields for an N x K matrix with the given widths (bits[N][G]).
 * hdr receives 14 u64 values: N, K, G, S, nS, off_row_off, off_slice_off,
 * off_wmap, off_scales, off_codes, total_bytes, code_bytes,
 * code_bytes_padded, row_pad.
 */
int vbqo_layout(int N, int K, const uint8_t *bits, uint64_t *hdr)
{
    int rc = check_shape(N, K);
    if (rc)
        return rc;
    uint64_t G = (uint64_t)K / 64, S = 32, nS = (G + S - 1) / S;
    uint64_t code_bytes = 0, padded_units = 0;
    for (int n = 0; n < N; n++) {
        uint64_t row = 0;
        for (uint64_t g = 0; g < G; g++) {
            int b = bits[(uint64_t)n * G + g];
            if (!valid_width(b))
                return VBQO_ERR_BITS;
            row += 8u * (uint64_t)b;
        }
        code_bytes += row;
        padded_units += (row + 127) / 128;
    }
    uint64_t off_row_off = 256;
    uint64_t off_slice_off = align256(off_row_off + 4u * ((uint64_t)N + 1));
    uint64_t off_wmap = align256(off_slice_off + 4u * (uint64_t)N * nS);
    uint64_t off_scales = align256(off_wmap + 8u * (uint64_t)N * nS);
    uint64_t off_codes = align256(off_scales + 2u * (uint64_t)N * G);
    hdr[0] = (uint64_t)N;
    hdr[1] = (uint64_t)K;
    hdr[2] = G;
    hdr[3] = S;
    hdr[4] = nS;
    hdr[5] = off_row_off;
    hdr[6] = off_slice_off;
    hdr[7] = off_wmap;
    hdr[8] = off_scales;
    hdr[9] = off_codes;
    hdr[10] = off_codes + 128u * padded_units;
    hdr[11] = code_bytes;
    hdr[12] = 128u * padded_units;
    hdr[13] = 128;
    return VBQO_OK;
}

static void put_u32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
    p[3] = (uint8_t)(v >> 24);
}

static void put_u64(uint8_t *p, uint64_t v)
{
    put_u32(p, (uint32_t)v);
    put_u32(p + 4, (uint32_t)(v >> 32));
}

static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static uint64_t get_u64(const uint8_t *p) { return (uint64_t)get_u32(p) | ((uint64_t)get_u32(p + 4) << 32); }

/* Bit position of code j (0..63) inside the 64*b-bit string of a b-bit group. */
static uint32_t code_bit_position(int j, int b)
{
    int half = j >= 32;
    int jj = j - 32 * half;
    uint32_t pos_in_half = (uint32_t)(jj * b); /* LSB-first inside the half */
    uint32_t unit = pos_in_half / 16, bit = pos_in_half % 16;
    /* word `unit`: low 16 bits from H0, high 16 bits from H1 */
    return unit * 32u + (uint32_t)half * 16u + bit;
}

/* Write the 8*b bytes of one group (codes q[0..63], width b). */
static void encode_group(const uint8_t *q, int b, uint8_t *out)
{
    memset(out, 0, (size_t)(8 * b));
    for (int j = 0; j < 64; j++) {
        uint32_t pos = code_bit_position(j, b);
        for (int i = 0; i < b; i++) {
            if ((q[j] >> i) & 1u) {
                uint32_t p = pos + (uint32_t)i;
                out[p / 8] |= (uint8_t)(1u << (p % 8));
            }
        }
    }
}

static void decode_group(const uint8_t *in, int b, uint8_t *q)
{
    for (int j = 0; j < 64; j++) {
        uint32_t pos = code_bit_position(j, b);
        uint32_t v = 0;
        for (int i = 0; i < b; i++) {
            uint32_t p = pos + (uint32_t)i;
            v |= (uint32_t)((in[p / 8] >> (p % 8)) & 1u) << i;
        }
        q[j] = (uint8_t)v;
    }
}

/*
 * Pack (q[N][K], bits[N][G], scales[N][G]) into blob (blob_bytes must equal
 * the layout's total_bytes).  Every byte of the blob is written.
 */
int vbqo_pack(int N, int K, const uint8_t *q, const uint8_t *bits, const uint16_t *scales, uint8_t *blob,
              uint64_t blob_bytes)
{
    uint64_t h[14];
    int rc = vbqo_layout(N, K, bits, h);
    if (rc)
        return rc;
    if (blob_bytes != h[10])
        return VBQO_ERR_SIZE;
    uint64_t G = h[2], nS = h[4];
    for (uint64_t n = 0; n < (uint64_t)N; n++)
        for (uint64_t g = 0; g < G; g++) {
            int b = bits[n * G + g];
            for (int j = 0; j < 64; j++)
                if (q[n * (uint64_t)K + 64 * g + (uint64_t)j] > (1u << b) - 1u)
                    return VBQO_ERR_CODE;
        }
    memset(blob, 0, (size_t)blob_bytes);
    put_u32(blob + 0, MAGIC);
    put_u32(blob + 4, 1);
    put_u32(blob + 8, (uint32_t)N);
    put_u32(blob + 12, (uint32_t)K);
    put_u32(blob + 16, (uint32_t)G);
    put_u32(blob + 20, 32);
    put_u32(blob + 24, (uint32_t)nS);
    put_u32(blob + 28, 128);
    for (int i = 0; i < 5; i++)
        put_u64(blob + 32 + 8 * i, h[5 + i]);
    put_u64(blob + 72, h[10]);
    put_u64(blob + 80, h[11]);
    put_u64(blob + 88, h[12]);

    uint8_t *row_off = blob + h[5], *slice_off = blob + h[6], *wmap = blob + h[7];
    uint8_t *sc = blob + h[8], *codes = blob + h[9];
    uint64_t unit = 0; /* running row start, 128-byte units */
    for (uint64_t n = 0; n < (uint64_t)N; n++) {
        put_u32(row_off + 4 * n, (uint32_t)unit);
        uint8_t *rec = codes + 128u * unit;
        uint64_t pos = 0;
        for (uint64_t t = 0; t < nS; t++) {
            put_u32(slice_off + 4 * (n * nS + t), (uint32_t)pos);
            uint64_t g0 = 32 * t, g1 = g0 + 32 < G ? g0 + 32 : G;
            uint32_t plane0 = 0, plane1 = 0;
            for (uint64_t g = g0; g < g1; g++) {
                int l = log2_width(bits[n * G + g]);
                plane0 |= (uint32_t)(l & 1) << (g - g0);
                plane1 |= (uint32_t)(l >> 1) << (g - g0);
            }
            put_u32(wmap + 8 * (n * nS + t), plane0);
            put_u32(wmap + 8 * (n * nS + t) + 4, plane1);
            for (int b = 1; b <= 8; b *= 2)
                for (uint64_t g = g0; g < g1; g++)
                    if (bits[n * G + g] == b) {
                        encode_group(q + n * (uint64_t)K + 64 * g, b, rec + pos);
                        pos += 8u * (uint64_t)b;
                    }
        }
        unit += (pos + 127) / 128;
        for (uint64_t g = 0; g < G; g++) {
            sc[2 * (n * G + g)] = (uint8_t)scales[n * G + g];
            sc[2 * (n * G + g) + 1] = (uint8_t)(scales[n * G + g] >> 8);
        }
    }
    put_u32(row_off + 4 * (uint64_t)N, (uint32_t)unit);
    return VBQO_OK;
}

/* Read the header; dims[0..1] receive N and K. */
int vbqo_header(const uint8_t *blob, uint64_t blob_bytes, uint64_t *hdr)
{
    if (blob_bytes < 256 || get_u32(blob) != MAGIC || get_u32(blob + 4) != 1)
        return VBQO_ERR_LAYOUT;
    hdr[0] = get_u32(blob + 8);
    hdr[1] = get_u32(blob + 12);
    hdr[2] = get_u32(blob + 16);
    hdr[3] = get_u32(blob + 20);
    hdr[4] = get_u32(blob + 24);
    for (int i = 0; i < 5; i++)
        hdr[5 + i] = get_u64(blob + 32 + 8 * i);
    hdr[10] = get_u64(blob + 72);
    hdr[11] = get_u64(blob + 80);
    hdr[12] = get_u64(blob + 88);
    hdr[13] = get_u32(blob + 28);
    if (hdr[10] != blob_bytes || check_shape((int)hdr[0], (int)hdr[1]) || hdr[2] != hdr[1] / 64 || hdr[3] != 32 ||
        hdr[4] != (hdr[2] + 31) / 32 || hdr[13] != 128)
        return VBQO_ERR_LAYOUT;
    return VBQO_OK;
}

/*
 * Unpack a blob back to q[N][K], bits[N][G], scales[N][G], reading it only
 * through the layout rules (row_off, slice_off, wmap, width buckets).
 */
int vbqo_unpack(const uint8_t *blob, uint64_t blob_bytes, uint8_t *q, uint8_t *bits, uint16_t *scales)
{
    uint64_t h[14];
    int rc = vbqo_header(blob, blob_bytes, h);
    if (rc)
        return rc;
    uint64_t N = h[0], K = h[1], G = h[2], nS = h[4];
    const uint8_t *row_off = blob + h[5], *slice_off = blob + h[6], *wmap = blob + h[7];
    const uint8_t *sc = blob + h[8], *codes = blob + h[9];
    for (uint64_t n = 0; n < N; n++) {
        const uint8_t *rec = codes + 128u * (uint64_t)get_u32(row_off + 4 * n);
        for (uint64_t t = 0; t < nS; t++) {
            const uint8_t *p = rec + get_u32(slice_off + 4 * (n * nS + t));
            uint32_t plane0 = get_u32(wmap + 8 * (n * nS + t));
            uint32_t plane1 = get_u32(wmap + 8 * (n * nS + t) + 4);
            uint64_t g0 = 32 * t, g1 = g0 + 32 < G ? g0 + 32 : G;
            for (uint64_t g = g0; g < g1; g++) {
                int l = (int)((plane0 >> (g - g0)) & 1u) | (int)(((plane1 >> (g - g0)) & 1u) << 1);
                bits[n * G + g] = (uint8_t)(1 << l);
            }
            for (int b = 1; b <= 8; b *= 2)
                for (uint64_t g = g0; g < g1; g++)
                    if (bits[n * G + g] == b) {
                        decode_group(p, b, q + n * K + 64 * g);
                        p += 8 * b;
                    }
        }
        for (uint64_t g = 0; g < G; g++)
            scales[n * G + g] = (uint16_t)(sc[2 * (n * G + g)] | (sc[2 * (n * G + g) + 1] << 8));
    }
    return VBQO_OK;
}

/* ---- dequant: w = s * (q - (2^b - 1)/2) ---- */

static int check_inputs(int N, int K, const uint8_t *q, const uint8_t *bits)
{
    int rc = check_shape(N, K);
    if (rc)
        return rc;
    uint64_t G = (uint64_t)K / 64;
    for (uint64_t n = 0; n < (uint64_t)N; n++)
        for (uint64_t g = 0; g < G; g++) {
            int b = bits[n * G + g];
            if (!valid_width(b))
                return VBQO_ERR_BITS;
            for (int j = 0; j < 64; j++)
                if (q[n * (uint64_t)K + 64 * g + (uint64_t)j] > (1u << b) - 1u)
                    return VBQO_ERR_CODE;
        }
    return VBQO_OK;
}

static double dequant_one(uint8_t q, int b, uint16_t s)
{
    double c = ((double)(1 << b) - 1.0) / 2.0;
    return vbqo_f16_to_f64(s) * ((double)q - c);
}

/* w[N][K] in fp32; the value is exact in fp32, so the cast does not round. */
int vbqo_dequant_f32(int N, int K, const uint8_t *q, const uint8_t *bits, const uint16_t *scales, float *w)
{
    int rc = check_inputs(N, K, q, bits);
    if (rc)
        return rc;
    uint64_t G = (uint64_t)K / 64;
    for (uint64_t n = 0; n < (uint64_t)N; n++)
        for (uint64_t k = 0; k < (uint64_t)K; k++)
            w[n * K + k] = (float)dequant_one(q[n * K + k], bits[n * G + k / 64], scales[n * G + k / 64]);
    return VBQO_OK;
}

/* w[N][K] as fp16 bit patterns, round-to-nearest-even of the exact value. */
int vbqo_dequant_f16(int N, int K, const uint8_t *q, const uint8_t *bits, const uint16_t *scales, uint16_t *w)
{
    int rc = check_inputs(N, K, q, bits);
    if (rc)
        return rc;
    uint64_t G = (uint64_t)K / 64;
    for (uint64_t n = 0; n < (uint64_t)N; n++)
        for (uint64_t k = 0; k < (uint64_t)K; k++)
            w[n * K + k] = vbqo_f64_to_f16_rne(dequant_one(q[n * K + k], bits[n * G + k / 64], scales[n * G + k / 64]));
    return VBQO_OK;
}

/*
 * y[m][n] = sum_k w[n][k] * x[m][k] in fp64 and bound[m][n] = sum_k |w||x|.
 * x is fp16 bit patterns with row stride ldx; y and bound are [M][N].
 * Each product is exact in fp64 (at most 19 + 11 significant bits).
 */
int vbqo_gemv(int N, int K, int M, const uint8_t *q, const uint8_t *bits, const uint16_t *scales, const uint16_t *x,
              int ldx, double *y, double *bound)
{
    int rc = check_inputs(N, K, q, bits);
    if (rc)
        return rc;
    if (M < 1 || ldx < K)
        return VBQO_ERR_SHAPE;
    uint64_t G = (uint64_t)K / 64;
    for (int m = 0; m < M; m++)
        for (uint64_t n = 0; n < (uint64_t)N; n++) {
            double acc = 0.0, mag = 0.0;
            for (uint64_t k = 0; k < (uint64_t)K; k++) {
                double w = dequant_one(q[n * K + k], bits[n * G + k / 64], scales[n * G + k / 64]);
                double xv = vbqo_f16_to_f64(x[(uint64_t)m * (uint64_t)ldx + k]);
                acc += w * xv;
                mag += fabs(w) * fabs(xv);
            }
            y[(uint64_t)m * N + n] = acc;
            bound[(uint64_t)m * N + n] = mag;
        }
    return VBQO_OK;
}

/* Same result from a packed blob: unpack, then the plain definition above. */
int vbqo_gemv_blob(const uint8_t *blob, uint64_t blob_bytes, int M, const uint16_t *x, int ldx, double *y,
                   double *bound)
{
    uint64_t h[14];
    int rc = vbqo_header(blob, blob_bytes, h);
    if (rc)
        return rc;
    uint64_t N = h[0], K = h[1], G = h[2];
    uint8_t *q = (uint8_t *)malloc(N * K);
    uint8_t *bits = (uint8_t *)malloc(N * G);
    uint16_t *sc = (uint16_t *)malloc(2 * N * G);
    if (!q || !bits || !sc) {
        free(q);
        free(bits);
        free(sc);
        return VBQO_ERR_SIZE;
    }
    rc = vbqo_unpack(blob, blob_bytes, q, bits, sc);
    if (!rc)
        rc = vbqo_gemv((int)N, (int)K, M, q, bits, sc, x, ldx, y, bound);
    free(q);
    free(bits);
    free(sc);
    return rc;
}

/* Dense control: y = W16 x with W16[N][K] fp16, fp64 sum, plus the bound. */
int vbqo_dense_gemv(int N, int K, int M, const uint16_t *w16, const uint16_t *x, int ldx, double *y, double *bound)
{
    if (N < 1 || K < 1 || M < 1 || ldx < K)
        return VBQO_ERR_SHAPE;
    for (int m = 0; m < M; m++)
        for (uint64_t n = 0; n < (uint64_t)N; n++) {
            double acc = 0.0, mag = 0.0;
            for (uint64_t k = 0; k < (uint64_t)K; k++) {
                double w = vbqo_f16_to_f64(w16[n * (uint64_t)K + k]);
                double xv = vbqo_f16_to_f64(x[(uint64_t)m * (uint64_t)ldx + k]);
                acc += w * xv;
                mag += fabs(w) * fabs(xv);
            }
            y[(uint64_t)m * N + n] = acc;
            bound[(uint64_t)m * N + n] = mag;
        }
    return VBQO_OK;
}

/*
 * Round-to-nearest quantizer for a given width map (the step before packing).
 * The pages learn the scales during training and give no rule for producing
 * codes from float weights; the reading fixed here is the plain one: per group
 * of 64 weights of width b, with c = (2^b - 1) / 2,
 *   a = max_j |w_j|   (fp32; fmaxf semantics, so a NaN weight is skipped)
 *   s = fp16_rne(a / c)          (the division in fp32, correctly rounded)
 *   q_j = min(max(rint(w_j / s + c), 0), 2^b - 1)
 * with w_j / s and the + c in fp32 (s widened exactly to fp32), rint rounding
 * half to even, and min/max with fmaxf/fminf semantics (a NaN quotient gives
 * q = 0).  Every operation is a single IEEE fp32 operation, so a device that
 * performs the same operations gets the same codes.  w is fp32 [N][ldw].
 */
int vbqo_quantize(int N, int K, const float *w, int ldw, const uint8_t *bits, uint8_t *q, uint16_t *scales)
{
    if (N < 1 || K < 64 || K % 64 != 0 || ldw < K)
        return VBQO_ERR_SHAPE;
    const int G = K / 64;
    for (int n = 0; n < N; n++)
        for (int g = 0; g < G; g++) {
            const int b = bits[(uint64_t)n * G + g];
            if (b != 1 && b != 2 && b != 4 && b != 8)
                return VBQO_ERR_BITS;
            const float c = (float)((1 << b) - 1) / 2.0f;
            const float top = (float)((1 << b) - 1);
            const float *wg = w + (uint64_t)n * (uint64_t)ldw + 64u * (uint64_t)g;
            float a = 0.0f;
            for (int j = 0; j < 64; j++)
                a = fmaxf(a, fabsf(wg[j]));
            const float ratio = a / c;
            const uint16_t sh = vbqo_f64_to_f16_rne((double)ratio);
            scales[(uint64_t)n * G + g] = sh;
            const float s = (float)vbqo_f16_to_f64(sh);
            for (int j = 0; j < 64; j++) {
                const float t = wg[j] / s;
                const float u = t + c;
                const float r = rintf(u);
                q[(uint64_t)n * K + 64u * g + j] = (uint8_t)fminf(fmaxf(r, 0.0f), top);
            }
        }
    return VBQO_OK;
}
