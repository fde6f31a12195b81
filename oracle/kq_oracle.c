/*
 * kq_oracle.c -- plain, slow CPU oracle for the k-quant decode matvec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source with the HIP library.
 *
 * What it computes (muser-book Ch 13 "The QKV + gate matvec family",
 * section 13.1): y_i = sum_j W[i,j] * x[j] for every output row i, where
 * every W[i,j] is the exact dequantized value of a k-quant super-block
 * element.  The decoders follow muser-book Ch 6 "The kquant family on the
 * reference lane": Q4_K (section 6.2, Figures 6.2 and 6.3), Q5_K and Q6_K
 * (section 6.4, Figures 6.4 and 6.5).  Arithmetic is IEEE binary64; the
 * dequantized weight is exact in binary64 (argument in oracle_dequant_block)
 * and the dot product is accumulated serially, in column order, in binary64.
 *
 * Readings taken where the pages do not print a step (listed again in the
 * design notes):
 *   - f16 headers are exact IEEE-754 binary16, subnormals included.
 *   - Q5_K: the 32 qh bytes are indexed by the element's position inside its
 *     32-element sub-block, and bit j of such a byte is the fifth code bit of
 *     sub-block j.
 *   - Q6_K: the block is two halves of 128 elements; a half is four quarters
 *     of 32.  Element l of quarter k of half n takes the low nibble (k = 0, 1)
 *     or the high nibble (k = 2, 3) of ql[64n + 32(k mod 2) + l] and bits
 *     2k, 2k+1 of qh[32n + l]; the 16 int8 scales each cover 16 consecutive
 *     elements.  Parity of this element order against real GGUF files is
 *     unpinned by the pages.
 */
#include <stdint.h>
#include <stdlib.h>
#include <math.h>
#include <string.h>

#define FMT_Q4_K 12
#define FMT_Q5_K 13
#define FMT_Q6_K 14

/* Figure 6.1: bytes per 256-element super-block. */
int oracle_block_bytes(int fmt) {
    switch (fmt) {
    case FMT_Q4_K: return 144;
    case FMT_Q5_K: return 176;
    case FMT_Q6_K: return 210;
    default: return -1;
    }
}

/* IEEE-754 binary16 -> binary64, exact (every binary16 value is a binary64
 * value).  1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static uint16_t le16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Ch 6 section 6.2, the get_scale_min closure: sub-block j (0..7) of the
 * 12-byte strip s.  j < 4: six low bits of s[j] and s[j+4].  j >= 4: the low
 * (sc) or high (m) nibble of s[j+4] below the top two bits of s[j-4] (sc) or
 * s[j] (m). */
static void scale_min_k4(const uint8_t* s, int j, int32_t* sc, int32_t* m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/*
 * Integer decode of one super-block.
 *   codes[256]: Q4_K 0..15, Q5_K 0..31, Q6_K signed -32..31 (offset applied)
 *   scale[16], minv[16]: Q4_K/Q5_K sc_j and m_j for j < 8 (rest 0);
 *                        Q6_K the 16 signed int8 scales (minv all 0)
 *   d, dmin: the f16 headers as binary64 (Q6_K: dmin = 0)
 * Sub-block of element e: e / 32 for Q4_K and Q5_K, e / 16 for Q6_K.
 * Returns 0, or -1 for an unknown format.
 */
int oracle_decode_block(int fmt, const uint8_t* b, int32_t* codes, int32_t* scale,
                        int32_t* minv, double* d, double* dmin) {
    memset(scale, 0, 16 * sizeof(int32_t));
    memset(minv, 0, 16 * sizeof(int32_t));
    if (fmt == FMT_Q4_K || fmt == FMT_Q5_K) {
        /* Figure 6.2 / 6.4: d @0, dmin @2, 12-byte strip @4; Q4_K qs @16,
         * Q5_K qh @16 and qs @48. */
        const uint8_t* s = b + 4;
        const uint8_t* qs = b + (fmt == FMT_Q4_K ? 16 : 48);
        const uint8_t* qh = b + 16;
        *d = oracle_f16_to_f64(le16(b));
        *dmin = oracle_f16_to_f64(le16(b + 2));
        for (int j = 0; j < 8; ++j) scale_min_k4(s, j, &scale[j], &minv[j]);
        /* Section 6.2: four groups of 64 elements; in group g the byte
         * qs[32g + l] gives element 64g + l its low nibble and element
         * 64g + 32 + l its high nibble. */
        for (int e = 0; e < 256; ++e) {
            int g = e / 64, r = e % 64, l = e % 32;
            int byte = qs[32 * g + l];
            int q = (r < 32) ? (byte & 15) : (byte >> 4);
            if (fmt == FMT_Q5_K) {
                int j = e / 32;                       /* sub-block index */
                q |= ((qh[l] >> j) & 1) << 4;         /* Figure 6.4: nibble | qh_bit << 4 */
            }
            codes[e] = q;
        }
        return 0;
    }
    if (fmt == FMT_Q6_K) {
        /* Figure 6.5: ql @0 (128 B), qh @128 (64 B), 16 x int8 sc @192,
         * d @208 (the last field). */
        const uint8_t* ql = b;
        const uint8_t* qh = b + 128;
        *d = oracle_f16_to_f64(le16(b + 208));
        *dmin = 0.0;
        for (int j = 0; j < 16; ++j) scale[j] = (int8_t)b[192 + j];
        for (int e = 0; e < 256; ++e) {
            int n = e / 128, k = (e % 128) / 32, l = e % 32;
            int lbyte = ql[64 * n + 32 * (k % 2) + l];
            int nib = (k < 2) ? (lbyte & 15) : (lbyte >> 4);
            int hi2 = (qh[32 * n + l] >> (2 * k)) & 3;
            codes[e] = (nib | (hi2 << 4)) - 32;       /* section 6.4: 0..63 shifted to -32..31 */
        }
        return 0;
    }
    return -1;
}

/*
 * Dequantize one super-block into w[256], exactly.
 * Q4_K/Q5_K (Ch 6 section 6.2): w = d * sc_j * q - dmin * m_j.
 * Q6_K (Ch 6 section 6.4):      w = d * sc_j * q.
 * Exactness: d and dmin are binary16, so integer multiples of 2^-24 of
 * magnitude below 2^16.  Q4_K/Q5_K: sc, m <= 63 and q <= 31, so d*sc,
 * d*sc*q and dmin*m are multiples of 2^-24 below 2^27 and the difference is
 * one below 2^28: at most 52 significant bits.  Q6_K: |sc| <= 128 and
 * |q| <= 32, so d*sc*q is a multiple of 2^-24 below 2^28.  Every step is
 * therefore exact in binary64.  (Infinite or NaN headers propagate as IEEE
 * arithmetic dictates.)
 */
int oracle_dequant_block(int fmt, const uint8_t* b, double* w) {
    int32_t codes[256], scale[16], minv[16];
    double d, dmin;
    if (oracle_decode_block(fmt, b, codes, scale, minv, &d, &dmin) != 0) return -1;
    int sub = (fmt == FMT_Q6_K) ? 16 : 32;
    for (int e = 0; e < 256; ++e) {
        int j = e / sub;
        w[e] = d * (double)scale[j] * (double)codes[e] - dmin * (double)minv[j];
    }
    return 0;
}

/* Dequantize `rows` rows of `cols` columns (row-major super-blocks, Ch 13
 * section 13.3: each row is one contiguous run of cols/256 blocks). */
int oracle_dequant(int fmt, const uint8_t* W, int64_t rows, int64_t cols, double* out) {
    int bb = oracle_block_bytes(fmt);
    if (bb < 0 || cols <= 0 || cols % 256) return -1;
    int64_t nb = cols / 256;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t b = 0; b < nb; ++b)
            if (oracle_dequant_block(fmt, W + (i * nb + b) * bb, out + i * cols + b * 256)) return -1;
    return 0;
}

/*
 * Embedding rows (Ch 6 section 6.7, the one-thread-per-output-element
 * embedding lookup): out[t][j] = W[ids[t], j], the exact weight, for t < n
 * and j < cols.  Each element is taken on its own, as that kernel does: the
 * row starts at ids[t] * row_bytes with row_bytes = (cols/256) * block
 * bytes (3,744 for a 6,656-wide Q4_K table, Ch 6 section 6.6); element j
 * lies in block j/256 of the row, which is decoded and its element j % 256
 * read out.  An id outside [0, rows) gives a row of NaN.  out is [n][cols]
 * binary64.
 */
int oracle_embed(int fmt, const uint8_t* W, int64_t rows, int64_t cols, const int32_t* ids, int64_t n,
                 double* out) {
    int bb = oracle_block_bytes(fmt);
    if (bb < 0 || cols <= 0 || cols % 256 || rows <= 0 || n < 0) return -1;
    int64_t row_bytes = (cols / 256) * bb;
    double w[256];
    for (int64_t t = 0; t < n; ++t) {
        int64_t id = ids[t];
        for (int64_t j = 0; j < cols; ++j) {
            if (id < 0 || id >= rows) {
                out[t * cols + j] = NAN;
                continue;
            }
            if (oracle_dequant_block(fmt, W + id * row_bytes + (j / 256) * bb, w)) return -1;
            out[t * cols + j] = w[j % 256];
        }
    }
    return 0;
}

/*
 * y[t][k] = sum_j W[r_k, j] * x[t][j] and s[t][k] = sum_j |W[r_k, j] * x[t][j]|
 * for the rows r_k = row_idx[k] (k < n_out; row_idx NULL means r_k = k) and
 * tokens t < ntok.  x is [ntok][ldx] float32; y and s are [ntok][n_out]
 * binary64.  Each row is decoded block by block and accumulated in column
 * order.  nthreads > 1 splits the rows over OpenMP threads; the arithmetic
 * of a row does not depend on it.
 */
int oracle_matvec(int fmt, const uint8_t* W, int64_t rows, int64_t cols,
                  const float* x, int64_t ldx, int32_t ntok,
                  const int64_t* row_idx, int64_t n_out,
                  double* y, double* s, int32_t nthreads) {
    int bb = oracle_block_bytes(fmt);
    if (bb < 0 || cols <= 0 || cols % 256 || ntok < 1 || ldx < cols) return -1;
    int64_t nb = cols / 256;
    int64_t row_bytes = nb * bb;
    for (int64_t k = 0; k < n_out; ++k) {
        int64_t r = row_idx ? row_idx[k] : k;
        if (r < 0 || r >= rows) return -2;
    }
    if (nthreads < 1) nthreads = 1;
    #pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t k = 0; k < n_out; ++k) {
        int64_t r = row_idx ? row_idx[k] : k;
        double w[256];
        for (int32_t t = 0; t < ntok; ++t) { y[t * n_out + k] = 0.0; s[t * n_out + k] = 0.0; }
        for (int64_t b = 0; b < nb; ++b) {
            oracle_dequant_block(fmt, W + r * row_bytes + b * bb, w);
            for (int32_t t = 0; t < ntok; ++t) {
                const float* xt = x + t * ldx + b * 256;
                double acc = y[t * n_out + k], mag = s[t * n_out + k];
                for (int e = 0; e < 256; ++e) {
                    double p = w[e] * (double)xt[e];
                    acc += p;
                    mag += fabs(p);
                }
                y[t * n_out + k] = acc;
                s[t * n_out + k] = mag;
            }
        }
    }
    return 0;
}
