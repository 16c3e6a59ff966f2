/*
 * q8_oracle.c -- plain CPU oracle for the narrow-batch q8_0 decode matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, and by nothing else.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * What it computes (all from the pages, restated):
 *
 *  - q8_0 block quantisation.  "Batched decode: co-decode N live sessions in
 *    one GPU pass" (antirez/ds4 PR #530), section "Why it's worth it -- the
 *    narrow-batch matmul" and the commit "CUDA: narrow-batch q8_0 matmul for
 *    2-4 token decode", names the q8_0 format, its 32-weight block and
 *    pre-quantised ("preq") activations, and says the model file is GGUF.
 *    The pages do not spell the encoding out; this follows its plainest
 *    reading (the GGUF q8_0 block): per 32 values one scale d = absmax/127,
 *    computed and applied in IEEE fp32 (correctly rounded division), values
 *    q = round-half-away-from-zero(x/d) clamped to [-127,127], and d stored
 *    as IEEE binary16 rounded to nearest-even with subnormals kept.  An
 *    all-zero block stores d = +0 and q = 0 without dividing, and so does a
 *    block whose scale underflows to zero; a block holding a NaN or an
 *    infinity stores q = 0 and a NaN scale (quantize_block states the rules).
 *
 *  - The narrow matmul.  Same page, same section: every 32-weight block is
 *    dotted against every live token's activation block.  For live token t
 *    gathered from slot s = batch_index[t] ("[feature] Enable Dynamic
 *    Batching" (quic/efficient-transformers PR #1305), section "Objective":
 *    batch_index selects the rows of a fixed, fully sized buffer):
 *        S[t,n,b] = sum_{i<32} qw[n,32b+i] * qx[s,32b+i]      (exact int32)
 *        y[t,n]   = sum_b S[t,n,b] * dw[n,b] * dx[s,b]        (real numbers)
 *    Each term is exact in double (|S| <= 2^19 needs 20 bits, the two fp16
 *    scales 11 bits each), so the only rounding is the double summation in
 *    ascending block order.  The oracle also returns A = sum_b |term|, the
 *    scale of the summation error any fp32 implementation may make.
 *
 *  - Pos-vector rotary position embedding (below, q8o_rope): the consumer
 *    of the QKV projection in a batched decode step.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * OpenMP only splits independent output rows; each output is computed by one
 * thread in the order written below.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define Q8O_BLOCK 32

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary32 <-> binary16, written from the format definitions.     */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * binary32 -> binary16, round to nearest, ties to even; overflow goes to
 * infinity, results below the normal range become binary16 subnormals.
 * NaN maps to a quiet NaN with the sign kept (payload not specified).
 */
uint16_t q8o_f32_to_f16(float f) {
    const uint32_t u = f32_bits(f);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t e = (u >> 23) & 0xffu;
    const uint32_t m = u & 0x7fffffu;

    if (e == 0xffu) { /* inf or NaN */
        return (uint16_t)(sign | (m ? 0x7e00u : 0x7c00u));
    }
    if (e == 0) {
        /* zero or binary32 subnormal: magnitude < 2^-126, far below half of
         * the smallest binary16 subnormal (2^-25), so it rounds to zero. */
        return sign;
    }
    /* value = M * 2^(E-23) with M the 24-bit significand, E unbiased. */
    const uint32_t M = m | 0x800000u;
    const int E = (int)e - 127;

    uint32_t shift; /* how many low bits of M fall below the binary16 quantum */
    if (E >= -14) {
        shift = 13; /* normal binary16: 11-bit significand */
    } else {
        /* subnormal binary16: quantum 2^-24, value/quantum = M * 2^(E+1) */
        const int s = -(E + 1);
        if (s > 24) return sign; /* below 2^-25: rounds to zero */
        shift = (uint32_t)s;
    }
    uint32_t r = M >> shift;
    const uint32_t rem = M & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (r & 1u))) r += 1u;

    if (E >= -14) {
        int E16 = E + 15; /* biased binary16 exponent, 1..30 when in range */
        if (r == (1u << 11)) { /* rounding carried into a new binade */
            r >>= 1;
            E16 += 1;
        }
        if (E16 >= 31) return (uint16_t)(sign | 0x7c00u); /* overflow */
        return (uint16_t)(sign | ((uint32_t)E16 << 10) | (r & 0x3ffu));
    }
    /* subnormal result; r == 0x400 is exactly the smallest normal 2^-14,
     * whose encoding is the same bit pattern. */
    return (uint16_t)(sign | r);
}

float q8o_f16_to_f32(uint16_t h) {
    const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    const uint32_t e = ((uint32_t)h >> 10) & 0x1fu;
    const uint32_t m = (uint32_t)h & 0x3ffu;
    if (e == 0x1fu) return bits_f32(sign | 0x7f800000u | (m << 13));
    if (e == 0) {
        /* zero or subnormal: m * 2^-24, exact in binary32 */
        const float v = (float)m * 0x1p-24f;
        return sign ? -v : v;
    }
    return bits_f32(sign | ((e - 15u + 127u) << 23) | (m << 13));
}

/* Bulk conversions, used by the exhaustive conversion test. */
void q8o_f32_to_f16_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = q8o_f32_to_f16(x[i]);
}

void q8o_f16_to_f32_array(const uint16_t* h, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = q8o_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------ */
/* q8_0 block quantisation                                                  */
/* ------------------------------------------------------------------------ */

/* Quantise one block of 32 values.  Returns the fp32 scale d (before it is
 * stored as binary16) so callers can check invariants against it.
 *
 * Blocks the pages' format leaves undefined get one stated rule each (the
 * GPU quantiser follows the same rules):
 *   - a block holding a NaN or an infinity stores q = 0 and the binary16
 *     quiet NaN 0x7E00 as its scale, so every output that uses the block is
 *     NaN (the function returns NaN);
 *   - a block whose scale a/127 rounds to zero (a == 0, or a below
 *     63.5 * 2^-149, where the quotient underflows) is the zero block,
 *     d = +0 and q = 0, with no division by zero;
 *   - otherwise the rule above, subnormal scales included. */
static float quantize_block(const float* x, int8_t* q, uint16_t* d16) {
    float a = 0.0f;
    int finite = 1;
    for (int i = 0; i < Q8O_BLOCK; ++i) {
        const float v = fabsf(x[i]);
        if (!(v <= FLT_MAX)) finite = 0; /* NaN or infinity */
        else if (v > a) a = v;
    }
    if (!finite) {
        for (int i = 0; i < Q8O_BLOCK; ++i) q[i] = 0;
        *d16 = 0x7e00u;
        return NAN;
    }
    const float d = a / 127.0f; /* IEEE fp32 division, rounded to nearest */
    if (d == 0.0f) {
        for (int i = 0; i < Q8O_BLOCK; ++i) q[i] = 0;
        *d16 = 0;
        return 0.0f;
    }
    for (int i = 0; i < Q8O_BLOCK; ++i) {
        float r = roundf(x[i] / d); /* half away from zero */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
    *d16 = q8o_f32_to_f16(d);
    return d;
}

/*
 * X: fp32 [rows][K] row-major.  q: int8 [rows][K].  d16: binary16 bits
 * [rows][K/32].  d32 (may be NULL): the fp32 scales before rounding to
 * binary16, [rows][K/32].  Returns 0, or -1 if K is not a multiple of 32.
 */
int q8o_quantize_rows(const float* X, int64_t rows, int64_t K, int8_t* q,
                      uint16_t* d16, float* d32) {
    if (K <= 0 || K % Q8O_BLOCK != 0 || rows < 0) return -1;
    const int64_t KB = K / Q8O_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < KB; ++b) {
            const float d = quantize_block(X + r * K + b * Q8O_BLOCK,
                                           q + r * K + b * Q8O_BLOCK,
                                           d16 + r * KB + b);
            if (d32) d32[r * KB + b] = d;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* The narrow matmul                                                        */
/* ------------------------------------------------------------------------ */

static int32_t block_dot(const int8_t* w, const int8_t* x) {
    int32_t s = 0;
    for (int i = 0; i < Q8O_BLOCK; ++i) s += (int32_t)w[i] * (int32_t)x[i];
    return s;
}

/*
 * Weights: qw int8 [N][K], dw binary16 bits [N][K/32] (canonical q8_0).
 * Activation slots: qx int8 [n_slots][K], dx binary16 bits [n_slots][K/32].
 * batch_index int32 [n_live]: token t reads slot batch_index[t].
 * rows int64 [n_rows]: which output rows to compute (NULL: all N rows, then
 * n_rows must equal N).
 * Y, A: double [n_live][n_rows]; Y = the exact-term double sum, A = sum of
 * |term|.  A token whose slot index is outside [0, n_slots) gets NaN in both.
 * Returns 0, or -1 on a malformed shape.
 */
int q8o_matmul(const int8_t* qw, const uint16_t* dw, int64_t N, int64_t K,
               const int8_t* qx, const uint16_t* dx, int n_slots,
               const int32_t* batch_index, int n_live, const int64_t* rows,
               int64_t n_rows, double* Y, double* A) {
    if (K <= 0 || K % Q8O_BLOCK != 0 || N <= 0 || n_live < 0) return -1;
    if (!rows && n_rows != N) return -1;
    const int64_t KB = K / Q8O_BLOCK;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t n = rows ? rows[i] : i;
        for (int t = 0; t < n_live; ++t) {
            const int s = batch_index[t];
            if (n < 0 || n >= N || s < 0 || s >= n_slots) {
                Y[(int64_t)t * n_rows + i] = NAN;
                A[(int64_t)t * n_rows + i] = NAN;
                continue;
            }
            double y = 0.0, a = 0.0;
            for (int64_t b = 0; b < KB; ++b) {
                const int32_t S = block_dot(qw + n * K + b * Q8O_BLOCK,
                                            qx + (int64_t)s * K + b * Q8O_BLOCK);
                const double term = (double)S *
                                    (double)q8o_f16_to_f32(dw[n * KB + b]) *
                                    (double)q8o_f16_to_f32(dx[(int64_t)s * KB + b]);
                y += term;
                a += fabs(term);
            }
            Y[(int64_t)t * n_rows + i] = y;
            A[(int64_t)t * n_rows + i] = a;
        }
    }
    return 0;
}

/*
 * Per-block integer dot products S[t][i][b] (int32 [n_live][n_rows][K/32])
 * for the selected rows, with the same conventions as q8o_matmul.  Tokens
 * with an out-of-range slot get S = 0.
 */
int q8o_block_dots(const int8_t* qw, int64_t N, int64_t K, const int8_t* qx,
                   int n_slots, const int32_t* batch_index, int n_live,
                   const int64_t* rows, int64_t n_rows, int32_t* S) {
    if (K <= 0 || K % Q8O_BLOCK != 0 || N <= 0 || n_live < 0) return -1;
    if (!rows && n_rows != N) return -1;
    const int64_t KB = K / Q8O_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t n = rows ? rows[i] : i;
        for (int t = 0; t < n_live; ++t) {
            const int s = batch_index[t];
            int32_t* out = S + ((int64_t)t * n_rows + i) * KB;
            for (int64_t b = 0; b < KB; ++b) {
                out[b] = (n < 0 || n >= N || s < 0 || s >= n_slots)
                             ? 0
                             : block_dot(qw + n * K + b * Q8O_BLOCK,
                                         qx + (int64_t)s * K + b * Q8O_BLOCK);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Pos-vector rotary position embedding.  "Batched decode: co-decode N live
 * sessions in one GPU pass" (antirez/ds4 PR #530), commit "CUDA: add
 * pos-vector RoPE tail variants": in a batched decode step each row (token)
 * sits at its own position, so the rotation takes a small array of
 * positions indexed by row, and every row must come out exactly as a
 * single-token launch would make it.  The pages name the operation, not its
 * formula; this is the plain rotary embedding with the "rotate half"
 * pairing of the Qwen family: in each head of head_dim values, values i and
 * i + head_dim/2 (i < head_dim/2) turn by the angle
 *     theta = pos * base^(-2i/head_dim)
 *     out_i          = a cos(theta) - b sin(theta)
 *     out_{i+half}   = a sin(theta) + b cos(theta)
 * with a, b the two inputs.  Everything in double; mag receives |a| + |b| of
 * each value's pair, the scale of the rounding error of any implementation.
 * Rows are n_rows rows of Y, row_stride floats apart; heads 0..n_heads-1
 * occupy the first n_heads*head_dim columns.  out and mag are
 * [n_rows][n_heads*head_dim].  Returns 1 for an invalid argument.
 * ------------------------------------------------------------------------ */
int q8o_rope(const float* Y, int64_t n_rows, int64_t row_stride, const int32_t* pos,
             int64_t n_heads, int64_t head_dim, double base, double* out, double* mag) {
    if (n_rows < 1 || n_heads < 1 || head_dim < 2 || (head_dim & 1) ||
        n_heads * head_dim > row_stride || !(base > 0.0))
        return 1;
    const int64_t half = head_dim / 2, width = n_heads * head_dim;
    for (int64_t t = 0; t < n_rows; ++t) {
        for (int64_t h = 0; h < n_heads; ++h) {
            for (int64_t i = 0; i < half; ++i) {
                const double theta = (double)pos[t] * pow(base, -2.0 * (double)i / (double)head_dim);
                const double c = cos(theta), sn = sin(theta);
                const double a = Y[t * row_stride + h * head_dim + i];
                const double b = Y[t * row_stride + h * head_dim + i + half];
                double* o = out + t * width + h * head_dim;
                double* m = mag + t * width + h * head_dim;
                o[i] = a * c - b * sn;
                o[i + half] = a * sn + b * c;
                m[i] = m[i + half] = fabs(a) + fabs(b);
            }
        }
    }
    return 0;
}

/* Number of OpenMP threads a parallel region here would use. */
int q8o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void q8o_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
