/*
 * CPU oracle for the submanifold sparse 3D convolution hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header or table with the GPU library.
 *
 * What it computes (page "mlx_backend/sparse_conv_metal.py", module docstring
 * and the `sparse_conv_metal` wrapper docstring):
 *
 *   out[n, co] = bias[co] + sum_k sum_ci feats[nbr[k, n], ci] * w[k, ci, co]
 *
 * with nbr a (K, N) int32 map, row-major (element k*N + n), in which the value
 * N marks a missing neighbour that contributes nothing (the kernel body skips
 * any nbr >= N).  Accumulation here is fp64; fp32 and bf16 inputs are widened
 * exactly.  Alongside each output the oracle returns S[n,co] = sum |f*w| over
 * the terms it added, which the tests use to normalise the fp32 tolerance.
 *
 * The input gradient (oracle_dgrad) is the adjoint of that linear map, from
 * its definition (the page gives only the forward; the gradient follows from
 * the formula): dfeats[m, ci] = sum over (k, n) with nbr[k, n] == m of
 * sum_co dout[n, co] * w[k, ci, co].  The weight gradient (oracle_wgrad) is
 * the derivative with respect to w: dw[k, ci, co] = sum over n with nbr[k, n]
 * present of feats[nbr[k, n], ci] * dout[n, co].
 *
 * Mixed dtypes (oracle_cast): the page's wrapper casts feats to the weights'
 * dtype before the kernel.  float32 -> bfloat16 is taken as the nearest
 * bfloat16 value with ties to the even significand (the IEEE default rounding),
 * NaN staying NaN; bfloat16 -> float32 is exact.  The forward of mixed inputs
 * is then oracle_forward on the cast features.
 *
 * The map itself is not on the page (the page receives it as an input).  This
 * oracle builds it from the plain definition
 *
 *   nbr[k, n] = m  if coords[m] == coords[n] + dilation * o_k,  else N
 *
 * where, with s = cbrt(K) odd and r = (s-1)/2, offset k = ((a*s)+b)*s + c has
 * o_k = (a-r, b-r, c-r): x slowest, z fastest, centre k = (K-1)/2.  This is the
 * cross-correlation convention of a dense 3D convolution with padding
 * dilation*r.  The lookup uses a sorted key array and binary search (library
 * qsort), which is a different data structure from anything a GPU builder
 * would use.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no fast-math).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <omp.h>

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_RANGE (-3)
#define ORC_E_DUP (-4)
#define ORC_E_MEM (-7)

#define COORD_BIAS (1 << 20)     /* coordinates must lie in [-2^20, 2^20) */

int oracle_version(void) { return 1; }

/* OpenMP threads the oracle's parallel loops use */
int oracle_threads(void) { return omp_get_max_threads(); }
/* threads of later parallel regions (n >= 1); used to time the oracle on one core */
int oracle_set_threads(int n) {
    if (n < 1) return ORC_E_ARG;
    omp_set_num_threads(n);
    return ORC_OK;
}

/* s if K is an odd perfect cube s^3, else -1 */
static int cube_side(int K) {
    if (K < 1) return -1;
    for (int s = 1; s * s * s <= K; s += 2)
        if (s * s * s == K) return s;
    return -1;
}

static int in_range(int64_t v) { return v >= -COORD_BIAS && v < COORD_BIAS; }

/* injective 63-bit key of an in-range coordinate triple */
static uint64_t coord_key(int64_t x, int64_t y, int64_t z) {
    return ((uint64_t)(x + COORD_BIAS) << 42) | ((uint64_t)(y + COORD_BIAS) << 21)
         | (uint64_t)(z + COORD_BIAS);
}

typedef struct { uint64_t key; int64_t idx; } keyed;

static int cmp_keyed(const void* a, const void* b) {
    uint64_t ka = ((const keyed*)a)->key, kb = ((const keyed*)b)->key;
    return (ka > kb) - (ka < kb);
}

/* Sorted (key, index) table of all coordinates.  Returns NULL and sets *err on
 * out-of-range or duplicate coordinates. */
static keyed* sorted_table(const int32_t* coords, int64_t N, int* err) {
    keyed* t = (keyed*)malloc((size_t)(N > 0 ? N : 1) * sizeof(keyed));
    if (!t) { *err = ORC_E_MEM; return NULL; }
    for (int64_t i = 0; i < N; ++i) {
        int64_t x = coords[3 * i], y = coords[3 * i + 1], z = coords[3 * i + 2];
        if (!in_range(x) || !in_range(y) || !in_range(z)) { free(t); *err = ORC_E_RANGE; return NULL; }
        t[i].key = coord_key(x, y, z);
        t[i].idx = i;
    }
    qsort(t, (size_t)N, sizeof(keyed), cmp_keyed);
    for (int64_t i = 1; i < N; ++i)
        if (t[i].key == t[i - 1].key) { free(t); *err = ORC_E_DUP; return NULL; }
    *err = ORC_OK;
    return t;
}

/* index of the voxel with this key, or -1 */
static int64_t lookup(const keyed* t, int64_t N, uint64_t key) {
    int64_t lo = 0, hi = N;            /* first element with t.key >= key */
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (t[mid].key < key) lo = mid + 1; else hi = mid;
    }
    return (lo < N && t[lo].key == key) ? t[lo].idx : -1;
}

/* neighbour list of one voxel: out[k * ld] for k < K */
static void neighbours_of(const keyed* t, const int32_t* coords, int64_t N, int s, int dilation,
                          int64_t n, int32_t* out, int64_t ld) {
    int r = (s - 1) / 2;
    int64_t cx = coords[3 * n], cy = coords[3 * n + 1], cz = coords[3 * n + 2];
    int k = 0;
    for (int a = 0; a < s; ++a)
        for (int b = 0; b < s; ++b)
            for (int c = 0; c < s; ++c, ++k) {
                int64_t x = cx + (int64_t)dilation * (a - r);
                int64_t y = cy + (int64_t)dilation * (b - r);
                int64_t z = cz + (int64_t)dilation * (c - r);
                int64_t m = -1;
                if (in_range(x) && in_range(y) && in_range(z)) m = lookup(t, N, coord_key(x, y, z));
                out[(int64_t)k * ld] = (int32_t)(m < 0 ? N : m);
            }
}

/* Full (K, N) map.  nbr must hold K*N int32. */
int oracle_nmap(const int32_t* coords, int64_t N, int K, int dilation, int32_t* nbr) {
    int s = cube_side(K);
    if (s < 0 || dilation < 1 || N < 0 || N >= INT32_MAX) return ORC_E_ARG;
    if (N == 0) return ORC_OK;
    int err;
    keyed* t = sorted_table(coords, N, &err);
    if (!t) return err;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) neighbours_of(t, coords, N, s, dilation, n, nbr + n, N);
    free(t);
    return ORC_OK;
}

/* Map columns for selected voxels only: nbr is (K, nrows), column j = rows[j]. */
int oracle_nmap_rows(const int32_t* coords, int64_t N, int K, int dilation,
                     const int64_t* rows, int64_t nrows, int32_t* nbr) {
    int s = cube_side(K);
    if (s < 0 || dilation < 1 || N < 0 || N >= INT32_MAX || nrows < 0) return ORC_E_ARG;
    for (int64_t j = 0; j < nrows; ++j) if (rows[j] < 0 || rows[j] >= N) return ORC_E_ARG;
    if (N == 0 || nrows == 0) return ORC_OK;
    int err;
    keyed* t = sorted_table(coords, N, &err);
    if (!t) return err;
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nrows; ++j) neighbours_of(t, coords, N, s, dilation, rows[j], nbr + j, nrows);
    free(t);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Forward.
 *   feats : (N, Ci) row-major, dtype 0 = float32, 1 = bfloat16 (raw uint16 bits)
 *   nbr   : (K, nrows) int32; column j lists the neighbours of output row j;
 *           any value v with (uint32)v >= N is missing (the page's kernel skips
 *           nbr >= N; an unsigned compare also treats negatives as missing)
 *   w     : (K, Ci, Co) row-major, same dtype as feats
 *   bias  : (Co,) float32 or NULL (zero)
 *   out   : (nrows, Co) fp64;  abs_sum: (nrows, Co) fp64 or NULL
 * ------------------------------------------------------------------------- */
static double widen(const void* p, int dtype, int64_t i) {
    if (dtype == 0) return (double)((const float*)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;   /* bf16 = top half of fp32 */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int oracle_forward(const void* feats, int dtype, int64_t N, int Ci,
                   const int32_t* nbr, int K, int64_t nrows,
                   const void* w, int Co, const float* bias,
                   double* out, double* abs_sum) {
    if ((dtype != 0 && dtype != 1) || N < 0 || Ci < 1 || Co < 1 || K < 1 || nrows < 0) return ORC_E_ARG;
    int err = ORC_OK;
    #pragma omp parallel
    {
        /* every thread reaches the worksharing loop (OpenMP requires it);
         * one without its buffers takes no rows' work */
        double* acc = (double*)malloc(sizeof(double) * (size_t)Co);
        double* sab = (double*)malloc(sizeof(double) * (size_t)Co);
        const int ok = acc && sab;
        if (!ok) {
            #pragma omp atomic write
            err = ORC_E_MEM;
        }
        {
            #pragma omp for schedule(dynamic, 64)
            for (int64_t j = 0; j < nrows; ++j) {
                if (!ok) continue;
                for (int co = 0; co < Co; ++co) { acc[co] = 0.0; sab[co] = 0.0; }
                for (int k = 0; k < K; ++k) {
                    uint32_t m = (uint32_t)nbr[(int64_t)k * nrows + j];
                    if ((int64_t)m >= N) continue;              /* missing neighbour */
                    for (int ci = 0; ci < Ci; ++ci) {
                        double f = widen(feats, dtype, (int64_t)m * Ci + ci);
                        int64_t wrow = ((int64_t)k * Ci + ci) * Co;
                        for (int co = 0; co < Co; ++co) {
                            double p = f * widen(w, dtype, wrow + co);
                            acc[co] += p;
                            sab[co] += fabs(p);
                        }
                    }
                }
                for (int co = 0; co < Co; ++co) {
                    out[j * Co + co] = acc[co] + (bias ? (double)bias[co] : 0.0);
                    if (abs_sum) abs_sum[j * Co + co] = sab[co];
                }
            }
        }
        free(acc);
        free(sab);
    }
    return err;
}

/* ---------------------------------------------------------------------------
 * Input gradient (dgrad) of the forward above: the adjoint of the linear map
 * feats -> out (bias contributes nothing), written from its definition
 *
 *   dfeats[m, ci] = sum over (k, n) with nbr[k, n] == m of
 *                   sum_co dout[n, co] * w[k, ci, co]
 *
 *   dout  : (N, Co) row-major, dtype 0 = float32, 1 = bfloat16 (raw bits)
 *   nbr   : (K, N) int32, the forward's map (missing: (uint32)v >= N)
 *   w     : (K, Ci, Co) row-major, same dtype as dout
 *   rows  : the nrows input rows m to compute
 *   out   : (nrows, Ci) fp64;  abs_sum: (nrows, Ci) fp64 (sum |dout*w|) or NULL
 * Every (k, n) entry of the map is scanned once to list, per requested row,
 * the terms that land on it (in increasing k, then n); the terms are then
 * summed in that order.  No symmetry of the map is assumed.
 * ------------------------------------------------------------------------- */
int oracle_dgrad(const void* dout, int dtype, int64_t N, int Co,
                 const int32_t* nbr, int K, const void* w, int Ci,
                 const int64_t* rows, int64_t nrows, double* out, double* abs_sum) {
    if ((dtype != 0 && dtype != 1) || N < 0 || Ci < 1 || Co < 1 || K < 1 || nrows < 0) return ORC_E_ARG;
    int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    int64_t* start = (int64_t*)calloc((size_t)nrows + 1, sizeof(int64_t));
    if (!slot || !start) {
        free(slot);
        free(start);
        return ORC_E_MEM;
    }
    for (int64_t m = 0; m < N; ++m) slot[m] = -1;
    for (int64_t j = 0; j < nrows; ++j) {
        if (rows[j] < 0 || rows[j] >= N || slot[rows[j]] >= 0) {
            free(slot);
            free(start);
            return ORC_E_ARG;
        }
        slot[rows[j]] = j;
    }
    /* terms per requested row, then their (k, n) lists */
    for (int k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            uint32_t m = (uint32_t)nbr[(int64_t)k * N + n];
            if ((int64_t)m < N && slot[m] >= 0) ++start[slot[m] + 1];
        }
    for (int64_t j = 0; j < nrows; ++j) start[j + 1] += start[j];
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
    int64_t* term = (int64_t*)malloc(sizeof(int64_t) * (size_t)(start[nrows] > 0 ? start[nrows] : 1));
    if (!fill || !term) {
        free(slot);
        free(start);
        free(fill);
        free(term);
        return ORC_E_MEM;
    }
    for (int64_t j = 0; j < nrows; ++j) fill[j] = start[j];
    for (int k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            uint32_t m = (uint32_t)nbr[(int64_t)k * N + n];
            if ((int64_t)m < N && slot[m] >= 0) term[fill[slot[m]]++] = (int64_t)k * N + n;
        }
    int err = ORC_OK;
    #pragma omp parallel
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)Ci);
        double* sab = (double*)malloc(sizeof(double) * (size_t)Ci);
        const int ok = acc && sab;
        if (!ok) {
            #pragma omp atomic write
            err = ORC_E_MEM;
        }
        {
            #pragma omp for schedule(dynamic, 16)
            for (int64_t j = 0; j < nrows; ++j) {
                if (!ok) continue;
                for (int ci = 0; ci < Ci; ++ci) { acc[ci] = 0.0; sab[ci] = 0.0; }
                for (int64_t q = start[j]; q < start[j + 1]; ++q) {
                    const int64_t k = term[q] / N, n = term[q] % N;
                    for (int ci = 0; ci < Ci; ++ci) {
                        const int64_t wrow = (k * Ci + ci) * Co;
                        for (int co = 0; co < Co; ++co) {
                            double p = widen(dout, dtype, n * Co + co) * widen(w, dtype, wrow + co);
                            acc[ci] += p;
                            sab[ci] += fabs(p);
                        }
                    }
                }
                for (int ci = 0; ci < Ci; ++ci) {
                    out[j * Ci + ci] = acc[ci];
                    if (abs_sum) abs_sum[j * Ci + ci] = sab[ci];
                }
            }
        }
        free(acc);
        free(sab);
    }
    free(slot);
    free(start);
    free(fill);
    free(term);
    return err;
}

/* ---------------------------------------------------------------------------
 * Weight gradient (wgrad) of the forward: its derivative with respect to w,
 * contracted with dout, from the definition
 *
 *   dw[k, ci, co] = sum over n with nbr[k, n] present of
 *                   feats[nbr[k, n], ci] * dout[n, co]
 *
 *   feats : (N, Ci), dout : (N, Co), same dtype (0 = float32, 1 = bfloat16)
 *   nbr   : (K, N) int32 (missing: (uint32)v >= N)
 *   dw    : (K, Ci, Co) fp64;  abs_sum: (K, Ci, Co) fp64 (sum |f*dout|) or NULL
 * Summed over n in increasing order; parallel over k.
 * ------------------------------------------------------------------------- */
int oracle_wgrad(const void* feats, const void* dout, int dtype, int64_t N, int Ci, int Co,
                 const int32_t* nbr, int K, double* dw, double* abs_sum) {
    if ((dtype != 0 && dtype != 1) || N < 0 || Ci < 1 || Co < 1 || K < 1) return ORC_E_ARG;
    int err = ORC_OK;
    #pragma omp parallel
    {
        double* dv = (double*)malloc(sizeof(double) * (size_t)Co);
        if (!dv) {
            #pragma omp atomic write
            err = ORC_E_MEM;
        }
        {
            #pragma omp for schedule(dynamic, 1)
            for (int k = 0; k < K; ++k) {
                if (!dv) continue;
                double* acc = dw + (int64_t)k * Ci * Co;
                double* sab = abs_sum ? abs_sum + (int64_t)k * Ci * Co : NULL;
                for (int64_t i = 0; i < (int64_t)Ci * Co; ++i) {
                    acc[i] = 0.0;
                    if (sab) sab[i] = 0.0;
                }
                for (int64_t n = 0; n < N; ++n) {
                    uint32_t m = (uint32_t)nbr[(int64_t)k * N + n];
                    if ((int64_t)m >= N) continue;
                    for (int co = 0; co < Co; ++co) dv[co] = widen(dout, dtype, n * Co + co);
                    for (int ci = 0; ci < Ci; ++ci) {
                        const double f = widen(feats, dtype, (int64_t)m * Ci + ci);
                        for (int co = 0; co < Co; ++co) {
                            const double p = f * dv[co];
                            acc[(int64_t)ci * Co + co] += p;
                            if (sab) sab[(int64_t)ci * Co + co] += fabs(p);
                        }
                    }
                }
            }
        }
        free(dv);
    }
    return err;
}

/* ---------------------------------------------------------------------------
 * Morton (Z-order) code of each coordinate, biased by 2^20 per axis:
 * bit 3b of the code is bit b of z, 3b+1 of y, 3b+2 of x (21 bits per axis,
 * 63-bit code).  Used only to check the locality schedule a builder reports.
 * ------------------------------------------------------------------------- */
int oracle_morton(const int32_t* coords, int64_t N, uint64_t* codes) {
    for (int64_t i = 0; i < N; ++i) {
        int64_t v[3] = { coords[3 * i], coords[3 * i + 1], coords[3 * i + 2] };
        if (!in_range(v[0]) || !in_range(v[1]) || !in_range(v[2])) return ORC_E_RANGE;
        uint64_t bx = (uint64_t)(v[0] + COORD_BIAS), by = (uint64_t)(v[1] + COORD_BIAS),
                 bz = (uint64_t)(v[2] + COORD_BIAS), c = 0;
        for (int b = 0; b < 21; ++b) {
            c |= ((bz >> b) & 1u) << (3 * b);
            c |= ((by >> b) & 1u) << (3 * b + 1);
            c |= ((bx >> b) & 1u) << (3 * b + 2);
        }
        codes[i] = c;
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Element-wise cast between float32 (dtype 0) and bfloat16 (dtype 1, raw bits).
 *
 * float32 -> bfloat16 from the definition of rounding to nearest, ties to
 * even: the two bfloat16 values that bracket x are its truncation t (top 16
 * bits, same sign, |t| <= |x|) and the next value away from zero t + 1; the
 * nearer one is chosen by comparing the exact distances in fp64, and a tie
 * goes to the one with an even significand.  Values are computed with an
 * unbounded exponent (the code after the largest finite bfloat16 is worth
 * 2^128), so a float32 that rounds past the largest finite value becomes
 * infinity, as IEEE overflow prescribes.  NaN maps to a quiet NaN of the
 * same sign.  bfloat16 -> float32 appends 16 zero bits (exact).
 * ------------------------------------------------------------------------- */
static double bf16_value_unbounded(uint16_t b) {
    const int sign = b >> 15, e = (b >> 7) & 0xff, m = b & 0x7f;
    const double mag = e == 0 ? ldexp((double)m, -126 - 7) : ldexp(1.0 + m / 128.0, e - 127);
    return sign ? -mag : mag;
}

static uint16_t bf16_nearest_even(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x40u);
    if (isinf(x) || (u & 0xffffu) == 0) return (uint16_t)(u >> 16);
    const uint16_t t = (uint16_t)(u >> 16), up = (uint16_t)(t + 1);
    const double dt = fabs((double)x - bf16_value_unbounded(t));
    const double du = fabs(bf16_value_unbounded(up) - (double)x);
    if (dt < du) return t;
    if (du < dt) return up;
    return (t & 1u) ? up : t;
}

int oracle_cast(const void* src, int src_dtype, void* dst, int dst_dtype, int64_t n) {
    if ((src_dtype != 0 && src_dtype != 1) || (dst_dtype != 0 && dst_dtype != 1) || n < 0) return ORC_E_ARG;
    if (src_dtype == dst_dtype) {
        memcpy(dst, src, (size_t)n * (src_dtype == 0 ? 4 : 2));
    } else if (src_dtype == 0) {
        for (int64_t i = 0; i < n; ++i) ((uint16_t*)dst)[i] = bf16_nearest_even(((const float*)src)[i]);
    } else {
        for (int64_t i = 0; i < n; ++i) ((uint32_t*)dst)[i] = (uint32_t)((const uint16_t*)src)[i] << 16;
    }
    return ORC_OK;
}
