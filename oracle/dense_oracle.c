/*
 * Dense-volume C oracle for submanifold 3x3x3 sparse convolution.
 *
 * TEST INFRASTRUCTURE ONLY: called from the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never from the HIP library, with which it
 * shares no code.
 *
 * It answers "which row sits at (b, z, y, x)?" with a dense int32 volume of
 * batch * res^3 cells (row or -1), so it uses none of the sort / search / hash
 * machinery of the device map builder.  The forward pass is the definition:
 * for every voxel, every present tap, every output and input channel, a
 * double-precision multiply-add, bias added once.
 *
 * Sources: lato.2_mrp_mlx working notes (CLAUDE.md), commit summary and
 * "Key facts" (submanifold 3x3x3, stride 1, output set = input set, KRSC
 * weights [out, kz, ky, kx, in], orientation flag).  Tap k <-> offset
 * (k/9 - 1, (k/3)%3 - 1, k%3 - 1); flip uses weight tap 26 - k.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_E_ARG (-1)
#define ORACLE_E_RANGE (-2)
#define ORACLE_E_DUP (-3)
#define ORACLE_E_OOM (-6)

/* nbr[i*27 + k] = row at coords[i] + offset(k), or -1. */
int oracle_neighbors(const int32_t *coords, int64_t n, int32_t res, int32_t batch, int32_t *nbr)
{
    if (n < 0 || res <= 0 || batch <= 0 || (n > 0 && (!coords || !nbr)))
        return ORACLE_E_ARG;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t *c = coords + 4 * i;
        if (c[0] < 0 || c[0] >= batch) return ORACLE_E_RANGE;
        for (int a = 1; a < 4; ++a)
            if (c[a] < 0 || c[a] >= res) return ORACLE_E_RANGE;
    }
    const int64_t r = res;
    const int64_t cells = (int64_t)batch * r * r * r;
    int32_t *vol = (int32_t *)malloc((size_t)cells * sizeof(int32_t));
    if (!vol) return ORACLE_E_OOM;
    memset(vol, 0xff, (size_t)cells * sizeof(int32_t)); /* every cell = -1 */
    for (int64_t i = 0; i < n; ++i) {
        const int32_t *c = coords + 4 * i;
        int64_t cell = ((c[0] * r + c[1]) * r + c[2]) * r + c[3];
        if (vol[cell] != -1) { free(vol); return ORACLE_E_DUP; }
        vol[cell] = (int32_t)i;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int32_t *c = coords + 4 * i;
        for (int k = 0; k < 27; ++k) {
            int64_t z = c[1] + k / 9 - 1, y = c[2] + (k / 3) % 3 - 1, x = c[3] + k % 3 - 1;
            int32_t v = -1;
            if (z >= 0 && z < r && y >= 0 && y < r && x >= 0 && x < r)
                v = vol[((c[0] * r + z) * r + y) * r + x];
            nbr[i * 27 + k] = v;
        }
    }
    free(vol);
    return ORACLE_OK;
}

/*
 * out[i*cout + o] = bias[o] + sum_{k: nbr[i,k] >= 0} sum_c W[o, k', c] * feats[nbr[i,k]*cin + c]
 * with W in KRSC [cout][27][cin] and k' = flip ? 26 - k : k.  Rows [row0, row1) only,
 * so that a bounded sample can be timed.
 */
int oracle_forward(const double *feats, const double *weight, const double *bias,
                   const int32_t *nbr, int64_t n, int32_t cin, int32_t cout, int32_t flip,
                   int64_t row0, int64_t row1, double *out)
{
    if (n < 0 || cin <= 0 || cout <= 0 || row0 < 0 || row1 > n || row0 > row1)
        return ORACLE_E_ARG;
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = row0; i < row1; ++i) {
        for (int32_t o = 0; o < cout; ++o) {
            double acc = 0.0;
            for (int k = 0; k < 27; ++k) {
                int32_t j = nbr[i * 27 + k];
                if (j < 0) continue;
                int kw = flip ? 26 - k : k;
                const double *w = weight + ((int64_t)o * 27 + kw) * cin;
                const double *f = feats + (int64_t)j * cin;
                for (int32_t c = 0; c < cin; ++c)
                    acc += w[c] * f[c];
            }
            if (bias) acc += bias[o];
            out[i * cout + o] = acc;
        }
    }
    return ORACLE_OK;
}

/* Subdivide: row 8i+q, q = 4dz + 2dy + dx, coords (b, 2z+dz, 2y+dy, 2x+dx). */
int oracle_subdivide(const int32_t *coords, int64_t n, int32_t *out_coords)
{
    if (n < 0 || (n > 0 && (!coords || !out_coords))) return ORACLE_E_ARG;
    for (int64_t i = 0; i < n; ++i)
        for (int q = 0; q < 8; ++q) {
            int32_t *o = out_coords + 4 * (8 * i + q);
            o[0] = coords[4 * i];
            o[1] = 2 * coords[4 * i + 1] + (q >> 2);
            o[2] = 2 * coords[4 * i + 2] + ((q >> 1) & 1);
            o[3] = 2 * coords[4 * i + 3] + (q & 1);
        }
    return ORACLE_OK;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by the parallel loops from now on (timing of the single-thread leg). */
int oracle_set_threads(int32_t threads)
{
    if (threads < 1) return ORACLE_E_ARG;
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(threads);
#endif
    return ORACLE_OK;
}
