/*
 * Plain C twin of the SubMConv3d oracle, for sizes the Python oracle cannot
 * finish in seconds and for the CPU baseline timing.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load this library. It shares no code with
 * the GPU library.
 *
 * Definition followed (trellis_sparse_mlx README: "What's in it" table for
 * the 3x3x3 / 1x1x1 kernel and the [N,4] coordinates; "Performance" for the
 * sum over offsets of each gathered row times that offset's weights;
 * "Correctness" for the c+d
 * cross-correlation and the naive per-voxel reference):
 *
 *   kmap[i][k] = row j with coords[j] == coords[i] + d_k (same batch item),
 *                or -1; d_k = (dx,dy,dz), k = 9(dx+1) + 3(dy+1) + (dz+1)
 *                for 3x3x3 and d_0 = 0 for 1x1x1; neighbours outside the
 *                grid are absent.
 *   out[i][o]  = bias[o] + sum_k sum_c feats[kmap[i][k]][c] * W[k][c][o]
 *                over the k with kmap[i][k] != -1, in fp64.
 *
 * The lookup is a lexicographic sort of the sites plus binary search (the
 * obvious approach; it is independent of the GPU path's hashing).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t b, x, y, z;
    int64_t row;
} site_t;

static int cmp_site(const void* pa, const void* pb) {
    const site_t* a = (const site_t*)pa;
    const site_t* b = (const site_t*)pb;
    if (a->b != b->b) return a->b < b->b ? -1 : 1;
    if (a->x != b->x) return a->x < b->x ? -1 : 1;
    if (a->y != b->y) return a->y < b->y ? -1 : 1;
    if (a->z != b->z) return a->z < b->z ? -1 : 1;
    return 0;
}

#define ORACLE_OK 0
#define ORACLE_ERR_RANGE (-2)
#define ORACLE_ERR_DUPLICATE (-3)
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-6)

/* Builds kmap [n][K] (K = 27 for ksize 3, 1 for ksize 1). Returns 0, or a
 * negative code for a site outside the grid/batch or a duplicated site. */
int oracle_kernel_map(const int32_t* coords, int64_t n, const int32_t* grid, int32_t batch,
                      int32_t ksize, int32_t* kmap) {
    if (n < 0 || (ksize != 1 && ksize != 3)) return ORACLE_ERR_ARG;
    const int K = ksize == 3 ? 27 : 1;
    if (n == 0) return ORACLE_OK;
    site_t* sites = (site_t*)malloc((size_t)n * sizeof(site_t));
    if (!sites) return ORACLE_ERR_NOMEM;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t* c = coords + 4 * i;
        if (c[0] < 0 || c[0] >= batch || c[1] < 0 || c[1] >= grid[0] || c[2] < 0 ||
            c[2] >= grid[1] || c[3] < 0 || c[3] >= grid[2]) {
            free(sites);
            return ORACLE_ERR_RANGE;
        }
        sites[i].b = c[0];
        sites[i].x = c[1];
        sites[i].y = c[2];
        sites[i].z = c[3];
        sites[i].row = i;
    }
    qsort(sites, (size_t)n, sizeof(site_t), cmp_site);
    for (int64_t i = 1; i < n; ++i) {
        if (cmp_site(&sites[i - 1], &sites[i]) == 0) {
            free(sites);
            return ORACLE_ERR_DUPLICATE;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int32_t* c = coords + 4 * i;
        for (int k = 0; k < K; ++k) {
            int dx = 0, dy = 0, dz = 0;
            if (K == 27) {
                dx = k / 9 - 1;
                dy = (k / 3) % 3 - 1;
                dz = k % 3 - 1;
            }
            site_t q;
            q.b = c[0];
            q.x = c[1] + dx;
            q.y = c[2] + dy;
            q.z = c[3] + dz;
            q.row = -1;
            int32_t found = -1;
            if (q.x >= 0 && q.x < grid[0] && q.y >= 0 && q.y < grid[1] && q.z >= 0 &&
                q.z < grid[2]) {
                const site_t* hit =
                    (const site_t*)bsearch(&q, sites, (size_t)n, sizeof(site_t), cmp_site);
                if (hit) found = (int32_t)hit->row;
            }
            kmap[i * K + k] = found;
        }
    }
    free(sites);
    return ORACLE_OK;
}

/* out[r][o] for the selected rows, in fp64. feats [n][cin], W [K][cin][cout]
 * (both already up-cast to fp64), bias [cout] or NULL, kmap [n][K]. */
int oracle_submconv_rows(const int32_t* kmap, int64_t n, int32_t K, const double* feats,
                         const double* W, const double* bias, int32_t cin, int32_t cout,
                         const int64_t* rows, int64_t nrows, double* out) {
    if (n < 0 || nrows < 0 || cin <= 0 || cout <= 0 || (K != 1 && K != 27)) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        double* o = out + r * (int64_t)cout;
        for (int32_t q = 0; q < cout; ++q) o[q] = bias ? bias[q] : 0.0;
        if (i < 0 || i >= n) continue;
        for (int32_t k = 0; k < K; ++k) {
            const int32_t j = kmap[i * K + k];
            if (j < 0) continue;
            const double* f = feats + (int64_t)j * cin;
            const double* w = W + (int64_t)k * cin * cout;
            for (int32_t c = 0; c < cin; ++c) {
                const double fc = f[c];
                const double* wr = w + (int64_t)c * cout;
                for (int32_t q = 0; q < cout; ++q) o[q] += fc * wr[q];
            }
        }
    }
    return ORACLE_OK;
}

/* Input gradient for the selected rows j, in fp64: the forward term
 * feats[j] @ W[k] of out[i] exists exactly when coords[i] + d_k = coords[j],
 * i.e. when a site i sits at coords[j] - d_k; it returns grad_out[i] @ W[k]^T
 * to row j. The site at coords[j] - d_k is found by the same sort + binary
 * search as oracle_kernel_map (not through kmap). grad_out [n][cout] and
 * W [K][cin][cout] up-cast to fp64; out [nrows][cin]. */
int oracle_backward_input_rows(const int32_t* coords, int64_t n, const int32_t* grid,
                               int32_t batch, int32_t ksize, const double* grad_out,
                               const double* W, int32_t cin, int32_t cout, const int64_t* rows,
                               int64_t nrows, double* out) {
    if (n < 0 || nrows < 0 || cin <= 0 || cout <= 0 || (ksize != 1 && ksize != 3))
        return ORACLE_ERR_ARG;
    const int K = ksize == 3 ? 27 : 1;
    site_t* sites = (site_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(site_t));
    if (!sites) return ORACLE_ERR_NOMEM;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t* c = coords + 4 * i;
        if (c[0] < 0 || c[0] >= batch || c[1] < 0 || c[1] >= grid[0] || c[2] < 0 ||
            c[2] >= grid[1] || c[3] < 0 || c[3] >= grid[2]) {
            free(sites);
            return ORACLE_ERR_RANGE;
        }
        sites[i].b = c[0];
        sites[i].x = c[1];
        sites[i].y = c[2];
        sites[i].z = c[3];
        sites[i].row = i;
    }
    qsort(sites, (size_t)n, sizeof(site_t), cmp_site);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t j = rows ? rows[r] : r;
        double* o = out + r * (int64_t)cin;
        for (int32_t c = 0; c < cin; ++c) o[c] = 0.0;
        if (j < 0 || j >= n) continue;
        const int32_t* cj = coords + 4 * j;
        for (int32_t k = 0; k < K; ++k) {
            const int dx = K == 27 ? k / 9 - 1 : 0, dy = K == 27 ? (k / 3) % 3 - 1 : 0,
                      dz = K == 27 ? k % 3 - 1 : 0;
            site_t key = {cj[0], cj[1] - dx, cj[2] - dy, cj[3] - dz, 0};
            if (key.x < 0 || key.x >= grid[0] || key.y < 0 || key.y >= grid[1] || key.z < 0 ||
                key.z >= grid[2])
                continue;
            const site_t* hit = (const site_t*)bsearch(&key, sites, (size_t)n, sizeof(site_t), cmp_site);
            if (!hit) continue;
            const double* g = grad_out + hit->row * (int64_t)cout;
            const double* w = W + (int64_t)k * cin * cout;
            for (int32_t c = 0; c < cin; ++c) {
                const double* wr = w + (int64_t)c * cout;
                double s = 0.0;
                for (int32_t q = 0; q < cout; ++q) s += wr[q] * g[q];
                o[c] += s;
            }
        }
    }
    free(sites);
    return ORACLE_OK;
}

/* Weight gradient in fp64: dW[k][c][q] = sum over rows i with
 * kmap[i][k] = j != -1 of feats[j][c] * grad_out[i][q]. */
int oracle_backward_weight(const int32_t* kmap, int64_t n, int32_t K, const double* feats,
                           const double* grad_out, int32_t cin, int32_t cout, double* dw) {
    if (n < 0 || cin <= 0 || cout <= 0 || (K != 1 && K != 27)) return ORACLE_ERR_ARG;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t k = 0; k < K; ++k) {
        for (int32_t c = 0; c < cin; ++c) {
            double* o = dw + ((int64_t)k * cin + c) * cout;
            for (int32_t q = 0; q < cout; ++q) o[q] = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                const int32_t j = kmap[i * K + k];
                if (j < 0) continue;
                const double f = feats[(int64_t)j * cin + c];
                const double* g = grad_out + i * (int64_t)cout;
                for (int32_t q = 0; q < cout; ++q) o[q] += f * g[q];
            }
        }
    }
    return ORACLE_OK;
}

/* Threads an OpenMP parallel region uses here (for reporting). */
int oracle_num_threads(void) {
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
