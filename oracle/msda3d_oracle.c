/*
 * msda3d_oracle.c -- plain CPU oracle for the 3-D (trilinear) variant of the
 * multi-scale deformable attention sampling core, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; it is compiled by gcc with
 * -O2 -ffp-contract=off.
 *
 * What it computes.  "Deformable attention: multi-scale sparse sampling and
 * detection practice", section 5.3: for point-cloud detection the sampling
 * points fall on 3-D voxel (or BEV) features instead of 2-D maps, the offsets
 * gain a z component, and bilinear interpolation becomes trilinear -- the 2-D
 * method with one more coordinate.  Read plainly, with the 2-D core of the
 * same page (sections 2.2, 2.3, 3.2) as the template:
 *
 *   out[b,q,m,:] = sum_l sum_k A[b,q,m,l,k] * T_l(value[b,:,m,:], loc[b,q,m,l,k])
 *
 * where level l is a Z_l x H_l x W_l volume flattened z-major
 * (start_l + (z*H_l + y)*W_l + x), a location is normalized (u, v, w) along
 * (x, y, z), the voxel coordinate is x = u*W - 0.5, y = v*H - 0.5,
 * z = w*Z - 0.5 (the grid_sample align_corners=False convention extended to
 * the third axis), and T_l sums the eight integer neighbours
 * (x0 + dx, y0 + dy, z0 + dz), dx, dy, dz in {0, 1}, with the tent weights
 * max(0, 1-|x-xi|) * max(0, 1-|y-yi|) * max(0, 1-|z-zi|); a neighbour outside
 * the volume contributes zero.
 *
 * The backward is the exact derivative: inside the cell [x0, x0+1) the
 * derivative of the x tent is -1 for dx = 0 and +1 for dx = 1 (likewise y, z),
 * and d x / d u = W, d y / d v = H, d z / d w = Z.
 *
 * Coordinate modes (bit flags), as in the 2-D oracle:
 *   bit 0 clear ("spec"): x = fmaf(u, (float)W, -0.5f), floored in fp32 (one
 *                      rounding, as the GPU library); fp64 after the floor.
 *   bit 0 set ("double"): every coordinate step in fp64.
 *   bit 1 ("align corners"): x = u*(W-1), y = v*(H-1), z = w*(Z-1);
 *                      derivatives scaled by (W-1, H-1, Z-1).
 * Accumulation is fp64, in the order l, k, neighbour (dz, dy, dx).
 *
 * Layouts (dense, row-major):
 *   value            [B, Nv, M, D]          float
 *   shapes           [L, 3]  rows (Z, H, W) int64
 *   level_start      [L]                    int64
 *   sampling_loc     [B, Nq, M, L, K, 3]    float, last axis (x, y, z)
 *   attn_weight      [B, Nq, M, L, K]       float
 *   out              [B, Nq, M*D]           double
 *   grad_out         [B, Nq, M*D]           float
 *   grad_value       [B, Nv, M, D]          double (overwritten)
 *   grad_loc         [B, Nq, M, L, K, 3]    double
 *   grad_attn        [B, Nq, M, L, K]       double
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MODE_DOUBLE 1
#define MODE_ALIGN 2

/* One of the eight neighbours of a sampling point. */
typedef struct {
    int64_t vox;            /* start_l + (zi*H + yi)*W + xi, or -1 outside the volume */
    double t[3];            /* tent weights along x, y, z                             */
    double dt[3];           /* their derivatives inside the cell                      */
} corner;

static double voxel_scale(int64_t n, int mode)
{
    return (mode & MODE_ALIGN) ? (double)(n - 1) : (double)n;
}

/* Voxel coordinate of normalized u on an axis of n voxels, floored; *p gets
 * the continuous coordinate. */
static double voxel_coord(float u, int64_t n, int mode, double *p)
{
    if (!(mode & MODE_DOUBLE)) {
        float c = (mode & MODE_ALIGN) ? u * (float)(n - 1) : fmaf(u, (float)n, -0.5f);
        *p = (double)c;
        return (double)floorf(c);
    }
    double c = (mode & MODE_ALIGN) ? (double)u * (double)(n - 1) : (double)u * (double)n - 0.5;
    *p = c;
    return floor(c);
}

/* The eight neighbours of (u, v, w) on a Z x H x W level starting at start;
 * neighbour c has offsets dx = c & 1, dy = (c >> 1) & 1, dz = c >> 2. */
static void corners(const float *uvw, int64_t Z, int64_t H, int64_t W, int64_t start, int mode,
                    corner nb[8])
{
    const int64_t n[3] = {W, H, Z};
    double p[3], f[3];
    for (int a = 0; a < 3; ++a) f[a] = voxel_coord(uvw[a], n[a], mode, &p[a]);
    for (int c = 0; c < 8; ++c) {
        corner *k = &nb[c];
        int inside = 1;
        double idx[3];
        for (int a = 0; a < 3; ++a) {
            int up = (c >> a) & 1;
            idx[a] = f[a] + (double)up;
            inside = inside && idx[a] >= 0.0 && idx[a] <= (double)(n[a] - 1);
            k->t[a] = fmax(0.0, 1.0 - fabs(p[a] - idx[a]));
            k->dt[a] = up ? 1.0 : -1.0;
        }
        if (!inside) {
            k->vox = -1;
            continue;
        }
        k->vox = start + ((int64_t)idx[2] * H + (int64_t)idx[1]) * W + (int64_t)idx[0];
    }
}

static int check_args(const int64_t *shapes, const int64_t *start, int64_t B, int64_t Nv,
                      int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K)
{
    if (!shapes || !start) return -1;
    if (B < 0 || Nv < 0 || Nq < 0 || M < 1 || D < 1 || L < 1 || K < 1) return -2;
    int64_t total = 0;
    for (int64_t l = 0; l < L; ++l) {
        if (shapes[3 * l] < 1 || shapes[3 * l + 1] < 1 || shapes[3 * l + 2] < 1) return -2;
        if (start[l] != total) return -2;
        total += shapes[3 * l] * shapes[3 * l + 1] * shapes[3 * l + 2];
    }
    if (total != Nv) return -2;
    return 0;
}

int oracle3d_forward(const float *value, const int64_t *shapes, const int64_t *start,
                     const float *loc, const float *attn, double *out, int64_t B, int64_t Nv,
                     int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K, int mode,
                     int threads)
{
    int rc = check_args(shapes, start, B, Nv, Nq, M, D, L, K);
    if (rc) return rc;
    if (B * Nq * M * D > 0 && (!value || !loc || !attn || !out)) return -1;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(static) collapse(2)
#endif
    for (int64_t b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int64_t m = 0; m < M; ++m) {
                double *o = out + ((b * Nq + q) * M + m) * D;
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t *s = shapes + 3 * l;
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t pt = (((b * Nq + q) * M + m) * L + l) * K + k;
                        double A = (double)attn[pt];
                        corner nb[8];
                        corners(loc + 3 * pt, s[0], s[1], s[2], start[l], mode, nb);
                        for (int c = 0; c < 8; ++c) {
                            if (nb[c].vox < 0) continue;
                            double w = A * nb[c].t[0] * nb[c].t[1] * nb[c].t[2];
                            const float *v = value + ((b * Nv + nb[c].vox) * M + m) * D;
                            for (int64_t d = 0; d < D; ++d) o[d] += w * (double)v[d];
                        }
                    }
                }
            }
    return 0;
}

int oracle3d_backward(const float *value, const int64_t *shapes, const int64_t *start,
                      const float *loc, const float *attn, const float *grad_out,
                      double *grad_value, double *grad_loc, double *grad_attn, int64_t B,
                      int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K,
                      int mode, int threads)
{
    int rc = check_args(shapes, start, B, Nv, Nq, M, D, L, K);
    if (rc) return rc;
    if (B * Nv * M * D > 0 && !grad_value) return -1;
    if (B * Nq * M > 0 && (!value || !loc || !attn || !grad_out || !grad_loc || !grad_attn))
        return -1;
    if (B * Nv * M * D > 0) memset(grad_value, 0, sizeof(double) * (size_t)(B * Nv * M * D));
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
    /* grad_value[b, :, m, :] receives only from points of the same (b, m) */
#pragma omp parallel for schedule(static) collapse(2)
#endif
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t q = 0; q < Nq; ++q) {
                const float *g = grad_out + ((b * Nq + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t *s = shapes + 3 * l;
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t pt = (((b * Nq + q) * M + m) * L + l) * K + k;
                        double A = (double)attn[pt];
                        corner nb[8];
                        corners(loc + 3 * pt, s[0], s[1], s[2], start[l], mode, nb);
                        double gA = 0.0, gd[3] = {0.0, 0.0, 0.0};
                        for (int c = 0; c < 8; ++c) {
                            if (nb[c].vox < 0) continue;
                            int64_t row = ((b * Nv + nb[c].vox) * M + m) * D;
                            const float *v = value + row;
                            double gv = 0.0; /* <g, value row> */
                            for (int64_t d = 0; d < D; ++d) gv += (double)g[d] * (double)v[d];
                            const double *t = nb[c].t, *dt = nb[c].dt;
                            gA += t[0] * t[1] * t[2] * gv;
                            gd[0] += dt[0] * t[1] * t[2] * gv;
                            gd[1] += t[0] * dt[1] * t[2] * gv;
                            gd[2] += t[0] * t[1] * dt[2] * gv;
                            double sc = A * t[0] * t[1] * t[2];
                            double *gvr = grad_value + row;
                            for (int64_t d = 0; d < D; ++d) gvr[d] += sc * (double)g[d];
                        }
                        grad_attn[pt] = gA;
                        grad_loc[3 * pt] = A * gd[0] * voxel_scale(s[2], mode);
                        grad_loc[3 * pt + 1] = A * gd[1] * voxel_scale(s[1], mode);
                        grad_loc[3 * pt + 2] = A * gd[2] * voxel_scale(s[0], mode);
                    }
                }
            }
    return 0;
}
