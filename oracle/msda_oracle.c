/*
 * msda_oracle.c -- plain CPU oracle for the multi-scale deformable attention
 * (MSDeformAttn) sampling core, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; it is compiled by gcc with
 * -O2 -ffp-contract=off so that no multiply-add is fused behind its back.
 *
 * What it computes (sources are the web pages this project follows):
 *
 *  - "Deformable attention: multi-scale sparse sampling and detection
 *    practice", section 2.2 (the multi-scale formula): for query q and head m
 *    the core returns  sum_l sum_k A[m,l,q,k] * x^l_m(p_q + dp[m,l,q,k]),
 *    where x^l_m is head m's slice of the (already projected) value of level
 *    l.  The value and output projections stay outside the core.
 *  - same page, section 2.3 (bilinear interpolation): the sample at a
 *    non-integer (x, y) is the sum over the four integer neighbours
 *    (x0,y0), (x0+1,y0), (x0,y0+1), (x0+1,y0+1) of the neighbour's value
 *    times the tent weight max(0, 1-|x-xi|) * max(0, 1-|y-yi|); a neighbour
 *    outside the feature map contributes zero.
 *  - same page, sections 2.3 and 3.2 (the grid_sample module with
 *    align_corners=False, the default convention here): a normalized
 *    coordinate u in [0,1] maps to the
 *    pixel coordinate u*W - 0.5 along the width (W) and v*H - 0.5 along the
 *    height (H); the last axis of a location is (x, y); each row of the
 *    level table is (H, W); the head outputs are concatenated head-major.
 *  - "Deformable DETR" tutorial, section 3.3: phi_l maps the normalized
 *    reference to level l's resolution.
 *
 * The backward pass is the exact derivative of that definition (the pages
 * state only that the interpolation is differentiable): with the tent
 * weights tx(x) = max(0, 1-|x-xi|) and ty(y), the derivative of tx is -1 for
 * the left neighbour x0 and +1 for the right neighbour x0+1 inside the cell
 * [x0, x0+1), and d x / d u = W, d y / d v = H.
 *
 * Coordinate modes (bit flags)
 *   bit 0 clear ("spec"): x = fmaf(u, (float)W, -0.5f), x0 = floorf(x), in fp32
 *                      with one rounding, as the GPU library does; everything
 *                      after the floor is fp64.
 *   bit 0 set ("double"): every coordinate step in fp64 (for finite differences).
 *   bit 1 ("align corners"): the other pixel convention, x = u*(W-1) and
 *                      y = v*(H-1) (grid_sample with align_corners=True): the
 *                      first page, section 2.3, advises making align_corners and
 *                      the coordinate scale a configuration option, and its
 *                      section 6 notes that some inference engines default to
 *                      True.  In spec mode the product is one fp32 multiply;
 *                      d x / d u = W-1 and d y / d v = H-1.
 * Accumulation is always fp64, in the order l, k, neighbour.
 *
 * Non-finite coordinates: every neighbour test fails, so such a point
 * contributes nothing and receives zero gradients.
 *
 * Layouts (dense, row-major):
 *   value            [B, Nv, M, D]          float
 *   spatial_shapes   [L, 2]  rows (H, W)    int64
 *   level_start      [L]                    int64
 *   sampling_loc     [B, Nq, M, L, K, 2]    float, last axis (x, y)
 *   attn_weight      [B, Nq, M, L, K]       float
 *   out              [B, Nq, M*D]           double
 *   grad_out         [B, Nq, M*D]           float
 *   grad_value       [B, Nv, M, D]          double (overwritten)
 *   grad_loc         [B, Nq, M, L, K, 2]    double
 *   grad_attn        [B, Nq, M, L, K]       double
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One neighbour of a sampling point: its flat pixel index within the
 * flattened multi-level sequence, its tent weights and their derivatives. */
typedef struct {
    int64_t pix;      /* start_l + yi*W + xi, or -1 when outside the map */
    double wx, wy;    /* tent weights along x and y                        */
    double dwx, dwy;  /* d wx / d x and d wy / d y                         */
} neighbour;

#define MODE_DOUBLE 1
#define MODE_ALIGN 2

/* d x / d u on an axis of n pixels */
static double pixel_scale(int64_t n, int mode)
{
    return (mode & MODE_ALIGN) ? (double)(n - 1) : (double)n;
}

/* Pixel coordinate of a normalized coordinate u on an axis of n pixels,
 * floored; *px receives the continuous coordinate. */
static double pixel_coord(float u, int64_t n, int mode, double *px)
{
    if (!(mode & MODE_DOUBLE)) {
        float p = (mode & MODE_ALIGN) ? u * (float)(n - 1) : fmaf(u, (float)n, -0.5f);
        *px = (double)p;
        return (double)floorf(p);
    }
    double p = (mode & MODE_ALIGN) ? (double)u * (double)(n - 1)
                                   : (double)u * (double)n - 0.5;
    *px = p;
    return floor(p);
}

/* The four integer neighbours of (u, v) on level (H, W) starting at start. */
static void neighbours(float u, float v, int64_t H, int64_t W, int64_t start,
                       int mode, neighbour nb[4])
{
    double x, y;
    double x0 = pixel_coord(u, W, mode, &x);
    double y0 = pixel_coord(v, H, mode, &y);
    for (int c = 0; c < 4; ++c) {
        double xi = x0 + (double)(c & 1);
        double yi = y0 + (double)(c >> 1);
        neighbour *n = &nb[c];
        int inside = (xi >= 0.0) && (xi <= (double)(W - 1)) &&
                     (yi >= 0.0) && (yi <= (double)(H - 1));
        if (!inside) {
            n->pix = -1;
            n->wx = n->wy = n->dwx = n->dwy = 0.0;
            continue;
        }
        n->pix = start + (int64_t)yi * W + (int64_t)xi;
        n->wx = fmax(0.0, 1.0 - fabs(x - xi));
        n->wy = fmax(0.0, 1.0 - fabs(y - yi));
        /* inside the cell [x0, x0+1): left neighbour slopes down, right up */
        n->dwx = (c & 1) ? 1.0 : -1.0;
        n->dwy = (c >> 1) ? 1.0 : -1.0;
    }
}

static int check_args(const int64_t *shapes, const int64_t *start, int64_t B,
                      int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                      int64_t K)
{
    if (!shapes || !start) return -1;
    if (B < 0 || Nv < 0 || Nq < 0 || M < 1 || D < 1 || L < 1 || K < 1) return -2;
    int64_t total = 0;
    for (int64_t l = 0; l < L; ++l) {
        if (shapes[2 * l] < 1 || shapes[2 * l + 1] < 1) return -2;
        if (start[l] != total) return -2;
        total += shapes[2 * l] * shapes[2 * l + 1];
    }
    if (total != Nv) return -2;
    return 0;
}

int oracle_forward(const float *value, const int64_t *shapes, const int64_t *start,
                   const float *loc, const float *attn, double *out,
                   int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                   int64_t L, int64_t K, int mode, int threads)
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
                    int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t pt = (((b * Nq + q) * M + m) * L + l) * K + k;
                        double A = (double)attn[pt];
                        neighbour nb[4];
                        neighbours(loc[2 * pt], loc[2 * pt + 1], H, W, start[l], mode, nb);
                        for (int c = 0; c < 4; ++c) {
                            if (nb[c].pix < 0) continue;
                            double w = A * nb[c].wx * nb[c].wy;
                            const float *v = value + ((b * Nv + nb[c].pix) * M + m) * D;
                            for (int64_t d = 0; d < D; ++d) o[d] += w * (double)v[d];
                        }
                    }
                }
            }
    return 0;
}

int oracle_backward(const float *value, const int64_t *shapes, const int64_t *start,
                    const float *loc, const float *attn, const float *grad_out,
                    double *grad_value, double *grad_loc, double *grad_attn,
                    int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                    int64_t L, int64_t K, int mode, int threads)
{
    int rc = check_args(shapes, start, B, Nv, Nq, M, D, L, K);
    if (rc) return rc;
    if (B * Nv * M * D > 0 && !grad_value) return -1;
    if (B * Nq * M > 0 && (!value || !loc || !attn || !grad_out || !grad_loc || !grad_attn))
        return -1;
    if (B * Nv * M * D > 0)
        memset(grad_value, 0, sizeof(double) * (size_t)(B * Nv * M * D));
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
    /* grad_value[b, :, m, :] only receives from points of the same (b, m),
     * so (b, m) slices are disjoint and the sum order stays fixed. */
#pragma omp parallel for schedule(static) collapse(2)
#endif
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t q = 0; q < Nq; ++q) {
                const float *g = grad_out + ((b * Nq + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t pt = (((b * Nq + q) * M + m) * L + l) * K + k;
                        double A = (double)attn[pt];
                        neighbour nb[4];
                        neighbours(loc[2 * pt], loc[2 * pt + 1], H, W, start[l], mode, nb);
                        double gA = 0.0, gx = 0.0, gy = 0.0;
                        for (int c = 0; c < 4; ++c) {
                            if (nb[c].pix < 0) continue;
                            int64_t row = ((b * Nv + nb[c].pix) * M + m) * D;
                            const float *v = value + row;
                            double gv = 0.0; /* <g, value row> */
                            for (int64_t d = 0; d < D; ++d) gv += (double)g[d] * (double)v[d];
                            double w = nb[c].wx * nb[c].wy;
                            gA += w * gv;
                            gx += nb[c].dwx * nb[c].wy * gv;
                            gy += nb[c].wx * nb[c].dwy * gv;
                            double s = A * w;
                            double *gvr = grad_value + row;
                            for (int64_t d = 0; d < D; ++d) gvr[d] += s * (double)g[d];
                        }
                        grad_attn[pt] = gA;
                        grad_loc[2 * pt] = A * gx * pixel_scale(W, mode);
                        grad_loc[2 * pt + 1] = A * gy * pixel_scale(H, mode);
                    }
                }
            }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
