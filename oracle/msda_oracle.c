/*
 * msda_oracle.c — plain, slow, obviously correct fp64 CPU oracle for the
 * multi-scale deformable attention core of Deformable DETR.
 *
 * TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
 * baseline are the only callers. It shares no code, header, table or helper
 * with the HIP library and never calls it.
 *
 * The operation has a plain definition (a sum of bilinear samples weighted by
 * attention weights), so the oracle is that definition written out in nested
 * loops in the order the pages state it, with no blocking, fusion or
 * reordering. It runs on one thread unless msda_oracle_set_threads asks for
 * more (the host-core baseline does): the forward then splits its queries
 * over threads, and the backward its (image, head) pairs, whose grad_value
 * slices are disjoint. Every output element is then still computed by one
 * thread with the same operations in the same order, so the results are
 * bit-identical for every thread count.
 *
 * Citations (page title, section):
 *   [P1] juhe.plus notes on a pure-PyTorch Deformable-DETR debug build,
 *        "Key point 1: get_reference_points" and "decoder data flow".
 *   [P2] "Deformable DETR model walkthrough (with source + paper)" (xdnf.cn),
 *        sections "overall flow", "transformer", "encoder" and "Decoder".
 *   [P4] "Deformable DETR: Deformable Transformers for End-to-End Object
 *        Detection" notes (phdsky.com), "Core insights / Insight 2" and
 *        "Key code".
 *
 * Readings taken where the pages are silent:
 *   - align_corners=False pixel convention: a normalised coordinate u in [0,1]
 *     maps to the continuous pixel coordinate u*W - 0.5, so pixel j's centre is
 *     u = (j + 0.5) / W. ([P2] "encoder": the core rescales locations to
 *     [-1, 1] and samples bilinearly with align_corners=False.)
 *   - zero padding: a corner outside the map reads 0; the sample is not
 *     renormalised ([P2] "encoder": padding_mode zeros).
 *   - the cell of a sample is [floor(x), floor(x)+1]; at an integer coordinate
 *     the derivative with respect to the location is the right derivative.
 *   - a non-finite or far-outside location contributes 0 and gets zero
 *     gradients.
 *   - the backward is the exact derivative of the forward (the pages train the
 *     op end to end through autograd and print no formula for it).
 */
#include "msda_oracle.h"

#include <math.h>
#include <string.h>

/* Threads of the forward and backward loops (OpenMP; 1 = serial). */
static int g_threads = 1;

void msda_oracle_set_threads(int n) { g_threads = n > 0 ? n : 1; }

int64_t msda_oracle_level_start_index(int L, const int64_t *shapes, int64_t *lsi_out)
{
    int64_t start = 0;
    for (int l = 0; l < L; ++l) {
        lsi_out[l] = start;
        start += shapes[2 * l + 0] * shapes[2 * l + 1];
    }
    return start;
}

/* [P1] "Key point 1" / [P2] "encoder": every pixel (i, j) of level lq is one
 * query; its centre normalised by the valid extent of its own level is
 * ((j+0.5)/(vr_x*W), (i+0.5)/(vr_y*H)); that point is then expressed on every
 * level l by multiplying with level l's valid ratios. */
void msda_oracle_reference_points_encoder(int B, int L, const int64_t *shapes,
                                          const double *valid_ratios, double *out)
{
    int64_t S = 0;
    for (int l = 0; l < L; ++l) S += shapes[2 * l] * shapes[2 * l + 1];

    for (int b = 0; b < B; ++b) {
        int64_t q = 0;
        for (int lq = 0; lq < L; ++lq) {
            const int64_t H = shapes[2 * lq + 0];
            const int64_t W = shapes[2 * lq + 1];
            const double vr_x_own = valid_ratios[(b * L + lq) * 2 + 0];
            const double vr_y_own = valid_ratios[(b * L + lq) * 2 + 1];
            for (int64_t i = 0; i < H; ++i) {
                for (int64_t j = 0; j < W; ++j, ++q) {
                    const double rx = ((double)j + 0.5) / (vr_x_own * (double)W);
                    const double ry = ((double)i + 0.5) / (vr_y_own * (double)H);
                    for (int l = 0; l < L; ++l) {
                        double *o = out + ((b * S + q) * L + l) * 2;
                        o[0] = rx * valid_ratios[(b * L + l) * 2 + 0];
                        o[1] = ry * valid_ratios[(b * L + l) * 2 + 1];
                    }
                }
            }
        }
    }
}

/* [P1] "decoder data flow", [P2] "Decoder": the decoder's normalised
 * reference point is scaled into each level's valid region. */
void msda_oracle_reference_points_decoder(int B, int64_t Nq, int L, const double *u,
                                          const double *valid_ratios, double *out)
{
    for (int b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int l = 0; l < L; ++l)
                for (int c = 0; c < 2; ++c)
                    out[((b * Nq + q) * L + l) * 2 + c] =
                        u[(b * Nq + q) * 2 + c] * valid_ratios[(b * L + l) * 2 + c];
}

/* [P4] "Key code" (MSDeformAttn.forward) and [P2] "encoder": where the
 * padding mask marks a position of the flattened value sequence, the
 * projected value is filled with zeros before sampling. The same map sends a
 * gradient with respect to the filled value back to the unfilled one (zero at
 * the masked positions), so it serves the backward as well. mask is [B,S]
 * (nonzero = padded); each of the S rows holds C = M*D numbers. */
void msda_oracle_masked_fill(int B, int64_t S, int64_t C, const unsigned char *mask, const double *x,
                             double *out)
{
    for (int b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t c = 0; c < C; ++c)
                out[(b * S + s) * C + c] = mask[b * S + s] ? 0.0 : x[(b * S + s) * C + c];
}

/* [P2] "encoder", [P4] "Key code": offsets are predicted in pixels of level l
 * and normalised by (W_l, H_l) before being added to the reference point. */
void msda_oracle_sampling_locations(int B, int64_t Nq, int M, int L, int K,
                                    const int64_t *shapes, const double *ref,
                                    const double *offset_px, double *loc)
{
    for (int b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int m = 0; m < M; ++m)
                for (int l = 0; l < L; ++l) {
                    const double H = (double)shapes[2 * l + 0];
                    const double W = (double)shapes[2 * l + 1];
                    const double *r = ref + ((b * Nq + q) * L + l) * 2;
                    for (int k = 0; k < K; ++k) {
                        const int64_t idx = ((((b * Nq + q) * M + m) * L + l) * K + k) * 2;
                        loc[idx + 0] = r[0] + offset_px[idx + 0] / W;
                        loc[idx + 1] = r[1] + offset_px[idx + 1] / H;
                    }
                }
}

/* [P4] "Insight 2": A is normalised so that it sums to 1 over all L*K samples
 * of one query and head; [P2] "encoder" applies softmax over that axis. */
void msda_oracle_softmax(int64_t rows, int n, const double *logits, double *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *x = logits + r * n;
        double *y = out + r * n;
        double mx = x[0];
        for (int i = 1; i < n; ++i)
            if (x[i] > mx) mx = x[i];
        double sum = 0.0;
        for (int i = 0; i < n; ++i) {
            y[i] = exp(x[i] - mx);
            sum += y[i];
        }
        for (int i = 0; i < n; ++i) y[i] /= sum;
    }
}

/* Sampling locations from 4-d box references (cx, cy, w, h) per query and
 * level, the iterative-refinement form of the walkthrough page's MSDeformAttn
 * source ("encoder" section, the reference_points.shape[-1] == 4 branch): the
 * offsets are taken relative to the box size,
 *   loc = ref[b,q,l,0:2] + offset / K * ref[b,q,l,2:4] * 0.5. */
void msda_oracle_sampling_locations_box(int B, int64_t Nq, int M, int L, int K, const double *ref,
                                        const double *offset, double *loc)
{
    for (int b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int m = 0; m < M; ++m)
                for (int l = 0; l < L; ++l) {
                    const double *r = ref + ((b * Nq + q) * L + l) * 4;
                    for (int k = 0; k < K; ++k) {
                        const int64_t idx = ((((b * Nq + q) * M + m) * L + l) * K + k) * 2;
                        loc[idx + 0] = r[0] + offset[idx + 0] / (double)K * r[2] * 0.5;
                        loc[idx + 1] = r[1] + offset[idx + 1] / (double)K * r[3] * 0.5;
                    }
                }
}

/* Its backward: grad_offset = grad_loc * ref_wh * 0.5 / K;
 * grad_ref[0:2] = sum over m, k of grad_loc, grad_ref[2:4] = sum over m, k of
 * grad_loc * offset * 0.5 / K. grad_ref [B,Nq,L,4] may be NULL. */
void msda_oracle_sampling_locations_box_backward(int B, int64_t Nq, int M, int L, int K, const double *ref,
                                                 const double *offset, const double *grad_loc, double *grad_ref,
                                                 double *grad_offset)
{
    if (grad_ref)
        for (int64_t i = 0; i < (int64_t)B * Nq * L * 4; ++i) grad_ref[i] = 0.0;
    for (int b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int m = 0; m < M; ++m)
                for (int l = 0; l < L; ++l) {
                    const double *r = ref + ((b * Nq + q) * L + l) * 4;
                    for (int k = 0; k < K; ++k) {
                        const int64_t idx = ((((b * Nq + q) * M + m) * L + l) * K + k) * 2;
                        grad_offset[idx + 0] = grad_loc[idx + 0] * r[2] * 0.5 / (double)K;
                        grad_offset[idx + 1] = grad_loc[idx + 1] * r[3] * 0.5 / (double)K;
                        if (grad_ref) {
                            double *gr = grad_ref + ((b * Nq + q) * L + l) * 4;
                            gr[0] += grad_loc[idx + 0];
                            gr[1] += grad_loc[idx + 1];
                            gr[2] += grad_loc[idx + 0] * offset[idx + 0] * 0.5 / (double)K;
                            gr[3] += grad_loc[idx + 1] * offset[idx + 1] * 0.5 / (double)K;
                        }
                    }
                }
}

/* Backward of the L*K softmax ([P4] "Insight 2" normalisation): with
 * A = softmax(x) over one row, dA_i/dx_j = A_i (delta_ij - A_j), so
 * grad_x_i = A_i (grad_A_i - sum_j A_j grad_A_j). */
void msda_oracle_softmax_backward(int64_t rows, int n, const double *attn, const double *grad_attn,
                                  double *grad_logits)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *a = attn + r * n;
        const double *ga = grad_attn + r * n;
        double dot = 0.0;
        for (int j = 0; j < n; ++j) dot += a[j] * ga[j];
        for (int i = 0; i < n; ++i) grad_logits[r * n + i] = a[i] * (ga[i] - dot);
    }
}

/* Backward of the location formation ([P2] "encoder", [P4] "Key code"):
 * loc = ref[b,q,l] + offset_px / (W_l, H_l), so grad_offset_px = grad_loc /
 * (W_l, H_l) and grad_ref[b,q,l] = sum over heads and points of grad_loc.
 * grad_ref may be NULL. */
void msda_oracle_sampling_locations_backward(int B, int64_t Nq, int M, int L, int K,
                                             const int64_t *shapes, const double *grad_loc,
                                             double *grad_ref, double *grad_offset_px)
{
    if (grad_ref)
        for (int64_t i = 0; i < (int64_t)B * Nq * L * 2; ++i) grad_ref[i] = 0.0;
    for (int b = 0; b < B; ++b)
        for (int64_t q = 0; q < Nq; ++q)
            for (int m = 0; m < M; ++m)
                for (int l = 0; l < L; ++l) {
                    const double H = (double)shapes[2 * l + 0];
                    const double W = (double)shapes[2 * l + 1];
                    for (int k = 0; k < K; ++k) {
                        const int64_t idx = ((((b * Nq + q) * M + m) * L + l) * K + k) * 2;
                        grad_offset_px[idx + 0] = grad_loc[idx + 0] / W;
                        grad_offset_px[idx + 1] = grad_loc[idx + 1] / H;
                        if (grad_ref) {
                            double *gr = grad_ref + ((b * Nq + q) * L + l) * 2;
                            gr[0] += grad_loc[idx + 0];
                            gr[1] += grad_loc[idx + 1];
                        }
                    }
                }
}

/* One bilinear sample's geometry on a level of size H x W: the pixel
 * coordinates of the top-left corner of its cell and the fractional parts.
 * Returns 0 if the location is non-finite or so far out that no corner can be
 * inside the map (then the sample contributes nothing). */
static int sample_cell(double lx, double ly, int64_t H, int64_t W,
                       int64_t *x0, int64_t *y0, double *fx, double *fy)
{
    const double x = lx * (double)W - 0.5; /* align_corners=False */
    const double y = ly * (double)H - 0.5;
    if (!(x > -2.0 && x < (double)W + 1.0 && y > -2.0 && y < (double)H + 1.0))
        return 0;
    const double fx0 = floor(x);
    const double fy0 = floor(y);
    *x0 = (int64_t)fx0;
    *y0 = (int64_t)fy0;
    *fx = x - fx0;
    *fy = y - fy0;
    return 1;
}

static int inside(int64_t xi, int64_t yi, int64_t H, int64_t W)
{
    return xi >= 0 && xi < W && yi >= 0 && yi < H;
}

static void forward_one_query(int b, int64_t q, int64_t S, int64_t Nq, int M, int D,
                              int L, int K, const int64_t *shapes, const int64_t *lsi,
                              const double *value, const double *loc,
                              const double *attn, double *out_row /* [M*D] */)
{
    for (int m = 0; m < M; ++m) {
        double *acc = out_row + m * D;
        for (int d = 0; d < D; ++d) acc[d] = 0.0;
        for (int l = 0; l < L; ++l) {
            const int64_t H = shapes[2 * l + 0];
            const int64_t W = shapes[2 * l + 1];
            for (int k = 0; k < K; ++k) {
                const int64_t sidx = (((b * Nq + q) * M + m) * L + l) * K + k;
                const double a = attn[sidx];
                int64_t x0, y0;
                double fx, fy;
                if (!sample_cell(loc[2 * sidx], loc[2 * sidx + 1], H, W, &x0, &y0, &fx, &fy))
                    continue;
                for (int dy = 0; dy < 2; ++dy) {
                    for (int dx = 0; dx < 2; ++dx) {
                        const int64_t xi = x0 + dx, yi = y0 + dy;
                        if (!inside(xi, yi, H, W)) continue; /* zero padding */
                        const double w = (dx ? fx : 1.0 - fx) * (dy ? fy : 1.0 - fy);
                        const int64_t s = lsi[l] + yi * W + xi;
                        const double *v = value + ((b * S + s) * M + m) * D;
                        for (int d = 0; d < D; ++d) acc[d] += a * w * v[d];
                    }
                }
            }
        }
    }
}

void msda_oracle_forward(int B, int64_t S, int64_t Nq, int M, int D, int L, int K,
                         const int64_t *shapes, const int64_t *lsi,
                         const double *value, const double *loc, const double *attn,
                         const int64_t *query_ids, int64_t n_ids, double *out)
{
    if (query_ids) {
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads)
        for (int64_t i = 0; i < n_ids; ++i) {
            const int b = (int)(query_ids[i] / Nq);
            const int64_t q = query_ids[i] % Nq;
            forward_one_query(b, q, S, Nq, M, D, L, K, shapes, lsi, value, loc, attn,
                              out + i * (int64_t)M * D);
        }
        return;
    }
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads)
    for (int64_t bq = 0; bq < (int64_t)B * Nq; ++bq)
        forward_one_query((int)(bq / Nq), bq % Nq, S, Nq, M, D, L, K, shapes, lsi, value, loc, attn,
                          out + bq * (int64_t)M * D);
}

/* Exact derivative of the forward. With x = lx*W - 0.5 and
 * w_c = (dx ? fx : 1-fx) * (dy ? fy : 1-fy):
 *   d out_d / d a    = sum_c w_c v_c[d]
 *   d out_d / d v_c  = a * w_c
 *   d out_d / d lx   = a * W * sum_c (d w_c / d fx) v_c[d]
 *   d out_d / d ly   = a * H * sum_c (d w_c / d fy) v_c[d]
 * with d w_c/d fx = (dx ? 1 : -1) * (dy ? fy : 1-fy) and likewise for fy. */
/* One (image b, head m) of the backward: every query's samples of head m, in
 * query order. The grad_value slice [b, :, m, :] receives contributions from
 * this pair only, and in the same order as from a loop over b, q, m. */
static void backward_one_head(int b, int m, int64_t S, int64_t Nq, int M, int D, int L, int K,
                              const int64_t *shapes, const int64_t *lsi,
                              const double *value, const double *loc, const double *attn,
                              const double *grad_out, double *grad_value,
                              double *grad_loc, double *grad_attn)
{
    for (int64_t q = 0; q < Nq; ++q) {
        const double *g = grad_out + ((b * Nq + q) * M + m) * D;
        for (int l = 0; l < L; ++l) {
            const int64_t H = shapes[2 * l + 0];
            const int64_t W = shapes[2 * l + 1];
            for (int k = 0; k < K; ++k) {
                const int64_t sidx = (((b * Nq + q) * M + m) * L + l) * K + k;
                const double a = attn[sidx];
                double ga = 0.0, glx = 0.0, gly = 0.0;
                int64_t x0, y0;
                double fx, fy;
                if (sample_cell(loc[2 * sidx], loc[2 * sidx + 1], H, W, &x0, &y0, &fx, &fy)) {
                    for (int dy = 0; dy < 2; ++dy) {
                        for (int dx = 0; dx < 2; ++dx) {
                            const int64_t xi = x0 + dx, yi = y0 + dy;
                            if (!inside(xi, yi, H, W)) continue;
                            const double wx = dx ? fx : 1.0 - fx;
                            const double wy = dy ? fy : 1.0 - fy;
                            const double dwx = dx ? 1.0 : -1.0; /* d wx / d fx */
                            const double dwy = dy ? 1.0 : -1.0; /* d wy / d fy */
                            const int64_t s = lsi[l] + yi * W + xi;
                            const double *v = value + ((b * S + s) * M + m) * D;
                            double *gv = grad_value + ((b * S + s) * M + m) * D;
                            double gdotv = 0.0;
                            for (int d = 0; d < D; ++d) {
                                gdotv += g[d] * v[d];
                                gv[d] += a * wx * wy * g[d];
                            }
                            ga += wx * wy * gdotv;
                            glx += dwx * wy * gdotv;
                            gly += wx * dwy * gdotv;
                        }
                    }
                }
                grad_attn[sidx] = ga;
                grad_loc[2 * sidx + 0] = a * (double)W * glx;
                grad_loc[2 * sidx + 1] = a * (double)H * gly;
            }
        }
    }
}

void msda_oracle_backward(int B, int64_t S, int64_t Nq, int M, int D, int L, int K,
                          const int64_t *shapes, const int64_t *lsi,
                          const double *value, const double *loc, const double *attn,
                          const double *grad_out, double *grad_value,
                          double *grad_loc, double *grad_attn)
{
    memset(grad_value, 0, sizeof(double) * (size_t)B * (size_t)S * (size_t)M * (size_t)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(g_threads)
    for (int b = 0; b < B; ++b)
        for (int m = 0; m < M; ++m)
            backward_one_head(b, m, S, Nq, M, D, L, K, shapes, lsi, value, loc, attn, grad_out,
                              grad_value, grad_loc, grad_attn);
}
