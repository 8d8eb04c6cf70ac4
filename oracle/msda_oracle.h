/*
 * msda_oracle.h — plain fp64 CPU oracle for multi-scale deformable attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load or call this code. The product library never
 * links, includes or calls it, and it shares no code with the HIP path.
 *
 * All arrays are dense, row-major, batch-first host arrays of double. Callers
 * upcast fp32 / bf16 inputs to double exactly before calling.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] juhe.plus notes on a pure-PyTorch Deformable-DETR debug build,
 *        "Key point 1: get_reference_points" and "decoder data flow".
 *   [P2] "Deformable DETR model walkthrough (with source + paper)" (xdnf.cn),
 *        sections "overall flow", "transformer", "encoder", "Decoder".
 *   [P4] "Deformable DETR: Deformable Transformers for End-to-End Object
 *        Detection" notes (phdsky.com), "Core insights / Insight 2"
 *        (the MSDeformAttn equation) and "Key code".
 */
#ifndef MSDA_ORACLE_H
#define MSDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exclusive prefix sum of H_l*W_l over levels ([P2] "transformer": the start
 * offset of each level inside the flattened sequence). shapes is [L][2]=(H,W).
 * Returns S = sum H_l*W_l. */
int64_t msda_oracle_level_start_index(int L, const int64_t *shapes, int64_t *lsi_out);

/* Encoder reference points ([P1] "Key point 1", [P2] "encoder"):
 * out[b, q, l, :] for q the pixel (i, j) of level lq (row-major within a level,
 * levels concatenated), shape [B, S, L, 2], (x, y) order. */
void msda_oracle_reference_points_encoder(int B, int L, const int64_t *shapes,
                                          const double *valid_ratios /* [B,L,2] */,
                                          double *out /* [B,S,L,2] */);

/* Decoder reference points ([P1] "decoder data flow", [P2] "Decoder"):
 * out[b,q,l,:] = u[b,q,:] * valid_ratios[b,l,:], shape [B,Nq,L,2]. */
void msda_oracle_reference_points_decoder(int B, int64_t Nq, int L,
                                          const double *u /* [B,Nq,2] */,
                                          const double *valid_ratios /* [B,L,2] */,
                                          double *out /* [B,Nq,L,2] */);

/* Sampling locations from 2-d references ([P2] "encoder", [P4] "Key code"):
 * loc[b,q,m,l,k,:] = ref[b,q,l,:] + offset_px[b,q,m,l,k,:] / (W_l, H_l). */
void msda_oracle_sampling_locations(int B, int64_t Nq, int M, int L, int K,
                                    const int64_t *shapes,
                                    const double *ref /* [B,Nq,L,2] */,
                                    const double *offset_px /* [B,Nq,M,L,K,2] */,
                                    double *loc /* [B,Nq,M,L,K,2] */);

/* Softmax over the last axis of length n, for `rows` rows
 * ([P4] "Insight 2": the weights of one query and head sum to 1 over all
 * levels and points, so n = L*K). */
void msda_oracle_softmax(int64_t rows, int n, const double *logits, double *out);

/* Locations from 4-d box references [B,Nq,L,4] = (cx, cy, w, h) ([P2]
 * MSDeformAttn source, the 4-d reference branch): loc = ref_xy + offset / K *
 * ref_wh * 0.5, and its backward (grad_ref [B,Nq,L,4] may be NULL). */
void msda_oracle_sampling_locations_box(int B, int64_t Nq, int M, int L, int K, const double *ref,
                                        const double *offset, double *loc);
void msda_oracle_sampling_locations_box_backward(int B, int64_t Nq, int M, int L, int K, const double *ref,
                                                 const double *offset, const double *grad_loc, double *grad_ref,
                                                 double *grad_offset);

/* Backward of msda_oracle_softmax ([P4] "Insight 2"): grad_logits[r,i] =
 * A[r,i] * (grad_A[r,i] - sum_j A[r,j] grad_A[r,j]). */
void msda_oracle_softmax_backward(int64_t rows, int n, const double *attn, const double *grad_attn,
                                  double *grad_logits);

/* Backward of msda_oracle_sampling_locations: grad_offset_px = grad_loc /
 * (W_l, H_l); grad_ref [B,Nq,L,2] (may be NULL) = sum over m, k of grad_loc. */
void msda_oracle_sampling_locations_backward(int B, int64_t Nq, int M, int L, int K,
                                             const int64_t *shapes, const double *grad_loc,
                                             double *grad_ref, double *grad_offset_px);

/* Threads of msda_oracle_forward and msda_oracle_backward (default 1). The
 * results are bit-identical for every count: each output element is computed
 * by one thread in the serial order. */
void msda_oracle_set_threads(int n);

/* Padding mask ([P4] "Key code", [P2] "encoder"): out = x with the rows of
 * the masked positions set to zero; x and out are [B,S,C], mask [B,S]
 * (nonzero = padded). Also the backward of that step. */
void msda_oracle_masked_fill(int B, int64_t S, int64_t C, const unsigned char *mask, const double *x,
                             double *out);

/* Forward ([P4] "Insight 2" equation, bracketed sum; [P2] "encoder" core:
 * bilinear sampling, zero padding, align_corners=False):
 * out[b,q,m*D+d] = sum_{l,k} A[b,q,m,l,k] * bilinear(value_l[b,:,:,m,d], loc).
 * If query_ids != NULL only the n_ids flat query ids (b*Nq+q) are computed and
 * out is [n_ids, M*D]; otherwise out is [B,Nq,M*D]. */
void msda_oracle_forward(int B, int64_t S, int64_t Nq, int M, int D, int L, int K,
                         const int64_t *shapes, const int64_t *lsi,
                         const double *value /* [B,S,M,D] */,
                         const double *loc /* [B,Nq,M,L,K,2] */,
                         const double *attn /* [B,Nq,M,L,K] */,
                         const int64_t *query_ids, int64_t n_ids,
                         double *out);

/* Backward: the exact derivative of msda_oracle_forward with respect to value,
 * loc and attn, given grad_out [B,Nq,M*D]. grad_value is overwritten. */
void msda_oracle_backward(int B, int64_t S, int64_t Nq, int M, int D, int L, int K,
                          const int64_t *shapes, const int64_t *lsi,
                          const double *value, const double *loc, const double *attn,
                          const double *grad_out,
                          double *grad_value /* [B,S,M,D] */,
                          double *grad_loc /* [B,Nq,M,L,K,2] */,
                          double *grad_attn /* [B,Nq,M,L,K] */);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_ORACLE_H */
