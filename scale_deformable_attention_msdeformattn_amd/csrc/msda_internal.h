// Internal declarations shared by the HIP translation units of libmsda.
// Not part of the public ABI (include/msda.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda.h"

namespace msda {

// Per-level sizes, passed to kernels by value (kernel arguments are
// wave-uniform and land in scalar registers).
struct Levels {
    int32_t H[MSDA_MAX_LEVELS];
    int32_t W[MSDA_MAX_LEVELS];
    int32_t start[MSDA_MAX_LEVELS];
};

// A validated call geometry. Every tensor of the call has fewer than 2^31
// elements and one batch of value fewer than 2^31 bytes, so 32-bit offsets
// suffice inside a batch.
struct Geometry {
    int32_t B, M, D, L, K;
    int32_t S, Nq;
    Levels lv;
    int64_t samples() const { return (int64_t)B * Nq * M * L * K; }
    int64_t queries() const { return (int64_t)B * Nq; }
    int32_t channels() const { return M * D; }
};

// Launchers (each returns a hipError_t from the launch).
hipError_t launch_reference_points(const Geometry &g, const float *valid_ratios,
                                   const float *query_ref, float *ref_out, hipStream_t st);
hipError_t launch_sampling_locations(const Geometry &g, const float *ref, const float *off,
                                     float *loc, hipStream_t st);
hipError_t launch_softmax(const Geometry &g, const float *logits, float *w, hipStream_t st);
hipError_t launch_forward(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                          const float *attn, float *out, hipStream_t st);
hipError_t launch_zero_fill(float *p, int64_t n, hipStream_t st);
hipError_t launch_backward(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                           const float *attn, const float *grad_out, float *grad_value,
                           float *grad_loc, float *grad_attn, hipStream_t st);

}  // namespace msda
