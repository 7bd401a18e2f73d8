// Internal interface between the C-ABI layer (gdn2_api.cpp) and the gfx950
// kernels (gdn2_fwd.hip). Not installed, not part of the ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gdn2 {

// Validated, resolved arguments of one forward call. Pointers are device
// pointers; optional ones are nullptr when omitted.
struct FwdParams {
    const uint16_t *q;     // [T, H, K] bf16
    const uint16_t *k;     // [T, H, K] bf16
    const uint16_t *v;     // [T, HV, V] bf16
    const float *g;        // [T, HV, K] or nullptr (= 0)
    const uint16_t *beta;  // [T, HV, K] bf16 or nullptr (= 1)
    const uint16_t *w;     // [T, HV, V] bf16 or nullptr (= 1)
    const float *h0;       // [N, HV, K, V] or nullptr (= 0)
    const int32_t *cu;     // [N + 1] or nullptr (one sequence of T tokens)
    uint16_t *out;         // [T, HV, V] bf16
    float *ht;             // [N, HV, K, V] or nullptr (not written)
    int64_t T;
    int32_t N, H, HV, K, V;
    float scale;           // already resolved (never 0)
};

// Enqueue the fused chunked forward on `stream`. Returns the launch status.
hipError_t launch_chunk_fwd(const FwdParams &p, hipStream_t stream);

}  // namespace gdn2
