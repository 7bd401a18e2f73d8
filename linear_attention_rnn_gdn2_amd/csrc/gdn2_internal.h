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
    // Sequence split (0: one workgroup walks each whole sequence). With
    // seg_chunks > 0 every sequence is cut into segments of seg_chunks
    // chunks (nseg per sequence at most) and the launch is one of:
    int32_t seg_chunks;
    int32_t nseg;
    int32_t pass;          // PASS_OUTPUT or PASS_TRANSITION
    float *wb;             // [N, HV, nseg, K, V] segment end state from a zero start (segment 0: from h0)
    float *wm;             // [N, HV, nseg, K, K] segment transition (state map S_in -> S_out minus wb)
    float *ws;             // [N, HV, nseg, K, V] entering state of segment j >= 1
};

enum { PASS_OUTPUT = 0, PASS_TRANSITION = 1 };

// Enqueue the fused chunked forward on `stream` (one pass, as p describes).
hipError_t launch_chunk_fwd(const FwdParams &p, hipStream_t stream);

// Enqueue the token-by-token forward (decode and short spans): one
// workgroup per (sequence, value head, 32 value columns).
hipError_t launch_recurrent_fwd(const FwdParams &p, hipStream_t stream);

// Enqueue the segment combine of a split forward: ws[j + 1] = wm[j] ws[j] +
// wb[j] in segment order, with ws[1] = wb[0].
hipError_t launch_seg_combine(const FwdParams &p, hipStream_t stream);

}  // namespace gdn2
