// Internal interface between the C-ABI layer (gdn2_api.cpp) and the gfx950
// kernels (gdn2_fwd.hip, gdn2_recurrent.hip, gdn2_bwd.hip). Not installed, not
// part of the ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gdn2_index.h"

namespace gdn2 {

// Validated, resolved arguments of one forward call. Pointers are device
// pointers; optional ones are nullptr when omitted.
struct FwdParams {
    // Element types: the io type (q, k, v, beta, w, out) is bf16 or fp16
    // (IO_BF16 / IO_F16); g is fp32, bf16 or fp16 (G_F32 / G_BF16 / G_F16).
    const uint16_t *q;     // [T, H, K] io
    const uint16_t *k;     // [T, H, K] io
    const uint16_t *v;     // [T, HV, V] io
    const void *g;         // [T, HV, K] g type, or nullptr (= 0)
    const uint16_t *beta;  // [T, HV, K] io, or nullptr (= 1)
    const uint16_t *w;     // [T, HV, V] io, or nullptr (= 1)
    const float *h0;       // [N, HV, K, V] (or [N, HV, V, K]) float32 or bf16, or nullptr (= 0)
    const void *cu;        // [N + 1] int32 or int64, or nullptr (one sequence of T tokens)
    uint16_t *out;         // [T, HV, V] io
    float *ht;             // [N, HV, K, V] (or [N, HV, V, K]) float32 or bf16, or nullptr (not written)
    int64_t T;
    int32_t N, H, HV, K, V;
    float scale;           // already resolved (never 0)
    int32_t io;            // IO_BF16 or IO_F16
    int32_t gtype;         // G_F32, G_BF16 or G_F16
    int32_t cu64;          // cu_seqlens is int64
    int32_t h0_bf16, ht_bf16;  // initial / final state stored as bf16 (element offsets count bf16s)
    // element strides of the token and head dimensions; the K or V
    // elements of one (token, head) row are contiguous
    int64_t sq, sk, sv, sw, sg, sb, so;          // per token
    int64_t hsq, hsk, hsv, hsw, hsg, hsb, hso;   // per head
    int32_t state_vmajor;  // initial/final state stored [N, HV, V, K]
    int32_t qk_l2norm;     // normalise q and k rows in the kernel
    // Sequence split (0: one workgroup walks each whole sequence). With
    // seg_chunks > 0 every sequence is cut into segments of seg_chunks
    // chunks (nseg per sequence at most) and the launch is one of:
    int32_t seg_chunks;
    int32_t nseg;
    int32_t pass;          // PASS_OUTPUT or PASS_TRANSITION
    // transition pass: 0 both walks of every segment (grid item parity), 1
    // only the end-state walks, 2 only the transition-map walks (K != V: the
    // map is K x K, walked by the square kernel)
    int32_t tonly;
    float *wb;             // [N, HV, nseg, K, V] segment end state from a zero start (segment 0: from h0)
    float *wm;             // [N, HV, nseg, K, K] segment transition (state map S_in -> S_out minus wb)
    float *ws;             // [N, HV, nseg, K, V] entering state of segment j >= 1
    // Optional: the K-major state entering every chunk, rounded to bf16
    // (the backward uses it as bf16 MFMA operands), written to
    // ckpt[slot][hv] with slot = cu[n] / 64 + n + c for chunk c of sequence
    // n (whole sequences, or the output pass of a split run; out may then
    // be nullptr: no output)
    uint16_t *ckpt;        // bf16 [slot][HV][K][V]
    // Optional, with ckpt (bf16 io, float32 g, no L2 normalisation): every
    // chunk's record (PrepRecord) at rec + (slot * HV + hv) * bwd_prep_bytes(K)
    char *rec;
    // Optional sequence filter (the backward's two-stream schedule): with
    // grp set, the workgroups of a sequence n with grp[n] != gsel return at
    // once, so that two launches with gsel 0 and 1 share the work
    const int32_t *grp = nullptr;  // [N]
    int32_t gsel = 0;
};

// Arguments of the backward kernels (all tensors dense, row-major).
struct BwdParams {
    // q, k, v, w, beta, d_out and their gradients share one 16-bit io type
    // (io: IO_BF16 or IO_F16); g and dg share gtype (G_F32, G_BF16, G_F16)
    const uint16_t *q, *k;       // [T, H, K]
    const uint16_t *v, *w;       // [T, HV, V]
    const void *g;               // [T, HV, K]
    const uint16_t *beta;        // [T, HV, K]
    const uint16_t *dout;        // [T, HV, V]
    int32_t io, gtype;
    const void *cu;              // [N + 1] int32 or int64, or nullptr
    int32_t cu64;
    const float *dht;            // [N, HV, K, V] gradient of the final state, or nullptr (zero)
    float *dh0;                  // [N, HV, K, V] gradient of the initial state, or nullptr
    uint16_t *dq, *dk;           // [T, H, K] io
    uint16_t *dv, *dw;           // [T, HV, V] io
    uint16_t *dbeta;             // [T, HV, K] io
    void *dg;                    // [T, HV, K] gtype
    // workspace
    float *dq_ws, *dk_ws;        // [T, HV, K] per value head (grouped heads only)
    const uint16_t *s_ckpt;      // [nslots, HV, K, V] bf16: state entering each chunk
    uint16_t *ds_ckpt;           // [nslots, HV, K, V] bf16: gradient of the state leaving each chunk
    char *prep;                  // [nslots, HV] x bwd_prep_bytes(K): each chunk's record (PrepRecord)
    int64_t T;
    int32_t N, H, HV, K, V;
    int32_t nslots;
    float scale;
    // Split state-gradient pass (seg_chunks > 0), as the forward's: segments
    // of seg_chunks chunks numbered in processing order (segment 0 holds the
    // sequence's last chunks); pass PASS_TRANSITION gives each segment's end
    // gradient from dht or zero (wb) and its K x K map (wm), the forward's
    // combine chains them (ws), PASS_OUTPUT walks every segment from its
    // entering gradient. wb, wm, ws: [N, HV, nseg, K, V] float32.
    int32_t seg_chunks, nseg, pass;
    float *wb, *wm, *ws;
    // Optional sequence filter, as FwdParams::grp
    const int32_t *grp = nullptr;  // [N]
    int32_t gsel = 0;
};

// Byte offsets of one chunk's record in BwdParams::prep (K = V = D): the
// chunk's WY quantities as the forward with checkpoints computed them, read
// by the state-gradient and gradient passes. QH, RR, wy_w, KB as bf16 [64][D],
// P, T as bf16 [64][64], and gamma = 2^G_last as float32 [D] with the sign
// bit set (-gamma, -0.0 when it underflows) for a flagged channel: strong
// decay, where k 2^-G would overflow, so that the channel's RR column holds
// the exact K-hat = k 2^(G_last - G) instead of RR (K-hat = RR gamma
// elsewhere).
struct PrepRecord {
    int D;
    __host__ __device__ constexpr int qh() const { return 0; }
    __host__ __device__ constexpr int rr() const { return 128 * D; }
    __host__ __device__ constexpr int wy() const { return 256 * D; }
    __host__ __device__ constexpr int kb() const { return 384 * D; }
    __host__ __device__ constexpr int p() const { return 512 * D; }
    __host__ __device__ constexpr int t() const { return 512 * D + 8192; }
    __host__ __device__ constexpr int gam() const { return 512 * D + 16384; }
    __host__ __device__ constexpr int bytes() const { return 516 * D + 16384; }
};
__host__ __device__ inline int64_t bwd_prep_bytes(int K) { return PrepRecord{K}.bytes(); }

enum { PASS_OUTPUT = 0, PASS_TRANSITION = 1 };
enum { IO_BF16 = 0, IO_F16 = 1 };
enum { G_F32 = 0, G_BF16 = 1, G_F16 = 2 };

// State buffers hold float32 or bf16 elements: the element at offset e, a
// pointer to it, and a store rounding to nearest even.
__host__ __device__ inline const float *state_at(const float *s, bool b16, int64_t e)
{
    return b16 ? reinterpret_cast<const float *>(reinterpret_cast<const uint16_t *>(s) + e) : s + e;
}
__host__ __device__ inline float *state_at(float *s, bool b16, int64_t e)
{
    return b16 ? reinterpret_cast<float *>(reinterpret_cast<uint16_t *>(s) + e) : s + e;
}
__device__ inline float state_ld(const float *s, bool b16, int64_t e)
{
    return b16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(s)[e] << 16) : s[e];
}
__device__ inline void state_st(float *s, bool b16, int64_t e, float x)
{
    if (b16) reinterpret_cast<__bf16 *>(s)[e] = (__bf16)x;
    else s[e] = x;
}

// Token range of sequence n of a call (clamped into [0, T]).
__host__ __device__ inline SeqRange seq_of(const FwdParams &p, int64_t n) { return seq_range(p.cu, p.cu64, p.T, n); }

// Enqueue the fused chunked forward on `stream` (one pass, as p describes).
hipError_t launch_chunk_fwd(const FwdParams &p, hipStream_t stream);
// The forward kernel at K != V ((128, 64) or (64, 128)), compiled in a
// translation unit of its own: whole sequences, a split run's output pass,
// or its end-state walks (tonly == 1) on `grid` workgroups.
hipError_t launch_chunk_fwd_mixed(const FwdParams &p, unsigned grid, hipStream_t stream);
// The backward's recompute (p.rec) at fp16 io or 16-bit g, in the same
// translation unit.
hipError_t launch_chunk_fwd_rec16(const FwdParams &p, unsigned grid, hipStream_t stream);

// Enqueue the token-by-token forward (decode and short spans): one
// workgroup per (sequence, value head, 32 value columns).
hipError_t launch_recurrent_fwd(const FwdParams &p, hipStream_t stream);

// The backward (after the forward with checkpoints and records): the
// sequential pass of the state gradient over chunks in reverse, the
// chunk-parallel gradients, and the sum of dq, dk over the value heads of
// each q/k head.
hipError_t launch_bwd_chunk(const BwdParams &p, hipStream_t stream);
hipError_t launch_bwd_state(const BwdParams &p, hipStream_t stream);
hipError_t launch_bwd_reduce(const BwdParams &p, hipStream_t stream);
// The backward's two-stream schedule: grp[n] = 0 for the nlong sequences
// with the most chunks (ties to the lower index), 1 for the others. One
// workgroup; meant for N up to a few hundred.
hipError_t launch_bwd_group(const BwdParams &p, int32_t nlong, int32_t *grp, hipStream_t stream);

// Enqueue the segment combine of a split forward: ws[j + 1] = wm[j] ws[j] +
// wb[j] in segment order, with ws[1] = wb[0].
hipError_t launch_seg_combine(const FwdParams &p, hipStream_t stream);

}  // namespace gdn2
