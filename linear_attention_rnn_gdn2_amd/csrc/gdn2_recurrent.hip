// Token-by-token GDN-2 forward for decode and short spans (CDNA4, gfx950).
//
// The recurrence of the FlashInfer chunk_gated_delta_rule2 docs (recurrence
// display equation), applied one token at a time: per token,
//
//   S <- diag(exp(g)) S;   e = (beta k)^T S;   vnew = w v - e;
//   S <- S + k vnew^T;     o = scale q^T S.
//
// Every value column of S evolves on its own once the per-row gates of the
// token are known, so one workgroup takes one (sequence, value head, block of
// 32 value columns) and keeps that K x 32 block of the float32 state in
// registers for the whole span: the state is read once and written once,
// which is all the HBM traffic a decode step needs besides the token's
// vectors. Thread layout (256 threads): lane v of each half-wave owns column
// v of the block, and the 8 half-waves own 8 groups of K/8 rows. The two
// column sums per token (e and o) reduce over the row groups: the two halves
// of a wave by a permlane32 swap, the four waves through LDS.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gdn2_internal.h"

namespace gdn2 {
namespace {

constexpr int RB_COLS = 32;   // value columns per workgroup
constexpr int RB_THR = 256;   // 4 waves = 8 half-waves = 8 row groups
constexpr int RB_GROUPS = 8;
constexpr float RB_LOG2E = 1.44269504088896340736f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

// The other half-wave's value (lanes v and v + 32 hold the same column).
__device__ __forceinline__ float half_swap_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int K, int V>
__global__ __launch_bounds__(RB_THR) void recurrent_fwd_kernel(FwdParams p)
{
    constexpr int RPG = K / RB_GROUPS;  // rows per group
    constexpr int NVB = V / RB_COLS;
    __shared__ float red_e[4][RB_COLS], red_o[4][RB_COLS];

    int item = blockIdx.x;
    const int vb = item % NVB;
    item /= NVB;
    const int hv = item % p.HV, n = item / p.HV;
    const int hk = hv / (p.HV / p.H);
    const int64_t tb = p.cu ? (int64_t)p.cu[n] : 0;
    const int64_t te = p.cu ? (int64_t)p.cu[n + 1] : p.T;

    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int v = lane & 31, rg = 2 * wave + (lane >> 5);
    const int col = vb * RB_COLS + v, r0 = rg * RPG;
    const int64_t shead = ((int64_t)n * p.HV + hv) * K * V;

    float S[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) S[i] = p.h0 ? p.h0[shead + (int64_t)(r0 + i) * V + col] : 0.0f;

    for (int64_t tok = tb; tok < te; ++tok) {
        // this token's q, k, beta, g on the group's rows (16-byte loads; every
        // lane of a half-wave reads the same addresses)
        const int64_t qk = (tok * p.H + hk) * K + r0, gv = (tok * p.HV + hv) * K + r0;
        f32x8 qv[RPG / 8], kv[RPG / 8], bk[RPG / 8];
        f32x4 gr[RPG / 4];
#pragma unroll
        for (int j = 0; j < RPG / 8; ++j) {
            qv[j] = __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(p.q + qk + 8 * j), f32x8);
            kv[j] = __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(p.k + qk + 8 * j), f32x8);
            bk[j] = kv[j];
            if (p.beta) bk[j] *= __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(p.beta + gv + 8 * j), f32x8);
        }
#pragma unroll
        for (int j = 0; j < RPG / 4; ++j) gr[j] = p.g ? *reinterpret_cast<const f32x4 *>(p.g + gv + 4 * j) : f32x4{0, 0, 0, 0};
        float e = 0.0f;
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            S[i] *= __builtin_amdgcn_exp2f(gr[i / 4][i % 4] * RB_LOG2E);
            e = fmaf(bk[i / 8][i % 8], S[i], e);
        }
        e = half_swap_sum(e);
        if (lane < 32) red_e[wave][v] = e;
        __syncthreads();
        e = red_e[0][v] + red_e[1][v] + red_e[2][v] + red_e[3][v];
        const int64_t vrow = (tok * p.HV + hv) * V + col;
        const float wv = (p.w ? bf16_to_f32(p.w[vrow]) : 1.0f) * bf16_to_f32(p.v[vrow]);
        const float vnew = wv - e;
        float o = 0.0f;
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            S[i] = fmaf(kv[i / 8][i % 8], vnew, S[i]);
            o = fmaf(qv[i / 8][i % 8], S[i], o);
        }
        o = half_swap_sum(o);
        if (lane < 32) red_o[wave][v] = o;
        __syncthreads();
        if (t < RB_COLS) {
            o = red_o[0][v] + red_o[1][v] + red_o[2][v] + red_o[3][v];
            p.out[vrow] = f32_to_bf16(o * p.scale);
        }
    }
    if (p.ht)
#pragma unroll
        for (int i = 0; i < RPG; ++i) p.ht[shead + (int64_t)(r0 + i) * V + col] = S[i];
}

}  // namespace

hipError_t launch_recurrent_fwd(const FwdParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)((int64_t)p.N * p.HV * (p.V / RB_COLS))), block(RB_THR);
    if (p.K == 128 && p.V == 128)
        hipLaunchKernelGGL((recurrent_fwd_kernel<128, 128>), grid, block, 0, stream, p);
    else if (p.K == 64 && p.V == 64)
        hipLaunchKernelGGL((recurrent_fwd_kernel<64, 64>), grid, block, 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn2
