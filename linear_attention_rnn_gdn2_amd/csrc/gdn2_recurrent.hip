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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// 8 consecutive 16-bit values of type io (IO_BF16 / IO_F16) as float32
template <int IO>
__device__ __forceinline__ f32x8 ld8_f32(const uint16_t *p)
{
    if constexpr (IO == IO_F16) return __builtin_convertvector(*reinterpret_cast<const f16x8 *>(p), f32x8);
    else return __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(p), f32x8);
}
template <int IO>
__device__ __forceinline__ float io_to_f32(uint16_t b)
{
    if constexpr (IO == IO_F16) return (float)__builtin_bit_cast(_Float16, b);
    else return __uint_as_float((uint32_t)b << 16);
}
template <int IO>
__device__ __forceinline__ uint16_t f32_to_io(float x)  // round to nearest even
{
    if constexpr (IO == IO_F16) return __builtin_bit_cast(uint16_t, (_Float16)x);
    else return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// The other half-wave's value (lanes v and v + 32 hold the same column).
__device__ __forceinline__ float half_swap_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// IO: element type of q, k, v, beta, w, out; G16: g is 16-bit (bf16 or fp16
// by p.gtype) instead of float32; L2N: q and k rows are L2-normalised here
// (x / max(|x|, 1e-12), with the sums of squares reduced along with e).
template <int K, int V, int IO, bool G16, bool L2N>
__global__ __launch_bounds__(RB_THR) void recurrent_fwd_kernel(FwdParams p)
{
    constexpr int RPG = K / RB_GROUPS;  // rows per group
    constexpr int NVB = V / RB_COLS;
    __shared__ float red_e[4][RB_COLS], red_o[4][RB_COLS];
    __shared__ f32x2 red_n[4];

    int item = blockIdx.x;
    const int vb = item % NVB;
    item /= NVB;
    const int hv = item % p.HV, n = item / p.HV;
    const int hk = hv / (p.HV / p.H);
    const SeqRange rng = seq_of(p, n);
    const int64_t tb = rng.b, te = rng.e;

    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int v = lane & 31, rg = 2 * wave + (lane >> 5);
    const int col = vb * RB_COLS + v, r0 = rg * RPG;
    const int64_t shead = ((int64_t)n * p.HV + hv) * K * V;
    const bool g_f16 = p.gtype == G_F16;

    // state element (row c, column v) at c * sr + v * sc
    const int sr = p.state_vmajor ? 1 : V, sc = p.state_vmajor ? K : 1;
    float S[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) S[i] = p.h0 ? state_ld(p.h0, p.h0_bf16, shead + (int64_t)(r0 + i) * sr + col * sc) : 0.0f;

    for (int64_t tok = tb; tok < te; ++tok) {
        // this token's q, k, beta, g on the group's rows (16-byte loads; every
        // lane of a half-wave reads the same addresses)
        const int64_t qo = tok * p.sq + hk * p.hsq + r0, ko = tok * p.sk + hk * p.hsk + r0;
        const int64_t go = tok * p.sg + hv * p.hsg + r0, bo = tok * p.sb + hv * p.hsb + r0;
        f32x8 qv[RPG / 8], kv[RPG / 8], bk[RPG / 8], gr[RPG / 8];
#pragma unroll
        for (int j = 0; j < RPG / 8; ++j) {
            qv[j] = ld8_f32<IO>(p.q + qo + 8 * j);
            kv[j] = ld8_f32<IO>(p.k + ko + 8 * j);
            bk[j] = kv[j];
            if (p.beta) bk[j] *= ld8_f32<IO>(p.beta + bo + 8 * j);
            if (!p.g) {
                gr[j] = f32x8{0, 0, 0, 0, 0, 0, 0, 0};
            } else if constexpr (G16) {
                const uint16_t *gh = static_cast<const uint16_t *>(p.g) + go + 8 * j;
                gr[j] = g_f16 ? ld8_f32<IO_F16>(gh) : ld8_f32<IO_BF16>(gh);
            } else {
                const float *gf = static_cast<const float *>(p.g) + go + 8 * j;
                gr[j] = __builtin_shufflevector(*reinterpret_cast<const f32x4 *>(gf),
                                                *reinterpret_cast<const f32x4 *>(gf + 4), 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
        float e = 0.0f, nq = 0.0f, nk = 0.0f;
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            S[i] *= __builtin_amdgcn_exp2f(gr[i / 8][i % 8] * RB_LOG2E);
            e = fmaf(bk[i / 8][i % 8], S[i], e);
            if constexpr (L2N) {
                nq = fmaf(qv[i / 8][i % 8], qv[i / 8][i % 8], nq);
                nk = fmaf(kv[i / 8][i % 8], kv[i / 8][i % 8], nk);
            }
        }
        e = half_swap_sum(e);
        if (lane < 32) red_e[wave][v] = e;
        if constexpr (L2N) {
            nq = half_swap_sum(nq);
            nk = half_swap_sum(nk);
            if (lane == 0) red_n[wave] = f32x2{nq, nk};
        }
        __syncthreads();
        e = red_e[0][v] + red_e[1][v] + red_e[2][v] + red_e[3][v];
        float rq = 1.0f, rk = 1.0f;  // reciprocal norms
        if constexpr (L2N) {
            const f32x2 ns = red_n[0] + red_n[1] + red_n[2] + red_n[3];
            rq = 1.0f / fmaxf(sqrtf(ns[0]), 1e-12f);
            rk = 1.0f / fmaxf(sqrtf(ns[1]), 1e-12f);
            e *= rk;
        }
        const float wv = (p.w ? io_to_f32<IO>(p.w[tok * p.sw + hv * p.hsw + col]) : 1.0f) *
                         io_to_f32<IO>(p.v[tok * p.sv + hv * p.hsv + col]);
        const float vnew = wv - e;
        const float kvn = L2N ? vnew * rk : vnew;  // (k / |k|) vnew^T = k (vnew / |k|)^T
        float o = 0.0f;
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            S[i] = fmaf(kv[i / 8][i % 8], kvn, S[i]);
            o = fmaf(qv[i / 8][i % 8], S[i], o);
        }
        o = half_swap_sum(o);
        if (lane < 32) red_o[wave][v] = o;
        __syncthreads();
        if (t < RB_COLS) {
            o = red_o[0][v] + red_o[1][v] + red_o[2][v] + red_o[3][v];
            p.out[tok * p.so + hv * p.hso + col] = f32_to_io<IO>(o * rq * p.scale);
        }
    }
    if (p.ht)
#pragma unroll
        for (int i = 0; i < RPG; ++i) state_st(p.ht, p.ht_bf16, shead + (int64_t)(r0 + i) * sr + col * sc, S[i]);
}

template <int K, int V, int IO, bool G16>
void launch_rec_l2(const FwdParams &p, dim3 grid, hipStream_t stream)
{
    if (p.qk_l2norm) hipLaunchKernelGGL((recurrent_fwd_kernel<K, V, IO, G16, true>), grid, dim3(RB_THR), 0, stream, p);
    else hipLaunchKernelGGL((recurrent_fwd_kernel<K, V, IO, G16, false>), grid, dim3(RB_THR), 0, stream, p);
}
template <int K, int V>
void launch_rec_typed(const FwdParams &p, dim3 grid, hipStream_t stream)
{
    const bool g16 = p.gtype != G_F32;
    if (p.io == IO_F16) {
        if (g16) launch_rec_l2<K, V, IO_F16, true>(p, grid, stream);
        else launch_rec_l2<K, V, IO_F16, false>(p, grid, stream);
    } else {
        if (g16) launch_rec_l2<K, V, IO_BF16, true>(p, grid, stream);
        else launch_rec_l2<K, V, IO_BF16, false>(p, grid, stream);
    }
}

}  // namespace

hipError_t launch_recurrent_fwd(const FwdParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)((int64_t)p.N * p.HV * (p.V / RB_COLS)));
    if (p.K == 128 && p.V == 128)
        launch_rec_typed<128, 128>(p, grid, stream);
    else if (p.K == 64 && p.V == 64)
        launch_rec_typed<64, 64>(p, grid, stream);
    else if (p.K == 128 && p.V == 64)
        launch_rec_typed<128, 64>(p, grid, stream);
    else if (p.K == 64 && p.V == 128)
        launch_rec_typed<64, 128>(p, grid, stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn2
