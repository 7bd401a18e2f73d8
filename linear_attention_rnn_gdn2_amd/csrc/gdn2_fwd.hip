// Fused GDN-2 chunked prefill forward for CDNA4 (gfx950).
//
// One workgroup of 256 threads (4 wave64s) owns one (sequence, value head)
// chain and walks its 64-token chunks in order. The K x V float32 state lives
// in registers, in the result layout of v_mfma_f32_16x16x32_bf16, split by
// value columns across the four waves. Per chunk (notation: rows r, s are
// positions in the chunk, G = inclusive in-chunk cumulative sum of the
// log-decay g per key channel, S = state entering the chunk):
//
//   E   load q, k, g, beta, v, w (coalesced 16-byte rows), cumulative sum of g
//       (in-thread + wave shuffles + one LDS exchange), every decay factor,
//       and the bf16 MFMA operands, written to LDS
//   AP  A_rs = sum_c beta_r k_r exp(G_r - G_s) k_s   (s < r)
//       P_rs = sum_c q_r exp(G_r - G_s) k_s          (s <= r)
//       on MFMA, one 16-row tile at a time, each tile factored about its own
//       midpoint row m: exp(G_r - G_m) * exp(G_m - G_s). Every factor stays
//       within exp(+-64) while no 8-token half-tile spans more than 64 in log
//       decay; otherwise the chunk takes an exact fallback that evaluates
//       exp(G_r - G_s) per pair (exponent <= 0, nothing can overflow).
//   T   T = (I + A)^{-1}: 16x16 diagonal blocks by forward substitution, then
//       the off-diagonal blocks level by level, all in float32.
//   WY  wy_w = T (beta k exp(G)),  wy_u = T (w v)          (MFMA)
//   S   U = wy_u - wy_w S;  O = scale (q exp(G)) S + scale P U;
//       S <- diag(exp(G_last)) S + (k exp(G_last - G))^T U    (MFMA)
//
// This is the chunked WY evaluation of the recurrence of the FlashInfer
// chunk_gated_delta_rule2 docs (recurrence display equation); the split into
// decay cumsum, decay-scaled K K^T with the erase gate, unit-lower-triangular
// inverse, w/u recompute and a sequential float32 state pass with intra plus
// inter output follows the FlashRT card ("Usage", WY chain) and the burn-gdn2
// README ("Fused CUDA kernels", "Numerical stability": 16-token tiles with
// tile-local log-space decay). Padded rows of a partial last chunk carry
// q = k = beta = v = w = 0 and g = 0, which makes them exact identity steps.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gdn2_internal.h"

namespace gdn2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int CH = 64;       // chunk length
constexpr int NTHR = 256;    // threads per workgroup (4 waves)
constexpr float HALF_SPAN_MAX = 64.0f;  // largest |G_r - G_mid| of the fast path

// ---------------------------------------------------------------- helpers --
__device__ __forceinline__ f32x8 bf16x8_to_f32(bf16x8 x) { return __builtin_convertvector(x, f32x8); }
__device__ __forceinline__ bf16x8 f32x8_to_bf16(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 f32x4_to_bf16(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

__device__ __forceinline__ bf16x8 ldg_bf16x8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x4 ldg_f32x4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

template <typename T>
__device__ __forceinline__ T lds_ld(const char *base, int off) { return *reinterpret_cast<const T *>(base + off); }
template <typename T>
__device__ __forceinline__ void lds_st(char *base, int off, T v) { *reinterpret_cast<T *>(base + off) = v; }

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// (row tile, column tile) of the 10 lower-triangular 16x16 tiles of a 64x64
// matrix, in row order.
__constant__ int8_t kTriI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kTriJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

// ------------------------------------------------------------ LDS layout --
// Byte offsets into one static LDS array. Row pitches are padded by 16 bytes
// (bf16) or 16 bytes (fp32) to spread rows over banks.
template <int K, int V>
struct Lds {
    static constexpr int KP = K + 8;   // bf16 elements per [row][K] row
    static constexpr int VP = V + 8;   // bf16 elements per [row][V] row
    static constexpr int CP = CH + 8;  // bf16 elements per [channel][token] row
    static constexpr int AP = CH + 4;  // fp32 elements per A/T row
    static constexpr int GP = K + 4;   // fp32 elements per G row (fallback)
    static constexpr int BP = 16 + 4;  // fp32 elements per scratch-block row
    // Region X, phase E/AP view (fast path): MFMA operands of A and P
    static constexpr int LB = 0;                        // beta k exp(G - G_mid)   [64][KP]
    static constexpr int LQ = LB + CH * KP * 2;         // q exp(G - G_mid)        [64][KP]
    static constexpr int RR = LQ + CH * KP * 2;         // k exp(G_mid(i) - G), 160 rows
    static constexpr int X_END1 = RR + 160 * KP * 2;
    static constexpr int GF = 0;                        // fallback: absolute G fp32 [64][GP]
    // Region X, phase T/WY view
    static constexpr int KBT = 0;                       // (beta k exp(G))^T       [K][CP]
    static constexpr int WVT = KBT + K * CP * 2;        // (w v)^T                 [V][CP]
    static constexpr int WYW = WVT + V * CP * 2;        // -wy_w                   [64][KP]
    static constexpr int TB = WYW + CH * KP * 2;        // T in bf16               [64][CP]
    static constexpr int BS = TB + CH * CP * 2;         // T_ii A_ik scratch       [6][16][BP]
    static constexpr int X_END2 = BS + 6 * 16 * BP * 4;
    // Region X, output staging (phase S, after WY)
    static constexpr int OST = 0;                       // out tile                [64][VP]
    static constexpr int X_END = X_END1 > X_END2 ? X_END1 : X_END2;
    // Persistent buffers
    static constexpr int QH = X_END;                    // q exp(G)                [64][KP]
    static constexpr int KHT = QH + CH * KP * 2;        // (k exp(G_last - G))^T   [K][CP]
    static constexpr int AB = KHT + K * CP * 2;         // A, then T, fp32         [64][AP]
    static constexpr int PB = AB + CH * AP * 4;         // P bf16                  [64][CP]
    static constexpr int GAM = PB + CH * CP * 2;        // exp(G_last) fp32        [K]
    static constexpr int TT = GAM + K * 4;              // tile totals of G        [4][K]
    static constexpr int TM = TT + 4 * K * 4;           // tile midpoints of G     [4][K]
    static constexpr int FL = TM + 4 * K * 4;           // per-wave fast-path flags [4]
    static constexpr int TOTAL = FL + 16;
    static_assert(OST + CH * VP * 2 <= WYW, "output staging must not overlap -wy_w");
    static_assert(GF + CH * GP * 4 <= X_END, "fallback G must fit region X");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Row offset of R_i (the column operand of row tile i) inside RR.
__device__ __forceinline__ int r_off(int i) { return (i * (i + 1) / 2) * 16; }  // 0,16,48,96

// ------------------------------------------------------------------ kernel --
template <int K, int V>
__global__ __launch_bounds__(NTHR, 1) void chunk_fwd_kernel(FwdParams p)
{
    using L = Lds<K, V>;
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];

    // thread maps
    constexpr int CGK = K / 8;                 // 8-channel groups along K
    constexpr int RPT = CH * CGK / NTHR;       // rows per thread in phase E
    constexpr int RGW = 64 / CGK;              // row groups per wave
    constexpr int CGV = V / 8;
    constexpr int RPTV = CH * CGV / NTHR;
    constexpr int VW = V / 4;                  // value columns per wave (phase S)
    constexpr int NCT = VW / 16;               // 16-column tiles per wave
    constexpr int NRT = K / 16;                // 16-row tiles of the state
    constexpr int NKS = K / 32;                // 32-deep k slabs over K
    constexpr int NCTK = K / 64;               // -wy_w column tiles per wave
    static_assert(RPT * RGW == 16, "a wave covers one 16-row tile in phase E");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;

    const int chain = blockIdx.x;
    const int n = chain / p.HV;
    const int hv = chain - n * p.HV;
    const int hk = hv / (p.HV / p.H);
    const int64_t tb = p.cu ? (int64_t)p.cu[n] : 0;
    const int64_t te = p.cu ? (int64_t)p.cu[n + 1] : p.T;

    // phase-E coordinates
    const int cg = tid % CGK, rg = tid / CGK, row0 = rg * RPT, c0k = cg * 8;
    const int rgl = rg % RGW;  // row group inside this wave's tile
    const int cgv = tid % CGV, row0v = (tid / CGV) * RPTV, c0v = cgv * 8;
    const int vbase = wv * VW;  // first value column owned by this wave in phase S

    // ---- state: rows 16*it + 4*q4 + e, column vbase + 16*jt + l16
    f32x4 S[NRT][NCT];
    for (int it = 0; it < NRT; ++it)
        for (int jt = 0; jt < NCT; ++jt)
            for (int e = 0; e < 4; ++e) {
                float x = 0.0f;
                if (p.h0)
                    x = p.h0[(((int64_t)n * p.HV + hv) * K + 16 * it + 4 * q4 + e) * V + vbase + 16 * jt + l16];
                S[it][jt][e] = x;
            }

    // P's blocks above the diagonal stay zero for the whole chain
    for (int i = tid; i < CH * L::CP / 2; i += NTHR) lds_st<uint32_t>(smem, L::PB + 4 * i, 0u);

    for (int64_t c0 = tb; c0 < te; c0 += CH) {
        const int len = (int)((te - c0) < CH ? (te - c0) : CH);

        // =========================== phase E ===========================
        float G[RPT][8], qf[RPT][8], kf[RPT][8], bk[RPT][8];
        for (int i = 0; i < RPT; ++i) {
            const int r = row0 + i;
            const bool ok = r < len;
            const int64_t t = c0 + r;
            f32x8 gq = {}, gk = {}, gb = {}, gg = {};
            if (ok) {
                gq = bf16x8_to_f32(ldg_bf16x8(p.q + (t * p.H + hk) * K + c0k));
                gk = bf16x8_to_f32(ldg_bf16x8(p.k + (t * p.H + hk) * K + c0k));
                if (p.beta) gb = bf16x8_to_f32(ldg_bf16x8(p.beta + (t * p.HV + hv) * K + c0k));
                else gb = f32x8{1, 1, 1, 1, 1, 1, 1, 1};
                if (p.g) {
                    const float *gp = p.g + (t * p.HV + hv) * K + c0k;
                    f32x4 a = ldg_f32x4(gp), b = ldg_f32x4(gp + 4);
                    gg = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
                }
            }
            for (int j = 0; j < 8; ++j) {
                qf[i][j] = gq[j];
                kf[i][j] = gk[j];
                bk[i][j] = gb[j] * gk[j];
                G[i][j] = (i ? G[i - 1][j] : 0.0f) + gg[j];
            }
        }
        float wvv[RPTV][8];
        for (int i = 0; i < RPTV; ++i) {
            const int r = row0v + i;
            f32x8 a = {}, b = {1, 1, 1, 1, 1, 1, 1, 1};
            if (r < len) {
                const int64_t t = c0 + r;
                a = bf16x8_to_f32(ldg_bf16x8(p.v + (t * p.HV + hv) * V + c0v));
                if (p.w) b = bf16x8_to_f32(ldg_bf16x8(p.w + (t * p.HV + hv) * V + c0v));
            }
            for (int j = 0; j < 8; ++j) wvv[i][j] = a[j] * b[j];
        }
        // tile-local inclusive scan across the wave's row groups
        for (int j = 0; j < 8; ++j) {
            const float tot = G[RPT - 1][j];
            float inc = tot;
            for (int d = 1; d < RGW; d <<= 1) {
                const float o = __shfl_up(inc, d * CGK, 64);
                if (rgl >= d) inc += o;
            }
            const float excl = inc - tot;
            for (int i = 0; i < RPT; ++i) G[i][j] += excl;
        }
        // tile midpoint (local row 7) and total (local row 15), per channel
        float gmid[8];
        bool fast_ok = true;
        for (int j = 0; j < 8; ++j) {
            gmid[j] = __shfl(G[7 % RPT][j], (7 / RPT) * CGK + cg, 64);
            for (int i = 0; i < RPT; ++i) fast_ok &= fabsf(G[i][j] - gmid[j]) <= HALF_SPAN_MAX;
        }
        const int wave_ok = __all(fast_ok);
        if (rgl == RGW - 1) {
            lds_st<f32x4>(smem, L::TT + 4 * (wv * K + c0k), f32x4{G[RPT - 1][0], G[RPT - 1][1], G[RPT - 1][2], G[RPT - 1][3]});
            lds_st<f32x4>(smem, L::TT + 4 * (wv * K + c0k + 4), f32x4{G[RPT - 1][4], G[RPT - 1][5], G[RPT - 1][6], G[RPT - 1][7]});
        }
        if (rgl == 7 / RPT) {
            lds_st<f32x4>(smem, L::TM + 4 * (wv * K + c0k), f32x4{gmid[0], gmid[1], gmid[2], gmid[3]});
            lds_st<f32x4>(smem, L::TM + 4 * (wv * K + c0k + 4), f32x4{gmid[4], gmid[5], gmid[6], gmid[7]});
        }
        if (lane == 0) lds_st<int>(smem, L::FL + 4 * wv, wave_ok);
        __syncthreads();  // ---------------------------------------- B1

        const bool fast = lds_ld<int>(smem, L::FL) & lds_ld<int>(smem, L::FL + 4) &
                          lds_ld<int>(smem, L::FL + 8) & lds_ld<int>(smem, L::FL + 12);
        // absolute (chunk-relative) references per channel
        float base[8], gm_abs[4][8], glast[8];
        for (int j = 0; j < 8; ++j) {
            float acc = 0.0f;
            for (int i = 0; i < 4; ++i) {
                if (i == wv) base[j] = acc;
                gm_abs[i][j] = acc + lds_ld<float>(smem, L::TM + 4 * (i * K + c0k + j));
                acc += lds_ld<float>(smem, L::TT + 4 * (i * K + c0k + j));
            }
            glast[j] = acc;
        }
        if (rg == 0)
            for (int j = 0; j < 8; ++j) lds_st<float>(smem, L::GAM + 4 * (c0k + j), __expf(glast[j]));

        // operands (bf16 packed 8 channels per row)
        bf16x8 kbg_rows[RPT];       // beta k exp(G), written after phase AP
        bf16x8 kh_rows[RPT];        // k exp(G_last - G), transposed into KHT
        if (fast) {
            float eGm[8], eKm[8], D[4][8];
            for (int j = 0; j < 8; ++j) {
                eGm[j] = __expf(gm_abs[wv][j]);
                eKm[j] = __expf(glast[j] - gm_abs[wv][j]);
                for (int i2 = 0; i2 < 4; ++i2) D[i2][j] = i2 > wv ? __expf(gm_abs[i2][j] - gm_abs[wv][j]) : 1.0f;
            }
            for (int i = 0; i < RPT; ++i) {
                const int r = row0 + i;
                f32x8 lb, lq, qh, kb, kh;
                f32x8 rf_k;
                for (int j = 0; j < 8; ++j) {
                    const float x = G[i][j] - gmid[j];
                    const float f = __expf(x), rf = __expf(-x);
                    lb[j] = bk[i][j] * f;
                    lq[j] = qf[i][j] * f;
                    qh[j] = qf[i][j] * (eGm[j] * f);
                    kb[j] = bk[i][j] * (eGm[j] * f);
                    kh[j] = kf[i][j] * (eKm[j] * rf);
                    rf_k[j] = kf[i][j] * rf;
                }
                lds_st<bf16x8>(smem, L::LB + 2 * (r * L::KP + c0k), f32x8_to_bf16(lb));
                lds_st<bf16x8>(smem, L::LQ + 2 * (r * L::KP + c0k), f32x8_to_bf16(lq));
                lds_st<bf16x8>(smem, L::QH + 2 * (r * L::KP + c0k), f32x8_to_bf16(qh));
                for (int i2 = wv; i2 < 4; ++i2) {
                    f32x8 rr;
                    for (int j = 0; j < 8; ++j) rr[j] = rf_k[j] * D[i2][j];
                    lds_st<bf16x8>(smem, L::RR + 2 * ((r_off(i2) + r) * L::KP + c0k), f32x8_to_bf16(rr));
                }
                kbg_rows[i] = f32x8_to_bf16(kb);
                kh_rows[i] = f32x8_to_bf16(kh);
            }
        } else {
            for (int i = 0; i < RPT; ++i) {
                const int r = row0 + i;
                f32x8 qh, kb, kh, ga;
                for (int j = 0; j < 8; ++j) {
                    ga[j] = base[j] + G[i][j];
                    const float eg = __expf(ga[j]), ek = __expf(glast[j] - ga[j]);
                    qh[j] = qf[i][j] * eg;
                    kb[j] = bk[i][j] * eg;
                    kh[j] = kf[i][j] * ek;
                }
                lds_st<f32x4>(smem, L::GF + 4 * (r * L::GP + c0k), f32x4{ga[0], ga[1], ga[2], ga[3]});
                lds_st<f32x4>(smem, L::GF + 4 * (r * L::GP + c0k + 4), f32x4{ga[4], ga[5], ga[6], ga[7]});
                lds_st<bf16x8>(smem, L::QH + 2 * (r * L::KP + c0k), f32x8_to_bf16(qh));
                kbg_rows[i] = f32x8_to_bf16(kb);
                kh_rows[i] = f32x8_to_bf16(kh);
            }
        }
        // (k exp(G_last - G))^T: channel c0k+j, rows row0 .. row0+RPT-1
        for (int j = 0; j < 8; ++j) {
            __bf16 col[RPT];
            for (int i = 0; i < RPT; ++i) col[i] = kh_rows[i][j];
            if constexpr (RPT == 4)
                lds_st<bf16x4>(smem, L::KHT + 2 * ((c0k + j) * L::CP + row0), bf16x4{col[0], col[1], col[2], col[3]});
            else
                lds_st<bf16x2>(smem, L::KHT + 2 * ((c0k + j) * L::CP + row0),
                                 bf16x2{col[0], col[1]});
        }
        __syncthreads();  // ---------------------------------------- B2

        // =========================== phase AP ==========================
        if (fast) {
            for (int tt = wv; tt < 20; tt += 4) {
                const bool isP = tt >= 10;
                const int t10 = isP ? tt - 10 : tt;
                const int i = kTriI[t10], j = kTriJ[t10];
                const int mb = isP ? L::LQ : L::LB;
                f32x4 acc = {0, 0, 0, 0};
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 a = lds_ld<bf16x8>(smem, mb + 2 * ((16 * i + l16) * L::KP + 32 * ks + 8 * q4));
                    const bf16x8 b = lds_ld<bf16x8>(smem, L::RR + 2 * ((r_off(i) + 16 * j + l16) * L::KP + 32 * ks + 8 * q4));
                    acc = mfma16(a, b, acc);
                }
                const int s = 16 * j + l16;
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * i + 4 * q4 + e;
                    if (!isP) lds_st<float>(smem, L::AB + 4 * (r * L::AP + s), s < r ? acc[e] : 0.0f);
                    else lds_st<__bf16>(smem, L::PB + 2 * (r * L::CP + s), (__bf16)(s <= r ? acc[e] : 0.0f));
                }
            }
        } else {
            // exact pairwise evaluation (exponents G_r - G_s <= 0)
            const int r = tid >> 2, s0 = (tid & 3) * 16;
            float accA[16], accP[16];
            for (int x = 0; x < 16; ++x) accA[x] = accP[x] = 0.0f;
            if (r < len) {
                const int64_t tr = c0 + r;
                for (int c8 = 0; c8 < K / 8; ++c8) {
                    const f32x8 qr = bf16x8_to_f32(ldg_bf16x8(p.q + (tr * p.H + hk) * K + 8 * c8));
                    const f32x8 kr = bf16x8_to_f32(ldg_bf16x8(p.k + (tr * p.H + hk) * K + 8 * c8));
                    f32x8 br = {1, 1, 1, 1, 1, 1, 1, 1};
                    if (p.beta) br = bf16x8_to_f32(ldg_bf16x8(p.beta + (tr * p.HV + hv) * K + 8 * c8));
                    const f32x4 gr0 = lds_ld<f32x4>(smem, L::GF + 4 * (r * L::GP + 8 * c8));
                    const f32x4 gr1 = lds_ld<f32x4>(smem, L::GF + 4 * (r * L::GP + 8 * c8 + 4));
                    for (int x = 0; x < 16; ++x) {
                        const int s = s0 + x;
                        if (s > r) break;
                        const f32x8 ks = bf16x8_to_f32(ldg_bf16x8(p.k + ((c0 + s) * p.H + hk) * K + 8 * c8));
                        const f32x4 gs0 = lds_ld<f32x4>(smem, L::GF + 4 * (s * L::GP + 8 * c8));
                        const f32x4 gs1 = lds_ld<f32x4>(smem, L::GF + 4 * (s * L::GP + 8 * c8 + 4));
                        for (int j = 0; j < 8; ++j) {
                            const float gr = j < 4 ? gr0[j] : gr1[j - 4];
                            const float gs = j < 4 ? gs0[j] : gs1[j - 4];
                            const float ex = __expf(gr - gs) * ks[j];
                            accA[x] += br[j] * kr[j] * ex;
                            accP[x] += qr[j] * ex;
                        }
                    }
                }
            }
            for (int x = 0; x < 16; ++x) {
                const int s = s0 + x;
                lds_st<float>(smem, L::AB + 4 * (r * L::AP + s), s < r ? accA[x] : 0.0f);
                lds_st<__bf16>(smem, L::PB + 2 * (r * L::CP + s), (__bf16)(s <= r ? accP[x] : 0.0f));
            }
        }
        __syncthreads();  // ---------------------------------------- B3

        // deferred operands into region X: (beta k exp(G))^T and (w v)^T
        for (int j = 0; j < 8; ++j) {
            __bf16 col[RPT];
            for (int i = 0; i < RPT; ++i) col[i] = kbg_rows[i][j];
            if constexpr (RPT == 4)
                lds_st<bf16x4>(smem, L::KBT + 2 * ((c0k + j) * L::CP + row0), bf16x4{col[0], col[1], col[2], col[3]});
            else
                lds_st<bf16x2>(smem, L::KBT + 2 * ((c0k + j) * L::CP + row0),
                                 bf16x2{col[0], col[1]});
        }
        for (int j = 0; j < 8; ++j) {
            __bf16 col[RPTV];
            for (int i = 0; i < RPTV; ++i) col[i] = (__bf16)wvv[i][j];
            if constexpr (RPTV == 4)
                lds_st<bf16x4>(smem, L::WVT + 2 * ((c0v + j) * L::CP + row0v), bf16x4{col[0], col[1], col[2], col[3]});
            else
                lds_st<bf16x2>(smem, L::WVT + 2 * ((c0v + j) * L::CP + row0v),
                                 bf16x2{col[0], col[1]});
        }

        // =========================== phase T ===========================
        // T1: wave wv inverts diagonal block wv (lanes 0..15 hold column l16)
        {
            const int d0 = 16 * wv;
            float tc[16];
            for (int r = 0; r < 16; ++r) {
                float acc = 0.0f;
                for (int s = 0; s < r; ++s) acc += lds_ld<float>(smem, L::AB + 4 * ((d0 + r) * L::AP + d0 + s)) * tc[s];
                tc[r] = r == l16 ? 1.0f : (r > l16 ? -acc : 0.0f);
            }
            if (lane < 16)
                for (int r = 0; r < 16; ++r) {
                    lds_st<float>(smem, L::AB + 4 * ((d0 + r) * L::AP + d0 + l16), tc[r]);
                    lds_st<__bf16>(smem, L::TB + 2 * ((d0 + r) * L::CP + d0 + l16), (__bf16)tc[r]);
                }
            // the products wy_w and wy_u read T's blocks (0,1) and (2,3): zero them
            if (wv == 0 || wv == 2) {
                const int rr = lane >> 2, cc = (lane & 3) * 4;
                lds_st<uint64_t>(smem, L::TB + 2 * ((d0 + rr) * L::CP + d0 + 16 + cc), 0ull);
            }
        }
        __syncthreads();  // ---------------------------------------- B4
        // T2: B_ik = T_ii A_ik for k < i, into scratch slot i(i-1)/2 + k
        {
            const int rr = lane >> 2, cc = (lane & 3) * 4;
            for (int slot = wv; slot < 6; slot += 4) {
                const int i = slot == 0 ? 1 : (slot < 3 ? 2 : 3);
                const int kb = slot - i * (i - 1) / 2;
                f32x4 acc = {0, 0, 0, 0};
                for (int s = 0; s < 16; ++s) {
                    const float t = lds_ld<float>(smem, L::AB + 4 * ((16 * i + rr) * L::AP + 16 * i + s));
                    const f32x4 a = lds_ld<f32x4>(smem, L::AB + 4 * ((16 * i + s) * L::AP + 16 * kb + cc));
                    acc += t * a;
                }
                lds_st<f32x4>(smem, L::BS + 4 * ((slot * 16 + rr) * L::BP + cc), acc);
            }
        }
        __syncthreads();  // ---------------------------------------- B5
        // T3..T5: T_ij = -sum_{k=j}^{i-1} B_ik T_kj, by distance d = i - j
        for (int d = 1; d <= 3; ++d) {
            if (wv < 4 - d) {
                const int j = wv, i = wv + d;
                const int rr = lane >> 2, cc = (lane & 3) * 4;
                f32x4 acc = {0, 0, 0, 0};
                for (int kb = j; kb < i; ++kb) {
                    const int slot = i * (i - 1) / 2 + kb;
                    for (int s = 0; s < 16; ++s) {
                        const float b = lds_ld<float>(smem, L::BS + 4 * ((slot * 16 + rr) * L::BP + s));
                        const f32x4 t = lds_ld<f32x4>(smem, L::AB + 4 * ((16 * kb + s) * L::AP + 16 * j + cc));
                        acc += b * t;
                    }
                }
                acc = -acc;
                lds_st<f32x4>(smem, L::AB + 4 * ((16 * i + rr) * L::AP + 16 * j + cc), acc);
                lds_st<bf16x4>(smem, L::TB + 2 * ((16 * i + rr) * L::CP + 16 * j + cc), f32x4_to_bf16(acc));
            }
            __syncthreads();  // ------------------------------------ B6..B8
        }

        // =========================== phase WY ==========================
        // -wy_w = -T (beta k exp(G)) for this wave's NCTK column tiles
        for (int jt = 0; jt < NCTK; ++jt) {
            const int cb = 16 * (wv * NCTK + jt);
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {0, 0, 0, 0};
                for (int ks = 0; ks <= (i >> 1); ++ks) {
                    const bf16x8 a = lds_ld<bf16x8>(smem, L::TB + 2 * ((16 * i + l16) * L::CP + 32 * ks + 8 * q4));
                    const bf16x8 b = lds_ld<bf16x8>(smem, L::KBT + 2 * ((cb + l16) * L::CP + 32 * ks + 8 * q4));
                    acc = mfma16(a, b, acc);
                }
                for (int e = 0; e < 4; ++e)
                    lds_st<__bf16>(smem, L::WYW + 2 * ((16 * i + 4 * q4 + e) * L::KP + cb + l16), (__bf16)(-acc[e]));
            }
        }
        // wy_u = T (w v) for this wave's value columns: U starts here
        f32x4 U[4][NCT];
        for (int jt = 0; jt < NCT; ++jt)
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {0, 0, 0, 0};
                for (int ks = 0; ks <= (i >> 1); ++ks) {
                    const bf16x8 a = lds_ld<bf16x8>(smem, L::TB + 2 * ((16 * i + l16) * L::CP + 32 * ks + 8 * q4));
                    const bf16x8 b = lds_ld<bf16x8>(smem, L::WVT + 2 * ((vbase + 16 * jt + l16) * L::CP + 32 * ks + 8 * q4));
                    acc = mfma16(a, b, acc);
                }
                U[i][jt] = acc;
            }
        __syncthreads();  // ---------------------------------------- B9

        // =========================== phase S ===========================
        // S as bf16 B operands: k slab ks holds state rows
        // {32ks + 4q4 + e} and {32ks + 16 + 4q4 + e}, e = 0..3, in that order;
        // the A operands are read with the same column order.
        bf16x8 Sb[NKS][NCT];
        for (int ks = 0; ks < NKS; ++ks)
            for (int jt = 0; jt < NCT; ++jt)
                Sb[ks][jt] = cat4(f32x4_to_bf16(S[2 * ks][jt]), f32x4_to_bf16(S[2 * ks + 1][jt]));
        f32x4 Y[4][NCT];
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * i + l16;
            for (int jt = 0; jt < NCT; ++jt) Y[i][jt] = f32x4{0, 0, 0, 0};
            for (int ks = 0; ks < NKS; ++ks) {
                const int cA = 32 * ks + 4 * q4, cB = cA + 16;
                const bf16x8 aw = cat4(lds_ld<bf16x4>(smem, L::WYW + 2 * (row * L::KP + cA)),
                                       lds_ld<bf16x4>(smem, L::WYW + 2 * (row * L::KP + cB)));
                const bf16x8 aq = cat4(lds_ld<bf16x4>(smem, L::QH + 2 * (row * L::KP + cA)),
                                       lds_ld<bf16x4>(smem, L::QH + 2 * (row * L::KP + cB)));
                for (int jt = 0; jt < NCT; ++jt) {
                    U[i][jt] = mfma16(aw, Sb[ks][jt], U[i][jt]);
                    Y[i][jt] = mfma16(aq, Sb[ks][jt], Y[i][jt]);
                }
            }
        }
        // U as bf16 B operands over tokens (same permuted order)
        bf16x8 Ub[2][NCT];
        for (int ks = 0; ks < 2; ++ks)
            for (int jt = 0; jt < NCT; ++jt)
                Ub[ks][jt] = cat4(f32x4_to_bf16(U[2 * ks][jt]), f32x4_to_bf16(U[2 * ks + 1][jt]));
        // intra-chunk output P U
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * i + l16;
            for (int ks = 0; ks <= (i >> 1); ++ks) {
                const int cA = 32 * ks + 4 * q4, cB = cA + 16;
                const bf16x8 ap = cat4(lds_ld<bf16x4>(smem, L::PB + 2 * (row * L::CP + cA)),
                                       lds_ld<bf16x4>(smem, L::PB + 2 * (row * L::CP + cB)));
                for (int jt = 0; jt < NCT; ++jt) Y[i][jt] = mfma16(ap, Ub[ks][jt], Y[i][jt]);
            }
        }
        // state: decay rows by exp(G_last), then add (k exp(G_last - G))^T U
        for (int it = 0; it < NRT; ++it) {
            const f32x4 gam = lds_ld<f32x4>(smem, L::GAM + 4 * (16 * it + 4 * q4));
            const int row = 16 * it + l16;
            bf16x8 ak[2];
            for (int ks = 0; ks < 2; ++ks) {
                const int cA = 32 * ks + 4 * q4, cB = cA + 16;
                ak[ks] = cat4(lds_ld<bf16x4>(smem, L::KHT + 2 * (row * L::CP + cA)),
                              lds_ld<bf16x4>(smem, L::KHT + 2 * (row * L::CP + cB)));
            }
            for (int jt = 0; jt < NCT; ++jt) {
                f32x4 s = S[it][jt] * gam;
                s = mfma16(ak[0], Ub[0][jt], s);
                s = mfma16(ak[1], Ub[1][jt], s);
                S[it][jt] = s;
            }
        }
        // output tile: stage through LDS, then 16-byte row stores
        for (int i = 0; i < 4; ++i)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e)
                    lds_st<__bf16>(smem, L::OST + 2 * ((16 * i + 4 * q4 + e) * L::VP + vbase + 16 * jt + l16),
                                   (__bf16)(p.scale * Y[i][jt][e]));
        __syncthreads();  // ---------------------------------------- B10
        for (int idx = tid; idx < CH * CGV; idx += NTHR) {
            const int r = idx / CGV, c8 = idx % CGV;
            if (r < len)
                *reinterpret_cast<bf16x8 *>(p.out + ((c0 + r) * p.HV + hv) * V + 8 * c8) =
                    lds_ld<bf16x8>(smem, L::OST + 2 * (r * L::VP + 8 * c8));
        }
    }

    if (p.ht)
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e)
                    p.ht[(((int64_t)n * p.HV + hv) * K + 16 * it + 4 * q4 + e) * V + vbase + 16 * jt + l16] = S[it][jt][e];
}

}  // namespace

hipError_t launch_chunk_fwd(const FwdParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.N * p.HV)), block(NTHR);
    if (p.K == 128 && p.V == 128)
        hipLaunchKernelGGL((chunk_fwd_kernel<128, 128>), grid, block, 0, stream, p);
    else if (p.K == 64 && p.V == 64)
        hipLaunchKernelGGL((chunk_fwd_kernel<64, 64>), grid, block, 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn2
