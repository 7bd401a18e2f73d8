// Fused GDN-2 chunked prefill forward for CDNA4 (gfx950).
//
// One workgroup of 512 threads (8 wave64s) owns one (sequence, value head)
// chain and walks its 64-token chunks in order. The waves have two roles:
//
//   state waves 0-3  hold the K x V float32 state in registers (result layout
//                    of v_mfma_f32_16x16x32_bf16, V split four ways), invert
//                    (I + A) and run the sequential state pass;
//   key waves 4-7    hold the next chunk's raw q, k, beta, g in registers
//                    (prefetched), build the decay factors and MFMA operands,
//                    and the pseudo-keys.
//
// Per chunk (rows r, s are positions in the chunk; G = inclusive in-chunk
// cumulative sum of the log-decay g per key channel, kept in log2 units;
// S = state entering the chunk):
//
//   E   cumulative sum of g (in-thread + wave DPP + LDS exchange of tile
//       totals), then the operands  KB = beta k 2^G,  QH = q 2^G,
//       RR = k 2^-G,  KT = k 2^(G_last - G)  (bf16, row-major in LDS)
//   AP  A_rs = sum_c KB_rc RR_sc   (s < r),   P_rs = sum_c QH_rc RR_sc  (s <= r)
//       on MFMA. 2^G_r 2^-G_s is exp(G_r - G_s) with one reference per
//       chunk; it is used for every channel whose |G| stays within 2^120.
//       Channels beyond that (extreme decay) get RR = 0 and their share of
//       A and P is added by an exact per-pair evaluation of exp(G_r - G_s).
//   T   T = (I + A)^{-1}, float32: diagonal 16x16 blocks by forward
//       substitution, then the block columns by fp32 MFMA chains
//       T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.
//   WY  wy_w = T KB,  wy_u = T (w v)                              (bf16 MFMA)
//   S   U = wy_u - wy_w S;  O = scale (QH S + P U);
//       S <- diag(2^G_last) S + KT^T U                             (bf16 MFMA)
//
// The two roles are software-pipelined across chunks: while the key waves
// build chunk n (phase E), the state waves run phase S of chunk n - 1.
// Operand transposes are LDS transpose reads (ds_read_b64_tr_b16) of the
// row-major tiles, and the output is computed transposed so that every lane
// stores four consecutive values of one output row straight to HBM.
//
// This is the chunked WY evaluation of the recurrence of the FlashInfer
// chunk_gated_delta_rule2 docs (recurrence display equation). The split into
// decay cumsum, decay-scaled K K^T with the erase gate, unit-lower-triangular
// inverse, w/u recompute and a sequential float32 state pass with intra plus
// inter output follows the FlashRT card ("Usage", 64-token WY chain) and the
// burn-gdn2 README ("Fused CUDA kernels"; "Numerical stability": naive
// factors overflow float32 under strong decay, hence the bounded reference
// and the exact fallback). Rows of a partial last chunk are zero-padded
// (q = k = v = 0, g = 0): exact identity steps.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gdn2_internal.h"

namespace gdn2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;       // chunk length
constexpr int NTHR = 512;    // threads per workgroup (8 waves)
constexpr int NROLE = 256;   // threads per role (4 waves)
constexpr float LOG2E = 1.44269504088896340736f;
// Largest |G| (log2 units) of the single-reference factorisation: 2^120 and
// 2^-120 are normal in float32 and bf16, and so is every product used.
constexpr float XLIM = 120.0f;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------- helpers --
__device__ __forceinline__ f32x8 bf16x8_to_f32(bf16x8 x) { return __builtin_convertvector(x, f32x8); }
__device__ __forceinline__ bf16x8 f32x8_to_bf16(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 f32x4_to_bf16(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

__device__ __forceinline__ bf16x8 ldg_bf16x8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x4 ldg_f32x4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T>
__device__ __forceinline__ T lds_ld(const char *base, int off) { return *reinterpret_cast<const T *>(base + off); }
template <typename T>
__device__ __forceinline__ void lds_st(char *base, int off, T v) { *reinterpret_cast<T *>(base + off) = v; }

// LDS transpose read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane s supplies the address of 4 consecutive bf16 of row k0 + s/4,
// columns c0 + 4 (s % 4); lane s receives column c0 + s of rows k0 .. k0 + 3.
__device__ __forceinline__ bf16x4 lds_tr(const char *base, int off)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + off));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// An opaque zero, produced inside a loop body, keeps LDS address arithmetic
// in that body: without it the compiler hoists dozens of loop-invariant
// addresses out of the chunk loop and pins a register for each.
__device__ __forceinline__ int opaque_zero()
{
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// The 20 lower-triangular 16x16 tiles of A (0..9) and P (10..19), each as
// (row tile i, column tile j). Tiles 0-3 are A's diagonal tiles, taken by
// the state waves so that each can invert its block at once; the key waves
// take tiles 4..19.
// Packed 2 bits per tile (no memory access, so no wait on the vector
// memory counter, which also counts the outstanding prefetch):
//   i = 0 1 2 3 1 2 2 3 3 3 0 1 1 2 2 2 3 3 3 3
//   j = 0 1 2 3 0 0 1 0 1 2 0 0 1 0 1 2 0 1 2 3
__device__ __forceinline__ int tile_i(int t) { return (int)((0xffa94fe9e4ull >> (2 * t)) & 3); }
__device__ __forceinline__ int tile_j(int t) { return (int)((0xe4910910e4ull >> (2 * t)) & 3); }

// ------------------------------------------------------------ LDS layout --
// Byte offsets into one static LDS array. Row pitches carry 16 bytes of
// padding to spread rows over banks. Regions that share space have disjoint
// lifetimes within the chunk pipeline (noted per line).
template <int K, int V>
struct Lds {
    static constexpr int KP = K + 8;   // bf16 elements per [token][K] row
    static constexpr int VP = V + 8;   // bf16 elements per [token][V] row
    static constexpr int CP = CH + 8;  // bf16 elements per [token][token] row
    static constexpr int AP = CH + 4;  // fp32 elements per [token][token] row
    static constexpr int NXB = K == 128 ? 16 : 8;  // exact channels per batch

    static constexpr int KB = 0;                                   // beta k 2^G          [64][KP]  E -> WY
    static constexpr int RR = KB + CH * KP * 2;                    // k 2^-G              [64][KP]  E -> AP
    static constexpr int PF = RR;                                  // P fp32 (exact path) [64][AP]  AP only
    static constexpr int RR_SZ = cmax(CH * KP * 2, CH * AP * 4);
    static constexpr int TB = RR + RR_SZ;                          // T bf16; blocks (0,1), (2,3) stay 0 [64][CP]
    static constexpr int QH = TB + CH * CP * 2;                    // q 2^G, by chunk parity [2][64][KP]
    static constexpr int QH_SZ = CH * KP * 2;
    static constexpr int KT = QH + 2 * QH_SZ;                      // k 2^(G_last - G)    [64][KP]  E -> S
    static constexpr int WV = KT + CH * KP * 2;                    // w v                 [64][VP]  T -> WY
    static constexpr int SB = WV;                                  // exact channels: G, beta k, q, k (fp32) [4][NXB][64]
    static constexpr int WV_SZ = cmax(CH * VP * 2, 4 * NXB * CH * 4);
    static constexpr int AB = WV + WV_SZ;                          // A, then T blocks, fp32 [64][AP]  AP -> T
    static constexpr int WYW = AB;                                 // -wy_w bf16          [64][KP]  WY -> S
    static constexpr int AB_SZ = cmax(CH * AP * 4, CH * KP * 2);
    static constexpr int PB = AB + AB_SZ;                          // P bf16              [64][CP]  AP -> S
    static constexpr int GAM = PB + CH * CP * 2;                   // 2^G_last fp32       [K]       E -> S
    static constexpr int TT = GAM + K * 4;                         // tile totals of G    [4][K]
    static constexpr int TX = TT + 4 * K * 4;                      // tile max |G - G(tile start)| [4][K]
    static constexpr int XF = TX + 4 * K * 4;                      // exact-channel flags [K] int
    static constexpr int XL = XF + K * 4;                          // exact-channel list  [K] int
    static constexpr int FL = XL + K * 4;                          // chunk flag, exact-channel count
    static constexpr int TOTAL = FL + 16;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Phase-E thread map of one role (4 waves over a 64-row x NC-column chunk,
// 8 columns per thread): wave w owns rows [16w, 16w + 16); inside a wave the
// row group varies fastest, so that consecutive lanes write consecutive rows.
template <int NC>
struct EMap {
    static constexpr int CG = NC / 8;              // column groups
    static constexpr int RGW = 64 / CG;            // row groups per wave
    static constexpr int RPT = 16 / RGW;           // rows per thread
    int rgl, cg, row0, c0;
    __device__ __forceinline__ explicit EMap(int rt)
    {
        const int lane = rt & 63, w = rt >> 6;
        rgl = lane % RGW;
        cg = lane / RGW;
        row0 = (w * RGW + rgl) * RPT;
        c0 = cg * 8;
    }
};

// Raw inputs of one chunk as loaded from HBM (bf16 kept packed), in the key
// waves' thread map: rows row0 + i, channels c0k .. c0k + 7. Rows past the
// end of the sequence hold a copy of its last row; the consumer zeroes them,
// so that no instruction touches the registers while the loads are in
// flight (a select right after a load would wait for it).
template <int RPT>
struct RawChunk {
    bf16x8 q[RPT], k[RPT], b[RPT];
    f32x4 g[RPT][2];
};

// Stand-ins for omitted gates: one row of ones (beta, w) or zeros (g), read
// with row stride 0. They live in global memory (not the constant address
// space) so that a pointer that may be either an input or a stand-in stays a
// global pointer: a flat load would also count against the LDS wait counter,
// and every later LDS wait would then wait for the HBM prefetch as well.
__device__ __attribute__((aligned(16))) uint16_t kOnesBf16[8] = {0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                                               0x3f80, 0x3f80, 0x3f80, 0x3f80};
__device__ __attribute__((aligned(16))) float kZerosF32[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// Straight-line loads: rows past the chunk end read the last valid row (the
// consumer masks them); omitted gates read the stand-in row.
template <int K, int RPT>
__device__ __forceinline__ void load_decay(RawChunk<RPT> &R, const FwdParams &p, int64_t c0, int len, int hv,
                                           int row0, int c0k)
{
    const float *gb = p.g ? p.g + (c0 * p.HV + hv) * K : kZerosF32;
    const int sg = p.g ? p.HV * K : 0, cgg = p.g ? c0k : 0;
    for (int i = 0; i < RPT; ++i) {
        const int r = row0 + i;
        const int rc = r < len ? r : len - 1;
        R.g[i][0] = ldg_f32x4(gb + (uint32_t)(rc * sg + cgg));
        R.g[i][1] = ldg_f32x4(gb + (uint32_t)(rc * sg + cgg) + 4);
    }
}

template <int K, int RPT>
__device__ __forceinline__ void load_keys(RawChunk<RPT> &R, const FwdParams &p, int64_t c0, int len, int hk,
                                          int hv, int row0, int c0k)
{
    // wave-uniform chunk bases + 32-bit per-lane offsets
    const uint16_t *qb = p.q + (c0 * p.H + hk) * K;
    const uint16_t *kb = p.k + (c0 * p.H + hk) * K;
    const uint16_t *bb = p.beta ? p.beta + (c0 * p.HV + hv) * K : kOnesBf16;
    const int sqk = p.H * K, sb = p.beta ? p.HV * K : 0, cb = p.beta ? c0k : 0;
    for (int i = 0; i < RPT; ++i) {
        const int r = row0 + i;
        const int rc = r < len ? r : len - 1;
        R.q[i] = ldg_bf16x8(qb + (uint32_t)(rc * sqk + c0k));
        R.k[i] = ldg_bf16x8(kb + (uint32_t)(rc * sqk + c0k));
        R.b[i] = ldg_bf16x8(bb + (uint32_t)(rc * sb + cb));
    }
}

// Value-side rows of one chunk (state waves): v and w, rows row0 + i,
// columns c0 .. c0 + 7; rows past the end repeat the last row (masked by the
// consumer).
template <int V, int RPTV>
__device__ __forceinline__ void load_values(bf16x8 *v, bf16x8 *w, const FwdParams &p, int64_t c0, int len, int hv,
                                            int row0, int c0v)
{
    const uint16_t *vb = p.v + (c0 * p.HV + hv) * V;
    const uint16_t *wb = p.w ? p.w + (c0 * p.HV + hv) * V : kOnesBf16;
    const int svw = p.HV * V, sw = p.w ? svw : 0, cw = p.w ? c0v : 0;
    for (int i = 0; i < RPTV; ++i) {
        const int r = row0 + i;
        const int rc = r < len ? r : len - 1;
        v[i] = ldg_bf16x8(vb + (uint32_t)(rc * svw + c0v));
        w[i] = ldg_bf16x8(wb + (uint32_t)(rc * sw + cw));
    }
}

// Reductions over the RGW consecutive lanes of a row group: DPP quad
// permutes (and a half-row mirror for 8 lanes).
template <int RGW>
__device__ __forceinline__ float group_max(float x)
{
    static_assert(RGW == 4 || RGW == 8, "4 or 8 lanes per row group");
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));
    if constexpr (RGW == 8)
        x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)));
    return x;
}

// Inclusive prefix sum over the RGW consecutive lanes of a row group
// (rgl = lane index inside the group).
template <int RGW>
__device__ __forceinline__ float group_scan(float x, int rgl)
{
    if constexpr (RGW == 4) {  // DPP row shifts by 1 and 2 lanes
        const float o1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
        if (rgl >= 1) x += o1;
        const float o2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
        if (rgl >= 2) x += o2;
    } else {
        for (int d = 1; d < RGW; d <<= 1) {
            const float o = __shfl_up(x, d, 64);
            if (rgl >= d) x += o;
        }
    }
    return x;
}

// ----------------------------------------------------------- chain context --
struct Chain {
    int n, hv, hk;
    int64_t tb, te;  // token range of the sequence
};

__device__ __forceinline__ int chunk_len(int64_t c0, int64_t te) { return (int)((te - c0) < CH ? (te - c0) : CH); }

// --------------------------------------------------------------- phase AP --
// One 16x16 tile of A (X = KB) or P (X = QH), computed transposed:
// C[s][r] = sum_c RR[s][c] X[r][c]. Lane (l16, q4) receives row r = 16i + l16,
// columns s = 16j + 4 q4 + e, e = 0..3.
template <int K, int V>
__device__ __forceinline__ f32x4 ap_tile(const char *smem, int i, int j, int xb, int l16, int q4)
{
    using L = Lds<K, V>;
    f32x4 acc = {0, 0, 0, 0};
    for (int ks = 0; ks < K / 32; ++ks) {
        const int c8 = 32 * ks + 8 * q4;
        const bf16x8 a = lds_ld<bf16x8>(smem, L::RR + 2 * ((16 * j + l16) * L::KP + c8));
        const bf16x8 b = lds_ld<bf16x8>(smem, xb + 2 * ((16 * i + l16) * L::KP + c8));
        acc = mfma_bf16(a, b, acc);
    }
    return acc;
}

// Keep the causal part of a tile: s < r for A, s <= r for P (only diagonal
// tiles have entries to drop).
__device__ __forceinline__ f32x4 ap_mask(f32x4 x, bool diag, bool isP, int l16, int q4)
{
    if (diag)
        for (int e = 0; e < 4; ++e) {
            const int s = 4 * q4 + e;
            x[e] = (isP ? s <= l16 : s < l16) ? x[e] : 0.0f;
        }
    return x;
}

// Exact-channel path of phase AP, run by all 512 threads with an identical
// barrier sequence. MFMA tiles give the contribution of the channels with
// bounded |G| (RR is zero on the others); every exact channel then adds
// beta_r k_r k_s exp(G_r - G_s) and q_r k_s exp(G_r - G_s) per pair,
// NXB channels per batch, with G rebuilt from g in float32.
template <int K, int V>
__device__ void exact_ap(char *smem, const FwdParams &p, const Chain &ch, int64_t c0, int len, int qb, int tid)
{
    using L = Lds<K, V>;
    constexpr int NXB = L::NXB;
    constexpr int TPC = NTHR / NXB;  // threads per channel in the fill step
    constexpr int RPX = CH / TPC;    // rows per thread in the fill step
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l16 = lane & 15, q4 = lane >> 4;

    // compact list of the exact channels (wave 0)
    if (wv == 0) {
        int cnt = 0;
        for (int cb = 0; cb < K; cb += 64) {
            const int c = cb + lane;
            const bool f = lds_ld<int>(smem, L::XF + 4 * c) != 0;
            const uint64_t m = __ballot(f);
            if (f) lds_st<int>(smem, L::XL + 4 * (cnt + __popcll(m & ((1ull << lane) - 1))), c);
            cnt += __popcll(m);
        }
        if (lane == 0) lds_st<int>(smem, L::FL + 4, cnt);
    }
    f32x4 acc[3];
    for (int m = 0; m < 3; ++m) {
        const int t = wv + 8 * m;
        if (t < 20) {
            const int i = tile_i(t), j = tile_j(t);
            acc[m] = ap_tile<K, V>(smem, i, j, t >= 10 ? qb : L::KB, l16, q4);
        }
    }
    __syncthreads();  // RR is read; the list is visible
    for (int m = 0; m < 3; ++m) {
        const int t = wv + 8 * m;
        if (t < 20) {
            const int i = tile_i(t), j = tile_j(t);
            const bool isP = t >= 10;
            const f32x4 x = ap_mask(acc[m], i == j, isP, l16, q4);
            lds_st<f32x4>(smem, (isP ? L::PF : L::AB) + 4 * ((16 * i + l16) * L::AP + 16 * j + 4 * q4), x);
        }
    }
    const int nx = lds_ld<int>(smem, L::FL + 4);
    const int r = tid >> 3, sb = tid & 7;
    float accA[8], accP[8];
    for (int u = 0; u < 8; ++u) accA[u] = accP[u] = 0.0f;
    const float *gp = p.g ? p.g + (c0 * p.HV + ch.hv) * K : nullptr;
    const uint16_t *qp = p.q + (c0 * p.H + ch.hk) * K;
    const uint16_t *kp = p.k + (c0 * p.H + ch.hk) * K;
    const uint16_t *bp = p.beta ? p.beta + (c0 * p.HV + ch.hv) * K : nullptr;
    for (int b0 = 0; b0 < nx; b0 += NXB) {
        const int nb = nx - b0 < NXB ? nx - b0 : NXB;
        __syncthreads();  // the previous batch is consumed
        {
            const int x = tid / TPC, ti = tid % TPC;
            float gs[RPX], bk[RPX], qs[RPX], kv[RPX];
            const int c = x < nb ? lds_ld<int>(smem, L::XL + 4 * (b0 + x)) : 0;
            float run = 0.0f;
            for (int u = 0; u < RPX; ++u) {
                const int rr = ti * RPX + u;
                const bool ok = x < nb && rr < len;
                const int64_t t = ok ? rr : 0;
                const float gv = ok && gp ? gp[t * p.HV * K + c] * LOG2E : 0.0f;
                const float qv = ok ? bf16_bits_to_f32(qp[t * p.H * K + c]) : 0.0f;
                const float kk = ok ? bf16_bits_to_f32(kp[t * p.H * K + c]) : 0.0f;
                const float bv = ok && bp ? bf16_bits_to_f32(bp[t * p.HV * K + c]) : 1.0f;
                run += gv;
                gs[u] = run;
                bk[u] = bv * kk;
                qs[u] = qv;
                kv[u] = kk;
            }
            // inclusive scan of the per-thread totals over the channel's TPC lanes
            float inc = run;
            for (int d = 1; d < TPC; d <<= 1) {
                const float o = __shfl_up(inc, d, TPC);
                if (ti >= d) inc += o;
            }
            const float excl = inc - run;
            if (x < nb)
                for (int u = 0; u < RPX; ++u) {
                    const int o = 4 * (x * CH + ti * RPX + u);
                    lds_st<float>(smem, L::SB + o, gs[u] + excl);
                    lds_st<float>(smem, L::SB + NXB * CH * 4 + o, bk[u]);
                    lds_st<float>(smem, L::SB + 2 * NXB * CH * 4 + o, qs[u]);
                    lds_st<float>(smem, L::SB + 3 * NXB * CH * 4 + o, kv[u]);
                }
        }
        __syncthreads();  // the batch is staged
        if (8 * sb <= r)
            for (int x = 0; x < nb; ++x) {
                const int o = 4 * x * CH;
                const float gr = lds_ld<float>(smem, L::SB + o + 4 * r);
                const float bkr = lds_ld<float>(smem, L::SB + NXB * CH * 4 + o + 4 * r);
                const float qsr = lds_ld<float>(smem, L::SB + 2 * NXB * CH * 4 + o + 4 * r);
                const f32x4 g0 = lds_ld<f32x4>(smem, L::SB + o + 4 * 8 * sb);
                const f32x4 g1 = lds_ld<f32x4>(smem, L::SB + o + 4 * (8 * sb + 4));
                const f32x4 k0 = lds_ld<f32x4>(smem, L::SB + 3 * NXB * CH * 4 + o + 4 * 8 * sb);
                const f32x4 k1 = lds_ld<f32x4>(smem, L::SB + 3 * NXB * CH * 4 + o + 4 * (8 * sb + 4));
                for (int u = 0; u < 8; ++u) {
                    const int s = 8 * sb + u;
                    const float gsu = u < 4 ? g0[u] : g1[u - 4];
                    const float ksu = u < 4 ? k0[u] : k1[u - 4];
                    const float wgt = ksu * ex2(gr - gsu);
                    accA[u] += s < r ? bkr * wgt : 0.0f;
                    accP[u] += s <= r ? qsr * wgt : 0.0f;
                }
            }
    }
    __syncthreads();  // every MFMA tile is stored
    {
        const int ab = L::AB + 4 * (r * L::AP + 8 * sb), pf = L::PF + 4 * (r * L::AP + 8 * sb);
        f32x4 a0 = lds_ld<f32x4>(smem, ab), a1 = lds_ld<f32x4>(smem, ab + 16);
        const f32x4 p0 = lds_ld<f32x4>(smem, pf), p1 = lds_ld<f32x4>(smem, pf + 16);
        f32x8 pv;
        for (int u = 0; u < 8; ++u) {
            const int s = 8 * sb + u;
            const float av = (u < 4 ? a0[u] : a1[u - 4]) + accA[u];
            if (u < 4) a0[u] = s < r ? av : 0.0f;
            else a1[u - 4] = s < r ? av : 0.0f;
            pv[u] = s <= r ? (u < 4 ? p0[u] : p1[u - 4]) + accP[u] : 0.0f;
        }
        lds_st<f32x4>(smem, ab, a0);
        lds_st<f32x4>(smem, ab + 16, a1);
        lds_st<bf16x8>(smem, L::PB + 2 * (r * L::CP + 8 * sb), f32x8_to_bf16(pv));
    }
    __syncthreads();  // A and P are complete
}

// ---------------------------------------------------------------- phase T1 --
// Diagonal block i of T = (I + A)^{-1} by forward substitution,
// T_rc = delta_rc - sum_{s<r} A_rs T_sc: lane l16 builds column l16 (every
// lane group redundantly) from the block's rows read as broadcasts. The
// block is written over A's block in AB (fp32) and into TB (bf16); lane
// group q4 writes rows 4 q4 .. 4 q4 + 3.
template <int K, int V>
__device__ __forceinline__ void t1_block(char *smem, int i, int l16, int q4)
{
    using L = Lds<K, V>;
    const int d0 = 16 * i;
    // the strictly lower triangle first (one wait), then a pure FMA chain
    float a[16][16];
    for (int r = 1; r < 16; ++r)
        for (int s4 = 0; s4 < r; s4 += 4) {
            const f32x4 x = lds_ld<f32x4>(smem, L::AB + 4 * ((d0 + r) * L::AP + d0 + s4));
            for (int e = 0; e < 4; ++e) a[r][s4 + e] = x[e];
        }
    float t[16];
    t[0] = l16 == 0 ? 1.0f : 0.0f;
    for (int r = 1; r < 16; ++r) {
        float acc0 = 0.0f, acc1 = 0.0f;
        for (int s2 = 0; s2 < r; ++s2) {
            if (s2 & 1) acc1 = fmaf(a[r][s2], t[s2], acc1);
            else acc0 = fmaf(a[r][s2], t[s2], acc0);
        }
        t[r] = (r == l16 ? 1.0f : 0.0f) - (acc0 + acc1);
    }
    f32x4 out;
    for (int e = 0; e < 4; ++e)
        out[e] = q4 == 0 ? t[e] : q4 == 1 ? t[4 + e] : q4 == 2 ? t[8 + e] : t[12 + e];
    for (int e = 0; e < 4; ++e) {
        lds_st<float>(smem, L::AB + 4 * ((d0 + 4 * q4 + e) * L::AP + d0 + l16), out[e]);
        lds_st<__bf16>(smem, L::TB + 2 * ((d0 + 4 * q4 + e) * L::CP + d0 + l16), (__bf16)out[e]);
    }
}

// ------------------------------------------------------------- key waves --
// Barrier sequence per iteration (must match state_role): B1, B2, then
// (exact_ap), B3, B4, B5.
template <int K, int V>
__device__ __forceinline__ void key_role(char *smem, const FwdParams &p, const Chain &ch, int tid, int nc)
{
    using L = Lds<K, V>;
    constexpr int CGK = K / 8;              // 8-channel groups along K
    constexpr int RPT = CH * CGK / NROLE;   // rows per thread
    constexpr int RGW = 64 / CGK;           // row groups per wave
    constexpr int NCTK = K / 64;            // -wy_w channel tiles per key wave
    static_assert(RPT * RGW == 16, "a key wave covers one 16-row tile");

    RawChunk<RPT> R;
    if (nc > 0) {
        const EMap<K> em(tid & (NROLE - 1));
        load_decay<K, RPT>(R, p, ch.tb, chunk_len(ch.tb, ch.te), ch.hv, em.row0, em.c0);
        load_keys<K, RPT>(R, p, ch.tb, chunk_len(ch.tb, ch.te), ch.hk, ch.hv, em.row0, em.c0);
        // complete the first chunk's loads before the loop, so that inside
        // it the vector memory counter only tracks the in-loop prefetch,
        // issued g first (a wait for g then leaves q, k, beta in flight)
        for (int i = 0; i < RPT; ++i) asm volatile("" ::"v"(R.q[i]), "v"(R.k[i]), "v"(R.b[i]), "v"(R.g[i][0]), "v"(R.g[i][1]));
    }

    char *const smem0 = smem;
    const int tid0 = tid;
    for (int it = 0; it <= nc; ++it) {
        // lane-derived values are recomputed per chunk (see opaque_zero)
        const int z = opaque_zero();
        char *smem = smem0 + z;
        const int tid = tid0 + z;
        const int lane = tid & 63, rw = __builtin_amdgcn_readfirstlane((tid >> 6) & 3), rt = tid & (NROLE - 1);
        const int l16 = lane & 15, q4 = lane >> 4;
        const EMap<K> em(rt);
        const int rgl = em.rgl, row0 = em.row0, c0k = em.c0;
        const int64_t c0 = ch.tb + (int64_t)it * CH;
        const bool act = it < nc;
        const int len = act ? chunk_len(c0, ch.te) : 0;
        const int qb = L::QH + (it & 1) * L::QH_SZ;

        // ---- E1: tile-local cumulative log2 decay, tile totals and spans
        float G[RPT][8];
        if (act) {
            for (int i = 0; i < RPT; ++i)
                for (int j = 0; j < 8; ++j)
                    G[i][j] = (i ? G[i - 1][j] : 0.0f) +
                              (row0 + i < len ? (j < 4 ? R.g[i][0][j] : R.g[i][1][j - 4]) * LOG2E : 0.0f);
            float tx[8];
            for (int j = 0; j < 8; ++j) {
                const float tot = G[RPT - 1][j];
                const float excl = group_scan<RGW>(tot, rgl) - tot;
                float m = 0.0f;
                for (int i = 0; i < RPT; ++i) {
                    G[i][j] += excl;
                    m = fmaxf(m, fabsf(G[i][j]));
                }
                tx[j] = group_max<RGW>(m);
            }
            if (rgl == RGW - 1) {
                lds_st<f32x4>(smem, L::TT + 4 * (rw * K + c0k), f32x4{G[RPT - 1][0], G[RPT - 1][1], G[RPT - 1][2], G[RPT - 1][3]});
                lds_st<f32x4>(smem, L::TT + 4 * (rw * K + c0k + 4), f32x4{G[RPT - 1][4], G[RPT - 1][5], G[RPT - 1][6], G[RPT - 1][7]});
            }
            if (rgl == 0) {
                lds_st<f32x4>(smem, L::TX + 4 * (rw * K + c0k), f32x4{tx[0], tx[1], tx[2], tx[3]});
                lds_st<f32x4>(smem, L::TX + 4 * (rw * K + c0k + 4), f32x4{tx[4], tx[5], tx[6], tx[7]});
            }
        }
        __syncthreads();  // ------------------------------------------ B1

        // ---- E3: chunk-relative G, exact-channel flags, operands
        bf16x8 ktr[RPT];
        f32x8 egl;
        if (act) {
            float base[8], glast[8];
            bool xf[8], anyx = false;
            for (int h = 0; h < 2; ++h) {
                f32x4 acc = {0, 0, 0, 0}, bs = {0, 0, 0, 0}, xm = {0, 0, 0, 0};
                for (int t = 0; t < 4; ++t) {
                    const f32x4 tt = lds_ld<f32x4>(smem, L::TT + 4 * (t * K + c0k + 4 * h));
                    const f32x4 tx = lds_ld<f32x4>(smem, L::TX + 4 * (t * K + c0k + 4 * h));
                    if (t == rw) bs = acc;
                    for (int e = 0; e < 4; ++e) xm[e] = fmaxf(xm[e], fabsf(acc[e]) + tx[e]);
                    acc += tt;
                }
                for (int e = 0; e < 4; ++e) {
                    base[4 * h + e] = bs[e];
                    glast[4 * h + e] = acc[e];
                    xf[4 * h + e] = !(xm[e] <= XLIM);  // NaN counts as extreme
                    anyx |= xf[4 * h + e];
                }
            }
            const bool wx = __any(anyx);  // every key wave covers all K channels
            if (rw == 0 && lane == 0) lds_st<int>(smem, L::FL, wx ? 1 : 0);
            if (wx && rw == 0 && rgl == 0) {
                lds_st<i32x4>(smem, L::XF + 4 * c0k, i32x4{xf[0], xf[1], xf[2], xf[3]});
                lds_st<i32x4>(smem, L::XF + 4 * (c0k + 4), i32x4{xf[4], xf[5], xf[6], xf[7]});
            }
            for (int j = 0; j < 8; ++j) egl[j] = ex2(glast[j]);
            for (int i = 0; i < RPT; ++i)
                for (int j = 0; j < 8; ++j) G[i][j] += base[j];
            const bf16x8 zero = {};
            for (int i = 0; i < RPT; ++i) {
                const int r = row0 + i;
                const bool ok = r < len;
                const f32x8 qf = bf16x8_to_f32(ok ? R.q[i] : zero);
                const f32x8 kf = bf16x8_to_f32(ok ? R.k[i] : zero);
                const f32x8 bk = bf16x8_to_f32(R.b[i]) * kf;
                f32x8 kb, qh, rr, kt;
                if (!wx) {
                    for (int j = 0; j < 8; ++j) {
                        const float eg = ex2(G[i][j]), ie = ex2(-G[i][j]);
                        kb[j] = bk[j] * eg;
                        qh[j] = qf[j] * eg;
                        rr[j] = kf[j] * ie;
                        kt[j] = rr[j] * egl[j];
                    }
                } else {
                    for (int j = 0; j < 8; ++j) {
                        const float eg = ex2(G[i][j]);
                        kb[j] = bk[j] * eg;
                        qh[j] = qf[j] * eg;
                        rr[j] = xf[j] ? 0.0f : kf[j] * ex2(-G[i][j]);
                        kt[j] = xf[j] ? kf[j] * ex2(glast[j] - G[i][j]) : rr[j] * egl[j];
                    }
                }
                lds_st<bf16x8>(smem, L::KB + 2 * (r * L::KP + c0k), f32x8_to_bf16(kb));
                lds_st<bf16x8>(smem, L::RR + 2 * (r * L::KP + c0k), f32x8_to_bf16(rr));
                lds_st<bf16x8>(smem, qb + 2 * (r * L::KP + c0k), f32x8_to_bf16(qh));
                ktr[i] = f32x8_to_bf16(kt);
            }
        }
        __syncthreads();  // ------------------------------------------ B2
        if (!act) break;

        // KT and 2^G_last of this chunk: the state waves read the previous
        // chunk's until B2
        for (int i = 0; i < RPT; ++i) lds_st<bf16x8>(smem, L::KT + 2 * ((row0 + i) * L::KP + c0k), ktr[i]);
        if (rw == 0 && rgl == 0) {
            lds_st<f32x4>(smem, L::GAM + 4 * c0k, f32x4{egl[0], egl[1], egl[2], egl[3]});
            lds_st<f32x4>(smem, L::GAM + 4 * (c0k + 4), f32x4{egl[4], egl[5], egl[6], egl[7]});
        }

        // ---- AP + T1: A's diagonal tile rw, then its block of T
        if (lds_ld<int>(smem, L::FL) == 0) {
            const f32x4 x = ap_mask(ap_tile<K, V>(smem, rw, rw, L::KB, l16, q4), true, false, l16, q4);
            lds_st<f32x4>(smem, L::AB + 4 * ((16 * rw + l16) * L::AP + 16 * rw + 4 * q4), x);
        } else {
            exact_ap<K, V>(smem, p, ch, c0, len, qb, tid);
        }
        t1_block<K, V>(smem, rw, l16, q4);
        __syncthreads();  // ------------------------------------------ B3

        // the next chunk's g, q, k, beta: issued while the state waves build
        // T's off-diagonal blocks (the issue stalls until the CU's memory
        // pipeline has room); T2, WY and phase E1 hide the latency
        if (it + 1 < nc) {
            load_decay<K, RPT>(R, p, c0 + CH, chunk_len(c0 + CH, ch.te), ch.hv, row0, c0k);
            load_keys<K, RPT>(R, p, c0 + CH, chunk_len(c0 + CH, ch.te), ch.hk, ch.hv, row0, c0k);
        } else {
            R = RawChunk<RPT>{};  // ends the live range of this chunk's values here
        }
        __syncthreads();  // ------------------------------------------ B4

        // ---- WY: -wy_w^T = -KB^T T^T for this wave's channel tiles, stored
        // row-major (token, channel) as -wy_w
        for (int jt = 0; jt < NCTK; ++jt) {
            const int ct = rw * NCTK + jt;
            bf16x8 ak[2];
            for (int ks = 0; ks < 2; ++ks) {
                const int off = L::KB + 2 * ((32 * ks + 8 * q4 + (l16 >> 2)) * L::KP + 16 * ct + 4 * (l16 & 3));
                ak[ks] = cat4(lds_tr(smem, off), lds_tr(smem, off + 2 * 4 * L::KP));
            }
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {0, 0, 0, 0};
                for (int ks = 0; ks <= (i >> 1); ++ks) {
                    const bf16x8 b = lds_ld<bf16x8>(smem, L::TB + 2 * ((16 * i + l16) * L::CP + 32 * ks + 8 * q4));
                    acc = mfma_bf16(ak[ks], b, acc);
                }
                lds_st<bf16x4>(smem, L::WYW + 2 * ((16 * i + l16) * L::KP + 16 * ct + 4 * q4), f32x4_to_bf16(-acc));
            }
        }
        __syncthreads();  // ------------------------------------------ B5
    }
}

// ----------------------------------------------------------- state waves --
template <int K, int V>
__device__ __forceinline__ void state_role(char *smem, const FwdParams &p, const Chain &ch, int tid, int nc)
{
    using L = Lds<K, V>;
    constexpr int CGV = V / 8;
    constexpr int RPTV = CH * CGV / NROLE;
    constexpr int VW = V / 4;     // value columns per state wave
    constexpr int NCT = VW / 16;  // 16-column tiles per state wave
    constexpr int NRT = K / 16;   // 16-row tiles of the state
    constexpr int NKS = K / 32;   // 32-deep k slabs over K

    // state: rows 16*it + 4*q4 + e, column vbase + 16*jt + l16
    f32x4 S[NRT][NCT];
    {
        const int lane = tid & 63, rw = tid >> 6;
        const int l16 = lane & 15, q4 = lane >> 4;
        const int vbase = rw * VW;
        if (p.h0) {
            const float *h0 = p.h0 + ((int64_t)ch.n * p.HV + ch.hv) * K * V;
            for (int it = 0; it < NRT; ++it)
                for (int jt = 0; jt < NCT; ++jt)
                    for (int e = 0; e < 4; ++e) S[it][jt][e] = h0[(16 * it + 4 * q4 + e) * V + vbase + 16 * jt + l16];
            // complete these loads here: left outstanding into the chunk
            // loop, they make every later write of S wait on the vector
            // memory counter, which then also waits for the v, w prefetch
            for (int it = 0; it < NRT; ++it)
                for (int jt = 0; jt < NCT; ++jt) asm volatile("" ::"v"(S[it][jt]));
        } else {
            for (int it = 0; it < NRT; ++it)
                for (int jt = 0; jt < NCT; ++jt) S[it][jt] = f32x4{0, 0, 0, 0};
        }
    }
    f32x4 U[4][NCT];  // wy_u, then U, of the chunk in the state pass

    char *const smem0 = smem;
    const int tid0 = tid;
    for (int it = 0; it <= nc; ++it) {
        const int z = opaque_zero();
        char *smem = smem0 + z;
        const int tid = tid0 + z;
        const int lane = tid & 63, rw = __builtin_amdgcn_readfirstlane(tid >> 6), rt = tid;
        const int l16 = lane & 15, q4 = lane >> 4;
        const int vbase = rw * VW;
        const int64_t c0 = ch.tb + (int64_t)it * CH;
        const bool act = it < nc;
        const int len = act ? chunk_len(c0, ch.te) : 0;

        // ---- S, first half (chunk it - 1): U = wy_u - wy_w S. S as bf16
        // operands: k slab ks holds state rows {32ks + 4q4 + e} then
        // {32ks + 16 + 4q4 + e}, e = 0..3; LDS operands are read with the
        // same k order, and U as bf16 operands (Ub) in the same way over
        // tokens.
        bf16x8 Ub[2][NCT], Sb[NKS][NCT];
        if (it > 0) {
            for (int ks = 0; ks < NKS; ++ks)
                for (int jt = 0; jt < NCT; ++jt)
                    Sb[ks][jt] = cat4(f32x4_to_bf16(S[2 * ks][jt]), f32x4_to_bf16(S[2 * ks + 1][jt]));
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * i + l16;
                for (int ks = 0; ks < NKS; ++ks) {
                    const int cA = 32 * ks + 4 * q4, cB = cA + 16;
                    const bf16x8 aw = cat4(lds_ld<bf16x4>(smem, L::WYW + 2 * (row * L::KP + cA)),
                                           lds_ld<bf16x4>(smem, L::WYW + 2 * (row * L::KP + cB)));
                    for (int jt = 0; jt < NCT; ++jt) U[i][jt] = mfma_bf16(aw, Sb[ks][jt], U[i][jt]);
                }
            }
            for (int ks = 0; ks < 2; ++ks)
                for (int jt = 0; jt < NCT; ++jt)
                    Ub[ks][jt] = cat4(f32x4_to_bf16(U[2 * ks][jt]), f32x4_to_bf16(U[2 * ks + 1][jt]));
        }
        __syncthreads();  // ------------------------------------------ B1

        // this chunk's v and w (stored as w v after B3; the latency hides
        // behind the rest of phase S, AP and T1)
        bf16x8 vr[RPTV], wr[RPTV];
        const EMap<V> emv(rt);
        if (act) load_values<V, RPTV>(vr, wr, p, c0, len, ch.hv, emv.row0, emv.c0);

        // ---- S, second half: the output, computed transposed,
        // O^T = scale (S^T QH^T + U^T P^T), stored as 4 consecutive values
        // of an output row per lane; then S <- diag(2^G_last) S + KT^T U,
        // with KT^T operands from transpose reads of the row-major KT
        // (tokens in the permuted order of Ub).
        if (it > 0) {
            const int64_t cp = c0 - CH;
            const int lenp = chunk_len(cp, ch.te);
            const int qbp = L::QH + ((it - 1) & 1) * L::QH_SZ;
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * i + l16;
                f32x4 Y[NCT];
                for (int jt = 0; jt < NCT; ++jt) Y[jt] = f32x4{0, 0, 0, 0};
                for (int ks = 0; ks < NKS; ++ks) {
                    const int cA = 32 * ks + 4 * q4, cB = cA + 16;
                    const bf16x8 bq = cat4(lds_ld<bf16x4>(smem, qbp + 2 * (row * L::KP + cA)),
                                           lds_ld<bf16x4>(smem, qbp + 2 * (row * L::KP + cB)));
                    for (int jt = 0; jt < NCT; ++jt) Y[jt] = mfma_bf16(Sb[ks][jt], bq, Y[jt]);
                }
                for (int ks = 0; ks <= (i >> 1); ++ks) {
                    const int cA = 32 * ks + 4 * q4, cB = cA + 16;
                    const bf16x8 bp = cat4(lds_ld<bf16x4>(smem, L::PB + 2 * (row * L::CP + cA)),
                                           lds_ld<bf16x4>(smem, L::PB + 2 * (row * L::CP + cB)));
                    for (int jt = 0; jt < NCT; ++jt) Y[jt] = mfma_bf16(Ub[ks][jt], bp, Y[jt]);
                }
                if (row < lenp)
                    for (int jt = 0; jt < NCT; ++jt)
                        *reinterpret_cast<bf16x4 *>(p.out + ((cp + row) * p.HV + ch.hv) * V + vbase + 16 * jt + 4 * q4) =
                            f32x4_to_bf16(Y[jt] * p.scale);
            }
            for (int rtile = 0; rtile < NRT; ++rtile) {
                const f32x4 gam = lds_ld<f32x4>(smem, L::GAM + 4 * (16 * rtile + 4 * q4));
                bf16x8 ak[2];
                for (int ks = 0; ks < 2; ++ks) {
                    const int off = L::KT + 2 * ((32 * ks + 4 * q4 + (l16 >> 2)) * L::KP + 16 * rtile + 4 * (l16 & 3));
                    ak[ks] = cat4(lds_tr(smem, off), lds_tr(smem, off + 2 * 16 * L::KP));
                }
                for (int jt = 0; jt < NCT; ++jt) {
                    f32x4 s = S[rtile][jt] * gam;
                    s = mfma_bf16(ak[0], Ub[0][jt], s);
                    s = mfma_bf16(ak[1], Ub[1][jt], s);
                    S[rtile][jt] = s;
                }
            }
        }
        __syncthreads();  // ------------------------------------------ B2
        if (!act) break;

        // ---- AP: the 16 tiles that are not A's diagonal, four per state wave
        if (lds_ld<int>(smem, L::FL) == 0) {
            const int qb = L::QH + (it & 1) * L::QH_SZ;
            for (int m = 0; m < 4; ++m) {
                const int t = 4 + rw + 4 * m;
                const int i = tile_i(t), j = tile_j(t);
                const bool isP = t >= 10;
                const f32x4 x = ap_mask(ap_tile<K, V>(smem, i, j, isP ? qb : L::KB, l16, q4), i == j, isP, l16, q4);
                if (isP) lds_st<bf16x4>(smem, L::PB + 2 * ((16 * i + l16) * L::CP + 16 * j + 4 * q4), f32x4_to_bf16(x));
                else lds_st<f32x4>(smem, L::AB + 4 * ((16 * i + l16) * L::AP + 16 * j + 4 * q4), x);
            }
        } else {
            exact_ap<K, V>(smem, p, ch, c0, len, L::QH + (it & 1) * L::QH_SZ, tid);
        }
        // w v of this chunk, row-major
        {
            const bf16x8 zero = {};
            for (int i = 0; i < RPTV; ++i) {
                const int r = emv.row0 + i;
                const f32x8 wv = bf16x8_to_f32(r < len ? vr[i] : zero) * bf16x8_to_f32(wr[i]);
                lds_st<bf16x8>(smem, L::WV + 2 * (r * L::VP + emv.c0), f32x8_to_bf16(wv));
            }
        }
        __syncthreads();  // ------------------------------------------ B3


        // ---- T2: block column j = rw of T by fp32 MFMA,
        // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, i = j+1..3. T_kj (k > j)
        // stay in registers in the MFMA result layout and feed later
        // products as B operands (k index 4*q4 + e in step e).
        if (rw < 3) {
            const int j = rw;
            f32x4 Tc[4];
            for (int i = 1; i < 4; ++i) {
                if (i <= j) continue;
                f32x4 X = {0, 0, 0, 0};
                for (int st = 0; st < 4; ++st) {  // k = j: T_jj from AB
                    const float a = lds_ld<float>(smem, L::AB + 4 * ((16 * i + l16) * L::AP + 16 * j + 4 * st + q4));
                    const float b = lds_ld<float>(smem, L::AB + 4 * ((16 * j + 4 * st + q4) * L::AP + 16 * j + l16));
                    X = mfma_f32(a, b, X);
                }
                for (int kb = 1; kb < 3; ++kb) {
                    if (kb <= j || kb >= i) continue;
                    for (int e = 0; e < 4; ++e) {
                        const float a = lds_ld<float>(smem, L::AB + 4 * ((16 * i + l16) * L::AP + 16 * kb + 4 * q4 + e));
                        X = mfma_f32(a, Tc[kb][e], X);
                    }
                }
                f32x4 Y = {0, 0, 0, 0};
                for (int e = 0; e < 4; ++e) {
                    const float a = -lds_ld<float>(smem, L::AB + 4 * ((16 * i + l16) * L::AP + 16 * i + 4 * q4 + e));
                    Y = mfma_f32(a, X[e], Y);
                }
                Tc[i] = Y;
                for (int e = 0; e < 4; ++e)
                    lds_st<__bf16>(smem, L::TB + 2 * ((16 * i + 4 * q4 + e) * L::CP + 16 * j + l16), (__bf16)Y[e]);
            }
        }
        __syncthreads();  // ------------------------------------------ B4

        // ---- WY: wy_u = T (w v) for this wave's value columns: U starts here
        for (int jt = 0; jt < NCT; ++jt) {
            bf16x8 bv[2];
            for (int ks = 0; ks < 2; ++ks) {
                const int off = L::WV + 2 * ((32 * ks + 8 * q4 + (l16 >> 2)) * L::VP + vbase + 16 * jt + 4 * (l16 & 3));
                bv[ks] = cat4(lds_tr(smem, off), lds_tr(smem, off + 2 * 4 * L::VP));
            }
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {0, 0, 0, 0};
                for (int ks = 0; ks <= (i >> 1); ++ks) {
                    const bf16x8 a = lds_ld<bf16x8>(smem, L::TB + 2 * ((16 * i + l16) * L::CP + 32 * ks + 8 * q4));
                    acc = mfma_bf16(a, bv[ks], acc);
                }
                U[i][jt] = acc;
            }
        }
        __syncthreads();  // ------------------------------------------ B5
    }

    const int lane = tid & 63, rw = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int vbase = rw * VW;
    if (p.ht)
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e)
                    p.ht[(((int64_t)ch.n * p.HV + ch.hv) * K + 16 * it + 4 * q4 + e) * V + vbase + 16 * jt + l16] =
                        S[it][jt][e];
}

// ------------------------------------------------------------------ kernel --
template <int K, int V>
__global__ __launch_bounds__(NTHR) void chunk_fwd_kernel(FwdParams p)
{
    using L = Lds<K, V>;
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    const int tid = threadIdx.x;

    Chain ch;
    ch.n = blockIdx.x / p.HV;
    ch.hv = blockIdx.x - ch.n * p.HV;
    ch.hk = ch.hv / (p.HV / p.H);
    ch.tb = p.cu ? (int64_t)p.cu[ch.n] : 0;
    ch.te = p.cu ? (int64_t)p.cu[ch.n + 1] : p.T;
    const int nc = (int)((ch.te - ch.tb + CH - 1) / CH);

    // P's blocks above the diagonal stay zero for the whole chain (ordered
    // before any use by the first barrier)
    for (int i = tid; i < CH * L::CP / 2; i += NTHR) lds_st<uint32_t>(smem, L::PB + 4 * i, 0u);
    // T's blocks (0,1) and (2,3), read by the WY products, stay zero too
    if (tid < 128) {
        const int b = tid >> 6, rr = (tid >> 2) & 15, cc = (tid & 3) * 4;
        lds_st<uint64_t>(smem, L::TB + 2 * ((32 * b + rr) * L::CP + 32 * b + 16 + cc), 0ull);
    }

    // a wave-uniform test, so that the two roles are separate branches and
    // not one exec-masked instruction stream (whose wait-counter analysis
    // would mix the roles' outstanding loads)
    if (__builtin_amdgcn_readfirstlane(tid) >= NROLE) key_role<K, V>(smem, p, ch, tid, nc);
    else state_role<K, V>(smem, p, ch, tid, nc);
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
