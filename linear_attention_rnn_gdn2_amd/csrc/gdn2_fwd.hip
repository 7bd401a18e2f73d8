// Fused GDN-2 chunked prefill forward for CDNA4 (gfx950).
//
// One workgroup of 512 threads (8 wave64s) owns one (sequence, value head)
// chain and walks its 64-token chunks in order. The waves have two roles:
//
//   state waves 0-3  hold the K x V float32 state in registers (result layout
//                    of v_mfma_f32_16x16x32_bf16, V split four ways), invert
//                    the four 16x16 diagonal blocks of (I + A) and run the
//                    sequential state pass;
//   key waves 4-7    hold the next chunk's raw inputs in registers (prefetched
//                    while the current chunk is processed), build every decay
//                    factor and MFMA operand, and finish the inverse and the
//                    pseudo-keys.
//
// Per chunk (rows r, s are positions in the chunk; G = inclusive in-chunk
// cumulative sum of the log-decay g per key channel; S = state entering the
// chunk):
//
//   E   cumulative sum of g (in-thread + wave shuffles + LDS exchange), the
//       decay factors and the bf16 operands, written to LDS
//   AP  A_rs = sum_c beta_r k_r exp(G_r - G_s) k_s   (s < r)
//       P_rs = sum_c q_r exp(G_r - G_s) k_s          (s <= r)
//       on MFMA, 16-row tile by tile, each tile factored about its midpoint
//       row m: exp(G_r - G_m) * exp(G_m - G_s). Each factor stays within
//       exp(+-64) while no 8-token half-tile spans more than 64 in log decay;
//       a chunk that breaks this takes an exact path that evaluates
//       exp(G_r - G_s) (exponent <= 0) per pair.
//   T   T = (I + A)^{-1}, float32: diagonal 16x16 blocks by forward
//       substitution, then each block column by fp32 MFMA chains
//       T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.
//   WY  wy_w = T (beta k exp(G)),  wy_u = T (w v)             (bf16 MFMA)
//   S   U = wy_u - wy_w S;  O = scale (q exp(G)) S + scale P U;
//       S <- diag(exp(G_last)) S + (k exp(G_last - G))^T U    (bf16 MFMA)
//
// This is the chunked WY evaluation of the recurrence of the FlashInfer
// chunk_gated_delta_rule2 docs (recurrence display equation). The split into
// decay cumsum, decay-scaled K K^T with the erase gate, unit-lower-triangular
// inverse, w/u recompute and a sequential float32 state pass with intra plus
// inter output follows the FlashRT card ("Usage", 64-token WY chain) and the
// burn-gdn2 README ("Fused CUDA kernels"; "Numerical stability": 16-token
// tiles, tile-local log-space decay, per-tile solve). Rows of a partial last
// chunk are zero-padded (q = k = v = 0, g = 0): exact identity steps.
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

constexpr int CH = 64;                  // chunk length
constexpr int NTHR = 512;               // threads per workgroup (8 waves)
constexpr int NROLE = 256;              // threads per role (4 waves)
constexpr float HALF_SPAN_MAX = 64.0f;  // largest |G_r - G_mid| of the factored path

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

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// (row tile, column tile) of the 10 lower-triangular 16x16 tiles of a 64x64
// matrix, in row order.
__constant__ int8_t kTriI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kTriJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

// ------------------------------------------------------------ LDS layout --
// Byte offsets into one static LDS array. Row pitches carry 16 bytes of
// padding to spread rows over banks.
template <int K, int V>
struct Lds {
    static constexpr int KP = K + 8;   // bf16 elements per [row][K] row
    static constexpr int VP = V + 8;   // bf16 elements per [row][V] row
    static constexpr int CP = CH + 8;  // bf16 elements per [channel][token] row
    static constexpr int AP = CH + 4;  // fp32 elements per A/T row
    static constexpr int GP = K + 4;   // fp32 elements per G row (exact path)
    // Region X, phases E/AP (factored path): MFMA operands of A and P
    static constexpr int LB = 0;                   // beta k exp(G - G_mid(tile))  [64][KP]
    static constexpr int LQ = LB + CH * KP * 2;    // q exp(G - G_mid(tile))       [64][KP]
    static constexpr int RR = LQ + CH * KP * 2;    // k exp(G_mid(tile) - G)       [64][KP]
    static constexpr int X_END = RR + CH * KP * 2;
    static constexpr int GF = 0;                   // exact path: G fp32           [64][GP]
    // Region X, phases T/WY/S
    static constexpr int WYW = 0;                  // -wy_w                        [64][KP]
    static constexpr int TB = WYW + CH * KP * 2;   // T in bf16                    [64][CP]
    static constexpr int OST = TB + CH * CP * 2;   // out tile (phase S -> next E1) [64][VP]
    // Transposed operands, written in phase E, read in phase WY
    static constexpr int KBT = X_END;              // (beta k exp(G))^T            [K][CP]
    static constexpr int WVT = KBT + K * CP * 2;   // (w v)^T                      [V][CP]
    // Persistent buffers
    static constexpr int QH = WVT + V * CP * 2;    // q exp(G)                     [64][KP]
    static constexpr int KHT = QH + CH * KP * 2;   // (k exp(G_last - G))^T        [K][CP]
    static constexpr int AB = KHT + K * CP * 2;    // A, diagonal blocks of T, fp32 [64][AP]
    static constexpr int PB = AB + CH * AP * 4;    // P bf16                       [64][CP]
    static constexpr int GAM = PB + CH * CP * 2;   // exp(G_last) fp32             [K]
    static constexpr int TT = GAM + K * 4;         // tile totals of G             [4][K]
    static constexpr int TM = TT + 4 * K * 4;      // tile midpoints of G          [4][K]
    static constexpr int SD = TM + 4 * K * 4;      // exp(G_mid(i) - G_mid(j)), i > j      [6][K]
    static constexpr int FL = SD + 6 * K * 4;      // per-wave factored-path flags [4]
    static constexpr int TOTAL = FL + 16;
    static_assert(OST + CH * VP * 2 <= X_END, "phase T/WY/S view must fit region X");
    static_assert(GF + CH * GP * 4 <= X_END, "exact-path G must fit region X");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// An opaque zero, produced inside a loop body, keeps LDS address arithmetic
// in that body: without it the compiler hoists dozens of loop-invariant
// addresses out of the chunk loop and pins a register for each.
__device__ __forceinline__ int opaque_zero()
{
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// Phase-E thread map of one role (4 waves over a 64-row x NC-column chunk,
// 8 columns per thread): wave w owns rows [16w, 16w + 16); inside a wave the
// row group varies fastest. Consecutive lanes therefore write consecutive
// rows of row-major arrays and consecutive tokens of [column][token] arrays,
// which keeps both kinds of LDS store free of 8-way bank conflicts.
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

// Slot of the pair (i, j), i > j, in SD.
__device__ __forceinline__ int d_slot(int i, int j) { return i * (i - 1) / 2 + j; }

// Raw inputs of one chunk as loaded from HBM (bf16 kept packed), in the key
// waves' thread map: rows row0 + i, channels c0k .. c0k + 7 (key side) and
// rows row0v + i, columns c0v .. c0v + 7 (value side). Rows past the end of
// the sequence are zero.
template <int RPT>
struct RawChunk {
    bf16x8 q[RPT], k[RPT], b[RPT];
    f32x4 g[RPT][2];
};

// Stand-ins for omitted gates: one row of ones (beta, w) or zeros (g), read
// with row stride 0.
__constant__ __attribute__((aligned(16))) uint16_t kOnesBf16[8] = {0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                                                 0x3f80, 0x3f80, 0x3f80, 0x3f80};
__constant__ __attribute__((aligned(16))) float kZerosF32[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// Straight-line loads: rows past the chunk end read the last valid row and
// are zeroed afterwards; omitted gates read the stand-in row.
template <int K, int RPT>
__device__ __forceinline__ void load_decay(RawChunk<RPT> &R, const FwdParams &p, int64_t c0, int len, int hv,
                                           int row0, int c0k)
{
    const float *gb = p.g ? p.g + (c0 * p.HV + hv) * K : kZerosF32;
    const int sg = p.g ? p.HV * K : 0, cgg = p.g ? c0k : 0;
    for (int i = 0; i < RPT; ++i) {
        const int r = row0 + i;
        const int rc = r < len ? r : len - 1;
        const bool ok = r < len;
        const f32x4 g0 = ldg_f32x4(gb + (uint32_t)(rc * sg + cgg));
        const f32x4 g1 = ldg_f32x4(gb + (uint32_t)(rc * sg + cgg) + 4);
        R.g[i][0] = ok ? g0 : f32x4{0, 0, 0, 0};
        R.g[i][1] = ok ? g1 : f32x4{0, 0, 0, 0};
    }
}

template <int K, int RPT>
__device__ __forceinline__ void load_keys(RawChunk<RPT> &R, const FwdParams &p, int64_t c0, int len, int hk,
                                          int hv, int row0, int c0k)
{
    const bf16x8 zero = {};
    // wave-uniform chunk bases + 32-bit per-lane offsets
    const uint16_t *qb = p.q + (c0 * p.H + hk) * K;
    const uint16_t *kb = p.k + (c0 * p.H + hk) * K;
    const uint16_t *bb = p.beta ? p.beta + (c0 * p.HV + hv) * K : kOnesBf16;
    const int sqk = p.H * K, sb = p.beta ? p.HV * K : 0, cb = p.beta ? c0k : 0;
    for (int i = 0; i < RPT; ++i) {
        const int r = row0 + i;
        const int rc = r < len ? r : len - 1;
        const bool ok = r < len;
        const bf16x8 q = ldg_bf16x8(qb + (uint32_t)(rc * sqk + c0k));
        const bf16x8 k = ldg_bf16x8(kb + (uint32_t)(rc * sqk + c0k));
        R.q[i] = ok ? q : zero;
        R.k[i] = ok ? k : zero;
        R.b[i] = ldg_bf16x8(bb + (uint32_t)(rc * sb + cb));
    }
}

// Value-side rows of one chunk (state waves): v and w, rows row0 + i,
// columns c0 .. c0 + 7; rows past the end are zero.
template <int V, int RPTV>
__device__ __forceinline__ void load_values(bf16x8 *v, bf16x8 *w, const FwdParams &p, int64_t c0, int len, int hv,
                                            int row0, int c0v)
{
    const bf16x8 zero = {};
    const uint16_t *vb = p.v + (c0 * p.HV + hv) * V;
    const uint16_t *wb = p.w ? p.w + (c0 * p.HV + hv) * V : kOnesBf16;
    const int svw = p.HV * V, sw = p.w ? svw : 0, cw = p.w ? c0v : 0;
    for (int i = 0; i < RPTV; ++i) {
        const int r = row0 + i;
        const int rc = r < len ? r : len - 1;
        const bf16x8 x = ldg_bf16x8(vb + (uint32_t)(rc * svw + c0v));
        v[i] = r < len ? x : zero;
        w[i] = ldg_bf16x8(wb + (uint32_t)(rc * sw + cw));
    }
}

// Store RPT rows x 8 channels (bf16, one vector per row) transposed into a
// [channel][token] array: channel c0 + j gets the RPT consecutive tokens
// row0 .. row0 + RPT - 1. The 16-bit transposition is done with byte
// permutes on packed pairs, so nothing is unpacked into separate registers.
template <int RPT>
__device__ __forceinline__ void st_transposed(char *smem, int base, int pitch, int c0, int row0, const bf16x8 *rows)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;  // low / high halves of (b, a)
    u32x4 w[RPT];
    for (int i = 0; i < RPT; ++i) w[i] = __builtin_bit_cast(u32x4, rows[i]);
    for (int m = 0; m < 4; ++m) {
        if constexpr (RPT == 4) {
            const uint2 e = {__builtin_amdgcn_perm(w[1][m], w[0][m], LO), __builtin_amdgcn_perm(w[3][m], w[2][m], LO)};
            const uint2 o = {__builtin_amdgcn_perm(w[1][m], w[0][m], HI), __builtin_amdgcn_perm(w[3][m], w[2][m], HI)};
            lds_st<uint2>(smem, base + 2 * ((c0 + 2 * m) * pitch + row0), e);
            lds_st<uint2>(smem, base + 2 * ((c0 + 2 * m + 1) * pitch + row0), o);
        } else {
            static_assert(RPT == 2, "2 or 4 rows per thread");
            lds_st<uint32_t>(smem, base + 2 * ((c0 + 2 * m) * pitch + row0), __builtin_amdgcn_perm(w[1][m], w[0][m], LO));
            lds_st<uint32_t>(smem, base + 2 * ((c0 + 2 * m + 1) * pitch + row0), __builtin_amdgcn_perm(w[1][m], w[0][m], HI));
        }
    }
}

// ----------------------------------------------------------- chain context --
struct Chain {
    int n, hv, hk;
    int64_t tb, te;  // token range of the chain's sequence
};

__device__ __forceinline__ int chunk_len(int64_t c0, int64_t te) { return (int)((te - c0) < CH ? (te - c0) : CH); }

__device__ __forceinline__ bool read_fast_flag(const char *smem, int fl)
{
    return lds_ld<int>(smem, fl) & lds_ld<int>(smem, fl + 4) & lds_ld<int>(smem, fl + 8) & lds_ld<int>(smem, fl + 12);
}

// ------------------------------------------------------- phase AP (shared) --
// Fills A (fp32, strictly lower) and P (bf16, lower with diagonal) for the
// chunk. Factored path: 20 MFMA tiles spread over the 8 waves. Exact path:
// thread (r, eight columns s) evaluates exp(G_r - G_s) per channel.
template <int K, int V>
__device__ __forceinline__ void phase_ap(char *smem, const FwdParams &p, const Chain &ch, int64_t c0, int len,
                                        bool fast, int tid)
{
    using L = Lds<K, V>;
    constexpr int NKS = K / 32;
    const int lane = tid & 63, wv = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
    if (fast) {
        for (int tt = wv; tt < 20; tt += 8) {
            const bool isP = tt >= 10;
            const int t10 = isP ? tt - 10 : tt;
            const int i = kTriI[t10], j = kTriJ[t10];
            const int mb = isP ? L::LQ : L::LB;
            // column operand of tile (i, j): k_s exp(G_mid(j) - G_s), times
            // exp(G_mid(i) - G_mid(j)) <= 1 per channel when j < i
            f32x4 acc = {0, 0, 0, 0};
            for (int ks = 0; ks < NKS; ++ks) {
                const int ch8 = 32 * ks + 8 * q4;
                const bf16x8 a = lds_ld<bf16x8>(smem, mb + 2 * ((16 * i + l16) * L::KP + ch8));
                bf16x8 b = lds_ld<bf16x8>(smem, L::RR + 2 * ((16 * j + l16) * L::KP + ch8));
                if (j < i) {
                    const int ds = L::SD + 4 * (d_slot(i, j) * K + ch8);
                    const f32x4 d0 = lds_ld<f32x4>(smem, ds), d1 = lds_ld<f32x4>(smem, ds + 16);
                    const f32x8 dd = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
                    b = f32x8_to_bf16(bf16x8_to_f32(b) * dd);
                }
                acc = mfma_bf16(a, b, acc);
            }
            const int s = 16 * j + l16;
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * i + 4 * q4 + e;
                if (!isP) lds_st<float>(smem, L::AB + 4 * (r * L::AP + s), s < r ? acc[e] : 0.0f);
                else lds_st<__bf16>(smem, L::PB + 2 * (r * L::CP + s), (__bf16)(s <= r ? acc[e] : 0.0f));
            }
        }
    } else {
        const int r = tid >> 3, s0 = (tid & 7) * 8;
        const int64_t tr = c0 + r;
#pragma unroll 1
        for (int x = 0; x < 8; ++x) {
            const int s = s0 + x;
            float aA = 0.0f, aP = 0.0f;
            if (s <= r && r < len) {
#pragma unroll 1
                for (int c8 = 0; c8 < K / 8; ++c8) {
                    const f32x8 qr = bf16x8_to_f32(ldg_bf16x8(p.q + (tr * p.H + ch.hk) * K + 8 * c8));
                    const f32x8 kr = bf16x8_to_f32(ldg_bf16x8(p.k + (tr * p.H + ch.hk) * K + 8 * c8));
                    f32x8 br = {1, 1, 1, 1, 1, 1, 1, 1};
                    if (p.beta) br = bf16x8_to_f32(ldg_bf16x8(p.beta + (tr * p.HV + ch.hv) * K + 8 * c8));
                    const f32x8 ks = bf16x8_to_f32(ldg_bf16x8(p.k + ((c0 + s) * p.H + ch.hk) * K + 8 * c8));
                    const f32x4 gr0 = lds_ld<f32x4>(smem, L::GF + 4 * (r * L::GP + 8 * c8));
                    const f32x4 gr1 = lds_ld<f32x4>(smem, L::GF + 4 * (r * L::GP + 8 * c8 + 4));
                    const f32x4 gs0 = lds_ld<f32x4>(smem, L::GF + 4 * (s * L::GP + 8 * c8));
                    const f32x4 gs1 = lds_ld<f32x4>(smem, L::GF + 4 * (s * L::GP + 8 * c8 + 4));
                    for (int j = 0; j < 8; ++j) {
                        const float gr = j < 4 ? gr0[j] : gr1[j - 4];
                        const float gs = j < 4 ? gs0[j] : gs1[j - 4];
                        const float ex = __expf(gr - gs) * ks[j];
                        aA += br[j] * kr[j] * ex;
                        aP += qr[j] * ex;
                    }
                }
            }
            lds_st<float>(smem, L::AB + 4 * (r * L::AP + s), s < r ? aA : 0.0f);
            lds_st<__bf16>(smem, L::PB + 2 * (r * L::CP + s), (__bf16)(s <= r ? aP : 0.0f));
        }
    }
}

// ------------------------------------------------------------- key waves --
// Barrier sequence per chunk (must match state_role): B1 .. B7.
template <int K, int V>
__device__ __forceinline__ void key_role(char *smem, const FwdParams &p, const Chain &ch, int tid)
{
    using L = Lds<K, V>;
    constexpr int CGK = K / 8;              // 8-channel groups along K
    constexpr int RPT = CH * CGK / NROLE;   // rows per thread
    constexpr int RGW = 64 / CGK;           // row groups per wave
    constexpr int NCTK = K / 64;            // -wy_w column tiles per key wave
    static_assert(RPT * RGW == 16, "a key wave covers one 16-row tile");

    RawChunk<RPT> R;
    if (ch.tb < ch.te) {
        const int rt = tid & (NROLE - 1);
        const EMap<K> em(rt);
        load_decay<K, RPT>(R, p, ch.tb, chunk_len(ch.tb, ch.te), ch.hv, em.row0, em.c0);
        load_keys<K, RPT>(R, p, ch.tb, chunk_len(ch.tb, ch.te), ch.hk, ch.hv, em.row0, em.c0);
    }

    char *const smem0 = smem;
    const int tid0 = tid;
    for (int64_t c0 = ch.tb; c0 < ch.te; c0 += CH) {
        // lane-derived values are recomputed per chunk (see opaque_zero)
        const int z = opaque_zero();
        char *smem = smem0 + z;
        const int tid = tid0 + z;
        const int lane = tid & 63, rw = (tid >> 6) & 3, rt = tid & (NROLE - 1);
        const int l16 = lane & 15, q4 = lane >> 4;
        const EMap<K> em(rt);
        const int cg = em.cg, row0 = em.row0, c0k = em.c0, rgl = em.rgl;
        const int len = chunk_len(c0, ch.te);

        // ---- E1: tile-local cumulative log decay, tile totals/midpoints
        float G[RPT][8], gmid[8];
        for (int i = 0; i < RPT; ++i)
            for (int j = 0; j < 8; ++j)
                G[i][j] = (i ? G[i - 1][j] : 0.0f) + (j < 4 ? R.g[i][0][j] : R.g[i][1][j - 4]);
        // inclusive scan of the row-group totals across the RGW lanes of a
        // column group (consecutive lanes)
        for (int j = 0; j < 8; ++j) {
            const float tot = G[RPT - 1][j];
            float inc = tot;
            if constexpr (RGW == 4) {  // quads: DPP row shifts by 1 and 2 lanes
                const float o1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(inc), 0x111, 0xf, 0xf, false));
                if (rgl >= 1) inc += o1;
                const float o2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(inc), 0x112, 0xf, 0xf, false));
                if (rgl >= 2) inc += o2;
            } else {
                for (int d = 1; d < RGW; d <<= 1) {
                    const float o = __shfl_up(inc, d, 64);
                    if (rgl >= d) inc += o;
                }
            }
            const float excl = inc - tot;
            for (int i = 0; i < RPT; ++i) G[i][j] += excl;
        }
        // tile midpoint (local row 7) from the lane that holds it
        bool fast_ok = true;
        for (int j = 0; j < 8; ++j) {
            if constexpr (RGW == 4) {  // quad broadcast of lane 1 (rows 4..7)
                static_assert(7 / RPT == 1, "row 7 sits in the quad's lane 1");
                gmid[j] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(G[7 % RPT][j]), 0x55, 0xf, 0xf, false));
            } else {
                gmid[j] = __shfl(G[7 % RPT][j], cg * RGW + 7 / RPT, 64);
            }
            for (int i = 0; i < RPT; ++i) fast_ok &= fabsf(G[i][j] - gmid[j]) <= HALF_SPAN_MAX;
        }
        const int wave_ok = __all(fast_ok);
        if (rgl == RGW - 1) {
            lds_st<f32x4>(smem, L::TT + 4 * (rw * K + c0k), f32x4{G[RPT - 1][0], G[RPT - 1][1], G[RPT - 1][2], G[RPT - 1][3]});
            lds_st<f32x4>(smem, L::TT + 4 * (rw * K + c0k + 4), f32x4{G[RPT - 1][4], G[RPT - 1][5], G[RPT - 1][6], G[RPT - 1][7]});
        }
        if (rgl == 7 / RPT) {
            lds_st<f32x4>(smem, L::TM + 4 * (rw * K + c0k), f32x4{gmid[0], gmid[1], gmid[2], gmid[3]});
            lds_st<f32x4>(smem, L::TM + 4 * (rw * K + c0k + 4), f32x4{gmid[4], gmid[5], gmid[6], gmid[7]});
        }
        if (lane == 0) lds_st<int>(smem, L::FL + 4 * rw, wave_ok);
        __syncthreads();  // ------------------------------------------ B1
        const bool fast = read_fast_flag(smem, L::FL);

        // ---- E3: decay factors and operands. Rows are handled in pairs so
        // that only two rows of the transposed operands are held at once.
        // chunk-relative references of this wave's tile: base (start),
        // glast (end of chunk); G_mid = base + gmid
        float eGm[8], eKm[8], base[8], glast[8];
        for (int j = 0; j < 8; ++j) {
            float acc = 0.0f;
            base[j] = 0.0f;
            for (int t = 0; t < 4; ++t) {
                if (t == rw) base[j] = acc;
                acc += lds_ld<float>(smem, L::TT + 4 * (t * K + c0k + j));
            }
            glast[j] = acc;
        }
        if (fast)
            for (int j = 0; j < 8; ++j) {
                eGm[j] = __expf(base[j] + gmid[j]);
                eKm[j] = __expf(glast[j] - base[j] - gmid[j]);
            }
        for (int pr = 0; pr < RPT; pr += 2) {
            bf16x8 kbg_rows[2], kh_rows[2];  // beta k exp(G); k exp(G_last - G)
            for (int i2 = 0; i2 < 2; ++i2) {
                const int i = pr + i2;
                const int r = row0 + i;
                const f32x8 qf = bf16x8_to_f32(R.q[i]), kf = bf16x8_to_f32(R.k[i]);
                const f32x8 bk = bf16x8_to_f32(R.b[i]) * kf;
                if (fast) {
                    f32x8 lb, lq, qh, kb, kh, rk;
                    for (int j = 0; j < 8; ++j) {
                        const float x = G[i][j] - gmid[j];
                        const float f = __expf(x), rf = __expf(-x);
                        lb[j] = bk[j] * f;
                        lq[j] = qf[j] * f;
                        qh[j] = qf[j] * (eGm[j] * f);
                        kb[j] = bk[j] * (eGm[j] * f);
                        kh[j] = kf[j] * (eKm[j] * rf);
                        rk[j] = kf[j] * rf;
                    }
                    lds_st<bf16x8>(smem, L::LB + 2 * (r * L::KP + c0k), f32x8_to_bf16(lb));
                    lds_st<bf16x8>(smem, L::LQ + 2 * (r * L::KP + c0k), f32x8_to_bf16(lq));
                    lds_st<bf16x8>(smem, L::QH + 2 * (r * L::KP + c0k), f32x8_to_bf16(qh));
                    lds_st<bf16x8>(smem, L::RR + 2 * (r * L::KP + c0k), f32x8_to_bf16(rk));
                    kbg_rows[i2] = f32x8_to_bf16(kb);
                    kh_rows[i2] = f32x8_to_bf16(kh);
                } else {
                    f32x8 qh, kb, kh, ga;
                    for (int j = 0; j < 8; ++j) {
                        ga[j] = base[j] + G[i][j];
                        const float eg = __expf(ga[j]), ek = __expf(glast[j] - ga[j]);
                        qh[j] = qf[j] * eg;
                        kb[j] = bk[j] * eg;
                        kh[j] = kf[j] * ek;
                    }
                    lds_st<f32x4>(smem, L::GF + 4 * (r * L::GP + c0k), f32x4{ga[0], ga[1], ga[2], ga[3]});
                    lds_st<f32x4>(smem, L::GF + 4 * (r * L::GP + c0k + 4), f32x4{ga[4], ga[5], ga[6], ga[7]});
                    lds_st<bf16x8>(smem, L::QH + 2 * (r * L::KP + c0k), f32x8_to_bf16(qh));
                    kbg_rows[i2] = f32x8_to_bf16(kb);
                    kh_rows[i2] = f32x8_to_bf16(kh);
                }
            }
            st_transposed<2>(smem, L::KHT, L::CP, c0k, row0 + pr, kh_rows);
            st_transposed<2>(smem, L::KBT, L::CP, c0k, row0 + pr, kbg_rows);
        }
        __syncthreads();  // ------------------------------------------ B2

        phase_ap<K, V>(smem, p, ch, c0, len, fast, tid);
        __syncthreads();  // ------------------------------------------ B3

        __syncthreads();  // ------------------------------------------ B4

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
                for (int st = 0; st < 4; ++st) {  // k = j: T_jj from LDS
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
        __syncthreads();  // ------------------------------------------ B5

        // ---- WY: -wy_w = -T (beta k exp(G)) for this wave's column tiles
        for (int jt = 0; jt < NCTK; ++jt) {
            const int cb = 16 * (rw * NCTK + jt);
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {0, 0, 0, 0};
                for (int ks = 0; ks <= (i >> 1); ++ks) {
                    const bf16x8 a = lds_ld<bf16x8>(smem, L::TB + 2 * ((16 * i + l16) * L::CP + 32 * ks + 8 * q4));
                    const bf16x8 b = lds_ld<bf16x8>(smem, L::KBT + 2 * ((cb + l16) * L::CP + 32 * ks + 8 * q4));
                    acc = mfma_bf16(a, b, acc);
                }
                for (int e = 0; e < 4; ++e)
                    lds_st<__bf16>(smem, L::WYW + 2 * ((16 * i + 4 * q4 + e) * L::KP + cb + l16), (__bf16)(-acc[e]));
            }
        }
        __syncthreads();  // ------------------------------------------ B6
        // Prefetch the next chunk while the state waves run phase S: every
        // workgroup issues its loads at about the same time, so the issue
        // stalls until HBM drains them; here that stall overlaps phase S.
        // Nothing else is outstanding, so no later register reload waits on
        // these loads (vector-memory operations complete in order).
        if (c0 + CH < ch.te) {
            load_decay<K, RPT>(R, p, c0 + CH, chunk_len(c0 + CH, ch.te), ch.hv, row0, c0k);
            load_keys<K, RPT>(R, p, c0 + CH, chunk_len(c0 + CH, ch.te), ch.hk, ch.hv, row0, c0k);
        }
        __syncthreads();  // ------------------------------------------ B7
    }
}

// ----------------------------------------------------------- state waves --
template <int K, int V>
__device__ __forceinline__ void state_role(char *smem, const FwdParams &p, const Chain &ch, int tid)
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
    } else {
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt) S[it][jt] = f32x4{0, 0, 0, 0};
    }
    }

    char *const smem0 = smem;
    const int tid0 = tid;
    for (int64_t c0 = ch.tb; c0 < ch.te; c0 += CH) {
        const int z = opaque_zero();
        char *smem = smem0 + z;
        const int tid = tid0 + z;
        const int lane = tid & 63, rw = tid >> 6, rt = tid;
        const int l16 = lane & 15, q4 = lane >> 4;
        const int vbase = rw * VW;
        const int len = chunk_len(c0, ch.te);
        // this chunk's v and w rows (consumed after phase E, so the load
        // latency is hidden behind it)
        const EMap<V> emv(rt);
        const int row0v = emv.row0, c0v = emv.c0;
        bf16x8 vr[RPTV], wr[RPTV];
        load_values<V, RPTV>(vr, wr, p, c0, len, ch.hv, row0v, c0v);
        // store the previous chunk's staged output (a full chunk: only the
        // sequence's last chunk can be partial)
        if (c0 > ch.tb)
            for (int idx = rt; idx < CH * CGV; idx += NROLE) {
                const int r = idx / CGV, c8 = idx % CGV;
                *reinterpret_cast<bf16x8 *>(p.out + ((c0 - CH + r) * p.HV + ch.hv) * V + 8 * c8) =
                    lds_ld<bf16x8>(smem, L::OST + 2 * (r * L::VP + 8 * c8));
            }
        __syncthreads();  // ------------------------------------------ B1
        const bool fast = read_fast_flag(smem, L::FL);
        // ---- E2 (overlaps the key waves' phase E3): cross-tile factors
        // exp(G_mid(i) - G_mid(j)), i > j, for phase AP, and exp(G_last)
        for (int pc = rt; pc < 4 * K; pc += NROLE) {
            const int i = pc / K, c = pc % K;
            float gm[4], acc = 0.0f;
            for (int t = 0; t < 4; ++t) {
                gm[t] = acc + lds_ld<float>(smem, L::TM + 4 * (t * K + c));
                acc += lds_ld<float>(smem, L::TT + 4 * (t * K + c));
            }
            float gmi = gm[0];
            for (int t = 1; t < 4; ++t) gmi = i == t ? gm[t] : gmi;
            if (fast)
                for (int t = 0; t < 3; ++t)
                    if (t < i) lds_st<float>(smem, L::SD + 4 * (d_slot(i, t) * K + c), __expf(gmi - gm[t]));
            if (i == 0) lds_st<float>(smem, L::GAM + 4 * c, __expf(acc));
        }
        {
            // (w v)^T: column c0v + j, tokens row0v ..
            bf16x8 wvb[RPTV];
            for (int i = 0; i < RPTV; ++i) wvb[i] = f32x8_to_bf16(bf16x8_to_f32(vr[i]) * bf16x8_to_f32(wr[i]));
            st_transposed<RPTV>(smem, L::WVT, L::CP, c0v, row0v, wvb);
        }
        __syncthreads();  // ------------------------------------------ B2

        phase_ap<K, V>(smem, p, ch, c0, len, fast, tid);
        __syncthreads();  // ------------------------------------------ B3

        // ---- T1: diagonal block rw of T by forward substitution. Lane l16
        // builds column l16 of T_ii; row r of A_ii is read from LDS as a
        // broadcast (every lane reads the same address).
        {
            const int d0 = 16 * rw;
            // the whole strictly-lower triangle first (one wait), then a pure
            // FMA chain
            float a[16][16];
            for (int r = 1; r < 16; ++r)
                for (int s4 = 0; s4 < r; s4 += 4) {
                    const f32x4 x = lds_ld<f32x4>(smem, L::AB + 4 * ((d0 + r) * L::AP + d0 + s4));
                    for (int e = 0; e < 4; ++e) a[r][s4 + e] = x[e];
                }
            float tc[16];
            tc[0] = l16 == 0 ? 1.0f : 0.0f;
            for (int r = 1; r < 16; ++r) {
                float acc0 = 0.0f, acc1 = 0.0f;
                for (int s2 = 0; s2 < r; ++s2) {
                    if (s2 & 1) acc1 += a[r][s2] * tc[s2];
                    else acc0 += a[r][s2] * tc[s2];
                }
                tc[r] = r == l16 ? 1.0f : (r > l16 ? -(acc0 + acc1) : 0.0f);
            }
            if (lane < 16)
                for (int r = 0; r < 16; ++r) {
                    lds_st<float>(smem, L::AB + 4 * ((d0 + r) * L::AP + d0 + l16), tc[r]);
                    lds_st<__bf16>(smem, L::TB + 2 * ((d0 + r) * L::CP + d0 + l16), (__bf16)tc[r]);
                }
            // wy_w and wy_u read T's blocks (0,1) and (2,3): keep them zero
            if (rw == 0 || rw == 2) {
                const int rr = lane >> 2, cc = (lane & 3) * 4;
                lds_st<uint64_t>(smem, L::TB + 2 * ((d0 + rr) * L::CP + d0 + 16 + cc), 0ull);
            }
        }
        __syncthreads();  // ------------------------------------------ B4
        __syncthreads();  // ------------------------------------------ B5

        // ---- WY: wy_u = T (w v) for this wave's value columns: U starts here
        f32x4 U[4][NCT];
        for (int jt = 0; jt < NCT; ++jt)
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {0, 0, 0, 0};
                for (int ks = 0; ks <= (i >> 1); ++ks) {
                    const bf16x8 a = lds_ld<bf16x8>(smem, L::TB + 2 * ((16 * i + l16) * L::CP + 32 * ks + 8 * q4));
                    const bf16x8 b = lds_ld<bf16x8>(smem, L::WVT + 2 * ((vbase + 16 * jt + l16) * L::CP + 32 * ks + 8 * q4));
                    acc = mfma_bf16(a, b, acc);
                }
                U[i][jt] = acc;
            }
        __syncthreads();  // ------------------------------------------ B6

        // ---- S: S as bf16 B operands: k slab ks holds state rows
        // {32ks + 4q4 + e} then {32ks + 16 + 4q4 + e}, e = 0..3; the A
        // operands are read with the same column order.
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
                    U[i][jt] = mfma_bf16(aw, Sb[ks][jt], U[i][jt]);
                    Y[i][jt] = mfma_bf16(aq, Sb[ks][jt], Y[i][jt]);
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
                for (int jt = 0; jt < NCT; ++jt) Y[i][jt] = mfma_bf16(ap, Ub[ks][jt], Y[i][jt]);
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
                s = mfma_bf16(ak[0], Ub[0][jt], s);
                s = mfma_bf16(ak[1], Ub[1][jt], s);
                S[it][jt] = s;
            }
        }
        // stage the output tile; it is stored at the start of the next chunk
        for (int i = 0; i < 4; ++i)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e)
                    lds_st<__bf16>(smem, L::OST + 2 * ((16 * i + 4 * q4 + e) * L::VP + vbase + 16 * jt + l16),
                                   (__bf16)(p.scale * Y[i][jt][e]));
        __syncthreads();  // ------------------------------------------ B7
    }

    const int rt = tid, lane = tid & 63, rw = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int vbase = rw * VW;
    if (ch.tb < ch.te) {
        // store the last chunk's staged output (rows < its length)
        const int64_t last = ch.tb + ((ch.te - ch.tb - 1) / CH) * CH;
        const int len = (int)(ch.te - last);
        for (int idx = rt; idx < CH * CGV; idx += NROLE) {
            const int r = idx / CGV, c8 = idx % CGV;
            if (r < len)
                *reinterpret_cast<bf16x8 *>(p.out + ((last + r) * p.HV + ch.hv) * V + 8 * c8) =
                    lds_ld<bf16x8>(smem, L::OST + 2 * (r * L::VP + 8 * c8));
        }
    }
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

    // P's blocks above the diagonal stay zero for the whole chain (ordered
    // before any use by the first barrier)
    for (int i = tid; i < CH * L::CP / 2; i += NTHR) lds_st<uint32_t>(smem, L::PB + 4 * i, 0u);

    if (tid >= NROLE) key_role<K, V>(smem, p, ch, tid);
    else state_role<K, V>(smem, p, ch, tid);
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
