// Fused GDN-2 chunked prefill forward for CDNA4 (gfx950).
//
// One workgroup of 512 threads (8 wave64s) owns one (sequence, value head)
// chain and walks its 64-token chunks in order. The waves have two roles:
//
//   state waves 0-3  hold the K x V float32 state in registers (result layout
//                    of v_mfma_f32_16x16x32_bf16, V split four ways), build
//                    the off-diagonal A/P tiles and T's off-diagonal blocks,
//                    and run the sequential state pass;
//   key waves 4-7    hold the next chunk's raw q, k, beta, g in registers
//                    (prefetched; key wave w owns K/4 channels over all 64
//                    rows), build the decay factors and MFMA operands, A's
//                    diagonal tiles with their inverses, and the pseudo-keys.
//
// Per chunk (rows r, s are positions in the chunk; G = inclusive in-chunk
// cumulative sum of the log-decay g per key channel, kept in log2 units;
// S = state entering the chunk):
//
//   E   cumulative sum of g over the chunk inside each key wave (in-thread,
//       DPP row scans, permlane row swaps), then the operands
//       KB = beta k 2^G,  QH = q 2^G,  RR = k 2^-G,  KT = k 2^(G_last - G)
//       (bf16, row-major in LDS)
//   AP  A_rs = sum_c KB_rc RR_sc   (s < r),   P_rs = sum_c QH_rc RR_sc  (s <= r)
//       on MFMA. 2^G_r 2^-G_s is exp(G_r - G_s) with one reference per
//       chunk; it is used for every channel whose |G| stays within 2^120.
//       Channels beyond that (extreme decay) get RR = 0 and their share of
//       A and P is added by an exact per-pair evaluation of exp(G_r - G_s).
//   T   T = (I + A)^{-1} in float32: diagonal 16x16 blocks by forward
//       substitution, then the block columns
//       T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj by MFMA on float32 values
//       split into high and low bf16 parts.
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

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {
namespace {

using namespace dev;

constexpr int NTHR = 512;    // threads per workgroup (8 waves)
constexpr int NROLE = 256;   // threads per role (4 waves)
constexpr float LOG2E = 1.44269504088896340736f;
// Largest |G| (log2 units) of the single-reference factorisation: 2^120 and
// 2^-120 are normal in float32 and bf16, and so is every product used.
constexpr float XLIM = 120.0f;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------- helpers --
// Element type of q, k, v, beta, w and out: bf16 (IO_BF16) or fp16 (IO_F16).
// Values are widened to float32 on load; the MFMA operands built from them
// are bf16 either way.
template <int IO>
struct IoT;
template <>
struct IoT<IO_BF16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
};
template <>
struct IoT<IO_F16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
};
template <int IO>
__device__ __forceinline__ float io_bits_to_f32(uint16_t b)
{
    if constexpr (IO == IO_F16) return (float)__builtin_bit_cast(_Float16, b);
    else return bf16_bits_to_f32(b);
}
template <typename T8>
__device__ __forceinline__ f32x8 to_f32x8(T8 x) { return __builtin_convertvector(x, f32x8); }
// The 16 bits of element j of a vector of eight 16-bit values, taken from
// its 32-bit words (extracting a 16-bit float element and bit-casting it,
// inside an unrolled loop, was compiled to the same element for every j).
template <typename T8>
__device__ __forceinline__ uint16_t bits16(T8 x, int j)
{
    const i32x4 w = __builtin_bit_cast(i32x4, x);
    return (uint16_t)((uint32_t)w[j >> 1] >> (16 * (j & 1)));
}

// A float32 4-vector as the sum of two bf16 4-vectors (high part rounded to
// nearest even, low part the rounded remainder).
struct Split4 {
    bf16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4(f32x4 x)
{
    Split4 r;
    r.hi = __builtin_convertvector(x, bf16x4);
    r.lo = __builtin_convertvector(x - __builtin_convertvector(r.hi, f32x4), bf16x4);
    return r;
}
// c + a b for float32 operands given as hi + lo bf16 parts: lo hi + hi lo +
// hi hi on v_mfma_f32_16x16x16_bf16, as two independent chains.
__device__ __forceinline__ f32x4 mfma3(Split4 a, Split4 b, f32x4 c)
{
    f32x4 d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, f32x4{0, 0, 0, 0}, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, c, 0, 0, 0);  // independent of d
    d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, d, 0, 0, 0);
    return c + d;
}

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
// the key waves so that each can invert its block at once; the state waves
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
    static constexpr int NXB = K == 128 ? 16 : 8;  // exact channels per batch (scalar path)
    // flagged channels on MFMA: slots per key wave, slots, bf16 pitch of an
    // operand row of XNS slots (bank-spread)
    static constexpr int XSW = K == 128 ? 8 : 4;
    static constexpr int XNS = 4 * XSW;
    static constexpr int XP = XNS + 4;

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
    static constexpr int XF = GAM + K * 4;                         // exact-channel flags [K] int
    static constexpr int XL = XF + K * 4;                          // exact-channel list  [K] int
    static constexpr int FL = XL + K * 4;                          // per key wave: any exact channel [4] int
    static constexpr int XN = FL + 16;                             // exact-channel count int
    static constexpr int XC = XN + 16;                             // per key wave: flagged-channel count [4] int
    static constexpr int NP = XC + 16;                             // q/k L2 norms: per key wave partial sums of squares [4][64] (q, k) fp32
    static constexpr int NRM = NP + 4 * CH * 8;                    // q/k L2 norms: reciprocal norms [64] (q, k) fp32  E -> exact AP
    static constexpr int XQ = NRM + CH * 8;                        // flagged channels: raw q, k, beta [3][XNS][64] io  E -> B2x
    static constexpr int TOTAL = XQ + 3 * XNS * CH * 2;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    // flagged channels on MFMA: staged G [XNS][64] fp32 in TB, row-side
    // operands (224 rows) in the QH buffer of the other parity, column-side
    // operands (160 rows) in WV
    static_assert(XNS * CH * 4 <= CH * CP * 2, "staged G in TB");
    static_assert(224 * XP * 2 <= QH_SZ, "row-side operands in a QH buffer");
    static_assert(160 * XP * 2 <= WV_SZ, "column-side operands in WV");
};

// Value-side thread map of the state waves (4 waves over a 64-row x
// NC-column chunk, 8 columns per thread): wave w owns rows [16w, 16w + 16);
// inside a wave the row group varies fastest, so that consecutive lanes
// write consecutive rows.
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
template <int RPT, int IO>
struct RawChunk {
    typename IoT<IO>::v8 q[RPT], k[RPT], b[RPT];
    f32x4 g[RPT][2];  // float32 g: 8 values; 16-bit g: the 8 values in g[i][0]
};

// Chunk loads are buffer loads: a scalar resource per (chunk, tensor) whose
// base is the chunk's first row of this head and whose range ends at the
// sequence's last row, plus 32-bit per-lane byte offsets. Rows past the end
// of the sequence read as zero in hardware (q = k = v = 0, g = 0: identity
// steps), so the consumers need no row masks. An omitted gate reads a
// 16-byte row of ones with row stride 0 (beta, w = 1; on padded rows k and v
// are zero); an omitted g, or values taken as zero, is a resource of length
// zero.
__device__ __attribute__((aligned(16))) uint16_t kOnes16[2][8] = {
    {0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80},   // bf16 1.0
    {0x3c00, 0x3c00, 0x3c00, 0x3c00, 0x3c00, 0x3c00, 0x3c00, 0x3c00}};  // fp16 1.0

template <int K, int RPT, int IO, bool G16>
__device__ __forceinline__ void load_decay(RawChunk<RPT, IO> &R, const FwdParams &p, int64_t c0, int len, int hv,
                                           int row0, int c0k)
{
    constexpr int ES = G16 ? 2 : 4;  // bytes per g element
    const int rs = (int)p.sg * ES;  // token stride (bytes)
    const char *gb = static_cast<const char *>(p.g);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gb ? gb + (c0 * p.sg + hv * p.hsg) * ES : nullptr, gb ? len * rs : 0);
    for (int i = 0; i < RPT; ++i) {
        const uint32_t o = (uint32_t)((row0 + i) * rs + ES * c0k);
        R.g[i][0] = buf_ld16<f32x4>(rg, o);
        if constexpr (!G16) R.g[i][1] = buf_ld16<f32x4>(rg, o + 16);
    }
}

// g of row i of a RawChunk as float32 (natural-log units)
template <int RPT, int IO, bool G16>
__device__ __forceinline__ f32x8 decay_row(const RawChunk<RPT, IO> &R, int i, bool g_f16)
{
    if constexpr (G16) {
        return g_f16 ? to_f32x8(__builtin_bit_cast(f16x8, R.g[i][0])) : to_f32x8(__builtin_bit_cast(bf16x8, R.g[i][0]));
    } else {
        return __builtin_shufflevector(R.g[i][0], R.g[i][1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

template <int K, int RPT, int IO>
__device__ __forceinline__ void load_keys(RawChunk<RPT, IO> &R, const FwdParams &p, int64_t c0, int len, int hk,
                                          int hv, int row0, int c0k)
{
    typedef typename IoT<IO>::v8 T8;
    const int rq = (int)p.sq * 2, rk = (int)p.sk * 2, rb = (int)p.sb * 2;  // token strides (bytes)
    const __amdgpu_buffer_rsrc_t bq = buf_rsrc(p.q + c0 * p.sq + hk * p.hsq, len * rq);
    const __amdgpu_buffer_rsrc_t bk = buf_rsrc(p.k + c0 * p.sk + hk * p.hsk, len * rk);
    const __amdgpu_buffer_rsrc_t rbb =
        p.beta ? buf_rsrc(p.beta + c0 * p.sb + hv * p.hsb, len * rb) : buf_rsrc(kOnes16[IO], 16);
    const int sb = p.beta ? rb : 0, cb = p.beta ? 2 * c0k : 0;
    for (int i = 0; i < RPT; ++i) {
        const int r = row0 + i;
        R.q[i] = buf_ld16<T8>(bq, (uint32_t)(r * rq + 2 * c0k));
        R.k[i] = buf_ld16<T8>(bk, (uint32_t)(r * rk + 2 * c0k));
        R.b[i] = buf_ld16<T8>(rbb, (uint32_t)(r * sb + cb));
    }
}

// Value-side rows of one chunk (state waves): v and w, rows row0 + i,
// columns c0 .. c0 + 7 (zero past the end of the sequence).
template <int V, int RPTV, int IO>
__device__ __forceinline__ void load_values(typename IoT<IO>::v8 *v, typename IoT<IO>::v8 *w, const FwdParams &p,
                                            int64_t c0, int len, int hv, int row0, int c0v, bool zero_v)
{
    typedef typename IoT<IO>::v8 T8;
    const int rs = (int)p.sv * 2, rsw = (int)p.sw * 2;  // token strides (bytes)
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(p.v + c0 * p.sv + hv * p.hsv, zero_v ? 0 : len * rs);
    const __amdgpu_buffer_rsrc_t rw =
        p.w ? buf_rsrc(p.w + c0 * p.sw + hv * p.hsw, zero_v ? 0 : len * rsw) : buf_rsrc(kOnes16[IO], 16);
    const int sw = p.w ? rsw : 0, cw = p.w ? 2 * c0v : 0;
    for (int i = 0; i < RPTV; ++i) {
        const int r = row0 + i;
        v[i] = buf_ld16<T8>(rv, (uint32_t)(r * rs + 2 * c0v));
        w[i] = buf_ld16<T8>(rw, (uint32_t)(r * sw + cw));
    }
}

// Key-wave thread map for phase E: key wave w owns the K/4 channels
// [w K/4, (w + 1) K/4) over all 64 rows of the chunk, so that the cumulative
// sum over the chunk stays inside the wave. lane = rg * NCG + cgl: cgl picks
// 8 channels, rg a group of RPT consecutive rows. Consecutive lanes hold the
// channel groups of one row, then of the next row group, so that 16-byte
// stores to a padded row-major tile fall in distinct banks.
template <int K>
struct KMap {
    static constexpr int NCG = K / 32;     // 8-channel groups per wave
    static constexpr int NRG = 64 / NCG;   // row groups per wave
    static constexpr int RPT = CH / NRG;   // rows per thread
    int rg, cgl, row0, c0;
    __device__ __forceinline__ explicit KMap(int rt)
    {
        const int lane = rt & 63, w = rt >> 6;
        cgl = lane % NCG;
        rg = lane / NCG;
        row0 = rg * RPT;
        c0 = w * (K / 4) + 8 * cgl;
    }
};

template <int D>
__device__ __forceinline__ float dpp_shr(float x)  // row_shr:D, zero shifted in
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + D, 0xf, 0xf, false));
}
template <int D>
__device__ __forceinline__ float dpp_ror(float x)  // row_ror:D
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + D, 0xf, 0xf, false));
}
template <int D>
__device__ __forceinline__ void row_scan_steps(float &s, float &t)
{
    if constexpr (D < 16) {
        s += dpp_shr<D>(s);
        t += dpp_ror<D>(t);
        row_scan_steps<2 * D>(s, t);
    }
}

// Inclusive prefix sum (incl) and total over the row groups of KMap: the
// lanes with equal lane % NCG form one sequence in lane order. DPP shifts
// scan inside each 16-lane row while DPP rotates form the row totals; the
// totals are carried across rows by permlane16 / permlane32 swaps, which
// hand every lane the values of both rows of its pair (both halves).
template <int NCG>
__device__ __forceinline__ void wave_scan(float x, int lane, float &incl, float &total)
{
    float s = x, t = x;
    row_scan_steps<NCG>(s, t);
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    const float ev = __uint_as_float(p16[0]), od = __uint_as_float(p16[1]);
    if (lane & 16) s += ev;
    const float pair = ev + od;
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
    const float lo = __uint_as_float(p32[0]), hi = __uint_as_float(p32[1]);
    if (lane & 32) s += lo;
    incl = s;
    total = lo + hi;
}

// One bit per lane of each KMap channel group (lanes cgl, cgl + NCG, ...).
template <int NCG>
__device__ __forceinline__ uint64_t group_lanes(int cgl)
{
    uint64_t m = 0;
    for (int i = 0; i < 64; i += NCG) m |= 1ull << i;
    return m << cgl;
}

// ----------------------------------------------------------- chain context --
// What one workgroup does: a token range of one sequence and value head,
// where its state starts and ends, and whether it writes the output.
struct Chain {
    int n, hv, hk;
    int64_t tb, te;   // token range (the sequence, or one segment of it)
    const float *s0;  // entering state [K][V] (nullptr: zero)
    float *s1;        // destination of the leaving state [K][V] (nullptr: none)
    bool s0_vm, s1_vm; // s0 / s1 stored V-major ([V][K]): the caller's states with that option
    bool s0_b16, s1_b16; // s0 / s1 hold bf16 elements (the caller's states may)
    bool ident;       // entering state is the identity (transition pass, K == V)
    bool zero_v;      // values taken as zero (transition pass)
    bool out;         // write the output rows
    uint16_t *ckpt;   // the state entering each chunk (bf16), chunk c at ckpt + c * HV * K * V (nullptr: none)
    char *rec;        // each chunk's record, chunk c at rec + c * HV * bwd_prep_bytes(K) (REC kernels)
};

// Copy a [64][K] bf16 tile from LDS (row pitch lp bytes) to a row-major
// global tile (row pitch 2 K bytes) in 16-byte pieces, piece e by thread
// t + i NT; xm flips sign bits (0x80008000: negate every element). Every
// LDS read is issued before the first store, so that the copy waits for
// LDS once instead of once per piece.
template <int K, int NT>
__device__ __forceinline__ void rec_tile(char *dst, const char *sm, int lo, int lp, int t, uint32_t xm)
{
    constexpr int PR = 2 * K / 16;  // pieces per row
    constexpr int NE = 64 * PR, NI = (NE + NT - 1) / NT;
    i32x4 x[NI];
    for (int i = 0; i < NI; ++i) {
        const int e0 = t + NT * i, e = e0 < NE ? e0 : NE - 1;  // a thread past the end re-reads the last piece
        x[i] = lds_ld<i32x4>(sm, lo + (e / PR) * lp + 16 * (e % PR));
    }
    const int m = (int)xm;
    for (int i = 0; i < NI; ++i) {
        const int e = t + NT * i;
        if (NE % NT == 0 || e < NE)
            *reinterpret_cast<i32x4 *>(dst + (e / PR) * (2 * K) + 16 * (e % PR)) =
                i32x4{x[i][0] ^ m, x[i][1] ^ m, x[i][2] ^ m, x[i][3] ^ m};
    }
}

// T (bf16 [64][64], LDS pitch lp) to the record: the 16x16 blocks above the
// diagonal are never written in LDS (the products skip them) and go out as
// zero; the diagonal blocks hold exact zeros above their diagonal. Reads
// first, then stores, as in rec_tile.
template <int NT>
__device__ __forceinline__ void rec_t(char *dst, const char *sm, int lo, int lp, int t)
{
    constexpr int NE = 64 * 8, NI = (NE + NT - 1) / NT;
    i32x4 x[NI];
    for (int i = 0; i < NI; ++i) {
        const int e0 = t + NT * i, e = e0 < NE ? e0 : NE - 1;
        const int r = e >> 3, cb = 16 * (e & 7);
        x[i] = (cb >> 5) > (r >> 4) ? i32x4{0, 0, 0, 0} : lds_ld<i32x4>(sm, lo + r * lp + cb);
    }
    for (int i = 0; i < NI; ++i) {
        const int e = t + NT * i;
        if (NE % NT == 0 || e < NE) *reinterpret_cast<i32x4 *>(dst + (e >> 3) * 128 + 16 * (e & 7)) = x[i];
    }
}

// Valid rows of the chunk starting at token c0 (0 past the end).
__device__ __forceinline__ int chunk_len(int64_t c0, int64_t te)
{
    return (int)(te - c0 <= 0 ? 0 : te - c0 < CH ? te - c0 : CH);
}

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

// The same tile from per-lane base pointers: rrb addresses RR row 16j + l16,
// xb the X row 16i + l16, both at column 8 q4.
template <int K>
__device__ __forceinline__ f32x4 ap_tile_at(const char *rrb, const char *xb)
{
    f32x4 acc = {0, 0, 0, 0};
    for (int ks = 0; ks < K / 32; ++ks) acc = mfma_bf16(lds_ld<bf16x8>(rrb, 64 * ks), lds_ld<bf16x8>(xb, 64 * ks), acc);
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
template <int K, int V, int IO, bool G16, bool L2N>
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
        if (lane == 0) lds_st<int>(smem, L::XN, cnt);
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
    const int nx = lds_ld<int>(smem, L::XN);
    const int r = tid >> 3, sb = tid & 7;
    float accA[8], accP[8];
    for (int u = 0; u < 8; ++u) accA[u] = accP[u] = 0.0f;
    const int64_t goff = c0 * p.sg + ch.hv * p.hsg;
    const float *gp = p.g ? static_cast<const float *>(p.g) + goff : nullptr;          // float32 g
    const uint16_t *gh = p.g ? static_cast<const uint16_t *>(p.g) + goff : nullptr;    // 16-bit g
    const bool g_f16 = p.gtype == G_F16;
    const uint16_t *qp = p.q + c0 * p.sq + ch.hk * p.hsq;
    const uint16_t *kp = p.k + c0 * p.sk + ch.hk * p.hsk;
    const uint16_t *bp = p.beta ? p.beta + c0 * p.sb + ch.hv * p.hsb : nullptr;
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
                float gv = 0.0f;
                if (ok && gp) {
                    if constexpr (G16) gv = (g_f16 ? io_bits_to_f32<IO_F16>(gh[t * p.sg + c])
                                                   : io_bits_to_f32<IO_BF16>(gh[t * p.sg + c])) * LOG2E;
                    else gv = gp[t * p.sg + c] * LOG2E;
                }
                float qv = ok ? io_bits_to_f32<IO>(qp[t * p.sq + c]) : 0.0f;
                float kk = ok ? io_bits_to_f32<IO>(kp[t * p.sk + c]) : 0.0f;
                const float bv = ok && bp ? io_bits_to_f32<IO>(bp[t * p.sb + c]) : 1.0f;
                if constexpr (L2N) {
                    const f32x2 nr = lds_ld<f32x2>(smem, L::NRM + 8 * (int)t);
                    qv *= nr[0];
                    kk *= nr[1];
                }
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
// Diagonal block of T = (I + A)^{-1} (blk: the block's first element in AB),
// solved by lanes 0-15 of one wave: lane l16 solves column l16 by
// right-looking forward substitution (as soon as t_c is known, its term is
// folded into every later row's accumulator, so that the dependent chain is
// one FMA and one subtraction per row). The block's rows are read as
// broadcasts, all in flight before the first use; with one lane group active
// they cost a quarter of the LDS bandwidth. Column l16 is written over A's
// block in AB (fp32, st_ab: row 0 of the column) and into TB (bf16, st_tb).
template <int K, int V>
__device__ __forceinline__ void t1_block(const char *blk, char *st_ab, char *st_tb, int l16)
{
    using L = Lds<K, V>;
    constexpr int RA = 4 * L::AP, RC = 2 * L::CP;
    f32x4 a[16][4];
    for (int r = 1; r < 16; ++r)
        for (int c4 = 0; 4 * c4 < r; ++c4) a[r][c4] = lds_ld<f32x4>(blk, r * RA + 16 * c4);
    for (int r = 1; r < 16; ++r)
        for (int c4 = 0; 4 * c4 < r; ++c4) asm volatile("" ::"v"(a[r][c4]));
    float acc[16], t[16];
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    for (int c = 0; c < 16; ++c) {
        t[c] = (c == l16 ? 1.0f : 0.0f) - acc[c];
        for (int r = c + 1; r < 16; ++r) acc[r] = fmaf(a[r][c >> 2][c & 3], t[c], acc[r]);
    }
    for (int r = 0; r < 16; ++r) {
        lds_st<float>(st_ab, r * RA, t[r]);
        lds_st<__bf16>(st_tb, r * RC, (__bf16)t[r]);
    }
}

// One 16-channel tile ct of the pseudo-keys, stored negated and row-major
// (token, channel) as -wy_w: -wy_w^T = -KB^T T^T, with KB^T operands from
// transpose reads of the row-major KB.
template <int K, int V>
__device__ __forceinline__ void wyw_tile(char *sm, int ct, int l16, int q4)
{
    using L = Lds<K, V>;
    constexpr int RK = 2 * L::KP, RC = 2 * L::CP;
    const char *const b_kbt = sm + (8 * q4 + (l16 >> 2)) * RK + 8 * (l16 & 3) + 32 * ct;  // KB transpose reads
    const char *const b_c8 = sm + l16 * RC + 16 * q4;              // T rows 16i + l16, columns 32ks + 8q4
    char *const b_wy = sm + l16 * RK + 8 * q4 + 32 * ct;           // -wy_w stores
    bf16x8 ak[2];
    for (int ks = 0; ks < 2; ++ks) {
        const int o = L::KB + 32 * ks * RK;
        ak[ks] = cat4(lds_tr(b_kbt, o), lds_tr(b_kbt, o + 4 * RK));
    }
    for (int i = 0; i < 4; ++i) {
        f32x4 acc = {0, 0, 0, 0};
        for (int ks = 0; ks <= (i >> 1); ++ks) acc = mfma_bf16(ak[ks], lds_ld<bf16x8>(b_c8, L::TB + 16 * i * RC + 64 * ks), acc);
        lds_st<bf16x4>(b_wy, L::WYW + 16 * i * RK, f32x4_to_bf16(-acc));
    }
}

// ------------------------------------------------ flagged channels, MFMA --
// A channel is flagged when its |G| leaves the single-reference range
// somewhere in the chunk (strong decay). Its share of A and P then uses
// tile-relative factors. For rows r in row tile i and s in column tile
// j < i, 2^(G_r - G_s) = 2^(G_r - R_i) 2^(R_i - G_s) with R_i = G at row
// 16 i - 1 (the end of tile i - 1): since g <= 0 both exponents are <= 0
// and both factors lie in [0, 1]. For the diagonal tile (i, i) the
// reference is row 16 i + 7, M_i: each exponent then spans at most 8
// tokens, within float32 range while every per-token |g| log2 e stays
// within XSUP. (The burn-gdn2 README's numerical-stability section: the
// factors stay tile-local, so strong decay cannot overflow them.)
// Key wave w gives its flagged channels slots XSW w .. XSW w + XSW - 1. In
// phase E it stages their G (float32, [slot][row] in TB); after B2 it builds
// the bf16 operands (row side X = beta k or q times 2^(G_r - ref), column
// side Y = k 2^(ref - G_s)), and after one more barrier every A / P tile
// adds sum over slots of Y_s X_r on v_mfma_f32_16x16x16_bf16, 16 slots per
// product. A chunk with more flagged channels in one key wave than it has
// slots, or with a flagged channel beyond XSUP, takes the scalar per-pair
// path (exact_ap) instead.
constexpr float XSUP = 15.0f;

// Operand rows (XP bf16 each). X, in the QH buffer of the other parity:
// X_off[isP][i - 1][16] for row tiles i = 1..3, X_mid[isP][i][16]. Y, in WV:
// Y_off for reference i, rows 0 .. 16 i - 1, at 8 (i - 1) i; Y_mid[i][16]
// at 96.
__device__ __forceinline__ int xrow_off(int isP, int i) { return 16 * (3 * isP + i - 1); }
__device__ __forceinline__ int xrow_mid(int isP, int i) { return 96 + 16 * (4 * isP + i); }
__device__ __forceinline__ int yrow_off(int i) { return 8 * (i - 1) * i; }
__device__ __forceinline__ int yrow_mid(int i) { return 96 + 16 * i; }

// How the chunk's A and P are formed: 0 single reference only, 1 flagged
// channels on MFMA, 2 the scalar per-pair path (the key waves' worst). The
// same for every thread (a scalar, so that the paths are uniform branches).
__device__ __forceinline__ int chunk_path(const char *fl)
{
    const i32x4 f = *reinterpret_cast<const i32x4 *>(fl);
    const int a = f[0] > f[1] ? f[0] : f[1], b = f[2] > f[3] ? f[2] : f[3];
    return __builtin_amdgcn_readfirstlane(a > b ? a : b);
}

// Bit b: some key wave owning a slot of product batch b (slots 16 b ..
// 16 b + 15) has a flagged channel.
template <int K, int V>
__device__ __forceinline__ int xbatches(const char *sm)
{
    using L = Lds<K, V>;
    const i32x4 c = lds_ld<i32x4>(sm, L::XC);
    int m = 0;
    for (int w = 0; w < 4; ++w)
        if (c[w] > 0) m |= 1 << (w * L::XSW / 16);
    return __builtin_amdgcn_readfirstlane(m);
}

// The flagged channels' share of tile (i, j) of A (isP 0) or P (isP 1) in
// ap_tile's transposed layout, added to acc; xb: byte offset of the X rows.
template <int K, int V>
__device__ __forceinline__ f32x4 xtile(const char *sm, int xb, int i, int j, int isP, int nbm, int l16, int q4,
                                       f32x4 acc)
{
    using L = Lds<K, V>;
    constexpr int XB2 = 2 * L::XP;  // bytes per operand row
    const int ya = L::WV + XB2 * ((i > j ? yrow_off(i) + 16 * j : yrow_mid(i)) + l16) + 8 * q4;
    const int xa = xb + XB2 * ((i > j ? xrow_off(isP, i) : xrow_mid(isP, i)) + l16) + 8 * q4;
    for (int b = 0; b < L::XNS / 16; ++b)
        if (nbm & (1 << b))
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_ld<bf16x4>(sm, ya + 32 * b), lds_ld<bf16x4>(sm, xa + 32 * b),
                                                             acc, 0, 0, 0);
    return acc;
}

// T's blocks (0, 1) and (2, 3) read as zero by the WY products; thread t of
// 128 clears 8 bytes (again after TB held staged G).
template <int K, int V>
__device__ __forceinline__ void zero_t_upper(char *sm, int t)
{
    using L = Lds<K, V>;
    const int b = t >> 6, rr = (t >> 2) & 15, cc = (t & 3) * 4;
    lds_st<uint64_t>(sm, L::TB + 2 * ((32 * b + rr) * L::CP + 32 * b + 16 + cc), 0ull);
}

// Wait for a chunk's raw inputs (the asm consumes the registers).
template <int RPT, int IO, bool G16>
__device__ __forceinline__ void await_raw(const RawChunk<RPT, IO> &R)
{
    for (int i = 0; i < RPT; ++i) {
        if constexpr (G16) asm volatile("" ::"v"(R.q[i]), "v"(R.k[i]), "v"(R.b[i]), "v"(R.g[i][0]));
        else asm volatile("" ::"v"(R.q[i]), "v"(R.k[i]), "v"(R.b[i]), "v"(R.g[i][0]), "v"(R.g[i][1]));
    }
}

// In-kernel q/k L2 normalisation, first half: the sums of squares of q and
// k over this lane's 8 channels of each of its rows, added over the lanes of
// the row group (the wave's K/4 channels) and stored per key wave,
// NP[wave][row] = (sum q^2, sum k^2). Phase E of the chunk adds the four
// waves' parts.
template <int K, int V, int RPT, int IO>
__device__ __forceinline__ void norm_partials(const RawChunk<RPT, IO> &R, char *sm, int rt)
{
    using L = Lds<K, V>;
    using M = KMap<K>;
    const M em(rt);
    const int w = rt >> 6;
    for (int i = 0; i < RPT; ++i) {
        const f32x8 qf = to_f32x8(R.q[i]), kf = to_f32x8(R.k[i]);
        float sq = 0.0f, sk = 0.0f;
        for (int j = 0; j < 8; ++j) {
            sq = fmaf(qf[j], qf[j], sq);
            sk = fmaf(kf[j], kf[j], sk);
        }
        for (int d = 1; d < M::NCG; d <<= 1) {
            sq += __shfl_xor(sq, d);
            sk += __shfl_xor(sk, d);
        }
        if (em.cgl == 0) lds_st<f32x2>(sm, L::NP + 8 * (w * CH + em.row0 + i), f32x2{sq, sk});
    }
}

// Flagged channels on MFMA, operand build (key waves, after B2): key wave
// rw fills its XSW slots, lane = row r: for slot k < cnt (the wave's
// flagged count) the row-side X (KB and QH forms) and column-side Y factors
// of every tile row r takes part in, from the G and raw q, k, beta that
// phase E staged; slots k >= cnt are zero. xb: byte offset of the X rows.
template <int K, int V, int IO, bool L2N>
__device__ __forceinline__ void xbuild(char *sm, int cnt, int rw, int r, int xb)
{
    using L = Lds<K, V>;
    constexpr int XSW = L::XSW, XB2 = 2 * L::XP;
    const int i0 = r >> 4, rl = r & 15;  // row tile, row within it
    float nq = 1.0f, nk = 1.0f;
    if constexpr (L2N) {
        const f32x2 nr = lds_ld<f32x2>(sm, L::NRM + 8 * r);
        nq = nr[0];
        nk = nr[1];
    }
    const int xo = xb + XB2 * (xrow_off(0, i0 > 0 ? i0 : 1) + rl), xoq = xo + XB2 * 48;  // X_off KB / QH (i0 >= 1)
    const int xm = xb + XB2 * (xrow_mid(0, i0) + rl), xmq = xm + XB2 * 64;              // X_mid KB / QH
    const int y1 = L::WV + XB2 * (yrow_off(1) + r), y2 = L::WV + XB2 * (yrow_off(2) + r),
              y3 = L::WV + XB2 * (yrow_off(3) + r);                                       // Y_off, reference tiles 1..3
    const int ym = L::WV + XB2 * (yrow_mid(i0) + rl);                                      // Y_mid
    for (int k = 0; k < XSW; ++k) {
        const int slot = XSW * rw + k, o = 2 * slot;
        __bf16 xkb = 0, xqh = 0, mkb = 0, mqh = 0, v1 = 0, v2 = 0, v3 = 0, vm = 0;
        if (k < cnt) {  // wave-uniform
            const int gs = L::TB + 4 * CH * slot, qs = L::XQ + 2 * CH * slot;
            const float Gr = lds_ld<float>(sm, gs + 4 * r), Mi = lds_ld<float>(sm, gs + 4 * (16 * i0 + 7));
            const float R1 = lds_ld<float>(sm, gs + 4 * 15), R2 = lds_ld<float>(sm, gs + 4 * 31),
                        R3 = lds_ld<float>(sm, gs + 4 * 47);
            const float qv = io_bits_to_f32<IO>(lds_ld<uint16_t>(sm, qs + 2 * r)) * nq;
            const float kv = io_bits_to_f32<IO>(lds_ld<uint16_t>(sm, qs + 2 * L::XNS * CH + 2 * r)) * nk;
            const float bk = io_bits_to_f32<IO>(lds_ld<uint16_t>(sm, qs + 4 * L::XNS * CH + 2 * r)) * kv;
            const float e = ex2(Gr - (i0 == 1 ? R1 : i0 == 2 ? R2 : R3)), em = ex2(Gr - Mi);
            xkb = (__bf16)(bk * e);
            xqh = (__bf16)(qv * e);
            mkb = (__bf16)(bk * em);
            mqh = (__bf16)(qv * em);
            v1 = (__bf16)(kv * ex2(R1 - Gr));
            v2 = (__bf16)(kv * ex2(R2 - Gr));
            v3 = (__bf16)(kv * ex2(R3 - Gr));
            vm = (__bf16)(kv * ex2(Mi - Gr));
        }
        if (i0 >= 1) {
            lds_st<__bf16>(sm, xo + o, xkb);
            lds_st<__bf16>(sm, xoq + o, xqh);
        }
        lds_st<__bf16>(sm, xm + o, mkb);
        lds_st<__bf16>(sm, xmq + o, mqh);
        if (i0 < 1) lds_st<__bf16>(sm, y1 + o, v1);
        if (i0 < 2) lds_st<__bf16>(sm, y2 + o, v2);
        if (i0 < 3) lds_st<__bf16>(sm, y3 + o, v3);
        lds_st<__bf16>(sm, ym + o, vm);
    }
}

// ------------------------------------------------------------- key waves --
// Barrier sequence per iteration (must match state_role): B2, then
// (exact_ap), B3, B4, B5. LDS addressing as in state_role: per-lane bases
// plus compile-time constants.
template <int K, int V, int IO, bool G16, bool L2N, bool REC>
__device__ __forceinline__ void key_role(char *smem, const FwdParams &p, const Chain &ch, int tid, int nc)
{
    using L = Lds<K, V>;
    using M = KMap<K>;
    constexpr int RPT = M::RPT;
    constexpr int NCTK = K / 64;            // -wy_w channel tiles per key wave
    constexpr int NCTK_KEY = NCTK > 1 ? NCTK - 1 : NCTK;  // of which the key wave computes
    constexpr int RK = 2 * L::KP, RC = 2 * L::CP, RA = 4 * L::AP;  // row pitches (bytes)

    const bool g_f16 = p.gtype == G_F16;
    RawChunk<RPT, IO> R;
    if (nc > 0) {
        const M em(tid & (NROLE - 1));
        load_decay<K, RPT, IO, G16>(R, p, ch.tb, chunk_len(ch.tb, ch.te), ch.hv, em.row0, em.c0);
        load_keys<K, RPT, IO>(R, p, ch.tb, chunk_len(ch.tb, ch.te), ch.hk, ch.hv, em.row0, em.c0);
        // complete the first chunk's loads before the loop, so that inside
        // it the vector memory counter only tracks the in-loop prefetch,
        // issued g first (a wait for g then leaves q, k, beta in flight)
        await_raw<RPT, IO, G16>(R);
        if constexpr (L2N) norm_partials<K, V, RPT, IO>(R, smem, tid & (NROLE - 1));
    }
    if constexpr (L2N) __syncthreads();  // ------------------- the first chunk's norms

    char *const smem0 = smem;
    const int tid0 = tid;
    for (int it = 0; it <= nc; ++it) {
        // lane-derived values are recomputed per chunk (see opaque_zero)
        const int z = opaque_zero();
        char *const sm = smem0 + z;
        const int tid = tid0 + z;
        const int lane = tid & 63, rw = __builtin_amdgcn_readfirstlane((tid >> 6) & 3), rt = tid & (NROLE - 1);
        const int l16 = lane & 15, q4 = lane >> 4;
        const M em(rt);
        const int row0 = em.row0, c0k = em.c0;
        const int o_e = row0 * RK + 2 * c0k;  // rows row0 + i, channels c0k .. c0k + 7
        const int o_c = 4 * c0k;              // fp32 per-channel records
        const int64_t c0 = ch.tb + (int64_t)it * CH;
        const bool act = it < nc;
        const int len = act ? chunk_len(c0, ch.te) : 0;
        const int qb = L::QH + (it & 1) * L::QH_SZ;
        char *const b_c = sm + o_c;

        // ---- E: cumulative log2 decay over the chunk (in-thread over RPT
        // rows, then across the wave's row groups), exact-channel flags and
        // the MFMA operands  KB = beta k 2^G,  QH = q 2^G,  RR = k 2^-G,
        // KT = k 2^(G_last - G)
        bf16x8 ktr[RPT];
        f32x8 egl;
        uint32_t wmask = 0;  // flagged channels of this wave (bit 8 cgl + j; wave-uniform)
        int wcnt = 0;
        if (act) {
            // all of this chunk's raw inputs are complete here: the next
            // chunk's g is issued below, and a later wait for q, k, beta
            // would otherwise also wait for it
            await_raw<RPT, IO, G16>(R);
            float G[RPT][8], glast[8];
            for (int i = 0; i < RPT; ++i) {
                const f32x8 gi = decay_row<RPT, IO, G16>(R, i, g_f16);
                for (int j = 0; j < 8; ++j) G[i][j] = (i ? G[i - 1][j] : 0.0f) + gi[j] * LOG2E;
            }
            for (int j = 0; j < 8; ++j) {
                float incl, tot;
                wave_scan<M::NCG>(G[RPT - 1][j], lane, incl, tot);
                const float excl = incl - G[RPT - 1][j];
                for (int i = 0; i < RPT; ++i) G[i][j] += excl;
                glast[j] = tot;
            }
            // a channel is exact if |G| leaves the single-reference range
            // anywhere in the chunk (NaN counts as extreme)
            const uint64_t mine = group_lanes<M::NCG>(em.cgl);
            bool xf[8];
            uint64_t anyb = 0;
            for (int j = 0; j < 8; ++j) {
                bool out = false;
                for (int i = 0; i < RPT; ++i) out |= !(fabsf(G[i][j]) <= XLIM);
                const uint64_t b = __ballot(out);
                xf[j] = (b & mine) != 0;
                anyb |= b;
            }
            const bool wx = anyb != 0;  // wave-uniform: any exact channel of this wave
            // this wave's path: 0 none flagged, 1 flagged channels on MFMA
            // (G staged in TB), 2 scalar per-pair path (too many flagged
            // channels for the wave's slots, or one whose per-token decay
            // exceeds XSUP: G's steps, the first one across lanes)
            int wst = 0;
            if (wx) {
                bool sup = false;
                for (int j = 0; j < 8; ++j) {
                    const uint64_t b = __ballot(xf[j]);
                    for (int g = 0; g < M::NCG; ++g)
                        if (b & group_lanes<M::NCG>(g)) wmask |= 1u << (8 * g + j);
                    const float prev = __shfl(G[RPT - 1][j], lane - M::NCG);
                    float st = fabsf(G[0][j] - (em.rg ? prev : 0.0f));
                    for (int i = 1; i < RPT; ++i) st = fmaxf(st, fabsf(G[i][j] - G[i - 1][j]));
                    sup |= xf[j] && !(st <= XSUP);
                }
                wcnt = __popc(wmask);
                wst = (__ballot(sup) != 0 || wcnt > L::XSW) ? 2 : 1;
            }
            if (wst == 1)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (xf[j]) {
                        const int cw = 8 * em.cgl + j;
                        const int slot = L::XSW * rw + __popc(wmask & ((1u << cw) - 1u));
                        for (int i = 0; i < RPT; ++i) {
                            const int r = row0 + i, qs = L::XQ + 2 * (CH * slot + r);
                            lds_st<float>(sm, L::TB + 4 * (CH * slot + r), G[i][j]);
                            lds_st<uint16_t>(sm, qs, bits16(R.q[i], j));
                            lds_st<uint16_t>(sm, qs + 2 * L::XNS * CH, bits16(R.k[i], j));
                            lds_st<uint16_t>(sm, qs + 4 * L::XNS * CH, bits16(R.b[i], j));
                        }
                    }
            if (lane == 0) {
                lds_st<int>(sm, L::FL + 4 * rw, wst);
                lds_st<int>(sm, L::XC + 4 * rw, wcnt);
            }
            if (em.rg == 0) {
                lds_st<i32x4>(b_c, L::XF, i32x4{xf[0], xf[1], xf[2], xf[3]});
                lds_st<i32x4>(b_c, L::XF + 16, i32x4{xf[4], xf[5], xf[6], xf[7]});
            }
            for (int j = 0; j < 8; ++j) egl[j] = ex2(glast[j]);
            // in-kernel L2 normalisation: the reciprocal norms of this
            // lane's rows from the key waves' partial sums (x / max(|x|, eps))
            float nq[RPT], nk[RPT];
            if constexpr (L2N) {
                for (int i = 0; i < RPT; ++i) {
                    const int o = L::NP + 8 * (row0 + i);
                    const f32x2 ss = lds_ld<f32x2>(sm, o) + lds_ld<f32x2>(sm, o + 8 * CH) +
                                     lds_ld<f32x2>(sm, o + 16 * CH) + lds_ld<f32x2>(sm, o + 24 * CH);
                    nq[i] = 1.0f / fmaxf(sqrtf(ss[0]), 1e-12f);
                    nk[i] = 1.0f / fmaxf(sqrtf(ss[1]), 1e-12f);
                    if (rw == 0 && em.cgl == 0) lds_st<f32x2>(sm, L::NRM + 8 * (row0 + i), f32x2{nq[i], nk[i]});
                }
            }
            char *const b_e = sm + o_e;
            for (int i = 0; i < RPT; ++i) {
                f32x8 qf = to_f32x8(R.q[i]);
                f32x8 kf = to_f32x8(R.k[i]);
                if constexpr (L2N) {
                    qf *= nq[i];
                    kf *= nk[i];
                }
                const f32x8 bk = to_f32x8(R.b[i]) * kf;
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
                lds_st<bf16x8>(b_e, L::KB + i * RK, f32x8_to_bf16(kb));
                lds_st<bf16x8>(b_e, L::RR + i * RK, f32x8_to_bf16(rr));
                lds_st<bf16x8>(b_e, qb + i * RK, f32x8_to_bf16(qh));
                ktr[i] = f32x8_to_bf16(kt);
                // the backward's record: RR, with K-hat in flagged channels
                if constexpr (REC) {
                    constexpr PrepRecord PR{K};
                    f32x8 rk;
                    for (int j = 0; j < 8; ++j) rk[j] = xf[j] ? kt[j] : rr[j];
                    *reinterpret_cast<bf16x8 *>(ch.rec + (int64_t)it * p.HV * PR.bytes() + PR.rr() +
                                                2 * ((row0 + i) * K + c0k)) = f32x8_to_bf16(rk);
                }
            }
            // the next chunk's g (this chunk's is consumed): a chunk period
            // ahead of its use, and issued last, so that no register copy
            // in this phase targets a load in flight. Issued past the last
            // chunk too, with an empty range (no memory access): an
            // unconditional load leaves the register allocator no value to
            // merge at the loop head
            load_decay<K, RPT, IO, G16>(R, p, c0 + CH, chunk_len(c0 + CH, ch.te), ch.hv, row0, c0k);
        }
        __syncthreads();  // ------------------------------------------ B2
        if (!act) break;

        // KT and 2^G_last of this chunk: the state waves read the previous
        // chunk's until B2
        {
            char *const b_e = sm + o_e;
            for (int i = 0; i < RPT; ++i) lds_st<bf16x8>(b_e, L::KT + i * RK, ktr[i]);
        }
        if (em.rg == 0) {
            lds_st<f32x4>(b_c, L::GAM, f32x4{egl[0], egl[1], egl[2], egl[3]});
            lds_st<f32x4>(b_c, L::GAM + 16, f32x4{egl[4], egl[5], egl[6], egl[7]});
        }

        // ---- AP + T1: A's diagonal tile rw, then its block of T
        const int path = chunk_path(sm + L::FL);
        if (path == 0) {
            const char *const b_k8 = sm + l16 * RK + 16 * q4 + rw * 16 * RK;  // rows 16 rw + l16, columns 8q4
            const f32x4 x = ap_mask(ap_tile_at<K>(b_k8 + L::RR, b_k8 + L::KB), true, false, l16, q4);
            lds_st<f32x4>(sm, L::AB + l16 * RA + 16 * q4 + rw * (16 * RA + 64), x);
        } else if (path == 1) {
            // flagged channels on MFMA: build their operands, then (after
            // one more barrier, which the state waves match) add them to the
            // diagonal tile
            const int xb = L::QH + ((it + 1) & 1) * L::QH_SZ;
            xbuild<K, V, IO, L2N>(sm, wcnt, rw, lane, xb);
            const char *const b_k8 = sm + l16 * RK + 16 * q4 + rw * 16 * RK;
            const f32x4 x0 = ap_tile_at<K>(b_k8 + L::RR, b_k8 + L::KB);
            __syncthreads();  // ----------------------------------------- B2x
            const f32x4 x = ap_mask(xtile<K, V>(sm, xb, rw, rw, 0, xbatches<K, V>(sm), l16, q4, x0), true, false, l16, q4);
            lds_st<f32x4>(sm, L::AB + l16 * RA + 16 * q4 + rw * (16 * RA + 64), x);
            if (rt < 128) zero_t_upper<K, V>(sm, rt);  // TB held the staged G
        } else {
            exact_ap<K, V, IO, G16, L2N>(sm, p, ch, c0, len, qb, tid);
            if (rt < 128) zero_t_upper<K, V>(sm, rt);  // TB may hold staged G
        }
        if (q4 == 0)
            t1_block<K, V>(sm + L::AB + rw * (16 * RA + 64), sm + L::AB + 4 * l16 + rw * (16 * RA + 64),
                           sm + L::TB + 2 * l16 + rw * (16 * RC + 32), l16);
        __syncthreads();  // ------------------------------------------ B3

        // the next chunk's q, k, beta (its g went out in phase E): issued
        // while the state waves build T's off-diagonal blocks (the issue
        // stalls until the CU's memory pipeline has room); WY and the next
        // phase E hide the latency
        load_keys<K, RPT, IO>(R, p, c0 + CH, chunk_len(c0 + CH, ch.te), ch.hk, ch.hv, row0, c0k);  // empty range past the end
        __syncthreads();  // ------------------------------------------ B4

        // ---- WY: -wy_w for this wave's channel tiles but the last when there
        // are two (that one goes to a state wave, which has the time)
        for (int jt = 0; jt < NCTK_KEY; ++jt) wyw_tile<K, V>(sm, rw * NCTK + jt, l16, q4);
        // the next chunk's norm partials (its q, k arrive here; phase E of
        // this chunk has read the previous ones)
        if constexpr (L2N)
            if (it + 1 < nc) norm_partials<K, V, RPT, IO>(R, sm, rt);
        // the backward's record of this chunk, last part: T (complete at B4)
        // and 2^G_last (negated in flagged channels); RR went out in phase
        // E, KB, QH and P from the state waves in phase T2
        if constexpr (REC) {
            constexpr PrepRecord PR{K};
            char *const rc = ch.rec + (int64_t)it * p.HV * PR.bytes();
            rec_t<NROLE>(rc + PR.t(), sm, L::TB, RC, rt);
            if (rt < K / 4) {
                const f32x4 gm = lds_ld<f32x4>(sm, L::GAM + 16 * rt);
                const i32x4 xf = lds_ld<i32x4>(sm, L::XF + 16 * rt);
                f32x4 gs;
                for (int e = 0; e < 4; ++e) gs[e] = xf[e] ? -gm[e] : gm[e];
                *reinterpret_cast<f32x4 *>(rc + PR.gam() + 16 * rt) = gs;
            }
        }
        __syncthreads();  // ------------------------------------------ B5
    }
}

// ---------------------------------------------------------------- phase T2 --
// Block column J of T below the diagonal, state wave J:
// T_iJ = -T_ii sum_{k=J}^{i-1} A_ik T_kJ, i = J+1..3, on bf16 MFMA with
// float32 operands split into high and low bf16 parts (three products; the
// dropped low x low term is 2^-16 relative). T_kJ (k > J) stay in registers
// in the MFMA result layout, which is the B operand layout of the 16x16x16
// product. Every A tile and diagonal block of the column is read before the
// first product, so that the dependent chain (two products per block row)
// waits for LDS once, not once per product.
template <int K, int V, int J>
__device__ __forceinline__ void t2_column(char *sm, int l16, int q4)
{
    using L = Lds<K, V>;
    constexpr int RA = 4 * L::AP, RC = 2 * L::CP;
    const char *const b_a4 = sm + l16 * RA + 16 * q4;                                // rows 16i + l16, columns 4q4
    const char *const b_tc = sm + 4 * q4 * RA + 4 * l16 + J * (16 * RA + 64);        // rows 4q4 + e, column l16
    f32x4 tjj, a[4][4];  // a[i][k]: A_ik for J <= k < i, T_ii for k = i
    for (int e = 0; e < 4; ++e) tjj[e] = lds_ld<float>(b_tc, L::AB + e * RA);
    for (int i = J + 1; i < 4; ++i)
        for (int k = J; k <= i; ++k) a[i][k] = lds_ld<f32x4>(b_a4, L::AB + 16 * i * RA + 64 * k);
    Split4 Tc[4];
    Tc[J] = split4(tjj);
    char *const b_tb = sm + 4 * q4 * RC + 2 * l16 + 32 * J;
    for (int i = J + 1; i < 4; ++i) {
        f32x4 X = {0, 0, 0, 0};
        for (int k = J; k < i; ++k) X = mfma3(split4(a[i][k]), Tc[k], X);
        const f32x4 Y = mfma3(split4(-a[i][i]), split4(X), f32x4{0, 0, 0, 0});
        Tc[i] = split4(Y);
        for (int e = 0; e < 4; ++e) lds_st<__bf16>(b_tb, L::TB + (16 * i + e) * RC, (__bf16)Y[e]);
    }
}

// The state waves' tiles of A and P (t = 4..19), four per wave, grouped so
// that a wave's tiles share operands: wave 0 A(3,0) P(3,0) A(3,1) P(3,1),
// wave 1 A(3,2) P(3,2) P(3,3) P(2,2), wave 2 A(2,0) P(2,0) A(2,1) P(2,1),
// wave 3 A(1,0) P(1,0) P(1,1) P(0,0). Four bits per entry (t - 4).
__device__ __forceinline__ int ap_tile_of(int rw, int m) { return 4 + (int)((0x6870a291bfe5d4c3ull >> (4 * (4 * rw + m))) & 15); }

// Phase AP of a state wave: its four tiles (ap_tile_of) of A and P from the
// single-reference operands. Each distinct operand tile is read once: the
// row side KB_i and QH_i of one row tile i (and QH_i2 of a second on odd
// waves) and the column side RR_ja, RR_jb: at most five operand tiles per
// wave instead of eight.
// Every read is issued before the first product, so that their LDS round
// trips overlap and the four accumulation chains interleave.
template <int K, int V>
__device__ __forceinline__ void state_ap_tiles(const char *sm, int o_k8, int it, int rw, f32x4 (&acc)[4])
{
    using L = Lds<K, V>;
    constexpr int RK = 2 * L::KP, NKS = K / 32;
    const char *const b_k8 = sm + o_k8;
    const int xq = L::QH + (it & 1) * L::QH_SZ;  // QH of this chunk for P tiles
    const int w = __builtin_amdgcn_readfirstlane(rw);
    const bool odd = (w & 1) != 0;
    const int ja = w == 1 ? 2 : 0, jb = ja + 1;            // column tiles
    const int i0 = w < 2 ? 3 : w == 2 ? 2 : 1, i2 = w == 1 ? 2 : 0;  // row tiles
    bf16x8 ra[NKS], rb[NKS], x0[NKS], x1[NKS], x2[NKS];
    for (int ks = 0; ks < NKS; ++ks) {
        ra[ks] = lds_ld<bf16x8>(b_k8, L::RR + 16 * ja * RK + 64 * ks);
        rb[ks] = lds_ld<bf16x8>(b_k8, L::RR + 16 * jb * RK + 64 * ks);
        x0[ks] = lds_ld<bf16x8>(b_k8, L::KB + 16 * i0 * RK + 64 * ks);
        x1[ks] = lds_ld<bf16x8>(b_k8, xq + 16 * i0 * RK + 64 * ks);
    }
    if (odd)
        for (int ks = 0; ks < NKS; ++ks) x2[ks] = lds_ld<bf16x8>(b_k8, xq + 16 * i2 * RK + 64 * ks);
    for (int m = 0; m < 4; ++m) acc[m] = f32x4{0, 0, 0, 0};
    if (odd) {
        for (int ks = 0; ks < NKS; ++ks) {
            acc[0] = mfma_bf16(ra[ks], x0[ks], acc[0]);
            acc[1] = mfma_bf16(ra[ks], x1[ks], acc[1]);
            acc[2] = mfma_bf16(rb[ks], x1[ks], acc[2]);
            acc[3] = mfma_bf16(ra[ks], x2[ks], acc[3]);
        }
    } else {
        for (int ks = 0; ks < NKS; ++ks) {
            acc[0] = mfma_bf16(ra[ks], x0[ks], acc[0]);
            acc[1] = mfma_bf16(ra[ks], x1[ks], acc[1]);
            acc[2] = mfma_bf16(rb[ks], x0[ks], acc[2]);
            acc[3] = mfma_bf16(rb[ks], x1[ks], acc[3]);
        }
    }
}

// The causal part of the four tiles: A as float32 into AB, P as bf16 into PB.
template <int K, int V>
__device__ __forceinline__ void state_ap_store(char *sm, const f32x4 (&acc)[4], int rw, int o_c4, int o_a4, int l16, int q4)
{
    using L = Lds<K, V>;
    constexpr int RC = 2 * L::CP, RA = 4 * L::AP;
    for (int m = 0; m < 4; ++m) {
        const int t = ap_tile_of(rw, m);
        const int i = tile_i(t), j = tile_j(t);
        const bool isP = t >= 10;
        const f32x4 x = ap_mask(acc[m], i == j, isP, l16, q4);
        if (isP) lds_st<bf16x4>(sm, L::PB + o_c4 + 16 * i * RC + 32 * j, f32x4_to_bf16(x));
        else lds_st<f32x4>(sm, L::AB + o_a4 + 16 * i * RA + 64 * j, x);
    }
}

// ----------------------------------------------------------- state waves --
// Register row order of the state. S is held in the MFMA result layout:
// lane (l16, q4) holds rows 4 q4 + e (e = 0..3) of each 16-row tile rt,
// column l16. Those rows stand for key channels in a permuted order: tile
// rt = 2 ks + h, lane quarter q4, element e is channel
// 32 ks + 8 q4 + 4 h + e. Then the bf16 operand built from the tile pair
// (2 ks, 2 ks + 1) holds channels 32 ks + 8 q4 .. + 7 in order, so the LDS
// operands it meets (wy_w and QH, stored in natural channel order) are one
// 16-byte read per lane instead of two 8-byte reads (which share banks at
// the padded row pitch).
__device__ __forceinline__ int state_chan(int rt, int q4, int e) { return 32 * (rt >> 1) + 8 * q4 + 4 * (rt & 1) + e; }

// LDS addressing in the chunk loops: every access is (per-lane base) +
// (compile-time constant). The lane parts are loop invariant; the per-chunk
// opaque zero is added to a handful of base pointers once per chunk, so the
// constants fold into the instructions' offset fields (and pairs of reads
// merge) instead of being hoisted out of the loop one register per address.
template <int K, int V, int IO, bool G16, bool L2N, bool REC>
__device__ __forceinline__ void state_role(char *smem, const FwdParams &p, const Chain &ch, int tid, int nc)
{
    using L = Lds<K, V>;
    constexpr int CGV = V / 8;
    constexpr int RPTV = CH * CGV / NROLE;
    constexpr int VW = V / 4;     // value columns per state wave
    constexpr int NCT = VW / 16;  // 16-column tiles per state wave
    constexpr int NRT = K / 16;   // 16-row tiles of the state
    constexpr int NKS = K / 32;   // 32-deep k slabs over K
    constexpr int RK = 2 * L::KP, RC = 2 * L::CP, RV = 2 * L::VP, RA = 4 * L::AP;  // row pitches (bytes)

    // state: rows 16*it + 4*q4 + e, column vbase + 16*jt + l16
    f32x4 S[NRT][NCT];
    if (ch.ident) {
        const int lane = tid & 63, rw = tid >> 6;
        const int l16 = lane & 15, q4 = lane >> 4;
        const int vbase = rw * VW;
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e) S[it][jt][e] = state_chan(it, q4, e) == vbase + 16 * jt + l16 ? 1.0f : 0.0f;
    } else if (ch.s0) {
        const int lane = tid & 63, rw = tid >> 6;
        const int l16 = lane & 15, q4 = lane >> 4;
        const int vbase = rw * VW;
        const float *h0 = ch.s0;
        const int sr = ch.s0_vm ? 1 : V, sc = ch.s0_vm ? K : 1;  // strides of (state row, column)
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e)
                    S[it][jt][e] = state_ld(h0, ch.s0_b16, state_chan(it, q4, e) * sr + (vbase + 16 * jt + l16) * sc);
        // complete these loads here: left outstanding into the chunk
        // loop, they make every later write of S wait on the vector
        // memory counter, which then also waits for the v, w prefetch
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt) asm volatile("" ::"v"(S[it][jt]));
    } else {
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt) S[it][jt] = f32x4{0, 0, 0, 0};
    }
    f32x4 U[4][NCT];  // wy_u, then U, of the chunk in the state pass
    if constexpr (L2N) __syncthreads();  // ------------------- the first chunk's norms (key waves)

    char *const smem0 = smem;
    const int tid0 = tid;
    for (int it = 0; it <= nc; ++it) {
        // lane-derived values are recomputed per chunk from an opaque copy
        // of the thread id (see opaque_zero)
        const int z = opaque_zero();
        char *const sm = smem0 + z;
        const int tid = tid0 + z;
        const int lane = tid & 63, rw = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l16 = lane & 15, q4 = lane >> 4;
        const int vbase = rw * VW;
        const EMap<V> emv(tid);
        // per-lane byte offsets of the access patterns
        const int o_c4 = l16 * RC + 8 * q4;                           // 64-column rows 16i + l16, columns 32ks + 4q4 (+16)
        const int o_k8 = l16 * RK + 16 * q4;                          // K-pitched rows, columns 32ks + 8q4
        const int o_c8 = l16 * RC + 16 * q4;                          // 64-column rows, columns 32ks + 8q4
        const int o_a4 = l16 * RA + 16 * q4;                          // fp32 tile rows 16i + l16, columns 4q4
        const int64_t c0 = ch.tb + (int64_t)it * CH;
        const bool act = it < nc;
        const int len = act ? chunk_len(c0, ch.te) : 0;
        const char *const b_k8 = sm + o_k8;
        const char *const b_c4 = sm + o_c4;

        // ---- S, first half (chunk it - 1): U = wy_u - wy_w S. S as bf16
        // operands: k slab ks holds channels 32ks + 8q4 + 0..7 (state_chan),
        // so wy_w and QH are read 8 consecutive channels per lane; U as
        // bf16 operands (Ub): token slab ks holds tokens {32ks + 4q4 + e}
        // then {32ks + 16 + 4q4 + e}, e = 0..3, and P is read in the same
        // token order.
        bf16x8 Ub[2][NCT], Sb[NKS][NCT];
        if (it > 0 && ch.ckpt) {
            // the state entering chunk it - 1, rounded to bf16 (for the backward)
            uint16_t *const dst = ch.ckpt + (int64_t)(it - 1) * p.HV * (K * V) + vbase + l16;
            for (int rt = 0; rt < NRT; ++rt)
                for (int jt = 0; jt < NCT; ++jt)
                    for (int e = 0; e < 4; ++e)
                        dst[state_chan(rt, q4, e) * V + 16 * jt] = __builtin_bit_cast(uint16_t, (__bf16)S[rt][jt][e]);
        }
        if (it > 0) {
            for (int ks = 0; ks < NKS; ++ks)
                for (int jt = 0; jt < NCT; ++jt)
                    Sb[ks][jt] = cat4(f32x4_to_bf16(S[2 * ks][jt]), f32x4_to_bf16(S[2 * ks + 1][jt]));
            for (int i = 0; i < 4; ++i)
                for (int ks = 0; ks < NKS; ++ks) {
                    const int o = L::WYW + 16 * i * RK + 64 * ks;
                    const bf16x8 aw = lds_ld<bf16x8>(b_k8, o);
                    for (int jt = 0; jt < NCT; ++jt) U[i][jt] = mfma_bf16(aw, Sb[ks][jt], U[i][jt]);
                }
            for (int ks = 0; ks < 2; ++ks)
                for (int jt = 0; jt < NCT; ++jt)
                    Ub[ks][jt] = cat4(f32x4_to_bf16(U[2 * ks][jt]), f32x4_to_bf16(U[2 * ks + 1][jt]));
            // the backward's record of chunk it - 1, last part: wy_w (held
            // negated here; the A tiles of chunk it overwrite it after B2)
            if constexpr (REC) {
                constexpr PrepRecord PR{K};
                rec_tile<K, NROLE>(ch.rec + (int64_t)(it - 1) * p.HV * PR.bytes() + PR.wy(), sm, L::WYW, RK, tid, 0x80008000u);
            }
        }

        // this chunk's v and w (stored as w v after B2; the latency hides
        // behind the rest of phase S, AP and T1); past the last chunk an
        // empty range (no memory access), so that the loads are
        // unconditional
        typename IoT<IO>::v8 vr[RPTV], wr[RPTV];
        load_values<V, RPTV, IO>(vr, wr, p, c0, len, ch.hv, emv.row0, emv.c0, ch.zero_v);

        // ---- S, second half: the output, computed transposed,
        // O^T = scale (S^T QH^T + U^T P^T), 4 consecutive values of an
        // output row per lane, staged in LDS and stored as 16-byte pieces;
        // then S <- diag(2^G_last) S + KT^T U,
        // with KT^T operands from transpose reads of the row-major KT
        // (tokens in the permuted order of Ub).
        if (it > 0) {
            const int64_t cp = c0 - CH;
            const int lenp = chunk_len(cp, ch.te);
            const char *const b_q = b_k8 + ((it - 1) & 1) * L::QH_SZ;
            if (ch.out) {
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * i + l16;
                    f32x4 Y[NCT];
                    for (int jt = 0; jt < NCT; ++jt) Y[jt] = f32x4{0, 0, 0, 0};
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int o = L::QH + 16 * i * RK + 64 * ks;
                        const bf16x8 bq = lds_ld<bf16x8>(b_q, o);
                        for (int jt = 0; jt < NCT; ++jt) Y[jt] = mfma_bf16(Sb[ks][jt], bq, Y[jt]);
                    }
                    for (int ks = 0; ks <= (i >> 1); ++ks) {
                        const int o = L::PB + 16 * i * RC + 64 * ks;
                        const bf16x8 bp = cat4(lds_ld<bf16x4>(b_c4, o), lds_ld<bf16x4>(b_c4, o + 32));
                        for (int jt = 0; jt < NCT; ++jt) Y[jt] = mfma_bf16(Ub[ks][jt], bp, Y[jt]);
                    }
                    // staged in this wave's columns of the free WV region
                    for (int jt = 0; jt < NCT; ++jt)
                        lds_st<typename IoT<IO>::v4>(sm, L::WV + row * RV + 2 * (vbase + 16 * jt + 4 * q4),
                                                     __builtin_convertvector(Y[jt] * p.scale, typename IoT<IO>::v4));
                }
                // ... and stored from there as 16-byte pieces of a row, the
                // wave's VW columns of a row contiguous (its own LDS writes
                // precede these reads: no barrier)
                constexpr int PPR = VW / 8, RPI = 64 / PPR;  // pieces per row, rows per store
                const int pr = lane / PPR, pc = 8 * (lane % PPR);
                for (int m = 0; m < CH / RPI; ++m) {
                    const int r = RPI * m + pr;
                    const i32x4 x = lds_ld<i32x4>(sm, L::WV + r * RV + 2 * (vbase + pc));
                    if (r < lenp) *reinterpret_cast<i32x4 *>(p.out + (cp + r) * p.so + ch.hv * p.hso + vbase + pc) = x;
                }
            }
            // KT transpose reads: lane group l16 & 3 reads 4 channels, which
            // become rows 4 (l16 & 3) + e of the A operand, in state_chan order
            const char *const b_kt = sm + (4 * q4 + (l16 >> 2)) * RK + 16 * (l16 & 3);
            const char *const b_g = sm + 32 * q4;
            for (int rtile = 0; rtile < NRT; ++rtile) {
                const int cb = 32 * (rtile >> 1) + 4 * (rtile & 1);  // state_chan(rtile, q4, e) - 8 q4 - e
                const f32x4 gam = lds_ld<f32x4>(b_g, L::GAM + 4 * cb);
                bf16x8 ak[2];
                for (int ks = 0; ks < 2; ++ks) {
                    const int o = L::KT + 32 * ks * RK + 2 * cb;
                    ak[ks] = cat4(lds_tr(b_kt, o), lds_tr(b_kt, o + 16 * RK));
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

        // ---- AP: the 16 tiles that are not A's diagonal, four per state
        // wave
        const int path = chunk_path(sm + L::FL);
        if (path == 0) {
            f32x4 acc[4];
            state_ap_tiles<K, V>(sm, o_k8, it, rw, acc);
            state_ap_store<K, V>(sm, acc, rw, o_c4, o_a4, l16, q4);
        } else if (path == 1) {
            // the flagged channels' share, once the key waves have built
            // their operands (a block of its own, so that the single-
            // reference block above compiles as if it were alone)
            f32x4 acc[4];
            state_ap_tiles<K, V>(sm, o_k8, it, rw, acc);
            __syncthreads();  // ----------------------------------------- B2x
            const int xb = L::QH + ((it + 1) & 1) * L::QH_SZ, nbm = xbatches<K, V>(sm);
            for (int m = 0; m < 4; ++m) {
                const int t = ap_tile_of(rw, m);
                acc[m] = xtile<K, V>(sm, xb, tile_i(t), tile_j(t), t >= 10 ? 1 : 0, nbm, l16, q4, acc[m]);
            }
            state_ap_store<K, V>(sm, acc, rw, o_c4, o_a4, l16, q4);
        } else {
            exact_ap<K, V, IO, G16, L2N>(sm, p, ch, c0, len, L::QH + (it & 1) * L::QH_SZ, tid);
        }
        // w v of this chunk, row-major (with flagged channels on MFMA, WV
        // holds their column-side operands until B3: stored after it)
        if (path != 1) {
            char *const b_wv = sm + emv.row0 * RV + 2 * emv.c0;
            for (int i = 0; i < RPTV; ++i) {
                const f32x8 wv = to_f32x8(vr[i]) * to_f32x8(wr[i]);
                lds_st<bf16x8>(b_wv, L::WV + i * RV, f32x8_to_bf16(wv));
            }
        }
        __syncthreads();  // ------------------------------------------ B3
        if (path == 1) {
            char *const b_wv = sm + emv.row0 * RV + 2 * emv.c0;
            for (int i = 0; i < RPTV; ++i) {
                const f32x8 wv = to_f32x8(vr[i]) * to_f32x8(wr[i]);
                lds_st<bf16x8>(b_wv, L::WV + i * RV, f32x8_to_bf16(wv));
            }
        }

        // ---- T2: block column j = rw of T (t2_column)
        if (rw == 0) t2_column<K, V, 0>(sm, l16, q4);
        else if (rw == 1) t2_column<K, V, 1>(sm, l16, q4);
        else if (rw == 2) t2_column<K, V, 2>(sm, l16, q4);
        // the backward's record of this chunk: KB, QH and P (final since B3)
        // from waves 1-3, whose block columns are short or empty and whose
        // memory queue is idle here (behind the key waves' loads of the next
        // chunk, these stores would hold up B4)
        if constexpr (REC) {
            if (rw > 0) {
                constexpr PrepRecord PR{K};
                char *const rc = ch.rec + (int64_t)it * p.HV * PR.bytes();
                rec_tile<K, NROLE - 64>(rc + PR.kb(), sm, L::KB, RK, tid - 64, 0u);
                rec_tile<K, NROLE - 64>(rc + PR.qh(), sm, L::QH + (it & 1) * L::QH_SZ, RK, tid - 64, 0u);
                rec_tile<64, NROLE - 64>(rc + PR.p(), sm, L::PB, RC, tid - 64, 0u);
            }
        }
        __syncthreads();  // ------------------------------------------ B4

        // ---- WY: the last -wy_w channel tile of key wave rw (K = 128), then
        // wy_u = T (w v) for this wave's value columns: U starts here
        if constexpr (K / 64 > 1) wyw_tile<K, V>(sm, rw * (K / 64) + K / 64 - 1, l16, q4);
        {
            const char *const b_vt = sm + (8 * q4 + (l16 >> 2)) * RV + 8 * (l16 & 3) + 2 * vbase;  // w v transpose reads
            const char *const b_c8 = sm + o_c8;
            for (int jt = 0; jt < NCT; ++jt) {
                bf16x8 bv[2];
                for (int ks = 0; ks < 2; ++ks) {
                    const int o = L::WV + 32 * ks * RV + 32 * jt;
                    bv[ks] = cat4(lds_tr(b_vt, o), lds_tr(b_vt, o + 4 * RV));
                }
                for (int i = 0; i < 4; ++i) {
                    f32x4 acc = {0, 0, 0, 0};
                    for (int ks = 0; ks <= (i >> 1); ++ks)
                        acc = mfma_bf16(lds_ld<bf16x8>(b_c8, L::TB + 16 * i * RC + 64 * ks), bv[ks], acc);
                    U[i][jt] = acc;
                }
            }
        }
        __syncthreads();  // ------------------------------------------ B5
    }

    if (ch.s1) {
        const int lane = tid & 63, rw = tid >> 6;
        const int l16 = lane & 15, q4 = lane >> 4;
        const int vbase = rw * VW;
        for (int it = 0; it < NRT; ++it)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e)
                    state_st(ch.s1, ch.s1_b16,
                             state_chan(it, q4, e) * (ch.s1_vm ? 1 : V) + (vbase + 16 * jt + l16) * (ch.s1_vm ? K : 1),
                             S[it][jt][e]);
    }
}

// ------------------------------------------------------------------ kernel --
template <int K, int V, int IO, bool G16, bool L2N, bool REC>
__global__ __launch_bounds__(NTHR) void chunk_fwd_kernel(FwdParams p)
{
    using L = Lds<K, V>;
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    const int tid = threadIdx.x;

    // work item: (sequence, value head), times the segment and, in the
    // transition pass, the kind (0: end state from the segment's entering
    // state or zero, 1: transition map from the identity with zero values)
    int item = blockIdx.x;
    const bool both = p.pass == PASS_TRANSITION && p.tonly == 0;
    const int kind = both ? item & 1 : p.pass == PASS_TRANSITION ? p.tonly - 1 : 0;
    if (both) item >>= 1;
    const int seg = p.seg_chunks ? item % p.nseg : 0;
    if (p.seg_chunks) item /= p.nseg;
    Chain ch;
    ch.n = item / p.HV;
    if constexpr (REC)  // (the backward's recompute only)
        if (p.grp && p.grp[ch.n] != p.gsel) return;  // the other launch's sequence
    ch.hv = item - ch.n * p.HV;
    ch.hk = ch.hv / (p.HV / p.H);
    const SeqRange sr = seq_of(p, ch.n);
    const int64_t sb = sr.b, se = sr.e;
    const int64_t shead = ((int64_t)ch.n * p.HV + ch.hv) * K * V;  // [N, HV, K, V] states
    ch.tb = sb;
    ch.te = se;
    ch.s0 = p.h0 ? state_at(p.h0, p.h0_bf16, shead) : nullptr;
    ch.s1 = p.ht ? state_at(p.ht, p.ht_bf16, shead) : nullptr;
    ch.s0_vm = ch.s1_vm = p.state_vmajor != 0;
    ch.s0_b16 = p.h0_bf16 != 0;
    ch.s1_b16 = p.ht_bf16 != 0;
    ch.ident = ch.zero_v = false;
    ch.out = p.out != nullptr;
    ch.ckpt = p.ckpt ? p.ckpt + (chunk_slot(sb, ch.n, 0) * p.HV + ch.hv) * (int64_t)(K * V) : nullptr;
    ch.rec = REC ? p.rec + (chunk_slot(sb, ch.n, 0) * p.HV + ch.hv) * bwd_prep_bytes(K) : nullptr;
    if (p.seg_chunks) {
        const int last = seg_last(sr, p.seg_chunks);
        if (seg > last) return;  // past the end of this sequence
        const int64_t span = (int64_t)p.seg_chunks * CH;
        ch.tb = sb + seg * span;
        ch.te = se < ch.tb + span ? se : ch.tb + span;
        // checkpoints and records of the segment's chunks (output pass)
        const int64_t skip = (int64_t)seg * p.seg_chunks * p.HV;
        if (ch.ckpt) ch.ckpt += skip * (K * V);
        if (ch.rec) ch.rec += skip * bwd_prep_bytes(K);
        const int64_t sseg = (((int64_t)ch.n * p.HV + ch.hv) * p.nseg + seg) * K * V;  // [N, HV, nseg, K, V]
        if (p.pass == PASS_TRANSITION) {
            // nothing follows the last segment; the first one's map is not needed
            if (seg >= last || (kind == 1 && seg == 0)) return;
            ch.out = false;
            ch.s1_vm = ch.s1_b16 = false;  // the workspace is K-major float32
            if (kind == 0) {
                if (seg > 0) ch.s0 = nullptr;
                ch.s1 = p.wb + sseg;
            } else {
                // the K x K map: this walk runs in the square kernel
                // (template V == K; a K != V run launches it for these
                // walks alone), so sseg strides K x K
                ch.s0 = nullptr;
                ch.ident = ch.zero_v = true;
                ch.s1 = p.wm + sseg;
            }
        } else {
            if (seg > 0) {
                ch.s0 = p.ws + sseg;
                ch.s0_vm = ch.s0_b16 = false;
            }
            if (seg < last) ch.s1 = nullptr;
        }
    }
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
    if (__builtin_amdgcn_readfirstlane(tid) >= NROLE) key_role<K, V, IO, G16, L2N, REC>(smem, p, ch, tid, nc);
    else state_role<K, V, IO, G16, L2N, REC>(smem, p, ch, tid, nc);
}

// ------------------------------------------------------ segment combine --
// The state pass is affine in the entering state, so a sequence cut into
// segments j = 0 .. last has S_{j+1} = M_j S_j + B_j, with B_j the end state
// of segment j from a zero start (from the true initial state for j = 0) and
// M_j its K x K transition. One workgroup per (sequence, value head, 16
// columns) applies the recurrence in float32 and stores every entering state
// S_j (j >= 1) for the output pass. The product M_j S_j runs on float32 MFMA
// (16x16x4): wave w owns the 16-row tiles w, w + 4 (K = 128) or w (K = 64)
// of the 16 columns, each an accumulator started at B_j. The sum over k is
// taken in the order k = q4 K/4 + kk (q4 the lane's k slot in an instruction,
// kk the instruction), so that a lane's operands for consecutive
// instructions are consecutive floats: M_j row-major and S_j transposed in
// LDS, both read 16 bytes at a time without bank conflicts. M_j goes to LDS
// once per workgroup, double-buffered: M_{j+1} and B_{j+1} are fetched while
// step j's products run, so a step costs one barrier and its products, not a
// memory round trip.
constexpr int CMB_COLS = 16;    // state columns per workgroup: one MFMA column tile
constexpr int CMB_THREADS = 256;  // four waves

template <int K>
struct CmbLds {
    static constexpr int P = K + 4;  // float pitch of a map row and of a transposed state column
    float m[2][K][P];                // M_j, row-major
    float st[2][CMB_COLS][P];        // S_j transposed: [column][row]
};

template <int K, int V>
__global__ __launch_bounds__(CMB_THREADS) void seg_combine_kernel(FwdParams p)
{
    constexpr int NT = CMB_THREADS, NL = K * K / 4 / NT;  // 16-byte pieces of a map per thread
    constexpr int RTW = K / 64;                           // 16-row tiles per wave
    constexpr int KQ = K / 4;                             // instructions per tile and step
    static_assert(K * K % (4 * NT) == 0 && V % CMB_COLS == 0 && K % 64 == 0, "combine tiling");
    __shared__ __attribute__((aligned(16))) CmbLds<K> L;
    const int ncb = V / CMB_COLS;
    const int chain = blockIdx.x / ncb, cb = blockIdx.x - chain * ncb;
    const int n = chain / p.HV;
    const int last = seg_last(seq_of(p, n), p.seg_chunks);
    if (last == 0) return;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, l16 = lane & 15, q4 = lane >> 4;
    const int64_t seg0 = (int64_t)chain * p.nseg * K * V;  // chain = n * HV + hv
    const int64_t map0 = (int64_t)chain * p.nseg * K * K;  // the maps: K x K each
    // this lane's elements (the MFMA result layout): rows row0[u] + e, e = 0..3,
    // column c of the block
    const int c = cb * CMB_COLS + l16;
    int row0[RTW];
    for (int u = 0; u < RTW; ++u) row0[u] = 16 * (w + 4 * u) + 4 * q4;
    // S_1 = B_0
    f32x4 s[RTW];
    for (int u = 0; u < RTW; ++u)
        for (int e = 0; e < 4; ++e) {
            const int64_t o = (int64_t)(row0[u] + e) * V + c;
            s[u][e] = p.wb[seg0 + o];
            p.ws[seg0 + (int64_t)K * V + o] = s[u][e];
        }
    if (last < 2) return;
    // M_1 and B_1
    f32x4 mr[NL], b[RTW];
    for (int i = 0; i < NL; ++i) mr[i] = *reinterpret_cast<const f32x4 *>(p.wm + map0 + (int64_t)K * K + 4 * (t + NT * i));
    for (int u = 0; u < RTW; ++u)
        for (int e = 0; e < 4; ++e) b[u][e] = p.wb[seg0 + (int64_t)K * V + (int64_t)(row0[u] + e) * V + c];
    for (int i = 0; i < NL; ++i) {
        const int x = 4 * (t + NT * i);
        *reinterpret_cast<f32x4 *>(&L.m[1][x / K][x % K]) = mr[i];
    }
    for (int j = 1; j < last; ++j) {
        const int bj = j & 1;
        for (int u = 0; u < RTW; ++u) *reinterpret_cast<f32x4 *>(&L.st[bj][l16][row0[u]]) = s[u];
        __syncthreads();  // M_j and S_j in LDS; step j - 1's reads of these buffers are done
        const bool more = j + 1 < last;
        f32x4 bn[RTW];
        for (int u = 0; u < RTW; ++u) bn[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (more) {
            for (int i = 0; i < NL; ++i)
                mr[i] = *reinterpret_cast<const f32x4 *>(p.wm + map0 + (int64_t)(j + 1) * K * K + 4 * (t + NT * i));
            for (int u = 0; u < RTW; ++u)
                for (int e = 0; e < 4; ++e)
                    bn[u][e] = p.wb[seg0 + (int64_t)(j + 1) * K * V + (int64_t)(row0[u] + e) * V + c];
        }
        // S_{j+1} = B_j + M_j S_j: lane (l16, q4) gives A = M[tile row l16][k]
        // and B = S[k][column l16] at k = q4 K/4 + kk
        f32x4 acc[RTW];
        for (int u = 0; u < RTW; ++u) acc[u] = b[u];
        const float *const sb = &L.st[bj][l16][q4 * KQ];
#pragma unroll 2
        for (int k4 = 0; k4 < KQ / 4; ++k4) {
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + 4 * k4);
            for (int u = 0; u < RTW; ++u) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(&L.m[bj][16 * (w + 4 * u) + l16][q4 * KQ + 4 * k4]);
                for (int e = 0; e < 4; ++e) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc[u], 0, 0, 0);
            }
        }
        for (int u = 0; u < RTW; ++u) {
            s[u] = acc[u];
            for (int e = 0; e < 4; ++e) p.ws[seg0 + (int64_t)(j + 1) * K * V + (int64_t)(row0[u] + e) * V + c] = s[u][e];
        }
        if (more)
            for (int i = 0; i < NL; ++i) {
                const int x = 4 * (t + NT * i);
                *reinterpret_cast<f32x4 *>(&L.m[bj ^ 1][x / K][x % K]) = mr[i];
            }
        for (int u = 0; u < RTW; ++u) b[u] = bn[u];
    }
}

}  // namespace

namespace {
// one instantiation per (K, V, io type, 16-bit g, L2 normalisation)
template <int K, int V, int IO, bool G16>
void launch_chunk_l2(const FwdParams &p, dim3 grid, hipStream_t stream)
{
    if (p.qk_l2norm) hipLaunchKernelGGL((chunk_fwd_kernel<K, V, IO, G16, true, false>), grid, dim3(NTHR), 0, stream, p);
    else hipLaunchKernelGGL((chunk_fwd_kernel<K, V, IO, G16, false, false>), grid, dim3(NTHR), 0, stream, p);
}
template <int K, int V>
void launch_chunk_typed(const FwdParams &p, dim3 grid, hipStream_t stream)
{
    const bool g16 = p.gtype != G_F32;
    if (p.io == IO_F16) {
        if (g16) launch_chunk_l2<K, V, IO_F16, true>(p, grid, stream);
        else launch_chunk_l2<K, V, IO_F16, false>(p, grid, stream);
    } else {
        if (g16) launch_chunk_l2<K, V, IO_BF16, true>(p, grid, stream);
        else launch_chunk_l2<K, V, IO_BF16, false>(p, grid, stream);
    }
}
}  // namespace

#ifdef GDN2_FWD_MIXED
// ----------------------------------------------- K != V translation unit --
// (also the backward's recompute at fp16 io or 16-bit g)
template <int D, int IO>
void launch_rec16(const FwdParams &p, dim3 grid, hipStream_t stream)
{
    if (p.gtype != G_F32) hipLaunchKernelGGL((chunk_fwd_kernel<D, D, IO, true, false, true>), grid, dim3(NTHR), 0, stream, p);
    else hipLaunchKernelGGL((chunk_fwd_kernel<D, D, IO, false, false, true>), grid, dim3(NTHR), 0, stream, p);
}

hipError_t launch_chunk_fwd_rec16(const FwdParams &p, unsigned grid, hipStream_t stream)
{
    if (!p.rec || (p.io == IO_BF16 && p.gtype == G_F32)) return hipErrorInvalidValue;
    if (p.K == 128 && p.io == IO_F16) launch_rec16<128, IO_F16>(p, dim3(grid), stream);
    else if (p.K == 128) launch_rec16<128, IO_BF16>(p, dim3(grid), stream);
    else if (p.K == 64 && p.io == IO_F16) launch_rec16<64, IO_F16>(p, dim3(grid), stream);
    else if (p.K == 64) launch_rec16<64, IO_BF16>(p, dim3(grid), stream);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_fwd_mixed(const FwdParams &p, unsigned grid, hipStream_t stream)
{
    if (p.rec || (p.pass == PASS_TRANSITION && p.tonly != 1)) return hipErrorInvalidValue;
    if (p.K == 128 && p.V == 64)
        launch_chunk_typed<128, 64>(p, dim3(grid), stream);
    else if (p.K == 64 && p.V == 128)
        launch_chunk_typed<64, 128>(p, dim3(grid), stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
#else
hipError_t launch_seg_combine(const FwdParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.N * p.HV * (p.V / CMB_COLS)));
    if (p.K == 128 && p.V == 128)
        hipLaunchKernelGGL((seg_combine_kernel<128, 128>), grid, dim3(CMB_THREADS), 0, stream, p);
    else if (p.K == 64 && p.V == 64)
        hipLaunchKernelGGL((seg_combine_kernel<64, 64>), grid, dim3(CMB_THREADS), 0, stream, p);
    else if (p.K == 128 && p.V == 64)
        hipLaunchKernelGGL((seg_combine_kernel<128, 64>), grid, dim3(CMB_THREADS), 0, stream, p);
    else if (p.K == 64 && p.V == 128)
        hipLaunchKernelGGL((seg_combine_kernel<64, 128>), grid, dim3(CMB_THREADS), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const FwdParams &p, hipStream_t stream)
{
    const int64_t items = (int64_t)p.N * p.HV * (p.seg_chunks ? p.nseg : 1);
    if (p.rec) {
        // the backward's recompute: K == V, no L2 normalisation; bf16 io with
        // float32 g here, the 16-bit combinations in the other translation unit
        if (p.qk_l2norm || !p.ckpt || p.pass != PASS_OUTPUT || p.K != p.V) return hipErrorInvalidValue;
        if (p.io != IO_BF16 || p.gtype != G_F32) return launch_chunk_fwd_rec16(p, (unsigned)items, stream);
        const dim3 grid((unsigned)items);
        if (p.K == 128)
            hipLaunchKernelGGL((chunk_fwd_kernel<128, 128, IO_BF16, false, false, true>), grid, dim3(NTHR), 0, stream, p);
        else if (p.K == 64)
            hipLaunchKernelGGL((chunk_fwd_kernel<64, 64, IO_BF16, false, false, true>), grid, dim3(NTHR), 0, stream, p);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (p.K != p.V) {
        if (p.pass != PASS_TRANSITION) return launch_chunk_fwd_mixed(p, (unsigned)items, stream);
        // a split run's transition pass: the end-state walks in the K x V
        // kernel, the K x K transition maps in the square one
        FwdParams p0 = p, p1 = p;
        p0.tonly = 1;
        p1.tonly = 2;
        const hipError_t e = launch_chunk_fwd_mixed(p0, (unsigned)items, stream);
        if (e != hipSuccess) return e;
        if (p.K == 128) launch_chunk_typed<128, 128>(p1, dim3((unsigned)items), stream);
        else launch_chunk_typed<64, 64>(p1, dim3((unsigned)items), stream);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(items * (p.pass == PASS_TRANSITION && p.tonly == 0 ? 2 : 1)));
    if (p.K == 128 && p.V == 128)
        launch_chunk_typed<128, 128>(p, grid, stream);
    else if (p.K == 64 && p.V == 64)
        launch_chunk_typed<64, 64>(p, grid, stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}
#endif

}  // namespace gdn2
