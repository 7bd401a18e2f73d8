// Backward of the GDN-2 chunked forward for CDNA4 (gfx950).
//
// Gradients of a scalar loss with respect to q, k, v, g, beta, w and the
// initial state, given the gradients of the output and of the final state.
// The chain rule is taken through the chunked WY form of the forward (per
// 64-token chunk, rows r, s; G = in-chunk cumulative sum of g per key
// channel; S_in the state entering the chunk, S_out the one leaving it):
//
//   QH = q e^G, KB = beta k e^G, RR = k e^-G, gamma = e^G_last, WV = w v
//   A = strict_tril(KB RR^T), P = tril(QH RR^T), T = (I + A)^-1
//   wy_w = T KB, wy_u = T WV, U = wy_u - wy_w S_in
//   O = scale (QH S_in + P U),  S_out = gamma S_in + (RR gamma)^T U
//
// (the chunked evaluation of the FlashInfer chunk_gated_delta_rule2
// recurrence display equation that the FlashRT card's 64-token WY chain and
// the burn-gdn2 README's "Fused CUDA kernels" section describe). Reversed:
//
//   dU    = scale P^T dO + RR (gamma dS_out)
//   dS_in = gamma dS_out + scale QH^T dO - wy_w^T dU
//   dQH   = scale dO S_in^T + dP RR,       dP = scale tril(dO U^T)
//   dKH   = U dS_out^T,  dgamma = rowsum(S_in dS_out) + colsum(dKH RR)
//   dwy_w = -dU S_in^T,  dT = dU WV^T + dwy_w KB^T,  dWV = T^T dU
//   dKB   = T^T dwy_w + dA RR,  dA = -strict_tril(T^T dT T^T)
//   dRR   = dA^T KB + dP^T QH + gamma dKH
//
// then through the decay factors to dq, dk, dbeta, dg (a reverse cumulative
// sum over the chunk) and through WV to dv, dw. Three launches follow the
// forward, which saves the state entering every chunk and every chunk's
// record (QH, RR, wy_w, KB, P, T, gamma):
//
//   state  (one workgroup per (sequence, value head), chunks in reverse)
//          the dS_in recurrence on MFMA, saving dS_out of every chunk
//   grads  (chunk-parallel)  every gradient of the chunk from its record,
//          the forward checkpoint S_in, the saved dS_out and dO
//   reduce dq, dk summed over the value heads of each q/k head
//
// Bounded decay: as in the forward's single-reference factorisation, every
// |G| (log2 units) of a chunk must stay within 2^120; a chunk beyond it
// (decided by the forward that writes the record, whose gamma is then NaN)
// has its gradients and, through gamma, the state gradient set to NaN.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gdn2_device.h"
#include "gdn2_internal.h"

namespace gdn2 {
namespace {

using namespace dev;

constexpr int CT = 512;  // threads per workgroup of the chunk-parallel kernels (8 waves)
constexpr int NW = CT / 64;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float XLIM = 120.0f;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// The record's gamma carries a flagged channel in its sign bit: the factor
// by which RR's column enters K-hat (gamma, or 1 where the column holds
// K-hat itself).
__device__ __forceinline__ f32x4 khat_factor(f32x4 g)
{
    f32x4 r;
    for (int e = 0; e < 4; ++e) r[e] = __builtin_signbit(g[e]) ? 1.0f : g[e];
    return r;
}

// Token range of sequence n (clamped into [0, T]).
__device__ __forceinline__ SeqRange seq_of(const BwdParams &p, int64_t n) { return seq_range(p.cu, p.cu64, p.T, n); }
// Element access in the caller's types: q, k, v, w, beta, d_out and their
// gradients in the io type (bf16 or fp16, p.io), g and dg in p.gtype
// (float32, bf16 or fp16). Wave-uniform branches on the kernel arguments.
__device__ __forceinline__ float io1_f32(uint16_t b, int io)
{
    return io == IO_F16 ? (float)__builtin_bit_cast(_Float16, b) : bf16_bits_to_f32(b);
}
__device__ __forceinline__ uint16_t f32_io1(float x, int io)
{
    return io == IO_F16 ? __builtin_bit_cast(uint16_t, (_Float16)x) : __builtin_bit_cast(uint16_t, (__bf16)x);
}
// 8 consecutive values (16 bytes, raw), widened to float32
__device__ __forceinline__ i32x4 ld_raw8(const uint16_t *p) { return *reinterpret_cast<const i32x4 *>(p); }
__device__ __forceinline__ f32x8 io8_f32(i32x4 raw, int io)
{
    return io == IO_F16 ? __builtin_convertvector(__builtin_bit_cast(f16x8, raw), f32x8)
                        : __builtin_convertvector(__builtin_bit_cast(bf16x8, raw), f32x8);
}
// the same values as a bf16 MFMA operand (exact for bf16 io, rounded for fp16)
__device__ __forceinline__ bf16x8 io8_bf16(i32x4 raw, int io)
{
    return io == IO_F16 ? f32x8_to_bf16(io8_f32(raw, io)) : __builtin_bit_cast(bf16x8, raw);
}
__device__ __forceinline__ void st_io8(uint16_t *p, f32x8 x, int io)
{
    if (io == IO_F16) *reinterpret_cast<f16x8 *>(p) = __builtin_convertvector(x, f16x8);
    else *reinterpret_cast<bf16x8 *>(p) = f32x8_to_bf16(x);
}
__device__ __forceinline__ float g_at(const BwdParams &p, int64_t i)
{
    if (p.gtype == G_F32) return static_cast<const float *>(p.g)[i];
    return io1_f32(static_cast<const uint16_t *>(p.g)[i], p.gtype == G_F16 ? IO_F16 : IO_BF16);
}
__device__ __forceinline__ void st_g4(const BwdParams &p, int64_t i, f32x4 x)
{
    if (p.gtype == G_F32) *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dg) + i) = x;
    else if (p.gtype == G_F16) *reinterpret_cast<f16x4 *>(static_cast<uint16_t *>(p.dg) + i) = __builtin_convertvector(x, f16x4);
    else *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(p.dg) + i) = __builtin_convertvector(x, bf16x4);
}

// One 16x16 tile Z[m0 + 4 q4 + e][n0 + l16] (element e of the result) of
// acc + X Y over k in [0, kd), X and Y bf16 in LDS at byte offsets xo, yo:
//   X[m][k] at xo + 2 (m lx + k)   (XT false: k contiguous)
//             xo + 2 (k lx + m)   (XT true: read with transpose reads)
//   Y[k][n] at yo + 2 (n ly + k)   (YT false: k contiguous)
//             yo + 2 (k ly + n)   (YT true: transpose reads)
// With yz, this lane's Y column (n0 + l16) is taken as zero.
template <bool XT, bool YT>
__device__ __forceinline__ f32x4 tile_mm(const char *sm, int xo, int lx, int yo, int ly, int m0, int n0, int kd,
                                         f32x4 acc, int l16, int q4, bool yz = false)
{
    for (int k0 = 0; k0 < kd; k0 += 32) {
        bf16x8 a, b;
        if constexpr (!XT) {
            a = lds_ld<bf16x8>(sm, xo + 2 * ((m0 + l16) * lx + k0 + 8 * q4));
        } else {
            const int o = xo + 2 * ((k0 + 8 * q4 + (l16 >> 2)) * lx + m0 + 4 * (l16 & 3));
            a = cat4(lds_tr(sm, o), lds_tr(sm, o + 8 * lx));
        }
        if constexpr (!YT) {
            b = lds_ld<bf16x8>(sm, yo + 2 * ((n0 + l16) * ly + k0 + 8 * q4));
        } else {
            const int o = yo + 2 * ((k0 + 8 * q4 + (l16 >> 2)) * ly + n0 + 4 * (l16 & 3));
            b = cat4(lds_tr(sm, o), lds_tr(sm, o + 8 * ly));
        }
        if (yz) b = bf16x8{};
        acc = mfma_bf16(a, b, acc);
    }
    return acc;
}

// MFMA operand from a bf16 row-major [D][D] matrix M in global memory:
// M[r0 + j][c] for j = 0..7 (8 rows of one column; a Y operand whose k runs
// down the rows), each row scaled by scl[r0 + j] if given.
__device__ __forceinline__ bf16x8 col_frag(const uint16_t *M, int ld, int r0, int c, const float *scl)
{
    f32x8 x;
    for (int j = 0; j < 8; ++j) x[j] = bf16_bits_to_f32(M[(int64_t)(r0 + j) * ld + c]) * (scl ? scl[r0 + j] : 1.0f);
    return f32x8_to_bf16(x);
}

// Store a tile (result layout) to an LDS matrix Z[m][n] at zo with pitch lz
// (bf16 or float32), each element scaled by s.
__device__ __forceinline__ void st_tile_bf(char *sm, int zo, int lz, int m0, int n0, f32x4 x, int l16, int q4)
{
    for (int e = 0; e < 4; ++e) lds_st<__bf16>(sm, zo + 2 * ((m0 + 4 * q4 + e) * lz + n0 + l16), (__bf16)x[e]);
}
__device__ __forceinline__ void st_tile_f32(char *sm, int zo, int lz, int m0, int n0, f32x4 x, int l16, int q4)
{
    for (int e = 0; e < 4; ++e) lds_st<float>(sm, zo + 4 * ((m0 + 4 * q4 + e) * lz + n0 + l16), x[e]);
}

// Keep entries with n < m (strict) or n <= m of a tile (m0, n0).
__device__ __forceinline__ f32x4 tril_mask(f32x4 x, int m0, int n0, bool strict, int l16, int q4)
{
    for (int e = 0; e < 4; ++e) {
        const int m = m0 + 4 * q4 + e, n = n0 + l16;
        x[e] = (strict ? n < m : n <= m) ? x[e] : 0.0f;
    }
    return x;
}

// Per-channel scans over a chunk's 64 rows, spread over all NT threads:
// thread (c = tid % D, part = tid / D) owns rows [RP part, RP part + RP) of
// channel c, RP = 64 D / NT; the parts' totals meet in an LDS scratch of
// [NT / D][D] floats at xo.
template <int D, int NT>
constexpr int scan_rows() { return 64 * D / NT; }

// This thread's rows of g (channel c, rows past the end of the sequence
// zero): 4-byte loads, consecutive lanes on consecutive channels.
template <int D, int NT, int RP = 64 * D / NT>
__device__ __forceinline__ void load_gcol(float (&v)[RP], const BwdParams &p, int64_t t0, int len, int hv, int tid)
{
    const int c = tid % D, r0 = (tid / D) * RP;
#pragma unroll
    for (int i = 0; i < RP; ++i)
        v[i] = r0 + i < len ? g_at(p, ((t0 + r0 + i) * p.HV + hv) * D + c) : 0.0f;
}

// G = cumsum(g) log2(e) per channel into float32 [64][D] (pitch D) at go,
// from load_gcol's values, and with gam >= 0 also 2^G_last [D] at gam.
// Returns whether |G| leaves the single-reference bound in this thread's
// rows. The caller synchronises before reading G or 2^G_last.
// With skip >= 0, channels whose int at skip + 4 c is nonzero are not
// stored (their slots are written by the caller).
template <int D, int NT, int RP = 64 * D / NT>
__device__ __forceinline__ bool scan_gcol(char *sm, int go, int xo, int gam, const float (&v)[RP], int tid,
                                          int skip = -1)
{
    constexpr int NP = NT / D;
    const int c = tid % D, part = tid / D;
    float loc[RP];
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < RP; ++i) loc[i] = run = fmaf(v[i], LOG2E, run);
    lds_st<float>(sm, xo + 4 * (part * D + c), run);
    __syncthreads();
    float off = 0.0f;
    for (int q = 0; q < NP; ++q)
        if (q < part) off += lds_ld<float>(sm, xo + 4 * (q * D + c));
    bool out = false;
    const bool keep = skip < 0 || lds_ld<int>(sm, skip + 4 * c) == 0;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const float G = loc[i] + off;
        out |= !(fabsf(G) <= XLIM);
        if (keep) lds_st<float>(sm, go + 4 * ((part * RP + i) * D + c), G);
    }
    if (gam >= 0 && part == NP - 1) lds_st<float>(sm, gam + 4 * c, ex2(loc[RP - 1] + off));
    return out;
}

// x[r][c] <- init[c] + sum_{s >= r} x[s][c] in place (float32, pitch ld
// floats, at xb): the reverse cumulative sum over the chunk.
template <int D, int NT>
__device__ __forceinline__ void rscan_rows(char *sm, int xb, int ld, int xo, float init, int tid)
{
    constexpr int RP = scan_rows<D, NT>(), NP = NT / D;
    const int c = tid % D, part = tid / D;
    float loc[RP];
    float run = 0.0f;
#pragma unroll
    for (int i = RP - 1; i >= 0; --i) loc[i] = run = run + lds_ld<float>(sm, xb + 4 * ((part * RP + i) * ld + c));
    lds_st<float>(sm, xo + 4 * (part * D + c), run);
    __syncthreads();
    float off = init;
    for (int q = NP - 1; q >= 0; --q)
        if (q > part) off += lds_ld<float>(sm, xo + 4 * (q * D + c));
#pragma unroll
    for (int i = 0; i < RP; ++i) lds_st<float>(sm, xb + 4 * ((part * RP + i) * ld + c), loc[i] + off);
}

// ------------------------------------------------------------ LDS layout --
// Regions of the chunk kernels (K = V = D); lifetimes by phase noted.
template <int D>
struct BL {
    static constexpr int RK = D + 8;   // bf16 pitch of [64][D]
    static constexpr int RC = 64 + 8;  // bf16 pitch of [64][64]
    static constexpr int RF = D + 4;   // float32 pitch of [64][D]
    static constexpr int TK = 64 * RK * 2, TC = 64 * RC * 2;
    static constexpr int QH = 0, KB = QH + TK, RR = KB + TK;  // all phases
    static constexpr int RGA = RR + TK;           // U; WV again; Y
    static constexpr int RGB = RGA + TK;          // WV; dO; dT, then dA
    static constexpr int RGC = RGB + TK;          // wy_w; dU
    static constexpr int RGD = RGC + TK;          // dwy_w
    static constexpr int PB = RGD + TK;           // P; dP
    static constexpr int TB = PB + TC;            // T (bf16)
    static constexpr int GAM = TB + TC;           // e^G_last [D] float32
    static constexpr int GMU = GAM + 4 * D;       // [D]: K-hat = RR GMU per channel (gamma, 1 if flagged)
    static constexpr int FLC = GMU + 4 * D;       // int [D]: 1 for a flagged channel (strong decay)
    static constexpr int XLS = FLC + 4 * D;       // int [D]: the flagged channels in order
    static constexpr int CSL = XLS + 4 * D;       // int [D]: a flagged channel's place in XLS
    static constexpr int DGM = CSL + 4 * D;       // rowsum(S_in dS_out) [D] float32
    static constexpr int DGP = DGM + 4 * D;       // colsum(dKH RR) per row group [2][D] float32
    static constexpr int XS = DGP + 8 * D;        // per-channel scans: the parts' totals [CT / D][D] float32
    static constexpr int FLG = XS + 4 * CT;       // int: any flagged channel; then (int) their number
    static constexpr int DWV = FLG + 16;          // dWV bf16 [64][D] (pitch D), for the epilogue's dv, dw
    // flagged channels' exact pass, NXB channels at a time: G, q, k, beta
    // float32 [4][NXB][64] in RGA; alpha, pi, kappa float32 [3][NXB][64] in RGC
    static constexpr int NXB = D / 8;
    static constexpr int TOTAL = DWV + 64 * D * 2;
    static constexpr int EF = 64 * RF * 4;        // epilogue: dQH, dKB, dRR, G float32 [64][RF]
    static constexpr int SIZE = cmax(TOTAL, 4 * EF);
    static_assert(TK >= TC, "[64][64] tiles in [64][D] regions");
    static_assert(4 * EF <= GAM, "the epilogue leaves GAM .. FLG intact");
    static_assert(4 * NXB * 64 * 4 <= TK && 3 * NXB * 64 * 4 <= TK, "exact pass in RGA, RGC");
    static_assert(RGC + 3 * NXB * 64 * 4 <= 3 * EF, "exact results below the epilogue's G tile");
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

// The 20 lower tiles (i >= j) of A (0..9) and P (10..19) of a chunk.
__device__ __forceinline__ void lower_tile(int t, int &i, int &j)
{
    const int u = t % 10;  // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
    i = u >= 6 ? 3 : u >= 3 ? 2 : u >= 1 ? 1 : 0;
    j = u - i * (i + 1) / 2;
}

// ------------------------------------------------------ flagged channels --
// A flagged channel (strong decay: |G| beyond the single-reference range in
// this chunk; the forward's record marks it with a negated gamma) took no part in
// the RR products: its share of A and P is exact per pair of rows. With
// E_rs = 2^(G_r - G_s) (G in log2 units, so E_rs = e^(G_r - G_s) in natural
// units), the share of the gradients is
//   alpha_r = sum_{s <= r} dA_rs k_s E_rs      -> d(beta k)_r
//   pi_r    = sum_{s <= r} dP_rs k_s E_rs      -> dq_r
//   kappa_r = sum_{r' >= r} (dA_r'r (beta k)_r' + dP_r'r q_r') E_r'r -> dk_r
//   dG_r   += (beta k)_r alpha_r + q_r pi_r - k_r kappa_r
// (dA is strictly and dP inclusively lower triangular, so the diagonal terms
// are the right ones). This pass takes channels b0 .. b0 + nb - 1 of the
// list XLS: it stages their G, q, k, beta in RGA (float32 [4][NXB][64]) and
// leaves alpha, pi, kappa in RGC (float32 [3][NXB][64]). Every thread takes
// part; it ends synchronised.
template <int D>
__device__ __forceinline__ void exact_pass(char *sm, const BwdParams &p, int64_t t0, int len, int hk, int hv, int b0,
                                           int nb, int tid)
{
    using L = BL<D>;
    constexpr int NXB = L::NXB, TPX = CT / NXB, RPX = 64 / TPX;  // threads per channel, rows per thread
    constexpr int A = 4 * 64 * NXB;                              // bytes per staged array
    const int x = tid / TPX, part = tid % TPX;
    const bool on = x < nb;
    const int c = on ? lds_ld<int>(sm, L::XLS + 4 * (b0 + x)) : 0;
    const int sx = L::RGA + 4 * 64 * x;  // this channel's staged rows
    float gl[RPX], run = 0.0f;
#pragma unroll
    for (int h = 0; h < RPX; ++h) {
        const int r = RPX * part + h;
        const bool ok = on && r < len;
        const int64_t tr = t0 + r;
        run += ok ? g_at(p, (tr * p.HV + hv) * D + c) * LOG2E : 0.0f;
        gl[h] = run;
        const float qv = ok ? io1_f32(p.q[(tr * p.H + hk) * D + c], p.io) : 0.0f;
        const float kv = ok ? io1_f32(p.k[(tr * p.H + hk) * D + c], p.io) : 0.0f;
        const float bv = ok ? io1_f32(p.beta[(tr * p.HV + hv) * D + c], p.io) : 0.0f;
        lds_st<float>(sm, sx + 1 * A + 4 * r, qv);
        lds_st<float>(sm, sx + 2 * A + 4 * r, kv);
        lds_st<float>(sm, sx + 3 * A + 4 * r, bv);
    }
    // inclusive cumulative sum over the channel's TPX threads
    float inc = run;
    for (int d = 1; d < TPX; d <<= 1) {
        const float o = __shfl_up(inc, d, TPX);
        if (part >= d) inc += o;
    }
#pragma unroll
    for (int h = 0; h < RPX; ++h) lds_st<float>(sm, sx + 4 * (RPX * part + h), gl[h] + inc - run);
    __syncthreads();
    // alpha and pi of row r run over s <= r, kappa over r' >= r: one term
    // of each kind per pair
    auto ap_term = [&](int r, float Gr, int s2, float &al, float &pi) {
        const float ke = lds_ld<float>(sm, sx + 2 * A + 4 * s2) * ex2(Gr - lds_ld<float>(sm, sx + 4 * s2));
        al = fmaf((float)lds_ld<__bf16>(sm, L::RGB + 2 * (r * L::RC + s2)), ke, al);
        pi = fmaf((float)lds_ld<__bf16>(sm, L::PB + 2 * (r * L::RC + s2)), ke, pi);
    };
    auto k_term = [&](int r, float Gr, int r2, float &ka) {
        const float e = ex2(lds_ld<float>(sm, sx + 4 * r2) - Gr);
        const float bk = lds_ld<float>(sm, sx + 3 * A + 4 * r2) * lds_ld<float>(sm, sx + 2 * A + 4 * r2);
        const float w = (float)lds_ld<__bf16>(sm, L::RGB + 2 * (r2 * L::RC + r)) * bk +
                        (float)lds_ld<__bf16>(sm, L::PB + 2 * (r2 * L::RC + r)) * lds_ld<float>(sm, sx + 1 * A + 4 * r2);
        ka = fmaf(w, e, ka);
    };
    auto put = [&](int r, float al, float pi, float ka) {
        const int ro = L::RGC + 4 * (64 * x + r);
        lds_st<float>(sm, ro, al);
        lds_st<float>(sm, ro + A, pi);
        lds_st<float>(sm, ro + 2 * A, ka);
    };
    if constexpr (RPX == 2) {
        // rows rl = part and rh = 63 - part. The sums of rl over s <= rl and
        // of rh over r' >= rh both have part + 1 terms, those of rl over
        // r' >= rl and of rh over s <= rh both 64 - part: each pair of sums
        // shares one loop (every sum keeps its order of terms), so a wave
        // runs 96 iterations instead of 192
        const int rl = part, rh = 63 - part;
        const float Gl = lds_ld<float>(sm, sx + 4 * rl), Gh = lds_ld<float>(sm, sx + 4 * rh);
        float al_l = 0.0f, pi_l = 0.0f, ka_l = 0.0f, al_h = 0.0f, pi_h = 0.0f, ka_h = 0.0f;
        for (int i = 0; i <= part; ++i) {
            ap_term(rl, Gl, i, al_l, pi_l);
            k_term(rh, Gh, rh + i, ka_h);
        }
        for (int i = 0; i < 64 - part; ++i) {
            k_term(rl, Gl, rl + i, ka_l);
            ap_term(rh, Gh, i, al_h, pi_h);
        }
        put(rl, al_l, pi_l, ka_l);
        put(rh, al_h, pi_h, ka_h);
    } else {
        const int r = part;
        const float Gr = lds_ld<float>(sm, sx + 4 * r);
        float al = 0.0f, pi = 0.0f, ka = 0.0f;
        for (int s2 = 0; s2 <= r; ++s2) ap_term(r, Gr, s2, al, pi);
        for (int r2 = r; r2 < 64; ++r2) k_term(r, Gr, r2, ka);
        put(r, al, pi, ka);
    }
    __syncthreads();
}

// ----------------------------------------------------- chunk-parallel kernel --
// Every gradient of one chunk, from its record, its checkpoints and its
// inputs.
template <int D>
__global__ __launch_bounds__(CT) void bwd_chunk_kernel(BwdParams p)
{
    using L = BL<D>;
    constexpr int RK = L::RK, RC = L::RC;
    constexpr int NTD = D / 16;      // 16-wide tiles across D
    constexpr int NMG = NW / NTD;    // waves per column tile
    constexpr int MPW = 4 / NMG;     // row tiles per wave
    static_assert(NW % NTD == 0 && 4 % NMG == 0, "tile split");
    constexpr int NU8 = 64 * D / 8 / CT;  // 16-byte row pieces per thread of a [64][D] bf16 tile
    __shared__ __attribute__((aligned(16))) char sm[L::SIZE];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
    // the [64][D] products' tiles of this wave: column tile ni, row tiles
    // mg, mg + NMG, ...
    const int ni = wv % NTD, mg = wv / NTD;

    // work item: (checkpoint slot, value head); the slot's sequence is the
    // last one whose first slot is not past it
    const int hv = blockIdx.x % p.HV;
    const int64_t slot = blockIdx.x / p.HV;
    int n;
    int64_t c;
    if (!slot_owner(p.cu, p.cu64, p.T, p.N, slot, &n, &c)) return;  // no chunk in this slot
    if (p.grp && p.grp[n] != p.gsel) return;  // the other launch's sequence
    const SeqRange sr = seq_of(p, n);
    const int64_t sb = sr.b, se = sr.e;
    const int64_t t0 = sb + c * 64;
    const int len = (int)(se - t0 < 64 ? se - t0 : 64);
    const int hk = hv / (p.HV / p.H);
    const int64_t kd_off = (int64_t)(slot * p.HV + hv) * D * D;  // checkpoint of this chunk

    {
        // ---- the chunk's record (QH, KB, RR, wy_w in RGC, P, T, gamma; a
        // chunk beyond the decay bound has gamma = NaN), and WV (bf16 in RGB)
        constexpr PrepRecord R{D};
        const char *rec = p.prep + (slot * p.HV + hv) * bwd_prep_bytes(D);
        // dO (bf16 [token][D]; rows past the end zero) rides along with the
        // record; it goes to LDS once WV is no longer needed there
        i32x4 xdo[NU8];
        i32x4 vr[NU8], wr[NU8];  // raw v, w rows: WV again and the epilogue's dv, dw
        {
            bf16x8 x[4][NU8], xpt[2];
            const int src[4] = {R.qh(), R.kb(), R.rr(), R.wy()};
#pragma unroll
            for (int u = 0; u < NU8; ++u) {
                const int e = tid + CT * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
#pragma unroll
                for (int m = 0; m < 4; ++m) x[m][u] = *reinterpret_cast<const bf16x8 *>(rec + src[m] + 2 * (r * D + c0));
                const int64_t tv = ((t0 + r) * p.HV + hv) * D + c0;
                vr[u] = r < len ? ld_raw8(p.v + tv) : i32x4{};
                wr[u] = r < len ? ld_raw8(p.w + tv) : i32x4{};
                xdo[u] = r < len ? ld_raw8(p.dout + tv) : i32x4{};
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {  // P, then T: 512 16-byte pieces each, one per thread
                const int r = tid >> 3, c0 = 8 * (tid & 7);
                xpt[m] = *reinterpret_cast<const bf16x8 *>(rec + (m ? R.t() : R.p()) + 2 * (r * 64 + c0));
            }
            const float xg = tid < D ? *reinterpret_cast<const float *>(rec + R.gam() + 4 * tid) : 0.0f;
            if (tid == 0) lds_st<int>(sm, L::FLG, 0);
            __syncthreads();
            const int dst[4] = {L::QH, L::KB, L::RR, L::RGC};
#pragma unroll
            for (int u = 0; u < NU8; ++u) {
                const int e = tid + CT * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
#pragma unroll
                for (int m = 0; m < 4; ++m) lds_st<bf16x8>(sm, dst[m] + 2 * (r * RK + c0), x[m][u]);
                lds_st<bf16x8>(sm, L::RGB + 2 * (r * RK + c0), f32x8_to_bf16(io8_f32(vr[u], p.io) * io8_f32(wr[u], p.io)));
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int r = tid >> 3, c0 = 8 * (tid & 7);
                lds_st<bf16x8>(sm, (m ? L::TB : L::PB) + 2 * (r * RC + c0), xpt[m]);
            }
            if (tid < D) {
                const bool fl = __builtin_signbit(xg);
                lds_st<float>(sm, L::GAM + 4 * tid, fabsf(xg));
                lds_st<float>(sm, L::GMU + 4 * tid, fl ? 1.0f : xg);
                lds_st<int>(sm, L::FLC + 4 * tid, fl ? 1 : 0);
                if (fl) lds_st<int>(sm, L::FLG, 1);
            }
            __syncthreads();
        }
        const bool flagged = lds_ld<int>(sm, L::FLG) != 0;  // workgroup-uniform
        const uint16_t *Sin = p.s_ckpt + kd_off;  // bf16 checkpoints
        const uint16_t *dSo = p.ds_ckpt + kd_off;
        const float *gmu = reinterpret_cast<const float *>(sm + L::GMU);

        // ---- U = T WV - wy_w S_in (bf16 [token][D] in RGA); wave wv takes
        // its column tile ni and row tiles mg, mg + NMG, ...
        {
            f32x4 wu[MPW], ws[MPW];
            for (int u = 0; u < MPW; ++u) {
                const int mi = mg + NMG * u;
                wu[u] = tile_mm<false, true>(sm, L::TB, RC, L::RGB, RK, 16 * mi, 16 * ni, 64, f32x4{0, 0, 0, 0}, l16, q4);
                ws[u] = f32x4{0, 0, 0, 0};
            }
            bf16x8 fr[D / 32];
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) fr[ks] = col_frag(Sin, D, 32 * ks + 8 * q4, 16 * ni + l16, nullptr);
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                for (int u = 0; u < MPW; ++u) {
                    const int mi = mg + NMG * u;
                    ws[u] = mfma_bf16(lds_ld<bf16x8>(sm, L::RGC + 2 * ((16 * mi + l16) * RK + 32 * ks + 8 * q4)), fr[ks], ws[u]);
                }
            for (int u = 0; u < MPW; ++u) st_tile_bf(sm, L::RGA, RK, 16 * (mg + NMG * u), 16 * ni, wu[u] - ws[u], l16, q4);
        }
        __syncthreads();

        // ---- dO to LDS (RGB)
#pragma unroll
        for (int u = 0; u < NU8; ++u) {
            const int e = tid + CT * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            lds_st<bf16x8>(sm, L::RGB + 2 * (r * RK + c0), io8_bf16(xdo[u], p.io));
        }
        __syncthreads();

        // ---- dU = scale P^T dO + RR (GMU dS_out) (bf16 in RGC), and
        // dKH = U dS_out^T (registers: the wave's tiles)
        f32x4 dKH[MPW], dQH[MPW], dKB[MPW], dRR[MPW];
        bf16x8 fs[D / 32];  // S_in row fragments, for dQH and dwy_w below
        {
            bf16x8 fr[D / 32], fc[D / 32];
            // row 16 ni + l16 of dS_out and of S_in, columns 32 ks + 8 q4 .. + 7:
            // MFMA operands as stored (bf16), and dgamma's direct part
            // rowsum(S_in dS_out) in float32 (lanes q4 = 0..3 of a row
            // together cover it; the waves of one column tile hold the same
            // rows, the first stores)
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const int64_t o = (int64_t)(16 * ni + l16) * D + 32 * ks + 8 * q4;
                fc[ks] = *reinterpret_cast<const bf16x8 *>(dSo + o);
                fs[ks] = *reinterpret_cast<const bf16x8 *>(Sin + o);
            }
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) fr[ks] = col_frag(dSo, D, 32 * ks + 8 * q4, 16 * ni + l16, gmu);
            float sdot = 0.0f;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const f32x8 a = __builtin_convertvector(fs[ks], f32x8), b = __builtin_convertvector(fc[ks], f32x8);
                for (int j = 0; j < 8; ++j) sdot = fmaf(a[j], b[j], sdot);
            }
            sdot += __shfl_xor(sdot, 16);
            sdot += __shfl_xor(sdot, 32);
            if (mg == 0 && q4 == 0) lds_st<float>(sm, L::DGM + 4 * (16 * ni + l16), sdot);
            f32x4 acc[MPW];
            for (int u = 0; u < MPW; ++u)
                acc[u] = tile_mm<true, true>(sm, L::PB, RC, L::RGB, RK, 16 * (mg + NMG * u), 16 * ni, 64, f32x4{0, 0, 0, 0}, l16,
                                             q4) * p.scale;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                for (int u = 0; u < MPW; ++u) {
                    const int mi = mg + NMG * u;
                    acc[u] = mfma_bf16(lds_ld<bf16x8>(sm, L::RR + 2 * ((16 * mi + l16) * RK + 32 * ks + 8 * q4)), fr[ks], acc[u]);
                }
            for (int u = 0; u < MPW; ++u) st_tile_bf(sm, L::RGC, RK, 16 * (mg + NMG * u), 16 * ni, acc[u], l16, q4);
            // dKH[r][c] = sum_v U[r][v] dS_out[c][v]
            for (int u = 0; u < MPW; ++u) dKH[u] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                for (int u = 0; u < MPW; ++u) {
                    const int mi = mg + NMG * u;
                    dKH[u] = mfma_bf16(lds_ld<bf16x8>(sm, L::RGA + 2 * ((16 * mi + l16) * RK + 32 * ks + 8 * q4)), fc[ks], dKH[u]);
                }
        }
        __syncthreads();

        // ---- dQH = scale dO S_in^T (registers), dwy_w = -dU S_in^T (bf16 in RGD)
        {
            f32x4 acc[MPW];
            for (int u = 0; u < MPW; ++u) dQH[u] = acc[u] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                for (int u = 0; u < MPW; ++u) {
                    const int o = 2 * ((16 * (mg + NMG * u) + l16) * RK + 32 * ks + 8 * q4);
                    dQH[u] = mfma_bf16(lds_ld<bf16x8>(sm, L::RGB + o), fs[ks], dQH[u]);
                    acc[u] = mfma_bf16(lds_ld<bf16x8>(sm, L::RGC + o), fs[ks], acc[u]);
                }
            for (int u = 0; u < MPW; ++u) {
                dQH[u] *= p.scale;
                st_tile_bf(sm, L::RGD, RK, 16 * (mg + NMG * u), 16 * ni, -acc[u], l16, q4);
            }
        }
        __syncthreads();

        // ---- dP = scale tril(dO U^T) (bf16 over P)
        for (int t = wv; t < 10; t += NW) {
            int i, j;
            lower_tile(t, i, j);
            const f32x4 x = tile_mm<false, false>(sm, L::RGB, RK, L::RGA, RK, 16 * i, 16 * j, D, f32x4{0, 0, 0, 0}, l16, q4);
            st_tile_bf(sm, L::PB, RC, 16 * i, 16 * j, tril_mask(x, 16 * i, 16 * j, false, l16, q4) * p.scale, l16, q4);
        }
        __syncthreads();

        // ---- WV again (bf16 in RGA), from the v and w rows held in registers
        // since the record load (no second read of either)
        {
#pragma unroll
            for (int u = 0; u < NU8; ++u) {
                const int e = tid + CT * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
                lds_st<bf16x8>(sm, L::RGA + 2 * (r * RK + c0), f32x8_to_bf16(io8_f32(vr[u], p.io) * io8_f32(wr[u], p.io)));
            }
        }
        __syncthreads();

        // ---- dT = strict_tril(dU WV^T + dwy_w KB^T) (bf16 in RGB, all 16 tiles)
        for (int t = wv; t < 16; t += NW) {
            const int i = t >> 2, j = t & 3;
            f32x4 x = tile_mm<false, false>(sm, L::RGC, RK, L::RGA, RK, 16 * i, 16 * j, D, f32x4{0, 0, 0, 0}, l16, q4);
            x = tile_mm<false, false>(sm, L::RGD, RK, L::KB, RK, 16 * i, 16 * j, D, x, l16, q4);
            st_tile_bf(sm, L::RGB, RC, 16 * i, 16 * j, tril_mask(x, 16 * i, 16 * j, true, l16, q4), l16, q4);
        }
        // ---- dWV = T^T dU (bf16 in DWV: dv = dWV w and dw = dWV v are formed
        // row-parallel in the epilogue); dKB = T^T dwy_w
#pragma unroll
        for (int u = 0; u < MPW; ++u) {
            const int mi = mg + NMG * u;
            const f32x4 x = tile_mm<true, true>(sm, L::TB, RC, L::RGC, RK, 16 * mi, 16 * ni, 64, f32x4{0, 0, 0, 0}, l16, q4);
            st_tile_bf(sm, L::DWV, D, 16 * mi, 16 * ni, x, l16, q4);
            dKB[u] = tile_mm<true, true>(sm, L::TB, RC, L::RGD, RK, 16 * mi, 16 * ni, 64, f32x4{0, 0, 0, 0}, l16, q4);
        }
        __syncthreads();

        // ---- Y = T^T dT (bf16 in RGA), then dA = -strict_tril(Y T^T) (bf16 in RGB)
        for (int t = wv; t < 16; t += NW) {
            const int i = t >> 2, j = t & 3;
            const f32x4 x = tile_mm<true, true>(sm, L::TB, RC, L::RGB, RC, 16 * i, 16 * j, 64, f32x4{0, 0, 0, 0}, l16, q4);
            st_tile_bf(sm, L::RGA, RC, 16 * i, 16 * j, x, l16, q4);
        }
        __syncthreads();
        for (int t = wv; t < 16; t += NW) {
            const int i = t >> 2, j = t & 3;
            const f32x4 x = tile_mm<false, false>(sm, L::RGA, RC, L::TB, RC, 16 * i, 16 * j, 64, f32x4{0, 0, 0, 0}, l16, q4);
            st_tile_bf(sm, L::RGB, RC, 16 * i, 16 * j, -tril_mask(x, 16 * i, 16 * j, true, l16, q4), l16, q4);
        }
        __syncthreads();

        // ---- dKB += dA RR; dRR = dA^T KB + dP^T QH; dQH += dP RR (with this
        // chunk's g issued first: the epilogue's cumulative sum needs it)
        float gv[scan_rows<D, CT>()];
        load_gcol<D, CT>(gv, p, t0, len, hv, tid);
        // a flagged channel's RR column holds K-hat: not an operand here
        const int colc = 16 * ni + l16;
        const bool fcol = flagged && lds_ld<int>(sm, L::FLC + 4 * colc) != 0;
        for (int u = 0; u < MPW; ++u) {
            const int mi = mg + NMG * u;
            dKB[u] = tile_mm<false, true>(sm, L::RGB, RC, L::RR, RK, 16 * mi, 16 * ni, 64, dKB[u], l16, q4, fcol);
            f32x4 x = tile_mm<true, true>(sm, L::RGB, RC, L::KB, RK, 16 * mi, 16 * ni, 64, f32x4{0, 0, 0, 0}, l16, q4);
            dRR[u] = tile_mm<true, true>(sm, L::PB, RC, L::QH, RK, 16 * mi, 16 * ni, 64, x, l16, q4);
            dQH[u] = tile_mm<false, true>(sm, L::PB, RC, L::RR, RK, 16 * mi, 16 * ni, 64, dQH[u], l16, q4, fcol);
        }
        __syncthreads();

        // ---- flagged channels: the exact pass, NXB at a time, folded into
        // this wave's tiles of a flagged column as the final dq (dQH), dbeta
        // (dKB), dk (dRR) and dG (dGf): the products above and dKH (K-hat
        // is the record's RR column there) give the rest
        f32x4 dGf[MPW];
        if (flagged) {
            if (wv == 0) {  // the flagged channels in order
                int cnt = 0;
                for (int cb = 0; cb < D; cb += 64) {
                    const int c = cb + lane;
                    const bool f = lds_ld<int>(sm, L::FLC + 4 * c) != 0;
                    const uint64_t m = __ballot(f);
                    if (f) {
                        const int pos = cnt + __popcll(m & ((1ull << lane) - 1));
                        lds_st<int>(sm, L::XLS + 4 * pos, c);
                        lds_st<int>(sm, L::CSL + 4 * c, pos);
                    }
                    cnt += __popcll(m);
                }
                if (lane == 0) lds_st<int>(sm, L::FLG, cnt);
            }
            __syncthreads();
            const int nx = lds_ld<int>(sm, L::FLG);
            const int mypos = fcol ? lds_ld<int>(sm, L::CSL + 4 * colc) : -1;
            constexpr int A = 4 * 64 * L::NXB;
            for (int b0 = 0; b0 < nx; b0 += L::NXB) {
                const int nb = nx - b0 < L::NXB ? nx - b0 : L::NXB;
                exact_pass<D>(sm, p, t0, len, hk, hv, b0, nb, tid);
                if (mypos >= b0 && mypos < b0 + nb) {
                    const int sx = L::RGA + 4 * 64 * (mypos - b0), rx = L::RGC + 4 * 64 * (mypos - b0);
                    const float Gl = lds_ld<float>(sm, sx + 4 * 63);
                    for (int u = 0; u < MPW; ++u)
                        for (int e = 0; e < 4; ++e) {
                            const int r = 16 * (mg + NMG * u) + 4 * q4 + e;
                            const float Gr = lds_ld<float>(sm, sx + 4 * r);
                            const float qq = lds_ld<float>(sm, sx + A + 4 * r), kk = lds_ld<float>(sm, sx + 2 * A + 4 * r);
                            const float bb = lds_ld<float>(sm, sx + 3 * A + 4 * r);
                            const float al = lds_ld<float>(sm, rx + 4 * r), pi = lds_ld<float>(sm, rx + A + 4 * r);
                            const float ka = lds_ld<float>(sm, rx + 2 * A + 4 * r);
                            const int ro = 2 * (r * RK + colc);
                            const float qh = (float)lds_ld<__bf16>(sm, L::QH + ro), kb = (float)lds_ld<__bf16>(sm, L::KB + ro);
                            const float kh = (float)lds_ld<__bf16>(sm, L::RR + ro);
                            const float eg = ex2(Gr), gq = dQH[u][e], gkb = dKB[u][e], dkh = dKH[u][e];
                            dQH[u][e] = gq * eg + pi;
                            dKB[u][e] = (gkb * eg + al) * kk;
                            dRR[u][e] = (gkb * eg + al) * bb + ka + dkh * ex2(Gl - Gr);
                            dGf[u][e] = gq * qh + gkb * kb + bb * kk * al + qq * pi - kk * ka - dkh * kh;
                        }
                }
                __syncthreads();  // the batch's staging and results are consumed
            }
        }

        // ---- epilogue. dKH enters as K-hat = RR gamma: dRR += gamma dKH and
        // dgamma += colsum(dKH RR), the latter reduced over the wave's rows
        // (each channel column belongs to one wave) onto rowsum(S_in dS_out).
        // (A flagged channel: K-hat is the RR column itself, so G_last gets
        // colsum(dKH RR) with factor 1 and dk its share from the fold.)
        // The decay factors' share of dG pairs each product's gradient with
        // the very bf16 factors that product used, the record's QH, KB and
        // RR: a pair (r, s) adds to dG_r and subtracts from dG_s the same
        // amount, and with other roundings these would no longer cancel in
        // the reverse cumulative sum under strong decay.
        {
            const int col = 16 * ni + l16;
            const float gc = lds_ld<float>(sm, L::GAM + 4 * col);
            float part = 0.0f;
            for (int u = 0; u < MPW; ++u)
                for (int e = 0; e < 4; ++e) {
                    part += dKH[u][e] * (float)lds_ld<__bf16>(sm, L::RR + 2 * ((16 * (mg + NMG * u) + 4 * q4 + e) * RK + col));
                    if (!fcol) dRR[u][e] += gc * dKH[u][e];
                }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            // one partial per (row group, column), summed in a fixed order
            // below (deterministic)
            if (q4 == 0) lds_st<float>(sm, L::DGP + 4 * (mg * D + col), part);
        }
        // the record's QH, KB, RR at this thread's row pieces, read before
        // the float32 tiles below overwrite them
        bf16x8 xq[NU8], xk[NU8], xr[NU8];
#pragma unroll
        for (int u = 0; u < NU8; ++u) {
            const int e = tid + CT * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            xq[u] = lds_ld<bf16x8>(sm, L::QH + 2 * (r * RK + c0));
            xk[u] = lds_ld<bf16x8>(sm, L::KB + 2 * (r * RK + c0));
            xr[u] = lds_ld<bf16x8>(sm, L::RR + 2 * (r * RK + c0));
        }
        constexpr int RF = L::RF, EF = L::EF;
        __syncthreads();  // every read of the regions below is done
        // the row-parallel part's k and beta, in flight from here
        i32x4 ek[NU8], eb[NU8];
#pragma unroll
        for (int u = 0; u < NU8; ++u) {
            const int e = tid + CT * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            const int64_t tk = ((t0 + r) * p.H + hk) * D + c0, tv = ((t0 + r) * p.HV + hv) * D + c0;
            ek[u] = r < len ? ld_raw8(p.k + tk) : i32x4{};
            eb[u] = r < len ? ld_raw8(p.beta + tv) : i32x4{};
        }
        if (tid < D) {
            // G_last's gradient: gamma rowsum(S_in dS_out) + GMU colsum(dKH RR)
            float cs = 0.0f;
            for (int m = 0; m < NMG; ++m) cs += lds_ld<float>(sm, L::DGP + 4 * (m * D + tid));
            const float dg0 = lds_ld<float>(sm, L::DGM + 4 * tid) * lds_ld<float>(sm, L::GAM + 4 * tid) +
                              cs * lds_ld<float>(sm, L::GMU + 4 * tid);
            lds_st<float>(sm, L::DGM + 4 * tid, dg0);
        }
        for (int u = 0; u < MPW; ++u) {
            const int mi = mg + NMG * u;
            st_tile_f32(sm, 0 * EF, RF, 16 * mi, 16 * ni, dQH[u], l16, q4);
            st_tile_f32(sm, 1 * EF, RF, 16 * mi, 16 * ni, dKB[u], l16, q4);
            st_tile_f32(sm, 2 * EF, RF, 16 * mi, 16 * ni, dRR[u], l16, q4);
        }
        scan_gcol<D, CT>(sm, 3 * EF, L::XS, -1, gv, tid, flagged ? L::FLC : -1);
        // a flagged column's G slot (pitch D, as scan_gcol's) carries its
        // final dG instead
        if (fcol)
            for (int u = 0; u < MPW; ++u) st_tile_f32(sm, 3 * EF, D, 16 * (mg + NMG * u), 16 * ni, dGf[u], l16, q4);
        __syncthreads();
        // row-parallel: dq, dk, dbeta, and dG (over dQH); a flagged channel's
        // tiles hold its final values
        const bool direct = p.H == p.HV;  // no grouped heads: dq, dk written here
#pragma unroll
        for (int u = 0; u < NU8; ++u) {
            const int e = tid + CT * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            const int o = 4 * (r * RF + c0);
            f32x8 dG = {};
            if (r < len) {
                const int64_t tk = ((t0 + r) * p.H + hk) * D + c0, tv = ((t0 + r) * p.HV + hv) * D + c0;
                const f32x8 kf = io8_f32(ek[u], p.io);
                const f32x8 bb = io8_f32(eb[u], p.io);
                const f32x8 fq = __builtin_convertvector(xq[u], f32x8);
                const f32x8 fk = __builtin_convertvector(xk[u], f32x8);
                const f32x8 fr = __builtin_convertvector(xr[u], f32x8);
                f32x8 dq, dk, db;
                for (int j = 0; j < 8; ++j) {
                    const float G = lds_ld<float>(sm, 3 * EF + 4 * (r * D + c0 + j));
                    const float gq = lds_ld<float>(sm, 0 * EF + o + 4 * j), gkb = lds_ld<float>(sm, 1 * EF + o + 4 * j);
                    const float grr = lds_ld<float>(sm, 2 * EF + o + 4 * j);
                    if (flagged && lds_ld<int>(sm, L::FLC + 4 * (c0 + j)) != 0) {
                        dq[j] = gq;
                        db[j] = gkb;
                        dk[j] = grr;
                        dG[j] = G;
                    } else {
                        const float eg = ex2(G), ie = ex2(-G);
                        dq[j] = gq * eg;
                        dk[j] = gkb * bb[j] * eg + grr * ie;
                        db[j] = gkb * kf[j] * eg;
                        dG[j] = gq * fq[j] + gkb * fk[j] - grr * fr[j];
                    }
                }
                if (direct) {
                    st_io8(p.dq + tk, dq, p.io);
                    st_io8(p.dk + tk, dk, p.io);
                } else {
                    *reinterpret_cast<f32x4 *>(p.dq_ws + tv) = __builtin_shufflevector(dq, dq, 0, 1, 2, 3);
                    *reinterpret_cast<f32x4 *>(p.dq_ws + tv + 4) = __builtin_shufflevector(dq, dq, 4, 5, 6, 7);
                    *reinterpret_cast<f32x4 *>(p.dk_ws + tv) = __builtin_shufflevector(dk, dk, 0, 1, 2, 3);
                    *reinterpret_cast<f32x4 *>(p.dk_ws + tv + 4) = __builtin_shufflevector(dk, dk, 4, 5, 6, 7);
                }
                st_io8(p.dbeta + tv, db, p.io);
                // dv = dWV w, dw = dWV v
                const f32x8 dwv = __builtin_convertvector(lds_ld<bf16x8>(sm, L::DWV + 2 * (r * D + c0)), f32x8);
                st_io8(p.dv + tv, dwv * io8_f32(wr[u], p.io), p.io);
                st_io8(p.dw + tv, dwv * io8_f32(vr[u], p.io), p.io);
            }
            lds_st<f32x4>(sm, o, __builtin_shufflevector(dG, dG, 0, 1, 2, 3));
            lds_st<f32x4>(sm, o + 16, __builtin_shufflevector(dG, dG, 4, 5, 6, 7));
        }
        __syncthreads();
        // dg = reverse cumulative sum of dG over the chunk; G_last's share
        // dgamma gamma reaches every row
        {
            const int c = tid % D;
            rscan_rows<D, CT>(sm, 0, RF, L::XS, lds_ld<float>(sm, L::DGM + 4 * c), tid);
        }
        __syncthreads();
        for (int e = tid; e < 64 * D / 4; e += CT) {
            const int r = e / (D / 4), c0 = 4 * (e % (D / 4));
            if (r < len)
                st_g4(p, ((t0 + r) * p.HV + hv) * D + c0, lds_ld<f32x4>(sm, 4 * (r * RF + c0)));
        }
    }
}

// -------------------------------------------------- state-gradient pass --
// One workgroup per (sequence, value head): dS (float32 [D][D], the result
// layout of 16x16 tiles, wave wv owning the 16 columns [16 wv, 16 wv + 16))
// walks the chunks in reverse; dS entering a chunk's step is the gradient
// of that chunk's S_out and is saved.
template <int D>
struct SL {
    static constexpr int RK = D + 8, RC = 64 + 8;
    static constexpr int TK = 64 * RK * 2, TC = 64 * RC * 2;
    static constexpr int QH = 0, RR = TK, WY = 2 * TK, DO = 3 * TK, PB = 4 * TK, GAM = 4 * TK + TC;
    static constexpr int SIZE = GAM + 4 * D;  // GAM: the record's gamma, negated in flagged channels
};

template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * (D / 16)) void bwd_state_kernel(BwdParams p)
{
    using L = SL<D>;
    constexpr int RK = L::RK, RC = L::RC;
    constexpr int ST = 64 * (D / 16);  // threads: one wave per 16 value columns
    constexpr int NRT = D / 16, VW = 16, NCT = 1, NKS = D / 32;
    __shared__ __attribute__((aligned(16))) char sm[L::SIZE];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
    // work item: (sequence, value head), times the segment and, in the
    // transition pass, the kind (0: end gradient, 1: map from the identity
    // with dO taken as zero)
    // (the whole-sequence instantiation folds all of this away)
    int item = blockIdx.x;
    const bool trans = SPLIT && p.pass == PASS_TRANSITION;
    const int kind = trans ? item & 1 : 0;
    if (trans) item >>= 1;
    const int seg = SPLIT ? item % p.nseg : 0;
    if (SPLIT) item /= p.nseg;
    const int n = item / p.HV, hv = item % p.HV;
    if (p.grp && p.grp[n] != p.gsel) return;  // the other launch's sequence
    const SeqRange sr = seq_of(p, n);
    const int64_t sb = sr.b, se = sr.e;
    const int nc = (int)chunks_of(sr);
    const int vbase = wv * VW;
    const int64_t head = ((int64_t)n * p.HV + hv) * D * D;

    // the chunks [c_lo, c_hi) walked, the entering gradient (src; nullptr:
    // zero), and where the leaving one goes
    int c_lo = 0, c_hi = nc;
    const float *src = p.dht ? p.dht + head : nullptr;
    float *dst = p.dh0 ? p.dh0 + head : nullptr;
    bool ident = false, zero_do = false, save = true;
    if constexpr (SPLIT) {
        const int last = seg_last(sr, p.seg_chunks);
        if (seg > last) return;  // past the start of this sequence
        c_lo = (last - seg) * p.seg_chunks;
        c_hi = c_lo + p.seg_chunks < nc ? c_lo + p.seg_chunks : nc;
        const int64_t sseg = (((int64_t)n * p.HV + hv) * p.nseg + seg) * D * D;
        if (trans) {
            // nothing follows the last segment; the first one's map is not needed
            if (seg >= last || (kind == 1 && seg == 0)) return;
            save = false;
            if (kind == 0) {
                if (seg > 0) src = nullptr;
                dst = p.wb + sseg;
            } else {
                src = nullptr;
                ident = zero_do = true;
                dst = p.wm + sseg;
            }
        } else {
            if (seg > 0) src = p.ws + sseg;
            if (seg < last) dst = nullptr;
        }
    }

    f32x4 dS[NRT][NCT];
    for (int rt = 0; rt < NRT; ++rt)
        for (int jt = 0; jt < NCT; ++jt)
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * rt + 4 * q4 + e, col = vbase + 16 * jt + l16;
                dS[rt][jt][e] = ident ? (row == col ? 1.0f : 0.0f) : src ? src[row * D + col] : 0.0f;
            }

    for (int c = c_hi - 1; c >= c_lo; --c) {
        const int64_t slot = chunk_slot(sb, n, c), t0 = sb + 64 * (int64_t)c;
        const int len = (int)(se - t0 < 64 ? se - t0 : 64);
        constexpr PrepRecord R{D};
        const char *rec = p.prep + (slot * p.HV + hv) * bwd_prep_bytes(D);
        // every load of the chunk's operands in flight before the first store
        constexpr int NU8 = 64 * D / 8 / ST, NUP = 64 * 8 / ST;
        bf16x8 xq[NU8], xr[NU8], xw[NU8], xp[NUP];
        i32x4 xo[NU8];
#pragma unroll
        for (int u = 0; u < NU8; ++u) {
            const int e = tid + ST * u, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            xq[u] = *reinterpret_cast<const bf16x8 *>(rec + R.qh() + 2 * (r * D + c0));
            xr[u] = *reinterpret_cast<const bf16x8 *>(rec + R.rr() + 2 * (r * D + c0));
            xw[u] = *reinterpret_cast<const bf16x8 *>(rec + R.wy() + 2 * (r * D + c0));
            xo[u] = r < len && !zero_do ? ld_raw8(p.dout + ((t0 + r) * p.HV + hv) * D + c0) : i32x4{};
        }
#pragma unroll
        for (int u = 0; u < NUP; ++u) {
            const int e = tid + ST * u, r = e >> 3, c0 = 8 * (e & 7);
            xp[u] = *reinterpret_cast<const bf16x8 *>(rec + R.p() + 2 * (r * 64 + c0));
        }
        const float xg = tid < D ? *reinterpret_cast<const float *>(rec + R.gam() + 4 * tid) : 0.0f;
        __syncthreads();  // the previous chunk's reads are done
#pragma unroll
        for (int u = 0; u < NU8; ++u) {
            const int e = tid + ST * u, r = e / (D / 8), c0 = 8 * (e % (D / 8)), o = 2 * (r * RK + c0);
            lds_st<bf16x8>(sm, L::QH + o, xq[u]);
            lds_st<bf16x8>(sm, L::RR + o, xr[u]);
            lds_st<bf16x8>(sm, L::WY + o, xw[u]);
            lds_st<bf16x8>(sm, L::DO + o, io8_bf16(xo[u], p.io));
        }
#pragma unroll
        for (int u = 0; u < NUP; ++u) {
            const int e = tid + ST * u, r = e >> 3, c0 = 8 * (e & 7);
            lds_st<bf16x8>(sm, L::PB + 2 * (r * RC + c0), xp[u]);
        }
        if (tid < D) lds_st<float>(sm, L::GAM + 4 * tid, xg);
        // the gradient of this chunk's S_out
        if (save) {
            uint16_t *dso = p.ds_ckpt + (slot * p.HV + hv) * D * D;  // rounded to bf16
            for (int rt = 0; rt < NRT; ++rt)
                for (int jt = 0; jt < NCT; ++jt)
                    for (int e = 0; e < 4; ++e)
                        dso[(16 * rt + 4 * q4 + e) * D + vbase + 16 * jt + l16] = __builtin_bit_cast(uint16_t, (__bf16)dS[rt][jt][e]);
        }
        __syncthreads();

        // dU = scale P^T dO + K-hat dS, K-hat = RR gamma (a flagged
        // channel's RR column holds K-hat itself, with factor 1): tokens x
        // this wave's columns. K-hat's factor times dS as bf16 operands: k
        // slab ks holds channels {32 ks + 4 q4 + e} then
        // {32 ks + 16 + 4 q4 + e}; RR is read in the same channel order.
        bf16x8 gS[NKS][NCT];
        for (int ks = 0; ks < NKS; ++ks) {
            const f32x4 g0 = khat_factor(lds_ld<f32x4>(sm, L::GAM + 4 * (32 * ks + 4 * q4)));
            const f32x4 g1 = khat_factor(lds_ld<f32x4>(sm, L::GAM + 4 * (32 * ks + 16 + 4 * q4)));
            for (int jt = 0; jt < NCT; ++jt)
                gS[ks][jt] = cat4(f32x4_to_bf16(dS[2 * ks][jt] * g0), f32x4_to_bf16(dS[2 * ks + 1][jt] * g1));
        }
        f32x4 dU[4][NCT];
        for (int mi = 0; mi < 4; ++mi)
            for (int jt = 0; jt < NCT; ++jt) {
                f32x4 acc = tile_mm<true, true>(sm, L::PB, RC, L::DO, RK, 16 * mi, vbase + 16 * jt, 64, f32x4{0, 0, 0, 0},
                                                l16, q4) * p.scale;
                for (int ks = 0; ks < NKS; ++ks) {
                    const int o = L::RR + 2 * ((16 * mi + l16) * RK + 32 * ks + 4 * q4);
                    acc = mfma_bf16(cat4(lds_ld<bf16x4>(sm, o), lds_ld<bf16x4>(sm, o + 32)), gS[ks][jt], acc);
                }
                dU[mi][jt] = acc;
            }
        // dS <- gamma dS + scale QH^T dO - wy_w^T dU; dU as bf16 operands:
        // k slab ks holds tokens {32 ks + 4 q4 + e} then {32 ks + 16 + 4 q4 + e}
        bf16x8 dUb[2][NCT];
        for (int ks = 0; ks < 2; ++ks)
            for (int jt = 0; jt < NCT; ++jt)
                dUb[ks][jt] = cat4(f32x4_to_bf16(dU[2 * ks][jt]), f32x4_to_bf16(dU[2 * ks + 1][jt]));
        for (int rt = 0; rt < NRT; ++rt) {
            const f32x4 gr = __builtin_elementwise_abs(lds_ld<f32x4>(sm, L::GAM + 4 * (16 * rt + 4 * q4)));
            for (int jt = 0; jt < NCT; ++jt) {
                f32x4 acc = tile_mm<true, true>(sm, L::QH, RK, L::DO, RK, 16 * rt, vbase + 16 * jt, 64, f32x4{0, 0, 0, 0},
                                                l16, q4) * p.scale;
                f32x4 neg = {0, 0, 0, 0};
                for (int ks = 0; ks < 2; ++ks) {
                    const int o = L::WY + 2 * ((32 * ks + 4 * q4 + (l16 >> 2)) * RK + 16 * rt + 4 * (l16 & 3));
                    neg = mfma_bf16(cat4(lds_tr(sm, o), lds_tr(sm, o + 32 * RK)), dUb[ks][jt], neg);
                }
                dS[rt][jt] = dS[rt][jt] * gr + acc - neg;
            }
        }
    }
    if (dst)
        for (int rt = 0; rt < NRT; ++rt)
            for (int jt = 0; jt < NCT; ++jt)
                for (int e = 0; e < 4; ++e) dst[(16 * rt + 4 * q4 + e) * D + vbase + 16 * jt + l16] = dS[rt][jt][e];
}

// ------------------------------------------------------------- reduce --
// dq, dk of q/k head h: the sums over its value heads h m .. h m + m - 1.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p)
{
    const int m = p.HV / p.H;
    const int64_t total = p.T * p.H * p.K;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = i % p.K, th = i / p.K, h = th % p.H, t = th / p.H;
        float sq = 0.0f, sk = 0.0f;
        for (int j = 0; j < m; ++j) {
            const int64_t o = (t * p.HV + h * m + j) * p.K + c;
            sq += p.dq_ws[o];
            sk += p.dk_ws[o];
        }
        p.dq[i] = f32_io1(sq, p.io);
        p.dk[i] = f32_io1(sk, p.io);
    }
}

// ------------------------------------------------------------- groups --
// The two-stream schedule's groups: rank every sequence by its chunk count
// (more first, ties to the lower index); the first nlong form group 0.
__global__ __launch_bounds__(256) void bwd_group_kernel(BwdParams p, int32_t nlong, int32_t *grp)
{
    for (int n = threadIdx.x; n < p.N; n += blockDim.x) {
        const int64_t cn = chunks_of(seq_of(p, n));
        int rank = 0;
        for (int j = 0; j < p.N; ++j) {
            const int64_t cj = chunks_of(seq_of(p, j));
            rank += cj > cn || (cj == cn && j < n);
        }
        grp[n] = rank < nlong ? 0 : 1;
    }
}

}  // namespace

hipError_t launch_bwd_group(const BwdParams &p, int32_t nlong, int32_t *grp, hipStream_t stream)
{
    if (p.N <= 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_group_kernel, dim3(1), dim3(256), 0, stream, p, nlong, grp);
    return hipGetLastError();
}

hipError_t launch_bwd_chunk(const BwdParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)((int64_t)p.nslots * p.HV));
    if (grid.x == 0) return hipSuccess;
    if (p.K == 128) {
        hipLaunchKernelGGL((bwd_chunk_kernel<128>), grid, dim3(CT), 0, stream, p);
    } else if (p.K == 64) {
        hipLaunchKernelGGL((bwd_chunk_kernel<64>), grid, dim3(CT), 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bwd_state(const BwdParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)((int64_t)p.N * p.HV * (p.seg_chunks ? p.nseg : 1) * (p.pass == PASS_TRANSITION ? 2 : 1)));
    if (grid.x == 0) return hipSuccess;
    const bool split = p.seg_chunks > 0;
    if (p.K == 128) {
        if (split) hipLaunchKernelGGL((bwd_state_kernel<128, true>), grid, dim3(64 * 8), 0, stream, p);
        else hipLaunchKernelGGL((bwd_state_kernel<128, false>), grid, dim3(64 * 8), 0, stream, p);
    } else if (p.K == 64) {
        if (split) hipLaunchKernelGGL((bwd_state_kernel<64, true>), grid, dim3(64 * 4), 0, stream, p);
        else hipLaunchKernelGGL((bwd_state_kernel<64, false>), grid, dim3(64 * 4), 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bwd_reduce(const BwdParams &p, hipStream_t stream)
{
    const int64_t total = p.T * p.H * p.K;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn2
