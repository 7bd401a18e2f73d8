// C-ABI entry points of libgdn2: argument validation and kernel dispatch.
//
// Every check runs on the host before anything is enqueued, so a rejected
// call leaves the stream untouched. The FlashInfer chunk_gated_delta_rule2
// documentation (parameter list) fixes the optional-argument defaults and the
// no-alias rule for the output state; the shapes are the Flash-GDN-2 README's
// quick-start layout in packed (varlen) form.
#include "../../include/gdn2.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <stddef.h>

#include <atomic>
#include <mutex>
#include <string>
#include <utility>

#include "gdn2_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

const char *dtype_name(int32_t d)
{
    switch (d) {
    case GDN2_DTYPE_BF16: return "bf16";
    case GDN2_DTYPE_F32: return "float32";
    case GDN2_DTYPE_I32: return "int32";
    case GDN2_DTYPE_F16: return "float16";
    case GDN2_DTYPE_I64: return "int64";
    default: return "unknown";
    }
}

int64_t elem_size(int32_t d)
{
    switch (d) {
    case GDN2_DTYPE_BF16:
    case GDN2_DTYPE_F16: return 2;
    case GDN2_DTYPE_I64: return 8;
    default: return 4;
    }
}

int64_t numel(const gdn2_tensor *t)
{
    int64_t n = 1;
    for (int d = 0; d < t->ndim; ++d) n *= t->shape[d];
    return n;
}

// How a tensor may be laid out in memory.
enum Layout {
    DENSE,  // row-major contiguous
    ROWS    // [tokens, heads, D]: the D elements of a row contiguous, token
            // and head strides free (non-negative, multiples of 16 bytes,
            // the token stride at least one row), rows 16-byte aligned
};

// Rank, dtype (one of two accepted: dtype2 < 0 for one), extents (-1 = any),
// non-negative extents, layout, non-NULL data when non-empty, 16-byte
// alignment.
int check_tensor(const gdn2_tensor *t, const char *name, int32_t dtype, int32_t dtype2, int ndim,
                 const int64_t *want, Layout layout = DENSE)
{
    if (t->ndim != ndim)
        return fail(GDN2_ERR_SHAPE, "%s: expected %d dimensions, got %d", name, ndim, t->ndim);
    if (t->dtype != dtype && t->dtype != dtype2) {
        if (dtype2 >= 0)
            return fail(GDN2_ERR_DTYPE, "%s: expected %s or %s, got %s", name, dtype_name(dtype), dtype_name(dtype2),
                        dtype_name(t->dtype));
        return fail(GDN2_ERR_DTYPE, "%s: expected %s, got %s", name, dtype_name(dtype), dtype_name(t->dtype));
    }
    for (int d = 0; d < ndim; ++d) {
        if (t->shape[d] < 0)
            return fail(GDN2_ERR_SHAPE, "%s: negative extent in dimension %d", name, d);
        if (want && want[d] >= 0 && t->shape[d] != want[d])
            return fail(GDN2_ERR_SHAPE, "%s: dimension %d is %lld, expected %lld", name, d,
                        (long long)t->shape[d], (long long)want[d]);
    }
    const int64_t es = elem_size(t->dtype);
    if (layout == ROWS) {
        const int64_t D = t->shape[2];
        if (D > 1 && t->stride[2] != 1)
            return fail(GDN2_ERR_LAYOUT, "%s: the last dimension must be contiguous (stride %lld)", name,
                        (long long)t->stride[2]);
        for (int d = 0; d < 2; ++d) {
            if (t->shape[d] <= 1) continue;
            if (t->stride[d] < 0 || (t->stride[d] * es) % 16 != 0)
                return fail(GDN2_ERR_LAYOUT, "%s: dimension %d stride %lld must be non-negative and a multiple of 16 bytes",
                            name, d, (long long)t->stride[d]);
        }
        if (t->shape[0] > 1) {
            if (t->stride[0] < D)
                return fail(GDN2_ERR_LAYOUT, "%s: token stride %lld is shorter than a row (%lld elements)", name,
                            (long long)t->stride[0], (long long)D);
            if (t->stride[0] * es * 64 > INT32_MAX)
                return fail(GDN2_ERR_LAYOUT, "%s: token stride %lld is too large (64 rows must span under 2 GiB)",
                            name, (long long)t->stride[0]);
        }
    } else {
        int64_t expect = 1;
        for (int d = ndim - 1; d >= 0; --d) {
            if (t->shape[d] > 1 && t->stride[d] != expect)
                return fail(GDN2_ERR_LAYOUT, "%s: not row-major contiguous (dimension %d stride %lld, expected %lld)",
                            name, d, (long long)t->stride[d], (long long)expect);
            expect *= t->shape[d];
        }
    }
    if (numel(t) > 0) {
        if (!t->data)
            return fail(GDN2_ERR_NULL_ARG, "%s: data is NULL but the tensor has elements", name);
        if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
            return fail(GDN2_ERR_LAYOUT, "%s: data pointer is not 16-byte aligned", name);
    }
    return GDN2_OK;
}

// Whether the [tokens, heads, D] rows of a ROWS tensor are pairwise disjoint:
// with the token and head dimensions taken in order of increasing stride,
// each stride must reach past everything the smaller ones span.
bool rows_disjoint(const gdn2_tensor *t)
{
    int64_t st[2] = {t->stride[0], t->stride[1]}, ex[2] = {t->shape[0], t->shape[1]};
    if (st[0] > st[1]) {
        std::swap(st[0], st[1]);
        std::swap(ex[0], ex[1]);
    }
    int64_t span = t->shape[2];  // elements one row covers
    for (int d = 0; d < 2; ++d) {
        if (ex[d] <= 1) continue;
        if (st[d] < span) return false;
        span += (ex[d] - 1) * st[d];
    }
    return true;
}

// Bytes from the first to one past the last element (strided tensors: the
// whole span, which is conservative for interleaved views).
int64_t span_bytes(const gdn2_tensor *t)
{
    if (numel(t) == 0) return 0;
    int64_t last = 0;
    for (int d = 0; d < t->ndim; ++d) last += (t->shape[d] - 1) * t->stride[d];
    return (last + 1) * elem_size(t->dtype);
}

bool overlaps(const gdn2_tensor *a, const gdn2_tensor *b)
{
    if (!a || !b || !a->data || !b->data) return false;
    const int64_t na = span_bytes(a), nb = span_bytes(b);
    if (na == 0 || nb == 0) return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a->data), pb = reinterpret_cast<uintptr_t>(b->data);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

int validate(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
             const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
             const gdn2_tensor *h0, const gdn2_tensor *cu, const gdn2_tensor *out,
             const gdn2_tensor *ht, gdn2::FwdParams *p, bool allow_inplace_state = false,
             bool state_vmajor = false)
{
    g_last_error.clear();
    if (!q) return fail(GDN2_ERR_NULL_ARG, "q is NULL");
    if (!k) return fail(GDN2_ERR_NULL_ARG, "k is NULL");
    if (!v) return fail(GDN2_ERR_NULL_ARG, "v is NULL");
    if (!out) return fail(GDN2_ERR_NULL_ARG, "out is NULL");
    int rc;
    if ((rc = check_tensor(q, "q", GDN2_DTYPE_BF16, GDN2_DTYPE_F16, 3, nullptr, ROWS))) return rc;
    const int32_t io = q->dtype;  // q, k, v, beta, w and out share one 16-bit type
    const int64_t T = q->shape[0], H = q->shape[1], K = q->shape[2];
    const int64_t qs[3] = {T, H, K};
    if ((rc = check_tensor(k, "k", io, -1, 3, qs, ROWS))) return rc;
    const int64_t vs_any[3] = {T, -1, -1};
    if ((rc = check_tensor(v, "v", io, -1, 3, vs_any, ROWS))) return rc;
    const int64_t HV = v->shape[1], V = v->shape[2];
    if (H < 1 || HV < H || HV % H != 0)
        return fail(GDN2_ERR_HEADS, "value heads (%lld) must be a positive multiple of q/k heads (%lld)",
                    (long long)HV, (long long)H);
    if ((K != 64 && K != 128) || (V != 64 && V != 128))
        return fail(GDN2_ERR_UNSUPPORTED, "(K, V) = (%lld, %lld) not supported; K and V must each be 64 or 128",
                    (long long)K, (long long)V);
    if (T > INT32_MAX)
        return fail(GDN2_ERR_SHAPE, "T = %lld exceeds the int32 range of cu_seqlens", (long long)T);
    const int64_t vs[3] = {T, HV, V}, gs[3] = {T, HV, K};
    if (w && (rc = check_tensor(w, "w", io, -1, 3, vs, ROWS))) return rc;
    if (g) {
        if (g->dtype != GDN2_DTYPE_F32 && g->dtype != GDN2_DTYPE_BF16 && g->dtype != GDN2_DTYPE_F16)
            return fail(GDN2_ERR_DTYPE, "g: expected float32, bf16 or float16, got %s", dtype_name(g->dtype));
        if ((rc = check_tensor(g, "g", g->dtype, -1, 3, gs, ROWS))) return rc;
    }
    if (beta && (rc = check_tensor(beta, "beta", io, -1, 3, gs, ROWS))) return rc;
    if ((rc = check_tensor(out, "out", io, -1, 3, vs, ROWS))) return rc;
    if (!rows_disjoint(out)) return fail(GDN2_ERR_LAYOUT, "out: rows overlap each other");
    int64_t N = 1;
    if (cu) {
        if ((rc = check_tensor(cu, "cu_seqlens", GDN2_DTYPE_I32, GDN2_DTYPE_I64, 1, nullptr))) return rc;
        N = cu->shape[0] - 1;
        if (N < 1) return fail(GDN2_ERR_SHAPE, "cu_seqlens needs at least 2 entries (N >= 1)");
        if (!cu->data) return fail(GDN2_ERR_NULL_ARG, "cu_seqlens: data is NULL");
    }
    if (N * HV > INT32_MAX)
        return fail(GDN2_ERR_SHAPE, "N * HV = %lld exceeds the grid limit", (long long)(N * HV));
    // states: [N, HV, K, V], or [N, HV, V, K] with the V-major layout option
    const int64_t ss[4] = {N, HV, state_vmajor ? V : K, state_vmajor ? K : V};
    if (h0 && (rc = check_tensor(h0, "initial_state", GDN2_DTYPE_F32, GDN2_DTYPE_BF16, 4, ss))) return rc;
    if (ht && (rc = check_tensor(ht, "final_state", GDN2_DTYPE_F32, GDN2_DTYPE_BF16, 4, ss))) return rc;

    const gdn2_tensor *inputs[] = {q, k, v, g, beta, w, h0, cu};
    const char *in_names[] = {"q", "k", "v", "g", "beta", "w", "initial_state", "cu_seqlens"};
    // final_state may be initial_state itself (same buffer) where the kernel
    // reads every state element before writing it (the recurrent path)
    const bool inplace = allow_inplace_state && h0 && ht && h0->data == ht->data && h0->dtype == ht->dtype;
    for (int i = 0; i < 8; ++i) {
        if (overlaps(out, inputs[i]))
            return fail(GDN2_ERR_ALIAS, "out overlaps %s", in_names[i]);
        if (overlaps(ht, inputs[i]) && !(inplace && inputs[i] == h0))
            return fail(GDN2_ERR_ALIAS, "final_state overlaps %s", in_names[i]);
    }
    if (overlaps(out, ht)) return fail(GDN2_ERR_ALIAS, "out overlaps final_state");

    if (p) {
        p->q = static_cast<const uint16_t *>(q->data);
        p->k = static_cast<const uint16_t *>(k->data);
        p->v = static_cast<const uint16_t *>(v->data);
        p->g = g ? g->data : nullptr;
        p->beta = beta ? static_cast<const uint16_t *>(beta->data) : nullptr;
        p->w = w ? static_cast<const uint16_t *>(w->data) : nullptr;
        p->h0 = h0 ? static_cast<const float *>(h0->data) : nullptr;
        p->cu = cu ? cu->data : nullptr;
        p->out = static_cast<uint16_t *>(out->data);
        p->ht = ht ? static_cast<float *>(ht->data) : nullptr;
        p->T = T;
        p->N = (int32_t)N;
        p->H = (int32_t)H;
        p->HV = (int32_t)HV;
        p->K = (int32_t)K;
        p->V = (int32_t)V;
        p->scale = scale == 0.0f ? (float)(1.0 / sqrt((double)K)) : scale;
        p->io = io == GDN2_DTYPE_F16 ? gdn2::IO_F16 : gdn2::IO_BF16;
        p->gtype = !g || g->dtype == GDN2_DTYPE_F32 ? gdn2::G_F32
                   : g->dtype == GDN2_DTYPE_BF16    ? gdn2::G_BF16
                                                    : gdn2::G_F16;
        p->cu64 = cu && cu->dtype == GDN2_DTYPE_I64;
        p->h0_bf16 = h0 && h0->dtype == GDN2_DTYPE_BF16;
        p->ht_bf16 = ht && ht->dtype == GDN2_DTYPE_BF16;
        // token and head strides (elements). A dimension of extent one is
        // only ever indexed at 0; its token stride is then taken as one row,
        // which keeps the kernels' chunk ranges (rows x token stride) whole.
        // An omitted tensor is never addressed.
        auto st = [](const gdn2_tensor *t, int d) { return t && t->shape[d] > 1 ? t->stride[d] : 0; };
        auto tok = [](const gdn2_tensor *t) { return !t ? 0 : t->shape[0] > 1 ? t->stride[0] : t->shape[2]; };
        p->sq = tok(q);
        p->sk = tok(k);
        p->sv = tok(v);
        p->sw = tok(w);
        p->sg = tok(g);
        p->sb = tok(beta);
        p->so = tok(out);
        p->hsq = st(q, 1);
        p->hsk = st(k, 1);
        p->hsv = st(v, 1);
        p->hsw = st(w, 1);
        p->hsg = st(g, 1);
        p->hsb = st(beta, 1);
        p->hso = st(out, 1);
        p->state_vmajor = 0;
        p->qk_l2norm = 0;
        p->ckpt = nullptr;
        p->rec = nullptr;
        p->tonly = 0;
    }
    return GDN2_OK;
}

// Options: fields past struct_size keep their defaults, so that callers
// built against an older, shorter struct keep working.
struct Options {
    int32_t split = 0, vmajor = 0, l2norm = 0;
};

int read_options(const gdn2_fwd_options *opts, Options *o)
{
    *o = Options{};
    if (!opts) return GDN2_OK;
    const int32_t sz = opts->struct_size;
    if (sz < (int32_t)(2 * sizeof(int32_t)))
        return fail(GDN2_ERR_SHAPE, "options: struct_size %d is smaller than %d", sz, (int)(2 * sizeof(int32_t)));
    if (opts->seq_split_chunks < -1)
        return fail(GDN2_ERR_SHAPE, "options: seq_split_chunks must be -1, 0 or positive (got %d)",
                    opts->seq_split_chunks);
    o->split = opts->seq_split_chunks;
    if (sz >= (int32_t)(offsetof(gdn2_fwd_options, state_layout) + sizeof(int32_t))) {
        if (opts->state_layout != GDN2_STATE_KV && opts->state_layout != GDN2_STATE_VK)
            return fail(GDN2_ERR_SHAPE, "options: state_layout must be GDN2_STATE_KV or GDN2_STATE_VK (got %d)",
                        opts->state_layout);
        o->vmajor = opts->state_layout == GDN2_STATE_VK;
    }
    if (sz >= (int32_t)(offsetof(gdn2_fwd_options, qk_l2norm) + sizeof(int32_t))) {
        if (opts->qk_l2norm != 0 && opts->qk_l2norm != 1)
            return fail(GDN2_ERR_SHAPE, "options: qk_l2norm must be 0 or 1 (got %d)", opts->qk_l2norm);
        o->l2norm = opts->qk_l2norm;
    }
    return GDN2_OK;
}

// Compute-unit count per device, looked up once.
int cu_count(int dev)
{
    static std::atomic<int> cache[64];
    if (dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Validation of a backward call: every tensor dense and row-major, bf16
// except g, dg and the states (float32). Fills the backward's parameters and
// the forward's (for the checkpoint pass) when p is given.
int validate_bwd(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v, const gdn2_tensor *g,
                 const gdn2_tensor *beta, const gdn2_tensor *w, float scale, const gdn2_tensor *h0,
                 const gdn2_tensor *cu, const gdn2_tensor *dout, const gdn2_tensor *dht, const gdn2_tensor *dq,
                 const gdn2_tensor *dk, const gdn2_tensor *dv, const gdn2_tensor *dg, const gdn2_tensor *dbeta,
                 const gdn2_tensor *dw, const gdn2_tensor *dh0, gdn2::BwdParams *p, gdn2::FwdParams *pf)
{
    g_last_error.clear();
    const gdn2_tensor *req[] = {q, k, v, g, beta, w, dout, dq, dk, dv, dg, dbeta, dw};
    const char *req_names[] = {"q", "k", "v", "g", "beta", "w", "d_out", "dq", "dk", "dv", "dg", "dbeta", "dw"};
    for (int i = 0; i < 13; ++i)
        if (!req[i]) return fail(GDN2_ERR_NULL_ARG, "%s is NULL (required by the backward)", req_names[i]);
    int rc;
    if ((rc = check_tensor(q, "q", GDN2_DTYPE_BF16, GDN2_DTYPE_F16, 3, nullptr))) return rc;
    const int32_t io = q->dtype;  // q, k, v, beta, w, d_out and the gradients share one 16-bit type
    const int64_t T = q->shape[0], H = q->shape[1], K = q->shape[2];
    if ((rc = check_tensor(v, "v", io, -1, 3, nullptr))) return rc;
    if (v->shape[0] != T) return fail(GDN2_ERR_SHAPE, "v: dimension 0 is %lld, expected %lld", (long long)v->shape[0], (long long)T);
    const int64_t HV = v->shape[1], V = v->shape[2];
    if (H < 1 || HV < H || HV % H != 0)
        return fail(GDN2_ERR_HEADS, "value heads (%lld) must be a positive multiple of q/k heads (%lld)",
                    (long long)HV, (long long)H);
    if (!((K == 64 && V == 64) || (K == 128 && V == 128)))
        return fail(GDN2_ERR_UNSUPPORTED,
                    "(K, V) = (%lld, %lld) not supported by the backward; it takes (64, 64) or (128, 128)",
                    (long long)K, (long long)V);
    if (T > INT32_MAX) return fail(GDN2_ERR_SHAPE, "T = %lld exceeds the int32 range", (long long)T);
    const int64_t qs[3] = {T, H, K}, vs[3] = {T, HV, V}, gs[3] = {T, HV, K};
    if ((rc = check_tensor(k, "k", io, -1, 3, qs))) return rc;
    if ((rc = check_tensor(w, "w", io, -1, 3, vs))) return rc;
    if (g->dtype != GDN2_DTYPE_F32 && g->dtype != GDN2_DTYPE_BF16 && g->dtype != GDN2_DTYPE_F16)
        return fail(GDN2_ERR_DTYPE, "g: expected float32, bf16 or float16, got %s", dtype_name(g->dtype));
    const int32_t gt = g->dtype;  // g and dg share one type
    if ((rc = check_tensor(g, "g", gt, -1, 3, gs))) return rc;
    if ((rc = check_tensor(beta, "beta", io, -1, 3, gs))) return rc;
    if ((rc = check_tensor(dout, "d_out", io, -1, 3, vs))) return rc;
    if ((rc = check_tensor(dq, "dq", io, -1, 3, qs))) return rc;
    if ((rc = check_tensor(dk, "dk", io, -1, 3, qs))) return rc;
    if ((rc = check_tensor(dv, "dv", io, -1, 3, vs))) return rc;
    if ((rc = check_tensor(dw, "dw", io, -1, 3, vs))) return rc;
    if ((rc = check_tensor(dg, "dg", gt, -1, 3, gs))) return rc;
    if ((rc = check_tensor(dbeta, "dbeta", io, -1, 3, gs))) return rc;
    int64_t N = 1;
    if (cu) {
        if ((rc = check_tensor(cu, "cu_seqlens", GDN2_DTYPE_I32, GDN2_DTYPE_I64, 1, nullptr))) return rc;
        N = cu->shape[0] - 1;
        if (N < 1) return fail(GDN2_ERR_SHAPE, "cu_seqlens needs at least 2 entries (N >= 1)");
        if (!cu->data) return fail(GDN2_ERR_NULL_ARG, "cu_seqlens: data is NULL");
    }
    const int64_t nslots = gdn2::slot_count(T, N);
    if (N * HV > INT32_MAX || nslots * HV > INT32_MAX)
        return fail(GDN2_ERR_SHAPE, "N * HV or the chunk count times HV exceeds the grid limit");
    const int64_t ss[4] = {N, HV, K, V};
    if (h0 && (rc = check_tensor(h0, "initial_state", GDN2_DTYPE_F32, -1, 4, ss))) return rc;
    if (dht && (rc = check_tensor(dht, "d_final_state", GDN2_DTYPE_F32, -1, 4, ss))) return rc;
    if (dh0 && (rc = check_tensor(dh0, "d_initial_state", GDN2_DTYPE_F32, -1, 4, ss))) return rc;

    const gdn2_tensor *ins[] = {q, k, v, g, beta, w, h0, cu, dout, dht};
    const char *in_names[] = {"q", "k", "v", "g", "beta", "w", "initial_state", "cu_seqlens", "d_out", "d_final_state"};
    const gdn2_tensor *outs[] = {dq, dk, dv, dg, dbeta, dw, dh0};
    const char *out_names[] = {"dq", "dk", "dv", "dg", "dbeta", "dw", "d_initial_state"};
    for (int o = 0; o < 7; ++o) {
        for (int i = 0; i < 10; ++i)
            if (overlaps(outs[o], ins[i])) return fail(GDN2_ERR_ALIAS, "%s overlaps %s", out_names[o], in_names[i]);
        for (int o2 = o + 1; o2 < 7; ++o2)
            if (overlaps(outs[o], outs[o2])) return fail(GDN2_ERR_ALIAS, "%s overlaps %s", out_names[o], out_names[o2]);
    }

    if (p) {
        *p = gdn2::BwdParams{};
        p->q = static_cast<const uint16_t *>(q->data);
        p->k = static_cast<const uint16_t *>(k->data);
        p->v = static_cast<const uint16_t *>(v->data);
        p->w = static_cast<const uint16_t *>(w->data);
        p->g = g->data;
        p->io = io == GDN2_DTYPE_F16 ? gdn2::IO_F16 : gdn2::IO_BF16;
        p->gtype = gt == GDN2_DTYPE_F32 ? gdn2::G_F32 : gt == GDN2_DTYPE_BF16 ? gdn2::G_BF16 : gdn2::G_F16;
        p->beta = static_cast<const uint16_t *>(beta->data);
        p->dout = static_cast<const uint16_t *>(dout->data);
        p->cu = cu ? cu->data : nullptr;
        p->cu64 = cu && cu->dtype == GDN2_DTYPE_I64;
        p->dht = dht ? static_cast<const float *>(dht->data) : nullptr;
        p->dh0 = dh0 ? static_cast<float *>(dh0->data) : nullptr;
        p->dq = static_cast<uint16_t *>(dq->data);
        p->dk = static_cast<uint16_t *>(dk->data);
        p->dv = static_cast<uint16_t *>(dv->data);
        p->dw = static_cast<uint16_t *>(dw->data);
        p->dbeta = static_cast<uint16_t *>(dbeta->data);
        p->dg = dg->data;
        p->T = T;
        p->N = (int32_t)N;
        p->H = (int32_t)H;
        p->HV = (int32_t)HV;
        p->K = (int32_t)K;
        p->V = (int32_t)V;
        p->nslots = (int32_t)nslots;
        p->scale = scale == 0.0f ? (float)(1.0 / sqrt((double)K)) : scale;
    }
    if (pf) {
        *pf = gdn2::FwdParams{};
        pf->q = static_cast<const uint16_t *>(q->data);
        pf->k = static_cast<const uint16_t *>(k->data);
        pf->v = static_cast<const uint16_t *>(v->data);
        pf->g = g->data;
        pf->beta = static_cast<const uint16_t *>(beta->data);
        pf->w = static_cast<const uint16_t *>(w->data);
        pf->h0 = h0 ? static_cast<const float *>(h0->data) : nullptr;
        pf->cu = cu ? cu->data : nullptr;
        pf->cu64 = cu && cu->dtype == GDN2_DTYPE_I64;
        pf->T = T;
        pf->N = (int32_t)N;
        pf->H = (int32_t)H;
        pf->HV = (int32_t)HV;
        pf->K = (int32_t)K;
        pf->V = (int32_t)V;
        pf->scale = scale == 0.0f ? (float)(1.0 / sqrt((double)K)) : scale;
        pf->io = io == GDN2_DTYPE_F16 ? gdn2::IO_F16 : gdn2::IO_BF16;
        pf->gtype = gt == GDN2_DTYPE_F32 ? gdn2::G_F32 : gt == GDN2_DTYPE_BF16 ? gdn2::G_BF16 : gdn2::G_F16;
        // dense row-major strides (elements)
        pf->sq = pf->sk = H * K;
        pf->hsq = pf->hsk = K;
        pf->sv = pf->sw = pf->so = HV * V;
        pf->hsv = pf->hsw = pf->hso = V;
        pf->sg = pf->sb = HV * K;
        pf->hsg = pf->hsb = K;
        pf->nseg = 1;
        pf->pass = gdn2::PASS_OUTPUT;
    }
    return GDN2_OK;
}

}  // namespace

namespace {
// Stream-ordered workspace from a pool the library owns on each device. Its
// release threshold is unlimited: memory freed at the end of a call stays in
// the pool for the next one instead of going back to the driver at the next
// synchronisation (the backward's workspace is gigabytes, and mapping it
// afresh every call costs a large share of a call). The pool thus keeps up
// to the largest workspace any call has used, until the process ends.
constexpr int kPoolDevices = 64;
std::once_flag pool_once[kPoolDevices];
hipMemPool_t pool_of[kPoolDevices];

hipError_t ws_alloc(void **ptr, size_t bytes, hipStream_t stream)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kPoolDevices) return hipMallocAsync(ptr, bytes, stream);
    std::call_once(pool_once[dev], [dev] {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess) {
            (void)hipGetLastError();
            return;  // no pool: the device's default one below
        }
        uint64_t keep = UINT64_MAX;
        if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) (void)hipGetLastError();
        pool_of[dev] = pool;
    });
    if (pool_of[dev]) return hipMallocFromPoolAsync(ptr, bytes, pool_of[dev], stream);
    return hipMallocAsync(ptr, bytes, stream);
}

// The backward's second stream with its fork and join events, one set per
// device, created on first use (at the default priority) and kept until
// the process ends. A call holds the device's lock from the fork to the
// join, so that calls from several host threads cannot interleave their
// event records.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool tried = false;
};
SideStream side_of[kPoolDevices];
std::mutex side_mu[kPoolDevices];

// The device's side stream, or nullptr (none could be made; or `stream` is
// being captured into a graph and the stream does not exist yet: creating
// one then would invalidate the capture). Call with side_mu[dev] held.
const SideStream *side_stream(int dev, hipStream_t stream)
{
    if (dev < 0 || dev >= kPoolDevices) return nullptr;
    SideStream &x = side_of[dev];
    if (x.s) return &x;
    if (x.tried) return nullptr;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return nullptr;
    }
    x.tried = true;
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;  // (what was made stays unused)
    }
    x.fork = f;
    x.join = j;
    x.s = s;
    return &x;
}

// Whether the backward runs as two groups of sequences on two streams: with
// whole sequences (no split) and between half of the compute units and all
// of them in (sequence, value head) chains, every chain's sequential passes
// run at once, and the chains of short sequences end long before the
// longest. The longer half of the sequences then runs its passes on the
// call's stream while the shorter half's run on the side stream, whose
// chunk-parallel gradient pass fills the units that the short chains leave
// idle. (Measured on MI355X, 8 sequences of 7 to 121 chunks, 32 heads, 256
// compute units: 3.92 ms as one group, 3.60 ms as two.)
bool bwd_two_groups(const gdn2::BwdParams &p, int32_t split, int ncu)
{
    const int64_t chains = (int64_t)p.N * p.HV;
    return split <= 0 && p.T > 0 && p.N >= 2 && ncu > 0 && 2 * chains > ncu && chains <= ncu;
}

// Workspace bytes per (sequence, value head, segment) of a split run: its
// end state from a zero start and its entering state (K x V each), and its
// transition map (K x K), all float32.
size_t split_item_bytes(const gdn2::FwdParams &p)
{
    return (2 * (size_t)p.K * p.V + (size_t)p.K * p.K) * sizeof(float);
}

// Bytes of the split run's workspace (segment end states, transitions and
// entering states) for segments of `split` chunks; 0 when the run would not
// split, SIZE_MAX when the count overflows.
size_t split_workspace_bytes(const gdn2::FwdParams &p, int32_t split)
{
    const int64_t nseg = split > 0 ? gdn2::seg_count(p.T, split) : 1;
    if (split <= 0 || nseg <= 1) return 0;
    if (nseg > INT32_MAX) return SIZE_MAX;
    const size_t items = (size_t)p.N * p.HV * (size_t)nseg;
    const size_t per = split_item_bytes(p);
    if (items / nseg != (size_t)p.N * p.HV || items > SIZE_MAX / per) return SIZE_MAX;
    return items * per;
}

// Enqueue the chunked forward of p on `stream`: whole sequences, or, with
// split > 0 giving more than one segment, the split run (transition pass,
// combine, output pass). Its workspace is `fixed` when given (the caller
// has checked that it is large enough), else stream-ordered
// (ws_alloc / hipFreeAsync on `stream`; if that allocation fails the
// sequences run whole). The transition pass writes no checkpoints or
// records; the output pass writes them per segment. Returns a gdn2 status
// (and sets the error message).
int run_forward(gdn2::FwdParams p, int32_t split, hipStream_t stream, void *fixed = nullptr)
{
    const size_t bytes = split_workspace_bytes(p, split);
    if (bytes > 0 && bytes != SIZE_MAX) {
        const int64_t nseg = gdn2::seg_count(p.T, split);
        const size_t items = (size_t)p.N * p.HV * (size_t)nseg;
        const size_t sz_b = items * p.K * p.V * sizeof(float), sz_m = items * p.K * p.K * sizeof(float);
        void *ws = fixed;
        const bool own = !fixed;
        if (own && ws_alloc(&ws, bytes, stream) != hipSuccess) ws = nullptr;
        if (ws) {
            p.seg_chunks = split;
            p.nseg = (int32_t)nseg;
            p.wb = static_cast<float *>(ws);
            p.wm = reinterpret_cast<float *>(static_cast<char *>(ws) + sz_b);
            p.ws = reinterpret_cast<float *>(static_cast<char *>(ws) + sz_b + sz_m);
            gdn2::FwdParams pt = p;
            pt.pass = gdn2::PASS_TRANSITION;
            pt.ckpt = nullptr;
            pt.rec = nullptr;
            hipError_t e = gdn2::launch_chunk_fwd(pt, stream);
            if (e == hipSuccess) e = gdn2::launch_seg_combine(p, stream);
            if (e == hipSuccess) e = gdn2::launch_chunk_fwd(p, stream);
            const hipError_t ef = own ? hipFreeAsync(ws, stream) : hipSuccess;
            if (e != hipSuccess)
                return fail(GDN2_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
            if (ef != hipSuccess)
                return fail(GDN2_ERR_HIP, "workspace release failed: %s", hipGetErrorString(ef));
            return GDN2_OK;
        }
        (void)hipGetLastError();  // no workspace: run the sequences whole instead
    }
    p.seg_chunks = 0;
    p.nseg = 1;
    const hipError_t e = gdn2::launch_chunk_fwd(p, stream);
    if (e != hipSuccess)
        return fail(GDN2_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN2_OK;
}

// Enqueue the backward's state-gradient pass: whole sequences, or, with
// split > 0 giving more than one segment, split like the forward
// (transition pass, the forward's combine in processing order, output pass).
hipError_t run_bwd_state(gdn2::BwdParams p, int32_t split, hipStream_t stream)
{
    const int64_t nseg = split > 0 ? gdn2::seg_count(p.T, split) : 1;
    if (split > 0 && nseg > 1 && nseg <= INT32_MAX) {
        const size_t state = (size_t)p.K * p.V * sizeof(float);
        const size_t one = (size_t)p.N * p.HV * (size_t)nseg * state;
        void *ws = nullptr;
        if (one / state == (size_t)p.N * p.HV * (size_t)nseg && ws_alloc(&ws, 3 * one, stream) == hipSuccess) {
            p.seg_chunks = split;
            p.nseg = (int32_t)nseg;
            p.wb = static_cast<float *>(ws);
            p.wm = reinterpret_cast<float *>(static_cast<char *>(ws) + one);
            p.ws = reinterpret_cast<float *>(static_cast<char *>(ws) + 2 * one);
            gdn2::BwdParams pt = p;
            pt.pass = gdn2::PASS_TRANSITION;
            gdn2::FwdParams pc{};
            pc.cu = p.cu;
            pc.cu64 = p.cu64;
            pc.T = p.T;
            pc.N = p.N;
            pc.H = p.H;
            pc.HV = p.HV;
            pc.K = p.K;
            pc.V = p.V;
            pc.seg_chunks = p.seg_chunks;
            pc.nseg = p.nseg;
            pc.wb = p.wb;
            pc.wm = p.wm;
            pc.ws = p.ws;
            p.pass = gdn2::PASS_OUTPUT;
            hipError_t e = gdn2::launch_bwd_state(pt, stream);
            if (e == hipSuccess) e = gdn2::launch_seg_combine(pc, stream);
            if (e == hipSuccess) e = gdn2::launch_bwd_state(p, stream);
            const hipError_t ef = hipFreeAsync(ws, stream);
            return e != hipSuccess ? e : ef;
        }
        (void)hipGetLastError();  // no workspace: whole sequences
    }
    p.seg_chunks = 0;
    p.nseg = 1;
    p.pass = gdn2::PASS_OUTPUT;
    return gdn2::launch_bwd_state(p, stream);
}
}  // namespace

// ------------------------------------------------- allocation-free entry --
// gdn2_chunk_fwd_noalloc takes the split run's workspace from this array
// instead of allocating one. Every GPU the library runs on holds its own
// copy until the process ends, at its own address. Host code uses that
// address as hipGetSymbolAddress returns it for the current device
// (scratch_on), never the array's name, which on the host is only a
// stand-in for the symbol.
static __device__ __align__(256) char scratch[GDN2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_addr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// The device address of `scratch` on device dev, which must be current:
// looked up once per device, the first time the entry point runs there.
void *scratch_on(int dev, hipError_t *err)
{
    std::call_once(scratch_once[dev], [dev] {
        void *ptr = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        scratch_addr[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    *err = scratch_err[dev];
    return scratch_addr[dev];
}

// The shortest segment length, at least `split`, whose workspace fits in
// `cap` bytes (-1: none does, so sequences run whole).
int32_t fit_split(const gdn2::FwdParams &p, int32_t split, size_t cap)
{
    if (split <= 0 || split_workspace_bytes(p, split) <= cap) return split;
    const size_t per_seg = (size_t)p.N * p.HV * split_item_bytes(p);
    const int64_t max_seg = (int64_t)(cap / per_seg);
    if (max_seg < 2) return -1;
    const int64_t chunks = (p.T + gdn2::CHUNK - 1) / gdn2::CHUNK;
    const int64_t L = (chunks + max_seg - 1) / max_seg;
    return L > INT32_MAX ? -1 : (int32_t)(L > split ? L : split);
}
}  // namespace

extern "C" {

int gdn2_chunk_fwd_noalloc(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                           const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                           const gdn2_tensor *initial_state, const gdn2_tensor *cu_seqlens,
                           const gdn2_tensor *out, const gdn2_tensor *final_state,
                           const gdn2_fwd_options *opts, hipStream_t stream)
{
    gdn2::FwdParams p;
    Options o;
    int rc = read_options(opts, &o);
    if (rc != GDN2_OK) return rc;
    rc = validate(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state, &p,
                  false, o.vmajor != 0);
    if (rc != GDN2_OK) return rc;
    p.state_vmajor = o.vmajor;
    p.qk_l2norm = o.l2norm;
    p.seg_chunks = 0;
    p.nseg = 1;
    p.pass = gdn2::PASS_OUTPUT;
    p.wb = p.wm = p.ws = nullptr;
    const size_t cap = GDN2_NOALLOC_SCRATCH_BYTES;
    int32_t split = o.split;
    if (split > 0) {
        const size_t need = split_workspace_bytes(p, split);
        if (need > cap)
            return fail(GDN2_ERR_UNSUPPORTED,
                        "seq_split_chunks %d needs %zu bytes of scratch; gdn2_chunk_fwd_noalloc holds %zu "
                        "(use longer segments, -1, or gdn2_chunk_fwd_opts)",
                        split, need, cap);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN2_ERR_HIP, "no current device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GDN2_ERR_UNSUPPORTED, "device %d: gdn2_chunk_fwd_noalloc serves devices 0..%d", dev,
                    kMaxDevices - 1);
    if (split == 0) split = fit_split(p, gdn2_split_plan(p.T, p.N, p.HV, cu_count(dev)), cap);
    void *ws = nullptr;
    if (split_workspace_bytes(p, split) > 0) {
        ws = scratch_on(dev, &e);
        if (!ws) return fail(GDN2_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
    }
    // ws is set whenever the run splits, so run_forward allocates nothing
    return run_forward(p, split, stream, ws);
}

int gdn2_chunk_bwd_check(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v, const gdn2_tensor *g,
                         const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                         const gdn2_tensor *initial_state, const gdn2_tensor *cu_seqlens, const gdn2_tensor *d_out,
                         const gdn2_tensor *d_final_state, const gdn2_tensor *dq, const gdn2_tensor *dk,
                         const gdn2_tensor *dv, const gdn2_tensor *dg, const gdn2_tensor *dbeta,
                         const gdn2_tensor *dw, const gdn2_tensor *d_initial_state)
{
    return validate_bwd(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, d_out, d_final_state, dq, dk, dv, dg,
                        dbeta, dw, d_initial_state, nullptr, nullptr);
}

int gdn2_chunk_bwd(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v, const gdn2_tensor *g,
                   const gdn2_tensor *beta, const gdn2_tensor *w, float scale, const gdn2_tensor *initial_state,
                   const gdn2_tensor *cu_seqlens, const gdn2_tensor *d_out, const gdn2_tensor *d_final_state,
                   const gdn2_tensor *dq, const gdn2_tensor *dk, const gdn2_tensor *dv, const gdn2_tensor *dg,
                   const gdn2_tensor *dbeta, const gdn2_tensor *dw, const gdn2_tensor *d_initial_state,
                   hipStream_t stream)
{
    gdn2::BwdParams p;
    gdn2::FwdParams pf;
    int rc = validate_bwd(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, d_out, d_final_state, dq, dk, dv,
                          dg, dbeta, dw, d_initial_state, &p, &pf);
    if (rc != GDN2_OK) return rc;
    // stream-ordered workspace: forward checkpoints, state-gradient
    // checkpoints, chunk records, per-value-head dq and dk
    const size_t state = (size_t)p.K * p.V * sizeof(uint16_t);  // bf16 checkpoints
    const size_t chunks = (size_t)p.nslots * (size_t)p.HV;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t sz_ck = up(chunks * state);
    const size_t sz_prep = up(chunks * (size_t)gdn2::bwd_prep_bytes(p.K));
    // per-value-head dq, dk only with grouped heads (otherwise written directly)
    const size_t sz_qk = p.H != p.HV ? up((size_t)p.T * p.HV * p.K * sizeof(float)) : 0;
    // the forward again, writing checkpoints and records (split into
    // segments as the forward itself would split this shape), then the
    // state-gradient and gradient passes; as one group of sequences or two
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess) ncu = cu_count(dev);
    const int32_t split = gdn2_split_plan(p.T, p.N, p.HV, ncu);
    const bool two = bwd_two_groups(p, split, ncu);
    const size_t sz_grp = two ? up((size_t)p.N * sizeof(int32_t)) : 0;  // each sequence's group
    const size_t total = 2 * sz_ck + sz_prep + 2 * sz_qk + sz_grp;
    void *ws = nullptr;
    if (total > 0 && ws_alloc(&ws, total, stream) != hipSuccess)
        return fail(GDN2_ERR_HIP, "backward workspace of %zu bytes could not be allocated", total);
    char *b = static_cast<char *>(ws);
    uint16_t *s_ckpt = reinterpret_cast<uint16_t *>(b);
    p.s_ckpt = s_ckpt;
    p.ds_ckpt = reinterpret_cast<uint16_t *>(b + sz_ck);
    p.prep = b + 2 * sz_ck;
    p.dq_ws = reinterpret_cast<float *>(b + 2 * sz_ck + sz_prep);
    p.dk_ws = reinterpret_cast<float *>(b + 2 * sz_ck + sz_prep + sz_qk);
    pf.ckpt = s_ckpt;
    pf.rec = p.prep;
    int frc = GDN2_OK;
    hipError_t e = hipSuccess;
    bool done = false;
    if (two && dev >= 0 && dev < kPoolDevices) {
        std::lock_guard<std::mutex> lock(side_mu[dev]);
        const SideStream *side = side_stream(dev, stream);
        if (side) {
            // group 0: the longer half of the sequences, on `stream`; group
            // 1, the others, on the side stream between the fork and the join
            int32_t *grp = reinterpret_cast<int32_t *>(b + 2 * sz_ck + sz_prep + 2 * sz_qk);
            p.grp = pf.grp = grp;
            e = gdn2::launch_bwd_group(p, p.N / 2, grp, stream);
            if (e == hipSuccess) e = hipEventRecord(side->fork, stream);
            if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
            if (e == hipSuccess) {
                const hipStream_t st[2] = {stream, side->s};
                gdn2::FwdParams fg[2] = {pf, pf};
                gdn2::BwdParams bg[2] = {p, p};
                for (int i = 0; i < 2; ++i) fg[i].gsel = bg[i].gsel = i;
                for (int i = 0; i < 2 && frc == GDN2_OK; ++i) frc = run_forward(fg[i], 0, st[i]);
                for (int i = 0; i < 2 && frc == GDN2_OK && e == hipSuccess; ++i) e = run_bwd_state(bg[i], 0, st[i]);
                for (int i = 0; i < 2 && frc == GDN2_OK && e == hipSuccess; ++i) e = gdn2::launch_bwd_chunk(bg[i], st[i]);
                // the join, whatever failed above: the call's stream waits
                // for everything the side stream was given
                const hipError_t ej = hipEventRecord(side->join, side->s);
                const hipError_t ew = ej == hipSuccess ? hipStreamWaitEvent(stream, side->join, 0) : ej;
                if (e == hipSuccess) e = ew;
            }
            if (frc == GDN2_OK && e == hipSuccess && p.H != p.HV) e = gdn2::launch_bwd_reduce(p, stream);
            done = true;
        }
    }
    if (!done) {
        p.grp = pf.grp = nullptr;
        if (p.T > 0) frc = run_forward(pf, split, stream);
        if (frc == GDN2_OK) {
            e = run_bwd_state(p, split, stream);
            if (e == hipSuccess && p.T > 0) e = gdn2::launch_bwd_chunk(p, stream);
            if (e == hipSuccess && p.T > 0 && p.H != p.HV) e = gdn2::launch_bwd_reduce(p, stream);
        }
    }
    const hipError_t ef = ws ? hipFreeAsync(ws, stream) : hipSuccess;
    if (frc != GDN2_OK) return frc;
    if (e != hipSuccess) return fail(GDN2_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    if (ef != hipSuccess) return fail(GDN2_ERR_HIP, "workspace release failed: %s", hipGetErrorString(ef));
    return GDN2_OK;
}

int gdn2_chunk_fwd_check(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                         const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w,
                         float scale, const gdn2_tensor *initial_state,
                         const gdn2_tensor *cu_seqlens, const gdn2_tensor *out,
                         const gdn2_tensor *final_state)
{
    return validate(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state,
                    nullptr);
}

int gdn2_chunk_fwd(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                   const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                   const gdn2_tensor *initial_state, const gdn2_tensor *cu_seqlens,
                   const gdn2_tensor *out, const gdn2_tensor *final_state, hipStream_t stream)
{
    return gdn2_chunk_fwd_opts(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state,
                               nullptr, stream);
}

int gdn2_chunk_fwd_opts(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                        const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                        const gdn2_tensor *initial_state, const gdn2_tensor *cu_seqlens,
                        const gdn2_tensor *out, const gdn2_tensor *final_state,
                        const gdn2_fwd_options *opts, hipStream_t stream)
{
    gdn2::FwdParams p;
    Options o;
    int rc = read_options(opts, &o);
    if (rc != GDN2_OK) return rc;
    rc = validate(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state, &p,
                  false, o.vmajor != 0);
    if (rc != GDN2_OK) return rc;
    int32_t split = o.split;
    p.state_vmajor = o.vmajor;
    p.qk_l2norm = o.l2norm;
    p.seg_chunks = 0;
    p.nseg = 1;
    p.pass = gdn2::PASS_OUTPUT;
    p.wb = p.wm = p.ws = nullptr;
    if (split == 0) {
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) == hipSuccess) ncu = cu_count(dev);
        split = gdn2_split_plan(p.T, p.N, p.HV, ncu);
    }
    return run_forward(p, split, stream);
}

int gdn2_recurrent_fwd(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                       const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                       const gdn2_tensor *initial_state, const gdn2_tensor *cu_seqlens,
                       const gdn2_tensor *out, const gdn2_tensor *final_state, hipStream_t stream)
{
    return gdn2_recurrent_fwd_opts(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state,
                                   nullptr, stream);
}

int gdn2_recurrent_fwd_opts(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                            const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                            const gdn2_tensor *initial_state, const gdn2_tensor *cu_seqlens,
                            const gdn2_tensor *out, const gdn2_tensor *final_state,
                            const gdn2_fwd_options *opts, hipStream_t stream)
{
    gdn2::FwdParams p;
    Options o;
    int rc = read_options(opts, &o);
    if (rc != GDN2_OK) return rc;
    rc = validate(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state, &p,
                  true, o.vmajor != 0);
    if (rc != GDN2_OK) return rc;
    p.state_vmajor = o.vmajor;
    p.qk_l2norm = o.l2norm;
    p.seg_chunks = 0;
    p.nseg = 1;
    p.pass = gdn2::PASS_OUTPUT;
    p.wb = p.wm = p.ws = nullptr;
    hipError_t e = gdn2::launch_recurrent_fwd(p, stream);
    if (e != hipSuccess)
        return fail(GDN2_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN2_OK;
}

int gdn2_recurrent_fwd_check(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                             const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w,
                             float scale, const gdn2_tensor *initial_state,
                             const gdn2_tensor *cu_seqlens, const gdn2_tensor *out,
                             const gdn2_tensor *final_state)
{
    return validate(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state, nullptr, true);
}

int gdn2_split_plan(int64_t T, int32_t N, int32_t HV, int32_t num_cu)
{
    // Split only when the (sequence, head) chains leave at least half of
    // the compute units idle and are long (32 chunks or more). Segments of
    // about sqrt(chunks per sequence) chunks balance the two serial parts of
    // a split run, the segment walk (L chunk steps) and the combine (one
    // step per segment, P = chunks / L); at least 8 chunks, so that
    // per-workgroup start-up and the composition of segment maps stay small.
    // (Measured on MI355X: 16 chains x 64 chunks are fastest at 8, 32
    // chains x 1024 chunks at 32.)
    if (T <= 0 || N <= 0 || HV <= 0 || num_cu <= 0) return 0;
    const int64_t chains = (int64_t)N * HV;
    const int64_t avg = ((T + 63) / 64 + N - 1) / N;
    if (2 * chains > num_cu || avg < 32) return 0;
    int64_t L = (int64_t)llround(sqrt((double)avg));
    if (L < 8) L = 8;
    return (int)L;
}

const char *gdn2_last_error(void) { return g_last_error.c_str(); }

int gdn2_abi_version(void) { return GDN2_ABI_VERSION; }

}  // extern "C"
