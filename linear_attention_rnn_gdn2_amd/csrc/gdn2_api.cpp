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

#include <atomic>
#include <string>

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
    default: return "unknown";
    }
}

int64_t elem_size(int32_t d) { return d == GDN2_DTYPE_BF16 ? 2 : 4; }

int64_t numel(const gdn2_tensor *t)
{
    int64_t n = 1;
    for (int d = 0; d < t->ndim; ++d) n *= t->shape[d];
    return n;
}

// Rank, dtype, extents (-1 = any), non-negative extents, row-major
// contiguity, non-NULL data when non-empty, 16-byte alignment.
int check_tensor(const gdn2_tensor *t, const char *name, int32_t dtype, int ndim,
                 const int64_t *want)
{
    if (t->ndim != ndim)
        return fail(GDN2_ERR_SHAPE, "%s: expected %d dimensions, got %d", name, ndim, t->ndim);
    if (t->dtype != dtype)
        return fail(GDN2_ERR_DTYPE, "%s: expected %s, got %s", name, dtype_name(dtype),
                    dtype_name(t->dtype));
    for (int d = 0; d < ndim; ++d) {
        if (t->shape[d] < 0)
            return fail(GDN2_ERR_SHAPE, "%s: negative extent in dimension %d", name, d);
        if (want && want[d] >= 0 && t->shape[d] != want[d])
            return fail(GDN2_ERR_SHAPE, "%s: dimension %d is %lld, expected %lld", name, d,
                        (long long)t->shape[d], (long long)want[d]);
    }
    int64_t expect = 1;
    for (int d = ndim - 1; d >= 0; --d) {
        if (t->shape[d] > 1 && t->stride[d] != expect)
            return fail(GDN2_ERR_LAYOUT, "%s: not row-major contiguous (dimension %d stride %lld, expected %lld)",
                        name, d, (long long)t->stride[d], (long long)expect);
        expect *= t->shape[d];
    }
    if (numel(t) > 0) {
        if (!t->data)
            return fail(GDN2_ERR_NULL_ARG, "%s: data is NULL but the tensor has elements", name);
        if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
            return fail(GDN2_ERR_LAYOUT, "%s: data pointer is not 16-byte aligned", name);
    }
    return GDN2_OK;
}

bool overlaps(const gdn2_tensor *a, const gdn2_tensor *b)
{
    if (!a || !b || !a->data || !b->data) return false;
    const int64_t na = numel(a) * elem_size(a->dtype), nb = numel(b) * elem_size(b->dtype);
    if (na == 0 || nb == 0) return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a->data), pb = reinterpret_cast<uintptr_t>(b->data);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

int validate(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
             const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
             const gdn2_tensor *h0, const gdn2_tensor *cu, const gdn2_tensor *out,
             const gdn2_tensor *ht, gdn2::FwdParams *p, bool allow_inplace_state = false)
{
    g_last_error.clear();
    if (!q) return fail(GDN2_ERR_NULL_ARG, "q is NULL");
    if (!k) return fail(GDN2_ERR_NULL_ARG, "k is NULL");
    if (!v) return fail(GDN2_ERR_NULL_ARG, "v is NULL");
    if (!out) return fail(GDN2_ERR_NULL_ARG, "out is NULL");
    int rc;
    if ((rc = check_tensor(q, "q", GDN2_DTYPE_BF16, 3, nullptr))) return rc;
    const int64_t T = q->shape[0], H = q->shape[1], K = q->shape[2];
    const int64_t qs[3] = {T, H, K};
    if ((rc = check_tensor(k, "k", GDN2_DTYPE_BF16, 3, qs))) return rc;
    const int64_t vs_any[3] = {T, -1, -1};
    if ((rc = check_tensor(v, "v", GDN2_DTYPE_BF16, 3, vs_any))) return rc;
    const int64_t HV = v->shape[1], V = v->shape[2];
    if (H < 1 || HV < H || HV % H != 0)
        return fail(GDN2_ERR_HEADS, "value heads (%lld) must be a positive multiple of q/k heads (%lld)",
                    (long long)HV, (long long)H);
    if (!((K == 64 && V == 64) || (K == 128 && V == 128)))
        return fail(GDN2_ERR_UNSUPPORTED, "(K, V) = (%lld, %lld) not supported; use (64, 64) or (128, 128)",
                    (long long)K, (long long)V);
    if (T > INT32_MAX)
        return fail(GDN2_ERR_SHAPE, "T = %lld exceeds the int32 range of cu_seqlens", (long long)T);
    const int64_t vs[3] = {T, HV, V}, gs[3] = {T, HV, K};
    if (w && (rc = check_tensor(w, "w", GDN2_DTYPE_BF16, 3, vs))) return rc;
    if (g && (rc = check_tensor(g, "g", GDN2_DTYPE_F32, 3, gs))) return rc;
    if (beta && (rc = check_tensor(beta, "beta", GDN2_DTYPE_BF16, 3, gs))) return rc;
    if ((rc = check_tensor(out, "out", GDN2_DTYPE_BF16, 3, vs))) return rc;
    int64_t N = 1;
    if (cu) {
        if ((rc = check_tensor(cu, "cu_seqlens", GDN2_DTYPE_I32, 1, nullptr))) return rc;
        N = cu->shape[0] - 1;
        if (N < 1) return fail(GDN2_ERR_SHAPE, "cu_seqlens needs at least 2 entries (N >= 1)");
        if (!cu->data) return fail(GDN2_ERR_NULL_ARG, "cu_seqlens: data is NULL");
    }
    if (N * HV > INT32_MAX)
        return fail(GDN2_ERR_SHAPE, "N * HV = %lld exceeds the grid limit", (long long)(N * HV));
    const int64_t ss[4] = {N, HV, K, V};
    if (h0 && (rc = check_tensor(h0, "initial_state", GDN2_DTYPE_F32, 4, ss))) return rc;
    if (ht && (rc = check_tensor(ht, "final_state", GDN2_DTYPE_F32, 4, ss))) return rc;

    const gdn2_tensor *inputs[] = {q, k, v, g, beta, w, h0, cu};
    const char *in_names[] = {"q", "k", "v", "g", "beta", "w", "initial_state", "cu_seqlens"};
    // final_state may be initial_state itself (same buffer) where the kernel
    // reads every state element before writing it (the recurrent path)
    const bool inplace = allow_inplace_state && h0 && ht && h0->data == ht->data;
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
        p->g = g ? static_cast<const float *>(g->data) : nullptr;
        p->beta = beta ? static_cast<const uint16_t *>(beta->data) : nullptr;
        p->w = w ? static_cast<const uint16_t *>(w->data) : nullptr;
        p->h0 = h0 ? static_cast<const float *>(h0->data) : nullptr;
        p->cu = cu ? static_cast<const int32_t *>(cu->data) : nullptr;
        p->out = static_cast<uint16_t *>(out->data);
        p->ht = ht ? static_cast<float *>(ht->data) : nullptr;
        p->T = T;
        p->N = (int32_t)N;
        p->H = (int32_t)H;
        p->HV = (int32_t)HV;
        p->K = (int32_t)K;
        p->V = (int32_t)V;
        p->scale = scale == 0.0f ? (float)(1.0 / sqrt((double)K)) : scale;
    }
    return GDN2_OK;
}

int read_options(const gdn2_fwd_options *opts, int32_t *split)
{
    *split = 0;
    if (!opts) return GDN2_OK;
    if (opts->struct_size < (int32_t)sizeof(gdn2_fwd_options))
        return fail(GDN2_ERR_SHAPE, "options: struct_size %d is smaller than %d", opts->struct_size,
                    (int)sizeof(gdn2_fwd_options));
    if (opts->seq_split_chunks < -1)
        return fail(GDN2_ERR_SHAPE, "options: seq_split_chunks must be -1, 0 or positive (got %d)",
                    opts->seq_split_chunks);
    *split = opts->seq_split_chunks;
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

}  // namespace

extern "C" {

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
    int rc = validate(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state, &p);
    if (rc != GDN2_OK) return rc;
    int32_t split = 0;
    if ((rc = read_options(opts, &split)) != GDN2_OK) return rc;
    p.seg_chunks = 0;
    p.nseg = 1;
    p.pass = gdn2::PASS_OUTPUT;
    p.wb = p.wm = p.ws = nullptr;
    if (split == 0) {
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) == hipSuccess) ncu = cu_count(dev);
        split = gdn2_split_plan(p.T, p.N, p.HV, ncu);
    }
    const int64_t chunks = (p.T + 63) / 64;
    const int64_t nseg = split > 0 ? (chunks + split - 1) / split : 1;
    if (split > 0 && nseg > 1 && nseg <= INT32_MAX) {
        // sequence split: transition pass, combine, output pass, all on
        // `stream`, with a stream-ordered workspace
        const size_t state = (size_t)p.K * p.V * sizeof(float);
        const size_t one = (size_t)p.N * p.HV * (size_t)nseg * state;
        void *ws = nullptr;
        if (one / state == (size_t)p.N * p.HV * (size_t)nseg && hipMallocAsync(&ws, 3 * one, stream) == hipSuccess) {
            p.seg_chunks = split;
            p.nseg = (int32_t)nseg;
            p.wb = static_cast<float *>(ws);
            p.wm = reinterpret_cast<float *>(static_cast<char *>(ws) + one);
            p.ws = reinterpret_cast<float *>(static_cast<char *>(ws) + 2 * one);
            gdn2::FwdParams pt = p;
            pt.pass = gdn2::PASS_TRANSITION;
            hipError_t e = gdn2::launch_chunk_fwd(pt, stream);
            if (e == hipSuccess) e = gdn2::launch_seg_combine(p, stream);
            if (e == hipSuccess) e = gdn2::launch_chunk_fwd(p, stream);
            const hipError_t ef = hipFreeAsync(ws, stream);
            if (e != hipSuccess)
                return fail(GDN2_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
            if (ef != hipSuccess)
                return fail(GDN2_ERR_HIP, "workspace release failed: %s", hipGetErrorString(ef));
            return GDN2_OK;
        }
        (void)hipGetLastError();  // no workspace: run the sequences whole instead
    }
    hipError_t e = gdn2::launch_chunk_fwd(p, stream);
    if (e != hipSuccess)
        return fail(GDN2_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return GDN2_OK;
}

int gdn2_recurrent_fwd(const gdn2_tensor *q, const gdn2_tensor *k, const gdn2_tensor *v,
                       const gdn2_tensor *g, const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                       const gdn2_tensor *initial_state, const gdn2_tensor *cu_seqlens,
                       const gdn2_tensor *out, const gdn2_tensor *final_state, hipStream_t stream)
{
    gdn2::FwdParams p;
    int rc = validate(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, out, final_state, &p, true);
    if (rc != GDN2_OK) return rc;
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
