// Index arithmetic of the packed (varlen) layout, shared by the host code and
// the kernels: a sequence's token range from cu_seqlens, the checkpoint slot
// of a chunk, the sequence that owns a slot, and the segments of a split
// walk. Plain C++ (no HIP types), so that a host program can check it on
// malformed input. Not part of the ABI.
//
// cu_seqlens is a device array that the host never reads (no
// synchronisation), so the kernels cannot reject a malformed one. Instead
// every range derived from it is clamped: 0 <= b <= e <= T for each
// sequence, whatever the array holds (entries past T, negative, or
// decreasing). A well-formed array (cu[0] = 0, non-decreasing, cu[N] = T,
// the FlashInfer docs' cu_seqlens) passes through unchanged; a malformed one
// gives unspecified values but every load and store stays inside the
// caller's buffers and the library's workspace.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GDN2_HD __host__ __device__
#else
#define GDN2_HD
#endif

namespace gdn2 {

constexpr int CHUNK = 64;  // tokens per chunk

struct SeqRange {
    int64_t b, e;  // tokens [b, e)
};

// Raw entry i of cu_seqlens (int32 or int64 elements).
GDN2_HD inline int64_t cu_raw(const void *cu, int cu64, int64_t i)
{
    return cu64 ? static_cast<const int64_t *>(cu)[i] : (int64_t) static_cast<const int32_t *>(cu)[i];
}

// Token range of sequence n: [cu[n], cu[n + 1]) clamped to 0 <= b <= e <= T;
// without cu_seqlens, one sequence of T tokens.
GDN2_HD inline SeqRange seq_range(const void *cu, int cu64, int64_t T, int64_t n)
{
    if (!cu) return SeqRange{0, T};
    int64_t b = cu_raw(cu, cu64, n), e = cu_raw(cu, cu64, n + 1);
    b = b < 0 ? 0 : b > T ? T : b;
    e = e < b ? b : e > T ? T : e;
    return SeqRange{b, e};
}

GDN2_HD inline int64_t chunks_of(SeqRange r) { return (r.e - r.b + CHUNK - 1) / CHUNK; }

// Checkpoint slot of chunk c of sequence n that starts at token b: unique
// over the chunks of a well-formed packed batch, and below T / 64 + N for
// every chunk of every clamped range (b <= T, chunks_of <= ceil((T - b) / 64)).
GDN2_HD inline int64_t chunk_slot(int64_t b, int64_t n, int64_t c) { return b / CHUNK + n + c; }

// Number of checkpoint slots of a batch of N sequences and T tokens.
GDN2_HD inline int64_t slot_count(int64_t T, int64_t N) { return T / CHUNK + N; }

// The sequence and chunk that own a checkpoint slot: the last sequence
// whose first slot is not past it (binary search; the first slots are
// non-decreasing for a well-formed array). Returns false when the slot holds
// no chunk (past the sequence's last chunk, or before its first one, which
// only a malformed array produces).
GDN2_HD inline bool slot_owner(const void *cu, int cu64, int64_t T, int N, int64_t slot, int *n_out, int64_t *c_out)
{
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_slot(seq_range(cu, cu64, T, mid).b, mid, 0) <= slot) lo = mid;
        else hi = mid - 1;
    }
    const SeqRange r = seq_range(cu, cu64, T, lo);
    const int64_t c = slot - chunk_slot(r.b, lo, 0);
    *n_out = lo;
    *c_out = c;
    return c >= 0 && c < chunks_of(r);
}

// Segments of a split walk: segment j of a sequence holds chunks
// [j L, min((j + 1) L, chunks)); the last segment index of a range (0 for
// an empty one). With nseg = ceil(ceil(T / 64) / L), every segment index of
// every clamped range is below nseg.
GDN2_HD inline int seg_last(SeqRange r, int L)
{
    const int64_t nch = chunks_of(r);
    return nch > 0 ? (int)((nch - 1) / L) : 0;
}
GDN2_HD inline int64_t seg_count(int64_t T, int L) { return ((T + CHUNK - 1) / CHUNK + L - 1) / L; }

}  // namespace gdn2
