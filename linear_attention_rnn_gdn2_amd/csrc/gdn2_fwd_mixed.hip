// The chunked forward at unequal head dimensions, (K, V) = (128, 64) and
// (64, 128), and the backward's recompute at fp16 io or 16-bit g: the kernel
// of gdn2_fwd.hip instantiated in a translation unit of its own, so that the
// library's sources compile in parallel. Only the entries
// launch_chunk_fwd_mixed and launch_chunk_fwd_rec16 are defined here.
#define GDN2_FWD_MIXED
#include "gdn2_fwd.hip"
