// The chunked forward at unequal head dimensions, (K, V) = (128, 64) and
// (64, 128): the kernel of gdn2_fwd.hip instantiated in a translation unit
// of its own, so that the library's sources compile in parallel. Only the
// entry launch_chunk_fwd_mixed is defined here.
#define GDN2_FWD_MIXED
#include "gdn2_fwd.hip"
