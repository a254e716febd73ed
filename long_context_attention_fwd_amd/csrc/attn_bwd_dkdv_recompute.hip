// attn_bwd_dkdv_recompute.hip -- the dK/dV kernel instances of the
// recomputing backward path (D = 128, contiguous tensors: the path that does
// not store dS), compiled as a unit of their own so that they can take the
// backend's max-ILP instruction-scheduling strategy: the same results, faster
// for these instances although they spill a few registers under it, while on
// the rest of the backward it adds spills to eleven kernels.  The source is
// attn_bwd.hip; this unit emits only the two explicit instantiations that
// file declares extern for it.
#define LCATTN_BWD_DKDV_UNIT 2
#include "attn_bwd.hip"
