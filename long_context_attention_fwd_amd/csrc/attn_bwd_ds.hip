// attn_bwd_ds.hip -- the dK/dV kernel instances of the backward that also
// store dS (D = 128, contiguous tensors), compiled as a unit of their own so
// that they can take another instruction-scheduling strategy than the rest of
// the backward (the backend's iterative ILP scheduler: the same results in a
// faster order for these instances, while it makes the recomputing path's
// dK/dV instances and the strided ones spill registers).  The source is
// attn_bwd.hip; this unit emits only the two explicit instantiations that
// file declares extern for it.
#define LCATTN_BWD_DKDV_UNIT 1
#include "attn_bwd.hip"
