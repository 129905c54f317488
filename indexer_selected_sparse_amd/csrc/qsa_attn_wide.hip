// Decode attention that selects from candidate lists of more than 4096
// entries per row (rows of 32768 blocks at K = 2048) with the 8-group
// register path of qsa_attn.hip.  Its kernels are built here, in a
// translation unit of their own: instantiated next to the 4-group kernels,
// they changed the 4-group kernels' register allocation.
#define QSA_ATTN_WIDE_TU
#include "qsa_attn.hip"

namespace qsa {

hipError_t launch_attn_select_wide(const qsa_attn &a, int budget, int ratio, const qsa_batch &b, const ListArgs &la,
                                   const float *scores, int64_t ld, int32_t *idx, void *out, void *ws,
                                   const qsa_paged_kv *pg, hipStream_t st) {
    return attn_select_impl<8>(a, budget, ratio, b, la, scores, ld, idx, out, ws, pg, st);
}

}  // namespace qsa
