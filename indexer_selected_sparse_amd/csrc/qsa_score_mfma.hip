// Matrix-core indexer scores for prefill (placeholder until the MFMA kernel lands).
#include "qsa_internal.hpp"

namespace qsa {

hipError_t launch_score_mfma(const qsa_indexer &ix, int ratio, const qsa_batch &b, float *scores,
                             int64_t ld, hipStream_t st) {
    (void)ix; (void)ratio; (void)b; (void)scores; (void)ld; (void)st;
    return hipErrorNotSupported;
}

}  // namespace qsa
