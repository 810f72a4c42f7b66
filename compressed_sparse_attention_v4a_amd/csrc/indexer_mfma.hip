// Matrix-core paths of the lightning indexer (filled in below as they land).
#include "internal.h"

namespace v4a {

bool indexer_mfma_supported(int T, int n_hI, int cI, int dt) {
  (void)T; (void)n_hI; (void)cI; (void)dt;
  return false;
}

hipError_t launch_indexer_scores_mfma(const IndexerArgs& a, float* scores, int64_t ld,
                                      hipStream_t s) {
  (void)a; (void)scores; (void)ld; (void)s;
  return hipErrorNotSupported;
}

}  // namespace v4a
