// l9_mfma_tt.hip -- the matrix-core tile kernels with A and B transposed:
// every tile shape, whole / ragged-K / edge modes, unsplit and split K
// (instantiated in their own source so that the orientations compile in
// parallel).
#include "l9_tile.h"

namespace sgemm {

hipError_t launch_mfma_tt(Shape shape, const Problem& p, hipStream_t s) {
  return launch_shape_t<true, true>(shape, p, s);
}

hipError_t launch_mfma_split_tt(Shape shape, const Problem& p, int64_t k_split, float* ws,
                                 hipStream_t s) {
  return launch_split_shape_t<true, true>(shape, p, k_split, ws, s);
}

}  // namespace sgemm
