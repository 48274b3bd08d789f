// l9_catalogue_second.hip -- the second half of the tile catalogue of
// l9_catalogue.h (two files so that they compile in parallel): row-major
// operands, every shape (whole, ragged-K and edge tiles), unsplit and over
// K slices.
#include "l9_catalogue.h"
#include "l9_tile.h"

namespace sgemm {
namespace {

#define SGEMM_CAT_TYPE(I, NAME, BM, BN, BK, WM, WN, UNROLL, GM, PRIO, KS, DEPTH, MS) \
  typedef MfmaTile<BM, BN, BK, WM, WN, UNROLL, GM, PRIO, KS, DEPTH, MS> Cat##I;
SGEMM_CATALOGUE_SECOND(SGEMM_CAT_TYPE)
#undef SGEMM_CAT_TYPE

// one launcher pair per entry (the tile over the whole problem, and over K
// slices into a workspace)
#define SGEMM_CAT_FNS(I, NAME, BM, BN, BK, WM, WN, UNROLL, GM, PRIO, KS, DEPTH, MS)       \
  hipError_t cat_launch_##I(const Problem& p, hipStream_t s) {                              \
    return launch_tiles<Cat##I>(p, s);                                                      \
  }                                                                                         \
  hipError_t cat_split_##I(const Problem& p, int64_t k_split, float* ws, hipStream_t s) { \
    return launch_split<Cat##I>(p, k_split, ws, s);                                         \
  }
SGEMM_CATALOGUE_SECOND(SGEMM_CAT_FNS)
#undef SGEMM_CAT_FNS

}  // namespace

#define SGEMM_CAT_ENTRY(I, NAME, BM, BN, BK, WM, WN, UNROLL, GM, PRIO, KS, DEPTH, MS) \
  {NAME, BK, cat_launch_##I, cat_split_##I},
const CatalogueEntry* catalogue_second(int* count) {
  static const CatalogueEntry entries[] = {SGEMM_CATALOGUE_SECOND(SGEMM_CAT_ENTRY)};
  *count = static_cast<int>(sizeof(entries) / sizeof(entries[0]));
  return entries;
}
#undef SGEMM_CAT_ENTRY

}  // namespace sgemm
