// Stream kernels (panels of at most 16 rows) for launches whose jobs are all 4-bit group-32.
// One translation unit per format set, so they compile in parallel.
#include "stream_impl.h"

namespace qg {

sweep_fn pick_stream_q4(bool mfma, int cls, int rows) { return pick_set<kSetQ4>(mfma, cls, rows); }

}  // namespace qg
