// Stream kernels (panels of at most 16 rows) for launches mixing 4- and 5-bit group-32 jobs.
// One translation unit per format set, so they compile in parallel.
#include "stream_impl.h"

namespace qg {

sweep_fn pick_stream_q4q5(bool mfma, int cls, int rows) { return pick_set<kSetQ4 | kSetQ5>(mfma, cls, rows); }

}  // namespace qg
