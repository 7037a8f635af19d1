// Stream kernels (panels of at most 16 rows) for launches with a group-64 or zero-point job.
// One translation unit per format set, so they compile in parallel.
#include "stream_impl.h"

namespace qg {

sweep_fn pick_stream_all(bool mfma, int cls, int rows) { return pick_set<kSetQ4 | kSetQ5 | kSetG64 | kSetZP>(mfma, cls, rows); }

}  // namespace qg
