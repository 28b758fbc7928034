// bwd_dq.hip -- the backward's destination pass (dQ): bwd.hip built with
// only that pass's launchers, so that the two passes compile in parallel.
#define GT_BWD_PART 1
#include "bwd.hip"
