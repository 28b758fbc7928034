// bwd_dkv.hip -- the backward's source pass (dK, dV): bwd.hip built with
// only that pass's launchers, so that the two passes compile in parallel.
#define GT_BWD_PART 2
#include "bwd.hip"
