// Every internal problem description and launcher, for the host entry points
// (fa_api.hip). The kernels include only their own header, so that a change to
// one kernel's description leaves the others' sources untouched. Not part of
// the public ABI (that is include/fa.h).
#pragma once

#include "fa_bwd_params.h"
#include "fa_fwd_params.h"
#include "fa_kvouter_params.h"
#include "fa_norm_params.h"
