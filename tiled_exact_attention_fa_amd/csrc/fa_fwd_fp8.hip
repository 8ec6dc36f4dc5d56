#include "fa_internal.h"
int fa_launch_fwd_fp8(const fa_fwd_params *, void *) { return fa_set_error(FA_ERR_UNSUPPORTED, "fp8 forward not built yet"); }
