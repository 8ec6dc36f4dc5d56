#include "fa_internal.h"
int fa_launch_decode(const fa_decode_params *, void *) { return fa_set_error(FA_ERR_UNSUPPORTED, "decode not built yet"); }
