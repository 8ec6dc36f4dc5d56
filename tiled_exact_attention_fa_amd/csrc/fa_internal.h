// Internal declarations shared by the host-side translation units of libfa.
#pragma once

#include "../../include/fa.h"

#define FA_DECODE_MAX_SPLITS 64
#define FA_DECODE_MAX_GROUP 16

// Records a reason for the calling thread's fa_last_error() and returns status.
int fa_set_error(int status, const char *fmt, ...);
void fa_clear_error();
int fa_dtype_size(int dt);

// FA_LOG: when the environment variable FA_LOG is set to anything but "0"
// (read once), every launch prints one line to stderr before it is enqueued:
// "[fa] <kernel> grid=<n> block=<n> lds=<bytes> <what fmt describes>".
bool fa_log_enabled();
void fa_log_launch(const char *kernel, unsigned grid, unsigned block, unsigned lds_bytes, const char *fmt, ...)
    __attribute__((format(printf, 5, 6)));

// Everything fa_check_decode_params checks except the workspace.
int fa_check_decode_inputs(const fa_decode_params *p);

// Device address of fa_decode_kvq_noalloc's scratch array on the current
// device (FA_DECODE_NOALLOC_MAX_BYTES bytes), looked up once per device.
int fa_decode_scratch(void **ptr);

// Kernel launchers, one per kernel family (defined in the .hip files).  They
// assume validated parameters and return FA_OK or FA_ERR_HIP.
int fa_launch_fwd_mfma(const fa_fwd_params *p, void *stream);
int fa_launch_fwd_fp8(const fa_fwd_params *p, void *stream);
int fa_launch_decode(const fa_decode_params *p, void *stream);
int fa_launch_kv_append(const fa_kv_append_params *p, void *stream);
int fa_launch_bwd(const fa_bwd_params *p, void *stream);
int fa_launch_fp8_quantize(const fa_fp8_quant_params *p, void *stream);
