// C ABI entry points of libfa: validate on the host, then enqueue the kernels.
#include "fa_internal.h"

extern "C" int fa_fwd(const fa_fwd_params *p, fa_stream_t stream) {
  const int st = fa_check_fwd_params(p);
  if (st != FA_OK) return st;
  if (p->B == 0 || p->Sq == 0) return FA_OK;
  if (p->in_dtype == FA_FP8_E4M3) return fa_launch_fwd_fp8(p, stream);
  return fa_launch_fwd_mfma(p, stream);
}

extern "C" int fa_decode_kvq(const fa_decode_params *p, fa_stream_t stream) {
  const int st = fa_check_decode_params(p);
  if (st != FA_OK) return st;
  if (p->B == 0) return FA_OK;
  return fa_launch_decode(p, stream);
}

extern "C" int fa_kv_append(const fa_kv_append_params *p, fa_stream_t stream) {
  const int st = fa_check_kv_append_params(p);
  if (st != FA_OK) return st;
  if (p->B == 0 || p->T == 0 || p->L == 0) return FA_OK;
  return fa_launch_kv_append(p, stream);
}

extern "C" int fa_bwd(const fa_bwd_params *p, fa_stream_t stream) {
  const int st = fa_check_bwd_params(p);
  if (st != FA_OK) return st;
  if (p->B == 0 || (p->Sq == 0 && p->Sk == 0)) return FA_OK;
  return fa_launch_bwd(p, stream);
}

extern "C" int fa_fp8_quantize(const fa_fp8_quant_params *p, fa_stream_t stream) {
  const int st = fa_check_fp8_quant_params(p);
  if (st != FA_OK) return st;
  if (p->B == 0 || p->S == 0) return FA_OK;
  return fa_launch_fp8_quantize(p, stream);
}
