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

extern "C" int fa_decode_kvq_noalloc(const fa_decode_params *p, fa_stream_t stream) {
  int st = fa_check_decode_inputs(p);
  if (st != FA_OK) return st;
  if (p->B == 0) return FA_OK;
  // the window's partial takes one more slot, as in fa_decode_kvq
  const size_t need = fa_decode_workspace_size(p->B, p->Hq, p->d, p->num_splits + (p->W > 0 ? 1 : 0));
  if (need > FA_DECODE_NOALLOC_MAX_BYTES)
    return fa_set_error(FA_ERR_WORKSPACE,
                        "fa_decode_kvq_noalloc: these sizes need %zu bytes of partial results, more than its "
                        "%d-byte scratch; use fa_decode_kvq with a workspace",
                        need, FA_DECODE_NOALLOC_MAX_BYTES);
  fa_decode_params q = *p;
  if ((st = fa_decode_scratch(&q.workspace)) != FA_OK) return st;
  q.workspace_bytes = FA_DECODE_NOALLOC_MAX_BYTES;
  return fa_launch_decode(&q, stream);
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
