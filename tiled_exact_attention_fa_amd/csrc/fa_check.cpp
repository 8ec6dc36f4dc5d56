// Host-only parameter validation for the libfa C ABI.  No HIP call is made here,
// so every error path can be exercised on a machine without a GPU.
#include "fa_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

namespace {
thread_local char g_last_error[512] = "";
}

extern "C" const char *fa_last_error(void) { return g_last_error; }

int fa_set_error(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void fa_clear_error() { g_last_error[0] = '\0'; }

bool fa_log_enabled() {
  static const bool on = [] {
    const char *e = std::getenv("FA_LOG");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
  }();
  return on;
}

void fa_log_launch(const char *kernel, unsigned grid, unsigned block, unsigned lds_bytes, const char *fmt, ...) {
  if (!fa_log_enabled()) return;
  char what[256];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(what, sizeof(what), fmt, ap);
  va_end(ap);
  // one fprintf per line, so lines from several threads do not interleave
  std::fprintf(stderr, "[fa] %s grid=%u block=%u lds=%u %s\n", kernel, grid, block, lds_bytes, what);
}

extern "C" const char *fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_ALIGNMENT: return "FA_ERR_ALIGNMENT";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_ERR_UNKNOWN";
  }
}

int fa_dtype_size(int dt) {
  switch (dt) {
    case FA_F32: return 4;
    case FA_F16: case FA_BF16: return 2;
    case FA_FP8_E4M3: case FA_INT8: return 1;
    default: return 0;
  }
}

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One tensor of `rows` rows of `d` elements per (batch, head) slice.
int check_tensor(const char *name, const void *ptr, const int64_t *strides, int nstr, int rows,
                 int d, int esize) {
  if (ptr == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fa_set_error(FA_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  for (int i = 0; i < nstr; ++i) {
    if (strides[i] < 0)
      return fa_set_error(FA_ERR_INVALID_ARG, "%s stride %d is negative", name, i);
    if ((strides[i] * esize) % 16 != 0)
      return fa_set_error(FA_ERR_ALIGNMENT, "%s stride %d (%lld elements) is not a multiple of 16 bytes",
                          name, i, static_cast<long long>(strides[i]));
  }
  if (nstr == 3) {
    if (rows > 1 && strides[2] < d)
      return fa_set_error(FA_ERR_INVALID_ARG, "%s sequence stride %lld < d=%d (rows overlap)", name,
                          static_cast<long long>(strides[2]), d);
    // The kernels form row * stride in 32 bits for every row of a tile (up to
    // 256), including rows past the end that the buffer range then reads as
    // zero; above 8 MiB per row such an offset could wrap back inside the
    // slice.  Checked whatever `rows` is: a short tensor still has full tiles.
    if (strides[2] * esize > (int64_t(1) << 23))
      return fa_set_error(FA_ERR_UNSUPPORTED, "%s sequence stride %lld elements exceeds 8 MiB per row", name,
                          static_cast<long long>(strides[2]));
    const int64_t extent = (static_cast<int64_t>(rows > 0 ? rows - 1 : 0) * strides[2] + d) * esize;
    if (extent >= (int64_t(1) << 31))
      return fa_set_error(FA_ERR_UNSUPPORTED, "%s: one (batch, head) slice spans %lld bytes (limit 2^31)",
                          name, static_cast<long long>(extent));
  }
  return FA_OK;
}

}  // namespace

extern "C" int fa_check_fwd_params(const fa_fwd_params *p) {
  fa_clear_error();
  if (p == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Sq < 0 || p->Sk < 0 || p->d <= 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "bad sizes B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d", p->B, p->Hq,
                        p->Hkv, p->Sq, p->Sk, p->d);
  if (p->Hq % p->Hkv != 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->d != 64 && p->d != 128)
    return fa_set_error(FA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", p->d);
  const int in = p->in_dtype, out = p->out_dtype;
  const bool pair_ok = (in == FA_F32 && out == FA_F32) || (in == FA_BF16 && out == FA_BF16) ||
                       (in == FA_F16 && out == FA_F16) || (in == FA_FP8_E4M3 && out == FA_BF16);
  if (!pair_ok)
    return fa_set_error(FA_ERR_UNSUPPORTED, "dtype pair in=%d out=%d not supported", in, out);
  if (in == FA_FP8_E4M3 && p->d != 128)
    return fa_set_error(FA_ERR_UNSUPPORTED, "fp8 forward supports head dim 128 only (d=%d)", p->d);
  if (p->fp8_p_bf16 != 0 && p->fp8_p_bf16 != 1)
    return fa_set_error(FA_ERR_INVALID_ARG, "fp8_p_bf16 must be 0 or 1");
  if (p->fp8_p_bf16 != 0 && in != FA_FP8_E4M3)
    return fa_set_error(FA_ERR_INVALID_ARG, "fp8_p_bf16 applies to fp8 inputs only");
  if (p->soft_exp2 != 0 && p->soft_exp2 != 1)
    return fa_set_error(FA_ERR_INVALID_ARG, "soft_exp2 must be 0 or 1");
  if (p->soft_exp2 != 0 && !((in == FA_BF16 || in == FA_F16) && p->d == 128))
    return fa_set_error(FA_ERR_UNSUPPORTED, "soft_exp2 is built for bf16/fp16 inputs with d = 128");
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f))
    return fa_set_error(FA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const int nblk = (p->q_block_descale != nullptr) + (p->k_block_descale != nullptr) + (p->v_block_descale != nullptr);
  if (nblk != 0 && nblk != 3)
    return fa_set_error(FA_ERR_INVALID_ARG, "block descales: give all three of q, k, v or none");
  if (nblk == 3) {
    if (in != FA_FP8_E4M3) return fa_set_error(FA_ERR_INVALID_ARG, "block descales need fp8 inputs");
    for (const float *bp : {p->q_block_descale, p->k_block_descale, p->v_block_descale})
      if ((reinterpret_cast<uintptr_t>(bp) & 3u) != 0)
        return fa_set_error(FA_ERR_ALIGNMENT, "block descales not 4-byte aligned");
  } else if (in == FA_FP8_E4M3) {
    const float ds[3] = {p->q_descale, p->k_descale, p->v_descale};
    for (float x : ds)
      if (!(std::isfinite(x) && x > 0.f))
        return fa_set_error(FA_ERR_INVALID_ARG, "fp8 descales must be finite and > 0");
  }
  if (p->B == 0 || p->Sq == 0) return FA_OK;  // nothing to compute or write
  const int ie = fa_dtype_size(in), oe = fa_dtype_size(out);
  int st;
  if ((st = check_tensor("q", p->q, p->q_strides, 3, p->Sq, p->d, ie)) != FA_OK) return st;
  if ((st = check_tensor("o", p->o, p->o_strides, 3, p->Sq, p->d, oe)) != FA_OK) return st;
  if (p->Sk > 0) {
    if ((st = check_tensor("k", p->k, p->k_strides, 3, p->Sk, p->d, ie)) != FA_OK) return st;
    if ((st = check_tensor("v", p->v, p->v_strides, 3, p->Sk, p->d, ie)) != FA_OK) return st;
  }
  if (p->lse != nullptr) {
    if ((reinterpret_cast<uintptr_t>(p->lse) & 3u) != 0)
      return fa_set_error(FA_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    if (p->lse_strides[0] < 0 || p->lse_strides[1] < 0)
      return fa_set_error(FA_ERR_INVALID_ARG, "lse strides must be >= 0");
  }
  return FA_OK;
}

extern "C" size_t fa_decode_workspace_size(int32_t B, int32_t Hq, int32_t d, int32_t num_splits) {
  if (B < 0 || Hq <= 0 || d <= 0 || num_splits <= 0 || num_splits > FA_DECODE_MAX_SPLITS) return 0;
  // per (split, batch, query head): d partial outputs + one log-sum-exp, float32
  const size_t rows = static_cast<size_t>(num_splits) * static_cast<size_t>(B) * static_cast<size_t>(Hq);
  const size_t o_bytes = rows * static_cast<size_t>(d) * sizeof(float);
  const size_t l_bytes = rows * sizeof(float);
  return ((o_bytes + 255) & ~size_t(255)) + ((l_bytes + 255) & ~size_t(255));
}

// Everything fa_check_decode_params checks except the workspace.
int fa_check_decode_inputs(const fa_decode_params *p) {
  fa_clear_error();
  if (p == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "params is NULL");
  if (p->kv_format != FA_KV_INT8_TOKHEAD_F16SCALE && p->kv_format != FA_KV_FP8_E4M3_TOKHEAD_F16SCALE)
    return fa_set_error(FA_ERR_UNSUPPORTED, "kv_format %d not supported", p->kv_format);
  if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->L < 0 || p->d <= 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "bad sizes B=%d Hq=%d Hkv=%d L=%d d=%d", p->B, p->Hq, p->Hkv,
                        p->L, p->d);
  if (p->Hq % p->Hkv != 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->Hq / p->Hkv > FA_DECODE_MAX_GROUP)
    return fa_set_error(FA_ERR_UNSUPPORTED, "query heads per cache head %d > %d", p->Hq / p->Hkv,
                        FA_DECODE_MAX_GROUP);
  if (p->d != 128) return fa_set_error(FA_ERR_UNSUPPORTED, "decode head dim %d not supported (128)", p->d);
  if (p->num_splits < 1 || p->num_splits > FA_DECODE_MAX_SPLITS)
    return fa_set_error(FA_ERR_INVALID_ARG, "num_splits=%d outside [1, %d]", p->num_splits,
                        FA_DECODE_MAX_SPLITS);
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f))
    return fa_set_error(FA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (p->B == 0) return FA_OK;
  int st;
  if ((st = check_tensor("q", p->q, p->q_strides, 2, 1, p->d, 2)) != FA_OK) return st;
  if ((st = check_tensor("o", p->o, p->o_strides, 2, 1, p->d, 2)) != FA_OK) return st;
  if (p->L > 0) {
    if ((st = check_tensor("k_cache", p->k_cache, p->kv_strides, 3, p->L, p->d, 1)) != FA_OK) return st;
    if ((st = check_tensor("v_cache", p->v_cache, p->kv_strides, 3, p->L, p->d, 1)) != FA_OK) return st;
    for (const void *sp : {p->k_scale, p->v_scale}) {
      if (sp == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "k_scale/v_scale is NULL");
      if ((reinterpret_cast<uintptr_t>(sp) & 1u) != 0)
        return fa_set_error(FA_ERR_ALIGNMENT, "k_scale/v_scale not 2-byte aligned");
    }
    for (int i = 0; i < 2; ++i)
      if (p->scale_strides[i] < 0)
        return fa_set_error(FA_ERR_INVALID_ARG, "scale stride %d is negative", i);
    const int64_t sext = static_cast<int64_t>(p->L) * 2;
    if (sext >= (int64_t(1) << 31)) return fa_set_error(FA_ERR_UNSUPPORTED, "scale slice too large");
  }
  if (p->lse != nullptr && (p->lse_strides[0] < 0 || p->lse_strides[1] < 0))
    return fa_set_error(FA_ERR_INVALID_ARG, "lse strides must be >= 0");
  if (p->W < 0) return fa_set_error(FA_ERR_INVALID_ARG, "window length W=%d is negative", p->W);
  if (p->W > 0) {
    if ((st = check_tensor("k_recent", p->k_recent, p->recent_strides, 3, p->W, p->d, 2)) != FA_OK) return st;
    if ((st = check_tensor("v_recent", p->v_recent, p->recent_strides, 3, p->W, p->d, 2)) != FA_OK) return st;
  }
  return FA_OK;
}

extern "C" int fa_check_decode_params(const fa_decode_params *p) {
  const int st = fa_check_decode_inputs(p);
  if (st != FA_OK || p->B == 0) return st;
  // the window's partial takes one more slot of the workspace
  const size_t need = fa_decode_workspace_size(p->B, p->Hq, p->d, p->num_splits + (p->W > 0 ? 1 : 0));
  if (p->workspace == nullptr || p->workspace_bytes < need)
    return fa_set_error(FA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", p->workspace_bytes, need);
  if (!aligned16(p->workspace)) return fa_set_error(FA_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  return FA_OK;
}

extern "C" int fa_check_kv_append_params(const fa_kv_append_params *p) {
  fa_clear_error();
  if (p == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "params is NULL");
  if (p->kv_format != FA_KV_INT8_TOKHEAD_F16SCALE && p->kv_format != FA_KV_FP8_E4M3_TOKHEAD_F16SCALE)
    return fa_set_error(FA_ERR_UNSUPPORTED, "kv_format %d not supported", p->kv_format);
  if (p->in_dtype != FA_BF16 && p->in_dtype != FA_F16)
    return fa_set_error(FA_ERR_UNSUPPORTED, "append input dtype %d not supported (bf16 or fp16)", p->in_dtype);
  if (p->B < 0 || p->H <= 0 || p->T < 0 || p->L < 0 || p->d <= 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "bad sizes B=%d H=%d T=%d L=%d d=%d", p->B, p->H, p->T, p->L, p->d);
  if (p->d != 128) return fa_set_error(FA_ERR_UNSUPPORTED, "append head dim %d not supported (128)", p->d);
  if (static_cast<int64_t>(p->B) * p->H * p->T >= (int64_t(1) << 31))
    return fa_set_error(FA_ERR_UNSUPPORTED, "B*H*T rows exceed 2^31");
  if (p->B == 0 || p->T == 0 || p->L == 0) return FA_OK;  // nothing can be written
  int st;
  if ((st = check_tensor("k_new", p->k_new, p->new_strides, 3, p->T, p->d, 2)) != FA_OK) return st;
  if ((st = check_tensor("v_new", p->v_new, p->new_strides, 3, p->T, p->d, 2)) != FA_OK) return st;
  if ((st = check_tensor("k_cache", p->k_cache, p->kv_strides, 3, p->L, p->d, 1)) != FA_OK) return st;
  if ((st = check_tensor("v_cache", p->v_cache, p->kv_strides, 3, p->L, p->d, 1)) != FA_OK) return st;
  for (const void *sp : {static_cast<const void *>(p->k_scale), static_cast<const void *>(p->v_scale)}) {
    if (sp == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "k_scale/v_scale is NULL");
    if ((reinterpret_cast<uintptr_t>(sp) & 1u) != 0)
      return fa_set_error(FA_ERR_ALIGNMENT, "k_scale/v_scale not 2-byte aligned");
  }
  for (int i = 0; i < 2; ++i)
    if (p->scale_strides[i] < 0) return fa_set_error(FA_ERR_INVALID_ARG, "scale stride %d is negative", i);
  return FA_OK;
}

extern "C" size_t fa_bwd_workspace_size(int32_t B, int32_t Hq, int32_t Sq) {
  if (B < 0 || Hq <= 0 || Sq < 0) return 0;
  const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(Hq) * static_cast<size_t>(Sq);
  return ((rows * sizeof(float) + 255) & ~size_t(255)) + 256;
}

extern "C" int fa_check_bwd_params(const fa_bwd_params *p) {
  fa_clear_error();
  if (p == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Sq < 0 || p->Sk < 0 || p->d <= 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "bad sizes B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d", p->B, p->Hq,
                        p->Hkv, p->Sq, p->Sk, p->d);
  if (p->Hq % p->Hkv != 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->d != 128) return fa_set_error(FA_ERR_UNSUPPORTED, "backward head dim %d not supported (128)", p->d);
  if (p->dtype != FA_BF16 && p->dtype != FA_F16)
    return fa_set_error(FA_ERR_UNSUPPORTED, "backward dtype %d not supported (bf16 or fp16)", p->dtype);
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f))
    return fa_set_error(FA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (p->wave_pingpong != 0 && p->wave_pingpong != 1)
    return fa_set_error(FA_ERR_INVALID_ARG, "wave_pingpong must be 0 or 1");
  if (p->B == 0 || (p->Sq == 0 && p->Sk == 0)) return FA_OK;
  int st;
  if (p->Sq > 0) {
    if ((st = check_tensor("q", p->q, p->q_strides, 3, p->Sq, p->d, 2)) != FA_OK) return st;
    if ((st = check_tensor("o", p->o, p->o_strides, 3, p->Sq, p->d, 2)) != FA_OK) return st;
    if ((st = check_tensor("dout", p->dout, p->do_strides, 3, p->Sq, p->d, 2)) != FA_OK) return st;
    if ((st = check_tensor("dq", p->dq, p->dq_strides, 3, p->Sq, p->d, 2)) != FA_OK) return st;
    if (p->lse == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "lse is NULL");
    if ((reinterpret_cast<uintptr_t>(p->lse) & 3u) != 0)
      return fa_set_error(FA_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    if (p->lse_strides[0] < 0 || p->lse_strides[1] < 0)
      return fa_set_error(FA_ERR_INVALID_ARG, "lse strides must be >= 0");
  }
  if (p->Sk > 0) {
    if ((st = check_tensor("k", p->k, p->k_strides, 3, p->Sk, p->d, 2)) != FA_OK) return st;
    if ((st = check_tensor("v", p->v, p->v_strides, 3, p->Sk, p->d, 2)) != FA_OK) return st;
    if ((st = check_tensor("dk", p->dk, p->dk_strides, 3, p->Sk, p->d, 2)) != FA_OK) return st;
    if ((st = check_tensor("dv", p->dv, p->dv_strides, 3, p->Sk, p->d, 2)) != FA_OK) return st;
  }
  const size_t need = fa_bwd_workspace_size(p->B, p->Hq, p->Sq);
  if (p->workspace == nullptr || p->workspace_bytes < need)
    return fa_set_error(FA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", p->workspace_bytes, need);
  if (!aligned16(p->workspace)) return fa_set_error(FA_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  return FA_OK;
}

extern "C" int fa_check_fp8_quant_params(const fa_fp8_quant_params *p) {
  fa_clear_error();
  if (p == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "params is NULL");
  if (p->in_dtype != FA_BF16 && p->in_dtype != FA_F16)
    return fa_set_error(FA_ERR_UNSUPPORTED, "quantise input dtype %d not supported (bf16 or fp16)", p->in_dtype);
  if (p->B < 0 || p->H <= 0 || p->S < 0 || p->d <= 0)
    return fa_set_error(FA_ERR_INVALID_ARG, "bad sizes B=%d H=%d S=%d d=%d", p->B, p->H, p->S, p->d);
  if (p->d != 128) return fa_set_error(FA_ERR_UNSUPPORTED, "quantise head dim %d not supported (128)", p->d);
  if (static_cast<int64_t>(p->B) * p->H * ((p->S + 63) / 64) >= (int64_t(1) << 31))
    return fa_set_error(FA_ERR_UNSUPPORTED, "too many blocks");
  if (p->B == 0 || p->S == 0) return FA_OK;
  int st;
  if ((st = check_tensor("x", p->x, p->x_strides, 3, p->S, p->d, 2)) != FA_OK) return st;
  if ((st = check_tensor("codes", p->codes, p->codes_strides, 3, p->S, p->d, 1)) != FA_OK) return st;
  if (p->scales == nullptr) return fa_set_error(FA_ERR_INVALID_ARG, "scales is NULL");
  if ((reinterpret_cast<uintptr_t>(p->scales) & 3u) != 0)
    return fa_set_error(FA_ERR_ALIGNMENT, "scales not 4-byte aligned");
  if (p->signs != nullptr && (reinterpret_cast<uintptr_t>(p->signs) & 3u) != 0)
    return fa_set_error(FA_ERR_ALIGNMENT, "signs not 4-byte aligned");
  return FA_OK;
}
