// Quantise-on-append: the write side of the quantised KV cache.
//
// What is computed (KV-cache quantisation overview, section 3, "before writing
// the cache" and "storage form"): each new key or value row — one token of one
// head, d = 128 bf16/fp16 values — becomes 128 one-byte codes and one fp16
// scale, symmetric, no zero point:
//   sc   = fp16(min(fp32(absmax / QMAX), 65504))        QMAX = 127 or 448
//   y    = fp32(x) / fp32(sc)                           correctly rounded
//   code = clamp(rint(y), -127, 127)                    int8
//        = E4M3FN(clamp(y, -448, 448)), nearest even    fp8
// and code 0 everywhere when sc == 0.  Row t of sequence b lands in cache slot
// positions[b] + t; slots outside [0, L) are skipped.
//
// MI355X design.  The work is a pure stream (256 bytes read, 130 written per
// row, no reuse), so it is shaped for HBM: a row is handled by one 16-lane
// group, each lane moving one 16-byte chunk in and one 8-byte chunk out, so a
// wavefront covers whole rows with fully coalesced 128-bit loads.  A group
// takes four consecutive rows, and with them the key row and the value row of
// each (batch, head, token): eight independent 16-byte loads are in flight per
// lane before the first is used, and the grid has a quarter as many
// workgroups as rows / 16.  The absmax is reduced over
// the group with lane exchanges only (no LDS, no barrier).  fp8 codes come from
// the hardware's packed E4M3FN conversion (round to nearest even), int8 codes
// from rint.
//
// The quotient x / sc is not a full IEEE division, yet every code equals the
// one the correctly rounded quotient gives.  With r the hardware reciprocal of
// sc, q0 = x r and one residual step q1 = q0 + (x - sc q0) r leave q1 within
// about one ulp of x / sc, and exactly equal to it whenever x / sc is
// representable.  A code can only depend on that ulp where x / sc lies next to
// a rounding boundary of the code (a half-integer for int8, a midpoint between
// neighbouring E4M3 values for fp8).  A boundary t = T 2^c has T below 2^9, sc
// = S 2^b has S below 2^11 (fp16) and x at most 11 significant bits (bf16 or
// fp16), so x - t sc is a multiple of 2^(b+c) or of x's own last bit: when x
// is close to t sc it is either zero or at least x / (T S) > 2^-20 x in size.
// x / sc is then either exactly on the boundary (q1 is exact and the tie goes
// to even, as for the correctly rounded quotient) or at least 2^-20 of its
// size away from it, well beyond the 2^-23 of an fp32 ulp.  The same holds
// for the clamp at +-QMAX.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

struct AppendArgs {
  const void *k_new;
  const void *v_new;
  unsigned char *k_cache;
  unsigned char *v_cache;
  _Float16 *k_scale;
  _Float16 *v_scale;
  const int *positions;
  unsigned rows;  // B * H * T, below 2^31
  int H, T, L;
  long long n_sb, n_sh, n_st;  // input strides, elements
  long long c_sb, c_sh, c_st;  // cache strides, bytes
  long long s_sb, s_sh;        // scale strides, elements
};

constexpr int kAppendThreads = 256;
constexpr int kGroupsPerBlock = kAppendThreads / 16;
constexpr int kRowsPerGroup = 4;
constexpr int kRowsPerBlock = kGroupsPerBlock * kRowsPerGroup;

// Eight input values of one 16-byte chunk, widened exactly to fp32.
template <bool BF16> __device__ __forceinline__ void widen8(const u32x4 w, float x[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    } else {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      // the element is copied out first: with this compiler, bit-casting the
      // vector-element expression w[i] itself yields element 0 for every i
      const unsigned wi = w[i];
      const h2 h = __builtin_bit_cast(h2, wi);
      x[2 * i] = static_cast<float>(h[0]);
      x[2 * i + 1] = static_cast<float>(h[1]);
    }
  }
}

// One row chunk -> 8 code bytes; sets sc16 to the row's scale.  Every lane of
// the 16-lane group must call it (the absmax is exchanged across the group).
template <bool BF16, bool FP8>
__device__ __forceinline__ u32x2 quantise8(const u32x4 raw, _Float16 &sc16) {
  float x[8];
  widen8<BF16>(raw, x);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  // the group's absmax by DPP exchanges within the 16-lane row
  amax = fmaxf(amax, row16_xor<8>(amax));
  amax = fmaxf(amax, row16_xor<4>(amax));
  amax = fmaxf(amax, row16_xor<2>(amax));
  amax = fmaxf(amax, row16_xor<1>(amax));
  constexpr float kQmax = FP8 ? 448.f : 127.f;
  sc16 = static_cast<_Float16>(fminf(amax / kQmax, 65504.f));
  const float scf = static_cast<float>(sc16);
  u32x2 out{0u, 0u};
  if (scf > 0.f) {
    float y[8];
    const float r = __builtin_amdgcn_rcpf(scf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = x[i] * r;
      const float q1 = __builtin_fmaf(__builtin_fmaf(-scf, q0, x[i]), r, q0);
      y[i] = fminf(fmaxf(q1, -kQmax), kQmax);
    }
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h], y[4 * h + 1], 0, false);
        out[h] = static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2], y[4 * h + 3], lo, true));
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        unsigned w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= (static_cast<unsigned>(static_cast<int>(rintf(y[4 * h + i]))) & 0xFFu) << (8 * i);
        out[h] = w;
      }
    }
  }
  return out;
}

template <bool BF16, bool FP8>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(const AppendArgs a) {
  const int tid = threadIdx.x;
  const int c = tid & 15;  // 8-element chunk of the row
  // rows < 2^31 (checked on the host), so 32-bit unsigned index math is exact;
  // the group takes kRowsPerGroup consecutive rows (consecutive tokens, so a
  // contiguous stretch of the input and of the cache)
  const unsigned r0 = (blockIdx.x * static_cast<unsigned>(kGroupsPerBlock) + static_cast<unsigned>(tid >> 4)) *
                      static_cast<unsigned>(kRowsPerGroup);
  // every lane stays live through the group exchange; only loads and stores
  // are predicated
  bool write[kRowsPerGroup];
  long long c_off[kRowsPerGroup], s_off[kRowsPerGroup];
  u32x4 kx[kRowsPerGroup], vx[kRowsPerGroup];
#pragma unroll
  for (int i = 0; i < kRowsPerGroup; ++i) {
    const unsigned r = r0 + i;
    write[i] = false;
    c_off[i] = s_off[i] = 0;
    long long in_off = 0;
    if (r < a.rows) {
      const int t = static_cast<int>(r % static_cast<unsigned>(a.T));
      const unsigned bh = r / static_cast<unsigned>(a.T);
      const int h = static_cast<int>(bh % static_cast<unsigned>(a.H));
      const long long b = bh / static_cast<unsigned>(a.H);
      const long long slot = static_cast<long long>(a.positions != nullptr ? a.positions[b] : 0) + t;
      write[i] = slot >= 0 && slot < a.L;
      in_off = b * a.n_sb + h * a.n_sh + t * a.n_st + 8 * c;
      c_off[i] = b * a.c_sb + h * a.c_sh + slot * a.c_st + 8 * c;
      s_off[i] = b * a.s_sb + h * a.s_sh + slot;
    }
    kx[i] = vx[i] = u32x4{0u, 0u, 0u, 0u};
    if (write[i]) {  // all loads of the group issued before any is used
      kx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(static_cast<const unsigned short *>(a.k_new) + in_off));
      vx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(static_cast<const unsigned short *>(a.v_new) + in_off));
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerGroup; ++i) {
    _Float16 ks, vs;
    const u32x2 kq = quantise8<BF16, FP8>(kx[i], ks);
    const u32x2 vq = quantise8<BF16, FP8>(vx[i], vs);
    if (write[i]) {
      // the cache is written once here and read by a later decode step, not by
      // this kernel: stream the codes past the caches (non-temporal stores)
      __builtin_nontemporal_store(kq, reinterpret_cast<u32x2 *>(a.k_cache + c_off[i]));
      __builtin_nontemporal_store(vq, reinterpret_cast<u32x2 *>(a.v_cache + c_off[i]));
      if (c == 0) {
        a.k_scale[s_off[i]] = ks;
        a.v_scale[s_off[i]] = vs;
      }
    }
  }
}

}  // namespace fa

int fa_launch_kv_append(const fa_kv_append_params *p, void *stream) {
  using namespace fa;
  AppendArgs a{};
  a.k_new = p->k_new;
  a.v_new = p->v_new;
  a.k_cache = static_cast<unsigned char *>(p->k_cache);
  a.v_cache = static_cast<unsigned char *>(p->v_cache);
  a.k_scale = static_cast<_Float16 *>(p->k_scale);
  a.v_scale = static_cast<_Float16 *>(p->v_scale);
  a.positions = p->positions;
  a.rows = static_cast<unsigned>(static_cast<long long>(p->B) * p->H * p->T);
  a.H = p->H;
  a.T = p->T;
  a.L = p->L;
  a.n_sb = p->new_strides[0];
  a.n_sh = p->new_strides[1];
  a.n_st = p->new_strides[2];
  a.c_sb = p->kv_strides[0];
  a.c_sh = p->kv_strides[1];
  a.c_st = p->kv_strides[2];
  a.s_sb = p->scale_strides[0];
  a.s_sh = p->scale_strides[1];
  const unsigned blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = p->in_dtype == FA_BF16;
  const bool fp8 = p->kv_format == FA_KV_FP8_E4M3_TOKHEAD_F16SCALE;
  const dim3 grid(blocks), block(kAppendThreads);
  fa_log_launch("kv_append_kernel", blocks, kAppendThreads, 0, "in=%s kv=%s B=%d H=%d T=%d L=%d",
                bf16 ? "bf16" : "f16", fp8 ? "fp8" : "int8", p->B, p->H, p->T, p->L);
  if (bf16 && fp8) hipLaunchKernelGGL((kv_append_kernel<true, true>), grid, block, 0, s, a);
  else if (bf16) hipLaunchKernelGGL((kv_append_kernel<true, false>), grid, block, 0, s, a);
  else if (fp8) hipLaunchKernelGGL((kv_append_kernel<false, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((kv_append_kernel<false, false>), grid, block, 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "kv append launch: %s", hipGetErrorString(e));
  return FA_OK;
}
