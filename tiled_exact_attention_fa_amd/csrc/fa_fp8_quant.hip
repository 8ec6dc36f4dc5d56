// fp8 inputs for the prefill: 64-row block scales, optional incoherent
// processing (a random-sign Hadamard rotation of each row).
//
// What is computed (FlashAttention-3 page, producer/consumer pseudocode box,
// "FP8 path": block-scale Q/K/V, incoherent processing reduces the error):
// for each 64-row block of a (batch, head) slice,
//   y    = x                                   or  y = (x * signs) H / sqrt(d)
//   s    = the smallest power of two at or above fp32(absmax(y) / 448)
//   code = E4M3FN(clamp(y / s, +-448)), nearest even;   s == 0: code 0
// (power-of-two block scales keep the ratio of any two of them a power of two,
// which the attention kernel relies on when it folds a V block's scale into
// the probabilities before their own e4m3 rounding)
// with H the Sylvester-Hadamard matrix of order d = 128.  Rotating Q and K by
// the same orthogonal matrix leaves Q K^T unchanged and spreads a channel
// outlier over all channels.  The rotation is the iterative fast transform in
// float32 — stages h = 1, 2, 4, ..., 64, each (a, b) -> (a + b, a - b) on pairs
// h apart — followed by one multiply by fp32(1/sqrt(128)); every rounding step
// is fixed, so the codes are reproducible bit for bit.
//
// MI355X design.  One workgroup of 256 threads per block: 16 lane groups of 16,
// each lane holding one 16-byte chunk (8 elements) of a row, a group 4 rows.
// The transform's first three stages stay inside a lane, the last four are
// lane exchanges within the group (xor 1, 2, 4, 8), each one or two DPP moves
// on the vector ALU rather than an LDS permute; the block absmax goes through
// the group's lanes and then 16 LDS words; y / s is one exponent adjustment
// (s is a power of two, so y * 2^-k is the correctly rounded quotient); codes
// leave as one 8-byte store per lane and row.  The whole block stays in
// registers between the absmax and the encode, so every input byte is read
// once.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

struct QuantArgs {
  const void *x;
  unsigned char *codes;
  float *scales;       // [B][H][nb]
  const float *signs;  // [128] or null
  int H, S, nb;
  long long x_sb, x_sh, x_ss;  // elements
  long long c_sb, c_sh, c_ss;  // bytes
};

constexpr int kQRows = 64;  // rows per block

// one transform stage across lanes: the lane whose chunk has bit X clear holds
// a (takes a + b), the other holds b (takes a - b).  Both are other + sgn * y
// with sgn = +-1 (bit X of the chunk): the product is exact and the sum is the
// same correctly rounded a + b or a - b, so the stage costs one multiply and
// one add whose other operand arrives through DPP.
template <int X>
__device__ __forceinline__ void xstage(float (&y)[8], float sgn) {
  // kept as a separate multiply and add (a fused form ties the add's output
  // to a register the DPP move must fill first)
#pragma clang fp contract(off)
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = row16_xor<X>(y[e]) + sgn * y[e];
}

template <bool BF16, bool ROT>
__global__ __launch_bounds__(256) void fp8_block_quant_kernel(const QuantArgs a) {
  __shared__ float s_max[16];
  const int tid = threadIdx.x;
  const int c = tid & 15;  // chunk: elements 8c .. 8c + 7
  const int g = tid >> 4;  // lane group: rows 4g .. 4g + 3 of the block
  const int blk = blockIdx.x % a.nb;
  const int bh = blockIdx.x / a.nb;
  const long long b = bh / a.H, h = bh % a.H;

  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = ROT ? a.signs[8 * c + e] : 1.f;

  float y[4][8];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = blk * kQRows + 4 * g + r;
    u32x4 raw{0u, 0u, 0u, 0u};
    if (row < a.S)  // read once: non-temporal
      raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
          static_cast<const unsigned short *>(a.x) + b * a.x_sb + h * a.x_sh + row * a.x_ss + 8 * c));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned w = raw[i];
      if constexpr (BF16) {
        y[r][2 * i] = __builtin_bit_cast(float, w << 16);
        y[r][2 * i + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
      } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 hv = __builtin_bit_cast(h2, w);
        y[r][2 * i] = static_cast<float>(hv[0]);
        y[r][2 * i + 1] = static_cast<float>(hv[1]);
      }
    }
    if constexpr (ROT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[r][e] *= sg[e];  // exact: +-1
      // stages h = 1, 2, 4 inside the lane
#pragma unroll
      for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & hs) == 0) {
            const float p = y[r][e], q = y[r][e + hs];
            y[r][e] = p + q;
            y[r][e + hs] = p - q;
          }
      // stages h = 8, 16, 32, 64 across the group
      xstage<1>(y[r], (c & 1) ? -1.f : 1.f);
      xstage<2>(y[r], (c & 2) ? -1.f : 1.f);
      xstage<4>(y[r], (c & 4) ? -1.f : 1.f);
      xstage<8>(y[r], (c & 8) ? -1.f : 1.f);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[r][e] *= 0.08838834764831845f;  // fp32(1/sqrt(128))
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[r][e]));
  }
  amax = fmaxf(amax, row16_xor<8>(amax));
  amax = fmaxf(amax, row16_xor<4>(amax));
  amax = fmaxf(amax, row16_xor<2>(amax));
  amax = fmaxf(amax, row16_xor<1>(amax));
  if (c == 0) s_max[g] = amax;
  __syncthreads();
  float bmax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, s_max[i]);
  // the smallest power of two at or above absmax / 448 (0 for an all-zero block)
  const float q448 = bmax / 448.f;
  int ex;
  const float mant = frexpf(q448, &ex);
  const int sexp = mant == 0.5f ? ex - 1 : ex;  // s = 2^sexp
  const float sc = q448 > 0.f ? ldexpf(1.f, sexp) : 0.f;
  if (tid == 0) a.scales[bh * static_cast<long long>(a.nb) + blk] = sc;

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = blk * kQRows + 4 * g + r;
    if (row >= a.S) continue;
    u32x2 out{0u, 0u};
    if (sc > 0.f) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = fminf(fmaxf(ldexpf(y[r][4 * hh + e], -sexp), -448.f), 448.f);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        out[hh] = static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true));
      }
    }
    // written once, read by a later kernel: non-temporal
    __builtin_nontemporal_store(out, reinterpret_cast<u32x2 *>(a.codes + b * a.c_sb + h * a.c_sh + row * a.c_ss + 8 * c));
  }
}

}  // namespace fa

int fa_launch_fp8_quantize(const fa_fp8_quant_params *p, void *stream) {
  using namespace fa;
  QuantArgs a{};
  a.x = p->x;
  a.codes = static_cast<unsigned char *>(p->codes);
  a.scales = p->scales;
  a.signs = p->signs;
  a.H = p->H;
  a.S = p->S;
  a.nb = (p->S + kQRows - 1) / kQRows;
  a.x_sb = p->x_strides[0];
  a.x_sh = p->x_strides[1];
  a.x_ss = p->x_strides[2];
  a.c_sb = p->codes_strides[0];
  a.c_sh = p->codes_strides[1];
  a.c_ss = p->codes_strides[2];
  const dim3 grid(static_cast<unsigned>(p->B) * p->H * a.nb), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = p->in_dtype == FA_BF16, rot = p->signs != nullptr;
  fa_log_launch("fp8_block_quant_kernel", grid.x, 256, 0, "in=%s rotate=%d B=%d H=%d S=%d", bf16 ? "bf16" : "f16",
                rot ? 1 : 0, p->B, p->H, p->S);
  if (bf16 && rot) hipLaunchKernelGGL((fp8_block_quant_kernel<true, true>), grid, block, 0, s, a);
  else if (bf16) hipLaunchKernelGGL((fp8_block_quant_kernel<true, false>), grid, block, 0, s, a);
  else if (rot) hipLaunchKernelGGL((fp8_block_quant_kernel<false, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((fp8_block_quant_kernel<false, false>), grid, block, 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "fp8 quantise launch: %s", hipGetErrorString(e));
  return FA_OK;
}
