// Prefill forward for fp8 (OCP E4M3FN) Q/K/V with per-tensor descales,
// bf16 output, on gfx950 8-bit matrix cores.
//
// Method: as the 16-bit kernel (FlashAttention interview canvas, panel 1
// "one-sentence answer" and "online softmax key state" boxes), with both
// products on fp8 MFMA, the low-precision lever of the FlashAttention-3 page
// ("new bottleneck on Hopper" box).  The three descales are folded into the
// score constant (q and k) and into the epilogue (v), so the codes feed the
// matrix cores unchanged.
//
// MI355X design.
//   * S^T = K Q^T and O^T = V^T P^T use the 32x32x64 f8f6f4 MFMA (each lane
//     supplies 32 bytes per operand).  The K tile is written to LDS in the row
//     order that makes lane half h's 32 score accumulators the keys
//     32h .. 32h+31 of the tile, i.e. exactly the 32 P^T bytes it feeds to the
//     next product; the matching V^T bytes are one contiguous 32-byte LDS read.
//   * P = exp2(s - m) is scaled by kPScale before it is rounded to e4m3, so
//     that small probabilities stay normal numbers; the factor is removed with
//     the row sum in the epilogue.  The row sum itself uses the unrounded fp32
//     probabilities.
//   * V is transposed in registers (4 keys x 8 columns per thread, byte
//     permutes) on its way into a double-buffered LDS stage.
#include "fa_device.hpp"
#include "fa_fwd_common.hpp"
#include "fa_internal.h"

#include <mutex>

namespace fa {

namespace f8 {

constexpr int BR = 128;   // query rows per workgroup (4 wavefronts x 32)
constexpr int BC = 64;    // keys per tile: one 64-deep MFMA for P V
constexpr int D = 128;
constexpr int KROW = D + 16;   // bytes per K row in LDS
constexpr int VROW = BC + 16;  // bytes per V^T row in LDS
constexpr int K_TILE = BC * KROW;
constexpr int V_TILE = D * VROW;
constexpr int STAGE = K_TILE + V_TILE;
constexpr int LDS_BYTES = 2 * STAGE;
// P is multiplied by kPScale before rounding to e4m3 (max 448).  With the
// lazy running max, P itself can reach 2^kSlack8, so kPScale * 2^kSlack8 = 256
// keeps every scaled probability at or below 256, and probabilities down to
// 2^-10 of the running max stay normal e4m3 numbers.
constexpr float kSlack8 = 4.0f;
constexpr float kPScale = 16.f;
constexpr float kLog2PScale = 4.f;

// LDS row of key kr of a tile: block mb = (kr >> 4) & 1, half h = kr >> 5,
// register i = kr & 15 of that block's accumulator, whose C row is
// 8 * (i >> 2) + 4 * h + (i & 3).
__device__ __forceinline__ int k_lds_row(int kr) {
  const int h = kr >> 5, mb = (kr >> 4) & 1, i = kr & 15;
  return 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
}

__device__ __forceinline__ f32x16 mma(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = E4M3 for both operands; block scales 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

}  // namespace f8

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void fwd_fp8_kernel(const FwdArgs a) {
  using namespace f8;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, a.nq, a.B * a.Hq, CAUSAL, bh, qt);
  const int b = bh / a.Hq, hq = bh - b * a.Hq, hk = hq / a.G;
  const int i0 = qt * BR;
  const int wrow0 = i0 + 32 * wave;
  const int row = wrow0 + l32;

  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(static_cast<const unsigned char *>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_ext);

  // Q: lane half h holds bytes [64h, 64h + 64) of its row; step s uses 32 of them
  i32x8 qf[2];
  {
    const bool ok = row < a.Sq;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const unsigned base = ok ? row * a.q_ss + 64u * h + 32u * s : kOOB;
      const u32x4 lo = buf_load16(rq, base);
      const u32x4 hi = buf_load16(rq, ok ? base + 16u : kOOB);
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    wait_vmem_all();
  }

  const int coff = a.Sk - a.Sq;
  int n_kt = (a.Sk + BC - 1) / BC;
  int w_kt = n_kt;
  if (CAUSAL) {
    const int last_wg = i0 + BR - 1 + coff;
    n_kt = min(n_kt, last_wg < 0 ? 0 : last_wg / BC + 1);
    const int last_w = wrow0 + 31 + coff;
    w_kt = min(n_kt, last_w < 0 ? 0 : last_w / BC + 1);
  }

  // K: thread t loads rows t/8 and t/8 + 32, 16-byte chunk t%8.
  // V: thread t loads keys 4*(t%16) .. +3 of the 8-byte column chunk t/16.
  // Loads go through a buffer resource placed at the tile's first row, so the
  // lane offsets are loop constants and rows past the keys read as zero.
  u32x4 kreg[2];
  u32x2 vreg[4];
  const int k_c = tid & 7, k_r = tid >> 3;
  const int v_g = tid & 15, v_c = tid >> 4;
  const unsigned char *kbase = static_cast<const unsigned char *>(a.k) + b * a.k_sb + hk * a.k_sh;
  const unsigned char *vbase = static_cast<const unsigned char *>(a.v) + b * a.v_sb + hk * a.v_sh;
  auto tile_rsrc = [&](const unsigned char *base, unsigned ss, unsigned ext, int j) {
    const unsigned long long shift = static_cast<unsigned long long>(j) * BC * ss;
    const unsigned recs = (j < n_kt && shift < ext) ? ext - static_cast<unsigned>(shift) : 0u;
    return make_rsrc(base + shift, recs);
  };
  unsigned koff[2], voff[4];
#pragma unroll
  for (int p = 0; p < 2; ++p) koff[p] = (k_r + 32 * p) * a.k_ss + 16u * k_c;
#pragma unroll
  for (int p = 0; p < 4; ++p) voff[p] = (4 * v_g + p) * a.v_ss + 8u * v_c;
  auto load_tile = [&](int j) {
    const __amdgpu_buffer_rsrc_t rkj = tile_rsrc(kbase, a.k_ss, a.k_ext, j);
    const __amdgpu_buffer_rsrc_t rvj = tile_rsrc(vbase, a.v_ss, a.v_ext, j);
#pragma unroll
    for (int p = 0; p < 2; ++p) kreg[p] = buf_load16(rkj, koff[p]);
#pragma unroll
    for (int p = 0; p < 4; ++p) vreg[p] = buf_load8(rvj, voff[p]);
  };
  auto store_tile = [&](int st) {
    unsigned char *ks = lds + st * STAGE;
    unsigned char *vt = ks + K_TILE;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *reinterpret_cast<u32x4 *>(ks + k_lds_row(k_r + 32 * p) * KROW + 16 * k_c) = kreg[p];
    // 4 keys x 8 columns -> 8 columns x 4 keys
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
      const unsigned x01 = __builtin_amdgcn_perm(vreg[1][hd], vreg[0][hd], 0x05010400u);  // k0c0 k1c0 k0c1 k1c1
      const unsigned x23 = __builtin_amdgcn_perm(vreg[3][hd], vreg[2][hd], 0x05010400u);
      const unsigned y01 = __builtin_amdgcn_perm(vreg[1][hd], vreg[0][hd], 0x07030602u);  // k0c2 k1c2 k0c3 k1c3
      const unsigned y23 = __builtin_amdgcn_perm(vreg[3][hd], vreg[2][hd], 0x07030602u);
      unsigned col[4];
      col[0] = __builtin_amdgcn_perm(x23, x01, 0x05040100u);
      col[1] = __builtin_amdgcn_perm(x23, x01, 0x07060302u);
      col[2] = __builtin_amdgcn_perm(y23, y01, 0x05040100u);
      col[3] = __builtin_amdgcn_perm(y23, y01, 0x07060302u);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<unsigned *>(vt + (8 * v_c + 4 * hd + e) * VROW + 4 * v_g) = col[e];
    }
  };

  float m_run = neg_inf();
  float l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  const float cscale = a.c;

  auto compute_tile = [&](int st, int j) {
    const unsigned char *ks = lds + st * STAGE;
    const unsigned char *vt = ks + K_TILE;
    const int j0 = j * BC;
    f32x16 sacc[2];
    u32x4 kr[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        kr[mb][q] = *reinterpret_cast<const u32x4 *>(ks + (32 * mb + l32) * KROW + 64 * h + 16 * q);
    __builtin_amdgcn_s_setprio(1);  // matrix phase first when two waves compete
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sacc[mb] = f32x16{};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 lo = kr[mb][2 * s], hi = kr[mb][2 * s + 1];
        const i32x8 kf{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sacc[mb] = mma(kf, qf[s], sacc[mb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // accumulator (block mb, register i, half h) is key 32h + 16mb + i
    const bool edge = (j0 + BC > a.Sk) || (CAUSAL && j0 + BC - 1 > wrow0 + coff);
    if (edge) {
      const int lim = min(a.Sk - 1 - j0, CAUSAL ? row + coff - j0 : BC);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * h + 16 * mb + i > lim) sacc[mb][i] = neg_inf();
    }
    // lazy running max as in the 16-bit kernel, with the smaller slack kSlack8
    float mxv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) mxv[i] = fmaxf(sacc[0][i], sacc[1][i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) mxv[i] = fmaxf(mxv[i], mxv[i + 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) mxv[i] = fmaxf(mxv[i], mxv[i + 4]);
    float mx = fmaxf(fmaxf(mxv[0], mxv[1]), fmaxf(mxv[2], mxv[3]));
    mx = fmaxf(mx, swap_halves(mx)) * cscale;
    const bool move = mx > m_run + kSlack8;
    if (wave_any(move)) {
      const float m_new = move ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    // p' = kPScale * p: the scale enters the exponent as log2(kPScale)
    const float m_use = ((m_run == neg_inf()) ? 0.f : m_run) - kLog2PScale;
    int pw[8];
    float ps[16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(__builtin_fmaf(sacc[mb][i + e], cscale, -m_use));
#pragma unroll
        for (int e = 0; e < 4; ++e) ps[i + e] = mb == 0 ? p[e] : ps[i + e] + p[e];
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        pw[4 * mb + i / 4] = w;
      }
    l_run += tree_sum16(ps);
    const i32x8 pf{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
    u32x4 vr[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 2; ++q) vr[db][q] = *reinterpret_cast<const u32x4 *>(vt + (32 * db + l32) * VROW + 32 * h + 16 * q);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const u32x4 lo = vr[db][0], hi = vr[db][1];
      const i32x8 vf{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      oacc[db] = mma(vf, pf, oacc[db]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int j = 0; j < n_kt; ++j) {
    const int st = j & 1;
    if (j + 1 < n_kt) load_tile(j + 1);
    if (j < w_kt) compute_tile(st, j);
    if (j + 1 < n_kt) store_tile(st ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + swap_halves(l_run);
  if (row < a.Sq) {
    const float inv = l_tot > 0.f ? a.o_mul / l_tot : 0.f;  // l_tot = kPScale * l: the factor cancels
    __bf16 *orow = static_cast<__bf16 *>(a.o) + b * a.o_sb + hq * a.o_sh + static_cast<long long>(row) * a.o_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * g + 4 * h) = __builtin_bit_cast(u32x2, out);
      }
    if (a.lse != nullptr && h == 0)
      a.lse[b * a.lse_sb + hq * a.lse_sh + row] =
          l_tot > 0.f ? (m_run + __log2f(l_tot) - kLog2PScale) * kLn2 : neg_inf();
  }
}

template <bool CAUSAL> int launch_fp8(const FwdArgs &args, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(args.nq) * args.B * args.Hq;
  hipLaunchKernelGGL(fwd_fp8_kernel<CAUSAL>, dim3(grid), dim3(256), 0, stream, args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "fp8 launch: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace fa

int fa_launch_fwd_fp8(const fa_fwd_params *p, void *stream) {
  using namespace fa;
  if (p->d != 128) return fa_set_error(FA_ERR_UNSUPPORTED, "fp8 forward supports d = 128 only");
  const FwdArgs args = make_fwd_args(p, f8::BR, 1);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p->causal ? launch_fp8<true>(args, s) : launch_fp8<false>(args, s);
}
