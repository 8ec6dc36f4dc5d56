// Prefill forward for fp8 (OCP E4M3FN) Q/K/V with per-tensor or per-block
// descales, bf16 output, on gfx950 8-bit matrix cores.
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
//   * bf16-probability mode (PB16): e4m3 keeps 3 mantissa bits, so each
//     probability fed to P V carries up to 2^-4 relative rounding, and a row
//     whose softmax rests on a few keys moves by up to about 2^-4 max|V|.  In
//     this mode P is rounded to bf16 instead, the V codes are converted
//     exactly to bf16 on their way into LDS (every E4M3FN value is a bf16
//     value), and P V runs on the 32x32x16 bf16 MFMA: 16 products per tile
//     and wavefront instead of 4, with the score side unchanged.  The K tile
//     then uses the 16-bit kernel's row order (bits 2 and 3 of the key index
//     swapped), which puts the score accumulators in the order of the bf16
//     P^T operand.
//   * V: with e4m3 probabilities the tile goes to LDS row-major, one 16-byte
//     load and store per thread like K, and the V^T operand comes from
//     gfx950's byte-transposing LDS read (ds_read_b64_tr_b8: four of them give
//     a lane the 32 keys of one head dimension), so no vector instruction
//     touches V.  With bf16 probabilities V is converted to bf16 and
//     transposed in registers (4 keys x 4 columns per thread, byte permutes)
//     on its way into LDS.
//   * At twice the bf16 matrix rate the softmax is as long as the products, so
//     the loop is software-pipelined like the 16-bit kernel: 8 wavefronts over
//     256 rows; P V of tile t carries the first half of tile t+1's softmax
//     between its MFMAs and S^T of tile t+2 the second half, with the K/V
//     staging riding along and one barrier per tile.
//   * Block descales (one per 64 rows of a (batch, head) slice; the
//     FlashAttention-3 page's block quantisation for fp8) cost no work per
//     element: the query row's descale sits in the lane's score constant; a K
//     tile's descale multiplies that constant once per tile (the tiles are the
//     64-row blocks); a V tile's descale sv enters the exponent as
//     log2(sv / sv_max), so P is rounded to e4m3 already weighted by it, and
//     the tile's row sum is divided by the same ratio once; sv_max, the
//     largest V descale of the slice, multiplies the output in the epilogue.
//     The descales of tile j travel with the staging unit loaded two
//     iterations ahead.
#include "fa_device.hpp"
#include "fa_fwd_common.hpp"
#include "fa_internal.h"

#include <mutex>
#include <type_traits>

namespace fa {

namespace f8 {

constexpr int NT = 512;   // threads per workgroup
constexpr int BR = 256;   // query rows per workgroup (8 wavefronts x 32)
constexpr int BC = 64;    // keys per tile: one 64-deep MFMA for P V
constexpr int D = 128;
constexpr int KROW = D + 16;   // bytes per K row in LDS
constexpr int VROW = BC + 16;  // bytes per V^T row in LDS (bf16-probability mode: see VROW16)
// e4m3 mode: V row-major, 160 bytes per key row, so that the eight rows a
// transposing read covers per 32 lanes start 40 dwords apart and fill the 64
// banks exactly
constexpr int VROWR = D + 32;
constexpr int K_TILE = BC * KROW;
constexpr int V_TILE = D * VROW;
static_assert(BC * VROWR == V_TILE, "row-major and transposed V tiles take the same bytes");
constexpr int ORow = D + 8;    // bf16 elements per row of the epilogue slab
constexpr int STAGES_BYTES = 2 * (K_TILE + V_TILE);
constexpr int SLAB_BYTES = NT / 64 * 32 * ORow * 2;
constexpr int LDS_BYTES = STAGES_BYTES > SLAB_BYTES ? STAGES_BYTES : SLAB_BYTES;
// P is multiplied by kPScale before rounding to e4m3 (max 448).  With the
// lazy running max, P itself can reach 2^kSlack8, so kPScale * 2^kSlack8 = 256
// keeps every scaled probability at or below 256, and probabilities down to
// 2^-10 of the running max stay normal e4m3 numbers.
constexpr float kSlack8 = 4.0f;
constexpr float kLog2PScale = 4.f;  // kPScale = 16

// bf16-probability mode: V^T rows of BC bf16 plus 16 bytes of padding (the
// 16-bit kernel's layout, conflict-free 16-byte reads)
constexpr int VROW16 = BC + 8;
constexpr int V_TILE16 = D * VROW16 * 2;  // bytes
static_assert(2 * (K_TILE + V_TILE16) <= LDS_BYTES, "bf16-P stages must fit the LDS");

// LDS row of key kr of a tile: block mb = (kr >> 4) & 1, half h = kr >> 5,
// register i = kr & 15 of that block's accumulator, whose C row is
// 8 * (i >> 2) + 4 * h + (i & 3).
__device__ __forceinline__ int k_lds_row(int kr) {
  const int h = kr >> 5, mb = (kr >> 4) & 1, i = kr & 15;
  return 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
}

// bf16-probability mode: bits 2 and 3 of the key index swapped, so that the
// S^T accumulator (block mb, register i, lane half h) holds key
// 32 mb + 16 (i >> 3) + 8 h + (i & 7), the order of the bf16 P^T operand
__device__ __forceinline__ int k_lds_row16(int kr) { return (kr & ~12) | ((kr & 4) << 1) | ((kr & 8) >> 1); }

__device__ __forceinline__ f32x16 mma16(u32x4 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mma(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = E4M3 for both operands; block scales 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// ds_read_b64_tr_b8: lane i of each 16-lane group gets, as its byte j, byte
// i % 8 of the 8 bytes addressed by lane 2 j + i / 8 of the group
__device__ __forceinline__ u32x2 lds_read_tr8(const unsigned char *p) {
  typedef int v2i32 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(p)));
}

}  // namespace f8

// Per-block descales: [B][H][nb] float32, one per 64 rows
struct Fp8BlockScales {
  const float *q, *k, *v;
  int nbq, nbk, Hkv;
};

// V operand fragments held between LDS reads and their MFMAs: two 32-byte
// fp8 fragments, or (bf16-probability mode) four 16-byte bf16 fragments
struct VFrag8 { u32x4 f[2][2]; };
struct VFrag16 { u32x4 f[4]; };

template <bool CAUSAL, bool BLK, bool PB16>
__global__ __attribute__((amdgpu_flat_work_group_size(f8::NT, f8::NT), amdgpu_waves_per_eu(2)))
void fwd_fp8_kernel(const FwdArgs a, const Fp8BlockScales bs) {
  using namespace f8;
  // lazy-max slack and log2 of the probability scale: e4m3 P is scaled by 16
  // (<= 256 under a slack of 4); bf16 P needs neither
  constexpr float kSlack = PB16 ? kRescaleSlack : kSlack8;
  constexpr float kLog2PS = PB16 ? 0.f : kLog2PScale;
  constexpr int VT = PB16 ? V_TILE16 : V_TILE;  // bytes per V stage
  using VF = std::conditional_t<PB16, VFrag16, VFrag8>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  unsigned char *kbuf = lds;                 // [2][BC][KROW]
  unsigned char *vbuf = lds + 2 * K_TILE;    // [2][D][VROW]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: the causal tile ranges, loop bounds and buffer resources stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, a.nq, a.B * a.Hq, a.G, CAUSAL, bh, qt);
  const int b = bh / a.Hq, hq = bh - b * a.Hq, hk = hq / a.G;
  const int i0 = qt * BR;
  const int wrow0 = i0 + 32 * wave;
  const int row = wrow0 + l32;

  const int coff = a.Sk - a.Sq;
  int n_kt = (a.Sk + BC - 1) / BC;
  int w_kt = n_kt;
  if (CAUSAL) {
    const int last_wg = i0 + BR - 1 + coff;
    n_kt = min(n_kt, last_wg < 0 ? 0 : last_wg / BC + 1);
    const int last_w = wrow0 + 31 + coff;
    w_kt = min(n_kt, last_w < 0 ? 0 : last_w / BC + 1);
  }

  // ---- staging: K (and V with e4m3 probabilities), thread t loads row t/8,
  // 16-byte chunk t%8; V with bf16 probabilities, thread t loads columns
  // 4*(t/16) .. +3 of keys 4*(t%16) .. +3 (one word per key).
  // Loads go through a buffer resource placed at the tile's first row, so the
  // lane offsets are loop constants and rows past the keys read as zero. ----
  const int k_c = tid & 7, k_r = tid >> 3;
  const int v_g = tid & 15, v_c = tid >> 4;
  const unsigned char *kbase = static_cast<const unsigned char *>(a.k) + b * a.k_sb + hk * a.k_sh;
  const unsigned char *vbase = static_cast<const unsigned char *>(a.v) + b * a.v_sb + hk * a.v_sh;
  // a tile at or past n_kt gets zero records; for a live tile the first row
  // (j * BC <= Sk - 1) starts inside the slice, so the 32-bit shift cannot
  // overflow and the records stay positive
  auto tile_rsrc = [&](const unsigned char *base, unsigned ss, unsigned ext, int j) {
    const bool live = j < n_kt;
    const unsigned shift = live ? static_cast<unsigned>(j * BC) * ss : 0u;
    return make_rsrc(base + shift, live ? ext - shift : 0u);
  };
  const unsigned koff = k_r * a.k_ss + 16u * k_c;
  unsigned voff[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) voff[p] = (4 * v_g + p) * a.v_ss + 4u * v_c;
  u32x4 kreg[2];
  unsigned vreg[2][4];  // bf16-probability mode
  u32x4 vrow8[2];       // e4m3 mode
  auto load_k_to = [&](u32x4 &dst, int j) { dst = buf_load16(tile_rsrc(kbase, a.k_ss, a.k_ext, j), koff); };
  // ---- block descales: the lane's query-row descale in the score constant,
  // the largest V descale of the slice, and per-tile descales loaded ahead
  // (vector buffer loads, so their waits stay in order with the staging) ----
  float cs_base = a.c;
  float sv_max = 1.f;
  float skr[2] = {1.f, 1.f}, svr[2] = {1.f, 1.f};
  // (without block descales these are never used; they point at the K/V codes)
  const float *kbs = BLK ? bs.k + static_cast<long long>(b * bs.Hkv + hk) * bs.nbk : static_cast<const float *>(a.k);
  const float *vbs = BLK ? bs.v + static_cast<long long>(b * bs.Hkv + hk) * bs.nbk : static_cast<const float *>(a.v);
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(kbs, BLK ? 4u * bs.nbk : 0u);
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(vbs, BLK ? 4u * bs.nbk : 0u);
  if constexpr (BLK) {
    const float *qbs = bs.q + static_cast<long long>(b * a.Hq + hq) * bs.nbq;
    cs_base = a.c * fmaxf(qbs[min(row, a.Sq - 1) / BC], 1e-30f);
    float vm = 0.f;
    for (int j = lane; j < bs.nbk; j += 64) vm = fmaxf(vm, vbs[j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) vm = fmaxf(vm, __shfl_xor(vm, off, 64));
    sv_max = vm > 0.f ? vm : 1.f;
  }
  auto load_scales = [&](int set, int j) {
    if constexpr (BLK) {
      skr[set] = __builtin_bit_cast(float, buf_load4(rks, 4u * static_cast<unsigned>(j)));
      svr[set] = __builtin_bit_cast(float, buf_load4(rvs, 4u * static_cast<unsigned>(j)));
    }
  };
  // score constant, log2 of the V-descale ratio and its inverse, of the tile
  // whose softmax runs next
  float cscale = a.c;
  float lr_t = 0.f, inv_t = 1.f;
  auto tile_consts = [&](float sk, float sv) {
    if constexpr (BLK) {
      cscale = cs_base * fmaxf(sk, 1e-30f);
      const float ratio = fmaxf(sv / sv_max, 0x1p-20f);
      lr_t = __log2f(ratio);
      inv_t = 1.f / ratio;
    }
  };

  auto load_v = [&](int set, int j) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(vbase, a.v_ss, a.v_ext, j);
    if constexpr (PB16) {
#pragma unroll
      for (int p = 0; p < 4; ++p) vreg[set][p] = buf_load4(r, voff[p]);
    } else {
      vrow8[set] = buf_load16(r, k_r * a.v_ss + 16u * k_c);
    }
  };
  auto store_k_from = [&](const u32x4 &src, int buf) {
    const int r = PB16 ? k_lds_row16(k_r) : k_lds_row(k_r);
    *reinterpret_cast<u32x4 *>(kbuf + buf * K_TILE + r * KROW + 16 * k_c) = src;
  };
  // e4m3 mode: the row as loaded; bf16 mode: 4 keys x 4 columns -> 4 columns x 4 keys
  auto store_v = [&](int set, int buf) {
    if constexpr (!PB16) {
      *reinterpret_cast<u32x4 *>(vbuf + buf * VT + k_r * VROWR + 16 * k_c) = vrow8[set];
      return;
    }
    const unsigned *r = vreg[set];
    const unsigned x01 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // k0c0 k1c0 k0c1 k1c1
    const unsigned x23 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
    const unsigned y01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // k0c2 k1c2 k0c3 k1c3
    const unsigned y23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
    {
      // each word of key pairs -> two bf16 (exact); column 4 v_c + e gets keys
      // 4 v_g .. 4 v_g + 3 as one 8-byte store
      auto lo = [](unsigned w) {
        return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
      };
      auto hi = [](unsigned w) {
        return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
      };
      unsigned char *vt = vbuf + buf * VT;
      const u32x2 col[4] = {u32x2{lo(x01), lo(x23)}, u32x2{hi(x01), hi(x23)}, u32x2{lo(y01), lo(y23)},
                            u32x2{hi(y01), hi(y23)}};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<u32x2 *>(vt + ((4 * v_c + e) * VROW16 + 4 * v_g) * 2) = col[e];
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  i32x8 qf[2];  // lane half h holds bytes [64h, 64h + 64) of its row; step s uses 32 of them

  // ---- blocks: 4 MFMAs each, operands read two MFMAs (four 16-byte reads)
  // ahead, softmax steps of the neighbouring tile dealt out over the slots ----
  constexpr int NM = 4;
  constexpr int RA = 2;
  constexpr int STEPS = 16;
  const unsigned char *k_lane = kbuf + l32 * KROW + 64 * h;
  // e4m3 mode, transposing V reads: lane s of 16-lane group g addresses key row
  // 32 (g >> 1) + 8 rd + (s >> 1), columns 32 i + 16 (g & 1) + 8 (s & 1) .. + 7,
  // so that read rd gives lane (m, h) keys 32 h + 8 rd .. + 7 of column 32 i + m
  const unsigned char *v_lane =
      vbuf + (32 * h + ((lane & 15) >> 1)) * VROWR + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  // MFMA i of S^T: key block i & 1, depth step i >> 1
  auto kfrag = [&](int buf, int i, int half) {
    return *reinterpret_cast<const u32x4 *>(k_lane + buf * K_TILE + (i & 1) * 32 * KROW + 32 * (i >> 1) + 16 * half);
  };
  // MFMA i of O^T: head-dim block i; bytes 16 half .. 16 half + 15 of the lane's 32
  auto vfrag = [&](int buf, int i, int half) {
    const unsigned char *p = v_lane + buf * VT + 32 * i + 2 * half * 8 * VROWR;
    const u32x2 lo = lds_read_tr8(p), hi = lds_read_tr8(p + 8 * VROWR);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // bf16-probability mode, MFMA i of O^T: head-dim block i >> 2, key step i & 3
  const unsigned char *v_lane16 = vbuf + (l32 * VROW16 + 8 * h) * 2;
  auto vfrag16 = [&](int buf, int i) {
    return *reinterpret_cast<const u32x4 *>(v_lane16 + buf * VT + ((i >> 2) * 32 * VROW16 + 16 * (i & 3)) * 2);
  };

  // ---- online softmax state ----
  float m_run = neg_inf();
  float l_run = 0.f;
  float alpha_p = 1.f;
  bool move_p = false;
  float m_use = 0.f;  // running max minus log2 kPScale (minus the tile's V-descale log ratio)

  // accumulator (block mb, register i, half h) is key 32h + 16mb + i, or in
  // bf16-probability mode 32mb + 16(i >> 3) + 8h + (i & 7)
  auto mask = [&](f32x16 s[2], int j) {
    const int j0 = j * BC;
    const bool edge = (j0 + BC > a.Sk) || (CAUSAL && j0 + BC - 1 > wrow0 + coff);
    if (edge) {
      // the lane's row and half taken afresh (see fresh_lane_id)
      const int fl = fresh_lane_id(), fh = fl >> 5;
      const int lim = min(a.Sk - 1 - j0, CAUSAL ? wrow0 + (fl & 31) + coff - j0 : BC);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = PB16 ? 32 * mb + 16 * (i >> 3) + 8 * fh + (i & 7) : 32 * fh + 16 * mb + i;
          if (key > lim) s[mb][i] = neg_inf();
        }
    }
  };
  // first half: tile max, lazy running-max update, exponents of s[0]
  float ta[11], ua[4], mxa;
  auto soft_a_step = [&](auto step_tag, f32x16 s[2]) {
    constexpr int st = decltype(step_tag)::value;
    auto sv = [&](int x) { return s[x >> 4][x & 15]; };
    if constexpr (st < 3) {
#pragma unroll
      for (int i = 4 * st; i < (st == 2 ? 10 : 4 * st + 4); ++i) {
        ta[i] = max3f(sv(3 * i), sv(3 * i + 1), sv(3 * i + 2));
        pin(ta[i]);
      }
      if constexpr (st == 2) {
        ta[10] = fmaxf(sv(30), sv(31));
        pin(ta[10]);
      }
    } else if constexpr (st == 3) {
      ua[0] = max3f(ta[0], ta[1], ta[2]);
      ua[1] = max3f(ta[3], ta[4], ta[5]);
      ua[2] = max3f(ta[6], ta[7], ta[8]);
      ua[3] = fmaxf(ta[9], ta[10]);
#pragma unroll
      for (int i = 0; i < 4; ++i) pin(ua[i]);
    } else if constexpr (st == 4) {
      mxa = max3f(ua[0], ua[1], fmaxf(ua[2], ua[3]));
      mxa = fmaxf(mxa, swap_halves(mxa));
      pin(mxa);
    } else if constexpr (st == 5) {
      mxa *= cscale;
      move_p = mxa > m_run + kSlack;
    } else if constexpr (st == 6) {
      const float m_new = move_p ? mxa : m_run;
      alpha_p = move_p ? fast_exp2(m_run - m_new) : 1.f;  // 0 when m_run = -inf
      m_run = m_new;
      // p' = kPScale * p: the scale enters the exponent as log2(kPScale)
      m_use = ((m_run == neg_inf()) ? 0.f : m_run) - kLog2PS - lr_t;
      pin(alpha_p);
      pin(m_use);
    } else if constexpr (st < 15) {
      constexpr int e = 2 * (st - 7);
      float p0 = fast_exp2(__builtin_fmaf(s[0][e], cscale, -m_use));
      float p1 = fast_exp2(__builtin_fmaf(s[0][e + 1], cscale, -m_use));
      pin(p0);
      pin(p1);
      s[0][e] = p0;
      s[0][e + 1] = p1;
    }
  };
  // second half: exponents of s[1]; P^T packed to e4m3, four keys per word;
  // row sum of the unrounded probabilities as a balanced tree; l update
  float ps[16], qa[8];
  // P^T packed: 8 words of e4m3, or 16 of bf16 pairs.  An e4m3 word is
  // written a half at a time; its first half goes over the word's previous
  // tile (dead once that tile's P V has issued), so no zeroing is needed.
  int pw[16] = {};
  auto pack_bf16 = [](float x0, float x1) {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(int, v2{static_cast<__bf16>(x0), static_cast<__bf16>(x1)});
  };
  auto soft_b_step = [&](auto step_tag, f32x16 s[2]) {
    constexpr int st = decltype(step_tag)::value;
    if constexpr (st < 8) {
      float p0 = fast_exp2(__builtin_fmaf(s[1][2 * st], cscale, -m_use));
      float p1 = fast_exp2(__builtin_fmaf(s[1][2 * st + 1], cscale, -m_use));
      pin(p0);
      pin(p1);
      s[1][2 * st] = p0;
      s[1][2 * st + 1] = p1;
      if constexpr (PB16) {
        pw[st] = pack_bf16(s[0][2 * st], s[0][2 * st + 1]);
        pin(pw[st]);
      } else if constexpr (st < 4) {
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(s[0][4 * st], s[0][4 * st + 1], pw[st], false);
        pw[st] = __builtin_amdgcn_cvt_pk_fp8_f32(s[0][4 * st + 2], s[0][4 * st + 3], w, true);
        pin(pw[st]);
      }
    } else {
      if constexpr (PB16) {
        pw[st] = pack_bf16(s[1][2 * (st - 8)], s[1][2 * (st - 8) + 1]);
        pin(pw[st]);
      }
      if constexpr (st < 12) {
        constexpr int q = st - 8;
        if constexpr (!PB16) {
          const int w = __builtin_amdgcn_cvt_pk_fp8_f32(s[1][4 * q], s[1][4 * q + 1], pw[4 + q], false);
          pw[4 + q] = __builtin_amdgcn_cvt_pk_fp8_f32(s[1][4 * q + 2], s[1][4 * q + 3], w, true);
          pin(pw[4 + q]);
        }
#pragma unroll
        for (int i = 4 * q; i < 4 * q + 4; ++i) {
          ps[i] = s[0][i] + s[1][i];
          pin(ps[i]);
        }
      } else if constexpr (st < 14) {
        constexpr int base = 4 * (st - 12);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qa[base + i] = ps[base + i] + ps[base + i + 8];
          pin(qa[base + i]);
        }
      } else if constexpr (st == 14) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qa[i] += qa[i + 4];
          pin(qa[i]);
        }
      } else {
        l_run = __builtin_fmaf(l_run, alpha_p, ((qa[0] + qa[2]) + (qa[1] + qa[3])) * inv_t);
        pin(l_run);
      }
    }
  };
  auto p_pack = [&](f32x16 s[2]) {
    if constexpr (PB16)
      s[0] = __builtin_bit_cast(f32x16, i32x16{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7], pw[8],
                                               pw[9], pw[10], pw[11], pw[12], pw[13], pw[14], pw[15]});
    else
      s[0] = __builtin_bit_cast(f32x16, i32x16{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7],
                                               0, 0, 0, 0, 0, 0, 0, 0});
  };
  auto rescale_o = [&]() {
    if (wave_any(move_p)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha_p;
    }
  };

  // first RA operand fragments of a block, read ahead by the caller
  auto k_init = [&](int buf, u32x4 (&kf)[RA][2]) {
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      kf[i][0] = kfrag(buf, i, 0);
      kf[i][1] = kfrag(buf, i, 1);
    }
  };
  auto v_init = [&](int buf, VF &vf) {
    if constexpr (PB16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vf.f[i] = vfrag16(buf, i);
    } else {
#pragma unroll
      for (int i = 0; i < RA; ++i) {
        vf.f[i][0] = vfrag(buf, i, 0);
        vf.f[i][1] = vfrag(buf, i, 1);
      }
    }
  };
  // S^T of K buffer `buf` into s, starting from the fragments kf; softmax
  // work on `sn` rides along: none (SOFT = 0), its second half (1) or both
  // halves (2)
  auto block_qk = [&](int buf, f32x16 s[2], f32x16 sn[2], auto soft_tag, auto &&extra, u32x4 (&kf)[RA][2]) {
    constexpr int SOFT = decltype(soft_tag)::value;
    s[0] = f32x16{};
    s[1] = f32x16{};
    static_for<NM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      s[i & 1] = mma(join(kf[i % RA][0], kf[i % RA][1]), qf[i >> 1], s[i & 1]);
      if constexpr (i + RA < NM) {
        kf[i % RA][0] = kfrag(buf, i + RA, 0);
        kf[i % RA][1] = kfrag(buf, i + RA, 1);
      }
      if constexpr (SOFT == 1)
        static_for<STEPS / NM>([&](auto K) {
          soft_b_step(std::integral_constant<int, i * (STEPS / NM) + decltype(K)::value>{}, sn);
        });
      if constexpr (SOFT == 2)
        static_for<2 * STEPS / NM>([&](auto K) {
          constexpr int st = i * (2 * STEPS / NM) + decltype(K)::value;
          if constexpr (st < STEPS) soft_a_step(std::integral_constant<int, st>{}, sn);
          else soft_b_step(std::integral_constant<int, st - STEPS>{}, sn);
        });
      extra(I);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (SOFT != 0) p_pack(sn);
    // the scores are first read in the next iteration: keep their MFMAs here,
    // between this block's softmax steps, rather than after the barrier
    pin(s[0]);
    pin(s[1]);
  };
  // O^T += V^T P^T of V buffer `buf`, P^T in the first 8 words of p,
  // starting from the fragments vf; the first softmax half of `sn` rides
  // along, and the slots past the last V read fetch the first fragments kn
  // of the next S^T block (K buffer kbn)
  auto block_pv = [&](int buf, const f32x16 &p, f32x16 sn[2], auto &&extra, VF &vf, int kbn,
                      u32x4 (&kn)[RA][2]) {
    if constexpr (PB16) {
      // 16 bf16 MFMAs: head-dim block i >> 2, key step i & 3; V^T read four
      // MFMAs ahead, the next S^T block's first K fragments in the last two slots
      constexpr int NPV = 16;
      const bf16x8 pf[4] = {__builtin_bit_cast(bf16x8, __builtin_shufflevector(p, p, 0, 1, 2, 3)),
                            __builtin_bit_cast(bf16x8, __builtin_shufflevector(p, p, 4, 5, 6, 7)),
                            __builtin_bit_cast(bf16x8, __builtin_shufflevector(p, p, 8, 9, 10, 11)),
                            __builtin_bit_cast(bf16x8, __builtin_shufflevector(p, p, 12, 13, 14, 15))};
      static_for<NPV>([&](auto I) {
        constexpr int i = decltype(I)::value;
        oacc[i >> 2] = mma16(vf.f[i % 4], pf[i & 3], oacc[i >> 2]);
        if constexpr (i + 4 < NPV) vf.f[i % 4] = vfrag16(buf, i + 4);
        if constexpr (i >= NPV - RA) {
          kn[i + RA - NPV][0] = kfrag(kbn, i + RA - NPV, 0);
          kn[i + RA - NPV][1] = kfrag(kbn, i + RA - NPV, 1);
        }
        soft_a_step(std::integral_constant<int, i * (STEPS / NPV)>{}, sn);
        extra(std::integral_constant<int, i / 4>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      const i32x16 pi = __builtin_bit_cast(i32x16, p);
      const i32x8 pf = __builtin_shufflevector(pi, pi, 0, 1, 2, 3, 4, 5, 6, 7);
      static_for<NM>([&](auto I) {
        constexpr int i = decltype(I)::value;
        oacc[i] = mma(join(vf.f[i % RA][0], vf.f[i % RA][1]), pf, oacc[i]);
        if constexpr (i + RA < NM) {
          vf.f[i % RA][0] = vfrag(buf, i + RA, 0);
          vf.f[i % RA][1] = vfrag(buf, i + RA, 1);
        } else {
          kn[i + RA - NM][0] = kfrag(kbn, i + RA - NM, 0);
          kn[i + RA - NM][1] = kfrag(kbn, i + RA - NM, 1);
        }
        static_for<STEPS / NM>([&](auto K) {
          soft_a_step(std::integral_constant<int, i * (STEPS / NM) + decltype(K)::value>{}, sn);
        });
        extra(I);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };

  // Two score register sets: sc[j & 1] holds S^T of tile j from its QK^T
  // until its softmax is done, then P^T (in its first 8 words) until its P V.
  f32x16 sc[2][2];

  // ---- prologue: K of tiles 0-2 and V of tile 0 staged, tile 0 through its
  // softmax, S^T of tile 1 formed, staging units 0 and 1 in flight; the first
  // tiles and the Q rows are fetched together ----
  // unit u = (K of tile u+3, V of tile u+1), written to LDS in iteration u
  // (with block descales, the unit also brings those of tile u + 1)
  auto load_unit = [&](int set, int u) {
    load_scales(set, u + 1);
    load_k_to(kreg[set], u + 3);
    load_v(set, u + 1);
  };
  u32x4 k0, k1, k2;
  load_k_to(k0, 0);
  load_k_to(k1, 1);
  load_v(0, 0);
  load_k_to(k2, 2);
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(static_cast<const unsigned char *>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_ext);
    const bool ok = row < a.Sq;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const unsigned base = ok ? row * a.q_ss + 64u * h + 32u * s : kOOB;
      qf[s] = join(buf_load16(rq, base), buf_load16(rq, ok ? base + 16u : kOOB));
    }
  }
  if constexpr (BLK) {  // tile 0's descales, before set 0 is reused for tile 1
    load_scales(0, 0);
    tile_consts(skr[0], svr[0]);
  }
  store_k_from(k0, 0);
  store_k_from(k1, 1);
  store_v(0, 0);
  load_unit(0, 0);
  __syncthreads();
  if (0 < w_kt) {
    u32x4 kf[RA][2];
    k_init(0, kf);
    block_qk(0, sc[0], sc[1], std::integral_constant<int, 0>{}, [](auto) {}, kf);
    mask(sc[0], 0);
    k_init(1, kf);
    block_qk(1, sc[1], sc[0], std::integral_constant<int, 2>{}, [](auto) {}, kf);
  }
  __syncthreads();
  store_k_from(k2, 0);
  load_unit(1, 1);
  __syncthreads();

  // Main loop, as in the 16-bit kernel: iteration t runs P V of tile t with
  // the first softmax half of tile t+1, then S^T of tile t+2 with the second
  // half; the wave's share of unit t (K of tile t+3 into the K buffer of tile
  // t+1, V of tile t+1 into the V buffer of tile t-1, neither read in this
  // iteration) rides along, and one barrier per iteration publishes it.
  auto iter = [&](auto set_tag, int t) {
    constexpr int cur = decltype(set_tag)::value;  // t & 1
    constexpr int nxt = cur ^ 1;
    // V of tile t and K of tile t+2 both sit in buffer cur
    VF vf;
    u32x4 kf[RA][2];
    v_init(cur, vf);  // first, so the reads overlap the rescale and mask
    tile_consts(skr[cur], svr[cur]);  // of tile t+1, loaded with unit t-1 (or in the prologue)
    rescale_o();
    mask(sc[nxt], t + 1);
    block_pv(cur, sc[cur][0], sc[nxt], [&](auto I) {
      if constexpr (decltype(I)::value == 1) store_k_from(kreg[cur], nxt);
      if constexpr (decltype(I)::value == 2) store_v(cur, nxt);
    }, vf, cur, kf);
    block_qk(cur, sc[cur], sc[nxt], std::integral_constant<int, 1>{}, [&](auto I) {
      if constexpr (decltype(I)::value == 1) load_unit(cur, t + 2);
    }, kf);
    __syncthreads();
  };
  // iterations past the wave's last tile (causal): staging only
  auto iter_stage = [&](auto set_tag, int t) {
    constexpr int cur = decltype(set_tag)::value;
    constexpr int nxt = cur ^ 1;
    store_k_from(kreg[cur], nxt);
    store_v(cur, nxt);
    load_unit(cur, t + 2);
    __syncthreads();
  };
  int t = 0;
  for (; t + 1 < w_kt; t += 2) {
    iter(std::integral_constant<int, 0>{}, t);
    iter(std::integral_constant<int, 1>{}, t + 1);
  }
  if (t < w_kt) {
    iter(std::integral_constant<int, 0>{}, t);
    ++t;
    if (t < n_kt) {
      iter_stage(std::integral_constant<int, 1>{}, t);
      ++t;
    }
  }
  for (; t + 1 < n_kt; t += 2) {
    iter_stage(std::integral_constant<int, 0>{}, t);
    iter_stage(std::integral_constant<int, 1>{}, t + 1);
  }
  if (t < n_kt) iter_stage(std::integral_constant<int, 0>{}, t);

  // ---- epilogue: O = o_mul * O_acc / l (l carries kPScale, which cancels),
  // transposed through LDS (free after the loop's last barrier) so that each
  // store writes whole rows.  The lane's indices are taken afresh (see
  // fresh_lane_id). ----
  const int elane = fresh_lane_id();
  const int el32 = elane & 31, eh = elane >> 5, erow = wrow0 + el32;
  auto other_half = [&](float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, eh == 0 ? r[1] : r[0]);
  };
  const float l_tot = l_run + other_half(l_run);
  {
    const float inv = l_tot > 0.f ? (BLK ? sv_max : a.o_mul) / l_tot : 0.f;
    __bf16 *slab = reinterpret_cast<__bf16 *>(lds) + wave * 32 * ORow;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<u32x2 *>(slab + el32 * ORow + 32 * db + 8 * g + 4 * eh) = __builtin_bit_cast(u32x2, out);
      }
    // the slab is private to the wavefront, whose LDS operations complete in order
    __bf16 *obase = static_cast<__bf16 *>(a.o) + b * a.o_sb + hq * a.o_sh;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + elane / 16, c = elane % 16;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(slab + r * ORow + 8 * c);
      const int orow_i = wrow0 + r;
      if (orow_i < a.Sq) *reinterpret_cast<u32x4 *>(obase + static_cast<long long>(orow_i) * a.o_ss + 8 * c) = v;
    }
  }
  if (erow < a.Sq && a.lse != nullptr && eh == 0)
    a.lse[b * a.lse_sb + hq * a.lse_sh + erow] = l_tot > 0.f ? (m_run + __log2f(l_tot) - kLog2PS) * kLn2 : neg_inf();
}

template <bool CAUSAL, bool BLK, bool PB16>
int launch_fp8(const FwdArgs &args, const Fp8BlockScales &bs, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(args.nq) * args.B * args.Hq;
  fa_log_launch("fwd_fp8_kernel", grid, f8::NT, f8::LDS_BYTES,
                "p=%s causal=%d block_descales=%d B=%d Hq=%d G=%d Sq=%d Sk=%d rows_per_wg=%d",
                PB16 ? "bf16" : "e4m3", CAUSAL ? 1 : 0, BLK ? 1 : 0, args.B, args.Hq, args.G, args.Sq, args.Sk,
                f8::BR);
  hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL, BLK, PB16>), dim3(grid), dim3(f8::NT), 0, stream, args, bs);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "fp8 launch: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace fa

int fa_launch_fwd_fp8(const fa_fwd_params *p, void *stream) {
  using namespace fa;
  if (p->d != 128) return fa_set_error(FA_ERR_UNSUPPORTED, "fp8 forward supports d = 128 only");
  FwdArgs args = make_fwd_args(p, f8::BR, 1);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->q_block_descale != nullptr) {
    // block descales replace the per-tensor ones
    args.c = p->softmax_scale * 1.4426950408889634f;
    args.o_mul = 1.f;
    const Fp8BlockScales bs{p->q_block_descale, p->k_block_descale, p->v_block_descale,
                            (p->Sq + f8::BC - 1) / f8::BC, (p->Sk + f8::BC - 1) / f8::BC, p->Hkv};
    if (p->fp8_p_bf16)
      return p->causal ? launch_fp8<true, true, true>(args, bs, s) : launch_fp8<false, true, true>(args, bs, s);
    return p->causal ? launch_fp8<true, true, false>(args, bs, s) : launch_fp8<false, true, false>(args, bs, s);
  }
  const Fp8BlockScales none{};
  if (p->fp8_p_bf16)
    return p->causal ? launch_fp8<true, false, true>(args, none, s) : launch_fp8<false, false, true>(args, none, s);
  return p->causal ? launch_fp8<true, false, false>(args, none, s) : launch_fp8<false, false, false>(args, none, s);
}
