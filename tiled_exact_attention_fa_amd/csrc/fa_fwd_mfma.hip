// Prefill forward for fp32 / bf16 / fp16 inputs on gfx950 matrix cores.
//
// Method (FlashAttention interview canvas, panel 1 "one-sentence answer" and
// "online softmax key state" boxes; panel 2, v1 card): K/V tiles are staged in
// on-chip memory, and for every tile the scores, the online-softmax update and
// the P V accumulation are done in registers, so the score matrix never reaches
// HBM.  One workgroup owns 128 query rows of one (batch, head) — the v2 card's
// partitioning of a single head across workgroups — and each of its four
// wavefronts owns 32 rows end to end, so no reduction crosses wavefronts.
//
// MI355X design.
//   * Scores are formed transposed, S^T = K Q^T, with 32x32 MFMA (K-depth 16 for
//     bf16/fp16, 2 for fp32).  Lane l then holds scores of query l%32 only: the
//     row max is an in-register max plus one exchange between the two 32-lane
//     halves, and the row sum needs no exchange until the epilogue.
//   * The K tile is written to LDS with bits 2 and 3 of the key index swapped
//     (16-bit types), which makes the score accumulators land exactly in the
//     register order of the P^T operand of O^T = V^T P^T: P is rounded in place
//     and fed back to the matrix core without any data movement.
//   * V is transposed in registers on its way to LDS, so every V^T operand is a
//     single 16-byte LDS read; both tiles are padded by 16 bytes per row, which
//     keeps 8-lane phases of 16-byte reads free of bank conflicts.
//   * K/V tiles are double-buffered in LDS: tile j+1 is fetched from HBM into
//     registers while tile j is computed, with one barrier per tile.
//   * Scores are kept in the log2 domain (scale * log2 e folded into one FMA) and
//     exponentiated with the hardware exp2.
//   * Causal tiles past a wavefront's last row are skipped; the mask is applied
//     only on tiles that cross the diagonal or the end of the keys.  Workgroups
//     are issued heaviest first and grouped so each XCD works on a contiguous
//     range of (batch, head) pairs, whose K/V then stay in that XCD's L2.
#include "fa_device.hpp"
#include "fa_fwd_common.hpp"
#include "fa_internal.h"

#include <mutex>
#include <type_traits>

namespace fa {

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  static constexpr int KW = 8;  // reduction elements per lane per instruction
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<_Float16> {
  static constexpr int KW = 8;
  typedef f16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KW = 1;
  typedef float frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename T, int D> struct Cfg {
  static constexpr int ES = sizeof(T);
  static constexpr int KW = Mfma<T>::KW;
  static constexpr int BR = 128;                // query rows per workgroup
  static constexpr int BC = ES == 4 ? 32 : 64;  // keys per tile
  static constexpr int EPC = 16 / ES;           // elements per 16-byte chunk
  static constexpr int CH = D / EPC;            // chunks per row
  static constexpr int PASSES = BC * CH / 256;  // 16-byte loads per thread per tile
  static constexpr int KPT = PASSES;            // keys per thread in the V transpose
  static constexpr int NG = BC / KPT;           // V key groups
  static constexpr int KROW = D + EPC;          // K row in LDS, +16 bytes
  static constexpr int VROW = BC + EPC;         // V^T row in LDS, +16 bytes
  static constexpr int K_TILE = BC * KROW;
  static constexpr int V_TILE = D * VROW;
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int QSTEPS = D / (2 * KW);   // MFMA steps over the head dim
  static constexpr int MB = BC / 32;            // 32-key blocks of S^T
  static constexpr int DB = D / 32;             // 32-column blocks of O^T
  static constexpr int LDS_BYTES = 2 * STAGE * ES;
  static_assert(BC * CH % 256 == 0, "tile must split evenly over 256 threads");
};


// Configuration of the 16-bit kernel: 8 wavefronts (two per SIMD) own 256 query
// rows, so each K/V tile is fetched and staged once for twice as many rows.
template <typename T, int D> struct Cfg16 {
  static constexpr int ES = sizeof(T);
  static constexpr int KW = 8;
  static constexpr int NT = 512;                // threads per workgroup
  static constexpr int BR = 256;                // query rows per workgroup
  static constexpr int BC = 64;                 // keys per tile
  static constexpr int EPC = 8;                 // elements per 16-byte chunk
  static constexpr int CH = D / EPC;            // chunks per row
  static constexpr int PASSES = BC * CH / NT;   // 16-byte loads per thread per tile (K or V)
  static constexpr int KPT = PASSES;            // keys per thread in the V transpose
  static constexpr int NG = BC / KPT;           // V key groups
  static constexpr int KROW = D + EPC;          // K row in LDS, +16 bytes
  static constexpr int VROW = BC + EPC;         // V^T row in LDS, +16 bytes
  static constexpr int K_TILE = BC * KROW;
  static constexpr int V_TILE = D * VROW;
  static constexpr int DB = D / 32;
  static constexpr int LDS_BYTES = 2 * (K_TILE + V_TILE) * ES;
  static_assert(BC * CH % NT == 0, "tile must split evenly over the workgroup");
};

// LDS row of key kr within a tile.  For 16-bit types bits 2 and 3 are swapped,
// so that the S^T accumulator of (register i, half h) holds key
// 32*(i/16) + 16*((i/8)%2) + 8*h + i%8 — the order the P^T operand needs.
template <int KW> __device__ __forceinline__ int k_lds_row(int kr) {
  if constexpr (KW == 8) return (kr & ~12) | ((kr & 4) << 1) | ((kr & 8) >> 1);
  else return kr;
}

// Key (within the tile) of S^T block mb, accumulator register i, lane half h.
template <int KW> __device__ __forceinline__ int acc_key(int mb, int i, int h) {
  if constexpr (KW == 8) return 32 * mb + 16 * (i >> 3) + 8 * h + (i & 7);
  else return 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
}

template <typename T> __device__ __forceinline__ T to_out(float x) { return static_cast<T>(x); }

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void fwd_mfma_kernel(const FwdArgs a) {
  using C = Cfg<T, D>;
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int KW = C::KW, BC = C::BC, EPC = C::EPC, CH = C::CH, ES = C::ES;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *lds = reinterpret_cast<T *>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, a.nq, a.B * a.Hq, CAUSAL, bh, qt);
  const int b = bh / a.Hq, hq = bh - b * a.Hq, hk = hq / a.G;
  const int i0 = qt * C::BR;
  const int wrow0 = i0 + 32 * wave;
  const int row = wrow0 + l32;  // query row of this lane

  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(static_cast<const T *>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_ext);
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(static_cast<const T *>(a.k) + b * a.k_sb + hk * a.k_sh, a.k_ext);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(static_cast<const T *>(a.v) + b * a.v_sb + hk * a.v_sh, a.v_ext);

  // ---- Q rows into registers: lane half h holds d in [D/2*h, D/2*h + D/2) ----
  frag qf[C::QSTEPS];
  {
    const bool ok = row < a.Sq;
#pragma unroll
    for (int c = 0; c < D / 2 / EPC; ++c) {
      const unsigned off = ok ? row * a.q_ss + ((D / 2) * h + c * EPC) * ES : kOOB;
      const u32x4 v = buf_load16(rq, off);
      if constexpr (KW == 8) {
        qf[c] = __builtin_bit_cast(frag, v);
      } else {
        // bit-cast the whole vector, then index (a bit-cast of a single
        // vector element is not reliable with this compiler)
        const f32x4 vf = __builtin_bit_cast(f32x4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * c + e] = vf[e];
      }
    }
    wait_vmem_all();
  }

  // ---- tile range of this workgroup and of this wavefront ----
  const int coff = a.Sk - a.Sq;  // causal: key j visible from row i iff j <= i + coff
  int n_kt = (a.Sk + BC - 1) / BC;
  int w_kt = n_kt;
  if (CAUSAL) {
    const int last_wg = i0 + C::BR - 1 + coff;
    n_kt = min(n_kt, last_wg < 0 ? 0 : last_wg / BC + 1);
    const int last_w = wrow0 + 31 + coff;
    w_kt = min(n_kt, last_w < 0 ? 0 : last_w / BC + 1);
  }

  // ---- global -> register staging of one K/V tile ----
  u32x4 kreg[C::PASSES], vreg[C::PASSES];
  const int k_c = tid % CH, k_r = tid / CH;          // K: chunk, first row
  const int v_g = tid % C::NG, v_c = tid / C::NG;    // V: key group, chunk
  auto load_tile = [&](int j) {
    const int j0 = j * BC;
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int kk = j0 + k_r + (256 / CH) * p;
      kreg[p] = buf_load16(rk, kk < a.Sk ? kk * a.k_ss + k_c * 16 : kOOB);
      const int vk = j0 + v_g * C::KPT + p;
      vreg[p] = buf_load16(rv, vk < a.Sk ? vk * a.v_ss + v_c * 16 : kOOB);
    }
  };
  auto store_tile = [&](int st) {
    T *ks = lds + st * C::STAGE;
    T *vt = ks + C::K_TILE;
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int kr = k_r + (256 / CH) * p;
      *reinterpret_cast<u32x4 *>(ks + k_lds_row<KW>(kr) * C::KROW + k_c * EPC) = kreg[p];
    }
    // transpose: this thread holds keys v_g*KPT .. +KPT-1 of d-chunk v_c
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      T col[C::KPT];
#pragma unroll
      for (int p = 0; p < C::KPT; ++p) {
        const T *src = reinterpret_cast<const T *>(&vreg[p]);
        col[p] = src[e];
      }
      T *dst = vt + (v_c * EPC + e) * C::VROW + v_g * C::KPT;
      if constexpr (C::KPT * ES == 16) {
        *reinterpret_cast<u32x4 *>(dst) = __builtin_bit_cast(u32x4, col);
      } else if constexpr (C::KPT * ES == 8) {
        *reinterpret_cast<u32x2 *>(dst) = __builtin_bit_cast(u32x2, col);
      } else {
        static_assert(C::KPT * ES == 4, "unexpected V transpose width");
        *reinterpret_cast<unsigned *>(dst) = __builtin_bit_cast(unsigned, col);
      }
    }
  };

  // ---- online-softmax state: running max (log2 units), lane-partial sum, O^T ----
  float m_run = neg_inf();
  float l_run = 0.f;
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  const float cscale = a.c;

  auto compute_tile = [&](int st, int j) {
    const T *ks = lds + st * C::STAGE;
    const T *vt = ks + C::K_TILE;
    const int j0 = j * BC;

    // S^T = K Q^T for this tile
    f32x16 sacc[C::MB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      sacc[mb] = f32x16{};
      const T *krow = ks + (32 * mb + l32) * C::KROW + (D / 2) * h;
#pragma unroll
      for (int c = 0; c < D / 2 / EPC; ++c) {
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(krow + c * EPC);
        if constexpr (KW == 8) {
          sacc[mb] = M::mma(__builtin_bit_cast(frag, kv), qf[c], sacc[mb]);
        } else {
          const f32x4 kf = __builtin_bit_cast(f32x4, kv);
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[mb] = M::mma(kf[e], qf[4 * c + e], sacc[mb]);
        }
      }
    }

    // mask (only tiles that cross the diagonal or the end of the keys)
    const bool edge = (j0 + BC > a.Sk) || (CAUSAL && j0 + BC - 1 > wrow0 + coff);
    if (edge) {
      const int lim = min(a.Sk - 1 - j0, CAUSAL ? row + coff - j0 : BC);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (acc_key<KW>(mb, i, h) > lim) sacc[mb][i] = neg_inf();
    }

    // online softmax.  The running max m moves only when this tile's max
    // exceeds it by more than kRescaleSlack (log2 units); otherwise the stale
    // m is kept and P may reach 2^kRescaleSlack.  O / l and the LSE do not
    // depend on the m used, so this is exact, and the O rescale runs only on
    // tiles where some row of the wavefront moved its m.
    float mxv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) mxv[i] = C::MB == 2 ? fmaxf(sacc[0][i], sacc[C::MB - 1][i]) : sacc[0][i];
#pragma unroll
    for (int i = 0; i < 8; ++i) mxv[i] = fmaxf(mxv[i], mxv[i + 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) mxv[i] = fmaxf(mxv[i], mxv[i + 4]);
    float mx = fmaxf(fmaxf(mxv[0], mxv[1]), fmaxf(mxv[2], mxv[3]));
    mx = fmaxf(mx, swap_halves(mx)) * cscale;
    const bool move = mx > m_run + kRescaleSlack;  // also true on the first live tile
    if (wave_any(move)) {
      const float m_new = move ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == neg_inf()) ? 0.f : m_run;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[mb][i] = fast_exp2(__builtin_fmaf(sacc[mb][i], cscale, -m_use));
    {
      float ps[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i] = C::MB == 2 ? sacc[0][i] + sacc[C::MB - 1][i] : sacc[0][i];
      l_run += tree_sum16(ps);
    }

    // O^T += V^T P^T
    if constexpr (KW == 8) {
      constexpr int PV = BC / 16;
      frag pf[PV];
#pragma unroll
      for (int t = 0; t < PV; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[t][e] = static_cast<T>(sacc[t >> 1][8 * (t & 1) + e]);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const T *vrow = vt + (32 * db + l32) * C::VROW + 8 * h;
#pragma unroll
        for (int t = 0; t < PV; ++t) {
          const u32x4 vv = *reinterpret_cast<const u32x4 *>(vrow + 16 * t);
          oacc[db] = M::mma(__builtin_bit_cast(frag, vv), pf[t], oacc[db]);
        }
      }
    } else {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const T *vrow = vt + (32 * db + l32) * C::VROW + 4 * h;
#pragma unroll
        for (int u = 0; u < BC / 8; ++u) {
          const f32x4 vv = *reinterpret_cast<const f32x4 *>(vrow + 8 * u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * u + e;
            oacc[db] = M::mma(vv[e], sacc[t >> 4][t & 15], oacc[db]);
          }
        }
      }
    }
  };

  // ---- main loop over K/V tiles, double-buffered ----
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

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l) ----
  const float l_tot = l_run + swap_halves(l_run);
  if (row < a.Sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *orow = static_cast<T *>(a.o) + b * a.o_sb + hq * a.o_sh + static_cast<long long>(row) * a.o_ss;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = to_out<T>(oacc[db][4 * g + e] * inv);
        T *dst = orow + 32 * db + 8 * g + 4 * h;
        if constexpr (ES == 4) *reinterpret_cast<u32x4 *>(dst) = __builtin_bit_cast(u32x4, out);
        else *reinterpret_cast<u32x2 *>(dst) = __builtin_bit_cast(u32x2, out);
      }
    if (a.lse != nullptr && h == 0)
      a.lse[b * a.lse_sb + hq * a.lse_sh + row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : neg_inf();
  }
}

// ---------------------------------------------------------------------------
// Kernel for the 16-bit types.  Per K/V tile a wavefront computes S^T = K Q^T,
// the online softmax and O^T += V^T P^T.  Global loads go through a buffer
// resource placed at the tile's first row, so per-lane offsets are loop
// constants and rows past the end of the keys (or tiles past the workgroup's
// range) read as zero without any per-lane address arithmetic.  LDS fragments
// are read a full 32-key block ahead of the MFMAs that consume them.
// ---------------------------------------------------------------------------
#ifndef FA16_WAVES_PER_EU
#define FA16_WAVES_PER_EU 2
#endif

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(FA16_WAVES_PER_EU)))
void fwd_mfma16_kernel(const FwdArgs a) {
  using C = Cfg16<T, D>;
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int BC = C::BC, EPC = C::EPC, CH = C::CH, ES = C::ES;
  constexpr int QS = D / 16;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *kbuf = reinterpret_cast<T *>(smem);   // [2][BC][KROW]
  T *vbuf = kbuf + 2 * C::K_TILE;          // [2][D][VROW]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, a.nq, a.B * a.Hq, CAUSAL, bh, qt);
  const int b = bh / a.Hq, hq = bh - b * a.Hq, hk = hq / a.G;
  const int i0 = qt * C::BR;
  const int wrow0 = i0 + 32 * wave;
  const int row = wrow0 + l32;

  // ---- Q rows into registers: lane half h holds d in [D/2*h, D/2*h + D/2) ----
  frag qf[QS];
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(static_cast<const T *>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_ext);
    const bool ok = row < a.Sq;
#pragma unroll
    for (int c = 0; c < QS; ++c)
      qf[c] = __builtin_bit_cast(frag, buf_load16(rq, ok ? row * a.q_ss + ((D / 2) * h + c * EPC) * ES : kOOB));
    wait_vmem_all();
  }

  const int coff = a.Sk - a.Sq;
  int n_kt = (a.Sk + BC - 1) / BC;
  int w_kt = n_kt;
  if (CAUSAL) {
    const int last_wg = i0 + C::BR - 1 + coff;
    n_kt = min(n_kt, last_wg < 0 ? 0 : last_wg / BC + 1);
    const int last_w = wrow0 + 31 + coff;
    w_kt = min(n_kt, last_w < 0 ? 0 : last_w / BC + 1);
  }

  // ---- per-tile buffer resources, loop-constant lane offsets ----
  const char *kbase = reinterpret_cast<const char *>(static_cast<const T *>(a.k) + b * a.k_sb + hk * a.k_sh);
  const char *vbase = reinterpret_cast<const char *>(static_cast<const T *>(a.v) + b * a.v_sb + hk * a.v_sh);
  auto tile_rsrc = [&](const char *base, unsigned ss, unsigned ext, int j) {
    const unsigned long long shift = static_cast<unsigned long long>(j) * BC * ss;
    const unsigned recs = (j < n_kt && shift < ext) ? ext - static_cast<unsigned>(shift) : 0u;
    return make_rsrc(base + shift, recs);
  };
  const int k_c = tid % CH, k_r = tid / CH;
  const int v_g = tid % C::NG, v_c = tid / C::NG;
  unsigned koff[C::PASSES], voff[C::PASSES];
#pragma unroll
  for (int p = 0; p < C::PASSES; ++p) {
    koff[p] = (k_r + (C::NT / CH) * p) * a.k_ss + k_c * 16;
    voff[p] = (v_g * C::KPT + p) * a.v_ss + v_c * 16;
  }
  // two register sets: tile j is fetched two iterations before it is staged
  u32x4 kreg[2][C::PASSES], vreg[2][C::PASSES];
  auto load_kv = [&](int set, int j) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, a.k_ss, a.k_ext, j);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase, a.v_ss, a.v_ext, j);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) kreg[set][p] = buf_load16(rk, koff[p]);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) vreg[set][p] = buf_load16(rv, voff[p]);
  };
  auto store_kv = [&](int set, int buf) {
    T *ks = kbuf + buf * C::K_TILE;
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p)
      *reinterpret_cast<u32x4 *>(ks + k_lds_row<8>(k_r + (C::NT / CH) * p) * C::KROW + k_c * EPC) = kreg[set][p];
    T *vt = vbuf + buf * C::V_TILE;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      T col[C::KPT];
#pragma unroll
      for (int p = 0; p < C::KPT; ++p) col[p] = reinterpret_cast<const T *>(&vreg[set][p])[e];
      T *dst = vt + (v_c * EPC + e) * C::VROW + v_g * C::KPT;
      if constexpr (C::KPT * ES == 8) *reinterpret_cast<u32x2 *>(dst) = __builtin_bit_cast(u32x2, col);
      else if constexpr (C::KPT * ES == 4) *reinterpret_cast<unsigned *>(dst) = __builtin_bit_cast(unsigned, col);
      else *reinterpret_cast<unsigned short *>(dst) = __builtin_bit_cast(unsigned short, col);
    }
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};

  // S^T = K Q^T from K buffer `buf`.  All 8 fragments of one 32-key block are
  // read before its MFMAs, and the next block's reads are issued as the
  // current block's fragments are consumed, so LDS latency hides behind MFMAs.
  auto qk = [&](int buf, f32x16 s[2]) {
    const T *kt = kbuf + buf * C::K_TILE + l32 * C::KROW + (D / 2) * h;
    u32x4 kf[QS];
#pragma unroll
    for (int c = 0; c < QS; ++c) kf[c] = *reinterpret_cast<const u32x4 *>(kt + c * EPC);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < QS; ++c) {
      s[0] = M::mma(__builtin_bit_cast(frag, kf[c]), qf[c], s[0]);
      kf[c] = *reinterpret_cast<const u32x4 *>(kt + 32 * C::KROW + c * EPC);
    }
#pragma unroll
    for (int c = 0; c < QS; ++c) s[1] = M::mma(__builtin_bit_cast(frag, kf[c]), qf[c], s[1]);
    // keep the reads QS fragments ahead of the MFMAs that consume them
    __builtin_amdgcn_sched_group_barrier(0x100, QS, 0);
#pragma unroll
    for (int c = 0; c < QS; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, QS, 0);
  };
  // O^T += V^T P^T from V buffer `buf`, same read-ahead scheme
  auto pv = [&](int buf, const frag pf[4]) {
    const T *vt = vbuf + buf * C::V_TILE + l32 * C::VROW + 8 * h;
    u32x4 vf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vf[i] = *reinterpret_cast<const u32x4 *>(vt + (i >> 2) * 32 * C::VROW + 16 * (i & 3));
#pragma unroll
    for (int i = 0; i < 4 * C::DB; ++i) {
      const int db = i >> 2, tt = i & 3;
      oacc[db] = M::mma(__builtin_bit_cast(frag, vf[i & 7]), pf[tt], oacc[db]);
      if (i + 8 < 4 * C::DB)
        vf[i & 7] = *reinterpret_cast<const u32x4 *>(vt + ((i + 8) >> 2) * 32 * C::VROW + 16 * ((i + 8) & 3));
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i + 8 < 4 * C::DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  float m_run = neg_inf();
  float l_run = 0.f;
  const float cscale = a.c;

  // ---- prologue: tile 0 staged, tiles 1 and 2 in flight ----
  load_kv(0, 0);
  load_kv(1, 1);
  store_kv(0, 0);
  load_kv(0, 2);
  __syncthreads();

  // iteration j computes tile j from stage j&1, stages tile j+1 (register set
  // (j+1)&1, fetched two iterations earlier) into stage (j+1)&1, which held
  // tile j-1, and refills that register set with tile j+3
  auto iter = [&](auto set_tag, int j) {
    constexpr int nset = decltype(set_tag)::value;  // (j + 1) & 1
    const int st = j & 1;
    if (j < w_kt) {
      f32x16 s_cur[2];
      __builtin_amdgcn_s_setprio(1);  // matrix phase first when two waves compete
      qk(st, s_cur);
      __builtin_amdgcn_s_setprio(0);
      const int j0 = j * BC;
      // mask (tiles that cross the diagonal or the end of the keys)
      const bool edge = (j0 + BC > a.Sk) || (CAUSAL && j0 + BC - 1 > wrow0 + coff);
      if (edge) {
        const int lim = min(a.Sk - 1 - j0, CAUSAL ? row + coff - j0 : BC);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (acc_key<8>(mb, i, h) > lim) s_cur[mb][i] = neg_inf();
      }
      // row max of the tile (max3 tree, then the other lane half)
      float t[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int x = 3 * i, y = 3 * i + 1, z = 3 * i + 2;
        t[i] = max3f(s_cur[x >> 4][x & 15], s_cur[y >> 4][y & 15], s_cur[z >> 4][z & 15]);
      }
      t[10] = fmaxf(s_cur[1][14], s_cur[1][15]);
      float mx = max3f(max3f(t[0], t[1], t[2]), max3f(t[3], t[4], t[5]), max3f(t[6], t[7], max3f(t[8], t[9], t[10])));
      mx = fmaxf(mx, swap_halves(mx)) * cscale;
      // lazy running max: move only when the tile max exceeds it by the slack
      const bool move = mx > m_run + kRescaleSlack;
      const float m_new = move ? mx : m_run;
      const float alpha = move ? fast_exp2(m_run - m_new) : 1.f;  // 0 when m_run = -inf
      m_run = m_new;
      if (wave_any(move)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
      }
      const float m_use = (m_run == neg_inf()) ? 0.f : m_run;
      frag pf[4];
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        unsigned w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(__builtin_fmaf(s_cur[tt >> 1][8 * (tt & 1) + 2 * e], cscale, -m_use));
          const float p1 = fast_exp2(__builtin_fmaf(s_cur[tt >> 1][8 * (tt & 1) + 2 * e + 1], cscale, -m_use));
          typedef T v2 __attribute__((ext_vector_type(2)));
          w[e] = __builtin_bit_cast(unsigned, v2{static_cast<T>(p0), static_cast<T>(p1)});
          // the row sum uses the unrounded probabilities: the LSE must not
          // carry the rounding of P to 16 bits
          ls[e] += p0 + p1;
        }
        pf[tt] = __builtin_bit_cast(frag, u32x4{w[0], w[1], w[2], w[3]});
      }
      l_run = __builtin_fmaf(l_run, alpha, (ls[0] + ls[1]) + (ls[2] + ls[3]));
      __builtin_amdgcn_s_setprio(1);
      pv(st, pf);
      __builtin_amdgcn_s_setprio(0);
    }
    store_kv(nset, st ^ 1);
    load_kv(nset, j + 3);
    __syncthreads();
  };
  for (int j = 0; j < n_kt; j += 2) {
    iter(std::integral_constant<int, 1>{}, j);
    if (j + 1 < n_kt) iter(std::integral_constant<int, 0>{}, j + 1);
  }

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l) ----
  const float l_tot = l_run + swap_halves(l_run);
  if (row < a.Sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *orow = static_cast<T *>(a.o) + b * a.o_sb + hq * a.o_sh + static_cast<long long>(row) * a.o_ss;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * g + 4 * h) = __builtin_bit_cast(u32x2, out);
      }
    if (a.lse != nullptr && h == 0)
      a.lse[b * a.lse_sb + hq * a.lse_sh + row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : neg_inf();
  }
}

template <typename T, int D, bool CAUSAL>
int launch_one(const FwdArgs &args, hipStream_t stream) {
  using C = Cfg<T, D>;
  void (*kern)(FwdArgs);
  if constexpr (sizeof(T) == 2) kern = fwd_mfma16_kernel<T, D, CAUSAL>;
  else kern = fwd_mfma_kernel<T, D, CAUSAL>;
  constexpr int threads = sizeof(T) == 2 ? Cfg16<T, D>::NT : 256;
  constexpr int lds_bytes = sizeof(T) == 2 ? Cfg16<T, D>::LDS_BYTES : C::LDS_BYTES;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  });
  if (attr_err != hipSuccess)
    return fa_set_error(FA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(attr_err));
  const unsigned grid = static_cast<unsigned>(args.nq) * args.B * args.Hq;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds_bytes, stream, args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "launch: %s", hipGetErrorString(e));
  return FA_OK;
}

template <typename T, int D> int launch_causal(const FwdArgs &args, bool causal, hipStream_t s) {
  return causal ? launch_one<T, D, true>(args, s) : launch_one<T, D, false>(args, s);
}

template <typename T> int launch_dtype(const FwdArgs &args, int d, bool causal, hipStream_t s) {
  return d == 64 ? launch_causal<T, 64>(args, causal, s) : launch_causal<T, 128>(args, causal, s);
}

}  // namespace fa

int fa_launch_fwd_mfma(const fa_fwd_params *p, void *stream) {
  using namespace fa;
  const int es = fa_dtype_size(p->in_dtype);
  const FwdArgs args = make_fwd_args(p, es == 2 ? 256 : 128, es);  // query rows per workgroup
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (p->in_dtype) {
    case FA_F32: return launch_dtype<float>(args, p->d, p->causal != 0, s);
    case FA_BF16: return launch_dtype<__bf16>(args, p->d, p->causal != 0, s);
    case FA_F16: return launch_dtype<_Float16>(args, p->d, p->causal != 0, s);
    default: return fa_set_error(FA_ERR_UNSUPPORTED, "dtype %d has no MFMA forward kernel", p->in_dtype);
  }
}
