// Prefill forward for fp32 / bf16 / fp16 inputs on gfx950 matrix cores.
//
// Method (FlashAttention interview canvas, panel 1 "one-sentence answer" and
// "online softmax key state" boxes; panel 2, v1 card): K/V tiles are staged in
// on-chip memory, and for every tile the scores, the online-softmax update and
// the P V accumulation are done in registers, so the score matrix never reaches
// HBM.  A workgroup owns a block of query rows of one (batch, head) — the v2
// card's partitioning of a single head across workgroups — and each wavefront
// owns 32 rows end to end, so no reduction crosses wavefronts.
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
//     single 16-byte LDS read; its rows are padded by 16 bytes, which keeps
//     16-byte reads free of bank conflicts.  In the 16-bit kernel K goes from
//     memory straight into LDS (direct-to-LDS buffer loads, no registers), in
//     unpadded rows whose 16-byte chunks are XOR-swizzled by the row instead;
//     the fp32 kernel pads its K rows.
//   * Scores are kept in the log2 domain (scale * log2 e folded into one FMA) and
//     exponentiated with the hardware exp2; the running max moves lazily.
//   * 16-bit kernel: O is divided by the sum of the probabilities as rounded
//     for P V (accumulated with v_dot2 against (1, 1) on the packed words), the
//     LSE by the sum of the unrounded ones.  O is then a weighted mean of V
//     rows whose weights carry only the 2^-9 (bf16) rounding of each
//     probability relative to the others: a row whose softmax rests on one key
//     returns that key's V row unchanged, where normalising by the unrounded
//     sum would scale it by up to 1 +- 2^-9.  On the long-context workload with
//     1 % outlier keys that moves the largest error of O from about 0.03 to
//     0.016 (bf16 output rounding is up to 0.0156 there).
//   * 16-bit kernel: 8 wavefronts over 256 rows, software-pipelined so that
//     every wavefront has MFMA, vector and LDS work in flight at once: P V of
//     tile t carries the first half of tile t+1's softmax between its MFMAs,
//     and S^T of tile t+2 the second half; K/V staging rides along too (K of
//     tile t+3 straight into LDS, V of tile t+1 from registers), with one
//     barrier per tile.
//   * Causal tiles past a wavefront's last row are skipped; the mask is applied
//     only on tiles that cross the diagonal or the end of the keys.  Workgroups
//     are issued heaviest first and grouped so each XCD works on a contiguous
//     range of (batch, head) pairs, whose K/V then stay in that XCD's L2.
#include "fa_device.hpp"
#include "fa_fwd_common.hpp"
#include "fa_internal.h"

#include <mutex>
#include <type_traits>
#include <utility>

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


// 16 bytes per lane from a buffer resource straight into LDS, bypassing the
// registers: lane i of the wavefront writes bytes [16 i, 16 i + 16) past
// lds_base (wave-uniform), whatever offset it reads from.  Words past the
// resource's end arrive as zeros.  The compiler tracks neither the LDS write
// nor its completion: wait for it with wait_vmem<N> before the barrier that
// publishes the bytes.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void *lds_base, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, off, 0, 0, 0);
}

// Keeps the compiler from moving memory operations across this point, so
// that counts of the loads issued after a direct-to-LDS load hold as written.
// No instruction is emitted.
__device__ __forceinline__ void mem_order() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(N): wait until at most N vector memory operations of this
// wavefront are outstanding.  They complete in the order issued, so this
// waits for all but the N most recent.
template <int N> __device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt holds six bits");
  mem_order();
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Configuration of the 16-bit kernel: 8 wavefronts (two per SIMD) own 256 query
// rows, so each K/V tile is fetched and staged once for twice as many rows.
// K rows sit in LDS unpadded, as whole kilobytes per wavefront load (the
// direct-to-LDS loads write 1 KiB runs); the 16-byte chunks of each row are
// XOR-swizzled by the row (ksw), so 16 lanes reading one chunk of 16
// consecutive rows cover all 64 banks.
template <typename T, int D, int NT_> struct Cfg16 {
  static constexpr int ES = sizeof(T);
  static constexpr int KW = 8;
  static constexpr int NT = NT_;                // threads per workgroup
  static constexpr int BR = NT / 2;             // query rows per workgroup (32 per wavefront)
  static constexpr int BC = 64;                 // keys per tile
  static constexpr int EPC = 8;                 // elements per 16-byte chunk
  static constexpr int CH = D / EPC;            // chunks per row
  static constexpr int PASSES = BC * CH / NT;   // 16-byte loads per thread per tile (K or V)
  static constexpr int KPT = PASSES;            // keys per thread in the V transpose
  static constexpr int NG = BC / KPT;           // V key groups
  static constexpr int NW = NT / 64;            // wavefronts
  static constexpr int KROW = D;                // K row in LDS (chunks swizzled, no padding)
  static constexpr int RPS = 256 / (D * ES);    // K rows per 256 bytes (one pass over the banks)
  static constexpr int VROW = BC + EPC;         // V^T row in LDS, +16 bytes
  static constexpr int SROW = D + EPC;          // epilogue slab row, +16 bytes
  static constexpr int K_TILE = BC * KROW;
  static constexpr int V_TILE = D * VROW;
  static constexpr int DB = D / 32;
  static constexpr int STAGE_BYTES = 2 * (K_TILE + V_TILE) * ES;
  static constexpr int SLAB_BYTES = NW * 32 * SROW * ES;
  static constexpr int LDS_BYTES = STAGE_BYTES > SLAB_BYTES ? STAGE_BYTES : SLAB_BYTES;
  static_assert(BC * CH % NT == 0, "tile must split evenly over the workgroup");
  static_assert(K_TILE * ES == NW * PASSES * 1024, "each wavefront's K loads fill whole kilobytes of the tile");
  static_assert(RPS >= 1 && 256 % (D * ES) == 0 && (32 / RPS) % CH == 0,
                "rows 32 apart must share their swizzle");
  // swizzle of LDS row r: stored chunk s holds the row's chunk s ^ ksw(r)
  static __device__ __forceinline__ int ksw(int r) { return (r / RPS) & (CH - 1); }
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
  map_block(blockIdx.x, a.nq, a.B * a.Hq, a.G, CAUSAL, bh, qt);
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
// the online softmax and O^T += V^T P^T, software-pipelined over three tiles
// (see the main loop).  Global loads go through a buffer resource placed at
// the tile's first row, so per-lane offsets are loop constants and rows past
// the end of the keys (or tiles past the workgroup's range) read as zero
// without any per-lane address arithmetic.  K tiles are loaded straight into
// LDS, so the compiler does not see when they land: each wavefront waits for
// its own K loads (vmcnt) before the barrier that publishes them.  LDS
// fragments are read four MFMAs ahead of the MFMAs that consume them.
// ---------------------------------------------------------------------------
#ifndef FA16_WAVES_PER_EU
#define FA16_WAVES_PER_EU 2
#endif


// SEXP: a quarter of the exponentials (the second of every other pair) by
// soft_exp2 on the FMA pipe, the FlashAttention-4 card's split between the
// exponential unit and the FMA units; off by default (on this part the
// transcendental shares the vector issue with the FMAs).
template <typename T, int D, bool CAUSAL, int NT, bool SEXP = false, bool WLSE = true>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(FA16_WAVES_PER_EU)))
void fwd_mfma16_kernel(const FwdArgs a) {
  using C = Cfg16<T, D, NT>;
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int BC = C::BC, EPC = C::EPC, CH = C::CH, ES = C::ES;
  constexpr int QS = D / 16;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *kbuf = reinterpret_cast<T *>(smem);   // [2][BC][KROW]
  T *vbuf = kbuf + 2 * C::K_TILE;          // [2][D][VROW]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: the causal tile ranges, loop bounds and buffer resources stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, a.nq, a.B * a.Hq, a.G, CAUSAL, bh, qt);
  const int b = bh / a.Hq, hq = bh - b * a.Hq, hk = hq / a.G;
  const int i0 = qt * C::BR;
  const int wrow0 = i0 + 32 * wave;
  const int row = wrow0 + l32;

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
  // a tile at or past n_kt gets zero records (its loads return zeros); for a
  // live tile the first row (j * BC <= Sk - 1) starts inside the slice, so the
  // 32-bit shift cannot overflow and the records stay positive
  auto tile_rsrc = [&](const char *base, unsigned ss, unsigned ext, int j) {
    const bool live = j < n_kt;
    const unsigned shift = live ? static_cast<unsigned>(j * BC) * ss : 0u;
    return make_rsrc(base + shift, live ? ext - shift : 0u);
  };
  // K: load p of wavefront w fills kilobyte p * NW + w of the tile, lane by
  // lane; each lane fetches the (key, chunk) that the row order and the
  // swizzle put at its 16 bytes
  const int v_g = tid % C::NG, v_c = tid / C::NG;
  unsigned koff[C::PASSES], voff[C::PASSES];
#pragma unroll
  for (int p = 0; p < C::PASSES; ++p) {
    const int pos = (p * C::NW + wave) * 1024 + lane * 16;  // byte within the K tile
    const int r = pos / (D * ES), sc16 = (pos % (D * ES)) / 16;
    koff[p] = k_lds_row<8>(r) * a.k_ss + (sc16 ^ C::ksw(r)) * 16;
    voff[p] = (v_g * C::KPT + p) * a.v_ss + v_c * 16;
  }
  auto k_dst = [&](int buf, int p) {
    return reinterpret_cast<unsigned char *>(kbuf + buf * C::K_TILE) + (p * C::NW + wave) * 1024;
  };
  auto load_k_lds = [&](int buf, int j) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(kbase, a.k_ss, a.k_ext, j);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) buf_load16_lds(r, k_dst(buf, p), koff[p]);
  };
  // the same placement through registers (the prologue's third K tile)
  auto load_k_to = [&](u32x4 *dst, int j) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(kbase, a.k_ss, a.k_ext, j);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) dst[p] = buf_load16(r, koff[p]);
  };
  auto store_k_from = [&](const u32x4 *src, int buf) {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) *reinterpret_cast<u32x4 *>(k_dst(buf, p) + lane * 16) = src[p];
  };
  u32x4 vreg[C::PASSES];
  auto load_v = [&](int j) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(vbase, a.v_ss, a.v_ext, j);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) vreg[p] = buf_load16(r, voff[p]);
  };
  auto store_v = [&](int buf) {
    T *vt = vbuf + buf * C::V_TILE;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      T col[C::KPT];
#pragma unroll
      for (int p = 0; p < C::KPT; ++p) col[p] = reinterpret_cast<const T *>(&vreg[p])[e];
      T *dst = vt + (v_c * EPC + e) * C::VROW + v_g * C::KPT;
      if constexpr (C::KPT * ES == 8) *reinterpret_cast<u32x2 *>(dst) = __builtin_bit_cast(u32x2, col);
      else if constexpr (C::KPT * ES == 4) *reinterpret_cast<unsigned *>(dst) = __builtin_bit_cast(unsigned, col);
      else *reinterpret_cast<unsigned short *>(dst) = __builtin_bit_cast(unsigned short, col);
    }
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  frag qf[QS];  // this lane's query row; lane half h holds d in [D/2*h, D/2*h + D/2)

  // ---- blocks of the main loop: MFMAs with LDS operands read RA ahead, and
  // softmax work of the neighbouring tile dealt out over the MFMA slots ----
  constexpr int RA = 4;
  constexpr int NQK = 2 * QS;     // MFMAs of S^T = K Q^T per tile
  constexpr int NPV = 4 * C::DB;  // MFMAs of O^T += V^T P^T per tile
  constexpr int STEPS = 16;       // steps of each softmax half
  static_assert(STEPS % NQK == 0 && STEPS % NPV == 0, "softmax steps must split evenly over the MFMA slots");
  // MFMA i of S^T: key block i & 1, head-dim step i >> 1 (two independent
  // chains).  Step j takes chunk j of the row in lane half 0 and chunk
  // CH/2 + j in half 1; the swizzle makes each step's address its own
  // register (rows l32 and l32 + 32 share it).
  int k_lane[QS];
#pragma unroll
  for (int j = 0; j < QS; ++j) k_lane[j] = l32 * C::KROW + (((CH / 2) * h + j) ^ C::ksw(l32)) * EPC;
  const T *v_lane = vbuf + l32 * C::VROW + 8 * h;
  auto kfrag = [&](int buf, int i) {
    return *reinterpret_cast<const u32x4 *>(kbuf + buf * C::K_TILE + (i & 1) * 32 * C::KROW + k_lane[i >> 1]);
  };
  // MFMA i of O^T: head-dim block i >> 2, key step i & 3
  auto vfrag = [&](int buf, int i) {
    return *reinterpret_cast<const u32x4 *>(v_lane + buf * C::V_TILE + (i >> 2) * 32 * C::VROW + 16 * (i & 3));
  };

  // ---- online softmax state ----
  float m_run = neg_inf();
  float l_run = 0.f;    // lane-partial sum of the unrounded probabilities (LSE)
  float lr_run = 0.f;   // ... of the probabilities as rounded for P V (O's divisor)
  float alpha_p = 1.f;  // rescale factor of the tile last through the first half
  bool move_p = false;  // whether it differs from 1 in this lane
  float m_use = 0.f;    // the running max its exponents are taken against
  const float cscale = a.c;

  // mask the keys of tile j past the end of the keys or the diagonal
  // (on edge tiles only; the lane's row and half are taken afresh from the
  // lane id, so they need not stay live through the loop)
  auto mask = [&](f32x16 s[2], int j) {
    const int j0 = j * BC;
    const bool edge = (j0 + BC > a.Sk) || (CAUSAL && j0 + BC - 1 > wrow0 + coff);
    if (edge) {
      const int fl = fresh_lane_id();
      const int lim = min(a.Sk - 1 - j0, CAUSAL ? wrow0 + (fl & 31) + coff - j0 : BC);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (acc_key<8>(mb, i, fl >> 5) > lim) s[mb][i] = neg_inf();
    }
  };
  // First half, in 16 steps: tile max (max3 tree, then the other lane half),
  // lazy running-max update, exponents of s[0].
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
      // lazy running max: move only when the tile max exceeds it by the slack
      move_p = mxa > m_run + kRescaleSlack;
    } else if constexpr (st == 6) {
      const float m_new = move_p ? mxa : m_run;
      alpha_p = move_p ? fast_exp2(m_run - m_new) : 1.f;  // 0 when m_run = -inf
      m_run = m_new;
      m_use = (m_run == neg_inf()) ? 0.f : m_run;
      pin(alpha_p);
      pin(m_use);
    } else if constexpr (st < 15) {
      constexpr int e = 2 * (st - 7);
      float p0 = fast_exp2(__builtin_fmaf(s[0][e], cscale, -m_use));
      const float x1 = __builtin_fmaf(s[0][e + 1], cscale, -m_use);
      float p1 = (SEXP && (st & 1)) ? soft_exp2(x1) : fast_exp2(x1);
      pin(p0);
      pin(p1);
      s[0][e] = p0;
      s[0][e + 1] = p1;
    }
  };
  // Second half, in 16 steps: exponents of s[1]; P^T rounded to 16 bits, two
  // scores per word; row sum of the unrounded probabilities (the LSE must not
  // carry the rounding of P) as a balanced tree; l update.
  float ps[16], qa[8];
  unsigned pw[16];
  auto pack2 = [&](float x0, float x1) {
    typedef T v2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, v2{static_cast<T>(x0), static_cast<T>(x1)});
  };
  // acc + the two rounded probabilities of a packed word (exact products)
  auto add_rounded = [&](unsigned w, float acc) {
    typedef T v2 __attribute__((ext_vector_type(2)));
    const v2 one = {static_cast<T>(1.f), static_cast<T>(1.f)};
    if constexpr (std::is_same<T, __bf16>::value)
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, w), one, acc, false);
    else
      return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, w), one, acc, false);
  };
  auto soft_b_step = [&](auto step_tag, f32x16 s[2]) {
    constexpr int st = decltype(step_tag)::value;
    if constexpr (st < 8) {
      float p0 = fast_exp2(__builtin_fmaf(s[1][2 * st], cscale, -m_use));
      const float x1 = __builtin_fmaf(s[1][2 * st + 1], cscale, -m_use);
      float p1 = (SEXP && (st & 1)) ? soft_exp2(x1) : fast_exp2(x1);
      pin(p0);
      pin(p1);
      s[1][2 * st] = p0;
      s[1][2 * st + 1] = p1;
      pw[st] = pack2(s[0][2 * st], s[0][2 * st + 1]);
      pin(pw[st]);
      if constexpr (st == 0) lr_run *= alpha_p;
      lr_run = add_rounded(pw[st], lr_run);
    } else {
      pw[st] = pack2(s[1][2 * (st - 8)], s[1][2 * (st - 8) + 1]);
      pin(pw[st]);
      lr_run = add_rounded(pw[st], lr_run);
      if constexpr (!WLSE) {
        // no LSE output: O needs only the rounded sum
      } else if constexpr (st < 12) {
        constexpr int mb = (st - 8) >> 1, base = 4 * ((st - 8) & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ps[8 * mb + base + i] = s[mb][2 * (base + i)] + s[mb][2 * (base + i) + 1];
          pin(ps[8 * mb + base + i]);
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
        l_run = __builtin_fmaf(l_run, alpha_p, (qa[0] + qa[2]) + (qa[1] + qa[3]));
        pin(l_run);
      }
    }
  };
  auto p_pack = [&](f32x16 s[2]) {
    s[0] = __builtin_bit_cast(f32x16, i32x16{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5],
                                             (int)pw[6], (int)pw[7], (int)pw[8], (int)pw[9], (int)pw[10], (int)pw[11],
                                             (int)pw[12], (int)pw[13], (int)pw[14], (int)pw[15]});
  };
  auto rescale_o = [&]() {
    if (wave_any(move_p)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha_p;
    }
  };

  // first RA operand fragments of a block, read ahead by the caller
  auto k_init = [&](int buf, u32x4 (&kf)[RA]) {
#pragma unroll
    for (int i = 0; i < RA; ++i) kf[i] = kfrag(buf, i);
  };
  auto v_init = [&](int buf, u32x4 (&vf)[RA]) {
#pragma unroll
    for (int i = 0; i < RA; ++i) vf[i] = vfrag(buf, i);
  };
  // S^T of K buffer `buf` into s, starting from the fragments kf; softmax
  // work on `sn` rides along: none (SOFT = 0), its second half (1) or both
  // halves (2)
  auto block_qk = [&](int buf, f32x16 s[2], f32x16 sn[2], auto soft_tag, auto &&extra, u32x4 (&kf)[RA]) {
    constexpr int SOFT = decltype(soft_tag)::value;
    s[0] = f32x16{};
    s[1] = f32x16{};
    static_for<NQK>([&](auto I) {
      constexpr int i = decltype(I)::value;
      s[i & 1] = M::mma(__builtin_bit_cast(frag, kf[i % RA]), qf[i >> 1], s[i & 1]);
      if constexpr (i + RA < NQK) kf[i % RA] = kfrag(buf, i + RA);
      if constexpr (SOFT == 1)
        static_for<STEPS / NQK>([&](auto K) {
          soft_b_step(std::integral_constant<int, i * (STEPS / NQK) + decltype(K)::value>{}, sn);
        });
      if constexpr (SOFT == 2)
        static_for<2 * STEPS / NQK>([&](auto K) {
          constexpr int st = i * (2 * STEPS / NQK) + decltype(K)::value;
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
  // O^T += V^T P^T of V buffer `buf`, P^T in p[0], starting from the
  // fragments vf; the first softmax half of `sn` rides along, and the slots
  // past the last V read fetch the first fragments kn of the next S^T block
  // (K buffer kbn), so that block starts without waiting on LDS
  auto block_pv = [&](int buf, const f32x16 &p, f32x16 sn[2], auto &&extra, u32x4 (&vf)[RA], int kbn,
                      u32x4 (&kn)[RA]) {
    frag pf[4];
    pf[0] = __builtin_bit_cast(frag, __builtin_shufflevector(p, p, 0, 1, 2, 3));
    pf[1] = __builtin_bit_cast(frag, __builtin_shufflevector(p, p, 4, 5, 6, 7));
    pf[2] = __builtin_bit_cast(frag, __builtin_shufflevector(p, p, 8, 9, 10, 11));
    pf[3] = __builtin_bit_cast(frag, __builtin_shufflevector(p, p, 12, 13, 14, 15));
    static_for<NPV>([&](auto I) {
      constexpr int i = decltype(I)::value;
      oacc[i >> 2] = M::mma(__builtin_bit_cast(frag, vf[i % RA]), pf[i & 3], oacc[i >> 2]);
      if constexpr (i + RA < NPV) vf[i % RA] = vfrag(buf, i + RA);
      else kn[i + RA - NPV] = kfrag(kbn, i + RA - NPV);
      static_for<STEPS / NPV>([&](auto K) {
        soft_a_step(std::integral_constant<int, i * (STEPS / NPV) + decltype(K)::value>{}, sn);
      });
      extra(I);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Two score register sets: sc[j & 1] holds S^T of tile j from its QK^T
  // until its softmax is done, then P^T (in its first half) until its P V.
  f32x16 sc[2][2];

  // ---- prologue: K of tiles 0-2 and V of tile 0 staged, tile 0 through its
  // softmax, S^T of tile 1 formed, V of tile 1 in flight.  The first tiles
  // and the Q rows are fetched together, so the prologue waits on one memory
  // round trip.  (K of tile 2 waits in registers until tile 0's buffer is
  // free.) ----
  load_k_lds(0, 0);
  load_k_lds(1, 1);
  mem_order();  // the loads below are counted as issued after these
  load_v(0);
  u32x4 k2[C::PASSES];
  load_k_to(k2, 2);
  // Q rows into registers
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(static_cast<const T *>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_ext);
    const bool ok = row < a.Sq;
#pragma unroll
    for (int c = 0; c < QS; ++c)
      qf[c] = __builtin_bit_cast(frag, buf_load16(rq, ok ? row * a.q_ss + ((D / 2) * h + c * EPC) * ES : kOOB));
  }
  store_v(0);
  load_v(1);
  // K of tiles 0 and 1 in LDS: everything but V of tile 0, K of tile 2, the
  // Q rows and V of tile 1 is done
  wait_vmem<3 * C::PASSES + QS>();
  __syncthreads();
  if (0 < w_kt) {
    u32x4 kf[RA];
    k_init(0, kf);
    block_qk(0, sc[0], sc[1], std::integral_constant<int, 0>{}, [](auto) {}, kf);
    mask(sc[0], 0);
    k_init(1, kf);
    block_qk(1, sc[1], sc[0], std::integral_constant<int, 2>{}, [](auto) {}, kf);
  }
  __syncthreads();
  store_k_from(k2, 0);
  __syncthreads();

  // Main loop.  Iteration t, for a wave whose rows reach tile t:
  //   O^T += V^T P^T of tile t, with the first half of tile t+1's softmax
  //   dealt out between its MFMAs;
  //   S^T of tile t+2, with the second half of tile t+1's softmax.
  // Every wave thus keeps matrix, vector and LDS work in flight together, and
  // the two waves of a SIMD fill each other's gaps.  Staging rides along:
  // K of tile t+3 goes straight into the K buffer of tile t+1 and V of tile
  // t+1 (fetched in the previous iteration) into the V buffer of tile t-1,
  // buffers no wave reads in this iteration; then V of tile t+2 is fetched.
  // One barrier per iteration publishes both, after the wave's own K loads
  // have landed.
  auto iter = [&](auto set_tag, int t) {
    constexpr int cur = decltype(set_tag)::value;  // t & 1
    constexpr int nxt = cur ^ 1;
    // V of tile t and K of tile t+2 both sit in buffer cur
    u32x4 vf[RA], kf[RA];
    v_init(cur, vf);  // first, so the reads overlap the rescale and mask
    rescale_o();
    mask(sc[nxt], t + 1);
    block_pv(cur, sc[cur][0], sc[nxt], [&](auto I) {
      if constexpr (decltype(I)::value == 0) {
        load_k_lds(nxt, t + 3);
        mem_order();
      }
      if constexpr (decltype(I)::value == 3) store_v(nxt);
    }, vf, cur, kf);
    block_qk(cur, sc[cur], sc[nxt], std::integral_constant<int, 1>{}, [&](auto I) {
      if constexpr (decltype(I)::value == 2) load_v(t + 2);
    }, kf);
    wait_vmem<C::PASSES>();  // this iteration's K loads; V of tile t+2 may be in flight
    __syncthreads();
  };
  // iterations past the wave's last tile (causal): staging only
  auto iter_stage = [&](auto set_tag, int t) {
    constexpr int nxt = decltype(set_tag)::value ^ 1;
    load_k_lds(nxt, t + 3);
    mem_order();
    store_v(nxt);
    load_v(t + 2);
    wait_vmem<C::PASSES>();
    __syncthreads();
  };
  // two loops with a single path each (the register sets alternate, so both
  // are unrolled by two and the second enters at the right parity)
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

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l).  The LDS is
  // free after the loop's last barrier: each wavefront transposes its 32 x D
  // block through its own LDS slab, so that global stores write whole rows
  // (16 lanes x 16 bytes per row) instead of 8-byte pieces of 32 rows.
  // The lane's indices are taken afresh from the lane id: kept live across
  // the loop, which does not use them, they would be spilled to scratch and
  // read back here, a memory round trip per work item. ----
  const int elane = fresh_lane_id();
  const int el32 = elane & 31, eh = elane >> 5, erow = wrow0 + el32;
  auto other_half = [&](float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, eh == 0 ? r[1] : r[0]);
  };
  const float l_tot = l_run + other_half(l_run);
  const float lr_tot = lr_run + other_half(lr_run);
  {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    T *slab = kbuf + wave * 32 * C::SROW;  // 32 rows of SROW elements (within LDS_BYTES)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = static_cast<T>(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<u32x2 *>(slab + el32 * C::SROW + 32 * db + 8 * g + 4 * eh) = __builtin_bit_cast(u32x2, out);
      }
    // the slab is private to the wavefront: LDS operations of one wavefront
    // complete in order, so its reads below see its writes above
    constexpr int RPI = 64 / CH;  // rows per store instruction
    T *obase = static_cast<T *>(a.o) + b * a.o_sb + hq * a.o_sh;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int r = k * RPI + elane / CH, c = elane % CH;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(slab + r * C::SROW + c * EPC);
      const int orow_i = wrow0 + r;
      if (orow_i < a.Sq) *reinterpret_cast<u32x4 *>(obase + static_cast<long long>(orow_i) * a.o_ss + c * EPC) = v;
    }
  }
  if (WLSE && erow < a.Sq && a.lse != nullptr && eh == 0)
    a.lse[b * a.lse_sb + hq * a.lse_sh + erow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : neg_inf();
}

template <typename T, int D, bool CAUSAL, int NT, bool SEXP = false, bool WLSE = true>
int launch_one(const FwdArgs &args, hipStream_t stream) {
  void (*kern)(FwdArgs);
  int lds_bytes;
  if constexpr (sizeof(T) == 2) {
    kern = fwd_mfma16_kernel<T, D, CAUSAL, NT, SEXP, WLSE>;
    lds_bytes = Cfg16<T, D, NT>::LDS_BYTES;
  } else {
    kern = fwd_mfma_kernel<T, D, CAUSAL>;
    lds_bytes = Cfg<T, D>::LDS_BYTES;
  }
  const unsigned grid = static_cast<unsigned>(args.nq) * args.B * args.Hq;
  fa_log_launch(sizeof(T) == 2 ? "fwd_mfma16_kernel" : "fwd_mfma_kernel", grid, NT, lds_bytes,
                "dtype=%s d=%d causal=%d B=%d Hq=%d G=%d Sq=%d Sk=%d rows_per_wg=%d soft_exp2=%d lse_sum=%d",
                sizeof(T) == 4 ? "f32" : (std::is_same<T, __bf16>::value ? "bf16" : "f16"), D, CAUSAL ? 1 : 0,
                args.B, args.Hq, args.G, args.Sq, args.Sk, sizeof(T) == 2 ? NT / 2 : Cfg<T, D>::BR, SEXP ? 1 : 0,
                WLSE ? 1 : 0);
  // the dynamic LDS limit is raised once per kernel and device, before the
  // kernel's first launch there (a host-side call, no stream work)
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static hipError_t attr_err[kMaxDevices] = {};
  int dev = -1;
  const hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return fa_set_error(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(de));
  if (dev < 0 || dev >= kMaxDevices) return fa_set_error(FA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::call_once(once[dev], [&] {
    attr_err[dev] = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  });
  if (attr_err[dev] != hipSuccess)
    return fa_set_error(FA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(attr_err[dev]));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lds_bytes, stream, args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "launch: %s", hipGetErrorString(e));
  return FA_OK;
}

template <typename T, int D, int NT> int launch_causal(const FwdArgs &args, bool causal, hipStream_t s) {
  return causal ? launch_one<T, D, true, NT>(args, s) : launch_one<T, D, false, NT>(args, s);
}

// Without an LSE output (args.lse null) the d = 128 kernel drops the row sum
// of the unrounded probabilities: O is divided by the sum of the rounded ones,
// which it keeps either way.
template <typename T, int NT> int launch_dtype(const FwdArgs &args, int d, bool causal, bool sexp, hipStream_t s) {
  if (sexp)  // validated: 16-bit inputs with d = 128
    return causal ? launch_one<T, 128, true, NT, true>(args, s) : launch_one<T, 128, false, NT, true>(args, s);
  if (d == 64) return launch_causal<T, 64, NT>(args, causal, s);
  if (args.lse == nullptr)
    return causal ? launch_one<T, 128, true, NT, false, false>(args, s)
                  : launch_one<T, 128, false, NT, false, false>(args, s);
  return launch_causal<T, 128, NT>(args, causal, s);
}

}  // namespace fa

int fa_launch_fwd_mfma(const fa_fwd_params *p, void *stream) {
  using namespace fa;
  const int es = fa_dtype_size(p->in_dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (es == 4) return launch_dtype<float, 256>(make_fwd_args(p, 128, es), p->d, p->causal != 0, false, s);
  // Short key ranges: workgroups of 256 threads (128 rows), two per compute
  // unit, so one workgroup's prologue and epilogue overlap the other's loop.
  // d = 64 up to 1024 keys: measured +13 % (causal) and +5.5 % at S = 512, +3 %
  // at 1024, neutral at 2048.  d = 128 up to 512 keys (with an LSE output and
  // the hardware exponential, the variants built for this launch): +2 %
  // causal and not at S = 512, but -4 % at 1024.
  const bool short64 = p->d == 64 && p->Sk <= 1024;
  const bool short128 = p->d == 128 && p->Sk <= 512 && p->lse != nullptr && p->soft_exp2 == 0;
  if (short64 || short128) {
    const FwdArgs args = make_fwd_args(p, 128, es);
    const bool c = p->causal != 0;
    switch (p->in_dtype) {
      case FA_BF16: return short64 ? launch_causal<__bf16, 64, 256>(args, c, s) : launch_causal<__bf16, 128, 256>(args, c, s);
      case FA_F16:
        return short64 ? launch_causal<_Float16, 64, 256>(args, c, s) : launch_causal<_Float16, 128, 256>(args, c, s);
      default: return fa_set_error(FA_ERR_UNSUPPORTED, "dtype %d has no MFMA forward kernel", p->in_dtype);
    }
  }
  constexpr int NT = 512;
  const FwdArgs args = make_fwd_args(p, NT / 2, es);  // 32 query rows per wavefront
  switch (p->in_dtype) {
    case FA_BF16: return launch_dtype<__bf16, NT>(args, p->d, p->causal != 0, p->soft_exp2 != 0, s);
    case FA_F16: return launch_dtype<_Float16, NT>(args, p->d, p->causal != 0, p->soft_exp2 != 0, s);
    default: return fa_set_error(FA_ERR_UNSUPPORTED, "dtype %d has no MFMA forward kernel", p->in_dtype);
  }
}
