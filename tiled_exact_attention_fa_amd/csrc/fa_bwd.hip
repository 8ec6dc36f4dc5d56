// Attention backward for bf16 / fp16 on gfx950 matrix cores, by recomputation.
//
// What is computed (FlashAttention interview canvas, panel 1 v1 card and panel
// 3 Q3: the forward keeps only O and one statistic per row, and the backward
// recomputes the local scores and probabilities from them): given dO, the
// gradients of O = softmax(tau Q K^T) V are
//     P  = exp(tau Q K^T - LSE)         recomputed tile by tile, never stored
//     dV = P^T dO        dP = dO V^T     dS = P * (dP - Dr),  Dr = rowsum(dO * O)
//     dQ = tau dS K      dK = tau dS^T Q
// (rowsum(dO * O) equals rowsum(P * dP), the softmax Jacobian's row term).
// Grouped-query heads: a key/value head's gradients sum over its query heads.
//
// MI355X design.  Three kernels, no atomics, so every result is deterministic:
//   * bwd_rowdot_kernel: Dr per query row, one 16-lane group per row.
//   * bwd_dkdv_kernel: a workgroup owns 256 keys of one (batch, kv head), a
//     wavefront 32 of them (8 wavefronts, two per SIMD); it walks every query
//     head of the group and every query tile that can see its keys, and keeps
//     dK^T and dV^T of its keys in registers until the end.  Per 32-row query
//     tile: S = Q K^T and dP = dO V^T with the keys' K rows in registers and V
//     rows in LDS as the B operands, then dV^T += dO^T P and dK^T += Q^T dS
//     with P and dS fed from the S and dP accumulators straight into the B
//     operand.
//   * bwd_dq_kernel: a workgroup owns 128 query rows of one (batch, head), a
//     wavefront 32 (two wavefronts per SIMD); per 32-key tile S^T = K Q^T and
//     dP^T = V dO^T with the rows' Q and dO in registers, then dQ^T += K^T dS^T.
//   * Each staged tile (query rows of Q and dO; keys of K and V) is written to
//     LDS once, row-major.  Row operands are read 16 bytes per lane in the
//     order of rows that puts the accumulators in operand order (below); the
//     transposed operands dO^T, Q^T and K^T come from the same rows through
//     gfx950's transposing LDS reads (ds_read_b64_tr_b16), so no tile is
//     stored twice.  Two LDS stages with register prefetch two tiles ahead:
//     one barrier per tile.
//   * The causal and ragged-edge masks are applied only on the tiles that
//     need them (a wave-uniform branch); every other tile runs the plain
//     exponential.  dP's accumulator starts at -Dr, so dS is one multiply.
//   * Optional two-role schedule for bwd_dkdv_kernel (the wave specialisation
//     of the FlashAttention-3 page's asynchrony section, on LDS barriers):
//     waves 0-3 run a tile's score phase while waves 4-7 run the previous
//     tile's accumulation phase, three barriers per tile.  Each wave still
//     takes every tile in the same order, so results equal the default
//     schedule's bit for bit.  On gfx950 it measured slower (the two roles
//     share each SIMD's issue slots, and the extra barriers cost more than the
//     overlap gains); it is kept selectable for that comparison.
// All products are 32x32x16 MFMAs on the input type with fp32 accumulation; P
// and dS are rounded to the input type only as MFMA operands.  Scores stay in
// the log2 domain (tau * log2 e folded into one multiply, hardware exp2).
#include "fa_device.hpp"
#include "fa_internal.h"

#include <type_traits>

namespace fa {

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *rowdot;  // [B][Hq][Sq]
  int B, Hq, Hkv, G, Sq, Sk;
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh, do_sb, do_sh;
  long long dq_sb, dq_sh, dk_sb, dk_sh, dv_sb, dv_sh, lse_sb, lse_sh;
  unsigned q_ss, k_ss, v_ss, o_ss, do_ss, dq_ss, dk_ss, dv_ss;  // row strides, bytes
  unsigned q_ext, k_ext, v_ext, o_ext, do_ext;                  // slice extents, bytes
  float c;      // softmax scale * log2(e)
  float scale;  // softmax scale
};

template <typename T> struct BwdMfma;
template <> struct BwdMfma<__bf16> {
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct BwdMfma<_Float16> {
  typedef f16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kBD = 128;      // head dim
constexpr int kEPC = 8;       // elements per 16-byte chunk
constexpr int kCH = kBD / kEPC;
constexpr int kTR = 32;       // rows of a staged tile

// Accumulator row order.  An operand row read from tile row perm_row(m) (bits
// 2 and 3 of m swapped) puts tile row 32 mb + 16 (i / 8) + 8 h + i % 8 in
// accumulator register i of lane half h — the order in which eight
// consecutive registers form the B operand of the next product.
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ int acc_row(int mb, int i, int h) { return 32 * mb + 16 * (i >> 3) + 8 * h + (i & 7); }

// LDS layout of a staged 32-row tile (256-byte rows, no padding inside a
// row): row r starts at byte 16 * (80 (r >> 2) + 20 (r & 3) + ((r >> 2) & 3)).
// In 16-byte units modulo 16 (the 64 four-byte banks), row r begins at
// 4 (r & 3) + ((r >> 2) & 3), so
//   * 16 lanes reading the same 16 bytes of 16 rows of one aligned group of
//     16 (the row operands) hit 16 different bank quads;
//   * 32 lanes of a transposing read, four consecutive rows times 64 bytes,
//     hit 16 different quads;
//   * 16 lanes storing one row's 16 chunks hit 16 different quads.
__host__ __device__ constexpr int row_off(int r) { return 16 * (80 * (r >> 2) + 20 * (r & 3) + ((r >> 2) & 3)); }
constexpr int kTileBytes = (row_off(kTR - 1) + 256 + 255) / 256 * 256;

// A 32-row x 128-element tile loaded by NT threads, one 16-byte chunk per
// thread and pass; 16 consecutive threads take one row (coalesced loads,
// conflict-free stores).
template <int NT> struct Tile {
  static constexpr int CPT = kTR * kCH / NT;  // chunks per thread
  u32x4 r[CPT];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, unsigned ss, int row0, int nrows) {
#pragma unroll
    for (int p = 0; p < CPT; ++p) {
      const int q = threadIdx.x + NT * p;
      const int rr = row0 + (q >> 4);
      r[p] = buf_load16(rs, rr < nrows ? static_cast<unsigned>(rr) * ss + (q & 15) * 16u : kOOB);
    }
  }
  __device__ __forceinline__ void store(char *dst) const {
#pragma unroll
    for (int p = 0; p < CPT; ++p) {
      const int q = threadIdx.x + NT * p;
      *reinterpret_cast<u32x4 *>(dst + row_off(q >> 4) + (q & 15) * 16) = r[p];
    }
  }
};

// Row operand: 16 bytes of this lane's tile row at byte `off` of it.
template <typename T> __device__ __forceinline__ typename BwdMfma<T>::frag lds_frag(const char *p) {
  return __builtin_bit_cast(typename BwdMfma<T>::frag, *reinterpret_cast<const u32x4 *>(p));
}

// Transposed operand from a staged tile: A[m][k] = tile[16 t + k][32 db + m]
// for the 32x32x16 product, lane (m, kh) holding k = 8 kh .. 8 kh + 7.  A
// ds_read_b64_tr_b16 gives lane i of each 16-lane group element i % 4 of the
// 8 bytes addressed by lane 4 j + i / 4, as its element j; so lane s of group
// g addresses row 16 t + 8 (g >> 1) + 4 rd + (s >> 2), columns
// 32 db + 16 (g & 1) + 4 (s & 3) .. + 3, and reads rd = 0, 1 give k = 8 kh +
// 0..3 and 4..7.  tr_lane() is the lane's part of that address; t and db
// move it by whole 4-row groups (5120 and 64 bytes), rd by 1296.
__device__ __forceinline__ int tr_lane(int lane) {
  const int g = (lane >> 4) & 3, s = lane & 15;
  return 2592 * (g >> 1) + 320 * (s >> 2) + 32 * (g & 1) + 8 * (s & 3);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p)));
}
template <typename T>
__device__ __forceinline__ typename BwdMfma<T>::frag tr_frag(const char *tile_lane, int t, int db) {
  const char *p = tile_lane + 5120 * t + 64 * db;
  const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 1296);
  return __builtin_bit_cast(typename BwdMfma<T>::frag, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

template <typename T> __device__ __forceinline__ unsigned pack2(float a, float b) {
  typedef T t2 __attribute__((ext_vector_type(2)));
  const t2 v = {static_cast<T>(a), static_cast<T>(b)};
  return __builtin_bit_cast(unsigned, v);
}

// ---- Dr = rowsum(dO * O): one 16-lane group per row, 16 rows per workgroup ----
template <typename T>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const BwdArgs a) {
  const int c = threadIdx.x & 15;
  const long long r = static_cast<long long>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const long long rows = static_cast<long long>(a.B) * a.Hq * a.Sq;
  float s = 0.f;
  long long i = 0, bh = 0;
  if (r < rows) {
    i = r % a.Sq;
    bh = r / a.Sq;
    const long long b = bh / a.Hq, h = bh % a.Hq;
    const char *orow = static_cast<const char *>(a.o) + (b * a.o_sb + h * a.o_sh) * 2 + i * a.o_ss;
    const char *drow = static_cast<const char *>(a.dout) + (b * a.do_sb + h * a.do_sh) * 2 + i * a.do_ss;
    const u32x4 ov = *reinterpret_cast<const u32x4 *>(orow + 16 * c);
    const u32x4 dv = *reinterpret_cast<const u32x4 *>(drow + 16 * c);
    typedef T t8 __attribute__((ext_vector_type(8)));
    const t8 o8 = __builtin_bit_cast(t8, ov), d8 = __builtin_bit_cast(t8, dv);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(static_cast<float>(o8[e]), static_cast<float>(d8[e]), s);
  }
  // the group's sum by DPP exchanges within the 16-lane row (no LDS permute)
  s += row16_xor<8>(s);
  s += row16_xor<4>(s);
  s += row16_xor<2>(s);
  s += row16_xor<1>(s);
  if (r < rows && c == 0) a.rowdot[r] = s;
}

// log2-domain LSE of a row; +inf for a row that sees no key, so its recomputed
// probabilities are exp2(-inf) = 0 rather than NaN
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == neg_inf() ? __builtin_inff() : lse * kLog2e;
}

// ---- dK, dV: a workgroup of 8 wavefronts owns 256 keys, a wavefront 32 ----
// (two wavefronts per SIMD).  The keys' K rows stay in registers as the B
// operand of S = Q K^T; their V rows are staged once in LDS (the register file
// holds K, dK^T and dV^T for two wavefronts per SIMD, not V as well) and read
// as the B operand of dP = dO V^T.  Query tiles are staged by all 512 threads,
// one 16-byte chunk each, double-buffered.
constexpr int kDkdvWaves = 8;
constexpr int kDkdvKeys = 32 * kDkdvWaves;
constexpr int kVRow = kBD + kEPC;  // V row in LDS, +16 bytes: 68 dwords, so 16 rows start on 16 bank quads

template <typename T, bool CAUSAL, bool PP>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2)))
void bwd_dkdv_kernel(const BwdArgs a) {
  using M = BwdMfma<T>;
  typedef typename M::frag frag;
  using Tl = Tile<512>;
  // two LDS stages: tile w is read from stage w & 1 while tile w + 1 is
  // written to the other one, so one barrier per tile suffices
  __shared__ __attribute__((aligned(256))) char sQ[2][kTileBytes];
  __shared__ __attribute__((aligned(256))) char sDO[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) float sL[2][kTR];   // log2-domain LSE of the tile's rows
  __shared__ __attribute__((aligned(16))) float sND[2][kTR];  // -Dr of the tile's rows
  __shared__ __attribute__((aligned(16))) T sV[kDkdvKeys * kVRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int kt = blockIdx.x / (a.B * a.Hkv);  // heaviest (earliest) key tiles first
  const int bh = blockIdx.x % (a.B * a.Hkv);
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int j0 = kt * kDkdvKeys;
  const int kw0 = j0 + 32 * wave;  // the wavefront's first key
  const int key = kw0 + l32;       // this lane's key (column of S, dP, dK^T, dV^T)
  const int coff = a.Sk - a.Sq;    // key j visible from row i iff j <= i + coff

  // K rows of this lane's key in registers (lane half h: elements 64 h .. 64 h + 63);
  // the workgroup's V rows into LDS, one 16-byte chunk per thread and pass
  frag kf[8];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const T *>(a.k) + b * a.k_sb + hk * a.k_sh, a.k_ext);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const T *>(a.v) + b * a.v_sb + hk * a.v_sh, a.v_ext);
    const bool ok = key < a.Sk;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      kf[c] = __builtin_bit_cast(frag, buf_load16(rk, ok ? key * a.k_ss + (64 * h + 8 * c) * 2 : kOOB));
#pragma unroll
    for (int p = 0; p < kDkdvKeys * kCH / 512; ++p) {
      const int idx = tid + 512 * p;
      const int r = idx / kCH, c = idx % kCH;
      const int kj = j0 + r;
      *reinterpret_cast<u32x4 *>(sV + r * kVRow + c * kEPC) = buf_load16(rv, kj < a.Sk ? kj * a.v_ss + c * 16 : kOOB);
    }
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dk[db] = dv[db] = f32x16{};

  // first query row that sees any key of this workgroup
  const int i_first = CAUSAL ? max(0, j0 - coff) : 0;
  const int t_first = i_first / kTR;
  const int n_qt = (a.Sq + kTR - 1) / kTR;

  // the work is the sequence of (query head of the group, query tile) items;
  // the staging pipeline runs straight through the head changes
  const int ntl = max(n_qt - t_first, 0);
  const int n_items = a.G * ntl;
  Tl tq, tdo;
  float l_st = 0.f, nd_st = 0.f;  // lse2 / -Dr of row tid of the staged tile (tid < kTR)
  // Items are loaded in order; the cursor keeps the loading item's head as
  // pointers (advanced when the head changes) and its tile index, so the
  // loop does no division or 64-bit address arithmetic per tile.
  const T *qh = static_cast<const T *>(a.q) + b * a.q_sb + static_cast<long long>(hk * a.G) * a.q_sh;
  const T *doh = static_cast<const T *>(a.dout) + b * a.do_sb + static_cast<long long>(hk * a.G) * a.do_sh;
  const float *lseh = a.lse + b * a.lse_sb + static_cast<long long>(hk * a.G) * a.lse_sh;
  const float *rdh = a.rowdot + (static_cast<long long>(b) * a.Hq + hk * a.G) * a.Sq;
  int lt = 0;  // tile of the next item to load
  auto load_next = [&]() {
    const int i0 = (t_first + lt) * kTR;
    tq.load(make_rsrc(qh, a.q_ext), a.q_ss, i0, a.Sq);
    tdo.load(make_rsrc(doh, a.do_ext), a.do_ss, i0, a.Sq);
    if (tid < kTR) {
      // rows past Sq: +inf LSE makes their probabilities exactly 0, so they
      // need no mask; their dO (and so dP and dS) is 0 as well
      const int i = i0 + tid;
      l_st = i < a.Sq ? lse2_of(lseh[i]) : __builtin_inff();
      nd_st = i < a.Sq ? -rdh[i] : 0.f;
    }
    if (++lt == ntl) {
      lt = 0;
      qh += a.q_sh;
      doh += a.do_sh;
      lseh += a.lse_sh;
      rdh += a.Sq;
    }
  };
  auto store_item = [&](int st) {
    tq.store(sQ[st]);
    tdo.store(sDO[st]);
    if (tid < kTR) {
      sL[st][tid] = l_st;
      sND[st][tid] = nd_st;
    }
  };
  if (n_items > 0) {
    load_next();
    store_item(0);
  }
  // K's fragments, V and tile 0 have landed: the loop's MFMAs then wait on
  // nothing but LDS, and the prefetch below stays in flight across a tile
  wait_vmem_all();
  if (n_items > 1) load_next();
  __syncthreads();

  const T *vrow = sV + (32 * wave + l32) * kVRow + 64 * h;  // B operand of dP: this lane's key
  const int arow = row_off(perm_row(l32)) + 128 * h;        // row operands: tile row perm_row(l32)
  const int trl = tr_lane(lane);
  const bool key_ok = kw0 + 32 <= a.Sk;  // wave-uniform
  // The three phases of query tile w: A forms S and dP - Dr (MFMA), B the
  // probabilities and dS (vector work), C dV^T += dO^T P and dK^T += Q^T dS
  // (MFMA).  Their results pass between phases in registers.
  f32x16 s, dp;
  frag pf[2], dsf[2];
  auto phase_a = [&](int w) {
    // S = Q K^T and dP - Dr = dO V^T - Dr, rows = queries (accumulator
    // order), columns = keys
    const int st = w & 1;
    const float *nd = sND[st] + 8 * h;
    const f32x4 n0 = *reinterpret_cast<const f32x4 *>(nd), n1 = *reinterpret_cast<const f32x4 *>(nd + 4);
    const f32x4 n2 = *reinterpret_cast<const f32x4 *>(nd + 16), n3 = *reinterpret_cast<const f32x4 *>(nd + 20);
    dp = f32x16{n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3],
                n2[0], n2[1], n2[2], n2[3], n3[0], n3[1], n3[2], n3[3]};
    s = f32x16{};
    const char *qr = sQ[st] + arow;
    const char *dr = sDO[st] + arow;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s = M::mma(lds_frag<T>(qr + 16 * c), kf[c], s);
      dp = M::mma(lds_frag<T>(dr + 16 * c), lds_frag<T>(reinterpret_cast<const char *>(vrow + 8 * c)), dp);
    }
  };
  int ct = 0;  // tile of the item phase B runs next (every wavefront runs B in item order)
  auto phase_b = [&](int w) {
    // P and dS, as B operands over query steps of 16
    const int st = w & 1;
    const int i0 = (t_first + ct) * kTR;
    ct = ct + 1 == ntl ? 0 : ct + 1;
    auto softmax_grad = [&](auto masked) {
      // masked tiles only: the lane's key taken afresh (see fresh_lane_id)
      const int mkey = decltype(masked)::value ? kw0 + (fresh_lane_id() & 31) : 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r0 = 16 * half + 8 * h;  // tile rows r0 .. r0 + 7 in registers 8 half ..
        const f32x4 l0 = *reinterpret_cast<const f32x4 *>(sL[st] + r0);
        const f32x4 l1 = *reinterpret_cast<const f32x4 *>(sL[st] + r0 + 4);
        unsigned pw[4], dw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float pv[2], dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 2 * e2 + u;
            const int ireg = 8 * half + e;
            const float l2 = e < 4 ? l0[e] : l1[e - 4];
            float p = fast_exp2(s[ireg] * a.c - l2);
            if constexpr (decltype(masked)::value) {
              bool vis = mkey < a.Sk;
              if (CAUSAL) vis = vis && mkey <= i0 + r0 + e + coff;
              p = vis ? p : 0.f;
            }
            pv[u] = p;
            dsv[u] = p * dp[ireg];
          }
          pw[e2] = pack2<T>(pv[0], pv[1]);
          dw[e2] = pack2<T>(dsv[0], dsv[1]);
        }
        pf[half] = __builtin_bit_cast(frag, u32x4{pw[0], pw[1], pw[2], pw[3]});
        dsf[half] = __builtin_bit_cast(frag, u32x4{dw[0], dw[1], dw[2], dw[3]});
      }
    };
    // the mask matters only on tiles that reach past the diagonal or Sk
    if (key_ok && (!CAUSAL || kw0 + 31 <= i0 + coff))
      softmax_grad(std::false_type{});
    else
      softmax_grad(std::true_type{});
  };
  auto phase_c = [&](int w) {
    // dV^T += dO^T P, dK^T += Q^T dS: rows = head dims, columns = keys
    const int st = w & 1;
    const char *dot = sDO[st] + trl;
    const char *qt = sQ[st] + trl;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dv[db] = M::mma(tr_frag<T>(dot, t, db), pf[t], dv[db]);
        dk[db] = M::mma(tr_frag<T>(qt, t, db), dsf[t], dk[db]);
      }
    }
  };
  // tile w + 1 into the stage tile w - 1 left; tile w + 2 into registers
  auto stage_next = [&](int w) {
    if (w + 1 < n_items) store_item((w + 1) & 1);
    if (w + 2 < n_items) load_next();
  };
  if constexpr (!PP) {
    for (int w = 0; w < n_items; ++w) {
      phase_a(w);
      phase_b(w);
      phase_c(w);
      stage_next(w);
      __syncthreads();
    }
  } else {
    // Wave-specialised schedule.  Round r has three slots, each ended by a
    // workgroup barrier.  Wavefronts 0-3 (one per SIMD) run A(r), B(r), C(r)
    // in them; wavefronts 4-7 run the same phases two slots later (B(r-1),
    // C(r-1), A(r)), so in the first two slots one wavefront of each SIMD
    // issues MFMAs while the other does vector work.  In the third slot every
    // thread stores tile r + 1 into the stage tile r - 1 left (its last
    // reader, C(r-1) of wavefronts 4-7, ended in slot two) and fetches tile
    // r + 2.  The roles run separate loops with the same barrier count, so
    // each keeps only its own phase results live.
    if (wave < kDkdvWaves / 2) {
      for (int r = 0; r < n_items; ++r) {
        phase_a(r);
        __syncthreads();
        phase_b(r);
        __syncthreads();
        phase_c(r);
        stage_next(r);
        __syncthreads();
      }
      // the other role's last round
      __syncthreads();
      __syncthreads();
      __syncthreads();
    } else {
      __syncthreads();
      __syncthreads();
      if (n_items > 0) {
        phase_a(0);
        stage_next(0);
      }
      __syncthreads();
      for (int r = 1; r <= n_items; ++r) {
        phase_b(r - 1);
        __syncthreads();
        phase_c(r - 1);
        __syncthreads();
        if (r < n_items) {
          phase_a(r);
          stage_next(r);
        }
        __syncthreads();
      }
    }
  }

  // ---- write dK = tau dK^T^T and dV: lane's key, dims 32 db + 8 m + 4 h .. +3
  // (the lane's key and half taken afresh: see fresh_lane_id) ----
  const int elane = fresh_lane_id();
  const int ekey = kw0 + (elane & 31), eh = elane >> 5;
  if (ekey < a.Sk) {
    char *dkrow = static_cast<char *>(a.dk) + (b * a.dk_sb + hk * a.dk_sh) * 2 + static_cast<long long>(ekey) * a.dk_ss;
    char *dvrow = static_cast<char *>(a.dv) + (b * a.dv_sb + hk * a.dv_sh) * 2 + static_cast<long long>(ekey) * a.dv_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = 32 * db + 8 * m + 4 * eh;
        *reinterpret_cast<u32x2 *>(dkrow + 2 * d0) =
            u32x2{pack2<T>(dk[db][4 * m] * a.scale, dk[db][4 * m + 1] * a.scale),
                  pack2<T>(dk[db][4 * m + 2] * a.scale, dk[db][4 * m + 3] * a.scale)};
        *reinterpret_cast<u32x2 *>(dvrow + 2 * d0) =
            u32x2{pack2<T>(dv[db][4 * m], dv[db][4 * m + 1]), pack2<T>(dv[db][4 * m + 2], dv[db][4 * m + 3])};
      }
  }
}

// ---- dQ: a workgroup owns 128 query rows, a wavefront 32; key tiles of 32 ----
template <typename T, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(const BwdArgs a) {
  using M = BwdMfma<T>;
  typedef typename M::frag frag;
  using Tl = Tile<256>;
  __shared__ __attribute__((aligned(256))) char sK[2][kTileBytes];
  __shared__ __attribute__((aligned(256))) char sV[2][kTileBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int nq = (a.Sq + 127) / 128;
  const int qt = nq - 1 - static_cast<int>(blockIdx.x) / (a.B * a.Hq);  // heaviest (last) rows first
  const int bh = blockIdx.x % (a.B * a.Hq);
  const int b = bh / a.Hq, hq = bh % a.Hq, hk = hq / a.G;
  const int i0 = qt * 128;
  const int rw0 = i0 + 32 * wave;  // the wavefront's first query row
  const int row = rw0 + l32;       // this lane's query row
  const int coff = a.Sk - a.Sq;

  frag qf[8], df[8];
  float l2 = __builtin_inff(), dd = 0.f;  // rows past Sq: +inf LSE, so P = 0 without a mask
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const T *>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_ext);
    const __amdgpu_buffer_rsrc_t rdo =
        make_rsrc(static_cast<const T *>(a.dout) + b * a.do_sb + hq * a.do_sh, a.do_ext);
    const bool ok = row < a.Sq;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      qf[c] = __builtin_bit_cast(frag, buf_load16(rq, ok ? row * a.q_ss + (64 * h + 8 * c) * 2 : kOOB));
      df[c] = __builtin_bit_cast(frag, buf_load16(rdo, ok ? row * a.do_ss + (64 * h + 8 * c) * 2 : kOOB));
    }
    if (ok) {
      l2 = lse2_of(a.lse[b * a.lse_sb + hq * a.lse_sh + row]);
      dd = a.rowdot[(static_cast<long long>(b) * a.Hq + hq) * a.Sq + row];
    }
  }
  // dP^T's accumulator starts at -Dr of the lane's row (its column), kept in
  // registers of its own for the whole loop
  f32x16 ndd;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndd[i] = -dd;
  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

  int n_kt = (a.Sk + kTR - 1) / kTR;
  if (CAUSAL) {
    const int last = min(i0 + 127, a.Sq - 1) + coff;  // last key any row of the workgroup sees
    n_kt = min(n_kt, last < 0 ? 0 : last / kTR + 1);
  }
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const T *>(a.k) + b * a.k_sb + hk * a.k_sh, a.k_ext);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const T *>(a.v) + b * a.v_sb + hk * a.v_sh, a.v_ext);
  Tl tk, tv;
  if (n_kt > 0) {
    tk.load(rk, a.k_ss, 0, a.Sk);
    tv.load(rv, a.v_ss, 0, a.Sk);
    tk.store(sK[0]);
    tv.store(sV[0]);
  }
  if (n_kt > 1) {
    tk.load(rk, a.k_ss, kTR, a.Sk);
    tv.load(rv, a.v_ss, kTR, a.Sk);
  }
  __syncthreads();
  const int arow = row_off(perm_row(l32)) + 128 * h;  // row operands: tile row perm_row(l32)
  const int trl = tr_lane(lane);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int j0 = kt * kTR;
    const int st = kt & 1;
    // S^T = K Q^T and dP^T - Dr = V dO^T - Dr: rows = keys (accumulator
    // order), columns = query rows
    f32x16 s = f32x16{}, dp = ndd;
    const char *kr = sK[st] + arow;
    const char *vr = sV[st] + arow;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s = M::mma(lds_frag<T>(kr + 16 * c), qf[c], s);
      dp = M::mma(lds_frag<T>(vr + 16 * c), df[c], dp);
    }
    frag dsf[2];
    auto softmax_grad = [&](auto masked) {
      // masked tiles only: the lane's row and half taken afresh (see fresh_lane_id)
      const int ml = decltype(masked)::value ? fresh_lane_id() : 0;
      const int mrow = rw0 + (ml & 31), mh = ml >> 5;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        unsigned dw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int ireg = 8 * half + 2 * e2 + u;
            float p = fast_exp2(s[ireg] * a.c - l2);
            if constexpr (decltype(masked)::value) {
              const int kj = j0 + acc_row(0, ireg, mh);
              bool vis = kj < a.Sk;
              if (CAUSAL) vis = vis && kj <= mrow + coff;
              p = vis ? p : 0.f;
            }
            dsv[u] = p * dp[ireg];
          }
          dw[e2] = pack2<T>(dsv[0], dsv[1]);
        }
        dsf[half] = __builtin_bit_cast(frag, u32x4{dw[0], dw[1], dw[2], dw[3]});
      }
    };
    // the mask matters only on tiles that reach past the diagonal or Sk
    if (j0 + kTR <= a.Sk && (!CAUSAL || j0 + kTR - 1 <= rw0 + coff))
      softmax_grad(std::false_type{});
    else
      softmax_grad(std::true_type{});
    // dQ^T += K^T dS^T: rows = head dims, columns = query rows
    const char *ktp = sK[st] + trl;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) dq[db] = M::mma(tr_frag<T>(ktp, t, db), dsf[t], dq[db]);
    if (kt + 1 < n_kt) {  // that stage was last read by tile kt - 1
      tk.store(sK[st ^ 1]);
      tv.store(sV[st ^ 1]);
    }
    if (kt + 2 < n_kt) {
      tk.load(rk, a.k_ss, j0 + 2 * kTR, a.Sk);
      tv.load(rv, a.v_ss, j0 + 2 * kTR, a.Sk);
    }
    __syncthreads();
  }

  // the lane's row and half taken afresh (see fresh_lane_id)
  const int elane = fresh_lane_id();
  const int erow = rw0 + (elane & 31), eh = elane >> 5;
  if (erow < a.Sq) {
    char *dqrow = static_cast<char *>(a.dq) + (b * a.dq_sb + hq * a.dq_sh) * 2 + static_cast<long long>(erow) * a.dq_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = 32 * db + 8 * m + 4 * eh;
        *reinterpret_cast<u32x2 *>(dqrow + 2 * d0) =
            u32x2{pack2<T>(dq[db][4 * m] * a.scale, dq[db][4 * m + 1] * a.scale),
                  pack2<T>(dq[db][4 * m + 2] * a.scale, dq[db][4 * m + 3] * a.scale)};
      }
  }
}

template <typename T>
int launch_bwd_typed(const BwdArgs &a, bool causal, bool pingpong, hipStream_t s) {
  const long long rows = static_cast<long long>(a.B) * a.Hq * a.Sq;
  const char *dt = std::is_same<T, __bf16>::value ? "bf16" : "f16";
  if (rows > 0) {
    fa_log_launch("bwd_rowdot_kernel", static_cast<unsigned>((rows + 15) / 16), 256, 0, "dtype=%s rows=%lld", dt, rows);
    hipLaunchKernelGGL(bwd_rowdot_kernel<T>, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, s, a);
  }
  const unsigned g_kv = static_cast<unsigned>((a.Sk + kDkdvKeys - 1) / kDkdvKeys) * a.B * a.Hkv;
  const unsigned g_q = static_cast<unsigned>((a.Sq + 127) / 128) * a.B * a.Hq;
  if (g_kv)
    fa_log_launch("bwd_dkdv_kernel", g_kv, 512, 0, "dtype=%s causal=%d B=%d Hq=%d Hkv=%d Sq=%d Sk=%d pingpong=%d",
                  dt, causal ? 1 : 0, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, pingpong ? 1 : 0);
  if (g_q)
    fa_log_launch("bwd_dq_kernel", g_q, 256, 0, "dtype=%s causal=%d B=%d Hq=%d Hkv=%d Sq=%d Sk=%d", dt,
                  causal ? 1 : 0, a.B, a.Hq, a.Hkv, a.Sq, a.Sk);
  if (g_kv) {
    if (causal) {
      if (pingpong)
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, true, true>), dim3(g_kv), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, true, false>), dim3(g_kv), dim3(512), 0, s, a);
    } else {
      if (pingpong)
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, false, true>), dim3(g_kv), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, false, false>), dim3(g_kv), dim3(512), 0, s, a);
    }
  }
  if (g_q) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<T, true>), dim3(g_q), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, false>), dim3(g_q), dim3(256), 0, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace fa

int fa_launch_bwd(const fa_bwd_params *p, void *stream) {
  using namespace fa;
  BwdArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.o = p->o;
  a.dout = p->dout;
  a.lse = p->lse;
  a.dq = p->dq;
  a.dk = p->dk;
  a.dv = p->dv;
  a.rowdot = static_cast<float *>(p->workspace);
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = p->Hq / p->Hkv;
  a.Sq = p->Sq;
  a.Sk = p->Sk;
  a.q_sb = p->q_strides[0];
  a.q_sh = p->q_strides[1];
  a.k_sb = p->k_strides[0];
  a.k_sh = p->k_strides[1];
  a.v_sb = p->v_strides[0];
  a.v_sh = p->v_strides[1];
  a.o_sb = p->o_strides[0];
  a.o_sh = p->o_strides[1];
  a.do_sb = p->do_strides[0];
  a.do_sh = p->do_strides[1];
  a.dq_sb = p->dq_strides[0];
  a.dq_sh = p->dq_strides[1];
  a.dk_sb = p->dk_strides[0];
  a.dk_sh = p->dk_strides[1];
  a.dv_sb = p->dv_strides[0];
  a.dv_sh = p->dv_strides[1];
  a.lse_sb = p->lse_strides[0];
  a.lse_sh = p->lse_strides[1];
  a.q_ss = static_cast<unsigned>(p->q_strides[2] * 2);
  a.k_ss = static_cast<unsigned>(p->k_strides[2] * 2);
  a.v_ss = static_cast<unsigned>(p->v_strides[2] * 2);
  a.o_ss = static_cast<unsigned>(p->o_strides[2] * 2);
  a.do_ss = static_cast<unsigned>(p->do_strides[2] * 2);
  a.dq_ss = static_cast<unsigned>(p->dq_strides[2] * 2);
  a.dk_ss = static_cast<unsigned>(p->dk_strides[2] * 2);
  a.dv_ss = static_cast<unsigned>(p->dv_strides[2] * 2);
  auto ext = [](int rows, long long ss_elems) {
    return rows > 0 ? static_cast<unsigned>(((static_cast<long long>(rows) - 1) * ss_elems + kBD) * 2) : 0u;
  };
  a.q_ext = ext(p->Sq, p->q_strides[2]);
  a.o_ext = ext(p->Sq, p->o_strides[2]);
  a.do_ext = ext(p->Sq, p->do_strides[2]);
  a.k_ext = ext(p->Sk, p->k_strides[2]);
  a.v_ext = ext(p->Sk, p->v_strides[2]);
  a.scale = p->softmax_scale;
  a.c = p->softmax_scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == FA_BF16) return launch_bwd_typed<__bf16>(a, p->causal != 0, p->wave_pingpong != 0, s);
  return launch_bwd_typed<_Float16>(a, p->causal != 0, p->wave_pingpong != 0, s);
}
