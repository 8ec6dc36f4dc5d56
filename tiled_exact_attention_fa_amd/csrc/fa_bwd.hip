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
//     wavefront 32 of them (8 wavefronts, two per SIMD); it walks every query head of the group and every
//     query tile that can see its keys, and keeps dK^T and dV^T of its keys in
//     registers until the end.  Per tile: S = Q K^T and dP = dO V^T with the
//     keys' K rows in registers and V rows in LDS as the B operands, then
//     dV^T += dO^T P and dK^T += Q^T dS with the probabilities fed from the
//     S accumulators straight into the B operand (the query tile is written
//     to LDS with bits 2 and 3 of the row index swapped, which puts the
//     accumulator registers in the operand's order).  The query tile is staged
//     twice, row-major for the first products and transposed for the second.
//   * bwd_dq_kernel: a workgroup owns 128 query rows of one (batch, head), a
//     wavefront 32 (two wavefronts per SIMD); per 32-key tile S^T = K Q^T and dP^T = V dO^T with the rows'
//     Q and dO in registers, then dQ^T += K^T dS^T, K staged both row-major
//     (permuted rows) and transposed.
//   * Both tile loops stage through two LDS buffers with register prefetch two
//     tiles ahead: one barrier per tile.
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
constexpr int kRow = kBD + kEPC;  // row-major tile row in LDS, +16 bytes

// LDS row holding tile row r: bits 2 and 3 swapped, so that accumulator
// register i of lane half h of 32-row block mb holds tile row
// 32 mb + 16 (i / 8) + 8 h + i % 8 — the order the B operand needs.
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ int acc_row(int mb, int i, int h) { return 32 * mb + 16 * (i >> 3) + 8 * h + (i & 7); }

// A tile of R rows x 128 elements, loaded by NT threads: thread (g, c) holds
// rows g * RPT .. g * RPT + RPT - 1 of chunk c, which it can write both
// row-major (one 16-byte store per row) and transposed (RPT elements of each of
// its 8 columns).
template <typename T, int R, int NT = 256> struct Tile {
  static constexpr int RPT = R * kCH / NT;   // rows per thread
  static constexpr int NG = R / RPT;         // row groups
  static constexpr int TROW = R + kEPC;      // transposed row in LDS (+16 bytes)
  u32x4 r[RPT];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, unsigned ss, int row0, int nrows) {
    const int g = threadIdx.x % NG, c = threadIdx.x / NG;
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
      const int rr = row0 + g * RPT + p;
      r[p] = buf_load16(rs, rr < nrows ? static_cast<unsigned>(rr) * ss + c * 16u : kOOB);
    }
  }
  __device__ __forceinline__ void store_rows(T *dst) const {
    const int g = threadIdx.x % NG, c = threadIdx.x / NG;
#pragma unroll
    for (int p = 0; p < RPT; ++p)
      *reinterpret_cast<u32x4 *>(dst + perm_row(g * RPT + p) * kRow + c * kEPC) = r[p];
  }
  __device__ __forceinline__ void store_transposed(T *dst) const {
    const int g = threadIdx.x % NG, c = threadIdx.x / NG;
#pragma unroll
    for (int e = 0; e < kEPC; ++e) {
      unsigned short col[RPT];
#pragma unroll
      for (int p = 0; p < RPT; ++p) {
        const u32x4 w = r[p];
        const unsigned word = w[e >> 1];
        col[p] = static_cast<unsigned short>((e & 1) ? (word >> 16) : (word & 0xFFFFu));
      }
      unsigned short *d = reinterpret_cast<unsigned short *>(dst + (c * kEPC + e) * TROW + g * RPT);
      if constexpr (RPT == 4) {
        *reinterpret_cast<u32x2 *>(d) = u32x2{col[0] | (static_cast<unsigned>(col[1]) << 16),
                                              col[2] | (static_cast<unsigned>(col[3]) << 16)};
      } else if constexpr (RPT == 2) {
        *reinterpret_cast<unsigned *>(d) = col[0] | (static_cast<unsigned>(col[1]) << 16);
      } else {
        static_assert(RPT == 1, "tile rows per thread");
        *d = col[0];
      }
    }
  }
};

// Row r of a 32x32 accumulator block as a 16-byte MFMA fragment from LDS.
template <typename T> __device__ __forceinline__ typename BwdMfma<T>::frag lds_frag(const T *p) {
  return __builtin_bit_cast(typename BwdMfma<T>::frag, *reinterpret_cast<const u32x4 *>(p));
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
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
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

template <typename T, bool CAUSAL, int BR>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2)))
void bwd_dkdv_kernel(const BwdArgs a) {
  using M = BwdMfma<T>;
  typedef typename M::frag frag;
  using Tl = Tile<T, BR, 512>;
  constexpr int MB = BR / 32;
  // two LDS stages: tile w is read from stage w & 1 while tile w + 1 is
  // written to the other one, so one barrier per tile suffices
  __shared__ __attribute__((aligned(16))) T sQ[2][BR * kRow];
  __shared__ __attribute__((aligned(16))) T sDO[2][BR * kRow];
  __shared__ __attribute__((aligned(16))) T sQt[2][kBD * Tl::TROW];
  __shared__ __attribute__((aligned(16))) T sDOt[2][kBD * Tl::TROW];
  __shared__ __attribute__((aligned(16))) float sL[2][BR];
  __shared__ __attribute__((aligned(16))) float sD[2][BR];
  __shared__ __attribute__((aligned(16))) T sV[kDkdvKeys * kRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int kt = blockIdx.x / (a.B * a.Hkv);  // heaviest (earliest) key tiles first
  const int bh = blockIdx.x % (a.B * a.Hkv);
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int j0 = kt * kDkdvKeys;
  const int key = j0 + 32 * wave + l32;  // this lane's key (column of S, dP, dK^T, dV^T)
  const int coff = a.Sk - a.Sq;          // key j visible from row i iff j <= i + coff

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
      *reinterpret_cast<u32x4 *>(sV + r * kRow + c * kEPC) = buf_load16(rv, kj < a.Sk ? kj * a.v_ss + c * 16 : kOOB);
    }
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dk[db] = dv[db] = f32x16{};

  // first query row that sees any key of this workgroup
  const int i_first = CAUSAL ? max(0, j0 - coff) : 0;
  const int t_first = i_first / BR;
  const int n_qt = (a.Sq + BR - 1) / BR;

  // the work is the sequence of (query head of the group, query tile) items;
  // the staging pipeline runs straight through the head changes
  const int ntl = max(n_qt - t_first, 0);
  const int n_items = a.G * ntl;
  Tl tq, tdo;
  float l_st = 0.f, d_st = 0.f;  // lse2 / row term of row tid of the staged tile (tid < BR)
  auto load_item = [&](int w) {
    const int hq = hk * a.G + w / ntl;
    const int i0 = (t_first + w % ntl) * BR;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const T *>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_ext);
    const __amdgpu_buffer_rsrc_t rdo =
        make_rsrc(static_cast<const T *>(a.dout) + b * a.do_sb + hq * a.do_sh, a.do_ext);
    tq.load(rq, a.q_ss, i0, a.Sq);
    tdo.load(rdo, a.do_ss, i0, a.Sq);
    if (tid < BR) {
      const int i = i0 + tid;
      l_st = i < a.Sq ? lse2_of(a.lse[b * a.lse_sb + hq * a.lse_sh + i]) : __builtin_inff();
      d_st = i < a.Sq ? a.rowdot[(static_cast<long long>(b) * a.Hq + hq) * a.Sq + i] : 0.f;
    }
  };
  auto store_item = [&](int st) {
    tq.store_rows(sQ[st]);
    tq.store_transposed(sQt[st]);
    tdo.store_rows(sDO[st]);
    tdo.store_transposed(sDOt[st]);
    if (tid < BR) {
      sL[st][tid] = l_st;
      sD[st][tid] = d_st;
    }
  };
  if (n_items > 0) {
    load_item(0);
    store_item(0);
  }
  if (n_items > 1) load_item(1);
  __syncthreads();

  const T *vrow = sV + (32 * wave + l32) * kRow + 64 * h;  // B operand of dP: this lane's key
  for (int w = 0; w < n_items; ++w) {
    const int st = w & 1;
    const int i0 = (t_first + w % ntl) * BR;
    {
      // S = Q K^T and dP = dO V^T, rows = queries (permuted), columns = keys
      f32x16 s[MB], dp[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb] = dp[mb] = f32x16{};
        const T *qr = sQ[st] + (32 * mb + l32) * kRow + 64 * h;
        const T *dr = sDO[st] + (32 * mb + l32) * kRow + 64 * h;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          s[mb] = M::mma(lds_frag<T>(qr + 8 * c), kf[c], s[mb]);
          dp[mb] = M::mma(lds_frag<T>(dr + 8 * c), lds_frag<T>(vrow + 8 * c), dp[mb]);
        }
      }
      // P and dS, as B operands over query steps of 16
      frag pf[BR / 16], dsf[BR / 16];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int r0 = 32 * mb + 16 * half + 8 * h;  // tile rows r0 .. r0 + 7 in registers 8 half ..
          const f32x4 l0 = *reinterpret_cast<const f32x4 *>(sL[st] + r0);
          const f32x4 l1 = *reinterpret_cast<const f32x4 *>(sL[st] + r0 + 4);
          const f32x4 d0 = *reinterpret_cast<const f32x4 *>(sD[st] + r0);
          const f32x4 d1 = *reinterpret_cast<const f32x4 *>(sD[st] + r0 + 4);
          unsigned pw[4], dw[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            float pv[2], dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int e = 2 * e2 + u;
              const int ireg = 8 * half + e;
              const int qi = i0 + r0 + e;
              const float l2 = e < 4 ? l0[e] : l1[e - 4];
              const float dd = e < 4 ? d0[e] : d1[e - 4];
              bool vis = qi < a.Sq && key < a.Sk;
              if (CAUSAL) vis = vis && key <= qi + coff;
              const float p = vis ? fast_exp2(s[mb][ireg] * a.c - l2) : 0.f;
              pv[u] = p;
              dsv[u] = p * (dp[mb][ireg] - dd);
            }
            pw[e2] = pack2<T>(pv[0], pv[1]);
            dw[e2] = pack2<T>(dsv[0], dsv[1]);
          }
          pf[2 * mb + half] = __builtin_bit_cast(frag, u32x4{pw[0], pw[1], pw[2], pw[3]});
          dsf[2 * mb + half] = __builtin_bit_cast(frag, u32x4{dw[0], dw[1], dw[2], dw[3]});
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS: rows = head dims, columns = keys
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const T *dot = sDOt[st] + (32 * db + l32) * Tl::TROW + 8 * h;
        const T *qtp = sQt[st] + (32 * db + l32) * Tl::TROW + 8 * h;
#pragma unroll
        for (int t = 0; t < BR / 16; ++t) {
          dv[db] = M::mma(lds_frag<T>(dot + 16 * t), pf[t], dv[db]);
          dk[db] = M::mma(lds_frag<T>(qtp + 16 * t), dsf[t], dk[db]);
        }
      }
    }
    if (w + 1 < n_items) store_item(st ^ 1);  // that stage was last read by tile w - 1
    if (w + 2 < n_items) load_item(w + 2);
    __syncthreads();
  }

  // ---- write dK = tau dK^T^T and dV: lane's key, dims 32 db + 8 m + 4 h .. +3 ----
  if (key < a.Sk) {
    char *dkrow = static_cast<char *>(a.dk) + (b * a.dk_sb + hk * a.dk_sh) * 2 + static_cast<long long>(key) * a.dk_ss;
    char *dvrow = static_cast<char *>(a.dv) + (b * a.dv_sb + hk * a.dv_sh) * 2 + static_cast<long long>(key) * a.dv_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = 32 * db + 8 * m + 4 * h;
        *reinterpret_cast<u32x2 *>(dkrow + 2 * d0) =
            u32x2{pack2<T>(dk[db][4 * m] * a.scale, dk[db][4 * m + 1] * a.scale),
                  pack2<T>(dk[db][4 * m + 2] * a.scale, dk[db][4 * m + 3] * a.scale)};
        *reinterpret_cast<u32x2 *>(dvrow + 2 * d0) =
            u32x2{pack2<T>(dv[db][4 * m], dv[db][4 * m + 1]), pack2<T>(dv[db][4 * m + 2], dv[db][4 * m + 3])};
      }
  }
}

// ---- dQ: a workgroup owns 128 query rows, a wavefront 32; key tiles of 64 ----
template <typename T, bool CAUSAL, int BC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(const BwdArgs a) {
  using M = BwdMfma<T>;
  typedef typename M::frag frag;
  using Tl = Tile<T, BC>;
  __shared__ __attribute__((aligned(16))) T sK[2][BC * kRow];
  __shared__ __attribute__((aligned(16))) T sV[2][BC * kRow];
  __shared__ __attribute__((aligned(16))) T sKt[2][kBD * Tl::TROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int nq = (a.Sq + 127) / 128;
  const int qt = nq - 1 - static_cast<int>(blockIdx.x) / (a.B * a.Hq);  // heaviest (last) rows first
  const int bh = blockIdx.x % (a.B * a.Hq);
  const int b = bh / a.Hq, hq = bh % a.Hq, hk = hq / a.G;
  const int i0 = qt * 128;
  const int row = i0 + 32 * wave + l32;  // this lane's query row
  const int coff = a.Sk - a.Sq;

  frag qf[8], df[8];
  float l2 = __builtin_inff(), dd = 0.f;
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
  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

  int n_kt = (a.Sk + BC - 1) / BC;
  if (CAUSAL) {
    const int last = min(i0 + 127, a.Sq - 1) + coff;  // last key any row of the workgroup sees
    n_kt = min(n_kt, last < 0 ? 0 : last / BC + 1);
  }
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const T *>(a.k) + b * a.k_sb + hk * a.k_sh, a.k_ext);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const T *>(a.v) + b * a.v_sb + hk * a.v_sh, a.v_ext);
  Tl tk, tv;
  auto store_tile = [&](int st) {
    tk.store_rows(sK[st]);
    tk.store_transposed(sKt[st]);
    tv.store_rows(sV[st]);
  };
  if (n_kt > 0) {
    tk.load(rk, a.k_ss, 0, a.Sk);
    tv.load(rv, a.v_ss, 0, a.Sk);
    store_tile(0);
  }
  if (n_kt > 1) {
    tk.load(rk, a.k_ss, BC, a.Sk);
    tv.load(rv, a.v_ss, BC, a.Sk);
  }
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int j0 = kt * BC;
    const int st = kt & 1;
    // S^T = K Q^T and dP^T = V dO^T: rows = keys (permuted), columns = query rows
    constexpr int MB = BC / 32;
    f32x16 s[MB], dp[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s[mb] = dp[mb] = f32x16{};
      const T *kr = sK[st] + (32 * mb + l32) * kRow + 64 * h;
      const T *vr = sV[st] + (32 * mb + l32) * kRow + 64 * h;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        s[mb] = M::mma(lds_frag<T>(kr + 8 * c), qf[c], s[mb]);
        dp[mb] = M::mma(lds_frag<T>(vr + 8 * c), df[c], dp[mb]);
      }
    }
    frag dsf[BC / 16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        unsigned dw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 2 * e2 + u, ireg = 8 * half + e;
            const int kj = j0 + acc_row(mb, ireg, h);
            bool vis = row < a.Sq && kj < a.Sk;
            if (CAUSAL) vis = vis && kj <= row + coff;
            const float p = vis ? fast_exp2(s[mb][ireg] * a.c - l2) : 0.f;
            dsv[u] = p * (dp[mb][ireg] - dd);
          }
          dw[e2] = pack2<T>(dsv[0], dsv[1]);
        }
        dsf[2 * mb + half] = __builtin_bit_cast(frag, u32x4{dw[0], dw[1], dw[2], dw[3]});
      }
    // dQ^T += K^T dS^T: rows = head dims, columns = query rows
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const T *ktp = sKt[st] + (32 * db + l32) * Tl::TROW + 8 * h;
#pragma unroll
      for (int t = 0; t < BC / 16; ++t) dq[db] = M::mma(lds_frag<T>(ktp + 16 * t), dsf[t], dq[db]);
    }
    if (kt + 1 < n_kt) store_tile(st ^ 1);  // that stage was last read by tile kt - 1
    if (kt + 2 < n_kt) {
      tk.load(rk, a.k_ss, j0 + 2 * BC, a.Sk);
      tv.load(rv, a.v_ss, j0 + 2 * BC, a.Sk);
    }
    __syncthreads();
  }

  if (row < a.Sq) {
    char *dqrow = static_cast<char *>(a.dq) + (b * a.dq_sb + hq * a.dq_sh) * 2 + static_cast<long long>(row) * a.dq_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = 32 * db + 8 * m + 4 * h;
        *reinterpret_cast<u32x2 *>(dqrow + 2 * d0) =
            u32x2{pack2<T>(dq[db][4 * m] * a.scale, dq[db][4 * m + 1] * a.scale),
                  pack2<T>(dq[db][4 * m + 2] * a.scale, dq[db][4 * m + 3] * a.scale)};
      }
  }
}

template <typename T>
int launch_bwd_typed(const BwdArgs &a, bool causal, hipStream_t s) {
  const long long rows = static_cast<long long>(a.B) * a.Hq * a.Sq;
  const char *dt = std::is_same<T, __bf16>::value ? "bf16" : "f16";
  if (rows > 0) {
    fa_log_launch("bwd_rowdot_kernel", static_cast<unsigned>((rows + 15) / 16), 256, 0, "dtype=%s rows=%lld", dt, rows);
    hipLaunchKernelGGL(bwd_rowdot_kernel<T>, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, s, a);
  }
  const unsigned g_kv = static_cast<unsigned>((a.Sk + kDkdvKeys - 1) / kDkdvKeys) * a.B * a.Hkv;
  const unsigned g_q = static_cast<unsigned>((a.Sq + 127) / 128) * a.B * a.Hq;
  constexpr int BR = 32, BC = 32;  // query rows per dK/dV tile, keys per dQ tile
  if (g_kv)
    fa_log_launch("bwd_dkdv_kernel", g_kv, 512, 0, "dtype=%s causal=%d B=%d Hq=%d Hkv=%d Sq=%d Sk=%d", dt,
                  causal ? 1 : 0, a.B, a.Hq, a.Hkv, a.Sq, a.Sk);
  if (g_q)
    fa_log_launch("bwd_dq_kernel", g_q, 256, 0, "dtype=%s causal=%d B=%d Hq=%d Hkv=%d Sq=%d Sk=%d", dt,
                  causal ? 1 : 0, a.B, a.Hq, a.Hkv, a.Sq, a.Sk);
  if (causal) {
    if (g_kv) hipLaunchKernelGGL((bwd_dkdv_kernel<T, true, BR>), dim3(g_kv), dim3(512), 0, s, a);
    if (g_q) hipLaunchKernelGGL((bwd_dq_kernel<T, true, BC>), dim3(g_q), dim3(256), 0, s, a);
  } else {
    if (g_kv) hipLaunchKernelGGL((bwd_dkdv_kernel<T, false, BR>), dim3(g_kv), dim3(512), 0, s, a);
    if (g_q) hipLaunchKernelGGL((bwd_dq_kernel<T, false, BC>), dim3(g_q), dim3(256), 0, s, a);
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
  if (p->dtype == FA_BF16) return launch_bwd_typed<__bf16>(a, p->causal != 0, s);
  return launch_bwd_typed<_Float16>(a, p->causal != 0, s);
}
