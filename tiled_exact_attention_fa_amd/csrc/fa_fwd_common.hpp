// Kernel arguments and workgroup scheduling shared by the prefill kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_internal.h"

namespace fa {

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int B, Hq, G, Sq, Sk, nq;
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh;  // element strides
  long long o_sb, o_sh, o_ss;
  long long lse_sb, lse_sh;
  unsigned q_ss, k_ss, v_ss;     // row strides in bytes (below 2^31 after validation)
  unsigned q_ext, k_ext, v_ext;  // bytes spanned by one (batch, head) slice
  float c;                       // softmax scale * log2(e) [* q and k descale]
  float o_mul;                   // output multiplier (v descale for fp8, else 1)
};

// blockIdx -> (batch*head, query tile).  Workgroups are handed to the 8 XCDs
// round-robin (XCD = blockIdx % 8).  When the (batch, head) count divides by 8,
// each XCD gets a contiguous range of (batch, head) pairs (consecutive query
// heads share one K/V head under GQA), so every K/V stream is read through one
// XCD's L2.  Within an XCD:
//   * causal (tiles of unequal length): longest tiles first, so the short
//     tiles fill the tail of the launch.  When a head has at most 8 query
//     tiles, the range is cut into groups of heads (a multiple of G heads;
//     they are whole GQA groups, the query heads of one K/V head kept
//     together, when the heads per XCD are a multiple of G, as in every
//     benchmarked shape; otherwise the XCD's range starts inside a GQA group
//     and the groups straddle K/V heads, which costs locality, not
//     correctness) whose tiles together about
//     fill the XCD's 32 compute units once, and each group is issued longest
//     first across its heads: a compute unit that drew a long tile then draws
//     a short one, so the pairs even out as under one order over the whole
//     range, while the K/V read at any one time is one group's.  Measured, that
//     cut the fetched bytes of B=4 H=16 S=2048 by 18 % and ran B=8 at that
//     length 5 % faster; with 16 or more tiles per head it ran 2 % slower, so
//     longer heads keep one longest-first order over the whole range;
//   * non-causal (equal tiles): head by head, so the workgroups resident at
//     any time read the K/V of only one or two heads, which stay in L2.
__device__ __forceinline__ void map_block(int bid, int nq, int nbh, int G, bool longest_first, int &bh, int &qt) {
  int base = 0, per = nbh, slot = bid;
  if ((nbh & 7) == 0) {
    per = nbh >> 3;
    base = (bid & 7) * per;
    slot = bid >> 3;
  }
  if (longest_first) {
    constexpr int kCusPerXcd = 32;
    int hg = per;  // heads per group
    if ((nbh & 7) == 0 && nq <= 8) hg = min(per, (kCusPerXcd / nq + G - 1) / G * G);
    const int grp = slot / (hg * nq), within = slot % (hg * nq);
    const int nh = min(hg, per - grp * hg);  // the last group may hold fewer heads
    bh = base + grp * hg + within % nh;
    qt = nq - 1 - within / nh;
  } else {
    bh = base + slot / nq;
    qt = slot % nq;
  }
}

inline unsigned slice_bytes(int rows, long long ss, int d, int es) {
  if (rows <= 0) return 0;
  return static_cast<unsigned>((static_cast<long long>(rows - 1) * ss + d) * es);
}

inline FwdArgs make_fwd_args(const fa_fwd_params *p, int br, int es) {
  FwdArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.o = p->o;
  a.lse = p->lse;
  a.B = p->B;
  a.Hq = p->Hq;
  a.G = p->Hq / p->Hkv;
  a.Sq = p->Sq;
  a.Sk = p->Sk;
  a.nq = (p->Sq + br - 1) / br;
  a.q_sb = p->q_strides[0];
  a.q_sh = p->q_strides[1];
  a.k_sb = p->k_strides[0];
  a.k_sh = p->k_strides[1];
  a.v_sb = p->v_strides[0];
  a.v_sh = p->v_strides[1];
  a.o_sb = p->o_strides[0];
  a.o_sh = p->o_strides[1];
  a.o_ss = p->o_strides[2];
  a.lse_sb = p->lse_strides[0];
  a.lse_sh = p->lse_strides[1];
  // a one-row tensor gets the virtual stride d: any row past the first then
  // starts at or beyond the slice end and reads as zero
  a.q_ss = static_cast<unsigned>((p->Sq > 1 ? p->q_strides[2] : p->d) * es);
  a.k_ss = static_cast<unsigned>((p->Sk > 1 ? p->k_strides[2] : p->d) * es);
  a.v_ss = static_cast<unsigned>((p->Sk > 1 ? p->v_strides[2] : p->d) * es);
  a.q_ext = slice_bytes(p->Sq, p->q_strides[2], p->d, es);
  a.k_ext = slice_bytes(p->Sk, p->k_strides[2], p->d, es);
  a.v_ext = slice_bytes(p->Sk, p->v_strides[2], p->d, es);
  a.c = p->softmax_scale * 1.4426950408889634f;
  a.o_mul = 1.f;
  if (p->in_dtype == FA_FP8_E4M3) {
    a.c *= p->q_descale * p->k_descale;
    a.o_mul = p->v_descale;
  }
  return a;
}

}  // namespace fa
