// One-token decode over an int8 or fp8-e4m3 KV cache with per-token-per-head
// fp16 scales, split over the cache length and merged by log-sum-exp, with an
// optional residual window of recent bf16 tokens.
//
// What is computed (KV-cache quantisation overview, section 1 "decode step" and
// section 3 "read path" and "residual window"; FlashAttention interview canvas,
// panel 1 "online softmax key state"): for each sequence b and query head h,
// the new query attends to the first seq_len[b] cached tokens of cache head
// h / G, whose keys and values are code * scale, together with the first
// recent_len[b] tokens of the bf16 window.  Decode reads every cached byte once
// per step and so is bound by HBM bandwidth (same overview, section 2).
//
// MI355X design.
//   * Kernel 1 (decode_split_kernel): one workgroup per (batch, cache head,
//     split).  All G query heads that share the cache head are served by the
//     same pass over the chunk, so every K/V byte is read from HBM once.  The
//     chunk's 32-token tiles are dealt to the four wavefronts in turn, so the
//     workgroup streams one contiguous stretch at a time; each wavefront keeps
//     two tiles of register prefetch and no barrier, and the four partial
//     states are merged through LDS at the end.  When a chunk has at most
//     2048 tokens, the chunk's key and value scales are staged in LDS once
//     (two coalesced 16-byte loads per thread when the scale rows are 16-byte
//     aligned, sixteen 2-byte loads otherwise) instead of four small loads per
//     tile and wavefront.
//   * The dequantisation is fused into the tile load and folded into the math:
//     int8 codes become exact fp16 values with two byte permutes and a packed
//     subtract (1024 + u in fp16 is 0x6400 | u); E4M3FN codes (every one of
//     them exact in fp16) go through the packed fp8 -> fp16 conversion.  The
//     key scale multiplies the score, and the value scale multiplies the
//     probability before it is rounded, so no dequantised tile is ever stored.
//   * S^T = K Q^T and O^T = V^T P^T run on 16x16x32 fp16 MFMA.  The value
//     operand needs 8 tokens of one head-dim column per lane; lanes load 8
//     bytes of each token row and the byte permutes of the fp16 conversion
//     also transpose, so V^T costs nothing extra.  The head-dim order inside a
//     16-row output block is permuted (row m of block j is column 8m + j),
//     which lets each lane load one contiguous 8-byte piece per token.
//   * The bf16 query is prescaled by a power of two per head so it converts to
//     fp16 exactly; the probabilities times value scales are prescaled by a
//     power of two per workgroup, chosen from the largest value scale of its
//     chunk, so they neither overflow nor lose range in fp16 (probabilities
//     reach 2^8 under the lazy running max, see kRescaleSlack).  Both factors are
//     undone in fp32.
//   * The residual window (decode_window_wg) gives one workgroup to the
//     window of each (batch, cache head).  These workgroups are appended to
//     the split kernel's grid, so they run in the tail of its stream rather
//     than in a launch of their own ahead of it.  The window's tokens are few
//     and unquantised bf16: it walks them with 16x16x32 bf16 MFMAs and an
//     exact running max, and writes its partial to one more workspace slot.
//   * Kernel 2 (decode_combine_kernel) merges the splits of one (batch, head):
//     with M = max_s lse_s and w_s = 2^(lse_s - M), LSE = M + log2 sum_s w_s and
//     O = sum_s w_s O_s / sum_s w_s, in the log2 domain; it writes bf16 O and
//     natural-log LSE.
#include "fa_device.hpp"
#include "fa_internal.h"

#include <mutex>

// Partial results of fa_decode_kvq_noalloc: a file-scope device array, so that
// entry point allocates nothing.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code this name is only a stand-in:
// kernels get the device address from fa_decode_scratch(), never the name.
static __device__ __attribute__((aligned(256))) unsigned char scratch[FA_DECODE_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device
}  // namespace

int fa_decode_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fa_set_error(FA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch[dev] = addr;
  }
  *ptr = g_scratch[dev];
  return FA_OK;
}

namespace fa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kDecodeThreads = 256;
constexpr int kTile = 32;  // tokens per step of one wavefront
constexpr int kD = 128;

struct DecodeArgs {
  const void *q;
  const void *k;
  const void *v;
  const void *ks;
  const void *vs;
  const int *seq_lens;
  void *o;
  float *lse;
  float *ws_o;  // [split][B][Hq][d] normalised partial outputs
  float *ws_l;  // [split][B][Hq]   partial log2-sum-exp (log2 units)
  const void *kr;        // residual window keys [B][Hkv][W][d] bf16, or null
  const void *vr;        // residual window values
  const int *rlens;      // [B] window tokens attended, or null for W
  int W;                 // window capacity (0 = no window)
  int nslots;            // partial slots: nsplit, plus one for the window
  long long r_sb, r_sh, r_st;
  int B, Hq, Hkv, G, L, nsplit, chunk;
  long long q_sb, q_sh, kv_sb, kv_sh, sc_sb, sc_sh, o_sb, o_sh, lse_sb, lse_sh;
  unsigned kv_ss;   // token stride in bytes
  unsigned kv_ext;  // bytes of one (batch, head) cache slice
  unsigned sc_ext;  // bytes of one (batch, head) scale slice
  int sc_vec;       // scale rows 16-byte aligned: vector loads, else 2-byte loads
  float c;          // softmax scale * log2(e)
};

__device__ __forceinline__ unsigned perm(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// fp16 pair minus 1152: turns (1152 + x) back into x exactly.
__device__ __forceinline__ unsigned unbias(unsigned w) {
  f16x2 h = __builtin_bit_cast(f16x2, w);
  h = h + f16x2{(_Float16)-1152.0f, (_Float16)-1152.0f};
  return __builtin_bit_cast(unsigned, h);
}

constexpr unsigned kMagic = 0x64646464u;  // fp16 high byte of 1024 + u

// Four int8 codes -> two dwords of exact fp16 pairs (d0,d1) and (d2,d3).
__device__ __forceinline__ void i8x4_to_f16(unsigned w, unsigned &lo, unsigned &hi) {
  const unsigned u = w ^ 0x80808080u;  // x + 128 as unsigned bytes
  lo = unbias(perm(kMagic, u, 0x04010400u));
  hi = unbias(perm(kMagic, u, 0x04030402u));
}

// Two tokens' codes for the same four head-dim columns (a from token t, b from
// token t') -> four dwords, one per column, each the fp16 pair (t, t').
__device__ __forceinline__ void i8_pair_transpose(unsigned a, unsigned b, unsigned out[4]) {
  const unsigned m01 = perm(b, a, 0x05010400u) ^ 0x80808080u;  // a0 b0 a1 b1
  const unsigned m23 = perm(b, a, 0x07030602u) ^ 0x80808080u;  // a2 b2 a3 b3
  out[0] = unbias(perm(kMagic, m01, 0x04010400u));
  out[1] = unbias(perm(kMagic, m01, 0x04030402u));
  out[2] = unbias(perm(kMagic, m23, 0x04010400u));
  out[3] = unbias(perm(kMagic, m23, 0x04030402u));
}

// Four E4M3FN codes -> two dwords of exact fp16 pairs (d0,d1) and (d2,d3).
__device__ __forceinline__ void f8x4_to_f16(unsigned w, unsigned &lo, unsigned &hi) {
  lo = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// E4M3FN counterpart of i8_pair_transpose.
__device__ __forceinline__ void f8_pair_transpose(unsigned a, unsigned b, unsigned out[4]) {
  const unsigned m01 = perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const unsigned m23 = perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  f8x4_to_f16(m01, out[0], out[1]);
  f8x4_to_f16(m23, out[2], out[3]);
}

// Exponent E with x = m * 2^E, m in [0.5, 1); 0 for x == 0.
__device__ __forceinline__ int exp_of(float x) {
  int e;
  (void)frexpf(x, &e);
  return x > 0.f ? e : 0;
}

// The value lane (l ^ 16) holds: v_permlane16_swap exchanges the odd rows of
// its first operand with the even rows of its second, so with x in both the
// second result holds, in each even row, the row above, and the first, in
// each odd row, the row below.  No LDS round trip (a width-64 shuffle would
// be an LDS permute).
__device__ __forceinline__ float xor16_lanes(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) == 0 ? r[1] : r[0]);
}

// Four fp16 scales at byte offset voff.  Offsets always go in the per-lane
// operand, which the buffer range check covers (the scalar offset operand is
// left at zero everywhere in this library).
template <bool VEC> __device__ __forceinline__ u32x2 load_scales4_at(__amdgpu_buffer_rsrc_t r, unsigned voff) {
  if constexpr (VEC) return buf_load8_nt(r, voff);
  // four 2-byte loads built into two 2-element vectors.  (Packed instead with
  // shifts and ORs, this compiler kept more of the three tiles' scales live
  // at once and spilled 16-24 bytes per thread to scratch inside the loop;
  // built this way the unaligned-scale kernels do not spill.)
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 lo, hi;
  lo[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, kNonTemporal);
  lo[1] = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 2u, 0, kNonTemporal);
  hi[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 4u, 0, kNonTemporal);
  hi[1] = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 6u, 0, kNonTemporal);
  return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Four fp16 scales of consecutive tokens starting at token t (a multiple of 4).
// VEC (rows 16-byte aligned) is a compile-time choice: a run-time one makes
// the compiler issue both forms and select, waiting on the loads at once.
template <bool VEC> __device__ __forceinline__ u32x2 load_scales4(__amdgpu_buffer_rsrc_t r, int t) {
  return load_scales4_at<VEC>(r, static_cast<unsigned>(t) * 2u);
}

struct TileRegs {
  u32x4 k[2][2];   // [token block][16-byte half]: 32 codes of one token row
  u32x2 v[8];      // 8 tokens x 8 codes of one 8-column chunk
  u32x2 ks[2];     // 4 fp16 key scales per token block
  u32x2 vs[2];     // 4 fp16 value scales per token block
};

// Merges the four wavefront partials in s_o / s_l into partial slot `slot`
// of the workspace: with M the largest wavefront lse2, lse2 = M + log2 sum 2^(lse2_w - M)
// and O = sum 2^(lse2_w - lse2) O_w.  Called by the whole workgroup after a barrier.
__device__ __forceinline__ void merge_waves_to_slot(const DecodeArgs &a, const float (*s_o)[FA_DECODE_MAX_GROUP][kD],
                                                    const float (*s_l)[FA_DECODE_MAX_GROUP], int slot, int b, int kvh) {
  const int G = a.G;
  for (int idx = threadIdx.x; idx < G * kD; idx += kDecodeThreads) {
    const int qn = idx / kD, d = idx % kD;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_l[w][qn]);
    float lse2 = neg_inf(), o = 0.f;
    if (M != neg_inf()) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) tot += fast_exp2(s_l[w][qn] - M);
      lse2 = M + __log2f(tot);
#pragma unroll
      for (int w = 0; w < 4; ++w) o += fast_exp2(s_l[w][qn] - lse2) * s_o[w][qn][d];
    }
    const long long row = (static_cast<long long>(slot) * a.B + b) * a.Hq + kvh * G + qn;
    a.ws_o[row * kD + d] = o;
    if (d == 0) a.ws_l[row] = lse2;
  }
}

// The residual window of one (batch, cache head): up to W bf16 tokens, cut
// into four contiguous quarters, one per wavefront, walked in 32-token tiles
// with the split kernel's matrix-core layout on bf16 operands: S^T = K Q^T as
// 16x16x32 bf16 MFMAs (lane (n, g) holds key and query elements 32g + 8s + j,
// so both operands are plain 16-byte row loads), the probabilities rounded to
// bf16 straight from the S^T accumulator into the B operand of O^T = V^T P^T,
// and V^T built from 16-byte row loads with 16-bit permutes (block j of the
// output holds head-dim column 8m + j in row m).  The running max is exact
// (no lazy slack), so probabilities stay <= 1.
__device__ __attribute__((always_inline)) void decode_window_wg(const DecodeArgs &a, int wid,
                                                              float (*s_o)[FA_DECODE_MAX_GROUP][kD],
                                                              float (*s_l)[FA_DECODE_MAX_GROUP]) {
  const int b = wid / a.Hkv;
  const int kvh = wid % a.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int G = a.G;

  int r = a.rlens != nullptr ? a.rlens[b] : a.W;
  r = min(max(r, 0), a.W);
  const int quarter = ((r + 3) / 4 + kTile - 1) / kTile * kTile;
  const int w0 = min(wave * quarter, r);
  const int w1 = min(w0 + quarter, r);

  // query column n (zero past G): elements 32g + 8s .. 32g + 8s + 7
  bf16x8 qf[4];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + b * a.q_sb + (kvh * G + (n < G ? n : 0)) * a.q_sh;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const u32x4 raw = n < G ? *reinterpret_cast<const u32x4 *>(qrow + 32 * g + 8 * s4) : u32x4{0u, 0u, 0u, 0u};
      qf[s4] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const char *kbase = reinterpret_cast<const char *>(static_cast<const __bf16 *>(a.kr) + b * a.r_sb + kvh * a.r_sh);
  const char *vbase = reinterpret_cast<const char *>(static_cast<const __bf16 *>(a.vr) + b * a.r_sb + kvh * a.r_sh);
  const unsigned rs = static_cast<unsigned>(a.r_st) * 2u;  // row stride, bytes

  float m_run = neg_inf();
  float l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) oacc[j] = f32x4{};

  for (int t0 = w0; t0 < w1; t0 += kTile) {
    // rows past the range read as zero through a buffer range that ends at
    // the wavefront's last token
    const int left = w1 - t0;
    const __amdgpu_buffer_rsrc_t tk = make_rsrc(kbase + static_cast<size_t>(t0) * rs, (left - 1) * rs + 2u * kD);
    const __amdgpu_buffer_rsrc_t tv = make_rsrc(vbase + static_cast<size_t>(t0) * rs, (left - 1) * rs + 2u * kD);
    u32x4 kf[2][4], vrow[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) kf[tb][s4] = buf_load16(tk, (16u * tb + n) * rs + 2u * (32 * g + 8 * s4));
#pragma unroll
    for (int e = 0; e < 8; ++e)  // token 4g + (e & 3) + 16 (e >> 2), columns 8n .. 8n + 7
      vrow[e] = buf_load16(tv, (4u * g + (e & 3) + 16u * (e >> 2)) * rs + 16u * n);

    f32x4 sacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sacc[tb] = f32x4{};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[tb][s4]), qf[s4], sacc[tb], 0, 0, 0);
    }
    float sc[8];
    float mx = neg_inf();
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * tb + 4 * g + i;
        const float s2 = tok < w1 ? sacc[tb][i] * a.c : neg_inf();
        sc[4 * tb + i] = s2;
        mx = fmaxf(mx, s2);
      }
    mx = fmaxf(mx, xor16_lanes(mx));
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx);      // finite: the tile holds a token
    const float alpha = fast_exp2(m_run - m_new);  // 0 while m_run is -inf
    float lsum = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = fast_exp2(sc[e] - m_new);
      lsum += pe;
      pf[e] = static_cast<__bf16>(pe);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // column 8n + j of the 8 tokens: 16-bit half (j & 1) of dword j / 2
      const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x4 w;
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2) w[p2] = perm(vrow[2 * p2 + 1][j >> 1], vrow[2 * p2][j >> 1], sel);
      oacc[j] = oacc[j] * alpha;
      oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pf, oacc[j], 0, 0, 0);
    }
  }

  float l_tot = l_run;
  l_tot += xor16_lanes(l_tot);
  l_tot += swap_halves(l_tot);
  if (n < G) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][n][32 * g + 8 * i + j] = oacc[j][i] * inv;
    if (g == 0) s_l[wave][n] = l_tot > 0.f ? m_run + __log2f(l_tot) : neg_inf();
  }
  __syncthreads();
  merge_waves_to_slot(a, s_o, s_l, a.nsplit, b, kvh);
}

// Scales of a chunk of at most this many tokens are staged in LDS once per
// workgroup (two coalesced 16-byte loads per thread) instead of being fetched
// tile by tile: four tiny global loads per tile cost about 5 % of the
// bandwidth of a stream shaped like this one.
constexpr int kStageTok = 2048;

template <bool SCVEC, bool FP8, bool STAGED = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void decode_split_kernel(const DecodeArgs a) {
  __shared__ float s_o[4][FA_DECODE_MAX_GROUP][kD];
  __shared__ float s_l[4][FA_DECODE_MAX_GROUP];
  __shared__ float s_vmax[4];
  __shared__ __attribute__((aligned(16))) _Float16 s_sc[STAGED ? 2 * kStageTok : 8];  // key scales, then value scales

  const int bid = blockIdx.x;
  // workgroups past the splits' own take the window, one per (batch, KV head),
  // and run in the tail of the split workgroups instead of in a launch of
  // their own ahead of them
  const int split_wgs = a.nsplit * a.Hkv * a.B;
  if (bid >= split_wgs) {
    decode_window_wg(a, bid - split_wgs, s_o, s_l);
    return;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: range bounds and buffer resources stay scalar
  const int n = lane & 15;   // query column (S^T, O^T) or row within a 16-row block
  const int g = lane >> 4;   // lane group: reduction slots 8g..8g+7

  const int split = bid % a.nsplit;
  const int kvh = (bid / a.nsplit) % a.Hkv;
  const int b = bid / (a.nsplit * a.Hkv);
  const int G = a.G;

  int len = a.seq_lens != nullptr ? a.seq_lens[b] : a.L;
  len = min(max(len, 0), a.L);
  const int c0 = split * a.chunk;
  const int c1 = min(c0 + a.chunk, len);
  // The chunk's 32-token tiles are dealt to the four wavefronts in turn (tile
  // i of a wavefront is tile 4i + wave of the chunk), so at any moment the
  // workgroup streams one contiguous stretch of the cache: measured on this
  // part, that reads about 7 % faster than four separate stretches.
  const int n_ct = c1 > c0 ? (c1 - c0 + kTile - 1) / kTile : 0;
  const int ntiles = n_ct > wave ? (n_ct - wave + 3) / 4 : 0;
  auto tile_t0 = [&](int i) { return c0 + kTile * (4 * i + wave); };
  // the value-scale pass below gives each wavefront one contiguous quarter
  const int quarter = ((a.chunk + 3) / 4 + kTile - 1) / kTile * kTile;
  const int v0 = c0 + wave * quarter;
  const int v1 = min(v0 + quarter, c1);

  const __amdgpu_buffer_rsrc_t rvs =
      make_rsrc(static_cast<const _Float16 *>(a.vs) + b * a.sc_sb + kvh * a.sc_sh, a.sc_ext);

  // ---- tile loads.  Each tile gets buffer resources based at its first token
  // and ending at the wavefront's last token, so tokens past the range read
  // as zero without per-lane checks, and every per-lane offset is a loop
  // constant.  The scales depend on the lane group only, so lanes of padding
  // query columns load the same, valid, values. ----
  const char *kslice = static_cast<const char *>(a.k) + b * a.kv_sb + kvh * a.kv_sh;
  const char *vslice = static_cast<const char *>(a.v) + b * a.kv_sb + kvh * a.kv_sh;
  const char *ksslice = reinterpret_cast<const char *>(static_cast<const _Float16 *>(a.ks) + b * a.sc_sb + kvh * a.sc_sh);
  const char *vsslice = reinterpret_cast<const char *>(static_cast<const _Float16 *>(a.vs) + b * a.sc_sb + kvh * a.sc_sh);
  const unsigned ss = a.kv_ss;
  unsigned k_off[2], v_off[8];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) k_off[tb] = (16u * tb + n) * ss + 32u * g;  // codes 32g .. 32g+31 of token 16tb+n
#pragma unroll
  for (int j = 0; j < 8; ++j)  // codes 8n .. 8n+7 of token 4g + (j & 3) + 16 (j >> 2)
    v_off[j] = (4u * g + (j & 3) + 16u * (j >> 2)) * ss + 8u * n;
  const unsigned s_off = 8u * g;  // scales of tokens 4g .. 4g+3 (+ 16 tb)
  // staged scales of a tile, from LDS; a tile past the chunk reads the first
  // tile's (its scores are masked)
  auto load_sc = [&](TileRegs &r, int t0) {
    const int rel = c1 - t0 > 0 ? t0 - c0 : 0;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      r.ks[tb] = *reinterpret_cast<const u32x2 *>(&s_sc[rel + 16 * tb + 4 * g]);
      r.vs[tb] = *reinterpret_cast<const u32x2 *>(&s_sc[kStageTok + rel + 16 * tb + 4 * g]);
    }
  };
  auto load_tile = [&](TileRegs &r, int t0, bool staged_sc = true) {
    const int left = c1 - t0;  // tokens of the chunk from t0 on
    if constexpr (STAGED) {
      if (staged_sc) load_sc(r, t0);
    }
    const unsigned kv_rec = left > 0 ? static_cast<unsigned>(left - 1) * ss + kD : 0u;
    // The range check of a buffer load is made per dword: a dword that
    // straddles the end of the range reads as zero in full.  The 8-byte scale
    // loads therefore get a range rounded up to whole groups of four tokens
    // (never past the cache slice: L is a multiple of 4 on this path); the
    // scores of the extra tokens are masked below.  The 2-byte loads take the
    // exact range.
    const int sc_tok = SCVEC ? min((left + 3) & ~3, a.L - t0) : left;
    const unsigned sc_rec = left > 0 ? static_cast<unsigned>(sc_tok) * 2u : 0u;
    const unsigned shift = left > 0 ? static_cast<unsigned>(t0) * ss : 0u;
    const __amdgpu_buffer_rsrc_t tk = make_rsrc(kslice + shift, kv_rec);
    const __amdgpu_buffer_rsrc_t tv = make_rsrc(vslice + shift, kv_rec);
    const __amdgpu_buffer_rsrc_t tks = make_rsrc(ksslice + (left > 0 ? 2u * t0 : 0u), sc_rec);
    const __amdgpu_buffer_rsrc_t tvs = make_rsrc(vsslice + (left > 0 ? 2u * t0 : 0u), sc_rec);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      r.k[tb][0] = buf_load16_nt(tk, k_off[tb]);
      r.k[tb][1] = buf_load16_nt(tk, k_off[tb] + 16u);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = buf_load8_nt(tv, v_off[j]);
    if constexpr (!STAGED) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        r.ks[tb] = load_scales4_at<SCVEC>(tks, s_off + 32u * tb);
        r.vs[tb] = load_scales4_at<SCVEC>(tvs, s_off + 32u * tb);
      }
    }
  };

  // The first two tiles are requested before the query and the value-scale
  // pass below, so the workgroup waits on one memory round trip, not three.
  TileRegs r0, r1, r2;
  // staged scales: 8 tokens per thread and array, the chunk starting at c0 (a
  // multiple of 32 tokens, so with aligned scale rows the 16-byte loads are
  // aligned; otherwise eight 2-byte loads per array); tokens past L read as
  // zero, those past c1 are masked where they are used
  u32x4 st_k{0u, 0u, 0u, 0u}, st_v{0u, 0u, 0u, 0u};
  if constexpr (STAGED) {
    const __amdgpu_buffer_rsrc_t rks = make_rsrc(ksslice, a.sc_ext);
    const bool in = 8 * tid < a.chunk;
    const unsigned off = in ? static_cast<unsigned>(c0 + 8 * tid) * 2u : kOOB;
    if constexpr (SCVEC) {
      st_k = buf_load16_nt(rks, off);
      st_v = buf_load16_nt(rvs, off);
    } else {
      const u32x2 k0 = load_scales4_at<false>(rks, off), k1 = load_scales4_at<false>(rks, off + 8u);
      const u32x2 v0s = load_scales4_at<false>(rvs, off), v1s = load_scales4_at<false>(rvs, off + 8u);
      st_k = u32x4{k0[0], k0[1], k1[0], k1[1]};
      st_v = u32x4{v0s[0], v0s[1], v1s[0], v1s[1]};
    }
  }
  load_tile(r0, tile_t0(0), false);  // staged scales of these two: after the barrier below
  load_tile(r1, tile_t0(1), false);
  // value scales of the first step of the prescale pass below (8 tokens per
  // lane; v0 is a multiple of 32 tokens, so every 16-byte load is aligned, and
  // tokens past the range are dropped there)
  const int vt0 = v0 + 8 * lane;
  u32x2 vs_lo0{0u, 0u}, vs_hi0{0u, 0u};
  if constexpr (!STAGED) {
    vs_lo0 = load_scales4<SCVEC>(rvs, vt0);
    vs_hi0 = load_scales4<SCVEC>(rvs, vt0 + 4);
  }

  // ---- query: lane (n, g) holds q[n][32g + 8s + j], prescaled into fp16 ----
  f16x8 qf[4];
  float cq;  // score multiplier for query n: softmax scale * log2 e / 2^eq
  {
    float qv[32];
    const bool real = n < G;
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + b * a.q_sb + (kvh * G + (real ? n : 0)) * a.q_sh;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // padding columns read row 0 (a valid address) and drop it, so the four
      // loads issue back to back without a branch
      u32x4 raw = *reinterpret_cast<const u32x4 *>(qrow + 32 * g + 8 * c);
      if (!real) raw = u32x4{0, 0, 0, 0};
      const bf16x8 hv = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[8 * c + e] = static_cast<float>(hv[e]);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(qv[e]));
    amax = fmaxf(amax, xor16_lanes(amax));
    amax = fmaxf(amax, swap_halves(amax));
    const int eq = amax > 0.f ? min(14 - exp_of(amax), 100) : 0;  // amax * 2^eq in [2^13, 2^14)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[c][e] = static_cast<_Float16>(ldexpf(qv[8 * c + e], eq));
    cq = ldexpf(a.c, -eq);
  }

  // ---- value-scale prescale of this workgroup: vs * 2^fw < 2^6, so with
  // p < 2^kRescaleSlack (= 2^8) every w = p * vs * 2^fw stays below 2^14 ----
  int fw = 0;
  {
    float vmax = 0.f;
    auto fold = [&](int t, u32x2 lo, u32x2 hi) {
      const f16x8 sv = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (t + e < v1) vmax = fmaxf(vmax, fabsf(static_cast<float>(sv[e])));
    };
    if constexpr (STAGED) {
      // the staged value scales of this thread's 8 tokens.  Slots at or past
      // c1 (the sequence's end inside this chunk) hold whatever the caller
      // left there, possibly Inf or NaN: they are zeroed, because a masked
      // token's weight is p * v_scale with p = 0, and 0 * Inf is NaN.
      f16x8 sv = __builtin_bit_cast(f16x8, st_v);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + 8 * tid + e >= c1) sv[e] = static_cast<_Float16>(0.f);
      if (8 * tid < a.chunk) {
        *reinterpret_cast<u32x4 *>(&s_sc[8 * tid]) = st_k;
        *reinterpret_cast<u32x4 *>(&s_sc[kStageTok + 8 * tid]) = __builtin_bit_cast(u32x4, sv);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vmax = fmaxf(vmax, fabsf(static_cast<float>(sv[e])));
    } else {
      fold(vt0, vs_lo0, vs_hi0);
      for (int t = vt0 + 8 * 64; t < v1; t += 8 * 64) fold(t, load_scales4<SCVEC>(rvs, t), load_scales4<SCVEC>(rvs, t + 4));
    }
    vmax = fmaxf(vmax, swap_halves(vmax));
    vmax = fmaxf(vmax, xor16_lanes(vmax));
    vmax = fmaxf(vmax, row16_xor<8>(vmax));
    vmax = fmaxf(vmax, row16_xor<4>(vmax));
    vmax = fmaxf(vmax, row16_xor<2>(vmax));
    vmax = fmaxf(vmax, row16_xor<1>(vmax));
    // every wavefront's tiles spread over the whole chunk: take the chunk's maximum
    if (lane == 0) s_vmax[wave] = vmax;
    __syncthreads();
    vmax = fmaxf(fmaxf(s_vmax[0], s_vmax[1]), fmaxf(s_vmax[2], s_vmax[3]));
    fw = vmax > 0.f ? min(6 - exp_of(vmax), 100) : 0;
  }
  if constexpr (STAGED) {  // the barrier above published the staged scales
    load_sc(r0, tile_t0(0));
    load_sc(r1, tile_t0(1));
  }
  const float wmul = ldexpf(1.f, fw);

  float m_run = neg_inf();
  float l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) oacc[j] = f32x4{};

  auto compute_tile = [&](const TileRegs &r, int t0) {
    // S^T = K Q^T, two 16-token blocks
    f32x4 sacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sacc[tb] = f32x4{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 raw = r.k[tb][s >> 1];
        unsigned w[4];
        if constexpr (FP8) {
          f8x4_to_f16(raw[2 * (s & 1)], w[0], w[1]);
          f8x4_to_f16(raw[2 * (s & 1) + 1], w[2], w[3]);
        } else {
          i8x4_to_f16(raw[2 * (s & 1)], w[0], w[1]);
          i8x4_to_f16(raw[2 * (s & 1) + 1], w[2], w[3]);
        }
        const f16x8 kf = __builtin_bit_cast(f16x8, u32x4{w[0], w[1], w[2], w[3]});
        sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[s], sacc[tb], 0, 0, 0);
      }
    }
    // scores in log2 units; tokens t0 + 16tb + 4g + i
    float sc[8];
    float mx = neg_inf();
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const f16x4 kscale = __builtin_bit_cast(f16x4, r.ks[tb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * tb + 4 * g + i;
        float s = sacc[tb][i] * (static_cast<float>(kscale[i]) * cq);
        s = tok < c1 ? s : neg_inf();
        sc[4 * tb + i] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, xor16_lanes(mx));
    mx = fmaxf(mx, swap_halves(mx));
    // lazy running max: the O rescale runs only when some row's max moved by
    // more than the slack (probabilities stay below 2^kRescaleSlack)
    const bool move = mx > m_run + kRescaleSlack;
    const float m_new = move ? mx : m_run;
    const float alpha = move ? fast_exp2(m_run - m_new) : 1.f;  // 0 when m_run = -inf
    const float m_use = m_new == neg_inf() ? 0.f : m_new;
    float lsum = 0.f;
    f16x8 pf;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const f16x4 vscale = __builtin_bit_cast(f16x4, r.vs[tb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(sc[4 * tb + i] - m_use);
        lsum += p;
        float vsc = static_cast<float>(vscale[i]);
        if constexpr (SCVEC && !STAGED) {
          // the 8-byte scale loads reach up to three slots past c1, which may
          // hold Inf or NaN; a masked token must weigh 0, not 0 * Inf
          const int tok = t0 + 16 * tb + 4 * g + i;
          vsc = tok < c1 ? vsc : 0.f;
        }
        pf[4 * tb + i] = static_cast<_Float16>(p * (vsc * wmul));
      }
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    // V^T operands: block j holds head-dim column 8n + j of tokens
    // {4g..4g+3, 16+4g..16+4g+3}; built pairwise from the 8-byte rows
    unsigned vt[8][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        unsigned out[4];
        if constexpr (FP8) f8_pair_transpose(r.v[2 * p][hd], r.v[2 * p + 1][hd], out);
        else i8_pair_transpose(r.v[2 * p][hd], r.v[2 * p + 1][hd], out);
#pragma unroll
        for (int k = 0; k < 4; ++k) vt[4 * hd + k][p] = out[k];
      }
    }
    if (wave_any(move)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) oacc[j] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f16x8 vf = __builtin_bit_cast(f16x8, u32x4{vt[j][0], vt[j][1], vt[j][2], vt[j][3]});
      oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf, oacc[j], 0, 0, 0);
    }
  };

  // ---- stream this wavefront's range, two tiles of prefetch (a ring of
  // three register tiles; loads past the range read zeros without touching
  // memory, so the loop body issues them unconditionally) ----
  if (ntiles > 0) {
    int t = 0;
    for (; t + 2 < ntiles; t += 3) {
      load_tile(r2, tile_t0(t + 2));
      compute_tile(r0, tile_t0(t));
      load_tile(r0, tile_t0(t + 3));
      compute_tile(r1, tile_t0(t + 1));
      load_tile(r1, tile_t0(t + 4));
      compute_tile(r2, tile_t0(t + 2));
    }
    if (t < ntiles) compute_tile(r0, tile_t0(t));
    if (t + 1 < ntiles) compute_tile(r1, tile_t0(t + 1));
  }

  // ---- wavefront partial: O_w = O_acc / (l 2^fw), lse2_w = m + log2 l ----
  float l_tot = l_run;
  l_tot += xor16_lanes(l_tot);
  l_tot += swap_halves(l_tot);
  if (n < G) {
    const float inv = l_tot > 0.f ? ldexpf(1.f / l_tot, -fw) : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][n][32 * g + 8 * i + j] = oacc[j][i] * inv;
    if (g == 0) s_l[wave][n] = l_tot > 0.f ? m_run + __log2f(l_tot) : neg_inf();
  }
  __syncthreads();

  // ---- merge the four wavefronts into this split's partial ----
  merge_waves_to_slot(a, s_o, s_l, split, b, kvh);
}

__global__ __attribute__((amdgpu_flat_work_group_size(128, 128)))
void decode_combine_kernel(const DecodeArgs a) {
  // one workgroup per (batch, query head); thread d owns output column d.
  // Partial slots (the splits, then the window's) are taken 16 at a time with
  // all loads of a group in flight, in one pass: each group's maximum joins
  // the running one and rescales what is summed so far (with 16 splits there
  // is a single group and no rescale).
  const int d = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const long long stride = static_cast<long long>(a.B) * a.Hq;
  constexpr int kGroup = 16;
  float M = neg_inf(), tot = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < a.nslots; s0 += kGroup) {
    float l[kGroup], v[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const bool ok = s0 + i < a.nslots;
      l[i] = ok ? a.ws_l[(s0 + i) * stride + bh] : neg_inf();
      v[i] = ok ? a.ws_o[((s0 + i) * stride + bh) * kD + d] : 0.f;
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) Mg = fmaxf(Mg, l[i]);
    if (Mg != neg_inf()) {
      const float r = fast_exp2(M - Mg);  // 0 while nothing has been summed (M = -inf)
      tot *= r;
      acc *= r;
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const float w = fast_exp2(l[i] - Mg);  // 0 for empty splits
        tot += w;
        acc += w * v[i];
      }
      M = Mg;
    }
  }
  float lse2 = neg_inf(), o = 0.f;
  if (M != neg_inf()) {
    lse2 = M + __log2f(tot);
    o = acc / tot;
  }
  __bf16 *orow = static_cast<__bf16 *>(a.o) + b * a.o_sb + h * a.o_sh;
  orow[d] = static_cast<__bf16>(o);
  if (d == 0 && a.lse != nullptr) a.lse[b * a.lse_sb + h * a.lse_sh] = lse2 * kLn2;
}

}  // namespace fa

int fa_launch_decode(const fa_decode_params *p, void *stream) {
  using namespace fa;
  DecodeArgs a{};
  a.q = p->q;
  a.k = p->k_cache;
  a.v = p->v_cache;
  a.ks = p->k_scale;
  a.vs = p->v_scale;
  a.seq_lens = p->seq_lens;
  a.o = p->o;
  a.lse = p->lse;
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.G = p->Hq / p->Hkv;
  a.L = p->L;
  a.nsplit = p->num_splits;
  // chunk length rounded up to whole 32-token tiles: every tile then starts on
  // a 64-byte boundary of the scale arrays
  a.chunk = ((p->L + p->num_splits - 1) / p->num_splits + kTile - 1) / kTile * kTile;
  a.q_sb = p->q_strides[0];
  a.q_sh = p->q_strides[1];
  a.kv_sb = p->kv_strides[0];
  a.kv_sh = p->kv_strides[1];
  a.sc_sb = p->scale_strides[0];
  a.sc_sh = p->scale_strides[1];
  a.o_sb = p->o_strides[0];
  a.o_sh = p->o_strides[1];
  a.lse_sb = p->lse_strides[0];
  a.lse_sh = p->lse_strides[1];
  a.kv_ss = p->L > 1 ? static_cast<unsigned>(p->kv_strides[2]) : 0u;
  a.kv_ext = p->L > 0 ? static_cast<unsigned>((static_cast<long long>(p->L - 1) * p->kv_strides[2] + p->d)) : 0u;
  a.sc_ext = static_cast<unsigned>(p->L) * 2u;
  // 8-byte scale loads need 16-byte aligned scale rows and a slice of whole
  // 4-token groups, so that no load straddles the end of the slice
  a.sc_vec = (reinterpret_cast<uintptr_t>(p->k_scale) % 16 == 0 && reinterpret_cast<uintptr_t>(p->v_scale) % 16 == 0 &&
              (p->scale_strides[0] * 2) % 16 == 0 && (p->scale_strides[1] * 2) % 16 == 0 && p->L % 4 == 0)
                 ? 1 : 0;
  a.c = p->softmax_scale * 1.4426950408889634f;
  const bool window = p->W > 0;
  a.kr = window ? p->k_recent : nullptr;
  a.vr = window ? p->v_recent : nullptr;
  a.rlens = window ? p->recent_lens : nullptr;
  a.W = window ? p->W : 0;
  a.r_sb = p->recent_strides[0];
  a.r_sh = p->recent_strides[1];
  a.r_st = p->recent_strides[2];
  a.nslots = p->num_splits + (window ? 1 : 0);
  const size_t rows = static_cast<size_t>(a.nslots) * p->B * p->Hq;
  a.ws_o = static_cast<float *>(p->workspace);
  a.ws_l = reinterpret_cast<float *>(static_cast<char *>(p->workspace) +
                                     ((rows * kD * sizeof(float) + 255) & ~size_t(255)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid1 = static_cast<unsigned>(p->num_splits + (window ? 1 : 0)) * p->Hkv * p->B;
  const dim3 g1(grid1), b1(kDecodeThreads);
  const bool fp8 = p->kv_format == FA_KV_FP8_E4M3_TOKHEAD_F16SCALE;
  const bool staged = a.chunk <= kStageTok;
  fa_log_launch("decode_split_kernel", grid1, kDecodeThreads, 0,
                "kv=%s scales=%s B=%d Hq=%d Hkv=%d L=%d splits=%d chunk=%d window=%d", fp8 ? "fp8" : "int8",
                staged ? (a.sc_vec ? "staged" : "staged2") : (a.sc_vec ? "vec8" : "scalar2"), a.B, a.Hq, a.Hkv, a.L,
                a.nsplit, a.chunk, a.W);
  if (staged && a.sc_vec && fp8) hipLaunchKernelGGL((decode_split_kernel<true, true, true>), g1, b1, 0, s, a);
  else if (staged && a.sc_vec) hipLaunchKernelGGL((decode_split_kernel<true, false, true>), g1, b1, 0, s, a);
  else if (staged && fp8) hipLaunchKernelGGL((decode_split_kernel<false, true, true>), g1, b1, 0, s, a);
  else if (staged) hipLaunchKernelGGL((decode_split_kernel<false, false, true>), g1, b1, 0, s, a);
  else if (a.sc_vec && fp8) hipLaunchKernelGGL((decode_split_kernel<true, true>), g1, b1, 0, s, a);
  else if (a.sc_vec) hipLaunchKernelGGL((decode_split_kernel<true, false>), g1, b1, 0, s, a);
  else if (fp8) hipLaunchKernelGGL((decode_split_kernel<false, true>), g1, b1, 0, s, a);
  else hipLaunchKernelGGL((decode_split_kernel<false, false>), g1, b1, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "decode split launch: %s", hipGetErrorString(e));
  fa_log_launch("decode_combine_kernel", static_cast<unsigned>(p->B) * p->Hq, kD, 0, "slots=%d", a.nslots);
  hipLaunchKernelGGL(decode_combine_kernel, dim3(static_cast<unsigned>(p->B) * p->Hq), dim3(kD), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return fa_set_error(FA_ERR_HIP, "decode combine launch: %s", hipGetErrorString(e));
  return FA_OK;
}
