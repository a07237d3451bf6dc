// Decode attention over the three-segment OSCAR pool on gfx950.
//
// One launch per decode step.  The grid holds, for every (sequence, KV head),
// a few BF16 units (sink + recent pages) and a split-K set of INT2 history
// chunks.  Each workgroup writes one partial (normalized o, natural-log lse)
// per query head; the workgroup that finishes last for a (sequence, KV head)
// merges all partials by log-sum-exp and writes the bf16 output (ModelScope/
// CSDN page, design section: separate INT2 and BF16 kernels merged by online
// softmax; here they are workgroups of one launch).
//
// INT2 history (per wave, tiles of SLOTS pages):
//   scores  S = codes . q'  on the int8 matrix cores.  q' = q R_K (the online
//           rotation, MarkTechPost article, "Outcome") is computed once per
//           workgroup and split into two int8 terms, q' ~ sq (a + b/256), so
//           the integer dot is exact and q' carries ~16 significant bits.
//           With the key dequantization k' = s (code - z) the logit is
//           sm * s * sq/256 * (S_ab - z * sum(256 a + b)).
//   P.V     on the bf16 matrix cores with the value codes as exact bf16
//           operands 1 + code/8 and the weights w = p * s_V as bf16:
//           sum w (code - z) = 8 (sum w (1 + code/8) - sum w) - sum w z.
//   softmax online, with a lazy running max (rescale only when a logit
//           exceeds the running max by more than 2^8).
// The GQA query heads of a KV head share every loaded page; the 16 columns
// of each MFMA tile hold (page slot, query head) pairs, so one score tile
// covers SLOTS pages and all softmax arithmetic is shared across them.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace oscar {
namespace {

// build-time tuning knobs (defaults are the measured best on MI355X)
#ifndef OSCAR_DECODE_WAVES
#define OSCAR_DECODE_WAVES 8
#endif
#ifndef OSCAR_DECODE_RING
#define OSCAR_DECODE_RING 2
#endif
#ifndef OSCAR_BF16_SLOTS
#define OSCAR_BF16_SLOTS 2
#endif
constexpr int kWaves = OSCAR_DECODE_WAVES;  // waves per workgroup
constexpr int kRing = OSCAR_DECODE_RING;    // INT2 tiles held per wave (1 computing + kRing-1 in flight)
constexpr int kThreads = 64 * kWaves;
constexpr float kNegBig = -1.0e30f;  // finite "no token yet" running max
constexpr float kLazy = 8.0f;        // log2 slack before the running max is raised
constexpr float kLn2 = 0.69314718055994530942f;

template <int D, int NG, int GQA>
struct DC {
  static constexpr int G = D / NG;
  static constexpr int SLOTS = (16 / GQA) < 4 ? (16 / GQA) : 4;  // INT2 pages per tile
  static constexpr int COLS = SLOTS * GQA;
  static constexpr int SLOTS_B = SLOTS < OSCAR_BF16_SLOTS ? SLOTS : OSCAR_BF16_SLOTS;  // BF16 pages per tile
  static constexpr int COLS_B = SLOTS_B * GQA;
  static constexpr int KW = D / 64;  // 32-bit K (and V) code words per record
  static constexpr int CB = D / 16;  // 16-channel blocks (P.V MFMAs per page)
  static constexpr int KB = D / 32;  // k=32 steps of the BF16 score MFMA
  static constexpr int BLK2 = 8 * D + 128 * NG;
  static constexpr int BLK16 = 64 * D;
  static constexpr int REC = D / 8;  // bytes per code record
};

template <int D, int GQA>
struct Smem {
  static constexpr int SLOTS = (16 / GQA) < 4 ? (16 / GQA) : 4;
  union {
    float part[kWaves][GQA][D + 1];   // per-wave partials, [D] = lse (log2)
    float wts[kWaves * GQA * (D + 1)];  // final-merge weights [unit][head]
  } u;
  v4i bq[SLOTS][2][D / 64][64];       // int8 q' B operands per lane (shared by the waves)
  float qr[GQA * D];                  // q' = q R_K (fp32)
  alignas(16) int8_t ta[GQA * D];     // int8 terms of q'
  alignas(16) int8_t tb[GQA * D];
  int sig[GQA * 2];                   // sum(256 a + b) per head and group
  float wred[kWaves];
  int last;
};

// ---------------------------------------------------------------- helpers --
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// max / sum over the columns of one 16-lane row that hold the same query head
template <int GQA>
__device__ __forceinline__ float slot_max(float x) {
  if constexpr (GQA < 16) x = fmaxf(x, dpp_row_ror<GQA>(x));
  if constexpr (2 * GQA < 16) x = fmaxf(x, dpp_row_ror<2 * GQA>(x));
  if constexpr (4 * GQA < 16) x = fmaxf(x, dpp_row_ror<4 * GQA>(x));
  return x;
}
template <int GQA>
__device__ __forceinline__ float slot_sum(float x) {
  if constexpr (GQA < 16) x += dpp_row_ror<GQA>(x);
  if constexpr (2 * GQA < 16) x += dpp_row_ror<2 * GQA>(x);
  if constexpr (4 * GQA < 16) x += dpp_row_ror<4 * GQA>(x);
  return x;
}
__device__ __forceinline__ float col_sum(float x) {  // over the 4 lane groups
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float col_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ v4s as_v4s(uint32_t lo, uint32_t hi) {
  v4s r;
  r[0] = (short)(lo & 0xFFFF);
  r[1] = (short)(lo >> 16);
  r[2] = (short)(hi & 0xFFFF);
  r[3] = (short)(hi >> 16);
  return r;
}
__device__ __forceinline__ v8bf as_v8bf(uint4 x) {
  return __builtin_bit_cast(v8bf, x);
}
// byte transpose: out[m].byte[b] = in[b].byte[m]
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t t01l = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
  const uint32_t t23l = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t t01h = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
  const uint32_t t23h = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
}

// online-softmax state of one wave: accumulators O^T[channel][column]
template <int D, int NG>
struct Acc {
  v4f o[D / 16];
  float m, l;
  float Z[NG];  // INT2 only: sum over tokens of weight * (operand bias + zero)
  __device__ void init() {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};
    m = kNegBig;
    l = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) Z[g] = 0.f;
  }
  __device__ void scale(float f) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] *= f;
    l *= f;
#pragma unroll
    for (int g = 0; g < NG; ++g) Z[g] *= f;
  }
  // lazy running max: raise m only when some logit exceeds it by kLazy
  __device__ __forceinline__ void update_max(const float lg[4]) {
    const float lmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (__any(lmax > m + kLazy)) {
      const float mn = fmaxf(m, col_max(lmax));
      scale(__builtin_amdgcn_exp2f(m - mn));
      m = mn;
    }
  }
};

// ------------------------------------------------------------- INT2 tile --
template <int D, int NG, int GQA>
struct I2Tile {
  using C = DC<D, NG, GQA>;
  uint32_t kw[C::SLOTS][C::KW];
  uint32_t vw[C::SLOTS][C::KW];
  uint32_t sc[8 * NG];  // own page's quad: K (s,z) x 4 tokens x NG, then V
  int nvalid;           // valid rows (a prefix) among this lane's 4 tokens
};

// Loads one tile: SLOTS consecutive logical pages of one KV head.  Code
// records of absent pages are read from physical page 0 (never used: their
// scales are zero and their logits -inf); scale words of tokens that are not
// history tokens are zeroed, so stale bits can never reach the arithmetic.
template <int D, int NG, int GQA>
__device__ __forceinline__ void i2_load(I2Tile<D, NG, GQA>& t, const DecodeParams& p,
                                        const int32_t* __restrict__ pt, const uint8_t* __restrict__ pool, int kvh,
                                        int tile_first, int page_end, int hist_len, int lane, int my_slot) {
  using C = DC<D, NG, GQA>;
  const int j = lane >> 4;
  const uint32_t rec_off = (uint32_t)lane * C::REC;
  int mine_id = -1;
  bool full = (tile_first + C::SLOTS) * kPage <= hist_len && tile_first + C::SLOTS <= page_end;
#pragma unroll
  for (int s = 0; s < C::SLOTS; ++s) {
    const int lp = tile_first + s;
    int id = -1;
    if (lp < page_end) id = pt[lp];
    const bool ok = id >= 0 && id < p.int2_num_pages;
    full = full && ok;
    if (s == my_slot) mine_id = ok ? id : -1;
    const uint8_t* blk = pool + ((size_t)(ok ? id : 0) * p.num_kv_heads + kvh) * C::BLK2;
    if constexpr (D == 128) {
      const uint4 x = *(const uint4*)(blk + rec_off);
      t.kw[s][0] = x.x;
      t.kw[s][1] = x.y;
      t.vw[s][0] = x.z;
      t.vw[s][1] = x.w;
    } else {
      const uint2 y = *(const uint2*)(blk + rec_off);
      t.kw[s][0] = y.x;
      t.vw[s][0] = y.y;
    }
  }
  const int base = (tile_first + my_slot) * kPage + 4 * j;
  const int nv = mine_id >= 0 ? min(max(hist_len - base, 0), 4) : 0;
  const uint4* sp =
      (const uint4*)(pool + ((size_t)max(mine_id, 0) * p.num_kv_heads + kvh) * C::BLK2 + 8 * D + j * 32 * NG);
  uint4 sx[2 * NG];
#pragma unroll
  for (int i = 0; i < 2 * NG; ++i) sx[i] = sp[i];
#pragma unroll
  for (int i = 0; i < 2 * NG; ++i) {
    t.sc[4 * i + 0] = sx[i].x;
    t.sc[4 * i + 1] = sx[i].y;
    t.sc[4 * i + 2] = sx[i].z;
    t.sc[4 * i + 3] = sx[i].w;
  }
  // lanes without a (slot, head) column exist only when SLOTS * GQA < 16
  const bool clean = C::COLS < 16 ? (!full || mine_id < 0) : !full;
  if (clean) {
    // word 4*i + e of the K (i < NG) and V (i >= NG) quads belongs to token
    // e / NG of this lane's quad
#pragma unroll
    for (int w = 0; w < 8 * NG; ++w)
      if ((w % (4 * NG)) / NG >= nv) t.sc[w] = 0u;
  }
  t.nvalid = nv;
}

// P.V operands from packed value codes, without per-code shifts.  A value
// word holds, for the lane's 4 tokens 4j+i and 4 channel blocks bb, the code
// at bits 16*(i&1) + 2*(2*bb + (i>>1)).  One shift by 4*bb - 6 bits puts the
// codes of tokens i = 0,1 at bits 6-7 of each 16-bit half and those of
// i = 2,3 at bits 8-9; OR-ing in an fp16 exponent then gives exact fp16
// values 16 + code (exponent 19) and 4 + code (exponent 17).  The biases 16
// and 4 are removed through the per-token correction sum Z.
template <int BB>
__device__ __forceinline__ uint32_t v_shift(uint32_t x) {
  if constexpr (BB == 0) return x << 6;
  if constexpr (BB == 1) return x << 2;
  if constexpr (BB == 2) return x >> 2;
  return x >> 6;
}
constexpr uint32_t kMaskLo = 0x00C000C0u, kExpLo = 0x4C004C00u;  // tokens i = 0,1: 16 + code
constexpr uint32_t kMaskHi = 0x03000300u, kExpHi = 0x44004400u;  // tokens i = 2,3: 4 + code
constexpr float kBiasLo = 16.f, kBiasHi = 4.f;

template <int D, int NG, int W0>
__device__ __forceinline__ void pv_block_pair(Acc<D, NG>& st, uint32_t x0, uint32_t x1, const v4i (&bw)[NG],
                                              uint32_t exp_lo, uint32_t exp_hi) {
  constexpr int G = D / NG;
  // the four channel blocks of this word pair, two pages per MFMA (k = 32)
  auto one = [&](auto bbc) {
    constexpr int BB = decltype(bbc)::value;
    constexpr int cblk = 4 * W0 + BB;
    constexpr int g = (cblk * 16) / G;
    const uint32_t y0 = v_shift<BB>(x0), y1 = v_shift<BB>(x1);
    const v4i a = {(int)((y0 & kMaskLo) | exp_lo), (int)((y0 & kMaskHi) | exp_hi), (int)((y1 & kMaskLo) | exp_lo),
                   (int)((y1 & kMaskHi) | exp_hi)};
    st.o[cblk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, bw[g]),
                                                        st.o[cblk], 0, 0, 0);
  };
  one(std::integral_constant<int, 0>{});
  one(std::integral_constant<int, 1>{});
  one(std::integral_constant<int, 2>{});
  one(std::integral_constant<int, 3>{});
}

// One INT2 tile.  Tokens outside the history (and every token of a lane
// whose column holds no (slot, head) pair) get logit -inf; their scale words
// are zero, so their weights are exactly zero.
template <int D, int NG, int GQA>
__device__ __forceinline__ void i2_compute(const I2Tile<D, NG, GQA>& t, Acc<D, NG>& st,
                                           const v4i (&bq)[DC<D, NG, GQA>::SLOTS][2][D / 64][64], float kappa,
                                           const float (&sig)[NG], int my_slot, int lane, uint32_t exp_lo,
                                           uint32_t exp_hi) {
  using C = DC<D, NG, GQA>;
  // the q' operands are read from LDS on every tile: an opaque lane index
  // keeps the compiler from hoisting them into 64 loop-invariant VGPRs
  asm volatile("" : "+v"(lane));
  // ---- scores on the int8 matrix cores
  v4i ca[NG], cb[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) ca[g] = cb[g] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < C::SLOTS; ++s) {
#pragma unroll
    for (int w = 0; w < C::KW; ++w) {
      const uint32_t x = t.kw[s][w];
      const v4i a = {(int)(x & 0x03030303u), (int)((x >> 2) & 0x03030303u), (int)((x >> 4) & 0x03030303u),
                     (int)((x >> 6) & 0x03030303u)};
      const int g = (NG == 1) ? 0 : w;
      const v4i b0 = bq[s][0][w][lane], b1 = bq[s][1][w][lane];
      ca[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b0, ca[g], 0, 0, 0);
      cb[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b1, cb[g], 0, 0, 0);
    }
  }
  // ---- logits (log2 domain)
  float lg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float sint = (float)(ca[g][i] * 256 + cb[g][i]);
      const uint32_t sz = t.sc[i * NG + g];
      acc += bf16_lo(sz) * (sint - bf16_hi(sz) * sig[g]);
    }
    lg[i] = fmaf(acc, kappa, i < t.nvalid ? 0.f : -INFINITY);
  }
  st.update_max(lg);
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(lg[i] - st.m);
  st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  // ---- fp16 weights w = p * s_V per group, and the correction
  //      Z += sum w * (bias + z) with the rounded weights
  v4i bw[C::SLOTS / 2][NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float w[4], zb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sz = t.sc[4 * NG + i * NG + g];
      w[i] = pr[i] * bf16_lo(sz);
      zb[i] = bf16_hi(sz) + (i < 2 ? kBiasLo : kBiasHi);
    }
    const h2 w01 = __builtin_convertvector(f2{w[0], w[1]}, h2);
    const h2 w23 = __builtin_convertvector(f2{w[2], w[3]}, h2);
    st.Z[g] += ((float)w01[0] * zb[0] + (float)w01[1] * zb[1]) + ((float)w23[0] * zb[2] + (float)w23[1] * zb[3]);
    const uint32_t u01 = __builtin_bit_cast(uint32_t, w01), u23 = __builtin_bit_cast(uint32_t, w23);
#pragma unroll
    for (int pp = 0; pp < C::SLOTS / 2; ++pp) {
      const bool m0 = my_slot == 2 * pp, m1 = my_slot == 2 * pp + 1;
      bw[pp][g] = v4i{(int)(m0 ? u01 : 0u), (int)(m0 ? u23 : 0u), (int)(m1 ? u01 : 0u), (int)(m1 ? u23 : 0u)};
    }
  }
  // ---- P.V on the fp16 matrix cores, two pages per MFMA
#pragma unroll
  for (int pp = 0; pp < C::SLOTS / 2; ++pp) {
    pv_block_pair<D, NG, 0>(st, t.vw[2 * pp][0], t.vw[2 * pp + 1][0], bw[pp], exp_lo, exp_hi);
    if constexpr (C::KW > 1) pv_block_pair<D, NG, 1>(st, t.vw[2 * pp][1], t.vw[2 * pp + 1][1], bw[pp], exp_lo, exp_hi);
  }
}

// ------------------------------------------------------------- BF16 tile --
template <int D, int GQA>
struct B16Tile {
  static constexpr int S = DC<D, 1, GQA>::SLOTS_B, KB = D / 32;
  uint4 k[S][KB];
  uint4 v[S][KB];
  int lp[S];  // logical page per slot, -1 when absent
};

// validity of position pos in a BF16 unit
struct B16Valid {
  int sink_end, r0, L;
  __device__ __forceinline__ bool operator()(int pos) const {
    return pos < sink_end || (pos >= r0 && pos < L);
  }
};

template <int D, int GQA>
__device__ __forceinline__ void b16_load(B16Tile<D, GQA>& t, const DecodeParams& p, const int32_t* __restrict__ pt,
                                         const uint8_t* __restrict__ pool, int kvh, int tile_first, int list_end,
                                         int n_sp, int first_rp, bool bf16_only, const B16Valid& valid, int lane) {
  using T = B16Tile<D, GQA>;
  const int j = lane >> 4, r = lane & 15;
#pragma unroll
  for (int s = 0; s < T::S; ++s) {
    const int li = tile_first + s;
    int lp = -1, id = -1;
    if (li < list_end) {
      lp = bf16_only ? li : (li < n_sp ? li : first_rp + (li - n_sp));
      id = pt[lp];
    }
    const bool ok = id >= 0 && id < p.bf16_num_pages;
    t.lp[s] = ok ? lp : -1;
    uint4 kx[T::KB], vx[T::KB];
#pragma unroll
    for (int q = 0; q < T::KB; ++q) kx[q] = vx[q] = uint4{0u, 0u, 0u, 0u};
    if (ok) {
      const uint8_t* blk = pool + ((size_t)id * p.num_kv_heads + kvh) * (64 * D);
      const uint4* kp = (const uint4*)(blk + r * 2 * D + j * (D / 2));
      const uint4* vp = (const uint4*)(blk + 32 * D + j * 8 * D + r * (D / 2));
#pragma unroll
      for (int q = 0; q < T::KB; ++q) {
        kx[q] = kp[q];
        vx[q] = vp[q];
      }
    }
    // zero tokens outside the sink / recent segments (stale or unwritten)
    const int p0 = lp * kPage;
    const bool partial = ok && !(valid(p0) && valid(p0 + kPage - 1));
    const bool kv_ok = !partial || valid(p0 + r);
    const uint32_t m01 = (!partial || valid(p0 + 4 * j) ? 0xFFFFu : 0u) |
                         (!partial || valid(p0 + 4 * j + 1) ? 0xFFFF0000u : 0u);
    const uint32_t m23 = (!partial || valid(p0 + 4 * j + 2) ? 0xFFFFu : 0u) |
                         (!partial || valid(p0 + 4 * j + 3) ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int q = 0; q < T::KB; ++q) {
      t.k[s][q] = kv_ok ? kx[q] : uint4{0u, 0u, 0u, 0u};
      t.v[s][q] = uint4{vx[q].x & m01, vx[q].y & m23, vx[q].z & m01, vx[q].w & m23};
    }
  }
}

template <int D, int GQA>
__device__ __forceinline__ void b16_compute(const B16Tile<D, GQA>& t, Acc<D, 1>& st,
                                            const v8bf (&bq)[DC<D, 1, GQA>::SLOTS_B][D / 32], float sm_log2,
                                            const B16Valid& valid, int my_slot, int lane) {
  using T = B16Tile<D, GQA>;
  const int j = lane >> 4;
  v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < T::S; ++s)
#pragma unroll
    for (int q = 0; q < T::KB; ++q) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(t.k[s][q]), bq[s][q], c, 0, 0, 0);
  int mlp = -1;
#pragma unroll
  for (int s = 0; s < T::S; ++s)
    if (s == my_slot) mlp = t.lp[s];
  float lg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = mlp >= 0 && valid(mlp * kPage + 4 * j + i);
    lg[i] = ok ? c[i] * sm_log2 : -INFINITY;
  }
  st.update_max(lg);
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(lg[i] - st.m);
  st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
#pragma unroll
  for (int s = 0; s < T::S; ++s) {
    const bool mine = (my_slot == s);
    const v4s bw = as_v4s(mine ? p01 : 0u, mine ? p23 : 0u);
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
      const uint4 x = t.v[s][e >> 1];
      const v4s a = (e & 1) ? as_v4s(x.z, x.w) : as_v4s(x.x, x.y);
      st.o[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bw, st.o[e], 0, 0, 0);
    }
  }
}

// -------------------------------------------------------- wave epilogue --
// Reduce a wave's column states to one (o, lse) per query head and store it
// in sm.part[wave].  INT2: channel of o[cb][i] is cb*16 + 4j + i and the
// numerator is acc - Z.  BF16: channel (4j + i) * D/16 + cb.
template <int D, int NG, int GQA, bool INT2>
__device__ __forceinline__ void wave_finish(Acc<D, NG>& st, Smem<D, GQA>& sm, int wave, int lane) {
  constexpr int G = D / NG;
  const int n = lane & 15, j = lane >> 4;
  st.l = col_sum(st.l);
#pragma unroll
  for (int g = 0; g < NG; ++g) st.Z[g] = col_sum(st.Z[g]);
  const float mh = slot_max<GQA>(st.m);
  st.scale(__builtin_amdgcn_exp2f(st.m - mh));
  st.l = slot_sum<GQA>(st.l);
#pragma unroll
  for (int g = 0; g < NG; ++g) st.Z[g] = slot_sum<GQA>(st.Z[g]);
#pragma unroll
  for (int cbk = 0; cbk < D / 16; ++cbk)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o[cbk][i] = slot_sum<GQA>(st.o[cbk][i]);
  if (n < GQA) {
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
#pragma unroll
    for (int cbk = 0; cbk < D / 16; ++cbk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float o;
        int c;
        if constexpr (INT2) {
          const int g = (cbk * 16) / G;
          o = (st.o[cbk][i] - st.Z[g]) * inv;
          c = cbk * 16 + 4 * j + i;
        } else {
          o = st.o[cbk][i] * inv;
          c = (4 * j + i) * (D / 16) + cbk;
        }
        sm.u.part[wave][n][c] = o;
      }
    }
    if (j == 0) sm.u.part[wave][n][D] = st.l > 0.f ? mh + __log2f(st.l) : -INFINITY;
  }
}

// ------------------------------------------------------------- kernel ----
template <int D, int NG, int GQA, bool BF16_ONLY>
__global__ void __launch_bounds__(kThreads)
    k_decode(const DecodeParams p, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ bf16_pt_all,
             const int32_t* __restrict__ int2_pt_all, const uint8_t* __restrict__ bf16_pool,
             const uint8_t* __restrict__ int2_pool, const uint16_t* __restrict__ qin, const float* __restrict__ r_k) {
  using C = DC<D, NG, GQA>;
  __shared__ Smem<D, GQA> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: page-table lookups then stay scalar loads and the
  // tile prefetch is never serialized behind a vector-memory wait
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int U = p.units_per_head;
  const int u = lin % U;
  const int kvh = (lin / U) % p.num_kv_heads;
  const int b = lin / (U * p.num_kv_heads);
  const int hq = p.num_kv_heads * GQA;

  int L = max(seq_lens[b], 0);
  L = min(L, kPage * p.bf16_pt_stride);
  if (!BF16_ONLY) L = min(L, p.sink + p.recent + kPage * p.int2_pt_stride);
  const int r0 = max(p.sink, L - p.recent);
  const int hist_len = BF16_ONLY ? 0 : r0 - p.sink;
  const int hist_pages = (hist_len + kPage - 1) / kPage;

  // ---- which pages this workgroup covers, and how many partials exist
  int total, first, end;
  bool int2_unit = false;
  const int n_sp = (min(L, p.sink) + kPage - 1) / kPage;
  const int first_rp = r0 / kPage;
  const int n_rp = r0 < L ? (L + kPage - 1) / kPage - first_rp : 0;
  if (BF16_ONLY) {
    const int npages = (L + kPage - 1) / kPage;
    const int chunks = max(1, min((npages + p.pages_per_chunk - 1) / p.pages_per_chunk, p.max_chunks));
    total = chunks;
    if (u >= chunks) return;
    first = u * p.pages_per_chunk;
    end = (u == chunks - 1) ? npages : min(first + p.pages_per_chunk, npages);
  } else {
    const int chunks = min((hist_pages + p.pages_per_chunk - 1) / p.pages_per_chunk, p.max_chunks);
    total = p.n_bf16_units + chunks;
    if (u < p.n_bf16_units) {
      const int nlist = n_sp + n_rp;
      first = u * p.bf16_pages_per_unit;
      end = (u == p.n_bf16_units - 1) ? nlist : min(first + p.bf16_pages_per_unit, nlist);
    } else {
      const int c = u - p.n_bf16_units;
      if (c >= chunks) return;
      int2_unit = true;
      first = c * p.pages_per_chunk;
      end = (c == chunks - 1) ? hist_pages : min(first + p.pages_per_chunk, hist_pages);
    }
  }

  if (!BF16_ONLY && int2_unit) {
    // ---------------------------------------------------- INT2 chunk unit
    const int my_slot = (n < C::COLS) ? n / GQA : C::SLOTS;
    const int ntiles = (end - first + C::SLOTS - 1) / C::SLOTS;
    const int32_t* __restrict__ ipt = int2_pt_all + (size_t)b * p.int2_pt_stride;
    // prologue: q' = q R_K on the bf16 matrix cores (R_K = R_hi + R_lo, both
    // bf16, so q' keeps ~2^-17 relative accuracy); wave w computes output
    // channels [16w, 16w + 16) for the query heads (MFMA rows) of this KV
    // head.  Its loads are issued before the first tiles' so that the
    // prologue runs while those are in flight.
    constexpr int KB = D / 32;
    uint4 qa[KB];
    float rv[KB][8];
    const bool qwave = wave < D / 16;
    if (qwave) {
      const uint16_t* qrow = qin + ((size_t)b * hq + kvh * GQA + (n < GQA ? n : 0)) * D;
      const float* rcol = r_k + (size_t)kvh * D * D + wave * 16 + n;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        qa[kb] = uint4{0u, 0u, 0u, 0u};
        if (n < GQA) qa[kb] = *(const uint4*)(qrow + kb * 32 + j * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) rv[kb][e] = rcol[(size_t)(kb * 32 + j * 8 + e) * D];
      }
    }
    // prefetch ring: tile wave + r*kWaves in slot r; tiles past the last one
    // load nothing but are fully initialized, so the buffers stay in VGPRs
    I2Tile<D, NG, GQA> ring[kRing];
    auto ld = [&](I2Tile<D, NG, GQA>& t, int tl) {
      i2_load<D, NG, GQA>(t, p, ipt, int2_pool, kvh, first + tl * C::SLOTS, tl < ntiles ? end : 0, hist_len, lane,
                          my_slot);
    };
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r) ld(ring[r], wave + r * kWaves);
    if (qwave) {
      v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = rv[kb][2 * e], x1 = rv[kb][2 * e + 1];
          hi[e] = pack_bf16x2(x0, x1);
          lo[e] = pack_bf16x2(x0 - bf16_lo(hi[e]), x1 - bf16_hi(hi[e]));
        }
        const v8bf av = as_v8bf(qa[kb]);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_v8bf(uint4{hi[0], hi[1], hi[2], hi[3]}), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_v8bf(uint4{lo[0], lo[1], lo[2], lo[3]}), c, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * j + i < GQA) sm.qr[(4 * j + i) * D + wave * 16 + n] = c[i];
    }
    __syncthreads();
    float amax = 0.f;
    for (int idx = tid; idx < GQA * D; idx += kThreads) amax = fmaxf(amax, fabsf(sm.qr[idx]));
    amax = wave_max(amax);
    if (lane == 0) sm.wred[wave] = amax;
    __syncthreads();
    amax = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, sm.wred[w]);
    const float sq = amax > 0.f ? amax / 127.f : 1.f;
    const float inv_sq = 1.f / sq;
    for (int idx = tid; idx < GQA * D; idx += kThreads) {
      const float x = sm.qr[idx] * inv_sq;
      const float a = fminf(fmaxf(rintf(x), -127.f), 127.f);
      const float bt = fminf(fmaxf(rintf((x - a) * 256.f), -127.f), 127.f);
      sm.ta[idx] = (int8_t)a;
      sm.tb[idx] = (int8_t)bt;
    }
    __syncthreads();
    for (int pair = wave; pair < GQA * NG; pair += kWaves) {
      const int h = pair / NG, g = pair % NG;
      int sacc = 0;
      for (int c = lane; c < C::G; c += 64) {
        const int idx = h * D + g * C::G + c;
        sacc += 256 * (int)sm.ta[idx] + (int)sm.tb[idx];
      }
      sacc = wave_sum_i(sacc);
      if (lane == 0) sm.sig[pair] = sacc;
    }
    // B operands: column n = (page slot, head), block-diagonal over slots;
    // every wave needs the same per-lane values, wave 0 builds them
    const int chd = n % GQA;
    if (wave == 0) {
#pragma unroll
      for (int s = 0; s < C::SLOTS; ++s)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int w = 0; w < C::KW; ++w) {
            uint32_t o4[4] = {0u, 0u, 0u, 0u};
            if (my_slot == s) {
              const int8_t* src = (tt == 0 ? sm.ta : sm.tb) + chd * D + w * 64 + j * 16;
              const uint4 x = *(const uint4*)src;
              const uint32_t in4[4] = {x.x, x.y, x.z, x.w};
              transpose4x4(in4, o4);
            }
            sm.bq[s][tt][w][lane] = v4i{(int)o4[0], (int)o4[1], (int)o4[2], (int)o4[3]};
          }
    }
    __syncthreads();
    float sig[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sig[g] = (float)sm.sig[chd * NG + g];
    const float kappa = p.sm_log2 * sq * (1.f / 256.f);
    // fp16 exponent patterns of the P.V operands, held in VGPRs so that each
    // operand is one and-or (bitop3) of a shifted code word
    uint32_t exp_lo = kExpLo, exp_hi = kExpHi;
    asm volatile("" : "+v"(exp_lo), "+v"(exp_hi));

    Acc<D, NG> st;
    st.init();
    int tile = wave;
    while (true) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        if (tile >= ntiles) break;
        ld(ring[(r + kRing - 1) % kRing], tile + (kRing - 1) * kWaves);
        i2_compute<D, NG, GQA>(ring[r], st, sm.bq, kappa, sig, my_slot, lane, exp_lo, exp_hi);
        tile += kWaves;
      }
      if (tile >= ntiles) break;
    }
    wave_finish<D, NG, GQA, true>(st, sm, wave, lane);
  } else {
    // ------------------------------------------- BF16 unit (sink + recent)
    constexpr int SB = C::SLOTS_B;
    const int my_slot = (n < C::COLS_B) ? n / GQA : SB;
    const B16Valid valid{BF16_ONLY ? L : min(L, p.sink), BF16_ONLY ? L : r0, L};
    // q (unrotated, bf16) as B operands
    v8bf bq[SB][D / 32];
    {
      const uint16_t* qh = qin + ((size_t)b * hq + kvh * GQA + (n % GQA)) * D + j * (D / 4);
#pragma unroll
      for (int s = 0; s < SB; ++s)
#pragma unroll
        for (int q = 0; q < D / 32; ++q) {
          uint4 x = uint4{0u, 0u, 0u, 0u};
          if (my_slot == s) x = *(const uint4*)(qh + q * 8);
          bq[s][q] = as_v8bf(x);
        }
    }
    const int ntiles = (end - first + SB - 1) / SB;
    Acc<D, 1> st;
    st.init();
    const int32_t* __restrict__ bpt = bf16_pt_all + (size_t)b * p.bf16_pt_stride;
    int tile = wave;
    B16Tile<D, GQA> cur;
    b16_load<D, GQA>(cur, p, bpt, bf16_pool, kvh, first + tile * SB, tile < ntiles ? end : 0, n_sp, first_rp,
                     BF16_ONLY, valid, lane);
    while (tile < ntiles) {
      const int nxt = tile + kWaves;
      B16Tile<D, GQA> nt;
      b16_load<D, GQA>(nt, p, bpt, bf16_pool, kvh, first + nxt * SB, nxt < ntiles ? end : 0, n_sp, first_rp,
                       BF16_ONLY, valid, lane);
      b16_compute<D, GQA>(cur, st, bq, p.sm_log2, valid, my_slot, lane);
      cur = nt;
      tile = nxt;
    }
    Acc<D, NG> st2;  // widen to the common epilogue type
    if constexpr (NG == 1) {
      st2 = st;
    } else {
#pragma unroll
      for (int i = 0; i < D / 16; ++i) st2.o[i] = st.o[i];
      st2.m = st.m;
      st2.l = st.l;
#pragma unroll
      for (int g = 0; g < NG; ++g) st2.Z[g] = 0.f;
    }
    wave_finish<D, NG, GQA, false>(st2, sm, wave, lane);
  }
  __syncthreads();

  // ---- merge the waves' partials into this workgroup's partial
  const size_t head_base = (size_t)b * p.num_kv_heads + kvh;
  const size_t pidx = (head_base * U + u) * GQA;
  for (int idx = tid; idx < GQA * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.u.part[w][h][D]);
    float o = 0.f, lse = -INFINITY;
    if (mx > -INFINITY) {
      float sw = 0.f, so = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float e = __builtin_amdgcn_exp2f(sm.u.part[w][h][D] - mx);
        sw += e;
        so += e * sm.u.part[w][h][c];
      }
      o = so / sw;
      lse = (mx + __log2f(sw)) * kLn2;
    }
    p.part_o[(pidx + h) * D + c] = o;
    if (c == 0) p.part_lse[pidx + h] = lse;
  }
  // ---- last workgroup of this (sequence, KV head) merges every partial.
  // Every wave drains its partial stores to L2 (s_waitcnt vmcnt(0)); then one
  // thread releases at device scope (L2 write-back) and takes a ticket; the
  // workgroup that takes the last ticket acquires and reads all partials.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(p.counters + head_base, 1u, __ATOMIC_RELEASE,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (uint32_t)(total - 1);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sm.last = last;
  }
  __syncthreads();
  if (!sm.last) return;
  const size_t p0 = head_base * U * GQA;
  // weights exp(lse_u - M_h) / sum_u exp(lse_u - M_h), in sm.u.wts[u * GQA + h]
  for (int h = wave; h < GQA; h += kWaves) {
    float mx = -INFINITY;
    for (int uu = lane; uu < total; uu += 64) mx = fmaxf(mx, p.part_lse[p0 + (size_t)uu * GQA + h]);
    mx = wave_max(mx);
    float sw = 0.f;
    for (int uu = lane; uu < total; uu += 64) {
      const float e = (mx > -INFINITY) ? expf(p.part_lse[p0 + (size_t)uu * GQA + h] - mx) : 0.f;
      sm.u.wts[uu * GQA + h] = e;
      sw += e;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sw += __shfl_xor(sw, o);
    const float inv = sw > 0.f ? 1.f / sw : 0.f;
    for (int uu = lane; uu < total; uu += 64) sm.u.wts[uu * GQA + h] *= inv;
  }
  __syncthreads();
  for (int idx = tid; idx < GQA * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    const float* src = p.part_o + (p0 + h) * D + c;  // partial u at src[u * GQA * D]
    float acc = 0.f;
    int uu = 0;
    for (; uu + 16 <= total; uu += 16) {  // 16 independent loads in flight
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = src[(size_t)(uu + k) * GQA * D];
#pragma unroll
      for (int k = 0; k < 16; ++k) acc += sm.u.wts[(uu + k) * GQA + h] * v[k];
    }
    for (; uu < total; ++uu) acc += sm.u.wts[uu * GQA + h] * src[(size_t)uu * GQA * D];
    p.out[((size_t)b * hq + kvh * GQA + h) * D + c] = (uint16_t)f32_to_bf16(acc);
  }
  if (tid == 0) __hip_atomic_store(p.counters + head_base, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------- oscar_merge --
template <int D>
__global__ void __launch_bounds__(256) k_merge(const MergeParams p) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.rows) return;
  const int a = p.row_offsets[row], e = p.row_offsets[row + 1];
  float mx = -INFINITY;
  for (int i = a + lane; i < e; i += 64) mx = fmaxf(mx, p.lse[i]);
  mx = wave_max(mx);
  constexpr int PER = D / 64;
  float acc[PER] = {};
  float sw = 0.f;
  if (mx > -INFINITY) {
    for (int i = a; i < e; ++i) {
      const float w = expf(p.lse[i] - mx);
      sw += w;
#pragma unroll
      for (int q = 0; q < PER; ++q) acc[q] += w * p.o[(size_t)i * D + lane * PER + q];
    }
  }
  const float inv = sw > 0.f ? 1.f / sw : 0.f;
#pragma unroll
  for (int q = 0; q < PER; ++q) p.out[(size_t)row * D + lane * PER + q] = (uint16_t)f32_to_bf16(acc[q] * inv);
}

template <int D, int NG, int GQA>
bool launch_decode_t(const DecodeParams& p, bool bf16_only, int grid, hipStream_t stream) {
  if (bf16_only)
    hipLaunchKernelGGL((k_decode<D, NG, GQA, true>), dim3(grid), dim3(kThreads), 0, stream, p, p.seq_lens, p.bf16_pt,
                       p.int2_pt, p.bf16_pool, p.int2_pool, p.q, p.r_k);
  else
    hipLaunchKernelGGL((k_decode<D, NG, GQA, false>), dim3(grid), dim3(kThreads), 0, stream, p, p.seq_lens, p.bf16_pt,
                       p.int2_pt, p.bf16_pool, p.int2_pool, p.q, p.r_k);
  return true;
}

}  // namespace

bool launch_decode(const DecodeParams& p, int head_dim, int n_groups, int gqa, bool bf16_only, int grid,
                   hipStream_t stream) {
#define OSCAR_DEC(D, NG, G) \
  if (head_dim == D && n_groups == NG && gqa == G) return launch_decode_t<D, NG, G>(p, bf16_only, grid, stream);
  OSCAR_DEC(128, 1, 2)
  OSCAR_DEC(128, 1, 4)
  OSCAR_DEC(128, 1, 8)
  OSCAR_DEC(128, 2, 2)
  OSCAR_DEC(128, 2, 4)
  OSCAR_DEC(128, 2, 8)
  OSCAR_DEC(64, 1, 2)
  OSCAR_DEC(64, 1, 4)
  OSCAR_DEC(64, 1, 8)
#undef OSCAR_DEC
  return false;
}

bool launch_merge(const MergeParams& p, hipStream_t stream) {
  const int grid = (p.rows + 3) / 4;
  if (grid == 0) return true;
  if (p.head_dim == 128)
    hipLaunchKernelGGL(k_merge<128>, dim3(grid), dim3(256), 0, stream, p);
  else if (p.head_dim == 64)
    hipLaunchKernelGGL(k_merge<64>, dim3(grid), dim3(256), 0, stream, p);
  else
    return false;
  return true;
}

}  // namespace oscar
