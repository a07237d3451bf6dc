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
//           workgroup in fp32 and split, per query head, into two int8 terms,
//           q' ~ sq (a + b/256), so the integer dot is exact and q' carries
//           ~16 significant bits.
//           With the key dequantization k' = s (code - z) the logit is
//           sm * s * sq/256 * (S_ab - z * sum(256 a + b)).
//   P.V     on the fp16 matrix cores.  The value codes become exact fp16
//           operands bias + code (bias 16 or 4, set by OR-ing an exponent
//           into the shifted code bits) and the weights w = p * s_V are
//           fp16:  sum w (code - z) = sum w (bias + code) - sum w (bias + z),
//           the second sum tracked from the same rounded weights.
//   softmax online, with a lazy running max (rescale only when a logit
//           exceeds the running max by more than 2^8).
// The GQA query heads of a KV head share every loaded page; the 16 columns
// of each MFMA tile hold (page slot, query head) pairs, so one score tile
// covers SLOTS pages and all softmax arithmetic is shared across them.
// Each wave keeps a ring of tiles in flight and is software-pipelined: the
// score MFMAs of tile i+1 are issued next to the softmax and P.V work of
// tile i, so matrix-core and vector work of one wave overlap.
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
#define OSCAR_DECODE_RING 3
#endif
#ifndef OSCAR_BF16_SLOTS
#define OSCAR_BF16_SLOTS 2
#endif
constexpr int kWaves = OSCAR_DECODE_WAVES;  // waves per workgroup
constexpr int kRing = OSCAR_DECODE_RING;    // INT2 tiles held per wave (ring of loads in flight)
constexpr int kThreads = 64 * kWaves;
constexpr float kNegBig = -1.0e30f;  // finite "no token yet" running max
constexpr float kLazy = 8.0f;        // log2 slack before the running max is raised
// History pages are read exactly once per step: their code and scale words
// are loaded non-temporal (cache policy bit NT), so that they do not push
// the page tables, R_K and q out of L2 (measured 0.5 us faster per
// 100K-token step, 8 % at 32 x 32K, than with the default policy).  BF16
// pages keep the default policy: their lanes read 16-byte pieces of lines
// that the next loads of the same lanes use: NT loads there measured 1.6x
// slower for the BF16-only kernel and 0.9 us slower for the 100K-token step.
constexpr int kKvPolicy = 2;
// Phase timeline of the profiling build.  Point k of wave w of logical
// workgroup lin lands in stamps[(lin * kWaves + w) * kStampSlots + k]:
// 0 start, 1 first tiles requested, 2 q' partials ready, 3 q' split
// barrier, 4 first score MFMAs issued, 5 loop end, 6 wave merge barrier,
// 7 partial stores acknowledged, 8 ticket taken, 9 fold written (last
// workgroup only), 10: 1 for the workgroup that folded, 11 q' FMAs done
// (R_K arrived), 12 q' split written (waves of the query heads only).
// Empty otherwise.
struct PhaseStamps {
#if OSCAR_PHASE_STAMPS
  uint64_t t[kStampSlots];
  __device__ __forceinline__ PhaseStamps() {
#pragma unroll
    for (int k = 0; k < kStampSlots; ++k) t[k] = 0;
  }
  __device__ __forceinline__ void at(int k) { t[k] = __builtin_amdgcn_s_memrealtime(); }
  __device__ __forceinline__ void set(int k, uint64_t v) { t[k] = v; }
  __device__ __forceinline__ void flush(uint64_t* dst, int lin, int wave, int lane) const {
    if (dst && lin < kStampWgs && lane == 0)
#pragma unroll
      for (int k = 0; k < kStampSlots; ++k) dst[((size_t)lin * kWaves + wave) * kStampSlots + k] = t[k];
  }
#else
  __device__ __forceinline__ void at(int) {}
  __device__ __forceinline__ void set(int, uint64_t) {}
  __device__ __forceinline__ void flush(uint64_t*, int, int, int) const {}
#endif
};
static_assert(kWaves == kStampWaves, "stamp area sized for the decode workgroup");

__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const u4v x = __builtin_nontemporal_load((const u4v*)p);
  return uint4{x[0], x[1], x[2], x[3]};
}

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
    struct {
      float part[kWaves][GQA][D + 1];  // per-wave partials, [D] = lse (log2)
      float raw[kWaves][16][D + 4];    // INT2 epilogue: a wave's accumulators per column
      float lz[kWaves][16][4];         // INT2 epilogue: per column l, Z[0], Z[1], reference
    } f;
    float qpart[kWaves][GQA][D];  // prologue: per-wave partial sums of q R_K
  } u;
  v4i bq[SLOTS][3][D / 64][64];      // int8 q' B operands per lane (terms a, b, c; shared by the waves)
  float kap[GQA];                    // logit factor sm * log2(e) * sq / 256 per query head
  float kap3[GQA];                   // the same with the third term: sm * log2(e) * sq / 65536
  int sig[GQA * 2];                  // sum(256 a + b) per head and group
  int sig3[GQA * 2];                 // sum(65536 a + 256 b + c) per head and group
  int dom[GQA];                      // 1: the head's q' has a dominant channel (three terms)
  int last;
  uint32_t qsync;                    // q' partials written (waves of the q' prologue)
};

// ---------------------------------------------------------------- helpers --
// Cross-lane reductions without LDS: DPP row rotations inside each 16-lane
// row, then the gfx950 permlane swaps, which exchange rows 0<->1, 2<->3
// (lane l meets l^16) and the two 32-lane halves (lane l meets l^32).
__device__ __forceinline__ uint32_t as_u(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float xor16_add(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int xor16_add(int x) {
  const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)r[0] + (int)r[1];
}
__device__ __forceinline__ int xor32_add(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)r[0] + (int)r[1];
}
template <int N>
__device__ __forceinline__ int dpp_row_ror_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x120 + N, 0xF, 0xF, false);
}
// every lane receives the reduction over its 16-lane row
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_row_ror<8>(x));
  x = fmaxf(x, dpp_row_ror<4>(x));
  x = fmaxf(x, dpp_row_ror<2>(x));
  return fmaxf(x, dpp_row_ror<1>(x));
}
__device__ __forceinline__ int row_sum_i(int x) {
  x += dpp_row_ror_i<8>(x);
  x += dpp_row_ror_i<4>(x);
  x += dpp_row_ror_i<2>(x);
  return x + dpp_row_ror_i<1>(x);
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_row_ror<8>(x);
  x += dpp_row_ror<4>(x);
  x += dpp_row_ror<2>(x);
  return x + dpp_row_ror<1>(x);
}
// every lane receives the reduction over the wave
__device__ __forceinline__ float wave_max(float x) { return xor32_max(xor16_max(row_max(x))); }
// lane 0's reduction order, the same value in every lane
__device__ __forceinline__ float wave_sum(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(xor32_add(xor16_add(row_sum(x))))));
}
__device__ __forceinline__ int wave_sum_i(int x) { return xor32_add(xor16_add(row_sum_i(x))); }
// over one 32-lane half
__device__ __forceinline__ int half_sum_i(int x) { return xor16_add(row_sum_i(x)); }
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
// over the 4 lane groups j (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float col_sum(float x) { return xor32_add(xor16_add(x)); }
__device__ __forceinline__ float col_max(float x) { return xor32_max(xor16_max(x)); }
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
// online-softmax state of one wave: accumulators O^T[channel][column]
//
// The weights are p = 2^(logit - ref) with ref = m + E.  m is the lazy
// running max of the logits (log2 units).  E (INT2 units only; 0 for BF16)
// is an integer exponent that follows the largest value scale s_V seen, so
// that the fp16 P.V weights w = p s_V stay inside fp16's normal range for
// any scale in [2^kEmin, 2^kEmax]: p <= 2^kLazy and s_V <= 2^(E + kSlack)
// give w <= 2^(kLazy + kSlack).  Numerator and denominator carry the same
// factor 2^-E, so the normalized output needs no correction and the
// partial's log2 normalizer is ref + log2(l).
constexpr float kSlack = 4.f;   // log2 slack of a value scale above 2^E before E is raised
constexpr float kEmin = -96.f, kEmax = 96.f;
template <int D, int NG>
struct Acc {
  v4f o[D / 16];
  float m, l;
  float E, ref, slim;  // value-scale exponent, exp2 reference m + E, 2^(E + kSlack)
  float Z[NG];  // INT2 only: sum over tokens of weight * (operand bias + zero)
  __device__ void init(bool int2) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};
    m = kNegBig;
    l = 0.f;
    E = int2 ? kEmin : 0.f;
    ref = m + E;
    slim = int2 ? __builtin_amdgcn_ldexpf(1.f, (int)(kEmin + kSlack)) : INFINITY;
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
  // new reference from the (already reduced) logit max mn and value-scale
  // max sm of the columns that share this state
  __device__ __forceinline__ void raise(float mn, float sm) {
    const float En = sm > slim ? fminf((float)(__builtin_amdgcn_frexp_expf(sm) - 1), kEmax) : E;
    const float rn = mn + En;
    scale(__builtin_amdgcn_exp2f(ref - rn));
    m = mn;
    E = En;
    ref = rn;
    slim = __builtin_amdgcn_ldexpf(1.f, (int)(En + kSlack));
  }
  // INT2 prefix tiles (two pages, every column its own state): lazy raise
  // when a logit exceeds m by kLazy or a value scale exceeds slim
  __device__ __forceinline__ void update_ref(const float lg[4], const float lg2[4], float smax) {
    const float lmax = fmaxf(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])),
                             fmaxf(fmaxf(lg2[0], lg2[1]), fmaxf(lg2[2], lg2[3])));
    if (__any(lmax > m + kLazy || smax > slim)) raise(fmaxf(m, col_max(lmax)), col_max(smax));
  }
  // INT2 tiles of k_decode: the columns n, n + SHARE, n + 2 SHARE, ... of a
  // 16-lane row (the pages of one query head) keep one state reference, so
  // that their states merge without rescaling
  template <int SHARE>
  __device__ __forceinline__ void update_ref(const float lg[4], float smax) {
    const float lmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (__any(lmax > m + kLazy || smax > slim))
      raise(slot_max<SHARE>(fmaxf(m, col_max(lmax))), slot_max<SHARE>(col_max(smax)));
  }
  // BF16 tiles (E = 0): the logit max alone
  template <int SHARE>
  __device__ __forceinline__ void update_max(const float lg[4]) {
    const float lmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (__any(lmax > m + kLazy)) {
      const float mn = slot_max<SHARE>(fmaxf(m, col_max(lmax)));
      scale(__builtin_amdgcn_exp2f(m - mn));
      m = mn;
      ref = mn;
    }
  }
};

// ------------------------------------------------------ q' int8 split ----
// q' of one query head, lane holding channels CPL*lane + e, split as
// q' ~ sq (a + b/256 + c/65536) with int8 a, b, c (sq = max|q'| / 127), so
// that its dot with the int8 key codes is exact on the matrix cores.  Two
// terms carry ~16 significant bits relative to max|q'|, which leaves the
// other channels enough bits unless one channel dominates; `dom` (the same
// in every lane) is set when max|q'| exceeds kDominant times the rms over the
// channels, and the kernels then add the third term.
constexpr float kDominant = 8.f;

// An LDS read that the compiler re-issues where it stands (a volatile access
// through an LDS pointer): loop-invariant operands read this way are not
// hoisted into registers for the whole loop.
typedef __attribute__((address_space(3))) v4i lds_v4i;
__device__ __forceinline__ v4i lds_read_fresh(const v4i* p) {
  return *(volatile const lds_v4i*)(const lds_v4i*)p;
}
template <int CPL>
__device__ __forceinline__ float split_query(const float (&x)[CPL], int (&a)[CPL], int (&b)[CPL], int (&c)[CPL],
                                             bool& dom) {
  float amax = 0.f, ss = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    amax = fmaxf(amax, fabsf(x[e]));
    ss = fmaf(x[e], x[e], ss);
  }
  amax = wave_max(amax);
  ss = wave_sum(ss);
  dom = amax * amax > kDominant * kDominant * ss * (1.f / (64 * CPL));
  // sq and its reciprocal need not be correctly rounded: the terms are
  // formed from y = x / sq (to within 1 ulp) and the dot is scaled by sq
  // itself, so only the rounding of the terms enters the result
  const float sq = amax > 0.f ? amax * (1.f / 127.f) : 1.f;
  const float inv_sq = __builtin_amdgcn_rcpf(sq);
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const float y = x[e] * inv_sq;
    const float af = fminf(fmaxf(rintf(y), -127.f), 127.f);
    const float r1 = (y - af) * 256.f;  // exact: af is the integer nearest y
    const float bf = fminf(fmaxf(rintf(r1), -127.f), 127.f);
    const float cf = fminf(fmaxf(rintf((r1 - bf) * 256.f), -127.f), 127.f);
    a[e] = (int)af;
    b[e] = (int)bf;
    c[e] = (int)cf;
  }
  return sq;
}

// ------------------------------------------------------------- INT2 tile --
template <int D, int NG, int GQA>
struct I2Tile {
  using C = DC<D, NG, GQA>;
  uint32_t kw[C::SLOTS][C::KW];
  uint32_t vw[C::SLOTS][C::KW];
  uint32_t sc[8 * NG];  // own page's quad: K (s,z) x 4 tokens x NG, then V
  int nvalid;           // valid rows (a prefix) among this lane's 4 tokens
  // keeps every register of the tile live (and in place) up to this point:
  // the registers of a ring slot are then never reused as temporaries while
  // the slot waits for its next load
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int s = 0; s < C::SLOTS; ++s)
#pragma unroll
      for (int w = 0; w < C::KW; ++w) asm volatile("" : "+v"(kw[s][w]), "+v"(vw[s][w]));
#pragma unroll
    for (int w = 0; w < 8 * NG; ++w) asm volatile("" : "+v"(sc[w]));
    asm volatile("" : "+v"(nvalid));
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < C::SLOTS; ++s)
#pragma unroll
      for (int w = 0; w < C::KW; ++w) kw[s][w] = vw[s][w] = 0u;
#pragma unroll
    for (int w = 0; w < 8 * NG; ++w) sc[w] = 0u;
    nvalid = 0;
  }
};

// Loads one tile: SLOTS consecutive logical history pages of one KV head,
// starting at logical page lp0.  The physical ids come from lanes idx0 ..
// idx0+SLOTS-1 of `pids` (-1 = absent; idx0 < 0: no page at all), so every
// code address is a uniform base plus the lane's record offset.  Code records
// of absent pages are not read (a zero-size buffer descriptor returns zeros);
// their scale words are read from physical page 0 and, like those of tokens
// that are not history tokens, zeroed, so stale bits can never reach the
// arithmetic (an absent page's logits are -inf).
template <int D, int NG, int GQA>
__device__ __forceinline__ void i2_fetch(I2Tile<D, NG, GQA>& t, const uint8_t* __restrict__ hpool,
                                         size_t page_bytes, int pids, int idx0, int lp0, int hist_len, int my_slot,
                                         int lane) {
  using C = DC<D, NG, GQA>;
  const int j = lane >> 4;
  int ids[C::SLOTS];
  bool full = (lp0 + C::SLOTS) * kPage <= hist_len;
  const int i0 = idx0 >= 0 ? idx0 : 0;
#pragma unroll
  for (int s = 0; s < C::SLOTS; ++s) {
    const int v = __builtin_amdgcn_readlane(pids, i0 + s);
    ids[s] = idx0 >= 0 ? v : -1;
    full = full && ids[s] >= 0;
  }
  int mine = -1;
#pragma unroll
  for (int s = 0; s < C::SLOTS; ++s)
    if (s == my_slot) mine = ids[s];
  // code records: one buffer descriptor per page (scalar registers), the
  // lane's record offset as the only per-lane address term
#pragma unroll
  for (int s = 0; s < C::SLOTS; ++s) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(hpool + (size_t)max(ids[s], 0) * page_bytes), (short)0, ids[s] >= 0 ? C::BLK2 : 0, kBufferFlags);
    if constexpr (D == 128) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * C::REC, 0, kKvPolicy);
      t.kw[s][0] = x[0];
      t.kw[s][1] = x[1];
      t.vw[s][0] = x[2];
      t.vw[s][1] = x[3];
    } else {
      const auto y = __builtin_amdgcn_raw_buffer_load_b64(rs, lane * C::REC, 0, kKvPolicy);
      t.kw[s][0] = y[0];
      t.vw[s][0] = y[1];
    }
  }
  const int base = (lp0 + my_slot) * kPage + 4 * j;
  const int nv = mine >= 0 ? min(max(hist_len - base, 0), 4) : 0;
  const uint4* sp = (const uint4*)(hpool + (size_t)max(mine, 0) * page_bytes + 8 * D + j * 32 * NG);
  uint4 sx[2 * NG];
#pragma unroll
  for (int i = 0; i < 2 * NG; ++i) sx[i] = nt_load(sp + i);
#pragma unroll
  for (int i = 0; i < 2 * NG; ++i) {
    t.sc[4 * i + 0] = sx[i].x;
    t.sc[4 * i + 1] = sx[i].y;
    t.sc[4 * i + 2] = sx[i].z;
    t.sc[4 * i + 3] = sx[i].w;
  }
  // lanes without a (slot, head) column exist only when SLOTS * GQA < 16
  const bool clean = C::COLS < 16 ? (!full || mine < 0) : !full;
  if (clean) {
    // word 4*i + e of the K (i < NG) and V (i >= NG) quads belongs to token
    // e / NG of this lane's quad
#pragma unroll
    for (int w = 0; w < 8 * NG; ++w)
      if ((w % (4 * NG)) / NG >= nv) t.sc[w] = 0u;
  }
  t.nvalid = nv;
}

// The 2-bit K codes of a record word as int8 operands: code c of channel
// 4b + k sits in byte 4k + b of component k; with a codebook each byte
// becomes 32 L[c] by one byte permute.
template <bool LUT>
__device__ __forceinline__ v4i k_operand(uint32_t x, uint32_t lut_k) {
  v4i a = {(int)(x & 0x03030303u), (int)((x >> 2) & 0x03030303u), (int)((x >> 4) & 0x03030303u),
           (int)((x >> 6) & 0x03030303u)};
  if constexpr (LUT) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = (int)__builtin_amdgcn_perm(lut_k, lut_k, (uint32_t)a[k]);
  }
  return a;
}

template <int NG>
struct I2Scores {
  v4i a[NG], b[NG], c[NG];  // integer dots with the int8 terms of q', per group (c: three-term mode)
};

// the integer dot of a score row as a float: 256 S_a + S_b (exact), or with
// the third term 65536 S_a + 256 S_b + S_c (rounded once to fp32)
template <bool T3>
__device__ __forceinline__ float score_int(int sa, int sb, int sc) {
  if constexpr (T3) return fmaf((float)sa, 65536.f, fmaf((float)sb, 256.f, (float)sc));
  return (float)(sa * 256 + sb);
}

// P.V operands from packed value codes as fp16 subnormals.  A value word
// holds, for the lane's 4 tokens 4j+i and 4 channel blocks bb, the code at
// bits 16*(i&1) + 2*(2*bb + (i>>1)).  A 2-bit code masked in place at bit p
// of a 16-bit half (exponent field zero) is the exact fp16 subnormal
// code * 2^(p-24), and the matrix cores take subnormal operands exactly.
// Blocks 0 and 1 take their codes from the word itself, blocks 2 and 3 from
// the word shifted right by 8, so the codes of tokens i = 0,1 sit at
// p = 4 (bb & 1) and those of i = 2,3 two bits higher; the weights of tokens
// i = 2,3 enter the B operand divided by 4, and block bb's accumulator holds
// sum w * code * 2^(4 (bb & 1) - 24), scaled back once in the epilogue.  The
// zero-point term sum w * z is tracked in Z from the same rounded weights.
constexpr uint32_t kSubMask = 0x00030003u;  // tokens i = 0,1 of an even block
constexpr float kHiWeight = 0.25f;           // weight factor of tokens i = 2,3
// 2^(24 - 4 (cblk & 1)): accumulator of channel block cblk to code units
__device__ __forceinline__ constexpr float pv_unit_inv(int cblk) { return (cblk & 1) ? 1048576.f : 16777216.f; }
constexpr float kBiasLut = 16.f;  // codebook operands: 16 + L[code]

// With a codebook every operand is 16 + L[code] (bias 16 for all tokens):
// the fp16 pattern 0x4C00 | 64 L[code], built by one byte permute per
// operand word from the shifted codes (selector 4 picks the 0x4C byte).
constexpr uint32_t kLutHigh = 0x4C4C4C4Cu, kLutSel = 0x04000400u;
template <int BB, int I>
__device__ __forceinline__ uint32_t lut_operand(uint32_t x, uint32_t lut_v) {
  // selector (x >> shift) & 0x00030003 | kLutSel in one three-input bit
  // operation (truth table 0xEA: (a & b) | c)
  const uint32_t sel = __builtin_amdgcn_bitop3_b32(x >> (4 * BB + 2 * I), 0x00030003u, kLutSel, 0xEA);
  return __builtin_amdgcn_perm(kLutHigh, lut_v, sel);
}

template <int D, int NG, int W0, bool LUT>
__device__ __forceinline__ void pv_block_pair(Acc<D, NG>& st, uint32_t x0, uint32_t x1, const v4i (&bw)[NG],
                                              uint32_t lut_v) {
  constexpr int G = D / NG;
  const uint32_t s0 = x0 >> 8, s1 = x1 >> 8;  // codes of blocks 2 and 3
  // the four channel blocks of this word pair, two pages per MFMA (k = 32)
  auto one = [&](auto bbc) {
    constexpr int BB = decltype(bbc)::value;
    constexpr int cblk = 4 * W0 + BB;
    constexpr int g = (cblk * 16) / G;
    v4i a;
    if constexpr (LUT) {
      a = v4i{(int)lut_operand<BB, 0>(x0, lut_v), (int)lut_operand<BB, 1>(x0, lut_v),
              (int)lut_operand<BB, 0>(x1, lut_v), (int)lut_operand<BB, 1>(x1, lut_v)};
    } else {
      constexpr uint32_t mlo = kSubMask << (4 * (BB & 1)), mhi = mlo << 2;
      const uint32_t y0 = BB < 2 ? x0 : s0, y1 = BB < 2 ? x1 : s1;
      a = v4i{(int)(y0 & mlo), (int)(y0 & mhi), (int)(y1 & mlo), (int)(y1 & mhi)};
    }
    st.o[cblk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, bw[g]),
                                                        st.o[cblk], 0, 0, 0);
  };
  one(std::integral_constant<int, 0>{});
  one(std::integral_constant<int, 1>{});
  one(std::integral_constant<int, 2>{});
  one(std::integral_constant<int, 3>{});
}

// Softmax of one INT2 tile from its scores: logits, online max and sum, and
// the fp16 P.V weights.  Tokens outside the history (and every token of a
// lane whose column holds no (slot, head) pair) get logit -inf; their scale
// words are zero, so their weights are exactly zero.
template <int D, int NG, int GQA>
struct I2Weights {
  v4i bw[DC<D, NG, GQA>::SLOTS / 2][NG];  // block-diagonal B operands of the P.V MFMAs
};
template <int D, int NG, int GQA, bool LUT, bool T3>
__device__ __forceinline__ I2Weights<D, NG, GQA> i2_softmax(const I2Tile<D, NG, GQA>& t, const I2Scores<NG>& S,
                                                           Acc<D, NG>& st, float kappa, const float (&sig)[NG],
                                                           int my_slot) {
  using C = DC<D, NG, GQA>;
  // ---- logits (log2 domain)
  float lg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      // with a codebook the integer dot holds 32 L[code]
      const float sint = score_int<T3>(S.a[g][i], S.b[g][i], S.c[g][i]) * (LUT ? 1.f / 32.f : 1.f);
      const uint32_t sz = t.sc[i * NG + g];
      acc += bf16_lo(sz) * (sint - bf16_hi(sz) * sig[g]);
    }
    lg[i] = fmaf(acc, kappa, i < t.nvalid ? 0.f : -INFINITY);
  }
  // value scales of the lane's tokens (zero for tokens outside the history)
  float sv[NG][4];
  float smax = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[g][i] = bf16_lo(t.sc[4 * NG + i * NG + g]);
      smax = fmaxf(smax, sv[g][i]);
    }
  st.template update_ref<GQA>(lg, smax);
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(lg[i] - st.ref);
  st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  // ---- fp16 weights w = p * s_V per group (tokens 2, 3 divided by 4
  //      unless with a codebook), and the correction Z += sum w' * z' with
  //      the rounded weights w' (z' = 4 z for tokens 2, 3; codebook
  //      operands: z' = 16 + z)
  I2Weights<D, NG, GQA> W;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float w[4], zb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sz = t.sc[4 * NG + i * NG + g];
      w[i] = pr[i] * sv[g][i];
      if constexpr (LUT) {
        zb[i] = bf16_hi(sz) + kBiasLut;
      } else if (i >= 2) {
        w[i] *= kHiWeight;
        zb[i] = bf16_hi(sz) * (1.f / kHiWeight);
      } else {
        zb[i] = bf16_hi(sz);
      }
    }
    const h2 w01 = __builtin_convertvector(f2{w[0], w[1]}, h2);
    const h2 w23 = __builtin_convertvector(f2{w[2], w[3]}, h2);
    st.Z[g] += ((float)w01[0] * zb[0] + (float)w01[1] * zb[1]) + ((float)w23[0] * zb[2] + (float)w23[1] * zb[3]);
    const uint32_t u01 = __builtin_bit_cast(uint32_t, w01), u23 = __builtin_bit_cast(uint32_t, w23);
#pragma unroll
    for (int pp = 0; pp < C::SLOTS / 2; ++pp) {
      const bool m0 = my_slot == 2 * pp, m1 = my_slot == 2 * pp + 1;
      W.bw[pp][g] = v4i{(int)(m0 ? u01 : 0u), (int)(m0 ? u23 : 0u), (int)(m1 ? u01 : 0u), (int)(m1 ? u23 : 0u)};
    }
  }
  return W;
}

// P.V of one INT2 tile on the fp16 matrix cores, two pages per MFMA.
template <int D, int NG, int GQA, bool LUT>
__device__ __forceinline__ void i2_pv(const I2Tile<D, NG, GQA>& t, const I2Weights<D, NG, GQA>& W, Acc<D, NG>& st,
                                      uint32_t lut_v) {
  using C = DC<D, NG, GQA>;
#pragma unroll
  for (int pp = 0; pp < C::SLOTS / 2; ++pp) {
    pv_block_pair<D, NG, 0, LUT>(st, t.vw[2 * pp][0], t.vw[2 * pp + 1][0], W.bw[pp], lut_v);
    if constexpr (C::KW > 1) pv_block_pair<D, NG, 1, LUT>(st, t.vw[2 * pp][1], t.vw[2 * pp + 1][1], W.bw[pp], lut_v);
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
  st.template update_max<GQA>(lg);
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(lg[i] - st.ref);
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
// INT2 units: one (o, lse) per query head h from the wave's columns
// s*GQA + h, which share one reference and so add without rescaling.  The
// sum over slots goes through LDS (fewer instructions on the wave's critical
// path than row rotations of every accumulator): each lane stores its raw
// accumulators (column n, channels 16 cb + 4j .. +3) and its column's l, Z
// and reference; then lane L sums and normalizes OPL consecutive channels of
// head L / (64 / GQA).  The numerator is acc * unit_inv(cb) - Z (codebook:
// acc - Z).  A wave's LDS accesses complete in issue order, so its own
// stores are visible to its later loads; the wavefront fence only keeps the
// compiler from reordering them.
template <int D, int NG, int GQA, bool LUT>
__device__ __forceinline__ void wave_finish_i2(Acc<D, NG>& st, Smem<D, GQA>& sm, int wave, int lane) {
  using C = DC<D, NG, GQA>;
  constexpr int G = D / NG, LPH = 64 / GQA, OPL = D / LPH, VW = OPL % 4 == 0 ? 4 : 2;
  static_assert(OPL % VW == 0 && G % OPL == 0 && OPL <= 16, "outputs per lane within one scale group");
  const int n = lane & 15, j = lane >> 4;
  st.l = col_sum(st.l);
#pragma unroll
  for (int g = 0; g < NG; ++g) st.Z[g] = col_sum(st.Z[g]);
  auto& F = sm.u.f;
  if (n < C::COLS) {
#pragma unroll
    for (int cbk = 0; cbk < D / 16; ++cbk) *(v4f*)&F.raw[wave][n][cbk * 16 + 4 * j] = st.o[cbk];
    if (j == 0) {
      F.lz[wave][n][0] = st.l;
#pragma unroll
      for (int g = 0; g < NG; ++g) F.lz[wave][n][1 + g] = st.Z[g];
      F.lz[wave][n][3] = st.ref;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int h = lane / LPH, c0 = (lane % LPH) * OPL;
  float l = 0.f, z = 0.f, acc[OPL];
#pragma unroll
  for (int s = 0; s < C::SLOTS; ++s) {
    const int col = s * GQA + h;
    l += F.lz[wave][col][0];
    z += F.lz[wave][col][1 + c0 / G];
#pragma unroll
    for (int e = 0; e < OPL; e += VW) {
      if constexpr (VW == 4) {
        const v4f x = *(const v4f*)&F.raw[wave][col][c0 + e];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[e + k] = s ? acc[e + k] + x[k] : x[k];
      } else {
        const float2 x = *(const float2*)&F.raw[wave][col][c0 + e];
        acc[e] = s ? acc[e] + x.x : x.x;
        acc[e + 1] = s ? acc[e + 1] + x.y : x.y;
      }
    }
  }
  const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
  const float a = (LUT ? 1.f : pv_unit_inv(c0 / 16)) * inv, zb = z * inv;
#pragma unroll
  for (int e = 0; e < OPL; ++e) F.part[wave][h][c0 + e] = fmaf(acc[e], a, -zb);
  if (lane % LPH == 0) F.part[wave][h][D] = l > 0.f ? F.lz[wave][h][3] + __log2f(l) : -INFINITY;
}

// BF16 units: the same reduction with row rotations; channel of o[cb][i] is
// (4j + i) * D/16 + cb.
template <int D, int GQA>
__device__ __forceinline__ void wave_finish_b16(Acc<D, 1>& st, Smem<D, GQA>& sm, int wave, int lane) {
  const int n = lane & 15, j = lane >> 4;
  st.l = slot_sum<GQA>(col_sum(st.l));
  const float mh = st.ref;  // shared by the head's columns (update_max<GQA>)
#pragma unroll
  for (int cbk = 0; cbk < D / 16; ++cbk)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o[cbk][i] = slot_sum<GQA>(st.o[cbk][i]);
  if (n < GQA) {
    const float inv = st.l > 0.f ? __builtin_amdgcn_rcpf(st.l) : 0.f;
#pragma unroll
    for (int cbk = 0; cbk < D / 16; ++cbk)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u.f.part[wave][n][(4 * j + i) * (D / 16) + cbk] = st.o[cbk][i] * inv;
    if (j == 0) sm.u.f.part[wave][n][D] = st.l > 0.f ? mh + __log2f(st.l) : -INFINITY;
  }
}

// ------------------------------------------------------------- kernel ----
// The plan argument: the length-aware plan's tables for the PACKED
// instantiations, an empty placeholder otherwise.
template <bool PACKED>
struct PlanArg {};
template <>
struct PlanArg<true> : PackedPlanArgs {};
// The prefix-shared units for the CASC instantiations.
template <bool CASC>
struct CascArg {};
template <>
struct CascArg<true> : CascArgs {};

// x / d for 0 <= x < 2^24 and 1 <= d < 2^24: the masks let the compiler use
// its short division (a float reciprocal and one correction) in place of the
// full 32-bit sequence; the workgroup's unit decoding sits on the path to its
// first page-table request
__device__ __forceinline__ int div24(int x, int d) {
  return (int)(((uint32_t)x & 0xFFFFFFu) / ((uint32_t)d & 0xFFFFFFu));
}

#ifndef OSCAR_LPT_MIN
#define OSCAR_LPT_MIN 256
#endif
// Workgroup order of uniform-plan launches with more workgroups than CUs (256
// on MI355X).  The hardware hands workgroup ids to the XCDs round robin and,
// within an XCD, each next id to the first CU that frees up.  Each XCD takes a
// contiguous range of units (xcd_remap) and runs every INT2 chunk of it before
// any of its BF16 units: the long units go first and the short ones fill the
// CUs that finish early (measured 127-130 against 132-136 us per step of a
// 32 x 32K-token batch, whose 1,024 chunks and 256 BF16 units run in five
// rounds).  Returns the logical unit of workgroup bid for n units, U per
// (sequence, KV head), the first nb of them BF16 units; n < 2^24.
__device__ __forceinline__ int longest_first(int bid, int n, int U, int nb) {
  constexpr int kXcd = 8;
  const int q = n / kXcd, r = n % kXcd;
  const int xcd = bid % kXcd, idx = bid / kXcd;
  const int a = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  const int len = xcd < r ? q + 1 : q;
  const int C = U - nb;
  if (nb <= 0 || C <= 0) return a + idx;
  // INT2 units among the units [0, x)
  auto count_int2 = [&](int x) {
    const int pq = div24(x, U);
    return pq * C + max(x - pq * U - nb, 0);
  };
  const int ia = count_int2(a), ni = count_int2(a + len) - ia;
  if (idx < ni) {
    const int rk = ia + idx, pq = div24(rk, C);
    return pq * U + nb + (rk - pq * C);
  }
  const int rb = (a - ia) + idx - ni, pq = div24(rb, nb);
  return pq * U + (rb - pq * nb);
}
// The leading scalar arguments are everything the first page-table and R_K
// requests depend on (16 dwords): the build preloads them into scalar
// registers at wave launch, so those requests are issued without waiting for
// the argument block.
template <int D, int NG, int GQA, bool BF16_ONLY, bool LUT, bool CASC, bool PACKED, bool IDS2 = false>
__global__ void __launch_bounds__(kThreads)
    k_decode(const int32_t* __restrict__ int2_pt_all, const float* __restrict__ r_k, const uint16_t* __restrict__ qin,
             const int32_t* __restrict__ seq_lens, int grid_n, int units_per_head, int num_kv_heads,
             int n_bf16_units, int pages_per_chunk, int int2_pt_stride, int max_len, int int2_num_pages,
             const DecodeParams p, const int32_t* __restrict__ bf16_pt_all, const uint8_t* __restrict__ bf16_pool,
             const uint8_t* __restrict__ int2_pool, const CascArg<CASC> ca, const PlanArg<PACKED> pa) {
  using C = DC<D, NG, GQA>;
  __shared__ Smem<D, GQA> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: page-table lookups then stay scalar loads and the
  // tile prefetch is never serialized behind a vector-memory wait
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, j = lane >> 4;
  int lin = xcd_remap(blockIdx.x, grid_n);
  PhaseStamps ps;
  ps.at(0);
  // With GQA <= kWaves / 2 the q' prologue runs on waves 0 .. kWaves/2 - 1
  // only, which meet at an LDS counter instead of a workgroup barrier; the
  // counter starts at zero before any wave can reach it.
  constexpr bool kQHalf = !BF16_ONLY && GQA <= kWaves / 2;
  if constexpr (kQHalf) {
    if (tid == 0) sm.qsync = 0u;
    __syncthreads();
  }
  // this workgroup's (sequence, KV head, unit), its head's units U and
  // partial slots [slot0, slot0 + head_slots)
  int U, u, kvh, b, head_slots, slot0;
  if constexpr (!BF16_ONLY && PACKED) {
    // the first 16 offsets are read with constant indices (one batch of
    // scalar loads next to the other arguments); longer batches continue
    // with a binary search over the rest
    constexpr int kReg = 16;
    int wo[kReg + 1], so[kReg + 1];
#pragma unroll
    for (int i = 0; i <= kReg; ++i) {
      wo[i] = pa.wg_off[i];
      so[i] = pa.slot_off[i];
    }
    int wb = 0, we = 0, sb = 0, se = 0;
    b = 0;
#pragma unroll
    for (int i = 0; i < kReg; ++i)
      if (i < p.batch && wo[i] <= lin) {
        b = i;
        wb = wo[i];
        we = wo[i + 1];
        sb = so[i];
        se = so[i + 1];
      }
    if (p.batch > kReg && lin >= wo[kReg]) {
      int lo = kReg, hi = p.batch;  // wg_off[lo] <= lin < wg_off[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pa.wg_off[mid] <= lin)
          lo = mid;
        else
          hi = mid;
      }
      b = lo;
      wb = pa.wg_off[b];
      we = pa.wg_off[b + 1];
      sb = pa.slot_off[b];
      se = pa.slot_off[b + 1];
    }
    U = (we - wb) / num_kv_heads;
    const int local = lin - wb;
    kvh = local / U;
    u = local % U;
    head_slots = (se - sb) / num_kv_heads;
    slot0 = sb + kvh * head_slots;
  } else {
    U = units_per_head;
    if (!BF16_ONLY && grid_n > OSCAR_LPT_MIN && grid_n < (1 << 24))
      lin = longest_first(blockIdx.x, grid_n, U, n_bf16_units);
    if (grid_n < (1 << 24)) {
      const int pair = div24(lin, U);
      u = lin - pair * U;
      b = div24(pair, num_kv_heads);
      kvh = pair - b * num_kv_heads;
    } else {
      u = lin % U;
      kvh = (lin / U) % num_kv_heads;
      b = lin / (U * num_kv_heads);
    }
    head_slots = p.slots_per_head;
    slot0 = (b * num_kv_heads + kvh) * head_slots;
  }
  const int max_chunks = (!BF16_ONLY && PACKED) ? U - n_bf16_units : p.max_chunks;
  const int hq = num_kv_heads * GQA;

  // Loads that do not depend on the sequence length are issued before its
  // value arrives: for an INT2 chunk the page ids of its planned page range
  // (clamped to the page table) and R_K and q for the rotation prologue.
  const int L_in = seq_lens[b];
  // prefix-shared unit of this sequence: its first S_u history pages and the
  // unit's prefix partials come from the prefix launch
  int S_u = 0, cch = 0;
  if constexpr (CASC) {
    for (int i = 0; i < p.n_casc; ++i)
      if (b >= ca.unit[i].first && b < ca.unit[i].first + ca.unit[i].count) {
        S_u = ca.unit[i].shared_pages;
        cch = ca.unit[i].chunks;
      }
  }
  constexpr int TPB = 64 / C::SLOTS;  // tiles whose page ids one VGPR holds
  static_assert((TPB & (TPB - 1)) == 0, "tiles per id batch: a power of two");
  // threads of the q' prologue: thread (rs, cg) owns rows [rs*RPS, rs*RPS +
  // RPS) of R_K and output channels 4cg .. 4cg+3 of q' = q R_K
  constexpr int QWAVES = kQHalf ? kWaves / 2 : kWaves;
  constexpr int CG = D / 4, RS = 64 * QWAVES / CG, RPS = D / RS;
  const int cg = tid % CG, rs = tid / CG;
  const bool qwave = wave < QWAVES;
  const bool int2_planned = !BF16_ONLY && u >= n_bf16_units;
  const int c_int2 = u - n_bf16_units;
  // IDS2: chunks of up to 2 * kIdBatch pages; a wave then holds the page
  // ids of its tiles TPB .. 2*TPB-1 in a second register
  constexpr int kIdBatch = 64 * kWaves;  // pages whose ids one register per wave holds
  int pid_raw = -1, pid2_raw = -1;
  float4 rr[RPS];
  uint32_t qq[GQA][RPS / 2];
  if (int2_planned) {
    // lane i*SLOTS + s: slot s of this wave's i-th tile, wave + i*kWaves
    const int i = lane / C::SLOTS, s = lane % C::SLOTS;
    const int lp = S_u + c_int2 * pages_per_chunk + (wave + i * kWaves) * C::SLOTS + s;
    const int pend = min(S_u + (c_int2 + 1) * pages_per_chunk, int2_pt_stride);
    if (lp < pend) pid_raw = int2_pt_all[(size_t)b * int2_pt_stride + lp];
    if constexpr (IDS2) {
      if (lp + kIdBatch < pend) pid2_raw = int2_pt_all[(size_t)b * int2_pt_stride + lp + kIdBatch];
    }
    if (qwave) {
      const float* rbase = r_k + (size_t)kvh * D * D + (size_t)(rs * RPS) * D + 4 * cg;
#pragma unroll
      for (int r = 0; r < RPS; ++r) rr[r] = *(const float4*)(rbase + (size_t)r * D);
      // the thread's RPS consecutive q channels of each head
      const uint16_t* qb = qin + ((size_t)b * hq + kvh * GQA) * D + rs * RPS;
#pragma unroll
      for (int h = 0; h < GQA; ++h) {
        if constexpr (RPS % 8 == 0) {
#pragma unroll
          for (int k = 0; k < RPS / 8; ++k) {
            const uint4 x = *(const uint4*)(qb + h * D + 8 * k);
            qq[h][4 * k] = x.x;
            qq[h][4 * k + 1] = x.y;
            qq[h][4 * k + 2] = x.z;
            qq[h][4 * k + 3] = x.w;
          }
        } else if constexpr (RPS == 4) {
          const uint2 x = *(const uint2*)(qb + h * D);
          qq[h][0] = x.x;
          qq[h][1] = x.y;
        } else {
          static_assert(RPS == 2, "row split");
          qq[h][0] = *(const uint32_t*)(qb + h * D);
        }
      }
    }
  }

  int L = min(max(L_in, 0), max_len);
  L = min(L, kPage * p.bf16_pt_stride);
  if (!BF16_ONLY) L = min(L, p.sink + p.recent + kPage * int2_pt_stride);
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
    const int chunks = max(1, min((npages + pages_per_chunk - 1) / pages_per_chunk, p.max_chunks));
    total = chunks;
    if (u >= chunks) return;
    first = u * pages_per_chunk;
    end = (u == chunks - 1) ? npages : min(first + pages_per_chunk, npages);
  } else {
    const int own_pages = max(hist_pages - S_u, 0);
    const int chunks = min(own_pages < (1 << 23) ? div24(own_pages + pages_per_chunk - 1, pages_per_chunk)
                                                 : (own_pages + pages_per_chunk - 1) / pages_per_chunk,
                           max_chunks);
    total = n_bf16_units + chunks;
    if (u < n_bf16_units) {
      const int nlist = n_sp + n_rp;
      first = u * p.bf16_pages_per_unit;
      end = (u == n_bf16_units - 1) ? nlist : min(first + p.bf16_pages_per_unit, nlist);
    } else {
      const int c = u - n_bf16_units;
      if (c >= chunks) return;
      int2_unit = true;
      first = S_u + c * pages_per_chunk;
      end = (c == chunks - 1) ? hist_pages : min(first + pages_per_chunk, hist_pages);
    }
  }

  if (!BF16_ONLY && int2_unit) {
    // ---------------------------------------------------- INT2 chunk unit
    constexpr int R = kRing;
    const int my_slot = (n < C::COLS) ? n / GQA : C::SLOTS;
    const int chd = n % GQA;
    const int ntiles = (end - first + C::SLOTS - 1) / C::SLOTS;
    // tiles of this wave (at most TPB, or 2 * TPB with IDS2: the host bounds
    // the chunk size)
    const int nt_w = wave < ntiles ? min((ntiles - 1 - wave) / kWaves + 1, IDS2 ? 2 * TPB : TPB) : 0;
    const size_t page_bytes = (size_t)num_kv_heads * C::BLK2;
    const uint8_t* __restrict__ hpool = int2_pool + (size_t)kvh * C::BLK2;
    // physical page ids of this wave's tiles wave + i*kWaves: lane i*SLOTS + s
    // holds slot s of tile i, -1 when absent or outside the history
    int pids, pids2 = -1;
    {
      const int i = lane / C::SLOTS, s = lane % C::SLOTS;
      const int lp = first + (wave + i * kWaves) * C::SLOTS + s;
      const bool ok = i < nt_w && lp < end && pid_raw >= 0 && pid_raw < int2_num_pages;
      pids = ok ? pid_raw : -1;
      if constexpr (IDS2) {
        const bool ok2 = i + TPB < nt_w && lp + kIdBatch < end && pid2_raw >= 0 && pid2_raw < int2_num_pages;
        pids2 = ok2 ? pid2_raw : -1;
      }
    }

    // ring of tiles in flight: the first R-1 tiles are requested before the
    // prologue computes q', so HBM is busy from the start
    I2Tile<D, NG, GQA> ring[R];
    auto fetch = [&](I2Tile<D, NG, GQA>& t, int i) {
      // lane of the first id of tile i in `pids`
      int id_lane = i * C::SLOTS;
      if constexpr (IDS2) {
        // the second batch of ids takes the place of the first once its
        // last tile has been requested (tiles are requested in order)
        if (i == TPB) pids = pids2;
        id_lane = (i % TPB) * C::SLOTS;
      }
      // tiles past this wave's last one read no page (all ids -1)
      i2_fetch<D, NG, GQA>(t, hpool, page_bytes, pids, i < nt_w ? id_lane : -1,
                           first + (wave + i * kWaves) * C::SLOTS, hist_len, my_slot, lane);
    };
#pragma unroll
    for (int r = 0; r < R - 1; ++r) fetch(ring[r], r);
    ps.at(1);

    // ---- prologue: q' = q R_K (fp32), per-head int8 split, B operands
    // (each slot's B operand is zero outside its own columns). With the q'
    // prologue on waves 0 .. QWAVES-1 only those waves clear it: their LDS
    // counter then orders every clear before the blocks written below; a
    // clear by a later wave could land on a block already written.
    if (qwave) {
      v4i* bqz = &sm.bq[0][0][0][0];
      for (int x = tid; x < C::SLOTS * 3 * C::KW * 64; x += 64 * QWAVES) bqz[x] = v4i{0, 0, 0, 0};
    }
    if (qwave) {
      float qacc[GQA][4];
#pragma unroll
      for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) qacc[h][e] = 0.f;
#pragma unroll
      for (int i = 0; i < RPS; ++i) {
#pragma unroll
        for (int h = 0; h < GQA; ++h) {
          const float qv = (i & 1) ? bf16_hi(qq[h][i >> 1]) : bf16_lo(qq[h][i >> 1]);
          qacc[h][0] = fmaf(qv, rr[i].x, qacc[h][0]);
          qacc[h][1] = fmaf(qv, rr[i].y, qacc[h][1]);
          qacc[h][2] = fmaf(qv, rr[i].z, qacc[h][2]);
          qacc[h][3] = fmaf(qv, rr[i].w, qacc[h][3]);
        }
      }
      ps.at(11);
      // sum the row segments held by this wave (lanes with equal cg)
      static_assert(CG == 16 || CG == 32, "one or two row segments per 32 lanes");
#pragma unroll
      for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (CG == 16) qacc[h][e] = xor16_add(qacc[h][e]);
          qacc[h][e] = xor32_add(qacc[h][e]);
        }
      if (lane < CG) {
#pragma unroll
        for (int h = 0; h < GQA; ++h)
          *(float4*)&sm.u.qpart[wave][h][4 * cg] = float4{qacc[h][0], qacc[h][1], qacc[h][2], qacc[h][3]};
      }
    }
    if constexpr (kQHalf) {
      // waves 0 .. QWAVES-1 meet here; the others go on to the split barrier
      // (their tile requests, scalar work queued behind that of the lower
      // waves, no longer hold the q' sums back)
      if (qwave) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_fetch_add(&sm.qsync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (__hip_atomic_load(&sm.qsync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)QWAVES)
          __builtin_amdgcn_s_sleep(1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
    } else {
      __syncthreads();
    }
    ps.at(2);
    if (wave < GQA) {
      // wave h finishes query head h: lane owns channels CPL*lane + e
      const int h = wave;
      constexpr int CPL = D / 64;
      float x[CPL];
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < QWAVES; ++w) v += sm.u.qpart[w][h][CPL * lane + e];
        x[e] = v;
      }
      int ta[CPL], tb[CPL], tc[CPL];
      bool dom;
      const float sq = split_query<CPL>(x, ta, tb, tc, dom);
      int sg = 0, sg3 = 0;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        sg += 256 * ta[e] + tb[e];
        sg3 += 65536 * ta[e] + 256 * tb[e] + tc[e];
      }
      // The B operand of lane group jj of 64-channel block w holds channels
      // c = 64w + 16jj + m in transposed order, channel 4b + k at byte 4k + b
      // (the order of the unpacked K codes), once per slot s at lane
      // 16jj + s*GQA + h.
      if constexpr (kQHalf) {
        // the terms in channel order to LDS (the q' rows of waves
        // QWAVES.. are unused), then one lane per (term, w, jj) block reads
        // its 16 channels, transposes the 4 x 4 bytes and writes the block
        // to every slot: no byte writes to shared 4-byte words
        int8_t* stage = (int8_t*)&sm.u.qpart[QWAVES + h][0][0];
        auto put = [&](int t, const int (&v)[CPL]) {
          if constexpr (CPL == 2)
            *(uint16_t*)&stage[t * D + 2 * lane] = (uint16_t)((v[0] & 0xff) | ((v[1] & 0xff) << 8));
          else
            stage[t * D + lane] = (int8_t)v[0];
        };
        put(0, ta);
        put(1, tb);
        put(2, tc);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (lane < 3 * C::KW * 4) {
          const int t = lane / (C::KW * 4), w = (lane / 4) % C::KW, jj = lane % 4;
          const v4i x = *(const v4i*)&stage[t * D + 64 * w + 16 * jj];
          // x[i] holds channels 4i .. 4i+3; out[k] = bytes k of x[0..3]
          const uint32_t lo01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
          const uint32_t hi01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
          const uint32_t lo23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
          const uint32_t hi23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
          const v4i blk = {(int)__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                           (int)__builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                           (int)__builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                           (int)__builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
          for (int s = 0; s < C::SLOTS; ++s) sm.bq[s][t][w][16 * jj + s * GQA + h] = blk;
        }
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const int c = CPL * lane + e;
          const int w = c / 64, jj = (c % 64) / 16, m = c % 16;
          const int byte = 4 * (m % 4) + m / 4;
#pragma unroll
          for (int s = 0; s < C::SLOTS; ++s) {
            const int l = 16 * jj + s * GQA + h;
            ((int8_t*)&sm.bq[s][0][w][l])[byte] = (int8_t)ta[e];
            ((int8_t*)&sm.bq[s][1][w][l])[byte] = (int8_t)tb[e];
            ((int8_t*)&sm.bq[s][2][w][l])[byte] = (int8_t)tc[e];
          }
        }
      }
      if constexpr (NG == 1) {
        sg = wave_sum_i(sg);
        sg3 = wave_sum_i(sg3);
        if (lane == 0) {
          sm.sig[h] = sg;
          sm.sig3[h] = sg3;
        }
      } else {
        // D = 128, G = 64: lanes 0-31 hold group 0, lanes 32-63 group 1
        sg = half_sum_i(sg);
        sg3 = half_sum_i(sg3);
        if ((lane & 31) == 0) {
          sm.sig[h * NG + (lane >> 5)] = sg;
          sm.sig3[h * NG + (lane >> 5)] = sg3;
        }
      }
      if (lane == 0) {
        sm.kap[h] = p.sm_log2 * sq * (1.f / 256.f);
        sm.kap3[h] = p.sm_log2 * sq * (1.f / 65536.f);
        sm.dom[h] = dom ? 1 : 0;
      }
      ps.at(12);
    }
    __syncthreads();
    ps.at(3);
    // three-term mode for the whole workgroup when any of its heads needs it
    int any_dom = 0;
#pragma unroll
    for (int h = 0; h < GQA; ++h) any_dom |= sm.dom[h];
    const bool t3 = NG == 1 && __builtin_amdgcn_readfirstlane(any_dom) != 0;
    const float kappa = t3 ? sm.kap3[chd] : sm.kap[chd];
    float sig[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sig[g] = (float)(t3 ? sm.sig3[chd * NG + g] : sm.sig[chd * NG + g]);

    Acc<D, NG> st;
    st.init(true);
    auto run = [&](auto t3c) {
      constexpr bool T3 = decltype(t3c)::value;
      // two-term mode: the loop-invariant B operands live in VGPRs
      v4i bqr[C::SLOTS][2][C::KW];
      if constexpr (!T3) {
#pragma unroll
        for (int s = 0; s < C::SLOTS; ++s)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int w = 0; w < C::KW; ++w) bqr[s][t][w] = sm.bq[s][t][w][lane];
      }
      const uint32_t lut_k = p.lut_k, lut_v = p.lut_v;
      // scores of one tile on the int8 matrix cores (block-diagonal B
      // operands: slot s's page meets only the columns of slot s); the
      // third term's operands stay in LDS
      auto scores = [&](const I2Tile<D, NG, GQA>& t) {
        I2Scores<NG> r;
#pragma unroll
        for (int g = 0; g < NG; ++g) r.a[g] = r.b[g] = r.c[g] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < C::SLOTS; ++s) {
#pragma unroll
          for (int w = 0; w < C::KW; ++w) {
            const v4i a = k_operand<LUT>(t.kw[s][w], lut_k);
            const int g = (NG == 1) ? 0 : w;
            if constexpr (T3) {
              // three-term mode (rare): every operand is read from LDS per
              // tile (volatile reads are not hoisted), so that this loop
              // needs no registers for them
              const v4i b0 = lds_read_fresh(&sm.bq[s][0][w][lane]);
              const v4i b1 = lds_read_fresh(&sm.bq[s][1][w][lane]);
              const v4i b2 = lds_read_fresh(&sm.bq[s][2][w][lane]);
              r.a[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b0, r.a[g], 0, 0, 0);
              r.b[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b1, r.b[g], 0, 0, 0);
              r.c[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b2, r.c[g], 0, 0, 0);
            } else {
              r.a[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bqr[s][0][w], r.a[g], 0, 0, 0);
              r.b[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bqr[s][1][w], r.b[g], 0, 0, 0);
            }
          }
        }
        return r;
      };
      I2Scores<NG> S = scores(ring[0]);
      ps.at(4);
      int i = 0;
      while (true) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (i >= nt_w) break;
          // Wave priority by phase: the fetch and the softmax (a short VALU
          // chain) at 2, the P.V operands and MFMAs at 1, the score MFMAs
          // at 0.  Of the two waves on a SIMD, the one in the VALU-heavy
          // phase issues first while the other one's MFMAs keep the matrix
          // core busy (measured 0.5 us faster per 100K-token step than a
          // flat priority).
          __builtin_amdgcn_s_setprio(2);
          fetch(ring[(r + R - 1) % R], i + R - 1);
          // softmax of tile i first: the wait for tile i+1's data comes
          // after it, next to the MFMAs that need that data
          const I2Weights<D, NG, GQA> W = i2_softmax<D, NG, GQA, LUT, T3>(ring[r], S, st, kappa, sig, my_slot);
          __builtin_amdgcn_s_setprio(0);
          S = scores(ring[(r + 1) % R]);
          __builtin_amdgcn_s_setprio(1);
          i2_pv<D, NG, GQA, LUT>(ring[r], W, st, lut_v);
          // slots r and r+1 hold arrived data (the loads of r+2 .. r+R-1 may
          // still be in flight and are left alone)
          ring[r].pin();
          ring[(r + 1) % R].pin();
          ++i;
        }
        if (i >= nt_w) break;
      }
      __builtin_amdgcn_s_setprio(0);
    };
    if (nt_w > 0) {
      // the three-term loop is compiled for one scale group per head only:
      // with two groups its registers would push the two-term loop into
      // spills (two groups keep ~16 bits of q' relative to its largest
      // channel)
      if (t3)
        run(std::bool_constant<NG == 1>{});
      else
        run(std::false_type{});
    }
    ps.at(5);
    wave_finish_i2<D, NG, GQA, LUT>(st, sm, wave, lane);
    ps.at(13);
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
    st.init(false);
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
    ps.at(5);
    wave_finish_b16<D, GQA>(st, sm, wave, lane);
    ps.at(13);
  }
  __syncthreads();
  ps.at(6);

  // ---- merge the waves' partials into this workgroup's partial
  const size_t head_base = (size_t)b * num_kv_heads + kvh;
  const size_t pidx = ((size_t)slot0 + u) * GQA;
  for (int idx = tid; idx < GQA * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.u.f.part[w][h][D]);
    float o = 0.f, lse = -INFINITY;
    if (mx > -INFINITY) {
      float sw = 0.f, so = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float e = __builtin_amdgcn_exp2f(sm.u.f.part[w][h][D] - mx);
        sw += e;
        so += e * sm.u.f.part[w][h][c];
      }
      o = so * __builtin_amdgcn_rcpf(sw);
      lse = mx + __log2f(sw);  // log2 units
    }
    // device-scope stores write through the XCD's L2, so no L2 write-back
    // is needed before the ticket below
    __hip_atomic_store(p.part_o + (pidx + h) * D + c, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c == 0) __hip_atomic_store(p.part_lse + pidx + h, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // ---- last workgroup of this (sequence, KV head) merges every partial.
  // Every wave waits until its device-scope partial stores have completed
  // (s_waitcnt vmcnt(0)); then one thread takes a ticket with a device-scope
  // atomic.  The workgroup that takes the last ticket invalidates its L2
  // (acquire) and reads all partials from the device-coherent level.  A
  // release on the ticket would also write back the whole L2 of the XCD,
  // which measured 1-3 us per workgroup; the partials never sit dirty in L2,
  // so it has nothing to publish.  Each head's counter has a 128-byte line
  // of its own.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
  __syncthreads();
  ps.at(7);
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(p.counters + head_base * kCounterStride, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (uint32_t)(total - 1);
    asm volatile("" ::"v"(last) : "memory");  // the ticket has returned before the stamp
    ps.at(14);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    ps.at(15);
    sm.last = last;
  }
  __syncthreads();
  ps.at(8);
  if (!sm.last) {
    ps.flush(p.stamps, lin, wave, lane);
    return;
  }
  ps.set(10, 1);
  const size_t p0 = (size_t)slot0 * GQA;
  // Folds partials u0 .. u1-1 of head h, channel c into (M, S, A): the log2
  // max, the sum of weights and the weighted sum of normalized outputs.  h
  // is the same in all 64 lanes of a wave (a wave covers 64 channels of one
  // head).  Per batch of 32 partials the lane's 32 partial values and the
  // head's 32 lse values (lane k holds partial ub + k) are requested
  // together, one memory round trip; max, weights and sum then come from
  // wave reductions and each weight reaches every lane through LDS.  Partial
  // rows are read through a buffer descriptor with the partial's offset in
  // the scalar operand.  Entries past the range carry weight 0 and re-read
  // the last partial, in bounds.
  auto fold = [&](int h_lane, int c, int u0, int u1, float& M, float& S, float& A) {
    const int h = __builtin_amdgcn_readfirstlane(h_lane);
    float* wb = &sm.u.f.lz[wave][0][0];       // 32 weights of the current batch
    const float* lsrc = p.part_lse + p0 + h;  // partial u at lsrc[u * GQA]
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.part_o + (p0 + h) * D), (short)0, (head_slots * GQA - h) * D * 4, kBufferFlags);
    M = -INFINITY;
    S = 0.f;
    A = 0.f;
    auto batch = [&](int ub) {
      // the lse values first (every lane loads, in range), so that the
      // weights are formed while the rows arrive
      const int uu = ub + lane;
      const float ev = lsrc[(size_t)min(uu, u1 - 1) * GQA];
      // -inf past the range: an add rather than a select, which the
      // compiler would turn into a branch that the load sinks into
      const float e = ev + ((lane < 32 && uu < u1) ? 0.f : -INFINITY);
      float o[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int ui = min(ub + k, u1 - 1);
        o[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ors, c * 4, ui * GQA * D * 4, 0));
      }
      // no branch on an empty batch (its weights are all 0), so that the
      // row loads stay ahead of the weights instead of sinking behind them
      const float mb = fmaxf(M, wave_max(e));
      const float ref = mb > -INFINITY ? mb : 0.f;
      const float f = __builtin_amdgcn_exp2f(M - ref);  // 0 while M = -inf
      const float w = __builtin_amdgcn_exp2f(e - ref);  // 0 past the range
      S = S * f + wave_sum(w);
      A *= f;
      // the 32 weights reach every lane through the wave's own LDS words
      // (broadcast reads), in the order of a per-weight readlane
      if (lane < 32) wb[lane] = w;
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
      for (int k = 0; k < 32; k += 4) {
        const v4f wk = *(const v4f*)&wb[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) A = fmaf(wk[i], o[k + i], A);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      M = mb;
    };
    // one batch (the common case) as straight-line code: a loop would make
    // the compiler wait for the lse load before issuing the rows
    if (u1 - u0 > 32) {
      for (int ub = u0; ub < u1; ub += 32) batch(ub);
    } else if (u1 > u0) {
      batch(u0);
    }
  };
  uint16_t* outp = p.out + ((size_t)b * hq + kvh * GQA) * D;
  if (BF16_ONLY || p.r_v == nullptr) {
    auto fold_out = [&](int idx) {
      const int h = idx / D, c = idx % D;
      float M, S, A;
      fold(h, c, 0, total + cch, M, S, A);
      outp[h * D + c] = (uint16_t)f32_to_bf16(S > 0.f ? A * __builtin_amdgcn_rcpf(S) : 0.f);
    };
    if constexpr (GQA * D == kThreads) {
      fold_out(tid);
    } else {
      for (int idx = tid; idx < GQA * D; idx += kThreads) fold_out(idx);
    }
  } else {
    // Values not absorbed: the INT2 partials hold V R_V.  Their merge is
    // rotated back by R_V^T (linear, so once per head after the merge) and
    // then merged with the BF16 units' partials, which hold V itself.
    constexpr int PER = (GQA * D + kThreads - 1) / kThreads;
    float M1[PER], S1[PER], A1[PER], M2[PER], S2[PER];
    float* a2 = &sm.u.f.part[0][0][0];  // [GQA][D] INT2 merge, rotated basis
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = tid + k * kThreads;
      if (idx < GQA * D) {
        const int h = idx / D, c = idx % D;
        float A2;
        fold(h, c, 0, n_bf16_units, M1[k], S1[k], A1[k]);
        fold(h, c, n_bf16_units, total + cch, M2[k], S2[k], A2);
        a2[h * D + c] = A2;
      }
    }
    __syncthreads();
    const float* rv = p.r_v + (size_t)kvh * D * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = tid + k * kThreads;
      if (idx < GQA * D) {
        const int h = idx / D, c = idx % D;
        // (A2 R_V^T)[c] = sum_j A2[j] R_V[c][j]
        const float4* row = (const float4*)(rv + (size_t)c * D);
        const float4* a = (const float4*)(a2 + h * D);
        float acc = 0.f;
#pragma unroll 8
        for (int j = 0; j < D / 4; ++j) {
          const float4 r4 = row[j], x4 = a[j];
          acc = fmaf(x4.x, r4.x, fmaf(x4.y, r4.y, fmaf(x4.z, r4.z, fmaf(x4.w, r4.w, acc))));
        }
        const float M = fmaxf(M1[k], M2[k]);
        float o = 0.f;
        if (M > -INFINITY) {
          const float w1 = __builtin_amdgcn_exp2f(M1[k] - M), w2 = __builtin_amdgcn_exp2f(M2[k] - M);
          const float Sx = w1 * S1[k] + w2 * S2[k];
          o = Sx > 0.f ? (w1 * A1[k] + w2 * acc) / Sx : 0.f;
        }
        outp[h * D + c] = (uint16_t)f32_to_bf16(o);
      }
    }
  }
  if (tid == 0)
    __hip_atomic_store(p.counters + head_base * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ps.at(9);
  ps.flush(p.stamps, lin, wave, lane);
}

// ------------------------------------------------ prefix (cascade) unit --
// Workgroups of the prefix launch: one per (unit, KV head, chunk of the
// shared pages).  The pages are attended once for all of the unit's queries:
// the 16 score columns are (member sequence, query head) pairs and every
// column sees every page, so a tile holds two consecutive pages (the k = 32
// of one fp16 P.V MFMA) and each lane carries 4 tokens of both.  Compared
// with one pass per sequence, the code unpacking, the score MFMAs and the
// P.V operand construction of a page are shared by 16 / GQA sequences.
template <int D, int NG>
struct PTile {
  static constexpr int KW = D / 64;
  uint32_t kw[2][KW];
  uint32_t vw[2][KW];
  uint32_t sc[2][8 * NG];  // per page: this lane's quad, K (s,z) x 4 tokens x NG, then V
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int w = 0; w < KW; ++w) asm volatile("" : "+v"(kw[s][w]), "+v"(vw[s][w]));
#pragma unroll
      for (int w = 0; w < 8 * NG; ++w) asm volatile("" : "+v"(sc[s][w]));
    }
  }
};

template <int D, int NG>
struct PSmem {
  union {
    float part[kWaves][16][D + 1];  // per-wave partials per column, [D] = lse (log2)
    float qpart[kWaves][16][D];     // prologue: per-wave partial sums of q R_K
  } u;
  v4i bq[3][D / 64][64];            // int8 q' B operands (dense: every column; terms a, b, c)
  float kap[16], kap3[16];
  int sig[16 * NG], sig3[16 * NG];
  int dom[16];
};

// Loads the tile of logical pages lp0, lp0 + 1 (physical ids from lanes idx0,
// idx0 + 1 of `pids`; idx0 < 0: no page).  Scale words of tokens at or past
// `valid_len` (the longest member history) are zeroed.
template <int D, int NG>
__device__ __forceinline__ void pt_fetch(PTile<D, NG>& t, const uint8_t* __restrict__ hpool, size_t page_bytes,
                                         int pids, int idx0, int lp0, int valid_len, int lane) {
  constexpr int BLK2 = 8 * D + 128 * NG, REC = D / 8;
  const int j = lane >> 4;
  const int i0 = idx0 >= 0 ? idx0 : 0;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int v = __builtin_amdgcn_readlane(pids, i0 + s);
    const int id = idx0 >= 0 ? v : -1;
    // an absent page reads as zeros (num_records 0)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(hpool + (size_t)max(id, 0) * page_bytes), (short)0, id >= 0 ? BLK2 : 0, kBufferFlags);
    if constexpr (D == 128) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * REC, 0, kKvPolicy);
      t.kw[s][0] = x[0];
      t.kw[s][1] = x[1];
      t.vw[s][0] = x[2];
      t.vw[s][1] = x[3];
    } else {
      const auto y = __builtin_amdgcn_raw_buffer_load_b64(rs, lane * REC, 0, kKvPolicy);
      t.kw[s][0] = y[0];
      t.vw[s][0] = y[1];
    }
#pragma unroll
    for (int i = 0; i < 2 * NG; ++i) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, 8 * D + j * 32 * NG + 16 * i, 0, kKvPolicy);
#pragma unroll
      for (int e = 0; e < 4; ++e) t.sc[s][4 * i + e] = x[e];
    }
    const int nv = min(max(valid_len - ((lp0 + s) * kPage + 4 * j), 0), 4);
    if (nv < 4) {
#pragma unroll
      for (int w = 0; w < 8 * NG; ++w)
        if ((w % (4 * NG)) / NG >= nv) t.sc[s][w] = 0u;
    }
  }
}

// Softmax of one prefix tile (both pages, every column): logits with tokens
// past the column's member history masked, online max and sum, and the dense
// fp16 P.V B operands.
template <int D, int NG, bool LUT, bool T3>
__device__ __forceinline__ void pt_softmax(const PTile<D, NG>& t, const I2Scores<NG> (&S)[2], Acc<D, NG>& st,
                                           float kappa, const float (&sig)[NG], int lp0, int hist_len, int lane,
                                           v4i (&bw)[NG]) {
  const int j = lane >> 4;
  float lg[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float sint = score_int<T3>(S[s].a[g][i], S[s].b[g][i], S[s].c[g][i]) * (LUT ? 1.f / 32.f : 1.f);
        const uint32_t sz = t.sc[s][i * NG + g];
        acc += bf16_lo(sz) * (sint - bf16_hi(sz) * sig[g]);
      }
      const bool ok = (lp0 + s) * kPage + 4 * j + i < hist_len;
      lg[s][i] = fmaf(acc, kappa, ok ? 0.f : -INFINITY);
    }
  float smax = 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int w = 0; w < 4 * NG; ++w) smax = fmaxf(smax, bf16_lo(t.sc[s][4 * NG + w]));
  st.update_ref(lg[0], lg[1], smax);
  float pr[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[s][i] = __builtin_amdgcn_exp2f(lg[s][i] - st.ref);
  st.l += ((pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3])) + ((pr[1][0] + pr[1][1]) + (pr[1][2] + pr[1][3]));
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    uint32_t u[2][2];
    float zsum = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float w[4], zb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t sz = t.sc[s][4 * NG + i * NG + g];
        w[i] = pr[s][i] * bf16_lo(sz);
        if constexpr (LUT) {
          zb[i] = bf16_hi(sz) + kBiasLut;
        } else if (i >= 2) {
          w[i] *= kHiWeight;
          zb[i] = bf16_hi(sz) * (1.f / kHiWeight);
        } else {
          zb[i] = bf16_hi(sz);
        }
      }
      const h2 w01 = __builtin_convertvector(f2{w[0], w[1]}, h2);
      const h2 w23 = __builtin_convertvector(f2{w[2], w[3]}, h2);
      zsum += ((float)w01[0] * zb[0] + (float)w01[1] * zb[1]) + ((float)w23[0] * zb[2] + (float)w23[1] * zb[3]);
      u[s][0] = __builtin_bit_cast(uint32_t, w01);
      u[s][1] = __builtin_bit_cast(uint32_t, w23);
    }
    st.Z[g] += zsum;
    bw[g] = v4i{(int)u[0][0], (int)u[0][1], (int)u[1][0], (int)u[1][1]};
  }
}

template <int D, int NG, int GQA, bool LUT, bool PACKED>
__global__ void __launch_bounds__(kThreads) k_decode_prefix(const DecodeParams p, const CascArgs ca,
                                                            const PlanArg<PACKED> pa) {
  constexpr int KW = D / 64, G = D / NG, BLK2 = 8 * D + 128 * NG;
  constexpr int MEMBERS = 16 / GQA;  // member sequences per unit (columns = members x heads)
  __shared__ PSmem<D, NG> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  // which unit, KV head and chunk
  int ui = 0;
  for (int i = 1; i < p.n_casc; ++i)
    if (lin >= ca.unit[i].wg_start) ui = i;
  const CascUnit cu = ca.unit[ui];
  const int rem = lin - cu.wg_start;
  const int kvh = rem / cu.chunks, c = rem % cu.chunks;
  const int hq = p.num_kv_heads * GQA;
  const int mcol = n / GQA, hcol = n % GQA;  // this lane's column: member, head
  // member histories (the same clamps as the decode launch) and each
  // member's first partial slot for this KV head (slot_m) in the decode
  // launch's layout
  int hist_len_m[MEMBERS], own_chunks_m[MEMBERS], slot_m[MEMBERS];
  int valid_len = 0, src = cu.first;
#pragma unroll
  for (int m = 0; m < MEMBERS; ++m) {
    hist_len_m[m] = 0;
    own_chunks_m[m] = 0;
    slot_m[m] = 0;
    if (m < cu.count) {
      const int sb = cu.first + m;
      int mc = p.max_chunks;
      if constexpr (PACKED) {
        const int um = (pa.wg_off[sb + 1] - pa.wg_off[sb]) / p.num_kv_heads;
        const int sm_ = (pa.slot_off[sb + 1] - pa.slot_off[sb]) / p.num_kv_heads;
        mc = um - p.n_bf16_units;
        slot_m[m] = pa.slot_off[sb] + kvh * sm_;
      } else {
        slot_m[m] = (sb * p.num_kv_heads + kvh) * p.slots_per_head;
      }
      int L = min(max(p.seq_lens[cu.first + m], 0), p.max_len);
      L = min(L, kPage * p.bf16_pt_stride);
      L = min(L, p.sink + p.recent + kPage * p.int2_pt_stride);
      const int hl = max(p.sink, L - p.recent) - p.sink;
      const int hp = (hl + kPage - 1) / kPage;
      hist_len_m[m] = min(hl, kPage * cu.shared_pages);
      own_chunks_m[m] = min((max(hp - cu.shared_pages, 0) + p.pages_per_chunk - 1) / p.pages_per_chunk, mc);
      if (hist_len_m[m] > valid_len) {
        valid_len = hist_len_m[m];
        src = cu.first + m;
      }
    }
  }
  int my_hist = 0;
#pragma unroll
  for (int m = 0; m < MEMBERS; ++m)
    if (m == mcol) my_hist = hist_len_m[m];

  // page ids of the chunk's pages, through the table of the member with the
  // longest history (each member's table maps the shared pages its own
  // history covers, and they are the same physical pages)
  const int first = c * cu.pages_per_chunk;
  const int end = min(first + cu.pages_per_chunk, cu.shared_pages);
  const int ntiles = (end - first + 1) / 2;
  constexpr int TPB = 32;  // tiles whose page ids one VGPR holds
  const int nt_w = wave < ntiles ? min((ntiles - 1 - wave) / kWaves + 1, TPB) : 0;
  int pids;
  {
    const int i = lane >> 1, s = lane & 1;
    const int lp = first + (wave + i * kWaves) * 2 + s;
    int id = -1;
    if (i < nt_w && lp < end && lp * kPage < valid_len && lp < p.int2_pt_stride)
      id = p.int2_pt[(size_t)src * p.int2_pt_stride + lp];
    pids = (id >= 0 && id < p.int2_num_pages) ? id : -1;
  }
  const size_t page_bytes = (size_t)p.num_kv_heads * BLK2;
  const uint8_t* __restrict__ hpool = p.int2_pool + (size_t)kvh * BLK2;

  constexpr int R = kRing;
  PTile<D, NG> ring[R];
  auto fetch = [&](PTile<D, NG>& t, int i) {
    pt_fetch<D, NG>(t, hpool, page_bytes, pids, i < nt_w ? 2 * i : -1, first + (wave + i * kWaves) * 2, valid_len,
                    lane);
  };
#pragma unroll
  for (int r = 0; r < R - 1; ++r) fetch(ring[r], r);

  // ---- prologue: q' = q R_K for the 16 columns, int8 split, B operands
  constexpr int CG = D / 4, RS = kThreads / CG, RPS = D / RS;
  const int cg = tid % CG, rs = tid / CG;
  {
    float4 rr[RPS];
    const float* rbase = p.r_k + (size_t)kvh * D * D + (size_t)(rs * RPS) * D + 4 * cg;
#pragma unroll
    for (int r = 0; r < RPS; ++r) rr[r] = *(const float4*)(rbase + (size_t)r * D);
#pragma unroll
    for (int m = 0; m < MEMBERS; ++m) {
      float qacc[GQA][4];
#pragma unroll
      for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) qacc[h][e] = 0.f;
      if (m < cu.count) {
        // the thread's RPS consecutive q channels of each head in one load
        const uint16_t* qb = p.q + ((size_t)(cu.first + m) * hq + kvh * GQA) * D + rs * RPS;
#pragma unroll
        for (int h = 0; h < GQA; ++h) {
          uint32_t qw[RPS / 2];
          if constexpr (RPS == 8) {
            const uint4 x = *(const uint4*)(qb + h * D);
            qw[0] = x.x;
            qw[1] = x.y;
            qw[2] = x.z;
            qw[3] = x.w;
          } else {
            static_assert(RPS == 2, "row split");
            qw[0] = *(const uint32_t*)(qb + h * D);
          }
#pragma unroll
          for (int i = 0; i < RPS; ++i) {
            const float qv = (i & 1) ? bf16_hi(qw[i >> 1]) : bf16_lo(qw[i >> 1]);
            qacc[h][0] = fmaf(qv, rr[i].x, qacc[h][0]);
            qacc[h][1] = fmaf(qv, rr[i].y, qacc[h][1]);
            qacc[h][2] = fmaf(qv, rr[i].z, qacc[h][2]);
            qacc[h][3] = fmaf(qv, rr[i].w, qacc[h][3]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (CG == 16) qacc[h][e] = xor16_add(qacc[h][e]);
          qacc[h][e] = xor32_add(qacc[h][e]);
        }
      if (lane < CG) {
#pragma unroll
        for (int h = 0; h < GQA; ++h)
          *(float4*)&sm.u.qpart[wave][m * GQA + h][4 * cg] = float4{qacc[h][0], qacc[h][1], qacc[h][2], qacc[h][3]};
      }
    }
  }
  __syncthreads();
  for (int col = wave; col < 16; col += kWaves) {
    constexpr int CPL = D / 64;
    float x[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += sm.u.qpart[w][col][CPL * lane + e];
      x[e] = v;
    }
    int ta[CPL], tb[CPL], tc[CPL];
    bool dom;
    const float sq = split_query<CPL>(x, ta, tb, tc, dom);
    int sg = 0, sg3 = 0;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int ch = CPL * lane + e;
      sg += 256 * ta[e] + tb[e];
      sg3 += 65536 * ta[e] + 256 * tb[e] + tc[e];
      const int w = ch / 64, jj = (ch % 64) / 16, mm = ch % 16;
      const int byte = 4 * (mm % 4) + mm / 4;
      const int l = 16 * jj + col;
      ((int8_t*)&sm.bq[0][w][l])[byte] = (int8_t)ta[e];
      ((int8_t*)&sm.bq[1][w][l])[byte] = (int8_t)tb[e];
      ((int8_t*)&sm.bq[2][w][l])[byte] = (int8_t)tc[e];
    }
    if constexpr (NG == 1) {
      sg = wave_sum_i(sg);
      sg3 = wave_sum_i(sg3);
      if (lane == 0) {
        sm.sig[col] = sg;
        sm.sig3[col] = sg3;
      }
    } else {
      sg = half_sum_i(sg);
      sg3 = half_sum_i(sg3);
      if ((lane & 31) == 0) {
        sm.sig[col * NG + (lane >> 5)] = sg;
        sm.sig3[col * NG + (lane >> 5)] = sg3;
      }
    }
    if (lane == 0) {
      sm.kap[col] = p.sm_log2 * sq * (1.f / 256.f);
      sm.kap3[col] = p.sm_log2 * sq * (1.f / 65536.f);
      sm.dom[col] = dom ? 1 : 0;
    }
  }
  __syncthreads();
  // three-term mode for the whole workgroup when any column needs it
  int any_dom = 0;
#pragma unroll
  for (int c2 = 0; c2 < 16; ++c2) any_dom |= sm.dom[c2];
  const bool t3 = NG == 1 && __builtin_amdgcn_readfirstlane(any_dom) != 0;
  const float kappa = t3 ? sm.kap3[n] : sm.kap[n];
  float sig[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) sig[g] = (float)(t3 ? sm.sig3[n * NG + g] : sm.sig[n * NG + g]);
  v4i bqr[2][KW];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int w = 0; w < KW; ++w) bqr[t][w] = sm.bq[t][w][lane];
  __syncthreads();  // the union's qpart is reused for the partials below

  const uint32_t lut_k = p.lut_k, lut_v = p.lut_v;
  Acc<D, NG> st;
  st.init(true);
  auto run = [&](auto t3c) {
    constexpr bool T3 = decltype(t3c)::value;
    // the third term's operands stay in LDS
    auto scores = [&](const PTile<D, NG>& t, I2Scores<NG> (&S)[2]) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int g = 0; g < NG; ++g) S[s].a[g] = S[s].b[g] = S[s].c[g] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          const v4i a = k_operand<LUT>(t.kw[s][w], lut_k);
          const int g = (NG == 1) ? 0 : w;
          S[s].a[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bqr[0][w], S[s].a[g], 0, 0, 0);
          S[s].b[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bqr[1][w], S[s].b[g], 0, 0, 0);
          if constexpr (T3) {
            const v4i b3 = lds_read_fresh(&sm.bq[2][w][lane]);  // not hoisted (registers)
            S[s].c[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b3, S[s].c[g], 0, 0, 0);
          }
        }
      }
    };
    I2Scores<NG> S[2];
    scores(ring[0], S);
    int i = 0;
    while (true) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (i >= nt_w) break;
        // wave priority by phase, as in k_decode
        __builtin_amdgcn_s_setprio(2);
        fetch(ring[(r + R - 1) % R], i + R - 1);
        v4i bw[NG];
        pt_softmax<D, NG, LUT, T3>(ring[r], S, st, kappa, sig, first + (wave + i * kWaves) * 2, my_hist, lane, bw);
        __builtin_amdgcn_s_setprio(0);
        scores(ring[(r + 1) % R], S);
        __builtin_amdgcn_s_setprio(1);
        pv_block_pair<D, NG, 0, LUT>(st, ring[r].vw[0][0], ring[r].vw[1][0], bw, lut_v);
        if constexpr (KW > 1) pv_block_pair<D, NG, 1, LUT>(st, ring[r].vw[0][1], ring[r].vw[1][1], bw, lut_v);
        ring[r].pin();
        ring[(r + 1) % R].pin();
        ++i;
      }
      if (i >= nt_w) break;
    }
    __builtin_amdgcn_s_setprio(0);
  };
  if (nt_w > 0) {
    // three terms for one scale group per head only, as in k_decode
    if (t3)
      run(std::bool_constant<NG == 1>{});
    else
      run(std::false_type{});
  }
  // ---- wave epilogue: one (o, lse) per column (no two columns share a head)
  st.l = col_sum(st.l);
#pragma unroll
  for (int g = 0; g < NG; ++g) st.Z[g] = col_sum(st.Z[g]);
  {
    const float inv = st.l > 0.f ? __builtin_amdgcn_rcpf(st.l) : 0.f;
#pragma unroll
    for (int cbk = 0; cbk < D / 16; ++cbk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = (cbk * 16) / G;
        const float acc = LUT ? st.o[cbk][i] : st.o[cbk][i] * pv_unit_inv(cbk);
        sm.u.part[wave][n][cbk * 16 + 4 * j + i] = (acc - st.Z[g]) * inv;
      }
    if (j == 0) sm.u.part[wave][n][D] = st.l > 0.f ? st.ref + __log2f(st.l) : -INFINITY;
  }
  __syncthreads();
  // ---- merge the waves and store each column's partial in its member's
  //      slot n_bf16_units + own chunks + c
  for (int idx = tid; idx < 16 * D; idx += kThreads) {
    const int col = idx / D, ch = idx % D;
    const int m = col / GQA, h = col % GQA;
    if (m >= cu.count) continue;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.u.part[w][col][D]);
    float o = 0.f, lse = -INFINITY;
    if (mx > -INFINITY) {
      float sw = 0.f, so = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float e = __builtin_amdgcn_exp2f(sm.u.part[w][col][D] - mx);
        sw += e;
        so += e * sm.u.part[w][col][ch];
      }
      o = so * __builtin_amdgcn_rcpf(sw);
      lse = mx + __log2f(sw);
    }
    int oc = 0, s0 = 0;
#pragma unroll
    for (int mm = 0; mm < MEMBERS; ++mm)
      if (mm == m) {
        oc = own_chunks_m[mm];
        s0 = slot_m[mm];
      }
    const size_t pidx = ((size_t)s0 + p.n_bf16_units + oc + c) * GQA + h;
    p.part_o[pidx * D + ch] = o;
    if (ch == 0) p.part_lse[pidx] = lse;
  }
}

// the leading scalar arguments of k_decode, in order
#define DECODE_LEAD_ARGS(p, grid)                                                                           \
  (p).int2_pt, (p).r_k, (p).q, (p).seq_lens, (grid), (p).units_per_head, (p).num_kv_heads, (p).n_bf16_units, \
      (p).pages_per_chunk, (p).int2_pt_stride, (p).max_len, (p).int2_num_pages

template <int D, int NG, int GQA>
bool launch_prefix_t(const DecodeParams& p, const CascArgs& casc, const PackedPlanArgs* packed, int grid,
                     hipStream_t stream) {
  auto go = [&](auto lut) {
    constexpr bool L = decltype(lut)::value;
    if (packed) {
      PlanArg<true> pa;
      static_cast<PackedPlanArgs&>(pa) = *packed;
      hipLaunchKernelGGL((k_decode_prefix<D, NG, GQA, L, true>), dim3(grid), dim3(kThreads), 0, stream, p, casc,
                         pa);
    } else {
      hipLaunchKernelGGL((k_decode_prefix<D, NG, GQA, L, false>), dim3(grid), dim3(kThreads), 0, stream, p, casc,
                         PlanArg<false>{});
    }
  };
  if (p.lut)
    go(std::true_type{});
  else
    go(std::false_type{});
  return true;
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

template <int D, int NG>
constexpr bool kLongChunks = D == 128 && NG == 1;

// the INT2 decode, with the prefix-unit bookkeeping compiled in only when
// the call has prefix units (CASC), the codebook operands only for a
// codebook pool (LUT) and the plan tables only for a length-aware plan
template <int D, int NG, int GQA, bool CASC>
void launch_int2_t(const DecodeParams& p, const CascArgs* casc, const PackedPlanArgs* packed, int grid,
                   hipStream_t stream) {
  CascArg<CASC> ca;
  if constexpr (CASC) static_cast<CascArgs&>(ca) = *casc;
  auto go = [&](auto lut, auto ids2) {
    constexpr bool L = decltype(lut)::value, I2 = decltype(ids2)::value;
    if (packed) {
      PlanArg<true> pa;
      static_cast<PackedPlanArgs&>(pa) = *packed;
      hipLaunchKernelGGL((k_decode<D, NG, GQA, false, L, CASC, true, I2>), dim3(grid), dim3(kThreads), 0, stream, DECODE_LEAD_ARGS(p, grid), p, p.bf16_pt, p.bf16_pool, p.int2_pool, ca, pa);
    } else {
      hipLaunchKernelGGL((k_decode<D, NG, GQA, false, L, CASC, false, I2>), dim3(grid), dim3(kThreads), 0, stream, DECODE_LEAD_ARGS(p, grid), p, p.bf16_pt, p.bf16_pool, p.int2_pool, ca,
                         PlanArg<false>{});
    }
  };
  auto go_lut = [&](auto ids2) {
    if (p.lut)
      go(std::true_type{}, ids2);
    else
      go(std::false_type{}, ids2);
  };
  // chunks longer than one batch of page ids per wave (the planner allows
  // them at D = 128 with one scale group per head)
  if constexpr (kLongChunks<D, NG>) {
    if (p.pages_per_chunk > 64 * kWaves) {
      go_lut(std::true_type{});
      return;
    }
  }
  go_lut(std::false_type{});
}

template <int D, int NG, int GQA>
bool launch_decode_t(const DecodeParams& p, const CascArgs* casc, const PackedPlanArgs* packed, bool bf16_only,
                     int grid, hipStream_t stream) {
  if (bf16_only)
    hipLaunchKernelGGL((k_decode<D, NG, GQA, true, false, false, false>), dim3(grid), dim3(kThreads), 0, stream, DECODE_LEAD_ARGS(p, grid), p, p.bf16_pt, p.bf16_pool, p.int2_pool, CascArg<false>{},
                       PlanArg<false>{});
  else if (p.n_casc > 0)
    launch_int2_t<D, NG, GQA, true>(p, casc, packed, grid, stream);
  else
    launch_int2_t<D, NG, GQA, false>(p, nullptr, packed, grid, stream);
  return true;
}

}  // namespace

bool launch_decode(const DecodeParams& p, const CascArgs* casc, const PackedPlanArgs* packed, int head_dim,
                   int n_groups, int gqa, bool bf16_only, int grid, hipStream_t stream) {
  if (p.n_casc > 0 && !casc) return false;
#define OSCAR_DEC(D, NG, G)                        \
  if (head_dim == D && n_groups == NG && gqa == G) \
    return launch_decode_t<D, NG, G>(p, casc, packed, bf16_only, grid, stream);
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

bool launch_decode_prefix(const DecodeParams& p, const CascArgs& casc, const PackedPlanArgs* packed, int head_dim,
                          int n_groups, int gqa, int grid, hipStream_t stream) {
  if (grid <= 0) return true;
#define OSCAR_PRE(D, NG, G)                        \
  if (head_dim == D && n_groups == NG && gqa == G) \
    return launch_prefix_t<D, NG, G>(p, casc, packed, grid, stream);
  OSCAR_PRE(128, 1, 2)
  OSCAR_PRE(128, 1, 4)
  OSCAR_PRE(128, 1, 8)
  OSCAR_PRE(128, 2, 2)
  OSCAR_PRE(128, 2, 4)
  OSCAR_PRE(128, 2, 8)
  OSCAR_PRE(64, 1, 2)
  OSCAR_PRE(64, 1, 4)
  OSCAR_PRE(64, 1, 8)
#undef OSCAR_PRE
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
