// Write path of the OSCAR INT2 cache on gfx950: rotate, clip, quantize, pack
// (MarkTechPost article, "The Serving System"; ModelScope/CSDN page, design
// section: the oldest recent token is demoted by a fused rotate / clip /
// quantize / pack kernel, four 2-bit codes per byte).
//
// Quantization of one token's group of G channels (values c after the clip):
//   s = bf16(fl32(max - min) / 3)  (1 when max == min or s underflows to 0)
//   z = bf16(fl32(-min / s))
//   code = clamp(rne(fl32(fl32(c / s) + z)), 0, 3)
// with IEEE fp32 division, so pre-rotated inputs give bit-exact codes.
//
// k_append_demote: one workgroup per (sequence, KV head); appends the new
//   token to the BF16 pool and demotes the token leaving the recent window,
//   rotating its key by R_K with fp32 FMAs.
// k_quantize_pack: bulk prefill of history.  The key rotation Y = K R_K is a
//   [16 tokens x D] x [D x D] contraction per page and runs on the bf16
//   matrix cores with R_K split as R_hi + R_lo (both bf16), which keeps
//   Y within ~2^-17 relative of the fp32 product; V is already rotated.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace oscar {
namespace {

__device__ __forceinline__ float wmin(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wmax(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// scale and zero (as bf16 bits) of a group with minimum mn and maximum mx
__device__ __forceinline__ void scale_zero(float mn, float mx, uint32_t& s_bits, uint32_t& z_bits, float& s,
                                           float& z) {
  const float d = mx - mn;
  s_bits = f32_to_bf16(d / 3.0f);
  s = bf16_to_f32(s_bits);
  if (d == 0.f || s == 0.f) {
    s_bits = 0x3F80u;
    s = 1.f;
  }
  z_bits = f32_to_bf16(-mn / s);
  z = bf16_to_f32(z_bits);
}
// Four-level codebook: the code of t = c/s + z is the number of thresholds
// (midpoints of consecutive levels, exact in fp32) strictly below t; off:
// the uniform levels 0..3 with round-to-nearest-even and clamp.
struct Thr {
  float b0, b1, b2;
  bool on;
};
__device__ __forceinline__ uint32_t thr_code(float t, const Thr& th) {
  return (uint32_t)(t > th.b0) + (uint32_t)(t > th.b1) + (uint32_t)(t > th.b2);
}
__device__ __forceinline__ uint32_t quant_code(float c, float s, float z, const Thr& th) {
  const float t = __fadd_rn(c / s, z);
  if (th.on) return thr_code(t, th);
  return (uint32_t)fminf(fmaxf(rintf(t), 0.f), 3.f);
}

// ------------------------------------------------------- append + demote --
// One workgroup of 256 threads per (sequence, KV head).  The rotation
// operands (thread (c, part) holds column c of R over rows part*RP .. +RP,
// for R_K and, when V is not absorbed, R_V) do not depend on the sequence,
// so their loads are issued first and overlap the length and page-table
// reads; the demoted token is read before the appended token is written
// (the caller may recycle the page of the oldest recent token for the
// newest one).
template <int D, int NG, bool VROT>
__global__ void __launch_bounds__(256) k_append_demote(const WriteParams p) {
  constexpr int G = D / NG;
  constexpr int KW = D / 64;
  constexpr int BLK2 = 8 * D + 128 * NG;
  constexpr int REC = D / 8;
  constexpr int PARTS = 256 / D, RP = D / PARTS;  // row split of the rotation
  __shared__ float kd[D];
  __shared__ float vd[D];
  __shared__ float yp[2][PARTS][D];    // [K/V][part] partial rotations
  __shared__ float red[2][D / 64][2];  // [K/V][64-channel block][min, max]
  __shared__ uint8_t codes[2][D];
  __shared__ uint32_t sz[2][NG];

  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.num_kv_heads, kvh = blockIdx.x % p.num_kv_heads;
  const size_t hb = (size_t)kvh;
  const int c = tid % D, part = tid / D;
  float rk[RP], rv[VROT ? RP : 1];
  {
    const float* src = p.r_k + hb * D * D + (size_t)(part * RP) * D + c;
#pragma unroll
    for (int i = 0; i < RP; ++i) rk[i] = src[(size_t)i * D];
    if constexpr (VROT) {
      const float* srv = p.r_v + hb * D * D + (size_t)(part * RP) * D + c;
#pragma unroll
      for (int i = 0; i < RP; ++i) rv[i] = srv[(size_t)i * D];
    }
  }
  const int L = p.seq_lens[b];
  if (L < 0) return;
  const int32_t* bpt = p.bf16_pt + (size_t)b * p.bf16_pt_stride;
  const int32_t* ipt = p.int2_pt + (size_t)b * p.int2_pt_stride;

  // appended token goes to position L
  int aid = -1;
  if (L / kPage < p.bf16_pt_stride) aid = bpt[L / kPage];
  const bool app = aid >= 0 && aid < p.bf16_num_pages;
  // demoted token d = L - W (the oldest recent token) goes to history slot d - S0
  const int d = L - p.recent;
  const int hs = d - p.sink;
  bool dem = d >= p.sink;
  int did = -1, iid = -1;
  if (dem) {
    if (d / kPage < p.bf16_pt_stride) did = bpt[d / kPage];
    if (hs / kPage < p.int2_pt_stride) iid = ipt[hs / kPage];
    dem = did >= 0 && did < p.bf16_num_pages && iid >= 0 && iid < p.int2_num_pages;
  }
  uint8_t* blk = p.int2_pool + ((size_t)max(iid, 0) * p.num_kv_heads + hb) * BLK2;
  const int slot = hs % kPage, jq = slot / 4, ti = slot % 4;
  // V record words hold four tokens: read the word this token goes into now
  uint32_t vold = 0;
  const bool v_thread = tid >= 64 && tid < 64 + 16 * KW;
  uint32_t* vdst = (uint32_t*)(blk + (16 * jq + (tid - 64) / KW) * REC + D / 16 + 4 * ((tid - 64) % KW));
  if (dem && v_thread && ti != 0) vold = *vdst;
  if (dem && tid < D) {
    const uint8_t* bb = p.bf16_pool + ((size_t)did * p.num_kv_heads + hb) * (64 * D);
    const int sl = d % kPage;
    kd[tid] = bf16_to_f32(((const uint16_t*)bb)[sl * D + tid]);
    vd[tid] = bf16_to_f32(((const uint16_t*)(bb + 32 * D))[(sl / 4) * D * 4 + tid * 4 + (sl % 4)]);
  }
  __syncthreads();  // the demoted token is in LDS before the append writes
  if (app && tid < D) {
    uint8_t* bb = p.bf16_pool + ((size_t)aid * p.num_kv_heads + hb) * (64 * D);
    const int sl = L % kPage;
    const size_t src = ((size_t)b * p.num_kv_heads + hb) * D + tid;
    ((uint16_t*)bb)[sl * D + tid] = p.k_new[src];
    ((uint16_t*)(bb + 32 * D))[(sl / 4) * D * 4 + tid * 4 + (sl % 4)] = p.v_new[src];
  }
  if (!dem) return;

  // y = k_d R_K (and v_d R_V): thread (c, part) sums rows part*RP .. +RP (fp32 FMA)
  {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) acc = fmaf(kd[part * RP + i], rk[i], acc);
    yp[0][part][c] = acc;
    if constexpr (VROT) {
      float av = 0.f;
#pragma unroll
      for (int i = 0; i < RP; ++i) av = fmaf(vd[part * RP + i], rv[i], av);
      yp[1][part][c] = av;
    }
  }
  __syncthreads();
  // quantization: threads (which, c), which = 0 for K and 1 for V; every
  // 64-lane wave lies inside one group because G >= 64
  const int which = tid / D;
  float x = 0.f;
  if (which < 2) {
    if (which == 0 || VROT) {
      x = 0.f;
#pragma unroll
      for (int q = 0; q < PARTS; ++q) x += yp[which][q][c];
    } else {
      x = vd[c];
    }
    const float tau = which == 0 ? p.tau_k[hb] : p.tau_v[hb];
    x = fminf(fmaxf(x, -tau), tau);
    const float mn = wmin(x), mx = wmax(x);
    if ((tid & 63) == 0) {
      red[which][c / 64][0] = mn;
      red[which][c / 64][1] = mx;
    }
  }
  __syncthreads();
  if (which < 2) {
    const int g = c / G;
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < G / 64; ++w) {
      mn = fminf(mn, red[which][g * (G / 64) + w][0]);
      mx = fmaxf(mx, red[which][g * (G / 64) + w][1]);
    }
    uint32_t sb, zb;
    float s, z;
    scale_zero(mn, mx, sb, zb, s, z);
    const Thr th = which == 0 ? Thr{p.thr_k[0], p.thr_k[1], p.thr_k[2], p.lut != 0}
                              : Thr{p.thr_v[0], p.thr_v[1], p.thr_v[2], p.lut != 0};
    codes[which][c] = (uint8_t)quant_code(x, s, z, th);
    if (c % G == 0) sz[which][g] = sb | (zb << 16);
  }
  __syncthreads();
  // pack into INT2 page iid, slot hs % 16
  if (tid < 4 * KW) {  // K: records (j, slot), word w
    const int jj = tid / KW, w = tid % KW;
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 16; ++m) word |= (uint32_t)codes[0][w * 64 + jj * 16 + m] << (2 * m);
    *(uint32_t*)(blk + (16 * jj + slot) * REC + 4 * w) = word;
  } else if (v_thread) {  // V: records (jq, r), word w
    const int r = (tid - 64) / KW, w = (tid - 64) % KW;
    uint32_t word = vold;  // the first token of a quad starts the word (vold = 0)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int pos = 16 * (ti & 1) + 2 * (2 * bb + (ti >> 1));
      word = (word & ~(3u << pos)) | ((uint32_t)codes[1][(4 * w + bb) * 16 + r] << pos);
    }
    *vdst = word;
  } else if (tid >= 128 && tid < 128 + 2 * NG) {  // scale/zero words
    const int wh = (tid - 128) / NG, g = (tid - 128) % NG;
    *(uint32_t*)(blk + 8 * D + jq * 32 * NG + wh * 16 * NG + (ti * NG + g) * 4) = sz[wh][g];
  }
}

// ----------------------------------------------------------- bulk quantize --
// One workgroup per compute unit converts R_K once and then streams pages of
// one KV head; each wave owns one page at a time and its own LDS area, so the
// page loop needs no workgroup barrier.  The next page's K and V are loaded
// while the current one is rotated and quantized.
#ifndef OSCAR_QP_WAVES
#define OSCAR_QP_WAVES 16
#endif
constexpr int kQpWaves = OSCAR_QP_WAVES;
// with V rotated on the matrix cores too, R_V takes another 64 KiB of LDS
constexpr int kQpWavesVrot = 8;
template <bool VROT>
constexpr int qp_waves() { return VROT ? kQpWavesVrot : kQpWaves; }

template <int D, int NG, bool VROT>
struct BulkSmem {
  static constexpr int W = qp_waves<VROT>();
  uint4 rb[2][D / 16][D / 32][64];              // R_K hi / lo as MFMA A operands, output channels permuted
  uint4 rbv[VROT ? 2 : 1][D / 16][D / 32][VROT ? 64 : 1];  // R_V the same way (rotated V only)
  uint8_t vcode[W][kPage][D];                   // per wave: V codes, one byte each
};

// min / max over the 4 lanes of a quad (lanes 4t .. 4t+3)
__device__ __forceinline__ float quad_min(float x) {
  x = fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  return fminf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
}
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
}
// min / max over lanes n, n+16, n+32, n+48 (the gfx950 permlane swaps
// exchange 16-lane rows 0<->1, 2<->3 and the two 32-lane halves)
__device__ __forceinline__ float col4_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float col4_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// c / s for a bf16 divisor s, given y = 1/s (correctly rounded): the
// product c*y corrected once by its fma residual (Markstein).  For every fp32
// significand of c and every bf16 significand of s this equals the IEEE
// quotient; away from underflow and overflow the exponents only scale it.
__device__ __forceinline__ float div_bf16(float c, float s, float y) {
  const float q0 = c * y;
  const float r = __builtin_fmaf(-s, q0, c);
  return __builtin_fmaf(r, y, q0);
}
// the code of quotient q with zero point z into byte e of word
__device__ __forceinline__ uint32_t code_into(uint32_t word, float q, float z, int e) {
  const float t = rintf(__fadd_rn(q, z));
  return __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(t, 0.f, 3.f), e, word);
}

// scale_zero with fewer IEEE divisions, bit for bit the same result, plus
// y = 1/s correctly rounded: d/3 and -mn/s by div_bf16 (3 is a bf16
// significand times 2), and 1/s from v_rcp_f32 with one fma correction, which
// for every bf16 significand of s turns any start within 2 ulp of 1/s into the
// correctly rounded reciprocal.  Operands near the ends of the range, and a
// zero minimum (whose quotient must keep its sign), take the IEEE division.
__device__ __forceinline__ void scale_zero_recip(float mn, float mx, uint32_t& s_bits, uint32_t& z_bits, float& s,
                                                 float& z, float& y) {
  const float d = mx - mn;
  float d3;
  if (d >= 0x1p-100f && d <= 0x1p100f)
    d3 = div_bf16(d, 3.0f, 0x1.555556p-2f);  // RN(1/3)
  else
    d3 = d / 3.0f;
  s_bits = f32_to_bf16(d3);
  s = bf16_to_f32(s_bits);
  if (d == 0.f || s == 0.f) {
    s_bits = 0x3F80u;
    s = 1.f;
  }
  const bool s_mid = s >= 0x1p-70f && s <= 0x1p70f;
  if (s_mid) {
    const float y0 = __builtin_amdgcn_rcpf(s);
    y = __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
  } else {
    y = 1.0f / s;
  }
  float zq;
  if (s_mid && fabsf(mn) >= 0x1p-100f && fabsf(mn) <= 0x1p56f)
    zq = div_bf16(-mn, s, y);
  else
    zq = -mn / s;
  z_bits = f32_to_bf16(zq);
  z = bf16_to_f32(z_bits);
}

// Scale, zero and codes of one group of clipped values x[N] (N % 4 == 0),
// four codes per word, one byte each, x[4q + e] in byte e of words[q].
//
// Fast path, taken when s >= 2^-70, |min|, |max| <= 2^56 and |z| <= 128:
// the quotient comes from the reciprocal (div_bf16, exact there) and the
// code is v_cvt_pk_u8_f32 of t = q + z, which rounds to nearest even and
// maps negatives to 0.  There t lies in [-0.26, 3.26]: (c - min)/s is at most
// 3(1 + 2^-8) because s is within 2^-9 of (max - min)/3, and z is within
// 2^-9 |z| <= 0.251 of -min/s; so the clamp to [0, 3] never acts.  Other
// groups take the IEEE division, round and clamp.
// The fast path of group_codes below without a branch: every operation of
// its common case, computed unconditionally, and `ok` set when this lane's
// group meets all the conditions under which that case is the one taken
// (d and |min| in [2^-100, 2^100] and [2^-100, 2^56], s in [2^-70, 2^70],
// |max| <= 2^56, |z| <= 128).  Where ok holds, the result is bit for bit
// that of group_codes.
template <int N>
__device__ __forceinline__ uint32_t group_codes_nb(const float (&x)[N], float mn, float mx, uint32_t (&words)[N / 4],
                                                   bool& ok) {
  const float d = mx - mn;
  const uint32_t s_bits = f32_to_bf16(div_bf16(d, 3.0f, 0x1.555556p-2f));
  const float s = bf16_to_f32(s_bits);
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float y = __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
  const uint32_t z_bits = f32_to_bf16(div_bf16(-mn, s, y));
  const float z = bf16_to_f32(z_bits);
  const float amn = fabsf(mn);
  ok = d >= 0x1p-100f && d <= 0x1p100f && s >= 0x1p-70f && s <= 0x1p70f && amn >= 0x1p-100f && amn <= 0x1p56f &&
       fabsf(mx) <= 0x1p56f && fabsf(z) <= 128.f;
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      word = __builtin_amdgcn_cvt_pk_u8_f32(__fadd_rn(div_bf16(x[4 * q + e], s, y), z), e, word);
    words[q] = word;
  }
  return s_bits | (z_bits << 16);
}

template <int N, bool LUT>
__device__ __forceinline__ uint32_t group_codes(const float (&x)[N], float mn, float mx, uint32_t (&words)[N / 4],
                                                const Thr& th) {
  if constexpr (!LUT) {
    // the common case without a branch; the whole wave takes the general
    // code below only when one of its groups is outside that case
    bool ok;
    const uint32_t sz = group_codes_nb<N>(x, mn, mx, words, ok);
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return sz;
  }
  uint32_t sb, zb;
  float s, z, y;
  scale_zero_recip(mn, mx, sb, zb, s, z, y);
  const bool fast = s >= 0x1p-70f && fmaxf(fabsf(mn), fabsf(mx)) <= 0x1p56f && fabsf(z) <= 128.f;
  if constexpr (LUT) {
    // codebook: the same t as below (exact quotient, then + z), compared
    // with the thresholds
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xq = x[4 * q + e];
        const float t = __fadd_rn(fast ? div_bf16(xq, s, y) : xq / s, z);
        word |= thr_code(t, th) << (8 * e);
      }
      words[q] = word;
    }
  } else {
  if (fast) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        word = __builtin_amdgcn_cvt_pk_u8_f32(__fadd_rn(div_bf16(x[4 * q + e], s, y), z), e, word);
      words[q] = word;
    }
  } else {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) word = code_into(word, x[4 * q + e] / s, z, e);
      words[q] = word;
    }
  }
  }
  return sb | (zb << 16);
}

template <int D, int NG, bool VROT>
struct BulkPage {  // one page's global inputs, as loaded
  uint4 ka[D / 32];          // K as MFMA B operands: token r, channels j*D/4 + ks*8 + e
  // V: rotated -> the same layout as K; else token t, channels w*64 + qq*16 + 0..15
  uint4 va[VROT ? D / 32 : D / 64 * 2];
  int id;                    // physical page (-1: none)
};

// Loads page `page` whose physical id (or -1) is `id`.  One buffer descriptor
// per page, based at its first token, bounds the loads: slots past the last
// token, and every slot of a page without a physical id, read as zero, with
// no branch around the loads.
template <int D, int NG, bool VROT>
__device__ __forceinline__ void bulk_load(BulkPage<D, NG, VROT>& pg, const WriteParams& p, int kvh, int page, int id,
                                          int lane) {
  constexpr int KB = D / 32, KW = D / 64;
  pg.id = id;
  const int j = lane >> 4, r = lane & 15, t = lane >> 2, qq = lane & 3;
  const int tok0 = page * kPage;
  const int ntok = id >= 0 ? min(kPage, p.num_tokens - tok0) : 0;  // tokens present in this page
  const int row = p.num_kv_heads * D * 2;                              // bytes per token
  const size_t base = (size_t)tok0 * row + (size_t)kvh * D * 2;
  const int nrec = __builtin_amdgcn_readfirstlane(max(ntok, 0) * row);  // wave-uniform
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const uint8_t*)p.k + base), (short)0, nrec, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const uint8_t*)p.v + base), (short)0, nrec, kBufferFlags);
  // the last token's row ends at its head's D channels, inside num_records
#pragma unroll
  for (int ks = 0; ks < KB; ++ks) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, r * row + j * (D / 2) + ks * 16, 0, 0);
    pg.ka[ks] = uint4{x[0], x[1], x[2], x[3]};
  }
  if constexpr (VROT) {
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rv, r * row + j * (D / 2) + ks * 16, 0, 0);
      pg.va[ks] = uint4{x[0], x[1], x[2], x[3]};
    }
  } else {
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      const auto x0 = __builtin_amdgcn_raw_buffer_load_b128(rv, t * row + w * 128 + qq * 32, 0, 0);
      const auto x1 = __builtin_amdgcn_raw_buffer_load_b128(rv, t * row + w * 128 + qq * 32 + 16, 0, 0);
      pg.va[2 * w] = uint4{x0[0], x0[1], x0[2], x0[3]};
      pg.va[2 * w + 1] = uint4{x1[0], x1[1], x1[2], x1[3]};
    }
  }
}

// Y^T = R^T X^T for one page on the bf16 matrix cores (R split hi + lo).  The
// A operands hold R's columns in the order that gives lane (j, r) token r's
// channels w*64 + j*16 + 4q + i in y[4w + q][i].
template <int D>
__device__ __forceinline__ void rotate_page(const uint4 (&xb)[D / 32], const uint4 (*rb)[D / 16][D / 32][64],
                                            int lane, float (&y)[D / 16][4]) {
  constexpr int KB = D / 32, OT = D / 16;
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) {
      const v8bf b = __builtin_bit_cast(v8bf, xb[ks]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, rb[0][ot][ks][lane]), b, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, rb[1][ot][ks][lane]), b, c, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) y[ot][i] = c[i];
  }
}

// Clip and quantize one rotated page in the rotate_page layout (the token's
// other channels sit in lanes r + 16, r + 32, r + 48).  CHANNEL_ORDER false:
// words[w][i] holds, in byte q, the code of channel w*64 + j*16 + 4q + i;
// true: words[w][q] holds, in byte i, that same code (channel order).  The
// group scale words are returned in sz.
template <int D, int NG, bool CHANNEL_ORDER, bool LUT>
__device__ __forceinline__ void quant_rotated(const float (&y)[D / 16][4], float tau, uint32_t (&words)[D / 64][4],
                                              uint32_t (&sz)[NG], const Thr& th) {
  constexpr int KW = D / 64, WPG = KW / NG;  // record words per group
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float x[WPG * 16];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < WPG * 16; ++u) {
      const int w = g * WPG + u / 16;
      const int i = CHANNEL_ORDER ? u % 4 : (u / 4) % 4, q = CHANNEL_ORDER ? (u / 4) % 4 : u % 4;
      x[u] = __builtin_amdgcn_fmed3f(y[4 * w + q][i], -tau, tau);
      mn = fminf(mn, x[u]);
      mx = fmaxf(mx, x[u]);
    }
    uint32_t ww[WPG * 4];
    sz[g] = group_codes<WPG * 16, LUT>(x, col4_min(mn), col4_max(mx), ww, th);
#pragma unroll
    for (int u = 0; u < WPG * 4; ++u) words[g * WPG + u / 4][u % 4] = ww[u];
  }
}

template <int D, int NG, bool VROT, bool LUT>
__device__ __forceinline__ void bulk_page(const BulkPage<D, NG, VROT>& pg, const WriteParams& p,
                                          BulkSmem<D, NG, VROT>& sm, int kvh, int page, int wave, int lane,
                                          float tau_k, float tau_v) {
  constexpr int KW = D / 64, OT = D / 16;
  constexpr int BLK2 = 8 * D + 128 * NG;
  constexpr int REC = D / 8;
  const int j = lane >> 4, r = lane & 15, t = lane >> 2, qq = lane & 3;
  const int tok0 = page * kPage;
  uint8_t(*vcode)[D] = sm.vcode[wave];
  const Thr th_k{p.thr_k[0], p.thr_k[1], p.thr_k[2], p.lut != 0};
  const Thr th_v{p.thr_v[0], p.thr_v[1], p.thr_v[2], p.lut != 0};
  // the page's INT2 block through a buffer descriptor: stores without a
  // physical page (num_records 0) or from lanes with nothing to store (offset
  // past the block) are dropped, so no store sits behind a branch
  const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(p.int2_pool + ((size_t)max(pg.id, 0) * p.num_kv_heads + kvh) * BLK2), (short)0,
      pg.id >= 0 ? BLK2 : 0, kBufferFlags);
  constexpr int kDrop = 1 << 20;  // an offset past every block
  const int sc0 = 8 * D;          // scale words: 8*NG per token quad
  // ---- keys: rotated on the matrix cores; each lane then holds the channels
  // of its own code record (j, r), word w
  uint32_t kwd[KW];
  {
    float y[OT][4];
    rotate_page<D>(pg.ka, sm.rb, lane, y);
    const bool tok_ok = pg.id >= 0 && tok0 + r < p.num_tokens;
    uint32_t words[KW][4], sz[NG];
    quant_rotated<D, NG, false, LUT>(y, tau_k, words, sz, th_k);
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      // byte q of word i holds code m = 4q + i at bits 8q; shifted by 2i
      const uint32_t word = words[w][0] | (words[w][1] << 2) | (words[w][2] << 4) | (words[w][3] << 6);
      kwd[w] = tok_ok ? word : 0u;
    }
    // scales of token r (zeros for slots past the last token)
#pragma unroll
    for (int g = 0; g < NG; ++g)
      __builtin_amdgcn_raw_buffer_store_b32(tok_ok ? sz[g] : 0u, out,
                                            j == g ? sc0 + 4 * ((r / 4) * 8 * NG + (r % 4) * NG + g) : kDrop, 0, 0);
  }
  if constexpr (VROT) {
    // ---- values rotated by R_V the same way; their codes go to LDS in
    // channel order for the record transposition below
    float y[OT][4];
    rotate_page<D>(pg.va, sm.rbv, lane, y);
    const bool tok_ok = pg.id >= 0 && tok0 + r < p.num_tokens;
    uint32_t words[KW][4], sz[NG];
    quant_rotated<D, NG, true, LUT>(y, tau_v, words, sz, th_v);
#pragma unroll
    for (int g = 0; g < NG; ++g)
      __builtin_amdgcn_raw_buffer_store_b32(
          tok_ok ? sz[g] : 0u, out, j == g ? sc0 + 4 * ((r / 4) * 8 * NG + 4 * NG + (r % 4) * NG + g) : kDrop, 0, 0);
#pragma unroll
    for (int w = 0; w < KW; ++w)
      *(uint4*)&vcode[r][w * 64 + j * 16] =
          tok_ok ? uint4{words[w][0], words[w][1], words[w][2], words[w][3]} : uint4{0u, 0u, 0u, 0u};
  } else {
    // ---- values (already rotated), lane = 4t + qq: channels w*64 + qq*16 + m
    const bool tok_ok = pg.id >= 0 && tok0 + t < p.num_tokens;
    float x[KW][16];
    float mn[KW], mx[KW];
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      const uint4 a0 = pg.va[2 * w], a1 = pg.va[2 * w + 1];
      const uint32_t xs[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      mn[w] = INFINITY;
      mx[w] = -INFINITY;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        x[w][2 * q] = __builtin_amdgcn_fmed3f(bf16_lo(xs[q]), -tau_v, tau_v);
        x[w][2 * q + 1] = __builtin_amdgcn_fmed3f(bf16_hi(xs[q]), -tau_v, tau_v);
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mn[w] = fminf(mn[w], x[w][m]);
        mx[w] = fmaxf(mx[w], x[w][m]);
      }
      mn[w] = quad_min(mn[w]);
      mx[w] = quad_max(mx[w]);
    }
    uint32_t words[KW][4];
    if constexpr (NG == 1 && KW == 2) {
      float xx[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) xx[u] = x[u / 16][u % 16];
      uint32_t ww[8];
      const uint32_t sz = group_codes<32, LUT>(xx, fminf(mn[0], mn[1]), fmaxf(mx[0], mx[1]), ww, th_v);
#pragma unroll
      for (int u = 0; u < 8; ++u) words[u / 4][u % 4] = ww[u];
      __builtin_amdgcn_raw_buffer_store_b32(tok_ok ? sz : 0u, out,
                                            qq == 0 ? sc0 + 4 * ((t / 4) * 8 * NG + 4 * NG + (t % 4) * NG) : kDrop,
                                            0, 0);
    } else {
      // one group per 64-channel word group w
      static_assert(NG == KW, "V groups are 64 channels wide here");
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        const uint32_t sz = group_codes<16, LUT>(x[w], mn[w], mx[w], words[w], th_v);
        __builtin_amdgcn_raw_buffer_store_b32(
            tok_ok ? sz : 0u, out, qq == 0 ? sc0 + 4 * ((t / 4) * 8 * NG + 4 * NG + (t % 4) * NG + w) : kDrop, 0, 0);
      }
    }
#pragma unroll
    for (int w = 0; w < KW; ++w)
      *(uint4*)&vcode[t][w * 64 + qq * 16] =
          tok_ok ? uint4{words[w][0], words[w][1], words[w][2], words[w][3]} : uint4{0u, 0u, 0u, 0u};
  }
  // the codes of the whole page are in this wave's LDS (one wave's LDS
  // accesses complete in order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ---- this lane's code record (j, r)
  uint32_t vwd[KW];
#pragma unroll
  for (int w = 0; w < KW; ++w) {
    uint32_t vword = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vword |= (uint32_t)vcode[4 * j + i][(4 * w + bb) * 16 + r] << (16 * (i & 1) + 2 * (2 * bb + (i >> 1)));
    vwd[w] = vword;
  }
  if constexpr (D == 128) {
    __builtin_amdgcn_raw_buffer_store_b128(v4u{kwd[0], kwd[1], vwd[0], vwd[1]}, out, lane * REC, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(v2u{kwd[0], vwd[0]}, out, lane * REC, 0, 0);
  }
  // the next page's codes reuse this wave's LDS
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// R (fp32) -> R_hi + R_lo (bf16) in A-operand order:
// rb[hl][ot][ks][lane (j, n)] element e = R[j*D/4 + ks*8 + e][pi(ot, n)],
// pi(ot, 4a + i) = (ot / 4)*64 + a*16 + (ot % 4)*4 + i, so that output row
// 4a + i of tile ot is that output channel
template <int D, int THREADS>
__device__ __forceinline__ void split_rotation(const float* __restrict__ r, uint4 (*rb)[D / 16][D / 32][64], int tid) {
  constexpr int KB = D / 32;
  for (int idx = tid; idx < D * D / 8; idx += THREADS) {
    const int lane_op = idx % 64, ks = (idx / 64) % KB, ot = idx / (64 * KB);
    const int j = lane_op >> 4, n = lane_op & 15;
    const int in0 = j * (D / 4) + ks * 8, out = (ot / 4) * 64 + (n / 4) * 16 + (ot % 4) * 4 + n % 4;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = r[(size_t)(in0 + 2 * e) * D + out], x1 = r[(size_t)(in0 + 2 * e + 1) * D + out];
      hi[e] = pack_bf16x2(x0, x1);
      lo[e] = pack_bf16x2(x0 - bf16_lo(hi[e]), x1 - bf16_hi(hi[e]));
    }
    rb[0][ot][ks][lane_op] = uint4{hi[0], hi[1], hi[2], hi[3]};
    rb[1][ot][ks][lane_op] = uint4{lo[0], lo[1], lo[2], lo[3]};
  }
}

template <int D, int NG, bool VROT, bool LUT>
__global__ void __launch_bounds__(64 * qp_waves<VROT>()) k_quantize_pack(const WriteParams p) {
  constexpr int W = qp_waves<VROT>(), THREADS = 64 * W;
  __shared__ BulkSmem<D, NG, VROT> sm;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int kvh = blockIdx.y;
  const int npages = (p.num_tokens + kPage - 1) / kPage;
  const int pg0 = blockIdx.x * p.pages_per_block;
  if (pg0 >= npages) return;
  const int pg_end = min(pg0 + p.pages_per_block, npages);
  // wave w handles pages pg0 + w + k*W, k < my_n (at most 64: the launch caps
  // pages per workgroup); lane k holds the k-th one's physical id
  const int first = pg0 + wave;
  const int my_n = first < pg_end ? (pg_end - first + W - 1) / W : 0;
  int my_ids = -1;
  if (lane < my_n) {
    const int id = p.page_ids[first + lane * W];
    my_ids = (id >= 0 && id < p.int2_num_pages) ? id : -1;
  }
  auto id_of = [&](int k) { return k < my_n ? __builtin_amdgcn_readlane(my_ids, k) : -1; };
  BulkPage<D, NG, VROT> cur;
  bulk_load<D, NG, VROT>(cur, p, kvh, first, id_of(0), lane);  // first page's loads overlap the R split
  split_rotation<D, THREADS>(p.r_k + (size_t)kvh * D * D, sm.rb, tid);
  if constexpr (VROT) split_rotation<D, THREADS>(p.r_v + (size_t)kvh * D * D, sm.rbv, tid);
  __syncthreads();
  const float tau_k = p.tau_k[kvh], tau_v = p.tau_v[kvh];
  // two pages per trip so that the current and next page alternate between
  // two register sets
  BulkPage<D, NG, VROT> nxt;
  for (int k = 0; k < my_n; k += 2) {
    bulk_load<D, NG, VROT>(nxt, p, kvh, first + (k + 1) * W, id_of(k + 1), lane);
    bulk_page<D, NG, VROT, LUT>(cur, p, sm, kvh, first + k * W, wave, lane, tau_k, tau_v);
    if (k + 1 >= my_n) break;
    bulk_load<D, NG, VROT>(cur, p, kvh, first + (k + 2) * W, id_of(k + 2), lane);
    bulk_page<D, NG, VROT, LUT>(nxt, p, sm, kvh, first + (k + 1) * W, wave, lane, tau_k, tau_v);
  }
}


// ------------------------------------------------------ BF16 page prefill --
template <int D>
__global__ void __launch_bounds__(256) k_write_bf16(const WriteParams p, int first_position) {
  const int kvh = blockIdx.y;
  const int lp = first_position / kPage + blockIdx.x;  // logical page
  if (lp >= p.bf16_pt_stride) return;
  const int id = p.bf16_pt[lp];
  if (id < 0 || id >= p.bf16_num_pages) return;
  uint16_t* blk = (uint16_t*)(p.bf16_pool + ((size_t)id * p.num_kv_heads + kvh) * (64 * D));
  for (int idx = threadIdx.x; idx < kPage * D; idx += 256) {
    const int slot = idx / D, c = idx % D;
    const int t = lp * kPage + slot - first_position;  // token index
    if (t < 0 || t >= p.num_tokens) continue;
    const size_t src = ((size_t)t * p.num_kv_heads + kvh) * D + c;
    blk[slot * D + c] = p.k[src];
    blk[16 * D + (slot / 4) * D * 4 + c * 4 + (slot % 4)] = p.v[src];
  }
}

template <int D, int NG>
void launch_ad(const WriteParams& p, hipStream_t s) {
  if (p.r_v)
    hipLaunchKernelGGL((k_append_demote<D, NG, true>), dim3(p.batch * p.num_kv_heads), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_append_demote<D, NG, false>), dim3(p.batch * p.num_kv_heads), dim3(256), 0, s, p);
}
template <int D, int NG, bool VROT>
void launch_qp_v(const WriteParams& p, hipStream_t s) {
  constexpr int W = qp_waves<VROT>();
  const int npages = (p.num_tokens + kPage - 1) / kPage;
  WriteParams q = p;
  q.pages_per_block = std::min(std::max(p.pages_per_block, 1), 64 * W);  // <= 64 pages per wave
  const int gx = (npages + q.pages_per_block - 1) / q.pages_per_block;
  if (gx == 0) return;
  if (p.lut)
    hipLaunchKernelGGL((k_quantize_pack<D, NG, VROT, true>), dim3(gx, p.num_kv_heads), dim3(64 * W), 0, s, q);
  else
    hipLaunchKernelGGL((k_quantize_pack<D, NG, VROT, false>), dim3(gx, p.num_kv_heads), dim3(64 * W), 0, s, q);
}
template <int D, int NG>
void launch_qp(const WriteParams& p, hipStream_t s) {
  if (p.r_v)
    launch_qp_v<D, NG, true>(p, s);
  else
    launch_qp_v<D, NG, false>(p, s);
}

template <int D>
void launch_wb(const WriteParams& p, int first_position, hipStream_t s) {
  if (p.num_tokens <= 0) return;
  const int first_lp = first_position / kPage;
  const int last_lp = (first_position + p.num_tokens - 1) / kPage;
  hipLaunchKernelGGL((k_write_bf16<D>), dim3(last_lp - first_lp + 1, p.num_kv_heads), dim3(256), 0, s, p,
                     first_position);
}

}  // namespace

bool launch_write_bf16(const WriteParams& p, int head_dim, int first_position, hipStream_t stream) {
  if (head_dim == 128) return launch_wb<128>(p, first_position, stream), true;
  if (head_dim == 64) return launch_wb<64>(p, first_position, stream), true;
  return false;
}

bool launch_append_demote(const WriteParams& p, int head_dim, int n_groups, hipStream_t stream) {
  if (head_dim == 128 && n_groups == 1) return launch_ad<128, 1>(p, stream), true;
  if (head_dim == 128 && n_groups == 2) return launch_ad<128, 2>(p, stream), true;
  if (head_dim == 64 && n_groups == 1) return launch_ad<64, 1>(p, stream), true;
  return false;
}

bool launch_quantize_pack(const WriteParams& p, int head_dim, int n_groups, hipStream_t stream) {
  if (head_dim == 128 && n_groups == 1) return launch_qp<128, 1>(p, stream), true;
  if (head_dim == 128 && n_groups == 2) return launch_qp<128, 2>(p, stream), true;
  if (head_dim == 64 && n_groups == 1) return launch_qp<64, 1>(p, stream), true;
  return false;
}

}  // namespace oscar
