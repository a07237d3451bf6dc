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
__device__ __forceinline__ uint32_t quant_code(float c, float s, float z) {
  const float t = __fadd_rn(c / s, z);
  return (uint32_t)fminf(fmaxf(rintf(t), 0.f), 3.f);
}

// ------------------------------------------------------- append + demote --
template <int D, int NG>
__global__ void __launch_bounds__(256) k_append_demote(const WriteParams p) {
  constexpr int G = D / NG;
  constexpr int KW = D / 64;
  constexpr int BLK2 = 8 * D + 128 * NG;
  constexpr int REC = D / 8;
  __shared__ float r_s[D * D];
  __shared__ float kd[D];
  __shared__ float vv[D];
  __shared__ float yk[2][D];
  __shared__ float red[2][D / 64][2];  // [K/V][64-channel block][min, max]
  __shared__ uint8_t codes[2][D];
  __shared__ uint32_t sz[2][NG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int b = blockIdx.x / p.num_kv_heads, kvh = blockIdx.x % p.num_kv_heads;
  const int L = p.seq_lens[b];
  if (L < 0) return;
  const int32_t* bpt = p.bf16_pt + (size_t)b * p.bf16_pt_stride;
  const int32_t* ipt = p.int2_pt + (size_t)b * p.int2_pt_stride;
  const size_t hb = (size_t)kvh;

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
  if (dem) {
    const uint8_t* blk = p.bf16_pool + ((size_t)did * p.num_kv_heads + hb) * (64 * D);
    const int slot = d % kPage;
    if (tid < D) {
      kd[tid] = bf16_to_f32(((const uint16_t*)blk)[slot * D + tid]);
      vv[tid] = bf16_to_f32(((const uint16_t*)(blk + 32 * D))[(slot / 4) * D * 4 + tid * 4 + (slot % 4)]);
    }
    const uint4* rsrc = (const uint4*)(p.r_k + hb * D * D);
    for (int i = tid; i < D * D / 4; i += 256) ((uint4*)r_s)[i] = rsrc[i];
  }
  __syncthreads();  // the demoted token is read before the append writes
  if (app && tid < D) {
    uint8_t* blk = p.bf16_pool + ((size_t)aid * p.num_kv_heads + hb) * (64 * D);
    const int slot = L % kPage;
    const size_t src = ((size_t)b * p.num_kv_heads + hb) * D + tid;
    ((uint16_t*)blk)[slot * D + tid] = p.k_new[src];
    ((uint16_t*)(blk + 32 * D))[(slot / 4) * D * 4 + tid * 4 + (slot % 4)] = p.v_new[src];
  }
  if (!dem) return;

  // y = k_d R_K: thread (c, half) sums half of the input channels (fp32 FMA)
  if (tid < 2 * D) {
    const int c = tid % D, hlf = tid / D;
    float acc = 0.f;
    const int i0 = hlf * (D / 2);
#pragma unroll 8
    for (int i = i0; i < i0 + D / 2; ++i) acc = fmaf(kd[i], r_s[i * D + c], acc);
    yk[hlf][c] = acc;
  }
  __syncthreads();
  // waves: channels c of K (which = 0) or V (which = 1); each 64-lane wave
  // lies inside one group because G >= 64
  const int which = tid / D, c = tid % D;
  float x = 0.f;
  if (which < 2) {
    x = which == 0 ? yk[0][c] + yk[1][c] : vv[c];
    const float tau = which == 0 ? p.tau_k[hb] : p.tau_v[hb];
    x = fminf(fmaxf(x, -tau), tau);
    const float mn = wmin(x), mx = wmax(x);
    if (lane == 0) {
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
    codes[which][c] = (uint8_t)quant_code(x, s, z);
    if (c % G == 0) sz[which][g] = sb | (zb << 16);
  }
  __syncthreads();
  // pack into INT2 page iid, slot hs % 16
  uint8_t* blk = p.int2_pool + ((size_t)iid * p.num_kv_heads + hb) * BLK2;
  const int slot = hs % kPage, jq = slot / 4, ti = slot % 4;
  if (tid < 4 * KW) {  // K: records (j, slot), word w
    const int jj = tid / KW, w = tid % KW;
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 16; ++m) word |= (uint32_t)codes[0][w * 64 + jj * 16 + m] << (2 * m);
    *(uint32_t*)(blk + (16 * jj + slot) * REC + 4 * w) = word;
  } else if (tid >= 64 && tid < 64 + 16 * KW) {  // V: records (jq, r), word w
    const int r = (tid - 64) / KW, w = (tid - 64) % KW;
    uint32_t* dst = (uint32_t*)(blk + (16 * jq + r) * REC + D / 16 + 4 * w);
    uint32_t word = ti == 0 ? 0u : *dst;  // first token of a quad starts the word
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int pos = 16 * (ti & 1) + 2 * (2 * bb + (ti >> 1));
      word = (word & ~(3u << pos)) | ((uint32_t)codes[1][(4 * w + bb) * 16 + r] << pos);
    }
    *dst = word;
  } else if (tid >= 128 && tid < 128 + 2 * NG) {  // scale/zero words
    const int wh = (tid - 128) / NG, g = (tid - 128) % NG;
    *(uint32_t*)(blk + 8 * D + jq * 32 * NG + wh * 16 * NG + (ti * NG + g) * 4) = sz[wh][g];
  }
}

// ----------------------------------------------------------- bulk quantize --
// One workgroup per (compute unit, KV head slice) converts R_K once and then
// streams pages; each wave owns one page at a time and its own LDS area, so
// the page loop needs no workgroup barrier.  The next page's K and V are
// loaded while the current one is rotated and quantized.
constexpr int kQpWaves = 8;
constexpr int kQpThreads = 64 * kQpWaves;

template <int D, int NG>
struct BulkSmem {
  uint4 rb[2][D / 16][D / 32][64];  // R_hi / R_lo as MFMA B operands
  // per wave: the rotated K tile, whose space then holds the K / V codes
  union PerWave {
    float y[kPage][D + 4];
    uint8_t code[2][kPage][D];
  } w[kQpWaves];
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

// Quantizes one token's channels held by the 4 lanes of a quad (lane = 4t +
// qq): this lane holds channels w*64 + qq*16 + m (w < D/64, m < 16) in
// vals[w][m].  Codes come back one byte each, 16 per word group w.
template <int D, int NG>
__device__ __forceinline__ void quant_lane(float (&vals)[D / 64][16], float tau, uint32_t (&codes)[D / 64][4],
                                           uint32_t (&szw)[NG]) {
  constexpr int KW = D / 64;
  float mn[KW], mx[KW];
#pragma unroll
  for (int w = 0; w < KW; ++w) {
    mn[w] = INFINITY;
    mx[w] = -INFINITY;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float x = __builtin_amdgcn_fmed3f(vals[w][m], -tau, tau);
      vals[w][m] = x;
      mn[w] = fminf(mn[w], x);
      mx[w] = fmaxf(mx[w], x);
    }
    mn[w] = quad_min(mn[w]);
    mx[w] = quad_max(mx[w]);
  }
  // words of one group: NG == 1 -> all words; NG == 2 (D = 128) -> word w
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float gmn = INFINITY, gmx = -INFINITY;
#pragma unroll
    for (int w = 0; w < KW; ++w)
      if (NG == 1 || w == g) {
        gmn = fminf(gmn, mn[w]);
        gmx = fmaxf(gmx, mx[w]);
      }
    uint32_t sb, zb;
    float s, z;
    scale_zero(gmn, gmx, sb, zb, s, z);
    szw[g] = sb | (zb << 16);
    // Away from the ends of the fp32 range the quotient comes from the
    // reciprocal with one Markstein correction (exact: see div_bf16); the
    // rest of the groups take the IEEE division.
    const bool fast = s >= 0x1p-70f && fmaxf(fabsf(gmn), fabsf(gmx)) <= 0x1p56f;
    const float y = 1.0f / s;
#pragma unroll
    for (int w = 0; w < KW; ++w)
      if (NG == 1 || w == g) {
        if (fast) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) word = code_into(word, div_bf16(vals[w][4 * q + e], s, y), z, e);
            codes[w][q] = word;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) word = code_into(word, vals[w][4 * q + e] / s, z, e);
            codes[w][q] = word;
          }
        }
      }
  }
}

// 16 one-byte codes (4 per word, values 0..3) -> one 32-bit word, code m at
// bits 2m
__device__ __forceinline__ uint32_t pack16(uint4 b) {
  auto one = [](uint32_t u) {  // 4 codes -> 8 bits
    const uint32_t t = u | (u >> 6);              // bits 0-3: codes 0,1; bits 16-19: codes 2,3
    return (t & 0xFu) | ((t >> 12) & 0xF0u);
  };
  return one(b.x) | (one(b.y) << 8) | (one(b.z) << 16) | (one(b.w) << 24);
}

template <int D, int NG>
struct BulkPage {  // one page's global inputs, as loaded
  uint4 ka[D / 32];          // K tile as MFMA A operands: token r, channels j*D/4 + ks*8 + e
  uint4 va[D / 64][2];       // V of token t, channels w*64 + qq*16 + 0..15
  int id;                    // physical page (-1: none)
};

template <int D, int NG>
__device__ __forceinline__ void bulk_load(BulkPage<D, NG>& pg, const WriteParams& p, int kvh, int page, int pg_end,
                                          int lane) {
  constexpr int KB = D / 32, KW = D / 64;
  const int id = page < pg_end ? p.page_ids[page] : -1;
  pg.id = (id >= 0 && id < p.int2_num_pages) ? id : -1;
  const int j = lane >> 4, r = lane & 15, t = lane >> 2, qq = lane & 3;
  const int tok0 = page * kPage;
  {
    const bool ok = pg.id >= 0 && tok0 + r < p.num_tokens;
    const uint4* src = (const uint4*)(p.k + ((size_t)(ok ? tok0 + r : 0) * p.num_kv_heads + kvh) * D + j * (D / 4));
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) pg.ka[ks] = ok ? src[ks] : uint4{0u, 0u, 0u, 0u};
  }
  {
    const bool ok = pg.id >= 0 && tok0 + t < p.num_tokens;
    const uint16_t* src = p.v + ((size_t)(ok ? tok0 + t : 0) * p.num_kv_heads + kvh) * D;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      pg.va[w][0] = ok ? *(const uint4*)(src + w * 64 + qq * 16) : uint4{0u, 0u, 0u, 0u};
      pg.va[w][1] = ok ? *(const uint4*)(src + w * 64 + qq * 16 + 8) : uint4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D, int NG>
__device__ __forceinline__ void bulk_page(const BulkPage<D, NG>& pg, const WriteParams& p, BulkSmem<D, NG>& sm,
                                          int kvh, int page, int wave, int lane, float tau_k, float tau_v) {
  constexpr int KW = D / 64, KB = D / 32, OT = D / 16;
  constexpr int BLK2 = 8 * D + 128 * NG;
  constexpr int REC = D / 8;
  const int j = lane >> 4, r = lane & 15, t = lane >> 2, qq = lane & 3;
  const int tok0 = page * kPage;
  auto& pw = sm.w[wave];
  // ---- Y = K R_K on the bf16 matrix cores (R split hi + lo)
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) {
      const v8bf a = __builtin_bit_cast(v8bf, pg.ka[ks]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, sm.rb[0][ot][ks][lane]), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, sm.rb[1][ot][ks][lane]), c, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pw.y[4 * j + i][ot * 16 + r] = c[i];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ---- quantize K (lane = 4t + qq) and V
  const bool tok_ok = pg.id >= 0 && tok0 + t < p.num_tokens;
  uint32_t kc[KW][4], vc[KW][4], szk[NG], szv[NG];
  {
    float vals[KW][16];
#pragma unroll
    for (int w = 0; w < KW; ++w)
#pragma unroll
      for (int m = 0; m < 16; m += 4) {
        const float4 x = *(const float4*)&pw.y[t][w * 64 + qq * 16 + m];
        vals[w][m] = x.x;
        vals[w][m + 1] = x.y;
        vals[w][m + 2] = x.z;
        vals[w][m + 3] = x.w;
      }
    quant_lane<D, NG>(vals, tau_k, kc, szk);
  }
  {
    float vals[KW][16];
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      const uint32_t xs[8] = {pg.va[w][0].x, pg.va[w][0].y, pg.va[w][0].z, pg.va[w][0].w,
                              pg.va[w][1].x, pg.va[w][1].y, pg.va[w][1].z, pg.va[w][1].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        vals[w][2 * q] = bf16_lo(xs[q]);
        vals[w][2 * q + 1] = bf16_hi(xs[q]);
      }
    }
    quant_lane<D, NG>(vals, tau_v, vc, szv);
  }
  // codes of tokens past the last one are zero
#pragma unroll
  for (int w = 0; w < KW; ++w)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kc[w][q] = tok_ok ? kc[w][q] : 0u;
      vc[w][q] = tok_ok ? vc[w][q] : 0u;
    }
  uint8_t* blk = p.int2_pool + ((size_t)max(pg.id, 0) * p.num_kv_heads + kvh) * BLK2;
  // scales of token t (zeros for slots past the last token)
  if (pg.id >= 0 && qq < NG) {
    const int g = qq;
    uint32_t* sc = (uint32_t*)(blk + 8 * D + (t / 4) * 32 * NG);
    sc[(t % 4) * NG + g] = tok_ok ? szk[g] : 0u;
    sc[4 * NG + (t % 4) * NG + g] = tok_ok ? szv[g] : 0u;
  }
  // the codes overwrite the rotated tile: every lane of the wave has read it
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int w = 0; w < KW; ++w) {
    *(uint4*)&pw.code[0][t][w * 64 + qq * 16] = uint4{kc[w][0], kc[w][1], kc[w][2], kc[w][3]};
    *(uint4*)&pw.code[1][t][w * 64 + qq * 16] = uint4{vc[w][0], vc[w][1], vc[w][2], vc[w][3]};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ---- this lane's code record (j, r)
  uint32_t kwd[KW], vwd[KW];
#pragma unroll
  for (int w = 0; w < KW; ++w) {
    kwd[w] = pack16(*(const uint4*)&pw.code[0][r][w * 64 + j * 16]);
    uint32_t vword = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vword |= (uint32_t)pw.code[1][4 * j + i][(4 * w + bb) * 16 + r] << (16 * (i & 1) + 2 * (2 * bb + (i >> 1)));
    vwd[w] = vword;
  }
  if (pg.id >= 0) {
    if constexpr (D == 128) {
      *(uint4*)(blk + lane * REC) = uint4{kwd[0], kwd[1], vwd[0], vwd[1]};
    } else {
      *(uint2*)(blk + lane * REC) = uint2{kwd[0], vwd[0]};
    }
  }
  // the next page's tile reuses this wave's LDS
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int NG>
__global__ void __launch_bounds__(kQpThreads) k_quantize_pack(const WriteParams p) {
  constexpr int KB = D / 32, OT = D / 16;
  __shared__ BulkSmem<D, NG> sm;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int kvh = blockIdx.y;
  const int npages = (p.num_tokens + kPage - 1) / kPage;
  const int pg0 = blockIdx.x * p.pages_per_block;
  if (pg0 >= npages) return;
  const int pg_end = min(pg0 + p.pages_per_block, npages);
  BulkPage<D, NG> cur;
  bulk_load<D, NG>(cur, p, kvh, pg0 + wave, pg_end, lane);  // first page's loads overlap the R_K split
  // R_K (fp32) -> R_hi + R_lo (bf16) in B-operand order:
  // rb[hl][ot][ks][lane (j, n)] element e = R[j*D/4 + ks*8 + e][ot*16 + n]
  {
    const float* rk = p.r_k + (size_t)kvh * D * D;
    for (int idx = tid; idx < D * D / 8; idx += kQpThreads) {
      // eight consecutive input rows of one output column: one operand lane
      const int lane_op = idx % 64, ks = (idx / 64) % KB, ot = idx / (64 * KB);
      const int j = lane_op >> 4, n = lane_op & 15;
      const int in0 = j * (D / 4) + ks * 8, out = ot * 16 + n;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = rk[(size_t)(in0 + 2 * e) * D + out], x1 = rk[(size_t)(in0 + 2 * e + 1) * D + out];
        hi[e] = pack_bf16x2(x0, x1);
        lo[e] = pack_bf16x2(x0 - bf16_lo(hi[e]), x1 - bf16_hi(hi[e]));
      }
      sm.rb[0][ot][ks][lane_op] = uint4{hi[0], hi[1], hi[2], hi[3]};
      sm.rb[1][ot][ks][lane_op] = uint4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
  __syncthreads();
  const float tau_k = p.tau_k[kvh], tau_v = p.tau_v[kvh];
  // wave w handles pages pg0 + w, pg0 + w + kQpWaves, ...; two pages per trip
  // so that the current and next page alternate between two register sets
  BulkPage<D, NG> nxt;
  for (int pg = pg0 + wave; pg < pg_end; pg += 2 * kQpWaves) {
    bulk_load<D, NG>(nxt, p, kvh, pg + kQpWaves, pg_end, lane);
    bulk_page<D, NG>(cur, p, sm, kvh, pg, wave, lane, tau_k, tau_v);
    if (pg + kQpWaves >= pg_end) break;
    bulk_load<D, NG>(cur, p, kvh, pg + 2 * kQpWaves, pg_end, lane);
    bulk_page<D, NG>(nxt, p, sm, kvh, pg + kQpWaves, wave, lane, tau_k, tau_v);
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
  hipLaunchKernelGGL((k_append_demote<D, NG>), dim3(p.batch * p.num_kv_heads), dim3(256), 0, s, p);
}
template <int D, int NG>
void launch_qp(const WriteParams& p, hipStream_t s) {
  const int npages = (p.num_tokens + kPage - 1) / kPage;
  const int gx = (npages + p.pages_per_block - 1) / p.pages_per_block;
  if (gx == 0) return;
  hipLaunchKernelGGL((k_quantize_pack<D, NG>), dim3(gx, p.num_kv_heads), dim3(kQpThreads), 0, s, p);
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
