// Offline calibration and the rotation error chain on gfx950, in fp32.
//
// What is computed (MarkTechPost article on OSCAR, "What OSCAR Does
// Differently"; ModelScope/CSDN page, design section and motivation section
// with its Figure 1):
//   gram        C = scale * X^T X per head: the query covariance C_Q over the
//               calibration queries of a KV head's query heads, and, applied
//               to the causal attention outputs O = S V, the score-weighted
//               value covariance C_S = (1/N) V^T S^T S V;
//   attention   causal softmax attention of the calibration draw (S V);
//   rotation    eigenvectors U of C by one-sided (Hestenes) Jacobi, ordered
//               by descending eigenvalue, each column's largest-magnitude
//               entry made positive, then R = U H P_br (Walsh-Hadamard by an
//               in-LDS butterfly, bit-reversed output columns);
//   clip        tau = a quantile of |x R| (linear interpolation between order
//               statistics), the order statistics found by radix selection
//               over the fp32 bit patterns of |x R|;
//   codebook    the normalized values t = c/s + z of the calibration set (the
//               write path's arithmetic) and fixed-end Lloyd-Max on them;
//   dequantize  INT2 pool pages back to dense vectors, s (L[code] - z) R^T
//               (L the pool's levels, 0..3 unless it uses a codebook);
//   error       the causal attention of the reference and of the quantized
//               keys/values side by side: per query row the score KL, the
//               summed squared logit error and the output error.
//
// Dense contractions (gram, attention, x R) run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).  Operand layout of that instruction, for lane l:
// A[l % 16][l / 16], B[l / 16][l % 16], and D[4 (l / 16) + r][l % 16] in
// accumulator element r.  The summation index of one instruction may be any
// bijection onto the 4 k-slots as long as A and B use the same one; the
// attention uses that freedom so that the softmax weights a lane holds in its
// score accumulator are exactly the P operand it feeds to P.V.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace oscar {
namespace {

constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ float ld1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ v4f ld4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return v4f{__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3])};
}
__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// sums / maxima over the 4 lanes l, l^16, l^32, l^48 (the gfx950 permlane
// swaps exchange 16-lane rows 0<->1, 2<->3 and the two 32-lane halves)
__device__ __forceinline__ float col4_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float col4_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// sum over all 64 lanes, result in every lane
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_row_ror<8>(x);
  x += dpp_row_ror<4>(x);
  x += dpp_row_ror<2>(x);
  x += dpp_row_ror<1>(x);
  return col4_sum(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_row_ror<8>(x));
  x = fmaxf(x, dpp_row_ror<4>(x));
  x = fmaxf(x, dpp_row_ror<2>(x));
  x = fmaxf(x, dpp_row_ror<1>(x));
  return col4_max(x);
}

// ---------------------------------------------------------------------------
// gram: part[split][h] = X[h][rows of split]^T X[h][rows of split]
// ---------------------------------------------------------------------------
// Grid (splits, heads), 4 waves; wave w owns the (D/2 x D/2) output quadrant
// (w / 2, w % 2) as (D/32)^2 tiles of 16 x 16.  Every instruction consumes 4
// rows: A = X[rows][i-tile]^T, B = X[rows][j-tile].
template <int D>
__global__ void __launch_bounds__(256) k_gram(const GramParams p) {
  constexpr int TW = D / 32;
  const int split = blockIdx.x, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ib = (wave >> 1) * (D / 2), jb = (wave & 1) * (D / 2);
  const int r_begin = split * p.rows_per_split;
  const int r_end = min(p.rows, r_begin + p.rows_per_split);
  const auto x = rsrc(p.x + (size_t)h * p.head_stride, (uint32_t)((size_t)p.rows * p.row_stride * 4));
  v4f acc[TW][TW];
#pragma unroll
  for (int a = 0; a < TW; ++a)
#pragma unroll
    for (int b = 0; b < TW; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
  const int col = lane & 15, sub = lane >> 4;
  // rows_per_split is a multiple of 16: only the last split can reach past
  // `rows`, and those rows read as zero
  for (int r0 = r_begin; r0 < r_end; r0 += 16) {
    float av[4][TW], bv[4][TW];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t row_off = (uint32_t)(r0 + 4 * u + sub) * (uint32_t)p.row_stride * 4u;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        av[u][t] = ld1(x, row_off + (ib + 16 * t + col) * 4);
        bv[u][t] = ld1(x, row_off + (jb + 16 * t + col) * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int a = 0; a < TW; ++a)
#pragma unroll
        for (int b = 0; b < TW; ++b) acc[a][b] = mfma4(av[u][a], bv[u][b], acc[a][b]);
  }
  float* out = p.part + ((size_t)split * p.heads + h) * D * D;
#pragma unroll
  for (int a = 0; a < TW; ++a)
#pragma unroll
    for (int b = 0; b < TW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(ib + 16 * a + 4 * sub + r) * D + jb + 16 * b + col] = acc[a][b][r];
}

// out[h] = scale * sum over splits of part[split][h], summed in split order
__global__ void __launch_bounds__(256) k_gram_reduce(const GramParams p, int dd) {
  const size_t n = (size_t)p.heads * dd;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int k = 0; k < p.splits; ++k) s += p.part[(size_t)k * n + e];
    p.out[e] = s * p.scale;
  }
}

// ---------------------------------------------------------------------------
// causal attention of the calibration draw; with ERR the reference and the
// quantized keys / values side by side
// ---------------------------------------------------------------------------
// One wave per (16-row query block, KV head, query head); a workgroup holds 4
// such tasks, the longest query blocks first.  Scores are computed transposed,
// S^T = K Q^T (keys on rows), so that the 16 queries are the accumulator
// columns: lane l owns query l % 16 and keys 4 (l / 16) + r of each 16-key
// tile.  The channel order of the score contraction is c = (D/4) (l / 16) + s
// at step s, so each lane reads a contiguous run of D/4 channels of its row.
// P.V computes O^T = V^T P^T with key order 4 (l / 16) + s at step s (the
// lane's own score element s) and output channel NT i + t for row i of
// channel tile t, so each lane's V operands and outputs are contiguous runs.
template <int D, bool ERR>
__global__ void __launch_bounds__(256) k_calib_attention(const CalibAttnParams p) {
  constexpr int KS = D / 4;   // score contraction steps
  constexpr int NT = D / 16;  // output channel tiles
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nblk = (p.tokens + 15) / 16;
  const int per_blk = p.kv_heads * p.gqa;
  const int task = blockIdx.x * 4 + wave;
  if (task >= nblk * per_blk) return;
  const int blk = nblk - 1 - task / per_blk;
  const int h = (task % per_blk) / p.gqa, hq = task % p.gqa;
  const int col = lane & 15, sub = lane >> 4;
  const int qrow = blk * 16 + col;
  const size_t qhead = (size_t)h * p.gqa + hq;

  const uint32_t qbytes = (uint32_t)((size_t)p.tokens * D * 4);
  const auto qr = rsrc(p.q + qhead * p.tokens * D, qbytes);
  const uint32_t kvbytes = (uint32_t)(((size_t)(p.tokens - 1) * p.kv_ns + D) * 4);
  const auto kr = rsrc(p.k + (size_t)h * p.kv_hs, kvbytes);
  const auto vr = rsrc(p.v + (size_t)h * p.kv_hs, kvbytes);
  __amdgpu_buffer_rsrc_t khr = kr, vhr = vr;
  if constexpr (ERR) {
    khr = rsrc(p.k_hat + (size_t)h * p.kv_hs, kvbytes);
    vhr = rsrc(p.v_hat + (size_t)h * p.kv_hs, kvbytes);
  }

  float qv[KS];
#pragma unroll
  for (int s4 = 0; s4 < KS / 4; ++s4) {
    const v4f x = ld4(qr, (uint32_t)(qrow * D + KS * sub + 4 * s4) * 4u);
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[4 * s4 + e] = x[e] * p.scale_log2;
  }
  v4f o[NT], oh[ERR ? NT : 1];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  if constexpr (ERR) {
#pragma unroll
    for (int t = 0; t < NT; ++t) oh[t] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float m = -INFINITY, zl = 0.f, zh = 0.f, bsum = 0.f, l2sum = 0.f;

  for (int kt = 0; kt <= blk; ++kt) {
    const int key0 = kt * 16;
    const uint32_t krow = (uint32_t)(key0 + col) * (uint32_t)p.kv_ns * 4u + (uint32_t)(KS * sub) * 4u;
    v4f sc = v4f{0.f, 0.f, 0.f, 0.f}, sch = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < KS / 4; ++s4) {
      const v4f kx = ld4(kr, krow + 16u * s4);
#pragma unroll
      for (int e = 0; e < 4; ++e) sc = mfma4(kx[e], qv[4 * s4 + e], sc);
      if constexpr (ERR) {
        const v4f hx = ld4(khr, krow + 16u * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sch = mfma4(hx[e], qv[4 * s4 + e], sch);
      }
    }
    // causal mask (only the diagonal tile has masked keys)
    float mt = -INFINITY;
    bool valid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      valid[r] = key0 + 4 * sub + r <= qrow;
      if (!valid[r]) {
        sc[r] = -INFINITY;
        sch[r] = -INFINITY;
      }
      mt = fmaxf(mt, sc[r]);
      if constexpr (ERR) mt = fmaxf(mt, sch[r]);
    }
    mt = col4_max(mt);
    const float m_new = fmaxf(m, mt);
    const float alpha = exp2f(m - m_new);
    m = m_new;
    float pr[4], ph[4];
    float ps = 0.f, phs = 0.f, bs = 0.f, l2 = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = exp2f(sc[r] - m_new);
      ps += pr[r];
      if constexpr (ERR) {
        ph[r] = exp2f(sch[r] - m_new);
        phs += ph[r];
        const float d = valid[r] ? sch[r] - sc[r] : 0.f;
        bs += pr[r] * d;
        l2 += d * d;
      }
    }
    zl = zl * alpha + ps;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] *= alpha;
    if constexpr (ERR) {
      zh = zh * alpha + phs;
      bsum = bsum * alpha + bs;
      l2sum += l2;
#pragma unroll
      for (int t = 0; t < NT; ++t) oh[t] *= alpha;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t vrow = (uint32_t)(key0 + 4 * sub + s) * (uint32_t)p.kv_ns * 4u + (uint32_t)(NT * col) * 4u;
      float vv[NT], hv[NT];
#pragma unroll
      for (int t4 = 0; t4 < NT / 4; ++t4) {
        const v4f x = ld4(vr, vrow + 16u * t4);
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[4 * t4 + e] = x[e];
        if constexpr (ERR) {
          const v4f y = ld4(vhr, vrow + 16u * t4);
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[4 * t4 + e] = y[e];
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] = mfma4(vv[t], pr[s], o[t]);
      if constexpr (ERR) {
#pragma unroll
        for (int t = 0; t < NT; ++t) oh[t] = mfma4(hv[t], ph[s], oh[t]);
      }
    }
  }

  const float z = col4_sum(zl);
  const float inv = 1.f / z;
  const bool row_ok = qrow < p.tokens;
  if constexpr (!ERR) {
    if (row_ok) {
      // lane owns channels 4 NT sub + (NT r + t)
      float* dst = p.out + (qhead * p.tokens + qrow) * D + 4 * NT * sub;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t4 = 0; t4 < NT / 4; ++t4)
          *(v4f*)(dst + NT * r + 4 * t4) =
              v4f{o[4 * t4][r] * inv, o[4 * t4 + 1][r] * inv, o[4 * t4 + 2][r] * inv, o[4 * t4 + 3][r] * inv};
      if (p.lse && sub == 0) p.lse[qhead * p.tokens + qrow] = (m + log2f(z)) * kLn2;
    }
  } else {
    const float zq = col4_sum(zh), b = col4_sum(bsum), l2 = col4_sum(l2sum);
    const float invh = 1.f / zq;
    float se = 0.f, sq = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = o[t][r] * inv, d = a - oh[t][r] * invh;
        se += d * d;
        sq += a * a;
      }
    se = col4_sum(se);
    sq = col4_sum(sq);
    if (row_ok && sub == 0) {
      // KL(p || p^) = sum_t p_t (l_t - l^_t) + ln(Z^ / Z), both sums taken
      // against the same running maximum; d = l^ - l in log2 units
      const float kl = logf(zq * inv) - kLn2 * b * inv;
      *(v4f*)(p.stats + (qhead * p.tokens + qrow) * 4) = v4f{kl, l2 * kLn2 * kLn2, se, sq};
    }
  }
}

// ---------------------------------------------------------------------------
// eigenbasis and rotation: one workgroup of D/8 waves per head
// ---------------------------------------------------------------------------
constexpr int kMaxSweeps = 24;
constexpr int kRefineSweeps = 6;
constexpr float kJacobiTol = 1.0e-6f;

// Pair k of round r of a round-robin tournament over 0..D-1: every index is
// in exactly one pair per round and every pair meets once in D-1 rounds.
template <int D>
__device__ __forceinline__ void tournament_pair(int r, int k, int& a, int& b) {
  if (k == 0) {
    a = D - 1;
    b = r;
  } else {
    a = r + k;
    a -= a >= D - 1 ? D - 1 : 0;
    b = r - k;
    b += b < 0 ? D - 1 : 0;
  }
}

template <int D>
struct EigSmem {
  float w[D * D];  // column-major working matrix W = C V (later U)
  float v[D * D];  // column-major accumulated rotations V
  float lam[D];
  float nrm[D];  // squared column norms of W during a sweep
  int pos[D];
  int rotated;
};

template <int D>
__global__ void __launch_bounds__(64 * (D / 8)) k_eigen_rotation(const EigParams p) {
  constexpr int NTHR = 64 * (D / 8);
  constexpr int RL = D / 64;        // rows per lane in whole-wave loops; 16-byte pieces per lane in sweeps
  constexpr int PPW = 4;            // pairs per wave per round (D/2 pairs, D/8 waves), one per 16-lane row
  extern __shared__ __align__(16) unsigned char smem_raw[];
  EigSmem<D>& sm = *reinterpret_cast<EigSmem<D>*>(smem_raw);
  const int h = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool second = h >= p.split;
  const int hm = second ? h - p.split : h;
  const float* c = (second ? p.cov2 : p.cov) + (size_t)hm * D * D;
  float* const eigvals = second ? p.eigvals2 : p.eigvals;
  for (int e = tid; e < D * D; e += NTHR) {
    const int row = e / D, cl = e % D;
    sm.w[cl * D + row] = c[e];
    sm.v[cl * D + row] = row == cl ? 1.f : 0.f;
  }
  __syncthreads();

  // one-sided Jacobi: rotate column pairs of W (and V) until all columns of
  // W are mutually orthogonal; then W = V diag(lambda) and V holds the
  // eigenvectors.  Rotations that mix a large column into a small one leak
  // their rounding into it, so after convergence V is renormalized, W is
  // formed again as C V from the input, and a few more sweeps remove what
  // the accumulated rounding had hidden.
  for (int phase = 0; phase < 2; ++phase) {
  if (phase == 1) {
    for (int i = wave; i < D; i += D / 8) {
      float nrm = 0.f;
#pragma unroll
      for (int u = 0; u < RL; ++u) nrm += sm.v[i * D + lane + 64 * u] * sm.v[i * D + lane + 64 * u];
      const float inv = 1.f / sqrtf(wave_sum(nrm));
#pragma unroll
      for (int u = 0; u < RL; ++u) sm.v[i * D + lane + 64 * u] *= inv;
    }
    __syncthreads();
    // W[:, col] = C V[:, col]; C is symmetric, so row j of c is column j
    for (int e = tid; e < D * D; e += NTHR) {
      const int cl = e / D, row = e % D;
      float acc = 0.f;
      for (int j = 0; j < D; ++j) acc = fmaf(c[j * D + row], sm.v[cl * D + j], acc);
      sm.w[cl * D + row] = acc;
    }
    __syncthreads();
  }
  for (int sweep = 0; sweep < (phase == 0 ? kMaxSweeps : kRefineSweeps); ++sweep) {
    // exact squared column norms at the start of every sweep; within the
    // sweep a rotation updates them as alpha - t gamma and beta + t gamma
    for (int i = wave; i < D; i += D / 8) {
      float sq = 0.f;
#pragma unroll
      for (int u = 0; u < RL; ++u) sq += sm.w[i * D + lane + 64 * u] * sm.w[i * D + lane + 64 * u];
      sq = wave_sum(sq);
      if (lane == 0) sm.nrm[i] = sq;
    }
    if (tid == 0) sm.rotated = 0;
    __syncthreads();
    int any = 0;
    // each 16-lane row of a wave owns one pair per round; lane sl of the row
    // holds rows 4 sl + 64 j + e (e < 4) of the pair's columns, so a row of
    // lanes reads a column as contiguous 16-byte pieces
    const int grp = lane >> 4, sl = lane & 15;
    for (int r = 0; r < D - 1; ++r) {
      int pa, pb;
      tournament_pair<D>(r, wave * PPW + grp, pa, pb);
      v4f xa[RL], xb[RL];
      float sg = 0.f;
#pragma unroll
      for (int j = 0; j < RL; ++j) {
        xa[j] = *(const v4f*)&sm.w[pa * D + 64 * j + 4 * sl];
        xb[j] = *(const v4f*)&sm.w[pb * D + 64 * j + 4 * sl];
#pragma unroll
        for (int e = 0; e < 4; ++e) sg = fmaf(xa[j][e], xb[j][e], sg);
      }
      sg += dpp_row_ror<8>(sg);
      sg += dpp_row_ror<4>(sg);
      sg += dpp_row_ror<2>(sg);
      const float ga = sg + dpp_row_ror<1>(sg);
      const float al = sm.nrm[pa], be = sm.nrm[pb];
      if (fabsf(ga) > kJacobiTol * __builtin_amdgcn_sqrtf(al * be) && ga != 0.f) {
        any = 1;
        const float zeta = (be - al) * __builtin_amdgcn_rcpf(2.f * ga);
        const float az = fabsf(zeta);
        const float t = copysignf(az > 1.0e18f ? 0.5f * __builtin_amdgcn_rcpf(az)
                                               : __builtin_amdgcn_rcpf(az + __builtin_amdgcn_sqrtf(1.f + az * az)),
                                  zeta);
        const float cs = __builtin_amdgcn_rsqf(1.f + t * t), sn = cs * t;
#pragma unroll
        for (int j = 0; j < RL; ++j) {
          const int ia = pa * D + 64 * j + 4 * sl, ib = pb * D + 64 * j + 4 * sl;
          const v4f va = *(const v4f*)&sm.v[ia], vb = *(const v4f*)&sm.v[ib];
          *(v4f*)&sm.w[ia] = cs * xa[j] - sn * xb[j];
          *(v4f*)&sm.w[ib] = sn * xa[j] + cs * xb[j];
          *(v4f*)&sm.v[ia] = cs * va - sn * vb;
          *(v4f*)&sm.v[ib] = sn * va + cs * vb;
        }
        if (sl == 0) {
          sm.nrm[pa] = al - t * ga;
          sm.nrm[pb] = be + t * ga;
        }
      }
      __syncthreads();
    }
    if (any) sm.rotated = 1;  // every writer stores the same value
    __syncthreads();
    const int again = sm.rotated;
    __syncthreads();
    if (!again) break;
  }
  }

  // eigenvalue of column i: the Rayleigh quotient v_i^T C v_i with C read
  // again (W carries the rounding of every rotation); sign: the column's
  // largest-magnitude entry (first on ties) made positive
  for (int e = tid; e < D * D; e += NTHR) sm.w[(e % D) * D + e / D] = c[e];
  __syncthreads();
  for (int i = wave; i < D; i += D / 8) {
    float dot = 0.f, amax = 0.f, nrm = 0.f;
#pragma unroll
    for (int u = 0; u < RL; ++u) {
      const int row = lane + 64 * u;
      float cv = 0.f;
      for (int j = 0; j < D; ++j) cv = fmaf(sm.w[j * D + row], sm.v[i * D + j], cv);
      const float x = sm.v[i * D + row];
      dot += x * cv;
      nrm += x * x;
      amax = fmaxf(amax, fabsf(x));
    }
    dot = wave_sum(dot);
    nrm = wave_sum(nrm);
    amax = wave_max(amax);
    float first = (float)D;
#pragma unroll
    for (int u = RL - 1; u >= 0; --u)
      if (fabsf(sm.v[i * D + lane + 64 * u]) == amax) first = (float)(lane + 64 * u);
    first = fminf(-wave_max(-first), (float)(D - 1));
    // the accumulated rotations drift from unit length by ~1e-5 over the
    // sweeps: renormalize (after every lane has read the column)
    const float inv = 1.f / sqrtf(nrm);
    const float sg = sm.v[i * D + (int)first] > 0.f ? inv : -inv;
#pragma unroll
    for (int u = 0; u < RL; ++u) sm.v[i * D + lane + 64 * u] *= sg;
    if (lane == 0) sm.lam[i] = dot / nrm;
  }
  __syncthreads();
  if (tid < D) {
    const float li = sm.lam[tid];
    int rank = 0;
    for (int j = 0; j < D; ++j) {
      const float lj = sm.lam[j];
      rank += (lj > li || (lj == li && j < tid)) ? 1 : 0;
    }
    sm.pos[tid] = rank;
  }
  __syncthreads();
  // U (column-major) into the W area: U[:, pos(i)] = V[:, i]
  for (int e = tid; e < D * D; e += NTHR) {
    const int i = e / D, row = e % D;
    sm.w[sm.pos[i] * D + row] = sm.v[i * D + row];
  }
  if (eigvals && tid < D) eigvals[(size_t)hm * D + sm.pos[tid]] = sm.lam[tid];
  __syncthreads();
  if (p.mix) {
    // rows of U times the Sylvester Hadamard matrix: butterflies over the
    // column index, (a, b) -> (a + b, a - b) for every bit
    for (int bit = 1; bit < D; bit <<= 1) {
      for (int e = tid; e < D * D / 2; e += NTHR) {
        const int row = e % D, pr = e / D;  // pair index over columns
        const int lo = ((pr & ~(bit - 1)) << 1) | (pr & (bit - 1));
        const float a = sm.w[lo * D + row], b = sm.w[(lo + bit) * D + row];
        sm.w[lo * D + row] = a + b;
        sm.w[(lo + bit) * D + row] = a - b;
      }
      __syncthreads();
    }
  }
  const float norm = p.mix ? 1.f / sqrtf((float)D) : 1.f;
  constexpr int LOG = D == 128 ? 7 : 6;
  float* out = (second ? p.r_out2 : p.r_out) + (size_t)hm * D * D;
  for (int e = tid; e < D * D; e += NTHR) {
    const int row = e / D, j = e % D;
    // output column j takes column br(j) of U H
    const int src = p.mix ? (int)(__builtin_bitreverse32((uint32_t)j) >> (32 - LOG)) : j;
    out[e] = sm.w[src * D + row] * norm;
  }
}

// ---------------------------------------------------------------------------
// clip thresholds: |x R| as ordered keys, then radix selection
// ---------------------------------------------------------------------------
// k_rotate_abs: grid (row blocks, heads), 4 waves, R in LDS.  Each wave forms
// 16 rows of y = x R (D/16 output tiles) and stores the bit patterns of |y|,
// which order like the values since they are non-negative.
template <int D>
__global__ void __launch_bounds__(256) k_rotate_abs(const ClipParams p) {
  constexpr int NT = D / 16;
  __shared__ float rs[D * D];
  const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, sub = lane >> 4;
  const bool rot = p.r != nullptr;
  if (rot) {
    const float* r = p.r + (size_t)h * D * D;
    for (int e = tid; e < D * D; e += 256) rs[e] = r[e];
  }
  __syncthreads();
  const auto x = rsrc(p.x + (size_t)h * p.head_stride, (uint32_t)((size_t)p.rows * p.row_stride * 4));
  uint32_t* keys = p.keys + (size_t)h * p.rows * D;
  const int nblk = (p.rows + 15) / 16;
  for (int blk = blockIdx.x * 4 + wave; blk < nblk; blk += gridDim.x * 4) {
    const int row0 = blk * 16;
    if (rot) {
      v4f acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
      // A = x[16 rows][4 channels], B = R[4 channels][16 columns]
      for (int s = 0; s < D / 4; ++s) {
        const float a = ld1(x, ((uint32_t)(row0 + col) * (uint32_t)p.row_stride + 4 * s + sub) * 4u);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma4(a, rs[(4 * s + sub) * D + 16 * t + col], acc[t]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row0 + 4 * sub + r;
          if (row < p.rows) keys[(size_t)row * D + 16 * t + col] = __float_as_uint(fabsf(acc[t][r]));
        }
    } else {
      for (int e = lane; e < 16 * D; e += 64) {
        const int row = row0 + e / D;
        if (row < p.rows)
          keys[(size_t)row * D + e % D] =
              __float_as_uint(fabsf(ld1(x, ((uint32_t)row * (uint32_t)p.row_stride + e % D) * 4u)));
      }
    }
  }
}

// Radix selection, 8 bits per pass from the top.  sel[h][2] holds, per head
// and target order statistic, {prefix of the key so far, rank among keys
// with that prefix}.  Pass `pass` histograms digit (3 - pass) of the keys
// whose upper bits match the prefix.
__global__ void __launch_bounds__(256) k_select_hist(const ClipParams p, int pass) {
  __shared__ uint32_t hist[2][256];
  const int h = blockIdx.y, tid = threadIdx.x;
  hist[0][tid] = 0;
  hist[1][tid] = 0;
  __syncthreads();
  const size_t m = (size_t)p.rows * p.dim;
  const uint32_t* keys = p.keys + (size_t)h * m;
  const int shift = 24 - 8 * pass;
  uint32_t pre0 = 0, pre1 = 0;
  if (pass > 0) {
    pre0 = p.sel[(h * 2 + 0) * 2];
    pre1 = p.sel[(h * 2 + 1) * 2];
  }
  const size_t chunk = (m + gridDim.x - 1) / gridDim.x;
  const size_t b = chunk * blockIdx.x, e = min(m, b + chunk);
  for (size_t i = b + tid; i < e; i += 256) {
    const uint32_t k = keys[i];
    const uint32_t hi = pass > 0 ? k >> (shift + 8) : 0u;
    const uint32_t d = (k >> shift) & 255u;
    if (hi == pre0) atomicAdd(&hist[0][d], 1u);
    if (hi == pre1) atomicAdd(&hist[1][d], 1u);
  }
  __syncthreads();
  uint32_t* dst = p.hist + ((size_t)h * gridDim.x + blockIdx.x) * 512;
  dst[tid] = hist[0][tid];
  dst[256 + tid] = hist[1][tid];
}

// One workgroup per head: sum the chunk histograms, find the digit holding
// each target rank, extend the prefix.  The last pass turns the two order
// statistics into tau = a + t (b - a) (fp64, rounded to fp32).
__global__ void __launch_bounds__(256) k_select_scan(const ClipParams p, int pass, int chunks) {
  __shared__ uint32_t cum[2][256];
  __shared__ uint32_t res[2][2];
  const int h = blockIdx.x, tid = threadIdx.x;
  uint32_t tot[2] = {0u, 0u};
  const uint32_t* hp = p.hist + (size_t)h * chunks * 512 + tid;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) {
    tot[0] += hp[(size_t)c * 512];
    tot[1] += hp[(size_t)c * 512 + 256];
  }
  cum[0][tid] = tot[0];
  cum[1][tid] = tot[1];
  __syncthreads();
  // inclusive prefix sums over the 256 digits
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t a = cum[0][tid] + (tid >= off ? cum[0][tid - off] : 0u);
    const uint32_t b = cum[1][tid] + (tid >= off ? cum[1][tid - off] : 0u);
    __syncthreads();
    cum[0][tid] = a;
    cum[1][tid] = b;
    __syncthreads();
  }
  for (int t = 0; t < 2; ++t) {
    uint32_t prefix, rank;
    if (pass == 0) {
      prefix = 0;
      rank = t == 0 ? p.rank_lo : p.rank_hi;
    } else {
      prefix = p.sel[(h * 2 + t) * 2];
      rank = p.sel[(h * 2 + t) * 2 + 1];
    }
    const uint32_t below = cum[t][tid] - tot[t];
    // the digit whose bucket holds the rank (the last digit takes any rest)
    if (below <= rank && (rank < cum[t][tid] || tid == 255)) {
      res[t][0] = (prefix << 8) | (uint32_t)tid;
      res[t][1] = rank - below;
    }
  }
  __syncthreads();
  if (tid < 2) {
    p.sel[(h * 2 + tid) * 2] = res[tid][0];
    p.sel[(h * 2 + tid) * 2 + 1] = res[tid][1];
  }
  if (pass == 3 && tid == 0) {
    const double a = (double)__uint_as_float(res[0][0]), b = (double)__uint_as_float(res[1][0]);
    p.tau[h] = (float)(a + p.frac * (b - a));
  }
}

// ---------------------------------------------------------------------------
// codebook calibration: normalized values, then fixed-end Lloyd-Max
// ---------------------------------------------------------------------------
// k_normalize: grid (row blocks, heads), 4 waves, R in LDS.  Each wave forms
// 16 rows of y = x R (as k_rotate_abs), clips them to +-tau, and per group of
// G channels of a row computes the write path's bf16 scale and zero and
// t = fl32(fl32(c / s) + z) for every value (IEEE divisions, as the write
// path's reference arithmetic).
__device__ __forceinline__ float row16_min(float x) {
  x = fminf(x, dpp_row_ror<8>(x));
  x = fminf(x, dpp_row_ror<4>(x));
  x = fminf(x, dpp_row_ror<2>(x));
  return fminf(x, dpp_row_ror<1>(x));
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_row_ror<8>(x));
  x = fmaxf(x, dpp_row_ror<4>(x));
  x = fmaxf(x, dpp_row_ror<2>(x));
  return fmaxf(x, dpp_row_ror<1>(x));
}

template <int D>
__global__ void __launch_bounds__(256) k_normalize(const CodebookParams p) {
  constexpr int NT = D / 16;
  __shared__ float rs[D * D];
  const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, sub = lane >> 4;
  const bool rot = p.r != nullptr;
  if (rot) {
    const float* r = p.r + (size_t)h * D * D;
    for (int e = tid; e < D * D; e += 256) rs[e] = r[e];
  }
  __syncthreads();
  const auto x = rsrc(p.x + (size_t)h * p.head_stride, (uint32_t)((size_t)p.rows * p.row_stride * 4));
  const float tau = p.tau[h];
  const int tiles_per_group = p.group_size / 16;
  float* tout = p.t + (size_t)h * p.rows * D;
  const int nblk = (p.rows + 15) / 16;
  for (int blk = blockIdx.x * 4 + wave; blk < nblk; blk += gridDim.x * 4) {
    const int row0 = blk * 16;
    v4f acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    if (rot) {
      for (int s = 0; s < D / 4; ++s) {
        const float a = ld1(x, ((uint32_t)(row0 + col) * (uint32_t)p.row_stride + 4 * s + sub) * 4u);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma4(a, rs[(4 * s + sub) * D + 16 * t + col], acc[t]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[t][r] = ld1(x, ((uint32_t)(row0 + 4 * sub + r) * (uint32_t)p.row_stride + 16 * t + col) * 4u);
    }
    // lane holds y[row0 + 4 sub + r][16 t + col]
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] = fminf(fmaxf(acc[t][r], -tau), tau);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * sub + r;
      for (int g = 0; g < D / p.group_size; ++g) {
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t / tiles_per_group == g) {
            mn = fminf(mn, acc[t][r]);
            mx = fmaxf(mx, acc[t][r]);
          }
        mn = row16_min(mn);
        mx = row16_max(mx);
        const float dl = mx - mn;
        float s = bf16_to_f32(f32_to_bf16(dl / 3.0f));
        if (dl == 0.f || s == 0.f) s = 1.f;
        const float z = bf16_to_f32(f32_to_bf16(-mn / s));
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t / tiles_per_group == g && row < p.rows)
            tout[(size_t)row * D + 16 * t + col] = __fadd_rn(acc[t][r] / s, z);
      }
    }
  }
}

// One Lloyd step, part 1: workgroup w sums (in fp64) the values of its
// chunk that fall in the cells [b0, b1) and [b1, b2) of the current levels.
__global__ void __launch_bounds__(256) k_lloyd_partial(const CodebookParams p) {
  __shared__ double red[4][256];
  const int tid = threadIdx.x;
  const double l1 = p.state[1], l2 = p.state[2];
  const double b0 = 0.5 * l1, b1 = 0.5 * (l1 + l2), b2 = 0.5 * (l2 + 3.0);
  const size_t n = (size_t)p.heads * p.rows * p.dim;
  const size_t chunk = (n + gridDim.x - 1) / gridDim.x;
  const size_t beg = chunk * blockIdx.x, end = min(n, beg + chunk);
  double s1 = 0.0, c1 = 0.0, s2 = 0.0, c2 = 0.0;
  for (size_t i = beg + tid; i < end; i += 256) {
    const double t = (double)p.t[i];
    if (t >= b0 && t < b1) {
      s1 += t;
      c1 += 1.0;
    } else if (t >= b1 && t < b2) {
      s2 += t;
      c2 += 1.0;
    }
  }
  red[0][tid] = s1;
  red[1][tid] = c1;
  red[2][tid] = s2;
  red[3][tid] = c2;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off)
#pragma unroll
      for (int k = 0; k < 4; ++k) red[k][tid] += red[k][tid + off];
    __syncthreads();
  }
  if (tid < 4) p.partial[(size_t)blockIdx.x * 4 + tid] = red[tid][0];
}

// part 2: sum the chunks in order and move each interior level to its cell's
// mean (an empty cell keeps its level); after the last step round the
// interior levels to the 1/32 grid and write the codebook.
__global__ void __launch_bounds__(64) k_lloyd_update(const CodebookParams p, int chunks, int last) {
  if (threadIdx.x != 0) return;
  double s1 = 0.0, c1 = 0.0, s2 = 0.0, c2 = 0.0;
  for (int w = 0; w < chunks; ++w) {
    s1 += p.partial[(size_t)w * 4 + 0];
    c1 += p.partial[(size_t)w * 4 + 1];
    s2 += p.partial[(size_t)w * 4 + 2];
    c2 += p.partial[(size_t)w * 4 + 3];
  }
  if (c1 > 0.0) p.state[1] = s1 / c1;
  if (c2 > 0.0) p.state[2] = s2 / c2;
  if (last) {
    p.levels[0] = 0.f;
    p.levels[1] = (float)(rint(p.state[1] * 32.0) / 32.0);
    p.levels[2] = (float)(rint(p.state[2] * 32.0) / 32.0);
    p.levels[3] = 3.f;
  }
}

__global__ void k_lloyd_init(const CodebookParams p) {
  if (threadIdx.x == 0) {
    p.state[0] = 0.0;
    p.state[1] = 1.0;
    p.state[2] = 2.0;
    p.state[3] = 3.0;
  }
}

// ---------------------------------------------------------------------------
// dequantize INT2 pages back to dense vectors in the model basis
// ---------------------------------------------------------------------------
// Grid (page chunks, KV heads), 4 waves.  R^T sits in LDS transposed so that
// the lanes of a wave read consecutive output channels.
template <int D, int NG>
__global__ void __launch_bounds__(256) k_dequantize(const DequantParams p) {
  constexpr int G = D / NG, BLK2 = 8 * D + 128 * NG, REC = D / 8;
  __shared__ float rt[D * D];    // rt[j][c] = R[c][j]
  __shared__ float yh[16][D];    // dequantized rotated page
  const int h = blockIdx.y, tid = threadIdx.x;
  const bool rot = p.r != nullptr;
  if (rot) {
    const float* r = p.r + (size_t)h * D * D;
    for (int e = tid; e < D * D; e += 256) rt[(e % D) * D + e / D] = r[e];
  }
  const int npages = (p.num_tokens + 15) / 16;
  for (int pg = blockIdx.x; pg < npages; pg += gridDim.x) {
    const int id = p.page_ids[pg];
    const bool ok = id >= 0 && id < p.int2_num_pages;
    const uint8_t* blk = p.int2_pool + ((size_t)(ok ? id : 0) * p.num_kv_heads + h) * BLK2;
    __syncthreads();  // previous page's yh fully consumed (and rt staged)
    for (int e = tid; e < 16 * D; e += 256) {
      const int tok = e / D, c = e % D;
      uint32_t code;
      if (p.which == 0) {
        // K: record 16 j + tok, word c / 64, channel c = w*64 + j*16 + m
        const int w = c / 64, j = (c / 16) % 4, mm = c % 16;
        const uint32_t word = *(const uint32_t*)(blk + (16 * j + tok) * REC + 4 * w);
        code = (word >> (2 * mm)) & 3u;
      } else {
        // V: record 16 (tok / 4) + (c % 16), word c / 64 after the K words,
        // channel block b = (c / 16) % 4, token slot i = tok % 4
        const int w = c / 64, bb = (c / 16) % 4, i = tok % 4;
        const uint32_t word = *(const uint32_t*)(blk + (16 * (tok / 4) + c % 16) * REC + 4 * (D / 64) + 4 * w);
        code = (word >> (16 * (i & 1) + 2 * (2 * bb + (i >> 1)))) & 3u;
      }
      const int q = tok / 4, g = c / G;
      const uint8_t* szp = blk + 8 * D + q * 32 * NG + (p.which ? 16 * NG : 0) + (tok % 4) * NG * 4 + g * 4;
      const uint32_t sz = *(const uint32_t*)szp;
      const float s = bf16_lo(sz), z = bf16_hi(sz);
      const float lvl = code == 0 ? p.levels[0] : code == 1 ? p.levels[1] : code == 2 ? p.levels[2] : p.levels[3];
      yh[tok][c] = ok ? s * (lvl - z) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < 16 * D; e += 256) {
      const int tok = e / D, c = e % D;
      const int t = pg * 16 + tok;
      float acc;
      if (rot) {
        acc = 0.f;
#pragma unroll 8
        for (int j = 0; j < D; ++j) acc = fmaf(yh[tok][j], rt[j * D + c], acc);
      } else {
        acc = yh[tok][c];
      }
      if (t < p.num_tokens) p.out[((size_t)t * p.num_kv_heads + h) * D + c] = acc;
    }
  }
}

}  // namespace

bool launch_gram(GramParams p, int dim, hipStream_t stream) {
  if (dim == 128)
    k_gram<128><<<dim3(p.splits, p.heads), 256, 0, stream>>>(p);
  else if (dim == 64)
    k_gram<64><<<dim3(p.splits, p.heads), 256, 0, stream>>>(p);
  else
    return false;
  const int dd = dim * dim;
  const int blocks = (int)std::min<size_t>(((size_t)p.heads * dd + 255) / 256, 2048);
  k_gram_reduce<<<blocks, 256, 0, stream>>>(p, dd);
  return true;
}

bool launch_calib_attention(const CalibAttnParams& p, int dim, bool err, hipStream_t stream) {
  const int tasks = ((p.tokens + 15) / 16) * p.kv_heads * p.gqa;
  const int grid = (tasks + 3) / 4;
  if (dim == 128) {
    if (err)
      k_calib_attention<128, true><<<grid, 256, 0, stream>>>(p);
    else
      k_calib_attention<128, false><<<grid, 256, 0, stream>>>(p);
  } else if (dim == 64) {
    if (err)
      k_calib_attention<64, true><<<grid, 256, 0, stream>>>(p);
    else
      k_calib_attention<64, false><<<grid, 256, 0, stream>>>(p);
  } else {
    return false;
  }
  return true;
}

bool launch_eigen_rotation(const EigParams& p, int dim, hipStream_t stream) {
  if (dim == 128) {
    constexpr size_t bytes = sizeof(EigSmem<128>);
    static bool attr = hipFuncSetAttribute((const void*)k_eigen_rotation<128>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
    if (!attr) return false;
    k_eigen_rotation<128><<<p.heads, 64 * 16, bytes, stream>>>(p);
  } else if (dim == 64) {
    constexpr size_t bytes = sizeof(EigSmem<64>);
    k_eigen_rotation<64><<<p.heads, 64 * 8, bytes, stream>>>(p);
  } else {
    return false;
  }
  return true;
}

bool launch_clip(const ClipParams& p, hipStream_t stream) {
  const int nblk = (p.rows + 15) / 16;
  const int gx = std::max(1, std::min((nblk + 3) / 4, std::max(1, 256 / p.heads)));
  if (p.dim == 128)
    k_rotate_abs<128><<<dim3(gx, p.heads), 256, 0, stream>>>(p);
  else if (p.dim == 64)
    k_rotate_abs<64><<<dim3(gx, p.heads), 256, 0, stream>>>(p);
  else
    return false;
  for (int pass = 0; pass < 4; ++pass) {
    k_select_hist<<<dim3(p.chunks, p.heads), 256, 0, stream>>>(p, pass);
    k_select_scan<<<p.heads, 256, 0, stream>>>(p, pass, p.chunks);
  }
  return true;
}

bool launch_codebook(const CodebookParams& p, int iterations, hipStream_t stream) {
  const int nblk = (p.rows + 15) / 16;
  const int gx = std::max(1, std::min((nblk + 3) / 4, std::max(1, 256 / p.heads)));
  if (p.dim == 128)
    k_normalize<128><<<dim3(gx, p.heads), 256, 0, stream>>>(p);
  else if (p.dim == 64)
    k_normalize<64><<<dim3(gx, p.heads), 256, 0, stream>>>(p);
  else
    return false;
  k_lloyd_init<<<1, 64, 0, stream>>>(p);
  for (int it = 0; it < iterations; ++it) {
    k_lloyd_partial<<<p.chunks, 256, 0, stream>>>(p);
    k_lloyd_update<<<1, 64, 0, stream>>>(p, p.chunks, it == iterations - 1);
  }
  return true;
}

bool launch_dequantize(const DequantParams& p, int dim, int n_groups, hipStream_t stream) {
  const int npages = (p.num_tokens + 15) / 16;
  const int gx = std::max(1, std::min(npages, std::max(1, 512 / p.num_kv_heads)));
  const dim3 grid(gx, p.num_kv_heads);
  if (dim == 128 && n_groups == 1)
    k_dequantize<128, 1><<<grid, 256, 0, stream>>>(p);
  else if (dim == 128 && n_groups == 2)
    k_dequantize<128, 2><<<grid, 256, 0, stream>>>(p);
  else if (dim == 64 && n_groups == 1)
    k_dequantize<64, 1><<<grid, 256, 0, stream>>>(p);
  else
    return false;
  return true;
}

}  // namespace oscar
