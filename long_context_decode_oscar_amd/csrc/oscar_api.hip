// Host side of liboscar: argument validation, pool layout, split-K planning,
// workspace layout and kernel launches behind the C ABI of include/oscar.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>

#include "../../include/oscar.h"
#include "common.h"
#include "kernels.h"

struct oscar_pool {
  oscar_config cfg;
  int n_groups;
  int gqa;
  float sm_scale;
  oscar_layout layout;
};

namespace {

thread_local std::string g_err;

oscar_status fail(oscar_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
oscar_status ok() {
  g_err.clear();
  return OSCAR_OK;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

oscar_status check_hip(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(OSCAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Number of compute units, for sizing the split-K grid (256 on MI355X).
int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

constexpr int kMaxChunks = 1024;
constexpr int kDecodeWaves = 8;  // waves per decode workgroup (decode.hip)

struct Plan {
  bool fits;  // false: the history needs more than kMaxChunks chunks
  int n_bf16_units, bf16_pages_per_unit, max_chunks, pages_per_chunk, units, slots, grid;
  size_t off_counters, off_lse, off_o, bytes;
};

int slots_for(int gqa) { return (16 / gqa) < 4 ? 16 / gqa : 4; }

// Longest INT2 chunk in pages: a decode wave holds the page ids of up to 64
// pages in one VGPR, 64 * kDecodeWaves per chunk; the D = 128, one-group
// kernels take a second batch in a second VGPR.
int chunk_cap(const oscar_config& c) {
  return (c.head_dim == 128 && c.group_size == 128 ? 128 : 64) * kDecodeWaves;
}

// Split-K plan.  Every (sequence, KV head) gets n_bf16_units workgroups for
// its sink + recent pages and up to max_chunks INT2 chunks of
// pages_per_chunk history pages; the chunk size is uniform so that shorter
// sequences simply use fewer chunks.  The grid aims at `target` workgroups
// (about one per compute unit, overridable with OSCAR_TARGET_WGS).
Plan make_plan(const oscar_pool* pool, int batch, int max_len, bool bf16_only) {
  const oscar_config& c = pool->cfg;
  Plan pl{};
  pl.fits = true;
  const int hkv = c.num_kv_heads;
  const int target = env_int("OSCAR_TARGET_WGS", num_cus());
  const int slots = slots_for(pool->gqa);
  max_len = max_len < 0 ? 0 : max_len;
  if (bf16_only) {
    const int npages = (max_len + oscar::kPage - 1) / oscar::kPage;
    pl.n_bf16_units = 0;
    pl.bf16_pages_per_unit = 0;
    int want = target / (batch * hkv);
    if (want < 1) want = 1;
    int ppc = (npages + want - 1) / want;
    ppc = ppc < 2 ? 2 : ((ppc + 1) / 2) * 2;
    pl.pages_per_chunk = ppc;
    pl.max_chunks = (npages + ppc - 1) / ppc;
    if (pl.max_chunks < 1) pl.max_chunks = 1;
  } else {
    const int list_max = c.sink_tokens / 16 + (c.recent_tokens + 15) / 16 + 1;
    const int per_unit = env_int("OSCAR_BF16_PAGES_PER_UNIT", 32);
    pl.n_bf16_units = (list_max + per_unit - 1) / per_unit;
    pl.bf16_pages_per_unit = (list_max + pl.n_bf16_units - 1) / pl.n_bf16_units;
    const int r0 = max_len - c.recent_tokens > c.sink_tokens ? max_len - c.recent_tokens : c.sink_tokens;
    const int hist_pages = (r0 - c.sink_tokens + 15) / 16;
    // INT2 chunks per (sequence, KV head) so that BF16 units + chunks fill
    // about `target` workgroups (one resident 8-wave workgroup per CU)
    int want = (target - batch * hkv * pl.n_bf16_units) / (batch * hkv);
    if (want < 1) want = 1;
    int ppc = (hist_pages + want - 1) / want;
    ppc = ((ppc + slots - 1) / slots) * slots;
    if (ppc < slots) ppc = slots;
    if (ppc > chunk_cap(c)) ppc = chunk_cap(c);
    pl.pages_per_chunk = ppc;
    pl.max_chunks = (hist_pages + ppc - 1) / ppc;
  }
  if (pl.max_chunks > kMaxChunks) {
    pl.fits = false;
    pl.max_chunks = kMaxChunks;
  }
  pl.units = pl.n_bf16_units + pl.max_chunks;
  if (pl.units < 1) pl.units = 1;
  pl.grid = batch * hkv * pl.units;
  pl.slots = pl.units;
  const size_t heads = (size_t)batch * hkv;
  const size_t parts = heads * pl.units * pool->gqa;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  pl.off_counters = 0;
  pl.off_lse = up(heads * oscar::kCounterStride * sizeof(uint32_t));
  pl.off_o = pl.off_lse + up(parts * sizeof(float));
  pl.bytes = pl.off_o + up(parts * c.head_dim * sizeof(float));
  return pl;
}

// ---- codebook ----
bool levels_ok(const float* l) {
  if (!(l[0] == 0.f && l[3] == 3.f && l[0] < l[1] && l[1] < l[2] && l[2] < l[3])) return false;
  for (int k = 1; k < 3; ++k)
    if (l[k] * 32.f != rintf(l[k] * 32.f)) return false;
  return true;
}
// byte c = scale * L[c] (exact integers for the valid levels)
uint32_t lut_word(const float* l, float scale) {
  uint32_t w = 0;
  for (int c = 0; c < 4; ++c) w |= ((uint32_t)lrintf(l[c] * scale) & 0xFFu) << (8 * c);
  return w;
}
void set_codebook(const oscar_pool* pool, oscar::DecodeParams& p) {
  p.lut = pool->cfg.codebook;
  p.lut_k = pool->cfg.codebook ? lut_word(pool->cfg.levels_k, 32.f) : 0u;
  p.lut_v = pool->cfg.codebook ? lut_word(pool->cfg.levels_v, 64.f) : 0u;
}
void set_codebook(const oscar_pool* pool, oscar::WriteParams& p) {
  p.lut = pool->cfg.codebook;
  for (int k = 0; k < 3; ++k) {
    p.thr_k[k] = 0.5f * (pool->cfg.levels_k[k] + pool->cfg.levels_k[k + 1]);
    p.thr_v[k] = 0.5f * (pool->cfg.levels_v[k] + pool->cfg.levels_v[k + 1]);
  }
}

// ---- prefix-shared (cascade) planning ----
struct CascPlan {
  int n = 0;              // units
  int max_chunks = 0;     // largest prefix chunk count of a unit
  int grid = 0;           // prefix workgroups
  oscar::CascUnit units[oscar::kMaxCascUnits];
};

// Splits each group into units of at most 16 / gqa sequences and the shared
// pages of each unit into chunks, about one prefix workgroup per CU in all.
oscar_status plan_cascade(const oscar_pool* pool, int batch, int int2_pt_stride, const oscar_prefix_group* groups,
                          int num_groups, CascPlan* cp) {
  const int hkv = pool->cfg.num_kv_heads, members = 16 / pool->gqa;
  if (num_groups < 0) return fail(OSCAR_ERR_INVALID, "negative num_groups");
  if (num_groups > 0 && !groups) return fail(OSCAR_ERR_INVALID, "groups must be non-null when num_groups > 0");
  long long total_pages = 0;
  int prev_end = 0;
  for (int g = 0; g < num_groups; ++g) {
    const oscar_prefix_group& pg = groups[g];
    if (pg.num_seqs < 1 || pg.first_seq < prev_end || (long long)pg.first_seq + pg.num_seqs > batch)
      return fail(OSCAR_ERR_INVALID, "prefix group %d: groups must be ordered, disjoint and inside the batch", g);
    if (pg.shared_pages < 0 || pg.shared_pages > int2_pt_stride)
      return fail(OSCAR_ERR_INVALID, "prefix group %d: shared_pages must be in [0, int2_pt_stride]", g);
    prev_end = pg.first_seq + pg.num_seqs;
    if (pg.shared_pages == 0) continue;
    for (int m = 0; m < pg.num_seqs; m += members) {
      if (cp->n == oscar::kMaxCascUnits)
        return fail(OSCAR_ERR_UNSUPPORTED, "more than %d prefix units of %d sequences", oscar::kMaxCascUnits, members);
      oscar::CascUnit& u = cp->units[cp->n++];
      u.first = pg.first_seq + m;
      u.count = std::min(members, pg.num_seqs - m);
      u.shared_pages = pg.shared_pages;
      total_pages += pg.shared_pages;
    }
  }
  const int target = env_int("OSCAR_TARGET_WGS", num_cus());
  int wg = 0;
  for (int i = 0; i < cp->n; ++i) {
    oscar::CascUnit& u = cp->units[i];
    // chunks of this unit in proportion to its pages, a tile being 2 pages
    // and a chunk at most 32 tiles per wave
    long long want = (long long)target * u.shared_pages / (hkv * std::max(1LL, total_pages));
    want = std::max(1LL, want);
    int ppc = (int)((u.shared_pages + want - 1) / want);
    ppc = std::min(std::max(2, (ppc + 1) / 2 * 2), 2 * 32 * kDecodeWaves);
    u.pages_per_chunk = ppc;
    u.chunks = (u.shared_pages + ppc - 1) / ppc;
    u.wg_start = wg;
    wg += hkv * u.chunks;
    cp->max_chunks = std::max(cp->max_chunks, u.chunks);
  }
  cp->grid = wg;
  return OSCAR_OK;
}

// Workspace of a decode with prefix units: every (sequence, KV head) gets the
// unit slots of the largest unit on top of the plain plan's.
Plan cascade_plan(const oscar_pool* pool, int batch, int max_len, const CascPlan& cp) {
  Plan pl = make_plan(pool, batch, max_len, false);
  const int hkv = pool->cfg.num_kv_heads;
  pl.slots = pl.units + cp.max_chunks;
  const size_t heads = (size_t)batch * hkv;
  const size_t parts = heads * pl.slots * pool->gqa;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  pl.off_lse = up(heads * oscar::kCounterStride * sizeof(uint32_t));
  pl.off_o = pl.off_lse + up(parts * sizeof(float));
  pl.bytes = pl.off_o + up(parts * pool->cfg.head_dim * sizeof(float));
  // the decode launch keeps the plain plan's workgroups: the extra slots are
  // filled by the prefix launch
  return pl;
}

// ---- length-aware ("packed") split-K plan ----
// With the host-side lengths the planner sizes every sequence's chunks from
// its own history: one common chunk size ppc (a multiple of the tile, at most
// chunk_cap pages) is chosen as the smallest that lets all units,
// BF16 units included, fit in R whole rounds of `target` workgroups, for the
// smallest R that can hold them.  Sequence b then has n_bf16_units +
// ceil(own_pages_b / ppc) units per KV head (own pages: its history past a
// prefix group's shared pages) and those units plus its prefix group's
// chunks as partial slots.  Returns false (use the uniform plan) for
// batches above kMaxPackedSeqs.
struct PackedPlan {
  int ppc, grid, slots;
  size_t off_lse, off_o, bytes;
  int32_t wg_off[oscar::kMaxPackedSeqs + 1];
  int32_t slot_off[oscar::kMaxPackedSeqs + 1];
};

bool plan_packed(const oscar_pool* pool, int batch, int max_len, const int32_t* host_lens, int bf16_pt_stride,
                 int int2_pt_stride, const Plan& base, const CascPlan& cp, PackedPlan* pp) {
  if (!host_lens || batch <= 0 || batch > oscar::kMaxPackedSeqs) return false;
  const oscar_config& c = pool->cfg;
  const int hkv = c.num_kv_heads, slots = slots_for(pool->gqa), nb = base.n_bf16_units;
  const int target = env_int("OSCAR_TARGET_WGS", num_cus());
  const int cap = chunk_cap(c);
  int own[oscar::kMaxPackedSeqs], cch[oscar::kMaxPackedSeqs];
  for (int b = 0; b < batch; ++b) {
    // the kernel's clamps of the length
    int L = std::min(std::max(host_lens[b], 0), max_len);
    L = std::min(L, oscar::kPage * bf16_pt_stride);
    L = std::min(L, c.sink_tokens + c.recent_tokens + oscar::kPage * int2_pt_stride);
    const int r0 = std::max(c.sink_tokens, L - c.recent_tokens);
    const int hp = (r0 - c.sink_tokens + oscar::kPage - 1) / oscar::kPage;
    int shared = 0;
    cch[b] = 0;
    for (int i = 0; i < cp.n; ++i)
      if (b >= cp.units[i].first && b < cp.units[i].first + cp.units[i].count) {
        shared = cp.units[i].shared_pages;
        cch[b] = cp.units[i].chunks;
      }
    own[b] = std::max(hp - shared, 0);
  }
  auto units = [&](int ppc) {
    long long u = 0;
    for (int b = 0; b < batch; ++b) u += nb + (own[b] + ppc - 1) / ppc;
    return u * hkv;
  };
  int ppc = -1;
  for (int r = 1; r <= 64 && ppc < 0; ++r) {
    const long long budget = (long long)r * target;
    if (units(cap) > budget) continue;
    int lo = 1, hi = cap / slots;  // smallest k with units(k * slots) <= budget
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (units(mid * slots) <= budget)
        hi = mid;
      else
        lo = mid + 1;
    }
    ppc = lo * slots;
  }
  if (ppc < 0) return false;
  pp->ppc = ppc;
  pp->wg_off[0] = pp->slot_off[0] = 0;
  for (int b = 0; b < batch; ++b) {
    const int ub = nb + (own[b] + ppc - 1) / ppc;
    pp->wg_off[b + 1] = pp->wg_off[b] + hkv * ub;
    pp->slot_off[b + 1] = pp->slot_off[b] + hkv * (ub + cch[b]);
  }
  pp->grid = pp->wg_off[batch];
  pp->slots = pp->slot_off[batch];
  const size_t heads = (size_t)batch * hkv, parts = (size_t)pp->slots * pool->gqa;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  pp->off_lse = up(heads * oscar::kCounterStride * sizeof(uint32_t));
  pp->off_o = pp->off_lse + up(parts * sizeof(float));
  pp->bytes = pp->off_o + up(parts * c.head_dim * sizeof(float));
  return true;
}

// ---- calibration helpers ----
constexpr size_t kSpan = (size_t)1 << 31;
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
bool supported_dim(int d) { return d == 64 || d == 128; }

// Row split of a gram: about 256 workgroups in all, each taking a multiple
// of 16 rows; returns the rows per split and sets `splits` so that the
// splits cover every row.
int gram_rows_per_split(int heads, int rows, int* splits) {
  const int blocks16 = (rows + 15) / 16;
  const int want = std::min(std::max(1, 256 / std::max(1, heads)), std::max(1, blocks16));
  const int rps = ((rows + want - 1) / want + 15) / 16 * 16;
  *splits = (rows + rps - 1) / rps;
  return rps;
}
int gram_splits(int heads, int rows) {
  int s = 0;
  gram_rows_per_split(heads, rows, &s);
  return s;
}
size_t gram_ws(int heads, int rows, int d) { return (size_t)gram_splits(heads, rows) * heads * d * d * 4; }

int clip_chunks(int heads) { return std::max(1, std::min(64, 256 / std::max(1, heads))); }
struct ClipWs {
  size_t keys, hist, sel, bytes;
};
ClipWs clip_ws(int heads, int rows, int d) {
  ClipWs w;
  w.keys = 0;
  w.hist = up256((size_t)heads * rows * d * 4);
  w.sel = w.hist + up256((size_t)heads * clip_chunks(heads) * 512 * 4);
  w.bytes = w.sel + up256((size_t)heads * 16);
  return w;
}

// x rows as used by gram / clip: one head's span must fit a buffer descriptor
oscar_status check_rows(const char* what, const float* x, int heads, int rows, int d, int64_t head_stride,
                        int64_t row_stride) {
  if (heads <= 0 || rows <= 0) return fail(OSCAR_ERR_INVALID, "%s: heads and rows must be positive", what);
  if (!supported_dim(d)) return fail(OSCAR_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128", what);
  if (!x || !aligned16(x)) return fail(OSCAR_ERR_INVALID, "%s: x must be non-null and 16-byte aligned", what);
  if (row_stride < d || row_stride % 4 || head_stride < 0 || head_stride % 4)
    return fail(OSCAR_ERR_INVALID, "%s: row_stride must be >= head_dim and strides multiples of 4", what);
  if ((size_t)rows * (size_t)row_stride * 4 >= kSpan) return fail(OSCAR_ERR_UNSUPPORTED, "%s: head span >= 2 GiB", what);
  return OSCAR_OK;
}

// calibration attention arguments (shared by oscar_calib_attention and
// oscar_attention_error)
oscar_status check_attn(int kv_heads, int gqa, int tokens, int d, const float* q, const float* k, const float* v,
                        int64_t hs, int64_t ns) {
  if (kv_heads <= 0 || gqa <= 0 || tokens <= 0)
    return fail(OSCAR_ERR_INVALID, "kv_heads, gqa and tokens must be positive");
  if (!supported_dim(d)) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!q || !k || !v || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(OSCAR_ERR_INVALID, "q, k and v must be non-null and 16-byte aligned");
  if (ns < d || ns % 4 || hs < 0 || hs % 4)
    return fail(OSCAR_ERR_INVALID, "kv_token_stride must be >= head_dim and strides multiples of 4");
  if ((size_t)tokens * d * 4 >= kSpan || (size_t)tokens * (size_t)ns * 4 >= kSpan)
    return fail(OSCAR_ERR_UNSUPPORTED, "per-head span >= 2 GiB");
  return OSCAR_OK;
}

float attn_scale_log2(float sm, int d) { return (sm > 0.f ? sm : 1.f / sqrtf((float)d)) * 1.4426950408889634f; }

oscar_status run_gram(int heads, int rows, int d, const float* x, int64_t hs, int64_t rs, float scale, float* out,
                      void* ws, hipStream_t stream) {
  oscar::GramParams p{};
  p.x = x;
  p.head_stride = hs;
  p.row_stride = rs;
  p.heads = heads;
  p.rows = rows;
  p.rows_per_split = gram_rows_per_split(heads, rows, &p.splits);
  p.scale = scale;
  p.part = (float*)ws;
  p.out = out;
  if (!oscar::launch_gram(p, d, stream)) return fail(OSCAR_ERR_UNSUPPORTED, "no gram kernel for this shape");
  return check_hip("gram launch");
}

oscar_status run_clip(int heads, int rows, int d, const float* x, int64_t hs, int64_t rs, const float* r,
                      double quantile, float* tau, void* ws, hipStream_t stream) {
  const ClipWs w = clip_ws(heads, rows, d);
  oscar::ClipParams p{};
  p.x = x;
  p.head_stride = hs;
  p.row_stride = rs;
  p.heads = heads;
  p.rows = rows;
  p.dim = d;
  p.r = r;
  p.keys = (uint32_t*)((char*)ws + w.keys);
  p.hist = (uint32_t*)((char*)ws + w.hist);
  p.sel = (uint32_t*)((char*)ws + w.sel);
  p.tau = tau;
  p.chunks = clip_chunks(heads);
  const double m = (double)rows * d;
  const double hpos = (m - 1.0) * quantile;
  const double lo = floor(hpos);
  p.rank_lo = (uint32_t)lo;
  p.rank_hi = (uint32_t)std::min(lo + 1.0, m - 1.0);
  p.frac = hpos - lo;
  if (!oscar::launch_clip(p, stream)) return fail(OSCAR_ERR_UNSUPPORTED, "no clip kernel for this shape");
  return check_hip("clip launch");
}

// Eigenbases of `heads` matrices of cov (and, with heads2 > 0, of heads2
// more from cov2) in one launch.
oscar_status run_rotation(int heads, int d, const float* cov, int mix, float* r, float* eig, hipStream_t stream,
                          int heads2 = 0, const float* cov2 = nullptr, float* r2 = nullptr) {
  oscar::EigParams p{cov, r, eig, cov2, r2, nullptr, heads + heads2, heads, mix};
  if (!oscar::launch_eigen_rotation(p, d, stream)) return fail(OSCAR_ERR_UNSUPPORTED, "eigen kernel unavailable");
  return check_hip("eigen/rotation launch");
}

constexpr int kLloydChunks = 128, kLloydIterations = 100;
struct CodebookWs {
  size_t t, partial, state, bytes;
};
CodebookWs codebook_ws(int heads, int rows, int d) {
  CodebookWs w;
  w.t = 0;
  w.partial = up256((size_t)heads * rows * d * 4);
  w.state = w.partial + up256((size_t)kLloydChunks * 4 * sizeof(double));
  w.bytes = w.state + 256;
  return w;
}

struct CalibWs {
  size_t part, o, cq, cs, clip, bytes;
};
CalibWs calib_ws(int hkv, int gqa, int n, int d) {
  CalibWs w;
  w.part = 0;
  w.o = up256(gram_ws(hkv, gqa * n, d));
  w.cq = w.o + up256((size_t)hkv * gqa * n * d * 4);
  w.cs = w.cq + up256((size_t)hkv * d * d * 4);
  w.clip = w.cs + up256((size_t)hkv * d * d * 4);
  w.bytes = w.clip + clip_ws(hkv, n, d).bytes;
  return w;
}

}  // namespace

extern "C" {

const char* oscar_status_string(oscar_status s) {
  switch (s) {
    case OSCAR_OK: return "OSCAR_OK";
    case OSCAR_ERR_INVALID: return "OSCAR_ERR_INVALID";
    case OSCAR_ERR_UNSUPPORTED: return "OSCAR_ERR_UNSUPPORTED";
    case OSCAR_ERR_WORKSPACE: return "OSCAR_ERR_WORKSPACE";
    case OSCAR_ERR_HIP: return "OSCAR_ERR_HIP";
  }
  return "OSCAR_ERR_UNKNOWN";
}

const char* oscar_last_error(void) { return g_err.c_str(); }

oscar_status oscar_pool_create(const oscar_config* cfg, oscar_pool** out, oscar_layout* layout) {
  if (!cfg || !out) return fail(OSCAR_ERR_INVALID, "cfg and out must be non-null");
  *out = nullptr;
  const oscar_config& c = *cfg;
  if (c.num_q_heads <= 0 || c.num_kv_heads <= 0 || c.head_dim <= 0 || c.group_size <= 0 || c.page_size <= 0 ||
      c.sink_tokens < 0 || c.recent_tokens <= 0 || !(c.sm_scale >= 0.f) || !isfinite(c.sm_scale))
    return fail(OSCAR_ERR_INVALID, "non-positive or non-finite configuration field");
  if (c.num_q_heads % c.num_kv_heads != 0)
    return fail(OSCAR_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d", c.num_q_heads,
                c.num_kv_heads);
  if (c.head_dim % c.group_size != 0)
    return fail(OSCAR_ERR_INVALID, "group_size %d does not divide head_dim %d", c.group_size, c.head_dim);
  if (c.sink_tokens % c.page_size != 0)
    return fail(OSCAR_ERR_INVALID, "sink_tokens %d is not a multiple of page_size %d", c.sink_tokens, c.page_size);
  const int gqa = c.num_q_heads / c.num_kv_heads;
  if (c.page_size != 16) return fail(OSCAR_ERR_UNSUPPORTED, "page_size must be 16");
  if (c.head_dim != 64 && c.head_dim != 128) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c.group_size != 64 && c.group_size != 128) return fail(OSCAR_ERR_UNSUPPORTED, "group_size must be 64 or 128");
  if (gqa != 2 && gqa != 4 && gqa != 8) return fail(OSCAR_ERR_UNSUPPORTED, "num_q_heads/num_kv_heads must be 2, 4 or 8");
  if (c.v_absorbed != 0 && c.v_absorbed != 1) return fail(OSCAR_ERR_INVALID, "v_absorbed must be 0 or 1");
  if (c.codebook != 0 && c.codebook != 1) return fail(OSCAR_ERR_INVALID, "codebook must be 0 or 1");
  if (c.codebook && (!levels_ok(c.levels_k) || !levels_ok(c.levels_v)))
    return fail(OSCAR_ERR_INVALID, "codebook levels must be 0 < L1 < L2 < 3 (ends 0 and 3), multiples of 1/32");
  oscar_pool* p = new (std::nothrow) oscar_pool;
  if (!p) return fail(OSCAR_ERR_INVALID, "out of host memory");
  p->cfg = c;
  p->n_groups = c.head_dim / c.group_size;
  p->gqa = gqa;
  p->sm_scale = c.sm_scale > 0.f ? c.sm_scale : 1.f / sqrtf((float)c.head_dim);
  p->layout.int2_head_block_bytes = (size_t)oscar::int2_block_bytes(c.head_dim, p->n_groups);
  p->layout.bf16_head_block_bytes = (size_t)oscar::bf16_block_bytes(c.head_dim);
  p->layout.int2_page_bytes = p->layout.int2_head_block_bytes * c.num_kv_heads;
  p->layout.bf16_page_bytes = p->layout.bf16_head_block_bytes * c.num_kv_heads;
  if (layout) *layout = p->layout;
  *out = p;
  return ok();
}

void oscar_pool_destroy(oscar_pool* pool) { delete pool; }

oscar_status oscar_decode_workspace_bytes(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                          int32_t bf16_only, size_t* bytes) {
  if (!pool || !bytes) return fail(OSCAR_ERR_INVALID, "pool and bytes must be non-null");
  if (batch < 0 || max_seq_len < 0) return fail(OSCAR_ERR_INVALID, "negative batch or max_seq_len");
  if (batch == 0) {
    *bytes = 0;
    return ok();
  }
  const Plan pl = make_plan(pool, batch, max_seq_len, bf16_only != 0);
  if (!pl.fits) return fail(OSCAR_ERR_UNSUPPORTED, "max_seq_len %d needs more than %d split-K chunks", max_seq_len, kMaxChunks);
  *bytes = pl.bytes + (OSCAR_PHASE_STAMPS ? oscar::kStampBytes + 256 : 0);
  return ok();
}

static oscar_status check_tables(const int32_t* bf16_pt, int32_t bf16_stride, int32_t bf16_pages,
                                 const int32_t* int2_pt, int32_t int2_stride, int32_t int2_pages, bool need_int2) {
  if (!bf16_pt || bf16_stride <= 0 || bf16_pages <= 0)
    return fail(OSCAR_ERR_INVALID, "BF16 page table, stride and page count must be given");
  if (need_int2 && (!int2_pt || int2_stride <= 0 || int2_pages <= 0))
    return fail(OSCAR_ERR_INVALID, "INT2 page table, stride and page count must be given");
  return ok();
}

}  // extern "C"

namespace {
// Decode with optional prefix groups (num_groups = 0: plain decode, one launch).
oscar_status decode_impl(const oscar_pool* pool, int32_t batch, int32_t max_seq_len, const void* q,
                         const int32_t* seq_lens, const int32_t* seq_lens_host, const int32_t* bf16_page_table,
                         int32_t bf16_pt_stride,
                         int32_t bf16_num_pages, const int32_t* int2_page_table, int32_t int2_pt_stride,
                         int32_t int2_num_pages, const void* bf16_pool, const void* int2_pool, const float* r_k,
                         const float* r_v, void* out, const oscar_prefix_group* groups, int32_t num_groups,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!pool) return fail(OSCAR_ERR_INVALID, "pool must be non-null");
  if (batch < 0 || max_seq_len < 0) return fail(OSCAR_ERR_INVALID, "negative batch or max_seq_len");
  if (batch == 0) return ok();
  if (!q || !seq_lens || !bf16_pool || !int2_pool || !r_k || !out)
    return fail(OSCAR_ERR_INVALID, "q, seq_lens, pools, r_k and out must be non-null");
  if (pool->cfg.v_absorbed && r_v) return fail(OSCAR_ERR_INVALID, "r_v must be NULL when V is absorbed");
  if (!pool->cfg.v_absorbed && !r_v) return fail(OSCAR_ERR_INVALID, "r_v is required when V is not absorbed");
  if (!aligned16(q) || !aligned16(bf16_pool) || !aligned16(int2_pool) || !aligned16(r_k) || !aligned16(r_v))
    return fail(OSCAR_ERR_INVALID, "q, pools, r_k and r_v must be 16-byte aligned");
  oscar_status st = check_tables(bf16_page_table, bf16_pt_stride, bf16_num_pages, int2_page_table, int2_pt_stride,
                                 int2_num_pages, true);
  if (st != OSCAR_OK) return st;
  CascPlan cp;
  if ((st = plan_cascade(pool, batch, int2_pt_stride, groups, num_groups, &cp)) != OSCAR_OK) return st;
  const Plan pl = cascade_plan(pool, batch, max_seq_len, cp);
  if (!pl.fits) return fail(OSCAR_ERR_UNSUPPORTED, "max_seq_len %d needs more than %d split-K chunks", max_seq_len, kMaxChunks);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < pl.bytes)
    return fail(OSCAR_ERR_WORKSPACE, "workspace must be 256-byte aligned and hold %zu bytes", pl.bytes);
  // profiling build: the phase timeline takes the workspace's last bytes
  // (from a 256-byte boundary)
  const bool stamps = OSCAR_PHASE_STAMPS && num_groups == 0 && workspace_bytes >= pl.bytes + oscar::kStampBytes + 256;
  const size_t ws_plan = stamps ? (workspace_bytes - oscar::kStampBytes) & ~(size_t)255 : workspace_bytes;
  // the length-aware plan when host lengths are given and its partials fit
  // the workspace (sized for the uniform plan of max_seq_len)
  PackedPlan pk;
  const bool packed = plan_packed(pool, batch, max_seq_len, seq_lens_host, bf16_pt_stride, int2_pt_stride, pl, cp,
                                  &pk) &&
                      pk.bytes <= ws_plan;
  const oscar_config& c = pool->cfg;
  oscar::DecodeParams p{};
  p.q = (const uint16_t*)q;
  p.seq_lens = seq_lens;
  p.bf16_pt = bf16_page_table;
  p.int2_pt = int2_page_table;
  p.bf16_pool = (const uint8_t*)bf16_pool;
  p.int2_pool = (const uint8_t*)int2_pool;
  p.r_k = r_k;
  p.r_v = r_v;
  p.out = (uint16_t*)out;
  p.counters = (uint32_t*)((char*)workspace + pl.off_counters);
  p.part_lse = (float*)((char*)workspace + pl.off_lse);
  p.part_o = (float*)((char*)workspace + pl.off_o);
  if (stamps) p.stamps = (uint64_t*)((char*)workspace + ws_plan);
  p.bf16_pt_stride = bf16_pt_stride;
  p.bf16_num_pages = bf16_num_pages;
  p.int2_pt_stride = int2_pt_stride;
  p.int2_num_pages = int2_num_pages;
  p.batch = batch;
  p.num_kv_heads = c.num_kv_heads;
  p.sink = c.sink_tokens;
  p.recent = c.recent_tokens;
  p.max_len = max_seq_len;
  p.n_bf16_units = pl.n_bf16_units;
  p.bf16_pages_per_unit = pl.bf16_pages_per_unit;
  p.max_chunks = pl.max_chunks;
  p.pages_per_chunk = pl.pages_per_chunk;
  p.units_per_head = pl.units;
  p.slots_per_head = pl.slots;
  p.sm_log2 = pool->sm_scale * 1.4426950408889634f;
  set_codebook(pool, p);
  p.n_casc = cp.n;
  oscar::CascArgs casc{};
  for (int i = 0; i < cp.n; ++i) casc.unit[i] = cp.units[i];
  int grid = pl.grid;
  oscar::PackedPlanArgs tables;
  const oscar::PackedPlanArgs* tables_arg = nullptr;
  if (packed) {
    p.pages_per_chunk = pk.ppc;
    p.part_lse = (float*)((char*)workspace + pk.off_lse);
    p.part_o = (float*)((char*)workspace + pk.off_o);
    grid = pk.grid;
    // when every sequence has the same units and slots (one sequence, or
    // equal lengths) the plan is uniform: the kernel then maps workgroups
    // by arithmetic instead of reading the offset tables
    const int hkv = c.num_kv_heads;
    const int u0 = pk.wg_off[1] / hkv, s0 = pk.slot_off[1] / hkv;
    bool same = true;
    for (int i = 0; i < batch; ++i)
      same = same && pk.wg_off[i + 1] - pk.wg_off[i] == hkv * u0 && pk.slot_off[i + 1] - pk.slot_off[i] == hkv * s0;
    if (same) {
      p.units_per_head = u0;
      p.slots_per_head = s0;
      p.max_chunks = u0 - pl.n_bf16_units;
    } else {
      for (int i = 0; i <= batch; ++i) {
        tables.wg_off[i] = pk.wg_off[i];
        tables.slot_off[i] = pk.slot_off[i];
      }
      for (int i = batch + 1; i <= oscar::kMaxPackedSeqs; ++i) tables.wg_off[i] = tables.slot_off[i] = pk.grid;
      tables_arg = &tables;
    }
  }
  // prefix partials first (same stream): the decode launch's merge reads them
  if (cp.grid > 0) {
    if (!oscar::launch_decode_prefix(p, casc, tables_arg, c.head_dim, pool->n_groups, pool->gqa, cp.grid,
                                     (hipStream_t)stream))
      return fail(OSCAR_ERR_UNSUPPORTED, "no prefix decode kernel for this shape");
    if ((st = check_hip("prefix decode launch")) != OSCAR_OK) return st;
  }
  if (!oscar::launch_decode(p, cp.n > 0 ? &casc : nullptr, tables_arg, c.head_dim, pool->n_groups, pool->gqa, false,
                            grid, (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no decode kernel for this shape");
  return check_hip("decode launch");
}
}  // namespace

extern "C" {

oscar_status oscar_decode_attention(const oscar_pool* pool, int32_t batch, int32_t max_seq_len, const void* q,
                                    const int32_t* seq_lens, const int32_t* seq_lens_host, const int32_t* bf16_page_table,
                                    int32_t bf16_pt_stride, int32_t bf16_num_pages,
                                    const int32_t* int2_page_table, int32_t int2_pt_stride,
                                    int32_t int2_num_pages, const void* bf16_pool, const void* int2_pool,
                                    const float* r_k, const float* r_v, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return decode_impl(pool, batch, max_seq_len, q, seq_lens, seq_lens_host, bf16_page_table, bf16_pt_stride, bf16_num_pages,
                     int2_page_table, int2_pt_stride, int2_num_pages, bf16_pool, int2_pool, r_k, r_v, out, nullptr, 0,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- decode without a workspace argument ----
// The scratch of oscar_decode_attention_noalloc: a fixed array in device
// memory, one copy per GPU the library runs on, held until the process ends.
// Host code reaches it only through the per-device address that
// hipGetSymbolAddress returns (kept in g_scratch_ptr).
static __device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void k_zero_words(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch address.  At the first call on a device the
// address is looked up and the whole array is cleared by a kernel on
// `stream` (a kernel rather than a memset, so that the clear can also sit in
// a captured graph); afterwards every decode leaves its counters at zero.
oscar_status current_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(OSCAR_ERR_HIP, "hipGetDevice failed");
  if (dev >= kMaxDevices) return fail(OSCAR_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(OSCAR_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const uint32_t words = OSCAR_NOALLOC_SCRATCH_BYTES / 4;
    hipLaunchKernelGGL(k_zero_words, dim3(256), dim3(256), 0, stream, (uint32_t*)ptr, words);
    const oscar_status st = check_hip("scratch clear launch");
    if (st != OSCAR_OK) return st;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return OSCAR_OK;
}
}  // namespace

extern "C" {

oscar_status oscar_decode_attention_noalloc(const oscar_pool* pool, int32_t batch, int32_t max_seq_len, const void* q,
                                            const int32_t* seq_lens, const int32_t* seq_lens_host, const int32_t* bf16_page_table,
                                            int32_t bf16_pt_stride, int32_t bf16_num_pages,
                                            const int32_t* int2_page_table, int32_t int2_pt_stride,
                                            int32_t int2_num_pages, const void* bf16_pool, const void* int2_pool,
                                            const float* r_k, const float* r_v, void* out, void* stream) {
  if (!pool) return fail(OSCAR_ERR_INVALID, "pool must be non-null");
  if (batch < 0 || max_seq_len < 0) return fail(OSCAR_ERR_INVALID, "negative batch or max_seq_len");
  if (batch == 0) return ok();
  const Plan pl = make_plan(pool, batch, max_seq_len, false);
  if (!pl.fits) return fail(OSCAR_ERR_UNSUPPORTED, "max_seq_len %d needs more than %d split-K chunks", max_seq_len, kMaxChunks);
  if (pl.bytes > OSCAR_NOALLOC_SCRATCH_BYTES)
    return fail(OSCAR_ERR_UNSUPPORTED,
                "batch %d at max_seq_len %d needs %zu bytes of decode scratch; the allocation-free decode holds %zu "
                "(use oscar_decode_attention with a workspace)",
                batch, max_seq_len, pl.bytes, (size_t)OSCAR_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const oscar_status st = current_scratch((hipStream_t)stream, &ws);
  if (st != OSCAR_OK) return st;
  return decode_impl(pool, batch, max_seq_len, q, seq_lens, seq_lens_host, bf16_page_table, bf16_pt_stride, bf16_num_pages,
                     int2_page_table, int2_pt_stride, int2_num_pages, bf16_pool, int2_pool, r_k, r_v, out, nullptr, 0,
                     ws, OSCAR_NOALLOC_SCRATCH_BYTES, stream);
}

oscar_status oscar_decode_cascade_workspace_bytes(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                                  int32_t int2_pt_stride, const oscar_prefix_group* groups,
                                                  int32_t num_groups, size_t* bytes) {
  if (!pool || !bytes) return fail(OSCAR_ERR_INVALID, "pool and bytes must be non-null");
  if (batch < 0 || max_seq_len < 0) return fail(OSCAR_ERR_INVALID, "negative batch or max_seq_len");
  if (batch == 0) {
    *bytes = 0;
    return ok();
  }
  CascPlan cp;
  oscar_status st = plan_cascade(pool, batch, int2_pt_stride, groups, num_groups, &cp);
  if (st != OSCAR_OK) return st;
  const Plan pl = cascade_plan(pool, batch, max_seq_len, cp);
  if (!pl.fits) return fail(OSCAR_ERR_UNSUPPORTED, "max_seq_len %d needs more than %d split-K chunks", max_seq_len, kMaxChunks);
  *bytes = pl.bytes;
  return ok();
}

oscar_status oscar_decode_attention_cascade(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                            const void* q, const int32_t* seq_lens, const int32_t* seq_lens_host,
                                            const int32_t* bf16_page_table, int32_t bf16_pt_stride,
                                            int32_t bf16_num_pages, const int32_t* int2_page_table,
                                            int32_t int2_pt_stride, int32_t int2_num_pages, const void* bf16_pool,
                                            const void* int2_pool, const float* r_k, const float* r_v, void* out,
                                            const oscar_prefix_group* groups, int32_t num_groups, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return decode_impl(pool, batch, max_seq_len, q, seq_lens, seq_lens_host, bf16_page_table, bf16_pt_stride, bf16_num_pages,
                     int2_page_table, int2_pt_stride, int2_num_pages, bf16_pool, int2_pool, r_k, r_v, out, groups,
                     num_groups, workspace, workspace_bytes, stream);
}

oscar_status oscar_bf16_decode_attention(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                         const void* q, const int32_t* seq_lens,
                                         const int32_t* bf16_page_table, int32_t bf16_pt_stride,
                                         int32_t bf16_num_pages, const void* bf16_pool, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!pool) return fail(OSCAR_ERR_INVALID, "pool must be non-null");
  if (batch < 0 || max_seq_len < 0) return fail(OSCAR_ERR_INVALID, "negative batch or max_seq_len");
  if (batch == 0) return ok();
  if (!q || !seq_lens || !bf16_pool || !out)
    return fail(OSCAR_ERR_INVALID, "q, seq_lens, bf16_pool and out must be non-null");
  if (!aligned16(q) || !aligned16(bf16_pool)) return fail(OSCAR_ERR_INVALID, "q and pool must be 16-byte aligned");
  oscar_status st = check_tables(bf16_page_table, bf16_pt_stride, bf16_num_pages, nullptr, 0, 0, false);
  if (st != OSCAR_OK) return st;
  const Plan pl = make_plan(pool, batch, max_seq_len, true);
  if (!pl.fits) return fail(OSCAR_ERR_UNSUPPORTED, "max_seq_len %d needs more than %d split-K chunks", max_seq_len, kMaxChunks);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < pl.bytes)
    return fail(OSCAR_ERR_WORKSPACE, "workspace must be 256-byte aligned and hold %zu bytes", pl.bytes);
  const oscar_config& c = pool->cfg;
  oscar::DecodeParams p{};
  p.q = (const uint16_t*)q;
  p.seq_lens = seq_lens;
  p.bf16_pt = bf16_page_table;
  p.bf16_pool = (const uint8_t*)bf16_pool;
  p.out = (uint16_t*)out;
  p.counters = (uint32_t*)((char*)workspace + pl.off_counters);
  p.part_lse = (float*)((char*)workspace + pl.off_lse);
  p.part_o = (float*)((char*)workspace + pl.off_o);
  p.bf16_pt_stride = bf16_pt_stride;
  p.bf16_num_pages = bf16_num_pages;
  p.int2_pt_stride = 1;
  p.batch = batch;
  p.num_kv_heads = c.num_kv_heads;
  p.sink = c.sink_tokens;
  p.recent = c.recent_tokens;
  p.max_len = max_seq_len;
  p.n_bf16_units = 0;
  p.max_chunks = pl.max_chunks;
  p.pages_per_chunk = pl.pages_per_chunk;
  p.units_per_head = pl.units;
  p.slots_per_head = pl.slots;
  p.sm_log2 = pool->sm_scale * 1.4426950408889634f;
  if (!oscar::launch_decode(p, nullptr, nullptr, c.head_dim, pool->n_groups, pool->gqa, true, pl.grid,
                            (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no decode kernel for this shape");
  return check_hip("bf16 decode launch");
}

oscar_status oscar_merge(int32_t rows, int32_t head_dim, const int32_t* row_offsets, const float* o_partials,
                         const float* lse_partials, void* out, void* stream) {
  if (rows < 0) return fail(OSCAR_ERR_INVALID, "negative rows");
  if (head_dim != 64 && head_dim != 128) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (rows == 0) return ok();
  if (!row_offsets || !o_partials || !lse_partials || !out)
    return fail(OSCAR_ERR_INVALID, "row_offsets, partials and out must be non-null");
  oscar::MergeParams p{rows, head_dim, row_offsets, o_partials, lse_partials, (uint16_t*)out};
  if (!oscar::launch_merge(p, (hipStream_t)stream)) return fail(OSCAR_ERR_UNSUPPORTED, "no merge kernel");
  return check_hip("merge launch");
}

oscar_status oscar_append_demote(const oscar_pool* pool, int32_t batch, const void* k_new, const void* v_new,
                                 const int32_t* seq_lens, const int32_t* bf16_page_table,
                                 int32_t bf16_pt_stride, int32_t bf16_num_pages,
                                 const int32_t* int2_page_table, int32_t int2_pt_stride,
                                 int32_t int2_num_pages, void* bf16_pool, void* int2_pool, const float* r_k,
                                 const float* r_v, const float* tau_k, const float* tau_v, void* stream) {
  if (!pool) return fail(OSCAR_ERR_INVALID, "pool must be non-null");
  if (batch < 0) return fail(OSCAR_ERR_INVALID, "negative batch");
  if (batch == 0) return ok();
  if (!k_new || !v_new || !seq_lens || !bf16_pool || !int2_pool || !r_k || !tau_k || !tau_v)
    return fail(OSCAR_ERR_INVALID, "k_new, v_new, seq_lens, pools, r_k, tau_k and tau_v must be non-null");
  if (pool->cfg.v_absorbed && r_v) return fail(OSCAR_ERR_INVALID, "r_v must be NULL when V is absorbed");
  if (!pool->cfg.v_absorbed && !r_v) return fail(OSCAR_ERR_INVALID, "r_v is required when V is not absorbed");
  if (!aligned16(r_k) || !aligned16(r_v) || !aligned16(bf16_pool) || !aligned16(int2_pool))
    return fail(OSCAR_ERR_INVALID, "pools, r_k and r_v must be 16-byte aligned");
  oscar_status st = check_tables(bf16_page_table, bf16_pt_stride, bf16_num_pages, int2_page_table, int2_pt_stride,
                                 int2_num_pages, true);
  if (st != OSCAR_OK) return st;
  const oscar_config& c = pool->cfg;
  oscar::WriteParams p{};
  p.k_new = (const uint16_t*)k_new;
  p.v_new = (const uint16_t*)v_new;
  p.seq_lens = seq_lens;
  p.bf16_pt = bf16_page_table;
  p.int2_pt = int2_page_table;
  p.bf16_pool = (uint8_t*)bf16_pool;
  p.int2_pool = (uint8_t*)int2_pool;
  p.bf16_pt_stride = bf16_pt_stride;
  p.bf16_num_pages = bf16_num_pages;
  p.int2_pt_stride = int2_pt_stride;
  p.int2_num_pages = int2_num_pages;
  p.r_k = r_k;
  p.r_v = r_v;
  p.tau_k = tau_k;
  p.tau_v = tau_v;
  p.batch = batch;
  p.num_kv_heads = c.num_kv_heads;
  p.sink = c.sink_tokens;
  p.recent = c.recent_tokens;
  set_codebook(pool, p);
  if (!oscar::launch_append_demote(p, c.head_dim, pool->n_groups, (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no append/demote kernel for this shape");
  return check_hip("append/demote launch");
}

oscar_status oscar_quantize_pack(const oscar_pool* pool, int32_t num_tokens, const void* k, const void* v,
                                 const int32_t* page_ids, int32_t int2_num_pages, void* int2_pool,
                                 const float* r_k, const float* r_v, const float* tau_k, const float* tau_v,
                                 void* stream) {
  if (!pool) return fail(OSCAR_ERR_INVALID, "pool must be non-null");
  if (num_tokens < 0) return fail(OSCAR_ERR_INVALID, "negative num_tokens");
  if (num_tokens == 0) return ok();
  if (!k || !v || !page_ids || !int2_pool || !r_k || !tau_k || !tau_v || int2_num_pages <= 0)
    return fail(OSCAR_ERR_INVALID, "k, v, page_ids, int2_pool, r_k, tau_k, tau_v and int2_num_pages must be given");
  if (pool->cfg.v_absorbed && r_v) return fail(OSCAR_ERR_INVALID, "r_v must be NULL when V is absorbed");
  if (!pool->cfg.v_absorbed && !r_v) return fail(OSCAR_ERR_INVALID, "r_v is required when V is not absorbed");
  if (!aligned16(k) || !aligned16(v) || !aligned16(int2_pool) || !aligned16(r_k) || !aligned16(r_v))
    return fail(OSCAR_ERR_INVALID, "k, v, int2_pool, r_k and r_v must be 16-byte aligned");
  const oscar_config& c = pool->cfg;
  oscar::WriteParams p{};
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.page_ids = page_ids;
  p.num_tokens = num_tokens;
  p.int2_pool = (uint8_t*)int2_pool;
  p.int2_num_pages = int2_num_pages;
  {
    // one 8-wave workgroup per compute unit (its LDS holds R_K twice), the
    // pages of each KV head split evenly over the workgroups given to it
    const int npages = (num_tokens + 15) / 16;
    const int per_head = std::max(1, num_cus() / std::max(1, c.num_kv_heads));
    p.pages_per_block = env_int("OSCAR_QP_PAGES_PER_BLOCK", (npages + per_head - 1) / per_head);
    if (p.pages_per_block < 8) p.pages_per_block = 8;
  }
  p.r_k = r_k;
  p.r_v = r_v;
  p.tau_k = tau_k;
  p.tau_v = tau_v;
  p.num_kv_heads = c.num_kv_heads;
  p.sink = c.sink_tokens;
  p.recent = c.recent_tokens;
  set_codebook(pool, p);
  if (!oscar::launch_quantize_pack(p, c.head_dim, pool->n_groups, (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no quantize/pack kernel for this shape");
  return check_hip("quantize/pack launch");
}

oscar_status oscar_write_bf16(const oscar_pool* pool, int32_t num_tokens, int32_t first_position, const void* k,
                              const void* v, const int32_t* bf16_page_table, int32_t bf16_pt_stride,
                              int32_t bf16_num_pages, void* bf16_pool, void* stream) {
  if (!pool) return fail(OSCAR_ERR_INVALID, "pool must be non-null");
  if (num_tokens < 0 || first_position < 0) return fail(OSCAR_ERR_INVALID, "negative num_tokens or first_position");
  if (num_tokens == 0) return ok();
  if (!k || !v || !bf16_pool) return fail(OSCAR_ERR_INVALID, "k, v and bf16_pool must be non-null");
  oscar_status st = check_tables(bf16_page_table, bf16_pt_stride, bf16_num_pages, nullptr, 0, 0, false);
  if (st != OSCAR_OK) return st;
  oscar::WriteParams p{};
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.num_tokens = num_tokens;
  p.bf16_pt = bf16_page_table;
  p.bf16_pt_stride = bf16_pt_stride;
  p.bf16_num_pages = bf16_num_pages;
  p.bf16_pool = (uint8_t*)bf16_pool;
  p.num_kv_heads = pool->cfg.num_kv_heads;
  if (!oscar::launch_write_bf16(p, pool->cfg.head_dim, first_position, (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no BF16 writer for this shape");
  return check_hip("bf16 write launch");
}

oscar_status oscar_calib_gram_workspace_bytes(int32_t heads, int32_t rows, int32_t head_dim, size_t* bytes) {
  if (!bytes || heads <= 0 || rows <= 0) return fail(OSCAR_ERR_INVALID, "bytes must be non-null, heads and rows positive");
  if (!supported_dim(head_dim)) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  *bytes = gram_ws(heads, rows, head_dim);
  return ok();
}

oscar_status oscar_calib_gram(int32_t heads, int32_t rows, int32_t head_dim, const float* x, int64_t head_stride,
                              int64_t row_stride, float scale, float* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  oscar_status st = check_rows("gram", x, heads, rows, head_dim, head_stride, row_stride);
  if (st != OSCAR_OK) return st;
  if (!out) return fail(OSCAR_ERR_INVALID, "out must be non-null");
  if (!workspace || workspace_bytes < gram_ws(heads, rows, head_dim))
    return fail(OSCAR_ERR_WORKSPACE, "gram needs %zu bytes of workspace", gram_ws(heads, rows, head_dim));
  return run_gram(heads, rows, head_dim, x, head_stride, row_stride, scale, out, workspace, (hipStream_t)stream);
}

oscar_status oscar_calib_attention(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim, float sm_scale,
                                   const float* q, const float* k, const float* v, int64_t kv_head_stride,
                                   int64_t kv_token_stride, float* out, float* lse, void* stream) {
  oscar_status st = check_attn(kv_heads, gqa, tokens, head_dim, q, k, v, kv_head_stride, kv_token_stride);
  if (st != OSCAR_OK) return st;
  if (!out || !aligned16(out)) return fail(OSCAR_ERR_INVALID, "out must be non-null and 16-byte aligned");
  oscar::CalibAttnParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.kv_hs = kv_head_stride;
  p.kv_ns = kv_token_stride;
  p.kv_heads = kv_heads;
  p.gqa = gqa;
  p.tokens = tokens;
  p.scale_log2 = attn_scale_log2(sm_scale, head_dim);
  if (!oscar::launch_calib_attention(p, head_dim, false, (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no calibration attention kernel for this shape");
  return check_hip("calibration attention launch");
}

oscar_status oscar_calib_rotation(int32_t heads, int32_t head_dim, const float* cov, int32_t mix, float* r,
                                  float* eigvals, void* stream) {
  if (heads <= 0) return fail(OSCAR_ERR_INVALID, "heads must be positive");
  if (!supported_dim(head_dim)) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!cov || !r) return fail(OSCAR_ERR_INVALID, "cov and r must be non-null");
  if (mix != 0 && mix != 1) return fail(OSCAR_ERR_INVALID, "mix must be 0 or 1");
  return run_rotation(heads, head_dim, cov, mix, r, eigvals, (hipStream_t)stream);
}

oscar_status oscar_calib_clip_workspace_bytes(int32_t heads, int32_t rows, int32_t head_dim, size_t* bytes) {
  if (!bytes || heads <= 0 || rows <= 0) return fail(OSCAR_ERR_INVALID, "bytes must be non-null, heads and rows positive");
  if (!supported_dim(head_dim)) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  *bytes = clip_ws(heads, rows, head_dim).bytes;
  return ok();
}

oscar_status oscar_calib_clip(int32_t heads, int32_t rows, int32_t head_dim, const float* x, int64_t head_stride,
                              int64_t row_stride, const float* r, double quantile, float* tau, void* workspace,
                              size_t workspace_bytes, void* stream) {
  oscar_status st = check_rows("clip", x, heads, rows, head_dim, head_stride, row_stride);
  if (st != OSCAR_OK) return st;
  if (!tau) return fail(OSCAR_ERR_INVALID, "tau must be non-null");
  if (!(quantile >= 0.0 && quantile <= 1.0)) return fail(OSCAR_ERR_INVALID, "quantile must be in [0, 1]");
  if ((size_t)rows * head_dim >= ((size_t)1 << 32)) return fail(OSCAR_ERR_UNSUPPORTED, "too many values per head");
  const size_t need = clip_ws(heads, rows, head_dim).bytes;
  if (!workspace || workspace_bytes < need) return fail(OSCAR_ERR_WORKSPACE, "clip needs %zu bytes of workspace", need);
  return run_clip(heads, rows, head_dim, x, head_stride, row_stride, r, quantile, tau, workspace,
                  (hipStream_t)stream);
}

oscar_status oscar_calib_codebook_workspace_bytes(int32_t heads, int32_t rows, int32_t head_dim, size_t* bytes) {
  if (!bytes || heads <= 0 || rows <= 0) return fail(OSCAR_ERR_INVALID, "bytes must be non-null, heads and rows positive");
  if (!supported_dim(head_dim)) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  *bytes = codebook_ws(heads, rows, head_dim).bytes;
  return ok();
}

oscar_status oscar_calib_codebook(int32_t heads, int32_t rows, int32_t head_dim, int32_t group_size, const float* x,
                                  int64_t head_stride, int64_t row_stride, const float* r, const float* tau,
                                  float* levels, void* workspace, size_t workspace_bytes, void* stream) {
  oscar_status st = check_rows("codebook", x, heads, rows, head_dim, head_stride, row_stride);
  if (st != OSCAR_OK) return st;
  if (group_size != 64 && group_size != 128) return fail(OSCAR_ERR_UNSUPPORTED, "group_size must be 64 or 128");
  if (head_dim % group_size) return fail(OSCAR_ERR_INVALID, "group_size must divide head_dim");
  if (!tau || !levels) return fail(OSCAR_ERR_INVALID, "tau and levels must be non-null");
  const CodebookWs w = codebook_ws(heads, rows, head_dim);
  if (!workspace || workspace_bytes < w.bytes || ((uintptr_t)workspace & 255u))
    return fail(OSCAR_ERR_WORKSPACE, "codebook fit needs %zu bytes of 256-byte aligned workspace", w.bytes);
  oscar::CodebookParams p{};
  p.x = x;
  p.head_stride = head_stride;
  p.row_stride = row_stride;
  p.heads = heads;
  p.rows = rows;
  p.dim = head_dim;
  p.group_size = group_size;
  p.r = r;
  p.tau = tau;
  p.t = (float*)((char*)workspace + w.t);
  p.partial = (double*)((char*)workspace + w.partial);
  p.state = (double*)((char*)workspace + w.state);
  p.levels = levels;
  p.chunks = kLloydChunks;
  if (!oscar::launch_codebook(p, kLloydIterations, (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no codebook kernel for this shape");
  return check_hip("codebook launch");
}

oscar_status oscar_calib_workspace_bytes(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim,
                                         size_t* bytes) {
  if (!bytes || kv_heads <= 0 || gqa <= 0 || tokens <= 0)
    return fail(OSCAR_ERR_INVALID, "bytes must be non-null, kv_heads, gqa and tokens positive");
  if (!supported_dim(head_dim)) return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  *bytes = calib_ws(kv_heads, gqa, tokens, head_dim).bytes;
  return ok();
}

oscar_status oscar_calibrate(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim, float sm_scale,
                             const float* q, const float* k, const float* v, int64_t kv_head_stride,
                             int64_t kv_token_stride, double clip_quantile, float* r_k, float* r_v, float* tau_k,
                             float* tau_v, float* c_q, float* c_s, void* workspace, size_t workspace_bytes,
                             void* stream) {
  oscar_status st = check_attn(kv_heads, gqa, tokens, head_dim, q, k, v, kv_head_stride, kv_token_stride);
  if (st != OSCAR_OK) return st;
  if (!r_k || !r_v || !tau_k || !tau_v) return fail(OSCAR_ERR_INVALID, "r_k, r_v, tau_k and tau_v must be non-null");
  if (!(clip_quantile >= 0.0 && clip_quantile <= 1.0)) return fail(OSCAR_ERR_INVALID, "clip_quantile must be in [0, 1]");
  const int rows = gqa * tokens;
  if ((size_t)rows * head_dim * 4 >= kSpan) return fail(OSCAR_ERR_UNSUPPORTED, "per-head query span >= 2 GiB");
  const CalibWs w = calib_ws(kv_heads, gqa, tokens, head_dim);
  if (!workspace || workspace_bytes < w.bytes || ((uintptr_t)workspace & 255u))
    return fail(OSCAR_ERR_WORKSPACE, "calibration needs %zu bytes of 256-byte aligned workspace", w.bytes);
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  float* cq = c_q ? c_q : (float*)(ws + w.cq);
  float* cs = c_s ? c_s : (float*)(ws + w.cs);
  float* o = (float*)(ws + w.o);
  const int64_t qhs = (int64_t)rows * head_dim;
  const float inv_rows = 1.f / (float)rows;
  if ((st = run_gram(kv_heads, rows, head_dim, q, qhs, head_dim, inv_rows, cq, ws + w.part, s)) != OSCAR_OK) return st;
  st = oscar_calib_attention(kv_heads, gqa, tokens, head_dim, sm_scale, q, k, v, kv_head_stride, kv_token_stride, o,
                             nullptr, stream);
  if (st != OSCAR_OK) return st;
  if ((st = run_gram(kv_heads, rows, head_dim, o, qhs, head_dim, inv_rows, cs, ws + w.part, s)) != OSCAR_OK) return st;
  // both eigenbases in one launch (one workgroup per matrix)
  if ((st = run_rotation(kv_heads, head_dim, cq, 1, r_k, nullptr, s, kv_heads, cs, r_v)) != OSCAR_OK) return st;
  if ((st = run_clip(kv_heads, tokens, head_dim, k, kv_head_stride, kv_token_stride, r_k, clip_quantile, tau_k,
                     ws + w.clip, s)) != OSCAR_OK)
    return st;
  return run_clip(kv_heads, tokens, head_dim, v, kv_head_stride, kv_token_stride, r_v, clip_quantile, tau_v,
                  ws + w.clip, s);
}

oscar_status oscar_dequantize(const oscar_pool* pool, int32_t num_tokens, const int32_t* page_ids,
                              int32_t int2_num_pages, const void* int2_pool, const float* r_k, const float* r_v,
                              float* k_out, float* v_out, void* stream) {
  if (!pool) return fail(OSCAR_ERR_INVALID, "pool must be non-null");
  if (num_tokens < 0) return fail(OSCAR_ERR_INVALID, "negative num_tokens");
  if (num_tokens == 0) return ok();
  if (!page_ids || !int2_pool || !k_out || !v_out || int2_num_pages <= 0)
    return fail(OSCAR_ERR_INVALID, "page_ids, int2_pool, k_out, v_out and int2_num_pages must be given");
  if (!aligned16(int2_pool)) return fail(OSCAR_ERR_INVALID, "int2_pool must be 16-byte aligned");
  const oscar_config& c = pool->cfg;
  oscar::DequantParams p{};
  p.page_ids = page_ids;
  p.int2_pool = (const uint8_t*)int2_pool;
  p.num_tokens = num_tokens;
  p.int2_num_pages = int2_num_pages;
  p.num_kv_heads = c.num_kv_heads;
  for (int which = 0; which < 2; ++which) {
    p.which = which;
    p.r = which ? r_v : r_k;
    p.out = which ? v_out : k_out;
    for (int k = 0; k < 4; ++k)
      p.levels[k] = c.codebook ? (which ? c.levels_v[k] : c.levels_k[k]) : (float)k;
    if (!oscar::launch_dequantize(p, c.head_dim, pool->n_groups, (hipStream_t)stream))
      return fail(OSCAR_ERR_UNSUPPORTED, "no dequantize kernel for this shape");
  }
  return check_hip("dequantize launch");
}

oscar_status oscar_attention_error(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim, float sm_scale,
                                   const float* q, const float* k, const float* v, const float* k_hat,
                                   const float* v_hat, int64_t kv_head_stride, int64_t kv_token_stride,
                                   float* stats, void* stream) {
  oscar_status st = check_attn(kv_heads, gqa, tokens, head_dim, q, k, v, kv_head_stride, kv_token_stride);
  if (st != OSCAR_OK) return st;
  if (!k_hat || !v_hat || !aligned16(k_hat) || !aligned16(v_hat))
    return fail(OSCAR_ERR_INVALID, "k_hat and v_hat must be non-null and 16-byte aligned");
  if (!stats || !aligned16(stats)) return fail(OSCAR_ERR_INVALID, "stats must be non-null and 16-byte aligned");
  oscar::CalibAttnParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.k_hat = k_hat;
  p.v_hat = v_hat;
  p.stats = stats;
  p.kv_hs = kv_head_stride;
  p.kv_ns = kv_token_stride;
  p.kv_heads = kv_heads;
  p.gqa = gqa;
  p.tokens = tokens;
  p.scale_log2 = attn_scale_log2(sm_scale, head_dim);
  if (!oscar::launch_calib_attention(p, head_dim, true, (hipStream_t)stream))
    return fail(OSCAR_ERR_UNSUPPORTED, "no attention error kernel for this shape");
  return check_hip("attention error launch");
}

}  // extern "C"
