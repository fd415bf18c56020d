// C ABI of the approximate-attention prefill: argument validation, work schedule and
// launches. All checks run on the host before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "apbv_internal.h"

// Scratch of the allocation-free scoring entry point (apbv_score_select_noalloc): the split
// statistics, the packed score rows and, when the caller passes no score buffer, the scores. The runtime gives every
// device the library runs on its own copy, held until the process ends. In host code this
// name is only a stand-in for the symbol: its device address comes from hipGetSymbolAddress
// (scratch_of_current_device below) and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[16u << 20];

namespace apbv {

namespace {

thread_local char g_err[512] = "";

apbv_status fail(apbv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Checked {
  int n, N, hq, hkv, d, G, l_a, l_q, l_p, pre_rows, min_block, max_block;
  int64_t q_stride, kv_stride;
  float scale;
};

apbv_status check_layout(const apbv_layout* L, Checked& c) {
  if (L == nullptr) return fail(APBV_EINVAL, "layout is NULL");
  if (L->n_blocks < 1 || L->n_blocks > APBV_MAX_BLOCKS)
    return fail(APBV_EINVAL, "n_blocks = %d outside 1..%d", L->n_blocks, APBV_MAX_BLOCKS);
  if (L->block_starts == nullptr) return fail(APBV_EINVAL, "block_starts is NULL");
  if (L->block_starts[0] != 0) return fail(APBV_EINVAL, "block_starts[0] = %d, expected 0", L->block_starts[0]);
  c.min_block = 0x7fffffff;
  c.max_block = 0;
  for (int v = 0; v < L->n_blocks; ++v) {
    const int64_t len = (int64_t)L->block_starts[v + 1] - L->block_starts[v];
    if (len <= 0) return fail(APBV_EINVAL, "block_starts not strictly increasing at block %d", v);
    c.min_block = len < c.min_block ? (int)len : c.min_block;
    c.max_block = len > c.max_block ? (int)len : c.max_block;
  }
  c.n = L->n_blocks;
  c.N = L->block_starts[c.n];
  if (L->hq <= 0 || L->hkv <= 0 || L->hq % L->hkv != 0)
    return fail(APBV_EINVAL, "hq = %d, hkv = %d: need positive with hq %% hkv == 0", L->hq, L->hkv);
  if (L->head_dim != 64 && L->head_dim != 128)
    return fail(APBV_EUNSUPPORTED, "head_dim = %d (supported: 64, 128)", L->head_dim);
  if (L->l_anchor < 0 || L->l_query < 0 || L->l_pass < 0)
    return fail(APBV_EINVAL, "negative l_anchor / l_query / l_pass");
  if (L->l_pass > c.min_block)
    return fail(APBV_EINVAL, "l_pass = %d exceeds the shortest block (%d)", L->l_pass, c.min_block);
  if (L->zigzag != 0 && L->zigzag != 1) return fail(APBV_EINVAL, "zigzag must be 0 or 1");
  if (!(L->scale >= 0.f) || isinf(L->scale)) return fail(APBV_EINVAL, "scale must be finite and >= 0");
  c.hq = L->hq;
  c.hkv = L->hkv;
  c.d = L->head_dim;
  c.G = L->hq / L->hkv;
  c.l_a = L->l_anchor;
  c.l_q = L->l_query;
  c.l_p = L->l_pass;
  const int64_t pre = (int64_t)c.l_a + (int64_t)c.n * c.l_p;
  if (pre > 0x7fffffff) return fail(APBV_EUNSUPPORTED, "prefix rows overflow int32");
  c.pre_rows = (int)pre;
  c.scale = L->scale == 0.f ? 1.0f / sqrtf((float)c.d) : L->scale;
  c.q_stride = L->q_row_stride == 0 ? (int64_t)c.hq * c.d : L->q_row_stride;
  c.kv_stride = L->kv_row_stride == 0 ? (int64_t)c.hkv * c.d : L->kv_row_stride;
  if (c.q_stride < (int64_t)c.hq * c.d || c.q_stride % 8 != 0)
    return fail(APBV_EINVAL, "q_row_stride = %lld must be >= hq*head_dim and a multiple of 8",
                (long long)c.q_stride);
  if (c.kv_stride < (int64_t)c.hkv * c.d || c.kv_stride % 8 != 0)
    return fail(APBV_EINVAL, "kv_row_stride = %lld must be >= hkv*head_dim and a multiple of 8",
                (long long)c.kv_stride);
  // tile loads address a K/V row with a 24-bit byte stride
  if (c.kv_stride >= (int64_t)1 << 22)
    return fail(APBV_EUNSUPPORTED, "kv_row_stride = %lld too large (limit 2^22 elements)",
                (long long)c.kv_stride);
  if ((int64_t)c.G * c.l_q > 0x7fffffff / 2) return fail(APBV_EUNSUPPORTED, "too many score rows");
  return APBV_OK;
}

apbv_status check_ptr(const void* p, const char* name, bool needed) {
  if (!needed) return APBV_OK;
  if (p == nullptr) return fail(APBV_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(APBV_EINVAL, "%s is not 16-byte aligned", name);
  return APBV_OK;
}

#define APBV_TRY(expr)                   \
  do {                                   \
    const apbv_status _s = (expr);       \
    if (_s != APBV_OK) return _s;        \
  } while (0)

int n_split_of(const Checked& c) { return (c.max_block + kScoreSplit - 1) / kScoreSplit; }

constexpr size_t kScratchBytes = sizeof(scratch);
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

// Device address of the scratch array on the calling thread's current device, looked up
// once per device with that device current.
apbv_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(APBV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(APBV_EUNSUPPORTED, "device %d: the scratch supports devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(APBV_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return APBV_OK;
}

}  // namespace

void build_schedule(Schedule& s, int32_t n_blocks, const int32_t* bs, int32_t zigzag,
                    int32_t tile_rows) {
  memset(&s, 0, sizeof(s));
  s.n_blocks = n_blocks;
  s.zigzag = zigzag;
  s.tile_rows = tile_rows;
  for (int v = 0; v <= n_blocks; ++v) s.bs[v] = bs[v];
  s.tiles_before[0] = 0;
  for (int v = 0; v < n_blocks; ++v) s.tiles_before[v + 1] = s.tiles_before[v] + s.tiles(v);
  const int nb = (n_blocks + 1) / 2;
  s.bucket_units[0] = 0;
  for (int b = 0; b < nb; ++b) {
    const int a = b, c = n_blocks - 1 - b;
    const int units = a != c ? (s.tiles(a) > s.tiles(c) ? s.tiles(a) : s.tiles(c))
                             : (s.tiles(a) + 1) / 2;
    s.bucket_units[b + 1] = s.bucket_units[b] + units;
  }
}

namespace {

// Checks of the scoring call and its parameters for blocks [v_begin, v_begin + v_count).
apbv_status score_params(const apbv_layout* layout, const Checked& c, const apbv_bf16* q_query,
                         const apbv_bf16* k_ctx, float* scores, int32_t* sel, void* workspace,
                         size_t workspace_bytes, ScoreParams& p) {
  APBV_TRY(check_ptr(q_query, "q_query", c.l_q > 0));
  APBV_TRY(check_ptr(k_ctx, "k_ctx", true));
  APBV_TRY(check_ptr(sel, "sel", c.l_p > 0));
  if (scores != nullptr && ((uintptr_t)scores & 3u) != 0)
    return fail(APBV_EINVAL, "scores is not 4-byte aligned");
  const int rows = c.G * c.l_q;
  if (score_colsum_lds_bytes(rows, c.d) > kMaxLdsBytes)
    return fail(APBV_EUNSUPPORTED, "G * l_query = %d score rows exceed the column-sum LDS", rows);
  const int n_split = n_split_of(c);
  const ScoreWorkspace ws = score_workspace(c.n, c.hkv, rows, n_split, c.N, c.d, scores == nullptr);
  const size_t need = ws.total;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(APBV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (workspace != nullptr && ((uintptr_t)workspace & 255u) != 0)
    return fail(APBV_EINVAL, "workspace is not 256-byte aligned");

  memset(&p, 0, sizeof(p));
  p.qq = q_query;
  p.kc = k_ctx;
  char* w = static_cast<char*>(workspace);
  p.stats = reinterpret_cast<float2*>(w + ws.stats);
  p.qp = reinterpret_cast<uint16_t*>(w + ws.qpack);
  p.scores = scores != nullptr ? scores : reinterpret_cast<float*>(w + ws.scores);
  p.sel = sel;
  p.kv_stride = c.kv_stride;
  p.hq = c.hq;
  p.hkv = c.hkv;
  p.group = c.G;
  p.l_query = c.l_q;
  p.rows = rows;
  p.q_rows = score_q_rows(rows);
  p.n_tokens = c.N;
  p.n_blocks = c.n;
  p.n_split = n_split;
  p.l_pass = c.l_p;
  p.v_begin = 0;
  p.v_count = c.n;
  p.scale_log2 = c.scale * 1.4426950408889634f;
  for (int v = 0; v <= c.n; ++v) p.bs[v] = layout->block_starts[v];
  return APBV_OK;
}

// Checks of the gather call and its parameters for prefix rows [row_begin, row_begin + count).
apbv_status gather_params(const apbv_layout* layout, const Checked& c, const apbv_bf16* k_anchor,
                          const apbv_bf16* v_anchor, const apbv_bf16* k_ctx,
                          const apbv_bf16* v_ctx, const int32_t* sel, apbv_bf16* k_pre,
                          apbv_bf16* v_pre, int32_t* sel_errors, GatherParams& p) {
  APBV_TRY(check_ptr(k_anchor, "k_anchor", c.l_a > 0));
  APBV_TRY(check_ptr(v_anchor, "v_anchor", c.l_a > 0));
  APBV_TRY(check_ptr(k_ctx, "k_ctx", c.l_p > 0));
  APBV_TRY(check_ptr(v_ctx, "v_ctx", c.l_p > 0));
  APBV_TRY(check_ptr(sel, "sel", c.l_p > 0));
  APBV_TRY(check_ptr(k_pre, "k_pre", c.pre_rows > 0));
  APBV_TRY(check_ptr(v_pre, "v_pre", c.pre_rows > 0));
  if (sel_errors != nullptr && ((uintptr_t)sel_errors & 3u) != 0)
    return fail(APBV_EINVAL, "sel_errors is not 4-byte aligned");
  memset(&p, 0, sizeof(p));
  p.sel_errors = sel_errors;
  for (int v = 0; v <= c.n; ++v) p.bs[v] = layout->block_starts[v];
  p.ka = k_anchor;
  p.va = v_anchor;
  p.kc = k_ctx;
  p.vc = v_ctx;
  p.sel = sel;
  p.kpre = k_pre;
  p.vpre = v_pre;
  p.kv_stride = c.kv_stride;
  p.hkv = c.hkv;
  p.l_anchor = c.l_a;
  p.l_pass = c.l_p;
  p.n_blocks = c.n;
  p.pre_rows = c.pre_rows;
  p.n_tokens = c.N;
  p.row_begin = 0;
  p.row_count = c.pre_rows;
  return APBV_OK;
}

// Checks of the attention call and its parameters for the whole schedule (the caller picks
// the unit range).
apbv_status attn_params(const apbv_layout* layout, const Checked& c, const apbv_bf16* q_ctx,
                        const apbv_bf16* k_pre, const apbv_bf16* v_pre, const apbv_bf16* k_ctx,
                        const apbv_bf16* v_ctx, apbv_bf16* out, float* lse, AttnParams& p) {
  APBV_TRY(check_ptr(q_ctx, "q_ctx", true));
  APBV_TRY(check_ptr(k_ctx, "k_ctx", true));
  APBV_TRY(check_ptr(v_ctx, "v_ctx", true));
  APBV_TRY(check_ptr(k_pre, "k_pre", c.pre_rows > 0));
  APBV_TRY(check_ptr(v_pre, "v_pre", c.pre_rows > 0));
  APBV_TRY(check_ptr(out, "out", true));
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return fail(APBV_EINVAL, "lse is not 4-byte aligned");
  if ((int64_t)c.hq * c.N > 0x7fffffffLL * 8) return fail(APBV_EUNSUPPORTED, "problem too large");
  memset(&p, 0, sizeof(p));
  build_schedule(p.sched, c.n, layout->block_starts, layout->zigzag, attn_tile_rows(c.d));
  p.q = q_ctx;
  p.kpre = k_pre;
  p.vpre = v_pre;
  p.kc = k_ctx;
  p.vc = v_ctx;
  p.out = out;
  p.lse = lse;
  p.q_stride = c.q_stride;
  p.kv_stride = c.kv_stride;
  p.hq = c.hq;
  p.hkv = c.hkv;
  p.group = c.G;
  p.l_anchor = c.l_a;
  p.l_pass = c.l_p;
  p.pre_rows = c.pre_rows;
  p.n_tokens = c.N;
  p.scale_log2 = c.scale * 1.4426950408889634f;
  return APBV_OK;
}

// Launch of the attention over buckets (zigzag) or blocks [range_begin, range_end).
apbv_status launch_attn_range(AttnParams& p, const Checked& c, int range_begin, int range_end,
                              hipStream_t stream) {
  p.unit_begin = p.sched.units_before(range_begin);
  p.n_units = p.sched.units_before(range_end) - p.unit_begin;
  if ((uint64_t)p.n_units * (uint64_t)p.hq >= (1ull << 32))
    return fail(APBV_EUNSUPPORTED, "grid too large");
  const hipError_t e = launch_attention(p, c.d, stream);
  if (e != hipSuccess) return fail(APBV_EHIP, "attention launch: %s", hipGetErrorString(e));
  return APBV_OK;
}

// Split of the whole-layer workspace: the scoring part (statistics and scores), rounded up
// to 256 bytes; the query partials follow it.
size_t layer_workspace_split(const Checked& c) {
  const size_t w = score_workspace_bytes(c.n, c.hkv, c.G * c.l_q, n_split_of(c), c.N, c.d, true);
  return (w + 255) & ~(size_t)255;
}

// Checks of the query-row call and its parameters.
apbv_status query_params(const Checked& c, const apbv_bf16* q_query, const apbv_bf16* k_query,
                         const apbv_bf16* v_query, const apbv_bf16* k_anchor,
                         const apbv_bf16* v_anchor, const apbv_bf16* k_ctx,
                         const apbv_bf16* v_ctx, apbv_bf16* out, float* lse, void* workspace,
                         size_t workspace_bytes, QueryParams& p, QueryPlan& q) {
  const bool any = c.l_q > 0;
  APBV_TRY(check_ptr(q_query, "q_query", any));
  APBV_TRY(check_ptr(k_query, "k_query", any));
  APBV_TRY(check_ptr(v_query, "v_query", any));
  APBV_TRY(check_ptr(k_anchor, "k_anchor", any && c.l_a > 0));
  APBV_TRY(check_ptr(v_anchor, "v_anchor", any && c.l_a > 0));
  APBV_TRY(check_ptr(k_ctx, "k_ctx", any));
  APBV_TRY(check_ptr(v_ctx, "v_ctx", any));
  APBV_TRY(check_ptr(out, "out", any));
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return fail(APBV_EINVAL, "lse is not 4-byte aligned");
  q = plan_query(c.l_a, c.N, c.l_q, c.hq, c.hkv, c.d);
  const size_t need = any ? q.o_bytes + q.lse_bytes : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(APBV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (workspace != nullptr && ((uintptr_t)workspace & 255u) != 0)
    return fail(APBV_EINVAL, "workspace is not 256-byte aligned");
  if ((uint64_t)q.row_tiles * c.hkv * q.n_chunks >= (1ull << 31))
    return fail(APBV_EUNSUPPORTED, "query grid too large");
  memset(&p, 0, sizeof(p));
  p.qq = q_query;
  p.kq = k_query;
  p.vq = v_query;
  p.ka = k_anchor;
  p.va = v_anchor;
  p.kc = k_ctx;
  p.vc = v_ctx;
  p.part_o = reinterpret_cast<float*>(workspace);
  p.part_lse = workspace == nullptr
                   ? nullptr
                   : reinterpret_cast<float*>(static_cast<char*>(workspace) + q.o_bytes);
  p.out = out;
  p.lse = lse;
  p.kv_stride = c.kv_stride;
  p.hq = c.hq;
  p.hkv = c.hkv;
  p.group = c.G;
  p.l_query = c.l_q;
  p.l_anchor = c.l_a;
  p.n_tokens = c.N;
  p.chunk_keys = q.chunk_keys;
  p.n_anchor_chunks = q.n_anchor_chunks;
  p.n_ctx_chunks = q.n_ctx_chunks;
  p.n_query_chunks = q.n_query_chunks;
  p.n_chunks = q.n_chunks;
  p.row_tiles = q.row_tiles;
  p.scale_log2 = c.scale * 1.4426950408889634f;
  return APBV_OK;
}

// Attention parameters of the anchor rows: the anchor opens the sequence, so its rows are
// dense causal attention over the anchor alone (one block, no prefix).
apbv_status anchor_params(const Checked& c, const apbv_bf16* q_anchor, const apbv_bf16* k_anchor,
                          const apbv_bf16* v_anchor, apbv_bf16* out, float* lse, AttnParams& p) {
  APBV_TRY(check_ptr(q_anchor, "q_anchor", true));
  APBV_TRY(check_ptr(k_anchor, "k_anchor", true));
  APBV_TRY(check_ptr(v_anchor, "v_anchor", true));
  APBV_TRY(check_ptr(out, "anchor_out", true));
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0)
    return fail(APBV_EINVAL, "anchor_lse is not 4-byte aligned");
  memset(&p, 0, sizeof(p));
  const int32_t bs[2] = {0, c.l_a};
  build_schedule(p.sched, 1, bs, 1, attn_tile_rows(c.d));
  p.q = q_anchor;
  p.kc = k_anchor;
  p.vc = v_anchor;
  p.out = out;
  p.lse = lse;
  p.q_stride = (int64_t)c.hq * c.d;
  p.kv_stride = (int64_t)c.hkv * c.d;
  p.hq = c.hq;
  p.hkv = c.hkv;
  p.group = c.G;
  p.n_tokens = c.l_a;
  p.scale_log2 = c.scale * 1.4426950408889634f;
  return APBV_OK;
}

// Split of one layer for the two-stream overlap. Attention of the buckets [late, n_buckets)
// needs the selections of blocks [0, early) only: with ZigZag, bucket b holds blocks b and
// n-1-b, so the late set's highest block is n-1-late and early = n-1-late. The late set is
// the smallest one whose workgroups (one per CU at a time) fill whole rounds of the compute
// units, so that splitting the attention into two launches adds no partial round; late = 0
// (one attention launch, only the last block scored beside it) when none does. Without
// passing blocks nothing is selected before attention: late = 0, early = 0.
void plan_layer(const Checked& c, const Schedule& s, int compute_units, int& late, int& early) {
  const int nb = s.n_buckets();
  late = 0;
  early = c.l_p == 0 ? 0 : c.n - 1;
  if (c.l_p == 0 || !s.zigzag || compute_units <= 0) return;
  for (int b = nb - 1; b >= 1; --b) {
    const int64_t wgs = (int64_t)(s.units_before(nb) - s.units_before(b)) * c.hq;
    if (wgs % compute_units == 0) {
      late = b;
      early = c.n - 1 - b;
      return;
    }
  }
}

}  // namespace
}  // namespace apbv

using namespace apbv;

extern "C" {


const char* apbv_version(void) { return "apbv-gfx950 0.1.0"; }

const char* apbv_last_error(void) { return g_err; }

const char* apbv_status_str(apbv_status s) {
  switch (s) {
    case APBV_OK: return "ok";
    case APBV_EINVAL: return "invalid argument";
    case APBV_EUNSUPPORTED: return "unsupported configuration";
    case APBV_EWORKSPACE: return "workspace missing or too small";
    case APBV_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

int32_t apbv_attn_tile_rows(int32_t head_dim) { return attn_tile_rows(head_dim); }

int32_t apbv_num_buckets(const apbv_layout* layout) {
  Checked c;
  if (check_layout(layout, c) != APBV_OK) return -1;
  return layout->zigzag ? (c.n + 1) / 2 : c.n;
}

apbv_status apbv_score_select_workspace(const apbv_layout* layout, size_t* bytes) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  if (bytes == nullptr) return fail(APBV_EINVAL, "bytes is NULL");
  *bytes = score_workspace_bytes(c.n, c.hkv, c.G * c.l_q, n_split_of(c), c.N, c.d, true);
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_score_select(const apbv_layout* layout, const apbv_bf16* q_query,
                              const apbv_bf16* k_ctx, float* scores, int32_t* sel,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  ScoreParams p;
  APBV_TRY(score_params(layout, c, q_query, k_ctx, scores, sel, workspace, workspace_bytes, p));
  const hipError_t e = launch_score_select(p, c.d, c.max_block, (hipStream_t)stream);
  if (e != hipSuccess) return fail(APBV_EHIP, "score/select launch: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_score_select_noalloc(const apbv_layout* layout, const apbv_bf16* q_query,
                                      const apbv_bf16* k_ctx, float* scores, int32_t* sel,
                                      void* stream) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  const size_t need =
      score_workspace_bytes(c.n, c.hkv, c.G * c.l_q, n_split_of(c), c.N, c.d, scores == nullptr);
  if (need > kScratchBytes)
    return fail(APBV_EUNSUPPORTED,
                "this layout needs %zu bytes of scratch, the allocation-free entry point has "
                "%zu (use apbv_score_select with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  APBV_TRY(scratch_of_current_device(&ws));
  ScoreParams p;
  APBV_TRY(score_params(layout, c, q_query, k_ctx, scores, sel, ws, kScratchBytes, p));
  const hipError_t e = launch_score_select(p, c.d, c.max_block, (hipStream_t)stream);
  if (e != hipSuccess) return fail(APBV_EHIP, "score/select launch: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_gather_passing(const apbv_layout* layout, const apbv_bf16* k_anchor,
                                const apbv_bf16* v_anchor, const apbv_bf16* k_ctx,
                                const apbv_bf16* v_ctx, const int32_t* sel, apbv_bf16* k_pre,
                                apbv_bf16* v_pre, int32_t* sel_errors, void* stream) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  GatherParams p;
  APBV_TRY(gather_params(layout, c, k_anchor, v_anchor, k_ctx, v_ctx, sel, k_pre, v_pre,
                         sel_errors, p));
  const hipError_t e = launch_gather(p, c.d, (hipStream_t)stream);
  if (e != hipSuccess) return fail(APBV_EHIP, "gather launch: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_schedule(const apbv_layout* layout, int32_t range_begin, int32_t range_end,
                          int32_t* units, int32_t capacity, int32_t* count) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  if (count == nullptr) return fail(APBV_EINVAL, "count is NULL");
  Schedule s;
  build_schedule(s, c.n, layout->block_starts, layout->zigzag, attn_tile_rows(c.d));
  const int nb = s.n_buckets();
  if (range_begin == 0 && range_end == 0) range_end = nb;
  if (range_begin < 0 || range_end > nb || range_begin > range_end)
    return fail(APBV_EINVAL, "range [%d, %d) outside [0, %d]", range_begin, range_end, nb);
  const int u0 = s.units_before(range_begin), u1 = s.units_before(range_end);
  *count = u1 - u0;
  if (units != nullptr) {
    if (capacity < *count) return fail(APBV_EINVAL, "capacity %d < %d units", capacity, *count);
    for (int u = u0; u < u1; ++u) {
      int va, ta, vb, tb;
      s.decode(u, va, ta, vb, tb);
      int32_t* o = units + 4 * (u - u0);
      o[0] = va; o[1] = va >= 0 ? ta : -1; o[2] = vb; o[3] = vb >= 0 ? tb : -1;
    }
  }
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_approx_attn_prefill(const apbv_layout* layout, const apbv_bf16* q_ctx,
                                     const apbv_bf16* k_pre, const apbv_bf16* v_pre,
                                     const apbv_bf16* k_ctx, const apbv_bf16* v_ctx,
                                     apbv_bf16* out, float* lse, int32_t range_begin,
                                     int32_t range_end, void* stream) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  AttnParams p;
  APBV_TRY(attn_params(layout, c, q_ctx, k_pre, v_pre, k_ctx, v_ctx, out, lse, p));
  const int nb = p.sched.n_buckets();
  if (range_begin == 0 && range_end == 0) range_end = nb;
  if (range_begin < 0 || range_end > nb || range_begin > range_end)
    return fail(APBV_EINVAL, "range [%d, %d) outside [0, %d]", range_begin, range_end, nb);
  APBV_TRY(launch_attn_range(p, c, range_begin, range_end, (hipStream_t)stream));
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_prefill_layer_plan(const apbv_layout* layout, int32_t compute_units,
                                    int32_t* late_bucket_begin, int32_t* early_blocks) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  if (late_bucket_begin == nullptr || early_blocks == nullptr)
    return fail(APBV_EINVAL, "late_bucket_begin / early_blocks is NULL");
  Schedule s;
  build_schedule(s, c.n, layout->block_starts, layout->zigzag, attn_tile_rows(c.d));
  int late, early;
  plan_layer(c, s, compute_units, late, early);
  *late_bucket_begin = late;
  *early_blocks = early;
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_prefill_layer(const apbv_layout* layout, const apbv_bf16* q_query,
                               const apbv_bf16* q_ctx, const apbv_bf16* k_ctx,
                               const apbv_bf16* v_ctx, const apbv_bf16* k_anchor,
                               const apbv_bf16* v_anchor, float* scores, int32_t* sel,
                               apbv_bf16* k_pre, apbv_bf16* v_pre, apbv_bf16* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream,
                               void* aux_stream, void* ready_event, void* done_event,
                               int32_t compute_units) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  ScoreParams sp;
  APBV_TRY(score_params(layout, c, q_query, k_ctx, scores, sel, workspace, workspace_bytes, sp));
  GatherParams gp;
  APBV_TRY(gather_params(layout, c, k_anchor, v_anchor, k_ctx, v_ctx, sel, k_pre, v_pre,
                         nullptr, gp));
  AttnParams ap;
  APBV_TRY(attn_params(layout, c, q_ctx, k_pre, v_pre, k_ctx, v_ctx, out, lse, ap));
  const int nb = ap.sched.n_buckets();
  hipStream_t s0 = (hipStream_t)stream;
  hipError_t e;
  if (aux_stream == nullptr) {   // the three steps in order on one stream
    if ((e = launch_score_select(sp, c.d, c.max_block, s0)) != hipSuccess ||
        (e = launch_gather(gp, c.d, s0)) != hipSuccess)
      return fail(APBV_EHIP, "layer launch: %s", hipGetErrorString(e));
    APBV_TRY(launch_attn_range(ap, c, 0, nb, s0));
    g_err[0] = 0;
    return APBV_OK;
  }
  if (ready_event == nullptr || done_event == nullptr)
    return fail(APBV_EINVAL, "an aux stream needs ready_event and done_event");
  if (aux_stream == stream) return fail(APBV_EINVAL, "aux_stream is the main stream");
  if (compute_units < 0) return fail(APBV_EINVAL, "compute_units = %d", compute_units);
  int cus = compute_units;
  if (cus == 0) {
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return fail(APBV_EHIP, "device query: %s", hipGetErrorString(e));
  }
  int late, early;
  plan_layer(c, ap.sched, cus, late, early);
  hipStream_t s1 = (hipStream_t)aux_stream;
  hipEvent_t ready = (hipEvent_t)ready_event, done = (hipEvent_t)done_event;
  const int split_row = c.l_a + early * c.l_p;
  // main stream: the early blocks' selections and prefix rows, then the late buckets
  sp.v_begin = 0;
  sp.v_count = early;
  gp.row_begin = 0;
  gp.row_count = split_row;
  if ((e = launch_score_select(sp, c.d, c.max_block, s0)) != hipSuccess ||
      (e = launch_gather(gp, c.d, s0)) != hipSuccess ||
      (e = hipEventRecord(ready, s0)) != hipSuccess)
    return fail(APBV_EHIP, "layer launch: %s", hipGetErrorString(e));
  APBV_TRY(launch_attn_range(ap, c, late, nb, s0));
  // aux stream, once the main stream has reached the attention: the remaining blocks
  sp.v_begin = early;
  sp.v_count = c.n - early;
  gp.row_begin = split_row;
  gp.row_count = c.pre_rows - split_row;
  if ((e = hipStreamWaitEvent(s1, ready, 0)) != hipSuccess ||
      (e = launch_score_select(sp, c.d, c.max_block, s1)) != hipSuccess ||
      (e = launch_gather(gp, c.d, s1)) != hipSuccess ||
      (e = hipEventRecord(done, s1)) != hipSuccess ||
      (e = hipStreamWaitEvent(s0, done, 0)) != hipSuccess)
    return fail(APBV_EHIP, "layer launch: %s", hipGetErrorString(e));
  // main stream: the early buckets, after the aux stream's selections and prefix rows
  APBV_TRY(launch_attn_range(ap, c, 0, late, s0));
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_query_forward_workspace(const apbv_layout* layout, size_t* bytes) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  if (bytes == nullptr) return fail(APBV_EINVAL, "bytes is NULL");
  const QueryPlan q = plan_query(c.l_a, c.N, c.l_q, c.hq, c.hkv, c.d);
  *bytes = c.l_q > 0 ? q.o_bytes + q.lse_bytes : 0;
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_query_forward(const apbv_layout* layout, const apbv_bf16* q_query,
                               const apbv_bf16* k_query, const apbv_bf16* v_query,
                               const apbv_bf16* k_anchor, const apbv_bf16* v_anchor,
                               const apbv_bf16* k_ctx, const apbv_bf16* v_ctx, apbv_bf16* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  QueryParams p;
  QueryPlan q;
  APBV_TRY(query_params(c, q_query, k_query, v_query, k_anchor, v_anchor, k_ctx, v_ctx, out, lse,
                        workspace, workspace_bytes, p, q));
  if (c.l_q > 0) {
    const hipError_t e = launch_query(p, c.d, (hipStream_t)stream);
    if (e != hipSuccess) return fail(APBV_EHIP, "query forward launch: %s", hipGetErrorString(e));
  }
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_layer_workspace(const apbv_layout* layout, size_t* bytes) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  if (bytes == nullptr) return fail(APBV_EINVAL, "bytes is NULL");
  *bytes = layer_workspace_split(c);
  const QueryPlan q = plan_query(c.l_a, c.N, c.l_q, c.hq, c.hkv, c.d);
  *bytes += c.l_q > 0 ? q.o_bytes + q.lse_bytes : 0;
  g_err[0] = 0;
  return APBV_OK;
}

apbv_status apbv_layer_forward(const apbv_layout* layout, const apbv_layer_io* io,
                               void* stream) {
  Checked c;
  APBV_TRY(check_layout(layout, c));
  if (io == nullptr) return fail(APBV_EINVAL, "io is NULL");
  hipStream_t s0 = (hipStream_t)stream;
  const size_t split = layer_workspace_split(c);
  if (io->workspace != nullptr && ((uintptr_t)io->workspace & 255u) != 0)
    return fail(APBV_EINVAL, "workspace is not 256-byte aligned");
  if (io->workspace_bytes < split && split > 0)
    return fail(APBV_EWORKSPACE, "workspace of at least %zu bytes needed, %zu given", split,
                io->workspace_bytes);
  // every part is validated before anything is launched
  const bool anchor_rows = io->anchor_out != nullptr && c.l_a > 0;
  AttnParams anc;
  if (anchor_rows) {
    APBV_TRY(anchor_params(c, io->q_anchor, io->k_anchor, io->v_anchor, io->anchor_out,
                           io->anchor_lse, anc));
  }
  ScoreParams sp;
  APBV_TRY(score_params(layout, c, io->q_query, io->k_ctx, io->scores, io->sel, io->workspace,
                        split, sp));
  GatherParams gp;
  APBV_TRY(gather_params(layout, c, io->k_anchor, io->v_anchor, io->k_ctx, io->v_ctx, io->sel,
                         io->k_pre, io->v_pre, nullptr, gp));
  AttnParams ap;
  APBV_TRY(attn_params(layout, c, io->q_ctx, io->k_pre, io->v_pre, io->k_ctx, io->v_ctx,
                       io->out, io->lse, ap));
  const bool query_rows = io->query_out != nullptr && c.l_q > 0;
  QueryParams qp;
  QueryPlan qplan;
  if (query_rows) {
    char* qws = io->workspace == nullptr ? nullptr : static_cast<char*>(io->workspace) + split;
    APBV_TRY(query_params(c, io->q_query, io->k_query, io->v_query, io->k_anchor, io->v_anchor,
                          io->k_ctx, io->v_ctx, io->query_out, io->query_lse, qws,
                          io->workspace_bytes - split, qp, qplan));
  }
  hipError_t e;
  if (anchor_rows) APBV_TRY(launch_attn_range(anc, c, 0, 1, s0));
  if ((e = launch_score_select(sp, c.d, c.max_block, s0)) != hipSuccess ||
      (e = launch_gather(gp, c.d, s0)) != hipSuccess)
    return fail(APBV_EHIP, "layer launch: %s", hipGetErrorString(e));
  APBV_TRY(launch_attn_range(ap, c, 0, ap.sched.n_buckets(), s0));
  if (query_rows && (e = launch_query(qp, c.d, s0)) != hipSuccess)
    return fail(APBV_EHIP, "query forward launch: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return APBV_OK;
}

}  // extern "C"
