// Rows of the query block, computed in the same forward as the context ("Riepilogo Tecnico:
// APB-V" on gist.science, Metodologia part 2, "Forward Fuso di Contesto e Query": the
// query's partial attention results over different key sets are merged through the
// log-sum-exp that flash attention returns). The query block closes the sequence, so its
// rows are exact: row i of head h sees every anchor key, every context key and the query
// block's keys 0..i.
//
// Two kernels:
//  1. query_partial_kernel: one workgroup = 8 waves x 32 rows over one chunk of keys of
//     one KV head (the chunk length is chosen so that the grid fills whole rounds of the
//     256 compute units), through the pipelined tile loop of attn_pipe.h. The rows are the
//     G heads of the KV group times the l_q query rows, packed into the MFMA row
//     dimension, so each K/V tile staged in LDS serves the whole group. It writes the
//     chunk's normalised fp32 output and lse.
//  2. query_merge_kernel: one wave per (head, row) folds the chunks through their lse and
//     writes the bf16 output and the row's lse.
#include "apbv_device.h"
#include "apbv_internal.h"
#include "attn_pipe.h"

namespace apbv {

namespace {

using namespace pipe;

template <int D>
__global__ __launch_bounds__(kWaves * 64) void query_partial_kernel(const QueryParams p) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[G::KELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t K1[G::KELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[G::VELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t V1[G::VELEMS];
  Loader<D> ld;
  ld.init();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // workgroup -> (row tile, KV head, chunk); the row tiles of one chunk and KV head read the
  // same keys and sit next to each other on one XCD
  const uint32_t total = (uint32_t)p.row_tiles * p.hkv * p.n_chunks;
  const uint32_t L = xcd_contiguous(blockIdx.x, total);
  const int pt = (int)(L % p.row_tiles);
  const int g = (int)((L / p.row_tiles) % p.hkv);
  const int c = (int)(L / ((uint32_t)p.row_tiles * p.hkv));

  // chunk -> key source; causal chunks count key positions from the query block's start
  const uint16_t *kb, *vb;
  int64_t stride;
  int len, kpos0;
  bool causal = false;
  if (c < p.n_anchor_chunks) {
    kpos0 = c * p.chunk_keys;
    len = min(p.chunk_keys, p.l_anchor - kpos0);
    stride = (int64_t)p.hkv * D;
    kb = p.ka + (int64_t)kpos0 * stride + g * D;
    vb = p.va + (int64_t)kpos0 * stride + g * D;
  } else if (c < p.n_anchor_chunks + p.n_ctx_chunks) {
    kpos0 = (c - p.n_anchor_chunks) * p.chunk_keys;
    len = min(p.chunk_keys, p.n_tokens - kpos0);
    stride = p.kv_stride;
    kb = p.kc + (int64_t)kpos0 * stride + g * D;
    vb = p.vc + (int64_t)kpos0 * stride + g * D;
  } else {
    kpos0 = (c - p.n_anchor_chunks - p.n_ctx_chunks) * p.chunk_keys;
    len = min(p.chunk_keys, p.l_query - kpos0);
    stride = (int64_t)p.hkv * D;
    kb = p.kq + (int64_t)kpos0 * stride + g * D;
    vb = p.vq + (int64_t)kpos0 * stride + g * D;
    causal = true;
  }

  // packed row r -> head g*G + r / l_q, query row r % l_q
  const int n_rows = p.group * p.l_query;
  const int wr0 = pt * kRows + wave * 32;            // first packed row of this wave
  const int r = wr0 + l32;
  const int rr = min(r, n_rows - 1);
  const int h = g * p.group + rr / p.l_query;
  const int i = rr % p.l_query;
  const bool wave_live = wr0 < n_rows;
  // range of query positions among the wave's rows (exact when they do not wrap)
  const int first = wr0 % p.l_query;
  const bool straight = first + 31 < p.l_query && wr0 + 31 < n_rows;
  const int pmin = straight ? first : 0;
  const int pmax = straight ? first + 31 : p.l_query - 1;

  bf16x8 qf[G::NK];
  {
    const uint16_t* qrow = p.qq + ((int64_t)i * p.hq + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < G::NK; ++ks) qf[ks] = as_bf16x8(load16(qrow + ks * 16));
  }
  f32x16 o[G::ND];
#pragma unroll
  for (int db = 0; db < G::ND; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (len + kKT - 1) / kKT;
  // tiles this wave computes: all of them, except that a causal chunk ends for the wave at
  // its last query position, and a wave past the packed rows computes nothing
  const int n_live = !wave_live ? 0
                     : !causal  ? ntiles
                     : pmax < kpos0 ? 0 : min(ntiles, (pmax - kpos0) / kKT + 1);
  auto source = [&](int t) -> KeySrc {
    KeySrc s;
    s.k = kb + (int64_t)t * kKT * stride;
    s.v = vb + (int64_t)t * kKT * stride;
    s.stride = stride;
    s.valid = min(kKT, len - t * kKT);
    return s;
  };
  auto mask_of = [&](int t) {
    TileMask m;
    m.key0 = kpos0 + t * kKT;
    m.valid = min(kKT, len - t * kKT);
    m.mask = m.valid < kKT || (causal && m.key0 + kKT - 1 > pmin);
    m.pos = causal ? i : kNoCausal;
    return m;
  };
  run_tiles<D>(ntiles, n_live, source, mask_of, qf, o, m_run, l_run, p.scale_log2, K0, K1, V0,
               V1, ld);

  // normalised partial output (fp32) and natural-log lse; a row that saw no key of this
  // chunk (causal chunk past the row) gets output 0 and lse -inf
  const float lt = l_run + swap_half(l_run);
  if (r < n_rows) {
    const int64_t prow = ((int64_t)c * p.hq + h) * p.l_query + i;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    float* orow = p.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < G::ND; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * half;
        const f32x16& ov = o[db];
        float4 w = {ov[4 * q4 + 0] * inv, ov[4 * q4 + 1] * inv, ov[4 * q4 + 2] * inv,
                    ov[4 * q4 + 3] * inv};
        *reinterpret_cast<float4*>(orow + d0) = w;
      }
    if (half == 0)
      p.part_lse[prow] = lt > 0.f ? (m_run + fast_log2(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

// One wave per (head, query row): out = sum_c exp(lse_c - M) o_c / sum_c exp(lse_c - M),
// lse = M + log(sum_c exp(lse_c - M)), M = max_c lse_c.
template <int D>
__global__ __launch_bounds__(256) void query_merge_kernel(const QueryParams p) {
  constexpr int E = D / 64;   // output columns per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // h * l_q + i
  const int n_rows = p.hq * p.l_query;
  if (row >= n_rows) return;
  const int h = row / p.l_query, i = row % p.l_query;
  float top = -INFINITY;
  for (int c = 0; c < p.n_chunks; ++c) top = fmaxf(top, p.part_lse[(int64_t)c * n_rows + row]);
  float acc[E], wsum = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int c = 0; c < p.n_chunks; ++c) {
    const float lc = p.part_lse[(int64_t)c * n_rows + row];
    if (lc == -INFINITY) continue;
    const float w = expf(lc - top);
    wsum += w;
    const float* src = p.part_o + ((int64_t)c * n_rows + row) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(w, src[e], acc[e]);
  }
  const float inv = 1.0f / wsum;
  uint16_t* dst = p.out + ((int64_t)i * p.hq + h) * D + lane * E;
  if (E == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[E - 1] * inv);
  } else {
    const uint32_t w = pack_bf16x2(acc[0] * inv, 0.f);
    dst[0] = (uint16_t)(w & 0xffffu);
  }
  if (p.lse != nullptr && lane == 0) p.lse[(int64_t)h * p.l_query + i] = top + logf(wsum);
}

}  // namespace

QueryPlan plan_query(int l_anchor, int n_tokens, int l_query, int hq, int hkv, int head_dim) {
  QueryPlan q;
  const int64_t rows = (int64_t)(hq / hkv) * l_query;
  q.row_tiles = (int)((rows + kRows - 1) / kRows);
  // chunk length: among multiples of 64 keys from 1024 to 8192, the one whose grid wastes
  // the least of its last round on 256 compute units (the largest such chunk on ties, for
  // fewer partials), preferring grids of at least two rounds
  auto chunks_of = [&](int ck) {
    return (l_anchor + ck - 1) / ck + (n_tokens + ck - 1) / ck + (l_query + ck - 1) / ck;
  };
  constexpr int kCUs = 256;
  int best = 8192;
  double best_eff = -1.0;
  for (int ck = 8192; ck >= 1024; ck -= 64) {
    const int64_t wgs = (int64_t)q.row_tiles * hkv * chunks_of(ck);
    const int64_t rounds = (wgs + kCUs - 1) / kCUs;
    const double eff = (double)wgs / (double)(rounds * kCUs) - (rounds < 2 ? 1.0 : 0.0);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = ck;
    }
  }
  q.chunk_keys = best;
  q.n_anchor_chunks = (l_anchor + best - 1) / best;
  q.n_ctx_chunks = (n_tokens + best - 1) / best;
  q.n_query_chunks = (l_query + best - 1) / best;
  q.n_chunks = q.n_anchor_chunks + q.n_ctx_chunks + q.n_query_chunks;
  const size_t prow = (size_t)q.n_chunks * hq * l_query;
  q.o_bytes = (prow * head_dim * sizeof(float) + 255) & ~(size_t)255;
  q.lse_bytes = (prow * sizeof(float) + 255) & ~(size_t)255;
  return q;
}

hipError_t launch_query(const QueryParams& p, int head_dim, hipStream_t stream) {
  if (p.l_query == 0) return hipSuccess;
  const dim3 g1((uint32_t)p.row_tiles * p.hkv * p.n_chunks);
  const dim3 g2((uint32_t)((p.hq * p.l_query + 3) / 4));
  if (head_dim == 128) {
    hipLaunchKernelGGL(query_partial_kernel<128>, g1, dim3(kWaves * 64), 0, stream, p);
    hipLaunchKernelGGL(query_merge_kernel<128>, g2, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(query_partial_kernel<64>, g1, dim3(kWaves * 64), 0, stream, p);
    hipLaunchKernelGGL(query_merge_kernel<64>, g2, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace apbv
