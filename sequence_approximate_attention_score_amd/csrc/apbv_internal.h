// Internal parameter blocks and launchers of the gfx950 kernels (host + device visible).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/apbv.h"

namespace apbv {

// ---------------------------------------------------------------- attention work schedule
// A work unit is up to two query tiles ("parts") processed one after the other by one
// workgroup for one query head. With ZigZag, bucket b holds blocks b and n-1-b; its unit t
// pairs tile t of block b with tile T-1-t of block n-1-b, so every unit of a bucket of
// equal blocks carries the same number of (row, key) pairs: the prefix lengths add to
// 2*l_anchor + (n-1)*l_pass and the causal spans add to T+1 tiles.
struct Schedule {
  int32_t n_blocks;
  int32_t zigzag;
  int32_t tile_rows;
  int32_t bs[APBV_MAX_BLOCKS + 1];
  int32_t tiles_before[APBV_MAX_BLOCKS + 1];      // block order: prefix sums of tile counts
  int32_t bucket_units[APBV_MAX_BLOCKS / 2 + 2];  // ZigZag: prefix sums of units per bucket

  __host__ __device__ int tiles(int v) const {
    return (bs[v + 1] - bs[v] + tile_rows - 1) / tile_rows;
  }
  __host__ __device__ int n_buckets() const { return zigzag ? (n_blocks + 1) / 2 : n_blocks; }
  __host__ __device__ int units_before(int range) const {
    return zigzag ? bucket_units[range] : tiles_before[range];
  }
  // Unit u -> parts (va, ta) and (vb, tb); a part with block -1 is absent.
  __host__ __device__ void decode(int u, int& va, int& ta, int& vb, int& tb) const {
    va = vb = -1;
    ta = tb = 0;
    if (zigzag) {
      const int nb = (n_blocks + 1) / 2;
      int b = 0;
      while (b + 1 < nb && bucket_units[b + 1] <= u) ++b;
      const int t = u - bucket_units[b];
      const int a = b, c = n_blocks - 1 - b;
      const int Ta = tiles(a);
      if (a != c) {
        const int Tc = tiles(c);
        if (t < Ta) { va = a; ta = t; }
        if (t < Tc) { vb = c; tb = Tc - 1 - t; }
      } else {
        va = a; ta = t;
        if (Ta - 1 - t != t) { vb = a; tb = Ta - 1 - t; }
      }
    } else {
      int v = 0;
      while (v + 1 < n_blocks && tiles_before[v + 1] <= u) ++v;
      va = v; ta = u - tiles_before[v];
    }
  }
};

void build_schedule(Schedule& s, int32_t n_blocks, const int32_t* bs, int32_t zigzag,
                    int32_t tile_rows);

// ---------------------------------------------------------------- attention
struct AttnParams {
  const uint16_t* q;
  const uint16_t* kpre;
  const uint16_t* vpre;
  const uint16_t* kc;
  const uint16_t* vc;
  uint16_t* out;
  float* lse;
  int64_t q_stride;     // elements between tokens of q
  int64_t kv_stride;    // elements between tokens of kc / vc
  int32_t hq, hkv, group;
  int32_t l_anchor, l_pass, pre_rows;
  int32_t n_tokens;
  float scale_log2;     // softmax scale * log2(e)
  int32_t unit_begin, n_units;
  Schedule sched;
};

int attn_tile_rows(int head_dim);
hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream);

// ---------------------------------------------------------------- query-block rows
// Keys of the query rows = [anchor | context | query block (causal)], cut into chunks of
// chunk_keys keys that never straddle two sources; chunk c of the grid computes the
// normalised partial output and lse of every query row over its keys, and the merge
// combines the chunks of a row through their lse.
struct QueryParams {
  const uint16_t* qq;   // [l_q, hq, d]
  const uint16_t* kq;   // [l_q, hkv, d]
  const uint16_t* vq;
  const uint16_t* ka;   // [l_a, hkv, d]
  const uint16_t* va;
  const uint16_t* kc;   // [N, hkv, d] with kv_stride
  const uint16_t* vc;
  float* part_o;        // [n_chunks, hq, l_q, d]
  float* part_lse;      // [n_chunks, hq, l_q] (natural log, -inf when no key is visible)
  uint16_t* out;        // [l_q, hq, d]
  float* lse;           // [hq, l_q] or null
  int64_t kv_stride;
  int32_t hq, hkv, group, l_query, l_anchor, n_tokens;
  int32_t chunk_keys, n_anchor_chunks, n_ctx_chunks, n_query_chunks, n_chunks, row_tiles;
  float scale_log2;
};

struct QueryPlan {
  int chunk_keys;   // keys per partial, a multiple of the 64-key tile
  int n_anchor_chunks, n_ctx_chunks, n_query_chunks, n_chunks, row_tiles;
  size_t o_bytes, lse_bytes;   // workspace parts, each rounded up to 256 bytes
};
QueryPlan plan_query(int l_anchor, int n_tokens, int l_query, int hq, int hkv, int head_dim);
hipError_t launch_query(const QueryParams& p, int head_dim, hipStream_t stream);

// ---------------------------------------------------------------- scoring + selection
struct ScoreParams {
  const uint16_t* qq;   // [l_q, hq, d]
  const uint16_t* kc;   // [N, hkv, d] with kv_stride
  uint16_t* qp;         // [hkv, q_rows, d] packed score rows (workspace)
  float* scores;        // [hkv, N]
  float2* stats;        // [n_blocks, hkv, n_split, rows] (max in log2 units, sum)
  int32_t* sel;         // [n_blocks, hkv, l_pass]
  int64_t kv_stride;
  int32_t hq, hkv, group, l_query, rows;   // rows = group * l_query
  int32_t q_rows;                          // rows rounded up to a multiple of 128
  int32_t n_tokens, n_blocks, n_split, l_pass;
  int32_t v_begin, v_count;   // blocks scored and selected by one launch
  float scale_log2;
  int32_t bs[APBV_MAX_BLOCKS + 1];
};

constexpr int kScoreSplit = 2048;   // keys per row-statistics workgroup

// Scoring workspace: split statistics, packed score rows, then (when the caller passes no
// score buffer) the scores, each part 256-byte aligned.
struct ScoreWorkspace {
  size_t stats, qpack, scores, total;   // byte offsets of the parts, and the size
};
ScoreWorkspace score_workspace(int n_blocks, int hkv, int rows, int n_split, int n_tokens,
                               int head_dim, bool need_scores);
inline size_t score_workspace_bytes(int n_blocks, int hkv, int rows, int n_split,
                                    int n_tokens, int head_dim, bool need_scores) {
  return score_workspace(n_blocks, hkv, rows, n_split, n_tokens, head_dim, need_scores).total;
}
inline int score_q_rows(int rows) { return (rows + 127) / 128 * 128; }
// LDS of one column-sum workgroup (two staged query chunks and the rows' log-sum-exps)
size_t score_colsum_lds_bytes(int rows, int head_dim);
constexpr size_t kMaxLdsBytes = 160 * 1024;   // per workgroup on gfx950
hipError_t launch_score_select(const ScoreParams& p, int head_dim, int max_block,
                               hipStream_t stream);

// ---------------------------------------------------------------- gather
struct GatherParams {
  const uint16_t* ka;
  const uint16_t* va;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* sel;
  uint16_t* kpre;
  uint16_t* vpre;
  int32_t* sel_errors;   // count of sel entries outside their own block, or null
  int64_t kv_stride;
  int32_t hkv, l_anchor, l_pass, n_blocks, pre_rows, n_tokens;
  int32_t row_begin, row_count;   // prefix rows written by one launch
  int32_t bs[APBV_MAX_BLOCKS + 1];
};

hipError_t launch_gather(const GatherParams& p, int head_dim, hipStream_t stream);

}  // namespace apbv
