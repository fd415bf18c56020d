// Passing-block selection for gfx950: query-to-context scores and per-(block, KV head)
// top-l_p (APB-V technical summary on gist.science, Metodologia part 1, "Meccanismo di
// Attenzione Approssimata": every host keeps the key/value pairs that its query-to-context
// attention scores rank highest, and hands them on as its passing block).
//
// Score of key j of block v, KV head g (R = G * l_query score rows, row r = head g*G + r/l_q,
// query row r % l_q):
//     s[g, j] = sum_r softmax_{j' in block v}(scale * q_r . k_j')_j
// Three kernels, all with a fixed reduction order (results are bitwise reproducible):
//   1. row statistics: per (block, KV head, 128-row group, 2048-key split) a running offset
//      (at most kTau below the row max, log2 units) and the sum of exp2 relative to it;
//      S^T = K . Q^T on MFMA puts one row per lane.
//   2. column sums: per (block, KV head, 256-key tile) the split statistics are folded into
//      each row's log-sum-exp, S = Q . K^T is recomputed on MFMA (one key per lane) and the
//      probabilities are summed down the rows.
//   3. selection: per (block, KV head) an exact radix select of the l_p-th largest score on
//      order-preserving 32-bit keys (kept in LDS), then a stable compaction (ties to the
//      lower row) that writes the chosen rows in ascending order, placed by block-wide
//      prefix sums.
#include "apbv_device.h"
#include "apbv_internal.h"

namespace apbv {

namespace {

constexpr int kThreads = 256;
constexpr int kKeyTile = 64;        // keys per LDS tile in the row-statistics kernel
constexpr int kColKeys = 256;       // keys per column-sum workgroup (64 per wave)
constexpr int kQChunk = 64;         // query rows staged in LDS at a time (column sums)
constexpr float kTau = 8.0f;        // log2 headroom of the lazy row offset (row statistics)

// ------------------------------------------------------------------ 1. row statistics
template <int D>
__global__ __launch_bounds__(kThreads, 4) void score_rowstats(const ScoreParams p) {
  constexpr int NK = D / 16;
  constexpr int KSTR = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * kKeyTile * KSTR];

  const int n_rg = (p.rows + 127) / 128;
  int b = blockIdx.x;
  const int split = b % p.n_split; b /= p.n_split;
  const int rg = b % n_rg; b /= n_rg;
  const int g = b % p.hkv;
  const int v = p.v_begin + b / p.hkv;
  const int lo = p.bs[v], hi = p.bs[v + 1];
  const int k_begin = lo + split * kScoreSplit;
  if (k_begin >= hi) return;   // the combiner reads only splits that hold keys
  const int k_end = min(hi, k_begin + kScoreSplit);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int row = rg * 128 + wave * 32 + l32;
  bf16x8 qf[NK];
  {
    const bool ok = row < p.rows;
    const int h = g * p.group + (ok ? row / p.l_query : 0);
    const int qi = ok ? row % p.l_query : 0;
    const uint16_t* qrow = p.qq + ((int64_t)qi * p.hq + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      qf[ks] = as_bf16x8(ok ? load16(qrow + ks * 16) : u32x4{0, 0, 0, 0});
  }

  // K tiles: the next tile's rows are fetched into registers while the current one is
  // computed, then stored into the other LDS stage (one barrier per tile)
  constexpr int CPT = kKeyTile * D / 8 / kThreads;   // 16-byte chunks per thread per tile
  u32x4 pre[CPT];
  auto fetch = [&](int k0) {
    const int valid = min(kKeyTile, k_end - k0);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = threadIdx.x + c * kThreads;
      const int kr = idx / (D / 8), col = idx % (D / 8);
      pre[c] = kr < valid ? load16(p.kc + (int64_t)(k0 + kr) * p.kv_stride + g * D + col * 8)
                          : u32x4{0, 0, 0, 0};
    }
  };
  fetch(k_begin);
  int buf = 0;
  float m = -INFINITY, l = 0.f;   // raw-logit offset, sum of exp2((s - m) * c) over this lane's keys
  for (int k0 = k_begin; k0 < k_end; k0 += kKeyTile, buf ^= 1) {
    const int valid = min(kKeyTile, k_end - k0);
    uint16_t* sKb = sK + buf * kKeyTile * KSTR;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = threadIdx.x + c * kThreads;
      store16(sKb + (idx / (D / 8)) * KSTR + (idx % (D / 8)) * 8, pre[c]);
    }
    __syncthreads();
    if (k0 + kKeyTile < k_end) fetch(k0 + kKeyTile);
    f32x16 s[kKeyTile / 32];
#pragma unroll
    for (int n = 0; n < kKeyTile / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[n][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int n = 0; n < kKeyTile / 32; ++n) {
        const bf16x8 a = as_bf16x8(load16(sKb + (n * 32 + l32) * KSTR + ks * 16 + half * 8));
        s[n] = mfma32(a, qf[ks], s[n]);
      }
    if (valid < kKeyTile) {   // ragged last tile: keys past the split end drop out
#pragma unroll
      for (int n = 0; n < kKeyTile / 32; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = n * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          s[n][r] = kk >= valid ? -INFINITY : s[n][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < kKeyTile / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[n][r]);
    mx = fmaxf(mx, swap_half(mx));
    // lazy offset: raised only when the tile maximum exceeds it by more than kTau (log2
    // units), so every exponential stays <= 2^kTau; the first tile always raises it
    if ((mx - m) * p.scale_log2 > kTau) {
      l = m == -INFINITY ? 0.f : l * fast_exp2((m - mx) * p.scale_log2);
      m = mx;
    }
    const float mc = m * p.scale_log2;
#pragma unroll
    for (int n = 0; n < kKeyTile / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) l += fast_exp2(fmaf(s[n][r], p.scale_log2, -mc));
  }
  l += swap_half(l);
  if (half == 0 && row < p.rows) {
    const int64_t idx = (((int64_t)v * p.hkv + g) * p.n_split + split) * p.rows + row;
    p.stats[idx] = make_float2(m * p.scale_log2, l);
  }
}

// ------------------------------------------------------------------ 2. column sums
template <int D>
__global__ __launch_bounds__(kThreads, 3) void score_colsum(const ScoreParams p, int rows_pad) {
  constexpr int NK = D / 16;
  constexpr int QSTR = D + 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem);                   // [2][kQChunk][QSTR]
  float* sL = reinterpret_cast<float*>(smem + 2 * kQChunk * QSTR * 2); // [rows_pad] lse2

  const int n_kt = (gridDim.x / (p.v_count * p.hkv));
  int b = blockIdx.x;
  const int kt = b % n_kt; b /= n_kt;
  const int g = b % p.hkv;
  const int v = p.v_begin + b / p.hkv;
  const int lo = p.bs[v], hi = p.bs[v + 1];
  const int kbase = lo + kt * kColKeys;
  if (kbase >= hi) return;

  // row log-sum-exp (log2 units) from the split statistics, splits in order
  const int nsp = (hi - lo + kScoreSplit - 1) / kScoreSplit;
  const float2* st = p.stats + ((int64_t)v * p.hkv + g) * p.n_split * p.rows;
  for (int r = threadIdx.x; r < rows_pad; r += kThreads) {
    float out = INFINITY;   // padding rows contribute exp2(-inf) = 0
    if (r < p.rows) {
      float M = -INFINITY;
      for (int s = 0; s < nsp; ++s) M = fmaxf(M, st[(int64_t)s * p.rows + r].x);
      float L = 0.f;
      for (int s = 0; s < nsp; ++s) {
        const float2 ml = st[(int64_t)s * p.rows + r];
        L += ml.y * fast_exp2(ml.x - M);
      }
      out = M + fast_log2(L);
    }
    sL[r] = out;
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  // K^T fragments (B operand): lane holds key l32 of each of the wave's two 32-key groups
  bf16x8 kf[2][NK];
  int key[2];
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    key[kg] = kbase + wave * 64 + kg * 32 + l32;
    const bool ok = key[kg] < hi;
    const uint16_t* krow = p.kc + (int64_t)(ok ? key[kg] : lo) * p.kv_stride + g * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      kf[kg][ks] = as_bf16x8(ok ? load16(krow + ks * 16) : u32x4{0, 0, 0, 0});
  }

  // query-row chunks: the next chunk is fetched into registers while the current one is
  // used, then stored into the other LDS stage (one barrier per chunk)
  constexpr int CPT = kQChunk * D / 8 / kThreads;   // 16-byte chunks per thread per chunk
  u32x4 pre[CPT];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = threadIdx.x + c * kThreads;
      const int r = c0 + idx / (D / 8), cc = idx % (D / 8);
      u32x4 val = {0, 0, 0, 0};
      if (r < p.rows) {
        const int h = g * p.group + r / p.l_query, qi = r % p.l_query;
        val = load16(p.qq + ((int64_t)qi * p.hq + h) * D + cc * 8);
      }
      pre[c] = val;
    }
  };
  fetch(0);
  __syncthreads();   // the row statistics in sL are complete
  float col[2] = {0.f, 0.f};
  int buf = 0;
  for (int c0 = 0; c0 < p.rows; c0 += kQChunk, buf ^= 1) {
    uint16_t* sQb = sQ + buf * kQChunk * QSTR;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = threadIdx.x + c * kThreads;
      store16(sQb + (idx / (D / 8)) * QSTR + (idx % (D / 8)) * 8, pre[c]);
    }
    __syncthreads();
    if (c0 + kQChunk < p.rows) fetch(c0 + kQChunk);
    // one 32-row block: S = Q.K^T for the wave's two 32-key groups, probabilities summed
    // into the column totals (rows past the end have lse = +inf and add 0)
    auto row_block = [&](int rb) {
      bf16x8 af[NK];
#pragma unroll
      for (int ks = 0; ks < NK; ++ks)
        af[ks] = as_bf16x8(load16(sQb + (rb * 32 + l32) * QSTR + ks * 16 + half * 8));
      const int rbase = c0 + rb * 32 + 4 * half;
      float lse[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) lse[r] = sL[rbase + 8 * (r / 4) + (r % 4)];
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) s = mfma32(af[ks], kf[kg][ks], s);
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc += fast_exp2(fmaf(s[r], p.scale_log2, -lse[r]));
        col[kg] += acc;
      }
    };
    const int nrb = min(kQChunk, p.rows - c0 + 31) / 32;
    if (nrb == kQChunk / 32) {
      // a full chunk as one straight-line block, so the exponentials of one row block
      // overlap the MFMAs of the next
#pragma unroll
      for (int rb = 0; rb < kQChunk / 32; ++rb) row_block(rb);
    } else {
      for (int rb = 0; rb < nrb; ++rb) row_block(rb);
    }
  }
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    const float tot = col[kg] + swap_half(col[kg]);
    if (half == 0 && key[kg] < hi) p.scores[(int64_t)g * p.n_tokens + key[kg]] = tot;
  }
}

// ------------------------------------------------------------------ 3. top-l_p selection
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive prefix sum over the workgroup's threads in thread order (wsum: one word of LDS
// per wave).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(x);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();   // wsum is reused by the next scan
  return before + inc - x;
}

// One workgroup of 1024 threads per (block, KV head). The block's scores are turned once
// into order-preserving 32-bit keys, held in LDS when the block has at most kSelCache rows
// (otherwise re-read from the score buffer by every pass).
//  * Radix select, 8 bits per pass from the top, finds the exact l_pass-th largest key T and
//    how many keys equal to T are still needed. Each wave counts into its own histogram (less
//    atomic contention); wave 0 sums them and finds the digit with one suffix scan over its
//    lanes (lane l holds digits 4l .. 4l+3).
//  * Stable compaction in row order: thread t owns a contiguous run of rows. It counts its
//    keys above T and equal to T; an exclusive scan of the equal counts gives how many tied
//    rows come before its run (ties go to the lower rows), a second scan of the rows it
//    keeps gives its output position.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelCache = 16384;   // rows whose keys stay in LDS (64 KB)

template <bool CACHED>
__global__ __launch_bounds__(kSelThreads) void select_topk(const ScoreParams p) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t keys[CACHED ? kSelCache : 1];
  __shared__ uint32_t sh_prefix, sh_need;
  __shared__ uint32_t wsum[kSelWaves];

  const int v = p.v_begin + blockIdx.x / p.hkv, g = blockIdx.x % p.hkv;
  const int lo = p.bs[v], hi = p.bs[v + 1];
  const int L = hi - lo;
  const float* sc = p.scores + (int64_t)g * p.n_tokens + lo;
  int32_t* out = p.sel + ((int64_t)v * p.hkv + g) * p.l_pass;
  if (p.l_pass == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto key = [&](int j) -> uint32_t {   // key of row lo + j
    if constexpr (CACHED) return keys[j];
    else return order_key(sc[j]);
  };
  if constexpr (CACHED) {
    for (int j = tid; j < L; j += kSelThreads) keys[j] = order_key(sc[j]);
  }

  uint32_t prefix = 0, need = (uint32_t)p.l_pass;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int j = tid; j < L; j += kSelThreads) {
      const uint32_t k = key(j);
      if ((k & hmask) == (prefix & hmask)) atomicAdd(&hist[wave][(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t b[4], s = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        b[e] = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) b[e] += hist[w][4 * lane + e];
        s += b[e];
      }
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t above = __shfl(incl, 63) - incl;   // keys with a digit of a higher lane
      // exactly one lane holds the digit d with count(digit > d) < need <= count(digit >= d)
      if (above < need && need <= above + s) {
        uint32_t acc = above;
        int d = 4 * lane;
        for (int e = 3; e >= 0; --e) {
          d = 4 * lane + e;
          if (acc + b[e] >= need) break;
          acc += b[e];
        }
        sh_prefix = prefix | ((uint32_t)d << shift);
        sh_need = need - acc;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    need = sh_need;
  }

  const uint32_t T = prefix;
  const int run = (L + kSelThreads - 1) / kSelThreads;
  const int r0 = min(tid * run, L), r1 = min((tid + 1) * run, L);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = r0; j < r1; ++j) {
    const uint32_t k = key(j);
    n_gt += k > T;
    n_eq += k == T;
  }
  const uint32_t eq_before = block_excl_scan(n_eq, wsum);
  const uint32_t eq_take = eq_before >= need ? 0u : min(n_eq, need - eq_before);
  uint32_t pos = block_excl_scan(n_gt + eq_take, wsum);
  uint32_t eq_seen = 0;
  for (int j = r0; j < r1; ++j) {
    const uint32_t k = key(j);
    if (k > T) {
      out[pos++] = lo + j;
    } else if (k == T) {
      if (eq_seen < eq_take) out[pos++] = lo + j;
      ++eq_seen;
    }
  }
}

}  // namespace

size_t score_workspace_bytes(int n_blocks, int hkv, int rows, int n_split, int n_tokens,
                             bool need_scores) {
  size_t stats = (size_t)n_blocks * hkv * n_split * rows * sizeof(float2);
  stats = (stats + 255) & ~(size_t)255;
  const size_t sc = need_scores ? (size_t)hkv * n_tokens * sizeof(float) : 0;
  return stats + sc;
}

size_t score_colsum_lds_bytes(int rows, int head_dim) {
  const int rows_pad = ((rows + kQChunk - 1) / kQChunk) * kQChunk;
  return 2 * (size_t)kQChunk * (head_dim + 8) * 2 + (size_t)(rows_pad > 0 ? rows_pad : 1) * 4;
}

hipError_t launch_score_select(const ScoreParams& p, int head_dim, int max_block,
                               hipStream_t stream) {
  if (p.v_count <= 0) return hipSuccess;
  const int n_rg = (p.rows + 127) / 128;
  if (p.rows > 0) {
    dim3 grid(p.v_count * p.hkv * n_rg * p.n_split);
    if (head_dim == 128)
      hipLaunchKernelGGL(score_rowstats<128>, grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(score_rowstats<64>, grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kt = (max_block + kColKeys - 1) / kColKeys;
    const int rows_pad = ((p.rows + kQChunk - 1) / kQChunk) * kQChunk;
    const size_t shm = score_colsum_lds_bytes(p.rows, head_dim);
    dim3 grid(p.v_count * p.hkv * n_kt);
    if (head_dim == 128)
      hipLaunchKernelGGL(score_colsum<128>, grid, dim3(kThreads), shm, stream, p, rows_pad);
    else
      hipLaunchKernelGGL(score_colsum<64>, grid, dim3(kThreads), shm, stream, p, rows_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.l_pass > 0) {
    if (max_block <= kSelCache)
      hipLaunchKernelGGL(select_topk<true>, dim3(p.v_count * p.hkv), dim3(kSelThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL(select_topk<false>, dim3(p.v_count * p.hkv), dim3(kSelThreads), 0,
                         stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace apbv
