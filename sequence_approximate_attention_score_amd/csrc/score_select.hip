// Passing-block selection for gfx950: query-to-context scores and per-(block, KV head)
// top-l_p (APB-V technical summary on gist.science, Metodologia part 1, "Meccanismo di
// Attenzione Approssimata": every host keeps the key/value pairs that its query-to-context
// attention scores rank highest, and hands them on as its passing block).
//
// Score of key j of block v, KV head g (R = G * l_query score rows, row r = head g*G + r/l_q,
// query row r % l_q):
//     s[g, j] = sum_r softmax_{j' in block v}(scale * q_r . k_j')_j
// Four kernels, all with a fixed reduction order (results are bitwise reproducible):
//   0. packing: the score rows of every KV head are laid out contiguously in the workspace,
//      [hkv][q_rows][d] with zero rows up to a multiple of 128, so both passes below fill
//      their LDS tiles with buffer loads straight into LDS at fixed per-lane offsets;
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

// A 64-row tile of d-element bf16 rows in LDS, rows padded to d + 8 elements (16 B) so that
// the MFMA operand reads are free of bank conflicts. It is filled in 1 KB segments (64
// lanes x 16 B, written in lane order): segment s by wave s % 4 of the workgroup; the
// padding slot of a row repeats the row's first 16 bytes.
template <int D>
struct Tile {
  static constexpr int STR = D + 8;            // elements per LDS row
  static constexpr int SLOT = STR / 8;         // 16-byte slots per LDS row
  static constexpr int SEGS = SLOT;            // 64 rows x SLOT slots / 64 lanes
  static constexpr int ELEMS = SEGS * 512;     // = 64 * STR
  static constexpr int LOADS = (SEGS + 3) / 4; // segments per wave
};

typedef __attribute__((address_space(3))) void lds_void;

// Byte offsets of this lane's load slots inside a tile whose rows are row_bytes apart
// (row_bytes < 2^24: a K/V row stride is below 2^23 bytes, a packed row is 2d bytes).
template <int D>
struct TileLoader {
  int off[Tile<D>::LOADS];
  int wave;   // uniform
  __device__ __forceinline__ void init(unsigned row_bytes) {
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < Tile<D>::LOADS; ++j) {
      const int q = (j * 4 + wave) * 64 + lane;
      const int r = q / Tile<D>::SLOT, c = q % Tile<D>::SLOT;
      off[j] = (int)__umul24((unsigned)r, row_bytes) + (c < D / 8 ? c * 16 : 0);
    }
  }
  // The tile's rows start at `base`; bytes at or past `bytes` from it read as zero (the
  // buffer's record count), so rows past the end of the data are never fetched.
  __device__ __forceinline__ void load(uint16_t* dst, const uint16_t* base, unsigned bytes) const {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, (int)bytes, 0x00020000);
#pragma unroll
    for (int j = 0; j < Tile<D>::LOADS; ++j) {
      const int seg = j * 4 + wave;
      const int o = off[j];   // (a member passed straight to the builtin loses the host stub)
      if (seg < Tile<D>::SEGS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + seg * 512), 16, o, 0, 0,
                                                 0);
    }
  }
};

// ------------------------------------------------------------------ 0. packed score rows
// Packed row r of KV head g is query row r % l_q of head g*G + r / l_q; rows r >= G*l_q of
// the padding are zero. One thread per 16 bytes.
template <int D>
__global__ __launch_bounds__(kThreads) void score_pack_q(const ScoreParams p) {
  constexpr int CPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (int64_t)p.hkv * p.q_rows * CPR) return;
  const int c = (int)(t % CPR);
  const int64_t gr = t / CPR;
  const int r = (int)(gr % p.q_rows), g = (int)(gr / p.q_rows);
  u32x4 val = {0, 0, 0, 0};
  if (r < p.rows) {
    const int h = g * p.group + r / p.l_query, qi = r % p.l_query;
    val = load16(p.qq + ((int64_t)qi * p.hq + h) * D + c * 8);
  }
  store16(p.qp + gr * D + c * 8, val);
}

// ------------------------------------------------------------------ 1. row statistics
template <int D>
__global__ __launch_bounds__(kThreads, 4) void score_rowstats(const ScoreParams p) {
  using T = Tile<D>;
  constexpr int NK = D / 16;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[T::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t K1[T::ELEMS];

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
  const int row = rg * 128 + wave * 32 + l32;   // below q_rows (a multiple of 128)
  bf16x8 qf[NK];
  {
    const uint16_t* qrow = p.qp + ((int64_t)g * p.q_rows + row) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) qf[ks] = as_bf16x8(load16(qrow + ks * 16));
  }

  const unsigned stride_b = (unsigned)p.kv_stride * 2u;
  TileLoader<D> ld;
  ld.init(stride_b);
  auto load = [&](uint16_t* dst, int k0) {
    ld.load(dst, p.kc + (int64_t)k0 * p.kv_stride + g * D,
            (unsigned)min(kKeyTile, k_end - k0) * stride_b);
  };
  int kofs = l32 * T::STR + half * 8;
  // an opaque lane offset keeps every LDS read "array + offset", so the reads of one
  // buffer carry that array's alias information past the loads into the other
  asm volatile("" : "+v"(kofs));

  float m = -INFINITY, l = 0.f;   // raw-logit offset, sum of exp2((s - m) * c) over this lane's keys
  auto tile = [&](const uint16_t* kb, int k0) {
    const int valid = min(kKeyTile, k_end - k0);
    f32x16 s[kKeyTile / 32];
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int n = 0; n < kKeyTile / 32; ++n) {
        const bf16x8 a = as_bf16x8(load16(kb + kofs + n * 32 * T::STR + ks * 16));
        s[n] = mfma32(a, qf[ks], ks == 0 ? zero : s[n]);
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
  };

  // two LDS stages: tile i+1 is loaded while tile i is computed, one barrier per tile
  load(K0, k_begin);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int k0 = k_begin; k0 < k_end; k0 += 2 * kKeyTile) {
    if (k0 + kKeyTile < k_end) load(K1, k0 + kKeyTile);
    tile(K0, k0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (k0 + kKeyTile >= k_end) break;
    if (k0 + 2 * kKeyTile < k_end) load(K0, k0 + 2 * kKeyTile);
    tile(K1, k0 + kKeyTile);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
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
  using T = Tile<D>;
  constexpr int NK = D / 16;
  __shared__ __attribute__((aligned(1024))) uint16_t Q0[T::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t Q1[T::ELEMS];
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sL = reinterpret_cast<float*>(smem);   // [rows_pad] row lse (log2 units)

  const int n_kt = (gridDim.x / (p.v_count * p.hkv));
  int b = blockIdx.x;
  const int kt = b % n_kt; b /= n_kt;
  const int g = b % p.hkv;
  const int v = p.v_begin + b / p.hkv;
  const int lo = p.bs[v], hi = p.bs[v + 1];
  const int kbase = lo + kt * kColKeys;
  if (kbase >= hi) return;

  // packed query-row chunks: chunk c0 is rows c0 .. c0+63 of this KV head's packed rows
  TileLoader<D> ld;
  ld.init(D * 2);
  const uint16_t* qg = p.qp + (int64_t)g * p.q_rows * D;
  auto load = [&](uint16_t* dst, int c0) {
    ld.load(dst, qg + (int64_t)c0 * D, (unsigned)(p.q_rows - c0) * (D * 2));
  };
  if (p.rows > 0) load(Q0, 0);

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
  int qofs = l32 * T::STR + half * 8;
  asm volatile("" : "+v"(qofs));   // keeps each chunk read "array + offset" (see row statistics)

  float col[2] = {0.f, 0.f};
  // one 32-row block: S = Q.K^T for the wave's two 32-key groups, probabilities summed
  // into the column totals (rows past the end have lse = +inf and add 0)
  auto row_block = [&](const uint16_t* qb, int c0, int rb) {
    bf16x8 af[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      af[ks] = as_bf16x8(load16(qb + qofs + rb * 32 * T::STR + ks * 16));
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
  auto chunk = [&](const uint16_t* qb, int c0) {
    const int nrb = min(kQChunk, p.rows - c0 + 31) / 32;
    if (nrb == kQChunk / 32) {
      // a full chunk as one straight-line block, so the exponentials of one row block
      // overlap the MFMAs of the next
#pragma unroll
      for (int rb = 0; rb < kQChunk / 32; ++rb) row_block(qb, c0, rb);
    } else {
      for (int rb = 0; rb < nrb; ++rb) row_block(qb, c0, rb);
    }
  };

  // two LDS stages: chunk i+1 is loaded while chunk i is used, one barrier per chunk (the
  // first barrier also publishes the row log-sum-exps)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c0 = 0; c0 < p.rows; c0 += 2 * kQChunk) {
    if (c0 + kQChunk < p.rows) load(Q1, c0 + kQChunk);
    chunk(Q0, c0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c0 + kQChunk >= p.rows) break;
    if (c0 + 2 * kQChunk < p.rows) load(Q0, c0 + 2 * kQChunk);
    chunk(Q1, c0 + kQChunk);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
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

ScoreWorkspace score_workspace(int n_blocks, int hkv, int rows, int n_split, int n_tokens,
                               int head_dim, bool need_scores) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  ScoreWorkspace w;
  w.stats = 0;
  w.qpack = up((size_t)n_blocks * hkv * n_split * rows * sizeof(float2));
  w.scores = w.qpack + up((size_t)hkv * score_q_rows(rows) * head_dim * 2);
  w.total = w.scores + (need_scores ? (size_t)hkv * n_tokens * sizeof(float) : 0);
  return w;
}

size_t score_colsum_lds_bytes(int rows, int head_dim) {
  const int rows_pad = ((rows + kQChunk - 1) / kQChunk) * kQChunk;
  return 2 * (size_t)kQChunk * (head_dim + 8) * 2 + (size_t)(rows_pad > 0 ? rows_pad : 1) * 4;
}

hipError_t launch_score_select(const ScoreParams& p, int head_dim, int max_block,
                               hipStream_t stream) {
  if (p.v_count <= 0) return hipSuccess;
  const int n_rg = (p.rows + 127) / 128;
  // the packed rows are written by the launch that starts at block 0 (a launch over later
  // blocks is ordered after it)
  if (p.rows > 0 && p.v_begin == 0) {
    const int64_t n = (int64_t)p.hkv * p.q_rows * (head_dim / 8);
    dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    if (head_dim == 128)
      hipLaunchKernelGGL(score_pack_q<128>, grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(score_pack_q<64>, grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
    const size_t shm = (size_t)(rows_pad > 0 ? rows_pad : 1) * 4;   // the row lse
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
