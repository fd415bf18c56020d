// Approximate-attention prefill kernel for gfx950 (bf16 MFMA, fp32 online softmax).
//
// Row i of context block v (head h, KV head g = h / G) attends to
//   the prefix k_pre[g, 0 : l_anchor + v*l_pass]   (anchor + passing blocks of blocks < v)
//   then its own block's keys bs[v] .. i           (causal, diagonal included)
// (APB-V technical summary on gist.science, Metodologia part 1, "Meccanismo di Attenzione
// Approssimata"; with one block and no prefix this is plain causal flash attention, as the
// page's "Limitazioni" paragraph notes).
//
// Design (default variant: one workgroup = 8 waves = one query tile of 256 rows of one head,
// 32 rows per wave, two waves per SIMD so one wave's softmax overlaps the other's MFMAs):
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: the K tile (shared by the waves) is the A
//    operand read from LDS, the wave's Q rows are the B operand held in registers. The
//    result puts one query row per lane (lanes l and l+32 share a row and split its keys),
//    so row max / sum are lane-local plus one permlane32 swap.
//  * O^T = V^T . P^T: the probabilities are already laid out as the B operand; the V^T
//    operand comes straight from a row-major V tile through ds_read_b64_tr_b16 (two
//    transposing 8-byte reads per operand), so the rescale factor of a row is lane-local.
//  * K and V tiles of 64 keys go global -> LDS with global_load_lds_dwordx4 (no register
//    staging) into padded rows (K: +16 B, V: +32 B), which keeps the 128-bit operand reads
//    and the transposing reads near the LDS peak while every LDS read address is a per-lane
//    base plus a compile-time offset; double-buffered, the next tile's loads in flight
//    while the current one is computed, one barrier per tile.
//  * Online softmax in log2 units with a lazy rescale: the running offset is only raised
//    when a tile's maximum exceeds it by more than 8 (probabilities stay <= 256), which is
//    exact up to rounding and skips almost every O rescale. Masking code runs only on
//    tiles that need it (ragged prefix end, causal diagonal).
//  * Grid = work units x heads, remapped so each XCD gets a contiguous range: the heads of
//    one KV group and one unit run side by side on the same XCD and share K/V in its L2.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "apbv_device.h"
#include "apbv_internal.h"

namespace apbv {

namespace {

constexpr float kLazyTau = 8.0f;   // log2 headroom before the running offset is raised

typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Shape of one kernel variant: NW waves, 32*RB query rows per wave, KT = 64 keys per tile.
// One LDS stage holds the K tile (rows padded to D+8 elements) followed by the V tile
// (rows padded to D+16 elements). Both are filled by global->LDS loads of 1 KB per wave
// (64 lanes x 16 B); the padding keeps the MFMA operand reads bank-conflict free while
// every LDS read is a per-lane base plus a compile-time offset.
template <int D, int NW, int RB, int KT>
struct Shape {
  static_assert(KT == 64, "the padded tile layout assumes 64-key tiles");
  static constexpr int M = NW * 32 * RB;           // query rows per tile
  static constexpr int KSTR = D + 8;               // K row stride (elements)
  static constexpr int VSTR = D + 16;              // V row stride (elements)
  static constexpr int KSLOT = KSTR / 8;           // 16-byte slots per K row
  static constexpr int VSLOT = VSTR / 8;
  static constexpr int SEGK = KT * KSLOT / 64;     // 1 KB segments of the K tile
  static constexpr int SEGV = KT * VSLOT / 64;
  static constexpr int SEG = SEGK + SEGV;
  static constexpr int LOADS = (SEG + NW - 1) / NW;  // load slots per lane per tile
  static constexpr int STAGE = SEG * 512;          // elements per LDS stage
  static constexpr int VOFF = SEGK * 512;          // V tile offset inside a stage
};

// Source of one key tile: K and V of its first row, row stride, valid rows (>= 1).
struct KeySrc {
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;
  int valid;
};

// Per-lane (row, column) of each load slot; padding slots repeat column 0 of their row.
template <int D, int NW, int RB, int KT>
struct LoadMap {
  int row[Shape<D, NW, RB, KT>::LOADS];
  int col[Shape<D, NW, RB, KT>::LOADS];
  __device__ __forceinline__ void init() {
    using S = Shape<D, NW, RB, KT>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < S::LOADS; ++j) {
      const int seg = j * NW + wave;
      const bool is_v = seg >= S::SEGK;
      const int slots = is_v ? S::VSLOT : S::KSLOT;
      const int q = (is_v ? seg - S::SEGK : seg) * 64 + lane;
      const int c = q % slots;
      row[j] = min(q / slots, KT - 1);
      col[j] = c < D / 8 ? c * 8 : 0;
    }
  }
};

// K and V tile -> one LDS stage, no registers involved. Rows past `valid` repeat the last
// valid row; those keys are masked in the scores, so their values only need to be finite.
template <int D, int NW, int RB, int KT>
__device__ __forceinline__ void load_tile(uint16_t* stage, const LoadMap<D, NW, RB, KT>& lm,
                                          const KeySrc& src) {
  using S = Shape<D, NW, RB, KT>;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < S::LOADS; ++j) {
    const int seg = j * NW + wave;
    if (seg < S::SEG) {
      const bool is_v = seg >= S::SEGK;
      const int off = min(lm.row[j], src.valid - 1) * (int)src.stride + lm.col[j];
      __builtin_amdgcn_global_load_lds((is_v ? src.v : src.k) + off, stage + seg * 512, 16, 0, 0);
    }
  }
}

// One key tile for one wave: S^T = K.Q^T, (masked) online softmax, O^T += V^T.P^T.
template <int D, int NW, int RB, int KT, bool MASK>
__device__ __forceinline__ void attend_tile(const uint16_t* stage, const bf16x8 (&qf)[RB][D / 16],
                                            f32x16 (&o)[RB][D / 32], float (&m_run)[RB],
                                            float (&l_run)[RB], float scale_log2, bool prefix,
                                            int key0, int valid, int wrow0) {
  using S = Shape<D, NW, RB, KT>;
  constexpr int ND = D / 32, NK = D / 16, NN = KT / 32;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const f32x16 zero = {};

  // S^T[key, row] for NN blocks of 32 keys; A = K rows from LDS, B = Q^T from registers
  const uint16_t* kbase = stage + l32 * S::KSTR + half * 8;
  f32x16 s[RB][NN];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const bf16x8 a = as_bf16x8(load16(kbase + n * 32 * S::KSTR + ks * 16));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        s[rb][n] = mfma32(a, qf[rb][ks], ks == 0 ? zero : s[rb][n]);
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (MASK) {
      const int row = wrow0 + rb * 32 + l32;
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = n * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          const bool dead = prefix ? (kk >= valid) : (key0 + kk > row);
          s[rb][n][r] = dead ? -INFINITY : s[rb][n][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < NN; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][n][r]);
    mx = fmaxf(mx, swap_half(mx));
    const float mxs = mx * scale_log2;
    if (mxs > m_run[rb] + kLazyTau) {
      if (m_run[rb] != -INFINITY) {     // the first visible tile needs no rescale (O = 0)
        const float alpha = fast_exp2(m_run[rb] - mxs);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
      }
      m_run[rb] = mxs;
    }
    const float mu = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
    float ls = 0.f;
#pragma unroll
    for (int n = 0; n < NN; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(s[rb][n][r], scale_log2, -mu));
        ls += e;
        s[rb][n][r] = e;
      }
    l_run[rb] += ls;
  }

  // O^T += V^T . P^T, 16 keys per MFMA. P^T element e of chunk c (lane half h) is key
  // 16c + 8(e/4) + 4h + e%4 (the S^T register order); the V^T operand is fetched with two
  // transposing reads: source lane j of each 16-lane group points at key row
  // 16c + 8t + 4h + j/4 and d columns 32db + 16*(group % 2) + 4*(j % 4) .. +3.
  const int grp = (lane >> 4) & 1, j16 = lane & 15;
  const uint16_t* vbase = stage + S::VOFF + (4 * half + (j16 >> 2)) * S::VSTR + 16 * grp + 4 * (j16 & 3);
#pragma unroll
  for (int c = 0; c < KT / 16; ++c) {
    bf16x8 pf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x16& sv = s[rb][c / 2];
      const int b0 = (c % 2) * 8;
      u32x4 w = {pack_bf16x2(sv[b0 + 0], sv[b0 + 1]), pack_bf16x2(sv[b0 + 2], sv[b0 + 3]),
                 pack_bf16x2(sv[b0 + 4], sv[b0 + 5]), pack_bf16x2(sv[b0 + 6], sv[b0 + 7])};
      pf[rb] = as_bf16x8(w);
    }
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const uint16_t* src = vbase + 16 * c * S::VSTR + 32 * db;
      const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
      const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 8 * S::VSTR));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 both = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      const bf16x8 va = __builtin_bit_cast(bf16x8, both);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma32(va, pf[rb], o[rb][db]);
    }
  }
}

template <int D, int NW, int RB, int KT>
__device__ __forceinline__ void process_tile(const AttnParams& p, int h, int g, int v, int t,
                                             uint16_t* lds, const LoadMap<D, NW, RB, KT>& lm) {
  using S = Shape<D, NW, RB, KT>;
  constexpr int M = S::M;
  constexpr int ND = D / 32;     // 32-wide d blocks of O^T
  constexpr int NK = D / 16;     // 16-deep k steps of S^T

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int lo = p.sched.bs[v], hi = p.sched.bs[v + 1];
  const int r0 = lo + t * M;
  const int r1 = min(r0 + M, hi);
  const int wrow0 = r0 + wave * 32 * RB;   // first row of this wave

  // Q^T fragments (B operand): lane holds row l32 of each row block, d = 16ks + 8half + e.
  // Rows past the tile end repeat a valid row; their outputs are never stored.
  bf16x8 qf[RB][NK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = min(wrow0 + rb * 32 + l32, r1 - 1);
    const uint16_t* qrow = p.q + (int64_t)row * p.q_stride + h * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) qf[rb][ks] = as_bf16x8(load16(qrow + ks * 16));
  }

  f32x16 o[RB][ND];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.f;
  }

  const int P = p.l_anchor + v * p.l_pass;
  const int n_pre = (P + KT - 1) / KT;
  const int n_loc = (r1 - lo + KT - 1) / KT;
  const int ntiles = n_pre + n_loc;

  auto source = [&](int i) -> KeySrc {
    KeySrc s;
    if (i < n_pre) {
      const int key0 = i * KT;
      const int64_t off = ((int64_t)g * p.pre_rows + key0) * D;
      s.k = p.kpre + off;
      s.v = p.vpre + off;
      s.stride = D;
      s.valid = min(KT, P - key0);
    } else {
      const int key0 = lo + (i - n_pre) * KT;
      const int64_t off = (int64_t)key0 * p.kv_stride + g * D;
      s.k = p.kc + off;
      s.v = p.vc + off;
      s.stride = p.kv_stride;
      s.valid = min(KT, r1 - key0);
    }
    return s;
  };

  load_tile<D, NW, RB, KT>(lds, lm, source(0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    const int buf = i & 1;
    if (i + 1 < ntiles) load_tile<D, NW, RB, KT>(lds + (buf ^ 1) * S::STAGE, lm, source(i + 1));
    const uint16_t* stage = lds + buf * S::STAGE;
    const bool prefix = i < n_pre;
    const int key0 = prefix ? i * KT : lo + (i - n_pre) * KT;
    const int valid = prefix ? min(KT, P - key0) : min(KT, r1 - key0);
    // a local tile entirely in the future of every row of this wave adds nothing
    const bool skip = !prefix && key0 > wrow0 + 32 * RB - 1;
    if (!skip) {
      const bool need_mask = prefix ? (valid < KT) : (key0 + KT - 1 > wrow0);
      if (need_mask)
        attend_tile<D, NW, RB, KT, true>(stage, qf, o, m_run, l_run, p.scale_log2, prefix, key0,
                                         valid, wrow0);
      else
        attend_tile<D, NW, RB, KT, false>(stage, qf, o, m_run, l_run, p.scale_log2, prefix, key0,
                                          valid, wrow0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // epilogue: O = O^T / l, bf16; lse = (m + log2 l) * ln 2
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lt = l_run[rb] + swap_half(l_run[rb]);
    const int row = wrow0 + rb * 32 + l32;
    if (row < r1) {
      const float inv = 1.0f / lt;
      uint16_t* orow = p.out + ((int64_t)row * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = db * 32 + 8 * q4 + 4 * half;
          const f32x16& ov = o[rb][db];
          u32x2 w = {pack_bf16x2(ov[4 * q4 + 0] * inv, ov[4 * q4 + 1] * inv),
                     pack_bf16x2(ov[4 * q4 + 2] * inv, ov[4 * q4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      if (p.lse != nullptr && half == 0)
        p.lse[(int64_t)h * p.n_tokens + row] = (m_run[rb] + fast_log2(lt)) * 0.69314718055994531f;
    }
  }
}

template <int D, int NW, int RB, int KT>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * Shape<D, NW, RB, KT>::STAGE];
  LoadMap<D, NW, RB, KT> lm;
  lm.init();
  const uint32_t total = (uint32_t)p.n_units * (uint32_t)p.hq;
  const uint32_t L = xcd_contiguous(blockIdx.x, total);
  const int unit = p.unit_begin + (int)(L / p.hq);
  const int h = (int)(L % p.hq);
  const int g = h / p.group;
  int va, ta, vb, tb;
  p.sched.decode(unit, va, ta, vb, tb);
  // one code path for both parts of a unit (keeps the kernel small for the instruction cache)
  for (int part = 0; part < 2; ++part) {
    const int v = part == 0 ? va : vb;
    const int t = part == 0 ? ta : tb;
    if (v >= 0) process_tile<D, NW, RB, KT>(p, h, g, v, t, lds, lm);
  }
}

// Kernel variant: NW waves per workgroup, 32*RB rows per wave, KT keys per tile.
// APBV_ATTN_CFG = "NWxRBxKT" ("8x1x64", "4x1x64", "4x2x64") overrides the default for
// tuning runs.
struct Cfg {
  int nw, rb, kt;
};
Cfg config() {
  static const Cfg c = [] {
    const Cfg def = {8, 1, 64};
    const char* e = getenv("APBV_ATTN_CFG");
    if (e == nullptr) return def;
    const Cfg known[] = {{4, 2, 64}, {4, 1, 64}, {8, 1, 64}};
    for (const Cfg& k : known) {
      char buf[16];
      snprintf(buf, sizeof(buf), "%dx%dx%d", k.nw, k.rb, k.kt);
      if (strcmp(buf, e) == 0) return k;
    }
    return def;
  }();
  return c;
}

template <int D, int NW, int RB, int KT>
void launch_one(const AttnParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_kernel<D, NW, RB, KT>), grid, dim3(NW * 64), 0, stream, p);
}

template <int D>
hipError_t launch_d(const AttnParams& p, dim3 grid, hipStream_t stream) {
  const Cfg c = config();
  if (c.nw == 4 && c.rb == 2) launch_one<D, 4, 2, 64>(p, grid, stream);
  else if (c.nw == 4) launch_one<D, 4, 1, 64>(p, grid, stream);
  else launch_one<D, 8, 1, 64>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace

int attn_tile_rows(int head_dim) {
  const Cfg c = config();
  return (head_dim == 64 || head_dim == 128) ? c.nw * 32 * c.rb : 0;
}

hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream) {
  const uint64_t total = (uint64_t)p.n_units * (uint64_t)p.hq;
  if (total == 0) return hipSuccess;
  if (p.sched.tile_rows != attn_tile_rows(head_dim)) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)total);
  return head_dim == 128 ? launch_d<128>(p, grid, stream) : launch_d<64>(p, grid, stream);
}

}  // namespace apbv
