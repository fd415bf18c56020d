// Approximate-attention prefill kernel for gfx950 (bf16 MFMA, fp32 online softmax).
//
// Row i of context block v (head h, KV head g = h / G) attends to
//   the prefix k_pre[g, 0 : l_anchor + v*l_pass]   (anchor + passing blocks of blocks < v)
//   then its own block's keys bs[v] .. i           (causal, diagonal included)
// (APB-V technical summary on gist.science, Metodologia part 1, "Meccanismo di Attenzione
// Approssimata"; with one block and no prefix this is plain causal flash attention, as the
// page's "Limitazioni" paragraph notes).
//
// Design (one workgroup = 4 waves = one query tile of 128*RB rows of one head):
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: the K tile (shared by the waves) is the A
//    operand read from LDS, the wave's Q rows are the B operand held in registers. The
//    result puts one query row per lane (lanes l and l+32 share a row and split its keys),
//    so row max / sum are lane-local plus one permlane32 swap.
//  * O^T = V^T . P^T: the probabilities are already laid out as the B operand; V is stored
//    transposed in LDS (key positions permuted to match the S^T register order), so the
//    rescale factor of a row is lane-local too.
//  * Online softmax in log2 units with a lazy rescale: the running offset is only raised
//    when a tile's maximum exceeds it by more than 8 (probabilities stay <= 256), which is
//    exact up to rounding and skips almost every O rescale.
//  * K/V tiles of 64 keys are double-buffered in LDS; the next tile's global loads are in
//    flight while the current one is computed; one barrier per tile.
//  * Grid = work units x heads, remapped so each XCD gets a contiguous range: the heads of
//    one KV group and one unit run side by side on the same XCD and share K/V in its L2.
#include "apbv_device.h"
#include "apbv_internal.h"

namespace apbv {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int KT = 64;             // keys per tile
constexpr float kLazyTau = 8.0f;   // log2 headroom before the running offset is raised

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;    // K tile row stride (bf16 elements, +16 B pad)
  static constexpr int VSTR = KT + 8;   // V^T tile row stride
  static constexpr int KCH = KT * D / 8 / kThreads;          // 16-B K chunks per thread
  static constexpr int VIT = (KT / 4) * (D / 8);             // 4-key x 8-d V items
  static constexpr int VPT = (VIT + kThreads - 1) / kThreads;  // V items per thread
};

// Source of one key tile: base row pointer for K and V, row stride, first key, valid rows.
struct KeySrc {
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;
  int valid;
};

template <int D>
struct Stage {
  u32x4 k[Tile<D>::KCH];
  u32x4 v[Tile<D>::VPT][4];
};

template <int D>
__device__ __forceinline__ void stage_load(Stage<D>& st, const KeySrc& src) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < Tile<D>::KCH; ++j) {
    const int c = tid + j * kThreads;
    const int row = c / (D / 8), col = c % (D / 8);
    st.k[j] = row < src.valid ? load16(src.k + row * src.stride + col * 8) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < Tile<D>::VPT; ++j) {
    const int it = tid + j * kThreads;
    const int kg = it / (D / 8), dg = it % (D / 8);
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int row = kg * 4 + y;
      st.v[j][y] = (it < Tile<D>::VIT && row < src.valid)
                       ? load16(src.v + row * src.stride + dg * 8)
                       : u32x4{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D>& st, uint16_t* sK, uint16_t* sV) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < Tile<D>::KCH; ++j) {
    const int c = tid + j * kThreads;
    const int row = c / (D / 8), col = c % (D / 8);
    store16(sK + row * Tile<D>::KSTR + col * 8, st.k[j]);
  }
#pragma unroll
  for (int j = 0; j < Tile<D>::VPT; ++j) {
    const int it = tid + j * kThreads;
    if (it < Tile<D>::VIT) {
      const int kg = it / (D / 8), dg = it % (D / 8);
      // keys 4kg..4kg+3 = 16c + 8x + 4b + y sit at V^T positions 16c + 8b + 4x + y
      const int pos = 16 * (kg / 4) + 8 * (kg % 2) + 4 * ((kg / 2) % 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo01 = __builtin_amdgcn_perm(st.v[j][1][w], st.v[j][0][w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(st.v[j][3][w], st.v[j][2][w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(st.v[j][1][w], st.v[j][0][w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(st.v[j][3][w], st.v[j][2][w], 0x07060302u);
        const int d = dg * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(sV + d * Tile<D>::VSTR + pos) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(sV + (d + 1) * Tile<D>::VSTR + pos) = u32x2{hi01, hi23};
      }
    }
  }
}

template <int D, int RB>
__device__ void process_tile(const AttnParams& p, int h, int g, int v, int t, uint16_t* sKbase,
                             uint16_t* sVbase) {
  constexpr int M = kWaves * 32 * RB;
  constexpr int ND = D / 32;     // 32-wide d blocks of O^T
  constexpr int NK = D / 16;     // 16-deep k steps of S^T
  constexpr int KSZ = KT * Tile<D>::KSTR;
  constexpr int VSZ = D * Tile<D>::VSTR;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int lo = p.sched.bs[v], hi = p.sched.bs[v + 1];
  const int r0 = lo + t * M;
  const int r1 = min(r0 + M, hi);
  const int wrow0 = r0 + wave * 32 * RB;   // first row of this wave

  // Q^T fragments (B operand): lane holds row l32 of each row block, d = 16ks + 8half + e
  bf16x8 qf[RB][NK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wrow0 + rb * 32 + l32;
    const uint16_t* qrow = p.q + (int64_t)row * p.q_stride + h * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      qf[rb][ks] = as_bf16x8(row < r1 ? load16(qrow + ks * 16) : u32x4{0, 0, 0, 0});
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

  Stage<D> st;
  stage_load<D>(st, source(0));
  stage_store<D>(st, sKbase, sVbase);
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    const int buf = i & 1;
    if (i + 1 < ntiles) stage_load<D>(st, source(i + 1));

    const uint16_t* sK = sKbase + buf * KSZ;
    const uint16_t* sV = sVbase + buf * VSZ;
    const bool prefix = i < n_pre;
    const int key0 = prefix ? i * KT : lo + (i - n_pre) * KT;
    const int valid = prefix ? min(KT, P - key0) : min(KT, r1 - key0);
    // whole tile in the future of every row of this wave: nothing to add
    const bool skip = !prefix && key0 > wrow0 + 32 * RB - 1;
    if (!skip) {
      f32x16 s[RB][KT / 32];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int n = 0; n < KT / 32; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[rb][n][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
        for (int n = 0; n < KT / 32; ++n) {
          const bf16x8 a = as_bf16x8(load16(sK + (n * 32 + l32) * Tile<D>::KSTR + ks * 16 + half * 8));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[rb][n] = mfma32(a, qf[rb][ks], s[rb][n]);
        }
      }

      const bool need_mask = prefix ? (valid < KT) : (key0 + KT - 1 > wrow0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (need_mask) {
          const int row = wrow0 + rb * 32 + l32;
#pragma unroll
          for (int n = 0; n < KT / 32; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kk = n * 32 + 8 * (r / 4) + 4 * half + (r % 4);
              const bool dead = prefix ? (kk >= valid) : (key0 + kk > row);
              if (dead) s[rb][n][r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int n = 0; n < KT / 32; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][n][r]);
        mx = fmaxf(mx, swap_half(mx));
        const float mxs = mx * p.scale_log2;
        if (mxs > m_run[rb] + kLazyTau) {
          const float alpha = fast_exp2(m_run[rb] - mxs);
          m_run[rb] = mxs;
          l_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
        }
        const float mu = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
        float ls = 0.f;
#pragma unroll
        for (int n = 0; n < KT / 32; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(s[rb][n][r], p.scale_log2, -mu));
            ls += e;
            s[rb][n][r] = e;
          }
        l_run[rb] += ls;
      }

      // O^T += V^T . P^T, 16 keys per MFMA
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
          const bf16x8 a = as_bf16x8(load16(sV + (db * 32 + l32) * Tile<D>::VSTR + c * 16 + half * 8));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma32(a, pf[rb], o[rb][db]);
        }
      }
    }

    if (i + 1 < ntiles) stage_store<D>(st, sKbase + (buf ^ 1) * KSZ, sVbase + (buf ^ 1) * VSZ);
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

template <int D, int RB>
__global__ __launch_bounds__(kThreads) void attn_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * KT * Tile<D>::KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * D * Tile<D>::VSTR];
  const uint32_t total = (uint32_t)p.n_units * (uint32_t)p.hq;
  const uint32_t L = xcd_contiguous(blockIdx.x, total);
  const int unit = p.unit_begin + (int)(L / p.hq);
  const int h = (int)(L % p.hq);
  const int g = h / p.group;
  int va, ta, vb, tb;
  p.sched.decode(unit, va, ta, vb, tb);
  if (va >= 0) process_tile<D, RB>(p, h, g, va, ta, sK, sV);
  if (vb >= 0) process_tile<D, RB>(p, h, g, vb, tb, sK, sV);
}

constexpr int kRB = 1;

}  // namespace

int attn_tile_rows(int head_dim) {
  return (head_dim == 64 || head_dim == 128) ? kWaves * 32 * kRB : 0;
}

hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream) {
  const uint64_t total = (uint64_t)p.n_units * (uint64_t)p.hq;
  if (total == 0) return hipSuccess;
  dim3 grid((uint32_t)total), block(kThreads);
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_kernel<128, kRB>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((attn_kernel<64, kRB>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace apbv
