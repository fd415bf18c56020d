// Approximate-attention prefill kernel for gfx950 (bf16 MFMA, fp32 online softmax).
//
// Row i of context block v (head h, KV head g = h / G) attends to
//   the prefix k_pre[g, 0 : l_anchor + v*l_pass]   (anchor + passing blocks of blocks < v)
//   then its own block's keys bs[v] .. i           (causal, diagonal included)
// (APB-V technical summary on gist.science, Metodologia part 1, "Meccanismo di Attenzione
// Approssimata"; with one block and no prefix this is plain causal flash attention, as the
// page's "Limitazioni" paragraph notes).
//
// Design (one workgroup = 8 waves = one query tile of 256 rows of one head,
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
#include "apbv_device.h"
#include "apbv_internal.h"
#include "attn_core.h"

namespace apbv {

namespace {

using tile::attend_tile;
using tile::KeySrc;
using tile::load_tile;
using tile::LoadMap;
using tile::Shape;

constexpr int kNoCausal = 1 << 30;   // position of a row that no causal source limits

template <int D, int NW, int RB, int KT>
__device__ __forceinline__ void process_tile(const AttnParams& p, int h, int g, int v, int t,
                                             uint16_t* lds0, uint16_t* lds1,
                                             const LoadMap<D, NW, RB, KT>& lm) {
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

  // Tile i is read from stage i % 2 while tile i + 1 streams into the other stage. The two
  // stages are separate LDS arrays and the loop is unrolled by two, so every LDS access
  // names its array statically: the compiler can then tell the reads of one stage from the
  // direct-to-LDS loads into the other and does not wait for those loads before reading.
  auto step = [&](int i, const uint16_t* stage, uint16_t* next) {
    if (i + 1 < ntiles) load_tile<D, NW, RB, KT>(next, lm, source(i + 1));
    const bool prefix = i < n_pre;
    const int key0 = prefix ? i * KT : lo + (i - n_pre) * KT;
    const int valid = prefix ? min(KT, P - key0) : min(KT, r1 - key0);
    // a local tile entirely in the future of every row of this wave adds nothing
    const bool skip = !prefix && key0 > wrow0 + 32 * RB - 1;
    if (!skip) {
      const bool need_mask = prefix ? (valid < KT) : (key0 + KT - 1 > wrow0);
      if (need_mask) {
        int pos[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) pos[rb] = prefix ? kNoCausal : wrow0 + rb * 32 + l32;
        attend_tile<D, NW, RB, KT, true>(stage, qf, o, m_run, l_run, p.scale_log2, key0, valid,
                                         pos);
      } else {
        const int pos[RB] = {};
        attend_tile<D, NW, RB, KT, false>(stage, qf, o, m_run, l_run, p.scale_log2, key0,
                                          valid, pos);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  load_tile<D, NW, RB, KT>(lds0, lm, source(0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = 0; i < ntiles; i += 2) {
    step(i, lds0, lds1);
    if (i + 1 < ntiles) step(i + 1, lds1, lds0);
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
  __shared__ __attribute__((aligned(1024))) uint16_t lds0[Shape<D, NW, RB, KT>::STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds1[Shape<D, NW, RB, KT>::STAGE];
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
    if (v >= 0) process_tile<D, NW, RB, KT>(p, h, g, v, t, lds0, lds1, lm);
  }
}

// One workgroup = 8 waves x 32 query rows (two waves per SIMD), 64-key tiles.
constexpr int kWaves = 8, kRowBlocks = 1, kKeys = 64;

template <int D>
hipError_t launch_d(const AttnParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_kernel<D, kWaves, kRowBlocks, kKeys>), grid, dim3(kWaves * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

int attn_tile_rows(int head_dim) {
  return (head_dim == 64 || head_dim == 128) ? kWaves * 32 * kRowBlocks : 0;
}

hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream) {
  const uint64_t total = (uint64_t)p.n_units * (uint64_t)p.hq;
  if (total == 0) return hipSuccess;
  if (p.sched.tile_rows != attn_tile_rows(head_dim)) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)total);
  return head_dim == 128 ? launch_d<128>(p, grid, stream) : launch_d<64>(p, grid, stream);
}

}  // namespace apbv
