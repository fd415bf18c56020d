// Approximate-attention prefill kernel for gfx950 (bf16 MFMA, fp32 online softmax).
//
// Row i of context block v (head h, KV head g = h / G) attends to
//   the prefix k_pre[g, 0 : l_anchor + v*l_pass]   (anchor + passing blocks of blocks < v)
//   then its own block's keys bs[v] .. i           (causal, diagonal included)
// (APB-V technical summary on gist.science, Metodologia part 1, "Meccanismo di Attenzione
// Approssimata"; with one block and no prefix this is plain causal flash attention, as the
// page's "Limitazioni" paragraph notes).
//
// One workgroup = one 256-row query tile of one head (8 waves x 32 rows), run through the
// pipelined tile loop of attn_pipe.h over the block's prefix tiles and then its own causal
// tiles. Grid = work units x heads, remapped so each XCD gets a contiguous range: the heads
// of one KV group and one unit run side by side on the same XCD and share K/V in its L2.
#include "apbv_device.h"
#include "apbv_internal.h"
#include "attn_pipe.h"

namespace apbv {

namespace {

using namespace pipe;

template <int D>
__device__ __forceinline__ void process_tile(const AttnParams& p, int h, int g, int v, int t,
                                             uint16_t* K0, uint16_t* K1, uint16_t* V0,
                                             uint16_t* V1, const Loader<D>& ld) {
  using G = Geo<D>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int lo = p.sched.bs[v], hi = p.sched.bs[v + 1];
  const int r0 = lo + t * kRows;
  const int r1 = min(r0 + kRows, hi);
  const int wrow0 = r0 + wave * 32;          // first row of this wave
  const int row = wrow0 + l32;

  // Q^T fragments (B operand): lane holds row l32, d = 16ks + 8half + e. Rows past the
  // tile end repeat a valid row; their outputs are never stored.
  bf16x8 qf[G::NK];
  {
    const uint16_t* qrow = p.q + (int64_t)min(row, r1 - 1) * p.q_stride + h * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < G::NK; ++ks) qf[ks] = as_bf16x8(load16(qrow + ks * 16));
  }
  f32x16 o[G::ND];
#pragma unroll
  for (int db = 0; db < G::ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int P = p.l_anchor + v * p.l_pass;
  const int n_pre = (P + kKT - 1) / kKT;
  const int n_loc = (r1 - lo + kKT - 1) / kKT;
  const int ntiles = n_pre + n_loc;
  // tiles this wave computes: every prefix tile, and local tiles up to its last row; a wave
  // whose rows all lie past the end of a short last tile computes nothing
  const int n_live = wrow0 >= r1 ? 0 : n_pre + min(n_loc, (wrow0 + 31 - lo) / kKT + 1);

  auto source = [&](int i) -> KeySrc {
    KeySrc s;
    if (i < n_pre) {
      const int key0 = i * kKT;
      const int64_t off = ((int64_t)g * p.pre_rows + key0) * D;
      s.k = p.kpre + off;
      s.v = p.vpre + off;
      s.stride = D;
      s.valid = min(kKT, P - key0);
    } else {
      const int key0 = lo + (i - n_pre) * kKT;
      const int64_t off = (int64_t)key0 * p.kv_stride + g * D;
      s.k = p.kc + off;
      s.v = p.vc + off;
      s.stride = p.kv_stride;
      s.valid = min(kKT, r1 - key0);
    }
    return s;
  };
  // mask parameters of tile i: prefix tiles are masked only past the prefix end; a local
  // tile is masked where it reaches past the wave's first row (causal diagonal)
  auto mask_of = [&](int i) {
    TileMask m;
    if (i < n_pre) {
      m.key0 = i * kKT;
      m.valid = min(kKT, P - m.key0);
      m.mask = m.valid < kKT;
      m.pos = kNoCausal;
    } else {
      m.key0 = lo + (i - n_pre) * kKT;
      m.valid = min(kKT, r1 - m.key0);
      m.mask = m.key0 + kKT - 1 > wrow0;
      m.pos = row;
    }
    return m;
  };
  run_tiles<D>(ntiles, n_live, source, mask_of, qf, o, m_run, l_run, p.scale_log2, K0, K1, V0,
               V1, ld);

  // epilogue: O = O^T / l, bf16; lse = (m + log2 l) * ln 2
  const float lt = l_run + swap_half(l_run);
  if (row < r1) {
    const float inv = 1.0f / lt;
    uint16_t* orow = p.out + ((int64_t)row * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < G::ND; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * half;
        const f32x16& ov = o[db];
        u32x2 w = {pack_bf16x2(ov[4 * q4 + 0] * inv, ov[4 * q4 + 1] * inv),
                   pack_bf16x2(ov[4 * q4 + 2] * inv, ov[4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (p.lse != nullptr && half == 0)
      p.lse[(int64_t)h * p.n_tokens + row] = (m_run + fast_log2(lt)) * 0.69314718055994531f;
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void attn_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t K0[Geo<D>::KELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t K1[Geo<D>::KELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[Geo<D>::VELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t V1[Geo<D>::VELEMS];
  Loader<D> ld;
  ld.init();
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
    if (v >= 0) {
      process_tile<D>(p, h, g, v, t, K0, K1, V0, V1, ld);
      __syncthreads();   // the next part refills the buffers
    }
  }
}

}  // namespace

int attn_tile_rows(int head_dim) { return (head_dim == 64 || head_dim == 128) ? kRows : 0; }

hipError_t launch_attention(const AttnParams& p, int head_dim, hipStream_t stream) {
  const uint64_t total = (uint64_t)p.n_units * (uint64_t)p.hq;
  if (total == 0) return hipSuccess;
  if (p.sched.tile_rows != attn_tile_rows(head_dim)) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)total);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_kernel<128>, grid, dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace apbv
