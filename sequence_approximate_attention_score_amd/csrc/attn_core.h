// Tile machinery shared by the gfx950 attention kernels (context rows and query-block rows):
// the LDS stage layout of a 64-key K/V tile, its global->LDS load, and the per-wave update
// of one tile: S^T = K.Q^T on MFMA, masked online softmax (log2 units, lazy rescale),
// O^T += V^T.P^T with transposing LDS reads of V.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "apbv_device.h"

namespace apbv {
namespace tile {

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

// Raw buffer descriptor over the rows of one tile (the byte offsets of a tile stay far
// below 2^31; the third-dword value is the gfx9 raw-buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, 0x7fffffff,
                                           0x00020000);
}

// K and V tile -> one LDS stage, no registers involved (buffer loads that write LDS: unlike
// the global form they leave the LDS-read counter to the LDS reads, so the reads of the
// current tile can wait for one another one at a time). Rows past `valid` repeat the last
// valid row; those keys are masked in the scores, so their values only need to be finite.
template <int D, int NW, int RB, int KT>
__device__ __forceinline__ void load_tile(uint16_t* stage, const LoadMap<D, NW, RB, KT>& lm,
                                          const KeySrc& src) {
  using S = Shape<D, NW, RB, KT>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(src.k), rv = tile_rsrc(src.v);
#pragma unroll
  for (int j = 0; j < S::LOADS; ++j) {
    const int seg = j * NW + wave;
    if (seg < S::SEG) {
      const bool is_v = seg >= S::SEGK;
      const int off = (min(lm.row[j], src.valid - 1) * (int)src.stride + lm.col[j]) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          is_v ? rv : rk, (__attribute__((address_space(3))) void*)(stage + seg * 512), 16, off,
          0, 0, 0);
    }
  }
}

// One key tile for one wave: S^T = K.Q^T, (masked) online softmax, O^T += V^T.P^T.
// With MASK, key kk of the tile (0..KT-1) is dropped for the lane's row rb when kk >= valid
// or key0 + kk > pos[rb] (causal: pos is the row's own key position; a row that never
// reaches a causal source passes a large pos).
template <int D, int NW, int RB, int KT, bool MASK>
__device__ __forceinline__ void attend_tile(const uint16_t* stage, const bf16x8 (&qf)[RB][D / 16],
                                            f32x16 (&o)[RB][D / 32], float (&m_run)[RB],
                                            float (&l_run)[RB], float scale_log2, int key0,
                                            int valid, const int (&pos)[RB]) {
  using S = Shape<D, NW, RB, KT>;
  constexpr int ND = D / 32, NK = D / 16, NN = KT / 32;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const f32x16 zero = {};

  // S^T[key, row] for NN blocks of 32 keys; A = K rows from LDS, B = Q^T from registers
  int kofs = l32 * S::KSTR + half * 8;
  asm volatile("" : "+v"(kofs));
  f32x16 s[RB][NN];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const bf16x8 a = as_bf16x8(load16(stage + (kofs + n * 32 * S::KSTR + ks * 16)));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        s[rb][n] = mfma32(a, qf[rb][ks], ks == 0 ? zero : s[rb][n]);
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (MASK) {
      const int lim = min(valid - 1, pos[rb] - key0);   // last visible key of the tile
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = n * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          s[rb][n][r] = kk > lim ? -INFINITY : s[rb][n][r];
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
  int vofs = S::VOFF + (4 * half + (j16 >> 2)) * S::VSTR + 16 * grp + 4 * (j16 & 3);
  asm volatile("" : "+v"(vofs));
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
      const int o0 = vofs + 16 * c * S::VSTR + 32 * db;
      const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(stage + o0));
      const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(stage + (o0 + 8 * S::VSTR)));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 both = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      const bf16x8 va = __builtin_bit_cast(bf16x8, both);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma32(va, pf[rb], o[rb][db]);
    }
  }
}

}  // namespace tile
}  // namespace apbv
