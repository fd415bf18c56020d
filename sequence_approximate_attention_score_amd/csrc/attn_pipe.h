// Pipelined flash-attention tile loop for gfx950, shared by the context-row attention
// kernel and the query-block kernel: one workgroup = 8 waves x 32 query rows (two waves per
// SIMD) walks a sequence of 64-key K/V tiles for one head.
//
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: the K tile (shared by the waves) is the A
//    operand read from LDS, the wave's Q rows are the B operand held in registers. The
//    result puts one query row per lane (lanes l and l+32 share a row and split its keys),
//    so row max / sum are lane-local plus one permlane32 swap.
//  * O^T = V^T . P^T: the probabilities are already laid out as the B operand; the V^T
//    operand comes straight from a row-major V tile through ds_read_b64_tr_b16 (two
//    transposing 8-byte reads per operand), so the rescale factor of a row is lane-local.
//  * Software pipeline inside each wave: while the exponentials of tile i are computed on
//    the vector ALU, the matrix core already computes the scores of tile i + 1; then
//    O += V_i^T P_i^T runs beside the row sums of tile i and the row maxima of tile i + 1.
//    The instruction order is fixed with scheduling groups so that every MFMA has vector
//    work issued behind it. K tiles therefore run one tile ahead of V tiles: two K buffers
//    and two V buffers (separate LDS arrays, padded rows: K +16 B, V +64 B, so that neither
//    operand read has bank conflicts), filled by buffer loads straight into LDS; the loads
//    of K_{i+2} and V_{i+1} are in flight during iteration i, one barrier per iteration.
//    The loop is unrolled by two so that every LDS access names its array statically.
//  * Online softmax in log2 units with a lazy rescale: the running offset is only raised
//    when a tile's maximum exceeds it by more than 8 (probabilities stay <= 256), which is
//    exact up to rounding and skips almost every O rescale. Mask code runs only on tiles
//    that need it.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "apbv_device.h"

namespace apbv {
namespace pipe {

constexpr int kWaves = 8;             // 32 query rows each, two per SIMD
constexpr int kKT = 64;               // keys per tile
constexpr int kRows = kWaves * 32;    // query rows per work tile
constexpr int kNoCausal = 1 << 30;    // position of a row that no causal source limits
constexpr float kTau = 8.0f;          // log2 headroom before the running offset is raised

// Source of one key tile: K and V of its first row, row stride (elements), valid rows.
struct KeySrc {
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;
  int valid;
};

// Mask parameters of one tile for one wave: whether any key of the wave's rows is masked,
// the first key's position, the valid keys, and the lane's causal position (kNoCausal when
// no causal limit applies). Key kk of the tile is dropped when kk >= valid or
// key0 + kk > pos.
struct TileMask {
  bool mask;
  int key0;
  int valid;
  int pos;
};

// Raw buffer descriptor over the rows of one tile (the byte offsets of a tile stay far
// below 2^31; the third-dword value is the gfx9 raw-buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, 0x7fffffff,
                                           0x00020000);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// sched_group_barrier classes. Transcendental ops (v_exp_f32) are a class of their own
// (0x400) that the plain vector class does not take, so the softmax groups name both.
constexpr int kSchedVALU = 0x2, kSchedMFMA = 0x8, kSchedDSRead = 0x100, kSchedTrans = 0x400;
constexpr int kSchedVector = kSchedVALU | kSchedTrans;

template <int D>
struct Geo {
  static constexpr int KSTR = D + 8;               // K row stride in LDS (elements)
  // V row stride in LDS (elements): a transposing read serves 32 lanes per pass, four
  // rows x two 32-byte column groups; a row stride of 16 or 48 mod 64 banks (dwords; d =
  // 128 gives 80, d = 64 gives 48) spreads the four rows 16 banks apart, so the eight
  // 8-bank pieces cover the 64 banks once
  static constexpr int VSTR = D + 32;
  static constexpr int KSLOT = KSTR / 8;           // 16-byte slots per padded row
  static constexpr int VSLOT = VSTR / 8;
  static constexpr int SEGK = kKT * KSLOT / 64;    // 1 KB load segments per K tile
  static constexpr int SEGV = kKT * VSLOT / 64;
  static constexpr int KELEMS = SEGK * 512;        // elements per K buffer
  static constexpr int VELEMS = SEGV * 512;
  // waves 0..3 load K tiles, waves 4..7 load V tiles
  static constexpr int LOADS = ((SEGK > SEGV ? SEGK : SEGV) + 3) / 4;
  static constexpr int NK = D / 16;                // 16-deep k steps of S^T
  static constexpr int ND = D / 32;                // 32-wide d blocks of O^T
};

// Per-lane source row / column of each load slot of this wave's half (K or V); padding
// slots repeat column 0 of their row.
template <int D>
struct Loader {
  int row[Geo<D>::LOADS];    // source row of the slot
  int colb[Geo<D>::LOADS];   // byte offset of the slot inside its row
  int wave4;        // wave index within its half (uniform)
  bool is_v;        // this wave loads V tiles (uniform)
  __device__ __forceinline__ void init() {
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    is_v = wave >= 4;
    wave4 = wave & 3;
    const int slots = is_v ? G::VSLOT : G::KSLOT;
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) {
      const int q = (j * 4 + wave4) * 64 + lane;
      const int c = q % slots;
      row[j] = min(q / slots, kKT - 1);
      colb[j] = c < D / 8 ? c * 16 : 0;
    }
  }
  // One tile (K or V rows from `base`, row stride `stride` elements, `valid` rows) into
  // `dst`. Rows past `valid` repeat the last valid row (masked later, only need to be
  // finite). Byte offsets are 24-bit products: a row index below 64 times a row stride
  // below 2^23 bytes (the C ABI rejects larger K/V strides).
  template <int SEGS>
  __device__ __forceinline__ void load(uint16_t* dst, const uint16_t* base, int64_t stride,
                                       int valid) const {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(base);
    const unsigned stride_b = (unsigned)stride * 2u;
#pragma unroll
    for (int j = 0; j < Geo<D>::LOADS; ++j) {
      const int seg = j * 4 + wave4;
      if (seg < SEGS) {
        const int off = (int)__umul24((unsigned)min(row[j], valid - 1), stride_b) + colb[j];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + seg * 512), 16, off, 0,
                                                 0, 0);
      }
    }
  }
};

// Scores s[n] (keys 32n .. 32n+31 of the tile, rows = the wave's 32 query rows) of one
// K tile, as 16 MFMAs.
template <int D>
__device__ __forceinline__ void tile_scores(const uint16_t* kbuf, int kofs,
                                            const bf16x8 (&qf)[D / 16], f32x16 (&s)[2]) {
  using G = Geo<D>;
  const f32x16 zero = {};
#pragma unroll
  for (int ks = 0; ks < G::NK; ++ks)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const bf16x8 a = as_bf16x8(load16(kbuf + (kofs + n * 32 * G::KSTR + ks * 16)));
      s[n] = mfma32(a, qf[ks], ks == 0 ? zero : s[n]);
    }
}

// Keys past `valid` or, for causal rows, past the row's own position become -inf.
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int key0, int valid, int pos) {
  const int half = (threadIdx.x & 63) >> 5;
  const int lim = min(valid - 1, pos - key0);   // last visible key of the tile
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = n * 32 + 8 * (r / 4) + 4 * half + (r % 4);
      s[n][r] = kk > lim ? -INFINITY : s[n][r];
    }
}

__device__ __forceinline__ float row_max(const f32x16 (&s)[2]) {
  float mx = -INFINITY;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[n][r]);
  return fmaxf(mx, swap_half(mx));
}

// One pipelined iteration for tile i (its scores in sc, row max mx): exponentials of tile i
// beside the scores of tile i + 1 (into sn, from kbuf), then O += V_i^T P_i^T beside the row
// sum of tile i and the row max of tile i + 1 (into mx_next). A tile with masked keys is
// masked here, before its row max is taken again; branches come first so that the two
// phases form one straight-line block whose instruction order the scheduling groups fix.
template <int D>
__device__ __forceinline__ void pipe_step(const uint16_t* kbuf, const uint16_t* vbuf, int kofs,
                                          int vofs, const bf16x8 (&qf)[D / 16],
                                          f32x16 (&o)[D / 32], f32x16 (&sc)[2], f32x16 (&sn)[2],
                                          float& mx, float& m_run, float& l_run,
                                          float scale_log2, bool mask, int key0, int valid,
                                          int pos) {
  using G = Geo<D>;
  if (mask) {
    mask_scores(sc, key0, valid, pos);
    mx = row_max(sc);
  }
  // lazy rescale of the running state (rare: taken when the row maximum grows by > kTau)
  const float mxs = mx * scale_log2;
  if (mxs > m_run + kTau) {
    if (m_run != -INFINITY) {     // the first visible tile needs no rescale (O = 0)
      const float alpha = fast_exp2(m_run - mxs);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < G::ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    m_run = mxs;
  }
  const float mu = m_run == -INFINITY ? 0.f : m_run;

  // phase A: P_i = exp2(scale * S_i - m) packed to bf16, beside S_{i+1} = K_{i+1} Q^T
  bf16x8 pf[4];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[n][r] = fast_exp2(fmaf(sc[n][r], scale_log2, -mu));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x16& sv = sc[c / 2];
    const int b0 = (c % 2) * 8;
    u32x4 w = {pack_bf16x2(sv[b0 + 0], sv[b0 + 1]), pack_bf16x2(sv[b0 + 2], sv[b0 + 3]),
               pack_bf16x2(sv[b0 + 4], sv[b0 + 5]), pack_bf16x2(sv[b0 + 6], sv[b0 + 7])};
    pf[c] = as_bf16x8(w);
  }
  tile_scores<D>(kbuf, kofs, qf, sn);

  // phase B: O^T += V_i^T P_i^T (16 keys per MFMA; P^T element e of chunk c in lane half h
  // is key 16c + 8(e/4) + 4h + e%4, and the V^T operand is fetched with two transposing
  // reads whose source lane j of each 16-lane group points at key row 16c + 8t + 4h + j/4
  // and d columns 32db + 16*(group % 2) + 4*(j % 4) .. +3), beside the row sum of P_i and
  // the row max of S_{i+1}
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int db = 0; db < G::ND; ++db) {
      const int o0 = vofs + 16 * c * G::VSTR + 32 * db;
      const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbuf + o0));
      const s16x4 p1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbuf + (o0 + 8 * G::VSTR)));
      const s16x8 both = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      o[db] = mfma32(__builtin_bit_cast(bf16x8, both), pf[c], o[db]);
    }
  float ls = 0.f;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) ls += sc[n][r];
  l_run += ls;
  mx = row_max(sn);

  // instruction order: phase A = per S MFMA one K read (two ahead) and 5 vector ops (the 32
  // exponentials included, two or three behind each MFMA), phase B = per PV MFMA two
  // transposing reads (four ahead) and 3 vector ops
  __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
#pragma unroll
  for (int j = 0; j < 2 * G::NK; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
    if (j + 2 < 2 * G::NK) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedVector, 5, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
  for (int j = 0; j < 4 * G::ND; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
    if (j + 2 < 4 * G::ND) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedVector, 3, 0);
  }
}


// The tile loop of one work tile. source(i) gives tile i's K/V rows, mask_of(i) its mask
// parameters for this wave; the wave computes tiles 0 .. n_live-1 (its rows see no key of
// later tiles) but takes part in every tile's loads and barriers. qf holds the wave's Q^T
// fragments; o, m_run and l_run carry the running output (transposed), offset and sum.
template <int D, class Source, class MaskOf>
__device__ __forceinline__ void run_tiles(int ntiles, int n_live, Source source, MaskOf mask_of,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                          float& m_run, float& l_run, float scale_log2,
                                          uint16_t* K0, uint16_t* K1, uint16_t* V0,
                                          uint16_t* V1, const Loader<D>& ld) {
  using G = Geo<D>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l32 = lane & 31;
  auto load_k = [&](uint16_t* dst, int i) {
    if (!ld.is_v && i < ntiles) {
      const KeySrc s = source(i);
      ld.template load<G::SEGK>(dst, s.k, s.stride, s.valid);
    }
  };
  auto load_v = [&](uint16_t* dst, int i) {
    if (ld.is_v && i < ntiles) {
      const KeySrc s = source(i);
      ld.template load<G::SEGV>(dst, s.v, s.stride, s.valid);
    }
  };

  int kofs = l32 * G::KSTR + half * 8;
  const int grp = (lane >> 4) & 1, j16 = lane & 15;
  int vofs = (4 * half + (j16 >> 2)) * G::VSTR + 16 * grp + 4 * (j16 & 3);
  // opaque lane offsets: every LDS read address stays "array + offset + constant", which
  // keeps the array's alias information on the read
  asm volatile("" : "+v"(kofs), "+v"(vofs));

  // prologue: K_0, V_0, K_1 in flight; scores of tile 0
  load_k(K0, 0);
  load_v(V0, 0);
  load_k(K1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sa[2], sb[2];
  tile_scores<D>(K0, kofs, qf, sa);
  float mx = row_max(sa);
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) sb[n][r] = 0.f;
  __syncthreads();   // K0 is refilled by iteration 0

  // iteration i reads K_{i+1} and V_i and refills the buffers of K_i and V_{i-1}
  auto iter = [&](int i, const uint16_t* kread, const uint16_t* vread, uint16_t* kload,
                  uint16_t* vload, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    load_k(kload, i + 2);
    load_v(vload, i + 1);
    if (i < n_live) {
      const TileMask tm = mask_of(i);
      pipe_step<D>(kread, vread, kofs, vofs, qf, o, sc, sn, mx, m_run, l_run, scale_log2,
                   tm.mask, tm.key0, tm.valid, tm.pos);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int i = 0; i < ntiles; i += 2) {
    iter(i, K1, V0, K0, V1, sa, sb);
    if (i + 1 < ntiles) iter(i + 1, K0, V1, K1, V0, sb, sa);
  }
}

}  // namespace pipe
}  // namespace apbv
