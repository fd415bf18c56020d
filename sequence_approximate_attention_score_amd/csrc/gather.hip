// Passing-block collection for gfx950 (APB-V technical summary on gist.science, Metodologia
// part 1, "Meccanismo di Attenzione Approssimata": each host collects the passing blocks of
// the hosts before it). On one GPU the anchor and every block's passing rows are written
// once into a head-major prefix per KV head:
//     k_pre[g] = k_anchor[:, g] ++ k_ctx[sel[0, g], g] ++ ... ++ k_ctx[sel[n-1, g], g]
// and block v later reads the first l_anchor + v*l_pass rows. Pure data movement: one
// 16-byte chunk per thread, a row's chunks on consecutive lanes (coalesced reads and writes).
#include "apbv_device.h"
#include "apbv_internal.h"

namespace apbv {

namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void gather_kernel(const GatherParams p) {
  constexpr int CH = D / 8;   // 16-byte chunks per row
  const int64_t per_tensor = (int64_t)p.hkv * p.row_count * CH;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= 2 * per_tensor) return;
  const int tensor = (int)(idx / per_tensor);
  int64_t rem = idx - tensor * per_tensor;
  const int ch = (int)(rem % CH);
  rem /= CH;
  const int row = p.row_begin + (int)(rem % p.row_count);
  const int g = (int)(rem / p.row_count);

  const uint16_t* src;
  if (row < p.l_anchor) {
    const uint16_t* a = tensor == 0 ? p.ka : p.va;
    src = a + ((int64_t)row * p.hkv + g) * D;
  } else {
    const int r = row - p.l_anchor;
    const int v = r / p.l_pass, k = r % p.l_pass;
    int j = p.sel[((int64_t)v * p.hkv + g) * p.l_pass + k];
    // an entry outside its own block is a caller error: counted (once per entry) when a
    // counter is given, and clamped into the block so that no read leaves the context
    const int lo = p.bs[v], hi = p.bs[v + 1];
    if (j < lo || j >= hi) {
      if (p.sel_errors != nullptr && tensor == 0 && ch == 0) atomicAdd(p.sel_errors, 1);
      j = j < lo ? lo : hi - 1;
    }
    const uint16_t* c = tensor == 0 ? p.kc : p.vc;
    src = c + (int64_t)j * p.kv_stride + g * D;
  }
  uint16_t* dst = (tensor == 0 ? p.kpre : p.vpre) + ((int64_t)g * p.pre_rows + row) * D;
  store16(dst + ch * 8, load16(src + ch * 8));
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, int head_dim, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)p.hkv * p.row_count * (head_dim / 8);
  if (total == 0) return hipSuccess;
  dim3 grid((uint32_t)((total + kThreads - 1) / kThreads));
  if (head_dim == 128)
    hipLaunchKernelGGL(gather_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(gather_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace apbv
