// Load-time cut of one rank's shard out of the full weight into the packed
// tile layout described in tp_internal.h ("AI Infrastructure series, Part 5",
// "What does it look like in vLLM ...": the weights are split as they load).
#include "tp_internal.h"

namespace tpk {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(PackArgs a, int64_t total_u4) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_u4) return;
  const int lane = (int)(c & 63);
  // 1 KiB index -> (tile pair, k-step, tile of the pair); see tile_index().
  const int64_t idx = c >> 6;
  const int64_t pair = idx / (2 * a.ksteps), rem = idx - pair * 2 * a.ksteps;
  const int64_t ks = rem >> 1, nt = 2 * pair + (rem & 1);
  const int g = lane >> 4, i = lane & 15;

  // Shard column of this lane and whether it exists.
  int64_t n;
  bool valid;
  if (a.gateup) {
    const int64_t col = (nt >> 1) * kTileN + i;  // output column within the gate (or up) half
    valid = col < a.out_n;
    n = (nt & 1) * a.out_n + col;
  } else {
    n = nt * kTileN + i;
    valid = n < a.shard_n;
  }
  // Shard column -> column of the full weight.
  int64_t wcol = 0;
  if (valid) {
    valid = false;
    for (int r = 0; r < a.n_ranges; ++r) {
      if (n >= a.dst[r] && n < a.dst[r] + a.len[r]) {
        wcol = a.src[r] + (n - a.dst[r]);
        valid = true;
      }
    }
  }
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t k = ks * kTileK + g * 8 + e;
    v[e] = (valid && k < a.shard_k) ? a.W[(a.row_begin + k) * a.ldw + wcol] : (uint16_t)0;
  }
  uint4 o;
  o.x = v[0] | ((uint32_t)v[1] << 16);
  o.y = v[2] | ((uint32_t)v[3] << 16);
  o.z = v[4] | ((uint32_t)v[5] << 16);
  o.w = v[6] | ((uint32_t)v[7] << 16);
  a.out[c] = o;
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const int64_t total = a.ksteps * a.ntiles * kTileU4;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

}  // namespace tpk
