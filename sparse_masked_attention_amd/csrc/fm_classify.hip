// Key-block min/max table and tile-class map.
//
// The column-wise sparse mask (FlashMask README "Overview"; FlashMask-3
// abstract) stores, per key column, query-row interval bounds. Reducing each
// bound vector to its min and max over a block of key columns is enough to
// decide, per (query block, key block) tile, whether the mask hides all of it,
// none of it, or part of it; the attention kernels skip the first kind and run
// the second without mask arithmetic.
#include <climits>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {

// One wave per (batch * mask head, key block): lanes stride over the block's
// columns, then a butterfly over the wave reduces the eight running values.
__global__ __launch_bounds__(256) void kblock_minmax_kernel(MaskArgs m, int BHm, int Nq, int N,
                                                            int block, int nkb,
                                                            int32_t* __restrict__ out) {
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wave >= (long long)BHm * nkb) return;  // whole waves leave together
  const int bhm = (int)(wave / nkb);
  const int kb = (int)(wave % nkb);
  const long long base = (long long)bhm * N;
  const long long c0 = (long long)kb * block;
  const long long c1 = c0 + block < N ? c0 + block : N;
  const bool has_lt = m.lts != nullptr;
  const bool has_ut = m.uts != nullptr && m.ute != nullptr;
  int mn[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int mx[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  for (long long c = c0 + lane; c < c1; c += 64) {
    int v[4];
    // N key columns; a missing lower interval is [Nq, Nq) (Nq query rows)
    v[0] = has_lt ? m.lts[base + c] : Nq;
    v[1] = (has_lt && m.lte != nullptr) ? m.lte[base + c] : Nq;
    v[2] = has_ut ? m.uts[base + c] : 0;
    v[3] = has_ut ? m.ute[base + c] : 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      mn[t] = min(mn[t], v[t]);
      mx[t] = max(mx[t], v[t]);
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      mn[t] = min(mn[t], __shfl_xor(mn[t], s, 64));
      mx[t] = max(mx[t], __shfl_xor(mx[t], s, 64));
    }
  }
  if (lane < 8) {
    // lane-indexed select, written out so no register is indexed dynamically
    int val = mn[0];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (lane == 2 * t) val = mn[t];
      if (lane == 2 * t + 1) val = mx[t];
    }
    out[((long long)bhm * nkb + kb) * 8 + lane] = val;
  }
}

__global__ __launch_bounds__(256) void classify_kernel(const int32_t* __restrict__ table, long long total,
                                                       int Nq, int Nk, int bq, int bk, int nqb, int nkb,
                                                       int causal, int8_t* __restrict__ out) {
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int kb = (int)(idx % nkb);
    const long long rest = idx / nkb;
    const int qb = (int)(rest % nqb);
    const long long bhm = rest / nqb;
    const long long r0 = (long long)qb * bq;
    const long long c0 = (long long)kb * bk;
    const int r1 = (int)(r0 + bq < Nq ? r0 + bq : Nq);
    const int c1 = (int)(c0 + bk < Nk ? c0 + bk : Nk);
    const BlockBounds t = load_bounds(table + (bhm * nkb + kb) * 8);
    out[idx] = (int8_t)tile_class(t, (int)r0, r1, (int)c0, c1, causal != 0);
  }
}

hipError_t launch_kblock_minmax(const MaskArgs& m, int B, int Nq, int N, int block, int32_t* out,
                                hipStream_t stream) {
  const int nkb = (int)(((long long)N + block - 1) / block);
  const long long waves = (long long)B * m.hm * nkb;
  const long long blocks = (waves + 3) / 4;
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kblock_minmax_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, m, B * m.hm,
                     Nq, N, block, nkb, out);
  return hipGetLastError();
}

hipError_t launch_classify(const int32_t* table, int B, int hm, int Nq, int Nk, int causal,
                           int block_q, int block_k, int8_t* out, hipStream_t stream) {
  const int nqb = (int)(((long long)Nq + block_q - 1) / block_q);
  const int nkb = (int)(((long long)Nk + block_k - 1) / block_k);
  const long long total = (long long)B * hm * nqb * nkb;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(classify_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, table, total, Nq,
                     Nk, block_q, block_k, nqb, nkb, causal, out);
  return hipGetLastError();
}

}  // namespace fm
