// Boundary vectors of one context-parallel rank's share of the query rows.
//
// The FlashMask-3 abstract has each rank localise the column-wise mask with
// no communication: the rank holds some chunks of the global query rows (and
// all keys), and every row bound stored per key column is re-expressed in the
// rank's local row numbering. With chunks [q0_c, q1_c) (sorted, disjoint;
// local rows are their rows in order) a global bound t maps to
//     local(t) = sum_c clamp(t - q0_c, 0, q1_c - q0_c),
// a monotone map, so a global row interval [a, b) becomes [local(a),
// local(b)) over exactly the local rows it held. A causal mask's edge (rows
// before the key) becomes the upper interval [0, local(j)), so the output is
// always the non-causal four-vector form.
#include <climits>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {

struct Chunks {
  int n;
  int q0[kMaxChunks];
  int q1[kMaxChunks];
};

__device__ inline int local_row(long long t, const Chunks& c) {
  long long out = 0;
  for (int i = 0; i < c.n; ++i) {
    const long long len = (long long)c.q1[i] - c.q0[i];
    const long long x = t - c.q0[i];
    out += x < 0 ? 0 : (x > len ? len : x);
  }
  return (int)out;
}

__global__ __launch_bounds__(256) void localize_kernel(MaskArgs m, long long total, int Nk, int n_rows,
                                                       Chunks c, int nq_local, int32_t* __restrict__ lts_o,
                                                       int32_t* __restrict__ lte_o, int32_t* __restrict__ uts_o,
                                                       int32_t* __restrict__ ute_o) {
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(idx % Nk);
    int a, b;
    if (m.lts != nullptr) {
      a = local_row(m.lts[idx], c);
      b = local_row(m.lte != nullptr ? m.lte[idx] : n_rows, c);
    } else {
      a = b = nq_local;                       // no lower interval
    }
    lts_o[idx] = a;
    lte_o[idx] = b;
    if (m.causal) {
      a = 0;                                  // global rows before key j
      b = local_row(j, c);
    } else if (m.uts != nullptr) {
      a = local_row(m.uts[idx], c);
      b = local_row(m.ute[idx], c);
    } else {
      a = b = 0;                              // no upper interval
    }
    uts_o[idx] = a;
    ute_o[idx] = b;
  }
}

hipError_t launch_localize(const MaskArgs& m, int B, int Nk, int n_rows, const int32_t* chunks,
                           int nchunks, int32_t* lts_o, int32_t* lte_o, int32_t* uts_o,
                           int32_t* ute_o, hipStream_t stream) {
  Chunks c{};
  c.n = nchunks;
  int nq = 0;
  for (int i = 0; i < nchunks; ++i) {
    c.q0[i] = chunks[2 * i];
    c.q1[i] = chunks[2 * i + 1];
    nq += c.q1[i] - c.q0[i];
  }
  const long long total = (long long)B * m.hm * Nk;
  if (total == 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(localize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, m, total, Nk, n_rows, c,
                     nq, lts_o, lte_o, uts_o, ute_o);
  return hipGetLastError();
}

}  // namespace fm
