// C ABI: argument checks, workspace layout and dispatch. Declarations and the
// contract of every entry point are in include/flashmask.h.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/flashmask.h"
#include "fm_internal.hpp"

namespace fm {
// The workspace of flashmask_bwd_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends. In host code `scratch` names a host
// stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, once per device (scratch_address below).
__device__ __align__(256) char scratch[FLASHMASK_NOALLOC_SCRATCH_BYTES];
}  // namespace fm

namespace {

using fm::kTableBlock;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// bf16: d = dv in {64, 128, 256, 512} and (d, dv) = (192, 128); fp32: d = dv
// in {64, 128, 256} and (192, 128). Forward and backward cover the same set.
bool supported(int d, int dv, fm_dtype_t dtype) {
  if (dtype == FM_BF16) return fm::bf16_dims(d, dv);
  if (dtype == FM_FP32) return fm::fp32_dims(d, dv);
  return false;
}

bool bwd_supported(int d, int dv, fm_dtype_t dtype) { return supported(d, dv, dtype); }

// some dv makes (d, dv) supported: the tile shape depends on d only
bool supported_d(int d, fm_dtype_t dtype) { return supported(d, d, dtype) || supported(d, 128, dtype); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t table_bytes(int B, int hm, int N) {
  return (size_t)B * hm * (size_t)ceil_div(N, kTableBlock) * 8 * sizeof(int32_t);
}

// Sizes the kernels can address (sizes already non-negative): 32-bit buffer
// offsets cover one (batch, head) slice of a tensor, and B * H * ceil(rows /
// 32) stays below 2^31 (32-row units index grids and queues). Each product
// is formed only where it cannot overflow: B * H < 2^62 always, and once
// below 2^31 it times ceil(rows / 32) < 2^26 stays below 2^57.
bool addressable(int B, int H, int Nq, int Nk, int d, int dv, fm_dtype_t dtype) {
  const long long lim = 1LL << 31;
  const long long rows = Nq > Nk ? Nq : Nk;
  const long long width = d > dv ? d : dv;
  if (rows * width * (dtype == FM_BF16 ? 2 : 4) >= lim) return false;
  const long long bh = (long long)B * H;
  return bh < lim && bh * ceil_div(rows, 32) < lim;
}

// Checks shared by the attention entry points; FM_SUCCESS when usable.
fm_status_t check_common(int B, int H, int Nq, int Nk, int d, int dv, fm_dtype_t dtype, int hm,
                         const int32_t* uts, const int32_t* ute, int causal) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d <= 0 || dv <= 0 || hm < 1)
    return FM_ERROR_INVALID_VALUE;
  if (dtype != FM_BF16 && dtype != FM_FP32) return FM_ERROR_INVALID_VALUE;
  if (H > 0 && hm != 1 && hm != H) return FM_ERROR_INVALID_VALUE;
  if (!causal && ((uts == nullptr) != (ute == nullptr))) return FM_ERROR_INVALID_VALUE;
  if (!supported(d, dv, dtype)) return FM_ERROR_NOT_SUPPORTED;
  return addressable(B, H, Nq, Nk, d, dv, dtype) ? FM_SUCCESS : FM_ERROR_NOT_SUPPORTED;
}

fm::MaskArgs mask_args(const int32_t* lts, const int32_t* lte, const int32_t* uts,
                       const int32_t* ute, int hm, int causal) {
  fm::MaskArgs m;
  m.lts = lts;
  m.lte = lts != nullptr ? lte : nullptr;
  const bool ut = !causal && uts != nullptr && ute != nullptr;
  m.uts = ut ? uts : nullptr;
  m.ute = ut ? ute : nullptr;
  m.hm = hm;
  m.causal = causal != 0;
  return m;
}

float resolve_scale(float s, int d) {
  if (!(s > 0.f)) return 1.0f / std::sqrt((float)d);  // also catches NaN
  return s;
}

// Device address of this GPU's `scratch`, looked up on the first call made
// with that device current and kept per device (atomic slots: host threads
// may race here, and each stores the same address). nullptr on a HIP error.
void* scratch_address() {
  static std::atomic<void*> slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = slots[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(fm::scratch)) != hipSuccess || p == nullptr) return nullptr;
    slots[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

const char* flashmask_status_string(fm_status_t status) {
  switch (status) {
    case FM_SUCCESS: return "success";
    case FM_ERROR_INVALID_VALUE: return "invalid argument";
    case FM_ERROR_NOT_SUPPORTED: return "head dim / dtype combination not supported";
    case FM_ERROR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FM_ERROR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int flashmask_table_block(void) { return kTableBlock; }

fm_status_t flashmask_tile_shape(int is_bwd, int d, fm_dtype_t dtype, int* block_q, int* block_k) {
  if (block_q == nullptr || block_k == nullptr) return FM_ERROR_INVALID_VALUE;
  if (!supported_d(d, dtype)) return FM_ERROR_NOT_SUPPORTED;
  *block_q = is_bwd ? fm::bwd_block_q(d, dtype == FM_BF16) : fm::fwd_block_q(d, dtype == FM_BF16);
  *block_k = is_bwd ? fm::bwd_block_k(d, dtype == FM_BF16) : fm::kFwdBlockK;
  return FM_SUCCESS;
}

size_t flashmask_workspace_size_qk(int is_bwd, int B, int H, int Nq, int Nk, int d, int dv, int hm,
                                   fm_dtype_t dtype) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || hm <= 0 || d <= 0 || dv <= 0) return 0;
  if (H > 0 && hm != 1 && hm != H) return 0;
  if (!supported(d, dv, dtype) || !addressable(B, H, Nq, Nk, d, dv, dtype)) return 0;
  size_t bytes = align_up(table_bytes(B, hm, Nk));
  if (is_bwd) {
    // delta, base-2 LSE, rowsum(dS), the dK/dV pass's work-queue counters
    bytes += 3 * align_up((size_t)B * H * Nq * sizeof(float)) + align_up(8 * sizeof(int));
  }
  return bytes;
}

size_t flashmask_workspace_size(int is_bwd, int B, int H, int N, int d, int dv, int hm,
                                fm_dtype_t dtype) {
  return flashmask_workspace_size_qk(is_bwd, B, H, N, N, d, dv, hm, dtype);
}

fm_status_t flashmask_tile_classify_qk(const int32_t* lts, const int32_t* lte, const int32_t* uts,
                                       const int32_t* ute, int B, int hm, int Nq, int Nk, int causal,
                                       int block_q, int block_k, int32_t* kblock_minmax,
                                       int8_t* tile_class, void* stream) {
  if (B < 0 || hm <= 0 || Nq < 0 || Nk < 0 || block_q < 1 || block_k < 1) return FM_ERROR_INVALID_VALUE;
  if (!causal && ((uts == nullptr) != (ute == nullptr))) return FM_ERROR_INVALID_VALUE;
  if ((long long)B * hm * Nk == 0) return FM_SUCCESS;   // no key column: no table, no tile
  if (kblock_minmax == nullptr || !aligned(kblock_minmax, 16)) return FM_ERROR_INVALID_VALUE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const fm::MaskArgs m = mask_args(lts, lte, uts, ute, hm, causal);
  if (fm::launch_kblock_minmax(m, B, Nq, Nk, block_k, kblock_minmax, s) != hipSuccess) return FM_ERROR_HIP;
  if (tile_class != nullptr && Nq > 0) {
    if (fm::launch_classify(kblock_minmax, B, hm, Nq, Nk, causal != 0, block_q, block_k, tile_class, s) !=
        hipSuccess)
      return FM_ERROR_HIP;
  }
  return FM_SUCCESS;
}

fm_status_t flashmask_tile_classify(const int32_t* lts, const int32_t* lte, const int32_t* uts,
                                    const int32_t* ute, int B, int hm, int N, int causal,
                                    int block_q, int block_k, int32_t* kblock_minmax,
                                    int8_t* tile_class, void* stream) {
  return flashmask_tile_classify_qk(lts, lte, uts, ute, B, hm, N, N, causal, block_q, block_k,
                                    kblock_minmax, tile_class, stream);
}

fm_status_t flashmask_fwd_qk(const void* q, const void* k, const void* v, const int32_t* lts,
                             const int32_t* lte, const int32_t* uts, const int32_t* ute, int hm,
                             const int32_t* kblock_minmax, int B, int H, int Nq, int Nk, int d,
                             int dv, fm_dtype_t dtype, int causal, float softmax_scale,
                             const float* sink, void* o, float* lse, int64_t* tile_counts,
                             void* workspace, size_t workspace_bytes, void* stream) {
  fm_status_t st = check_common(B, H, Nq, Nk, d, dv, dtype, hm, uts, ute, causal);
  if (st != FM_SUCCESS) return st;
  if ((long long)B * H * Nq == 0) return FM_SUCCESS;
  if (q == nullptr || o == nullptr || lse == nullptr) return FM_ERROR_INVALID_VALUE;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return FM_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return FM_ERROR_INVALID_VALUE;
  if (kblock_minmax != nullptr && !aligned(kblock_minmax, 16)) return FM_ERROR_INVALID_VALUE;
  const size_t need = flashmask_workspace_size_qk(0, B, H, Nq, Nk, d, dv, hm, dtype);
  if (kblock_minmax == nullptr && Nk > 0 && (workspace == nullptr || workspace_bytes < need))
    return FM_ERROR_WORKSPACE_TOO_SMALL;
  if (workspace != nullptr && !aligned(workspace, kAlign)) return FM_ERROR_INVALID_VALUE;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  fm::AttnArgs a{};
  a.mask = mask_args(lts, lte, uts, ute, hm, causal);
  const int32_t* table = kblock_minmax;
  if (table == nullptr && Nk > 0) {
    int32_t* t = reinterpret_cast<int32_t*>(workspace);
    if (fm::launch_kblock_minmax(a.mask, B, Nq, Nk, kTableBlock, t, s) != hipSuccess) return FM_ERROR_HIP;
    table = t;
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.table = table;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.dv = dv;
  a.is_bf16 = dtype == FM_BF16;
  a.scale = resolve_scale(softmax_scale, d);
  a.out = o;
  a.lse_out = lse;
  a.sink = sink;
  a.tile_counts = reinterpret_cast<unsigned long long*>(tile_counts);
  if (fm::launch_fwd(a, s) != hipSuccess) return FM_ERROR_HIP;
  return FM_SUCCESS;
}

fm_status_t flashmask_fwd(const void* q, const void* k, const void* v, const int32_t* lts,
                          const int32_t* lte, const int32_t* uts, const int32_t* ute, int hm,
                          const int32_t* kblock_minmax, int B, int H, int N, int d, int dv,
                          fm_dtype_t dtype, int causal, float softmax_scale, void* o, float* lse,
                          int64_t* tile_counts, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return flashmask_fwd_qk(q, k, v, lts, lte, uts, ute, hm, kblock_minmax, B, H, N, N, d, dv, dtype,
                          causal, softmax_scale, nullptr, o, lse, tile_counts, workspace,
                          workspace_bytes, stream);
}

fm_status_t flashmask_bwd_qk(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const int32_t* lts,
                             const int32_t* lte, const int32_t* uts, const int32_t* ute, int hm,
                             const int32_t* kblock_minmax, int B, int H, int Nq, int Nk, int d,
                             int dv, fm_dtype_t dtype, int causal, float softmax_scale,
                             const float* sink, void* dq, void* dk, void* dv_out, float* dsink,
                             int64_t* tile_counts, void* workspace, size_t workspace_bytes,
                             void* stream) {
  fm_status_t st = check_common(B, H, Nq, Nk, d, dv, dtype, hm, uts, ute, causal);
  if (st != FM_SUCCESS) return st;
  if (!bwd_supported(d, dv, dtype)) return FM_ERROR_NOT_SUPPORTED;
  if ((long long)B * H * (Nq > Nk ? Nq : Nk) == 0) {
    // no row: the sink's gradient is an empty sum
    if (sink != nullptr && dsink != nullptr && H > 0 &&
        fm::launch_sink_zero(sink, dsink, H, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
      return FM_ERROR_HIP;
    return FM_SUCCESS;
  }
  // the query side (Q, O, LSE, dO, dQ) may be empty, or the key side (K, V, dK, dV)
  if (Nq > 0 && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr))
    return FM_ERROR_INVALID_VALUE;
  if (Nk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv_out == nullptr))
    return FM_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv_out, 16))
    return FM_ERROR_INVALID_VALUE;
  if (kblock_minmax != nullptr && !aligned(kblock_minmax, 16)) return FM_ERROR_INVALID_VALUE;
  const size_t need = flashmask_workspace_size_qk(1, B, H, Nq, Nk, d, dv, hm, dtype);
  if (workspace == nullptr || workspace_bytes < need) return FM_ERROR_WORKSPACE_TOO_SMALL;
  if (!aligned(workspace, kAlign)) return FM_ERROR_INVALID_VALUE;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  fm::AttnArgs a{};
  a.mask = mask_args(lts, lte, uts, ute, hm, causal);
  const int32_t* table = kblock_minmax;
  if (table == nullptr && Nk > 0) {
    int32_t* t = reinterpret_cast<int32_t*>(ws);
    if (fm::launch_kblock_minmax(a.mask, B, Nq, Nk, kTableBlock, t, s) != hipSuccess) return FM_ERROR_HIP;
    table = t;
  }
  ws += align_up(table_bytes(B, hm, Nk));
  a.delta = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)B * H * Nq * sizeof(float));
  a.lse2 = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)B * H * Nq * sizeof(float));
  a.pdsum = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)B * H * Nq * sizeof(float));
  a.queue = reinterpret_cast<int*>(ws);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.table = table;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.dv = dv;
  a.is_bf16 = dtype == FM_BF16;
  a.scale = resolve_scale(softmax_scale, d);
  a.dq = dq;
  a.dk = dk;
  a.dv_out = dv_out;
  a.sink = sink;
  a.dsink = dsink;
  a.tile_counts = reinterpret_cast<unsigned long long*>(tile_counts);
  if (fm::launch_bwd(a, s) != hipSuccess) return FM_ERROR_HIP;
  return FM_SUCCESS;
}

fm_status_t flashmask_bwd(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, const int32_t* lts,
                          const int32_t* lte, const int32_t* uts, const int32_t* ute, int hm,
                          const int32_t* kblock_minmax, int B, int H, int N, int d, int dv,
                          fm_dtype_t dtype, int causal, float softmax_scale, void* dq, void* dk,
                          void* dv_out, int64_t* tile_counts, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return flashmask_bwd_qk(q, k, v, o, lse, dout, lts, lte, uts, ute, hm, kblock_minmax, B, H, N, N,
                          d, dv, dtype, causal, softmax_scale, nullptr, dq, dk, dv_out, nullptr,
                          tile_counts, workspace, workspace_bytes, stream);
}

fm_status_t flashmask_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, const int32_t* lts,
                                  const int32_t* lte, const int32_t* uts, const int32_t* ute, int hm,
                                  const int32_t* kblock_minmax, int B, int H, int Nq, int Nk, int d,
                                  int dv, fm_dtype_t dtype, int causal, float softmax_scale,
                                  const float* sink, void* dq, void* dk, void* dv_out, float* dsink,
                                  int64_t* tile_counts, void* stream) {
  fm_status_t st = check_common(B, H, Nq, Nk, d, dv, dtype, hm, uts, ute, causal);
  if (st != FM_SUCCESS) return st;
  const size_t need = flashmask_workspace_size_qk(1, B, H, Nq, Nk, d, dv, hm, dtype);
  if (need > (size_t)FLASHMASK_NOALLOC_SCRATCH_BYTES) return FM_ERROR_WORKSPACE_TOO_SMALL;
  if ((long long)B * H * (Nq > Nk ? Nq : Nk) == 0)   // no row or key: needs no workspace
    return flashmask_bwd_qk(q, k, v, o, lse, dout, lts, lte, uts, ute, hm, kblock_minmax, B, H, Nq,
                            Nk, d, dv, dtype, causal, softmax_scale, sink, dq, dk, dv_out, dsink,
                            tile_counts, nullptr, 0, stream);
  void* ws = scratch_address();
  if (ws == nullptr) return FM_ERROR_HIP;
  return flashmask_bwd_qk(q, k, v, o, lse, dout, lts, lte, uts, ute, hm, kblock_minmax, B, H, Nq, Nk,
                          d, dv, dtype, causal, softmax_scale, sink, dq, dk, dv_out, dsink, tile_counts,
                          ws, (size_t)FLASHMASK_NOALLOC_SCRATCH_BYTES, stream);
}

int flashmask_max_chunks(void) { return fm::kMaxChunks; }

fm_status_t flashmask_localize(const int32_t* lts, const int32_t* lte, const int32_t* uts,
                               const int32_t* ute, int B, int hm, int Nk, int n_rows, int causal,
                               const int32_t* chunks, int nchunks, int32_t* lts_out,
                               int32_t* lte_out, int32_t* uts_out, int32_t* ute_out, void* stream) {
  if (B < 0 || hm < 1 || Nk < 0 || n_rows < 0) return FM_ERROR_INVALID_VALUE;
  if (!causal && ((uts == nullptr) != (ute == nullptr))) return FM_ERROR_INVALID_VALUE;
  if (chunks == nullptr || nchunks < 1 || nchunks > fm::kMaxChunks) return FM_ERROR_INVALID_VALUE;
  for (int i = 0; i < nchunks; ++i) {
    const int a = chunks[2 * i], b = chunks[2 * i + 1];
    if (a < 0 || b > n_rows || b <= a) return FM_ERROR_INVALID_VALUE;
    if (i > 0 && a < chunks[2 * i - 1]) return FM_ERROR_INVALID_VALUE;
  }
  if ((long long)B * hm * Nk == 0) return FM_SUCCESS;
  if (lts_out == nullptr || lte_out == nullptr || uts_out == nullptr || ute_out == nullptr)
    return FM_ERROR_INVALID_VALUE;
  const fm::MaskArgs m = mask_args(lts, lte, uts, ute, hm, causal);
  if (fm::launch_localize(m, B, Nk, n_rows, chunks, nchunks, lts_out, lte_out, uts_out, ute_out,
                          reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FM_ERROR_HIP;
  return FM_SUCCESS;
}

}  // extern "C"
