// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fm {

// Column granularity of the key-block table the attention kernels consume.
constexpr int kTableBlock = 64;

// Tile shapes the attention kernels classify (query rows x key columns).
constexpr int kFwdBlockK = 64;
// forward query-block height: 4 waves x 32 rows (4 x 16 in the wide-head-dim
// forward at bf16 d = 512)
inline int fwd_block_q(int d, int is_bf16) { return is_bf16 && d == 512 ? 64 : 128; }
constexpr int kBwdBlockK = 128;
// backward query-block height: 64 rows for bf16 with d <= 128, else 32 (32
// everywhere in the second tile configuration, FM_ALT_TILES)
#ifdef FM_ALT_TILES
inline int bwd_block_q(int d, int is_bf16) { (void)d; (void)is_bf16; return 32; }
#else
inline int bwd_block_q(int d, int is_bf16) { return (is_bf16 && d <= 128) ? 64 : 32; }
#endif
// backward key-block width: 64 keys where the wide-head-dim kernels serve the
// Q/K head dim d (bf16 512 and 256; fp32 256 and 192), else kBwdBlockK
inline int bwd_block_k(int d, int is_bf16) {
  return (is_bf16 ? (d == 512 || d == 256) : (d == 256 || d == 192)) ? 64 : kBwdBlockK;
}

// Head dims with kernels compiled in, as (d, dv) pairs per dtype.
inline bool bf16_dims(int d, int dv) {
  return (d == dv && (d == 64 || d == 128 || d == 256 || d == 512)) || (d == 192 && dv == 128);
}
inline bool fp32_dims(int d, int dv) {
  return (d == dv && (d == 64 || d == 128 || d == 256)) || (d == 192 && dv == 128);
}
// The shapes served by the wide-head-dim kernels of fm_wide.hip (chosen by
// measurement against the 32-row kernels): the backward at bf16 d = dv = 512
// and 256, fp32 d = dv = 256 and (d, dv) = (192, 128); the forward at those
// and at bf16 (192, 128).
inline bool wide_bwd_dims(int d, int dv, bool is_bf16) {
  if (is_bf16) return (d == 512 && dv == 512) || (d == 256 && dv == 256);
  return (d == 256 && dv == 256) || (d == 192 && dv == 128);
}
inline bool wide_fwd_dims(int d, int dv, bool is_bf16) {
  return wide_bwd_dims(d, dv, is_bf16) || (is_bf16 && d == 192 && dv == 128);
}

struct MaskArgs {
  const int32_t* lts;  // [B, hm, Nk] or nullptr
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
  int hm;
  int causal;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // backward input (forward output)
  const float* lse;   // backward input
  const void* dout;   // backward input
  MaskArgs mask;
  const int32_t* table;  // [B, hm, ceil(N / kTableBlock), 8]
  int B, H, Nq, Nk, d, dv;   // Nq query rows, Nk keys
  int is_bf16;
  float scale;
  void* out;          // forward: O
  float* lse_out;     // forward: logsumexp
  void* dq;
  void* dk;
  void* dv_out;
  float* delta;       // backward workspace: float32 [B, H, N]
  float* lse2;        // backward workspace: float32 [B, H, N], base-2 logsumexp
  float* pdsum;       // backward workspace: float32 [B, H, Nq], rowsum(dS) (sink gradient)
  int* queue;         // backward workspace: 8 work-queue counters of the bf16 dK/dV pass
  const float* sink;  // per-head sink logits [H] or nullptr
  float* dsink;       // backward: d loss / d sink [H] or nullptr
  unsigned long long* tile_counts;
};

// table over Nk key columns; missing vectors take the neutral bounds of Nq rows
hipError_t launch_kblock_minmax(const MaskArgs& m, int B, int Nq, int Nk, int block, int32_t* out,
                                hipStream_t stream);
hipError_t launch_classify(const int32_t* table, int B, int hm, int Nq, int Nk, int causal,
                           int block_q, int block_k, int8_t* out, hipStream_t stream);
// at most this many query-row chunks per rank in flashmask_localize
constexpr int kMaxChunks = 64;
hipError_t launch_localize(const MaskArgs& m, int B, int Nk, int n_rows, const int32_t* chunks,
                           int nchunks, int32_t* lts_o, int32_t* lte_o, int32_t* uts_o,
                           int32_t* ute_o, hipStream_t stream);
hipError_t launch_fwd(const AttnArgs& a, hipStream_t stream);
hipError_t launch_bwd(const AttnArgs& a, hipStream_t stream);
hipError_t launch_sink_zero(const float* sink, float* dsink, int H, hipStream_t stream);
hipError_t launch_bwd_dq(const AttnArgs& a, hipStream_t stream);
// wide head dims: the forward; the backward's dQ and dK/dV passes (delta and
// the base-2 LSE already in the workspace)
hipError_t launch_wide_fwd(const AttnArgs& a, hipStream_t stream);
hipError_t launch_wide_bwd(const AttnArgs& a, hipStream_t stream);

}  // namespace fm
