// Wide head dims: bf16 with d = dv = 512 and 256, fp32 with d = dv = 256 and
// with (d, dv) = (192, 128); and the forward at bf16 (d, dv) = (192, 128).
//
// The pages list large head dims among the method's features (FlashMask
// README, "News" and "Key Features"); the computation is the same as at
// the narrower dims (FlashMask README, "Formulation": S = scale Q K^T plus
// the column-wise mask bias, softmax, P V; and its gradient, with
// dS = P (dP - delta)), only the rows are wider.
//
// Every product here uses the 16x16 MFMA forms (v_mfma_f32_16x16x32_bf16,
// v_mfma_f32_16x16x4_f32): lane (n = lane % 16, k-group g = lane / 16)
// operands, and a 16x16 accumulator in which lane (n, g) holds M index
// 4 g + e in register e. With 16 rows (or keys) per wave a lane keeps a
// quarter of its row of Q and dO (or K and V) as operands, 64 registers at
// 1 KiB rows, so a whole output row fits in accumulators: each tile's
// scores are formed once, with no split of the output columns.
//
// Contractions over a tile's rows (P V, dS K, P^T dO, dS^T Q) take the
// other operand in the order of the score accumulators: element e of lane
// group g is tile row 16 (e / 4) + 4 g + e % 4. bf16 reads such a column
// block with two transposed LDS reads (ds_read_b64_tr_b16), fp32 with one
// float per MFMA step.
//
// The three kernels keep the decomposition of the narrower ones (query-major
// forward and dQ pass, key-major dK/dV pass, each tile classified from the
// key-block table). Tiles of 32 rows move into LDS by LDS DMA (one 16-byte
// piece per lane, one instruction per tile row), two stages deep: the next
// visible tile loads while the current one is computed (the forward at one
// workgroup per CU waits for a tile's K and its V apart, so that each load
// has a tile and a half to arrive). With rows of at most 512 bytes (bf16
// d = 256, (192, 128)) two workgroups share a CU; wider rows take a CU each.
#include <type_traits>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {

struct WideParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
  const int32_t* table;  // [B, hm, ceil(Nk / 64), 8]
  void* o;
  float* lse;
  const float* sink;
  unsigned long long* counts;
  const void* dout;
  const float* lse2;     // base-2 LSE (+inf for a fully masked row)
  const float* delta;    // rowsum(dO * O)
  float* pdsum;          // rowsum(dS) for the sink gradient, or nullptr
  void* dq;
  void* dk;
  void* dv;
  int B, H, Nq, Nk, hm, causal, has_lt, has_lte, has_ut;
  float scale, sl2;
  int nqb, nkb64;   // query blocks (or steps); 64-key table entries
};

// Waves per SIMD a kernel is built for: 2 (two workgroups per CU, at most 256
// registers per lane) where rows are at most 512 bytes, else 1.
template <typename T, int D, int DV>
constexpr int wide_occupancy() {
  return (int)sizeof(T) * D <= 512 && (int)sizeof(T) * DV <= 512 ? 2 : 1;
}

// ---------------------------------------------------------------- MFMA forms
template <typename T>
struct W16;
template <>
struct W16<float> {
  using op = float;
  static constexpr int KC = 4;   // contraction depth of one MFMA
  __device__ static f32x4 mma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};
template <>
struct W16<bf16> {
  using op = bf16x8;
  static constexpr int KC = 32;
  __device__ static f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) { return mfma16(a, b, c); }
};

// Operands of global row `row` (W wide) for lane (n, g): step c holds
// elements [c KC + g KC / 4, + KC / 4). Rows at or past n_rows read 0.
template <typename T, int W>
__device__ inline void load_row_ops(typename W16<T>::op (&r)[W / W16<T>::KC], const T* base, int row,
                                    int n_rows, int g) {
  constexpr int KC = W16<T>::KC;
  const bool ok = row < n_rows;
#pragma unroll
  for (int c = 0; c < W / KC; ++c) {
    if constexpr (std::is_same<T, float>::value) {
      r[c] = ok ? base[(long long)row * W + KC * c + g] : 0.f;
    } else {
      r[c] = ok ? *reinterpret_cast<const bf16x8*>(base + (long long)row * W + KC * c + 8 * g) : bf16x8{};
    }
  }
}

// LDS row stride (bytes) of a tile W elements wide. bf16: 32 bytes of
// padding, with which both access patterns are free of bank conflicts (the
// row reads, 16 rows at one 16-byte chunk, and the transposed reads, 4 rows
// x 32 bytes per 16-lane group; measured: 16, 48 or 80 bytes leave 20-29%
// of the cycles of the d = 512 kernels in bank conflicts, 32 none). fp32:
// 16 bytes, which puts the 4 rows of a column read (rows 4 apart) on
// disjoint banks.
template <typename T, int W>
constexpr int row_stride() {
  return sizeof(T) == 2 ? W * 2 + 32 : W * 4 + 16;
}

// The same operand step of LDS tile row `row` (row stride rsb bytes).
template <typename T>
__device__ inline typename W16<T>::op row_op(const FM_LDS char* t, int rsb, int row, int c, int g) {
  if constexpr (std::is_same<T, float>::value) {
    return *reinterpret_cast<const FM_LDS float*>(t + row * rsb + (4 * c + g) * 4);
  } else {
    return *reinterpret_cast<const FM_LDS bf16x8*>(t + row * rsb + (32 * c + 8 * g) * 2);
  }
}

// Column col0 + n of the 32 rows of an LDS tile as the operand of a
// contraction over those rows, in score-accumulator order. bf16: the whole
// contraction (32 rows) in one operand, from two transposed reads (each
// 16-lane group reads a 4-row x 16-column block; lane n of group g receives
// rows 4 g .. 4 g + 3, then 16 + 4 g .. 16 + 4 g + 3, of column col0 + n).
// fp32: step s of 8, row 16 (s / 4) + 4 g + s % 4.
__device__ inline bf16x8 col_tr(const FM_LDS char* t, int rsb, int col0, int lane) {
  const int sl = lane & 15, g = lane >> 4;
  const FM_LDS char* pa = t + (4 * g + (sl >> 2)) * rsb + (col0 + 4 * (sl & 3)) * 2;
  return cat(lds_read_tr(pa), lds_read_tr(pa + 16 * rsb));
}
__device__ inline float col_f32(const FM_LDS char* t, int rsb, int col, int s, int g) {
  return *reinterpret_cast<const FM_LDS float*>(t + (16 * (s / 4) + 4 * g + s % 4) * rsb + col * 4);
}

// Step s of the two score-shaped accumulators (rows 16 mt + 4 g + e) as the
// operand of a contraction over their rows (bf16: all 32 rows, rounded to
// nearest even).
template <typename T>
__device__ inline typename W16<T>::op acc_op(const f32x4 (&a)[2], int s) {
  if constexpr (std::is_same<T, float>::value) {
    return a[s / 4][s % 4];
  } else {
    (void)s;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)a[e / 4][e % 4];
    return v;
  }
}

// A chain of N MFMA steps with operands read from LDS: the reads run PF steps
// ahead of the products through a ring of registers, and a fence per step
// keeps that order (VALU, SALU and transcendental work may cross it).
// Without the fences the scheduler hoists the reads of a whole unrolled
// chain ahead of its first product and the registers run out.
template <int N, int PF, typename Rd, typename Step>
__device__ inline void chain(Rd rd, Step step) {
  constexpr int P = PF < N ? PF : N;
  decltype(rd(0)) ring[P];
#pragma unroll
  for (int t = 0; t < P; ++t) ring[t] = rd(t);
#pragma unroll
  for (int t = 0; t < N; ++t) {
    const auto a = ring[t % P];
    if (t + P < N) ring[t % P] = rd(t + P);
    step(t, a);
    __builtin_amdgcn_sched_barrier(0x406);
  }
}

// max / sum over the four lanes of one accumulator column (n, n + 16,
// n + 32, n + 48): a swap of 16-lane rows, then of 32-lane halves
__device__ inline float max_x4(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_x32(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ inline float sum_x4(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return sum_x32(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// Whether the mask hides element (row i, key j), from key j's bounds.
// Bitwise operators throughout: every operand is evaluated and the result
// is a plain select, with no branch per element (short-circuit forms let the
// bound loads move into per-element branches, and the vector element writes
// under that divergent control flow came out wrong).
__device__ inline bool hidden(const WideParams& p, int i, int j, int lts, int lte, int uts, int ute) {
  const int lte_v = p.has_lte ? lte : p.Nq;
  bool m = (j >= p.Nk) | (i >= p.Nq) | ((p.causal != 0) & (j > i));
  m |= (p.has_lt != 0) & (lts <= i) & (i < lte_v);
  m |= (p.has_ut != 0) & (uts <= i) & (i < ute);
  return m;
}

// Appends the visible tiles among [base, base + 256) of a workgroup's walk
// to `list`, from position cnt: thread t tests tile base + t with cls(tile,
// bits), which returns 0 for a tile the mask hides from the whole workgroup
// and otherwise sets bits to the four waves' classes (2 bits each). An entry
// is the tile index with the bits above bit 24. Returns the new count, the
// same in every thread.
template <typename Cls>
__device__ inline int scan_chunk(FM_LDS int* list, FM_LDS int* wsum, int cnt, int base, int n, Cls cls) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = base + tid;
  unsigned bits = 0;
  const bool valid = t < n && cls(t, bits) != 0;
  const unsigned long long bal = __ballot(valid);
  const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
  if (lane == 0) wsum[w] = __builtin_popcountll(bal);
  __syncthreads();
  int off = cnt, add = 0;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const int v = wsum[ww];
    if (ww < w) off += v;
    add += v;
  }
  if (valid) list[off + rank] = (int)((unsigned)t | (bits << 24));
  __syncthreads();
  return cnt + uniform(add);
}

// Runs the tiles of `list` [0, cnt) through two LDS stages: tile it + 1
// loads while tile it is computed. At step it only tile it's loads are in
// flight; once every wave has them (the barrier) every wave is also done
// with tile it - 1, whose stage then takes tile it + 1: one barrier per tile.
template <typename Issue, typename Compute>
__device__ inline void run_list(const FM_LDS int* list, int cnt, Issue issue, Compute compute) {
  auto step = [&](int it, auto stage_c) {
    const unsigned entry = uniform_u32((unsigned)list[it]);
    wait_vmcnt<0>();
    lds_barrier();
    if (it + 1 < cnt) issue(uniform_u32((unsigned)list[it + 1]), std::integral_constant<int, 1 - decltype(stage_c)::value>{});
    compute(entry, stage_c);
  };
  if (cnt > 0) issue(uniform_u32((unsigned)list[0]), std::integral_constant<int, 0>{});
  for (int it = 0; it < cnt; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < cnt) step(it + 1, std::integral_constant<int, 1>{});
  }
}

// The forward's tiles through the same two LDS stages with K (and the keys'
// bounds) and V waited for apart: tile it's K is needed from the start of
// its step, its V only after the scores and softmax. Each step passes two
// barriers: at the first (K of tile it landed everywhere; every wave is done
// with V of tile it - 1) V of tile it + 1 is issued; at the second (V of
// tile it landed; every wave is done with K of tile it) K of tile it + 2.
// Every load then has a step and a half to arrive instead of one. Loads are
// counted per wave: a K issue is NK instructions, a V issue NV.
template <int NK, int NV, typename IssueK, typename IssueV, typename Scores, typename Product>
__device__ inline void run_list_kv(const FM_LDS int* list, int cnt, IssueK issue_k, IssueV issue_v, Scores scores,
                                   Product product) {
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto entry = [&](int it) { return uniform_u32((unsigned)list[it]); };
  auto step = [&](int it, auto stage_c) {
    using SN = std::integral_constant<int, 1 - decltype(stage_c)::value>;
    const unsigned e = entry(it);
    // K of tile it; V of tile it and K of tile it + 1 may stay in flight
    if (it + 1 < cnt) wait_vmcnt<NV + NK>();
    else wait_vmcnt<NV>();
    lds_barrier();
    if (it + 1 < cnt) issue_v(entry(it + 1), SN{});
    scores(e, stage_c);
    // V of tile it; K of tile it + 1 and V of tile it + 1 may stay in flight
    if (it + 1 < cnt) wait_vmcnt<NK + NV>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (it + 2 < cnt) issue_k(entry(it + 2), stage_c);
    product(e, stage_c);
  };
  if (cnt > 0) {
    issue_k(entry(0), S0{});
    issue_v(entry(0), S0{});
  }
  if (cnt > 1) issue_k(entry(1), S1{});
  for (int it = 0; it < cnt; it += 2) {
    step(it, S0{});
    if (it + 1 < cnt) step(it + 1, S1{});
  }
}

// Rows [r0, r0 + 32) of a row-major head slice (resource r, CP 16-byte
// pieces per row) into an LDS tile with row stride rsb bytes: wave w moves
// rows w, w + 4, ..., one instruction per row (kDmaPerWave per wave). Rows
// past the slice read 0.
constexpr int kDmaPerWave = 8;
template <int CP>
__device__ inline void dma_rows(__amdgpu_buffer_rsrc_t r, FM_LDS char* dst, int rsb, int r0, int w, int lane) {
  static_assert(CP <= 64, "one instruction per row");
#pragma unroll
  for (int k = 0; k < kDmaPerWave; ++k) {
    const int row = w + 4 * k;
    if (CP == 64 || lane < CP)
      load_lds16(r, dst + row * rsb, (uint32_t)(r0 + row) * (uint32_t)(CP * 16) + 16u * (uint32_t)lane);
  }
}

// A buffer resource over `n` int32 or float values at base (none when absent)
template <typename V>
__device__ inline __amdgpu_buffer_rsrc_t vec_rsrc(const V* base, long long off, int n, bool present) {
  return make_rsrc(present ? base + off : nullptr, present ? (uint32_t)n * 4u : 0u);
}

// ---------------------------------------------------------------- forward
// Workgroup: 128 query rows (32 per wave, as two 16-row blocks) and every
// output column. Per visible 32-key tile (K, V and the keys' bounds in LDS):
// S^T = K Q^T (Q in registers), the tile's mask, online softmax,
// O^T += V^T P^T. Each K and V operand read from LDS feeds one MFMA per row
// block.
template <typename T, int D, int DV>
struct WFwd {
  // 16-row blocks per wave: two where Q and O of 32 rows fit the registers
  static constexpr int RB = (int)sizeof(T) * D <= 512 || sizeof(T) == 4 ? 2 : 1;
  static constexpr int WR = 16 * RB, BR = 4 * WR, BC = 32;
  static constexpr int RSK = row_stride<T, D>(), RSV = row_stride<T, DV>();   // LDS row strides (bytes)
  static constexpr int CPK = D * (int)sizeof(T) / 16, CPV = DV * (int)sizeof(T) / 16;
  static constexpr int KT = BC * RSK, VT = BC * RSV;
  static constexpr int STAGE = KT + VT + 4 * BC * 4;     // K, V, LTS/LTE/UTS/UTE of the keys
  static constexpr int LIST = 512;
};

// -inf on the hidden elements of two S^T blocks (lane: row i; keys
// kbase + 16 jb + 4 g + e) from the keys' bounds in vl ([4][32]), read four
// keys at a time before any test.
__device__ inline void mask_rows(f32x4 (&s)[2], const FM_LDS int* vl, int kbase, int i, const WideParams& p, int g) {
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int kl = 16 * jb + 4 * g;
    const i32x4 lts4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 0 * 32 + kl);
    const i32x4 lte4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 1 * 32 + kl);
    const i32x4 uts4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 2 * 32 + kl);
    const i32x4 ute4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 3 * 32 + kl);
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool m = hidden(p, i, kbase + kl + e, lts4[e], lte4[e], uts4[e], ute4[e]);
      out[e] = m ? kNegInf : s[jb][e];
    }
    s[jb] = out;
  }
}

// Classes of 32-key tile t for a query-major workgroup (rows [r0, r1), four
// waves of wr rows from r0) from its 64-key table entry; the tile counters
// take the entry's own class once (even t), at the 64-key width of the
// reported tile shape.
__device__ inline int qmajor_class(const int32_t* table, const WideParams& p, int r0, int r1, int wr, int t,
                                   unsigned& bits, unsigned (&cnt)[3]) {
  const BlockBounds bb = load_bounds(table + (long long)(t >> 1) * 8);
  const bool causal = p.causal != 0;
  const int c0 = 32 * t, c1 = min(p.Nk, c0 + 32);
  if ((t & 1) == 0) {
    const int e = tile_class(bb, r0, r1, c0, min(p.Nk, c0 + 64), causal);
    cnt[0] += e == 0;
    cnt[1] += e == 1;
    cnt[2] += e == 2;
  }
  const int wgc = tile_class(bb, r0, r1, c0, c1, causal);
  if (wgc == 0) return 0;
  const bool ragged = c1 - c0 < 32;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const int a0 = r0 + wr * ww;
    int cl = 0;
    if (a0 < p.Nq) {
      cl = tile_class(bb, a0, min(p.Nq, a0 + wr), c0, c1, causal);
      if (ragged && cl == 2) cl = 1;
    }
    bits |= (unsigned)cl << (2 * ww);
  }
  return wgc;
}

// Adds per-thread tile counts into the call's counters (once per workgroup).
__device__ inline void flush_counts(unsigned long long* counts, unsigned* wcount, const unsigned (&cnt)[3]) {
  if (counts == nullptr) return;
  atomicAdd(&wcount[0], cnt[0]);
  atomicAdd(&wcount[1], cnt[1]);
  atomicAdd(&wcount[2], cnt[2]);
  __syncthreads();
  if (threadIdx.x < 3) atomicAdd(counts + threadIdx.x, (unsigned long long)wcount[threadIdx.x]);
}

template <typename T, int D, int DV>
__global__ __launch_bounds__(256, (wide_occupancy<T, D, DV>())) void wide_fwd_kernel(WideParams p) {
  using X = W16<T>;
  using C = WFwd<T, D, DV>;
  constexpr int KC = X::KC, PF = wide_occupancy<T, D, DV>() > 1 ? 3 : 6, RB = C::RB;
  __shared__ __attribute__((aligned(16))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[C::STAGE];
  __shared__ int list_[C::LIST];
  __shared__ int wsum_[4];
  __shared__ unsigned wcount_[3];
  FM_LDS int* list = (FM_LDS int*)list_;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  int bh, blk;
  xcd_order((int)blockIdx.x, p.B * p.H, p.nqb, bh, blk);   // a head's blocks on one XCD
  const int qb = p.nqb - 1 - blk;                           // heavy (late) blocks first
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int r0 = qb * C::BR, r1 = min(Nq, r0 + C::BR);
  const int i0 = r0 + C::WR * w + n16;   // this lane's row in row block 0 (block rb: i0 + 16 rb)
  if (tid < 3) wcount_[tid] = 0;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(uniform_ptr(reinterpret_cast<const T*>(p.k) + kslice * D), (uint32_t)Nk * (uint32_t)(C::CPK * 16));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(uniform_ptr(reinterpret_cast<const T*>(p.v) + kslice * DV), (uint32_t)Nk * (uint32_t)(C::CPV * 16));
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  // bound vector w for wave w's share of each tile's loads
  const __amdgpu_buffer_rsrc_t rb = w == 0   ? vec_rsrc(p.lts, vrow, Nk, p.has_lt != 0)
                                    : w == 1 ? vec_rsrc(p.lte, vrow, Nk, p.has_lte != 0)
                                    : w == 2 ? vec_rsrc(p.uts, vrow, Nk, p.has_ut != 0)
                                             : vec_rsrc(p.ute, vrow, Nk, p.has_ut != 0);
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;

  typename X::op qf[RB][D / KC];
  f32x4 oacc[RB][DV / 16];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    load_row_ops<T, D>(qf[r], reinterpret_cast<const T*>(p.q) + qslice * D, i0 + 16 * r, Nq, g);
#pragma unroll
    for (int mb = 0; mb < DV / 16; ++mb) oacc[r][mb] = f32x4{};
    m_run[r] = kNegInf;
    l_run[r] = 0.f;
  }
  unsigned cnt3[3] = {0u, 0u, 0u};

  // K and the keys' bounds of a tile, and its V
  auto issue_k = [&](unsigned entry, auto stage_c) {
    FM_LDS char* st = (FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0);
    const int c0 = (int)(entry & 0xFFFFFFu) * C::BC;
    dma_rows<C::CPK>(rk, st, C::RSK, c0, w, lane);
    if (lane < 8) load_lds16(rb, st + C::KT + C::VT + w * C::BC * 4, (uint32_t)(c0 + 4 * lane) * 4u);
  };
  auto issue_v = [&](unsigned entry, auto stage_c) {
    FM_LDS char* st = (FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0);
    const int c0 = (int)(entry & 0xFFFFFFu) * C::BC;
    dma_rows<C::CPV>(rv, st + C::KT, C::RSV, c0, w, lane);
  };

  // the tile's scores and softmax leave P in s (kept across the second
  // barrier of the step), then O^T += V^T P^T
  f32x4 s[RB][2];
  auto scores = [&](unsigned entry, auto stage_c) {
    const int wc = (int)((entry >> (24 + 2 * w)) & 3u);
    if (wc == 0) return;
    const FM_LDS char* kst = (const FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0);
    const FM_LDS int* vl = (const FM_LDS int*)(kst + C::KT + C::VT);
    const int c0 = (int)(entry & 0xFFFFFFu) * C::BC;
    // S^T for the tile's two 16-key blocks (the two chains alternating),
    // each K operand for every row block
#pragma unroll
    for (int r = 0; r < RB; ++r) s[r][0] = s[r][1] = f32x4{};
    chain<2 * (D / KC), PF>([&](int t) { return row_op<T>(kst, C::RSK, 16 * (t & 1) + n16, t >> 1, g); },
                            [&](int t, typename X::op a) {
#pragma unroll
                              for (int r = 0; r < RB; ++r) s[r][t & 1] = X::mma(a, qf[r][t >> 1], s[r][t & 1]);
                            });
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (wc == 1) mask_rows(s[r], vl, c0, i0 + 16 * r, p, g);
      // online softmax, base 2: the offset (and O and the row sum with it)
      // moves only when some row's maximum outgrew it by more than the
      // slack; a row with nothing open keeps offset -inf
      float mx = fmaxf(fmaxf(fmaxf(s[r][0][0], s[r][0][1]), fmaxf(s[r][0][2], s[r][0][3])),
                       fmaxf(fmaxf(s[r][1][0], s[r][1][1]), fmaxf(s[r][1][2], s[r][1][3])));
      mx = max_x4(mx);
      if (__ballot((mx - m_run[r]) * p.sl2 > 8.0f) != 0) {
        const float m_new = fmaxf(m_run[r], mx);
        const float alpha = m_new == kNegInf ? 1.f : fast_exp2((m_run[r] - m_new) * p.sl2);
        l_run[r] *= alpha;
#pragma unroll
        for (int mb = 0; mb < DV / 16; ++mb) oacc[r][mb] *= alpha;
        m_run[r] = m_new;
      }
      const float msl = (m_run[r] == kNegInf ? 0.f : m_run[r]) * p.sl2;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv = fast_exp2(__builtin_fmaf(s[r][jb][e], p.sl2, -msl));
          // bf16: the row sum takes the rounded values the PV product uses
          if constexpr (!std::is_same<T, float>::value) pv = (float)(bf16)pv;
          s[r][jb][e] = pv;
          l_run[r] += pv;
        }
    }
  };
  auto product = [&](unsigned entry, auto stage_c) {
    const int wc = (int)((entry >> (24 + 2 * w)) & 3u);
    if (wc == 0) return;
    const FM_LDS char* vst = (const FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0) + C::KT;
    // O^T += V^T P^T over the tile's 32 keys, each V operand for every row block
    if constexpr (std::is_same<T, float>::value) {
      constexpr int NB = DV / 16;
      chain<NB * 8, PF>([&](int t) { return col_f32(vst, C::RSV, 16 * (t % NB) + n16, t / NB, g); },
                        [&](int t, float a) {
#pragma unroll
                          for (int r = 0; r < RB; ++r)
                            oacc[r][t % NB] = X::mma(a, acc_op<T>(s[r], t / NB), oacc[r][t % NB]);
                        });
    } else {
      bf16x8 pop[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) pop[r] = acc_op<T>(s[r], 0);
      chain<DV / 16, PF>([&](int t) { return col_tr(vst, C::RSV, 16 * t, lane); },
                         [&](int t, bf16x8 a) {
#pragma unroll
                           for (int r = 0; r < RB; ++r) oacc[r][t] = X::mma(a, pop[r], oacc[r][t]);
                         });
    }
  };

  const int nkt = (Nk + C::BC - 1) / C::BC;
  int cnt = 0;
  for (int base = 0; base < nkt; base += 256) {
    cnt = scan_chunk(list, (FM_LDS int*)wsum_, cnt, base, nkt,
                     [&](int t, unsigned& bits) { return qmajor_class(table, p, r0, r1, C::WR, t, bits, cnt3); });
    if (cnt > C::LIST - 256 || base + 256 >= nkt) {
      if constexpr (wide_occupancy<T, D, DV>() == 1) {
        // one workgroup per CU: nothing else hides a tile's load latency
        // (a K issue also moves the keys' bounds: one instruction more)
        run_list_kv<kDmaPerWave + 1, kDmaPerWave>(list, cnt, issue_k, issue_v, scores, product);
      } else {
        // two workgroups per CU: the other one's tiles hide it, and a second
        // barrier per tile measured slower
        run_list(
            list, cnt,
            [&](unsigned e, auto st) {
              issue_k(e, st);
              issue_v(e, st);
            },
            [&](unsigned e, auto st) {
              scores(e, st);
              product(e, st);
            });
      }
      cnt = 0;
    }
  }

#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int i = i0 + 16 * r;
    const float lt = sum_x4(l_run[r]);
    float inv, row_lse;
    finish_row(lt, m_run[r], p.scale, p.sink != nullptr ? p.sink[h] : kNegInf, p.sink != nullptr, inv, row_lse);
    if (i < Nq) {
      // lane: row i, columns 16 mb + 4 g + e
      T* og = reinterpret_cast<T*>(p.o) + (qslice + i) * DV + 4 * g;
#pragma unroll
      for (int mb = 0; mb < DV / 16; ++mb) {
        if constexpr (std::is_same<T, float>::value) {
          *reinterpret_cast<f32x4*>(og + 16 * mb) = oacc[r][mb] * inv;
        } else {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(oacc[r][mb][e] * inv);
          *reinterpret_cast<bf16x4*>(og + 16 * mb) = v4;
        }
      }
      if (g == 0) p.lse[qslice + i] = row_lse;
    }
  }
  flush_counts(p.counts, wcount_, cnt3);
}

// ---------------------------------------------------------------- dQ pass
// Workgroup: 64 query rows, every dQ column. Q and dO rows in registers;
// per visible 32-key tile (K and V in LDS):
//   S^T = K Q^T, dP^T = V dO^T, the tile's mask,
//   P = exp2(S scale log2e - LSE2), dS = P (dP - delta),
//   dQ^T += K^T dS^T.
// delta and LSE2 come from the preprocess. dQ sums over the keys in a fixed
// order in registers and is written once.
template <typename T, int D, int DV>
struct WDq {
  static constexpr int BR = 64, BC = 32;
  static constexpr int RSK = row_stride<T, D>(), RSV = row_stride<T, DV>();   // LDS row strides (bytes)
  static constexpr int CPK = D * (int)sizeof(T) / 16, CPV = DV * (int)sizeof(T) / 16;
  static constexpr int KT = BC * RSK, VT = BC * RSV;
  static constexpr int STAGE = KT + VT + 4 * BC * 4;
  static constexpr int LIST = 512;
};

template <typename T, int D, int DV>
__global__ __launch_bounds__(256, (wide_occupancy<T, D, DV>())) void wide_dq_kernel(WideParams p) {
  using X = W16<T>;
  using C = WDq<T, D, DV>;
  constexpr int KC = X::KC, PF = 6;
  __shared__ __attribute__((aligned(16))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[C::STAGE];
  __shared__ int list_[C::LIST];
  __shared__ int wsum_[4];
  FM_LDS int* list = (FM_LDS int*)list_;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  int bh, blk;
  xcd_order((int)blockIdx.x, p.B * p.H, p.nqb, bh, blk);
  const int qb = p.nqb - 1 - blk;
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int r0 = qb * C::BR, r1 = min(Nq, r0 + C::BR);
  const int i = r0 + 16 * w + n16;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(uniform_ptr(reinterpret_cast<const T*>(p.k) + kslice * D), (uint32_t)Nk * (uint32_t)(C::CPK * 16));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(uniform_ptr(reinterpret_cast<const T*>(p.v) + kslice * DV), (uint32_t)Nk * (uint32_t)(C::CPV * 16));
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  const __amdgpu_buffer_rsrc_t rb = w == 0   ? vec_rsrc(p.lts, vrow, Nk, p.has_lt != 0)
                                    : w == 1 ? vec_rsrc(p.lte, vrow, Nk, p.has_lte != 0)
                                    : w == 2 ? vec_rsrc(p.uts, vrow, Nk, p.has_ut != 0)
                                             : vec_rsrc(p.ute, vrow, Nk, p.has_ut != 0);
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;

  typename X::op qf[D / KC], dof[DV / KC];
  load_row_ops<T, D>(qf, reinterpret_cast<const T*>(p.q) + qslice * D, i, Nq, g);
  load_row_ops<T, DV>(dof, reinterpret_cast<const T*>(p.dout) + qslice * DV, i, Nq, g);
  // a row past Nq gets LSE2 = +inf, so its P (and dQ, not stored) is 0
  const float lse2 = i < Nq ? p.lse2[qslice + i] : __builtin_inff();
  const float delta = i < Nq ? p.delta[qslice + i] : 0.f;
  f32x4 dq[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) dq[mb] = f32x4{};
  float pd = 0.f;   // this lane's part of rowsum(dS)
  unsigned cnt3[3] = {0u, 0u, 0u};   // (the dK/dV pass reports the tiles)

  auto issue = [&](unsigned entry, auto stage_c) {
    FM_LDS char* st = (FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0);
    const int c0 = (int)(entry & 0xFFFFFFu) * C::BC;
    dma_rows<C::CPK>(rk, st, C::RSK, c0, w, lane);
    dma_rows<C::CPV>(rv, st + C::KT, C::RSV, c0, w, lane);
    if (lane < 8) load_lds16(rb, st + C::KT + C::VT + w * C::BC * 4, (uint32_t)(c0 + 4 * lane) * 4u);
  };

  auto compute = [&](unsigned entry, auto stage_c) {
    const int wc = (int)((entry >> (24 + 2 * w)) & 3u);
    if (wc == 0) return;
    const FM_LDS char* kst = (const FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0);
    const FM_LDS char* vst = kst + C::KT;
    const FM_LDS int* vl = (const FM_LDS int*)(kst + C::KT + C::VT);
    const int c0 = (int)(entry & 0xFFFFFFu) * C::BC;
    // S^T and dP^T for the tile's two 16-key blocks: step u of a product is
    // block u & 1, operand step u >> 1; the two products alternate while
    // both have steps left
    constexpr int NS = 2 * (D / KC), ND = 2 * (DV / KC), NMIN = NS < ND ? NS : ND;
    auto is_dp = [](int t) { return t < 2 * NMIN ? (t & 1) != 0 : ND > NS; };
    auto ustep = [](int t) { return t < 2 * NMIN ? t >> 1 : t - NMIN; };
    f32x4 s[2] = {f32x4{}, f32x4{}}, dp[2] = {f32x4{}, f32x4{}};
    chain<NS + ND, PF>(
        [&](int t) {
          const int u = ustep(t);
          return is_dp(t) ? row_op<T>(vst, C::RSV, 16 * (u & 1) + n16, u >> 1, g)
                          : row_op<T>(kst, C::RSK, 16 * (u & 1) + n16, u >> 1, g);
        },
        [&](int t, typename X::op a) {
          const int u = ustep(t);
          if (is_dp(t)) dp[u & 1] = X::mma(a, dof[u >> 1], dp[u & 1]);
          else s[u & 1] = X::mma(a, qf[u >> 1], s[u & 1]);
        });
    if (wc == 1) mask_rows(s, vl, c0, i, p, g);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ds = fast_exp2(__builtin_fmaf(s[jb][e], p.sl2, -lse2)) * (dp[jb][e] - delta);
        pd += ds;
        s[jb][e] = ds;
      }
    // dQ^T += K^T dS^T over the tile's 32 keys (dQ takes the scale at the end)
    if constexpr (std::is_same<T, float>::value) {
      constexpr int NB = D / 16;
      chain<NB * 8, PF>([&](int t) { return col_f32(kst, C::RSK, 16 * (t % NB) + n16, t / NB, g); },
                        [&](int t, float a) { dq[t % NB] = X::mma(a, acc_op<T>(s, t / NB), dq[t % NB]); });
    } else {
      const bf16x8 dsop = acc_op<T>(s, 0);
      chain<D / 16, PF>([&](int t) { return col_tr(kst, C::RSK, 16 * t, lane); },
                        [&](int t, bf16x8 a) { dq[t] = X::mma(a, dsop, dq[t]); });
    }
  };

  const int nkt = (Nk + C::BC - 1) / C::BC;
  int cnt = 0;
  for (int base = 0; base < nkt; base += 256) {
    cnt = scan_chunk(list, (FM_LDS int*)wsum_, cnt, base, nkt,
                     [&](int t, unsigned& bits) { return qmajor_class(table, p, r0, r1, 16, t, bits, cnt3); });
    if (cnt > C::LIST - 256 || base + 256 >= nkt) {
      run_list(list, cnt, issue, compute);
      cnt = 0;
    }
  }

  pd = sum_x4(pd);
  if (p.pdsum != nullptr && i < Nq && g == 0) p.pdsum[qslice + i] = pd;
  if (i < Nq) {
    T* dqg = reinterpret_cast<T*>(p.dq) + (qslice + i) * D + 4 * g;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4*>(dqg + 16 * mb) = dq[mb] * p.scale;
      } else {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)(dq[mb][e] * p.scale);
        *reinterpret_cast<bf16x4*>(dqg + 16 * mb) = v4;
      }
    }
  }
}

// ---------------------------------------------------------------- dK/dV pass
// Workgroup: 64 keys (16 per wave), every dK and dV column. K and V rows of
// the lane's key in registers; per visible 32-row query step (Q, dO, LSE2
// and delta in LDS):
//   S = Q K^T, dP = dO V^T, the mask from the key's own bounds,
//   P = exp2(S scale log2e - LSE2), dS = P (dP - delta),
//   dV^T += dO^T P and dK^T += Q^T dS (dK takes the scale once, at the end).
// At d = dv = 512 the key's operands (128 registers) and the dK and dV
// accumulators (256) fill most of a lane's 512; one 8-byte value of the
// prologue goes to scratch until the epilogue.
template <typename T, int D, int DV>
struct WKv {
  static constexpr int BKC = 64, BQ = 32;
  static constexpr int RSQ = row_stride<T, D>(), RSO = row_stride<T, DV>();   // LDS row strides (bytes)
  static constexpr int CPQ = D * (int)sizeof(T) / 16, CPO = DV * (int)sizeof(T) / 16;
  static constexpr int QT = BQ * RSQ, OT = BQ * RSO;
  static constexpr int STAGE = QT + OT + 2 * BQ * 4;   // Q, dO, LSE2, delta
  static constexpr int LIST = 512;
};

template <typename T, int D, int DV>
__global__ __launch_bounds__(256, (wide_occupancy<T, D, DV>())) void wide_dkdv_kernel(WideParams p) {
  using X = W16<T>;
  using C = WKv<T, D, DV>;
  constexpr int KC = X::KC, PF = 4;
  __shared__ __attribute__((aligned(16))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[C::STAGE];
  __shared__ int list_[C::LIST];
  __shared__ int wsum_[4];
  __shared__ unsigned wcount_[3];
  FM_LDS int* list = (FM_LDS int*)list_;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  const int BH = p.B * p.H;
  int bh, kb;
  xcd_order((int)blockIdx.x, BH, p.nkb64, bh, kb);   // early (heavy) key blocks first
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const bool causal = p.causal != 0;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int c0 = kb * C::BKC, c1 = min(Nk, c0 + C::BKC);
  const int wc0 = c0 + 16 * w;
  const int j = wc0 + n16;   // this lane's key
  if (tid < 3) wcount_[tid] = 0;
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(uniform_ptr(reinterpret_cast<const T*>(p.q) + qslice * D), (uint32_t)Nq * (uint32_t)(C::CPQ * 16));
  const __amdgpu_buffer_rsrc_t rdo =
      make_rsrc(uniform_ptr(reinterpret_cast<const T*>(p.dout) + qslice * DV), (uint32_t)Nq * (uint32_t)(C::CPO * 16));
  // wave 0 moves each step's LSE2 values, wave 1 its delta values
  const __amdgpu_buffer_rsrc_t rrow = make_rsrc(uniform_ptr(w == 0 ? p.lse2 + qslice : p.delta + qslice),
                                                (uint32_t)Nq * 4u);

  // the key's rows as B operands
  typename X::op kr[D / KC], vr[DV / KC];
  load_row_ops<T, D>(kr, reinterpret_cast<const T*>(p.k) + kslice * D, j, Nk, g);
  load_row_ops<T, DV>(vr, reinterpret_cast<const T*>(p.v) + kslice * DV, j, Nk, g);
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  int k_lts = 0, k_lte = 0, k_uts = 0, k_ute = 0;
  if (j < Nk) {
    if (p.has_lt) {
      k_lts = p.lts[vrow + j];
      k_lte = p.has_lte ? p.lte[vrow + j] : Nq;
    }
    if (p.has_ut) {
      k_uts = p.uts[vrow + j];
      k_ute = p.ute[vrow + j];
    }
  }
  f32x4 dkacc[D / 16], dvacc[DV / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) dkacc[mb] = f32x4{};
#pragma unroll
  for (int mb = 0; mb < DV / 16; ++mb) dvacc[mb] = f32x4{};
  // bounds of the workgroup's 64 keys (one table entry); a wave's 16 keys
  // lie inside them, so the same bounds classify its part (possibly as
  // partial where its own keys alone would not be)
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;
  const BlockBounds kbnd = load_bounds(table + (long long)kb * 8);
  unsigned cnt3[3] = {0u, 0u, 0u};

  auto cls = [&](int t, unsigned& bits) {
    const int q0 = 32 * t, q1 = min(Nq, q0 + 32);
    const int wgc = tile_class(kbnd, q0, q1, c0, c1, causal);
    cnt3[0] += wgc == 0;
    cnt3[1] += wgc == 1;
    cnt3[2] += wgc == 2;
    if (wgc == 0) return 0;
    const bool ragged = q1 - q0 < 32 || c1 - c0 < C::BKC;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const int a0 = c0 + 16 * ww;
      int cl = 0;
      if (a0 < Nk) {
        cl = tile_class(kbnd, q0, q1, a0, min(Nk, a0 + 16), causal);
        if (ragged && cl == 2) cl = 1;
      }
      bits |= (unsigned)cl << (2 * ww);
    }
    return wgc;
  };

  auto issue = [&](unsigned entry, auto stage_c) {
    FM_LDS char* st = (FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0);
    const int q0 = (int)(entry & 0xFFFFFFu) * C::BQ;
    dma_rows<C::CPQ>(rq, st, C::RSQ, q0, w, lane);
    dma_rows<C::CPO>(rdo, st + C::QT, C::RSO, q0, w, lane);
    if (w < 2 && lane < 8) load_lds16(rrow, st + C::QT + C::OT + w * C::BQ * 4, (uint32_t)(q0 + 4 * lane) * 4u);
  };

  auto compute = [&](unsigned entry, auto stage_c) {
    const int wc = (int)((entry >> (24 + 2 * w)) & 3u);
    if (wc == 0) return;
    const FM_LDS char* qst = (const FM_LDS char*)(decltype(stage_c)::value ? stage1 : stage0);
    const FM_LDS char* dost = qst + C::QT;
    const FM_LDS float* lse_l = (const FM_LDS float*)(qst + C::QT + C::OT);
    const FM_LDS float* del_l = lse_l + C::BQ;
    const int q0 = (int)(entry & 0xFFFFFFu) * C::BQ;
    // S and dP for the step's two 16-row halves (lane: key j; rows
    // 16 mt + 4 g + e), the two products alternating while both have steps
    // left
    constexpr int NS = 2 * (D / KC), ND = 2 * (DV / KC), NMIN = NS < ND ? NS : ND;
    auto is_dp = [](int t) { return t < 2 * NMIN ? (t & 1) != 0 : ND > NS; };
    auto ustep = [](int t) { return t < 2 * NMIN ? t >> 1 : t - NMIN; };
    f32x4 s[2] = {f32x4{}, f32x4{}}, dp[2] = {f32x4{}, f32x4{}};
    chain<NS + ND, PF>(
        [&](int t) {
          const int u = ustep(t);
          return is_dp(t) ? row_op<T>(dost, C::RSO, 16 * (u & 1) + n16, u >> 1, g)
                          : row_op<T>(qst, C::RSQ, 16 * (u & 1) + n16, u >> 1, g);
        },
        [&](int t, typename X::op a) {
          const int u = ustep(t);
          if (is_dp(t)) dp[u & 1] = X::mma(a, vr[u >> 1], dp[u & 1]);
          else s[u & 1] = X::mma(a, kr[u >> 1], s[u & 1]);
        });
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int il = 16 * mt + 4 * g;
      const f32x4 lse4 = *reinterpret_cast<const FM_LDS f32x4*>(lse_l + il);
      const f32x4 del4 = *reinterpret_cast<const FM_LDS f32x4*>(del_l + il);
      f32x4 pv4, ds4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool m = (wc == 1) & hidden(p, q0 + il + e, j, k_lts, k_lte, k_uts, k_ute);
        const float sv = m ? kNegInf : s[mt][e];
        const float pv = fast_exp2(__builtin_fmaf(sv, p.sl2, -lse4[e]));
        pv4[e] = pv;
        ds4[e] = pv * (dp[mt][e] - del4[e]);   // dS; the scale goes on dK at the end
      }
      s[mt] = pv4;
      dp[mt] = ds4;
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the step's 32 rows, the two
    // products alternating while both have steps left; step u of a product
    // is column block u % NB, row step u / NB
    constexpr int NST = 32 / KC, NKB = D / 16, NVB = DV / 16;
    constexpr int NK = NKB * NST, NV = NVB * NST, NM = NK < NV ? NK : NV;
    auto is_k = [](int t) { return t < 2 * NM ? (t & 1) != 0 : NK > NV; };
    auto kstep = [](int t) { return t < 2 * NM ? t >> 1 : t - NM; };
    if constexpr (std::is_same<T, float>::value) {
      chain<NK + NV, PF>(
          [&](int t) {
            const int u = kstep(t);
            return is_k(t) ? col_f32(qst, C::RSQ, 16 * (u % NKB) + n16, u / NKB, g)
                           : col_f32(dost, C::RSO, 16 * (u % NVB) + n16, u / NVB, g);
          },
          [&](int t, float a) {
            const int u = kstep(t);
            if (is_k(t)) dkacc[u % NKB] = X::mma(a, acc_op<T>(dp, u / NKB), dkacc[u % NKB]);
            else dvacc[u % NVB] = X::mma(a, acc_op<T>(s, u / NVB), dvacc[u % NVB]);
          });
    } else {
      const bf16x8 pop = acc_op<T>(s, 0), dsop = acc_op<T>(dp, 0);
      chain<NK + NV, PF>(
          [&](int t) {
            const int u = kstep(t);
            return is_k(t) ? col_tr(qst, C::RSQ, 16 * u, lane) : col_tr(dost, C::RSO, 16 * u, lane);
          },
          [&](int t, bf16x8 a) {
            const int u = kstep(t);
            if (is_k(t)) dkacc[u] = X::mma(a, dsop, dkacc[u]);
            else dvacc[u] = X::mma(a, pop, dvacc[u]);
          });
    }
  };

  const int nqt = (Nq + C::BQ - 1) / C::BQ;
  int cnt = 0;
  for (int base = 0; base < nqt; base += 256) {
    cnt = scan_chunk(list, (FM_LDS int*)wsum_, cnt, base, nqt, cls);
    if (cnt > C::LIST - 256 || base + 256 >= nqt) {
      run_list(list, cnt, issue, compute);
      cnt = 0;
    }
  }

  // lane: key j, dK and dV columns 16 mb + 4 g + e
  if (j < Nk) {
    T* dkg = reinterpret_cast<T*>(p.dk) + (kslice + j) * D + 4 * g;
    T* dvg = reinterpret_cast<T*>(p.dv) + (kslice + j) * DV + 4 * g;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4*>(dkg + 16 * mb) = dkacc[mb] * p.scale;
      } else {
        bf16x4 k4;
#pragma unroll
        for (int e = 0; e < 4; ++e) k4[e] = (bf16)(dkacc[mb][e] * p.scale);
        *reinterpret_cast<bf16x4*>(dkg + 16 * mb) = k4;
      }
    }
#pragma unroll
    for (int mb = 0; mb < DV / 16; ++mb) {
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4*>(dvg + 16 * mb) = dvacc[mb];
      } else {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)dvacc[mb][e];
        *reinterpret_cast<bf16x4*>(dvg + 16 * mb) = v4;
      }
    }
  }
  flush_counts(p.counts, wcount_, cnt3);
}

// ---------------------------------------------------------------- launch

static WideParams wide_params(const AttnArgs& a) {
  WideParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.lts = a.mask.lts;
  p.lte = a.mask.lte;
  p.uts = a.mask.uts;
  p.ute = a.mask.ute;
  p.table = a.table;
  p.o = a.out;
  p.lse = a.lse_out;
  p.sink = a.sink;
  p.counts = a.tile_counts;
  p.dout = a.dout;
  p.lse2 = a.lse2;
  p.delta = a.delta;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv_out;
  p.B = a.B;
  p.H = a.H;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.hm = a.mask.hm;
  p.causal = a.mask.causal;
  p.has_lt = a.mask.lts != nullptr;
  p.has_lte = a.mask.lts != nullptr && a.mask.lte != nullptr;
  p.has_ut = !a.mask.causal && a.mask.uts != nullptr && a.mask.ute != nullptr;
  p.scale = a.scale;
  p.sl2 = a.scale * kLog2e;
  p.nkb64 = (a.Nk + kTableBlock - 1) / kTableBlock;
  return p;
}

template <typename T, int D, int DV>
static hipError_t launch_wide_fwd_t(const AttnArgs& a, hipStream_t stream) {
  WideParams p = wide_params(a);
  p.nqb = (a.Nq + WFwd<T, D, DV>::BR - 1) / WFwd<T, D, DV>::BR;
  const long long grid = (long long)a.B * a.H * p.nqb;
  hipLaunchKernelGGL((wide_fwd_kernel<T, D, DV>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t launch_wide_bwd_t(const AttnArgs& a, hipStream_t stream) {
  WideParams p = wide_params(a);
  p.pdsum = a.sink != nullptr ? a.pdsum : nullptr;
  p.nqb = (a.Nq + 63) / 64;
  long long grid = (long long)a.B * a.H * p.nqb;
  hipLaunchKernelGGL((wide_dq_kernel<T, D, DV>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  grid = (long long)a.B * a.H * p.nkb64;
  hipLaunchKernelGGL((wide_dkdv_kernel<T, D, DV>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// the shapes compiled in (kept in step with wide_fwd_dims() and wide_bwd_dims())
hipError_t launch_wide_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.is_bf16 && a.d == 512 && a.dv == 512) return launch_wide_fwd_t<bf16, 512, 512>(a, stream);
  if (a.is_bf16 && a.d == 256 && a.dv == 256) return launch_wide_fwd_t<bf16, 256, 256>(a, stream);
  if (a.is_bf16 && a.d == 192 && a.dv == 128) return launch_wide_fwd_t<bf16, 192, 128>(a, stream);
  if (!a.is_bf16 && a.d == 256 && a.dv == 256) return launch_wide_fwd_t<float, 256, 256>(a, stream);
  if (!a.is_bf16 && a.d == 192 && a.dv == 128) return launch_wide_fwd_t<float, 192, 128>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_wide_bwd(const AttnArgs& a, hipStream_t stream) {
  if (a.is_bf16 && a.d == 512 && a.dv == 512) return launch_wide_bwd_t<bf16, 512, 512>(a, stream);
  if (a.is_bf16 && a.d == 256 && a.dv == 256) return launch_wide_bwd_t<bf16, 256, 256>(a, stream);
  if (!a.is_bf16 && a.d == 256 && a.dv == 256) return launch_wide_bwd_t<float, 256, 256>(a, stream);
  if (!a.is_bf16 && a.d == 192 && a.dv == 128) return launch_wide_bwd_t<float, 192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fm
