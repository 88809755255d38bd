// Wide head dims: bf16 with d = dv = 512 and fp32 with d = dv = 256.
//
// The pages list large head dims among the method's features (FlashMask
// README, "News" and "Key Features"); the computation is the same as at
// the narrower dims (FlashMask README, "Formulation": S = scale Q K^T plus
// the column-wise mask bias, softmax, P V; and its gradient, with
// dS = P (dP - delta)), only the rows are wider.
//
// At these widths one row of Q, K, V or dO is 1 KiB, so a lane that keeps
// its row as MFMA operands spends 128 registers on it (of 512 at one wave
// per SIMD). The kernels keep the decomposition of the narrower ones
// (query-major forward and dQ pass, key-major dK/dV pass, the same per-tile
// classification from the key-block table) and bound their accumulators by
// splitting the output columns into chunks, one workgroup per chunk; the
// workgroups of one tile's chunks each form its scores (and dP) again.
// Tiles go through LDS with plain 16-byte loads, one stage, no pipelining.
//
// MFMA in the forward and dQ pass: v_mfma_f32_32x32x16_bf16 (bf16) and
// v_mfma_f32_32x32x2_f32 (fp32), both with lane (n = lane % 32, k-group =
// lane / 32) operands and the 32x32 accumulator layout in which lane (n, h)
// holds M index 8 * (r / 4) + 4 * h + r % 4 in register r. A product whose
// contraction runs over such an accumulator's M index (P V, dS K) takes the
// other operand's rows in that same order. The dK/dV pass uses the 16x16
// forms instead (its section says why and how).
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

// ---------------------------------------------------------------- element types
template <typename T>
struct Wt;
template <>
struct Wt<float> {
  using op = float;
  static constexpr int KC = 2;   // contraction depth of one MFMA
  __device__ static f32x16 mma(float a, float b, f32x16 c) { return mfma32f(a, b, c); }
};
template <>
struct Wt<bf16> {
  using op = bf16x8;
  static constexpr int KC = 16;
  __device__ static f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) { return mfma32(a, b, c); }
};

// LDS row stride in elements: 16 bytes of padding keep rows 16-byte aligned
// and move each row 4 banks on
template <typename T, int W>
constexpr int lds_stride() {
  return W + 16 / (int)sizeof(T);
}

// Operands of `row` (W wide, in global memory) for a lane's n index: step c
// holds elements [c KC + h KC / 2, + KC / 2). Rows at or past n_rows read 0.
template <typename T, int W>
__device__ inline void load_row_ops(typename Wt<T>::op (&r)[W / Wt<T>::KC], const T* g, int row,
                                    int n_rows, int hh) {
  constexpr int KC = Wt<T>::KC;
  const bool ok = row < n_rows;
#pragma unroll
  for (int c = 0; c < W / KC; ++c) {
    if constexpr (std::is_same<T, float>::value) {
      r[c] = ok ? g[(long long)row * W + KC * c + hh] : 0.f;
    } else {
      r[c] = ok ? *reinterpret_cast<const bf16x8*>(g + (long long)row * W + KC * c + 8 * hh) : bf16x8{};
    }
  }
}

// The row operand of LDS row `row` at step c.
template <typename T>
__device__ inline typename Wt<T>::op row_op(const FM_LDS T* t, int rs, int row, int c, int hh) {
  if constexpr (std::is_same<T, float>::value) {
    return t[row * rs + 2 * c + hh];
  } else {
    return *reinterpret_cast<const FM_LDS bf16x8*>(t + row * rs + 16 * c + 8 * hh);
  }
}

// Column n of LDS rows [r0, r0 + 32) at step s of a contraction over those
// rows in accumulator order.
template <typename T>
__device__ inline typename Wt<T>::op col_op(const FM_LDS T* t, int rs, int r0, int n, int s, int hh) {
  if constexpr (std::is_same<T, float>::value) {
    return t[(r0 + 8 * (s / 4) + 4 * hh + (s % 4)) * rs + n];
  } else {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[(r0 + 16 * s + 8 * (e / 4) + 4 * hh + (e % 4)) * rs + n];
    return v;
  }
}

// Step s of an accumulator as the operand whose k runs over its M index
// (bf16: rounded to nearest even).
template <typename T>
__device__ inline typename Wt<T>::op acc_op(const f32x16& a, int s) {
  if constexpr (std::is_same<T, float>::value) {
    return a[s];
  } else {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)a[8 * s + e];
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
  decltype(rd(0)) ring[PF];
#pragma unroll
  for (int t = 0; t < PF; ++t) ring[t] = rd(t);
#pragma unroll
  for (int t = 0; t < N; ++t) {
    const auto a = ring[t % PF];
    if (t + PF < N) ring[t % PF] = rd(t + PF);
    step(t, a);
    __builtin_amdgcn_sched_barrier(0x406);
  }
}

// Rows [g0, g0 + R) of a row-major global matrix (row stride gw elements),
// columns [col0, col0 + W), into LDS with row stride rs; rows at or past
// n_rows as zeros. 16-byte pieces spread over the workgroup's 256 threads.
template <typename T, int R, int W>
__device__ inline void stage(FM_LDS T* t, int rs, const T* g, long long gw, int col0, int g0, int n_rows) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int CPR = W / EPC;
  for (int x = threadIdx.x; x < R * CPR; x += 256) {
    const int row = x / CPR, c = x % CPR;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (g0 + row < n_rows) v = *reinterpret_cast<const u32x4*>(g + (long long)(g0 + row) * gw + col0 + c * EPC);
    *reinterpret_cast<FM_LDS u32x4*>(t + row * rs + c * EPC) = v;
  }
}

// Key bounds of keys [c0, c0 + 64) into vl ([4][64]: LTS, LTE, UTS, UTE),
// absent vectors as 0 (the has_* flags gate their use).
__device__ inline void stage_bounds(FM_LDS int* vl, const WideParams& p, long long vrow, int c0) {
  const int vsel = threadIdx.x >> 6, kk = threadIdx.x & 63;
  const int32_t* src = vsel == 0 ? p.lts : vsel == 1 ? p.lte : vsel == 2 ? p.uts : p.ute;
  const bool present = src != nullptr && (vsel < 2 ? p.has_lt : p.has_ut);
  vl[vsel * 64 + kk] = (present && c0 + kk < p.Nk) ? src[vrow + c0 + kk] : 0;
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

// -inf on the hidden elements of an S^T block (keys x rows) of a query-major
// kernel: lane row i, key kbase + kl0 + M index; bounds from vl, read four
// keys at a time before any test.
__device__ inline void mask_st(f32x16& s, const FM_LDS int* vl, int kl0, int kbase, int i,
                               const WideParams& p, int hh) {
  f32x16 out;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int kl = kl0 + 8 * g + 4 * hh;
    const i32x4 lts4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 0 * 64 + kl);
    const i32x4 lte4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 1 * 64 + kl);
    const i32x4 uts4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 2 * 64 + kl);
    const i32x4 ute4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 3 * 64 + kl);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool m = hidden(p, i, kbase + kl + e, lts4[e], lte4[e], uts4[e], ute4[e]);
      out[4 * g + e] = m ? kNegInf : s[4 * g + e];
    }
  }
  s = out;
}

// Query-major item order: chunk fastest (the chunks of one query block read
// the same K tiles together), heavy (late) query blocks first.
__device__ inline void qmajor_item(int nch, const WideParams& p, int& ch, int& bh, int& qb) {
  const int t = (int)blockIdx.x;
  ch = t % nch;
  const int rest = t / nch;
  const int BH = p.B * p.H;
  bh = rest % BH;
  qb = p.nqb - 1 - rest / BH;
}

// ---------------------------------------------------------------- forward
// Workgroup: 128 query rows (32 per wave), output columns
// [ch DVC, (ch + 1) DVC) of O. Per visible 64-key tile: S^T = K Q^T (Q in
// registers), the tile's mask, online softmax, O^T += V^T P^T.
template <typename T, int D, int DV, int DVC>
__global__ __launch_bounds__(256, 1) void wide_fwd_kernel(WideParams p) {
  using X = Wt<T>;
  constexpr int BC = 64, BR = 128, NCH = DV / DVC, KC = X::KC;
  constexpr int KS = lds_stride<T, D>(), VS = lds_stride<T, DVC>();
  __shared__ __attribute__((aligned(16))) T ks_[BC * KS];
  __shared__ __attribute__((aligned(16))) T vs_[BC * VS];
  __shared__ int vl_[4 * 64];
  FM_LDS T* ks = (FM_LDS T*)ks_;
  FM_LDS T* vs = (FM_LDS T*)vs_;
  FM_LDS int* vl = (FM_LDS int*)vl_;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  int ch, bh, qb;
  qmajor_item(NCH, p, ch, bh, qb);
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const bool causal = p.causal != 0;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int r0 = qb * BR, r1 = min(Nq, r0 + BR);
  const int i = r0 + 32 * w + l32;
  const T* kg = reinterpret_cast<const T*>(p.k) + kslice * D;
  const T* vg = reinterpret_cast<const T*>(p.v) + kslice * DV;
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;

  typename X::op qf[D / KC];
  load_row_ops<T, D>(qf, reinterpret_cast<const T*>(p.q) + qslice * D, i, Nq, hh);
  f32x16 oacc[DVC / 32];
#pragma unroll
  for (int mb = 0; mb < DVC / 32; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  unsigned cnt0 = 0, cnt1 = 0, cnt2 = 0;

  for (int kb = 0; kb < p.nkb64; ++kb) {
    const BlockBounds bb = load_bounds(table + (long long)kb * 8);
    const int c0 = kb * BC, c1 = min(Nk, c0 + BC);
    const int wgc = tile_class(bb, r0, r1, c0, c1, causal);
    cnt0 += wgc == 0;
    cnt1 += wgc == 1;
    cnt2 += wgc == 2;
    if (wgc == 0) continue;
    int wc = 0;
    const int a0 = r0 + 32 * w;
    if (a0 < Nq) {
      wc = tile_class(bb, a0, min(Nq, a0 + 32), c0, c1, causal);
      if (c1 - c0 < BC && wc == 2) wc = 1;
    }
    __syncthreads();   // the last tile's readers are done
    stage<T, BC, D>(ks, KS, kg, D, 0, c0, Nk);
    stage<T, BC, DVC>(vs, VS, vg, DV, ch * DVC, c0, Nk);
    stage_bounds(vl, p, vrow, c0);
    __syncthreads();
    if (wc == 0) continue;
    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      s[jb] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / KC; ++c) s[jb] = X::mma(row_op<T>(ks, KS, jb * 32 + l32, c, hh), qf[c], s[jb]);
      if (wc == 1) mask_st(s[jb], vl, jb * 32, c0, i, p, hh);
    }
    // online softmax, base 2; a row with nothing open keeps offset -inf
    const float mx = max_x32(max_acc(s));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f((m_run - m_use) * p.sl2);
    const float msl = m_use * p.sl2;
    float rs = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2f(__builtin_fmaf(s[jb][r], p.sl2, -msl));
        // bf16: the row sum takes the rounded values the PV product uses
        if constexpr (!std::is_same<T, float>::value) pv = (float)(bf16)pv;
        s[jb][r] = pv;
        rs += pv;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < DVC / 32; ++mb) oacc[mb] *= alpha;
    // O^T += V^T P^T over the tile's 64 keys
#pragma unroll
    for (int mb = 0; mb < DVC / 32; ++mb)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int st = 0; st < 32 / KC; ++st)
          oacc[mb] = X::mma(col_op<T>(vs, VS, jb * 32, 32 * mb + l32, st, hh), acc_op<T>(s[jb], st), oacc[mb]);
  }

  const float lt = sum_x32(l_run);
  float inv, row_lse;
  finish_row(lt, m_run, p.scale, p.sink != nullptr ? p.sink[h] : kNegInf, p.sink != nullptr, inv, row_lse);
  if (i < Nq) {
    T* og = reinterpret_cast<T*>(p.o) + (qslice + i) * DV + ch * DVC;
#pragma unroll
    for (int mb = 0; mb < DVC / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // this lane's columns 32 mb + 8 g + 4 h + e, e < 4
        if constexpr (std::is_same<T, float>::value) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = oacc[mb][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(og + 32 * mb + 8 * g + 4 * hh) = v4;
        } else {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(oacc[mb][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(og + 32 * mb + 8 * g + 4 * hh) = v4;
        }
      }
    if (ch == 0 && hh == 0) p.lse[qslice + i] = row_lse;
  }
  if (ch == 0 && p.counts != nullptr && tid == 0) {
    atomicAdd(p.counts + 0, (unsigned long long)cnt0);
    atomicAdd(p.counts + 1, (unsigned long long)cnt1);
    atomicAdd(p.counts + 2, (unsigned long long)cnt2);
  }
}

// ---------------------------------------------------------------- dQ pass
// Workgroup: 128 query rows, dQ columns [ch DC, (ch + 1) DC). Q and dO rows
// in registers; per visible 64-key tile (K and V in LDS):
//   S^T = K Q^T, dP^T = V dO^T, the tile's mask,
//   P = exp2(S scale log2e - LSE2), dS = P (dP - delta),
//   dQ^T += K^T dS^T (this chunk's columns of K).
// delta and LSE2 come from the preprocess. dQ sums over the keys in a fixed
// order in registers and is written once.
template <typename T, int D, int DV, int DC>
__global__ __launch_bounds__(256, 1) void wide_dq_kernel(WideParams p) {
  using X = Wt<T>;
  constexpr int BC = 64, BR = 128, NCH = D / DC, KC = X::KC;
  constexpr int KS = lds_stride<T, D>(), VS = lds_stride<T, DV>();
  __shared__ __attribute__((aligned(16))) T ks_[BC * KS];
  __shared__ __attribute__((aligned(16))) T vs_[BC * VS];
  __shared__ int vl_[4 * 64];
  FM_LDS T* ks = (FM_LDS T*)ks_;
  FM_LDS T* vs = (FM_LDS T*)vs_;
  FM_LDS int* vl = (FM_LDS int*)vl_;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  int ch, bh, qb;
  qmajor_item(NCH, p, ch, bh, qb);
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const bool causal = p.causal != 0;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int r0 = qb * BR, r1 = min(Nq, r0 + BR);
  const int i = r0 + 32 * w + l32;
  const T* kg = reinterpret_cast<const T*>(p.k) + kslice * D;
  const T* vg = reinterpret_cast<const T*>(p.v) + kslice * DV;
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;

  typename X::op qf[D / KC], dof[DV / KC];
  load_row_ops<T, D>(qf, reinterpret_cast<const T*>(p.q) + qslice * D, i, Nq, hh);
  load_row_ops<T, DV>(dof, reinterpret_cast<const T*>(p.dout) + qslice * DV, i, Nq, hh);
  // a row past Nq gets LSE2 = +inf, so its P (and dQ, not stored) is 0
  const float lse2 = i < Nq ? p.lse2[qslice + i] : __builtin_inff();
  const float delta = i < Nq ? p.delta[qslice + i] : 0.f;
  f32x16 dq[DC / 32];
#pragma unroll
  for (int mb = 0; mb < DC / 32; ++mb) dq[mb] = f32x16{};
  float pd = 0.f;   // this lane's part of rowsum(dS)

  for (int kb = 0; kb < p.nkb64; ++kb) {
    const BlockBounds bb = load_bounds(table + (long long)kb * 8);
    const int c0 = kb * BC, c1 = min(Nk, c0 + BC);
    if (tile_class(bb, r0, r1, c0, c1, causal) == 0) continue;
    int wc = 0;
    const int a0 = r0 + 32 * w;
    if (a0 < Nq) {
      wc = tile_class(bb, a0, min(Nq, a0 + 32), c0, c1, causal);
      if (c1 - c0 < BC && wc == 2) wc = 1;
    }
    __syncthreads();
    stage<T, BC, D>(ks, KS, kg, D, 0, c0, Nk);
    stage<T, BC, DV>(vs, VS, vg, DV, 0, c0, Nk);
    stage_bounds(vl, p, vrow, c0);
    __syncthreads();
    if (wc == 0) continue;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < D / KC; ++c) s = X::mma(row_op<T>(ks, KS, jb * 32 + l32, c, hh), qf[c], s);
#pragma unroll
      for (int c = 0; c < DV / KC; ++c) dp = X::mma(row_op<T>(vs, VS, jb * 32 + l32, c, hh), dof[c], dp);
      if (wc == 1) mask_st(s, vl, jb * 32, c0, i, p, hh);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ds = exp2f(__builtin_fmaf(s[r], p.sl2, -lse2)) * (dp[r] - delta);
        pd += ds;
        s[r] = ds;
      }
#pragma unroll
      for (int mb = 0; mb < DC / 32; ++mb)
#pragma unroll
        for (int st = 0; st < 32 / KC; ++st)
          dq[mb] = X::mma(col_op<T>(ks, KS, jb * 32, ch * DC + 32 * mb + l32, st, hh), acc_op<T>(s, st), dq[mb]);
    }
  }

  pd = sum_x32(pd);
  if (ch == 0 && p.pdsum != nullptr && i < Nq && hh == 0) p.pdsum[qslice + i] = pd;
  if (i < Nq) {
    T* dqg = reinterpret_cast<T*>(p.dq) + (qslice + i) * D + ch * DC;
#pragma unroll
    for (int mb = 0; mb < DC / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if constexpr (std::is_same<T, float>::value) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = dq[mb][4 * g + e] * p.scale;
          *reinterpret_cast<f32x4*>(dqg + 32 * mb + 8 * g + 4 * hh) = v4;
        } else {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(dq[mb][4 * g + e] * p.scale);
          *reinterpret_cast<bf16x4*>(dqg + 32 * mb + 8 * g + 4 * hh) = v4;
        }
      }
  }
}

// ---------------------------------------------------------------- dK/dV pass
// 16x16 MFMAs (v_mfma_f32_16x16x32_bf16, v_mfma_f32_16x16x4_f32): lane
// (n = lane % 16, k-group g = lane / 16) operands, and a 16x16 accumulator
// in which lane (n, g) holds M index 4 g + e in register e. With 16 keys per
// wave a lane keeps a quarter of its key's K and V rows (64 registers each
// at these widths) where the 32x32 shape would need all 256 architectural
// VGPRs for the two rows.
template <typename T>
struct W16;
template <>
struct W16<float> {
  using op = float;
  static constexpr int KC = 4;
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

// Operand step c of a row (k along the row): elements [c KC + g KC / 4, + KC / 4)
template <typename T>
__device__ inline typename W16<T>::op row_op16(const FM_LDS T* t, int rs, int row, int c, int g) {
  if constexpr (std::is_same<T, float>::value) {
    return t[row * rs + 4 * c + g];
  } else {
    return *reinterpret_cast<const FM_LDS bf16x8*>(t + row * rs + 32 * c + 8 * g);
  }
}

// The 32 rows of a query step in the order of the S accumulators: operand
// step s, k-group g, element e is row 16 (e / 4) + 4 g + e % 4 (bf16, one
// step) or row 16 (s / 4) + 4 g + s % 4 (fp32, eight steps).
template <typename T>
__device__ inline typename W16<T>::op col_op16(const FM_LDS T* t, int rs, int n, int s, int g) {
  if constexpr (std::is_same<T, float>::value) {
    return t[(16 * (s / 4) + 4 * g + (s % 4)) * rs + n];
  } else {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[(16 * (e / 4) + 4 * g + (e % 4)) * rs + n];
    return v;
  }
}

// The same step of the two S-shaped accumulators (rows 16 mt + 4 g + e).
template <typename T>
__device__ inline typename W16<T>::op acc_op16(const f32x4 (&a)[2], int s) {
  if constexpr (std::is_same<T, float>::value) {
    return a[s / 4][s % 4];
  } else {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)a[e / 4][e % 4];
    return v;
  }
}

// Workgroup: 64 keys (16 per wave), chunk ch of NCH: dK columns
// [ch KCK, (ch + 1) KCK) and dV columns [ch KCV, (ch + 1) KCV), KCK = D / NCH,
// KCV = DV / NCH.
// K and V rows of the lane's key in registers; per visible 32-row query
// step (Q, dO, LSE2 and delta in LDS):
//   S = Q K^T, dP = dO V^T, the mask from the key's own bounds,
//   P = exp2(S scale log2e - LSE2), dS = P (dP - delta),
//   dV^T += dO^T P and dK^T += Q^T dS (this chunk's columns; dK takes the
//   scale once, at the end).
template <typename T, int D, int DV, int NCH>
__global__ __launch_bounds__(256, 1) void wide_dkdv_kernel(WideParams p) {
  using X = W16<T>;
  constexpr int KCK = D / NCH, KCV = DV / NCH;
  static_assert(KCK * NCH == D && KCV * NCH == DV && KCK % 16 == 0 && KCV % 16 == 0, "column chunks");
  constexpr int KW = 16, BKC = 64, BQ = 32, KC = X::KC;
  constexpr int QS = lds_stride<T, D>(), OS = lds_stride<T, DV>();
  __shared__ __attribute__((aligned(16))) T qs_[BQ * QS];
  __shared__ __attribute__((aligned(16))) T dos_[BQ * OS];
  __shared__ float lse_s[BQ];
  __shared__ float del_s[BQ];
  FM_LDS T* qs = (FM_LDS T*)qs_;
  FM_LDS T* dos = (FM_LDS T*)dos_;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane >> 4;
  const int n16 = lane & 15;
  const int BH = p.B * p.H;
  const int ch = (int)(blockIdx.x % NCH);
  const int rest = (int)(blockIdx.x / NCH);
  const int bh = rest % BH;
  const int kb = rest / BH;
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const bool causal = p.causal != 0;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int c0 = kb * BKC, c1 = min(Nk, c0 + BKC);
  const int wc0 = c0 + KW * w;
  const int j = wc0 + n16;   // this lane's key
  const T* qg = reinterpret_cast<const T*>(p.q) + qslice * D;
  const T* dog = reinterpret_cast<const T*>(p.dout) + qslice * DV;

  // the key's rows as B operands: step c holds [c KC + g KC / 4, + KC / 4)
  typename X::op kr[D / KC], vr[DV / KC];
  {
    const T* kg = reinterpret_cast<const T*>(p.k) + kslice * D;
    const T* vg = reinterpret_cast<const T*>(p.v) + kslice * DV;
    const bool ok = j < Nk;
#pragma unroll
    for (int c = 0; c < D / KC; ++c) {
      if constexpr (std::is_same<T, float>::value) {
        kr[c] = ok ? kg[(long long)j * D + 4 * c + g] : 0.f;
      } else {
        kr[c] = ok ? *reinterpret_cast<const bf16x8*>(kg + (long long)j * D + 32 * c + 8 * g) : bf16x8{};
      }
    }
#pragma unroll
    for (int c = 0; c < DV / KC; ++c) {
      if constexpr (std::is_same<T, float>::value) {
        vr[c] = ok ? vg[(long long)j * DV + 4 * c + g] : 0.f;
      } else {
        vr[c] = ok ? *reinterpret_cast<const bf16x8*>(vg + (long long)j * DV + 32 * c + 8 * g) : bf16x8{};
      }
    }
  }
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
  constexpr int NKB = KCK / 16, NVB = KCV / 16;   // 16-column blocks of the chunk
  f32x4 dkacc[NKB], dvacc[NVB];
#pragma unroll
  for (int mb = 0; mb < NKB; ++mb) dkacc[mb] = f32x4{};
#pragma unroll
  for (int mb = 0; mb < NVB; ++mb) dvacc[mb] = f32x4{};
  // bounds of the workgroup's 64 keys (one table entry); a wave's 16 keys
  // lie inside them, so the same bounds classify its part (possibly as
  // partial where its own keys alone would not be)
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;
  const BlockBounds kbnd = load_bounds(table + (long long)kb * 8);
  unsigned cnt0 = 0, cnt1 = 0, cnt2 = 0;

  for (int qb = 0; qb < p.nqb; ++qb) {
    const int q0 = qb * BQ, q1 = min(Nq, q0 + BQ);
    const int wgc = tile_class(kbnd, q0, q1, c0, c1, causal);
    cnt0 += wgc == 0;
    cnt1 += wgc == 1;
    cnt2 += wgc == 2;
    if (wgc == 0) continue;
    int wc = 0;
    if (wc0 < Nk) {
      wc = tile_class(kbnd, q0, q1, wc0, min(Nk, wc0 + KW), causal);
      if (wc == 2 && (q1 - q0 < BQ || c1 - c0 < BKC)) wc = 1;
    }
    __syncthreads();   // the last step's readers are done
    stage<T, BQ, D>(qs, QS, qg, D, 0, q0, Nq);
    stage<T, BQ, DV>(dos, OS, dog, DV, 0, q0, Nq);
    if (tid < BQ) {
      const bool ok = q0 + tid < Nq;
      lse_s[tid] = ok ? p.lse2[qslice + q0 + tid] : __builtin_inff();
      del_s[tid] = ok ? p.delta[qslice + q0 + tid] : 0.f;
    }
    __syncthreads();
    if (wc == 0) continue;
    // S = Q K^T and dP = dO V^T for the step's two 16-row halves (lane:
    // key j; rows 16 mt + 4 g + e); the two chains alternate while both
    // have steps left (D / KC and DV / KC of them)
    constexpr int NSS = D / KC, NSD = DV / KC, NSMIN = NSS < NSD ? NSS : NSD;
    auto is_dp = [](int t) { return t < 2 * NSMIN ? (t & 1) != 0 : NSD > NSS; };
    auto sstep = [](int t) { return t < 2 * NSMIN ? t >> 1 : t - NSMIN; };
    f32x4 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{};
      dp[mt] = f32x4{};
      chain<NSS + NSD, 2>(
          [&](int t) {
            return is_dp(t) ? row_op16<T>(dos, OS, 16 * mt + n16, sstep(t), g)
                            : row_op16<T>(qs, QS, 16 * mt + n16, sstep(t), g);
          },
          [&](int t, typename X::op a) {
            if (is_dp(t)) dp[mt] = X::mma(a, vr[sstep(t)], dp[mt]);
            else s[mt] = X::mma(a, kr[sstep(t)], s[mt]);
          });
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int il = 16 * mt + 4 * g + e;
        const bool m = (wc == 1) & hidden(p, q0 + il, j, k_lts, k_lte, k_uts, k_ute);
        const float sv = m ? kNegInf : s[mt][e];
        const float pv = exp2f(__builtin_fmaf(sv, p.sl2, -lse_s[il]));
        s[mt][e] = pv;
        dp[mt][e] = pv * (dp[mt][e] - del_s[il]);   // dS; the scale goes on dK at the end
      }
    // P and dS as operands once (bf16: rounded), then dV^T += dO^T P and
    // dK^T += Q^T dS over the step's 32 rows, the two products alternating
    // while both have steps left; step u of a product is column block
    // u / NST, row step u % NST
    constexpr int NST = 32 / KC;
    typename X::op pop[NST], dsop[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      pop[st] = acc_op16<T>(s, st);
      dsop[st] = acc_op16<T>(dp, st);
    }
    constexpr int NMIN = (NKB < NVB ? NKB : NVB) * NST;
    auto is_k = [](int t) { return t < 2 * NMIN ? (t & 1) != 0 : NKB > NVB; };
    auto step_of = [](int t) { return t < 2 * NMIN ? t >> 1 : t - NMIN; };
    chain<(NKB + NVB) * NST, 2>(
        [&](int t) {
          const int u = step_of(t), mb = u / NST, st = u % NST;
          return is_k(t) ? col_op16<T>(qs, QS, ch * KCK + 16 * mb + n16, st, g)
                         : col_op16<T>(dos, OS, ch * KCV + 16 * mb + n16, st, g);
        },
        [&](int t, typename X::op a) {
          const int u = step_of(t), mb = u / NST, st = u % NST;
          if (is_k(t)) dkacc[mb] = X::mma(a, dsop[st], dkacc[mb]);
          else dvacc[mb] = X::mma(a, pop[st], dvacc[mb]);
        });
  }

  // lane: key j, dK columns ch KCK + 16 mb + 4 g + e, dV columns ch KCV + ...
  if (j < Nk) {
    T* dkg = reinterpret_cast<T*>(p.dk) + (kslice + j) * D + ch * KCK;
    T* dvg = reinterpret_cast<T*>(p.dv) + (kslice + j) * DV + ch * KCV;
#pragma unroll
    for (int mb = 0; mb < NKB; ++mb) {
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4*>(dkg + 16 * mb + 4 * g) = dkacc[mb] * p.scale;
      } else {
        bf16x4 k4;
#pragma unroll
        for (int e = 0; e < 4; ++e) k4[e] = (bf16)(dkacc[mb][e] * p.scale);
        *reinterpret_cast<bf16x4*>(dkg + 16 * mb + 4 * g) = k4;
      }
    }
#pragma unroll
    for (int mb = 0; mb < NVB; ++mb) {
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4*>(dvg + 16 * mb + 4 * g) = dvacc[mb];
      } else {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)dvacc[mb][e];
        *reinterpret_cast<bf16x4*>(dvg + 16 * mb + 4 * g) = v4;
      }
    }
  }
  if (ch == 0 && p.counts != nullptr && tid == 0) {
    atomicAdd(p.counts + 0, (unsigned long long)cnt0);
    atomicAdd(p.counts + 1, (unsigned long long)cnt1);
    atomicAdd(p.counts + 2, (unsigned long long)cnt2);
  }
}

// ---------------------------------------------------------------- launch
// Column chunks per shape: the forward's O chunk (DVC columns), the dQ
// pass's dQ chunk (DC) and the number of dK/dV chunks (NCH).
template <typename T, int D, int DV>
struct WideCfg;
template <>
struct WideCfg<bf16, 512, 512> {
  static constexpr int DVC = 256, DC = 128, NCH = 2;
};
template <>
struct WideCfg<float, 256, 256> {
  static constexpr int DVC = 256, DC = 128, NCH = 1;
};
template <>
struct WideCfg<float, 192, 128> {
  static constexpr int DVC = 128, DC = 192, NCH = 1;
};

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
  using C = WideCfg<T, D, DV>;
  WideParams p = wide_params(a);
  p.nqb = (a.Nq + 127) / 128;
  const long long grid = (long long)a.B * a.H * p.nqb * (DV / C::DVC);
  hipLaunchKernelGGL((wide_fwd_kernel<T, D, DV, C::DVC>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t launch_wide_bwd_t(const AttnArgs& a, hipStream_t stream) {
  using C = WideCfg<T, D, DV>;
  WideParams p = wide_params(a);
  p.pdsum = a.sink != nullptr ? a.pdsum : nullptr;
  p.nqb = (a.Nq + 127) / 128;
  long long grid = (long long)a.B * a.H * p.nqb * (D / C::DC);
  hipLaunchKernelGGL((wide_dq_kernel<T, D, DV, C::DC>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.nqb = (a.Nq + 31) / 32;
  grid = (long long)a.B * a.H * p.nkb64 * C::NCH;
  hipLaunchKernelGGL((wide_dkdv_kernel<T, D, DV, C::NCH>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// the shapes compiled in (kept in step with wide_dims())
hipError_t launch_wide_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.is_bf16 && a.d == 512 && a.dv == 512) return launch_wide_fwd_t<bf16, 512, 512>(a, stream);
  if (!a.is_bf16 && a.d == 256 && a.dv == 256) return launch_wide_fwd_t<float, 256, 256>(a, stream);
  if (!a.is_bf16 && a.d == 192 && a.dv == 128) return launch_wide_fwd_t<float, 192, 128>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_wide_bwd(const AttnArgs& a, hipStream_t stream) {
  if (a.is_bf16 && a.d == 512 && a.dv == 512) return launch_wide_bwd_t<bf16, 512, 512>(a, stream);
  if (!a.is_bf16 && a.d == 256 && a.dv == 256) return launch_wide_bwd_t<float, 256, 256>(a, stream);
  if (!a.is_bf16 && a.d == 192 && a.dv == 128) return launch_wide_bwd_t<float, 192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fm
