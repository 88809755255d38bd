// Forward kernels: O = softmax(scale * Q K^T + M) V and its logsumexp.
//
// The operation is the FlashMask README "Formulation"; M is the column-wise
// sparse mask (README "Overview", FlashMask-3 abstract). Work is tiled the
// FlashAttention way (the FlashMask abstract calls FlashMask an extension of
// it): each workgroup owns a block of query rows, streams key/value tiles
// through LDS and keeps a running row max and row sum (online softmax), so
// nothing of size N x N exists. Tiles the per-key-block table proves hidden
// are never loaded; tiles it proves untouched run without mask arithmetic.
//
// gfx950 mapping (bf16 path):
//   * 4 waves x 32 query rows = 128 rows per workgroup; key tiles of 64.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     each lane then owns one query row (its column of S^T) and 32 of the 64
//     keys, so the row max needs one cross-half exchange and the row sum none
//     until the end, and the probabilities are already laid out as the B
//     operand of O^T += V^T P^T (the MFMA contraction index is permuted to
//     match the accumulator layout; the same permutation is applied to V^T).
//   * K and V tiles arrive by buffer loads straight into LDS (no VGPR
//     staging), double buffered; out-of-range rows read as zero.
//   * V^T operands come from the row-major V tile with ds_read_b64_tr_b16.
//   * A workgroup first compacts the list of key tiles it must visit (with a
//     per-wave class for each), so hidden tiles cost nothing in the loop.
#include <type_traits>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
  const int32_t* table;  // [B, hm, nkb, 8] at 64-column blocks
  void* o;
  float* lse;
  const float* sink;     // forward: per-head sink logits [H], or nullptr
  float* pdsum;          // dQ passes with a sink: rowsum(dS) per row, [B, H, Nq]
  unsigned long long* counts;
  // dQ mode (backward): dO and the forward's O and natural-log LSE in; dQ
  // out, and per row the base-2 LSE and delta = rowsum(dO * O) out for the
  // dK/dV pass
  const void* dout;
  const void* o_in;
  const float* lse_in;
  float* lse2;
  float* delta;
  void* dq;
  int* qzero;            // bf16 dQ pass: the dK/dV pass's 8 work-queue counters, zeroed here
  int B, H, Nq, Nk, hm, causal;   // Nq query rows, Nk keys
  int has_lt, has_lte, has_ut;
  float scale, sl2;
  int nqb, nkb;
};

// ---------------------------------------------------------------- shared mask test
// Apply the element test to a 32x32 S^T block held in the MFMA accumulator
// layout: lane (i = lane % 32, h = lane / 32), register r holds key
// 8 * (r / 4) + 4 * h + r % 4 of the block. `vl` points at the tile's four
// boundary vectors in LDS ([4][64] int32) and `kl0` is the block's first key
// within the tile.
__device__ inline void mask_block(f32x16& s, const FM_LDS int* vl, int kl0, int kbase, int i,
                                  const FwdParams& p, int hh) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int kl = kl0 + 8 * g + 4 * hh;
    i32x4 lts4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 0 * 64 + kl);
    i32x4 lte4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 1 * 64 + kl);
    i32x4 uts4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 2 * 64 + kl);
    i32x4 ute4 = *reinterpret_cast<const FM_LDS i32x4*>(vl + 3 * 64 + kl);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = kbase + kl + e;
      bool m = (j >= p.Nk) || (p.causal && j > i);
      const int lte_v = p.has_lte ? lte4[e] : p.Nq;
      m = m || (p.has_lt && lts4[e] <= i && i < lte_v);
      m = m || (p.has_ut && uts4[e] <= i && i < ute4[e]);
      if (m) s[4 * g + e] = kNegInf;
    }
  }
}

// ---------------------------------------------------------------- bf16 kernel
// One query-major kernel serves two passes:
//   MODE 0, forward: O and LSE with online softmax;
//   MODE 1, the dQ pass of the backward: with the forward's LSE and
//     delta = rowsum(dO * O) known per row, P = exp(S - LSE) and
//     dS = P * (dO V^T - delta) need no running state, and
//     dQ^T += K^T dS^T takes the place of O^T += V^T P^T.
// Both stream K/V tiles through LDS with the same classification, scan and
// pipeline; each wave owns 32 query rows (its lanes hold one row each in the
// transposed score layout S^T = K Q^T).
constexpr int kModeFwd = 0;
constexpr int kModeDq = 1;
// dQ pass that also sums rowsum(dS) per row (for the sink gradient)
constexpr int kModeDqSink = 2;

// D: head dim of Q and K; DV: head dim of V (and O, dO).
template <int D, int DV, int MODE>
struct QCfg {
  static constexpr int NW = 4;
  static constexpr int WR = 32;                           // query rows per wave
  static constexpr int BR = WR * NW;                      // query rows per workgroup
  static constexpr int BC = 64;                           // keys per tile
  // 32-key blocks per inner step (1 keeps registers within budget; the
  // second tile configuration, FM_ALT_TILES, takes 1 everywhere)
#ifdef FM_ALT_TILES
  static constexpr int JBS = 1;
#else
  static constexpr int JBS = (D > 128 || DV > 128 || MODE != kModeFwd) ? 1 : 2;
#endif
  static constexpr int CHK = D / 8;                       // 16-byte chunks per K row
  static constexpr int CHV = DV / 8;                      // 16-byte chunks per V row
  static constexpr int KT = BC * D * 2;                   // bytes of one K tile
  static constexpr int VT = BC * DV * 2;                  // bytes of one V tile
  static constexpr int LOADS_K = KT / (NW * 1024);        // per wave
  static constexpr int LOADS_V = VT / (NW * 1024);
  static constexpr int VEC = 4 * BC * 4;                  // the tile's boundary vectors
  static constexpr int STAGE = KT + VT + VEC;
#ifdef FM_ALT_TILES
  static constexpr int LIST = 2 * NW * 64;                // compacted tile list entries
#else
  static constexpr int LIST = 1024;                       // compacted tile list entries
#endif
  static constexpr int LOADS_PER_TILE = LOADS_K + LOADS_V + 1;  // waves 0-3 (they stage a vector)
  // two workgroups per CU when both fit in LDS and 256 registers
  static constexpr int WG_PER_CU = (D <= 128 && DV <= 128) ? 2 : 1;
};

// XOR swizzle of the 16-byte chunk index within a row: 32 consecutive rows
// read at one chunk (row operand reads) and 8 rows x 4 chunks (transposed
// reads) both spread over the LDS banks.
template <int D>
__device__ inline int fswz(int row) {
  static_assert(D == 64 || D == 128 || D == 192, "row width");
  if constexpr (D == 192) return (row >> 1) & 7;   // 24 chunks: stay inside each group of 8
  else if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
  else return 4 * (row & 1) + ((row >> 1) & 3);
}

// Running-max slack, in log2 units: the max used to scale P only moves when
// a row's new max exceeds it by more than this, so the O rescale is rare;
// P then stays below 2^8, well inside bf16 and fp32 range. Exact either way,
// since O and the row sum always use the same offset.
constexpr float kRescaleSlack = 8.0f;

template <int D, int DV, int MODE>
__global__ __launch_bounds__(256, (QCfg<D, DV, MODE>::WG_PER_CU)) void qmajor_bf16_kernel(FwdParams p) {
  using C = QCfg<D, DV, MODE>;
  constexpr bool DQ = MODE != kModeFwd;
  constexpr bool PD = MODE == kModeDqSink;
  // Two pipeline stages as separate LDS objects.
  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE];
  __shared__ int list[C::LIST];           // visible key blocks
  __shared__ unsigned list_cls[C::LIST];  // their per-wave classes, 2 bits each
  __shared__ int wsum[C::NW];
  __shared__ unsigned wcount[3];
  __shared__ uint32_t mwords[C::NW][C::BC];  // per wave: masked-row word of each key

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int BH = p.B * p.H;
  int bh, qb;
  xcd_order((int)blockIdx.x, BH, p.nqb, bh, qb);
  qb = p.nqb - 1 - qb;                                   // heavy (late) query blocks first
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const long long qslice = (long long)bh * Nq;           // rows of Q, O, dO, LSE
  const long long kslice = (long long)bh * Nk;           // rows of K, V
  const int r0 = qb * C::BR;
  const int r1 = min(Nq, r0 + C::BR);
  const int wr0 = r0 + C::WR * w;                       // this wave's first row
  const int i = wr0 + l32;                              // this lane's row
  const uint32_t qbytes = (uint32_t)Nq * D * 2;    // one head of Q
  const uint32_t kbytes = (uint32_t)Nk * D * 2;    // one head of K
  const uint32_t vbytes = (uint32_t)Nk * DV * 2;   // one head of V
  const uint32_t obytes = (uint32_t)Nq * DV * 2;   // one head of O or dO

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const bf16*>(p.q) + qslice * D, qbytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const bf16*>(p.k) + kslice * D, kbytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const bf16*>(p.v) + kslice * DV, vbytes);
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  const int32_t* vecs[4] = {p.lts, p.lte, p.uts, p.ute};
  // each wave stages one of the four boundary vectors (absent ones read as 0)
  const int32_t* my_vec = vecs[w & 3];
  const bool vec_present = my_vec != nullptr && (w < 2 ? p.has_lt : p.has_ut);
  const __amdgpu_buffer_rsrc_t rvec =
      make_rsrc(vec_present ? my_vec + vrow : p.table, vec_present ? (uint32_t)Nk * 4 : 0u);

  // This lane's row of Q (and dO) as B operands: chunk c holds
  // [i][16c + 8h .. +7]. Rows past Nq read as zero.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, buffer_load16(rq, (uint32_t)(i * D + 16 * c + 8 * hh) * 2));
  bf16x8 dof[DQ ? DV / 16 : 1];
  float row_lse2 = 0.f, row_delta = 0.f;
  float row_pd = 0.f;   // this lane's part of rowsum(dS) (kModeDqSink)
  if constexpr (DQ) {
    const __amdgpu_buffer_rsrc_t rdo =
        make_rsrc(reinterpret_cast<const bf16*>(p.dout) + qslice * DV, obytes);
#pragma unroll
    for (int c = 0; c < DV / 16; ++c)
      dof[c] = __builtin_bit_cast(bf16x8, buffer_load16(rdo, (uint32_t)(i * DV + 16 * c + 8 * hh) * 2));
    // delta_i = dO_i . O_i: this lane holds half of row i (the chunks of
    // its half-wave), the other half-wave the rest
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(reinterpret_cast<const bf16*>(p.o_in) + qslice * DV, obytes);
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    float dl = 0.f;
#pragma unroll
    for (int c = 0; c < DV / 16; ++c) {
      const bf16x8 oc = __builtin_bit_cast(bf16x8, buffer_load16(ro, (uint32_t)(i * DV + 16 * c + 8 * hh) * 2));
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        dl = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{dof[c][e], dof[c][e + 1]}, bf16x2_t{oc[e], oc[e + 1]}, dl, false);
    }
    row_delta = sum_x32(dl);
    // base-2 LSE; a fully masked row (LSE -inf) gets +inf, so its P is 0
    const float l = i < Nq ? p.lse_in[qslice + i] : kNegInf;
    row_lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
    if (hh == 0 && i < Nq) {
      p.delta[qslice + i] = row_delta;
      p.lse2[qslice + i] = row_lse2;
    }
  }

  constexpr int NO = DQ ? D / 32 : DV / 32;   // 32-column blocks of the output
  f32x16 oacc[NO];               // O^T (forward) or dQ^T (dQ pass)
#pragma unroll
  for (int mb = 0; mb < NO; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  if (tid < 3) wcount[tid] = 0;
  unsigned cnt0 = 0, cnt1 = 0, cnt2 = 0;
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb * 8;
  const bool causal = p.causal != 0, has_lt = p.has_lt != 0, has_lte = p.has_lte != 0,
             has_ut = p.has_ut != 0;

  // --- issue the loads of one key tile into a stage
  auto issue = [&](int kb, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const int kbase = kb * C::BC;
    FM_LDS char* st = (FM_LDS char*)(S ? stage1 : stage0);
#pragma unroll
    for (int u = 0; u < C::LOADS_K; ++u) {
      const int g = (w * C::LOADS_K + u) * 64 + lane;   // physical chunk in the K tile
      const int row = g / C::CHK, pch = g % C::CHK;
      load_lds16(rk, st + (w * C::LOADS_K + u) * 1024,
                 (uint32_t)((kbase + row) * D + 8 * (pch ^ fswz<D>(row))) * 2);
    }
#pragma unroll
    for (int u = 0; u < C::LOADS_V; ++u) {
      const int g = (w * C::LOADS_V + u) * 64 + lane;   // physical chunk in the V tile
      const int row = g / C::CHV, pch = g % C::CHV;
      load_lds16(rv, st + C::KT + (w * C::LOADS_V + u) * 1024,
                 (uint32_t)((kbase + row) * DV + 8 * (pch ^ fswz<DV>(row))) * 2);
    }
    // waves 0-3: 16 lanes x 16 bytes = one 64-key vector each
    if (w < 4 && lane < 16) load_lds16(rvec, st + C::KT + C::VT + w * 256, (uint32_t)(kbase + 4 * lane) * 4);
  };

  using KW = std::integral_constant<int, D>;    // K tile width tag
  using VW = std::integral_constant<int, DV>;   // V tile width tag
  // row operand read (32 rows of a W-wide tile at one 16-byte chunk)
  auto row_read = [&](auto w_c, const FM_LDS char* t, int row, int chunk) {
    constexpr int W = decltype(w_c)::value;
    return lds_read_b128(t + row * W * 2 + ((chunk ^ fswz<W>(row)) << 4));
  };
  // transposed operand read: for MFMA contraction chunk c (16 keys) and
  // column block mb, 4 consecutive keys of one column per lane, twice
  auto tr_read = [&](auto w_c, const FM_LDS char* t, int c, int mb) {
    constexpr int W = decltype(w_c)::value;
    const int sl = lane & 15;
    const int row_a = 16 * c + 4 * hh + (sl >> 2);
    const int row_b = row_a + 8;
    const int col = 32 * mb + 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
    const FM_LDS char* pa = t + row_a * W * 2 + (((col >> 3) ^ fswz<W>(row_a)) << 4) + (col & 7) * 2;
    const FM_LDS char* pb = t + row_b * W * 2 + (((col >> 3) ^ fswz<W>(row_b)) << 4) + (col & 7) * 2;
    return cat(lds_read_tr(pa), lds_read_tr(pb));
  };

  // --- one key tile of work for this wave
  auto compute = [&](int kb, unsigned cls, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const int wc = (int)((cls >> (2 * w)) & 3u);
    if (wc == 0) return;
    const int kbase = kb * C::BC;
    const FM_LDS char* kst = (const FM_LDS char*)(S ? stage1 : stage0);
    const FM_LDS char* vst = kst + C::KT;
    const FM_LDS int* vl = (const FM_LDS int*)(kst + C::KT + C::VT);
    constexpr int JBS = C::JBS;
    constexpr int FPF = 3;   // operand ring depth of the forward S and PV products
    if (wc == 1) {
      // one key per lane: which of this wave's 32 rows the mask hides for it
      // (absent vectors were staged as zeros, and has_* gates their use)
      mwords[w][lane] = key_row_mask(kbase + lane, wr0, Nk, causal, has_lt, has_ut, vl[lane],
                                     has_lte ? vl[64 + lane] : Nq, vl[128 + lane], vl[192 + lane]);
      __builtin_amdgcn_wave_barrier();
    }
    // S^T starts at the mask's additive bias (-inf where masked, else 0): the
    // MFMAs apply the mask, and the code after them is the same for every
    // tile class. Element test: bit l32 (this lane's row) of the word of
    // the element's key.
    auto bias = [&](f32x16& sx, int kb32) {
      if (wc == 1) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int kl = kb32 * 32 + 8 * g + 4 * hh;
          const u32x4 w4 = *(const FM_LDS u32x4*)(FM_LDS uint32_t*)&mwords[w][kl];
#pragma unroll
          for (int e = 0; e < 4; ++e) sx[4 * g + e] = mask_bias(w4[e], l32);
        }
      } else {
        sx = f32x16{};
      }
    };
    if constexpr (DQ) {
      // dQ pass, one 32-key half at a time (two workgroups per CU hide the
      // latencies; holding both halves at once would need one per CU)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        f32x16 s, dp;
        const int row = jb * 32 + l32;
        // S^T = K Q^T + bias, dP^T = V dO^T. The two chains alternate while
        // both have steps left, and the K / V operands are read PF MFMAs
        // ahead through a ring of registers (a deeper ring spills at two
        // waves per SIMD), with a fence per step holding that order. Written
        // twice: a partial tile starts S at the mask's bias, a full one at
        // zero, taken by the first MFMA as an inline constant.
        constexpr int PF = 2;
        constexpr int NS = D / 16, NP = DV / 16, NSP = NS + NP, NMIN = NS < NP ? NS : NP;
        auto is_s = [](int t) { return t < 2 * NMIN ? (t & 1) == 0 : NS > NP; };
        auto chunk = [](int t) { return t < 2 * NMIN ? t >> 1 : t - NMIN; };
        auto rd = [&](int t) {
          return is_s(t) ? row_read(KW{}, kst, row, 2 * chunk(t) + hh) : row_read(VW{}, vst, row, 2 * chunk(t) + hh);
        };
        auto sdp_chain = [&](auto part_c) {
          constexpr bool PART = decltype(part_c)::value;
          if constexpr (PART) bias(s, jb);   // also right for a full tile (zero bias)
          bf16x8 ring[PF];
#pragma unroll
          for (int t = 0; t < PF; ++t) ring[t] = rd(t);
#pragma unroll
          for (int t = 0; t < NSP; ++t) {
            const bf16x8 a = ring[t % PF];
            if (t + PF < NSP) ring[t % PF] = rd(t + PF);
            if (is_s(t)) s = mfma32(a, qf[chunk(t)], (!PART && chunk(t) == 0) ? f32x16{} : s);
            else dp = mfma32(a, dof[chunk(t)], chunk(t) == 0 ? f32x16{} : dp);
            __builtin_amdgcn_sched_barrier(0x406);
          }
        };
        if constexpr (PD) {
          sdp_chain(std::true_type{});   // one chain (two spill here: the dS row sum holds registers)
        } else {
          if (wc == 1) sdp_chain(std::true_type{});
          else sdp_chain(std::false_type{});
        }
        // dS = P (dP - delta) with P = exp2(S * scale * log2e - LSE2)
        bf16x8 pf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(__builtin_fmaf(s[r], p.sl2, -row_lse2));
          const float dsv = pv * (dp[r] - row_delta);
          pf[r / 8][r % 8] = (bf16)dsv;
          if constexpr (PD) row_pd += dsv;   // the sink gradient's row sum of dS, in fp32
        }
        // dQ^T += K^T dS^T over the half's keys
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = mfma32(tr_read(KW{}, kst, 2 * jb + cc, mb), pf[cc], oacc[mb]);
      }
    } else {
#pragma unroll
    for (int hk = 0; hk < C::BC / 32 / JBS; ++hk) {
      f32x16 s[JBS];
      // S^T = K Q^T: the JBS accumulation chains alternate, and each K
      // operand is read FPF MFMAs ahead through a ring of registers. A fence
      // per step keeps reads and MFMAs in that order (the scheduler, short of
      // registers, otherwise sinks each read to its MFMA and every MFMA waits
      // out an LDS latency); VALU, SALU and transcendental work may cross it.
      // Written twice: a partial tile starts the chains at the mask's bias,
      // a full one at zero, which the first MFMA then takes as an inline
      // constant (one shared start would cost a register move per element).
      auto s_chain = [&](auto part_c) {
        constexpr bool PART = decltype(part_c)::value;
        if constexpr (PART) {   // (also right for a full tile: zero bias)
#pragma unroll
          for (int jj = 0; jj < JBS; ++jj) bias(s[jj], hk * JBS + jj);
        }
        constexpr int NS = JBS * (D / 16);
        auto rd = [&](int t) {
          return row_read(KW{}, kst, (hk * JBS + t % JBS) * 32 + l32, 2 * (t / JBS) + hh);
        };
        bf16x8 ring[FPF];
#pragma unroll
        for (int t = 0; t < FPF; ++t) ring[t] = rd(t);
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const bf16x8 a = ring[t % FPF];
          if (t + FPF < NS) ring[t % FPF] = rd(t + FPF);
          if (!PART && t < JBS) s[t % JBS] = mfma32(a, qf[t / JBS], f32x16{});
          else s[t % JBS] = mfma32(a, qf[t / JBS], s[t % JBS]);
          __builtin_amdgcn_sched_barrier(0x406);
        }
      };
      if (wc == 1) s_chain(std::true_type{});
      else s_chain(std::false_type{});
      bf16x8 pf[2 * JBS];
      float mx = max_acc(s);
      mx = max_x32(mx);
      // move the offset (and rescale O and the sum) only when some row's max
      // outgrew it by more than the slack; a row with nothing open keeps -inf
      if (__ballot((mx - m_run) * p.sl2 > kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == kNegInf ? 1.f : fast_exp2((m_run - m_new) * p.sl2);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < DV / 32; ++mb) oacc[mb] *= alpha;
        m_run = m_new;
      }
      const float msl = (m_run == kNegInf ? 0.f : m_run) * p.sl2;
#pragma unroll
      for (int jj = 0; jj < JBS; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pf[2 * jj + r / 8][r % 8] = (bf16)fast_exp2(__builtin_fmaf(s[jj][r], p.sl2, -msl));
      // row sum of the rounded probabilities (the values the PV MFMA
      // uses), two per v_dot2_f32_bf16
      float rs = l_run;
#pragma unroll
      for (int c = 0; c < 2 * JBS; ++c) rs = sum8_bf16(pf[c], rs);
      l_run = rs;
      // O^T += V^T P^T, V operands through the same kind of ring
      {
        constexpr int NMB = DV / 32, NPV = 2 * JBS * NMB;
        auto rd = [&](int t) { return tr_read(VW{}, vst, 2 * JBS * hk + t / NMB, t % NMB); };
        bf16x8 ring[FPF];
#pragma unroll
        for (int t = 0; t < FPF; ++t) ring[t] = rd(t);
#pragma unroll
        for (int t = 0; t < NPV; ++t) {
          const bf16x8 a = ring[t % FPF];
          if (t + FPF < NPV) ring[t % FPF] = rd(t + FPF);
          oacc[t % NMB] = mfma32(a, pf[t / NMB], oacc[t % NMB]);
          __builtin_amdgcn_sched_barrier(0x406);
        }
      }
    }
    }
  };

  // --- scan the key blocks, compact the visible ones, process in chunks
  constexpr int NT = C::NW * 64;
  int cnt = 0;
  for (int base = 0; base < p.nkb; base += NT) {
    const int kb = base + tid;
    unsigned bits = 0;
    bool valid = false;
    if (kb < p.nkb) {
      const BlockBounds bb = load_bounds(table + (long long)kb * 8);
      const int c0 = kb * C::BC, c1 = min(Nk, c0 + C::BC);
      const int wgc = tile_class(bb, r0, r1, c0, c1, causal);
      cnt0 += wgc == 0;
      cnt1 += wgc == 1;
      cnt2 += wgc == 2;
      if (wgc != 0) {
        valid = true;
        const bool ragged = c1 - c0 < C::BC;
#pragma unroll
        for (int ww = 0; ww < C::NW; ++ww) {
          const int a0 = r0 + C::WR * ww;
          int cl = 0;
          if (a0 < Nq) {
            cl = tile_class(bb, a0, min(Nq, a0 + C::WR), c0, c1, causal);
            if (ragged && cl == 2) cl = 1;
          }
          bits |= (unsigned)cl << (2 * ww);
        }
      }
    }
    const unsigned long long bal = __ballot(valid);
    const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
    if (lane == 0) wsum[w] = __builtin_popcountll(bal);
    __syncthreads();
    int off = cnt, add = 0;
#pragma unroll
    for (int ww = 0; ww < C::NW; ++ww) {
      const int v = wsum[ww];
      if (ww < w) off += v;
      add += v;
    }
    if (valid) {
      list[off + rank] = kb;
      list_cls[off + rank] = bits;
    }
    __syncthreads();
    cnt += add;
    if (cnt > C::LIST - NT || base + NT >= p.nkb) {
      // process the compacted list with a two-stage load pipeline
      auto step = [&](int it, auto stage_c) {
        constexpr int S = decltype(stage_c)::value;
        // uniform across the wave: keeps the class tests scalar branches
        const int kb_it = uniform(list[it]);
        const unsigned cls_it = uniform_u32(list_cls[it]);
        // Tile it is the only load in flight. Once every wave has it (the
        // barrier), every wave is also done with tile it - 1, whose stage
        // then takes tile it + 1: one barrier per tile.
        wait_vmcnt<0>();
        lds_barrier();
        if (it + 1 < cnt) issue(list[it + 1], std::integral_constant<int, 1 - S>{});
        compute(kb_it, cls_it, stage_c);
      };
      if (cnt > 0) issue(list[0], std::integral_constant<int, 0>{});
      for (int it = 0; it < cnt; it += 2) {
        step(it, std::integral_constant<int, 0>{});
        if (it + 1 < cnt) step(it + 1, std::integral_constant<int, 1>{});
      }
      cnt = 0;
    }
  }

  // --- epilogue: each wave writes its 32 rows of O (or dQ). A lane holds
  // its own row, 4 consecutive columns per register group, so stores straight
  // from registers would touch 32 rows per instruction. The rows go through
  // LDS instead (the stage buffers are free once the last tile is done: every
  // wave has passed its final barrier and no load into LDS is in flight), and
  // each store then writes whole rows, 16 bytes per lane.
  constexpr int W = DQ ? D : DV;   // output row width
  constexpr int CH = W / 8;        // 16-byte chunks per row
  static_assert(2 * 32 * W * 2 <= C::STAGE, "two waves' rows fit one stage");
  __syncthreads();   // every wave is done with the stages
  float mul;
  if constexpr (!DQ) {
    // normalise, store O (bf16) and the natural-log LSE
    const float lt = sum_x32(l_run);
    float row_lse;
    finish_row(lt, m_run, p.scale, p.sink != nullptr ? p.sink[h] : kNegInf, p.sink != nullptr, mul, row_lse);
    if (i < Nq && hh == 0) p.lse[qslice + i] = row_lse;
  } else {
    mul = p.scale;   // dQ = scale * dS K
    if constexpr (PD) {
      // rowsum(dS) for the sink gradient (see sink_grad_kernel)
      const float pd = sum_x32(row_pd);
      if (i < Nq && hh == 0) p.pdsum[qslice + i] = pd;
    }
  }
  FM_LDS char* ost = (FM_LDS char*)(w < 2 ? stage0 : stage1) + (w & 1) * 32 * W * 2;
  // row r, chunk c at r * W * 2 + 16 (c ^ (r & 7)): rows spread over the banks
#pragma unroll
  for (int mb = 0; mb < W / 32; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (bf16)(oacc[mb][4 * g + e] * mul);
      const int col = 32 * mb + 8 * g + 4 * hh;
      *reinterpret_cast<FM_LDS bf16x4*>(ost + l32 * W * 2 + (((col >> 3) ^ (l32 & 7)) << 4) + (col & 7) * 2) = v4;
    }
  __builtin_amdgcn_wave_barrier();
  bf16* outg = reinterpret_cast<bf16*>(DQ ? p.dq : p.o) + (qslice + wr0) * W;
#pragma unroll
  for (int k = 0; k < CH / 2; ++k) {
    const int f = 64 * k + lane;
    const int row = f / CH, c = f % CH;
    const u32x4 val = *reinterpret_cast<const FM_LDS u32x4*>(ost + row * W * 2 + ((c ^ (row & 7)) << 4));
    if (wr0 + row < Nq) *reinterpret_cast<u32x4*>(outg + (long long)row * W + 8 * c) = val;
  }
  if constexpr (DQ) {
    // the dK/dV pass that follows on this stream takes work from these
    // counters (wave 0 of one workgroup: lane l zeroes counter l % 8)
    if (p.qzero != nullptr && blockIdx.x == 0 && w == 0) p.qzero[lane & 7] = 0;
  }
  if (p.counts != nullptr) {
    atomicAdd(&wcount[0], cnt0);
    atomicAdd(&wcount[1], cnt1);
    atomicAdd(&wcount[2], cnt2);
    __syncthreads();
    if (tid < 3) atomicAdd(p.counts + tid, (unsigned long long)wcount[tid]);
  }
}

// ---------------------------------------------------------------- fp32 kernel
// Same tiling and classification with v_mfma_f32_32x32x2_f32; K and V tiles
// are staged through registers into padded LDS rows. Probabilities stay fp32.
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p) {
  constexpr int BC = 64, BR = 128, KS = D + 1, VS = D + 4;
  __shared__ float ks[BC * KS];
  __shared__ float vs[BC * VS];
  __shared__ int vl[4 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  const int qb = p.nqb - 1 - (int)(blockIdx.x / BH);
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int r0 = qb * BR, r1 = min(Nq, r0 + BR);
  const int i = r0 + 32 * w + (lane & 31);
  const float* qg = reinterpret_cast<const float*>(p.q) + qslice * D;
  const float* kg = reinterpret_cast<const float*>(p.k) + kslice * D;
  const float* vg = reinterpret_cast<const float*>(p.v) + kslice * D;
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb * 8;

  float qf[D / 2];
#pragma unroll
  for (int t = 0; t < D / 2; ++t) qf[t] = i < Nq ? qg[(long long)i * D + 2 * t + hh] : 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  unsigned cnt0 = 0, cnt1 = 0, cnt2 = 0;

  for (int kb = 0; kb < p.nkb; ++kb) {
    const BlockBounds bb = load_bounds(table + (long long)kb * 8);
    const int c0 = kb * BC, c1 = min(Nk, c0 + BC);
    const int wgc = tile_class(bb, r0, r1, c0, c1, p.causal != 0);
    cnt0 += wgc == 0;
    cnt1 += wgc == 1;
    cnt2 += wgc == 2;
    if (wgc == 0) continue;
    int wc = 0;
    const int a0 = r0 + 32 * w;
    if (a0 < Nq) {
      wc = tile_class(bb, a0, min(Nq, a0 + 32), c0, c1, p.causal != 0);
      if (c1 - c0 < BC && wc == 2) wc = 1;
    }
    __syncthreads();
    for (int t = tid; t < BC * D; t += 256) {
      const int row = t / D, col = t % D;
      const bool ok = c0 + row < Nk;
      ks[row * KS + col] = ok ? kg[(long long)(c0 + row) * D + col] : 0.f;
      vs[row * VS + col] = ok ? vg[(long long)(c0 + row) * D + col] : 0.f;
    }
    {
      const int vsel = tid >> 6, kk = tid & 63;
      const int32_t* src = vsel == 0 ? p.lts : vsel == 1 ? p.lte : vsel == 2 ? p.uts : p.ute;
      const bool present = src != nullptr && (vsel < 2 ? p.has_lt : p.has_ut);
      vl[vsel * 64 + kk] = (present && c0 + kk < Nk) ? src[vrow + c0 + kk] : 0;
    }
    __syncthreads();
    if (wc == 0) continue;
    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      s[jb] = f32x16{};
      const int row = jb * 32 + (lane & 31);
#pragma unroll
      for (int t = 0; t < D / 2; ++t) s[jb] = mfma32f(ks[row * KS + 2 * t + hh], qf[t], s[jb]);
    }
    if (wc == 1) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) mask_block(s[jb], (const FM_LDS int*)vl, jb * 32, c0, i, p, hh);
    }
    float mx = max_acc(s);
    mx = max_x32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f((m_run - m_use) * p.sl2);
    const float msl = m_use * p.sl2;
    float rs = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[jb][r] = exp2f(__builtin_fmaf(s[jb][r], p.sl2, -msl));
        rs += s[jb][r];
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = jb * 32 + 8 * (t / 4) + 4 * hh + (t % 4);
          oacc[mb] = mfma32f(vs[key * VS + 32 * mb + (lane & 31)], s[jb][t], oacc[mb]);
        }
  }

  const float lt = sum_x32(l_run);
  float inv, row_lse;
  finish_row(lt, m_run, p.scale, p.sink != nullptr ? p.sink[h] : kNegInf, p.sink != nullptr, inv, row_lse);
  if (i < Nq) {
    float* og = reinterpret_cast<float*>(p.o) + (qslice + i) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = oacc[mb][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(og + 32 * mb + 8 * g + 4 * hh) = v4;
      }
    if (hh == 0) p.lse[qslice + i] = row_lse;
  }
  if (p.counts != nullptr && tid == 0) {
    atomicAdd(p.counts + 0, (unsigned long long)cnt0);
    atomicAdd(p.counts + 1, (unsigned long long)cnt1);
    atomicAdd(p.counts + 2, (unsigned long long)cnt2);
  }
}

// ---------------------------------------------------------------- launch
template <int D, int DV, int MODE>
static hipError_t launch_qmajor(FwdParams p, hipStream_t stream) {
  using C = QCfg<D, DV, MODE>;
  p.nqb = (p.Nq + C::BR - 1) / C::BR;
  const long long grid = (long long)p.B * p.H * p.nqb;
  hipLaunchKernelGGL((qmajor_bf16_kernel<D, DV, MODE>), dim3((unsigned)grid), dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 dQ pass
// The fp32 backward's dQ without atomics: query-major like the fp32
// forward, 4 waves x 32 rows per workgroup. Each lane holds its row of Q and
// dO as MFMA B operands; per visible 64-key tile, K and V go to LDS, then
//   S^T = K Q^T and dP^T = V dO^T (masked like the forward),
//   P = exp2(S * scale * log2e - LSE2), dS = P (dP - delta),
//   dQ^T += K^T dS^T,
// with LSE2 and delta from the preprocess. dQ sums in registers over the keys
// in a fixed order and is written once: bitwise deterministic.
template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(FwdParams p) {
  constexpr int BC = 64, BR = 128, KS = D + 1, VS = D + 4;
  __shared__ float ks[BC * KS];
  __shared__ float vs[BC * VS];
  __shared__ int vl[4 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  const int qb = p.nqb - 1 - (int)(blockIdx.x / BH);
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int r0 = qb * BR, r1 = min(Nq, r0 + BR);
  const int i = r0 + 32 * w + (lane & 31);
  const float* qg = reinterpret_cast<const float*>(p.q) + qslice * D;
  const float* kg = reinterpret_cast<const float*>(p.k) + kslice * D;
  const float* vg = reinterpret_cast<const float*>(p.v) + kslice * D;
  const float* dog = reinterpret_cast<const float*>(p.dout) + qslice * D;
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb * 8;

  float qf[D / 2], dof[D / 2];
#pragma unroll
  for (int t = 0; t < D / 2; ++t) {
    qf[t] = i < Nq ? qg[(long long)i * D + 2 * t + hh] : 0.f;
    dof[t] = i < Nq ? dog[(long long)i * D + 2 * t + hh] : 0.f;
  }
  // a row past Nq gets LSE2 = +inf, so its P (and dQ, not stored) is 0
  const float lse2 = i < Nq ? p.lse2[qslice + i] : __builtin_inff();
  const float delta = i < Nq ? p.delta[qslice + i] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) dq[mb] = f32x16{};
  float pd = 0.f;   // this lane's part of rowsum(dS), for the sink gradient

  for (int kb = 0; kb < p.nkb; ++kb) {
    const BlockBounds bb = load_bounds(table + (long long)kb * 8);
    const int c0 = kb * BC, c1 = min(Nk, c0 + BC);
    const int wgc = tile_class(bb, r0, r1, c0, c1, p.causal != 0);
    if (wgc == 0) continue;
    int wc = 0;
    const int a0 = r0 + 32 * w;
    if (a0 < Nq) {
      wc = tile_class(bb, a0, min(Nq, a0 + 32), c0, c1, p.causal != 0);
      if (c1 - c0 < BC && wc == 2) wc = 1;
    }
    __syncthreads();
    for (int t = tid; t < BC * D; t += 256) {
      const int row = t / D, col = t % D;
      const bool ok = c0 + row < Nk;
      ks[row * KS + col] = ok ? kg[(long long)(c0 + row) * D + col] : 0.f;
      vs[row * VS + col] = ok ? vg[(long long)(c0 + row) * D + col] : 0.f;
    }
    {
      const int vsel = tid >> 6, kk = tid & 63;
      const int32_t* src = vsel == 0 ? p.lts : vsel == 1 ? p.lte : vsel == 2 ? p.uts : p.ute;
      const bool present = src != nullptr && (vsel < 2 ? p.has_lt : p.has_ut);
      vl[vsel * 64 + kk] = (present && c0 + kk < Nk) ? src[vrow + c0 + kk] : 0;
    }
    __syncthreads();
    if (wc == 0) continue;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const int row = jb * 32 + (lane & 31);
#pragma unroll
      for (int t = 0; t < D / 2; ++t) {
        s = mfma32f(ks[row * KS + 2 * t + hh], qf[t], s);
        dp = mfma32f(vs[row * VS + 2 * t + hh], dof[t], dp);
      }
      if (wc == 1) mask_block(s, (const FM_LDS int*)vl, jb * 32, c0, i, p, hh);
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        ds[r] = exp2f(__builtin_fmaf(s[r], p.sl2, -lse2)) * (dp[r] - delta);
        pd += ds[r];
      }
      // dQ^T += K^T dS^T over the block's 32 keys
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = jb * 32 + 8 * (t / 4) + 4 * hh + (t % 4);
          dq[mb] = mfma32f(ks[key * KS + 32 * mb + (lane & 31)], ds[t], dq[mb]);
        }
    }
  }

  pd = sum_x32(pd);
  if (p.pdsum != nullptr && i < Nq && hh == 0) p.pdsum[qslice + i] = pd;
  if (i < Nq) {
    float* dqg = reinterpret_cast<float*>(p.dq) + (qslice + i) * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = dq[mb][4 * g + e] * p.scale;
        *reinterpret_cast<f32x4*>(dqg + 32 * mb + 8 * g + 4 * hh) = v4;
      }
  }
}

// the bf16 (d, dv) pairs compiled in (kept in step with bf16_dims())
template <int MODE>
static hipError_t dispatch_qmajor(int d, int dv, const FwdParams& p, hipStream_t stream) {
  if (d == 64 && dv == 64) return launch_qmajor<64, 64, MODE>(p, stream);
  if (d == 128 && dv == 128) return launch_qmajor<128, 128, MODE>(p, stream);
  if constexpr (MODE != kModeFwd) {   // (the (192, 128) forward runs the wide-head-dim kernels)
    if (d == 192 && dv == 128) return launch_qmajor<192, 128, MODE>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_fwd_f32(FwdParams p, hipStream_t stream) {
  p.nqb = (p.Nq + 127) / 128;
  const long long grid = (long long)p.B * p.H * p.nqb;
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, hipStream_t stream) {
  FwdParams p{};
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
  p.nkb = (a.Nk + kFwdBlockK - 1) / kFwdBlockK;
  if (wide_fwd_dims(a.d, a.dv, a.is_bf16)) return launch_wide_fwd(a, stream);
  if (a.is_bf16) {
    return dispatch_qmajor<kModeFwd>(a.d, a.dv, p, stream);
  } else {
    switch (a.d) {
      case 64: return launch_fwd_f32<64>(p, stream);
      case 128: return launch_fwd_f32<128>(p, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fm

namespace fm {

// dQ pass of the backward (query-major; see qmajor_bf16_kernel).
hipError_t launch_bwd_dq(const AttnArgs& a, hipStream_t stream) {
  FwdParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.lts = a.mask.lts;
  p.lte = a.mask.lte;
  p.uts = a.mask.uts;
  p.ute = a.mask.ute;
  p.table = a.table;
  p.dout = a.dout;
  p.o_in = a.o;
  p.lse_in = a.lse;
  p.lse2 = a.lse2;
  p.delta = a.delta;
  p.dq = a.dq;
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
  p.nkb = (a.Nk + kFwdBlockK - 1) / kFwdBlockK;
  if (!a.is_bf16) {
    // fp32: delta and the base-2 LSE come from the preprocess, already run
    p.pdsum = a.sink != nullptr ? a.pdsum : nullptr;
    p.nqb = (p.Nq + 127) / 128;
    const long long grid = (long long)p.B * p.H * p.nqb;
    switch (a.d) {
      case 64: hipLaunchKernelGGL(dq_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p); break;
      case 128: hipLaunchKernelGGL(dq_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // the dK/dV pass that follows on this stream takes work from these counters
  p.qzero = a.queue;
  if (a.sink != nullptr) {
    p.pdsum = a.pdsum;
    return dispatch_qmajor<kModeDqSink>(a.d, a.dv, p, stream);
  }
  return dispatch_qmajor<kModeDq>(a.d, a.dv, p, stream);
}

}  // namespace fm
