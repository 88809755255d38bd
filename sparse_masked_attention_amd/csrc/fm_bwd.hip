// Backward kernels: dQ, dK, dV of O = softmax(scale * Q K^T + M) V.
//
// The pages give the forward (FlashMask README "Formulation") and say FlashMask
// ships forward and backward kernels (README "Overview"). The gradient is the
// analytic one of that expression, recomputing the probabilities from the
// saved logsumexp so nothing of size N x N is stored (the FlashMask abstract
// credits FlashAttention with removing that O(N^2) memory):
//   P = exp(scale * Q K^T - LSE) on open pairs, dV = P^T dO,
//   dS = P * (dO V^T - delta), delta_i = sum_m dO[i][m] * O[i][m],
//   dQ = scale * dS K, dK = scale * dS^T Q.
//
// Two passes, no atomics (every gradient sums in a fixed order, so the
// results repeat bitwise):
//   * dQ pass, query-major (fm_fwd.hip: qmajor_bf16_kernel in its dQ mode,
//     dq_f32_kernel for fp32): each workgroup owns query rows, walks their
//     visible key tiles and sums dQ in registers. The bf16 pass also forms
//     delta and the base-2 LSE; for fp32 bwd_pre_kernel does.
//   * dK/dV pass, key-major (this file): a workgroup (4 waves) owns 128 keys,
//     32 per wave; K and V of those keys stay in registers as MFMA operands,
//     dK and dV accumulate in registers.
// gfx950 mapping of the bf16 dK/dV pass:
//   * It walks the query blocks (64 rows; 32 at d > 128) the mask leaves
//     visible, found by the same per-block min/max classification as the
//     forward, with a per-wave class so a wave whose 32 keys are hidden does
//     no math.
//   * Q and dO tiles (plus LSE and delta) arrive by buffer loads straight into
//     LDS, through three stages. P and dS are formed in the S = Q K^T accumulator
//     layout, which is directly the A operand of dV += P^T dO and
//     dK += dS^T Q; the Q/dO operands come from ds_read_b64_tr_b16.
//   * Because each lane owns one key, the element mask test of a partial tile
//     uses four per-lane registers (that key's bounds) and no memory.
//   * Workgroups are persistent (one per CU, taking key blocks from per-XCD
//     work queues) where the output rows can be staged through LDS: the next
//     key block's scan, first tiles, K and V are under way before the
//     finished block's dK and dV are stored.
#include <atomic>
#include <type_traits>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
  const int32_t* table;  // [B, hm, ceil(Nk/64), 8]
  float* delta;
  float* lse2;       // logsumexp in base-2 units; +inf for fully masked rows
  void* dq;
  void* dk;
  void* dv;
  unsigned long long* counts;
  int* queue;        // persistent dK/dV pass: one work-queue counter per queue, zero at launch
  int B, H, Nq, Nk, hm, causal;   // Nq query rows, Nk keys
  int has_lt, has_lte, has_ut;
  float scale, sl2;
  int nqb, nkb, nkb64;
  int nqueue, per_queue;
};

// ---------------------------------------------------------------- preprocess
// fp32 path and the wide head dims: delta_i = sum_m dO[i][m] * O[i][m] in
// float32; LSE in base-2 units (+inf where the row is fully masked, so
// exp2(s - LSE2) is 0 there). 16 threads per row, 16-byte chunks. (The
// other bf16 dims compute delta and the base-2 LSE inside their dQ pass.)
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  const long long rows = (long long)p.B * p.H * p.Nq;
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    const T* dog = reinterpret_cast<const T*>(p.dout) + row * D;
    const T* og = reinterpret_cast<const T*>(p.o) + row * D;
#pragma unroll
    for (int c = t; c < D / EPC; c += 16) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(dog + c * EPC);
      const u32x4 b = *reinterpret_cast<const u32x4*>(og + c * EPC);
      if constexpr (sizeof(T) == 2) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
      } else {
        const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += x[e] * y[e];
      }
    }
  }
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 16);
  if (row < rows && t == 0) {
    p.delta[row] = acc;
    const float l = p.lse[row];
    p.lse2[row] = l == kNegInf ? __builtin_inff() : l * kLog2e;
  }
}

// ---------------------------------------------------------------- dK / dV kernel
// Key-major: a workgroup (4 waves) owns 128 keys, 32 per wave, and walks the
// query blocks the mask leaves visible. K and V of the lane's key are MFMA B
// operands held in registers; dK and dV accumulate in registers. dQ is not
// formed here (the query-major dQ pass does it without atomics). (At
// d = dv = 256 the wide-head-dim kernels run the backward: dK and dV of 32
// keys per wave do not fit this kernel's registers.)
// D: head dim of Q and K (and dQ, dK); DV: head dim of V (and dO, dV).
template <int D, int DV>
struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr int KW = 32;                 // keys per wave
  static constexpr int BKC = NW * KW;           // keys per workgroup
#ifdef FM_ALT_TILES
  static constexpr int BQ = 32;                 // query rows per step (second configuration)
#else
  static constexpr int BQ = D > 128 ? 32 : 64;  // query rows per step
#endif
  static constexpr int CHQ = D / 8;             // 16-byte chunks per Q row
  static constexpr int CHO = DV / 8;            // 16-byte chunks per dO row
  static constexpr int QT = BQ * D * 2;         // bytes of one Q tile
  static constexpr int OT = BQ * DV * 2;        // bytes of one dO tile
  static constexpr int LOADS_Q = QT / (NW * 1024);
  static constexpr int LOADS_O = OT / (NW * 1024);
  static constexpr int STAGE = QT + OT + 2 * BQ * 4;  // Q, dO, LSE2, delta
  static constexpr int LIST = 1024;
  static constexpr int LOADS_PER_STEP = LOADS_Q + LOADS_O + 1;   // waves 0/1 add LSE2 / delta
  // Where a wave's 32 dK (and dV) rows fit a quarter of a stage, the rows go
  // out staged through LDS and the workgroups are persistent.
  static constexpr bool PERSIST = D == DV && NW * KW * D * 2 <= STAGE;
  static constexpr int NSTORE = D / 16 + DV / 16;   // 16-byte row stores per lane of dK and dV
};

// Chunk swizzle shared by row reads (32 rows, one chunk) and transposed reads
// (8 rows x 4 chunks) of the Q and dO tiles.
template <int W>
__device__ inline int swz(int row) {
  static_assert(W == 64 || W == 128 || W == 192, "row width");
  if constexpr (W == 192) return (row >> 1) & 7;   // 24 chunks: stay inside each group of 8
  else if constexpr (W == 128) return 4 * (row & 3) + ((row >> 2) & 3);
  else return 4 * (row & 1) + ((row >> 1) & 3);
}

// byte address of element (row, col) of a swizzled row-major bf16 tile W wide
template <int W>
__device__ inline const FM_LDS char* tile_addr(const FM_LDS char* base, int row, int col) {
  return base + row * W * 2 + (((col >> 3) ^ swz<W>(row)) << 4) + (col & 7) * 2;
}

template <int D, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  using C = BwdCfg<D, DV>;
  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[C::STAGE];
  __shared__ int list[C::LIST];
  __shared__ int wsum[C::NW];
  __shared__ unsigned wcount[3];
  __shared__ int next_item;
  constexpr bool kPersist = C::PERSIST;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  // This lane's index, its half-wave and index in it. They are re-derived
  // through an opaque copy before each pass over a tile list, so addresses
  // computed from them are not hoisted out of the item loop, where they would
  // hold registers through the scan and the epilogue as well.
  int lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  auto refresh_lane = [&]() {
    lane = opaque_v(tid) & 63;
    hh = lane >> 5;
    l32 = lane & 31;
  };
  const int BH = p.B * p.H;
  const int Nq = p.Nq, Nk = p.Nk;
  const uint32_t qbytes = (uint32_t)Nq * D * 2;    // one head of Q
  const uint32_t kbytes = (uint32_t)Nk * D * 2;    // one head of K
  const uint32_t vbytes = (uint32_t)Nk * DV * 2;   // one head of V
  const uint32_t obytes = (uint32_t)Nq * DV * 2;   // one head of dO
  const bool causal = p.causal != 0, has_lt = p.has_lt != 0, has_ut = p.has_ut != 0;
  if (tid < 3) wcount[tid] = 0;
  unsigned cnt0 = 0, cnt1 = 0, cnt2 = 0;

  // --- work items: (head, 128-key block). Without
  // persistence, workgroup t does item t. Persistent workgroups (one per CU)
  // take items from work queues: queue qi holds the items t = n * nqueue + qi
  // in the order n = 0, 1, ..., which with 8 queues keeps every item of a
  // head on one XCD (workgroup g serves queue g % 8 and the hardware deals
  // workgroups to the 8 XCDs in turn), heavy (early) key blocks first. A
  // workgroup takes its next item once the current one's tiles are done, and
  // ends when its queue is empty: every wave reaches the end.
  const int qi = kPersist ? (int)blockIdx.x % p.nqueue : 0;
  int item;
  if constexpr (kPersist) {
    if (tid == 0) next_item = atomicAdd(p.queue + qi, 1);
    __syncthreads();
    item = uniform(next_item);         // the same value in every lane and wave
    // unsigned: a counter holding anything but a ticket of this call ends
    // the workgroup instead of naming an item
    if ((unsigned)item >= (unsigned)p.per_queue) return;
  } else {
    item = (int)blockIdx.x;
  }

  // per-item state
  int bh, kb, c0, c1, wc0, j;
  long long qslice, kslice;
  __amdgpu_buffer_rsrc_t rq, rk, rv, rdo, rlse, rdel;
  const int32_t* table;
  bool tail;
  int k_lts, k_lte, k_uts, k_ute;
  auto setup = [&](int it) {
    xcd_order(kPersist ? it * p.nqueue + qi : it, BH, p.nkb, bh, kb);
    const int b = bh / p.H, h = bh % p.H;
    const int hmi = p.hm == 1 ? 0 : h;
    qslice = (long long)bh * Nq;           // rows of Q, dO, LSE, delta
    kslice = (long long)bh * Nk;           // rows of K, V, dK, dV
    c0 = kb * C::BKC;
    c1 = min(Nk, c0 + C::BKC);
    tail = c1 - c0 < C::BKC;
    wc0 = c0 + C::KW * w;                  // this wave's first key
    j = wc0 + l32;                         // this lane's key
    rq = make_rsrc(reinterpret_cast<const bf16*>(p.q) + qslice * D, qbytes);
    rk = make_rsrc(reinterpret_cast<const bf16*>(p.k) + kslice * D, kbytes);
    rv = make_rsrc(reinterpret_cast<const bf16*>(p.v) + kslice * DV, vbytes);
    rdo = make_rsrc(reinterpret_cast<const bf16*>(p.dout) + qslice * DV, obytes);
    rlse = make_rsrc(p.lse2 + qslice, (uint32_t)Nq * 4);
    rdel = make_rsrc(p.delta + qslice, (uint32_t)Nq * 4);
    table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;
  };
  // this lane's key bounds (the element test needs nothing else)
  auto load_key_bounds = [&]() {
    const int b = bh / p.H, h = bh % p.H;
    const long long vrow = ((long long)b * p.hm + (p.hm == 1 ? 0 : h)) * Nk;
    k_lts = Nq; k_lte = Nq; k_uts = 0; k_ute = 0;   // empty intervals
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
  };
  // K and V of this lane's key as the B operands of S = Q K^T and dP = dO V^T
  bf16x8 kB[D / 16], vB[DV / 16];
  auto load_kv = [&]() {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      kB[c] = __builtin_bit_cast(bf16x8, buffer_load16(rk, (uint32_t)(j * D + 16 * c + 8 * hh) * 2));
#pragma unroll
    for (int c = 0; c < DV / 16; ++c)
      vB[c] = __builtin_bit_cast(bf16x8, buffer_load16(rv, (uint32_t)(j * DV + 16 * c + 8 * hh) * 2));
  };

  f32x16 dvacc[DV / 32], dkacc[D / 32];
  auto zero_acc = [&]() {
#pragma unroll
    for (int mb = 0; mb < DV / 32; ++mb) dvacc[mb] = f32x16{};
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) dkacc[mb] = f32x16{};
  };

  auto issue = [&](unsigned entry, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    FM_LDS char* st = (FM_LDS char*)(S == 0 ? stage0 : S == 1 ? stage1 : stage2);
    const int q0 = (int)(entry & 0xFFFFFFu) * C::BQ;
#pragma unroll
    for (int u = 0; u < C::LOADS_Q; ++u) {
      const int g = (w * C::LOADS_Q + u) * 64 + lane;
      const int row = g / C::CHQ, pch = g % C::CHQ;
      load_lds16(rq, st + (w * C::LOADS_Q + u) * 1024,
                 (uint32_t)((q0 + row) * D + 8 * (pch ^ swz<D>(row))) * 2);
    }
#pragma unroll
    for (int u = 0; u < C::LOADS_O; ++u) {
      const int g = (w * C::LOADS_O + u) * 64 + lane;
      const int row = g / C::CHO, pch = g % C::CHO;
      load_lds16(rdo, st + C::QT + (w * C::LOADS_O + u) * 1024,
                 (uint32_t)((q0 + row) * DV + 8 * (pch ^ swz<DV>(row))) * 2);
    }
    // BQ base-2 LSE values then BQ delta values, 16 bytes per lane
    if (w < 2 && lane < C::BQ / 4)
      load_lds16(w == 0 ? rlse : rdel, st + C::QT + C::OT + w * C::BQ * 4, (uint32_t)(q0 + 4 * lane) * 4);
  };

  auto compute = [&](unsigned entry, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const int wc = (int)((entry >> (24 + 2 * w)) & 3u);
    if (wc == 0) return;
    const FM_LDS char* qst = (const FM_LDS char*)(S == 0 ? stage0 : S == 1 ? stage1 : stage2);
    const FM_LDS char* dost = qst + C::QT;
    const FM_LDS float* lse_l = (const FM_LDS float*)(qst + C::QT + C::OT);
    const FM_LDS float* del_l = lse_l + C::BQ;
    const int q0 = (int)(entry & 0xFFFFFFu) * C::BQ;
    bf16x8 pB[C::BQ / 16], dsB[C::BQ / 16];
    constexpr int NIB = C::BQ / 32;          // 32-row halves of the tile
    // The S accumulators start at the mask's additive bias (-inf where the
    // element is masked, else 0), so the MFMAs apply the mask and the code
    // below is the same for every tile class.
    f32x16 sacc[NIB], dpacc[NIB];
    if (wc == 1) {
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        // masked rows of this lane's key among rows q0 + 32 ib + [0, 32)
        // (rows past Nq too: their staged LSE is not +inf), shifted so that
        // bit 8 g + e is the row of register 4 g + e
        const int rb = q0 + 32 * ib;
        const uint32_t mw = (key_row_mask(j, rb, Nk, causal, has_lt, has_ut, k_lts, k_lte, k_uts, k_ute) |
                             row_bits(Nq, rb + 32, rb)) >> (4 * hh);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[ib][r] = mask_bias(mw, 8 * (r / 4) + r % 4);
      }
    } else {
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) sacc[ib] = f32x16{};
    }
    // Every MFMA below takes one operand from LDS. Those operands are read
    // PF MFMAs ahead through a ring of registers, in source order: with
    // registers this short the compiler keeps the written order, so the
    // order written here is the one that runs. extra(t) is VALU work for
    // the other row half, placed after MFMA t.
    constexpr int PF = 4;
    // Left alone, the scheduler sinks each read to just before its MFMA to
    // save registers, and every MFMA then waits out a full LDS latency. A
    // fence per step keeps reads and MFMAs where they are written; VALU,
    // SALU and transcendental work may still cross (mask 0x406).
    auto step_fence = [] { __builtin_amdgcn_sched_barrier(0x406); };
    // S = Q K^T + bias and dP = dO V^T for rows 32 ib .. 32 ib + 31; the two
    // accumulation chains alternate while both have steps left
    constexpr int NS = D / 16, NP = DV / 16, NSP = NS + NP, NSPMIN = NS < NP ? NS : NP;
    static_assert(NSP >= PF, "prefetch ring deeper than the S / dP steps");
    auto sdp = [&](int ib, auto extra) {
      dpacc[ib] = f32x16{};
      const int row = 32 * ib + l32;
      auto is_s = [](int t) { return t < 2 * NSPMIN ? (t & 1) == 0 : NS > NP; };
      auto chunk = [](int t) { return t < 2 * NSPMIN ? t >> 1 : t - NSPMIN; };
      auto rd = [&](int t) {
        return is_s(t) ? lds_read_b128(tile_addr<D>(qst, row, 16 * chunk(t) + 8 * hh))
                       : lds_read_b128(tile_addr<DV>(dost, row, 16 * chunk(t) + 8 * hh));
      };
      bf16x8 ring[PF];
#pragma unroll
      for (int t = 0; t < PF; ++t) ring[t] = rd(t);
#pragma unroll
      for (int t = 0; t < NSP; ++t) {
        const bf16x8 a = ring[t % PF];
        if (t + PF < NSP) ring[t % PF] = rd(t + PF);
        if (is_s(t)) sacc[ib] = mfma32(a, kB[chunk(t)], sacc[ib]);
        else dpacc[ib] = mfma32(a, vB[chunk(t)], dpacc[ib]);
        extra(t);
        step_fence();
      }
    };
    // P = exp2(S * scale * log2e - LSE2) and dS = P (dP - delta), as bf16
    // B operands, one accumulator register r of half ib at a time; fully
    // masked rows have LSE2 = +inf. Registers 4 g .. 4 g + 3 hold 4
    // consecutive rows whose LSE2 and delta come as one 16-byte read each,
    // issued one group ahead.
    f32x4 lsev[4], delv[4];
    auto probs_read = [&](int ib, int g) {
      const int rl = 32 * ib + 8 * g + 4 * hh;   // first of the 4 rows
      lsev[g] = *reinterpret_cast<const FM_LDS f32x4*>(lse_l + rl);
      delv[g] = *reinterpret_cast<const FM_LDS f32x4*>(del_l + rl);
    };
    auto probs_row = [&](int ib, int r) {
      const int g = r / 4, e = r % 4;
      if (e == 0 && g + 1 < 4) probs_read(ib, g + 1);
      const float pv = fast_exp2(__builtin_fmaf(sacc[ib][r], p.sl2, -lsev[g][e]));
      pB[2 * ib + r / 8][r % 8] = (bf16)pv;
      dsB[2 * ib + r / 8][r % 8] = (bf16)(pv * (dpacc[ib][r] - delv[g][e]));
    };
    // the 16 rows of half ib spread evenly over NT MFMA steps
    auto probs_spread = [&](int ib, int t, int NT) {
#pragma unroll
      for (int r = (16 * t + NT - 1) / NT; r < (16 * (t + 1) + NT - 1) / NT; ++r) probs_row(ib, r);
    };
    // dV += P^T dO and dK += dS^T Q over the 16-row chunks cc and cc + 1; the
    // dO / Q operands come by transposed reads, and dV and dK steps alternate
    // while both have steps left
    constexpr int NV2 = DV / 32, NK2 = D / 32, NC = NV2 + NK2;
    constexpr int NCMIN = NV2 < NK2 ? NV2 : NK2;
    static_assert(2 * NC >= PF, "prefetch ring deeper than the dV / dK steps");
    const int sl = lane & 15;
    const int cl = 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
    auto dvdk = [&](int cc, auto extra) {
      auto is_v = [](int u) { return u < 2 * NCMIN ? (u & 1) == 0 : NV2 > NK2; };
      auto mblk = [](int u) { return u < 2 * NCMIN ? u >> 1 : u - NCMIN; };
      auto rd = [&](int t) {
        const int c = cc + t / NC, u = t % NC;
        const int ra = 16 * c + 4 * hh + (sl >> 2);
        const int rb = ra + 8;
        if (is_v(u)) {
          const int col = 32 * mblk(u) + cl;
          return cat(lds_read_tr(tile_addr<DV>(dost, ra, col)), lds_read_tr(tile_addr<DV>(dost, rb, col)));
        }
        const int col = 32 * mblk(u) + cl;
        return cat(lds_read_tr(tile_addr<D>(qst, ra, col)), lds_read_tr(tile_addr<D>(qst, rb, col)));
      };
      bf16x8 ring[PF];
#pragma unroll
      for (int t = 0; t < PF; ++t) ring[t] = rd(t);
#pragma unroll
      for (int t = 0; t < 2 * NC; ++t) {
        const bf16x8 a = ring[t % PF];
        if (t + PF < 2 * NC) ring[t % PF] = rd(t + PF);
        const int c = cc + t / NC, u = t % NC;
        if (is_v(u)) dvacc[mblk(u)] = mfma32(pB[c], a, dvacc[mblk(u)]);
        else dkacc[mblk(u)] = mfma32(dsB[c], a, dkacc[mblk(u)]);
        extra(t);
        step_fence();
      }
    };
    // Pipelined over the two row halves: the exponentials of one half run on
    // the VALU between the MFMAs of the other; the scheduling fences keep
    // the compiler from regrouping the phases.
    auto none = [](int) {};
    sdp(0, none);
    __builtin_amdgcn_sched_barrier(0);
    probs_read(0, 0);
    if constexpr (NIB == 2) {
      sdp(1, [&](int t) { probs_spread(0, t, NSP); });
      __builtin_amdgcn_sched_barrier(0);
      probs_read(1, 0);
      dvdk(0, [&](int t) { probs_spread(1, t, 2 * NC); });
      __builtin_amdgcn_sched_barrier(0);
      dvdk(2, none);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) probs_row(0, r);
      __builtin_amdgcn_sched_barrier(0);
      dvdk(0, none);
    }
  };


  // --- scan the current item's query blocks from `base` on, compacting the
  // visible ones into the list, until the list is nearly full or no block
  // is left
  int cnt = 0, base = 0;
  auto scan = [&]() {
    // bounds of keys c0 .. c0 + 63 (waves 0, 1), c0 + 64 .. c0 + 127 (waves
    // 2, 3) and of both (read here, each time: kept across the tile loop
    // they would only take registers)
    static_assert(C::BKC == 128 && C::KW == 32, "two 64-key table entries per item, one per wave pair");
    const BlockBounds kb_lo = load_bounds(table + (long long)(c0 / 64) * 8);
    BlockBounds kb_hi = kb_lo, kbnd = kb_lo;
    if (c0 / 64 + 1 < p.nkb64) {   // else keys c0 + 64 .. are past Nk
      kb_hi = load_bounds(table + (long long)(c0 / 64 + 1) * 8);
      kbnd.lts_mn = min(kb_lo.lts_mn, kb_hi.lts_mn); kbnd.lts_mx = max(kb_lo.lts_mx, kb_hi.lts_mx);
      kbnd.lte_mn = min(kb_lo.lte_mn, kb_hi.lte_mn); kbnd.lte_mx = max(kb_lo.lte_mx, kb_hi.lte_mx);
      kbnd.uts_mn = min(kb_lo.uts_mn, kb_hi.uts_mn); kbnd.uts_mx = max(kb_lo.uts_mx, kb_hi.uts_mx);
      kbnd.ute_mn = min(kb_lo.ute_mn, kb_hi.ute_mn); kbnd.ute_mx = max(kb_lo.ute_mx, kb_hi.ute_mx);
    }
    cnt = 0;
    do {
      const int qb = base + tid;
      unsigned entry = 0;
      bool valid = false;
      if (qb < p.nqb) {
        const int r0 = qb * C::BQ, r1 = min(Nq, r0 + C::BQ);
        const int wgc = tile_class(kbnd, r0, r1, c0, c1, causal);
        cnt0 += wgc == 0;
        cnt1 += wgc == 1;
        cnt2 += wgc == 2;
        if (wgc != 0) {
          valid = true;
          const bool ragged = tail || (r1 - r0 < C::BQ);
          int bits = 0;
#pragma unroll
          for (int ww = 0; ww < C::NW; ++ww) {
            const int a0 = c0 + C::KW * ww;
            int cls = 0;
            if (a0 < Nk) {
              cls = tile_class(ww < 2 ? kb_lo : kb_hi, r0, r1, a0, min(Nk, a0 + C::KW), causal);
              if (ragged && cls == 2) cls = 1;
            }
            bits |= cls << (2 * ww);
          }
          entry = (unsigned)qb | ((unsigned)bits << 24);
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
      if (valid) list[off + rank] = (int)entry;
      __syncthreads();
      cnt += uniform(add);   // the same in every lane: the loops over the list stay scalar
      base += 256;
    } while (cnt <= C::LIST - 256 && base < p.nqb);
  };

  // --- the list's tiles. Three stages: tile it + 2 loads into the stage tile
  // it - 1 used, so one barrier per step covers both hazards (every wave's
  // loads of tile it have landed; no wave still reads the stage being
  // refilled), and each tile's loads have two steps to arrive. Steps below
  // `skip` know their tile has landed already.
  int skip = 0;
  auto issue_first = [&]() {
    if (cnt > 0) issue((unsigned)list[0], std::integral_constant<int, 0>{});
    if (cnt > 1) issue((unsigned)list[1], std::integral_constant<int, 1>{});
  };
  auto run = [&]() {
    auto step = [&](int it, auto stage_c) {
      constexpr int S = decltype(stage_c)::value;
      // uniform across the wave: keeps the class tests scalar branches
      const unsigned entry_it = uniform_u32((unsigned)list[it]);
      if (it >= skip) {
        if (it + 1 < cnt) {
          // tile it + 1's loads may stay in flight (waves 0 and 1 issue one
          // more load per tile, LSE2 / delta)
          if (w < 2) wait_vmcnt<C::LOADS_PER_STEP>();
          else wait_vmcnt<C::LOADS_PER_STEP - 1>();
        } else {
          wait_vmcnt<0>();
        }
      }
      lds_barrier();
      if (it + 2 < cnt) issue((unsigned)list[it + 2], std::integral_constant<int, (S + 2) % 3>{});
      compute(entry_it, stage_c);
    };
    for (int it = 0; it < cnt; it += 3) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < cnt) step(it + 1, std::integral_constant<int, 1>{});
      if (it + 2 < cnt) step(it + 2, std::integral_constant<int, 2>{});
    }
  };

  // key row kr, 16-byte chunk c of a W-wide staged row at kr * W * 2 + 16 (c ^ (kr & 7));
  // eh, el32: this lane's half-wave and index in it
  auto stage_rows = [&](FM_LDS char* st, const f32x16* acc, float mul, int eh, int el32, auto w_c) {
    constexpr int W = decltype(w_c)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r / 4) + 4 * eh + (r % 4);
#pragma unroll
      for (int mb = 0; mb < W / 32; ++mb) {
        const int col = 32 * mb + el32;
        *reinterpret_cast<FM_LDS bf16*>(st + kr * W * 2 + (((col >> 3) ^ (kr & 7)) << 4) + (col & 7) * 2) =
            (bf16)(acc[mb][r] * mul);
      }
    }
  };

  // --- first item: K and V, the key bounds and the table entries before the
  // scan. The wait also tells the compiler that nothing of its own is in
  // flight inside the tile loop, where its waits would otherwise stall on
  // the tile prefetch as well (the loads into LDS are invisible to it).
  setup(item);
  load_kv();
  load_key_bounds();
  zero_acc();
  wait_vmcnt<0>();
  scan();
  issue_first();
  for (;;) {
    refresh_lane();
    run();
    if (base < p.nqb) {   // more query blocks of this item
      scan();
      issue_first();
      skip = 0;
      continue;
    }
    if constexpr (!kPersist) {
      // --- write dK = scale * dS^T Q and dV for this wave's keys straight
      // from registers (a lane holds one column of 16 keys: 2 bytes per lane
      // and store; the rows are too wide for the stages)
      wait_vmcnt<0>();  // no load into LDS may still be in flight when the wave ends
      if (wc0 < Nk) {
        bf16* dkg = reinterpret_cast<bf16*>(p.dk) + kslice * D;
        bf16* dvg = reinterpret_cast<bf16*>(p.dv) + kslice * DV;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = wc0 + 8 * (r / 4) + 4 * hh + (r % 4);
          if (key < Nk) {
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
              dkg[(long long)key * D + 32 * mb + l32] = (bf16)(dkacc[mb][r] * p.scale);
#pragma unroll
            for (int mb = 0; mb < DV / 32; ++mb)
              dvg[(long long)key * DV + 32 * mb + l32] = (bf16)dvacc[mb][r];
          }
        }
      }
      break;
    } else {
      // --- the item is done. Its dK and dV rows (this wave's 32 keys) go out
      // through buffer resources that end at the last key, so stores past Nk
      // are dropped and every wave issues the same C::NSTORE stores.
      const int nrow = uniform(max(0, min(C::KW, Nk - wc0)));
      const __amdgpu_buffer_rsrc_t rdk =
          make_rsrc(uniform_ptr(reinterpret_cast<bf16*>(p.dk) + (kslice + wc0) * D),
                    nrow > 0 ? (uint32_t)(nrow * D) * 2 : 0u);
      const __amdgpu_buffer_rsrc_t rdv =
          make_rsrc(uniform_ptr(reinterpret_cast<bf16*>(p.dv) + (kslice + wc0) * DV),
                    nrow > 0 ? (uint32_t)(nrow * DV) * 2 : 0u);
      // the next item: its ticket is taken here (nothing else is in flight)
      __syncthreads();   // no wave still reads this item's list, stages or the last ticket
      if (tid == 0) next_item = atomicAdd(p.queue + qi, 1);
      __syncthreads();
      const int nitem = uniform(next_item);
      const bool more = (unsigned)nitem < (unsigned)p.per_queue;   // the same in every wave
      if (more) {
        // Start the next item before this one's stores: its scan, its first
        // two tiles (stages 0 and 1), then its K, V and key bounds. The
        // stores below are then the last vector-memory operations in flight,
        // and a wait that leaves just them outstanding finds all of this
        // landed.
        item = nitem;
        setup(item);
        base = 0;
        scan();
        issue_first();
        load_kv();
        load_key_bounds();
      }
      __builtin_amdgcn_sched_barrier(0);
      // dK = scale * dS^T Q, then dV, through this wave's quarter of stage 2
      // (free: the next item's first tiles are in stages 0 and 1). A lane
      // holds one column of 16 keys; staged, each store writes whole rows,
      // 16 bytes per lane.
      FM_LDS char* est = (FM_LDS char*)stage2 + w * C::KW * D * 2;
      // The lane index is re-derived here through an opaque copy: addresses
      // computed from it cannot then be hoisted above the tile loop, where
      // they would hold registers for the whole item.
      const int elane = opaque_v(tid) & 63;
      auto store_rows = [&](__amdgpu_buffer_rsrc_t r, int ld, auto w_c) {
        constexpr int W = decltype(w_c)::value;
        constexpr int CH = W / 8;
#pragma unroll
        for (int k = 0; k < CH / 2; ++k) {
          const int f = 64 * k + elane;
          const int row = f / CH, c = f % CH;
          const u32x4 val = *reinterpret_cast<const FM_LDS u32x4*>(est + row * W * 2 + ((c ^ (row & 7)) << 4));
          __builtin_amdgcn_raw_buffer_store_b128(val, r, (uint32_t)(row * ld + 8 * c) * 2, 0, 0);
        }
      };
      stage_rows(est, dkacc, p.scale, elane >> 5, elane & 31, std::integral_constant<int, D>{});
      __builtin_amdgcn_wave_barrier();
      store_rows(rdk, D, std::integral_constant<int, D>{});
      stage_rows(est, dvacc, 1.f, elane >> 5, elane & 31, std::integral_constant<int, DV>{});
      __builtin_amdgcn_wave_barrier();
      store_rows(rdv, DV, std::integral_constant<int, DV>{});
      __builtin_amdgcn_sched_barrier(0);
      // the next item's first two tiles, K, V and key bounds have landed;
      // only the stores may be in flight. (Waited for on both paths, so that
      // the compiler also sees K and V landed wherever the loop continues.)
      wait_vmcnt<C::NSTORE>();
      if (!more) break;
      zero_acc();
      skip = 2;
    }
  }
  wait_vmcnt<0>();
  if (p.counts != nullptr) {
    atomicAdd(&wcount[0], cnt0);
    atomicAdd(&wcount[1], cnt1);
    atomicAdd(&wcount[2], cnt2);
    __syncthreads();
    if (tid < 3) atomicAdd(p.counts + tid, (unsigned long long)wcount[tid]);
  }
}

// ---------------------------------------------------------------- fp32 kernel
// dK and dV of the fp32 backward (dQ comes from the query-major fp32 dQ
// pass): the same key-major decomposition with v_mfma_f32_32x32x2_f32 and
// everything staged through LDS with plain loads (no pipelining): 4 waves x
// 32 keys, query steps of 32 rows. K and V of the lane's key sit in
// registers as B operands.
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_f32_kernel(BwdParams p) {
  constexpr int KW = 32, BKC = 128, BQ = 32, S1 = D + 1;
  __shared__ float qs[BQ * S1];
  __shared__ float dos[BQ * S1];
  __shared__ float lse_s[BQ];
  __shared__ float del_s[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  const int kb = (int)(blockIdx.x / BH);
  const int b = bh / p.H, h = bh % p.H;
  const int hmi = p.hm == 1 ? 0 : h;
  const int Nq = p.Nq, Nk = p.Nk;
  const long long qslice = (long long)bh * Nq, kslice = (long long)bh * Nk;
  const int c0 = kb * BKC, c1 = min(Nk, c0 + BKC);
  const int wc0 = c0 + KW * w;
  const int j = wc0 + l32;
  const float* qg = reinterpret_cast<const float*>(p.q) + qslice * D;
  const float* kg = reinterpret_cast<const float*>(p.k) + kslice * D;
  const float* vg = reinterpret_cast<const float*>(p.v) + kslice * D;
  const float* dog = reinterpret_cast<const float*>(p.dout) + qslice * D;

  float kr[D / 2], vr[D / 2];
#pragma unroll
  for (int t = 0; t < D / 2; ++t) {
    kr[t] = j < Nk ? kg[(long long)j * D + 2 * t + hh] : 0.f;
    vr[t] = j < Nk ? vg[(long long)j * D + 2 * t + hh] : 0.f;
  }
  const long long vrow = ((long long)b * p.hm + hmi) * Nk;
  int k_lts = Nq, k_lte = Nq, k_uts = 0, k_ute = 0;   // empty intervals
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
  f32x16 dvacc[D / 32], dkacc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    dvacc[mb] = f32x16{};
    dkacc[mb] = f32x16{};
  }
  const int32_t* table = p.table + ((long long)b * p.hm + hmi) * p.nkb64 * 8;
  BlockBounds kbnd = load_bounds(table + (long long)(c0 / 64) * 8);
  if (c0 / 64 + 1 < p.nkb64) {
    const BlockBounds q = load_bounds(table + (long long)(c0 / 64 + 1) * 8);
    kbnd.lts_mn = min(kbnd.lts_mn, q.lts_mn); kbnd.lts_mx = max(kbnd.lts_mx, q.lts_mx);
    kbnd.lte_mn = min(kbnd.lte_mn, q.lte_mn); kbnd.lte_mx = max(kbnd.lte_mx, q.lte_mx);
    kbnd.uts_mn = min(kbnd.uts_mn, q.uts_mn); kbnd.uts_mx = max(kbnd.uts_mx, q.uts_mx);
    kbnd.ute_mn = min(kbnd.ute_mn, q.ute_mn); kbnd.ute_mx = max(kbnd.ute_mx, q.ute_mx);
  }
  const BlockBounds wbnd = load_bounds(table + (long long)(min(wc0, Nk - 1) / 64) * 8);
  unsigned cnt0 = 0, cnt1 = 0, cnt2 = 0;

  for (int qb = 0; qb < p.nqb; ++qb) {
    const int q0 = qb * BQ, q1 = min(Nq, q0 + BQ);
    const int wgc = tile_class(kbnd, q0, q1, c0, c1, p.causal != 0);
    cnt0 += wgc == 0;
    cnt1 += wgc == 1;
    cnt2 += wgc == 2;
    if (wgc == 0) continue;
    int wc = 0;
    if (wc0 < Nk) {
      wc = tile_class(wbnd, q0, q1, wc0, min(Nk, wc0 + KW), p.causal != 0);
      if (wc == 2 && (q1 - q0 < BQ || c1 - c0 < BKC)) wc = 1;
    }
    __syncthreads();  // previous step's readers are done
    for (int t = tid; t < BQ * D; t += 256) {
      const int row = t / D, col = t % D;
      const bool ok = q0 + row < Nq;
      qs[row * S1 + col] = ok ? qg[(long long)(q0 + row) * D + col] : 0.f;
      dos[row * S1 + col] = ok ? dog[(long long)(q0 + row) * D + col] : 0.f;
    }
    if (tid < BQ) {
      const bool ok = q0 + tid < Nq;
      lse_s[tid] = ok ? p.lse2[qslice + q0 + tid] : __builtin_inff();
      del_s[tid] = ok ? p.delta[qslice + q0 + tid] : 0.f;
    }
    __syncthreads();
    f32x16 pr = f32x16{}, dsr = f32x16{};
    if (wc != 0) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 2; ++t) {
        sacc = mfma32f(qs[l32 * S1 + 2 * t + hh], kr[t], sacc);
        dpacc = mfma32f(dos[l32 * S1 + 2 * t + hh], vr[t], dpacc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 8 * (r / 4) + 4 * hh + (r % 4);
        const int i = q0 + il;
        float sv = sacc[r];
        if (wc == 1) {
          bool m = (i >= Nq) || (j >= Nk) || (p.causal && j > i);
          m = m || (k_lts <= i && i < k_lte) || (k_uts <= i && i < k_ute);
          if (m) sv = kNegInf;
        }
        const float pv = exp2f(__builtin_fmaf(sv, p.sl2, -lse_s[il]));
        pr[r] = pv;
        dsr[r] = pv * (dpacc[r] - del_s[il]) * p.scale;
      }
      // dV += P^T dO and dK += dS^T Q over the step's 32 rows
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int il = 8 * (t / 4) + 4 * hh + (t % 4);
          dvacc[mb] = mfma32f(pr[t], dos[il * S1 + 32 * mb + l32], dvacc[mb]);
          dkacc[mb] = mfma32f(dsr[t], qs[il * S1 + 32 * mb + l32], dkacc[mb]);
        }
    }
  }
  if (wc0 < Nk) {
    float* dkg = reinterpret_cast<float*>(p.dk) + kslice * D;
    float* dvg = reinterpret_cast<float*>(p.dv) + kslice * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = wc0 + 8 * (r / 4) + 4 * hh + (r % 4);
        if (key < Nk) {
          dkg[(long long)key * D + 32 * mb + l32] = dkacc[mb][r];
          dvg[(long long)key * D + 32 * mb + l32] = dvacc[mb][r];
        }
      }
  }
  if (p.counts != nullptr && tid == 0) {
    atomicAdd(p.counts + 0, (unsigned long long)cnt0);
    atomicAdd(p.counts + 1, (unsigned long long)cnt1);
    atomicAdd(p.counts + 2, (unsigned long long)cnt2);
  }
}

// ---------------------------------------------------------------- launch
template <int D, typename T>
static hipError_t launch_pre(const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H * p.Nq;
  const long long blocks = (rows + 15) / 16;
  hipLaunchKernelGGL((bwd_pre_kernel<D, T>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// compute units of the current device, cached per device. Host threads may
// call this at once: each slot is an atomic, and a thread that finds it
// empty queries the runtime and stores the (same) answer.
static int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int DV>
static hipError_t launch_bwd_bf16(BwdParams p, const AttnArgs& a, hipStream_t stream) {
  using C = BwdCfg<D, DV>;
  p.nqb = (p.Nq + C::BQ - 1) / C::BQ;
  // the dQ pass also writes delta and the base-2 LSE the dK/dV pass reads
  const hipError_t e = launch_bwd_dq(a, stream);
  if (e != hipSuccess) return e;
  const long long items = (long long)p.B * p.H * p.nkb;
  long long grid = items;
  if constexpr (C::PERSIST) {
    // one workgroup per CU, 8 queues (one per XCD) when the heads split
    // evenly over them; the dQ pass has zeroed the counters
    if (a.queue == nullptr) return hipErrorInvalidValue;
    p.queue = a.queue;
    p.nqueue = (p.B * p.H) % 8 == 0 ? 8 : 1;
    p.per_queue = (int)(items / p.nqueue);
    const int ncu = cu_count();
    if (ncu <= 0) return hipErrorInvalidDevice;
    const long long slots = ncu >= p.nqueue ? ncu / p.nqueue * p.nqueue : p.nqueue;
    grid = items < slots ? items : slots;
  }
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, DV>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_f32(BwdParams p, const AttnArgs& a, hipStream_t stream) {
  p.nqb = (p.Nq + 31) / 32;
  // delta and the base-2 LSE, then the query-major dQ pass (no atomics),
  // then dK and dV
  hipError_t e = launch_pre<D, float>(p, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd_dq(a, stream);
  if (e != hipSuccess) return e;
  const long long grid = (long long)p.B * p.H * p.nkb;
  hipLaunchKernelGGL(bwd_f32_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- sink gradient
// d loss / d s_h = -sum over the head's rows of p_i * D_i, with p_i =
// exp(s_h - LSE_i) the sink's share of row i (the sink is one more softmax
// entry with a zero value vector, so d O_i / d s_h = -p_i * O_i) and
// D_i = rowsum(P * dP)_i = dO_i . O_i. D_i is not taken from the bf16 O:
// this sum over every row would collect O's rounding. Instead
// D_i = rowsum(dS)_i + delta_i * (1 - p_i), which equals it exactly because
// dS = P (dP - delta) and the row of P sums to 1 - p_i; rowsum(dS) comes from
// the dQ pass, where the delta error cancels. One workgroup per head, a
// fixed summation order (per-thread strides, then wave shuffles, then the 4
// waves in order): deterministic. `have_rows` is false when no row saw a key
// (then every O_i, and so every term, is 0).
__global__ __launch_bounds__(256) void sink_grad_kernel(const float* __restrict__ lse2,
                                                        const float* __restrict__ delta,
                                                        const float* __restrict__ dssum,
                                                        const float* __restrict__ sink,
                                                        float* __restrict__ dsink, int B, int H,
                                                        int Nq, int have_rows) {
  const int h = blockIdx.x;
  const float s2 = sink[h] * kLog2e;
  float acc = 0.f;
  if (have_rows) {
    for (int b = 0; b < B; ++b) {
      const long long base = ((long long)b * H + h) * Nq;
      for (int i = threadIdx.x; i < Nq; i += 256) {
        const float pi = exp2f(s2 - lse2[base + i]);
        acc += pi * (dssum[base + i] + delta[base + i] * (1.f - pi));
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) dsink[h] = -(((part[0] + part[1]) + part[2]) + part[3]);
}

static hipError_t launch_sink_grad(const AttnArgs& a, bool have_rows, hipStream_t stream) {
  if (a.sink == nullptr || a.dsink == nullptr || a.H == 0) return hipSuccess;
  hipLaunchKernelGGL(sink_grad_kernel, dim3((unsigned)a.H), dim3(256), 0, stream, a.lse2, a.delta, a.pdsum,
                     a.sink, a.dsink, a.B, a.H, a.Nq, have_rows ? 1 : 0);
  return hipGetLastError();
}

// dsink = 0 for a problem with no query row or no batch element
hipError_t launch_sink_zero(const float* sink, float* dsink, int H, hipStream_t stream) {
  AttnArgs a{};
  a.sink = sink;
  a.dsink = dsink;
  a.H = H;
  return launch_sink_grad(a, false, stream);
}

// ---------------------------------------------------------------- zero fill
// Gradients of a side with no partner (no keys, or no query rows) are zero.
__global__ __launch_bounds__(256) void zero_kernel(u32x4* __restrict__ p, long long n16) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

static hipError_t launch_zero(void* p, long long bytes, hipStream_t stream) {
  const long long n16 = bytes / 16;   // row sizes are multiples of 16 bytes
  if (n16 == 0) return hipSuccess;
  long long blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

static hipError_t launch_bwd_main(const AttnArgs& a, hipStream_t stream);

hipError_t launch_bwd(const AttnArgs& a, hipStream_t stream) {
  const long long elt = a.is_bf16 ? 2 : 4;
  if (a.Nk == 0) {
    const hipError_t e = launch_zero(a.dq, (long long)a.B * a.H * a.Nq * a.d * elt, stream);
    if (e != hipSuccess) return e;
    return launch_sink_grad(a, false, stream);
  }
  if (a.Nq == 0) {
    hipError_t e = launch_zero(a.dk, (long long)a.B * a.H * a.Nk * a.d * elt, stream);
    if (e != hipSuccess) return e;
    e = launch_zero(a.dv_out, (long long)a.B * a.H * a.Nk * a.dv * elt, stream);
    if (e != hipSuccess) return e;
    return launch_sink_grad(a, false, stream);
  }
  const hipError_t e = launch_bwd_main(a, stream);
  if (e != hipSuccess) return e;
  // delta and the base-2 LSE are in the workspace now (dQ pass or preprocess)
  return launch_sink_grad(a, true, stream);
}

static hipError_t launch_bwd_main(const AttnArgs& a, hipStream_t stream) {
  BwdParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.dout = a.dout;
  p.lts = a.mask.lts;
  p.lte = a.mask.lte;
  p.uts = a.mask.uts;
  p.ute = a.mask.ute;
  p.table = a.table;
  p.delta = a.delta;
  p.lse2 = a.lse2;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv_out;
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
  p.nkb = (a.Nk + kBwdBlockK - 1) / kBwdBlockK;
  p.nkb64 = (a.Nk + kTableBlock - 1) / kTableBlock;
  if (wide_bwd_dims(a.d, a.dv, a.is_bf16)) {
    // delta and the base-2 LSE, then the wide dQ and dK/dV passes
    p.nqb = (p.Nq + 31) / 32;
    // (the preprocess reads rows of O and dO, dv wide)
    const hipError_t e = a.is_bf16   ? (a.dv == 512 ? launch_pre<512, bf16>(p, stream)
                                                    : launch_pre<256, bf16>(p, stream))
                         : a.dv == 256 ? launch_pre<256, float>(p, stream)
                                       : launch_pre<128, float>(p, stream);
    if (e != hipSuccess) return e;
    return launch_wide_bwd(a, stream);
  }
  if (a.is_bf16) {
    // the bf16 (d, dv) pairs compiled in (kept in step with bf16_dims())
    if (a.d == 64 && a.dv == 64) return launch_bwd_bf16<64, 64>(p, a, stream);
    if (a.d == 128 && a.dv == 128) return launch_bwd_bf16<128, 128>(p, a, stream);
    if (a.d == 192 && a.dv == 128) return launch_bwd_bf16<192, 128>(p, a, stream);
  } else {
    switch (a.d) {
      case 64: return launch_bwd_f32<64>(p, a, stream);
      case 128: return launch_bwd_f32<128>(p, a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fm
