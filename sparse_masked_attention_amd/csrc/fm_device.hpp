// Device-side building blocks for the gfx950 kernels: vector types, buffer
// resources, the MFMA and transposed-LDS-read builtins, wait counters and the
// tile-classification rule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define FM_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------- buffers
// A raw buffer resource whose reads past `bytes` return zero without touching
// memory; this is what makes ragged tails (N not a multiple of a tile) safe.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ inline uint32_t uniform_u32(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

// 16 bytes per lane from `voffset` straight into LDS at lds_base + 16 * lane.
// Written as inline assembly on purpose: the compiler then does not track the
// LDS write, so it adds no wait of its own before later LDS reads; the caller
// orders the data with wait_vmcnt<>() and a barrier before anyone reads it.
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, FM_LDS void* lds_base, uint32_t voffset) {
  const uint32_t m0 = uniform_u32((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(r)
               : "memory", "m0");
}

__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that waits only for this wave's LDS operations (not for
// outstanding global loads, which may be prefetches still in flight). The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A copy of x the compiler must treat as unknown: values computed from it
// stay after this point instead of being hoisted out of enclosing loops.
__device__ inline int opaque_v(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The additive mask bias of one score: -inf where bit `bit` of w is set,
// else 0, in two instructions (a signed one-bit field is 0 or all ones, and
// all ones shifted left by 23 are the bits of -inf).
__device__ inline float mask_bias(uint32_t w, uint32_t bit) {
  return __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_sbfe((int)w, bit, 1u) << 23);
}

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// a wave-uniform pointer the compiler also knows to be uniform (scalar registers)
template <typename T>
__device__ inline T* uniform_ptr(T* x) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
  return reinterpret_cast<T*>(((unsigned long long)hi << 32) | lo);
}

// ---------------------------------------------------------------- LDS reads
__device__ inline bf16x8 lds_read_b128(const FM_LDS void* p) {
  return *reinterpret_cast<const FM_LDS bf16x8*>(p);
}

// Transposed read: in each group of 16 lanes, lane t receives element t % 4 of
// the 4 x 16-bit words addressed by lanes t/4, t/4 + 4, t/4 + 8, t/4 + 12 of
// its group. Pointed at a 4-row x 16-column block of a row-major bf16 tile
// (lane s -> row s/4, columns 4*(s%4)..+3), lane t gets 4 consecutive rows of
// column t.
__device__ inline bf16x4 lds_read_tr(const FM_LDS void* p) {
  typedef FM_LDS bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ inline bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------- MFMA
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma32f(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- math
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + sum of the 8 bf16 values of v, two per v_dot2_f32_bf16
__device__ inline float sum8_bf16(bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[e], v[e + 1]}, one, acc, false);
  return acc;
}

// Max over the 16 * NA accumulator values of a lane. A plain chain: measured
// faster than a balanced tree here, since the chain can start on the first
// accumulator while later MFMAs still run.
template <int NA>
__device__ inline float max_acc(const f32x16 (&s)[NA]) {
  float m = -__builtin_inff();
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, s[a][r]);
  return m;
}

// Combine x of lanes l and l ^ 32 (the two halves of a wave hold the same
// rows for different columns). v_permlane32_swap runs on the VALU, so the
// result never waits behind LDS traffic the way a ds_bpermute would; both
// halves receive the same bits because max and + are commutative.
__device__ inline float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- block order
// Workgroups are dispatched to the 8 XCDs round-robin by workgroup index, and
// each XCD has its own L2. Map grid index t to (head, block) so that every
// head stays on one XCD (its K/V, or Q/dO, stream is shared in that L2) while
// block indices still rise with t across all heads: callers put their
// heaviest blocks at low indices, and those must start first on every XCD,
// or the longest blocks end up in the tail of the launch. Falls back to
// head-fastest order when heads don't split evenly over the XCDs. A
// bijection on [0, heads * per_head) either way.
__device__ inline void xcd_order(int t, int heads, int per_head, int& head, int& blk) {
  constexpr int kXcd = 8;
  if (heads % kXcd == 0) {
    const int hpx = heads / kXcd;            // heads per XCD
    const int x = t % kXcd, m = t / kXcd;
    head = x + kXcd * (m % hpx);
    blk = m / hpx;
  } else {
    head = t % heads;
    blk = t / heads;
  }
}

// ---------------------------------------------------------------- row masks
// Bit r of the result is set when row q0 + r (0 <= r < 32) lies in [a, b).
// A key column's masked rows are a union of such intervals, so one word per
// (key, 32-row window) replaces an interval test per (row, key) element.
// Any int32 a, b is fine (clamped to the window before subtracting).
__device__ inline uint32_t row_bits(int a, int b, int q0) {
  const int lo = min(max(a, q0), q0 + 32) - q0;
  const int hi = max(min(max(b, q0), q0 + 32) - q0, lo);
  return (uint32_t)((1ull << hi) - (1ull << lo));
}

// Masked rows of key column j within the window [q0, q0 + 32): the causal
// part (rows before j), the lower interval [lts, lte) and the upper interval
// [uts, ute) (has_ut is false for causal masks). Keys at or past N mask
// every row.
__device__ inline uint32_t key_row_mask(int j, int q0, int N, bool causal, bool has_lt,
                                        bool has_ut, int lts, int lte, int uts, int ute) {
  uint32_t m = causal ? row_bits(q0, j, q0) : 0u;
  if (has_lt) m |= row_bits(lts, lte, q0);
  if (has_ut) m |= row_bits(uts, ute, q0);
  return j >= N ? ~0u : m;
}

// ---------------------------------------------------------------- row epilogue
// From a row's sum lt of exp(S - m) over its open keys (m the running
// offset, in raw score units before `scale`): the factor that turns the
// accumulated sum of P V into O, and the natural-log LSE. With a sink logit
// s (one more always-open entry with a zero value vector) the normaliser
// becomes exp(lse0) + exp(s): LSE = logaddexp(lse0, s), computed in the log
// domain so a large s cannot overflow, and O shrinks by exp(lse0 - LSE). A
// row with nothing open has O = 0 and LSE = -inf (s with a sink).
__device__ inline void finish_row(float lt, float m, float scale, float s, bool has_sink,
                                  float& inv, float& lse) {
  if (!(lt > 0.f)) {
    inv = 0.f;
    lse = has_sink ? s : kNegInf;
    return;
  }
  const float lse0 = m * scale + __logf(lt);
  if (!has_sink) {
    inv = 1.f / lt;
    lse = lse0;
    return;
  }
  const float hi = fmaxf(lse0, s);
  lse = hi + log1pf(__expf(-fabsf(lse0 - s)));
  inv = __expf(lse0 - lse) / lt;
}

// ---------------------------------------------------------------- mask rule
// Per key block: min/max of LTS, LTE, UTS, UTE (8 int32, in that order).
struct BlockBounds {
  int lts_mn, lts_mx, lte_mn, lte_mx, uts_mn, uts_mx, ute_mn, ute_mx;
};

__device__ inline BlockBounds load_bounds(const int32_t* t) {
  const i32x4* p = reinterpret_cast<const i32x4*>(t);
  i32x4 a = p[0], b = p[1];
  return BlockBounds{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Class of the tile rows [r0, r1) x columns [c0, c1) (both already clipped to
// N): 0 = every element masked (skip), 2 = no element masked, 1 = partial.
__device__ inline int tile_class(const BlockBounds& t, int r0, int r1, int c0, int c1, bool causal) {
  bool full = (causal && c0 > r1 - 1) || (t.lts_mx <= r0 && t.lte_mn >= r1) ||
              (!causal && t.uts_mx <= r0 && t.ute_mn >= r1);
  if (full) return 0;
  bool causal_free = !causal || (c1 - 1 <= r0);
  bool lt_free = (t.lte_mx <= r0) || (t.lts_mn >= r1);
  bool ut_free = causal || (t.ute_mx <= r0) || (t.uts_mn >= r1);
  return (causal_free && lt_free && ut_free) ? 2 : 1;
}

}  // namespace fm
