// Device-side helpers shared by the gfx950 kernels: chunk loads, orderable
// keys, wave64 / workgroup reductions and the cross-workgroup completion
// counter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_internal.hpp"

namespace ssd {

// dtype tags: 0 = float32 logits, 1 = bfloat16 logits
template <int DT> struct Dt;
template <> struct Dt<0> {
  using T = float;
  static constexpr int kPerVec = 4;      // elements per 16-byte load
  static constexpr int kKeyBits = 32;
  __device__ static float to_f(T v) { return v; }
};
template <> struct Dt<1> {
  using T = uint16_t;
  static constexpr int kPerVec = 8;
  static constexpr int kKeyBits = 16;
  __device__ static float to_f(T v) { return __uint_as_float(uint32_t(v) << 16); }
};

__device__ __forceinline__ bool is_finite_f(float x) { return __builtin_isfinite(x); }
__device__ __forceinline__ float pivot_of(float m) { return is_finite_f(m) ? m : 0.0f; }

// Order-preserving integer image of a logit (dtype bits; -0 folded onto +0),
// so larger key <=> larger value. bf16 values are exact in float, so the key
// is taken from the top 16 bits of the widened value.
template <int DT> __device__ __forceinline__ uint32_t key_of(float x);
template <> __device__ __forceinline__ uint32_t key_of<0>(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
template <> __device__ __forceinline__ uint32_t key_of<1>(float x) {
  uint32_t b = __float_as_uint(x) >> 16;
  if (b == 0x8000u) b = 0u;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
template <int DT> __device__ __forceinline__ float value_of_key(uint32_t k);
template <> __device__ __forceinline__ float value_of_key<0>(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
template <> __device__ __forceinline__ float value_of_key<1>(uint32_t k) {
  uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(b << 16);
}

// 64-bit rank key: key descending, then token index ascending.
__device__ __forceinline__ uint64_t rank_key(uint32_t key, int32_t idx) {
  return (uint64_t(key) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(idx));
}

// Unpack one 16-byte vector into floats x[o .. o + kPerVec).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& r, float* x) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (DT == 1) {
      x[2 * q] = __uint_as_float(w[q] << 16);
      x[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    } else {
      x[q] = __uint_as_float(w[q]);
    }
  }
}

// Raw dtype bits of one entry (bf16: the 16 stored bits).
template <int DT> __device__ __forceinline__ uint32_t raw_bits(typename Dt<DT>::T v);
template <> __device__ __forceinline__ uint32_t raw_bits<0>(float v) { return __float_as_uint(v); }
template <> __device__ __forceinline__ uint32_t raw_bits<1>(uint16_t v) { return uint32_t(v); }
// -inf as a packed 32-bit word of the dtype
template <int DT> __device__ __forceinline__ constexpr uint32_t neg_inf_word() {
  return DT == 1 ? 0xFF80FF80u : 0xFF800000u;
}

// One 16-byte vector built from per-entry reads of base[loc0 .. loc0+PV);
// entries at or past `lim` read as -inf. Indices are clamped so every read
// is unconditional and in bounds (lim >= 1).
template <int DT>
__device__ __forceinline__ uint4 gather_vec(const typename Dt<DT>::T* __restrict__ base, int loc0, int lim) {
  constexpr uint32_t kNeg = DT == 1 ? 0xFF80u : 0xFF800000u;
  uint32_t e[Dt<DT>::kPerVec];
#pragma unroll
  for (int q = 0; q < Dt<DT>::kPerVec; ++q) {
    const int l = loc0 + q;
    const uint32_t v = raw_bits<DT>(base[uint32_t(l < lim ? l : lim - 1)]);
    e[q] = l < lim ? v : kNeg;
  }
  if constexpr (DT == 1)
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
  else
    return make_uint4(e[0], e[1], e[2], e[3]);
}

// A chunk of 256 x PT entries held as raw 16-byte vectors, so callers need
// not keep PT floats per row live. STRIDED: vector j of thread t covers chunk entries
// (j*256 + t)*PV .. +PV (each wave load is one contiguous 1 KiB span);
// contiguous: entries t*32 + j*PV .. +PV. Entries past the row end read as
// -inf. Whole vectors of a 16-byte aligned row are single loads, all issued
// before the first use; a vector straddling the row end, or any vector of
// an unaligned row, is read per entry.
template <int DT, bool STRIDED, int PT = kPerThread>
struct ChunkVecs {
  static constexpr int PV = Dt<DT>::kPerVec;
  static constexpr int NV = PT / PV;
  static constexpr int kSpan = kThreads * PT;   // entries per chunk
  uint4 raw[NV];

  __device__ static int local(int tid, int j) {
    return STRIDED ? (j * kThreads + tid) * PV : tid * PT + j * PV;
  }
  __device__ static int64_t first(int64_t c0, int tid, int j) { return c0 + local(tid, j); }

  __device__ void issue_full(const typename Dt<DT>::T* __restrict__ row, int64_t c0, int tid) {
    const typename Dt<DT>::T* base = row + c0;
#pragma unroll
    for (int j = 0; j < NV; ++j) raw[j] = *reinterpret_cast<const uint4*>(base + uint32_t(local(tid, j)));
  }
  __device__ void load(const typename Dt<DT>::T* __restrict__ row, int64_t c0, int64_t V, bool aligned, int tid) {
    if (aligned && V - c0 >= kSpan) {
      issue_full(row, c0, tid);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      load_partial(row, c0, V, aligned, tid);
    }
  }
  // Tail chunk of an aligned row: whole vectors inside the row are single
  // loads (masked per lane), vectors wholly past the end read -inf; the one
  // vector straddling the end is filled in by patch_tail.
  __device__ void issue_tail(const typename Dt<DT>::T* __restrict__ row, int64_t c0, int lim, int tid) {
    const typename Dt<DT>::T* base = row + c0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int l = local(tid, j);
      raw[j].x = raw[j].y = raw[j].z = raw[j].w = neg_inf_word<DT>();
      if (l + PV <= lim) raw[j] = *reinterpret_cast<const uint4*>(base + uint32_t(l));
    }
  }
  // The vectors partition the chunk into PV-entry blocks, so at most one of
  // them (block lim / PV, when lim is not a multiple of PV) straddles the
  // end: one thread gathers it, one vector's worth of registers.
  __device__ void patch_tail(const typename Dt<DT>::T* __restrict__ row, int64_t c0, int lim, int tid) {
    const int vi = lim / PV;
    const int owner = STRIDED ? vi % kThreads : vi / NV;
    if (lim % PV != 0 && tid == owner) {
      const int js = STRIDED ? vi / kThreads : vi % NV;
      const uint4 g = gather_vec<DT>(row + c0, vi * PV, lim);
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (j == js) raw[j] = g;
    }
  }
  // unaligned row: per-entry reads, one vector at a time (rare path)
  __device__ void gather_all(const typename Dt<DT>::T* __restrict__ row, int64_t c0, int lim, int tid) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      raw[j] = gather_vec<DT>(row + c0, local(tid, j), lim);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // tail chunk (entries past V read -inf) or unaligned row
  __device__ void load_partial(const typename Dt<DT>::T* __restrict__ row, int64_t c0, int64_t V, bool aligned,
                               int tid) {
    const int64_t rem = V - c0;
    const int lim = rem < kSpan ? int(rem) : kSpan;
    if (aligned) {
      issue_tail(row, c0, lim, tid);
      __builtin_amdgcn_sched_barrier(0);
      patch_tail(row, c0, lim, tid);
    } else {
      gather_all(row, c0, lim, tid);
    }
  }
  __device__ void get(int j, float (&v)[PV]) const { unpack16<DT>(raw[j], v); }
  // Make the held vectors opaque to the optimiser, so values derived from
  // them are recomputed afterwards instead of being kept live in registers.
  __device__ void opaque() {
#pragma unroll
    for (int j = 0; j < NV; ++j) asm volatile("" : "+v"(raw[j].x), "+v"(raw[j].y), "+v"(raw[j].z), "+v"(raw[j].w));
  }
};

// The same chunk of two rows, with all loads of both in flight together
// when both rows are 16-byte aligned and the chunk is full.
template <int DT, bool STRIDED, int PT>
__device__ __forceinline__ void load_pair(ChunkVecs<DT, STRIDED, PT>& x, const typename Dt<DT>::T* __restrict__ rx,
                                          ChunkVecs<DT, STRIDED, PT>& y, const typename Dt<DT>::T* __restrict__ ry,
                                          int64_t c0, int64_t V, int tid) {
  const bool ax = (reinterpret_cast<uintptr_t>(rx) & 15u) == 0;
  const bool ay = (reinterpret_cast<uintptr_t>(ry) & 15u) == 0;
  if (ax && ay && V - c0 >= ChunkVecs<DT, STRIDED, PT>::kSpan) {
    x.issue_full(rx, c0, tid);
    y.issue_full(ry, c0, tid);
    __builtin_amdgcn_sched_barrier(0);
  } else if (ax && ay) {
    const int lim = int(V - c0);
    x.issue_tail(rx, c0, lim, tid);
    y.issue_tail(ry, c0, lim, tid);
    __builtin_amdgcn_sched_barrier(0);
    x.patch_tail(rx, c0, lim, tid);
    y.patch_tail(ry, c0, lim, tid);
  } else {
    x.load_partial(rx, c0, V, ax, tid);
    y.load_partial(ry, c0, V, ay, tid);
  }
}

// n / d for n < 2^31 (make_fastdiv(d)); uniform operands stay on the scalar unit.
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// ---- wave64 reductions on DPP lane moves (no LDS traffic) ----
// Within each row of 16 lanes: quad swaps, half-row mirror, row mirror;
// across rows: row_bcast15 / row_bcast31 fold rows 0+1 and 2+3, then 0..3.
// The full result lands in lane 63 (read with readlane: wave-uniform).
// Rows a row_mask leaves out keep `old`, which is the operation's identity.
namespace dpp {
constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kMirror = 0x140;
constexpr int kBcast15 = 0x142;
constexpr int kBcast31 = 0x143;
constexpr int kWaveShr1 = 0x138;   // wave_shr:1 (across rows)
constexpr int shr(int n) { return 0x110 + n; }
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int mov(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float movf(float old, float v) {
  return __int_as_float(mov<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double movd(double v) {   // 0.0 where the row is masked
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const int lo = mov<CTRL, ROWS>(0, int(uint32_t(b)));
  const int hi = mov<CTRL, ROWS>(0, int(uint32_t(b >> 32)));
  return __longlong_as_double(int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)));
}
// The same move for a reduction read from lane 63 only: no `old` operand.
// The permutes write every lane; a row broadcast leaves the rows outside its
// mask unwritten, and lane 63's chain (row 3, then rows 2 and 3) never reads
// them, so no zero has to be placed first.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double movd63(double v) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const int lo = __builtin_amdgcn_mov_dpp(int(uint32_t(b)), CTRL, ROWS, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(int(uint32_t(b >> 32)), CTRL, ROWS, 0xF, true);
  return __longlong_as_double(int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)));
}
__device__ __forceinline__ float lane63f(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }
__device__ __forceinline__ double lane63d(double v) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(b)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(b >> 32)), 63);
  return __longlong_as_double(int64_t((uint64_t(hi) << 32) | lo));
}
}  // namespace dpp

// wave max of a float, uniform result (NaN operands are ignored, as fmaxf
// does). The max runs on a signed-integer image of the bits that orders
// floats as their values (-0 just below +0), so each step is one DPP max.
__device__ __forceinline__ float wave_max_u(float v) {
  using namespace dpp;
  int i = __float_as_int(v == v ? v : -__builtin_inff());
  i ^= (i >> 31) & 0x7FFFFFFF;
  auto mx = [](int a, int b) { return a > b ? a : b; };
  const int id = int(0x80000000u);   // identity of the max for rows a row_mask leaves out
  i = mx(i, mov<kXor1>(id, i));
  i = mx(i, mov<kXor2>(id, i));
  i = mx(i, mov<kHalfMirror>(id, i));
  i = mx(i, mov<kMirror>(id, i));
  i = mx(i, mov<kBcast15, 0xA>(id, i));
  i = mx(i, mov<kBcast31, 0xC>(id, i));
  i = __builtin_amdgcn_readlane(i, 63);
  i ^= (i >> 31) & 0x7FFFFFFF;
  return __int_as_float(i);
}
// wave min of an unsigned int, uniform result
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  using namespace dpp;
  auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  const int id = -1;   // 0xFFFFFFFF: identity of min for rows a row_mask leaves out
  v = mn(v, uint32_t(mov<kXor1>(id, int(v))));
  v = mn(v, uint32_t(mov<kXor2>(id, int(v))));
  v = mn(v, uint32_t(mov<kHalfMirror>(id, int(v))));
  v = mn(v, uint32_t(mov<kMirror>(id, int(v))));
  v = mn(v, uint32_t(mov<kBcast15, 0xA>(id, int(v))));
  v = mn(v, uint32_t(mov<kBcast31, 0xC>(id, int(v))));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
// wave sum of a double, uniform result (fixed order: deterministic)
__device__ __forceinline__ double wave_sum_u(double v) {
  using namespace dpp;
  v += movd63<kXor1>(v);
  v += movd63<kXor2>(v);
  v += movd63<kHalfMirror>(v);
  v += movd63<kMirror>(v);
  v += movd63<kBcast15, 0xA>(v);
  v += movd63<kBcast31, 0xC>(v);
  return lane63d(v);
}
// inclusive prefix sum of an int over lanes 0..63
__device__ __forceinline__ int wave_scan_i(int v) {
  using namespace dpp;
  v += mov<shr(1)>(0, v);
  v += mov<shr(2)>(0, v);
  v += mov<shr(4)>(0, v);
  v += mov<shr(8)>(0, v);
  v += mov<kBcast15, 0xA>(0, v);
  v += mov<kBcast31, 0xC>(0, v);
  return v;
}

// ---- wave64 reductions and scans (DPP lane moves; call with the whole wave
// active). Reductions return the same value in every lane. ----
__device__ __forceinline__ float wave_max(float v) { return wave_max_u(v); }
__device__ __forceinline__ double wave_sum(double v) { return wave_sum_u(v); }
__device__ __forceinline__ int wave_sum_i(int v) {
  using namespace dpp;
  v += mov<kXor1>(0, v);
  v += mov<kXor2>(0, v);
  v += mov<kHalfMirror>(0, v);
  v += mov<kMirror>(0, v);
  v += mov<kBcast15, 0xA>(0, v);
  v += mov<kBcast31, 0xC>(0, v);
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  using namespace dpp;
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, uint32_t(mov<kXor1>(0, int(v))));
  v = mx(v, uint32_t(mov<kXor2>(0, int(v))));
  v = mx(v, uint32_t(mov<kHalfMirror>(0, int(v))));
  v = mx(v, uint32_t(mov<kMirror>(0, int(v))));
  v = mx(v, uint32_t(mov<kBcast15, 0xA>(0, int(v))));
  v = mx(v, uint32_t(mov<kBcast31, 0xC>(0, int(v))));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
// inclusive prefix sum over lanes 0..63 (lane is unused; kept for callers)
__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
  (void)lane;
  return wave_scan_i(v);
}
__device__ __forceinline__ double wave_incl_scan_d(double v, int lane) {
  using namespace dpp;
  (void)lane;
  v += movd<shr(1)>(v);
  v += movd<shr(2)>(v);
  v += movd<shr(4)>(v);
  v += movd<shr(8)>(v);
  v += movd<kBcast15, 0xA>(v);
  v += movd<kBcast31, 0xC>(v);
  return v;
}
// the value of lane lane - 1 (0 in lane 0)
__device__ __forceinline__ double wave_shift_up1_d(double v) { return dpp::movd<dpp::kWaveShr1>(v); }
// lane l's value (l the same in every lane)
__device__ __forceinline__ double lane_d(double v, int l) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b >> 32)), l));
  return __longlong_as_double(int64_t((uint64_t(hi) << 32) | lo));
}

// ---- workgroup (4 waves) reductions; all threads must call ----
__device__ __forceinline__ double block_sum(double v, double* sm4) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm4[w] = v;
  __syncthreads();
  return (sm4[0] + sm4[1]) + (sm4[2] + sm4[3]);
}
__device__ __forceinline__ int block_sum_i(int v, int* sm4) {
  v = wave_sum_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm4[w] = v;
  __syncthreads();
  return (sm4[0] + sm4[1]) + (sm4[2] + sm4[3]);
}

// ---- cross-workgroup exchange inside one kernel ----
// Workgroups on different XCDs do not share an L2, so partial results that
// another workgroup of the same launch reads are stored and loaded with
// device-scope (sc1) accesses, which are coherent across the XCDs' L2s.
// A device-scope release fence would also work but writes back the whole L2
// of the XCD on every arrival, which serialises thousands of workgroups.
__device__ __forceinline__ void dev_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t dev_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void dev_store32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_load32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Loads and stores of data exchanged between workgroups of one launch
// (COH: device-scope, as dev_load / dev_store) or only across launches
// (plain: kernel boundaries make them visible).
template <bool COH>
__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  if constexpr (COH) return dev_load(p);
  else return *p;
}
template <bool COH>
__device__ __forceinline__ void st64(uint64_t* p, uint64_t v) {
  if constexpr (COH) dev_store(p, v);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ void st32(int32_t* p, int32_t v) {
  if constexpr (COH) dev_store32(reinterpret_cast<uint32_t*>(p), uint32_t(v));
  else *p = v;
}
__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return uint64_t(__float_as_uint(a)) | (uint64_t(__float_as_uint(b)) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t w) { return __uint_as_float(uint32_t(w)); }
__device__ __forceinline__ uint64_t dbits(double v) { return uint64_t(__double_as_longlong(v)); }
__device__ __forceinline__ double bits_d(uint64_t w) { return __longlong_as_double((long long)w); }

// Weight that moves a sum of exp2((z - pa) * c) onto pivot pb (pa <= pb):
// 2^((pa - pb) * c), with the same float c as the per-entry exponentials so
// that the merged sum equals the sum taken with pivot pb directly.
__device__ __forceinline__ double rescale(float pa, float pb, float c32) {
  return double(__builtin_amdgcn_exp2f((pa - pb) * c32));
}

// Merge per-chunk (max, sum of exp2((z - pivot) * c)) partials of NR rows:
// row r's S partials sit at part + (r * S + chunk) * 2 (two 64-bit words:
// max in the low half of the first, sum in the second). One wave handles
// RPW rows at a time with one lane per chunk; a lane folds chunks lane,
// lane+64, ... in order, then fixed butterflies combine the lanes, so the
// result is the same on every run. Writes the merged row max (m_out, may be
// nullptr), its pivot and the sum relative to that pivot.
template <int RPW>
__device__ void merge_rows(const uint64_t* part, int NR, int S, float c32, float* piv_out,
                           double* s_out, float* m_out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int r0 = w * RPW; r0 < NR; r0 += 4 * RPW) {
    float ml[RPW];
    double sl[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      ml[j] = -__builtin_inff();
      sl[j] = 0.0;
    }
    for (int cc = lane; cc < S; cc += 64) {
      float qm[RPW];
      double qs[RPW];
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        qm[j] = -__builtin_inff();
        qs[j] = 0.0;
        if (r0 + j < NR) {
          const uint64_t* p = part + (int64_t(r0 + j) * S + cc) * 2;
          qm[j] = lo_f(dev_load(p));
          qs[j] = bits_d(dev_load(p + 1));
        }
      }
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        const float nm = fmaxf(ml[j], qm[j]);
        const float pn = pivot_of(nm);
        double acc = 0.0;
        if (sl[j] > 0.0) acc += sl[j] * rescale(pivot_of(ml[j]), pn, c32);
        if (qs[j] > 0.0) acc += qs[j] * rescale(pivot_of(qm[j]), pn, c32);
        ml[j] = nm;
        sl[j] = acc;
      }
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const float m = wave_max(ml[j]);
      const float pm = pivot_of(m);
      const double t = sl[j] > 0.0 ? sl[j] * rescale(pivot_of(ml[j]), pm, c32) : 0.0;
      const double sum = wave_sum(t);
      if (lane == 0 && r0 + j < NR) {
        piv_out[r0 + j] = pm;
        s_out[r0 + j] = sum;
        if (m_out) m_out[r0 + j] = m;
      }
    }
  }
}

// merge_rows for S <= 64 chunks per row, all partials in one round trip:
// each row gets a segment of G lanes (G = S rounded up to a power of two),
// one lane per chunk; segmented butterflies give the row max and the

// All-reduce over aligned segments of G lanes (G a power of two <= 64): the
// in-row DPP steps (quad swaps, half-row mirror, row mirror) reduce segments
// of up to 16 lanes; wider ones add one or two shuffles across rows.
__device__ __forceinline__ float seg_max(float v, int G) {
  using namespace dpp;
  if (G >= 2) v = fmaxf(v, movf<kXor1>(v, v));
  if (G >= 4) v = fmaxf(v, movf<kXor2>(v, v));
  if (G >= 8) v = fmaxf(v, movf<kHalfMirror>(v, v));
  if (G >= 16) v = fmaxf(v, movf<kMirror>(v, v));
  if (G >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if (G >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ double seg_sum(double v, int G) {
  using namespace dpp;
  if (G >= 2) v += movd<kXor1>(v);
  if (G >= 4) v += movd<kXor2>(v);
  if (G >= 8) v += movd<kHalfMirror>(v);
  if (G >= 16) v += movd<kMirror>(v);
  if (G >= 32) v += __shfl_xor(v, 16);
  if (G >= 64) v += __shfl_xor(v, 32);
  return v;
}

// rescaled sum (fixed order, deterministic).
__device__ inline void merge_rows_seg(const uint64_t* part, int NR, int S, float c32, float* piv_out,
                                      double* s_out) {
  int G = 1;
  while (G < S) G <<= 1;
  const int per_wave = 64 / G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int seg = lane / G, cl = lane - seg * G;
  for (int r0 = w * per_wave; r0 < NR; r0 += 4 * per_wave) {
    const int r = r0 + seg;
    float m = -__builtin_inff();
    double s = 0.0;
    if (r < NR && cl < S) {
      const uint64_t* p = part + (int64_t(r) * S + cl) * 2;
      m = lo_f(dev_load(p));
      s = bits_d(dev_load(p + 1));
    }
    const float mr = seg_max(m, G);
    const float pr = pivot_of(mr);
    const double t = seg_sum(s > 0.0 ? s * rescale(pivot_of(m), pr, c32) : 0.0, G);
    if (cl == 0 && r < NR) {
      piv_out[r] = pr;
      s_out[r] = t;
    }
  }
}

// exp2((z - piv) * c32) up to a factor common to a whole chunk, in one
// fused multiply-add: with P = piv * c32 rounded to float, the argument
// z * c32 - P is formed with a single rounding. Since the chunk's masses all
// share P, their sum is the sum of exp2((z - piv) * c32) times
// exp2(piv * c32 - P); scaled_mass_fix returns the inverse of that factor,
// from the product's rounding error, which the fused multiply-add gives
// exactly. Callers multiply their chunk total by it once.
struct ScaledPivot {
  float P;     // piv * c32, rounded
  float fix;   // exp2(P - piv * c32)
};
__device__ __forceinline__ ScaledPivot scaled_pivot(float piv, float c32) {
  const float P = piv * c32;
  const float err = __builtin_fmaf(piv, c32, -P);   // piv * c32 - P, exact
  return ScaledPivot{P, __builtin_amdgcn_exp2f(-err)};
}
__device__ __forceinline__ float scaled_mass(float z, float c32, float P) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(z, c32, -P));
}

// Statistics of one loaded chunk: the workgroup max m of the raw logits and
// the sum of exp2((z - pivot_of(m)) * c32). Each wave sums scaled_mass
// against its own maximum (per-thread float sums, double across lanes, then
// the wave's fix), so no barrier separates the max from the sum; one
// barrier then combines the four waves, rescaling each wave's sum to the
// chunk max. Called by every thread; both results are valid in every thread
// (sm_f: 4 floats, sm_s: 4 doubles of LDS).
template <int DT, int PT>
__device__ __forceinline__ void chunk_max_sum(const ChunkVecs<DT, true, PT>& cv, float c32, float* sm_f,
                                              double* sm_s, float& m_out, double& s_out) {
  constexpr int PV = Dt<DT>::kPerVec;
  using CV = ChunkVecs<DT, true, PT>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float m = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < CV::NV; ++j) {
    float v[PV];
    cv.get(j, v);
#pragma unroll
    for (int e = 0; e < PV; ++e) m = fmaxf(m, v[e]);
  }
  m = wave_max_u(m);
  const ScaledPivot sp = scaled_pivot(pivot_of(m), c32);
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < CV::NV; ++j) {
    float v[PV];
    cv.get(j, v);
#pragma unroll
    for (int e = 0; e < PV; ++e) sum += scaled_mass(v[e], c32, sp.P);
  }
  const double wsum = wave_sum_u(double(sum)) * double(sp.fix);
  if (lane == 0) {
    sm_f[w] = m;
    sm_s[w] = wsum;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(sm_f[0], sm_f[1]), fmaxf(sm_f[2], sm_f[3]));
  const float pM = pivot_of(M);
  double t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = sm_s[i] > 0.0 ? sm_s[i] * rescale(pivot_of(sm_f[i]), pM, c32) : 0.0;
  m_out = M;
  s_out = (t[0] + t[1]) + (t[2] + t[3]);
}

// Count this workgroup in; returns true in every thread of the workgroup that
// arrives last, which then reads the others' partials with dev_load. All
// data a workgroup leaves for others is stored by its thread 0 with
// dev_store, and thread 0 waits for those stores to complete before it
// moves the counter, so they are visible to whoever arrives last. The last
// arrival re-arms the counter for the next launch. No workgroup waits for
// another, so this cannot deadlock.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* sm_flag) {
  if (threadIdx.x == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (prev == expected - 1u);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sm_flag = last ? 1 : 0;
  }
  __syncthreads();
  return *sm_flag != 0;
}


}  // namespace ssd
