// Device-side primitives shared by the libpkv kernels (gfx950): element conversions, streaming
// and direct-to-LDS loads, explicit wait counters, cross-row lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pkv {
namespace dev {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2;
constexpr int kTile = 16;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

template <int DT>
constexpr int elem_size() { return DT == DT_F32 ? 4 : 2; }

__device__ inline float neg_inf() { return -__builtin_inff(); }
__device__ inline float qnan() { return __builtin_nanf(""); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two packed 16-bit elements -> two floats (exact).
template <int DT>
__device__ inline void unpack2(uint32_t w, float& lo, float& hi) {
  if constexpr (DT == DT_BF16) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  } else {
    lo = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
    hi = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
  }
}

// float -> element bits, round to nearest even.
template <int DT>
__device__ inline void store_elem(void* base, int64_t idx, float x) {
  if constexpr (DT == DT_F32) {
    static_cast<float*>(base)[idx] = x;
  } else if constexpr (DT == DT_BF16) {
    uint32_t u = __float_as_uint(x);
    uint16_t r;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      r = 0x7fc0;  // NaN
    } else {
      r = static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
    static_cast<uint16_t*>(base)[idx] = r;
  } else {
    static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);
  }
}

// Element x rounded to the storage type, as raw bits (bf16: round to nearest even, NaN kept).
template <int DT>
__device__ inline uint32_t elem_bits(float x) {
  if constexpr (DT == DT_F32) {
    return __float_as_uint(x);
  } else if constexpr (DT == DT_BF16) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  } else {
    const _Float16 h = static_cast<_Float16>(x);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
  }
}

// N consecutive elements (8 bytes, or a multiple of 16) stored at base[idx...], rounded as
// store_elem rounds them, with 8- or 16-byte stores; base + idx must be aligned to that size.
template <int DT, int N>
__device__ inline void store_row(void* base, int64_t idx, const float (&x)[N]) {
  constexpr int E = elem_size<DT>();
  static_assert(N * E == 8 || (N * E) % 16 == 0, "whole 8- or 16-byte stores");
  char* dst = static_cast<char*>(base) + idx * E;
  if constexpr (N * E == 8) {
    u32x2 w;
    if constexpr (E == 4) {
      w = u32x2{elem_bits<DT>(x[0]), elem_bits<DT>(x[1])};
    } else {
      w = u32x2{elem_bits<DT>(x[0]) | (elem_bits<DT>(x[1]) << 16), elem_bits<DT>(x[2]) | (elem_bits<DT>(x[3]) << 16)};
    }
    *reinterpret_cast<u32x2*>(dst) = w;
    return;
  }
#pragma unroll
  for (int c = 0; c < (N * E) / 16; ++c) {
    u32x4 w;
    if constexpr (E == 4) {
      w = u32x4{elem_bits<DT>(x[4 * c]), elem_bits<DT>(x[4 * c + 1]), elem_bits<DT>(x[4 * c + 2]),
                elem_bits<DT>(x[4 * c + 3])};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = elem_bits<DT>(x[8 * c + 2 * i]) | (elem_bits<DT>(x[8 * c + 2 * i + 1]) << 16);
    }
    *reinterpret_cast<u32x4*>(dst + 16 * c) = w;
  }
}

// Rotary embedding of one pair (x1, x2) = (x[i], x[i + D/2]) by the angle whose cosine and sine
// are c and s: y1 = x1 c - x2 s, y2 = x2 c + x1 s, in float32 with each product and each sum
// rounded to nearest even (contraction into fused multiply-adds is switched off here, so the
// result is the same on every path that calls it).
__device__ inline void rope_pair(float x1, float x2, float c, float s, float& y1, float& y2) {
#pragma clang fp contract(off)
  const float a = x1 * c, b = x2 * s, e = x2 * c, f = x1 * s;
  y1 = a - b;
  y2 = e + f;
}

// 16 bytes of elements <-> floats: 8 for 16-bit types, 4 for float32.
template <int DT>
struct Vec16 {
  static constexpr int N = DT == DT_F32 ? 4 : 8;
  __device__ static void unpack(const u32x4& w, float (&x)[N]) {
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) unpack2<DT>(w[i], x[2 * i], x[2 * i + 1]);
    }
  }
  __device__ static u32x4 pack(const float (&x)[N]) {
    u32x4 w;
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = elem_bits<DT>(x[2 * i]) | (elem_bits<DT>(x[2 * i + 1]) << 16);
    }
    return w;
  }
};

// Global-address-space byte pointer (loads through it are global_load, never flat_load).
typedef const __attribute__((address_space(1))) char* gptr;
typedef const __attribute__((address_space(1))) u32x4* gptr_u32x4;
typedef const __attribute__((address_space(1))) u32x2* gptr_u32x2;

// Generic pointer known to address global memory -> global address space.
__device__ inline gptr to_gptr(const char* p) { return (gptr)p; }

// Streaming loads of K/V rows: each byte is used once, so they are marked non-temporal (the
// nt bit), which keeps the caches free for the rest of the stream.
__device__ inline u32x4 stream_load16(gptr p) {
  return __builtin_nontemporal_load(reinterpret_cast<gptr_u32x4>(p));
}

// N 32-bit words from 4N contiguous bytes (N in {2, 4, 8}).
template <int N>
__device__ inline void load_words(gptr p, uint32_t (&w)[N]) {
  if constexpr (N == 2) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<gptr_u32x2>(p));
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4 v = stream_load16(p + 16 * i);
      w[4 * i + 0] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// Cross-row exchanges on VALU (gfx950 permlane swaps): lane l sees lanes l ^ 16 / l ^ 32.
// Both lanes of a pair combine the two values in the same order, so results are identical.
__device__ inline void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ inline void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ inline float max_rows4(float x) {   // max over lanes {l, l^16, l^32, l^48}
  float a, b;
  swap16(x, a, b);
  x = fmaxf(a, b);
  swap32(x, a, b);
  return fmaxf(a, b);
}
__device__ inline float sum_rows4(float x) {   // sum over lanes {l, l^16, l^32, l^48}
  float a, b;
  swap16(x, a, b);
  x = a + b;
  swap32(x, a, b);
  return a + b;
}

// s_waitcnt that waits until at most `n` vector-memory operations (loads and stores: gfx9
// counts both in vmcnt) of this wave are outstanding (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Device-scope (agent) relaxed store and load of a float: the access carries the device scope,
// so it is coherent across the XCDs, whose L2 caches are private, without a cache write-back or
// invalidate.  Used for values one workgroup hands to another within a launch.
__device__ inline void dev_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float dev_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resource over `bytes` bytes from `base` (raw addressing, stride 0); loads past the end
// return zeros.
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ inline BufRes make_bufres(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// 16-byte device-scope store of floats at byte offset `off` of a buffer (16-byte aligned);
// cache-policy 16 sets the sc1 bit, as dev_store does for a single word.
__device__ inline void dev_store16(BufRes r, uint32_t off, f32x4 v);

// 16-byte device-scope load at byte offset `off` of a buffer: the cache-policy operand 16 sets
// the sc1 bit (device scope), as dev_load does for a single word.
__device__ inline f32x4 dev_load16(BufRes r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 16);
  return f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
}
__device__ inline void dev_store16(BufRes r, uint32_t off, f32x4 v) {
  const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, int(off), 0, 16);
}

// 16-byte LDS read issued as inline assembly.  The K stages are filled by direct-to-LDS loads
// whose completion this kernel tracks itself (explicit vmcnt waits), so these reads are kept
// out of the compiler's conservative alias tracking.  The values may only be used after
// lds_wait_all() has passed them through its wait.
__device__ inline u32x4 lds_read16(uint32_t lds_addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}

// 4-byte LDS write issued as inline assembly, for values that lanes of one wave hand to each
// other while direct-to-LDS loads are in flight: as with lds_read16, the compiler does not see it
// as an LDS access and so does not make it wait for those loads.  lds_wait_writes() orders it
// before later reads of the same wave.
__device__ inline void lds_write32(uint32_t lds_addr, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr), "v"(v));
}
__device__ inline void lds_wait_writes() { asm volatile("s_waitcnt lgkmcnt(0)"); }

// 8-byte LDS read issued as inline assembly (same rules as lds_read16).
__device__ inline u32x2 lds_read8(uint32_t lds_addr) {
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N - 1, so that I can be a template argument.
template <int I, int N, class F>
__device__ inline void static_for_from(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ inline void static_for(F&& f) { static_for_from<0, N>(f); }

// lds_read16 of lds_addr + OFF, the constant in the instruction's offset field.
template <int OFF>
__device__ inline u32x4 lds_read16_at(uint32_t lds_addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF));
  return r;
}

// lds_write32 to lds_addr + OFF, the constant in the instruction's offset field.
template <int OFF>
__device__ inline void lds_write32_at(uint32_t lds_addr, float v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  asm volatile("ds_write_b32 %0, %1 offset:%2" : : "v"(lds_addr), "v"(v), "i"(OFF));
}

// lds_read8 of lds_addr + OFF, the constant in the instruction's offset field.
template <int OFF>
__device__ inline u32x2 lds_read8_at(uint32_t lds_addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFF));
  return r;
}

// Four 16-byte LDS reads pinned as landed while the LATER LDS operations issued after them are
// still in flight: s_waitcnt lgkmcnt(LATER).  LDS operations of a wave complete in order, so
// every read older than the LATER newest ones has landed (other operations counted by lgkmcnt
// only make the wait longer).
template <int LATER>
__device__ inline void lds_wait_older4(u32x4 (&r)[4]) {
  static_assert(LATER >= 0 && LATER < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "i"(LATER));
}

// s_waitcnt lgkmcnt(0) for reads issued with lds_read8/16; each value read is then passed
// through lds_pin(), which the compiler cannot move above the wait (both are volatile asm), so
// no use of the value can be scheduled before the data has landed.
__device__ inline void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)"); }
template <class T>
__device__ inline void lds_pin(T& r) { asm volatile("" : "+v"(r)); }

// This lane's V bytes of one token row (8, 16 or 32) read from LDS as 32-bit words.
template <int VB>
struct LdsRows;
template <>
struct LdsRows<8> {
  u32x2 r;
  __device__ void read(uint32_t a) { r = lds_read8(a); }
  __device__ void pin() { lds_pin(r); }
  __device__ void words(uint32_t (&w)[2]) const { w[0] = r.x; w[1] = r.y; }
};
template <>
struct LdsRows<16> {
  u32x4 r;
  __device__ void read(uint32_t a) { r = lds_read16(a); }
  __device__ void pin() { lds_pin(r); }
  __device__ void words(uint32_t (&w)[4]) const { w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w; }
};
template <>
struct LdsRows<32> {
  u32x4 r0, r1;
  __device__ void read(uint32_t a) { r0 = lds_read16(a); r1 = lds_read16(a + 16); }
  __device__ void pin() { lds_pin(r0); lds_pin(r1); }
  __device__ void words(uint32_t (&w)[8]) const {
    w[0] = r0.x; w[1] = r0.y; w[2] = r0.z; w[3] = r0.w;
    w[4] = r1.x; w[5] = r1.y; w[6] = r1.z; w[7] = r1.w;
  }
};

// s_waitcnt lgkmcnt(0) that the compiler cannot schedule uses of `r` above: the registers are
// operands of the waiting instruction.
template <int N>
__device__ inline void lds_wait_all(u32x4 (&r)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "operand count");
  if constexpr (N == 1) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]));
  } else if constexpr (N == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]));
  } else if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),
                   "+v"(r[6]), "+v"(r[7]));
  }
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at
// lds_dst + 16 l (lds_dst is a wave-uniform LDS byte address).  Completion is tracked by vmcnt.
template <int AUX>
__device__ inline void dma16_to_lds(gptr src, uint32_t lds_dst) {
  __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                            static_cast<uintptr_t>(lds_dst)),
                                   16, 0, AUX);
}

// Cache-policy bits of the K-row copies (non-temporal: streamed once).
constexpr int kDmaPolicy = 2;

// LDS byte address of a __shared__ object.
__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// A wave-uniform global pointer, forced into scalar registers (SGPR base + VGPR offset loads).
__device__ inline gptr uniform_gptr(const char* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr>((static_cast<uint64_t>(hi) << 32) | lo);
}

}  // namespace dev
}  // namespace pkv
