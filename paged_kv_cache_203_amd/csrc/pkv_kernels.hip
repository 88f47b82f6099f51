// HIP kernels for paged decode attention on CDNA4 (gfx950).
//
// Work unit.  One workgroup of NW wavefronts handles one (sequence b, KV head, partition): the
// G = Hq / Hkv query heads of a GQA group read each K/V row of that KV head once.  The unit's
// tokens are cut into tiles of 16 (a tile never straddles a page, since page_size is a multiple
// of 16); wave w takes tiles w, w + NW, w + 2 NW, ...  The order in which a token is reduced
// depends only on its logical position and the partition size, never on physical page ids or
// on the rest of the batch, so results are bitwise invariant under page relabelling, prefix
// sharing and batch composition.
//
// Per tile (16 tokens):
//  * page-table resolution: one scalar load of page_table[b][t0 / page_size] (prefetched one tile
//    ahead); the tile's 16 slots are contiguous rows of that page.
//  * QK: S^T (16 tokens x 16 head slots) = K_tile (16 x D) . Q^T (D x 16) on MFMA.  Lane l feeds
//    token l % 16 and a 16-byte slice of its K row straight from a global load, so K needs no
//    LDS staging; the G query heads (zero-padded to 16 columns) share every K read.
//  * online softmax in the MFMA output layout: lane l holds tokens 4*(l/16)..+3 of head l % 16;
//    the running max is kept per head (base-2 domain, exp2), the running sum per lane.
//  * p hand-off: each wave writes its 16 x G probabilities to a private LDS slot and reads them
//    back broadcast in the PV layout.
//  * PV on VALU in float32: lane l owns D/16 contiguous dims of token 4r + l/16 in round r, so the
//    V loads of a round are 4 whole rows (coalesced) and p stays exact float32 (no rounding of
//    probabilities to 16 bits).
// At the end the waves' (max, sum, accumulator) triples are merged in LDS in wave order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_launch.h"

namespace pkv {
namespace {

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

// N 32-bit words from 4N contiguous bytes (N in {2, 4, 8}).
template <int N>
__device__ inline void load_words(const char* p, uint32_t (&w)[N]) {
  if constexpr (N == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * i);
      w[4 * i + 0] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// Registers of one tile for one lane.
template <int NKL, int VW>
struct TileRegs {
  u32x4 k[NKL];          // K: 16-byte slices of token (lane % 16)
  uint32_t v[4][VW];     // V: round r holds dims of token 4r + lane / 16
};

template <int DT, int D, int GP, int NW, bool PARTIAL>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams p) {
  constexpr int E = elem_size<DT>();
  constexpr int NKL = D * E / 64;    // 16-byte K slices per lane per tile
  constexpr int VPL = D / 16;        // V elements per lane per token
  constexpr int VW = VPL * E / 4;    // V words per lane per token
  static_assert(GP == 4 || GP == 8 || GP == 16, "padded group");

  __shared__ float p_lds[NW][kTile][GP];
  __shared__ float a_lds[NW][GP];
  __shared__ float o_lds[NW][GP][D];
  __shared__ float m_lds[NW][GP];
  __shared__ float l_lds[NW][GP];
  __shared__ int bad_lds[NW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.group;

  // ---- work unit ------------------------------------------------------------------------
  int id = blockIdx.x;
  const int kvh = id % p.hkv;
  id /= p.hkv;
  const int b = id % p.batch;
  const int part = PARTIAL ? id / p.batch : 0;

  const int L = p.context_lens[b];
  int t_begin = 0, t_end = L;
  if constexpr (PARTIAL) {
    if (L <= 0 || L > p.capacity) return;          // nothing to write (the merge handles it)
    t_begin = part * p.partition_tokens;
    if (t_begin >= L) return;                      // partition past the end: not written
    t_end = min(L, t_begin + p.partition_tokens);
  } else {
    if (L <= 0 || L > p.capacity) {
      const float fill = L <= 0 ? 0.f : qnan();
      for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int g = idx / D, d = idx % D;
        store_elem<DT>(p.out, (int64_t(b) * p.hq + kvh * G + g) * D + d, fill);
      }
      return;
    }
  }
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;

  // ---- per-lane constants -----------------------------------------------------------------
  const int row = lane & 15;      // MFMA: token row (K) / head column (Q, S)
  const int kq = lane >> 4;       // MFMA: k-group; PV: token within a round
  const int head_col = row;
  const uint32_t head_off = uint32_t(kvh) * D * E;
  const uint32_t k_off = uint32_t(row) * p.tok_stride + head_off + 16u * kq;
  const uint32_t v_off = uint32_t(kq) * p.tok_stride + head_off + uint32_t(row) * VPL * E;
  const uint32_t v_round = 4u * p.tok_stride;
  const char* const kpool = static_cast<const char*>(p.k_pool);
  const char* const vpool = static_cast<const char*>(p.v_pool);
  const int32_t* const table = p.page_table + int64_t(b) * p.max_pages;
  const int page_mask = (1 << p.page_shift) - 1;

  // Q^T operand: lane holds q[head_col][16-byte slices c * 64 + 16 kq], zero for padded heads.
  u32x4 qreg[NKL];
  {
    const char* qrow = static_cast<const char*>(p.q) +
                       (int64_t(b) * p.hq + int64_t(kvh) * G + head_col) * D * E;
#pragma unroll
    for (int c = 0; c < NKL; ++c) {
      qreg[c] = (head_col < G) ? *reinterpret_cast<const u32x4*>(qrow + 64 * c + 16 * kq)
                               : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m_run = neg_inf();   // running max of head `head_col` (base-2 domain)
  float l_run = 0.f;         // running sum over this lane's rows
  float o[GP][VPL];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[g][e] = 0.f;
  bool bad = false;

  auto page_of = [&](int tile) -> int {
    const int t0 = t_begin + tile * kTile;
    return __builtin_amdgcn_readfirstlane(table[t0 >> p.page_shift]);
  };
  auto load_tile = [&](int tile, int page, TileRegs<NKL, VW>& r) {
    const int t0 = t_begin + tile * kTile;
    const int64_t base = int64_t(page) * p.page_stride + int64_t(t0 & page_mask) * p.tok_stride;
    const char* kb = kpool + base;
    const char* vb = vpool + base;
#pragma unroll
    for (int c = 0; c < NKL; ++c) r.k[c] = *reinterpret_cast<const u32x4*>(kb + k_off + 64 * c);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) load_words<VW>(vb + v_off + rr * v_round, r.v[rr]);
  };
  auto page_ok = [&](int page) { return page >= 0 && page < p.num_pages; };

  TileRegs<NKL, VW> cur, nxt;
  int tile = wave;
  int page_cur = 0, page_nxt = 0;
  if (tile < n_tiles) {
    page_cur = page_of(tile);
    if (page_ok(page_cur)) load_tile(tile, page_cur, cur);
  }
  if (tile + NW < n_tiles) page_nxt = page_of(tile + NW);

  for (; tile < n_tiles; tile += NW) {
    const int t_next = tile + NW;
    if (t_next < n_tiles && page_ok(page_nxt)) load_tile(t_next, page_nxt, nxt);
    const int page_after = (t_next + NW < n_tiles) ? page_of(t_next + NW) : 0;

    if (page_ok(page_cur)) {
      const int t0 = t_begin + tile * kTile;
      const bool masked = t0 + kTile > t_end;

      // ---- S^T = K . Q^T -----------------------------------------------------------------
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKL; ++c) {
        if constexpr (DT == DT_BF16) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[c]),
                                                        __builtin_bit_cast(bf16x8, qreg[c]), acc,
                                                        0, 0, 0);
        } else if constexpr (DT == DT_F16) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, cur.k[c]),
                                                       __builtin_bit_cast(f16x8, qreg[c]), acc,
                                                       0, 0, 0);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(cur.k[c][i]),
                                                       __uint_as_float(qreg[c][i]), acc, 0, 0, 0);
        }
      }

      // ---- online softmax (lane: head `head_col`, tokens 4 kq + i) --------------------------
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = acc[i] * p.scale_log2;
        if (masked && t0 + 4 * kq + i >= t_end) s[i] = neg_inf();
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(s[i] - m_new);
      l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m_run = m_new;

      if (head_col < GP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p_lds[wave][4 * kq + i][head_col] = pr[i];
        if (kq == 0) a_lds[wave][head_col] = alpha;
      }
      const bool rescale = __ballot(head_col < G && alpha != 1.f) != 0;
      __builtin_amdgcn_wave_barrier();

      // ---- PV ---------------------------------------------------------------------------
      if (rescale) {
        float a[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) a[g] = a_lds[wave][g];
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
          for (int e = 0; e < VPL; ++e) o[g][e] *= a[g];
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float pg[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) pg[g] = p_lds[wave][4 * rr + kq][g];
        float v[VPL];
        if constexpr (DT == DT_F32) {
#pragma unroll
          for (int e = 0; e < VPL; ++e) v[e] = __uint_as_float(cur.v[rr][e]);
        } else {
#pragma unroll
          for (int e = 0; e < VPL / 2; ++e) unpack2<DT>(cur.v[rr][e], v[2 * e], v[2 * e + 1]);
        }
        if (masked && t0 + 4 * rr + kq >= t_end) {
#pragma unroll
          for (int e = 0; e < VPL; ++e) v[e] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
          for (int e = 0; e < VPL; ++e) o[g][e] = fmaf(pg[g], v[e], o[g][e]);
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      bad = true;
    }

    cur = nxt;
    page_cur = page_nxt;
    page_nxt = page_after;
  }

  // ---- merge the waves ------------------------------------------------------------------
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < VPL; ++e) {
      o[g][e] += __shfl_xor(o[g][e], 16);
      o[g][e] += __shfl_xor(o[g][e], 32);
    }
  if (lane < GP) {
    m_lds[wave][lane] = m_run;
    l_lds[wave][lane] = l_run;
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < VPL; ++e) o_lds[wave][g][lane * VPL + e] = o[g][e];
  }
  if (lane == 0) bad_lds[wave] = bad ? 1 : 0;
  __syncthreads();

  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= bad_lds[w];

  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int g = idx / D, d = idx % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, m_lds[w][g]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = fast_exp2(m_lds[w][g] - M);
      lsum = fmaf(sc, l_lds[w][g], lsum);
      osum = fmaf(sc, o_lds[w][g][d], osum);
    }
    const int h = kvh * G + g;
    const float val = any_bad ? qnan() : osum / lsum;
    if constexpr (PARTIAL) {
      const int64_t rowi = (int64_t(b) * p.hq + h) * p.max_partitions + part;
      p.partial_out[rowi * D + d] = val;
      if (d == 0) p.partial_lse[rowi] = any_bad ? qnan() : (M + __builtin_amdgcn_logf(lsum)) * kLn2;
    } else {
      store_elem<DT>(p.out, (int64_t(b) * p.hq + h) * D + d, val);
    }
  }
}

// One wavefront per (sequence, query head): out = sum_p w_p o_p / sum_p w_p, w_p = e^(lse_p - M).
template <int DT, int D>
__global__ __launch_bounds__(64) void merge_kernel(const MergeParams p) {
  constexpr int DPL = D / 64;   // dims per lane
  const int lane = threadIdx.x;
  const int b = blockIdx.x / p.hq;
  const int h = blockIdx.x % p.hq;
  const int L = p.context_lens[b];
  const int64_t orow = (int64_t(b) * p.hq + h) * D;
  if (L <= 0 || L > p.capacity) {
    const float fill = L <= 0 ? 0.f : qnan();
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_elem<DT>(p.out, orow + lane * DPL + e, fill);
    if (p.lse_out && lane == 0) p.lse_out[int64_t(b) * p.hq + h] = L <= 0 ? neg_inf() : qnan();
    return;
  }
  const int n = (L + p.partition_tokens - 1) / p.partition_tokens;
  const int64_t prow = (int64_t(b) * p.hq + h) * p.max_partitions;
  const float* lse = p.partial_lse + prow;
  float M = neg_inf();
  for (int i = 0; i < n; ++i) M = fmaxf(M, lse[i]);
  float wsum = 0.f;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  for (int i = 0; i < n; ++i) {
    const float w = fast_exp2((lse[i] - M) * kLog2e);
    wsum += w;
    const float* po = p.partial_out + (prow + i) * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, po[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) store_elem<DT>(p.out, orow + lane * DPL + e, acc[e] / wsum);
  if (p.lse_out && lane == 0)
    p.lse_out[int64_t(b) * p.hq + h] = M + __builtin_amdgcn_logf(wsum) * kLn2;
}

// One workgroup per sequence: copy the new K and V rows (all KV heads, contiguous in both the
// source and the destination slot) with 16-byte loads and stores.
__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  const int b = blockIdx.x;
  const int L = p.context_lens[b];
  if (L < 0 || L >= p.capacity) return;
  const int page = p.page_table[int64_t(b) * p.max_pages + (L >> p.page_shift)];
  if (page < 0 || page >= p.num_pages) return;
  const int64_t dst = int64_t(page) * p.page_stride +
                      int64_t(L & ((1 << p.page_shift) - 1)) * p.row_bytes;
  const int64_t src = int64_t(b) * p.row_bytes;
  const int nvec = p.row_bytes / 16;
  for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k_new) + src + 16 * i);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.v_new) + src + 16 * i);
    *reinterpret_cast<u32x4*>(static_cast<char*>(p.k_pool) + dst + 16 * i) = kv;
    *reinterpret_cast<u32x4*>(static_cast<char*>(p.v_pool) + dst + 16 * i) = vv;
  }
}

// One workgroup checks every row and writes the status word (no pre-clearing needed).
__global__ __launch_bounds__(1024) void validate_kernel(const ValidateParams p) {
  __shared__ int status;
  if (threadIdx.x == 0) status = 0;
  __syncthreads();
  int local = 0;
  const int64_t entries = int64_t(p.batch) * p.max_pages;
  for (int64_t idx = threadIdx.x; idx < entries; idx += blockDim.x) {
    const int b = int(idx / p.max_pages), i = int(idx % p.max_pages);
    const int64_t L = int64_t(p.context_lens[b]) + p.extra_tokens;
    if (L <= 0) continue;
    int64_t n = (L + p.page_size - 1) / p.page_size;
    if (n > p.max_pages) {
      if (i == 0) local |= 2;
      n = p.max_pages;
    }
    if (i >= n) continue;
    const int pg = p.page_table[idx];
    if (pg < 0 || pg >= p.num_pages) local |= 1;
    if (p.check_append_unique) {
      for (int b2 = 0; b2 < p.batch; ++b2) {
        if (b2 == b) continue;
        const int64_t L2 = p.context_lens[b2];
        if (L2 < 0 || L2 + p.extra_tokens <= 0) continue;
        const int64_t j = L2 / p.page_size;
        if (j >= p.max_pages) continue;
        if (p.page_table[int64_t(b2) * p.max_pages + j] == pg) {
          local |= 4;
          break;
        }
      }
    }
  }
  if (local) atomicOr(&status, local);
  __syncthreads();
  if (threadIdx.x == 0) *p.device_status = status;
}

constexpr int kWaves = 4;

template <int DT, int D, int GP>
hipError_t launch_decode_t(const DecodeParams& p, bool partial, hipStream_t stream) {
  const int64_t units = int64_t(p.batch) * p.hkv * (partial ? p.max_partitions : 1);
  if (units == 0) return hipSuccess;
  if (partial)
    hipLaunchKernelGGL((decode_kernel<DT, D, GP, kWaves, true>), dim3(unsigned(units)),
                       dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<DT, D, GP, kWaves, false>), dim3(unsigned(units)),
                       dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_decode_d(const DecodeParams& p, int gp, bool partial, hipStream_t stream) {
  switch (gp) {
    case 4: return launch_decode_t<DT, D, 4>(p, partial, stream);
    case 8: return launch_decode_t<DT, D, 8>(p, partial, stream);
    case 16: return launch_decode_t<DT, D, 16>(p, partial, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_decode_dt(const DecodeParams& p, int head_dim, int gp, bool partial,
                            hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_decode_d<DT, 64>(p, gp, partial, stream);
    case 128: return launch_decode_d<DT, 128>(p, gp, partial, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_merge_dt(const MergeParams& p, int head_dim, hipStream_t stream) {
  const int64_t units = int64_t(p.batch) * p.hq;
  if (units == 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<DT, 64>), dim3(unsigned(units)), dim3(64), 0, stream, p);
  else if (head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<DT, 128>), dim3(unsigned(units)), dim3(64), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int group_pad,
                         bool partial, hipStream_t stream) {
  switch (dtype) {
    case DT_F32: return launch_decode_dt<DT_F32>(p, head_dim, group_pad, partial, stream);
    case DT_BF16: return launch_decode_dt<DT_BF16>(p, head_dim, group_pad, partial, stream);
    case DT_F16: return launch_decode_dt<DT_F16>(p, head_dim, group_pad, partial, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t stream) {
  switch (dtype) {
    case DT_F32: return launch_merge_dt<DT_F32>(p, head_dim, stream);
    case DT_BF16: return launch_merge_dt<DT_BF16>(p, head_dim, stream);
    case DT_F16: return launch_merge_dt<DT_F16>(p, head_dim, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(p.batch)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_validate(const ValidateParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
