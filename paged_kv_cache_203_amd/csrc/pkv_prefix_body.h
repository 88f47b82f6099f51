// Shared-prefix (cascade) decode on CDNA4 (gfx950): the prefix partitions as a dense problem on
// the matrix cores.
//
// When every sequence of a batch begins with the same prefix, held once in the pool, the query
// rows of all sequences that read one KV head (sequence b, query head kvh * G + g: B x G rows)
// attend to the same prefix tokens.  Over the prefix, decode attention for those rows is then one
// dense product per KV head, S = Q K^T (rows x tokens) and O = softmax(S) V, instead of B
// separate matrix-vector products over the same pages.  A workgroup takes 128 query rows (8 waves
// x 16 rows: two waves per SIMD, which measured faster than 4 x 32 at one wave per SIMD) and one
// partition of the prefix, and streams the partition in blocks of 64 tokens, so each prefix page
// is read once per 128 rows:
//  * K block: direct-to-LDS loads, row-major; the 16-byte slices of token t are XOR-swizzled by
//    t, which keeps the MFMA operand reads free of bank conflicts.
//  * V block: loaded into registers and written to LDS transposed (dims x tokens, two tokens per
//    32-bit word), so the PV operand — eight tokens of one dim per lane — is two 8-byte reads.
//    The transposed rows are padded to 144 bytes, which spreads those reads over all banks.
//  * S^T tiles (16 tokens x 16 rows) = K . Q^T on MFMA; online softmax in base 2 in that layout,
//    where a lane holds one row (m16), so rescaling the row's output is lane-local.
//  * O^T (dims x rows) += V^T . P on MFMA.  The k order of this product is free, so P is taken
//    straight from the S^T registers (tokens 4 kq + i of two adjacent tiles) and V^T is read in
//    the same token order.  P is split as hi + lo in the 16-bit input type and both halves are
//    multiplied, which keeps each probability to about 2^-14 relative (bf16) or 2^-20 (fp16).
// Loads of block n + 1 are in flight while block n is computed (two LDS buffers); the rows'
// lengths, the partition's page ids and the q operands load together at the start.  Each (row,
// partition) writes its normalised partial output and log-sum-exp in the split-KV layout; the
// suffix partitions are the split path's partition body, run in the same grid (cascade_kernel),
// and the merge is the split path's kernel.  The same body in its per-sequence mode is multi-query
// decode (prefix_kernel).  Each output element is its own MFMA dot product and the softmax is per
// row, so a row's bits do not depend on the other rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kTB = 64;                 // tokens per block

// NW waves per workgroup, each with RBW blocks of 16 query rows.
template <int D, int NW, int RBW>
struct PrefixGeo {
  static constexpr int ROWS = NW * 16 * RBW;        // query rows per workgroup
  static constexpr int RB = D * 2;                  // bytes of one token row (16-bit types)
  static constexpr int SPR = RB / 16;               // 16-byte slices per row: 8 or 16
  static constexpr int SWZ = SPR - 1;
  static constexpr int NKL = SPR / 4;               // MFMA k-steps over the head dim: 2 or 4
  static constexpr int KB = kTB * RB;               // K block bytes
  static constexpr int KDMA = KB / 1024 / NW;       // direct-to-LDS loads per wave per block
  static constexpr int VST = kTB * 2 + 16;          // bytes per transposed V row (padded)
  static constexpr int VTB = D * VST;               // transposed V block bytes
  static constexpr int NDT = D / 16;                // 16-dim output tiles
  static constexpr int VTASKS = (kTB / 2) * (D / 8);              // (token pair, slice) tasks
  static constexpr int VTASK = (VTASKS + NW * 64 - 1) / (NW * 64);  // ... per thread
  static_assert(KDMA >= 1 && KB % (1024 * NW) == 0, "whole direct-to-LDS loads per wave");
};

template <int D>
struct PrefixShared {
  using Geo = PrefixGeo<D, 1, 1>;   // the buffers do not depend on the wave layout
  char k[2][Geo::KB] __attribute__((aligned(16)));
  char vt[2][Geo::VTB] __attribute__((aligned(16)));
  int pid[kMaxPrefixPageIds];   // page ids of the partition's prefix pages
  int wend[16];                 // per wave: largest token limit of its rows
  int wbad[16];                 // per wave: first out-of-range page id seen (kMaxPrefixPageIds: none)
};

template <int DT>
__device__ inline f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two probabilities as packed 16-bit hi and lo parts: x = hi + lo + e.  bf16: hi is x truncated
// to 8 significant bits, so x - hi is exact in float and its truncation leaves |e| < 2^-14 |x|.
// fp16: hi and lo rounded toward zero to 11 bits, |e| < 2^-20 |x| (absolute 2^-24 below 2^-14).
template <int DT>
__device__ inline void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  if constexpr (DT == DT_BF16) {
    const uint32_t h0 = __float_as_uint(x0) & 0xffff0000u, h1 = __float_as_uint(x1) & 0xffff0000u;
    hi = (h0 >> 16) | h1;
    const float r0 = x0 - __uint_as_float(h0), r1 = x1 - __uint_as_float(h1);
    lo = (__float_as_uint(r0) >> 16) | (__float_as_uint(r1) & 0xffff0000u);
  } else {
    const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
    hi = __builtin_bit_cast(uint32_t, h);
    const float r0 = x0 - static_cast<float>(h[0]), r1 = x1 - static_cast<float>(h[1]);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
  }
}

// MQ = false: the shared-prefix partitions (rows: every sequence's query heads of one KV head;
// pages: prefix_pages).  MQ = true: multi-query decode (rows: the T new query tokens x G heads of
// one sequence and KV head, query j limited to tokens t <= L - T + j; pages: the sequence's own
// page-table row).
// Workgroup `id` of the grid (see below) with its LDS `sm`; the kernels that run it pass their
// block index, or its offset within a fused grid.
template <int DT, int D, int NW, int RBW, bool MQ>
__device__ inline void prefix_body(const PrefixParams& p, int id, PrefixShared<D>& sm) {
  using Geo = PrefixGeo<D, NW, RBW>;
  static_assert(NW <= 16, "per-wave slots");
  constexpr int kRowsWG = Geo::ROWS;
  constexpr int NKL = Geo::NKL, NDT = Geo::NDT, RB = Geo::RB, VST = Geo::VST;

  const int tid = threadIdx.x;
  const int lane = tid & 63, m16 = lane & 15, kq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroup -> (row tile, KV head, partition[, sequence]).  Workgroups that read the same
  // pages (same head, partition and sequence) are a multiple of Hkv apart, so they share an XCD
  // (and its L2) when Hkv is a multiple of the XCD count.
  int part, kvh, rt, sb = 0;
  if constexpr (MQ) {
    kvh = id % p.hkv;
    id /= p.hkv;
    sb = id % p.batch;
    id /= p.batch;
    part = id % p.max_partitions;
    rt = id / p.max_partitions;
  } else {
    const int S = p.prefix_tokens / p.partition_tokens;
    part = id % S;
    id /= S;
    kvh = id % p.hkv;
    rt = id / p.hkv;
  }
  const int t_lo = part * p.partition_tokens, t_hi = t_lo + p.partition_tokens;
  const int rows = MQ ? p.q_tokens * p.group : p.batch * p.group;
  const int ps_mask = (1 << p.page_shift) - 1;

  // This lane's query rows (blocks rb < RBW): r = rt * ROWS + (wave * RBW + rb) * 16 + m16.
  // A row attends to prefix tokens t < lim (its length, capped at the partition end); rows past
  // the batch, padding rows and rows longer than the page table allows have lim = 0.
  int lim[RBW];
  int64_t qrow[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = rt * kRowsWG + (wave * RBW + rb) * 16 + m16;
    lim[rb] = 0;
    qrow[rb] = -1;
    if (r < rows) {
      const int g = r % p.group;
      if constexpr (MQ) {
        const int j = r / p.group;   // the query token
        qrow[rb] = (int64_t(sb) * p.q_tokens + j) * p.hq + int64_t(kvh) * p.group + g;
        const int L = p.context_lens[sb];
        const int Lj = L - p.q_tokens + 1 + j;
        if (L > 0 && L <= p.capacity && Lj > 0) lim[rb] = min(Lj, t_hi);
      } else {
        const int b = r / p.group;
        qrow[rb] = int64_t(b) * p.hq + int64_t(kvh) * p.group + g;
        const int L = p.context_lens[b];
        if (L > 0 && L <= p.capacity) lim[rb] = min(L, t_hi);
      }
    }
  }

  int my_end = lim[0], lane_min = lim[0];
#pragma unroll
  for (int rb = 1; rb < RBW; ++rb) {
    my_end = max(my_end, lim[rb]);
    lane_min = min(lane_min, lim[rb]);
  }
  const int my_lim_any = my_end;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) my_end = max(my_end, __shfl_xor(my_end, off));
  if (lane == 0) sm.wend[wave] = my_end;

  // Stage the ids of all the partition's pages, and note the first out-of-range one.  Shared
  // prefix: every one is a prefix page (the partition ends at or before prefix_tokens).  Multi-
  // query: entries past the table's width stand for tokens no row reaches, and read as page 0.
  // These loads, the lengths above and the q operands below are in flight together.
  const int n_ids = p.partition_tokens >> p.page_shift;
  int first_bad = kMaxPrefixPageIds;
  for (int i = tid; i < n_ids; i += NW * 64) {
    const int idx = (t_lo >> p.page_shift) + i;
    int pg;
    if constexpr (MQ)
      pg = idx < p.max_pages ? p.page_table[int64_t(sb) * p.max_pages + idx] : 0;
    else
      pg = p.prefix_pages[idx];
    const bool bad_id = pg < 0 || pg >= p.num_pages;
    if (bad_id) pg = 0;   // read page 0 instead; rows that reach this page get NaN
    sm.pid[i] = pg;
    const uint64_t m = __ballot(bad_id);
    if (m) first_bad = min(first_bad, i - lane + __builtin_ctzll(m));
  }
  if (lane == 0) sm.wbad[wave] = first_bad;

  // Q^T operands: lane holds row m16 of block rb, 16-byte slices 4c + kq (zero past the batch).
  u32x4 qop[RBW][NKL];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int c = 0; c < NKL; ++c)
      qop[rb][c] = qrow[rb] >= 0
                       ? *reinterpret_cast<gptr_u32x4>(to_gptr(static_cast<const char*>(p.q)) +
                                                       qrow[rb] * RB + 64 * c + 16 * kq)
                       : u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  int wg_end = 0, bad_idx = kMaxPrefixPageIds;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wg_end = max(wg_end, sm.wend[w]);
    bad_idx = min(bad_idx, sm.wbad[w]);
  }
  if (wg_end <= t_lo) return;   // no row of this tile reaches the partition (uniform)
  // Blocks cover [t_lo, t_lo + NB * 64), inside the partition (its length is a multiple of 64).
  const int NB = (wg_end - t_lo + kTB - 1) / kTB;
  const int64_t bad_from = t_lo + (int64_t(bad_idx) << p.page_shift);   // first token of a bad page

  // Per-lane load geometry.  K: load i of this wave fills LDS bytes (wave * KDMA + i) * 1024 +
  // 16 lane of the block: token kt[i], holding slice kj[i] (the swizzled position's slice).
  int kt[Geo::KDMA], kj[Geo::KDMA];
#pragma unroll
  for (int i = 0; i < Geo::KDMA; ++i) {
    const int byte = (wave * Geo::KDMA + i) * 1024 + 16 * lane;
    kt[i] = byte / RB;
    kj[i] = ((byte % RB) / 16) ^ (kt[i] & Geo::SWZ);
  }
  // V: task k covers tokens 2 tp, 2 tp + 1 and 16-byte slice c.  Four lanes share a token's 64
  // contiguous bytes; sixteen token pairs per wave.  Threads past the task count have none.
  int vtp[Geo::VTASK], vc[Geo::VTASK];
  bool vhas[Geo::VTASK];
#pragma unroll
  for (int k = 0; k < Geo::VTASK; ++k) {
    const int f = tid + NW * 64 * k;
    vhas[k] = f < Geo::VTASKS;
    const int hi = f / 64;
    vc[k] = (hi % (D / 32)) * 4 + (f % 4);
    vtp[k] = (hi / (D / 32)) * 16 + (f / 4) % 16;
  }

  const char* kpool = static_cast<const char*>(p.k_pool) + int64_t(kvh) * RB;
  const char* vpool = static_cast<const char*>(p.v_pool) + int64_t(kvh) * RB;
  u32x4 vreg[Geo::VTASK][2];

  // Start block n's loads: V rows into registers, K rows into LDS buffer bf.
  auto issue = [&](int n, int bf) {
    const int rel0 = n * kTB;
    int64_t voff[Geo::VTASK], koff[Geo::KDMA];
#pragma unroll
    for (int k = 0; k < Geo::VTASK; ++k) {
      const int rel = vhas[k] ? rel0 + 2 * vtp[k] : rel0;
      voff[k] = int64_t(sm.pid[rel >> p.page_shift]) * p.page_stride +
                int64_t((t_lo + rel) & ps_mask) * p.tok_stride + 16 * vc[k];
    }
#pragma unroll
    for (int i = 0; i < Geo::KDMA; ++i) {
      const int rel = rel0 + kt[i];
      koff[i] = int64_t(sm.pid[rel >> p.page_shift]) * p.page_stride +
                int64_t((t_lo + rel) & ps_mask) * p.tok_stride + 16 * kj[i];
    }
#pragma unroll
    for (int k = 0; k < Geo::VTASK; ++k) {
      if (!vhas[k]) continue;
      const gptr v = to_gptr(vpool + voff[k]);
      vreg[k][0] = *reinterpret_cast<gptr_u32x4>(v);
      vreg[k][1] = *reinterpret_cast<gptr_u32x4>(v + p.tok_stride);
    }
    const uint32_t kdst = lds_addr(sm.k[bf]) + uint32_t(wave * Geo::KDMA) * 1024u;
#pragma unroll
    for (int i = 0; i < Geo::KDMA; ++i)
      dma16_to_lds<0>(to_gptr(kpool + koff[i]), kdst + uint32_t(i) * 1024u);
  };

  // Write block n's V rows (in registers) to LDS buffer bf transposed: word (d, tp) holds tokens
  // 2 tp and 2 tp + 1 of dim d.  Tokens at or past wg_end are written as zeros, so unused slots
  // of the last prefix page cannot turn a zero probability into NaN.
  auto write_vt = [&](int n, int bf) {
    const uint32_t base = lds_addr(sm.vt[bf]);
    const int t_abs = t_lo + n * kTB;
#pragma unroll
    for (int k = 0; k < Geo::VTASK; ++k) {
      if (!vhas[k]) continue;
      const int t0 = t_abs + 2 * vtp[k];
      const u32x4 a = t0 < wg_end ? vreg[k][0] : u32x4{0u, 0u, 0u, 0u};
      const u32x4 b = t0 + 1 < wg_end ? vreg[k][1] : u32x4{0u, 0u, 0u, 0u};
      const uint32_t col = base + uint32_t(8 * vc[k]) * VST + 4u * uint32_t(vtp[k]);
      static_for<4>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        const uint32_t lo = (a[w] & 0xffffu) | (b[w] << 16);
        const uint32_t hi = (a[w] >> 16) | (b[w] & 0xffff0000u);
        lds_write32_at<(2 * w) * VST>(col, __uint_as_float(lo));
        lds_write32_at<(2 * w + 1) * VST>(col, __uint_as_float(hi));
      });
    }
  };

  float m_run[RBW], l_run[RBW];
  f32x4 o[RBW][NDT];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m_run[rb] = neg_inf();
    l_run[rb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // A wave whose rows all end before the partition only helps load the blocks.
  const bool wave_active = __ballot(my_lim_any > t_lo) != 0;
  // This lane's operand reads within a buffer: K slice 4 c + kq of token row m16 (swizzled), and
  // the V^T row of dim m16 at tokens 8 kq ..; tile, dim-tile and token offsets are constants in
  // the read instructions.
  uint32_t krd[NKL];
#pragma unroll
  for (int c = 0; c < NKL; ++c) krd[c] = uint32_t(m16) * RB + uint32_t((4 * c + kq) ^ (m16 & Geo::SWZ)) * 16u;
  const uint32_t vrd = uint32_t(m16) * VST + 8u * uint32_t(kq);

  auto compute = [&](int n, int bf) {
    if (!wave_active) return;
    const uint32_t kb = lds_addr(sm.k[bf]);
    const uint32_t vb = lds_addr(sm.vt[bf]);
    const int t0 = t_lo + n * kTB;

    // ---- S^T tiles = K . Q^T -----------------------------------------------------------------
    f32x4 s[RBW][4];
    uint32_t ka[NKL];
#pragma unroll
    for (int c = 0; c < NKL; ++c) ka[c] = kb + krd[c];
    static_for<2>([&](auto tpc) {
      constexpr int tp = 2 * decltype(tpc)::value;   // tile pair: tiles tp, tp + 1
      u32x4 kop[2 * NKL];
      static_for<2 * NKL>([&](auto ic) {
        constexpr int i = decltype(ic)::value, j = i / NKL, c = i % NKL;
        kop[i] = lds_read16_at<(16 * (tp + j)) * RB>(ka[c]);
      });
      lds_wait_all<2 * NKL>(kop);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NKL; ++c) acc = mfma32<DT>(kop[j * NKL + c], qop[rb][c], acc);
          s[rb][tp + j] = acc;
        }
    });

    // ---- online softmax (lane: row m16 of block rb, tokens 16 tt + 4 kq + i) -----------------
    const bool need_mask = __ballot(lane_min < t0 + kTB) != 0;
    float alpha[RBW];
    bool rescale = false;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float mx = neg_inf();
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[rb][tt][i] *= p.scale_log2;
      if (need_mask) {   // only blocks where some row ends
        const int lrel = lim[rb] - t0 - 4 * kq;   // token 16 tt + 4 kq + i is masked when 16 tt + i >= lrel
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * tt + i >= lrel) s[rb][tt][i] = neg_inf();
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[rb][tt][i]);
      mx = max_rows4(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      const float m_use = m_new == neg_inf() ? 0.f : m_new;   // nothing unmasked yet
      alpha[rb] = fast_exp2(m_run[rb] - m_use);
      m_run[rb] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(s[rb][tt][i] - m_use);
          s[rb][tt][i] = e;
          ls += e;
        }
      l_run[rb] = l_run[rb] * alpha[rb] + ls;
      rescale = rescale || alpha[rb] != 1.f;
    }
    if (__ballot(rescale) != 0) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[rb][dt] *= alpha[rb];
    }

    // ---- O^T += V^T . P, 32 tokens per MFMA k-step -------------------------------------------
    static_for<2>([&](auto uc) {
      constexpr int u = decltype(uc)::value;   // tokens 32 u .. 32 u + 31 of the block
      u32x4 ph[RBW], pl[RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x4& t = s[rb][2 * u + w / 2];
          split_pair<DT>(t[2 * (w % 2)], t[2 * (w % 2) + 1], h[w], l[w]);
        }
        ph[rb] = u32x4{h[0], h[1], h[2], h[3]};
        pl[rb] = u32x4{l[0], l[1], l[2], l[3]};
      }
      u32x2 va[NDT][2];
      const uint32_t va0 = vb + vrd;
      static_for<NDT>([&](auto dc) {
        constexpr int dt = decltype(dc)::value;
        va[dt][0] = lds_read8_at<16 * dt * VST + 64 * u>(va0);
        va[dt][1] = lds_read8_at<16 * dt * VST + 64 * u + 32>(va0);
      });
      lds_wait();
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        lds_pin(va[dt][0]);
        lds_pin(va[dt][1]);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const u32x4 av = {va[dt][0].x, va[dt][0].y, va[dt][1].x, va[dt][1].y};
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          o[rb][dt] = mfma32<DT>(av, ph[rb], o[rb][dt]);
          o[rb][dt] = mfma32<DT>(av, pl[rb], o[rb][dt]);
        }
      }
    });
  };

  issue(0, 0);
  write_vt(0, 0);
  wait_vmcnt<0>();
  lds_wait_writes();
  __syncthreads();
  for (int n = 0; n < NB; ++n) {
    const int bf = n & 1;
    if (n + 1 < NB) issue(n + 1, bf ^ 1);
    compute(n, bf);
    if (n + 1 < NB) write_vt(n + 1, bf ^ 1);
    wait_vmcnt<0>();
    lds_wait_writes();
    __syncthreads();
  }

  // ---- normalised partials (lane: dims 16 dt + 4 kq + i of row m16) ----------------------------
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const float l = sum_rows4(l_run[rb]);
    if (lim[rb] <= t_lo) continue;   // the row does not reach this partition: not written
    const int64_t orow = qrow[rb] * p.max_partitions + part;
    const bool bad = lim[rb] > bad_from;
    const float inv = bad ? qnan() : 1.f / l;
    float* dst = p.partial_out + orow * D + 4 * kq;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[rb][dt] * inv;
    if (kq == 0)
      p.partial_lse[orow] = bad ? qnan() : (m_run[rb] + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

// Wave layout of the shared-prefix partitions: kPrefixWaves waves of kPrefixRowBlocks x 16 query rows.
constexpr int kPrefixWaves = 8, kPrefixRowBlocks = 1;

}  // namespace
}  // namespace pkv
