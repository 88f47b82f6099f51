// HIP kernels for paged decode attention on CDNA4 (gfx950).
//
// The hot loop (HeadPipe) streams one KV head of one sequence through one wavefront:
//  * Tiles of 16 tokens; a tile never straddles a page (page_size is a multiple of 16), so its
//    16 rows sit at one page-table entry: page_table[b][t0 / page_size], slot t0 % page_size.
//    Page ids are fetched one per lane for 64 tiles at a time and broadcast with readlane.
//  * K rows are copied global -> LDS with 16-byte direct-to-LDS loads, 16 lanes per row, so every
//    load instruction reads whole rows.  In LDS, slice j of token t sits at j ^ (t & SWZ), which
//    keeps the MFMA-layout reads below free of bank conflicts.
//  * V rows are copied to LDS the same way (row-major; for 16-bit head_dim 128 the 16-byte chunks
//    of rows 4..7 and 12..15 of a tile swap halves, which spreads the PV operand reads over all
//    banks).
//  * S^T (16 tokens x 16 head slots) = K_tile . Q^T on MFMA: the G query heads of the GQA group
//    (zero-padded to 16 columns) share every K row read.
//  * Online softmax in the MFMA output layout (lane l: tokens 4(l/16)..+3 of head l % 16), base 2.
//  * PV, for 16-bit K/V and head_dim 128, on MFMA as well: O^T (dims x head slots) += V^T . P,
//    with P straight from the score registers, each probability as a high and a low 16-bit part
//    (about 16 significant bits), and V^T cut out of 8-byte LDS reads of four token rows.  For
//    fp32 and head_dim 64, p goes through a per-wave LDS slot to the PV layout and PV
//    accumulates in float32 on VALU.  Either way the accumulation is float32.
//  * DEPTH tiles are in flight per wave (K and V stages in LDS), waited for with explicit vmcnt
//    counts; no tile byte passes through registers on its way in.
// The order in which a token is reduced depends only on its logical position and on the token
// range a wave is given, never on physical page ids, so results are bitwise invariant under
// page relabelling and prefix sharing.
//
// Kernels:
//  * decode_kernel: one workgroup per (sequence, partition, group of KV heads).  Partitions are
//    fixed multiples of partition_tokens, so a sequence's bits never depend on the batch.
//  * step_kernel: one whole decode step in one launch, with the work split evenly over the GPU —
//    the batch's tiles are cut into one contiguous range per workgroup, and a range may cover
//    pieces of several sequences.  The workgroup that holds a sequence's last tile first writes
//    the appended token's K/V rows into the pool, then reads them back with that tile.  The
//    last workgroup to finish a piece of a sequence merges the sequence's pieces.
//  * cascade_kernel: shared-prefix decode in one grid, the suffix partitions (decode_kernel's
//    partial mode) and then the prefix partitions on the matrix cores (pkv_prefix_body.h).
//  * merge kernels: log-sum-exp combination of partial results.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_arrival.h"
#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_prefix_body.h"

namespace pkv {
namespace {

using namespace dev;

// Tiles handled per wave between page-table refreshes: one page id per lane.
constexpr int kChunk = 64;

// Geometry of one tile of one KV head.
template <int DT, int D>
struct TileGeo {
  static constexpr int E = elem_size<DT>();
  static constexpr int RB = D * E;              // bytes of one row (one token, one KV head)
  static constexpr int SPR = RB / 16;           // 16-byte slices per row: 8, 16 or 32
  static constexpr int NKL = SPR / 4;           // MFMA k-chunks per tile = DMA loads per tile
  static constexpr int TPI = 64 / SPR;          // rows per DMA load instruction
  static constexpr int KTILE = kTile * RB;      // K bytes of one tile
  static constexpr int SWZ = (SPR < 16 ? SPR : 16) - 1;
  static constexpr int VPL = D / 16;            // V elements per lane per token
  static constexpr int VB = VPL * E;            // V bytes per lane per token: 8, 16 or 32
  static constexpr int VW = VB / 4;             // ... in 32-bit words
  static constexpr int LOADS = 2 * NKL;         // vector-memory instructions per tile (K, V)
};

// Tiles in flight per wave: two, except where two K and V stages of eight waves would not fit
// in LDS (fp32, head_dim 128).
template <int DT, int D>
constexpr int pipe_depth() { return DT == DT_F32 && D == 128 ? 1 : 2; }

// LDS of a decode workgroup: per-wave K and V stages (reused for the wave's epilogue) and p
// slots.
template <int DT, int D, int GP, int NW, int DEPTH>
struct DecodeShared {
  using Geo = TileGeo<DT, D>;
  static constexpr int EPI = (GP * D + 3 * GP) * 4;        // o[GP][D], m[GP], l[GP], bad
  static constexpr int STAGES = 2 * DEPTH * Geo::KTILE;    // K stages, then V stages
  static constexpr int WREG = STAGES > EPI ? STAGES : EPI;
  char w[NW][WREG] __attribute__((aligned(16)));
  float p[NW][kTile][GP] __attribute__((aligned(16)));   // rows read 16 bytes at a time
  float a[NW][GP] __attribute__((aligned(16)));
};

// HeadSource::causal0 when no column has a causal limit (leaves room for adding a query index).
constexpr int kNoCausalLimit = 1 << 30;

// What one wave streams: one KV head of one sequence over logical tokens [t_begin, t_end).
struct HeadSource {
  const char* kpool;
  const char* vpool;
  const int32_t* table;      // page-table row of the sequence
  int page_shift, num_pages;
  int tok_stride;            // bytes between consecutive slots of a page
  int64_t page_stride;
  int head_off;              // kvh * row bytes
  int t_begin, t_end;        // t_begin is a multiple of 16
  int sub, stride;           // this wave takes tiles sub, sub + stride, ...
  const char* q_group;       // q rows of the wave's GQA group (used by HeadPipe::prefetch)
  // Rotary embedding of q (HeadPipe with ROPE): the cache rows [D/2] at the query's position;
  // rope_pos < 0 leaves q as it is.
  const float* rope_cos;
  const float* rope_sin;
  int rope_pos;
  // Multi-query decode: query column c of the wave attends to tokens t < causal0 + q_j (q_j: the
  // column's query token, a HeadPipe lane constant) as well as t < t_end; a large value when
  // every column sees the whole range.
  int causal0 = kNoCausalLimit;
  // 1: this source's tile loads keep the default cache policy instead of the non-temporal one,
  // because another wave of the workgroup loads the same rows in the same round and should find
  // them in L2.
  int keep = 0;
  // Two waves that share this head's tiles and their LDS stages: 1 loads the K rows, 2 the V
  // rows, and both wait for each other around every tile; 0: this wave loads both.
  int part = 0;
};

// MQ: multi-query decode through the step (per-lane q rows and causal limits, columns that may
// see no token); the other instances compile to the plain decode code.
template <int DT, int D, int GP, int DEPTH, bool ROPE = false, bool MQ = false>
struct HeadPipe {
  using Geo = TileGeo<DT, D>;
  static constexpr int NKL = Geo::NKL, VPL = Geo::VPL, VW = Geo::VW;
  // Rotary embedding: slice 4c + kq of q (elements (4c + kq) * RW4 * 4 ...) pairs with slice
  // 4(c + NKL/2) + kq, half a head further on, in the same lane.
  static constexpr int RW4 = Vec16<DT>::N / 4;   // float4s of cos (or sin) per slice
  static constexpr uint32_t VSTAGE0 = DEPTH * Geo::KTILE;   // LDS offset of V stage 0
  // PV on the matrix cores (16-bit K/V, head_dim 128): O^T (dims x heads) += V^T . P with
  // mfma_f32_16x16x32, one 16-dim tile per instruction.  The MFMA's k index 8 kq + u stands for
  // token 4 kq + u % 4 of the tile, taken once with the high and once with the low 16-bit part of
  // its probability (u < 4: hi, u >= 4: lo), so P keeps about 16 significant bits and every
  // probability a lane needs is its own score register.  Otherwise PV is fp32 FMA on the VALU.
  static constexpr bool MPV = DT != DT_F32 && D == 128;
  static constexpr int NDT = D / 16;       // 16-dim output tiles (MPV)

  // per-lane constants
  int lane, m16, kq;
  uint32_t dma_off[NKL];   // byte offset (within a tile of this head) of this lane's K slice
  uint32_t vdma_off[NKL];  // ... and of its V slice (V stages are not swizzled)
  uint32_t rd_off[NKL];    // LDS offset of this lane's MFMA operand slice
  uint32_t v_rd;           // LDS offset (within a V stage) of this lane's dims of row kq
  uint32_t v_rd2;          // MPV: ... of its second group of dims (see init)
  uint32_t lds_base;       // this wave's K stages, then its V stages
  int64_t q_off;           // MQ: byte offset of this lane's q row from the source's q_group
  int q_j;                 // MQ: this lane's query token
  uint32_t p_lds;          // LDS address of this wave's p[16][GP]: a tile's probabilities
  uint32_t a_lds;          // LDS address of this wave's a[GP]: the tile's rescale factors
  // per-head state
  u32x4 qreg[NKL];
  // What prefetch() loaded for the next run(): its q operand and its first chunk's page ids.
  u32x4 q_pref[NKL];
  int pv_pref;
  bool pref_ready = false;
  f32x4 rope_cs[ROPE ? NKL / 2 : 1][2][RW4];   // prefetched cos, sin of this lane's pairs
  float m_run, l_run;
  float o[MPV ? 1 : GP][MPV ? 1 : VPL];
  // MPV: tile j of O^T; lane (m16, kq) holds head m16, dims 64 (j / 4) + 16 kq + 4 i + j % 4.
  f32x4 o4[MPV ? NDT : 1];
  bool bad;

  __device__ void init(int tok_stride, uint32_t lds, float* p, float* a) {
    lane = threadIdx.x & 63;
    m16 = lane & 15;
    kq = lane >> 4;
    q_off = int64_t(m16) * Geo::RB;
    q_j = 0;
    const int d_row = lane / Geo::SPR, d_pos = lane % Geo::SPR;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int t_in = Geo::TPI * i + d_row;
      dma_off[i] = uint32_t(t_in) * tok_stride + uint32_t(d_pos ^ (t_in & Geo::SWZ)) * 16u;
      // MPV: slot s of V row t holds 16-byte chunk s ^ 8 ((t >> 2) & 1), so that the PV operand
      // reads of rows 4 kq + i take the two halves of the banks for even and odd kq (lanes 0..31
      // of an 8-byte read are served together).
      const int vsw = MPV ? 8 * ((t_in >> 2) & 1) : 0;
      vdma_off[i] = uint32_t(t_in) * tok_stride + uint32_t(d_pos ^ vsw) * 16u;
    }
#pragma unroll
    for (int c = 0; c < NKL; ++c)
      rd_off[c] = uint32_t(m16) * Geo::RB + uint32_t((4 * c + kq) ^ (m16 & Geo::SWZ)) * 16u;
    if constexpr (MPV) {
      // Dims 64 h + 4 m16 .. + 3 of row 4 kq: chunk 8 h + m16 / 2 at slot 8 (h ^ (kq & 1)) + m16 / 2.
      const uint32_t row = uint32_t(4 * kq) * Geo::RB + 8u * uint32_t(m16);
      v_rd = row + 128u * uint32_t(kq & 1);
      v_rd2 = row + 128u * uint32_t(1 - (kq & 1));
    } else {
      v_rd = uint32_t(kq) * Geo::RB + uint32_t(m16) * Geo::VB;
      v_rd2 = 0;
    }
    lds_base = lds;
    p_lds = lds_addr(p);
    a_lds = lds_addr(a);
  }

  // Q^T operand: lane holds q[head m16][16-byte slices 4c + kq]; zero for padded heads.
  // `q_group` points at the first query head of the GQA group.
  __device__ void load_q(const char* q_group, int G) {
    const char* qrow = q_group + (MQ ? q_off : int64_t(m16) * Geo::RB);
#pragma unroll
    for (int c = 0; c < NKL; ++c)
      qreg[c] = (m16 < G) ? *reinterpret_cast<const u32x4*>(qrow + 64 * c + 16 * kq)
                          : u32x4{0u, 0u, 0u, 0u};
  }

  // Page ids of chunk c0 of `s` (lane j: the chunk's tile min(j, nc - 1)).
  __device__ int chunk_pages(const HeadSource& s, int c0, int nc) const {
    const int jt = c0 + min(lane, nc - 1);
    return s.table[(s.t_begin + (s.sub + jt * s.stride) * kTile) >> s.page_shift];
  }

  __device__ static int tiles_of(const HeadSource& s) {
    const int n_tiles = (s.t_end - s.t_begin + kTile - 1) / kTile;
    return n_tiles > s.sub ? (n_tiles - s.sub + s.stride - 1) / s.stride : 0;
  }

  // Start the loads of the next run()'s q operand and first page ids, so that their latency
  // overlaps the current work; the next run() on `s` then takes them instead of loading.
  __device__ void prefetch(const HeadSource& s, int G) {
    const char* qrow = s.q_group + (MQ ? q_off : int64_t(m16) * Geo::RB);
#pragma unroll
    for (int c = 0; c < NKL; ++c)
      q_pref[c] = (m16 < G) ? *reinterpret_cast<const u32x4*>(qrow + 64 * c + 16 * kq)
                            : u32x4{0u, 0u, 0u, 0u};
    const int n_my = tiles_of(s);
    pv_pref = n_my > 0 ? chunk_pages(s, 0, min(kChunk, n_my)) : 0;
    if constexpr (ROPE) {
      const bool on = s.rope_pos >= 0;
      const int64_t row = int64_t(on ? s.rope_pos : 0) * (D / 2);
#pragma unroll
      for (int c = 0; c < NKL / 2; ++c)
#pragma unroll
        for (int r = 0; r < RW4; ++r) {
          const int64_t i = row + (4 * c + kq) * Vec16<DT>::N + 4 * r;
          rope_cs[c][0][r] = on ? *reinterpret_cast<const f32x4*>(s.rope_cos + i) : f32x4{1.f, 1.f, 1.f, 1.f};
          rope_cs[c][1][r] = on ? *reinterpret_cast<const f32x4*>(s.rope_sin + i) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    pref_ready = true;
  }

  // Rotate the q operand by the prefetched cache rows (each pair's halves are in this lane).
  __device__ void rope_q() {
    constexpr int N = Vec16<DT>::N;
#pragma unroll
    for (int c = 0; c < NKL / 2; ++c) {
      float x1[N], x2[N], y1[N], y2[N];
      Vec16<DT>::unpack(qreg[c], x1);
      Vec16<DT>::unpack(qreg[c + NKL / 2], x2);
#pragma unroll
      for (int j = 0; j < N; ++j)
        rope_pair(x1[j], x2[j], rope_cs[c][0][j / 4][j % 4], rope_cs[c][1][j / 4][j % 4], y1[j], y2[j]);
      qreg[c] = Vec16<DT>::pack(y1);
      qreg[c + NKL / 2] = Vec16<DT>::pack(y2);
    }
  }

  __device__ void reset() {
    m_run = neg_inf();
    l_run = 0.f;
    if constexpr (MPV) {
#pragma unroll
      for (int j = 0; j < NDT; ++j) o4[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[g][e] = 0.f;
    }
    bad = false;
  }

  // Issue one tile: its V rows, then its K rows, into LDS stage `st` by direct-to-LDS loads (every
  // load of the stream writes LDS only).  An out-of-range page id reads page 0 instead (the tile
  // is then skipped and the head's result is NaN).
  __device__ void issue(const HeadSource& s, int st, int tile, int page) {
    const int t0 = s.t_begin + tile * kTile;
    const int pg = (page >= 0 && page < s.num_pages) ? page : 0;
    const int64_t base = int64_t(pg) * s.page_stride +
                         int64_t(t0 & ((1 << s.page_shift) - 1)) * s.tok_stride + s.head_off;
    const uint32_t kdst = lds_base + uint32_t(st * Geo::KTILE);
    const gptr vb = uniform_gptr(s.vpool + base);
    const uint32_t vdst = lds_base + VSTAGE0 + uint32_t(st * Geo::KTILE);
    const gptr kb = uniform_gptr(s.kpool + base);
    if (s.part == 1) {
#pragma unroll
      for (int i = 0; i < NKL; ++i) dma16_to_lds<kDmaPolicy>(kb + dma_off[i], kdst + uint32_t(i * 1024));
    } else if (s.part == 2) {
#pragma unroll
      for (int i = 0; i < NKL; ++i) dma16_to_lds<kDmaPolicy>(vb + vdma_off[i], vdst + uint32_t(i * 1024));
    } else if (s.keep) {
#pragma unroll
      for (int i = 0; i < NKL; ++i) dma16_to_lds<0>(vb + vdma_off[i], vdst + uint32_t(i * 1024));
#pragma unroll
      for (int i = 0; i < NKL; ++i) dma16_to_lds<0>(kb + dma_off[i], kdst + uint32_t(i * 1024));
    } else {
#pragma unroll
      for (int i = 0; i < NKL; ++i) dma16_to_lds<kDmaPolicy>(vb + vdma_off[i], vdst + uint32_t(i * 1024));
#pragma unroll
      for (int i = 0; i < NKL; ++i) dma16_to_lds<kDmaPolicy>(kb + dma_off[i], kdst + uint32_t(i * 1024));
    }
  }

  // Attend to the tile held in stage `st` (its loads have completed).
  __device__ void process(const HeadSource& s, int st, int tile, float scale_log2, int G) {
    const int t0 = s.t_begin + tile * kTile;
    const bool masked = t0 + kTile > (MQ ? min(s.t_end, s.causal0) : s.t_end);
    const uint32_t ks = lds_base + uint32_t(st * Geo::KTILE);

    // ---- S^T = K . Q^T ---------------------------------------------------------------------
    u32x4 kops[NKL];
#pragma unroll
    for (int c = 0; c < NKL; ++c) kops[c] = lds_read16(ks + rd_off[c]);
    u32x2 vr[2][4];   // MPV: the V^T operand rows, read now so that they land during QK and softmax
    if constexpr (MPV) {
      static_assert(NKL == 4, "head_dim 128, 16-bit");
      pv_read(st, vr);
      lds_wait_older4<8>(kops);
    } else {
      lds_wait_all<NKL>(kops);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKL; ++c) {
      if constexpr (DT == DT_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kops[c]),
                                                      __builtin_bit_cast(bf16x8, qreg[c]), acc,
                                                      0, 0, 0);
      } else if constexpr (DT == DT_F16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kops[c]),
                                                     __builtin_bit_cast(f16x8, qreg[c]), acc,
                                                     0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kops[c][i]),
                                                     __uint_as_float(qreg[c][i]), acc, 0, 0, 0);
      }
    }

    // ---- online softmax (lane: head m16, tokens 4 kq + i) ------------------------------------
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = acc[i] * scale_log2;
      if (masked && t0 + 4 * kq + i >= (MQ ? min(s.t_end, s.causal0 + q_j) : s.t_end)) sc[i] = neg_inf();
    }
    const float mx = max_rows4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float m_new = fmaxf(m_run, mx);
    // MQ: a column may have seen no token yet (its maximum is then -inf)
    const float m_use = MQ && m_new == neg_inf() ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - m_use);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;

    if constexpr (MPV) {
      pv_mfma(vr, t0, masked, s.t_end, pr, alpha, G);
      return;
    }

    // The probabilities move from the score layout (lane: head m16, tokens 4 kq + i) to the PV
    // layout (lane: dims of token row 4 rr + kq, all heads) through the wave's LDS slots.  These
    // accesses are inline assembly (lds_write32 / lds_read16), so the compiler does not make them
    // wait for the direct-to-LDS K loads in flight, which never touch these slots.
    if (m16 < GP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_write32(p_lds + uint32_t((4 * kq + i) * GP + m16) * 4u, pr[i]);
      if (kq == 0) lds_write32(a_lds + uint32_t(m16) * 4u, alpha);
    }
    const bool rescale = __ballot(m16 < G && alpha != 1.f) != 0;
    lds_wait_writes();
    __builtin_amdgcn_wave_barrier();

    // ---- PV ----------------------------------------------------------------------------------
    constexpr int NR = GP / 4;               // 16-byte reads per row of p (or of a)
    if (rescale) {
      u32x4 av[NR];
#pragma unroll
      for (int c = 0; c < NR; ++c) av[c] = lds_read16(a_lds + 16u * c);
      lds_wait_all<NR>(av);
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[g][e] *= __uint_as_float(av[g / 4][g % 4]);
    }
    constexpr int RPW = NR + VW / 4 <= 3 ? 4 : 2;   // rows of p and V read per wait
    const uint32_t vs = lds_base + VSTAGE0 + uint32_t(st * Geo::KTILE) + v_rd;
#pragma unroll
    for (int r0 = 0; r0 < 4; r0 += RPW) {
      u32x4 pv[RPW * NR];
      uint32_t vw[RPW][VW];   // this lane's V words of rows 4 rr + kq
      LdsRows<Geo::VB> vrows[RPW];
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        vrows[j].read(vs + uint32_t(4 * (r0 + j)) * Geo::RB);
#pragma unroll
        for (int c = 0; c < NR; ++c)
          pv[j * NR + c] = lds_read16(p_lds + uint32_t((4 * (r0 + j) + kq) * GP + 4 * c) * 4u);
      }
      lds_wait();
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        vrows[j].pin();
#pragma unroll
        for (int c = 0; c < NR; ++c) lds_pin(pv[j * NR + c]);
        vrows[j].words(vw[j]);
      }
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
      const int rr = r0 + j;
      float pg[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) pg[g] = __uint_as_float(pv[j * NR + g / 4][g % 4]);
      float v[VPL];
      if constexpr (DT == DT_F32) {
#pragma unroll
        for (int e = 0; e < VPL; ++e) v[e] = __uint_as_float(vw[j][e]);
      } else {
#pragma unroll
        for (int e = 0; e < VPL / 2; ++e) unpack2<DT>(vw[j][e], v[2 * e], v[2 * e + 1]);
      }
      if (masked && t0 + 4 * rr + kq >= s.t_end) {
#pragma unroll
        for (int e = 0; e < VPL; ++e) v[e] = 0.f;
      }
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[g][e] = fmaf(pg[g], v[e], o[g][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // PV on the matrix cores for the tile in stage `st` (MPV): this lane's column is query head m16
  // and its k values are tokens 4 kq .. 4 kq + 3, so the rescale by alpha and the probabilities
  // are lane-local.  The A operand (V^T) of tile j is dim 64 (j / 4) + 4 m16 + j % 4 of those
  // four tokens, cut out of two 8-byte reads per token row; tokens at or past t_end read as zero
  // (their slots may hold anything, and 0 x NaN is NaN).
  // The eight 8-byte reads of the V^T operand rows of stage `st` (MPV): dims 64 h + 4 m16 .. + 3
  // of token rows 4 kq + i.
  __device__ void pv_read(int st, u32x2 (&r)[2][4]) const {
    const uint32_t vs = lds_base + VSTAGE0 + uint32_t(st * Geo::KTILE);
    const uint32_t a0 = vs + v_rd, a1 = vs + v_rd2;
    r[0][0] = lds_read8_at<0 * Geo::RB>(a0);
    r[0][1] = lds_read8_at<1 * Geo::RB>(a0);
    r[0][2] = lds_read8_at<2 * Geo::RB>(a0);
    r[0][3] = lds_read8_at<3 * Geo::RB>(a0);
    r[1][0] = lds_read8_at<0 * Geo::RB>(a1);
    r[1][1] = lds_read8_at<1 * Geo::RB>(a1);
    r[1][2] = lds_read8_at<2 * Geo::RB>(a1);
    r[1][3] = lds_read8_at<3 * Geo::RB>(a1);
  }

  __device__ void pv_mfma(u32x2 (&r)[2][4], int t0, bool masked, int t_end, const float (&pr)[4],
                          float alpha, int G) {
    const bool rescale = __ballot(m16 < G && alpha != 1.f) != 0;
    if (rescale) {
#pragma unroll
      for (int j = 0; j < NDT; ++j) o4[j] *= alpha;
    }
    uint32_t h01, l01, h23, l23;
    split_pair<DT>(pr[0], pr[1], h01, l01);
    split_pair<DT>(pr[2], pr[3], h23, l23);
    const u32x4 pop = {h01, h23, l01, l23};
    lds_wait();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_pin(r[h][i]);
    if (masked) {   // r[h][i] holds token 4 kq + i only
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t mi = t0 + 4 * kq + i < t_end ? ~0u : 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) r[h][i] = u32x2{r[h][i].x & mi, r[h][i].y & mi};
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // element jj of the four dims read: low (jj even) or high halves of word jj / 2
        constexpr uint32_t kSel[2] = {0x05040100u, 0x07060302u};
        const int w = jj >> 1;
        const uint32_t v01 = __builtin_amdgcn_perm(r[h][1][w], r[h][0][w], kSel[jj & 1]);
        const uint32_t v23 = __builtin_amdgcn_perm(r[h][3][w], r[h][2][w], kSel[jj & 1]);
        o4[4 * h + jj] = mfma32<DT>(u32x4{v01, v23, v01, v23}, pop, o4[4 * h + jj]);
      }
  }

  // All of this wave's tiles: chunks of up to 64 tiles, DEPTH tiles in flight.
  // Wait until the oldest stage in flight has landed, given that `later` stages were issued
  // after it (at most N): every load but the newest later * LOADS has completed.
  template <int N>
  __device__ static void wait_stage(int later) {
    if constexpr (N == 0) {
      wait_vmcnt<0>();
    } else {
      if (later >= N) wait_vmcnt<N * Geo::LOADS>();
      else wait_stage<N - 1>(later);
    }
  }
  // The same for a wave that loads half of every tile (NKL loads).
  template <int N>
  __device__ static void wait_stage_half(int later) {
    if constexpr (N == 0) {
      wait_vmcnt<0>();
    } else {
      if (later >= N) wait_vmcnt<N * NKL>();
      else wait_stage_half<N - 1>(later);
    }
  }

  // Stream all of this wave's tiles of `s`.  With has_next, the loads of the next run()'s q and
  // first page ids (for `next`) start as the last chunk begins (see prefetch).  When prefetch() ran for `s`,
  // its q is taken here and its first page ids are used.  `at_start` runs once per call, on
  // every wave, after all of this wave's earlier memory operations have completed and before
  // any load of `s`'s tiles is issued.
  // lockstep: every wave of the workgroup streams the same tile list (one wave per KV head, or
  // waves that split a head's query heads); a barrier per round of DEPTH tiles then keeps the
  // waves together, so that the rows of all heads of a token are read close in time and no wave
  // falls behind the others.  Waves that share their stages (s.part) meet at a barrier around
  // every tile instead.
  __device__ void run(const HeadSource& s, float scale_log2, int G) {
    run(s, scale_log2, G, s, false, false, [] {});
  }
  template <class AtStart>
  __device__ void run(const HeadSource& s, float scale_log2, int G, const HeadSource& next,
                      bool has_next, bool lockstep, AtStart&& at_start) {
    const int n_my = tiles_of(s);
    const bool had_pref = pref_ready;
    if (pref_ready) {
#pragma unroll
      for (int c = 0; c < NKL; ++c) qreg[c] = q_pref[c];
      if constexpr (ROPE) rope_q();
      pref_ready = false;
    }
    for (int c0 = 0; c0 < n_my; c0 += kChunk) {
      const int nc = min(kChunk, n_my - c0);
      // Lane j holds the page id of this wave's chunk tile min(j, nc - 1).
      const int page_vec = (c0 == 0 && had_pref) ? pv_pref : chunk_pages(s, c0, nc);
      // The page ids (and anything older) have landed before the next piece's prefetch is
      // issued, so no later wait for them can also wait for the prefetch.
      wait_vmcnt<0>();
      if (c0 == 0) at_start();
      if (has_next && c0 + kChunk >= n_my) prefetch(next, G);   // the last chunk
      auto page_at = [&](int k) { return __builtin_amdgcn_readlane(page_vec, min(k, nc - 1)); };
      auto tile_at = [&](int k) { return s.sub + (c0 + min(k, nc - 1)) * s.stride; };
      auto ok = [&](int pg) { return pg >= 0 && pg < s.num_pages; };

      // The first DEPTH stages are always loaded (a chunk shorter than DEPTH tiles repeats its
      // last tile), so that the count of loads in flight is the same on every path into the loop.
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) issue(s, d, tile_at(d), page_at(d));
      int k = 0;
      // Steady state: every stage is refilled with a tile of the chunk, so the loads issued
      // after stage d's are always those of DEPTH - 1 stages.
      for (; k + 2 * DEPTH <= nc; k += DEPTH) {
        if (lockstep && !s.part) __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          if (s.part) {
            wait_vmcnt<(DEPTH - 1) * NKL>();
            __builtin_amdgcn_s_barrier();   // the partner's half of the tile has landed too
          } else {
            wait_vmcnt<(DEPTH - 1) * Geo::LOADS>();
          }
          if (ok(page_at(k + d))) process(s, d, tile_at(k + d), scale_log2, G); else bad = true;
          if (s.part) __builtin_amdgcn_s_barrier();   // the partner is done with the stage
          issue(s, d, tile_at(k + d + DEPTH), page_at(k + d + DEPTH));
        }
      }
      // Tail: only tiles of the chunk are loaded, so the loads issued after stage d's (tile
      // k + d) are those of tiles k + d + 1 ... k + d + DEPTH - 1 that exist.
      for (; k < nc; k += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          if (s.part) {
            wait_stage_half<DEPTH - 1>(nc - 1 - (k + d));
          } else {
            wait_stage<DEPTH - 1>(nc - 1 - (k + d));
          }
          if (k + d < nc) {
            if (s.part) __builtin_amdgcn_s_barrier();
            if (ok(page_at(k + d))) process(s, d, tile_at(k + d), scale_log2, G); else bad = true;
            if (s.part) __builtin_amdgcn_s_barrier();
          }
          if (k + d + DEPTH < nc) issue(s, d, tile_at(k + d + DEPTH), page_at(k + d + DEPTH));
        }
      }
      wait_vmcnt<0>();   // nothing is in flight here; this states it for the next chunk
    }
    if (n_my == 0) {   // no tiles of `s` for this wave
      wait_vmcnt<0>();
      at_start();
      if (has_next) prefetch(next, G);
    }
  }

  // Reduce the wave's state across its 4 row groups and store it at `ep` (LDS):
  // o[GP][D], then m[GP], l[GP], bad.
  __device__ void to_lds(float* ep) {
    l_run = sum_rows4(l_run);
    if constexpr (MPV) {
      if (m16 < GP) {   // dims 64 h + 16 kq + 4 q .. + 3 of head m16: 16-byte writes
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(ep + m16 * D + 64 * h + 16 * kq + 4 * q) =
                f32x4{o4[4 * h][q], o4[4 * h + 1][q], o4[4 * h + 2][q], o4[4 * h + 3][q]};
      }
    } else {
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[g][e] = sum_rows4(o[g][e]);
      if (lane < 16) {
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
          for (int e = 0; e < VPL; ++e) ep[g * D + lane * VPL + e] = o[g][e];
      }
    }
    if (lane < GP) {
      ep[GP * D + lane] = m_run;
      ep[GP * D + GP + lane] = l_run;
      ep[GP * D + 2 * GP + lane] = bad ? 1.f : 0.f;
    }
  }

  // Finish a head that this wave served alone, from registers: for each query head g < G of
  // the group, emit(g, d0, vals, lse) with vals[e] = o / l for dims d0 + e (lanes 0..15 each
  // hold VPL dims), lse in natural log.  The same arithmetic as combine_waves with one wave
  // (its weight 2^0 is exactly 1), so the results are identical.
  template <class Emit>
  __device__ void finish_direct(int G, Emit emit) {
    l_run = sum_rows4(l_run);
    if constexpr (MPV) {
      // Lane (m16, kq) of a real head: dims 64 h + 16 kq .. + 15 of head m16.
      if (m16 < G) {
        // MQ, l = 0: a column with no token in this range (output 0, lse -inf)
        const float lse = bad ? qnan() : (m_run + __builtin_amdgcn_logf(fmaf(1.f, l_run, 0.f))) * kLn2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float vals[16];
#pragma unroll
          for (int e = 0; e < 16; ++e)
            vals[e] = bad ? qnan() : MQ && !(l_run > 0.f) ? 0.f : fmaf(1.f, o4[4 * h + e % 4][e / 4], 0.f) / fmaf(1.f, l_run, 0.f);
          emit(m16, 64 * h + 16 * kq, vals, lse);
        }
      }
      return;
    }
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < VPL; ++e) o[g][e] = sum_rows4(o[g][e]);
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g >= G) break;
      const float lg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_run), g));
      const float mg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), g));
      float vals[VPL];
#pragma unroll
      for (int e = 0; e < VPL; ++e) vals[e] = bad ? qnan() : MQ && !(lg > 0.f) ? 0.f : fmaf(1.f, o[g][e], 0.f) / fmaf(1.f, lg, 0.f);
      const float lse = bad ? qnan() : (mg + __builtin_amdgcn_logf(fmaf(1.f, lg, 0.f))) * kLn2;
      if (lane < 16) emit(g, lane * VPL, vals, lse);
    }
  }
};

// Combine the waves that served one head (waves h_in, h_in + hpw, ...) and hand each output
// element to `emit(h_in, g, d, value, lse, nan)`: value = o / l, lse in natural log.  EMPTY_OK:
// a column may have no token in any wave (multi-query decode): value 0, lse -inf.
template <int D, int GP, int WREG, bool EMPTY_OK, class Emit>
__device__ void combine_waves(const char* w_lds, int hpw, int wph, int G, int nthreads, Emit emit) {
  for (int idx = threadIdx.x; idx < hpw * G * D; idx += nthreads) {
    const int h_in = idx / (G * D);
    const int g = (idx / D) % G;
    const int d = idx % D;
    float M = neg_inf();
    float any_bad = 0.f;
    for (int k = 0; k < wph; ++k) {
      const float* e = reinterpret_cast<const float*>(w_lds + (h_in + k * hpw) * WREG);
      M = fmaxf(M, e[GP * D + g]);
      any_bad += e[GP * D + 2 * GP];
    }
    const float Mu = EMPTY_OK && M == neg_inf() ? 0.f : M;
    float lsum = 0.f, osum = 0.f;
    for (int k = 0; k < wph; ++k) {
      const float* e = reinterpret_cast<const float*>(w_lds + (h_in + k * hpw) * WREG);
      const float sc = fast_exp2(e[GP * D + g] - Mu);
      lsum = fmaf(sc, e[GP * D + GP + g], lsum);
      osum = fmaf(sc, e[g * D + d], osum);
    }
    const bool nan_out = any_bad != 0.f;
    const bool empty = EMPTY_OK && !(lsum > 0.f);
    emit(h_in, g, d, nan_out ? qnan() : empty ? 0.f : osum / lsum,
         nan_out ? qnan() : empty ? neg_inf() : (M + __builtin_amdgcn_logf(lsum)) * kLn2, nan_out);
  }
}

// ---------------------------------------------------------------------------------------------
// Fixed partitions
// ---------------------------------------------------------------------------------------------

// One workgroup per (sequence, partition, group of KV heads).  Wave w serves KV head
// hg * HPW + w % HPW and takes that head's tiles w / HPW, + WPH, ... (HPW heads per workgroup,
// WPH = NW / HPW waves per head).
// Workgroup `id` of the grid with its LDS `sm` (a kernel of its own, or part of a fused grid).
template <int DT, int D, int GP, int NW, int DEPTH, bool PARTIAL>
__device__ inline void decode_body(const DecodeParams& p, int id,
                                   DecodeShared<DT, D, GP, NW, DEPTH>& sm) {
  using Geo = TileGeo<DT, D>;
  using Shm = DecodeShared<DT, D, GP, NW, DEPTH>;
  static_assert(GP == 4 || GP == 8 || GP == 16, "padded group");
  static_assert((DEPTH - 1) * Geo::LOADS < 64, "vmcnt range");

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.group;
  const int HPW = p.heads_per_wg;
  const int WPH = NW / HPW;

  const int nhg = p.hkv / HPW;
  const int hg = id % nhg;
  id /= nhg;
  const int b = id % p.batch;
  const int part = PARTIAL ? p.part_begin + id / p.batch : 0;
  const int kvh = hg * HPW + wave % HPW;

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
      for (int idx = threadIdx.x; idx < HPW * G * D; idx += NW * 64) {
        const int h = (hg * HPW + idx / (G * D)) * G + (idx / D) % G;
        store_elem<DT>(p.out, (int64_t(b) * p.hq + h) * D + idx % D, fill);
      }
      return;
    }
  }

  HeadPipe<DT, D, GP, DEPTH> hp;
  hp.init(p.tok_stride, lds_addr(sm.w[wave]), &sm.p[wave][0][0], &sm.a[wave][0]);
  hp.load_q(static_cast<const char*>(p.q) + (int64_t(b) * p.hq + int64_t(kvh) * G) * Geo::RB, G);
  hp.reset();
  HeadSource src;
  src.kpool = static_cast<const char*>(p.k_pool);
  src.vpool = static_cast<const char*>(p.v_pool);
  src.table = p.page_table + int64_t(b) * p.max_pages;
  src.page_shift = p.page_shift;
  src.num_pages = p.num_pages;
  src.tok_stride = p.tok_stride;
  src.page_stride = p.page_stride;
  src.head_off = kvh * Geo::RB;
  src.t_begin = t_begin;
  src.t_end = t_end;
  src.sub = wave / HPW;
  src.stride = WPH;
  hp.run(src, p.scale_log2, G);
  hp.to_lds(reinterpret_cast<float*>(sm.w[wave]));
  __syncthreads();

  combine_waves<D, GP, Shm::WREG, false>(&sm.w[0][0], HPW, WPH, G, NW * 64,
      [&](int h_in, int g, int d, float val, float lse, bool) {
        const int h = (hg * HPW + h_in) * G + g;
        if constexpr (PARTIAL) {
          const int64_t rowi = (int64_t(b) * p.hq + h) * p.max_partitions + part;
          p.partial_out[rowi * D + d] = val;
          if (d == 0) p.partial_lse[rowi] = lse;
        } else {
          store_elem<DT>(p.out, (int64_t(b) * p.hq + h) * D + d, val);
        }
      });
}

template <int DT, int D, int GP, int NW, int DEPTH, bool PARTIAL>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams p) {
  __shared__ DecodeShared<DT, D, GP, NW, DEPTH> sm;
  decode_body<DT, D, GP, NW, DEPTH, PARTIAL>(p, blockIdx.x, sm);
}

// Shared-prefix decode, both kinds of partition in one grid: workgroups [0, n_dec) take the
// suffix partitions (as decode_kernel's partial mode), [n_pre0, n_pre0 + prefix units) the prefix
// partitions on the matrix cores (as prefix_kernel); n_pre0 is n_dec rounded up to a multiple of
// 8, so that a prefix workgroup keeps the XCD (block index mod 8) it has in a grid of its own,
// and the workgroups in between do nothing.  The two kinds share no data, so they run side by
// side: blocks are dispatched in index order, and the prefix workgroups take the compute units
// that the short suffix partitions leave early.  One LDS allocation serves either kind.
template <int DT, int D, int GP, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void cascade_kernel(const DecodeParams d, const PrefixParams pp,
                                                          int n_dec, int n_pre0) {
  static_assert(NW == kPrefixWaves, "one block size for both kinds of workgroup");
  union Shared {
    DecodeShared<DT, D, GP, NW, DEPTH> dec;
    PrefixShared<D> pre;
  };
  __shared__ Shared sm;
  const int id = blockIdx.x;
  if (id < n_dec)
    decode_body<DT, D, GP, NW, DEPTH, true>(d, id, sm.dec);
  else if (id >= n_pre0)
    prefix_body<DT, D, NW, kPrefixRowBlocks, false>(pp, id - n_pre0, sm.pre);
}

// ---------------------------------------------------------------------------------------------
// Balanced decode step
// ---------------------------------------------------------------------------------------------

// Tiles attended by sequence b in a step (0 for padding rows and rows whose length exceeds the
// page table's capacity; the latter get NaN outputs from the merge).
__device__ inline int step_tiles(const StepParams& p, int b) {
  const int L = p.a.context_lens[b];
  const int att = L < 0 ? 0 : L + p.append;
  if (att <= 0 || att > p.a.capacity) return 0;
  return (att + kTile - 1) / kTile;
}

// The split of a step's work over the workgroup ranges.  Every sequence b weighs 4 units per
// tile plus `su` start units: a range that starts a new sequence pays one pipeline drain and
// refill, so it gets that much less streaming.  `wpre` is the exclusive prefix of the weights
// (B + 1 entries, in LDS); the `groups` ranges cut the weighted line [0, WT) evenly, and a range
// owns the tiles whose weighted start falls in it.  Everything depends on the lengths only.
// The start weight was measured: three tiles with one wave per KV head (12 units: 113.5 us for
// the Llama-3-8B-shaped step, against 115.5 us at 8 and 118 us at 4; with PV on the matrix
// cores 16 and 20 units measure the same), six when several waves share a head (24 units: with
// PV on the matrix cores, 40.2 us for the Qwen2-7B-shaped step with its pairs of waves sharing
// stages, against 41.7 at 16, and 41.1 against 41.8 on another device, where 32 and 40 gave 41.9
// and 41.4).
__device__ inline int start_units(int waves_per_head) { return waves_per_head == 1 ? 12 : 24; }

struct StepSplit {
  const int* wpre;
  int B;
  int64_t WT, groups;
  int su;   // start units per sequence

  // Tiles of the sequences before b (the exclusive tile prefix).
  __device__ int tiles_before(int b) const { return (wpre[b] - su * b) >> 2; }
  __device__ int total_tiles() const { return tiles_before(B); }
  __device__ int64_t bound(int64_t w) const { return w * WT / groups; }

  // The last b in [0, B] with f(b) <= x, for f nondecreasing with f(0) <= x: up to
  // kParallelSearch entries are compared by the wave's lanes at once (the count of b in [1, B]
  // with f(b) <= x), longer batches are bisected.
  static constexpr int kParallelSearch = 256;
  template <class F>
  __device__ int last_le(F f, int64_t x) const {
    if (B <= kParallelSearch) {
      const int lane = threadIdx.x & 63;
      int c = 0;
      for (int i0 = 1; i0 <= B; i0 += 64) {
        const uint64_t m = __ballot(i0 + lane <= B && f(i0 + lane) <= x);
        c += __popcll(m);
        if (~m != 0) break;
      }
      return c;
    }
    int l = 0, r = B + 1;
    while (r - l > 1) {
      const int m = (l + r) >> 1;
      if (f(m) <= x) l = m; else r = m;
    }
    return l;
  }
  // The last b in [0, B] with wpre[b] <= x.
  __device__ int seq_at(int64_t x) const { return last_le([&](int b) { return int64_t(wpre[b]); }, x); }
  // The sequence holding tile t (tiles_before(b) <= t < tiles_before(b + 1)).
  __device__ int seq_of_tile(int t) const {
    return last_le([&](int b) { return int64_t(tiles_before(b)); }, t);
  }
  // The first tile whose weighted start (wpre[b] + su + 4 k for tile k of b) is >= x.
  __device__ int first_tile_at(int64_t x) const {
    const int b = seq_at(x);
    if (b >= B) return total_tiles();
    const int64_t o = x - wpre[b] - su;
    const int t0 = tiles_before(b);
    const int k = o <= 0 ? 0 : int((o + 3) >> 2);
    return min(t0 + k, tiles_before(b + 1));
  }
  __device__ int range_lo(int64_t w) const { return first_tile_at(bound(w)); }
  // Within sequence b (n tiles, weighted starts base + 4 k with base = wpre[b] + su),
  // no search is needed: the range owning weighted position x, and how many of b's tiles range
  // w holds.
  __device__ int64_t range_of_pos(int64_t x) const { return ((x + 1) * groups - 1) / WT; }
  __device__ int tiles_in(int64_t w, int64_t base, int n) const {
    const int64_t o0 = bound(w) - base, o1 = bound(w + 1) - base;
    const int64_t k0 = o0 <= 0 ? 0 : min<int64_t>(n, (o0 + 3) >> 2);
    const int64_t k1 = o1 <= 0 ? 0 : min<int64_t>(n, (o1 + 3) >> 2);
    return int(k1 - k0);
  }
};

// Row (in head_dim rows) of q, out and lse_out for sequence b and head h of the step.  The
// multi-query step (q_tokens = T > 1) runs over T x Hq heads: head kvh * G + c (G = T x the GQA
// group QG) is query token c / QG of query head kvh * QG + c % QG, whose rows are [b, T, Hq].
__device__ inline int64_t step_row(const StepParams& p, int b, int h) {
  const int T = p.q_tokens;
  if (T <= 1) return int64_t(b) * p.a.hq + h;
  const int G = p.a.group, QG = G / T, HQ = p.a.hq / T;
  const int kvh = h / G, c = h - kvh * G;
  return (int64_t(b) * T + c / QG) * HQ + int64_t(kvh) * QG + c % QG;
}

// A piece of `tiles` tiles arrives on its sequence's counter (pkv_arrival.h): the word is first
// raised to this call's floor, so that a count an earlier call left behind starts again from zero,
// then the tiles are added.  Returns the tiles this call had counted before.
__device__ inline int arrive(uint64_t* counter, uint32_t generation, int tiles) {
  __hip_atomic_fetch_max(counter, arrival_floor(generation), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t old = __hip_atomic_fetch_add(counter, uint64_t(tiles), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  return int(arrival_count(old));
}

// Exclusive prefix sum of the weights 4 * step_tiles(b) + su over the batch into `wpre`
// (B + 1 entries), and the tokens attended in each sequence's last tile (1..16) into `tail`, so
// that no later step needs the lengths from global memory.  `scan` is NT / 64 ints of scratch
// (or more).  All threads of the block take part.
template <int NT>
__device__ void weight_prefix(const StepParams& p, int su, int* wpre, uint8_t* tail, int* scan) {
  const int B = p.a.batch;
  const int tid = threadIdx.x;
  const int seg = (B + NT - 1) / NT;
  const int lo = min(B, tid * seg), hi = min(B, lo + seg);
  int local = 0;
  for (int b = lo; b < hi; ++b) local += 4 * step_tiles(p, b) + su;
  // Inclusive scan within each wave by shuffles; the waves' totals meet in LDS (one barrier).
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if ((tid & 63) >= off) incl += v;
  }
  if ((tid & 63) == 63) scan[tid >> 6] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int wv = 0; wv < NT / 64; ++wv) {
    before += wv < (tid >> 6) ? scan[wv] : 0;
    total += scan[wv];
  }
  int run = before + incl - local;
  for (int b = lo; b < hi; ++b) {
    wpre[b] = run;
    const int n = step_tiles(p, b);
    run += 4 * n + su;
    tail[b] = uint8_t(n > 0 ? p.a.context_lens[b] + p.append - (n - 1) * kTile : 0);
  }
  if (tid == NT - 1) wpre[B] = total;
  __syncthreads();
}

// Merge of sequence b's pieces for the NH query heads of head group hg:
// out = sum_p w_p o_p / sum_p w_p with w_p = 2^((lse_p - M) log2 e), pieces in workgroup order.
// Each thread takes two float4 columns and issues the loads of up to kMU pieces of both at once
// (16-byte device-scope loads of the partial rows, one device-scope load of each log-sum-exp),
// carrying a running maximum from one group of pieces to the next.
// `flags` (NT ints of LDS) receives which of the first NT candidate ranges hold a piece; all
// threads of the block take part.
template <int DT, int D, int NT, bool MQ>
__device__ void step_merge(const StepParams& p, const StepSplit& sp, int b, int hg, int NH, int S,
                           int E, int* flags) {
  constexpr int kMU = 8, kCols = 2;
  const DecodeParams& a = p.a;
  const int n = E - S;
  const int64_t base = sp.wpre[b] + sp.su;   // weighted start of the sequence's first tile
  const int64_t w_lo = sp.range_of_pos(base);
  const int npc = int(sp.range_of_pos(base + 4 * int64_t(n - 1)) - w_lo + 1);   // candidate ranges
  // A range at least one tile wide (4 weight units) holds a tile of every sequence it lies
  // inside, so every candidate holds a piece and no flags are needed.
  const bool dense = sp.WT >= 4 * sp.groups;
  if (!dense) {
    if (threadIdx.x < min(npc, NT)) flags[threadIdx.x] = sp.tiles_in(w_lo + threadIdx.x, base, n) > 0;
    __syncthreads();
  }
  const int ncol = NH * (D / 4);
  // Byte offsets below are relative to the first candidate's partial rows.
  const int64_t row0 = (w_lo + b) * a.hq;
  const BufRes rows = make_bufres(p.ws_out + row0 * D, uint32_t(npc) * uint32_t(a.hq * D * 4));
  for (int c0 = threadIdx.x; c0 < ncol; c0 += NT * kCols) {
    float m[kCols], l[kCols], o[kCols][4];
    int h[kCols], d0[kCols];
#pragma unroll
    for (int k = 0; k < kCols; ++k) {
      const int c = min(c0 + k * NT, ncol - 1);   // a spare column repeats the last one
      h[k] = hg * NH + c / (D / 4);
      d0[k] = (c % (D / 4)) * 4;
      m[k] = neg_inf();
      l[k] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[k][j] = 0.f;
    }
    // Pieces k0 .. k0 + kMU - 1: their log-sum-exps and rows, in flight together.
    auto load_round = [&](int k0, float (&ls)[kCols][kMU], f32x4 (&vs)[kCols][kMU]) {
#pragma unroll
      for (int u = 0; u < kMU; ++u) {
        const int k = k0 + u;
        const bool ok = k < npc && (dense || (k < NT ? flags[k] != 0 : sp.tiles_in(w_lo + k, base, n) > 0));
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          const int64_t row = int64_t(k) * a.hq + h[c];
          ls[c][u] = ok ? dev_load(&p.ws_lse[row0 + row]) : neg_inf();
          vs[c][u] = ok ? dev_load16(rows, uint32_t(row * D + d0[c]) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    };
    // Fold one round into the running (m, l, o), pieces in order.
    auto combine = [&](const float (&ls)[kCols][kMU], const f32x4 (&vs)[kCols][kMU]) {
#pragma unroll
      for (int k = 0; k < kCols; ++k) {
        float mc = m[k];
#pragma unroll
        for (int u = 0; u < kMU; ++u) mc = fmaxf(mc, ls[k][u]);
        const float mu = MQ && mc == neg_inf() ? 0.f : mc;   // MQ: no piece saw a token of the column
        const float r = fast_exp2((m[k] - mu) * kLog2e);
        l[k] *= r;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[k][j] *= r;
#pragma unroll
        for (int u = 0; u < kMU; ++u) {
          const float wt = fast_exp2((ls[k][u] - mu) * kLog2e);
          l[k] += wt;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[k][j] = fmaf(wt, vs[k][u][j], o[k][j]);
        }
        m[k] = mc;
      }
    };
    // Two register sets: the next round's loads are issued before the current round is folded,
    // so a sequence cut into many pieces pays about one round trip, not one per round.  The fold
    // order (and so every bit of the result) is that of one round after the other.
    float lsA[kCols][kMU], lsB[kCols][kMU];
    f32x4 vsA[kCols][kMU], vsB[kCols][kMU];
    load_round(0, lsA, vsA);
    for (int k0 = 0;;) {
      const bool more_b = k0 + kMU < npc;
      if (more_b) load_round(k0 + kMU, lsB, vsB);
      combine(lsA, vsA);
      k0 += kMU;
      if (!more_b) break;
      const bool more_a = k0 + kMU < npc;
      if (more_a) load_round(k0 + kMU, lsA, vsA);
      combine(lsB, vsB);
      k0 += kMU;
      if (!more_a) break;
    }
#pragma unroll
    for (int k = 0; k < kCols; ++k) {
      const int c = c0 + k * NT;
      if (c >= ncol) continue;
      const int64_t row = MQ ? step_row(p, b, h[k]) : int64_t(b) * a.hq + h[k];
      const int64_t obase = row * D + d0[k];
      const bool empty = MQ && !(l[k] > 0.f);
#pragma unroll
      for (int j = 0; j < 4; ++j) store_elem<DT>(p.out, obase + j, empty ? 0.f : o[k][j] / l[k]);
      if (d0[k] == 0 && p.lse_out)
        p.lse_out[row] = empty ? neg_inf() : m[k] + __builtin_amdgcn_logf(l[k]) * kLn2;
    }
  }
  __syncthreads();   // `flags` may be rewritten next
}

template <int DT, int D, int GP, int NW, int DEPTH, bool ROPE, bool MQ = false>
__global__ __launch_bounds__(NW * 64) void step_kernel(const StepParams p) {
  using Geo = TileGeo<DT, D>;
  using Shm = DecodeShared<DT, D, GP, NW, DEPTH>;
  static_assert((DEPTH - 1) * Geo::LOADS < 64, "vmcnt range");
  __shared__ Shm sm;
  __shared__ int wpre[kMaxStepBatch + 1];
  __shared__ uint8_t ltail[kMaxStepBatch];   // tokens attended in each sequence's last tile
  __shared__ int scan[NW * 64];

  const DecodeParams& a = p.a;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group;
  const int HPW = a.heads_per_wg;
  const int WPH = NW / HPW;
  const int nhg = a.hkv / HPW;
  const int hg = blockIdx.x % nhg;
  const int w = blockIdx.x / nhg;
  const int kvh = hg * HPW + wave % HPW;
  // This wave's query heads of the group: gs .. gs + Gw - 1 (all of them unless the waves of a
  // KV head split them; then every wave streams all of the head's tiles, in lockstep).
  const bool qsplit = p.qsplit != 0;
  const int GW = qsplit ? (G + WPH - 1) / WPH : G;
  const int gs = qsplit ? (wave / HPW) * GW : 0;
  const int Gw = qsplit ? min(GW, G - gs) : G;
  const bool own_heads = WPH == 1 || qsplit;   // the wave alone finishes its query heads
  // Two waves per KV head share its LDS stages: the first loads K, the second V, so that each
  // byte a compute unit has in flight is a different one (loading every row twice halved the
  // distinct bytes in flight and capped the stream).
  const int part = qsplit && WPH == 2 ? (wave < HPW ? 1 : 2) : 0;

  __shared__ int merging[2];
  int split_first = -1, split_last = -1;   // sequences whose piece here is split
  int first_tiles = 0, last_tiles = 0;      // ... and the tiles of those pieces

  const int su = start_units(WPH);
  weight_prefix<NW * 64>(p, su, wpre, ltail, scan);
  const int B = a.batch;
  const StepSplit sp{wpre, B, wpre[B], p.groups, su};
  auto prefix = [&](int x) { return sp.tiles_before(x); };   // tiles of the sequences before x
  // Rows without tiles (padding, or longer than the page table can address): 0 / NaN outputs,
  // written by one workgroup each.
  for (int bb = blockIdx.x; bb < B; bb += gridDim.x) {
    if (prefix(bb + 1) != prefix(bb)) continue;
    const bool pad = a.context_lens[bb] < 0 || a.context_lens[bb] + p.append <= 0;
    for (int i = threadIdx.x; i < a.hq * D; i += NW * 64)
      store_elem<DT>(p.out, int64_t(bb) * a.hq * D + i, pad ? 0.f : qnan());
    if (p.lse_out)
      for (int h = threadIdx.x; h < a.hq; h += NW * 64)
        p.lse_out[int64_t(bb) * a.hq + h] = pad ? neg_inf() : qnan();
  }
  const int lo = sp.range_lo(w);
  const int hi = sp.range_lo(w + 1);
  if (lo >= hi) return;

  int b = sp.seq_of_tile(lo);   // the sequence holding tile `lo`

  HeadPipe<DT, D, GP, DEPTH, ROPE, MQ> hp;
  hp.init(a.tok_stride, lds_addr(sm.w[part ? wave % HPW : wave]), &sm.p[wave][0][0], &sm.a[wave][0]);
  if constexpr (MQ) {
    // This lane's q row within the KV head's rows ([b, T, Hq]), from its column gs + m16.
    const int c = gs + (threadIdx.x & 15);
    const int QG = G / p.q_tokens, HQ = a.hq / p.q_tokens;
    hp.q_off = (int64_t(c / QG) * HQ + c % QG) * Geo::RB;
    hp.q_j = c / QG;
  }

  // This wave's source for sequence bb: the tiles of bb in this range, for its KV head.
  auto source = [&](int bb) {
    HeadSource src;
    const int tb = max(lo, prefix(bb)) - prefix(bb);
    const int te = min(hi, prefix(bb + 1)) - prefix(bb);
    src.kpool = static_cast<const char*>(a.k_pool);
    src.vpool = static_cast<const char*>(a.v_pool);
    src.table = a.page_table + int64_t(bb) * a.max_pages;
    src.page_shift = a.page_shift;
    src.num_pages = a.num_pages;
    src.tok_stride = a.tok_stride;
    src.page_stride = a.page_stride;
    src.head_off = kvh * Geo::RB;
    src.t_begin = tb * kTile;
    // tokens attended: (n - 1) whole tiles plus ltail[bb] (n = the sequence's tiles)
    const int n_bb = prefix(bb + 1) - prefix(bb);
    src.t_end = te < n_bb ? te * kTile : (n_bb - 1) * kTile + ltail[bb];
    src.sub = qsplit ? 0 : wave / HPW;
    src.stride = qsplit ? 1 : WPH;
    src.keep = qsplit && !part ? 1 : 0;
    src.part = part;   // the waves that split the head's query heads load its tiles alike
    src.q_group = static_cast<const char*>(a.q) +
                  (MQ ? step_row(p, bb, kvh * G) : int64_t(bb) * a.hq + int64_t(kvh) * G + gs) * Geo::RB;
    src.rope_cos = p.rope_cos;
    src.rope_sin = p.rope_sin;
    src.rope_pos = -1;
    if constexpr (MQ) src.causal0 = (n_bb - 1) * kTile + ltail[bb] - p.q_tokens + 1;
    if constexpr (ROPE) {
      const int L = (n_bb - 1) * kTile + ltail[bb] - 1;   // the new token's position
      src.rope_pos = L >= 0 && L < p.rope_rows ? L : -1;
    }
    return src;
  };
  // The next sequence after bb with tiles in this range, or B.
  auto next_seq = [&](int bb) {
    for (++bb; bb < B && prefix(bb) < hi; ++bb)
      if (prefix(bb + 1) > prefix(bb)) return bb;
    return B;
  };

  // Each piece's q and first page ids are loaded while the previous piece drains; the first
  // piece's load while the appended rows are written (they read neither the pools nor the rows).
  HeadSource cur = source(b);
  hp.prefetch(cur, Gw);

  // The appended rows of every sequence whose last tile lies in this range are written first;
  // the barrier (which waits for the stores) orders them before any load of those tiles.  No
  // other workgroup reads those slots in this step.
  if (p.append) {
    const int row_bytes = a.hkv * Geo::RB;
    for (int bb = b; bb < B && prefix(bb) < hi; ++bb) {
      if (prefix(bb + 1) == prefix(bb) || prefix(bb + 1) > hi) continue;
      const int L = (prefix(bb + 1) - prefix(bb) - 1) * kTile + ltail[bb] - 1;   // the new row's slot
      const int page = a.page_table[int64_t(bb) * a.max_pages + (L >> a.page_shift)];
      if (page < 0 || page >= a.num_pages) continue;
      const int64_t dst = int64_t(page) * a.page_stride +
                          int64_t(L & ((1 << a.page_shift) - 1)) * a.tok_stride +
                          int64_t(hg) * HPW * Geo::RB;
      const int64_t srco = int64_t(bb) * row_bytes + int64_t(hg) * HPW * Geo::RB;
      for (int i = threadIdx.x; i < HPW * Geo::RB / 16; i += NW * 64) {
        const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.v_new) + srco + 16 * i);
        *reinterpret_cast<u32x4*>(static_cast<char*>(p.v_pool_w) + dst + 16 * i) = vv;
        if constexpr (!ROPE) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k_new) + srco + 16 * i);
          *reinterpret_cast<u32x4*>(static_cast<char*>(p.k_pool_w) + dst + 16 * i) = kv;
        }
      }
      if constexpr (ROPE) {
        // The key is written rotated: thread i takes 16-byte chunk j of the first half of a head
        // and the matching chunk of the second half (the pairs' partners).  A position without
        // a row in the rotary cache writes NaN, so the row's output shows it.
        using V = Vec16<DT>;
        constexpr int HALF = Geo::RB / 32;   // 16-byte chunks per half head
        const bool on = L < p.rope_rows;
        const float* cs = p.rope_cos + int64_t(on ? L : 0) * (D / 2);
        const float* sn = p.rope_sin + int64_t(on ? L : 0) * (D / 2);
        for (int i = threadIdx.x; i < HPW * HALF; i += NW * 64) {
          const int j = i % HALF;
          const int64_t off = int64_t(i / HALF) * Geo::RB + 16 * j;
          const char* src = static_cast<const char*>(p.k_new) + srco + off;
          float x1[V::N], x2[V::N], y1[V::N], y2[V::N];
          V::unpack(*reinterpret_cast<const u32x4*>(src), x1);
          V::unpack(*reinterpret_cast<const u32x4*>(src + Geo::RB / 2), x2);
#pragma unroll
          for (int e = 0; e < V::N; ++e) {
            rope_pair(x1[e], x2[e], cs[j * V::N + e], sn[j * V::N + e], y1[e], y2[e]);
            if (!on) y1[e] = y2[e] = qnan();
          }
          char* d = static_cast<char*>(p.k_pool_w) + dst + off;
          *reinterpret_cast<u32x4*>(d) = V::pack(y1);
          *reinterpret_cast<u32x4*>(d + Geo::RB / 2) = V::pack(y2);
        }
      }
    }
    __syncthreads();
  }

  // The range's first piece, when split, is counted as soon as the next piece starts: every wave
  // has then waited for its own stores, and the barrier (the waves reach it together) makes that
  // true of the whole partial.  Its result is read at the end of the range.  A range's first
  // piece is the tail of a sequence whose other pieces end at the end of their ranges, so the
  // count almost never comes in last, and the workgroup that finishes a range rarely has two
  // merges to do.
  int early_b = -1, early_tiles = 0, early_ret = 0;
  auto count_first = [&] {
    if (early_b < 0 || early_tiles == 0) return;
    __syncthreads();   // every wave's partial stores have completed
    if (threadIdx.x == 0)
      early_ret = arrive(&p.ws_count[int64_t(early_b) * nhg + hg], p.generation, early_tiles);
    early_tiles = 0;
  };
  while (true) {
    const int nb = next_seq(b);
    const bool has_next = nb < B;
    const HeadSource nxt = source(has_next ? nb : b);
    hp.reset();
    hp.run(cur, a.scale_log2, Gw, nxt, has_next, own_heads, count_first);

    const int n_b = prefix(b + 1) - prefix(b);
    const int tb = max(lo, prefix(b)) - prefix(b);
    const int te = min(hi, prefix(b + 1)) - prefix(b);
    const bool whole = tb == 0 && te == n_b;   // this workgroup holds all of the sequence
    const int64_t slot = int64_t(w) + b;
    if (own_heads) {
      // The wave finishes its query heads from registers, with no barrier.
      hp.finish_direct(Gw, [&](int g, int d0, const auto& vals, float lse) {
        constexpr int N = sizeof(vals) / sizeof(float);   // contiguous dims from d0
        const int h = kvh * G + gs + g;
        if (whole) {
          const int64_t row = MQ ? step_row(p, b, h) : int64_t(b) * a.hq + h;
          store_row<DT, N>(p.out, row * D + d0, vals);
          if (d0 == 0 && p.lse_out) p.lse_out[row] = lse;
        } else {   // device-scope stores: written through to where every XCD reads
          const BufRes row = make_bufres(&p.ws_out[(slot * a.hq + h) * D], uint32_t(D * 4));
#pragma unroll
          for (int c = 0; c < N / 4; ++c)
            dev_store16(row, uint32_t(d0 + 4 * c) * 4u,
                        f32x4{vals[4 * c], vals[4 * c + 1], vals[4 * c + 2], vals[4 * c + 3]});
          if (d0 == 0) dev_store(&p.ws_lse[slot * a.hq + h], lse);
        }
      });
    } else {
      hp.to_lds(reinterpret_cast<float*>(sm.w[wave]));
      __syncthreads();
      combine_waves<D, GP, Shm::WREG, MQ>(&sm.w[0][0], HPW, WPH, G, NW * 64,
          [&](int h_in, int g, int d, float val, float lse, bool) {
            const int h = (hg * HPW + h_in) * G + g;
            if (whole) {
              const int64_t row = MQ ? step_row(p, b, h) : int64_t(b) * a.hq + h;
              store_elem<DT>(p.out, row * D + d, val);
              if (d == 0 && p.lse_out) p.lse_out[row] = lse;
            } else {
              dev_store(&p.ws_out[(slot * a.hq + h) * D + d], val);
              if (d == 0) dev_store(&p.ws_lse[slot * a.hq + h], lse);
            }
          });
      __syncthreads();   // the LDS epilogue area is reused by the next piece
    }

    if (!whole) {   // a split piece starts or ends the range
      if (tb > 0) {
        split_first = b;
        first_tiles = te - tb;
        early_b = b, early_tiles = first_tiles;
      } else {
        split_last = b;
        last_tiles = te - tb;
      }
    }
    if (!has_next) break;
    b = nb;
    cur = nxt;
  }

  // Count the split pieces' tiles in (at most two pieces: the range's first and last; the first
  // one was usually counted already, see count_first); the workgroup that brings a sequence's
  // count to its number of tiles merges all of its pieces.
  // The hand-off between workgroups, which may run on different XCDs (each XCD's L2 is not
  // coherent with the others), is the agent-scope release / acquire pattern of the AMDGPU memory
  // model without its cache maintenance, which has nothing to act on here:
  //  * producer: the partials are agent-scope relaxed atomic stores (global/buffer stores with
  //    sc1, written through to the device's coherence point); s_waitcnt vmcnt(0) waits until
  //    every one of this thread's stores is complete; the barrier (a workgroup fence plus
  //    s_barrier, which the compiler does not move memory operations across) orders all threads'
  //    completed stores before thread 0's agent-scope counter update (relaxed agent-scope
  //    atomicrmw: global_atomic_umax / global_atomic_add, which act at agent scope as emitted);
  //  * consumer: the merging workgroup reads the final count from its own update's return value,
  //    passes a barrier, and only then issues its loads of the partials, as agent-scope relaxed
  //    atomic loads (sc1), which return the value at the coherence point, not an L2 copy.
  // A release would add buffer_wbl2 (write back L2 lines that plain stores dirtied) and an acquire
  // buffer_inv (drop L2 lines that plain loads could hit); the partials are never written or read
  // by plain accesses, so the write-back and the invalidate are not needed.
  if (split_first < 0 && split_last < 0) return;
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x < 2) {
    const int sb = threadIdx.x == 0 ? split_first : split_last;
    const int tiles = threadIdx.x == 0 ? first_tiles : last_tiles;
    int last = 0;
    if (sb >= 0) {
      const bool counted = threadIdx.x == 0 && early_b == sb && early_tiles == 0;
      const int old = counted ? early_ret
                              : arrive(&p.ws_count[int64_t(sb) * nhg + hg], p.generation, tiles);
      last = old + tiles == prefix(sb + 1) - prefix(sb);
    }
    merging[threadIdx.x] = last;
  }
  __syncthreads();
  for (int i = 0; i < 2; ++i) {
    const int sb = i == 0 ? split_first : split_last;
    if (!merging[i]) continue;
    step_merge<DT, D, NW * 64, MQ>(p, sp, sb, hg, HPW * a.group, prefix(sb), prefix(sb + 1), scan);
    if (threadIdx.x == 0)   // ready for the next call
      __hip_atomic_store(&p.ws_count[int64_t(sb) * nhg + hg], uint64_t(0), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One wavefront per (sequence, query head): out = sum_p w_p o_p / sum_p w_p, w_p = e^(lse_p - M),
// partitions in order.  The loads are batched so that the chain of dependent round trips is
// short: the first 64 log-sum-exps load together with the length (lane i takes partition i), the
// maximum is a wave reduction, and then the partial rows of up to kBatch partitions load at once;
// the weights and the sums are the same sequential ones partition after partition.
template <int DT, int D>
__global__ __launch_bounds__(64) void merge_kernel(const MergeParams p) {
  constexpr int DPL = D / 64;   // dims per lane
  constexpr int kBatch = 16;    // partial rows in flight per lane
  const int lane = threadIdx.x;
  const int b = blockIdx.x / p.hq;   // row (sequence, or sequence x query token)
  const int h = blockIdx.x % p.hq;
  const int64_t prow = (int64_t(b) * p.hq + h) * p.max_partitions;
  const float* lse = p.partial_lse + prow;
  const float lse0 = lane < p.max_partitions ? lse[lane] : neg_inf();   // used below n only
  int L = p.context_lens[p.q_tokens > 1 ? b / p.q_tokens : b];
  if (p.q_tokens > 1 && L > 0 && L <= p.capacity) L = max(L - p.q_tokens + 1 + b % p.q_tokens, 0);
  const int64_t orow = (int64_t(b) * p.hq + h) * D;
  if (L <= 0 || L > p.capacity) {
    const float fill = L <= 0 ? 0.f : qnan();
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_elem<DT>(p.out, orow + lane * DPL + e, fill);
    if (p.lse_out && lane == 0) p.lse_out[int64_t(b) * p.hq + h] = L <= 0 ? neg_inf() : qnan();
    return;
  }
  const int n = (L + p.partition_tokens - 1) / p.partition_tokens;
  float M = lane < n ? lse0 : neg_inf();
  for (int i0 = 64; i0 < n; i0 += 64) M = fmaxf(M, i0 + lane < n ? lse[i0 + lane] : neg_inf());
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float wsum = 0.f;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int cnt = min(64, n - i0);
    const float lv = i0 == 0 ? lse0 : (lane < cnt ? lse[i0 + lane] : neg_inf());
    const float wl = lane < cnt ? fast_exp2((lv - M) * kLog2e) : 0.f;   // partition i0 + lane
    for (int j0 = 0; j0 < cnt; j0 += kBatch) {
      float v[kBatch][DPL];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {   // rows past the partitions repeat the last one
        const float* po = p.partial_out + (prow + i0 + min(j0 + u, cnt - 1)) * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) v[u][e] = po[e];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j0 + u >= cnt) break;
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j0 + u));
        wsum += w;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
      }
    }
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

// One workgroup per (source, destination) page pair: both pools' pages copied with 16-byte loads
// and stores.  Pairs naming a page outside the pool, or a page onto itself, are skipped.
__global__ __launch_bounds__(256) void copy_pages_kernel(const CopyPagesParams p) {
  const int src = p.pairs[2 * blockIdx.x], dst = p.pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= p.num_pages || dst < 0 || dst >= p.num_pages || src == dst) return;
  const int64_t s0 = int64_t(src) * p.page_bytes, d0 = int64_t(dst) * p.page_bytes;
  for (int64_t i = threadIdx.x; i < p.page_bytes / 16; i += blockDim.x) {
    const u32x4 k = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k_pool) + s0 + 16 * i);
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.v_pool) + s0 + 16 * i);
    *reinterpret_cast<u32x4*>(static_cast<char*>(p.k_pool) + d0 + 16 * i) = k;
    *reinterpret_cast<u32x4*>(static_cast<char*>(p.v_pool) + d0 + 16 * i) = v;
  }
}

// Zero `words` 16-byte words from `dst` (vector stores; used instead of a memset so that the
// clearing is an ordinary kernel node when a caller captures the stream).
__global__ __launch_bounds__(256) void zero_kernel(u32x4* dst, uint64_t words) {
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < words; i += uint64_t(gridDim.x) * 256)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
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

constexpr int kWaves = 8;

template <int DT, int D, int GP>
hipError_t launch_decode_t(const DecodeParams& p, bool partial, hipStream_t stream) {
  const int64_t units = int64_t(p.batch) * (p.hkv / p.heads_per_wg) *
                       (partial ? p.max_partitions - p.part_begin : 1);
  if (units <= 0) return hipSuccess;
  if (partial)
    hipLaunchKernelGGL((decode_kernel<DT, D, GP, kWaves, pipe_depth<DT, D>(), true>), dim3(unsigned(units)),
                       dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<DT, D, GP, kWaves, pipe_depth<DT, D>(), false>), dim3(unsigned(units)),
                       dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int DT, int D, int GP>
hipError_t launch_step_t(const StepParams& p, hipStream_t stream) {
  const int nhg = p.a.hkv / p.a.heads_per_wg;
  if (p.rope_cos) {
    hipLaunchKernelGGL((step_kernel<DT, D, GP, kWaves, pipe_depth<DT, D>(), true>), dim3(unsigned(p.groups * nhg)),
                       dim3(kWaves * 64), 0, stream, p);
    return hipGetLastError();
  }
  if (p.q_tokens > 1) {
    if constexpr (DT == DT_F32) {
      return hipErrorInvalidValue;   // the multi-query step takes 16-bit types only
    } else {
      hipLaunchKernelGGL((step_kernel<DT, D, GP, kWaves, pipe_depth<DT, D>(), false, true>),
                         dim3(unsigned(p.groups * nhg)), dim3(kWaves * 64), 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((step_kernel<DT, D, GP, kWaves, pipe_depth<DT, D>(), false>), dim3(unsigned(p.groups * nhg)),
                     dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

// Dispatch over (dtype, head_dim, padded group) to a templated launcher F<DT, D, GP>.
template <template <int, int, int> class F, class P>
hipError_t dispatch_shape(const P& p, int dtype, int head_dim, int gp, hipStream_t stream, bool flag) {
#define PKV_GP(DT, D)                                                      \
  switch (gp) {                                                            \
    case 4: return F<DT, D, 4>::run(p, stream, flag);                      \
    case 8: return F<DT, D, 8>::run(p, stream, flag);                      \
    case 16: return F<DT, D, 16>::run(p, stream, flag);                    \
    default: return hipErrorInvalidValue;                                  \
  }
#define PKV_D(DT)                                                          \
  switch (head_dim) {                                                      \
    case 64: PKV_GP(DT, 64)                                                \
    case 128: PKV_GP(DT, 128)                                              \
    default: return hipErrorInvalidValue;                                  \
  }
  switch (dtype) {
    case DT_F32: PKV_D(DT_F32)
    case DT_BF16: PKV_D(DT_BF16)
    case DT_F16: PKV_D(DT_F16)
    default: return hipErrorInvalidValue;
  }
#undef PKV_D
#undef PKV_GP
}

template <int DT, int D, int GP>
struct DecodeLaunch {
  static hipError_t run(const DecodeParams& p, hipStream_t s, bool partial) {
    return launch_decode_t<DT, D, GP>(p, partial, s);
  }
};

// The shared-prefix grid of cascade_kernel: the suffix partitions (decode_kernel's partial mode
// from d.part_begin), then the prefix partitions (prefix_kernel's grid), from a multiple of 8.
template <int DT, int D, int GP>
hipError_t launch_cascade_t(const DecodeParams& d, const PrefixParams& pp, hipStream_t stream) {
  constexpr int ROWS = PrefixGeo<D, kPrefixWaves, kPrefixRowBlocks>::ROWS;
  const int64_t n_dec = int64_t(d.batch) * (d.hkv / d.heads_per_wg) *
                        (d.max_partitions > d.part_begin ? d.max_partitions - d.part_begin : 0);
  const int64_t tiles = (int64_t(pp.batch) * pp.group + ROWS - 1) / ROWS;
  const int64_t n_pre = pp.prefix_tokens > 0 ? tiles * pp.hkv * (pp.prefix_tokens / pp.partition_tokens) : 0;
  const int64_t n_pre0 = n_pre > 0 ? (n_dec + 7) / 8 * 8 : n_dec;
  const int64_t total = n_pre0 + n_pre;
  if (total == 0) return hipSuccess;
  if (total > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((cascade_kernel<DT, D, GP, kWaves, pipe_depth<DT, D>()>), dim3(unsigned(total)),
                     dim3(kWaves * 64), 0, stream, d, pp, int(n_dec), int(n_pre0));
  return hipGetLastError();
}

struct CascadeArgs {
  const DecodeParams* d;
  const PrefixParams* pp;
};

template <int DT, int D, int GP>
struct CascadeLaunch {
  static hipError_t run(const CascadeArgs& a, hipStream_t s, bool) {
    if constexpr (DT == DT_F32) {
      return hipErrorInvalidValue;   // no prefix kernel for fp32
    } else {
      return launch_cascade_t<DT, D, GP>(*a.d, *a.pp, s);
    }
  }
};

template <int DT, int D, int GP>
struct StepLaunch {
  static hipError_t run(const StepParams& p, hipStream_t s, bool) { return launch_step_t<DT, D, GP>(p, s); }
};

template <int DT>
hipError_t launch_merge_dt(const MergeParams& p, int head_dim, hipStream_t stream) {
  const int64_t units = int64_t(p.batch) * (p.q_tokens > 1 ? p.q_tokens : 1) * p.hq;
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

int decode_waves() { return kWaves; }

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int group_pad,
                         bool partial, hipStream_t stream) {
  return dispatch_shape<DecodeLaunch>(p, dtype, head_dim, group_pad, stream, partial);
}

hipError_t launch_cascade(const DecodeParams& d, const PrefixParams& pp, int dtype, int head_dim,
                          int group_pad, hipStream_t stream) {
  if (d.batch == 0) return hipSuccess;
  return dispatch_shape<CascadeLaunch>(CascadeArgs{&d, &pp}, dtype, head_dim, group_pad, stream, false);
}

hipError_t launch_step(const StepParams& p, int dtype, int head_dim, int group_pad,
                       hipStream_t stream) {
  if (p.a.batch == 0) return hipSuccess;
  return dispatch_shape<StepLaunch>(p, dtype, head_dim, group_pad, stream, false);
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

hipError_t launch_copy_pages(const CopyPagesParams& p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_pages_kernel, dim3(unsigned(p.n)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_zero(void* dst, uint64_t bytes, hipStream_t stream) {
  const uint64_t words = bytes / 16;
  if (words == 0) return hipSuccess;
  const uint64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                     stream, static_cast<u32x4*>(dst), words);
  return hipGetLastError();
}

hipError_t launch_validate(const ValidateParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
