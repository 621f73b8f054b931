// HIP kernels of the verify pass for gfx950 (CDNA4).
//
// Pass structure per layer (rows = sequences x positions, typically 1 x 9):
//   k_gemm<QKV>    weight-streaming MFMA GEMM; epilogue: RMSNorm row scale, bias,
//                  RoPE, K/V append into the static cache at position len+slot
//   k_attn         split-KV causal GQA attention (MFMA) over position-aligned spans
//   k_combine      fixed-order merge of the span partials -> bf16 attention output
//   k_gemm<RESID>  O projection; epilogue: residual add, next RMSNorm's gain and
//                  sum-of-squares partials
//   k_gemm<SWIGLU> gate/up projection; epilogue: row scale, silu(gate)*up
//   k_gemm<RESID>  down projection (k split across workgroups, reduced in split order by the
//                  last workgroup to finish)
// then k_gemm<ARGMAX> (LM head with per-tile argmax) and k_accept (argmax merge,
// longest-prefix accept, commit).  The pass is captured once into a hipGraph.
#include "device.h"

#include <algorithm>
#include <cstdlib>

namespace sf {

#if SF_CHECKS
__device__ unsigned int g_checks = 0;
hipError_t read_checks(uint32_t* bits, bool clear) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(bits, HIP_SYMBOL(g_checks), sizeof(uint32_t));
  if (e == hipSuccess && clear) {
    const uint32_t zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_checks), &zero, sizeof(uint32_t));
  }
  return e;
}
#else
hipError_t read_checks(uint32_t* bits, bool) {
  *bits = 0;
  return hipErrorNotSupported;
}
#endif

// Squares of the residual block for the next norm's sums; one array per row count, shared by
// every epilogue instance of a kernel (they run one after another).
template <int kRealRows>
__device__ __forceinline__ float* resid_sq() {
  __shared__ float sq[32 * kRealRows];
  return sq;
}

// Epilogues of one 32-row n block for real rows r0 .. r0+kRealRows-1: val(nl, m) is output
// (n_local nl, local row m) before the row scale; rscale holds the folded RMSNorm's row scales.
// Called by every thread of the workgroup.
template <int EPI, int kRealRows, int kThreads, typename Val>
__device__ void gemm_epilogue(const GemmArgs& g, int nb, int r0, const float* rscale, Val val) {
  // Every product is rounded before it is added (no fused multiply-add): the epilogues are
  // instantiated in several kernels, and a sequence's result must not depend on which one ran
  // it, whatever the compiler would fuse in each.
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  if constexpr (EPI == kEpiQkv) {
    // Packed rows of n block nb: 0..15 = head dims i0..i0+15, 16..31 = their RoPE partners.
    const int half = g.dh >> 1, bph = g.dh >> 5;
    const int qb = g.nq * bph, kvb = g.nkv * bph;
    int sec, head, blk;
    if (nb < qb) { sec = 0; head = nb / bph; blk = nb - head * bph; }
    else if (nb < qb + kvb) { sec = 1; head = (nb - qb) / bph; blk = nb - qb - head * bph; }
    else { sec = 2; head = (nb - qb - kvb) / bph; blk = nb - qb - kvb - head * bph; }
    // Loads first (bias, length, RoPE table), stores after, as in the residual epilogue.
    constexpr int kIt = (16 * kRealRows + kThreads - 1) / kThreads;
    float y1v[kIt], y2v[kIt];
    float2 csv[kIt];
    int posv[kIt];
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
      const int it = tid + j * kThreads, p = it & 15, m = it >> 4, mr = r0 + m;
      posv[j] = -1;
      y1v[j] = y2v[j] = 0.f;
      csv[j] = make_float2(0.f, 0.f);
      if (it < 16 * kRealRows && mr < g.rows) {
        const int i = blk * 16 + p;
        const float s = rscale[m];
        y1v[j] = val(p, m) * s + g.bias[nb * 32 + p];
        y2v[j] = val(p + 16, m) * s + g.bias[nb * 32 + p + 16];
        const int b = mr / g.T, slot = mr - b * g.T;
        const int pos = g.len[b] + slot;
        check(pos < g.cap, kChkPos);
        posv[j] = pos;
        if (sec != 2 && pos < g.cap) csv[j] = g.rope[(size_t)pos * half + i];
      }
    }
#pragma unroll
    for (int j = 0; j < kIt; ++j) {
      const int it = tid + j * kThreads, p = it & 15, m = it >> 4, mr = r0 + m;
      const int pos = posv[j];
      if (pos < 0 || pos >= g.cap) continue;
      const int i = blk * 16 + p;
      const int b = mr / g.T;
      const float y1 = y1v[j], y2 = y2v[j];
      if (sec == 2) {
        uint16_t* dst = g.vc + (size_t)b * g.seq_stride + ((size_t)head * g.cap + pos) * g.dh;
        dst[i] = f2bf(y1);
        dst[i + half] = f2bf(y2);
      } else {
        const float2 cs = csv[j];
        const float o1 = y1 * cs.x - y2 * cs.y;
        const float o2 = y2 * cs.x + y1 * cs.y;
        if (sec == 0) {
          float* dst = g.q + ((size_t)mr * g.nq + head) * g.dh;
          dst[i] = o1;
          dst[i + half] = o2;
        } else {
          uint16_t* dst = g.kc + (size_t)b * g.seq_stride + ((size_t)head * g.cap + pos) * g.dh;
          dst[i] = f2bf(o1);
          dst[i + half] = f2bf(o2);
        }
      }
    }
  } else if constexpr (EPI == kEpiResid) {
    float* const sq = resid_sq<kRealRows>();
    // Every load of a thread's outputs (residual, result or split partials, gain) is issued
    // before its first store; stored one after another, each output waited one round trip.
    constexpr int kIt = (32 * kRealRows + kThreads - 1) / kThreads;
    float vin[kIt], gin[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int e = tid + i * kThreads, nl = e & 31, m = e >> 5, mr = r0 + m;
      vin[i] = gin[i] = 0.f;
      if (e < 32 * kRealRows && mr < g.rows) {
        const int n = nb * 32 + nl;
        vin[i] = g.x[(size_t)mr * g.n_out + n] + val(nl, m);
        gin[i] = g.gain_next[n];
      }
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int e = tid + i * kThreads, nl = e & 31, m = e >> 5, mr = r0 + m;
      if (e >= 32 * kRealRows) break;
      float v = 0.f;
      if (mr < g.rows) {
        const int n = nb * 32 + nl;
        const size_t o = (size_t)mr * g.n_out + n;
        v = vin[i];
        g.x[o] = v;
        store_split(g.a_next, g.rows, mr, n, v * gin[i]);
        if (g.hidden) g.hidden[o] = f2bf(v);
      }
      sq[e] = v * v;
    }
    __syncthreads();
    if (tid < kRealRows && r0 + tid < g.rows) {
      float s = 0.f;
#pragma unroll
      for (int nl = 0; nl < 32; ++nl) s += sq[tid * 32 + nl];
      g.ssq_out[(size_t)(r0 + tid) * g.nb + nb] = s;
    }
  } else if constexpr (EPI == kEpiSwiglu) {
    // Packed rows of n block nb: 0..15 = gate rows j0..j0+15, 16..31 = up rows j0..j0+15.
    for (int it = tid; it < 16 * kRealRows; it += kThreads) {
      const int p = it & 15, m = it >> 4, mr = r0 + m;
      if (mr >= g.rows) continue;
      const float s = rscale[m];
      const float gt = val(p, m) * s;
      const float up = val(p + 16, m) * s;
      const float hv = gt / (1.0f + expf(-gt)) * up;
      store_split(g.h, g.rows, mr, nb * 16 + p, hv);
    }
  } else if constexpr (EPI == kEpiArgmax) {
    const int m = tid, mr = r0 + m;
    if (m < kRealRows && mr < g.rows) {
      const float s = rscale[m];
      float best = -INFINITY;
      int bi = nb * 32;
      for (int nl = 0; nl < 32; ++nl) {
        const float v = val(nl, m) * s;
        check(v == v, kChkNaN);
        if (g.logits) g.logits[(size_t)mr * g.vocab + nb * 32 + nl] = v;
        if (v > best) { best = v; bi = nb * 32 + nl; }
      }
      g.amax[(size_t)mr * g.nb + nb] = make_float2(best, __int_as_float(bi));
    }
  }
}

// ----------------------------------------------------------------------------------------------
// Skinny GEMM: Y[m][n] = sum_k A[m][k] * W[n][k] for m < rows.  A has 2*rows rows (bf16 hi
// parts, then lo parts) and Y[m] = acc[m] + acc[rows + m]; 2*rows <= 32*MT.
// W is pre-packed in tiles of 32 rows x 16 k, one 16-byte fragment per lane in the operand
// order of v_mfma_f32_32x32x16_bf16, so one wave load of a tile reads one contiguous
// kilobyte.  A workgroup owns one 32-row n block; its NW waves split the k tiles.  Each wave
// keeps two 8-tile batches in flight (the next batch's weights and activations requested
// before the current batch's MFMAs) and the waves' accumulators are added in wave order,
// so results do not depend on scheduling.
//
// WIDE (more than 64 rows, batched verify): the rows are split into groups of 64; the
// workgroup of group rg holds two hi m tiles (operand rows 64rg .. 64rg+63) and two lo m tiles
// (rows + 64rg ..), so each weight tile feeds four MFMAs, and the groups of one block share
// the block's weights through L2 (see the index mapping below).  A row's arithmetic is the
// same as in the compact layout: the per-row result does not depend on the batch.
// GATED: the kernel of a gated pass (see gated_off); the check sits in separate instances
// because reading the flag at entry delays every kernel's first loads (7B verify +1.4%).
template <int EPI, int MT, int NW, int KH = kHalf, bool WIDE = false, bool GATED = false>
__global__ __launch_bounds__(NW * 64) void k_gemm(const GemmArgs g) {
  if constexpr (GATED)
    if (gated_off(g.gate)) return;
  static_assert(!WIDE || MT == 4, "wide row groups hold two hi and two lo m tiles");
  constexpr int kThreads = NW * 64;
  constexpr int kRealRows = MT * 16;
  __shared__ float tile[NW][MT * 1024];
  __shared__ float rscale[kRealRows + NW];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // WIDE: workgroup (block split bs, row group rg) has linear index ((bs/8)*G + rg)*8 + bs%8
  // (G row groups).  Workgroups go to the 8 XCDs round-robin by index, so the G row groups of
  // one block split run on the same XCD and are dispatched close together: the block's
  // weights come from HBM once and from that XCD's L2 for the other row groups.
  const int G = WIDE ? (g.rows + 63) / 64 : 1;
  int bs = blockIdx.x, rg = 0;
  if (WIDE) {
    const int q = blockIdx.x >> 3;
    rg = q % G;
    bs = (q / G) * 8 + (blockIdx.x & 7);
    if (bs >= g.nb * g.sp) return;   // padding of the last group of 8 block splits
  }
  const int nb = bs / g.sp, spi = bs - nb * g.sp;
  const int r0 = rg * 64;   // first real row of this workgroup
  const int U = g.sp * NW, u = spi * NW + wave;
  const int kt0 = (int)(((long)g.kb * u) / U), kt1 = (int)(((long)g.kb * (u + 1)) / U);

  constexpr bool kScaled = (EPI == kEpiQkv || EPI == kEpiSwiglu || EPI == kEpiArgmax);
  // Row scale of the folded RMSNorm.  Wave w owns rows w, w+NW, ...; lane l sums parts
  // l, l+64 in that order, then the wave reduces across lanes: the same order for a row
  // whatever the number of rows.  The loads are issued before the first weight batch and
  // summed right after it is requested, so they add no latency and hold no registers
  // during the weight stream.
  constexpr int kRowsPerWave = (kRealRows + NW - 1) / NW;
  float ssq_v[kRowsPerWave][kSsqPerLane];
  if constexpr (kScaled) {
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.ssq_in, (short)0, g.rows * g.nparts_in * 4, kBufferWord3);
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int mr = r0 + wave + NW * j;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) {
        const int p = lane + 64 * i;
        const int off = (mr < g.rows && p < g.nparts_in) ? (mr * g.nparts_in + p) * 4 : 0x7FFFFFF0;
        ssq_v[j][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0));
      }
    }
  }
  auto row_scales = [&]() {
    if constexpr (kScaled) {
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kSsqPerLane; ++i) t += ssq_v[j][i];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
        const int m = wave + NW * j;
        if (lane == 0 && m < kRealRows) rscale[m] = (r0 + m < g.rows) ? 1.0f / sqrtf(t / (float)g.k + g.eps) : 0.f;
      }
    }
  };

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x16){};

  // Raw buffer loads: the hardware range check returns zeros for tiles at or past kt1, and
  // for activation rows past 2*rows, without touching memory, so every batch issues all of
  // its loads unconditionally.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + (size_t)nb * g.kb * 64), (short)0, kt1 * 1024, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.a, (short)0, (int)act_bytes(2 * g.rows, g.k), kBufferWord3);
  const int ext_rows = 2 * g.rows;
  const int tsp = act_tile_pieces(ext_rows);
  const int a_lane = ((lane >> 5) * ext_rows + (lane & 31)) * 16;   // operand (k half, row) of tile 0, m tile 0
  // First operand row of m tile mt, and whether this lane's row of it is a real one.
  int mt_row0[MT];
  bool mt_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (WIDE) {
      mt_row0[mt] = (mt < 2) ? r0 + mt * 32 : g.rows + r0 + (mt - 2) * 32;
      mt_ok[mt] = r0 + (mt & 1) * 32 + (lane & 31) < g.rows;
    } else {
      mt_row0[mt] = mt * 32;
      mt_ok[mt] = mt * 32 + (lane & 31) < ext_rows;
    }
  }

  auto load = [&](int kt, u32x4 (&w)[KH], u32x4 (&a)[MT][KH]) {
#pragma unroll
    for (int t = 0; t < KH; ++t)
      w[t] = __builtin_amdgcn_raw_buffer_load_b128(wres, (kt + t) * 1024 + lane * 16, 0, kCacheStream);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int t = 0; t < KH; ++t) {
        const int off = (mt_ok[mt] && kt + t < kt1) ? a_lane + ((kt + t) * tsp + mt_row0[mt]) * 16 : 0x7FFFFFF0;
        a[mt][t] = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
      }
    }
  };
  auto mma = [&](const u32x4 (&w)[KH], const u32x4 (&a)[MT][KH]) {
#pragma unroll
    for (int t = 0; t < KH; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w[t]), as_bf16x8(a[mt][t]), acc[mt], 0, 0, 0);
  };
  {
    u32x4 w0[KH], w1[KH], a0[MT][KH], a1[MT][KH];
    load(kt0, w0, a0);
    __builtin_amdgcn_sched_barrier(0);
    row_scales();
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = kt0; kt < kt1; kt += 2 * KH) {
      load(kt + KH, w1, a1);
      __builtin_amdgcn_sched_barrier(0);
      mma(w0, a0);
      __builtin_amdgcn_sched_barrier(0);
      load(kt + 2 * KH, w0, a0);
      __builtin_amdgcn_sched_barrier(0);
      mma(w1, a1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Cross-wave sum in wave order: every wave stores its accumulators, then each thread adds
  // the NW images of its share of the outputs into wave 0's image.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) tile[wave][mt * 1024 + lane * 16 + r] = acc[mt][r];
  __syncthreads();
  for (int e = tid; e < MT * 1024; e += kThreads) {
    float v = tile[0][e];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += tile[w][e];
    tile[0][e] = v;
  }
  __syncthreads();
  const float* img = tile[0];

  // k split over g.sp workgroups per block: each stores its partial tile (agent-coherent,
  // so the others see it without a cache flush) and counts its arrival on the block's
  // counter; the one whose arrival brings the count to sp adds the partials in split order
  // and runs the epilogue.  That last arriver also puts the counter back to zero, so every
  // counter stays in [0, sp) and is zero between launches (no growth, no wrap).
  __shared__ int last_arrival;
  const bool split = g.sp > 1;
  float* const pblk = g.part + (size_t)nb * g.sp * g.rows * 32;   // [split][row][32]
  // hi + lo of output (n_local nl, local row m) from this workgroup's tile
  auto tval = [&](int nl, int m) {
    return WIDE ? img[tile_idx(nl, m)] + img[tile_idx(nl, 64 + m)]
                : img[tile_idx(nl, m)] + img[tile_idx(nl, g.rows + m)];
  };
  if (split) {
    for (int e = tid; e < 32 * kRealRows; e += kThreads) {
      const int nl = e & 31, m = e >> 5;
      if (r0 + m < g.rows) st<true>(pblk + ((size_t)spi * g.rows + r0 + m) * 32 + nl, tval(nl, m));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) last_arrival = split_arrive(g.counters + nb * G + rg, g.sp);
    __syncthreads();
    if (!last_arrival) return;
    asm volatile("" ::: "memory");
  }

  // ------------------------------------------------------------------ epilogues
  // Output (n_local, m) of real row m: hi-part row m plus lo-part row rows + m (or the sum of
  // the splits' partials).
  auto val = [&](int nl, int m) {
    if (!split) return tval(nl, m);
    float s = 0.f;
    for (int q = 0; q < g.sp; ++q) s += ld<true>(pblk + ((size_t)q * g.rows + r0 + m) * 32 + nl);
    return s;
  };
  gemm_epilogue<EPI, kRealRows, kThreads>(g, nb, r0, rscale, val);
}

// ----------------------------------------------------------------------------------------------
// NF4 skinny GEMM: Y[m][n] = sum_b scale[n][b] * sum_{k in block b} level[code[n][k]] * A[m][k]
// for m < rows <= 64, blocks of 64 inputs.  Packed weights, per 32-row block and 64-input
// block, 1088 bytes: 1 KB of codes (lane l: row l%32, inputs 8*(l/32) .. +8 of each of the
// four 16-input k tiles, one dword per tile holding the 8 codes two per byte, even input in
// the low nibble) then the 32 rows' scales as bf16.  A code byte indexes a 256-entry LDS
// table of bf16 level pairs, which is one dword of a v_mfma_f32_32x32x16_bf16 operand; the
// table is stored 32 times, copy c in bank c, and lane l reads copy l%32, so a wave's lookups
// never conflict.  The block's four k tiles run into a block accumulator with the activations
// as the A operand (so a lane's 16 outputs share its weight row and its block scale), and the
// total gains scale * block accumulator.
// Everything after the k loop (cross-wave sum in wave order, k split by last arrival,
// epilogues) is k_gemm's, with the accumulator image transposed.

// Position of output (n_local nl, operand row m) in the transposed accumulator image: lane
// nl + 32*((m%8)/4), register 4*((m%32)/8) + m%4 of m tile m/32.
__device__ __forceinline__ int tile_idx_t(int nl, int m) {
  const int ml = m & 31;
  return (m >> 5) * 1024 + ((nl & 31) + (((ml >> 2) & 1) << 5)) * 16 + ((ml >> 3) << 2) + (ml & 3);
}

// bf16 bits of level i, selected from immediates: no memory load, so filling the table does
// not wait behind the weight loads already in flight (loads complete in issue order).
__device__ __forceinline__ uint32_t nf4_bits(int i) {
  uint32_t w = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w = (i >> 1) == q ? ((uint32_t)kNf4Bits[2 * q] | ((uint32_t)kNf4Bits[2 * q + 1] << 16)) : w;
  return (w >> ((i & 1) * 16)) & 0xFFFFu;
}

// NR (1 or 2) consecutive 32-row blocks per workgroup share every activation load.
template <int EPI, int MT, int NW, int KB, int NR, bool GATED = false>
__global__ __launch_bounds__(NW * 64) void k_gemm_nf4(const GemmArgs g) {
  if constexpr (GATED)
    if (gated_off(g.gate)) return;
  constexpr int kThreads = NW * 64;
  constexpr int kRealRows = MT * 16;
  constexpr int kTab = 256 * 32, kImg = NR * MT * 1024;
  // The level-pair table (code byte -> bf16 pair, 32 bank-rotated copies) during the k loop,
  // then the waves' accumulator images.
  __shared__ uint32_t lds[kTab > NW * kImg ? kTab : NW * kImg];
  uint32_t* const tab = lds;
  float* const tile = (float*)lds;
  __shared__ float rscale[kRealRows + NW];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nb0 = (blockIdx.x / g.sp) * NR, spi = blockIdx.x % g.sp;
  const int nblk = g.kb / 4;                                   // 64-input blocks
  const int U = g.sp * NW, u = spi * NW + wave;
  const int b0 = (int)(((long)nblk * u) / U), b1 = (int)(((long)nblk * (u + 1)) / U);

  constexpr bool kScaled = (EPI == kEpiQkv || EPI == kEpiSwiglu || EPI == kEpiArgmax);
  constexpr int kRowsPerWave = (kRealRows + NW - 1) / NW;
  float ssq_v[kRowsPerWave][kSsqPerLane];
  if constexpr (kScaled) {
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.ssq_in, (short)0, g.rows * g.nparts_in * 4, kBufferWord3);
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int mr = wave + NW * j;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) {
        const int p = lane + 64 * i;
        const int off = (mr < g.rows && p < g.nparts_in) ? (mr * g.nparts_in + p) * 4 : 0x7FFFFFF0;
        ssq_v[j][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0));
      }
    }
  }
  auto row_scales = [&]() {
    if constexpr (kScaled) {
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kSsqPerLane; ++i) t += ssq_v[j][i];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
        const int m = wave + NW * j;
        if (lane == 0 && m < kRealRows) rscale[m] = (m < g.rows) ? 1.0f / sqrtf(t / (float)g.k + g.eps) : 0.f;
      }
    }
  };

  f32x16 acc[NR][MT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[r][mt] = (f32x16){};

  // Buffer range checks return zeros for blocks at or past b1 and for operand rows past
  // 2*rows, so every batch issues all of its loads.
  __amdgpu_buffer_rsrc_t wres[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r)
    wres[r] = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)g.w + (size_t)(nb0 + r) * nblk * kNf4BlockBytes), (short)0, b1 * kNf4BlockBytes,
        kBufferWord3);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.a, (short)0, (int)act_bytes(2 * g.rows, g.k), kBufferWord3);
  const int ext_rows = 2 * g.rows;
  const int tsp = act_tile_pieces(ext_rows);
  const int a_lane = ((lane >> 5) * ext_rows + (lane & 31)) * 16;
  bool mt_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) mt_ok[mt] = mt * 32 + (lane & 31) < ext_rows;

  struct Stage {
    u32x4 c[KB][NR];
    uint16_t s[KB][NR];
    u32x4 a[KB][MT][4];
  };
  auto load = [&](int b, Stage& st) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int bo = (b + i) * kNf4BlockBytes;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        st.c[i][r] = __builtin_amdgcn_raw_buffer_load_b128(wres[r], bo + lane * 16, 0, kCacheStream);
        st.s[i][r] = __builtin_amdgcn_raw_buffer_load_b16(wres[r], bo + 1024 + (lane & 31) * 2, 0, kCacheStream);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kt = (b + i) * 4 + t;
          const int off = (mt_ok[mt] && b + i < b1) ? a_lane + (kt * tsp + mt * 32) * 16 : 0x7FFFFFF0;
          st.a[i][mt][t] = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
        }
    }
  };
  const uint32_t tab_lane = (lane & 31) * 4;
  auto mma = [&](const Stage& st) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        f32x16 part[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) part[mt] = (f32x16){};
        const uint32_t cw[4] = {st.c[i][r].x, st.c[i][r].y, st.c[i][r].z, st.c[i][r].w};
        u32x4 wv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            d[j] = *(const uint32_t*)((const char*)tab + ((((cw[t] >> (8 * j)) & 0xFFu) << 7) | tab_lane));
          wv[t] = (u32x4){d[0], d[1], d[2], d[3]};
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 w = as_bf16x8(wv[t]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            part[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(st.a[i][mt][t]), w, part[mt], 0, 0, 0);
        }
        const float sc = __uint_as_float((uint32_t)st.s[i][r] << 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[r][mt][q] = fmaf(sc, part[mt][q], acc[r][mt][q]);
      }
    }
  };
  {
    Stage s0, s1;
    load(b0, s0);
    __builtin_amdgcn_sched_barrier(0);
    // Entry e (codes of an even and an odd input, low nibble first) -> their bf16 level pair;
    // thread t fills entry t's 32 copies starting at copy `lane`, so no store conflicts.
    for (int e = tid; e < 256; e += kThreads) {
      const uint32_t v = nf4_bits(e & 15) | (nf4_bits(e >> 4) << 16);
      for (int c = 0; c < 32; ++c) tab[e * 32 + ((c + lane) & 31)] = v;
    }
    row_scales();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    for (int b = b0; b < b1; b += 2 * KB) {
      load(b + KB, s1);
      __builtin_amdgcn_sched_barrier(0);
      mma(s0);
      __builtin_amdgcn_sched_barrier(0);
      load(b + 2 * KB, s0);
      __builtin_amdgcn_sched_barrier(0);
      mma(s1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __syncthreads();   // every wave is done with the table
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 16; ++q) tile[wave * kImg + (r * MT + mt) * 1024 + lane * 16 + q] = acc[r][mt][q];
  __syncthreads();
  for (int e = tid; e < kImg; e += kThreads) {
    float v = tile[e];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += tile[w * kImg + e];
    tile[e] = v;
  }
  __syncthreads();

  __shared__ int last_arrival;
  const bool split = g.sp > 1;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int nb = nb0 + r;
    const float* img = tile + r * MT * 1024;
    float* const pblk = g.part + (size_t)nb * g.sp * g.rows * 32;   // [split][row][32]
    auto tval = [&](int nl, int m) { return img[tile_idx_t(nl, m)] + img[tile_idx_t(nl, g.rows + m)]; };
    if (split) {
      for (int e = tid; e < 32 * kRealRows; e += kThreads) {
        const int nl = e & 31, m = e >> 5;
        if (m < g.rows) st<true>(pblk + ((size_t)spi * g.rows + m) * 32 + nl, tval(nl, m));
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) last_arrival = split_arrive(g.counters + nb, g.sp);
      __syncthreads();
      if (!last_arrival) continue;   // workgroup-uniform
      asm volatile("" ::: "memory");
    }
    auto val = [&](int nl, int m) {
      if (!split) return tval(nl, m);
      float s = 0.f;
      for (int q = 0; q < g.sp; ++q) s += ld<true>(pblk + ((size_t)q * g.rows + m) * 32 + nl);
      return s;
    };
    gemm_epilogue<EPI, kRealRows, kThreads>(g, nb, 0, rscale, val);
    __syncthreads();   // the next block's partial stores reuse nothing, but keep the epilogues apart
  }
}

template <int EPI, bool GATED>
static hipError_t gemm_nf4_mt(const GemmArgs& g, int mt, hipStream_t s) {
  const dim3 block(256);
  switch (mt) {
    case 1:
      // Two row blocks per workgroup halve the activation traffic, where that still leaves a
      // workgroup per CU (gate/up at the 14B shape: 864 blocks; 32.5 -> 25.4 us).
      if (g.nb % 2 == 0 && g.nb / 2 * g.sp >= 256)
        k_gemm_nf4<EPI, 1, 4, 1, 2, GATED><<<dim3(g.nb / 2 * g.sp), block, 0, s>>>(g);
      else
        k_gemm_nf4<EPI, 1, 4, 2, 1, GATED><<<dim3(g.nb * g.sp), block, 0, s>>>(g);
      break;
    case 2: k_gemm_nf4<EPI, 2, 4, 1, 1, GATED><<<dim3(g.nb * g.sp), block, 0, s>>>(g); break;
    default: k_gemm_nf4<EPI, 4, 4, 1, 1, GATED><<<dim3(g.nb * g.sp), block, 0, s>>>(g); break;
  }
  return hipGetLastError();
}

template <int EPI>
static hipError_t gemm_nf4(const GemmArgs& g, hipStream_t s) {
  if (g.rows < 1 || g.rows > 64 || g.kb % 4) return hipErrorInvalidValue;
  const int mt = (2 * g.rows + 31) / 32;
  if (g.gate) return gemm_nf4_mt<EPI, true>(g, mt, s);
  return gemm_nf4_mt<EPI, false>(g, mt, s);
}

hipError_t launch_gemm_nf4(int epi, const GemmArgs& g, hipStream_t s) {
  switch (epi) {
    case kEpiQkv: return gemm_nf4<kEpiQkv>(g, s);
    case kEpiResid: return gemm_nf4<kEpiResid>(g, s);
    case kEpiSwiglu: return gemm_nf4<kEpiSwiglu>(g, s);
  }
  return hipErrorInvalidValue;
}

// Pack NF4 projections: block (32-row block nb, 64-input block b) of 1088 bytes from row
// pointer tables (rows [0, N): codes, two per byte, even input in the low nibble; rows
// [N, 2N): bf16 scales per 64 inputs).  One thread per lane of a block; a lane's dword for k
// tile t is the 4 source bytes of its 8 inputs.
__global__ void k_pack_nf4(uint8_t* dst, const uint8_t* const* rowptr, int N, int nb, int nblk) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)nb * nblk * 64) return;
  const int lane = (int)(idx & 63);
  const size_t blk = idx >> 6;
  const int b = (int)(blk % nblk), n_blk = (int)(blk / nblk);
  const int row = n_blk * kTileN + (lane & 31);
  const uint8_t* codes = rowptr[row];
  uint32_t out[4];
  for (int t = 0; t < 4; ++t) {
    const int k0 = b * kNf4Block + t * 16 + (lane >> 5) * 8;
    uint32_t v = 0;
    for (int j = 0; j < 4; ++j) {
      v |= (uint32_t)codes[(k0 >> 1) + j] << (8 * j);   // codes of inputs k0+2j, k0+2j+1
    }
    out[t] = v;
  }
  uint8_t* d = dst + blk * kNf4BlockBytes;
  *(uint4*)(d + lane * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  if (lane < 32) ((uint16_t*)(d + 1024))[lane] = ((const uint16_t*)rowptr[N + row])[b];
}

hipError_t launch_pack_nf4(uint8_t* dst, const uint8_t* const* rowptr, int N, int nblk, hipStream_t s) {
  if (N % kTileN || nblk < 1) return hipErrorInvalidValue;
  const size_t total = (size_t)(N / kTileN) * nblk * 64;
  k_pack_nf4<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dst, rowptr, N, N / kTileN, nblk);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------------
// Batched GEMM (more than 64 rows).  The per-output arithmetic is k_gemm's: wave w of split spi
// accumulates k tiles [kb*u/U, kb*(u+1)/U) (u = 4*spi + w, U = 4*sp) in one MFMA chain per
// output tile, the waves' sums are added in wave order and the splits' in split order, so a
// row's result does not depend on the batch.  What changes is the work per wave: kBlocks 32-row
// weight blocks x four m tiles (hi and lo parts of 64 real rows), 4*kBlocks MFMAs per k tile
// against (kBlocks + 4) KB of operands, where the row-group mode of k_gemm does 4 MFMAs per
// 5 KB.  The accumulators and a ring of kStages k tiles of operands stay in registers, loaded
// kStages-1 tiles ahead of the MFMAs that use them.
// The launch covers G 64-row groups from row row0.
template <int EPI, int kStages, int kBlocks>
__device__ __forceinline__ void gemm_b_body(const GemmArgs& g, int row0, int G) {
  constexpr int NW = 4, kThreads = 256, kRealRows = 64, MT = 4;
  // Cross-wave images of one weight block: wave w's accumulator register r of m tile mt, lane l
  // at red[w][(mt*16 + r)*kRedPitch + l].  Consecutive lanes hit consecutive banks when the
  // images are written, and the odd pitch spreads the epilogue's reads over the banks.
  constexpr int kRedPitch = 65, kRedWave = MT * 16 * kRedPitch;
  __shared__ float red[NW * kRedWave];
  __shared__ float rscale[kRealRows + NW];
  __shared__ int last_arrival;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // Workgroup (group split gs, row group rg) has linear index ((gs/8)*G + rg)*8 + gs%8: the G
  // row groups of one group of weight blocks run on the same XCD (workgroups go to the XCDs
  // round-robin by index) and close together in time, so the weights come from HBM once.
  const int ngroups = g.nb / kBlocks;
  const int q = blockIdx.x >> 3;
  const int rg = q % G;
  const int gs = (q / G) * 8 + (blockIdx.x & 7);
  if (gs >= ngroups * g.sp) return;   // padding of the last group of 8
  const int bgrp = gs / g.sp, spi = gs - bgrp * g.sp;
  const int nb0 = bgrp * kBlocks, r0 = row0 + rg * 64;
  const int U = g.sp * NW, u = spi * NW + wave;
  const int kt0 = (int)(((long)g.kb * u) / U), kt1 = (int)(((long)g.kb * (u + 1)) / U);

  constexpr bool kScaled = (EPI == kEpiQkv || EPI == kEpiSwiglu || EPI == kEpiArgmax);
  constexpr int kRowsPerWave = kRealRows / NW;
  float ssq_v[kRowsPerWave][kSsqPerLane];
  if constexpr (kScaled) {
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.ssq_in, (short)0, g.rows * g.nparts_in * 4, kBufferWord3);
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int mr = r0 + wave + NW * j;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) {
        const int p = lane + 64 * i;
        const int off = (mr < g.rows && p < g.nparts_in) ? (mr * g.nparts_in + p) * 4 : 0x7FFFFFF0;
        ssq_v[j][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0));
      }
    }
  }

  __amdgpu_buffer_rsrc_t wres[kBlocks];
#pragma unroll
  for (int j = 0; j < kBlocks; ++j)
    wres[j] = __builtin_amdgcn_make_buffer_rsrc((void*)(g.w + (size_t)(nb0 + j) * g.kb * 64), (short)0, kt1 * 1024,
                                                kBufferWord3);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.a, (short)0, (int)act_bytes(2 * g.rows, g.k), kBufferWord3);
  const int ext_rows = 2 * g.rows;
  const int tsp = act_tile_pieces(ext_rows);
  const int a_lane = ((lane >> 5) * ext_rows + (lane & 31)) * 16;
  int mt_row0[MT];
  bool mt_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    mt_row0[mt] = (mt < 2 ? 0 : g.rows) + r0 + (mt & 1) * 32;
    mt_ok[mt] = r0 + (mt & 1) * 32 + (lane & 31) < g.rows;
  }
  // One k tile of operands: the four weight fragments, then the four operand fragments.
  // Lanes whose source is out of range (tiles at or past kt1, rows past the batch) read zeros.
  auto load = [&](int kt, u32x4 (&f)[kBlocks + MT]) {
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) f[j] = __builtin_amdgcn_raw_buffer_load_b128(wres[j], kt * 1024 + lane * 16, 0, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int off = (mt_ok[mt] && kt < kt1) ? a_lane + (kt * tsp + mt_row0[mt]) * 16 : 0x7FFFFFF0;
      f[kBlocks + mt] = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
    }
  };

  f32x16 acc[kBlocks][MT];
#pragma unroll
  for (int j = 0; j < kBlocks; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x16){};

  u32x4 ring[kStages][kBlocks + MT];
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) load(kt0 + i, ring[i]);
  if constexpr (kScaled) {
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) t += ssq_v[j][i];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
      const int m = wave + NW * j;
      if (lane == 0) rscale[m] = (r0 + m < g.rows) ? 1.0f / sqrtf(t / (float)g.k + g.eps) : 0.f;
    }
  }
  auto mma = [&](const u32x4 (&f)[kBlocks + MT]) {
#pragma unroll
    for (int j = 0; j < kBlocks; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[j][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(f[j]), as_bf16x8(f[kBlocks + mt]), acc[j][mt], 0,
                                                              0, 0);
  };
  // Unrolled by kStages so that every ring slot is a fixed set of registers.
  for (int kt = kt0; kt < kt1; kt += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      load(kt + s + kStages - 1, ring[(s + kStages - 1) % kStages]);
      if (kt + s < kt1) mma(ring[s]);
    }
  }
  __syncthreads();

  // Per weight block: the waves' images in LDS, summed in wave order into wave 0's.
  const bool split = g.sp > 1;
#pragma unroll
  for (int j = 0; j < kBlocks; ++j) {   // unrolled: acc[j] must stay in registers
    const int nb = nb0 + j;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave * kRedWave + (mt * 16 + r) * kRedPitch + lane] = acc[j][mt][r];
    __syncthreads();
    for (int e = tid; e < kRedWave; e += kThreads) {
      float v = red[e];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += red[w * kRedWave + e];
      red[e] = v;
    }
    __syncthreads();
    // Output (n_local nl, operand row e) in 32x32 MFMA output order: lane (e & 31) + 32*((nl&7)>>2),
    // register 4*(nl>>3) + (nl&3) of m tile e >> 5.
    auto at = [&](int nl, int e) {
      return red[((e >> 5) * 16 + ((nl >> 3) << 2) + (nl & 3)) * kRedPitch + (e & 31) + (((nl & 7) >> 2) << 5)];
    };
    auto tval = [&](int nl, int m) { return at(nl, m) + at(nl, 64 + m); };
    if (split) {
      float* const pblk = g.part + (size_t)nb * g.sp * g.rows * 32;
      for (int e = tid; e < 32 * kRealRows; e += kThreads) {
        const int nl = e & 31, m = e >> 5;
        if (r0 + m < g.rows) st<true>(pblk + ((size_t)spi * g.rows + r0 + m) * 32 + nl, tval(nl, m));
      }
    } else {
      gemm_epilogue<EPI, kRealRows, kThreads>(g, nb, r0, rscale, tval);
    }
    __syncthreads();
  }
  if (!split) return;
  // k split: as in k_gemm, the last of the sp workgroups of this group of blocks and row group
  // adds the partials in split order and runs the epilogues.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) last_arrival = split_arrive(g.counters + nb0 * ((g.rows + 63) / 64) + r0 / 64, g.sp);
  __syncthreads();
  if (!last_arrival) return;
  asm volatile("" ::: "memory");
  for (int j = 0; j < kBlocks; ++j) {
    const float* const pblk = g.part + (size_t)(nb0 + j) * g.sp * g.rows * 32;
    auto val = [&](int nl, int m) {
      float s = 0.f;
      for (int q2 = 0; q2 < g.sp; ++q2) s += ld<true>(pblk + ((size_t)q2 * g.rows + r0 + m) * 32 + nl);
      return s;
    };
    gemm_epilogue<EPI, kRealRows, kThreads>(g, nb0 + j, r0, rscale, val);
    __syncthreads();
  }
}

// Two weight blocks per wave keep each wave within 256 registers, so two workgroups share a CU
// and one's epilogue overlaps the other's k loop: 32-sequence verify 20.0 -> 18.1 ms and a
// 512-token prefill 27.0 -> 23.6 ms against four blocks per wave at one workgroup per CU.
template <int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_b(const GemmArgs g, int row0, int G) {
  gemm_b_body<EPI, 3, 2>(g, row0, G);
}

// ----------------------------------------------------------------------------------------------
// LDS-staged batched GEMM for passes of more than 64 rows: the residual projections whose k
// range is split (O and down; 4 blocks x 4 row tiles per workgroup) and the unsplit gate/up and
// LM head (8 blocks x 2 row tiles).  A workgroup of eight waves owns NBT 32-row weight blocks x RT
// 32-row row tiles of one k split, and wave w computes the two blocks of pair w % (NBT/2)
// against row tile w / (NBT/2) (its hi and lo m tiles: four MFMAs per k tile).  The NBT weight
// fragments and 2*RT activation fragments of every k tile go from memory straight into an LDS
// ring (buffer loads with an LDS destination: four stages of two k tiles, three loads per wave
// per stage), so one fetch of a weight fragment feeds 2*RT MFMAs and one of an activation
// fragment NBT, against four and two in the row-group kernel; the next k tile's fragments are
// read from LDS while the current tile's MFMAs run, and one barrier per stage both publishes a
// stage and frees the slot that is refilled next.
// Per output, the arithmetic is k_gemm's: split spi's k range is walked in the compact
// kernel's four wave chunks in turn, each chunk an MFMA chain from zero over its k tiles in
// order, and the chunk results are added in chunk order into a running sum (the first one
// copied), which is the compact kernel's chain-then-wave-order sum; hi and lo sums are then
// added, and the splits' partials are added in split order by the last arriver.  So a row's
// result is bitwise the one of a single-sequence pass.
constexpr int kTiledRing = 6144;   // u32x4 of the LDS ring: 96 KB
template <int EPI, int NBT, int RT>
__global__ __launch_bounds__(512, 1) void k_gemm_t(const GemmArgs g, int row0, int G) {
  static_assert(EPI == kEpiResid || EPI == kEpiSwiglu || EPI == kEpiArgmax, "no QKV epilogue here");
  constexpr bool kScaled = (EPI == kEpiSwiglu || EPI == kEpiArgmax);
  constexpr int NW = 8, kThreads = NW * 64, KT = 2, S = 4;
  constexpr int kPairs = NBT / 2, kRealRows = 32 * RT;
  static_assert(kPairs * RT == NW, "one wave per (block pair, row tile)");
  constexpr int kFr = NBT + 2 * RT;        // 1 KB fragments per k tile: weight blocks, then (row tile, hi/lo)
  constexpr int kLoads = KT * kFr / NW;    // LDS-destination loads per wave per stage
  static_assert(KT * kFr == kLoads * NW, "a stage's loads divide evenly over the waves");
  constexpr int kStage = KT * kFr * 64;    // u32x4 per stage
  constexpr int kImgPitch = 33;            // output image row pitch (floats)
  // After the k loop the ring holds the output image, the residual epilogue's squares and the
  // split arrival flag: the kernel has no other LDS array (a second one makes the compiler
  // wait for every LDS-destination load before each LDS read, serialising the ring).
  constexpr int kImgFloats = NBT * kRealRows * kImgPitch, kSqFloats = 32 * kRealRows;
  static_assert(kImgFloats + kSqFloats + kRealRows + 1 <= kTiledRing * 4, "image, squares, scales and flag fit");
  // Loads of stages s+2 .. s+3 may still be in flight when stage s+1 must have landed.
  constexpr int kAhead = kLoads * (S - 2);
  static_assert(kAhead < 16, "vmcnt immediate");
  static_assert(S * kStage <= kTiledRing, "ring size");
  // (sized by a constant, not by the template arguments: the LDS-destination load builtin
  // must not see a dependent type)
  __shared__ u32x4 ring[kTiledRing];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // Workgroup (group split gs, row group rg) has linear index ((gs/8)*G + rg)*8 + gs%8, as in
  // k_gemm_b: the row groups of one group of blocks share its weights through one XCD's L2.
  const int q = blockIdx.x >> 3;
  const int rg = q % G;
  const int gs = (q / G) * 8 + (blockIdx.x & 7);
  if (gs >= (g.nb / NBT) * g.sp) return;   // padding of the last group of 8
  const int nt = gs / g.sp, spi = gs - nt * g.sp;
  const int nb0 = nt * NBT, r0 = row0 + rg * kRealRows;
  const int pr = wave % kPairs, rt = wave / kPairs;
  const bool wave_rows = r0 + rt * 32 < g.rows;
  const int U = 4 * g.sp;
  auto bound = [&](int u) { return __builtin_amdgcn_readfirstlane((int)(((long)g.kb * u) / U)); };
  const int kt0 = bound(4 * spi), kt1 = bound(4 * spi + 4);
  const int ext = 2 * g.rows, tsp = act_tile_pieces(ext);

  // This wave's loads: entry e = wave*kLoads + p of a stage is k tile e / kFr, fragment
  // f = e % kFr (weight block nb0 + f, or activation row tile (f-NBT)/2, part (f-NBT)%2).  The
  // buffer range check returns zeros for weight tiles at or past kt1 and for rows past the
  // batch (their base offset lies past the activation buffer).
  __amdgpu_buffer_rsrc_t src[kLoads];
  int voff[kLoads], step[kLoads], ldst[kLoads], tof[kLoads];
#pragma unroll
  for (int p = 0; p < kLoads; ++p) {
    const int e = wave * kLoads + p, t = e / kFr, f = e - t * kFr;
    tof[p] = t;
    ldst[p] = (t * kFr + f) * 64;
    if (f < NBT) {
      src[p] = __builtin_amdgcn_make_buffer_rsrc((void*)(g.w + (size_t)(nb0 + f) * g.kb * 64), (short)0, kt1 * 1024,
                                                 kBufferWord3);
      voff[p] = lane * 16;
      step[p] = 1024;
    } else {
      const int rr = (f - NBT) >> 1, h = (f - NBT) & 1, row = r0 + rr * 32 + (lane & 31);
      src[p] = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)act_bytes(ext, g.k), kBufferWord3);
      voff[p] = row < g.rows ? ((lane >> 5) * ext + h * g.rows + row) * 16 : 0x40000000;
      step[p] = tsp * 16;
    }
  }
  auto issue = [&](int st_, int slot) {
#pragma unroll
    for (int p = 0; p < kLoads; ++p) {
      const int kt = kt0 + st_ * KT + tof[p];
      // (plain locals: the builtin rejects operands whose type depends on the template arguments)
      const __amdgpu_buffer_rsrc_t r = src[p];
      const int off = voff[p] + kt * step[p], dst = slot * kStage + ldst[p];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&ring[dst], 16, off, 0, 0, 0);
    }
  };
  // Own loads of the next stage landed, every wave's too, and every wave is done with the
  // slot refilled next (its LDS reads completed).
  auto wait_bar = [&]() {
    __builtin_amdgcn_s_waitcnt((kAhead & 15) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
  };
  auto rd = [&](int slot, int t, u32x4 (&f)[4]) {
    const u32x4* base = ring + slot * kStage + t * kFr * 64 + lane;
    f[0] = base[(2 * pr) * 64];
    f[1] = base[(2 * pr + 1) * 64];
    f[2] = base[(NBT + 2 * rt) * 64];
    f[3] = base[(NBT + 2 * rt + 1) * 64];
  };

  f32x16 acc[2][2], sum[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[j][h] = sum[j][h] = (f32x16){};
  int chunk = 0;
  int bnd = bound(4 * spi + 1);
  const int nst = (kt1 - kt0 + KT - 1) / KT;

#pragma unroll
  for (int st_ = 0; st_ < S - 1; ++st_) issue(st_, st_);
  // Row scale of the folded RMSNorm (gate/up, LM head), as k_gemm computes it: wave w owns rows
  // w, w+NW, ...; lane l sums parts l, l+64, l+128 in that order, then the wave reduces across
  // lanes.  Lane j keeps the scale of row w + NW*j until the ring is free after the k loop.  The
  // loads go out after the ring's first stages, so both latencies overlap.
  float my_scale = 0.f;
  if constexpr (kScaled) {
    constexpr int kRowsPerWave = kRealRows / NW;
    static_assert(kRowsPerWave <= 64, "one row per lane");
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.ssq_in, (short)0, g.rows * g.nparts_in * 4, kBufferWord3);
    float ssq_v[kRowsPerWave][kSsqPerLane];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int mr = r0 + wave + NW * j;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) {
        const int pp = lane + 64 * i;
        const int off = (mr < g.rows && pp < g.nparts_in) ? (mr * g.nparts_in + pp) * 4 : 0x7FFFFFF0;
        ssq_v[j][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0));
      }
    }
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int mr = r0 + wave + NW * j;
      float t2 = 0.f;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) t2 += ssq_v[j][i];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) t2 += __shfl_xor(t2, o);
      const float sc = (mr < g.rows) ? 1.0f / sqrtf(t2 / (float)g.k + g.eps) : 0.f;
      if (lane == j) my_scale = sc;
    }
  }
  wait_bar();
  u32x4 wf[2][4];
  rd(0, 0, wf[0]);
  for (int s0 = 0; s0 < nst; s0 += S) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int st_ = s0 + i;
      if (st_ < nst) {
        // Slot (i-1) % S was read by every wave before the last barrier: refill it.
        issue(st_ + S - 1, (i + S - 1) % S);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          const int kt = kt0 + st_ * KT + t;
          if (t + 1 < KT) {
            rd(i, t + 1, wf[(t + 1) & 1]);
          } else {
            wait_bar();
            rd((i + 1) % S, 0, wf[(t + 1) & 1]);
          }
          if (__builtin_expect(kt < kt1 && wave_rows, 1)) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              acc[j][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wf[t & 1][j]), as_bf16x8(wf[t & 1][2]),
                                                                  acc[j][0], 0, 0, 0);
              acc[j][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wf[t & 1][j]), as_bf16x8(wf[t & 1][3]),
                                                                  acc[j][1], 0, 0, 0);
            }
          }
          // End of a chunk (rare; kept out of the loop's straight-line path).
          if (__builtin_expect(kt + 1 == bnd, 0)) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                sum[j][h] = chunk == 0 ? acc[j][h] : sum[j][h] + acc[j][h];
                acc[j][h] = (f32x16){};
              }
            ++chunk;
            bnd = bound(4 * spi + chunk + 1);
          }
        }
      }
    }
  }
  // Every load has landed (the stages past the end included) and every wave is done reading
  // the ring before it becomes the output image.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* const img = reinterpret_cast<float*>(ring);
  float* const sq = img + kImgFloats;
  float* const rscale = sq + kSqFloats;
  int* const last_arrival = reinterpret_cast<int*>(rscale + kRealRows);
  if constexpr (kScaled)
    if (lane < kRealRows / NW) rscale[wave + NW * lane] = my_scale;
  if (wave_rows) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int nl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), m = rt * 32 + (lane & 31);
        img[((2 * pr + j) * kRealRows + m) * kImgPitch + nl] = sum[j][0][r] + sum[j][1][r];
      }
  }
  __syncthreads();
  if constexpr (EPI != kEpiResid) {
    // Unsplit (gate/up, LM head): the epilogues read the image.
    for (int nbl = 0; nbl < NBT; ++nbl) {
      auto val = [&](int nl, int m) { return img[(nbl * kRealRows + m) * kImgPitch + nl]; };
      gemm_epilogue<EPI, kRealRows, kThreads>(g, nb0 + nbl, r0, rscale, val);
      __syncthreads();
    }
    return;
  }
  // k split: every workgroup stores its partial tile; the last of the sp workgroups of this
  // group of blocks and row group adds the partials in split order and runs the residual
  // epilogue.
  for (int e = tid; e < NBT * 32 * kRealRows; e += kThreads) {
    const int nl = e & 31, m = (e >> 5) % kRealRows, nbl = e / (32 * kRealRows);
    if (r0 + m < g.rows)
      st<true>(g.part + (((size_t)(nb0 + nbl) * g.sp + spi) * g.rows + r0 + m) * 32 + nl,
               img[(nbl * kRealRows + m) * kImgPitch + nl]);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) *last_arrival = split_arrive(g.counters + nt * G + rg, g.sp);
  __syncthreads();
  if (!*last_arrival) return;
  asm volatile("" ::: "memory");
  // The residual epilogue of gemm_epilogue for all NBT blocks, with every load of a thread's
  // outputs (the splits' partials, the residual, the next norm's gain) issued before any of
  // its stores: the per-output form waits for one load round trip per output in turn.
  // Thread t owns outputs e = t + kThreads*i: column nl = e%32, row m = (e/32)%kRealRows of
  // block e/(32*kRealRows).
  {
#pragma clang fp contract(off)
  constexpr int kPer = NBT * 32 * kRealRows / kThreads;
  static_assert(kPer * kThreads == NBT * 32 * kRealRows && (32 * kRealRows) % kThreads == 0, "output split");
  float tot[kPer], xv[kPer], gn[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) tot[i] = 0.f;
  for (int q2 = 0; q2 < g.sp; ++q2) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + kThreads * i, nl = e & 31, m = (e >> 5) % kRealRows, nbl = e / (32 * kRealRows);
      const int mr = min(r0 + m, g.rows - 1);
      tot[i] += ld<true>(g.part + (((size_t)(nb0 + nbl) * g.sp + q2) * g.rows + mr) * 32 + nl);
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + kThreads * i, nl = e & 31, m = (e >> 5) % kRealRows, nbl = e / (32 * kRealRows);
    const int mr = min(r0 + m, g.rows - 1), n = (nb0 + nbl) * 32 + nl;
    xv[i] = g.x[(size_t)mr * g.n_out + n];
    gn[i] = g.gain_next[n];
  }
  constexpr int kPerBlock = 32 * kRealRows / kThreads;
#pragma unroll
  for (int nbl = 0; nbl < NBT; ++nbl) {
#pragma unroll
    for (int i = nbl * kPerBlock; i < (nbl + 1) * kPerBlock; ++i) {
      const int e = tid + kThreads * i, nl = e & 31, m = (e >> 5) % kRealRows, mr = r0 + m;
      float v = 0.f;
      if (mr < g.rows) {
        const int n = (nb0 + nbl) * 32 + nl;
        const size_t o = (size_t)mr * g.n_out + n;
        v = xv[i] + tot[i];
        g.x[o] = v;
        store_split(g.a_next, g.rows, mr, n, v * gn[i]);
        if (g.hidden) g.hidden[o] = f2bf(v);
      }
      sq[e - nbl * 32 * kRealRows] = v * v;
    }
    __syncthreads();
    if (tid < kRealRows && r0 + tid < g.rows) {
      float t2 = 0.f;
#pragma unroll
      for (int nl = 0; nl < 32; ++nl) t2 += sq[tid * 32 + nl];
      g.ssq_out[(size_t)(r0 + tid) * g.nb + nb0 + nbl] = t2;
    }
    __syncthreads();
  }
  }
}

// The LDS-staged kernel is the default for passes of more than 64 rows wherever it applies (the
// split O and down, the gate/up, the LM head); SF_TILED=0 selects the row-group kernel instead
// (the same results).
static bool tiled_enabled() {
  static const bool on = [] {
    const char* v = getenv("SF_TILED");
    return !(v && atoi(v) == 0);
  }();
  return on;
}

template <int EPI, int NW>
static hipError_t gemm_mt(const GemmArgs& g, hipStream_t s) {
  const int mt = (2 * g.rows + 31) / 32;
  const dim3 grid(g.nb * g.sp), block(NW * 64);
  if (g.rows > 64) {
    // A gated pass is a drafter step of one row per sequence (at most 64 rows), never here.
    if (g.gate) return hipErrorInvalidValue;
    const int G = (g.rows + 63) / 64;
    // Row groups before the one holding row_lo are skipped (their outputs are not needed).
    const int rg_lo = std::min(std::max(g.row_lo, 0), g.rows - 1) / 64;
    if (EPI == kEpiResid && g.sp > 1 && g.nb % 4 == 0 && g.kb >= 8 * g.sp && tiled_enabled()) {
      if constexpr (EPI == kEpiResid) {
        const int r0t = (rg_lo * 64 / 128) * 128, Gt = (g.rows - r0t + 127) / 128;
        const int ngs = (g.nb / 4) * g.sp;
        k_gemm_t<EPI, 4, 4><<<dim3(((ngs + 7) / 8) * 8 * Gt), dim3(512), 0, s>>>(g, r0t, Gt);
      }
    } else if ((EPI == kEpiSwiglu || EPI == kEpiArgmax) && g.sp == 1 && g.nb % 8 == 0 && g.kb >= 8 &&
               tiled_enabled()) {
      if constexpr (EPI == kEpiSwiglu || EPI == kEpiArgmax) {
        const int r0t = rg_lo * 64, Gt = G - rg_lo;
        const int ngs = g.nb / 8;
        k_gemm_t<EPI, 8, 2><<<dim3(((ngs + 7) / 8) * 8 * Gt), dim3(512), 0, s>>>(g, r0t, Gt);
      }
    } else if (g.nb % 2 == 0) {
      const int ngs = (g.nb / 2) * g.sp;
      k_gemm_b<EPI><<<dim3(((ngs + 7) / 8) * 8 * (G - rg_lo)), dim3(256), 0, s>>>(g, rg_lo * 64, G - rg_lo);
    } else {
      const int nbs = g.nb * g.sp;
      k_gemm<EPI, 4, 4, 4, true><<<dim3(((nbs + 7) / 8) * 8 * G), dim3(256), 0, s>>>(g);
    }
    return hipGetLastError();
  }
  switch (mt) {
    case 1:
      if (g.gate) k_gemm<EPI, 1, NW, 4, false, true><<<grid, block, 0, s>>>(g);
      else if (g.kh == 4) k_gemm<EPI, 1, NW, 4><<<grid, block, 0, s>>>(g);
      else k_gemm<EPI, 1, NW><<<grid, block, 0, s>>>(g);
      break;
    case 2:
      if (g.gate) k_gemm<EPI, 2, NW, kHalf, false, true><<<grid, block, 0, s>>>(g);
      else k_gemm<EPI, 2, NW><<<grid, block, 0, s>>>(g);
      break;
    case 3:
    case 4:
      if (g.gate) k_gemm<EPI, 4, NW, 4, false, true><<<grid, block, 0, s>>>(g);
      else k_gemm<EPI, 4, NW, 4><<<grid, block, 0, s>>>(g);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// More than two m tiles (prefill chunks) need the register file of 4-wave workgroups.
template <int EPI>
static hipError_t gemm_nw(const GemmArgs& g, hipStream_t s) {
  const bool wide = (2 * g.rows + 31) / 32 > 2;
  return (g.nw == 4 || wide) ? gemm_mt<EPI, 4>(g, s) : gemm_mt<EPI, 8>(g, s);
}

hipError_t launch_gemm(int epi, const GemmArgs& g, hipStream_t s) {
  switch (epi) {
    case kEpiQkv: return gemm_nw<kEpiQkv>(g, s);
    case kEpiResid: return gemm_nw<kEpiResid>(g, s);
    case kEpiSwiglu: return gemm_nw<kEpiSwiglu>(g, s);
    case kEpiArgmax: return gemm_nw<kEpiArgmax>(g, s);
  }
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------------------------
// Embedding: row r = (sequence b, slot i) takes [pending or stage.first, d_1..d_k, 0...][i],
// writes the fp32 residual, x * ln1 gain as hi/lo bf16 rows, and per-32-column sums of
// squares.  Thread t handles columns 8t..8t+7; four consecutive lanes form a 32-column block.
template <bool GATED>
__global__ __launch_bounds__(256) void k_embed(const EmbedArgs e) {
  if constexpr (GATED)
    if (gated_off(e.gate)) return;
  const int r = blockIdx.x;
  const int b = r / e.T, slot = r - b * e.T;
  int tok;
  if (slot == 0) {
    tok = (e.stage->flags & kFlagFirst) ? e.stage->first[b] : e.next[b];
  } else {
    const int j = slot - 1;
    tok = (j < e.stage->k[b]) ? e.stage->draft[b * e.kmax + j] : 0;
  }
  if (threadIdx.x == 0) check(tok >= 0 && tok < e.V, kChkToken);
  tok = min(max(tok, 0), e.V - 1);
  const uint16_t* src = e.embed + (size_t)tok * e.H;
  const int nparts = e.H >> 5;
  for (int c8 = threadIdx.x; c8 < (e.H >> 3); c8 += blockDim.x) {
    const u32x4 u = *(const u32x4*)(src + c8 * 8);
    const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = c8 * 8 + j;
      const float v = __uint_as_float(j & 1 ? (wds[j >> 1] & 0xFFFF0000u) : (wds[j >> 1] << 16));
      e.x[(size_t)r * e.H + col] = v;
      store_split(e.a, e.rows, r, col, v * e.gain[col]);
      s += v * v;
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if ((c8 & 3) == 0) e.ssq[(size_t)r * nparts + (c8 >> 2)] = s;
  }
}

hipError_t launch_embed(const EmbedArgs& e, hipStream_t s) {
  if (e.gate) k_embed<true><<<e.rows, 256, 0, s>>>(e);
  else k_embed<false><<<e.rows, 256, 0, s>>>(e);
  return hipGetLastError();
}

constexpr int kWarmMinLen = 4096;

// Workgroups [0, nx*nkv*B*ngroups): attention spans (span x, kv head, sequence x row group, in
// that order of the index); then a.warm.nwarm warm-up workgroups for the O projection, starting
// at an index that is a multiple of 8 (the ones before it, fewer than 8, exit).
template <int DH, bool GATED = false>
__global__ __launch_bounds__(256, 2) void k_attn(const AttnArgs a, int nx, int natt) {
  if constexpr (GATED)
    if (gated_off(a.gate)) return;
  const int bid = blockIdx.x;
  if (bid >= natt) {
    // The warm-up pays only when attention runs long enough to hide it (measured at the 7B
    // shape: attention plus warm-up 5.9 -> 8.3 us at context 512 for O 9.2 -> 7.1 us; at
    // context 8192 the 16 us of attention hide it): below kWarmMinLen positions it exits.
    const int q = bid - ((natt + 7) & ~7);
    if (q >= 0 && a.len[0] + a.T >= kWarmMinLen) warm_gemm(a.warm, q);
    return;
  }
  const int G = a.nq / a.nkv, ngroups = (a.T * G + 63) / 64;
  const int x = bid % nx, rest = bid / nx, kvh = rest % a.nkv, z = rest / a.nkv;
  attn_spans<DH, false>(a, x, nx, kvh, z / ngroups, z % ngroups);
}

template <int DH, bool GATED = false>
__global__ __launch_bounds__(256) void k_combine(const AttnArgs a) {
  if constexpr (GATED)
    if (gated_off(a.gate)) return;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.rows * a.nq) return;
  combine_pair<DH, false>(a, item / a.nq, item % a.nq);
}

hipError_t launch_attention(const AttnArgs& a, int dh, int B, hipStream_t s) {
  const int G = a.nq / a.nkv;
  const int ngroups = (a.T * G + 63) / 64;
  // One workgroup per span (workgroups past a sequence's length exit at once).  Capping the
  // grid so that workgroups take several spans each measured slower for the 32-sequence
  // batch (2048 workgroups: 21.2 ms per pass, 4096: 22.2, one per span: 20.8).  A span's
  // partial does not depend on the choice.
  const int nx = a.nchunk;
  const int natt = nx * a.nkv * B * ngroups;
  const int grid = a.warm.w ? ((natt + 7) & ~7) + a.warm.nwarm : natt;
  const int ncomb = (a.rows * a.nq + 3) / 4;
  if (dh == 128) {
    if (a.gate) {
      k_attn<128, true><<<grid, 256, 0, s>>>(a, nx, natt);
      k_combine<128, true><<<ncomb, 256, 0, s>>>(a);
    } else {
      k_attn<128><<<grid, 256, 0, s>>>(a, nx, natt);
      k_combine<128><<<ncomb, 256, 0, s>>>(a);
    }
  } else if (dh == 64) {
    if (a.gate) {
      k_attn<64, true><<<grid, 256, 0, s>>>(a, nx, natt);
      k_combine<64, true><<<ncomb, 256, 0, s>>>(a);
    } else {
      k_attn<64><<<grid, 256, 0, s>>>(a, nx, natt);
      k_combine<64><<<ncomb, 256, 0, s>>>(a);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int attention_spans(int cap) { return span_of(cap - 1) + 1; }

// ----------------------------------------------------------------------------------------------
// Accept: per sequence, merge the LM head's per-block (max, index) pairs into the greedy
// choice at each of the T positions (largest value, lowest index on ties; the merge is
// order independent), count the leading drafts that match, and commit.  Wave w merges the
// rows w, w+16, ... of the sequence.
template <bool GATED>
__global__ __launch_bounds__(1024) void k_accept(const AcceptArgs a) {
  if constexpr (GATED)
    if (gated_off(a.gate)) return;
  __shared__ int tgt[kMaxRows];   // one per slot: up to k_max+1 in a verify, a whole prefill chunk
  const int b = blockIdx.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // The merge is order independent, so the parts of a row may be split over waves: with S
  // slots to reduce, each gets max(1, 16/S) waves (all sixteen for a one-row drafter step),
  // each lane keeping sixteen loads in flight.
  __shared__ float red_v[16];
  __shared__ int red_i[16];
  const int nslots = a.T - a.slot_lo;
  const int wps = (a.has_head && nslots > 0 && nslots <= 16) ? 16 / nslots : 1;
  if (a.has_head) {
    for (int slot = tid; slot < a.slot_lo; slot += 1024) tgt[slot] = 0;
    for (int item = wave; item < nslots * wps; item += 16) {
      const int slot = a.slot_lo + item / wps, part = item % wps;
      const float2* row = a.amax + (size_t)(b * a.T + slot) * a.nparts;
      const int stride = 64 * wps;
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      // Batches of sixteen loads, the last one masked, so every batch is one round trip.
      for (int p = lane + 64 * part; p < a.nparts; p += 16 * stride) {
        float2 e[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          e[u] = (p + u * stride < a.nparts) ? row[p + u * stride] : make_float2(-INFINITY, __int_as_float(0x7FFFFFFF));
#pragma unroll
        for (int u = 0; u < 16; ++u) amax_merge(bv, bi, e[u].x, __float_as_int(e[u].y));
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax_merge(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
      if (wps == 1) {
        if (lane == 0) tgt[slot] = (bi == 0x7FFFFFFF) ? 0 : bi;
      } else if (lane == 0) {
        red_v[item] = bv;
        red_i[item] = bi;
      }
    }
    if (wps > 1) {
      __syncthreads();
      if (tid < nslots) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
        for (int q = 0; q < wps; ++q) amax_merge(bv, bi, red_v[tid * wps + q], red_i[tid * wps + q]);
        tgt[a.slot_lo + tid] = (bi == 0x7FFFFFFF) ? 0 : bi;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    Stage* st = a.stage;
    const int flags = st->flags;
    int k = st->k[b];
    check(k >= 0 && k <= a.T - 1, kChkK);
    k = min(max(k, 0), a.T - 1);
    int M = 0;
    if (a.has_head) {
      if (flags & kFlagForce) {
        M = k;
      } else {
        while (M < k && st->draft[b * st->kmax + M] == tgt[M]) ++M;
      }
      a.result[b] = M;
      for (int j = 0; j < a.T; ++j) a.result[a.B + b * a.T + j] = tgt[j];
      if (!(flags & kFlagNoCommit)) {
        check(a.cap == 0 || a.len[b] + M + 1 <= a.cap, kChkCommit);
        a.len[b] += M + 1;
        a.next[b] = tgt[M];
      }
      if (a.draft_out) {
        const int s = st->step[b];
        if (s < kMaxDraftSteps) a.draft_out[b * kMaxDraftSteps + s] = tgt[0];
        st->step[b] = s + 1;
      }
    } else {
      a.result[b] = 0;
      if (!(flags & kFlagNoCommit)) {
        check(a.cap == 0 || a.len[b] + k + 1 <= a.cap, kChkCommit);
        a.len[b] += k + 1;
      }
    }
  }
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t s) {
  if (a.T < 1 || a.T > kMaxRows) return hipErrorInvalidValue;
  if (a.gate) k_accept<true><<<a.B, 1024, 0, s>>>(a);
  else k_accept<false><<<a.B, 1024, 0, s>>>(a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------------
// Set-up and small state kernels.
__global__ void k_pack(uint4* dst, const uint16_t* const* rowptr, int nb, int kb) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)nb * kb * 64;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const size_t t = idx >> 6;
  const int kt = (int)(t % kb), n_blk = (int)(t / kb);
  const int row = n_blk * kTileN + (lane & 31);
  const int k0 = kt * kTileK + (lane >> 5) * 8;
  dst[idx] = *(const uint4*)(rowptr[row] + k0);
}

hipError_t launch_pack(uint4* dst, const uint16_t* const* rowptr, int nb, int kb, hipStream_t s) {
  const size_t total = (size_t)nb * kb * 64;
  k_pack<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dst, rowptr, nb, kb);
  return hipGetLastError();
}

__global__ void k_gather_f32(float* dst, const uint16_t* const* eltptr, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = eltptr[i] ? bf2f(*eltptr[i]) : 0.f;
}

hipError_t launch_gather_f32(float* dst, const uint16_t* const* eltptr, int n, hipStream_t s) {
  k_gather_f32<<<(n + 255) / 256, 256, 0, s>>>(dst, eltptr, n);
  return hipGetLastError();
}

// theta(p, i) = p * base^(-2i/dh) in double precision, stored as float (cos, sin).
__global__ void k_rope_table(float2* rope, int cap, int half, double base) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)cap * half) return;
  const int p = (int)(idx / half), i = (int)(idx - (size_t)p * half);
  const double inv_freq = pow(base, -2.0 * (double)i / (double)(2 * half));
  const double th = (double)p * inv_freq;
  rope[idx] = make_float2((float)cos(th), (float)sin(th));
}

hipError_t launch_rope_table(float2* rope, int cap, int half, double base, hipStream_t s) {
  const size_t total = (size_t)cap * half;
  k_rope_table<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(rope, cap, half, base);
  return hipGetLastError();
}

// which: bit 0 = set length, bit 1 = set pending token.
__global__ void k_set_state(int32_t* len, int32_t* next, int seq, int new_len, int new_next, int which) {
  if (threadIdx.x == 0) {
    if (which & 1) len[seq] = new_len;
    if (which & 2) next[seq] = new_next;
  }
}

hipError_t launch_set_state(int32_t* len, int32_t* next, int seq, int new_len, int new_next, int which,
                            hipStream_t s) {
  k_set_state<<<1, 64, 0, s>>>(len, next, seq, new_len, new_next, which);
  return hipGetLastError();
}

// Snapshot save (copy the live rows out, record length and pending token) or restore (copy
// the saved rows back at the saved length, then reinstate length and pending token).  One
// 16-byte unit of K and of V per thread and step; positions past the capacity are skipped.
__global__ __launch_bounds__(256) void k_snapshot(const SnapArgs a, int save) {
  const int units = a.dh / 8;
  const size_t total = (size_t)a.L * a.B * a.nkv * a.T * units;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    size_t t = idx / units;
    const int u = (int)(idx - t * units);
    const int slot = (int)(t % a.T);
    t /= a.T;
    const int h = (int)(t % a.nkv);
    t /= a.nkv;
    const int b = (int)(t % a.B);
    const int l = (int)(t / a.B);
    const int pos = (save ? a.len[b] : a.slen[b]) + slot;
    if (pos >= a.cap) continue;
    const size_t po = (size_t)l * a.layer_stride + (size_t)b * a.seq_stride + ((size_t)h * a.cap + pos) * a.dh + u * 8;
    const size_t so = ((((size_t)l * a.B + b) * a.nkv + h) * a.T + slot) * a.dh + u * 8;
    if (save) {
      *(uint4*)(a.sk + so) = *(const uint4*)(a.kpool + po);
      *(uint4*)(a.sv + so) = *(const uint4*)(a.vpool + po);
    } else {
      *(uint4*)(a.kpool + po) = *(const uint4*)(a.sk + so);
      *(uint4*)(a.vpool + po) = *(const uint4*)(a.sv + so);
    }
  }
  if (blockIdx.x == 0)
    for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
      if (save) {
        a.slen[b] = a.len[b];
        a.snext[b] = a.next[b];
      } else {
        a.len[b] = a.slen[b];
        a.next[b] = a.snext[b];
      }
    }
}

hipError_t launch_snapshot(const SnapArgs& a, int save, hipStream_t s) {
  if (a.L < 1 || a.B < 1 || a.nkv < 1 || a.T < 1 || a.dh % 8) return hipErrorInvalidValue;
  const size_t units = (size_t)a.L * a.B * a.nkv * a.T * (a.dh / 8);
  const int grid = (int)std::min<size_t>((units + 255) / 256, 1024);
  k_snapshot<<<grid, 256, 0, s>>>(a, save);
  return hipGetLastError();
}

// Zero n ints (a fill kernel, so that callers may capture it in a graph).
__global__ void k_zero(int* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_zero(int* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 1024);
  k_zero<<<grid, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

// Device-resident drafts -> fixed staging block (draft [B][kmax], k [B] or all kmax).
__global__ void k_stage_device(Stage* st, const int32_t* draft, const int32_t* k, int B, int kmax, int flags) {
  const int t = threadIdx.x;
  if (t == 0) { st->flags = flags; st->kmax = kmax; }
  for (int i = t; i < B; i += blockDim.x) {
    st->k[i] = k ? k[i] : kmax;
    st->step[i] = 0;
  }
  for (int i = t; i < B * kmax; i += blockDim.x) st->draft[i] = draft[i];
}

// ----------------------------------------------------------------------------------------------
// Round bookkeeping ([ShardFlow] "Speculative Decoding: The Idea": the drafter guesses k tokens,
// the verifier checks them in one pass and the agreed prefix is committed; the drafter is then
// rewound in place to the committed stream, "Why It Kept Breaking", fix 4).  Thread b owns
// sequence b.
//   begin:     remember the verifier's length; the drafter commits each step; the verifier
//              takes k drafts.
//   stage:     the drafter's k step outputs become the verifier's drafts.
//   reconcile: with M accepted and L the old length: M < k: the drafter's K/V of positions
//              L .. L+M is right, so its length becomes L+M+1 and its pending token the
//              verifier's target[M].  M = k: its last draft d_k was never fed to it, so the
//              next (non-committing) step feeds d_k at L+k and finish counts it.
//   finish:    the drafter's length takes the catch-up step; its pending token is the
//              verifier's.
__global__ void k_round(const RoundArgs a, int phase) {
  const int b = threadIdx.x;
  if (phase == kRoundBegin) {
    if (b == 0) {
      a.dstage->flags = 0;
      a.dstage->kmax = 0;
      a.vstage->flags = 0;
      a.vstage->kmax = a.vkmax;
    }
    if (b < a.B) {
      a.scratch[b] = a.vlen[b];
      a.dstage->k[b] = 0;
      a.dstage->step[b] = 0;
      a.vstage->k[b] = a.k;
    }
  } else if (phase == kRoundStage) {
    if (b < a.B)
      for (int j = 0; j < a.vkmax; ++j) a.vstage->draft[b * a.vkmax + j] = (j < a.k) ? a.dout[b * kMaxDraftSteps + j] : 0;
  } else if (phase == kRoundReconcile) {
    if (b == 0) a.dstage->flags = kFlagNoCommit;
    if (b < a.B) {
      const int M = a.vres[b], L = a.scratch[b];
      if (M < a.k) {
        a.dlen[b] = L + M + 1;
        a.dnext[b] = a.vres[a.B + b * a.vT + M];
        a.scratch[a.B + b] = 0;
      } else {
        a.scratch[a.B + b] = 1;
      }
    }
    __syncthreads();
    if (b == 0) {   // the catch-up pass runs only if some sequence needs it
      int any = 0;
      for (int i = 0; i < a.B; ++i) any |= a.scratch[a.B + i];
      a.scratch[2 * a.B] = any;
    }
  } else {
    if (b == 0) a.dstage->flags = 0;
    if (b < a.B) {
      a.dlen[b] += a.scratch[a.B + b];
      a.dnext[b] = a.vnext[b];
    }
  }
}

hipError_t launch_round(const RoundArgs& r, int phase, hipStream_t s) {
  if (r.B < 1 || r.B > kMaxSeqs || r.k < 1 || r.k > r.vkmax || r.vkmax >= kMaxK || r.k >= kMaxDraftSteps)
    return hipErrorInvalidValue;
  k_round<<<1, kMaxSeqs, 0, s>>>(r, phase);
  return hipGetLastError();
}

hipError_t launch_stage_device(Stage* stage, const int32_t* draft, const int32_t* k, int B, int kmax,
                               int flags, hipStream_t s) {
  k_stage_device<<<1, 256, 0, s>>>(stage, draft, k, B, kmax, flags);
  return hipGetLastError();
}

// Copy positions [0, n_pos) of one sequence between the pool (layer stride given, kv heads
// at stride cap*dh) and a dense [layers][nkv][src_positions][dh] buffer.
__global__ void k_copy_kv(uint16_t* pool, uint16_t* src, long pool_layer_stride, int nkv, int cap,
                          int dh, int n_layers, int n_pos, int src_positions, int to_pool) {
  const size_t units_per_row = dh / 8;
  const size_t total = (size_t)n_layers * nkv * n_pos * units_per_row;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t u = idx % units_per_row;
    size_t t = idx / units_per_row;
    const int pos = (int)(t % n_pos);
    t /= n_pos;
    const int h = (int)(t % nkv);
    const int l = (int)(t / nkv);
    uint4* pp = (uint4*)(pool + (size_t)l * pool_layer_stride + ((size_t)h * cap + pos) * dh) + u;
    uint4* sp = (uint4*)(src + (((size_t)l * nkv + h) * src_positions + pos) * dh) + u;
    if (to_pool) *pp = *sp; else *sp = *pp;
  }
}

hipError_t launch_copy_kv(uint16_t* pool, uint16_t* src, long pool_layer_stride, int nkv, int cap,
                          int dh, int n_layers, int n_pos, int src_positions, int to_pool, hipStream_t s) {
  k_copy_kv<<<2048, 256, 0, s>>>(pool, src, pool_layer_stride, nkv, cap, dh, n_layers, n_pos, src_positions,
                                 to_pool);
  return hipGetLastError();
}

}  // namespace sf
