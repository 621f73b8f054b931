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
//   k_gemm<RESID>  down projection (split-K across workgroups, deterministic)
// then k_gemm<ARGMAX> (LM head with per-tile argmax) and k_accept (argmax merge,
// longest-prefix accept, commit).  The pass is captured once into a hipGraph.
#include "sf_internal.h"

#include <math.h>

namespace sf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even (inputs are finite or inf; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Activations feeding an MFMA are carried as two bf16 values, hi = bf16(v) and
// lo = bf16(v - hi) (about 16 significant bits), stored as rows r and rows + r of the
// operand matrix; the weights are bf16 and the products accumulate in fp32.
__device__ __forceinline__ void store_split(uint16_t* base, size_t row_stride, int rows, int r, int col, float v) {
  const uint16_t hi = f2bf(v);
  base[(size_t)r * row_stride + col] = hi;
  base[(size_t)(rows + r) * row_stride + col] = f2bf(v - bf2f(hi));
}

// Word 3 of a raw buffer resource on gfx9-family GPUs (gfx950 included).
constexpr int kBufferWord3 = 0x00020000;
// RMSNorm sum-of-squares partials (one per 32 columns) read per lane: hidden <= 64*32*2.
constexpr int kSsqPerLane = 2;
// Weight tiles per pipelined half-batch.
constexpr int kHalf = 8;
// Cache policy of the weight stream: non-temporal (each weight byte is read once per pass).
constexpr int kCacheStream = 2;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Element (n_local, m) of a 32 x (32*MT) accumulator tile kept in 32x32 MFMA output order:
// lane l, register r of m-tile mt holds n_local = 8*(r/4) + 4*(l/32) + r%4, m = mt*32 + l%32.
__device__ __forceinline__ int tile_idx(int nl, int m) {
  const int lane = (m & 31) + (((nl & 7) >> 2) << 5);
  const int r = ((nl >> 3) << 2) + (nl & 3);
  return (m >> 5) * 1024 + lane * 16 + r;
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
template <int EPI, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void k_gemm(const GemmArgs g) {
  constexpr int kThreads = NW * 64;
  constexpr int kRealRows = MT * 16;
  __shared__ float tile[MT * 1024];
  __shared__ float rscale[kRealRows + NW];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nb = blockIdx.x / g.sp, spi = blockIdx.x - nb * g.sp;
  const int U = g.sp * NW, u = spi * NW + wave;
  const int kt0 = (int)(((long)g.kb * u) / U), kt1 = (int)(((long)g.kb * (u + 1)) / U);

  constexpr bool kScaled = (EPI == kEpiQkv || EPI == kEpiSwiglu || EPI == kEpiArgmax);
  // Row scale of the folded RMSNorm.  Wave w owns rows w, w+NW, ...; lane l sums parts
  // l, l+64 in that order, then the wave reduces across lanes: the same order for a row
  // whatever the number of rows.  The loads are issued here and summed after the weight
  // stream, so they never delay it.
  constexpr int kRowsPerWave = (kRealRows + NW - 1) / NW;
  float ssq_v[kRowsPerWave][kSsqPerLane];
  if constexpr (kScaled) {
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.ssq_in, (short)0, g.rows * g.nparts_in * 4, kBufferWord3);
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int m = wave + NW * j;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) {
        const int p = lane + 64 * i;
        const int off = (m < g.rows && p < g.nparts_in) ? (m * g.nparts_in + p) * 4 : 0x7FFFFFF0;
        ssq_v[j][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0));
      }
    }
  }

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x16){};

  // Raw buffer loads: the hardware range check returns zeros for tiles at or past kt1, and
  // for activation rows past 2*rows, without touching memory, so every batch issues all of
  // its loads unconditionally.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + (size_t)nb * g.kb * 64), (short)0, kt1 * 1024, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.a, (short)0, 2 * kMaxRows * g.k * 2, kBufferWord3);
  const int ext_rows = 2 * g.rows;
  const int a_lane = ((lane & 31) * g.k + (lane >> 5) * 8) * 2;

  auto load = [&](int kt, u32x4 (&w)[kHalf], u32x4 (&a)[MT][kHalf]) {
#pragma unroll
    for (int t = 0; t < kHalf; ++t)
      w[t] = __builtin_amdgcn_raw_buffer_load_b128(wres, (kt + t) * 1024 + lane * 16, 0, kCacheStream);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bool row_ok = mt * 32 + (lane & 31) < ext_rows;
#pragma unroll
      for (int t = 0; t < kHalf; ++t) {
        const int off = (row_ok && kt + t < kt1) ? a_lane + (mt * 32 * g.k + (kt + t) * kTileK) * 2 : 0x7FFFFFF0;
        a[mt][t] = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
      }
    }
  };
  auto mma = [&](const u32x4 (&w)[kHalf], const u32x4 (&a)[MT][kHalf]) {
#pragma unroll
    for (int t = 0; t < kHalf; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w[t]), as_bf16x8(a[mt][t]), acc[mt], 0, 0, 0);
  };
  {
    u32x4 w0[kHalf], w1[kHalf], a0[MT][kHalf], a1[MT][kHalf];
    load(kt0, w0, a0);
    for (int kt = kt0; kt < kt1; kt += 2 * kHalf) {
      load(kt + kHalf, w1, a1);
      __builtin_amdgcn_sched_barrier(0);
      mma(w0, a0);
      __builtin_amdgcn_sched_barrier(0);
      load(kt + 2 * kHalf, w0, a0);
      __builtin_amdgcn_sched_barrier(0);
      mma(w1, a1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

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
  // Cross-wave sum in wave order.
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* t = &tile[mt * 1024 + lane * 16 + r];
          *t = (w == 0) ? acc[mt][r] : *t + acc[mt][r];
        }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogues
  // Output (n_local, m) of real row m: hi-part row m plus lo-part row rows + m.
  auto val = [&](int nl, int m) { return tile[tile_idx(nl, m)] + tile[tile_idx(nl, g.rows + m)]; };
  if constexpr (EPI == kEpiQkv) {
    // Packed rows of n block nb: 0..15 = head dims i0..i0+15, 16..31 = their RoPE partners.
    for (int it = tid; it < 16 * kRealRows; it += kThreads) {
      const int p = it & 15, m = it >> 4;
      if (m >= g.rows) continue;
      const int half = g.dh >> 1, bph = g.dh >> 5;
      const int qb = g.nq * bph, kvb = g.nkv * bph;
      int sec, head, blk;
      if (nb < qb) { sec = 0; head = nb / bph; blk = nb - head * bph; }
      else if (nb < qb + kvb) { sec = 1; head = (nb - qb) / bph; blk = nb - qb - head * bph; }
      else { sec = 2; head = (nb - qb - kvb) / bph; blk = nb - qb - kvb - head * bph; }
      const int i = blk * 16 + p;
      const float s = rscale[m];
      const float y1 = val(p, m) * s + g.bias[nb * 32 + p];
      const float y2 = val(p + 16, m) * s + g.bias[nb * 32 + p + 16];
      const int b = m / g.T, slot = m - b * g.T;
      const int pos = g.len[b] + slot;
      if (pos < g.cap) {
        if (sec == 2) {
          uint16_t* dst = g.vc + (size_t)b * g.seq_stride + ((size_t)head * g.cap + pos) * g.dh;
          dst[i] = f2bf(y1);
          dst[i + half] = f2bf(y2);
        } else {
          const float2 cs = g.rope[(size_t)pos * half + i];
          const float o1 = y1 * cs.x - y2 * cs.y;
          const float o2 = y2 * cs.x + y1 * cs.y;
          if (sec == 0) {
            float* dst = g.q + ((size_t)m * g.nq + head) * g.dh;
            dst[i] = o1;
            dst[i + half] = o2;
          } else {
            uint16_t* dst = g.kc + (size_t)b * g.seq_stride + ((size_t)head * g.cap + pos) * g.dh;
            dst[i] = f2bf(o1);
            dst[i + half] = f2bf(o2);
          }
        }
      }
    }
  } else if constexpr (EPI == kEpiResid) {
    __shared__ float sq[32 * kRealRows];
    for (int e = tid; e < 32 * kRealRows; e += kThreads) {
      const int nl = e & 31, m = e >> 5;
      float v = 0.f;
      if (m < g.rows) {
        const int n = nb * 32 + nl;
        const size_t o = (size_t)m * g.n_out + n;
        v = g.x[o] + val(nl, m);
        g.x[o] = v;
        store_split(g.a_next, g.n_out, g.rows, m, n, v * g.gain_next[n]);
        if (g.hidden) g.hidden[o] = f2bf(v);
      }
      sq[e] = v * v;
    }
    __syncthreads();
    if (tid < kRealRows && tid < g.rows) {
      float s = 0.f;
#pragma unroll
      for (int nl = 0; nl < 32; ++nl) s += sq[tid * 32 + nl];
      g.ssq_out[(size_t)tid * g.nb + nb] = s;
    }
  } else if constexpr (EPI == kEpiSwiglu) {
    // Packed rows of n block nb: 0..15 = gate rows j0..j0+15, 16..31 = up rows j0..j0+15.
    for (int it = tid; it < 16 * kRealRows; it += kThreads) {
      const int p = it & 15, m = it >> 4;
      if (m >= g.rows) continue;
      const float s = rscale[m];
      const float gt = val(p, m) * s;
      const float up = val(p + 16, m) * s;
      const float hv = gt / (1.0f + expf(-gt)) * up;
      store_split(g.h, g.ffn, g.rows, m, nb * 16 + p, hv);
    }
  } else if constexpr (EPI == kEpiPartial) {
    // Unscaled partial sums of this workgroup's k range: part[spi][m][n].
    float* dst = g.part + (size_t)spi * g.rows * g.n_out;
    for (int e = tid; e < 32 * kRealRows; e += kThreads) {
      const int nl = e & 31, m = e >> 5;
      if (m < g.rows) dst[(size_t)m * g.n_out + nb * 32 + nl] = val(nl, m);
    }
  } else if constexpr (EPI == kEpiArgmax) {
    const int m = tid;
    if (m < g.rows && m < kRealRows) {
      const float s = rscale[m];
      float best = -INFINITY;
      int bi = nb * 32;
      for (int nl = 0; nl < 32; ++nl) {
        const float v = val(nl, m) * s;
        if (g.logits) g.logits[(size_t)m * g.vocab + nb * 32 + nl] = v;
        if (v > best) { best = v; bi = nb * 32 + nl; }
      }
      g.amax[(size_t)m * g.nb + nb] = make_float2(best, __int_as_float(bi));
    }
  }
}

template <int EPI, int NW>
static hipError_t gemm_mt(const GemmArgs& g, hipStream_t s) {
  const int mt = (2 * g.rows + 31) / 32;
  const dim3 grid(g.nb * g.sp), block(NW * 64);
  switch (mt) {
    case 1: k_gemm<EPI, 1, NW><<<grid, block, 0, s>>>(g); break;
    case 2: k_gemm<EPI, 2, NW><<<grid, block, 0, s>>>(g); break;
    case 3:
    case 4: k_gemm<EPI, 4, NW><<<grid, block, 0, s>>>(g); break;
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
    case kEpiPartial: return gemm_nw<kEpiPartial>(g, s);
  }
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------------------------
// Reductions of split-K partials, in split order, fused with the epilogue the undivided
// GEMM would have run.
constexpr int kMaxSplit = 8;

// Row scale 1/sqrt(mean(x^2) + eps) from the per-32-column sums of squares, summed in the
// same order as the GEMM prologue: lane l takes parts l, l+64, then a cross-lane tree.
__device__ float row_scale(const float* ssq, int nparts, int k, float eps, int m, int lane) {
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kSsqPerLane; ++i) {
    const int p = lane + 64 * i;
    t += (p < nparts) ? ssq[(size_t)m * nparts + p] : 0.f;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
  return 1.0f / sqrtf(t / (float)k + eps);
}

// QKV: workgroup (row m, 512 output pairs).  Item (n block, pair p): rows p and p+16 of the
// packed block are a RoPE pair (or two plain V dims).
__global__ __launch_bounds__(256) void k_reduce_qkv(const GemmArgs g) {
  __shared__ float sc;
  const int m = blockIdx.y;
  if (threadIdx.x < 64) {
    const float v = row_scale(g.ssq_in, g.nparts_in, g.k, g.eps, m, threadIdx.x);
    if (threadIdx.x == 0) sc = v;
  }
  __syncthreads();
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= g.nb * 16) return;
  const int nb = item >> 4, p = item & 15;
  const int n1 = nb * 32 + p, n2 = n1 + 16;
  // Partials of up to kMaxSplit splits, all loads issued before the (ordered) sum.
  float p1[kMaxSplit], p2[kMaxSplit];
#pragma unroll
  for (int q = 0; q < kMaxSplit; ++q) {
    const float* pq = g.part + ((size_t)min(q, g.sp - 1) * g.rows + m) * g.n_out;
    p1[q] = pq[n1];
    p2[q] = pq[n2];
  }
  float a1 = 0.f, a2 = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxSplit; ++q)
    if (q < g.sp) { a1 += p1[q]; a2 += p2[q]; }
  const float y1 = a1 * sc + g.bias[n1];
  const float y2 = a2 * sc + g.bias[n2];
  const int half = g.dh >> 1, bph = g.dh >> 5;
  const int qb = g.nq * bph, kvb = g.nkv * bph;
  int sec, head, blk;
  if (nb < qb) { sec = 0; head = nb / bph; blk = nb - head * bph; }
  else if (nb < qb + kvb) { sec = 1; head = (nb - qb) / bph; blk = nb - qb - head * bph; }
  else { sec = 2; head = (nb - qb - kvb) / bph; blk = nb - qb - kvb - head * bph; }
  const int i = blk * 16 + p;
  const int b = m / g.T, slot = m - b * g.T;
  const int pos = g.len[b] + slot;
  if (pos >= g.cap) return;
  if (sec == 2) {
    uint16_t* dst = g.vc + (size_t)b * g.seq_stride + ((size_t)head * g.cap + pos) * g.dh;
    dst[i] = f2bf(y1);
    dst[i + half] = f2bf(y2);
  } else {
    const float2 cs = g.rope[(size_t)pos * half + i];
    const float o1 = y1 * cs.x - y2 * cs.y;
    const float o2 = y2 * cs.x + y1 * cs.y;
    if (sec == 0) {
      float* dst = g.q + ((size_t)m * g.nq + head) * g.dh;
      dst[i] = o1;
      dst[i + half] = o2;
    } else {
      uint16_t* dst = g.kc + (size_t)b * g.seq_stride + ((size_t)head * g.cap + pos) * g.dh;
      dst[i] = f2bf(o1);
      dst[i + half] = f2bf(o2);
    }
  }
}

// Residual: workgroup (row m, 256 columns).  x += sum of partials; next norm's input as
// hi/lo bf16; sum of squares per 32-column block (a 32-lane tree, fixed order).
__global__ __launch_bounds__(256) void k_reduce_resid(const GemmArgs g) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  float v = 0.f;
  if (n < g.n_out) {
    float pv[kMaxSplit];
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q) pv[q] = g.part[((size_t)min(q, g.sp - 1) * g.rows + m) * g.n_out + n];
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q)
      if (q < g.sp) acc += pv[q];
    const size_t o = (size_t)m * g.n_out + n;
    v = g.x[o] + acc;
    g.x[o] = v;
    store_split(g.a_next, g.n_out, g.rows, m, n, v * g.gain_next[n]);
    if (g.hidden) g.hidden[o] = f2bf(v);
  }
  float sq = v * v;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) sq += __shfl_xor(sq, o);
  if ((threadIdx.x & 31) == 0 && n < g.n_out) g.ssq_out[(size_t)m * (g.n_out / 32) + (n >> 5)] = sq;
}

hipError_t launch_reduce(int epi, const GemmArgs& g, hipStream_t s) {
  if (epi == kEpiQkv) {
    k_reduce_qkv<<<dim3((g.nb * 16 + 255) / 256, g.rows), 256, 0, s>>>(g);
  } else if (epi == kEpiResid) {
    k_reduce_resid<<<dim3((g.n_out + 255) / 256, g.rows), 256, 0, s>>>(g);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------------
// Embedding: row r = (sequence b, slot i) takes [pending or stage.first, d_1..d_k, 0...][i],
// writes the fp32 residual, x * ln1 gain as hi/lo bf16 rows, and per-32-column sums of
// squares.  Thread t handles columns 8t..8t+7; four consecutive lanes form a 32-column block.
__global__ __launch_bounds__(256) void k_embed(const EmbedArgs e) {
  const int r = blockIdx.x;
  const int b = r / e.T, slot = r - b * e.T;
  int tok;
  if (slot == 0) {
    tok = (e.stage->flags & kFlagFirst) ? e.stage->first[b] : e.next[b];
  } else {
    const int j = slot - 1;
    tok = (j < e.stage->k[b]) ? e.stage->draft[b * e.kmax + j] : 0;
  }
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
      store_split(e.a, e.H, e.rows, r, col, v * e.gain[col]);
      s += v * v;
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if ((c8 & 3) == 0) e.ssq[(size_t)r * nparts + (c8 >> 2)] = s;
  }
}

hipError_t launch_embed(const EmbedArgs& e, hipStream_t s) {
  k_embed<<<e.rows, 256, 0, s>>>(e);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------------
// Attention, phase 1 (MFMA).  Workgroup (span x, kv head, sequence x row group) takes up to 64
// query rows of one KV head (slot-major: row = slot*G + head-in-group, G = nq/nkv) against
// the span's positions [x*kSpan, (x+1)*kSpan), in chunks of 64 position-aligned keys.
// Wave w owns query rows 16w..16w+15: S = Q K^T and O += P V are 16x16x32 bf16 MFMAs, the
// softmax is the usual running (max, sum) per row in base 2.  K is staged in LDS row-major,
// V transposed, P goes through LDS to change from the MFMA output layout to the input one.
// Q and P enter the MFMAs as bf16 hi + lo pairs (two MFMAs each); K and V are the bf16 cache.
// Spans are fixed by absolute position, so a row's result does not depend on the length.
constexpr int kSpanChunks = 1;
constexpr int kSpan = kSpanChunks * kChunk;
// Spans a row can need at the largest cache capacity, held 64 per register slot in the merge.
constexpr int kSpanSlots = (kMaxCapacity / kSpan + 63) / 64;

template <int DH>
__global__ __launch_bounds__(256) void k_attn(const AttnArgs a) {
  constexpr int KP = DH + 8;        // K row pitch (bf16): 16-byte aligned, conflict-free b128 reads
  constexpr int VP = kChunk + 8;    // V^T row pitch
  constexpr int PP = kChunk + 8;    // P row pitch
  __shared__ __attribute__((aligned(16))) uint16_t Kl[kChunk * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DH * VP];
  __shared__ __attribute__((aligned(16))) uint16_t Pl[4][2][16 * PP];   // [wave][hi, lo]

  const int x = blockIdx.x, kvh = blockIdx.y;
  const int G = a.nq / a.nkv, nrows = a.T * G;
  const int ngroups = (nrows + 63) / 64;
  const int b = blockIdx.z / ngroups, rg = blockIdx.z - b * ngroups;
  const int L = a.len[b];
  const int plast = L + a.T - 1;
  const int span0 = x * kSpan;
  if (span0 > plast) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wrow0 = rg * 64 + wave * 16;         // first query row of this wave
  const bool active = wrow0 < nrows;

  // K/V of a chunk: each thread loads kKvPerThread 16-byte pieces of K and of V, all
  // issued before any is used (positions past the last row's are zero).
  const uint16_t* kbase = a.kc + (size_t)b * a.seq_stride + (size_t)kvh * a.cap * DH;
  const uint16_t* vbase = a.vc + (size_t)b * a.seq_stride + (size_t)kvh * a.cap * DH;
  constexpr int kKvPerThread = kChunk * DH / 8 / 256;
  u32x4 kreg[kKvPerThread], vreg[kKvPerThread];
  auto load_kv = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kKvPerThread; ++u) {
      const int idx = tid + u * 256;
      const int j = idx / (DH / 8), d8 = (idx - j * (DH / 8)) * 8;
      const int pos = min(c0 + j, plast);
      kreg[u] = *(const u32x4*)(kbase + (size_t)pos * DH + d8);
      vreg[u] = *(const u32x4*)(vbase + (size_t)pos * DH + d8);
      if (c0 + j > plast) { kreg[u] = (u32x4){0u, 0u, 0u, 0u}; vreg[u] = kreg[u]; }
    }
  };
  load_kv(span0);

  // Q as the MFMA A operand: lane holds row wrow0 + l16, dims ks*32 + 8*g4 .. +8, as a
  // bf16 hi part (qa) and lo part (ql).
  bf16x8 qa[DH / 32], ql[DH / 32];
  {
    const int qr = wrow0 + l16;
    const bool ok = qr < nrows;
    const int qc = min(qr, nrows - 1);
    const int slot = qc / G;
    const int hh = kvh * G + (qc - slot * G);
    const float* qp = a.q + ((size_t)(b * a.T + slot) * a.nq + hh) * DH;
    float qv[DH / 32][8];
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[ks][e] = qp[ks * 32 + g4 * 8 + e];
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) {
      uint16_t t[8], tl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ok ? qv[ks][e] : 0.f;
        t[e] = f2bf(v);
        tl[e] = f2bf(v - bf2f(t[e]));
      }
      u32x4 u, ul;
      u.x = t[0] | ((uint32_t)t[1] << 16);
      u.y = t[2] | ((uint32_t)t[3] << 16);
      u.z = t[4] | ((uint32_t)t[5] << 16);
      u.w = t[6] | ((uint32_t)t[7] << 16);
      ul.x = tl[0] | ((uint32_t)tl[1] << 16);
      ul.y = tl[2] | ((uint32_t)tl[3] << 16);
      ul.z = tl[4] | ((uint32_t)tl[5] << 16);
      ul.w = tl[6] | ((uint32_t)tl[7] << 16);
      qa[ks] = as_bf16x8(u);
      ql[ks] = as_bf16x8(ul);
    }
  }
  // Positions of the 4 rows this lane holds in the MFMA output layout (rows 4*g4 + r).
  int prow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qr = wrow0 + 4 * g4 + r;
    prow[r] = (qr < nrows) ? L + qr / G : -1;
  }

  f32x4 o[DH / 16];
#pragma unroll
  for (int nt = 0; nt < DH / 16; ++nt) o[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mrun[4], lrun[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { mrun[r] = -INFINITY; lrun[r] = 0.f; }


  for (int ci = 0; ci < kSpanChunks; ++ci) {
    const int c0 = span0 + ci * kChunk;
    if (c0 > plast) break;
    if (ci > 0) load_kv(c0);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kKvPerThread; ++u) {
      const int idx = tid + u * 256;
      const int j = idx / (DH / 8), d8 = (idx - j * (DH / 8)) * 8;
      *(u32x4*)(&Kl[j * KP + d8]) = kreg[u];
      const uint32_t vw[4] = {vreg[u].x, vreg[u].y, vreg[u].z, vreg[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        Vt[(d8 + 2 * t) * VP + j] = (uint16_t)(vw[t] & 0xFFFFu);
        Vt[(d8 + 2 * t + 1) * VP + j] = (uint16_t)(vw[t] >> 16);
      }
    }
    __syncthreads();
    float alpha[4];
    if (active) {
      f32x4 sc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sc[kt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) {
          const bf16x8 kb8 = as_bf16x8(*(const u32x4*)(&Kl[(kt * 16 + l16) * KP + ks * 32 + g4 * 8]));
          sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb8, sc[kt], 0, 0, 0);
          sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[ks], kb8, sc[kt], 0, 0, 0);
        }
      }
      // Scale, causal mask, running softmax.  Lane holds rows 4*g4+r, keys kt*16 + l16.
      float mloc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int kp = c0 + kt * 16 + l16;
          float v = sc[kt][r] * a.scale_log2;
          v = (kp <= prow[r]) ? v : -INFINITY;
          sc[kt][r] = v;
          m = fmaxf(m, v);
        }
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        m = fmaxf(m, __shfl_xor(m, 4));
        m = fmaxf(m, __shfl_xor(m, 8));
        mloc[r] = m;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mnew = fmaxf(mrun[r], mloc[r]);
        alpha[r] = (mnew == -INFINITY) ? 1.f : exp2f(mrun[r] - mnew);
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const float pv = (mnew == -INFINITY) ? 0.f : exp2f(sc[kt][r] - mnew);
          sc[kt][r] = pv;
          ls += pv;
        }
        ls += __shfl_xor(ls, 1);
        ls += __shfl_xor(ls, 2);
        ls += __shfl_xor(ls, 4);
        ls += __shfl_xor(ls, 8);
        lrun[r] = lrun[r] * alpha[r] + ls;
        mrun[r] = mnew;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t hi = f2bf(sc[kt][r]);
          Pl[wave][0][(4 * g4 + r) * PP + kt * 16 + l16] = hi;
          Pl[wave][1][(4 * g4 + r) * PP + kt * 16 + l16] = f2bf(sc[kt][r] - bf2f(hi));
        }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int nt = 0; nt < DH / 16; ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nt][r] *= alpha[r];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x4 pa = *(const u32x4*)(&Pl[wave][0][l16 * PP + ks * 32 + g4 * 8]);
          const u32x4 pl = *(const u32x4*)(&Pl[wave][1][l16 * PP + ks * 32 + g4 * 8]);
          const bf16x8 vb = as_bf16x8(*(const u32x4*)(&Vt[(nt * 16 + l16) * VP + ks * 32 + g4 * 8]));
          o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa), vb, o[nt], 0, 0, 0);
          o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pl), vb, o[nt], 0, 0, 0);
        }
      }
    }
  }
  if (!active) return;
  const size_t rstride = DH + 2;
  float* pbase = a.part + (((size_t)b * a.nkv + kvh) * a.nchunk + x) * (size_t)nrows * rstride;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qr = wrow0 + 4 * g4 + r;
    if (qr >= nrows) continue;
    float* pr = pbase + (size_t)qr * rstride;
#pragma unroll
    for (int nt = 0; nt < DH / 16; ++nt) pr[nt * 16 + l16] = o[nt][r];
    if (l16 == 0) { pr[DH] = mrun[r]; pr[DH + 1] = lrun[r]; }
  }
}

// Attention, phase 2: one wave per (row, q head); merge spans 0..p/kSpan in order.  Span
// maxima and sums are spread over lanes; the weighted sum of partial outputs runs over
// spans in increasing order.
template <int DH>
__global__ __launch_bounds__(256) void k_combine(const AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.rows * a.nq) return;
  const int r = item / a.nq, h = item - r * a.nq;
  const int G = a.nq / a.nkv, nrows = a.T * G;
  const int b = r / a.T, slot = r - b * a.T;
  const int kvh = h / G, qr = slot * G + (h - kvh * G);
  const int p = a.len[b] + slot;
  const int np = p / kSpan + 1;
  const size_t rstride = DH + 2;
  const size_t sstride = (size_t)nrows * rstride;
  const float* base = a.part + ((size_t)b * a.nkv + kvh) * a.nchunk * sstride + (size_t)qr * rstride;
  // Lane l holds span l + 64*i of the row in slot i.
  float ms[kSpanSlots], ws[kSpanSlots];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSpanSlots; ++i) {
    const int sp = lane + 64 * i;
    ms[i] = (sp < np) ? base[sp * sstride + DH] : -INFINITY;
    ws[i] = (sp < np) ? base[sp * sstride + DH + 1] : 0.f;
    M = fmaxf(M, ms[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float Ls = 0.f;
#pragma unroll
  for (int i = 0; i < kSpanSlots; ++i) {
    const float w = (ms[i] == -INFINITY) ? 0.f : exp2f(ms[i] - M);
    Ls += ws[i] * w;   // slot order, then the cross-lane tree
    ws[i] = w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) Ls += __shfl_xor(Ls, o);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int i = 0; i < kSpanSlots; ++i) {
    const int j0 = 64 * i;
    if (j0 >= np) break;
    const int j1 = min(np, j0 + 64);
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* pj = base + (size_t)(j + u) * sstride;
        v0[u] = pj[lane];
        v1[u] = (DH > 64) ? pj[lane + 64] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = __shfl(ws[i], j + u - j0);
        o0 += w * v0[u];
        o1 += w * v1[u];
      }
    }
    for (; j < j1; ++j) {
      const float w = __shfl(ws[i], j - j0);
      const float* pj = base + (size_t)j * sstride;
      o0 += w * pj[lane];
      if (DH > 64) o1 += w * pj[lane + 64];
    }
  }
  const float inv = 1.0f / Ls;
  const size_t qd = (size_t)a.nq * DH;
  store_split(a.out, qd, a.rows, r, h * DH + lane, o0 * inv);
  if (DH > 64) store_split(a.out, qd, a.rows, r, h * DH + lane + 64, o1 * inv);
}

hipError_t launch_attention(const AttnArgs& a, int dh, int B, hipStream_t s) {
  const int G = a.nq / a.nkv;
  const int ngroups = (a.T * G + 63) / 64;
  const dim3 grid(a.nchunk, a.nkv, B * ngroups);
  const int ncomb = (a.rows * a.nq + 3) / 4;
  if (dh == 128) {
    k_attn<128><<<grid, 256, 0, s>>>(a);
    k_combine<128><<<ncomb, 256, 0, s>>>(a);
  } else if (dh == 64) {
    k_attn<64><<<grid, 256, 0, s>>>(a);
    k_combine<64><<<ncomb, 256, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int attention_spans(int cap) { return (cap + kSpan - 1) / kSpan; }

// ----------------------------------------------------------------------------------------------
// Accept: per sequence, merge the LM head's per-block (max, index) pairs into the greedy
// choice at each of the T positions (largest value, lowest index on ties; the merge is
// order independent), count the leading drafts that match, and commit.  Wave w merges the
// rows w, w+16, ... of the sequence.
__device__ __forceinline__ void amax_merge(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__global__ __launch_bounds__(1024) void k_accept(const AcceptArgs a) {
  __shared__ int tgt[kMaxRows];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  if (a.has_head) {
    for (int slot = wave; slot < a.T; slot += 16) {
      const float2* row = a.amax + (size_t)(b * a.T + slot) * a.nparts;
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      int p = lane;
      for (; p + 7 * 64 < a.nparts; p += 8 * 64) {
        float2 e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = row[p + u * 64];
#pragma unroll
        for (int u = 0; u < 8; ++u) amax_merge(bv, bi, e[u].x, __float_as_int(e[u].y));
      }
      for (; p < a.nparts; p += 64) amax_merge(bv, bi, row[p].x, __float_as_int(row[p].y));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax_merge(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
      if (lane == 0) tgt[slot] = (bi == 0x7FFFFFFF) ? 0 : bi;
    }
  }
  __syncthreads();
  if (tid == 0) {
    Stage* st = a.stage;
    const int flags = st->flags;
    int k = st->k[b];
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
      if (!(flags & kFlagNoCommit)) a.len[b] += k + 1;
    }
  }
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t s) {
  k_accept<<<a.B, 1024, 0, s>>>(a);
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
