// HIP kernels of the verify pass for gfx950 (CDNA4).
//
// Pass structure per layer (rows = sequences x positions, typically 1 x 9):
//   k_gemm<QKV>    weight-streaming MFMA GEMM; epilogue: RMSNorm row scale, bias,
//                  RoPE, K/V append into the static cache at position len+slot
//   k_attn         split-KV causal GQA attention over position-aligned chunks
//   k_combine      fixed-order merge of the chunk partials -> bf16 attention output
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

// Word 3 of a raw buffer resource on gfx9-family GPUs (gfx950 included).
constexpr int kBufferWord3 = 0x00020000;
// RMSNorm sum-of-squares partials (one per 16 columns) read per lane: hidden <= 64*16*4.
constexpr int kSsqPerLane = 4;
// Cache policy of the weight stream: non-temporal (each weight byte is read once per pass).
constexpr int kCacheStream = 2;

// Element (n_local, m) of a 16 x (16*MT) accumulator tile stored in MFMA output order:
// lane l of m-tile mt holds rows 4*(l/16)+r, column l%16.
__device__ __forceinline__ int tile_idx(int nl, int m) {
  return (m >> 4) * 256 + ((((nl >> 2) << 4) + (m & 15)) << 2) + (nl & 3);
}

// ----------------------------------------------------------------------------------------------
// Skinny GEMM: Y[m][n] = sum_k A[m][k] * W[n][k] for m < rows (<= 16*MT).
// W is packed in 16x32 tiles, one 16-byte bf16x8 fragment per lane, so a wave's load of one
// tile is one contiguous kilobyte.  Each wave streams its share of the k tiles of one
// n block, all loads of a batch issued before the first MFMA.  Waves are combined in LDS;
// with sp > 1 the workgroups of one n block are combined by the last one to finish, in
// fixed order, so results do not depend on scheduling.
template <int EPI, int MT>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const GemmArgs g) {
  __shared__ float red[kGemmWaves][MT * 256];
  __shared__ float tile[MT * 256];
  __shared__ float rscale[MT * 16];
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nb = blockIdx.x / g.sp, spi = blockIdx.x - nb * g.sp;
  const int U = g.sp * kGemmWaves, u = spi * kGemmWaves + wave;
  const int kt0 = (int)(((long)g.kb * u) / U), kt1 = (int)(((long)g.kb * (u + 1)) / U);

  constexpr bool kScaled = (EPI == kEpiQkv || EPI == kEpiSwiglu || EPI == kEpiArgmax);
  // Row scale of the folded RMSNorm.  Wave w owns rows w, w+8, ...; lane l sums parts
  // l, l+64, l+128, l+192 in that order, then the wave reduces across lanes: the same
  // order for a row whatever the number of rows.  The loads are issued here and summed
  // after the weight stream, so they never delay it.
  constexpr int kRowsPerWave = (MT * 16) / kGemmWaves;
  float ssq_v[kRowsPerWave][kSsqPerLane];
  if constexpr (kScaled) {
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.ssq_in, (short)0, g.rows * g.nparts_in * 4, kBufferWord3);
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int m = wave + kGemmWaves * j;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) {
        const int p = lane + 64 * i;
        const int off = (m < g.rows && p < g.nparts_in) ? (m * g.nparts_in + p) * 4 : 0x7FFFFFF0;
        ssq_v[j][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sres, off, 0, 0));
      }
    }
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Raw buffer loads: the hardware range check returns zeros for tiles at or past kt1
  // without touching memory, so every batch issues all of its loads unconditionally.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + (size_t)nb * g.kb * 64), (short)0, kt1 * 1024, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.a, (short)0, kMaxRows * g.k * 2, kBufferWord3);
  const int a_lane = ((lane & 15) * g.k + (lane >> 4) * 8) * 2;

  for (int kt = kt0; kt < kt1; kt += kBatch) {
    u32x4 w[kBatch];
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
      w[t] = __builtin_amdgcn_raw_buffer_load_b128(wres, (kt + t) * 1024 + lane * 16, 0, kCacheStream);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      u32x4 a[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t)
        a[t] = __builtin_amdgcn_raw_buffer_load_b128(ares, a_lane + (mt * 16 * g.k + (kt + t) * kTileK) * 2, 0, 0);
      // Keep every load of the batch ahead of the first MFMA (memory-level parallelism).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < kBatch; ++t)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[t]), as_bf16x8(a[t]), acc[mt], 0, 0, 0);
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][mt * 256 + lane * 4 + r] = acc[mt][r];

  if constexpr (kScaled) {
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < kSsqPerLane; ++i) t += ssq_v[j][i];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
      const int m = wave + kGemmWaves * j;
      if (lane == 0) rscale[m] = (m < g.rows) ? 1.0f / sqrtf(t / (float)g.k + g.eps) : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < MT * 256; e += kGemmThreads) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kGemmWaves; ++w) s += red[w][e];
    tile[e] = s;
  }
  __syncthreads();

  if (g.sp > 1) {
    float* mine = g.part + ((size_t)nb * g.sp + spi) * (MT * 256);
    for (int e = tid; e < MT * 256; e += kGemmThreads) mine[e] = tile[e];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int old = atomicAdd(&g.counters[nb], 1);
      last_flag = (old == g.sp - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    const float* all = g.part + (size_t)nb * g.sp * (MT * 256);
    for (int e = tid; e < MT * 256; e += kGemmThreads) {
      float s = 0.f;
      for (int q = 0; q < g.sp; ++q) s += __builtin_nontemporal_load(all + (size_t)q * (MT * 256) + e);
      tile[e] = s;
    }
    if (tid == 0) g.counters[nb] = 0;
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogues
  if constexpr (EPI == kEpiQkv) {
    // Packed rows of n block nb: 0..7 = head dims i0..i0+7, 8..15 = their RoPE partners i0+dh/2..
    const int p = tid & 7, m = tid >> 3;
    if (m < g.rows && m < MT * 16) {
      const int half = g.dh >> 1, bph = g.dh >> 4;
      const int qb = g.nq * bph, kvb = g.nkv * bph;
      int sec, head, blk;
      if (nb < qb) { sec = 0; head = nb / bph; blk = nb - head * bph; }
      else if (nb < qb + kvb) { sec = 1; head = (nb - qb) / bph; blk = nb - qb - head * bph; }
      else { sec = 2; head = (nb - qb - kvb) / bph; blk = nb - qb - kvb - head * bph; }
      const int i = blk * 8 + p;
      const float s = rscale[m];
      const float y1 = tile[tile_idx(p, m)] * s + g.bias[nb * 16 + p];
      const float y2 = tile[tile_idx(p + 8, m)] * s + g.bias[nb * 16 + p + 8];
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
    float* sq = &red[0][0];
    for (int e = tid; e < 16 * MT * 16; e += kGemmThreads) {
      const int nl = e & 15, m = e >> 4;
      float v = 0.f;
      if (m < g.rows) {
        const int n = nb * 16 + nl;
        const size_t o = (size_t)m * g.n_out + n;
        v = g.x[o] + tile[tile_idx(nl, m)];
        g.x[o] = v;
        g.a_next[o] = f2bf(v * g.gain_next[n]);
        if (g.hidden) g.hidden[o] = f2bf(v);
      }
      sq[e] = v * v;
    }
    __syncthreads();
    if (tid < MT * 16 && tid < g.rows) {
      float s = 0.f;
#pragma unroll
      for (int nl = 0; nl < 16; ++nl) s += sq[tid * 16 + nl];
      g.ssq_out[(size_t)tid * g.nb + nb] = s;
    }
  } else if constexpr (EPI == kEpiSwiglu) {
    // Packed rows of n block nb: 0..7 = gate rows j0..j0+7, 8..15 = up rows j0..j0+7.
    const int p = tid & 7, m = tid >> 3;
    if (m < g.rows && m < MT * 16) {
      const float s = rscale[m];
      const float gt = tile[tile_idx(p, m)] * s;
      const float up = tile[tile_idx(p + 8, m)] * s;
      const float hv = gt / (1.0f + expf(-gt)) * up;
      g.h[(size_t)m * g.ffn + nb * 8 + p] = f2bf(hv);
    }
  } else if constexpr (EPI == kEpiArgmax) {
    const int m = tid;
    if (m < g.rows && m < MT * 16) {
      const float s = rscale[m];
      float best = -INFINITY;
      int bi = nb * 16;
      for (int nl = 0; nl < 16; ++nl) {
        const float v = tile[tile_idx(nl, m)] * s;
        if (g.logits) g.logits[(size_t)m * g.vocab + nb * 16 + nl] = v;
        if (v > best) { best = v; bi = nb * 16 + nl; }
      }
      g.amax[(size_t)m * g.nb + nb] = make_float2(best, __int_as_float(bi));
    }
  }
}

template <int EPI>
static hipError_t gemm_mt(const GemmArgs& g, hipStream_t s) {
  const int mt = (g.rows + 15) / 16;
  const dim3 grid(g.nb * g.sp), block(kGemmThreads);
  switch (mt) {
    case 1: k_gemm<EPI, 1><<<grid, block, 0, s>>>(g); break;
    case 2: k_gemm<EPI, 2><<<grid, block, 0, s>>>(g); break;
    case 3:
    case 4: k_gemm<EPI, 4><<<grid, block, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, const GemmArgs& g, hipStream_t s) {
  switch (epi) {
    case kEpiQkv: return gemm_mt<kEpiQkv>(g, s);
    case kEpiResid: return gemm_mt<kEpiResid>(g, s);
    case kEpiSwiglu: return gemm_mt<kEpiSwiglu>(g, s);
    case kEpiArgmax: return gemm_mt<kEpiArgmax>(g, s);
  }
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------------------------
// Embedding: row r = (sequence b, slot i) takes [pending or stage.first, d_1..d_k, 0...][i],
// writes the fp32 residual, bf16(x * ln1 gain) and per-16-column sums of squares.
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
  const int nparts = e.H >> 4;
  for (int blk = threadIdx.x; blk < nparts; blk += blockDim.x) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int col = blk * 16 + c;
      const float v = bf2f(src[col]);
      e.x[(size_t)r * e.H + col] = v;
      e.a[(size_t)r * e.H + col] = f2bf(v * e.gain[col]);
      s += v * v;
    }
    e.ssq[(size_t)r * nparts + blk] = s;
  }
}

hipError_t launch_embed(const EmbedArgs& e, hipStream_t s) {
  k_embed<<<e.rows, 256, 0, s>>>(e);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------------
// Attention, phase 1: workgroup (chunk c, kv head, sequence x row group) scores up to 16
// query rows (slot-major: row = slot*G + head-in-group) against the chunk's 64 positions.
// Lane j of a wave owns key c*64+j; the causal rule masks keys past the row's position.
// Output per row: running max m, sum l and unnormalised o[dh] (base-2 exponentials).
template <int DH>
__global__ __launch_bounds__(256) void k_attn(const AttnArgs a) {
  __shared__ float Ks[kChunk][DH + 1];
  __shared__ float Vs[kChunk][DH + 1];
  const int c = blockIdx.x, kvh = blockIdx.y;
  const int G = a.nq / a.nkv, nrows = a.T * G;
  const int ngroups = (nrows + kAttnRows - 1) / kAttnRows;
  const int b = blockIdx.z / ngroups, rg = blockIdx.z - b * ngroups;
  const int L = a.len[b];
  const int plast = L + a.T - 1;
  const int c0 = c * kChunk;
  if (c0 > plast) return;

  const uint16_t* kb = a.kc + (size_t)b * a.seq_stride + ((size_t)kvh * a.cap + c0) * DH;
  const uint16_t* vb = a.vc + (size_t)b * a.seq_stride + ((size_t)kvh * a.cap + c0) * DH;
  for (int idx = threadIdx.x; idx < kChunk * DH / 8; idx += 256) {
    const int j = idx / (DH / 8), d8 = (idx - j * (DH / 8)) * 8;
    uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
    if (c0 + j <= plast && c0 + j < a.cap) {
      kv4 = *(const uint4*)(kb + (size_t)j * DH + d8);
      vv4 = *(const uint4*)(vb + (size_t)j * DH + d8);
    }
    const uint32_t kw[4] = {kv4.x, kv4.y, kv4.z, kv4.w};
    const uint32_t vw[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Ks[j][d8 + 2 * t] = __uint_as_float(kw[t] << 16);
      Ks[j][d8 + 2 * t + 1] = __uint_as_float(kw[t] & 0xFFFF0000u);
      Vs[j][d8 + 2 * t] = __uint_as_float(vw[t] << 16);
      Vs[j][d8 + 2 * t + 1] = __uint_as_float(vw[t] & 0xFFFF0000u);
    }
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_end = min(nrows, (rg + 1) * kAttnRows);
  for (int qr = rg * kAttnRows + wave; qr < row_end; qr += 4) {
    const int slot = qr / G, hh = kvh * G + (qr - slot * G);
    const int r = b * a.T + slot;
    const int p = L + slot;
    float* out = a.part + ((((size_t)b * a.nkv + kvh) * a.nchunk + c) * nrows + qr) * (DH + 2);
    if (c0 > p) {
      for (int d = lane; d < DH; d += 64) out[d] = 0.f;
      if (lane == 0) { out[DH] = -INFINITY; out[DH + 1] = 0.f; }
      continue;
    }
    const float* qv = a.q + ((size_t)r * a.nq + hh) * DH;
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < DH; ++d) s += qv[d] * Ks[lane][d];
    const bool valid = (c0 + lane <= p);
    s = valid ? s * a.scale_log2 : -INFINITY;
    float mx = s;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float pj = valid ? exp2f(s - mx) : 0.f;
    float l = pj;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    float o0 = 0.f, o1 = 0.f;
    for (int j = 0; j < kChunk; ++j) {
      const float pb = __shfl(pj, j);
      o0 += pb * Vs[j][lane];
      if (DH > 64) o1 += pb * Vs[j][lane + 64];
    }
    out[lane] = o0;
    if (DH > 64) out[lane + 64] = o1;
    if (lane == 0) { out[DH] = mx; out[DH + 1] = l; }
  }
}

// Attention, phase 2: one wave per (row, q head); merge chunks 0..p/64 in order.
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
  const int nc = p / kChunk + 1;
  const float* base = a.part + (((size_t)b * a.nkv + kvh) * a.nchunk * nrows + qr) * (DH + 2);
  const size_t cstride = (size_t)nrows * (DH + 2);
  float mx = -INFINITY;
  for (int c = 0; c < nc; ++c) mx = fmaxf(mx, base[c * cstride + DH]);
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float* pc = base + c * cstride;
    const float w = exp2f(pc[DH] - mx);
    l += pc[DH + 1] * w;
    o0 += pc[lane] * w;
    if (DH > 64) o1 += pc[lane + 64] * w;
  }
  const float inv = 1.0f / l;
  uint16_t* dst = a.out + (size_t)r * a.nq * DH + (size_t)h * DH;
  dst[lane] = f2bf(o0 * inv);
  if (DH > 64) dst[lane + 64] = f2bf(o1 * inv);
}

hipError_t launch_attention(const AttnArgs& a, int dh, int B, hipStream_t s) {
  const int G = a.nq / a.nkv;
  const int ngroups = (a.T * G + kAttnRows - 1) / kAttnRows;
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

// ----------------------------------------------------------------------------------------------
// Accept: per sequence, merge the LM head's per-tile (max, index) pairs into the greedy
// choice at each of the T positions (largest value, lowest index on ties), count the
// leading drafts that match, and commit.
__global__ __launch_bounds__(1024) void k_accept(const AcceptArgs a) {
  __shared__ float sv[1024];
  __shared__ int si[1024];
  __shared__ int tgt[kMaxRows];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (a.has_head) {
    for (int slot = 0; slot < a.T; ++slot) {
      const float2* row = a.amax + (size_t)(b * a.T + slot) * a.nparts;
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int p = tid; p < a.nparts; p += 1024) {
        const float2 e = row[p];
        const int ei = __float_as_int(e.y);
        if (e.x > bv || (e.x == bv && ei < bi)) { bv = e.x; bi = ei; }
      }
      sv[tid] = bv;
      si[tid] = bi;
      __syncthreads();
      for (int w = 512; w > 0; w >>= 1) {
        if (tid < w) {
          const float ov = sv[tid + w];
          const int oi = si[tid + w];
          if (ov > sv[tid] || (ov == sv[tid] && oi < si[tid])) { sv[tid] = ov; si[tid] = oi; }
        }
        __syncthreads();
      }
      if (tid == 0) tgt[slot] = (si[0] == 0x7FFFFFFF) ? 0 : si[0];
      __syncthreads();
    }
  }
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
  const int row = n_blk * 16 + (lane & 15);
  const int k0 = kt * kTileK + (lane >> 4) * 8;
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
