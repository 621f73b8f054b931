// Device helpers of the verify kernels: bf16 conversion, DPP row reductions, coherent
// store/load helpers, the MFMA-order activation layout, and the attention span and
// span-merge bodies.
#pragma once

#include "sf_internal.h"

#include <math.h>

namespace sf {

// A pass whose kernels carry a gate runs only while the device flag is set; the kernels of a
// gated-off pass return at once (whole launches, so split arrival counters stay consistent).
// Every kernel a one-row-per-sequence pass can launch (compact and NF4 GEMMs of any m-tile
// count, attention, merge, embed, accept) has a gated instance that checks it.
__device__ __forceinline__ bool gated_off(const int* gate) { return gate && *gate == 0; }

// Checking build (SF_CHECKS=1, a library of its own): a violated invariant sets its bit in a
// per-device word with a vector atomic; the regular build compiles the checks away.
#ifndef SF_CHECKS
#define SF_CHECKS 0
#endif
#if SF_CHECKS
extern __device__ unsigned int g_checks;
#endif
__device__ __forceinline__ void check(bool ok, unsigned bit) {
#if SF_CHECKS
  if (!ok) atomicOr(&g_checks, bit);
#else
  (void)ok;
  (void)bit;
#endif
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one instruction instead of four).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Lane permutations inside a 16-lane DPP row (no LDS traffic, unlike __shfl_xor).
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
// Max and sum over the 16 lanes of a DPP row, every lane receiving the result: partners
// lane^1, lane^2 (quad permutes), then the mirrored half-row and row, which pair each
// group with a lane of the group it has not met yet -- the grouping of an xor tree.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v + dpp<kDppMirror>(v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Stores and loads of data that other workgroups of the same kernel read.  With kCoh the
// access is agent-coherent (a relaxed agent-scope atomic: the store is written through to
// memory and the load is served coherently), as the split-K partials of the GEMM need;
// without it these are ordinary accesses.
template <bool kCoh, typename T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (kCoh) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool kCoh, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (kCoh) return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Activations feeding an MFMA are carried as two bf16 values, hi = bf16(v) and
// lo = bf16(v - hi) (about 16 significant bits), as operand rows r and rows + r; the weights
// are bf16 and the products accumulate in fp32.
//
// Operand layout ("MFMA order"): for a matrix of ext = 2*rows operand rows and K columns,
// the 8 bf16 values of row r, columns 16t + 8h .. 16t + 8h + 7 (tile t, k half h) are the
// 16 bytes at index t*act_tile_pieces(ext) + h*ext + r.  One 32x32x16 MFMA's operand of a k
// tile is then 2*ext consecutive 16-byte pieces, so a wave's load of it touches a few cache
// lines instead of one line per row; each tile starts on a 128-byte line.
__device__ __forceinline__ size_t act_index(int ext, int r, int col) {
  return ((size_t)(col >> 4) * act_tile_pieces(ext) + ((col >> 3) & 1) * ext + r) * 8 + (col & 7);
}
template <bool kCoh = false>
__device__ __forceinline__ void store_split(uint16_t* base, int rows, int r, int col, float v) {
  const uint16_t hi = f2bf(v);
  st<kCoh>(base + act_index(2 * rows, r, col), hi);
  st<kCoh>(base + act_index(2 * rows, rows + r, col), f2bf(v - bf2f(hi)));
}

// Word 3 of a raw buffer resource on gfx9-family GPUs (gfx950 included).
constexpr int kBufferWord3 = 0x00020000;
// RMSNorm sum-of-squares partials (one per 32 columns) read per lane: hidden <= 64*32*3.
constexpr int kSsqPerLane = 3;
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
// Attention, phase 1 (MFMA).  Workgroup (x0, kv head, sequence x row group) takes up to 64
// query rows of one KV head (slot-major: row = slot*G + head-in-group, G = nq/nkv) against
// spans x0, x0 + xstep, ... (span_first(x) .. + span_chunks(x) chunks), each in chunks of 64
// position-aligned keys, writing one partial per span; each chunk's K/V loads are issued
// while the previous chunk is computed.  Spans are one chunk below position 2048 and four
// chunks from there on: every span's partial costs about as many bytes as its K/V, so long
// contexts (and batches of them) write four times fewer partials and merge fewer spans,
// while short contexts, where each chunk is about 3 us of latency-bound work, keep the
// short critical path (four-chunk spans everywhere measured 0.27 ms slower per 7B verify at
// contexts 512 and 2048).
// Wave w owns query rows 16w..16w+15: S = Q K^T and O += P V are 16x16x32 bf16 MFMAs, the
// softmax is the usual running (max, sum) per row in base 2.  K is staged in LDS row-major,
// V transposed, P goes through LDS to change from the MFMA output layout to the input one.
// Q and P enter the MFMAs as bf16 hi + lo pairs (two MFMAs each); K and V are the bf16 cache.
// Spans are fixed by absolute position, so a row's result does not depend on the length.
constexpr int kSpanSplit = 2048;                      // first position of the four-chunk spans
constexpr int kShortSpans = kSpanSplit / kChunk;      // one-chunk spans below it
constexpr int kLongChunks = 4;
__host__ __device__ constexpr int span_first(int x) {
  return x < kShortSpans ? x * kChunk : kSpanSplit + (x - kShortSpans) * kLongChunks * kChunk;
}
__host__ __device__ constexpr int span_chunks(int x) { return x < kShortSpans ? 1 : kLongChunks; }
__host__ __device__ constexpr int span_of(int p) {
  return p < kSpanSplit ? p / kChunk : kShortSpans + (p - kSpanSplit) / (kLongChunks * kChunk);
}
// Spans a row can need at the largest cache capacity, held 64 per register slot in the merge.
constexpr int kSpanSlots = (span_of(kMaxCapacity - 1) + 1 + 63) / 64;

template <int DH, bool kCoh>
__device__ void attn_spans(const AttnArgs& a, int x0, int xstep, int kvh, int b, int rg) {
  constexpr int KP = DH + 8;        // K row pitch (bf16): 16-byte aligned, conflict-free b128 reads
  constexpr int VP = kChunk + 8;    // V^T row pitch
  static_assert(DH % 64 == 0 && kChunk == 64, "K/V piece mapping and V^T swizzle assume 64-position chunks");
  // Piece idx of a chunk's K/V (16 bytes: 8 dims of one position) -> position j and first dim:
  // a wave's 64 pieces are 8 positions x 8 dim groups, so that the transposed V stores of a
  // wave (rows d, column j, column groups swizzled by (d/8)%8) fall in 32 different banks.
  auto piece = [](int idx, int& j, int& d8) {
    j = (idx >> 3) & 63;
    d8 = (((idx >> 9) << 3) | (idx & 7)) * 8;
  };
  // V^T element (d, j) sits in row d at column group (j/8) ^ ((d/8) % 8): 16-byte groups of 8
  // positions stay contiguous for the PV operand reads.
  auto vt_col = [](int d, int j) { return ((((j >> 3) ^ ((d >> 3) & 7)) << 3) | (j & 7)); };
  constexpr int PP = kChunk + 8;    // P row pitch
  __shared__ __attribute__((aligned(16))) uint16_t Kl[kChunk * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DH * VP];
  __shared__ __attribute__((aligned(16))) uint16_t Pl[4][2][16 * PP];   // [wave][hi, lo]

  const int G = a.nq / a.nkv, nrows = a.T * G;
  const int L = a.len[b];
  const int plast = L + a.T - 1;
  if (threadIdx.x == 0 && x0 == 0) check(plast < a.cap, kChkPos);
  int x = x0, span0 = span_first(x);
  if (span0 > plast) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wrow0 = rg * 64 + wave * 16;         // first query row of this wave
  const bool active = wrow0 < nrows;

  // K/V of a chunk: each thread loads kKvPerThread 16-byte pieces of K and of V, all
  // issued before any is used.  Positions past the last row's are read at the last position
  // and zeroed when staged in LDS, not here: a select on a loaded value right after the load
  // would make the wave wait for the load at once, so the next chunk's loads would not
  // overlap the current chunk's work.
  const uint16_t* kbase = a.kc + (size_t)b * a.seq_stride + (size_t)kvh * a.cap * DH;
  const uint16_t* vbase = a.vc + (size_t)b * a.seq_stride + (size_t)kvh * a.cap * DH;
  constexpr int kKvPerThread = kChunk * DH / 8 / 256;
  u32x4 kreg[kKvPerThread], vreg[kKvPerThread];
  auto load_kv = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kKvPerThread; ++u) {
      const int idx = tid + u * 256;
      int j, d8;
      piece(idx, j, d8);
      const int pos = min(c0 + j, plast);
      kreg[u] = *(const u32x4*)(kbase + (size_t)pos * DH + d8);
      vreg[u] = *(const u32x4*)(vbase + (size_t)pos * DH + d8);
    }
  };
  // Q as the MFMA A operand: lane holds row wrow0 + l16, dims ks*32 + 8*g4 .. +8, as a
  // bf16 hi part (qa) and lo part (ql).  The Q loads go out first and are converted while
  // the K/V loads are still in flight.
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
    load_kv(span0);
    __builtin_amdgcn_sched_barrier(0);
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
      // Keep the conversion here, ahead of the K/V wait, rather than next to its first use.
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w), "+v"(ul.x), "+v"(ul.y), "+v"(ul.z), "+v"(ul.w));
      qa[ks] = as_bf16x8(u);
      ql[ks] = as_bf16x8(ul);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // Positions of the 4 rows this lane holds in the MFMA output layout (rows 4*g4 + r).
  int prow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qr = wrow0 + 4 * g4 + r;
    prow[r] = (qr < nrows) ? L + qr / G : -1;
  }

  for (;;) {   // spans x0, x0 + xstep, ... up to the last position
    f32x4 o[DH / 16];
#pragma unroll
    for (int nt = 0; nt < DH / 16; ++nt) o[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float mrun[4], lrun[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { mrun[r] = -INFINITY; lrun[r] = 0.f; }

    const int nch = span_chunks(x);
    for (int ci = 0; ci < nch; ++ci) {
      const int c0 = span0 + ci * kChunk;
      if (c0 > plast) break;
      __syncthreads();   // every wave is done with the previous chunk's K and V
#pragma unroll
      for (int u = 0; u < kKvPerThread; ++u) {
        const int idx = tid + u * 256;
        int j, d8;
        piece(idx, j, d8);
        const bool past = c0 + j > plast;
        const u32x4 kz = past ? (u32x4){0u, 0u, 0u, 0u} : kreg[u];
        const u32x4 vz = past ? (u32x4){0u, 0u, 0u, 0u} : vreg[u];
        *(u32x4*)(&Kl[j * KP + d8]) = kz;
        const uint32_t vw[4] = {vz.x, vz.y, vz.z, vz.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          Vt[(d8 + 2 * t) * VP + vt_col(d8, j)] = (uint16_t)(vw[t] & 0xFFFFu);
          Vt[(d8 + 2 * t + 1) * VP + vt_col(d8, j)] = (uint16_t)(vw[t] >> 16);
        }
      }
      // The next chunk's K/V loads (this span's next chunk, else the first chunk of this
      // workgroup's next span) go out now and land while this chunk is computed.
      {
        const int nc = (ci + 1 < nch && c0 + kChunk <= plast) ? c0 + kChunk : span_first(x + xstep);
        if (nc <= plast) load_kv(nc);
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
          mloc[r] = row16_max(m);
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
          lrun[r] = lrun[r] * alpha[r] + row16_sum(ls);
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
            const int vd = nt * 16 + l16;
            const bf16x8 vb = as_bf16x8(*(const u32x4*)(&Vt[vd * VP + vt_col(vd, ks * 32 + g4 * 8)]));
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa), vb, o[nt], 0, 0, 0);
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pl), vb, o[nt], 0, 0, 0);
          }
        }
      }
    }
    if (active) {
      const size_t rstride = DH + 2;
      float* pbase = a.part + (((size_t)b * a.nkv + kvh) * a.nchunk + x) * (size_t)nrows * rstride;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qr = wrow0 + 4 * g4 + r;
        if (qr >= nrows) continue;
        float* pr = pbase + (size_t)qr * rstride;
#pragma unroll
        for (int nt = 0; nt < DH / 16; ++nt) st<kCoh>(pr + nt * 16 + l16, o[nt][r]);
        if (l16 == 0) { st<kCoh>(pr + DH, mrun[r]); st<kCoh>(pr + DH + 1, lrun[r]); }
      }
    }
    x += xstep;
    span0 = span_first(x);
    if (span0 > plast) break;
  }
}

// Attention, phase 2: one wave per (row, q head); merge spans 0..span_of(p) in order.  Span
// maxima and sums are spread over lanes; the weighted sum of partial outputs runs over
// spans in increasing order.
template <int DH, bool kCoh>
__device__ void combine_pair(const AttnArgs& a, int r, int h) {
  const int lane = threadIdx.x & 63;
  const int G = a.nq / a.nkv, nrows = a.T * G;
  const int b = r / a.T, slot = r - b * a.T;
  const int kvh = h / G, qr = slot * G + (h - kvh * G);
  const int p = a.len[b] + slot;
  const int np = span_of(p) + 1;
  const size_t rstride = DH + 2;
  const size_t sstride = (size_t)nrows * rstride;
  const float* base = a.part + ((size_t)b * a.nkv + kvh) * a.nchunk * sstride + (size_t)qr * rstride;
  // Lane l holds span l + 64*i of the row in slot i.
  float ms[kSpanSlots], ws[kSpanSlots];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSpanSlots; ++i) {
    const int sp = lane + 64 * i;
    ms[i] = (sp < np) ? ld<kCoh>(base + sp * sstride + DH) : -INFINITY;
    ws[i] = (sp < np) ? ld<kCoh>(base + sp * sstride + DH + 1) : 0.f;
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
        v0[u] = ld<kCoh>(pj + lane);
        v1[u] = (DH > 64) ? ld<kCoh>(pj + lane + 64) : 0.f;
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
      o0 += w * ld<kCoh>(pj + lane);
      if (DH > 64) o1 += w * ld<kCoh>(pj + lane + 64);
    }
  }
  const float inv = 1.0f / Ls;
  store_split<kCoh>(a.out, a.rows, r, h * DH + lane, o0 * inv);
  if (DH > 64) store_split<kCoh>(a.out, a.rows, r, h * DH + lane + 64, o1 * inv);
}

// k split by last arrival: each of the sp workgroups of one output block calls this once,
// after its partial tile is stored agent-coherently and those stores have completed; exactly
// one of them (the one whose arrival completes the count) gets true and then reads the
// others' partials with agent-coherent loads.  That one puts the counter back to zero: all sp
// arrivals of this launch have happened, and the next launch that uses the counter starts
// after this kernel has ended, so a counter is zero between launches and never exceeds sp.
__device__ __forceinline__ bool split_arrive(int* counter, int sp) {
  const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1 != sp) return false;
  __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// One warm-up workgroup (index q among wa.nwarm): read the head tiles of the GEMM workgroups
// q, q + nwarm, ... with cached 16-byte loads, eight in flight per thread.
__device__ __forceinline__ void warm_gemm(const WarmArgs& wa, int q) {
  uint32_t acc = 0;
  for (int i = q; i < wa.n; i += wa.nwarm) {
    const int nb = i / wa.sp, spi = i - nb * wa.sp;
    const int t1 = (int)((long)wa.kb * (spi + 1) / wa.sp);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(wa.w + (size_t)nb * wa.kb * 64), (short)0, t1 * 1024, kBufferWord3);
    for (int w = 0; w < 4; ++w) {
      const int u = spi * 4 + w, U = wa.sp * 4;
      const int a = (int)(((long)wa.kb * u) / U), b = min((int)(((long)wa.kb * (u + 1)) / U), a + wa.head);
      for (int j = a * 64 + (int)threadIdx.x; j < b * 64; j += 256 * 8) {
        u32x4 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = j + e * 256;
          v[e] = __builtin_amdgcn_raw_buffer_load_b128(r, jj < b * 64 ? jj * 16 : 0x7FFFFFF0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc ^= v[e].x ^ v[e].y ^ v[e].z ^ v[e].w;
      }
    }
  }
  if (acc == 0x9E3779B9u) wa.sink[0] = acc;
}

__device__ __forceinline__ void amax_merge(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

}  // namespace sf
