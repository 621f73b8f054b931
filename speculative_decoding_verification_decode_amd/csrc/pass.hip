// Persistent pass kernel for gfx950: one launch runs the whole forward pass of a small batch
// (at most kPassRows rows), from the embedding through every layer to the LM head argmax,
// the longest-prefix accept and the commit.
//
// Why one kernel: at 9 rows the pass is a stream of weight bytes, and between dependent
// kernels the GPU idles for a few microseconds each time (dispatch plus cache write-back
// and invalidation), nine times per layer.  Here the pass is a list of work items in
// dependency order, dealt round-robin to one workgroup per compute unit:
//
//   embed blocks | per layer: QKV blocks, attention (kv head x strided spans), span merge,
//   O blocks, gate/up blocks, down blocks x k splits | LM head blocks | final accept
//
// Every item waits only for items earlier in the list, so with all workgroups resident the
// pass always progresses.  A finished item stores the pass epoch into its done flag.  A GEMM
// wave issues its first weight loads, which depend on nothing, and then waits only for the
// producers of its own k range; the RMSNorm row scale, which needs whole rows, is applied
// in the epilogue after a wait for all producers.  Data that other workgroups read is
// stored agent-coherently (written through) before the flag, and every buffer a GEMM reads
// is written once per pass, so a reader's cache never holds an older copy.  Waits are
// bounded: a wait that gives up sets a sticky abort flag that the host reports as an error.
#include "device.h"

namespace sf {

constexpr int kPassThreads = 256;         // four waves
constexpr int kSpinLimit = 1 << 20;       // polls before a wait gives up (about a second)
constexpr int kPB = 4;                    // weight tiles per pipelined batch (two batches in flight per wave)

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Diagnostics timeline: slot 0 item start, 1 dependencies met, 2 compute done, 3 item end.
__device__ __forceinline__ void mark(const PassArgs& P, int gi, int slot) {
  if (P.trace && threadIdx.x == 0) P.trace[4 * (size_t)gi + slot] = __builtin_amdgcn_s_memrealtime();
}

// Wave-wide wait until flags[lo + i*stride] == epoch for every i < n.
__device__ bool wait_flags(const PassArgs& P, int lo, int n, int stride, int epoch) {
  const int lane = threadIdx.x & 63;
  for (int c = 0; c < n; c += 64) {
    const int i = c + lane;
    const int* f = P.flags + lo + (long)min(i, n - 1) * stride;
    int spins = 0;
    while (true) {
      const bool ok = (i >= n) || ld<true>(f) == epoch;
      if (__ballot(ok) == __ballot(1)) break;
      if (++spins > kSpinLimit) {
        if (lane == 0) st<true>(P.abort_flag, 1);
        return false;
      }
      if ((spins & 63) == 0 && ld<true>(P.abort_flag) != 0) return false;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  compiler_fence();
  return true;
}

// All of this workgroup's stores are complete, then the item's flag is set.
__device__ void publish(const PassArgs& P, int idx, int epoch) {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) st<true>(P.flags + idx, epoch);
}

// ---------------------------------------------------------------------------------------------
// Item layout.
struct Layout {
  const PassArgs& P;
  __device__ int lbase(int l) const { return P.nb_h + l * P.per_layer; }
  // Flag of 32-column block nb of x[l] (the embedding for l = 0, else the down reduction).
  __device__ int xflag(int l) const { return l == 0 ? 0 : lbase(l - 1) + P.off_down; }
  __device__ int xstride(int l) const { return l == 0 ? 1 : P.sp_d; }
  // Flag of QKV block nb / O block nb of layer l (the split-0 item's index).
  __device__ int qkv_flag(int l, int nb) const { return lbase(l) + nb * P.sp_q; }
  __device__ int o_flag(int l, int nb) const { return lbase(l) + P.off_o + nb * P.sp_o; }
  __device__ int head_base() const { return P.nb_h + P.L * P.per_layer; }
};

// ---------------------------------------------------------------------------------------------
// One wave's share of a weight block: tiles [kt0, kt1) of the packed 32-row block `wblk`
// against activation rows [0, ext_rows) of `act` (bf16 hi/lo operand rows in MFMA order).  The first two
// batches of weight tiles are requested before `wait` runs; the activations only after it.
template <typename Wait>
__device__ f32x16 stream_block(const PassArgs& P, int gi, const uint4* wblk, int kt0, int kt1, const uint16_t* act,
                               int k, int ext_rows, Wait wait) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc((void*)wblk, (short)0, kt1 * 1024, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ares =
      __builtin_amdgcn_make_buffer_rsrc((void*)act, (short)0, (int)act_bytes(ext_rows, k), kBufferWord3);
  const int tsp = act_tile_pieces(ext_rows);
  const bool row_ok = (lane & 31) < ext_rows;
  const int a_lane = ((lane >> 5) * ext_rows + (lane & 31)) * 16;   // operand (k half, row) of tile 0
  u32x4 w0[kPB], w1[kPB], a0[kPB], a1[kPB];
  auto loadw = [&](int kt, u32x4 (&w)[kPB]) {
#pragma unroll
    for (int t = 0; t < kPB; ++t)
      w[t] = __builtin_amdgcn_raw_buffer_load_b128(wres, (kt + t) * 1024 + lane * 16, 0, kCacheStream);
  };
  auto loada = [&](int kt, u32x4 (&a)[kPB]) {
#pragma unroll
    for (int t = 0; t < kPB; ++t) {
      const int off = (row_ok && kt + t < kt1) ? a_lane + (kt + t) * tsp * 16 : 0x7FFFFFF0;
      a[t] = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
    }
  };
  f32x16 acc = {};
  auto mma = [&](const u32x4 (&w)[kPB], const u32x4 (&a)[kPB]) {
#pragma unroll
    for (int t = 0; t < kPB; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w[t]), as_bf16x8(a[t]), acc, 0, 0, 0);
  };
  loadw(kt0, w0);
  loadw(kt0 + kPB, w1);
  wait();
  mark(P, gi, 1);
  loada(kt0, a0);
  loada(kt0 + kPB, a1);
  for (int kt = kt0; kt < kt1; kt += 2 * kPB) {
    __builtin_amdgcn_sched_barrier(0);
    mma(w0, a0);
    __builtin_amdgcn_sched_barrier(0);
    loadw(kt + 2 * kPB, w0);
    loada(kt + 2 * kPB, a0);
    __builtin_amdgcn_sched_barrier(0);
    mma(w1, a1);
    __builtin_amdgcn_sched_barrier(0);
    loadw(kt + 3 * kPB, w1);
    loada(kt + 3 * kPB, a1);
    __builtin_amdgcn_sched_barrier(0);
  }
  mark(P, gi, 2);
  return acc;
}

struct PassLds {
  float tile[1024];      // 32 x 32 accumulator tile in MFMA output order
  float val[kPassRows * 32];   // block outputs [row][32] (hi + lo, summed over k splits)
  float rscale[kPassRows];
  float sq[32 * kPassRows];
  int last;
  int next_item;
  int epoch;
};

// Sum of the four waves' accumulators, in wave order, into lds.tile.
__device__ void reduce_waves(PassLds& lds, const f32x16& acc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float* t = &lds.tile[lane * 16 + r];
        *t = (w == 0) ? acc[r] : *t + acc[r];
      }
    }
    __syncthreads();
  }
}

// RMSNorm row scales 1/sqrt(mean(x^2) + eps) from per-32-column sums of squares.  Wave w
// owns rows w, w+4, ..., w+12; lane l sums parts l, l+64, then a cross-lane tree.  The
// loads are issued first (SsqRegs) and summed after the weight stream.
struct SsqRegs {
  float v[kPassRows / 4][kSsqPerLane];
};
__device__ SsqRegs ssq_load(const float* ssq, int nparts, int R) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  SsqRegs r;
#pragma unroll
  for (int j = 0; j < kPassRows / 4; ++j) {
    const int m = wave + 4 * j;
#pragma unroll
    for (int i = 0; i < kSsqPerLane; ++i) {
      const int p = lane + 64 * i;
      r.v[j][i] = (m < R && p < nparts) ? ssq[(size_t)m * nparts + p] : 0.f;
    }
  }
  return r;
}
__device__ void row_scales(PassLds& lds, const SsqRegs& r, int k, float eps, int R) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kPassRows / 4; ++j) {
    const int m = wave + 4 * j;
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kSsqPerLane; ++i) t += r.v[j][i];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o);
    if (lane == 0 && m < R) lds.rscale[m] = 1.0f / sqrtf(t / (float)k + eps);
  }
  __syncthreads();
}

__device__ __forceinline__ float tval(const PassLds& lds, int R, int nl, int m) {
  return lds.tile[tile_idx(nl, m)] + lds.tile[tile_idx(nl, R + m)];
}

// Block outputs into lds.val, summing k splits: with sp > 1 each split stores its values to
// part ([split][row][32] for this block, written through) and counts its arrival; only the
// split that brings the count to a multiple of sp continues, after adding the partials in
// split order.  Returns false for the others.
__device__ bool block_values(const PassArgs& P, PassLds& lds, float* part, int sp, int sidx, int* counter) {
  const int tid = threadIdx.x, R = P.R;
  for (int e = tid; e < 32 * kPassRows; e += kPassThreads) {
    const int nl = e & 31, m = e >> 5;
    if (m < R) {
      const float v = tval(lds, R, nl, m);
      lds.val[e] = v;
      if (sp > 1) st<true>(part + ((size_t)sidx * kPassRows + m) * 32 + nl, v);
    }
  }
  if (sp > 1) {
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds.last = ((old + 1) % sp) == 0;
    }
    __syncthreads();
    if (!lds.last) return false;
    compiler_fence();
    for (int e = tid; e < 32 * kPassRows; e += kPassThreads) {
      const int m = e >> 5;
      if (m < R) {
        float acc = 0.f;
        for (int q = 0; q < sp; ++q) acc += part[(size_t)q * kPassRows * 32 + e];
        lds.val[e] = acc;
      }
    }
  }
  __syncthreads();
  return true;
}

// Packed (value, index) key whose unsigned maximum is the largest value, lowest index first.
__device__ __forceinline__ unsigned long long amax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v + 0.0f);   // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(~(uint32_t)idx);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Tiles of wave u of U splitting kb tiles.
__device__ __forceinline__ void wave_range(int kb, int u, int U, int& kt0, int& kt1) {
  kt0 = (int)(((long)kb * u) / U);
  kt1 = (int)(((long)kb * (u + 1)) / U);
}

// ---------------------------------------------------------------------------------------------
// Items.

__device__ int row_token(const PassArgs& P, int m) {
  const int b = m / P.T, slot = m - b * P.T;
  const Stage* st = P.stage;
  int tok;
  if (slot == 0) {
    tok = (st->flags & kFlagFirst) ? st->first[b] : P.next[b];
  } else {
    const int j = slot - 1;
    tok = (j < st->k[b]) ? st->draft[b * P.kmax + j] : 0;
  }
  return min(max(tok, 0), P.V - 1);
}

// Embedding of 32 columns for every row: x[0], x * ln1 as hi/lo, sums of squares.
__device__ void item_embed(const PassArgs& P, int gi, int nb, int epoch) {
  const int tid = threadIdx.x, m = tid >> 4, c = nb * 32 + (tid & 15) * 2;
  const int H = P.H, R = P.R;
  float s = 0.f;
  if (m < R) {
    const uint32_t w = *(const uint32_t*)(P.embed + (size_t)row_token(P, m) * H + c);
    const float v0 = __uint_as_float(w << 16), v1 = __uint_as_float(w & 0xFFFF0000u);
    const float* g1 = P.layers[0].g1;
    st<true>(P.x + (size_t)m * H + c, v0);
    st<true>(P.x + (size_t)m * H + c + 1, v1);
    store_split<true>(P.a, R, m, c, v0 * g1[c]);
    store_split<true>(P.a, R, m, c + 1, v1 * g1[c + 1]);
    s = v0 * v0 + v1 * v1;
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 8);
  if (m < R && (tid & 15) == 0) st<true>(P.ssq + (size_t)m * P.nb_h + nb, s);
  publish(P, gi, epoch);
}

// QKV block nb of layer l, k split sidx of sp_q: bias, RoPE, q and the K/V append at positions
// len + slot (by the split that completes the block).
__device__ void item_qkv(const PassArgs& P, PassLds& lds, int gi, int l, int nb, int sidx, int epoch) {
  const Layout Lo{P};
  const int wave = wave_id(), H = P.H, R = P.R, sp = P.sp_q;
  const PassLayer& Ly = P.layers[l];
  int kt0, kt1;
  wave_range(P.kb_h, sidx * 4 + wave, 4 * sp, kt0, kt1);
  const int xs = Lo.xstride(l);
  SsqRegs sr;
  const f32x16 acc = stream_block(P, gi, Ly.wqkv + (size_t)nb * P.kb_h * 64, kt0, kt1, P.a + (size_t)l * 2 * kPassRows * H,
                                  H, 2 * R, [&] {
                                    wait_flags(P, Lo.xflag(l), P.nb_h, xs, epoch);
                                    sr = ssq_load(P.ssq + (size_t)l * kPassRows * P.nb_h, P.nb_h, R);
                                  });
  row_scales(lds, sr, H, P.eps, R);
  reduce_waves(lds, acc);
  float* part = P.qpart + (((size_t)l * P.nb_qkv + nb) * sp) * kPassRows * 32;
  if (!block_values(P, lds, part, sp, sidx, P.dcount + ((size_t)l * 3 + 0) * P.cnt_stride + nb)) return;
  const int tid = threadIdx.x, p = tid & 15, m = tid >> 4;
  if (m < R) {
    const int dh = P.dh, half = dh >> 1, bph = dh >> 5;
    const int qb = P.nq * bph, kvb = P.nkv * bph;
    int sec, head, blk;
    if (nb < qb) { sec = 0; head = nb / bph; blk = nb - head * bph; }
    else if (nb < qb + kvb) { sec = 1; head = (nb - qb) / bph; blk = nb - qb - head * bph; }
    else { sec = 2; head = (nb - qb - kvb) / bph; blk = nb - qb - kvb - head * bph; }
    const int i = blk * 16 + p;
    const float s = lds.rscale[m];
    const float y1 = lds.val[m * 32 + p] * s + Ly.bqkv[nb * 32 + p];
    const float y2 = lds.val[m * 32 + p + 16] * s + Ly.bqkv[nb * 32 + p + 16];
    const int b = m / P.T, slot = m - b * P.T;
    const int pos = P.len[b] + slot;
    if (pos < P.cap) {
      const size_t kvo = (size_t)l * P.layer_stride + (size_t)b * P.seq_stride + ((size_t)head * P.cap + pos) * dh;
      if (sec == 2) {
        st<true>(P.vpool + kvo + i, f2bf(y1));
        st<true>(P.vpool + kvo + i + half, f2bf(y2));
      } else {
        const float2 cs = P.rope[(size_t)pos * half + i];
        const float o1 = y1 * cs.x - y2 * cs.y;
        const float o2 = y2 * cs.x + y1 * cs.y;
        if (sec == 0) {
          float* dst = P.q + ((size_t)l * kPassRows + m) * P.Q + (size_t)head * dh;
          st<true>(dst + i, o1);
          st<true>(dst + i + half, o2);
        } else {
          st<true>(P.kpool + kvo + i, f2bf(o1));
          st<true>(P.kpool + kvo + i + half, f2bf(o2));
        }
      }
    }
  }
  publish(P, Lo.qkv_flag(l, nb), epoch);
}

__device__ AttnArgs attn_args(const PassArgs& P, int l) {
  AttnArgs a{};
  a.q = P.q + (size_t)l * kPassRows * P.Q;
  a.kc = P.kpool + (size_t)l * P.layer_stride;
  a.vc = P.vpool + (size_t)l * P.layer_stride;
  a.seq_stride = P.seq_stride;
  a.cap = P.cap;
  a.len = P.len;
  a.T = P.T;
  a.nq = P.nq;
  a.nkv = P.nkv;
  a.nchunk = P.nchunk;
  a.scale_log2 = P.scale_log2;
  a.part = P.apart;
  a.out = P.o + (size_t)l * 2 * kPassRows * P.Q;
  a.rows = P.R;
  return a;
}

// Attention of (kv head, sequence, row group) over spans a, a + A, a + 2A, ...
template <int DH>
__device__ void item_attn(const PassArgs& P, int gi, int l, int i, int epoch) {
  const Layout Lo{P};
  const int A = P.attn_a;
  const int ia = i % A;
  int rest = i / A;
  const int rg = rest % P.ngroups;
  rest /= P.ngroups;
  const int b = rest % P.B, kvh = rest / P.B;
  const int G = P.nq / P.nkv, bph = DH / 32;
  const int sq = P.sp_q;
  wait_flags(P, Lo.qkv_flag(l, kvh * G * bph), G * bph, sq, epoch);                   // q heads of the group
  wait_flags(P, Lo.qkv_flag(l, P.nq * bph + kvh * bph), bph, sq, epoch);              // k head
  wait_flags(P, Lo.qkv_flag(l, (P.nq + P.nkv) * bph + kvh * bph), bph, sq, epoch);    // v head
  mark(P, gi, 1);
  const AttnArgs aa = attn_args(P, l);
  const int plast = P.len[b] + P.T - 1;
  for (int x = ia; x * kSpan <= plast; x += A) attn_span<DH, true>(aa, x, kvh, b, rg);
  mark(P, gi, 2);
  publish(P, gi, epoch);
}

// Span merge of pairs (head h, row r) 4c .. 4c+3, head-major.
template <int DH>
__device__ void item_comb(const PassArgs& P, int gi, int l, int c, int epoch) {
  const Layout Lo{P};
  const int R = P.R, G = P.nq / P.nkv;
  const int h0 = (4 * c) / R, h1 = min(P.nq - 1, (4 * c + 3) / R);
  const int per_kvh = P.B * P.ngroups * P.attn_a;
  const int k0 = h0 / G, k1 = h1 / G;
  wait_flags(P, Lo.lbase(l) + P.off_attn + k0 * per_kvh, (k1 - k0 + 1) * per_kvh, 1, epoch);
  mark(P, gi, 1);
  const int pair = 4 * c + wave_id();
  if (pair < P.nq * R) combine_pair<DH, true>(attn_args(P, l), pair % R, pair / R);
  mark(P, gi, 2);
  publish(P, gi, epoch);
}

// O projection block nb, k split sidx of sp_o: x_mid = x + o W^T, x_mid * ln2 as hi/lo, sums of
// squares (by the split that completes the block).
__device__ void item_oproj(const PassArgs& P, PassLds& lds, int gi, int l, int nb, int sidx, int epoch) {
  const Layout Lo{P};
  const int wave = wave_id(), H = P.H, R = P.R, sp = P.sp_o;
  const PassLayer& Ly = P.layers[l];
  int kt0, kt1;
  wave_range(P.kb_q, sidx * 4 + wave, 4 * sp, kt0, kt1);
  const f32x16 acc = stream_block(P, gi, Ly.wo + (size_t)nb * P.kb_q * 64, kt0, kt1, P.o + (size_t)l * 2 * kPassRows * P.Q,
                                  P.Q, 2 * R, [&] {
                                    const int hh0 = kt0 * kTileK / P.dh, hh1 = (kt1 * kTileK - 1) / P.dh;
                                    const int c0 = (hh0 * R) / 4, c1 = ((hh1 + 1) * R + 3) / 4;
                                    wait_flags(P, Lo.lbase(l) + P.off_comb + c0, c1 - c0, 1, epoch);
                                  });
  reduce_waves(lds, acc);
  float* part = P.opart + (((size_t)l * P.nb_h + nb) * sp) * kPassRows * 32;
  if (!block_values(P, lds, part, sp, sidx, P.dcount + ((size_t)l * 3 + 1) * P.cnt_stride + nb)) return;
  const int tid = threadIdx.x;
  const float* xin = P.x + (size_t)l * kPassRows * H;
  float* xo = P.xm + (size_t)l * kPassRows * H;
  uint16_t* ao = P.am + (size_t)l * 2 * kPassRows * H;
  for (int e = tid; e < 32 * kPassRows; e += kPassThreads) {
    const int nl = e & 31, m = e >> 5;
    float v = 0.f;
    if (m < R) {
      const int n = nb * 32 + nl;
      const size_t o = (size_t)m * H + n;
      v = xin[o] + lds.val[e];
      st<true>(xo + o, v);
      store_split<true>(ao, R, m, n, v * Ly.g2[n]);
    }
    lds.sq[e] = v * v;
  }
  __syncthreads();
  if (tid < R) {
    float s = 0.f;
#pragma unroll
    for (int nl = 0; nl < 32; ++nl) s += lds.sq[tid * 32 + nl];
    st<true>(P.ssqm + ((size_t)l * kPassRows + tid) * P.nb_h + nb, s);
  }
  publish(P, Lo.o_flag(l, nb), epoch);
}

// gate/up block nb: h = silu(gate) * up for 16 ffn columns, as hi/lo.
__device__ void item_gateup(const PassArgs& P, PassLds& lds, int gi, int l, int nb, int epoch) {
  const Layout Lo{P};
  const int wave = wave_id(), H = P.H, R = P.R;
  const PassLayer& Ly = P.layers[l];
  int kt0, kt1;
  wave_range(P.kb_h, wave, 4, kt0, kt1);
  SsqRegs sr;
  const f32x16 acc = stream_block(P, gi, Ly.wgu + (size_t)nb * P.kb_h * 64, kt0, kt1, P.am + (size_t)l * 2 * kPassRows * H,
                                  H, 2 * R, [&] {
                                    wait_flags(P, Lo.o_flag(l, 0), P.nb_h, P.sp_o, epoch);
                                    sr = ssq_load(P.ssqm + (size_t)l * kPassRows * P.nb_h, P.nb_h, R);
                                  });
  row_scales(lds, sr, H, P.eps, R);
  reduce_waves(lds, acc);
  const int tid = threadIdx.x, p = tid & 15, m = tid >> 4;
  if (m < R) {
    const float s = lds.rscale[m];
    const float gt = tval(lds, R, p, m) * s;
    const float up = tval(lds, R, p + 16, m) * s;
    const float hv = gt / (1.0f + expf(-gt)) * up;
    store_split<true>(P.h + (size_t)l * 2 * kPassRows * P.F, R, m, nb * 16 + p, hv);
  }
  publish(P, gi, epoch);
}

// Down projection block nb, k split sidx of sp_d.  Each split stores its partial sums; the
// split that arrives last adds them in split order, adds the residual and writes the next
// layer's input (and its norm operand and sums of squares).
__device__ void item_down(const PassArgs& P, PassLds& lds, int gi, int l, int nb, int sidx, int epoch) {
  const Layout Lo{P};
  const int wave = wave_id(), H = P.H, R = P.R, sp = P.sp_d;
  const PassLayer& Ly = P.layers[l];
  int kt0, kt1;
  wave_range(P.kb_f, sidx * 4 + wave, 4 * sp, kt0, kt1);
  const f32x16 acc = stream_block(P, gi, Ly.wd + (size_t)nb * P.kb_f * 64, kt0, kt1, P.h + (size_t)l * 2 * kPassRows * P.F,
                                  P.F, 2 * R, [&] {
                                    wait_flags(P, Lo.lbase(l) + P.off_gu + kt0, kt1 - kt0, 1, epoch);
                                  });
  reduce_waves(lds, acc);
  const int tid = threadIdx.x;
  float* part = P.dpart + (((size_t)l * P.nb_h + nb) * sp) * kPassRows * 32;
  if (!block_values(P, lds, part, sp, sidx, P.dcount + ((size_t)l * 3 + 2) * P.cnt_stride + nb)) return;
  const bool last_layer = (l + 1 == P.L);
  const float* xin = P.xm + (size_t)l * kPassRows * H;
  float* xo = P.x + (size_t)(l + 1) * kPassRows * H;
  uint16_t* ao = P.a + (size_t)(l + 1) * 2 * kPassRows * H;
  for (int e = tid; e < 32 * kPassRows; e += kPassThreads) {
    const int nl = e & 31, m = e >> 5;
    float v = 0.f;
    if (m < R) {
      const int n = nb * 32 + nl;
      const size_t o = (size_t)m * H + n;
      v = xin[o] + lds.val[e];
      st<true>(xo + o, v);
      store_split<true>(ao, R, m, n, v * Ly.gnext[n]);
      if (last_layer && P.hidden) P.hidden[o] = f2bf(v);
    }
    lds.sq[e] = v * v;
  }
  __syncthreads();
  if (tid < R) {
    float s = 0.f;
#pragma unroll
    for (int nl = 0; nl < 32; ++nl) s += lds.sq[tid * 32 + nl];
    st<true>(P.ssq + ((size_t)(l + 1) * kPassRows + tid) * P.nb_h + nb, s);
  }
  publish(P, Lo.lbase(l) + P.off_down + nb * sp, epoch);
}

// LM head block nb: logits of 32 vocabulary entries, folded into the per-row maximum.
__device__ void item_head(const PassArgs& P, PassLds& lds, int gi, int nb, int epoch) {
  const Layout Lo{P};
  const int wave = wave_id(), H = P.H, R = P.R, L = P.L;
  int kt0, kt1;
  wave_range(P.kb_h, wave, 4, kt0, kt1);
  const int xs = Lo.xstride(L);
  SsqRegs sr;
  const f32x16 acc = stream_block(P, gi, P.head + (size_t)nb * P.kb_h * 64, kt0, kt1, P.a + (size_t)L * 2 * kPassRows * H,
                                  H, 2 * R, [&] {
                                    wait_flags(P, Lo.xflag(L), P.nb_h, xs, epoch);
                                    sr = ssq_load(P.ssq + (size_t)L * kPassRows * P.nb_h, P.nb_h, R);
                                  });
  row_scales(lds, sr, H, P.eps, R);
  reduce_waves(lds, acc);
  const int m = threadIdx.x;
  if (m < R) {
    const float s = lds.rscale[m];
    float best = -INFINITY;
    int bi = nb * 32;
    for (int nl = 0; nl < 32; ++nl) {
      const float v = tval(lds, R, nl, m) * s;
      if (P.logits) P.logits[(size_t)m * P.V + nb * 32 + nl] = v;
      if (v > best) { best = v; bi = nb * 32 + nl; }
    }
    __hip_atomic_fetch_max(P.amax + m, amax_key(best, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(P.hcount, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  publish(P, gi, epoch);
}

// Final item: per-row greedy targets, longest agreeing prefix, commit; resets the per-pass
// maxima and head counter and advances the epoch.
__device__ void item_final(const PassArgs& P, int epoch) {
  const Layout Lo{P};
  __shared__ int tgt[kPassRows];
  const int tid = threadIdx.x, R = P.R;
  if (tid == 0) {
    int spins = 0;
    while (ld<true>(P.checkin) < (int)gridDim.x) {
      if (++spins > kSpinLimit) { st<true>(P.abort_flag, 1); break; }
      if ((spins & 63) == 0 && ld<true>(P.abort_flag) != 0) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (P.has_head) {
    if (tid == 0) {
      int spins = 0;
      while (ld<true>(P.hcount) < P.nb_head) {
        if (++spins > kSpinLimit) { st<true>(P.abort_flag, 1); break; }
        if ((spins & 63) == 0 && ld<true>(P.abort_flag) != 0) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    compiler_fence();
    if (tid < R) {
      const unsigned long long key = ld<true>(P.amax + tid);
      const uint32_t idx = ~(uint32_t)(key & 0xFFFFFFFFull);
      tgt[tid] = (key == 0ull || idx >= (uint32_t)P.V) ? 0 : (int)idx;
    }
  } else if (tid < 64) {
    wait_flags(P, Lo.xflag(P.L), P.nb_h, Lo.xstride(P.L), epoch);
  }
  __syncthreads();
  if (tid == 0) {
    Stage* st_ = P.stage;
    const int flags = st_->flags;
    for (int b = 0; b < P.B; ++b) {
      const int k = min(max(st_->k[b], 0), P.T - 1);
      int M = 0;
      if (P.has_head) {
        if (flags & kFlagForce) {
          M = k;
        } else {
          while (M < k && st_->draft[b * P.kmax + M] == tgt[b * P.T + M]) ++M;
        }
        P.result[b] = M;
        for (int j = 0; j < P.T; ++j) P.result[P.B + b * P.T + j] = tgt[b * P.T + j];
        if (!(flags & kFlagNoCommit)) {
          P.len[b] += M + 1;
          P.next[b] = tgt[b * P.T + M];
        }
        if (P.draft_out) {
          const int s = st_->step[b];
          if (s < kMaxDraftSteps) P.draft_out[b * kMaxDraftSteps + s] = tgt[b * P.T];
          st_->step[b] = s + 1;
        }
      } else {
        P.result[b] = 0;
        if (!(flags & kFlagNoCommit)) P.len[b] += k + 1;
      }
    }
    P.result[kResultStatus] = ld<true>(P.abort_flag);
    st<true>(P.hcount, 0);
    st<true>(P.checkin, 0);
    st<true>(P.queue + ((epoch + 1) & 1), 0);   // the next pass takes items from the other slot
    st<true>(P.epoch, epoch + 1);
  }
  if (tid < R) st<true>(P.amax + tid, 0ull);
}

template <int DH>
__device__ void run_item(const PassArgs& P, PassLds& lds, int gi, int epoch);

template <int DH>
__global__ __launch_bounds__(kPassThreads, 2) void k_pass(const PassArgs P) {
  __shared__ PassLds lds;
  // Every workgroup reads the epoch and then checks in; the final item advances the epoch only
  // after all have checked in, so a workgroup that starts late still sees this pass's epoch
  // (and takes items from this pass's counter).
  if (threadIdx.x == 0) {
    lds.epoch = ld<true>(P.epoch);
    __hip_atomic_fetch_add(P.checkin, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const int epoch = lds.epoch;
  // Items are taken from a counter in list order (one counter per epoch parity; the final item
  // clears the other one for the next pass).  The next index is requested when an item starts,
  // so its latency is hidden by the item.  A workgroup's next item always comes after its
  // current one, so the lowest unfinished item is always being run: no deadlock.
  int* queue = P.queue + (epoch & 1);
  if (threadIdx.x == 0) lds.next_item = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int gi = lds.next_item;
  while (gi < P.n_items) {
    int nxt = 0;
    if (threadIdx.x == 0) nxt = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    mark(P, gi, 0);
    run_item<DH>(P, lds, gi, epoch);
    __syncthreads();  // LDS of this item is free for the next
    mark(P, gi, 3);
    if (threadIdx.x == 0) lds.next_item = nxt;
    __syncthreads();
    gi = lds.next_item;
  }
}

template <int DH>
__device__ void run_item(const PassArgs& P, PassLds& lds, int gi, int epoch) {
  const int per_layer = P.per_layer;
  {
    if (gi < P.nb_h) {
      item_embed(P, gi, gi, epoch);
      return;
    }
    const int j = gi - P.nb_h;
    const int l = j / per_layer;
    if (l < P.L) {
      const int r = j - l * per_layer;
      if (r < P.off_attn) item_qkv(P, lds, gi, l, r / P.sp_q, r % P.sp_q, epoch);
      else if (r < P.off_comb) item_attn<DH>(P, gi, l, r - P.off_attn, epoch);
      else if (r < P.off_o) item_comb<DH>(P, gi, l, r - P.off_comb, epoch);
      else if (r < P.off_gu) item_oproj(P, lds, gi, l, (r - P.off_o) / P.sp_o, (r - P.off_o) % P.sp_o, epoch);
      else if (r < P.off_down) item_gateup(P, lds, gi, l, r - P.off_gu, epoch);
      else {
        const int d = r - P.off_down;
        item_down(P, lds, gi, l, d / P.sp_d, d % P.sp_d, epoch);
      }
    } else {
      const int r = j - P.L * per_layer;
      if (P.has_head && r < P.nb_head) item_head(P, lds, gi, r, epoch);
      else item_final(P, epoch);
    }
  }
}

hipError_t launch_pass(const PassArgs& p, int grid, hipStream_t s) {
  if (p.dh == 128) k_pass<128><<<grid, kPassThreads, 0, s>>>(p);
  else if (p.dh == 64) k_pass<64><<<grid, kPassThreads, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sf
