// Internal declarations shared by the kernels and the host runtime of libsf.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sf {

constexpr int kWave = 64;
constexpr int kTileN = 32;                    // weight rows per packed tile (32x32x16 MFMA)
constexpr int kTileK = 16;                    // reduction depth per packed tile
constexpr int kBatch = 16;                    // weight tiles a wave loads before using them
constexpr int kChunk = 64;                    // attention: KV positions per chunk (position aligned)
constexpr int kMaxRows = 512;                 // rows (sequences x positions) per pass
constexpr int kMaxSeqs = 64;
constexpr int kMaxK = 16;                     // drafts per sequence (k_max <= 15, T <= 16)
constexpr int kMaxDraftSteps = 256;
constexpr int kPrefillChunk = 512;            // default prompt positions per prefill pass
static_assert(kPrefillChunk <= kMaxRows, "a prefill chunk is one pass");
constexpr int kMaxCapacity = 16384;  // positions per sequence

// GEMM activation operand layout with `ext` operand rows: for each 16-column k tile, the 2*ext
// 16-byte pieces (k half, row) are contiguous, padded to whole 128-byte lines so that no cache
// line holds pieces of two tiles (a consumer of a k range never touches a neighbouring tile).
__host__ __device__ constexpr int act_tile_pieces(int ext) { return (2 * ext + 7) & ~7; }
__host__ __device__ constexpr size_t act_bytes(int ext, int k) { return (size_t)(k / 16) * act_tile_pieces(ext) * 16; }

// Stage flags (device side).
constexpr int kFlagNoCommit = 1;
constexpr int kFlagForce = 2;
constexpr int kFlagFirst = 8;
// Invariant bits of the checking build (the SF_CHECK_* values of sf.h).
constexpr unsigned kChkToken = 1u, kChkK = 2u, kChkPos = 4u, kChkCommit = 8u, kChkNaN = 16u;                 // row 0 of each sequence takes stage.first, not the pending token

// Staging block: one host->device copy per pass.
struct Stage {
  int32_t flags;
  int32_t kmax;
  int32_t pad[2];
  int32_t k[kMaxSeqs];
  int32_t first[kMaxSeqs];
  int32_t step[kMaxSeqs];
  int32_t draft[kMaxSeqs * kMaxK];
};

enum Epi { kEpiQkv = 0, kEpiResid = 1, kEpiSwiglu = 2, kEpiArgmax = 3 };

// NF4 projections: the 16 levels as bf16 bits (quantiles of the standard normal distribution
// with an exact zero, normalised to [-1, 1]: the 4-bit NormalFloat table, each level rounded
// to bf16), 64-input blocks, and the packed block of 1 KB of codes + 32 bf16 row scales.
constexpr uint16_t kNf4Bits[16] = {0xBF80, 0xBF32, 0xBF06, 0xBECA, 0xBE92, 0xBE3D, 0xBDBA, 0x0000,
                                   0x3DA3, 0x3E25, 0x3E7C, 0x3EAD, 0x3EE2, 0x3F10, 0x3F39, 0x3F80};
constexpr int kNf4Block = 64;
constexpr int kNf4BlockBytes = 1024 + 64;
constexpr int kNf4MaxRows = 64;               // rows per pass of the NF4 GEMM (up to four m tiles)

struct GemmArgs {
  const uint4* w;          // packed weight tiles [nb][kb][64 lanes] x 16 B (32 rows x 16 k per tile)
  const uint16_t* a;       // bf16 activations [2*rows][k]: hi parts, then lo parts
  int k, kb, nb, rows;     // in-features, k tiles (k/16), 32-row n blocks, valid rows
  int sp;                  // workgroups splitting each block's k range
  float* part;             // split partials [nb][sp][rows][32] (sp > 1)
  int* counters;           // [nb] arrivals of the splits of each block (sp > 1); zero between launches
  int nw;                  // waves per workgroup: 4 or 8
  int row_lo;              // batched kernel: outputs of rows below row_lo are not needed (0: all)
  int kh;                  // weight tiles per pipelined batch (4 or 8) for single-tile row counts
  // RMSNorm folded into the consumer: row scale = 1/sqrt(sum(ssq_in[r][*])/k + eps)
  const float* ssq_in;
  int nparts_in;
  float eps;
  // positions
  int T;                   // positions per sequence; row r -> sequence r/T, slot r%T
  const int32_t* len;      // committed length per sequence
  int cap;
  // kEpiQkv
  const float* bias;       // packed bias, fp32 [nb*16]
  float* q;                // [rows][nq][dh]
  uint16_t* kc;            // layer base of K pool, [seq][nkv][cap][dh]
  uint16_t* vc;
  long seq_stride;         // elements between sequences in the pool
  const float2* rope;      // (cos, sin) [cap][dh/2]
  int nq, nkv, dh;
  // kEpiResid
  float* x;                // residual [rows][n_out]
  uint16_t* a_next;        // x * gain_next as hi/lo bf16 rows [2*rows][n_out]
  const float* gain_next;  // [n_out]
  float* ssq_out;          // [rows][nb]: sums of squares of x per 32 columns
  uint16_t* hidden;        // optional bf16(x) [rows][n_out]
  int n_out;               // output features (also the partial buffer's row length)
  // kEpiSwiglu
  uint16_t* h;             // silu(gate)*up as hi/lo bf16 rows [2*rows][ffn]
  int ffn;
  // kEpiArgmax
  float2* amax;            // [rows][nb] (value, index bits)
  float* logits;           // optional fp32 [rows][vocab]
  int vocab;
  const int* gate;        // nullptr, or the pass runs only while *gate != 0 (device flag)
};

struct EmbedArgs {
  const uint16_t* embed;   // [V][H]
  const Stage* stage;
  const int32_t* len;
  const int32_t* next;
  const float* gain;       // first layer's ln1
  float* x;
  uint16_t* a;             // x * gain as hi/lo bf16 rows [2*rows][H]
  float* ssq;              // [rows][H/32]
  int rows, T, H, V, kmax;
  const int* gate;        // nullptr, or the pass runs only while *gate != 0 (device flag)
};

// L2 warm-up of a compact GEMM that runs later in the same pass: its workgroup i (grid index i,
// n workgroups, sp per 32-row block, 4 waves each splitting the block split's k tiles) will
// stream, per wave, k tiles from kt0; the warm-up reads the first `head` tiles of every wave's
// range with cached loads (head >= the range: all of them).  Workgroup i of every launch runs on
// XCD i % 8, so a warm-up workgroup whose index matches i modulo 8 leaves the lines in the L2
// that GEMM workgroup reads through.
struct WarmArgs {
  const uint4* w;          // packed weight tiles of the GEMM (nullptr: no warm-up)
  int kb, sp, n, head;
  int nwarm;               // warm-up workgroups (a multiple of 8); workgroup q takes i = q, q+nwarm, ...
  uint32_t* sink;          // one word the loads' checksum may reach (keeps them alive)
};

struct AttnArgs {
  const float* q;
  const uint16_t* kc;
  const uint16_t* vc;
  long seq_stride;
  int cap;
  const int32_t* len;
  int T, nq, nkv, nchunk;  // nchunk: number of position spans (attention_spans(cap))
  float scale_log2;        // log2(e)/sqrt(dh)
  float* part;             // [seq][nkv][span][T*G][dh+2]
  uint16_t* out;           // combine output as hi/lo bf16 rows [2*rows][nq*dh]
  int rows;
  int dh;
  const int* gate;        // nullptr, or the pass runs only while *gate != 0 (device flag)
  WarmArgs warm;          // the O projection's weights, read into L2 while attention runs
};

struct AcceptArgs {
  const float2* amax;      // [rows][nparts]
  int nparts;
  Stage* stage;
  int32_t* len;
  int32_t* next;
  int32_t* result;         // accepted[B] then target[B][T]
  int32_t* draft_out;      // [B][kMaxDraftSteps]
  int B, T, has_head;
  int slot_lo;             // targets of slots below slot_lo are not computed (reported as 0)
  int cap;                 // cache capacity (checking build: a commit past it is recorded; 0: unchecked)
  const int* gate;        // nullptr, or the pass runs only while *gate != 0 (device flag)
};

// Launchers (kernels.hip).
hipError_t launch_gemm(int epi, const GemmArgs& g, hipStream_t s);
// Checking build: read (and optionally clear) the current device's invariant word; the
// regular build returns hipErrorNotSupported.
hipError_t read_checks(uint32_t* bits, bool clear);
hipError_t launch_embed(const EmbedArgs& e, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int dh, int B, hipStream_t s);
int attention_spans(int cap);
hipError_t launch_accept(const AcceptArgs& a, hipStream_t s);
hipError_t launch_gemm_nf4(int epi, const GemmArgs& g, hipStream_t s);
hipError_t launch_pack_nf4(uint8_t* dst, const uint8_t* const* rowptr, int N, int nblk, hipStream_t s);
hipError_t launch_pack(uint4* dst, const uint16_t* const* rowptr, int nb, int kb, hipStream_t s);
hipError_t launch_gather_f32(float* dst, const uint16_t* const* eltptr, int n, hipStream_t s);
hipError_t launch_rope_table(float2* rope, int cap, int half, double base, hipStream_t s);
hipError_t launch_set_state(int32_t* len, int32_t* next, int seq, int new_len, int new_next, int which,
                            hipStream_t s);
// Device-resident speculative round (drafter cache d, verifier cache v, both of B sequences
// in step): the bookkeeping kernels that run between the captured passes.
enum RoundPhase { kRoundBegin = 0, kRoundStage = 1, kRoundReconcile = 2, kRoundFinish = 3 };
struct RoundArgs {
  Stage* dstage;           // drafter staging block (draft-step flags, step counters)
  Stage* vstage;           // verifier staging block (k and the drafts)
  int32_t *dlen, *dnext;   // drafter length / pending token
  const int32_t* vlen;     // verifier length / pending token
  const int32_t* vnext;
  const int32_t* dout;     // drafter's step outputs [B][kMaxDraftSteps]
  const int32_t* vres;     // verifier results: accepted[B], target[B][vT]
  int32_t* scratch;        // [B] verifier length before the verify, [B] catch-up flag
  int B, k, vkmax, vT;
};
hipError_t launch_round(const RoundArgs& r, int phase, hipStream_t s);
hipError_t launch_zero(int* p, size_t n, hipStream_t s);
hipError_t launch_stage_device(Stage* stage, const int32_t* draft, const int32_t* k, int B, int kmax,
                               int flags, hipStream_t s);
hipError_t launch_copy_kv(uint16_t* pool, uint16_t* src, long pool_layer_stride, int nkv, int cap,
                          int dh, int n_layers, int n_pos, int src_positions, int to_pool, hipStream_t s);
// State snapshot of every sequence: (length, pending token) and the K/V rows at positions
// [length, length+T) of every layer, the rows one pass of T positions writes.
struct SnapArgs {
  uint16_t *kpool, *vpool;   // [layer][seq][kv head][position][dh]
  uint16_t *sk, *sv;         // [layer][seq][kv head][T][dh]
  int32_t *len, *next;       // live state [B]
  int32_t *slen, *snext;     // saved state [B]
  long layer_stride, seq_stride;
  int L, B, nkv, cap, dh, T;
};
hipError_t launch_snapshot(const SnapArgs& a, int save, hipStream_t s);

}  // namespace sf
