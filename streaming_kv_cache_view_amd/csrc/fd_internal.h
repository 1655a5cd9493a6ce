// Internal interface between the C-ABI layer (fd_api.cpp) and the kernels (fd_kernels.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fdattn.h"

namespace fd {

constexpr int kMaxHalf = 64;      // D/2 for D = 128
constexpr int kTileKeys = 64;     // keys per K/V tile in the streaming kernel
constexpr int kVerifyBlock = 32;  // keys per MFMA block in the verify kernel
constexpr int kVerifyWaves = 4;             // waves per verify workgroup, fp32 path
constexpr int kVerifyBlocksPerWave = 1;
constexpr int kVerifyWavesDma = 5;          // bf16 path: waves per workgroup, one 32-key block each
                                            // (31 units x 8 kv heads at the backbone shapes: every CU)
constexpr int kVerifyMaxDrafts = 8;         // draft blocks verified by one batched call

// Everything a kernel needs about one call, passed by value as a kernel argument.
struct KParams {
  int32_t V, F, T, P, Hq, Hkv, D, G;
  int32_t W;          // window rows P + V*F*T
  int32_t S_cap;      // cache rows per head
  int32_t s_new;      // slot of the newest frame: t mod F
  int32_t out_bf16;   // 1 -> bf16 output, 0 -> fp32
  // streaming kernel work decomposition
  int32_t HPW;        // query heads per workgroup: G if G <= 2, else 4
  int32_t TBW;        // 32-token query blocks per workgroup (4 / HPW)
  int32_t n_hsub;     // ceil(G / HPW): with G > 2 not a multiple of 4 the last subset has G mod 4
                      // heads, the rows of the others idle
  int32_t nqb;        // ceil(qtok / (32*TBW))
  // query segments of the bf16 attention kernel: a segment is the query tokens of one frame
  // (or of the prefix), with one key-tile sequence
  int32_t qmode;      // 0 streaming: segment v = view v's newest frame (queries [V*T][Hq][D]);
                      // 1 full window: segment v*F + j = view v's frame of age j, segment V*F =
                      //   the prefix (queries [W][Hq][D] in cache-row order)
  int32_t seg0;       // first segment of this launch
  int32_t nseg;       // segments (and chunks) per row block of this launch
  int32_t qtok;       // query tokens per segment of this launch (T, or P for the prefix)
  int32_t whole;      // 0: the row block's segments laid end to end and cut into nseg equal
                      //    chunks (split segments merged by a second kernel);
                      // 1: chunk c is segment nseg-1-c whole (no split, no merge)
  // verify.  A call verifies n_drafts draft blocks of B tokens over one window; draft d's
  // reasoning rows and block rows sit in cache rows W + d*tail_stride + [0, n_tails[d] + B).
  int32_t rot_new;    // rotation pass: 1 -> only the prefix rows and the newest slot of every view
                      //   (a persistent key view whose older frames were rotated by earlier calls)
  int32_t merge_mode;   // streaming attention, a view cut once (split between two workgroups): 1 ->
                        //   merged by whichever piece finishes second; 0 -> by the merge kernel;
                        //   2 -> as 1 with the second piece made to finish second (tests)
  int32_t n_tail, B, nblk, n_split;   // n_tail: draft 0's; nblk: key blocks of the longest key list;
                                      // n_split: partial slots per (kv head, row block)
  int32_t n_ws, n_ts;   // bf16 path: units over the window's blocks, and per draft over its tail
  int32_t n_rb;       // 32-row blocks of every draft's G*B query rows: n_drafts * nrb_d
  int32_t nrb_d;      // 32-row blocks of one draft's G*B query rows
  int32_t n_drafts;
  int32_t tail_stride;
  int32_t n_tails[kVerifyMaxDrafts];
  int64_t pos_base;
  int64_t t;          // newest frame
  float sm_scale_log2;  // log2(e) / sqrt(D)
  float pad1;
  double log2_theta;    // log2(rope_theta): frequencies computed in-kernel without a memory load
  double inv_freq[kMaxHalf];  // theta^(-2i/D), fp64
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Verify split bookkeeping shared by host and kernels.  A row block's keys are the window's
// 32-key blocks (inside the prefix and inside each frame slot: contiguous positions) followed by
// the 32-key blocks of its own draft's tail rows.
constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }
constexpr int verify_window_blocks(int P, int V, int F, int T) {
  return ceil_div(P, kVerifyBlock) + V * F * ceil_div(T, kVerifyBlock);
}
inline int verify_blocks(int P, int V, int F, int T, int tail_rows) {
  return verify_window_blocks(P, V, F, T) + ceil_div(tail_rows, kVerifyBlock);
}
// splits per kv head: each workgroup covers blocks_per_wg key blocks
inline int verify_splits(int nblk, int blocks_per_wg) { return ceil_div(nblk, blocks_per_wg); }
// fp32 words of one (kv head, split) partial: O[32][D], m[32], l[32]
constexpr size_t verify_partial_words(int D) { return (size_t)32 * D + 64; }
// bf16 path: O^T in fp16 (32*D halves, the split kernel's accumulator order), each (row, 32-wide
// d slice) scaled by a power of two; then fp32 (m, l)[32] and the inverse scales [D/32][32]
constexpr size_t verify_dma_partial_words(int D) { return (size_t)16 * D + 64 + D; }
// bf16 path: key blocks per workgroup ("unit"); units over the window's blocks; units over one
// draft's tail of tail_rows rows (reasoning rows + block rows); partial slots per (kv head, row
// block) with tails up to tail_rows: one per unit
constexpr int kVerifyUnitBlocks = kVerifyWavesDma;
constexpr int verify_window_units(int P, int V, int F, int T) {
  return ceil_div(verify_window_blocks(P, V, F, T), kVerifyUnitBlocks);
}
constexpr int verify_tail_units(int tail_rows) { return ceil_div(ceil_div(tail_rows, kVerifyBlock), kVerifyUnitBlocks); }
constexpr int verify_dma_slots(int P, int V, int F, int T, int tail_rows) {
  return verify_window_units(P, V, F, T) + verify_tail_units(tail_rows);
}
// 32-row blocks of the G*B query rows of one kv head (at most kVerifyMaxRowBlocks)
constexpr int kVerifyMaxRowBlocks = 4;
inline int verify_row_blocks(int G, int B) { return ceil_div(G * B, 32); }
constexpr size_t kVerifyWsHeader = 256;

// Streaming kernel (bf16 path) work split.  A row block is the 128 query rows of one
// (kv head, head subset, token block); its views' tile sequences are laid end to end (longest
// view, shortest, second longest, ...) and cut into V equal chunks, one workgroup each.  A
// view cut between chunks leaves one (m, l, O) partial per piece, merged by a second kernel;
// the workspace holds, after the rotated keys and queries, two partial slots per (row block,
// chunk): a chunk's first job may continue a view, its last may be continued.
// A slot: O[128][D] in fp16 (each row scaled by a power of two), then (m, l, 1/scale, 0) in
// fp32 per row.
constexpr size_t stream_partial_words(int D) { return (size_t)64 * D + 512; }
// rotated, scaled queries (fp16, [rows][Hq][D]) after the rotated keys: rows = V*T (streaming)
// or W (full window)
inline size_t stream_qrot_bytes(int rows, int Hq, int D) { return align256(size_t(rows) * Hq * D * 2); }
// tile table of the attention kernel: an int2 per tile of every segment's key sequence (the
// diagonal at full length), between the queries and the partials.  Segment of frame age j of
// view v: prefix, the v*F + j earlier frames, the diagonal; the prefix segment: its tiles.
inline size_t stream_tiles_bytes(int qmode, int P, int T, int V, int F) {
  const size_t nP = (size_t(P) + 63) / 64, tps = (size_t(T) + 63) / 64;
  size_t n = 0;
  if (qmode == 0) {
    for (int v = 0; v < V; ++v) n += nP + (size_t(v) * F + F - 1) * tps + tps;
  } else {
    for (int sg = 0; sg < V * F; ++sg) n += nP + size_t(sg) * tps + tps;
    n += nP;
  }
  return align256(n * 8);
}
// merge descriptors of a streaming call (after the tile table): an int4 per (32*TBW-token
// block, chunk boundary)
inline size_t stream_merge_desc_bytes(int nqb, int V) { return align256(size_t(nqb) * (V > 1 ? V - 1 : 0) * 16); }
// merge tickets of a streaming call (after the descriptors): a counter per (row block, chunk
// boundary) taken by the two pieces of the view the boundary cuts once
inline size_t stream_flags_bytes(int n_rb, int V) { return V > 1 ? align256(size_t(n_rb) * V * 4) : 0; }
inline size_t stream_partial_bytes(int n_rb, int nseg, int D) {
  return size_t(n_rb) * nseg * 2 * stream_partial_words(D) * sizeof(float);
}

// Range report of the rotation pass (bf16 streaming and prefill workspaces, after everything
// else): int32 kRopeReportMagic, int32 slot count n of the last launch, 8 bytes unused, then one
// byte per wave of that launch (4 per workgroup), nonzero if a rotated operand the wave rounded
// to fp16 reached |x| >= 65520 (fd_stream_overflow, fd_prefill_overflow).
constexpr int32_t kRopeReportMagic = 0x564f4446;
constexpr int kRopeReportHeader = 16;
inline size_t rope_report_bytes(int max_workgroups) { return align256(kRopeReportHeader + size_t(max_workgroups) * 4); }
// workgroups of the largest rotation pass a streaming (prefill: full-window) call launches, and
// the byte offset of the report in the bf16 workspace
int rope_max_workgroups(const KParams& p, bool prefill);
size_t stream_report_offset(const KParams& p);
size_t prefill_report_offset(const KParams& p);

// Static device scratch of fd_verify_attn_noalloc (a file-scope __device__ array, one copy per
// GPU, held until the process ends): the verify workspace of any call it accepts.
constexpr size_t kVerifyScratchBytes = FD_VERIFY_SCRATCH_BYTES;
// This device's address of that array (looked up once per device with hipGetSymbolAddress);
// nullptr with *status = FD_ERR_HIP if the lookup fails.
void* verify_scratch(int* status);

int launch_insert(const KParams& p, int esize, void* kc, void* vc, const void* kn, const void* vn,
                  int slot, void* stream);
// kn / vn non-null: the new frames' K and V ([V][T][Hkv][D]) are inserted into ring slot
// s_new by the same launch sequence (the rotation pass), before the attention reads them
// kview non-null: the rotated keys go to (and are read from) the caller's persistent view
// [Hkv][W][D] instead of the workspace; with p.rot_new only the prefix and the newest slot's rows
// are rotated into it, the older frames' rows being kept from earlier calls
int launch_stream(const KParams& p, int in_bf16, const void* q, const void* kc, const void* vc,
                  void* out, void* ws, void* stream, const void* kn = nullptr, const void* vn = nullptr,
                  void* kview = nullptr);
int launch_prefill(const KParams& p, const void* q, const void* kc, const void* vc, void* out, void* ws,
                   void* stream);
int launch_kv_project(const KParams& p, int hidden, int slot, const void* x, const void* w, void* kc, void* vc,
                      void* stream);
// kview non-null (bf16 only): the window's keys already rotated at their positions, fp16
// [Hkv][W][D] (the streaming calls' workspace start, or launch_rotate_window), read instead of
// rotating the window's keys in registers
int launch_verify(const KParams& p, int in_bf16, const void* qb, const void* kb, const void* vb,
                  void* kc, void* vc, void* out, void* ws, void* stream, const void* kview = nullptr);
// The rotation pass alone (keys only): kview [Hkv][W][D] of the QK^T operand type
int launch_rotate_window(const KParams& p, int in_bf16, const void* kc, void* kview, void* stream);

}  // namespace fd
