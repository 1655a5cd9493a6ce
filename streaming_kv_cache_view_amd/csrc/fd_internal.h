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
constexpr int kVerifyWavesDma = 5;          // bf16 path (5: 31 splits x 8 kv heads at config 4, about one workgroup per CU)
constexpr int kVerifyBlocksPerWaveDma = 1;

// Everything a kernel needs about one call, passed by value as a kernel argument.
struct KParams {
  int32_t V, F, T, P, Hq, Hkv, D, G;
  int32_t W;          // window rows P + V*F*T
  int32_t S_cap;      // cache rows per head
  int32_t s_new;      // slot of the newest frame: t mod F
  int32_t out_bf16;   // 1 -> bf16 output, 0 -> fp32
  // streaming kernel work decomposition
  int32_t HPW;        // query heads per workgroup (min(G, 4))
  int32_t TBW;        // 32-token query blocks per workgroup (4 / HPW)
  int32_t n_hsub;     // G / HPW
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
  // verify
  int32_t n_tail, B, nblk, n_split;
  int32_t n_rb;       // 32-row blocks of the G*B verify query rows
  int64_t pos_base;
  int64_t t;          // newest frame
  float sm_scale_log2;  // log2(e) / sqrt(D)
  float pad1;
  double log2_theta;    // log2(rope_theta): frequencies computed in-kernel without a memory load
  double inv_freq[kMaxHalf];  // theta^(-2i/D), fp64
};

// Verify split bookkeeping shared by host and kernels.
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int verify_blocks(int P, int V, int F, int T, int tail_rows) {
  return ceil_div(P, kVerifyBlock) + V * F * ceil_div(T, kVerifyBlock) + ceil_div(tail_rows, kVerifyBlock);
}
// splits per kv head: each workgroup covers blocks_per_wg key blocks
inline int verify_splits(int nblk, int blocks_per_wg) { return ceil_div(nblk, blocks_per_wg); }
// fp32 words of one (kv head, split) partial: O[32][D], m[32], l[32]
constexpr size_t verify_partial_words(int D) { return (size_t)32 * D + 64; }
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
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
constexpr size_t stream_partial_words(int D) { return (size_t)128 * D + 256; }   // O[128][D], (m, l)[128]
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
inline size_t stream_partial_bytes(int n_rb, int nseg, int D) {
  return size_t(n_rb) * nseg * 2 * stream_partial_words(D) * sizeof(float);
}

int launch_insert(const KParams& p, int esize, void* kc, void* vc, const void* kn, const void* vn,
                  int slot, void* stream);
// kn / vn non-null: the new frames' K and V ([V][T][Hkv][D]) are inserted into ring slot
// s_new by the same launch sequence (the rotation pass), before the attention reads them
int launch_stream(const KParams& p, int in_bf16, const void* q, const void* kc, const void* vc,
                  void* out, void* ws, void* stream, const void* kn = nullptr, const void* vn = nullptr);
int launch_prefill(const KParams& p, const void* q, const void* kc, const void* vc, void* out, void* ws,
                   void* stream);
int launch_kv_project(const KParams& p, int hidden, int slot, const void* x, const void* w, void* kc, void* vc,
                      void* stream);
int launch_verify(const KParams& p, int in_bf16, const void* qb, const void* kb, const void* vb,
                  void* kc, void* vc, void* out, void* ws, void* stream);

}  // namespace fd
