// C ABI: argument validation on the host, then a launch on the caller's stream.
// Every check runs before any HIP call, so every error code is reachable without a GPU.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "fd_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_geom(const fd_geom* g) {
  if (!g) return FD_ERR_NULL;
  if (g->n_views < 1 || g->n_frames < 1 || g->tok_per_frame < 1 || g->prefix_len < 0 ||
      g->n_q_heads < 1 || g->n_kv_heads < 1 || g->tail_cap < 0)
    return FD_ERR_GEOM;
  if (g->n_q_heads % g->n_kv_heads != 0) return FD_ERR_GEOM;
  if (g->head_dim != 64 && g->head_dim != 128) return FD_ERR_GEOM;
  if (!std::isfinite(g->rope_theta) || !(g->rope_theta > 1.0)) return FD_ERR_GEOM;
  if (g->pos_base < 0 || g->pos_base >= (int64_t(1) << 31)) return FD_ERR_GEOM;
  const int64_t window = int64_t(g->prefix_len) +
                         int64_t(g->n_views) * g->n_frames * int64_t(g->tok_per_frame);
  const int64_t rows = window + g->tail_cap;
  if (rows * g->head_dim >= (int64_t(1) << 31)) return FD_ERR_GEOM;
  if (int64_t(g->n_views) * g->tok_per_frame * g->n_q_heads * int64_t(g->head_dim) >= (int64_t(1) << 31))
    return FD_ERR_GEOM;
  if ((g->in_dtype != FD_F32 && g->in_dtype != FD_BF16) ||
      (g->out_dtype != FD_F32 && g->out_dtype != FD_BF16))
    return FD_ERR_DTYPE;
  return FD_OK;
}

// How the streaming calls merge a view cut once, process-wide (fd_stream_merge_mode)
std::atomic<int32_t> g_merge_mode{1};

fd::KParams make_params(const fd_geom* g, int64_t t) {
  fd::KParams p{};
  p.merge_mode = g_merge_mode.load(std::memory_order_relaxed);
  p.V = g->n_views;
  p.F = g->n_frames;
  p.T = g->tok_per_frame;
  p.P = g->prefix_len;
  p.Hq = g->n_q_heads;
  p.Hkv = g->n_kv_heads;
  p.D = g->head_dim;
  p.G = p.Hq / p.Hkv;
  p.W = p.P + p.V * p.F * p.T;
  p.S_cap = p.W + g->tail_cap;
  p.s_new = int32_t(t % p.F);
  p.out_bf16 = g->out_dtype == FD_BF16;
  p.HPW = p.G <= 2 ? p.G : 4;   // G > 2 not a multiple of 4: the last head subset is ragged
  p.TBW = 4 / p.HPW;
  p.n_hsub = fd::ceil_div(p.G, p.HPW);
  p.nqb = fd::ceil_div(p.T, 32 * p.TBW);
  p.qmode = 0;   // streaming: one segment per view (its newest frame)
  p.seg0 = 0;
  p.nseg = p.V;
  p.qtok = p.T;
  p.whole = 0;
  p.pos_base = g->pos_base;
  p.t = t;
  p.sm_scale_log2 = float(1.4426950408889634 / std::sqrt(double(p.D)));
  for (int i = 0; i < p.D / 2; ++i) p.inv_freq[i] = std::pow(g->rope_theta, -2.0 * i / p.D);
  p.log2_theta = std::log2(g->rope_theta);
  return p;
}

int esize(const fd_geom* g) { return g->in_dtype == FD_BF16 ? 2 : 4; }

// Persistent key view: frames of the stream are grouped in periods of 2^24 / T frames; at newest
// frame t the view holds every window row rotated at its position + (t mod period) * T.  A frame
// row keeps that value from the call that inserted it to the end of the period (its position
// falls by T per frame while the offset grows by T), so within a period a call rotates only the
// prefix rows and the new frames; the offset stays below 2^24 positions.
int64_t view_period(const fd_geom* g) {
  const int64_t n = (int64_t(1) << 24) / g->tok_per_frame;
  return n > 1 ? n : 1;
}
int64_t view_shift(const fd_geom* g, int64_t t) { return (t % view_period(g)) * g->tok_per_frame; }

// Shared by fd_stream_attn_view and fd_stream_attn_insert_view (k_new, v_new null: no insert).
int stream_view_call(const fd_geom* g, const void* k_new, const void* v_new, const void* q_new, void* k_cache,
                     void* v_cache, int64_t t, void* k_view, int64_t view_frame, void* out, void* ws,
                     size_t ws_bytes, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!q_new || !k_cache || !v_cache || !out || !k_view) return FD_ERR_NULL;
  if (t < g->n_frames - 1) return FD_ERR_FRAME;
  if (g->pos_base + view_shift(g, t) >= (int64_t(1) << 31)) return FD_ERR_GEOM;
  if (!ws || ws_bytes < fd_stream_workspace_bytes(g)) return FD_ERR_WORKSPACE;
  if ((k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)) || !aligned16(q_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned16(ws) || !aligned16(k_view))
    return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, t);
  p.pos_base += view_shift(g, t);
  const int64_t per = view_period(g);
  p.rot_new = (view_frame >= g->n_frames - 1 && (t == view_frame || t == view_frame + 1) &&
               t / per == view_frame / per) ? 1 : 0;
  return fd::launch_stream(p, g->in_dtype == FD_BF16, q_new, k_cache, v_cache, out, ws, hip_stream, k_new, v_new,
                           k_view);
}

}  // namespace

extern "C" {

int64_t fd_cache_rows(const fd_geom* g) {
  if (check_geom(g) != FD_OK) return -1;
  return int64_t(g->prefix_len) + int64_t(g->n_views) * g->n_frames * g->tok_per_frame + g->tail_cap;
}

int fd_key_position(const fd_geom* g, int64_t newest_frame, int64_t row, int64_t* pos) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!pos) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  const int64_t P = g->prefix_len, T = g->tok_per_frame, F = g->n_frames;
  const int64_t W = P + int64_t(g->n_views) * F * T;
  if (row < 0 || row >= W + g->tail_cap) return FD_ERR_GEOM;
  if (row < P || row >= W) {
    *pos = g->pos_base + row;
    return FD_OK;
  }
  const int64_t rr = row - P;
  const int64_t v = rr / (F * T), s = (rr / T) % F, i = rr % T;
  const int64_t age = F - 1 - ((newest_frame - s) % F);
  *pos = g->pos_base + P + (v * F + age) * T + i;
  return FD_OK;
}

int fd_kv_insert_frame(const fd_geom* g, void* k_cache, void* v_cache, const void* k_new,
                       const void* v_new, int64_t frame_idx, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!k_cache || !v_cache || !k_new || !v_new) return FD_ERR_NULL;
  if (frame_idx < 0) return FD_ERR_FRAME;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, frame_idx);
  return fd::launch_insert(p, esize(g), k_cache, v_cache, k_new, v_new, int(frame_idx % g->n_frames),
                           hip_stream);
}

int fd_kv_project_insert(const fd_geom* g, const void* x_new, const void* w_kv, int32_t hidden, void* k_cache,
                         void* v_cache, int64_t frame_idx, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (g->in_dtype != FD_BF16) return FD_ERR_DTYPE;
  if (!x_new || !w_kv || !k_cache || !v_cache) return FD_ERR_NULL;
  const int64_t M = int64_t(g->n_views) * g->tok_per_frame, N = 2 * int64_t(g->n_kv_heads) * g->head_dim;
  // k in chunks of 64; 32-bit byte offsets into x and w
  if (hidden < 64 || hidden % 64 != 0 || N % 128 != 0 || M * hidden * 2 >= (int64_t(1) << 31) ||
      N * hidden * 2 >= (int64_t(1) << 31))
    return FD_ERR_GEOM;
  if (frame_idx < 0) return FD_ERR_FRAME;
  if (!aligned16(x_new) || !aligned16(w_kv) || !aligned16(k_cache) || !aligned16(v_cache)) return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, frame_idx);
  return fd::launch_kv_project(p, hidden, int(frame_idx % g->n_frames), x_new, w_kv, k_cache, v_cache, hip_stream);
}

size_t fd_stream_workspace_bytes(const fd_geom* g) {
  if (check_geom(g) != FD_OK) return 0;
  const size_t window = size_t(g->prefix_len) + size_t(g->n_views) * g->n_frames * g->tok_per_frame;
  const size_t krot = size_t(g->n_kv_heads) * window * g->head_dim * (g->in_dtype == FD_BF16 ? 2 : 4);
  if (g->in_dtype != FD_BF16) return krot;
  // rotated keys, queries, tile table, merge descriptors and tickets, partial slots (bf16 only),
  // then the rotation pass's range report
  const fd::KParams p = make_params(g, g->n_frames - 1);
  return fd::stream_report_offset(p) + fd::rope_report_bytes(fd::rope_max_workgroups(p, false));
}

size_t fd_prefill_workspace_bytes(const fd_geom* g) {
  if (check_geom(g) != FD_OK || g->in_dtype != FD_BF16) return 0;
  // rotated keys, every window row's queries, tile table (every segment is attended whole by one
  // workgroup: no partials), then the rotation pass's range report
  const fd::KParams p = make_params(g, g->n_frames - 1);
  return fd::prefill_report_offset(p) + fd::rope_report_bytes(fd::rope_max_workgroups(p, true));
}

namespace {

// The rotation pass's range report at byte `off` of a bf16 workspace: copied to the host on the
// caller's stream (after the work queued before it), then the waves that left the fp16 range
// counted.
int read_rope_report(const void* ws, size_t off, size_t bytes, void* hip_stream) {
  std::vector<unsigned char> h(bytes);
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (hipMemcpyAsync(h.data(), static_cast<const unsigned char*>(ws) + off, bytes, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return FD_ERR_HIP;
  int32_t head[2];
  std::memcpy(head, h.data(), sizeof(head));
  if (head[0] != fd::kRopeReportMagic || head[1] < 0 || size_t(fd::kRopeReportHeader) + size_t(head[1]) > bytes)
    return FD_ERR_WORKSPACE;   // no bf16 call of this kind has completed on the workspace
  int n = 0;
  for (int32_t i = 0; i < head[1]; ++i) n += h[fd::kRopeReportHeader + i] != 0;
  return n;
}

}  // namespace

int fd_stream_overflow(const fd_geom* g, const void* ws, size_t ws_bytes, void* hip_stream) {
  const int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!ws) return FD_ERR_NULL;
  if (ws_bytes < fd_stream_workspace_bytes(g)) return FD_ERR_WORKSPACE;
  if (g->in_dtype != FD_BF16) return 0;   // fp32 operands: no fp16 rounding
  const fd::KParams p = make_params(g, g->n_frames - 1);
  return read_rope_report(ws, fd::stream_report_offset(p), fd::rope_report_bytes(fd::rope_max_workgroups(p, false)),
                          hip_stream);
}

int fd_prefill_overflow(const fd_geom* g, const void* ws, size_t ws_bytes, void* hip_stream) {
  const int st = check_geom(g);
  if (st != FD_OK) return st;
  if (g->in_dtype != FD_BF16) return FD_ERR_DTYPE;
  if (!ws) return FD_ERR_NULL;
  if (ws_bytes < fd_prefill_workspace_bytes(g)) return FD_ERR_WORKSPACE;
  const fd::KParams p = make_params(g, g->n_frames - 1);
  return read_rope_report(ws, fd::prefill_report_offset(p), fd::rope_report_bytes(fd::rope_max_workgroups(p, true)),
                          hip_stream);
}

int fd_prefill_attn(const fd_geom* g, const void* q_win, const void* k_cache, const void* v_cache,
                    int64_t newest_frame, void* out, void* ws, size_t ws_bytes, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (g->in_dtype != FD_BF16) return FD_ERR_DTYPE;
  if (!q_win || !k_cache || !v_cache || !out) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  if (!ws || ws_bytes < fd_prefill_workspace_bytes(g)) return FD_ERR_WORKSPACE;
  if (!aligned16(q_win) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(ws))
    return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, newest_frame);
  p.qmode = 1;
  return fd::launch_prefill(p, q_win, k_cache, v_cache, out, ws, hip_stream);
}

int fd_stream_attn(const fd_geom* g, const void* q_new, const void* k_cache, const void* v_cache,
                   int64_t newest_frame, void* out, void* ws, size_t ws_bytes, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!q_new || !k_cache || !v_cache || !out) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  if (!ws || ws_bytes < fd_stream_workspace_bytes(g)) return FD_ERR_WORKSPACE;
  if (!aligned16(q_new) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(ws))
    return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, newest_frame);
  return fd::launch_stream(p, g->in_dtype == FD_BF16, q_new, k_cache, v_cache, out, ws, hip_stream);
}

int fd_stream_attn_insert(const fd_geom* g, const void* k_new, const void* v_new, const void* q_new,
                          void* k_cache, void* v_cache, int64_t newest_frame, void* out, void* ws,
                          size_t ws_bytes, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!k_new || !v_new || !q_new || !k_cache || !v_cache || !out) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  if (!ws || ws_bytes < fd_stream_workspace_bytes(g)) return FD_ERR_WORKSPACE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned16(ws))
    return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, newest_frame);
  return fd::launch_stream(p, g->in_dtype == FD_BF16, q_new, k_cache, v_cache, out, ws, hip_stream, k_new,
                           v_new);
}

int32_t fd_stream_merge_mode(int32_t mode) {
  if (mode < 0 || mode > 2) return g_merge_mode.load(std::memory_order_relaxed);
  return g_merge_mode.exchange(mode, std::memory_order_relaxed);
}

int64_t fd_view_shift(const fd_geom* g, int64_t newest_frame) {
  if (check_geom(g) != FD_OK || newest_frame < 0) return -1;
  return view_shift(g, newest_frame);
}

int fd_stream_attn_view(const fd_geom* g, const void* q_new, const void* k_cache, const void* v_cache,
                        int64_t newest_frame, void* k_view, int64_t view_frame, void* out, void* ws,
                        size_t ws_bytes, void* hip_stream) {
  return stream_view_call(g, nullptr, nullptr, q_new, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                          newest_frame, k_view, view_frame, out, ws, ws_bytes, hip_stream);
}

int fd_stream_attn_insert_view(const fd_geom* g, const void* k_new, const void* v_new, const void* q_new,
                               void* k_cache, void* v_cache, int64_t newest_frame, void* k_view,
                               int64_t view_frame, void* out, void* ws, size_t ws_bytes, void* hip_stream) {
  if (!k_new || !v_new) return FD_ERR_NULL;
  return stream_view_call(g, k_new, v_new, q_new, k_cache, v_cache, newest_frame, k_view, view_frame, out, ws,
                          ws_bytes, hip_stream);
}

size_t fd_verify_workspace_bytes(const fd_geom* g, int32_t blk_len) {
  if (check_geom(g) != FD_OK) return 0;
  if (blk_len < 1 || blk_len > g->tail_cap) return 0;
  const int G = g->n_q_heads / g->n_kv_heads;
  if (blk_len > 32 || fd::verify_row_blocks(G, blk_len) > fd::kVerifyMaxRowBlocks) return 0;
  // partial slots per (kv head, row block) for the longest tail: split-KV workgroups of the fp32
  // kernel; window and tail units of the bf16 kernel
  const int S = g->in_dtype == FD_BF16
                    ? fd::verify_dma_slots(g->prefix_len, g->n_views, g->n_frames, g->tok_per_frame, g->tail_cap)
                    : fd::verify_splits(fd::verify_blocks(g->prefix_len, g->n_views, g->n_frames,
                                                          g->tok_per_frame, g->tail_cap),
                                        fd::kVerifyWaves * fd::kVerifyBlocksPerWave);
  const size_t pw = g->in_dtype == FD_BF16 ? fd::verify_dma_partial_words(g->head_dim)
                                           : fd::verify_partial_words(g->head_dim);
  return fd::kVerifyWsHeader + size_t(g->n_kv_heads) * fd::verify_row_blocks(G, blk_len) * S * pw * sizeof(float);
}

size_t fd_verify_batched_workspace_bytes(const fd_geom* g, int32_t n_drafts, int32_t blk_len) {
  if (check_geom(g) != FD_OK || g->in_dtype != FD_BF16) return 0;
  if (n_drafts < 1 || n_drafts > fd::kVerifyMaxDrafts || blk_len < 1 || blk_len > 32 || blk_len > g->tail_cap)
    return 0;
  const int G = g->n_q_heads / g->n_kv_heads;
  if (fd::verify_row_blocks(G, blk_len) > fd::kVerifyMaxRowBlocks) return 0;
  // every draft's tail fits in tail_cap: its slots are at most those of a tail_cap-row tail
  const int S = fd::verify_dma_slots(g->prefix_len, g->n_views, g->n_frames, g->tok_per_frame, g->tail_cap);
  return fd::kVerifyWsHeader + size_t(g->n_kv_heads) * n_drafts * fd::verify_row_blocks(G, blk_len) *
                                                   S * fd::verify_dma_partial_words(g->head_dim) * sizeof(float);
}

namespace {

// Checks shared by the verify entry points (everything but the workspace), in the order the
// header documents.
int check_verify_args(const fd_geom* g, const void* q_blk, const void* k_blk, const void* v_blk,
                      const void* k_cache, const void* v_cache, int64_t newest_frame, int32_t n_tail,
                      int32_t blk_len, const void* out) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!q_blk || !k_blk || !v_blk || !k_cache || !v_cache || !out) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  if (n_tail < 0 || blk_len < 1 || int64_t(n_tail) + blk_len > g->tail_cap) return FD_ERR_TAIL;
  if (blk_len > 32 || fd::verify_row_blocks(g->n_q_heads / g->n_kv_heads, blk_len) > fd::kVerifyMaxRowBlocks)
    return FD_ERR_TAIL;
  return FD_OK;
}

bool verify_aligned(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_cache,
                    const void* v_cache, const void* out) {
  return aligned16(q_blk) && aligned16(k_blk) && aligned16(v_blk) && aligned16(k_cache) && aligned16(v_cache) &&
         aligned16(out);
}

int launch_verify_checked(const fd_geom* g, const void* q_blk, const void* k_blk, const void* v_blk, void* k_cache,
                          void* v_cache, int64_t newest_frame, int32_t n_tail, int32_t blk_len, void* out,
                          void* ws, void* hip_stream) {
  fd::KParams p = make_params(g, newest_frame);
  p.n_tail = n_tail;
  p.B = blk_len;
  p.n_drafts = 1;
  p.tail_stride = 0;
  p.n_tails[0] = n_tail;
  p.nrb_d = fd::verify_row_blocks(p.G, blk_len);
  p.n_rb = p.nrb_d;
  p.nblk = fd::verify_blocks(p.P, p.V, p.F, p.T, n_tail + blk_len);
  if (g->in_dtype == FD_BF16) {
    p.n_ws = fd::verify_window_units(p.P, p.V, p.F, p.T);
    p.n_ts = fd::verify_tail_units(n_tail + blk_len);
    p.n_split = p.n_ws + p.n_ts;
  } else {
    p.n_split = fd::verify_splits(p.nblk, fd::kVerifyWaves * fd::kVerifyBlocksPerWave);
  }
  return fd::launch_verify(p, g->in_dtype == FD_BF16, q_blk, k_blk, v_blk, k_cache, v_cache, out, ws,
                           hip_stream);
}

}  // namespace

int fd_verify_attn(const fd_geom* g, const void* q_blk, const void* k_blk, const void* v_blk,
                   void* k_cache, void* v_cache, int64_t newest_frame, int32_t n_tail,
                   int32_t blk_len, void* out, void* ws, size_t ws_bytes, void* hip_stream) {
  const int st = check_verify_args(g, q_blk, k_blk, v_blk, k_cache, v_cache, newest_frame, n_tail, blk_len, out);
  if (st != FD_OK) return st;
  if (!ws || ws_bytes < fd_verify_workspace_bytes(g, blk_len)) return FD_ERR_WORKSPACE;
  if (!verify_aligned(q_blk, k_blk, v_blk, k_cache, v_cache, out) || !aligned16(ws)) return FD_ERR_ALIGN;
  return launch_verify_checked(g, q_blk, k_blk, v_blk, k_cache, v_cache, newest_frame, n_tail, blk_len, out, ws,
                               hip_stream);
}

int fd_verify_attn_batched(const fd_geom* g, int32_t n_drafts, const void* k_view, const void* q_blk,
                           const void* k_blk, const void* v_blk, void* k_cache, void* v_cache,
                           int64_t newest_frame, const int32_t* n_tails, int32_t tail_stride,
                           int32_t blk_len, void* out, void* ws, size_t ws_bytes, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (g->in_dtype != FD_BF16) return FD_ERR_DTYPE;
  if (!q_blk || !k_blk || !v_blk || !k_cache || !v_cache || !out || !n_tails) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  if (n_drafts < 1 || n_drafts > fd::kVerifyMaxDrafts || blk_len < 1 || blk_len > 32) return FD_ERR_TAIL;
  const int G = g->n_q_heads / g->n_kv_heads;
  if (fd::verify_row_blocks(G, blk_len) > fd::kVerifyMaxRowBlocks) return FD_ERR_TAIL;
  // draft d's rows W + d*tail_stride + [0, n_tails[d] + blk_len) inside the tail, without overlap
  for (int d = 0; d < n_drafts; ++d) {
    const int64_t need = int64_t(n_tails[d]) + blk_len;
    if (n_tails[d] < 0) return FD_ERR_TAIL;
    if (d + 1 < n_drafts && need > tail_stride) return FD_ERR_TAIL;
    if (int64_t(d) * (n_drafts > 1 ? tail_stride : 0) + need > g->tail_cap) return FD_ERR_TAIL;
  }
  if (n_drafts > 1 && tail_stride < 1) return FD_ERR_TAIL;
  if (!ws || ws_bytes < fd_verify_batched_workspace_bytes(g, n_drafts, blk_len)) return FD_ERR_WORKSPACE;
  if (!verify_aligned(q_blk, k_blk, v_blk, k_cache, v_cache, out) || !aligned16(ws) || !aligned16(k_view))
    return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, newest_frame);
  p.B = blk_len;
  p.n_drafts = n_drafts;
  p.tail_stride = n_drafts > 1 ? tail_stride : 0;
  int maxtail = 0;
  for (int d = 0; d < n_drafts; ++d) {
    p.n_tails[d] = n_tails[d];
    maxtail = n_tails[d] > maxtail ? n_tails[d] : maxtail;
  }
  p.n_tail = n_tails[0];
  p.nrb_d = fd::verify_row_blocks(p.G, blk_len);
  p.n_rb = n_drafts * p.nrb_d;
  p.nblk = fd::verify_blocks(p.P, p.V, p.F, p.T, maxtail + blk_len);
  p.n_ws = fd::verify_window_units(p.P, p.V, p.F, p.T);
  p.n_ts = fd::verify_tail_units(maxtail + blk_len);
  p.n_split = p.n_ws + p.n_ts;
  return fd::launch_verify(p, 1, q_blk, k_blk, v_blk, k_cache, v_cache, out, ws, hip_stream, k_view);
}

int fd_rotate_window(const fd_geom* g, const void* k_cache, int64_t newest_frame, void* k_view, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!k_cache || !k_view) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  if (!aligned16(k_cache) || !aligned16(k_view)) return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, newest_frame);
  return fd::launch_rotate_window(p, g->in_dtype == FD_BF16, k_cache, k_view, hip_stream);
}

int fd_verify_attn_noalloc(const fd_geom* g, const void* q_blk, const void* k_blk, const void* v_blk,
                           void* k_cache, void* v_cache, int64_t newest_frame, int32_t n_tail,
                           int32_t blk_len, void* out, void* hip_stream) {
  int st = check_verify_args(g, q_blk, k_blk, v_blk, k_cache, v_cache, newest_frame, n_tail, blk_len, out);
  if (st != FD_OK) return st;
  if (fd_verify_workspace_bytes(g, blk_len) > fd::kVerifyScratchBytes) return FD_ERR_SCRATCH;
  if (!verify_aligned(q_blk, k_blk, v_blk, k_cache, v_cache, out)) return FD_ERR_ALIGN;
  void* ws = fd::verify_scratch(&st);   // this device's static scratch array (no allocation)
  if (!ws) return st;
  return launch_verify_checked(g, q_blk, k_blk, v_blk, k_cache, v_cache, newest_frame, n_tail, blk_len, out, ws,
                               hip_stream);
}

const char* fd_status_str(int status) {
  switch (status) {
    case FD_OK: return "ok";
    case FD_ERR_NULL: return "null pointer";
    case FD_ERR_GEOM: return "invalid geometry";
    case FD_ERR_DTYPE: return "invalid dtype";
    case FD_ERR_FRAME: return "invalid frame index (window not full)";
    case FD_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FD_ERR_TAIL: return "invalid tail / block length";
    case FD_ERR_WORKSPACE: return "workspace missing or too small";
    case FD_ERR_HIP: return "HIP launch failed";
    case FD_ERR_SCRATCH: return "problem larger than the static scratch of fd_verify_attn_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
