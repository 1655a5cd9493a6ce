// C ABI: argument validation on the host, then a launch on the caller's stream.
// Every check runs before any HIP call, so every error code is reachable without a GPU.
#include <cmath>
#include <cstdint>

#include "fd_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_geom(const fd_geom* g) {
  if (!g) return FD_ERR_NULL;
  if (g->n_views < 1 || g->n_frames < 1 || g->tok_per_frame < 1 || g->prefix_len < 0 ||
      g->n_q_heads < 1 || g->n_kv_heads < 1 || g->tail_cap < 0)
    return FD_ERR_GEOM;
  if (g->n_q_heads % g->n_kv_heads != 0) return FD_ERR_GEOM;
  const int G = g->n_q_heads / g->n_kv_heads;
  if (!(G == 1 || G == 2 || G % 4 == 0)) return FD_ERR_GEOM;
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

fd::KParams make_params(const fd_geom* g, int64_t t) {
  fd::KParams p{};
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
  p.HPW = p.G < 4 ? p.G : 4;
  p.TBW = 4 / p.HPW;
  p.n_hsub = p.G / p.HPW;
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
  const fd::KParams p = make_params(g, g->n_frames - 1);
  const int n_rb = p.Hkv * p.n_hsub * p.nqb;
  return fd::align256(krot) + fd::stream_qrot_bytes(p.V * p.T, p.Hq, p.D) +
         fd::stream_tiles_bytes(0, p.P, p.T, p.V, p.F) + fd::stream_partial_bytes(n_rb, p.V, p.D);
}

size_t fd_prefill_workspace_bytes(const fd_geom* g) {
  if (check_geom(g) != FD_OK || g->in_dtype != FD_BF16) return 0;
  const fd::KParams p = make_params(g, g->n_frames - 1);
  const size_t krot = size_t(p.Hkv) * p.W * p.D * 2;
  // every segment is attended whole by one workgroup: no partials
  return fd::align256(krot) + fd::stream_qrot_bytes(p.W, p.Hq, p.D) + fd::stream_tiles_bytes(1, p.P, p.T, p.V, p.F);
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

size_t fd_verify_workspace_bytes(const fd_geom* g, int32_t blk_len) {
  if (check_geom(g) != FD_OK) return 0;
  if (blk_len < 1 || blk_len > g->tail_cap) return 0;
  const int G = g->n_q_heads / g->n_kv_heads;
  if (blk_len > 32 || fd::verify_row_blocks(G, blk_len) > fd::kVerifyMaxRowBlocks) return 0;
  const int nblk = fd::verify_blocks(g->prefix_len, g->n_views, g->n_frames, g->tok_per_frame,
                                     g->tail_cap);
  const int S = fd::verify_splits(nblk, fd::kVerifyWaves * fd::kVerifyBlocksPerWave);   // the larger count
  return fd::kVerifyWsHeader + size_t(g->n_kv_heads) * fd::verify_row_blocks(G, blk_len) * S *
                                   fd::verify_partial_words(g->head_dim) * sizeof(float);
}

int fd_verify_attn(const fd_geom* g, const void* q_blk, const void* k_blk, const void* v_blk,
                   void* k_cache, void* v_cache, int64_t newest_frame, int32_t n_tail,
                   int32_t blk_len, void* out, void* ws, size_t ws_bytes, void* hip_stream) {
  int st = check_geom(g);
  if (st != FD_OK) return st;
  if (!q_blk || !k_blk || !v_blk || !k_cache || !v_cache || !out) return FD_ERR_NULL;
  if (newest_frame < g->n_frames - 1) return FD_ERR_FRAME;
  if (n_tail < 0 || blk_len < 1 || int64_t(n_tail) + blk_len > g->tail_cap) return FD_ERR_TAIL;
  if (blk_len > 32 || fd::verify_row_blocks(g->n_q_heads / g->n_kv_heads, blk_len) > fd::kVerifyMaxRowBlocks)
    return FD_ERR_TAIL;
  if (!ws || ws_bytes < fd_verify_workspace_bytes(g, blk_len)) return FD_ERR_WORKSPACE;
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned16(ws))
    return FD_ERR_ALIGN;
  fd::KParams p = make_params(g, newest_frame);
  p.n_tail = n_tail;
  p.B = blk_len;
  p.n_rb = fd::verify_row_blocks(p.G, blk_len);
  p.nblk = fd::verify_blocks(p.P, p.V, p.F, p.T, n_tail + blk_len);
  p.n_split = fd::verify_splits(p.nblk, g->in_dtype == FD_BF16
                                            ? fd::kVerifyWavesDma * fd::kVerifyBlocksPerWaveDma
                                            : fd::kVerifyWaves * fd::kVerifyBlocksPerWave);
  return fd::launch_verify(p, g->in_dtype == FD_BF16, q_blk, k_blk, v_blk, k_cache, v_cache, out, ws,
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
    default: return "unknown status";
  }
}

}  // extern "C"
