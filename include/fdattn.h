/*
 * fdattn.h -- C ABI of the MI355X (gfx950) streaming-prefill attention library.
 *
 * The library implements the attention hot path of FlashDrive's streaming
 * inference:
 *   - a new window prefills only the newest frame of every camera view and
 *     reuses the K/V of the earlier frames (FlashDrive README, technique list,
 *     "Streaming inference"; FlashDrive technical summary, Methodology
 *     section 1, "Algorithmic Shortcut");
 *   - the token order is view-major and the new frame is placed at the end of
 *     its own view's segment; a streaming mask keeps cross-view causality
 *     (technical summary, Methodology section 1, "Token Layout");
 *   - keys are cached before rotary embedding and rotated on the fly at the
 *     position they hold in the current window (technical summary,
 *     Methodology section 1, "Positional Encoding");
 *   - the target model verifies an 8-token draft block in one forward pass
 *     (README technique list, "Speculative reasoning"; technical summary,
 *     Methodology section 2).
 *
 * Conventions shared by every call
 * --------------------------------
 *   - Every pointer argument except `g` is a DEVICE pointer on the current
 *     HIP device, 16-byte aligned.  The caller owns every buffer (caches,
 *     inputs, outputs, workspace); the library allocates nothing and keeps no
 *     state between calls (one exception: the static scratch array behind
 *     fd_verify_attn_noalloc), so calls on different streams with disjoint
 *     buffers may run concurrently.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t, NULL = default
 *     stream), like any kernel launch.
 *   - Validation runs on the host before anything is enqueued; on error the
 *     call returns a negative fd_status and has no effect.  A failed launch
 *     returns FD_ERR_HIP.
 *   - One call handles one layer; a multi-layer model loops over layers.
 *
 * Geometry and the physical K/V cache (one layer)
 * -----------------------------------------------
 *   N       = P + V*F*T           window rows (keys) per head
 *   S_cap   = N + tail_cap        cache rows per head (fd_cache_rows)
 *   k_cache, v_cache : [Hkv][S_cap][D] of in_dtype, row-major
 *     rows [0, P)                      text prefix, written by the caller
 *     rows P + (v*F + s)*T + i         token i of the frame held in slot s of view v
 *     rows N + r, r < tail_cap         reasoning tokens then the verify block
 *   Frame g of a view lives in slot g mod F (fd_kv_insert_frame).  At newest
 *   frame t, slot s holds frame t - ((t - s) mod F); its age inside the view
 *   is j = F-1 - ((t - s) mod F), and its token i sits at logical position
 *       pos = pos_base + P + (v*F + j)*T + i.
 *   Prefix row i sits at pos_base + i; tail row r at pos_base + N + r.
 *   Keys are stored pre-RoPE; every kernel rotates them at these positions.
 *
 * RoPE and attention
 * ------------------
 *   Rotate-half RoPE with inverse frequency theta^(-2i/D): the pair
 *   (x[i], x[i+D/2]) is rotated by pos * theta^(-2i/D).  Query head h reads
 *   kv head h / (Hq/Hkv).  Scores are scaled by 1/sqrt(D); query position p_q
 *   sees key position p_k iff p_k <= p_q.  Accumulation is fp32 throughout.
 *   bf16 inputs: rotated K, and rotated Q scaled by log2(e)/sqrt(D), are rounded
 *   (to nearest even) to fp16 for Q K^T on the fp16 matrix cores; softmax
 *   probabilities are rounded to bf16 for P V (bf16 matrix cores, V exact).
 *   fp16 operand range: a rotated element of a stored pair (x, y) = (x[i],
 *   x[i+D/2]) has magnitude at most sqrt(x^2 + y^2), so no rotated operand
 *   overflows while every key pair has sqrt(x^2 + y^2) < 65520 (e.g. every
 *   stored key element |x| <= 46000) and every query pair has
 *   sqrt(x^2 + y^2) * log2(e)/sqrt(D) < 65520 (D = 128: |x| <= 3.6e5).  Above
 *   that an element can round to +-inf, depending on the key's or query's
 *   position: a score that becomes -inf drops its key silently, one that
 *   becomes +inf or NaN (inf * 0, inf - inf) makes the whole output row NaN.
 *   The calls run on regardless; the rotation pass of a streaming or prefill
 *   call records every operand it rounds out of the fp16 range, and
 *   fd_stream_overflow / fd_prefill_overflow report it afterwards.  (The verify
 *   calls rotate their reasoning-tail and block keys and their queries
 *   themselves and record nothing.)  fp32 inputs have no such bound.
 *   fp32 inputs: both products on the fp32 matrix cores.  Outputs are fp32
 *   unless out_dtype is FD_BF16.
 */
#ifndef FDATTN_H
#define FDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FD_F32 = 0, FD_BF16 = 1 } fd_dtype;

typedef enum {
  FD_OK = 0,
  FD_ERR_NULL = -1,       /* a required pointer is NULL                              */
  FD_ERR_GEOM = -2,       /* geometry out of range (see fd_geom)                     */
  FD_ERR_DTYPE = -3,      /* in_dtype / out_dtype not an fd_dtype                    */
  FD_ERR_FRAME = -4,      /* frame index < 0, or newest frame < F-1 (window not full) */
  FD_ERR_ALIGN = -5,      /* a device pointer is not 16-byte aligned                 */
  FD_ERR_TAIL = -6,       /* n_tail < 0, blk_len < 1, or n_tail + blk_len > tail_cap  */
  FD_ERR_WORKSPACE = -7,  /* workspace NULL or smaller than fd_verify_workspace_bytes */
  FD_ERR_HIP = -8,        /* the kernel launch failed                                */
  FD_ERR_SCRATCH = -9     /* fd_verify_attn_noalloc: the call needs more scratch than
                             its static array holds (FD_VERIFY_SCRATCH_BYTES)            */
} fd_status;

/* One layer's geometry.  Constraints checked by every call:
 *   n_views, n_frames, tok_per_frame, n_q_heads, n_kv_heads >= 1; prefix_len, tail_cap >= 0;
 *   n_q_heads % n_kv_heads == 0 (any group G = n_q_heads / n_kv_heads; the streaming
 *   calls take query heads four at a time, so with G > 2 not a multiple of 4 the last four
 *   of each kv head's group are partly idle); head_dim is 64 or 128; rope_theta finite and > 1;
 *   0 <= pos_base < 2^31; S_cap * head_dim < 2^31.                                         */
typedef struct fd_geom {
  int32_t n_views;        /* V: camera views                                  */
  int32_t n_frames;       /* F: frames per view in one window (ring slots)    */
  int32_t tok_per_frame;  /* T: tokens per frame                              */
  int32_t prefix_len;     /* P: static text-prefix tokens before the views    */
  int32_t n_q_heads;      /* Hq                                               */
  int32_t n_kv_heads;     /* Hkv                                              */
  int32_t head_dim;       /* D: 64 or 128                                     */
  int32_t tail_cap;       /* rows after the window: reasoning tokens + block  */
  double rope_theta;      /* RoPE base                                        */
  int64_t pos_base;       /* position of the window's first token (0 normally) */
  int32_t in_dtype;       /* fd_dtype of queries, keys, values and caches     */
  int32_t out_dtype;      /* fd_dtype of attention outputs                    */
} fd_geom;

/* Rows of one head's K (or V) cache: P + V*F*T + tail_cap; -1 on invalid geometry. */
int64_t fd_cache_rows(const fd_geom* g);

/* Logical position of physical cache row `row` (0 <= row < S_cap) at newest frame
 * `newest_frame`, as defined above.  Host-side helper; returns an fd_status. */
int fd_key_position(const fd_geom* g, int64_t newest_frame, int64_t row, int64_t* pos);

/* Insert the new frame of every view into its ring slot (Token Layout passage:
 * the new frame goes to the end of each view's segment, the oldest one drops out).
 *   k_new, v_new : [V][T][Hkv][D] in_dtype, pre-RoPE K and V of frame `frame_idx`.
 *   Writes k_cache/v_cache rows P + (v*F + frame_idx mod F)*T + i for every v, i, head:
 *   a bit-exact copy.  No other cache row is touched.  frame_idx >= 0.              */
int fd_kv_insert_frame(const fd_geom* g, void* k_cache, void* v_cache,
                       const void* k_new, const void* v_new,
                       int64_t frame_idx, void* hip_stream);

/* Project the new frame of every view to K and V and insert them into its ring slot, in one
 * kernel (Technical Summary, "5. System Optimizations", "Kernel Fusion": the Q, K, V
 * projections are merged into single kernels; here the K/V projection's epilogue is the
 * insert of the Token Layout passage).  bf16 inputs only.
 *   x_new  : [V*T][hidden] bf16, row v*T + i the hidden state of token i of view v's new frame.
 *   w_kv   : [2*Hkv*D][hidden] bf16, one output feature per row (as a linear layer stores
 *            it): rows [0, Hkv*D) the K projection (feature h*D + d = head h, dimension d),
 *            rows [Hkv*D, 2*Hkv*D) the V projection.
 *   Writes k_cache/v_cache rows P + (v*F + frame_idx mod F)*T + i, every head: the sums in
 *   fp32, rounded to bf16 (nearest even), pre-RoPE.  No other cache row is touched.
 *   hidden: a multiple of 64 (FD_ERR_GEOM otherwise; also when x or w exceed 2 GiB).
 *   frame_idx >= 0.                                                                      */
int fd_kv_project_insert(const fd_geom* g, const void* x_new, const void* w_kv, int32_t hidden,
                         void* k_cache, void* v_cache, int64_t frame_idx, void* hip_stream);

/* Bytes of workspace fd_stream_attn needs: the window's keys rotated at their current
 * positions, Hkv*N*D elements of fp16 (bf16 inputs) or fp32 (fp32 inputs); for bf16 inputs
 * also the new frames' queries rotated at their positions (fp16, V*T*Hq*D elements), a
 * table of the attention kernel's key tiles (8 bytes per 64-key tile), the merge kernel's
 * descriptors (16 bytes per query-token block and chunk boundary), a 4-byte merge ticket per
 * (block of 128 query rows, chunk), cleared by every call, and the partial results of
 * views whose key range is split between workgroups (fp16 O with a per-row scale and fp32
 * (m, l): about 2*V*(2*D + 16)*128 bytes per block of 128 query rows).  0 on invalid geometry.
 * The size depends on the geometry only, so one workspace serves every layer.            */
size_t fd_stream_workspace_bytes(const fd_geom* g);

/* Streaming-prefill attention of the new frame of every view (Token Layout and
 * Positional Encoding passages).
 *   q_new  : [V*T][Hq][D] in_dtype, pre-RoPE; row v*T + i is token i of view v's
 *            newest frame, which sits at position pos_base + P + (v*F + F-1)*T + i.
 *   k_cache, v_cache : as above, holding frames newest_frame-F+1 .. newest_frame in
 *            their slots (the caller inserts in order; the library does not check).
 *   out    : [V*T][Hq][D] out_dtype.
 *   ws     : device workspace of ws_bytes >= fd_stream_workspace_bytes(g); the call first
 *            rotates every window key at its shifted position into it (the cache keeps
 *            the pre-RoPE keys), then attends over it.  No initial contents required;
 *            calls that share one workspace must not overlap.  On return its first
 *            Hkv*N*D elements (fp16 for bf16 inputs, fp32 for fp32) hold the rotated window,
 *            [Hkv][N][D] in cache-row order: the k_view of fd_verify_attn_batched.
 *   Keys seen by token i of view v: the prefix, every frame of views < v, frames
 *   of view v older than the newest, and tokens <= i of view v's newest frame.
 *   newest_frame >= F-1 (full window); tail rows are not read.                      */
int fd_stream_attn(const fd_geom* g, const void* q_new,
                   const void* k_cache, const void* v_cache,
                   int64_t newest_frame, void* out, void* ws, size_t ws_bytes,
                   void* hip_stream);

/* The window step's insert and attention in one launch sequence: exactly
 * fd_kv_insert_frame(g, k_cache, v_cache, k_new, v_new, newest_frame) followed by
 * fd_stream_attn(g, q_new, k_cache, v_cache, newest_frame, out, ws, ws_bytes), with the copy
 * of the new frames done by the rotation pass that reads them anyway (Token Layout passage:
 * the new frame of each view goes to the end of its segment; Positional Encoding: keys are
 * cached pre-RoPE and rotated at their current positions), so the insert's own launch and its
 * pass over the new rows disappear.
 *   k_new, v_new : [V][T][Hkv][D] in_dtype, pre-RoPE K and V of frame newest_frame.
 *   q_new, out, ws : as for fd_stream_attn.
 *   k_cache, v_cache : hold frames newest_frame-F+1 .. newest_frame-1 in their slots; on
 *            return slot newest_frame mod F holds the new frame (bit-exact copy), and no other
 *            cache row has changed.
 *   Errors as for both calls.  newest_frame >= F-1.                                 */
int fd_stream_attn_insert(const fd_geom* g, const void* k_new, const void* v_new, const void* q_new,
                          void* k_cache, void* v_cache, int64_t newest_frame, void* out, void* ws,
                          size_t ws_bytes, void* hip_stream);

/* Streaming-prefill attention with a persistent rotated-key view (Positional Encoding
 * passage: keys cached pre-RoPE and re-encoded at their shifted positions every window).  The
 * scores depend on query and key positions only through their difference (rotary encoding:
 * R(a)^T R(b) = R(b - a)), so rotating every key and query of a window at its position plus one
 * common offset gives the attention of the shifted positions exactly, up to rounding.  With the
 * offset (newest_frame mod n) * T (n = max(1, 2^24 / T) frames, fd_view_shift), a frame's keys
 * keep their rotated value from the call that brings the frame in until the offset wraps:
 * their position falls by T per window while the offset grows by T.  A call then rotates only
 * the prefix rows (whose positions do not move) and the new frames, instead of the whole window.
 *   k_view     : caller-owned [Hkv][N][D] rotated keys (fp16 for bf16 inputs, fp32 for fp32),
 *                cache-row order, kept per layer across calls; row x holds cache row x rotated
 *                at fd_key_position(row x) + fd_view_shift(newest_frame).
 *   view_frame : the newest_frame of the last call that updated this k_view (or -1).  If it is
 *                newest_frame - 1 or newest_frame and the offset has not wrapped in between,
 *                only the prefix and the newest slot of every view are rotated into k_view;
 *                otherwise every window row is.  The caller must not have changed any other
 *                key row of the window since that call (the library does not check).  Pass
 *                newest_frame as view_frame to the next call.
 *   Other arguments, results and errors as for fd_stream_attn (fd_stream_attn_view) and
 *   fd_stream_attn_insert (fd_stream_attn_insert_view); the workspace's first Hkv*N*D
 *   elements are not used.  FD_ERR_GEOM if pos_base + fd_view_shift(newest_frame) >= 2^31.
 *   On return k_view serves fd_verify_attn_batched as its k_view for the same newest_frame
 *   when the verify's geometry has pos_base raised by fd_view_shift(g, newest_frame) (every
 *   position moves by the same amount, so the verify's scores are unchanged).           */
int fd_stream_attn_view(const fd_geom* g, const void* q_new, const void* k_cache, const void* v_cache,
                        int64_t newest_frame, void* k_view, int64_t view_frame, void* out, void* ws,
                        size_t ws_bytes, void* hip_stream);
int fd_stream_attn_insert_view(const fd_geom* g, const void* k_new, const void* v_new, const void* q_new,
                               void* k_cache, void* v_cache, int64_t newest_frame, void* k_view,
                               int64_t view_frame, void* out, void* ws, size_t ws_bytes, void* hip_stream);
/* The common position offset of a persistent key view at newest_frame (above); -1 on invalid
 * geometry or a negative frame. */
int64_t fd_view_shift(const fd_geom* g, int64_t newest_frame);

/* How the bf16 streaming calls (fd_stream_attn and its insert / view forms) merge a view whose
 * key range two workgroups share, for tests and tuning.  1 (default): by the workgroup of
 * whichever piece finishes second (a piece stores its partial and takes a ticket unless the
 * other's ticket is already there; no workgroup waits for another); 0: by a separate merge
 * kernel; 2: as 1, with the second piece's workgroup waiting a bounded time for the first
 * piece's ticket so that it is the second piece that merges (tests).  Every mode gives the same
 * bits (the work split never cuts a view twice).  Sets the mode, process-wide, for calls made
 * after it when 0 <= mode <= 2 and returns the mode in force before the call; any other value
 * (say -1) changes nothing and returns the present mode. */
int32_t fd_stream_merge_mode(int32_t mode);

/* Bytes of workspace fd_prefill_attn needs (bf16 inputs): the window's keys and every
 * window row's queries rotated (fp16) and the key-tile table.  0 on invalid geometry or
 * fp32 inputs.  The size depends on the geometry only.                              */
size_t fd_prefill_workspace_bytes(const fd_geom* g);

/* Non-streaming (cold-start) prefill: every token of the window is a query, under the same
 * mask (README technique list, "Streaming inference": streaming prefills the newest frame
 * only and reuses the rest; the first window of a stream has nothing to reuse.  Technical
 * Summary, Methodology 1, "Token Layout").
 *   q_win  : [W][Hq][D] bf16, pre-RoPE, in cache-row order: row x is the token held in cache
 *            row x (rows [0, P) the prefix; row P + (v*F + s)*T + i token i of the frame in
 *            view v's ring slot s), at the position fd_key_position gives for that row.
 *   k_cache, v_cache : as for fd_stream_attn (window at newest_frame).
 *   out    : [W][Hq][D] out_dtype, cache-row order.
 *   ws     : device workspace of ws_bytes >= fd_prefill_workspace_bytes(g); no initial
 *            contents required; calls that share one workspace must not overlap.
 *   The token in row x sees every key at a position <= its own: prefix tokens the prefix
 *   up to themselves; a token of view v's frame of age j the prefix, every frame of views
 *   < v, view v's frames older than j and its own frame up to itself.  For the newest
 *   frames this is fd_stream_attn's output.  bf16 inputs only (FD_ERR_DTYPE otherwise);
 *   newest_frame >= F-1.                                                              */
int fd_prefill_attn(const fd_geom* g, const void* q_win,
                    const void* k_cache, const void* v_cache,
                    int64_t newest_frame, void* out, void* ws, size_t ws_bytes,
                    void* hip_stream);

/* Bytes of workspace fd_verify_attn needs for blocks of up to blk_len tokens
 * (any n_tail with n_tail + blk_len <= tail_cap): (m, l, O) partials per (kv head,
 * 32-row block of query rows, key split) -- for bf16 inputs O in fp16 with a per-(row, 32-wide
 * slice) scale, for fp32 inputs all fp32; 0 on invalid arguments.                  */
size_t fd_verify_workspace_bytes(const fd_geom* g, int32_t blk_len);

/* Speculative-verify attention of a draft block of blk_len tokens (README technique
 * list, "Speculative reasoning"; technical summary, Methodology section 2).
 *   q_blk  : [B][Hq][D] in_dtype, pre-RoPE; token b sits at pos_base + N + n_tail + b.
 *   k_blk, v_blk : [B][Hkv][D] in_dtype, pre-RoPE.  They are copied bit-exactly into
 *            cache rows N + n_tail + b (the tail), and attended from the inputs.
 *   k_cache, v_cache : window at newest_frame plus n_tail valid reasoning rows
 *            N .. N+n_tail-1 (written by the caller).
 *   out    : [B][Hq][D] out_dtype.  Block token b sees the whole window, all n_tail
 *            reasoning rows and block tokens <= b.
 *   ws     : device workspace of ws_bytes >= fd_verify_workspace_bytes(g, blk_len);
 *            scratch for split-KV partial results, no initial contents required.
 *            Calls that share one workspace must not overlap.
 *   Requires 1 <= blk_len <= 32, (Hq/Hkv) * blk_len <= 128 (the query rows of one kv
 *   head, in up to four 32-row blocks), n_tail >= 0, n_tail + blk_len <= tail_cap,
 *   newest_frame >= F-1.                                                            */
int fd_verify_attn(const fd_geom* g, const void* q_blk,
                   const void* k_blk, const void* v_blk,
                   void* k_cache, void* v_cache, int64_t newest_frame,
                   int32_t n_tail, int32_t blk_len,
                   void* out, void* ws, size_t ws_bytes, void* hip_stream);

/* Bytes of workspace fd_verify_attn_batched needs for n_drafts blocks of blk_len tokens (any
 * tail lengths that fit in tail_cap); 0 on invalid arguments or fp32 inputs. */
size_t fd_verify_batched_workspace_bytes(const fd_geom* g, int32_t n_drafts, int32_t blk_len);

/* Speculative verify of n_drafts independent draft blocks over one window in one launch
 * (README technique list, "Speculative reasoning"; Technical Summary, Methodology section 2:
 * a drafted block is verified in one forward; Review, "Results": the draft block-size
 * ablation).  Each draft is a separate continuation of the same window -- e.g. one per sampled
 * trajectory -- with its own reasoning rows; one launch covers every draft, so the window's
 * K and V blocks that several drafts read are served from the GPU's caches after the first.
 * bf16 inputs only (FD_ERR_DTYPE otherwise).
 *   n_drafts : 1 .. 8.
 *   k_view  : NULL, or the window's keys already rotated at their positions for newest_frame:
 *             [Hkv][N][D] fp16 in cache-row order (row x = cache row x rotated at the position
 *             fd_key_position gives it).  The streaming calls (fd_stream_attn,
 *             fd_stream_attn_insert, fd_prefill_attn) leave exactly this at the start of their
 *             workspace, valid until the workspace is reused; fd_rotate_window writes it alone.
 *             With a view the window's keys are read from it instead of being rotated again;
 *             the cache stays pre-RoPE either way.  NULL: they are rotated here.
 *   q_blk   : [n_drafts][B][Hq][D], k_blk, v_blk : [n_drafts][B][Hkv][D], pre-RoPE.
 *   n_tails : HOST array of n_drafts reasoning-row counts.  Draft d's reasoning rows are cache
 *             rows N + d*tail_stride + r (r < n_tails[d], written by the caller) at positions
 *             pos_base + N + r; its block token b is copied into row N + d*tail_stride +
 *             n_tails[d] + b and sits at position pos_base + N + n_tails[d] + b.
 *   tail_stride : cache rows between consecutive drafts' tails (ignored for one draft).  Needs
 *             n_tails[d] + B <= tail_stride for every draft but the last, and (n_drafts-1)*
 *             tail_stride + n_tails[last] + B <= tail_cap (FD_ERR_TAIL otherwise).
 *   out     : [n_drafts][B][Hq][D] out_dtype.  Draft d's token b sees the whole window, its own
 *             n_tails[d] reasoning rows and its own block tokens <= b, nothing of other drafts.
 *   ws      : as for fd_verify_attn (no initial contents required), ws_bytes >=
 *             fd_verify_batched_workspace_bytes(g, n_drafts, B).
 *   With n_drafts = 1 and no view this is fd_verify_attn.  1 <= B <= 32, G*B <= 128.  */
int fd_verify_attn_batched(const fd_geom* g, int32_t n_drafts, const void* k_view,
                           const void* q_blk, const void* k_blk, const void* v_blk,
                           void* k_cache, void* v_cache, int64_t newest_frame,
                           const int32_t* n_tails, int32_t tail_stride, int32_t blk_len,
                           void* out, void* ws, size_t ws_bytes, void* hip_stream);

/* Rotate the window's keys at their positions for newest_frame into k_view (Positional
 * Encoding passage: keys cached pre-RoPE, rotated at their shifted positions): k_view
 * [Hkv][N][D] fp16 (bf16 inputs) or fp32 (fp32 inputs), cache-row order; the cache is only
 * read.  The same rotation the streaming calls perform first; use it to give
 * fd_verify_attn_batched a view when no streaming call ran on this window.  newest_frame >= F-1. */
int fd_rotate_window(const fd_geom* g, const void* k_cache, int64_t newest_frame, void* k_view,
                     void* hip_stream);

/* Bytes of the static device array behind fd_verify_attn_noalloc (per GPU). */
#define FD_VERIFY_SCRATCH_BYTES (32u << 20)

/* fd_verify_attn for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, semantics,
 * kernels and results as fd_verify_attn, without the workspace: the split-KV partials go to a
 * static __device__ array of FD_VERIFY_SCRATCH_BYTES (32 MiB) that the library holds on each
 * GPU it runs on until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine); its first call on a device looks up that device's address of
 * the array once.  Calls needing more than FD_VERIFY_SCRATCH_BYTES of workspace
 * (fd_verify_workspace_bytes(g, blk_len)) return FD_ERR_SCRATCH before anything is enqueued;
 * the config-4 backbone shapes need 5 MiB at blk_len 8 and 20 MiB at blk_len 32.
 * Every call on one GPU shares its array: calls that overlap on one GPU (concurrent streams,
 * or host threads) race and give undefined results; calls ordered on one stream are safe. */
int fd_verify_attn_noalloc(const fd_geom* g, const void* q_blk,
                           const void* k_blk, const void* v_blk,
                           void* k_cache, void* v_cache, int64_t newest_frame,
                           int32_t n_tail, int32_t blk_len,
                           void* out, void* hip_stream);

/* Range report of the last streaming (fd_stream_attn*) or prefill call made on a workspace
 * (Technical Summary, Methodology 1, "Positional Encoding": keys are rotated when used; with
 * bf16 inputs the rotated keys and queries are rounded to fp16, whose range ends at 65504).
 *   ws, ws_bytes : that call's workspace (ws_bytes as for the call).
 *   hip_stream   : the stream the call ran on (nullptr: the null stream); the report is read
 *                  after the work queued on it, which this call waits for (a host copy of a
 *                  few KB; no device memory is allocated).
 *   Returns the number of waves of that call's rotation pass (64 rows x chunk pairs each)
 *   that rounded a rotated key or query element to +-inf (|x| >= 65520), 0 if none; 0 for
 *   fp32 inputs (fd_stream_overflow).  Errors: geometry / null / FD_ERR_WORKSPACE when
 *   ws_bytes is too small or no bf16 call of that kind has completed on the workspace
 *   (the record's tag is missing), FD_ERR_DTYPE for fd_prefill_overflow with fp32 inputs,
 *   FD_ERR_HIP if the copy fails.  The report describes the workspace's last call only. */
int fd_stream_overflow(const fd_geom* g, const void* ws, size_t ws_bytes, void* hip_stream);
int fd_prefill_overflow(const fd_geom* g, const void* ws, size_t ws_bytes, void* hip_stream);

/* Static description of a status code. */
const char* fd_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FDATTN_H */
