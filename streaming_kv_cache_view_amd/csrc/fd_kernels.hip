// gfx950 (MI355X) kernels of the streaming-prefill attention path.
//
//  insert_kernel       bit copy of the new frame's pre-RoPE K/V into ring slot t mod F
//                      (FlashDrive technical summary, Methodology 1, "Token Layout").
//  rope_window_kernel  once per call: every window key rotated at its current (shifted)
//                      position (Methodology 1, "Positional Encoding") into a caller
//                      workspace, in the QK^T operand format; the cache stays unrotated.
//                      For bf16 inputs it also rotates and scales the queries.  Its
//                      inserting instantiation also copies the new frame into its ring slot
//                      (fd_stream_attn_insert).
//  stream_pp_kernel    (bf16) attention of the new frame's tokens over the view-major window,
//                      two wave groups in MFMA / softmax ping-pong; the streaming mask is
//                      generated from the view / slot / token indices, never loaded.  The
//                      views of a block of query rows are balanced across workgroups, and
//                      a view split between two of them is merged by the one that
//                      finishes second.  stream_pp2_kernel runs a cold start's frame and
//                      prefix segments in one launch.
//  stream_merge_kernel (bf16) fixed-order merge of views split more than once.
//  stream_attn_kernel  (fp32) the same attention, both groups in the same phase.
//  kv_project_kernel   (bf16) K/V projection of the new frames (MFMA GEMM) whose epilogue
//                      writes them, pre-RoPE, into the ring slot (Technical Summary,
//                      "Kernel Fusion").
//  verify_dma_kernel (bf16) / verify_split_kernel (fp32) + verify_merge_kernel
//                      speculative-verify attention of a short draft block over the whole
//                      window + reasoning tail (README technique list, "Speculative
//                      reasoning"; Methodology 2): split-KV over all CUs, then a fixed-order
//                      log-sum-exp merge.
//
// MFMA orientation.  Both attention kernels compute S^T = K Q^T and O^T = V^T P^T on 32x32
// MFMAs: for bf16 inputs S^T on v_mfma_f32_32x32x16_f16 (rotated Q, K rounded to fp16) and
// O^T on v_mfma_f32_32x32x16_bf16; for fp32 inputs both on v_mfma_f32_32x32x2_f32.  In the
// 32x32 accumulator layout lane l holds column l%32 and rows 8*(i/4) + 4*(l/32) + i%4, so
// with the query as the column every lane owns exactly one query row: the softmax row
// max / sum is lane-local plus one exchange between lane halves, the P^T accumulator is
// already in the B-operand layout of the PV product, and O^T rescaling needs no shuffles.
// Operand k-slices are addressed as "16-byte chunks": lane half h supplies elements
// [2E*u + E*h, +E) of chunk u (E = 8 16-bit or 4 fp32); A and B use the same mapping, so the
// reduction is exact whatever order the hardware assigns inside a slice.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "fd_internal.h"

namespace fd {
namespace {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr double kTwoPiHi = 6.283185307179586;       // double nearest 2*pi
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;

// (cos a, sin a) of an fp64 angle: Cody-Waite reduction by pi/2 in fp64 (exact enough for
// |a| < 2^31), then fp32 polynomials on [-pi/4, pi/4] and the quadrant's swap / signs.  The
// polynomial coefficients are the first four of fdlibm's double-precision __kernel_sin and
// __kernel_cos (Sun Microsystems' freely distributable libm), rounded to fp32; error < 1 ulp of
// fp32 on the reduced range.
__device__ inline float2 cs_angle(double a) {
#pragma clang fp contract(off)   // the same roundings wherever it is inlined
  const double k = rint(a * 0.63661977236758134);           // 2/pi
  const double r = fma(-k, 1.5707963267948966, a) - k * 6.123233995736766e-17;
  const float x = static_cast<float>(r), x2 = x * x;
  const float sn = x * (1.f + x2 * (-1.6666667163e-1f + x2 * (8.3333337680e-3f + x2 * (-1.9841270114e-4f + x2 * 2.7557314297e-6f))));
  const float cn = 1.f + x2 * (-0.5f + x2 * (4.1666667908e-2f + x2 * (-1.3888889225e-3f + x2 * (2.4801587642e-5f - x2 * 2.7557314297e-7f))));
  const int q = static_cast<int>(static_cast<long long>(k) & 3);
  float c = (q & 1) ? sn : cn, s = (q & 1) ? cn : sn;
  if (q == 1 || q == 2) c = -c;
  if (q >= 2) s = -s;
  return make_float2(c, s);
}

// cos/sin of (base + offset) from cos/sin of base and of offset.
// (cos, sin) of 2*pi*r for r in revolutions: the fraction of r is taken in fp64 (exact for
// |r| < 2^31), then the hardware sin / cos units, which take revolutions (max error 1.3e-7
// over [-0.5, 0.5], measured on gfx950).
__device__ inline float2 cs_rev(double r) {
  const float f = static_cast<float>(r - rint(r));
  return make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
}

// Complex product and rotation with every rounding spelled out (explicit fma after a rounded
// product), so that each instantiation of a kernel rounds a rotated key identically.
__device__ inline float2 cmul(float2 a, float2 b) {
  return make_float2(__builtin_fmaf(a.x, b.x, -(a.y * b.y)), __builtin_fmaf(a.y, b.x, a.x * b.y));
}
// (a, b) rotated by the angle whose (cos, sin) is cs: (a cos - b sin, b cos + a sin)
__device__ inline float2 rot2(float a, float b, float2 cs) {
  return make_float2(__builtin_fmaf(a, cs.x, -(b * cs.y)), __builtin_fmaf(b, cs.x, a * cs.y));
}

// MFMA operand formats.  A "16-byte chunk" holds E elements of the operand type.
struct BF16Ops {  // bf16 operands, v_mfma_f32_32x32x16_bf16
  static constexpr int E = 8;
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline void unpack(u32x4 x, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(x[j] << 16);
      f[2 * j + 1] = __uint_as_float(x[j] & 0xffff0000u);
    }
  }
  __device__ static inline u32x4 pack(const float* f) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<bf16>(f[j]);  // RNE
    return __builtin_bit_cast(u32x4, v);
  }
};

struct F16Ops {  // fp16 operands, v_mfma_f32_32x32x16_f16
  static constexpr int E = 8;
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline u32x4 pack(const float* f) {
    f16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<_Float16>(f[j]);  // RNE
    return __builtin_bit_cast(u32x4, v);
  }
};

struct F32Ops {  // fp32 operands, v_mfma_f32_32x32x2_f32 (four per chunk)
  static constexpr int E = 4;
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
    return c;
  }
  __device__ static inline void unpack(u32x4 x, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
  }
  __device__ static inline u32x4 pack(const float* f) {
    u32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __float_as_uint(f[e]);
    return x;
  }
};

// Per input dtype: how stored values are read (In), and the operand formats of the two
// products.  For bf16 inputs the rotated Q and K are rounded to fp16 (11 significant bits
// instead of 8; same MFMA rate): with +-8-sigma outliers in K, bf16-rounded rotated keys
// alone cost ~3e-2 max-abs in the output, fp16 ~3e-3.  P and V stay bf16 (V is the
// stored value, exactly; P in [0, 1]).
template <typename T>
struct Path;
template <>
struct Path<bf16> {
  using In = BF16Ops;
  using QK = F16Ops;
  using PV = BF16Ops;
  using QKT = _Float16;
};
template <>
struct Path<float> {
  using In = F32Ops;
  using QK = F32Ops;
  using PV = F32Ops;
  using QKT = float;
};

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// receives, for k = 0..3, element j%4 of the four 16-bit values addressed by lane
// 4k + j/4 of its group.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ inline u32x2 ds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): the wave's 64
// chunks land contiguously at lds_block (wave-uniform), lane i at +16i.
__device__ inline void g2lds16(const void* g, void* lds_block) {
  typedef __attribute__((address_space(1))) const void gvoid;
  typedef __attribute__((address_space(3))) void lvoid;
  __builtin_amdgcn_global_load_lds((gvoid*)(g), (lvoid*)(lds_block), 16, 0, 0);
}
// Workgroup barrier without the release/acquire fences of __syncthreads (which make the
// compiler wait for every outstanding memory operation, loads meant to stay in flight across
// the barrier included).  Callers
// order what crosses it with explicit waits; the empty asm keeps the compiler from moving
// memory operations across it.
__device__ inline void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Kernel arguments wanted early, loaded together into scalar registers.  A kernel's first read
// of each 64-byte line of its arguments otherwise waits for that line on its own, between
// integer work and branches, and a prologue touching five lines paid ~1 us of such waits before
// its first global load.  Naming one field per line here issues the scalar loads back to back,
// behind a single wait, and leaves the lines in the scalar cache for the other fields.
template <typename T>
__device__ __forceinline__ void sreg_use(const T& x) {
  asm volatile("" : : "s"(x));
}
template <typename... Ts>
__device__ __forceinline__ void kernarg_early(const Ts&... xs) {
  (sreg_use(xs), ...);
}
// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima)
constexpr int kWaitVm0 = 0x0F70;

// s_waitcnt vmcnt(n), n < 64
constexpr int wait_vm(int n) { return kWaitVm0 | (n & 15) | ((n >> 4) << 14); }
// s_waitcnt lgkmcnt(0) (vmcnt, expcnt left at their maxima): this wave's LDS writes are done,
// as a bare s_barrier requires before other waves read them
constexpr int kWaitLgkm0 = 0xC07F;
// LDS address of a pointer into __shared__ memory
__device__ inline uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const void lvoid;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lvoid*)(p)));
}
// The same 16-byte-per-lane global -> LDS load as g2lds16 (lane i lands at lds + 16i; gbase
// and lds wave-uniform, voff the lane's byte offset from gbase), issued from inline assembly.
// The compiler does not see it as an LDS write and so inserts no wait for it before later
// LDS reads of other buffers: loads can stay in flight across whole compute phases.  The
// caller makes the data visible with s_waitcnt vmcnt(n) (vector loads complete in issue
// order) and a barrier, and keeps the target out of reach of LDS reads until then.  Each
// load is preceded by one wait state after the write of M0 (the compiler does not see that
// the assembly reads M0).
__device__ inline void g2lds16_async(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(gbase), "{m0}"(lds) : "memory");
}
// A wave-uniform pointer in scalar registers.  A vector instruction (v_readfirstlane) writes
// them, and a vector memory instruction that reads an SGPR needs five wait states after such
// a write; the compiler does not see the reads inside the inline-assembly loads above, so the
// wait states are issued here, tied to the registers.
template <typename T>
__device__ inline T* uni_ptr(T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  asm volatile("s_nop 4" : "+s"(lo), "+s"(hi));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}
// The same with an instruction offset OFF, which the hardware adds to both addresses: the
// lane's global byte gbase + voff + OFF lands at LDS lds + OFF + 16i.
template <int OFF>
__device__ inline void g2lds16_async_at(const void* gbase, uint32_t voff, uint32_t lds) {
  static_assert(OFF >= 0 && OFF < 4096, "instruction offset field");
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%2" : : "v"(voff), "s"(gbase), "i"(OFF), "{m0}"(lds) : "memory");
}


// N contiguous stored elements of T (N * sizeof(T) a multiple of 16) -> floats.
template <typename T, int N>
__device__ inline void load_f(const T* src, float* f) {
  using In = typename Path<T>::In;
#pragma unroll
  for (int c = 0; c < N / In::E; ++c) In::unpack(ld16(src + c * In::E), f + c * In::E);
}
// N floats -> N operand elements of format Ops at dst (16-byte aligned).
template <typename Ops, typename U, int N>
__device__ inline void store_ops(U* dst, const float* f) {
#pragma unroll
  for (int c = 0; c < N / Ops::E; ++c) st16(dst + c * Ops::E, Ops::pack(f + c * Ops::E));
}

// Rotate N (x1, x2) pairs by the angles of frequencies i0 .. i0+N-1 at position base + r:
// cs(base) comes from `cb`, cs(r) from the per-offset table row `cr`.
template <int N>
__device__ inline void rope_pairs(float* x1, float* x2, const float2* cb, const float2* cr, int i0) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float2 cs = cmul(cb[i0 + j], cr[i0 + j]);
    const float a = x1[j], b = x2[j];
    x1[j] = a * cs.x - b * cs.y;
    x2[j] = b * cs.x + a * cs.y;
  }
}

// Position of the frame slot `s` of view `v` at the current window (age = F-1 - (t-s) mod F).
__device__ inline int64_t slot_pos(const KParams& p, int v, int s) {
  const int age = p.F - 1 - ((p.s_new - s + p.F) % p.F);
  return p.pos_base + p.P + static_cast<int64_t>(v * p.F + age) * p.T;
}

// ---------------------------------------------------------------------------------------
// Insert: k_new/v_new [V][T][Hkv][D] -> cache [Hkv][S_cap][D], rows P + (v*F + slot)*T + i.
// One thread per 16-byte chunk; blockIdx.y selects K (0) or V (1).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void insert_kernel(const KParams p, int chunks_per_row,
                                                     const u32x4* __restrict__ kn,
                                                     const u32x4* __restrict__ vn,
                                                     u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                     int slot) {
  const int64_t total = static_cast<int64_t>(p.V) * p.T * p.Hkv * chunks_per_row;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= total) return;
  const u32x4* src = blockIdx.y ? vn : kn;
  u32x4* dst = blockIdx.y ? vc : kc;
  const int c = static_cast<int>(e % chunks_per_row);
  const int64_t row = e / chunks_per_row;  // (v*T + i)*Hkv + h
  const int h = static_cast<int>(row % p.Hkv);
  const int64_t vi = row / p.Hkv;
  const int i = static_cast<int>(vi % p.T), v = static_cast<int>(vi / p.T);
  const int64_t crow = static_cast<int64_t>(h) * p.S_cap + p.P + static_cast<int64_t>(v * p.F + slot) * p.T + i;
  dst[crow * chunks_per_row + c] = src[e];
}

// ---------------------------------------------------------------------------------------
// Swizzle of the V^T tile rows: the 16-byte chunk index is XORed with a function of the
// row (d), so that both the transposing writes (rows 8 apart) and the PV operand reads
// (32 consecutive rows) spread over all LDS banks without padding.
__device__ inline int vswz(int d) { return (d ^ (d >> 3)) & 7; }

// Offset (in keys) of the group of 4 consecutive keys 4*kg inside a V^T tile row.  For
// 16-bit operands the keys of each 16-key block are permuted so that the 8 keys a PV
// B-operand lane holds (keys 4h..4h+3 and 8+4h..8+4h+3 of the block) are contiguous.
template <int E>
__device__ inline int vgroup_pos(int kg) {
  if constexpr (E == 8) {
    const int a = kg & 3;
    return (kg >> 2) * 16 + (a & 1) * 8 + (a >> 1) * 4;
  } else {
    return 4 * kg;
  }
}

// Write 4 keys x E d-values (one 16-byte chunk per key, in rv[0..3]) into V^T rows
// d0 .. d0+E-1 of a tile whose rows are `rowb` bytes long.
template <typename T, int E, int SWM>
__device__ inline void store_vt(unsigned char* Vb, int rowb, int d0, int kg, const u32x4* rv) {
  const int bo = vgroup_pos<E>(kg) * static_cast<int>(sizeof(T));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = d0 + e;
    unsigned char* dst = Vb + d * rowb + ((((bo >> 4) ^ (vswz(d) & SWM)) << 4) | (bo & 15));
    if constexpr (E == 8) {
      const uint32_t w0 = rv[0][e >> 1], w1 = rv[1][e >> 1], w2 = rv[2][e >> 1], w3 = rv[3][e >> 1];
      u32x2 val;
      if (e & 1) {
        val[0] = (w0 >> 16) | (w1 & 0xffff0000u);
        val[1] = (w2 >> 16) | (w3 & 0xffff0000u);
      } else {
        val[0] = (w0 & 0xffffu) | (w1 << 16);
        val[1] = (w2 & 0xffffu) | (w3 << 16);
      }
      *reinterpret_cast<u32x2*>(dst) = val;
    } else {
      const u32x4 val = {rv[0][e], rv[1][e], rv[2][e], rv[3][e]};
      *reinterpret_cast<u32x4*>(dst) = val;
    }
  }
}

struct TileInfo {
  int row0, len, ktok0;
  bool diag;
  int64_t pos0;
};

// Tile table of the streaming kernel (bf16 path), written once per call by the rotation
// pass, one key-tile sequence per query segment.  A segment is the queries of one frame: in a
// streaming call view v's newest frame, in a full-window call every frame (view v, age j) and
// the prefix.  Frame (v, j)'s sequence is the prefix tiles, every frame of views < v, view
// v's frames older than j (all frames in age order, so the walk -- and every sum -- is the
// same at every ring phase), then its own frame (the diagonal, masked per
// token); the prefix segment's is the prefix tiles, masked per token.  A row block whose
// tokens end early uses a prefix of the diagonal.  Entry (segment, t) = {first key row,
// len | diag << 7 | (first key's token within its segment) << 8}: key rows index the
// rotated window and the cache alike.
struct StreamTiles {
  int nP, tps, ndmax, V, F, qmode;
  __device__ explicit StreamTiles(const KParams& p) {
    constexpr int TK = kTileKeys;
    nP = (p.P + TK - 1) / TK;
    tps = (p.T + TK - 1) / TK;
    ndmax = tps;
    V = p.V;
    F = p.F;
    qmode = p.qmode;
  }
  // segment sg: the view v and frame age j of its queries (j < 0: the prefix segment)
  __device__ void seg(int sg, int& v, int& j) const {
    if (qmode == 0) {
      v = sg;
      j = F - 1;
    } else if (sg < V * F) {
      v = sg / F;
      j = sg - v * F;
    } else {
      v = 0;
      j = -1;
    }
  }
  __device__ int segments() const { return qmode == 0 ? V : V * F + (nP > 0 ? 1 : 0); }
  __device__ int view_len(int sg) const {
    int v, j;
    seg(sg, v, j);
    return j < 0 ? nP : nP + (v * F + j) * tps + ndmax;
  }
  __device__ int offset(int sg) const {   // first entry of segment sg
    int o = 0;
    for (int u = 0; u < sg; ++u) o += view_len(u);
    return o;
  }
  // ring slot of the frame of age a (age F-1 = the newest, in slot s_new)
  __device__ static int slot_of_age(const KParams& p, int a) { return (p.s_new + 1 + a) % p.F; }
  // first query row of segment sg: [V*T] rows (streaming) or cache-row order [W] (full window)
  __device__ int qrow0(const KParams& p, int sg) const {
    int v, j;
    seg(sg, v, j);
    if (qmode == 0) return v * p.T;
    return j < 0 ? 0 : p.P + (v * F + slot_of_age(p, j)) * p.T;
  }
  __device__ int2 desc(const KParams& p, int sg, int t) const {
    constexpr int TK = kTileKeys;
    int v, j;
    seg(sg, v, j);
    int row0, seglen, k, diag = 0;
    if (j < 0) {   // the prefix segment: prefix tiles, causal among prefix tokens
      row0 = 0;
      seglen = p.P;
      k = t;
      diag = 1;
    } else if (t < nP) {   // prefix
      row0 = 0;
      seglen = p.P;
      k = t;
    } else {
      const int nfull = v * F + j;   // every frame of views < v, then view v's older frames
      const int f = min((t - nP) / tps, nfull);
      k = t - nP - f * tps;
      int u, sl;
      if (f == nfull) {   // the queries' own frame: the diagonal
        u = v;
        sl = slot_of_age(p, j);
        diag = 1;
      } else if (f < v * F) {   // frames of earlier views, in age order as well
        u = f / F;
        sl = slot_of_age(p, f - u * F);
      } else {
        u = v;
        sl = slot_of_age(p, f - v * F);   // age f - v*F < j
      }
      row0 = p.P + (u * F + sl) * p.T;
      seglen = p.T;
    }
    const int len = min(TK, seglen - k * TK);
    return make_int2(row0 + k * TK, len | (diag << 7) | ((k * TK) << 8));
  }
};

// ---------------------------------------------------------------------------------------
// Window rotation pass of the streaming-prefill call.  Every key of the window is rotated
// once, in registers, at the position it holds in the current window (technical summary,
// Methodology 1, "Positional Encoding": keys are cached pre-RoPE and rotated on the fly at
// shifted positions), and written to the workspace as the QK^T operand format (fp16 for
// bf16 inputs).  The attention kernel that follows then streams rotated tiles, so a key
// is rotated once per window instead of once per workgroup that reads it.
// Key workgroup = 256 threads = RPW window rows x up to kRopeHeads kv heads; thread = (row,
// 16-byte chunk of the first half of the row and its RoPE partner chunk), so a row's angles
// are computed once (fp64 reduction, cs_angle) for every head of the workgroup.
// For bf16 inputs the workgroups past the first nkb also rotate the queries (the new frames'
// tokens, or every window token for a cold start) at their positions, scale them by
// log2(e)/sqrt(D) and store them as fp16 in the input's [tokens][Hq][D] order: the attention
// kernel loads its QK^T operands straight from there.  Such a workgroup takes 32 tokens and
// up to four query heads of one kv head; thread = (token, chunk pair), the heads sharing the
// token's angles.
// Every thread loads its frequencies, then issues all of its row loads, then computes its
// angles while the rows are in flight: no barrier.
// ---------------------------------------------------------------------------------------
__device__ inline int64_t row_pos(const KParams& p, int x) {
  if (x < p.P) return p.pos_base + x;
  const int rr = x - p.P;
  const int v = rr / (p.F * p.T), s = (rr / p.T) % p.F, i = rr % p.T;
  return slot_pos(p, v, s) + i;
}

constexpr int kRopeQTok = 32;   // tokens per query workgroup of the rotation pass
constexpr int kRopeHeads = 2;   // kv heads per key workgroup of the rotation pass (sharing angles)
// key rows of the rotation pass: every window row, or with rot_new only the prefix and the newest
// ring slot of every view (rope_row)
__host__ __device__ inline int rope_rows(const KParams& p) { return p.rot_new ? p.P + p.V * p.T : p.W; }
// window row of entry i of that list
__device__ inline int rope_row(const KParams& p, int i) {
  if (!p.rot_new || i < p.P) return i;
  const int k = i - p.P, v = k / p.T;
  return p.P + (v * p.F + p.s_new) * p.T + (k - v * p.T);
}
// key workgroups of the rotation pass: RPW = 256 / (D/2 / E) rows (E elements per 16-byte chunk of
// the input type) times ceil(Hkv / kRopeHeads) head groups
template <typename T, int D>
inline int rope_key_workgroups(const KParams& p) {
  constexpr int RPW = 256 / (D / 2 / (16 / static_cast<int>(sizeof(T))));
  return ceil_div(rope_rows(p), RPW) * ceil_div(p.Hkv, kRopeHeads);
}

// The new frames to insert in the same pass (kn == nullptr: none).  Rows of ring slot s_new
// are then read from kn / vn ([V][T][Hkv][D], pre-RoPE) instead of the cache, and copied into
// the cache rows (K and V) on the way, so that the attention kernel that follows reads them
// there: fd_kv_insert_frame and the rotation in one pass.
template <typename T>
struct NewFrame {
  const T* kn;
  const T* vn;
  T* kc;
  T* vc;
};
// Bookkeeping workgroups at the front of the rotation pass: one for the tile table, one more for
// the merge descriptors and tickets when there are any
__host__ __device__ constexpr int rope_bookkeeping_workgroups(bool tiles, bool mdesc) {
  return tiles ? (mdesc ? 2 : 1) : 0;
}
__host__ __device__ constexpr int rope_q_heads(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

// Work split of the streaming kernel (bf16 path).  A row block is 128 query rows (the
// HPW heads x TBW 32-token blocks of one kv head and head subset).  The launch covers nseg
// query segments (StreamTiles; in a streaming call the views); for each the row block has a
// tile sequence of view_tiles tiles.  They are laid end to end in the order nseg-1, 0,
// nseg-2, 1, ... (long and short alternate) and the ntot tiles are cut into nseg chunks,
// chunk c = [bnd(c), bnd(c+1)).  Every segment has at least one tile, so no chunk is empty.
// With `whole` set (cold start: many more workgroups than CUs) the order is nseg-1, nseg-2,
// ..., 0 (longest first) and chunk c is exactly the c-th segment of it: the dispatcher hands
// the longest jobs out first and the rest fill in, with no split and no merge.
struct StreamSplit {
  int nP, tps, ndiag, V, F, ntot, seg0, qmode, vf, whole;
  __host__ __device__ StreamSplit(const KParams& p, int qb) {
    constexpr int TK = kTileKeys;
    nP = (p.P + TK - 1) / TK;
    tps = (p.T + TK - 1) / TK;
    const int qend = (qb + 1) * 32 * p.TBW;
    ndiag = ((p.qtok < qend ? p.qtok : qend) + TK - 1) / TK;
    V = p.nseg;   // segments of this launch: the "views" of a row block
    F = p.F;
    seg0 = p.seg0;
    qmode = p.qmode;
    vf = p.V * p.F;
    whole = p.whole;
    ntot = 0;
    for (int u = 0; u < V; ++u) ntot += view_tiles(u);
  }
  // tiles of segment seg0 + u for this row block (StreamTiles: frame (v, j) of a full window
  // is segment v*F + j, after v*F + j earlier frames)
  __host__ __device__ int view_tiles(int u) const {
    const int sg = seg0 + u;
    if (qmode == 0) return nP + (sg * F + F - 1) * tps + ndiag;
    return sg < vf ? nP + sg * tps + ndiag : ndiag;
  }
  __host__ __device__ int order(int oi) const {
    if (whole) return V - 1 - oi;
    return (oi & 1) ? oi / 2 : V - 1 - oi / 2;
  }
  __host__ __device__ int bnd(int c) const {
    if (whole) {
      int pos = 0;
      for (int oi = 0; oi < c; ++oi) pos += view_tiles(order(oi));
      return pos;
    }
    // floor(c*ntot / V) by an fp64 division, exact for c*ntot < 2^53: the quotient is rounded
    // correctly, and a quotient that is not an integer lies at least 1/V below the next one,
    // far more than its rounding error (a 64-bit integer division is ~10x the instructions)
    const int64_t a = static_cast<int64_t>(c) * ntot;
    return a < (int64_t(1) << 53) ? static_cast<int>(static_cast<double>(a) / V) : static_cast<int>(a / V);
  }
  // start of view v in the end-to-end order
  __host__ __device__ int start(int v) const {
    int pos = 0;
    for (int oi = 0; oi < V; ++oi) {
      const int u = order(oi);
      if (u == v) break;
      pos += view_tiles(u);
    }
    return pos;
  }
  // the chunk holding tile x of the end-to-end order
  __host__ __device__ int chunk_of(int x) const {
    int c = 0;
    for (int i = 1; i < V; ++i)
      if (bnd(i) <= x) c = i;
    return c;
  }
};

// Merge descriptor of chunk boundary cb (1 <= cb < nseg) of the row blocks of token block qb,
// written by the rotation pass: the view that boundary cuts, if cb is the first boundary inside
// it (a boundary at a view's start cuts none; no view is cut twice, stream_merge_kernel):
// x = the view (-1: nothing to merge), y = its first and last chunks cf | cl << 16,
// z = the slot of its piece in chunk cf (1: that chunk's last job, 0: its only job), w = the
// view's first output row.
// The cut behind it, on the host too: x = the view (-1: none), y = its first chunk, z = its last,
// w = its first tile in the end-to-end order.
__host__ __device__ inline int4 stream_cut(const KParams& p, const StreamSplit& sp, int cb) {
  const int x = sp.bnd(cb);
  int v = -1, sv = 0, nv = 0;   // the view holding tile x of the end-to-end order
  for (int oi = 0, pos = 0; oi < sp.V; ++oi) {
    const int u = sp.order(oi), n = sp.view_tiles(u);
    if (x < pos + n) {
      v = u;
      sv = pos;
      nv = n;
      break;
    }
    pos += n;
  }
  if (v < 0 || sv == x || sp.chunk_of(sv) != cb - 1) return int4{-1, 0, 0, 0};
  return int4{v, cb - 1, sp.chunk_of(sv + nv - 1), sv};
}
__device__ inline int4 stream_merge_desc(const KParams& p, int qb, int cb) {
  const StreamSplit sp(p, qb);
  const int4 c = stream_cut(p, sp, cb);
  if (c.x < 0) return c;
  return int4{c.x, c.y | (c.z << 16), c.w > sp.bnd(c.y) ? 1 : 0, StreamTiles(p).qrow0(p, p.seg0 + c.x)};
}
// Whether a view of a streaming launch is cut by two or more chunk boundaries, which the split
// never does (stream_merge_kernel); a launch that found one would be refused.
inline bool stream_view_cut_twice(const KParams& p) {
  for (int qb = 0; qb < p.nqb; ++qb) {
    const StreamSplit sp(p, qb);
    for (int cb = 1; cb < p.nseg; ++cb) {
      const int4 c = stream_cut(p, sp, cb);
      if (c.x >= 0 && c.z > c.y + 1) return true;
    }
  }
  return false;
}

template <typename T, int D, bool INS>   // INS: the new frames are inserted by this pass (nf)
__global__ __launch_bounds__(256) void rope_window_kernel(const KParams p, const T* __restrict__ kc,
                                                          typename Path<T>::QKT* __restrict__ krot,
                                                          int nkb, const T* __restrict__ q,
                                                          typename Path<T>::QKT* __restrict__ qrot,
                                                          int2* __restrict__ tiles, int4* __restrict__ mdesc,
                                                          unsigned* __restrict__ flags, const NewFrame<T> nf,
                                                          unsigned char* __restrict__ report) {
#pragma clang fp contract(off)   // every instantiation rounds a rotated row the same way
  using In = typename Path<T>::In;
  using QK = typename Path<T>::QK;
  // each value rounded to fp32 first, then to the operand type: no fused multiply-add-convert
  // (v_fma_mix rounds once, straight to fp16, and the compiler picks it in some instantiations
  // only, so the two rotation passes would differ in the last bit of a few keys)
  auto pack_rounded = [](float* f) {
#pragma unroll
    for (int e = 0; e < In::E; ++e) asm volatile("" : "+v"(f[e]));
    return QK::pack(f);
  };
  using QKT = typename Path<T>::QKT;
  constexpr int E = In::E;
  constexpr int H2 = D / 2;
  constexpr int CH = H2 / E;       // threads per row (RoPE chunk pairs)
  constexpr int RPW = 256 / CH;     // key rows per workgroup
  const int tid = threadIdx.x;
  // Range report (bf16 inputs, report non-null): every wave writes its slot, 1 if a rotated
  // operand it rounded to fp16 left the fp16 range (|x| >= 65520 rounds to inf), else 0;
  // workgroup 0 records the slot count of this launch (rope_report)
  auto report_wave = [&](bool bad) {
    if (!report) return;
    const bool any = __ballot(bad ? 1 : 0) != 0ull;
    if ((tid & 63) == 0) report[kRopeReportHeader + 4 * blockIdx.x + (tid >> 6)] = any ? 1 : 0;
  };
  auto out_of_fp16 = [](float x) { return !(fabsf(x) < 65520.f); };
  if (report && blockIdx.x == 0 && tid == 0) {
    reinterpret_cast<int32_t*>(report)[0] = kRopeReportMagic;
    reinterpret_cast<int32_t*>(report)[1] = static_cast<int32_t>(4 * gridDim.x);
  }
  // bookkeeping workgroups (with a tile table): 0 the attention kernel's tile table, 1 (with
  // merge descriptors) the descriptors and the cleared merge tickets, side by side
  const int nbk = rope_bookkeeping_workgroups(tiles != nullptr, mdesc != nullptr);
  if (static_cast<int>(blockIdx.x) < nbk) {
    report_wave(false);
    if (blockIdx.x == 0) {
      const StreamTiles tt(p);
      for (int sg = 0, o = 0; sg < tt.segments(); o += tt.view_len(sg), ++sg)
        for (int t = tid; t < tt.view_len(sg); t += 256) tiles[o + t] = tt.desc(p, sg, t);
    } else {
      const int nb = p.nseg - 1;   // the merge kernel's descriptors, [nqb][nseg - 1]
      for (int e = tid; e < p.nqb * nb; e += 256) mdesc[e] = stream_merge_desc(p, e / nb, e % nb + 1);
      if (flags)   // the attention kernel's merge tickets, cleared for this call
        for (int e = tid; e < p.Hkv * p.n_hsub * p.nqb * p.nseg; e += 256) flags[e] = 0u;
    }
    return;
  }
  const int bx = static_cast<int>(blockIdx.x) - nbk;   // rotation workgroup
  if (bx >= nkb) {   // query rows (token, head kvh*G + hh)
    // thread (token tl, RoPE chunk pair c) for the workgroup's GH heads of kv head kvh, which
    // share the token's angles; frequencies loaded first, angles computed while the rows fly.
    // Streaming: the newest frames' tokens [V*T]; full window: every window token [W]
    const int kvh = (bx - nkb) % p.Hkv, tl = tid / CH, c = tid % CH;
    const int G = p.G, GH = rope_q_heads(G), NTOK = p.qmode == 0 ? p.V * p.T : p.W;
    const int qb = (bx - nkb) / p.Hkv, hsub = qb % (G / GH), tok0 = (qb / (G / GH)) * kRopeQTok;
    const int tg = tok0 + tl;
    bool bad = false;
    if (tl < kRopeQTok && tg < NTOK) {
    const float sc = p.sm_scale_log2;
    double fr[E];
#pragma unroll
    for (int e = 0; e < E; ++e) fr[e] = p.inv_freq[E * c + e] * kInvTwoPi;
    u32x4 raw[4][2];
    const int64_t base = (static_cast<int64_t>(tg) * p.Hq + kvh * G + hsub * GH) * D;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      if (hh >= GH) continue;
      raw[hh][0] = ld16(q + base + hh * D + E * c);
      raw[hh][1] = ld16(q + base + hh * D + H2 + E * c);
    }
    float2 cs[E];
    {
      const int v = tg / p.T, it = tg - v * p.T;
      const double pos = static_cast<double>(
          p.qmode == 0 ? p.pos_base + p.P + static_cast<int64_t>(v * p.F + p.F - 1) * p.T + it : row_pos(p, tg));
#pragma unroll
      for (int e = 0; e < E; ++e) cs[e] = cs_rev(pos * fr[e]);
    }
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      if (hh >= GH) continue;
      float x1[E], x2[E];
      In::unpack(raw[hh][0], x1);
      In::unpack(raw[hh][1], x2);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float2 r = rot2(x1[e], x2[e], cs[e]);
        x1[e] = r.x * sc;
        x2[e] = r.y * sc;
        bad |= out_of_fp16(x1[e]) | out_of_fp16(x2[e]);
      }
      st16(qrot + base + hh * D + E * c, pack_rounded(x1));
      st16(qrot + base + hh * D + H2 + E * c, pack_rounded(x2));
    }
    }
    report_wave(bad);
    return;
  }
  // ---- keys: thread (row r, RoPE chunk pair c) of the workgroup's RPW rows, for HG kv heads
  // that share the row's angles; the thread's frequencies are loaded before its rows, so the
  // angles are computed while the rows are in flight
  const int nhg = (p.Hkv + kRopeHeads - 1) / kRopeHeads;
  const int rb = bx / nhg, hg = bx % nhg;
  const int r = tid / CH, c = tid % CH, xi = rb * RPW + r;
  const bool live = xi < rope_rows(p);
  const int x = live ? rope_row(p, xi) : 0;   // window row
  double fr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) fr[e] = p.inv_freq[E * c + e];
  int64_t nrow = -1;   // INS: the row's index in k_new / v_new ([V*T] rows) if it is a new-frame row
  if (INS && live && x >= p.P) {
    if (p.rot_new) {
      nrow = xi - p.P;   // every listed row past the prefix is in the newest slot
    } else {
      const int xr = x - p.P, v = xr / (p.F * p.T), sl = (xr / p.T) % p.F, i = xr % p.T;
      if (sl == p.s_new) nrow = v * p.T + i;
    }
  }
  u32x4 raw[kRopeHeads][2], vraw[kRopeHeads][2];
  bool kbad = false;
#pragma unroll
  for (int hh = 0; hh < kRopeHeads; ++hh) {
    const int kvh = hg * kRopeHeads + hh;
    if (!live || kvh >= p.Hkv) continue;
    const T* src = kc + (static_cast<int64_t>(kvh) * p.S_cap + x) * D;
    if (INS && nrow >= 0) {
      src = nf.kn + (nrow * p.Hkv + kvh) * D;
      vraw[hh][0] = ld16(nf.vn + (nrow * p.Hkv + kvh) * D + E * c);
      vraw[hh][1] = ld16(nf.vn + (nrow * p.Hkv + kvh) * D + H2 + E * c);
    }
    raw[hh][0] = ld16(src + E * c);
    raw[hh][1] = ld16(src + H2 + E * c);
  }
  float2 cs[E];
  {
    const double pos = static_cast<double>(live ? row_pos(p, x) : 0);
#pragma unroll
    for (int e = 0; e < E; ++e) cs[e] = cs_angle(pos * fr[e]);
  }
#pragma unroll
  for (int hh = 0; hh < kRopeHeads; ++hh) {
    const int kvh = hg * kRopeHeads + hh;
    if (!live || kvh >= p.Hkv) continue;
    float x1[E], x2[E];
    In::unpack(raw[hh][0], x1);
    In::unpack(raw[hh][1], x2);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float2 rr2 = rot2(x1[e], x2[e], cs[e]);
      x1[e] = rr2.x;
      x2[e] = rr2.y;
      kbad |= out_of_fp16(rr2.x) | out_of_fp16(rr2.y);
    }
    QKT* dst = krot + (static_cast<int64_t>(kvh) * p.W + x) * D;
    st16(dst + E * c, pack_rounded(x1));
    st16(dst + H2 + E * c, pack_rounded(x2));
    if (INS && nrow >= 0) {   // the new frame's row into the cache: K as read, V
      const int64_t cdst = (static_cast<int64_t>(kvh) * p.S_cap + x) * D;
      st16(nf.kc + cdst + E * c, raw[hh][0]);
      st16(nf.kc + cdst + H2 + E * c, raw[hh][1]);
      st16(nf.vc + cdst + E * c, vraw[hh][0]);
      st16(nf.vc + cdst + H2 + E * c, vraw[hh][1]);
    }
  }
  report_wave(kbad);
}


// ---------------------------------------------------------------------------------------
// Streaming-prefill attention over the rotated window.
// Workgroup = 8 waves over 128 query rows that share one kv head: HPW query heads x
// (32*TBW) tokens of one view's new frame.  Waves w and w+4 own the same 32 rows (query
// head (w%4)%HPW, tokens 32*((w%4)/HPW) + [0, 32)); wave group g = w/4 takes the key
// tiles t = g, g+2, g+4, ... of the workgroup's key sequence, so every SIMD runs two waves
// whose MFMA and VALU work interleave; the groups merge (m, l, O) at the end.
// blockIdx.x = ((view_rank*nqb + qb)*n_hsub + hsub)*Hkv + kvh: consecutive workgroups are
// dealt round-robin to the 8 XCDs, so each XCD keeps one kv head's K/V in its L2, and the
// largest views (longest key ranges) are dispatched first.
// Key sequence: TK-row tiles inside segments of contiguous positions -- the prefix, the
// slots of views < v, the older slots of view v, and last the newest slot of view v, the
// only one needing a per-element (causal) mask, generated from indices; its tiles past the
// workgroup's last query token are skipped.
// Per group and iteration (one workgroup barrier): MFMA + online softmax on its current
// tile | copy its next tile from registers into LDS | issue the global loads of the tile
// after that.  K tiles (already rotated) sit in padded rows; V keeps its natural [key][d]
// layout with 16-byte chunks XOR-swizzled by key, and for 16-bit inputs the PV operand is
// read with the transposing LDS load, so no lane shuffles V.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(512) void stream_attn_kernel(const KParams p, const T* __restrict__ q,
                                                          const typename Path<T>::QKT* __restrict__ krot,
                                                          const T* __restrict__ vc, void* __restrict__ out) {
  using In = typename Path<T>::In;
  using QK = typename Path<T>::QK;
  using PV = typename Path<T>::PV;
  using QKT = typename Path<T>::QKT;
  static_assert(QK::E == PV::E, "operand chunk widths must agree");
  constexpr bool k16 = sizeof(T) == 2;
  constexpr int E = QK::E;                       // elements per 16-byte chunk
  constexpr int TK = (!k16 && D == 128) ? 32 : 64;   // keys per tile (LDS budget)
  constexpr int NKB = TK / 32;                   // 32-key MFMA blocks per tile
  constexpr int H2 = D / 2;
  constexpr int CH = H2 / E;                     // chunks per half row (Q staging)
  constexpr int NU = CH;                         // k-chunks of the QK^T operands
  constexpr int RPP = 256 / CH;                  // Q staging rows per pass (256 threads)
  constexpr int QS = D + E;                      // Q staging row stride (elements, padded)
  constexpr int KROWB = (D + E) * static_cast<int>(sizeof(QKT));   // padded K tile row bytes
  constexpr int KCH = D * static_cast<int>(sizeof(QKT)) / 16;      // data chunks per K row
  constexpr int VROWB = D * static_cast<int>(sizeof(T));
  constexpr int VCH = VROWB / 16;                // 16-byte chunks per V row
  constexpr int NKL = TK * KCH / 256;            // K chunks copied per staging thread
  constexpr int NVL = TK * VCH / 256;            // V chunks copied per staging thread
  constexpr int KSLOT = TK * KROWB;
  constexpr int SLOT = KSLOT + TK * VROWB;
  constexpr int QBYTES = 128 * QS * static_cast<int>(sizeof(QKT));
  constexpr int MBYTES = 4 * 32 * (D + 4) * 4;   // group merge buffer
  constexpr int B1 = 4 * SLOT > QBYTES + 16 * H2 * 8 ? 4 * SLOT : QBYTES + 16 * H2 * 8;
  constexpr int BUFB = B1 > MBYTES ? B1 : MBYTES;
  constexpr int ND = D / 32;
  constexpr int CPB = 32 / (2 * E);
  constexpr int NC = TK / (2 * E);               // PV chunks per tile
  constexpr float kTau = 8.f;                    // log2 growth of a row max forcing a rescale
  static_assert(NKL >= 1 && NVL >= 1 && (TK * KCH) % 256 == 0 && (TK * VCH) % 256 == 0,
                "tile too small for the staging map");

  __shared__ float2 csq[4][H2];                  // cos/sin(query block base * f_i)
  __shared__ float red_m[4][32], red_l[4][32];
  __shared__ __attribute__((aligned(16))) unsigned char buf[BUFB];
  float2 (*csA)[H2] = reinterpret_cast<float2 (*)[H2]>(buf + QBYTES);             // prologue only
  float2 (*csB)[H2] = reinterpret_cast<float2 (*)[H2]>(buf + QBYTES + 8 * H2 * 8);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int grp = w >> 2, wr = w & 3, gt = tid & 255;   // group, row set, thread in group
  int bid = blockIdx.x;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int hsub = bid % p.n_hsub;
  bid /= p.n_hsub;
  const int qb = bid % p.nqb;
  const int v = p.V - 1 - bid / p.nqb;
  const int tok0 = qb * 32 * p.TBW;
  const int head = kvh * p.G + hsub * p.HPW + (wr % p.HPW);
  // the last head subset of a group of G = 4k + r heads (r != 0) holds r heads: the rows of the
  // others read zero queries and store nothing
  const bool head_live = hsub * p.HPW + (wr % p.HPW) < p.G;
  const int my_tok = tok0 + 32 * (wr / p.HPW) + l32;
  const int64_t qpos0 = p.pos_base + p.P + static_cast<int64_t>(v * p.F + p.F - 1) * p.T;
  const float sc = p.sm_scale_log2;

  // ---- tile sequence
  const int tps = (p.T + TK - 1) / TK;
  const int hasP = p.P > 0 ? 1 : 0;
  const int nfull = v * p.F + p.F - 1;
  const int tok_end = tok0 + 32 * p.TBW;
  const int ndiag = (min(p.T, tok_end) + TK - 1) / TK;
  const int ntiles = hasP * ((p.P + TK - 1) / TK) + nfull * tps + ndiag;
  struct Cursor {
    int e, k, nk, seglen, row0;
    bool diag;
  };
  auto enter = [&](Cursor& c, int e) {
    c.e = e;
    c.k = 0;
    if (e < hasP) {
      c.row0 = 0;
      c.seglen = p.P;
      c.nk = (p.P + TK - 1) / TK;
      c.diag = false;
      return;
    }
    e -= hasP;
    int u, s;
    if (e < nfull) {   // frames in age order (views < v, then view v's older frames)
      if (e < v * p.F) {
        u = e / p.F;
        s = StreamTiles::slot_of_age(p, e - u * p.F);
      } else {
        u = v;
        s = StreamTiles::slot_of_age(p, e - v * p.F);
      }
      c.nk = tps;
      c.diag = false;
    } else {
      u = v;
      s = p.s_new;
      c.nk = ndiag;
      c.diag = true;
    }
    c.row0 = p.P + (u * p.F + s) * p.T;
    c.seglen = p.T;
  };
  auto advance = [&](Cursor& c) {
    if (++c.k == c.nk) enter(c, c.e + 1);
  };

  // ---- register staging of a tile by the 256 threads of a group (plain copies).  Rows past
  // the tile's end are clamped to its last row: loads stay in bounds and those keys are
  // masked (P = 0) before they can contribute.
  u32x4 rkv[NKL + NVL];
  auto load_tile = [&](const Cursor& c) {
    const int row0 = c.row0 + c.k * TK, lastr = min(TK, c.seglen - c.k * TK) - 1;
    const QKT* kb = krot + (static_cast<int64_t>(kvh) * p.W + row0) * D;
    const T* vb = vc + (static_cast<int64_t>(kvh) * p.S_cap + row0) * D;
#pragma unroll
    for (int m = 0; m < NKL; ++m) {
      const int qc = gt + 256 * m;
      rkv[m] = ld16(kb + min(qc / KCH, lastr) * D + (qc % KCH) * (16 / static_cast<int>(sizeof(QKT))));
    }
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      const int qc = gt + 256 * m;
      rkv[NKL + m] = ld16(vb + min(qc / VCH, lastr) * D + (qc % VCH) * (16 / static_cast<int>(sizeof(T))));
    }
  };
  auto vswz = [](int key) { return (2 * (key & 7)) & (VCH - 1); };
  auto store_tile = [&](int slot) {
    unsigned char* Kb = buf + slot * SLOT;
    unsigned char* Vb = Kb + KSLOT;
#pragma unroll
    for (int m = 0; m < NKL; ++m) {
      const int qc = gt + 256 * m;
      st16(Kb + (qc / KCH) * KROWB + (qc % KCH) * 16, rkv[m]);
    }
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      const int qc = gt + 256 * m, key = qc / VCH;
      st16(Vb + key * VROWB + (((qc % VCH) ^ vswz(key)) << 4), rkv[NKL + m]);
    }
  };

  // ---- prologue: query rotation (through LDS into operand registers), first tiles in flight
  Cursor cn;   // the group's tile whose loads are in flight
  enter(cn, 0);
  if (grp == 1) advance(cn);
  const int ngt = (ntiles - grp + 1) / 2;        // tiles of this group
  if (ngt > 0) load_tile(cn);
  for (int e = tid; e < 16 * H2; e += 512) {
    const int tb = e / (8 * H2), a = (e / H2) % 8, i = e % H2;
    const float2 v2 = cs_angle((tb == 0 ? 8.0 * a : static_cast<double>(a)) * p.inv_freq[i]);
    if (tb == 0) csA[a][i] = v2;
    else csB[a][i] = v2;
  }
  for (int e = tid; e < 4 * H2; e += 512) {
    const int ww = e / H2, i = e % H2;
    csq[ww][i] = cs_angle(static_cast<double>(qpos0 + tok0 + 32 * (ww / p.HPW)) * p.inv_freq[i]);
  }
  __syncthreads();
  {
    QKT* Ql = reinterpret_cast<QKT*>(buf);
    const int kc_ = gt % CH, kr0 = gt / CH;
#pragma unroll
    for (int ps = 0; ps < (64 + RPP - 1) / RPP; ++ps) {
      const int rq = kr0 + ps * RPP;
      if (RPP > 64 && rq >= 64) continue;
      const int row = 64 * grp + rq;
      const int ww = row >> 5, r = row & 31;
      const int hl = hsub * p.HPW + (ww % p.HPW);   // head within the kv head's group (>= G: none)
      const int hd = kvh * p.G + hl;
      const int tk = tok0 + 32 * (ww / p.HPW) + r;
      float x1[E], x2[E];
      if (tk < p.T && hl < p.G) {
        const T* src = q + (static_cast<int64_t>(v * p.T + tk) * p.Hq + hd) * D;
        In::unpack(ld16(src + E * kc_), x1);
        In::unpack(ld16(src + H2 + E * kc_), x2);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) x1[e] = x2[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = E * kc_ + e;
        const float2 cs = cmul(csq[ww][i], cmul(csA[r >> 3][i], csB[r & 7][i]));
        const float a = x1[e], b = x2[e];
        x1[e] = a * cs.x - b * cs.y;
        x2[e] = b * cs.x + a * cs.y;
      }
      st16(Ql + row * QS + E * kc_, QK::pack(x1));
      st16(Ql + row * QS + H2 + E * kc_, QK::pack(x2));
    }
  }
  __syncthreads();
  u32x4 qf[NU];
  {
    const QKT* Ql = reinterpret_cast<const QKT*>(buf);
#pragma unroll
    for (int u = 0; u < NU; ++u) qf[u] = ld16(Ql + (32 * wr + l32) * QS + 2 * E * u + E * h);
  }
  __syncthreads();

  // lane constants of the operand reads
  const int krd = l32 * KROWB + h * 16;                  // QK A operand: row l32, chunk 2u+h
  const int key0 = 4 * h + ((lane & 15) >> 2);           // PV A operand (16-bit): key 16c+key0 (+8)
  int voff[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    if constexpr (k16) {
      const int cb2 = (32 * d + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
      voff[d] = key0 * VROWB + ((((cb2 >> 4) ^ vswz(key0)) << 4) | (cb2 & 15));
    } else {
      voff[d] = 32 * d + l32;
    }
  }

  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;   // accumulators refer to m_ref: P = exp2(sc*s - m_ref)

  auto compute = [&](int slot, const Cursor& c) {
    const unsigned char* Kb = buf + slot * SLOT;
    const unsigned char* Vb = Kb + KSLOT;
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      u32x4 ka[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) ka[u] = ld16(Kb + krd + kb * 32 * KROWB + u * 32);
      s[kb] = f32x16{};
#pragma unroll
      for (int u = 0; u < NU; ++u) s[kb] = QK::mma(ka[u], qf[u], s[kb]);
    }
    const int ktok0 = c.k * TK, len = min(TK, c.seglen - ktok0);
    if (c.diag || len < TK) {   // generated mask: tile end, causal newest slot
      // key kk = 32kb + 8(i/4) + 4h + i%4 is visible iff kk < lim
      const int lim = (c.diag ? min(len, my_tok - ktok0 + 1) : len) - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) < lim) ? s[kb][i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kb][i], s[kb][i + 1]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sc;
    if (__ballot(mx > m_ref + kTau) != 0) {   // rare: a row maximum grew by more than 2^kTau
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] *= alpha;
      m_ref = m_new;
    }
    const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[kb][i], sc, -mu));
        s[kb][i] = pr;
        lsum += pr;
      }
    }
    l_run += lsum;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int kb = cc / CPB;
      float pv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) pv[e] = s[kb][E * (cc % CPB) + e];
      const u32x4 bop = PV::pack(pv);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        u32x4 a;
        if constexpr (k16) {
          // A operand = V^T[32d + l%32][keys 16cc + 4h + {0..3}, 16cc + 8 + 4h + {0..3}]
          const u32x2 lo = ds_read_tr16(Vb + voff[d] + 16 * cc * VROWB);
          const u32x2 hi = ds_read_tr16(Vb + voff[d] + (16 * cc + 8) * VROWB);
          a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          // fp32: element e of chunk cc holds key 8cc + 4h + e at column 32d + l%32
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = 8 * cc + 4 * h + e, col = voff[d];
            a[e] = *reinterpret_cast<const uint32_t*>(Vb + key * VROWB + ((((col >> 2) ^ vswz(key)) << 4) | ((col & 3) << 2)));
          }
        }
        o[d] = PV::mma(a, bop, o[d]);
      }
    }
  };

  // ---- main pipeline (per group: compute tile j, stage tile j+1, load tile j+2)
  auto slot_of = [&](int j) { return 2 * (j & 1) + grp; };
  Cursor cc = cn;
  if (ngt > 0) store_tile(slot_of(0));
  if (ngt > 1) {
    advance(cn);
    advance(cn);
    load_tile(cn);
  }
  __syncthreads();
  const int niter = (ntiles + 1) / 2;
  for (int j = 0; j < niter; ++j) {
    if (j < ngt) compute(slot_of(j), cc);
    if (j + 1 < ngt) store_tile(slot_of(j + 1));
    if (j + 2 < ngt) {
      advance(cn);
      advance(cn);
      load_tile(cn);
    }
    advance(cc);
    advance(cc);
    __syncthreads();
  }

  // ---- merge the two groups (same rows, disjoint key tiles), then O / l
  const float l_half = l_run + __shfl_xor(l_run, 32);
  float* mb = reinterpret_cast<float*>(buf) + wr * 32 * (D + 4);
  if (grp == 1) {
    if (lane < 32) {
      red_m[wr][l32] = m_ref;
      red_l[wr][l32] = l_half;
    }
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig)
        *reinterpret_cast<f32x4*>(mb + l32 * (D + 4) + 32 * d + 8 * ig + 4 * h) =
            f32x4{o[d][4 * ig], o[d][4 * ig + 1], o[d][4 * ig + 2], o[d][4 * ig + 3]};
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = red_m[wr][l32], l1 = red_l[wr][l32];
    const float M = fmaxf(m_ref, m1);
    const float a0 = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - M);
    const float a1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    const float inv = 1.f / (a0 * l_half + a1 * l1);
    if (my_tok < p.T && head_live) {
      const int64_t obase = (static_cast<int64_t>(v * p.T + my_tok) * p.Hq + head) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int d0 = 32 * d + 8 * ig + 4 * h;
          const f32x4 ov = *reinterpret_cast<const f32x4*>(mb + l32 * (D + 4) + d0);
          const f32x4 r = {(o[d][4 * ig] * a0 + ov[0] * a1) * inv, (o[d][4 * ig + 1] * a0 + ov[1] * a1) * inv,
                           (o[d][4 * ig + 2] * a0 + ov[2] * a1) * inv, (o[d][4 * ig + 3] * a0 + ov[3] * a1) * inv};
          if (p.out_bf16) {
            bf16 b4[4] = {static_cast<bf16>(r[0]), static_cast<bf16>(r[1]), static_cast<bf16>(r[2]), static_cast<bf16>(r[3])};
            *reinterpret_cast<u32x2*>(static_cast<bf16*>(out) + obase + d0) = *reinterpret_cast<const u32x2*>(b4);
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) + obase + d0) = r;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Streaming-prefill attention for bf16 inputs: two wave groups in ping-pong.
//
// Same work split as the kernel above (workgroup = 128 query rows of one kv head, two groups
// of four waves taking alternate key tiles, one LDS merge at the end), but the two groups run
// half a tile out of phase.  Wave w and wave w+4 share a SIMD; at every half-step one of
// them is in its MFMA phase (PV of tile k-1, then QK^T of tile k: 2x16 MFMAs for D = 128,
// operands from LDS) while the other is in its VALU phase (mask, row max, exp2, row sum,
// P -> bf16 of tile k, then staging of the group's next tile).  A workgroup barrier separates
// the half-steps, so the two phases of one SIMD's waves overlap instead of contending.
//
// Tiles move HBM/L2 -> LDS by direct loads (global_load_lds, no registers); a group's LDS
// ring holds two tiles.  The barrier between half-steps is a bare s_barrier: each wave orders
// what crosses it with explicit waits (its tile loads) or by consuming its LDS reads.
//
// Softmax bookkeeping.  Q is scaled by log2(e)/sqrt(D) before the fp16 rounding, so QK^T is
// already in log2 units.  The QK^T accumulator starts at -m_ref (the row's reference max),
// so the MFMA output is the exponent itself; m_ref is raised (and O, l rescaled) only when a
// tile's maximum exceeds it by more than kTau, so exp2 arguments stay <= kTau.
// ---------------------------------------------------------------------------------------

// max / sum of a value over the two lane halves (lane l and lane l ^ 32)
__device__ inline float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Output store of 4 consecutive elements (bf16 or fp32 output).
__device__ inline void store_out4(void* out, int out_bf16, int64_t idx, const f32x4& r) {
  if (out_bf16) {
    bf16 b4[4] = {static_cast<bf16>(r[0]), static_cast<bf16>(r[1]), static_cast<bf16>(r[2]), static_cast<bf16>(r[3])};
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(out) + idx) = *reinterpret_cast<const u32x2*>(b4);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = r;
  }
}

// Staging map of the bf16 streaming kernel's 64-key K and V tiles (rows of D 16-bit
// elements, KCH 16-byte chunks each).  Wave wr of a group fills rows [16wr, 16wr+16) with
// NL = KCH/4 loads of 1 KB; load m of lane ln fetches tile row r = (wr*NL + m)*(64/KCH) +
// ln/KCH, chunk (ln % KCH) ^ swz(r), and lands at LDS byte 1024*(wr*NL + m) + 16*ln, so LDS row
// r holds chunk c at position c ^ swz(r).  K rows use kswz (the 16 rows of one QK^T operand
// read fall in 16 distinct bank groups), V rows vswz (the 32 lanes of a transposing read fall
// in 32 distinct bank pairs).  Between loads m and 0 the row moves by 1024 bytes in memory
// and in LDS, and the chunk index by XOR 4m for K and not at all for V: a whole tile needs one
// lane offset per wave (instruction offsets 1024m), which check() proves for every lane.
template <int D>
struct StageMap {
  static constexpr int KCH = D * 2 / 16, RPI = 64 / KCH, NL = KCH / 4;
  static constexpr int KPR = 16 / KCH, VPR = 16 / KCH;   // rows per 256-byte bank row
  static constexpr uint32_t kswz(uint32_t r) { return (r / KPR) & (KCH - 1); }
  static constexpr uint32_t vswz(uint32_t r) { return 4 * ((r / VPR) & (KCH / 4 - 1)); }
  static constexpr uint32_t row(uint32_t wr, uint32_t m, uint32_t ln) { return (wr * NL + m) * RPI + ln / KCH; }
  static constexpr uint32_t k_off(uint32_t wr, uint32_t m, uint32_t ln) {
    return row(wr, m, ln) * (D * 2) + (((ln % KCH) ^ kswz(row(wr, m, ln))) << 4);
  }
  static constexpr uint32_t v_off(uint32_t wr, uint32_t m, uint32_t ln) {
    return row(wr, m, ln) * (D * 2) + (((ln % KCH) ^ vswz(row(wr, m, ln))) << 4);
  }
  static constexpr bool check() {
    for (uint32_t wr = 0; wr < 4; ++wr)
      for (uint32_t ln = 0; ln < 64; ++ln)
        for (uint32_t m = 0; m < NL; ++m) {
          if (k_off(wr, m, ln) != (k_off(wr, 0, ln) ^ (64 * m)) + 1024 * m) return false;
          if (v_off(wr, m, ln) != v_off(wr, 0, ln) + 1024 * m) return false;
        }
    return RPI * D * 2 == 1024 && NL * 256 == 64 * KCH;
  }
};
static_assert(StageMap<128>::check() && StageMap<64>::check(), "whole-tile staging offsets");


// Slot of the partial of a job of view v in chunk c: two per (row block, chunk), 0 for the
// chunk's first job (which starts at bnd(c)), 1 for its last.  A slot holds the piece's
// unnormalised O[128][D] in fp16, each row multiplied by a power of two 2^s that brings its
// largest magnitude into [2^14, 2^15) (so no row overflows or leaves the normal range, and
// each value keeps fp16's 11 significant bits), then per row the fp32 (row max m, row sum l,
// 2^-s, 0).
// Half offset, within a row of a stored streaming partial, of its 4 values at columns col .. col+3
// (col a multiple of 4).  The 8 values of lane c of a row's D/8 lanes go out as two 8-byte units,
// columns 8c .. 8c+3 at unit c and 8c+4 .. 8c+7 at unit D/8 + c, so that each store instruction of
// a wave writes whole runs of a row (device-scope stores are 8 bytes wide, and a lane's two halves
// side by side would leave every run half written per instruction).
template <int D>
__host__ __device__ constexpr int partial_col(int col) {
  return 4 * (((col >> 2) & 1) ? D / 8 + (col >> 3) : (col >> 3));
}
static_assert(partial_col<128>(0) == 0 && partial_col<128>(4) == 64 && partial_col<128>(8) == 4 &&
                  partial_col<128>(124) == 124 && partial_col<64>(60) == 60,
              "partial row layout");
template <int D>
__device__ inline float* stream_slot(float* part, const KParams& p, int rbi, int c, int which) {
  return part + (static_cast<int64_t>(rbi * p.nseg + c) * 2 + which) * stream_partial_words(D);
}
// 2^e as a float, for integer e in [-126, 127]
__device__ inline float exp2_int(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }
// Exponent s of a partial row's scale: |x| < 2^(E+1) for the row's largest magnitude
// mx = 1.f * 2^E, so 2^(14 - E) maps it into [2^14, 2^15); clamped so 2^s and 2^-s are normal
// floats (mx = 0 or subnormal takes the largest scale).
__device__ inline int partial_row_scale(float mx) {
  const int e_bits = static_cast<int>((__float_as_uint(mx) >> 23) & 0xff);
  return min(max(141 - e_bits, -126), 126);
}

// Merge of the views whose tiles were split between two chunks, by a separate kernel (merge mode
// 0; otherwise the attention kernel merges them itself).  No view is cut more than once: for a
// row block, view u has a + b*u tiles, and the order V-1, 0, V-2, 1, ... pairs views whose tiles
// sum to exactly two chunks, so a pair starts and ends on chunk boundaries, its long view
// (longer than one chunk, shorter than two) is cut once and its short view is whole; with V odd
// the middle view is one chunk exactly.  The host checks this (stream_view_cut_twice) before
// every streaming launch.  Chunk boundary c (between chunks c - 1 and c) cuts at most one view,
// as the rotation pass's descriptor for (token block, c) records (stream_merge_desc); its two
// pieces combine by merge_two, the function the attention kernel's own merge calls, so the two
// give the same bits.
// Workgroup = 256 threads over one (boundary, row block), which takes the row block's D/16
// groups of kMergeItems / (HPW*D/4) tokens (all HPW heads) in turn.  Item e (thread tid takes
// e = tid and tid + 256) is token e / (HPW*D/4), head (e / (D/4)) % HPW, columns 4*(e % (D/4))
// .. +3: a token's heads are adjacent rows of the output, so each store instruction of a wave
// writes 1 KB (fp32) of contiguous output.
constexpr int kMergeItems = 512;   // 4-column items per merge workgroup
// Polls (each then s_sleep 16, ~1,000 cycles) for which the second piece of a view cut once waits
// for the first piece's ticket in the test mode that makes the second piece merge (merge_mode 2)
constexpr int kMergeTestPolls = 4096;
// 4 fp16 values (as stored) to fp32
__device__ inline f32x4 f16x4_to_f32(u32x2 x) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  const f16x4 h = __builtin_bit_cast(f16x4, x);
  return f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]), static_cast<float>(h[3])};
}
// The merge of the two pieces of a view cut once, for 4 consecutive columns of a row: piece i's
// (row max m_i, row sum l_i, inverse scale s_i) and its 4 stored fp16 values x_i give
// sum_i 2^(m_i - M) s_i x_i / sum_i 2^(m_i - M) l_i, M = max(m_0, m_1).  The merge kernel and the
// attention kernel's own merge both call it on the same stored values, so they give the same bits.
__device__ __forceinline__ f32x4 merge_two(float m0, float l0, float s0, u32x2 x0, float m1, float l1, float s1,
                                           u32x2 x1) {
  const float M = fmaxf(m0, m1);
  const float w0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
  const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
  const float inv = 1.f / __builtin_fmaf(w1, l1, w0 * l0);
  const float a0 = w0 * s0, a1 = w1 * s1;
  const f32x4 h0 = f16x4_to_f32(x0), h1 = f16x4_to_f32(x1);
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(a1, h1[e], a0 * h0[e]) * inv;
  return r;
}
template <int D>
__global__ __launch_bounds__(256) void stream_merge_kernel(const KParams p, const int4* __restrict__ mdesc,
                                                           const float* __restrict__ part, void* __restrict__ out) {
  constexpr int CG = D / 4, NSUB = D / 16, IPT = kMergeItems / 256;
  // blockIdx.x = (((c - 1)*n_hsub + hsub)*nqb + qb)*Hkv + kvh: the kv head fastest, as in the
  // attention kernel, so (for Hkv a multiple of 8) a row block's partials are merged on the XCD
  // whose L2 they were written through
  int bid = blockIdx.x;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int qb = bid % p.nqb;
  bid /= p.nqb;
  const int hsub = bid % p.n_hsub;
  const int cb = bid / p.n_hsub + 1;   // boundary between chunks cb - 1 and cb
  const int rbi = (kvh * p.n_hsub + hsub) * p.nqb + qb;
  const int4 dsc = mdesc[qb * (p.nseg - 1) + cb - 1];   // stream_merge_desc
  if (dsc.x < 0) return;   // the boundary cuts no view
  const int cf = dsc.y & 0xffff, cl = dsc.y >> 16, which_cf = dsc.z, qrow0 = dsc.w;   // cl == cf + 1
  const int per_tok = p.HPW * CG, ntok = kMergeItems / per_tok;
  for (int sub = 0; sub < NSUB; ++sub) {   // the row block's token groups in turn
  int row[IPT], col[IPT];
  int64_t obase[IPT];
  bool live[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int e = threadIdx.x + 256 * k;
    const int tr = sub * ntok + e / per_tok, hl = (e % per_tok) / CG;   // token within the row block, head
    col[k] = 4 * (e % CG);
    row[k] = 32 * (hl + p.HPW * (tr >> 5)) + (tr & 31);   // partial row (ww = row/32: token block, head)
    const int tok = qb * 32 * p.TBW + tr;
    live[k] = tok < p.qtok && hsub * p.HPW + hl < p.G;   // a ragged last head subset: heads past G are none
    obase[k] = (static_cast<int64_t>(qrow0 + tok) * p.Hq + kvh * p.G + hsub * p.HPW + hl) * D + col[k];
  }
  {
    const float* s0 = stream_slot<D>(const_cast<float*>(part), p, rbi, cf, which_cf);
    const float* s1 = stream_slot<D>(const_cast<float*>(part), p, rbi, cl, 0);
    f32x4 ml0[IPT], ml1[IPT];
    u32x2 x0[IPT], x1[IPT];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      ml0[k] = *reinterpret_cast<const f32x4*>(s0 + 64 * D + 4 * row[k]);
      x0[k] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const _Float16*>(s0) + row[k] * D + partial_col<D>(col[k]));
      ml1[k] = *reinterpret_cast<const f32x4*>(s1 + 64 * D + 4 * row[k]);
      x1[k] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const _Float16*>(s1) + row[k] * D + partial_col<D>(col[k]));
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k)
      if (live[k])
        store_out4(out, p.out_bf16, obase[k],
                   merge_two(ml0[k][0], ml0[k][1], ml0[k][2], x0[k], ml1[k][0], ml1[k][1], ml1[k][2], x1[k]));
  }
  }   // token groups
}

// ---------------------------------------------------------------------------------------
// Streaming-prefill attention for bf16 inputs over the rotated window.
// Workgroup = 8 waves over the 128 query rows of one row block (HPW query heads x 32*TBW
// tokens sharing one kv head); blockIdx.x = ((chunk*nqb + qb)*n_hsub + hsub)*Hkv + kvh, so
// consecutive workgroups are dealt round-robin to the 8 XCDs and each XCD keeps one kv
// head's K/V in its L2.  The workgroup runs the jobs of its chunk (StreamSplit): pieces of
// views' key sequences, each with the view's queries (loaded from the rotation pass's
// output) -- the prefix, the slots of views < v, the older slots of view v and last the
// newest slot of view v, the only one needing a per-token (causal) mask.
// Waves w and w+4 own the same 32 rows; wave group g = w/4 takes the job's tiles g, g+2, ...
// Half-steps separated by a barrier: one group in its MFMA phase (PV of its tile k-1 and
// QK^T of its tile k, operands read from LDS two MFMAs ahead), the other in its VALU phase
// (softmax of its tile k and the global -> LDS loads of its tile k+1).  The two groups merge
// (m, l, O) through LDS at the end of a job; a whole view is normalised and written, a
// piece goes to its partial slot for stream_merge_kernel.
// ---------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void stream_pp_body(const KParams& p, const int block, const _Float16* __restrict__ qrot,
                                               const _Float16* __restrict__ krot, const bf16* __restrict__ vc,
                                               void* __restrict__ out, float* __restrict__ part,
                                               const int2* __restrict__ tiles, const int4* __restrict__ mdesc,
                                               unsigned* __restrict__ flags) {
  using QK = F16Ops;
  using PV = BF16Ops;
  constexpr int E = 8;                           // 16-bit elements per 16-byte chunk
  constexpr int TK = 64;                         // keys per tile
  constexpr int NKB = TK / 32;                   // 32-key MFMA blocks per tile
  constexpr int H2 = D / 2;
  constexpr int NU = D / 16;                     // k-steps of QK^T
  constexpr int KROWB = D * 2;                   // K tile row (bytes; chunks XOR-swizzled)
  constexpr int KCH = D * 2 / 16;                // 16-byte chunks per K row
  constexpr int VROWB = D * 2;
  constexpr int VCH = VROWB / 16;
  constexpr int NKL = TK * KCH / 256;            // direct K loads per thread and tile
  constexpr int NVL = TK * VCH / 256;            // direct V loads per thread and tile
  constexpr int KSLOT = TK * KROWB;
  constexpr int SLOT = KSLOT + TK * VROWB;
  constexpr int MBYTES = 4 * 32 * (D + 4) * 4;
  constexpr int BUFB = 4 * SLOT > MBYTES ? 4 * SLOT : MBYTES;
  constexpr int ND = D / 32;
  constexpr int NC = TK / 16;                    // PV k-chunks per tile
  constexpr int NMF = NC * ND;                   // PV MFMAs per tile (== QK MFMAs per tile)
  constexpr float kTau = 8.f;
  static_assert(NMF == NKB * NU, "PV and QK^T phases must pair one to one");
  static_assert(NKL >= 1 && NVL >= 1 && (TK * KCH) % 256 == 0 && (TK * VCH) % 256 == 0, "staging map");

  __shared__ float red_m[4][32], red_l[4][32];
  __shared__ __attribute__((aligned(16))) unsigned char buf[BUFB];
  __shared__ int s_ready;

  const int tid0 = threadIdx.x;
  // wave-uniform values in scalar registers (the index arithmetic of staging and masking)
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  int bid = block;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int hsub = bid % p.n_hsub;
  bid /= p.n_hsub;
  const int qb = bid % p.nqb;
  const int chunk = bid / p.nqb;
  const int rbi = (kvh * p.n_hsub + hsub) * p.nqb + qb;   // row block
  const int tok0 = qb * 32 * p.TBW;

  // ---- tile sequence of view v: StreamTiles (its table, tiles); its length for this row block
  const StreamSplit sp(p, qb);
  const StreamTiles stt(p);
  // ---- this workgroup's chunk [c0, c1) of the row block's segments laid end to end
  const int c0 = sp.bnd(chunk), c1 = sp.bnd(chunk + 1);

  // LDS swizzles of the K and V tiles (StageMap)
  auto kswz = [](uint32_t r) { return StageMap<D>::kswz(r); };
  auto vswz = [](uint32_t key) { return StageMap<D>::vswz(key); };
  int vstart = 0;   // start of segment v in the end-to-end order
  u32x4 qf[NU];     // QK^T B operand: the lane's query row, d in [16u + 8h, 16u + 8h + 8)
  int pf = 0;       // the job's first tile and query operands were issued during the last epilogue
  for (int oi = 0; oi < p.nseg; ++oi) {
  const int v = sp.order(oi);   // segment p.seg0 + v of this launch
  const int nv = sp.view_tiles(v);
  const int sv = vstart;
  vstart += nv;
  const int ja = max(c0, sv) - sv, jb = min(c1, sv + nv) - sv;   // this job: tiles [ja, jb) of view v
  if (ja >= jb) continue;
  // Lane indices from an opaque copy of the thread index: nothing derived from them is
  // hoisted out of this loop (it would stay live across every job's main loop).
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = tid >> 6;
  const int grp = w >> 2, wr = w & 3, gt = tid & 255;
  const int head = kvh * p.G + hsub * p.HPW + (wr % p.HPW);
  // the last head subset of a group of G = 4k + r heads (r != 0) holds r heads: the rows of the
  // others read zero queries and store nothing
  const bool head_live = hsub * p.HPW + (wr % p.HPW) < p.G;
  const int my_tok = tok0 + 32 * (wr / p.HPW) + l32;
  // lane constants of the operand reads.  QK A operand: row l32, chunk (2u+h) ^ kswz(l32),
  // at krd0 ^ 32u.  PV A operand: keys 16c+key0 (+8), columns 32d + 16((lane>>4)&1) +
  // 4(lane&3) with the V swizzle, at voff0 ^ 64d.  (The swizzles XOR whole chunk indices, so
  // the step in u or d is an XOR of the byte offset.)
  const int krd0 = l32 * KROWB + ((h ^ kswz(l32)) << 4);
  const int key0 = 4 * h + ((lane & 15) >> 2);
  const int voff0 = [&] {
    const int cb2 = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    return key0 * VROWB + ((((cb2 >> 4) ^ vswz(key0)) << 4) | (cb2 & 15));
  }();

  const int ntiles = jb - ja;
  // The job's tiles t = 0 .. ntiles-1 (tile ja + t of view v): group g takes t = g, g+2, ...
  // and keeps tile t in LDS slot (t + 3) & 3 (tile 0 in slot 3, the one the epilogue leaves
  // free, so the next job's tile 0 can land during it).  Table entries are read with scalar loads.
  const int2* jt = tiles + (stt.offset(p.seg0 + v) + ja);
  const int qrow0 = stt.qrow0(p, p.seg0 + v);   // query / output row of the segment's token 0

  // ---- staging of one tile by the group's 256 threads, straight from HBM/L2 into LDS
  // (global_load_lds, 16 bytes per lane; each instruction fills 1 KB of LDS linearly, lane i
  // at +16i, so the swizzles are applied by choosing which global chunk a lane fetches; the
  // map and its swizzles are StageMap's).  LDS has 64 four-byte banks (256 bytes per bank row).
  const uint32_t lds_buf = lds_addr(buf);
  using SM = StageMap<D>;
  static_assert(SM::NL == NKL && SM::NL == NVL, "staging map");
  auto stage = [&](const int2* tab, int t) {
    const int2 d = tab[t];
    const int row0 = d.x, lastr = (d.y & 127) - 1;
    const uint32_t Kb = lds_buf + ((t + 3) & 3) * SLOT, Vb = Kb + KSLOT;
    const int wrs = uni(wr);
    const unsigned char* kb = reinterpret_cast<const unsigned char*>(krot + (static_cast<int64_t>(kvh) * p.W + row0) * D);
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(vc + (static_cast<int64_t>(kvh) * p.S_cap + row0) * D);
    uint32_t ln = lane;
    asm volatile("" : "+v"(ln));   // recompute the lane terms here rather than keep them live
    if (lastr == TK - 1) {   // whole tile: one lane offset, instruction offsets 1024m
      const uint32_t ko = SM::k_off(wrs, 0, ln), kl = uni(Kb + wrs * NKL * 1024);
      g2lds16_async_at<0>(kb, ko, kl);
      if constexpr (NKL > 1) g2lds16_async_at<1024>(kb, ko ^ 64, kl);
      if constexpr (NKL > 2) g2lds16_async_at<2048>(kb, ko ^ 128, kl);
      if constexpr (NKL > 3) g2lds16_async_at<3072>(kb, ko ^ 192, kl);
      const uint32_t vo = SM::v_off(wrs, 0, ln), vl = uni(Vb + wrs * NVL * 1024);
      g2lds16_async_at<0>(vb, vo, vl);
      if constexpr (NVL > 1) g2lds16_async_at<1024>(vb, vo, vl);
      if constexpr (NVL > 2) g2lds16_async_at<2048>(vb, vo, vl);
      if constexpr (NVL > 3) g2lds16_async_at<3072>(vb, vo, vl);
      return;
    }
    // Rows past the tile's end are clamped to its last row: in bounds, and those keys are masked.
    const uint32_t lr = static_cast<uint32_t>(lastr);
#pragma unroll
    for (int m = 0; m < NKL; ++m) {
      const uint32_t r = min(SM::row(wrs, m, ln), lr) * (D * 2);
      g2lds16_async(kb, r + (SM::k_off(wrs, m, ln) & (D * 2 - 1)), Kb + (wrs * NKL + m) * 1024);
      g2lds16_async(vb, r + (SM::v_off(wrs, m, ln) & (D * 2 - 1)), Vb + (wrs * NVL + m) * 1024);
    }
  };

  // the lane's query row of the segment whose token 0 is query row r0 (rotated and scaled by the
  // rotation pass)
  auto load_q = [&](int r0) {
    const bool valid = my_tok < p.qtok && head_live;
    const _Float16* src = qrot + (static_cast<int64_t>(r0 + (valid ? my_tok : 0)) * p.Hq + (valid ? head : 0)) * D + E * h;
#pragma unroll
    for (int u = 0; u < NU; ++u) qf[u] = valid ? ld16(src + 2 * E * u) : u32x4{0u, 0u, 0u, 0u};
  };

  // ---- prologue: tile t = grp of the job lands while the query operands load (tile 0 and the
  // queries may already be in flight)
  if (grp < ntiles && !(pf && grp == 0)) stage(jt, uni(grp));
  if (!pf) load_q(qrow0);

  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x16{};
  f32x16 s[NKB];
  u32x4 pb[NC];
  float m_ref = 0.f, l_run = 0.f;   // S accumulators start at -m_ref; P = exp2(S)
  f32x16 negm = f32x16{};
  bool fresh = true;                // no key has contributed to this row yet

  // MFMA phase at half-step st: PV of tile st-2 (P in pb) and QK^T of tile st, one of each
  // per step.  The operand reads of step t+2 are issued before the MFMAs of step t (the
  // schedule is pinned with sched_group_barrier: the MFMA pipe would otherwise wait on every
  // LDS read).
  auto mfma_phase = [&](auto pv_t, auto qk_t, int st) {
    constexpr bool DO_PV = decltype(pv_t)::value, DO_QK = decltype(qk_t)::value;
    constexpr int RD = (DO_PV ? 2 : 0) + (DO_QK ? 1 : 0);   // LDS reads per step
    constexpr int MF = (DO_PV ? 1 : 0) + (DO_QK ? 1 : 0);   // MFMAs per step
    constexpr int LEAD = 2;
    const unsigned char* Kb = buf + ((st + 3) & 3) * SLOT;
    const unsigned char* Vb = buf + ((st + 1) & 3) * SLOT + KSLOT;   // slot of tile st-2
    u32x4 va[NMF], ka[NMF];
    auto read = [&](int t) {
      if constexpr (DO_PV) {
        const int cc = t / ND, d = t % ND;
        const int vo = voff0 ^ (64 * d);
        const u32x2 lo = ds_read_tr16(Vb + vo + 16 * cc * VROWB);
        const u32x2 hi = ds_read_tr16(Vb + vo + (16 * cc + 8) * VROWB);
        va[t] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      if constexpr (DO_QK) {
        const int kb = t / NU, u = t % NU;
        ka[t] = ld16(Kb + (krd0 ^ (32 * u)) + kb * 32 * KROWB);
      }
    };
#pragma unroll
    for (int t = 0; t < LEAD; ++t) read(t);
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      if (t + LEAD < NMF) read(t + LEAD);
      if constexpr (DO_PV) {
        const int cc = t / ND, d = t % ND;
        o[d] = PV::mma(va[t], pb[cc], o[d]);
      }
      if constexpr (DO_QK) {
        const int kb = t / NU, u = t % NU;
        s[kb] = QK::mma(ka[t], qf[u], u == 0 ? negm : s[kb]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, LEAD * RD, 0);
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      if (t + LEAD < NMF) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
    }
  };

  // VALU phase: softmax of a tile (S in s[], relative to m_ref; meta its table entry's
  // second word) -> pb, l_run.
  auto softmax = [&](int meta) {
    const int ktok0 = meta >> 8, len = meta & 127;
    const bool diag = (meta & 128) != 0;
    if (diag || len < TK) {   // generated mask: tile end, causal newest slot
      // key kk = 32kb + 8(i/4) + 4h + i%4 is visible iff kk < lim
      const int lim = (diag ? min(len, my_tok - ktok0 + 1) : len) - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) < lim) ? s[kb][i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kb][i], s[kb][i + 1]));
    }
    mx = xhalf_max(mx);
    const bool need = fresh || mx > kTau;
    if (__ballot(need) != 0) {   // first keys of a row, or a row max grew by more than 2^kTau
      const float delta = (need && mx != -INFINITY) ? mx : 0.f;
      const float alpha = fresh ? 0.f : __builtin_amdgcn_exp2f(-delta);   // O, l are 0 if fresh
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] *= alpha;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] -= delta;
      m_ref += delta;
      fresh = fresh && mx == -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) negm[i] = -m_ref;
    }
    float ls[4] = {0.f, 0.f, 0.f, 0.f};   // four partial sums: short dependency chains
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pr = __builtin_amdgcn_exp2f(s[kb][i]);
        s[kb][i] = pr;
        ls[i & 3] += pr;
      }
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      float pv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) pv[e] = s[cc / 2][E * (cc % 2) + e];
      pb[cc] = PV::pack(pv);
    }
  };

  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // tile 0 has landed
  wg_barrier();
  // ---- half-steps st = 0 .. ntiles+1: the group of tile st (st & 1) is in its MFMA phase
  // (QK^T of tile st, PV of tile st-2), the other group in its VALU phase (softmax of tile
  // st-1, then staging of tile st+1 into the slot of tile st-3, whose K was read in MFMA
  // phase st-3 and V in MFMA phase st-1).  Tile indices depend on st only.
  for (int st = 0; st < ntiles + 2; ++st) {
    int stv = st;
    asm volatile("" : "+v"(stv));
    if (((st - grp) & 1) == 0) {
      const bool pv = stv >= 2 && stv - 2 < ntiles, qk = stv < ntiles;
      if (pv && qk) mfma_phase(std::true_type{}, std::true_type{}, st);
      else if (qk) mfma_phase(std::false_type{}, std::true_type{}, st);
      else if (pv) mfma_phase(std::true_type{}, std::false_type{}, st);
    } else if (stv >= 1 && stv - 1 < ntiles) {
      const int meta = jt[st - 1].y;
      if (stv + 1 < ntiles) stage(jt, st + 1);
      softmax(meta);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);   // tile st+1 has landed
    }
    wg_barrier();
  }

  // ---- the next job's first tile (group 0, into slot 3) and query operands, in flight during
  // this epilogue (which uses LDS below slot 3 only)
  pf = 0;
  {
    int vs2 = vstart;
    for (int oi2 = oi + 1; oi2 < p.nseg; ++oi2) {
      const int v2 = sp.order(oi2), nv2 = sp.view_tiles(v2);
      const int ja2 = max(c0, vs2) - vs2, jb2 = min(c1, vs2 + nv2) - vs2;
      vs2 += nv2;
      if (ja2 >= jb2) continue;
      if (grp == 0) stage(tiles + (stt.offset(p.seg0 + v2) + ja2), 0);
      load_q(stt.qrow0(p, p.seg0 + v2));
      pf = 1;
      break;
    }
  }
  static_assert(MBYTES <= 3 * SLOT, "the epilogue leaves slot 3 free");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  wg_barrier();
  // ---- merge the two groups (same rows, disjoint key tiles), then O / l
  const float m_eff = fresh ? -INFINITY : m_ref;
  const float l_half = xhalf_sum(l_run);
  float* mb = reinterpret_cast<float*>(buf) + wr * 32 * (D + 4);
  if (grp == 1) {
    if (lane < 32) {
      red_m[wr][l32] = m_eff;
      red_l[wr][l32] = l_half;
    }
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig)
        *reinterpret_cast<f32x4*>(mb + l32 * (D + 4) + 32 * d + 8 * ig + 4 * h) =
            f32x4{o[d][4 * ig], o[d][4 * ig + 1], o[d][4 * ig + 2], o[d][4 * ig + 3]};
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // LDS only: the prefetched loads stay in flight
  wg_barrier();
  const bool whole = ja == 0 && jb == nv;
  if (grp == 0) {   // combined rows, in place in LDS (normalised if the job covers the view)
    const float m1 = red_m[wr][l32], l1 = red_l[wr][l32];
    const float M = fmaxf(m_eff, m1);
    const float a0 = (m_eff == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_eff - M);
    const float a1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    const float lsum = a0 * l_half + a1 * l1;
    const float inv = whole ? 1.f / lsum : 1.f;
    const float f0 = a0 * inv, f1 = a1 * inv;
    // the other group's rows read all at once, then combined and written back: left to itself
    // the compiler read, waited and wrote one cell at a time (16 serialized LDS round trips)
    f32x4 ov[ND][4];
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) ov[d][ig] = *reinterpret_cast<const f32x4*>(mb + l32 * (D + 4) + 32 * d + 8 * ig + 4 * h);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        f32x4* cell = reinterpret_cast<f32x4*>(mb + l32 * (D + 4) + 32 * d + 8 * ig + 4 * h);
        const f32x4 v = ov[d][ig];
        *cell = f32x4{o[d][4 * ig] * f0 + v[0] * f1, o[d][4 * ig + 1] * f0 + v[1] * f1,
                      o[d][4 * ig + 2] * f0 + v[2] * f1, o[d][4 * ig + 3] * f0 + v[3] * f1};
      }
    }
    if (h == 0) {   // (each lane has read its own entries above)
      red_m[wr][l32] = M;
      red_l[wr][l32] = lsum;
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // LDS only: the prefetched loads stay in flight
  wg_barrier();
  // ---- a view cut once (two pieces, stream_merge_desc) is merged here by whichever of its
  // pieces finishes second.  Both pieces store their partials with device-scope stores, wait for
  // them, and take a ticket on the boundary's counter (device-scope atomic add).  The piece that
  // draws ticket 1 reads the other's stored partial with device-scope loads, quantises its own
  // rows exactly as it stored them, and merges (merge_two, the first piece's values first), so
  // the result has the same bits whichever piece merges.  No piece waits for another.  The
  // second piece is its chunk's first job and the first piece its chunk's last, so it is
  // normally the first piece, on a workgroup that finishes early, that merges; it reads the
  // counter first, and when the second piece's ticket is already there it merges at once
  // without storing its own partial (nobody would read it).
  // Ordering: every access the two workgroups share is a relaxed device-scope atomic (8-byte
  // stores and loads of the partial, the counter's add and load), which the hardware performs
  // at device coherence (written through past the XCD's L2, read from there).  A piece takes its
  // ticket only after s_waitcnt vmcnt(0) on every wave and a barrier, i.e. after all its partial
  // stores have completed, and the merging piece issues its loads of the other's partial only
  // after the counter value it read has returned.  So the merger reads complete data without a
  // release / acquire fence, which at device scope would write back or invalidate the whole L2.
  int role = 0;      // 1: first piece of a view cut once, 2: its second piece
  int which_a = 0;   // role 2: the first piece's slot in its chunk
  if (!whole && mdesc && p.merge_mode != 0) {
    if (jb < nv) {
      const int4 d = mdesc[qb * (p.nseg - 1) + chunk];   // boundary chunk + 1
      role = (d.x == v && (d.y >> 16) == chunk + 1) ? 1 : 0;
    } else {
      const int4 d = mdesc[qb * (p.nseg - 1) + chunk - 1];   // boundary chunk (ja > 0 here)
      role = (d.x == v && (d.y & 0xffff) == chunk - 1 && (d.y >> 16) == chunk) ? 2 : 0;
      which_a = d.z;
    }
  }
  // ---- rows out, 16 bytes per lane and whole rows per group of lanes.  Row r of the block
  // is token tok0 + 32*((r/32)/HPW) + r%32 of query head kvh*G + hsub*HPW + (r/32)%HPW.
  const float* rows = reinterpret_cast<const float*>(buf);
  constexpr int TPQ = D / 8;   // lanes per row of a partial (aligned groups within a wave), 8 values each
  // lane c of its group holds 8 values of a row, scaled by that row's power of two 2^sc (the
  // largest magnitude over the row's lanes) and rounded to fp16: the stored partial's values.
  // Each thread covers rows rb + RPQ*k; all of them are read from LDS before any is scaled.
  constexpr int RPQ = 512 / TPQ, NPQ = 128 / RPQ;
  const int qc = tid % TPQ, rb = tid / TPQ;
  f32x4 qv[NPQ][2];
  auto read_rows = [&]() {
#pragma unroll
    for (int k = 0; k < NPQ; ++k) {
      const float* src = rows + (rb + RPQ * k) * (D + 4) + 8 * qc;
      qv[k][0] = *reinterpret_cast<const f32x4*>(src);
      qv[k][1] = *reinterpret_cast<const f32x4*>(src + 4);
    }
  };
  auto quant_rows = [&](u32x4 (&pk)[NPQ], int (&sc)[NPQ]) {
    float mx[NPQ];
#pragma unroll
    for (int k = 0; k < NPQ; ++k) {
      mx[k] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) mx[k] = fmaxf(mx[k], fmaxf(fabsf(qv[k][0][e]), fabsf(qv[k][1][e])));
    }
#pragma unroll
    for (int o = 1; o < TPQ; o <<= 1)
#pragma unroll
      for (int k = 0; k < NPQ; ++k) mx[k] = fmaxf(mx[k], __shfl_xor(mx[k], o));
#pragma unroll
    for (int k = 0; k < NPQ; ++k) {
      sc[k] = partial_row_scale(mx[k]);
      const float mul = exp2_int(sc[k]);
      float x8[8] = {qv[k][0][0], qv[k][0][1], qv[k][0][2], qv[k][0][3],
                     qv[k][1][0], qv[k][1][1], qv[k][1][2], qv[k][1][3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) x8[e] *= mul;
      pk[k] = F16Ops::pack(x8);
    }
  };
  if (whole) {
    // every row this thread writes read from LDS first, then stored (one LDS round trip, not one
    // per row pass): TPR lanes per row, 512 / TPR rows per pass
    auto store_rows = [&](auto bf16_out) {
      constexpr bool B16 = decltype(bf16_out)::value;
      constexpr int TPR = B16 ? D / 8 : D / 4, RPP = 512 / TPR, NPASS = 128 / RPP, NV = B16 ? 2 : 1;
      const int c = tid % TPR, r0 = tid / TPR;
      f32x4 vals[NPASS][NV];
#pragma unroll
      for (int k = 0; k < NPASS; ++k)
#pragma unroll
        for (int j = 0; j < NV; ++j)
          vals[k][j] = *reinterpret_cast<const f32x4*>(rows + (r0 + RPP * k) * (D + 4) + (B16 ? 8 * c + 4 * j : 4 * c));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NPASS; ++k) {
        const int r = r0 + RPP * k, ww = r >> 5, tk = tok0 + 32 * (ww / p.HPW) + (r & 31);
        if (tk >= p.qtok || hsub * p.HPW + (ww % p.HPW) >= p.G) continue;
        const int hd = kvh * p.G + hsub * p.HPW + (ww % p.HPW);
        const int64_t obase = (static_cast<int64_t>(qrow0 + tk) * p.Hq + hd) * D;
        if constexpr (B16) {
          float x8[8] = {vals[k][0][0], vals[k][0][1], vals[k][0][2], vals[k][0][3],
                         vals[k][1][0], vals[k][1][1], vals[k][1][2], vals[k][1][3]};
          st16(static_cast<bf16*>(out) + obase + 8 * c, BF16Ops::pack(x8));
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + obase + 4 * c) = vals[k][0];
        }
      }
    };
    if (p.out_bf16) store_rows(std::true_type{});
    else store_rows(std::false_type{});
  } else {   // this job's piece of view v: unnormalised O scaled per row and rounded to fp16,
             // then (row max M, row sum l, 1 / scale) (stream_slot)
    unsigned* const cnt = role != 0 ? flags + rbi * p.nseg + (role == 1 ? chunk + 1 : chunk) : nullptr;
    bool merge_now = false;   // merge the view here, from this piece's rows and the other's partial
    if (role == 1) {   // a first piece whose second piece has taken its ticket merges at once, storing nothing
      if (tid == 0) s_ready = static_cast<int>(__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      wg_barrier();
      merge_now = s_ready != 0;
    }
    if (!merge_now) {
      float* slot = stream_slot<D>(part, p, rbi, chunk, (sv + ja == c0) ? 0 : 1);   // first job, or last
      u32x4 pkq[NPQ];
      int scq[NPQ];
      read_rows();
      __builtin_amdgcn_sched_barrier(0);
      quant_rows(pkq, scq);
#pragma unroll
      for (int k = 0; k < NPQ; ++k) {
        const int r = rb + RPQ * k, c = qc;
        const u32x4 pk = pkq[k];
        const f32x4 mlv = f32x4{red_m[r >> 5][r & 31], red_l[r >> 5][r & 31], exp2_int(-scq[k]), 0.f};
        uint64_t* dst = reinterpret_cast<uint64_t*>(reinterpret_cast<_Float16*>(slot) + r * D);   // partial_col
        const uint64_t lo = (static_cast<uint64_t>(pk[1]) << 32) | pk[0], hi = (static_cast<uint64_t>(pk[3]) << 32) | pk[2];
        if (role != 0) {   // read by the other piece's workgroup within this launch: device scope
          __hip_atomic_store(dst + c, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(dst + TPQ + c, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (c == 0) {
            uint64_t* mdst = reinterpret_cast<uint64_t*>(slot + 64 * D + 4 * r);
            __hip_atomic_store(mdst, (static_cast<uint64_t>(__float_as_uint(mlv[1])) << 32) | __float_as_uint(mlv[0]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mdst + 1, static_cast<uint64_t>(__float_as_uint(mlv[2])), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          dst[c] = lo;
          dst[TPQ + c] = hi;
          if (c == 0) *reinterpret_cast<f32x4*>(slot + 64 * D + 4 * r) = mlv;
        }
      }
      if (role != 0) {   // every lane's stores complete, then the ticket
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        wg_barrier();
        if (tid == 0) {
          if (role == 2 && p.merge_mode == 2)   // test mode: the second piece lets the first take ticket 0
            for (int i = 0; i < kMergeTestPolls && __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u; ++i)
              __builtin_amdgcn_s_sleep(16);
          s_ready = static_cast<int>(__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        wg_barrier();
        merge_now = s_ready == 1;   // the other piece's partial is stored
      }
    }
    if (merge_now) {
      const float* other = role == 1 ? stream_slot<D>(part, p, rbi, chunk + 1, 0)
                                     : stream_slot<D>(part, p, rbi, chunk - 1, which_a);
      // the other piece's rows and this piece's rows all requested before the first is used
      uint64_t o0[NPQ], o1[NPQ], om[NPQ], os[NPQ];
#pragma unroll
      for (int k = 0; k < NPQ; ++k) {
        const int r = rb + RPQ * k;
        const uint64_t* osrc = reinterpret_cast<const uint64_t*>(reinterpret_cast<const _Float16*>(other) + r * D);
        const uint64_t* oml = reinterpret_cast<const uint64_t*>(other + 64 * D + 4 * r);
        o0[k] = __hip_atomic_load(osrc + qc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // partial_col
        o1[k] = __hip_atomic_load(osrc + TPQ + qc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        om[k] = __hip_atomic_load(oml, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        os[k] = __hip_atomic_load(oml + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      read_rows();
      __builtin_amdgcn_sched_barrier(0);
      u32x4 ownq[NPQ];
      int scq[NPQ];
      quant_rows(ownq, scq);
#pragma unroll
      for (int k = 0; k < NPQ; ++k) {
        const int r = rb + RPQ * k, c = qc;
        const u32x4 own = ownq[k];
        const float m_o = __uint_as_float(static_cast<uint32_t>(om[k])), l_o = __uint_as_float(static_cast<uint32_t>(om[k] >> 32));
        const float s_o = __uint_as_float(static_cast<uint32_t>(os[k]));
        const float m_s = red_m[r >> 5][r & 31], l_s = red_l[r >> 5][r & 31], s_s = exp2_int(-scq[k]);
        const u32x2 x_o0{static_cast<uint32_t>(o0[k]), static_cast<uint32_t>(o0[k] >> 32)};
        const u32x2 x_o1{static_cast<uint32_t>(o1[k]), static_cast<uint32_t>(o1[k] >> 32)};
        const u32x2 x_s0{own[0], own[1]}, x_s1{own[2], own[3]};
        const f32x4 r0 = role == 1 ? merge_two(m_s, l_s, s_s, x_s0, m_o, l_o, s_o, x_o0)
                                   : merge_two(m_o, l_o, s_o, x_o0, m_s, l_s, s_s, x_s0);
        const f32x4 r1 = role == 1 ? merge_two(m_s, l_s, s_s, x_s1, m_o, l_o, s_o, x_o1)
                                   : merge_two(m_o, l_o, s_o, x_o1, m_s, l_s, s_s, x_s1);
        const int ww = r >> 5, tk = tok0 + 32 * (ww / p.HPW) + (r & 31);
        if (tk >= p.qtok || hsub * p.HPW + (ww % p.HPW) >= p.G) continue;
        const int hd = kvh * p.G + hsub * p.HPW + (ww % p.HPW);
        const int64_t obase = (static_cast<int64_t>(qrow0 + tk) * p.Hq + hd) * D + 8 * c;
        store_out4(out, p.out_bf16, obase, r0);
        store_out4(out, p.out_bf16, obase + 4, r1);
      }
    }
  }
  wg_barrier();   // LDS is reused by the next job (this job's output stores drain meanwhile)
  }   // jobs
}

template <int D>
__global__ __launch_bounds__(512) void stream_pp_kernel(const KParams p, const _Float16* __restrict__ qrot,
                                                        const _Float16* __restrict__ krot,
                                                        const bf16* __restrict__ vc, void* __restrict__ out,
                                                        float* __restrict__ part, const int2* __restrict__ tiles,
                                                        const int4* __restrict__ mdesc, unsigned* __restrict__ flags) {
  stream_pp_body<D>(p, blockIdx.x, qrot, krot, vc, out, part, tiles, mdesc, flags);
}

// Two launches of the attention kernel in one, for a cold start: workgroups [0, n0) run the frame
// segments (p0), the rest the prefix segment (p1).  The prefix's short jobs come last, after the
// frames' longest-first order (and longest first among themselves), and fill the tail of that
// launch instead of a launch of their own on half the CUs.
template <int D>
__global__ __launch_bounds__(512) void stream_pp2_kernel(const KParams p0, const KParams p1, const int n0,
                                                         const _Float16* __restrict__ qrot,
                                                         const _Float16* __restrict__ krot,
                                                         const bf16* __restrict__ vc, void* __restrict__ out,
                                                         const int2* __restrict__ tiles) {
  const int b = blockIdx.x;
  if (b < n0) {
    stream_pp_body<D>(p0, b, qrot, krot, vc, out, nullptr, tiles, nullptr, nullptr);
  } else {   // the prefix's row blocks last token block first: the longest key ranges start first
    const int hb = p1.Hkv * p1.n_hsub, bp = b - n0;
    stream_pp_body<D>(p1, (p1.nqb - 1 - bp / hb) * hb + bp % hb, qrot, krot, vc, out, nullptr, tiles, nullptr, nullptr);
  }
}

// ---------------------------------------------------------------------------------------
// K/V projection of the new frames with the ring-slot insert as its epilogue (bf16).
// C[m][n] = sum_k X[m][k] W[n][k]: m = v*T + i the token i of view v's new frame (X
// [V*T][hidden]), n the output feature (W [2*Hkv*D][hidden], one feature per row as a linear
// layer stores it): n < Hkv*D is K head n/D, dimension n%D; the next Hkv*D are V.  The fp32
// sums are rounded to bf16 and written pre-RoPE straight into the cache rows of ring slot s:
// row P + (v*F + s)*T + i of head n/D (Technical Summary, 5. System Optimizations, "Kernel
// Fusion"; Methodology 1, "Token Layout").
// Workgroup tile 64 (m) x 128 (n), eight waves of 32 x 32 (two per SIMD, so one wave's LDS
// reads overlap the other's MFMAs), k in chunks of 64; both tiles go straight to LDS (direct
// loads) through a ring of kPS stages, two chunks in flight while one is multiplied.  Rows of
// 64 bf16 (128 B, eight 16-byte chunks) with chunk c of row r at position c ^ ((r >> 1) & 7),
// so the 16 rows one operand read touches land in 16 distinct bank groups.
// v_mfma_f32_32x32x16_bf16: A = 32 rows of X, B = 32 rows of W (both k-contiguous).
// ---------------------------------------------------------------------------------------
constexpr int kPM = 64, kPN = 128, kPK = 64, kPS = 4, kPW = 8;
__device__ inline uint32_t proj_swz(uint32_t r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(64 * kPW) void kv_project_kernel(const KParams p, int hidden, int slot,
                                                         const bf16* __restrict__ x, const bf16* __restrict__ w,
                                                         bf16* __restrict__ kc, bf16* __restrict__ vc) {
  constexpr int ROWB = kPK * 2;                 // 128 bytes per staged row
  constexpr int ABYTES = kPM * ROWB, BBYTES = kPN * ROWB, STAGE = ABYTES + BBYTES;   // 8 + 16 KB
  constexpr int NA = ABYTES / 1024, NL = STAGE / 1024 / kPW;   // A instructions; loads per wave
  static_assert(STAGE % (1024 * kPW) == 0, "whole 1 KB loads per wave");
  __shared__ __attribute__((aligned(16))) unsigned char buf[kPS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int M = p.V * p.T, N = 2 * p.Hkv * p.D;
  const int nblk = N / kPN;
  const int m0 = (blockIdx.x / nblk) * kPM, n0 = (blockIdx.x % nblk) * kPN;
  const int wm = (wv >> 2) * 32, wn = (wv & 3) * 32;   // this wave's 32 x 32 sub-tile
  uint32_t ln = lane;
  asm volatile("" : "+v"(ln));
  // direct loads: instruction j of a stage fills staged rows 8j .. 8j+7 (1 KB) of A (j < 8)
  // or of B (j - 8); lane i takes row 8j + i/8 and fetches its chunk (i%8) ^ swz(row).  Wave
  // w issues instructions NL*w .. NL*w + NL-1.  Global offsets per lane are fixed; the k chunk
  // moves the base.
  const uint32_t rowb = static_cast<uint32_t>(hidden) * 2;
  uint32_t off[NL];
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int j = NL * wv + q;
    const uint32_t r = 8 * (j < NA ? j : j - NA) + ln / 8;
    const int row = j < NA ? min(m0 + static_cast<int>(r), M - 1)   // rows past M repeat the last
                           : n0 + static_cast<int>(r);
    off[q] = static_cast<uint32_t>(row) * rowb + (((ln % 8) ^ proj_swz(r)) << 4);
  }
  const uint32_t lds0 = lds_addr(buf);
  auto stage = [&](int kc_, int sb) {
    const unsigned char* xa = uni_ptr(reinterpret_cast<const unsigned char*>(x) + static_cast<int64_t>(kc_) * ROWB);
    const unsigned char* wb = uni_ptr(reinterpret_cast<const unsigned char*>(w) + static_cast<int64_t>(kc_) * ROWB);
    const uint32_t la = lds0 + sb * STAGE;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int j = NL * wv + q;
      g2lds16_async(j < NA ? xa : wb, off[q], __builtin_amdgcn_readfirstlane(la + j * 1024));
    }
  };

  f32x16 acc = f32x16{};
  const int nk = hidden / kPK;
  for (int c = 0; c < kPS - 1 && c < nk; ++c) stage(c, c);
  for (int kk = 0; kk < nk; ++kk) {
    // chunk kk has landed once at most the loads of the chunks issued after it are pending
    static_assert(kPS <= 4, "waits below cover at most two chunks in flight");
    switch (min(kPS - 2, nk - 1 - kk)) {
      case 2: __builtin_amdgcn_s_waitcnt(wait_vm(2 * NL)); break;
      case 1: __builtin_amdgcn_s_waitcnt(wait_vm(NL)); break;
      default: __builtin_amdgcn_s_waitcnt(kWaitVm0); break;
    }
    wg_barrier();   // ... for every wave; and every wave is done with chunk kk-1
    const int sb = kk % kPS;
    if (kk + kPS - 1 < nk) stage(kk + kPS - 1, (kk + kPS - 1) % kPS);   // the slot of chunk kk-1
    const unsigned char* A = buf + sb * STAGE;
    const unsigned char* B = A + ABYTES;
#pragma unroll
    for (int u = 0; u < kPK / 16; ++u) {   // 16-wide k steps: chunk 2u + h
      const uint32_t ra = wm + l32;
      const u32x4 a = ld16(A + ra * ROWB + (((2 * u + h) ^ proj_swz(ra)) << 4));
      const uint32_t rb = wn + l32;
      const u32x4 b = ld16(B + rb * ROWB + (((2 * u + h) ^ proj_swz(rb)) << 4));
      acc = BF16Ops::mma(a, b, acc);
    }
  }

  // epilogue: lane l32 holds feature n = n0 + wn + l32 of tokens m = m0 + wm + 8(i/4) + 4h
  // + i%4; 32 lanes write 32 consecutive dimensions of one head (64 contiguous bytes)
  const int n = n0 + wn + l32;
  const int kv = n / (p.Hkv * p.D), hd = (n / p.D) % p.Hkv, d = n % p.D;
  bf16* dst = kv == 0 ? kc : vc;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + wm + 8 * (i >> 2) + 4 * h + (i & 3);
    if (m >= M) continue;
    const int v = m / p.T, ti = m - v * p.T;
    const int64_t row = p.P + static_cast<int64_t>(v * p.F + slot) * p.T + ti;
    dst[(static_cast<int64_t>(hd) * p.S_cap + row) * p.D + d] = static_cast<bf16>(acc[i]);
  }
}

// ---------------------------------------------------------------------------------------
// Verify, split-KV part.  Rows: r = hh*B + b (query head kvh*G + hh, block token b), in
// 32-row MFMA blocks, one workgroup per (kv head, row block, split).  Keys are numbered by cache row x: window rows [0, W), reasoning rows
// [W, W+n_tail), block rows [W+n_tail, W+n_tail+B) (read from k_blk / v_blk and copied into
// the cache here).  They are cut into 32-key blocks inside segments of contiguous
// positions; wave w of split s takes block (s*4 + w): its K rows are loaded straight into
// registers (lane l32 holds key l32, both halves of every RoPE pair) and rotated there, its
// V rows go through a per-wave swizzled V^T tile in LDS.  All global loads are issued
// before the rotation tables are built.  The four waves merge in LDS and the workgroup
// writes one (m, l, O) partial per (kv head, split).
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void verify_split_kernel(const KParams p, const T* __restrict__ qb,
                                                           const T* __restrict__ kb,
                                                           const T* __restrict__ vb, T* __restrict__ kc,
                                                           T* __restrict__ vc, float* __restrict__ part) {
  using In = typename Path<T>::In;
  using QK = typename Path<T>::QK;
  using PV = typename Path<T>::PV;
  constexpr int E = QK::E;
  constexpr int H2 = D / 2;
  constexpr int NU = D / (2 * E);
  constexpr int ND = D / 32;
  constexpr int CPB = 32 / (2 * E);
  constexpr int VROW = 32 * static_cast<int>(sizeof(T));   // V^T row: 32 keys
  constexpr int SWM = VROW / 16 >= 8 ? 7 : VROW / 16 - 1;  // chunk swizzle mask
  constexpr int DCH = D / E;
  constexpr int NVI = (8 * DCH + 63) / 64;
  constexpr int RS = H2 + 2;                               // padded offset-table row (float2)
  constexpr int OS = D + 4;
  constexpr int VB = 4 * D * VROW;
  constexpr int OB = 2 * 32 * OS * 4;
  constexpr int UB = VB > OB ? VB : OB;

  __shared__ float2 csA[4][H2];     // cos/sin(8a f_i)
  __shared__ float2 csB[8][H2];     // cos/sin(b f_i)
  __shared__ __attribute__((aligned(16))) float2 csr[32][RS];  // cos/sin(r f_i), r < 32
  __shared__ float2 csq[H2];        // cos/sin(first block position * f_i)
  __shared__ float2 csb[4][H2];     // cos/sin(key block base * f_i), one per wave
  __shared__ float red_m[4][32], red_l[4][32];
  __shared__ __attribute__((aligned(16))) unsigned char ubuf[UB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  // blockIdx.x = (split * n_rb + rb) * Hkv + kvh: the row blocks of one split run side by
  // side on one XCD and read the same K / V
  const int kvh = blockIdx.x % p.Hkv, rb = (blockIdx.x / p.Hkv) % p.n_rb, split = blockIdx.x / (p.Hkv * p.n_rb);
  const int qr = 32 * rb + l32, hh = qr / p.B, bq = qr % p.B;   // query row qr = hh*B + b
  const bool qvalid = hh < p.G;
  const int head = kvh * p.G + hh;
  const int tailbase = p.W + p.n_tail;  // cache row of block token 0
  const float sc = p.sm_scale_log2;

  // ---- this wave's key block
  const int nbp = (p.P + 31) / 32, nbs = (p.T + 31) / 32, nslot = p.V * p.F;
  const int j = split * kVerifyWaves + w;
  int x0 = 0, len = 0;
  int64_t pos0 = 0;
  if (j < p.nblk) {
    if (j < nbp) {
      x0 = 32 * j;
      len = min(32, p.P - x0);
      pos0 = p.pos_base + x0;
    } else if (j - nbp < nslot * nbs) {
      const int jj = j - nbp, vs = jj / nbs, st = 32 * (jj % nbs);
      x0 = p.P + vs * p.T + st;
      len = min(32, p.T - st);
      pos0 = slot_pos(p, vs / p.F, vs % p.F) + st;
    } else {
      const int st = 32 * (j - nbp - nslot * nbs);
      x0 = p.W + st;
      len = min(32, p.n_tail + p.B - st);
      pos0 = p.pos_base + p.W + st;
    }
  }

  // ---- issue every global load first
  u32x4 qraw[NU], kraw[NU];
  const int xk = x0 + l32;
  const bool kvalid = l32 < len;
  const bool k_from_blk = xk >= tailbase;
  {
    const T* qsrc = qb + (static_cast<int64_t>(bq) * p.Hq + head) * D;
    const T* ksrc = k_from_blk ? kb + (static_cast<int64_t>(xk - tailbase) * p.Hkv + kvh) * D
                               : kc + (static_cast<int64_t>(kvh) * p.S_cap + xk) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      qraw[u] = qvalid ? ld16(qsrc + 2 * E * u + E * h) : u32x4{};
      kraw[u] = kvalid ? ld16(ksrc + 2 * E * u + E * h) : u32x4{};
    }
  }
  u32x4 rv[NVI][4];
#pragma unroll
  for (int jv = 0; jv < NVI; ++jv) {
    const int it = lane + 64 * jv;
    const int dc = it % DCH, kg = it / DCH;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int key = 4 * kg + jj, x = x0 + key;
      rv[jv][jj] = u32x4{};
      if (it < 8 * DCH && key < len) {
        const T* src = x >= tailbase ? vb + (static_cast<int64_t>(x - tailbase) * p.Hkv + kvh) * D
                                     : vc + (static_cast<int64_t>(kvh) * p.S_cap + x) * D;
        rv[jv][jj] = ld16(src + E * dc);
        if (x >= tailbase && rb == 0) st16(vc + (static_cast<int64_t>(kvh) * p.S_cap + x) * D + E * dc, rv[jv][jj]);
      }
    }
  }
  if (kvalid && k_from_blk && rb == 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) st16(kc + (static_cast<int64_t>(kvh) * p.S_cap + xk) * D + 2 * E * u + E * h, kraw[u]);
  }

  // ---- rotation tables (overlap the loads in flight)
  for (int e = tid; e < 12 * H2; e += 256) {
    const int a = e / H2, i = e % H2;
    if (a < 4) csA[a][i] = cs_angle(8.0 * a * p.inv_freq[i]);
    else csB[a - 4][i] = cs_angle(static_cast<double>(a - 4) * p.inv_freq[i]);
  }
  if (tid < H2) csq[tid] = cs_angle(static_cast<double>(p.pos_base + tailbase) * p.inv_freq[tid]);
  if (lane < H2) csb[w][lane] = cs_angle(static_cast<double>(pos0) * p.inv_freq[lane]);
  __syncthreads();
  for (int e = tid; e < 32 * H2; e += 256) {
    const int r = e / H2, i = e % H2;
    csr[r][i] = cmul(csA[r >> 3][i], csB[r & 7][i]);
  }
  __syncthreads();

  // ---- rotate Q and K in registers (chunks u and u + NU/2 hold the two halves of a pair)
  u32x4 qf[NU], kf[NU];
  {
    float fq[NU][E], fk[NU][E];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      In::unpack(qraw[u], fq[u]);
      In::unpack(kraw[u], fk[u]);
    }
#pragma unroll
    for (int u = 0; u < NU / 2; ++u) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = 2 * E * u + E * h + e;
        const float2 cq = cmul(csq[i], csr[bq][i]);
        const float2 ck = cmul(csb[w][i], csr[l32][i]);
        float a = fq[u][e], b = fq[u + NU / 2][e];
        fq[u][e] = a * cq.x - b * cq.y;
        fq[u + NU / 2][e] = b * cq.x + a * cq.y;
        a = fk[u][e];
        b = fk[u + NU / 2][e];
        fk[u][e] = a * ck.x - b * ck.y;
        fk[u + NU / 2][e] = b * ck.x + a * ck.y;
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      qf[u] = QK::pack(fq[u]);
      kf[u] = QK::pack(fk[u]);
    }
  }
  f32x16 s = f32x16{};
#pragma unroll
  for (int u = 0; u < NU; ++u) s = QK::mma(kf[u], qf[u], s);

  float m_run = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kk = 8 * (i >> 2) + 4 * h + (i & 3);
    const bool ok = (kk < len) & ((x0 + kk - tailbase) <= bq);
    s[i] = ok ? s[i] * sc : -INFINITY;
    m_run = fmaxf(m_run, s[i]);
  }
  m_run = fmaxf(m_run, __shfl_xor(m_run, 32));
  const float mu = (m_run == -INFINITY) ? 0.f : m_run;
  float l_run = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pr = __builtin_amdgcn_exp2f(s[i] - mu);
    s[i] = pr;
    l_run += pr;
  }

  // ---- V^T block of this wave in LDS, then O^T = V^T P^T
  unsigned char* Vw = ubuf + w * D * VROW;
#pragma unroll
  for (int jv = 0; jv < NVI; ++jv) {
    const int it = lane + 64 * jv;
    if (it < 8 * DCH) store_vt<T, E, SWM>(Vw, VROW, E * (it % DCH), it / DCH, rv[jv]);
  }
  __syncthreads();
  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x16{};
#pragma unroll
  for (int c = 0; c < CPB; ++c) {
    float pv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) pv[e] = s[E * c + e];
    const u32x4 bop = PV::pack(pv);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int dr = 32 * d + l32;
      o[d] = PV::mma(ld16(Vw + dr * VROW + (((2 * c + h) ^ (vswz(dr) & SWM)) << 4)), bop, o[d]);
    }
  }
  __syncthreads();   // V^T tiles are dead: the space is reused for the merge

  // ---- merge the four waves (same rows, different keys)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (lane < 32) {
    red_m[w][l32] = m_run;
    red_l[w][l32] = l_tot;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, red_m[ww][l32]);
  float L = 0.f;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww)
    if (red_m[ww][l32] != -INFINITY) L += red_l[ww][l32] * __builtin_amdgcn_exp2f(red_m[ww][l32] - M);
  const float scale = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  float* obuf = reinterpret_cast<float*>(ubuf);
  float* ob = obuf + (w & 1) * 32 * OS;
  if (w < 2) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const f32x4 r = {o[d][4 * ig] * scale, o[d][4 * ig + 1] * scale, o[d][4 * ig + 2] * scale, o[d][4 * ig + 3] * scale};
        *reinterpret_cast<f32x4*>(ob + l32 * OS + 32 * d + 8 * ig + 4 * h) = r;
      }
  }
  __syncthreads();
  if (w >= 2) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        f32x4* dst = reinterpret_cast<f32x4*>(ob + l32 * OS + 32 * d + 8 * ig + 4 * h);
        const f32x4 r = {o[d][4 * ig] * scale, o[d][4 * ig + 1] * scale, o[d][4 * ig + 2] * scale, o[d][4 * ig + 3] * scale};
        *dst = *dst + r;
      }
  }
  __syncthreads();
  float* dstp = part + ((static_cast<int64_t>(kvh) * p.n_rb + rb) * p.n_split + split) * verify_partial_words(D);
  for (int e = tid; e < 32 * D / 4; e += 256) {
    const int r = e / (D / 4), c = e % (D / 4);
    const f32x4 a = *reinterpret_cast<const f32x4*>(obuf + r * OS + 4 * c);
    const f32x4 b = *reinterpret_cast<const f32x4*>(obuf + 32 * OS + r * OS + 4 * c);
    *reinterpret_cast<f32x4*>(dstp + r * D + 4 * c) = a + b;
  }
  if (w == 0 && lane < 32) {
    dstp[32 * D + l32] = M;
    dstp[32 * D + 32 + l32] = L;
  }
}

// ---------------------------------------------------------------------------------------
// Verify for bf16 inputs, split-KV part.  A call verifies n_drafts draft blocks of B tokens over
// one window.  Draft d's query rows r = hh*B + b (query head kvh*G + hh, block token b) form nrb_d
// 32-row MFMA blocks; row block rb (of draft rb / nrb_d) attends to the window's keys and then to
// its own draft's tail: reasoning rows W + d*tail_stride + [0, n_tails[d]) and the block rows
// after them, which are read from k_blk / v_blk (and copied into the cache here).  Keys are cut
// into 32-key blocks inside segments of contiguous positions (the prefix, each frame slot, the
// tail).  One workgroup per (kv head, row block, split); its NW waves take one key block each.
//
// Every global read of a workgroup is issued up front, straight into LDS (global_load_lds from
// per-lane addresses): the row block's raw query rows (each wave fetches a share), then each
// wave's K block, then its V block.  Vector memory operations complete in issue order, so a wave
// waits for its queries and keys alone, rotates them and runs Q K^T and the softmax while its
// values are still landing; only P V waits for them.
//   * The queries are rotated once per workgroup, cooperatively, in LDS.
//   * A key's angle is its block's base angle (in revolutions, fraction taken in fp64 once per
//     wave and frequency) plus its offset in the block times the frequency (fp32), then the
//     hardware sin / cos.
//   * With a rotated window view (VIEW), window blocks arrive already rotated (fp16) and only
//     tail blocks are rotated here.
// The waves fold into one (m, l, O) partial per (kv head, row block, split), in a fixed order;
// verify_merge_kernel combines the splits.
// ---------------------------------------------------------------------------------------

// Direct global -> LDS load of 16 bytes per lane from a per-lane 64-bit global address (no scalar
// base register), landing at LDS lds + 16*lane (lds wave-uniform).  From inline assembly: the
// compiler does not see the load, so the caller orders it with explicit s_waitcnt vmcnt; one
// wait state follows the write of M0.
__device__ inline void g2lds16_va(const void* gaddr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gaddr), "{m0}"(lds) : "memory");
}

// Key block j of a row block of draft d (the window's blocks, then the draft's tail blocks):
// first cache row, length (0: past the list), position of its first key, and the cache row of
// the draft's block token 0 (rows from there on come from k_blk / v_blk).
struct VerifyBlock {
  int x0, len, tailbase;
  int64_t pos0;
};
__device__ inline VerifyBlock verify_block(const KParams& p, int d, int j) {
  const int nbp = (p.P + 31) / 32, nbs = (p.T + 31) / 32, nslot = p.V * p.F;
  const int trow0 = p.W + d * p.tail_stride, ntd = p.n_tails[d];
  VerifyBlock b{0, 0, trow0 + ntd, 0};
  if (j < nbp) {
    b.x0 = 32 * j;
    b.len = min(32, p.P - b.x0);
    b.pos0 = p.pos_base + b.x0;
  } else if (j - nbp < nslot * nbs) {
    const int jj = j - nbp, vs = jj / nbs, st = 32 * (jj % nbs);
    b.x0 = p.P + vs * p.T + st;
    b.len = min(32, p.T - st);
    b.pos0 = slot_pos(p, vs / p.F, vs % p.F) + st;
  } else {
    const int st = 32 * (j - nbp - nslot * nbs);
    if (st < ntd + p.B) {
      b.x0 = trow0 + st;
      b.len = min(32, ntd + p.B - st);
      b.pos0 = p.pos_base + p.W + st;
    }
  }
  return b;
}

// s_waitcnt vmcnt(n) for a wave-uniform n that is a multiple of NIB up to 4*NIB (the
// immediate-operand form for each case)
template <int NIB>
__device__ inline void wait_vm_blocks(int nblk) {
  static_assert(4 * NIB < 64, "vmcnt field");
  switch (nblk) {
    case 0: __builtin_amdgcn_s_waitcnt(wait_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(wait_vm(NIB)); break;
    case 2: __builtin_amdgcn_s_waitcnt(wait_vm(2 * NIB)); break;
    case 3: __builtin_amdgcn_s_waitcnt(wait_vm(3 * NIB)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vm(4 * NIB)); break;
  }
}

// Speculative verify, bf16 inputs: the split-KV kernel.  blockIdx.x = unit * Hkv + kvh, so the
// units of one kv head run on one XCD (round-robin dispatch over 8 XCDs, Hkv a multiple of 8).
// Unit u < n_ws covers the window's key blocks [8u, 8u + 8) for every row block of every
// draft: the window's K and V are read once per call, however many drafts.  Unit
// n_ws + d*n_ts + t covers draft d's tail blocks [8t, 8t + 8) (its reasoning rows, then its
// block rows) for draft d's row blocks.  Five waves, one 32-key block each (248 workgroups at
// the backbone shapes: every CU busy), loaded straight into LDS: K first, V once the rotation tables are built and the queries
// rotated, so that work runs while K lands.  A key's rotation is the product of its block's
// base angle (fp64 fraction, one per frequency) and a shared table of (cos, sin)(r f) for the
// 32 offsets r of a block.  Per row block: every wave computes S^T = K Q^T for its block; the
// row maxima meet in LDS; each wave writes P = 2^(S - M) (bf16) for its block to LDS; wave
// w < D/32 then computes O^T = V^T P^T for d-slice w over all the unit's blocks, so O is never
// folded across waves, and the unit's partial (O in accumulator order, the row max M, the row
// sum) goes to the workspace for verify_merge_dma_kernel.
template <int D, bool VIEW>
__global__ __launch_bounds__(64 * kVerifyWavesDma) void verify_dma_kernel(
    const KParams p, const bf16* __restrict__ qb, const bf16* __restrict__ kb, const bf16* __restrict__ vb,
    bf16* __restrict__ kc, bf16* __restrict__ vc, const _Float16* __restrict__ kview, float* __restrict__ part) {
  using QK = F16Ops;
  using PV = BF16Ops;
  constexpr int NW = kVerifyWavesDma;            // waves, one 32-key block each
  constexpr int NT = 64 * NW;
  constexpr int NB = kVerifyUnitBlocks;          // blocks per workgroup
  constexpr int E = 8;
  constexpr int H2 = D / 2;
  constexpr int NU = D / 16;                     // QK^T k-steps (chunks 2u + h)
  constexpr int NS = D / 32;                     // d-slices of O (one 32x32 accumulator each)
  constexpr int ROWB = D * 2;                    // K / V / Q row bytes
  constexpr int KCH = ROWB / 16;                 // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;               // rows per 1 KB direct load
  constexpr int BLKB = 32 * ROWB;                // 32 rows of K, V or Q
  constexpr int NIB = BLKB / 1024;               // direct loads per 32 rows
  constexpr int QR = 7;                          // row blocks whose queries are resident at once
  constexpr int KPR = 16 / KCH;                  // rows per 256-byte bank row
  constexpr int PBYTES = NB * 2 * 1024 > H2 * 32 * 8 ? NB * 2 * 1024 : H2 * 32 * 8;   // P^T operands;
                                                 // first the angle table
  static_assert(NB == NW && NS <= NW, "work split");
  auto kswz = [](uint32_t r) { return (r / KPR) & (KCH - 1); };
  auto vswz = [](uint32_t key) { return 4 * ((key / KPR) & (KCH / 4 - 1)); };
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };

  __shared__ __attribute__((aligned(16))) unsigned char ktile[NB * BLKB];
  __shared__ __attribute__((aligned(16))) unsigned char vtile[NB * BLKB];
  __shared__ __attribute__((aligned(16))) unsigned char qbuf[QR * BLKB];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[PBYTES];       // first: the angle table
  __shared__ double frev[H2];                    // theta^(-2i/D) / (2 pi): revolutions per position
  __shared__ float2 cbase[NB][H2];               // (cos, sin) of each block's first position
  __shared__ float red_m[NW][32], red_l[NW][32];
  float2* const ang = reinterpret_cast<float2*>(pbuf);   // ang[i*32 + r] = (cos, sin)(r f_i)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  kernarg_early(p.V, p.B, p.tail_stride, p.log2_theta, qb, part);   // lines 0x00 .. 0xc0, the pointers
  const int kvh = blockIdx.x % p.Hkv, unit = blockIdx.x / p.Hkv;
  const bool tail_unit = unit >= p.n_ws;
  const int dt = tail_unit ? (unit - p.n_ws) / p.n_ts : 0;   // a tail unit's draft
  const int tsp = tail_unit ? (unit - p.n_ws) % p.n_ts : 0;   // its tail split
  const int slot = tail_unit ? p.n_ws + tsp : unit;           // its partial slot
  const int rb_lo = tail_unit ? dt * p.nrb_d : 0, rb_hi = tail_unit ? rb_lo + p.nrb_d : p.n_rb;
  const int n_wblk = verify_window_blocks(p.P, p.V, p.F, p.T);
  // block jb of this unit: window block NB*u + jb, or tail block NB*t + jb of draft dt
  auto block = [&](int jb) -> VerifyBlock {
    if (tail_unit) return verify_block(p, dt, n_wblk + NB * tsp + jb);
    const int j = NB * unit + jb;
    return j < n_wblk ? verify_block(p, 0, j) : VerifyBlock{0, 0, p.W, 0};
  };
  // The unit's blocks that hold keys are a prefix of its NB blocks, counted in closed form: every
  // window block holds keys, and draft dt's tail has ceil((n_tails[dt] + B) / 32) blocks.  (Taking
  // block(jb).len for each jb instead put five block descriptors, their divisions and a kernel-
  // argument load with a full wait per block ahead of the first K load: ~2 us of the kernel.)
  const int nbu = tail_unit ? min(NB, ceil_div(p.n_tails[dt] + p.B, kVerifyBlock) - NB * tsp)
                            : min(NB, n_wblk - NB * unit);
  if (nbu <= 0) return;   // a tail split past this draft's tail (whole workgroup)
  const int bmask = uni((1 << nbu) - 1);

  // ---- this wave's block
  const VerifyBlock bk = block(w);
  const int x0 = uni(bk.x0), klen = uni(bk.len), tailb = uni(bk.tailbase);
  const bool rot = !VIEW || x0 >= p.W;

  // ---- queries of row blocks rb0 .. rb0 + nr - 1 into qbuf (row block j at qbuf + j*BLKB):
  // the nr*NIB 1 KB loads go round-robin to the waves; row r of a block at LDS row r with
  // 16-byte chunk c at position c ^ kswz(r); rows past G*B read any valid row (zeroed later)
  const uint32_t lq = lds_addr(qbuf);
  auto load_q = [&](int rb0, int nr) {
    for (int L = w; L < nr * NIB; L += NW) {
      const int rb = rb0 + L / NIB, i = L % NIB;
      const int d = rb / p.nrb_d, rbl = rb - d * p.nrb_d;
      const int r = RPL * i + lane / KCH, pc = lane % KCH;
      const int qr2 = 32 * rbl + r, hh2 = qr2 / p.B;
      const int hq = hh2 < p.G ? hh2 : 0, b2 = hh2 < p.G ? qr2 % p.B : 0;
      const bf16* src = qb + (static_cast<int64_t>(d * p.B + b2) * p.Hq + kvh * p.G + hq) * D;
      g2lds16_va(src + 8 * (pc ^ kswz(r)), uni(lq + L * 1024));
    }
  };
  // ---- K or V of this wave's block.  A whole block of contiguous cache (or view) rows takes one
  // scalar base and the lane's offsets; a ragged block, or one reaching the draft's block rows,
  // takes per-lane addresses with its rows clamped to the last (those keys are masked).
  auto row_of = [&](const bf16* cache, const bf16* blk, int x) -> const unsigned char* {
    return reinterpret_cast<const unsigned char*>(
        x >= tailb ? blk + (static_cast<int64_t>(dt * p.B + x - tailb) * p.Hkv + kvh) * D
                   : cache + (static_cast<int64_t>(kvh) * p.S_cap + x) * D);
  };
  auto load_kv = [&](bool is_v) {
    const uint32_t ldst = uni(lds_addr(is_v ? vtile : ktile) + w * BLKB);
    if (klen == 32 && x0 + 32 <= tailb) {
      const unsigned char* base =
          (!is_v && !rot) ? reinterpret_cast<const unsigned char*>(kview + (static_cast<int64_t>(kvh) * p.W + x0) * D)
                          : reinterpret_cast<const unsigned char*>((is_v ? vc : kc) + (static_cast<int64_t>(kvh) * p.S_cap + x0) * D);
      base = uni_ptr(base);
#pragma unroll
      for (int m = 0; m < NIB; ++m) {
        const uint32_t r = RPL * m + lane / KCH, c = lane % KCH;
        g2lds16_async(base, r * ROWB + 16 * (c ^ (is_v ? vswz(r) : kswz(r))), ldst + m * 1024);
      }
    } else {
      const uint32_t lr = static_cast<uint32_t>(klen - 1);
#pragma unroll
      for (int m = 0; m < NIB; ++m) {
        const uint32_t r = RPL * m + lane / KCH, c = lane % KCH;
        const int x = x0 + static_cast<int>(min(r, lr));
        const unsigned char* src =
            is_v ? row_of(vc, vb, x)
                 : (rot ? row_of(kc, kb, x)
                        : reinterpret_cast<const unsigned char*>(kview + (static_cast<int64_t>(kvh) * p.W + x) * D));
        g2lds16_va(src + 16 * (c ^ (is_v ? vswz(r) : kswz(r))), ldst + m * 1024);
      }
    }
  };

  // ---- the first row blocks' queries and this wave's K in flight (V once the tables are built
  // and the queries rotated: issuing it here would stall that work behind a full load queue)
  const int nr0 = min(QR, rb_hi - rb_lo);
  load_q(rb_lo, nr0);
  if (klen > 0) load_kv(false);

  // ---- rotation tables while K lands: frequencies (fp64), then (cos, sin)(r f_i) for the 32
  // offsets (fp32 revolutions r f_i, hardware sin / cos) and the fraction of each block's base
  // angle pos0 f_i (fp64) through the hardware sin / cos
  if (tid < H2) frev[tid] = exp2(-(2.0 * tid / D) * p.log2_theta) * kInvTwoPi;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  wg_barrier();
  for (int e = tid; e < H2 * 32; e += NT) {
    const int i = e / 32, r = e % 32;
    const float rv = static_cast<float>(r) * static_cast<float>(frev[i]);
    const float f = rv - rintf(rv);
    ang[e] = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
  }
  if (rot && klen > 0 && lane < H2) cbase[w][lane] = cs_rev(static_cast<double>(bk.pos0) * frev[lane]);

  // ---- queries of row blocks rb0 .. rb0 + nr - 1, rotated in place in LDS (fp16, scaled into
  // log2 units; rows past G*B zero): item (row block, row, quarter of the RoPE pairs)
  auto rotate_q = [&](int rb0, int nr) {
    constexpr int QT = 32 * (H2 / 4);   // items per row block
    static_assert(H2 % 4 == 0, "query rotation split");
    for (int it2 = tid; it2 < nr * QT; it2 += NT) {
      const int j = it2 / QT, it = it2 - j * QT, rb = rb0 + j;
      unsigned char* const qb0 = qbuf + j * BLKB;
      const int d = rb / p.nrb_d, rbl = rb - d * p.nrb_d;
      const int r = it / (H2 / 4), i0 = 4 * (it % (H2 / 4));   // pairs (i, i + D/2), i in [i0, i0 + 4)
      const int qr2 = 32 * rbl + r, hh2 = qr2 / p.B, b2 = qr2 % p.B;
      const float qs = hh2 < p.G ? p.sm_scale_log2 : 0.f;
      const double qpos = static_cast<double>(p.pos_base + p.W + p.n_tails[d] + b2);
      // 8-byte halves of the 16-byte chunks holding elements i0 and i0 + D/2
      unsigned char* c1 = qb0 + r * ROWB + (((i0 / E) ^ kswz(r)) << 4) + 2 * (i0 % E);
      unsigned char* c2 = qb0 + r * ROWB + ((((i0 + H2) / E) ^ kswz(r)) << 4) + 2 * (i0 % E);
      const u32x2 a2 = *reinterpret_cast<const u32x2*>(c1), b2v = *reinterpret_cast<const u32x2*>(c2);
      float x1[4], x2[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        x1[2 * j] = __uint_as_float(a2[j] << 16);
        x1[2 * j + 1] = __uint_as_float(a2[j] & 0xffff0000u);
        x2[2 * j] = __uint_as_float(b2v[j] << 16);
        x2[2 * j + 1] = __uint_as_float(b2v[j] & 0xffff0000u);
      }
      _Float16 y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 cq = cs_rev(qpos * frev[i0 + e]);
        const float a = x1[e], b = x2[e];
        y1[e] = static_cast<_Float16>((a * cq.x - b * cq.y) * qs);
        y2[e] = static_cast<_Float16>((b * cq.x + a * cq.y) * qs);
      }
      *reinterpret_cast<u32x2*>(c1) = __builtin_bit_cast(u32x2, y1);
      *reinterpret_cast<u32x2*>(c2) = __builtin_bit_cast(u32x2, y2);
    }
  };
  if (klen > 0) __builtin_amdgcn_s_waitcnt(wait_vm(NIB));   // this wave's query loads have landed
  else __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  wg_barrier();   // every query share, the angle table and the base angles visible
  rotate_q(rb_lo, nr0);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  wg_barrier();   // the rotated queries visible
  if (klen > 0) load_kv(true);

  // ---- K (row l32, both halves of every RoPE pair) into registers: rotated here by
  // (cos, sin)(pos0 f) x (cos, sin)(l32 f), or read rotated from the view; kept for every row block
  u32x4 kf[NU];
  if (klen > 0) {
    __builtin_amdgcn_s_waitcnt(wait_vm(NIB));   // K has landed (V in flight)
    const unsigned char* Kt = ktile + w * BLKB;
    if (rot) {
      float fk[2][E];
#pragma unroll
      for (int u = 0; u < NU / 2; ++u) {
        // this step's K chunks and the 16 angle factors it needs, read before any is used: left
        // to itself the compiler waited after nearly every LDS read here (~40 serialized round
        // trips per wave over the four steps)
        const u32x4 k0 = ld16(Kt + l32 * ROWB + (((2 * u + h) ^ kswz(l32)) << 4));
        const u32x4 k1 = ld16(Kt + l32 * ROWB + (((2 * (u + NU / 2) + h) ^ kswz(l32)) << 4));
        float2 cb[E], an[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = 2 * E * u + E * h + e;
          cb[e] = cbase[w][i];
          an[e] = ang[i * 32 + l32];
        }
        __builtin_amdgcn_sched_barrier(0);
        BF16Ops::unpack(k0, fk[0]);
        BF16Ops::unpack(k1, fk[1]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float2 ck = cmul(cb[e], an[e]);
          const float a = fk[0][e], c = fk[1][e];
          fk[0][e] = a * ck.x - c * ck.y;
          fk[1][e] = c * ck.x + a * ck.y;
        }
        kf[u] = QK::pack(fk[0]);
        kf[u + NU / 2] = QK::pack(fk[1]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) kf[u] = ld16(Kt + l32 * ROWB + (((2 * u + h) ^ kswz(l32)) << 4));
    }
  }

  const int sl = w < NS ? w : 0;   // this wave's d-slice of O^T (waves w < NS)
  const int key0 = 4 * h + ((lane & 15) >> 2);
  const int vrd = [&] {   // V^T operand read offset of d-slice sl (ds_read_tr16 layout)
    const int cb2 = (32 * sl + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    return key0 * ROWB + ((((cb2 >> 4) ^ vswz(key0)) << 4) | (cb2 & 15));
  }();
  const size_t pw = verify_dma_partial_words(D);
  for (int rc = rb_lo; rc < rb_hi; rc += QR) {
  const int nr = min(QR, rb_hi - rc);
  if (rc > rb_lo) {   // the next row blocks' queries, once every wave is done with qbuf
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    wg_barrier();
    load_q(rc, nr);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    wg_barrier();
    rotate_q(rc, nr);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    wg_barrier();
  }
  for (int rb = rc; rb < rc + nr; ++rb) {
    const int d = rb / p.nrb_d, rbl = rb - d * p.nrb_d;
    const int bq = (32 * rbl + l32) % p.B;                        // this lane's query block token
    const int tb = tail_unit ? tailb : p.W + d * p.tail_stride + p.n_tails[d];   // draft d's block rows
    u32x4 qf[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) qf[u] = ld16(qbuf + (rb - rc) * BLKB + l32 * ROWB + (((2 * u + h) ^ kswz(l32)) << 4));
    f32x16 sv = f32x16{};
    float mx = -INFINITY;
    if (klen > 0) {
#pragma unroll
      for (int u = 0; u < NU; ++u) sv = QK::mma(kf[u], qf[u], sv);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 8 * (i >> 2) + 4 * h + (i & 3);
        const bool ok = (kk < klen) & ((x0 + kk - tb) <= bq);   // block rows: causal
        sv[i] = ok ? sv[i] : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
    }
    mx = xhalf_max(mx);
    if (lane < 32) red_m[w][l32] = mx;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    wg_barrier();   // every row max; every wave has read qbuf and (first row block) the angle table
    float M = red_m[0][l32];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, red_m[ww][l32]);
    const float mu = M == -INFINITY ? 0.f : M;
    float lsum = 0.f;
    if (klen > 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = __builtin_amdgcn_exp2f(sv[i] - mu);
        lsum += sv[i];
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float pv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) pv[e] = sv[E * cc + e];
        st16(pbuf + ((w * 2 + cc) * 64 + lane) * 16, PV::pack(pv));
      }
    }
    lsum = xhalf_sum(lsum);
    if (lane < 32) red_l[w][l32] = lsum;
    if (rb == rb_lo) __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's V has landed
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    wg_barrier();   // P, row sums and every V tile visible

    // ---- O^T slice sl over the unit's blocks (waves w < NS)
    f32x16 o = f32x16{};
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      if (w >= NS || ((bmask >> jb) & 1) == 0) continue;
      const unsigned char* Vt = vtile + jb * BLKB;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const u32x2 lo = ds_read_tr16(Vt + vrd + 16 * cc * ROWB);
        const u32x2 hi = ds_read_tr16(Vt + vrd + (16 * cc + 8) * ROWB);
        const u32x4 pb = ld16(pbuf + ((jb * 2 + cc) * 64 + lane) * 16);
        o = PV::mma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, o);
      }
    }
    // the draft's block rows into the cache (their K / V came from k_blk / v_blk), once
    if (tail_unit && rb == rb_lo && klen > 0 && x0 + klen > tailb) {
      const unsigned char* Kt = ktile + w * BLKB;
      const unsigned char* Vt = vtile + w * BLKB;
      for (int e = lane; e < 32 * KCH; e += 64) {
        const int r = e / KCH, c = e % KCH, x = x0 + r;
        if (r < klen && x >= tailb) {
          const int64_t o2 = (static_cast<int64_t>(kvh) * p.S_cap + x) * D + 8 * c;
          st16(kc + o2, ld16(Kt + r * ROWB + ((c ^ kswz(r)) << 4)));
          st16(vc + o2, ld16(Vt + r * ROWB + ((c ^ vswz(r)) << 4)));
        }
      }
    }
    if (w < NS) {   // the partial (verify_dma_partial_words): O^T slice sl of row l32 in fp16, scaled
      // by a power of two that brings the slice's largest magnitude (this lane's 16 values and
      // its partner's in the other half) into [2^14, 2^15); then (m, l) pairs and 1/scale in fp32
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) L += red_l[ww][l32];
      float* dst = part + ((static_cast<int64_t>(kvh) * p.n_rb + rb) * p.n_split + slot) * pw;
      float mxo = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) mxo = fmaxf(mxo, fabsf(o[i]));
      const int sc = partial_row_scale(xhalf_max(mxo));
      const float mul = exp2_int(sc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        const f16x4 hv = f16x4{static_cast<_Float16>(o[4 * j] * mul), static_cast<_Float16>(o[4 * j + 1] * mul),
                               static_cast<_Float16>(o[4 * j + 2] * mul), static_cast<_Float16>(o[4 * j + 3] * mul)};
        *reinterpret_cast<u32x2*>(reinterpret_cast<_Float16*>(dst) + ((sl * 4 + j) * 64 + lane) * 4) =
            __builtin_bit_cast(u32x2, hv);
      }
      if (lane < 32) {
        dst[16 * D + 64 + 32 * sl + l32] = exp2_int(-sc);
        if (sl == 0) *reinterpret_cast<f32x2*>(dst + 16 * D + 2 * l32) = f32x2{M, L};
      }
    }
  }
  }   // row-block chunks
}

// Verify merge: fixed-order log-sum-exp combination of the n_split partials of each kv head.
// One workgroup per (kv head, row), kv head = blockIdx % Hkv as in the split kernel, so each
// reads partials from its own XCD's L2; thread (split group sg, 4 consecutive d).  Each thread
// folds splits sg, sg + SG, ... (all its loads in flight together), then the split groups
// are folded in LDS in index order.
__global__ __launch_bounds__(256) void verify_merge_kernel(const KParams p, const float* __restrict__ part,
                                                           void* __restrict__ out) {
  constexpr int MAXF = 8;   // splits folded per thread per pass
  const int kvh = blockIdx.x % p.Hkv, r = blockIdx.x / p.Hkv;   // kv head k on the XCD that wrote it
  const int rr = r % 32;                                        // row within row block r / 32
  const int dft = (r / 32) / p.nrb_d, rl = r - 32 * p.nrb_d * dft;   // draft, row within the draft
  const int hh = rl / p.B, b = rl % p.B;
  if (hh >= p.G) return;
  const int cpr = p.D / 4;                    // 4-float chunks per row
  const int sg = threadIdx.x / cpr, c = threadIdx.x % cpr;
  const int SG = 256 / cpr;                   // split groups
  const size_t pw = verify_partial_words(p.D);
  const float* base = part + (static_cast<size_t>(kvh) * p.n_rb + r / 32) * p.n_split * pw;
  float M = -INFINITY, L = 0.f;
  f32x4 acc = f32x4{};
  for (int s0 = sg; s0 < p.n_split; s0 += SG * MAXF) {
    float mm[MAXF], ll[MAXF];
    f32x4 ov[MAXF];
#pragma unroll
    for (int j = 0; j < MAXF; ++j) {
      const int s = s0 + j * SG;
      mm[j] = -INFINITY;
      ll[j] = 0.f;
      ov[j] = f32x4{};
      if (s < p.n_split) {
        const float* ps = base + s * pw;
        mm[j] = ps[32 * p.D + rr];
        ll[j] = ps[32 * p.D + 32 + rr];
        ov[j] = *reinterpret_cast<const f32x4*>(ps + rr * p.D + 4 * c);
      }
    }
#pragma unroll
    for (int j = 0; j < MAXF; ++j) {
      if (mm[j] == -INFINITY) continue;
      if (mm[j] > M) {
        const float f = __builtin_amdgcn_exp2f(M - mm[j]);
        acc *= f;
        L *= f;
        M = mm[j];
      }
      const float wgt = __builtin_amdgcn_exp2f(mm[j] - M);
      acc += wgt * ov[j];
      L += wgt * ll[j];
    }
  }
  __shared__ float sM[256], sL[256];
  __shared__ f32x4 sA[256];
  sM[threadIdx.x] = M;
  sL[threadIdx.x] = L;
  sA[threadIdx.x] = acc;
  __syncthreads();
  if (sg != 0) return;
  float Mt = -INFINITY;
  for (int g = 0; g < SG; ++g) Mt = fmaxf(Mt, sM[g * cpr + c]);
  float Lt = 0.f;
  f32x4 At = f32x4{};
  for (int g = 0; g < SG; ++g) {
    const float mg = sM[g * cpr + c];
    if (mg == -INFINITY) continue;
    const float f = __builtin_amdgcn_exp2f(mg - Mt);
    Lt += f * sL[g * cpr + c];
    At += f * sA[g * cpr + c];
  }
  const f32x4 res = At * (1.f / Lt);
  const int64_t oidx = (static_cast<int64_t>(dft * p.B + b) * p.Hq + kvh * p.G + hh) * p.D + 4 * c;
  if (p.out_bf16) {
    bf16 b4[4] = {static_cast<bf16>(res[0]), static_cast<bf16>(res[1]), static_cast<bf16>(res[2]), static_cast<bf16>(res[3])};
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(out) + oidx) = *reinterpret_cast<const u32x2*>(b4);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oidx) = res;
  }
}

// Verify merge for the bf16 split kernel: fixed-order log-sum-exp combination, per (kv head, query
// row), of the partials of the row's draft: the window units' and that draft's tail units', NH
// key groups each.  O is stored in fp16 in the accumulator order of the split kernel: element
// (row q, d = 32s + 8j + 4h + e) at half ((s*4 + j)*64 + q + 32h)*4 + e, times the scale of
// (row q, slice s) whose inverse follows the rows' (m, l) pairs.  One workgroup per (kv head,
// 32-row block, 4-column chunk c = (s, j, h)), kv head = blockIdx % Hkv as in the split kernel (the
// partials' XCD); thread (slot group sg, row q).  The 32 rows of a chunk are 256 contiguous bytes
// of a slot, and a row's (m, l) pair and slice scale are contiguous over the rows too, so every
// load of a wave reads whole lines (with one workgroup per row, each lane's 8 bytes sat in a
// line of its own and every line was fetched by 16 workgroups).
template <int D>
__global__ __launch_bounds__(256) void verify_merge_dma_kernel(const KParams p, const float* __restrict__ part,
                                                               void* __restrict__ out) {
  constexpr int MAXF = 4;                     // slots folded per thread per pass
  constexpr int CPR = D / 4;                  // 4-column chunks per row
  constexpr int SG = 256 / 32;                // slot groups
  kernarg_early(p.Hkv, p.B, p.n_tails[0], part);   // lines 0x00, 0x40, 0x80, the pointers
  const int kvh = blockIdx.x % p.Hkv, r = blockIdx.x / p.Hkv;
  const int c = r % CPR, rb = r / CPR;
  const int dft = rb / p.nrb_d;               // draft
  const int sg = threadIdx.x / 32, q = threadIdx.x % 32;
  const int rl = 32 * (rb - p.nrb_d * dft) + q;   // row within the draft
  const int hh = rl / p.B, b = rl % p.B;
  const int s = c / 8, j = (c % 8) / 2, hf = c % 2;
  const int ooff = ((s * 4 + j) * 64 + q + 32 * hf) * 4;   // (halves) 4 consecutive d of row q
  // slots of this draft: the window units', then its own tail units'
  const int ntb = ceil_div(p.n_tails[dft] + p.B, kVerifyBlock);
  const int n_used = p.n_ws + ceil_div(ntb, kVerifyUnitBlocks);
  const size_t pw = verify_dma_partial_words(D);
  const float* base = part + (static_cast<size_t>(kvh) * p.n_rb + rb) * p.n_split * pw;
  float M = -INFINITY, L = 0.f;
  f32x4 acc = f32x4{};
  for (int s0 = sg; s0 < n_used; s0 += SG * MAXF) {
    // every load of the batch issued back to back: a slot past n_used re-reads the last one
    // and is dropped below (max -inf, weight 0), so no branch splits the loads
    float mm[MAXF], ll[MAXF], os[MAXF];
    u32x2 ov[MAXF];
#pragma unroll
    for (int jj = 0; jj < MAXF; ++jj) {
      const float* ps = base + min(s0 + jj * SG, n_used - 1) * pw;
      const f32x2 ml = *reinterpret_cast<const f32x2*>(ps + 16 * D + 2 * q);
      mm[jj] = ml[0];
      ll[jj] = ml[1];
      os[jj] = ps[16 * D + 64 + 32 * s + q];
      ov[jj] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const _Float16*>(ps) + ooff);
    }
    float Mn = M;
#pragma unroll
    for (int jj = 0; jj < MAXF; ++jj) {
      if (s0 + jj * SG >= n_used) mm[jj] = -INFINITY;
      Mn = fmaxf(Mn, mm[jj]);
    }
    const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    acc *= r;
    L *= r;
#pragma unroll
    for (int jj = 0; jj < MAXF; ++jj) {
      const float wgt = mm[jj] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm[jj] - Mn);
      typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
      const f16x4 hv = __builtin_bit_cast(f16x4, ov[jj]);
      acc += (wgt * os[jj]) * f32x4{static_cast<float>(hv[0]), static_cast<float>(hv[1]), static_cast<float>(hv[2]),
                                    static_cast<float>(hv[3])};
      L += wgt * ll[jj];
    }
    M = Mn;
  }
  __shared__ float sM[256], sL[256];
  __shared__ f32x4 sA[256];
  sM[threadIdx.x] = M;
  sL[threadIdx.x] = L;
  sA[threadIdx.x] = acc;
  __syncthreads();
  if (sg != 0 || hh >= p.G) return;
  // every group's (M, L, acc) read first, then folded in group order (read one group at a time
  // under the branch, the LDS round trips ran back to back)
  float mgs[SG], lgs[SG];
  f32x4 ags[SG];
#pragma unroll
  for (int g = 0; g < SG; ++g) {
    mgs[g] = sM[g * 32 + q];
    lgs[g] = sL[g * 32 + q];
    ags[g] = sA[g * 32 + q];
  }
  __builtin_amdgcn_sched_barrier(0);
  float Mt = -INFINITY;
#pragma unroll
  for (int g = 0; g < SG; ++g) Mt = fmaxf(Mt, mgs[g]);
  float Lt = 0.f;
  f32x4 At = f32x4{};
#pragma unroll
  for (int g = 0; g < SG; ++g) {
    if (mgs[g] == -INFINITY) continue;
    const float f = __builtin_amdgcn_exp2f(mgs[g] - Mt);
    Lt += f * lgs[g];
    At += f * ags[g];
  }
  const f32x4 res = At * (1.f / Lt);
  const int64_t oidx = (static_cast<int64_t>(dft * p.B + b) * p.Hq + kvh * p.G + hh) * p.D + 4 * c;
  if (p.out_bf16) {
    bf16 b4[4] = {static_cast<bf16>(res[0]), static_cast<bf16>(res[1]), static_cast<bf16>(res[2]), static_cast<bf16>(res[3])};
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(out) + oidx) = *reinterpret_cast<const u32x2*>(b4);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oidx) = res;
  }
}

template <typename T, int D>
int launch_stream_t(const KParams& p, const void* q, const void* kc, const void* vc, void* out, void* ws,
                    hipStream_t st, const void* kn, const void* vn, void* kview) {
  using QKT = typename Path<T>::QKT;
  QKT* krot = static_cast<QKT*>(kview ? kview : ws);   // the rotated keys: the caller's view, or the workspace
  // bf16 path: rotated, scaled queries, the tile table and the partial slots of split views
  // after the keys
  const bool b16 = std::is_same<T, bf16>::value;
  QKT* qrot = reinterpret_cast<QKT*>(static_cast<unsigned char*>(ws) + align256(size_t(p.Hkv) * p.W * D * sizeof(QKT)));
  int2* tiles = b16 ? reinterpret_cast<int2*>(reinterpret_cast<unsigned char*>(qrot) + stream_qrot_bytes(p.V * p.T, p.Hq, D))
                    : nullptr;
  int4* mdesc = b16 && p.V > 1 ? reinterpret_cast<int4*>(reinterpret_cast<unsigned char*>(tiles) +
                                                          stream_tiles_bytes(0, p.P, p.T, p.V, p.F))
                               : nullptr;
  const int n_rb = p.Hkv * p.n_hsub * p.nqb;
  unsigned* flags = mdesc ? reinterpret_cast<unsigned*>(reinterpret_cast<unsigned char*>(mdesc) +
                                                        stream_merge_desc_bytes(p.nqb, p.V))
                          : nullptr;
  float* part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(qrot) + stream_qrot_bytes(p.V * p.T, p.Hq, D) +
                                         stream_tiles_bytes(0, p.P, p.T, p.V, p.F) + stream_merge_desc_bytes(p.nqb, p.V) +
                                         stream_flags_bytes(n_rb, p.V));
  const int nkb = rope_key_workgroups<T, D>(p);
  const int nqk = b16 ? ceil_div(p.V * p.T, kRopeQTok) * (p.G / rope_q_heads(p.G)) : 0;
  const NewFrame<T> nf{static_cast<const T*>(kn), static_cast<const T*>(vn),
                       kn ? const_cast<T*>(static_cast<const T*>(kc)) : nullptr,
                       kn ? const_cast<T*>(static_cast<const T*>(vc)) : nullptr};
  if (mdesc && stream_view_cut_twice(p)) return FD_ERR_GEOM;   // the split never cuts a view twice
  unsigned char* report = b16 ? static_cast<unsigned char*>(ws) + stream_report_offset(p) : nullptr;
  const int nbk = rope_bookkeeping_workgroups(tiles != nullptr, mdesc != nullptr);
  if (kn)
    hipLaunchKernelGGL((rope_window_kernel<T, D, true>), dim3(nbk + nkb + nqk * p.Hkv), dim3(256), 0, st, p,
                       static_cast<const T*>(kc), krot, nkb, static_cast<const T*>(q), qrot, tiles, mdesc, flags, nf,
                       report);
  else
    hipLaunchKernelGGL((rope_window_kernel<T, D, false>), dim3(nbk + nkb + nqk * p.Hkv), dim3(256), 0, st, p,
                       static_cast<const T*>(kc), krot, nkb, static_cast<const T*>(q), qrot, tiles, mdesc, flags, nf,
                       report);
  if (hipGetLastError() != hipSuccess) return FD_ERR_HIP;
  const int grid = p.Hkv * p.n_hsub * p.nqb * p.V;   // p.nseg == p.V for a streaming call
  if constexpr (std::is_same<T, bf16>::value) {
    hipLaunchKernelGGL((stream_pp_kernel<D>), dim3(grid), dim3(512), 0, st, p, static_cast<const QKT*>(qrot),
                       static_cast<const QKT*>(krot), static_cast<const T*>(vc), out, part, tiles, mdesc, flags);
    if (hipGetLastError() != hipSuccess) return FD_ERR_HIP;
    if (p.V > 1 && p.merge_mode == 0)   // a workgroup per (chunk boundary, row block)
      hipLaunchKernelGGL((stream_merge_kernel<D>), dim3((p.V - 1) * (grid / p.V)), dim3(256), 0, st, p, mdesc,
                         part, out);
  } else {
    hipLaunchKernelGGL((stream_attn_kernel<T, D>), dim3(grid), dim3(512), 0, st, p, static_cast<const T*>(q),
                       static_cast<const QKT*>(krot), static_cast<const T*>(vc), out);
  }
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

// Full-window (cold-start) prefill, bf16: one rotation pass for the window's keys and every
// window row's queries, then the attention kernel over the V*F frame segments, one workgroup
// per (row block, segment), longest segments first (V*F times more workgroups than a
// streaming call, so the dispatcher balances them without splitting any), and over the
// prefix segment.
template <int D>
int launch_prefill_t(const KParams& p, const void* q, const void* kc, const void* vc, void* out, void* ws,
                     hipStream_t st) {
  using QKT = _Float16;
  QKT* krot = static_cast<QKT*>(ws);
  QKT* qrot = reinterpret_cast<QKT*>(static_cast<unsigned char*>(ws) + align256(size_t(p.Hkv) * p.W * D * sizeof(QKT)));
  int2* tiles = reinterpret_cast<int2*>(reinterpret_cast<unsigned char*>(qrot) + stream_qrot_bytes(p.W, p.Hq, D));
  const int nkb = rope_key_workgroups<bf16, D>(p), nqk = ceil_div(p.W, kRopeQTok) * (p.G / rope_q_heads(p.G));
  hipLaunchKernelGGL((rope_window_kernel<bf16, D, false>), dim3(rope_bookkeeping_workgroups(true, false) + nkb + nqk * p.Hkv),
                     dim3(256), 0, st, p,
                     static_cast<const bf16*>(kc), krot, nkb, static_cast<const bf16*>(q), qrot, tiles, nullptr, nullptr,
                     NewFrame<bf16>{nullptr, nullptr, nullptr, nullptr},
                     static_cast<unsigned char*>(ws) + prefill_report_offset(p));
  if (hipGetLastError() != hipSuccess) return FD_ERR_HIP;
  KParams pf = p;   // the frame segments
  pf.seg0 = 0;
  pf.nseg = p.V * p.F;
  pf.qtok = p.T;
  pf.nqb = ceil_div(p.T, 32 * p.TBW);
  pf.whole = 1;
  const int grid = pf.Hkv * pf.n_hsub * pf.nqb * pf.nseg;
  if (p.P > 0) {
    KParams pp = p;   // the prefix segment, in the same launch after the frames
    pp.seg0 = p.V * p.F;
    pp.nseg = 1;
    pp.qtok = p.P;
    pp.nqb = ceil_div(p.P, 32 * p.TBW);
    pp.whole = 1;
    hipLaunchKernelGGL((stream_pp2_kernel<D>), dim3(grid + pp.Hkv * pp.n_hsub * pp.nqb), dim3(512), 0, st, pf, pp, grid,
                       static_cast<const QKT*>(qrot), static_cast<const QKT*>(krot), static_cast<const bf16*>(vc), out,
                       tiles);
  } else {
    hipLaunchKernelGGL((stream_pp_kernel<D>), dim3(grid), dim3(512), 0, st, pf, static_cast<const QKT*>(qrot),
                       static_cast<const QKT*>(krot), static_cast<const bf16*>(vc), out, nullptr, tiles, nullptr, nullptr);
  }
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

template <typename T, int D>
int launch_verify_t(const KParams& p, const void* qb, const void* kb, const void* vb, void* kc, void* vc,
                    void* out, void* ws, hipStream_t st, const void* kview) {
  float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kVerifyWsHeader);
  if constexpr (std::is_same<T, bf16>::value) {
    const dim3 grid(p.Hkv * (p.n_ws + p.n_drafts * p.n_ts)), block(64 * kVerifyWavesDma);
    if (kview)
      hipLaunchKernelGGL((verify_dma_kernel<D, true>), grid, block, 0, st, p, static_cast<const T*>(qb),
                         static_cast<const T*>(kb), static_cast<const T*>(vb), static_cast<T*>(kc), static_cast<T*>(vc),
                         static_cast<const _Float16*>(kview), part);
    else
      hipLaunchKernelGGL((verify_dma_kernel<D, false>), grid, block, 0, st, p, static_cast<const T*>(qb),
                         static_cast<const T*>(kb), static_cast<const T*>(vb), static_cast<T*>(kc), static_cast<T*>(vc),
                         static_cast<const _Float16*>(nullptr), part);
    if (hipGetLastError() != hipSuccess) return FD_ERR_HIP;
    hipLaunchKernelGGL((verify_merge_dma_kernel<D>), dim3(p.Hkv * p.n_rb * (D / 4)), dim3(256), 0, st, p,
                       static_cast<const float*>(part), out);
  } else {
    hipLaunchKernelGGL((verify_split_kernel<T, D>), dim3(p.Hkv * p.n_rb * p.n_split), dim3(256), 0, st, p,
                       static_cast<const T*>(qb), static_cast<const T*>(kb), static_cast<const T*>(vb),
                       static_cast<T*>(kc), static_cast<T*>(vc), part);
    if (hipGetLastError() != hipSuccess) return FD_ERR_HIP;
    hipLaunchKernelGGL(verify_merge_kernel, dim3(p.Hkv * p.n_rb * 32), dim3(256), 0, st, p,
                       static_cast<const float*>(part), out);
  }
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

// The rotation pass alone (keys only, no queries, no tile table, no insert).
template <typename T, int D>
int launch_rotate_window_t(const KParams& p, const void* kc, void* kview, hipStream_t st) {
  const int nkb = rope_key_workgroups<T, D>(p);
  hipLaunchKernelGGL((rope_window_kernel<T, D, false>), dim3(nkb), dim3(256), 0, st, p, static_cast<const T*>(kc),
                     static_cast<typename Path<T>::QKT*>(kview), nkb, static_cast<const T*>(nullptr),
                     static_cast<typename Path<T>::QKT*>(nullptr), static_cast<int2*>(nullptr), nullptr, nullptr,
                     NewFrame<T>{nullptr, nullptr, nullptr, nullptr}, nullptr);
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

// Scratch of fd_verify_attn_noalloc: the split-KV partials of verify calls made by callers that
// cannot allocate.  In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress (verify_scratch below), once per device.
static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];

}  // namespace

int rope_max_workgroups(const KParams& p, bool prefill) {
  KParams q = p;
  q.rot_new = 0;   // the whole window: the largest key grid
  const int nkb = p.D == 128 ? rope_key_workgroups<bf16, 128>(q) : rope_key_workgroups<bf16, 64>(q);
  const int rows = prefill ? p.W : p.V * p.T;
  return rope_bookkeeping_workgroups(true, !prefill && p.V > 1) + nkb +
         ceil_div(rows, kRopeQTok) * (p.G / rope_q_heads(p.G)) * p.Hkv;
}

size_t stream_report_offset(const KParams& p) {
  const int n_rb = p.Hkv * p.n_hsub * p.nqb;
  return align256(size_t(p.Hkv) * p.W * p.D * 2) + stream_qrot_bytes(p.V * p.T, p.Hq, p.D) +
         stream_tiles_bytes(0, p.P, p.T, p.V, p.F) + stream_merge_desc_bytes(p.nqb, p.V) + stream_flags_bytes(n_rb, p.V) +
         stream_partial_bytes(n_rb, p.V, p.D);
}

size_t prefill_report_offset(const KParams& p) {
  return align256(size_t(p.Hkv) * p.W * p.D * 2) + stream_qrot_bytes(p.W, p.Hq, p.D) +
         stream_tiles_bytes(1, p.P, p.T, p.V, p.F);
}

void* verify_scratch(int* status) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = FD_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {   // first call on this device, with it current
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *status = FD_ERR_HIP;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

int launch_insert(const KParams& p, int esize, void* kc, void* vc, const void* kn, const void* vn, int slot,
                  void* stream) {
  const int chunks = p.D * esize / 16;
  const int64_t total = static_cast<int64_t>(p.V) * p.T * p.Hkv * chunks;
  const unsigned grid = static_cast<unsigned>((total + 255) / 256);
  hipLaunchKernelGGL(insert_kernel, dim3(grid, 2), dim3(256), 0, static_cast<hipStream_t>(stream), p, chunks,
                     static_cast<const u32x4*>(kn), static_cast<const u32x4*>(vn), static_cast<u32x4*>(kc),
                     static_cast<u32x4*>(vc), slot);
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

int launch_kv_project(const KParams& p, int hidden, int slot, const void* x, const void* w, void* kc, void* vc,
                      void* stream) {
  const int M = p.V * p.T, N = 2 * p.Hkv * p.D;
  const unsigned grid = static_cast<unsigned>(((M + kPM - 1) / kPM) * (N / kPN));
  hipLaunchKernelGGL(kv_project_kernel, dim3(grid), dim3(64 * kPW), 0, static_cast<hipStream_t>(stream), p, hidden,
                     slot, static_cast<const bf16*>(x), static_cast<const bf16*>(w), static_cast<bf16*>(kc),
                     static_cast<bf16*>(vc));
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

int launch_stream(const KParams& p, int in_bf16, const void* q, const void* kc, const void* vc, void* out,
                  void* ws, void* stream, const void* kn, const void* vn, void* kview) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_bf16) {
    return p.D == 128 ? launch_stream_t<bf16, 128>(p, q, kc, vc, out, ws, st, kn, vn, kview)
                      : launch_stream_t<bf16, 64>(p, q, kc, vc, out, ws, st, kn, vn, kview);
  }
  return p.D == 128 ? launch_stream_t<float, 128>(p, q, kc, vc, out, ws, st, kn, vn, kview)
                    : launch_stream_t<float, 64>(p, q, kc, vc, out, ws, st, kn, vn, kview);
}

int launch_prefill(const KParams& p, const void* q, const void* kc, const void* vc, void* out, void* ws,
                   void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  return p.D == 128 ? launch_prefill_t<128>(p, q, kc, vc, out, ws, st) : launch_prefill_t<64>(p, q, kc, vc, out, ws, st);
}

int launch_verify(const KParams& p, int in_bf16, const void* qb, const void* kb, const void* vb, void* kc,
                  void* vc, void* out, void* ws, void* stream, const void* kview) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_bf16) {
    return p.D == 128 ? launch_verify_t<bf16, 128>(p, qb, kb, vb, kc, vc, out, ws, st, kview)
                      : launch_verify_t<bf16, 64>(p, qb, kb, vb, kc, vc, out, ws, st, kview);
  }
  return p.D == 128 ? launch_verify_t<float, 128>(p, qb, kb, vb, kc, vc, out, ws, st, nullptr)
                    : launch_verify_t<float, 64>(p, qb, kb, vb, kc, vc, out, ws, st, nullptr);
}

int launch_rotate_window(const KParams& p, int in_bf16, const void* kc, void* kview, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_bf16)
    return p.D == 128 ? launch_rotate_window_t<bf16, 128>(p, kc, kview, st) : launch_rotate_window_t<bf16, 64>(p, kc, kview, st);
  return p.D == 128 ? launch_rotate_window_t<float, 128>(p, kc, kview, st) : launch_rotate_window_t<float, 64>(p, kc, kview, st);
}

}  // namespace fd
