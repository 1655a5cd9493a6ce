// gfx950 (MI355X) kernels of the streaming-prefill attention path.
//
//  insert_kernel       bit copy of the new frame's pre-RoPE K/V into ring slot t mod F
//                      (FlashDrive technical summary, Methodology 1, "Token Layout").
//  stream_attn_kernel  attention of the new frame's tokens over the view-major window:
//                      K tiles are staged HBM -> registers -> LDS with RoPE applied in
//                      registers at each key's current (shifted) position (Methodology 1,
//                      "Positional Encoding"); the streaming mask is generated from the
//                      view / slot / token indices, never loaded.
//  verify_split_kernel + verify_merge_kernel
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

#include "fd_internal.h"

namespace fd {
namespace {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr double kTwoPiHi = 6.283185307179586;       // double nearest 2*pi
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;

// (cos a, sin a) of an fp64 angle: reduction to [-pi, pi] in fp64, then fp32 sincos.
__device__ inline float2 cs_angle(double a) {
  const double k = rint(a * kInvTwoPi);
  const double r = fma(-k, kTwoPiHi, a) - k * kTwoPiLo;
  float s, c;
  sincosf(static_cast<float>(r), &s, &c);
  return make_float2(c, s);
}

// cos/sin of (base + offset) from cos/sin of base and of offset.
__device__ inline float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.y * b.x + a.x * b.y);
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
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

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
// Streaming-prefill attention.
// Workgroup = 4 waves = 128 query rows that share one kv head: HPW query heads x (32*TBW)
// tokens of one view's new frame; wave w owns query head (w % HPW) of the group and
// tokens [32*(w / HPW), +32).  blockIdx.x = ((view_rank*nqb + qb)*n_hsub + hsub)*Hkv + kvh,
// so consecutive workgroups (dealt round-robin to the 8 XCDs) take different kv heads and
// the largest views (the longest key ranges) are dispatched first.
// Keys are walked as 64-row tiles inside segments with contiguous positions: the prefix,
// then every slot of views 0..v.  Only the newest slot of view v needs a per-element mask.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void stream_attn_kernel(const KParams p, const T* __restrict__ q,
                                                          const T* __restrict__ kc,
                                                          const T* __restrict__ vc,
                                                          void* __restrict__ out) {
  using QK = typename Path<T>::QK;
  using PV = typename Path<T>::PV;
  using QKT = typename Path<T>::QKT;
  static_assert(QK::E == PV::E, "operand chunk widths must agree");
  constexpr int E = QK::E;
  constexpr int H2 = D / 2;
  constexpr int NU = D / (2 * E);        // 16-byte k-chunks per operand row
  constexpr int KS = D + E;              // padded LDS row stride of K / Q tiles (elements)
  constexpr int VS = kTileKeys + E;      // padded LDS row stride of the V^T tile
  constexpr int ND = D / 32;             // 32-row blocks of O^T
  constexpr int CPB = 32 / (2 * E);      // PV chunks per 32-key block
  constexpr int NC = kTileKeys / (2 * E);
  constexpr int KB = kTileKeys * KS * static_cast<int>(sizeof(QKT));
  constexpr int QB = 128 * KS * static_cast<int>(sizeof(QKT));
  constexpr int KVB = KB + D * VS * static_cast<int>(sizeof(T));
  constexpr int BUF = QB > KVB ? QB : KVB;

  __shared__ float2 cs_r[kTileKeys][H2];  // cos/sin(r * inv_freq_i), r < 64
  __shared__ float2 csb[4][H2];           // cos/sin(base position * inv_freq_i)
  __shared__ __attribute__((aligned(16))) unsigned char buf[BUF];
  QKT* const Kl = reinterpret_cast<QKT*>(buf);           // rotated K tile [64][KS]
  T* const Vl = reinterpret_cast<T*>(buf + KB);          // V^T tile [D][VS]
  QKT* const Ql = reinterpret_cast<QKT*>(buf);           // rotated Q rows [128][KS] (prologue)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  int bid = blockIdx.x;
  const int kvh = bid % p.Hkv;
  bid /= p.Hkv;
  const int hsub = bid % p.n_hsub;
  bid /= p.n_hsub;
  const int qb = bid % p.nqb;
  const int v = p.V - 1 - bid / p.nqb;
  const int tok0 = qb * 32 * p.TBW;                      // first token of the workgroup
  const int head = kvh * p.G + hsub * p.HPW + (w % p.HPW);
  const int my_tok = tok0 + 32 * (w / p.HPW) + l32;      // this lane's query token
  const int64_t qpos0 = p.pos_base + p.P + static_cast<int64_t>(v * p.F + p.F - 1) * p.T;
  const float sc = p.sm_scale_log2;

  // Per-offset rotation table and the query-block bases.
  for (int e = tid; e < kTileKeys * H2; e += 256)
    cs_r[e / H2][e % H2] = cs_angle(static_cast<double>(e / H2) * p.inv_freq[e % H2]);
  for (int e = tid; e < 4 * H2; e += 256) {
    const int ww = e / H2, i = e % H2;
    csb[ww][i] = cs_angle(static_cast<double>(qpos0 + tok0 + 32 * (ww / p.HPW)) * p.inv_freq[i]);
  }
  __syncthreads();

  // Stage the 128 query rows (rotated at their positions) in LDS.
  {
    constexpr int PQ = H2 / 2;
    const int row = tid >> 1, part = tid & 1;
    const int ww = row >> 5, r = row & 31;
    const int hd = kvh * p.G + hsub * p.HPW + (ww % p.HPW);
    const int tk = tok0 + 32 * (ww / p.HPW) + r;
    float x1[PQ], x2[PQ];
    if (tk < p.T) {
      const T* src = q + (static_cast<int64_t>(v * p.T + tk) * p.Hq + hd) * D;
      load_f<T, PQ>(src + part * PQ, x1);
      load_f<T, PQ>(src + H2 + part * PQ, x2);
    } else {
#pragma unroll
      for (int j = 0; j < PQ; ++j) x1[j] = x2[j] = 0.f;
    }
    rope_pairs<PQ>(x1, x2, csb[ww], cs_r[r], part * PQ);
    store_ops<QK, QKT, PQ>(Ql + row * KS + part * PQ, x1);
    store_ops<QK, QKT, PQ>(Ql + row * KS + H2 + part * PQ, x2);
  }
  __syncthreads();
  u32x4 qf[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) qf[u] = ld16(Ql + (32 * w + l32) * KS + 2 * E * u + E * h);
  __syncthreads();

  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // One 64-key tile: physical rows [row0, row0+len) of kv head kvh at positions pos0 + r.
  auto tile = [&](int row0, int len, int64_t pos0, bool diag, int ktok0) {
    if (w == 0) {
      for (int i = lane; i < H2; i += 64) csb[0][i] = cs_angle(static_cast<double>(pos0) * p.inv_freq[i]);
    }
    __syncthreads();
    {  // K: HBM -> registers, RoPE, -> LDS
      constexpr int PK = H2 / 4;
      const int r = tid >> 2, qq = tid & 3;
      float x1[PK], x2[PK];
      if (r < len) {
        const T* src = kc + (static_cast<int64_t>(kvh) * p.S_cap + row0 + r) * D;
        load_f<T, PK>(src + qq * PK, x1);
        load_f<T, PK>(src + H2 + qq * PK, x2);
      } else {
#pragma unroll
        for (int j = 0; j < PK; ++j) x1[j] = x2[j] = 0.f;
      }
      rope_pairs<PK>(x1, x2, csb[0], cs_r[r], qq * PK);
      store_ops<QK, QKT, PK>(Kl + r * KS + qq * PK, x1);
      store_ops<QK, QKT, PK>(Kl + r * KS + H2 + qq * PK, x2);
    }
    {  // V: HBM -> registers -> LDS transposed (V^T[d][key], keys permuted for bf16)
      constexpr int DV = D / 16;
      const int dg = tid & 15, kg = tid >> 4;
      T vals[4][DV];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 4 * kg + j;
        if (key < len) {
          const T* src = vc + (static_cast<int64_t>(kvh) * p.S_cap + row0 + key) * D + dg * DV;
          if constexpr (DV * sizeof(T) % 16 == 0) {
#pragma unroll
            for (int c = 0; c < DV * static_cast<int>(sizeof(T)) / 16; ++c)
              *reinterpret_cast<u32x4*>(&vals[j][c * 16 / sizeof(T)]) = ld16(src + c * 16 / sizeof(T));
          } else {
            *reinterpret_cast<u32x2*>(&vals[j][0]) = *reinterpret_cast<const u32x2*>(src);
          }
        } else {
#pragma unroll
          for (int d = 0; d < DV; ++d) vals[j][d] = static_cast<T>(0.f);
        }
      }
      int pbase;
      if constexpr (E == 8) {
        const int a = kg & 3;
        pbase = (kg >> 2) * 16 + (a & 1) * 8 + (a >> 1) * 4;
      } else {
        pbase = 4 * kg;
      }
#pragma unroll
      for (int d = 0; d < DV; ++d) {
        T* dst = Vl + (dg * DV + d) * VS + pbase;
        if constexpr (E == 8) {
          bf16 t4[4] = {vals[0][d], vals[1][d], vals[2][d], vals[3][d]};
          *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<const u32x2*>(t4);
        } else {
          f32x4 t4 = {vals[0][d], vals[1][d], vals[2][d], vals[3][d]};
          *reinterpret_cast<f32x4*>(dst) = t4;
        }
      }
    }
    __syncthreads();

    // S^T = K Q^T for the two 32-key blocks.
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int u = 0; u < NU; ++u) s[kb] = QK::mma(ld16(Kl + (32 * kb + l32) * KS + 2 * E * u + E * h), qf[u], s[kb]);
    }
    // Mask (generated), online softmax in base 2.
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool ok = kk < len && (!diag || ktok0 + kk <= my_tok);
        const float x = ok ? s[kb][i] * sc : -INFINITY;
        s[kb][i] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float mu = (m_new == -INFINITY) ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pr = __builtin_amdgcn_exp2f(s[kb][i] - mu);
        s[kb][i] = pr;
        lsum += pr;
      }
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int kb = c / CPB;
      float pv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) pv[e] = s[kb][E * (c % CPB) + e];
      const u32x4 bop = PV::pack(pv);
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] = PV::mma(ld16(Vl + (32 * d + l32) * VS + 2 * E * c + E * h), bop, o[d]);
    }
  };

  for (int st = 0; st < p.P; st += kTileKeys)
    tile(st, min(kTileKeys, p.P - st), p.pos_base + st, false, 0);
  const int tok_end = tok0 + 32 * p.TBW;  // keys of the newest slot beyond this are masked for all rows
  for (int u = 0; u <= v; ++u) {
    for (int s = 0; s < p.F; ++s) {
      const int seg = p.P + (u * p.F + s) * p.T;
      const int64_t segpos = slot_pos(p, u, s);
      const bool diag = (u == v) && (s == p.s_new);
      const int tmax = diag ? min(p.T, tok_end) : p.T;
      for (int st = 0; st < tmax; st += kTileKeys)
        tile(seg + st, min(kTileKeys, p.T - st), segpos + st, diag, st);
    }
  }

  // Epilogue: O / l, this lane's query row.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (my_tok < p.T) {
    const int64_t obase = (static_cast<int64_t>(v * p.T + my_tok) * p.Hq + head) * D;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = 32 * d + 8 * ig + 4 * h;
        const f32x4 r = {o[d][4 * ig] * inv, o[d][4 * ig + 1] * inv, o[d][4 * ig + 2] * inv, o[d][4 * ig + 3] * inv};
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

// ---------------------------------------------------------------------------------------
// Verify, split-KV part.  Rows: r = hh*B + b (query head kvh*G + hh, block token b), one
// 32-row MFMA block.  Keys are numbered by cache row x: window rows [0, W), reasoning rows
// [W, W+n_tail), block rows [W+n_tail, W+n_tail+B) (read from k_blk / v_blk and copied into
// the cache here).  They are cut into 32-key blocks inside segments of contiguous
// positions; wave w of split s takes block (s*4 + w).  The four waves merge in LDS and the
// workgroup writes one (m, l, O) partial per (kv head, split).
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
  constexpr int VS = 32 + E;
  constexpr int OS = D + 4;
  constexpr int VST_BYTES = 4 * D * VS * static_cast<int>(sizeof(T));
  constexpr int OB_BYTES = 2 * 32 * OS * 4;
  constexpr int UB = VST_BYTES > OB_BYTES ? VST_BYTES : OB_BYTES;

  __shared__ float2 cs_r[32][H2];
  __shared__ float2 csq[H2];
  __shared__ float2 csb[4][H2];
  __shared__ float red_m[4][32], red_l[4][32];
  __shared__ __attribute__((aligned(16))) unsigned char ubuf[UB];
  T* const vst = reinterpret_cast<T*>(ubuf) ;
  float* const obuf = reinterpret_cast<float*>(ubuf);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int kvh = blockIdx.x % p.Hkv, split = blockIdx.x / p.Hkv;
  const int hh = l32 / p.B, bq = l32 % p.B;
  const bool qvalid = hh < p.G;
  const int head = kvh * p.G + hh;
  const int tailbase = p.W + p.n_tail;  // cache row of block token 0
  const float sc = p.sm_scale_log2;

  for (int e = tid; e < 32 * H2; e += 256)
    cs_r[e / H2][e % H2] = cs_angle(static_cast<double>(e / H2) * p.inv_freq[e % H2]);
  if (tid < H2) csq[tid] = cs_angle(static_cast<double>(p.pos_base + tailbase) * p.inv_freq[tid]);
  __syncthreads();

  // Query fragments, rotated in registers: lane half h holds elements [2E*u + E*h, +E) of
  // chunk u; chunks u and u + NU/2 hold the two halves of the same RoPE pairs.
  u32x4 qf[NU];
  {
    float f[NU][E];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (qvalid) In::unpack(ld16(qb + (static_cast<int64_t>(bq) * p.Hq + head) * D + 2 * E * u + E * h), f[u]);
      else {
#pragma unroll
        for (int e = 0; e < E; ++e) f[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < NU / 2; ++u) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = 2 * E * u + E * h + e;
        const float2 cs = cmul(csq[i], cs_r[bq][i]);
        const float a = f[u][e], b = f[u + NU / 2][e];
        f[u][e] = a * cs.x - b * cs.y;
        f[u + NU / 2][e] = b * cs.x + a * cs.y;
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) qf[u] = QK::pack(f[u]);
  }

  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int nbp = (p.P + 31) / 32, nbs = (p.T + 31) / 32, nslot = p.V * p.F;

  for (int k = 0; k < kVerifyBlocksPerWave; ++k) {
    const int j = (split * kVerifyWaves + w) * kVerifyBlocksPerWave + k;
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
    if (lane < H2) csb[w][lane] = cs_angle(static_cast<double>(pos0) * p.inv_freq[lane]);
    __syncthreads();

    // K rows: lane l32 holds key x0 + l32; rotate in registers.
    u32x4 kf[NU];
    {
      const int x = x0 + l32;
      const bool kv = l32 < len;
      const bool from_blk = x >= tailbase;
      const T* src = from_blk ? kb + (static_cast<int64_t>(x - tailbase) * p.Hkv + kvh) * D
                              : kc + (static_cast<int64_t>(kvh) * p.S_cap + x) * D;
      float f[NU][E];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (kv) {
          const u32x4 raw = ld16(src + 2 * E * u + E * h);
          if (from_blk) st16(kc + (static_cast<int64_t>(kvh) * p.S_cap + x) * D + 2 * E * u + E * h, raw);
          In::unpack(raw, f[u]);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) f[u][e] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < NU / 2; ++u) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = 2 * E * u + E * h + e;
          const float2 cs = cmul(csb[w][i], cs_r[l32][i]);
          const float a = f[u][e], b = f[u + NU / 2][e];
          f[u][e] = a * cs.x - b * cs.y;
          f[u + NU / 2][e] = b * cs.x + a * cs.y;
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) kf[u] = QK::pack(f[u]);
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int u = 0; u < NU; ++u) s = QK::mma(kf[u], qf[u], s);

    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = 8 * (i >> 2) + 4 * h + (i & 3);
      const bool ok = kk < len && (x0 + kk - tailbase) <= bq;
      const float x = ok ? s[i] * sc : -INFINITY;
      s[i] = x;
      mloc = fmaxf(mloc, x);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float mu = (m_new == -INFINITY) ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pr = __builtin_amdgcn_exp2f(s[i] - mu);
      s[i] = pr;
      lsum += pr;
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] *= alpha;

    // V rows -> this wave's LDS V^T block (keys permuted for bf16), copying block rows.
    {
      constexpr int DV = D / 8;
      const int kg = lane >> 3, dg = lane & 7;
      T vals[4][DV];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = 4 * kg + jj;
        const int x = x0 + key;
        if (key < len) {
          const bool from_blk = x >= tailbase;
          const T* src = (from_blk ? vb + (static_cast<int64_t>(x - tailbase) * p.Hkv + kvh) * D
                                   : vc + (static_cast<int64_t>(kvh) * p.S_cap + x) * D) + dg * DV;
#pragma unroll
          for (int c = 0; c < DV * static_cast<int>(sizeof(T)) / 16; ++c) {
            const u32x4 raw = ld16(src + c * 16 / sizeof(T));
            *reinterpret_cast<u32x4*>(&vals[jj][c * 16 / sizeof(T)]) = raw;
            if (from_blk) st16(vc + (static_cast<int64_t>(kvh) * p.S_cap + x) * D + dg * DV + c * 16 / sizeof(T), raw);
          }
        } else {
#pragma unroll
          for (int d = 0; d < DV; ++d) vals[jj][d] = static_cast<T>(0.f);
        }
      }
      int pbase;
      if constexpr (E == 8) {
        const int a = kg & 3;
        pbase = (kg >> 2) * 16 + (a & 1) * 8 + (a >> 1) * 4;
      } else {
        pbase = 4 * kg;
      }
      T* vw = vst + w * D * VS;
#pragma unroll
      for (int d = 0; d < DV; ++d) {
        T* dst = vw + (dg * DV + d) * VS + pbase;
        if constexpr (E == 8) {
          bf16 t4[4] = {vals[0][d], vals[1][d], vals[2][d], vals[3][d]};
          *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<const u32x2*>(t4);
        } else {
          f32x4 t4 = {vals[0][d], vals[1][d], vals[2][d], vals[3][d]};
          *reinterpret_cast<f32x4*>(dst) = t4;
        }
      }
    }
    __syncthreads();
    {
      const T* vw = vst + w * D * VS;
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        float pv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) pv[e] = s[E * c + e];
        const u32x4 bop = PV::pack(pv);
#pragma unroll
        for (int d = 0; d < ND; ++d) o[d] = PV::mma(ld16(vw + (32 * d + l32) * VS + 2 * E * c + E * h), bop, o[d]);
      }
    }
    __syncthreads();
  }

  // Merge the four waves (rows are shared, key ranges differ).
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
  float* dstp = part + (static_cast<int64_t>(kvh) * p.n_split + split) * verify_partial_words(D);
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

// Verify merge: fixed-order log-sum-exp combination of the n_split partials of each kv head.
// Grid = Hkv * 4 workgroups; thread = (row in an 8-row group, 4 consecutive d).
__global__ __launch_bounds__(256) void verify_merge_kernel(const KParams p, const float* __restrict__ part,
                                                           void* __restrict__ out) {
  const int kvh = blockIdx.x >> 2, rg = blockIdx.x & 3;
  const int r = rg * 8 + (threadIdx.x >> 5);
  const int d0 = 4 * (threadIdx.x & 31);
  if (d0 >= p.D) return;
  const int hh = r / p.B, b = r % p.B;
  if (hh >= p.G) return;
  const size_t pw = verify_partial_words(p.D);
  const float* base = part + static_cast<size_t>(kvh) * p.n_split * pw;
  float M = -INFINITY, L = 0.f;
  f32x4 acc = f32x4{};
  for (int s = 0; s < p.n_split; ++s) {
    const float* ps = base + s * pw;
    const float m = ps[32 * p.D + r];
    if (m == -INFINITY) continue;
    const float l = ps[32 * p.D + 32 + r];
    const f32x4 ov = *reinterpret_cast<const f32x4*>(ps + r * p.D + d0);
    if (m > M) {
      const float c = __builtin_amdgcn_exp2f(M - m);
      acc *= c;
      L *= c;
      M = m;
    }
    const float wgt = __builtin_amdgcn_exp2f(m - M);
    acc += wgt * ov;
    L += wgt * l;
  }
  const f32x4 res = acc * (1.f / L);
  const int64_t oidx = (static_cast<int64_t>(b) * p.Hq + kvh * p.G + hh) * p.D + d0;
  if (p.out_bf16) {
    bf16 b4[4] = {static_cast<bf16>(res[0]), static_cast<bf16>(res[1]), static_cast<bf16>(res[2]), static_cast<bf16>(res[3])};
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(out) + oidx) = *reinterpret_cast<const u32x2*>(b4);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oidx) = res;
  }
}

template <typename T, int D>
int launch_stream_t(const KParams& p, const void* q, const void* kc, const void* vc, void* out,
                    hipStream_t st) {
  const int grid = p.Hkv * p.n_hsub * p.nqb * p.V;
  hipLaunchKernelGGL((stream_attn_kernel<T, D>), dim3(grid), dim3(256), 0, st, p,
                     static_cast<const T*>(q), static_cast<const T*>(kc), static_cast<const T*>(vc), out);
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

template <typename T, int D>
int launch_verify_t(const KParams& p, const void* qb, const void* kb, const void* vb, void* kc, void* vc,
                    void* out, void* ws, hipStream_t st) {
  float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kVerifyWsHeader);
  hipLaunchKernelGGL((verify_split_kernel<T, D>), dim3(p.Hkv * p.n_split), dim3(256), 0, st, p,
                     static_cast<const T*>(qb), static_cast<const T*>(kb), static_cast<const T*>(vb),
                     static_cast<T*>(kc), static_cast<T*>(vc), part);
  if (hipGetLastError() != hipSuccess) return FD_ERR_HIP;
  hipLaunchKernelGGL(verify_merge_kernel, dim3(p.Hkv * 4), dim3(256), 0, st, p,
                     static_cast<const float*>(part), out);
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_HIP;
}

}  // namespace

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

int launch_stream(const KParams& p, int in_bf16, const void* q, const void* kc, const void* vc, void* out,
                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_bf16) {
    return p.D == 128 ? launch_stream_t<bf16, 128>(p, q, kc, vc, out, st)
                      : launch_stream_t<bf16, 64>(p, q, kc, vc, out, st);
  }
  return p.D == 128 ? launch_stream_t<float, 128>(p, q, kc, vc, out, st)
                    : launch_stream_t<float, 64>(p, q, kc, vc, out, st);
}

int launch_verify(const KParams& p, int in_bf16, const void* qb, const void* kb, const void* vb, void* kc,
                  void* vc, void* out, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_bf16) {
    return p.D == 128 ? launch_verify_t<bf16, 128>(p, qb, kb, vb, kc, vc, out, ws, st)
                      : launch_verify_t<bf16, 64>(p, qb, kb, vb, kc, vc, out, ws, st);
  }
  return p.D == 128 ? launch_verify_t<float, 128>(p, qb, kb, vb, kc, vc, out, ws, st)
                    : launch_verify_t<float, 64>(p, qb, kb, vb, kc, vc, out, ws, st);
}

}  // namespace fd
