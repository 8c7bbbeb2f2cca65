// Chunkwise forward pass of key-only-gated linear attention (GLA) for gfx950.
//
// Recurrence (x-techcon article on GTR, section 架构 / Architecture; the
// printed formula is lost, the surrounding sentences fix it):
//   S_t = diag(alpha_t) S_{t-1} + k_t^T v_t ,  o_t = q_t S_t ,  alpha = exp(log_gate).
// Chunked evaluation (same article, section 算子 / Operator: 64-token chunks,
// per-chunk state contributions, a pass over chunk-boundary states, per-chunk
// outputs).  With E = log2(e) * (inclusive cumulative log-gate from the chunk
// start) and S_prev the state entering the chunk:
//   o_tau  = (q_tau * 2^E_tau) S_prev + sum_{sigma<=tau} (sum_i q_tau,i k_sigma,i 2^(E_tau,i - E_sigma,i)) v_sigma
//   S_next = diag(2^E_last) S_prev + (k * 2^(E_last - E))^T V
//
// Work split.  A "segment" is `seg_len` consecutive chunks of one sequence.
//   gla_seg_state : one workgroup per segment walks its chunks and sums their
//                   state contributions (the segment's own aggregate).
//   gla_seg_scan  : one thread per (sequence, state element) runs the
//                   boundary recurrence over segments -> state entering each.
//   gla_seg_out   : one workgroup per segment starts from that state, walks
//                   its chunks, writes outputs and carries the state in MFMA
//                   accumulator registers from chunk to chunk.
//
// Inside a chunk (256 threads = 4 waves, 16-token sub-blocks = MFMA tiles):
//   * the four input tiles are read once from HBM, rows addressed through the
//     scan-direction map (no permuted copy);
//   * the gate is prefix-summed in LDS;
//   * every exponential factor that reaches an MFMA operand is <= 1, except on
//     the four diagonal 16x16 score tiles, which are referenced at the
//     sub-block midpoint (factors <= 2^8); when a sub-block's gate range is too
//     wide for that, the tile is formed exactly in fp32 on the VALU instead;
//   * scores are transposed tiles P^T = K Q^T written to LDS only;
//   * wave w owns value columns [16w, 16w+16): it forms O^T = V^T P^T +
//     S^T (q 2^E)^T for those columns and carries S[:, 16w:16w+16].
//
// MFMA fragment convention (checked on gfx950): for v_mfma_f32_16x16x32_f16
// lane l holds A row l%16 and B column l%16 with k-slots 8*(l/16)+e, and the
// 16x16 fp32 result holds column l%16, rows 4*(l/16)+r.  Operands here use the
// logical k of slot (g = l/16, e) = (e < 4 ? 4g+e : 16+4g+e-4) inside each
// 32-wide k block, so a result tile pair feeds straight back in as an operand.
// The fp32 path issues eight v_mfma_f32_16x16x4_f32 over the same fragments.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_internal.h"
#include "gla_profile.h"

namespace gtr {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdE = 68;  // padded row length of the fp32 cumulative-gate tile

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// LDS-only barrier: waits for this wave's LDS traffic, not for its global loads,
// so prefetched global loads stay in flight across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- element I/O
struct IoF32 {
  using T = float;
  static constexpr int V = 4;  // elements per 16-byte access
  __device__ static void cvt(u4 r, float *x) {
    x[0] = __uint_as_float(r.x); x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z); x[3] = __uint_as_float(r.w);
  }
  __device__ static float load1(const T *p) { return *p; }
  __device__ static void store4(T *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }
};

struct IoF16 {
  using T = _Float16;
  static constexpr int V = 8;
  __device__ static void cvt(u4 r, float *x) {
    h8 h = __builtin_bit_cast(h8, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)h[e];
  }
  __device__ static float load1(const T *p) { return (float)*p; }
  __device__ static void store4(T *p, f4 v) {
    h4 h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
    *reinterpret_cast<h4 *>(p) = h;
  }
};

struct IoBF16 {
  using T = uint16_t;  // raw bfloat16 bits
  static constexpr int V = 8;
  __device__ static void cvt(u4 r, float *x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = __uint_as_float(r[w] << 16);
      x[2 * w + 1] = __uint_as_float(r[w] & 0xffff0000u);
    }
  }
  __device__ static float load1(const T *p) { return __uint_as_float((uint32_t)*p << 16); }
  __device__ static uint32_t rne(float f) {  // round to nearest even, quiet NaN kept
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
  __device__ static void store4(T *p, f4 v) {
    u2 w = {rne(v.x) | (rne(v.y) << 16), rne(v.z) | (rne(v.w) << 16)};
    *reinterpret_cast<u2 *>(p) = w;
  }
};

// ------------------------------------------------------------ MFMA operands
template <typename Op> struct Frag;
template <> struct Frag<_Float16> { h8 v; };
template <> struct Frag<float> { f8 v; };

__device__ __forceinline__ f4 mma(const Frag<_Float16> &a, const Frag<_Float16> &b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma(const Frag<float> &a, const Frag<float> &b, f4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

template <typename Op> struct OpTraits;
template <> struct OpTraits<_Float16> {
  static constexpr int LD = 72;          // padded LDS row (elements): 144 B
  static constexpr float kDiagRange = 16.f;  // widest log2 gate range of a 16-token
                                             // sub-block handled by midpoint scaling
};
template <> struct OpTraits<float> {
  static constexpr int LD = 68;          // 272 B
  static constexpr float kDiagRange = 100.f;
};

// Fragment rows from a row-major LDS tile: elements [k0, k0+4) and [k0+16, k0+20).
__device__ __forceinline__ Frag<_Float16> ld_frag(const _Float16 *row_k0) {
  h4 lo = *reinterpret_cast<const h4 *>(row_k0);
  h4 hi = *reinterpret_cast<const h4 *>(row_k0 + 16);
  Frag<_Float16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> ld_frag(const float *row_k0) {
  f4 lo = *reinterpret_cast<const f4 *>(row_k0);
  f4 hi = *reinterpret_cast<const f4 *>(row_k0 + 16);
  Frag<float> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
// Per-k factors (fp32 vector in LDS) for the same slots.
__device__ __forceinline__ f8 ld_factors(const float *vec_k0) {
  f4 lo = *reinterpret_cast<const f4 *>(vec_k0);
  f4 hi = *reinterpret_cast<const f4 *>(vec_k0 + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void scale(Frag<_Float16> &f, f8 s) {
  h8 hs = __builtin_convertvector(s, h8);
  f.v = f.v * hs;
}
__device__ __forceinline__ void scale(Frag<float> &f, f8 s) { f.v = f.v * s; }

__device__ __forceinline__ void to_op(const f4 &lo, const f4 &hi, Frag<_Float16> &f) {
  f8 x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  f.v = __builtin_convertvector(x, h8);
}
__device__ __forceinline__ void to_op(const f4 &lo, const f4 &hi, Frag<float> &f) {
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// score-tile slots: (query sub-block a, key sub-block b), b <= a, slot = a(a+1)/2 + b
__device__ __forceinline__ int tile_a(int s) { return s >= 6 ? 3 : (s >= 3 ? 2 : (s >= 1 ? 1 : 0)); }
__device__ __forceinline__ int tile_slot(int a, int b) { return (a * (a + 1)) / 2 + b; }

// per-dim vectors (64 floats each) of one chunk, in LDS
enum : int {
  kR0 = 0, kR1, kR2, kR3,   // E at the end of sub-block 0..3 (kR3 = E_last)
  kDec,                     // 2^E_last: decay of the state across the chunk
  kH0, kH1, kH2, kH3,       // 2^((E_end(a-1) - E_end(a))/2): diagonal-tile midpoint factor
  kP2R1, kP2R2, kP2R3,      // 2^E_end(a-1): query factor from sub-block start to chunk start
  kP2L0, kP2L1, kP2L2,      // 2^(E_last - E_end(b)): key factor from sub-block end to chunk end
  kC20, kC30, kC31,         // 2^(E_end(a-1) - E_end(b)), b < a-1: between-sub-block factor
  kNumVec
};

// ----------------------------------------------------------- scan direction
// Grid index of scan position t (see gtr_gla.h for the four orders).
__device__ __forceinline__ int grid_index(int t, int n_tok, int gh, int gw, int dir) {
  if (dir & 1) t = n_tok - 1 - t;
  if (dir & 2) {
    int col = t / gh;
    int row = t - col * gh;
    return row * gw + col;
  }
  (void)gw;
  return t;
}

struct Seq {
  int n_tok, gh, gw, dir;
  size_t base;  // element offset of this sequence: bh * n_tok * 64
  __device__ size_t row(int t) const {
    return base + (size_t)grid_index(t, n_tok, gh, gw, dir) * kHead;
  }
};

// -------------------------------------------------------------- shared memory
template <typename Op, bool kOut> struct Smem;

template <typename Op> struct Smem<Op, true> {
  static constexpr int LD = OpTraits<Op>::LD;
  Op qs[kChunk * LD];   // q * 2^(E - E_end(a-1))      row-major [token][dim]
  Op qh[kChunk * LD];   // q * 2^E                      row-major
  Op ks[kChunk * LD];   // k * 2^(E_end(b) - E)         row-major
  Op kbt[kChunk * LD];  // k * 2^(E_last - E)           transposed [dim][token]
  Op vt[kChunk * LD];   // v                            transposed [dim][token]
  float e[kChunk * kLdE];
  Op pt[10 * 256];      // score tiles P^T, 4 values per lane, lane-ordered
  float vec[kNumVec * kHead];
  float tot[4 * kHead];
};

template <typename Op> struct Smem<Op, false> {
  static constexpr int LD = OpTraits<Op>::LD;
  Op kbt[kChunk * LD];
  Op vt[kChunk * LD];
  float e[kChunk * kLdE];
  float vec[kNumVec * kHead];
  float tot[4 * kHead];
};

// ------------------------------------------------------------------- params
struct Params {
  const void *q, *k, *v, *g;
  void *out;
  int n_tok, gh, gw, dir;
  int n_chunk, seg_len, n_seg, n_seg_grid;
  float *agg, *agg_log2;
  const float *prev;
};

template <class Io> struct Layout {
  static constexpr int V = Io::V;
  static constexpr int TPR = kHead / V;         // threads per token row
  static constexpr int RPP = kThreads / TPR;    // rows per pass
  static constexpr int NP = kChunk / RPP;       // passes per chunk
};

template <class Io, bool kQ>
__device__ __forceinline__ void load_chunk(const Params &p, const Seq &sq, int c, int tid,
                                           u4 *rq, u4 *rk, u4 *rv, u4 *rg) {
  using L = Layout<Io>;
  using T = typename Io::T;
  const int col0 = (tid % L::TPR) * L::V;
#pragma unroll
  for (int pp = 0; pp < L::NP; ++pp) {
    const int tau = pp * L::RPP + tid / L::TPR;
    const int t = c * kChunk + tau;
    if (t < p.n_tok) {
      const size_t off = sq.row(t) + col0;
      if constexpr (kQ) rq[pp] = *reinterpret_cast<const u4 *>(static_cast<const T *>(p.q) + off);
      rk[pp] = *reinterpret_cast<const u4 *>(static_cast<const T *>(p.k) + off);
      rv[pp] = *reinterpret_cast<const u4 *>(static_cast<const T *>(p.v) + off);
      rg[pp] = *reinterpret_cast<const u4 *>(static_cast<const T *>(p.g) + off);
    } else {  // tail of the last chunk: no key, no value, no decay, no query
      const u4 z = {0u, 0u, 0u, 0u};
      if constexpr (kQ) rq[pp] = z;
      rk[pp] = z;
      rv[pp] = z;
      rg[pp] = z;
    }
  }
}

// Cumulative log2-gate of the chunk into sm.e and the per-dim vectors into sm.vec.
// Ends with the LDS barrier after which e and vec are readable by every wave.
template <class Io, typename Op, bool kOut>
__device__ __forceinline__ void gate_prefix(Smem<Op, kOut> &sm, const u4 *rg, int tid) {
  using L = Layout<Io>;
  const int col0 = (tid % L::TPR) * L::V;
#pragma unroll
  for (int pp = 0; pp < L::NP; ++pp) {
    const int tau = pp * L::RPP + tid / L::TPR;
    float x[L::V];
    Io::cvt(rg[pp], x);
#pragma unroll
    for (int e = 0; e < L::V; e += 4) {
      f4 w = {x[e] * kLog2e, x[e + 1] * kLog2e, x[e + 2] * kLog2e, x[e + 3] * kLog2e};
      *reinterpret_cast<f4 *>(&sm.e[tau * kLdE + col0 + e]) = w;
    }
  }
  lds_sync();
  // wave p scans tokens [16p, 16p+16) of dim i = lane
  const int lane = tid & 63, p = tid >> 6;
  float loc[16];
  float run = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    run += sm.e[(16 * p + u) * kLdE + lane];
    loc[u] = run;
  }
  sm.tot[p * kHead + lane] = run;
  lds_sync();
  const float R0 = sm.tot[lane];
  const float R1 = R0 + sm.tot[kHead + lane];
  const float R2 = R1 + sm.tot[2 * kHead + lane];
  const float R3 = R2 + sm.tot[3 * kHead + lane];
  const float off = p == 0 ? 0.f : (p == 1 ? R0 : (p == 2 ? R1 : R2));
#pragma unroll
  for (int u = 0; u < 16; ++u) sm.e[(16 * p + u) * kLdE + lane] = off + loc[u];
  float *vec = sm.vec;
  if (p == 0) {
    vec[kR0 * kHead + lane] = R0;
    vec[kR1 * kHead + lane] = R1;
    vec[kR2 * kHead + lane] = R2;
    vec[kR3 * kHead + lane] = R3;
    vec[kDec * kHead + lane] = fast_exp2(R3);
  } else if (p == 1) {
    vec[kP2L0 * kHead + lane] = fast_exp2(R3 - R0);
    vec[kP2L1 * kHead + lane] = fast_exp2(R3 - R1);
    vec[kP2L2 * kHead + lane] = fast_exp2(R3 - R2);
  } else if (kOut && p == 2) {
    vec[kH0 * kHead + lane] = fast_exp2(-0.5f * R0);
    vec[kH1 * kHead + lane] = fast_exp2(0.5f * (R0 - R1));
    vec[kH2 * kHead + lane] = fast_exp2(0.5f * (R1 - R2));
    vec[kH3 * kHead + lane] = fast_exp2(0.5f * (R2 - R3));
  } else if (kOut && p == 3) {
    vec[kP2R1 * kHead + lane] = fast_exp2(R0);
    vec[kP2R2 * kHead + lane] = fast_exp2(R1);
    vec[kP2R3 * kHead + lane] = fast_exp2(R2);
    vec[kC20 * kHead + lane] = fast_exp2(R1 - R0);
    vec[kC30 * kHead + lane] = fast_exp2(R2 - R0);
    vec[kC31 * kHead + lane] = fast_exp2(R2 - R1);
  }
  lds_sync();
}

// Scaled operand tiles.  kOut: qs, qh, ks (row-major) and kbt, vt (transposed);
// otherwise only kbt and vt.
template <class Io, typename Op, bool kOut>
__device__ __forceinline__ void prep(Smem<Op, kOut> &sm, const u4 *rq, const u4 *rk, const u4 *rv,
                                     int tid) {
  using L = Layout<Io>;
  constexpr int LD = OpTraits<Op>::LD;
  const int col0 = (tid % L::TPR) * L::V;
#pragma unroll
  for (int pp = 0; pp < L::NP; ++pp) {
    const int tau = pp * L::RPP + tid / L::TPR;
    const int a = tau >> 4;
    float kx[L::V], vx[L::V], qx[L::V];
    Io::cvt(rk[pp], kx);
    Io::cvt(rv[pp], vx);
    if constexpr (kOut) Io::cvt(rq[pp], qx);
    float E[L::V];
#pragma unroll
    for (int e = 0; e < L::V; e += 4) {
      f4 w = *reinterpret_cast<const f4 *>(&sm.e[tau * kLdE + col0 + e]);
      E[e] = w.x; E[e + 1] = w.y; E[e + 2] = w.z; E[e + 3] = w.w;
    }
    if constexpr (kOut) {
      const float *Rprev = a > 0 ? &sm.vec[(kR0 + a - 1) * kHead + col0] : nullptr;
      const float *Ra = &sm.vec[(kR0 + a) * kHead + col0];
      const float *P2R = a > 0 ? &sm.vec[(kP2R1 + a - 1) * kHead + col0] : nullptr;
      const float *P2L = a < 3 ? &sm.vec[(kP2L0 + a) * kHead + col0] : nullptr;
      Op qs[L::V], qh[L::V], ks[L::V];
#pragma unroll
      for (int e = 0; e < L::V; ++e) {
        const float rp = Rprev ? Rprev[e] : 0.f;
        const float qsv = qx[e] * fast_exp2(E[e] - rp);
        const float qhv = P2R ? qsv * P2R[e] : qsv;
        const float ksv = kx[e] * fast_exp2(Ra[e] - E[e]);
        const float kbv = P2L ? ksv * P2L[e] : ksv;
        qs[e] = (Op)qsv;
        qh[e] = (Op)qhv;
        ks[e] = (Op)ksv;
        sm.kbt[(col0 + e) * LD + tau] = (Op)kbv;
        sm.vt[(col0 + e) * LD + tau] = (Op)vx[e];
      }
#pragma unroll
      for (int e = 0; e < L::V; ++e) {
        sm.qs[tau * LD + col0 + e] = qs[e];
        sm.qh[tau * LD + col0 + e] = qh[e];
        sm.ks[tau * LD + col0 + e] = ks[e];
      }
    } else {
      const float *El = &sm.vec[kR3 * kHead + col0];
#pragma unroll
      for (int e = 0; e < L::V; ++e) {
        sm.kbt[(col0 + e) * LD + tau] = (Op)(kx[e] * fast_exp2(El[e] - E[e]));
        sm.vt[(col0 + e) * LD + tau] = (Op)vx[e];
      }
    }
  }
  lds_sync();
}

// Exact fp32 diagonal score tile (a, a), used when the sub-block's gate range is
// too wide for midpoint scaling.  Reads q and k rows again from global memory.
template <class Io, typename Op>
__device__ f4 exact_diag(const Params &p, const Seq &sq, const Smem<Op, true> &sm, int c, int a,
                         int lane) {
  using T = typename Io::T;
  const int g = lane >> 4, l16 = lane & 15;
  const int tau = 16 * a + l16;
  const int t_tau = c * kChunk + tau;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if (t_tau >= p.n_tok) return acc;
  const T *qrow = static_cast<const T *>(p.q) + sq.row(t_tau);
  const T *krow[4];
  bool ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sig = 16 * a + 4 * g + r;
    ok[r] = sig <= tau;  // sig <= tau < n_tok, so the row exists
    krow[r] = ok[r] ? static_cast<const T *>(p.k) + sq.row(c * kChunk + sig) : qrow;
  }
  for (int i = 0; i < kHead; ++i) {
    const float qi = Io::load1(qrow + i);
    const float et = sm.e[tau * kLdE + i];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (ok[r]) {
        const int sig = 16 * a + 4 * g + r;
        acc[r] += qi * Io::load1(krow[r] + i) * fast_exp2(et - sm.e[sig * kLdE + i]);
      }
    }
  }
  return acc;
}

// Score tiles P^T[sigma][tau] of this chunk into sm.pt (lower block triangle only).
template <class Io, typename Op>
__device__ __forceinline__ void scores(const Params &p, const Seq &sq, Smem<Op, true> &sm, int c,
                                       int tid) {
  constexpr int LD = OpTraits<Op>::LD;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  for (int s = wave; s < 10; s += 4) {
    const int a = tile_a(s);
    const int b = s - (a * (a + 1)) / 2;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    if (a == b) {
      const float rng = (a > 0 ? sm.vec[(kR0 + a - 1) * kHead + lane] : 0.f) -
                        sm.vec[(kR0 + a) * kHead + lane];
      const bool fast = __all(rng <= OpTraits<Op>::kDiagRange);
      if (fast) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int k0 = 32 * kb + 4 * g;
          Frag<Op> A = ld_frag(&sm.ks[(16 * b + l16) * LD + k0]);
          Frag<Op> B = ld_frag(&sm.qs[(16 * a + l16) * LD + k0]);
          const f8 h = ld_factors(&sm.vec[(kH0 + a) * kHead + k0]);
          scale(A, h);
          scale(B, h);
          acc = mma(A, B, acc);
        }
      } else {
        acc = exact_diag<Io, Op>(p, sq, sm, c, a, lane);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r > l16) acc[r] = 0.f;  // keys after the query
    } else {
      const int cvec = (a == 2) ? kC20 : (b == 0 ? kC30 : kC31);  // used when b < a-1
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int k0 = 32 * kb + 4 * g;
        Frag<Op> A = ld_frag(&sm.ks[(16 * b + l16) * LD + k0]);
        Frag<Op> B = ld_frag(&sm.qs[(16 * a + l16) * LD + k0]);
        if (b < a - 1) scale(B, ld_factors(&sm.vec[cvec * kHead + k0]));
        acc = mma(A, B, acc);
      }
    }
    Op *dst = &sm.pt[s * 256 + lane * 4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r] = (Op)acc[r];
  }
  lds_sync();
}

// ------------------------------------------------------------------ kernels
// kOut = false: segment aggregate (gla_seg_state).  kOut = true: outputs (gla_seg_out).
template <class Io, typename Op, bool kOut>
__device__ __forceinline__ void segment_body(const Params &p) {
  using L = Layout<Io>;
  using T = typename Io::T;
  constexpr int LD = OpTraits<Op>::LD;
  __shared__ Smem<Op, kOut> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int bh = blockIdx.x / p.n_seg_grid;
  const int seg = blockIdx.x - bh * p.n_seg_grid;
  Seq sq{p.n_tok, p.gh, p.gw, p.dir, (size_t)bh * p.n_tok * kHead};

  // state columns [16*wave, 16*wave+16): S[it][r] = S[16it+4g+r][16*wave+l16]
  f4 S[4];
  const size_t st_off = ((size_t)bh * p.n_seg + seg) * kStateElems + wave * 1024 + lane;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[it][r] = (kOut && p.prev) ? p.prev[st_off + (it * 4 + r) * 64] : 0.f;
  }
  float log2_decay = 0.f;  // wave 0, lane = key dim: sum of E_last over the segment

  const int c_begin = seg * p.seg_len;
  const int c_end = min(c_begin + p.seg_len, p.n_chunk);
  u4 rq[L::NP], rk[L::NP], rv[L::NP], rg[L::NP];
  load_chunk<Io, kOut>(p, sq, c_begin, tid, rq, rk, rv, rg);

  for (int c = c_begin; c < c_end; ++c) {
    u4 nq[L::NP], nk[L::NP], nv[L::NP], ng[L::NP];
    const bool more = c + 1 < c_end;
    if (more) load_chunk<Io, kOut>(p, sq, c + 1, tid, nq, nk, nv, ng);

    gate_prefix<Io, Op, kOut>(sm, rg, tid);
    if (!kOut && wave == 0) log2_decay += sm.vec[kR3 * kHead + lane];
    prep<Io, Op, kOut>(sm, rq, rk, rv, tid);

    Frag<Op> vf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) vf[kb] = ld_frag(&sm.vt[(16 * wave + l16) * LD + 32 * kb + 4 * g]);

    if constexpr (kOut) {
      scores<Io, Op>(p, sq, sm, c, tid);
      Frag<Op> sf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) to_op(S[2 * kb], S[2 * kb + 1], sf[kb]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb <= (tt >> 1); ++kb) {
          f4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
          const Op *plo = &sm.pt[tile_slot(tt, 2 * kb) * 256 + lane * 4];
#pragma unroll
          for (int r = 0; r < 4; ++r) lo[r] = (float)plo[r];
          if (2 * kb + 1 <= tt) {
            const Op *phi = &sm.pt[tile_slot(tt, 2 * kb + 1) * 256 + lane * 4];
#pragma unroll
            for (int r = 0; r < 4; ++r) hi[r] = (float)phi[r];
          }
          Frag<Op> pf;
          to_op(lo, hi, pf);
          acc = mma(vf[kb], pf, acc);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          acc = mma(sf[kb], ld_frag(&sm.qh[(16 * tt + l16) * LD + 32 * kb + 4 * g]), acc);
        const int t = c * kChunk + 16 * tt + l16;
        if (t < p.n_tok) Io::store4(static_cast<T *>(p.out) + sq.row(t) + 16 * wave + 4 * g, acc);
      }
    }

    // carry the state over the chunk: S <- diag(2^E_last) S + (k 2^(E_last-E))^T V
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const f4 dec = *reinterpret_cast<const f4 *>(&sm.vec[kDec * kHead + 16 * it + 4 * g]);
      S[it] = S[it] * dec;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        S[it] = mma(ld_frag(&sm.kbt[(16 * it + l16) * LD + 32 * kb + 4 * g]), vf[kb], S[it]);
    }

    if (more) {
#pragma unroll
      for (int pp = 0; pp < L::NP; ++pp) {
        if constexpr (kOut) rq[pp] = nq[pp];
        rk[pp] = nk[pp];
        rv[pp] = nv[pp];
        rg[pp] = ng[pp];
      }
    }
  }

  if constexpr (!kOut) {
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) p.agg[st_off + (it * 4 + r) * 64] = S[it][r];
    if (wave == 0) p.agg_log2[((size_t)bh * p.n_seg + seg) * kHead + lane] = log2_decay;
  }
}

template <class Io, typename Op>
__global__ __launch_bounds__(kThreads) void gla_seg_state(Params p) {
  segment_body<Io, Op, false>(p);
}

template <class Io, typename Op>
__global__ __launch_bounds__(kThreads) void gla_seg_out(Params p) {
  segment_body<Io, Op, true>(p);
}

// Boundary-state recurrence over segments, one thread per (sequence, state
// element): prev[seg] = state entering segment seg; prev[0] = s0 (or 0).
__global__ __launch_bounds__(kThreads) void gla_seg_scan(const float *agg, const float *agg_log2,
                                                         float *prev, const float *s0,
                                                         float *s_final, int bh_count, int n_seg) {
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  const int bh = (int)(gid / kStateElems);
  const int e = (int)(gid - (long)bh * kStateElems);
  if (bh >= bh_count) return;
  // register order -> (i, j): e = w*1024 + x*64 + l, i = 16(x/4) + 4(l/16) + x%4, j = 16w + l%16
  const int w = e >> 10, x = (e >> 6) & 15, l = e & 63;
  const int i = 16 * (x >> 2) + 4 * (l >> 4) + (x & 3);
  const int j = 16 * w + (l & 15);
  const size_t sbase = (size_t)bh * n_seg;
  float s = s0 ? s0[(size_t)bh * kStateElems + i * kHead + j] : 0.f;
  const int steps = s_final ? n_seg : n_seg - 1;
  prev[sbase * kStateElems + e] = s;
  for (int seg = 0; seg < steps; ++seg) {
    s = fast_exp2(agg_log2[(sbase + seg) * kHead + i]) * s + agg[(sbase + seg) * kStateElems + e];
    if (seg + 1 < n_seg) prev[(sbase + seg + 1) * kStateElems + e] = s;
  }
  if (s_final) s_final[(size_t)bh * kStateElems + i * kHead + j] = s;
}

template <class Io, typename Op>
int launch_typed(const LaunchArgs &a) {
  Params p{a.q, a.k, a.v, a.g, a.out, a.n_tok, a.grid_h, a.grid_w, a.direction,
           a.n_chunk, a.seg_len, a.n_seg, a.n_seg, a.agg, a.agg_log2, nullptr};
  const bool need_scan = a.n_seg > 1 || a.s0 != nullptr || a.s_final != nullptr;
  if (need_scan) {
    const int n_state_seg = a.s_final ? a.n_seg : a.n_seg - 1;
    if (n_state_seg > 0) {
      Params ps = p;
      ps.n_seg_grid = n_state_seg;
      profile_mark(kKernelSegState, a.stream, true);
      hipLaunchKernelGGL((gla_seg_state<Io, Op>), dim3((unsigned)(a.bh * n_state_seg)),
                         dim3(kThreads), 0, a.stream, ps);
      profile_mark(kKernelSegState, a.stream, false);
    }
    const long threads = (long)a.bh * kStateElems;
    profile_mark(kKernelSegScan, a.stream, true);
    hipLaunchKernelGGL(gla_seg_scan, dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, a.stream, a.agg, a.agg_log2, a.prev, a.s0, a.s_final,
                       a.bh, a.n_seg);
    profile_mark(kKernelSegScan, a.stream, false);
    p.prev = a.prev;
  }
  profile_mark(kKernelSegOut, a.stream, true);
  hipLaunchKernelGGL((gla_seg_out<Io, Op>), dim3((unsigned)(a.bh * a.n_seg)), dim3(kThreads), 0,
                     a.stream, p);
  profile_mark(kKernelSegOut, a.stream, false);
  return (int)hipGetLastError();
}

}  // namespace

int launch_gla(const LaunchArgs &a) {
  switch (a.dtype) {
    case 0: return launch_typed<IoF32, float>(a);
    case 1: return launch_typed<IoF16, _Float16>(a);
    case 2: return launch_typed<IoBF16, _Float16>(a);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace gtr
