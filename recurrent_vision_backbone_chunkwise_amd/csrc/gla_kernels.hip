// Chunkwise forward pass of key-only-gated linear attention (GLA) for gfx950.
//
// Recurrence (x-techcon article on GTR, section 架构 / Architecture; the
// printed formula is lost, the surrounding sentences fix it):
//   S_t = diag(alpha_t) S_{t-1} + k_t^T v_t ,  o_t = q_t S_t ,  alpha = exp(log_gate).
// Chunked evaluation (same article, section 算子 / Operator: 64-token chunks,
// per-chunk state contributions, a pass over chunk-boundary states, per-chunk
// outputs).  With E = log2(e) * (inclusive cumulative log-gate from the chunk
// start) and S_prev the state entering the chunk:
//   o_tau  = (q_tau 2^E_tau) S_prev + sum_{sigma<=tau} (sum_i q_tau,i k_sigma,i 2^(E_tau,i - E_sigma,i)) v_sigma
//   S_next = diag(2^E_last) S_prev + (k 2^(E_last - E))^T V
//
// Work split.  A "segment" is `seg_len` consecutive chunks of one sequence; one
// workgroup owns a segment and walks its chunks with the state held in MFMA
// accumulator registers.  The state entering a segment comes either from
//   * gla_seg_state + gla_seg_scan (separate launches: segment aggregates, then
//     one thread per state element runs the boundary recurrence over segments),
//     followed by gla_seg_out; or
//   * gla_fused (one launch): each workgroup first forms its segment's
//     aggregate and publishes it, then combines the aggregates of the segments
//     before it in scan order (waiting on per-segment flags), then writes its
//     outputs.  Workgroups take segments in the order they start (an atomic
//     ticket), so every segment a workgroup waits for belongs to a workgroup
//     that is already running.
//
// Inside a chunk (256 threads = 4 waves; wave w owns tokens [16w, 16w+16), a
// 16-token sub-block; lane l owns dims [4(l%16), +4) of tokens 16w+4(l/16)+r):
//   * inputs are read once from HBM, rows addressed through the scan-direction
//     map (no permuted copy);
//   * the gate prefix runs in registers plus one cross-lane scan per wave;
//   * every exponential factor that reaches an MFMA operand is <= 1, except on
//     the four diagonal 16x16 score tiles, which are referenced at the
//     sub-block midpoint (factors <= 2^8); when a sub-block's gate range is too
//     wide for that, the tile is formed exactly in fp32 on the VALU;
//   * scores are transposed tiles P^T = K Q^T held in LDS only;
//   * wave w owns value columns [16w, 16w+16): it forms O^T = V^T P^T +
//     S^T (q 2^E)^T for those columns and carries S[:, 16w:16w+16].
//
// Head dims.  The tiles are 64 wide.  Narrower heads load zeros past d_k or
// d_v and drop those stores; with d_v = 128 each 64-column value block is a
// sequence of its own (the recurrence is independent per value column); with
// d_k = 128 every chunk runs as two passes, one per 64-wide key block, each
// carrying its block's state and adding its part to the same outputs.
//
// MFMA fragment convention (checked on gfx950): for v_mfma_f32_16x16x32_f16
// lane l holds A row l%16 and B column l%16 with k-slots 8*(l/16)+e, and the
// 16x16 fp32 result holds column l%16, rows 4*(l/16)+r.  Operands here use the
// logical k of slot (g = l/16, e) = (e < 4 ? 4g+e : 16+4g+e-4) inside each
// 32-wide k block, so a result tile pair feeds straight back in as an operand.
// Transposed 16-bit operands are read with ds_read_b64_tr_b16: inside each
// 16-lane group, lane 4a+b receives element b of the 8-byte rows that lanes
// a, a+4, a+8, a+12 address.  The fp32 path issues eight
// v_mfma_f32_16x16x4_f32 over the same fragments.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>

#include <map>
#include <mutex>
#include <type_traits>

#include "gla_index.h"
#include "gla_internal.h"
#include "gla_profile.h"

namespace gtr {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSpinLimit = 1 << 22;  // ~seconds of polling before a wait gives up

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s4 lds_s4;
typedef __attribute__((address_space(3))) _Float16 lds_h;

// LDS-only barrier: waits for this wave's LDS traffic, not for its global loads,
// so prefetched global loads stay in flight across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ f4 exp2v(f4 x) {
  return f4{fast_exp2(x.x), fast_exp2(x.y), fast_exp2(x.z), fast_exp2(x.w)};
}

// ---------------------------------------------------------------- element I/O
// Each thread moves 4 consecutive elements of a token row per access.
// kLagGates: position t of the scan takes the gate of position t-1 (none at
// t = 0); Lagged<> sets it.  Plain: the element format without that flag.
struct IoF32 {
  static constexpr bool kLagGates = false;
  using Plain = IoF32;
  using T = float;
  using Raw = u4;  // 16 bytes
  __device__ static f4 to_f4(Raw r) { return __builtin_bit_cast(f4, r); }
  __device__ static float from_bits(uint32_t b) { return __uint_as_float(b); }
  __device__ static T narrow(float v) { return v; }
  __device__ static Raw pack(f4 v) { return __builtin_bit_cast(u4, v); }
};

struct IoF16 {
  static constexpr bool kLagGates = false;
  using Plain = IoF16;
  using T = _Float16;
  using Raw = u2;  // 8 bytes
  __device__ static h4 to_h4(Raw r) { return __builtin_bit_cast(h4, r); }
  __device__ static f4 to_f4(Raw r) { return __builtin_convertvector(to_h4(r), f4); }
  __device__ static float from_bits(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }
  __device__ static T narrow(float v) { return (_Float16)v; }
  __device__ static Raw pack(f4 v) { return __builtin_bit_cast(u2, __builtin_convertvector(v, h4)); }
};

struct IoBF16 {
  static constexpr bool kLagGates = false;
  using Plain = IoBF16;
  using T = uint16_t;  // raw bfloat16 bits
  using Raw = u2;
  __device__ static f4 to_f4(Raw r) {
    return f4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
              __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
  }
  __device__ static h4 to_h4(Raw r) { return __builtin_convertvector(to_f4(r), h4); }
  __device__ static float from_bits(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static T narrow(float v) { return (T)rne(v); }
  __device__ static uint32_t rne(float f) {  // round to nearest even, quiet NaN kept
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
  __device__ static Raw pack(f4 v) { return u2{rne(v.x) | (rne(v.y) << 16), rne(v.z) | (rne(v.w) << 16)}; }
};

// An element format whose gates are read one scan position late (the
// backward pass's reversed scan, where the state gradient at t decays by the
// gate of the position after t in the forward order).
template <class B> struct Lagged : B {
  static constexpr bool kLagGates = true;
  using Plain = B;
};

// ------------------------------------------------------------ MFMA operands
template <typename Op> struct OpT;
// LD: row stride (elements) of tiles read as row fragments (16 consecutive rows
// at 136 B spread one 8-byte read per lane over all 32 banks); LDT: of tiles
// read transposed (4 rows x 4 column groups at 160 B per row hit distinct banks).
// kDiagMin: smallest gate product over a 16-token sub-block (per key dim) that
// midpoint scaling handles (2^-16 keeps every scaled fp16 operand within 2^+-8).
template <> struct OpT<_Float16> {
  using V4 = h4;
  using V8 = h8;
  using Bits = uint16_t;          // one output element in the I/O format
  static constexpr int LDO = 72;  // row stride of the output tile (16 rows hit distinct banks)
  static constexpr int LD = 68;
  static constexpr int LDT = 80;
  static constexpr float kDiagMin = 1.52587890625e-05f;  // 2^-16
};
template <> struct OpT<float> {
  using V4 = f4;
  using V8 = f8;
  using Bits = uint32_t;
  static constexpr int LDO = 68;
  static constexpr int LD = 68;
  static constexpr int LDT = 68;
  static constexpr float kDiagMin = 7.888609052210118e-31f;  // 2^-100
};

template <typename Op> using op4 = typename OpT<Op>::V4;
template <typename Op> using op8 = typename OpT<Op>::V8;

__device__ __forceinline__ f4 mma(const h8 &a, const h8 &b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma(const f8 &a, const f8 &b, f4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ h8 cat(const h4 &lo, const h4 &hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f8 cat(const f4 &lo, const f4 &hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row fragment: elements [k0, k0+4) and [k0+16, k0+20) of one LDS row.
template <typename Op> __device__ __forceinline__ op8<Op> frag_row(const Op *row_k0) {
  return cat(*reinterpret_cast<const op4<Op> *>(row_k0),
             *reinterpret_cast<const op4<Op> *>(row_k0 + 16));
}

// Transposed fragment of a row-major [token][dim] LDS tile: lane l gets
// tile[r0 + 4(l/16) + e][c0 + l%16] for e = 0..3 and tile[r0 + 16 + 4(l/16) + e][...].
__device__ __forceinline__ h4 tr4(const _Float16 *tile, int row, int col) {
  lds_h *base = (lds_h *)(tile);
  lds_s4 *ptr = (lds_s4 *)(base + row * OpT<_Float16>::LDT + col);
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(ptr));
}
__device__ __forceinline__ h8 frag_tr(const _Float16 *tile, int r0, int c0, int lane) {
  const int src = lane & 15, g = lane >> 4;
  const int row = r0 + 4 * g + (src >> 2), col = c0 + 4 * (src & 3);
  return cat(tr4(tile, row, col), tr4(tile, row + 16, col));
}
__device__ __forceinline__ f8 frag_tr(const float *tile, int r0, int c0, int lane) {
  constexpr int LD = OpT<float>::LDT;
  const int g = lane >> 4, col = c0 + (lane & 15);
  f8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = tile[(r0 + 4 * g + e) * LD + col];
    f[4 + e] = tile[(r0 + 16 + 4 * g + e) * LD + col];
  }
  return f;
}

template <typename Op, class Io> struct ToOp : ToOp<Op, typename Io::Plain> {};
template <> struct ToOp<_Float16, IoF16> {
  __device__ static h4 cvt(u2 r) { return IoF16::to_h4(r); }
};
template <> struct ToOp<_Float16, IoBF16> {
  __device__ static h4 cvt(u2 r) { return IoBF16::to_h4(r); }
};
template <> struct ToOp<float, IoF32> {
  __device__ static f4 cvt(u4 r) { return IoF32::to_f4(r); }
};
template <> struct ToOp<float, IoF16> {  // fp32 operands for 16-bit I/O (backward pass)
  __device__ static f4 cvt(u2 r) { return IoF16::to_f4(r); }
};
template <> struct ToOp<float, IoBF16> {
  __device__ static f4 cvt(u2 r) { return IoBF16::to_f4(r); }
};

__device__ __forceinline__ void cvt4(f4 x, h4 &y) { y = __builtin_convertvector(x, h4); }
__device__ __forceinline__ void cvt4(f4 x, f4 &y) { y = x; }
template <typename Op> __device__ __forceinline__ op4<Op> to4(f4 x) {
  op4<Op> y;
  cvt4(x, y);
  return y;
}

// score-tile slots: (query sub-block a, key sub-block b), b <= a, slot = a(a+1)/2 + b
__device__ __forceinline__ int tile_a(int s) { return s >= 6 ? 3 : (s >= 3 ? 2 : (s >= 1 ? 1 : 0)); }
__device__ __forceinline__ int tile_slot(int a, int b) { return (a * (a + 1)) / 2 + b; }

constexpr uint32_t kOob = 0x80000000u;  // beyond every buffer range: loads give 0, stores drop

// One sequence's tensors as buffer resources: byte offsets are 32-bit and
// uniform bases live in scalar registers.  A sequence is one (batch, head) and
// one 64-wide block of value columns: q, k and log_gate rows hold d_k elements,
// v and out rows d_v, and the v/out resources start at the block's first
// column.  Every range is at most 2^31 bytes (checked on the host), so kOob
// plus a column offset is past all of them.
struct Seq {
  __amdgpu_buffer_rsrc_t q, k, v, g, o;
  int n_tok, gh, gw, dir;
  float rcp_gh;
  uint32_t kpitch, vpitch;  // bytes per grid cell of q/k/log_gate and of v/out
  int dk, dv;               // key dims, value columns of this block (<= 64)
};

// Byte offset of (cell, col), or kOob for a missing row or a masked column.
__device__ __forceinline__ uint32_t cell_at(uint32_t cell, uint32_t pitch, uint32_t col) {
  return (cell == kNoRow || col == kOob) ? kOob : cell * pitch + col;
}
// Byte offset in a q/k/log_gate row of 4 key dims starting at d (kOob past d_k).
template <class Io> __device__ __forceinline__ uint32_t key_col(const Seq &sq, int d) {
  return d < sq.dk ? (uint32_t)d * (uint32_t)sizeof(typename Io::T) : kOob;
}
// Byte offset in a v/out row of this block's 4 value columns starting at j.
template <class Io> __device__ __forceinline__ uint32_t val_col(const Seq &sq, int j) {
  return j < sq.dv ? (uint32_t)j * (uint32_t)sizeof(typename Io::T) : kOob;
}

// Grid cell whose log_gate row holds the gate of scan position t (t < n_tok):
// t's own, or with lagged gates the one before it (kNoRow at t = 0: no decay).
template <class Io> __device__ __forceinline__ uint32_t gate_cell(const Seq &sq, int t) {
  if constexpr (!Io::kLagGates) return token_cell(sq, t);
  return t > 0 ? token_cell(sq, t - 1) : kNoRow;
}

// -------------------------------------------------------------- shared memory
// Gate factors below are products of alpha = exp(log_gate) over token ranges of
// the chunk; with E the log2 cumulative gate from the chunk start they equal
// the exponentials named in the comments.
// Every member is 16-byte aligned so that fragment reads compile to single
// 8- and 16-byte LDS accesses.
// NQ = 0: a walk that only carries the state (no outputs) and needs kb, vv,
// tot and dec alone.  NQ = -1: the backward chunk kernel, which reads the
// query/key factor tiles (qs, ks, hv, cv, rowoff) but neither the state
// operand kb nor the score and query tiles (pt, qh, dcum).  Arrays a layout
// does not use shrink to one element, so its workgroups take less LDS (more
// of them fit on a CU).
template <typename Op, int NQ> struct Smem {
  static constexpr int LD = OpT<Op>::LD;
  static constexpr int LDT = OpT<Op>::LDT;
  static constexpr bool kOutTiles = NQ != 0;    // qs, ks, hv, cv, rowoff
  static constexpr bool kStateTiles = NQ >= 0;  // kb
  static constexpr bool kQueryTiles = NQ > 0;   // pt, dcum, qh
  static constexpr int kSlots = NQ > 0 ? NQ : 1;
  alignas(16) Op qs[kOutTiles ? kChunk * LD : 1];   // q 2^(E - E_end(a-1))     [token][dim]
  alignas(16) Op ks[kOutTiles ? kChunk * LD : 1];   // k 2^(E_end(b) - E)  (gla_fused reuses qs after its walk)
  alignas(16) Op kb[kStateTiles ? kChunk * LDT : 1];  // k 2^(E_last - E)
  alignas(16) Op vv[kChunk * LDT];                  // v
  alignas(16) Op pt[kQueryTiles ? 10 * 256 : 1];    // score tiles P^T, 4 values per lane, lane-ordered
  alignas(16) float tot[4 * kHead];                 // gate product of each 16-token sub-block
  alignas(16) Op hv[kOutTiles ? 4 * kHead : 1];     // 2^((E_end(a-1) - E_end(a))/2): diagonal-tile midpoint factor
  alignas(16) Op cv[kOutTiles ? 3 * kHead : 1];     // 2^(E_end(a-1) - E_end(b)) for (a,b) = (2,0), (3,0), (3,1)
  alignas(16) float dec[kHead];                     // 2^E_last: decay of the state across the chunk
  // One slot per chunk whose outputs wait for the state entering the segment
  // (NQ = 1 when outputs are stored as each chunk completes).
  alignas(16) uint32_t rowoff[kSlots][kOutTiles ? kChunk : 1];  // grid cell of each token (kNoRow past the end)
  alignas(16) float dcum[kSlots][kQueryTiles ? kHead : 1];      // decay from the segment start to the chunk start
  alignas(16) Op qh[kSlots][kQueryTiles ? kChunk * LD : 1];     // q 2^E
};

// ------------------------------------------------------------------- params
struct Params {
  const void *q, *k, *v, *g;
  void *out;
  int bh_count, n_tok, gh, gw, dir;  // bh_count: sequences (batch x head x value block)
  float rcp_gh;
  int dk, dv, nvb;  // key dims, value dims, 64-wide value blocks per head
  int n_chunk, seg_len, n_seg, n_seg_grid;
  float *agg, *agg_dec;    // [seq][n_seg][key block][4096] state contribution, [..][64] decay per key dim
  const float *prev;       // [seq][n_seg][key block][4096] register order (separate-launch path)
  int prev_seq, prev_step;  // prev entries per sequence, and between consecutive segments
  const float *s0;         // user initial state, row-major [B*H][d_k][d_v], nullable
  float *s_final;          // user final state, row-major, nullable
  int *sync;               // fused path: header and per-XCD work words (kSync* words)
  long long *flags;        // [bh][n_seg] fused path: segment payload published (epoch + 1)
  int fold_block;          // fused path: segments per fold block
  int batch, n_batch;      // fused path: sequences per batch an XCD takes, and batches
  int n_pre;               // fused path: batches 0 .. n_pre-1 start out assigned to XCDs 0 .. n_pre-1
  // a slice of the key dims (backward pass, d_k > 64): q/k/log_gate rows hold
  // kpitch elements (0: dk) and the slice's dk dims start at column kcol
  int kpitch, kcol;
  int prev_nk, prev_kb;    // backward chunk kernel: key blocks per entry of prev, and the slice's block
  int vb;                  // backward chunk kernel: the value block (of nvb) a pass covers
  int vmode;               // backward chunk kernel: kVSingle, kVFirst or kVLast (value blocks summed)
  float *accf, *acco;      // backward chunk kernel, d_v > 64: fp32 sums over the value blocks so far
};

template <class Io> __device__ __forceinline__ Seq seq_of(const Params &p, int seq) {
  using T = typename Io::T;
  constexpr uint32_t elt = sizeof(T);
  const int bh = seq / p.nvb, vb = seq - bh * p.nvb;
  const int kp = p.kpitch ? p.kpitch : p.dk;
  const size_t kbase = (size_t)bh * p.n_tok * kp + p.kcol;
  const size_t vbase = (size_t)bh * p.n_tok * p.dv + (size_t)kHead * vb;
  const uint32_t kbytes = (uint32_t)p.n_tok * (uint32_t)kp * elt - (uint32_t)p.kcol * elt;
  const uint32_t vbytes = (uint32_t)p.n_tok * (uint32_t)p.dv * elt - (uint32_t)(kHead * vb) * elt;
  auto rsrc = [](const void *ptr, size_t base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(static_cast<const T *>(ptr) + base),
                                             (short)0, (int)bytes, 0x00020000);
  };
  return Seq{rsrc(p.q, kbase, kbytes), rsrc(p.k, kbase, kbytes), rsrc(p.v, vbase, vbytes),
             rsrc(p.g, kbase, kbytes), rsrc(p.out, vbase, vbytes), p.n_tok, p.gh, p.gw, p.dir,
             p.rcp_gh, (uint32_t)kp * elt, (uint32_t)p.dv * elt, p.dk,
             min(kHead, p.dv - kHead * vb)};
}

// Element (i, j) of a sequence's state in the caller's row-major [B*H][d_k][d_v]
// layout, or -1 outside it (i counts within the head, j within the value block).
__device__ __forceinline__ long long user_state_index(const Params &p, int seq, int i, int j) {
  const int bh = seq / p.nvb, vb = seq - bh * p.nvb;
  const int jj = kHead * vb + j;
  if (i >= p.dk || jj >= p.dv) return -1;
  return ((long long)bh * p.dk + i) * p.dv + jj;
}
// Row i = 0 of a sequence's value block in the caller's state, and whether
// this lane's column j of the block exists.
__device__ __forceinline__ size_t user_state_row0(const Params &p, int seq, int j, bool &col_ok) {
  const int bh = seq / p.nvb, vb = seq - bh * p.nvb;
  col_ok = kHead * vb + j < p.dv;
  return (size_t)bh * p.dk * p.dv + (size_t)(kHead * vb + j);
}

// Register-order state layout: (wave w, lane l, reg x) holds element (i, j) with
// i = 16(x/4) + 4(l/16) + x%4 and j = 16w + l%16, at offset w*1024 + x*64 + l.
__device__ __forceinline__ int state_i(int x, int lane) { return 16 * (x >> 2) + 4 * (lane >> 4) + (x & 3); }

// This thread's slice of one chunk: 4 consecutive tokens 16w+4(l/16)+r, dims
// 4(l%16)..+3 of one 64-wide key block and of the value block, of each tensor
// (zeros past the end of the sequence and past d_k or d_v: no key, no value,
// no decay, no query there), and the tokens' grid cells.
template <class Io> struct Rows {
  typename Io::Raw q[4], k[4], v[4], g[4];
  uint32_t off[4];  // grid cells (kNoRow past the end)
  uint32_t before;  // lagged gates: grid cell of the position before the first (kNoRow at the start)
};

template <class Io>
__device__ __forceinline__ typename Io::Raw buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(typename Io::Raw) == 16)
    return __builtin_bit_cast(typename Io::Raw, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  else
    return __builtin_bit_cast(typename Io::Raw, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

// Outputs are written once and not read again by the call: non-temporal stores,
// which leave fewer dirty lines in the caches for later reads to wait behind
// (128x128 four-direction round: 281-288 -> 271-274 us; the state kernel that
// follows each call's outputs went from 24 to 20.6 us).
template <class Io>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, typename Io::Raw v) {
  if constexpr (sizeof(typename Io::Raw) == 16)
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 2);
  else
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 2);
}

// kFirst: the chunk's first key block, which also finds the tokens' grid
// cells and loads v; later key blocks reuse the cells.  With lagged gates each
// position's gate row is that of the position before it along the scan.
template <class Io, bool kOut, bool kFirst>
__device__ __forceinline__ void load_chunk(const Seq &sq, int c, int kb, int wave, int lane, Rows<Io> &x) {
  const int dq = lane & 15;
  if constexpr (kFirst) cells4<Io::kLagGates>(sq, c * kChunk + 16 * wave + 4 * (lane >> 4), x.off, x.before);
  const uint32_t kc = key_col<Io>(sq, kHead * kb + 4 * dq);
  const uint32_t vc = val_col<Io>(sq, 4 * dq);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t o = cell_at(x.off[r], sq.kpitch, kc);
    uint32_t gcell = x.off[r];
    if constexpr (Io::kLagGates)
      if (gcell != kNoRow) gcell = r == 0 ? x.before : x.off[r - 1];
    x.g[r] = buf_load<Io>(sq.g, cell_at(gcell, sq.kpitch, kc));
    x.k[r] = buf_load<Io>(sq.k, o);
    if constexpr (kFirst) x.v[r] = buf_load<Io>(sq.v, cell_at(x.off[r], sq.vpitch, vc));
    if constexpr (kOut) x.q[r] = buf_load<Io>(sq.q, o);
  }
}

// Products across the four 16-lane rows of a wave: x holds this row's value;
// returns the product over rows < g (before) and over rows > g (after), and the
// product over all rows.  Two cross-row swaps, no LDS.
__device__ __forceinline__ void row_products(float x, int g, float &before, float &after, float &all) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float e = __uint_as_float(s16[0]), o = __uint_as_float(s16[1]);  // rows (0,0,2,2), (1,1,3,3)
  const float partner = (g & 1) ? e : o;                                 // row g^1
  const float pair = e * o;                                              // rows {0,1} or {2,3}
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
  const float lo = __uint_as_float(s32[0]), hi = __uint_as_float(s32[1]);  // rows {0,1}, rows {2,3}
  before = ((g & 2) ? lo : 1.f) * ((g & 1) ? partner : 1.f);
  after = ((g & 2) ? 1.f : hi) * ((g & 1) ? 1.f : partner);
  all = lo * hi;
}

// First half of a chunk's operand preparation, local to each wave.  Gate
// products of this thread's 4 tokens x 4 dims inside its wave's 16-token
// sub-block scale the inputs: qs = q * (product of alpha from the sub-block
// start through the token), ks = k * (product of alpha after the token to the
// sub-block end).  qs, ks and (first key block) v go to LDS, the sub-block
// product to sm.tot, the grid cells to sm.rowoff[slot].  One exp2 per element;
// the rest are multiplications and cross-row swaps.
template <class Io, typename Op, bool kOut, int NQ>
__device__ __forceinline__ void prep_local(Smem<Op, NQ> &sm, const Rows<Io> &x, int wave, int lane,
                                           int slot, op4<Op> *qs, op4<Op> *ks, bool first) {
  constexpr int LD = OpT<Op>::LD, LDT = OpT<Op>::LDT;
  const int g = lane >> 4, dq = lane & 15;
  f4 a[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = exp2v(Io::to_f4(x.g[r]) * kLog2e);
  const f4 p1 = a[0] * a[1], p2 = p1 * a[2], p3 = p2 * a[3];  // prefix products in the group
  const f4 s2 = a[3], s1 = a[2] * a[3], s0 = a[1] * s1;        // suffix products in the group
  f4 before, after, all;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float b, f, t;
    row_products(p3[d], g, b, f, t);
    before[d] = b;
    after[d] = f;
    all[d] = t;
  }
  const f4 pq[4] = {a[0] * before, p1 * before, p2 * before, p3 * before};
  const f4 pk[4] = {s0 * after, s1 * after, s2 * after, after};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tau = 16 * wave + 4 * g + r;
    ks[r] = ToOp<Op, Io>::cvt(x.k[r]) * to4<Op>(pk[r]);
    if (first) *reinterpret_cast<op4<Op> *>(&sm.vv[tau * LDT + 4 * dq]) = ToOp<Op, Io>::cvt(x.v[r]);
    if constexpr (kOut) {
      qs[r] = ToOp<Op, Io>::cvt(x.q[r]) * to4<Op>(pq[r]);
      *reinterpret_cast<op4<Op> *>(&sm.qs[tau * LD + 4 * dq]) = qs[r];
      *reinterpret_cast<op4<Op> *>(&sm.ks[tau * LD + 4 * dq]) = ks[r];
    }
  }
  if (g == 0) *reinterpret_cast<f4 *>(&sm.tot[wave * kHead + 4 * dq]) = all;
  if (kOut && first && dq == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.rowoff[slot][16 * wave + 4 * g + r] = x.off[r];
  }
}

// Sub-block products t_0..t_3 of this lane's dims.
template <typename Op, int NQ>
__device__ __forceinline__ void sub_block_products(const Smem<Op, NQ> &sm, int lane, f4 *t) {
  const int dq = lane & 15;
#pragma unroll
  for (int a = 0; a < 4; ++a) t[a] = *reinterpret_cast<const f4 *>(&sm.tot[a * kHead + 4 * dq]);
}

// Second half, after the sub-block products of all waves are visible:
// kb = ks * (product from the sub-block end to the chunk end), qh = qs *
// (product from the chunk start to the sub-block start), and the per-dim
// factor vectors.
template <class Io, typename Op, bool kOut, int NQ>
__device__ __forceinline__ void prep_chunk(Smem<Op, NQ> &sm, const op4<Op> *qs, const op4<Op> *ks,
                                           int wave, int lane, int slot) {
  constexpr int LD = OpT<Op>::LD, LDT = OpT<Op>::LDT;
  const int g = lane >> 4, dq = lane & 15;
  const f4 one = {1.f, 1.f, 1.f, 1.f};
  f4 t[4];
  sub_block_products(sm, lane, t);
  const f4 fk = wave == 0 ? t[1] * t[2] * t[3] : (wave == 1 ? t[2] * t[3] : (wave == 2 ? t[3] : one));
  const op4<Op> fkh = to4<Op>(fk);
  op4<Op> fqh = {};
  if constexpr (kOut)
    fqh = to4<Op>(wave == 0 ? one : (wave == 1 ? t[0] : (wave == 2 ? t[0] * t[1] : t[0] * t[1] * t[2])));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tau = 16 * wave + 4 * g + r;
    if constexpr (Smem<Op, NQ>::kStateTiles)
      *reinterpret_cast<op4<Op> *>(&sm.kb[tau * LDT + 4 * dq]) = ks[r] * fkh;
    if constexpr (kOut && Smem<Op, NQ>::kQueryTiles)
      *reinterpret_cast<op4<Op> *>(&sm.qh[slot][tau * LD + 4 * dq]) = qs[r] * fqh;
  }
  if (g == 0) {
    if (wave == 0) {
      *reinterpret_cast<f4 *>(&sm.dec[4 * dq]) = t[0] * t[1] * t[2] * t[3];
    } else if (kOut && wave == 1) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {  // 2^(-T_a/2) = 1/sqrt(product over sub-block a)
        const f4 h = {__builtin_amdgcn_rsqf(t[a].x), __builtin_amdgcn_rsqf(t[a].y),
                      __builtin_amdgcn_rsqf(t[a].z), __builtin_amdgcn_rsqf(t[a].w)};
        *reinterpret_cast<op4<Op> *>(&sm.hv[a * kHead + 4 * dq]) = to4<Op>(h);
      }
    } else if (kOut && wave == 2) {
      *reinterpret_cast<op4<Op> *>(&sm.cv[0 * kHead + 4 * dq]) = to4<Op>(t[1]);
      *reinterpret_cast<op4<Op> *>(&sm.cv[1 * kHead + 4 * dq]) = to4<Op>(t[1] * t[2]);
      *reinterpret_cast<op4<Op> *>(&sm.cv[2 * kHead + 4 * dq]) = to4<Op>(t[2]);
    }
  }
}

// One element of a q/k/log_gate row, as float: by address (elem) or through a
// buffer resource (key_elem).
template <class Io> __device__ __forceinline__ float elem(const typename Io::T *p) {
  if constexpr (sizeof(typename Io::T) == 4)
    return Io::from_bits(__float_as_uint(*reinterpret_cast<const float *>(p)));
  else
    return Io::from_bits(*reinterpret_cast<const uint16_t *>(p));
}
template <class Io> __device__ __forceinline__ float key_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(typename Io::T) == 4)
    return Io::from_bits(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  else
    return Io::from_bits(__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}

// Exact fp32 diagonal score tile (a, a) of key block kb for a sub-block whose
// gate range is too wide for midpoint scaling.  Re-reads q, k and log_gate
// elements from global memory.
template <class Io>
__device__ f4 exact_diag(const Seq &sq, int c, int a, int kb, int lane) {
  constexpr uint32_t elt = sizeof(typename Io::T);
  const int g = lane >> 4, l16 = lane & 15;
  const int t0 = c * kChunk + 16 * a;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if (t0 + l16 >= sq.n_tok) return acc;  // query beyond the sequence
  const uint32_t qrow = token_cell(sq, t0 + l16) * sq.kpitch;
  uint32_t krow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {  // keys 4g+r <= l16 < n_tok exist; later keys are masked
    const int sl = 4 * g + r;
    krow[r] = token_cell(sq, sl <= l16 ? t0 + sl : t0 + l16) * sq.kpitch;
  }
  const int i_end = min(kHead * (kb + 1), sq.dk);
  for (int i = kHead * kb; i < i_end; ++i) {
    // log2 gate sums from the sub-block start at the query and at each key
    float run = 0.f;
    float e_sig[4] = {0.f, 0.f, 0.f, 0.f};
    for (int u = 0; u <= l16; ++u) {
      run += key_elem<Io>(sq.g, cell_at(gate_cell<Io>(sq, t0 + u), sq.kpitch, i * elt)) * kLog2e;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (u == 4 * g + r) e_sig[r] = run;
    }
    const float qi = key_elem<Io>(sq.q, qrow + i * elt);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r <= l16) acc[r] += qi * key_elem<Io>(sq.k, krow[r] + i * elt) * fast_exp2(run - e_sig[r]);
  }
  return acc;
}

// Off-diagonal score tile (a, b), b < a: P^T[sigma][tau] = ks_sigma . (qs_tau * factor).
template <typename Op, int NQ>
__device__ __forceinline__ void off_tile(Smem<Op, NQ> &sm, int a, int b, int lane) {
  constexpr int LD = OpT<Op>::LD;
  const int g = lane >> 4, l16 = lane & 15;
  const int cvec = (a == 2) ? 0 : (b == 0 ? 1 : 2);  // used when b < a-1
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int k0 = 32 * kb + 4 * g;
    op8<Op> B = frag_row<Op>(&sm.qs[(16 * a + l16) * LD + k0]);
    if (b < a - 1) B = B * frag_row<Op>(&sm.cv[cvec * kHead + k0]);
    acc = mma(frag_row<Op>(&sm.ks[(16 * b + l16) * LD + k0]), B, acc);
  }
  *reinterpret_cast<op4<Op> *>(&sm.pt[tile_slot(a, b) * 256 + lane * 4]) = to4<Op>(acc);
}

// Score tiles P^T[sigma][tau] of this chunk into sm.pt (lower block triangle
// only).  Wave w forms the diagonal tile (w, w) and the off-diagonal tiles
// (1,0),(2,1) | (2,0),(3,2) | (3,0) | (3,1).
template <class Io, typename Op, int NQ>
__device__ __forceinline__ void scores(const Seq &sq, Smem<Op, NQ> &sm, int c, int kb, int wave, int lane) {
  constexpr int LD = OpT<Op>::LD;
  const int g = lane >> 4, l16 = lane & 15;
  {
    const int a = wave;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    if (__all(sm.tot[a * kHead + lane] >= OpT<Op>::kDiagMin)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int k0 = 32 * kb + 4 * g;
        const op8<Op> h = frag_row<Op>(&sm.hv[a * kHead + k0]);
        acc = mma(frag_row<Op>(&sm.ks[(16 * a + l16) * LD + k0]) * h,
                  frag_row<Op>(&sm.qs[(16 * a + l16) * LD + k0]) * h, acc);
      }
    } else {
      acc = exact_diag<Io>(sq, c, a, kb, lane);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > l16) acc[r] = 0.f;  // keys after the query
    *reinterpret_cast<op4<Op> *>(&sm.pt[tile_slot(a, a) * 256 + lane * 4]) = to4<Op>(acc);
  }
  if (wave == 0) {
    off_tile(sm, 1, 0, lane);
    off_tile(sm, 2, 1, lane);
  } else if (wave == 1) {
    off_tile(sm, 2, 0, lane);
    off_tile(sm, 3, 2, lane);
  } else if (wave == 2) {
    off_tile(sm, 3, 0, lane);
  } else {
    off_tile(sm, 3, 1, lane);
  }
}

// Largest of a wave's 64 values of v (unsigned), in every lane: across the
// four 16-lane rows with two row swaps, then within each row with DPP
// rotations by 8, 4, 2 and 1 lanes.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)s16[0], (uint32_t)s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max((uint32_t)s32[0], (uint32_t)s32[1]);
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false));  // row_ror:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false));  // row_ror:1
  return __builtin_amdgcn_readfirstlane(v);
}

// A state slice S (this wave's 16 columns, 16 values per lane) becomes an fp16
// MFMA operand through an exact power of two 2^k chosen from its largest
// magnitude m, so that m 2^k lies in [2^14, 2^15): nothing overflows fp16's
// 65504, and small states keep fp16's full precision instead of falling into
// its subnormal range.  Returns 2^k and sets unscale = 2^-k, by which the
// fp32 product is multiplied back (exactly).  A zero, infinite or NaN slice
// keeps k = 0.
__device__ __forceinline__ float state_scale(const f4 *S, float &unscale) {
  uint32_t m = 0;
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = max(m, __float_as_uint(S[it][r]) & 0x7fffffffu);
  m = wave_max(m);
  int k = 0;
  if (m != 0 && m < 0x7f800000u) k = min(126, max(-126, 14 - ((int)(m >> 23) - 127)));
  unscale = __uint_as_float((uint32_t)(127 - k) << 23);
  return __uint_as_float((uint32_t)(127 + k) << 23);
}

// How a walk treats each chunk.
enum : int {
  kAgg = 0,    // state only: no queries, no outputs
  kStore = 1,  // outputs formed with the state carried so far and stored
  kKeep = 2,   // outputs formed with the state carried so far and kept in registers
};

// O^T[16w:16w+16][chunk] = V^T P^T + S^T (q 2^E)^T for one key block, added to
// keep[tt] (kAcc: an earlier key block's part).  The last key block (kFinal)
// rounds the sum to the I/O format into the output tile ot[token][dim]
// (kStore) or leaves it in keep (kKeep); earlier ones leave it in keep.
template <class Io, typename Op, int kMode, bool kAcc, bool kFinal, int NQ>
__device__ __forceinline__ void outputs(const Smem<Op, NQ> &sm, int wave, int lane, int slot,
                                        const op8<Op> *vf, const f4 *S, typename OpT<Op>::Bits *ot,
                                        f4 *keep) {
  constexpr int LD = OpT<Op>::LD;
  constexpr bool kScaled = sizeof(Op) == 2;  // 16-bit operands: the state goes through state_scale
  const int g = lane >> 4, l16 = lane & 15;
  op8<Op> sf[2];
  float unscale = 1.f;
  const float scale = kScaled ? state_scale(S, unscale) : 1.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) sf[kb] = cat(to4<Op>(S[2 * kb] * scale), to4<Op>(S[2 * kb + 1] * scale));
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kAcc) acc = keep[tt];
    if constexpr (kScaled) {  // the state term on its own accumulator, scaled back, then the scores
      f4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        st = mma(sf[kb], frag_row<Op>(&sm.qh[slot][(16 * tt + l16) * LD + 32 * kb + 4 * g]), st);
      acc += st * unscale;
    }
#pragma unroll
    for (int kb = 0; kb <= (tt >> 1); ++kb) {
      const op4<Op> lo = *reinterpret_cast<const op4<Op> *>(&sm.pt[tile_slot(tt, 2 * kb) * 256 + lane * 4]);
      op4<Op> hi = {};
      if (2 * kb + 1 <= tt)
        hi = *reinterpret_cast<const op4<Op> *>(&sm.pt[tile_slot(tt, 2 * kb + 1) * 256 + lane * 4]);
      acc = mma(vf[kb], cat(lo, hi), acc);
    }
    if constexpr (!kScaled) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc = mma(sf[kb], frag_row<Op>(&sm.qh[slot][(16 * tt + l16) * LD + 32 * kb + 4 * g]), acc);
    }
    if constexpr (kMode == kStore && kFinal)
      *reinterpret_cast<typename Io::Raw *>(&ot[(16 * tt + l16) * OpT<Op>::LDO + 16 * wave + 4 * g]) =
          Io::pack(acc);
    else
      keep[tt] = acc;
  }
}

// S <- diag(2^E_last) S + (k 2^(E_last-E))^T V for this wave's value columns.
template <typename Op, int NQ>
__device__ __forceinline__ void carry_state(const Smem<Op, NQ> &sm, int lane, const op8<Op> *vf, f4 *S) {
  const int g = lane >> 4;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    S[it] *= *reinterpret_cast<const f4 *>(&sm.dec[16 * it + 4 * g]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) S[it] = mma(frag_tr(sm.kb, 32 * kb, 16 * it, lane), vf[kb], S[it]);
  }
}

// Stores a finished output tile: this thread's 4 tokens (grid cells cell[r])
// x 4 dims, so each store instruction writes whole rows of the value block.
template <class Io, typename Op>
__device__ __forceinline__ void flush_tile(const Seq &sq, const typename OpT<Op>::Bits *ot,
                                           const uint32_t *cell, int wave, int lane) {
  const int g = lane >> 4, dq = lane & 15;
  const uint32_t vc = val_col<Io>(sq, 4 * dq);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const typename Io::Raw v =
        *reinterpret_cast<const typename Io::Raw *>(&ot[(16 * wave + 4 * g + r) * OpT<Op>::LDO + 4 * dq]);
    buf_store<Io>(sq.o, cell_at(cell[r], sq.vpitch, vc), v);
  }
}

// One chunk, using LDS slot `slot` for what must outlive it, as NK passes, one
// per 64-wide key block: each pass carries its block's state S[kb] and adds its
// part of the outputs (the scores and q S both sum over key dims); v is loaded
// and staged once.  Barriers per pass: (1) sub-block products and grid cells
// visible, (2) operand tiles visible, (3) score tiles visible.  Everything a
// wave reads from LDS after the last barrier of a pass (pt, qh, kb, dec) is
// written only after the first barrier of the next pass, which no wave passes
// before every wave has finished this one; v and the output grid cells, which
// the next chunk overwrites before its first barrier, are read into registers
// before the second one.  The next pass's rows (the next key block, or the next
// chunk's first) are loaded into x as soon as this pass's have gone to LDS,
// and arrive while the rest of this pass computes.  seg_dec[kb] (wave 0, lanes
// < 16, dims 4*lane..+3) accumulates the chunk decays; kKeep also records the
// decay from the segment start to this chunk in sm.dcum[slot].  kStore: the
// previous chunk's output tile (complete at this chunk's first barrier,
// rewritten only after its last pass's third) is stored after the first
// barrier; pend carries the grid cells of the tile's tokens from chunk to chunk.
template <class Io, typename Op, int kMode, int NK, int NQ>
__device__ __forceinline__ void chunk(const Seq &sq, Smem<Op, NQ> &sm, Rows<Io> &x, int c, int c_end,
                                      int wave, int lane, int slot, f4 (*S)[4], f4 *seg_dec, f4 *keep,
                                      typename OpT<Op>::Bits *ot, uint32_t *pend, bool have_pend) {
  constexpr bool kOut = kMode != kAgg;
  op8<Op> vf[2];
  f4 part[4];  // outputs summed over the key blocks so far
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    const bool first = kb == 0;
    op4<Op> qs[4], ks[4];
    prep_local<Io, Op, kOut>(sm, x, wave, lane, slot, qs, ks, first);
    uint32_t cur[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) cur[r] = x.off[r];
    if (kb + 1 < NK)
      load_chunk<Io, kOut, false>(sq, c, kb + 1, wave, lane, x);
    else if (c + 1 < c_end)
      load_chunk<Io, kOut, true>(sq, c + 1, 0, wave, lane, x);
    lds_sync();
    if constexpr (kMode == kStore) {
      if (first) {
        if (have_pend) flush_tile<Io, Op>(sq, ot, pend, wave, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) pend[r] = cur[r];
      }
    }
    // kept outputs need each key block's query tile and decays until the
    // segment's entering state is known: LDS slots slot * NK + kb
    const int qslot = kMode == kKeep ? slot * NK + kb : slot;
    prep_chunk<Io, Op, kOut>(sm, qs, ks, wave, lane, qslot);
    if (first) {
#pragma unroll
      for (int b = 0; b < 2; ++b) vf[b] = frag_tr(sm.vv, 32 * b, 16 * wave, lane);
    }
    if (kMode != kStore && wave == 0 && lane < 16) {
      f4 t[4];
      sub_block_products(sm, lane, t);
      if constexpr (kMode == kKeep) *reinterpret_cast<f4 *>(&sm.dcum[qslot][4 * lane]) = seg_dec[kb];
      seg_dec[kb] *= t[0] * t[1] * t[2] * t[3];
    }
    lds_sync();
    if constexpr (kOut) {
      scores<Io, Op>(sq, sm, c, kb, wave, lane);
      lds_sync();
      f4 *acc = kMode == kKeep ? keep : part;
      if (kb == 0 && kb + 1 == NK)
        outputs<Io, Op, kMode, false, true>(sm, wave, lane, qslot, vf, S[kb], ot, acc);
      else if (kb == 0)
        outputs<Io, Op, kMode, false, false>(sm, wave, lane, qslot, vf, S[kb], ot, acc);
      else if (kb + 1 == NK)
        outputs<Io, Op, kMode, true, true>(sm, wave, lane, qslot, vf, S[kb], ot, acc);
      else
        outputs<Io, Op, kMode, true, false>(sm, wave, lane, qslot, vf, S[kb], ot, acc);
    }
    carry_state<Op>(sm, lane, vf, S[kb]);
  }
}

// Walks chunks [c_begin, c_end) of sequence `seq`, carrying S (kAgg or kStore):
// kStore writes the outputs (S must hold the state entering the first chunk);
// kAgg only carries S (from zero: the segment's own aggregate) and multiplies
// the chunk decays into seg_dec.
template <class Io, typename Op, int kMode, int NK, int NQ>
__device__ __forceinline__ void walk(const Params &p, int seq, Smem<Op, NQ> &sm, int c_begin, int c_end,
                                     int wave, int lane, f4 (*S)[4], f4 *seg_dec,
                                     typename OpT<Op>::Bits *ot = nullptr) {
  static_assert(kMode != kKeep, "kKeep walks are unrolled by their kernel");
  const Seq sq = seq_of<Io>(p, seq);
  Rows<Io> x;
  uint32_t pend[4];
  load_chunk<Io, kMode != kAgg, true>(sq, c_begin, 0, wave, lane, x);
  for (int c = c_begin; c < c_end; ++c)
    chunk<Io, Op, kMode, NK>(sq, sm, x, c, c_end, wave, lane, 0, S, seg_dec, nullptr, ot, pend,
                             c > c_begin);
  if constexpr (kMode == kStore) {
    lds_sync();  // the last output tile is complete
    flush_tile<Io, Op>(sq, ot, pend, wave, lane);
  }
}

// Writes key block kb of a register-order state into the caller's row-major
// [B*H][d_k][d_v] state (elements past d_k or d_v are not written).
__device__ __forceinline__ void store_user_state(const Params &p, float *dst, int seq, int kb, int wave,
                                                 int lane, const f4 *S) {
  bool col_ok;
  float *d = dst + user_state_row0(p, seq, 16 * wave + (lane & 15), col_ok);
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int i = kHead * kb + state_i(x, lane);
    if (col_ok && i < p.dk) d[(size_t)i * p.dv] = S[x >> 2][x & 3];
  }
}

// ------------------------------------------------------------------ kernels
// Workspace layout: [seq][segment][key block] then 4096 register-order state
// elements, or 64 decays.
template <int NK> __device__ __forceinline__ size_t ws_block(const Params &p, int seq, int seg, int kb) {
  return ((size_t)seq * p.n_seg + seg) * NK + kb;
}

template <class Io, typename Op, int NK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NK == 1 ? 3 : 2, NK == 1 ? 3 : 2))) void gla_seg_state(Params p) {
  __shared__ Smem<Op, 0> sm;  // state only
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = blockIdx.x / p.n_seg_grid;
  const int seg = blockIdx.x - seq * p.n_seg_grid;
  f4 S[NK][4] = {};
  f4 sdec[NK];
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) sdec[kb] = f4{1.f, 1.f, 1.f, 1.f};
  const int c0 = seg * p.seg_len;
  walk<Io, Op, kAgg, NK>(p, seq, sm, c0, min(c0 + p.seg_len, p.n_chunk), wave, lane, S, sdec);
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    const size_t st = ws_block<NK>(p, seq, seg, kb) * kStateElems + wave * 1024 + lane;
#pragma unroll
    for (int x = 0; x < 16; ++x) p.agg[st + x * 64] = S[kb][x >> 2][x & 3];
    if (wave == 0 && lane < 16)
      *reinterpret_cast<f4 *>(&p.agg_dec[ws_block<NK>(p, seq, seg, kb) * kHead + 4 * lane]) = sdec[kb];
  }
}

// (Its output tile brings LDS to 63.6 KB at 16-bit I/O, two workgroups per CU;
// with fp32 operands to 118 KB, one.)
template <typename Op> constexpr int kOutOccupancy = sizeof(Op) == 4 ? 1 : 2;
template <class Io, typename Op, int NK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    kOutOccupancy<Op>, kOutOccupancy<Op>))) void gla_seg_out(Params p) {
  __shared__ Smem<Op, 1> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = blockIdx.x / p.n_seg;
  const int seg = blockIdx.x - seq * p.n_seg;
  // The entering state, read through a buffer resource that is empty when
  // there is none (every load then returns 0): no branch, so these loads and
  // the first chunk's are in flight together.
  f4 S[NK][4];
  {
    const size_t entry = ((size_t)seq * p.prev_seq + (size_t)seg * p.prev_step) * NK;
    const float *src = p.prev ? p.prev + entry * kStateElems : nullptr;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(src), (short)0, p.prev ? NK * kStateElems * (int)sizeof(float) : 0, 0x00020000);
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int x = 0; x < 16; ++x)
        S[kb][x >> 2][x & 3] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(r, (kb * kStateElems + wave * 1024 + x * 64 + lane) * 4, 0, 0));
  }
  __shared__ __attribute__((aligned(16))) typename OpT<Op>::Bits ot[kChunk * OpT<Op>::LDO];
  f4 unused[NK];
  const int c0 = seg * p.seg_len;
  walk<Io, Op, kStore, NK>(p, seq, sm, c0, min(c0 + p.seg_len, p.n_chunk), wave, lane, S, unused, ot);
}

// Boundary-state recurrence over segments, one thread per (sequence, key
// block, state element): prev[seg] = state entering segment seg; prev[0] = s0
// (or 0).  Loads of a batch of segments are issued together; only the fused
// multiply-adds are sequential.  Segments are NK*4096 floats apart, a
// compile-time stride, so a batch's loads share one address.
template <int NK>
__global__ __launch_bounds__(kThreads) void gla_seg_scan(Params p) {
  constexpr int kBatch = 32;
  constexpr int kPerSeq = NK * kStateElems;
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  const int seq = (int)(gid / kPerSeq);
  if (seq >= p.bh_count) return;
  const int eb = (int)(gid - (long)seq * kPerSeq);
  const int kb = eb / kStateElems, e = eb - kb * kStateElems;
  const int w = e >> 10, x = (e >> 6) & 15, l = e & 63;
  const int i = state_i(x, l);
  const int n_seg = p.n_seg;
  const size_t first = (size_t)seq * n_seg * NK + kb;  // workspace block of segment 0
  const float *agg = p.agg + first * kStateElems + e;
  const float *dec = p.agg_dec + first * kHead + i;
  float *prev = const_cast<float *>(p.prev) + first * kStateElems + e;
  const long long user = (p.s0 || p.s_final) ? user_state_index(p, seq, kHead * kb + i, 16 * w + (l & 15)) : -1;
  const int steps = p.s_final ? n_seg : n_seg - 1;
  // The first batch's loads go out before s0 is read (clamped, so they are
  // valid even with no step), so the s0 branch does not delay them.
  float av[kBatch], dv[kBatch];
  auto issue = [&](int b0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int seg = max(min(b0 + u, steps - 1), 0);
      av[u] = agg[(size_t)seg * kPerSeq];
      dv[u] = dec[(size_t)seg * NK * kHead];
    }
  };
  issue(0);
  float s = (p.s0 && user >= 0) ? p.s0[user] : 0.f;
  prev[0] = s;
  for (int b0 = 0; b0 < steps; b0 += kBatch) {
    if (b0 > 0) issue(b0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (b0 + u < steps) {
        s = dv[u] * s + av[u];
        if (b0 + u + 1 < n_seg) prev[(size_t)(b0 + u + 1) * kPerSeq] = s;
      }
    }
  }
  if (p.s_final && user >= 0) p.s_final[user] = s;
}

// The same recurrence for chains of at most 64 steps, as a scan across the
// lanes of a wave.  Lane u of a group of P lanes (P the smallest power of two
// >= the steps) holds segment u's aggregate for 16 consecutive state elements
// (one row i, 16 columns) and its decay for that row; log2(P) rounds of
// ds_bpermute combine each lane's block with the block before it:
//   (D_e, A_e) then (D_l, A_l)  ->  (D_e D_l, D_l A_e + A_l),
// after which lane u holds the state after segments 0..u from zero and the
// product of their decays, and writes the state entering segment u + 1 (plus
// the product times s0).  Loads and stores are 16-byte vectors; every lane of
// a wave takes part in every round (lanes past the steps carry the identity).
__device__ __forceinline__ float lane_from(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

template <int NK>
__global__ __launch_bounds__(kThreads) void gla_seg_scan_lanes(Params p) {
  constexpr int kGroups = kStateElems / 16;  // element groups per state block
  const int n_seg = p.n_seg;
  const int steps = p.s_final ? n_seg : n_seg - 1;
  int P = 1;
  while (P < steps) P <<= 1;
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  const long grp = gid / P;
  const int u = (int)(gid - grp * P), lane = threadIdx.x & 63;
  const long seq_l = grp / (NK * kGroups);
  const bool valid = seq_l < p.bh_count;
  const int seq = valid ? (int)seq_l : 0;
  const int rg = (int)(grp - seq_l * (NK * kGroups)) & (NK * kGroups - 1);
  const int kb = rg / kGroups, e0 = 16 * (rg % kGroups);
  const int w = e0 >> 10, x = (e0 >> 6) & 15, i = state_i(x, e0 & 63);
  const bool have = valid && u < steps;
  const size_t blk = ((size_t)seq * n_seg + (size_t)min(u, max(steps - 1, 0))) * NK + kb;
  f4 A[4];
  float D = have ? p.agg_dec[blk * kHead + i] : 1.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    A[q] = have ? *reinterpret_cast<const f4 *>(p.agg + blk * kStateElems + e0 + 4 * q) : f4{0.f, 0.f, 0.f, 0.f};
  for (int k = 1; k < P; k <<= 1) {
    const int src = (lane - k) & 63;
    const float De = lane_from(D, src);
    f4 Ae[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) Ae[q][c] = lane_from(A[q][c], src);
    if (u >= k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) A[q] = D * Ae[q] + A[q];
      D = De * D;
    }
  }
  if (!valid) return;
  // s0 for these 16 elements (row i of key block kb, columns 16 w .. 16 w + 15 of the value block)
  f4 S0[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const long long ui = p.s0 ? user_state_index(p, seq, kHead * kb + i, 16 * w + 4 * q + c) : -1;
      S0[q][c] = ui >= 0 ? p.s0[ui] : 0.f;
    }
  float *prev = const_cast<float *>(p.prev);
  const size_t first = (size_t)seq * n_seg * NK + kb;  // workspace block of segment 0
  if (u == 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<f4 *>(prev + first * kStateElems + e0 + 4 * q) = S0[q];
  if (!have) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) A[q] = D * S0[q] + A[q];
  if (u + 1 < n_seg) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f4 *>(prev + (first + (size_t)(u + 1) * NK) * kStateElems + e0 + 4 * q) = A[q];
  } else if (p.s_final) {  // u = n_seg - 1: the state after the sequence
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const long long ui = user_state_index(p, seq, kHead * kb + i, 16 * w + 4 * q + c);
        if (ui >= 0) p.s_final[ui] = A[q][c];
      }
  }
}

// ------------------------------------------------------------ one-launch path
//
// The caller's fp32 state of sequence `bh` (s0 or s_final, row-major
// [B*H][d_k][d_v]) as a buffer resource, and the byte offset of this thread's
// element (row i, column 16 wave + lane%16 of the value block), or -1 (out of
// range: reads 0, stores dropped) past d_k or d_v.  The head dims pass through
// an empty asm statement, so these offsets are formed where they are used, not
// hoisted out of the workgroup's loop and held (spilled) across every segment.
struct UserState {
  __amdgpu_buffer_rsrc_t r;
  int dk, dv, j;
};
__device__ __forceinline__ UserState user_state(const Params &p, const float *base, int bh, int wave, int lane) {
  int dk = p.dk, dv = p.dv;
  asm volatile("" : "+s"(dk), "+s"(dv));
  const int bhh = bh / p.nvb, j = kHead * (bh - bhh * p.nvb) + 16 * wave + (lane & 15);
  return UserState{__builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base) + (size_t)bhh * dk * dv, (short)0,
                                                     dk * dv * (int)sizeof(float), 0x00020000),
                   dk, dv, j};
}
__device__ __forceinline__ int user_state_off(const UserState &u, int i) {
  return (i < u.dk && u.j < u.dv) ? (i * u.dv + u.j) * (int)sizeof(float) : -1;
}

//
// Exchange between workgroups.  All segments of a sequence are processed on
// one XCD (take_work), so the aggregates, block prefixes and flags that pass
// between them go through that XCD's L2 and never cross the fabric: the
// producer writes a payload with plain stores, waits until they have completed
// (they are then in L2), synchronises the workgroup, and one thread stores the
// segment's flag; consumers poll the flag and read payloads with non-temporal
// loads, which do not hit in the CU's L1 and are served by L2.  Measured on
// MI355X: no stale read in 256000 reads within an XCD.  Plain loads there hit
// stale L1 lines, and across XCDs the L2s are not coherent with each other:
// that is why a sequence never spans two XCDs.  Flags only ever hold epochs
// and grow from call to call, so a stale copy can never pass for a fresh one.
constexpr int kNonTemporal = 2;  // buffer-access cache policy: nt

// XCC_ID (hardware register 20, bits 3:0): the XCD this wave runs on.  Waves
// with equal ids share one L2.
__device__ __forceinline__ int xcc_slot() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcdSlots - 1));
}

// A sequence's segment flags as a buffer resource (8 bytes per segment).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t flag_rsrc(const Params &p, int bh) {
  return __builtin_amdgcn_make_buffer_rsrc(p.flags + (size_t)bh * p.n_seg, (short)0, p.n_seg * 8, 0x00020000);
}
__device__ __forceinline__ long long read_flag(__amdgpu_buffer_rsrc_t f, int s) {
  return __builtin_bit_cast(long long, __builtin_amdgcn_raw_buffer_load_b64(f, s * 8, 0, kNonTemporal));
}

// Bounded wait until segment s's flag reaches `want`.  A wait that gives up
// records -1 in the error word and returns false.
__device__ __forceinline__ bool wait_flag(int *sync, __amdgpu_buffer_rsrc_t f, int s, long long want) {
  for (int spins = 0; read_flag(f, s) < want; ++spins) {
    if (spins > kSpinLimit) {
      __hip_atomic_store(sync + kSyncErrorWord, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Waits until this wave's stores have completed.
__device__ __forceinline__ void stores_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work of one XCD.  Sequences are handed out in batches of p.batch.  XCD x
// starts with batch x (x < p.n_pre); later batches come from a counter shared
// by all XCDs.  The workgroups of an XCD take tickets t = 0, 1, ... of its
// current batch, ticket t being segment t / k of the batch's sequence t % k
// (k sequences in the batch).  Tickets follow scan order within each sequence,
// so every segment a workgroup waits for holds a smaller ticket, taken by a
// running workgroup of the same XCD (which is why a workgroup may leave while
// another one of its XCD still has work: no ticket waits on a later one).
// The XCD's 64-bit work word holds (tag << 32) + next ticket, the tag being
// 0 (the starting batch, or none),
// batch + 1, kStolen or kBatchDone.  The workgroup whose ticket is the first
// past the end of its batch takes the next batch and keeps its ticket 0;
// workgroups past it wait until it has.  When the counter runs out, that
// workgroup takes over the starting batch of an XCD whose work word no
// workgroup has touched yet (changing it to kStolen, so that XCD's workgroups
// take no ticket of it), which covers an XCD that never runs a workgroup of
// this launch.
constexpr unsigned kBatchDone = 0xffffffffu, kStolen = 0xfffffffeu;
__device__ __forceinline__ unsigned long long *work_word(const Params &p, int slot) {
  return reinterpret_cast<unsigned long long *>(p.sync + kSyncSlotWord + slot * kSlotStride);
}
// Takes the next ticket of the XCD's batch: the returned word, read by take_work.
__device__ __forceinline__ unsigned long long work_add(const Params &p, int slot) {
  return __hip_atomic_fetch_add(work_word(p, slot), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Turns the word a work_add returned into a segment: writes the sequence and
// segment to out[0], out[1] (out[0] = -1: no work left).
__device__ void take_work(const Params &p, int slot, unsigned long long v, int *out) {
  unsigned long long *word = work_word(p, slot);
  auto start = [&](int b) {  // this workgroup starts batch b with ticket 0
    __hip_atomic_store(word, ((unsigned long long)b + 1ull) << 32 | 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    out[0] = b * p.batch;
    out[1] = 0;
  };
  for (int spins = 0;; v = work_add(p, slot)) {
    const unsigned tag = (unsigned)(v >> 32), t = (unsigned)v;
    if (tag == kBatchDone) {
      out[0] = -1;
      return;
    }
    const int b = tag == 0 ? (slot < p.n_pre ? slot : -1) : (tag == kStolen ? -1 : (int)tag - 1);
    const int first = b * p.batch, k = b < 0 ? 0 : min(p.batch, p.bh_count - first);
    const unsigned n_in = (unsigned)k * (unsigned)p.n_seg;
    if (t < n_in) {
      if (tag == 0 && t == 0)  // this XCD has begun its starting batch
        __hip_atomic_fetch_or(p.sync + kSyncStartedWord, 1 << slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      out[0] = first + (int)(t % (unsigned)k);
      out[1] = (int)(t / (unsigned)k);
      return;
    }
    if (t == n_in) {  // the next batch for this XCD (none beyond the starting ones: no counter)
      const int nb = p.n_pre >= p.n_batch ? p.n_batch
                                          : p.n_pre + __hip_atomic_fetch_add(p.sync + kSyncNextBatchWord, 1,
                                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (nb < p.n_batch) {
        start(nb);
        return;
      }
      // none left: a starting batch that its XCD has not begun (the started
      // mask only saves compare-exchanges; the exchange itself decides)
      const unsigned started =
          (unsigned)__hip_atomic_load(p.sync + kSyncStartedWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int y = 0; y < p.n_pre; ++y) {
        unsigned long long zero = 0;
        if (y != slot && !(started >> y & 1u) &&
            __hip_atomic_compare_exchange_strong(work_word(p, y), &zero, (unsigned long long)kStolen << 32,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          start(y);
          return;
        }
      }
      __hip_atomic_store(word, (unsigned long long)kBatchDone << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      out[0] = -1;
      return;
    }
    // Another workgroup of this XCD is taking the next batch.  With no batch
    // beyond the starting ones, that workgroup can only take over a starting
    // batch that another XCD has not begun.  After a batch of this XCD's own
    // (b >= 0) it is a workgroup that has just finished a segment, and such a
    // batch is left only where an XCD runs no workgroup of this launch: leave
    // now rather than poll the work word beside the working ones (the taker
    // works it alone).  Without one (an XCD with no starting batch, or whose
    // batch was taken), it acts at launch, where a batch whose XCD has not
    // begun yet is common: wait, and work the batch it takes with all the
    // workgroups of this XCD.  (Leaving then left such a batch to one
    // workgroup: 64x64 B1 H12 with 2-chunk segments took 1.2 ms per
    // four-call round instead of 0.10 ms.)
    if (p.n_pre >= p.n_batch && b >= 0) {
      out[0] = -1;
      return;
    }
    while ((unsigned)(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) == tag) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(p.sync + kSyncErrorWord, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        out[0] = -1;
        return;
      }
    }
  }
}

// A sequence's payload slots: per segment and key block (slot s * NK + kb), a
// 64x64 fp32 state (the segment's aggregate, or for a block's last segment
// the block prefix) in f4 register order, then the segment's 64 decays of
// that key block.
template <int NK> __device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const Params &p, int bh) {
  return __builtin_amdgcn_make_buffer_rsrc(p.agg + (size_t)bh * p.n_seg * NK * kSlotFloats, (short)0,
                                           p.n_seg * NK * kSlotFloats * (int)sizeof(float), 0x00020000);
}
// Byte offsets: f4 `it` of thread (wave, lane) of slot s's state (rows
// 16 it + 4(lane/16) + 0..3, column 16 wave + lane%16), and decay `row`.
__device__ __forceinline__ int slot_state_off(int s, int wave, int it, int lane) {
  return (s * kSlotFloats + ((wave * 4 + it) * 64 + lane) * 4) * (int)sizeof(float);
}
__device__ __forceinline__ int slot_decay_off(int s, int row) {
  return (s * kSlotFloats + kStateElems + row) * (int)sizeof(float);
}
__device__ __forceinline__ f4 slot_load(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}
__device__ __forceinline__ void slot_store(__amdgpu_buffer_rsrc_t r, int off, f4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, 0);
}

// Writes the NK key blocks of state X (and, kDecay, their decays dec[kb]
// held by wave 0, lanes < 16) to segment s's slots, then raises its flag.
// Every thread of the workgroup calls it.
template <bool kDecay, int NK>
__device__ __forceinline__ void publish(const Params &p, __amdgpu_buffer_rsrc_t r, int bh, int s, int tid,
                                        const f4 (*X)[4], const f4 *dec, long long want) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
#pragma unroll
    for (int it = 0; it < 4; ++it) slot_store(r, slot_state_off(s * NK + kb, wave, it, lane), X[kb][it]);
    if (kDecay && wave == 0 && lane < 16) slot_store(r, slot_decay_off(s * NK + kb, 4 * lane), dec[kb]);
  }
  stores_complete();  // this wave's payload is in L2 ...
  __syncthreads();    // ... for every wave ...
  if (tid == 0)       // ... before the flag is raised
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, want), flag_rsrc(p, bh), s * 8, 0, 0);
}

// Workgroups per CU: fp32 operands take 100-137 KB of LDS, one; two key
// blocks (a query tile per key block and kept chunk) 64-98 KB, one; 16-bit
// ones 54-73 KB, two.  The 54 KB of one-chunk segments would let three share
// a CU, but three leave 168 registers per lane and the fold then spills to
// scratch (40x40 B1 H6 with one-chunk segments: 80-90 us per call with three,
// 15 us with two).
template <typename Op, int kSeg, int NK>
constexpr int kFusedOccupancy = sizeof(Op) == 4 || NK == 2 ? 1 : 2;

// One launch.  A persistent grid; each workgroup repeatedly takes a segment
// (at most kSeg chunks) of a sequence of its XCD and:
//   1. walks it from a zero state, keeping each chunk's outputs in registers
//      (intra-segment part: scores plus the state carried inside the segment)
//      and ending with the segment's own aggregate A and decay D;
//   2. publishes (A, D) for the later segments of its block (segments are
//      grouped in blocks of p.fold_block);
//   3. forms S_prev, the state entering the segment, by folding in a fixed
//      order the aggregates of the earlier segments of its block and the
//      entering term: the prefix published by the previous block's last
//      segment, or s0 in the first block;
//   4. if it is a block's last segment, publishes that block's prefix
//      D S_prev + A; the sequence's last segment writes it as s_final;
//   5. adds each chunk's share of S_prev, (q 2^E * Dcum) S_prev with Dcum the
//      decay from the segment start to the chunk, and stores the outputs.
// Inputs are read from HBM once.  The fold order depends only on the shape,
// so a call gives bitwise the same result however its workgroups run.
template <class Io, typename Op, int kSeg, int NK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    kFusedOccupancy<Op, kSeg, NK>, kFusedOccupancy<Op, kSeg, NK>))) void gla_fused(Params p) {
  __shared__ Smem<Op, kSeg * NK> sm;
  __shared__ int s_work[2];
  __shared__ int s_fail;
  __shared__ long long s_epoch;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int slot = xcc_slot();
  if (tid == 0) {
    // flag value of this call: the epoch (calls completed on this workspace) + 1;
    // earlier calls left at most the epoch.  Read together with the first ticket.
    const long long e = __hip_atomic_load(reinterpret_cast<long long *>(p.sync + kSyncEpochWord), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long v = work_add(p, slot);
    s_epoch = e;
    take_work(p, slot, v, s_work);
  }
  __syncthreads();
  // uniform: scalar registers
  const long long want = (long long)(((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((int)(s_epoch >> 32)) << 32) |
                                     (unsigned)__builtin_amdgcn_readfirstlane((int)s_epoch)) + 1;
  const int G = p.fold_block;
  // the current segment (uniform across the workgroup: scalar registers, so the
  // buffer resources built from them stay scalar), and its first chunk's rows
  int bh = __builtin_amdgcn_readfirstlane(s_work[0]), seg = __builtin_amdgcn_readfirstlane(s_work[1]);
  while (bh >= 0) {
    if (tid == 0) s_fail = 0;
    __syncthreads();  // s_work has been read by every thread before it is rewritten below
    // the next ticket's work-word increment, issued now so that it returns during the walk
    unsigned long long next_word = 0;
    if (tid == kThreads - 1) next_word = work_add(p, slot);
    const int c0 = seg * p.seg_len, c1 = min(c0 + p.seg_len, p.n_chunk);
    const Seq sq = seq_of<Io>(p, bh);
    const __amdgpu_buffer_rsrc_t slots = slot_rsrc<NK>(p, bh);

    // 1. the segment from a zero state
    Rows<Io> x;
    load_chunk<Io, true, true>(sq, c0, 0, wave, lane, x);
    f4 keep[kSeg][4];
    f4 L[NK][4] = {};
    f4 sdec[NK];
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) sdec[kb] = f4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int j = 0; j < kSeg; ++j)
      if (c0 + j < c1)
        chunk<Io, Op, kKeep, NK>(sq, sm, x, c0 + j, c1, wave, lane, j, L, sdec, keep[j], nullptr, nullptr,
                                 false);
    // decay across the whole segment (key dim 64 kb + i at kb * 64 + i); tot
    // is not read after a chunk's last barrier, so wave 0 may overwrite it
    // while others finish
    float *segdec = sm.tot;
    static_assert(sizeof(sm.tot) >= NK * kHead * sizeof(float), "segment decays fit in tot");
    if (wave == 0 && lane < 16)
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) *reinterpret_cast<f4 *>(&segdec[kb * kHead + 4 * lane]) = sdec[kb];
    lds_sync();  // segdec visible; qs (the fold's scratch below) no longer read

    // 2. the aggregate, for the later segments of this block
    const int blk0 = seg - seg % G;          // first segment of this block
    const bool blk_last = seg % G == G - 1;  // publishes the block prefix instead
    const bool has_next = seg + 1 < p.n_seg;
    if (has_next && !blk_last) publish<true, NK>(p, slots, bh, seg, tid, L, sdec, want);

    // 3. S_prev: first the aggregates of this block's earlier segments ...
    const int n_a = seg - blk0;
    const bool has_p = blk0 > 0;  // ... then the prefix of the previous block, or s0
    const bool have_prev = seg > 0 || p.s0 != nullptr;
    const __amdgpu_buffer_rsrc_t fl = flag_rsrc(p, bh);
    if (have_prev && tid < n_a && !wait_flag(p.sync, fl, blk0 + tid, want)) s_fail = 1;
    __syncthreads();  // every awaited aggregate is visible
    f4 S[NK][4] = {};
    if (have_prev) {
      // Horner's rule over the block's earlier segments, oldest first:
      // X <- D_u X + A_u (per key block), and prod = product of their decays,
      // for the entering term.  Each round trip brings kBatch aggregates and
      // their decays; the decays (one per thread) go through LDS to the rows
      // each thread holds.
      // Two aggregates per round trip: four keep 32 more registers live beside
      // the kept outputs, which spilled them at 3-chunk segments (40x40 B8 H6:
      // 114 -> 112 us per round without the spills).
      constexpr int kBatch = 2;
      constexpr int kDecays = NK * kHead;                                            // decays per aggregate
      static_assert(kBatch * kDecays <= kThreads, "one decay per thread");
      float *dlds = reinterpret_cast<float *>(sm.qs);  // [2][kBatch][NK * 64], alternating
      static_assert(sizeof(sm.qs) >= 2 * kBatch * kDecays * sizeof(float), "decays fit in the query tile");
      f4 prod[NK][4];
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it) prod[kb][it] = f4{1.f, 1.f, 1.f, 1.f};
      for (int u0 = 0, half = 0; u0 < n_a; u0 += kBatch, half ^= 1) {
        f4 a[kBatch][NK][4];
#pragma unroll
        for (int v = 0; v < kBatch; ++v)
#pragma unroll
          for (int kb = 0; kb < NK; ++kb)
#pragma unroll
            for (int it = 0; it < 4; ++it)
              a[v][kb][it] =
                  slot_load(slots, slot_state_off((blk0 + min(u0 + v, n_a - 1)) * NK + kb, wave, it, lane));
        if (tid < kBatch * kDecays) {
          const int v = tid / kDecays, kb = tid % kDecays / kHead, row = tid % kHead;
          dlds[half * kBatch * kDecays + tid] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(
                         slots, slot_decay_off((blk0 + min(u0 + v, n_a - 1)) * NK + kb, row), 0, kNonTemporal));
        }
        lds_sync();
#pragma unroll
        for (int v = 0; v < kBatch; ++v)
          if (u0 + v < n_a)
#pragma unroll
            for (int kb = 0; kb < NK; ++kb)
#pragma unroll
              for (int it = 0; it < 4; ++it) {
                const f4 d = *reinterpret_cast<const f4 *>(
                    &dlds[(half * kBatch + v) * kDecays + kb * kHead + 16 * it + 4 * g]);
                S[kb][it] = d * S[kb][it] + a[v][kb][it];
                prod[kb][it] *= d;
              }
      }
      if (has_p) {  // the chain between blocks: this wait is its only step per block
        if (tid == 0 && !wait_flag(p.sync, fl, blk0 - 1, want)) s_fail = 1;
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < NK; ++kb)
#pragma unroll
          for (int it = 0; it < 4; ++it)
            S[kb][it] += prod[kb][it] * slot_load(slots, slot_state_off((blk0 - 1) * NK + kb, wave, it, lane));
      } else if (p.s0) {
        const UserState u = user_state(p, p.s0, bh, wave, lane);
#pragma unroll
        for (int kb = 0; kb < NK; ++kb)
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            f4 e;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              e[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   u.r, user_state_off(u, kHead * kb + 16 * it + 4 * g + r), 0, 0));
            S[kb][it] += prod[kb][it] * e;
          }
      }
      if (s_fail) {  // a wait gave up: poison this segment and everything after it
#pragma unroll
        for (int kb = 0; kb < NK; ++kb)
#pragma unroll
          for (int it = 0; it < 4; ++it)
            S[kb][it] = f4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      }
    }

    // 4. the state after the segment: the next block's entering term, or s_final
    if (blk_last && has_next) {
      f4 after[NK][4];
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it)
          after[kb][it] =
              L[kb][it] + *reinterpret_cast<const f4 *>(&segdec[kb * kHead + 16 * it + 4 * g]) * S[kb][it];
      publish<false, NK>(p, slots, bh, seg, tid, after, sdec, want);
    }
    if (p.s_final && !has_next) {
      const UserState u = user_state(p, p.s_final, bh, wave, lane);
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const f4 after =
              L[kb][it] + *reinterpret_cast<const f4 *>(&segdec[kb * kHead + 16 * it + 4 * g]) * S[kb][it];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(after[r]), u.r,
                                                  user_state_off(u, kHead * kb + 16 * it + 4 * g + r), 0, 0);
        }
    }

    // 5. add each chunk's share of S_prev and store (16-bit operands: S_prev
    // scaled as in outputs(); the decays Dcum <= 1 only shrink it further)
    const uint32_t col = val_col<Io>(sq, 16 * wave + 4 * g);
    constexpr int LD = OpT<Op>::LD;
    constexpr bool kScaled = sizeof(Op) == 2;
    float unscale[NK], scale[NK];
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      unscale[kb] = 1.f;
      scale[kb] = kScaled && have_prev ? state_scale(S[kb], unscale[kb]) : 1.f;
    }
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
      if (c0 + j >= c1) break;
      if (have_prev) {
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) {  // each key block's share, scaled on its own
          const int qslot = j * NK + kb;
          op8<Op> sf[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f4 d0 = *reinterpret_cast<const f4 *>(&sm.dcum[qslot][32 * h + 4 * g]) * scale[kb];
            const f4 d1 = *reinterpret_cast<const f4 *>(&sm.dcum[qslot][32 * h + 16 + 4 * g]) * scale[kb];
            sf[h] = cat(to4<Op>(S[kb][2 * h] * d0), to4<Op>(S[kb][2 * h + 1] * d1));
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            f4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < 2; ++h)
              st = mma(sf[h], frag_row<Op>(&sm.qh[qslot][(16 * tt + l16) * LD + 32 * h + 4 * g]), st);
            keep[j][tt] += st * unscale[kb];
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        buf_store<Io>(sq.o, cell_at(sm.rowoff[j][16 * tt + l16], sq.vpitch, col), Io::pack(keep[j][tt]));
    }
    // the next ticket (its work-word increment returned long ago; taking the
    // next batch, when this one has run out, waits here, off the fold's path)
    if (tid == kThreads - 1) take_work(p, slot, next_word, s_work);
    __syncthreads();  // the next ticket is visible; the LDS tiles are free for the next walk
    bh = __builtin_amdgcn_readfirstlane(s_work[0]);
    seg = __builtin_amdgcn_readfirstlane(s_work[1]);
  }

  // Every workgroup counts itself out once it has found no work left; the last
  // one resets the work words and the batch counter and advances the epoch, so
  // the next call on this workspace (ordered after this kernel by the stream)
  // starts clean.  Each workgroup's last access to the work words returned a
  // value before it counts itself out, so none is still in flight.
  if (tid == 0) {
    if (__hip_atomic_fetch_add(p.sync + kSyncExitedWord, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        (int)gridDim.x - 1) {
      for (int x = 0; x < kXcdSlots; ++x)
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(p.sync + kSyncSlotWord + x * kSlotStride), 0ull,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.sync + kSyncNextBatchWord, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.sync + kSyncStartedWord, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.sync + kSyncExitedWord, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(reinterpret_cast<long long *>(p.sync + kSyncEpochWord), s_epoch + 1, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Launches `kernel`, bracketed by dispatch-timestamped events while profiling.
// GTR_GLA_SCAN=lanes (measurement and test aid, read at every launch):
// boundary scans of at most 64 steps run across lanes (gla_seg_scan_lanes)
// instead of one lane per element.  Measured on MI355X it is the slower of the
// two (4.7 -> 6.3 us per scan at 40x40 B1 H6, 4.8 -> 7.5 us at 128x128 B1 H16),
// so it is off by default.
bool scan_across_lanes() {
  const char *e = std::getenv("GTR_GLA_SCAN");
  return e && e[0] == 'l';
}

template <typename K, typename... Args>
void launch(int id, K kernel, unsigned blocks, hipStream_t stream, Args... args) {
  hipEvent_t t0, t1;
  if (profile_events(id, stream, &t0, &t1))
    hipExtLaunchKernelGGL(kernel, dim3(blocks), dim3(kThreads), 0, stream, t0, t1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kThreads), 0, stream, args...);
}

template <class Io, typename Op, int NK>
int launch_typed(const LaunchArgs &a) {
  Params p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.out = a.out;
  p.bh_count = a.bh; p.n_tok = a.n_tok; p.gh = a.grid_h; p.gw = a.grid_w; p.dir = a.direction;
  p.dk = a.d_k; p.dv = a.d_v; p.nvb = a.nvb;
  p.rcp_gh = 1.0f / (float)a.grid_h;
  p.n_chunk = a.n_chunk; p.seg_len = a.seg_len; p.n_seg = a.n_seg; p.n_seg_grid = a.n_seg;
  p.agg = a.agg; p.agg_dec = a.agg_dec; p.s0 = a.s0; p.s_final = a.s_final;
  p.flags = a.flags; p.sync = a.sync;
  p.prev_seq = a.n_seg;
  p.prev_step = 1;
  const unsigned n_blocks = (unsigned)(a.bh * a.n_seg);
  // fp32 operands on 16-bit I/O serve only the backward's state passes: no
  // output or one-launch kernels are built for them
  constexpr bool kStatesOnly = sizeof(typename Io::T) == 2 && sizeof(Op) == 4;
  if constexpr (kStatesOnly) {
    if (a.fused || a.outputs_only || !a.states_only) return (int)hipErrorInvalidValue;
  }
  if (a.fused) {
    if constexpr (kStatesOnly || Io::kLagGates) {
      return (int)hipErrorInvalidValue;
    } else {
      p.fold_block = a.fold_block;
      p.batch = a.batch;
      p.n_batch = (a.bh + a.batch - 1) / a.batch;
      p.n_pre = min(p.n_batch, min(a.xcds, kXcdSlots));
      const unsigned grid = (unsigned)a.grid;
      // fp32 operands with two key blocks keep at most two chunks (three
      // would need 184 KB of LDS); the planner caps the segment length
      constexpr int kMaxSeg = sizeof(Op) == 4 && NK == 2 ? 2 : kMaxFusedChunks;
      if (a.seg_len <= 1)
        launch(kKernelFused, gla_fused<Io, Op, 1, NK>, grid, a.stream, p);
      else if (a.seg_len == 2)
        launch(kKernelFused, gla_fused<Io, Op, 2, NK>, grid, a.stream, p);
      else if constexpr (kMaxSeg >= 3) {
        if (a.seg_len == 3)
          launch(kKernelFused, gla_fused<Io, Op, 3, NK>, grid, a.stream, p);
        else
          return (int)hipErrorInvalidValue;  // the planner caps fused segments at kMaxFusedChunks
      } else {
        return (int)hipErrorInvalidValue;
      }
      return (int)hipGetLastError();
    }
  }
  const bool need_scan =
      a.n_seg > 1 || a.s0 != nullptr || a.s_final != nullptr || a.states_only || a.want_prev;
  if (a.outputs_only) {
    p.prev = a.prev;
    if (a.prev_per_chunk) {
      p.prev_seq = a.n_chunk;
      p.prev_step = a.seg_len;
    }
  } else if (need_scan) {
    const int n_state_seg = a.s_final ? a.n_seg : a.n_seg - 1;
    if (n_state_seg > 0) {
      Params ps = p;
      ps.n_seg_grid = n_state_seg;
      launch(kKernelSegState, gla_seg_state<Io, Op, NK>, (unsigned)(a.bh * n_state_seg), a.stream, ps);
    }
    p.prev = a.prev;
    const int steps = a.s_final ? a.n_seg : a.n_seg - 1;
    int P = 1;
    while (P < steps) P <<= 1;
    const long lanes = (long)a.bh * NK * (kStateElems / 16) * P;
    if (steps <= 64 && lanes / kThreads < (1L << 30) && scan_across_lanes()) {
      launch(kKernelSegScan, gla_seg_scan_lanes<NK>, (unsigned)((lanes + kThreads - 1) / kThreads), a.stream, p);
    } else {
      const long threads = (long)a.bh * NK * kStateElems;
      launch(kKernelSegScan, gla_seg_scan<NK>, (unsigned)((threads + kThreads - 1) / kThreads), a.stream, p);
    }
  }
  if (a.states_only) return (int)hipGetLastError();
  if constexpr (!kStatesOnly) launch(kKernelSegOut, gla_seg_out<Io, Op, NK>, n_blocks, a.stream, p);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------ backward pass
//
// Gradients of the recurrence (chain rule through S_t = diag(alpha_t) S_{t-1}
// + k_t^T v_t, o_t = q_t S_t).  With G_t = dL/dS_t, which obeys the same kind
// of recurrence run backwards (G_t = q_t^T dout_t + diag(alpha_{t+1}) G_{t+1}):
//   dq_t = S_t dout_t^T,   dk_t = G_t v_t^T,   dv_t = k_t G_t,
//   dlog_gate_t = sum_{u >= t} (q_u dq_u - k_u dk_u)  (+ rowsum(dS_final S_final)).
// Read along the reversed scan, G is a forward state with keys q, values dout
// and each position's gate taken from the next position, so dv is a forward
// pass of this library and its state scan gives G at every chunk boundary.
// dq and dk contract a state over its value side instead of its key side;
// gla_bwd_dqk forms them per chunk from the boundary states.

// Transposed fragment (as frag_tr) of a row-major tile with row stride `stride`.
__device__ __forceinline__ h8 frag_tr_ld(const _Float16 *tile, int stride, int r0, int c0, int lane) {
  const int src = lane & 15, g = lane >> 4;
  const int row = r0 + 4 * g + (src >> 2), col = c0 + 4 * (src & 3);
  auto tr = [&](int r) {
    lds_s4 *ptr = (lds_s4 *)((lds_h *)tile + r * stride + col);
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(ptr));
  };
  return cat(tr(row), tr(row + 16));
}
__device__ __forceinline__ f8 frag_tr_ld(const float *tile, int stride, int r0, int c0, int lane) {
  const int g = lane >> 4, col = c0 + (lane & 15);
  f8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = tile[(r0 + 4 * g + e) * stride + col];
    f[4 + e] = tile[(r0 + 16 + 4 * g + e) * stride + col];
  }
  return f;
}

// Per-dim factor 2^(E_start(a) - E_end(b)) between key sub-block b and query
// sub-block a > b (1 for adjacent blocks).
template <typename Op, int NQ>
__device__ __forceinline__ float block_factor(const Smem<Op, NQ> &sm, int a, int b, int i) {
  if (b == a - 1) return 1.f;
  const int idx = (a == 2) ? 0 : (b == 0 ? 1 : 2);
  return (float)sm.cv[idx * kHead + i];
}

// One workgroup per chunk.  The forward chunk preparation runs with the query
// set to one, which leaves in LDS exactly the factors needed here:
//   qs = 2^(E_tau - E_start(a))       (per token and dim, <= 1)
//   ks = kop 2^(E_end(b) - E_sigma)   (keys referenced to their sub-block end)
//   hv, cv, tot                       (midpoint and block-pair factors)
//   vv = a                            (the score query rows)
// Wave w owns the 16 tokens of sub-block a = w and all 64 dims.  It forms its
// transposed score tiles P^T = b a^T against key blocks b <= a on MFMA
// (sigma < tau on the diagonal tile) and keeps them in registers, where they
// already are the B operand of the next contraction; then, per 16-dim tile,
//   out^T = 2^(E_tau - E_start(a)) (S 2^E_start(a) a^T + sum_{b<a} (ks c_ab)^T P^T
//           + hv (ks hv)^T P_aa^T) + P[tau][tau] kop_tau,
// every MFMA operand factor <= 1 except the diagonal midpoint factors (<= 2^8);
// a diagonal sub-block whose gate range is too wide for that is summed exactly
// in fp32 (its score tile goes through LDS for that).  `off` receives out
// without its self term (sigma = tau) in fp32: the gate gradient sums
// q dq - k dk, where the self terms of dq and dk are equal and cancel, so
// leaving them out keeps their rounding out of it.  kX (the dk pass, kop = q):
// `off` receives instead the gate-gradient term q dq - k dk of each position
// and dim, with dq from `pair` (the dq pass's `off`) and k from `kx`, so the
// gate kernel reads one array instead of four, and `tot` the chunk's sum of
// that term per dim (this pass's chunks, along the reversed scan), which the
// gate kernel's running sums start from.  With the scores in
// registers the kernel needs 77 KB of LDS with fp32 operands: two workgroups
// per CU.  For 16-bit I/O the scores' operands a and b are inputs, exact in
// fp16, so those tiles run as fp16 MFMAs (exact products, fp32 sums): the
// same results for an eighth of the instructions.
// Value blocks of a backward pass over d_v > 64: the result sums over them, so
// the first block's pass leaves its sums in fp32 (accf: with the self term,
// acco: without) and the last adds its own and writes out and off; a single
// block writes them directly.
enum : int { kVSingle = 0, kVFirst = 1, kVLast = 2 };

// Sum of x over each 16-lane row of a wave, in every lane of the row (DPP
// rotations by 8, 4, 2 and 1 lanes within the row).
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}

template <class Io, typename Op, bool kX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gla_bwd_dqk(Params p, void *out, float *off,
                                                                                           const float *pair,
                                                                                           const void *kx, float *tot) {
  using T = typename Io::T;
  constexpr int LD = OpT<Op>::LD;
  __shared__ Smem<Op, -1> sm;
  __shared__ __attribute__((aligned(16))) Op bs[kChunk * LD];  // score keys b [sigma][j], then kop [tau][i]
  __shared__ float self_score[kChunk];                         // P [tau][tau]
  __shared__ float dtile[4][16 * 16];                          // diagonal P^T [sigma][tau] of each sub-block
  __shared__ float xsum[kX ? 4 : 1][kHead];                    // kX: each wave's sum of the term per dim
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int seq = blockIdx.x / p.n_chunk, c = blockIdx.x - seq * p.n_chunk;
  const int a = wave;  // this wave's token sub-block
  const Seq sq = seq_of<Io>(p, seq * p.nvb + p.vb);  // k: kop, v: a, g: gates, o: b (read only); value block vb
  const int kp = p.kpitch ? p.kpitch : p.dk;  // out and kx rows: kp elements, this slice from kcol
  const auto orsrc = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<T *>(out) + (size_t)seq * p.n_tok * kp + p.kcol, (short)0,
      (int)((uint32_t)p.n_tok * (uint32_t)kp * sizeof(T) - (uint32_t)p.kcol * sizeof(T)), 0x00020000);

  // rows i = 16t + l16 of the state entering the chunk, for the four 16-dim
  // tiles t, at the k-slots of an MFMA operand (register-order workspace layout)
  float srow[4][16];
  {
    const float *st =
        p.prev + ((((size_t)seq * p.nvb + p.vb) * p.n_chunk + c) * p.prev_nk + p.prev_kb) * kStateElems;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 16 * t + l16;
      const int x = 4 * (i >> 4) + (i & 3), lo = 16 * ((i & 15) >> 2);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 * kb + (e < 4 ? 4 * g4 + e : 16 + 4 * g4 + e - 4);
          srow[t][8 * kb + e] = st[(j >> 4) * 1024 + x * 64 + lo + (j & 15)];
        }
    }
  }
  Rows<Io> x;
  load_chunk<Io, false, true>(sq, c, 0, wave, lane, x);
  typename Io::Raw brow[4];
  {
    const uint32_t vc = val_col<Io>(sq, 4 * l16);
#pragma unroll
    for (int r = 0; r < 4; ++r) brow[r] = buf_load<Io>(sq.o, cell_at(x.off[r], sq.vpitch, vc));
  }
  const typename Io::Raw one = Io::pack(f4{1.f, 1.f, 1.f, 1.f});
#pragma unroll
  for (int r = 0; r < 4; ++r) x.q[r] = one;
  op4<Op> qs[4], ks[4];
  prep_local<Io, Op, true, -1>(sm, x, wave, lane, 0, qs, ks, true);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<op4<Op> *>(&bs[(16 * wave + 4 * g4 + r) * LD + 4 * l16]) = ToOp<Op, Io>::cvt(brow[r]);
  lds_sync();
  prep_chunk<Io, Op, true, -1>(sm, qs, ks, wave, lane, 0);
  lds_sync();

  const int tau = 16 * a + l16;
  const uint32_t cell = sm.rowoff[0][tau];
  // kX: dq and k at this lane's position and result dims, for all four tiles;
  // issued now (clamped to valid rows and dims, results past them are not
  // stored) so that they arrive while the MFMAs run
  f4 xdq[4], xkk[4];
  if constexpr (kX) {
    const size_t prow = (size_t)seq * p.n_tok + (cell == kNoRow ? 0u : cell);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int d = min(16 * t + 4 * g4, p.dk - 4);
      xdq[t] = *reinterpret_cast<const f4 *>(pair + prow * p.dk + d);
      const T *kr = static_cast<const T *>(kx) + prow * kp + p.kcol + d;
      xkk[t] = f4{elem<Io>(kr), elem<Io>(kr + 1), elem<Io>(kr + 2), elem<Io>(kr + 3)};
    }
  }

  // P^T tiles of sub-block a: rows sigma = 16b + 4 g4 + r, column tau = 16a + l16
  // (zero for b > a and, on the diagonal tile, for sigma >= tau), packed in
  // pairs as B operands over sigma in [32 kb, 32 kb + 32)
  op8<Op> pf[2];
  {
    f4 tile[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      if (b <= a) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const op8<Op> fb = frag_row<Op>(&bs[(16 * b + l16) * LD + 32 * kb + 4 * g4]);
          const op8<Op> fa = frag_row<Op>(&sm.vv[(16 * a + l16) * OpT<Op>::LDT + 32 * kb + 4 * g4]);
          if constexpr (sizeof(T) == 2 && sizeof(Op) == 4)  // 16-bit inputs are exact in fp16:
            acc = mma(__builtin_convertvector(fb, h8), __builtin_convertvector(fa, h8), acc);  // same sums
          else
            acc = mma(fb, fa, acc);
        }
      }
      if (b == a) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sl = 4 * g4 + r;  // sigma within the sub-block; tau within it is l16
          if (sl == l16) self_score[16 * a + l16] = acc[r];
          if (sl >= l16) acc[r] = 0.f;
          dtile[a][sl * 16 + l16] = acc[r];
        }
      }
      tile[b] = acc;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) pf[kb] = cat(to4<Op>(tile[2 * kb]), to4<Op>(tile[2 * kb + 1]));
  }
  lds_sync();
  // every wave has read the score keys: the tile now takes kop itself (this
  // barrier also publishes the self scores and diagonal tiles)
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<op4<Op> *>(&bs[(16 * wave + 4 * g4 + r) * LD + 4 * l16]) = ToOp<Op, Io>::cvt(x.k[r]);
  lds_sync();

  const bool exact = !__all(sm.tot[a * kHead + lane] >= OpT<Op>::kDiagMin);
  const bool live = c * kChunk + tau < p.n_tok;
  const float self = self_score[tau];
  // the P^T pair holding the own sub-block (a is uniform across the wave, so
  // this is a select, not an indexed register access in the loop below)
  const op8<Op> pown = a >= 2 ? pf[1] : pf[0];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i_row = 16 * t + l16;  // this lane's operand row
    float es = 1.f;                  // 2^E_start(a) for dim i_row
    for (int a2 = 0; a2 < a; ++a2) es *= sm.tot[a2 * kHead + i_row];
    f4 acc = {0.f, 0.f, 0.f, 0.f}, accd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {  // state entering the chunk
      op8<Op> sf;
#pragma unroll
      for (int e = 0; e < 8; ++e) sf[e] = (Op)(srow[t][8 * kb + e] * es);
      acc = mma(sf, frag_row<Op>(&sm.vv[tau * OpT<Op>::LDT + 32 * kb + 4 * g4]), acc);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {  // earlier sub-blocks
      if (2 * kb >= a) break;
      const float f0 = block_factor(sm, a, 2 * kb, i_row);
      const float f1 = 2 * kb + 1 < a ? block_factor(sm, a, 2 * kb + 1, i_row) : 0.f;
      op8<Op> xk = frag_tr_ld(sm.ks, LD, 32 * kb, 16 * t, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) xk[e] = (Op)((float)xk[e] * (e < 4 ? f0 : f1));
      acc = mma(xk, pf[kb], acc);
    }
    if (!exact) {  // own sub-block (pair a / 2), referenced at its midpoint
      const int kb = a >> 1;
      const float h = (float)sm.hv[a * kHead + i_row];
      op8<Op> xk = frag_tr_ld(sm.ks, LD, 32 * kb, 16 * t, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) xk[e] = (Op)(((e < 4) == ((a & 1) == 0)) ? (float)xk[e] * h : 0.f);
      accd = mma(xk, pown, accd);
    }
    const int d0 = 16 * t + 4 * g4;  // dims of this lane's results
    f4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float f1 = (float)sm.qs[tau * LD + d0 + r];
      o[r] = f1 * (acc[r] + (float)sm.hv[a * kHead + d0 + r] * accd[r]);
    }
    if (exact && live) {  // exact fp32 sum over the earlier tokens of the own sub-block
      constexpr uint32_t elt = sizeof(T);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = d0 + r;
        if (i >= p.dk) continue;
        float ex = 0.f;
        float run = key_elem<Io>(sq.g, cell_at(gate_cell<Io>(sq, c * kChunk + tau), sq.kpitch, i * elt)) * kLog2e;
        for (int s2 = tau - 1; s2 >= 16 * a; --s2) {
          const uint32_t cs = sm.rowoff[0][s2];
          // 2^(E_tau - E_s2): the log2 gates of tokens s2+1 .. tau
          ex += dtile[a][(s2 - 16 * a) * 16 + l16] * key_elem<Io>(sq.k, cs * sq.kpitch + i * elt) * fast_exp2(run);
          run += key_elem<Io>(sq.g, cell_at(gate_cell<Io>(sq, c * kChunk + s2), sq.kpitch, i * elt)) * kLog2e;
        }
        o[r] = (float)sm.qs[tau * LD + i] * acc[r] + ex;
      }
    }
    f4 full;
#pragma unroll
    for (int r = 0; r < 4; ++r) full[r] = o[r] + self * (float)bs[tau * LD + d0 + r];
    const bool here = cell != kNoRow && d0 < p.dk;
    const size_t at = ((size_t)seq * p.n_tok + (cell == kNoRow ? 0u : cell)) * p.dk + d0;
    if (p.vmode == kVFirst) {  // this value block's sums, for the last block to add to
      if (here) {
        *reinterpret_cast<f4 *>(p.accf + at) = full;
        *reinterpret_cast<f4 *>(p.acco + at) = o;
      }
      continue;
    }
    if (p.vmode == kVLast && here) {
      full += *reinterpret_cast<const f4 *>(p.accf + at);
      o += *reinterpret_cast<const f4 *>(p.acco + at);
    }
    f4 w = o;
    if constexpr (kX) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w[r] = (float)bs[tau * LD + d0 + r] * xdq[t][r] - xkk[t][r] * o[r];
        // the wave's 16 tokens of dim d0 + r (missing tokens and dims count 0)
        const float sr = row_sum16(here ? w[r] : 0.f);
        if (l16 == 0) xsum[a][d0 + r] = sr;
      }
    }
    buf_store<Io>(orsrc, cell_at(cell, sq.kpitch, key_col<Io>(sq, d0)), Io::pack(full));
    if (here) *reinterpret_cast<f4 *>(off + at) = w;
  }
  if constexpr (kX) {
    if (p.vmode != kVFirst) {  // uniform: the first of two value blocks writes no term
      lds_sync();
      if (tid < kHead)
        tot[((size_t)seq * p.n_chunk + c) * kHead + tid] = xsum[0][tid] + xsum[1][tid] + xsum[2][tid] + xsum[3][tid];
    }
  }
}

// Grid cell of scan position t (plain arguments; see token_cell).
__device__ __forceinline__ uint32_t scan_cell(int t, int n_tok, int gh, int gw, int dir, float rcp_gh) {
  const int p = (dir & 1) ? n_tok - 1 - t : t;
  if (!(dir & 2)) return (uint32_t)p;
  int row, col;
  col_major_pos(p, gh, rcp_gh, row, col);
  return (uint32_t)(row * gw + col);
}


// x_t (the gate-gradient term q_t dq_t - k_t dk_t, fp32) for the 64 tokens of
// one chunk: thread (r, i) of 256 takes tokens 16r .. 16r+15 of dim i, so each
// wave reads whole rows; tokens past the end give 0.  The 16 loads are
// unconditional (a masked position reads the sequence's first element), so no
// branch holds one back until the previous one has returned.
__device__ __forceinline__ void dgate_terms(const float *xs, size_t base, int c, int r, int i, int n_tok, int gh,
                                            int gw, int dir, float rcp_gh, int d_k, float *x) {
  float v[16];
  bool ok[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int t = c * kChunk + 16 * r + u;
    ok[u] = t < n_tok && i < d_k;
    v[u] = xs[ok[u] ? base + (size_t)scan_cell(t, n_tok, gh, gw, dir, rcp_gh) * d_k + i : base];
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) x[u] = ok[u] ? v[u] : 0.f;
}

// dlog_gate_t = sum over the positions u from t to the end of the forward
// scan of x_u (plus rowsum(dS_final S_final)).  Read along the reversed scan
// (`dir`), the one the dk pass's chunks follow, that is a running sum from
// its start: the earlier chunks' totals (written by the dk pass), then the
// sum inside the chunk, quarter by quarter.
// d_k dims of xs (rows of d_k); dg rows and the states' row blocks hold kp
// dims (dg and the state pointers start at the slice's first dim).
template <class Io>
__global__ __launch_bounds__(kThreads) void gla_dgate_apply(const float *xs, const float *ds_final,
                                                            const float *s_final,
                                                            const float *totals, typename Io::T *dg, int n_tok,
                                                            int gh, int gw, int dir, float rcp_gh, int d_k,
                                                            int d_v, int n_chunk, int kp) {
  __shared__ float part[4][kHead];
  const int seq = blockIdx.x / n_chunk, c = blockIdx.x - seq * n_chunk;
  const int r = threadIdx.x >> 6, i = threadIdx.x & 63;
  const size_t base = (size_t)seq * n_tok * d_k;
  float x[16];
  dgate_terms(xs, base, c, r, i, n_tok, gh, gw, dir, rcp_gh, d_k, x);
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) sum += x[u];
  part[r][i] = sum;
  // what precedes this quarter: the earlier quarters, the earlier chunks, the final-state term
  // (batches of independent loads: a clamped index, then a masked add)
  float run = 0.f;
  if (i < d_k) {
    if (r == 0 && ds_final && s_final) {  // rows of d_v floats, d_v a multiple of 4
      const f4 *a = reinterpret_cast<const f4 *>(ds_final + ((size_t)seq * kp + i) * d_v);
      const f4 *b = reinterpret_cast<const f4 *>(s_final + ((size_t)seq * kp + i) * d_v);
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < d_v / 4; j0 += 4) {
        f4 av[4], bv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = min(j0 + e, d_v / 4 - 1);
          av[e] = a[j];
          bv[e] = b[j];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + e < d_v / 4) acc += av[e] * bv[e];
      }
      run = acc.x + acc.y + acc.z + acc.w;
    }
    const float *tot = totals + (size_t)seq * n_chunk * kHead + i;
    constexpr int kBatch = 8;
    for (int c2 = r; c2 < c; c2 += 4 * kBatch) {
      float tv[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) tv[e] = tot[(size_t)min(c2 + 4 * e, n_chunk - 1) * kHead];
#pragma unroll
      for (int e = 0; e < kBatch; ++e)
        if (c2 + 4 * e < c) run += tv[e];
    }
  }
  __syncthreads();
  float earlier = 0.f;
  for (int r2 = 0; r2 < r; ++r2) earlier += part[r2][i];
  __syncthreads();
  part[r][i] = run;  // this thread's share of the earlier chunks and the final-state term
  __syncthreads();
  run = earlier + part[0][i] + part[1][i] + part[2][i] + part[3][i];
  if (i >= d_k) return;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int t = c * kChunk + 16 * r + u;
    run += x[u];
    if (t < n_tok)
      dg[((size_t)seq * n_tok + scan_cell(t, n_tok, gh, gw, dir, rcp_gh)) * kp + i] = Io::narrow(run);
  }
}


}  // namespace

namespace {
__global__ __launch_bounds__(kThreads) void gla_state_copy(const float *s0, float *s_final, long long n) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) s_final[i] = s0 ? s0[i] : 0.f;
}
}  // namespace

int launch_state_copy(const float *s0, float *s_final, long long n, hipStream_t stream) {
  hipLaunchKernelGGL(gla_state_copy, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, s0, s_final, n);
  return (int)hipGetLastError();
}

// Working memory of gtr_gla_fwd_static: a fixed array in this library's device
// code, one copy per device, held until the process ends.  Host code must not
// use the name `scratch` as an address (on the host it is only a stand-in for
// the symbol): static_scratch() gives each device's own address.
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

int static_scratch(int device, void **ptr) {
  static std::mutex m;
  static std::map<int, void *> addr;
  std::lock_guard<std::mutex> lock(m);
  auto it = addr.find(device);
  if (it == addr.end()) {
    void *p = nullptr;  // queried with `device` current (the caller's current device)
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
    }
    it = addr.emplace(device, p).first;
  }
  *ptr = it->second;
  return (int)hipSuccess;
}

int launch_gla(const LaunchArgs &a) {
  const bool two = a.nk == 2;
  if (a.lag_gates) {  // the backward pass's reversed scan: three launches
    if (a.fused) return (int)hipErrorInvalidValue;
    switch (a.dtype) {
      case 0: return two ? launch_typed<Lagged<IoF32>, float, 2>(a) : launch_typed<Lagged<IoF32>, float, 1>(a);
      case 1:
        if (a.fp32_operands)
          return two ? launch_typed<Lagged<IoF16>, float, 2>(a) : launch_typed<Lagged<IoF16>, float, 1>(a);
        return two ? launch_typed<Lagged<IoF16>, _Float16, 2>(a) : launch_typed<Lagged<IoF16>, _Float16, 1>(a);
      case 2:
        if (a.fp32_operands)
          return two ? launch_typed<Lagged<IoBF16>, float, 2>(a) : launch_typed<Lagged<IoBF16>, float, 1>(a);
        return two ? launch_typed<Lagged<IoBF16>, _Float16, 2>(a) : launch_typed<Lagged<IoBF16>, _Float16, 1>(a);
      default: return (int)hipErrorInvalidValue;
    }
  }
  if (a.fp32_operands && !a.fused) {
    switch (a.dtype) {
      case 1: return two ? launch_typed<IoF16, float, 2>(a) : launch_typed<IoF16, float, 1>(a);
      case 2: return two ? launch_typed<IoBF16, float, 2>(a) : launch_typed<IoBF16, float, 1>(a);
      default: break;
    }
  }
  switch (a.dtype) {
    case 0: return two ? launch_typed<IoF32, float, 2>(a) : launch_typed<IoF32, float, 1>(a);
    case 1: return two ? launch_typed<IoF16, _Float16, 2>(a) : launch_typed<IoF16, _Float16, 1>(a);
    case 2: return two ? launch_typed<IoBF16, _Float16, 2>(a) : launch_typed<IoBF16, _Float16, 1>(a);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace gtr


// ------------------------------------------------------- backward launchers
namespace gtr {
namespace {

// ds0 = diag(alpha_0) G_0: one thread per state element.
// d_k dims per sequence (a slice when kp > d_k: g rows and the states' row
// blocks hold kp dims, and the pointers start at the slice's first dim).
template <class Io>
__global__ __launch_bounds__(kThreads) void gla_ds0(const typename Io::T *g, const float *g0, float *ds0,
                                                    int n_tok, int gh, int gw, int dir, float rcp_gh,
                                                    int d_k, int d_v, long long n, int kp) {
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= n) return;
  const long long per_seq = (long long)d_k * d_v;
  const long long seq = gid / per_seq;
  const int i = (int)((gid - seq * per_seq) / d_v), j = (int)(gid - seq * per_seq - (long long)i * d_v);
  const size_t at = ((size_t)seq * n_tok + scan_cell(0, n_tok, gh, gw, dir, rcp_gh)) * kp + i;
  const size_t e = ((size_t)seq * kp + i) * d_v + j;
  ds0[e] = expf(elem<Io>(g + at)) * g0[e];
}

template <class Io, typename Op>
int launch_bwd_typed(const BwdArgs &a) {
  Params p{};
  p.q = a.kop; p.k = a.kop; p.v = a.aop; p.g = a.g; p.out = const_cast<void *>(a.bop);
  p.bh_count = a.bh; p.n_tok = a.n_tok; p.gh = a.grid_h; p.gw = a.grid_w; p.dir = a.direction;
  p.rcp_gh = 1.0f / (float)a.grid_h;
  p.dk = a.d_k; p.dv = a.d_v;
  p.kpitch = a.kpitch; p.kcol = a.kcol;
  p.nvb = a.nvb > 0 ? a.nvb : 1; p.vb = a.vb; p.vmode = a.vmode; p.accf = a.accf; p.acco = a.acco;
  p.n_chunk = a.n_chunk; p.prev = a.prev;
  p.prev_nk = a.prev_nk > 0 ? a.prev_nk : 1;
  p.prev_kb = a.prev_kb;
  // the dk pass (which forms the gate-gradient term from `pair`) runs along
  // the reversed scan with lagged gates; the dq pass along the forward scan
  if (a.pair && a.lag_gates && a.totals)
    launch(kKernelBwdDqk, gla_bwd_dqk<Lagged<Io>, Op, true>, (unsigned)(a.bh * a.n_chunk), a.stream, p, a.out,
           a.off, a.pair, a.kx, a.totals);
  else if (!a.pair && !a.lag_gates)
    launch(kKernelBwdDqk, gla_bwd_dqk<Io, Op, false>, (unsigned)(a.bh * a.n_chunk), a.stream, p, a.out, a.off,
           a.pair, a.kx, a.totals);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace

// fp32 MFMA operands for every I/O type: the gate gradient sums dq and dk terms
// whose pairs cancel between the two kernels, so their operands must not carry
// 16-bit rounding (or 16-bit underflow of strongly decayed factors).
int launch_gla_bwd_dqk(const BwdArgs &a) {
  switch (a.dtype) {
    case 0: return launch_bwd_typed<IoF32, float>(a);
    case 1: return launch_bwd_typed<IoF16, float>(a);
    case 2: return launch_bwd_typed<IoBF16, float>(a);
    default: return (int)hipErrorInvalidValue;
  }
}

namespace {
template <class Io>
int launch_dgate_typed(const float *xs, const float *ds_final, const float *s_final, const float *totals, void *dg,
                       int bh, int grid_h, int grid_w, int d_k, int d_v, int n_chunk, int direction, int kp,
                       hipStream_t stream) {
  using T = typename Io::T;
  const int n_tok = grid_h * grid_w;
  const float rcp = 1.0f / (float)grid_h;
  const dim3 grid((unsigned)(bh * n_chunk));
  // the chunk totals come from the dk pass, whose chunks follow the reversed scan
  launch(kKernelBwdDgate, gla_dgate_apply<Io>, grid.x, stream, xs, ds_final, s_final,
         totals, static_cast<T *>(dg), n_tok, grid_h, grid_w, direction ^ 1, rcp,
         d_k, d_v, n_chunk, kp);
  return (int)hipGetLastError();
}

template <class Io>
int launch_ds0_typed(const void *g, const float *g0, float *ds0, int bh, int grid_h, int grid_w, int d_k,
                     int d_v, int direction, int kp, hipStream_t stream) {
  const long long n = (long long)bh * d_k * d_v;
  launch(kKernelBwdDs0, gla_ds0<Io>, (unsigned)((n + kThreads - 1) / kThreads), stream,
         static_cast<const typename Io::T *>(g), g0, ds0, grid_h * grid_w, grid_h, grid_w, direction,
         1.0f / (float)grid_h, d_k, d_v, n, kp);
  return (int)hipGetLastError();
}
}  // namespace

int launch_dgate(const float *x, const float *ds_final, const float *s_final, const float *totals, void *dg,
                 int bh, int grid_h, int grid_w, int d_k, int d_v, int n_chunk, int direction, int dtype,
                 int kp, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_dgate_typed<IoF32>(x, ds_final, s_final, totals, dg, bh, grid_h, grid_w, d_k, d_v, n_chunk, direction, kp, stream);
    case 1: return launch_dgate_typed<IoF16>(x, ds_final, s_final, totals, dg, bh, grid_h, grid_w, d_k, d_v, n_chunk, direction, kp, stream);
    case 2: return launch_dgate_typed<IoBF16>(x, ds_final, s_final, totals, dg, bh, grid_h, grid_w, d_k, d_v, n_chunk, direction, kp, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

int launch_ds0(const void *g, const float *g0, float *ds0, int bh, int grid_h, int grid_w, int d_k, int d_v,
               int direction, int dtype, int kp, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_ds0_typed<IoF32>(g, g0, ds0, bh, grid_h, grid_w, d_k, d_v, direction, kp, stream);
    case 1: return launch_ds0_typed<IoF16>(g, g0, ds0, bh, grid_h, grid_w, d_k, d_v, direction, kp, stream);
    case 2: return launch_ds0_typed<IoBF16>(g, g0, ds0, bh, grid_h, grid_w, d_k, d_v, direction, kp, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace gtr
