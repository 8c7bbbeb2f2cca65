// Internal interface between the host entry points (gla_api.cpp) and the
// kernel launchers (gla_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace gtr {

constexpr int kChunk = 64;   // tokens per chunk (the pages' operator uses 64)
constexpr int kHead = 64;    // width of a key or value block (d_k, d_v <= 2 blocks)
constexpr int kStateElems = kHead * kHead;
constexpr int kMaxFusedChunks = 3;  // chunks per segment of the one-launch path (outputs held in registers)
// One-launch path: segments are grouped in blocks of at most this many; each
// segment folds the aggregates of the earlier segments of its block.
constexpr int kMaxFoldBlock = 32;
constexpr int kSlotFloats = kStateElems + kHead;  // one segment's payload: a state and 64 decays

struct LaunchArgs {
  const void *q, *k, *v, *g;
  void *out;
  int bh;            // sequences: B*H*nvb (each head's value columns in 64-wide blocks)
  int d_k, d_v;      // head dims (multiples of 4, at most 128)
  int nk, nvb;       // 64-wide key blocks (1 or 2) and value blocks per head
  int grid_h, grid_w;
  int n_tok;         // grid_h*grid_w
  int direction;
  int dtype;         // GTR_DTYPE_*
  int n_chunk;       // ceil(n_tok / 64)
  int seg_len;       // chunks per segment
  int n_seg;         // ceil(n_chunk / seg_len)
  // workspace (float32), all in the register-order state layout
  float *agg;        // [seq][n_seg][nk][4096] segment state contributions
  float *agg_dec;    // [seq][n_seg][nk][64]   segment decay factor per key dim
  float *prev;       // [seq][n_seg][nk][4096] state entering each segment
  int *sync;         // fused path: header + per-XCD work words (zeroed at allocation)
  long long *flags;  // [bh][n_seg] fused path: payload-published flags (64-bit epochs), after the work words
  int fold_block;    // fused path: segments per fold block
  int batch;         // fused path: sequences an XCD claims at a time
  int grid;          // fused path: persistent workgroups
  int xcds;          // fused path: XCDs of the device (their L2s are not coherent with each other)
  const float *s0;   // user initial state, row-major [B*H][d_k][d_v], nullable
  float *s_final;    // user final state, row-major [B*H][d_k][d_v], nullable
  bool fused;        // one launch (gla_fused) instead of three
  bool states_only;  // split path without outputs: only the states entering each segment (prev)
  bool want_prev;    // split path: write prev for every segment even where the outputs need no scan
  bool fp32_operands;  // fp32 MFMA operands for 16-bit I/O too (backward pass, split path)
  bool outputs_only;   // split path: only the output kernel, entering each segment with prev as given
  bool lag_gates;      // scan position t takes the gate of position t-1, none at t = 0 (backward)
  bool prev_per_chunk; // outputs_only: prev holds the state entering every chunk ([seq][n_chunk]);
                       // each segment enters with the entry of its first chunk
  hipStream_t stream;
};

// One launch of the backward chunk kernel (gla_bwd_dqk): for every 64-token
// chunk of every sequence, along `direction`,
//   out_tau = 2^E_tau * (S_prev a_tau^T) + sum_{sigma <= tau} (a_tau . b_sigma) kop_sigma * 2^(E_tau - E_sigma)
// with E the log2 cumulative gate from the chunk start (per d_k dim) and S_prev
// the state entering the chunk.  Used for dq (kop = k, a = dout, b = v, forward
// states) and dk (kop = q, a = v, b = dout, reversed scan, state gradients).
struct BwdArgs {
  const void *kop, *aop, *bop, *g;  // [bh][grid][d_k], [bh][grid][d_v] twice, [bh][grid][d_k]
  void *out;                        // [bh][grid][d_k]
  float *off;                       // [bh][grid][d_k] fp32: out without its self term (sigma = tau), or
                                    // with `pair` set, the gate-gradient term kop * pair - kx * that
  const float *pair;                // nullable [bh][grid][d_k] fp32: the other pass's `off` (dq)
  const void *kx;                   // with `pair`: [bh][grid][d_k] keys k
  float *totals;                    // with `pair`: [bh][n_chunk][64] fp32, each chunk's sum of the
                                    // gate-gradient term per dim (chunks along this pass's scan)
  const float *prev;                // [bh][n_chunk][prev_nk][4096] register order; key block prev_kb
  int prev_nk, prev_kb;             // (prev_nk 0 counts as 1)
  int bh, grid_h, grid_w, n_tok, direction, dtype, n_chunk, d_k, d_v;
  int kpitch, kcol;                 // d_k > 64: a slice of d_k dims from column kcol of rows of kpitch
                                    // elements (kop, g, kx, out); kpitch 0: rows of d_k
  int nvb, vb;                      // d_v > 64: value block vb of nvb (aop, bop columns and prev
                                    // entries [bh][nvb][n_chunk]...); nvb 0 counts as 1
  int vmode;                        // 0: one value block; 1: first of two (sums to accf, acco, no
                                    // out or off); 2: last (adds them, writes out and off)
  float *accf, *acco;               // [bh][grid][d_k] fp32, with nvb = 2
  bool lag_gates;                   // as in LaunchArgs
  hipStream_t stream;
};

// Synchronisation words of the one-launch path (32-bit words of one zeroed
// allocation): a header (64-bit epoch in words 0-1, error word, count of
// workgroups that found no work left, next batch to hand out, mask of XCDs
// that have begun their starting batch), one 64-bit work
// word per XCD on its own 128-byte line (XCC_ID has 4 bits: 16 lines), then
// one 64-bit flag per segment.  Their positions do not depend on the shape.
constexpr int kSyncHeader = 32;
constexpr int kSyncEpochWord = 0, kSyncErrorWord = 3, kSyncExitedWord = 4, kSyncNextBatchWord = 5,
              kSyncStartedWord = 6;
constexpr int kXcdSlots = 16;
constexpr int kSlotStride = 32;
constexpr int kSyncSlotWord = kSyncHeader;
constexpr int kSyncFlagWord = kSyncHeader + kXcdSlots * kSlotStride;

// Float workspace bytes for (sequences, n_seg, key blocks): agg, prev and agg_dec.
inline size_t workspace_bytes(size_t seqs, size_t n_seg, size_t nk) {
  return seqs * n_seg * nk * (2 * (size_t)kStateElems + kHead) * sizeof(float);
}
// Float workspace bytes of the one-launch path: one payload slot per segment
// and key block (aggregate or block prefix, and decays), none for a single
// segment.
inline size_t fused_workspace_bytes(size_t seqs, size_t n_seg, size_t nk) {
  return n_seg > 1 ? seqs * n_seg * nk * (size_t)kSlotFloats * sizeof(float) : 0;
}
// Synchronisation words for `n_flags` segment flags.
inline size_t sync_words(size_t n_flags) { return kSyncFlagWord + 2 * n_flags; }

// Host helpers shared by the entry points (defined in gla_api.cpp): record an
// error message for gtr_gla_last_error() and return `code`; clear it; check a
// device pointer against the current device and a byte count; whether pointer
// queries are switched off (GTR_GLA_SKIP_POINTER_CHECKS=1); whether `stream`
// is being captured.
int set_error(int code, const char *fmt, ...);
void clear_error();
int check_device_pointer(const void *p, size_t bytes, int device, const char *name);
bool pointer_checks_off();
bool stream_capturing(hipStream_t stream);

// A device buffer of at least `bytes`, cached per (owner, device, stream)
// (defined in gla_api.cpp).  A buffer that a larger call replaces is kept,
// not freed, until gtr_gla_release_workspaces(): a graph captured on that
// stream may still refer to it.  Growing is refused while `stream` is being
// captured (GTR_ERR_CAPTURE); a failed allocation gives GTR_ERR_ALLOC.
enum BufferOwner { kBufBackward = 1, kBufSwiglu = 2 };
int stream_buffer(int owner, int device, hipStream_t stream, size_t bytes, const char *what, void **out);

// Backward-pass launchers (hipError_t values).
int launch_gla_bwd_dqk(const BwdArgs &a);
// dlog_gate_t = sum_{u >= t} x_u + rowsum(ds_final * s_final) along `direction`, with
// x = q dq - k dk per position and dim (fp32 [bh][grid][d_k], dq and dk without their cancelling
// self terms, as the backward chunk kernel's dk pass writes it); totals: [bh][n_chunk][64] fp32,
// the sum of x over each chunk of the reversed scan (direction ^ 1), as the dk pass writes them.
// ds_final / s_final may be null.  dg rows and the states' row blocks hold kp >= d_k dims; dg,
// ds_final and s_final point at the first of the d_k dims computed.
int launch_dgate(const float *x, const float *ds_final, const float *s_final, const float *totals, void *dg,
                 int bh, int grid_h, int grid_w, int d_k, int d_v, int n_chunk, int direction, int dtype,
                 int kp, hipStream_t stream);
// ds0[i][j] = alpha_0[i] g0[i][j] (alpha of the first scan position), row-major [bh][kp][d_v], for
// d_k rows from where g, g0 and ds0 point (g rows hold kp dims).
int launch_ds0(const void *g, const float *g0, float *ds0, int bh, int grid_h, int grid_w, int d_k, int d_v,
               int direction, int dtype, int kp, hipStream_t stream);

// Chunks per segment of the three-launch path for `seqs` sequences of
// n_chunk chunks (defined in gla_api.cpp).
long long split_segment_length(long long seqs, int n_chunk);

// Enqueues the kernels for one call.  Returns a hipError_t value.
int launch_gla(const LaunchArgs &a);

// Size of the fixed device array gtr_gla_fwd_static takes its working memory
// from (GTR_GLA_STATIC_SCRATCH_BYTES), and that array's address on `device`,
// which must be the current device (queried once per device; hipError_t value).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
int static_scratch(int device, void **ptr);

// s_final[i] = s0 ? s0[i] : 0 for i < n (a call with no tokens).  Returns a hipError_t value.
int launch_state_copy(const float *s0, float *s_final, long long n, hipStream_t stream);

}  // namespace gtr
