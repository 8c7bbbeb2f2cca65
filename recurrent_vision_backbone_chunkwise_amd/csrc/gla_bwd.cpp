// Host entry point of the backward pass (gtr_gla_bwd in include/gtr_gla.h):
// validation, a per-(device, stream) workspace and the launch sequence.
//
// Gradients of S_t = diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t (the
// recurrence of the x-techcon article on GTR, section 架构 / Architecture):
//   1. the states entering every 64-token chunk (forward state and scan kernels);
//   2. dv, and the state gradients G entering every chunk of the reversed scan:
//      a forward pass along the reversed direction with queries k, keys q,
//      values dout and dS_final as its initial state, in which each position
//      takes the gate of the position before it along that scan (the kernels
//      read it in place);
//   3. dq and 4. dk with the backward chunk kernel;
//   5. dlog_gate = reverse running sum of q dq - k dk (+ rowsum(dS_final S_final)), from
//      dq and dk without their self terms, which cancel in it;
//   6. ds0 = diag(alpha_0) G_0.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gla_internal.h"
#include "gtr_gla.h"

namespace {

using gtr::set_error;

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

struct Layout {  // byte offsets into the workspace
  size_t fwd, rev, sfin, g0, totals, dq_off, dk_off, total;
};

Layout layout(long long bh, long long n_tok, int n_chunk, int d_k, int d_v) {
  Layout l{};
  const size_t scan = round256(gtr::workspace_bytes((size_t)bh, (size_t)n_chunk, 1));
  l.fwd = 0;
  l.rev = l.fwd + scan;
  l.sfin = l.rev + scan;
  l.g0 = l.sfin + round256((size_t)bh * d_k * d_v * sizeof(float));
  l.totals = l.g0 + round256((size_t)bh * d_k * d_v * sizeof(float));
  l.dq_off = l.totals + round256((size_t)bh * n_chunk * gtr::kHead * sizeof(float));
  l.dk_off = l.dq_off + round256((size_t)bh * n_tok * d_k * sizeof(float));
  l.total = l.dk_off + round256((size_t)bh * n_tok * d_k * sizeof(float));
  return l;
}

int launched(int err) {
  if (err != (int)hipSuccess)
    return set_error(GTR_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
  return GTR_OK;
}

}  // namespace

extern "C" {

int gtr_gla_bwd(const void *q, const void *k, const void *v, const void *log_gate, const void *dout,
                const float *s0, const float *ds_final, void *dq, void *dk, void *dv, void *dlog_gate,
                float *ds0, int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction,
                int dtype, hipStream_t stream) {
  gtr::clear_error();
  if (B < 0 || H < 0 || grid_h < 0 || grid_w < 0 || d_k <= 0 || d_v <= 0)
    return set_error(GTR_ERR_INVALID_ARG, "sizes must be >= 0 and head sizes > 0");
  if (direction < 0 || direction > 3) return set_error(GTR_ERR_INVALID_ARG, "direction %d not in 0..3", direction);
  if (dtype < 0 || dtype > 2) return set_error(GTR_ERR_INVALID_ARG, "dtype %d not in 0..2", dtype);
  if (d_k % 4 || d_v % 4 || d_k > gtr::kHead || d_v > gtr::kHead)
    return set_error(GTR_ERR_UNSUPPORTED, "backward: d_k=%d d_v=%d, head dims must be multiples of 4 up to 64",
                     d_k, d_v);
  const long long n_tok = (long long)grid_h * grid_w, bh = (long long)B * H;
  if (n_tok > (1LL << 23)) return set_error(GTR_ERR_INVALID_ARG, "grid %dx%d has more than 2^23 tokens", grid_h, grid_w);
  if (bh > (1LL << 20)) return set_error(GTR_ERR_INVALID_ARG, "B*H = %lld exceeds 2^20", bh);
  const int elt = dtype == GTR_DTYPE_F32 ? 4 : 2;
  const size_t kb = (size_t)bh * n_tok * d_k * elt, vb = (size_t)bh * n_tok * d_v * elt;
  const size_t sb = (size_t)bh * d_k * d_v * sizeof(float);
  const bool empty = bh == 0 || n_tok == 0;
  const void *ins[7] = {q, k, v, log_gate, dout, s0, ds_final};
  const size_t in_bytes[7] = {kb, kb, vb, kb, vb, sb, sb};
  const char *in_names[7] = {"q", "k", "v", "log_gate", "dout", "s0", "ds_final"};
  const void *outs[5] = {dq, dk, dv, dlog_gate, ds0};
  const size_t out_bytes[5] = {kb, kb, vb, kb, sb};
  const char *out_names[5] = {"dq", "dk", "dv", "dlog_gate", "ds0"};
  if (!empty)
    for (int i = 0; i < 5; ++i)
      if (i < 4 && (!ins[i] || !outs[i]))
        return set_error(GTR_ERR_INVALID_ARG, "null tensor pointer (%s or %s)", in_names[i], out_names[i]);
  if (!empty && !dout) return set_error(GTR_ERR_INVALID_ARG, "null tensor pointer (dout)");
  for (int i = 0; i < 7; ++i)
    if (ins[i] && (reinterpret_cast<uintptr_t>(ins[i]) & 15u))
      return set_error(GTR_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", in_names[i], ins[i]);
  for (int i = 0; i < 5; ++i) {
    if (!outs[i]) continue;
    if (reinterpret_cast<uintptr_t>(outs[i]) & 15u)
      return set_error(GTR_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", out_names[i], outs[i]);
    for (int j = 0; j < 7; ++j)
      if (ins[j] && overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return set_error(GTR_ERR_ALIAS, "%s overlaps %s", out_names[i], in_names[j]);
    for (int j = 0; j < i; ++j)
      if (outs[j] && overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return set_error(GTR_ERR_ALIAS, "%s overlaps %s", out_names[i], out_names[j]);
  }
  if (empty && (bh == 0 || !ds0)) return GTR_OK;
  int n_dev = 0, device = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev <= 0 || hipGetDevice(&device) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(GTR_ERR_NO_DEVICE, "no HIP device available");
  }
  if (!gtr::stream_capturing(stream) && !gtr::pointer_checks_off()) {
    for (int i = 0; i < 7; ++i)
      if (ins[i] && in_bytes[i]) {
        const int rc = gtr::check_device_pointer(ins[i], in_bytes[i], device, in_names[i]);
        if (rc != GTR_OK) return rc;
      }
    for (int i = 0; i < 5; ++i)
      if (outs[i] && out_bytes[i]) {
        const int rc = gtr::check_device_pointer(outs[i], out_bytes[i], device, out_names[i]);
        if (rc != GTR_OK) return rc;
      }
  }
  if (empty)  // no tokens: S_final = s0, so dL/ds0 = dL/dS_final
    return launched(gtr::launch_state_copy(ds_final, ds0, bh * d_k * d_v, stream));

  const int n_chunk = (int)((n_tok + gtr::kChunk - 1) / gtr::kChunk);
  const Layout lay = layout(bh, n_tok, n_chunk, d_k, d_v);
  void *wsp = nullptr;
  int rc = gtr::stream_buffer(gtr::kBufBackward, device, stream, lay.total, "backward", &wsp);
  if (rc != GTR_OK) return rc;
  char *ws = static_cast<char *>(wsp);
  auto scan_area = [&](size_t off, gtr::LaunchArgs &a) {
    float *f = reinterpret_cast<float *>(ws + off);
    const size_t st = (size_t)bh * n_chunk * gtr::kStateElems;
    a.agg = f;
    a.prev = f + st;
    a.agg_dec = f + 2 * st;
  };
  float *sfin = ds_final ? reinterpret_cast<float *>(ws + lay.sfin) : nullptr;
  float *g0 = ds0 ? reinterpret_cast<float *>(ws + lay.g0) : nullptr;

  gtr::LaunchArgs f{};  // 1. states entering each chunk
  f.q = q; f.k = k; f.v = v; f.g = log_gate; f.out = nullptr;
  f.bh = (int)bh; f.d_k = d_k; f.d_v = d_v; f.nk = 1; f.nvb = 1;
  f.grid_h = grid_h; f.grid_w = grid_w; f.n_tok = (int)n_tok; f.direction = direction; f.dtype = dtype;
  f.n_chunk = n_chunk; f.seg_len = 1; f.n_seg = n_chunk;
  f.s0 = s0; f.s_final = sfin; f.fused = false; f.states_only = true; f.stream = stream;
  f.fp32_operands = true;  // the boundary states feed sums whose terms cancel (dlog_gate)
  scan_area(lay.fwd, f);
  if ((rc = launched(gtr::launch_gla(f))) != GTR_OK) return rc;
  gtr::LaunchArgs r = f;  // 2. the state gradients along the reversed scan, then dv from them
  r.q = k; r.k = q; r.v = dout; r.out = dv; r.lag_gates = true;
  r.direction = direction ^ 1;
  r.s0 = ds_final; r.s_final = g0;
  scan_area(lay.rev, r);
  if ((rc = launched(gtr::launch_gla(r))) != GTR_OK) return rc;
  gtr::LaunchArgs o = r;  // dv alone needs no fp32 operands
  o.states_only = false; o.outputs_only = true; o.fp32_operands = false; o.s0 = nullptr; o.s_final = nullptr;
  // segments of the forward path's length, each entering with the state of its first chunk
  o.prev_per_chunk = true;
  o.seg_len = (int)gtr::split_segment_length(bh, n_chunk);
  o.n_seg = (n_chunk + o.seg_len - 1) / o.seg_len;
  if ((rc = launched(gtr::launch_gla(o))) != GTR_OK) return rc;
  gtr::BwdArgs b{};  // 3. dq
  float *dq_off = reinterpret_cast<float *>(ws + lay.dq_off), *dk_off = reinterpret_cast<float *>(ws + lay.dk_off);
  b.kop = k; b.aop = dout; b.bop = v; b.g = log_gate; b.out = dq; b.off = dq_off; b.prev = f.prev;
  b.bh = (int)bh; b.grid_h = grid_h; b.grid_w = grid_w; b.n_tok = (int)n_tok; b.direction = direction;
  b.dtype = dtype; b.n_chunk = n_chunk; b.d_k = d_k; b.d_v = d_v; b.stream = stream;
  if ((rc = launched(gtr::launch_gla_bwd_dqk(b))) != GTR_OK) return rc;
  // 4. dk, and beside it the gate-gradient term x = q dq - k dk (in dk_off)
  b.kop = q; b.aop = v; b.bop = dout; b.out = dk; b.off = dk_off; b.prev = r.prev; b.lag_gates = true;
  b.pair = dq_off; b.kx = k;
  b.direction = direction ^ 1;
  if ((rc = launched(gtr::launch_gla_bwd_dqk(b))) != GTR_OK) return rc;
  // 5. dlog_gate
  if ((rc = launched(gtr::launch_dgate(dk_off, ds_final, sfin, reinterpret_cast<float *>(ws + lay.totals),
                                       dlog_gate, (int)bh, grid_h, grid_w, d_k, d_v, n_chunk, direction,
                                       dtype, stream))) != GTR_OK)
    return rc;
  if (ds0)  // 6. ds0
    return launched(gtr::launch_ds0(log_gate, g0, ds0, (int)bh, grid_h, grid_w, d_k, d_v, direction, dtype,
                                    stream));
  return GTR_OK;
}

}  // extern "C"
