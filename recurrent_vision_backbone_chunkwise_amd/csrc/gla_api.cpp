// Host entry points of the GLA forward library: argument validation (before
// any HIP call), a per-(device, stream) workspace cache, and dispatch to the
// kernel launchers.  See include/gtr_gla.h for the contract.

#include "gtr_gla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "gla_internal.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr long long kMaxTokens = 1LL << 23;  // element offsets inside a sequence fit in 32 bits
constexpr long long kMaxSeqs = 1LL << 20;
constexpr int kMaxHeadDim = 2 * gtr::kHead;  // two 64-wide key or value blocks

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int elem_size(int dtype) { return dtype == GTR_DTYPE_F32 ? 4 : 2; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

struct Shape {
  long long bh, n_tok;
  int dk, dv;
  int nk, nvb;     // 64-wide key blocks and value blocks per head
  long long seqs;  // sequences the kernels walk: B*H*nvb
  int n_chunk, seg_len, n_seg;
  bool fused;
  int fold_block;  // one-launch path: segments per fold block
  bool empty;      // B*H == 0 or no tokens: nothing to compute
};

// Launch structure and segment length for a shape.
//  * split: the length split_segment_length picks; the boundary scan runs in
//    its own kernel.
//  * fused: segments of at most kMaxFusedChunks chunks (each chunk's outputs
//    wait in registers for the state entering the segment), grouped in blocks
//    of kFoldBlock segments.  Measured on MI355X (3-chunk segments, fp16, four
//    directions): blocks of 4, 8, 16 and 32 took 342, 338, 383 and 433 us per
//    128x128 B1 H16 round; folds cost more than the chain between blocks.
// Automatic choice, from four-direction rounds measured on MI355X (64x64
// heads; us per round, three launches against one):
//  * the one launch wins where a sequence has at most 48 chunks, there are
//    at least as many sequences as XCDs, and the segments fill about one
//    round of resident workgroups (two per CU at 16-bit I/O, one at fp32),
//    with the shortest segments that fit best:
//      1-chunk segments: 24x24 B4 H6 69.4 -> 56.4, 32x32 B3 H6 80.7 -> 69.0,
//        40x40 B2 H6 80.3 -> 72.3, 40x40 B1 H8 67.6 -> 64.3;
//      2-chunk: 48x48 B1 H16 102.7 -> 86.0 (1-chunk: 91), 40x40 B4 H6
//        100.1 -> 85.1 (1-chunk: 90.5), 16x16 B32 H6 118 -> 82;
//      3-chunk, allowed one more workgroup per CU: 40x40 B8 H6 145 -> 112
//        (2-chunk: 121.5), 32x32 B16 H6 149 -> 122;
//      fp32: 32x32 B4 H6 130 -> 110 (2-chunk), 48x48 B1 H16 182 -> 145 and
//        40x40 B8 H6 289 -> 258 (3-chunk);
//  * three launches win with longer sequences (64x64 B1 H12: 98 against 104;
//    128x128 B1 H4: 125 against 183), fewer sequences than XCDs (40x40 B1
//    H6: 61.1 against 64.7), more segments than about one round (40x40 B16
//    H6: 187 against 194), and where a sequence would be one segment, for
//    which they launch only their output kernel (8x8 B16 H8: 25.3 against
//    44.1).
// The one launch's occupancy makes the choice depend on the element type;
// gtr_gla_plan, which takes none, reports it for 16-bit I/O.
constexpr int kFoldBlock = 8;
constexpr int kAutoFusedChunks = 48;
constexpr int kAssumedXcds = 8;         // MI355X; used where no device is queried
constexpr long long kAssumedCus = 256;  // MI355X; the automatic choice is made before any HIP call

// Segment length of the automatic one-launch choice, or 0 for three launches.
int auto_fused_length(long long seqs, int nk, int n_chunk, int dtype) {
  if (nk != 1 || n_chunk > kAutoFusedChunks || seqs < kAssumedXcds) return 0;
  const long long round = (dtype == GTR_DTYPE_F32 ? 1 : 2) * kAssumedCus;  // resident workgroups
  for (int len = 1; len <= gtr::kMaxFusedChunks && len < n_chunk; ++len) {  // two segments or more
    const long long segments = seqs * ((n_chunk + len - 1) / len);
    if (segments <= (len == gtr::kMaxFusedChunks ? round + kAssumedCus : round)) return len;
  }
  return 0;
}

// `bh` counts the sequences the kernels walk (B*H*value blocks); `nk` the key
// blocks, which only the three-launch path handles beyond one.
void plan(long long bh, int nk, int n_chunk, int path, int chunks_per_segment, int dtype, Shape *sh) {
  sh->fold_block = 0;
  if (bh == 0 || n_chunk == 0) {
    sh->fused = false;
    sh->seg_len = sh->n_seg = 0;
    return;
  }
  const int auto_len =
      path == GTR_PATH_AUTO && chunks_per_segment <= gtr::kMaxFusedChunks ? auto_fused_length(bh, nk, n_chunk, dtype) : 0;
  sh->fused = path == GTR_PATH_FUSED || auto_len > 0;
  long long len = chunks_per_segment;
  if (sh->fused) {
    // each kept chunk holds a query tile per key block in LDS: with fp32
    // operands and two key blocks, two chunks fill it
    const int max_len = nk == 2 && dtype == GTR_DTYPE_F32 ? 2 : gtr::kMaxFusedChunks;
    if (len <= 0) len = auto_len > 0 ? auto_len : max_len;
    len = std::min<long long>(len, max_len);
  } else if (len <= 0) {
    len = gtr::split_segment_length(bh, n_chunk);
  }
  if (len > n_chunk) len = n_chunk;
  sh->seg_len = (int)len;
  sh->n_seg = (int)((n_chunk + len - 1) / len);
  if (sh->fused) {
    // blocks of at most kFoldBlock segments, balanced: 9 segments fold as 5 + 4
    // rather than 8 + 1, which shortens the fold on the path to the last block
    // (40x40 B8 H6: 117.7 -> 115.0 us per round)
    const int blocks = (sh->n_seg + kFoldBlock - 1) / kFoldBlock;
    sh->fold_block = (sh->n_seg + blocks - 1) / blocks;
    // measurement aid: GTR_GLA_FOLD_BLOCK=n sets the fold block size (1..32)
    static const int forced = [] {
      const char *e = std::getenv("GTR_GLA_FOLD_BLOCK");
      return e ? std::atoi(e) : 0;
    }();
    if (forced >= 1 && forced <= gtr::kMaxFoldBlock) sh->fold_block = std::min(forced, sh->n_seg);
  }
}

// Shape, direction and dtype checks; fills `shape`.
int validate_shape(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction,
                   int dtype, int chunks_per_segment, int path, Shape *shape) {
  if (B < 0 || H < 0 || grid_h < 0 || grid_w < 0 || d_k <= 0 || d_v <= 0)
    return fail(GTR_ERR_INVALID_ARG,
                "sizes must be >= 0 and head sizes > 0 (B=%d H=%d grid=%dx%d d_k=%d d_v=%d)", B, H,
                grid_h, grid_w, d_k, d_v);
  if (direction < 0 || direction > 3)
    return fail(GTR_ERR_INVALID_ARG, "direction %d not in 0..3", direction);
  if (dtype < 0 || dtype > 2) return fail(GTR_ERR_INVALID_ARG, "dtype %d not in 0..2", dtype);
  if (path < 0 || path > 2) return fail(GTR_ERR_INVALID_ARG, "path %d not in 0..2", path);
  const long long n_tok = (long long)grid_h * grid_w;
  const long long bh = (long long)B * H;
  if (n_tok > kMaxTokens)
    return fail(GTR_ERR_INVALID_ARG, "grid %dx%d has more than 2^23 tokens", grid_h, grid_w);
  if (bh > kMaxSeqs) return fail(GTR_ERR_INVALID_ARG, "B*H = %lld exceeds 2^20", bh);
  if (d_k % 4 || d_v % 4 || d_k > kMaxHeadDim || d_v > kMaxHeadDim)
    return fail(GTR_ERR_UNSUPPORTED, "d_k=%d d_v=%d: head dims must be multiples of 4, at most %d",
                d_k, d_v, kMaxHeadDim);
  // byte offsets inside one sequence's rows stay below 2^31
  if (n_tok * std::max(d_k, d_v) * elem_size(dtype) > (1LL << 31))
    return fail(GTR_ERR_INVALID_ARG, "%lld tokens of %d elements exceed 2^31 bytes per sequence",
                n_tok, std::max(d_k, d_v));
  shape->bh = bh;
  shape->n_tok = n_tok;
  shape->dk = d_k;
  shape->dv = d_v;
  shape->nk = (d_k + gtr::kHead - 1) / gtr::kHead;
  shape->nvb = (d_v + gtr::kHead - 1) / gtr::kHead;
  shape->seqs = bh * shape->nvb;
  shape->empty = bh == 0 || n_tok == 0;
  shape->n_chunk = (int)((n_tok + gtr::kChunk - 1) / gtr::kChunk);
  plan(shape->seqs, shape->nk, shape->n_chunk, path, chunks_per_segment, dtype, shape);
  if (shape->seqs * shape->n_seg * shape->nk > 0x7fffffffLL)
    return fail(GTR_ERR_INVALID_ARG, "too many segments (%lld)", shape->seqs * shape->n_seg);
  // a sequence's payload slots are addressed with 32-bit byte offsets
  if (shape->fused &&
      (long long)shape->n_seg * shape->nk * gtr::kSlotFloats * (long long)sizeof(float) >= (1LL << 31))
    return fail(GTR_ERR_INVALID_ARG,
                "one-launch path: %d segments of %d chunks exceed its per-sequence workspace; use longer "
                "segments, GTR_PATH_SPLIT or GTR_PATH_AUTO",
                shape->n_seg, shape->seg_len);
  return GTR_OK;
}

// Everything that can be checked without touching the HIP runtime.
int validate(const void *q, const void *k, const void *v, const void *g, const void *out, int B,
             int H, int grid_h, int grid_w, int d_k, int d_v, int direction, int dtype,
             const float *s0, const float *s_final, int chunks_per_segment, int path,
             Shape *shape) {
  int rc = validate_shape(B, H, grid_h, grid_w, d_k, d_v, direction, dtype, chunks_per_segment,
                          path, shape);
  if (rc != GTR_OK) return rc;
  // tensors of zero elements may be null
  if (!shape->empty && (!q || !k || !v || !g || !out))
    return fail(GTR_ERR_INVALID_ARG, "null tensor pointer (q=%p k=%p v=%p log_gate=%p out=%p)", q, k,
                v, g, out);
  const void *ptrs[7] = {q, k, v, g, out, s0, s_final};
  const char *names[7] = {"q", "k", "v", "log_gate", "out", "s0", "s_final"};
  for (int i = 0; i < 7; ++i)
    if (ptrs[i] && (reinterpret_cast<uintptr_t>(ptrs[i]) & 15u))
      return fail(GTR_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
  const size_t kb = (size_t)(shape->bh * shape->n_tok * d_k) * elem_size(dtype);
  const size_t vb = (size_t)(shape->bh * shape->n_tok * d_v) * elem_size(dtype);
  const size_t sb = (size_t)shape->bh * d_k * d_v * sizeof(float);
  const void *ins[5] = {q, k, v, g, s0};
  const size_t in_bytes[5] = {kb, kb, vb, kb, sb};
  for (int i = 0; i < 5; ++i) {
    if (!ins[i]) continue;
    if (overlaps(out, vb, ins[i], in_bytes[i]))
      return fail(GTR_ERR_ALIAS, "out overlaps %s", names[i]);
    if (s_final && overlaps(s_final, sb, ins[i], in_bytes[i]))
      return fail(GTR_ERR_ALIAS, "s_final overlaps %s", names[i]);
  }
  if (s_final && overlaps(s_final, sb, out, vb)) return fail(GTR_ERR_ALIAS, "s_final overlaps out");
  return GTR_OK;
}

// Device memory of the current device, at least `bytes` long from `p`.
int check_device_range(const void *p, size_t bytes, int device, const char *name) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(GTR_ERR_POINTER, "%s=%p is not memory known to the HIP runtime", name, p);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(GTR_ERR_POINTER, "%s=%p is not device memory (type %d)", name, p, (int)attr.type);
  if (attr.device != device)
    return fail(GTR_ERR_POINTER, "%s=%p lives on device %d, current device is %d", name, p,
                attr.device, device);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) == hipSuccess && base) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), x = reinterpret_cast<uintptr_t>(p);
    if (x + bytes > b + size)
      return fail(GTR_ERR_POINTER, "%s=%p: allocation ends %zu bytes short of the tensor", name, p,
                  (size_t)(x + bytes - (b + size)));
  } else {
    (void)hipGetLastError();
  }
  return GTR_OK;
}

// Fused-path synchronisation words live at positions that do not depend on a
// call's shape: [header][per-XCD work words][cap_flags flags].  The header and
// work words return to zero (the epoch aside) after every call and flags only
// hold epochs, so any shape can follow any other on the same workspace.
struct Workspace {
  void *data = nullptr;  // float32 aggregates and boundary states
  size_t data_bytes = 0;
  int *sync = nullptr;   // zero-initialised
  size_t cap_flags = 0;
};

// Guards the workspaces, the other cached buffers and the retired list.
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::map<std::tuple<int, int, hipStream_t>, std::pair<void *, size_t>> g_bufs;  // (owner, device, stream)
// Buffers replaced by larger ones, with their devices.  A graph captured
// earlier may still refer to them, so they are freed only by
// gtr_gla_release_workspaces.
std::vector<std::pair<int, void *>> g_retired;

void retire(int device, void *p) {
  if (p) g_retired.push_back({device, p});
}

// hipMalloc for the workspaces.  GTR_GLA_TEST_FAIL_ALLOC=1 makes it fail, so
// that tests can reach the allocation-failure paths.
hipError_t workspace_malloc(void **p, size_t bytes) {
  const char *s = std::getenv("GTR_GLA_TEST_FAIL_ALLOC");
  if (s && s[0] == '1') {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  return hipMalloc(p, bytes);
}

// `need_sync`: the call uses the synchronisation words, with `flags` flags.
int get_workspace(int device, hipStream_t stream, size_t bytes, bool need_sync, size_t flags,
                  void **data, int **sync, long long **flag_words) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace &ws = g_ws[{device, stream}];
  const bool sync_ok = !need_sync || (ws.sync && ws.cap_flags >= flags);
  auto hand_out = [&] {
    *data = ws.data;
    *sync = ws.sync;
    // 64-bit flags after the work words (an even word offset: 8-byte aligned)
    *flag_words = ws.sync ? reinterpret_cast<long long *>(ws.sync + gtr::kSyncFlagWord) : nullptr;
  };
  if (ws.data_bytes >= bytes && sync_ok) {
    hand_out();
    return GTR_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    cs = hipStreamCaptureStatusNone;
  }
  if (cs != hipStreamCaptureStatusNone)
    return fail(GTR_ERR_CAPTURE,
                "workspace must grow (%zu -> %zu bytes, %zu -> %zu flags) "
                "while the stream is being captured; make one call of this shape before capturing",
                ws.data_bytes, bytes, ws.cap_flags, flags);
  // Kernels queued earlier, and graphs captured earlier, may still use the
  // old buffers: they are retired, not freed.
  // A failed allocation leaves the cached buffers as they were.
  if (ws.data_bytes < bytes) {
    const size_t want = bytes + bytes / 4;  // headroom for slightly larger calls
    void *p = nullptr;
    if (workspace_malloc(&p, want) != hipSuccess) {
      (void)hipGetLastError();
      return fail(GTR_ERR_ALLOC, "hipMalloc of %zu workspace bytes failed", want);
    }
    retire(device, ws.data);
    ws.data = p;
    ws.data_bytes = want;
  }
  if (!sync_ok) {
    const size_t flag_cap = std::max(ws.cap_flags, flags + flags / 4);
    const size_t words = gtr::sync_words(flag_cap);
    void *p = nullptr;
    if (workspace_malloc(&p, words * sizeof(int)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(GTR_ERR_ALLOC, "hipMalloc of %zu sync words failed", words);
    }
    // synchronous clear, so that kernels on any stream see zeros
    if (hipMemset(p, 0, words * sizeof(int)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(p);
      return fail(GTR_ERR_ALLOC, "clearing %zu sync words failed", words);
    }
    retire(device, ws.sync);
    ws.sync = static_cast<int *>(p);
    ws.cap_flags = flag_cap;
  }
  hand_out();
  return GTR_OK;
}

// CU and XCD counts of a device, queried once (MI355X: 256 and 8).  They size
// the one-launch path's persistent grid and its sequence batches.
struct DeviceShape {
  int cus = 256, xcds = kAssumedXcds;
};
constexpr long long kMaxBatch = 16;  // sequences an XCD claims at a time

const DeviceShape &device_shape(int device) {
  static std::mutex m;
  static std::map<int, DeviceShape> cache;
  std::lock_guard<std::mutex> lock(m);
  auto it = cache.find(device);
  if (it != cache.end()) return it->second;
  DeviceShape d;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && v > 0) d.cus = v;
  else (void)hipGetLastError();
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, device) == hipSuccess && v > 0) d.xcds = v;
  else (void)hipGetLastError();
  return cache.emplace(device, d).first->second;
}

bool skip_pointer_checks() {
  static const bool skip = [] {
    const char *s = std::getenv("GTR_GLA_SKIP_POINTER_CHECKS");
    return s && s[0] == '1';
  }();
  return skip;
}

}  // namespace

namespace gtr {

// Segment length of the three-launch path.  Each CU walks its workgroups'
// chunks, two workgroups already saturate it and one alone runs about 1.35x
// slower per chunk (measured on MI355X), so the cost of a length s is the chunk
// load of the busiest CU in the output kernel, half that for the state kernel
// (which moves 3/5 of the bytes and skips the last segment), plus the
// boundary scan, which grows with the segment count.
long long split_segment_length(long long bh, int n_chunk) {
  constexpr long long kCUs = 256;
  auto load = [&](long long groups, long long s) {
    const long long waves = (groups + kCUs - 1) / kCUs;
    return (double)(waves * s) * (waves <= 1 ? 1.35 : 1.0);
  };
  long long best = 1;
  double best_cost = 1e300;
  for (long long s = 1; s <= 32 && s <= n_chunk; ++s) {
    const long long n_seg = (n_chunk + s - 1) / s;
    const double cost = load(bh * n_seg, s) + 0.5 * load(bh * (n_seg - 1), s) + 0.06 * (double)n_seg;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

int set_error(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int check_device_pointer(const void *p, size_t bytes, int device, const char *name) {
  return check_device_range(p, bytes, device, name);
}

bool pointer_checks_off() { return skip_pointer_checks(); }

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

int stream_buffer(int owner, int device, hipStream_t stream, size_t bytes, const char *what, void **out) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  auto &buf = g_bufs[std::make_tuple(owner, device, stream)];
  if (buf.second < bytes) {
    if (stream_capturing(stream))
      return set_error(GTR_ERR_CAPTURE,
                       "%s workspace must grow (%zu -> %zu bytes) while the stream is being captured; "
                       "make one call of this shape before capturing",
                       what, buf.second, bytes);
    void *p = nullptr;
    const size_t want = bytes + bytes / 4;  // headroom for slightly larger calls
    if (workspace_malloc(&p, want) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(GTR_ERR_ALLOC, "hipMalloc of %zu %s workspace bytes failed", want, what);
    }
    retire(device, buf.first);
    buf = {p, want};
  }
  *out = buf.first;
  return GTR_OK;
}

}  // namespace gtr

namespace {

// All host-side checks of one call, including the device-pointer queries.
int check_call(const void *q, const void *k, const void *v, const void *log_gate, void *out, int B,
               int H, int grid_h, int grid_w, int d_k, int d_v, int direction, int dtype,
               const float *s0, float *s_final, int chunks_per_segment, int path, Shape *sh,
               int *device, hipStream_t stream, bool check_stream) {
  g_last_error.clear();
  int rc = validate(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction, dtype, s0,
                    s_final, chunks_per_segment, path, sh);
  if (rc != GTR_OK) return rc;
  // nothing to compute and no state to hand back: no device work at all
  if (sh->empty && (sh->bh == 0 || !s_final)) return GTR_OK;
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev <= 0) {
    (void)hipGetLastError();
    return fail(GTR_ERR_NO_DEVICE, "no HIP device available");
  }
  if (hipGetDevice(device) != hipSuccess) {
    (void)hipGetLastError();
    return fail(GTR_ERR_NO_DEVICE, "hipGetDevice failed");
  }
  bool capturing = false;
  if (check_stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
      (void)hipGetLastError();
    } else {
      capturing = cs != hipStreamCaptureStatusNone;
    }
  }
  // Pointer queries are not capture-safe on every runtime; calls being captured
  // rely on the same checks having passed for an eager call before capture.
  if (!capturing && !skip_pointer_checks()) {
    const size_t kb = (size_t)(sh->bh * sh->n_tok * d_k) * elem_size(dtype);
    const size_t vb = (size_t)(sh->bh * sh->n_tok * d_v) * elem_size(dtype);
    const size_t sb = (size_t)sh->bh * d_k * d_v * sizeof(float);
    const void *ptrs[7] = {q, k, v, log_gate, out, s0, s_final};
    const char *names[7] = {"q", "k", "v", "log_gate", "out", "s0", "s_final"};
    const size_t sizes[7] = {kb, kb, vb, kb, vb, sb, sb};
    for (int i = 0; i < 7; ++i) {
      if (!ptrs[i] || sizes[i] == 0) continue;
      rc = check_device_range(ptrs[i], sizes[i], *device, names[i]);
      if (rc != GTR_OK) return rc;
    }
  }
  return GTR_OK;
}

}  // namespace

extern "C" {

int gtr_gla_check(const void *q, const void *k, const void *v, const void *log_gate, void *out,
                  int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction, int dtype,
                  const float *s0, float *s_final, int chunks_per_segment, int path) {
  Shape sh;
  int device = 0;
  return check_call(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction, dtype, s0,
                    s_final, chunks_per_segment, path, &sh, &device, nullptr, false);
}

int gtr_gla_fwd_ex(const void *q, const void *k, const void *v, const void *log_gate, void *out,
                   int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction,
                   int dtype, const float *s0, float *s_final, int chunks_per_segment, int path,
                   hipStream_t stream) {
  Shape sh;
  int device = 0;
  int rc = check_call(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction, dtype, s0,
                      s_final, chunks_per_segment, path, &sh, &device, stream, true);
  if (rc != GTR_OK) return rc;
  if (sh.empty) {
    // no tokens: the state after the sequence is the state before it
    if (sh.bh == 0 || !s_final) return GTR_OK;
    const int err = gtr::launch_state_copy(s0, s_final, sh.bh * d_k * d_v, stream);
    if (err != (int)hipSuccess)
      return fail(GTR_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
    return GTR_OK;
  }

  gtr::LaunchArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = log_gate;
  a.out = out;
  a.bh = (int)sh.seqs;
  a.d_k = d_k;
  a.d_v = d_v;
  a.nk = sh.nk;
  a.nvb = sh.nvb;
  a.grid_h = grid_h;
  a.grid_w = grid_w;
  a.n_tok = (int)sh.n_tok;
  a.direction = direction;
  a.dtype = dtype;
  a.n_chunk = sh.n_chunk;
  a.seg_len = sh.seg_len;
  a.n_seg = sh.n_seg;
  a.s0 = s0;
  a.s_final = s_final;
  a.stream = stream;
  // A single fused segment needs no state passing: the fused kernel covers it
  // with an empty wait list; the split path needs its scan only for n_seg > 1 or a state.
  a.fused = sh.fused;
  const bool need_ws = sh.fused || sh.n_seg > 1 || s0 || s_final;
  if (need_ws) {
    void *ws = nullptr;
    int *sync = nullptr;
    long long *flags = nullptr;
    const size_t bytes = sh.fused ? gtr::fused_workspace_bytes(sh.seqs, sh.n_seg, sh.nk)
                                  : gtr::workspace_bytes(sh.seqs, sh.n_seg, sh.nk);
    rc = get_workspace(device, stream, bytes, sh.fused, sh.fused ? sh.seqs * sh.n_seg : 0, &ws, &sync, &flags);
    if (rc != GTR_OK) return rc;
    float *f = static_cast<float *>(ws);
    const size_t st = (size_t)sh.seqs * sh.n_seg * sh.nk * gtr::kStateElems;
    a.agg = f;
    a.prev = sh.fused ? nullptr : f + st;  // the one-launch path keeps no entering states
    a.agg_dec = sh.fused ? nullptr : f + 2 * st;  // (its decays sit in each segment's payload slot)
    a.sync = sync;
    a.flags = flags;
  }
  if (sh.fused) {
    const DeviceShape &ds = device_shape(device);
    const int occupancy = dtype == GTR_DTYPE_F32 || sh.nk == 2 ? 1 : 2;  // workgroups per CU (as the kernel's bounds)
    a.fold_block = sh.fold_block;
    a.xcds = ds.xcds;
    // one batch per XCD where every segment fits in one round of resident
    // workgroups (16x16 B32 H6, 2-chunk segments: 12 batches of at most 16
    // sequences left four XCDs a second round); otherwise batches of at most
    // kMaxBatch sequences, handed out as XCDs free up
    const long long per_xcd_seqs = (sh.seqs + ds.xcds - 1) / ds.xcds;
    const bool one_round = per_xcd_seqs * sh.n_seg * ds.xcds <= (long long)occupancy * ds.cus;
    a.batch = (int)(one_round ? per_xcd_seqs : std::min<long long>(kMaxBatch, per_xcd_seqs));
    const long long per_xcd = (long long)a.batch * sh.n_seg;
    a.grid = (int)std::max<long long>(1, std::min<long long>((long long)occupancy * ds.cus, per_xcd * ds.xcds));
  }
  const int err = gtr::launch_gla(a);
  if (err != (int)hipSuccess)
    return fail(GTR_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
  return GTR_OK;
}

int gtr_gla_fwd_static(const void *q, const void *k, const void *v, const void *log_gate, void *out, int B,
                       int H, int grid_h, int grid_w, int d_k, int d_v, int direction, int dtype,
                       hipStream_t stream) {
  Shape sh;
  int device = 0;
  int rc = check_call(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction, dtype, nullptr,
                      nullptr, 0, GTR_PATH_SPLIT, &sh, &device, stream, true);
  if (rc != GTR_OK || sh.empty) return rc;
  // Three launches, whose boundary states (the only working memory) must fit
  // the fixed array: the planner's segment length, or the shortest longer one
  // (up to 32 chunks) that fits; a single segment per sequence needs none.
  auto ws_bytes = [&](long long n_seg) {
    return n_seg > 1 ? gtr::workspace_bytes((size_t)sh.seqs, (size_t)n_seg, (size_t)sh.nk) : (size_t)0;
  };
  long long seg_len = sh.seg_len, n_seg = sh.n_seg;
  while (ws_bytes(n_seg) > gtr::kStaticScratchBytes && seg_len < std::min<long long>(32, sh.n_chunk)) {
    ++seg_len;
    n_seg = (sh.n_chunk + seg_len - 1) / seg_len;
  }
  if (ws_bytes(n_seg) > gtr::kStaticScratchBytes)
    return fail(GTR_ERR_SCRATCH,
                "gtr_gla_fwd_static: %lld sequences of %d chunks need %zu bytes of boundary states even with "
                "%lld-chunk segments; its fixed array holds %zu (use gtr_gla_fwd)",
                sh.seqs, sh.n_chunk, ws_bytes(n_seg), seg_len, gtr::kStaticScratchBytes);
  gtr::LaunchArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = log_gate;
  a.out = out;
  a.bh = (int)sh.seqs;
  a.d_k = d_k;
  a.d_v = d_v;
  a.nk = sh.nk;
  a.nvb = sh.nvb;
  a.grid_h = grid_h;
  a.grid_w = grid_w;
  a.n_tok = (int)sh.n_tok;
  a.direction = direction;
  a.dtype = dtype;
  a.n_chunk = sh.n_chunk;
  a.seg_len = (int)seg_len;
  a.n_seg = (int)n_seg;
  a.stream = stream;
  if (n_seg > 1) {
    void *ptr = nullptr;
    const int e = gtr::static_scratch(device, &ptr);
    if (e != (int)hipSuccess)
      return fail(GTR_ERR_LAUNCH, "gtr_gla_fwd_static: the fixed array's device address: %s",
                  hipGetErrorString((hipError_t)e));
    float *f = static_cast<float *>(ptr);
    const size_t st = (size_t)sh.seqs * n_seg * sh.nk * gtr::kStateElems;
    a.agg = f;
    a.prev = f + st;
    a.agg_dec = f + 2 * st;
  }
  const int err = gtr::launch_gla(a);
  if (err != (int)hipSuccess)
    return fail(GTR_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
  return GTR_OK;
}

int gtr_gla_fwd(const void *q, const void *k, const void *v, const void *log_gate, void *out, int B,
                int H, int grid_h, int grid_w, int d_k, int d_v, int direction, int dtype,
                hipStream_t stream) {
  return gtr_gla_fwd_ex(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction, dtype,
                        nullptr, nullptr, 0, GTR_PATH_AUTO, stream);
}

int gtr_gla_fwd_f32(const void *q, const void *k, const void *v, const void *log_gate, void *out,
                    int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction,
                    hipStream_t stream) {
  return gtr_gla_fwd(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction,
                     GTR_DTYPE_F32, stream);
}

int gtr_gla_fwd_f16(const void *q, const void *k, const void *v, const void *log_gate, void *out,
                    int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction,
                    hipStream_t stream) {
  return gtr_gla_fwd(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction,
                     GTR_DTYPE_F16, stream);
}

int gtr_gla_fwd_bf16(const void *q, const void *k, const void *v, const void *log_gate, void *out,
                     int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction,
                     hipStream_t stream) {
  return gtr_gla_fwd(q, k, v, log_gate, out, B, H, grid_h, grid_w, d_k, d_v, direction,
                     GTR_DTYPE_BF16, stream);
}

size_t gtr_gla_workspace_bytes_ex(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dtype,
                                  int chunks_per_segment, int path) {
  Shape sh;
  if (validate_shape(B, H, grid_h, grid_w, d_k, d_v, 0, dtype, chunks_per_segment, path, &sh) !=
      GTR_OK)
    return 0;
  if (sh.empty) return 0;
  return (sh.fused ? gtr::fused_workspace_bytes(sh.seqs, sh.n_seg, sh.nk)
                   : gtr::workspace_bytes(sh.seqs, sh.n_seg, sh.nk)) +
         (sh.fused ? gtr::sync_words((size_t)(sh.seqs * sh.n_seg)) * sizeof(int) : 0);
}

size_t gtr_gla_workspace_bytes(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int dtype) {
  return gtr_gla_workspace_bytes_ex(B, H, grid_h, grid_w, d_k, d_v, dtype, 0, GTR_PATH_AUTO);
}

int gtr_gla_plan(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunks_per_segment,
                 int path, int *seg_len, int *n_seg, int *fused) {
  Shape sh;
  g_last_error.clear();
  const int rc = validate_shape(B, H, grid_h, grid_w, d_k, d_v, 0, GTR_DTYPE_F16, chunks_per_segment,
                                path, &sh);
  if (rc != GTR_OK) return rc;
  if (seg_len) *seg_len = sh.seg_len;
  if (n_seg) *n_seg = sh.n_seg;
  if (fused) *fused = sh.fused ? 1 : 0;
  return GTR_OK;
}

const char *gtr_gla_last_error(void) { return g_last_error.c_str(); }

int gtr_gla_version(void) { return kVersion; }

int gtr_gla_stream_status(hipStream_t stream) {
  g_last_error.clear();
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) {
    (void)hipGetLastError();
    return fail(GTR_ERR_NO_DEVICE, "no HIP device available");
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
    return fail(GTR_ERR_CAPTURE, "stream status cannot be read while the stream is being captured");
  (void)hipGetLastError();
  int *sync = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_ws.find({device, stream});
    if (it != g_ws.end()) sync = it->second.sync;
  }
  if (hipStreamSynchronize(stream) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    return fail(GTR_ERR_LAUNCH, "stream synchronisation failed: %s", hipGetErrorString(e));
  }
  if (!sync) return GTR_OK;
  int word = 0;
  if (hipMemcpy(&word, sync + gtr::kSyncErrorWord, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    return fail(GTR_ERR_LAUNCH, "reading the workspace status failed: %s", hipGetErrorString(e));
  }
  if (word == 0) return GTR_OK;
  const int zero = 0;
  (void)hipMemcpy(sync + gtr::kSyncErrorWord, &zero, sizeof(int), hipMemcpyHostToDevice);
  return fail(GTR_ERR_TIMEOUT, "a wait between workgroups of the one-launch path gave up on this stream");
}

void gtr_gla_release_workspaces(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  std::vector<std::pair<int, void *>> all = g_retired;
  for (auto &kv : g_ws) {
    if (kv.second.data) all.push_back({kv.first.first, kv.second.data});
    if (kv.second.sync) all.push_back({kv.first.first, kv.second.sync});
  }
  for (auto &kv : g_bufs)
    if (kv.second.first) all.push_back({std::get<1>(kv.first), kv.second.first});
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) (void)hipGetLastError();
  int synced = -1;
  std::sort(all.begin(), all.end());
  for (auto &dp : all) {
    if (dp.first != synced) {  // once per device, before its first free
      if (hipSetDevice(dp.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        continue;
      }
      synced = dp.first;
    }
    (void)hipFree(dp.second);
  }
  (void)hipSetDevice(cur);
  (void)hipGetLastError();
  g_ws.clear();
  g_bufs.clear();
  g_retired.clear();
}

}  // extern "C"
