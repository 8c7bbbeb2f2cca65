// Spatial SwiGLU block of a GTR layer (include/gtr_swiglu.h) for gfx950.
//
// The block (x-techcon article on GTR, section 架构 / Architecture: SwiGLU
// with a 3 x 3 per-channel convolution in the value branch, so that adjacent
// patches exchange information) runs as three steps on the caller's stream:
//   1. u = x W_in           rocBLAS GEMM, fp32 accumulation; u stored in fp16
//                           for fp16 I/O, else in fp32
//   2. h = SiLU(u_g) * (DWConv3x3(u_v) + b)   swiglu_mix below, h in the I/O
//                           type, except fp16 for bf16 I/O
//   3. out = h W_out        rocBLAS GEMM, fp32 accumulation; for bf16 I/O on
//                           fp16 operands (W_out converted first) into fp32,
//                           then rounded to bf16
// The projections are plain dense GEMMs, the library's job; the step between
// them is bandwidth-bound elementwise work with a 3 x 3 neighbourhood, done by
// one kernel that stages each tile's value columns (with a one-token halo) in
// LDS and writes h once.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "gla_internal.h"
#include "gla_profile.h"
#include "gtr_swiglu.h"

namespace gtr {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef uint16_t b4 __attribute__((ext_vector_type(4)));

constexpr int kMixThreads = 256;

// Four consecutive elements of the I/O type, widened to or narrowed from fp32.
__device__ __forceinline__ f4 load4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ f4 load4(const _Float16 *p) {
  return __builtin_convertvector(*reinterpret_cast<const h4 *>(p), f4);
}
__device__ __forceinline__ f4 load4(const uint16_t *p) {  // bfloat16 bits
  const b4 b = *reinterpret_cast<const b4 *>(p);
  return f4{__uint_as_float((uint32_t)b.x << 16), __uint_as_float((uint32_t)b.y << 16),
            __uint_as_float((uint32_t)b.z << 16), __uint_as_float((uint32_t)b.w << 16)};
}
__device__ __forceinline__ void store4(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }
__device__ __forceinline__ void store4(_Float16 *p, f4 v) {
  *reinterpret_cast<h4 *>(p) = __builtin_convertvector(v, h4);
}
__device__ __forceinline__ uint16_t bf16_rne(float f) {  // round to nearest even, quiet NaN kept
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void store4(uint16_t *p, f4 v) {
  *reinterpret_cast<b4 *>(p) = b4{bf16_rne(v.x), bf16_rne(v.y), bf16_rne(v.z), bf16_rne(v.w)};
}

// Tiles of kTileY x kTileX tokens of one image and kSlice channels.  The value
// columns of the tile and its one-token halo are staged once in LDS (fp32), so
// each value is read from memory about 1.4 times instead of nine; the gate is
// read once and h written once.  Thread t handles channel group t % 16 (four
// channels) for every 16th token of the tile; its nine taps and bias stay in
// registers.  u is [tokens][2F] of type U (gate in [0, F), value in [F, 2F));
// h is [tokens][F].
constexpr int kTileY = 8, kTileX = 16, kSlice = 64;
constexpr int kGroups = kSlice / 4;                        // 16 channel groups
constexpr int kHaloY = kTileY + 2, kHaloX = kTileX + 2;    // 10 x 18 positions

__device__ __forceinline__ f4 load4(const f4 *p) { return *p; }

template <typename T, typename U, typename H>
__global__ __launch_bounds__(kMixThreads) void swiglu_mix(const U *__restrict__ u,
                                                          const T *__restrict__ conv_w,
                                                          const T *__restrict__ conv_b,
                                                          H *__restrict__ h, int grid_h, int grid_w,
                                                          int F, int slices, int tiles_x, int tiles_y) {
  __shared__ f4 val[kHaloY * kHaloX * kGroups];  // 46 KB
  const int tid = threadIdx.x;
  // block -> (image, tile row, tile column, channel slice), slice fastest
  unsigned b = blockIdx.x;
  const int slice = (int)(b % (unsigned)slices);
  b /= (unsigned)slices;
  const int tile_x = (int)(b % (unsigned)tiles_x);
  b /= (unsigned)tiles_x;
  const int tile_y = (int)(b % (unsigned)tiles_y);
  const int image = (int)(b / (unsigned)tiles_y);
  const int x0 = tile_x * kTileX, y0 = tile_y * kTileY, c0 = slice * kSlice;
  const size_t ld = 2 * (size_t)F;
  const size_t image_base = (size_t)image * grid_h * grid_w;
  const int j = tid % kGroups;
  const int c = c0 + 4 * j;
  const bool live = c < F;
  // Every load of the tile goes out before any is used: the halo's value
  // columns (zero outside the grid and past F) and this thread's gates.  The
  // loads are unconditional (a position outside the grid or past F reads
  // element 0, which exists, and is zeroed afterwards), so no branch separates
  // them and all are in flight together.
  constexpr int kStaged = kHaloY * kHaloX * kGroups;
  constexpr int kPerThread = (kStaged + kMixThreads - 1) / kMixThreads;  // 12
  constexpr int kTokensPerThread = kTileY * kTileX * kGroups / kMixThreads;  // 8
  f4 staged[kPerThread];
  bool staged_ok[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int i = tid + k * kMixThreads;
    const int pos = i / kGroups;
    const int yy = y0 - 1 + pos / kHaloX, xx = x0 - 1 + pos % kHaloX;
    const int cc = c0 + 4 * (i % kGroups);
    staged_ok[k] = i < kStaged && yy >= 0 && yy < grid_h && xx >= 0 && xx < grid_w && cc < F;
    const size_t at = staged_ok[k] ? (image_base + (size_t)yy * grid_w + xx) * ld + F + cc : 0;
    staged[k] = load4(u + at);
  }
  f4 gate[kTokensPerThread];
  bool gate_ok[kTokensPerThread];
#pragma unroll
  for (int k = 0; k < kTokensPerThread; ++k) {
    const int t = tid / kGroups + k * (kMixThreads / kGroups);
    const int y = y0 + t / kTileX, x = x0 + t % kTileX;
    gate_ok[k] = live && y < grid_h && x < grid_w;
    gate[k] = load4(u + (gate_ok[k] ? (image_base + (size_t)y * grid_w + x) * ld + c : 0));
  }
  const int cl = live ? c : 0;
  f4 w[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) w[k] = load4(conv_w + (size_t)k * F + cl);
  f4 bias = load4((conv_b ? conv_b : conv_w) + cl);  // unconditional as well; no bias: zero
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  if (!conv_b) bias = zero;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    if (!staged_ok[k]) staged[k] = zero;
#pragma unroll
  for (int k = 0; k < kTokensPerThread; ++k)
    if (!gate_ok[k]) gate[k] = zero;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    if (tid + k * kMixThreads < kStaged) val[tid + k * kMixThreads] = staged[k];
  __syncthreads();
  if (!live) return;
#pragma unroll
  for (int k = 0; k < kTokensPerThread; ++k) {
    const int t = tid / kGroups + k * (kMixThreads / kGroups);
    const int ty = t / kTileX, tx = t - ty * kTileX;
    const int y = y0 + ty, x = x0 + tx;
    if (y >= grid_h || x >= grid_w) continue;
    f4 acc = bias;
#pragma unroll
    for (int dy = 0; dy < 3; ++dy)
#pragma unroll
      for (int dx = 0; dx < 3; ++dx)
        acc += w[dy * 3 + dx] * val[((ty + dy) * kHaloX + tx + dx) * kGroups + j];
    f4 sg;
#pragma unroll
    for (int e = 0; e < 4; ++e) sg[e] = gate[k][e] / (1.f + __expf(-gate[k][e]));  // SiLU; -inf gives -0
    store4(h + (image_base + (size_t)y * grid_w + x) * F + c, sg * acc);
  }
}

template <typename T, typename U, typename H>
int launch_mix(const void *u_ws, const void *conv_w, const void *conv_b, void *h, int B, int grid_h,
               int grid_w, int F, hipStream_t stream) {
  const U *u = static_cast<const U *>(u_ws);
  auto kernel = swiglu_mix<T, U, H>;
  const int slices = (F + kSlice - 1) / kSlice;
  const int tiles_x = (grid_w + kTileX - 1) / kTileX, tiles_y = (grid_h + kTileY - 1) / kTileY;
  const dim3 grid((unsigned)((long long)B * tiles_y * tiles_x * slices));  // < 2^31 (checked on the host)
  hipEvent_t t0, t1;
  if (profile_events(kKernelSwigluMix, stream, &t0, &t1))
    hipExtLaunchKernelGGL(kernel, grid, dim3(kMixThreads), 0, stream, t0, t1, 0, u,
                          static_cast<const T *>(conv_w), static_cast<const T *>(conv_b),
                          static_cast<H *>(h), grid_h, grid_w, F, slices, tiles_x, tiles_y);
  else
    hipLaunchKernelGGL(kernel, grid, dim3(kMixThreads), 0, stream, u, static_cast<const T *>(conv_w),
                       static_cast<const T *>(conv_b), static_cast<H *>(h), grid_h, grid_w, F, slices,
                       tiles_x, tiles_y);
  return (int)hipGetLastError();
}

// Elementwise format changes around the bf16 output projection, four
// elements per thread (n is a multiple of 8): bf16 -> fp16 (exact for
// magnitudes from 2^-17 to 65504) and fp32 -> bf16 (round to nearest even).
constexpr int kConvThreads = 256;
__global__ __launch_bounds__(kConvThreads) void bf16_to_f16(const uint16_t *__restrict__ src,
                                                             _Float16 *__restrict__ dst, long long n4) {
  for (long long i = blockIdx.x * (long long)kConvThreads + threadIdx.x; i < n4;
       i += (long long)gridDim.x * kConvThreads)
    store4(dst + 4 * i, load4(src + 4 * i));
}
__global__ __launch_bounds__(kConvThreads) void f32_to_bf16(const float *__restrict__ src,
                                                             uint16_t *__restrict__ dst, long long n4) {
  for (long long i = blockIdx.x * (long long)kConvThreads + threadIdx.x; i < n4;
       i += (long long)gridDim.x * kConvThreads)
    store4(dst + 4 * i, load4(src + 4 * i));
}
template <typename K, typename S, typename D>
int launch_convert(K kernel, const S *src, D *dst, long long n, hipStream_t stream) {
  const long long n4 = n / 4;
  const unsigned blocks = (unsigned)std::min<long long>(4096, (n4 + kConvThreads - 1) / kConvThreads);
  if (blocks == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kConvThreads), 0, stream, src, dst, n4);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------ host side

constexpr long long kMaxTokens = 1LL << 24;
constexpr int kMaxWidth = 1 << 16;

int elem_bytes(int dtype) { return dtype == GTR_DTYPE_F32 ? 4 : 2; }
// u keeps the I/O precision for fp16 (one more fp16 rounding, well inside the
// fp16 tolerance) and fp32 otherwise (bf16 has no precision to spare).
int u_bytes_per_elem(int dtype) { return dtype == GTR_DTYPE_F16 ? 2 : 4; }
// h is fp16 for bf16 I/O: a bf16 h would add a rounding of 2^-9 that the
// output projection passes on at about unit gain.
int h_bytes_per_elem(int dtype) { return dtype == GTR_DTYPE_F32 ? 4 : 2; }

rocblas_datatype blas_type(int dtype) {
  return dtype == GTR_DTYPE_F32 ? rocblas_datatype_f32_r
                                : (dtype == GTR_DTYPE_F16 ? rocblas_datatype_f16_r : rocblas_datatype_bf16_r);
}

struct Sizes {
  long long tokens;
  size_t u_bytes, h_bytes;  // workspace parts, each rounded up to 256 bytes
  size_t out32_bytes;       // bf16 I/O: the fp32 output and fp16 W_out, in u's part once u is read
};

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

int validate(int B, int grid_h, int grid_w, int C, int F, int dtype, Sizes *sz) {
  if (dtype < 0 || dtype > 2) return set_error(GTR_ERR_INVALID_ARG, "dtype %d not in 0..2", dtype);
  if (B < 0 || grid_h < 0 || grid_w < 0)
    return set_error(GTR_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d grid=%dx%d)", B, grid_h, grid_w);
  if (C < 8 || F < 8 || C % 8 || F % 8 || C > kMaxWidth || F > kMaxWidth)
    return set_error(GTR_ERR_UNSUPPORTED, "C=%d F=%d: widths must be multiples of 8 from 8 to %d", C,
                     F, kMaxWidth);
  const long long tokens = (long long)B * grid_h * grid_w;
  if (tokens > kMaxTokens)
    return set_error(GTR_ERR_INVALID_ARG, "%lld tokens exceed 2^24", tokens);
  const long long blocks = (long long)B * ((grid_h + kTileY - 1) / kTileY) *
                           ((grid_w + kTileX - 1) / kTileX) * ((F + kSlice - 1) / kSlice);
  if (blocks >= (1LL << 31))
    return set_error(GTR_ERR_INVALID_ARG, "%lld workgroups of %dx%d tokens exceed 2^31", blocks, kTileY,
                     kTileX);
  sz->tokens = tokens;
  sz->u_bytes = round256((size_t)tokens * 2 * F * u_bytes_per_elem(dtype));
  sz->h_bytes = round256((size_t)tokens * F * h_bytes_per_elem(dtype));
  sz->out32_bytes = 0;
  if (dtype == GTR_DTYPE_BF16) {
    sz->out32_bytes = round256((size_t)tokens * C * sizeof(float));
    sz->u_bytes = std::max(sz->u_bytes, sz->out32_bytes + round256((size_t)F * C * sizeof(_Float16)));
  }
  return GTR_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

std::mutex g_mu;  // guards the rocBLAS handles (one per device)
std::map<int, rocblas_handle> g_blas;

int blas_handle(int device, rocblas_handle *h) {
  auto it = g_blas.find(device);
  if (it != g_blas.end()) {
    *h = it->second;
    return GTR_OK;
  }
  rocblas_handle nh = nullptr;
  if (rocblas_create_handle(&nh) != rocblas_status_success)
    return set_error(GTR_ERR_ALLOC, "rocblas_create_handle failed on device %d", device);
  g_blas[device] = nh;
  *h = nh;
  return GTR_OK;
}

// Row-major C[rows][n] = A[rows][k] B[k][n], as the column-major product
// C^T = B^T A^T that rocBLAS computes.
int gemm(rocblas_handle h, int rows, int n, int k, const void *a, rocblas_datatype at, const void *b,
         rocblas_datatype bt, void *c, rocblas_datatype ct, const char *what) {
  const float one = 1.f, zero = 0.f;
  const rocblas_status st =
      rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, n, rows, k, &one, b, bt, n, a,
                      at, k, &zero, c, ct, n, c, ct, n, rocblas_datatype_f32_r,
                      rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success)
    return set_error(GTR_ERR_LAUNCH, "%s: rocblas_gemm_ex failed (%s)", what, rocblas_status_to_string(st));
  return GTR_OK;
}

}  // namespace
}  // namespace gtr

extern "C" {

size_t gtr_swiglu_workspace_bytes(int B, int grid_h, int grid_w, int C, int F, int dtype) {
  gtr::Sizes sz;
  if (gtr::validate(B, grid_h, grid_w, C, F, dtype, &sz) != GTR_OK || sz.tokens == 0) return 0;
  return sz.u_bytes + sz.h_bytes;
}

int gtr_swiglu_fwd(const void *x, const void *w_in, const void *conv_w, const void *conv_b,
                   const void *w_out, void *out, int B, int grid_h, int grid_w, int C, int F,
                   int dtype, hipStream_t stream) {
  using namespace gtr;
  clear_error();
  Sizes sz;
  int rc = validate(B, grid_h, grid_w, C, F, dtype, &sz);
  if (rc != GTR_OK) return rc;
  if (sz.tokens == 0) return GTR_OK;  // nothing to compute
  if (!x || !w_in || !conv_w || !w_out || !out)
    return set_error(GTR_ERR_INVALID_ARG, "null pointer (x=%p w_in=%p conv_w=%p w_out=%p out=%p)", x,
                     w_in, conv_w, w_out, out);
  const size_t e = elem_bytes(dtype);
  const void *ptrs[6] = {x, w_in, conv_w, conv_b, w_out, out};
  const char *names[6] = {"x", "w_in", "conv_w", "conv_b", "w_out", "out"};
  const size_t bytes[6] = {(size_t)sz.tokens * C * e, (size_t)C * 2 * F * e, (size_t)9 * F * e,
                           (size_t)F * e, (size_t)F * C * e, (size_t)sz.tokens * C * e};
  for (int i = 0; i < 6; ++i)
    if (ptrs[i] && (reinterpret_cast<uintptr_t>(ptrs[i]) & 15u))
      return set_error(GTR_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
  for (int i = 0; i < 5; ++i)
    if (ptrs[i] && overlaps(out, bytes[5], ptrs[i], bytes[i]))
      return set_error(GTR_ERR_ALIAS, "out overlaps %s", names[i]);
  int n_dev = 0, device = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev <= 0 || hipGetDevice(&device) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(GTR_ERR_NO_DEVICE, "no HIP device available");
  }
  const bool capturing = stream_capturing(stream);
  if (!capturing && !pointer_checks_off()) {
    for (int i = 0; i < 6; ++i) {
      if (!ptrs[i]) continue;
      rc = check_device_pointer(ptrs[i], bytes[i], device, names[i]);
      if (rc != GTR_OK) return rc;
    }
  }

  std::lock_guard<std::mutex> lock(g_mu);
  void *ws = nullptr;
  rc = stream_buffer(kBufSwiglu, device, stream, sz.u_bytes + sz.h_bytes, "Spatial SwiGLU", &ws);
  if (rc != GTR_OK) return rc;
  rocblas_handle blas = nullptr;
  rc = blas_handle(device, &blas);
  if (rc != GTR_OK) return rc;
  if (rocblas_set_stream(blas, stream) != rocblas_status_success)
    return set_error(GTR_ERR_LAUNCH, "rocblas_set_stream failed");
  void *u = ws;
  void *h = static_cast<char *>(ws) + sz.u_bytes;
  const rocblas_datatype t = blas_type(dtype);
  const int M = (int)sz.tokens;
  {
    ProfileScope scope(kKernelSwigluIn, stream);
    rc = gemm(blas, M, 2 * F, C, x, t, w_in, t, u,
              dtype == GTR_DTYPE_F16 ? rocblas_datatype_f16_r : rocblas_datatype_f32_r, "input projection");
  }
  if (rc != GTR_OK) return rc;
  int err;
  switch (dtype) {
    case GTR_DTYPE_F32: err = launch_mix<float, float, float>(u, conv_w, conv_b, h, B, grid_h, grid_w, F, stream); break;
    case GTR_DTYPE_F16: err = launch_mix<_Float16, _Float16, _Float16>(u, conv_w, conv_b, h, B, grid_h, grid_w, F, stream); break;
    default: err = launch_mix<uint16_t, float, _Float16>(u, conv_w, conv_b, h, B, grid_h, grid_w, F, stream); break;
  }
  if (err != (int)hipSuccess)
    return set_error(GTR_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
  if (dtype != GTR_DTYPE_BF16) {
    ProfileScope scope(kKernelSwigluOut, stream);
    return gemm(blas, M, C, F, h, t, w_out, t, out, t, "output projection");
  }
  // bf16: fp16 operands (h as the mix wrote it, W_out converted) into an fp32
  // product, rounded once to bf16; u has been read, so its part holds both
  float *out32 = static_cast<float *>(u);
  _Float16 *w16 = reinterpret_cast<_Float16 *>(static_cast<char *>(u) + sz.out32_bytes);
  {
    ProfileScope scope(kKernelSwigluOut, stream);
    err = launch_convert(bf16_to_f16, static_cast<const uint16_t *>(w_out), w16, (long long)F * C, stream);
    if (err != (int)hipSuccess)
      return set_error(GTR_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
    rc = gemm(blas, M, C, F, h, rocblas_datatype_f16_r, w16, rocblas_datatype_f16_r, out32,
              rocblas_datatype_f32_r, "output projection");
    if (rc != GTR_OK) return rc;
    err = launch_convert(f32_to_bf16, out32, static_cast<uint16_t *>(out), (long long)sz.tokens * C, stream);
  }
  if (err != (int)hipSuccess)
    return set_error(GTR_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)err));
  return GTR_OK;
}

}  // extern "C"
