// Scan-direction index map of the GLA kernels: scan position t -> grid cell,
// for the four orders of the x-techcon article on GTR (section 架构 /
// Architecture: left-to-right, right-to-left, top-to-bottom, bottom-to-top;
// gtr_gla.h gives the formulas).  Applied to load and store addresses, so no
// permuted copy of any tensor is made.
//
// The functions take any struct M with the fields n_tok, gh, gw (grid
// height and width), dir (0..3) and rcp_gh (1.0f / gh, rounded to float):
// the kernels pass their per-sequence descriptor, and host code (the index
// tests) a plain struct with the same fields.  They are compiled for both.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gtr {

constexpr uint32_t kNoRow = 0xffffffffu;  // grid cell of a scan position past the end

// Column-major position p -> (row, col) with grid height gh: p / gh from a
// float reciprocal, then one exact correction step.  p < 2^23, so float(p) is
// exact, and the float quotient is off from the true one by at most one.
__host__ __device__ __forceinline__ void col_major_pos(int p, int gh, float rcp_gh, int &row, int &col) {
  col = (int)((float)p * rcp_gh);
  row = p - col * gh;
  if (row < 0) {
    --col;
    row += gh;
  } else if (row >= gh) {
    ++col;
    row -= gh;
  }
}

// Grid cell of scan position t (t < n_tok).
template <class M> __host__ __device__ __forceinline__ uint32_t token_cell(const M &m, int t) {
  const int p = (m.dir & 1) ? m.n_tok - 1 - t : t;
  if (!(m.dir & 2)) return (uint32_t)p;
  int row, col;
  col_major_pos(p, m.gh, m.rcp_gh, row, col);
  return (uint32_t)(row * m.gw + col);
}

// Grid cells of scan positions t0 .. t0+3 (kNoRow past the end) and, with
// kBefore, of t0 - 1 (kNoRow before the start).  Consecutive scan positions
// step by one grid cell along the scan, so only the first needs a division.
template <bool kBefore, class M>
__host__ __device__ __forceinline__ void cells4(const M &m, int t0, uint32_t *cell, uint32_t &before) {
  const bool rev = m.dir & 1;
  const int p0 = rev ? m.n_tok - 1 - t0 : t0;
  if (!(m.dir & 2)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = rev ? p0 - r : p0 + r;
      cell[r] = t0 + r < m.n_tok ? (uint32_t)p : kNoRow;
    }
    if constexpr (kBefore) before = t0 > 0 && t0 <= m.n_tok ? (uint32_t)(rev ? p0 + 1 : p0 - 1) : kNoRow;
    return;
  }
  int row, col;
  col_major_pos(p0, m.gh, m.rcp_gh, row, col);
  if constexpr (kBefore) {  // one step back along the scan
    int br = row, bc = col;
    if (rev) {
      if (++br == m.gh) {
        br = 0;
        ++bc;
      }
    } else if (--br < 0) {
      br = m.gh - 1;
      --bc;
    }
    before = t0 > 0 && t0 <= m.n_tok ? (uint32_t)(br * m.gw + bc) : kNoRow;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    cell[r] = t0 + r < m.n_tok ? (uint32_t)(row * m.gw + col) : kNoRow;
    if (rev) {
      if (--row < 0) {
        row = m.gh - 1;
        --col;
      }
    } else if (++row == m.gh) {
      row = 0;
      ++col;
    }
  }
}

}  // namespace gtr
