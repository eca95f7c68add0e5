// Host-side codebook construction for libkvq.
//
// Lloyd-Max scalar codebook for N(0,1/d) ("AXELRAM: Quantize Once, Never
// Dequantize", Abstract: the optimal quantizer depends only on d and b once
// the orthogonal transform has made every coordinate N(0,1/d)) and Lloyd
// k-means for product-quantization codebooks ("LOOKAT" summary page, AI
// Summary: codebook learning per subspace).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr double kInvSqrt2Pi = 0.39894228040143267794;  // 1/sqrt(2*pi)
constexpr double kInvSqrt2 = 0.70710678118654752440;

inline double gauss_density(double x) { return std::isinf(x) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * x * x); }
// Upper tail probability P(X >= x) of the standard normal.
inline double gauss_tail(double x) { return 0.5 * std::erfc(x * kInvSqrt2); }

}  // namespace

// The density is even, so the optimal quantizer is odd-symmetric: work on the
// positive half only.  With L = 2^b levels there are H = L/2 positive levels
// y_1 < ... < y_H and cell edges 0 = e_0 < e_1 < ... < e_H = +inf.  Alternate
// (a) edges at midpoints of neighbouring levels and (b) levels at the
// conditional means E[X | e_{k-1} <= X < e_k] = (phi(e_{k-1}) - phi(e_k)) /
// (Q(e_{k-1}) - Q(e_k)) until the levels stop moving.
void lloyd_max_gaussian(int b, double* levels, double* thresholds) {
  const int L = 1 << b;
  const int H = L / 2;
  std::vector<double> y(H), e(H + 1);
  for (int k = 0; k < H; ++k) y[k] = 2.5 * (k + 0.5) / H;
  for (int iter = 0; iter < 1000000; ++iter) {
    e[0] = 0.0;
    for (int k = 1; k < H; ++k) e[k] = 0.5 * (y[k - 1] + y[k]);
    e[H] = INFINITY;
    double moved = 0.0;
    for (int k = 0; k < H; ++k) {
      const double mass = gauss_tail(e[k]) - gauss_tail(e[k + 1]);
      const double mean = (gauss_density(e[k]) - gauss_density(e[k + 1])) / mass;
      moved = std::fmax(moved, std::fabs(mean - y[k]));
      y[k] = mean;
    }
    if (moved < 1e-15) break;
  }
  for (int k = 0; k < H; ++k) {
    levels[H + k] = y[k];
    levels[H - 1 - k] = -y[k];
  }
  for (int j = 0; j + 1 < L; ++j) thresholds[j] = 0.5 * (levels[j] + levels[j + 1]);
  thresholds[H - 1] = 0.0;
}

// Lloyd k-means in double precision on n vectors of `dim` floats found at
// train[r * stride + 0 .. dim).  start[c] is the training row that seeds
// centroid c.  Assignment: smallest squared distance, lowest index on ties.
// Update: member mean; a centroid without members keeps its position.
void kmeans_lloyd(const float* train, int64_t n, int dim, int stride, int K, int iters, const int64_t* start,
                  double* cent) {
  for (int c = 0; c < K; ++c)
    for (int k = 0; k < dim; ++k) cent[c * dim + k] = train[start[c] * stride + k];
  std::vector<int> owner(n);
  std::vector<double> acc((size_t)K * dim);
  std::vector<int64_t> members(K);
  for (int it = 0; it < iters; ++it) {
    for (int64_t r = 0; r < n; ++r) {
      const float* x = train + r * stride;
      int best = 0;
      double best_d = INFINITY;
      for (int c = 0; c < K; ++c) {
        double dist = 0.0;
        for (int k = 0; k < dim; ++k) {
          const double diff = (double)x[k] - cent[c * dim + k];
          dist += diff * diff;
        }
        if (dist < best_d) {
          best_d = dist;
          best = c;
        }
      }
      owner[r] = best;
    }
    std::fill(acc.begin(), acc.end(), 0.0);
    std::fill(members.begin(), members.end(), 0);
    for (int64_t r = 0; r < n; ++r) {
      members[owner[r]]++;
      for (int k = 0; k < dim; ++k) acc[(size_t)owner[r] * dim + k] += train[r * stride + k];
    }
    for (int c = 0; c < K; ++c)
      if (members[c] > 0)
        for (int k = 0; k < dim; ++k) cent[c * dim + k] = acc[(size_t)c * dim + k] / (double)members[c];
  }
}

// Grid of equal cells over y in [-1, 1] for the encode kernel's threshold search: code(y) = (thresholds
// in cells below y's cell) + (y >= the threshold inside y's cell, if any).  That is exact as long as no
// cell holds two thresholds and no threshold lies within the rounding of y's cell index of a cell
// boundary; the grid is chosen so that every threshold sits in [7%, 93%] of its cell, computed with the
// same fp32 fused multiply-add the kernel uses.  The kernel finds y's cell through y * inv + shift + 2^20,
// whose float spacing (1/8) moves it by at most 1/16 of a cell; the shift is a multiple of 1/8, so that
// adding 2^20 to it is exact.
bool choose_encode_cells(const float* t, int n, int* n_cells, float* cell_inv, float* cell_shift) {
  double min_gap = 1.0;
  for (int j = 0; j + 1 < n; ++j) min_gap = std::min(min_gap, (double)t[j + 1] - (double)t[j]);
  double w = std::max(min_gap / 3.0, 2.0005 / (kEncodeMaxCells - 4));
  for (int iter = 0; iter < 400; ++iter, w *= 0.997) {
    const float inv = (float)(1.0 / w);
    const int off = (int)std::ceil(1.0001 * (double)inv) + 1;
    const int cells = 2 * off + 1;
    if (cells > kEncodeMaxCells) return false;
    for (int k = 0; k < 4; ++k) {
      const float shift = (float)off + 0.5f + 0.125f * (float)k;  // a multiple of 1/8
      bool good = true;
      double prev_cell = -1e30;
      for (int j = 0; j < n && good; ++j) {
        const float v = std::fmaf(t[j], inv, shift);
        const double fr = (double)v - std::floor((double)v);
        if (fr < 0.07 || fr > 0.93 || std::floor((double)v) == prev_cell) good = false;
        prev_cell = std::floor((double)v);
      }
      if (good) {
        *n_cells = cells;
        *cell_inv = inv;
        *cell_shift = shift;
        return true;
      }
    }
  }
  return false;
}

}  // namespace kvq
