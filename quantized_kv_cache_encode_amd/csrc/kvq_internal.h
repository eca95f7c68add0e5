// Internal declarations shared by the host API and the kernel translation units
// of libkvq.  Not installed; the public interface is include/kvq.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kvq {

// Threads of a read-path workgroup (8 waves of 64): one workgroup per compute unit
// keeps two waves on each SIMD.
constexpr int kReadThreads = 512;

// Everything a read-path kernel needs, passed by value as the kernel argument.
struct AttnParams {
  const void* q;             // [B][Hq][D] fp16 or fp32
  const uint8_t* codes;      // [B][Hkv][T_cap][bytes per key]
  const float* norms;        // [B][Hkv][T_cap] (Hadamard/Lloyd-Max only)
  const void* v;             // [B][Hkv][T_cap][D] fp16 or fp32
  const int32_t* seq_lens;   // [B] or nullptr (= T_cap)
  const float* pq_cent;      // [Hkv][M][K][D/M] (PQ only)
  float* scores;             // score kernel output [B][Hq][T_cap]
  float* ws;                 // split partials [B][Hq][n_splits][D+2]
  unsigned* counters;        // [units] arrival counters of the split merge (zero between calls)
  void* out;                 // [B][Hq][D] fp16 or fp32
  int64_t T_cap;
  int64_t split_len;         // tokens per split (multiple of 64)
  int B, Hq, Hkv, G;         // G = Hq / Hkv
  int n_groups;              // G / heads-per-workgroup
  int n_splits;
  int q_f16, out_f16;
  int pq_K;
  float zscale;              // softmax scale * log2(e)
  float levels[16];
  uint32_t signs[8];         // bit i set <=> coordinate i is negated
  // fused append (Hadamard/Lloyd-Max only): one new key per (b, kv head) stored at position len-1 and
  // attended in the same call; new_keys == nullptr disables it
  const void* new_keys;      // [B][Hkv][D] fp16 or fp32
  uint8_t* app_codes;        // the code cache, written at the new rows (same buffer as codes)
  float* app_norms;          // the norm cache, written at the new rows (same buffer as norms)
  int new_f16;
  int pot_mant;              // power-of-two codec: the mantissa term is on (fused append)
  float thresholds[15];
  // values as codes of the same codec (kvq_decode_attn_qv): [B][Hkv][T_cap][bytes per key] and norms
  const uint8_t* vcodes;
  const float* vnorms;
  int waves;                 // decode workgroup size in waves: 8, or 12 (chosen by the host with the splits)
};

struct EncodeParams {
  const void* keys;          // [B][Hkv][T_new][D]
  uint8_t* codes;            // [B][Hkv][T_cap][bytes per key]
  float* norms;              // [B][Hkv][T_cap]
  const int32_t* write_pos;  // [B] or nullptr
  const float* pq_cent;      // PQ only
  int64_t T_new, T_cap, t0;
  int B, Hkv;
  int pq_K;
  float thresholds[15];
  uint32_t signs[8];
  // cell search of the Hadamard/Lloyd-Max encode: y (|y| <= 1) falls in cell floor(y * cell_inv +
  // cell_shift) of n_cells; every threshold sits at least 7% of a cell away from a cell boundary, no cell
  // holds two, and cell_shift is a multiple of 1/8 (choose_encode_cells)
  int n_cells;
  float cell_inv, cell_shift;
  int64_t key_begin, key_end;  // the keys [key_begin, key_end) of [B*Hkv*T_new] this launch encodes
  int64_t keys_per_block;      // the contiguous keys each workgroup encodes (Hadamard and power-of-two)
  int rows_whole;              // T_new == T_cap, t0 == 0 and no write_pos: key i of the launch goes to row i
  int pot_mant;                // power-of-two codec: the mantissa term is on
  uint32_t tnew_magic, hkv_magic;  // n / T_new and n / Hkv for n < 2^31: (umulhi(n, magic) + n) >> shift
  int tnew_shift, hkv_shift;
};

// Magic number and shift for division by d >= 1 of any n < 2^31 (round-up method).
inline void fast_div_magic(uint32_t d, uint32_t* magic, int* shift) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  *shift = l;
  *magic = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
  if (d == 1) *magic = 0;
}

constexpr int kEncodeMaxCells = 1024;

// Kernel launchers.  Each returns hipSuccess or the launch error; an
// unsupported template combination returns hipErrorNotSupported without
// launching.  heads_per_wg is the number of query heads one workgroup serves.
hipError_t launch_hlm_decode(int D, int bits, int heads_per_wg, bool v_f16, const AttnParams& p, dim3 grid,
                             hipStream_t s);
hipError_t launch_hlm_score(int D, int bits, int heads_per_wg, const AttnParams& p, dim3 grid, hipStream_t s);
hipError_t launch_hlm_decode_qv(int D, int bits, int heads_per_wg, const AttnParams& p, dim3 grid, hipStream_t s);
// PQ launchers take the code width cb: 8 (one byte per subspace) or 4 (two subspaces per byte).
hipError_t launch_pq_decode(int D, int M, int cb, int heads_per_wg, bool v_f16, const AttnParams& p, dim3 grid,
                            hipStream_t s);
hipError_t launch_pq_score(int D, int M, int cb, int heads_per_wg, const AttnParams& p, dim3 grid, hipStream_t s);
hipError_t launch_hlm_encode(int D, int bits, bool k_f16, const EncodeParams& p, hipStream_t s);
hipError_t launch_pot_decode(int D, int bits, int heads_per_wg, bool v_f16, const AttnParams& p, dim3 grid,
                             hipStream_t s);
hipError_t launch_pot_score(int D, int bits, int heads_per_wg, const AttnParams& p, dim3 grid, hipStream_t s);
hipError_t launch_pot_encode(int D, int bits, bool k_f16, const EncodeParams& p, hipStream_t s);
hipError_t launch_pq_encode(int D, int M, int cb, bool k_f16, const EncodeParams& p, hipStream_t s);

// Exact attention over calibration samples (sign-pattern selection).
constexpr int kCalibMaxT = 8192;  // keys per calibration sample (scores held in LDS)
struct CalibParams {
  const void* q;     // [n][Hq][D]
  const void* keys;  // [n][Hkv][T][D]
  const void* v;     // [n][Hkv][T][D]
  float* out;        // [n][Hq][D] fp32
  int n, Hq, Hkv, T;
  int q_f16, k_f16, v_f16;
  float scale;
};
hipError_t launch_exact_attn(int D, const CalibParams& p, hipStream_t s);
hipError_t launch_rel_err(const float* oh, const float* o, int64_t n, float* errors, int c, hipStream_t s);
hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t s);

// Sets the calling thread's kvq_last_error() message and returns `status` (a kvq_status).
int set_error(int status, const char* msg);

// Cell grid for the encode's threshold search (codebook.cpp); false if none fits kEncodeMaxCells.
bool choose_encode_cells(const float* thresholds, int n_thresholds, int* n_cells, float* cell_inv, float* cell_shift);

// Host codebook construction (codebook.cpp).
void lloyd_max_gaussian(int b, double* levels, double* thresholds);
void kmeans_lloyd(const float* train, int64_t n, int dim, int stride, int K, int iters, const int64_t* start,
                  double* cent);

}  // namespace kvq
