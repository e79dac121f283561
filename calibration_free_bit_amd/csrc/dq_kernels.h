// dq_kernels.h -- launch interface between the C ABI (dq_api.hip) and the
// kernels (dq_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

constexpr int kTileCols = 64;   // columns of one independent tile
constexpr int kRowsPerStep = 64;  // rows of one BCD pass workgroup step
constexpr int kPassGrid = 512;  // target workgroups of one BCD pass (two per CU)
constexpr int kXcds = 8;        // dies; workgroups are dispatched to them in turn

// Geometry of one BCD pass. Work is the flattened list of (tile, row step)
// pairs, tile-major; workgroup w owns steps [w L, (w+1) L). The workgroups
// that touch tile t are floor(t S / L) .. floor(((t+1) S - 1) / L); each
// writes one partial (segment) per column of t.
struct PassGeom {
  int64_t ldw, M, N;
  int64_t S;        // row steps per tile
  int64_t n_tiles;  // column tiles
  int64_t total;    // n_tiles * S
  int64_t L;        // row steps per workgroup
  int64_t n_wg;     // workgroups launched
  int64_t max_seg;  // most segments any tile has
};
// Workspace: two alternating [n_tiles][max_seg][64][2] float64 buffers of
// column partial sums, then (for some shapes) the passes' tile-major copy of
// the block scales.

// Rows per chunk of the column-norm initialization's partial sums: 256, or
// more when the chunk count would exceed the grid's y limit (65535). Its
// workspace holds [n_tiles][chunks][64] float64, chunks <= ceil(M / 256).
constexpr int kColnormRows = 256;
inline int64_t colnorm_chunk_rows(int64_t M) {
  const int64_t per = (M + 65534) / 65535;  // rows per chunk so that chunks <= 65535
  return per <= kColnormRows ? kColnormRows : (per + 3) / 4 * 4;
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_init_colnorm(const void* W, int64_t ldw, int64_t M, int64_t N, void* a, uint16_t* b,
                               double* part, hipStream_t st);

// Rows per thread of the packing / report kernel, and the report kernel's
// workgroups (256 threads; one float64 triple each in the workspace).
constexpr int kPackRows = 4;
inline int64_t report_workgroups(int64_t M, int64_t N) {
  return (((M + kPackRows - 1) / kPackRows) * (N / 16) + 255) / 256;
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_report(const void* W, int64_t ldw, int64_t M, int64_t N, const void* a,
                         const uint16_t* b, const uint8_t* prev, uint8_t* packed, double* report,
                         double* part, hipStream_t st);

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_init(const void* W, int64_t ldw, int64_t M, int64_t N, void* a, uint16_t* b,
                       hipStream_t st);

// Per-iteration statistics of dq_bcd_iterate: out [n_iters + 1][3] receives,
// for the state after k iterations, sum (W - a Q b)^2, sum W^2 and the codes
// changed since state k - 1 (0 for k = 0). codes holds [M][N * bits / 8]
// state codes; part holds the per-workgroup sums (n_wg and the report
// kernel's workgroups, 3 float64 each).
struct IterStats {
  double* out;
  uint8_t* codes;
  double* part;
};

// n_iters BCD passes and the final column update; with from_init (and no
// stats) the first pass starts from the absmax initialization it forms
// itself, so a and b need not hold a state on entry. With a_work (no
// stats), the passes keep the block scales there in the tile-major layout
// [n_tiles][M][64 / G], copied from a first (unless from_init) and back to
// a at the end; a_work holds tile_major_a_bytes.
template <int WT, int GRID, int AFMT, int G>
hipError_t launch_iterate(const void* W, void* a, uint16_t* b, double* part, const PassGeom& g,
                          int n_iters, const IterStats* stats, bool from_init, void* a_work,
                          hipStream_t st);

// Bytes of the tile-major copy of the block scales (elements of 1 or 2 bytes).
inline int64_t tile_major_a_bytes(const PassGeom& g, int group, int scale_bytes) {
  return g.n_tiles * g.M * (kTileCols / group) * scale_bytes;
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_pack(const void* W, int64_t ldw, int64_t M, int64_t N, const void* a,
                       const uint16_t* b, uint8_t* packed, hipStream_t st);

template <int GRID, int AFMT, int G>
hipError_t launch_act(const uint16_t* X, int64_t ldx, int64_t T, int64_t N, const uint16_t* b,
                      uint8_t* xq, void* xs, hipStream_t st);

}  // namespace dq
