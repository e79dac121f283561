// dq_kernels.hip -- HIP kernels of the DualQuant solver for gfx950 (MI355X).
//
// One BCD iteration ("DualQuant" reproduction README, "Core equations" and
// its flowchart; paper summary §4.3, App. A-B) is ONE pass over W:
//
//   for every (row i, block g):  Q1 = q(W/(a b))          (codes of the state)
//                                a' = Pi(sum W R / sum R^2), R = Q1 D_b
//                                Q2 = q(W/(a' b))          (requantize)
//   for every column j:          b' = Pi(sum W S / sum S^2), S = D_a' Q2
//
// The row/block update only needs the G columns of its block and the column
// update only needs a' of the same column stripe, so the problem splits into
// independent 64-column tiles spanning all rows. A workgroup streams a range
// of row steps of a tile: every lane owns LC (16 or 8) contiguous columns of
// one row, keeps those elements in registers between the two requantizations,
// and accumulates float64 column sums for its columns across the rows it
// visits. At the end of its range the workgroup reduces those sums through
// LDS and writes one partial per column. The column update b' is formed by
// the NEXT pass: each of its workgroups adds the partials of its tile in a
// fixed order (the kernel boundary makes them visible; no fences or
// atomics), and a small kernel writes b after the last pass. Partials
// alternate between two buffers so a pass never overwrites what it reads.
// Q is never stored: it is recomputed from (W, a, b) whenever needed, so
// one iteration reads W once. Two variants of the pass add work to the same
// stream of rows: one measures the state it starts from (per-iteration
// statistics), one forms the absmax initialization itself (the first pass
// of a whole solve).
//
// Every sum of the least-squares updates is accumulated in float64 in a
// fixed order, so results are deterministic. Each product is exact (at most
// 26 significant bits), so a sum is exact as long as its terms span less
// than about 2^(27 - log2 of their count) in magnitude, which holds for
// ordinary weights; then the summation order does not matter at all.
#include <hip/hip_runtime.h>

#include <utility>

#include "dq_device.h"
#include "dq_kernels.h"

namespace dq {

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Re-decide exactly the element slots of N fast codes where some lane of
// the wave may differ from the exact rounding (after fast_n returned true
// in some lane). w: the weights, a: the block scale of each group of BL
// elements, b: the column scale of each element. Under kSlotMask the lanes
// whose ends differ are few (about one per flagged wave on the workloads):
// their difference words are OR-ed into scalar registers, so the slots are
// tested by scalar branches and only those where some lane differs are
// re-decided. Otherwise (or with MASK false) each slot is tested with a
// vector compare.
template <int GRID, int N, int BL, bool MASK = Grid<GRID>::kSlotMask>
__device__ __forceinline__ void redecide(const float* y, float* q, const uint32_t* diff, const uint32_t* hiw,
                                         const float* w, const float* a, const float* b) {
  using Gr = Grid<GRID>;
  if constexpr (MASK) {
    constexpr int ND = N / Gr::kPerWord;
    uint32_t mine = 0u;
#pragma unroll
    for (int d = 0; d < ND; ++d) mine |= diff[d];
    uint64_t lanes = __builtin_amdgcn_ballot_w64(mine != 0u);
    uint32_t D[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) D[d] = 0u;
    while (lanes != 0u) {
      const int l = __builtin_ctzll(lanes);
      lanes &= lanes - 1u;
#pragma unroll
      for (int d = 0; d < ND; ++d) D[d] |= (uint32_t)__builtin_amdgcn_readlane((int)diff[d], l);
    }
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (Gr::field(D, e) != 0u) {
        // the new code replaces q[e] in its own register (a tied operand),
        // so that the path without re-decisions needs no register copies
        const float r = Gr::resolve(q[e], hiw, e, w[e], a[e / BL], b[e]);
        asm("v_mov_b32 %0, %1" : "+v"(q[e]) : "v"(r));
      }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (wave_any(Gr::near(y, q, diff, e))) q[e] = Gr::exact(y[e], w[e], a[e / BL], b[e]);
  }
}

// The value of lane (lane ^ M) within each quad of lanes (M = 1 or 2), by a
// DPP quad permutation (VALU moves instead of an LDS round trip). Every
// source lane of a quad permutation exists, so bound_ctrl (zero for a
// missing source) never applies; setting it lets the compiler fold the
// float32 move into the add that consumes it. Called with every lane of
// the wave active.
template <int M>
__device__ __forceinline__ double quad_xor(double v) {
  static_assert(M == 1 || M == 2, "quad permutations");
  constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), kCtrl, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
template <int M>
__device__ __forceinline__ float quad_xor(float v) {
  static_assert(M == 1 || M == 2, "quad permutations");
  constexpr int kCtrl = M == 1 ? 0xB1 : 0x4E;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}
// The value of lane 7 - (lane & 7) within each group of 8 lanes (DPP
// row_half_mirror): pairs every lane of one quad with one of the other.
__device__ __forceinline__ float half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
}
__device__ __forceinline__ double half_mirror(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), 0x141, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), 0x141, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
// Largest v over the aligned group of K lanes (K = 1, 2, 4 or 8) holding
// this lane, for v >= 0 and not NaN (a block's absolute maximum, where the
// per-lane maxima already dropped NaN). Such floats order as their bit
// patterns, so each step is one unsigned max with the DPP move folded in
// (a float max would first quiet the moved value).
template <int K>
__device__ __forceinline__ float max_join(float v) {
  static_assert(K == 1 || K == 2 || K == 4 || K == 8, "groups of 1, 2, 4 or 8 lanes");
  uint32_t u = __float_as_uint(v);
  if constexpr (K >= 2) u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  if constexpr (K >= 4) u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  if constexpr (K >= 8) u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));
  return __uint_as_float(u);
}

// Sum of v over the aligned group of K lanes (K = 1, 2, 4 or 8) holding
// this lane, in every lane of the group: pairs, then quads, then the two
// quads of a group of 8. The order of the additions is fixed.
template <int K, class T>
__device__ __forceinline__ T lane_join(T v) {
  static_assert(K == 1 || K == 2 || K == 4 || K == 8, "groups of 1, 2, 4 or 8 lanes");
  if constexpr (K >= 2) v += quad_xor<1>(v);
  if constexpr (K >= 4) v += quad_xor<2>(v);
  if constexpr (K >= 8) v += half_mirror(v);
  return v;
}

// ------------------------------------------------------------------ init

// One thread per (row, block): absmax -> a = Pi(absmax / qmax), 1 if zero.
template <int WT, int GRID, int AFMT, int G>
__global__ void __launch_bounds__(256) init_rtn_kernel(const void* __restrict__ W, int64_t ldw,
                                                       int64_t M, int64_t N, void* __restrict__ a_,
                                                       uint16_t* __restrict__ b) {
  using AT = typename ScaleStore<AFMT>::T;
  const int64_t nblk = N / G;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < M * nblk) {
    const int64_t row = idx / nblk, blk = idx - row * nblk;
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < G / 8; ++c) {
      float v[8];
      load8<WT>(W, row * ldw + blk * G + 8 * c, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[k]));
    }
    const double s = amax > 0.0f ? project<AFMT>((double)amax / (double)Grid<GRID>::qmax) : 1.0;
    reinterpret_cast<AT*>(a_)[idx] = encode_scale<AFMT>(s);
  }
  if (idx < N) b[idx] = 0x3C00u;  // fp16 1.0
}

// ------------------------------------------- column-norm initialization

// Partial column sums of |W| over chunks of chunk_rows rows, one workgroup
// per (tile, chunk). A lane owns 8 contiguous columns of every 32nd row of
// the chunk (kColnormUnroll rows loaded before any is added) and adds its
// rows in order; then the 32 row-lanes of each column are added in a fixed
// tree (four runs of 8 through LDS, then the four runs by DPP).
constexpr int kColnormUnroll = 8;
template <int WT>
__global__ void __launch_bounds__(256) colnorm_partial_kernel(const void* __restrict__ W, int64_t ldw,
                                                              int64_t M, int64_t N,
                                                              int64_t chunk_rows,
                                                              double* __restrict__ part) {
  constexpr int kRowLanes = 256 / (kTileCols / 8);  // 32
  __shared__ double s_sum[kRowLanes][kTileCols];
  const int c8 = threadIdx.x % (kTileCols / 8), rl = threadIdx.x / (kTileCols / 8);
  const int64_t tile = blockIdx.x, chunk = blockIdx.y;
  const int64_t col = tile * kTileCols + c8 * 8;
  const int64_t r0 = chunk * chunk_rows, r1 = min(r0 + chunk_rows, M);
  double acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0;
  if (col < N) {  // N is a multiple of 16: a lane's 8 columns are all in range or all out
    for (int64_t r = r0 + rl; r < r1; r += kRowLanes * kColnormUnroll) {
      float v[kColnormUnroll][8];
#pragma unroll
      for (int u = 0; u < kColnormUnroll; ++u) {
        const int64_t ru = min(r + (int64_t)kRowLanes * u, r1 - 1);  // rows past the chunk add 0
        load8<WT>(W, ru * ldw + col, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kColnormUnroll; ++u) {
        const bool in = r + (int64_t)kRowLanes * u < r1;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += in ? (double)__builtin_fabsf(v[u][k]) : 0.0;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) s_sum[rl][c8 * 8 + k] = acc[k];
  __syncthreads();
  const int c = threadIdx.x >> 2, quarter = threadIdx.x & 3;
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kRowLanes / 4; ++i) t += s_sum[quarter * (kRowLanes / 4) + i][c];
  t += quad_xor<1>(t);
  t += quad_xor<2>(t);
  if (quarter == 0) part[(tile * gridDim.y + chunk) * kTileCols + c] = t;
}

// b_j = Pi_fp16(sum_i |W_ij| / M), 1 for an all-zero column; the chunks are
// added in order, eight loads in flight at a time.
static __global__ void __launch_bounds__(kTileCols) colnorm_b_kernel(const double* __restrict__ part,
                                                              int64_t n_chunks, int64_t M, int64_t N,
                                                              uint16_t* __restrict__ b) {
  const int64_t tile = blockIdx.x, j = tile * kTileCols + threadIdx.x;
  if (j >= N) return;
  const double* __restrict__ pc = part + tile * n_chunks * kTileCols + threadIdx.x;
  double sum = 0.0;
  for (int64_t k0 = 0; k0 < n_chunks; k0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = k0 + u < n_chunks ? pc[(k0 + u) * kTileCols] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  const double bj = sum > 0.0 ? project<kScaleFp16>(sum / (double)M) : 1.0;
  b[j] = encode_scale<kScaleFp16>(bj);
}

// a = Pi_Fa(max_{j in block} |W_ij / b_j| / qmax), 1 for a zero block. One
// lane per 8 columns of kColnormRowsPerLane consecutive rows, G/8 lanes per
// block (joined by DPP). The quotients are first formed in float32 from
// 1-ulp reciprocals of b (relative error below 2^-22 after the division by
// qmax) and projected on the certified path, which brackets that error; a
// wave with any block it cannot certify recomputes its blocks from
// correctly rounded float64 quotients, as the definition reads.
constexpr int kColnormRowsPerLane = 4;
template <int WT, int GRID, int AFMT, int G>
__global__ void __launch_bounds__(256) colnorm_a_kernel(const void* __restrict__ W, int64_t ldw,
                                                        int64_t M, int64_t N,
                                                        const uint16_t* __restrict__ b,
                                                        void* __restrict__ a_) {
  using AT = typename ScaleStore<AFMT>::T;
  constexpr int R = kColnormRowsPerLane;
  constexpr int LPB = G / 8;  // lanes per block; a block never straddles a wave
  static_assert(LPB <= 8, "a block's lanes lie in one group of 8");
  const int64_t nch = N / 8;
  const int64_t n_rg = (M + R - 1) / R;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = idx < n_rg * nch;
  const int64_t cidx = live ? idx : 0;  // dead lanes compute on chunk 0
  const int64_t rg = cidx / nch, col = (cidx - rg * nch) * 8;
  float w[R][8];
#pragma unroll
  for (int u = 0; u < R; ++u) load8<WT>(W, min(rg * R + u, M - 1) * ldw + col, w[u]);
  float bf[8], rb[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    bf[k] = fp16_bits_to_float(b[col + k]);
    rb[k] = __builtin_amdgcn_rcpf(bf[k]);
  }
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int64_t r = rg * R + u;
    float wmax = 0.0f, ymax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float aw = __builtin_fabsf(w[u][k]);
      wmax = __builtin_fmaxf(wmax, aw);
      ymax = __builtin_fmaxf(ymax, aw * rb[k]);
    }
    wmax = max_join<LPB>(wmax);
    ymax = max_join<LPB>(ymax);
    // a zero block is exactly the case wmax == 0; a non-zero block whose
    // float32 quotients underflow is left to the certified path's range test
    bool unsure = false;
    float s = 1.0f;
    if (wmax > 0.0f) s = ls_scale_fast<AFMT>((double)ymax, (double)Grid<GRID>::qmax, unsure);
    if (wave_any(unsure)) {
      double m = 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = __builtin_fmax(m, (double)__builtin_fabsf(w[u][k]) / (double)bf[k]);
      if constexpr (LPB >= 2) m = __builtin_fmax(m, quad_xor<1>(m));
      if constexpr (LPB >= 4) m = __builtin_fmax(m, quad_xor<2>(m));
      if constexpr (LPB >= 8) m = __builtin_fmax(m, half_mirror(m));
      s = m > 0.0 ? (float)project<AFMT>(m / (double)Grid<GRID>::qmax) : 1.0f;
    }
    if (live && r < M && (threadIdx.x % LPB) == 0)
      reinterpret_cast<AT*>(a_)[r * (N / G) + col / G] = encode_scale<AFMT>((double)s);
  }
}

// ------------------------------------------------------------ BCD pass

constexpr int kThreads = 256;  // 4 waves
constexpr float kRowSure = 0x1p-19f;  // bracket of the float32 row sums (32 units of 2^-24)
constexpr int kPrefetch = 1;   // row steps in flight per lane

// Columns per lane of a pass. A workgroup step always covers 64 rows of a
// 64-column tile, with 4 waves of 16 columns per lane or 8 waves of 8; two
// workgroups share a CU either way, so the narrower lanes give each SIMD 4
// waves instead of 2 for about 10 % more instructions per element (the
// per-row work is shared by fewer elements) within 128 registers per lane.
// Measured per pass: the 8-column form is faster where the second
// requantization is mostly skipped and memory waits are longer (power-of-
// two and E4M3 block scales: NVFP4 4096x14336 54.0 -> 48.6 us, MXINT4
// 14336x4096 38.6 -> 36.2 us), the 16-column form where it runs for almost
// every wave (fp16 block scales, which move every iteration: INT4-G64
// 14336x4096 38.3 against 39.9 us).
template <int AFMT>
constexpr int pass_lane_cols() {
  return AFMT == kScaleFp16 ? 16 : 8;
}
template <int LC>
constexpr int pass_threads() {
  return 64 * (kRowsPerStep * kTileCols / (64 * LC));
}

// Column update from the partials of one pass: b'_j = Pi_fp16(sum num /
// sum den) over the segments of column j's tile, added in segment order.
// Segment geometry of a tile: the first workgroup whose range touches it and
// how many do. Every count here is below 2^31 (the host checks), so 32-bit
// division is exact.
__device__ __forceinline__ uint32_t tile_first_wg(const PassGeom& g, uint32_t tile) {
  return (tile * (uint32_t)g.S) / (uint32_t)g.L;
}
__device__ __forceinline__ uint32_t tile_n_seg(const PassGeom& g, uint32_t tile) {
  return ((tile + 1) * (uint32_t)g.S - 1) / (uint32_t)g.L - tile_first_wg(g, tile) + 1;
}

// The partials of one column of a tile, loaded kBatch at a time (all in
// flight together) and added in segment order.
struct ColumnPartials {
  static constexpr int kBatch = 8;  // loads in flight
  const double2* pt;
  int64_t n_seg;
  double2 v[kBatch];

  // An inactive instance loads nothing and sums to the empty sums.
  __device__ __forceinline__ ColumnPartials(const double* __restrict__ part, const PassGeom& g,
                                            int64_t tile, int col, bool active = true) {
    n_seg = active ? tile_n_seg(g, (uint32_t)tile) : 0;
    pt = active ? reinterpret_cast<const double2*>(part + tile * g.max_seg * (kTileCols * 2)) + col
                : nullptr;
    load(0);
  }
  __device__ __forceinline__ void load(int64_t s0) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      v[k] = s0 + k < n_seg ? pt[(s0 + k) * kTileCols] : make_double2(0.0, 0.0);
  }
  // sums in segment order, then the projected least-squares scale
  __device__ __forceinline__ float finish() {
    double nsum = 0.0, dsum = 0.0;
    for (int64_t s0 = 0; s0 < n_seg; s0 += kBatch) {
      if (s0 > 0) load(s0);
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (s0 + k < n_seg) {
          nsum += v[k].x;
          dsum += v[k].y;
        }
      }
    }
    return (float)ls_scale<kScaleFp16>(nsum, dsum);
  }
};

__device__ __forceinline__ float column_scale(const double* __restrict__ part, const PassGeom& g,
                                              int64_t tile, int col) {
  ColumnPartials cp(part, g, tile, col);
  return cp.finish();
}

// One BCD iteration. b of the state comes from the partial column sums of
// the previous pass (part_in) when there is one, else from b in memory;
// this pass's partial column sums go to part_out.
//
// The kPassStats variant also measures the state it starts from, (a, b) and its
// codes Q: the float64 sums of (W - a Q b)^2 and W^2, and the number of
// codes that differ from the codes in st.codes (the previous state's, when
// st.has_prev), which it then overwrites with Q. Each thread sums its own
// elements in order and the workgroup adds its threads in a fixed tree into
// st.part[blockIdx.x][3], so the result does not depend on timing.
struct PassStats {
  uint8_t* codes;  // [M][N * bits / 8] codes of the previous state, then of this one
  double* part;    // [n_wg][3] per-workgroup sums
  int has_prev;
};

// Pass variants: a plain iteration; one that also measures its starting
// state (above); and the first iteration of a whole solve, which starts
// from the absmax initialization (a = Pi_Fa(absmax / qmax) per block, 1 for
// a zero block; b = 1) formed from the rows it reads instead of from a and
// b in memory.
enum : int { kPassPlain = 0, kPassStats = 1, kPassInit = 2 };

template <int WT, int GRID, int AFMT, int G, int MODE, int LC>
__global__ void __launch_bounds__(pass_threads<LC>(), pass_threads<LC>() / 128)
    bcd_pass_kernel(const void* __restrict__ W, const double* __restrict__ part_in, void* __restrict__ a_,
                    int32_t gM, int32_t gN, int32_t gldw, int32_t gS, int32_t gL, int32_t gtotal,
                    int32_t gn_tiles, int32_t gmax_seg, const uint16_t* __restrict__ b,
                    double* __restrict__ part_out, PassStats st, int32_t a_tiled) {
  // the geometry comes as 32-bit scalars so that it arrives in preloaded
  // kernel-argument registers
  PassGeom g;
  g.M = gM; g.N = gN; g.ldw = gldw; g.S = gS; g.L = gL; g.total = gtotal;
  g.n_tiles = gn_tiles; g.max_seg = gmax_seg; g.n_wg = 0;
  using AT = typename ScaleStore<AFMT>::T;
  using Word = typename Grid<GRID>::Word;
  constexpr bool STATS = MODE == kPassStats;
  constexpr bool INIT = MODE == kPassInit;
  // The first pass of a whole solve under power-of-two block scales: with
  // b = 1 and a = 2^k the quotient W / (a b) is exact, so rounding it is the
  // decision itself (no tie flag, no exact re-decision).
  constexpr bool kExactQ = INIT && AFMT == kScaleE8M0;
  constexpr int CB = Grid<GRID>::kBits;     // bits per stored code
  constexpr int PT = pass_threads<LC>();     // threads (two workgroups per CU: PT / 128 waves per SIMD)
  constexpr int LPR = kTileCols / LC;       // lanes per row of a tile
  constexpr int RPW = 64 / LPR;             // rows per wave per step
  constexpr int RPS = PT / 64 * RPW;        // rows per workgroup per step
  constexpr int BL = G < LC ? G : LC;       // elements of one block inside a lane
  constexpr int NB = LC / BL;               // blocks (or block parts) per lane
  constexpr int LPB = G > LC ? G / LC : 1;  // lanes sharing one block
  // LDS of the column reduction: row c' = e * LPR + sub holds the sums of
  // column sub * LC + e from every row-lane. With this order and a pitch of
  // 68 doubles the lanes of one store (same e) and of one load (rows r*4 + pi)
  // spread over distinct banks.
  constexpr int kRedStride = 68;
  constexpr int EB = WT == kWBF16 ? 2 : 4;  // bytes per W element
  static_assert(RPS == kRowsPerStep, "geometry mismatch");
  static_assert(LC == 8 || LC == 16, "a lane's columns are all in range or all out (N % 16 == 0)");
  static_assert(LPR <= 8 && LPB <= LPR, "a block's lanes lie in one group of 8 (lane_join)");
  static_assert(RPS == 64, "the reduction's LDS pitch assumes 64 row-lanes");

  __shared__ __align__(16) float s_b[kTileCols];
  __shared__ __align__(16) float s_rb[kTileCols];
  __shared__ double s_red[kTileCols * kRedStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPR, rl = lane / LPR;
  const int64_t nblk = g.N / G;
  AT* __restrict__ a = reinterpret_cast<AT*>(a_);
  // block scale of (row, column c of tile t): row-major [M][N / G] at
  // row * N / G + c / G, or tile-major [n_tiles][M][64 / G] (one-byte
  // scales only) at t * M * 64 / G + row * 64 / G + (c - 64 t) / G
  constexpr int TB = kTileCols / G;
  const bool tiled = AFMT != kScaleFp16 && a_tiled;
  const int64_t a_rs = tiled ? TB : nblk;
  double st_sse = 0.0, st_w2 = 0.0;
  int st_changed = 0;

  // Step bookkeeping in 32 bits (the host keeps S * n_tiles below 2^31 and
  // rows below 2^31, so S * RPS + RPS fits in uint32): uniform counters stay
  // in scalar registers and compare there.
  const uint32_t S32 = (uint32_t)g.S, M32 = (uint32_t)g.M;
  uint32_t f = blockIdx.x * (uint32_t)g.L;
  const uint32_t f_first = f;
  const uint32_t f_end = min(f + (uint32_t)g.L, (uint32_t)g.total);
  while (f < f_end) {
    const uint32_t tile = f / S32;
    const uint32_t seg_end = min(f_end, (tile + 1) * S32);
    const int64_t tcol = (int64_t)tile * kTileCols;
    const int64_t col0 = tcol + sub * LC;
    const bool lane_cols_ok = col0 < g.N;
    const int64_t ccol = lane_cols_ok ? col0 : (tiled ? tcol : 0);  // clamped column for loads
    const int64_t a_tile = tiled ? ((int64_t)tile * g.M * TB + (ccol - tcol) / G) : ccol / G;

    // Raw loads of row steps, issued kPrefetch steps ahead of their use
    // (a ring of register buffers). Rows past M (last step of a tile) read
    // row M-1; out of range values are zeroed before use.
    RawRow<WT, LC> raw[kPrefetch];
    AT a_raw[kPrefetch][NB];
    auto issue = [&](uint32_t st, int slot) {
      const int64_t r = min(st * RPS + wave * RPW + rl, M32 - 1);
      raw[slot].load(W, r * g.ldw + ccol);
      if constexpr (!INIT) {
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) a_raw[slot][bl] = a[a_tile + r * a_rs + bl * BL / G];
      }
    };
    uint32_t step = f - tile * S32;
#pragma unroll
    for (int d = 0; d < kPrefetch; ++d)
      if (f + d < seg_end) issue(step + d, d);

    if (f != f_first) __syncthreads();  // LDS of the previous segment is no longer read
    if (tid < kTileCols) {
      const int64_t j = tcol + tid;
      float bj = 1.0f;
      if (j < g.N && !INIT) bj = part_in ? column_scale(part_in, g, tile, tid) : fp16_bits_to_float(b[j]);
      s_b[tid] = bj;
      s_rb[tid] = 1.0f / bj;
    }
    __syncthreads();

    // this lane's column scales and their reciprocals. With 16 columns per
    // lane and the grids rounded by two conversions they are copied to
    // registers for the whole segment: read through the LDS pointers, the
    // compiler kept two copies of the codes across the re-decision branch
    // (16 register moves per row step); the integer grids compile to the
    // same loop either way and read LDS. With 8 columns per lane each row
    // step reads them from LDS (below), which keeps the 128-register budget.
    float lb_r[LC], lrb_r[LC];
    const float* lb = s_b + sub * LC;
    const float* lrb = s_rb + sub * LC;
    int lds_off4 = sub * LC / 4;  // the lane's first column scale, in float4 units
    if constexpr (LC == 16 && Grid<GRID>::kTwoEnded) {
#pragma unroll
      for (int e = 0; e < LC; ++e) {
        lb_r[e] = s_b[sub * LC + e];
        lrb_r[e] = s_rb[sub * LC + e];
      }
      lb = lb_r;
      lrb = lrb_r;
    }
    double cn[LC], cd[LC];
#pragma unroll
    for (int e = 0; e < LC; ++e) { cn[e] = 0.0; cd[e] = 0.0; }

    // W pointer (bytes) and block-scale index of this lane's row, advanced
    // by one step of RPS rows at a time.
    const int64_t wstep = (int64_t)RPS * g.ldw * EB;
    const int64_t astep = (int64_t)RPS * a_rs;
    uint32_t row = step * RPS + wave * RPW + rl;
    const char* wp = reinterpret_cast<const char*>(W) + ((int64_t)row * g.ldw + ccol) * EB;
    int64_t ai = a_tile + (int64_t)row * a_rs;

    // One row step; the ring slot is a compile-time constant so that no
    // in-flight register is ever copied (the loop below is unrolled by
    // kPrefetch).
    auto row_step = [&]<int SLOT>() {
      const float* lbs = lb;
      const float* lrbs = lrb;
      float lb8[LC], lrb8[LC];
      if constexpr (LC == 8) {
        // an opaque offset keeps these loads inside the loop
        asm volatile("" : "+v"(lds_off4));
        const float4* b4 = reinterpret_cast<const float4*>(s_b) + lds_off4;
        const float4* rb4 = reinterpret_cast<const float4*>(s_rb) + lds_off4;
#pragma unroll
        for (int i = 0; i < LC / 4; ++i) {
          const float4 u = b4[i], v = rb4[i];
          lb8[4 * i] = u.x; lb8[4 * i + 1] = u.y; lb8[4 * i + 2] = u.z; lb8[4 * i + 3] = u.w;
          lrb8[4 * i] = v.x; lrb8[4 * i + 1] = v.y; lrb8[4 * i + 2] = v.z; lrb8[4 * i + 3] = v.w;
        }
        lbs = lb8;
        lrbs = lrb8;
      }
      const bool row_ok = row < M32;
      // rows past M occur only in the last step of a tile, columns past N
      // only in the last tile
      const bool full = (step + 1) * RPS <= M32 && tcol + kTileCols <= g.N;

      float w[LC];
      raw[SLOT].unpack(w);
      float a_old[NB];
      if constexpr (INIT) {
        // the absmax start, from this row's block (shuffles join the lanes
        // of a block wider than a lane); certified float32 projection
        float amax[NB];
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
          amax[bl] = 0.0f;
#pragma unroll
          for (int k = 0; k < BL; ++k) amax[bl] = __builtin_fmaxf(amax[bl], __builtin_fabsf(w[bl * BL + k]));
        }
        amax[0] = max_join<LPB>(amax[0]);
        bool unsure = false;
#pragma unroll
        for (int bl = 0; bl < NB; ++bl)
          a_old[bl] = amax[bl] > 0.0f ? ls_scale_fast<AFMT>((double)amax[bl], (double)Grid<GRID>::qmax, unsure)
                                      : 1.0f;
        if (wave_any(unsure)) {
#pragma unroll
          for (int bl = 0; bl < NB; ++bl)
            a_old[bl] = amax[bl] > 0.0f
                            ? (float)project<AFMT>((double)amax[bl] / (double)Grid<GRID>::qmax)
                            : 1.0f;
        }
      } else {
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) a_old[bl] = decode_scale<AFMT>(a_raw[SLOT][bl]);
      }
      const bool ok = row_ok && lane_cols_ok;
      if (!full) {
#pragma unroll
        for (int e = 0; e < LC; ++e) w[e] = ok ? w[e] : 0.0f;
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) a_old[bl] = ok ? a_old[bl] : 1.0f;
      }
      // refill this slot with the step kPrefetch ahead
      if (f + kPrefetch < seg_end) {
        if ((step + kPrefetch + 1) * RPS <= M32) {  // that step is entirely inside M
          raw[SLOT].load(wp + kPrefetch * wstep, 0);
          if constexpr (!INIT) {
#pragma unroll
            for (int bl = 0; bl < NB; ++bl) a_raw[SLOT][bl] = a[ai + kPrefetch * astep + bl * BL / G];
          }
        } else {
          issue(step + kPrefetch, SLOT);
        }
      }

      // Q1 = q(W / (a b)) with the current state, fused with the row/block
      // least-squares sums (R = Q1 D_b). If any element of the wave lies
      // near a rounding midpoint the sums are redone with exact codes.
      float q[LC];    // Q1 here; becomes Q2 below
      float wrb[LC];  // W / b (rounded), shared by both requantizations
      // Row least-squares sums, first in float32 in two interleaved chains
      // per lane. Every term W R and R^2 is non-negative (a non-zero code
      // has the sign of its weight), so each fused multiply-add adds at most
      // one rounding of a partial sum no larger than the whole sum: at most
      // BL / 2 units of 2^-24 (relative) per chain, one for joining the
      // chains and one per join across the lanes of a block (log2 LPB), at
      // most 11 (BL = 16, G = 64) for the numerator and the denominator
      // alike. Their quotient with a
      // 1-ulp reciprocal is then within 25 units, inside the certified
      // projection's bracket of kRowSure = 32 units. A wave with a block
      // the bracket cannot decide redoes its sums in float64, where every
      // product is exact.
      float numf[NB], denf[NB];
      auto row_sums_f32 = [&]() {
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
          float n0 = 0.0f, n1 = 0.0f, d0 = 0.0f, d1 = 0.0f;
#pragma unroll
          for (int k = 0; k < BL; k += 2) {
            const int e = bl * BL + k;
            const float R0 = q[e] * lbs[e], R1 = q[e + 1] * lbs[e + 1];  // exact products
            n0 = __builtin_fmaf(w[e], R0, n0);
            d0 = __builtin_fmaf(R0, R0, d0);
            n1 = __builtin_fmaf(w[e + 1], R1, n1);
            d1 = __builtin_fmaf(R1, R1, d1);
          }
          numf[bl] = n0 + n1;
          denf[bl] = d0 + d1;
        }
      };
      double num[NB], den[NB];
      auto row_sums_f64 = [&]() {
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
          num[bl] = 0.0;
          den[bl] = 0.0;
#pragma unroll
          for (int k = 0; k < BL; ++k) {
            const int e = bl * BL + k;
            const double R = (double)(q[e] * lbs[e]);  // exact product
            num[bl] = __builtin_fma((double)w[e], R, num[bl]);
            den[bl] = __builtin_fma(R, R, den[bl]);
          }
        }
      };
      {
        float ra[NB], y[LC];
#pragma unroll
        for (int bl = 0; bl < NB; ++bl)
          ra[bl] = recip_scale<AFMT>(a_old[bl]);
#pragma unroll
        for (int e = 0; e < LC; ++e) wrb[e] = w[e] * lrbs[e];
        if constexpr (Grid<GRID>::kScaledEnds && !kExactQ) {
          uint32_t diff[LC / 4], hiw[LC / 4];
          if (wave_any(Grid<GRID>::template fast_scaled<LC, BL>(wrb, ra, q, diff, hiw)))
            redecide<GRID, LC, BL>(y, q, diff, hiw, w, a_old, lbs);
        } else {
#pragma unroll
          for (int bl = 0; bl < NB; ++bl)
#pragma unroll
            for (int k = 0; k < BL; ++k) y[bl * BL + k] = wrb[bl * BL + k] * ra[bl];
          if constexpr (kExactQ) {
            Grid<GRID>::template nearest_n<LC>(y, q);
          } else {
            uint32_t diff[LC / 4], hiw[LC / 4];
            if (wave_any(Grid<GRID>::template fast_n<LC>(y, q, diff, hiw)))
              redecide<GRID, LC, BL>(y, q, diff, hiw, w, a_old, lbs);
          }
        }
        row_sums_f32();
      }
      if constexpr (STATS) {
        // the state (a, b) this pass starts from, with its codes Q1
        if (ok) {
#pragma unroll
          for (int bl = 0; bl < NB; ++bl)
#pragma unroll
            for (int k = 0; k < BL; ++k) {
              const int e = bl * BL + k;
              // a Q b is exact in float64: q b is exact in float32
              const double wk = (double)w[e];
              const double d = wk - (double)(q[e] * lbs[e]) * (double)a_old[bl];
              st_sse = __builtin_fma(d, d, st_sse);
              st_w2 = __builtin_fma(wk, wk, st_w2);
            }
          uint8_t* cp = st.codes + row * (g.N * CB / 8) + ccol * CB / 8;
#pragma unroll
          for (int i = 0; i < LC / 8; ++i) {  // 8 codes per word, CB bytes
            const Word c = Grid<GRID>::encode8(q + 8 * i);
            if (st.has_prev) st_changed += Grid<GRID>::count_diff(c, *reinterpret_cast<const Word*>(cp + i * CB));
            *reinterpret_cast<Word*>(cp + i * CB) = c;
          }
        }
      }
      // blocks wider than a lane: add the sums of the block's lanes
      numf[0] = lane_join<LPB>(numf[0]);
      denf[0] = lane_join<LPB>(denf[0]);

      // project, synchronize the copy that assigns codes, store. The
      // float32 denominator is 0 exactly when every code of the block is 0
      // (a non-zero R^2 is at least 2^-66, a normal float32).
      float a_new[NB];
      bool unsure = false;
#pragma unroll
      for (int bl = 0; bl < NB; ++bl)
        a_new[bl] = denf[bl] > 0.0f ? project_certified<AFMT>(numf[bl], denf[bl], kRowSure, unsure) : 1.0f;
      if (wave_any(unsure)) {
        row_sums_f64();
        num[0] = lane_join<LPB>(num[0]);
        den[0] = lane_join<LPB>(den[0]);
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) a_new[bl] = (float)ls_scale<AFMT>(num[bl], den[bl]);
      }
#pragma unroll
      for (int bl = 0; bl < NB; ++bl)
        if (ok && (sub % LPB) == 0) a[ai + bl * BL / G] = encode_scale<AFMT>((double)a_new[bl]);

      // Q2 = q(W / (a' b)). Where no block scale of the wave changed, Q2 is
      // Q1 (same quotient, same decision) and is not recomputed.
      bool changed = false;
#pragma unroll
      for (int bl = 0; bl < NB; ++bl) changed |= a_new[bl] != a_old[bl];
      if (wave_any(changed)) {
        float ra[NB], y[LC];
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) ra[bl] = recip_scale<AFMT>(a_new[bl]);
        if constexpr (Grid<GRID>::kScaledEnds && !kExactQ) {
          uint32_t diff[LC / 4], hiw[LC / 4];
          if (wave_any(Grid<GRID>::template fast_scaled<LC, BL>(wrb, ra, q, diff, hiw)))
            redecide<GRID, LC, BL>(y, q, diff, hiw, w, a_new, lbs);
        } else {
#pragma unroll
          for (int bl = 0; bl < NB; ++bl)
#pragma unroll
            for (int k = 0; k < BL; ++k) y[bl * BL + k] = wrb[bl * BL + k] * ra[bl];
          if constexpr (kExactQ) {
            Grid<GRID>::template nearest_n<LC>(y, q);
          } else {
            uint32_t diff[LC / 4], hiw[LC / 4];
            if (wave_any(Grid<GRID>::template fast_n<LC>(y, q, diff, hiw)))
              redecide<GRID, LC, BL>(y, q, diff, hiw, w, a_new, lbs);
          }
        }
      }

      // column least-squares sums in float64, S = D_a' Q2
#pragma unroll
      for (int bl = 0; bl < NB; ++bl) {
#pragma unroll
        for (int k = 0; k < BL; ++k) {
          const int e = bl * BL + k;
          const double S = (double)(a_new[bl] * q[e]);  // exact product
          cn[e] = __builtin_fma((double)w[e], S, cn[e]);
          cd[e] = __builtin_fma(S, S, cd[e]);
        }
      }
    };
    auto advance = [&]() {
      if constexpr (LC == 8) {
        // Issue priority by progress. A SIMD issues from its oldest ready
        // wave, so of the two workgroups on a CU the first dispatched runs
        // ahead and the other finishes its last steps alone, with half the
        // waves. A workgroup lowers its waves' priority as it passes a half,
        // three quarters and nine tenths of its steps, which lets the one
        // behind catch up. Timing only: every result is the same.
        const uint32_t done = f - f_first + 1, L32 = (uint32_t)g.L;
        if (10 * done >= 9 * L32) __builtin_amdgcn_s_setprio(0);
        else if (4 * done >= 3 * L32) __builtin_amdgcn_s_setprio(1);
        else if (2 * done >= L32) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(3);
      }
      ++f;
      ++step;
      row += RPS;
      wp += wstep;
      ai += astep;
      return f < seg_end;
    };
    auto run_slots = [&]<int... S>(std::integer_sequence<int, S...>) {
      while (((row_step.template operator()<S>(), advance()) && ...)) {
      }
    };
    run_slots(std::make_integer_sequence<int, kPrefetch>{});

    // ---- reduce the RPS row-lanes of each column, write this segment's partial
    const int64_t seg = (int64_t)blockIdx.x - tile_first_wg(g, tile);
    double* __restrict__ pw = part_out + (tile * g.max_seg + seg) * (kTileCols * 2);
#pragma unroll
    for (int qn = 0; qn < 2; ++qn) {
#pragma unroll
      for (int e = 0; e < LC; ++e) {
        s_red[(e * LPR + sub) * kRedStride + wave * RPW + rl] = qn ? cd[e] : cn[e];
      }
      __syncthreads();
      constexpr int kParts = PT / kTileCols;  // threads per LDS row
      const int cr = tid / kParts, pi = tid % kParts;    // LDS row, part of its row-lanes
      double acc = 0.0;
      const int c = (cr % LPR) * LC + cr / LPR;  // the column of LDS row cr
#pragma unroll 8
      for (int r = 0; r < RPS / kParts; ++r) acc += s_red[cr * kRedStride + r * kParts + pi];
      acc = lane_join<kParts>(acc);
      if (pi == 0) pw[c * 2 + qn] = acc;
      __syncthreads();
    }
  }

  if constexpr (STATS) {  // s_red is free: every segment ended with a barrier
    s_red[tid] = st_sse;
    s_red[PT + tid] = st_w2;
    s_red[2 * PT + tid] = (double)st_changed;
    __syncthreads();
    for (int h = PT / 2; h > 0; h >>= 1) {
      if (tid < h)
        for (int i = 0; i < 3; ++i) s_red[i * PT + tid] += s_red[i * PT + tid + h];
      __syncthreads();
    }
    if (tid < 3) st.part[(int64_t)blockIdx.x * 3 + tid] = s_red[tid * PT];
  }
}

// Final column update of a dq_bcd_iterate call: writes b from the last
// pass's partials. One thread per column.
static __global__ void __launch_bounds__(kTileCols)
    bcd_column_kernel(const double* __restrict__ part, uint16_t* __restrict__ b, PassGeom g) {
  const int64_t tile = blockIdx.x;
  const int64_t j = tile * kTileCols + threadIdx.x;
  if (j < g.N) b[j] = __half_as_ushort(__float2half_rn(column_scale(part, g, tile, threadIdx.x)));
}

// ------------------------------------------------------------------ pack

// One thread per (16 columns, kPackRows rows), 8 (4-bit codes) or 16
// (8-bit codes) bytes out per row; the column reciprocals are formed once
// per thread. Codes come from the float32 estimate of W/(a b) (reciprocals:
// relative error below 4 units of 2^-24); a wave with any element near a
// rounding midpoint re-decides those element slots exactly, as the pass
// kernel does.
//
// With REPORT the kernel also measures the state: per workgroup it writes
// the float64 sums of (W - a Q b)^2 and W^2 and the number of codes that
// differ from prev (if given) to part[blockIdx.x][3]; packed may then be
// null. Each thread sums its elements in order, then the workgroup adds the
// threads in a fixed tree, so the result does not depend on timing.
template <int WT, int GRID, int AFMT, int G, bool REPORT>
__global__ void __launch_bounds__(256) pack_kernel(const void* __restrict__ W, int64_t ldw,
                                                   int64_t M, int64_t N, const void* __restrict__ a_,
                                                   const uint16_t* __restrict__ b,
                                                   uint8_t* __restrict__ packed,
                                                   const uint8_t* __restrict__ prev,
                                                   double* __restrict__ part) {
  using AT = typename ScaleStore<AFMT>::T;
  using Word = typename Grid<GRID>::Word;
  constexpr int BL = G < 16 ? G : 16;  // elements of one block in this thread
  constexpr int NB = 16 / BL;
  constexpr int B = Grid<GRID>::kBits;  // 4: two codes per byte; 8: one
  const int64_t nch = N / 16;
  const int64_t n_rg = (M + kPackRows - 1) / kPackRows;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = idx < n_rg * nch;
  const int64_t cidx = live ? idx : 0;  // dead lanes compute on element 0
  const int64_t rg = cidx / nch, col = (cidx - rg * nch) * 16;
  const uint4 bv0 = *reinterpret_cast<const uint4*>(b + col);
  const uint4 bv1 = *reinterpret_cast<const uint4*>(b + col + 8);
  const uint32_t bw[8] = {bv0.x, bv0.y, bv0.z, bv0.w, bv1.x, bv1.y, bv1.z, bv1.w};
  float bj[16], rb[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    bj[k] = fp16_bits_to_float((uint16_t)(bw[k >> 1] >> (16 * (k & 1))));
    rb[k] = __builtin_amdgcn_rcpf(bj[k]);
  }
  double sse = 0.0, w2 = 0.0;
  int changed = 0;
#pragma unroll
  for (int r = 0; r < kPackRows; ++r) {
    const int64_t row_raw = rg * kPackRows + r;
    const bool ok = live && row_raw < M;
    const int64_t row = ok ? row_raw : 0;
    RawRow<WT, 16> raw;
    raw.load(W, row * ldw + col);
    float av[NB];
#pragma unroll
    for (int bl = 0; bl < NB; ++bl)
      av[bl] = decode_scale<AFMT>(reinterpret_cast<const AT*>(a_)[row * (N / G) + (col + bl * BL) / G]);
    float w[16], y[16], q[16];
    raw.unpack(w);
    uint32_t diff[4], hiw[4];
    if constexpr (Grid<GRID>::kScaledEnds) {
      float wrb[16], ra[NB];
#pragma unroll
      for (int k = 0; k < 16; ++k) wrb[k] = w[k] * rb[k];
#pragma unroll
      for (int bl = 0; bl < NB; ++bl) ra[bl] = recip_scale<AFMT>(av[bl]);
      if (wave_any(Grid<GRID>::template fast_scaled<16, BL>(wrb, ra, q, diff, hiw)))
        redecide<GRID, 16, BL>(y, q, diff, hiw, w, av, bj);
    } else {
#pragma unroll
      for (int bl = 0; bl < NB; ++bl) {
        const float ra = recip_scale<AFMT>(av[bl]);
#pragma unroll
        for (int k = bl * BL; k < (bl + 1) * BL; ++k) y[k] = w[k] * rb[k] * ra;
      }
      if (wave_any(Grid<GRID>::template fast_n<16>(y, q, diff, hiw)))
        redecide<GRID, 16, BL>(y, q, diff, hiw, w, av, bj);
    }
    const Word c0 = Grid<GRID>::encode8(q), c1 = Grid<GRID>::encode8(q + 8);
    if (ok && (!REPORT || packed)) {
      uint8_t* dst = packed + row * (N * B / 8) + col * B / 8;
      *reinterpret_cast<Word*>(dst) = c0;
      *reinterpret_cast<Word*>(dst + B) = c1;
    }
    if constexpr (REPORT) {
      if (ok) {
#pragma unroll
        for (int bl = 0; bl < NB; ++bl)
#pragma unroll
          for (int k = bl * BL; k < (bl + 1) * BL; ++k) {
            // a Q b is exact in float64: q b is exact in float32
            const double wk = (double)w[k];
            const double d = wk - (double)(q[k] * bj[k]) * (double)av[bl];
            sse = __builtin_fma(d, d, sse);
            w2 = __builtin_fma(wk, wk, w2);
          }
        if (prev) {
          const uint8_t* src = prev + row * (N * B / 8) + col * B / 8;
          changed += Grid<GRID>::count_diff(c0, *reinterpret_cast<const Word*>(src)) +
                     Grid<GRID>::count_diff(c1, *reinterpret_cast<const Word*>(src + B));
        }
      }
    }
  }
  if constexpr (REPORT) {
    __shared__ double s_part[3][256];
    s_part[0][threadIdx.x] = sse;
    s_part[1][threadIdx.x] = w2;
    s_part[2][threadIdx.x] = (double)changed;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if ((int)threadIdx.x < h)
        for (int i = 0; i < 3; ++i) s_part[i][threadIdx.x] += s_part[i][threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x < 3) part[(int64_t)blockIdx.x * 3 + threadIdx.x] = s_part[threadIdx.x][0];
  }
}

// Adds the per-workgroup report sums in a fixed order: thread t takes the
// workgroups t, t + 256, ... in turn, then a fixed tree over the threads.
static __global__ void __launch_bounds__(256) report_reduce_kernel(const double* __restrict__ part,
                                                                   int64_t n, double* __restrict__ out) {
  __shared__ double s_part[3][256];
  double acc[3] = {0.0, 0.0, 0.0};
  for (int64_t k = threadIdx.x; k < n; k += 256)
    for (int i = 0; i < 3; ++i) acc[i] += part[k * 3 + i];
  for (int i = 0; i < 3; ++i) s_part[i][threadIdx.x] = acc[i];
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h)
      for (int i = 0; i < 3; ++i) s_part[i][threadIdx.x] += s_part[i][threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x < 3) out[threadIdx.x] = s_part[threadIdx.x][0];
}

// ------------------------------------------------------- activation side

// One lane per 8 consecutive channels of kActTokens consecutive tokens (one
// 16-byte load of X per token, one of b), G/8 lanes per block: X' = X D_b
// (exact in float32 for bf16 X), block absmax by lane shuffles,
// s = Pi(absmax / qmax), codes from the float32 estimate X' * (1/s) with the
// exact re-decision of a wave that has an element near a rounding midpoint.
// All loads are issued before any arithmetic, and b is converted once for
// the lane's tokens. The projection of absmax / qmax takes the certified
// float32 path of the pass kernel and falls back to float64 for a wave
// with a quotient near a rounding boundary of the scale format.
constexpr int kActTokens = 4;

template <int GRID, int AFMT, int G>
__global__ void __launch_bounds__(256) act_quant_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                        int64_t T, int64_t N,
                                                        const uint16_t* __restrict__ b,
                                                        uint8_t* __restrict__ xq,
                                                        void* __restrict__ xs_) {
  using AT = typename ScaleStore<AFMT>::T;
  constexpr int LPB = G / 8;  // lanes per block; a block never straddles a wave
  constexpr int B = Grid<GRID>::kBits;
  const int64_t nch = N / 8;
  const int64_t n_tg = (T + kActTokens - 1) / kActTokens;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = idx < n_tg * nch;
  const int64_t cidx = live ? idx : 0;  // dead lanes compute on chunk 0
  const int64_t tg = cidx / nch, col = (cidx - tg * nch) * 8;
  uint4 xv[kActTokens];
#pragma unroll
  for (int u = 0; u < kActTokens; ++u) {
    const int64_t t = min(tg * kActTokens + u, T - 1);  // tokens past T read the last one
    xv[u] = *reinterpret_cast<const uint4*>(X + t * ldx + col);
  }
  const uint4 bv = *reinterpret_cast<const uint4*>(b + col);
  const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
  float bf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) bf[k] = fp16_bits_to_float((uint16_t)(bw[k >> 1] >> (16 * (k & 1))));
#pragma unroll
  for (int u = 0; u < kActTokens; ++u) {
    const int64_t t = tg * kActTokens + u;
    const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
    float x[8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float xk = (k & 1) ? bf16_hi(xw[k >> 1]) : bf16_lo(xw[k >> 1]);
      x[k] = xk * bf[k];  // exact product
      amax = __builtin_fmaxf(amax, __builtin_fabsf(x[k]));
    }
    static_assert(LPB <= 8, "a block's lanes lie in one group of 8");
    amax = max_join<LPB>(amax);
    bool unsure = false;
    float sf = ls_scale_fast<AFMT>((double)amax, (double)Grid<GRID>::qmax, unsure);
    if (wave_any(unsure))
      sf = amax > 0.0f ? (float)project<AFMT>((double)amax / (double)Grid<GRID>::qmax) : 1.0f;
    float y[8], q[8];
    if constexpr (AFMT == kScaleE8M0) {
      // a power-of-two scale: y = X b / s is exact (X b is, and so is the
      // scaling by 2^-k down to the float32 subnormals, below any rounding
      // decision), so rounding y itself is the exact decision
      const float rs = recip_pow2(sf);
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = x[k] * rs;
      Grid<GRID>::template nearest_n<8>(y, q);
    } else {
      const float rs = __builtin_amdgcn_rcpf(sf);
      uint32_t diff[2], hiw[2];
      const float one[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (Grid<GRID>::kScaledEnds) {
        if (wave_any(Grid<GRID>::template fast_scaled<8, 8>(x, &rs, q, diff, hiw)))
          redecide<GRID, 8, 8>(y, q, diff, hiw, x, &sf, one);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = x[k] * rs;
        if (wave_any(Grid<GRID>::template fast_n<8>(y, q, diff, hiw)))
          redecide<GRID, 8, 8, false>(y, q, diff, hiw, x, &sf, one);  // per slot: measured faster here
      }
    }
    if (live && t < T) {
      Grid<GRID>::store8(xq + t * (N * B / 8) + col * B / 8, q);
      if ((threadIdx.x % LPB) == 0)
        reinterpret_cast<AT*>(xs_)[t * (N / G) + col / G] = encode_scale<AFMT>((double)sf);
    }
  }
}

// ------------------------------------------------------------- launchers

static inline unsigned blocks_for(int64_t n, int threads) {
  return (unsigned)((n + threads - 1) / threads);
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_init(const void* W, int64_t ldw, int64_t M, int64_t N, void* a, uint16_t* b,
                       hipStream_t st) {
  const int64_t n = max(M * (N / G), N);
  init_rtn_kernel<WT, GRID, AFMT, G><<<blocks_for(n, 256), 256, 0, st>>>(W, ldw, M, N, a, b);
  return hipGetLastError();
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_init_colnorm(const void* W, int64_t ldw, int64_t M, int64_t N, void* a, uint16_t* b,
                               double* part, hipStream_t st) {
  const int64_t n_tiles = (N + kTileCols - 1) / kTileCols;
  const int64_t chunk_rows = colnorm_chunk_rows(M);
  const int64_t n_chunks = (M + chunk_rows - 1) / chunk_rows;
  colnorm_partial_kernel<WT><<<dim3((unsigned)n_tiles, (unsigned)n_chunks), 256, 0, st>>>(
      W, ldw, M, N, chunk_rows, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  colnorm_b_kernel<<<(unsigned)n_tiles, kTileCols, 0, st>>>(part, n_chunks, M, N, b);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n_rg = (M + kColnormRowsPerLane - 1) / kColnormRowsPerLane;
  colnorm_a_kernel<WT, GRID, AFMT, G><<<blocks_for(n_rg * (N / 8), 256), 256, 0, st>>>(W, ldw, M, N, b, a);
  return hipGetLastError();
}

template <int WT, int GRID, int AFMT, int G, int MODE>
hipError_t launch_pass(const void* W, const double* in, void* a, bool a_tiled, uint16_t* b, double* out,
                       const PassGeom& g, const PassStats& ps, hipStream_t st) {
  // The first pass of a solve reads W cold from HBM: it takes the 8-column
  // form for every format, whose four waves per SIMD keep more loads in
  // flight (solves from the absmax start with W evicted: 14336x4096 INT4-G64
  // 777 -> 773 us, 4096x14336 831 -> 821 us).
  constexpr int LC = MODE == kPassInit ? 8 : pass_lane_cols<AFMT>();
  bcd_pass_kernel<WT, GRID, AFMT, G, MODE, LC><<<(unsigned)g.n_wg, pass_threads<LC>(), 0, st>>>(
      W, in, a, (int32_t)g.M, (int32_t)g.N, (int32_t)g.ldw, (int32_t)g.S, (int32_t)g.L,
      (int32_t)g.total, (int32_t)g.n_tiles, (int32_t)g.max_seg, b, out, ps, a_tiled ? 1 : 0);
  return hipGetLastError();
}

// Block scales between the caller's row-major layout [M][N / G] and the
// tile-major one [n_tiles][M][64 / G] of a call's passes. The 64 / G scales
// of one (row, tile) form a unit. A workgroup moves 64 rows x 32 tiles
// through LDS: eight unit loads per thread in flight, rows read across
// tiles and tiles written down rows, both contiguous.
constexpr int kRelayRows = 64, kRelayTiles = 32;
template <int BYTES> struct UnitOf;
template <> struct UnitOf<1> { using T = uint8_t; };
template <> struct UnitOf<2> { using T = uint16_t; };
template <> struct UnitOf<4> { using T = uint32_t; };
template <> struct UnitOf<8> { using T = uint64_t; };

template <int AFMT, int G, bool TO_TILED>
__global__ void __launch_bounds__(256)
    relayout_a_kernel(const void* __restrict__ src_, void* __restrict__ dst_, int64_t M, int64_t N) {
  constexpr int TB = kTileCols / G;
  using U = typename UnitOf<TB * sizeof(typename ScaleStore<AFMT>::T)>::T;
  constexpr int kPer = kRelayRows * kRelayTiles / 256;  // units per thread
  __shared__ U s[kRelayRows * (kRelayTiles + 1)];        // [row][tile], padded
  const U* __restrict__ src = reinterpret_cast<const U*>(src_);
  U* __restrict__ dst = reinterpret_cast<U*>(dst_);
  const int64_t n_tiles = N / kTileCols;                  // N % 64 == 0 here
  const int64_t n_tc = (n_tiles + kRelayTiles - 1) / kRelayTiles;
  const int64_t r0 = (int64_t)(blockIdx.x / n_tc) * kRelayRows;
  const int64_t t0 = (int64_t)(blockIdx.x % n_tc) * kRelayTiles;
  U v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + 256 * j;
    const int r = TO_TILED ? i / kRelayTiles : i % kRelayRows;
    const int t = TO_TILED ? i % kRelayTiles : i / kRelayRows;
    const int64_t row = r0 + r, tile = t0 + t;
    v[j] = 0;
    if (row < M && tile < n_tiles) v[j] = TO_TILED ? src[row * n_tiles + tile] : src[tile * M + row];
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + 256 * j;
    const int r = TO_TILED ? i / kRelayTiles : i % kRelayRows;
    const int t = TO_TILED ? i % kRelayTiles : i / kRelayRows;
    s[r * (kRelayTiles + 1) + t] = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + 256 * j;
    const int r = TO_TILED ? i % kRelayRows : i / kRelayTiles;
    const int t = TO_TILED ? i / kRelayRows : i % kRelayTiles;
    const int64_t row = r0 + r, tile = t0 + t;
    if (row < M && tile < n_tiles) {
      const U u = s[r * (kRelayTiles + 1) + t];
      if (TO_TILED)
        dst[tile * M + row] = u;
      else
        dst[row * n_tiles + tile] = u;
    }
  }
}

// The same, one scale at a time: for a last tile narrower than 64 columns,
// or row-major scales not aligned to a unit.
template <int AFMT, int G, bool TO_TILED>
__global__ void __launch_bounds__(256)
    relayout_a_scalar_kernel(const void* __restrict__ src_, void* __restrict__ dst_, int64_t M, int64_t N) {
  using AT = typename ScaleStore<AFMT>::T;
  constexpr int TB = kTileCols / G;
  const AT* __restrict__ src = reinterpret_cast<const AT*>(src_);
  AT* __restrict__ dst = reinterpret_cast<AT*>(dst_);
  const int64_t nblk = N / G;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * nblk) return;
  // consecutive threads: consecutive scales of a row
  const int64_t row = idx / nblk, blk = idx - row * nblk, tile = blk / TB;
  const int64_t tm = (tile * M + row) * TB + blk % TB;
  if (TO_TILED)
    dst[tm] = src[idx];
  else
    dst[idx] = src[tm];
}

template <int AFMT, int G, bool TO_TILED>
hipError_t launch_relayout_a(const void* src, void* dst, const PassGeom& g, hipStream_t st) {
  constexpr int U = kTileCols / G * sizeof(typename ScaleStore<AFMT>::T);
  const uintptr_t row_major = reinterpret_cast<uintptr_t>(TO_TILED ? src : dst);
  if (g.N % kTileCols == 0 && row_major % U == 0) {
    const int64_t blocks =
        ((g.M + kRelayRows - 1) / kRelayRows) * ((g.n_tiles + kRelayTiles - 1) / kRelayTiles);
    relayout_a_kernel<AFMT, G, TO_TILED><<<(unsigned)blocks, 256, 0, st>>>(src, dst, g.M, g.N);
  } else {
    const int64_t n = g.M * (g.N / G);
    relayout_a_scalar_kernel<AFMT, G, TO_TILED><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(src, dst, g.M, g.N);
  }
  return hipGetLastError();
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_iterate(const void* W, void* a, uint16_t* b, double* part, const PassGeom& g,
                          int n_iters, const IterStats* stats, bool from_init, void* a_work,
                          hipStream_t st) {
  // partial buffers alternate between passes: pass k reads the partials of
  // pass k-1 (its column update) and writes its own to the other buffer
  const int64_t half = g.n_tiles * g.max_seg * kTileCols * 2;
  hipError_t err = hipSuccess;
  const bool tiled = a_work && !stats && n_iters > 0;
  void* pa = tiled ? a_work : a;  // the block scales the passes read and write
  if (tiled && !from_init) err = launch_relayout_a<AFMT, G, true>(a, a_work, g, st);
  for (int it = 0; it < n_iters && err == hipSuccess; ++it) {
    const double* in = it == 0 ? nullptr : part + ((it - 1) & 1) * half;
    double* out = part + (it & 1) * half;
    if (stats) {
      const PassStats ps{stats->codes, stats->part, it > 0 ? 1 : 0};
      err = launch_pass<WT, GRID, AFMT, G, kPassStats>(W, in, a, false, b, out, g, ps, st);
      if (err == hipSuccess) {
        report_reduce_kernel<<<1, 256, 0, st>>>(stats->part, g.n_wg, stats->out + 3 * it);
        err = hipGetLastError();
      }
    } else if (it == 0 && from_init) {
      err = launch_pass<WT, GRID, AFMT, G, kPassInit>(W, in, pa, tiled, b, out, g, PassStats{}, st);
    } else {
      err = launch_pass<WT, GRID, AFMT, G, kPassPlain>(W, in, pa, tiled, b, out, g, PassStats{}, st);
    }
  }
  if (err == hipSuccess && tiled) err = launch_relayout_a<AFMT, G, false>(a_work, a, g, st);
  if (err == hipSuccess && n_iters > 0) {
    bcd_column_kernel<<<(unsigned)g.n_tiles, kTileCols, 0, st>>>(part + ((n_iters - 1) & 1) * half, b, g);
    err = hipGetLastError();
  }
  if (err == hipSuccess && n_iters > 0 && stats) {
    // the final state, against the codes the last pass left
    err = launch_report<WT, GRID, AFMT, G>(W, g.ldw, g.M, g.N, a, b, stats->codes, nullptr,
                                           stats->out + 3 * n_iters, stats->part, st);
  }
  return err;
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_pack(const void* W, int64_t ldw, int64_t M, int64_t N, const void* a,
                       const uint16_t* b, uint8_t* packed, hipStream_t st) {
  const int64_t n_rg = (M + kPackRows - 1) / kPackRows;
  pack_kernel<WT, GRID, AFMT, G, false><<<blocks_for(n_rg * (N / 16), 256), 256, 0, st>>>(
      W, ldw, M, N, a, b, packed, nullptr, nullptr);
  return hipGetLastError();
}

template <int WT, int GRID, int AFMT, int G>
hipError_t launch_report(const void* W, int64_t ldw, int64_t M, int64_t N, const void* a,
                         const uint16_t* b, const uint8_t* prev, uint8_t* packed, double* report,
                         double* part, hipStream_t st) {
  const int64_t n_wg = report_workgroups(M, N);
  pack_kernel<WT, GRID, AFMT, G, true><<<(unsigned)n_wg, 256, 0, st>>>(W, ldw, M, N, a, b, packed, prev,
                                                                       part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  report_reduce_kernel<<<1, 256, 0, st>>>(part, n_wg, report);
  return hipGetLastError();
}

template <int GRID, int AFMT, int G>
hipError_t launch_act(const uint16_t* X, int64_t ldx, int64_t T, int64_t N, const uint16_t* b,
                      uint8_t* xq, void* xs, hipStream_t st) {
  const int64_t n_tg = (T + kActTokens - 1) / kActTokens;
  act_quant_kernel<GRID, AFMT, G><<<blocks_for(n_tg * (N / 8), 256), 256, 0, st>>>(X, ldx, T, N, b, xq,
                                                                                 xs);
  return hipGetLastError();
}

// Explicit instantiation of every supported (weight type, grid, scale
// format, group) combination.
#define DQ_INST_WGA(WT, GR, AF, G)                                                               \
  template hipError_t launch_init<WT, GR, AF, G>(const void*, int64_t, int64_t, int64_t, void*,  \
                                                 uint16_t*, hipStream_t);                         \
  template hipError_t launch_init_colnorm<WT, GR, AF, G>(const void*, int64_t, int64_t, int64_t, \
                                                         void*, uint16_t*, double*, hipStream_t); \
  template hipError_t launch_iterate<WT, GR, AF, G>(const void*, void*, uint16_t*, double*,      \
                                                    const PassGeom&, int, const IterStats*, bool,  \
                                                    void*, hipStream_t);                           \
  template hipError_t launch_pack<WT, GR, AF, G>(const void*, int64_t, int64_t, int64_t,          \
                                                 const void*, const uint16_t*, uint8_t*,          \
                                                 hipStream_t);                                    \
  template hipError_t launch_report<WT, GR, AF, G>(const void*, int64_t, int64_t, int64_t,        \
                                                   const void*, const uint16_t*, const uint8_t*,  \
                                                   uint8_t*, double*, double*, hipStream_t);
#define DQ_INST_GA(GR, AF, G)                                                                    \
  DQ_INST_WGA(kWF32, GR, AF, G)                                                                  \
  DQ_INST_WGA(kWBF16, GR, AF, G)                                                                 \
  template hipError_t launch_act<GR, AF, G>(const uint16_t*, int64_t, int64_t, int64_t,          \
                                            const uint16_t*, uint8_t*, void*, hipStream_t);
#define DQ_INST_A(GR, AF) DQ_INST_GA(GR, AF, 16) DQ_INST_GA(GR, AF, 32) DQ_INST_GA(GR, AF, 64)
#define DQ_INST(GR) DQ_INST_A(GR, kScaleFp16) DQ_INST_A(GR, kScaleE8M0) DQ_INST_A(GR, kScaleE4M3)

#ifndef DQ_GRID_INST
DQ_INST(kGridInt4)
DQ_INST(kGridE2M1)
DQ_INST(kGridInt8)
DQ_INST(kGridE4M3)
#else
DQ_INST(DQ_GRID_INST)
#endif

}  // namespace dq
