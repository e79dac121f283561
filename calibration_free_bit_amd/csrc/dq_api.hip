// dq_api.hip -- the C ABI declared in include/dq.h: argument validation,
// workspace sizing and dispatch to the templated kernels. Everything is
// enqueued on the caller's stream; nothing is allocated.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "dq.h"
#include "dq_device.h"
#include "dq_kernels.h"

namespace {

using dq::PassGeom;

constexpr int kAbiVersion = 1;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int elem_size(int32_t w_type) { return w_type == DQ_W_F32 ? 4 : 2; }

// Shape and format checks shared by every entry point.
int check_problem(const dq_problem* p) {
  if (!p) return DQ_ERR_INVALID_ARG;
  if (p->group != 16 && p->group != 32 && p->group != 64) return DQ_ERR_UNSUPPORTED;
  if (p->grid != DQ_GRID_INT4 && p->grid != DQ_GRID_E2M1 && p->grid != DQ_GRID_INT8 &&
      p->grid != DQ_GRID_E4M3)
    return DQ_ERR_UNSUPPORTED;
  if (p->a_fmt != DQ_SCALE_FP16 && p->a_fmt != DQ_SCALE_E8M0 && p->a_fmt != DQ_SCALE_E4M3)
    return DQ_ERR_UNSUPPORTED;
  if (p->b_fmt != DQ_SCALE_FP16) return DQ_ERR_UNSUPPORTED;
  if (p->w_type != DQ_W_F32 && p->w_type != DQ_W_BF16) return DQ_ERR_UNSUPPORTED;
  if (p->rows < 1 || p->cols < 1 || p->cols % p->group != 0) return DQ_ERR_SHAPE;
  // the pass kernel takes its geometry as 32-bit kernel arguments
  if (p->rows >= (int64_t(1) << 31) || p->ldw >= (int64_t(1) << 31)) return DQ_ERR_SHAPE;
  if (p->ldw < p->cols || (p->ldw * elem_size(p->w_type)) % 16 != 0) return DQ_ERR_SHAPE;
  if (p->rows > (int64_t(1) << 40) / p->ldw) return DQ_ERR_SHAPE;  // keep offsets far from overflow
  // the pass kernel's tile/step bookkeeping is 32-bit
  if (ceil_div(p->rows, dq::kRowsPerStep) * ceil_div(p->cols, dq::kTileCols) >= (int64_t(1) << 31))
    return DQ_ERR_SHAPE;
  return DQ_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

struct Workspace {
  PassGeom g;
  size_t bytes;        // everything but dq_bcd_iterate with statistics
  size_t pass_bytes;   // the two partial-sum buffers of the passes
  size_t codes_bytes;  // one state's codes (statistics)
  size_t stats_bytes;  // dq_bcd_iterate with statistics
  size_t a_work_bytes; // the passes' tile-major block scales, after the partials (or 0)
  bool a_tiled;        // the passes keep the block scales tile-major
};

Workspace pass_geometry(const dq_problem* p) {
  Workspace w{};
  PassGeom& g = w.g;
  g.ldw = p->ldw;
  g.M = p->rows;
  g.N = p->cols;
  g.S = ceil_div(p->rows, dq::kRowsPerStep);
  g.n_tiles = ceil_div(p->cols, dq::kTileCols);
  g.total = g.S * g.n_tiles;
  // at least 4 row steps per workgroup once there are 256 workgroups (one
  // per CU): fewer prologues and partials per tile for small matrices. In
  // the Llama-3.1-8B set (two streams) this takes the 1024x4096 k/v
  // projections from 512 to 256 workgroups: 87.7 -> 86.9 ms per step.
  g.L = std::max<int64_t>(ceil_div(g.total, dq::kPassGrid), std::min<int64_t>(4, g.total / 256));
  g.n_wg = ceil_div(g.total, g.L);
  g.max_seg = 0;
  for (int64_t t = 0; t < g.n_tiles; ++t) {
    const int64_t first = (t * g.S) / g.L, last = ((t + 1) * g.S - 1) / g.L;
    g.max_seg = std::max(g.max_seg, last - first + 1);
  }
  // two alternating buffers of [n_tiles][max_seg][64][2] float64 partials;
  // the column-norm initialization uses [n_tiles][chunks][64] float64
  const size_t pass_bytes = 2 * size_t(g.n_tiles) * size_t(g.max_seg) * dq::kTileCols * 2 * sizeof(double);
  const size_t init_bytes = size_t(g.n_tiles) * size_t(ceil_div(p->rows, dq::kColnormRows)) *
                            dq::kTileCols * sizeof(double);
  // the report uses [workgroups][3] float64
  const int64_t report_wg = dq::report_workgroups(p->rows, p->cols);
  const size_t report_bytes = size_t(report_wg) * 3 * sizeof(double);
  // A tile's workgroups own row ranges; a row of block scales spans many
  // tiles, so in the row-major layout one cache line of scales is written by
  // the workgroups of many tiles. Where a tile's k-th row range always lands
  // on die k (whole segments, a multiple of kXcds per tile, workgroups
  // dispatched to the dies in turn) those writes meet in one L2. Otherwise,
  // for one-byte scales (E8M0, E4M3) large enough to matter, the passes use
  // a tile-major copy in the workspace: NVFP4 on 4096x14336 fetched and
  // wrote 1.47x its algorithmic bytes with the row-major scales. fp16 scales
  // stay row-major: in the Llama-3.1-8B set the copies of its 4096x14336
  // matrices cost more than they saved (87.1 against 86.5 ms per step).
  const int scale_bytes = p->a_fmt == DQ_SCALE_FP16 ? 2 : 1;
  const bool aligned = g.S % g.L == 0 && (g.S / g.L) % dq::kXcds == 0;
  w.a_tiled = !aligned && scale_bytes == 1 && p->rows * (p->cols / p->group) >= (int64_t(1) << 20);
  w.a_work_bytes = w.a_tiled ? align256(dq::tile_major_a_bytes(g, p->group, scale_bytes)) : 0;
  w.bytes = align256(std::max({align256(pass_bytes) + w.a_work_bytes, init_bytes, report_bytes}));
  // with statistics: the partials, the (unused) room of the tile-major
  // scales, the codes of a state, then the per-workgroup sums of a pass or
  // of the final report
  const int code_bits = (p->grid == DQ_GRID_INT8 || p->grid == DQ_GRID_E4M3) ? 8 : 4;
  w.pass_bytes = align256(pass_bytes);
  w.codes_bytes = align256(size_t(p->rows) * size_t(p->cols) * code_bits / 8);
  const size_t sums_bytes = align256(size_t(std::max(g.n_wg, report_wg)) * 3 * sizeof(double));
  w.stats_bytes = std::max(w.bytes, w.pass_bytes + w.a_work_bytes + w.codes_bytes + sums_bytes);
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DQ_OK : DQ_ERR_HIP; }

// Scratch of dq_bcd_iterate_noalloc: the two alternating buffers of partial
// column sums, in a fixed array that every GPU the library runs on holds
// for the life of the process. Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) unsigned char scratch[DQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or nullptr on failure.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Calls f.template operator()<WT, GRID, AFMT, G>() for p's format.
template <class F>
int dispatch(const dq_problem& p, F&& f) {
  auto by_group = [&]<int WT, int GR, int AF>() -> int {
    switch (p.group) {
      case 16: return f.template operator()<WT, GR, AF, 16>();
      case 32: return f.template operator()<WT, GR, AF, 32>();
      case 64: return f.template operator()<WT, GR, AF, 64>();
    }
    return DQ_ERR_UNSUPPORTED;
  };
  auto by_afmt = [&]<int WT, int GR>() -> int {
    switch (p.a_fmt) {
      case DQ_SCALE_FP16: return by_group.template operator()<WT, GR, dq::kScaleFp16>();
      case DQ_SCALE_E8M0: return by_group.template operator()<WT, GR, dq::kScaleE8M0>();
      case DQ_SCALE_E4M3: return by_group.template operator()<WT, GR, dq::kScaleE4M3>();
    }
    return DQ_ERR_UNSUPPORTED;
  };
  auto by_grid = [&]<int WT>() -> int {
    switch (p.grid) {
      case DQ_GRID_INT4: return by_afmt.template operator()<WT, dq::kGridInt4>();
      case DQ_GRID_E2M1: return by_afmt.template operator()<WT, dq::kGridE2M1>();
      case DQ_GRID_INT8: return by_afmt.template operator()<WT, dq::kGridInt8>();
      case DQ_GRID_E4M3: return by_afmt.template operator()<WT, dq::kGridE4M3>();
    }
    return DQ_ERR_UNSUPPORTED;
  };
  switch (p.w_type) {
    case DQ_W_F32: return by_grid.template operator()<dq::kWF32>();
    case DQ_W_BF16: return by_grid.template operator()<dq::kWBF16>();
  }
  return DQ_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

int dq_abi_version(void) { return kAbiVersion; }

const char* dq_status_string(int status) {
  switch (status) {
    case DQ_OK: return "ok";
    case DQ_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad count)";
    case DQ_ERR_SHAPE: return "inconsistent shape (rows/cols/ld, or cols not a multiple of G)";
    case DQ_ERR_UNSUPPORTED: return "unsupported format combination";
    case DQ_ERR_WORKSPACE: return "workspace missing or too small";
    case DQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t dq_workspace_bytes(const dq_problem* p) {
  if (check_problem(p) != DQ_OK) return 0;
  return pass_geometry(p).bytes;
}

size_t dq_stats_workspace_bytes(const dq_problem* p) {
  if (check_problem(p) != DQ_OK) return 0;
  return pass_geometry(p).stats_bytes;
}

int dq_init_rtn(const dq_problem* p, const void* W, void* a, uint16_t* b, void* stream) {
  if (int s = check_problem(p)) return s;
  if (!W || !a || !b || !aligned16(W)) return DQ_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    return hip_status(dq::launch_init<WT, GR, AF, G>(W, p->ldw, p->rows, p->cols, a, b, st));
  });
}

int dq_init_colnorm(const dq_problem* p, const void* W, void* a, uint16_t* b, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (int s = check_problem(p)) return s;
  if (!W || !a || !b || !aligned16(W)) return DQ_ERR_INVALID_ARG;
  const Workspace ws = pass_geometry(p);
  if (!workspace || workspace_bytes < ws.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return DQ_ERR_WORKSPACE;
  double* part = static_cast<double*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    return hip_status(dq::launch_init_colnorm<WT, GR, AF, G>(W, p->ldw, p->rows, p->cols, a, b, part, st));
  });
}

int dq_bcd_iterate(const dq_problem* p, const void* W, void* a, uint16_t* b, int32_t n_iters,
                   void* workspace, size_t workspace_bytes, double* stats, void* stream) {
  if (int s = check_problem(p)) return s;
  if (!W || !a || !b || !aligned16(W) || n_iters < 0) return DQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(stats) & 7u) return DQ_ERR_INVALID_ARG;
  if (n_iters == 0 && !stats) return DQ_OK;
  const Workspace ws = pass_geometry(p);
  if (!workspace || workspace_bytes < (stats ? ws.stats_bytes : ws.bytes) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return DQ_ERR_WORKSPACE;
  double* part = static_cast<double*>(workspace);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint8_t* codes = base + ws.pass_bytes + ws.a_work_bytes;
  const dq::IterStats its{stats, codes, reinterpret_cast<double*>(codes + ws.codes_bytes)};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    if (n_iters == 0)  // row 0 alone: the state passed in, no code changed
      return hip_status(dq::launch_report<WT, GR, AF, G>(W, p->ldw, p->rows, p->cols, a, b, nullptr,
                                                         nullptr, stats, its.part, st));
    void* a_work = ws.a_tiled && !stats ? base + ws.pass_bytes : nullptr;
    return hip_status(dq::launch_iterate<WT, GR, AF, G>(W, a, b, part, ws.g, n_iters, stats ? &its : nullptr,
                                                        false, a_work, st));
  });
}

int dq_bcd_iterate_noalloc(const dq_problem* p, const void* W, void* a, uint16_t* b, int32_t n_iters,
                           void* stream) {
  if (int s = check_problem(p)) return s;
  if (!W || !a || !b || !aligned16(W) || n_iters < 0) return DQ_ERR_INVALID_ARG;
  const Workspace ws = pass_geometry(p);
  if (ws.pass_bytes > DQ_NOALLOC_SCRATCH_BYTES) return DQ_ERR_WORKSPACE;
  if (n_iters == 0) return DQ_OK;
  // every pass writes its partials before the next one reads them and the
  // first pass reads none, so the scratch needs no clearing
  double* part = static_cast<double*>(scratch_address());
  if (!part) return DQ_ERR_HIP;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    return hip_status(
        dq::launch_iterate<WT, GR, AF, G>(W, a, b, part, ws.g, n_iters, nullptr, false, nullptr, st));
  });
}

int dq_solve(const dq_problem* p, const void* W, void* a, uint16_t* b, int32_t n_iters,
             uint8_t* packed, void* workspace, size_t workspace_bytes, void* stream) {
  if (int s = check_problem(p)) return s;
  const bool byte_codes = p->grid == DQ_GRID_INT8 || p->grid == DQ_GRID_E4M3;
  if (!W || !a || !b || !packed || !aligned16(W) || !aligned16(b) || n_iters < 0 ||
      (reinterpret_cast<uintptr_t>(packed) & (byte_codes ? 15u : 7u)))
    return DQ_ERR_INVALID_ARG;
  const Workspace ws = pass_geometry(p);
  if (!workspace || workspace_bytes < ws.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return DQ_ERR_WORKSPACE;
  double* part = static_cast<double*>(workspace);
  void* a_work = ws.a_tiled ? static_cast<uint8_t*>(workspace) + ws.pass_bytes : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    hipError_t e = hipSuccess;
    if (n_iters == 0)
      e = dq::launch_init<WT, GR, AF, G>(W, p->ldw, p->rows, p->cols, a, b, st);
    else
      e = dq::launch_iterate<WT, GR, AF, G>(W, a, b, part, ws.g, n_iters, nullptr, true, a_work, st);
    if (e == hipSuccess)
      e = dq::launch_pack<WT, GR, AF, G>(W, p->ldw, p->rows, p->cols, a, b, packed, st);
    return hip_status(e);
  });
}

int dq_pack_codes(const dq_problem* p, const void* W, const void* a, const uint16_t* b,
                  uint8_t* packed, void* stream) {
  if (int s = check_problem(p)) return s;
  const bool byte_codes = p->grid == DQ_GRID_INT8 || p->grid == DQ_GRID_E4M3;
  if (!W || !a || !b || !packed || !aligned16(W) || !aligned16(b) ||
      (reinterpret_cast<uintptr_t>(packed) & (byte_codes ? 15u : 7u)))
    return DQ_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    return hip_status(dq::launch_pack<WT, GR, AF, G>(W, p->ldw, p->rows, p->cols, a, b, packed, st));
  });
}

int dq_quant_report(const dq_problem* p, const void* W, const void* a, const uint16_t* b,
                    const uint8_t* prev_packed, uint8_t* packed, double* report, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (int s = check_problem(p)) return s;
  const uintptr_t code_align = (p->grid == DQ_GRID_INT8 || p->grid == DQ_GRID_E4M3) ? 15u : 7u;
  if (!W || !a || !b || !report || !aligned16(W) || !aligned16(b) ||
      (reinterpret_cast<uintptr_t>(packed) & code_align) ||
      (reinterpret_cast<uintptr_t>(prev_packed) & code_align) ||
      (reinterpret_cast<uintptr_t>(report) & 7u))
    return DQ_ERR_INVALID_ARG;
  const Workspace ws = pass_geometry(p);
  if (!workspace || workspace_bytes < ws.bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return DQ_ERR_WORKSPACE;
  double* part = static_cast<double*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    return hip_status(dq::launch_report<WT, GR, AF, G>(W, p->ldw, p->rows, p->cols, a, b, prev_packed,
                                                       packed, report, part, st));
  });
}

int dq_rescale_quantize_act(const dq_problem* p, const void* X, int64_t tokens, int64_t ldx,
                            const uint16_t* b, uint8_t* xq, void* x_scales, void* stream) {
  if (int s = check_problem(p)) return s;
  if (p->w_type != DQ_W_BF16) return DQ_ERR_UNSUPPORTED;  // X' = X D_b is exact only for bf16 X
  if (tokens < 0 || ldx < p->cols || (ldx * 2) % 16 != 0) return DQ_ERR_SHAPE;
  if (tokens > (int64_t(1) << 40) / ldx) return DQ_ERR_SHAPE;  // keep offsets and grids in range
  if (tokens == 0) return DQ_OK;
  if (!X || !b || !xq || !x_scales || !aligned16(X) || !aligned16(b) || !aligned16(xq))
    return DQ_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* Xh = static_cast<const uint16_t*>(X);
  return dispatch(*p, [&]<int WT, int GR, int AF, int G>() {
    if constexpr (WT != dq::kWBF16) {
      return int(DQ_ERR_UNSUPPORTED);
    } else {
      return hip_status(dq::launch_act<GR, AF, G>(Xh, ldx, tokens, p->cols, b, xq, x_scales, st));
    }
  });
}

}  // extern "C"
