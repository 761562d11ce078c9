// C ABI of the DBSCAN library: argument checks, workspace carving and the
// launch sequence of one fit.  See include/dbscan.h for the contract.
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <numeric>

#include "dbscan.h"
#include "internal.h"

namespace dbk {

int pick_dim(int d) {
  for (int D : kDims)
    if (D >= d) return D;
  return 0;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static int64_t pad_points(int64_t n, int D) {
  const int64_t m = pad_multiple(D);
  return (n + m - 1) / m * m;
}

static int64_t tile_capacity(int64_t n_pad, int D) {
  const int64_t nb = n_pad / block_points(D);
  const int64_t all = nb * (nb + 1) / 2;
  return all < kTileListCap ? all : kTileListCap;
}

constexpr int kRegions = 25;

// Region sizes in carve order; every region starts 256-byte aligned.
static size_t regions(int64_t n_pad, int D, size_t* out) {
  const size_t np = (size_t)n_pad;
  const size_t S = (size_t)row_stride(D);
  const size_t nb = np / (size_t)block_points(D);
  size_t sz[kRegions] = {
      sizeof(Status),                // status
      np * S * sizeof(float),        // pts
      np * sizeof(unsigned),         // count
      np,                            // core
      np * sizeof(int),              // parent
      np * sizeof(int),              // bmin
      np * sizeof(int),              // cmin
      np * sizeof(int),              // core_list
      np * S * sizeof(float),        // core_pts
      (np / 1024 + 1) * sizeof(unsigned),  // block_sums
      12 * sizeof(unsigned),         // bbox
      np * sizeof(unsigned),         // keys_in
      np * sizeof(unsigned),         // keys_out
      np * sizeof(int),              // idx_in
      np * sizeof(int),              // perm
      np * S * sizeof(float),        // sorted_pts
      nb * 2 * S * sizeof(float),    // boxes
      (size_t)tile_capacity(n_pad, D) * sizeof(uint2),  // tiles
      np / 64 * 2 * S * sizeof(float),                   // boxes64
      np / (64 * (size_t)lane_points(D)) * 2 * S * sizeof(float),  // boxes_w
      np * (size_t)screen_stride(D) * sizeof(float),  // srow
      np * sizeof(float),            // ncol
      np * sizeof(float),            // nexp
      (7 * S + 1) * sizeof(float),   // pca
      prune_sort_bytes(n_pad),       // key sort counts
  };
  size_t total = 0;
  for (int r = 0; r < kRegions; ++r) {
    if (out) out[r] = total;
    total += align_up(sz[r], 256);
  }
  return total;
}

size_t layout_min_bytes(int64_t n, int d) {
  const int D = pick_dim(d);
  if (n < 0 || n > INT32_MAX || D == 0) return 0;
  return regions(pad_points(n < 1 ? 1 : n, D), D, nullptr);
}

bool carve(Layout& L, void* ws, size_t ws_bytes) {
  size_t off[kRegions];
  const size_t need = regions(L.n_pad, L.D, off);
  if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws & 255u)) return false;
  char* b = static_cast<char*>(ws);
  L.status = reinterpret_cast<Status*>(b + off[0]);
  L.pts = reinterpret_cast<float*>(b + off[1]);
  L.count = reinterpret_cast<unsigned*>(b + off[2]);
  L.core = reinterpret_cast<unsigned char*>(b + off[3]);
  L.parent = reinterpret_cast<int*>(b + off[4]);
  L.bmin = reinterpret_cast<int*>(b + off[5]);
  L.cmin = reinterpret_cast<int*>(b + off[6]);
  L.core_list = reinterpret_cast<int*>(b + off[7]);
  L.core_pts = reinterpret_cast<float*>(b + off[8]);
  L.block_sums = reinterpret_cast<unsigned*>(b + off[9]);
  L.bbox = reinterpret_cast<unsigned*>(b + off[10]);
  L.keys_in = reinterpret_cast<unsigned*>(b + off[11]);
  L.keys_out = reinterpret_cast<unsigned*>(b + off[12]);
  L.idx_in = reinterpret_cast<int*>(b + off[13]);
  L.perm = reinterpret_cast<int*>(b + off[14]);
  L.sorted_pts = reinterpret_cast<float*>(b + off[15]);
  L.boxes = reinterpret_cast<float*>(b + off[16]);
  L.tiles = reinterpret_cast<uint2*>(b + off[17]);
  L.tile_cap = (unsigned long long)tile_capacity(L.n_pad, L.D);
  L.boxes64 = reinterpret_cast<float*>(b + off[18]);
  L.boxes_w = reinterpret_cast<float*>(b + off[19]);
  L.srow = reinterpret_cast<float*>(b + off[20]);
  L.ncol = reinterpret_cast<float*>(b + off[21]);
  L.nexp = reinterpret_cast<float*>(b + off[22]);
  L.pca = reinterpret_cast<float*>(b + off[23]);
  L.sort_hist = reinterpret_cast<unsigned*>(b + off[24]);
  L.bytes_min = need;
  const size_t spare = ws_bytes - need;
  L.edges = reinterpret_cast<uint2*>(b + need);
  L.edge_cap = spare / sizeof(uint2);
  if (L.edge_cap == 0) L.edges = nullptr;
  return true;
}

WalkArgs walk_args(Walk w, int64_t count) {
  if (w.seed == 0 || count <= 1) return WalkArgs{1, 0};
  if (w.seed == 1) return WalkArgs{-1, count - 1};
  // a multiplier in [3, 2^14) coprime with count, and an offset, from the
  // seed (a fixed bijection of 0 .. count-1)
  const uint64_t h = (uint64_t)w.seed * 0x9E3779B97F4A7C15ull;
  int64_t mul = 3 + (int64_t)((h >> 20) % 16000u);
  while (std::gcd(mul, count) != 1) mul = mul + 1 < 16384 ? mul + 1 : 3;
  return WalkArgs{mul, (int64_t)((h >> 7) % (uint64_t)count)};
}

}  // namespace dbk

using namespace dbk;

namespace {

constexpr uint32_t kKnownFlags = DBSCAN_FLAG_TIME_PHASES |
                                  DBSCAN_FLAG_FORCE_TILE_MERGE |
                                  DBSCAN_FLAG_PRUNE_TILES |
                                  DBSCAN_FLAG_SCREEN |
                                  DBSCAN_FLAG_REVERSE_SCHEDULE |
                                  DBSCAN_FLAG_EXPANDED |
                                  DBSCAN_FLAG_SHUFFLE_SCHEDULE;

int check_args(int64_t n, int32_t d, float eps, int32_t min_pts) {
  if (n < 0 || n > (int64_t)INT32_MAX) return DBSCAN_ERR_INVALID_ARG;
  if (d < 1 || d > DBSCAN_MAX_D) return DBSCAN_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || std::isinf(eps)) return DBSCAN_ERR_INVALID_ARG;
  if (min_pts < 1) return DBSCAN_ERR_INVALID_ARG;
  return DBSCAN_OK;
}

int map_hip(hipError_t e) {
  if (e == hipSuccess) return DBSCAN_OK;
  if (e == hipErrorNoDevice || e == hipErrorNoBinaryForGpu ||
      e == hipErrorInvalidDeviceFunction || e == hipErrorInsufficientDriver)
    return DBSCAN_ERR_NO_DEVICE;
  if (e == hipErrorOutOfMemory) return DBSCAN_ERR_OOM;
  return DBSCAN_ERR_HIP;
}

int have_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return DBSCAN_ERR_NO_DEVICE;
  }
  return DBSCAN_OK;
}

// Phase timing with HIP events on the fit's stream.
struct PhaseTimer {
  bool on = false;
  hipEvent_t ev[6] = {};
  hipStream_t s = nullptr;
  explicit PhaseTimer(bool enable, hipStream_t stream) : s(stream) {
    if (!enable) return;
    on = true;
    for (auto& e : ev)
      if (hipEventCreate(&e) != hipSuccess) on = false;
  }
  void mark(int k) {
    if (on) (void)hipEventRecord(ev[k], s);
  }
  float ms(int a, int b) {
    float t = 0.f;
    if (on && hipEventElapsedTime(&t, ev[a], ev[b]) != hipSuccess) t = -1.f;
    return t;
  }
  ~PhaseTimer() {
    for (auto& e : ev)
      if (e) (void)hipEventDestroy(e);
  }
};

#define DB_TRY(expr)                      \
  do {                                    \
    hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) {               \
      (void)hipStreamSynchronize(stream); \
      if (info) info->hip_error = (int32_t)e_; \
      return map_hip(e_);                 \
    }                                     \
  } while (0)

// Graph export: after the fit's regions come the row cursors and the
// row-offset scan totals; the rest of the workspace holds the captured
// pairs and, once they are scattered, serves as the row sort's second
// buffer (4 bytes per graph entry: 4n + 8 per pair).
size_t graph_fixed_bytes(int64_t n_pad) {
  return align_up((size_t)n_pad * sizeof(unsigned), 256) +
         align_up(((size_t)n_pad / 1024 + 2) * sizeof(unsigned long long), 256);
}

bool carve_graph(Layout& L, GraphLayout& G, void* ws, size_t ws_bytes) {
  if (!carve(L, ws, ws_bytes)) return false;
  const size_t spare = ws_bytes - L.bytes_min;
  const size_t fixed = graph_fixed_bytes(L.n_pad);
  const size_t alt_min = (size_t)L.n_pad * sizeof(int);
  if (spare < fixed + alt_min) return false;
  char* b = static_cast<char*>(ws) + L.bytes_min;
  G.cursor = reinterpret_cast<unsigned*>(b);
  b += align_up((size_t)L.n_pad * sizeof(unsigned), 256);
  G.row_sums = reinterpret_cast<unsigned long long*>(b);
  b += align_up(((size_t)L.n_pad / 1024 + 2) * sizeof(unsigned long long), 256);
  const size_t rest = spare - fixed;
  G.alt = b;
  L.edges = reinterpret_cast<uint2*>(b);
  L.edge_cap = (rest - alt_min) / sizeof(uint2);
  return true;
}

// ---- fixed scratch of the no-allocation entry point ------------------------
// One copy of this array lives on every GPU the library runs on, from the
// code object's load until the process ends.  In host code its name is a
// host-side stand-in, not a device address: the device address of the
// current GPU's copy comes from hipGetSymbolAddress, once per device, and
// only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[DBSCAN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxScratchDevices] = {};

// The current device's copy of `scratch`, looked up on this device's first
// call and kept.
int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return map_hip(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return DBSCAN_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return e != hipSuccess ? map_hip(e) : DBSCAN_ERR_HIP;
    }
    scratch_addr[dev] = ptr;
  }
  *out = scratch_addr[dev];
  return DBSCAN_OK;
}

}  // namespace

extern "C" {

size_t dbscan_workspace_bytes(int64_t n, int32_t d) {
  if (d < 1 || d > DBSCAN_MAX_D) return 0;
  return layout_min_bytes(n, d);
}

size_t dbscan_workspace_bytes_with_edges(int64_t n, int32_t d,
                                         int64_t max_edges) {
  const size_t base = dbscan_workspace_bytes(n, d);
  if (base == 0 || max_edges < 0) return 0;
  return align_up(base + (size_t)max_edges * sizeof(uint2), 256);
}

int dbscan_abi_version(void) { return DBSCAN_ABI_VERSION; }

const char* dbscan_status_string(int status) {
  switch (status) {
    case DBSCAN_OK: return "ok";
    case DBSCAN_ERR_INVALID_ARG: return "invalid argument";
    case DBSCAN_ERR_NONFINITE: return "a coordinate is NaN or infinite";
    case DBSCAN_ERR_NO_DEVICE: return "no usable gfx950 HIP device";
    case DBSCAN_ERR_OOM: return "device memory allocation failed";
    case DBSCAN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case DBSCAN_ERR_HIP: return "HIP runtime error";
    case DBSCAN_ERR_CAPACITY: return "output buffer too small (size reported)";
    case DBSCAN_ERR_TOO_LARGE:
      return "input too large for the fixed scratch of the no-allocation entry";
    default: return "unknown status";
  }
}

int dbscan_fit_device_ex(const float* d_points, int64_t n, int32_t d,
                         float eps, int32_t min_pts, int32_t* d_labels,
                         int32_t* d_counts, void* d_workspace,
                         size_t workspace_bytes, void* hip_stream,
                         uint32_t flags, dbscan_info* info) {
  if (info) std::memset(info, 0, sizeof(*info));
  int st = check_args(n, d, eps, min_pts);
  if (st != DBSCAN_OK) return st;
  // bits 16..31 carry the shuffle's seed, and only with the shuffle flag
  if ((flags & 0xffffu) & ~kKnownFlags) return DBSCAN_ERR_INVALID_ARG;
  if ((flags >> 16) && !(flags & DBSCAN_FLAG_SHUFFLE_SCHEDULE))
    return DBSCAN_ERR_INVALID_ARG;
  if ((flags & DBSCAN_FLAG_SHUFFLE_SCHEDULE) &&
      (flags & DBSCAN_FLAG_REVERSE_SCHEDULE))
    return DBSCAN_ERR_INVALID_ARG;
  if ((flags & DBSCAN_FLAG_EXPANDED) && (flags & DBSCAN_FLAG_PRUNE_TILES))
    return DBSCAN_ERR_INVALID_ARG;
  if (n > 0 && (d_points == nullptr || d_labels == nullptr))
    return DBSCAN_ERR_INVALID_ARG;
  if (n == 0) return DBSCAN_OK;
  st = have_device();
  if (st != DBSCAN_OK) return st;
  (void)hipGetLastError();  // launch checks below must not see older errors

  Layout L{};
  L.n = n;
  L.d = d;
  L.D = pick_dim(d);
  L.stride = row_stride(L.D);
  L.n_pad = pad_points(n, L.D);
  L.expanded = (flags & DBSCAN_FLAG_EXPANDED) != 0;
  if (!carve(L, d_workspace, workspace_bytes)) return DBSCAN_ERR_WORKSPACE;

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  // eps^2 rounded once in fp32, as the comparison threshold of every pair
  volatile float eps_v = eps;
  const float eps2 = eps_v * eps_v;
  const bool want_edges =
      L.edge_cap > 0 && !(flags & DBSCAN_FLAG_FORCE_TILE_MERGE);
  const bool prune = (flags & DBSCAN_FLAG_PRUNE_TILES) != 0;
  // the hoisted-norm form is always evaluated behind the screen
  const bool screen = (flags & (DBSCAN_FLAG_SCREEN | DBSCAN_FLAG_EXPANDED)) != 0;
  const Walk walk{(flags & DBSCAN_FLAG_REVERSE_SCHEDULE)   ? 1u
                  : (flags & DBSCAN_FLAG_SHUFFLE_SCHEDULE) ? 2u + (flags >> 16)
                                                           : 0u};
  PhaseTimer tm((flags & DBSCAN_FLAG_TIME_PHASES) != 0, stream);
  int64_t pass1 = 0;

  tm.mark(0);
  DB_TRY(launch_prepare(L, d_points, stream));
  if (prune) DB_TRY(launch_prune(L, block_points(L.D), eps2, stream));
  if (screen)
    DB_TRY(launch_screen(L, prune ? L.sorted_pts : L.pts, eps2, stream));
  tm.mark(1);
  DB_TRY(launch_count(L, eps2, want_edges, prune, screen, walk, stream,
                      &pass1));
  tm.mark(2);
  DB_TRY(launch_core(L, min_pts, d_counts, stream));
  tm.mark(3);
  // The merge is chosen on the device from the pair count: one launch
  // links the recorded pairs or compacts the cores for the tile merge,
  // which follows and exits at once when it is not needed.  No host round
  // trip until the end.
  // An edge area that holds every pair i<j can never overflow: then the
  // tile merge is not enqueued at all.
  const bool tiles_possible =
      !want_edges || 0.5 * (double)n * (double)(n - 1) > (double)L.edge_cap;
  DB_TRY(launch_merge_edges(L, want_edges, walk, prune, stream));
  if (tiles_possible)
    DB_TRY(launch_merge_tiles(L, eps2, want_edges, walk, stream));
  tm.mark(4);
  DB_TRY(launch_label(L, d_labels, stream));
  tm.mark(5);
  // the one synchronisation of a fit: the status block, then the stream
  Status host_st;
  DB_TRY(hipMemcpyAsync(&host_st, L.status, sizeof(Status),
                        hipMemcpyDeviceToHost, stream));
  DB_TRY(hipStreamSynchronize(stream));
  if (host_st.nonfinite) return DBSCAN_ERR_NONFINITE;
  const int64_t n_core = host_st.n_core;
  const bool edges_ok = want_edges && host_st.n_edges <= L.edge_cap;
  if (!edges_ok && n_core > 0 && (int64_t)host_st.n_core_list != n_core)
    return DBSCAN_ERR_HIP;

  if (info) {
    info->n_core = n_core;
    info->n_edges = want_edges ? (int64_t)host_st.n_edges : 0;
    info->edge_capacity = (int64_t)L.edge_cap;
    const int64_t nb = L.n_pad / block_points(L.D);
    info->tiles_total = nb * (nb + 1) / 2;
    info->tiles_kept = prune && host_st.n_tiles <= L.tile_cap
                           ? (int64_t)host_st.n_tiles
                           : info->tiles_total;
    info->pass1_pairs = pass1;
    // the tile merge evaluates every point against the cores, padded to
    // whole column blocks
    const int64_t T = block_points(L.D);
    info->pass2_pairs =
        edges_ok ? 0 : L.n_pad * ((n_core + T - 1) / T * T);
    info->merge_mode = edges_ok ? DBSCAN_MERGE_EDGES : DBSCAN_MERGE_TILES;
    if (tm.on) {
      info->timed = 1;
      info->ms_layout = tm.ms(0, 1);
      info->ms_count = tm.ms(1, 2);
      info->ms_core = tm.ms(2, 3);
      info->ms_merge = tm.ms(3, 4);
      info->ms_label = tm.ms(4, 5);
      info->ms_total = tm.ms(0, 5);
    }
  }
  return DBSCAN_OK;
}

int dbscan_fit_device(const float* d_points, int64_t n, int32_t d, float eps,
                      int32_t min_pts, int32_t* d_labels, int32_t* d_counts,
                      void* d_workspace, size_t workspace_bytes,
                      void* hip_stream) {
  return dbscan_fit_device_ex(d_points, n, d, eps, min_pts, d_labels, d_counts,
                              d_workspace, workspace_bytes, hip_stream, 0u,
                              nullptr);
}

int dbscan_fit_counts(const float* points, int64_t n, int32_t d, float eps,
                      int32_t min_pts, int32_t* labels, int32_t* counts) {
  int st = check_args(n, d, eps, min_pts);
  if (st != DBSCAN_OK) return st;
  if (n > 0 && (points == nullptr || labels == nullptr))
    return DBSCAN_ERR_INVALID_ARG;
  if (n == 0) return DBSCAN_OK;
  st = have_device();
  if (st != DBSCAN_OK) return st;

  const size_t pts_bytes = (size_t)n * d * sizeof(float);
  const size_t lab_bytes = (size_t)n * sizeof(int32_t);
  const size_t ws_min = dbscan_workspace_bytes(n, d);
  float* d_pts = nullptr;
  int32_t* d_lab = nullptr;
  int32_t* d_cnt = nullptr;
  void* d_ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t stream = nullptr;
  int rc = DBSCAN_OK;
  hipError_t e = hipStreamCreate(&stream);
  if (e != hipSuccess) return map_hip(e);
  do {
    if ((e = hipMalloc(&d_pts, pts_bytes)) != hipSuccess) break;
    if ((e = hipMalloc(&d_lab, lab_bytes)) != hipSuccess) break;
    if (counts && (e = hipMalloc(&d_cnt, lab_bytes)) != hipSuccess) break;
    // edge area: up to a quarter of the free memory, at most 16 GiB, and
    // no more than every pair i<j of the input could take
    size_t free_b = 0, total_b = 0;
    if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) free_b = 0;
    size_t edge_bytes = free_b / 4;
    if (edge_bytes > ((size_t)16 << 30)) edge_bytes = (size_t)16 << 30;
    const double all_pairs = 0.5 * (double)n * (double)(n - 1) * sizeof(uint2);
    if ((double)edge_bytes > all_pairs) edge_bytes = (size_t)all_pairs;
    ws_bytes = ws_min + align_up(edge_bytes, 256);
    if (hipMalloc(&d_ws, ws_bytes) != hipSuccess) {
      (void)hipGetLastError();
      ws_bytes = ws_min;  // no edge area: the tile merge is used
      if ((e = hipMalloc(&d_ws, ws_bytes)) != hipSuccess) break;
    }
    if ((e = hipMemcpyAsync(d_pts, points, pts_bytes, hipMemcpyHostToDevice,
                            stream)) != hipSuccess)
      break;
    rc = dbscan_fit_device(d_pts, n, d, eps, min_pts, d_lab, d_cnt, d_ws,
                           ws_bytes, stream);
    if (rc != DBSCAN_OK) break;
    if ((e = hipMemcpyAsync(labels, d_lab, lab_bytes, hipMemcpyDeviceToHost,
                            stream)) != hipSuccess)
      break;
    if (counts && (e = hipMemcpyAsync(counts, d_cnt, lab_bytes,
                                      hipMemcpyDeviceToHost, stream)) !=
                      hipSuccess)
      break;
    e = hipStreamSynchronize(stream);
  } while (false);
  if (rc == DBSCAN_OK && e != hipSuccess) rc = map_hip(e);
  (void)hipStreamSynchronize(stream);
  if (d_ws) (void)hipFree(d_ws);
  if (d_cnt) (void)hipFree(d_cnt);
  if (d_lab) (void)hipFree(d_lab);
  if (d_pts) (void)hipFree(d_pts);
  (void)hipStreamDestroy(stream);
  return rc;
}

int dbscan_fit(const float* points, int64_t n, int32_t d, float eps,
               int32_t min_pts, int32_t* labels) {
  return dbscan_fit_counts(points, n, d, eps, min_pts, labels, nullptr);
}

int dbscan_fit_device_noalloc(const float* d_points, int64_t n, int32_t d,
                              float eps, int32_t min_pts, int32_t* d_labels,
                              int32_t* d_counts, void* hip_stream) {
  int st = check_args(n, d, eps, min_pts);
  if (st != DBSCAN_OK) return st;
  if (n > 0 && (d_points == nullptr || d_labels == nullptr))
    return DBSCAN_ERR_INVALID_ARG;
  if (n == 0) return DBSCAN_OK;
  if (dbscan_workspace_bytes(n, d) > (size_t)DBSCAN_NOALLOC_SCRATCH_BYTES)
    return DBSCAN_ERR_TOO_LARGE;
  st = have_device();
  if (st != DBSCAN_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != DBSCAN_OK) return st;
  // the scratch beyond the fit's minimum is its edge area; the fit clears
  // what must start at zero (status block, counts, forest) itself
  return dbscan_fit_device_ex(d_points, n, d, eps, min_pts, d_labels,
                              d_counts, ws, (size_t)DBSCAN_NOALLOC_SCRATCH_BYTES,
                              hip_stream, 0u, nullptr);
}

size_t dbscan_graph_workspace_bytes(int64_t n, int32_t d, int64_t max_pairs) {
  const size_t base = dbscan_workspace_bytes(n, d);
  if (base == 0 || max_pairs < 0) return 0;
  const int64_t n_pad = pad_points(n < 1 ? 1 : n, pick_dim(d));
  return base + graph_fixed_bytes(n_pad) +
         align_up((size_t)n_pad * sizeof(int) + (size_t)max_pairs * sizeof(uint2),
                  256);
}

int dbscan_graph_device(const float* d_points, int64_t n, int32_t d, float eps,
                        int64_t* d_row_ptr, int32_t* d_col_idx,
                        int64_t col_capacity, int64_t* nnz_out,
                        void* d_workspace, size_t workspace_bytes,
                        void* hip_stream, uint32_t flags, dbscan_info* info) {
  if (info) std::memset(info, 0, sizeof(*info));
  int st = check_args(n, d, eps, 1);
  if (st != DBSCAN_OK) return st;
  if (flags & ~(DBSCAN_FLAG_TIME_PHASES | DBSCAN_FLAG_PRUNE_TILES |
                DBSCAN_FLAG_SCREEN | DBSCAN_FLAG_EXPANDED))
    return DBSCAN_ERR_INVALID_ARG;
  if ((flags & DBSCAN_FLAG_EXPANDED) && (flags & DBSCAN_FLAG_PRUNE_TILES))
    return DBSCAN_ERR_INVALID_ARG;
  if (d_row_ptr == nullptr || col_capacity < 0 ||
      (col_capacity > 0 && d_col_idx == nullptr) ||
      (n > 0 && d_points == nullptr))
    return DBSCAN_ERR_INVALID_ARG;
  st = have_device();
  if (st != DBSCAN_OK) return st;
  (void)hipGetLastError();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (n == 0) {
    const int64_t zero = 0;
    DB_TRY(hipMemcpyAsync(d_row_ptr, &zero, sizeof(zero),
                          hipMemcpyHostToDevice, stream));
    DB_TRY(hipStreamSynchronize(stream));
    if (nnz_out) *nnz_out = 0;
    return DBSCAN_OK;
  }

  Layout L{};
  GraphLayout G{};
  L.n = n;
  L.d = d;
  L.D = pick_dim(d);
  L.stride = row_stride(L.D);
  L.n_pad = pad_points(n, L.D);
  L.expanded = (flags & DBSCAN_FLAG_EXPANDED) != 0;
  if (!carve_graph(L, G, d_workspace, workspace_bytes))
    return DBSCAN_ERR_WORKSPACE;

  volatile float eps_v = eps;
  const float eps2 = eps_v * eps_v;
  const bool prune = (flags & DBSCAN_FLAG_PRUNE_TILES) != 0;
  const bool screen = (flags & (DBSCAN_FLAG_SCREEN | DBSCAN_FLAG_EXPANDED)) != 0;
  const unsigned long long col_cap = (unsigned long long)col_capacity;
  PhaseTimer tm((flags & DBSCAN_FLAG_TIME_PHASES) != 0, stream);
  int64_t pass1 = 0;

  tm.mark(0);
  DB_TRY(launch_prepare(L, d_points, stream));
  if (prune) DB_TRY(launch_prune(L, block_points(L.D), eps2, stream));
  if (screen)
    DB_TRY(launch_screen(L, prune ? L.sorted_pts : L.pts, eps2, stream));
  tm.mark(1);
  DB_TRY(launch_count(L, eps2, true, prune, screen, Walk{0}, stream, &pass1));
  tm.mark(2);
  DB_TRY(launch_row_offsets(L, G, d_row_ptr, d_col_idx, col_cap, stream));
  Status host_st;
  int64_t nnz = 0;
  DB_TRY(hipMemcpyAsync(&host_st, L.status, sizeof(Status),
                        hipMemcpyDeviceToHost, stream));
  DB_TRY(hipMemcpyAsync(&nnz, d_row_ptr + n, sizeof(nnz),
                        hipMemcpyDeviceToHost, stream));
  DB_TRY(hipStreamSynchronize(stream));
  if (host_st.nonfinite) return DBSCAN_ERR_NONFINITE;
  const unsigned long long n_pairs = host_st.n_edges;
  if (nnz_out) *nnz_out = nnz;
  if (info) {
    info->n_edges = (int64_t)n_pairs;
    info->edge_capacity = (int64_t)L.edge_cap;
    const int64_t nb = L.n_pad / block_points(L.D);
    info->tiles_total = nb * (nb + 1) / 2;
    info->tiles_kept = prune && host_st.n_tiles <= L.tile_cap
                           ? (int64_t)host_st.n_tiles
                           : info->tiles_total;
    info->pass1_pairs = pass1;
    info->merge_mode = DBSCAN_MERGE_EDGES;
  }
  // every row holds its point and one entry per pair it belongs to
  if ((unsigned long long)nnz != (unsigned long long)n + 2ull * n_pairs)
    return DBSCAN_ERR_HIP;
  if ((unsigned long long)nnz > col_cap) return DBSCAN_ERR_CAPACITY;
  if (n_pairs > L.edge_cap) return DBSCAN_ERR_WORKSPACE;

  tm.mark(3);
  DB_TRY(launch_graph_scatter(L, G, n_pairs, d_row_ptr, d_col_idx, stream));
  tm.mark(4);
  DB_TRY(launch_graph_sort(L, G, d_row_ptr, d_col_idx, nnz, stream));
  tm.mark(5);
  DB_TRY(hipMemcpyAsync(&host_st, L.status, sizeof(Status),
                        hipMemcpyDeviceToHost, stream));
  DB_TRY(hipStreamSynchronize(stream));
  if (host_st.graph_bad) return DBSCAN_ERR_HIP;
  if (info && tm.on) {
    info->timed = 1;
    info->ms_layout = tm.ms(0, 1);
    info->ms_count = tm.ms(1, 2);
    info->ms_core = tm.ms(2, 3);
    info->ms_merge = tm.ms(3, 4);
    info->ms_label = tm.ms(4, 5);
    info->ms_total = tm.ms(0, 5);
  }
  return DBSCAN_OK;
}

}  // extern "C"
