// Contiguous cluster ids from smallest-member labels (an extra entry point).
//
// A point whose label is its own index is the smallest member (the head) of
// its cluster; numbering the heads in ascending index with an exclusive
// scan numbers the clusters 0..K-1 in ascending order of their label, and
// every member takes its head's number.  Cluster sizes are counted with
// atomics aggregated per wave.  (Scan-based offsets as in the Times-C
// summary, Sec. 3.1.)
#include <climits>

#include "dbscan.h"
#include "device.h"
#include "internal.h"

namespace dbk {

struct RelabelStatus {
  unsigned int k;        // clusters
  unsigned int bad;      // a label that is not a valid smallest-member label
  unsigned int pad[14];
};

__global__ void k_zero_relabel_status(RelabelStatus* st) {
  unsigned* w = reinterpret_cast<unsigned*>(st);
  if (threadIdx.x < sizeof(RelabelStatus) / 4) w[threadIdx.x] = 0u;
}

__device__ __forceinline__ bool is_head(const int* labels, int64_t n,
                                        int64_t i) {
  return i < n && labels[i] == (int)i;
}

__global__ __launch_bounds__(256) void k_head_totals(
    const int* __restrict__ labels, int64_t n, unsigned* __restrict__ sums) {
  __shared__ unsigned sh[4];
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
  unsigned c = 0;
  for (int q = 0; q < 4; ++q) c += is_head(labels, n, base + q) ? 1u : 0u;
  unsigned tot;
  block_excl_scan(c, sh, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void k_scan_heads(unsigned* sums,
                                                    int64_t nblk,
                                                    RelabelStatus* st) {
  __shared__ unsigned sh[4];
  unsigned carry = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    const unsigned v = b < nblk ? sums[b] : 0u;
    unsigned tot;
    const unsigned ex = block_excl_scan(v, sh, &tot);
    if (b < nblk) sums[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) st->k = carry;
}

// ids[i] = number of heads before i (meaningful where i is a head)
__global__ __launch_bounds__(256) void k_head_ids(
    const int* __restrict__ labels, int64_t n,
    const unsigned* __restrict__ sums, int* __restrict__ ids) {
  __shared__ unsigned sh[4];
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
  bool h[4];
  unsigned c = 0;
  for (int q = 0; q < 4; ++q) {
    h[q] = is_head(labels, n, base + q);
    c += h[q] ? 1u : 0u;
  }
  unsigned tot;
  unsigned pos = sums[blockIdx.x] + block_excl_scan(c, sh, &tot);
  for (int q = 0; q < 4; ++q)
    if (h[q]) ids[base + q] = (int)pos++;
}

__global__ void k_zero_sizes(int* __restrict__ sizes,
                             const RelabelStatus* __restrict__ st) {
  const int64_t k = st->k;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < k;
       c += (int64_t)gridDim.x * blockDim.x)
    sizes[c] = 0;
}

__global__ void k_relabel_out(const int* __restrict__ labels, int64_t n,
                              const int* __restrict__ ids,
                              int* __restrict__ out, int* __restrict__ sizes,
                              RelabelStatus* __restrict__ st) {
  // n is not padded: keep every lane in the loop so the wave-wide
  // aggregation below always runs with the whole wave
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t span = (n + stride - 1) / stride * stride;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < span;
       i += stride) {
    int id = -1;
    if (i < n) {
      const int l = labels[i];
      if (l >= 0 && l < n && labels[l] == l) id = ids[l];
      else if (l != -1) st->bad = 1u;
      out[i] = id;
    }
    if (sizes) {
      // one atomic per distinct id in the wave
      // leader: the lowest pending lane; at least that lane is cleared
      // on every pass, so the loop ends within 64 passes
      bool pending = id >= 0;
      for (uint64_t pm = ballot(pending); pm != 0; pm = ballot(pending)) {
        const int lead = __builtin_amdgcn_readlane(id, (int)__builtin_ctzll(pm));
        const bool mine = pending && id == lead;
        const uint64_t same = ballot(mine);
        if (mine) {
          if (bits_below(same) == 0) atomicAdd(sizes + lead, (int)__popcll(same));
          pending = false;
        }
      }
    }
  }
}

}  // namespace dbk

using namespace dbk;

static size_t relabel_bytes(int64_t n) {
  const size_t nb = (size_t)(n > 0 ? n : 1);
  return 256 + ((nb / 1024 + 2) * 4 + 255) / 256 * 256 + (nb * 4 + 255) / 256 * 256;
}

extern "C" size_t dbscan_relabel_workspace_bytes(int64_t n) {
  if (n < 0 || n > (int64_t)INT32_MAX) return 0;
  return relabel_bytes(n);
}

extern "C" int dbscan_relabel_device(const int32_t* d_labels, int64_t n,
                                     int32_t* d_ids, int32_t* d_sizes,
                                     int64_t* n_clusters, void* d_workspace,
                                     size_t workspace_bytes,
                                     void* hip_stream) {
  if (n_clusters) *n_clusters = 0;
  if (n < 0 || n > (int64_t)INT32_MAX) return DBSCAN_ERR_INVALID_ARG;
  if (n > 0 && (d_labels == nullptr || d_ids == nullptr)) return DBSCAN_ERR_INVALID_ARG;
  if (n == 0) return DBSCAN_OK;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return DBSCAN_ERR_NO_DEVICE;
  }
  if (d_workspace == nullptr || ((uintptr_t)d_workspace & 255u) ||
      workspace_bytes < relabel_bytes(n))
    return DBSCAN_ERR_WORKSPACE;
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char* b = static_cast<char*>(d_workspace);
  RelabelStatus* st = reinterpret_cast<RelabelStatus*>(b);
  const int64_t nblk = (n + 1023) / 1024;
  unsigned* sums = reinterpret_cast<unsigned*>(b + 256);
  int* ids = reinterpret_cast<int*>(
      b + 256 + ((size_t)(n / 1024 + 2) * 4 + 255) / 256 * 256);
  k_zero_relabel_status<<<1, 64, 0, s>>>(st);
  k_head_totals<<<(unsigned)nblk, 256, 0, s>>>(d_labels, n, sums);
  k_scan_heads<<<1, 256, 0, s>>>(sums, nblk, st);
  k_head_ids<<<(unsigned)nblk, 256, 0, s>>>(d_labels, n, sums, ids);
  if (d_sizes) k_zero_sizes<<<1024, 256, 0, s>>>(d_sizes, st);
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  k_relabel_out<<<(unsigned)g, 256, 0, s>>>(d_labels, n, ids, d_ids, d_sizes,
                                            st);
  hipError_t e = hipGetLastError();
  RelabelStatus host;
  if (e == hipSuccess)
    e = hipMemcpyAsync(&host, st, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e == hipErrorNoBinaryForGpu ||
                                      e == hipErrorInvalidDeviceFunction
                                  ? DBSCAN_ERR_NO_DEVICE
                                  : DBSCAN_ERR_HIP;
  if (host.bad) return DBSCAN_ERR_INVALID_ARG;
  if (n_clusters) *n_clusters = host.k;
  return DBSCAN_OK;
}
