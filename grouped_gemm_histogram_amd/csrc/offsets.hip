// offsets.hip -- per-expert histogram (sentinel bin counted out), exclusive scan,
// and the stable counting-sort permutation.
//
// The transformers PR #45621 write-up, section 2: sentinel rows must not be
// computed (no clamping onto the last expert); they are left out of the
// histogram or sorted as the largest key, and offsets[-1] is the number of
// valid rows.  Here the sentinel is bin E of an (E+1)-bin histogram; offsets
// stops before it, and the permutation places bin E last.
//
// Three small launches, no atomics on global memory, deterministic:
//   1. hist:    one workgroup per chunk of rows (256 rows up to 16384 rows, else
//               1024), LDS histogram over E+1 bins.
//   2. scan:    one workgroup; per-bin exclusive scan over chunks (a thread
//               per bin), then the exclusive scan over bins (first wave) -> offsets; a
//               chunk's cursor for a bin is its place in the bin plus the bin's
//               offset.
//   3. scatter: one wave per chunk walks its rows in order, 64 at a time; a
//               row's rank among equal ids in the same 64 comes from ballots
//               over the id bits (lanes with equal ids), so ties keep flat
//               order without any atomic.
// A launch of at most one chunk (decode sizes) runs all three in one workgroup.  The
// layer above decode sizes counts the histogram in its routing launch instead (chunks
// of 16 tokens, stored bin-major), then scans each bin over the chunks and scatters.

#include <mutex>

#include "device_common.h"
#include "launch.h"
#include "route_device.h"

namespace moe {

constexpr int kChunk = 1024;      // rows per chunk of large launches (and the one-workgroup limit)
constexpr int kSmallChunk = 256;  // rows per chunk up to kSmallChunkMaxRows rows
constexpr long long kSmallChunkMaxRows = 16384;

// Rows per chunk for R rows: short chunks shorten each scatter wave's serial walk;
// beyond kSmallChunkMaxRows rows the longer chunks keep the per-bin scan over chunks short.
__host__ __device__ inline int chunk_rows(long long R) {
  return R <= kSmallChunkMaxRows ? kSmallChunk : kChunk;
}
constexpr int kMaxBins = 1025;    // E + 1 with E <= 1024

__device__ __forceinline__ int bin_of(int id, int E) { return (id >= 0 && id < E) ? id : E; }

__global__ __launch_bounds__(256) void hist_kernel(const int* __restrict__ ids, int R, int E, int chunk,
                                                   int* __restrict__ chunk_hist) {
  __shared__ int h[kMaxBins];
  const int nb = E + 1;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * chunk;
  const int r1 = min(R, r0 + chunk);
  for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) atomicAdd(&h[bin_of(ids[r], E)], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += blockDim.x) chunk_hist[(size_t)blockIdx.x * nb + i] = h[i];
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// One workgroup of kScanThreads threads.  chunk_hist [nchunks][E+1] becomes, in place,
// each (chunk, bin)'s first position within its bin (the exclusive scan of the bin's
// counts over chunks); offsets[b] is the bin's base (the exclusive scan of the bin
// totals), which the scatter adds.  A thread scans one bin over the chunks, loading up to
// kScanBatch chunk counts at once (neighbouring threads read neighbouring bins); a small
// workgroup leaves each thread the registers for the whole batch.  The first wave then
// scans the bin totals (lane runs of consecutive bins and a wave scan).
constexpr int kScanThreads = 256;
constexpr int kScanBatch = 64;
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int* __restrict__ chunk_hist, int nchunks,
                                                            int E, int* __restrict__ offsets) {
  __shared__ int tot[kMaxBins];
  const int nb = E + 1;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        v[i] = (c0 + i < nchunks) ? chunk_hist[(size_t)(c0 + i) * nb + b] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (c0 + i < nchunks) chunk_hist[(size_t)(c0 + i) * nb + b] = run;
        run += v[i];
      }
    }
    tot[b] = run;
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  const int per = (nb + kWave - 1) / kWave;
  const int b0 = lane_id() * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < nb) s += tot[b0 + i];
  int base = wave_inclusive_scan(s) - s;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b >= nb) break;
    offsets[b] = base;   // offsets[E] = valid rows
    base += tot[b];
  }
}

// One wave places rows [r0, r1) (at most kSteps * 64 rows) in order; cursor[b] (LDS)
// holds the next position of bin b and is advanced.
template <int kSteps>
__device__ __forceinline__ void scatter_rows(const int* __restrict__ ids, int r0, int r1, int E, int id_bits,
                                             int* cursor, int* __restrict__ sorted_rows,
                                             int* __restrict__ row_pos) {
  const int lane = lane_id();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  // all of the chunk's ids are loaded up front (one round trip instead of one per step)
  int keys[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int r = r0 + i * kWave + lane;
    keys[i] = (r < r1) ? bin_of(ids[r], E) : 0;
  }
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int base = r0 + i * kWave;
    if (base >= r1) break;
    const int r = base + lane;
    const bool active = r < r1;
    const int key = keys[i];
    uint64_t same = __ballot(active);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lt_mask);
    const int cnt = __popcll(same);
    int pos = 0;
    if (active) pos = cursor[key] + rank;
    __builtin_amdgcn_wave_barrier();
    if (active && rank == cnt - 1) cursor[key] = pos + 1;
    __builtin_amdgcn_wave_barrier();
    if (active) {
      sorted_rows[pos] = r;
      row_pos[r] = pos;
    }
  }
}

// One wave per chunk of kSteps * 64 rows.
template <int kSteps>
__global__ __launch_bounds__(64) void scatter_kernel(const int* __restrict__ ids, int R, int E,
                                                     int id_bits,
                                                     const int* __restrict__ chunk_base,
                                                     const int* __restrict__ offsets,
                                                     int* __restrict__ sorted_rows,
                                                     int* __restrict__ row_pos) {
  __shared__ int cursor[kMaxBins];
  const int nb = E + 1;
  // first position of each bin in this chunk: the chunk's place within the bin plus the
  // bin's base
  for (int i = lane_id(); i < nb; i += kWave) cursor[i] = chunk_base[(size_t)blockIdx.x * nb + i] + offsets[i];
  __syncthreads();
  constexpr int chunk = kSteps * kWave;
  const int r0 = blockIdx.x * chunk;
  scatter_rows<kSteps>(ids, r0, min(R, r0 + chunk), E, id_bits, cursor, sorted_rows, row_pos);
}

// R <= kChunk: the histogram by the whole workgroup (LDS atomics), then the bin scan and
// the scatter by its first wave alone (lane runs of consecutive bins and a wave scan), so
// that one workgroup barrier suffices.
__device__ __forceinline__ void offsets_single(const int* __restrict__ ids, int R, int E, int id_bits,
                                               int* __restrict__ offsets, int* __restrict__ sorted_rows,
                                               int* __restrict__ row_pos) {
  __shared__ int cnt[kMaxBins];
  const int nb = E + 1;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) cnt[b] = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += blockDim.x) atomicAdd(&cnt[bin_of(ids[r], E)], 1);
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  // exclusive bases: offsets[b], and (in place) the scatter cursors
  const int per = (nb + kWave - 1) / kWave;
  const int b0 = lane_id() * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < nb) s += cnt[b0 + i];
  int base = wave_inclusive_scan(s) - s;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b >= nb) break;
    const int c = cnt[b];
    offsets[b] = base;   // offsets[E] = valid rows
    cnt[b] = base;
    base += c;
  }
  __builtin_amdgcn_wave_barrier();
  scatter_rows<kChunk / kWave>(ids, 0, R, E, id_bits, cnt, sorted_rows, row_pos);
}

__global__ __launch_bounds__(1024) void offsets_single_kernel(const int* __restrict__ ids, int R, int E,
                                                              int id_bits, int* __restrict__ offsets,
                                                              int* __restrict__ sorted_rows,
                                                              int* __restrict__ row_pos) {
  offsets_single(ids, R, E, id_bits, offsets, sorted_rows, row_pos);
}

// Decode sizes (T*k <= kChunk): routing and offsets in one workgroup, one launch instead
// of two.  The 16 waves route the tokens (a wave per token, as the routing kernel does),
// then the workgroup builds the offsets from the ids it has just written: the barrier
// makes a workgroup's global writes visible to its own waves.
template <int EPL>
__global__ __launch_bounds__(1024) void route_offsets_single_kernel(const float* __restrict__ logits, int T, int E,
                                                                    int k, long long valid_rows, int renorm,
                                                                    int* __restrict__ ids, float* __restrict__ weights,
                                                                    int id_bits, int* __restrict__ offsets,
                                                                    int* __restrict__ sorted_rows,
                                                                    int* __restrict__ row_pos) {
  for (int t = (int)(threadIdx.x >> 6); t < T; t += (int)(blockDim.x >> 6))
    route_token<EPL>(logits, t, E, k, valid_rows, renorm, ids, weights);
  __syncthreads();
  offsets_single(ids, T * k, E, id_bits, offsets, sorted_rows, row_pos);
}

// ---- The layer's path above decode sizes: routing fused with the histogram.
//
// A workgroup of kRouteWaves waves routes kRouteWaves consecutive tokens (a wave each), so
// its chunk is those tokens' kRouteWaves*k flat rows.  It counts the chunk's bins in LDS as
// the ids are written and stores the counts bin-major, hist[b * nchunks + c], so that the
// per-bin scan over chunks reads contiguous words.  Then one workgroup per bin scans its
// counts over the chunks (in place, exclusive) and stores the bin's total, and one wave
// per chunk places the chunk's rows, starting from the exclusive scan of the bin totals
// (which every such wave computes for itself; chunk 0's wave also stores it as offsets).
// Same outputs as routing followed by the three-launch offsets above, one launch fewer.
constexpr int kRouteWaves = 16;

template <int EPL>
__global__ __launch_bounds__(kRouteWaves * kWave) void route_hist_kernel(
    const float* __restrict__ logits, int T, int E, int k, long long valid_rows, int renorm,
    int* __restrict__ ids, float* __restrict__ weights, int nchunks, int* __restrict__ hist) {
  __shared__ int h[kMaxBins];
  const int nb = E + 1;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * kRouteWaves + (int)(threadIdx.x >> 6);
  if (t < T) {
    const int id = route_token<EPL>(logits, t, E, k, valid_rows, renorm, ids, weights);
    if (id >= 0) atomicAdd(&h[id], 1);   // id is in [0, E]: E for a sentinel row
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[(size_t)i * nchunks + blockIdx.x] = h[i];
}

// One workgroup per bin b: hist[b][0, nchunks) becomes its exclusive scan over chunks, and
// tot[b] the bin's total.  kScanPer consecutive chunks per thread per pass.
constexpr int kBinScanThreads = 256;
constexpr int kScanPer = 4;
__global__ __launch_bounds__(kBinScanThreads) void scan_bins_kernel(int* __restrict__ hist, int nchunks,
                                                                   int* __restrict__ tot) {
  __shared__ int wsum[kBinScanThreads / kWave];
  int* row = hist + (size_t)blockIdx.x * nchunks;
  const int lane = lane_id(), wv = (int)(threadIdx.x >> 6);
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += kBinScanThreads * kScanPer) {
    const int cb = c0 + (int)threadIdx.x * kScanPer;
    int v[kScanPer], s = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      v[i] = (cb + i < nchunks) ? row[cb + i] : 0;
      s += v[i];
    }
    const int incl = wave_inclusive_scan(s);
    if (lane == kWave - 1) wsum[wv] = incl;
    __syncthreads();
    int before = carry, pass = 0;
#pragma unroll
    for (int w = 0; w < kBinScanThreads / kWave; ++w) {
      if (w < wv) before += wsum[w];
      pass += wsum[w];
    }
    int run = before + incl - s;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      if (cb + i < nchunks) row[cb + i] = run;
      run += v[i];
    }
    carry += pass;
    __syncthreads();   // wsum is rewritten by the next pass
  }
  if (threadIdx.x == 0) tot[blockIdx.x] = carry;
}

// One wave per chunk of chunk_rows (<= kSteps * 64) flat rows.  hist holds each (bin,
// chunk)'s first place within its bin, tot the bin totals.
template <int kSteps>
__global__ __launch_bounds__(64) void scatter_binmajor_kernel(const int* __restrict__ ids, int R, int E,
                                                              int id_bits, int chunk_rows, int nchunks,
                                                              const int* __restrict__ hist,
                                                              const int* __restrict__ tot,
                                                              int* __restrict__ offsets,
                                                              int* __restrict__ sorted_rows,
                                                              int* __restrict__ row_pos) {
  __shared__ int cursor[kMaxBins];
  const int nb = E + 1;
  const int lane = lane_id();
  const int c = blockIdx.x;
  // bin bases: the exclusive scan of the totals over bins, lane l summing a run of
  // consecutive bins
  const int per = (nb + kWave - 1) / kWave;
  const int b0 = lane * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < nb) s += tot[b0 + i];
  int base = wave_inclusive_scan(s) - s;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b >= nb) break;
    cursor[b] = base + hist[(size_t)b * nchunks + c];
    if (c == 0) offsets[b] = base;   // offsets[E] = valid rows
    base += tot[b];
  }
  __syncthreads();
  const int r0 = c * chunk_rows;
  scatter_rows<kSteps>(ids, r0, min(R, r0 + chunk_rows), E, id_bits, cursor, sorted_rows, row_pos);
}

size_t route_offsets_workspace_bytes(long long T, int E) {
  const long long nchunks = (T + kRouteWaves - 1) / kRouteWaves;
  return (size_t)((nchunks > 0 ? nchunks : 1) + 1) * (size_t)(E + 1) * sizeof(int);
}

namespace {
struct RouteChunks {
  int nchunks, chunk, id_bits;
  int* hist;
  int* tot;
};
RouteChunks route_chunks(int T, int E, int k, void* workspace) {
  RouteChunks c;
  c.nchunks = (T + kRouteWaves - 1) / kRouteWaves;
  c.chunk = kRouteWaves * k;
  c.hist = static_cast<int*>(workspace);
  c.tot = c.hist + (size_t)c.nchunks * (E + 1);
  c.id_bits = 1;
  while ((1 << c.id_bits) <= E) ++c.id_bits;   // bins 0..E need id_bits bits
  return c;
}
bool route_chunks_ok(int T, int E, int k) {
  return T >= 1 && k >= 1 && k * kRouteWaves <= 4 * kWave && E >= 1 && E <= kMaxBins - 1;
}
}  // namespace

hipError_t launch_route_hist(const float* logits, int T, int E, int k, long long valid_rows, int renorm,
                             int* ids, float* weights, void* workspace, hipStream_t stream) {
  if (!route_chunks_ok(T, E, k)) return hipErrorInvalidValue;
  const RouteChunks c = route_chunks(T, E, k, workspace);
#define MOE_ROUTE_HIST_CASE(EPL)                                                                             \
  hipLaunchKernelGGL(route_hist_kernel<EPL>, dim3(c.nchunks), dim3(kRouteWaves * kWave), 0, stream, logits, \
                     T, E, k, valid_rows, renorm, ids, weights, c.nchunks, c.hist);                          \
  break;
  switch ((E + kWave - 1) / kWave) {
    case 1: MOE_ROUTE_HIST_CASE(1)
    case 2: MOE_ROUTE_HIST_CASE(2)
    case 3: case 4: MOE_ROUTE_HIST_CASE(4)
    case 5: case 6: case 7: case 8: MOE_ROUTE_HIST_CASE(8)
    default: MOE_ROUTE_HIST_CASE(16)
  }
#undef MOE_ROUTE_HIST_CASE
  return hipGetLastError();
}

hipError_t launch_offsets_from_hist(const int* ids, int T, int E, int k, int* offsets, int* sorted_rows,
                                    int* row_pos, void* workspace, hipStream_t stream) {
  if (!route_chunks_ok(T, E, k)) return hipErrorInvalidValue;
  const RouteChunks c = route_chunks(T, E, k, workspace);
  hipLaunchKernelGGL(scan_bins_kernel, dim3(E + 1), dim3(kBinScanThreads), 0, stream, c.hist, c.nchunks, c.tot);
#define MOE_SCATTER_BM(STEPS)                                                                               \
  hipLaunchKernelGGL(scatter_binmajor_kernel<STEPS>, dim3(c.nchunks), dim3(kWave), 0, stream, ids, T * k, E, \
                     c.id_bits, c.chunk, c.nchunks, c.hist, c.tot, offsets, sorted_rows, row_pos);
  if (c.chunk <= kWave) {
    MOE_SCATTER_BM(1)
  } else if (c.chunk <= 2 * kWave) {
    MOE_SCATTER_BM(2)
  } else {
    MOE_SCATTER_BM(4)
  }
#undef MOE_SCATTER_BM
  return hipGetLastError();
}

// Scratch of the allocation-free entry point: one array per GPU, in the code object's
// device memory, holding the per-chunk histograms that the workspace argument holds
// otherwise.  Every entry the kernels read is written first by hist_kernel, so nothing
// needs clearing.  Calls that overlap on one GPU share it and race.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

size_t build_offsets_noalloc_capacity() { return kNoAllocScratchBytes; }

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
}  // namespace

hipError_t build_offsets_noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    // the device address of this GPU's copy (the array's name is a host-side stand-in)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

size_t build_offsets_workspace_bytes(long long R, int E) {
  const long long nchunks = (R + chunk_rows(R) - 1) / chunk_rows(R);
  return (size_t)(nchunks > 0 ? nchunks : 1) * (size_t)(E + 1) * sizeof(int);
}

hipError_t launch_build_offsets(const int* ids, int R, int E, int* offsets, int* sorted_rows,
                                int* row_pos, void* workspace, hipStream_t stream) {
  const int chunk = chunk_rows(R);
  const int nchunks = (R + chunk - 1) / chunk;
  int* chunk_hist = static_cast<int*>(workspace);
  int id_bits = 1;
  while ((1 << id_bits) <= E) ++id_bits;   // bins 0..E need id_bits bits
  if (R <= kChunk) {
    hipLaunchKernelGGL(offsets_single_kernel, dim3(1), dim3(1024), 0, stream, ids, R, E, id_bits, offsets,
                       sorted_rows, row_pos);
    return hipGetLastError();
  }
  if (nchunks > 0)
    hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(256), 0, stream, ids, R, E, chunk, chunk_hist);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, chunk_hist, nchunks, E,
                     offsets);
  if (nchunks > 0) {
    if (chunk == kSmallChunk)
      hipLaunchKernelGGL(scatter_kernel<kSmallChunk / kWave>, dim3(nchunks), dim3(64), 0, stream, ids, R, E,
                         id_bits, chunk_hist, offsets, sorted_rows, row_pos);
    else
      hipLaunchKernelGGL(scatter_kernel<kChunk / kWave>, dim3(nchunks), dim3(64), 0, stream, ids, R, E, id_bits,
                         chunk_hist, offsets, sorted_rows, row_pos);
  }
  return hipGetLastError();
}

hipError_t launch_route_offsets_single(const float* logits, int T, int E, int k, long long valid_rows, int renorm,
                                       int* ids, float* weights, int* offsets, int* sorted_rows, int* row_pos,
                                       hipStream_t stream) {
  if ((long long)T * k > kChunk || E < 1 || E > kMaxBins - 1) return hipErrorInvalidValue;
  int id_bits = 1;
  while ((1 << id_bits) <= E) ++id_bits;   // bins 0..E need id_bits bits
#define MOE_ROUTE_OFFS_CASE(EPL)                                                                              \
  hipLaunchKernelGGL(route_offsets_single_kernel<EPL>, dim3(1), dim3(1024), 0, stream, logits, T, E, k,      \
                     valid_rows, renorm, ids, weights, id_bits, offsets, sorted_rows, row_pos);              \
  break;
  switch ((E + kWave - 1) / kWave) {
    case 1: MOE_ROUTE_OFFS_CASE(1)
    case 2: MOE_ROUTE_OFFS_CASE(2)
    case 3: case 4: MOE_ROUTE_OFFS_CASE(4)
    case 5: case 6: case 7: case 8: MOE_ROUTE_OFFS_CASE(8)
    default: MOE_ROUTE_OFFS_CASE(16)
  }
#undef MOE_ROUTE_OFFS_CASE
  return hipGetLastError();
}

}  // namespace moe
