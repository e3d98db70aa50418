// libibp_ceiling: the gather-copy floor against which libibp's decompression
// is measured (include/ibp_ceiling.h).  For every output row it reads the
// stored bytes of the requested slot and writes the whole row: the reads and
// writes of a decompression without its decode, so that the ratio of the two
// times says how much the decode itself costs on top of the memory traffic
// (explainer page "Reducing the GPU Memory Bottleneck with Lossless
// Compression for ML -- Extended", section "Results", which compares the
// decompressor with the ideal rate of the same transfer).
//
// A task is 4 KiB of output.  By default a task is one row, or a 4 KiB chunk
// of a longer row: its id and byte count are wave-uniform loads (both
// indexed by the output row, so neither waits for the other), then each lane
// issues up to four 16-byte loads of the slot and four non-temporal 16-byte
// stores.  Packed tasks (rows shorter than 4 KiB whose 16-byte unit count is
// a power of two) hold 4 KiB / S rows, each lane loading the id and byte
// count of its own row.  Waves loop over tasks when the caller caps the
// grid.  The slot loads take the default cache policy or the non-temporal
// one (the benchmark takes the best of a few grids, both task shapes and
// both load policies, as a floor should).
//
// ibp_ceiling_copy is the plain contiguous copy the benchmark quotes as the
// practical rate of a streaming read/write mix: workgroups stride over 16 KiB
// tiles, each lane loading four 16-byte units (one per 4 KiB quarter of the
// tile, so that each load instruction of the workgroup covers 4 KiB in a
// row) and then storing them, loads and stores non-temporal.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "ibp_ceiling.h"

namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr uint32_t kTaskUnits = 256;  // 16-byte units per task
constexpr int kPerLane = kTaskUnits / kWave;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CopyTensor {
  const u32x4* src;
  const uint32_t* src_bytes;  // per output row
  const int64_t* ids;
  u32x4* dst;
  uint64_t n_rows;
  uint64_t n_out;
  uint64_t task_end;  // tasks of tensors [0, this one]
  uint32_t units;     // 16-byte units per row
  uint32_t cpr;       // 4 KiB chunks per row; 0: packed rows
  uint32_t shift;     // packed: log2(units)
  uint32_t pad;
};

struct CopyBatch {
  uint32_t count;
  uint32_t pad;
  uint64_t tasks;
  CopyTensor t[IBP_CEILING_MAX_TENSORS];
};

// a 16-byte unit of a slot, with the load policy the launch chose
template <bool NT>
__device__ __forceinline__ u32x4 load_unit(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void gather_copy_kernel(CopyBatch b) {
  const uint32_t lane = threadIdx.x % kWave;
  const uint64_t nwaves = (uint64_t)gridDim.x * kWaves;
  for (uint64_t task = (uint64_t)blockIdx.x * kWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
       task < b.tasks; task += nwaves) {
    uint32_t k = 0;
    uint64_t begin = 0;
    while (k + 1 < b.count && task >= b.t[k].task_end) begin = b.t[k++].task_end;
    const CopyTensor& t = b.t[k];
    const uint64_t local = task - begin;
    if (t.cpr == 0) {  // packed rows: every lane its own row
      uint64_t row[kPerLane];
      uint32_t col[kPerLane], lim[kPerLane];
      int64_t id[kPerLane];
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const uint64_t g = local * kTaskUnits + (uint32_t)j * kWave + lane;
        row[j] = g >> t.shift;
        col[j] = (uint32_t)(g & (t.units - 1));
        id[j] = -1;
        lim[j] = 0;
        if (row[j] < t.n_out) {
          id[j] = t.ids ? t.ids[row[j]] : (int64_t)row[j];
          lim[j] = t.src_bytes[row[j]];
        }
      }
      u32x4 v[kPerLane];
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const bool in = id[j] >= 0 && (uint64_t)id[j] < t.n_rows;
        v[j] = u32x4{0u, 0u, 0u, 0u};
        if (in && col[j] < std::min<uint32_t>((lim[j] + 15u) / 16u, t.units))
          v[j] = load_unit<NT>(t.src + (uint64_t)id[j] * t.units + col[j]);
      }
#pragma unroll
      for (int j = 0; j < kPerLane; ++j)
        if (row[j] < t.n_out) __builtin_nontemporal_store(v[j], &t.dst[row[j] * t.units + col[j]]);
      continue;
    }
    const uint64_t r = t.cpr == 1 ? local : local / t.cpr;  // output row (wave-uniform)
    const uint32_t chunk = (uint32_t)(local - r * t.cpr);
    const int64_t id = t.ids ? t.ids[r] : (int64_t)r;
    const uint32_t nb = t.src_bytes[r];
    const uint32_t limit = id >= 0 && (uint64_t)id < t.n_rows
                               ? std::min<uint32_t>((nb + 15u) / 16u, t.units) : 0u;
    const u32x4* s = t.src + (id >= 0 && (uint64_t)id < t.n_rows ? (uint64_t)id : 0ull) * t.units;
    u32x4* d = t.dst + r * t.units;
    u32x4 v[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const uint32_t col = chunk * kTaskUnits + (uint32_t)j * kWave + lane;
      v[j] = u32x4{0u, 0u, 0u, 0u};
      if (col < limit) v[j] = load_unit<NT>(s + col);
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const uint32_t col = chunk * kTaskUnits + (uint32_t)j * kWave + lane;
      if (col < t.units) __builtin_nontemporal_store(v[j], &d[col]);
    }
  }
}

constexpr uint32_t kTileUnits = kThreads * kPerLane;  // 16-byte units of a copy tile

__global__ __launch_bounds__(kThreads) void tile_copy_kernel(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst,
                                                             uint64_t n_units) {
  const uint64_t tiles = (n_units + kTileUnits - 1) / kTileUnits;
  for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint64_t b = t * kTileUnits + threadIdx.x;
    u32x4 v[kPerLane];
    if (t * kTileUnits + kTileUnits <= n_units) {  // a whole tile
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) v[j] = __builtin_nontemporal_load(src + b + j * kThreads);
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) __builtin_nontemporal_store(v[j], dst + b + j * kThreads);
    } else {  // the last, partial tile
#pragma unroll
      for (int j = 0; j < kPerLane; ++j)
        if (b + j * kThreads < n_units) dst[b + j * kThreads] = src[b + j * kThreads];
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" int ibp_ceiling_gather_copy(const ibp_copy_tensor* tensors, uint64_t n_tensors,
                                       uint32_t max_workgroups, uint32_t flags, void* stream) {
  if (n_tensors > IBP_CEILING_MAX_TENSORS || (n_tensors && !tensors)) return -1;
  if (flags & ~(IBP_CEILING_PACK | IBP_CEILING_STREAM_LOADS)) return -1;
  const bool pack = flags & IBP_CEILING_PACK;
  CopyBatch b{};
  uint64_t tasks = 0;
  for (uint64_t i = 0; i < n_tensors; ++i) {
    const ibp_copy_tensor& x = tensors[i];
    if (x.n_out == 0) continue;
    if (x.row_bytes == 0 || x.row_bytes % 16 || x.row_bytes > (1ull << 26)) return -1;
    if (!x.src || !x.src_bytes || !x.dst || x.n_rows == 0) return -1;
    if (!aligned16(x.src) || !aligned16(x.dst) || ((uintptr_t)x.src_bytes & 3) ||
        ((uintptr_t)x.ids & 7))
      return -1;
    if (!x.ids && x.n_out > x.n_rows) return -1;
    if (x.n_out > (1ull << 40)) return -1;
    CopyTensor& t = b.t[b.count];
    t.src = (const u32x4*)x.src;
    t.src_bytes = x.src_bytes;
    t.ids = x.ids;
    t.dst = (u32x4*)x.dst;
    t.n_rows = x.n_rows;
    t.n_out = x.n_out;
    t.units = (uint32_t)(x.row_bytes / 16);
    if (pack && t.units < kTaskUnits && (t.units & (t.units - 1)) == 0) {
      t.cpr = 0;
      t.shift = (uint32_t)__builtin_ctz(t.units);
      tasks += (x.n_out * t.units + kTaskUnits - 1) / kTaskUnits;
    } else {
      t.cpr = (t.units + kTaskUnits - 1) / kTaskUnits;
      tasks += x.n_out * t.cpr;
    }
    t.task_end = tasks;
    ++b.count;
  }
  if (b.count == 0) return 0;
  b.tasks = tasks;
  const uint64_t wgs = (tasks + kWaves - 1) / kWaves;
  const uint32_t grid = (uint32_t)std::min<uint64_t>(
      wgs, max_workgroups ? std::min<uint32_t>(max_workgroups, 1u << 20) : 1u << 20);
  if (flags & IBP_CEILING_STREAM_LOADS)
    hipLaunchKernelGGL(gather_copy_kernel<true>, dim3(grid), dim3(kThreads), 0,
                       (hipStream_t)stream, b);
  else
    hipLaunchKernelGGL(gather_copy_kernel<false>, dim3(grid), dim3(kThreads), 0,
                       (hipStream_t)stream, b);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int ibp_ceiling_copy(const void* src, void* dst, uint64_t n_bytes,
                                uint32_t max_workgroups, void* stream) {
  if (n_bytes == 0) return 0;
  if (!src || !dst || n_bytes % 16 || !aligned16(src) || !aligned16(dst)) return -1;
  const uint64_t n_units = n_bytes / 16;
  const uint64_t tiles = (n_units + kTileUnits - 1) / kTileUnits;
  const uint32_t grid = (uint32_t)std::min<uint64_t>(
      tiles, max_workgroups ? std::min<uint32_t>(max_workgroups, 1u << 20) : 1u << 20);
  hipLaunchKernelGGL(tile_copy_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, n_units);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
