// Read-bandwidth probe: the achievable HBM read rate for the access pattern of
// the decode kernels, measured on the machine at hand and reported beside
// the nominal 8 TB/s.
//
// The buffer is read as tiles of tile_bytes (a multiple of 1 KB), in the
// given order (a permutation of tile indices: 4 KB tiles in random order are
// what the decode kernels read, one (block, kv head) tile of K or V at a
// time) or in index order when order is NULL.  Each wave reads a contiguous
// run of the ordered pieces (1 KB each: one 16-byte non-temporal load per
// lane), sixteen pieces in flight (the waves past the end of a small buffer
// read nothing).  Measured on MI355X against interleaved
// assignments, fewer pieces in flight and other grid sizes, this shape read
// fastest in both orders (interleaving with four in flight, its earlier
// form, read random 4 KB tiles 7% slower).  Each work-group writes the XOR
// of every 32-bit word it read to sink, so no load is dead and the XOR of
// all sink words is the XOR of the whole buffer (each tile is read once
// when order is a permutation).
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeUnroll = 16;

__global__ __launch_bounds__(kProbeWaves * 64) void read_probe_kernel(
    const char *__restrict__ buf, long long tile_bytes, long long num_tiles,
    const int32_t *__restrict__ order, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long long wave =
      (long long)blockIdx.x * kProbeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long nwaves = (long long)gridDim.x * kProbeWaves;
  const long long per_tile = tile_bytes >> 10;
  const long long total = num_tiles * per_tile;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // Each wave takes its own contiguous range of the ordered pieces, a whole
  // number of batches of kProbeUnroll, so that a small buffer keeps sixteen
  // loads in flight per wave on fewer waves rather than one load each on
  // all of them; the (tile, piece) position advances by one per load (a
  // division per load made the probe ALU-bound).
  const long long per_wave =
      ((total + nwaves - 1) / nwaves + kProbeUnroll - 1) / kProbeUnroll * kProbeUnroll;
  const long long first = wave * per_wave;
  const long long end = min(total, first + per_wave);
  long long t = first / per_tile;
  long long j = first - t * per_tile;
  // Out-of-range entries of order are clamped: the probe never reads
  // outside the buffer.
  auto tile_of = [&](long long id) -> long long { return min(max(id, 0LL), num_tiles - 1); };
  auto advance = [&]() {
    if (++j == per_tile) {
      j = 0;
      ++t;
    }
  };
  long long pc = first;
  for (; pc + kProbeUnroll - 1 < end; pc += kProbeUnroll) {
    // The order entries of this batch (it spans at most kProbeUnroll tiles),
    // one per lane, fetched with one load.
    const long long tb = t;
    const int ord = order ? order[min(tb + lane, num_tiles - 1)] : 0;
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const long long tile =
          order ? tile_of(__builtin_amdgcn_readlane(ord, (int)(t - tb))) : t;
      v[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(buf + tile * tile_bytes + (j << 10)) + lane);
      advance();
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; pc < end; ++pc) {
    const long long tile = order ? tile_of(order[t]) : t;
    acc ^= __builtin_nontemporal_load(
        reinterpret_cast<const u32x4 *>(buf + tile * tile_bytes + (j << 10)) + lane);
    advance();
  }
  // XOR of every word this work-group read: over the lanes, then the waves.
  uint32_t w = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) w ^= (uint32_t)__shfl_xor((int)w, m);
  __shared__ uint32_t s_fold[kProbeWaves];
  if (lane == 0) s_fold[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t all = 0;
#pragma unroll
    for (int i = 0; i < kProbeWaves; ++i) all ^= s_fold[i];
    sink[blockIdx.x] = all;
  }
}

}  // namespace

hipError_t launch_read_probe(const void *buf, long long tile_bytes, long long num_tiles,
                             const int32_t *order, uint32_t *sink, hipStream_t stream) {
  if (num_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel, dim3(PA_READ_PROBE_SINK_WORDS), dim3(kProbeWaves * 64),
                     0, stream, static_cast<const char *>(buf), tile_bytes, num_tiles, order,
                     sink);
  return hipGetLastError();
}

}  // namespace pa
