// Read-bandwidth probe: the achievable HBM read rate for the access pattern of
// the decode kernels, measured on the machine at hand and reported beside
// the nominal 8 TB/s.
//
// The buffer is read as tiles of tile_bytes (a multiple of 1 KB), in the
// given order (a permutation of tile indices: 4 KB tiles in random order are
// what the decode kernels read, one (block, kv head) tile of K or V at a
// time) or in index order when order is NULL.  Each wave reads 1 KB pieces
// with one 16-byte non-temporal load per lane, four pieces in flight.  Each
// work-group writes the XOR of every 32-bit word it read to sink, so no load
// is dead and the XOR of all sink words is the XOR of the whole buffer (each
// tile is read once when order is a permutation).
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeWaves * 64) void read_probe_kernel(
    const char *__restrict__ buf, long long tile_bytes, long long num_tiles,
    const int32_t *__restrict__ order, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const long long nwaves = (long long)gridDim.x * kProbeWaves;
  const long long per_tile = tile_bytes >> 10;
  const long long total = num_tiles * per_tile;
  u32x4 acc = {0u, 0u, 0u, 0u};
  auto piece = [&](long long pc) -> const u32x4 * {
    const long long t = pc / per_tile;
    const long long j = pc - t * per_tile;
    // Out-of-range entries of order are clamped: the probe never reads
    // outside the buffer.
    const long long tile = order ? min(max((long long)order[t], 0LL), num_tiles - 1) : t;
    return reinterpret_cast<const u32x4 *>(buf + tile * tile_bytes + (j << 10)) + lane;
  };
  // With an order, waves stride over the pieces (neighbouring waves read
  // neighbouring pieces of the scattered tiles, as the decode work-groups
  // do); in index order each wave streams its own contiguous range.
  const long long per_wave = (total + nwaves - 1) / nwaves;
  const long long first = order ? wave : wave * per_wave;
  const long long end = order ? total : min(total, first + per_wave);
  const long long step = order ? nwaves : 1;
  long long pc = first;
  for (; pc + (kProbeUnroll - 1) * step < end; pc += kProbeUnroll * step) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = __builtin_nontemporal_load(piece(pc + u * step));
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; pc < end; pc += step) acc ^= __builtin_nontemporal_load(piece(pc));
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
