// One decode step through the C ABI alone (include/pa.h): no PyTorch, only
// the HIP runtime for device memory.  For every sequence the newest token's
// slot is resolved (pa_compute_slots), its K/V rows are written into the
// pools (pa_cache_write) and paged attention runs over the whole context
// (pa_decode), on one stream.
//
//   decode_step DIR
//
// DIR/meta.txt holds "S H Hkv D B NB MB dtype max_context_len scale
// partition_size" (dtype as pa_dtype_t); the arrays are raw little-endian
// files: q.bin [S][H][D], kc.bin and vc.bin [NB][Hkv][B][D], tables.bin int32
// [S][MB], ctx.bin int32 [S], new_k.bin and new_v.bin [S][Hkv][D].  Writes
// slots.bin (int64 [S]), out.bin [S][H][D], kc_out.bin and vc_out.bin.
// Exits 1 with pa_last_error() on any failure.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "pa.h"

namespace {

std::vector<char> read_file(const std::string &path) {
  FILE *f = std::fopen(path.c_str(), "rb");
  if (!f) {
    std::fprintf(stderr, "cannot open %s\n", path.c_str());
    std::exit(1);
  }
  std::fseek(f, 0, SEEK_END);
  const long n = std::ftell(f);
  std::fseek(f, 0, SEEK_SET);
  std::vector<char> buf(n);
  if (n && std::fread(buf.data(), 1, n, f) != (size_t)n) {
    std::fprintf(stderr, "short read %s\n", path.c_str());
    std::exit(1);
  }
  std::fclose(f);
  return buf;
}

void write_file(const std::string &path, const void *data, size_t n) {
  FILE *f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(data, 1, n, f) != n) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    std::exit(1);
  }
  std::fclose(f);
}

void hip_ok(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

void pa_ok(pa_status_t st, const char *what) {
  if (st != PA_OK) {
    std::fprintf(stderr, "%s: status %d: %s\n", what, (int)st, pa_last_error());
    std::exit(1);
  }
}

// Device copy of a host buffer (the caller frees it).
void *to_device(const std::vector<char> &h) {
  void *d = nullptr;
  hip_ok(hipMalloc(&d, h.size() ? h.size() : 1), "hipMalloc");
  if (!h.empty()) hip_ok(hipMemcpy(d, h.data(), h.size(), hipMemcpyHostToDevice), "hipMemcpy");
  return d;
}

std::vector<char> to_host(const void *d, size_t n) {
  std::vector<char> h(n);
  if (n) hip_ok(hipMemcpy(h.data(), d, n, hipMemcpyDeviceToHost), "hipMemcpy");
  return h;
}

}  // namespace

int main(int argc, char **argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  int S, H, Hkv, D, B, NB, MB, dt, max_ctx, P;
  float scale;
  {
    FILE *f = std::fopen((dir + "/meta.txt").c_str(), "r");
    if (!f || std::fscanf(f, "%d %d %d %d %d %d %d %d %d %f %d", &S, &H, &Hkv, &D, &B, &NB, &MB,
                          &dt, &max_ctx, &scale, &P) != 11) {
      std::fprintf(stderr, "bad meta.txt\n");
      return 1;
    }
    std::fclose(f);
  }
  const pa_dtype_t dtype = (pa_dtype_t)dt;
  const size_t e = dtype == PA_F32 ? 4 : 2;

  const std::vector<char> kc = read_file(dir + "/kc.bin"), vc = read_file(dir + "/vc.bin");
  void *d_q = to_device(read_file(dir + "/q.bin"));
  void *d_kc = to_device(kc), *d_vc = to_device(vc);
  void *d_tables = to_device(read_file(dir + "/tables.bin"));
  void *d_ctx = to_device(read_file(dir + "/ctx.bin"));
  void *d_nk = to_device(read_file(dir + "/new_k.bin"));
  void *d_nv = to_device(read_file(dir + "/new_v.bin"));
  void *d_slots = nullptr, *d_out = nullptr, *d_ws = nullptr;
  hip_ok(hipMalloc(&d_slots, sizeof(int64_t) * S), "hipMalloc");
  const size_t out_bytes = (size_t)S * H * D * e;
  hip_ok(hipMalloc(&d_out, out_bytes), "hipMalloc");
  const size_t ws_bytes = pa_decode_workspace_size(S, H, Hkv, D, B, max_ctx, P, dtype);
  if (ws_bytes == (size_t)-1) pa_ok(PA_ERR_INVALID_ARGUMENT, "pa_decode_workspace_size");
  if (ws_bytes) hip_ok(hipMalloc(&d_ws, ws_bytes), "hipMalloc");

  hipStream_t stream;
  hip_ok(hipStreamCreate(&stream), "hipStreamCreate");
  pa_ok(pa_compute_slots((int64_t *)d_slots, (const int32_t *)d_tables, MB, (const int32_t *)d_ctx,
                         nullptr, nullptr, S, S, B, NB, stream),
        "pa_compute_slots");
  pa_ok(pa_cache_write(d_nk, d_nv, d_kc, d_vc, (const int64_t *)d_slots, S, Hkv, D, B, NB, dtype,
                       stream),
        "pa_cache_write");
  pa_ok(pa_decode(d_out, d_q, d_kc, d_vc, (const int32_t *)d_tables, (const int32_t *)d_ctx, S, H,
                  Hkv, D, B, NB, MB, max_ctx, scale, P, d_ws, ws_bytes, dtype, stream),
        "pa_decode");
  hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize");

  const std::vector<char> slots = to_host(d_slots, sizeof(int64_t) * S);
  const std::vector<char> out = to_host(d_out, out_bytes);
  const std::vector<char> kc_out = to_host(d_kc, kc.size()), vc_out = to_host(d_vc, vc.size());
  write_file(dir + "/slots.bin", slots.data(), slots.size());
  write_file(dir + "/out.bin", out.data(), out.size());
  write_file(dir + "/kc_out.bin", kc_out.data(), kc_out.size());
  write_file(dir + "/vc_out.bin", vc_out.data(), vc_out.size());
  for (void *p : {d_q, d_kc, d_vc, d_tables, d_ctx, d_nk, d_nv, d_slots, d_out, d_ws})
    if (p) hip_ok(hipFree(p), "hipFree");
  hip_ok(hipStreamDestroy(stream), "hipStreamDestroy");
  std::printf("decode_step ok (%s)\n", pa_version());
  return 0;
}
