// Paged prefill on the matrix cores (gfx950), fp16 and bf16.
//
// What is computed: the per-token step of P2 §2.1 for every prompt token.
// The last qlen tokens of sequence s are queries (their K/V already written
// to the pool by the cache write); query row j sits at position
// p = ctx - qlen + j and attends causally to tokens 0..p, each token's K/V
// found through block_tables[s] (P3 §2-§3).  A prefix cached earlier (P3 §3,
// shared prefixes save prefill work) is simply not among the queries.
//
// Work decomposition: one work-group of NW waves per (sequence, 16-row query
// tile, query head); waves take 16-token chunks of the context round-robin.
// The products are the grouped-query decode kernel's, with the 16 query rows
// of the tile as the N side:
//
//   S^T[t][r] = sum_d K[t][d] Q[r][d]      v_mfma_f32_16x16x32  (D/32 of them)
//   O[r][d]  += sum_t P[r][t] V[t][d]      v_mfma_f32_16x16x16  (D/16 tiles)
//
// K and V are read with contiguous 1 KB non-temporal wave loads and reach
// the operand layouts through a per-wave LDS tile (K: 16-byte A-layout reads;
// V: ds_read_b64_tr_b16 transposed reads).  Column r carries its own causal
// limit p_r; the mask is applied only on chunks that reach past the tile's
// first position.  The context is streamed in windows of 4096 tokens whose
// block ids are staged in LDS; the online softmax (lazy reference max, as in
// the decode kernel) carries across windows, so no merge pass is needed.
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyMax = 8.f;          // log2 units: weights stay <= 256
constexpr int kRows = 16;                // query rows per work-group
constexpr int kWindow = kMaxPartition;   // tokens whose block ids are staged at once

template <int DT, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_kernel(PrefillArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NW * 64 >= kMaxPartBlocks, "one thread per staged block id");
  constexpr int E = 2;
  constexpr int ROW = D * E;                 // bytes per token row
  constexpr int PITCH = ROW + 32;            // LDS row pitch: 16-byte rows, spread banks
  constexpr int KI = D / 32;                 // first-product steps
  constexpr int NT = D / 16;                 // output tiles of 16 dims
  constexpr int LPT = ROW / 16;              // lanes per row for the wave loads
  constexpr int TPL = 64 / LPT;              // rows per wave load
  constexpr int VL = kChunk / TPL;           // loads per chunk and operand

  __shared__ int s_tbl[kMaxPartBlocks];
  constexpr int kTileBytes = kChunk * PITCH;
  constexpr int kMergeBytes = NW * kRows * (D + 2) * 4;
  constexpr int kLdsBytes =
      (2 * NW * kTileBytes > kMergeBytes) ? 2 * NW * kTileBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  const int H = a.num_heads;
  const int G = H / a.num_kv_heads;
  const int item = blockIdx.x;
  const int h = item % H;
  const int tile = (item / H) % a.num_tiles;
  const int s = item / (H * a.num_tiles);
  const int kvh = h / G;
  const int r0 = tile * kRows;

  const int ctx = a.context_lens[s];
  const int q0 = a.query_start[s], q1 = a.query_start[s + 1];
  const int qlen = q1 - q0;
  const bool bad = ctx < 0 || ctx > a.max_context_len ||
                   ctx > a.max_blocks_per_seq * a.block_size || qlen < 0 || qlen > ctx ||
                   qlen > a.max_query_len || q0 < 0 || q1 > a.num_tokens;
  const float nan = __builtin_nanf("");
  if (bad) {
    // Rows of this tile that lie in the sequence's range and in the output.
    for (int idx = tid; idx < kRows * D; idx += NW * 64) {
      const int r = idx / D, d = idx - r * D;
      const long long row = (long long)q0 + r0 + r;
      if (row >= 0 && row < q1 && row < a.num_tokens)
        store_out<DT>(a.out, ((size_t)row * H + h) * D + d, &nan, 1);
    }
    return;
  }
  if (r0 >= qlen) return;                    // uniform over the work-group
  const int nrows = min(kRows, qlen - r0);
  const int pos0 = ctx - qlen + r0;          // position of the tile's first row
  const int t1 = pos0 + nrows;               // tokens the tile attends to
  const int cpos = pos0 + min(c16, nrows - 1);   // causal limit of column c16

  // Q fragments (B layout: lane l holds row l%16, dims 32i + 8*(l/16) ..+7);
  // columns past the tile's rows are zero and never stored.
  u32x4 qf[KI];
  {
    const bool live = c16 < nrows;
    const char *qrow = reinterpret_cast<const char *>(a.q) +
                       ((size_t)(q0 + r0 + (live ? c16 : 0)) * H + h) * ROW;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(qrow + 64 * i + 16 * g4);
      qf[i] = live ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const size_t head_stride = (size_t)a.block_size * D;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const char *kbase = reinterpret_cast<const char *>(a.k_cache) + kvh * head_stride * E;
  const char *vbase = reinterpret_cast<const char *>(a.v_cache) + kvh * head_stride * E;
  const int v_row = lane / LPT, v_col = lane % LPT;
  const int v_off = v_row * ROW + 16 * v_col;
  constexpr int kChunkBytes = kChunk * ROW;

  unsigned char *ktile = s_buf + wave * 2 * kTileBytes;
  unsigned char *tile_v = ktile + kTileBytes;
  const unsigned char *tr_base = tile_v + (4 * g4 + c16 / 4) * PITCH + 8 * (c16 % 4);
  float m = kNegInf, l = 0.f;
  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool poison = false;
  for (int w0 = 0; w0 < t1; w0 += kWindow) {
    const int wend = min(t1, w0 + kWindow);
    const int nblk = (wend - w0 + a.block_size - 1) >> a.log2_block;
    __syncthreads();                          // the previous window's ids are consumed
    bool bad_id = false;
    if (tid < nblk) {
      const int id = a.block_tables[(size_t)s * a.max_blocks_per_seq + (w0 >> a.log2_block) + tid];
      bad_id = id < 0 || id >= a.num_blocks;
      s_tbl[tid] = id;
    }
    if (__syncthreads_or(bad_id)) {
      poison = true;
      break;
    }
    const int nch = (wend - w0 + kChunk - 1) / kChunk;
    const int nch_w = nch > wave ? (nch - wave + NW - 1) / NW : 0;
    int my_ids = 0;
    if (lane < nch_w) my_ids = s_tbl[((wave + NW * lane) * kChunk) >> a.log2_block];

    auto chunk_offset = [&](int k) -> size_t {
      const int phys = __builtin_amdgcn_readlane(my_ids, k);
      const int tok = (wave + NW * k) * kChunk;
      const int off = tok & (a.block_size - 1);
      return ((size_t)phys * block_stride + (size_t)off * D) * E;
    };
    // Run-out chunks past the wave's last one load through an empty
    // descriptor (zeros, no memory access) and are never consumed.
    auto load = [&](u32x4 *kb, u32x4 *vb, int k, int last) {
      const size_t off = chunk_offset(min(k, last));
      const int range = k <= last ? kChunkBytes : 0;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + off), (short)0, range, kBufferFlags);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + off), (short)0, range, kBufferFlags);
#pragma unroll
      for (int j = 0; j < VL; ++j)
        kb[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, v_off + j * TPL * ROW, 0, kStreamPolicy);
#pragma unroll
      for (int j = 0; j < VL; ++j)
        vb[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, v_off + j * TPL * ROW, 0, kStreamPolicy);
      __builtin_amdgcn_sched_barrier(0);
    };

    auto consume = [&](const u32x4 *kb, const u32x4 *vb, int k) {
      const int tc = w0 + (wave + NW * k) * kChunk;
      const bool diag = tc + kChunk - 1 > pos0;   // some (token, row) pair is masked
#pragma unroll
      for (int j = 0; j < VL; ++j)
        *reinterpret_cast<u32x4 *>(ktile + (v_row + j * TPL) * PITCH + 16 * v_col) = kb[j];
      u32x4 ka[KI];
#pragma unroll
      for (int i = 0; i < KI; ++i)
        ka[i] = *reinterpret_cast<const u32x4 *>(ktile + c16 * PITCH + 64 * i + 16 * g4);
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KI; ++i) sacc = mfma_k32<DT>(ka[i], qf[i], sacc);
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = sacc[r] * a.scale_log2;
      u32x4 vr[VL];
#pragma unroll
      for (int j = 0; j < VL; ++j) vr[j] = vb[j];
      if (diag) {
        // Causal mask by select; V rows past the tile's last position are
        // zeroed (whatever those slots hold must not meet a zero weight).
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tc + 4 * g4 + r > cpos) sc[r] = kNegInf;
#pragma unroll
        for (int j = 0; j < VL; ++j)
          if (tc + v_row + j * TPL >= t1) vr[j] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < VL; ++j)
        *reinterpret_cast<u32x4 *>(tile_v + (v_row + j * TPL) * PITCH + 16 * v_col) = vr[j];

      const float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (__builtin_amdgcn_ballot_w64(mloc > m + kLazyMax)) {
        const float cm = max_xor32(max_xor16(mloc));
        const float mnew = fmaxf(m, cm);
        const float corr = mnew == kNegInf ? 1.f : exp2_fast(m - mnew);
        l *= corr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float cr = __shfl(corr, 4 * g4 + r);
#pragma unroll
          for (int n = 0; n < NT; ++n) o[n][r] *= cr;
        }
        m = mnew;
      }
      const float msafe = m == kNegInf ? 0.f : m;
      float pw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pw[r] = exp2_fast(sc[r] - msafe);
        l += pw[r];
      }
      uint32_t h01, l01, h23, l23;
      split2<DT>(pw[0], pw[1], h01, l01);
      split2<DT>(pw[2], pw[3], h23, l23);
      const u32x2 phi = {h01, h23}, plo = {l01, l23};
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(tr_base + 32 * n));
        const u32x2 vf = __builtin_bit_cast(u32x2, t);
        o[n] = mfma_k16<DT>(phi, vf, o[n]);
        o[n] = mfma_k16<DT>(plo, vf, o[n]);
      }
    };

    constexpr int NBUF = 2;
    u32x4 kb[NBUF][VL], vb[NBUF][VL];
    if (nch_w > 0) {
      const int last = nch_w - 1;
      load(kb[0], vb[0], 0, last);
      for (int k0 = 0; k0 < nch_w; k0 += NBUF) {
#pragma unroll
        for (int i = 0; i < NBUF; ++i) {
          const int k = k0 + i;
          if (k >= nch_w) break;
          load(kb[(i + 1) % NBUF], vb[(i + 1) % NBUF], k + 1, last);
          consume(kb[i], vb[i], k);
        }
      }
    }
  }

  if (poison) {
    for (int idx = tid; idx < nrows * D; idx += NW * 64) {
      const int r = idx / D, d = idx - r * D;
      store_out<DT>(a.out, ((size_t)(q0 + r0 + r) * H + h) * D + d, &nan, 1);
    }
    return;
  }

  l = sum_xor32(sum_xor16(l));
  __syncthreads();
  float *s_m = reinterpret_cast<float *>(s_buf);                // [NW][kRows]
  float *s_l = s_m + NW * kRows;                                 // [NW][kRows]
  float *s_o = s_l + NW * kRows;                                 // [NW][kRows][D]
  if (g4 == 0) {
    s_m[wave * kRows + c16] = m;
    s_l[wave * kRows + c16] = l;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = 4 * g4 + r;
    if (q < nrows) {
#pragma unroll
      for (int n = 0; n < NT; ++n) s_o[(wave * kRows + q) * D + 16 * n + c16] = o[n][r];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nrows * D; idx += NW * 64) {
    const int q = idx / D, d = idx - q * D;
    float Mw = s_m[q];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mw = fmaxf(Mw, s_m[w * kRows + q]);
    const float Ms = Mw == kNegInf ? 0.f : Mw;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2_fast(s_m[w * kRows + q] - Ms);
      L += f * s_l[w * kRows + q];
      O += f * s_o[(w * kRows + q) * D + d];
    }
    const float r = L == 0.f ? 0.f : O / L;
    store_out<DT>(a.out, ((size_t)(q0 + r0 + q) * H + h) * D + d, &r, 1);
  }
}

template <int DT, int D>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream) {
  const long n = (long)a.num_seqs * a.num_heads * a.num_tiles;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<DT, D, kGqaWaves>), dim3((unsigned)n), dim3(kGqaWaves * 64),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace

int prefill_rows_per_tile() { return kRows; }

hipError_t launch_prefill(const PrefillArgs &a, int dt, hipStream_t stream) {
  switch (dt * 1000 + a.head_dim) {
    case kF16 * 1000 + 64: return launch_prefill_t<kF16, 64>(a, stream);
    case kF16 * 1000 + 128: return launch_prefill_t<kF16, 128>(a, stream);
    case kBF16 * 1000 + 64: return launch_prefill_t<kBF16, 64>(a, stream);
    case kBF16 * 1000 + 128: return launch_prefill_t<kBF16, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
