// Paged prefill on the matrix cores (gfx950), fp16 and bf16.
//
// What is computed: the per-token step of P2 §2.1 for every prompt token.
// The last qlen tokens of sequence s are queries (their K/V already written
// to the pool by the cache write); query row j sits at position
// p = ctx - qlen + j and attends causally to tokens 0..p, each token's K/V
// found through block_tables[s] (P3 §2-§3).  A prefix cached earlier (P3 §3,
// shared prefixes save prefill work) is simply not among the queries.
//
// Work decomposition: one work-group of 8 waves per (sequence, 256-row query
// tile, query head); wave w owns rows 32w .. 32w+31 of the tile as two
// 16-row subtiles, so each wave holds the complete softmax state of its rows
// and no cross-wave merge is needed.  Every K and V operand read from LDS
// feeds both subtiles' products, which halves the LDS traffic per flop
// against one subtile per wave, and each K/V chunk brought in serves 256
// query rows, so the context is streamed once per 256 rows.  The work-group
// walks the context in 32-token chunks that all eight waves share:
//
//   * K and V of a chunk go from HBM straight into LDS (buffer loads with
//     the LDS bit: no registers), the waves sharing the 1 KB loads, into one
//     of two stages, so the next chunk streams in while this one is used.
//     Rows are stored with their 16-byte pieces XOR-swizzled by the row index,
//     which makes both operand reads below conflict-free.
//   * S^T = K Q^T: two v_mfma_f32_16x16x32 tiles (tokens 0-15 and 16-31 as M,
//     the wave's 16 rows as N), K read in the A layout.
//   * O += P V on v_mfma_f32_16x16x32 with the 32 tokens as the contraction:
//     a lane's 8 weights are tokens 4g..4g+3 of each token tile, which is the
//     first product's output layout, and the matching V values come from two
//     ds_read_b64_tr_b16 reads (one per token tile).  fp16 feeds P rounded to
//     fp16; bf16 feeds P as a truncated high part plus the remainder (two
//     products), keeping ~16 significant bits per weight.
//   * Online softmax per row with the lazy reference max of the decode
//     kernels; the causal limit of each row is applied on chunks that reach
//     past the wave's first position, and waves skip chunks that lie wholly
//     after their rows.
// Block ids are staged in LDS per 4096-token window.
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyMax = 8.f;          // log2 units: weights stay <= 256
constexpr int kPfWaves = 8;
constexpr int kSub = 2;                  // 16-row subtiles per wave
constexpr int kRows = 16 * kSub * kPfWaves;   // query rows per work-group
constexpr int kCh = 32;                  // tokens per chunk
constexpr int kWindow = kMaxPartition;   // tokens whose block ids are staged at once
// s_waitcnt immediate for vmcnt(0) (expcnt and lgkmcnt left at their
// maxima): the wave's own loads, the LDS-bound ones included, have landed.
constexpr int kWaitVmcnt0 = 0x0f70;

// fp32 weights (a, b) as packed 16-bit values for the A operand.
template <int DT>
__device__ __forceinline__ uint32_t pack_p(float a, float b) {
  if constexpr (DT == kF16) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    // one v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
  } else {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                                 0x07060302u);                         // truncated high halves
  }
}

// Remainders a - hi(a), b - hi(b) of the bf16 high parts, packed likewise.
__device__ __forceinline__ uint32_t pack_lo_bf16(float a, float b) {
  const float ra = a - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xffff0000u);
  const float rb = b - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, b) & 0xffff0000u);
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, rb), __builtin_bit_cast(uint32_t, ra),
                               0x07060302u);
}

// KT: the pools' storage type, DT or kFP8 (E4M3 codes, widened exactly to
// DT as they are staged in LDS, so the tiles and products are DT's).
template <int DT, int KT, int D>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_kernel(PrefillArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(KT == DT || KT == kFP8, "pool type");
  constexpr bool kF8 = KT == kFP8;
  constexpr int EKV = kF8 ? 1 : 2;           // bytes per element of the pools
  static_assert(kPfWaves * 64 >= kMaxPartBlocks, "one thread per staged block id");
  constexpr int E = 2;
  constexpr int ROW = D * E;                 // bytes per token row
  constexpr int PIECES = ROW / 16;           // 16-byte pieces per row
  constexpr int RPL = 1024 / ROW;            // rows per 1 KB wave load
  constexpr int NLD = kCh * ROW / 1024;      // 1 KB loads per operand and chunk
  constexpr int LPW = (NLD + kPfWaves - 1) / kPfWaves;   // of them per wave (at most)
  constexpr int KI = D / 32;                 // first-product steps
  constexpr int NT = D / 16;                 // output tiles of 16 dims
  constexpr int STAGE = kCh * ROW;           // bytes of one operand in one stage

  __shared__ int s_tbl[kMaxPartBlocks];
  __shared__ __attribute__((aligned(1024))) unsigned char s_k0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char s_v0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char s_k1[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char s_v1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  const int H = a.num_heads;
  const int G = H / a.num_kv_heads;
  const int item = blockIdx.x;
  const int h = item % H;
  // Tiles with more rows of context first: they take longest.
  const int tile = a.num_tiles - 1 - (item / H) % a.num_tiles;
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
    for (int idx = tid; idx < kRows * D; idx += kPfWaves * 64) {
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
  // This wave's rows: wr0 .. wr0 + wrows - 1 of the tile (wrows may be 0);
  // subtile u holds rows wr0 + 16u .. + srows[u] - 1.
  const int wr0 = 16 * kSub * wave;
  const int wrows = max(0, min(16 * kSub, nrows - wr0));
  const int wpos0 = pos0 + wr0;              // position of the wave's first row
  const int wlast = pos0 + wr0 + max(wrows, 1) - 1;
  int srows[kSub], cpos[kSub];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    srows[u] = max(0, min(16, nrows - wr0 - 16 * u));
    cpos[u] = pos0 + wr0 + 16 * u + min(c16, max(srows[u], 1) - 1);   // causal limit of column c16
  }

  u32x4 qf[kSub][KI];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    const bool live = c16 < srows[u];
    const char *qrow = reinterpret_cast<const char *>(a.q) +
                       ((size_t)(q0 + r0 + wr0 + 16 * u + (live ? c16 : 0)) * H + h) * ROW;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (live) v = *reinterpret_cast<const u32x4 *>(qrow + 64 * i + 16 * g4);
      qf[u][i] = v;
    }
  }

  const size_t head_stride = (size_t)a.block_size * D;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const char *kbase = reinterpret_cast<const char *>(a.k_cache) + kvh * head_stride * EKV;
  const char *vbase = reinterpret_cast<const char *>(a.v_cache) + kvh * head_stride * EKV;

  // DMA addressing: lane l of a 1 KB load lands at LDS byte 16l of it, i.e.
  // row l / PIECES, physical piece l % PIECES, which holds logical piece
  // (l % PIECES) ^ (row % PIECES).
  const int dma_row = lane / PIECES;                         // row within the load
  const int dma_pp = lane % PIECES;

  // Operand reads.  K (A layout, token tile tt): row 16tt + c16, logical
  // piece 4i + g4.  V (transposed reads, token tile tt, dims 16n..): row
  // 16tt + 4g4 + c16/4, logical byte 32n + 8(c16%4).
  auto k_addr = [&](int tt, int i) -> int {
    const int row = 16 * tt + c16;
    return row * ROW + (((4 * i + g4) ^ (row % PIECES)) << 4);
  };
  auto v_addr = [&](int tt, int n) -> int {
    const int row = 16 * tt + 4 * g4 + c16 / 4;
    const int lb = 32 * n + 8 * (c16 % 4);
    return row * ROW + (((lb >> 4) ^ (row % PIECES)) << 4) + (lb & 15);
  };

  // Row sums of the weights come from the matrix cores too: P times a
  // 32x16 matrix of ones puts row 4g4+r's sum in lsum[u][r] of every lane of
  // group g4, the layout of the output tiles (and of the weights as they
  // enter the products, so numerator and denominator use the same values).
  constexpr uint32_t kOnes = DT == kF16 ? 0x3C003C00u : 0x3F803F80u;
  const u32x4 ones = {kOnes, kOnes, kOnes, kOnes};
  float m[kSub];
  f32x4 o[kSub][NT], lsum[kSub];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    m[u] = kNegInf;
    lsum[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NT; ++n) o[u][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  bool poison = false;
  for (int w0 = 0; w0 < t1; w0 += kWindow) {
    const int wend = min(t1, w0 + kWindow);
    const int nblk = (wend - w0 + a.block_size - 1) >> a.log2_block;
    __syncthreads();                          // the previous window is fully consumed
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
    const int nch = (wend - w0 + kCh - 1) / kCh;

    // Issue this wave's share of chunk k into stage (sk, sv).  Rows at or
    // past wend load through an empty range (zeros; their weights are zero).
    auto dma = [&](int k, unsigned char *sk, unsigned char *sv) {
      const int tc = w0 + k * kCh;
#pragma unroll
      for (int jj = 0; jj < LPW; ++jj) {
        const int j = wave + kPfWaves * jj;              // 1 KB load index within the chunk
        if (j >= NLD) break;                             // uniform
        const int trow0 = tc + j * RPL;                  // first token of the load
        const bool any = trow0 < wend;
        const int phys =
            __builtin_amdgcn_readfirstlane(any ? s_tbl[(trow0 - w0) >> a.log2_block] : 0);
        const int off = trow0 & (a.block_size - 1);
        const size_t base = ((size_t)phys * block_stride + (size_t)off * D) * E;
        const int range = any ? RPL * ROW : 0;
        const int row = dma_row;
        const int voff = (trow0 + row < wend)
                             ? row * ROW + ((dma_pp ^ ((j * RPL + row) % PIECES)) << 4)
                             : 0x7ffffff0;
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + base), (short)0, range, kBufferFlags);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + base), (short)0, range, kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void *)(sk + j * 1024), 16, voff, 0, 0,
            kStreamPolicy);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (__attribute__((address_space(3))) void *)(sv + j * 1024), 16, voff, 0, 0,
            kStreamPolicy);
      }
    };

    auto compute = [&](int k, const unsigned char *sk, const unsigned char *sv) {
      const int tc = w0 + k * kCh;
      if (wrows == 0 || tc > wlast) return;      // uniform: the chunk is after this wave's rows
      const bool diag = tc + kCh - 1 > wpos0;
      // Every operand read of the chunk is issued first (K in the A layout,
      // V transposed; V does not depend on the weights), so their LDS
      // latency overlaps; then the four independent score accumulations
      // (two token tiles x two subtiles) interleave on the matrix cores.
      u32x4 ka[2][KI];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < KI; ++i) ka[tt][i] = *reinterpret_cast<const u32x4 *>(sk + k_addr(tt, i));
      u32x4 vf[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(sv + v_addr(0, n)));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(sv + v_addr(1, n)));
        const u32x2 w0v = __builtin_bit_cast(u32x2, v0), w1v = __builtin_bit_cast(u32x2, v1);
        vf[n] = u32x4{w0v.x, w0v.y, w1v.x, w1v.y};
      }
      f32x4 acc[2][kSub];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int u = 0; u < kSub; ++u) acc[tt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KI; ++i)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int u = 0; u < kSub; ++u) acc[tt][u] = mfma_k32<DT>(ka[tt][i], qf[u][i], acc[tt][u]);
      float sc[kSub][2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int u = 0; u < kSub; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[u][tt][r] = acc[tt][u][r] * a.scale_log2;
      if (diag) {
#pragma unroll
        for (int u = 0; u < kSub; ++u)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (tc + 16 * tt + 4 * g4 + r > cpos[u]) sc[u][tt][r] = kNegInf;
      }
      u32x4 pa_hi[kSub], pa_lo[kSub];
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        float mloc = sc[u][0][0];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sc[u][tt][r]);
        if (__builtin_amdgcn_ballot_w64(mloc > m[u] + kLazyMax)) {
          const float cm = max_xor32(max_xor16(mloc));
          const float mnew = fmaxf(m[u], cm);
          const float corr = mnew == kNegInf ? 1.f : exp2_fast(m[u] - mnew);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float cr = __shfl(corr, 4 * g4 + r);
            lsum[u][r] *= cr;
#pragma unroll
            for (int n = 0; n < NT; ++n) o[u][n][r] *= cr;
          }
          m[u] = mnew;
        }
        const float msafe = m[u] == kNegInf ? 0.f : m[u];
        float p[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[tt][r] = exp2_fast(sc[u][tt][r] - msafe);
        pa_hi[u] = u32x4{pack_p<DT>(p[0][0], p[0][1]), pack_p<DT>(p[0][2], p[0][3]),
                         pack_p<DT>(p[1][0], p[1][1]), pack_p<DT>(p[1][2], p[1][3])};
        pa_lo[u] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (DT == kBF16)
          pa_lo[u] = u32x4{pack_lo_bf16(p[0][0], p[0][1]), pack_lo_bf16(p[0][2], p[0][3]),
                           pack_lo_bf16(p[1][0], p[1][1]), pack_lo_bf16(p[1][2], p[1][3])};
        lsum[u] = mfma_k32<DT>(pa_hi[u], ones, lsum[u]);
        if constexpr (DT == kBF16) lsum[u] = mfma_k32<DT>(pa_lo[u], ones, lsum[u]);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          o[u][n] = mfma_k32<DT>(pa_hi[u], vf[n], o[u][n]);
          if constexpr (DT == kBF16) o[u][n] = mfma_k32<DT>(pa_lo[u], vf[n], o[u][n]);
        }
      }
    };

    if constexpr (kF8) {
      // E4M3 pools: thread t < 2D loads 16 codes of one row of the chunk
      // (row t / (D/16), bytes 16 (t % (D/16)) ..) into registers one chunk
      // ahead, and widens them into the swizzled tile once the stage is free.
      constexpr int TPR = D / 16;                      // threads per pool row
      const bool stager = tid < kCh * TPR;
      const int srow = tid / TPR, spart = tid % TPR;
      u32x4 ck = {0u, 0u, 0u, 0u}, cv = {0u, 0u, 0u, 0u};
      auto fload = [&](int k) __attribute__((always_inline)) {
        ck = u32x4{0u, 0u, 0u, 0u};
        cv = u32x4{0u, 0u, 0u, 0u};
        const int t = w0 + k * kCh + srow;
        if (stager && t < wend) {                      // rows past the window stay zero
          const int phys = s_tbl[(t - w0) >> a.log2_block];
          const size_t off = ((size_t)phys * block_stride + (size_t)(t & (a.block_size - 1)) * D) +
                             16 * spart;
          ck = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kbase + off));
          cv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vbase + off));
        }
      };
      auto put = [&](unsigned char *st, const u32x4 &w) __attribute__((always_inline)) {
        const u32x4 lo = {fp8_pair<DT, false>(w.x), fp8_pair<DT, true>(w.x),
                          fp8_pair<DT, false>(w.y), fp8_pair<DT, true>(w.y)};
        const u32x4 hi = {fp8_pair<DT, false>(w.z), fp8_pair<DT, true>(w.z),
                          fp8_pair<DT, false>(w.w), fp8_pair<DT, true>(w.w)};
        const int sw = srow % PIECES;
        *reinterpret_cast<u32x4 *>(st + srow * ROW + (((2 * spart) ^ sw) << 4)) = lo;
        *reinterpret_cast<u32x4 *>(st + srow * ROW + (((2 * spart + 1) ^ sw) << 4)) = hi;
      };
      auto fcommit = [&](unsigned char *sk, unsigned char *sv) __attribute__((always_inline)) {
        if (stager) {
          put(sk, ck);
          put(sv, cv);
        }
      };
      fload(0);
      fcommit(s_k0, s_v0);
      for (int k = 0; k < nch; k += 2) {
        __syncthreads();                               // chunk k in stage 0; stage 1 is free
        if (k + 1 < nch) fload(k + 1);
        compute(k, s_k0, s_v0);
        if (k + 1 >= nch) break;
        fcommit(s_k1, s_v1);
        __syncthreads();                               // chunk k+1 in stage 1; stage 0 is free
        if (k + 2 < nch) fload(k + 2);
        compute(k + 1, s_k1, s_v1);
        if (k + 2 < nch) fcommit(s_k0, s_v0);
      }
      continue;
    }
    dma(0, s_k0, s_v0);
    for (int k = 0; k < nch; k += 2) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);       // this wave's part of chunk k has landed
      __syncthreads();                                // chunk k is in stage 0 for every wave
      if (k + 1 < nch) dma(k + 1, s_k1, s_v1);
      compute(k, s_k0, s_v0);
      if (k + 1 >= nch) break;
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();                                // chunk k+1 in stage 1; stage 0 is free
      if (k + 2 < nch) dma(k + 2, s_k0, s_v0);
      compute(k + 1, s_k1, s_v1);
    }
  }

  if (poison) {
    for (int idx = tid; idx < nrows * D; idx += kPfWaves * 64) {
      const int r = idx / D, d = idx - r * D;
      store_out<DT>(a.out, ((size_t)(q0 + r0 + r) * H + h) * D + d, &nan, 1);
    }
    return;
  }
  if (wrows == 0) return;

  // out = O / l for each row this lane holds (rows 4*g4 + r of subtile u,
  // dims 16n + c16), as O times one reciprocal per row (v_rcp_f32, within
  // an ulp): a row with context has l >= 1, since its reference max is one
  // of its own scores, whose weight is at least 1; an empty row has l = 0
  // and gives 0.  (IEEE division of every element cost the work-group's
  // tail ~950 VALU instructions per wave.)
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = 4 * g4 + r;
      const float lr = lsum[u][r];
      float inv = lr == 0.f ? 0.f : __builtin_amdgcn_rcpf(lr);
      if constexpr (kF8) inv *= a.v_scale;     // the tiles held V codes
      if (q < srows[u]) {
        const size_t rowbase = ((size_t)(q0 + r0 + wr0 + 16 * u + q) * H + h) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const float v = o[u][n][r] * inv;
          store_out<DT>(a.out, rowbase + 16 * n + c16, &v, 1);
        }
      }
    }
  }
}

template <int DT, int KT, int D>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream) {
  const long n = (long)a.num_seqs * a.num_heads * a.num_tiles;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<DT, KT, D>), dim3((unsigned)n), dim3(kPfWaves * 64), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

static_assert(kRows == kPrefillRows, "the host sizes the grid with kPrefillRows");

hipError_t launch_prefill(const PrefillArgs &a, int dt, int kv_dt, hipStream_t stream) {
  const bool f8 = kv_dt == kFP8;
  if (!f8 && kv_dt != dt) return hipErrorInvalidValue;
  switch (dt * 1000 + a.head_dim + (f8 ? 1 : 0)) {
    case kF16 * 1000 + 64: return launch_prefill_t<kF16, kF16, 64>(a, stream);
    case kF16 * 1000 + 128: return launch_prefill_t<kF16, kF16, 128>(a, stream);
    case kBF16 * 1000 + 64: return launch_prefill_t<kBF16, kBF16, 64>(a, stream);
    case kBF16 * 1000 + 128: return launch_prefill_t<kBF16, kBF16, 128>(a, stream);
    case kF16 * 1000 + 65: return launch_prefill_t<kF16, kFP8, 64>(a, stream);
    case kF16 * 1000 + 129: return launch_prefill_t<kF16, kFP8, 128>(a, stream);
    case kBF16 * 1000 + 65: return launch_prefill_t<kBF16, kFP8, 64>(a, stream);
    case kBF16 * 1000 + 129: return launch_prefill_t<kBF16, kFP8, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
