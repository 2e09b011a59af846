// PagedAttention decode for grouped-query attention on the matrix cores
// (gfx950): fp16 and bf16 queries over pools of the same type or of E4M3
// codes with per-pool scales.
//
// Same result as the vector kernel (P1 §1 first formula over the context
// gathered through the block table, P3 §2-§3), but the G query heads that
// share a kv head are processed together: each K/V chunk is read once and
// used by all G rows, which turns the per-chunk work into two small dense
// products.
//
// Work decomposition: one work-group of NW waves per (sequence, kv head,
// tile of up to 16 query heads, partition); waves take 16-token chunks
// round-robin.  More than 16 query heads per kv head (down to one kv head
// for all of them) take several tiles, which the work-group order places
// on one XCD, so after the first the kv head's K/V come from its L2.  Per
// chunk:
//
//   S^T[t][q] = sum_d K[t][d] Q[q][d]      v_mfma_f32_16x16x32  (D/32 of them)
//   O[q][d]  += sum_t P[q][t] V[t][d]      v_mfma_f32_16x16x16  (D/16 tiles)
//
// with the 16 tokens of the chunk as the M (then K) dimension and up to 16
// query heads as N (rows q >= G are zero padding).  The output layout of the
// first product (lane l holds tokens 4*(l/16)..+3 of query l%16) is exactly
// the A-operand layout of the second, so the probabilities never leave their
// registers.  P is fed as two 16-bit halves (hi = truncated P, lo = the
// remainder) so the product keeps ~16 significant bits of every weight; the
// accumulation is fp32.
//
// Operand sourcing: Q is loaded once into the B layout of the first
// product.  K and V of a chunk are loaded with contiguous 1 KB wave loads
// (the A-operand pattern straight from memory, 16 rows x 64 B per load,
// streams more slowly) and written to per-wave LDS tiles whose row pitch is
// padded to D*2+32 bytes.  K is read back in the A layout (lane l: token
// l%16, 16 bytes of dims per step); V is needed with tokens along each lane
// (B layout of the second product), the transpose of how it sits in the
// pool, and is read back with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16), one per 16-dim output tile.
//
// Online softmax per query column, with a lazy reference: the running max m
// is only raised when a chunk's max exceeds it by more than 8 (log2 units),
// so the rescale of O (which needs the factors moved from query-column lanes
// to output-row lanes) is rare; unnormalised weights stay below 2^8, far
// from fp32 or bf16 limits, and the final o/l is independent of the
// reference chosen.
//
// E4M3 pools: each lane widens the 16 codes it loaded to 16 values of the
// query's type (exact) as it writes them to the LDS tile, so the tiles, the
// products and the softmax are those of the 16-bit path.  The K pool scale is
// folded into the score scale and the V pool scale is applied to the
// accumulated output.
//
// Appending decode: the newest token's K/V rows come from the input (staged in
// LDS by the prologue, as pool rows: quantised first for E4M3 pools, and
// written over the pool's row in the chunk's LDS tiles, so whatever the slot
// held before never counts), and the work-group of the partition holding the
// token stores them into its slot.
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyMax = 8.f;          // log2 units: weights stay <= 256
constexpr int kGMax = kGqaTile;          // query heads per tile

// Stage one 16-byte pool load (lane column col of a token row) in an LDS
// tile row of 16-bit values: as it is, or widened from 16 E4M3 codes to 32
// bytes of the query's type.
template <int DT, int KT>
__device__ __forceinline__ void stage16(unsigned char *row, int col, const u32x4 &w) {
  if constexpr (KT == kFP8) {
    const u32x4 lo = {fp8_pair<DT, false>(w.x), fp8_pair<DT, true>(w.x),
                      fp8_pair<DT, false>(w.y), fp8_pair<DT, true>(w.y)};
    const u32x4 hi = {fp8_pair<DT, false>(w.z), fp8_pair<DT, true>(w.z),
                      fp8_pair<DT, false>(w.w), fp8_pair<DT, true>(w.w)};
    *reinterpret_cast<u32x4 *>(row + 32 * col) = lo;
    *reinterpret_cast<u32x4 *>(row + 32 * col + 16) = hi;
  } else {
    *reinterpret_cast<u32x4 *>(row + 16 * col) = w;
  }
}

// Three waves per SIMD fit without spilling at head_dim 128 (153 VGPRs).
template <int DT, int KT, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3)))
void decode_gqa_kernel(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NW * 64 >= kMaxPartBlocks, "one thread per staged block id");
  static_assert(KT == DT || KT == kFP8, "pool type");
  constexpr bool kF8 = KT == kFP8;
  constexpr int E = 2;                       // bytes per element of q, out and the tiles
  constexpr int EKV = kF8 ? 1 : 2;           // bytes per element of the pools
  constexpr int ROW = D * E;                 // bytes per token row of q and of a tile
  constexpr int ROWKV = D * EKV;             // bytes per token row in the pools
  constexpr int PITCH = ROW + 32;            // LDS row pitch: 16-byte rows, spread banks
  constexpr int KI = D / 32;                 // first-product steps
  constexpr int NT = D / 16;                 // output tiles of 16 dims
  constexpr int LPT = ROWKV / 16;            // lanes per pool row for the K/V loads
  constexpr int TPL = 64 / LPT;              // rows per K/V wave load
  constexpr int VL = kChunk / TPL;           // K/V loads per chunk

  __shared__ int s_tbl[kMaxPartBlocks];
  __shared__ u32x4 s_new[2][LPT];           // the newest token's K and V pool rows (appending)
  // K and V tiles (one pair per wave) during the loop; reused for the
  // cross-wave merge afterwards.
  constexpr int kTileBytes = kChunk * PITCH;
  constexpr int kMergeBytes = NW * kGMax * (D + 2) * 4;
  constexpr int kLdsBytes =
      (2 * NW * kTileBytes > kMergeBytes) ? 2 * NW * kTileBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;                  // lane group (0..3)
  const int c16 = lane & 15;                 // lane within group

  const int Hkv = a.num_kv_heads, S = a.num_seqs, H = a.num_heads;
  const int G = H / Hkv;
  const int NQT = (G + kGMax - 1) / kGMax;  // query tiles per kv head
  const int item = group_on_xcd(blockIdx.x, gridDim.x, NQT);
  const int qt = item % NQT;
  const int kvh = (item / NQT) % Hkv;
  const int s = (item / (NQT * Hkv)) % S;
  const int p = item / (NQT * Hkv * S);
  const int Gt = min(kGMax, G - kGMax * qt);  // query heads on this tile
  const int hb = kvh * G + kGMax * qt;        // its first query head
  const int P = a.partition_size;
  const int t0 = p * P;
  const int b0 = t0 >> a.log2_block;

  // Prologue loads, issued together: context length, table window, and the
  // Q fragments (B layout: lane l holds query l%16, dims 32i + 8*(l/16) ..+7).
  const int ctx = a.context_lens[s];
  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks_per_seq + b0;
  const int window = min(P >> a.log2_block, a.max_blocks_per_seq - b0);
  const int id = tid < window ? trow[tid] : -1;
  // K and V: contiguous wave loads (every load instruction reads whole 1 KB
  // of the chunk), lane l reads row (l/LPT) + TPL*j, bytes 16*(l%LPT).
  const int v_row = lane / LPT, v_col = lane % LPT;
  const bool append = a.new_k != nullptr;                  // uniform (kernel argument)
  // Lanes 0..LPT-1 (wave 0, row 0) of the first tile write the newest
  // token's pool rows.
  const bool new_lane = append && tid < LPT;
  u32x4 nk = {0u, 0u, 0u, 0u}, nv = {0u, 0u, 0u, 0u};
  if constexpr (kF8) {
    // Quantised as the separate cache write does, four elements per lane
    // over wave 0 (K on lanes 0..D/4-1, V on the next D/4).
    constexpr int NE = D / 4;
    if (append && tid < 2 * NE) {
      const bool isv = tid >= NE;
      const int w = isv ? tid - NE : tid;
      const u32x2 raw = *reinterpret_cast<const u32x2 *>(
          static_cast<const char *>(isv ? a.new_v : a.new_k) +
          ((size_t)s * Hkv + kvh) * ROW + 8 * w);
      const float sc = isv ? a.v_scale : a.k_scale;
      const uint32_t word = e4m3_code(lo_f32<DT>(raw.x) / sc) |
                            (e4m3_code(hi_f32<DT>(raw.x) / sc) << 8) |
                            (e4m3_code(lo_f32<DT>(raw.y) / sc) << 16) |
                            (e4m3_code(hi_f32<DT>(raw.y) / sc) << 24);
      reinterpret_cast<uint32_t *>(&s_new[isv ? 1 : 0][0])[w] = word;
    }
  } else if (new_lane) {
    const size_t new_off = ((size_t)s * Hkv + kvh) * ROW + 16 * v_col;
    nk = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(a.new_k) + new_off);
    nv = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(a.new_v) + new_off);
    s_new[0][v_col] = nk;
    s_new[1][v_col] = nv;
  }
  u32x4 qf[KI];
  {
    const bool live = c16 < Gt;
    const char *qrow = reinterpret_cast<const char *>(a.q) +
                       ((size_t)s * H + hb + (live ? c16 : 0)) * ROW;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(qrow + 64 * i + 16 * g4);
      qf[i] = live ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const bool bad_ctx = ctx < 0 || ctx > a.max_context_len ||
                       ctx > a.max_blocks_per_seq * a.block_size;
  const int nps = bad_ctx ? 1 : (ctx + P - 1) / P;
  if (p >= (nps > 0 ? nps : 1)) return;
  const bool direct = nps <= 1;
  const int t1 = bad_ctx ? t0 : min(t0 + P, ctx);
  const int nblk = bad_ctx ? 0 : ((t1 - t0 + a.block_size - 1) >> a.log2_block);
  const bool bad_id = tid < nblk && (id < 0 || id >= a.num_blocks);
  if (tid < nblk) s_tbl[tid] = id;
  const bool poison = __syncthreads_or(bad_id) || bad_ctx;

  const size_t head_stride = (size_t)a.block_size * D;
  const size_t block_stride = head_stride * Hkv;
  // The new token's slot, written by the partition that holds the token.
  // Like the separate cache write, it needs only the token's own slot to be
  // valid (a bad id elsewhere in the table poisons the output, not the write).
  if (new_lane && qt == 0 && !bad_ctx && ctx > t0 && ctx <= t1) {
    const int tn = ctx - 1;
    const int phys = s_tbl[(tn - t0) >> a.log2_block];
    if (phys >= 0 && phys < a.num_blocks) {
      const size_t dst = ((size_t)phys * block_stride + kvh * head_stride +
                          (size_t)(tn & (a.block_size - 1)) * D) * EKV + 16 * v_col;
      if constexpr (kF8) {            // the codes, staged before the barrier above
        nk = s_new[0][v_col];
        nv = s_new[1][v_col];
      }
      *reinterpret_cast<u32x4 *>(static_cast<char *>(a.k_store) + dst) = nk;
      *reinterpret_cast<u32x4 *>(static_cast<char *>(a.v_store) + dst) = nv;
    }
  }

  if (poison) {
    const float nan = __builtin_nanf("");
    for (int idx = tid; idx < Gt * D; idx += NW * 64) {
      const int q = idx / D, d = idx - q * D;
      const int h = hb + q;
      if (direct) {
        store_out<DT>(a.out, ((size_t)s * H + h) * D + d, &nan, 1);
      } else {
        const size_t part = ((size_t)s * H + h) * a.num_partitions + p;
        a.ws_o[part * D + d] = nan;
        if (d == 0) {
          a.ws_ml[2 * part] = __builtin_inff();
          a.ws_ml[2 * part + 1] = nan;
        }
      }
    }
    return;
  }

  const int nch = (t1 - t0 + kChunk - 1) / kChunk;
  const int nch_w = nch > wave ? (nch - wave + NW - 1) / NW : 0;
  int my_ids = 0;
  if (lane < nch_w) my_ids = s_tbl[((wave + NW * lane) * kChunk) >> a.log2_block];

  const char *kbase =
      scalar_ptr(reinterpret_cast<const char *>(a.k_cache) + kvh * head_stride * EKV);
  const char *vbase =
      scalar_ptr(reinterpret_cast<const char *>(a.v_cache) + kvh * head_stride * EKV);
  const int v_off = v_row * ROWKV + 16 * v_col;
  constexpr int kChunkBytes = kChunk * ROWKV;

  auto chunk_offset = [&](int k) -> size_t {
    const int phys = __builtin_amdgcn_readlane(my_ids, k);
    const int tok = (wave + NW * k) * kChunk;
    const int off = tok & (a.block_size - 1);
    return ((size_t)phys * block_stride + (size_t)off * D) * EKV;
  };
  // Chunks past the wave's last one (the pipeline's run-out) are loaded
  // through an empty descriptor: such loads return zeros without touching
  // memory, and their registers are never consumed.
  auto load = [&](u32x4 *kb, u32x4 *vb, int k, int last) {
    const size_t off = chunk_offset(min(k, last));
    const int range = k <= last ? kChunkBytes : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + off), (short)0, range, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + off), (short)0, range, kBufferFlags);
#pragma unroll
    for (int j = 0; j < VL; ++j)
      kb[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, v_off + j * TPL * ROWKV, 0, kStreamPolicy);
#pragma unroll
    for (int j = 0; j < VL; ++j)
      vb[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, v_off + j * TPL * ROWKV, 0, kStreamPolicy);
    __builtin_amdgcn_sched_barrier(0);
  };

  unsigned char *ktile = s_buf + wave * 2 * kTileBytes;
  unsigned char *tile = ktile + kTileBytes;
  // Transposed-read addresses: for tile n, lane (g4, c16) points at row
  // 4*g4 + c16/4, dims 16n + 4*(c16%4) .. +3; ds_read_b64_tr_b16 then hands
  // lane (g4, c16) the four values V[4*g4 + e][16n + c16], e = 0..3, which is
  // the B operand of the second product.
  const unsigned char *tr_base = tile + (4 * g4 + c16 / 4) * PITCH + 8 * (c16 % 4);
  float m = kNegInf;           // running reference max of query column c16
  float l = 0.f;               // this lane's share of the column's weight sum
  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 16-token chunk starting at token tc; rows at or past tend are masked.
  auto consume = [&](const u32x4 *kb, const u32x4 *vb, int tc, int tend) {
    const bool tail = tc + kChunk > tend;                // wave-uniform
    // Appending: this chunk holds the newest token (wave-uniform); lanes
    // 0..LPT-1 write its row over the pool's in the tiles.
    const bool inject = append && tc < ctx && ctx <= tc + kChunk;
    const int rn = ctx - 1 - tc;
    // K: through this wave's LDS tile into the A layout (lane l: token l%16,
    // bytes 64i + 16*(l/16) of its row).  Rows past the context are left as
    // they are: their scores are replaced by -inf below, by select.
#pragma unroll
    for (int j = 0; j < VL; ++j) stage16<DT, KT>(ktile + (v_row + j * TPL) * PITCH, v_col, kb[j]);
    if (inject && lane < LPT) stage16<DT, KT>(ktile + rn * PITCH, lane, s_new[0][lane]);
    u32x4 ka[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i)
      ka[i] = *reinterpret_cast<const u32x4 *>(ktile + c16 * PITCH + 64 * i + 16 * g4);
    // S^T for tokens 4*g4 + r of the chunk, query c16.
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KI; ++i) sacc = mfma_k32<DT>(ka[i], qf[i], sacc);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = sacc[r] * a.scale_log2;
    u32x4 vr[VL];
#pragma unroll
    for (int j = 0; j < VL; ++j) vr[j] = vb[j];
    if (tail) {
      // Tokens past the context: score -inf, V row zeroed (whatever the slot
      // holds must not meet a zero weight as NaN).
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (tc + 4 * g4 + r >= tend) sc[r] = kNegInf;
#pragma unroll
      for (int j = 0; j < VL; ++j)
        if (tc + v_row + j * TPL >= tend) vr[j] = u32x4{0u, 0u, 0u, 0u};
    }
    // V: stage the chunk in this wave's LDS tile.
#pragma unroll
    for (int j = 0; j < VL; ++j) stage16<DT, KT>(tile + (v_row + j * TPL) * PITCH, v_col, vr[j]);
    if (inject && lane < LPT) stage16<DT, KT>(tile + rn * PITCH, lane, s_new[1][lane]);

    // Raise the reference only when some score exceeds it by kLazyMax: every
    // lane of a query column holds the column's m, so the test needs no
    // cross-lane traffic; the column max is formed only on that rare path.
    const float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__builtin_amdgcn_ballot_w64(mloc > m + kLazyMax)) {
      const float cm = max_xor32(max_xor16(mloc));
      const float mnew = fmaxf(m, cm);
      const float corr = mnew == kNegInf ? 1.f : exp2_fast(m - mnew);
      l *= corr;
      // Output row q = 4*g4 + r needs the factor of query column q.
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

  // Software pipeline over NBUF register buffers: while chunk k is consumed,
  // chunks k+1 .. k+NBUF-1 are in flight.
  constexpr int NBUF = kGqaBuffers;
  u32x4 kb[NBUF][VL], vb[NBUF][VL];
  if (nch_w > 0) {
    const int last = nch_w - 1;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) load(kb[i], vb[i], i, last);
    for (int k0 = 0; k0 < nch_w; k0 += NBUF) {
#pragma unroll
      for (int i = 0; i < NBUF; ++i) {
        const int k = k0 + i;
        if (k >= nch_w) break;
        load(kb[(i + NBUF - 1) % NBUF], vb[(i + NBUF - 1) % NBUF], k + NBUF - 1, last);
        consume(kb[i], vb[i], t0 + (wave + NW * k) * kChunk, t1);
      }
    }
  }

  // Column sums over the four lane groups.
  l = sum_xor32(sum_xor16(l));

  // Cross-wave merge through LDS (the V tiles are dead now).
  __syncthreads();
  float *s_m = reinterpret_cast<float *>(s_buf);                // [NW][kGMax]
  float *s_l = s_m + NW * kGMax;                                 // [NW][kGMax]
  float *s_o = s_l + NW * kGMax;                                 // [NW][kGMax][D]
  if (g4 == 0) {
    s_m[wave * kGMax + c16] = m;
    s_l[wave * kGMax + c16] = l;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = 4 * g4 + r;
    if (q < Gt) {
#pragma unroll
      for (int n = 0; n < NT; ++n) s_o[(wave * kGMax + q) * D + 16 * n + c16] = o[n][r];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < Gt * D; idx += NW * 64) {
    const int q = idx / D, d = idx - q * D;
    float Mw = s_m[q];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mw = fmaxf(Mw, s_m[w * kGMax + q]);
    const float Ms = Mw == kNegInf ? 0.f : Mw;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2_fast(s_m[w * kGMax + q] - Ms);
      L += f * s_l[w * kGMax + q];
      O += f * s_o[(w * kGMax + q) * D + d];
    }
    if constexpr (kF8) O *= a.v_scale;        // the tiles held V codes
    const int h = hb + q;
    if (direct) {
      const float r = L == 0.f ? 0.f : O / L;
      store_out<DT>(a.out, ((size_t)s * H + h) * D + d, &r, 1);
    } else {
      const size_t part = ((size_t)s * H + h) * a.num_partitions + p;
      a.ws_o[part * D + d] = O;
      if (d == 0) {
        a.ws_ml[2 * part] = Mw;
        a.ws_ml[2 * part + 1] = L;
      }
    }
  }
}

template <int DT, int KT, int D>
hipError_t launch_gqa_t(const DecodeArgs &a, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  const long n = (long)a.num_seqs * a.num_kv_heads * ((G + kGMax - 1) / kGMax) * a.num_partitions;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_gqa_kernel<DT, KT, D, kGqaWaves>), dim3((unsigned)n),
                     dim3(kGqaWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gqa(const DecodeArgs &a, int dt, int kv_dt, hipStream_t stream) {
  const bool f8 = kv_dt == kFP8;
  if (!f8 && kv_dt != dt) return hipErrorInvalidValue;
  switch ((f8 ? 10000 : 0) + dt * 1000 + a.head_dim) {
    case kF16 * 1000 + 64: return launch_gqa_t<kF16, kF16, 64>(a, stream);
    case kF16 * 1000 + 128: return launch_gqa_t<kF16, kF16, 128>(a, stream);
    case kBF16 * 1000 + 64: return launch_gqa_t<kBF16, kBF16, 64>(a, stream);
    case kBF16 * 1000 + 128: return launch_gqa_t<kBF16, kBF16, 128>(a, stream);
    case 10000 + kF16 * 1000 + 64: return launch_gqa_t<kF16, kFP8, 64>(a, stream);
    case 10000 + kF16 * 1000 + 128: return launch_gqa_t<kF16, kFP8, 128>(a, stream);
    case 10000 + kBF16 * 1000 + 64: return launch_gqa_t<kBF16, kFP8, 64>(a, stream);
    case 10000 + kBF16 * 1000 + 128: return launch_gqa_t<kBF16, kFP8, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
