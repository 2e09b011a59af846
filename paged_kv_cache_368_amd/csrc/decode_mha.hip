// PagedAttention decode on the vector ALUs, and the log-sum-exp merge of
// split-context partitions, for gfx950.
//
// What is computed (P1 §1, first formula; P2 §2.1 steps 4-5; P3 §2): for
// sequence s and query head h,
//     out[s][h] = softmax(scale * q[s][h] . K^T) V
// over the s's first context_lens[s] tokens, each token's K/V row fetched
// from the physical block block_tables[s][t / B] at offset t % B (P3 §3).
//
// Work decomposition.  One work-group of 4 waves owns one (sequence, head,
// partition), or R consecutive partitions of one (sequence, head) taken one
// after the other when the context is split many ways (each still written as
// its own partial: the context length and q are loaded once, and the next
// partition's slice of the block table while this one streams).  The
// partition's slice of the block table is staged once into LDS; each wave
// then keeps the ids of the chunks it owns in one VGPR (lane k = its k-th
// chunk) and reads them with v_readlane, so no dependent memory load sits
// between one chunk's K/V loads and the next.  Waves take the partition's
// 16-token chunks round-robin, so at any moment the work-group streams four
// neighbouring chunks.
//
// Lane layout.  A K or V row of one token is D * elem bytes = LPT lanes x 16
// bytes (LPT = 16 for fp16/bf16 D=128 and fp32 D=64), so one 16-byte load per
// lane covers 64/LPT whole rows and every load of the wave is one contiguous
// kilobyte.  A lane's partial q.k is reduced over its LPT-lane row with DPP;
// each row keeps its own online-softmax state (running max m, running sum l,
// unnormalised output o) for the tokens that land on it, so the inner loop
// has no cross-row traffic at all.  Rows, then waves, are merged once at the
// end with the same max-rescaled sums.
//
// Pipelining.  K and V of chunk k+1 are issued before chunk k is consumed
// (double-buffered registers): P1 §4's overlap of the next block's loads with
// the current block's arithmetic, kept inside the kernel.
//
// Masking.  Tokens past the context in the last chunk get score -inf and
// their V words are zeroed by select, so whatever the unused slots hold
// (NaN in the tests) never reaches the result.
//
// Appending decode (pa_append_decode, pa_append_decode_fp8): the newest
// token of each sequence (position context_lens - 1) arrives as an input row
// (quantised here for E4M3 pools).  The row is kept in LDS; the partition
// that holds the token streams the pool only up to the token before it
// (whatever the slot held before never counts) and takes the new row as one
// extra masked chunk after its loop, and one work-group per (sequence, kv
// head) stores it into the slot for later steps: the slot resolution, the
// cache write and the attention of a decode step in one launch.
#include "pa_device.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_inff();

template <int KT, int D>
struct MhaShape {
  static constexpr int kE = Storage<KT>::kBytes;  // bytes per K/V element
  static constexpr int kEpl = 16 / kE;          // elements per lane per load
  static constexpr int kLpt = D / kEpl;         // lanes per token row
  static constexpr int kTpl = 64 / kLpt;        // token rows per wave load
  static constexpr int kLoads = kChunk / kTpl;  // loads per chunk, K and V each
  static_assert(kLpt == 4 || kLpt == 8 || kLpt == 16 || kLpt == 32, "row width");
};

// Per-lane dot of the lane's slice of q and of a K row: 16 bytes of K, and
// q in its own type (16 bytes, or 32 bytes against 16 E4M3 codes).
template <int QT, int KT>
__device__ __forceinline__ float lane_dot(const u32x4 *q, const u32x4 &k) {
  if constexpr (KT == kF32) {
    float acc = as_f32(q[0].x) * as_f32(k.x);
    acc = __builtin_fmaf(as_f32(q[0].y), as_f32(k.y), acc);
    acc = __builtin_fmaf(as_f32(q[0].z), as_f32(k.z), acc);
    acc = __builtin_fmaf(as_f32(q[0].w), as_f32(k.w), acc);
    return acc;
  } else if constexpr (KT == kFP8) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    const uint32_t qw[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = dot2<QT>(qw[2 * i], fp8_pair<QT, false>(kw[i]), acc);
      acc = dot2<QT>(qw[2 * i + 1], fp8_pair<QT, true>(kw[i]), acc);
    }
    return acc;
  } else {
    float acc = dot2<KT>(q[0].x, k.x, 0.f);
    acc = dot2<KT>(q[0].y, k.y, acc);
    acc = dot2<KT>(q[0].z, k.z, acc);
    acc = dot2<KT>(q[0].w, k.w, acc);
    return acc;
  }
}

// o[0..EPL) += p * (the lane's 16 bytes of a V row)
template <int KT>
__device__ __forceinline__ void lane_axpy(float *o, float p, const u32x4 &v) {
  if constexpr (KT == kF32) {
    o[0] = __builtin_fmaf(p, as_f32(v.x), o[0]);
    o[1] = __builtin_fmaf(p, as_f32(v.y), o[1]);
    o[2] = __builtin_fmaf(p, as_f32(v.z), o[2]);
    o[3] = __builtin_fmaf(p, as_f32(v.w), o[3]);
  } else if constexpr (KT == kFP8) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);   // bytes 0, 1
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);    // bytes 2, 3
      const float f0 = lo[0], f1 = lo[1], f2 = hi[0], f3 = hi[1];
      o[4 * i] = __builtin_fmaf(p, f0, o[4 * i]);
      o[4 * i + 1] = __builtin_fmaf(p, f1, o[4 * i + 1]);
      o[4 * i + 2] = __builtin_fmaf(p, f2, o[4 * i + 2]);
      o[4 * i + 3] = __builtin_fmaf(p, f3, o[4 * i + 3]);
    }
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __builtin_fmaf(p, lo_f32<KT>(w[i]), o[2 * i]);
      o[2 * i + 1] = __builtin_fmaf(p, hi_f32<KT>(w[i]), o[2 * i + 1]);
    }
  }
}

// DT: type of q and out; KT: storage type of the K/V pools (DT, or kFP8 with
// DT fp16/bf16).
template <int DT, int KT, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mha_kernel(DecodeArgs a) {
  using Sh = MhaShape<KT, D>;
  constexpr int E = Sh::kE, EPL = Sh::kEpl, LPT = Sh::kLpt, TPL = Sh::kTpl, NL = Sh::kLoads;
  constexpr int EQ = Storage<DT>::kBytes;         // bytes per q / out element
  constexpr int QW = EPL * EQ / 16;               // 16-byte words of q per lane
  static_assert(NW * 64 >= kMaxPartBlocks, "one thread per staged block id");

  __shared__ int s_tbl[kMaxPartBlocks];
  __shared__ float s_o[NW][D];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ u32x4 s_new[2][LPT];           // the newest token's K and V rows (appending)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform

  const int H = a.num_heads, S = a.num_seqs;
  const int G = H / a.num_kv_heads;
  const int item = group_on_xcd(blockIdx.x, gridDim.x, G);
  const int h = item % H;
  const int s = (item / H) % S;
  const int pg = item / (H * S);              // partitions pg * R .. pg * R + R - 1
  const int R = a.parts_per_group;
  const int kvh = h / G;
  const int row = lane / LPT;
  const int col = lane % LPT;
  const int P = a.partition_size;
  const size_t row_out = ((size_t)s * H + h) * D;

  // Issue the three independent prologue loads together: the context length,
  // the first partition's window of the block table (every entry the window can
  // hold that exists in the table, whatever the context turns out to be) and
  // q, a 16-byte slice per lane (every row of the wave holds the same slice).
  const int ctx = a.context_lens[s];
  // Partition pp's window of the block table: entry tid, if the table has it.
  auto table_entry = [&](int pp) -> int {
    const int bb = (pp * P) >> a.log2_block;
    const int window = min(P >> a.log2_block, a.max_blocks_per_seq - bb);
    return tid < window ? a.block_tables[(size_t)s * a.max_blocks_per_seq + bb + tid] : -1;
  };
  int id = table_entry(pg * R);
  u32x4 qv[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i)
    qv[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(a.q) +
                                             (row_out + col * EPL) * EQ + 16 * i);
  const bool append = a.new_k != nullptr;                      // uniform (kernel argument)
  // The newest token's K and V rows go to LDS (s_new) for the extra chunk and
  // the slot write.  Pools of the query's type: lanes 0..LPT-1 of wave 0 copy
  // their 16-byte slices.  E4M3 pools: the rows arrive in the query's type
  // and are quantised here exactly as the separate cache write does, four
  // elements per lane over the whole of wave 0 (K on lanes 0..D/4-1, V on the
  // next D/4), so the conversion stays short next to the prologue's loads.
  if (append && wave == 0) {
    const size_t row_in = ((size_t)s * a.num_kv_heads + kvh) * D * EQ;
    if constexpr (KT == kFP8) {
      constexpr int NE = D / 4;
      if (lane < 2 * NE) {
        const bool isv = lane >= NE;
        const int w = isv ? lane - NE : lane;
        const u32x2 raw = *reinterpret_cast<const u32x2 *>(
            static_cast<const char *>(isv ? a.new_v : a.new_k) + row_in + 4 * w * EQ);
        const float sc = isv ? a.v_scale : a.k_scale;
        const uint32_t word = e4m3_code(lo_f32<DT>(raw.x) / sc) |
                              (e4m3_code(hi_f32<DT>(raw.x) / sc) << 8) |
                              (e4m3_code(lo_f32<DT>(raw.y) / sc) << 16) |
                              (e4m3_code(hi_f32<DT>(raw.y) / sc) << 24);
        reinterpret_cast<uint32_t *>(&s_new[isv ? 1 : 0][0])[w] = word;
      }
    } else if (lane < LPT) {
      s_new[0][col] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.new_k) +
                                                       row_in + 16 * col);
      s_new[1][col] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.new_v) +
                                                       row_in + 16 * col);
    }
  }

  const bool bad_ctx = ctx < 0 || ctx > a.max_context_len ||
                       ctx > a.max_blocks_per_seq * a.block_size;
  const int nps = bad_ctx ? 1 : (ctx + P - 1) / P;
  const int nps1 = nps > 0 ? nps : 1;
  const bool direct = nps <= 1;
  // The work-group's partitions one after the other, each written as its own
  // partial; the next one's table window is loaded before this one streams.
  for (int rr = 0; rr < R; ++rr) {
    const int p = pg * R + rr;
    if (p >= nps1) break;                             // uniform over the work-group
    const int t0 = p * P;
    const int id_next = rr + 1 < R && p + 1 < nps1 ? table_entry(p + 1) : -1;
    const int t1 = bad_ctx ? t0 : min(t0 + P, ctx);
    const int nblk = bad_ctx ? 0 : ((t1 - t0 + a.block_size - 1) >> a.log2_block);

    // Stage the block ids in use; flag any outside the pool.
    const bool bad_id = tid < nblk && (id < 0 || id >= a.num_blocks);
    if (tid < nblk) s_tbl[tid] = id;
    const bool poison = __syncthreads_or(bad_id) || bad_ctx;

    const size_t part = ((size_t)s * H + h) * a.num_partitions + p;
    // The new token's slot: written by the first query head of its kv head, in
    // the partition that holds the token (one 16-byte slice per lane of row 0).
    const size_t head_stride = (size_t)a.block_size * D;        // elements per (block, head) tile
    const size_t block_stride = head_stride * a.num_kv_heads;
    // Like the separate cache write, it needs only the token's own slot to be
    // valid (a bad id elsewhere in the table poisons the output, not the write).
    if (append && tid < LPT && !bad_ctx && ctx > t0 && ctx <= t1 && h % G == 0) {
      const int tn = ctx - 1;
      const int phys = s_tbl[(tn - t0) >> a.log2_block];
      if (phys >= 0 && phys < a.num_blocks) {
        const size_t dst = ((size_t)phys * block_stride + kvh * head_stride +
                            (size_t)(tn & (a.block_size - 1)) * D + col * EPL) * E;
        *reinterpret_cast<u32x4 *>(static_cast<char *>(a.k_store) + dst) = s_new[0][col];
        *reinterpret_cast<u32x4 *>(static_cast<char *>(a.v_store) + dst) = s_new[1][col];
      }
    }
    if (poison) {
      const float nan = __builtin_nanf("");
      if (direct) {
        if (tid < D) {
          float v = nan;
          store_out<DT>(a.out, row_out + tid, &v, 1);
        }
      } else {
        if (tid < D) store_partial(a.ws_o + part * D + tid, nan);
        if (tid == 0) {
          store_partial(a.ws_ml + 2 * part, __builtin_inff());
          store_partial(a.ws_ml + 2 * part + 1, nan);
        }
      }
      __syncthreads();                              // s_tbl is rewritten next
      id = id_next;
      continue;
    }

    // Tokens read from the pool: [t0, tp); the newest token, when appending,
    // comes from LDS instead.
    const bool holds_new = append && ctx > t0 && ctx <= t1;        // uniform
    const int tp = holds_new ? ctx - 1 : t1;
    const int nch = (tp - t0 + kChunk - 1) / kChunk;
    const int nch_w = nch > wave ? (nch - wave + NW - 1) / NW : 0;
    // This wave's chunk k is partition chunk wave + NW*k; lane k keeps its block id.
    int my_ids = 0;
    if (lane < nch_w) my_ids = s_tbl[((wave + NW * lane) * kChunk) >> a.log2_block];

    const char *kbase =
        scalar_ptr(reinterpret_cast<const char *>(a.k_cache) + kvh * head_stride * E);
    const char *vbase =
        scalar_ptr(reinterpret_cast<const char *>(a.v_cache) + kvh * head_stride * E);
    const int lane_off = (row * D + col * EPL) * E;

    // Byte offset (from the kv head's first tile) of this wave's chunk k.
    auto chunk_offset = [&](int k) -> size_t {
      const int phys = __builtin_amdgcn_readlane(my_ids, k);
      const int tok = (wave + NW * k) * kChunk;                 // relative to t0, block aligned
      const int off = tok & (a.block_size - 1);
      return ((size_t)phys * block_stride + (size_t)off * D) * E;
    };

    // K and V of one chunk are read through two buffer descriptors whose base
    // is the chunk's first row (scalar registers) and whose range is the chunk:
    // every lane then needs only its 32-bit offset, and nothing outside the
    // chunk can be touched.
    constexpr int kChunkBytes = kChunk * D * E;
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
      for (int j = 0; j < NL; ++j)
        kb[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + j * TPL * D * E, 0,
                                                       kStreamPolicy);
#pragma unroll
      for (int j = 0; j < NL; ++j)
        vb[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, lane_off + j * TPL * D * E, 0,
                                                       kStreamPolicy);
      // Keep the scheduler from sinking these loads below the compute that
      // follows: they must be in flight while the previous chunk is consumed.
      __builtin_amdgcn_sched_barrier(0);
    };

    float m = kNegInf, l = 0.f;
    float o[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = 0.f;

    // One 16-token chunk starting at token tc; rows at or past tend are masked.
    auto consume = [&](const u32x4 *kb, const u32x4 *vb, int tc, int tend) {
      float sc[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j)
        sc[j] = group_sum<LPT>(lane_dot<DT, KT>(qv, kb[j])) * a.scale_log2;
      const bool tail = tc + kChunk > tend;                     // last chunk: mask past the context
      bool valid[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        valid[j] = !tail || (tc + j * TPL + row < tend);
        sc[j] = valid[j] ? sc[j] : kNegInf;
      }
      float mloc = sc[0];
#pragma unroll
      for (int j = 1; j < NL; ++j) mloc = fmaxf(mloc, sc[j]);
      const float mnew = fmaxf(m, mloc);
      const float msafe = mnew == kNegInf ? 0.f : mnew;
      const float corr = exp2_fast(m - msafe);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i] *= corr;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const float pj = exp2_fast(sc[j] - msafe);
        psum += pj;
        const u32x4 v = valid[j] ? vb[j] : u32x4{0u, 0u, 0u, 0u};
        lane_axpy<KT>(o, pj, v);
      }
      l = l * corr + psum;
      m = mnew;
    };

    // Software pipeline over NBUF register buffers: while chunk k is consumed,
    // chunks k+1 .. k+NBUF-1 are in flight.  Loads past the last chunk go
    // through an empty descriptor (see load).
    constexpr int NBUF = KT == kFP8 ? kDecodeBuffersFp8 : kDecodeBuffers;
    u32x4 kb[NBUF][NL], vb[NBUF][NL];
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
          consume(kb[i], vb[i], t0 + (wave + NW * k) * kChunk, tp);
        }
      }
    }
    // The newest token as a chunk of one valid row (row 0 of wave 0).
    if (holds_new && wave == 0) {
      u32x4 kn[NL], vn[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const bool mine = j == 0 && row == 0;
        kn[j] = mine ? s_new[0][col] : u32x4{0u, 0u, 0u, 0u};
        vn[j] = mine ? s_new[1][col] : u32x4{0u, 0u, 0u, 0u};
      }
      consume(kn, vn, ctx - 1, ctx);
    }

    // Merge the rows of this wave (lanes with equal col, different row).
    float M = m;
#pragma unroll
    for (int msk = LPT; msk < 64; msk <<= 1) M = fmaxf(M, __shfl_xor(M, msk));
    {
      const float Ms = M == kNegInf ? 0.f : M;
      const float w = exp2_fast(m - Ms);
      l *= w;
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i] *= w;
    }
#pragma unroll
    for (int msk = LPT; msk < 64; msk <<= 1) {
      l += __shfl_xor(l, msk);
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i] += __shfl_xor(o[i], msk);
    }
    if (row == 0) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) s_o[wave][col * EPL + i] = o[i];
      if (col == 0) {
        s_m[wave] = M;
        s_l[wave] = l;
      }
    }
    __syncthreads();

    // Merge the NW waves; thread d < D owns output element d.
    if (tid < D) {
      float Mw = s_m[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) Mw = fmaxf(Mw, s_m[w]);
      const float Ms = Mw == kNegInf ? 0.f : Mw;
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2_fast(s_m[w] - Ms);
        L += f * s_l[w];
        O += f * s_o[w][tid];
      }
      if constexpr (KT == kFP8) O *= a.v_scale;   // values are code * V pool scale
      if (direct) {
        const float r = L == 0.f ? 0.f : O / L;   // NaN (a poisoned partition) propagates
        store_out<DT>(a.out, row_out + tid, &r, 1);
      } else {
        store_partial(a.ws_o + part * D + tid, O);
        if (tid == 0) {
          store_partial(a.ws_ml + 2 * part, Mw);
          store_partial(a.ws_ml + 2 * part + 1, L);
        }
      }
    }
    id = id_next;
  }
}

// Log-sum-exp merge of split-context partitions: one work-group of NW waves
// per (s, h): one wave when the launch has at most kMergeBatch partitions
// (its one batch of loads is the whole merge, combined in registers), four
// otherwise.
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
// Wave w takes partitions w, w + NW, ... in batches of kMergeBatch whose loads
// are all issued before any is used, keeping its own running (max, sum,
// output) with the same rescaling as the decode loop; several waves are
// combined through LDS.  The first batch is loaded together with the
// context length, before the sequence's partition count is known (clamped
// to the launch's partition count, so every load stays in the workspace;
// partitions past the sequence's count are never used).  Sequences that fit
// one partition were written directly by the decode kernel and are skipped.
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 8;

template <int DT, int D, int NW>
__global__ __launch_bounds__(NW * 64) void merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;                  // output elements per lane
  __shared__ float s_o[NW][D];
  __shared__ float s_m[NW], s_l[NW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x;                 // s * H + h
  const int s = item / a.num_heads;
  const size_t base = (size_t)item * a.num_partitions;
  float mp[kMergeBatch], lp[kMergeBatch], op[kMergeBatch][PER];
  auto load = [&](int p0, int plast) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int p = min(p0 + u * NW, plast);   // clamped loads are never used
      mp[u] = a.ws_ml[2 * (base + p)];
      lp[u] = a.ws_ml[2 * (base + p) + 1];
      const float *src = a.ws_o + (base + p) * D + lane * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i) op[u][i] = src[i];
    }
  };
  const int ctx = a.context_lens[s];
  load(wave, a.num_partitions - 1);
  const int P = a.partition_size;
  if (ctx < 0 || ctx > a.max_context_len || ctx > a.max_blocks_per_seq * a.block_size) return;
  const int nps = (ctx + P - 1) / P;
  if (nps <= 1) return;                        // uniform over the work-group

  float m = kNegInf, l = 0.f;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int p0 = wave; p0 < nps; p0 += NW * kMergeBatch) {
    if (p0 != wave) load(p0, nps - 1);
    float mb = m;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (p0 + u * NW < nps) mb = fmaxf(mb, mp[u]);
    const float ms = mb == kNegInf ? 0.f : mb;
    const float c = exp2_fast(m - ms);
    l *= c;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] *= c;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (p0 + u * NW < nps) {
        const float f = exp2_fast(mp[u] - ms);
        l = __builtin_fmaf(f, lp[u], l);
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] = __builtin_fmaf(f, op[u][i], o[i]);
      }
    }
    m = mb;
  }
  if constexpr (NW == 1) {
    // One wave: its running (max, sum, output) is the merge.
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const float r = l == 0.f ? 0.f : o[i] / l;   // NaN (a poisoned partition) propagates
      store_out<DT>(a.out, (size_t)item * D + lane * PER + i, &r, 1);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) s_o[wave][lane * PER + i] = o[i];
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float Mw = s_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mw = fmaxf(Mw, s_m[w]);
    const float Ms = Mw == kNegInf ? 0.f : Mw;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2_fast(s_m[w] - Ms);
      L += f * s_l[w];
      O += f * s_o[w][d];
    }
    const float r = L == 0.f ? 0.f : O / L;    // NaN (a poisoned partition) propagates
    store_out<DT>(a.out, (size_t)item * D + d, &r, 1);
  }
}

// Partitions per vector work-group: four when the context is split at least
// eight ways and that still leaves 4096 work-groups (four rounds of the
// 1024 that 256 CUs hold at once), else one.  On 8 sequences x 32 heads of
// 64 partitions: 639-641 against 642-644 us per call.
inline int mha_parts_per_group(long items, int np) {
  constexpr int R = 4;
  return np >= 2 * R && items * ((np + R - 1) / R) >= 4096 ? R : 1;
}

template <int DT, int KT, int D>
hipError_t launch_mha_kt(const DecodeArgs &a, hipStream_t stream) {
  DecodeArgs b = a;
  b.parts_per_group = mha_parts_per_group((long)a.num_seqs * a.num_heads, a.num_partitions);
  const long groups = (a.num_partitions + b.parts_per_group - 1) / b.parts_per_group;
  const long n = (long)a.num_seqs * a.num_heads * groups;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_mha_kernel<DT, KT, D, kDecodeWaves>), dim3((unsigned)n),
                     dim3(kDecodeWaves * 64), 0, stream, b);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_mha_t(const DecodeArgs &a, hipStream_t stream) {
  return launch_mha_kt<DT, DT, D>(a, stream);
}

template <int DT, int D>
hipError_t launch_mha_fp8_t(const DecodeArgs &a, hipStream_t stream) {
  if constexpr (DT == kF32) return hipErrorInvalidValue;
  else return launch_mha_kt<DT, kFP8, D>(a, stream);
}

template <int DT, int D>
hipError_t launch_merge_t(const DecodeArgs &a, hipStream_t stream) {
  const long n = (long)a.num_seqs * a.num_heads;
  if (n <= 0) return hipSuccess;
  if (a.num_partitions <= kMergeBatch)
    hipLaunchKernelGGL((merge_kernel<DT, D, 1>), dim3((unsigned)n), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((merge_kernel<DT, D, kMergeWaves>), dim3((unsigned)n),
                       dim3(kMergeWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

#define PA_DISPATCH(FN, dt, D, ...)                                        \
  switch (dt * 1000 + D) {                                                 \
    case kF32 * 1000 + 64: return FN<kF32, 64>(__VA_ARGS__);               \
    case kF32 * 1000 + 128: return FN<kF32, 128>(__VA_ARGS__);             \
    case kF16 * 1000 + 64: return FN<kF16, 64>(__VA_ARGS__);               \
    case kF16 * 1000 + 128: return FN<kF16, 128>(__VA_ARGS__);             \
    case kBF16 * 1000 + 64: return FN<kBF16, 64>(__VA_ARGS__);             \
    case kBF16 * 1000 + 128: return FN<kBF16, 128>(__VA_ARGS__);           \
    default: return hipErrorInvalidValue;                                  \
  }

hipError_t launch_decode_mha(const DecodeArgs &a, int dt, int kv_dt, hipStream_t stream) {
  if (kv_dt == kFP8) {
    PA_DISPATCH(launch_mha_fp8_t, dt, a.head_dim, a, stream)
  }
  if (kv_dt != dt) return hipErrorInvalidValue;
  PA_DISPATCH(launch_mha_t, dt, a.head_dim, a, stream)
}

hipError_t launch_merge(const DecodeArgs &a, int dt, hipStream_t stream) {
  PA_DISPATCH(launch_merge_t, dt, a.head_dim, a, stream)
}

}  // namespace pa
