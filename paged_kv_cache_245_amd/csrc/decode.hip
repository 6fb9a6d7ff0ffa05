// decode.hip - paged decode attention for gfx950: one query per request at its
// last position, over every token of its logical context, read through the
// request's block table (arcyou teardown of vLLM paged attention, section
// "PagedAttention: the KV cache is paged, like virtual memory"; every new token
// re-reads all past K/V: kenhuang vLLM course, "PagedAttention (intuition)").
//
// Decode is a stream over the pool: ~G flop per byte of K/V, far below the MFMA
// or VALU ridge, so the design goal is that every compute unit streams K/V at
// its full rate from the first to the last microsecond.
//
// Work split (balanced mode, the default). The requests' blocks are laid end to
// end (request 0's blocks, then request 1's, ...), T blocks in all, and
// workgroup w of W takes blocks [w*T/W, (w+1)*T/W): every workgroup gets the
// same number of blocks whatever the length mix, and streams them in order.
// A workgroup has one wavefront per kv head (up to 8), so together they read
// whole token rows: a 16-token block of 8 kv heads x 128 dims is one contiguous
// 32 KiB read. A workgroup's range is cut at request boundaries into segments;
// each segment keeps an online softmax (running max m, sum of exponentials l,
// unnormalised output acc). A segment that is a whole request writes the final
// output; otherwise it stores (m, l, acc) in slot (request + worker), and a
// merge kernel combines a request's slots: out = sum(2^(m_i-M) acc_i) /
// sum(2^(m_i-M) l_i), M = max m_i. The slot index is unique because walking the
// block axis, every segment boundary advances the request, the worker, or both,
// so (request + worker) strictly increases from segment to segment. When the
// requests outnumber the workers, most are whole: each worker then records the
// request (if any) whose first cut falls at the start of its range, and the
// merge grid runs over those records instead of over every request.
// Fixed-partition mode (an explicit partition size, or very large batches):
// one workgroup per (request, partition of P keys, group of kv heads).
//
// Per wavefront and per pair of 16-token blocks (32 keys), with MFMA 16x16x32 bf16:
//   S^T[16 keys x 16 heads] = K[16 x D] . Q^T[D x 16]     (D/32 MFMAs per block)
//     A operand: lane (n = lane%16, g4 = lane/16) holds 8 dims of key n's row;
//     B operand: the G query heads of this kv head in columns 0..G-1 (rest 0).
//     Result: lane (n, g4) holds head n's scores for keys 4 g4 .. 4 g4 + 3.
//   O^T[16 dims x 16 heads] += V^T[16 x 32 keys] . P^T[32 keys x 16 heads]
//     B operand = the lane's own 8 probabilities (4 keys of each block), so the
//     softmax output never moves between lanes. A operand = V of those same 8
//     keys: the lane loads D/16 consecutive dims of each of the 8 rows and
//     transposes the 8 x (D/16) tile in registers. Lane (n, g4) ends up owning
//     head n, dims (D/4) g4 .. (D/4) g4 + D/4 - 1.
//   Probabilities are rounded to bf16 for the PV product; l sums the fp32 values.
//   Scores are in log2 units (scale * log2 e), so each exponential is v_exp_f32.
// The next pair's K/V is loaded before the current pair is used (two register
// buffers), and a segment's block ids are fetched 64 at a time into one VGPR.
// In balanced mode a worker streams its segments back to back: the next
// segment's first pair is issued while the current segment's last pair is
// attended, and segment results are staged in LDS and written after the
// worker's last segment (see stream_range).
//
// fp32 pools use a plain VALU kernel (lanes over keys for q.k, lanes over dims
// for PV) in fixed-partition mode.
#include <algorithm>
#include <cstdlib>

#include "pa_device.h"

namespace pa {
namespace {

constexpr int kMaxBalancedSeqs = 8192;  // requests whose block prefix sums fit in LDS

template <int D>
struct VRowT;
template <>
struct VRowT<128> { typedef u32x4 type; };
template <>
struct VRowT<64> { typedef u32x2 type; };

template <class T, bool kNT>
__device__ __forceinline__ T load_kv(const uint16_t* p) {
  if constexpr (kNT) return __builtin_nontemporal_load((const T*)p);
  else return *(const T*)p;
}

// K and V of one pair of blocks as seen by one lane.
template <int D>
struct Tile {
  u32x4 k0[D / 32], k1[D / 32];
  typename VRowT<D>::type v[8];
};

// Byte offsets of one lane's K and V pieces inside a block (the same for every
// block): K row n, dims 8 g4 + 32 c; V rows 4 g4 .. 4 g4 + 3, dims (D/16) n ...
struct LaneOffsets {
  uint32_t k;  // + 64 c for chunk c
  uint32_t v;  // + j * row_bytes for row j
  uint32_t row_bytes;
};

template <int D>
__device__ __forceinline__ LaneOffsets lane_offsets(int kvh, int Hkv, int n, int g4) {
  LaneOffsets o;
  o.row_bytes = (uint32_t)(Hkv * D * 2);
  o.k = (uint32_t)(kv_row(0, n, kvh, Hkv, D) * 2) + 16u * g4;
  o.v = (uint32_t)(kv_row(0, 4 * g4, kvh, Hkv, D) * 2) + (uint32_t)(D / 16) * 2u * n;
  return o;
}

template <int D, bool kNT>
__device__ __forceinline__ void load_pair(Tile<D>& t, const uint16_t* K, const uint16_t* V,
                                          int32_t id0, int32_t id1, bool two,
                                          const LaneOffsets& o) {
  typedef typename VRowT<D>::type VRow;
  // wavefront-uniform block bases (the block id is a scalar), per-lane fixed offsets
  const int64_t block_bytes = (int64_t)kBlock * o.row_bytes;
  const char* kb0 = (const char*)K + (int64_t)id0 * block_bytes;
  const char* vb0 = (const char*)V + (int64_t)id0 * block_bytes;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) t.k0[c] = load_kv<u32x4, kNT>((const uint16_t*)(kb0 + o.k + 64 * c));
#pragma unroll
  for (int j = 0; j < 4; ++j) t.v[j] = load_kv<VRow, kNT>((const uint16_t*)(vb0 + o.v + j * o.row_bytes));
  if (two) {
    const char* kb1 = (const char*)K + (int64_t)id1 * block_bytes;
    const char* vb1 = (const char*)V + (int64_t)id1 * block_bytes;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) t.k1[c] = load_kv<u32x4, kNT>((const uint16_t*)(kb1 + o.k + 64 * c));
#pragma unroll
    for (int j = 0; j < 4; ++j) t.v[4 + j] = load_kv<VRow, kNT>((const uint16_t*)(vb1 + o.v + j * o.row_bytes));
  } else {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) t.k1[c] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) t.v[4 + j] = VRow{};
  }
}

// Online-softmax update with one pair of blocks; `valid` = keys of the pair
// (0..32, in order) that belong to the range being attended. kCols (short-chunk
// mode): this lane's column also masks the keys from col_valid on (its position's
// causal limit), and a column that has seen no key yet keeps m = -inf, l = 0 and
// acc = 0 (the max is taken as 0 in the exponentials while it is -inf).
template <int D, bool kCols = false>
__device__ __forceinline__ void attend_pair(Tile<D>& t, const u32x4* qb, f32x4* acc, float& m,
                                            float& lsum, float scale_log2, int valid, int g4,
                                            int col_valid = 32) {
  constexpr int kDL = D / 16;
  typedef typename VRowT<D>::type VRow;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k0[c]), as_bf16x8(qb[c]), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k1[c]), as_bf16x8(qb[c]), s1, 0, 0, 0);
  }
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = s0[i] * scale_log2;
    sc[4 + i] = s1[i] * scale_log2;
  }
  if (valid < 32) {  // keys past the range: score -inf (by selection), V row 0
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j >> 2) * 16 + 4 * g4 + (j & 3) >= valid) {
        sc[j] = -INFINITY;
        t.v[j] = VRow{};
      }
    }
  }
  if constexpr (kCols) {
    if (col_valid < 32) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((j >> 2) * 16 + 4 * g4 + (j & 3) >= col_valid) sc[j] = -INFINITY;
    }
  }
  float tmax = sc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const float m_new = fmaxf(m, tmax);
  const float m_use = (kCols && m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2(m - m_use);
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = fast_exp2(sc[j] - m_use);
    psum += p[j];
  }
  lsum = lsum * alpha + psum;
  m = m_new;
  const u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                    pack_bf16x2(p[6], p[7])};
#pragma unroll
  for (int d = 0; d < kDL; ++d) {
    u32x4 va;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t lo = t.v[2 * u][d >> 1];
      const uint32_t hi = t.v[2 * u + 1][d >> 1];
      va[u] = (d & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    acc[d] *= alpha;
    acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), acc[d], 0, 0, 0);
  }
}

// acc[d][i] of lane (n, g4) is dim (D/16) * (4 g4 + i) + d of head n.
template <int D>
__device__ __forceinline__ void store_final(uint16_t* O, int64_t qo_row, const f32x4* acc,
                                            float lsum, int g4) {
  constexpr int kDL = D / 16;
  const float inv = 1.f / lsum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint16_t* dst = O + qo_row + kDL * (4 * g4 + i);
    if constexpr (D == 128) {
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(acc[2 * t][i] * inv, acc[2 * t + 1][i] * inv);
      *(u32x4*)dst = w;
    } else {
      u32x2 w;
#pragma unroll
      for (int t = 0; t < 2; ++t) w[t] = pack_bf16x2(acc[2 * t][i] * inv, acc[2 * t + 1][i] * inv);
      *(u32x2*)dst = w;
    }
  }
}

// The partial (m, l, acc) of one (segment, q head). kBf16 (shared-prefix mode,
// its own kernel instantiation): acc is stored in bf16 (rounded to nearest
// even), as the prefix pass stores its own, so the merge reads both lists alike,
// at half the bytes.
template <int D, bool kBf16 = false>
__device__ __forceinline__ void store_partial(const DecodeArgs& a, int64_t pidx, const f32x4* acc,
                                              float m, float lsum, int g4) {
  constexpr int kDL = D / 16;
  if constexpr (kBf16) {
    uint32_t* dst = (uint32_t*)((uint16_t*)a.part_acc + pidx * D);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t2 = 0; t2 < kDL; t2 += 2)
        dst[(kDL * (4 * g4 + i) + t2) / 2] = pack_bf16x2(acc[t2][i], acc[t2 + 1][i]);
  } else {
    float* dst = a.part_acc + pidx * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t4 = 0; t4 < kDL; t4 += 4)
        *(f32x4*)(dst + kDL * (4 * g4 + i) + t4) =
            f32x4{acc[t4][i], acc[t4 + 1][i], acc[t4 + 2][i], acc[t4 + 3][i]};
  }
  if (g4 == 0) {
    a.part_ml[2 * pidx] = m;
    a.part_ml[2 * pidx + 1] = lsum;
  }
}

// One wavefront attends keys of blocks [blk_a, blk_b) of request s (kv head kvh),
// keys limited to the first `end_tok` tokens, and writes the final output (whole)
// or the partial state into partial row pidx_base + q head.
template <int D, bool kNT, bool kBf16 = false>
__device__ __forceinline__ void decode_segment(const DecodeArgs& a, int s, int kvh, int blk_a,
                                               int blk_b, int end_tok, bool whole,
                                               int64_t pidx_base, int64_t pidx_stride) {
  constexpr int kChunks = D / 32;
  constexpr int kDL = D / 16;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int h = kvh * G + n;
  const bool head_ok = n < G;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v;
  const int64_t qo_row = ((int64_t)s * a.num_q_heads + h) * D;

  u32x4 qb[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    qb[c] = head_ok ? *(const u32x4*)((const uint16_t*)a.q + qo_row + 32 * c + 8 * g4)
                    : u32x4{0, 0, 0, 0};
  f32x4 acc[kDL];
#pragma unroll
  for (int t = 0; t < kDL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  bool poisoned = false;

  // block ids of this segment, 64 per refill: lane i holds the id of block base + i
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  int base = blk_a;
  int32_t idv = (lane < blk_b - base) ? table[base + lane] : 0;
  auto block_id = [&](int b) -> int32_t {
    if (b - base >= 64) {
      base += 64;
      idv = (lane < blk_b - base) ? table[base + lane] : 0;
    }
    int32_t id = __builtin_amdgcn_readlane(idv, b - base);
    if (!block_ok(id, a.num_blocks)) {
      poisoned = true;
      id = 0;
    }
    return id;
  };
  const LaneOffsets offs = lane_offsets<D>(kvh, Hkv, n, g4);
  auto issue = [&](Tile<D>& t, int b) {
    const bool two = b + 1 < blk_b;
    const int32_t id0 = block_id(b);
    const int32_t id1 = two ? block_id(b + 1) : 0;
    load_pair<D, kNT>(t, K, V, id0, id1, two, offs);
  };

  end_tok = min(end_tok, 16 * blk_b);  // a segment may stop before the request does
  Tile<D> ta, tb;
  int b = blk_a;
  issue(ta, b);
  while (true) {
    if (b + 2 < blk_b) issue(tb, b + 2);
    attend_pair<D>(ta, qb, acc, m, lsum, a.scale_log2, min(32, end_tok - 16 * b), g4);
    b += 2;
    if (b >= blk_b) break;
    if (b + 2 < blk_b) issue(ta, b + 2);
    attend_pair<D>(tb, qb, acc, m, lsum, a.scale_log2, min(32, end_tok - 16 * b), g4);
    b += 2;
    if (b >= blk_b) break;
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (poisoned) lsum = __builtin_nanf("");
  if (!head_ok) return;
  if (whole)
    store_final<D>((uint16_t*)a.out, qo_row, acc, lsum, g4);
  else
    store_partial<D, kBf16>(a, pidx_base + (int64_t)h * pidx_stride, acc, m, lsum, g4);
}

// Lean variant of decode_segment, for a decode that shares compute units with a
// concurrently running prefill: the prefill's eight wavefronts leave 96 of the
// 512 registers per SIMD lane, so this wavefront holds one 16-token block of K
// and V at a time (no second buffer, no block pair). Per block, with lane (n, g4)
// as in decode_segment:
//   S^T[16 keys x 16 heads] = K . Q^T    (D/32 MFMA 16x16x32 bf16)
//   O^T[16 dims x 16 heads] += V^T . P^T (D/16 MFMA 16x16x16 bf16: the lane's own
//     4 probabilities are its B operand; its A operand is element d of each of
//     the 4 V rows it loaded, so the output layout is decode_segment's)
template <int D, bool kNT>
__device__ __forceinline__ void decode_segment_lean(const DecodeArgs& a, int s, int kvh, int blk_a,
                                                    int blk_b, int end_tok, bool whole,
                                                    int64_t pidx_base, int64_t pidx_stride,
                                                    u32x4* q_lds) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef typename VRowT<D>::type VRow;
  constexpr int kChunks = D / 32;
  constexpr int kDL = D / 16;
  // The lane index is made opaque here, so that the per-lane addresses derived from
  // it are computed per segment instead of being hoisted out of the caller's
  // segment loop and held (or spilled) across it.
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int h = kvh * G + n;
  const bool head_ok = n < G;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v;
  const int64_t qo_row = ((int64_t)s * a.num_q_heads + h) * D;

  // The query operands wait in LDS (q_lds: D/32 x 64 slots, each lane its own) and
  // are read again for every block, instead of D/8 registers held across the loop.
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    q_lds[c * 64 + lane] = head_ok ? *(const u32x4*)((const uint16_t*)a.q + qo_row + 32 * c + 8 * g4)
                                   : u32x4{0, 0, 0, 0};
  f32x4 acc[kDL];
#pragma unroll
  for (int t = 0; t < kDL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  bool poisoned = false;

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  int base = blk_a;
  int32_t idv = (lane < blk_b - base) ? table[base + lane] : 0;
  const LaneOffsets o = lane_offsets<D>(kvh, Hkv, n, g4);
  const int64_t block_bytes = (int64_t)kBlock * o.row_bytes;
  end_tok = min(end_tok, 16 * blk_b);
  for (int b = blk_a; b < blk_b; ++b) {
    if (b - base >= 64) {
      base += 64;
      idv = (lane < blk_b - base) ? table[base + lane] : 0;
    }
    int32_t id = __builtin_amdgcn_readlane(idv, b - base);
    if (!block_ok(id, a.num_blocks)) {
      poisoned = true;
      id = 0;
    }
    const char* kb = (const char*)K + (int64_t)id * block_bytes;
    const char* vb = (const char*)V + (int64_t)id * block_bytes;
    u32x4 k[kChunks];
    VRow v[4];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) k[c] = load_kv<u32x4, kNT>((const uint16_t*)(kb + o.k + 64 * c));
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = load_kv<VRow, kNT>((const uint16_t*)(vb + o.v + j * o.row_bytes));

    // a compiler barrier: the query reads below stay inside the loop (hoisted, they
    // would hold their registers across it)
    asm volatile("" ::: "memory");
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      // one query chunk live at a time (the scheduling barriers keep the next
      // chunk's read below this product)
      const u32x4 qc = q_lds[c * 64 + lane];
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[c]), as_bf16x8(qc), s0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = s0[i] * a.scale_log2;
    const int valid = min(16, end_tok - 16 * b);
    if (valid < 16) {  // keys past the range: score -inf (by selection), V row 0
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (4 * g4 + j >= valid) {
          sc[j] = -INFINITY;
          v[j] = VRow{};
        }
      }
    }
    float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - m_new);
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = fast_exp2(sc[j] - m_new);
      psum += p[j];
    }
    lsum = lsum * alpha + psum;
    m = m_new;
    const v4i16 pb = __builtin_bit_cast(v4i16, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
#pragma unroll
    for (int d = 0; d < kDL; ++d) {
      const int sh = 16 * (d & 1);
      const uint32_t e0 = (v[0][d >> 1] >> sh) & 0xffffu, e1 = (v[1][d >> 1] >> sh) & 0xffffu;
      const uint32_t e2 = (v[2][d >> 1] >> sh) & 0xffffu, e3 = (v[3][d >> 1] >> sh) & 0xffffu;
      const v4i16 va = __builtin_bit_cast(v4i16, u32x2{e0 | (e1 << 16), e2 | (e3 << 16)});
      acc[d] *= alpha;
      acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[d], 0, 0, 0);
    }
    // and the next block's loads stay below this block's products (one block of K
    // and V live at a time)
    asm volatile("" ::: "memory");
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (poisoned) lsum = __builtin_nanf("");
  if (!head_ok) return;
  if (whole)
    store_final<D>((uint16_t*)a.out, qo_row, acc, lsum, g4);
  else
    store_partial<D>(a, pidx_base + (int64_t)h * pidx_stride, acc, m, lsum, g4);
}

// Worker holding global block b when T >= W blocks are split over W workers
// (worker w owns blocks [w*T/W, (w+1)*T/W), never an empty range).
__device__ __forceinline__ int worker_of(int64_t b, int64_t T, int W) {
  return (int)(((b + 1) * W + T - 1) / T) - 1;
}

// Keys of request s that the balanced kernel reads from the pool: all of its
// context, or in append mode all but the newest token (the merge attends that one).
template <bool kAppend>
__device__ __forceinline__ int pool_keys(const DecodeArgs& a, int s) {
  const int L = min(a.context_lens[s], a.max_context_len);
  return kAppend ? L - 1 : L;
}

// Blocks of request s the balanced kernel reads: those holding its pool keys,
// less the first skip_blocks (shared-prefix mode).
template <bool kAppend>
__device__ __forceinline__ int request_blocks(const DecodeArgs& a, int s) {
  const int n = pool_keys<kAppend>(a, s);
  return n > 0 ? max(((n + 15) >> 4) - a.skip_blocks, 0) : 0;
}

// Segment results wait in LDS until the worker's range is done. Vector-memory
// operations retire in order, so a store holds up every later wait on a load
// until the store is acknowledged; under a full read stream that costs several
// microseconds per store, once per segment. Staged, the stores all go out after
// the last load is used. Each wavefront has a.ring_bytes of LDS, filled
// front to back with records: a 16-byte header (request; top bit set for a
// whole request), then for a whole request the final bf16 words of its 4 G
// lanes (what store_final writes), else their fp32 acc followed by (m, l) per
// head. A segment whose record does not fit any more is stored directly. The
// host sizes the buffer (a.ring_bytes per wavefront, at most kRingCapPerWave)
// so that the workgroups the kernel's registers admit on a compute unit still
// fit its LDS beside their prefix sums.
constexpr int kRingCapPerWave = 15 * 1024;
__host__ __device__ constexpr size_t ring_offset(int S) { return ((size_t)(S + 1) * 4 + 15) & ~(size_t)15; }

// A worker's whole block range [lo, hi) for one kv head, segment after segment,
// with the next segment's first pair of blocks issued while the current
// segment's last pair is attended (decode_segment starts each segment cold:
// block ids, then the first pair, then the products). The issue cursor runs
// one pair ahead of the attend cursor, so it is in the attended segment or the
// one after it; the block ids of the segment after the issue cursor's are
// fetched when the cursor enters a segment.
// kCols: short-chunk mode (see DecodeArgs); lane column n is position n / G, q head
// n % G, the C = n_cols * G columns in use.
template <int D, bool kNT, bool kAppend, bool kBf16, bool kCols = false>
__device__ __forceinline__ void stream_range(const DecodeArgs& a, const int32_t* cum, int first, int lo,
                                             int hi, int w, int kvh) {
  constexpr int kChunks = D / 32;
  constexpr int kDL = D / 16;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int G = a.group;
  const int C = kCols ? a.n_cols * G : G;      // columns in use
  const int pc = kCols ? n / G : 0;            // this lane's position (short-chunk mode)
  const int Hkv = a.num_kv_heads;
  const int h = kvh * G + (kCols ? n % G : n);
  const bool lane_ok = n < C;
  // rows of request s in short-chunk mode: [query_start_loc[s], query_start_loc[s + 1])
  auto chunk_of = [&](int s, int& q0, int& nq) {
    q0 = kCols ? a.query_start_loc[s] : s;
    nq = kCols ? a.query_start_loc[s + 1] - q0 : 1;
  };
  // output row (the q row) and partial row of (request s, this lane's column)
  auto out_row = [&](int s, int q0) -> int64_t { return ((int64_t)(kCols ? q0 + pc : s) * a.num_q_heads + h) * D; };
  auto part_row = [&](int s) -> int64_t {
    return kCols ? (((int64_t)s + w) * a.n_cols + pc) * a.num_q_heads + h : ((int64_t)s + w) * a.num_q_heads + h;
  };
  const uint16_t* __restrict__ K = (const uint16_t*)a.k;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v;
  const LaneOffsets offs = lane_offsets<D>(kvh, Hkv, n, g4);

  // segment of request s (or a later one) that starts at pos: table indices [b0, b1)
  struct Span { int s, b0, b1, end; };
  auto span_from = [&](int s, int pos) {
    while (__builtin_amdgcn_readfirstlane(cum[s + 1]) <= pos) ++s;
    const int cs = __builtin_amdgcn_readfirstlane(cum[s]);
    const int ce = __builtin_amdgcn_readfirstlane(cum[s + 1]);
    Span r;
    r.s = s;
    r.end = min(ce, hi);
    r.b0 = a.skip_blocks + pos - cs;
    r.b1 = a.skip_blocks + r.end - cs;
    return r;
  };
  auto ids_of = [&](const Span& sp, int base) -> int32_t {
    const int32_t* table = a.block_tables + (int64_t)sp.s * a.max_blocks;
    return (lane < sp.b1 - base) ? table[base + lane] : 0;
  };

  // attend cursor: segment A, next block ab
  Span A = span_from(first, lo);
  int ab = A.b0;
  int end_tok = min(pool_keys<kAppend>(a, A.s), 16 * A.b1);
  bool whole = !kAppend && !a.partial_only && lo == __builtin_amdgcn_readfirstlane(cum[A.s]) &&
               A.end == __builtin_amdgcn_readfirstlane(cum[A.s + 1]);
  // issue cursor: segment I (starts as A), next block ib, its ids idv from ibase;
  // the segment N after I and its first ids
  Span I = A;
  int ib = I.b0, ibase = I.b0;
  int32_t idv = ids_of(I, ibase);
  bool has_n = I.end < hi, i_live = true;
  Span N = I;
  int32_t idv_n = 0;
  if (has_n) {
    N = span_from(I.s + 1, I.end);
    idv_n = ids_of(N, N.b0);
  }
  bool pois_a = false, pois_next = false;
  // segment A's chunk (short-chunk mode): its first q row and row count, whether this
  // lane's column is one of its positions, and that position's causal limit
  int q0A, nqA;
  chunk_of(A.s, q0A, nqA);
  bool col_ok = lane_ok && (!kCols || pc < nqA);
  int col_lim = kCols ? pool_keys<kAppend>(a, A.s) - nqA + pc + 1 : 0;

  u32x4 qb[kChunks];
  auto load_q = [&](int s, int q0) {
    const int64_t qo_row = out_row(s, q0);
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      qb[c] = col_ok ? *(const u32x4*)((const uint16_t*)a.q + qo_row + 32 * c + 8 * g4) : u32x4{0, 0, 0, 0};
  };
  load_q(A.s, q0A);
  f32x4 acc[kDL];
#pragma unroll
  for (int t = 0; t < kDL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  auto block_id = [&](int b) -> int32_t {
    if (b - ibase >= 64) {
      ibase += 64;
      idv = ids_of(I, ibase);
    }
    int32_t id = __builtin_amdgcn_readlane(idv, b - ibase);
    if (!block_ok(id, a.num_blocks)) {
      if (I.s == A.s) pois_a = true; else pois_next = true;
      id = 0;
    }
    return id;
  };
  // issue the pair at the issue cursor, then move the cursor on
  auto issue_next = [&](Tile<D>& t) {
    if (!i_live) return;
    const bool two = ib + 1 < I.b1;
    const int32_t id0 = block_id(ib);
    const int32_t id1 = two ? block_id(ib + 1) : 0;
    load_pair<D, kNT>(t, K, V, id0, id1, two, offs);
    ib += 2;
    if (ib >= I.b1) {
      if (has_n) {
        I = N;
        ib = I.b0;
        ibase = I.b0;
        idv = idv_n;
        has_n = I.end < hi;
        if (has_n) {
          N = span_from(I.s + 1, I.end);
          idv_n = ids_of(N, N.b0);
        }
      } else {
        i_live = false;
      }
    }
  };
  // this wavefront's records, after the prefix sums; written out after the last segment
  constexpr int kWordsFinal = D / 32;             // u32 words per (lane, row group i) of a final
  const int li = n * 4 + g4;                      // record row of this lane (n < C)
  const int final_bytes = 16 + 4 * C * (4 * kWordsFinal * 4);
  const int part_bytes = (16 + 4 * C * (16 * kDL) + 8 * C + 15) & ~15;  // records stay 16-byte aligned
  const int ring_bytes = a.ring_bytes;
  char* ring = (char*)cum + ring_offset(a.num_seqs) + (size_t)(threadIdx.x >> 6) * ring_bytes;
  int used = 0;  // bytes of records (wavefront-uniform)
  auto flush = [&]() {
    int off = 0;
    while (off < used) {
      const char* rec = ring + off;
      const int meta = __builtin_amdgcn_readfirstlane(*(const int*)rec);
      const int rs = meta & 0x7fffffff;
      int rq0 = rs, rnq = 1;  // the chunk's first q row and row count (short-chunk mode)
      if constexpr (kCols) {
        rq0 = __builtin_amdgcn_readfirstlane(((const int*)rec)[1]);
        rnq = __builtin_amdgcn_readfirstlane(((const int*)rec)[2]);
      }
      const bool rok = lane_ok && (!kCols || pc < rnq);
      if (meta < 0) {
        if (rok) {
          const uint32_t* src = (const uint32_t*)(rec + 16) + li * 4 * kWordsFinal;
          uint16_t* O = (uint16_t*)a.out + out_row(rs, rq0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint16_t* dst = O + kDL * (4 * g4 + i);
            if constexpr (D == 128)
              *(u32x4*)dst = *(const u32x4*)(src + 4 * i);
            else
              *(u32x2*)dst = *(const u32x2*)(src + 2 * i);
          }
        }
        off += final_bytes;
      } else {
        if (rok) {
          const f32x4* src = (const f32x4*)(rec + 16) + li * kDL;
#pragma unroll
          for (int d = 0; d < kDL; ++d) acc[d] = src[d];
          const float2 ml = ((const float2*)(rec + 16 + 4 * C * 16 * kDL))[n];
          store_partial<D, kBf16>(a, part_row(rs), acc, ml.x, ml.y, g4);
        }
        off += part_bytes;
      }
    }
    used = 0;
  };
  // attend the pair at the attend cursor; at the end of segment A, record (or store)
  // its result and move A on (returns false after the worker's last segment)
  auto attend_next = [&](Tile<D>& t) -> bool {
    attend_pair<D, kCols>(t, qb, acc, m, lsum, a.scale_log2, min(32, end_tok - 16 * ab), g4, col_lim - 16 * ab);
    ab += 2;
    if (ab < A.b1) return true;
    float l = lsum;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (pois_a) l = __builtin_nanf("");
    {
      // a record while it fits (C <= 16 columns: at most 8,336 bytes), else a direct store
      const int bytes = whole ? final_bytes : part_bytes;
      if (used + bytes > ring_bytes) {
        if (col_ok) {
          if (whole)
            store_final<D>((uint16_t*)a.out, out_row(A.s, q0A), acc, l, g4);
          else
            store_partial<D, kBf16>(a, part_row(A.s), acc, m, l, g4);
        }
      } else {
        char* rec = ring + used;
        if (lane == 0) {
          ((int*)rec)[0] = A.s | (whole ? (int)0x80000000 : 0);
          if constexpr (kCols) {
            ((int*)rec)[1] = q0A;
            ((int*)rec)[2] = nqA;
          }
        }
        if (col_ok) {
          if (whole) {
            // the words store_final would write: row group i holds dims kDL (4 g4 + i) ..
            const float inv = 1.f / l;
            uint32_t* dst = (uint32_t*)(rec + 16) + li * 4 * kWordsFinal;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (D == 128) {
                u32x4 wv;
#pragma unroll
                for (int t2 = 0; t2 < 4; ++t2) wv[t2] = pack_bf16x2(acc[2 * t2][i] * inv, acc[2 * t2 + 1][i] * inv);
                *(u32x4*)(dst + 4 * i) = wv;
              } else {
                u32x2 wv;
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) wv[t2] = pack_bf16x2(acc[2 * t2][i] * inv, acc[2 * t2 + 1][i] * inv);
                *(u32x2*)(dst + 2 * i) = wv;
              }
            }
          } else {
            f32x4* dst = (f32x4*)(rec + 16) + li * kDL;
#pragma unroll
            for (int d = 0; d < kDL; ++d) dst[d] = acc[d];
            if (g4 == 0) ((float2*)(rec + 16 + 4 * C * 16 * kDL))[n] = float2{m, l};
          }
        }
        used += bytes;
      }
    }
    if (A.end >= hi) return false;
    const int pos = A.end;
    A = span_from(A.s + 1, pos);
    ab = A.b0;
    end_tok = min(pool_keys<kAppend>(a, A.s), 16 * A.b1);
    whole = !kAppend && !a.partial_only && pos == __builtin_amdgcn_readfirstlane(cum[A.s]) &&
            A.end == __builtin_amdgcn_readfirstlane(cum[A.s + 1]);
    pois_a = pois_next;
    pois_next = false;
    if constexpr (kCols) {
      chunk_of(A.s, q0A, nqA);
      col_ok = lane_ok && pc < nqA;
      col_lim = pool_keys<kAppend>(a, A.s) - nqA + pc + 1;
    }
    load_q(A.s, q0A);
#pragma unroll
    for (int t2 = 0; t2 < kDL; ++t2) acc[t2] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    lsum = 0.f;
    return true;
  };

  Tile<D> ta, tb;
  issue_next(ta);
  while (true) {
    issue_next(tb);
    if (!attend_next(ta)) break;
    issue_next(ta);
    if (!attend_next(tb)) break;
  }
  flush();
}

// Balanced mode: grid (W, kv-head groups); dynamic LDS holds S+1 ints and, but
// for the lean kernel, each wavefront's staged results (a.ring_bytes).
// kAppend: the pool is read up to each request's newest token and every segment
// leaves a partial, which the merge combines with the newest key.
// kLean: one wavefront per workgroup, segments through decode_segment_lean;
// otherwise each wavefront streams its range through stream_range.
// kCols: short-chunk mode (see DecodeArgs).
template <int D, int NW, bool kAppend, bool kLean, bool kBf16 = false, bool kCols = false>
__device__ __forceinline__ void balanced_body(const DecodeArgs& a) {
  extern __shared__ int32_t cum[];
  __shared__ u32x4 q_lds[kLean ? (D / 32) * 64 : 1];  // the lean segments' query operands
  __shared__ int32_t wave_total[NW];
  constexpr int kThreads = 64 * NW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int S = a.num_seqs;

  // prefix sums of blocks per request: each thread scans a contiguous run
  const int per = (S + kThreads - 1) / kThreads;
  const int r0 = min(tid * per, S), r1 = min(r0 + per, S);
  int mine = 0;
  for (int r = r0; r < r1; ++r) mine += request_blocks<kAppend>(a, r);
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  if (lane == 63) wave_total[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wave; ++i) before += wave_total[i];
  int run = before + incl - mine;
  for (int r = r0; r < r1; ++r) {
    cum[r] = run;
    run += request_blocks<kAppend>(a, r);
  }
  if (tid == kThreads - 1) cum[S] = run;
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int r = tid; r <= S; r += kThreads) a.cum_blocks[r] = cum[r];
    // A request with no key has no segment, and a merge over split requests only
    // does not visit it: its output (NaN, as the merge would give) is written here.
    if (a.merge_splits) {
      for (int r = r0; r < r1; ++r) {
        if (a.context_lens[r] > 0) continue;
        uint16_t* o = (uint16_t*)a.out + (int64_t)r * a.num_q_heads * D;
        for (int e = 0; e < a.num_q_heads * D; ++e) o[e] = 0x7FC0u;  // bf16 quiet NaN
      }
    }
  }

  // Split over W = min(workgroups, T) workers, so that every worker owns at least
  // one block (the merge relies on it); surplus workgroups idle.
  const int64_t T = cum[S];
  const int W = (int)min((int64_t)gridDim.x, T), w = blockIdx.x;
  const bool recorder = blockIdx.y == 0 && tid == 0 && a.split_req != nullptr;
  if (w >= W) {
    if (recorder) a.split_req[w] = -1;
    return;
  }
  const int lo = (int)((int64_t)w * T / W), hi = (int)((int64_t)(w + 1) * T / W);
  const int kvh = blockIdx.y * NW + wave;

  // first request whose blocks reach past lo
  int first = 0, last = S - 1;
  while (first < last) {
    const int mid = (first + last) >> 1;
    if (cum[mid + 1] > lo) last = mid; else first = mid + 1;
  }
  // A request is split when a cut between workers falls inside it; it is recorded
  // by the worker after its first cut only, so the merge can run over the split
  // requests alone (W <= T: every worker's range is non-empty).
  if (recorder)
    a.split_req[w] = (lo > cum[first] && worker_of(cum[first], T, W) == w - 1) ? first : -1;
  if (lo >= hi || kvh >= a.num_kv_heads) return;  // no barrier after this point
  // More attended blocks than the pool holds means blocks are shared (prefix
  // sharing): keep them cacheable. Otherwise stream K/V past the caches.
  const bool nt = a.nontemporal >= 0 ? a.nontemporal != 0 : T <= a.num_blocks;
  if constexpr (!kLean) {
    if (nt)
      stream_range<D, true, kAppend, kBf16, kCols>(a, cum, __builtin_amdgcn_readfirstlane(first), lo, hi, w, kvh);
    else
      stream_range<D, false, kAppend, kBf16, kCols>(a, cum, __builtin_amdgcn_readfirstlane(first), lo, hi, w, kvh);
  } else {
    int s = __builtin_amdgcn_readfirstlane(first);
    int pos = lo;
    while (pos < hi) {
      const int cs = __builtin_amdgcn_readfirstlane(cum[s]);
      const int ce = __builtin_amdgcn_readfirstlane(cum[s + 1]);
      if (ce > pos) {
        const int seg_end = min(ce, hi);
        const int n_keys = pool_keys<kAppend>(a, s);
        const bool whole = !kAppend && !a.partial_only && pos == cs && seg_end == ce;
        const int64_t slot = (int64_t)s + w;
        const int b0 = a.skip_blocks + pos - cs, b1 = a.skip_blocks + seg_end - cs;  // table indices
        if (nt)
          decode_segment_lean<D, true>(a, s, kvh, b0, b1, n_keys, whole, slot * a.num_q_heads, 1, q_lds);
        else
          decode_segment_lean<D, false>(a, s, kvh, b0, b1, n_keys, whole, slot * a.num_q_heads, 1, q_lds);
        pos = seg_end;
      }
      ++s;
    }
  }
}

template <int D, int NW, bool kAppend, bool kBf16 = false>
__global__ __launch_bounds__(64 * NW) void decode_bf16_balanced_kernel(DecodeArgs a) {
  balanced_body<D, NW, kAppend, false, kBf16>(a);
}

// Short-chunk mode: the balanced decode with the columns of a kv head's score tile
// spread over the chunk's positions (pa_prefill_chunk_short).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_bf16_chunk_kernel(DecodeArgs a) {
  balanced_body<D, NW, false, false, false, true>(a);
}

// The lean decode: grid (W, kv heads), one wavefront each, within 96 registers so
// that one fits on every SIMD beside a running prefill workgroup.
template <int D, bool kAppend>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(5))) void decode_bf16_lean_kernel(DecodeArgs a) {
  balanced_body<D, 1, kAppend, true>(a);
}

// (M, den, o) of one fold combined with another's (M2, den2, o2), each relative
// to its own maximum; either may be empty (M = -inf, den = 0, o = 0).
template <int kE>
__device__ __forceinline__ void combine_folds(float& M, float& den, float* o, float M2, float den2,
                                              const float* o2) {
  const float Mn = fmaxf(M, M2);
  if (Mn == -INFINITY) return;  // both empty
  const float w1 = fast_exp2(M - Mn), w2 = fast_exp2(M2 - Mn);
  den = den * w1 + den2 * w2;
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = o[e] * w1 + o2[e] * w2;
  M = Mn;
}

// q heads merged by one workgroup of decode_merge_balanced_kernel (one wavefront
// each): with many short requests the merge is dispatch-bound, so workgroups
// take several heads.
constexpr int kMergeHeads = 8;

// Merge of split-KV partials (m, l, acc) of one (request, q head): partial i is
// row row0 + i * rstep of the workspace. Returns M = max_i m_i (-inf for none),
// o = sum_i 2^(m_i - M) acc_i and den = sum_i 2^(m_i - M) l_i; the caller divides.
// Partials are read eight at a time, all loads of a batch issued before any use,
// and folded into a running (M, den, o) rescaled to the batch maximum.
// kTwo (shared-prefix mode): partials np .. np + np2 - 1 come from a second
// list, rows row2 + i of acc2 / ml2, folded in the same batches as the first
// list's; both lists then hold their accumulators in bf16.
template <int D, bool kTwo = false>
__device__ __forceinline__ void fold_partials(const float* part_acc, const float* part_ml, int64_t row0,
                                              int64_t rstep, int np, int lane, float (&o)[D / 64], float& den,
                                              float& M, const uint16_t* acc2 = nullptr, const float* ml2 = nullptr,
                                              int64_t row2 = 0, int np2 = 0) {
  constexpr int kE = D / 64;
  constexpr int kBatch = 8;
  M = -INFINITY;
  den = 0.f;
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = 0.f;
  const int n = kTwo ? np + np2 : np;
  for (int i0 = 0; i0 < n; i0 += kBatch) {
    float mi[kBatch], li[kBatch], ai[kBatch][kE];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j;
      const bool in = i < n, second = kTwo && i >= np;
      const float* ml = second ? ml2 : part_ml;
      const int64_t r = !in ? row0 : second ? row2 + (i - np) : row0 + (int64_t)i * rstep;
      mi[j] = in ? ml[2 * r] : -INFINITY;
      li[j] = in ? ml[2 * r + 1] : 0.f;
      if constexpr (kTwo) {
        // the row's list is selected by pointer, so no branch holds back the
        // batch's loads
        const uint16_t* src = (second ? acc2 : (const uint16_t*)part_acc) + r * D + kE * lane;
#pragma unroll
        for (int e = 0; e < kE; ++e) ai[j][e] = in ? bf16_bits_to_f32(src[e]) : 0.f;
      } else {
        const float* src = part_acc + r * D + kE * lane;
#pragma unroll
        for (int e = 0; e < kE; ++e) ai[j][e] = in ? src[e] : 0.f;
      }
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, mi[j]);
    const float alpha = fast_exp2(M - mb);  // 0 on the first batch
    den *= alpha;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wgt = fast_exp2(mi[j] - mb);  // 0 for padding
      den += wgt * li[j];
#pragma unroll
      for (int e = 0; e < kE; ++e) o[e] += wgt * ai[j][e];
    }
    M = mb;
  }
}

// Balanced mode merge, one wavefront per (q head, request); lanes own D/64 dims.
// In append mode (kAppend) every request is merged here: its partials (none when
// the newest token is its only one) and its newest key, read from a.new_k /
// a.new_v and attended as one more partial with m = its score, l = 1 and acc =
// its V row. The wavefront of the group's first q head also stores that K/V row
// into the request's slot at position L - 1, after the decode kernel has read
// the pool.
template <int D, bool kAppend>
__global__ __launch_bounds__(64 * kMergeHeads) void decode_merge_balanced_kernel(DecodeArgs a) {
  constexpr int kE = D / 64;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kMergeHeads + (threadIdx.x >> 6);  // one wavefront per q head
  if (h >= a.num_q_heads) return;  // whole wavefront; the kernel has no barrier
  // grid over requests, or (many more requests than workers) over the workers'
  // records of split requests: most requests are then whole and need no merge
  const int s = a.merge_splits ? a.split_req[blockIdx.y] : (int)blockIdx.y;
  if (s < 0) return;
  uint16_t* O = (uint16_t*)a.out;
  const int64_t orow = ((int64_t)s * a.num_q_heads + h) * D + kE * lane;
  // The kernel is a short chain of dependent loads, so it is written without
  // early branches: the request's length, the block prefix sums that locate its
  // partials and, in append mode, the newest token's q, K, V and block id are
  // all requested first (every index is in range whatever their values); the
  // partials follow.
  const int L = min(a.context_lens[s], a.max_context_len);
  const int64_t T = a.cum_blocks[a.num_seqs];
  const int64_t c0 = a.cum_blocks[s], c1 = a.cum_blocks[s + 1];
  const int kvh = h / a.group;
  const int last = max(L - 1, 0);
  float qf[kE];
  uint32_t kb[kE], vb[kE];
  int32_t id = 0;
  if constexpr (kAppend) {
    const int64_t nrow = ((int64_t)s * a.num_kv_heads + kvh) * D + kE * lane;
    const uint16_t* qp = (const uint16_t*)a.q + orow;
    const uint16_t* kp = (const uint16_t*)a.new_k + nrow;
    const uint16_t* vp = (const uint16_t*)a.new_v + nrow;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      qf[e] = bf16_bits_to_f32(qp[e]);
      kb[e] = kp[e];
      vb[e] = vp[e];
    }
    id = a.block_tables[(int64_t)s * a.max_blocks + (last >> 4)];  // last < 16 * max_blocks
  }
  const int64_t Tn = max(T, (int64_t)1);
  const int W = (int)min((int64_t)a.num_workers, Tn);  // as in the decode kernel
  const int w0 = worker_of(c0, Tn, W);
  const int w1 = worker_of(max(c1 - 1, c0), Tn, W);
  const bool has_blocks = c1 > c0;  // false for L <= 0
  if (!kAppend && !a.partial_only && L > 0 && w0 == w1) return;  // one segment: written by the decode kernel
  const int np = has_blocks ? w1 - w0 + 1 : 0;
  // partial of worker w0 + i for this (request, head) is row (s + w0 + i) * Hq + h
  const int64_t row0 = ((int64_t)s + w0) * a.num_q_heads + h;
  float o[kE], den, M;
  if (a.pre_parts > 0)  // shared-prefix mode: the prefix's partials of this (request, head) follow the tail's
    fold_partials<D, true>(a.part_acc, a.part_ml, row0, a.num_q_heads, np, lane, o, den, M, a.pre_acc, a.pre_ml,
                           ((int64_t)s * a.num_q_heads + h) * a.pre_parts, a.pre_parts);
  else
    fold_partials<D>(a.part_acc, a.part_ml, row0, a.num_q_heads, np, lane, o, den, M);
  if constexpr (kAppend) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) part = __builtin_fmaf(qf[e], bf16_bits_to_f32(kb[e]), part);
    const float sn = wave_sum(part) * a.scale_log2;  // the same value in every lane
    const float mb = fmaxf(M, sn);
    const float alpha = fast_exp2(M - mb);  // 0 when there is no partial
    const float wn = fast_exp2(sn - mb);
    den = den * alpha + wn;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[e] = __builtin_fmaf(wn, bf16_bits_to_f32(vb[e]), o[e] * alpha);
    if (!block_ok(id, a.num_blocks)) {
      den = __builtin_nanf("");  // as for any out-of-range block id
    } else if (L > 0 && h % a.group == 0) {
      const int64_t row = kv_row(id, last & 15, kvh, a.num_kv_heads, D) + kE * lane;
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        ((uint16_t*)a.k)[row + e] = (uint16_t)kb[e];
        ((uint16_t*)a.v)[row + e] = (uint16_t)vb[e];
      }
    }
  }
  if (L <= 0) den = __builtin_nanf("");  // no key (in append mode, no newest token): NaN
  const float inv = 1.f / den;
  if constexpr (kE == 2)
    *(uint32_t*)(O + orow) = pack_bf16x2(o[0] * inv, o[1] * inv);
  else
    O[orow] = f32_to_bf16_bits(o[0] * inv);
}

// Short-chunk mode merge, one wavefront per (q head, request, kP positions): the
// partials of (request s, position p, head h) are rows ((s + w) n_cols + p) Hq + h
// for the workers w0 .. w1 that read its blocks; a request read by one worker
// was written by the decode kernel. The wavefront's lanes split into kP groups of
// 64 / kP, one position each, every lane holding D kP / 64 dims, so that a
// wavefront folds kP positions at once: the merge is a short chain of dependent
// loads, and fewer, wider wavefronts wait through fewer rounds of it. Every
// position attends key 0, which the first partial holds, so a fold's first batch
// has a finite maximum.
template <int D, int kP>
__global__ __launch_bounds__(64 * kMergeHeads) void decode_merge_chunk_kernel(DecodeArgs a) {
  constexpr int kLP = 64 / kP;  // lanes per position
  constexpr int kE = D / kLP;   // dims per lane
  constexpr int kBatch = 8;     // partials per round, all loads issued first
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * kMergeHeads + (threadIdx.x >> 6);
  if (h >= a.num_q_heads) return;  // the kernel has no barrier and no cross-lane operation
  const int groups = (a.n_cols + kP - 1) / kP;
  const int s = blockIdx.x / groups;  // grid x: (request, group of kP positions)
  const int pg = (blockIdx.x % groups) * kP;
  const int p = pg + lane / kLP;
  const int dim0 = (lane % kLP) * kE;
  const int q0 = a.query_start_loc[s], nq = a.query_start_loc[s + 1] - q0;
  const int L = min(a.context_lens[s], a.max_context_len);
  const int64_t T = a.cum_blocks[a.num_seqs];
  const int64_t c0 = a.cum_blocks[s], c1 = a.cum_blocks[s + 1];
  if (p >= nq || p >= a.n_cols || L <= 0) return;  // no such position (a chunk with rows has keys)
  const int64_t Tn = max(T, (int64_t)1);
  const int W = (int)min((int64_t)a.num_workers, Tn);  // as in the decode kernel
  const int w0 = worker_of(c0, Tn, W);
  const int w1 = worker_of(max(c1 - 1, c0), Tn, W);
  if (w0 == w1) return;  // one segment: written by the decode kernel
  const int np = w1 - w0 + 1;
  const int64_t rstep = (int64_t)a.n_cols * a.num_q_heads;
  const int64_t row0 = ((int64_t)s + w0) * rstep + (int64_t)p * a.num_q_heads + h;
  float M = -INFINITY, den = 0.f, o[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = 0.f;
  for (int i0 = 0; i0 < np; i0 += kBatch) {
    float mi[kBatch], li[kBatch], ai[kBatch][kE];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = i0 + j < np;
      const int64_t r = row0 + (in ? i0 + j : 0) * rstep;
      mi[j] = in ? a.part_ml[2 * r] : -INFINITY;
      li[j] = in ? a.part_ml[2 * r + 1] : 0.f;
      const float* src = a.part_acc + r * D + dim0;
      if constexpr (kE % 4 == 0) {
#pragma unroll
        for (int v = 0; v < kE / 4; ++v) {
          const f32x4 x = in ? *(const f32x4*)(src + 4 * v) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) ai[j][4 * v + t] = x[t];
        }
      } else {
#pragma unroll
        for (int e = 0; e < kE; ++e) ai[j][e] = in ? src[e] : 0.f;
      }
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, mi[j]);
    const float alpha = fast_exp2(M - mb);  // 0 on the first round
    den *= alpha;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wgt = fast_exp2(mi[j] - mb);  // 0 for padding
      den += wgt * li[j];
#pragma unroll
      for (int e = 0; e < kE; ++e) o[e] += wgt * ai[j][e];
    }
    M = mb;
  }
  const float inv = 1.f / den;
  uint16_t* O = (uint16_t*)a.out + ((int64_t)(q0 + p) * a.num_q_heads + h) * D + dim0;
  if constexpr (kE == 1) {
    *O = f32_to_bf16_bits(o[0] * inv);
  } else if constexpr (kE == 2) {
    *(uint32_t*)O = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else if constexpr (kE == 4) {
    *(u32x2*)O = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
  } else {
    static_assert(kE == 8, "dims per lane");
    *(u32x4*)O = u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                       pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
  }
}

// Short-chunk mode merge for requests split over many workers (more than eight
// partials each on average): one wavefront per (q head, request, position) whose
// four 16-lane groups fold every fourth partial each, so the chain of rounds of
// eight loads is a quarter as long; the groups' results are combined across lanes
// (each lane holds D/16 dims). A group may meet only partials without a key (its
// workers lie past the position's causal limit): its maximum is then taken as 0
// in the exponentials, and it contributes nothing.
template <int D>
__global__ __launch_bounds__(64 * kMergeHeads) void decode_merge_chunk_split_kernel(DecodeArgs a) {
  constexpr int kE = D / 16;   // dims per lane
  constexpr int kBatch = 8;    // partials per group and round, all loads issued first
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, dl = lane & 15;
  const int h = blockIdx.y * kMergeHeads + (threadIdx.x >> 6);
  if (h >= a.num_q_heads) return;  // whole wavefront; the kernel has no barrier
  const int s = blockIdx.x / a.n_cols, p = blockIdx.x % a.n_cols;  // grid x: (request, position)
  const int q0 = a.query_start_loc[s], nq = a.query_start_loc[s + 1] - q0;
  const int L = min(a.context_lens[s], a.max_context_len);
  const int64_t T = a.cum_blocks[a.num_seqs];
  const int64_t c0 = a.cum_blocks[s], c1 = a.cum_blocks[s + 1];
  if (p >= nq || L <= 0) return;  // whole wavefront: no such position
  const int64_t Tn = max(T, (int64_t)1);
  const int W = (int)min((int64_t)a.num_workers, Tn);  // as in the decode kernel
  const int w0 = worker_of(c0, Tn, W);
  const int w1 = worker_of(max(c1 - 1, c0), Tn, W);
  if (w0 == w1) return;  // one segment: written by the decode kernel
  const int np = w1 - w0 + 1;
  const int64_t rstep = (int64_t)a.n_cols * a.num_q_heads;
  const int64_t row0 = ((int64_t)s + w0) * rstep + (int64_t)p * a.num_q_heads + h;
  float M = -INFINITY, den = 0.f, o[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = 0.f;
  for (int i0 = grp; i0 < np; i0 += 4 * kBatch) {
    float mi[kBatch], li[kBatch], ai[kBatch][kE];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + 4 * j;
      const bool in = i < np;
      const int64_t r = row0 + (in ? i : 0) * rstep;
      mi[j] = in ? a.part_ml[2 * r] : -INFINITY;
      li[j] = in ? a.part_ml[2 * r + 1] : 0.f;
      const float* src = a.part_acc + r * D + dl * kE;
#pragma unroll
      for (int v = 0; v < kE / 4; ++v) {
        const f32x4 x = in ? *(const f32x4*)(src + 4 * v) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) ai[j][4 * v + t] = x[t];
      }
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, mi[j]);
    const float mb_use = mb == -INFINITY ? 0.f : mb;
    const float alpha = fast_exp2(M - mb_use);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wgt = fast_exp2(mi[j] - mb_use);  // 0 for padding and empty partials
      den += wgt * li[j];
#pragma unroll
      for (int e = 0; e < kE; ++e) o[e] += wgt * ai[j][e];
    }
    M = mb;
  }
  // combine the four groups: lanes 16 and 32 apart hold the same dims
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const float M2 = __shfl_xor(M, off, 64);
    const float den2 = __shfl_xor(den, off, 64);
    float o2[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) o2[e] = __shfl_xor(o[e], off, 64);
    const float Mn = fmaxf(M, M2);
    const float Mn_use = Mn == -INFINITY ? 0.f : Mn;  // both empty: stay empty
    const float w1 = fast_exp2(M - Mn_use), w2 = fast_exp2(M2 - Mn_use);
    den = den * w1 + den2 * w2;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[e] = o[e] * w1 + o2[e] * w2;
    M = Mn;
  }
  if (grp != 0) return;  // every group holds the result; group 0 stores it
  const float inv = 1.f / den;  // partial 0 holds key 0, which every position attends
  uint16_t* O = (uint16_t*)a.out + ((int64_t)(q0 + p) * a.num_q_heads + h) * D + dl * kE;
  if constexpr (kE == 4) {
    *(u32x2*)O = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
  } else {
    static_assert(kE == 8, "dims per lane");
    *(u32x4*)O = u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                       pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
  }
}

// Balanced mode merge for requests split over many workers (many partials each):
// kWideThreads threads per (q head, request). Groups of D/4 threads own 4 dims
// each; group g folds partials g, g + kG, g + 2 kG, ... (kG = kWideThreads /
// (D/4) groups), so a request split over 256 workers costs one round of loads
// (eight partials per group) instead of one round per eight partials. The group
// results are combined through LDS, and group 0 finishes as
// decode_merge_balanced_kernel does (newest token included in append mode).
// As there, every load that does not depend on another (the request's length
// and block prefix sums, and in append mode the newest token's q, K, V and
// block id) is requested first.
constexpr int kWideThreads = 1024;

template <int D, bool kAppend, bool kBf16Parts = false>
__global__ __launch_bounds__(kWideThreads) void decode_merge_wide_kernel(DecodeArgs a) {
  constexpr int kT = D / 4;              // threads per group, one float4 of dims each
  constexpr int kG = kWideThreads / kT;  // groups
  constexpr int kBatch = 8;              // partials per group and round, all loads issued first
  const int tid = threadIdx.x;
  const int grp = tid / kT, ti = tid % kT;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  uint16_t* O = (uint16_t*)a.out;
  const int64_t orow = ((int64_t)s * a.num_q_heads + h) * D + 4 * ti;
  const int L = min(a.context_lens[s], a.max_context_len);
  const int64_t T = a.cum_blocks[a.num_seqs];
  const int64_t c0 = a.cum_blocks[s], c1 = a.cum_blocks[s + 1];
  const int kvh = h / a.group;
  const int last = max(L - 1, 0);
  u32x2 qw{0, 0}, kw{0, 0}, vw{0, 0};
  int32_t id = 0;
  if constexpr (kAppend) {
    if (grp == 0) {
      const int64_t nrow = ((int64_t)s * a.num_kv_heads + kvh) * D + 4 * ti;
      qw = *(const u32x2*)((const uint16_t*)a.q + orow);
      kw = *(const u32x2*)((const uint16_t*)a.new_k + nrow);
      vw = *(const u32x2*)((const uint16_t*)a.new_v + nrow);
      id = a.block_tables[(int64_t)s * a.max_blocks + (last >> 4)];  // last < 16 * max_blocks
    }
  }
  const int64_t Tn = max(T, (int64_t)1);
  const int W = (int)min((int64_t)a.num_workers, Tn);  // as in the decode kernel
  const int w0 = worker_of(c0, Tn, W);
  const int w1 = worker_of(max(c1 - 1, c0), Tn, W);
  if (!kAppend && !a.partial_only && L > 0 && w0 == w1) return;  // one segment: written by the decode kernel
  const int np = c1 > c0 ? w1 - w0 + 1 : 0;
  const int64_t row0 = ((int64_t)s + w0) * a.num_q_heads + h;
  const int64_t rstep = a.num_q_heads;

  float M = -INFINITY, den = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = grp; i0 < np; i0 += kG * kBatch) {
    float mi[kBatch], li[kBatch];
    f32x4 ai[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j * kG;
      const bool in = i < np;
      const int64_t r = row0 + (int64_t)(in ? i : 0) * rstep;
      mi[j] = in ? a.part_ml[2 * r] : -INFINITY;
      li[j] = in ? a.part_ml[2 * r + 1] : 0.f;
      if constexpr (kBf16Parts) {  // shared-prefix mode: bf16 accumulators
        const u32x2 b = in ? *(const u32x2*)((const uint16_t*)a.part_acc + r * D + 4 * ti) : u32x2{0, 0};
        ai[j] = f32x4{bf16_bits_to_f32(b[0] & 0xffffu), bf16_bits_to_f32(b[0] >> 16),
                      bf16_bits_to_f32(b[1] & 0xffffu), bf16_bits_to_f32(b[1] >> 16)};
      } else {
        ai[j] = in ? *(const f32x4*)(a.part_acc + r * D + 4 * ti) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, mi[j]);
    const float alpha = fast_exp2(M - mb);  // the first partial of the group is real: mb is finite
    den *= alpha;
    o *= alpha;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wgt = fast_exp2(mi[j] - mb);  // 0 for padding
      den += wgt * li[j];
      o += wgt * ai[j];
    }
    M = mb;
  }
  __shared__ float sM[kG], sDen[kG];
  __shared__ f32x4 sO[kG][kT];
  if (ti == 0) {
    sM[grp] = M;
    sDen[grp] = den;
  }
  sO[grp][ti] = o;
  __syncthreads();
  if (grp != 0) return;  // no barrier below
  float Mt = -INFINITY;
#pragma unroll
  for (int g = 0; g < kG; ++g) Mt = fmaxf(Mt, sM[g]);
  den = 0.f;
  o = f32x4{0.f, 0.f, 0.f, 0.f};
  if (Mt > -INFINITY) {  // else no partial at all
#pragma unroll 8
    for (int g = 0; g < kG; ++g) {
      const float wgt = fast_exp2(sM[g] - Mt);  // 0 for groups without a partial
      den += wgt * sDen[g];
      o += wgt * sO[g][ti];
    }
  }
  M = Mt;
  if (a.pre_parts > 0) {  // shared-prefix mode: the prefix's partials of this (request, head)
    const int64_t p0 = ((int64_t)s * a.num_q_heads + h) * a.pre_parts;
    float M2 = -INFINITY, den2 = 0.f;
    f32x4 o2 = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.pre_parts; ++j) {
      const float mj = a.pre_ml[2 * (p0 + j)];
      const float lj = a.pre_ml[2 * (p0 + j) + 1];
      const u32x2 bj = *(const u32x2*)(a.pre_acc + (p0 + j) * D + 4 * ti);  // 4 bf16
      const f32x4 aj = {bf16_bits_to_f32(bj[0] & 0xffffu), bf16_bits_to_f32(bj[0] >> 16),
                        bf16_bits_to_f32(bj[1] & 0xffffu), bf16_bits_to_f32(bj[1] >> 16)};
      const float mb = fmaxf(M2, mj);
      const float alpha = fast_exp2(M2 - mb), wgt = fast_exp2(mj - mb);
      den2 = den2 * alpha + wgt * lj;
      o2 = o2 * alpha + wgt * aj;
      M2 = mb;
    }
    float ov[4] = {o[0], o[1], o[2], o[3]}, ov2[4] = {o2[0], o2[1], o2[2], o2[3]};
    combine_folds<4>(M, den, ov, M2, den2, ov2);
    o = f32x4{ov[0], ov[1], ov[2], ov[3]};
  }
  if constexpr (kAppend) {
    // the newest key as one more partial (m = its score, l = 1, acc = its V row)
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      part = __builtin_fmaf(bf16_bits_to_f32(qw[e] & 0xffffu), bf16_bits_to_f32(kw[e] & 0xffffu), part);
      part = __builtin_fmaf(bf16_bits_to_f32(qw[e] >> 16), bf16_bits_to_f32(kw[e] >> 16), part);
    }
#pragma unroll
    for (int off = kT / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);  // within the group
    const float sn = part * a.scale_log2;
    const float mb = fmaxf(M, sn);
    const float alpha = fast_exp2(M - mb);  // 0 when there is no partial
    const float wn = fast_exp2(sn - mb);
    den = den * alpha + wn;
    const float vv[4] = {bf16_bits_to_f32(vw[0] & 0xffffu), bf16_bits_to_f32(vw[0] >> 16),
                         bf16_bits_to_f32(vw[1] & 0xffffu), bf16_bits_to_f32(vw[1] >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(wn, vv[e], o[e] * alpha);
    if (!block_ok(id, a.num_blocks)) {
      den = __builtin_nanf("");  // as for any out-of-range block id
    } else if (L > 0 && h % a.group == 0) {
      const int64_t row = kv_row(id, last & 15, kvh, a.num_kv_heads, D) + 4 * ti;
      *(u32x2*)((uint16_t*)a.k + row) = kw;
      *(u32x2*)((uint16_t*)a.v + row) = vw;
    }
  }
  if (L <= 0) den = __builtin_nanf("");  // no key (in append mode, no newest token): NaN
  const float inv = 1.f / den;
  *(u32x2*)(O + orow) = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
}

// Fixed-partition mode: grid (partitions, kv-head groups, requests).
template <int D, int NW, bool kNT>
__global__ __launch_bounds__(64 * NW) void decode_bf16_grid_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.y * NW + (threadIdx.x >> 6);
  if (kvh >= a.num_kv_heads) return;  // whole wavefront; the kernel has no barrier
  const int s = blockIdx.z;
  const int part = blockIdx.x;
  const int P = a.partition_tokens;
  const int L = min(a.context_lens[s], a.max_context_len);
  if (L <= 0) {
    const int n = lane & 15, g4 = lane >> 4;
    if (part == 0 && n < a.group) {
      uint16_t* O = (uint16_t*)a.out;
      const int64_t qo_row = ((int64_t)s * a.num_q_heads + kvh * a.group + n) * D;
      for (int i = 0; i < D / 4; ++i) O[qo_row + (D / 4) * g4 + i] = 0x7fc0;
    }
    return;
  }
  const int start = part * P;
  if (start >= L) return;
  const int end = min(start + P, L);
  const int nparts = (L + P - 1) / P;
  decode_segment<D, kNT>(a, s, kvh, start >> 4, (end + 15) >> 4, end, nparts == 1,
                         (int64_t)s * a.num_q_heads * a.max_parts + part, a.max_parts);
}

// fp32 pools, fixed-partition mode: one wavefront per (request, kv head, partition).
template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  constexpr int kE = D / 64;  // dims per lane
  constexpr int kMaxG = 16;
  __shared__ float qs[kMaxG][D];
  __shared__ float ps[kMaxG][64];
  const int lane = threadIdx.x;
  const int kvh = blockIdx.y;
  const int s = blockIdx.z;
  const int part = blockIdx.x;
  const int P = a.partition_tokens;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const float* __restrict__ Q = (const float*)a.q;
  const float* __restrict__ K = (const float*)a.k;
  const float* __restrict__ V = (const float*)a.v;
  float* __restrict__ O = (float*)a.out;
  const int64_t head0 = (int64_t)s * a.num_q_heads + (int64_t)kvh * G;

  const int L = min(a.context_lens[s], a.max_context_len);
  if (L <= 0) {
    if (part == 0)
      for (int g = 0; g < G; ++g)
        for (int e = 0; e < kE; ++e) O[(head0 + g) * D + lane + 64 * e] = __builtin_nanf("");
    return;
  }
  const int start = part * P;
  if (start >= L) return;
  const int end = min(start + P, L);
  const int nparts = (L + P - 1) / P;

  for (int g = 0; g < G; ++g)
    for (int e = 0; e < kE; ++e)
      qs[g][lane + 64 * e] = Q[(head0 + g) * D + lane + 64 * e] * a.scale_log2;
  __syncthreads();

  float acc[kMaxG][kE];
  float m[kMaxG], l[kMaxG];
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[g][e] = 0.f;
  }
  bool poisoned = false;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;

  for (int t0 = start; t0 < end; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < end;
    float sc[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) sc[g] = 0.f;
    if (valid) {
      int32_t id = table_block(table, t);
      if (!block_ok(id, a.num_blocks)) { poisoned = true; id = 0; }
      const float* kr = K + kv_row(id, t & 15, kvh, Hkv, D);
      for (int d = 0; d < D; d += 4) {
        const f32x4 k4 = *(const f32x4*)(kr + d);
#pragma unroll
        for (int g = 0; g < kMaxG; ++g)
          if (g < G)
            sc[g] += qs[g][d] * k4[0] + qs[g][d + 1] * k4[1] + qs[g][d + 2] * k4[2] +
                     qs[g][d + 3] * k4[3];
      }
    }
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
      if (g < G) {
        const float x = valid ? sc[g] : -INFINITY;
        const float m_new = fmaxf(m[g], wave_max(x));
        const float alpha = fast_exp2(m[g] - m_new);
        const float p = valid ? fast_exp2(x - m_new) : 0.f;
        l[g] = l[g] * alpha + wave_sum(p);
        m[g] = m_new;
        ps[g][lane] = p;
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[g][e] *= alpha;
      }
    }
    __syncthreads();
    const int cnt = min(64, end - t0);
    for (int i = 0; i < cnt; ++i) {
      const int tt = t0 + i;
      int32_t id = table_block(table, tt);
      if (!block_ok(id, a.num_blocks)) { poisoned = true; id = 0; }
      const float* vr = V + kv_row(id, tt & 15, kvh, Hkv, D);
      float vv[kE];
#pragma unroll
      for (int e = 0; e < kE; ++e) vv[e] = vr[lane + 64 * e];
#pragma unroll
      for (int g = 0; g < kMaxG; ++g)
        if (g < G)
#pragma unroll
          for (int e = 0; e < kE; ++e) acc[g][e] += ps[g][i] * vv[e];
    }
    __syncthreads();
  }

  poisoned = __any(poisoned);
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) {
    if (g >= G) continue;
    const float lg = poisoned ? __builtin_nanf("") : l[g];
    if (nparts == 1) {
      const float inv = 1.f / lg;
#pragma unroll
      for (int e = 0; e < kE; ++e) O[(head0 + g) * D + lane + 64 * e] = acc[g][e] * inv;
    } else {
      const int64_t pidx = (head0 + g) * a.max_parts + part;
#pragma unroll
      for (int e = 0; e < kE; ++e) a.part_acc[pidx * D + lane + 64 * e] = acc[g][e];
      if (lane == 0) {
        a.part_ml[2 * pidx] = m[g];
        a.part_ml[2 * pidx + 1] = lg;
      }
    }
  }
}

// Fixed-partition merge: one wavefront per (q head, request); lanes own D/64 dims.
template <int D, bool kBf16>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kE = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int L = min(a.context_lens[s], a.max_context_len);
  if (L <= 0) return;
  const int P = a.partition_tokens;
  const int nparts = (L + P - 1) / P;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.max_parts;
  float o[kE], den;
  float M;
  fold_partials<D>(a.part_acc, a.part_ml, base, 1, nparts, lane, o, den, M);
  const float inv = 1.f / den;
  const int64_t orow = ((int64_t)s * a.num_q_heads + h) * D + kE * lane;
  if constexpr (kBf16) {
    uint16_t* O = (uint16_t*)a.out;
    if constexpr (kE == 2)
      *(uint32_t*)(O + orow) = pack_bf16x2(o[0] * inv, o[1] * inv);
    else
      O[orow] = f32_to_bf16_bits(o[0] * inv);
  } else {
    float* O = (float*)a.out;
#pragma unroll
    for (int e = 0; e < kE; ++e) O[orow + e] = o[e] * inv;
  }
}

template <int D, int NW, bool kNT>
void launch_grid(const DecodeArgs& a, hipStream_t stream) {
  const int groups = (a.num_kv_heads + NW - 1) / NW;
  hipLaunchKernelGGL((decode_bf16_grid_kernel<D, NW, kNT>), dim3(a.max_parts, groups, a.num_seqs),
                     dim3(64 * NW), 0, stream, a);
}

// The balanced kernel with a.ring_bytes set: LDS per wavefront for staged segment
// results, from the compute unit's LDS shared by the workgroups that the
// kernel's registers admit there, less the prefix sums (0: direct stores).
// kCols: the short-chunk kernel instead.
template <int D, int NW, bool kAppend, bool kBf16, bool kCols = false>
void launch_balanced(const DecodeArgs& args, hipStream_t stream) {
  constexpr auto kernel = kCols ? decode_bf16_chunk_kernel<D, NW> : decode_bf16_balanced_kernel<D, NW, kAppend, kBf16>;
  static const int64_t lds_per_wg = [] {
    int dev = 0, lds = 65536, wgs = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
      lds = 65536;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&wgs, kernel, 64 * NW, 0) != hipSuccess || wgs < 1)
      wgs = 8;
    (void)hipGetLastError();
    return (int64_t)lds / wgs - 1024;  // slack for static LDS and allocation granules
  }();
  DecodeArgs a = args;
  const int64_t per_wave = (lds_per_wg - (int64_t)ring_offset(a.num_seqs)) / NW;
  a.ring_bytes = (int32_t)(std::max<int64_t>(0, std::min<int64_t>(kRingCapPerWave, per_wave)) & ~(int64_t)15);
  const size_t lds = ring_offset(a.num_seqs) + (size_t)NW * a.ring_bytes;
  const int groups = (a.num_kv_heads + NW - 1) / NW;
  hipLaunchKernelGGL(kernel, dim3(a.num_workers, groups), dim3(64 * NW), lds, stream, a);
}

template <int D, int NW>
void launch_bf16_nw(const DecodeArgs& a, hipStream_t stream) {
  if (a.query_start_loc != nullptr) {
    launch_balanced<D, NW, false, false, true>(a, stream);
  } else if (a.num_workers > 0 && a.lean) {
    const size_t lds = sizeof(int32_t) * (size_t)(a.num_seqs + 1);
    if (a.new_k != nullptr)
      hipLaunchKernelGGL((decode_bf16_lean_kernel<D, true>), dim3(a.num_workers, a.num_kv_heads), dim3(64),
                         lds, stream, a);
    else
      hipLaunchKernelGGL((decode_bf16_lean_kernel<D, false>), dim3(a.num_workers, a.num_kv_heads), dim3(64),
                         lds, stream, a);
  } else if (a.num_workers > 0) {
    if (a.new_k != nullptr)
      launch_balanced<D, NW, true, false>(a, stream);
    else if (a.partial_only)  // shared-prefix mode: bf16 partials
      launch_balanced<D, NW, false, true>(a, stream);
    else
      launch_balanced<D, NW, false, false>(a, stream);
  } else if (a.nontemporal > 0) {
    launch_grid<D, NW, true>(a, stream);
  } else {
    launch_grid<D, NW, false>(a, stream);
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& args, bool bf16, hipStream_t stream) {
  // More requests than workers, every one needing its own merge only when a cut
  // between workers falls inside it (no newest token, no prefix partials): the
  // merge runs over the decode kernel's records of split requests.
  DecodeArgs a = args;
  a.merge_splits = a.num_workers > 0 && a.new_k == nullptr && !a.partial_only && a.pre_parts == 0 &&
                   a.query_start_loc == nullptr && a.num_seqs > a.num_workers;
  if (bf16) {
    switch (decode_waves(a.num_kv_heads)) {
      case 1: launch_bf16_nw<D, 1>(a, stream); break;
      case 2: launch_bf16_nw<D, 2>(a, stream); break;
      case 4: launch_bf16_nw<D, 4>(a, stream); break;
      default: launch_bf16_nw<D, 8>(a, stream); break;
    }
  } else {
    hipLaunchKernelGGL(decode_f32_kernel<D>, dim3(a.max_parts, a.num_kv_heads, a.num_seqs),
                       dim3(64), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid(a.num_q_heads, a.num_seqs);
  if (a.query_start_loc != nullptr && a.num_workers > 8 * a.num_seqs) {
    // requests split over more than eight workers on average: partials folded by four
    // lane groups per wavefront
    hipLaunchKernelGGL((decode_merge_chunk_split_kernel<D>),
                       dim3(a.num_seqs * a.n_cols, (a.num_q_heads + kMergeHeads - 1) / kMergeHeads),
                       dim3(64 * kMergeHeads), 0, stream, a);
  } else if (a.query_start_loc != nullptr) {
    // positions per wavefront: the chunk length's power of two, at most 4
    const int kp = a.n_cols >= 3 ? 4 : a.n_cols;
    const dim3 grid(a.num_seqs * ((a.n_cols + kp - 1) / kp), (a.num_q_heads + kMergeHeads - 1) / kMergeHeads);
    if (kp == 4)
      hipLaunchKernelGGL((decode_merge_chunk_kernel<D, 4>), grid, dim3(64 * kMergeHeads), 0, stream, a);
    else if (kp == 2)
      hipLaunchKernelGGL((decode_merge_chunk_kernel<D, 2>), grid, dim3(64 * kMergeHeads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_chunk_kernel<D, 1>), grid, dim3(64 * kMergeHeads), 0, stream, a);
  } else if (a.num_workers > 0) {
    dim3 hgrid((a.num_q_heads + kMergeHeads - 1) / kMergeHeads, a.merge_splits ? a.num_workers : a.num_seqs);
    // requests split over more than eight workers on average: the wide merge
    const bool wide = a.num_workers > 8 * a.num_seqs;
    if (wide && a.new_k != nullptr)
      hipLaunchKernelGGL((decode_merge_wide_kernel<D, true>), mgrid, dim3(kWideThreads), 0, stream, a);
    else if (wide && a.partial_only)
      hipLaunchKernelGGL((decode_merge_wide_kernel<D, false, true>), mgrid, dim3(kWideThreads), 0, stream, a);
    else if (wide)
      hipLaunchKernelGGL((decode_merge_wide_kernel<D, false>), mgrid, dim3(kWideThreads), 0, stream, a);
    else if (a.new_k != nullptr)
      hipLaunchKernelGGL((decode_merge_balanced_kernel<D, true>), hgrid, dim3(64 * kMergeHeads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_balanced_kernel<D, false>), hgrid, dim3(64 * kMergeHeads), 0, stream, a);
  } else if (a.max_parts > 1) {
    if (bf16)
      hipLaunchKernelGGL((decode_merge_kernel<D, true>), mgrid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_kernel<D, false>), mgrid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

int decode_waves(int num_kv_heads) {
  int nw = num_kv_heads >= 8 ? 8 : num_kv_heads >= 4 ? 4 : num_kv_heads >= 2 ? 2 : 1;
  const char* e = getenv("PA_DECODE_WAVES");  // tuning override: 1, 2, 4 or 8
  if (e != nullptr) {
    const int v = atoi(e);
    if (v == 1 || v == 2 || v == 4 || v == 8) nw = v;
  }
  return nw;
}

int decode_max_balanced_seqs() { return kMaxBalancedSeqs; }

hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (head_dim == 128) return launch_decode_d<128>(a, bf16, stream);
  return launch_decode_d<64>(a, bf16, stream);
}

}  // namespace pa
