// prefill.hip - causal chunked-prefill attention over a paged KV cache, gfx950.
//
// A request's chunk of n new tokens continues after c = L - n cached tokens: a
// long prompt is split across steps and every step brings the computed count
// closer to the total (arcyou teardown of vLLM paged attention, section
// "Continuous batching: rebuild the batch every step"). Row i of the chunk is
// at absolute position c + i and attends keys 0 .. c + i; keys come from the
// request's block table (same page, section "PagedAttention: the KV cache is
// paged, like virtual memory").
//
// Workgroup = 4 wavefronts = 128 "packed" query rows of one (request, kv head):
// row r is (position r / G, query head kvh*G + r % G), so all G heads that
// share a kv head share every K/V tile (grouped-query attention). Keys are
// processed in tiles of 32 (two 16-token blocks), staged in LDS:
//   Ks  [32 keys][D]  row-major (padded rows),
//   Vt  [D][32 keys]  transposed, key order permuted to match the P layout.
// Per wavefront and tile, with MFMA 32x32x16 bf16:
//   S^T[32 keys x 32 rows] = K . Q^T       (D/16 MFMAs; Q^T stays in registers)
//     lane (col = lane%32, half = lane/32) holds keys 8(r/4) + 4 half + r%4 of
//     row col, r = 0..15, so each row's softmax needs one cross-lane step.
//   O^T[32 d x 32 rows] += V^T . P^T       (2 MFMAs per 32 output d values)
//     P^T is the lane's own 16 probabilities (bf16), split in two k=16 halves;
//     Vt stores key k at position (k with bits 2 and 3 swapped) so each lane's
//     8 keys of an operand are one 16-byte LDS read.
// fp32 online softmax (log2 units, one v_exp_f32 per score), fp32 accumulation.
// Masked scores are set to -inf by selection; keys beyond the context are
// staged as zeros, so no NaN from unused slots can reach the products.
// Workgroups are ordered heaviest (last) query tile first; consecutive
// workgroups take different kv heads of one request, so with 8 kv heads each
// XCD's L2 serves one kv head's K/V to every query tile of that head.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kRows = 128;  // packed query rows per workgroup
constexpr int kBN = 32;     // keys per tile
constexpr int kThreads = 256;

template <int D, int G>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int kPos = kRows / G;       // query positions per workgroup
  constexpr int kKStride = D + 8;       // LDS halfwords per key row
  constexpr int kVStride = kBN + 8;     // LDS halfwords per transposed-V row
  constexpr int kPieces = D / 8;        // 16-byte pieces per key row
  constexpr int kStageIters = kBN * kPieces / kThreads;
  static_assert(kStageIters >= 1 && kBN * kPieces % kThreads == 0, "staging");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * kVStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int Hkv = a.num_kv_heads;
  const int kvh = blockIdx.x % Hkv;
  const int s = blockIdx.x / Hkv;
  const int tile = gridDim.y - 1 - blockIdx.y;

  const int q0 = a.query_start_loc[s];
  int nq = a.query_start_loc[s + 1] - q0;
  int L = a.seq_lens[s];
  nq = min(nq, a.max_query_len);
  nq = min(nq, a.num_tokens - q0);
  L = min(L, a.max_seq_len);
  L = min(L, a.max_blocks * 16);
  const int pos0 = tile * kPos;
  if (q0 < 0 || pos0 >= nq) return;  // uniform over the workgroup
  // A chunk longer than its context is inconsistent: stay in bounds, output NaN.
  bool poisoned = L < nq;
  const int cached = max(L - nq, 0);

  const int col = lane & 31;
  const int half = lane >> 5;
  const int r = wave * 32 + col;
  const int pos = pos0 + r / G;
  const int h = kvh * G + r % G;
  const bool row_ok = pos < nq;
  const int64_t qrow = ((int64_t)(q0 + (row_ok ? pos : 0)) * a.num_q_heads + h) * D;

  u32x4 qb[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qb[c] = row_ok ? *(const u32x4*)(a.q + qrow + 16 * c + 8 * half) : u32x4{0, 0, 0, 0};

  const int row_limit = cached + pos;                   // last key this row sees
  const int kv_end = cached + min(pos0 + kPos, nq);     // keys the workgroup needs
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY;
  float lsum = 0.f;

  for (int key0 = 0; key0 < kv_end; key0 += kBN) {
#pragma unroll
    for (int it = 0; it < kStageIters; ++it) {
      const int idx = tid + kThreads * it;
      const int tok = idx / kPieces;
      const int pc = idx % kPieces;
      const int key = key0 + tok;
      u32x4 kk = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (key < L) {
        int32_t id = table_block(table, key);
        if (!block_ok(id, a.num_blocks)) { poisoned = true; id = 0; }
        const int64_t off = kv_row(id, key & 15, kvh, Hkv, D) + 8 * pc;
        kk = *(const u32x4*)(a.k + off);
        vv = *(const u32x4*)(a.v + off);
      }
      *(u32x4*)&Ks[tok * kKStride + 8 * pc] = kk;
      const int vpos = (tok & ~12) | ((tok & 4) << 1) | ((tok & 8) >> 1);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Vt[(8 * pc + e) * kVStride + vpos] = (uint16_t)(vv[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();

    f32x16 st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4 ka = *(const u32x4*)&Ks[col * kKStride + 16 * c + 8 * half];
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qb[c]), st, 0, 0, 0);
    }
    float sc[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 8 * (i >> 2) + 4 * half + (i & 3);
      float x = st[i] * a.scale_log2;
      x = key > row_limit ? -INFINITY : x;
      sc[i] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - m_new);
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(sc[i] - m_new);
      psum += p[i];
    }
    lsum = lsum * alpha + psum;
    m = m_new;
    const u32x4 pb0 = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                       pack_bf16x2(p[6], p[7])};
    const u32x4 pb1 = {pack_bf16x2(p[8], p[9]), pack_bf16x2(p[10], p[11]),
                       pack_bf16x2(p[12], p[13]), pack_bf16x2(p[14], p[15])};
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint16_t* vrow = &Vt[(32 * dt + col) * kVStride + 8 * half];
      const u32x4 va0 = *(const u32x4*)(vrow);
      const u32x4 va1 = *(const u32x4*)(vrow + 16);
      o[dt] *= alpha;
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va0), as_bf16x8(pb0), o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va1), as_bf16x8(pb1), o[dt], 0, 0, 0);
    }
    __syncthreads();
  }

  poisoned = __syncthreads_or(poisoned);
  lsum += __shfl_xor(lsum, 32, 64);
  if (!row_ok) return;
  const float inv = poisoned ? __builtin_nanf("") : 1.f / lsum;
  uint16_t* orow = a.out + qrow;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      // o[dt][4 grp + i] is d = 32 dt + 8 grp + 4 half + i
      const int i0 = 4 * grp;
      u32x2 w = {pack_bf16x2(o[dt][i0] * inv, o[dt][i0 + 1] * inv),
                 pack_bf16x2(o[dt][i0 + 2] * inv, o[dt][i0 + 3] * inv)};
      *(u32x2*)(orow + 32 * dt + 8 * grp + 4 * half) = w;
    }
  }
}

template <int D, int G>
hipError_t launch_dg(const PrefillArgs& a, hipStream_t stream) {
  constexpr int kPos = kRows / G;
  dim3 grid(a.num_seqs * a.num_kv_heads, (a.max_query_len + kPos - 1) / kPos);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_dg<D, 1>(a, stream);
    case 2: return launch_dg<D, 2>(a, stream);
    case 4: return launch_dg<D, 4>(a, stream);
    case 8: return launch_dg<D, 8>(a, stream);
    case 16: return launch_dg<D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, hipStream_t stream) {
  if (head_dim == 128) return launch_d<128>(a, group, stream);
  return launch_d<64>(a, group, stream);
}

}  // namespace pa
