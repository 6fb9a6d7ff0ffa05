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
// This is a dense contraction (QK^T and PV), so it runs on bf16 MFMA.
// Workgroup = 4 wavefronts = 128 "packed" query rows of one (request, kv head):
// row r is (position r / G, query head kvh*G + r % G), so all G heads sharing a
// kv head share every K/V tile (grouped-query attention). Keys go in tiles of
// 64 (four 16-token blocks), staged in LDS:
//   Ks [64 keys][D]   row-major; 16-byte chunks XOR-swizzled by row,
//   Vt [D][64 keys]   transposed; each 8-key run is one 16-byte chunk, the
//                     chunks XOR-swizzled by row, keys ordered to match P.
// Staging: wavefronts 0-1 copy K rows (8 x 16 B per lane); wavefronts 2-3 load
// an 8-key x 8-dim patch of V per lane, transpose it in registers and store
// eight 16-byte runs. The next tile is loaded into registers while the current
// one is used, so global latency hides behind the MFMA work.
// Per wavefront (32 rows) and tile, with MFMA 32x32x16 bf16:
//   S^T[32 keys x 32 rows] = K . Q^T for each 32-key half (D/16 MFMAs each;
//     Q^T stays in registers). Lane (col = lane%32, half = lane/32) holds keys
//     8(i/4) + 4 half + i%4 (i = 0..15) of row col, so a row's softmax needs
//     one cross-lane step.
//   O^T[32 dims x 32 rows] += V^T . P^T (4 MFMAs of 16 keys per 32 dims):
//     P^T is the lane's own probabilities (bf16), V^T one 16-byte LDS read.
// fp32 online softmax in log2 units (one FMA and one v_exp_f32 per score), fp32
// accumulation; the running max moves only when a tile exceeds it by 2^8, so the
// output is rescaled rarely (exact: numerator and denominator share the max).
// Only tiles that cross the causal diagonal evaluate the mask.
// Masked scores are set to -inf by selection; keys beyond the context are
// staged as zeros, so no NaN from unused slots can reach the products.
// Workgroups are ordered heaviest (last) query tile first; consecutive
// workgroups take different kv heads of one request, so with 8 kv heads each
// XCD's L2 serves one kv head's K/V to every query tile of that head.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kRows = 128;  // packed query rows per workgroup
constexpr int kBN = 64;     // keys per tile
constexpr int kThreads = 256;

// LDS slot (in 16-byte chunks) of chunk `ch` of K row `row` (kCh chunks per row).
template <int kCh>
__device__ __forceinline__ int k_slot(int row, int ch) {
  if constexpr (kCh == 16) return row * 16 + (ch ^ (row & 15));
  else return row * kCh + (ch ^ ((row >> 1) & (kCh - 1)));
}

// LDS slot of chunk `ch` (keys 8 ch .. 8 ch + 7, permuted) of transposed-V row d.
__device__ __forceinline__ int v_slot(int d, int ch) { return d * 8 + (ch ^ ((d >> 1) & 7)); }

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int kPos = kRows / G;        // query positions per workgroup
  constexpr int kKCh = D / 8;            // 16-byte chunks per key row
  constexpr int kKRowsPerThr = kBN * kKCh / 128;
  constexpr int kKRowStep = 128 / kKCh;  // rows between one K-lane's loads
  constexpr float kRescale = 8.f;        // log2 headroom before the running max is moved
  // two stages of K and transposed V
  __shared__ u32x4 Ks[2][kBN * kKCh];
  __shared__ u32x4 Vt[2][D * 8];

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

  const float c_log2 = a.scale_log2;
  const int row_limit = cached + pos;                // last key this row sees
  const int kv_end = cached + min(pos0 + kPos, nq);  // keys the workgroup needs
  const int first_limit = cached + pos0;             // smallest row limit in the workgroup
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const int nblocks = (L + 15) >> 4;
  const int64_t block_elems = (int64_t)kBlock * Hkv * D;
  const int row_elems = Hkv * D;

  // staging roles (wavefront-uniform): threads 0..127 copy K, 128..255 transpose V
  const bool k_role = tid < 128;
  const int st = tid & 127;
  const int kc = st % kKCh, kr = st / kKCh;  // K: chunk kc of rows kr + kKRowStep j
  // V: dims 8 vd .. 8 vd + 7 of keys 16 vu + 8 (j/4) + 4 vh + j%4 (first D threads)
  const int vd = st % (D / 8), vuh = st / (D / 8), vu = vuh >> 1, vh = vuh & 1;
  const bool v_active = st < D;
  // per-lane element offsets inside a block (kv head kvh), fixed for the whole kernel
  const int k_off = kvh * D + 8 * kc;
  const int v_off = kvh * D + 8 * vd;
  u32x4 stage[8];

  auto stage_load = [&](int t) {
    const int key0 = t * kBN;
    const uint16_t* kbase[kBN / 16];
    const uint16_t* vbase[kBN / 16];
#pragma unroll
    for (int q = 0; q < kBN / 16; ++q) {
      const int blk = (key0 >> 4) + q;
      int32_t id = blk < nblocks ? table[blk] : 0;
      if (!block_ok(id, a.num_blocks)) { poisoned = true; id = 0; }
      kbase[q] = a.k + (int64_t)id * block_elems;
      vbase[q] = a.v + (int64_t)id * block_elems;
    }
    const bool full = key0 + kBN <= L;  // uniform: no key of the tile is past the context
    if (k_role) {
#pragma unroll
      for (int j = 0; j < kKRowsPerThr; ++j) {
        const int row = kr + kKRowStep * j;
        const uint16_t* src = kbase[row >> 4] + (row & 15) * row_elems + k_off;
        stage[j] = (full || key0 + row < L) ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
      }
    } else if (v_active) {
      const uint16_t* vb = vbase[0];
#pragma unroll
      for (int q = 1; q < kBN / 16; ++q) vb = vu == q ? vbase[q] : vb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = 8 * (j >> 2) + 4 * vh + (j & 3);  // token inside block vu
        const uint16_t* src = vb + tok * row_elems + v_off;
        stage[j] = (full || key0 + 16 * vu + tok < L) ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto stage_store = [&](int buf) {
    if (k_role) {
#pragma unroll
      for (int j = 0; j < kKRowsPerThr; ++j) Ks[buf][k_slot<kKCh>(kr + kKRowStep * j, kc)] = stage[j];
    } else if (v_active) {
      // transpose 8 keys x 8 dims: run e holds dim 8 vd + e of the 8 keys
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x4 run;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t lo = stage[2 * u][e >> 1];
          const uint32_t hi = stage[2 * u + 1][e >> 1];
          run[u] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        Vt[buf][v_slot(8 * vd + e, 2 * vu + vh)] = run;
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY;  // running max (log2 units), moved only when exceeded by kRescale
  float lsum = 0.f;

  stage_load(0);
  stage_store(0);
  __syncthreads();
  if (n_tiles > 1) stage_load(1);

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int key0 = t * kBN;
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 ka = Ks[buf][k_slot<kKCh>(32 * kb + col, 2 * c + half)];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qb[c]), sacc[kb], 0, 0, 0);
      }
    }
    // scores are transformed in place: raw -> masked -> probability
    if (key0 + kBN - 1 > first_limit) {  // tile crosses the causal diagonal of some row
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          sacc[kb][i] = key > row_limit ? -INFINITY : sacc[kb][i];
        }
    }
    float tmax = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * c_log2;
    // move the running max (and rescale) only when this tile exceeds it by kRescale:
    // numerator and denominator share the same max, so the result is unchanged
    const bool grow = tmax > m + kRescale;
    if (__any(grow)) {
      const float m_new = grow ? tmax : m;
      const float alpha = fast_exp2(m - m_new);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      m = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(__builtin_fmaf(sacc[kb][i], c_log2, -m));
        sacc[kb][i] = e;
        psum += e;
      }
    lsum += psum;
    u32x4 pb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x16& e = sacc[u >> 1];
      const int b = 8 * (u & 1);
      pb[u] = u32x4{pack_bf16x2(e[b], e[b + 1]), pack_bf16x2(e[b + 2], e[b + 3]),
                    pack_bf16x2(e[b + 4], e[b + 5]), pack_bf16x2(e[b + 6], e[b + 7])};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x4 va = Vt[buf][v_slot(32 * dt + col, 2 * u + half)];
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb[u]), o[dt], 0, 0, 0);
      }
    }
    // tile t+1 goes to the other buffer, last read by tile t-1 (before the previous barrier)
    if (t + 1 < n_tiles) stage_store(buf ^ 1);
    __syncthreads();
    if (t + 2 < n_tiles) stage_load(t + 2);
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
      // o[dt][4 grp + i] is dim 32 dt + 8 grp + 4 half + i
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
