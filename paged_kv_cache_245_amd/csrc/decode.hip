// decode.hip - paged decode attention for gfx950: one query per request at its
// last position, over every token of its logical context, read through the
// request's block table (arcyou teardown of vLLM paged attention, section
// "PagedAttention: the KV cache is paged, like virtual memory"; every new token
// re-reads all past K/V: kenhuang vLLM course, "PagedAttention (intuition)").
//
// Work split. A request's context is cut into partitions of P keys (a multiple
// of 16). One wavefront owns one (request, kv head, partition) and keeps a
// running softmax over it: max m, sum of exponentials l and the unnormalised
// output acc (the usual online-softmax recurrence). A request that fits in one
// partition is finished in place; otherwise each partition stores (m, l, acc)
// and decode_merge_kernel combines them: out = sum(2^(m_p-M) acc_p) /
// sum(2^(m_p-M) l_p), M = max m_p. Scores are kept in log2 units (the scale is
// pre-multiplied by log2 e) so every exponential is one v_exp_f32.
//
// bf16 kernel, per wavefront and per pair of 16-token blocks (32 keys):
//   S^T[16 keys x 16 heads] = K[16 x D] . Q^T[D x 16]   (D/32 MFMA 16x16x32 per block)
//     A operand = K rows: lane (n = lane%16, g4 = lane/16) loads 16 B of key n's
//     row at d = 32c + 8 g4; a block of one kv head is 16 rows of 2*D bytes.
//     B operand = the group's G query heads in columns 0..G-1 (columns >= G are 0).
//     Result: lane holds the scores of head n for keys 4 g4 .. 4 g4 + 3.
//   O^T[16 d x 16 heads] += V^T[16 d x 32 keys] . P^T[32 keys x 16 heads]
//     (D/16 MFMA 16x16x32, one per 16 output d values)
//     B operand = the lane's own 8 probabilities (4 keys of each block), so the
//     softmax output needs no cross-lane movement; the k index of the product
//     is mapped to those 8 keys. A operand = the same 8 keys of V: the lane
//     loads D/16 consecutive d values of each of the 8 rows (one 16-byte load
//     per row for D=128) and transposes the 8 x (D/16) tile in registers.
//     Output lane (n, g4) owns head n, d = (D/4) g4 .. (D/4) g4 + D/4 - 1.
//   The probabilities are rounded to bf16 for the PV product; the running sum
//   l uses the fp32 values.
// K/V loads are 16 B per lane; for each row all its bytes are requested by the
// same instruction group, so each 16-token block is fetched as 16 fully used
// 2*D-byte segments. Block ids are wavefront-uniform scalar loads.
//
// fp32 kernel: a plain VALU kernel (lanes over keys for q.k, lanes over d for
// PV) with the same partition / merge scheme, for fp32 pools.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kDecodeWaves = 4;  // kv heads per workgroup in the bf16 kernel

template <int D>
struct VRowT;
template <>
struct VRowT<128> { typedef u32x4 type; };
template <>
struct VRowT<64> { typedef u32x2 type; };

template <int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_bf16_kernel(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int kChunks = D / 32;  // MFMA k-chunks of q.k
  constexpr int kDL = D / 16;      // d values per lane per V row == PV tiles
  typedef typename VRowT<D>::type VRow;

  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.y * kDecodeWaves + (threadIdx.x >> 6);
  if (kvh >= a.num_kv_heads) return;  // whole wavefront; the kernel has no barrier
  const int s = blockIdx.z;
  const int part = blockIdx.x;
  const int P = a.partition_tokens;
  const int G = a.group;
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int h = kvh * G + n;
  const bool head_ok = n < G;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v;
  uint16_t* __restrict__ O = (uint16_t*)a.out;
  const int64_t qo_row = ((int64_t)s * a.num_q_heads + h) * D;

  int L = a.context_lens[s];
  L = min(L, a.max_context_len);
  if (L <= 0) {
    if (part == 0 && head_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < kDL; ++t) O[qo_row + kDL * (4 * g4 + i) + t] = 0x7fc0;
    }
    return;
  }
  const int start = part * P;
  if (start >= L) return;
  const int end = min(start + P, L);
  const int nparts = (L + P - 1) / P;

  u32x4 qb[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    qb[c] = head_ok ? *(const u32x4*)(Q + qo_row + 32 * c + 8 * g4) : u32x4{0, 0, 0, 0};

  f32x4 acc[kDL];
#pragma unroll
  for (int t = 0; t < kDL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;
  bool poisoned = false;

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const int Hkv = a.num_kv_heads;
  const int row_stride = Hkv * D;  // elements between consecutive tokens of a block
  const int b_end = (end + 15) >> 4;

  for (int b = start >> 4; b < b_end; b += 2) {
    const bool two = b + 1 < b_end;
    int32_t id0 = table_block(table, b * 16);
    int32_t id1 = two ? table_block(table, (b + 1) * 16) : 0;
    if (!block_ok(id0, a.num_blocks)) { poisoned = true; id0 = 0; }
    if (!block_ok(id1, a.num_blocks)) { poisoned = true; id1 = 0; }

    const uint16_t* k0 = K + kv_row(id0, n, kvh, Hkv, D) + 8 * g4;
    const uint16_t* k1 = K + kv_row(id1, n, kvh, Hkv, D) + 8 * g4;
    const uint16_t* v0 = V + kv_row(id0, 4 * g4, kvh, Hkv, D) + kDL * n;
    const uint16_t* v1 = V + kv_row(id1, 4 * g4, kvh, Hkv, D) + kDL * n;
    u32x4 ka0[kChunks], ka1[kChunks];
    VRow vr[8];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) ka0[c] = *(const u32x4*)(k0 + 32 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) vr[j] = *(const VRow*)(v0 + j * row_stride);
    if (two) {
#pragma unroll
      for (int c = 0; c < kChunks; ++c) ka1[c] = *(const u32x4*)(k1 + 32 * c);
#pragma unroll
      for (int j = 0; j < 4; ++j) vr[4 + j] = *(const VRow*)(v1 + j * row_stride);
    } else {
#pragma unroll
      for (int c = 0; c < kChunks; ++c) ka1[c] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) vr[4 + j] = VRow{};
    }

    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka0[c]), as_bf16x8(qb[c]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka1[c]), as_bf16x8(qb[c]), s1, 0, 0, 0);
    }
    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = s0[i] * a.scale_log2;
      sc[4 + i] = s1[i] * a.scale_log2;
    }
    if ((b + 2) * 16 > end) {  // keys past the partition end: score -inf, V row 0
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = (b + (j >> 2)) * 16 + 4 * g4 + (j & 3);
        if (key >= end) {
          sc[j] = -INFINITY;
          vr[j] = VRow{};
        }
      }
    }
    float tmax = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - m_new);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(sc[j] - m_new);
      psum += p[j];
    }
    lsum = lsum * alpha + psum;
    m = m_new;
    const u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
#pragma unroll
    for (int t = 0; t < kDL; ++t) {
      u32x4 va;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t lo = vr[2 * u][t >> 1];
        const uint32_t hi = vr[2 * u + 1][t >> 1];
        va[u] = (t & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      acc[t] *= alpha;
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pb), acc[t], 0, 0, 0);
    }
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (poisoned) lsum = __builtin_nanf("");
  if (!head_ok) return;
  // lane (n, g4), acc[t][i] is head h at d = kDL * (4 g4 + i) + t
  if (nparts == 1) {
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
  } else {
    const int64_t pidx = ((int64_t)s * a.num_q_heads + h) * a.max_parts + part;
    float* dst = a.part_acc + pidx * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int t4 = 0; t4 < kDL; t4 += 4) {
        *(f32x4*)(dst + kDL * (4 * g4 + i) + t4) =
            f32x4{acc[t4][i], acc[t4 + 1][i], acc[t4 + 2][i], acc[t4 + 3][i]};
      }
    }
    if (g4 == 0) {
      a.part_ml[2 * pidx] = m;
      a.part_ml[2 * pidx + 1] = lsum;
    }
  }
}

// fp32 pools: one wavefront per (request, kv head, partition); G <= 16 query heads.
template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  constexpr int kE = D / 64;  // d values per lane
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

  int L = a.context_lens[s];
  L = min(L, a.max_context_len);
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

// Combine the partitions of every request longer than one partition.
// One wavefront per (query head, request); lanes own D/64 consecutive d values.
template <int D, bool kBf16>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kE = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int L = a.context_lens[s];
  L = min(L, a.max_context_len);
  if (L <= 0) return;
  const int P = a.partition_tokens;
  const int nparts = (L + P - 1) / P;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.max_parts;
  const float* ml = a.part_ml + 2 * base;
  const float* pacc = a.part_acc + base * D;

  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);
  float den = 0.f;
  for (int p = lane; p < nparts; p += 64) den += fast_exp2(ml[2 * p] - M) * ml[2 * p + 1];
  den = wave_sum(den);

  float o[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(ml[2 * p] - M);
    const float* src = pacc + (int64_t)p * D + kE * lane;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[e] += w * src[e];
  }
  const float inv = 1.f / den;
  const int64_t orow = ((int64_t)s * a.num_q_heads + h) * D + kE * lane;
  if constexpr (kBf16) {
    uint16_t* O = (uint16_t*)a.out;
    if constexpr (kE == 2) {
      *(uint32_t*)(O + orow) = pack_bf16x2(o[0] * inv, o[1] * inv);
    } else {
      O[orow] = f32_to_bf16_bits(o[0] * inv);
    }
  } else {
    float* O = (float*)a.out;
#pragma unroll
    for (int e = 0; e < kE; ++e) O[orow + e] = o[e] * inv;
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) {
    dim3 grid(a.max_parts, (a.num_kv_heads + kDecodeWaves - 1) / kDecodeWaves, a.num_seqs);
    hipLaunchKernelGGL(decode_bf16_kernel<D>, grid, dim3(64 * kDecodeWaves), 0, stream, a);
  } else {
    dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL(decode_f32_kernel<D>, grid, dim3(64), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  dim3 mgrid(a.num_q_heads, a.num_seqs);
  if (bf16)
    hipLaunchKernelGGL((decode_merge_kernel<D, true>), mgrid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, false>), mgrid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (head_dim == 128) return launch_decode_d<128>(a, bf16, stream);
  return launch_decode_d<64>(a, bf16, stream);
}

}  // namespace pa
