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
// Workgroup = 8 wavefronts = 256 "packed" query rows of one (request, kv head):
// row r is (position r / G, query head kvh*G + r % G), so all G heads sharing a
// kv head share every K/V tile (grouped-query attention). Keys go in tiles of
// 64 (four 16-token blocks), staged in double-buffered LDS, K and V both
// row-major [64 keys][D] with their 16-byte chunks XOR-swizzled by row (no bank
// conflicts for either operand read). Wavefronts 0-3 stage K and 4-7 stage V,
// one block each, with direct global-to-LDS loads (global_load_lds_dwordx4: each
// instruction fills 1 KiB of LDS, lane l's 16 bytes at offset 16 l, so the
// swizzle is applied on the source side). Tile t + 2 is loaded into the stage
// tile t has just released, right after the barrier that ends tile t, and lands
// while tile t + 1 is computed (one barrier per tile).
// Per wavefront (32 rows) and tile, with MFMA 32x32x16 bf16:
//   S^T[32 keys x 32 rows] = K . Q^T for each 32-key half (D/16 MFMAs each;
//     Q^T stays in registers; K operands are read four chunks ahead). Lane
//     (col = lane%32, half = lane/32) holds keys 8(i/4) + 4 half + i%4
//     (i = 0..15) of row col, so a row's softmax needs one cross-lane step.
//   O^T[32 dims x 32 rows] += V^T . P^T (4 MFMAs of 16 keys per 32 dims):
//     P^T is the lane's own probabilities (bf16); V^T comes from two
//     transposed 8-byte LDS reads (ds_read_b64_tr_b16) whose key order matches
//     P, read four products ahead.
// fp32 online softmax in log2 units (one FMA and one v_exp_f32 per score), fp32
// accumulation; the running max moves only when a tile exceeds it by 2^8, so the
// output is rescaled rarely (exact: numerator and denominator share the max).
// Only tiles that cross the causal diagonal evaluate the mask.
// Masked scores are set to -inf by selection. Rows past the context are not
// loaded: the stage keeps the finite rows of two tiles before (or the zeros it
// starts with), so no NaN from unused pool slots can reach the products, and
// their probabilities are exactly zero.
// The tile loop is unrolled by two, so the LDS stage of every operand read is an
// immediate offset.
// Append mode (pa_prefill_chunk_append): the chunk's own keys and values are
// staged from the caller's new K/V rows instead of the pool (a block that holds
// both cached and new tokens is read in two masked passes), and each workgroup
// stores the new rows of its own query positions and kv head into the pool
// through the block table. No workgroup reads a new token's slot, so the stores
// need no ordering against the reads; the rows are loaded before the first
// tiles and stored after the first barrier.
// Work items (request, kv head, query tile) run request by request, the
// heaviest request first and its query tiles heaviest first: workgroup i of the
// dispatch order takes the item of rank i (see item_of_rank). Consecutive
// workgroups take the kv heads of one (request, tile) in turn, so with 8 kv
// heads each XCD (which receives every 8th workgroup) serves one kv head's K/V
// from its L2, and the query tiles of one request start together and read the
// same keys at about the same time.
#include <type_traits>

#include "pa_device.h"

namespace pa {
namespace {

constexpr int kWaves = 8;             // wavefronts per workgroup, 32 query rows each
constexpr int kRows = 32 * kWaves;    // packed query rows per workgroup
constexpr int kBN = 64;               // keys per tile
constexpr int kThreads = 64 * kWaves;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposed 8-byte LDS read. Reached through a restrict pointer, the read
// carries an alias scope, so the compiler does not hold it behind the
// direct-to-LDS loads of the other stage still in flight (the kernel orders
// those itself: a wait and a barrier before any stage is read).
__device__ __forceinline__ v4i16 lds_read_tr(const lds_v4i16* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// Physical 16-byte chunk of logical chunk `ch` in row `row` of a staged tile.
// K rows: the row's low 4 bits (16-lane K reads hit 16 distinct chunks).
// V rows: a transposed read by 32 lanes covers 4 consecutive keys x 32 dims,
// i.e. 4 logical chunks of 4 rows; the XOR spreads those 16 pieces over 16
// distinct bank groups (D = 128: rows are 256 B, one full pass over the 64
// banks, so the XOR takes 4 x (row & 3); D = 64: rows are 128 B and alternate
// bank halves, so rows 2 apart are told apart by 4 x ((row >> 1) & 1)).
template <int kCh>
__device__ __forceinline__ int k_phys(int row, int ch) {
  if constexpr (kCh == 16) return ch ^ (row & 15);
  else return ch ^ ((row >> 1) & 7);
}
template <int kCh>
__device__ __forceinline__ int v_phys(int row, int ch) {
  if constexpr (kCh == 16) return ch ^ (4 * (row & 3));
  else return ch ^ (4 * ((row >> 1) & 1));
}

// Work items are (request, kv head, query tile); an item's cost is the number
// of 64-key tiles it reads, ceil((cached + min((tile + 1) kPos, nq)) / 64), and a
// request's level is the cost of its heaviest tile, ceil((cached + nq) / 64).
// Items run request by request, in non-increasing level (ties by request
// index); within a request, query tiles from the last (heaviest) to the first,
// the kv heads of each tile in turn. Grouping by request keeps the K/V of few
// requests in flight on each XCD's L2 at once: ordering single items heaviest
// first interleaves every request's tiles over the whole launch, and tiles of
// one (request, kv head) that start far apart in time re-read its K/V from
// beyond the L2. Ordering requests by level keeps the longest-first balance.
// Each workgroup finds its item itself from the requests' lengths: a binary
// search on the level c with count(c) = items of requests of level >= c.
struct ReqShape {
  int nq, cached, tiles;  // rows of the chunk, cached keys, query tiles (0: no work)
};

__device__ __forceinline__ ReqShape req_shape(const PrefillArgs& a, int r, int kPos) {
  ReqShape q{0, 0, 0};
  const int q0 = a.query_start_loc[r];
  int nq = a.query_start_loc[r + 1] - q0;
  int L = a.seq_lens[r];
  nq = min(nq, a.max_query_len);
  nq = min(nq, a.num_tokens - q0);
  L = min(L, a.max_seq_len);
  L = min(L, a.max_blocks * 16);
  if (q0 < 0 || nq <= 0) return q;
  q.nq = nq;
  q.cached = max(L - nq, 0);
  q.tiles = (nq + kPos - 1) / kPos;
  return q;
}

// Level of a request with work: the cost of its heaviest (last) query tile.
__device__ __forceinline__ int req_level(const ReqShape& q) { return (q.cached + q.nq + 63) / 64; }

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Items of requests of level >= c (one wavefront, lanes over requests).
__device__ int64_t items_level_ge(const PrefillArgs& a, int c, int kPos, int lane) {
  int64_t acc = 0;
  for (int r = lane; r < a.num_seqs; r += 64) {
    const ReqShape q = req_shape(a, r, kPos);
    if (q.tiles > 0 && req_level(q) >= c) acc += (int64_t)a.num_kv_heads * q.tiles;
  }
  return wave_sum_i64(acc);
}

// The item of rank `rank` in the order above, as (request, kv head, tile), or
// request -1 when rank >= the number of items. Run by one whole wavefront;
// every lane gets the result.
__device__ void item_of_rank(const PrefillArgs& a, int64_t rank, int kPos, int lane, int out[3]) {
  out[0] = -1;
  out[1] = out[2] = 0;
  if (items_level_ge(a, 1, kPos, lane) <= rank) return;
  // a level is at most ceil(max(L, nq) / 64) over the clamped lengths
  int lo = 1, hi = (max(a.max_seq_len, a.max_query_len) + 63) / 64 + 1;  // count(lo) > rank >= count(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (items_level_ge(a, mid, kPos, lane) > rank) lo = mid;
    else hi = mid;
  }
  const int c = lo;
  const int64_t j = rank - items_level_ge(a, c + 1, kPos, lane);  // rank among requests of level c
  int64_t acc = 0;
  for (int base = 0; base < a.num_seqs; base += 64) {
    const int r = base + lane;
    int64_t n = 0;
    int tiles = 0;
    if (r < a.num_seqs) {
      const ReqShape q = req_shape(a, r, kPos);
      tiles = q.tiles;
      if (q.tiles > 0 && req_level(q) == c) n = (int64_t)a.num_kv_heads * q.tiles;
    }
    int64_t incl = n;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    const uint64_t hit = __ballot(r < a.num_seqs && j < acc + incl);
    if (hit != 0) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int64_t off = j - (acc + incl - n);  // meaningful on lane src
      out[0] = __shfl(r, src, 64);
      out[1] = __shfl((int)(off % a.num_kv_heads), src, 64);
      out[2] = __shfl(tiles - 1 - (int)(off / a.num_kv_heads), src, 64);
      return;
    }
    acc += __shfl(incl, 63, 64);
  }
}

template <int D, int G, bool kCross, bool kAppend>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(!(kCross && kAppend), "append mode is for causal chunks");
  constexpr int kPos = kRows / G;            // query positions per workgroup
  constexpr int kCh = D / 8;                 // 16-byte chunks per key row
  constexpr int kTileCh = kBN * kCh;         // chunks per staged tile of K (or V)
  constexpr int kInstr = 2 * kTileCh / kThreads;  // 16-byte pieces per lane and tile
  constexpr float kRescale = 8.f;            // log2 headroom before the running max is moved
  static_assert(kInstr * kThreads == 2 * kTileCh && (kInstr * 64) % kCh == 0, "staging");
  // two stages of K and V, both row-major [64 keys][D]
  __shared__ u32x4 Ks[2][kTileCh];
  __shared__ u32x4 Vs[2][kTileCh];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hkv = a.num_kv_heads;
  // the workgroup's (request, kv head, query tile) and, in shared-prefix mode,
  // its range [k_lo, L) of prefix keys
  int s, kvh, tile, q0, nq, L, k_lo = 0;
  bool poisoned = false;
  if constexpr (kCross) {
    // Shared-prefix mode: the rows are the decode queries of the num_seqs requests
    // (one position each), and every row attends keys [k_lo, L) of the prefix that
    // all requests share, read through block table row 0, with no causal mask.
    s = 0;
    kvh = blockIdx.x % Hkv;
    tile = blockIdx.x / Hkv;
    q0 = 0;
    nq = a.num_seqs;
    k_lo = blockIdx.y * a.key_chunk;
    L = min(k_lo + a.key_chunk, a.prefix_keys);
    if (tile * kPos >= nq || k_lo >= L) return;  // uniform over the workgroup
  } else {
    __shared__ int item[3];  // this workgroup's (request, kv head, query tile)
    if (wave == 0) {
      int mine[3];
      item_of_rank(a, blockIdx.x + (int64_t)gridDim.x * blockIdx.y, kPos, lane, mine);
      if (lane == 0) {
        item[0] = mine[0];
        item[1] = mine[1];
        item[2] = mine[2];
      }
    }
    __syncthreads();
    s = item[0];
    if (s < 0) return;  // uniform: more workgroups than items
    kvh = item[1];
    tile = item[2];
    q0 = a.query_start_loc[s];
    nq = a.query_start_loc[s + 1] - q0;
    L = a.seq_lens[s];
    nq = min(nq, a.max_query_len);
    nq = min(nq, a.num_tokens - q0);
    L = min(L, a.max_seq_len);
    L = min(L, a.max_blocks * 16);
    if (q0 < 0 || tile * kPos >= nq) return;  // uniform over the workgroup
    // A chunk longer than its context is inconsistent: stay in bounds, output NaN.
    poisoned = L < nq;
  }
  const int pos0 = tile * kPos;
  const int cached = kCross ? 0 : max(L - nq, 0);

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
  // last key this row sees, keys the workgroup needs, smallest row limit in it
  const int row_limit = kCross ? L - 1 : cached + pos;
  const int kv_end = kCross ? L : cached + min(pos0 + kPos, nq);
  const int first_limit = kCross ? L - 1 : cached + pos0;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int t0 = k_lo / kBN;  // first tile (k_lo is a multiple of kBN)
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const int nblocks = (L + 15) >> 4;
  const int64_t block_elems = (int64_t)kBlock * Hkv * D;
  const int row_elems = Hkv * D;

  // Staging: wavefronts 0-3 copy K, 4-7 copy V; wavefront w takes block w % 4 of
  // the tile. Piece i of lane l is LDS chunk slot ((w%4)*kInstr + i)*64 + l, i.e.
  // row slot/kCh, physical chunk slot%kCh, which holds logical chunk
  // k_phys/v_phys(row, physical): each piece is one direct global-to-LDS load.
  const int sblk = wave & 3;          // block of the tile this wavefront copies
  const bool s_is_v = wave >= 4;      // wavefront-uniform
  int src_off[kInstr];                // element offsets inside a block (tile-independent)
#pragma unroll
  for (int i = 0; i < kInstr; ++i) {
    const int slot = (sblk * kInstr + i) * 64 + lane;
    const int row = slot / kCh;
    const int ch = s_is_v ? v_phys<kCh>(row, slot % kCh) : k_phys<kCh>(row, slot % kCh);
    src_off[i] = (row & 15) * row_elems + kvh * D + 8 * ch;
  }
  // block ids this wavefront copies, 64 tiles at a time: lane j holds tile id_tile0 + j
  int id_tile0 = t0;
  auto fetch_ids = [&]() {
    const int blk = 4 * (id_tile0 + lane) + sblk;
    return blk < nblocks ? table[blk] : 0;
  };
  int32_t idv = fetch_ids();
  typedef __attribute__((address_space(3))) void lds_void;
  auto stage_load = [&](int t, int buf) {
    const int key0 = t * kBN;
    if (t - id_tile0 >= 64) {  // tiles are staged in order
      id_tile0 += 64;
      idv = fetch_ids();
    }
    int32_t id = __builtin_amdgcn_readlane(idv, t - id_tile0);
    if (!block_ok(id, a.num_blocks)) { poisoned = true; id = 0; }
    const uint16_t* src = (s_is_v ? a.v : a.k) + (int64_t)id * block_elems;
    u32x4* dst = s_is_v ? &Vs[buf][0] : &Ks[buf][0];
    const int kb = key0 + 16 * sblk;  // first key of this wavefront's block
    const bool full = kb + 16 <= L;   // uniform: the whole block is in range
    // append mode: keys >= cached are the chunk's own, in the input rows
    // q0 + key - cached (the same [Hkv][D] layout as a pool row)
    // (the base of those rows is formed only for lanes that read them)
    const bool has_new = kAppend && kb + 16 > cached;  // uniform
    const uint16_t* nbase = nullptr;
    if constexpr (kAppend) nbase = (s_is_v ? a.new_v : a.new_k) + (int64_t)(q0 + kb - cached) * row_elems;
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      // row of the tile, and key of the block (kb + (row & 15) = kb + 64 i / kCh + lane / kCh)
      const int row = ((sblk * kInstr + i) * 64 + lane) / kCh;
      const bool in_range = full || key0 + row < L;  // past the context: not loaded
      lds_void* to = (lds_void*)&dst[(sblk * kInstr + i) * 64];
      if (!has_new) {
        if (in_range) __builtin_amdgcn_global_load_lds((const void*)(src + src_off[i]), to, 16, 0, 0);
      } else {
        // a block holding both cached and new tokens is read in two masked passes
        const bool from_new = (lane / kCh) >= cached - kb - (64 * i) / kCh;
        if (in_range && !from_new) __builtin_amdgcn_global_load_lds((const void*)(src + src_off[i]), to, 16, 0, 0);
        if (in_range && from_new) __builtin_amdgcn_global_load_lds((const void*)(nbase + src_off[i]), to, 16, 0, 0);
      }
    }
  };

  // Append mode: this workgroup's share of the chunk's new rows (positions pos0 ..
  // pos0 + kPos - 1, kv head kvh, K then V), 16 bytes a piece, kStore pieces per
  // thread and round. The first round is loaded here and stored after the first
  // barrier; further rounds (G <= 2) are copied there in turn.
  constexpr int kPieces = kAppend ? 2 * kPos * kCh : 0;
  constexpr int kStore = 4;
  u32x4 cp[kStore];
  int64_t cp_dst[kStore];  // 2 x (16-byte piece index in the pool tensor) + tensor, or -1
  auto copy_load = [&](int round) {
#pragma unroll
    for (int j = 0; j < kStore; ++j) {
      const int piece = (round * kStore + j) * kThreads + tid;
      const int v = piece >= kPos * kCh;  // 0: K, 1: V
      const int rem = piece - v * kPos * kCh;
      const int p = pos0 + rem / kCh, ch = rem % kCh;
      cp_dst[j] = -1;
      if (piece < kPieces && p < nq && cached + p < L) {
        int32_t id = table[(cached + p) >> 4];
        if (block_ok(id, a.num_blocks)) {
          const int64_t row = kv_row(id, (cached + p) & 15, kvh, Hkv, D) + 8 * ch;
          const uint16_t* srcp = (v ? a.new_v : a.new_k) + ((int64_t)(q0 + p) * Hkv + kvh) * D + 8 * ch;
          cp[j] = *(const u32x4*)srcp;
          cp_dst[j] = (row >> 3) * 2 + v;
        }
      }
    }
  };
  auto copy_store = [&]() {
#pragma unroll
    for (int j = 0; j < kStore; ++j) {
      if (cp_dst[j] < 0) continue;
      uint16_t* pool = const_cast<uint16_t*>((cp_dst[j] & 1) ? a.v : a.k);
      *(u32x4*)(pool + (cp_dst[j] >> 1) * 8) = cp[j];
    }
  };
  if constexpr (kAppend) copy_load(0);

  // Per-lane LDS byte addresses of the MFMA operands in stage 0 (stage 1 is +kTileCh*16).
  //   K (A of S^T): row 32 kb + col, logical chunk 2c + half  -> one per c, kb by offset
  //   V (A of O^T, transposed read): lane (i = lane%16, group g = lane/16) supplies row
  //   16u + 8rr + 4 half + i/4 and dims 32 dt + 16 (g&1) + 4 (i%4)   -> one per dt
  uint32_t k_addr[D / 16], v_addr[D / 32];
  const uint32_t ks0 = (uint32_t)(uintptr_t)&Ks[0][0], vs0 = (uint32_t)(uintptr_t)&Vs[0][0];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) k_addr[c] = ks0 + 16u * (col * kCh + k_phys<kCh>(col, 2 * c + half));
  {
    const int i = lane & 15, g = lane >> 4;
    const int vrow = 4 * half + (i >> 2);  // + 16u + 8rr, which leave row & 3 unchanged
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int dim = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
      v_addr[dt] = vs0 + 16u * (vrow * kCh + v_phys<kCh>(vrow, dim >> 3)) + 2u * (dim & 7);
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY;  // running max (log2 units), moved only when exceeded by kRescale
  float lsum = 0.f;

  // the stages start as zeros (rows past the context are never loaded)
  for (int i = tid; i < 2 * kTileCh; i += kThreads) {
    (&Ks[0][0])[i] = u32x4{0, 0, 0, 0};
    (&Vs[0][0])[i] = u32x4{0, 0, 0, 0};
  }
  __syncthreads();
  stage_load(t0, 0);
  if (t0 + 1 < n_tiles) stage_load(t0 + 1, 1);
  // both tiles landed (a partial count would not do: rows past the context skip
  // their loads) and are visible to every wavefront
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (kAppend) {
    copy_store();
#pragma unroll 1
    for (int round = 1; round * kStore * kThreads < kPieces; ++round) {
      copy_load(round);
      copy_store();
    }
  }

  // one tile; the LDS stage is a compile-time constant so that operand
  // addresses take it as an immediate offset
  auto tile_step = [&](int t, auto stage) __attribute__((always_inline)) {
    constexpr int buf = decltype(stage)::value;
    const int key0 = t * kBN;
    constexpr uint32_t koff = buf * kTileCh * 16u, voff = buf * kTileCh * 16u;
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
    {
      typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
      // K operands run kAhead chunks ahead of the MFMAs that use them, so LDS
      // latency hides behind the MFMAs of the chunks in between
      constexpr int kAhead = 4;
      u32x4 ka[kAhead][2];
#pragma unroll
      for (int c = 0; c < kAhead; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ka[c][kb] = *(lds_u32x4*)(uintptr_t)(k_addr[c] + koff + kb * 32 * kCh * 16);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMAs
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[c % kAhead][kb]), as_bf16x8(qb[c]),
                                                             sacc[kb], 0, 0, 0);
        if (c + kAhead < D / 16) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            ka[c % kAhead][kb] = *(lds_u32x4*)(uintptr_t)(k_addr[c + kAhead] + koff + kb * 32 * kCh * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // scores are transformed in place: raw -> masked -> probability
    if (key0 + kBN - 1 > first_limit) {  // tile crosses the causal diagonal (or the end)
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
    {
      // V^T operands (two transposed reads each) run kAhead products ahead of
      // their MFMAs. Product j is (u = j / (D/32), dt = j % (D/32)); its operand
      // holds keys 16u + 4 half + 0..3 and 16u + 8 + 4 half + 0..3.
      constexpr int kProducts = 4 * (D / 32);
      constexpr int kAhead = 4;
      v4i16 vlo[kAhead], vhi[kAhead];
      auto vread = [&](int j, int r) {
        const uint32_t base = v_addr[j % (D / 32)] + voff + (j / (D / 32)) * 16 * kCh * 16;
        vlo[r] = lds_read_tr((const lds_v4i16*)(uintptr_t)base);
        vhi[r] = lds_read_tr((const lds_v4i16*)(uintptr_t)(base + 8 * kCh * 16));
      };
#pragma unroll
      for (int j = 0; j < kAhead; ++j) vread(j, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kProducts; ++j) {
        const bf16x8 va =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[j % kAhead], vhi[j % kAhead], 0, 1, 2, 3, 4, 5, 6, 7));
        const int dt = j % (D / 32), u = j / (D / 32);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16x8(pb[u]), o[dt], 0, 0, 0);
        if (j + kAhead < kProducts) vread(j + kAhead, j % kAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // tile t+1 (this wavefront's loads, issued a tile ago) has landed; after the
    // barrier every wavefront's has, and tile t's stage is free for tile t+2
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < n_tiles) stage_load(t + 2, buf);
  };
  for (int t = t0; t < n_tiles; t += 2) {
    tile_step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_tiles) tile_step(t + 1, std::integral_constant<int, 1>{});
  }

  poisoned = __syncthreads_or(poisoned);
  lsum += __shfl_xor(lsum, 32, 64);
  if (!row_ok) return;
  if constexpr (kCross) {
    // partial (m, l, acc) of row (request pos, q head h) over key range blockIdx.y
    const int64_t pidx = ((int64_t)pos * a.num_q_heads + h) * a.key_splits + blockIdx.y;
    uint16_t* dst = a.part_acc + pidx * D;  // acc in bf16 (not divided by l)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)  // o[dt][4 grp + i] is dim 32 dt + 8 grp + 4 half + i
        *(u32x2*)(dst + 32 * dt + 8 * grp + 4 * half) =
            u32x2{pack_bf16x2(o[dt][4 * grp], o[dt][4 * grp + 1]), pack_bf16x2(o[dt][4 * grp + 2], o[dt][4 * grp + 3])};
    if (half == 0) {
      a.part_ml[2 * pidx] = m;
      a.part_ml[2 * pidx + 1] = poisoned ? __builtin_nanf("") : lsum;
    }
    return;
  }
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

template <int D, int G, bool kCross>
hipError_t launch_dg(const PrefillArgs& a, hipStream_t stream) {
  constexpr int kPos = kRows / G;
  if constexpr (kCross) {
    // (query tile, kv head) pairs along x, key ranges along y
    dim3 grid(a.num_kv_heads * ((a.num_seqs + kPos - 1) / kPos), a.key_splits);
    hipLaunchKernelGGL((prefill_bf16_kernel<D, G, true, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    dim3 grid(a.num_seqs * a.num_kv_heads, (a.max_query_len + kPos - 1) / kPos);
    if (a.new_k != nullptr)
      hipLaunchKernelGGL((prefill_bf16_kernel<D, G, false, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<D, G, false, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, bool kCross>
hipError_t launch_d(const PrefillArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_dg<D, 1, kCross>(a, stream);
    case 2: return launch_dg<D, 2, kCross>(a, stream);
    case 4: return launch_dg<D, 4, kCross>(a, stream);
    case 8: return launch_dg<D, 8, kCross>(a, stream);
    case 16: return launch_dg<D, 16, kCross>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, hipStream_t stream) {
  if (head_dim == 128) return launch_d<128, false>(a, group, stream);
  return launch_d<64, false>(a, group, stream);
}

hipError_t launch_prefix_attention(const PrefillArgs& a, int head_dim, int group, hipStream_t stream) {
  if (head_dim == 128) return launch_d<128, true>(a, group, stream);
  return launch_d<64, true>(a, group, stream);
}

}  // namespace pa
