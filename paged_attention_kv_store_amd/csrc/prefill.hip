// Chunked-prefill attention over a paged KV cache (bf16, head_dim 128).
//
// A chunk is L query rows of one sequence that follow P0 = ctx - L tokens
// already in the cache; the chunk's own K/V rows are stored too, so its keys
// are positions 0 .. ctx-1. Row i (position P0 + i) sees keys 0 .. P0 + i
// when causal, else all ctx keys.
//
// Work unit: one workgroup of 4 wavefronts per (q-tile, kv-head, chunk). The
// G q-heads that share the kv-head are packed with the query rows into the
// matrix rows ("M rows": m = query_row * G + head), so a workgroup covers
// 128 M rows = 128/G query rows and each K/V byte staged in LDS serves all G
// heads. Wave w owns two 16-row tiles of M rows: tile t holds rows
// 16(w + 4t) .. 16(w + 4t) + 15, so the rows of a short chunk (a few query
// rows) spread over the waves instead of filling the first wave's tiles.
//
// The keys are walked in 64-token tiles gathered through the block table
// straight into LDS with direct-to-LDS loads (double-buffered: the next
// tile's loads are in flight while the current one is consumed), 16-byte
// pieces XOR-swizzled by row, with one swizzle for K and another for V, each
// chosen (by measurement on gfx950) so that its read pattern below is free
// of bank conflicts. Per 16 keys:
//  * S^T = K Q^T on 16x16x32 bf16 MFMA (A = 16 K rows from LDS, B = the
//    wave's Q rows kept in registers) gives each lane the scores of keys
//    4*(l/16)+r for M row l%16;
//  * causal / context mask, online softmax in fp32 (log2 domain, lazy
//    rescaling), P rounded to bf16;
//  * O += P V on 16x16x32 bf16 MFMA over 32 keys at a time: the scores of
//    two 16-key tiles are already laid out as the A operand (8 keys per
//    lane); the B operand (the same 8 keys of one column per lane) comes
//    from two transposing LDS reads (ds_read_b64_tr_b16), which hand each
//    lane four key rows of one column from the row-major V tile. Output
//    column block c of the accumulator holds columns 16c .. 16c+15.
//
// E4M3 caches (FP8 = true): the same kernel with a register-staged gather:
// each lane fetches 16 codes of a row, and once they have landed converts
// them exactly to bf16 (every E4M3 value is a bf16 value) and writes them
// into the same swizzled bf16 LDS tile, so the matrix work is unchanged. The
// kv-head's K scale is folded into the logit multiplier and its V scale into
// the final normalisation.
#include "common.h"
#include "device_utils.h"

#include <type_traits>

namespace pkv {

namespace {

constexpr int kD = 128;               // head_dim
constexpr int kPW = 4;                // waves per workgroup
constexpr int kPThreads = 64 * kPW;
constexpr int kMRows = 32 * kPW;      // M rows per workgroup
constexpr int kKvTile = 64;           // keys per LDS tile
constexpr int kRowPieces = kD * 2 / 16;   // 16-byte pieces per K/V row (16)
constexpr int kXcds = 8;              // accelerator complex dies, each with its own L2
// Raw byte-addressed buffer descriptors for the whole-tile gather: the
// record count never limits a load (offsets stay below 16 pool rows), and
// the last word is the plain-buffer configuration of this GPU family.
constexpr int kBufferRecords = 0x7fffffff;
constexpr int kBufferConfig = 0x00020000;

// LDS position (in 16-byte units) of piece c of key row t in a tile: piece
// c ^ sk(t) for K, c ^ sv(t) for V, where sk(t) = t mod 16 and sv(t) =
// 2 (t mod 8) + bit 3 of t. A transposing read of V takes 32 bytes (two
// pieces 2c', 2c'+1) from each of 8 rows per half-wave: sv / 2 = t mod 8
// puts those 8 rows on 8 different bank groups.
__device__ __forceinline__ int k_swizzle(int t) { return t & 15; }
__device__ __forceinline__ int v_swizzle(int t) { return ((t & 7) << 1) | ((t >> 3) & 1); }
__device__ __forceinline__ int swz_k(int t, int c) { return t * kRowPieces + (c ^ k_swizzle(t)); }
__device__ __forceinline__ int swz_v(int t, int c) { return t * kRowPieces + (c ^ v_swizzle(t)); }

// Rank of an item's cost: 1 + its 64-key tiles (0 for a q-tile past the end
// of its chunk), capped at kOrderBuckets - 1.
constexpr int kOrderBuckets = 4096;
constexpr int kOrderMaxItems = 8192;   // (chunk, q-tile) items ranked in LDS

template <int BQ>
__device__ __forceinline__ int item_cost(const PrefillParams& p, int j) {
  const int c = j / p.num_q_tiles, qt = j % p.num_q_tiles;
  const int q_start = min(max(p.cu_seqlens_q[c], 0), p.total_q);
  const int L = min(max(p.cu_seqlens_q[c + 1], q_start), p.total_q) - q_start;
  const int r0 = qt * BQ;
  if (r0 >= L) return 0;
  const int ctx = min(max(p.context_lens[c], 0), p.max_ctx);
  const int kv_end = p.causal ? min(ctx, max(ctx - L, 0) + min(r0 + BQ, L)) : ctx;
  return min(1 + (kv_end + kKvTile - 1) / kKvTile, kOrderBuckets - 1);
}

}  // namespace

template <int G, bool FP8>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams p) {
  constexpr int BQ = kMRows / G;      // query rows per workgroup
  __shared__ uint4 s_k[2][kKvTile * kRowPieces];
  __shared__ uint4 s_v[2][kKvTile * kRowPieces];
  __shared__ int s_bad;

  // Work item of this workgroup. Workgroups are handed to the 8 XCDs round
  // robin (id % 8), each XCD with its own L2, and start in id order as
  // earlier ones finish.
  //  * Longest first (the usual case): id = rank * kv_heads + kv-head, where
  //    rank orders the (chunk, q-tile) items by their key tiles, most first,
  //    so the long items start at once and the short ones fill the tail.
  //    With 8 kv-heads every XCD serves one kv-head, all its items in that
  //    order, and the q-tiles of a chunk share the XCD's L2.
  //  * Otherwise (too many items to rank in LDS): item i = x * (items/8) +
  //    id/8 for x = id % 8 gives every XCD a contiguous range of items, the
  //    kv-head slowest and the q-tiles of a chunk adjacent, the q-tiles with
  //    more keys first.
  const int nqt = p.num_q_tiles;
  const int tid = threadIdx.x;
  int qt, c, g;
  if (p.longest_first) {
    // Two workgroups share a compute unit, id b and id b + C on C units:
    // ids C .. 2C-1 take the first round's ranks in reverse, so that each
    // unit pairs a costly item with a cheaper one.
    int b = blockIdx.x;
    if (p.pair_span > 0 && b >= p.pair_span && b < 2 * p.pair_span) b = 3 * p.pair_span - 1 - b;
    g = b % p.num_kv_heads;
    // (chunk, q-tile) item j = chunk * num_q_tiles + q-tile
    const int j = item_of_rank<kPThreads, kOrderBuckets>(
        b / p.num_kv_heads, nqt * p.num_seqs, [&](int i) { return item_cost<BQ>(p, i); },
        reinterpret_cast<int*>(s_v[1]), reinterpret_cast<uint16_t*>(s_k[1]));
    if (j < 0) return;
    c = j / nqt;
    qt = j % nqt;
  } else {
    const int per_xcd = gridDim.x / kXcds;
    const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (item >= nqt * p.num_seqs * p.num_kv_heads) return;
    qt = nqt - 1 - item % nqt;
    c = (item / nqt) % p.num_seqs;
    g = item / (nqt * p.num_seqs);
  }
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, qg = lane >> 4;

  const int q_start = min(max(p.cu_seqlens_q[c], 0), p.total_q);
  const int q_end = min(max(p.cu_seqlens_q[c + 1], q_start), p.total_q);
  const int L = q_end - q_start;
  const int r0 = qt * BQ;
  if (r0 >= L) return;
  const int ctx = min(max(p.context_lens[c], 0), p.max_ctx);
  const int P0 = max(ctx - L, 0);
  const int r_last = min(r0 + BQ, L) - 1;                 // last query row of the tile
  const int kv_end = p.causal ? min(ctx, P0 + r_last + 1) : ctx;
  const int n_kv = (kv_end + kKvTile - 1) / kKvTile;
  const int64_t row_elems = (int64_t)p.num_kv_heads * kD;
  const int bs = p.block_size;
  const int32_t* bt = p.block_tables + (int64_t)(p.table_row_is_first_q ? q_start : c) * p.max_blocks;
  // A negative scale is applied as |scale| to negated q (exact in bf16), so
  // the scale is > 0 below and the row max of raw scores gives the max of
  // scaled ones. A zero scale is taken as the smallest normal float: every
  // weight 2^(FLT_MIN * x - m) then rounds to exactly what scale 0 gives,
  // and a masked -inf score still yields weight 0 rather than NaN.
  // (E4M3: the multiplier includes the kv-head's K scale; a NaN one stays
  // NaN, as the dequantised definition gives NaN rows then.)
  const float eff = FP8 ? p.scale_log2 * p.k_scale[g] : p.scale_log2;
  const float scale = (eff != eff) ? eff : fmaxf(fabsf(eff), __FLT_MIN__);
  const uint32_t qsign = eff < 0.f ? 0x80008000u : 0u;

  // ---- the wave's Q rows (B operand of S^T = K Q^T) ----------------------
  // tile t, lane l: M row mr = 16(w + 4t) + l%16 (query row r0 + mr/G, head
  // mr%G); step s holds head_dim elements [32s + 8qg, 32s + 8qg + 8).
  bf16x8_t qf[2][4];
  int qpos[2];          // absolute position of the lane's softmax row
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mr = 16 * (w + kPW * t) + n;
    const int qi = r0 + mr / G;
    qpos[t] = P0 + qi;
    const bool live = qi < L;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)(q_start + qi) * p.num_q_heads + g * G + mr % G) * kD + 8 * qg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (live) v = load16(qrow + 32 * s);
      v.x ^= qsign;
      v.y ^= qsign;
      v.z ^= qsign;
      v.w ^= qsign;
      qf[t][s] = bit_cast_to<bf16x8_t>(v);
    }
  }

  // ---- cooperative K/V tile gather, global memory straight into LDS -------
  // A direct-to-LDS load puts lane j's 16 bytes at (wave's LDS base) + 16j.
  // Load i of wave w fills LDS rows 16i + 4w .. +3 of the tile, so lane j
  // fetches key row t = 16i + 4w + j/16, piece (j%16) ^ sk(t) of K and
  // (j%16) ^ sv(t) of V: the swizzled layout comes out of the choice of
  // source addresses. Rows 16i .. 16i+15 of
  // a tile lie in one block (block_size is a power of two >= 16), so a tile
  // needs four block ids, all workgroup-uniform, scalar-loaded a tile ahead.
  // Rows past the context are read from the last live row instead (finite
  // values; their weight is zero), so no NaN from a dead row reaches P.V.
  const int lbs = p.block_size_log2;
  const int64_t row_bytes = row_elems * 2;
  const int lrow = 4 * w + (lane >> 4);          // tile row of load 0, minus 16i
  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + g * kD * 2;
  const char* vbase = reinterpret_cast<const char*>(p.v_cache) + g * kD * 2;
  bool bad = false;
  auto tile_blocks = [&](int kt, int (&ids)[4]) {
    const int kv0 = min(kt, max(n_kv - 1, 0)) * kKvTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) ids[i] = bt[min(kv0 + 16 * i, max(ctx - 1, 0)) >> lbs];
  };
  // Within a tile the swizzle of row 16i + lrow depends only on lrow, so a
  // lane's byte offset from the start of its block row is the same for every
  // load of every whole tile (32 bits: 15 rows of a pool row plus 256 bytes).
  const uint32_t koff_lane = (uint32_t)lrow * (uint32_t)row_bytes + ((lane & 15) ^ k_swizzle(lrow)) * 16;
  const uint32_t voff_lane = (uint32_t)lrow * (uint32_t)row_bytes + ((lane & 15) ^ v_swizzle(lrow)) * 16;
  auto gather = [&](int kt, int buf, const int (&ids)[4]) {
    const int kv0 = kt * kKvTile;
    if (kv0 + kKvTile <= ctx) {
      // whole tile: each load's block row is workgroup-uniform, so its
      // address is a scalar base plus the lane's constant offset
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int blk = __builtin_amdgcn_readfirstlane(ids[i]);
        if ((unsigned)blk >= (unsigned)p.num_blocks) {
          blk = 0;
          bad = true;
        }
        // pool rows fit 32 bits (checked on the host)
        const uint32_t row = ((uint32_t)blk << lbs) + (uint32_t)((kv0 + 16 * i) & (bs - 1));
        const uint64_t off = (uint64_t)row * (uint64_t)(uint32_t)row_bytes;
        const int lds_pos = (16 * i + 4 * w) * kRowPieces;
        // buffer descriptors based at the block row: the lane's offset is
        // the 32-bit vector offset, nothing is added per lane
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(kbase + off), (short)0, kBufferRecords, kBufferConfig);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(vbase + off), (short)0, kBufferRecords, kBufferConfig);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (void __attribute__((address_space(3)))*)(&s_k[buf][lds_pos]), 16, koff_lane, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (void __attribute__((address_space(3)))*)(&s_v[buf][lds_pos]), 16, voff_lane, 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int blk = ids[i];
      if ((unsigned)blk >= (unsigned)p.num_blocks) {
        blk = 0;
        bad = true;
      }
      const int t = 16 * i + lrow;
      const int pos = min(kv0 + t, ctx - 1);
      // pool rows fit 32 bits (checked on the host): one 32 x 32 -> 64-bit multiply
      const uint32_t row = ((uint32_t)blk << lbs) + (uint32_t)(pos & (bs - 1));
      const uint64_t off = (uint64_t)row * (uint64_t)(uint32_t)row_bytes;
      const int lds_pos = (16 * i + 4 * w) * kRowPieces;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(kbase + off + ((lane & 15) ^ k_swizzle(t)) * 16),
          (void __attribute__((address_space(3)))*)(&s_k[buf][lds_pos]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(vbase + off + ((lane & 15) ^ v_swizzle(t)) * 16),
          (void __attribute__((address_space(3)))*)(&s_v[buf][lds_pos]), 16, 0, 0);
    }
  };
  // E4M3 caches: wave w fetches rows 16w .. 16w+15 of a tile (one block);
  // lane l of slot i takes codes 16c .. 16c+15 (c = l % 8) of row
  // t = 16w + 8i + l/8 into registers, and once they have landed writes
  // them as bf16 pieces 2c and 2c+1 of row t at their swizzled places.
  const char* kbase8 = reinterpret_cast<const char*>(p.k_cache) + g * kD;
  const char* vbase8 = reinterpret_cast<const char*>(p.v_cache) + g * kD;
  uint4 st_k[2], st_v[2];
  auto gather8 = [&](int kt, const int (&ids)[4]) {
    const int kv0 = kt * kKvTile;
    int blk = w == 0 ? ids[0] : w == 1 ? ids[1] : w == 2 ? ids[2] : ids[3];
    if ((unsigned)blk >= (unsigned)p.num_blocks) {
      blk = 0;
      bad = true;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 16 * w + 8 * i + (lane >> 3);
      const int pos = min(kv0 + t, ctx - 1);
      const int64_t off = (((int64_t)blk << lbs) + (pos & (bs - 1))) * row_elems + (lane & 7) * 16;
      st_k[i] = load16(kbase8 + off);
      st_v[i] = load16(vbase8 + off);
    }
  };
  auto store8 = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 16 * w + 8 * i + (lane >> 3);
      const int c = 2 * (lane & 7);
      const uint2 k0 = e4m3x4_to_bf16(st_k[i].x), k1 = e4m3x4_to_bf16(st_k[i].y);
      const uint2 k2 = e4m3x4_to_bf16(st_k[i].z), k3 = e4m3x4_to_bf16(st_k[i].w);
      s_k[buf][swz_k(t, c)] = make_uint4(k0.x, k0.y, k1.x, k1.y);
      s_k[buf][swz_k(t, c + 1)] = make_uint4(k2.x, k2.y, k3.x, k3.y);
      const uint2 v0 = e4m3x4_to_bf16(st_v[i].x), v1 = e4m3x4_to_bf16(st_v[i].y);
      const uint2 v2 = e4m3x4_to_bf16(st_v[i].z), v3 = e4m3x4_to_bf16(st_v[i].w);
      s_v[buf][swz_v(t, c)] = make_uint4(v0.x, v0.y, v1.x, v1.y);
      s_v[buf][swz_v(t, c + 1)] = make_uint4(v2.x, v2.y, v3.x, v3.y);
    }
  };
  // all of this thread's loads (direct-to-LDS or staged) have landed (vmcnt 0)
  auto wait_loads = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };

  float m_ref[2] = {neg_inf(), neg_inf()};   // per softmax row (lane's n), scaled units
  float nm_ref[2] = {0.f, 0.f};               // -m_ref, or 0 while the row has seen no key
  f32x4_t acc[2][8];                          // acc[t][c][r] = O[row 4qg + r of tile t][16c + n]
  f32x4_t lsum[2];                            // lsum[t][r]   = sum of P over row 4qg + r of tile t
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    lsum[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // bf16 ones: P times a ones column gives the row sums of the rounded weights
  bf16x8_t ones = bit_cast_to<bf16x8_t>(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  // keys below this bound are visible to every row of the wave
  const int lim_wave = p.causal ? min(P0 + r0 + (16 * w) / G + 1, ctx) : ctx;
  // Whether M-row tile t of the wave holds a live query row (wave-uniform).
  // Short chunks (a few query rows, as in verifying drafted tokens) leave
  // most tiles empty; their matrix work is skipped, while the wave still
  // takes its share of the cooperative gather and every barrier.
  const bool live0 = r0 + (16 * w) / G < L;
  const bool live1 = r0 + (16 * (w + kPW)) / G < L;

  // byte offset, within key row kb + n / 4 of a V tile, of the 8-byte piece
  // lane n reads for column block c: columns 16c + 4(n % 4), i.e. half n % 2
  // of 16-byte piece 2c + (n % 4) / 2, at its swizzled place (the row's
  // swizzle depends on the row mod 16 = 4qg + n / 4 for both reads)
  int vtr_off[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    vtr_off[c] = (((2 * c + ((n & 3) >> 1)) ^ v_swizzle(4 * qg + (n >> 2))) * 16) + (n & 1) * 8;
  if (tid == 0) s_bad = 0;
  int ids_next[4], ids_after[4];
  if (n_kv > 0) {
    int ids0[4];
    tile_blocks(0, ids0);
    tile_blocks(1, ids_next);
    if constexpr (FP8) gather8(0, ids0);
    else gather(0, 0, ids0);
  }
  wait_loads();
  if (FP8 && n_kv > 0) store8(0);
  __syncthreads();

  // The tile loop runs two tiles per trip, one per LDS buffer, so that each
  // copy of the body knows its buffer at compile time and the buffer offset
  // folds into the LDS instructions' immediate fields.
  auto tile_step = [&](int kt, auto buf_tag) {
    constexpr int buf = decltype(buf_tag)::value;
    const bool more = kt + 1 < n_kv;
    tile_blocks(kt + 2, ids_after);
    // the other buffer was last read before the previous barrier
    if (more) {
      if constexpr (FP8) gather8(kt + 1, ids_next);
      else gather(kt + 1, buf ^ 1, ids_next);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) ids_next[i] = ids_after[i];
    const int kv0 = kt * kKvTile;
    // an empty asm that claims to modify the ones operand keeps its four
    // registers resident; otherwise the compiler rebuilds the tuple with
    // three moves before every row-sum step
    asm volatile("" : "+v"(ones));
    const uint4* sk = s_k[buf];
    const uint4* sv = s_v[buf];

#pragma unroll
    for (int sub = 0; sub < kKvTile / 32; ++sub) {
      const int tb = 32 * sub;              // first key of the 32-key block, tile-relative
      if (kv0 + tb >= kv_end || !live0) break;
      // Slot u = 0..7 of a lane stands for key tb + 16*(u/4) + 4qg + u%4: the
      // keys of two 16-key score tiles, in the order their scores arrive.
      // K rows tb + 16h + n, pieces 4s + qg (elements 32s + 8qg .. +8)
      bf16x8_t kf[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[h][s] = bit_cast_to<bf16x8_t>(sk[swz_k(tb + 16 * h + n, 4 * s + qg)]);
      // B operands of P.V by transposing LDS reads, issued here so that their
      // latency overlaps the softmax below
      const char* vrow = reinterpret_cast<const char*>(sv) + (tb + 4 * qg + (n >> 2)) * (kRowPieces * 16);
      bf16x8_t vb[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        typedef short tr4_t __attribute__((ext_vector_type(4)));
        const char* a = vrow + vtr_off[c];
        const tr4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) tr4_t*)(a));
        const tr4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) tr4_t*)(a + 16 * kRowPieces * 16));
        vb[c] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                        0, 1, 2, 3, 4, 5, 6, 7);
      }
      const int keyq = kv0 + tb + 4 * qg;   // key of slot 0
      const bool full = kv0 + tb + 32 <= lim_wave;   // no key of the block is masked for this wave
      // Scores of both tiles first, as four independent accumulation chains
      // (tile, 16-key half): the K fragments are dead before any softmax
      // starts, and the chains do not wait on each other. A tile without a
      // live row has zero q, so its scores are computed and ignored.
      // (Bit-identical to scoring and finishing one tile at a time, and 2-3%
      // faster on the mixed prefill in interleaved A/B runs.)
      f32x4_t sc[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) sc[t][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            sc[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h][s], qf[t][s], sc[t][h], 0, 0, 0);

      // Softmax weights of tile t as the A operand of P.V; rescales tile t's
      // sums and accumulators where its reference max rises, then adds its
      // P.V and row sums. Tile 0's products are issued before tile 1's
      // softmax, which needs none of their results.
      auto tile_softmax_pv = [&](auto t_tag) {
        constexpr int t = decltype(t_tag)::value;
        float x[8];   // raw scores q.k
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[4 * h + r] = sc[t][h][r];
        if (!full) {
          const int lim = p.causal ? min(qpos[t] + 1, ctx) : ctx;   // visible keys < lim
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = (keyq + 16 * (u / 4) + (u % 4) < lim) ? x[u] : neg_inf();
        }
        // scale > 0 is finite, so a row max of -inf stays -inf. A row's
        // maximum clears the threshold exactly when the maximum of one of
        // its four lanes does, so each lane tests its own and the row's
        // maximum (a reduction across the lanes) is formed only when some
        // reference rises.
        const float lane_max = max8(x);
        if (__any(lane_max * scale > m_ref[t] + kRescaleThreshold)) {
          const float mt = max_across_rows(lane_max) * scale;
          const float m_new = fmaxf(m_ref[t], mt);
          const float alpha = (m_new == neg_inf()) ? 1.f : fast_exp2(m_ref[t] - m_new);
          m_ref[t] = m_new;
          nm_ref[t] = (m_new == neg_inf()) ? 0.f : -m_new;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = __shfl(alpha, 4 * qg + r, 64);   // factor of row 4qg + r
            lsum[t][r] *= a;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[t][i][r] *= a;
          }
        }
        // weight 2^(scale*x - m): a masked score (-inf) gives exactly 0, since
        // scale > 0 and m is finite (0 while the row has seen no key)
        const float nm = nm_ref[t];
        uint32_t pw[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          pw[h] = pack_bf16x2(fast_exp2(fmaf(x[2 * h], scale, nm)), fast_exp2(fmaf(x[2 * h + 1], scale, nm)));
        const bf16x8_t pa = bit_cast_to<bf16x8_t>(make_uint4(pw[0], pw[1], pw[2], pw[3]));
        lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, ones, lsum[t], 0, 0, 0);
        // O += P V (operands read at the top of the step)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb[c], acc[t][c], 0, 0, 0);
      };
      tile_softmax_pv(std::integral_constant<int, 0>{});
      if (live1) tile_softmax_pv(std::integral_constant<int, 1>{});
    }
    wait_loads();
    if (FP8 && more) store8(buf ^ 1);
    __syncthreads();
  };
  for (int kt = 0; kt < n_kv; kt += 2) {
    tile_step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < n_kv) tile_step(kt + 1, std::integral_constant<int, 1>{});
  }

  // ---- normalise and write ------------------------------------------------
  // a block id outside the pool, met by any thread's gather, poisons the tile
  if (bad) s_bad = 1;
  __syncthreads();
  const bool poisoned = s_bad != 0;
  const float vsc = FP8 ? p.v_scale[g] : 1.f;   // E4M3: the kv-head's V scale
  if (p.part_m != nullptr) {
    // partials for a later merge: row 4qg + r of tile t has its reference max in
    // the lane whose n is 4qg + r; sums are replicated over n
    if (g == 0 && qt == 0 && w == 0)
      for (int i = lane; i < L; i += 64) p.seq_prefix[q_start + i] = ctx;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = __shfl(m_ref[t], 4 * qg + r, 64);
        const int mr = 16 * (w + kPW * t) + 4 * qg + r;
        const int qi = r0 + mr / G;
        if (qi >= L) continue;
        const int64_t row = (int64_t)(q_start + qi) * p.num_q_heads + g * G + mr % G;
        float* po = p.part_o + row * kD + n;
#pragma unroll
        for (int c = 0; c < 8; ++c) po[16 * c] = acc[t][c][r] * vsc;
        if (n == 0) {
          p.part_m[row] = m;
          p.part_l[row] = poisoned ? __builtin_nanf("") : lsum[t][r];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mr = 16 * (w + kPW * t) + 4 * qg + r;
      const int qi = r0 + mr / G;
      if (qi >= L) continue;
      const float inv = poisoned ? __builtin_nanf("") : vsc / lsum[t][r];
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) +
                       ((int64_t)(q_start + qi) * p.num_q_heads + g * G + mr % G) * kD + n;
#pragma unroll
      for (int c = 0; c < 8; ++c) orow[16 * c] = f32_to_bf16_rne(acc[t][c][r] * inv);
    }
  }
}

template <bool FP8>
static hipError_t launch_prefill_t(const PrefillParams& p, int head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int bq = kMRows / p.group;
  PrefillParams q = p;
  q.num_q_tiles = (p.max_q_len + bq - 1) / bq;
  q.longest_first = (int64_t)q.num_q_tiles * p.num_seqs <= kOrderMaxItems;
  const int64_t items = (int64_t)q.num_q_tiles * p.num_seqs * p.num_kv_heads;
  if (items > 0x7fffffff - kXcds) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((items + kXcds - 1) / kXcds * kXcds));
  const int cus = device_compute_units();
  q.pair_span = (q.longest_first && (int64_t)grid.x >= 2 * (int64_t)cus) ? cus : 0;
  switch (p.group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<1, FP8>), grid, dim3(kPThreads), 0, stream, q); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<2, FP8>), grid, dim3(kPThreads), 0, stream, q); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<4, FP8>), grid, dim3(kPThreads), 0, stream, q); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<8, FP8>), grid, dim3(kPThreads), 0, stream, q); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<16, FP8>), grid, dim3(kPThreads), 0, stream, q); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  return launch_prefill_t<false>(p, head_dim, stream);
}

hipError_t launch_prefill_fp8(const PrefillParams& p, int head_dim, hipStream_t stream) {
  return launch_prefill_t<true>(p, head_dim, stream);
}

}  // namespace pkv
