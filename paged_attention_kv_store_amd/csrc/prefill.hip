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
// heads. Wave w owns M rows 32w .. 32w+31 as two 16-row tiles.
//
// The keys are walked in 64-token tiles gathered through the block table
// into LDS (double-buffered: the next tile's global loads are in flight while
// the current one is consumed), 16-byte pieces XOR-swizzled by row so that
// both access patterns below are free of bank conflicts. Per 16 keys:
//  * S^T = K Q^T on 16x16x32 bf16 MFMA (A = 16 K rows from LDS, B = the
//    wave's Q rows kept in registers) gives each lane the scores of keys
//    4*(l/16)+r for M row l%16;
//  * causal / context mask, online softmax in fp32 (log2 domain, lazy
//    rescaling), P rounded to bf16;
//  * O += P V on 16x16x16 bf16 MFMA: P is already laid out as the A operand;
//    the B operand (4 keys of one column per lane) comes from whole V rows
//    read from LDS with two in-lane byte permutes.
#include "common.h"
#include "device_utils.h"

namespace pkv {

namespace {

constexpr int kD = 128;               // head_dim
constexpr int kPW = 4;                // waves per workgroup
constexpr int kPThreads = 64 * kPW;
constexpr int kMRows = 32 * kPW;      // M rows per workgroup
constexpr int kKvTile = 64;           // keys per LDS tile
constexpr int kRowPieces = kD * 2 / 16;   // 16-byte pieces per K/V row (16)

// LDS position (in 16-byte units) of piece c of key row t in a tile.
__device__ __forceinline__ int swz(int t, int c) { return t * kRowPieces + (c ^ (t & 15)); }

struct KvStage {
  uint4 k[4];
  uint4 v[4];
};

}  // namespace

template <int G>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillParams p) {
  constexpr int BQ = kMRows / G;      // query rows per workgroup
  __shared__ uint4 s_k[2][kKvTile * kRowPieces];
  __shared__ uint4 s_v[2][kKvTile * kRowPieces];
  __shared__ int s_bad;

  const int qt = blockIdx.x, g = blockIdx.y, c = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
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
  const int32_t* bt = p.block_tables + (int64_t)c * p.max_blocks;
  const float scale = p.scale_log2;

  // ---- the wave's Q rows (B operand of S^T = K Q^T) ----------------------
  // tile t, lane l: M row mr = 32w + 16t + l%16 (query row r0 + mr/G, head
  // mr%G); step s holds head_dim elements [32s + 8qg, 32s + 8qg + 8).
  bf16x8_t qf[2][4];
  int qpos[2];          // absolute position of the lane's softmax row
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mr = 32 * w + 16 * t + n;
    const int qi = r0 + mr / G;
    qpos[t] = P0 + qi;
    const bool live = qi < L;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)(q_start + qi) * p.num_q_heads + g * G + mr % G) * kD + 8 * qg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (live) v = load16(qrow + 32 * s);
      qf[t][s] = bit_cast_to<bf16x8_t>(v);
    }
  }

  // ---- cooperative K/V tile gather (global -> registers -> LDS) ----------
  // thread tid moves pieces f = i*256 + tid, i = 0..3: key row f/16, piece f%16
  bool bad = false;
  auto gather = [&](int kt, KvStage& st) {
    const int kv0 = kt * kKvTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = i * kPThreads + tid;
      const int t = f / kRowPieces, piece = f % kRowPieces;
      const int pos = kv0 + t;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (pos < ctx) {   // keys past the context read as zeros (never NaN garbage)
        int blk = bt[pos / bs];
        if ((unsigned)blk >= (unsigned)p.num_blocks) {
          blk = 0;
          bad = true;
        }
        const int64_t off = ((int64_t)blk * bs + pos % bs) * row_elems + g * kD + piece * 8;
        kv = load16(reinterpret_cast<const uint16_t*>(p.k_cache) + off);
        vv = load16(reinterpret_cast<const uint16_t*>(p.v_cache) + off);
      }
      st.k[i] = kv;
      st.v[i] = vv;
    }
  };
  auto to_lds = [&](int buf, const KvStage& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = i * kPThreads + tid;
      const int t = f / kRowPieces, piece = f % kRowPieces;
      s_k[buf][swz(t, piece)] = st.k[i];
      s_v[buf][swz(t, piece)] = st.v[i];
    }
  };

  float m_ref[2] = {neg_inf(), neg_inf()};   // per softmax row (lane's n)
  float l_part[2] = {0.f, 0.f};
  f32x4_t acc[2][8];                          // acc[t][i][r] = O[row 16t + 4qg + r][8n + i]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (tid == 0) s_bad = 0;
  KvStage stage;
  if (n_kv > 0) {
    gather(0, stage);
    to_lds(0, stage);
  }
  __syncthreads();

  for (int kt = 0; kt < n_kv; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < n_kv;
    if (more) gather(kt + 1, stage);
    const int kv0 = kt * kKvTile;
    const uint4* sk = s_k[buf];
    const uint4* sv = s_v[buf];

#pragma unroll
    for (int sub = 0; sub < kKvTile / 16; ++sub) {
      const int tb = 16 * sub;              // first key of the sub-tile, tile-relative
      if (kv0 + tb >= kv_end) break;
      // K rows tb + n, pieces 4s + qg (elements 32s + 8qg .. +8)
      bf16x8_t kf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[s] = bit_cast_to<bf16x8_t>(sk[swz(tb + n, 4 * s + qg)]);
      // V rows tb + 4qg + st, piece n (columns 8n .. 8n+7)
      uint32_t vd[4][4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint4 v = sv[swz(tb + 4 * qg + st, n)];
        vd[st][0] = v.x;
        vd[st][1] = v.y;
        vd[st][2] = v.z;
        vd[st][3] = v.w;
      }
      const int keyq = kv0 + tb + 4 * qg;   // key position of the lane's r = 0
      short4_t pa[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[t][s], sc, 0, 0, 0);
        const int lim = p.causal ? min(qpos[t] + 1, ctx) : ctx;   // visible keys < lim
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (keyq + r < lim) ? sc[r] * scale : neg_inf();
        float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mt = fmaxf(mt, shfl_xor_f(mt, 16));
        mt = fmaxf(mt, shfl_xor_f(mt, 32));
        if (__any(mt > m_ref[t] + kRescaleThreshold)) {
          const float m_new = fmaxf(m_ref[t], mt);
          const float alpha = (m_new == neg_inf()) ? 1.f : fast_exp2(m_ref[t] - m_new);
          l_part[t] *= alpha;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = __shfl(alpha, 4 * qg + r, 64);   // factor of row 4qg + r
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[t][i][r] *= a;
          }
          m_ref[t] = m_new;
        }
        const float mb = (m_ref[t] == neg_inf()) ? 0.f : m_ref[t];
        uint32_t pw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          pw[h] = pack_bf16x2(fast_exp2(x[2 * h] - mb), fast_exp2(x[2 * h + 1] - mb));
          l_part[t] += bf16_lo(pw[h]) + bf16_hi(pw[h]);
        }
        pa[t] = __builtin_bit_cast(short4_t, make_uint2(pw[0], pw[1]));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t b0 = __builtin_amdgcn_perm(vd[1][i / 2], vd[0][i / 2], sel);
        const uint32_t b1 = __builtin_amdgcn_perm(vd[3][i / 2], vd[2][i / 2], sel);
        const short4_t vb = __builtin_bit_cast(short4_t, make_uint2(b0, b1));
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[t], vb, acc[t][i], 0, 0, 0);
      }
    }
    if (more) {
      // the other buffer was last read before the previous barrier
      to_lds(buf ^ 1, stage);
    }
    __syncthreads();
  }

  // ---- normalise and write ------------------------------------------------
  // a block id outside the pool, met by any thread's gather, poisons the tile
  if (bad) s_bad = 1;
  __syncthreads();
  const bool poisoned = s_bad != 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float l = l_part[t];
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);          // row sum of M row 16t + n (all lanes with this n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lr = __shfl(l, 4 * qg + r, 64);   // sum of row 16t + 4qg + r
      const int mr = 32 * w + 16 * t + 4 * qg + r;
      const int qi = r0 + mr / G;
      if (qi >= L) continue;
      const float inv = poisoned ? __builtin_nanf("") : 1.f / lr;
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(acc[t][2 * h][r] * inv, acc[t][2 * h + 1][r] * inv);
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) +
                       ((int64_t)(q_start + qi) * p.num_q_heads + g * G + mr % G) * kD + 8 * n;
      *reinterpret_cast<uint4*>(orow) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int bq = kMRows / p.group;
  const dim3 grid((p.max_q_len + bq - 1) / bq, p.num_kv_heads, p.num_seqs);
  switch (p.group) {
    case 1: hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(kPThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(kPThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(prefill_kernel<4>, grid, dim3(kPThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(prefill_kernel<8>, grid, dim3(kPThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
