// Grouped-query attention decode for gfx950: split-KV partial softmax + exact combine.
//
// One query per sequence attends to the first seq_lens[b] keys of a contiguous
// cache.  This is a batched matrix-vector product with per-request lengths and
// arithmetic intensity near 1 (x G for grouped heads), so it is bound by HBM
// bandwidth ("MHA -> GQA" blog, sections 3.1 and 3.2).  The keys of each
// sequence are cut into splits; every split produces a partial (max, sum,
// unnormalised output) and a second kernel merges the partials with the same
// rescaling that makes tiled softmax exact (FlashAttention-3 page, the recap
// of tiling + softmax rescaling and the HN remark on splitting/combining the
// softmax).
//
// Split kernel (bf16): single-wave workgroups.  Each K/V row is read from HBM
// once and serves all G query heads of its group through MFMA 16x16x32:
// S^T = K . Q^T (bf16, the heads as the 16 columns) and O^T += V^T . P^T
// (bf16: P = P_hi + P_lo as two bf16 MFMAs, so P keeps about 16 bits, and any
// finite bf16 V is an exact operand).  K rows are loaded straight into the
// MFMA operand registers; V rows are staged through the wave's LDS and
// transposed.  Tiles are 32 keys; the next tile's loads are in flight while
// the current one is finished.
// Work assignment: for large caches the tiles of every (sequence, KV head)
// are laid end to end and each resident workgroup streams an equal share of
// them, crossing sequence ends, so ragged lengths stay balanced over the
// chip; otherwise (or with an explicit split) one workgroup per fixed split.
// Combine kernel: one wave per (sequence, query head) merges the partials.
#include <algorithm>
#include <climits>

#include "common.h"
#include "launch.h"

namespace mqkv {

namespace {

constexpr int kTK = 32;      // keys per tile: two 16-key MFMA blocks
constexpr int kMinTiles = 4;  // balanced mode: at least this many tiles per workgroup
constexpr int kWavesPerCU = 12;  // split-kernel workgroups resident per CU (3 per SIMD)
constexpr int64_t kBalancedMinTiles = 16384;  // auto: balanced split from this many tiles at capacity
constexpr int kShortSplit = 64;               // auto: keys per split below that
// Fused small-cache decode: waves per workgroup; it is chosen for caches of at
// most kFusedWaves tiles (one tile per wave), or of at most kFusedManyTiles
// tiles when there are at least kFusedManySegs segments to fill the chip.
constexpr int kFusedWaves = 8;
constexpr int kFusedManyTiles = 32;
constexpr int kFusedManySegs = 128;

template <int D>
struct DecodeLds {
  static constexpr int kVld = kTK + 8;  // V^T row stride (bf16 elements)
  static constexpr size_t kBytes = (size_t)D * kVld * sizeof(uint16_t);
};

// Position in a V^T row of key k (0..31) of a tile: the P^T operand lane group
// kg holds keys {4kg..4kg+3} of the first 16-key block then the same of the
// second block, so those eight keys are stored contiguously.
__device__ __forceinline__ int vt_pos32(int k) { return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3); }

// A K/V cache row is read once per call.  When the caches are large (STREAM),
// rows are loaded with the non-temporal hint so the stream does not allocate in
// the caches: it then neither evicts data that is reused (a projection weight
// that fits the Infinity Cache) nor has to write back, while it streams, the
// dirty lines earlier kernels left there.  Small caches (a few MB, which stay
// resident from one decode step to the next) use ordinary loads.
constexpr int64_t kStreamBytes = (int64_t)64 << 20;  // K + V capacity from which STREAM is used
template <bool STREAM>
__device__ __forceinline__ u32x4_t ld16_kv(const void* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return ld16(p);
}

// Keys of sequence b that are attended (lengths beyond the cache are clamped).
__device__ __forceinline__ int seq_len(const int32_t* seq_lens, int b, int Lmax) {
  return min(max(seq_lens[b], 0), Lmax);
}

// Balanced work split.  The tiles of all (sequence, KV head, query-head block)
// segments are laid end to end, sequence-major; segment (b, g, qb) holds
// ceil(len_b / 32) tiles.  Workgroup w streams tiles [w*tpw, (w+1)*tpw) of that
// line, crossing segment ends, so every workgroup moves the same number of
// bytes whatever the length mix.  Computed by one wave from seq_lens:
// the total tile count T, and (when t >= 0) the sequence holding tile t with the
// number of tiles before that sequence.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
struct TileLine {
  int64_t total;
  int b;          // sequence holding tile t (-1 if none)
  int64_t base;   // tiles before sequence b
};
__device__ TileLine tile_line(const int32_t* seq_lens, int B, int Lmax, int per_seq, int64_t t) {
  const int lane = threadIdx.x & 63;
  TileLine r{0, -1, 0};
  int64_t carry = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const int64_t v = bb < B ? (int64_t)((seq_len(seq_lens, bb, Lmax) + kTK - 1) / kTK) * per_seq : 0;
    int64_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int64_t excl = carry + incl - v;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(v > 0 && excl <= t && t < carry + incl);
    if (r.b < 0 && hit != 0) {
      const int l = __builtin_ctzll(hit);
      r.b = b0 + l;
      r.base = __shfl(excl, l, 64);
    }
    carry += __shfl(incl, 63, 64);
  }
  // every lane holds the same values: make them scalar
  r.total = uniform64(carry);
  r.b = __builtin_amdgcn_readfirstlane(r.b);
  r.base = uniform64(r.base);
  return r;
}
__device__ __forceinline__ int64_t balanced_tpw(int64_t total, int nwg) {
  const int64_t t = (total + nwg - 1) / nwg;
  return t > kMinTiles ? t : kMinTiles;
}

// One single-wave workgroup per work unit.  A unit is a run of tiles of one
// (sequence, KV head, block of 16 query heads) segment:
//  * aligned mode (split > 0): unit = the split-th piece of split keys of one
//    segment; partial slot = split index;
//  * balanced mode (split == 0): the workgroup's tiles of the balanced line,
//    one unit per segment they touch; partial slot = workgroup - first
//    workgroup of the segment.
// Per unit, MFMA 16x16x32 layout: A (16 x 32): lane l holds row l%16, k slot
// group l/16; B (32 x 16): column l%16, the same k group; D (16 x 16): column
// l%16, rows 4*(l/16) + i.
// NW = 1: the split kernel (one wave per workgroup, partials to the workspace).
// NW > 1: the fused small-cache kernel (see attn_decode_fused_bf16 below):
// one workgroup per segment, its NW waves take contiguous tile ranges, and
// their partials are merged in LDS into O and LSE (OUT_BF16: the output type).
template <int D, bool STREAM, int NW = 1, bool OUT_BF16 = true>
__global__ __launch_bounds__(64 * NW, NW == 1 ? 3 : 1) void attn_decode_split_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_o, float* __restrict__ part_ml,
    int B, int Hq, int Hkv, int Lmax, int64_t q_stride, float c, int split, int n_slot, int n_qblk,
    const int32_t* __restrict__ block_table, int page_size, int pages_per_seq, int num_pages,
    void* __restrict__ o_out = nullptr, float* __restrict__ lse_out = nullptr) {
  using S = DecodeLds<D>;
  constexpr int DS = D / 32;                       // k-steps of the score MFMA
  constexpr int DB = D / 16;                       // 16-row blocks of O^T
  constexpr int VTASK = (kTK / 4) * (D / 8) / 64;  // V 4x8 blocks per lane
  constexpr int kVtElems = (int)(S::kBytes / sizeof(uint16_t));
  extern __shared__ __align__(16) uint16_t smem[];
  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  uint16_t* Vt = smem + wave * kVtElems;  // this wave's V^T staging

  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const int G = Hq / Hkv;
  const int64_t row_stride = (int64_t)Hkv * D;
  // Fused mode: a wave's partial (its O^T accumulators, the row max and sum)
  // as a record of 4 DB + 2 floats per lane, lane-fastest, in the wave's own
  // V^T region (free once its last tile is done).
  constexpr int kRec = 4 * DB + 2;
  static_assert(NW == 1 || (size_t)kRec * 64 * 4 <= S::kBytes, "a wave's record fits its V^T region");
  float* rec = reinterpret_cast<float*>(Vt);
  auto emit_lds = [&](const f32x4_t (&acc)[DB], float m, float l) {
    wave_lds_sync();  // this wave's last V^T reads are done
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) rec[(db * 4 + e) * 64 + lane] = acc[db][e];
    rec[(4 * DB) * 64 + lane] = m;
    rec[(4 * DB + 1) * 64 + lane] = l;
  };

  // Process tiles [tb, tb + ntile) of segment (b, g, qblk) and write its partial to `slot`.
  auto unit = [&](int b, int g, int qblk, int tb, int ntile, int slot) {
    const int len = seq_len(seq_lens, b, Lmax);
    const int kbeg = tb * kTK;
    const int kend = min((tb + ntile) * kTK, len);
    const int nt = (kend - kbeg + kTK - 1) / kTK;
    const int col = qblk * 16 + l16;  // query head within the group
    const bool hvalid = col < G;
    const int h = g * G + (hvalid ? col : 0);

    // Q^T operand: at k-step st lane (col, g4) holds d-chunk 4*st + g4 of its
    // head (the four lanes of a row then read 64 contiguous bytes per K load)
    u32x4_t qf[DS];
    {
      const uint16_t* qp = q + (int64_t)b * q_stride + (int64_t)h * D + g4 * 8;
#pragma unroll
      for (int st = 0; st < DS; ++st) qf[st] = hvalid ? ld16(qp + st * 32) : u32x4_t{0, 0, 0, 0};
    }
    const uint16_t* kbase = kc + (int64_t)g * D + g4 * 8;
    const uint16_t* vbase = vc + (int64_t)g * D;
    // Cache row of key k = block offset + k, per 16-key block (one page holds
    // whole 16-key blocks): the sequence's rows for a contiguous cache, the
    // page's rows for a paged one.  A block past the keys, or on a page id
    // outside the page pool, gets kNoRow and reads as zeros.
    constexpr int64_t kNoRow = INT64_MIN;
    auto block_off = [&](int ks) -> int64_t {
      if (ks >= kend) return kNoRow;
      if (block_table == nullptr) return (int64_t)b * Lmax;
      const int pg = block_table[(int64_t)b * pages_per_seq + ks / page_size];
      if (pg < 0 || pg >= num_pages) return kNoRow;
      return (int64_t)pg * page_size + ks % page_size - ks;
    };

    // K goes straight into the A-operand registers (lane = key row); V is staged
    // through LDS to be transposed.  V tasks are 4 keys x 8 dimensions, with
    // consecutive lanes on consecutive key groups so that one 8-byte LDS store
    // covers whole V^T rows.
    u32x4_t kr[2][DS];
    u32x4_t rv[VTASK][4];
    // block offsets of the tile that load_tile will fetch next; each call
    // looks up the following tile's, so a paged cache's table reads are one
    // tile ahead of the K/V loads that depend on them
    int64_t off_next[2] = {block_off(kbeg), block_off(kbeg + 16)};
    auto load_tile = [&](int t) {
      const int k0 = kbeg + t * kTK;
      const int64_t off[2] = {off_next[0], off_next[1]};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int gk = k0 + kb * 16 + l16;
#pragma unroll
        for (int st = 0; st < DS; ++st)
          kr[kb][st] = (gk < kend && off[kb] != kNoRow)
                           ? ld16_kv<STREAM>(kbase + (off[kb] + gk) * row_stride + st * 32)
                           : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < VTASK; ++j) {
        const int ti = lane + j * 64;
        const int a = ti % (kTK / 4), dg = ti / (kTK / 4);
        const int64_t vo = off[a >> 2];  // keys 4a..4a+3 lie in 16-key block a/4
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int gk = k0 + a * 4 + jj;
          rv[j][jj] = (gk < kend && vo != kNoRow) ? ld16_kv<STREAM>(vbase + (vo + gk) * row_stride + dg * 8)
                                                  : u32x4_t{0, 0, 0, 0};
        }
      }
      off_next[0] = block_off(k0 + kTK);
      off_next[1] = block_off(k0 + kTK + 16);
    };
    // V^T of the tile in LDS as the raw bf16 values (P.V runs on bf16 matrix
    // cores, where any finite bf16 V is an exact operand)
    auto store_v = [&]() {
#pragma unroll
      for (int j = 0; j < VTASK; ++j) {
        const int ti = lane + j * 64;
        const int a = ti % (kTK / 4), dg = ti / (kTK / 4);
        const int cpos = vt_pos32(a * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dimension 2e of keys 4a..4a+3 (the low halves), then dimension 2e + 1
          u32x2_t lo, hi;
          lo[0] = __builtin_amdgcn_perm(rv[j][1][e], rv[j][0][e], 0x05040100u);
          lo[1] = __builtin_amdgcn_perm(rv[j][3][e], rv[j][2][e], 0x05040100u);
          hi[0] = __builtin_amdgcn_perm(rv[j][1][e], rv[j][0][e], 0x07060302u);
          hi[1] = __builtin_amdgcn_perm(rv[j][3][e], rv[j][2][e], 0x07060302u);
          st8(Vt + (dg * 8 + 2 * e) * S::kVld + cpos, lo);
          st8(Vt + (dg * 8 + 2 * e + 1) * S::kVld + cpos, hi);
        }
      }
    };

    f32x4_t acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x4_t{};
    float m_run = -INFINITY, l_run = 0.0f;

    load_tile(0);
    for (int t = 0; t < nt; ++t) {
      wave_lds_sync();  // the previous tile's V^T reads are done before overwriting
      store_v();
      wave_lds_sync();
      const int k0 = kbeg + t * kTK;
      f32x4_t sb[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
      for (int st = 0; st < DS; ++st)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sb[kb] = mfma16_bf16(kr[kb][st], qf[st], sb[kb]);
      if (t + 1 < nt) load_tile(t + 1);  // in flight while this tile is finished

      // lane (col, g4) holds keys kb*16 + 4*g4 + i of its query head
      if (k0 + kTK > kend) {
        const int rel = kend - 1 - k0 - 4 * g4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb * 16 + i > rel) sb[kb][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(sb[0][0], sb[0][1]), fmaxf(sb[0][2], sb[0][3])),
                       fmaxf(fmaxf(sb[1][0], sb[1][1]), fmaxf(sb[1][2], sb[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = max_xor32(mx);
      const float mt = mx * c;
      if (__builtin_amdgcn_ballot_w64(mt > m_run + 8.0f) != 0) {
        // only this row's own growth moves its max (rows sharing the wave do not matter)
        const float mn = (mt > m_run + 8.0f) ? mt : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        m_run = mn;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
      }
      // P^T operand: slots 0-3 = keys 4*g4+i of block 0, slots 4-7 = the same of block 1.
      // P = P_hi + P_lo, both bf16 (P_lo the rounding residual of P_hi): two
      // bf16 MFMAs carry P to about 16 bits, against fp32 P's row sum
      u32x4_t ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kb = e >> 1, i = (e & 1) * 2;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[kb][i], c, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[kb][i + 1], c, -m_run));
        const uint32_t w = pack_bf16(p0, p1);
        ph[e] = w;
        pl[e] = pack_bf16(p0 - bf16lo(w), p1 - bf16hi(w));
        l_run += p0 + p1;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4_t vf = ld16(Vt + (db * 16 + l16) * S::kVld + g4 * 8);
        acc[db] = mfma16_bf16(vf, ph, acc[db]);
        acc[db] = mfma16_bf16(vf, pl, acc[db]);
      }
    }

    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if constexpr (NW > 1) {
      emit_lds(acc, m_run, l_tot);
    } else if (hvalid) {
      const int64_t pidx = ((int64_t)b * Hq + h) * n_slot + slot;
      float* po = part_o + pidx * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        st16(po + db * 16 + 4 * g4, u32x4_t{__float_as_uint(acc[db][0]), __float_as_uint(acc[db][1]),
                                            __float_as_uint(acc[db][2]), __float_as_uint(acc[db][3])});
      if (g4 == 0)
        st16(part_ml + pidx * 4, u32x4_t{__float_as_uint(m_run), __float_as_uint(l_tot), 0u, 0u});
    }
  };

  if constexpr (NW > 1) {
    // Fused mode: workgroup = segment (b, g, qblk); wave w takes tiles
    // [w ntb / NW, (w + 1) ntb / NW) of it (none when the segment is short).
    const int seg_id = blockIdx.x;
    const int qblk = seg_id % n_qblk, bg = seg_id / n_qblk;
    const int b = bg / Hkv, g = bg % Hkv;
    const int ntb = (seq_len(seq_lens, b, Lmax) + kTK - 1) / kTK;
    const int tb = (int)((int64_t)wave * ntb / NW), te = (int)((int64_t)(wave + 1) * ntb / NW);
    if (te > tb) {
      unit(b, g, qblk, tb, te - tb, 0);
    } else {  // no keys for this wave: a record that weighs nothing
      f32x4_t zero[DB];
#pragma unroll
      for (int i = 0; i < DB; ++i) zero[i] = f32x4_t{};
      emit_lds(zero, -INFINITY, 0.0f);
    }
    __syncthreads();
    // Merge, exactly as the combine kernel does: the largest max M over the
    // waves, O = sum_w 2^(m_w - M) acc_w / L, L = sum_w 2^(m_w - M) l_w.  Wave
    // w' merges the 16-row blocks db = w', w' + NW, ...; lane (head column
    // l16, group g4) as in a record.
    const int col = qblk * 16 + l16;
    const bool hvalid = col < G;
    const int h = g * G + (hvalid ? col : 0);
    const float* recs = reinterpret_cast<const float*>(smem);
    constexpr int kRegion = kVtElems / 2;  // floats per wave region
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, recs[w * kRegion + (4 * DB) * 64 + lane]);
    float L = 0.0f, wt[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = recs[w * kRegion + (4 * DB) * 64 + lane];
      wt[w] = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      L = __builtin_fmaf(wt[w], recs[w * kRegion + (4 * DB + 1) * 64 + lane], L);
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;  // no keys: O = 0
    for (int db = wave; db < DB; db += NW) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v = __builtin_fmaf(wt[w], recs[w * kRegion + (db * 4 + e) * 64 + lane], v);
        const float r = v * inv;
        if (hvalid) {
          const int64_t oi = ((int64_t)b * Hq + h) * D + db * 16 + 4 * g4 + e;
          if constexpr (OUT_BF16)
            static_cast<uint16_t*>(o_out)[oi] = f32_to_bf16(r);
          else
            static_cast<float*>(o_out)[oi] = r;
        }
      }
    }
    if (lse_out != nullptr && wave == 0 && g4 == 0 && hvalid)
      lse_out[(int64_t)b * Hq + h] = (M + __builtin_log2f(L)) * kLn2;
    return;
  }

  // Work assignment; a single call site keeps one copy of the unit code.
  const int per_seq = Hkv * n_qblk;
  int64_t t = 0, t1 = 0, tpw = 1, base = 0;
  int b = 0;
  bool aligned_done = false;
  if (split > 0) {
    // aligned mode: (sequence, KV head, query block, split), splits of one
    // segment neighbours, each XCD a contiguous range
    const int n_split = (Lmax + split - 1) / split;
    int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int sidx = lid % n_split;
    lid /= n_split;
    const int qblk = lid % n_qblk;
    const int bg = lid / n_qblk;
    b = bg / Hkv;
    if (sidx * split >= seq_len(seq_lens, b, Lmax)) return;
    // express the split as tiles of the (b, g, qblk) segment
    t = sidx * (split / kTK);
    t1 = t + split / kTK;
    base = -(int64_t)(bg % Hkv * n_qblk + qblk);  // segment index carried in base (see below)
  } else {
    const int64_t total = tile_line(seq_lens, B, Lmax, per_seq, -1).total;
    tpw = balanced_tpw(total, gridDim.x);
    t = (int64_t)blockIdx.x * tpw;
    t1 = min(total, t + tpw);
    if (t >= t1) return;
    const TileLine at = tile_line(seq_lens, B, Lmax, per_seq, t);
    b = at.b;
    base = at.base;
  }
  while (t < t1 && b < B) {
    int seg, tb, n, slot;
    if (split > 0) {
      if (aligned_done) break;
      aligned_done = true;
      seg = (int)(-base);
      tb = (int)t;
      n = (int)(t1 - t);
      slot = (int)(t / (split / kTK));
    } else {
      const int ntb = (seq_len(seq_lens, b, Lmax) + kTK - 1) / kTK;  // tiles per segment of b
      const int64_t local = t - base;
      if (ntb == 0 || local >= (int64_t)ntb * per_seq) {  // past sequence b (or it is empty)
        base += (int64_t)ntb * per_seq;
        ++b;
        continue;
      }
      seg = (int)(local / ntb);  // g * n_qblk + qblk within sequence b
      tb = (int)(local % ntb);
      n = (int)min((int64_t)(ntb - tb), t1 - t);
      const int64_t seg_start = base + (int64_t)seg * ntb;
      slot = (int)((int64_t)blockIdx.x - seg_start / tpw);
    }
    unit(b, seg / n_qblk, seg % n_qblk, tb, n, slot);
    t += n;
  }
}

// fp32 split kernel: one wave per (sequence, query head, split); lane j scores key j
// of each 64-key chunk, every lane accumulates D/64 output elements.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_split_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_o, float* __restrict__ part_ml,
    int Hq, int Hkv, int Lmax, int64_t q_stride, float c, int split, int n_slot) {
  constexpr int PER = D / 64;
  __shared__ float qs[D];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int len = min(seq_lens[b], Lmax);
  const int kbeg = s * split;
  if (kbeg >= len) return;
  const int kend = min(kbeg + split, len);
  for (int i = lane; i < D; i += 64) qs[i] = q[(int64_t)b * q_stride + (int64_t)h * D + i];
  __syncthreads();
  const int64_t row_stride = (int64_t)Hkv * D;
  const float* kb = kc + (int64_t)b * Lmax * row_stride + (int64_t)g * D;
  const float* vb = vc + (int64_t)b * Lmax * row_stride + (int64_t)g * D;
  float acc[PER] = {};
  float m = -INFINITY, l = 0.0f;
  for (int k0 = kbeg; k0 < kend; k0 += 64) {
    const int key = k0 + lane;
    float sc = -INFINITY;
    if (key < kend) {
      float dot = 0.0f;
      for (int i = 0; i < D; ++i) dot = __builtin_fmaf(qs[i], kb[(int64_t)key * row_stride + i], dot);
      sc = dot * c;
    }
    float mx = sc;
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float mn = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    const float p = (key < kend) ? __builtin_amdgcn_exp2f(sc - mn) : 0.0f;
    float ps_sum = p;
    for (int o = 32; o > 0; o >>= 1) ps_sum += __shfl_xor(ps_sum, o, 64);
    l = l * alpha + ps_sum;
    m = mn;
    __syncthreads();
    ps[lane] = p;
    __syncthreads();
    const int nk = min(64, kend - k0);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float a = acc[e] * alpha;
      for (int j = 0; j < nk; ++j) a = __builtin_fmaf(ps[j], vb[(int64_t)(k0 + j) * row_stride + e * 64 + lane], a);
      acc[e] = a;
    }
  }
  const int64_t pidx = ((int64_t)b * Hq + h) * n_slot + s;
#pragma unroll
  for (int e = 0; e < PER; ++e) part_o[pidx * D + e * 64 + lane] = acc[e];
  if (lane == 0) st16(part_ml + pidx * 4, u32x4_t{__float_as_uint(m), __float_as_uint(l), 0u, 0u});
}

// Combine the partials of every unit: one wave per (sequence, query head).
// The number of units of (b, h) follows from the same work split the split
// kernel used (one pass over seq_lens).  Then, 16 units at a time, every lane
// loads one unit's (max, sum) and its D/64 elements of all 16 units' partial
// outputs at once, so the statistics and the outputs cost one round trip
// together; the weights are applied once the wave's maximum is known.
// A sequence with no keys has no units: O = 0, LSE = -inf.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(
    const int32_t* __restrict__ seq_lens, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, void* __restrict__ o, float* __restrict__ lse, int B, int Hq,
    int Hkv, int Lmax, int split, int n_slot, int n_qblk, int nwg) {
  constexpr int EPL = D / 64;  // output elements per lane
  constexpr int U = 16;        // units per round
  const int lane = threadIdx.x;
  const int b = blockIdx.y, h = blockIdx.x;
  const int64_t bh = (int64_t)b * Hq + h;
  const float* ml = part_ml + bh * n_slot * 4;
  const float* po = part_o + bh * n_slot * D;
  // The first round's statistics and outputs are loaded before the number of
  // units is known, so those loads overlap the pass over seq_lens.  Slots
  // below n_slot lie inside the workspace; the values of slots past the unit
  // count (stale or never written) are replaced below, never used.
  const int pre = min(U, n_slot);
  float m_pre = -INFINITY, l_pre = 0.0f, v_pre[U][EPL] = {};
  if (pre > 0) {
    const int sl = lane < pre ? lane : 0;
    const u32x4_t st = ld16(ml + 4 * sl);
    m_pre = __uint_as_float(st[0]);
    l_pre = __uint_as_float(st[1]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e) v_pre[u][e] = u < pre ? po[(int64_t)u * D + e * 64 + lane] : 0.0f;
  }
  const int len = seq_len(seq_lens, b, Lmax);
  int n;
  if (split > 0) {
    n = min((len + split - 1) / split, n_slot);
  } else {
    const int G = Hq / Hkv, per_seq = Hkv * n_qblk;
    const int g = h / G, qblk = (h % G) / 16;
    // tiles of all sequences (the line's total) and before sequence b, in one scan
    int64_t carry = 0, base = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int bb = b0 + lane;
      const int64_t v = bb < B ? (int64_t)((seq_len(seq_lens, bb, Lmax) + kTK - 1) / kTK) * per_seq : 0;
      int64_t incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (b >= b0 && b < b0 + 64) base = carry + __shfl(incl - v, b - b0, 64);
      carry += __shfl(incl, 63, 64);
    }
    const int64_t tpw = balanced_tpw(carry, nwg);
    const int ntb = (len + kTK - 1) / kTK;
    const int64_t s0 = base + (int64_t)(g * n_qblk + qblk) * ntb;
    n = ntb > 0 ? (int)((s0 + ntb - 1) / tpw - s0 / tpw + 1) : 0;
    n = min(n, n_slot);
  }

  float M = -INFINITY, L = 0.0f;  // running max (log2 units) and sum over the rounds so far
  float acc[EPL];                 // O * L
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += U) {
    const int cnt = min(U, n - c0);
    // this lane's unit statistics (lanes >= cnt: none) and every unit's outputs
    float m_l, l_l, v[U][EPL];
    if (c0 == 0) {
      m_l = lane < cnt ? m_pre : -INFINITY;
      l_l = lane < cnt ? l_pre : 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[u][e] = u < cnt ? v_pre[u][e] : 0.0f;
    } else {
      const int sl = c0 + (lane < cnt ? lane : 0);
      const u32x4_t st = ld16(ml + 4 * sl);
      m_l = lane < cnt ? __uint_as_float(st[0]) : -INFINITY;
      l_l = lane < cnt ? __uint_as_float(st[1]) : 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[u][e] = u < cnt ? po[(int64_t)(c0 + u) * D + e * 64 + lane] : 0.0f;
    }
    float mr = m_l;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mr = fmaxf(mr, __shfl_xor(mr, off, 64));
    const float Mn = fmaxf(M, mr);
    // rescale what the earlier rounds accumulated (no earlier round: factor 1)
    const float a = M == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float w = lane < cnt ? __builtin_amdgcn_exp2f(m_l - Mn) : 0.0f;
    float lw = w * l_l;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lw += __shfl_xor(lw, off, 64);
    L = L * a + lw;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wu = __shfl(w, u, 64);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(wu, v[u][e], acc[e]);
    }
    M = Mn;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;  // no keys: O = 0
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int64_t oi = bh * D + e * 64 + lane;
    const float r = acc[e] * inv;
    if constexpr (OUT_BF16)
      static_cast<uint16_t*>(o)[oi] = f32_to_bf16(r);
    else
      static_cast<float*>(o)[oi] = r;
  }
  if (lse != nullptr && lane == 0) lse[bh] = (M + __builtin_log2f(L)) * kLn2;
}

template <int D>
hipError_t launch_split_bf16(const DecodeArgs& a, hipStream_t s, int& nwg) {
  const int G = a.Hq / a.Hkv;
  const int n_qblk = (G + 15) / 16;
  int64_t nblk;
  if (a.split > 0) {
    nblk = (int64_t)a.B * a.Hkv * n_qblk * ((a.Lmax + a.split - 1) / a.split);
  } else {
    // balanced mode: one resident wave per slot of the chip
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t tiles_max = (int64_t)a.B * a.Hkv * n_qblk * ((a.Lmax + kTK - 1) / kTK);
    nblk = std::min((int64_t)cus * kWavesPerCU, (tiles_max + kMinTiles - 1) / kMinTiles);
  }
  if (nblk > 0x7fffffff || nblk < 1) return hipErrorInvalidValue;
  nwg = (int)nblk;
  const bool stream = (int64_t)a.B * a.Lmax * a.Hkv * D * 4 >= kStreamBytes;
  auto kern = stream ? attn_decode_split_bf16_kernel<D, true> : attn_decode_split_bf16_kernel<D, false>;
  const size_t lds = DecodeLds<D>::kBytes;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64), lds, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.seq_lens, a.part_o, a.part_ml, a.B,
                     a.Hq, a.Hkv, a.Lmax, a.q_stride, fmaxf(a.scale * kLog2e, 1e-30f), a.split, a.n_slot,
                     n_qblk, a.block_table, a.page_size, a.pages_per_seq, a.num_pages, nullptr, nullptr);
  return hipGetLastError();
}

// Fused small-cache decode: one workgroup of kFusedWaves waves per (sequence,
// KV head, block of 16 query heads); the waves split the segment's tiles and
// merge their partials in LDS, so there is no workspace traffic and no second
// kernel.  For short caches the split path's cost is latency (one or two tiles
// per wave, then the combine launch and its round trips); here it is one
// launch.
template <int D>
hipError_t launch_fused_bf16(const DecodeArgs& a, hipStream_t s) {
  const int n_qblk = (a.Hq / a.Hkv + 15) / 16;
  const int64_t nblk = (int64_t)a.B * a.Hkv * n_qblk;
  if (nblk > 0x7fffffff || nblk < 1) return hipErrorInvalidValue;
  const bool stream = (int64_t)a.B * a.Lmax * a.Hkv * D * 4 >= kStreamBytes;
  const size_t lds = (size_t)kFusedWaves * DecodeLds<D>::kBytes;
  auto kern = stream ? (a.out_bf16 ? attn_decode_split_bf16_kernel<D, true, kFusedWaves, true>
                                   : attn_decode_split_bf16_kernel<D, true, kFusedWaves, false>)
                     : (a.out_bf16 ? attn_decode_split_bf16_kernel<D, false, kFusedWaves, true>
                                   : attn_decode_split_bf16_kernel<D, false, kFusedWaves, false>);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64 * kFusedWaves), lds, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.seq_lens, a.part_o, a.part_ml, a.B,
                     a.Hq, a.Hkv, a.Lmax, a.q_stride, fmaxf(a.scale * kLog2e, 1e-30f), a.split, a.n_slot,
                     n_qblk, a.block_table, a.page_size, a.pages_per_seq, a.num_pages, a.o, a.lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_f32(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lmax + a.split - 1) / a.split), (unsigned)a.Hq, (unsigned)a.B);
  hipLaunchKernelGGL(attn_decode_split_f32_kernel<D>, grid, dim3(64), 0, s, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, a.seq_lens, a.part_o, a.part_ml, a.Hq,
                     a.Hkv, a.Lmax, a.q_stride, a.scale * kLog2e, a.split, a.n_slot);
  return hipGetLastError();
}

}  // namespace

int decode_auto_split(int B, int Hq, int Hkv, int Lmax, bool bf16) {
  // Balanced work split when the cache at capacity holds enough 32-key tiles to
  // give every resident wave of the chip several; short splits otherwise, where
  // the time is latency and one or two tiles per wave are best.
  const int64_t n_qblk = (Hq / Hkv + 15) / 16;
  const int64_t tiles = (int64_t)B * Hkv * n_qblk * ((Lmax + kTK - 1) / kTK);
  return (bf16 && tiles >= kBalancedMinTiles) ? 0 : kShortSplit;
}

int decode_slots(int B, int Hq, int Hkv, int Lmax, int kv_split, bool bf16) {
  const int split = kv_split > 0 ? kv_split : decode_auto_split(B, Hq, Hkv, Lmax, bf16);
  if (split > 0) return (Lmax + split - 1) / split;
  const int tiles = (Lmax + kTK - 1) / kTK;
  return (tiles + kMinTiles - 1) / kMinTiles + 1;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  // The library's own split on a short cache: the fused kernel instead, where
  // it is the faster one.  A wave's tiles are a chain of dependent loads, so
  // with few segments it pays only at one tile per wave; with many segments
  // the chip is full and the saved combine launch and workspace round trip win.
  if (a.in_bf16 && a.auto_split && a.split > 0) {
    const int64_t ntile = ((int64_t)a.Lmax + kTK - 1) / kTK;
    const int64_t nseg = (int64_t)a.B * a.Hkv * ((a.Hq / a.Hkv + 15) / 16);
    if (ntile <= kFusedWaves || (nseg >= kFusedManySegs && ntile <= kFusedManyTiles))
      return a.d == 64 ? launch_fused_bf16<64>(a, s) : launch_fused_bf16<128>(a, s);
  }
  hipError_t e;
  int nwg = 1;
  if (a.in_bf16)
    e = a.d == 64 ? launch_split_bf16<64>(a, s, nwg) : launch_split_bf16<128>(a, s, nwg);
  else
    e = a.d == 64 ? launch_split_f32<64>(a, s) : launch_split_f32<128>(a, s);
  if (e != hipSuccess) return e;
  const int n_qblk = (a.Hq / a.Hkv + 15) / 16;
  const dim3 grid((unsigned)a.Hq, (unsigned)a.B);  // (query head, sequence)
#define MQKV_COMB(DD, OB)                                                                        \
  if (a.d == DD && a.out_bf16 == OB)                                                            \
    hipLaunchKernelGGL((attn_decode_combine_kernel<DD, OB>), grid, dim3(64), 0, s, a.seq_lens,   \
                       a.part_o, a.part_ml, a.o, a.lse, a.B, a.Hq, a.Hkv, a.Lmax, a.split, a.n_slot,   \
                       n_qblk, nwg);
  MQKV_COMB(64, true)
  MQKV_COMB(64, false)
  MQKV_COMB(128, true)
  MQKV_COMB(128, false)
#undef MQKV_COMB
  return hipGetLastError();
}

}  // namespace mqkv
