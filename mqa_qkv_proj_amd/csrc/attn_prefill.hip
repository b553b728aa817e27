// Grouped-query attention prefill for gfx950: tiled exact attention with an
// online softmax.
//
// What is computed: O = softmax(scale . Q K^T) V per query head, where query
// head h reads KV head h / (H_q/H_kv) ("MHA -> GQA" blog, section 3.2), with an
// optional bottom-right causal mask.  Tiling the keys and rescaling the
// running softmax state gives the exact result with memory linear in the
// sequence length (FlashAttention-3 page, "FlashAttention recap").
//
// Design (bf16 inputs, CDNA4 wave64, MFMA 32x32x16):
//  * One workgroup = 8 waves = 256 query rows of one KV head: F query heads of
//    the group x (256/F) positions, F = the largest power of two dividing
//    G = H_q/H_kv (at most 32).  Every LDS K/V tile is reused by all F heads.
//    d=64 grids use 4-wave workgroups (128 rows), three per CU.
//  * Scores are computed transposed, S^T = K . Q^T: the accumulator then holds
//    one query per lane column, so the row max and row sum are in-lane
//    reductions plus one exchange with the lane 32 away.  Q stays in VGPRs.
//  * exp2 form of the softmax: p = exp2(S*c - m), c = scale*log2(e), one FMA
//    per score.  The running max is only raised when a row's max grows by more
//    than 8 (log2 units); until then p <= 2^8, which keeps fp32 sums exact in
//    form and skips most accumulator rescales.
//  * P is rounded to fp16 and O^T += V^T . P^T runs as an fp16 MFMA.  fp16 P
//    carries 3 more mantissa bits than bf16, which keeps the error of
//    outlier-heavy rows inside the bf16 tolerance.  A small pre-pass writes V
//    once as fp16 V^T tile images, in the key order the P operand holds, into
//    caller-provided workspace.  Each image carries a power-of-two exponent
//    (0 for values inside fp16's range) so the conversion is exact for every
//    finite bf16 V; the accumulator follows it with exact rescales.
//  * Software pipeline over 32-key halves: the softmax of one half runs on the
//    vector unit while the matrix cores compute the next half's scores and
//    this half's P.V; the operands of each MFMA are read from LDS one slot
//    ahead.  The pipeline runs across tile boundaries: three LDS stages hold
//    the tile being consumed, the next tile (complete) and the tile being
//    copied in, with one barrier per 64-key tile.
//  * Tiles reach LDS by LDS-DMA (buffer loads that write LDS directly): no
//    staging registers and no LDS store instructions.  d=128 K rows keep 16
//    bytes of padding per row (the pad lanes of a copy point past the buffer,
//    so they fetch nothing and land only on padding) so that the operand reads
//    of 16 consecutive rows hit distinct banks; d=64 K rows are unpadded with
//    their 16-byte chunks swizzled to the same effect; the V^T images carry
//    padding.  The copies are issued by the four older waves, between the
//    MFMAs of the pipelined steps.
//  * Causal: tiles beyond the block's diagonal are never visited, only tiles
//    that cross a row's limit are masked (a separate, unpipelined loop), and
//    the heaviest query blocks are dispatched first.  Workgroup ids are
//    remapped so that each XCD serves a contiguous range of (batch, KV head)
//    blocks and keeps their K/V in its L2.
//  * Packed batches of unequal lengths (with a workspace that holds a
//    schedule): one workgroup of the V-image pre-pass lists the row blocks of
//    the whole batch heaviest first, and persistent workgroups claim them in
//    that order with an atomic counter (FlashAttention-3 page, closing
//    section: persistent kernels, variable length).
// fp32 inputs use a plain one-row-per-thread kernel (fp32 throughout).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mqkv {

namespace {

constexpr int kWaves = 8;           // waves per workgroup (32 query rows each)
constexpr int kThreads = kWaves * 64;
constexpr int kRows = kWaves * 32;  // query rows per workgroup
constexpr int kBK = 64;             // keys per K/V tile: two 32-key halves
constexpr int kStages = 3;          // K/V tiles resident in LDS
constexpr float kTau = 8.0f;        // lazy-rescale threshold (log2 units)
// Row-block schedule of a packed batch (persistent workers): kSchedHdr header
// words (number of row blocks listed, claim counter, two unused), then one
// (sequence, query block) pair of int32 per row block, heaviest first.
constexpr int kSchedHdr = 4;
constexpr int kPlanMaxB = 1024;  // sequences a schedule is planned for
constexpr int kPlanBins = 1024;  // cost classes of the counting sort

// LDS image of one K/V tile.  Rows carry 16 bytes of padding, which keeps the
// MFMA operand reads of 16 consecutive rows on distinct banks.  LDS-DMA copies
// 1 KB per instruction (64 lanes x 16 bytes, lane-linear), so each image is a
// whole number of copies.
template <int D, bool F8 = false>
struct PrefillLds {
  // K row pitch in 16-bit units: bf16 rows of D + 8 elements, or (F8) e4m3 rows
  // of D + 16 bytes whose padding also carries the tile's quantisation scale.
  // d = 64 bf16 rows carry no padding: their 16-byte chunks are swizzled
  // instead (kSwizzle), which keeps a stage at 17 KB so that three 4-wave
  // workgroups share a CU's LDS.
  static constexpr bool kSwizzle = D == 64 && !F8;
  static constexpr int kKld = F8 ? (D + 16) / 2 : kSwizzle ? D : D + 8;
  static constexpr int kVld = kBK + 8;  // V^T row pitch (fp16 elements)
  static constexpr int kK = kBK * kKld;
  static constexpr int kV = D * kVld;
  static constexpr int kStage = kK + kV;
  static constexpr size_t kBytes = kStages * kStage * sizeof(uint16_t);
  static constexpr int kKChunks = kKld / 8;  // 16-byte chunks per K row, padding included
  // Position of chunk c of K row r in its LDS row (kSwizzle): c ^ ((r / 2) % 8).
  // The 16 rows that one 16-lane pass of a ds_read_b128 reads (rows r0 .. r0+15,
  // one chunk each) then cover all 16 16-byte bank groups: a 128-byte row
  // spans 8 groups, so group = 8 (r % 2) + position, and positions differ for
  // the 8 rows of each parity.
  static __device__ __forceinline__ int kpos(int r, int c) { return kSwizzle ? c ^ ((r >> 1) & 7) : c; }
  static constexpr int kKCopies = kK * 2 / 1024;
  static constexpr int kVCopies = kV * 2 / 1024;
  static_assert(kK * 2 % 1024 == 0 && kV * 2 % 1024 == 0, "tile images are whole 1 KB copies");
};

// Position, inside a 16-key group, of key 4a + j (a = 0..3) in the V^T rows:
// keys {0-3, 8-11} first (lane half 0 of the P operand), then {4-7, 12-15}.
__device__ __forceinline__ int vt_pos(int a) { return ((a & 1) << 3) | ((a >> 1) << 2); }

// Rows and lengths of sequence b: b-major fixed lengths, or the packed
// variable-length layout (cu_q == nullptr selects the former).  Packed offsets
// and lengths are clamped to the buffers and to the maximum lengths the grid
// was sized for, so no value of the device-side offsets leads outside them.
struct SeqSpan {
  int64_t q0, kv0;  // first row of the sequence in q / o and in k / v
  int Lq, Lkv;
};
__device__ __forceinline__ SeqSpan seq_span(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
                                            int b, int Lq, int Lkv, int total_q, int total_kv) {
  if (cu_q == nullptr) return SeqSpan{(int64_t)b * Lq, (int64_t)b * Lkv, Lq, Lkv};
  const int q0 = min(max(cu_q[b], 0), total_q), q1 = min(max(cu_q[b + 1], q0), total_q);
  const int k0 = min(max(cu_kv[b], 0), total_kv), k1 = min(max(cu_kv[b + 1], k0), total_kv);
  return SeqSpan{q0, k0, min(q1 - q0, Lq), min(k1 - k0, Lkv)};
}

// V of one (batch, KV head, 64-key tile) written as the LDS image the prefill
// kernel uses for P.V: V^T in fp16, one padded row per head dimension, keys in
// P-operand order.  The tile is stored as V * 2^-s with its power-of-two
// exponent s (v_tile_exp: 0 unless the tile lies beyond fp16's range or is
// entirely tiny), so the conversion is exact for every finite bf16 tile; s
// rides in row 0's padding (int32 at element kBK).  Keys at or past L_kv are
// zeros, so every image is a full tile.  Called by all (kBK/4)*(D/8) threads of
// the workgroup, task ti each (a workgroup barrier inside); `red` is LDS for
// one int per wave.
template <int D>
__device__ __forceinline__ void v_image_tile(const uint16_t* __restrict__ v, uint16_t* __restrict__ img, int Hkv,
                                             int64_t kv_stride, int ntiles, int b, int g, int t, const SeqSpan& sp,
                                             int ti, uint32_t* red) {
  using S = PrefillLds<D>;
  constexpr int NW = (kBK / 4) * (D / 8) / 64;  // waves taking part
  // consecutive lanes take consecutive key groups: one store instruction then
  // covers whole image rows
  const int kg = ti % (kBK / 4), dg = ti / (kBK / 4);
  const uint32_t kv_bytes = (uint32_t)((int64_t)sp.Lkv * kv_stride * 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(v + sp.kv0 * kv_stride, kv_bytes);
  const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
  u32x4_t rv[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    rv[jj] = bld16(rs, (uint32_t)(t * kBK + kg * 4 + jj) * row_bytes + (uint32_t)(g * D * 2) + dg * 16);
  // the tile's largest exponent field: per lane, per wave, then over the waves
  uint32_t em = 0;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int e = 0; e < 4; ++e) em = max(em, bf16x2_expmax(rv[jj][e]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) em = max(em, (uint32_t)__shfl_xor((int)em, o, 64));
  if ((ti & 63) == 0) red[ti >> 6] = em;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) em = max(em, red[w]);
  const int sv = v_tile_exp(em);
  auto cv = [&](float x) { return __builtin_amdgcn_ldexpf(x, -sv); };
  uint16_t* out = img + (((int64_t)b * Hkv + g) * ntiles + t) * S::kV;
  const int col = (kg >> 2) * 16 + vt_pos(kg & 3);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // rv[jj][e] = V[key jj][d = 8dg+2e, 8dg+2e+1] (bf16 pair)
    u32x2_t lo, hi;
    lo[0] = pack_f16(cv(bf16lo(rv[0][e])), cv(bf16lo(rv[1][e])));
    lo[1] = pack_f16(cv(bf16lo(rv[2][e])), cv(bf16lo(rv[3][e])));
    hi[0] = pack_f16(cv(bf16hi(rv[0][e])), cv(bf16hi(rv[1][e])));
    hi[1] = pack_f16(cv(bf16hi(rv[2][e])), cv(bf16hi(rv[3][e])));
    st8(out + (dg * 8 + 2 * e) * S::kVld + col, lo);
    st8(out + (dg * 8 + 2 * e + 1) * S::kVld + col, hi);
  }
  if (ti == 0) *reinterpret_cast<int32_t*>(out + kBK) = sv;
}

// What the planning workgroup of a packed batch needs (persistent schedule).
struct PlanArgs {
  const int32_t* cu_q;
  int32_t* sched;  // kSchedHdr words, then `cap` (sequence, query block) pairs
  int B, Lq_max, total_q;
  int P;       // query positions per row block
  int causal;
  int shift;   // cost class = key tiles >> shift (fits kPlanBins)
  int cap;     // row blocks the list holds
};

// Key tiles that row block qb of a sequence with lq queries and lkv keys runs
// (the attention kernel's own count: causal blocks stop at their last row's
// limit).
__device__ __forceinline__ int block_tiles(int lq, int lkv, int qb, int P, int causal) {
  int kv_end = lkv;
  if (causal) kv_end = min(lkv, min(qb * P + P, lq) - 1 + (lkv - lq) + 1);
  return kv_end > 0 ? (kv_end + kBK - 1) / kBK : 0;
}

// Exclusive prefix sum of one value per thread over the workgroup (T threads,
// buf holds T ints); `total` receives the sum of all.
__device__ __forceinline__ int block_exclusive_scan(int v, int* buf, int tid, int T, int& total) {
  buf[tid] = v;
  __syncthreads();
  for (int o = 1; o < T; o <<= 1) {
    const int x = tid >= o ? buf[tid - o] : 0;
    __syncthreads();
    buf[tid] += x;
    __syncthreads();
  }
  total = buf[T - 1];
  const int incl = buf[tid];
  __syncthreads();
  return incl - v;
}

// The schedule of a packed batch: every (sequence, query block) row block with
// at least one query row, sorted by the key tiles it runs, most first (a
// counting sort over kPlanBins cost classes; the order inside a class is
// arbitrary).  Longest-processing-time-first order: the workers that take the
// list in order finish together up to the last blocks, the lightest.  Run by
// one workgroup of T threads; at most kPlanMaxB sequences.
__device__ void plan_row_blocks(const PlanArgs& a, const int32_t* __restrict__ cu_kv, int Lkv_max, int total_kv,
                                int tid, int T) {
  __shared__ int first[kPlanMaxB], lq_of[kPlanMaxB], lkv_of[kPlanMaxB], cls[kPlanBins], buf[256];
  const int B = a.B, P = a.P;
  // lengths and row blocks of each sequence; row block ids start at first[b]
  const int per = (B + T - 1) / T, b0 = tid * per;
  int mine = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < B) {
      const SeqSpan sp = seq_span(a.cu_q, cu_kv, b, a.Lq_max, Lkv_max, a.total_q, total_kv);
      lq_of[b] = sp.Lq;
      lkv_of[b] = sp.Lkv;
      mine += (sp.Lq + P - 1) / P;
    }
  }
  for (int i = tid; i < kPlanBins; i += T) cls[i] = 0;
  int n = 0;
  int at = block_exclusive_scan(mine, buf, tid, T, n);
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < B) {
      first[b] = at;
      at += (lq_of[b] + P - 1) / P;
    }
  }
  __syncthreads();
  // row block e -> (sequence, query block): the last sequence starting at or
  // before e (sequences without queries start where the next one does)
  auto locate = [&](int e, int& b, int& qb) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= e) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    qb = e - first[lo];
  };
  auto cost_class = [&](int b, int qb) {
    return min(block_tiles(lq_of[b], lkv_of[b], qb, P, a.causal) >> a.shift, kPlanBins - 1);
  };
  for (int e = tid; e < n; e += T) {
    int b, qb;
    locate(e, b, qb);
    atomicAdd(&cls[cost_class(b, qb)], 1);
  }
  __syncthreads();
  // first list slot of each class, the costliest class first: each thread
  // takes kPlanBins / T consecutive classes counted from the top
  const int cpt = kPlanBins / T;
  int cnt = 0;
  for (int i = 0; i < cpt; ++i) cnt += cls[kPlanBins - 1 - (tid * cpt + i)];
  int unused = 0;
  int slot = block_exclusive_scan(cnt, buf, tid, T, unused);
  for (int i = 0; i < cpt; ++i) {
    const int c = kPlanBins - 1 - (tid * cpt + i);
    const int k = cls[c];
    cls[c] = slot;
    slot += k;
  }
  __syncthreads();
  int2* list = reinterpret_cast<int2*>(a.sched + kSchedHdr);
  for (int e = tid; e < n; e += T) {
    int b, qb;
    locate(e, b, qb);
    const int at_list = atomicAdd(&cls[cost_class(b, qb)], 1);
    if (at_list < a.cap) list[at_list] = int2{b, qb};
  }
  if (tid == 0) {
    a.sched[0] = min(n, a.cap);
    a.sched[1] = 0;  // claim counter
  }
}

// PLAN: workgroup 0 plans the row-block schedule of a packed batch; the
// others write the V images (workgroup i: image i - 1).
template <int D, bool PLAN = false>
__global__ __launch_bounds__((kBK / 4) * (D / 8)) void prefill_v_image_kernel(
    const uint16_t* __restrict__ v, uint16_t* __restrict__ img, int Lkv, int Hkv, int64_t kv_stride, int ntiles,
    const int32_t* __restrict__ cu_kv, int total_kv, PlanArgs plan) {
  __shared__ uint32_t red[4];
  const int ti = threadIdx.x;  // one task of 4 keys x 8 dimensions per thread
  int id = blockIdx.x;
  if constexpr (PLAN) {
    if (id == 0) {
      plan_row_blocks(plan, cu_kv, Lkv, total_kv, ti, (int)blockDim.x);
      return;
    }
    --id;
  }
  const int t = id % ntiles;
  id /= ntiles;
  const int g = id % Hkv;
  const int b = id / Hkv;
  const SeqSpan sp = seq_span(cu_kv, cu_kv, b, Lkv, Lkv, total_kv, total_kv);
  if (t * kBK >= sp.Lkv) return;  // a tile no query of this sequence reads (the whole workgroup)
  v_image_tile<D>(v, img, Hkv, kv_stride, ntiles, b, g, t, sp, ti, red);
}

// ---- FP8 (e4m3) quantisation with incoherent processing ("FlashAttention-3"
// page, FP8 section): a random orthogonal matrix, here a Hadamard transform
// with random signs, spreads outlier features of Q and K before the cast.
// The transform is the fast Walsh-Hadamard butterfly: stage `st` pairs
// elements i and i ^ st (a + b to the lower index, a - b to the upper); the
// stages commute, so each layout below runs them in whatever order its
// element-to-lane mapping makes cheapest.

__device__ __forceinline__ void bfly(float& lo, float& hi) {
  const float a = lo, b = hi;
  lo = a + b;
  hi = a - b;
}
// The butterfly with the partner element held by lane ^ lm (`upper`: this lane
// holds the upper index).
__device__ __forceinline__ float bfly_x(float x, int lm, bool upper) {
  const float y = __shfl_xor(x, lm, 64);
  return upper ? y - x : x + y;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Code of x / s (a correctly rounded fp32 division, so the rounding decision
// is a function of the fp32 values alone) after saturating to +-448 (the
// conversion gives NaN past the range); round to nearest even.  Four values
// to one dword, first value in the low byte.
__device__ __forceinline__ uint32_t e4m3x4(float x0, float x1, float x2, float x3, float s) {
  auto sat = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(x0 / s), sat(x1 / s), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(x2 / s), sat(x3 / s), lo, true);
}

// One Q row (D = 128) inside the attention kernel, where the lane pair
// (l, l ^ 32) owns the row: the lane with half hf holds the elements
// 64a + 32hf + j (a < D/64, j < 32), exactly the bytes of the fp8 MFMA B
// operand it supplies.  Loads the bf16 row, applies the map (signs != nullptr),
// and returns the fragments qf[2a + c] = bytes 64a + 32hf + 16c.. and the
// row's scale max |q'| / 448 (1 for an all-zero or absent row).
template <int D>
__device__ __forceinline__ float q_row_fp8(const uint16_t* __restrict__ qp, bool valid,
                                           const float* __restrict__ signs, int hf, u32x4_t (&qf)[D / 32]) {
  constexpr int A = D / 64;
  float x[A][32];
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t w = valid ? ld16(qp + 64 * a + 32 * hf + 8 * c) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[a][8 * c + 2 * e] = bf16lo(w[e]);
        x[a][8 * c + 2 * e + 1] = bf16hi(w[e]);
      }
    }
  if (signs != nullptr) {
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32x4_t sg = ld16(signs + 64 * a + 32 * hf + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[a][4 * c + e] *= __uint_as_float(sg[e]);
      }
#pragma unroll
    for (int st = 1; st < 32; st <<= 1)  // index bits 0..4: inside the lane
#pragma unroll
      for (int a = 0; a < A; ++a)
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if ((j & st) == 0) bfly(x[a][j], x[a][j + st]);
#pragma unroll
    for (int a = 0; a < A; ++a)  // index bit 5: across the lane pair
#pragma unroll
      for (int j = 0; j < 32; ++j) x[a][j] = bfly_x(x[a][j], 32, hf != 0);
#pragma unroll
    for (int sa = 1; sa < A; sa <<= 1)  // index bits 6..: across the a blocks
#pragma unroll
      for (int a = 0; a < A; ++a)
        if ((a & sa) == 0)
#pragma unroll
          for (int j = 0; j < 32; ++j) bfly(x[a][j], x[a + sa][j]);
    const float nrm = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
      for (int j = 0; j < 32; ++j) x[a][j] *= nrm;
  }
  float am = 0.0f;
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int j = 0; j < 32; ++j) am = fmaxf(am, fabsf(x[a][j]));
  am = fmaxf(am, __shfl_xor(am, 32, 64));
  const float s = am > 0.0f ? am / 448.0f : 1.0f;
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int j = 16 * c + 4 * w;
        qf[2 * a + c][w] = e4m3x4(x[a][j], x[a][j + 1], x[a][j + 2], x[a][j + 3], s);
      }
  return s;
}

// K and V of one (batch, KV head, 64-key tile) of an FP8 call, one pass over
// both: V as the fp16 image of the bf16 path, K as the e4m3 LDS image the
// attention kernel copies: 64 rows of D code bytes + 16 bytes of padding, with
// the tile's scale (max |k'| over the tile / 448) in row 0's padding.  Keys at
// or past L_kv are zero rows.  A K row is held by 16 lanes, 8 elements each
// (element 8(l % 16) + e); a wave covers 4 rows per 16-byte load and takes 16
// rows in 4 loads, all in flight together.
template <int D>
__global__ __launch_bounds__(256) void prefill_fp8_kv_kernel(const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v, int Lkv, int Hkv,
                                                             int64_t kv_stride, const float* __restrict__ signs,
                                                             uint8_t* __restrict__ k8img, uint16_t* __restrict__ vimg,
                                                             int ntiles) {
  static_assert(D == 128, "16 lanes of 8 elements per K row");
  constexpr int kPitch = D + 16, kPass = 4;
  __shared__ float wmax[4];
  __shared__ uint32_t vred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15;  // element block 8 li .. 8 li + 7 of a row
  int id = blockIdx.x;
  const int t = id % ntiles;
  id /= ntiles;
  const int g = id % Hkv;
  const int b = id / Hkv;
  const SeqSpan sp{(int64_t)b * Lkv, (int64_t)b * Lkv, Lkv, Lkv};
  const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(k + sp.kv0 * kv_stride, (uint32_t)((int64_t)Lkv * kv_stride * 2));  // rows >= L_kv read 0
  u32x4_t raw[kPass];
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const int r = wave * 16 + p * 4 + (lane >> 4);
    raw[p] = bld16(rs, (uint32_t)(t * kBK + r) * row_bytes + (uint32_t)(g * D * 2) + li * 16);
  }
  v_image_tile<D>(v, vimg, Hkv, kv_stride, ntiles, b, g, t, sp, tid, vred);
  float x[kPass][8];
#pragma unroll
  for (int p = 0; p < kPass; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[p][2 * e] = bf16lo(raw[p][e]);
      x[p][2 * e + 1] = bf16hi(raw[p][e]);
    }
  if (signs != nullptr) {
    const u32x4_t s0 = ld16(signs + 8 * li), s1 = ld16(signs + 8 * li + 4);
#pragma unroll
    for (int p = 0; p < kPass; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[p][e] *= __uint_as_float(s0[e]);
        x[p][4 + e] *= __uint_as_float(s1[e]);
      }
#pragma unroll
    for (int st = 1; st < 8; st <<= 1)  // index bits 0..2: inside the lane
#pragma unroll
      for (int p = 0; p < kPass; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & st) == 0) bfly(x[p][e], x[p][e + st]);
#pragma unroll
    for (int lm = 1; lm < 16; lm <<= 1)  // index bits 3..6: across the 16 lanes of the row
#pragma unroll
      for (int p = 0; p < kPass; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[p][e] = bfly_x(x[p][e], lm, (li & lm) != 0);
    const float nrm = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
    for (int p = 0; p < kPass; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[p][e] *= nrm;
  }
  float am = 0.0f;
#pragma unroll
  for (int p = 0; p < kPass; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[p][e]));
  am = wave_max(am);
  if (lane == 0) wmax[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = am > 0.0f ? am / 448.0f : 1.0f;
  uint8_t* img = k8img + (((int64_t)b * Hkv + g) * ntiles + t) * (kBK * kPitch);
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const int r = wave * 16 + p * 4 + (lane >> 4);
    st8(img + r * kPitch + li * 8, u32x2_t{e4m3x4(x[p][0], x[p][1], x[p][2], x[p][3], s),
                                           e4m3x4(x[p][4], x[p][5], x[p][6], x[p][7], s)});
  }
  if (wave == 0)  // the padding of row `lane`: the scale in row 0's, zeros elsewhere
    st16(img + lane * kPitch + D, u32x4_t{lane == 0 ? __float_as_uint(s) : 0u, 0u, 0u, 0u});
}

// s_waitcnt vmcnt(0) with the other counters left alone: the LDS-DMA copies a
// wave issued have landed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// F8: each lane pair quantises its Q row to e4m3 in the prologue (after the
// map with `signs`), K arrives as per-tile e4m3 LDS images k8img with the tile
// scale in row 0's padding, and the scores run on the fp8 MFMA 32x32x64; P and
// V are as in the bf16 path.
// PERSIST: the workgroups are persistent workers over the row-block list that
// plan_row_blocks wrote into `sched` (heaviest first).  Worker w runs unit w
// first; while a unit runs, its first lane claims the next one, gridDim.x plus
// the count taken from `claim` by one vector atomic, so every worker runs
// until the list is exhausted, whichever units it is handed.
template <int D, bool CAUSAL, bool OUT_BF16, bool F8 = false, int NW = kWaves, int KP = 1, bool PERSIST = false>
__global__ __launch_bounds__(NW * 64, KP == 1 ? 2 : 1) void attn_prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vimg,
    void* __restrict__ o, float* __restrict__ lse, int Lq_max, int Lkv_max, int Hq, int Hkv,
    int64_t q_stride, int64_t kv_stride, float c, int F, int n_hg, int n_qb, int ntiles,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv, int total_q, int total_kv,
    const float* __restrict__ signs, const uint8_t* __restrict__ k8img, const int32_t* __restrict__ sched,
    int32_t* __restrict__ claim) {
  using S = PrefillLds<D, F8>;
  constexpr int DS = D / 16;  // MFMA k-steps over the head dimension
  constexpr int KS8 = D / 64;  // fp8 MFMA k-steps (64 bytes each)
  constexpr int KF = F8 ? 2 * KS8 : DS;  // 16-byte operand fragments per row of a half
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  // KP key parities: the waves form NW/KP groups of 32 query rows, and the
  // wave of parity kp in a group takes the key tiles kp, kp + KP, ... of those
  // rows; the KP partial results of a row are merged at the end (exact
  // rescaling).  An LDS stage then holds KP consecutive tiles.
  constexpr int RG = NW / KP;  // 32-row groups per workgroup
  static_assert(NW % KP == 0 && (KP == 1 || !F8), "key parities");
  constexpr int kStageP = KP * PrefillLds<D, F8>::kStage;  // LDS stage: KP tiles
  // Tile copies are issued by the first kFillWaves waves only: the hardware
  // favours the older wave of the two that share a SIMD, so those waves run
  // ahead and would otherwise wait at the tile barrier.
  constexpr int kFillWaves = 4 < NW ? 4 : NW;
  constexpr int KCP = (S::kKCopies + kFillWaves - 1) / kFillWaves;  // K copies per filling wave
  constexpr int VCP = (S::kVCopies + kFillWaves - 1) / kFillWaves;  // V copies per filling wave
  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wq = __builtin_amdgcn_readfirstlane(wave);
  const int kp = wq / RG;  // this wave's key parity

  const int G = Hq / Hkv;
  const int P = RG * 32 / F;  // positions per workgroup
  // One unit: sequence b, KV head g, head group hg, query block qb.
  auto run_unit = [&](const int b, const int g, const int hg, const int qb) __attribute__((always_inline)) {
  const int p0 = qb * P;
  const SeqSpan sp = seq_span(cu_q, cu_kv, b, Lq_max, Lkv_max, total_q, total_kv);
  if (p0 >= sp.Lq) return;  // the whole workgroup: no query rows here (packed batches only)
  const int Lq = sp.Lq, Lkv = sp.Lkv;
  const int off = Lkv - Lq;

  // ---- this lane's query row (column of the S^T tile)
  const int r = (wave % RG) * 32 + l32;
  const int h = g * G + hg * F + r / P;
  const int pos = p0 + r % P;
  const bool valid = pos < Lq;
  const int lim = CAUSAL ? min(pos + off, Lkv - 1) : Lkv - 1;  // last visible key

  u32x4_t qf[KF];
  float crow = c;  // score scale of this lane's row (F8: times the row's quantisation scale)
  if constexpr (F8) {
    // B operand of the fp8 MFMA: column = this query row, bytes 64 s + 32 hf ..
    crow = c * q_row_fp8<D>(q + (sp.q0 + pos) * q_stride + (int64_t)h * D, valid, signs, hf, qf);
  } else {
    const uint16_t* qp = q + (sp.q0 + pos) * q_stride + (int64_t)h * D + hf * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = valid ? ld16(qp + s * 16) : u32x4_t{0, 0, 0, 0};
  }

  const int last_pos = min(p0 + P, Lq) - 1;
  const int kv_end = CAUSAL ? min(Lkv, last_pos + off + 1) : Lkv;
  const int mask_from = CAUSAL ? min(Lkv, p0 + off + 1) : Lkv;  // first key some row cannot see
  const int nt = (kv_end + kBK - 1) / kBK;

  // ---- tile copies (LDS-DMA, no registers): K straight from the K rows, with
  // the lanes that fall on row padding pointed past the buffer, so they fetch
  // nothing and land only on padding bytes, which are never read; V from its
  // prepared image.  Rows at or past L_kv are past the buffer end too: their
  // LDS rows (zeros or stale) only ever meet masked keys.
  const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
  const uint32_t kv_bytes = (uint32_t)((int64_t)Lkv * kv_stride * 2);
  const char* kbase = reinterpret_cast<const char*>(k + sp.kv0 * kv_stride);
  const uint16_t* vbase = vimg + ((int64_t)b * Hkv + g) * ntiles * S::kV;
  constexpr uint32_t kNoCopy = 0x80000000u;  // beyond any buffer (spans are below 2 GiB)
  uint32_t koff[KCP];
#pragma unroll
  for (int i = 0; i < KCP; ++i) {
    const int slot = (wave + i * kFillWaves) * 64 + lane;
    // this lane's 16 bytes land on LDS chunk position `pos` of row `row`; it
    // fetches the K chunk that belongs there
    const int row = slot / S::kKChunks, pos = slot % S::kKChunks;
    const int ch = S::kSwizzle ? S::kpos(row, pos) : pos;
    koff[i] = F8 ? (uint32_t)lane * 16
                 : ch < D / 8 ? (uint32_t)row * row_bytes + (uint32_t)(g * D * 2) + ch * 16 : kNoCopy;
  }
  const uint8_t* k8base = F8 ? k8img + ((int64_t)b * Hkv + g) * ntiles * (S::kK * 2) : nullptr;
  // The copy of a stage (tiles u KP .. u KP + KP - 1) is split into numbered
  // parts (per tile: K copies, then V copies) so that the pipelined steps can
  // issue them one at a time between MFMAs.
  constexpr int kTileParts = KCP + VCP;
  constexpr int kParts = KP * kTileParts;
  __amdgpu_buffer_rsrc_t krs[KP], vrs[KP];
  uint16_t* ks_dst[KP];
  uint16_t* vs_dst[KP];
  bool fill_on[KP];
  auto fill_begin = [&](int u, int st) {
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int t = u * KP + j;
      fill_on[j] = wq < kFillWaves && t < nt;
      ks_dst[j] = smem + st * kStageP + j * S::kStage;
      vs_dst[j] = ks_dst[j] + S::kK;
      const int tc = t < nt ? t : 0;  // descriptors of a tile that is not copied are never used
      if constexpr (F8) {
        krs[j] = make_rsrc(k8base + (int64_t)tc * (S::kK * 2), S::kK * 2);
      } else {
        const uint32_t k0b = (uint32_t)(tc * kBK) * row_bytes;
        krs[j] = make_rsrc(kbase + k0b, kv_bytes - k0b);
      }
      vrs[j] = make_rsrc(vbase + (int64_t)tc * S::kV, S::kV * 2);
    }
  };
  auto fill_part = [&](auto part) {
    constexpr int j = part / kTileParts, i = part % kTileParts;
    if constexpr (j < KP) {
      if constexpr (i < KCP) {
        const int cp = wq + i * kFillWaves;
        if (fill_on[j] && cp < S::kKCopies) dma16(krs[j], ks_dst[j] + cp * 512, koff[i], F8 ? cp * 1024 : 0);
      } else {
        const int cp = wq + (i - KCP) * kFillWaves;
        if (fill_on[j] && cp < S::kVCopies) dma16(vrs[j], vs_dst[j] + cp * 512, (uint32_t)lane * 16, cp * 1024);
      }
    }
  };
  auto fill = [&](int u, int st) {
    fill_begin(u, st);
    static_for<0, kParts>([&](auto i) { fill_part(i); });
  };

  f32x16_t acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16_t{};
  float m_run = -INFINITY;  // running max of S*c (log2 units)
  float l_run = 0.0f;       // this lane's share of the running sum

  // this wave's tile in stage st
  auto k_of = [&](int st) -> const uint16_t* { return smem + st * kStageP + kp * S::kStage; };
  auto v_of = [&](int st) -> const uint16_t* { return smem + st * kStageP + kp * S::kStage + S::kK; };
  // The V tile in stage st is V * 2^-s with its exponent s in row 0's padding
  // (0 unless the tile lies outside fp16's range).  acc holds O * l * 2^-sig;
  // before a tile's P.V it is brought to that tile's exponent by an exact
  // power-of-two rescale.
  auto v_exp_of = [&](int st) -> int { return *reinterpret_cast<const int32_t*>(v_of(st) + kBK); };
  int sig = 0;
  auto v_rescale = [&](int sv_any) {
    const int sv = __builtin_amdgcn_readfirstlane(sv_any);
    if (sv != sig) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = __builtin_amdgcn_ldexpf(acc[i][e], sig - sv);
      sig = sv;
    }
  };
  // Scale of the scores of the tile in stage st (F8: the tile's K scale rides
  // in row 0's padding, bytes D..D+3).
  float cc = crow;
  auto tile_c = [&](int st) -> float {
    if constexpr (F8) return crow * *reinterpret_cast<const float*>(k_of(st) + D / 2);
    return crow;
  };
  // 16-byte fragment f of the MFMA A operand (key row r of a K stage):
  // bf16: k-step f; F8: bytes 64 (f/2) + 32 hf + 16 (f%2).
  auto kfrag = [&](const uint16_t* ks, int r, int f) -> u32x4_t {
    if constexpr (F8)
      return ld16(reinterpret_cast<const char*>(ks) + r * S::kKld * 2 + (f >> 1) * 64 + hf * 32 + (f & 1) * 16);
    if constexpr (S::kSwizzle) return ld16(ks + r * S::kKld + S::kpos(r, 2 * f + hf) * 8);
    return ld16(ks + r * S::kKld + f * 16 + hf * 8);
  };
  // score MFMA over fragments [f, f + 1] (F8) or fragment f (bf16)
  auto smfma = [&](const u32x4_t* kfr, int f, f32x16_t acc_s) -> f32x16_t {
    if constexpr (F8) return mfma32_f8(kfr[f], kfr[f + 1], qf[f], qf[f + 1], acc_s);
    return mfma32_bf16(kfr[f], qf[f], acc_s);
  };

  // S^T for the 32 keys [32j, 32j + 32) of the tile held in K rows `ks`.
  auto qk = [&](const uint16_t* ks, int j) {
    f32x16_t sc = f32x16_t{};
    u32x4_t kr[KF];
#pragma unroll
    for (int f = 0; f < KF; ++f) kr[f] = kfrag(ks, j * 32 + l32, f);
#pragma unroll
    for (int f = 0; f < KF; f += F8 ? 2 : 1) sc = smfma(kr, f, sc);
    return sc;
  };
  // Element i of a half starting at key kbase is key kbase + 8(i/4) + 4hf + (i%4);
  // keys past this row's limit get -inf.
  auto mask = [&](f32x16_t& sc, int kb) {
    const int rel = lim - kb - 4 * hf;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + (i & 3) > rel) sc[i] = -INFINITY;
  };
  // Row max of a half (log2 units).  The running max moves only when a row's
  // max grows by more than kTau, and then only for that row, so a row's result
  // does not depend on the other rows that share the wave.
  auto update_max = [&](const f32x16_t& sc) {
    float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
    mx = fmaxf(mx, sc[15]);
    mx = max_xor32(mx);
    const float mt = mx * cc;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kTau) != 0) {
      const float mn = (mt > m_run + kTau) ? mt : m_run;
      // a row whose max does not move keeps alpha = 1 (exp2(0) exactly), also when
      // it has seen no key yet (m = -inf, where the difference would be NaN)
      const float alpha = mn == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    }
  };
  // P = exp2(S*c - m) rounded to fp16 (the MFMA B operand), and its row sum.
  // A row that has seen no visible key yet (m = -inf, possible only in a packed
  // batch with L_q > L_kv under the causal mask) gets P = 0 rather than NaN.
  auto softmax = [&](const f32x16_t& sc, u32x4_t (&pf)[2]) {
    const float nm = m_run == -INFINITY ? 0.0f : -m_run;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e], cc, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e + 1], cc, nm));
        pf[hb][e] = pack_f16(p0, p1);
      }
    // row sum of the fp16-rounded P actually multiplied into V (fp32 accumulation)
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // copy the element out first: a bit_cast applied to a vector element
        // lvalue reads element 0 with this compiler
        const uint32_t w = pf[hb][e];
        l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), ones, l_run, false);
      }
  };
  // O^T += V^T P^T over the 32 keys [32j, 32j + 32) of the tile held in `vt`.
  auto pv = [&](const uint16_t* vt, int j, const u32x4_t (&pf)[2]) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      u32x4_t vf[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vf[db] = ld16(vt + (db * 32 + l32) * S::kVld + (j * 2 + hb) * 16 + hf * 8);
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma32_f16(vf[db], pf[hb], acc[db]);
    }
  };
  // K fragments (MFMA A operand) of the 32 keys [32j, 32j + 32) of a tile.
  auto load_kf = [&](u32x4_t (&kf)[KF], const uint16_t* ks, int j) {
    static_for<0, KF>([&](auto f) { kf[f] = kfrag(ks, j * 32 + l32, f); });
  };
  // One pipelined step.  On entry `sc` holds the scores of the current half
  // and `kf` the K fragments of the next half.  The step turns `sc` into P,
  // computes the next half's scores into `sc`, adds P V for the current half
  // (V^T `vc`, keys 32jc..) and, when NEXT, reads the K fragments of the half
  // after that (`kn`, keys 32jn..) into `kf`.  The source order is the issue
  // order: each score MFMA is followed by one V read and exponentials, each
  // P.V MFMA by a row-sum step and one K read, so the vector and LDS units
  // work while the matrix cores run and every operand is in flight long
  // before it is used.  Fences keep the compiler from regrouping.
  // With bf16 scores (SPREAD) a half's exponentials are split between two
  // steps: those of its first 16 keys are computed under the previous step's
  // P.V MFMAs (carried in `pl`, their max in `ml`, with the half's score scale
  // `cn`), the rest under its own score MFMAs, which spreads the vector work
  // evenly under the matrix work (measured 1-3% faster at d = 128, and 1-3% at
  // d = 64 with three workgroups per CU, where two per CU had made it 6%
  // slower).  With fp8 scores (two MFMAs per step) every exponential of the
  // half follows the score MFMAs: the split measured 8% slower there.
  // P is computed with the running max as it stands, while the half's row max
  // is folded in beside it; only if some row's max grew by more than kTau
  // (rare after the first half) is the max raised, O and l rescaled and P
  // recomputed, before any of P is used.  So the exponentials do not wait for
  // the max reduction, and every one of them uses the running max that holds
  // when the half's P is consumed.
  auto step = [&](f32x16_t& sc, u32x4_t& pl, float& ml, u32x4_t (&kf)[KF], const uint16_t* vc, int jc,
                  const uint16_t* kn, int jn, float cn, auto next_tag, auto part0) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr int PART0 = part0;
    constexpr bool SPREAD = !F8;
    u32x4_t pf[2];
    u32x4_t vf[2 * DB];
    f32x16_t sn = f32x16_t{};
    float mx = SPREAD ? ml : sc[0];
    if constexpr (SPREAD) pf[0] = pl;
    static_for<0, 8>([&](auto i) {
      if constexpr (!SPREAD) {  // all 16 pairs of the current half, one per slot
        constexpr int hb = i >> 2, e = i & 3;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e], cc, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e + 1], cc, -m_run));
        pf[hb][e] = pack_f16(p0, p1);
        mx = fmaxf(fmaxf(mx, sc[hb * 8 + 2 * e]), sc[hb * 8 + 2 * e + 1]);
      }
      if constexpr (F8) {
        if constexpr (i % (8 / KS8) == 0) sn = smfma(kf, 2 * (i / (8 / KS8)), sn);
      } else if constexpr (i < DS) {
        sn = smfma(kf, i, sn);
      }
      if constexpr (SPREAD && i % 2 == 1) {  // keys 16.. of the current half: one pair every other slot
        constexpr int e = i / 2;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 + 2 * e], cc, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 + 2 * e + 1], cc, -m_run));
        pf[1][e] = pack_f16(p0, p1);
        // keep the exponentials here: the compiler would otherwise sink them past
        // the max check into its no-rescale branch, away from the MFMAs
        asm volatile("" ::"v"(pf[1][e]));
        mx = fmaxf(fmaxf(mx, sc[8 + 2 * e]), sc[8 + 2 * e + 1]);
      }
      if constexpr (i < 2 * DB)
        vf[i] = ld16(vc + ((i % DB) * 32 + l32) * S::kVld + (jc * 2 + i / DB) * 16 + hf * 8);
      __builtin_amdgcn_sched_barrier(0);
    });
    mx = max_xor32(mx);
    const float mt = mx * cc;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kTau) != 0) {
      const float mn = (mt > m_run + kTau) ? mt : m_run;
      // a row whose max does not move keeps alpha = 1 (exp2(0) exactly), also when
      // it has seen no key yet (m = -inf, where the difference would be NaN)
      const float alpha = mn == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e], cc, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e + 1], cc, -m_run));
          pf[hb][e] = pack_f16(p0, p1);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    if constexpr (SPREAD) ml = -INFINITY;
    static_for<0, 2 * DB>([&](auto i) {
      constexpr int hb = i / DB, db = i % DB;
      acc[db] = mfma32_f16(vf[i], pf[hb], acc[db]);
      static_for<db * 4 / DB, (db + 1) * 4 / DB>([&](auto e) {
        const uint32_t w = pf[hb][(int)e];
        l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), ones, l_run, false);
      });
      if constexpr (NEXT && i < KF) kf[i] = kfrag(kn, jn * 32 + l32, i);
      if constexpr (PART0 >= 0) fill_part(std::integral_constant<int, PART0 + i>{});
      // keys 0..15 of the next half, spread over the P.V MFMAs
      if constexpr (SPREAD) static_for<i * 4 / (2 * DB), (i + 1) * 4 / (2 * DB)>([&](auto e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sn[2 * e], cn, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sn[2 * e + 1], cn, -m_run));
        pl[(int)e] = pack_f16(p0, p1);
        ml = fmaxf(fmaxf(ml, sn[2 * e]), sn[2 * e + 1]);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    sc = sn;
  };
  // The P of keys 0..15 of the half held in `s` (and their max), as the
  // SPREAD step carries it from one step to the next.
  auto first_p = [&](const f32x16_t& s, u32x4_t& plq, float& mlq) {
    mlq = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e], cc, -m_run));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e + 1], cc, -m_run));
      plq[e] = pack_f16(p0, p1);
      mlq = fmaxf(fmaxf(mlq, s[2 * e]), s[2 * e + 1]);
    }
  };
  // Last step of the pipeline: P V for the current half only.
  auto drain = [&](const f32x16_t& sc, const uint16_t* vc, int jc) {
    u32x4_t pf[2];
    softmax(sc, pf);
    pv(vc, jc, pf);
  };

  // Three LDS stages: while tile t is consumed, tile t + 1 is complete in LDS
  // (its first scores are computed under tile t's second half) and tile t + 2
  // is being copied in.  One barrier per tile publishes the copy.  With KP key
  // parities the stages hold KP tiles each and this wave's tiles are
  // kp, kp + KP, ...; every wave passes the same nu barriers.
  const int nu = (nt + KP - 1) / KP;
  fill(0, 0);
  if (nu > 1) fill(1, 1);
  wait_dma();
  __syncthreads();

  // Tiles below every row's causal limit run software-pipelined: the softmax of
  // one 32-key half is computed while the scores of the next half and the
  // P.V products of this half are in the matrix cores.
  const int t_mask = min(nt, mask_from / kBK);
  const int tm = t_mask > kp ? (t_mask - kp + KP - 1) / KP : 0;  // this wave's unmasked tiles
  const int ntw = nt > kp ? (nt - kp + KP - 1) / KP : 0;         // all of this wave's tiles
  int u = 0, st0 = 0;
  f32x16_t sc = f32x16_t{};
  u32x4_t pf[2];
  u32x4_t kf[KF];
  u32x4_t pl = u32x4_t{0, 0, 0, 0};  // the step's carried P of keys 0..15 of the current half
  float ml = -INFINITY;
  int sv_cur = v_exp_of(0);  // V exponent of this wave's current tile (read one tile ahead)
  if (tm > 0) {
    cc = tile_c(0);
    sc = qk(k_of(0), 0);
    update_max(sc);
    if constexpr (!F8) first_p(sc, pl, ml);
    load_kf(kf, k_of(0), 1);
  }
  for (; u + 1 < tm; ++u) {
    const int st1 = st0 == 2 ? 0 : st0 + 1;
    const int st2 = st1 == 2 ? 0 : st1 + 1;
    fill_begin(u + 2, st2);
    // d = 128: the younger wave of each SIMD (waves NW/2..) issues first in the
    // step after the barrier, so the pair leaves it out of phase rather than
    // contending for the matrix core together (1% on the long-context
    // prefill; at d = 64 it measured 1% slower)
    if constexpr (D == 128) {
      if (wave >= NW / 2) __builtin_amdgcn_s_setprio(3);
    }
    cc = tile_c(st0);
    v_rescale(sv_cur);
    sv_cur = v_exp_of(st1);  // this wave's next tile is complete in LDS
    // the second step computes the scores of the next tile (stage st1), under that tile's scale
    step(sc, pl, ml, kf, v_of(st0), 0, k_of(st1), 0, cc, std::true_type{}, std::integral_constant<int, 0>{});
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
    step(sc, pl, ml, kf, v_of(st0), 1, k_of(st1), 1, tile_c(st1), std::true_type{},
         std::integral_constant<int, 2 * DB>{});
    static_for<4 * DB, kParts>([&](auto i) { fill_part(i); });
    wait_dma();
    __syncthreads();
    st0 = st1;
  }
  if (u < tm) {  // last unmasked tile: the pipeline drains
    const int st1 = st0 == 2 ? 0 : st0 + 1;
    const int st2 = st1 == 2 ? 0 : st1 + 1;
    if (u + 2 < nu) fill(u + 2, st2);
    cc = tile_c(st0);
    v_rescale(sv_cur);
    step(sc, pl, ml, kf, v_of(st0), 0, k_of(st1), 0, cc, std::false_type{}, std::integral_constant<int, -1>{});
    update_max(sc);
    drain(sc, v_of(st0), 1);
    wait_dma();
    __syncthreads();
    st0 = st1;
    ++u;
  }
  // Tiles that cross some row's limit (at most a few per workgroup): masked,
  // one half after the other.
  for (; u < ntw; ++u) {
    const int st1 = st0 == 2 ? 0 : st0 + 1;
    const int st2 = st1 == 2 ? 0 : st1 + 1;
    if (u + 2 < nu) fill(u + 2, st2);
    cc = tile_c(st0);
    v_rescale(v_exp_of(st0));
    const int t = u * KP + kp;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sc = qk(k_of(st0), j);
      mask(sc, t * kBK + 32 * j);
      update_max(sc);
      softmax(sc, pf);
      pv(v_of(st0), j, pf);
    }
    wait_dma();
    __syncthreads();
    st0 = st1;
  }
  // no tile of this wave left: keep the barrier cadence and the copies
  for (; u < nu; ++u) {
    const int st1 = st0 == 2 ? 0 : st0 + 1;
    const int st2 = st1 == 2 ? 0 : st1 + 1;
    if (u + 2 < nu) fill(u + 2, st2);
    wait_dma();
    __syncthreads();
    st0 = st1;
  }

  if constexpr (KP > 1) {
    // Merge the key parities of each row (the stages are free now): the wave
    // of parity 1 leaves its running max, sum, V exponent and accumulators in
    // LDS; the wave of parity 0 brings both to the larger max and exponent.
    static_assert(KP == 2, "two key parities");
    constexpr int kRec = DB * 16 + 3;  // floats per lane
    float* xr = reinterpret_cast<float*>(smem) + (wave % RG) * kRec * 64 + lane;
    if (kp == 1) {
      xr[0] = m_run;
      xr[64] = l_run;
      xr[128] = __int_as_float(sig);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xr[(3 + db * 16 + e) * 64] = acc[db][e];
    }
    __syncthreads();
    if (kp == 1) return;
    const float m1 = xr[0], l1 = xr[64];
    const int s1 = __float_as_int(xr[128]);
    const float M = fmaxf(m_run, m1);
    // a side that has seen no key (max -inf) weighs 0, also when both have not
    const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
    const int Sx = max(sig, s1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc[db][e] = __builtin_amdgcn_ldexpf(acc[db][e] * a0, sig - Sx) +
                     __builtin_amdgcn_ldexpf(xr[(3 + db * 16 + e) * 64] * a1, s1 - Sx);
    l_run = l_run * a0 + l1 * a1;
    m_run = M;
    sig = Sx;
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  const float l_tot = l_run + xor32(l_run);
  if (!valid) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;  // a row that sees no key: O = 0
  const int64_t orow = ((sp.q0 + pos) * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + 8 * g4 + 4 * hf;
      // O = acc / l * 2^sig (exactly acc / l when sig = 0)
      auto ov = [&](float a) { return __builtin_amdgcn_ldexpf(a * inv, sig); };
      const float v0 = ov(acc[db][4 * g4 + 0]), v1 = ov(acc[db][4 * g4 + 1]);
      const float v2 = ov(acc[db][4 * g4 + 2]), v3 = ov(acc[db][4 * g4 + 3]);
      if constexpr (OUT_BF16) {
        u32x2_t pk;
        pk[0] = pack_bf16(v0, v1);
        pk[1] = pack_bf16(v2, v3);
        st8(static_cast<uint16_t*>(o) + orow + d0, pk);
      } else {
        st16(static_cast<float*>(o) + orow + d0,
             u32x4_t{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)});
      }
    }
  }
  if (lse != nullptr && hf == 0) {
    const int64_t li = cu_q != nullptr ? (int64_t)h * total_q + sp.q0 + pos : ((int64_t)b * Hq + h) * Lq + pos;
    lse[li] = (m_run + __builtin_log2f(l_tot)) * kLn2;
  }
  };

  if constexpr (!PERSIST) {
    // ---- block -> (b, g, head group, query block), heaviest causal blocks first
    int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = n_qb - 1 - (lid % n_qb);
    lid /= n_qb;
    const int hg = lid % n_hg;
    lid /= n_hg;
    const int g = lid % Hkv;
    const int b = lid / Hkv;
    run_unit(b, g, hg, qb);
  } else {
    // ---- persistent worker: unit u is row block u / HG of the list, KV head
    // and head group u % HG
    __shared__ int next_unit;
    const int HG = Hkv * n_hg;
    const int n_units = __builtin_amdgcn_readfirstlane(sched[0]) * HG;
    int unit = blockIdx.x;
    while (unit < n_units) {
      int nxt = 0;
      if (tid == 0) nxt = (int)gridDim.x + atomicAdd(claim, 1);  // read after the unit
      const int e = unit / HG, j = unit - e * HG;
      const int2 rb = reinterpret_cast<const int2*>(sched + kSchedHdr)[e];
      run_unit(__builtin_amdgcn_readfirstlane(rb.x), j / n_hg, j % n_hg, __builtin_amdgcn_readfirstlane(rb.y));
      __syncthreads();  // every wave is done with the unit's LDS
      if (tid == 0) next_unit = nxt;
      __syncthreads();
      unit = next_unit;
    }
  }
}

// ----------------------------------------------------------------------------- fp32 path
// One query row per thread, 64 rows per workgroup, K/V tiles of 32 keys in LDS.
template <int D>
__global__ __launch_bounds__(64) void attn_prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Lq, int Lkv, int Hq, int Hkv,
    int64_t q_stride, int64_t kv_stride, float scale, int causal) {
  constexpr int TK = 32;
  __shared__ float Ks[TK][D];
  __shared__ float Vs[TK][D];
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int pos = blockIdx.x * 64 + threadIdx.x;
  const bool valid = pos < Lq;
  const int off = Lkv - Lq;
  const int lim = causal ? min(pos + off, Lkv - 1) : Lkv - 1;
  const int blk_last = min((int)(blockIdx.x * 64 + 63), Lq - 1);
  const int kv_end = causal ? min(Lkv, blk_last + off + 1) : Lkv;

  float qr[D], acc[D];
  const float* qp = q + ((int64_t)b * Lq + (valid ? pos : 0)) * q_stride + (int64_t)h * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qr[i] = qp[i] * scale;
    acc[i] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int k0 = 0; k0 < kv_end; k0 += TK) {
    __syncthreads();
    for (int e = threadIdx.x; e < TK * D; e += 64) {
      const int key = e / D, dd = e % D;
      float kv = 0.0f, vv = 0.0f;
      if (k0 + key < Lkv) {
        const int64_t ro = ((int64_t)b * Lkv + k0 + key) * kv_stride + (int64_t)g * D + dd;
        kv = k[ro];
        vv = v[ro];
      }
      Ks[key][dd] = kv;
      Vs[key][dd] = vv;
    }
    __syncthreads();
    for (int j = 0; j < TK; ++j) {
      const int key = k0 + j;
      if (key > lim) break;
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) s = __builtin_fmaf(qr[i], Ks[j][i], s);
      const float mn = fmaxf(m, s);
      const float alpha = __expf(m - mn);
      const float p = __expf(s - mn);
      l = l * alpha + p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = __builtin_fmaf(p, Vs[j][i], acc[i] * alpha);
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = 1.0f / l;
  float* op = o + (((int64_t)b * Lq + pos) * Hq + h) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) op[i] = acc[i] * inv;
  if (lse) lse[((int64_t)b * Hq + h) * Lq + pos] = m + __logf(l);
}

// Row-block schedule of a packed batch: the workgroup shape its persistent
// workers use (d = 128: 8 waves; d = 64: 4 waves, two workgroups per CU),
// where the schedule sits in the workspace (after the V images) and its size.
struct VarlenSched {
  int nw, P;
  int64_t cap;   // row blocks the list holds
  size_t off;    // byte offset in the workspace
  size_t bytes;  // workspace bytes with the schedule; 0: no schedule possible
};
inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }
inline VarlenSched varlen_sched(int B, int Lkv_max, int total_q, int Hq, int Hkv, int d) {
  VarlenSched v{};
  if (B < 1 || B > kPlanMaxB || Lkv_max < 1 || total_q < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return v;
  if (d != 64 && d != 128) return v;
  const int G = Hq / Hkv;
  int F = 1;
  while (F < 32 && (G % (2 * F)) == 0) F *= 2;
  v.nw = d == 64 ? 4 : 8;
  v.P = v.nw * 32 / F;
  // sum over sequences of ceil(L_q / P) <= total_q / P + B
  v.cap = (int64_t)B + ((int64_t)total_q + v.P - 1) / v.P;
  if (v.cap * Hkv * (G / F) > 0x3fffffff) return v;
  v.off = round256(prefill_workspace_bytes(B, Lkv_max, Hkv, d, true));
  v.bytes = v.off + round256(sizeof(int32_t) * (kSchedHdr + 2 * v.cap));
  return v;
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_bf16_persistent(const PrefillArgs& a, hipStream_t s, const VarlenSched& vs, uint16_t* img,
                                  int ntiles, int F, int n_hg) {
  int32_t* sched = reinterpret_cast<int32_t*>(static_cast<char*>(a.ws) + vs.off);
  int shift = 0;
  while ((ntiles >> shift) >= kPlanBins) ++shift;
  const PlanArgs plan{a.cu_q, sched, a.B, a.Lq, a.total_q, vs.P, a.causal ? 1 : 0, shift, (int)vs.cap};
  const int64_t nimg = (int64_t)a.B * a.Hkv * ntiles;
  hipLaunchKernelGGL((prefill_v_image_kernel<D, true>), dim3((unsigned)(nimg + 1)), dim3((kBK / 4) * (D / 8)), 0,
                     s, (const uint16_t*)a.v, img, a.Lkv, a.Hkv, a.kv_stride, ntiles, a.cu_kv, a.total_kv, plan);
  constexpr int NWP = D == 64 ? 4 : 8;
  auto kern = attn_prefill_bf16_kernel<D, CAUSAL, OUT_BF16, false, NWP, 1, true>;
  const int threads = vs.nw * 64;
  const size_t lds = PrefillLds<D>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // one worker per resident workgroup slot, never more than the list can hold
  int dev = 0, cus = 0, per_cu = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, threads, lds);
  if (e != hipSuccess) return e;
  const int64_t units = vs.cap * a.Hkv * n_hg;
  const int64_t workers = std::min<int64_t>((int64_t)std::max(per_cu, 1) * cus, units);
  const float c = fmaxf(a.scale * kLog2e, 1e-30f);
  hipLaunchKernelGGL(kern, dim3((unsigned)workers), dim3(threads), lds, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, img, a.o, a.lse, a.Lq, a.Lkv, a.Hq, a.Hkv, a.q_stride, a.kv_stride, c, F,
                     n_hg, 0, ntiles, a.cu_q, a.cu_kv, a.total_q, a.total_kv, nullptr, nullptr, sched, sched + 1);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  int F = 1;
  while (F < 32 && (G % (2 * F)) == 0) F *= 2;
  const int n_hg = G / F;
  const int ntiles = (a.Lkv + kBK - 1) / kBK;
  auto grid = [&](int nw, int& n_qb) {
    const int P = nw * 32 / F;
    n_qb = (a.Lq + P - 1) / P;
    return (int64_t)a.B * a.Hkv * n_hg * n_qb;
  };
  int n_qb = 0;
  int64_t nblk = grid(kWaves, n_qb);
  // d=64 grids run 4-wave workgroups: three of them fit a CU (LDS 51 KB
  // each with the swizzled K rows, 149 VGPRs), twelve waves where one 8-wave
  // workgroup (149 VGPRs) leaves eight; with the heaviest causal blocks
  // dispatched first a CU also pairs heavy blocks with light ones, where an
  // 8-wave workgroup alone would hold the CU for the longest key range.  Each
  // row's arithmetic is the same either way (bit-identical outputs).
  // Measured against 8-wave workgroups on the TinyLlama-shaped prefills:
  // L = 2048 / 512 / 128 8-11% faster per call with two per CU; with three per
  // CU, B = 4 at L = 2048 and B = 8 at L = 1024 6% and 8% faster.
  int nw = kWaves, kp = 1;
  if (D == 64) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    nw = 4;
    // Fewer 128-row blocks than CUs: 8 waves per block, each row group's key
    // tiles split between two waves (even / odd tiles, merged at the end), so
    // the longest block finishes in half the steps on a CU that would
    // otherwise run it alone.  With more blocks than CUs the CUs are full
    // anyway and the merge and doubled copies only cost (measured: L = 512 and
    // 128 prefills 7% and 5% faster, L = 2048 7.5% slower with the split).
    if (nw == 4 && grid(4, n_qb) <= cus) kp = 2;
  }
  if (nw != kWaves) nblk = grid(nw, n_qb);
  const int64_t nimg = (int64_t)a.B * a.Hkv * ntiles;
  if (nblk > 0x7fffffff || nimg > 0x7fffffff) return hipErrorInvalidValue;
  if (a.ws_bytes < prefill_workspace_bytes(a.B, a.Lkv, a.Hkv, D, true)) return hipErrorInvalidValue;
  uint16_t* img = static_cast<uint16_t*>(a.ws);
  // A packed batch of unequal lengths whose workspace also holds a row-block
  // schedule runs on persistent workers that take the row blocks heaviest
  // first.  With every sequence at the maximum lengths the grid below already
  // runs the heaviest blocks first and keeps each (sequence, KV head) on one
  // XCD's L2, which measured 3-12% faster than the persistent workers there
  // (batches of one and two sequences); with unequal lengths the grid runs the
  // sequences one after another and leaves a long last sequence to a few XCDs
  // (measured 1.15-3x slower than the workers).
  const VarlenSched vs = varlen_sched(a.B, a.Lkv, a.total_q, a.Hq, a.Hkv, D);
  const bool equal = (int64_t)a.total_q == (int64_t)a.B * a.Lq && (int64_t)a.total_kv == (int64_t)a.B * a.Lkv;
  if (a.cu_q != nullptr && !equal && vs.bytes > 0 && a.ws_bytes >= vs.bytes)
    return launch_bf16_persistent<D, CAUSAL, OUT_BF16>(a, s, vs, img, ntiles, F, n_hg);
  hipLaunchKernelGGL(prefill_v_image_kernel<D>, dim3((unsigned)nimg), dim3((kBK / 4) * (D / 8)), 0, s,
                     (const uint16_t*)a.v, img, a.Lkv, a.Hkv, a.kv_stride, ntiles, a.cu_kv, a.total_kv,
                     PlanArgs{});
  auto kern = attn_prefill_bf16_kernel<D, CAUSAL, OUT_BF16, false, kWaves>;
  size_t lds = PrefillLds<D>::kBytes;
  int threads = kWaves * 64;
  if constexpr (D == 64) {
    if (nw == 4 && kp == 2) {  // 128 rows per workgroup: 4 row groups x 2 key parities
      kern = attn_prefill_bf16_kernel<D, CAUSAL, OUT_BF16, false, 8, 2>;
      lds = 2 * PrefillLds<D>::kBytes;
      threads = 8 * 64;
    } else if (nw == 4) {
      kern = attn_prefill_bf16_kernel<D, CAUSAL, OUT_BF16, false, 4>;
      threads = 4 * 64;
    }
  }
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // scale 0 is run as a tiny positive scale: masked scores stay -inf after the
  // multiply and every visible score maps to exp2(0) = 1 exactly.
  const float c = fmaxf(a.scale * kLog2e, 1e-30f);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(threads), lds, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, img, a.o, a.lse, a.Lq, a.Lkv, a.Hq, a.Hkv,
                     a.q_stride, a.kv_stride, c, F, n_hg, n_qb, ntiles, a.cu_q, a.cu_kv, a.total_q, a.total_kv,
                     nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

// Workspace of an FP8 call: the V images, then the K e4m3 tile images.
struct Fp8Ws {
  size_t v, k8, total;
};
inline Fp8Ws fp8_ws(int B, int Lkv, int Hkv, int d) {
  const int64_t ntiles = (Lkv + kBK - 1) / kBK;
  Fp8Ws w{};
  w.v = round256(prefill_workspace_bytes(B, Lkv, Hkv, d, true));
  w.k8 = round256((size_t)B * Hkv * ntiles * kBK * (d + 16));
  w.total = w.v + w.k8;
  return w;
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_fp8(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  int F = 1;
  while (F < 32 && (G % (2 * F)) == 0) F *= 2;
  const int P = kRows / F;
  const int n_hg = G / F;
  const int n_qb = (a.Lq + P - 1) / P;
  const int ntiles = (a.Lkv + kBK - 1) / kBK;
  const int64_t nblk = (int64_t)a.B * a.Hkv * n_hg * n_qb;
  const int64_t nimg = (int64_t)a.B * a.Hkv * ntiles;
  if (nblk > 0x7fffffff || nimg > 0x7fffffff) return hipErrorInvalidValue;
  const Fp8Ws w = fp8_ws(a.B, a.Lkv, a.Hkv, D);
  if (a.ws_bytes < w.total) return hipErrorInvalidValue;
  char* base = static_cast<char*>(a.ws);
  uint16_t* img = reinterpret_cast<uint16_t*>(base);
  uint8_t* k8 = reinterpret_cast<uint8_t*>(base + w.v);
  hipLaunchKernelGGL(prefill_fp8_kv_kernel<D>, dim3((unsigned)nimg), dim3(256), 0, s, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.Lkv, a.Hkv, a.kv_stride, a.signs, k8, img, ntiles);
  auto kern = attn_prefill_bf16_kernel<D, CAUSAL, OUT_BF16, true>;
  const size_t lds = PrefillLds<D, true>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const float c = fmaxf(a.scale * kLog2e, 1e-30f);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kThreads), lds, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, img, a.o, a.lse, a.Lq, a.Lkv, a.Hq, a.Hkv, a.q_stride, a.kv_stride, c, F,
                     n_hg, n_qb, ntiles, nullptr, nullptr, 0, 0, a.signs, k8, nullptr, nullptr);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const PrefillArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lq + 63) / 64), (unsigned)a.Hq, (unsigned)a.B);
  hipLaunchKernelGGL(attn_prefill_f32_kernel<D>, grid, dim3(64), 0, s, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Lq, a.Lkv, a.Hq,
                     a.Hkv, a.q_stride, a.kv_stride, a.scale, a.causal ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int B, int Lkv, int Hkv, int d, bool bf16) {
  if (!bf16 || B <= 0 || Lkv <= 0 || Hkv <= 0) return 0;
  const int64_t ntiles = (Lkv + kBK - 1) / kBK;
  const int64_t per = d == 64 ? PrefillLds<64>::kV : PrefillLds<128>::kV;
  return (size_t)((int64_t)B * Hkv * ntiles * per * 2);
}

size_t prefill_varlen_workspace_bytes(int B, int Lkv_max, int total_q, int Hq, int Hkv, int d) {
  return varlen_sched(B, Lkv_max, total_q, Hq, Hkv, d).bytes;
}

size_t prefill_fp8_workspace_bytes(int B, int Lq, int Lkv, int Hq, int Hkv, int d) {
  if (B <= 0 || Lq <= 0 || Lkv <= 0 || Hq <= 0 || Hkv <= 0 || d != 128) return 0;
  return fp8_ws(B, Lkv, Hkv, d).total;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (!a.in_bf16) return a.d == 64 ? launch_f32<64>(a, s) : launch_f32<128>(a, s);
  if (a.fp8) {
    if (a.d != 128 || a.cu_q != nullptr) return hipErrorInvalidValue;
    if (a.causal) return a.out_bf16 ? launch_fp8<128, true, true>(a, s) : launch_fp8<128, true, false>(a, s);
    return a.out_bf16 ? launch_fp8<128, false, true>(a, s) : launch_fp8<128, false, false>(a, s);
  }
#define MQKV_PF(D, C, O) \
  if (a.d == D && a.causal == C && a.out_bf16 == O) return launch_bf16<D, C, O>(a, s);
  MQKV_PF(64, true, true)
  MQKV_PF(64, true, false)
  MQKV_PF(64, false, true)
  MQKV_PF(64, false, false)
  MQKV_PF(128, true, true)
  MQKV_PF(128, true, false)
  MQKV_PF(128, false, true)
  MQKV_PF(128, false, false)
#undef MQKV_PF
  return hipErrorInvalidValue;
}

}  // namespace mqkv
