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
//  * One workgroup = 4 waves = 128 query rows of one KV head: F query heads of
//    the group x (128/F) positions, F = the largest power of two dividing
//    G = H_q/H_kv (at most 32).  Every LDS K/V tile is reused by all F heads.
//  * Scores are computed transposed, S^T = K . Q^T: the accumulator then holds
//    one query per lane column, so the row max and row sum are in-lane
//    reductions plus one exchange with the lane 32 away.  Q stays in VGPRs.
//  * exp2 form of the softmax: p = exp2(S*c - m), c = scale*log2(e), one FMA
//    per score.  The running max is only raised when a row's max grows by more
//    than 8 (log2 units); until then p <= 2^8, which keeps fp32 sums exact in
//    form and skips most accumulator rescales.
//  * P is rounded to fp16 and O^T += V^T . P^T runs as an fp16 MFMA: V is
//    converted bf16 -> fp16 (exact for |v| in fp16's normal range) while it is
//    transposed into LDS.  fp16 P carries 3 more mantissa bits than bf16,
//    which keeps the error of outlier-heavy rows inside the bf16 tolerance.
//  * K tiles go to LDS as-is; V tiles are transposed (d-major, keys
//    contiguous, in the order the P operand holds them).  Both are double
//    buffered with a register prefetch of the next tile.
//  * Causal: tiles beyond the block's diagonal are never visited, only tiles
//    that cross a row's limit are masked, and the heaviest query blocks are
//    dispatched first.  Workgroup ids are remapped so that each XCD serves a
//    contiguous range of (batch, KV head) blocks and keeps their K/V in its L2.
// fp32 inputs use a plain one-row-per-thread kernel (fp32 throughout).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mqkv {

namespace {

#ifndef MQKV_PF_WAVES
#define MQKV_PF_WAVES 8  // waves per workgroup (32 query rows each)
#endif
#ifndef MQKV_PF_BK
#define MQKV_PF_BK 64    // keys per K/V tile (a multiple of 64)
#endif
constexpr int kWaves = MQKV_PF_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = kWaves * 32;  // query rows per workgroup
constexpr int kBK = MQKV_PF_BK;
constexpr int kStages = 2;  // K/V tiles resident in LDS (double buffer)
constexpr float kTau = 8.0f;        // lazy-rescale threshold (log2 units)
#ifndef MQKV_PF_OCC
#define MQKV_PF_OCC 2  // minimum waves per SIMD the register budget must allow
#endif

template <int D>
struct PrefillLds {
  static constexpr int kKld = D + 8;        // K row stride (bf16 elements)
  static constexpr int kVld = kBK + 8;      // V^T row stride (fp16 elements)
  static constexpr int kK = kBK * kKld;     // elements per K stage
  static constexpr int kV = D * kVld;       // elements per V^T stage
  static constexpr int kStage = kK + kV;
  static constexpr size_t kBytes = kStages * kStage * sizeof(uint16_t);
};

// Position, inside a 16-key group, of key 4a + j (a = 0..3) in the V^T rows:
// keys {0-3, 8-11} first (lane half 0 of the P operand), then {4-7, 12-15}.
__device__ __forceinline__ int vt_pos(int a) { return ((a & 1) << 3) | ((a >> 1) << 2); }

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, MQKV_PF_OCC) void attn_prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* __restrict__ o, float* __restrict__ lse, int Lq, int Lkv, int Hq, int Hkv,
    int64_t q_stride, int64_t kv_stride, float c, int F, int n_hg, int n_qb) {
  using S = PrefillLds<D>;
  constexpr int DS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int KCH = kBK * D / 8 / kThreads;  // 16B K chunks per thread
  static_assert(KCH >= 1 && KCH * kThreads == kBK * D / 8, "K tile split over threads");
  constexpr int VT = (kBK / 4) * (D / 8);      // 4x8 V tasks per tile
  constexpr int VTPT = (VT + kThreads - 1) / kThreads;  // V tasks per thread
  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- block -> (b, g, head group, query block), heaviest causal blocks first
  const int G = Hq / Hkv;
  const int P = kRows / F;  // positions per workgroup
  int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = n_qb - 1 - (lid % n_qb);
  lid /= n_qb;
  const int hg = lid % n_hg;
  lid /= n_hg;
  const int g = lid % Hkv;
  const int b = lid / Hkv;
  const int p0 = qb * P;
  const int off = Lkv - Lq;

  // ---- this lane's query row (column of the S^T tile)
  const int r = wave * 32 + l32;
  const int h = g * G + hg * F + r / P;
  const int pos = p0 + r % P;
  const bool valid = pos < Lq;
  const int lim = CAUSAL ? min(pos + off, Lkv - 1) : Lkv - 1;  // last visible key

  u32x4_t qf[DS];
  {
    const uint16_t* qp = q + ((int64_t)b * Lq + pos) * q_stride + (int64_t)h * D + hf * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = valid ? ld16(qp + s * 16) : u32x4_t{0, 0, 0, 0};
  }

  const int last_pos = min(p0 + P, Lq) - 1;
  const int kv_end = CAUSAL ? min(Lkv, last_pos + off + 1) : Lkv;
  const int mask_from = CAUSAL ? min(Lkv, p0 + off + 1) : Lkv;  // first key some row cannot see
  const int nt = (kv_end + kBK - 1) / kBK;

  // K/V rows of batch b through bounds-checked buffer resources: a key >= L_kv
  // lands at or past the resource end and reads zeros.
  const uint32_t kv_bytes = (uint32_t)((int64_t)Lkv * kv_stride * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (int64_t)b * Lkv * kv_stride, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + (int64_t)b * Lkv * kv_stride, kv_bytes);
  const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
  const uint32_t head_off = (uint32_t)(g * D * 2);

  u32x4_t rk[KCH];
  u32x4_t rv[VTPT][4];
  auto load_tile = [&](int t) {
    const int k0 = t * kBK;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int ci = tid + j * kThreads;
      const int key = ci / (D / 8), dc = ci % (D / 8);
      rk[j] = bld16(krs, (uint32_t)(k0 + key) * row_bytes + head_off + dc * 16);
    }
#pragma unroll
    for (int j = 0; j < VTPT; ++j) {
      const int ti = tid + j * kThreads;
      const int kg = ti / (D / 8), dg = ti % (D / 8);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = k0 + kg * 4 + jj;
        rv[j][jj] = bld16(vrs, (ti < VT ? (uint32_t)key * row_bytes : kv_bytes) + head_off + dg * 16);
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks = smem + buf * S::kStage;
    uint16_t* Vt = Ks + S::kK;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int ci = tid + j * kThreads;
      const int key = ci / (D / 8), dc = ci % (D / 8);
      st16(Ks + key * S::kKld + dc * 8, rk[j]);
    }
#pragma unroll
    for (int j = 0; j < VTPT; ++j) {
      const int ti = tid + j * kThreads;
      if (ti < VT) {
        const int kg = ti / (D / 8), dg = ti % (D / 8);
        const int col = (kg >> 2) * 16 + vt_pos(kg & 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // rv[j][jj][e] = V[key jj][d = 8dg+2e, 8dg+2e+1] (bf16 pair)
          u32x2_t lo, hi;
          lo[0] = pack_f16(bf16lo(rv[j][0][e]), bf16lo(rv[j][1][e]));
          lo[1] = pack_f16(bf16lo(rv[j][2][e]), bf16lo(rv[j][3][e]));
          hi[0] = pack_f16(bf16hi(rv[j][0][e]), bf16hi(rv[j][1][e]));
          hi[1] = pack_f16(bf16hi(rv[j][2][e]), bf16hi(rv[j][3][e]));
          st8(Vt + (dg * 8 + 2 * e) * S::kVld + col, lo);
          st8(Vt + (dg * 8 + 2 * e + 1) * S::kVld + col, hi);
        }
      }
    }
  };

  f32x16_t acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16_t{};
  float m_run = -INFINITY;  // running max of S*c (log2 units)
  float l_run = 0.0f;       // this lane's share of the running sum

  // One 32-key half: scores -> online softmax -> O^T += V^T P^T.  The two halves
  // are issued back to back so that one half's softmax (VALU) runs while the
  // other half's MFMAs are in flight.
  const uint16_t* Ks;
  const uint16_t* Vt;
  int k0;
    auto half = [&](f32x16_t sc, int kb, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      if constexpr (MASK) {
        // key - k0 - 4*hf of element i is 32kb + 8(i/4) + (i%4); mask keys beyond lim
        const int rel = lim - k0 - 4 * hf - 32 * kb;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) > rel) sc[i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
      mx = fmaxf(mx, sc[15]);
      mx = fmaxf(mx, xor32(mx));
      const float mt = mx * c;
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kTau) != 0) {
        // only this row's own growth moves its max, so a row's result does not
        // depend on the other rows that share the wave
        const float mn = (mt > m_run + kTau) ? mt : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        m_run = mn;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
      }
      u32x4_t pf[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e], c, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hb * 8 + 2 * e + 1], c, -m_run));
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
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        u32x4_t vf[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
          vf[db] = ld16(Vt + (db * 32 + l32) * S::kVld + (kb * 2 + hb) * 16 + hf * 8);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32_f16(vf[db], pf[hb], acc[db]);
      }
    };
    auto tile = [&](auto mask_tag) {
#pragma unroll
      for (int sub = 0; sub < kBK / 64; ++sub) {
        f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
        for (int st = 0; st < DS; ++st)
          s0 = mfma32_bf16(ld16(Ks + (sub * 64 + l32) * S::kKld + st * 16 + hf * 8), qf[st], s0);
#pragma unroll
        for (int st = 0; st < DS; ++st)
          s1 = mfma32_bf16(ld16(Ks + (sub * 64 + 32 + l32) * S::kKld + st * 16 + hf * 8), qf[st], s1);
        half(s0, 2 * sub, mask_tag);
        half(s1, 2 * sub + 1, mask_tag);
      }
    };

  // Tiles below every row's causal limit run without masking; the loop is split
  // so that the masked body is a separate piece of code.
  const int t_mask = min(nt, mask_from / kBK);
  auto iter = [&](int t, auto mask_tag) {
    const int buf = t & 1;
    if (t + 1 < nt) load_tile(t + 1);
    Ks = smem + buf * S::kStage;
    Vt = Ks + S::kK;
    k0 = t * kBK;
    tile(mask_tag);
    if (t + 1 < nt) store_tile(buf ^ 1);
    __syncthreads();
  };
  load_tile(0);
  store_tile(0);
  __syncthreads();
  int t = 0;
  for (; t < t_mask; ++t) iter(t, std::false_type{});
  for (; t < nt; ++t) iter(t, std::true_type{});

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  const float l_tot = l_run + xor32(l_run);
  if (!valid) return;
  const float inv = 1.0f / l_tot;
  const int64_t orow = (((int64_t)b * Lq + pos) * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + 8 * g4 + 4 * hf;
      const float v0 = acc[db][4 * g4 + 0] * inv, v1 = acc[db][4 * g4 + 1] * inv;
      const float v2 = acc[db][4 * g4 + 2] * inv, v3 = acc[db][4 * g4 + 3] * inv;
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
  if (lse != nullptr && hf == 0)
    lse[((int64_t)b * Hq + h) * Lq + pos] = (m_run + __builtin_log2f(l_tot)) * kLn2;
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

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  int F = 1;
  while (F < 32 && (G % (2 * F)) == 0) F *= 2;
  const int P = kRows / F;
  const int n_hg = G / F;
  const int n_qb = (a.Lq + P - 1) / P;
  const int64_t nblk = (int64_t)a.B * a.Hkv * n_hg * n_qb;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  auto kern = attn_prefill_bf16_kernel<D, CAUSAL, OUT_BF16>;
  const size_t lds = PrefillLds<D>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // scale 0 is run as a tiny positive scale: masked scores stay -inf after the
  // multiply and every visible score maps to exp2(0) = 1 exactly.
  const float c = fmaxf(a.scale * kLog2e, 1e-30f);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kThreads), lds, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.lse, a.Lq, a.Lkv, a.Hq, a.Hkv,
                     a.q_stride, a.kv_stride, c, F, n_hg, n_qb);
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

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (!a.in_bf16) return a.d == 64 ? launch_f32<64>(a, s) : launch_f32<128>(a, s);
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
