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
// Split kernel (bf16): one wave per (sequence, KV head, split, block of 32
// query heads of the group).  Each K/V row is read from HBM once and serves
// all G query heads of its group through MFMA: S^T = K . Q^T (bf16 MFMA with
// the heads as the 32 columns) and O^T += V^T . P^T (fp16 MFMA).  K/V tiles of
// 64 keys are loaded with coalesced 16-byte loads (the next tile is prefetched
// into registers while the current one is computed) and staged in the wave's
// own LDS region: K as-is, V transposed and converted to fp16.  No workgroup
// barrier is used, so waves with different split lengths never wait on each
// other.  Splits that start beyond seq_lens[b] exit at once.
// Combine kernel: one workgroup per (sequence, query head), one thread per
// output element.
#include "common.h"
#include "launch.h"

namespace mqkv {

namespace {

constexpr int kTK = 64;  // keys per tile
constexpr int kWaves = 4;

template <int D>
struct DecodeLds {
  static constexpr int kKld = D + 8;
  static constexpr int kVld = kTK + 8;
  static constexpr int kK = kTK * kKld;
  static constexpr int kWave = kK + D * kVld;  // elements per wave
  static constexpr size_t kBytes = (size_t)kWaves * kWave * sizeof(uint16_t);
};

__device__ __forceinline__ int vt_pos(int a) { return ((a & 1) << 3) | ((a >> 1) << 2); }

template <int D>
__global__ __launch_bounds__(kWaves * 64) void attn_decode_split_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_o, float* __restrict__ part_ml,
    int Hq, int Hkv, int Lmax, int64_t q_stride, float c, int split, int n_split, int n_qblk,
    int n_sgrp) {
  using S = DecodeLds<D>;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int KCH = kTK * D / 8 / 64;          // K chunks per lane
  constexpr int VTASK = (kTK / 4) * (D / 8) / 64;  // V 4x8 tasks per lane
  extern __shared__ __align__(16) uint16_t smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int sgrp = lid % n_sgrp;
  lid /= n_sgrp;
  const int qblk = lid % n_qblk;
  const int bg = lid / n_qblk;
  const int b = bg / Hkv, g = bg % Hkv;
  const int s = sgrp * kWaves + wave;
  if (s >= n_split) return;
  const int len = min(seq_lens[b], Lmax);  // lengths beyond the cache are clamped (caller error)
  const int kbeg = s * split;
  if (kbeg >= len) return;
  const int kend = min(kbeg + split, len);
  const int nt = (kend - kbeg + kTK - 1) / kTK;

  const int G = Hq / Hkv;
  const int col = qblk * 32 + l32;  // query head within the group
  const bool hvalid = col < G;
  const int h = g * G + (hvalid ? col : 0);

  uint16_t* Ks = smem + wave * S::kWave;
  uint16_t* Vt = Ks + S::kK;

  u32x4_t qf[DS];
  {
    const uint16_t* qp = q + (int64_t)b * q_stride + (int64_t)h * D + hf * 8;
#pragma unroll
    for (int t = 0; t < DS; ++t) qf[t] = hvalid ? ld16(qp + t * 16) : u32x4_t{0, 0, 0, 0};
  }

  const int64_t row_stride = (int64_t)Hkv * D;
  const uint16_t* kbase = kc + ((int64_t)b * Lmax) * row_stride + (int64_t)g * D;
  const uint16_t* vbase = vc + ((int64_t)b * Lmax) * row_stride + (int64_t)g * D;

  u32x4_t rk[KCH];
  u32x4_t rv[VTASK][4];
  auto load_tile = [&](int t) {
    const int k0 = kbeg + t * kTK;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int ci = lane + j * 64;
      const int key = ci / (D / 8), dc = ci % (D / 8);
      const int gk = k0 + key;
      rk[j] = (gk < kend) ? ld16(kbase + (int64_t)gk * row_stride + dc * 8) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < VTASK; ++j) {
      const int ti = lane + j * 64;
      const int kg = ti / (D / 8), dg = ti % (D / 8);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int gk = k0 + kg * 4 + jj;
        rv[j][jj] = (gk < kend) ? ld16(vbase + (int64_t)gk * row_stride + dg * 8) : u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int ci = lane + j * 64;
      const int key = ci / (D / 8), dc = ci % (D / 8);
      st16(Ks + key * S::kKld + dc * 8, rk[j]);
    }
#pragma unroll
    for (int j = 0; j < VTASK; ++j) {
      const int ti = lane + j * 64;
      const int kg = ti / (D / 8), dg = ti % (D / 8);
      const int cpos = (kg >> 2) * 16 + vt_pos(kg & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x2_t lo, hi;
        lo[0] = pack_f16(bf16lo(rv[j][0][e]), bf16lo(rv[j][1][e]));
        lo[1] = pack_f16(bf16lo(rv[j][2][e]), bf16lo(rv[j][3][e]));
        hi[0] = pack_f16(bf16hi(rv[j][0][e]), bf16hi(rv[j][1][e]));
        hi[1] = pack_f16(bf16hi(rv[j][2][e]), bf16hi(rv[j][3][e]));
        st8(Vt + (dg * 8 + 2 * e) * S::kVld + cpos, lo);
        st8(Vt + (dg * 8 + 2 * e + 1) * S::kVld + cpos, hi);
      }
    }
  };

  f32x16_t acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  load_tile(0);
  for (int t = 0; t < nt; ++t) {
    wave_lds_sync();  // previous tile's LDS reads are done before overwriting
    store_tile();
    wave_lds_sync();
    if (t + 1 < nt) load_tile(t + 1);
    const int k0 = kbeg + t * kTK;

    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4_t a = ld16(Ks + (kb * 32 + l32) * S::kKld + st * 16 + hf * 8);
        sacc[kb] = mfma32_bf16(a, qf[st], sacc[kb]);
      }

    const bool masked = (k0 + kTK > kend);
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (key >= kend) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, xor32(mx));
    const float mt = mx * c;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + 8.0f) != 0) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    }
    u32x4_t pf[4];
    float ls = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c, -m_run));
        if (masked) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
          p[i] = (key >= kend) ? 0.0f : p[i];
        }
        ls += p[i];
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[kb * 2 + hb][e] = pack_f16(p[hb * 8 + 2 * e], p[hb * 8 + 2 * e + 1]);
    }
    l_run += ls;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4_t a = ld16(Vt + (db * 32 + l32) * S::kVld + ks * 16 + hf * 8);
        acc[db] = mfma32_f16(a, pf[ks], acc[db]);
      }
  }

  const float l_tot = l_run + xor32(l_run);
  if (!hvalid) return;
  const int64_t pidx = ((int64_t)b * Hq + h) * n_split + s;
  float* po = part_o + pidx * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + 8 * g4 + 4 * hf;
      st16(po + d0, u32x4_t{__float_as_uint(acc[db][4 * g4]), __float_as_uint(acc[db][4 * g4 + 1]),
                            __float_as_uint(acc[db][4 * g4 + 2]), __float_as_uint(acc[db][4 * g4 + 3])});
    }
  if (hf == 0) {
    part_ml[pidx * 2 + 0] = m_run;
    part_ml[pidx * 2 + 1] = l_tot;
  }
}

// fp32 split kernel: one wave per (sequence, query head, split); lane j scores key j
// of each 64-key chunk, every lane accumulates D/64 output elements.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_split_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_o, float* __restrict__ part_ml,
    int Hq, int Hkv, int Lmax, int64_t q_stride, float c, int split, int n_split) {
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
  const int64_t pidx = ((int64_t)b * Hq + h) * n_split + s;
#pragma unroll
  for (int e = 0; e < PER; ++e) part_o[pidx * D + e * 64 + lane] = acc[e];
  if (lane == 0) {
    part_ml[pidx * 2 + 0] = m;
    part_ml[pidx * 2 + 1] = l;
  }
}

// Combine the partials of every split of one (sequence, query head).
template <bool OUT_BF16>
__global__ void attn_decode_combine_kernel(const int32_t* __restrict__ seq_lens,
                                           const float* __restrict__ part_o,
                                           const float* __restrict__ part_ml, void* __restrict__ o,
                                           float* __restrict__ lse, int Hq, int D, int split,
                                           int n_split) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int dd = threadIdx.x;
  const int n = min((seq_lens[b] + split - 1) / split, n_split);
  const float* ml = part_ml + (int64_t)bh * n_split * 2;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.0f, acc = 0.0f;
  const float* po = part_o + (int64_t)bh * n_split * D;
  for (int s = 0; s < n; ++s) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
    L = __builtin_fmaf(w, ml[2 * s + 1], L);
    acc = __builtin_fmaf(w, po[(int64_t)s * D + dd], acc);
  }
  const float val = acc / L;
  if constexpr (OUT_BF16)
    static_cast<uint16_t*>(o)[(int64_t)bh * D + dd] = f32_to_bf16(val);
  else
    static_cast<float*>(o)[(int64_t)bh * D + dd] = val;
  if (lse != nullptr && dd == 0) lse[bh] = (M + __builtin_log2f(L)) * kLn2;
}

template <int D>
hipError_t launch_split_bf16(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int n_qblk = (G + 31) / 32;
  const int n_sgrp = (a.n_split + kWaves - 1) / kWaves;
  const int64_t nblk = (int64_t)a.B * a.Hkv * n_qblk * n_sgrp;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  auto kern = attn_decode_split_bf16_kernel<D>;
  const size_t lds = DecodeLds<D>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kWaves * 64), lds, s, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.seq_lens, a.part_o, a.part_ml, a.Hq,
                     a.Hkv, a.Lmax, a.q_stride, a.scale * kLog2e, a.split, a.n_split, n_qblk, n_sgrp);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_f32(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_split, (unsigned)a.Hq, (unsigned)a.B);
  hipLaunchKernelGGL(attn_decode_split_f32_kernel<D>, grid, dim3(64), 0, s, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, a.seq_lens, a.part_o, a.part_ml, a.Hq,
                     a.Hkv, a.Lmax, a.q_stride, a.scale * kLog2e, a.split, a.n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.in_bf16)
    e = a.d == 64 ? launch_split_bf16<64>(a, s) : launch_split_bf16<128>(a, s);
  else
    e = a.d == 64 ? launch_split_f32<64>(a, s) : launch_split_f32<128>(a, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(a.B * a.Hq));
  if (a.out_bf16)
    hipLaunchKernelGGL(attn_decode_combine_kernel<true>, grid, dim3(a.d), 0, s, a.seq_lens, a.part_o,
                       a.part_ml, a.o, a.lse, a.Hq, a.d, a.split, a.n_split);
  else
    hipLaunchKernelGGL(attn_decode_combine_kernel<false>, grid, dim3(a.d), 0, s, a.seq_lens,
                       a.part_o, a.part_ml, a.o, a.lse, a.Hq, a.d, a.split, a.n_split);
  return hipGetLastError();
}

}  // namespace mqkv
