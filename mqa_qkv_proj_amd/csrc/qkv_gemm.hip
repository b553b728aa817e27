// Fused QKV projection GEMM for gfx950.
//
// qkv[M, N] = x[M, K] . W[K, N] (+ bias[N]) -- one GEMM for Q, K and V together
// ("Optimize LlamaAttention by fusing QKV projections", transformers PR #40092,
// the diff of LlamaAttention.forward).  The split into Q/K/V is free: callers
// address the packed rows with a token stride.
//
// bf16 path: bf16 MFMA with fp32 accumulation, bf16 output (RNE).  Kernels,
// chosen by shape in launch_qkv_gemm:
//  * M <= 32, N <= 4096, K % 128 == 0: streaming kernel on 16-column blocks
//    (W streamed through an LDS ring filled by LDS-DMA, no k split);
//  * M <= 128 otherwise: register-staged skinny kernel, k split over
//    workgroups with a fixed-order reduce kernel;
//  * M > 128, K % 64 == 0, N % 8 == 0: LDS-DMA fed 128x128 / 64x128 tiles, the
//    W tile kept row-major and read with transposing LDS loads;
//  * anything else: register-prefetched tiles with W transposed into LDS by
//    the loading threads.
// fp32 path: plain LDS-tiled fp32 FMA (a correctness path for the tiny fp32 layer).
#include "common.h"
#include "launch.h"

namespace mqkv {

// The append epilogue for one output element (see KvAppend): a no-op unless an
// append is requested, n is a K or V column and row m's position is valid.
template <typename T>
__device__ __forceinline__ void append_store(const KvAppend& a, int m, int n, T v) {
  if (a.k_cache == nullptr || n < a.kcol) return;
  const int len = a.seq_lens[m];
  if (len < 1 || len > a.L_max) return;
  const bool is_k = n < a.vcol;
  T* cache = static_cast<T*>(is_k ? a.k_cache : a.v_cache);
  cache[((int64_t)m * a.L_max + (len - 1)) * (a.vcol - a.kcol) + (n - (is_k ? a.kcol : a.vcol))] = v;
}

template <int BM, int BN, int BK, int WM, int WN, int KS>
struct GemmCfg {
  static constexpr int kWaves = WM * WN * KS;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kPad = 8;                 // bf16 elements of padding per LDS row
  static constexpr int kLd = BK + kPad;
  static constexpr int kMI = BM / WM / 32;       // 32x32 blocks per wave (rows)
  static constexpr int kNI = BN / WN / 32;       // 32x32 blocks per wave (cols)
  static constexpr int kSteps = BK / 16;         // MFMA k-steps per tile
  static constexpr int kStepsPerWave = kSteps / KS;
  static constexpr int kAChunks = BM * BK / 8 / kThreads;     // 16B chunks of x per thread
  static constexpr int kBTasks = (BK / 4) * (BN / 8);          // 4x8 W blocks per tile
  static constexpr int kBTasksPerThread = (kBTasks + kThreads - 1) / kThreads;
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "tile");
  static_assert(kSteps % KS == 0, "k split");
  static_assert((BM * BK / 8) % kThreads == 0, "x chunks");
  static constexpr int kLdsTile = (BM + BN) * kLd;  // elements per stage
};

template <int BM, int BN, int BK, int WM, int WN, int KS>
__global__ __launch_bounds__(WM* WN* KS * 64) void qkv_gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int K, int N, KvAppend app) {
  using C = GemmCfg<BM, BN, BK, WM, WN, KS>;
  extern __shared__ __align__(16) uint16_t smem[];
  // stage s: x tile at smem + s*kLdsTile, transposed W tile right after it
  auto As = [&](int st) { return smem + st * C::kLdsTile; };
  auto Bs = [&](int st) { return smem + st * C::kLdsTile + BM * C::kLd; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wk = wave / (WM * WN);
  const int wmn = wave % (WM * WN);
  const int wm = wmn / WN, wn = wmn % WN;
  const int l32 = lane & 31, hf = lane >> 5;

  const int nbn = (N + BN - 1) / BN;
  const int nbm = (M + BM - 1) / BM;
  const int lid = xcd_remap(blockIdx.x, nbn * nbm);
  // logical order: the n-tiles of one m-row are neighbours (they share x rows).
  const int bm = lid / nbn, bn = lid % nbn;
  const int m0 = bm * BM, n0 = bn * BN;
  const int nk = (K + BK - 1) / BK;

  u32x4_t ra[C::kAChunks];
  u32x4_t rb[C::kBTasksPerThread][4];

  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < C::kAChunks; ++j) {
      const int ci = tid + j * C::kThreads;
      const int r = ci / (BK / 8), kc = ci % (BK / 8);
      const int gm = m0 + r, gk = k0 + kc * 8;
      ra[j] = (gm < M && gk < K) ? ld16(x + (int64_t)gm * K + gk) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < C::kBTasksPerThread; ++j) {
      const int ti = tid + j * C::kThreads;
      const int kg = ti % (BK / 4), ng = ti / (BK / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gk = k0 + kg * 4 + r, gn = n0 + ng * 8;
        rb[j][r] = (ti < C::kBTasks && gk < K && gn < N) ? ld16(w + (int64_t)gk * N + gn)
                                                         : u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < C::kAChunks; ++j) {
      const int ci = tid + j * C::kThreads;
      const int r = ci / (BK / 8), kc = ci % (BK / 8);
      st16(As(buf) + r * C::kLd + kc * 8, ra[j]);
    }
#pragma unroll
    for (int j = 0; j < C::kBTasksPerThread; ++j) {
      const int ti = tid + j * C::kThreads;
      if (ti < C::kBTasks) {
        // consecutive lanes take consecutive 4-row groups: one 8-byte store
        // instruction then covers whole rows of the transposed tile
        const int kg = ti % (BK / 4), ng = ti / (BK / 4);
        // rb[j][r].e holds W[k0+4kg+r][n0+8ng+2e .. +1]; write column n as 4 k values.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x2_t lo, hi;
          lo[0] = __builtin_amdgcn_perm(rb[j][1][e], rb[j][0][e], 0x05040100u);
          lo[1] = __builtin_amdgcn_perm(rb[j][3][e], rb[j][2][e], 0x05040100u);
          hi[0] = __builtin_amdgcn_perm(rb[j][1][e], rb[j][0][e], 0x07060302u);
          hi[1] = __builtin_amdgcn_perm(rb[j][3][e], rb[j][2][e], 0x07060302u);
          st8(Bs(buf) + (ng * 8 + 2 * e) * C::kLd + kg * 4, lo);
          st8(Bs(buf) + (ng * 8 + 2 * e + 1) * C::kLd + kg * 4, hi);
        }
      }
    }
  };

  f32x16_t acc[C::kMI][C::kNI];
#pragma unroll
  for (int i = 0; i < C::kMI; ++i)
#pragma unroll
    for (int j = 0; j < C::kNI; ++j) acc[i][j] = f32x16_t{};

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const uint16_t* A = As(buf);
    const uint16_t* Bt = Bs(buf);
#pragma unroll
    for (int s = 0; s < C::kStepsPerWave; ++s) {
      const int ks = wk * C::kStepsPerWave + s;
      u32x4_t af[C::kMI], bfr[C::kNI];
#pragma unroll
      for (int i = 0; i < C::kMI; ++i)
        af[i] = ld16(A + (wm * (BM / WM) + i * 32 + l32) * C::kLd + ks * 16 + hf * 8);
#pragma unroll
      for (int j = 0; j < C::kNI; ++j)
        bfr[j] = ld16(Bt + (wn * (BN / WN) + j * 32 + l32) * C::kLd + ks * 16 + hf * 8);
#pragma unroll
      for (int i = 0; i < C::kMI; ++i)
#pragma unroll
        for (int j = 0; j < C::kNI; ++j) acc[i][j] = mfma32_bf16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  if constexpr (KS > 1) {
    // Reduce the k-split partial sums through LDS (the tile buffers are free now).
    float* red = reinterpret_cast<float*>(smem);
    constexpr int kTileF = (BM / WM) * (BN / WN);
    if (wk > 0) {
#pragma unroll
      for (int i = 0; i < C::kMI; ++i)
#pragma unroll
        for (int j = 0; j < C::kNI; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            red[((wk - 1) * WM * WN + wmn) * kTileF + ((i * C::kNI + j) * 16 + e) * 64 + lane] =
                acc[i][j][e];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int p = 1; p < KS; ++p)
#pragma unroll
      for (int i = 0; i < C::kMI; ++i)
#pragma unroll
        for (int j = 0; j < C::kNI; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            acc[i][j][e] += red[((p - 1) * WM * WN + wmn) * kTileF + ((i * C::kNI + j) * 16 + e) * 64 + lane];
  }

#pragma unroll
  for (int j = 0; j < C::kNI; ++j) {
    const int gn = n0 + wn * (BN / WN) + j * 32 + l32;
    if (gn >= N) continue;
    const float bv = bias ? bf16_to_f32(bias[gn]) : 0.0f;
#pragma unroll
    for (int i = 0; i < C::kMI; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gm = m0 + wm * (BM / WM) + i * 32 + 8 * (e / 4) + 4 * hf + (e % 4);
        if (gm < M) {
          const uint16_t r = f32_to_bf16(acc[i][j][e] + bv);
          out[(int64_t)gm * N + gn] = r;
          append_store(app, gm, gn, r);
        }
      }
    }
  }
}

// fp32 path: 64x64 tile, 256 threads, 4x4 outputs per thread, k tile 16.
__global__ __launch_bounds__(256) void qkv_gemm_f32_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ out, int M, int K,
                                                           int N, KvAppend app) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = tid; e < 64 * 16; e += 256) {
      const int r = e / 16, kk = e % 16;
      As[kk][r] = (m0 + r < M && k0 + kk < K) ? x[(int64_t)(m0 + r) * K + k0 + kk] : 0.0f;
      const int kr = e / 64, nn = e % 64;
      Bs[kr][nn] = (k0 + kr < K && n0 + nn < N) ? w[(int64_t)(k0 + kr) * N + n0 + nn] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn < N) {
        const float r = acc[i][j] + (bias ? bias[gn] : 0.0f);
        out[(int64_t)gm * N + gn] = r;
        append_store(app, gm, gn, r);
      }
    }
  }
}

// ----------------------------------------------------------------------------- copy-fed tiles
// Workgroup tile BM x 128, k tile 64, 4 waves as 2 x 2.  Both operand tiles reach
// LDS by LDS-DMA (buffer loads that write LDS directly, no staging registers):
//  * x tile: BM rows of 64 k (k-contiguous) + 16 bytes of padding per row;
//  * W tile: 64 rows of 128 n (n-contiguous, as W is stored) + 64 bytes of
//    padding per row.  The MFMA B operand (8 consecutive k of one n per lane)
//    is read with the transposing LDS load ds_read_b64_tr_b16: within each 16
//    lanes, lane 4j+q reads 4 n of k-row j and lane i receives column i of the
//    4 rows, so no VALU transposition is needed.
// The row paddings keep both operand reads on distinct LDS banks; the lanes of
// a copy that fall on padding point past the buffer, so they fetch nothing and
// land only on padding bytes, which are never read.  Two
// LDS stages: the copy of k tile t+1 runs while tile t is multiplied, one
// barrier per k tile.  All operand reads of a 16-deep k step are issued
// together and waited for once, a step ahead of their MFMAs.  Requires
// K % 64 == 0.
constexpr int kCfBN = 128, kCfBK = 64, kCfThreads = 256;
constexpr int kCfXld = kCfBK + 8;   // x tile row pitch (bf16 elements): 9 chunks of 16 B
constexpr int kCfWld = kCfBN + 32;  // W tile row pitch: 20 chunks of 16 B
template <int BM>
struct CfLds {
  static constexpr int kX = BM * kCfXld;
  static constexpr int kW = kCfBK * kCfWld;
  static constexpr int kStage = kX + kW;
  static constexpr int kXCopies = kX * 2 / 1024;
  static constexpr int kWCopies = kW * 2 / 1024;
  static constexpr int kXcp = (kXCopies + 3) / 4;  // copies per wave
  static constexpr int kWcp = (kWCopies + 3) / 4;
  static constexpr size_t kBytes = 2 * (size_t)kStage * sizeof(uint16_t);
  static_assert(kX * 2 % 1024 == 0 && kW * 2 % 1024 == 0, "tiles are whole 1 KB copies");
};

// B operand of a 32x32x16 MFMA from a row-major W tile: two transposing reads
// (k rows r and r+4 of this lane's group; HI_BYTES apart) that wait for
// themselves.  Written as one asm block because the compiler treats the
// builtin form as aliasing every LDS-DMA copy in flight and waits for all of
// them first, which would serialize the copy pipeline; the callers order these
// reads after the copies they need with their own vmcnt waits.
template <int HI_BYTES>
__device__ __forceinline__ u32x4_t lds_tr16_pair(const uint16_t* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
  u32x2_t lo, hi;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo), "=&v"(hi)
      : "v"(a), "i"(HI_BYTES)
      : "memory");
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// All operand fragments of one 16-deep k step: the MI x rows (A) and the two
// transposed W pairs (B), read in one asm block that waits for itself once,
// so a k step costs one LDS round trip rather than one per B pair.
template <int MI, int HI_BYTES>
__device__ __forceinline__ void lds_step_frags(const uint16_t* pa0, const uint16_t* pa1, const uint16_t* pb0,
                                               const uint16_t* pb1, u32x4_t (&a)[MI], u32x4_t (&b)[2]) {
  auto addr = [](const uint16_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
  };
  u32x2_t l0, h0, l1, h1;
  if constexpr (MI == 2) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b64_tr_b16 %2, %8\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %4, %9\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%10\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1)
        : "v"(addr(pa0)), "v"(addr(pa1)), "v"(addr(pb0)), "v"(addr(pb1)), "i"(HI_BYTES)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b64_tr_b16 %1, %6\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "ds_read_b64_tr_b16 %4, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1)
        : "v"(addr(pa0)), "v"(addr(pb0)), "v"(addr(pb1)), "i"(HI_BYTES)
        : "memory");
    (void)pa1;
  }
  b[0] = u32x4_t{l0[0], l0[1], h0[0], h0[1]};
  b[1] = u32x4_t{l1[0], l1[1], h1[0], h1[1]};
}

template <int BM>
__global__ __launch_bounds__(kCfThreads, 2) void qkv_gemm_cf_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ out, int M, int K, int N, KvAppend app) {
  using L = CfLds<BM>;
  constexpr int MI = BM / 64;  // 32-row MFMA blocks per wave
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wq = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hf = lane >> 5;

  const int nbn = (N + kCfBN - 1) / kCfBN, nbm = (M + BM - 1) / BM;
  const int lid = xcd_remap(blockIdx.x, nbn * nbm);
  const int bm = lid / nbn, bn = lid % nbn;  // the n tiles of one m row are neighbours
  const int m0 = bm * BM, n0 = bn * kCfBN;
  const int nk = K / kCfBK;

  // ---- copy maps: slot (copy * 64 + lane) of a tile image -> global byte offset
  constexpr uint32_t kNoCopy = 0x80000000u;
  const uint32_t xrow = (uint32_t)K * 2, wrow = (uint32_t)N * 2;
  uint32_t xoff[L::kXcp], woff[L::kWcp];
#pragma unroll
  for (int i = 0; i < L::kXcp; ++i) {
    const int slot = (wave + 4 * i) * 64 + lane;
    const int r = slot / 9, ch = slot % 9;
    xoff[i] = ch < 8 ? (uint32_t)r * xrow + ch * 16 : kNoCopy;
  }
#pragma unroll
  for (int i = 0; i < L::kWcp; ++i) {
    const int slot = (wave + 4 * i) * 64 + lane;
    const int r = slot / 20, ch = slot % 20;
    woff[i] = ch < 16 ? (uint32_t)r * wrow + ch * 16 : kNoCopy;
  }
  // x rows at or past M and W rows past K lie past their buffer ends: they
  // fetch nothing, and their LDS rows only feed outputs that are not stored.
  const uint64_t xbytes = (uint64_t)M * K * 2, wbytes = (uint64_t)K * N * 2;
  auto copy_tile = [&](int kt, int st) {
    uint16_t* xs = smem + st * L::kStage;
    uint16_t* ws = xs + L::kX;
    const uint64_t xb = (uint64_t)m0 * K * 2 + (uint64_t)kt * kCfBK * 2;
    const uint64_t wb = (uint64_t)kt * kCfBK * N * 2 + (uint64_t)n0 * 2;
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(reinterpret_cast<const char*>(x) + xb, (uint32_t)min(xbytes - xb, (uint64_t)0x7fffffff));
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(reinterpret_cast<const char*>(w) + wb, (uint32_t)min(wbytes - wb, (uint64_t)0x7fffffff));
#pragma unroll
    for (int i = 0; i < L::kXcp; ++i) {
      const int cp = wq + 4 * i;
      if (cp < L::kXCopies) dma16(xr, xs + cp * 512, xoff[i], 0);
    }
#pragma unroll
    for (int i = 0; i < L::kWcp; ++i) {
      const int cp = wq + 4 * i;
      if (cp < L::kWCopies) dma16(wr, ws + cp * 512, woff[i], 0);
    }
  };

  f32x16_t acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i) acc[i][0] = acc[i][1] = f32x16_t{};

  // operand fragments of one 16-deep k step
  const int bg = lane >> 4, bp = lane & 15;                   // transposing-read lane group
  const int b_n = 16 * (bg & 1) + 4 * (bp & 3), b_k = 8 * (bg >> 1) + (bp >> 2);
  auto frags = [&](const uint16_t* xs, const uint16_t* ws, int ks, u32x4_t (&a)[MI], u32x4_t (&b)[2]) {
    const uint16_t* pa = xs + (wm * (BM / 2) + l32) * kCfXld + ks * 16 + hf * 8;
    const uint16_t* pb = ws + (ks * 16 + b_k) * kCfWld + wn * 64 + b_n;
    lds_step_frags<MI, 4 * kCfWld * 2>(pa, pa + 32 * kCfXld, pb, pb + 32, a, b);
  };

  copy_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies landed
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) copy_tile(kt + 1, st ^ 1);
    const uint16_t* xs = smem + st * L::kStage;
    const uint16_t* ws = xs + L::kX;
    u32x4_t a[2][MI], b[2][2];
    frags(xs, ws, 0, a[0], b[0]);
    static_for<0, kCfBK / 16>([&](auto ks) {
      constexpr int cur = ks & 1;
      if constexpr (ks + 1 < kCfBK / 16) frags(xs, ws, ks + 1, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32_bf16(a[cur][i], b[cur][j], acc[i][j]);
    });
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int gn = n0 + wn * 64 + j * 32 + l32;
    if (gn >= N) continue;
    const float bv = bias ? bf16_to_f32(bias[gn]) : 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gm = m0 + wm * (BM / 2) + i * 32 + 8 * (e / 4) + 4 * hf + (e % 4);
        if (gm < M) {
          const uint16_t r = f32_to_bf16(acc[i][j][e] + bv);
          out[(int64_t)gm * N + gn] = r;
          append_store(app, gm, gn, r);
        }
      }
    }
  }
}

template <int BM>
static hipError_t launch_gemm_cf(const void* x, const void* w, const void* bias, void* out, int M, int K,
                                 int N, hipStream_t s, const KvAppend& app) {
  auto kern = qkv_gemm_cf_kernel<BM>;
  const size_t lds = CfLds<BM>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int nblk = ((M + BM - 1) / BM) * ((N + kCfBN - 1) / kCfBN);
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(kCfThreads), lds, s, (const uint16_t*)x, (const uint16_t*)w,
                     (const uint16_t*)bias, (uint16_t*)out, M, K, N, app);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- skinny M
// M <= 128 (decode batches, short prompts): the weight is streamed once and is
// the whole cost, so the grid is widened by splitting the k range over
// workgroups.  Workgroup = 2 waves, tile = 32 rows x 32 columns x a k range;
// each 128-deep chunk of W is loaded with 16-byte loads two chunks ahead and
// written to LDS transposed; x fragments come straight from L2 in MFMA layout.
// With several k ranges, fp32 partial tiles go to the workspace and a second
// kernel adds them (fixed order), adds the bias and rounds to bf16.
constexpr int kSkBN = 32, kSkBK = 128, kSkLd = kSkBK + 8, kSkThreads = 128;
constexpr int kSkMaxChunks = 8;  // k range <= 1024 rows
constexpr int kSkDepth = 3;      // chunks in flight ahead of the one being multiplied

__global__ __launch_bounds__(kSkThreads) void qkv_gemm_skinny_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ out, float* __restrict__ part, int M, int K, int N, int krange, int ksplit,
    int nbm, KvAppend app) {
  __shared__ __align__(16) uint16_t Bs[2][kSkBN * kSkLd];
  __shared__ __align__(16) float red[16 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bm = lid % nbm;  // row blocks of one (column block, k range) are neighbours: W reuse in L2
  lid /= nbm;
  const int ks = lid % ksplit;
  const int bn = lid / ksplit;
  const int m0 = bm * 32, n0 = bn * kSkBN;
  const int kbeg = ks * krange, kend = min(K, kbeg + krange);
  const int nchunk = (kend - kbeg + kSkBK - 1) / kSkBK;

  const uint32_t wbytes = (uint32_t)((int64_t)K * N * 2);
  const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, wbytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, xbytes);
  // W task of this thread: rows 4*kg..4*kg+3 of a chunk, columns 8*ng..8*ng+7 of the tile
  const int kg = tid >> 2, ng = tid & 3;
  const int xrow = m0 + l32;

  // A chunk = 4 W rows-segments (16 B each) + this wave's 4 x fragments; every
  // load is issued unconditionally (out-of-range offsets read zeros), so the
  // waits on the in-order load counter stay exact.
  u32x4_t rw[kSkDepth][4], rx[kSkDepth][4];
  auto load_chunk = [&](int c, u32x4_t (&w4)[4], u32x4_t (&x4)[4]) {
    const int kw = kbeg + c * kSkBK + kg * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = kw + j;
      w4[j] = bld16(wr, (c < nchunk && kk < kend) ? (uint32_t)((int64_t)kk * N + n0 + ng * 8) * 2 : wbytes);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kk = kbeg + c * kSkBK + (wave * 4 + st) * 16 + hf * 8;
      x4[st] = bld16(xr, (c < nchunk && xrow < M && kk < kend) ? (uint32_t)((int64_t)xrow * K + kk) * 2 : xbytes);
    }
  };
  auto store_chunk = [&](int buf, const u32x4_t (&w4)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x2_t lo, hi;
      lo[0] = __builtin_amdgcn_perm(w4[1][e], w4[0][e], 0x05040100u);
      lo[1] = __builtin_amdgcn_perm(w4[3][e], w4[2][e], 0x05040100u);
      hi[0] = __builtin_amdgcn_perm(w4[1][e], w4[0][e], 0x07060302u);
      hi[1] = __builtin_amdgcn_perm(w4[3][e], w4[2][e], 0x07060302u);
      st8(&Bs[buf][(ng * 8 + 2 * e) * kSkLd + kg * 4], lo);
      st8(&Bs[buf][(ng * 8 + 2 * e + 1) * kSkLd + kg * 4], hi);
    }
  };

  f32x16_t acc = f32x16_t{};
#pragma unroll
  for (int c = 0; c < kSkDepth; ++c) load_chunk(c, rw[c], rx[c]);
#pragma unroll
  for (int c = 0; c < kSkMaxChunks; ++c) {
    if (c >= nchunk) break;
    const int r = c % kSkDepth;
    store_chunk(c & 1, rw[r]);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 4; ++st)
      acc = mfma32_bf16(rx[r][st], ld16(&Bs[c & 1][l32 * kSkLd + (wave * 4 + st) * 16 + hf * 8]), acc);
    if (c + kSkDepth < kSkMaxChunks) load_chunk(c + kSkDepth, rw[r], rx[r]);
  }
  // add the two waves' k-step halves
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[e * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (wave == 1) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] += red[e * 64 + lane];
  const int n = n0 + l32;
  if (ksplit == 1) {
    const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 8 * (e >> 2) + 4 * hf + (e & 3);
      if (m < M) {
        const uint16_t r = f32_to_bf16(acc[e] + bv);
        out[(int64_t)m * N + n] = r;
        append_store(app, m, n, r);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 8 * (e >> 2) + 4 * hf + (e & 3);
      if (m < M) part[((int64_t)ks * M + m) * N + n] = acc[e];
    }
  }
}

// ----------------------------------------------------------------------------- LDS-DMA wait helpers
// s_waitcnt immediate: vmcnt(n), expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ----------------------------------------------------------------------------- skinny M <= 32, streamed
// M <= 32 with K % 128 == 0 and a narrow W: the weight is the whole cost, so a
// workgroup owns 16 columns of W over all of K and streams them.  Its 4 waves
// take the 32-row k steps in turn (wave w: steps w, w+4, ...), each through a
// ring of D LDS slots of its own (one step's W rows, 32 x 32 B, and x columns,
// MB blocks of 16 rows x 32 k) filled by LDS-DMA D steps ahead: no register
// staging and no barrier until the 4 waves' sums are added in LDS, in wave
// order, at the end.  MFMA 16x16x32; the B operand is read with
// ds_read_b64_tr_b16 from the row-major W slot, whose rows are stored with
// index bits 2 and 3 swapped so that the two 16-lane groups of a read (rows r
// and r+8) land on different LDS banks; x is stored in A-fragment order.  With
// one workgroup per 16 columns there is no k split: no partials and no second
// kernel.
constexpr int kS16BN = 16, kS16Threads = 256;
template <int MB, int D>
__global__ __launch_bounds__(kS16Threads, 2) void qkv_gemm_stream16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ out, int M, int K, int N, KvAppend app) {
  constexpr int kSlot = (1 + MB) * 512;     // bf16 elements: W rows, then x blocks
  constexpr int kAhead = (D - 1) * (1 + MB);  // loads issued after a step's own
  static_assert(kAhead <= 63, "vmcnt range");
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = xcd_remap(blockIdx.x, gridDim.x) * kS16BN;
  const int nst = K >> 7;  // 32-row k steps per wave

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((int64_t)K * N * 2));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * K * 2));
  // W copy: lane l -> slot row l/2 (k row with bits 2,3 swapped), 16 B chunk l%2
  const int srow = lane >> 1;
  const int krow = (srow & ~12) | ((srow & 4) << 1) | ((srow & 8) >> 1);
  const uint32_t w_lane = (uint32_t)krow * N * 2 + (uint32_t)n0 * 2 + (lane & 1) * 16;
  // x block b: slot position l holds row 16b + l%16, k group l/16; rows past M
  // point past x and leave their LDS bytes untouched
  uint32_t x_lane[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int row = b * 16 + (lane & 15);
    x_lane[b] = row < M ? (uint32_t)row * K * 2 + (lane >> 4) * 16 : 0x80000000u;
  }
  uint16_t* ring = smem + wq * D * kSlot;
  auto issue = [&](int i, int slot) {
    const uint32_t k0 = (uint32_t)((i * 4 + wq) * 32);
    uint16_t* sp = ring + slot * kSlot;
    dma16(wr, sp, w_lane + k0 * (uint32_t)N * 2, 0);
#pragma unroll
    for (int b = 0; b < MB; ++b) dma16(xr, sp + (1 + b) * 512, x_lane[b] + k0 * 2, 0);
  };
  // B operand: lane group g holds k rows 8g..8g+7 of column l%16
  const int bg = lane >> 4, bp = lane & 15;
  const int b_off = (16 * (bg >> 1) + 4 * (bg & 1) + (bp >> 2)) * kS16BN + 4 * (bp & 3);

  f32x4_t acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = f32x4_t{};

  static_for<0, D>([&](auto j) {
    if (j < nst) issue(j, j);
  });
  for (int i0 = 0; i0 < nst; i0 += D) {
    static_for<0, D>([&](auto j) {
      const int i = i0 + j;
      if (i < nst) {
        if (i + D - 1 < nst) wait_vmcnt<kAhead>();
        else wait_vmcnt<0>();
        const uint16_t* sp = ring + j * kSlot;
        const u32x4_t bf = lds_tr16_pair<8 * kS16BN * 2>(sp + b_off);
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[b] = mfma16_bf16(ld16(sp + (1 + b) * 512 + lane * 8), bf, acc[b]);
        if (i + D < nst) {
          wait_lgkm0();
          issue(i + D, j);
        }
      }
    });
  }
  wait_vmcnt<0>();

  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wq * MB + b) * 4 + e) * 64 + lane] = acc[b][e];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < MB; ++q) {
    const int idx = q * kS16Threads + tid;  // (b, e, lane) with lane fastest
    const int ln = idx & 63, e = (idx >> 6) & 3, b = idx >> 8;
    float v = red[idx];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) v += red[wv * MB * 256 + idx];
    const int m = b * 16 + 4 * (ln >> 4) + e, n = n0 + (ln & 15);
    if (m < M) {
      const uint16_t r = f32_to_bf16(v + (bias ? bf16_to_f32(bias[n]) : 0.0f));
      out[(int64_t)m * N + n] = r;
      append_store(app, m, n, r);
    }
  }
}

template <int MB, int D>
static hipError_t launch_stream16(const void* x, const void* w, const void* bias, void* out, int M, int K, int N,
                                  hipStream_t s, const KvAppend& app) {
  auto kern = qkv_gemm_stream16_kernel<MB, D>;
  const size_t lds = (size_t)4 * D * (1 + MB) * 512 * sizeof(uint16_t);
  static_assert((size_t)4 * D * (1 + MB) * 512 * 2 >= (size_t)4 * MB * 4 * 64 * 4, "reduction fits");
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(N / kS16BN)), dim3(kS16Threads), lds, s, (const uint16_t*)x,
                     (const uint16_t*)w, (const uint16_t*)bias, (uint16_t*)out, M, K, N, app);
  return hipGetLastError();
}

// Sum the k-range partials in a fixed order, add the bias, round to bf16.  The
// loads of 8 k ranges are issued together (branch-free: buffer loads past the
// end return zeros), so the kernel waits for one memory round trip per 8
// ranges rather than one per range.
constexpr int kMaxKsplit = 16;
__global__ __launch_bounds__(256) void qkv_gemm_reduce_kernel(const float* __restrict__ part,
                                                              const uint16_t* __restrict__ bias,
                                                              uint16_t* __restrict__ out, int M, int N,
                                                              int ksplit, KvAppend app) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // 4 consecutive outputs
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  const int n = (int)(i % N);
  // loads past the last k range fall outside the buffer and read zeros
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(part, (uint32_t)(ksplit * total * 4));
  f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < ksplit; k0 += 8) {
    u32x4_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = bld16(pr, (uint32_t)(((int64_t)(k0 + k) * total + i) * 4));
#pragma unroll
    for (int k = 0; k < 8; ++k) s += __builtin_bit_cast(f32x4_t, v[k]);
  }
  u32x2_t pk;
  const float b0 = bias ? bf16_to_f32(bias[n]) : 0.0f, b1 = bias ? bf16_to_f32(bias[n + 1]) : 0.0f;
  const float b2 = bias ? bf16_to_f32(bias[n + 2]) : 0.0f, b3 = bias ? bf16_to_f32(bias[n + 3]) : 0.0f;
  pk[0] = pack_bf16(s[0] + b0, s[1] + b1);
  pk[1] = pack_bf16(s[2] + b2, s[3] + b3);
  st8(out + i, pk);
  // four consecutive columns never straddle the K/V boundaries (multiples of d)
  if (app.k_cache != nullptr && n >= app.kcol) {
    const int m = (int)(i / N), len = app.seq_lens[m];
    if (len >= 1 && len <= app.L_max) {
      const bool is_k = n < app.vcol;
      uint16_t* cache = static_cast<uint16_t*>(is_k ? app.k_cache : app.v_cache);
      st8(cache + ((int64_t)m * app.L_max + (len - 1)) * (app.vcol - app.kcol) + (n - (is_k ? app.kcol : app.vcol)),
          pk);
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN, int KS>
static hipError_t launch_gemm_bf16(const void* x, const void* w, const void* bias, void* out,
                                   int M, int K, int N, hipStream_t s, const KvAppend& app) {
  using C = GemmCfg<BM, BN, BK, WM, WN, KS>;
  const size_t lds = 2 * C::kLdsTile * sizeof(uint16_t);
  auto kern = qkv_gemm_bf16_kernel<BM, BN, BK, WM, WN, KS>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  const int nblk = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(C::kThreads), lds, s, (const uint16_t*)x,
                     (const uint16_t*)w, (const uint16_t*)bias, (uint16_t*)out, M, K, N, app);
  return hipGetLastError();
}

SkinnyPlan plan_skinny(int64_t M, int64_t K, int64_t N) {
  SkinnyPlan p{};
  // 32-bit buffer offsets cover W and x
  if (M > 128 || N % kSkBN != 0 || K * N * 2 >= ((int64_t)1 << 31) || M * K * 2 >= ((int64_t)1 << 31)) return p;
  p.nbm = (int)((M + 31) / 32);
  // 16-column streaming kernel, no k split: used where its one workgroup per
  // 16 columns does not exceed one per CU.  On wider W its 32-byte row pieces
  // (a quarter of a cache line per workgroup) stream worse than the skinny
  // kernel with a k split plus the reduce kernel (measured at N = 5120..12288).
  if (M <= 32 && K % 128 == 0 && N % kS16BN == 0 && N / kS16BN <= 256) {
    p.stream16 = true;
    p.krange = (int)K;
    p.ksplit = 1;
    p.ok = true;
    return p;
  }
  const int64_t base = (N / kSkBN) * p.nbm;
  // about three workgroups per CU; each k range a multiple of the 128-deep chunk
  // and at most kSkMaxChunks chunks
  int64_t ks = (768 + base - 1) / base;
  const int64_t kmin = (K + kSkMaxChunks * kSkBK - 1) / (kSkMaxChunks * kSkBK);
  const int64_t kmax = (K + 255) / 256;
  if (ks > kmax) ks = kmax;
  if (ks > kMaxKsplit) ks = kMaxKsplit;
  if (ks < kmin) ks = kmin;
  if (ks < 1) ks = 1;
  int64_t kr = (K + ks - 1) / ks;
  kr = (kr + kSkBK - 1) / kSkBK * kSkBK;
  p.krange = (int)kr;
  p.ksplit = (int)((K + kr - 1) / kr);
  if (p.ksplit * M * N * 4 >= ((int64_t)1 << 31)) return SkinnyPlan{};  // partials in 32-bit offsets
  p.ws_bytes = p.ksplit > 1 ? (size_t)p.ksplit * M * N * 4 : 0;
  p.ok = true;
  return p;
}

hipError_t launch_qkv_gemm(const void* x, const void* w, const void* bias, void* out, int64_t M,
                           int64_t K, int64_t N, bool bf16, void* ws, size_t ws_bytes, hipStream_t s,
                           const KvAppend& app) {
  if (!bf16) {
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(qkv_gemm_f32_kernel, grid, dim3(256), 0, s, (const float*)x, (const float*)w,
                       (const float*)bias, (float*)out, (int)M, (int)K, (int)N, app);
    return hipGetLastError();
  }
  const int m = (int)M, k = (int)K, n = (int)N;
  const SkinnyPlan p = plan_skinny(M, K, N);
  if (p.ok && p.stream16)
    return M > 16 ? launch_stream16<2, 6>(x, w, bias, out, m, k, n, s, app)
                  : launch_stream16<1, 8>(x, w, bias, out, m, k, n, s, app);
  if (p.ok && (p.ksplit == 1 || (ws != nullptr && ws_bytes >= p.ws_bytes))) {
    const int64_t nblk = (N / kSkBN) * p.nbm * p.ksplit;
    hipLaunchKernelGGL(qkv_gemm_skinny_kernel, dim3((unsigned)nblk), dim3(kSkThreads), 0, s,
                       (const uint16_t*)x, (const uint16_t*)w, (const uint16_t*)bias, (uint16_t*)out,
                       (float*)ws, m, k, n, p.krange, p.ksplit, p.nbm, app);
    if (p.ksplit > 1) {
      const int64_t quads = (M * N + 3) / 4;
      hipLaunchKernelGGL(qkv_gemm_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s,
                         (const float*)ws, (const uint16_t*)bias, (uint16_t*)out, m, n, p.ksplit, app);
    }
    return hipGetLastError();
  }
#ifndef MQKV_GEMM_CF
#define MQKV_GEMM_CF 1
#endif
  if (MQKV_GEMM_CF && K % kCfBK == 0 && N % 8 == 0 && (uint64_t)K * N * 2 < 0x80000000ull) {
    const int64_t t128 = ((M + 127) / 128) * ((N + kCfBN - 1) / kCfBN);
    if (t128 >= 256) return launch_gemm_cf<128>(x, w, bias, out, m, k, n, s, app);
    if (M > 128) return launch_gemm_cf<64>(x, w, bias, out, m, k, n, s, app);
  }
  // Pick the largest tile that still gives the chip (256 CUs) a full wave of workgroups.
  const int64_t big = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t mid = ((M + 63) / 64) * ((N + 63) / 64);
  if (big >= 256) return launch_gemm_bf16<128, 128, 64, 2, 2, 1>(x, w, bias, out, m, k, n, s, app);
  if (M > 32 && mid >= 128) return launch_gemm_bf16<64, 64, 64, 2, 2, 1>(x, w, bias, out, m, k, n, s, app);
  return launch_gemm_bf16<32, 32, 256, 1, 1, 4>(x, w, bias, out, m, k, n, s, app);
}

}  // namespace mqkv
