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
//  * M <= 128, K % 256 == 0, N % 64 == 0 (for M <= 32 only on wide weights):
//    8-wave workgroups over all of K, each wave streaming its own share of the
//    rows, the waves' sums added in LDS (one kernel);
//  * M <= 128 otherwise: register-staged skinny kernel, k split over
//    workgroups with a fixed-order reduce kernel;
//  * M > 128, K % 64 == 0, N % 8 == 0: LDS-DMA fed tiles (128 or 64 rows, 128
//    or 160 columns, picked so the tiles fill the CUs), the W tile kept
//    row-major and read with transposing LDS loads;
//  * anything else: register-prefetched tiles with W transposed into LDS by
//    the loading threads.
// fp32 path: plain LDS-tiled fp32 FMA (a correctness path for the tiny fp32 layer).
//
// Every kernel's epilogue can also rotate the Q and K heads (rotary position
// embedding, see ProjEpilogue) before the output is rounded, and append the
// new token's K and V rows to the KV caches.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace mqkv {

// The append epilogue for one output element (see ProjEpilogue): a no-op unless an
// append is requested, n is a K or V column and row m's position is valid.
template <typename T>
__device__ __forceinline__ void append_store(const ProjEpilogue& a, int m, int n, T v) {
  if (a.k_cache == nullptr || n < a.kcol) return;
  const int len = a.seq_lens[m];
  if (len < 1 || len > a.L_max) return;
  const bool is_k = n < a.vcol;
  T* cache = static_cast<T*>(is_k ? a.k_cache : a.v_cache);
  cache[((int64_t)m * a.L_max + (len - 1)) * (a.vcol - a.kcol) + (n - (is_k ? a.kcol : a.vcol))] = v;
}

// ----------------------------------------------------------------------------- rotary embedding
// sin and cos of a (radians).  Cody and Waite's argument reduction: a = k pi/2
// + r with k the integer nearest a 2/pi and r = a - k P1 - k P2, pi/2 = P1 + P2
// split into its fp32 value and the fp32 remainder; each product is exact
// inside its FMA, so r carries an error near one ulp of r plus k times the
// 2.6e-15 left of pi/2 (1e-8 at |a| = 2^22).  On |r| <= pi/4 the Taylor series
// of sin to r^9 and of cos to r^10 are within 3e-9; k mod 4 picks and signs them.
__device__ __forceinline__ void rope_sincos(float a, float& s, float& c) {
  const float k = __builtin_rintf(a * 0.636619772367581343f);
  float r = __builtin_fmaf(-k, 1.57079637050628662109375f, a);
  r = __builtin_fmaf(-k, -4.37113900018624283e-8f, r);
  const float r2 = r * r;
  float ps = __builtin_fmaf(r2, 2.75573192239858907e-6f, -1.98412698412698413e-4f);
  ps = __builtin_fmaf(r2, ps, 8.33333333333333333e-3f);
  ps = __builtin_fmaf(r2, ps, -1.66666666666666667e-1f);
  ps = __builtin_fmaf(r2 * r, ps, r);
  float pc = __builtin_fmaf(r2, -2.75573192239858907e-7f, 2.48015873015873016e-5f);
  pc = __builtin_fmaf(r2, pc, -1.38888888888888889e-3f);
  pc = __builtin_fmaf(r2, pc, 4.16666666666666667e-2f);
  pc = __builtin_fmaf(r2, pc, -0.5f);
  pc = __builtin_fmaf(r2, pc, 1.0f);
  const int q = (int)k;
  const float sq = (q & 1) ? pc : ps, cq = (q & 1) ? ps : pc;
  s = (q & 2) ? -sq : sq;
  c = ((q + 1) & 2) ? -cq : cq;
}

// The value held by the neighbouring lane (lane ^ 1).  In every output layout
// here a lane's partner column n ^ 1 is held by that lane, for the same rows.
// Both lanes of a pair must be active.
__device__ __forceinline__ float pair_partner(float v) {
  // DPP quad_perm [1, 0, 3, 2]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ int rope_position(const ProjEpilogue& e, int m) {
  if (e.pos) return e.pos[m];
  return min(max(e.seq_lens[m] - 1, 0), e.L_max - 1);
}

// Column n (a Q or K column) of a row at position p: v is its value, w the
// value of the other column of its plane (n ^ 1), th the plane's frequency.
__device__ __forceinline__ float rope_turn(float v, float w, int n, int p, float th) {
  float sn, cs;
  rope_sincos((float)p * th, sn, cs);
  return __builtin_fmaf(w, (n & 1) ? sn : -sn, v * cs);
}

__device__ __forceinline__ float rope_freq(const ProjEpilogue& e, int n) {
  return e.inv_freq[(n & (e.rope_d - 1)) >> 1];
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
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int K, int N, ProjEpilogue app) {
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
    if (gn >= N) continue;  // N is even: both columns of a plane are in or out
    const float bv = bias ? bf16_to_f32(bias[gn]) : 0.0f;
    const bool rot = app.inv_freq != nullptr && gn < app.vcol;  // uniform over 32 columns
    const float th = rot ? rope_freq(app, gn) : 0.0f;
#pragma unroll
    for (int i = 0; i < C::kMI; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gm = m0 + wm * (BM / WM) + i * 32 + 8 * (e / 4) + 4 * hf + (e % 4);
        float v = acc[i][j][e] + bv;
        if (rot) {
          const float w = pair_partner(v);
          if (gm < M) v = rope_turn(v, w, gn, rope_position(app, gm), th);
        }
        if (gm < M) {
          const uint16_t r = f32_to_bf16(v);
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
                                                           int N, ProjEpilogue app) {
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
  const int gn0 = n0 + tx * 4;  // 4 columns: two whole planes, all on one side of vcol
  const bool rot = app.inv_freq != nullptr && gn0 < app.vcol;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
    float r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = gn0 + j < N ? acc[i][j] + (bias ? bias[gn0 + j] : 0.0f) : 0.0f;
    if (rot) {
      const int p = rope_position(app, gm);
      float t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = rope_turn(r[j], r[j ^ 1], gn0 + j, p, rope_freq(app, gn0 + j));
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = t[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = gn0 + j;
      if (gn < N) {
        out[(int64_t)gm * N + gn] = r[j];
        append_store(app, gm, gn, r[j]);
      }
    }
  }
}

// ----------------------------------------------------------------------------- copy-fed tiles
// Workgroup tile BM x BN, k tile 64, WM x WN x KW waves: WM x WN positions of
// (32 MI) x (32 NI) blocks of 32x32x16 MFMAs, each position held by KW waves
// that take the 16-deep k steps of every k tile in turn (KW = 2 puts two
// waves on every SIMD of a 4-position tile, which hides the operand-read and
// barrier latency of one wave behind the other's MFMAs); their sums are added
// through LDS at the end.  Both operand tiles reach LDS by LDS-DMA (buffer
// loads that write LDS directly, no staging registers) into a ring of ST
// stages, the copies of a tile issued ST-1 tiles ahead of its use; one barrier
// per k tile publishes the copies and frees the stage being refilled.
//  * x tile: BM rows of 64 k (k-contiguous) + 16 bytes of padding per row;
//  * W tile: 64 rows of BN n (n-contiguous, as W is stored), row pitch
//    padded to 16 dwords past a multiple of 64.  The MFMA B operand (8
//    consecutive k of one n per lane) is read with the transposing LDS load
//    ds_read_b64_tr_b16: within each 16 lanes, lane 4j+q reads 4 n of k-row j
//    and lane i receives column i of the 4 rows, so no VALU transposition is
//    needed.
// The row pitches keep both operand reads on distinct LDS banks (x: 36 dwords
// per row; W: consecutive k rows 16 banks apart, the lane groups of a read 8
// banks apart); the lanes of a copy that fall on padding point past the
// buffer, so they fetch nothing and land only on padding bytes, which are
// never read.  Every stage of the ring is an LDS array of its own, and the
// operand reads are compiler builtins: the compiler then knows which stage
// each read and each copy touches, so it waits only for the copies into the
// stage being read (which the explicit per-tile wait has already retired) and
// is free to issue the next k step's reads under the current step's MFMAs.
// The epilogue stages the sums in LDS in 32-row passes over the freed stages
// and writes 16-byte row pieces.  Requires K % 64 == 0.
constexpr int kTBK = 64;
constexpr int kTXld = kTBK + 8;  // x tile row pitch (bf16): 9 chunks of 16 B
// W tile row pitch (bf16) for BN columns: the data rounded up to 16 dwords
// past a multiple of 64 dwords
constexpr int tile_wpitch(int bn) {
  int p = bn / 2;
  while (p % 64 != 16) ++p;
  return p * 2;
}
template <int BM, int BN, int WM, int WN, int KW, int ST>
struct TileCfg {
  static constexpr int kNW = WM * WN * KW;  // waves
  static constexpr int kThreads = kNW * 64;
  static constexpr int kMI = BM / WM / 32;  // 32-row MFMA blocks per wave
  static constexpr int kNI = BN / WN / 32;  // 32-column MFMA blocks per wave
  static constexpr int kKS = kTBK / 16 / KW;  // k steps per wave per k tile
  static constexpr int kWld = tile_wpitch(BN);
  static constexpr int kX = BM * kTXld;
  static constexpr int kW = kTBK * kWld;
  static constexpr int kSink = kX + kW;    // 1 KB past the tiles: where surplus copies land
  static constexpr int kStage = kX + kW + 512;
  static constexpr int kXChunks = kTXld / 8, kWChunks = kWld / 8;  // 16-byte chunks per row
  static constexpr int kXCopies = kX * 2 / 1024, kWCopies = kW * 2 / 1024;
  static constexpr int kXcp = (kXCopies + kNW - 1) / kNW, kWcp = (kWCopies + kNW - 1) / kNW;  // per wave
  static constexpr int kCopies = kXcp + kWcp;  // DMA instructions of every wave per k tile
  static constexpr size_t kBytes = (size_t)ST * kStage * sizeof(uint16_t);
  static_assert(kMI * WM * 32 == BM && kNI * WN * 32 == BN && kKS * KW * 16 == kTBK, "wave layout");
  static_assert(kX * 2 % 1024 == 0 && kW * 2 % 1024 == 0, "tiles are whole 1 KB copies");
  static_assert(kBytes <= 160 * 1024, "LDS");
};

// B-operand half of a 32x32x16 MFMA from a row-major W tile in LDS: a
// transposing read of 4 k rows (lane 4j+q of each 16-lane group reads 4
// columns of row j, lane i receives column i of the 4 rows).  As a builtin the
// compiler knows which LDS array it reads and orders it after exactly the
// copies into that array.
__device__ __forceinline__ u32x2_t lds_tr16(const uint16_t* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p)));
}
// Compiler-level fence around a bare s_barrier: keeps LDS accesses on their
// side of it (the barrier builtin alone does not order memory for the
// optimizer).
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// B operand of a 32x32x16 MFMA from a row-major W tile: two transposing reads
// (k rows r and r+4 of this lane's group; HI_BYTES apart) that wait for
// themselves (the 16-column streaming kernel's reads).  Written as one asm
// block because the compiler treats the builtin form as aliasing every LDS-DMA
// copy in flight and waits for all of them first, which would serialize the
// copy pipeline; the callers order these reads after the copies they need
// with their own vmcnt waits.
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

// s_waitcnt immediate: vmcnt(n), expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// cos and sin of the rotation angle of every (row, plane) of a BM-row tile:
// (cos, sin) of row r, plane i at tab[r * pitch + i], P = d / 2 planes;
// rows past M take position 0.  Thread t fills planes 4g .. 4g + 3, g = t mod
// (P / 4), of rows t / (P / 4) + k * THREADS / (P / 4).  Its positions and
// frequencies are loaded by prefetch() before the main loop, so that their
// latency hides under it; fill() evaluates the angles with the arithmetic of
// rope_turn, so every kernel rotates alike.
template <int BM, int THREADS>
struct RopeTable {
  static constexpr int kMaxRows = BM * 16 / THREADS;  // rows per thread at P = 64
  static_assert(kMaxRows >= 1 && BM * 8 % THREADS == 0, "table split");
  int pos[kMaxRows];
  float th[4];
  __device__ __forceinline__ void prefetch(const ProjEpilogue& app, int m0, int M, int tid) {
    const int groups = app.rope_d >> 3, rows = BM * groups / THREADS;  // groups = P / 4
    const int g = tid % groups, q = tid / groups;
#pragma unroll
    for (int c = 0; c < 4; ++c) th[c] = app.inv_freq[4 * g + c];
#pragma unroll
    for (int k = 0; k < kMaxRows; ++k) {
      const int m = m0 + q + k * (THREADS / groups);
      pos[k] = (k < rows && m < M) ? rope_position(app, m) : 0;
    }
  }
  // the rows [r0, r0 + nr) of the table, at tab[(row - r0) * pitch + plane]
  __device__ __forceinline__ void fill(const ProjEpilogue& app, float2* tab, int pitch, int tid, int r0,
                                       int nr) const {
    const int P = app.rope_d >> 1, groups = P >> 2, rows = BM * groups / THREADS;
    const int g = tid % groups, q = tid / groups;
#pragma unroll
    for (int k = 0; k < kMaxRows; ++k) {
      if (k >= rows) break;
      const int row = q + k * (THREADS / groups);
      if (row < r0 || row >= r0 + nr) continue;
      float2 cs[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) rope_sincos((float)pos[k] * th[c], cs[c].y, cs[c].x);
      float2* dst = tab + (row - r0) * pitch + 4 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[c] = cs[c];
    }
  }
};

// Epilogue passes: the tile's rows are handled 32 at a time.  In a pass, the
// k-step group g of every 32-row block in it writes its fp32 sums to stage g
// (rows of BN + 8 floats: rows 4 apart fall 32 banks apart), the rotation
// table of the pass's rows goes to stage KW (rows of d/2 + 2 float2) followed
// by the tile's bias (BN bf16); then every thread takes 8-column row pieces.
constexpr int kEpiRows = 32;
template <int BM, int BN, int WM, int WN, int KW, int ST>
struct TileEpiFit {
  using L = TileCfg<BM, BN, WM, WN, KW, ST>;
  static constexpr int kPitch = BN + 8;
  static constexpr size_t kStageBytes = (size_t)L::kStage * 2;
  static_assert(KW + 1 <= ST, "a stage per k-step group plus one for the table");
  static_assert((size_t)kEpiRows * kPitch * 4 <= kStageBytes, "staging rows fit a stage");
  static_assert((size_t)kEpiRows * (128 / 2 + 2) * 8 + BN * 2 <= kStageBytes, "table and bias fit a stage");
};

template <int BM, int BN, int WM, int WN, int KW, int ST>
__global__ __launch_bounds__(WM * WN * KW * 64, 1) void qkv_gemm_tiles_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ out, int M, int K, int N, ProjEpilogue app) {
  using L = TileCfg<BM, BN, WM, WN, KW, ST>;
  using EF = TileEpiFit<BM, BN, WM, WN, KW, ST>;
  constexpr int MI = L::kMI, NI = L::kNI, NW = L::kNW;
  static_assert(ST >= 2 && ST <= 4, "ring of 2 to 4 stages");
  // the ring: one LDS array per stage (unused arrays take 16 bytes)
  __shared__ __align__(16) uint16_t ring0[L::kStage];
  __shared__ __align__(16) uint16_t ring1[L::kStage];
  __shared__ __align__(16) uint16_t ring2[ST > 2 ? L::kStage : 8];
  __shared__ __align__(16) uint16_t ring3[ST > 3 ? L::kStage : 8];
  auto stage = [&](auto sidx) -> uint16_t* {
    constexpr int i = decltype(sidx)::value;
    if constexpr (i == 0) return ring0;
    else if constexpr (i == 1) return ring1;
    else if constexpr (i == 2) return ring2;
    else return ring3;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wq = __builtin_amdgcn_readfirstlane(wave);
  const int pos = wave % (WM * WN), kg = wave / (WM * WN);  // tile position, k-step group
  const int wm = pos / WN, wn = pos % WN;
  const int l32 = lane & 31, hf = lane >> 5;

  const int nbn = (N + BN - 1) / BN, nbm = (M + BM - 1) / BM;
  // Tiles in groups of kGM row tiles, column-major inside a group: an XCD's
  // contiguous share of ids covers a few columns of a few row tiles, so both
  // the x rows and the W columns it reads are reused in its L2 (one row of
  // tiles per XCD would stream all of W through every XCD).
  constexpr int kGM = 8;
  const int lid = xcd_remap(blockIdx.x, nbn * nbm);
  const int grp = lid / (kGM * nbn), goff = lid % (kGM * nbn), gm0 = grp * kGM, gsz = min(kGM, nbm - gm0);
  const int bm = gm0 + goff % gsz, bn = goff / gsz;
  const int m0 = bm * BM, n0 = bn * BN;
  const int nk = K / kTBK;
  // rotary embedding: this thread's positions and frequencies, loaded now
  const bool rope = app.inv_freq != nullptr && n0 < app.vcol;  // uniform over the workgroup
  RopeTable<BM, L::kThreads> rtab;
  if (rope) rtab.prefetch(app, m0, M, tid);

  // ---- copy maps: slot (copy * 64 + lane) of a tile image -> global byte offset
  constexpr uint32_t kNoCopy = 0x80000000u;
  const uint32_t xrow = (uint32_t)K * 2, wrow = (uint32_t)N * 2;
  uint32_t xoff[L::kXcp], woff[L::kWcp];
#pragma unroll
  for (int i = 0; i < L::kXcp; ++i) {
    const int slot = (wave + NW * i) * 64 + lane;
    const int r = slot / L::kXChunks, ch = slot % L::kXChunks;
    xoff[i] = (ch < kTBK / 8 && wave + NW * i < L::kXCopies) ? (uint32_t)r * xrow + ch * 16 : kNoCopy;
  }
#pragma unroll
  for (int i = 0; i < L::kWcp; ++i) {
    const int slot = (wave + NW * i) * 64 + lane;
    const int r = slot / L::kWChunks, ch = slot % L::kWChunks;
    // chunks of columns at or past N (a ragged last tile) fetch nothing: their
    // LDS columns feed only outputs that are not stored
    woff[i] = (ch < BN / 8 && n0 + ch * 8 < N && wave + NW * i < L::kWCopies) ? (uint32_t)r * wrow + ch * 16
                                                                              : kNoCopy;
  }
  // x rows at or past M and W rows past K lie past their buffer ends: they
  // fetch nothing, and their LDS rows only feed outputs that are not stored.
  const uint64_t xbytes = (uint64_t)M * K * 2, wbytes = (uint64_t)K * N * 2;
  // Every wave issues exactly L::kCopies copies per k tile, unconditionally:
  // a wave's surplus copies fetch nothing (all offsets past the buffer) into
  // the stage's sink, and the tiles past the last one (kt >= nk: the ring
  // runs whole rounds) fetch nothing into a stage no tile reads again.  So
  // one constant vmcnt retires a tile, and the compiler, which sees every
  // copy and which stage it fills, needs no waits of its own before the reads.
  auto copy_tile = [&](int kt, uint16_t* xs) {
    uint16_t* ws = xs + L::kX;
    const bool live = kt < nk;
    const uint64_t xb = live ? (uint64_t)m0 * K * 2 + (uint64_t)kt * kTBK * 2 : 0;
    const uint64_t wb = live ? (uint64_t)kt * kTBK * N * 2 + (uint64_t)n0 * 2 : 0;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(reinterpret_cast<const char*>(x) + xb,
                                                live ? (uint32_t)min(xbytes - xb, (uint64_t)0x7fffffff) : 0u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(reinterpret_cast<const char*>(w) + wb,
                                                live ? (uint32_t)min(wbytes - wb, (uint64_t)0x7fffffff) : 0u);
#pragma unroll
    for (int i = 0; i < L::kXcp; ++i) {
      const int cp = wq + NW * i;
      dma16(xr, cp < L::kXCopies ? xs + cp * 512 : xs + L::kSink, xoff[i], 0);
    }
#pragma unroll
    for (int i = 0; i < L::kWcp; ++i) {
      const int cp = wq + NW * i;
      dma16(wr, cp < L::kWCopies ? ws + cp * 512 : xs + L::kSink, woff[i], 0);
    }
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x16_t{};

  // operand fragments of one 16-deep k step: MI x-row fragments (A), NI
  // transposed W pairs (B: k rows r and r + 4 of the lane's group)
  const int bg = lane >> 4, bp = lane & 15;  // transposing-read lane group
  const int b_n = 16 * (bg & 1) + 4 * (bp & 3), b_k = 8 * (bg >> 1) + (bp >> 2);
  // Every read indexes its stage array directly (one index, no chain of
  // derived pointers), so the compiler keeps track of which array it reads.
  const int a_idx = (wm * (32 * MI) + l32) * kTXld + hf * 8;
  const int b_idx = L::kX + b_k * L::kWld + wn * (32 * NI) + b_n;
  auto frags = [&](const uint16_t* st, int ks, u32x4_t (&a)[MI], u32x4_t (&b)[NI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i) a[i] = ld16(st + (a_idx + ks * 16 + i * 32 * kTXld));
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int o = b_idx + ks * 16 * L::kWld + j * 32;
      const u32x2_t lo = lds_tr16(st + o), hi = lds_tr16(st + (o + 4 * L::kWld));
      b[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
  };

  static_for<0, ST - 1>([&](auto s) { copy_tile(s, stage(s)); });
  // The k loop, unrolled over the ring so that every stage is named statically;
  // it runs whole rounds of ST tiles, those past the last one without reads or
  // MFMAs.
  for (int kt0 = 0; kt0 < nk; kt0 += ST) {
    static_for<0, ST>([&](auto s) {
      const int kt = kt0 + s;
      // Tile kt is in LDS once every wave has waited for its own copies of it
      // and passed the barrier, which also tells that every wave's reads of
      // the previous tile are done, so its stage may be refilled.  A bare
      // barrier: __syncthreads' fence would also wait for the copies of the
      // later tiles, which would leave one tile of lookahead whatever ST is.
      wait_vmcnt<(ST - 2) * L::kCopies>();
      bare_barrier();
      constexpr int sn = (s + ST - 1) % ST;
      copy_tile(kt + ST - 1, stage(std::integral_constant<int, sn>{}));
      if (kt < nk) {  // uniform
        const uint16_t* st = stage(s);
        u32x4_t a[2][MI], b[2][NI];
        frags(st, kg, a[0], b[0]);
        static_for<0, L::kKS>([&](auto kk) {
          constexpr int cur = kk & 1;
          if constexpr (kk + 1 < L::kKS) frags(st, (kk + 1) * KW + kg, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) acc[i][j] = mfma32_bf16(a[cur][i], b[cur][j], acc[i][j]);
        });
      }
    });
  }

  // ---- epilogue, in passes of 32 rows over the freed stages: k-step group g
  // writes its sums to stage g, the rotation table and the bias go to stage
  // KW; then every thread takes 8-column row pieces of the pass, adds the
  // groups' sums in group order (a fixed order, so the result does not depend
  // on timing), adds the bias, rotates, rounds to bf16 and writes one 16-byte
  // piece (and the cache append).  A piece holds 4 whole planes of one head,
  // so the rotation needs nothing from other threads.
  constexpr int kPitch = EF::kPitch;
  float2* tab = reinterpret_cast<float2*>(stage(std::integral_constant<int, KW>{}));
  const int tpitch = (app.rope_d >> 1) + 2;  // float2 per table row: 16-byte aligned rows
  // rows of the table filled at once: as many whole 32-row passes as the stage
  // holds beside the bias (all 128 at d = 64), so fewer passes pay for a fill
  int tb_rows = kEpiRows;
  while (tb_rows * 2 <= BM && (size_t)tb_rows * 2 * tpitch * 8 + BN * 2 <= EF::kStageBytes) tb_rows *= 2;
  uint16_t* bstg = reinterpret_cast<uint16_t*>(tab + (rope ? tb_rows * tpitch : 0));
  constexpr int kPieces = kEpiRows * BN / 8, kPerRow = BN / 8;
  wait_vmcnt<0>();  // the copies past the last tile (nothing fetched) have landed
  static_for<0, BM / kEpiRows>([&](auto ps) {
    constexpr int r0 = ps * kEpiRows;
    // every wave is done with the ring, or with the previous pass's rows
    wait_lgkm0();
    bare_barrier();
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (wm * (32 * MI) + i * 32 != r0) continue;  // the pass is one 32-row block
      static_for<0, KW>([&](auto g) {
        if (kg == g) {
          float* stg = reinterpret_cast<float*>(stage(g));
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              stg[(8 * (e / 4) + 4 * hf + (e % 4)) * kPitch + wn * (32 * NI) + j * 32 + l32] = acc[i][j][e];
        }
      });
    }
    const int tb0 = r0 - r0 % tb_rows;  // first row of the table block holding this pass
    if (rope && r0 == tb0) rtab.fill(app, tab, tpitch, tid, r0, tb_rows);
    if (bias && tid < BN / 8 && n0 + tid * 8 < N) st16(bstg + tid * 8, ld16(bias + n0 + tid * 8));
    wait_lgkm0();
    bare_barrier();

#pragma unroll
    for (int k = 0; k < (kPieces + L::kThreads - 1) / L::kThreads; ++k) {
      const int c = tid + k * L::kThreads, r = c / kPerRow, cg = c % kPerRow;
      const int gm = m0 + r0 + r, gn = n0 + cg * 8;
      if (c >= kPieces || gm >= M || gn >= N) continue;  // N % 8 == 0: a piece is wholly in or out
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      static_for<0, KW>([&](auto g) {
        const float* stg = reinterpret_cast<const float*>(stage(g)) + r * kPitch + cg * 8;
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(stg);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(stg + 4);
        if constexpr (g == 0) {
          v[0] = lo[0], v[1] = lo[1], v[2] = lo[2], v[3] = lo[3];
          v[4] = hi[0], v[5] = hi[1], v[6] = hi[2], v[7] = hi[3];
        } else {
          v[0] += lo[0], v[1] += lo[1], v[2] += lo[2], v[3] += lo[3];
          v[4] += hi[0], v[5] += hi[1], v[6] += hi[2], v[7] += hi[3];
        }
      });
      if (bias) {
        const u32x4_t bb = ld16(bstg + cg * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] += __builtin_bit_cast(float, bb[q] << 16);
          v[2 * q + 1] += __builtin_bit_cast(float, bb[q] & 0xffff0000u);
        }
      }
      if (rope && gn < app.vcol) {
        const float2* t = tab + (r0 - tb0 + r) * tpitch + ((gn & (app.rope_d - 1)) >> 1);
        const f32x4_t c01 = *reinterpret_cast<const f32x4_t*>(t), c23 = *reinterpret_cast<const f32x4_t*>(t + 2);
        const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};  // (cos, sin) x 4
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x0 = v[2 * q], x1 = v[2 * q + 1], cq = cs[2 * q], sq = cs[2 * q + 1];
          v[2 * q] = __builtin_fmaf(x1, -sq, x0 * cq);      // rope_turn of the even column
          v[2 * q + 1] = __builtin_fmaf(x0, sq, x1 * cq);   // and of the odd one
        }
      }
      const u32x4_t pk = u32x4_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                                 pack_bf16(v[6], v[7])};
      st16(out + (int64_t)gm * N + gn, pk);
      if (app.k_cache != nullptr && gn >= app.kcol) {  // a piece never straddles the K/V boundaries
        const int len = app.seq_lens[gm];
        if (len >= 1 && len <= app.L_max) {
          const bool is_k = gn < app.vcol;
          uint16_t* cache = static_cast<uint16_t*>(is_k ? app.k_cache : app.v_cache);
          st16(cache + ((int64_t)gm * app.L_max + (len - 1)) * (app.vcol - app.kcol) +
                   (gn - (is_k ? app.kcol : app.vcol)),
               pk);
        }
      }
    }
  });
}

template <int BM, int BN, int WM, int WN, int KW, int ST>
static hipError_t launch_gemm_tiles(const void* x, const void* w, const void* bias, void* out, int M, int K, int N,
                                    hipStream_t s, const ProjEpilogue& app) {
  using L = TileCfg<BM, BN, WM, WN, KW, ST>;
  const int nblk = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((qkv_gemm_tiles_kernel<BM, BN, WM, WN, KW, ST>), dim3(nblk), dim3(L::kThreads), 0, s,
                     (const uint16_t*)x, (const uint16_t*)w, (const uint16_t*)bias, (uint16_t*)out, M, K, N, app);
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
    int nbm, ProjEpilogue app) {
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
    const bool rot = app.inv_freq != nullptr && n0 < app.vcol;  // 32 columns, one side of vcol
    const float th = rot ? rope_freq(app, n) : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 8 * (e >> 2) + 4 * hf + (e & 3);
      float v = acc[e] + bv;
      if (rot) {
        const float w = pair_partner(v);
        if (m < M) v = rope_turn(v, w, n, rope_position(app, m), th);
      }
      if (m < M) {
        const uint16_t r = f32_to_bf16(v);
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

// ----------------------------------------------------------------------------- decode width, register transpose
// M <= 32, K % 256 == 0, N % 64 == 0, too wide for the 16-column stream (the
// grouped-query decode projections): the weight is the whole cost.  MFMA
// 16x16x32 wants eight consecutive k of one column per lane, and W is stored
// k-major, so each lane loads eight 8-byte row pieces (rows kb*8 .. kb*8+7 of
// a 32-row step, columns 4j .. 4j+3) and builds the operands of four MFMAs
// from them with byte permutes: MFMA t takes column 4j + t in lane j.  The
// outputs of the four MFMAs are four interleaved column sets, so nothing
// passes through LDS and no barrier is needed until the end: a wave loads its
// whole slice (NS steps) at once and multiplies as the pieces arrive.  A
// workgroup of 8 waves covers 64 columns and a k range of 8*NS*32 rows (wave
// w: the w-th eighth); the waves' sums are added in LDS in wave order and
// written as one fp32 partial per k range, which qkv_gemm_reduce_kernel adds
// (fixed order) with the bias and epilogue.
constexpr int kRtBN = 64, kRtWaves = 8, kRtStep = 32;

__device__ __forceinline__ u32x2_t bld8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

template <int MB, int NS>
__global__ __launch_bounds__(kRtWaves * 64) void qkv_gemm_rt_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ w,
                                                                    float* __restrict__ part, int M, int K, int N,
                                                                    int nbn) {
  constexpr int R = MB * 16;  // rows of x covered
  __shared__ __align__(16) float red[4 * R * kRtBN];  // four waves' sums
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, kb = lane >> 4;
  // neighbouring column strips of one k range go to one XCD
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bn = lid % nbn, ks = lid / nbn;
  const int n0 = bn * kRtBN;
  const int kw = (ks * kRtWaves + wave) * (NS * kRtStep) + kb * 8;  // this lane's first row of W
  const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((int64_t)K * N * 2));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, xbytes);
  u32x2_t wv[NS][8];
  u32x4_t xv[NS][MB];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      wv[s][r] = bld8(wr, (uint32_t)(((int64_t)(kw + s * kRtStep + r) * N + n0 + 4 * j) * 2));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + j;
      xv[s][mb] = bld16(xr, m < M ? (uint32_t)(((int64_t)m * K + kw + s * kRtStep) * 2) : xbytes);
    }
  }
  f32x4_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mb][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // column 4j + t of rows 0..7: dword q packs rows 2q (low half) and 2q + 1
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
      u32x4_t b;
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = __builtin_amdgcn_perm(wv[s][2 * q + 1][t >> 1], wv[s][2 * q][t >> 1], sel);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][t] = mfma16_bf16(xv[s][mb], b, acc[mb][t]);
    }
  }
  // acc[mb][t][e] = sum for row mb*16 + 4kb + e, column n0 + 4j + t.  The
  // eight waves' sums are added pairwise through LDS in a fixed order (wave w
  // adds wave w + 4's, then w + 2's, then w + 1's, each staged in LDS slot w),
  // and wave 0 writes the partial: four
  // consecutive columns per (row, lane), 16-byte stores.
  auto put = [&](int to) {
    float* dst = red + to * (R * kRtBN) + lane * 4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        st16(dst + (mb * 4 + e) * 256,
             u32x4_t{__float_as_uint(acc[mb][0][e]), __float_as_uint(acc[mb][1][e]), __float_as_uint(acc[mb][2][e]),
                     __float_as_uint(acc[mb][3][e])});
  };
  auto take = [&](int from) {
    const float* src = red + from * (R * kRtBN) + lane * 4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4_t v = __builtin_bit_cast(f32x4_t, ld16(src + (mb * 4 + e) * 256));
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mb][t][e] += v[t];
      }
  };
#pragma unroll
  for (int half = 4; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) put(wave - half);
    __syncthreads();
    if (wave < half) take(wave);
    __syncthreads();
  }
  if (wave != 0) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = mb * 16 + 4 * kb + e;
      if (row < M)
        st16(part + ((int64_t)ks * M + row) * N + n0 + 4 * j,
             u32x4_t{__float_as_uint(acc[mb][0][e]), __float_as_uint(acc[mb][1][e]), __float_as_uint(acc[mb][2][e]),
                     __float_as_uint(acc[mb][3][e])});
    }
}

template <int MB>
static hipError_t launch_rt(const SkinnyPlan& p, const void* x, const void* w, void* ws, int M, int K, int N,
                            hipStream_t s) {
  const int nbn = N / kRtBN;
  const dim3 grid((unsigned)(nbn * p.ksplit)), block(kRtWaves * 64);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, (const uint16_t*)x, (const uint16_t*)w, (float*)ws, M, K, N, nbn);
  };
  switch (p.rt_ns) {
    case 1: args(qkv_gemm_rt_kernel<MB, 1>); break;
    case 2: args(qkv_gemm_rt_kernel<MB, 2>); break;
    default: args(qkv_gemm_rt_kernel<MB, 4>); break;
  }
  return hipGetLastError();
}

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
    uint16_t* __restrict__ out, int M, int K, int N, ProjEpilogue app) {
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
    v += bias ? bf16_to_f32(bias[n]) : 0.0f;
    if (app.inv_freq != nullptr && n0 < app.vcol) {  // 16 columns, one side of vcol
      const float w = pair_partner(v);                // thread tid ^ 1 holds column n ^ 1, row m
      if (m < M) v = rope_turn(v, w, n, rope_position(app, m), rope_freq(app, n));
    }
    if (m < M) {
      const uint16_t r = f32_to_bf16(v);
      out[(int64_t)m * N + n] = r;
      append_store(app, m, n, r);
    }
  }
}

template <int MB, int D>
static hipError_t launch_stream16(const void* x, const void* w, const void* bias, void* out, int M, int K, int N,
                                  hipStream_t s, const ProjEpilogue& app) {
  auto kern = qkv_gemm_stream16_kernel<MB, D>;
  const size_t lds = (size_t)4 * D * (1 + MB) * 512 * sizeof(uint16_t);
  static_assert((size_t)4 * D * (1 + MB) * 512 * 2 >= (size_t)4 * MB * 4 * 64 * 4, "reduction fits");
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(N / kS16BN)), dim3(kS16Threads), lds, s, (const uint16_t*)x,
                     (const uint16_t*)w, (const uint16_t*)bias, (uint16_t*)out, M, K, N, app);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- small M, wide workgroups
// M <= 128 (short prompts, decode batches on wide weights): one kernel, no k split
// across workgroups.  A workgroup of NW waves owns 64 columns of W (whole
// 128-byte lines of each row) and a 16 MB-row tile of the output over all of
// K: wave w streams the K/NW rows [w K/NW, (w + 1) K/NW) of the strip through
// a ring of D LDS slots of its own (32 k rows x 64 columns, 4 KB), filled by
// LDS-DMA D steps ahead, and takes its x fragments (the MFMA A operand, 8
// consecutive k of one row per lane) straight from memory; no barrier until
// the end, where the NW waves' sums are added in LDS in wave order.  MFMA
// 16x16x32.  A slot stores k rows with index bits 2 and 3 swapped (so the
// lanes of a B-operand read pair up k rows 8g..8g+7) and the 16-byte chunks of
// slot row r at positions XOR 2((r >> 1) & 3), which puts the 8 rows a read
// touches on distinct banks while row r + 8 keeps row r's offsets.
constexpr int kWdBN = 64, kWdWaves = 8;
__device__ __forceinline__ int wd_swz(int r) { return 2 * ((r >> 1) & 3); }
template <int NW, int MB, int D>
__global__ __launch_bounds__(NW * 64) void qkv_gemm_wide_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ out, int M, int K, int N, ProjEpilogue app) {
  constexpr int kThreads = NW * 64;
  constexpr int kSlot = 32 * kWdBN;     // bf16 elements per slot
  constexpr int kLoads = 4 + MB;        // vector-memory instructions per step (4 W copies, MB x loads)
  constexpr int kAhead = (D - 1) * kLoads;
  static_assert(kAhead <= 63, "vmcnt range");
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrt = (M + 16 * MB - 1) / (16 * MB);
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = lid % nrt, cs = lid / nrt;  // the row tiles of one strip are neighbours: W reuse in L2
  const int n0 = cs * kWdBN, m0 = rt * 16 * MB;
  const int kw = K / NW;                     // k rows per wave
  const int nst = kw >> 5;                   // 32-row steps per wave
  const uint32_t kbeg = (uint32_t)(wq * kw);

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((int64_t)K * N * 2));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * K * 2));
  // W copy c of a step, lane l: slot row 8c + l/8, slot chunk l%8, holding
  // chunk (l%8) ^ swz of k row (slot row with bits 2,3 swapped)
  uint32_t w_lane[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int sr = 8 * c + (lane >> 3);
    const int kr = (sr & ~12) | ((sr & 4) << 1) | ((sr & 8) >> 1);
    w_lane[c] = (uint32_t)kr * N * 2 + (uint32_t)n0 * 2 + (uint32_t)(((lane & 7) ^ wd_swz(sr)) * 16);
  }
  // x block b: lane l holds row m0 + 16b + l%16, k group l/16; rows past M read zeros
  uint32_t x_lane[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int row = m0 + b * 16 + (lane & 15);
    x_lane[b] = row < M ? (uint32_t)row * K * 2 + (lane >> 4) * 16 : 0x80000000u;
  }
  uint16_t* ring = smem + wq * D * kSlot;
  u32x4_t xf[D][MB];
  auto issue = [&](int i, int slot) {
    const uint32_t k0 = kbeg + (uint32_t)i * 32;
    uint16_t* sp = ring + slot * kSlot;
#pragma unroll
    for (int c = 0; c < 4; ++c) dma16(wr, sp + c * 512, w_lane[c] + k0 * (uint32_t)N * 2, 0);
#pragma unroll
    for (int b = 0; b < MB; ++b) xf[slot][b] = bld16(xr, x_lane[b] + k0 * 2);
  };
  // B operand of column block cb: lane group g (k rows 8g..8g+7 of column l%16)
  // reads slot rows 16(g>>1) + 4(g&1) + j and, 8 rows on, the second half
  const int bg = lane >> 4, bp = lane & 15;
  const int br = 16 * (bg >> 1) + 4 * (bg & 1) + (bp >> 2);
  int b_off[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    b_off[cb] = br * kWdBN + (((2 * cb + ((bp & 3) >> 1)) ^ wd_swz(br)) * 8) + 4 * (bp & 1);

  f32x4_t acc[MB][4];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[b][cb] = f32x4_t{};

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
        u32x4_t bf[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) bf[cb] = lds_tr16_pair<8 * kWdBN * 2>(sp + b_off[cb]);
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[b][cb] = mfma16_bf16(xf[j][b], bf[cb], acc[b][cb]);
        if (i + D < nst) issue(i + D, j);
      }
    });
  }
  wait_vmcnt<0>();

  // the NW waves' sums, added in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  constexpr int kPer = MB * 4 * 4 * 64;  // floats per wave
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wq * kPer + ((b * 4 + cb) * 4 + e) * 64 + lane] = acc[b][cb][e];
  __syncthreads();
  static_assert(kPer % kThreads == 0, "outputs per thread");
#pragma unroll
  for (int q = 0; q < kPer / kThreads; ++q) {
    const int idx = q * kThreads + tid;  // (b, cb, e, lane), lane fastest
    const int ln = idx & 63, e = (idx >> 6) & 3, cb = (idx >> 8) & 3, b = idx >> 10;
    float v = red[idx];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) v += red[wv * kPer + idx];
    const int m = m0 + b * 16 + 4 * (ln >> 4) + e, n = n0 + cb * 16 + (ln & 15);
    v += bias ? bf16_to_f32(bias[n]) : 0.0f;
    if (app.inv_freq != nullptr && n0 + cb * 16 < app.vcol) {  // 16 columns, one side of vcol
      const float pw = pair_partner(v);                        // thread tid ^ 1 holds column n ^ 1, row m
      if (m < M) v = rope_turn(v, pw, n, rope_position(app, m), rope_freq(app, n));
    }
    if (m < M) {
      const uint16_t r = f32_to_bf16(v);
      out[(int64_t)m * N + n] = r;
      append_store(app, m, n, r);
    }
  }
}

template <int NW, int MB, int D>
static hipError_t launch_wide(const void* x, const void* w, const void* bias, void* out, int M, int K, int N,
                              hipStream_t s, const ProjEpilogue& app) {
  auto kern = qkv_gemm_wide_kernel<NW, MB, D>;
  const size_t lds = (size_t)NW * D * 32 * kWdBN * sizeof(uint16_t);
  static_assert((size_t)D * 32 * kWdBN * 2 >= (size_t)MB * 4 * 4 * 64 * 4, "reduction fits");
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int nblk = (N / kWdBN) * ((M + 16 * MB - 1) / (16 * MB));
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(NW * 64), lds, s, (const uint16_t*)x, (const uint16_t*)w,
                     (const uint16_t*)bias, (uint16_t*)out, M, K, N, app);
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
                                                              int ksplit, ProjEpilogue app) {
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
  if (bias) {
    s[0] += bf16_to_f32(bias[n]);
    s[1] += bf16_to_f32(bias[n + 1]);
    s[2] += bf16_to_f32(bias[n + 2]);
    s[3] += bf16_to_f32(bias[n + 3]);
  }
  if (app.inv_freq != nullptr && n < app.vcol) {  // two whole planes
    const int p = rope_position(app, (int)(i / N));
    const float t0 = rope_turn(s[0], s[1], n, p, rope_freq(app, n));
    const float t1 = rope_turn(s[1], s[0], n + 1, p, rope_freq(app, n + 1));
    const float t2 = rope_turn(s[2], s[3], n + 2, p, rope_freq(app, n + 2));
    const float t3 = rope_turn(s[3], s[2], n + 3, p, rope_freq(app, n + 3));
    s = f32x4_t{t0, t1, t2, t3};
  }
  u32x2_t pk;
  pk[0] = pack_bf16(s[0], s[1]);
  pk[1] = pack_bf16(s[2], s[3]);
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
                                   int M, int K, int N, hipStream_t s, const ProjEpilogue& app) {
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
  if (M > 128 || K * N * 2 >= ((int64_t)1 << 31) || M * K * 2 >= ((int64_t)1 << 31)) return p;
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
  // Wide workgroups (8 waves over all of K, no partials).  Measured against
  // the k-split skinny kernel + reduce: better at every M > 32 (TinyLlama
  // width, M = 128: 14.7 -> 8.4 us warm, 20.2 -> 16.6 us cold); 16-row tiles
  // while the grid stays within 256 workgroups (M = 64: 10.9 -> 6.3 us warm),
  // 32-row tiles otherwise (a tile re-reads the whole strip of W).  At M <= 32
  // only with at least 192 strips (N = 12288: 38.2 -> 32.5 us cold); narrower
  // weights stream better split over k.
  if (K % (kWdWaves * 32) == 0 && N % kWdBN == 0) {
    const int64_t strips = N / kWdBN;
    if (M > 32 || strips * ((M + 31) / 32) >= 192) {
      p.wide = true;
      p.wide_mb = (M > 32 && M <= 64 && strips * ((M + 15) / 16) <= 256) ? 1 : 2;
      p.krange = (int)K;
      p.ksplit = 1;
      p.ok = true;
      return p;
    }
  }
  // Register-transpose kernel (M <= 32): 8 waves per 64 columns, each wave
  // NS = 4, 2 or 1 steps of 32 rows.  A CU streams its workgroups' bytes at a
  // rate bounded by the loads it keeps in flight, so the choice minimises the
  // bytes of the busiest CU (workgroups spread over 256 CUs, rounded up, times
  // 64 columns x 256 NS rows), counting the fp32 partials written and read
  // back as bytes spread over all CUs.
  if (M <= 32 && K % 256 == 0 && N % kRtBN == 0) {
    const int64_t strips = N / kRtBN;
    int ns = 0;
    int64_t best = 0;
    for (int c = 4; c >= 1; c /= 2) {
      if (K % (256 * c) != 0) continue;
      const int64_t ksp = K / (256 * c);
      const int64_t cost = (strips * ksp + 255) / 256 * (256 * c * kRtBN * 2) + ksp * M * N * 8 / 256;
      if (ns == 0 || cost < best) ns = c, best = cost;
    }
    p.rt_ns = ns;
    p.krange = 256 * ns;
    p.ksplit = (int)(K / p.krange);
    if (p.ksplit * M * N * 4 >= ((int64_t)1 << 31)) return SkinnyPlan{};
    p.ws_bytes = (size_t)p.ksplit * M * N * 4;
    p.ok = true;
    return p;
  }
  if (N % kSkBN != 0) return SkinnyPlan{};
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
                           const ProjEpilogue& app) {
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
  if (p.ok && p.wide)
    return p.wide_mb == 1 ? launch_wide<kWdWaves, 1, 2>(x, w, bias, out, m, k, n, s, app)
                          : launch_wide<kWdWaves, 2, 2>(x, w, bias, out, m, k, n, s, app);
  if (p.ok && p.rt_ns > 0 && ws != nullptr && ws_bytes >= p.ws_bytes) {
    hipError_t e = M > 16 ? launch_rt<2>(p, x, w, ws, m, k, n, s) : launch_rt<1>(p, x, w, ws, m, k, n, s);
    if (e != hipSuccess) return e;
    const int64_t quads = (M * N + 3) / 4;
    hipLaunchKernelGGL(qkv_gemm_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s,
                       (const float*)ws, (const uint16_t*)bias, (uint16_t*)out, m, n, p.ksplit, app);
    return hipGetLastError();
  }
  if (p.ok && p.rt_ns == 0 && (p.ksplit == 1 || (ws != nullptr && ws_bytes >= p.ws_bytes))) {
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
  if (K % kTBK == 0 && N % 8 == 0 && (uint64_t)K * N * 2 < 0x80000000ull && (uint64_t)M * K * 2 < 0x80000000ull) {
    // Tile shape: the one-workgroup-per-CU configuration with the most tiles
    // that still fit one round on the CUs (ties: the larger tile, which reads
    // fewer operand bytes per FLOP); shapes with more tiles than that run the
    // 128 x 160 tile two workgroups per CU, or 128 x 128 tiles when their
    // rounds on the CUs take less time.
    int dev = 0, cus = 256;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const int64_t t160 = tiles(128, 160), t128 = tiles(128, 128), t64_160 = tiles(64, 160), t64 = tiles(64, 128);
    int64_t best = 0;
    int pick = -1;
    const int64_t cand[4] = {t160, t128, t64_160, t64};  // larger tiles first
    for (int c = 0; c < 4; ++c)
      if (cand[c] <= cus && cand[c] > best) best = cand[c], pick = c;
    switch (pick) {
      case 0: return launch_gemm_tiles<128, 160, 4, 1, 2, 3>(x, w, bias, out, m, k, n, s, app);
      case 1: return launch_gemm_tiles<128, 128, 2, 2, 2, 3>(x, w, bias, out, m, k, n, s, app);
      case 2: return launch_gemm_tiles<64, 160, 2, 1, 2, 4>(x, w, bias, out, m, k, n, s, app);
      case 3: return launch_gemm_tiles<64, 128, 2, 2, 2, 4>(x, w, bias, out, m, k, n, s, app);
      default: {  // more tiles than CUs
        // Rounds of 128 x 160 tiles two per CU against rounds of 128 x 128
        // tiles one per CU; one round of the latter measured 0.58 of one of the
        // former ([2048,4096] x [4096,6144]: 2 rounds 140 us against 3 rounds
        // 127 us; M = 4096: 3 rounds 227 us against 6 rounds 252 us).
        const int64_t r160 = (t160 + 2 * cus - 1) / (2 * cus), r128 = (t128 + cus - 1) / cus;
        if (58 * r128 < 100 * r160)
          return launch_gemm_tiles<128, 128, 2, 2, 2, 3>(x, w, bias, out, m, k, n, s, app);
        return launch_gemm_tiles<128, 160, 4, 1, 1, 2>(x, w, bias, out, m, k, n, s, app);
      }
    }
  }
  // Pick the largest tile that still gives the chip (256 CUs) a full wave of workgroups.
  const int64_t big = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t mid = ((M + 63) / 64) * ((N + 63) / 64);
  if (big >= 256) return launch_gemm_bf16<128, 128, 64, 2, 2, 1>(x, w, bias, out, m, k, n, s, app);
  if (M > 32 && mid >= 128) return launch_gemm_bf16<64, 64, 64, 2, 2, 1>(x, w, bias, out, m, k, n, s, app);
  return launch_gemm_bf16<32, 32, 256, 1, 1, 4>(x, w, bias, out, m, k, n, s, app);
}

}  // namespace mqkv
