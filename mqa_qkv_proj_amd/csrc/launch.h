// Host-side launchers of the gfx950 kernels (called by the C ABI after validation).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqkv {

hipError_t launch_qkv_gemm(const void* x, const void* w, const void* bias, void* out, int64_t M,
                           int64_t K, int64_t N, bool bf16, hipStream_t s);

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Lq, Lkv, Hq, Hkv, d;
  int64_t q_stride, kv_stride;
  bool causal;
  float scale;
  bool in_bf16, out_bf16;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  int B, Hq, Hkv, d, Lmax;
  int64_t q_stride;
  float scale;
  int split;       // keys per split
  int n_split;     // splits per sequence at capacity: ceil(Lmax / split)
  float* part_o;   // [B, Hq, n_split, d]
  float* part_ml;  // [B, Hq, n_split, 2]  (running max in log2 units, sum)
  bool in_bf16, out_bf16;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace mqkv
