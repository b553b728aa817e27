// Host-side launchers of the gfx950 kernels (called by the C ABI after validation).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqkv {

// Skinny-M (<= 128 rows) projection plan: k range split over workgroups.
struct SkinnyPlan {
  bool ok;        // the skinny path applies
  bool stream16;  // 16-column streaming kernel (M <= 32, K % 128 == 0), no k split
  bool wide;      // 8-wave workgroups over all of K (K % 256 == 0, N % 64 == 0), no k split
  int wide_mb;    // 16-row blocks per wide tile (1 or 2)
  int rt_ns;      // > 0: register-transpose kernel, 32-row k steps per wave (ksplit k ranges)
  int nbm;        // 32-row blocks
  int ksplit;     // k ranges
  int krange;     // rows of W per k range (a multiple of 128)
  size_t ws_bytes;  // fp32 partials needed when ksplit > 1
};
SkinnyPlan plan_skinny(int64_t M, int64_t K, int64_t N);

// Optional projection epilogue work, applied to each output element in fp32
// before its rounding:
//  * rotary embedding (inv_freq != nullptr): the columns n < vcol (Q and K
//    heads) are turned in planes (2i, 2i+1) of each head by the angle
//    fp32(position(m) * inv_freq[i]), i = (n mod d) / 2, the bias added first;
//    position(m) = pos[m], or with pos == nullptr seq_lens[m] - 1 clamped to
//    [0, L_max - 1] (the decode row's own cache slot);
//  * KV-cache append (k_cache != nullptr): the K and V columns of row m are
//    also written to the caches [rows, L_max, H_kv, d] at token position
//    seq_lens[m] - 1 (row m is sequence m's new token).
struct ProjEpilogue {
  void* k_cache;
  void* v_cache;
  const int32_t* seq_lens;
  int kcol;   // first K column (H_q * d)
  int vcol;   // first V column ((H_q + H_kv) * d); H_kv * d = vcol - kcol
  int L_max;
  const float* inv_freq;  // [d / 2]
  const int32_t* pos;     // [M] or nullptr
  int rope_d;             // head dimension d (64 or 128)
};

hipError_t launch_qkv_gemm(const void* x, const void* w, const void* bias, void* out, int64_t M,
                           int64_t K, int64_t N, bool bf16, void* ws, size_t ws_bytes, hipStream_t s,
                           const ProjEpilogue& app);

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
  void* ws;         // bf16 inputs: V^T tile images (prefill_workspace_bytes)
  size_t ws_bytes;
  // Packed variable-length batch (bf16 only): sequence b owns tokens
  // [cu_q[b], cu_q[b+1]) of q / o and [cu_kv[b], cu_kv[b+1]) of k / v; Lq and
  // Lkv are then the maximum lengths.  nullptr: fixed lengths, b-major.
  const int32_t* cu_q = nullptr;
  const int32_t* cu_kv = nullptr;
  int total_q = 0, total_kv = 0;
  // FP8 scores (bf16 inputs, d = 128): Q and K quantised to e4m3 after the
  // incoherent map with these signs (nullptr: no map); workspace per
  // prefill_fp8_workspace_bytes.
  bool fp8 = false;
  const float* signs = nullptr;
};
size_t prefill_fp8_workspace_bytes(int B, int Lq, int Lkv, int Hq, int Hkv, int d);
size_t prefill_workspace_bytes(int B, int Lkv, int Hkv, int d, bool bf16);
// V images plus the row-block schedule of a packed batch (persistent
// workers); 0 when no schedule is planned for the shape (B > 1024).
size_t prefill_varlen_workspace_bytes(int B, int Lkv_max, int total_q, int Hq, int Hkv, int d);
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
  int split;       // keys per aligned split; 0 = balanced work split (bf16 only)
  int n_slot;      // partial slots per (sequence, query head): decode_slots(Lmax, kv_split)
  float* part_o;   // [B, Hq, n_slot, d]
  float* part_ml;  // [B, Hq, n_slot, 4]  (running max in log2 units, sum, V exponent as int32, unused)
  bool in_bf16, out_bf16;
  // Paged caches (bf16 only): k/v are [num_pages, page_size, Hkv, d] pages and key j
  // of sequence b lives in page block_table[b * pages_per_seq + j / page_size]
  // (Lmax = pages_per_seq * page_size).  nullptr: contiguous [B, Lmax, Hkv, d].
  const int32_t* block_table = nullptr;
  int page_size = 0, pages_per_seq = 0, num_pages = 0;
  // The caller left the split to the library (kv_split = 0): on short caches
  // the fused kernel then runs instead of the split kernel and the combine.
  bool auto_split = false;
};
// The library's choice for kv_split == 0 (0 = balanced work split, else keys
// per split), and the partial slots per (sequence, query head) a call needs.
// The workspace query has no dtype, so it sizes for the larger of the two.
int decode_auto_split(int B, int Hq, int Hkv, int Lmax, bool bf16);
int decode_slots(int B, int Hq, int Hkv, int Lmax, int kv_split, bool bf16);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace mqkv
