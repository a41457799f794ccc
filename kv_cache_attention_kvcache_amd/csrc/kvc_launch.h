// Host-side launchers of the kvc kernels.  The C entry points validate their
// arguments and then call exactly one of these; every launcher returns the
// hipError_t of its last launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvc {

// One layer of a cache: element pointers already offset to that layer.
struct LayerView {
  void* k;
  void* v;
  const int32_t* seqlens;
  int32_t batch, max_seq, n_kv_heads, head_dim, dtype;
  float* k_scale;  // int8 caches: (batch, n_kv_heads, max_seq) scales of this layer; else null
  float* v_scale;
  int32_t rolling;  // rolling window: position p in slot p mod max_seq
  // Ragged calls: row b brings tokens [cu_tokens[b], cu_tokens[b+1]) of the packed
  // q / k_new / v_new / out; null for calls with the same T tokens in every row.
  const int32_t* cu_tokens;
  int32_t n_tokens, max_tokens;  // ragged calls: packed token rows; bound on any row's count
  int32_t row_filter;            // kRowsAll, or one half of a mixed call (see row_selected)
};

constexpr int kRowsAll = 0;       // every row of the batch
constexpr int kRowsDecode = 1;    // mixed call, decode launch: rows with exactly one token
constexpr int kRowsPrefill = 2;   // mixed call, prefill launch: rows with more than one token

// Row b's first packed token and token count in a call with T tokens per row
// (ragged calls: from cu_tokens).  count = -1: a malformed range (negative,
// decreasing, past n_tokens or longer than max_tokens) -- the row is skipped.
struct RowTokens {
  int first, count;
};
__device__ __forceinline__ RowTokens row_tokens(const LayerView& kv, int b, int T) {
  if (!kv.cu_tokens) return RowTokens{b * T, T};
  const int a = kv.cu_tokens[b], e = kv.cu_tokens[b + 1];
  if (a < 0 || e < a || e > kv.n_tokens || e - a > kv.max_tokens) return RowTokens{0, -1};
  return RowTokens{a, e - a};
}
// Whether a row with `count` new tokens belongs to this launch.
__device__ __forceinline__ bool row_selected(const LayerView& kv, int count) {
  if (count < 0) return false;
  return kv.row_filter == kRowsAll || (kv.row_filter == kRowsDecode ? count == 1 : count > 1);
}

// Keys query t (of T new tokens of row b, P = seqlens[b]) attends, or -1 if the
// row is out of range (skipped, KVC_DEV_CAPACITY).  Linear cache, or T > 1:
// P + t + 1 while P + T <= max_seq.  Rolling window, T = 1: the min(P + 1, max_seq)
// filled slots.
__device__ __forceinline__ int attended_keys(const LayerView& kv, int start, int T, int t) {
  if (start < 0) return -1;
  if (kv.rolling && T == 1) return start < kv.max_seq ? start + 1 : kv.max_seq;
  if (start > kv.max_seq - T) return -1;
  return start + t + 1;
}

// Slot of absolute position pos (written by the append of a call with T tokens).
__device__ __forceinline__ int slot_of(const LayerView& kv, int pos) {
  return kv.rolling ? pos % kv.max_seq : pos;
}

struct RopeAppendParams {
  LayerView kv;
  const void* q;
  void* q_out;
  const void* k_new;
  const void* v_new;
  int32_t T, n_q_heads;
  float inv_freq[64];  // float32 frequencies, head_dim / 2 of them
  int32_t* dev_err;
};
hipError_t launch_rope_append(const RopeAppendParams& p, hipStream_t s);
// Same call on an int8 cache: q/q_out/k_new/v_new bfloat16, K/V quantized per vector.
hipError_t launch_rope_append_q8(const RopeAppendParams& p, hipStream_t s);

// Split-KV attention over rows (b, t): row b's query t attends to keys 0..seqlens[b]+t.
// Decode is T = 1.  With one split per row ("direct") the output is written
// straight away; otherwise float32 partials go to the workspace and
// launch_split_combine folds them.
struct SplitParams {
  LayerView kv;
  const void* q;
  void* out;
  float* ws_o;   // (batch*T, n_q_heads, max_splits, head_dim)
  float* ws_ml;  // (batch*T, n_q_heads, max_splits, 2): running max (log2 units) and sum
  int32_t T, n_q_heads, split_keys, max_splits;
  float scale_log2;  // softmax scale * log2(e)
  int32_t direct;
  int32_t* dev_err;
};
hipError_t launch_split_attention(const SplitParams& p, hipStream_t s);
hipError_t launch_split_combine(const SplitParams& p, hipStream_t s);

// bfloat16 decode (T = 1): persistent split-KV over a balanced tile partition.
// A segment is (row, KV head, block of gb query heads); workgroup w of n_wg
// takes the flattened tiles [w N / n_wg, (w+1) N / n_wg).
struct DecodeParams {
  LayerView kv;
  const void* q;
  void* out;
  float* ws_o;   // (n_wg, 2, gb, head_dim): unnormalised partial outputs
  float* ws_ml;  // (n_wg, 2, gb, 2): running max (log2 units) and sum
  int32_t n_q_heads, n_wg, gb, n_hb;
  float scale_log2;
  int32_t* dev_err;
};
// Query heads per block: 4 or 8 on vector ALUs; an int8 cache whose group
// fits 32 heads takes the matrix-core kernel with one 32-head block per KV head.
int decode_bf16_block(int dtype, int group);
constexpr int kDecodeQ8Block = 32;  // the matrix-core int8 kernel's query-head block
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t s);

struct PrefillParams {
  LayerView kv;
  const void* q;
  void* out;
  int32_t T, n_q_heads;
  float scale_log2;
  int32_t* dev_err;
  int32_t n_cus;  // compute units of the device: a grid smaller than this takes 4-wave workgroups
};
hipError_t launch_prefill_mfma(const PrefillParams& p, hipStream_t s);

// Fused decode step (T = 1): RoPE + append + attention over the whole row in
// one launch, one workgroup per (row, KV head).
struct DecodeStepParams {
  LayerView kv;
  const void* q;      // (batch, 1, n_q_heads, head_dim), raw
  const void* k_new;  // (batch, 1, n_kv_heads, head_dim), raw
  const void* v_new;
  void* out;          // (batch, 1, n_q_heads, head_dim)
  int32_t n_q_heads;
  float scale_log2;
  float inv_freq[64];
  int32_t* dev_err;
};
constexpr int kDecodeStepMaxGroup = 16;  // query heads per KV head
hipError_t launch_decode_step(const DecodeStepParams& p, hipStream_t s);

struct CloneParams {
  LayerView src;  // layer 0 view; n_layers below
  LayerView dst;
  int32_t* dst_seqlens;
  int32_t n_layers, src_len;
  int32_t* dev_err;
};
hipError_t launch_clone(const CloneParams& p, hipStream_t s);

}  // namespace kvc
