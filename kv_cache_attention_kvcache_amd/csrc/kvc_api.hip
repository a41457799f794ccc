// The C entry points of libkvc: validate on the host, then launch on the
// caller's stream.  Nothing here allocates or synchronises.  The state kept
// across calls is per device: the CU count, and the address of the static
// decode scratch once kvc_attn_decode_noalloc has looked it up.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "kvc.h"
#include "kvc_launch.h"

// Scratch of kvc_attn_decode_noalloc: a fixed array in device memory that every
// call on a device shares (each device holds its own copy for the life of the
// process).  In host code the array's name is not a device address; its address
// on the current device is looked up once per device with hipGetSymbolAddress
// (device_scratch below) and only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[KVC_DECODE_SCRATCH_MAX_BYTES];

namespace {

constexpr int32_t kDefaultSplitKeys = 512;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cache(const kvc_cache* c) {
  if (!c || !c->k || !c->v || !c->seqlens) return KVC_E_ARG;
  if (!aligned16(c->k) || !aligned16(c->v) || (reinterpret_cast<uintptr_t>(c->seqlens) & 3u)) return KVC_E_ARG;
  if (c->dtype != KVC_F32 && c->dtype != KVC_BF16 && c->dtype != KVC_I8) return KVC_E_DTYPE;
  if (c->dtype == KVC_I8 && (!c->k_scale || !c->v_scale || (reinterpret_cast<uintptr_t>(c->k_scale) & 3u) ||
                             (reinterpret_cast<uintptr_t>(c->v_scale) & 3u)))
    return KVC_E_ARG;
  if (c->n_layers < 1 || c->batch < 1 || c->max_seq < 1 || c->n_kv_heads < 1) return KVC_E_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return KVC_E_SHAPE;
  if (c->rolling != 0 && c->rolling != 1) return KVC_E_ARG;
  return KVC_OK;
}

int check_heads(const kvc_cache* c, int32_t n_q_heads) {
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0) return KVC_E_SHAPE;
  return KVC_OK;
}

size_t elem_bytes(int32_t dtype) { return dtype == KVC_F32 ? 4 : dtype == KVC_BF16 ? 2 : 1; }

kvc::LayerView layer_view(const kvc_cache* c, int32_t layer) {
  const size_t esz = elem_bytes(c->dtype);
  const size_t layer_vecs = size_t(c->batch) * c->max_seq * c->n_kv_heads;
  const size_t layer_bytes = layer_vecs * c->head_dim * esz;
  kvc::LayerView v;
  v.k = static_cast<uint8_t*>(c->k) + size_t(layer) * layer_bytes;
  v.v = static_cast<uint8_t*>(c->v) + size_t(layer) * layer_bytes;
  v.seqlens = c->seqlens;
  v.batch = c->batch;
  v.max_seq = c->max_seq;
  v.n_kv_heads = c->n_kv_heads;
  v.head_dim = c->head_dim;
  v.dtype = c->dtype;
  v.rolling = c->rolling;
  v.k_scale = c->dtype == KVC_I8 ? c->k_scale + size_t(layer) * layer_vecs : nullptr;
  v.v_scale = c->dtype == KVC_I8 ? c->v_scale + size_t(layer) * layer_vecs : nullptr;
  v.cu_tokens = nullptr;  // the same T tokens in every row, unless a ragged call sets it
  v.n_tokens = 0;
  v.max_tokens = 0;
  v.row_filter = kvc::kRowsAll;
  return v;
}

// A ragged call's rows: row b brings tokens [cu_tokens[b], cu_tokens[b+1]) of the packed tensors.
void set_ragged(kvc::LayerView& v, const int32_t* cu_tokens, int32_t n_tokens, int32_t max_tokens, int filter) {
  v.cu_tokens = cu_tokens;
  v.n_tokens = n_tokens;
  v.max_tokens = max_tokens;
  v.row_filter = filter;
}

int check_ragged(const kvc_cache* c, const int32_t* cu_tokens, int32_t n_tokens, int32_t max_tokens) {
  if (!cu_tokens || (reinterpret_cast<uintptr_t>(cu_tokens) & 3u)) return KVC_E_ARG;
  if (n_tokens < 0 || max_tokens < 1) return KVC_E_ARG;
  if (int64_t(c->batch) * max_tokens > 0x7fffffffLL) return KVC_E_ARG;
  return KVC_OK;
}

bool resolve_scale(float scale, int32_t head_dim, float* out) {
  if (isnan(scale) || isinf(scale)) return false;
  *out = scale > 0.f ? scale : float(1.0 / sqrt(double(head_dim)));
  return true;
}

// Workgroups the bfloat16 decode spreads its tiles over: one per CU.  (On
// MI355X a second resident workgroup per CU adds memory-level parallelism past
// what HBM3E serves well: 256 workgroups stream the 72K-token cache about 15%
// faster than 512.)  The CU count is a read-only device property, cached per
// device on first use.
int32_t default_decode_workers() {
  constexpr int kMaxDev = 64;
  static std::atomic<int32_t> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDev) {
    const int32_t v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (dev < kMaxDev) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

struct DecodePlan {
  int32_t gb, n_hb, n_wg;
};

DecodePlan decode_plan(const kvc_cache* c, int32_t n_q_heads, int32_t n_workers) {
  DecodePlan pl;
  const int32_t group = n_q_heads / c->n_kv_heads;
  pl.gb = kvc::decode_bf16_block(c->dtype, group);
  pl.n_hb = (group + pl.gb - 1) / pl.gb;
  pl.n_wg = n_workers > 0 ? n_workers : default_decode_workers();
  return pl;
}

size_t decode_ws_bytes(const kvc_cache* c, int32_t n_q_heads, int32_t n_workers) {
  if (c->dtype != KVC_F32) {  // bfloat16 and int8 caches share the split-KV plan
    const DecodePlan pl = decode_plan(c, n_q_heads, n_workers);
    if (pl.n_wg <= 0) return 0;
    return size_t(pl.n_wg) * 2 * size_t(pl.gb) * size_t(c->head_dim + 2) * sizeof(float);
  }
  const int64_t max_splits = (int64_t(c->max_seq) + kDefaultSplitKeys - 1) / kDefaultSplitKeys;
  if (max_splits <= 1) return 0;  // every row fits one split: written directly
  return size_t(c->batch) * size_t(n_q_heads) * size_t(max_splits) * size_t(c->head_dim + 2) * sizeof(float);
}

// The scratch array's address on the current device (null if it cannot be had).
// Looked up on a device's first kvc_attn_decode_noalloc call, with that device
// current, then kept.
void* device_scratch() {
  constexpr int kMaxDev = 64;
  static std::atomic<void*> addr[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  addr[dev].store(p, std::memory_order_release);
  return p;
}

int launch_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_E_LAUNCH; }

// Validation and launch shared by the uniform and the ragged append (T: tokens per
// row, or the bound on them).
int rope_append_impl(const kvc_cache* cache, int32_t layer, const void* q, void* q_out, const void* k_new,
                     const void* v_new, int32_t T, int32_t n_q_heads, float rope_base, const int32_t* cu_tokens,
                     int32_t n_tokens, int32_t* dev_err, void* stream) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (layer < 0 || layer >= cache->n_layers || T < 1) return KVC_E_ARG;
  if (!q || !q_out || !k_new || !v_new) return KVC_E_ARG;
  if (!aligned16(q) || !aligned16(q_out) || !aligned16(k_new) || !aligned16(v_new)) return KVC_E_ARG;
  if (!(rope_base > 1.f) || isinf(rope_base)) return KVC_E_ARG;
  if ((st = check_heads(cache, n_q_heads)) != KVC_OK) return st;
  if (int64_t(cache->batch) * T > 0x7fffffffLL) return KVC_E_ARG;
  if (cache->rolling && T > cache->max_seq) return KVC_E_ARG;  // one call must not overwrite its own tokens
  kvc::RopeAppendParams p;
  p.kv = layer_view(cache, layer);
  if (cu_tokens) set_ragged(p.kv, cu_tokens, n_tokens, T, kvc::kRowsAll);
  p.q = q;
  p.q_out = q_out;
  p.k_new = k_new;
  p.v_new = v_new;
  p.T = T;
  p.n_q_heads = n_q_heads;
  // inv_freq[i] = base^(-2i/D): evaluated in double, rounded once to float.
  for (int i = 0; i < 64; ++i)
    p.inv_freq[i] = i < cache->head_dim / 2 ? float(pow(double(rope_base), -2.0 * i / cache->head_dim)) : 0.f;
  p.dev_err = dev_err;
  if (cache->dtype == KVC_I8) return launch_status(kvc::launch_rope_append_q8(p, static_cast<hipStream_t>(stream)));
  return launch_status(kvc::launch_rope_append(p, static_cast<hipStream_t>(stream)));
}

// The split-KV decode of bfloat16 and int8 caches over the rows a layer view selects.
int decode_bf16_impl(const kvc_cache* cache, const kvc::LayerView& lv, const void* q_rot, void* out,
                     int32_t n_q_heads, float sc, int32_t n_workers, void* workspace, int32_t* dev_err,
                     hipStream_t s) {
  const DecodePlan pl = decode_plan(cache, n_q_heads, n_workers);
  if (pl.n_wg <= 0) return KVC_E_LAUNCH;
  // Flattened tile indices and in-row byte offsets are 32-bit.
  const int64_t tiles = int64_t(cache->batch) * cache->n_kv_heads * pl.n_hb * ((int64_t(cache->max_seq) + 31) / 32);
  const int64_t row_span = int64_t(cache->max_seq) * cache->n_kv_heads * cache->head_dim * 2;  // bfloat16 bound
  if (tiles >= (int64_t(1) << 31) || row_span >= (int64_t(1) << 31)) return KVC_E_SHAPE;
  if (int64_t(cache->batch) * cache->n_kv_heads * pl.n_hb * pl.gb > 0x7fffffffLL) return KVC_E_SHAPE;
  kvc::DecodeParams p;
  p.kv = lv;
  p.q = q_rot;
  p.out = out;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + size_t(pl.n_wg) * 2 * pl.gb * cache->head_dim;
  p.n_q_heads = n_q_heads;
  p.n_wg = pl.n_wg;
  p.gb = pl.gb;
  p.n_hb = pl.n_hb;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.dev_err = dev_err;
  return launch_status(kvc::launch_decode_bf16(p, s));
}

// The bfloat16 prefill kernel over the rows a layer view selects (T: tokens per row, or their bound).
int prefill_bf16_impl(const kvc_cache* cache, const kvc::LayerView& lv, const void* q_rot, void* out, int32_t T,
                      int32_t n_q_heads, float sc, int32_t* dev_err, hipStream_t s) {
  // The kernel's buffer descriptors span one head row with 32-bit byte offsets.
  if (int64_t(cache->max_seq) * cache->n_kv_heads * cache->head_dim * 2 >= (int64_t(1) << 31)) return KVC_E_SHAPE;
  kvc::PrefillParams p;
  p.kv = lv;
  p.q = q_rot;
  p.out = out;
  p.T = T;
  p.n_q_heads = n_q_heads;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.dev_err = dev_err;
  p.n_cus = default_decode_workers();  // the CU count (0 if unknown: 8-wave workgroups)
  return launch_status(kvc::launch_prefill_mfma(p, s));
}

// Float32: one split spanning the whole cache per query row, written directly.
int prefill_f32_impl(const kvc_cache* cache, const kvc::LayerView& lv, const void* q_rot, void* out, int32_t T,
                     int32_t n_q_heads, float sc, int32_t* dev_err, hipStream_t s) {
  kvc::SplitParams p;
  p.kv = lv;
  p.q = q_rot;
  p.out = out;
  p.T = T;
  p.n_q_heads = n_q_heads;
  p.split_keys = int32_t((int64_t(cache->max_seq) + 63) / 64 * 64);
  p.max_splits = 1;
  p.direct = 1;
  p.ws_o = nullptr;
  p.ws_ml = nullptr;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.dev_err = dev_err;
  return launch_status(kvc::launch_split_attention(p, s));
}

int decode_impl(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out, int32_t n_q_heads, float scale,
                int32_t n_workers, void* workspace, size_t workspace_bytes, bool static_scratch, int32_t* dev_err,
                void* stream) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (layer < 0 || layer >= cache->n_layers) return KVC_E_ARG;
  if (!q_rot || !out || !aligned16(q_rot) || !aligned16(out)) return KVC_E_ARG;
  if ((st = check_heads(cache, n_q_heads)) != KVC_OK) return st;
  if (n_workers < 0) return KVC_E_ARG;
  float sc;
  if (!resolve_scale(scale, cache->head_dim, &sc)) return KVC_E_ARG;
  const size_t need = decode_ws_bytes(cache, n_q_heads, n_workers);
  if (static_scratch) {
    if (need > KVC_DECODE_SCRATCH_MAX_BYTES) return KVC_E_SCRATCH;
    if (need > 0) {
      workspace = device_scratch();
      workspace_bytes = KVC_DECODE_SCRATCH_MAX_BYTES;
      if (!workspace) return KVC_E_LAUNCH;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return KVC_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cache->dtype != KVC_F32)  // bfloat16 or int8 cache
    return decode_bf16_impl(cache, layer_view(cache, layer), q_rot, out, n_q_heads, sc, n_workers, workspace,
                            dev_err, s);
  // float32: split-KV over fixed 512-key splits.
  kvc::SplitParams p;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.kv = layer_view(cache, layer);
  p.q = q_rot;
  p.out = out;
  p.T = 1;
  p.n_q_heads = n_q_heads;
  p.split_keys = kDefaultSplitKeys;
  p.max_splits = int32_t((int64_t(cache->max_seq) + kDefaultSplitKeys - 1) / kDefaultSplitKeys);
  p.direct = need == 0;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.direct ? nullptr
                     : p.ws_o + size_t(cache->batch) * n_q_heads * size_t(p.max_splits) * cache->head_dim;
  p.dev_err = dev_err;
  hipError_t e = kvc::launch_split_attention(p, s);
  if (e == hipSuccess && !p.direct) e = kvc::launch_split_combine(p, s);
  return launch_status(e);
}

}  // namespace

extern "C" {

int kvc_rope_append(const kvc_cache* cache, int32_t layer, const void* q, void* q_out, const void* k_new,
                    const void* v_new, int32_t T, int32_t n_q_heads, float rope_base, int32_t* dev_err,
                    void* stream) {
  return rope_append_impl(cache, layer, q, q_out, k_new, v_new, T, n_q_heads, rope_base, nullptr, 0, dev_err,
                          stream);
}

int kvc_rope_append_ragged(const kvc_cache* cache, int32_t layer, const void* q, void* q_out, const void* k_new,
                           const void* v_new, const int32_t* cu_tokens, int32_t n_tokens, int32_t max_tokens,
                           int32_t n_q_heads, float rope_base, int32_t* dev_err, void* stream) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if ((st = check_ragged(cache, cu_tokens, n_tokens, max_tokens)) != KVC_OK) return st;
  if (layer < 0 || layer >= cache->n_layers) return KVC_E_ARG;
  if (n_tokens == 0) return KVC_OK;  // no row brings a token: nothing to read or write
  return rope_append_impl(cache, layer, q, q_out, k_new, v_new, max_tokens, n_q_heads, rope_base, cu_tokens,
                          n_tokens, dev_err, stream);
}

size_t kvc_decode_workspace_bytes(const kvc_cache* cache, int32_t n_q_heads, int32_t n_workers) {
  if (check_cache(cache) != KVC_OK || check_heads(cache, n_q_heads) != KVC_OK) return 0;
  if (n_workers < 0) return 0;
  return decode_ws_bytes(cache, n_q_heads, n_workers);
}

int kvc_attn_decode(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out, int32_t n_q_heads,
                    float scale, int32_t n_workers, void* workspace, size_t workspace_bytes, int32_t* dev_err,
                    void* stream) {
  return decode_impl(cache, layer, q_rot, out, n_q_heads, scale, n_workers, workspace, workspace_bytes, false,
                     dev_err, stream);
}

int kvc_attn_decode_noalloc(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out,
                            int32_t n_q_heads, float scale, int32_t n_workers, int32_t* dev_err, void* stream) {
  return decode_impl(cache, layer, q_rot, out, n_q_heads, scale, n_workers, nullptr, 0, true, dev_err, stream);
}

int kvc_attn_prefill(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out, int32_t T,
                     int32_t n_q_heads, float scale, int32_t* dev_err, void* stream) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (layer < 0 || layer >= cache->n_layers || T < 1) return KVC_E_ARG;
  if (!q_rot || !out || !aligned16(q_rot) || !aligned16(out)) return KVC_E_ARG;
  if ((st = check_heads(cache, n_q_heads)) != KVC_OK) return st;
  float sc;
  if (!resolve_scale(scale, cache->head_dim, &sc)) return KVC_E_ARG;
  if (cache->dtype == KVC_I8) return KVC_E_DTYPE;  // prefill reads bfloat16 or float32 caches
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvc::LayerView lv = layer_view(cache, layer);
  lv.rolling = 0;  // prefill keeps the linear rule P + T <= max_seq, rolling window or not
  if (cache->dtype == KVC_BF16) return prefill_bf16_impl(cache, lv, q_rot, out, T, n_q_heads, sc, dev_err, s);
  return prefill_f32_impl(cache, lv, q_rot, out, T, n_q_heads, sc, dev_err, s);
}

int kvc_attn_mixed(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out, const int32_t* cu_tokens,
                   int32_t n_tokens, int32_t max_tokens, int32_t n_q_heads, float scale, int32_t n_workers,
                   void* workspace, size_t workspace_bytes, int32_t* dev_err, void* stream) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (layer < 0 || layer >= cache->n_layers) return KVC_E_ARG;
  if ((st = check_ragged(cache, cu_tokens, n_tokens, max_tokens)) != KVC_OK) return st;
  if (n_tokens == 0) return KVC_OK;  // no row brings a token: nothing to attend
  if (!q_rot || !out || !aligned16(q_rot) || !aligned16(out)) return KVC_E_ARG;
  if ((st = check_heads(cache, n_q_heads)) != KVC_OK) return st;
  if (n_workers < 0) return KVC_E_ARG;
  float sc;
  if (!resolve_scale(scale, cache->head_dim, &sc)) return KVC_E_ARG;
  if (cache->dtype == KVC_I8) return KVC_E_DTYPE;  // its prefill rows need a bfloat16 or float32 cache
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cache->dtype == KVC_F32) {
    // One launch: a direct split per query row handles decode and prefill rows alike.
    kvc::LayerView lv = layer_view(cache, layer);
    set_ragged(lv, cu_tokens, n_tokens, max_tokens, kvc::kRowsAll);
    return prefill_f32_impl(cache, lv, q_rot, out, max_tokens, n_q_heads, sc, dev_err, s);
  }
  const size_t need = decode_ws_bytes(cache, n_q_heads, n_workers);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return KVC_E_WORKSPACE;
  if (max_tokens > 1) {  // rows with a chunk: the matrix-core prefill, linear rule as in kvc_attn_prefill
    kvc::LayerView lv = layer_view(cache, layer);
    lv.rolling = 0;
    set_ragged(lv, cu_tokens, n_tokens, max_tokens, kvc::kRowsPrefill);
    if ((st = prefill_bf16_impl(cache, lv, q_rot, out, max_tokens, n_q_heads, sc, dev_err, s)) != KVC_OK) return st;
  }
  // rows with one token: the split-KV decode over those rows only
  kvc::LayerView lv = layer_view(cache, layer);
  set_ragged(lv, cu_tokens, n_tokens, max_tokens, kvc::kRowsDecode);
  return decode_bf16_impl(cache, lv, q_rot, out, n_q_heads, sc, n_workers, workspace, dev_err, s);
}

int kvc_decode_step(const kvc_cache* cache, int32_t layer, const void* q, const void* k_new, const void* v_new,
                    void* out, int32_t n_q_heads, float scale, float rope_base, int32_t* dev_err, void* stream) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (cache->dtype == KVC_I8) return KVC_E_DTYPE;  // the fused step keeps float32 / bfloat16 caches
  if (layer < 0 || layer >= cache->n_layers) return KVC_E_ARG;
  if (!q || !k_new || !v_new || !out) return KVC_E_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return KVC_E_ARG;
  if (!(rope_base > 1.f) || isinf(rope_base)) return KVC_E_ARG;
  if ((st = check_heads(cache, n_q_heads)) != KVC_OK) return st;
  if (n_q_heads / cache->n_kv_heads > kvc::kDecodeStepMaxGroup) return KVC_E_SHAPE;
  if (int64_t(cache->batch) * cache->n_kv_heads > 0x7fffffffLL) return KVC_E_SHAPE;
  float sc;
  if (!resolve_scale(scale, cache->head_dim, &sc)) return KVC_E_ARG;
  kvc::DecodeStepParams p;
  p.kv = layer_view(cache, layer);
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.out = out;
  p.n_q_heads = n_q_heads;
  p.scale_log2 = sc * 1.4426950408889634f;
  for (int i = 0; i < 64; ++i)
    p.inv_freq[i] = i < cache->head_dim / 2 ? float(pow(double(rope_base), -2.0 * i / cache->head_dim)) : 0.f;
  p.dev_err = dev_err;
  return launch_status(kvc::launch_decode_step(p, static_cast<hipStream_t>(stream)));
}

int kvc_prefill_clone(const kvc_cache* src, int32_t src_len, const kvc_cache* dst, int32_t* dev_err,
                      void* stream) {
  int st = check_cache(src);
  if (st != KVC_OK) return st;
  if ((st = check_cache(dst)) != KVC_OK) return st;
  if (src->dtype != dst->dtype) return KVC_E_DTYPE;
  if (src->batch != 1) return KVC_E_SHAPE;
  if (src->n_layers != dst->n_layers || src->n_kv_heads != dst->n_kv_heads || src->head_dim != dst->head_dim)
    return KVC_E_SHAPE;
  if (dst->max_seq < src->max_seq) return KVC_E_CAPACITY;
  if (src_len < 0 || src_len > src->max_seq) return KVC_E_CAPACITY;
  if (src->n_layers > 65535) return KVC_E_SHAPE;
  kvc::CloneParams p;
  p.src = layer_view(src, 0);
  p.dst = layer_view(dst, 0);
  p.dst_seqlens = dst->seqlens;
  p.n_layers = src->n_layers;
  p.src_len = src_len;
  p.dev_err = dev_err;
  return launch_status(kvc::launch_clone(p, static_cast<hipStream_t>(stream)));
}

const char* kvc_status_string(int status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_E_ARG: return "invalid argument (null or misaligned pointer, T < 1, layer out of range, bad scale/base/split)";
    case KVC_E_SHAPE: return "unsupported or mismatched shape (head_dim not 64/128, n_q_heads % n_kv_heads, descriptor mismatch)";
    case KVC_E_CAPACITY: return "capacity (clone destination max_seq smaller than source, or src_len out of range)";
    case KVC_E_DTYPE: return "unsupported or mismatched element type";
    case KVC_E_WORKSPACE: return "decode workspace missing, misaligned or too small";
    case KVC_E_LAUNCH: return "HIP kernel launch failed";
    case KVC_E_SCRATCH: return "the call needs more scratch than the library's static decode buffer holds";
    default: return "unknown status";
  }
}

}  // extern "C"
