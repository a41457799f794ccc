// Fused RoPE + in-place K/V append (one token row per workgroup).
//
// Tiny-GPT post, "Two Gotchas That Break It Quietly" (Gotcha 1): new tokens
// are rotated at positions offset by the row's start, with a float32 angle
// table.  nanochat post, "What the KV cache looks like on disk": the new K/V
// slices are written in place at each row's cache_seqlens offset.
//
// Element-wise and HBM-bound: per token it reads (Hq + 2 Hkv) head vectors
// and writes the same amount.  A workgroup takes one (row, token): it
// evaluates cos/sin of the token's head_dim/2 angles once into LDS, then
// rotates every q head and k head with 4-pair vectors and copies v with
// 16-byte vectors.  The grid is batch x T; in a ragged call T is the bound on
// any row's tokens, and a workgroup past its row's count returns at once.
#include "kvc_device.h"
#include "kvc_launch.h"
#include "kvc.h"

namespace kvc {

template <typename T>
struct Vec4;  // four consecutive elements <-> float

template <>
struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

template <>
struct Vec4<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* x) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* x) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendParams p) {
  constexpr int HALF = D / 2;
  constexpr int QUADS = HALF / 4;  // 4-pair groups per head vector
  __shared__ __align__(16) float cs[HALF];
  __shared__ __align__(16) float sn[HALF];

  // Grid: batch x T (ragged calls: T = max_tokens).  Workgroup (b, t) takes row b's
  // token t, which is packed row `row` of q / q_out / k_new / v_new.
  const int b = blockIdx.x / p.T;
  const int t = blockIdx.x - b * p.T;
  const RowTokens rt = row_tokens(p.kv, b, p.T);
  if (rt.count < 0) {
    if (t == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_TOKENS);
    return;
  }
  if (t >= rt.count) return;
  const int row = rt.first + t;
  const int start = p.kv.seqlens[b];
  if (start < 0 || (!p.kv.rolling && start > p.kv.max_seq - rt.count)) {
    if (t == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_CAPACITY);
    return;
  }
  const int pos = start + t;  // absolute position: the rotation angle
  if (threadIdx.x < HALF) {
    // One float32 product, as the angle table is built; full-range sincos.
    const float theta = __fmul_rn(static_cast<float>(pos), p.inv_freq[threadIdx.x]);
    float s, c;
    sincosf(theta, &s, &c);
    cs[threadIdx.x] = c;
    sn[threadIdx.x] = s;
  }
  __syncthreads();

  const int hq = p.n_q_heads;
  const int hkv = p.kv.n_kv_heads;
  const T* q_row = static_cast<const T*>(p.q) + size_t(row) * hq * D;
  T* q_out_row = static_cast<T*>(p.q_out) + size_t(row) * hq * D;
  const T* k_row = static_cast<const T*>(p.k_new) + size_t(row) * hkv * D;
  const size_t slot = (size_t(b) * p.kv.max_seq + slot_of(p.kv, pos)) * hkv * D;
  T* k_slot = static_cast<T*>(p.kv.k) + slot;

  const int n_items = (hq + hkv) * QUADS;
  for (int it = threadIdx.x; it < n_items; it += blockDim.x) {
    const int head = it / QUADS;
    const int i0 = (it - head * QUADS) * 4;
    const T* src = head < hq ? q_row + head * D : k_row + (head - hq) * D;
    T* dst = head < hq ? q_out_row + head * D : k_slot + (head - hq) * D;
    float a[4], b2[4], ra[4], rb[4];
    Vec4<T>::load(src + i0, a);
    Vec4<T>::load(src + i0 + HALF, b2);
    const float4 c4 = *reinterpret_cast<const float4*>(&cs[i0]);
    const float4 s4 = *reinterpret_cast<const float4*>(&sn[i0]);
    const float c[4] = {c4.x, c4.y, c4.z, c4.w};
    const float s[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) rope_pair(a[j], b2[j], c[j], s[j], ra[j], rb[j]);
    Vec4<T>::store(dst + i0, ra);
    Vec4<T>::store(dst + i0 + HALF, rb);
  }

  // v: a bit copy into the slot.
  const uint4* v_src = reinterpret_cast<const uint4*>(static_cast<const T*>(p.v_new) + size_t(row) * hkv * D);
  uint4* v_dst = reinterpret_cast<uint4*>(static_cast<T*>(p.kv.v) + slot);
  const int n_vec = hkv * D * int(sizeof(T)) / 16;
  for (int it = threadIdx.x; it < n_vec; it += blockDim.x) v_dst[it] = v_src[it];
}

// int8 cache (Cake paper, Section 5.1 "Compression methods", Section 5.5):
// the queries are rotated into q_out (bfloat16) exactly as above; each new
// key -- rotated with the same pair rotation and rounded to bfloat16, the
// value a bfloat16 cache would hold -- and each value vector is quantized per
// (token, KV head): s = amax / 127 in float32, codes round_half_even(x / s)
// in [-127, 127] (float32 quotient), s = 0 and codes 0 for an all-zero
// vector.  One wave per vector: a lane holds head_dim / 64 of its elements.
template <int D>
__global__ __launch_bounds__(256) void rope_append_q8_kernel(RopeAppendParams p) {
  constexpr int HALF = D / 2;
  constexpr int QUADS = HALF / 4;
  constexpr int EPL = D / kWave;  // elements per lane
  __shared__ __align__(16) float cs[HALF];
  __shared__ __align__(16) float sn[HALF];

  // Grid: batch x T (ragged calls: T = max_tokens).  Workgroup (b, t) takes row b's
  // token t, which is packed row `row` of q / q_out / k_new / v_new.
  const int b = blockIdx.x / p.T;
  const int t = blockIdx.x - b * p.T;
  const RowTokens rt = row_tokens(p.kv, b, p.T);
  if (rt.count < 0) {
    if (t == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_TOKENS);
    return;
  }
  if (t >= rt.count) return;
  const int row = rt.first + t;
  const int start = p.kv.seqlens[b];
  if (start < 0 || (!p.kv.rolling && start > p.kv.max_seq - rt.count)) {
    if (t == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_CAPACITY);
    return;
  }
  const int pos = start + t;  // absolute position: the rotation angle
  if (threadIdx.x < HALF) {
    const float theta = __fmul_rn(static_cast<float>(pos), p.inv_freq[threadIdx.x]);
    float s, c;
    sincosf(theta, &s, &c);
    cs[threadIdx.x] = c;
    sn[threadIdx.x] = s;
  }
  __syncthreads();

  const int hq = p.n_q_heads;
  const int hkv = p.kv.n_kv_heads;
  const bf16_t* q_row = static_cast<const bf16_t*>(p.q) + size_t(row) * hq * D;
  bf16_t* q_out_row = static_cast<bf16_t*>(p.q_out) + size_t(row) * hq * D;
  for (int it = threadIdx.x; it < hq * QUADS; it += blockDim.x) {
    const int head = it / QUADS;
    const int i0 = (it - head * QUADS) * 4;
    float a[4], b2[4], ra[4], rb[4];
    Vec4<bf16_t>::load(q_row + head * D + i0, a);
    Vec4<bf16_t>::load(q_row + head * D + i0 + HALF, b2);
#pragma unroll
    for (int j = 0; j < 4; ++j) rope_pair(a[j], b2[j], cs[i0 + j], sn[i0 + j], ra[j], rb[j]);
    Vec4<bf16_t>::store(q_out_row + head * D + i0, ra);
    Vec4<bf16_t>::store(q_out_row + head * D + i0 + HALF, rb);
  }

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int slot = slot_of(p.kv, pos);
  const size_t vec0 = (size_t(b) * p.kv.max_seq + slot) * hkv;  // this slot's first (head) vector
  for (int vi = wave; vi < 2 * hkv; vi += blockDim.x / kWave) {
    const bool is_k = vi < hkv;
    const int g = is_k ? vi : vi - hkv;
    const bf16_t* src = static_cast<const bf16_t*>(is_k ? p.k_new : p.v_new) + (size_t(row) * hkv + g) * D;
    float x[EPL];
#pragma unroll
    for (int u = 0; u < EPL; ++u) {
      const int e = lane + kWave * u;
      if (is_k) {
        const int i = e < HALF ? e : e - HALF;
        float xr, yr;
        rope_pair(bf16_to_f32(src[i]), bf16_to_f32(src[i + HALF]), cs[i], sn[i], xr, yr);
        x[u] = bf16_to_f32(f32_to_bf16(e < HALF ? xr : yr));
      } else {
        x[u] = bf16_to_f32(src[e]);
      }
    }
    float am = 0.f;
#pragma unroll
    for (int u = 0; u < EPL; ++u) am = fmaxf(am, fabsf(x[u]));
    am = wave_max(am);
    const float sc = am / 127.f;
    int8_t* dst = static_cast<int8_t*>(is_k ? p.kv.k : p.kv.v) + (vec0 + g) * D;
#pragma unroll
    for (int u = 0; u < EPL; ++u) {
      const float c = sc > 0.f ? fminf(fmaxf(rintf(x[u] / sc), -127.f), 127.f) : 0.f;
      dst[lane + kWave * u] = static_cast<int8_t>(c);
    }
    if (lane == 0) (is_k ? p.kv.k_scale : p.kv.v_scale)[(size_t(b) * hkv + g) * p.kv.max_seq + slot] = sc;
  }
}

hipError_t launch_rope_append_q8(const RopeAppendParams& p, hipStream_t s) {
  const dim3 grid(p.kv.batch * p.T), block(256);
  if (p.kv.head_dim == 128) hipLaunchKernelGGL((rope_append_q8_kernel<128>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((rope_append_q8_kernel<64>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rope_append(const RopeAppendParams& p, hipStream_t s) {
  const dim3 grid(p.kv.batch * p.T);
  const dim3 block(256);
  if (p.kv.dtype == KVC_BF16) {
    if (p.kv.head_dim == 128) hipLaunchKernelGGL((rope_append_kernel<bf16_t, 128>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((rope_append_kernel<bf16_t, 64>), grid, block, 0, s, p);
  } else {
    if (p.kv.head_dim == 128) hipLaunchKernelGGL((rope_append_kernel<float, 128>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((rope_append_kernel<float, 64>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
