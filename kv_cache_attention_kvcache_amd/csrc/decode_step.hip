// Fused decode step: RoPE + in-place K/V append + attention over the whole
// row, in one launch with no workspace.
//
// Tiny-GPT post, "Why the GPU Shrugs": at small shapes a cached decode step
// is bound by kernel launches, not arithmetic.  nanochat post, "What the KV
// cache looks like on disk": the new K/V slices are written in place at each
// row's offset and attention runs against the full cache in a single kernel
// launch.  The result is that of kvc_rope_append (T = 1) followed by
// kvc_attn_decode, up to the order of float32 additions.
//
// Workgroup (b, g) owns row b's KV head g and its G = Hq / Hkv query heads:
//   1. cos/sin of the row position P = seqlens[b] into LDS; the G query heads
//      and the key rotated with the same float32 pair rotation as
//      rope_append_kernel and rounded to the storage type once; the key and
//      the value written to slot P; the rounded queries kept in LDS;
//   2. keys 0..P in tiles of 256: thread = key for the scores, an online
//      softmax per head (wave reductions, then across the 4 waves through
//      LDS); for the weighted sum of V wave w takes every fourth key of the
//      tile and lane l the head dims l, l + 64, for all G heads at once; the
//      four waves' sums are added in a fixed order at the end.
// The kernel is bound by memory latency, not bandwidth: a key's V load is
// issued in chunks of 16 per lane before any of them is used (a loop that
// loads and uses one key per iteration waits for every load in turn: 64
// round trips per tile instead of 4), and a key row's loads all at once.
// The slot this workgroup wrote is read back by it after a barrier.
#include "kvc_device.h"
#include "kvc_launch.h"
#include "kvc.h"

namespace kvc {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;  // keys per tile: one per thread
constexpr int kWaves = kThreads / kWave;
constexpr int kVChunk = 16;  // V loads in flight per lane in the weighted sum (kVChunk * kWaves divides kTile)

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16_t x) { return bf16_to_f32(x); }
template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f32_to_bf16(x); }

// Eight consecutive elements as float (two 16-byte loads for float32, one for bfloat16).
__device__ __forceinline__ void load8(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  x[0] = bf16_lo(a.x); x[1] = bf16_hi(a.x); x[2] = bf16_lo(a.y); x[3] = bf16_hi(a.y);
  x[4] = bf16_lo(a.z); x[5] = bf16_hi(a.z); x[6] = bf16_lo(a.w); x[7] = bf16_hi(a.w);
}

// G: query heads per KV head rounded up to the template's bound (GB); heads
// h >= G are padding and skipped with uniform branches.
template <typename T, int D, int GB>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(DecodeStepParams p) {
  constexpr int HALF = D / 2;
  constexpr int kDU = D / kWave;  // head dims per lane in the weighted sum of V
  __shared__ float cs[HALF], sn[HALF];
  __shared__ __align__(16) float qs[GB][D];     // rotated, rounded queries
  __shared__ float pr[GB][kTile];               // one tile's probabilities
  __shared__ float red[kWaves][GB];             // per-wave partial max / sum
  __shared__ float part[kWaves][GB][D];         // per-wave sums of V, folded at the end

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int hq = p.n_q_heads;
  const int hkv = p.kv.n_kv_heads;
  const int G = hq / hkv;
  const int b = blockIdx.x / hkv;
  const int g = blockIdx.x - b * hkv;

  const int pos = p.kv.seqlens[b];  // absolute position of the new token: its rotation angle
  const int n_keys = attended_keys(p.kv, pos, 1, 0);
  if (n_keys < 0) {
    if (g == 0 && tid == 0) report(p.dev_err, KVC_DEV_CAPACITY);
    return;
  }

  // ---- 1. rotate the group's queries and the key at position pos; append.
  if (tid < HALF) {
    const float theta = __fmul_rn(static_cast<float>(pos), p.inv_freq[tid]);
    float s, c;
    sincosf(theta, &s, &c);
    cs[tid] = c;
    sn[tid] = s;
  }
  __syncthreads();
  const size_t slot = ((size_t(b) * p.kv.max_seq + slot_of(p.kv, pos)) * hkv + g) * D;
  for (int e = tid; e < (G + 1) * HALF; e += kThreads) {
    const int hh = e / HALF;  // hh < G: query head g G + hh; hh == G: the key
    const int i = e - hh * HALF;
    const T* src = hh < G ? static_cast<const T*>(p.q) + (size_t(b) * hq + g * G + hh) * D
                          : static_cast<const T*>(p.k_new) + (size_t(b) * hkv + g) * D;
    float xr, yr;
    rope_pair(to_f(src[i]), to_f(src[i + HALF]), cs[i], sn[i], xr, yr);
    const T xt = from_f<T>(xr), yt = from_f<T>(yr);
    if (hh < G) {
      qs[hh][i] = to_f(xt);
      qs[hh][i + HALF] = to_f(yt);
    } else {
      T* k_slot = static_cast<T*>(p.kv.k) + slot;
      k_slot[i] = xt;
      k_slot[i + HALF] = yt;
    }
  }
  {
    const T* v_src = static_cast<const T*>(p.v_new) + (size_t(b) * hkv + g) * D;
    T* v_slot = static_cast<T*>(p.kv.v) + slot;
    for (int i = tid; i < D; i += kThreads) v_slot[i] = v_src[i];
  }
  __syncthreads();  // queries in LDS; this workgroup's K/V slot written and visible to it

  // ---- 2. attention over the row's filled slots, online softmax across 256-key tiles.
  const size_t key_stride = size_t(hkv) * D;
  const T* k_base = static_cast<const T*>(p.kv.k) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;
  const T* v_base = static_cast<const T*>(p.kv.v) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;
  float m_run[GB], l_run[GB], acc[GB][kDU];
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int u = 0; u < kDU; ++u) acc[h][u] = 0.f;
  }

  for (int j0 = 0; j0 < n_keys; j0 += kTile) {
    const int j = j0 + tid;
    float s[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) s[h] = 0.f;
    if (j < n_keys) {
      const T* krow = k_base + size_t(j) * key_stride;
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 8) {
        float kx[8];
        load8(krow + d0, kx);
#pragma unroll
        for (int h = 0; h < GB; ++h) {
          if (h < G) {
#pragma unroll
            for (int u = 0; u < 8; ++u) s[h] = fmaf(qs[h][d0 + u], kx[u], s[h]);
          }
        }
      }
    }
    // Tile max per head, across the workgroup.
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      s[h] = j < n_keys ? s[h] * p.scale_log2 : -INFINITY;
      if (h < G) {
        const float wm = wave_max(s[h]);
        if (lane == 0) red[wave][h] = wm;
      }
    }
    __syncthreads();
    float m_new[GB], alpha[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      float mt = red[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mt = fmaxf(mt, red[w][h]);
      m_new[h] = fmaxf(m_run[h], mt);  // finite: key j0 < n_keys is in every tile
      alpha[h] = exp2f(m_run[h] - m_new[h]);
    }
    __syncthreads();  // red is reused for the sums
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      if (h < G) {
        const float pj = exp2f(s[h] - m_new[h]);  // 0 past the last key
        pr[h][tid] = pj;
        const float ws = wave_sum(pj);
        if (lane == 0) red[wave][h] = ws;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      float lt = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) lt += red[w][h];
      l_run[h] = l_run[h] * alpha[h] + lt;
      m_run[h] = m_new[h];
    }
    // Weighted sum of V: this wave's keys i = wave, wave + 4, ... of the tile,
    // this lane's head dims lane + 64 u, every head of the group.
    const int n_in = min(kTile, n_keys - j0);
#pragma unroll
    for (int h = 0; h < GB; ++h)
#pragma unroll
      for (int u = 0; u < kDU; ++u) acc[h][u] *= alpha[h];
    // The chunk's kVChunk loads are issued back to back before any is used: a
    // key past the tile's last is read at the last key's index (a filled slot)
    // and weighted by its probability, 0.  i stays below kTile.
    const T* vrow = v_base + size_t(j0) * key_stride + lane;
    for (int i0 = wave; i0 < n_in; i0 += kVChunk * kWaves) {
      float vv[kVChunk][kDU];
#pragma unroll
      for (int c = 0; c < kVChunk; ++c) {
        const int ic = min(i0 + kWaves * c, n_in - 1);
#pragma unroll
        for (int u = 0; u < kDU; ++u) vv[c][u] = to_f(vrow[size_t(ic) * key_stride + kWave * u]);
      }
#pragma unroll
      for (int c = 0; c < kVChunk; ++c) {
        const int i = i0 + kWaves * c;
#pragma unroll
        for (int h = 0; h < GB; ++h) {
          if (h < G) {
            const float ph = pr[h][i];
#pragma unroll
            for (int u = 0; u < kDU; ++u) acc[h][u] = fmaf(ph, vv[c][u], acc[h][u]);
          }
        }
      }
    }
    __syncthreads();  // pr and red are rewritten by the next tile
  }

  // ---- fold the four waves' sums (fixed order), normalise and store.
#pragma unroll
  for (int h = 0; h < GB; ++h)
    if (h < G)
#pragma unroll
      for (int u = 0; u < kDU; ++u) part[wave][h][lane + kWave * u] = acc[h][u];
  __syncthreads();
  for (int o = tid; o < G * D; o += kThreads) {
    const int h = o / D;
    const int d = o - h * D;
    const float sum = (part[0][h][d] + part[1][h][d]) + (part[2][h][d] + part[3][h][d]);
    float lr = l_run[0];
#pragma unroll
    for (int hh = 1; hh < GB; ++hh) lr = hh == h ? l_run[hh] : lr;
    static_cast<T*>(p.out)[(size_t(b) * hq + g * G + h) * D + d] = from_f<T>(sum / lr);
  }
}

template <typename T, int D>
hipError_t launch_t(const DecodeStepParams& p, hipStream_t s) {
  const int G = p.n_q_heads / p.kv.n_kv_heads;
  const dim3 grid(p.kv.batch * p.kv.n_kv_heads), block(kThreads);
  if (G <= 1) hipLaunchKernelGGL((decode_step_kernel<T, D, 1>), grid, block, 0, s, p);
  else if (G <= 2) hipLaunchKernelGGL((decode_step_kernel<T, D, 2>), grid, block, 0, s, p);
  else if (G <= 4) hipLaunchKernelGGL((decode_step_kernel<T, D, 4>), grid, block, 0, s, p);
  else if (G <= 8) hipLaunchKernelGGL((decode_step_kernel<T, D, 8>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((decode_step_kernel<T, D, kDecodeStepMaxGroup>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step(const DecodeStepParams& p, hipStream_t s) {
  if (p.kv.dtype == KVC_BF16)
    return p.kv.head_dim == 128 ? launch_t<bf16_t, 128>(p, s) : launch_t<bf16_t, 64>(p, s);
  return p.kv.head_dim == 128 ? launch_t<float, 128>(p, s) : launch_t<float, 64>(p, s);
}

}  // namespace kvc
