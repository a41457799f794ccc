// Split-KV flash-decode on vector ALUs (no MFMA): the attention of one query
// token per (row, head) against the whole cached prefix.  The same kernel,
// with one split per query row written directly, is the float32 prefill and
// the float32 mixed call (rows (b, t) for t below the row's token count).
//
// Tiny-GPT post, Gotcha 2: a decode query sees every cached key.  nanochat
// post: attention runs against the full cache, the KV heads shared by groups
// of query heads (GQA).  Cake paper, Section 3: decode is memory-bound, which
// is why nothing here reshapes it into matrix-core work.
//
// Work unit = (row, KV head, block of GB query heads of its group, split of
// split_keys keys).  Four waves per workgroup take 64-key tiles of the split
// in turn and keep their own online-softmax state:
//   * a tile of K (then of V) is read from HBM with coalesced 16-byte loads
//     (16 lanes per 256-byte row) into registers one tile ahead, then staged
//     through this wave's LDS buffer;
//   * scores: lane j owns key j and forms all GB dot products from its K row
//     (padded LDS stride, conflict-free) against the query, whose bfloat16
//     pairs are wave-uniform and are read through the scalar cache, with
//     v_dot2_f32_bf16 (two multiply-adds per instruction);
//   * the tile max per head is a DPP + permute all-reduce; probabilities are
//     exp2 of log2-scaled scores;
//   * values: lane l owns two head dims and walks the keys in pairs, reading
//     (p_j, p_j+1) as one broadcast bfloat16 pair and (v_j, v_j+1) from two
//     conflict-free LDS rows, again with v_dot2_f32_bf16.
// The four waves fold their states in LDS at the end and write one partial
// (unnormalised o, running max, sum) per query head -- or, when a row has a
// single split, the normalised output directly.  The combine kernel folds
// the partials of a row's splits.
#include "kvc_device.h"
#include "kvc_launch.h"
#include "kvc.h"

namespace kvc {

namespace {

constexpr int kTile = 64;   // keys per wave tile
constexpr int kWaves = 4;   // waves per workgroup

template <typename T, int D, int GB>
struct SplitCfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kRowBytes = D * int(sizeof(T));
  static constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per K/V row
  static constexpr int kKStride = kRowBytes + 16;       // padded K row stride in LDS
  static constexpr int kBufBytes = kTile * kKStride;    // K or V tile buffer per wave
  static constexpr int kPBytes = 2 * kTile * GB * 4;    // probabilities + score slot per wave
  // Value phase: a unit is one dword of a V row (bf16: 2 dims, f32: 1 dim).
  static constexpr int kUnits = kBf16 ? D / 2 : D;
  static constexpr int kUnitsPerLane = kUnits >= kWave ? kUnits / kWave : 1;
  static constexpr int kLanesPerGroup = kUnits / kUnitsPerLane;  // lanes covering one row
  static constexpr int kKeyGroups = kWave / kLanesPerGroup;      // lane groups splitting the keys
  static constexpr int kDimsPerLane = kUnitsPerLane * (kBf16 ? 2 : 1);
  static constexpr int kLoadsPerLane = kTile * kChunks / kWave;
  static constexpr int kSmemBytes = kWaves * (kBufBytes + kPBytes);
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) u32x4_t* const_uint4_ptr;

template <typename T, int D, int GB>
__global__ __launch_bounds__(256, 1) void split_attention_kernel(SplitParams p) {
  using C = SplitCfg<T, D, GB>;
  extern __shared__ __align__(16) uint8_t smem[];

  const int hkv = p.kv.n_kv_heads;
  const int group = p.n_q_heads / hkv;
  const int n_hb = group / GB;  // query-head blocks per KV head
  int x = blockIdx.x;
  const int split = x % p.max_splits;
  x /= p.max_splits;
  const int hb_all = x % (hkv * n_hb);
  const int row = x / (hkv * n_hb);  // b * T + t
  const int g = hb_all / n_hb;
  const int h0 = g * group + (hb_all - g * n_hb) * GB;
  const int b = row / p.T;
  const int t = row - b * p.T;
  const RowTokens rt = row_tokens(p.kv, b, p.T);  // ragged calls: T = max_tokens
  if (rt.count < 0) {
    if (split == 0 && hb_all == 0 && t == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_TOKENS);
    return;
  }
  if (t >= rt.count || !row_selected(p.kv, rt.count)) return;
  const size_t tok = size_t(rt.first) + t;  // packed row of this query and its output

  const int n_keys = attended_keys(p.kv, p.kv.seqlens[b], rt.count, t);  // keys 0 .. start + t
  if (n_keys < 0) {
    if (split == 0 && hb_all == 0 && t == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_CAPACITY);
    return;
  }
  const int k_begin = split * p.split_keys;
  if (k_begin >= n_keys) return;
  const int k_end = min(k_begin + p.split_keys, n_keys);

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  uint8_t* buf = smem + wave * (C::kBufBytes + C::kPBytes);
  uint8_t* pbuf = buf + C::kBufBytes;

  const size_t key_stride = size_t(hkv) * D;  // elements between consecutive positions
  const T* k_base = static_cast<const T*>(p.kv.k) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;
  const T* v_base = static_cast<const T*>(p.kv.v) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;
  // The query block is read-only for the whole kernel: address it as constant
  // memory so that its wave-uniform loads go through the scalar cache.
  const const_uint4_ptr q_vec = reinterpret_cast<const_uint4_ptr>(
      reinterpret_cast<uintptr_t>(static_cast<const T*>(p.q) + (tok * p.n_q_heads + h0) * D));

  // Online-softmax state (log2 units); lpart is this lane's share of the sum.
  float m[GB], lpart[GB], acc[GB][C::kDimsPerLane];
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    m[h] = -INFINITY;
    lpart[h] = 0.f;
#pragma unroll
    for (int i = 0; i < C::kDimsPerLane; ++i) acc[h][i] = 0.f;
  }

  // Value-phase lane roles.
  const int kgrp = lane / C::kLanesPerGroup;
  const int unit0 = (lane % C::kLanesPerGroup) * C::kUnitsPerLane;

  uint4 kreg[C::kLoadsPerLane], vreg[C::kLoadsPerLane];
  auto load_tile = [&](int k0, uint4* kr, uint4* vr) {
#pragma unroll
    for (int i = 0; i < C::kLoadsPerLane; ++i) {
      const int f = lane + i * kWave;
      const int r = f / C::kChunks;
      const int c = f - r * C::kChunks;
      const int key = k0 + r;
      if (key < k_end) {
        kr[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(k_base + key * key_stride) + c * 16);
        vr[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(v_base + key * key_stride) + c * 16);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);  // keys past the end: zeros, never the (possibly poisoned) slot
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](const uint4* r_, int stride) {
#pragma unroll
    for (int i = 0; i < C::kLoadsPerLane; ++i) {
      const int f = lane + i * kWave;
      const int r = f / C::kChunks;
      const int c = f - r * C::kChunks;
      *reinterpret_cast<uint4*>(buf + r * stride + c * 16) = r_[i];
    }
  };

  int k0 = k_begin + wave * kTile;
  if (k0 < k_end) load_tile(k0, kreg, vreg);
  for (; k0 < k_end; k0 += kWaves * kTile) {
    // ---- scores: lane j <-> key k0 + j
    store_tile(kreg, C::kKStride);
    wave_lds_fence();
    float s[GB];
    uint4 kc[C::kChunks];  // this lane's K row
    {
      const uint4* krow = reinterpret_cast<const uint4*>(buf + lane * C::kKStride);
#pragma unroll
      for (int c = 0; c < C::kChunks; ++c) kc[c] = krow[c];
    }
    // One head at a time (a real loop): only that head's query is live in
    // SGPRs, read through the scalar cache; scores go to a per-wave LDS slot.
    float* sbuf = reinterpret_cast<float*>(pbuf) + kTile * GB;
#pragma unroll 1
    for (int h = 0; h < GB; ++h) {
      const const_uint4_ptr qh = q_vec + h * C::kChunks;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int c = 0; c < C::kChunks; ++c) {
        const u32x4_t qc = qh[c];
        if constexpr (C::kBf16) {
          a0 = dot2_bf16(qc.x, kc[c].x, a0);
          a1 = dot2_bf16(qc.y, kc[c].y, a1);
          a0 = dot2_bf16(qc.z, kc[c].z, a0);
          a1 = dot2_bf16(qc.w, kc[c].w, a1);
        } else {
          a0 = fmaf(__uint_as_float(qc.x), __uint_as_float(kc[c].x), a0);
          a1 = fmaf(__uint_as_float(qc.y), __uint_as_float(kc[c].y), a1);
          a0 = fmaf(__uint_as_float(qc.z), __uint_as_float(kc[c].z), a0);
          a1 = fmaf(__uint_as_float(qc.w), __uint_as_float(kc[c].w), a1);
        }
      }
      sbuf[lane * GB + h] = a0 + a1;
    }
    wave_lds_fence();
#pragma unroll
    for (int h = 0; h < GB; ++h) s[h] = sbuf[lane * GB + h];
    wave_lds_fence();
    // ---- stage V over K, then fetch the next tile while the ALUs work
    store_tile(vreg, C::kRowBytes);
    const int k_next = k0 + kWaves * kTile;
    if (k_next < k_end) load_tile(k_next, kreg, vreg);

    const bool valid = k0 + lane < k_end;
    float pr[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      const float sl = valid ? s[h] * p.scale_log2 : -INFINITY;
      const float m_new = fmaxf(m[h], wave_max(sl));  // finite: every tile holds a valid key
      const float alpha = exp2f(m[h] - m_new);
      pr[h] = exp2f(sl - m_new);
      lpart[h] = lpart[h] * alpha + pr[h];
      m[h] = m_new;
#pragma unroll
      for (int i = 0; i < C::kDimsPerLane; ++i) acc[h][i] *= alpha;
    }
    // ---- probabilities to LDS
    if constexpr (C::kBf16) {
      // (p_2i, p_2i+1) of head h as one bfloat16 pair at dword i * GB + h.
      bf16_t* pb = reinterpret_cast<bf16_t*>(pbuf);
#pragma unroll
      for (int h = 0; h < GB; ++h) pb[((lane >> 1) * GB + h) * 2 + (lane & 1)] = f32_to_bf16(pr[h]);
    } else {
      float* pf = reinterpret_cast<float*>(pbuf);
#pragma unroll
      for (int h = 0; h < GB; ++h) pf[lane * GB + h] = pr[h];
    }
    wave_lds_fence();
    // ---- values
    if constexpr (C::kBf16) {
      constexpr int kPairs = kTile / 2 / C::kKeyGroups;
      const uint32_t* vrows = reinterpret_cast<const uint32_t*>(buf);
      const uint32_t* pp = reinterpret_cast<const uint32_t*>(pbuf);
#pragma unroll 4
      for (int ii = 0; ii < kPairs; ++ii) {
        const int i = kgrp * kPairs + ii;
        uint32_t pw[GB];
#pragma unroll
        for (int h = 0; h < GB; ++h) pw[h] = pp[i * GB + h];
#pragma unroll
        for (int u = 0; u < C::kUnitsPerLane; ++u) {
          const uint32_t v0 = vrows[(2 * i) * (D / 2) + unit0 + u];
          const uint32_t v1 = vrows[(2 * i + 1) * (D / 2) + unit0 + u];
          const uint32_t lo = pack_lo16(v0, v1);  // (v_2i[d], v_2i+1[d])
          const uint32_t hi = pack_hi16(v0, v1);  // (v_2i[d+1], v_2i+1[d+1])
#pragma unroll
          for (int h = 0; h < GB; ++h) {
            acc[h][2 * u] = dot2_bf16(pw[h], lo, acc[h][2 * u]);
            acc[h][2 * u + 1] = dot2_bf16(pw[h], hi, acc[h][2 * u + 1]);
          }
        }
      }
    } else {
      constexpr int kKeys = kTile / C::kKeyGroups;
      const float* vrows = reinterpret_cast<const float*>(buf);
      const float* pf = reinterpret_cast<const float*>(pbuf);
#pragma unroll 4
      for (int jj = 0; jj < kKeys; ++jj) {
        const int j = kgrp * kKeys + jj;
#pragma unroll
        for (int u = 0; u < C::kUnitsPerLane; ++u) {
          const float vv = vrows[j * D + unit0 + u];
#pragma unroll
          for (int h = 0; h < GB; ++h) acc[h][u] = fmaf(pf[j * GB + h], vv, acc[h][u]);
        }
      }
    }
    wave_lds_fence();
  }

  // ---- this wave's totals
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    lpart[h] = wave_sum(lpart[h]);
    if constexpr (C::kKeyGroups > 1) {
#pragma unroll
      for (int i = 0; i < C::kDimsPerLane; ++i) acc[h][i] += __shfl_xor(acc[h][i], 32);
    }
  }
  __syncthreads();  // every wave is done with its tile buffers
  // Fold the four waves: per wave m[GB], l[GB], o[GB][D] in LDS.
  float* red = reinterpret_cast<float*>(smem);
  float* red_m = red;                       // [wave][GB]
  float* red_l = red + kWaves * GB;         // [wave][GB]
  float* red_o = red + 2 * kWaves * GB;     // [wave][GB][D]
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      red_m[wave * GB + h] = m[h];
      red_l[wave * GB + h] = lpart[h];
    }
  }
  if (kgrp == 0) {
#pragma unroll
    for (int h = 0; h < GB; ++h) {
#pragma unroll
      for (int i = 0; i < C::kDimsPerLane; ++i) {
        // bf16: unit u covers dims 2(unit0+u) and +1; f32: dim unit0+u.
        const int d = C::kBf16 ? 2 * unit0 + i : unit0 + i;
        red_o[(wave * GB + h) * D + d] = acc[h][i];
      }
    }
  }
  __syncthreads();
  const bool single = n_keys <= p.split_keys;  // this row has one split
  for (int e = threadIdx.x; e < GB * D; e += blockDim.x) {
    const int h = e / D;
    const int d = e - h * D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, red_m[w * GB + h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(red_m[w * GB + h] - mm);  // 0 for a wave that had no tile
      o += f * red_o[(w * GB + h) * D + d];
      l += f * red_l[w * GB + h];
    }
    const size_t qh = size_t(row) * p.n_q_heads + h0 + h;  // workspace slot of (row, head)
    if (p.direct || single) {
      const float y = o / l;
      const size_t oi = (tok * p.n_q_heads + h0 + h) * D + d;
      if constexpr (C::kBf16) static_cast<bf16_t*>(p.out)[oi] = f32_to_bf16(y);
      else static_cast<float*>(p.out)[oi] = y;
    } else {
      p.ws_o[(qh * p.max_splits + split) * D + d] = o;
      if (d == 0) {
        p.ws_ml[(qh * p.max_splits + split) * 2] = mm;
        p.ws_ml[(qh * p.max_splits + split) * 2 + 1] = l;
      }
    }
  }
}

// One workgroup of 64 lanes per (row, query head): fold the row's split partials.
template <typename T, int D>
__global__ __launch_bounds__(64) void split_combine_kernel(SplitParams p) {
  constexpr int kPer = D / kWave;
  const int qh = blockIdx.x;  // row * Hq + h: the workspace slot
  const int row = qh / p.n_q_heads;
  const int b = row / p.T;
  const int t = row - b * p.T;
  const RowTokens rt = row_tokens(p.kv, b, p.T);
  if (t >= rt.count || !row_selected(p.kv, rt.count)) return;  // includes malformed rows (count -1)
  const size_t oq = (size_t(rt.first) + t) * p.n_q_heads + (qh - row * p.n_q_heads);  // packed (token, head)
  const int n_keys = attended_keys(p.kv, p.kv.seqlens[b], rt.count, t);
  if (n_keys < 0) return;
  const int n_split = (n_keys + p.split_keys - 1) / p.split_keys;
  if (n_split <= 1) return;  // written directly by the split pass
  const float* ml = p.ws_ml + size_t(qh) * p.max_splits * 2;
  const float* o = p.ws_o + size_t(qh) * p.max_splits * D;
  float mm = -INFINITY;
  for (int s = 0; s < n_split; ++s) mm = fmaxf(mm, ml[2 * s]);
  float acc[kPer], den = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float f = exp2f(ml[2 * s] - mm);
    den += f * ml[2 * s + 1];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] += f * o[s * D + threadIdx.x + i * kWave];
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int d = threadIdx.x + i * kWave;
    if constexpr (sizeof(T) == 2) static_cast<bf16_t*>(p.out)[oq * D + d] = f32_to_bf16(acc[i] * inv);
    else static_cast<float*>(p.out)[oq * D + d] = acc[i] * inv;
  }
}

template <typename T, int D, int GB>
hipError_t launch_split_t(const SplitParams& p, hipStream_t s) {
  using C = SplitCfg<T, D, GB>;
  const int group = p.n_q_heads / p.kv.n_kv_heads;
  const long long n_blocks = (long long)p.max_splits * p.kv.n_kv_heads * (group / GB) * p.kv.batch * p.T;
  if (n_blocks <= 0 || n_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const auto kern = split_attention_kernel<T, D, GB>;
  static bool attr_set = false;  // raise the dynamic LDS limit once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kSmemBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(unsigned(n_blocks)), dim3(kWaves * kWave), C::kSmemBytes, s, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_split_d(const SplitParams& p, hipStream_t s) {
  const int group = p.n_q_heads / p.kv.n_kv_heads;
  if (group % 8 == 0) return launch_split_t<T, D, 8>(p, s);
  if (group % 4 == 0) return launch_split_t<T, D, 4>(p, s);
  if (group % 2 == 0) return launch_split_t<T, D, 2>(p, s);
  return launch_split_t<T, D, 1>(p, s);
}

}  // namespace

hipError_t launch_split_attention(const SplitParams& p, hipStream_t s) {
  if (p.kv.dtype != KVC_F32) return hipErrorInvalidValue;  // bfloat16 decode has its own kernel
  return p.kv.head_dim == 128 ? launch_split_d<float, 128>(p, s) : launch_split_d<float, 64>(p, s);
}

hipError_t launch_split_combine(const SplitParams& p, hipStream_t s) {
  const dim3 grid(p.kv.batch * p.T * p.n_q_heads);
  if (p.kv.dtype != KVC_F32) return hipErrorInvalidValue;
  if (p.kv.head_dim == 128) hipLaunchKernelGGL((split_combine_kernel<float, 128>), grid, dim3(kWave), 0, s, p);
  else hipLaunchKernelGGL((split_combine_kernel<float, 64>), grid, dim3(kWave), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
