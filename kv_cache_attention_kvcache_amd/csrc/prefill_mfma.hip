// Causal prefill attention on bfloat16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// Tiny-GPT post, Gotcha 2: a multi-token prompt attends causally.  Cake
// paper, Section 3 "Chunk Prefill" and Section 4 (Figure 4): a later chunk
// attends to every earlier token, so its cost grows with its start.  Read as
// absolute-position causality: query t of row b, at position P + t with
// P = seqlens[b], sees keys 0 .. P + t.
//
// This is the dense contraction of the path, so it runs on matrix cores.
// One workgroup = 128 queries of one query head (4 waves x 32 queries),
// looping over 64-key tiles of its KV head:
//   * S^T = K Q^T on MFMA: the K tile is the A operand from LDS (padded rows,
//     conflict-free), the wave's 32 query rows are the B operand held in
//     registers for the whole loop.  Computing S transposed leaves each lane
//     with 32 scores of ONE query, so the softmax max and sum are in-lane
//     plus one exchange with the lane 32 away.  The K rows are fed to the
//     MFMA in a permuted order so that each lane's scores are exactly the
//     8-key runs the P*V step needs as its B operand -- no shuffles.
//   * O^T += V^T P^T on MFMA: V is stored transposed in LDS (d-major, padded;
//     transposed in registers with byte permutes while staging), P^T comes
//     straight from the score registers rounded to bfloat16.
//   * Only tiles that reach past a wave's first query position are masked;
//     fully hidden tiles are never loaded.  The next tile's K/V is fetched
//     into registers while the current one is computed.
//   * Workgroups are ordered so that the query heads sharing a KV head run
//     on the same XCD (its L2 serves their common K/V stream), longest
//     (latest) query tiles first.
#include "kvc_device.h"
#include "kvc_launch.h"
#include "kvc.h"

namespace kvc {

namespace {

constexpr int kBM = 128;  // queries per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kWQ = 32;   // queries per wave
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer descriptor, 32-bit data format (gfx9 family)
constexpr float kLazyLog2 = 8.f;  // probabilities may reach 2^8 before the running max is raised
constexpr uint32_t kBf16One2 = 0x3F803F80u;  // (1.0, 1.0) as a bfloat16 pair

// 2^x on the transcendental unit, without the denormal-result fix-up of exp2f:
// softmax weights below 2^-126 flush to zero, which the float32 sums cannot see.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Row of the K tile fed to MFMA A-operand row i (i < 32) so that the score
// registers of each lane hold runs of 8 consecutive keys: output rows
// {0-3, 8-11} of a lane in the first half map to keys 0-7, and so on.
__device__ __forceinline__ int perm_row(int i) {
  return ((i >> 4) << 4) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillParams p) {
  constexpr int kKStride = D * 2 + 16;        // bytes per K row in LDS
  constexpr int kVStride = kBN * 2 + 16;      // bytes per transposed V row (one head dim)
  constexpr int kKD = D / 16;                 // MFMA k-steps over the head dim
  constexpr int kDB = D / 32;                 // 32-dim output blocks
  constexpr int kKLoads = kBN * D * 2 / 16 / 256;  // 16-byte K loads per thread per tile
  __shared__ __align__(16) uint8_t k_lds[kBN * kKStride];
  __shared__ __align__(16) uint8_t v_lds[D * kVStride];

  const int hq = p.n_q_heads;
  const int hkv = p.kv.n_kv_heads;
  const int group = hq / hkv;
  const int n_qt = (p.T + kBM - 1) / kBM;
  const int n_wg = n_qt * hq * p.kv.batch;
  // XCD-aware order: consecutive logical ids land on one XCD.
  const int x = blockIdx.x;
  const int lid = (n_wg % 8 == 0) ? (x % 8) * (n_wg / 8) + x / 8 : x;
  const int qt = n_qt - 1 - lid % n_qt;  // latest tiles first
  const int rest = lid / n_qt;
  const int h = rest % hq;
  const int b = rest / hq;
  const int g = h / group;

  const int start = p.kv.seqlens[b];
  if (start < 0 || start > p.kv.max_seq - p.T) {
    if (qt == n_qt - 1 && h == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_CAPACITY);
    return;
  }
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int half = lane >> 5;   // which half of the wave
  const int l32 = lane & 31;

  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kWQ;                       // this wave's first query
  const int kend_wg = start + min(q0 + kBM, p.T);        // keys the workgroup needs
  const int kend_w = qw0 < p.T ? start + min(qw0 + kWQ, p.T) : 0;  // keys this wave needs
  const int n_tiles = (kend_wg + kBN - 1) / kBN;

  // The wave's queries as MFMA B operand: lane holds query qw0 + l32,
  // head dims [16 kd + 8 half, +8) for each k-step kd.
  const int my_t = qw0 + l32;
  const int my_pos = start + my_t;
  uint4 qf[kKD];
  {
    const bf16_t* qrow = static_cast<const bf16_t*>(p.q) + (size_t(b) * p.T + my_t) * hq * D + size_t(h) * D;
#pragma unroll
    for (int kd = 0; kd < kKD; ++kd)
      qf[kd] = my_t < p.T ? *reinterpret_cast<const uint4*>(qrow + 16 * kd + 8 * half) : make_uint4(0, 0, 0, 0);
  }

  const size_t key_stride = size_t(hkv) * D;
  const bf16_t* k_base = static_cast<const bf16_t*>(p.kv.k) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;
  const bf16_t* v_base = static_cast<const bf16_t*>(p.kv.v) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;

  // Staging roles.  K: thread loads 16-byte chunks f = tid + 256 i of the tile.
  // V: thread owns keys 4 kq .. 4 kq + 3 and head dims 8 dc .. 8 dc + 7.
  // Loads are range-checked buffer loads whose descriptor starts at the tile's
  // first key: keys at or past kend_wg read as zeros, with no branch.
  const int kq = tid & 15;
  const int dc = tid >> 4;
  const bool v_active = dc < D / 8;
  const int row_bytes = hkv * D * 2;
  const int k_off = (tid / (D / 8)) * row_bytes + (tid % (D / 8)) * 16;  // + i * (256 / (D/8)) rows
  const int v_off = 4 * kq * row_bytes + dc * 16;                         // + r rows
  uint4 kreg[kKLoads], vreg[4];
  auto tile_rsrc = [&](const bf16_t* base, int kb0) {
    const int left = (kend_wg - kb0 - 1) * row_bytes + D * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base) + size_t(kb0) * key_stride, (short)0,
                                             left > 0 ? left : 0, kRsrcWord3);
  };
  auto load_tile = [&](int kb0) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(k_base, kb0);
#pragma unroll
    for (int i = 0; i < kKLoads; ++i)
      kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rk, k_off + i * (256 / (D / 8)) * row_bytes, 0, 0));
    if (v_active) {
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(v_base, kb0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off + r * row_bytes, 0, 0));
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int f = tid + 256 * i;
      const int r = f / (D / 8);
      const int c = f % (D / 8);
      *reinterpret_cast<uint4*>(k_lds + r * kKStride + c * 16) = kreg[i];
    }
    if (v_active) {
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int u = dd >> 1;
        const uint32_t w0 = u4_get(vreg[0], u), w1 = u4_get(vreg[1], u);
        const uint32_t w2 = u4_get(vreg[2], u), w3 = u4_get(vreg[3], u);
        uint2 out;
        out.x = (dd & 1) ? pack_hi16(w0, w1) : pack_lo16(w0, w1);
        out.y = (dd & 1) ? pack_hi16(w2, w3) : pack_lo16(w2, w3);
        *reinterpret_cast<uint2*>(v_lds + (8 * dc + dd) * kVStride + 8 * kq) = out;
      }
    }
  };

  f32x16_t o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c = p.scale_log2;
  const int arow = perm_row(l32);

  load_tile(0);
  for (int it = 0; it < n_tiles; ++it) {
    __syncthreads();  // all waves are done with the previous tile
    store_tile();
    __syncthreads();
    const int kb0 = it * kBN;
    if (it + 1 < n_tiles) load_tile(kb0 + kBN);
    if (kb0 >= kend_w) continue;  // nothing visible to this wave here

    // ---- S^T for 2 blocks of 32 keys (the first k-step starts from a zero accumulator)
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint8_t* arow_p = k_lds + (32 * kb + arow) * kKStride + 16 * half;
#pragma unroll
      for (int kd = 0; kd < kKD; ++kd) {
        const uint4 a = *reinterpret_cast<const uint4*>(arow_p + 32 * kd);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, qf[kd]),
                                                        kd == 0 ? f32x16_t{} : s[kb], 0, 0, 0);
      }
    }
    // Score register r of block kb belongs to key kb0 + 32 kb + 8 half + (r & 7) + 16 (r >> 3).
    if (kb0 + kBN - 1 > start + qw0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb0 + 32 * kb + 8 * half + (r & 7) + 16 * (r >> 3);
          s[kb][r] = key > my_pos ? -INFINITY : s[kb][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;  // this query's tile max, log2 units (finite: key 0 is visible)
    // Lazy maximum: m is raised (and o, l rescaled) only when a score exceeds it
    // by more than 2^8; otherwise probabilities up to 2^8 are accumulated as they
    // are.  The decision is wave-uniform.
    if (__ballot(mx > m + kLazyLog2)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);  // 0 on the first visible tile (m = -inf)
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    uint4 pf[4];  // B operands of the 4 k-steps of 16 keys
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(fmaf(s[kb][8 * hh + 2 * j], c, -m));
          const float p1 = fast_exp2(fmaf(s[kb][8 * hh + 2 * j + 1], c, -m));
          w[j] = pack_bf16x2(p0, p1);
          l = dot2_bf16(w[j], kBf16One2, l);  // the sum of the rounded probabilities P*V uses
        }
        pf[2 * kb + hh] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const uint4 a = *reinterpret_cast<const uint4*>(v_lds + (32 * db + l32) * kVStride + 32 * ks + 16 * half);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, pf[ks]), o[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store: o[db] register r holds head dim 32 db + 8 (r >> 2) + 4 half + (r & 3).
  const float l_tot = l + __shfl_xor(l, 32);
  if (my_t < p.T) {
    const float inv = 1.f / l_tot;
    bf16_t* orow = static_cast<bf16_t*>(p.out) + (size_t(b) * p.T + my_t) * hq * D + size_t(h) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * half;
        uint2 w;
        w.x = pack_bf16x2(o[db][4 * j] * inv, o[db][4 * j + 1] * inv);
        w.y = pack_bf16x2(o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams& p, hipStream_t s) {
  const int n_qt = (p.T + kBM - 1) / kBM;
  const long long n_wg = (long long)n_qt * p.n_q_heads * p.kv.batch;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.kv.head_dim == 128)
    hipLaunchKernelGGL((prefill_mfma_kernel<128>), dim3(unsigned(n_wg)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<64>), dim3(unsigned(n_wg)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
