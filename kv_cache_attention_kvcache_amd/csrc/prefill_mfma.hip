// Causal prefill attention on bfloat16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// Tiny-GPT post, Gotcha 2: a multi-token prompt attends causally.  Cake
// paper, Section 3 "Chunk Prefill" and Section 4 (Figure 4): a later chunk
// attends to every earlier token, so its cost grows with its start.  Read as
// absolute-position causality: query t of row b, at position P + t with
// P = seqlens[b], sees keys 0 .. P + t.
//
// This is the dense contraction of the path, so it runs on matrix cores.
// One workgroup = 256 queries of one query head (8 waves x 32 queries),
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
//     fully hidden tiles are never loaded.  P*V of the previous tile runs
//     beside the softmax of the current one.  The next tile's V is fetched
//     into registers while the current one is computed.
//   * At head_dim 128 the K tiles skip the registers: buffer loads write them
//     straight into one of four LDS buffers, two tiles ahead, with the 16-byte
//     chunks of each row XOR-swizzled by the row index so the MFMA operand
//     reads stay conflict-free without padding (a DMA fills LDS contiguously).
//     The four buffers are one array, so a lane's eight swizzled read
//     addresses serve every buffer and block through the instruction offset.
//     Each step then needs one barrier, and the waits on those loads are
//     written out (vmcnt with lgkmcnt), since the fence of __syncthreads would
//     wait for every load in flight, the next tiles' included.  Other head
//     sizes stage K through registers into two padded buffers.
//   * Workgroups are ordered so that the query heads sharing a KV head run
//     on the same XCD (its L2 serves their common K/V stream), longest
//     (latest) query tiles first.
//   * In a ragged call (the prefill half of kvc_attn_mixed) each row has its
//     own token count and first packed row; the grid covers the largest count
//     and workgroups past a row's tokens, or of rows with fewer than two
//     tokens, return at once.
#include <type_traits>
#include "kvc_device.h"
#include "kvc_launch.h"
#include "kvc.h"

namespace kvc {

namespace {

constexpr int kBN = 64;   // keys per tile
constexpr int kWQ = 32;   // queries per wave
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer descriptor, 32-bit data format (gfx9 family)
constexpr float kLazyBound = 256.f;  // probabilities may reach 2^8 before the running max is raised
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

// WAVES = 8: 256 queries per workgroup, one workgroup per CU (two waves per SIMD).
// WAVES = 4: 128 queries per workgroup, for calls whose 8-wave grid has fewer
// workgroups than the device has CUs (a short prompt at few heads): twice the
// workgroups, so more CUs have work.  Same tiles, pipeline and register budget.
template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void prefill_mfma_kernel(PrefillParams p) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kBM = kWQ * WAVES;            // queries per workgroup
  constexpr int kKStride = D * 2 + 16;        // bytes per K row in LDS
  constexpr int kVStride = kBN * 2 + 16;      // bytes per transposed V row (one head dim)
  constexpr int kKD = D / 16;                 // MFMA k-steps over the head dim
  constexpr int kDB = D / 32;                 // 32-dim output blocks
  constexpr int kKLoads = kBN * D * 2 / 16 / kThreads;  // 16-byte K loads per thread per tile
  // head_dim 128: K goes from memory straight into LDS (buffer_load ... lds), four buffers,
  // 16-byte chunks XOR-swizzled per row; otherwise register-staged into two padded buffers.
  constexpr bool kDma = D == 128;
  constexpr int kDmaBytes = kBN * D * 2;
  __shared__ __align__(16) uint8_t k_lds[kDma ? 1 : 2][kDma ? 16 : kBN * kKStride];
  __shared__ __align__(16) uint8_t k_dma[kDma ? 4 * kDmaBytes : 16];
  uint8_t* const k_dma0 = k_dma;
  uint8_t* const k_dma1 = k_dma + (kDma ? kDmaBytes : 0);
  uint8_t* const k_dma2 = k_dma + (kDma ? 2 * kDmaBytes : 0);
  uint8_t* const k_dma3 = k_dma + (kDma ? 3 * kDmaBytes : 0);
  __shared__ __align__(16) uint8_t v_lds[2][D * kVStride];    // V^T tiles, two buffers

  const int hq = p.n_q_heads;
  const int hkv = p.kv.n_kv_heads;
  const int group = hq / hkv;
  const int n_qt = (p.T + kBM - 1) / kBM;
  // XCD-aware order.  Workgroup x runs on XCD x mod 8, and each XCD starts its
  // workgroups in the order of x / 8.  The query heads of one KV head share its
  // K/V stream, so they go to one XCD, whose L2 serves them all.  When the
  // (row, KV head) groups split evenly over the 8 XCDs, group k goes to XCD
  // k mod 8: every XCD gets a share of every row, so rows of unequal length (a
  // ragged call's chunk beside idle rows) still spread over the whole chip.
  // Within an XCD, all its heads' latest (longest) query tiles start first,
  // then the next latest, and so on.  Otherwise, when at least the (row, query
  // head) pairs split evenly, XCD i takes a consecutive run of them, in the
  // same longest-first order; else workgroups go in plain order.
  const int x = blockIdx.x;
  int qt, rest;
  if ((p.kv.batch * hkv) % 8 == 0) {
    const int rpx = hq * p.kv.batch / 8;  // (row, head) pairs per XCD
    const int j = x / 8;                  // start order within the XCD
    qt = n_qt - 1 - j / rpx;
    const int r = j % rpx;
    const int kg = (r / group) * 8 + x % 8;  // (row, KV head) group b * hkv + g
    rest = (kg / hkv) * hq + (kg % hkv) * group + r % group;
  } else if ((hq * p.kv.batch) % 8 == 0) {
    const int rpx = hq * p.kv.batch / 8;
    const int j = x / 8;
    qt = n_qt - 1 - j / rpx;
    rest = (x % 8) * rpx + j % rpx;
  } else {
    qt = n_qt - 1 - x % n_qt;
    rest = x / n_qt;
  }
  const int h = rest % hq;
  const int b = rest / hq;
  const int g = h / group;

  // This row's new tokens (ragged calls: its own count, packed from `tok0`; the
  // grid is sized for max_tokens) and whether this launch handles it.
  const RowTokens rt = row_tokens(p.kv, b, p.T);
  if (!row_selected(p.kv, rt.count)) {
    if (rt.count < 0 && qt == 0 && h == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_TOKENS);
    return;
  }
  const int T = rt.count;
  const size_t tok0 = size_t(rt.first);
  if (qt * kBM >= T) return;  // a query tile past this row's tokens
  const int start = p.kv.seqlens[b];
  if (start < 0 || start > p.kv.max_seq - T) {
    if (qt == 0 && h == 0 && threadIdx.x == 0) report(p.dev_err, KVC_DEV_CAPACITY);
    return;
  }
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int half = lane >> 5;   // which half of the wave
  const int l32 = lane & 31;

  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kWQ;                       // this wave's first query
  const int kend_wg = start + min(q0 + kBM, T);          // keys the workgroup needs
  const int n_tiles = (kend_wg + kBN - 1) / kBN;

  // The wave's queries as MFMA B operand: lane holds query qw0 + l32,
  // head dims [16 kd + 8 half, +8) for each k-step kd.
  const int my_t = qw0 + l32;
  const int my_pos = start + my_t;
  uint4 qf[kKD];
  {
    const bf16_t* qrow = static_cast<const bf16_t*>(p.q) + (tok0 + my_t) * hq * D + size_t(h) * D;
#pragma unroll
    for (int kd = 0; kd < kKD; ++kd)
      qf[kd] = my_t < T ? *reinterpret_cast<const uint4*>(qrow + 16 * kd + 8 * half) : make_uint4(0, 0, 0, 0);
  }

  const size_t key_stride = size_t(hkv) * D;
  const bf16_t* k_base = static_cast<const bf16_t*>(p.kv.k) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;
  const bf16_t* v_base = static_cast<const bf16_t*>(p.kv.v) + size_t(b) * p.kv.max_seq * key_stride + size_t(g) * D;

  // Staging roles.  K: thread loads 16-byte chunks f = tid + kThreads i of the tile.
  // V: thread owns keys 2 kq, 2 kq + 1 and, for each u < kVPer, head dims
  // 8 dc_u .. 8 dc_u + 7 with dc_u = dc + (kThreads / 32) u.
  // Loads are range-checked buffer loads whose descriptor starts at the tile's
  // first key: keys at or past kend_wg read as zeros, with no branch.
  constexpr int kDcStep = kThreads / 32;                      // head-dim groups staged side by side
  constexpr int kVPer = (D / 8 + kDcStep - 1) / kDcStep;      // groups per thread
  const int kq = tid & 31;
  const int dc = tid >> 5;
  const int row_bytes = hkv * D * 2;
  const int k_off = (tid / (D / 8)) * row_bytes + (tid % (D / 8)) * 16;  // + i * (kThreads / (D/8)) rows
  const int v_off = 2 * kq * row_bytes + dc * 16;                         // + r rows, + 16 kDcStep u bytes
  uint4 kreg[kKLoads], vreg[kVPer][2];
  auto tile_rsrc = [&](const bf16_t* base, int kb0) {
    const int left = (kend_wg - kb0 - 1) * row_bytes + D * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base) + size_t(kb0) * key_stride, (short)0,
                                             left > 0 ? left : 0, kRsrcWord3);
  };
  auto load_k = [&](int tile) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(k_base, tile * kBN);
#pragma unroll
    for (int i = 0; i < kKLoads; ++i)
      kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rk, k_off + i * (kThreads / (D / 8)) * row_bytes, 0, 0));
  };
  auto load_v = [&](int tile) {
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(v_base, tile * kBN);
#pragma unroll
    for (int u = 0; u < kVPer; ++u)
      if (dc + kDcStep * u < D / 8) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
          vreg[u][r] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off + 16 * kDcStep * u + r * row_bytes, 0, 0));
      }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int f = tid + kThreads * i;
      const int r = f / (D / 8);
      const int c = f % (D / 8);
      *reinterpret_cast<uint4*>(k_lds[buf] + r * kKStride + c * 16) = kreg[i];
    }
  };
  auto store_v = [&](int buf) {  // transposed: V^T rows are head dims
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int dcu = dc + kDcStep * u;
      if (dcu >= D / 8) continue;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int e = dd >> 1;
        const uint32_t w0 = u4_get(vreg[u][0], e), w1 = u4_get(vreg[u][1], e);
        *reinterpret_cast<uint32_t*>(v_lds[buf] + (8 * dcu + dd) * kVStride + 4 * kq) =
            (dd & 1) ? pack_hi16(w0, w1) : pack_lo16(w0, w1);
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

  // S^T of one tile: 2 blocks of 32 keys, the first k-step from a zero accumulator.
  // All 16 K fragments are read first; the two blocks' chains alternate.
  auto qk_from = [&](const uint8_t* kbase, f32x16_t* s) {
    uint4 kf[2 * kKD];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kd = 0; kd < kKD; ++kd) {
        const int r = 32 * kb + arow;
        kf[kb * kKD + kd] =
            kDma ? *reinterpret_cast<const uint4*>(kbase + (r * 16 + ((2 * kd + half) ^ (r & 15))) * 16)
                 : *reinterpret_cast<const uint4*>(kbase + r * kKStride + 16 * half + 32 * kd);
      }
#pragma unroll
    for (int kd = 0; kd < kKD; ++kd)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[kb * kKD + kd]),
                                                        __builtin_bit_cast(bf16x8_t, qf[kd]),
                                                        kd == 0 ? f32x16_t{} : s[kb], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKD, 0);  // every K fragment read first
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kKD, 0);  // then the score MFMAs
  };
  auto qk = [&](int buf, f32x16_t* s) { qk_from(k_lds[buf], s); };
  // Keys past a query's position get score -inf.  Only tiles that reach past
  // the wave's first query need it; a tile wholly past every query of the wave
  // masks to -inf throughout and contributes exact zeros.
  auto mask = [&](int t, f32x16_t* s) {
    const int kb0 = t * kBN;
    if (kb0 + kBN - 1 > start + qw0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // score register r of block kb belongs to key kb0 + 32 kb + 8 half + (r & 7) + 16 (r >> 3)
          const int key = kb0 + 32 * kb + 8 * half + (r & 7) + 16 * (r >> 3);
          s[kb][r] = key > my_pos ? -INFINITY : s[kb][r];
        }
    }
  };
  // Probabilities of one tile's (masked) scores against the running maximum
  // m, as the bfloat16 B operands of P*V, and the sum of the rounded values
  // in lt.  Branch-free, so that it interleaves with the previous tile's P*V
  // MFMAs.  No per-tile maximum is taken first: the caller checks lt instead.
  auto probs = [&](const f32x16_t* s, uint4* pf, float& lt) {
    lt = 0.f;
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
          lt = dot2_bf16(w[j], kBf16One2, lt);  // the sum of the rounded probabilities P*V uses
        }
        pf[2 * kb + hh] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };
  // Lazy maximum: m is raised only when a probability would exceed 2^8, which
  // the row sum lt reveals (it bounds every term; it is inf or NaN on the first
  // tile, where m = -inf).  Then the tile's true maximum is taken and the
  // probabilities are recomputed; returns the factor that rescales o and l.
  auto raise_max = [&](const f32x16_t* s, uint4* pf, float& lt) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;  // this query's tile max, log2 units
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);  // 0 on the first tile (m = -inf)
    m = m_new;
    probs(s, pf, lt);
    return alpha;
  };
  // The V^T fragments of one tile (A operands of the 4 k-steps x kDB output blocks).
  auto read_v = [&](int buf, uint4* vf) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        vf[ks * kDB + db] =
            *reinterpret_cast<const uint4*>(v_lds[buf] + (32 * db + l32) * kVStride + 32 * ks + 16 * half);
  };
  // O^T += V^T P^T for one tile.
  auto pv = [&](const uint4* vf, const uint4* pf) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[ks * kDB + db]),
                                                        __builtin_bit_cast(bf16x8_t, pf[ks]), o[db], 0, 0, 0);
  };
  // Softmax of one tile's masked scores into pf, with the lazy rescale of o and l.
  auto soft = [&](f32x16_t* s, uint4* pf) {
    float lt;
    probs(s, pf, lt);
    if (__ballot(!(lt <= kLazyBound)) != 0) {
      // A real (wave-uniform) branch: without the asm the compiler if-converts
      // this block and multiplies o by alpha = 1 on every tile.
      asm volatile("");
      const float alpha = raise_max(s, pf, lt);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    l += lt;
  };

  // Software pipeline over the workgroup's tiles.  Entering step j (after a
  // barrier): K(j) sits in k_lds[j&1], V(j-1) in v_lds[(j-1)&1], P(j-1) in
  // registers, and the staging registers hold K(j+1) and V(j).  The step issues
  // the score MFMAs of tile j, stores K(j+1) and V(j) into the buffers the last
  // barrier freed, starts the loads of K(j+2) and V(j+1), reads the V^T
  // fragments of tile j-1, masks S(j), then accumulates P(j-1) V(j-1) beside
  // the softmax of tile j: one barrier per tile.  Loads past the last tile read
  // zeros (the range check), so every step runs unconditionally.
  auto step = [&](int j, const uint4* pf_prev, uint4* pf_cur) {
    f32x16_t s[2];
    uint4 vf[4 * kDB];
    qk(j & 1, s);
    store_k((j + 1) & 1);
    store_v(j & 1);
    load_k(j + 2);
    load_v(j + 1);
    read_v((j - 1) & 1, vf);
    mask(j, s);
    pv(vf, pf_prev);
    soft(s, pf_cur);
    __syncthreads();
  };
  if constexpr (kDma) {
    typedef __attribute__((address_space(3))) void* lds_ptr;
    constexpr int kKDma = kDmaBytes / 16 / kThreads;  // 1 KB DMA instructions per wave per tile
    constexpr int kVLoads = 2 * kVPer;                  // V loads per thread per tile
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto dma_k = [&](int tile, uint8_t* dst) {
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(k_base, tile * kBN);
#pragma unroll
      for (int i = 0; i < kKDma; ++i) {
        const int blk = i * WAVES + wave_u;  // this instruction's 1 KB of the tile in LDS
        const int pch = blk * 64 + lane;     // LDS chunk the lane's 16 bytes land in
        const int r = pch >> 4;
        const int c = (pch & 15) ^ (r & 15);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(dst + blk * 1024), 16, r * row_bytes + c * 16, 0, 0, 0);
      }
    };
    // vmcnt(vm) with lgkmcnt(0): every LDS access of this wave done, and all but its vm latest
    // vector memory instructions.
    auto wait_vm = [&](auto vmc) {
      constexpr int vm = decltype(vmc)::value;
      __builtin_amdgcn_s_waitcnt((vm & 0xF) | ((vm >> 4) << 14) | (7 << 4));
    };
    auto barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    uint4 pa[4], pb[4];
    dma_k(0, k_dma0);
    dma_k(1, k_dma1);
    load_v(0);
    wait_vm(std::integral_constant<int, 0>{});
    store_v(0);
    load_v(1);
    dma_k(2, k_dma2);
    wait_vm(std::integral_constant<int, kKDma + kVLoads>{});
    barrier();
    {
      f32x16_t s[2];
      qk_from(k_dma0, s);
      mask(0, s);
      soft(s, pa);
    }
    wait_vm(std::integral_constant<int, kKDma + kVLoads>{});
    barrier();  // every wave has read K(0) before K(4) lands in its buffer
    // Step j: K(j) in kc, K(j+1) landed or in flight, V(j) in registers, V(j-1) in v_lds.
    auto dstep = [&](int j, const uint8_t* kc, uint8_t* kn2, const uint4* pf_prev, uint4* pf_cur) {
      f32x16_t s[2];
      uint4 vf[4 * kDB];
      qk_from(kc, s);
      store_v(j & 1);
      dma_k(j + 2, kn2);
      load_v(j + 1);
      read_v((j - 1) & 1, vf);
      mask(j, s);
      pv(vf, pf_prev);
      soft(s, pf_cur);
      wait_vm(std::integral_constant<int, kKDma + kVLoads>{});  // K(j+1) has landed
      barrier();
    };
    int j = 1;
    for (; j + 3 < n_tiles; j += 4) {
      dstep(j, k_dma1, k_dma3, pa, pb);
      dstep(j + 1, k_dma2, k_dma0, pb, pa);
      dstep(j + 2, k_dma3, k_dma1, pa, pb);
      dstep(j + 3, k_dma0, k_dma2, pb, pa);
    }
    if (j < n_tiles) dstep(j, k_dma1, k_dma3, pa, pb);
    if (j + 1 < n_tiles) dstep(j + 1, k_dma2, k_dma0, pb, pa);
    if (j + 2 < n_tiles) dstep(j + 2, k_dma3, k_dma1, pa, pb);
    // The last steps issued loads of tiles past the end (no memory is read for them); none
    // may still be writing this workgroup's LDS when it exits.
    wait_vm(std::integral_constant<int, 0>{});
    {
      uint4 vf[4 * kDB];
      read_v((n_tiles - 1) & 1, vf);
      pv(vf, ((n_tiles - 1) & 1) ? pb : pa);
    }
  } else {
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  load_k(1);
  store_k(1);
  load_v(1);
  load_k(2);
  __syncthreads();
  uint4 pa[4], pb[4];  // P(j) of even and odd tiles
  {
    f32x16_t s[2];
    qk(0, s);
    mask(0, s);
    soft(s, pa);
  }
  __syncthreads();  // every wave has read K(0) before step 1 stores K(2) over it
  int j = 1;
  for (; j + 1 < n_tiles; j += 2) {
    step(j, pa, pb);
    step(j + 1, pb, pa);
  }
  if (j < n_tiles) step(j, pa, pb);
  {
    uint4 vf[4 * kDB];
    read_v((n_tiles - 1) & 1, vf);
    pv(vf, ((n_tiles - 1) & 1) ? pb : pa);
  }
  }

  // ---- normalise and store: o[db] register r holds head dim 32 db + 8 (r >> 2) + 4 half + (r & 3).
  const float l_tot = l + __shfl_xor(l, 32);
  if (my_t < T) {
    const float inv = 1.f / l_tot;
    bf16_t* orow = static_cast<bf16_t*>(p.out) + (tok0 + my_t) * hq * D + size_t(h) * D;
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

template <int WAVES>
hipError_t launch_waves(const PrefillParams& p, hipStream_t s) {
  const int n_qt = (p.T + kWQ * WAVES - 1) / (kWQ * WAVES);
  const long long n_wg = (long long)n_qt * p.n_q_heads * p.kv.batch;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.kv.head_dim == 128)
    hipLaunchKernelGGL((prefill_mfma_kernel<128, WAVES>), dim3(unsigned(n_wg)), dim3(64 * WAVES), 0, s, p);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<64, WAVES>), dim3(unsigned(n_wg)), dim3(64 * WAVES), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillParams& p, hipStream_t s) {
  // 8-wave workgroups unless their grid would leave CUs without a workgroup.
  const long long n_wg8 = (long long)((p.T + kWQ * 8 - 1) / (kWQ * 8)) * p.n_q_heads * p.kv.batch;
  return n_wg8 < p.n_cus ? launch_waves<4>(p, s) : launch_waves<8>(p, s);
}

}  // namespace kvc
