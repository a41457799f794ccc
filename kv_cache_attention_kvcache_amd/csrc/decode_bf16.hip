// Split-KV flash-decode for bfloat16 and int8 caches, on vector ALUs (no MFMA).
//
// Tiny-GPT post, Gotcha 2: a decode query sees every cached key.  nanochat
// post ("What the KV cache looks like on disk"): attention runs against the
// full cache, with KV heads shared by groups of query heads (GQA).  Cake paper,
// Section 3: decode is memory-bound -- here it moves about 8 flops per K/V byte
// at a GQA group of 8 -- so nothing is reshaped into matrix-core work.
//
// Work partition.  A segment is (row b, KV head g, block hb of GB query heads
// of its group); it holds ceil(L_b / 32) tiles of 32 keys, L_b = seqlens[b]+1
// (min(seqlens[b]+1, max_seq) filled slots in a rolling window).
// All segments laid end to end form N tiles; the grid is persistent (one
// workgroup per CU by default) and workgroup w takes the tiles
// [w N / P, (w+1) N / P) -- the same K/V bytes per workgroup whatever the
// lengths, so batch 1 at 73K keys and batch 64 with ragged lengths balance
// alike.  The range is cut into runs (its intersection with each segment);
// the four waves of the workgroup take the tiles of a run in turn.  At the end
// of a run the waves fold their softmax states in LDS; a run that is a whole
// segment writes the normalised output, any other run a float32 partial
// (unnormalised o, running max, sum).  A workgroup writes at most two partials
// (its first run and its last), and the combine kernel folds them per segment.
// In a ragged call (the decode half of kvc_attn_mixed) only rows with exactly
// one new token have tiles, and a row's query and output sit at its packed row.
//
// One 32-key tile, per wave:
//   * K and V are read with coalesced 16-byte buffer loads, 16 lanes per
//     256-byte row (8 per 128-byte row at head_dim 64).  The buffer's range
//     check returns zeros for keys at or past L_b, so no lane reads a slot of
//     the cache it must not.  The next tile of the wave is always in flight
//     while the current one is computed.
//   * Scores: each lane dots its 8 head dims of its K rows against those dims
//     of all GB queries (v_dot2_f32_bf16), then a DPP transpose-reduction
//     across the lanes of a row sums the partial dots and leaves every lane
//     with complete scores of one query head for two or four keys.  The lanes
//     load the queries in a lane-dependent head order so that every exchange
//     is a single add with a DPP operand (no selects).
//   * Softmax: exp2 of log2-scaled scores against a per-head running maximum
//     that is raised lazily -- only when a score exceeds it by more than 2^8
//     (a ballot), so most tiles skip the max reduction and the rescale.
//   * P*V: probabilities go to LDS as bfloat16 key pairs; V goes to LDS as
//     key-pair-packed dims; each lane then owns head_dim/64 output dims of all
//     GB heads and accumulates with v_dot2_f32_bf16 (two keys per product).
//
// int8 caches (Cake paper, Section 5.1 "Compression methods" and Section 5.5:
// 8-bit quantization halves the bytes to move): a lane loads the 8 int8 codes
// of its 8 head dims (8-byte loads, 8 lanes per 128-byte row) and widens them
// to bfloat16 pairs, which hold every code exactly; everything after that is
// the bfloat16 path.  Each lane also loads the float32 scales of the keys it
// keeps after the reduction, with the tile: a key's K scale multiplies its
// scores, its V scale multiplies the probability that weights its codes in
// P*V, while the softmax sum takes the unscaled probability.
#include "kvc_device.h"
#include "kvc_launch.h"
#include "kvc.h"

namespace kvc {

namespace {

constexpr int kTileKeys = 32;   // keys per wave tile
constexpr int kWaves = 4;       // waves per workgroup
constexpr float kLazyLog2 = 8.f;  // probabilities may reach 2^8 before the max is raised
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

template <int D, int GB>
struct Cfg {
  static constexpr int LPR = D / 8;                 // lanes per K/V row (16 bytes each)
  static constexpr int RPI = kWave / LPR;           // rows per load instruction (= row groups)
  static constexpr int NR = kTileKeys / RPI;        // K/V rows (slots) per lane per tile
  static constexpr int S = LPR == 16 ? 4 : 3;       // transpose-reduction steps
  static constexpr int HB = GB == 8 ? 3 : 2;        // steps that split the head axis
  static constexpr int NRK = NR >> (S - HB);        // rows a lane keeps after the reduction
  static constexpr int NPK = NRK / 2;               // key pairs a lane keeps
  static constexpr int DL = D / kWave;              // output dims per lane in P*V
  static constexpr int NPAIR = kTileKeys / 2;       // key pairs per tile
  static constexpr int kVBytes = NPAIR * D * 4;     // V tile, key-pair packed
  static constexpr int kPBytes = NPAIR * GB * 4;    // probabilities, key-pair packed
  static constexpr int kWaveLds = kVBytes + kPBytes;
  static constexpr int kMergeBytes = kWaves * GB * (D + 2) * 4;
  static constexpr int kLds = kWaves * kWaveLds > kMergeBytes ? kWaves * kWaveLds : kMergeBytes;
  static_assert(NPK >= 1 && NR % 2 == 0, "tile shape");
};

// DPP control of reduction step k: lane x exchanges with x ^ m_k inside its row
// group.  head_dim 128 (16-lane groups): m = 8 (row_ror:8), 7 (row_half_mirror),
// 2, 1 (quad perms).  head_dim 64 (8-lane groups): 7, 2, 1.
template <int LPR, int K>
constexpr int step_ctrl() {
  if constexpr (LPR == 16) return K == 0 ? 0x128 : K == 1 ? 0x141 : K == 2 ? 0x4E : 0xB1;
  else return K == 0 ? 0x141 : K == 1 ? 0x4E : 0xB1;
}
template <int LPR, int K>
constexpr int step_mask() {
  if constexpr (LPR == 16) return K == 0 ? 8 : K == 1 ? 7 : K == 2 ? 2 : 1;
  else return K == 0 ? 7 : K == 1 ? 2 : 1;
}

// gh: the linear map (over GF(2)) from a lane's index x within its row group
// to the XOR applied to its query-head order.  It satisfies gh(m_k) = GB/2^(k+1)
// for the head-splitting steps and gh(m_k) = 0 for the row-splitting ones, so
// that the value a lane sends at every step is exactly the one its partner keeps.
template <int LPR, int GB>
__host__ __device__ constexpr int gh(int x) {
  // images of the lane-index bits 0..3
  constexpr int img128_8[4] = {0, 1, 3, 4};
  constexpr int img128_4[4] = {0, 0, 1, 2};
  constexpr int img64_8[3] = {1, 2, 7};
  constexpr int img64_4[3] = {0, 1, 3};
  int r = 0;
  for (int bit = 0; bit < (LPR == 16 ? 4 : 3); ++bit) {
    if ((x >> bit) & 1) {
      if constexpr (LPR == 16) r ^= GB == 8 ? img128_8[bit] : img128_4[bit];
      else r ^= GB == 8 ? img64_8[bit] : img64_4[bit];
    }
  }
  return r;
}

// Lane (within row group 0) that holds the scores of head h after the reduction.
template <int LPR, int GB>
__host__ __device__ constexpr int lane_of_head(int h) {
  for (int x = 0; x < LPR; ++x)
    if (gh<LPR, GB>(x) == h) return x;
  return 0;
}

template <int K>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), K, 0xf, 0xf, true));
}

// 16-byte buffer load with the non-temporal hint: K/V are streamed once per
// call, and keeping them out of the caches' retention lifts the sustained read
// rate (measured on MI355X: about 5.6 -> 6.6 TB/s for 256-byte rows at a 2 KiB stride).
constexpr int kCpolNT = 2;
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, kCpolNT);
}

// What a lane loads of one K/V row (its 8 head dims) and how it becomes the
// four bfloat16 pairs the dot products take.
template <bool Q8>
struct Elem;
template <>
struct Elem<false> {  // bfloat16: 16 bytes
  typedef u32x4_t Raw;
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, int off) { return buffer_load16(r, off); }
  static __device__ __forceinline__ u32x4_t widen(const Raw& w) { return w; }
};
template <>
struct Elem<true> {  // int8 codes: 8 bytes, widened exactly (|code| <= 127 fits bfloat16's 8 significant bits)
  typedef u32x2_t Raw;
  static constexpr int kBytes = 1;
  static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolNT);
  }
  static __device__ __forceinline__ uint32_t pair(uint32_t w, int byte) {
    return pack_bf16x2(static_cast<float>(static_cast<int8_t>(w >> (8 * byte))),
                       static_cast<float>(static_cast<int8_t>(w >> (8 * byte + 8))));
  }
  static __device__ __forceinline__ u32x4_t widen(const Raw& w) {
    return u32x4_t{pair(w.x, 0), pair(w.x, 2), pair(w.y, 0), pair(w.y, 2)};
  }
};

// Keys row b's decode query attends, and their 32-key tiles (0 when negative):
// -1 out of range (KVC_DEV_CAPACITY); -2 not in this launch (a ragged call's row
// with no token or with a prefill chunk); -3 a malformed token range (KVC_DEV_TOKENS).
__device__ __forceinline__ int row_keys(const LayerView& kv, int b) {
  if (kv.cu_tokens) {
    const RowTokens rt = row_tokens(kv, b, 1);
    if (rt.count < 0) return -3;
    if (rt.count != 1 || !row_selected(kv, rt.count)) return -2;
  }
  return attended_keys(kv, kv.seqlens[b], 1, 0);
}
// Packed row of row b's query and output (row b itself unless the call is ragged).
__device__ __forceinline__ int row_token(const LayerView& kv, int b) { return kv.cu_tokens ? kv.cu_tokens[b] : b; }
__device__ __forceinline__ int row_tiles(const LayerView& kv, int b) {
  const int n = row_keys(kv, b);
  return n < 0 ? 0 : (n + kTileKeys - 1) / kTileKeys;
}

// The value of lane 0, known to the compiler to be wave-uniform (an SGPR).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return uniform(x);
}

__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Tiles of all segments (N) and the segment holding flattened tile t.
struct SegPos {
  int b, sr, nt, base;  // row, segment within row, tiles per segment of row b, first tile
};

__device__ int total_tiles(const DecodeParams& p, int lane) {
  int n = 0;
  for (int b0 = 0; b0 < p.kv.batch; b0 += kWave) {
    const int b = b0 + lane;
    n += wave_sum_i(b < p.kv.batch ? row_tiles(p.kv, b) : 0);
  }
  return n * p.kv.n_kv_heads * p.n_hb;
}

__device__ SegPos find_segment(const DecodeParams& p, int t, int lane) {
  const int spr = p.kv.n_kv_heads * p.n_hb;  // segments per row
  int cum = 0;
  for (int b0 = 0; b0 < p.kv.batch; b0 += kWave) {
    const int b = b0 + lane;
    const int nt = b < p.kv.batch ? row_tiles(p.kv, b) : 0;
    const int incl = wave_incl_scan_i(nt * spr, lane);
    const int total = uniform(__shfl(incl, kWave - 1));
    if (cum + total > t) {
      const unsigned long long hit = __ballot(cum + incl > t);
      const int first = __builtin_ctzll(hit);
      SegPos s;
      s.b = uniform(b0 + first);
      s.nt = uniform(__shfl(nt, first));
      const int row_base = uniform(cum + __shfl(incl, first) - s.nt * spr);
      s.sr = (t - row_base) / s.nt;
      s.base = row_base + s.sr * s.nt;
      return s;
    }
    cum += total;
  }
  SegPos s = {0, 0, 0, 0};
  return s;  // not reached for t < N
}

// Flattened tile index w N / P where workgroup w's range starts.
__device__ __forceinline__ int range_begin(long long w, int n, int n_wg) { return int(w * n / n_wg); }

template <int D, int GB, bool Q8>
__global__ __launch_bounds__(kWaves * kWave, 1) void decode_bf16_kernel(DecodeParams p) {
  using C = Cfg<D, GB>;
  using E = Elem<Q8>;
  using Raw = typename E::Raw;
  constexpr int LPR = C::LPR;
  __shared__ __align__(16) uint8_t smem[C::kLds];

  const int wave = uniform(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int x = lane % LPR;      // lane within its row group
  const int rg = lane / LPR;     // row group
  const int ghx = gh<LPR, GB>(x);

  const int n_tiles = total_tiles(p, lane);
  const int t_begin = range_begin(blockIdx.x, n_tiles, p.n_wg);
  const int t_end = range_begin(blockIdx.x + 1LL, n_tiles, p.n_wg);
  if (t_begin >= t_end) return;

  const int hq = p.n_q_heads;
  const int hkv = p.kv.n_kv_heads;
  const int group = hq / hkv;
  const int spr = hkv * p.n_hb;
  const int row_bytes = hkv * D * E::kBytes;  // bytes between consecutive positions of one head
  const float c = p.scale_log2;

  uint8_t* vlds = smem + wave * C::kWaveLds;
  uint32_t* plds = reinterpret_cast<uint32_t*>(vlds + C::kVBytes);

  // Per-lane byte offset of slot s's row within a tile: row = 2 (s/2 * RPI + rg) + (s & 1).
  const int lane_off = 2 * rg * row_bytes + x * 8 * E::kBytes;
  // The slots a lane keeps after the row-splitting steps start at off_keep;
  // their rows (for the int8 scales) are fixed for the whole call.
  int off_keep = 0;
#pragma unroll
  for (int k = C::HB; k < C::S; ++k) off_keep += ((x >> (C::S - 1 - k)) & 1) * ((C::NR >> (k - C::HB)) / 2);
  int sc_off[C::NRK];  // byte offset of kept row r's scale within a tile's (dense) scale run
#pragma unroll
  for (int r = 0; r < C::NRK; ++r) {
    const int slot = r + off_keep;
    sc_off[r] = (2 * ((slot >> 1) * C::RPI + rg) + (slot & 1)) * 4;
  }

  SegPos seg = find_segment(p, t_begin, lane);
  int t = t_begin;
  bool first_run = true;
  while (t < t_end) {
    const int seg_end = seg.base + seg.nt;
    const int run_end = min(t_end, seg_end);
    const bool complete = t == seg.base && run_end == seg_end;
    const int g = seg.sr / p.n_hb;
    const int hb = seg.sr - g * p.n_hb;
    const int L = row_keys(p.kv, seg.b);  // >= 1: the run has tiles
    const int j0 = t - seg.base, j1 = run_end - seg.base;  // local tiles of the run

    // Segment bases (row b, position 0, KV head g).
    const size_t vec0 = size_t(seg.b) * p.kv.max_seq * hkv + g;
    const uint8_t* kseg = static_cast<const uint8_t*>(p.kv.k) + vec0 * D * E::kBytes;
    const uint8_t* vseg = static_cast<const uint8_t*>(p.kv.v) + vec0 * D * E::kBytes;
    const size_t sc0 = (size_t(seg.b) * hkv + g) * p.kv.max_seq;  // scales are head-major
    const float* ksseg = Q8 ? p.kv.k_scale + sc0 : nullptr;
    const float* vsseg = Q8 ? p.kv.v_scale + sc0 : nullptr;

    // Queries of this block in this lane's head order: slot h holds head h ^ gh(x), dims [8x, 8x+8).
    u32x4_t q[GB];
    {
      const bf16_t* qrow =
          static_cast<const bf16_t*>(p.q) + (size_t(row_token(p.kv, seg.b)) * hq + g * group + hb * GB) * D;
#pragma unroll
      for (int h = 0; h < GB; ++h) {
        const int head = h ^ ghx;
        q[h] = hb * GB + head < group ? *reinterpret_cast<const u32x4_t*>(qrow + head * D + 8 * x)
                                      : u32x4_t{0u, 0u, 0u, 0u};
      }
    }

    float mh = -INFINITY;  // running max (log2 units) of head ghx
    float lpart = 0.f;     // this lane's share of the sum of head ghx
    float acc[GB][C::DL];
#pragma unroll
    for (int h = 0; h < GB; ++h)
#pragma unroll
      for (int i = 0; i < C::DL; ++i) acc[h][i] = 0.f;

    auto rsrc_at = [&](const uint8_t* base, int j) {
      const int key0 = j * kTileKeys;
      const int left = (L - key0 - 1) * row_bytes + D * E::kBytes;  // valid bytes from the tile's first row
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + size_t(key0) * row_bytes, (short)0,
                                               left > 0 ? left : 0, kRsrcWord3);
    };
    auto issue = [&](const uint8_t* base, int j, Raw* buf) {
      const __amdgpu_buffer_rsrc_t r = rsrc_at(base, j);
#pragma unroll
      for (int s = 0; s < C::NR; ++s) {
        const int off = lane_off + (2 * (s >> 1) * C::RPI + (s & 1)) * row_bytes;
        buf[s] = E::load(r, off);
      }
    };
    // int8: the scales of this lane's kept rows of tile j (zeros past the row's length).
    auto issue_sc = [&](const float* base, int j, float* buf) {
      if constexpr (Q8) {
        const int key0 = j * kTileKeys;
        const int left = (L - key0) * 4;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(base) + key0, (short)0, left > 0 ? left : 0, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < C::NRK; ++i)
          buf[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, sc_off[i], 0, kCpolNT));
      }
    };

    // Tile j: K in kb and V in vb, one register stage each: the wave's next K
    // tile is issued as soon as this one's dots are formed, its next V tile as
    // soon as this one is in LDS.  (A second K stage, keeping two K tiles in
    // flight, streamed about 2% slower: more partial-row requests in flight
    // cost the memory side more than they hide.)
    // k_next / v_next: tiles to issue into kb / vb once they are consumed (-1: none).
    auto process = [&](int j, Raw* kb, float* ksb, Raw* vb, float* vsb, int k_next, int v_next) {
      // ---- partial dots of slot s against the GB queries, then the head-splitting
      // steps of the transpose-reduction (independent per slot, so each slot is
      // reduced as soon as its dots are formed).
      float R[C::NR][1];
#pragma unroll
      for (int s = 0; s < C::NR; ++s) {
        float r8[GB];
        const u32x4_t kw = E::widen(kb[s]);
#pragma unroll
        for (int h = 0; h < GB; ++h) {
          float a = dot2_bf16(q[h].x, kw.x, 0.f);
          a = dot2_bf16(q[h].y, kw.y, a);
          a = dot2_bf16(q[h].z, kw.z, a);
          r8[h] = dot2_bf16(q[h].w, kw.w, a);
        }
#define KVC_HSTEP(K)                                                         \
  if constexpr (K < C::HB) {                                                 \
    constexpr int n = GB >> K;                                               \
    _Pragma("unroll") for (int h = 0; h < n / 2; ++h)                        \
      r8[h] += dpp<step_ctrl<LPR, K>()>(r8[h + n / 2]);                      \
  }
        KVC_HSTEP(0)
        KVC_HSTEP(1)
        KVC_HSTEP(2)
#undef KVC_HSTEP
        R[s][0] = r8[0];
      }
      float ks[C::NRK];  // this tile's K scales, taken before the stage is reused
#pragma unroll
      for (int r = 0; r < C::NRK; ++r) ks[r] = Q8 ? ksb[r] : 1.f;
      if (k_next >= 0) {  // this K stage is free again
        issue(kseg, k_next, kb);
        issue_sc(ksseg, k_next, ksb);
      }
      // ---- row-splitting steps: the lane keeps the half of its slots its index bit selects
      int off = 0;
#define KVC_RSTEP(K)                                                         \
  if constexpr (K >= C::HB && K < C::S) {                                    \
    constexpr int nr = C::NR >> (K - C::HB);                                 \
    const int bit = (x >> (C::S - 1 - K)) & 1;                               \
    _Pragma("unroll") for (int r = 0; r < nr / 2; ++r) {                     \
      const float keep = bit ? R[r + nr / 2][0] : R[r][0];                   \
      const float send = bit ? R[r][0] : R[r + nr / 2][0];                   \
      R[r][0] = keep + dpp<step_ctrl<LPR, K>()>(send);                       \
    }                                                                        \
    off += bit * (nr / 2);                                                   \
  }
      KVC_RSTEP(2)
      KVC_RSTEP(3)
#undef KVC_RSTEP
      // ---- softmax of head ghx over this lane's NRK keys
      const int key0 = j * kTileKeys;
      float y[C::NRK];
#pragma unroll
      for (int r = 0; r < C::NRK; ++r) {
        const int slot = r + off;
        const int row = 2 * ((slot >> 1) * C::RPI + rg) + (slot & 1);
        y[r] = key0 + row < L ? R[r][0] * (Q8 ? c * ks[r] : c) : -INFINITY;
      }
      bool raise = false;
#pragma unroll
      for (int r = 0; r < C::NRK; ++r) raise |= y[r] > mh + kLazyLog2;
      if (__ballot(raise)) {
        float ym = y[0];
#pragma unroll
        for (int r = 1; r < C::NRK; ++r) ym = fmaxf(ym, y[r]);
        // lanes of one head: the row-splitting partners, then the other row groups
        if constexpr (C::S - C::HB >= 1) ym = fmaxf(ym, __shfl_xor(ym, step_mask<LPR, C::S - 1>()));
        if constexpr (C::S - C::HB >= 2) ym = fmaxf(ym, __shfl_xor(ym, step_mask<LPR, C::S - 2>()));
#pragma unroll
        for (int o = LPR; o < kWave; o <<= 1) ym = fmaxf(ym, __shfl_xor(ym, o));
        const float m_new = fmaxf(mh, ym);  // finite: key 0 of the tile is always valid
        const float alpha = exp2f(mh - m_new);
        lpart *= alpha;
        mh = m_new;
#pragma unroll
        for (int h = 0; h < GB; ++h) {
          const float ah = __shfl(alpha, lane_of_head<LPR, GB>(h));
#pragma unroll
          for (int i = 0; i < C::DL; ++i) acc[h][i] *= ah;
        }
      }
      float pr[C::NRK];
#pragma unroll
      for (int r = 0; r < C::NRK; ++r) {
        pr[r] = exp2f(y[r] - mh);
        lpart += pr[r];
      }
      // ---- probabilities and V to this wave's LDS, both key-pair packed
      wave_lds_fence();  // the previous tile's P*V reads are done
#pragma unroll
      for (int jp = 0; jp < C::NPK; ++jp) {
        const int pair = ((2 * jp + off) >> 1) * C::RPI + rg;
        if constexpr (Q8)
          plds[pair * GB + ghx] = pack_bf16x2(pr[2 * jp] * vsb[2 * jp], pr[2 * jp + 1] * vsb[2 * jp + 1]);
        else
          plds[pair * GB + ghx] = pack_bf16x2(pr[2 * jp], pr[2 * jp + 1]);
      }
#pragma unroll
      for (int sp = 0; sp < C::NR / 2; ++sp) {
        const int pair = sp * C::RPI + rg;
        const u32x4_t v0 = E::widen(vb[2 * sp]), v1 = E::widen(vb[2 * sp + 1]);
        uint4 a, b;
        a.x = pack_lo16(v0.x, v1.x); a.y = pack_hi16(v0.x, v1.x);
        a.z = pack_lo16(v0.y, v1.y); a.w = pack_hi16(v0.y, v1.y);
        b.x = pack_lo16(v0.z, v1.z); b.y = pack_hi16(v0.z, v1.z);
        b.z = pack_lo16(v0.w, v1.w); b.w = pack_hi16(v0.w, v1.w);
        uint4* dst = reinterpret_cast<uint4*>(vlds + (pair * D + 8 * x) * 4);
        dst[0] = a;
        dst[1] = b;
      }
      if (v_next >= 0) {
        issue(vseg, v_next, vb);
        issue_sc(vsseg, v_next, vsb);
      }
      wave_lds_fence();
      // ---- P*V: lane owns dims [DL*lane, DL*lane + DL) of all GB heads
#pragma unroll 4
      for (int i = 0; i < C::NPAIR; ++i) {
        uint32_t pw[GB];
#pragma unroll
        for (int h4 = 0; h4 < GB / 4; ++h4) {
          const uint4 w4 = *reinterpret_cast<const uint4*>(plds + i * GB + 4 * h4);
          pw[4 * h4] = w4.x; pw[4 * h4 + 1] = w4.y; pw[4 * h4 + 2] = w4.z; pw[4 * h4 + 3] = w4.w;
        }
        uint32_t vw[C::DL];
        if constexpr (C::DL == 2) {
          const uint2 v2 = *reinterpret_cast<const uint2*>(vlds + (i * D + 2 * lane) * 4);
          vw[0] = v2.x;
          vw[1] = v2.y;
        } else {
          vw[0] = *reinterpret_cast<const uint32_t*>(vlds + (i * D + lane) * 4);
        }
#pragma unroll
        for (int h = 0; h < GB; ++h)
#pragma unroll
          for (int d = 0; d < C::DL; ++d) acc[h][d] = dot2_bf16(pw[h], vw[d], acc[h][d]);
      }
    };

    // The wave's tiles of this run: j0 + wave, j0 + wave + 4, ...
    Raw kb[C::NR], vb[C::NR];
    float ksb[C::NRK], vsb[C::NRK];
    int j = j0 + wave;
    if (j < j1) {
      issue(kseg, j, kb);
      issue_sc(ksseg, j, ksb);
      issue(vseg, j, vb);
      issue_sc(vsseg, j, vsb);
    }
    auto next = [&](int jj) { return jj < j1 ? jj : -1; };
    for (; j < j1; j += kWaves) process(j, kb, ksb, vb, vsb, next(j + kWaves), next(j + kWaves));

    // ---- fold the four waves' states of this run
    // sum of head ghx over the lanes that hold it (row-splitting partners, then row groups)
    if constexpr (C::S - C::HB >= 1) lpart += __shfl_xor(lpart, step_mask<LPR, C::S - 1>());
    if constexpr (C::S - C::HB >= 2) lpart += __shfl_xor(lpart, step_mask<LPR, C::S - 2>());
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) lpart += __shfl_xor(lpart, o);
    __syncthreads();  // every wave is done with its V / P buffers
    float* red_ml = reinterpret_cast<float*>(smem);            // [wave][GB][2]
    float* red_o = red_ml + kWaves * GB * 2;                   // [wave][GB][D]
    if (rg == 0) {  // lane lane_of_head(h) of row group 0 holds head h's max and sum
#pragma unroll
      for (int h = 0; h < GB; ++h)
        if (x == lane_of_head<LPR, GB>(h)) {
          red_ml[(wave * GB + h) * 2] = mh;
          red_ml[(wave * GB + h) * 2 + 1] = lpart;
        }
    }
#pragma unroll
    for (int h = 0; h < GB; ++h)
#pragma unroll
      for (int d = 0; d < C::DL; ++d) red_o[(wave * GB + h) * D + C::DL * lane + d] = acc[h][d];
    __syncthreads();
    const int slot = first_run ? 0 : 1;
    for (int e = threadIdx.x; e < GB * D; e += kWaves * kWave) {
      const int h = e / D;
      const int d = e - h * D;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, red_ml[(w * GB + h) * 2]);
      float o = 0.f, l = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(red_ml[(w * GB + h) * 2] - mm);  // 0 for a wave with no tile here
        o += f * red_o[(w * GB + h) * D + d];
        l += f * red_ml[(w * GB + h) * 2 + 1];
      }
      if (complete) {
        if (hb * GB + h < group)
          static_cast<bf16_t*>(p.out)[(size_t(row_token(p.kv, seg.b)) * hq + g * group + hb * GB + h) * D + d] =
              f32_to_bf16(o / l);
      } else {
        const size_t ps = (size_t(blockIdx.x) * 2 + slot) * GB + h;
        p.ws_o[ps * D + d] = o;
        if (d == 0) {
          p.ws_ml[ps * 2] = mm;
          p.ws_ml[ps * 2 + 1] = l;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next run

    first_run = false;
    t = run_end;
    if (t < t_end) {  // next segment (rows of length 0 hold no tiles and are skipped)
      seg.base = seg_end;
      if (++seg.sr == spr) {
        seg.sr = 0;
        do {
          ++seg.b;
          seg.nt = row_tiles(p.kv, seg.b);
        } while (seg.nt == 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// int8 caches on matrix cores.
//
// At a GQA group of 8, widening the int8 codes and forming the 2 x 8 products
// of every cached element pair on vector ALUs costs more ALU time per HBM
// byte than the chip has (that path streams about 1.6 TB/s).  Here the
// products run on MFMA (v_mfma_f32_32x32x16_bf16) and the vector ALUs only
// widen codes and run the softmax.  A segment is (row, KV head) with all its
// query heads (G <= 32) as the 32 columns of the MFMA B operand; the tile
// partition, the per-run fold of the four waves and the partials are those of
// decode_bf16_kernel with a 32-head block.
//
// One 32-key tile, per wave:
//   * S^T = K Q^T.  Lane (A row i, half h) holds the key of tile row
//     perm_key(i): the order that leaves each lane with two 8-key runs of its
//     head's scores, which is the B operand P*V needs.  The head-dim axis of
//     the contraction is permuted the same way for K and for Q: at k-step
//     2m + e a lane's 8 elements are head dims 32m + 16h + 8e .. +8, so each
//     16-byte load of 16 codes gives the lane two k-steps.  Codes widen to
//     bfloat16 exactly (|code| <= 127).
//   * The tile's 32 K scales and 32 V scales go through wave-private LDS (one
//     load per lane).  A key's K scale multiplies its scores, its V scale the
//     probability that weights its codes in P*V; the softmax sum takes the
//     unscaled probability.  Lazy running max per head as in the vector path.
//   * V^T in LDS as bfloat16 key pairs per head dim; O^T += V^T P^T.
constexpr int kQ8Cols = kDecodeQ8Block;  // query heads per segment (MFMA columns)
// Tiles whose loads are in flight per wave.  One streams fastest: the K loads take 32 bytes
// of 32 rows each, and a second tile's worth of such partial-row requests slows the memory
// side more than it hides latency (measured at 72K context: 272 us against 282-285 us at
// batch 8; three tiles no longer fit the registers).
#ifndef KVC_Q8_STAGES
#define KVC_Q8_STAGES 1
#endif
constexpr int kQ8Stages = KVC_Q8_STAGES;

// Tile row fed as A-operand row i so that output register r of lane (column,
// half h) holds key 16 (r >> 3) + 8 h + (r & 7).
__device__ __forceinline__ int perm_key(int i) {
  return ((i >> 4) << 4) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3);
}

__device__ __forceinline__ uint32_t i8_pair_bf16(uint32_t w, int byte) {
  return pack_bf16x2(static_cast<float>(static_cast<int8_t>(w >> (8 * byte))),
                     static_cast<float>(static_cast<int8_t>(w >> (8 * byte + 8))));
}

template <int D>
__global__ __launch_bounds__(kWaves * kWave, 2) void decode_q8_mfma_kernel(DecodeParams p) {
  // Compiled for two workgroups per CU, which caps a wave at 256 registers and keeps every
  // MFMA operand in VGPRs (a 512-register budget brings AGPR copies); launched one per CU,
  // which streams faster.
  constexpr int GB = kQ8Cols;
  constexpr int kM = D / 32;                      // 16-byte K loads per lane per tile
  constexpr int kKD = D / 16;                     // MFMA k-steps of S^T
  constexpr int kDB = D / 32;                     // 32-dim blocks of O^T
  constexpr int kVItems = 16 * (D / 16) / kWave;  // (key pair, 16-dim group) items per lane
  constexpr int kVStride = 80;                    // bytes per head-dim row of V^T: 16 key pairs + pad
  constexpr int kWaveLds = D * kVStride + 64 * 4;
  constexpr int kMerge = kWaves * GB * (D + 2) * 4;
  constexpr int kLds = kWaves * kWaveLds > kMerge ? kWaves * kWaveLds : kMerge;
  __shared__ __align__(16) uint8_t smem[kLds];

  const int wave = uniform(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int n_tiles = total_tiles(p, lane);
  const int t_begin = range_begin(blockIdx.x, n_tiles, p.n_wg);
  const int t_end = range_begin(blockIdx.x + 1LL, n_tiles, p.n_wg);
  if (t_begin >= t_end) return;

  const int hq = p.n_q_heads;
  const int hkv = p.kv.n_kv_heads;
  const int group = hq / hkv;
  const int spr = hkv;  // one 32-head block per KV head
  const int row_bytes = hkv * D;
  const float c = p.scale_log2;
  const int key_a = perm_key(l32);  // this lane's A-operand key within a tile

  uint8_t* vt = smem + wave * kWaveLds;                           // V^T of the wave's tile
  float* scl = reinterpret_cast<float*>(vt + D * kVStride);       // [0,32) K scales, [32,64) V scales

  SegPos seg = find_segment(p, t_begin, lane);
  int t = t_begin;
  bool first_run = true;
  while (t < t_end) {
    const int seg_end = seg.base + seg.nt;
    const int run_end = min(t_end, seg_end);
    const bool complete = t == seg.base && run_end == seg_end;
    const int g = seg.sr;
    const int L = row_keys(p.kv, seg.b);  // >= 1: the run has tiles
    const int j0 = t - seg.base, j1 = run_end - seg.base;

    const size_t vec0 = size_t(seg.b) * p.kv.max_seq * hkv + g;
    const uint8_t* kseg = static_cast<const uint8_t*>(p.kv.k) + vec0 * D;
    const uint8_t* vseg = static_cast<const uint8_t*>(p.kv.v) + vec0 * D;
    const size_t sc0 = (size_t(seg.b) * hkv + g) * p.kv.max_seq;  // scales are head-major
    const float* ksseg = p.kv.k_scale + sc0;
    const float* vsseg = p.kv.v_scale + sc0;

    // Q^T B operands: lane (column = query head l32 of the group, half): head
    // dims 32m + 16 half + 8e .. +8 at k-step 2m + e; zero for padding heads.
    u32x4_t qb[kKD];
    {
      const bool valid = l32 < group;
      const bf16_t* qrow = static_cast<const bf16_t*>(p.q) +
                           (size_t(row_token(p.kv, seg.b)) * hq + g * group + (valid ? l32 : 0)) * D;
#pragma unroll
      for (int m = 0; m < kM; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          qb[2 * m + e] = valid ? *reinterpret_cast<const u32x4_t*>(qrow + 32 * m + 16 * half + 8 * e)
                                : u32x4_t{0u, 0u, 0u, 0u};
    }
    f32x16_t o[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float mh = -INFINITY, lpart = 0.f;  // head l32's running max (log2 units) and this lane's share of its sum

    auto rsrc_at = [&](const void* base, int j, int unit, int per_key) {
      const int key0 = j * kTileKeys;
      const int left = (L - key0 - 1) * per_key + unit;  // valid bytes from the tile's first key
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(base)) +
                                                   size_t(key0) * per_key,
                                               (short)0, left > 0 ? left : 0, kRsrcWord3);
    };
    struct Stage {
      u32x4_t k[kM];
      u32x4_t v[kVItems][2];
      float ks, vs;
    };
    auto issue = [&](int j, Stage& st) {
      const __amdgpu_buffer_rsrc_t rk = rsrc_at(kseg, j, D, row_bytes);
      const __amdgpu_buffer_rsrc_t rv = rsrc_at(vseg, j, D, row_bytes);
      // Each load takes part of a row (other loads of this wave take the rest), so the
      // lines must stay cached between them: no streaming hint here.
#pragma unroll
      for (int m = 0; m < kM; ++m)
        st.k[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, key_a * row_bytes + 32 * m + 16 * half, 0, 0);
#pragma unroll
      for (int it = 0; it < kVItems; ++it) {
        const int i = lane + kWave * it;
        const int kp = i & 15, dg = i >> 4;  // lanes of one key pair read consecutive 16-dim groups
        st.v[it][0] = __builtin_amdgcn_raw_buffer_load_b128(rv, 2 * kp * row_bytes + 16 * dg, 0, 0);
        st.v[it][1] = __builtin_amdgcn_raw_buffer_load_b128(rv, (2 * kp + 1) * row_bytes + 16 * dg, 0, 0);
      }
      const __amdgpu_buffer_rsrc_t rks = rsrc_at(ksseg, j, 4, 4);
      const __amdgpu_buffer_rsrc_t rvs = rsrc_at(vsseg, j, 4, 4);
      st.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, l32 * 4, 0, kCpolNT));
      st.vs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, l32 * 4, 0, kCpolNT));
    };
    auto process = [&](int j, Stage& st, int j_next) {
      // ---- V^T key pairs and the scales into the wave's LDS (the last tile's reads are done)
      wave_lds_fence();
#pragma unroll
      for (int it = 0; it < kVItems; ++it) {
        const int i = lane + kWave * it;
        const int kp = i & 15, dg = i >> 4;
#pragma unroll
        for (int dd = 0; dd < 16; ++dd) {
          const uint32_t wa = st.v[it][0][dd >> 2], wb = st.v[it][1][dd >> 2];
          const int sh = 8 * (dd & 3);
          *reinterpret_cast<uint32_t*>(vt + (16 * dg + dd) * kVStride + 4 * kp) =
              pack_bf16x2(static_cast<float>(static_cast<int8_t>(wa >> sh)),
                          static_cast<float>(static_cast<int8_t>(wb >> sh)));
        }
      }
      scl[lane] = half ? st.vs : st.ks;  // K scale of key l32, or V scale of key l32
      // ---- S^T = K Q^T, each K code run widened to its two A operands just before use
      f32x16_t s;
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const u32x4_t w = st.k[m];
        const u32x4_t a0 = {i8_pair_bf16(w.x, 0), i8_pair_bf16(w.x, 2), i8_pair_bf16(w.y, 0), i8_pair_bf16(w.y, 2)};
        const u32x4_t a1 = {i8_pair_bf16(w.z, 0), i8_pair_bf16(w.z, 2), i8_pair_bf16(w.w, 0), i8_pair_bf16(w.w, 2)};
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                    __builtin_bit_cast(bf16x8_t, qb[2 * m]),
                                                    m == 0 ? f32x16_t{} : s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                    __builtin_bit_cast(bf16x8_t, qb[2 * m + 1]), s, 0, 0, 0);
      }
      if (j_next >= 0) issue(j_next, st);  // the stage's codes are consumed: it takes tile j_next
      wave_lds_fence();  // V^T and the scales are visible to the whole wave
      // ---- softmax of head l32 over this lane's 16 keys: key(r) = 16 (r >> 3) + 8 half + (r & 7),
      // register r of the scores (scaled in place); scales read from LDS four at a time
      const int key0 = j * kTileKeys;
      float tm = -INFINITY;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 a = *reinterpret_cast<const float4*>(scl + 16 * (q4 >> 1) + 8 * half + 4 * (q4 & 1));
        const float kk[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * q4 + u;
          const int key = key0 + 16 * (r >> 3) + 8 * half + (r & 7);
          s[r] = key < L ? s[r] * (c * kk[u]) : -INFINITY;
          tm = fmaxf(tm, s[r]);
        }
      }
      tm = fmaxf(tm, __shfl_xor(tm, 32));  // the head's max over the tile (both halves)
      if (__ballot(tm > mh + kLazyLog2)) {
        const float m_new = fmaxf(mh, tm);  // finite: key key0 is always valid
        const float alpha = exp2f(mh - m_new);
        mh = m_new;
        lpart *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      u32x4_t pf[2];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const float4 b0 = *reinterpret_cast<const float4*>(scl + 32 + 16 * ks2 + 8 * half);
        const float4 b1 = *reinterpret_cast<const float4*>(scl + 32 + 16 * ks2 + 8 * half + 4);
        const float vv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * ks2 + 2 * i;
          const float p0 = exp2f(s[r] - mh), p1 = exp2f(s[r + 1] - mh);
          lpart += p0 + p1;
          w[i] = pack_bf16x2(p0 * vv[2 * i], p1 * vv[2 * i + 1]);
        }
        pf[ks2] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vt + (32 * db + l32) * kVStride + (8 * ks2 + 4 * half) * 4);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                          __builtin_bit_cast(bf16x8_t, pf[ks2]), o[db], 0, 0, 0);
        }
    };

    // The wave's tiles of this run: j0 + wave, j0 + wave + 4, ...; kQ8Stages tiles in flight.
    Stage st[kQ8Stages];
    int j = j0 + wave;
#pragma unroll
    for (int i = 0; i < kQ8Stages; ++i)
      if (j + i * kWaves < j1) issue(j + i * kWaves, st[i]);
    auto next = [&](int jj) { return jj < j1 ? jj : -1; };
    while (j < j1) {
#pragma unroll
      for (int i = 0; i < kQ8Stages; ++i) {
        if (j < j1) process(j, st[i], next(j + kQ8Stages * kWaves));
        j += kWaves;
      }
    }

    // ---- fold the four waves' states of this run (as decode_bf16_kernel, 32 heads)
    lpart += __shfl_xor(lpart, 32);
    __syncthreads();
    float* red_ml = reinterpret_cast<float*>(smem);   // [wave][GB][2]
    float* red_o = red_ml + kWaves * GB * 2;          // [wave][GB][D]
    if (half == 0) {
      red_ml[(wave * GB + l32) * 2] = mh;
      red_ml[(wave * GB + l32) * 2 + 1] = lpart;
    }
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(red_o + (wave * GB + l32) * D + 32 * db + 8 * r4 + 4 * half) =
            make_float4(o[db][4 * r4], o[db][4 * r4 + 1], o[db][4 * r4 + 2], o[db][4 * r4 + 3]);
    __syncthreads();
    const int slot = first_run ? 0 : 1;
    for (int e = threadIdx.x; e < group * D && e < GB * D; e += kWaves * kWave) {
      const int h = e / D;
      const int d = e - h * D;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, red_ml[(w * GB + h) * 2]);
      float ov = 0.f, l = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(red_ml[(w * GB + h) * 2] - mm);  // 0 for a wave with no tile here
        ov += f * red_o[(w * GB + h) * D + d];
        l += f * red_ml[(w * GB + h) * 2 + 1];
      }
      if (complete) {
        static_cast<bf16_t*>(p.out)[(size_t(row_token(p.kv, seg.b)) * hq + g * group + h) * D + d] =
            f32_to_bf16(ov / l);
      } else {
        const size_t ps = (size_t(blockIdx.x) * 2 + slot) * GB + h;
        p.ws_o[ps * D + d] = ov;
        if (d == 0) {
          p.ws_ml[ps * 2] = mm;
          p.ws_ml[ps * 2 + 1] = l;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next run

    first_run = false;
    t = run_end;
    if (t < t_end) {
      seg.base = seg_end;
      if (++seg.sr == spr) {
        seg.sr = 0;
        do {
          ++seg.b;
          seg.nt = row_tiles(p.kv, seg.b);
        } while (seg.nt == 0);
      }
    }
  }
}

// Fold the partials of one (segment, query head): one workgroup each.
template <int D, int GB>
__global__ __launch_bounds__(256) void decode_bf16_combine_kernel(DecodeParams p) {
  constexpr int kChunks = D / 4;          // 16-byte chunks of an o row
  constexpr int kPI = 256 / kChunks;      // partials processed side by side
  __shared__ float red[kPI][D];
  __shared__ float red_l[kPI];
  __shared__ float red_m[4];

  const int spr = p.kv.n_kv_heads * p.n_hb;
  const int h = blockIdx.x % GB;
  const int seg = blockIdx.x / GB;
  const int b = seg / spr;
  const int sr = seg - b * spr;
  const int g = sr / p.n_hb;
  const int hb = sr - g * p.n_hb;
  const int hq = p.n_q_heads;
  const int group = hq / p.kv.n_kv_heads;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;

  const int nt = row_tiles(p.kv, b);
  if (nt == 0) {
    if (sr == 0 && h == 0 && threadIdx.x == 0) {
      const int why = row_keys(p.kv, b);
      if (why == -1) report(p.dev_err, KVC_DEV_CAPACITY);
      if (why == -3) report(p.dev_err, KVC_DEV_TOKENS);
    }
    return;
  }
  if (hb * GB + h >= group) return;  // padding head of the last block
  // N and this segment's first tile
  int n_all = 0, before = 0;
  for (int b0 = 0; b0 < p.kv.batch; b0 += kWave) {
    const int bb = b0 + lane;
    const int v = bb < p.kv.batch ? row_tiles(p.kv, bb) : 0;
    n_all += wave_sum_i(v);
    before += wave_sum_i(bb < b ? v : 0);
  }
  const int n_tiles = n_all * spr;
  const int base = before * spr + sr * nt;
  // workgroup holding tile t: the largest w with w N / P <= t
  auto wg_of = [&](int t) { return int(((long long)(t + 1) * p.n_wg - 1) / n_tiles); };
  const int w_first = wg_of(base);
  const int w_last = wg_of(base + nt - 1);
  if (w_first == w_last) return;  // written directly by the split pass
  // Partials: w_first's run here (its first run -- slot 0 -- if its range starts at this
  // segment, else its last -- slot 1), then the first run (slot 0) of every later
  // workgroup up to w_last.  Workgroups with an empty range (fewer tiles than
  // workgroups) wrote nothing and are skipped.
  const int count = w_last - w_first + 1;
  const int slot0 = range_begin(w_first, n_tiles, p.n_wg) == base ? 0 : 1;
  auto part = [&](int i) { return (size_t(w_first + i) * 2 + (i == 0 ? slot0 : 0)) * GB + h; };
  // With at least as many tiles as workgroups every workgroup holds a tile, so none of
  // w_first..w_last is empty and the check (two 64-bit divisions per partial) is skipped.
  const bool may_be_empty = n_tiles < p.n_wg;
  auto empty = [&](int i) {
    return may_be_empty &&
           range_begin(w_first + i, n_tiles, p.n_wg) == range_begin(w_first + i + 1LL, n_tiles, p.n_wg);
  };

  // This thread folds partials pi, pi + kPI, ... (16 bytes of each o row).  Their
  // loads are issued kCh at a time before any is used -- the first kCh before
  // the maximum pass, so both passes wait for memory once -- because a loop
  // that loads and uses one partial per iteration waits for every load in
  // turn.  A slot past the last partial is read at the last one's index and
  // not used.
  const int ck = threadIdx.x % kChunks;
  const int pi = threadIdx.x / kChunks;
  constexpr int kCh = 8;
  float4 ov[kCh];
  float mv[kCh], lv[kCh];
  auto fetch = [&](int i0) {
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const size_t ps = part(min(i0 + kPI * c, count - 1));
      mv[c] = p.ws_ml[ps * 2];
      lv[c] = p.ws_ml[ps * 2 + 1];
      ov[c] = *reinterpret_cast<const float4*>(p.ws_o + ps * D + 4 * ck);
    }
  };
  fetch(pi);

  float mx = -INFINITY;
  for (int i = threadIdx.x; i < count; i += blockDim.x)
    if (!empty(i)) mx = fmaxf(mx, p.ws_ml[part(i) * 2]);
  mx = wave_max(mx);
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  for (int i0 = pi; i0 < count; i0 += kCh * kPI) {
    if (i0 != pi) fetch(i0);
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int i = i0 + kPI * c;
      if (i >= count || empty(i)) continue;
      const float f = exp2f(mv[c] - M);
      a.x += f * ov[c].x; a.y += f * ov[c].y; a.z += f * ov[c].z; a.w += f * ov[c].w;
      den += f * lv[c];
    }
  }
  *reinterpret_cast<float4*>(&red[pi][4 * ck]) = a;
  if (ck == 0) red_l[pi] = den;
  __syncthreads();
  if (threadIdx.x < D) {
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int k = 0; k < kPI; ++k) {
      o += red[k][threadIdx.x];
      l += red_l[k];
    }
    static_cast<bf16_t*>(p.out)[(size_t(row_token(p.kv, b)) * hq + g * group + hb * GB + h) * D + threadIdx.x] =
        f32_to_bf16(o / l);
  }
}

template <int D, int GB>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  if (p.kv.dtype == KVC_I8)
    hipLaunchKernelGGL((decode_bf16_kernel<D, GB, true>), dim3(p.n_wg), dim3(kWaves * kWave), 0, s, p);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<D, GB, false>), dim3(p.n_wg), dim3(kWaves * kWave), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n_comb = (long long)p.kv.batch * p.kv.n_kv_heads * p.n_hb * GB;
  hipLaunchKernelGGL((decode_bf16_combine_kernel<D, GB>), dim3(unsigned(n_comb)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_q8(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_q8_mfma_kernel<D>), dim3(p.n_wg), dim3(kWaves * kWave), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n_comb = (long long)p.kv.batch * p.kv.n_kv_heads * kQ8Cols;
  hipLaunchKernelGGL((decode_bf16_combine_kernel<D, kQ8Cols>), dim3(unsigned(n_comb)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int decode_bf16_block(int dtype, int group) {
  if (dtype == KVC_I8 && group <= kQ8Cols) return kQ8Cols;  // the matrix-core int8 kernel: one block per KV head
  return group <= 4 ? 4 : 8;
}

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t s) {
  if (p.gb == kQ8Cols) return p.kv.head_dim == 128 ? launch_q8<128>(p, s) : launch_q8<64>(p, s);
  if (p.kv.head_dim == 128) return p.gb == 4 ? launch_t<128, 4>(p, s) : launch_t<128, 8>(p, s);
  return p.gb == 4 ? launch_t<64, 4>(p, s) : launch_t<64, 8>(p, s);
}

}  // namespace kvc
