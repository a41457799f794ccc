// Streaming-read and matrix-core ceiling kernels (declared in ceilings.h).
#include "ceilings.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kLoadsInFlight = 8;  // 16-byte loads per lane issued before any is consumed
constexpr uint32_t kNeverXor = 0x9e3779b9u;

// A "piece" is 256 bytes of one row: 16 lanes x 16 bytes.  Wave w of W takes
// pieces [w P / W, (w + 1) P / W) of the P = rows * row_bytes / 256 pieces; its
// four 16-lane groups take consecutive pieces.
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint8_t* __restrict__ buf, int64_t rows,
                                                              int32_t pieces_per_row, int64_t stride,
                                                              uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t n_waves = int64_t(gridDim.x) * (kThreads / 64);
  const int64_t wave = int64_t(blockIdx.x) * (kThreads / 64) + threadIdx.x / 64;
  const int64_t pieces = rows * pieces_per_row;
  const int64_t p0 = wave * pieces / n_waves, p1 = (wave + 1) * pieces / n_waves;
  uint32_t acc = 0;
  for (int64_t base = p0; base < p1; base += 4 * kLoadsInFlight) {
    u32x4 v[kLoadsInFlight];
#pragma unroll
    for (int k = 0; k < kLoadsInFlight; ++k) {
      const int64_t pc = base + 4 * k + lane / 16;
      if (pc < p1) {
        const int64_t r = pc / pieces_per_row, c = pc - r * pieces_per_row;
        const u32x4* src = reinterpret_cast<const u32x4*>(buf + r * stride + c * 256 + (lane & 15) * 16);
        v[k] = NT ? __builtin_nontemporal_load(src) : *src;
      } else {
        v[k] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < kLoadsInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == kNeverXor) sink[0] = acc;
}

// Decode's own read assignment: K and V are (rows, keys, heads, 256 bytes).  The
// (row, head) segments are cut into `parts` contiguous key ranges, one per
// workgroup (workgroup w: segment w / parts, part w % parts), as the decode
// kernel deals its tiles.  The four waves take 32-key tiles of the range in turn;
// a lane reads 16 bytes of four key rows per tile step, from K and from V, all
// sixteen loads issued before any is consumed.
__global__ __launch_bounds__(kThreads) void decode_read_kernel(const uint8_t* __restrict__ k,
                                                              const uint8_t* __restrict__ v, int32_t n_keys,
                                                              int32_t heads, int32_t parts, uint32_t* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
  const int seg = blockIdx.x / parts, part = blockIdx.x % parts;
  const int row = seg / heads, head = seg % heads;
  const int k0 = int(int64_t(part) * n_keys / parts), k1 = int(int64_t(part + 1) * n_keys / parts);
  const int64_t key_stride = int64_t(heads) * 256;
  const int64_t base = (int64_t(row) * n_keys * heads + head) * 256 + (lane & 15) * 16;
  uint32_t acc = 0;
  for (int t = k0 + wave * 32; t < k1; t += 4 * 32) {
    if (t + 32 <= k1) {
      u32x4 a[kLoadsInFlight], b[kLoadsInFlight];
#pragma unroll
      for (int i = 0; i < kLoadsInFlight; ++i) {
        const int64_t off = base + int64_t(t + 4 * i + lane / 16) * key_stride;
        a[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
        b[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
      }
#pragma unroll
      for (int i = 0; i < kLoadsInFlight; ++i) acc ^= a[i].x ^ a[i].y ^ a[i].z ^ a[i].w ^ b[i].x ^ b[i].y ^ b[i].z ^ b[i].w;
    } else {
      for (int i = 0; i < kLoadsInFlight; ++i) {
        const int key = t + 4 * i + lane / 16;
        if (key < k1) {
          const int64_t off = base + int64_t(key) * key_stride;
          const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
          const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
          acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
        }
      }
    }
  }
  if (acc == kNeverXor) sink[0] = acc;
}

// 32-bit integer hash (multiply-xorshift) for the random operands.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// Each wave cycles its products through 8 A and 8 B operand registers.  Constant
// operands: every register holds the same small pattern, so the matrix cores'
// inputs hardly change between products.  Random operands: A uniform in
// [-2, 2) and B uniform in [0, 1) (the range of softmax weights), different in
// every register and lane, so consecutive products see fresh data as in
// attention.
template <int CH, bool RANDOM>
__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(int32_t iters, float* sink) {
  bf16x8 a[8], b[8];
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (RANDOM) {
        const float ua = float(mix32(t * 131u + j * 8 + i) >> 8) * (1.f / 16777216.f);
        const float ub = float(mix32(t * 977u + j * 8 + i + 0x5555u) >> 8) * (1.f / 16777216.f);
        a[j][i] = static_cast<__bf16>(ua * 4.f - 2.f);
        b[j][i] = static_cast<__bf16>(ub);
      } else {
        a[j][i] = static_cast<__bf16>(float(threadIdx.x & 7) * 0.125f);
        b[j][i] = static_cast<__bf16>(float(i) * -0.25f);
      }
    }
  f32x16 c[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) c[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < CH; ++k)
        c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + u) & 7], b[(3 * k + u) & 7], c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) s += c[k][0] + c[k][15];
  if (s == 1.2345e30f) sink[0] = s;
}

// LDS reads in the prefill kernel's pattern: each of a workgroup's 8 waves reads
// a 64-row tile of 272-byte rows (256 bytes of data + 16 of padding) as 16
// MFMA A fragments (lane (l32, half) reads 16 bytes at row perm(l32) + 32 kb,
// byte 16 half + 32 kd), every iteration, and folds them into an XOR.
constexpr int kLdsThreads = 512;
constexpr int kLdsRow = 272;

__global__ __launch_bounds__(kLdsThreads) void lds_read_kernel(int32_t iters, uint32_t* sink) {
  __shared__ __align__(16) uint8_t tile[64 * kLdsRow];
  const int tid = threadIdx.x, half = (tid & 63) >> 5, l32 = tid & 31;
  for (int i = tid; i < 64 * kLdsRow / 16; i += kLdsThreads)
    reinterpret_cast<u32x4*>(tile)[i] = u32x4{uint32_t(i), uint32_t(i) * 3u, uint32_t(i) * 5u, uint32_t(i) * 7u};
  __syncthreads();
  const int row = ((l32 >> 4) << 4) | (((l32 >> 2) & 1) << 3) | (((l32 >> 3) & 1) << 2) | (l32 & 3);
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");  // the tile is read again every iteration
    u32x4 f[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kd = 0; kd < 8; ++kd)
        f[kb * 8 + kd] = *reinterpret_cast<const u32x4*>(tile + (32 * kb + row) * kLdsRow + 16 * half + 32 * kd);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += f[i].x ^ f[i].y ^ f[i].z ^ f[i].w;
  }
  if (acc == kNeverXor) sink[0] = acc;
}

// Reads of an int8 cache: codes (rows, max_seq, heads, 128 bytes) for K and for V, and
// float32 scales (rows, heads, max_seq) for each, of keys [0, n_keys) of every row.
// Whole 128-byte rows are loaded straight into per-wave LDS (buffer_load_dwordx4 ... lds,
// eight lanes per row), one 32-key tile at a time per wave; the buffers' range checks
// return zeros past a row's keys.  The data are folded into an XOR written to *sink only
// for an impossible value, so nothing can be removed.  Each wave waits for its own loads
// (vmcnt) before it touches its stage.
constexpr int kQ8Tile = 32;
constexpr int kQ8Stage = 8 * 1024 + 512;  // K codes, V codes, K scales, V scales of one tile
typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ void q8_wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// One tile of one head: 32 key rows of 128 bytes at a `row_bytes` stride from k_head/v_head,
// and the head's 32 scales, into `stage`.
__device__ __forceinline__ void q8_issue(uint8_t* stage, const uint8_t* k_head, const uint8_t* v_head,
                                         const float* ks_head, const float* vs_head, int key0, int n_keys,
                                         int row_bytes, int lane) {
  const int left = (n_keys - key0 - 1) * row_bytes + 128;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(k_head) + size_t(key0) * row_bytes, (short)0, left > 0 ? left : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(v_head) + size_t(key0) * row_bytes, (short)0, left > 0 ? left : 0, 0x00020000);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int off = (8 * n + lane / 8) * row_bytes + 16 * (lane % 8);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(stage + 1024 * n), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(stage + 4096 + 1024 * n), 16, off, 0, 0, 0);
  }
  const int sleft = (n_keys - key0) * 4;  // lanes 32..63 read past the tile's scales: zeros or the next keys'
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ks_head) + key0, (short)0,
                                                                      sleft > 0 ? sleft : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(vs_head) + key0, (short)0,
                                                                      sleft > 0 ? sleft : 0, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(stage + 8192), 4, 4 * lane, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_ptr)(stage + 8192 + 256), 4, 4 * lane, 0, 0, 0);
}

__device__ __forceinline__ uint32_t q8_use(const uint8_t* stage, int lane) {
  q8_wait_all();
  const uint32_t a = *reinterpret_cast<const uint32_t*>(stage + 16 * lane) ^
                     *reinterpret_cast<const uint32_t*>(stage + 4096 + 16 * lane) ^
                     *reinterpret_cast<const uint32_t*>(stage + 8192 + 4 * lane);
  __builtin_amdgcn_s_waitcnt(0);  // the stage's reads are done before the next loads land in it
  return a;
}

// mode 0, the decode kernel's assignment: workgroup w streams key range w % parts of segment
// (row, head) = divmod(w / parts, heads); its four waves take the range's tiles in turn.
// mode 1, all heads of a key range: workgroup w streams key range w % parts of row w / parts,
// wave h taking heads 2h and 2h + 1 of every tile, so the four waves read whole key rows.
__global__ __launch_bounds__(kThreads) void q8_read_kernel(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                          const float* __restrict__ ks, const float* __restrict__ vs,
                                                          int32_t n_keys, int32_t max_seq, int32_t heads, int32_t mode,
                                                          int32_t parts, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t stages[4][kQ8Stage];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int row_bytes = heads * 128;
  const int nt = (n_keys + kQ8Tile - 1) / kQ8Tile;
  uint8_t* stage = stages[wave];
  uint32_t acc = 0;
  if (mode == 0) {
    const int seg = blockIdx.x / parts, part = blockIdx.x % parts;
    const int row = seg / heads, head = seg % heads;
    const int j0 = int(int64_t(part) * nt / parts), j1 = int(int64_t(part + 1) * nt / parts);
    const uint8_t* kh = k + size_t(row) * max_seq * row_bytes + head * 128;
    const uint8_t* vh = v + size_t(row) * max_seq * row_bytes + head * 128;
    const float* ksh = ks + (size_t(row) * heads + head) * max_seq;
    const float* vsh = vs + (size_t(row) * heads + head) * max_seq;
    for (int j = j0 + wave; j < j1; j += 4) {
      q8_issue(stage, kh, vh, ksh, vsh, j * kQ8Tile, n_keys, row_bytes, lane);
      acc ^= q8_use(stage, lane);
    }
  } else {
    const int row = blockIdx.x / parts, part = blockIdx.x % parts;
    const int j0 = int(int64_t(part) * nt / parts), j1 = int(int64_t(part + 1) * nt / parts);
    for (int j = j0; j < j1; ++j)
      for (int h = 2 * wave; h < 2 * wave + 2 && h < heads; ++h) {
        const uint8_t* kh = k + size_t(row) * max_seq * row_bytes + h * 128;
        const uint8_t* vh = v + size_t(row) * max_seq * row_bytes + h * 128;
        q8_issue(stage, kh, vh, ks + (size_t(row) * heads + h) * max_seq, vs + (size_t(row) * heads + h) * max_seq,
                 j * kQ8Tile, n_keys, row_bytes, lane);
        acc ^= q8_use(stage, lane);
      }
  }
  if (acc == kNeverXor) sink[0] = acc;
}

// Writes `rows` runs of n16 16-byte vectors, run r starting r * stride16 vectors into buf.
// Thread i writes vector i of every run in turn (no loop over i): consecutive workgroups
// cover consecutive 4 KB of each run, so the stores in flight sweep every run in address
// order -- with one run, a contiguous streaming write.
__global__ __launch_bounds__(kThreads) void stream_write_kernel(uint8_t* __restrict__ buf, int64_t n16, int32_t rows,
                                                                int64_t stride16) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n16) return;
  for (int r = 0; r < rows; ++r)
    reinterpret_cast<u32x4*>(buf)[r * stride16 + i] = u32x4{uint32_t(i), uint32_t(r), 2u, 3u};
}

}  // namespace

extern "C" int kvc_ceiling_stream_read(const void* buf, int64_t rows, int32_t row_bytes, int64_t stride_bytes,
                                       int32_t nontemporal, int32_t workgroups, uint32_t* sink,
                                       hipStream_t stream) {
  if (!buf || !sink || rows < 1 || row_bytes < 256 || row_bytes % 256 != 0 || stride_bytes < row_bytes ||
      stride_bytes % 16 != 0 || workgroups < 1 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return -1;
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(workgroups), dim3(kThreads), 0, stream, p, rows,
                       row_bytes / 256, stride_bytes, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(workgroups), dim3(kThreads), 0, stream, p, rows,
                       row_bytes / 256, stride_bytes, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int kvc_ceiling_mfma_bf16(int32_t iters, int32_t chains, int32_t random_operands, int32_t workgroups,
                                     float* sink, hipStream_t stream) {
  if (!sink || iters < 1 || workgroups < 1 || (chains != 2 && chains != 4)) return -1;
  const dim3 grid(workgroups), block(kThreads);
  if (random_operands) {
    if (chains == 2) hipLaunchKernelGGL((mfma_bf16_kernel<2, true>), grid, block, 0, stream, iters, sink);
    else hipLaunchKernelGGL((mfma_bf16_kernel<4, true>), grid, block, 0, stream, iters, sink);
  } else {
    if (chains == 2) hipLaunchKernelGGL((mfma_bf16_kernel<2, false>), grid, block, 0, stream, iters, sink);
    else hipLaunchKernelGGL((mfma_bf16_kernel<4, false>), grid, block, 0, stream, iters, sink);
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int kvc_ceiling_lds_read(int32_t iters, int32_t workgroups, uint32_t* sink, hipStream_t stream) {
  if (!sink || iters < 1 || workgroups < 1) return -1;
  hipLaunchKernelGGL(lds_read_kernel, dim3(workgroups), dim3(kLdsThreads), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int kvc_ceiling_decode_read(const void* k, const void* v, int32_t rows, int32_t n_keys, int32_t heads,
                                       int32_t parts, uint32_t* sink, hipStream_t stream) {
  if (!k || !v || !sink || rows < 1 || n_keys < 1 || heads < 1 || parts < 1 ||
      (reinterpret_cast<uintptr_t>(k) & 15) != 0 || (reinterpret_cast<uintptr_t>(v) & 15) != 0)
    return -1;
  const int64_t n_wg = int64_t(rows) * heads * parts;
  if (n_wg > 0x7fffffffLL || int64_t(n_keys) * parts > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL(decode_read_kernel, dim3(unsigned(n_wg)), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), n_keys, heads, parts, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int kvc_ceiling_q8_read(const void* k, const void* v, const float* k_scale, const float* v_scale,
                                   int32_t rows, int32_t n_keys, int32_t max_seq, int32_t heads, int32_t mode,
                                   int32_t parts, uint32_t* sink, hipStream_t stream) {
  if (!k || !v || !k_scale || !v_scale || !sink || rows < 1 || n_keys < 1 || max_seq < n_keys || heads < 1 ||
      heads > 8 || parts < 1 || (mode != 0 && mode != 1) || (reinterpret_cast<uintptr_t>(k) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(v) & 15) != 0)
    return -1;
  const int64_t n_wg = int64_t(rows) * (mode == 0 ? heads : 1) * parts;
  if (n_wg > 0x7fffffffLL || int64_t(max_seq) * heads * 128 >= (int64_t(1) << 31)) return -1;
  hipLaunchKernelGGL(q8_read_kernel, dim3(unsigned(n_wg)), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), k_scale, v_scale, n_keys, max_seq,
                     heads, mode, parts, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int kvc_ceiling_stream_write(void* buf, int64_t run_bytes, int32_t rows, int64_t stride_bytes,
                                        hipStream_t stream) {
  if (!buf || run_bytes < 16 || run_bytes % 16 != 0 || rows < 1 || stride_bytes % 16 != 0 ||
      (rows > 1 && stride_bytes < run_bytes) || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return -1;
  const int64_t n16 = run_bytes / 16, wg = (n16 + kThreads - 1) / kThreads;
  if (wg > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL(stream_write_kernel, dim3(unsigned(wg)), dim3(kThreads), 0, stream, static_cast<uint8_t*>(buf),
                     n16, rows, stride_bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
