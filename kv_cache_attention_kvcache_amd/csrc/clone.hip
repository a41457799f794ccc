// Batch-1 -> batch-N prefill clone (nanochat post, "The prefill trick, 12 lines").
//
// For every layer, positions [0, src_len) of the single source row are one
// contiguous run of src_len * n_kv_heads * head_dim elements, and so is the
// same run of each destination row.  The copy kernel reads each 16-byte
// vector of the source run once and writes it to every empty destination
// row (read once, write N times: HBM-bound).  Its grid has one thread per
// source vector (no grid-stride loop unless the grid would pass 2^31
// workgroups), so the workgroups in flight at any moment cover a narrow,
// advancing stretch of each row: the writes sweep every row in address
// order.  A persistent grid whose threads stride over the whole run spread
// the writes over the full 2.4 GB at once and wrote 10% slower (measured on
// MI355X: 552 against about 500 us for 8 rows of a 73,728-token cache).
// A second, one-workgroup kernel then sets the destination lengths, so no
// block reads a length another block may already have changed.  An int8 cache also has one float32 scale
// per (KV head, position) for K and for V, head-major: per layer, each KV
// head's positions [0, src_len) are one run, copied the same way (grid planes
// 2 and 3), 4 bytes at a time.
#include "kvc_device.h"
#include "kvc_launch.h"
#include "kvc.h"

namespace kvc {

namespace {

__device__ __forceinline__ size_t elem_bytes(int dtype) { return dtype == KVC_F32 ? 4 : dtype == KVC_BF16 ? 2 : 1; }

__global__ __launch_bounds__(256) void clone_copy_kernel(CloneParams p) {
  if (p.src.seqlens[0] != p.src_len) return;  // reported by clone_lengths_kernel
  const int layer = blockIdx.y;
  const int n_rows = p.dst.batch;
  if (blockIdx.z >= 2) {  // scales of an int8 cache
    const int hkv = p.src.n_kv_heads;
    const size_t n = size_t(p.src_len) * hkv;
    const float* src = (blockIdx.z == 2 ? p.src.k_scale : p.src.v_scale) + size_t(layer) * hkv * p.src.max_seq;
    float* dst0 = blockIdx.z == 2 ? p.dst.k_scale : p.dst.v_scale;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x) {
      const size_t h = i / p.src_len, pos = i - h * p.src_len;
      const float val = src[h * p.src.max_seq + pos];
      for (int r = 0; r < n_rows; ++r)
        if (p.dst.seqlens[r] == 0) dst0[((size_t(layer) * n_rows + r) * hkv + h) * p.dst.max_seq + pos] = val;
    }
    return;
  }
  const bool is_v = blockIdx.z != 0;
  const size_t esz = elem_bytes(p.src.dtype);
  const size_t tok_bytes = size_t(p.src.n_kv_heads) * p.src.head_dim * esz;
  const size_t n_vec = size_t(p.src_len) * tok_bytes / 16;
  const uint8_t* src = static_cast<const uint8_t*>(is_v ? p.src.v : p.src.k) +
                       size_t(layer) * p.src.max_seq * tok_bytes;  // source batch is 1
  uint8_t* dst0 = static_cast<uint8_t*>(is_v ? p.dst.v : p.dst.k);
  const size_t dst_row_bytes = size_t(p.dst.max_seq) * tok_bytes;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_vec; i += size_t(gridDim.x) * blockDim.x) {
    const uint4 val = reinterpret_cast<const uint4*>(src)[i];
    for (int r = 0; r < n_rows; ++r) {
      if (p.dst.seqlens[r] != 0) continue;  // not empty: skipped, reported below
      uint8_t* dst = dst0 + (size_t(layer) * n_rows + r) * dst_row_bytes;
      reinterpret_cast<uint4*>(dst)[i] = val;
    }
  }
}

__global__ __launch_bounds__(256) void clone_lengths_kernel(CloneParams p) {
  const bool src_ok = p.src.seqlens[0] == p.src_len;
  if (!src_ok) {
    if (threadIdx.x == 0) report(p.dev_err, KVC_DEV_SRC_LEN);
    return;
  }
  for (int r = threadIdx.x; r < p.dst.batch; r += blockDim.x) {
    if (p.dst_seqlens[r] == 0) p.dst_seqlens[r] = p.src_len;
    else report(p.dev_err, KVC_DEV_NOT_EMPTY);
  }
}

}  // namespace

hipError_t launch_clone(const CloneParams& p, hipStream_t s) {
  const size_t esz = p.src.dtype == KVC_F32 ? 4 : p.src.dtype == KVC_BF16 ? 2 : 1;
  const size_t n_vec = size_t(p.src_len) * p.src.n_kv_heads * p.src.head_dim * esz / 16;
  if (n_vec > 0) {
    const size_t want = (n_vec + 255) / 256;  // one thread per source vector
    const unsigned gx = unsigned(want < 0x7fffffffu ? want : 0x7fffffffu);
    const unsigned planes = p.src.dtype == KVC_I8 ? 4 : 2;  // K, V (and their scales)
    hipLaunchKernelGGL(clone_copy_kernel, dim3(gx, p.n_layers, planes), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(clone_lengths_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
