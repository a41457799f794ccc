// Measured ceilings of one MI355X: what a plain streaming read and a plain
// matrix-core loop reach on this chip, so that the attention kernels'
// bandwidth and TFLOP/s can be stated against measured limits as well as the
// published ones (8 TB/s HBM3E, 2.5 PFLOP/s dense bfloat16).
//
// This library is measurement infrastructure, separate from libkvc: it holds
// no part of the attention method.  Both calls are asynchronous on `stream`,
// allocate nothing and return 0 or a negative code (-1: bad argument, before
// any launch; -2: launch failure).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

// Reads `rows` rows of `row_bytes` bytes, row r starting at buf + r * stride_bytes,
// with 16-byte vector loads, 16 lanes per 256 bytes, and folds every word into an
// XOR that is written to *sink only if it equals a value no test data produces
// (so the loads cannot be removed).  row_bytes is a positive multiple of 256 and
// at most stride_bytes; buf is 16-byte aligned and holds rows * stride_bytes bytes
// (device memory, owned by the caller).  `nontemporal` != 0 puts the
// non-temporal hint on every load.  `workgroups` persistent workgroups of 256
// threads share the rows evenly.
int kvc_ceiling_stream_read(const void* buf, int64_t rows, int32_t row_bytes, int64_t stride_bytes,
                            int32_t nontemporal, int32_t workgroups, uint32_t* sink, hipStream_t stream);

// Reads K and V laid out (rows, n_keys, heads, 256 bytes), each a contiguous,
// 16-byte aligned device buffer of rows * n_keys * heads * 256 bytes owned by the
// caller, in the decode kernel's assignment: rows * heads * parts workgroups of
// 256 threads, workgroup w streaming keys [p n_keys / parts, (p + 1) n_keys / parts)
// of segment (row, head) = divmod(w / parts, heads), p = w % parts, with
// non-temporal 16-byte loads and no arithmetic but an XOR written to *sink only
// for an impossible value.  Bytes read per call = 2 * rows * n_keys * heads * 256.
int kvc_ceiling_decode_read(const void* k, const void* v, int32_t rows, int32_t n_keys, int32_t heads,
                            int32_t parts, uint32_t* sink, hipStream_t stream);

// Every wave of `workgroups` workgroups of 256 threads runs `iters` rounds of
// 8 x `chains` (chains 2 or 4) v_mfma_f32_32x32x16_bf16 products (32768 flops
// each), cycling through 8 A and 8 B operand registers; *sink is written only
// for an impossible result.  random_operands == 0: every operand register holds
// one small constant pattern.  random_operands != 0: A uniform in [-2, 2) and B
// uniform in [0, 1), different per register and lane, as attention's scores and
// weights are; the matrix cores then draw more power and the clock they hold
// can be lower.  Flops per call = workgroups * 4 waves * iters * 8 * chains * 32768.
int kvc_ceiling_mfma_bf16(int32_t iters, int32_t chains, int32_t random_operands, int32_t workgroups, float* sink,
                          hipStream_t stream);

// Every wave of `workgroups` workgroups of 512 threads (8 waves) reads, `iters`
// times, a 16 KB tile from LDS in the prefill kernel's MFMA-operand pattern: 16
// ds_read_b128 per lane, rows of 256 data bytes padded to 272.  *sink is written
// only for an impossible XOR.  Bytes read per call = workgroups * 8 * iters * 16384.
int kvc_ceiling_lds_read(int32_t iters, int32_t workgroups, uint32_t* sink, hipStream_t stream);

// Reads an int8 KV cache -- codes (rows, max_seq, heads, 128 bytes) for K and for V, and
// float32 scales (rows, heads, max_seq) for each, all caller-owned device memory, the code
// buffers 16-byte aligned -- over keys [0, n_keys) of every row, with whole 128-byte rows
// loaded straight into LDS (buffer_load_dwordx4 ... lds) one 32-key tile per wave at a time
// and no arithmetic but an XOR written to *sink only for an impossible value.  mode 0: the
// decode kernel's assignment, rows * heads * parts workgroups, each one key range of one
// (row, head).  mode 1: all heads of a key range, rows * parts workgroups, wave h reading
// heads 2h and 2h + 1 (heads <= 8).  Bytes read per call = 2 * rows * n_keys * heads * (128 + 4).
int kvc_ceiling_q8_read(const void* k, const void* v, const float* k_scale, const float* v_scale, int32_t rows,
                        int32_t n_keys, int32_t max_seq, int32_t heads, int32_t mode, int32_t parts, uint32_t* sink,
                        hipStream_t stream);

// Writes `rows` runs of `run_bytes` (a multiple of 16) into the 16-byte aligned device
// buffer, run r starting at r * stride_bytes (a multiple of 16, at least run_bytes when
// rows > 1), the buffer holding (rows - 1) * stride_bytes + run_bytes bytes.  Thread i
// stores 16-byte vector i of every run (the prefill clone's write pattern without its
// read); with rows = 1, a contiguous streaming write.  Bytes written per call =
// rows * run_bytes.
int kvc_ceiling_stream_write(void* buf, int64_t run_bytes, int32_t rows, int64_t stride_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
