// host_common.h -- host-side helpers shared by the forward and backward entry
// points of the library (internal; not part of the C ABI).
#ifndef RA_HOST_COMMON_H
#define RA_HOST_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ring_attention_chunk.h"

namespace ra_host {

// Largest global position a chunk or query segment may describe.
constexpr int64_t kPosLimit = 0x7ffffffeLL;

// Message of the last failed call on this host thread (ra_last_error).
extern thread_local char g_err[512];

// Records the message and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char* what);

int check_dims(int dtype, int batch, int q_heads, int kv_heads, int head_dim);
int check_chunk(const ra_kv_chunk& c, int idx, int head_dim);

// Position step of a chunk or query segment: 0 stands for 1 (contiguous).
int64_t pos_step(int64_t s);
// True when offset + step * [0, len) lies in [0, kPosLimit] (len >= 1, step >= 1).
bool positions_fit(int64_t offset, int64_t len, int64_t step);

// 16-byte loads allowed for rows of `head_dim` elements at stride `stride`.
bool vec_ok(const void* p, int64_t stride, int head_dim, int64_t elem);
bool chunk_vec_ok(const ra_kv_chunk& c, int head_dim, int64_t elem);

// Kernel timer hooks (ra_kernel_timer): an event pair around one kernel launch.
void timer_begin(hipStream_t s);
void timer_end(hipStream_t s);

// Stream-ordered copy of `bytes` (a multiple of 4) of host memory to device
// memory at `dst`, carried as kernel arguments of small copy kernels: the
// runtime captures arguments when a launch is enqueued, so the host bytes need
// to stay valid only for this call, and no host-to-device copy engine or
// staging buffer is involved. Meant for descriptor tables of a few KB.
hipError_t upload_table(void* dst, const void* src, size_t bytes, hipStream_t s);

}  // namespace ra_host

#endif  // RA_HOST_COMMON_H
