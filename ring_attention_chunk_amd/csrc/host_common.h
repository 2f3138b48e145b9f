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

// Stream-ordered writer of a descriptor table into device memory at `dst`.
// Appended bytes gather in a fixed 2 KB window that reaches the device as the
// kernel arguments of a small copy kernel; the runtime captures arguments when
// a launch is enqueued, so the caller's host arrays are read only during the
// call, and neither host nor device memory is allocated. Every append and
// padding is a whole number of 4-byte words.
constexpr int kUploadWords = 512;
struct UploadWindow {
  uint32_t w[kUploadWords];
};

class TableUpload {
 public:
  TableUpload(void* dst, hipStream_t s) : dst_((char*)dst), s_(s) {}
  void put(const void* p, size_t n);
  // zero bytes until the table is `total` bytes long
  void zero_to(size_t total);
  size_t size() const { return base_ + fill_; }
  // uploads the last window; returns the first launch error, if any
  hipError_t finish();

 private:
  void flush();
  char* dst_;
  hipStream_t s_;
  size_t base_ = 0;  // bytes already sent
  size_t fill_ = 0;  // bytes in the window
  hipError_t err_ = hipSuccess;
  UploadWindow win_;
};

}  // namespace ra_host

#endif  // RA_HOST_COMMON_H
