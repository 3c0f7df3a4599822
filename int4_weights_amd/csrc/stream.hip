// stream.hip -- moe_stream_read: a plain streaming read of device memory, the
// measured counterpart of the HBM peak that the memory-bound kernels of the
// path are compared with.  It is not a step of the method.
//
// Each lane keeps eight 16-byte nontemporal loads in flight over a grid-stride
// walk of the buffer, one 256-lane workgroup per CU: 32 KB in flight per CU.
// Of 4, 8 or 16 loads per lane, 256 to 1024 lanes and 1 to 8 workgroups per
// CU, grid-stride or one contiguous slice per workgroup, this was the fastest
// for an 8 GiB read (7.3-7.4 TB/s on one MI355X; 4 loads per lane with two
// workgroups per CU, the same bytes in flight, 6.8).  The loaded words are
// XOR-folded and the fold is written once per workgroup so that no load can
// be dropped.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kStreamU = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const v4i* __restrict__ x, int64_t n16,
                                                           uint32_t* __restrict__ out) {
  __shared__ uint32_t s_fold[4];
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nt = (int64_t)gridDim.x * blockDim.x;
  v4i acc = {0, 0, 0, 0};
  for (int64_t i = tid; i < n16; i += nt * kStreamU) {
    v4i v[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const int64_t j = i + (int64_t)u * nt;
      v[u] = j < n16 ? __builtin_nontemporal_load(x + j) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) acc ^= v[u];
  }
  uint32_t f = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) f ^= (uint32_t)__shfl_xor((int)f, off, 64);
  if (lane_id() == 0) s_fold[threadIdx.x >> 6] = f;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s_fold[0] ^ s_fold[1] ^ s_fold[2] ^ s_fold[3];
}

int stream_read_grid() { return device_info().cus; }

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s) {
  stream_read_kernel<<<stream_read_grid(), 256, 0, s>>>((const v4i*)buf, bytes / 16, out);
  return hipGetLastError();
}

}  // namespace moe
