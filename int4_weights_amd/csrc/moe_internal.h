// moe_internal.h -- launchers behind the C ABI (host side, C++ linkage).
// Arguments are validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct DeviceInfo {
  int cus;  // compute units of the current device
};
DeviceInfo device_info();

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int K, uint8_t* q, float* sf, hipStream_t s);
// INT8 (1, 1, 128): wn = 0 writes scales [rows, K/128]; wn = N (rows = E*N) writes them [E, K/128, N]
hipError_t launch_quant_int8(const uint16_t* x, int64_t rows, int K, int wn, int8_t* q, float* sf, hipStream_t s);
hipError_t launch_quant_weight_fp8(const uint16_t* w, int E, int N, int K, uint8_t* q, float* sfw, hipStream_t s);
hipError_t launch_pack_weight_fp8(const uint8_t* q, int E, int N, int K, uint8_t* packed, hipStream_t s);
hipError_t launch_pack_weight_int4(const uint8_t* q4, const uint16_t* s16, int E, int N, int K, uint8_t* q4_packed,
                                   uint16_t* s16_packed, hipStream_t s);
hipError_t launch_quant_weight_int4(const uint16_t* w, int E, int N, int K, uint8_t* q4, uint16_t* s16,
                                    hipStream_t s);

struct RouteArgs {
  const int32_t* ids;
  int T, k, E, R;
  int masked;       // 0 = contiguous, 1 = masked
  int align;        // contiguous alignment
  int max_m;        // masked capacity per expert
  const uint8_t* payload;
  int64_t row_bytes;
  const uint8_t* payload2;
  int64_t row_bytes2;
  uint8_t* packed;
  uint8_t* packed2;
  int64_t rows_cap;
  int32_t* counts;
  int32_t* seg_offsets;
  int32_t* m_indices;
  int32_t* output_index;
  int32_t* dev_status;
  int32_t* ws;      // workspace (large path): chunk counts [nchunks*E] then status [nchunks]
  int nchunks;
  const uint16_t* xq;  // quantising pack: bf16 token rows [T, K] (nullptr: copy payload rows)
  int K;               // quantising pack: packed = E4M3 codes [rows_cap, K], packed2 = fp32 scales [rows_cap, K/128]
};
constexpr int kRouteSmallMax = 4096;   // routes handled by the single-launch path
constexpr int kRouteChunk = 1024;      // routes per counting workgroup (large path)
int64_t route_workspace_bytes(int R, int E);
constexpr int kMaxDevices = 64;
// the fixed device scratch of moe_route_pack_noalloc: its size, and its address on the current device
int64_t route_scratch_bytes();
hipError_t route_scratch_ptr(int32_t** out);
hipError_t launch_route_pack(const RouteArgs& a, hipStream_t s);

struct GemmArgs {
  const uint8_t* A;      // fp8 or int8 codes [rows, K] or bf16 [rows, K] (int4 and bf16 paths)
  const float* SFA;      // [rows, K/128] (fp8 and int8 paths)
  const uint8_t* W;      // fp8 or int8 [E, N, K], int4 or fp4 [E, N, K/2], or bf16 [E, N, K]
  const void* SW;        // SFW fp32 [E, N/128, K/128], S16 fp16 [E, N, K/128], E8M0 bytes [E, N, K/32] (fp4)
                         // or fp32 [E, K/128, N] (int8)
  uint16_t* D;           // bf16 [rows, N]
  uint8_t* Q;            // SwiGLU GEMM: E4M3 [rows, N/2] (instead of D)
  float* SQ;             // SwiGLU GEMM: fp32 [rows, N/256]
  const int32_t* counts;
  const int32_t* seg_offsets;
  int E;
  int masked;
  int64_t rows_cap;      // rows of A/D (contiguous) ; masked: E*max_m
  int max_m;
  int N, K;
  int wpacked;           // W in the fragment-packed order (moe_pack_weight_fp8 / _int4)
};
hipError_t launch_gemm_fp8(const GemmArgs& a, int expected_m, hipStream_t s);
hipError_t launch_gemm_fp8_swiglu(const GemmArgs& a, int expected_m, hipStream_t s);
hipError_t launch_gemm_int4(const GemmArgs& a, int expected_m, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmArgs& a, int expected_m, hipStream_t s);
hipError_t launch_gemm_fp4(const GemmArgs& a, int expected_m, hipStream_t s);
hipError_t launch_gemm_int8(const GemmArgs& a, int expected_m, hipStream_t s);
hipError_t launch_quant_weight_fp4(const uint16_t* w, int E, int N, int K, uint8_t* w4, uint8_t* sw, hipStream_t s);
hipError_t launch_pack_weight_fp4(const uint8_t* w4, const uint8_t* sw, int E, int N, int K, uint8_t* w4p,
                                  uint8_t* swp, hipStream_t s);

struct SwigluArgs {
  const uint16_t* gu;    // bf16 [rows, 2I]: gate columns then up columns
  uint8_t* q;            // E4M3 [rows, I]
  float* sf;             // fp32 [rows, I/128]
  const int32_t* counts;
  const int32_t* seg_offsets;
  int E;
  int masked;
  int max_m;
  int64_t rows_cap;      // rows of gate_up / q (masked: E*max_m)
  int I;
};
hipError_t launch_swiglu_quant(const SwigluArgs& a, hipStream_t s);

int stream_read_grid();
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s);
hipError_t launch_combine(const uint16_t* Y, int64_t y_rows, const int32_t* oi, const float* w, int T, int k,
                          int N, uint16_t* Z, hipStream_t s);

}  // namespace moe
