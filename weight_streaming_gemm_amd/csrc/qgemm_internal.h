// qgemm_internal.h — launch wrappers shared by the kernel and API translation
// units of the library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

struct StreamArgs {
  const uint8_t* packed;
  int64_t hdr_off;       // byte offset of the header region
  uint32_t quant_bytes;  // sizes of the two regions (< 2^31)
  uint32_t hdr_bytes;
  const void* xq;        // binary16 operand layout (layout.h)
  const void* xs;        // fp32 sub-block sums
  float* y;              // output [R][N]
  float* part;           // partial tiles, 2 per workgroup
  uint32_t* cnt;         // per tile arrival counters, zero between launches
  int64_t N, NS;
  int KB, R;
  int64_t T;             // tiles of 4 * NT sub-tiles
  int64_t I;             // T * KB steps
  int64_t P;             // workgroups (<= I)
  int RT, NT;
};

hipError_t launch_pack(const uint8_t* canon, uint8_t* packed, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_xprep(const uint16_t* x, void* xq, void* xs, int R, int64_t K, int RT, hipStream_t st);
hipError_t launch_stream(const StreamArgs& a, hipStream_t st);
int stream_occupancy(int RT, int NT);   // resident workgroups per CU
hipError_t launch_dequant(const uint8_t* packed, float* w, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_argmax(const float* y, int R, int64_t N, int32_t* idx, hipStream_t st);

}  // namespace qg
