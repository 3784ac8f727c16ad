// qgemm_internal.h — launch wrappers shared by the kernel and API translation
// units of the library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

struct MfmaArgs {
  const uint8_t* packed;
  const void* xq;       // binary16 operand layout (layout.h)
  const void* xs;       // fp32 sub-block sums
  float* out;           // y (S == 1) or split partials [S][R][N]
  int64_t N, KB, NS;
  int R, S, RT, NT;
  int64_t kbs;          // blocks per split
  int64_t hdr_off;      // byte offset of the header region
};

hipError_t launch_pack(const uint8_t* canon, uint8_t* packed, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_xprep(const uint16_t* x, void* xq, void* xs, int R, int64_t K, int RT, hipStream_t st);
hipError_t launch_mfma(const MfmaArgs& a, hipStream_t st);
hipError_t launch_reduce(const float* part, float* y, int64_t RN, int S, hipStream_t st);
hipError_t launch_dequant(const uint8_t* packed, float* w, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_argmax(const float* y, int R, int64_t N, int32_t* idx, hipStream_t st);

}  // namespace qg
