// Host launchers of the packing and widening kernels (pack.hip), called by the
// C ABI and the backward launcher.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace vlgqa {

hipError_t launch_cu_seqlens(const int32_t* lengths, int64_t batch, int32_t* cu,
                             hipStream_t stream);
hipError_t launch_pack(const void* padded, const int32_t* cu, int64_t batch, int64_t S,
                       int64_t row_bytes, int64_t total, void* packed, hipStream_t stream);
hipError_t launch_unpack(const void* packed, const int32_t* cu, int64_t batch, int64_t S,
                         int64_t row_bytes, void* padded, hipStream_t stream);
// n E4M3 codes (a multiple of 16, 16-byte aligned) -> n bf16 values, exactly
hipError_t launch_widen_e4m3(const void* codes, void* bf16, int64_t n, hipStream_t stream);

}  // namespace vlgqa
