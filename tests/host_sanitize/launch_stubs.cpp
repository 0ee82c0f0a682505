// Device-side entry points of libsegattn replaced for the sanitized host build:
// every launcher fails with hipErrorNotSupported, so a validation case that
// reached a launch would surface as SA_E_HIP instead of its expected status.
// The block sizes are the attention kernels' (they enter the host's tile
// counts before any launch).
#include "../../diffusion_transformer_attention_segment_amd/csrc/internal.h"

namespace segattn {

hipError_t launch_append_bf16(const AppendArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_append_fp8(const AppendArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_append_int8(const AppendArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sparse_select(const SelectArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t sparse_select_scratch(float**) { return hipErrorNotSupported; }
hipError_t launch_attention_bf16(AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention_fp8(AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention_combine(const AttnArgs&, int, hipStream_t) { return hipErrorNotSupported; }
int attention_block_m_bf16() { return 256; }
int attention_block_m_fp8() { return 256; }
hipError_t launch_camera(const CameraArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gather(const GatherArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_dequant(const DequantArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace segattn
