// Host-side launchers of the attention kernels (defined in the .hip files).
#pragma once

#include "attn_device.h"

namespace attn {

template <int D>
hipError_t launch_prep_kv(const PrepParams &p, const RopeTable &tab, hipStream_t stream);

template <int D, bool CAUSAL>
hipError_t launch_attn_bf16(const FwdParams &p, const RopeTable &tab, hipStream_t stream);

template <int D, bool CAUSAL>
hipError_t launch_attn_f32(const F32Params &p, const RopeTable &tab, hipStream_t stream);

}  // namespace attn
