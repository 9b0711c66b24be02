// Host-side launchers of the attention kernels (defined in the .hip files).
#pragma once

#include "attn_device.h"

namespace attn {

template <int D>
hipError_t launch_prep_kv(const PrepParams &p, const RopeTable &tab, hipStream_t stream);

// The attention launchers take optional start/stop events that the runtime records with the
// kernel's own dispatch (hipExtLaunchKernel), so their interval is the kernel's execution.
template <int D, bool CAUSAL>
hipError_t launch_attn_bf16(const FwdParams &p, const RopeTable &tab, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop);

// Workgroups of the bf16 forward kernel (one-launch form) one CU holds at once; 0 on error.
template <int D>
int fwd_bf16_wgs_per_cu(bool dual);

// head_dim 256: one wave per 32 query rows, prepared K/V streamed into registers
template <bool CAUSAL>
hipError_t launch_attn_d256(const FwdParams &p, const RopeTable &tab, hipStream_t stream, hipEvent_t ev_start,
                            hipEvent_t ev_stop);

template <int D, bool CAUSAL>
hipError_t launch_attn_f32(const F32Params &p, const RopeTable &tab, hipStream_t stream,
                           hipEvent_t ev_start, hipEvent_t ev_stop);

template <typename T, int D>
hipError_t launch_merge(const MergeParams &p, hipStream_t stream);

template <int D>
hipError_t launch_decode(const DecodeParams &p, const RopeTable &tab, hipStream_t stream);

template <int D>
hipError_t launch_bwd(const BwdParams &p, const RopeTable &tab, hipStream_t stream);

}  // namespace attn
